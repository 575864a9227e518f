import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP path")
    # the tests load what is built; they build only when nothing is (the
    # build script is loaded by path: importing the package needs the library)
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "gpb_build", os.path.join(ROOT, "gather_plan_build_amd", "build.py"))
    gbuild = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(gbuild)
    if not os.path.exists(gbuild.LIB):
        gbuild.build()
    import oracle.build as obuild
    obuild.build(force=False)


@pytest.fixture(scope="session")
def orc():
    import oracle
    return oracle.default()
