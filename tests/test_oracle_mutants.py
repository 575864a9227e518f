"""Planted mistakes in the oracle must fail a pin.

Each case rewrites one line of oracle/gpb_oracle.c (a dropped term, a wrong
index or bound, an inclusive instead of exclusive sum, a missing zero fill),
builds the variant with gcc in a temporary directory and runs every pin of
tests/pins.py against it in a child process.  The child must fail.  The
numpy closed form, the oracle's second route, gets the same treatment: a
child process replaces it with a rewritten copy before running the pins.
This is CPU-only and never touches the product library."""
import os
import subprocess
import sys
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "gpb_oracle.c")

MUTANTS = {
    "slot0_not_reserved_src": ("src[s] = i + 1;", "src[s] = i;"),
    "slot0_not_reserved_inverse": ("= w * CAP + i + 1;", "= w * CAP + i;"),
    "current_base_drops_prefix": ("current_bases[r] = PS * run_slots + PS * prefix_pages[r];",
                                  "current_bases[r] = PS * run_slots;"),
    "q_starts_inclusive": ("q_starts[r] = run_tokens;",
                           "q_starts[r] = run_tokens + cur_tokens[r];"),
    "k_bases_in_pages": ("k_bases[r] = PS * run_slots;", "k_bases[r] = run_slots;"),
    "q_bases_in_pages": ("q_bases[r] = PS * run_cur_pages;", "q_bases[r] = run_cur_pages;"),
    "kv_lens_page_padded": ("kv_lens[r] = PS * prefix_pages[r] + cur_tokens[r];",
                            "kv_lens[r] = PS * (prefix_pages[r] + C);"),
    "owner_skips_pool_entries": ("owner[s] = NP + writer[i];", "owner[s] = writer[i];"),
    "single_writer": ("int32_t w = i % W;", "int32_t w = 0;"),
    "prefix_owner_not_modulo": ("owner[s] = slot_pages[s] % NP;", "owner[s] = 0;"),
    "no_staging_zero": ("memset(staging, 0, (size_t)(n_staging_rows * RB));", ";"),
    "sentinel_not_zeroed": ("if (e < 0 || p < 0) { memset(out, 0, (size_t)page_bytes); continue; }",
                            "if (e < 0 || p < 0) { continue; }"),
    "gather_row_stride": ("table[e] + (int64_t)p * page_bytes", "table[e] + (int64_t)p * RB"),
    "floor_not_ceil": ("return (a + b - 1) / b;", "return a / b;"),
    "dummy_page_accepted": ("if (p < 1 || p >= n_pool_pages || seen[p])",
                            "if (p < 0 || p >= n_pool_pages || seen[p])"),
    "duplicates_accepted": ("if (p < 1 || p >= n_pool_pages || seen[p])",
                            "if (p < 1 || p >= n_pool_pages)"),
    "capacity_off_by_one": ("if (1 + total_cur_pages > staging_cap_pages)",
                            "if (total_cur_pages > staging_cap_pages)"),
    "token_page_index": ("int32_t s = slot_base[r] + prefix_pages[r] + j / PS;",
                         "int32_t s = slot_base[r] + prefix_pages[r];"),
    "prefix_span_end": ("prefix_span[2 * r + 1] = running_slots + prefix_pages[r];",
                        "prefix_span[2 * r + 1] = running_slots + n;"),
    "inverse_not_cleared": ("for (int32_t p = 0; p < n_pool_pages; p++) page_inverse[p] = -1;",
                            ";"),
    "mixed_locs_from_k_base": ("mixed_locs[t] = current_bases[r] + j;",
                               "mixed_locs[t] = k_bases[r] + j;"),
    "token_req_off_by_one": ("      token_req[token + j] = r;", "      token_req[token + j] = r + (j == 0);"),
    "topk_offset_skips_prefix": ("    dense_row += page_size * pages;",
                                 "    dense_row += page_size * (pages - prefix_pages[r]);"),
    "segment_kv_len_padded": ("    segments[4 * r + 3] = page_size * prefix_pages[r] + cur_tokens[r];",
                              "    segments[4 * r + 3] = page_size * pages;"),
    "current_slot_not_advanced": ("      current_slots[i++] = slot++;",
                                  "      current_slots[i++] = slot;"),
    "pool_loc_wrong_page": ("      pool_locs[token++] = req_pages[first_cur + j / page_size] * page_size + j % page_size;",
                            "      pool_locs[token++] = req_pages[first_cur] * page_size + j % page_size;"),
    "gather_slots_uses_k": ("    int32_t s = slots[k];", "    int32_t s = k;"),
    "fill_skips_pool": ("    else memcpy(pool + q * RB, row, (size_t)RB);", "    else (void)q;"),
    "page_ntok_full_pages": ("                             ? cur_tokens[r] - k * page_size : page_size;",
                             "                             ? page_size : page_size;"),
    "page_token0_unpaged": ("      cur_page_token0[i] = token + k * page_size;",
                            "      cur_page_token0[i] = token + k;"),
    "stray_row_not_flagged": ("if (row < 0 || row >= n_staging_rows) { bad = 1; continue; }",
                              "if (row < 0 || row >= n_staging_rows) { continue; }"),
    "staging_rows_via_page_inverse": (
        "staging_rows[t] = staging_page_inverse[loc / PS] * PS + loc % PS;",
        "staging_rows[t] = page_inverse[loc / PS] * PS + loc % PS;"),
    "staging_row_drops_offset": (
        "staging_rows[t] = staging_page_inverse[loc / PS] * PS + loc % PS;",
        "staging_rows[t] = staging_page_inverse[loc / PS] * PS;"),
    "slab_stride_short": ("= w * CAP + i + 1;", "= w * (CAP - 1) + i + 1;"),
    "current_span_starts_at_base": (
        "current_span[2 * r + 0] = running_slots + prefix_pages[r];",
        "current_span[2 * r + 0] = running_slots;"),
    "q_lens_in_pages": ("q_lens[r] = cur_tokens[r];", "q_lens[r] = C;"),
    "page_inverse_off_by_one": ("page_inverse[slot_pages[s]] = s;",
                                "page_inverse[slot_pages[s]] = s + 1;"),
    "counts_drop_prefix": ("S += prefix_pages[r] + C;", "S += C;"),
    "segment_first_row_is_token": ("segments[4 * r + 2] = dense_row;",
                                   "segments[4 * r + 2] = token;"),
    "prefix_slot_not_advanced": ("prefix_slots[u++] = slot++;", "prefix_slots[u++] = slot;"),
    "fill_skips_staging": ("else memcpy(staging + d * RB, row, (size_t)RB);",
                           "else (void)d;"),
    # the variant reads seen[n_pool_pages], one byte past a heap block: it lands
    # in malloc's rounding or the next block's header, never outside the heap
    "last_page_accepted": ("if (p < 1 || p >= n_pool_pages || seen[p])",
                           "if (p < 1 || p > n_pool_pages || seen[p])"),
    "slot_pages_reversed": ("slot_pages[s] = req_pages[s];",
                            "slot_pages[s] = req_pages[S - 1 - s];"),
    "record_owner_of_list_index": ("records[4 * k + 1] = owner[s];",
                                   "records[4 * k + 1] = owner[k];"),
    "record_src_of_list_index": ("records[4 * k + 2] = src[s];",
                                 "records[4 * k + 2] = src[k];"),
    "record_gather_slot_field": (
        "int32_t s = records[4 * k + 0], e = records[4 * k + 1], p = records[4 * k + 2];",
        "int32_t s = k, e = records[4 * k + 1], p = records[4 * k + 2];"),
    "writer_rows_global": ("writer_rows[k] = (int32_t)(staging_rows[t] - w * slab_rows);",
                           "writer_rows[k] = (int32_t)staging_rows[t];"),
    "writer_page_row0_global": ("writer_page_row0[i] = k - writer_offsets[w];",
                                "writer_page_row0[i] = k;"),
    "writer_list_skips_tail": (
        "int32_t end = (q + 1) * PS < cur_tokens[r] ? (q + 1) * PS : cur_tokens[r];",
        "int32_t end = (q + 1) * PS < cur_tokens[r] ? (q + 1) * PS : cur_tokens[r] - 1;"),
    "writer_list_page_index": ("if (i % W != w) continue;", "if (q % W != w) continue;"),
}

CHILD = r"""
import os, sys
sys.path[:0] = [{root!r}, {tests!r}]
import oracle, pins
try:
    pins.run_all(oracle.Oracle({lib!r}), n_random=40)
except AssertionError as e:
    print("PIN FAILED:", e, flush=True)
    os._exit(3)   # a mutant may have corrupted the heap: skip teardown
except ValueError as e:
    print("REJECTED A VALID BATCH:", e, flush=True)
    os._exit(4)
print("ALL PINS PASSED")
"""


def _build_variant(name, old, new, tmp):
    text = open(SRC).read()
    assert text.count(old) >= 1, "mutation target not found: " + old
    text = text.replace(old, new, 1)
    c = os.path.join(tmp, name + ".c")
    so = os.path.join(tmp, name + ".so")
    open(c, "w").write(text)
    subprocess.run(["gcc", "-O1", "-std=c11", "-w", "-shared", "-fPIC", "-o", so, c],
                   check=True)
    return so


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    old, new = MUTANTS[name]
    with tempfile.TemporaryDirectory() as tmp:
        so = _build_variant(name, old, new, tmp)
        code = CHILD.format(root=ROOT, tests=HERE, lib=so)
        r = subprocess.run([sys.executable, "-c", code], capture_output=True,
                           text=True, timeout=300)
    assert r.returncode in (3, 4), "planted mistake %s was not caught by a pin (rc %d):\n%s" % (
        name, r.returncode, r.stdout[-2000:] + r.stderr[-2000:])


CLOSED_FORM = os.path.join(ROOT, "oracle", "closed_form.py")

CLOSED_FORM_MUTANTS = {
    "cf_page_cursor_skips_current": ("page_cursor += P + C", "page_cursor += P"),
    "cf_tail_not_zero": ("block = np.zeros((C * PS, RB), dtype=np.uint8)",
                         "block = np.ones((C * PS, RB), dtype=np.uint8)"),
    "cf_token_cursor_frozen": ("token_cursor += c", "token_cursor += 0"),
    "cf_pool_page_not_scaled": ("pool_rows[page * PS:(page + 1) * PS]",
                                "pool_rows[page:page + PS]"),
    "cf_prefix_page_offset": ("int(req_pages[page_cursor + k])",
                              "int(req_pages[page_cursor + k + 1 if k + 1 < P else k])"),
}

CF_CHILD = r"""
import os, sys
sys.path[:0] = [{root!r}, {tests!r}]
import oracle, pins
from oracle import closed_form
src = open({path!r}).read()
assert src.count({old!r}) >= 1, "mutation target not found"
exec(compile(src.replace({old!r}, {new!r}, 1), {path!r}, "exec"), closed_form.__dict__)
try:
    pins.run_all(oracle.default(), n_random=40)
except AssertionError as e:
    print("PIN FAILED:", e, flush=True)
    os._exit(3)
print("ALL PINS PASSED")
"""


@pytest.mark.parametrize("name", sorted(CLOSED_FORM_MUTANTS))
def test_planted_closed_form_mistake_is_caught(name):
    old, new = CLOSED_FORM_MUTANTS[name]
    code = CF_CHILD.format(root=ROOT, tests=HERE, path=CLOSED_FORM, old=old, new=new)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 3, "planted mistake %s was not caught by a pin (rc %d):\n%s" % (
        name, r.returncode, r.stdout[-2000:] + r.stderr[-2000:])


def test_unmutated_closed_form_passes_in_child():
    """Control for the mechanism above: the same re-exec with nothing changed
    passes every pin."""
    old = CLOSED_FORM_MUTANTS["cf_token_cursor_frozen"][0]
    code = CF_CHILD.format(root=ROOT, tests=HERE, path=CLOSED_FORM, old=old, new=old)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0 and "ALL PINS PASSED" in r.stdout, r.stdout[-2000:] + r.stderr[-2000:]


def test_unmutated_oracle_passes_in_child():
    code = CHILD.format(root=ROOT, tests=HERE,
                        lib=os.path.join(ROOT, "oracle", "liboracle.so"))
    import oracle
    oracle.default()   # make sure the library is built
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
