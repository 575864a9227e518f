"""MI355X-native KV-compose hot path: per-batch plan build, per-layer current
row scatter and slot-dense page gather (libgpb.so, HIP for gfx950).

Importing this package loads libgpb.so and fails loudly if it is missing.
"""
from .binding import (BatchMeta, GpbError, Plan, Sources, compose_gather,  # noqa: F401
                      compose_gather_slots, compose_gather_records, compose_layer,
                      compose_consume, compose_layer_ahead, compose_layer_fill,
                      compose_layer_noalloc, compose_consume_fill,
                      compose_layer_ahead_fill,
                      current_row_fill, writer_counts,
                      compose_gather_groups, compose_layer_groups,
                      current_row_scatter_groups,
                      current_row_scatter, plan_build, plan_sizes, staging_clear,
                      strerror, LIB_PATH, PLAN_FIELDS, STATUS_BAD_DESCRIPTOR,
                      STATUS_BAD_STAGING_ROW, STATUS_BAD_PLAN_INPUT,
                      STATUS_LAYER_MISMATCH)
from .runner import ComposeRunner, layer_groups, layer_groups_two_launch  # noqa: F401
