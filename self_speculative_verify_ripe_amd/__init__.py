"""RIPE self-speculative verification attention for MI355X (gfx950).

The compute lives in ``libripe.so`` (HIP kernels behind the C ABI of
include/ripe.h); this package is its Python binding.
"""
from .binding import (DTYPES, LAYOUTS, RIPE_BF16, RIPE_BYTES_CACHE,  # noqa: F401
                      RIPE_BYTES_WORKSPACE, RIPE_F32, RIPE_LAYOUT_DEEPEST, RIPE_LAYOUT_FULL,
                      RIPE_LAYOUT_RIPE, STATUS, RipeError, make_desc, ripe_commit, ripe_desc_t,
                      ripe_group_t, ripe_layout_bytes, ripe_verify_attn, pack_groups, new_workspace,
                      ripe_accept_desc_t, make_accept_desc, ripe_accept_workspace_bytes, ripe_accept,
                      commit_args, pack_parents, ripe_position_error, RIPE_BYTES_POSERR_WORKSPACE,
                      ripe_verify_attn_noalloc, ripe_position_error_tail, RIPE_TAIL_STATS,
                      TAIL_FIELDS)
