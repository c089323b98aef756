"""Thin ctypes binding of libripe.so (the C ABI in include/ripe.h).

Argument marshalling only: device buffers are torch tensors on the GPU (or
raw device addresses), host arrays are NumPy / Python sequences, and every
step of the computation runs in the library's HIP kernels.  If the library
is missing, importing this module raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Iterable, Optional, Sequence

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("RIPE_LIB", os.path.join(_PKG, "libripe.so"))

RIPE_LAYOUT_FULL, RIPE_LAYOUT_DEEPEST, RIPE_LAYOUT_RIPE = 0, 1, 2
RIPE_F32, RIPE_BF16 = 0, 1
RIPE_BYTES_CACHE, RIPE_BYTES_WORKSPACE, RIPE_BYTES_POSERR_WORKSPACE = 0, 1, 2
RIPE_WORKSPACE_ZERO_BYTES = 16640  # leading workspace bytes that must be zero before its first use
STATUS = {0: "RIPE_OK", -1: "RIPE_EINVAL", -2: "RIPE_ERANGE", -3: "RIPE_ECAPACITY",
          -4: "RIPE_EUNSUPPORTED", -5: "RIPE_EWORKSPACE", -6: "RIPE_EHIP"}
LAYOUTS = {"full": RIPE_LAYOUT_FULL, "deepest": RIPE_LAYOUT_DEEPEST, "ripe": RIPE_LAYOUT_RIPE}
DTYPES = {"f32": RIPE_F32, "bf16": RIPE_BF16}


class RipeError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what} failed: {STATUS.get(status, status)}")
        self.status = status


class ripe_desc_t(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "layout", "dtype", "R", "W", "batch", "t_max", "n_kv_heads", "head_dim", "n_q_heads",
        "max_rows", "max_groups", "split_len", "page_len", "n_pages")]


class ripe_group_t(ctypes.Structure):
    _fields_ = [("seq", ctypes.c_int32), ("depth", ctypes.c_int32), ("row_start", ctypes.c_int32),
                ("n_rows", ctypes.c_int32)]


class ripe_accept_desc_t(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("k", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("temperature", ctypes.c_float)]


def _load():
    # torch ships its own HIP runtime under the same soname as /opt/rocm's.
    # Load torch first so that libripe.so binds to the runtime torch already
    # uses: one process, one HIP runtime.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libripe.so not built ({LIB_PATH}); run "
                          "python self_speculative_verify_ripe_amd/build.py")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    lib.ripe_layout_bytes.argtypes = [ctypes.POINTER(ripe_desc_t), ctypes.c_int32]
    lib.ripe_layout_bytes.restype = ctypes.c_int64
    lib.ripe_verify_attn.argtypes = [ctypes.POINTER(ripe_desc_t), P, ctypes.POINTER(ctypes.c_int32),
                                     ctypes.POINTER(ripe_group_t), ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_float, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.ripe_verify_attn.restype = ctypes.c_int
    lib.ripe_verify_attn_noalloc.argtypes = [ctypes.POINTER(ripe_desc_t), P, ctypes.POINTER(ctypes.c_int32),
                                             ctypes.POINTER(ripe_group_t), ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_float, P, P, P, P, P, P]
    lib.ripe_verify_attn_noalloc.restype = ctypes.c_int
    lib.ripe_verify_attn_inflight.argtypes = [ctypes.POINTER(ripe_desc_t), P, ctypes.POINTER(ctypes.c_int32),
                                              ctypes.POINTER(ripe_group_t), ctypes.POINTER(ctypes.c_int32),
                                              ctypes.c_int32, ctypes.c_int32, ctypes.c_float, P, P, P, P, P, P,
                                              ctypes.c_size_t, P]
    lib.ripe_verify_attn_inflight.restype = ctypes.c_int
    lib.ripe_commit.argtypes = [ctypes.POINTER(ripe_desc_t), P, ctypes.POINTER(ctypes.c_int32),
                                ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32), P,
                                ctypes.c_int32, P]
    lib.ripe_commit.restype = ctypes.c_int
    lib.ripe_accept_workspace_bytes.argtypes = [ctypes.POINTER(ripe_accept_desc_t)]
    lib.ripe_accept_workspace_bytes.restype = ctypes.c_int64
    lib.ripe_accept.argtypes = [ctypes.POINTER(ripe_accept_desc_t)] + [P] * 9 + [ctypes.c_size_t, P]
    lib.ripe_accept.restype = ctypes.c_int
    lib.ripe_position_error.argtypes = [ctypes.POINTER(ripe_desc_t), P, ctypes.POINTER(ctypes.c_int32),
                                        ctypes.POINTER(ripe_group_t), ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_float, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.ripe_position_error.restype = ctypes.c_int
    lib.ripe_position_error_tail.argtypes = [P, P, ctypes.POINTER(ctypes.c_int32), ctypes.c_int32,
                                             ctypes.c_int32, ctypes.c_int32, ctypes.c_double, P, P]
    lib.ripe_position_error_tail.restype = ctypes.c_int
    I32P = ctypes.POINTER(ctypes.c_int32)
    lib.ripe_verify_attn_paged.argtypes = [ctypes.POINTER(ripe_desc_t), P, I32P, I32P,
                                           ctypes.POINTER(ripe_group_t), I32P, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_float, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.ripe_verify_attn_paged.restype = ctypes.c_int
    lib.ripe_commit_paged.argtypes = [ctypes.POINTER(ripe_desc_t), P, I32P, I32P, I32P, I32P, P,
                                      ctypes.c_int32, P]
    lib.ripe_commit_paged.restype = ctypes.c_int
    return lib


lib = _load()


def make_desc(layout, dtype, R, W, batch, t_max, n_kv_heads, head_dim, n_q_heads,
              max_rows=0, max_groups=0, split_len=0, page_len=0, n_pages=0) -> ripe_desc_t:
    layout = LAYOUTS[layout] if isinstance(layout, str) else int(layout)
    dtype = DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
    return ripe_desc_t(layout, dtype, R, W, batch, t_max, n_kv_heads, head_dim, n_q_heads,
                       max_rows, max_groups, split_len, page_len, n_pages)


def _table(desc: ripe_desc_t, block_table) -> np.ndarray:
    """A block table as a C-contiguous int32 array [batch, t_max / page_len]."""
    if desc.page_len <= 0:
        raise ValueError("block_table given for an unpaged descriptor")
    tab = np.ascontiguousarray(np.asarray(block_table, dtype=np.int32))
    if tab.size != desc.batch * (desc.t_max // desc.page_len):
        raise ValueError("block_table must have batch * (t_max / page_len) entries")
    return tab


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def _i32(a, n: Optional[int] = None):
    arr = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    if n is not None and arr.size != n:
        raise ValueError(f"expected {n} entries, got {arr.size}")
    return arr


def pack_groups(groups: Iterable) -> np.ndarray:
    """Groups as a contiguous int32 array [n, 4] of (seq, depth, row_start,
    n_rows), the memory layout of ripe_group_t.  Pack once and reuse it to
    keep per-call host work minimal."""
    if isinstance(groups, np.ndarray):
        arr = np.ascontiguousarray(groups, dtype=np.int32).reshape(-1, 4)
        return arr
    rows = []
    for g in groups:
        if isinstance(g, tuple):
            rows.append(g)
        else:
            rows.append((g.seq, g.depth, g.row_start, g.n_rows))
    return np.ascontiguousarray(np.array(rows, dtype=np.int32).reshape(-1, 4))


def _groups(groups):
    arr = groups if (isinstance(groups, np.ndarray) and groups.dtype == np.int32
                     and groups.ndim == 2 and groups.flags["C_CONTIGUOUS"]) else pack_groups(groups)
    return arr.ctypes.data_as(ctypes.POINTER(ripe_group_t)), arr.shape[0], arr


def ripe_layout_bytes(desc: ripe_desc_t, kind: int = RIPE_BYTES_CACHE) -> int:
    n = int(lib.ripe_layout_bytes(ctypes.byref(desc), int(kind)))
    if n < 0:
        raise RipeError(n, "ripe_layout_bytes")
    return n


def new_workspace(desc: ripe_desc_t, device="cuda"):
    """A workspace big enough for any verify call within the descriptor's
    bounds, zero-filled (its leading counters must start at zero)."""
    import torch
    return torch.zeros(ripe_layout_bytes(desc, RIPE_BYTES_WORKSPACE), dtype=torch.uint8,
                       device=device)


def pack_parents(groups: Iterable) -> np.ndarray:
    """Each group's in-flight parent block as an int32 array [n, 2] of
    (parent_row_start, parent_rows); (0, 0) for groups without one."""
    rows = []
    for g in groups:
        if isinstance(g, tuple):
            rows.append((g[4], g[5]) if len(g) >= 6 else (0, 0))
        else:
            rows.append((getattr(g, "parent_row_start", 0), getattr(g, "parent_rows", 0)))
    return np.ascontiguousarray(np.array(rows, dtype=np.int32).reshape(-1, 2))


def ripe_verify_attn(desc: ripe_desc_t, cache, seq_len: Sequence[int], groups: Iterable,
                     n_rows: int, softmax_scale: float, q, kv_new, out, lse=None, plane_sel=None,
                     workspace=None, workspace_bytes: Optional[int] = None, stream=None,
                     parents=None, block_table=None) -> None:
    """Launch verification attention (asynchronous on ``stream``).  Groups
    with an in-flight parent block (``parents`` [n, 2], or groups carrying
    parent_row_start / parent_rows) go through ripe_verify_attn_inflight;
    a paged cache (``block_table``) through ripe_verify_attn_paged."""
    sl = seq_len if (isinstance(seq_len, np.ndarray) and seq_len.dtype == np.int32
                     and seq_len.flags["C_CONTIGUOUS"]) else _i32(seq_len, desc.batch)
    if sl.size != desc.batch:
        raise ValueError("seq_len must have one entry per sequence")
    gptr, ng, _keep = _groups(groups)
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if parents is None and not isinstance(groups, np.ndarray):
        parents = pack_parents(groups)
        if not parents.any():
            parents = None
    if block_table is not None:
        tab = _table(desc, block_table)
        par = None if parents is None else np.ascontiguousarray(parents, dtype=np.int32).reshape(-1, 2)
        if par is not None and par.shape[0] != ng:
            raise ValueError("parents must have one (row_start, n_rows) pair per group")
        I32P = ctypes.POINTER(ctypes.c_int32)
        st = lib.ripe_verify_attn_paged(ctypes.byref(desc), _ptr(cache), tab.ctypes.data_as(I32P),
                                        sl.ctypes.data_as(I32P), gptr,
                                        None if par is None else par.ctypes.data_as(I32P), ng,
                                        int(n_rows), float(softmax_scale), _ptr(q), _ptr(kv_new), _ptr(out),
                                        _ptr(lse), _ptr(plane_sel), _ptr(workspace), int(workspace_bytes),
                                        _stream(stream))
        what = "ripe_verify_attn_paged"
    elif parents is None:
        st = lib.ripe_verify_attn(ctypes.byref(desc), _ptr(cache),
                                  sl.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), gptr, ng,
                                  int(n_rows), float(softmax_scale), _ptr(q), _ptr(kv_new), _ptr(out),
                                  _ptr(lse), _ptr(plane_sel), _ptr(workspace), int(workspace_bytes),
                                  _stream(stream))
        what = "ripe_verify_attn"
    else:
        par = np.ascontiguousarray(parents, dtype=np.int32).reshape(-1, 2)
        if par.shape[0] != ng:
            raise ValueError("parents must have one (row_start, n_rows) pair per group")
        st = lib.ripe_verify_attn_inflight(ctypes.byref(desc), _ptr(cache),
                                           sl.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), gptr,
                                           par.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), ng,
                                           int(n_rows), float(softmax_scale), _ptr(q), _ptr(kv_new),
                                           _ptr(out), _ptr(lse), _ptr(plane_sel), _ptr(workspace),
                                           int(workspace_bytes), _stream(stream))
        what = "ripe_verify_attn_inflight"
    if st != 0:
        raise RipeError(st, what)


def ripe_verify_attn_noalloc(desc: ripe_desc_t, cache, seq_len: Sequence[int], groups: Iterable,
                             n_rows: int, softmax_scale: float, q, kv_new, out, lse=None, plane_sel=None,
                             stream=None) -> None:
    """ripe_verify_attn without a workspace: the split partials use the
    library's static device scratch (asynchronous on ``stream``; calls that
    overlap on one GPU race on that scratch)."""
    sl = _i32(seq_len, desc.batch)
    gptr, ng, _keep = _groups(groups)
    st = lib.ripe_verify_attn_noalloc(ctypes.byref(desc), _ptr(cache),
                                      sl.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), gptr, ng,
                                      int(n_rows), float(softmax_scale), _ptr(q), _ptr(kv_new), _ptr(out),
                                      _ptr(lse), _ptr(plane_sel), _stream(stream))
    if st != 0:
        raise RipeError(st, "ripe_verify_attn_noalloc")


def ripe_position_error(desc: ripe_desc_t, cache, seq_len: Sequence[int], groups: Iterable,
                        n_rows: int, softmax_scale: float, q, kv_new, err, cond=None, out_f32=None,
                        lse=None, workspace=None, workspace_bytes: Optional[int] = None,
                        stream=None) -> None:
    """Per-position substitution error of a FULL cache (asynchronous on
    ``stream``): err and cond [n_groups, t_max] float32 on the device."""
    sl = _i32(seq_len, desc.batch)
    if sl.size != desc.batch:
        raise ValueError("seq_len must have one entry per sequence")
    gptr, ng, _keep = _groups(groups)
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.ripe_position_error(ctypes.byref(desc), _ptr(cache), sl.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                 gptr, ng, int(n_rows), float(softmax_scale), _ptr(q), _ptr(kv_new), _ptr(err),
                                 _ptr(cond), _ptr(out_f32), _ptr(lse), _ptr(workspace), int(workspace_bytes),
                                 _stream(stream))
    if st != 0:
        raise RipeError(st, "ripe_position_error")


RIPE_TAIL_STATS = 8
TAIL_FIELDS = ("tail_positions", "tail_share", "tail_in_window", "window_share", "ill_conditioned",
               "ill_conditioned_share", "total", "positions")


def ripe_position_error_tail(err, T: Sequence[int], window: int, stats, cond=None, tail_frac: float = 0.01,
                             row_stride: Optional[int] = None, stream=None) -> None:
    """Tail figures of error rows (asynchronous on ``stream``): err (and
    cond) [n_rows, row_stride] float32 on the device, T one prefix length per
    row, stats [n_rows, RIPE_TAIL_STATS] float64 on the device (fields in
    TAIL_FIELDS order)."""
    t = np.ascontiguousarray(np.asarray(T, dtype=np.int32).reshape(-1))
    if row_stride is None:
        row_stride = int(err.shape[-1])
    st = lib.ripe_position_error_tail(_ptr(err), _ptr(cond), t.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                      int(t.size), int(row_stride), int(window), float(tail_frac), _ptr(stats),
                                      _stream(stream))
    if st != 0:
        raise RipeError(st, "ripe_position_error_tail")


def ripe_commit(desc: ripe_desc_t, cache, seq_len, n_accept: Sequence[int],
                src_row: Sequence[int], kv_new, n_rows: int, stream=None, block_table=None) -> np.ndarray:
    """Commit accepted rows; returns the updated committed lengths (an int32
    array; ``seq_len`` is updated in place when it is an int32 NumPy array).
    A paged cache takes its ``block_table`` (ripe_commit_paged)."""
    inplace = isinstance(seq_len, np.ndarray) and seq_len.dtype == np.int32 and \
        seq_len.flags["C_CONTIGUOUS"]
    sl = seq_len if inplace else _i32(seq_len, desc.batch).copy()
    na = _i32(n_accept, desc.batch)
    sr = _i32(src_row, desc.batch)
    I32P = ctypes.POINTER(ctypes.c_int32)
    if block_table is not None:
        tab = _table(desc, block_table)
        st = lib.ripe_commit_paged(ctypes.byref(desc), _ptr(cache), tab.ctypes.data_as(I32P),
                                   sl.ctypes.data_as(I32P), na.ctypes.data_as(I32P), sr.ctypes.data_as(I32P),
                                   _ptr(kv_new), int(n_rows), _stream(stream))
        what = "ripe_commit_paged"
    else:
        st = lib.ripe_commit(ctypes.byref(desc), _ptr(cache), sl.ctypes.data_as(I32P), na.ctypes.data_as(I32P),
                             sr.ctypes.data_as(I32P), _ptr(kv_new), int(n_rows), _stream(stream))
        what = "ripe_commit"
    if st != 0:
        raise RipeError(st, what)
    return sl


def make_accept_desc(batch: int, k: int, vocab: int, temperature: float) -> ripe_accept_desc_t:
    return ripe_accept_desc_t(int(batch), int(k), int(vocab), float(temperature))


def ripe_accept_workspace_bytes(desc: ripe_accept_desc_t) -> int:
    n = int(lib.ripe_accept_workspace_bytes(ctypes.byref(desc)))
    if n < 0:
        raise RipeError(n, "ripe_accept_workspace_bytes")
    return n


def ripe_accept(desc: ripe_accept_desc_t, target_logits, draft_logits, tokens, has_fallback, rand,
                n_accept, branch, next_token, workspace=None, workspace_bytes: Optional[int] = None,
                stream=None) -> None:
    """Accept / rollback (asynchronous on ``stream``); every array is a device tensor."""
    if workspace is None:
        import torch
        workspace = torch.empty(ripe_accept_workspace_bytes(desc), dtype=torch.uint8,
                                device=n_accept.device)
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    st = lib.ripe_accept(ctypes.byref(desc), _ptr(target_logits), _ptr(draft_logits), _ptr(tokens),
                         _ptr(has_fallback), _ptr(rand), _ptr(n_accept), _ptr(branch), _ptr(next_token),
                         _ptr(workspace), int(workspace_bytes), _stream(stream))
    if st != 0:
        raise RipeError(st, "ripe_accept")


def commit_args(n_accept, branch, primary_rows, fallback_rows):
    """ripe_commit's n_accept / src_row (host int32 arrays) from an accept
    result: the kept tokens start at the first draft row of the chosen
    chain's group.  primary_rows / fallback_rows: first row of each
    sequence's primary / fallback group (fallback ignored where unused)."""
    n = _i32(n_accept)
    br = _i32(branch, n.size)
    src = np.where(br == 1, _i32(fallback_rows, n.size), _i32(primary_rows, n.size)).astype(np.int32)
    src[n == 0] = 0
    return n, src
