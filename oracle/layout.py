"""Byte layout of one recurrent layer's cache -- TEST INFRASTRUCTURE ONLY.

An independent NumPy statement of the cache byte layout that the C ABI
declares, used to build device buffers for parity tests and to compare the
buffers the commit kernel writes, byte for byte.  It shares no code with the
library (which computes addresses in C++).

Layout (E = element bytes, T = t_max, a multiple of 32; We = min(W, T);
BW = min(32, We)); the K region comes first, then the V region:

* FULL     K [B][R][Hkv][T][D]              V [B][R][Hkv][T/32][D][32]
* DEEPEST  K [B][Hkv][T][D]                 V [B][Hkv][T/32][D][32]
* RIPE     K deep [B][Hkv][T][D]            V deep [B][Hkv][T/32][D][32]
             then ring [B][R-1][Hkv][We][D]   then ring [B][R-1][Hkv][We/BW][D][BW]

V is stored transposed in blocks of 32 positions (each head dimension's 32
values contiguous).  Plane p is stored at index p - 1 (plane R deepest);
RIPE keeps position j's planes 1..R-1 in ring slot j mod We.

The memory model follows the RIPE abstract (zhuanzhiai.com paper page):
one shared plane costs T positions per sequence, the full cache R*T, RIPE
T + W*(R-1).
"""
from __future__ import annotations

import numpy as np

from .ripe_oracle import DEEPEST, FULL, RIPE, LogicalCache, layout_code

ELEM_BYTES = {"f32": 4, "bf16": 2}


def ring_width(W: int, t_max: int) -> int:
    return min(max(W, 0), t_max)


def layout_elements(layout, R: int, W: int, B: int, t_max: int, Hkv: int, D: int) -> int:
    """Elements (K and V together) one recurrent layer's cache holds."""
    layout = layout_code(layout)
    if layout == FULL:
        per_seq = R * t_max
    elif layout == DEEPEST:
        per_seq = t_max
    else:
        per_seq = t_max + ring_width(W, t_max) * (R - 1)
    return 2 * B * Hkv * D * per_seq


def layout_bytes(layout, dtype: str, R: int, W: int, B: int, t_max: int, Hkv: int, D: int) -> int:
    return layout_elements(layout, R, W, B, t_max, Hkv, D) * ELEM_BYTES[dtype]


def _to_bytes(x: np.ndarray, dtype: str) -> np.ndarray:
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x32.reshape(-1).view(np.uint8)
    bits = x32.reshape(-1).view(np.uint32)
    finite = ~np.isnan(x32.reshape(-1))
    if np.any(bits[finite] & 0xFFFF):
        raise ValueError("value not representable in bf16")
    return (bits >> 16).astype(np.uint16).view(np.uint8)


def _from_bytes(buf: np.ndarray, dtype: str, n: int) -> np.ndarray:
    if dtype == "f32":
        return buf[: 4 * n].view(np.float32).astype(np.float64)
    u16 = buf[: 2 * n].view(np.uint16).astype(np.uint32)
    return (u16 << 16).view(np.float32).astype(np.float64)


def _blocked_v(v: np.ndarray, width: int) -> np.ndarray:
    """[..., n, D] -> [..., n/width, D, width]."""
    *lead, n, D = v.shape
    v = v.reshape(*lead, n // width, width, D)
    return np.swapaxes(v, -1, -2)


def _unblocked_v(v: np.ndarray) -> np.ndarray:
    """[..., n/width, D, width] -> [..., n, D]."""
    *lead, nb, D, width = v.shape
    return np.swapaxes(v, -1, -2).reshape(*lead, nb * width, D)


def _logical_arrays(cache: LogicalCache):
    """Dense float64 arrays of what each region holds (NaN where nothing)."""
    B, R, T, H, D = cache.B, cache.R, cache.t_max, cache.Hkv, cache.D
    if cache.layout == FULL:
        K = np.full((B, R, H, T, D), np.nan)
        V = np.full((B, R, H, T, D), np.nan)
        for b in range(B):
            for p in range(1, R + 1):
                k, v = cache.dense_plane(b, p)
                K[b, p - 1] = np.moveaxis(k, 0, 1)
                V[b, p - 1] = np.moveaxis(v, 0, 1)
        return [(K, V, 32)]
    deepK = np.full((B, H, T, D), np.nan)
    deepV = np.full((B, H, T, D), np.nan)
    for b in range(B):
        k, v = cache.dense_plane(b, R)
        deepK[b] = np.moveaxis(k, 0, 1)
        deepV[b] = np.moveaxis(v, 0, 1)
    regions = [(deepK, deepV, 32)]
    if cache.layout == RIPE:
        We = ring_width(cache.W, T)
        if We > 0:
            ringK = np.full((B, R - 1, H, We, D), np.nan)
            ringV = np.full((B, R - 1, H, We, D), np.nan)
            filled = np.zeros((B, R - 1, We), dtype=bool)
            for b in range(B):
                for p in range(1, R):
                    for j in cache.held_positions(b, p):
                        s = j % We
                        if filled[b, p - 1, s]:
                            raise ValueError("two held positions share a ring slot")
                        filled[b, p - 1, s] = True
                        k, v = cache.get(b, p, j, j + 1)
                        ringK[b, p - 1, :, s] = k[0]
                        ringV[b, p - 1, :, s] = v[0]
            regions.append((ringK, ringV, min(32, We)))
    return regions


def encode(cache: LogicalCache) -> np.ndarray:
    """The cache's bytes in the ABI layout (uint8 array).  Slots the layout
    does not currently hold are filled with a quiet NaN, so a kernel that
    reads them produces NaN."""
    regions = _logical_arrays(cache)
    k_parts = [_to_bytes(K, cache.dtype) for K, _, _ in regions]
    v_parts = [_to_bytes(_blocked_v(V, w), cache.dtype) for _, V, w in regions]
    out = np.concatenate(k_parts + v_parts)
    expect = layout_bytes(cache.layout, cache.dtype, cache.R, cache.W, cache.B, cache.t_max,
                          cache.Hkv, cache.D)
    assert out.size == expect
    return out


def decode(buf: np.ndarray, layout, dtype: str, R: int, W: int, B: int, t_max: int, Hkv: int,
           D: int, seq_len) -> LogicalCache:
    """Inverse of ``encode`` for the positions the layout holds given the
    committed lengths ``seq_len``."""
    layout = layout_code(layout)
    E = ELEM_BYTES[dtype]
    cache = LogicalCache(layout, dtype, R, W, B, t_max, Hkv, D)
    buf = np.ascontiguousarray(buf, dtype=np.uint8)
    T = t_max
    We = ring_width(W, T) if layout == RIPE else 0
    if layout == FULL:
        shapes = [((B, R, Hkv, T, D), 32)]
    else:
        shapes = [((B, Hkv, T, D), 32)]
        if We > 0:
            shapes.append(((B, R - 1, Hkv, We, D), min(32, We)))
    arrays_k, arrays_v = [], []
    off = 0
    for shp, _ in shapes:
        n = int(np.prod(shp))
        arrays_k.append(_from_bytes(buf[off:off + n * E], dtype, n).reshape(shp))
        off += n * E
    for shp, w in shapes:
        n = int(np.prod(shp))
        *lead, nn, dd = shp
        blocked = _from_bytes(buf[off:off + n * E], dtype, n).reshape(*lead, nn // w, dd, w)
        arrays_v.append(_unblocked_v(blocked))
        off += n * E
    for b in range(B):
        Tb = int(seq_len[b])
        cache.seq_len[b] = Tb
        if layout == FULL:
            K, V = arrays_k[0], arrays_v[0]
            for p in range(1, R + 1):
                cache.put_range(b, p, 0, np.moveaxis(K[b, p - 1, :, :Tb], 0, 1),
                                np.moveaxis(V[b, p - 1, :, :Tb], 0, 1))
            continue
        K, V = arrays_k[0], arrays_v[0]
        cache.put_range(b, R, 0, np.moveaxis(K[b, :, :Tb], 0, 1), np.moveaxis(V[b, :, :Tb], 0, 1))
        if layout == RIPE and We > 0:
            rK, rV = arrays_k[1], arrays_v[1]
            for p in range(1, R):
                for j in range(max(0, Tb - W), Tb):
                    s = j % We
                    cache.put(b, p, j, rK[b, p - 1, :, s], rV[b, p - 1, :, s])
    return cache
