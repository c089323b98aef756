"""Byte layout of one recurrent layer's cache -- TEST INFRASTRUCTURE ONLY.

An independent NumPy statement of the cache byte layout that the C ABI
declares, used to build device buffers for parity tests and to compare the
buffers the commit kernel writes, byte for byte.  It shares no code with the
library (which computes addresses in C++).

Layout (E = element bytes, T = t_max, a multiple of 32; We = min(W, T));
the K region comes first, then the V region:

* FULL     K [B][R][Hkv][T][D]              V [B][R][Hkv][T/8][D][8]
* DEEPEST  K [B][Hkv][T][D]                 V [B][Hkv][T/8][D][8]
* RIPE     K deep [B][Hkv][T][D]            V deep [B][Hkv][T/8][D][8]
             then ring [B][R-1][Hkv][We][D]   then ring [B][R-1][Hkv][We*D] (below)

V is stored transposed in blocks of V_BLOCK = 8 positions (each head
dimension's 8 values contiguous).  A ring's V of one (sequence, plane, head)
holds its We slots as floor(We/8) such blocks [D][8] followed, when We is
not a multiple of 8, by one narrower block [D][We mod 8] (``ring_v_offset``).
Plane p is stored at index p - 1 (plane R deepest); RIPE keeps position j's
planes 1..R-1 in ring slot j mod We.

Paged caches (page length P, N pages): the main region becomes a pool,
K [N][planes][Hkv][P][D] and V [N][planes][Hkv][P/8][D][8] (planes = R for
FULL, the plane index dropped otherwise), and block k of sequence b
(positions [kP, kP + P)) lives in page table[b][k]; the RIPE ring stays one
per sequence.  encode_paged builds it by moving each block of the unpaged
encoding to its page.

The memory model follows the RIPE abstract (zhuanzhiai.com paper page):
one shared plane costs T positions per sequence, the full cache R*T, RIPE
T + W*(R-1).
"""
from __future__ import annotations

import numpy as np

from .ripe_oracle import DEEPEST, FULL, RIPE, LogicalCache, layout_code

ELEM_BYTES = {"f32": 4, "bf16": 2}
V_BLOCK = 8  # positions per transposed V block


def ring_width(W: int, t_max: int) -> int:
    return min(max(W, 0), t_max)


def ring_v_offset(slot: int, d: int, We: int, D: int) -> int:
    """Element offset of V (ring slot, head dimension d) within one
    (sequence, plane, head) ring of We slots: blocks of V_BLOCK slots stored
    [D][V_BLOCK], the last We mod V_BLOCK slots as one block
    [D][We mod V_BLOCK]."""
    if not (0 <= slot < We and 0 <= d < D):
        raise IndexError((slot, d))
    n = V_BLOCK
    full = (We // n) * n
    if slot < full:
        return (slot // n) * n * D + d * n + slot % n
    w = We - full
    return full * D + d * w + (slot - full)


def ring_v_offsets(We: int, D: int) -> np.ndarray:
    """ring_v_offset for every (slot, d): int array [We, D]."""
    return np.array([[ring_v_offset(s, d, We, D) for d in range(D)] for s in range(We)], dtype=np.int64)


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


def _region_views(buf_elems: np.ndarray, layout, R: int, W: int, B: int, t_max: int, Hkv: int,
                  D: int):
    """Named array views of a flat element buffer: K and V of the main region
    (FULL planes or the deep plane) and, for RIPE, of the ring.  Main V views
    are blocked [..., n/V_BLOCK, D, V_BLOCK]; the ring V view is [B, R-1, Hkv, We*D],
    indexed through ring_v_offsets."""
    layout = layout_code(layout)
    T = t_max
    if layout == FULL:
        main = (B, R, Hkv, T, D)
    else:
        main = (B, Hkv, T, D)
    We = ring_width(W, T) if layout == RIPE else 0
    parts = [("main", main, V_BLOCK)]
    if We > 0:
        parts.append(("ring", (B, R - 1, Hkv, We, D), None))
    views = {}
    off = 0
    for kind in ("K", "V"):
        for name, shp, w in parts:
            n = int(np.prod(shp))
            flat = buf_elems[off:off + n]
            if kind == "K":
                views[(kind, name)] = flat.reshape(shp)
            elif w is None:
                views[(kind, name)] = flat.reshape(*shp[:3], shp[3] * shp[4])
            else:
                *lead, nn, dd = shp
                views[(kind, name)] = flat.reshape(*lead, nn // w, dd, w)
            off += n
    assert off == buf_elems.size
    return views


def _bits(x: np.ndarray, dtype: str) -> np.ndarray:
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x32.view(np.uint32)
    bits = x32.view(np.uint32)
    finite = ~np.isnan(x32)
    if np.any(bits[finite] & 0xFFFF):
        raise ValueError("value not representable in bf16")
    return (bits >> 16).astype(np.uint16)


def encode(cache: LogicalCache) -> np.ndarray:
    """The cache's bytes in the ABI layout (uint8 array).  Slots the layout
    does not currently hold are filled with a quiet NaN, so a kernel that
    reads them produces NaN."""
    B, R, T, H, D = cache.B, cache.R, cache.t_max, cache.Hkv, cache.D
    n = layout_elements(cache.layout, R, cache.W, B, T, H, D)
    if cache.dtype == "f32":
        buf = np.full(n, 0x7FC00000, dtype=np.uint32)
    else:
        buf = np.full(n, 0x7FC0, dtype=np.uint16)
    views = _region_views(buf, cache.layout, R, cache.W, B, T, H, D)
    kmain, vmain = views[("K", "main")], views[("V", "main")]
    main_planes = range(1, R + 1) if cache.layout == FULL else [R]
    for b in range(B):
        for p in main_planes:
            if (b, p) not in cache._dense:
                continue
            k, v, held = cache._dense[(b, p)]
            kt = np.moveaxis(k, 0, 1)          # [H, T, D]
            vt = np.moveaxis(v, 0, 1)
            kd = kmain[b, p - 1] if cache.layout == FULL else kmain[b]
            vd = vmain[b, p - 1] if cache.layout == FULL else vmain[b]
            kd[:, held] = _bits(kt[:, held], cache.dtype)
            vblk = _bits(np.swapaxes(vt.reshape(H, T // V_BLOCK, V_BLOCK, D), -1, -2), cache.dtype)
            hb = held.reshape(T // V_BLOCK, V_BLOCK)
            vd[...] = np.where(hb[None, :, None, :], vblk, vd)
    if cache.layout == RIPE and ("K", "ring") in views:
        We = ring_width(cache.W, T)
        voff = ring_v_offsets(We, D)
        kring, vring = views[("K", "ring")], views[("V", "ring")]
        filled = np.zeros((B, R - 1, We), dtype=bool)
        for (b, p), store in cache._sparse.items():
            for j, (k, v) in store.items():
                s = j % We
                if filled[b, p - 1, s]:
                    raise ValueError("two held positions share a ring slot")
                filled[b, p - 1, s] = True
                kring[b, p - 1, :, s] = _bits(k, cache.dtype)
                vring[b, p - 1][:, voff[s]] = _bits(v, cache.dtype)
    return buf.view(np.uint8)


def decode(buf: np.ndarray, layout, dtype: str, R: int, W: int, B: int, t_max: int, Hkv: int,
           D: int, seq_len) -> LogicalCache:
    """Inverse of ``encode`` for the positions the layout holds given the
    committed lengths ``seq_len``."""
    layout = layout_code(layout)
    cache = LogicalCache(layout, dtype, R, W, B, t_max, Hkv, D)
    raw = np.ascontiguousarray(buf, dtype=np.uint8)
    elems = raw.view(np.uint32 if dtype == "f32" else np.uint16)
    views = _region_views(elems, layout, R, W, B, t_max, Hkv, D)

    def val(x):
        if dtype == "f32":
            return np.ascontiguousarray(x).view(np.float32).astype(np.float64)
        return (np.asarray(x, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)

    T = t_max
    kmain, vmain = views[("K", "main")], views[("V", "main")]
    for b in range(B):
        Tb = int(seq_len[b])
        cache.seq_len[b] = Tb
        planes = range(1, R + 1) if layout == FULL else [R]
        for p in planes:
            kd = kmain[b, p - 1] if layout == FULL else kmain[b]          # [H, T, D]
            vd = vmain[b, p - 1] if layout == FULL else vmain[b]          # [H, T/8, D, 8]
            k = np.moveaxis(val(kd[:, :Tb]), 0, 1)
            v = np.moveaxis(np.swapaxes(val(vd), -1, -2).reshape(Hkv, T, D)[:, :Tb], 0, 1)
            cache.put_range(b, p, 0, k, v)
        if layout == RIPE and ("K", "ring") in views:
            We = ring_width(W, T)
            voff = ring_v_offsets(We, D)
            kring, vring = views[("K", "ring")], views[("V", "ring")]
            for p in range(1, R):
                for j in range(max(0, Tb - W), Tb):
                    s = j % We
                    cache.put(b, p, j, val(kring[b, p - 1, :, s]),
                              val(vring[b, p - 1][:, voff[s]]))
    return cache


def paged_layout_elements(layout, R: int, W: int, B: int, t_max: int, Hkv: int, D: int, page_len: int,
                          n_pages: int) -> int:
    """Elements (K and V together) of a paged cache."""
    layout = layout_code(layout)
    planes = R if layout == FULL else 1
    ring = B * ring_width(W, t_max) * (R - 1) if layout == RIPE else 0
    return 2 * Hkv * D * (n_pages * page_len * planes + ring)


def _pool_views(elems: np.ndarray, layout, R: int, W: int, B: int, t_max: int, Hkv: int, D: int, P: int, N: int):
    """K/V views of a paged buffer: pools [N, planes, H, P, D] and
    [N, planes, H, P/8, D, 8] (planes = 1 unless FULL), rings as unpaged."""
    layout = layout_code(layout)
    planes = R if layout == FULL else 1
    We = ring_width(W, t_max) if layout == RIPE else 0
    pool = (N, planes, Hkv, P, D)
    ring = (B, R - 1, Hkv, We, D)
    n_pool, n_ring = int(np.prod(pool)), (int(np.prod(ring)) if We > 0 else 0)
    views, off = {}, 0
    for kind in ("K", "V"):
        views[(kind, "pool")] = elems[off:off + n_pool].reshape(pool) if kind == "K" else \
            elems[off:off + n_pool].reshape(N, planes, Hkv, P // V_BLOCK, D, V_BLOCK)
        off += n_pool
        if We > 0:
            flat = elems[off:off + n_ring]
            views[(kind, "ring")] = flat.reshape(ring) if kind == "K" else \
                flat.reshape(B, R - 1, Hkv, We * D)
            off += n_ring
    assert off == elems.size
    return views


def encode_paged(cache: LogicalCache, table, page_len: int, n_pages: int) -> np.ndarray:
    """Bytes of the paged layout: the unpaged encoding's main-region block k
    of sequence b moved to page table[b][k] (negative entries: block not
    stored), the ring unchanged.  Two blocks mapped to one page must agree
    wherever both hold a value (ValueError otherwise); page slots no block
    holds are quiet NaNs."""
    B, R, T, H, D, P, N = cache.B, cache.R, cache.t_max, cache.Hkv, cache.D, page_len, n_pages
    if P <= 0 or T % P or P % 32:
        raise ValueError("page length")
    table = np.asarray(table).reshape(B, T // P)
    flat = encode(cache).view(np.uint32 if cache.dtype == "f32" else np.uint16)
    src = _region_views(flat, cache.layout, R, cache.W, B, T, H, D)
    n = paged_layout_elements(cache.layout, R, cache.W, B, T, H, D, P, N)
    nan = 0x7FC00000 if cache.dtype == "f32" else 0x7FC0
    out = np.full(n, nan, dtype=flat.dtype)
    dst = _pool_views(out, cache.layout, R, cache.W, B, T, H, D, P, N)
    written = np.zeros((N, R if cache.layout == FULL else 1, P), dtype=bool)
    main_planes = list(range(1, R + 1)) if cache.layout == FULL else [R]
    for b in range(B):
        for k in range(T // P):
            pg = int(table[b, k])
            if pg < 0:
                continue
            if pg >= N:
                raise ValueError("page out of range")
            for pi, p in enumerate(main_planes):
                if (b, p) not in cache._dense:
                    continue
                held = cache._dense[(b, p)][2][k * P:(k + 1) * P]
                ks = src[("K", "main")][b, p - 1] if cache.layout == FULL else src[("K", "main")][b]
                vs = src[("V", "main")][b, p - 1] if cache.layout == FULL else src[("V", "main")][b]
                kblk = ks[:, k * P:(k + 1) * P]                        # [H, P, D]
                vblk = vs[:, k * P // V_BLOCK:(k + 1) * P // V_BLOCK]  # [H, P/8, D, 8]
                kd, vd = dst[("K", "pool")][pg, pi], dst[("V", "pool")][pg, pi]
                both = held & written[pg, pi]
                vmask = held.reshape(P // V_BLOCK, V_BLOCK)
                if both.any():
                    bv = both.reshape(P // V_BLOCK, V_BLOCK)
                    if not (np.array_equal(kd[:, both], kblk[:, both]) and
                            np.array_equal(np.where(bv[None, :, None, :], vd, 0),
                                           np.where(bv[None, :, None, :], vblk, 0))):
                        raise ValueError(f"page {pg} shared with different contents")
                kd[:, held] = kblk[:, held]
                vd[...] = np.where(vmask[None, :, None, :], vblk, vd)
                written[pg, pi] |= held
    if ("K", "ring") in src:
        dst[("K", "ring")][...] = src[("K", "ring")]
        dst[("V", "ring")][...] = src[("V", "ring")]
    return out.view(np.uint8)


def decode_paged(buf: np.ndarray, layout, dtype: str, R: int, W: int, B: int, t_max: int, Hkv: int, D: int,
                 seq_len, table, page_len: int, n_pages: int) -> LogicalCache:
    """Inverse of encode_paged for the committed positions: the blocks are
    gathered back to the unpaged layout, which decode reads."""
    P, N, T = page_len, n_pages, t_max
    table = np.asarray(table).reshape(B, T // P)
    elems = np.ascontiguousarray(buf, dtype=np.uint8).view(np.uint32 if dtype == "f32" else np.uint16)
    src = _pool_views(elems, layout, R, W, B, T, Hkv, D, P, N)
    flat = np.full(layout_elements(layout, R, W, B, T, Hkv, D), 0x7FC00000 if dtype == "f32" else 0x7FC0,
                   dtype=elems.dtype)
    dst = _region_views(flat, layout, R, W, B, T, Hkv, D)
    full = layout_code(layout) == FULL
    for b in range(B):
        for k in range(T // P):
            if k * P >= int(seq_len[b]):
                break
            pg = int(table[b, k])
            for pi in range(R if full else 1):
                kd = dst[("K", "main")][b, pi] if full else dst[("K", "main")][b]
                vd = dst[("V", "main")][b, pi] if full else dst[("V", "main")][b]
                kd[:, k * P:(k + 1) * P] = src[("K", "pool")][pg, pi]
                vd[:, k * P // V_BLOCK:(k + 1) * P // V_BLOCK] = src[("V", "pool")][pg, pi]
    if ("K", "ring") in src:
        dst[("K", "ring")][...] = src[("K", "ring")]
        dst[("V", "ring")][...] = src[("V", "ring")]
    return decode(flat.view(np.uint8), layout, dtype, R, W, B, T, Hkv, D, seq_len)
