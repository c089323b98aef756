"""Seeded synthetic workloads shaped like the RIPE pages' looped-model caches.

The RIPE abstract (zhuanzhiai.com paper page, opening and second sentences)
describes a looped model whose KV cache keeps one K/V plane per loop of each
recurrent layer, R planes in all, and reports that the planes close in on the
deepest one by a constant factor per loop (0.88 on Huginn, 0.81 on Raven).  The five workloads below restate the
benchmark configurations c1..c5 of this repository; the values are synthetic:

* deepest plane K_R, V_R ~ N(0, 1);
* plane p = plane R + decay**(R - p) * N(0, 1) (noise term times ``tail_mult``
  at a seeded 1% of positions in c2, to mimic heavy-tail error positions);
  with ``convention="pages"`` the noise scale is decay**(p - 1) instead, so
  that the planes approach the deepest one as the loops proceed (plane 1 at
  unit distance, each loop closer by the factor decay);
* draft-row K/V for every depth follow the same model;
* queries ~ N(0, 1) / sqrt(D) with softmax scale 1 (the 1/sqrt(D) folded in).

Every value is rounded to the workload's storage dtype here, so the oracle and
the GPU path consume bit-identical inputs.  Nothing in this module selects
planes, computes attention or lays out bytes.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

ROOT_SEED = 20261203
BLOCK = 32  # positions per independently seeded block of prefix values

__all__ = [
    "ROOT_SEED", "Group", "PlaneModel", "Case", "make_case", "round_to",
    "CONFIG_NAMES", "device_kv_rows",
]

CONFIG_NAMES = ("c1", "c2", "c3", "c4", "c5")


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float values to ``dtype`` ('f32' or 'bf16', nearest-even) and
    return them as float64 so that later float64 arithmetic sees exactly the
    stored values."""
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x32.astype(np.float64)
    if dtype != "bf16":
        raise ValueError(dtype)
    bits = x32.view(np.uint32).astype(np.uint64)
    rounded = (bits + 0x7FFF + ((bits >> 16) & 1)) >> 16
    out = (rounded << 16).astype(np.uint32).view(np.float32)
    return out.astype(np.float64)


@dataclass(frozen=True)
class Group:
    """One draft block or branch: rows [row_start, row_start + n_rows) of the
    query tensor, issued for sequence ``seq`` at loop depth ``depth``.  A
    group verified while its parent block is still in flight names the
    parent's rows (parent_row_start, parent_rows) in the draft tensors."""
    seq: int
    depth: int
    row_start: int
    n_rows: int
    parent_row_start: int = 0
    parent_rows: int = 0


class PlaneModel:
    """Seeded prefix K/V values for every (sequence, plane, position).

    Values are generated per 32-position block from their own seed, so any
    subset of planes and positions can be produced without materialising the
    whole R-plane cache.
    """

    def __init__(self, key: int, R: int, Hkv: int, D: int, decay: float, dtype: str,
                 tail: Optional[dict] = None, tail_mult: float = 1.0, convention: str = "workload"):
        self.key, self.R, self.Hkv, self.D = key, R, Hkv, D
        self.decay, self.dtype = decay, dtype
        self.convention = convention
        self.noise_scale = noise_scale(decay, R, convention)
        self.tail = tail or {}
        self.tail_mult = tail_mult

    def _normal(self, kind: int, b: int, p: int, blk: int) -> np.ndarray:
        ss = np.random.SeedSequence(self.key, spawn_key=(kind, b, p, blk))
        return np.random.default_rng(ss).standard_normal((BLOCK, self.Hkv, self.D))

    def values(self, kind: int, b: int, p: int, j0: int, j1: int) -> np.ndarray:
        """K (kind 0) or V (kind 1) of sequence b, plane p (1..R, R deepest),
        positions [j0, j1): float64 array [j1 - j0, Hkv, D]."""
        if not 1 <= p <= self.R:
            raise ValueError(p)
        out = np.empty((max(j1 - j0, 0), self.Hkv, self.D))
        if j1 <= j0:
            return out
        tail = self.tail.get(b)
        for blk in range(j0 // BLOCK, (j1 - 1) // BLOCK + 1):
            lo, hi = max(j0, blk * BLOCK), min(j1, (blk + 1) * BLOCK)
            base = self._normal(kind, b, 0, blk)
            if p < self.R:
                noise = self._normal(kind, b, p, blk) * self.noise_scale(p)
                if tail is not None:
                    pos = np.arange(blk * BLOCK, (blk + 1) * BLOCK)
                    mult = np.where(np.isin(pos, tail), self.tail_mult, 1.0)
                    noise = noise * mult[:, None, None]
                base = base + noise
            blockv = round_to(base, self.dtype)
            out[lo - j0:hi - j0] = blockv[lo - blk * BLOCK:hi - blk * BLOCK]
        return out


@dataclass
class Case:
    """A seeded workload: cache geometry, committed lengths, draft blocks,
    queries, draft-row K/V for every depth and a commit choice."""
    name: str
    layout: str          # 'full' | 'deepest' | 'ripe'
    dtype: str           # 'f32' | 'bf16'
    R: int
    W: int
    B: int
    t_max: int
    Hkv: int
    Hq: int
    D: int
    L_r: int
    seq_len: np.ndarray  # int64 [B]
    blocks: List[Tuple[int, int]]  # per sequence (row_start, n_rows)
    n_rows: int
    scale: float
    planes: PlaneModel
    q: np.ndarray        # float64 [n_rows, Hq, D]
    kv_new: np.ndarray   # float64 [2, R, n_rows, Hkv, D]
    n_accept: np.ndarray  # int64 [B]
    src_row: np.ndarray   # int64 [B]
    fixed_groups: Optional[List[Group]] = None
    depths: Tuple[int, ...] = field(default_factory=tuple)

    def groups_at(self, r: int, seqs=None) -> List[Group]:
        """One group per sequence (its draft block) at depth r."""
        if self.fixed_groups is not None:
            raise ValueError("this workload has fixed mixed-depth groups")
        seqs = range(self.B) if seqs is None else seqs
        return [Group(b, r, *self.blocks[b]) for b in seqs]

    def groups(self) -> List[Group]:
        if self.fixed_groups is None:
            raise ValueError("use groups_at(r)")
        return list(self.fixed_groups)


def _uniform_lengths(rng, B, lo, hi):
    return rng.integers(lo, hi + 1, size=B).astype(np.int64)


def noise_scale(decay: float, R: int, convention: str = "workload"):
    """Scale of plane p's difference from plane R (p < R): decay**(R - p)
    ("workload": the plane next to the deepest differs most) or
    decay**(p - 1) ("pages": the planes approach the deepest geometrically)."""
    if convention == "workload":
        return lambda p: decay ** (R - p)
    if convention == "pages":
        return lambda p: decay ** (p - 1)
    raise ValueError(convention)


def _draft_kv(key, R, n_rows, Hkv, D, decay, dtype, convention="workload"):
    scale = noise_scale(decay, R, convention)
    rng = np.random.default_rng(np.random.SeedSequence(key, spawn_key=(3,)))
    base = rng.standard_normal((2, n_rows, Hkv, D))
    kv = np.empty((2, R, n_rows, Hkv, D))
    kv[:, R - 1] = round_to(base, dtype)
    for p in range(1, R):
        noise = rng.standard_normal((2, n_rows, Hkv, D))
        kv[:, p - 1] = round_to(base + scale(p) * noise, dtype)
    return kv


def make_case(name: str, layout: Optional[str] = None, *, B: Optional[int] = None,
              T_range: Optional[Tuple[int, int]] = None, t_max: Optional[int] = None,
              W: Optional[int] = None, R: Optional[int] = None, seed_offset: int = 0,
              dtype: Optional[str] = None, k: Optional[int] = None,
              Hkv: Optional[int] = None, Hq: Optional[int] = None,
              D: Optional[int] = None, convention: str = "workload") -> Case:
    """Build workload ``name`` (c1..c5).  Keyword overrides shrink a workload
    for oracle-speed tests while keeping its structure; ``convention`` picks
    the direction of the plane decay (see noise_scale)."""
    idx = CONFIG_NAMES.index(name)
    key = ROOT_SEED + 1 + idx + 1000 * seed_offset
    rng = np.random.default_rng(np.random.SeedSequence(key, spawn_key=(1,)))
    tail = None
    tail_mult = 1.0
    fixed_groups = None
    depths: Tuple[int, ...] = ()
    if name == "c1":
        cfg = dict(layout="ripe", dtype="f32", R=4, W=8, B=1, T=(128, 128), Hkv=4, Hq=4, D=64,
                   L_r=1, k=4, decay=0.88)
        depths = (1, 2, 3, 4)
    elif name == "c2":
        cfg = dict(layout="ripe", dtype="bf16", R=32, W=64, B=1, T=(1024, 1024), Hkv=40, Hq=40,
                   D=128, L_r=4, k=8, decay=0.88)
        depths = (4, 32)
    elif name == "c3":
        cfg = dict(layout="ripe", dtype="bf16", R=32, W=64, B=16, T=(2048, 4096), Hkv=8, Hq=32,
                   D=128, L_r=4, k=8, decay=0.81)
        depths = tuple(range(1, 33))
    elif name == "c4":
        cfg = dict(layout="ripe", dtype="bf16", R=32, W=64, B=16, T=(4096, 4096), Hkv=8, Hq=32,
                   D=128, L_r=4, k=4, decay=0.81)
        depths = (8, 16)
    elif name == "c5":
        full = (layout == "full")
        cfg = dict(layout=layout or "ripe", dtype="bf16", R=32, W=64, B=4 if full else 64,
                   T=(8192, 8192) if full else (4096, 8192), Hkv=8, Hq=32, D=128, L_r=4, k=8,
                   decay=0.81)
        depths = tuple(range(1, 33))
    else:
        raise ValueError(name)
    if layout is not None:
        cfg["layout"] = layout
    for kname, val in (("B", B), ("W", W), ("R", R), ("dtype", dtype), ("k", k), ("Hkv", Hkv),
                       ("Hq", Hq), ("D", D)):
        if val is not None:
            cfg[kname] = val
    if T_range is not None:
        cfg["T"] = T_range
    Rv, Bv, kk = cfg["R"], cfg["B"], cfg["k"]
    depths = tuple(d for d in depths if d <= Rv) or (Rv,)
    seq_len = _uniform_lengths(rng, Bv, *cfg["T"])
    if t_max is None:
        t_max = int(-(-(int(seq_len.max()) + 2 * kk) // 32) * 32)
    if name == "c2":
        tail_mult = 8.0
        tail = {}
        for b in range(Bv):
            trng = np.random.default_rng(np.random.SeedSequence(key, spawn_key=(9, b)))
            n_tail = int(np.floor(0.01 * seq_len[b]))
            tail[b] = np.sort(trng.choice(int(seq_len[b]), size=n_tail, replace=False))
    blocks = []
    n_accept = np.zeros(Bv, dtype=np.int64)
    src_row = np.zeros(Bv, dtype=np.int64)
    if name == "c4":
        # primary branch (k rows at r1) and, for a seeded 40% of sequences, a
        # fallback branch (k rows at r2); each branch is causal within itself.
        r1, r2 = (8, 16) if Rv >= 16 else (max(1, Rv // 4), max(1, Rv // 2))
        fixed_groups = []
        row = 0
        has_fb = rng.random(Bv) < 0.4
        for b in range(Bv):
            fixed_groups.append(Group(b, r1, row, kk))
            blocks.append((row, kk))
            start_fb = row + kk
            row += kk
            if has_fb[b]:
                fixed_groups.append(Group(b, r2, row, kk))
                row += kk
            n_accept[b] = rng.integers(0, kk + 1)
            use_fb = has_fb[b] and rng.random() < 0.5
            src_row[b] = start_fb if use_fb else blocks[b][0]
        n_rows = row
        depths = (r1, r2)
    else:
        for b in range(Bv):
            blocks.append((b * kk, kk))
        n_rows = Bv * kk
        if name == "c1":
            n_accept[:] = 3
        else:
            n_accept[:] = rng.integers(0, kk + 1, size=Bv)
        src_row[:] = [blk[0] for blk in blocks]
    planes = PlaneModel(key, Rv, cfg["Hkv"], cfg["D"], cfg["decay"], cfg["dtype"], tail, tail_mult,
                        convention)
    kv_new = _draft_kv(key, Rv, n_rows, cfg["Hkv"], cfg["D"], cfg["decay"], cfg["dtype"], convention)
    qrng = np.random.default_rng(np.random.SeedSequence(key, spawn_key=(4,)))
    q = round_to(qrng.standard_normal((n_rows, cfg["Hq"], cfg["D"])) / np.sqrt(cfg["D"]),
                 cfg["dtype"])
    return Case(name=name, layout=cfg["layout"], dtype=cfg["dtype"], R=Rv, W=cfg["W"], B=Bv,
                t_max=int(t_max), Hkv=cfg["Hkv"], Hq=cfg["Hq"], D=cfg["D"], L_r=cfg["L_r"],
                seq_len=seq_len, blocks=blocks, n_rows=n_rows, scale=1.0, planes=planes, q=q,
                kv_new=kv_new, n_accept=n_accept, src_row=src_row, fixed_groups=fixed_groups,
                depths=depths)


def device_kv_rows(seed: int, R: int, n: int, Hkv: int, D: int, decay: float, device,
                   torch_dtype=None, planes=None):
    """Draft-row style K/V for ``n`` positions drawn on the device with a seeded
    torch generator: tensor [2, R, n, Hkv, D] in ``torch_dtype``.  Planes not
    listed in ``planes`` (1-based) are left as zeros, to save time when only a
    subset is consumed.  Used to fill large caches through the commit call."""
    import torch
    torch_dtype = torch_dtype or torch.bfloat16
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    base = torch.randn((2, n, Hkv, D), generator=gen, device=device, dtype=torch.float32)
    out = torch.zeros((2, R, n, Hkv, D), device=device, dtype=torch_dtype)
    want = set(range(1, R + 1)) if planes is None else set(planes)
    for p in range(1, R + 1):
        noise = torch.randn((2, n, Hkv, D), generator=gen, device=device, dtype=torch.float32)
        if p not in want:
            continue
        if p == R:
            out[:, p - 1] = base.to(torch_dtype)
        else:
            out[:, p - 1] = (base + (decay ** (R - p)) * noise).to(torch_dtype)
    return out
