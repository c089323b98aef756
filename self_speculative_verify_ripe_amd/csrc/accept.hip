// accept.hip -- accept / rollback after verification, for gfx950.
//
// What is computed (LoopSpec summary, rit.work blog, section on the second
// branch; RIPE abstract, zhuanzhiai.com paper page): per sequence, the
// primary draft chain is checked against the depth-R target distributions;
// if its first token is rejected and a fallback chain exists (drawn from the
// residual of a deeper state's distribution after the first proposal), the
// fallback is checked against the residual target; after two rejections
// decoding restarts.  Greedy checks keep the target's arg max; speculative
// sampling keeps each output's probability under ordinary decoding.  The
// rules are spelled out beside the declaration of ripe_accept.
//
// How: four launches (two for greedy calls).  The per-index work is spread
// over (sequence, slice of the vocabulary) work-groups; the decisions run on
// one work-group per sequence, or again in every work-group of a sweep that
// needs them, which costs less than a launch of their own.
//   accept_stats_kernel     per (row, slice): arg max (lowest index on ties),
//                           max, and sum exp((z - max) / tau) (a table-driven
//                           exp, below); rows no decision can read are skipped
//   accept_decide_kernel    per sequence: combines the slices into each row's
//                           statistics; greedy decisions (final), or the
//                           primary chain's speculative tests; and, sampling,
//                           per (sequence with a fallback, quarter slice) the
//                           fallback's residual masses, before the tests say
//                           whether they are needed
//   accept_drawsum_kernel   per (sequence, quarter slice): the fallback's tests
//                           where the primary's first token was rejected, then
//                           sums of the final draw's weights over tiles of 64
//                           indices
//   accept_pick_kernel      per sequence: the part, then the tile, then the index
//                           where the running sum crosses u * total
// Probabilities, sums and decisions are in double; the logits are float.
// Sums run in a fixed order for a given vocabulary size, so repeated calls
// give the same result.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "accept.h"

namespace ripe {

constexpr int kAcceptThreads = 256;

// Row numbering within a sequence: target rows of chain c at c * (k+1) + i,
// draft rows at 2 (k+1) + c k + i.
__device__ inline int target_row(int k, int c, int i) { return c * (k + 1) + i; }
__device__ inline int draft_row(int k, int c, int i) { return 2 * (k + 1) + c * k + i; }

__device__ inline const float* row_ptr(const AcceptParams& p, int b, int r) {
  const int k = p.k;
  if (r < 2 * (k + 1)) return p.target + (size_t(b) * 2 * (k + 1) + r) * p.V;
  return p.draft + (size_t(b) * 2 * k + (r - 2 * (k + 1))) * p.V;
}

// Loads per thread issued together by the per-index loops, so that each
// thread has several reads in flight instead of waiting on every element.
constexpr int kLoadBatch = 8;
// Logits per thread the row statistics keep in registers: a slice of up to
// kHeld * 256 indices (every slice up to a 256K vocabulary) is read once.
constexpr int kHeld = kAcceptSliceMin / kAcceptThreads;

// z[t] for t < t1, else `other`.  The load itself is unconditional, from
// index min(t, t1 - 1) (callers have t1 > 0), so the compiler keeps the
// batch's loads together instead of branching around each one.
__device__ inline float load_or(const float* z, int t, int t1, float other) {
  const float v = z[min(t, t1 - 1)];
  return t < t1 ? v : other;
}

// ---------------------------------------------------------------------------
// work-group reductions (256 threads = 4 wavefronts)
// ---------------------------------------------------------------------------
__device__ inline void better(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) { v = v2; i = i2; }
}

__device__ inline void wg_argmax(float& v, int& i) {
  __shared__ float sv[kAcceptThreads / 64];
  __shared__ int si[kAcceptThreads / 64];
  for (int off = 32; off > 0; off >>= 1) {
    const float v2 = __shfl_xor(v, off);
    const int i2 = __shfl_xor(i, off);
    better(v, i, v2, i2);
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { sv[w] = v; si[w] = i; }
  __syncthreads();
  v = sv[0];
  i = si[0];
  for (int x = 1; x < kAcceptThreads / 64; ++x) better(v, i, sv[x], si[x]);
  __syncthreads();
}

// Sum over the work-group in a fixed order (lanes by xor tree, then wavefronts).
__device__ inline double wg_sum(double x) {
  __shared__ double s[kAcceptThreads / 64];
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) s[w] = x;
  __syncthreads();
  double t = 0.0;
  for (int x2 = 0; x2 < kAcceptThreads / 64; ++x2) t += s[x2];
  __syncthreads();
  return t;
}

// ---------------------------------------------------------------------------
// decisions and draws
// ---------------------------------------------------------------------------
struct Dist {           // softmax of one row: exp((z - M) * inv_tau) / S
  const float* z;
  double M, S;
};

__device__ inline double prob_of(const Dist& d, double inv_tau, float z) {
  return exp((double(z) - d.M) * inv_tau) / d.S;
}

// The weights a final draw uses, as a function of the index.  With the
// fallback's residual target r(t) = max(0, a - c) / Wr (a itself when Wr = 0)
// and its draft distribution q'(t) = max(0, m - c) / Wm (0 when Wm = 0):
//   kDrawRow       a(t)                      (a bonus token)
//   kDrawResidual  max(0, a(t) - c(t))       (a rejection inside a chain)
//   kDrawFallbackR r(t)
//   kDrawRestart   max(0, r(t) - q'(t))      (both first tokens rejected)
enum DrawKind { kDrawRow = 0, kDrawResidual = 1, kDrawFallbackR = 2, kDrawRestart = 3 };

struct DrawSpec {
  int kind;
  Dist a, c, m;
  double Wr, Wm;
};

enum Stage { kStageDone = 0, kStageFallback = 1, kStageDraw = 2 };

// The weight of one index from its logits in rows a, c and m (rows a kind
// does not use alias a, so every load is valid).
__device__ inline double weight_of(const DrawSpec& s, double inv_tau, float za, float zc, float zm) {
  switch (s.kind) {
    case kDrawRow: return prob_of(s.a, inv_tau, za);
    case kDrawResidual: return fmax(prob_of(s.a, inv_tau, za) - prob_of(s.c, inv_tau, zc), 0.0);
    case kDrawFallbackR: {
      const double pa = prob_of(s.a, inv_tau, za);
      return s.Wr > 0.0 ? fmax(pa - prob_of(s.c, inv_tau, zc), 0.0) / s.Wr : pa;
    }
    default: {  // kDrawRestart: max(0, r - q'), with c's probability computed once
      const double pa = prob_of(s.a, inv_tau, za), pc = prob_of(s.c, inv_tau, zc);
      const double r = s.Wr > 0.0 ? fmax(pa - pc, 0.0) / s.Wr : pa;
      const double q = s.Wm > 0.0 ? fmax(prob_of(s.m, inv_tau, zm) - pc, 0.0) / s.Wm : 0.0;
      return fmax(r - q, 0.0);
    }
  }
}

__device__ inline double weight(const DrawSpec& s, double inv_tau, int t) {
  return weight_of(s, inv_tau, s.a.z[t], s.c.z[t], s.m.z[t]);
}

// First index whose running sum of weights exceeds u * total; the last index
// with weight > 0 when rounding leaves none.  Returns -1 if the total is 0.
// Running sums are taken over tiles of 64 consecutive indices: wavefront w
// owns tiles w, w + 4, ... and reduces each tile with a shuffle tree (reads
// stay coalesced); a scan over the tile sums in index order finds the tile
// where the sum crosses u * total, and one wavefront scans that tile.
constexpr int kTile = 64;
constexpr int kLdsTiles = 2048;               // tile sums kept in LDS per round

__device__ inline double wave_sum(double x) {
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// Inclusive prefix sum over the 64 lanes (lane order).
__device__ inline double wave_inclusive_scan(double x) {
  const int lane = threadIdx.x & 63;
  for (int off = 1; off < 64; off <<= 1) {
    const double y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

__device__ int wg_draw(const DrawSpec& s, double inv_tau, int V, double u) {
  __shared__ double tile_sum[kLdsTiles];
  __shared__ double s_base;
  __shared__ int s_tile;
  __shared__ int s_last;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n_tiles = (V + kTile - 1) / kTile;
  // total weight and the last index with weight > 0
  double part = 0.0;
  int last = -1;
  for (int t = threadIdx.x; t < V; t += kAcceptThreads) {
    const double w = weight(s, inv_tau, t);
    part += w;
    if (w > 0.0) last = t;
  }
  const double total = wg_sum(part);
  if (!(total > 0.0)) return -1;
  const double target = u * total;
  if (threadIdx.x == 0) { s_last = -1; s_tile = -1; s_base = 0.0; }
  __syncthreads();
  atomicMax(&s_last, last);
  // rounds of up to kLdsTiles tiles: tile sums, then a serial walk over them
  double base = 0.0;  // running sum before the round's first tile
  for (int r0 = 0; r0 < n_tiles; r0 += kLdsTiles) {
    const int r1 = min(n_tiles, r0 + kLdsTiles);
    for (int tile = r0 + wave; tile < r1; tile += kAcceptThreads / 64) {
      const int t = tile * kTile + lane;
      const double w = t < V ? weight(s, inv_tau, t) : 0.0;
      const double ts = wave_sum(w);
      if (lane == 0) tile_sum[tile - r0] = ts;
    }
    __syncthreads();
    if (wave == 0) {
      // walk the tile sums 64 at a time in index order
      double run = base;
      int hit = -1;
      for (int i0 = 0; i0 < r1 - r0; i0 += 64) {
        const bool in = i0 + lane < r1 - r0;
        const double ts = in ? tile_sum[i0 + lane] : 0.0;
        const double incl = wave_inclusive_scan(ts);
        const unsigned long long over = __ballot(in && run + incl > target);
        if (over != 0ull) {
          const int l = __ffsll(static_cast<long long>(over)) - 1;
          hit = r0 + i0 + l;
          run += __shfl(incl - ts, l);  // running sum before the crossing tile
          break;
        }
        run += __shfl(incl, 63);
      }
      if (lane == 0) { s_tile = hit; s_base = run; }
    }
    __syncthreads();
    base = s_base;
    if (s_tile >= 0) break;
    __syncthreads();
  }
  int result = s_last;
  const int hit_tile = s_tile;
  if (hit_tile >= 0) {
    // wavefront 0 scans the crossing tile
    __shared__ int s_idx;
    if (threadIdx.x == 0) s_idx = -1;
    __syncthreads();
    if (wave == 0) {
      const int t = hit_tile * kTile + lane;
      const double w = t < V ? weight(s, inv_tau, t) : 0.0;
      const double run = base + wave_inclusive_scan(w);
      const unsigned long long over = __ballot(run > target && t < V);
      if (lane == 0 && over != 0ull) s_idx = hit_tile * kTile + __ffsll(static_cast<long long>(over)) - 1;
    }
    __syncthreads();
    if (s_idx >= 0) result = s_idx;
  }
  __syncthreads();
  return result;
}

__device__ inline bool in_vocab(int t, int V) { return t >= 0 && t < V; }



// The rows a, c, m of a state, with the statistics it carries.
__device__ inline Dist dist_in(const AcceptParams& p, int b, const SeqState& s, int w) {
  return Dist{row_ptr(p, b, w == 0 ? s.ra : (w == 1 ? s.rc : s.rm)), double(s.M[w]), s.S[w]};
}

// Copy the statistics of rows ra, rc, rm into the state (rows a state's kind
// does not use are copied too and never read).
__device__ inline void carry_rows(SeqState& s, const RowStat* st) {
  const int r[3] = {s.ra, s.rc, s.rm};
  for (int w = 0; w < 3; ++w) {
    s.S[w] = st[r[w]].S;
    s.M[w] = st[r[w]].M;
  }
}

__device__ inline DrawSpec spec_of(const AcceptParams& p, int b, const SeqState& s) {
  DrawSpec d;
  d.kind = s.kind;
  d.a = dist_in(p, b, s, 0);
  d.c = s.kind == kDrawRow ? d.a : dist_in(p, b, s, 1);
  d.m = (s.kind == kDrawRestart || s.kind == kDrawFallbackR) ? dist_in(p, b, s, 2) : d.a;
  d.Wr = s.Wr;
  d.Wm = s.Wm;
  return d;
}

// rows no decision can read: the fallback's target row 0 (position 0 is
// scored by the primary's row 0), fallback rows without a fallback, and draft
// rows in greedy mode
__device__ inline bool row_unused(const AcceptParams& p, int r, bool fb) {
  const int k = p.k;
  const bool is_draft = r >= 2 * (k + 1);
  const int chain = is_draft ? (r - 2 * (k + 1)) / k : r / (k + 1);
  return r == target_row(k, 1, 0) || (chain == 1 && !fb) || (is_draft && p.greedy);
}

// ---------------------------------------------------------------------------
// e^x for the row statistics
// ---------------------------------------------------------------------------
// One exp per logit is most of the row statistics' time, which the
// double-precision pipes bound, not memory: at a 64K vocabulary (12.6 M
// logits) the kernel took 27.6 us with the library's exp and 17.3 us with
// the exp taken out; the table below brings it to about 24 us.  With
// N = rint(256 x / ln 2) = 256 n + j (0 <= j < 256), r = x - N ln 2 / 256
// is taken in two steps (Cody and Waite's reduction: ln 2 / 256 split into a
// head of 32 significant bits, so that N * head is exact, and the double
// nearest the rest), and e^x = 2^n 2^(j/256) e^r: 2^(j/256) from a table
// that each work-group fills in LDS with the library's exp2, e^r from its
// Taylor series to degree 4 (|r| <= ln 2 / 512, so the truncation is below
// 4e-17 relative), the power of two applied with ldexp, which also rounds
// results below the normal range correctly.  About 12 double operations and
// one LDS read per logit, against about 25 for the library's exp, within 2
// units in the last place of it; x = 0 gives exactly 1.  x < -746 (e^x below
// half the smallest subnormal) and x = -inf give 0; NaN stays NaN.
constexpr int kExpTable = 256;
constexpr double kLn2Head = 0x1.62e42feep-1;         // ln 2 to 32 significant bits
constexpr double kLn2Rest = 1.9082149292705877e-10;  // ln 2 - kLn2Head, to double
constexpr double kTableScale = 369.3299304675746;     // 256 / ln 2, to double

__device__ inline void fill_exp_table(double* t) {  // every thread of the work-group, then a barrier
  for (int j = threadIdx.x; j < kExpTable; j += kAcceptThreads) t[j] = exp2(double(j) / kExpTable);
  __syncthreads();
}

__device__ inline double exp_tab(const double* t, double x) {
  if (!(x >= -746.0)) return x != x ? x : 0.0;
  const double nd = rint(x * kTableScale);
  const int n = int(nd);
  const double r = fma(-nd, kLn2Rest / kExpTable, fma(-nd, kLn2Head / kExpTable, x));
  const double e = fma(fma(fma(fma(r, 1.0 / 24.0, 1.0 / 6.0), r, 0.5), r, 1.0), r, 1.0);
  return ldexp(t[n & (kExpTable - 1)] * e, n >> 8);
}

// ---------------------------------------------------------------------------
// 1. row statistics per slice
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kAcceptThreads) void accept_stats_kernel(const AcceptParams p) {
  const int rows = 4 * p.k + 2;
  const int sl = blockIdx.x % p.split;
  const int br = blockIdx.x / p.split;
  const int b = br / rows, r = br % rows;
  if (row_unused(p, r, p.has_fb[b] != 0)) return;
  const float* z = row_ptr(p, b, r);
  const int t0 = sl * p.slice;
  const int t1 = min(p.V, t0 + p.slice);
  float mv = -INFINITY;
  int mi = 0x7fffffff;
  double s = 0.0;
  const bool sum = !p.greedy;
  __shared__ double etab[kExpTable];
  if (sum) fill_exp_table(etab);
  if (t1 - t0 <= kHeld * kAcceptThreads) {
    // the whole slice in registers: one read of the logits serves both passes
    float zv[kHeld];
#pragma unroll
    for (int j = 0; j < kHeld; ++j) zv[j] = load_or(z, t0 + threadIdx.x + j * kAcceptThreads, t1, -INFINITY);
#pragma unroll
    for (int j = 0; j < kHeld; ++j)
      if (t0 + int(threadIdx.x) + j * kAcceptThreads < t1) better(mv, mi, zv[j], t0 + threadIdx.x + j * kAcceptThreads);
    wg_argmax(mv, mi);
    if (sum && mv > -INFINITY) {
      const double M = mv;
#pragma unroll
      for (int j = 0; j < kHeld; ++j)
        if (t0 + int(threadIdx.x) + j * kAcceptThreads < t1) s += exp_tab(etab, (double(zv[j]) - M) * p.inv_tau);
      s = wg_sum(s);
    }
  } else {
    // longer slices: kLoadBatch loads in flight per thread, the slice read twice
    for (int t = t0 + threadIdx.x; t < t1; t += kLoadBatch * kAcceptThreads) {
      float zv[kLoadBatch];
#pragma unroll
      for (int j = 0; j < kLoadBatch; ++j) zv[j] = load_or(z, t + j * kAcceptThreads, t1, -INFINITY);
#pragma unroll
      for (int j = 0; j < kLoadBatch; ++j)
        if (t + j * kAcceptThreads < t1) better(mv, mi, zv[j], t + j * kAcceptThreads);
    }
    wg_argmax(mv, mi);
    if (sum && mv > -INFINITY) {
      const double M = mv;
      for (int t = t0 + threadIdx.x; t < t1; t += kLoadBatch * kAcceptThreads) {
        float zv[kLoadBatch];
#pragma unroll
        for (int j = 0; j < kLoadBatch; ++j) zv[j] = load_or(z, t + j * kAcceptThreads, t1, 0.f);
#pragma unroll
        for (int j = 0; j < kLoadBatch; ++j)
          if (t + j * kAcceptThreads < t1) s += exp_tab(etab, (double(zv[j]) - M) * p.inv_tau);
      }
      s = wg_sum(s);
    }
  }
  if (threadIdx.x == 0) p.part[size_t(br) * p.split + sl] = RowStat{s, mv, mi};
}

// ---------------------------------------------------------------------------
// 2. row statistics, greedy decisions, the primary chain's tests
// ---------------------------------------------------------------------------
constexpr int kMaxRows = 4 * 64 + 2;  // rows of one sequence at the largest k
constexpr int kWaves = kAcceptThreads / 64;
constexpr int kRowBatch = 4;          // rows whose slice statistics one wavefront loads together

// One row's statistics from its slices', across a wavefront (lane i holds
// slice i; lanes past the slices hold {0, -inf, INT_MAX}); every lane
// returns them.
__device__ inline RowStat combine_one(const AcceptParams& p, const RowStat& st) {
  float M = st.M;
  int arg = st.arg;
  for (int off = 32; off > 0; off >>= 1) {  // better() is a total order: every lane ends equal
    const float M2 = __shfl_xor(M, off);
    const int a2 = __shfl_xor(arg, off);
    better(M, arg, M2, a2);
  }
  double S = 0.0;
  if (!p.greedy) S = wave_sum(st.M > -INFINITY ? st.S * exp((double(st.M) - double(M)) * p.inv_tau) : 0.0);
  return RowStat{S, M, arg};
}

// The sequence's row statistics into out[rows] (LDS), for every row a
// decision can read: the max and lowest arg max over the slices, and
// S = sum_i S_i exp((M_i - M) / tau) by a fixed xor tree over the slices.
// Lane i holds slice i (split <= 64); wavefront w takes rows w, w + kWaves, ...
__device__ void combine_rows(const AcceptParams& p, int b, bool fb, RowStat* out) {
  const int rows = 4 * p.k + 2, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const RowStat* base = p.part + size_t(b) * rows * p.split;
  for (int r0 = wave; r0 < rows; r0 += kRowBatch * kWaves) {
    RowStat st[kRowBatch];
#pragma unroll
    for (int j = 0; j < kRowBatch; ++j) {
      const int r = r0 + j * kWaves;
      const bool use = r < rows && lane < p.split && !row_unused(p, r, fb);
      st[j] = use ? base[size_t(r) * p.split + lane] : RowStat{0.0, -INFINITY, 0x7fffffff};
    }
#pragma unroll
    for (int j = 0; j < kRowBatch; ++j) {
      const int r = r0 + j * kWaves;
      if (r >= rows || row_unused(p, r, fb)) continue;  // the same for the whole wavefront
      const RowStat c = combine_one(p, st[j]);
      if (lane == 0) out[r] = c;
    }
  }
}

__device__ inline double uniform_of(uint32_t w) { return double(w) * (1.0 / 4294967296.0); }

// ---------------------------------------------------------------------------
// the fallback's residual masses, per quarter slice (in the decisions' launch)
// ---------------------------------------------------------------------------
// For every sequence with a fallback, before its primary chain is decided:
// the rows involved are fixed (a, c: the primary's first target and draft
// rows; m: the fallback's first draft row), and this part combines their
// statistics itself, as the decisions do, so it needs nothing from them.  A
// sequence whose first token is then accepted leaves its sums unread.
__device__ void residual_part(const AcceptParams& p, int b, int part) {
  __shared__ RowStat s_r[3];
  const int k = p.k, rows = 4 * k + 2;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ra = target_row(k, 0, 0), rc = draft_row(k, 0, 0), rm = draft_row(k, 1, 0);
  if (wave < 3) {
    const int r = wave == 0 ? ra : (wave == 1 ? rc : rm);
    const RowStat* base = p.part + (size_t(b) * rows + r) * p.split;
    const RowStat c = combine_one(p, lane < p.split ? base[lane] : RowStat{0.0, -INFINITY, 0x7fffffff});
    if (lane == 0) s_r[wave] = c;
  }
  __syncthreads();
  const Dist a{row_ptr(p, b, ra), double(s_r[0].M), s_r[0].S};
  const Dist c{row_ptr(p, b, rc), double(s_r[1].M), s_r[1].S};
  const Dist m{row_ptr(p, b, rm), double(s_r[2].M), s_r[2].S};
  const int n_parts = p.split * kPartsPerSlice;
  const int per_part = (p.slice + kPartsPerSlice - 1) / kPartsPerSlice;
  const int t0 = part * per_part;
  const int t1 = min(p.V, t0 + per_part);
  double wr = 0.0, wm = 0.0;
  for (int t = t0 + threadIdx.x; t < t1; t += kLoadBatch * kAcceptThreads) {
    float za[kLoadBatch], zc[kLoadBatch], zm[kLoadBatch];
#pragma unroll
    for (int j = 0; j < kLoadBatch; ++j) {
      za[j] = load_or(a.z, t + j * kAcceptThreads, t1, 0.f);
      zc[j] = load_or(c.z, t + j * kAcceptThreads, t1, 0.f);
      zm[j] = load_or(m.z, t + j * kAcceptThreads, t1, 0.f);
    }
#pragma unroll
    for (int j = 0; j < kLoadBatch; ++j)
      if (t + j * kAcceptThreads < t1) {
        const double pc = prob_of(c, p.inv_tau, zc[j]);
        wr += fmax(prob_of(a, p.inv_tau, za[j]) - pc, 0.0);
        wm += fmax(prob_of(m, p.inv_tau, zm[j]) - pc, 0.0);
      }
  }
  wr = wg_sum(wr);
  wm = wg_sum(wm);
  if (threadIdx.x == 0) {
    p.sums[(size_t(b) * n_parts + part) * 2] = wr;
    p.sums[(size_t(b) * n_parts + part) * 2 + 1] = wm;
  }
}

__global__ __launch_bounds__(kAcceptThreads) void accept_decide_kernel(const AcceptParams p) {
  if (int(blockIdx.x) >= p.B) {  // (sampling) the residual-mass parts of sequences with a fallback
    const int n_parts = p.split * kPartsPerSlice;
    const int q = int(blockIdx.x) - p.B;
    if (p.has_fb[q / n_parts] != 0) residual_part(p, q / n_parts, q % n_parts);
    return;
  }
  __shared__ RowStat s_st[kMaxRows];
  __shared__ int s_acc[128];
  const int b = blockIdx.x;
  const int k = p.k, V = p.V;
  const int rows = 4 * k + 2;
  const bool fb = p.has_fb[b] != 0;
  const int32_t* tok = p.tokens + size_t(b) * 2 * k;
  const uint32_t* rw = p.rand + size_t(b) * (2 * k + 1);
  // Every test runs on a thread of its own, its inputs loaded with the
  // slices' statistics: thread i < k primary token i (its logits in the
  // target and draft rows, its uniform); greedy calls also thread k + i,
  // fallback token i.  Thread 0 then only reads the outcomes.
  const int i = threadIdx.x;
  int t = -1;
  float zt = 0.f, zd = 0.f;
  double u = 0.0;
  if (i < k) {
    t = tok[i];
    if (!p.greedy) {
      u = uniform_of(rw[i]);
      if (in_vocab(t, V)) {
        zt = row_ptr(p, b, target_row(k, 0, i))[t];
        zd = row_ptr(p, b, draft_row(k, 0, i))[t];
      }
    }
  } else if (p.greedy && i < 2 * k) {
    t = tok[i];
  }
  const double u_draw = p.greedy ? 0.0 : uniform_of(rw[2 * k]);
  combine_rows(p, b, fb, s_st);
  __syncthreads();
  if (!p.greedy)  // (for the launches that follow; greedy decisions are final here)
    for (int r = threadIdx.x; r < rows; r += kAcceptThreads)
      if (!row_unused(p, r, fb)) p.stats[size_t(b) * rows + r] = s_st[r];
  if (p.greedy) {
    // primary token i: the arg max of target row i; the fallback's token 0
    // is scored by the primary's target row 0, its token i >= 1 by its own
    if (i < k) s_acc[i] = in_vocab(t, V) && t == s_st[target_row(k, 0, i)].arg;
    if (i >= k && i < 2 * k) {
      const int f = i - k;
      s_acc[i] = in_vocab(t, V) && t == s_st[f == 0 ? target_row(k, 0, 0) : target_row(k, 1, f)].arg;
    }
    __syncthreads();
    if (threadIdx.x != 0) return;
    int j = 0, n, br, nx;
    while (j < k && s_acc[j]) ++j;
    if (j == k || j > 0 || !fb) {
      n = j; br = 0; nx = s_st[target_row(k, 0, j)].arg;
    } else if (!s_acc[k]) {
      n = 0; br = 0; nx = s_st[target_row(k, 0, 0)].arg;
    } else {
      j = 1;
      while (j < k && s_acc[k + j]) ++j;
      n = j; br = 1; nx = s_st[target_row(k, 1, j)].arg;
    }
    p.n_accept[b] = n;
    p.branch[b] = br;
    p.next_token[b] = nx;
    SeqState ss = {};
    ss.stage = kStageDone;
    p.state[b] = ss;
    return;
  }
  // primary chain: token i is accepted iff u q_i(t) < p_i(t)
  if (i < k) {
    bool acc = false;
    if (in_vocab(t, V)) {
      const RowStat& rt = s_st[target_row(k, 0, i)];
      const RowStat& rd = s_st[draft_row(k, 0, i)];
      const double pt = exp((double(zt) - double(rt.M)) * p.inv_tau) / rt.S;
      const double qt = exp((double(zd) - double(rd.M)) * p.inv_tau) / rd.S;
      acc = u * qt < pt;
    }
    s_acc[i] = acc;
  }
  __syncthreads();
  if (threadIdx.x != 0) return;
  int j = 0;
  while (j < k && s_acc[j]) ++j;
  SeqState ss = {};
  ss.u = u_draw;
  if (j == k) {
    ss.stage = kStageDraw; ss.kind = kDrawRow; ss.ra = target_row(k, 0, k); ss.n = k; ss.branch = 0;
  } else if (j > 0 || !fb) {
    ss.stage = kStageDraw; ss.kind = kDrawResidual; ss.ra = target_row(k, 0, j); ss.rc = draft_row(k, 0, j);
    ss.n = j; ss.branch = 0;
  } else {
    ss.stage = kStageFallback; ss.ra = target_row(k, 0, 0); ss.rc = draft_row(k, 0, 0); ss.rm = draft_row(k, 1, 0);
  }
  carry_rows(ss, s_st);
  p.state[b] = ss;
}

// ---------------------------------------------------------------------------
// the fallback chain's tests (in the draw sums' launch)
// ---------------------------------------------------------------------------
// Taken by every work-group of a sequence left at the fallback stage, the
// same inputs and arithmetic in each; every thread returns the final state.
__device__ SeqState fallback_decide(const AcceptParams& p, int b, SeqState ss) {
  const int k = p.k, V = p.V;
  const double it = p.inv_tau;
  const int32_t* tok = p.tokens + size_t(b) * 2 * k;
  const uint32_t* rw = p.rand + size_t(b) * (2 * k + 1);
  const RowStat* st = p.stats + size_t(b) * (4 * k + 2);
  // the inputs of every test are loaded together: thread 0 the fallback's
  // first token y, its uniform, its logits in rows a, c, m (the primary's
  // first target and draft rows, the fallback's first draft row) and the
  // statistics of the bonus row k; thread i in 1 .. k-1 the fallback chain's
  // token i, its uniform, its rows' statistics and logits; wavefront 0 the
  // residual masses
  __shared__ int s_acc[64];
  __shared__ RowStat s_rt[65], s_rd[64];
  __shared__ double s_w[2];
  __shared__ SeqState s_ss;
  const int i = threadIdx.x;
  int y = -1;
  double u = 0.0;
  float z1 = 0.f, z2 = 0.f, z3 = 0.f;
  RowStat rt = {}, rd = {};
  if (i == 0) {
    y = tok[k];
    u = uniform_of(rw[k]);
    rt = st[target_row(k, 1, k)];
    if (in_vocab(y, V)) {
      z1 = row_ptr(p, b, target_row(k, 0, 0))[y];
      z2 = row_ptr(p, b, draft_row(k, 0, 0))[y];
      z3 = row_ptr(p, b, draft_row(k, 1, 0))[y];
    }
  } else if (i < k) {
    y = tok[k + i];
    u = uniform_of(rw[k + i]);
    rt = st[target_row(k, 1, i)];
    rd = st[draft_row(k, 1, i)];
    if (in_vocab(y, V)) {
      z1 = row_ptr(p, b, target_row(k, 1, i))[y];
      z2 = row_ptr(p, b, draft_row(k, 1, i))[y];
    }
  }
  if (i < 64) {
    // the residual masses: the parts' sums, lane l taking parts l, l + 64,
    // ... in order, then a fixed xor tree over the lanes
    double Wr = 0.0, Wm = 0.0;
    const int n_parts = p.split * kPartsPerSlice;
    for (int q = i; q < n_parts; q += 64) {
      Wr += p.sums[(size_t(b) * n_parts + q) * 2];
      Wm += p.sums[(size_t(b) * n_parts + q) * 2 + 1];
    }
    Wr = wave_sum(Wr);
    Wm = wave_sum(Wm);
    if (i == 0) {
      s_w[0] = Wr;
      s_w[1] = Wm;
    }
  }
  // threads 1 .. k-1: the fallback chain's test at position i, u q'_i(y_i) < p'_i(y_i)
  if (i == 0) s_rt[k] = rt;
  if (i >= 1 && i < k) {
    s_rt[i] = rt;
    s_rd[i] = rd;
    s_acc[i] = in_vocab(y, V) && u * (exp((double(z2) - double(rd.M)) * it) / rd.S) <
                                     exp((double(z1) - double(rt.M)) * it) / rt.S;
  }
  __syncthreads();
  if (i == 0) {
    // the fallback's first token y: accepted iff u q'(y) < r(y), with the
    // residual target r = max(0, p_a - p_c) / Wr (p_a when Wr = 0) and the
    // fallback's draft distribution q' = max(0, p_m - p_c) / Wm (0 when Wm = 0)
    const double Wr = s_w[0], Wm = s_w[1];
    ss.Wr = Wr;
    ss.Wm = Wm;
    ss.kind = kDrawRestart;
    bool acc = false;
    if (in_vocab(y, V)) {
      const double pa = exp((double(z1) - double(ss.M[0])) * it) / ss.S[0];
      const double pc = exp((double(z2) - double(ss.M[1])) * it) / ss.S[1];
      const double pm = exp((double(z3) - double(ss.M[2])) * it) / ss.S[2];
      const double r = Wr > 0.0 ? fmax(pa - pc, 0.0) / Wr : pa;
      const double q = Wm > 0.0 ? fmax(pm - pc, 0.0) / Wm : 0.0;
      acc = u * q < r;
    }
    if (!acc) {
      ss.n = 0; ss.branch = 0;  // restart: draw from max(0, r - q')
    } else {
      int jj = 1;
      while (jj < k && s_acc[jj]) ++jj;
      ss.n = jj; ss.branch = 1;
      if (jj == k) {
        ss.kind = kDrawRow; ss.ra = target_row(k, 1, k);
        ss.S[0] = s_rt[k].S; ss.M[0] = s_rt[k].M;
      } else {
        ss.kind = kDrawResidual; ss.ra = target_row(k, 1, jj); ss.rc = draft_row(k, 1, jj);
        ss.S[0] = s_rt[jj].S; ss.M[0] = s_rt[jj].M;
        ss.S[1] = s_rd[jj].S; ss.M[1] = s_rd[jj].M;
      }
    }
    ss.stage = kStageDraw;
    s_ss = ss;
  }
  __syncthreads();
  return s_ss;
}

// ---------------------------------------------------------------------------
// 3. tile sums of the final draw's weights, per quarter slice
// ---------------------------------------------------------------------------
constexpr int kMaxPartTiles = 1024;  // tiles per part at the largest vocabulary (2^24 over 64 slices)
__global__ __launch_bounds__(kAcceptThreads) void accept_drawsum_kernel(const AcceptParams p) {
  __shared__ int s_last;
  __shared__ double s_ts[kMaxPartTiles];
  // kPartsPerSlice parts per slice, so that a small batch still fills the chip
  const int n_parts = p.split * kPartsPerSlice;
  const int part = blockIdx.x % n_parts;
  const int b = blockIdx.x / n_parts;
  SeqState ss = p.state[b];
  if (ss.stage == kStageFallback) {
    // the fallback's tests first; part 0 records the final state after the
    // primary states, which the launch's other work-groups are still reading
    ss = fallback_decide(p, b, ss);
    if (part == 0 && threadIdx.x == 0) p.state[p.B + b] = ss;
  }
  if (ss.stage != kStageDraw) return;
  const DrawSpec d = spec_of(p, b, ss);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int per_part = (p.slice / kAcceptTile + kPartsPerSlice - 1) / kPartsPerSlice;  // tiles
  const int tile0 = part * per_part;
  const int tile1 = min(p.n_tiles, tile0 + per_part);
  if (threadIdx.x == 0) s_last = -1;
  __syncthreads();
  int last = -1;
  constexpr int kWaves = kAcceptThreads / 64;
  for (int tw = tile0 + wave; tw < tile1; tw += kLoadBatch * kWaves) {
    // this wavefront's next kLoadBatch tiles: loads first, then the sums
    float za[kLoadBatch], zc[kLoadBatch], zm[kLoadBatch];
#pragma unroll
    for (int j = 0; j < kLoadBatch; ++j) {
      // tiles past tile1 load index V - 1 and are not used
      const int t = tw + j * kWaves < tile1 ? (tw + j * kWaves) * kAcceptTile + lane : p.V;
      za[j] = load_or(d.a.z, t, p.V, 0.f);
      zc[j] = load_or(d.c.z, t, p.V, 0.f);
      zm[j] = load_or(d.m.z, t, p.V, 0.f);
    }
#pragma unroll
    for (int j = 0; j < kLoadBatch; ++j) {
      const int tile = tw + j * kWaves;
      if (tile >= tile1) break;
      const int t = tile * kAcceptTile + lane;
      const double w = t < p.V ? weight_of(d, p.inv_tau, za[j], zc[j], zm[j]) : 0.0;
      if (w > 0.0) last = t;
      const double ts = wave_sum(w);
      if (lane == 0) {
        p.tiles[size_t(b) * p.n_tiles + tile] = ts;
        s_ts[tile - tile0] = ts;
      }
    }
  }
  atomicMax(&s_last, last);
  __syncthreads();
  if (threadIdx.x == 0) {
    p.last[size_t(b) * n_parts + part] = s_last;
    // the part's total: its tile sums added in tile order (the pick walks the
    // crossing part's tiles in the same order from 0, so its running sums
    // meet this total exactly)
    double tot = 0.0;
    for (int tile = tile0; tile < tile1; ++tile) tot += s_ts[tile - tile0];
    p.ptot[size_t(b) * n_parts + part] = tot;
  }
}

// ---------------------------------------------------------------------------
// 4. the index where the running sum crosses u * total
// ---------------------------------------------------------------------------
// The running sum is taken part by part (each part's total), then tile by
// tile inside the crossing part, then index by index inside the crossing
// tile; the part totals and the tiles inside a part are added in order from
// 0, as the part totals were formed, so every level meets the next exactly.
constexpr int kMaxParts = kAcceptMaxSplit * kPartsPerSlice;
__global__ __launch_bounds__(kAcceptThreads) void accept_pick_kernel(const AcceptParams p) {
  __shared__ double s_v[kMaxPartTiles > kMaxParts ? kMaxPartTiles : kMaxParts];
  __shared__ double s_total, s_base;
  __shared__ int s_hit;
  const int b = blockIdx.x;
  const int n_parts = p.split * kPartsPerSlice;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // the part totals do not depend on the state: loaded with it
  for (int q = threadIdx.x; q < n_parts; q += kAcceptThreads) s_v[q] = p.ptot[size_t(b) * n_parts + q];
  const SeqState s0 = p.state[b], s1 = p.state[p.B + b];  // (s1: the final state after a fallback)
  SeqState ss = s0.stage == kStageFallback ? s1 : s0;
  __syncthreads();
  if (ss.stage != kStageDraw) return;
  const DrawSpec spec = spec_of(p, b, ss);
  if (threadIdx.x == 0) {
    double total = 0.0;
    for (int q = 0; q < n_parts; ++q) total += s_v[q];
    const double target = ss.u * total;
    double base = 0.0;
    int hit = -1;
    for (int q = 0; q < n_parts && hit < 0; ++q) {
      if (base + s_v[q] > target) hit = q;
      else base += s_v[q];
    }
    s_total = total;
    s_base = base;
    s_hit = hit;
  }
  __syncthreads();
  const double total = s_total;
  if (!(total > 0.0)) {
    // a residual with no mass (possible only through rounding): draw from
    // the row's target distribution, or from r after a restart, in this
    // work-group
    ss.kind = ss.kind == kDrawRestart ? kDrawFallbackR : kDrawRow;
    const int t = wg_draw(spec_of(p, b, ss), p.inv_tau, p.V, ss.u);
    if (threadIdx.x == 0) {
      p.n_accept[b] = ss.n;
      p.branch[b] = ss.branch;
      p.next_token[b] = t;
    }
    return;
  }
  const double target = ss.u * total;
  const int part = s_hit;
  int result = -1;
  if (part >= 0) {
    // the crossing part's tiles, in order from the part's start
    const int per_part = (p.slice / kAcceptTile + kPartsPerSlice - 1) / kPartsPerSlice;
    const int tile0 = part * per_part;
    const int tile1 = min(p.n_tiles, tile0 + per_part);
    __syncthreads();
    for (int tile = tile0 + threadIdx.x; tile < tile1; tile += kAcceptThreads)
      s_v[tile - tile0] = p.tiles[size_t(b) * p.n_tiles + tile];
    __syncthreads();
    if (threadIdx.x == 0) {
      const double base = s_base;
      double pre = 0.0;
      int hit = -1;
      for (int tile = tile0; tile < tile1 && hit < 0; ++tile) {
        if (base + (pre + s_v[tile - tile0]) > target) hit = tile;
        else pre += s_v[tile - tile0];
      }
      s_hit = hit;
      s_base = base + pre;
    }
    __syncthreads();
    const int hit = s_hit;
    if (wave == 0 && hit >= 0) {
      const int t = hit * kAcceptTile + lane;
      const double w = t < p.V ? weight(spec, p.inv_tau, t) : 0.0;
      const double incl = s_base + wave_inclusive_scan(w);
      const unsigned long long over = __ballot(t < p.V && incl > target);
      const unsigned long long pos = __ballot(t < p.V && w > 0.0);
      if (over != 0ull)
        result = hit * kAcceptTile + __ffsll(static_cast<long long>(over)) - 1;
      else if (pos != 0ull)  // rounding left no crossing in the tile: its last index with weight > 0
        result = hit * kAcceptTile + 63 - __builtin_clzll(pos);
    }
  }
  if (wave != 0) return;
  if (result < 0) {  // rounding left no crossing: the last index with weight > 0
    for (int i = 0; i < n_parts; ++i) result = max(result, p.last[size_t(b) * n_parts + i]);
  }
  if (lane == 0) {
    p.n_accept[b] = ss.n;
    p.branch[b] = ss.branch;
    p.next_token[b] = result;
  }
}

hipError_t launch_accept(const AcceptParams& p, hipStream_t stream) {
  if (p.B <= 0) return hipSuccess;
  void* args[] = {const_cast<AcceptParams*>(&p)};
  const int rows = 4 * p.k + 2;
  const int parts = p.B * p.split * kPartsPerSlice;
  struct Launch {
    const void* fn;
    int grid;
  };
  // greedy decisions are final after the second launch; sampling runs the
  // residual-mass parts in the second launch's grid after its B sequences
  const Launch all[] = {{reinterpret_cast<const void*>(&accept_stats_kernel), p.B * rows * p.split},
                        {reinterpret_cast<const void*>(&accept_decide_kernel), p.greedy ? p.B : p.B + parts},
                        {reinterpret_cast<const void*>(&accept_drawsum_kernel), parts},
                        {reinterpret_cast<const void*>(&accept_pick_kernel), p.B}};
  const int n = p.greedy ? 2 : 4;
  for (int i = 0; i < n; ++i) {
    const hipError_t e = hipLaunchKernel(all[i].fn, dim3(all[i].grid), dim3(kAcceptThreads), args, 0, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace ripe
