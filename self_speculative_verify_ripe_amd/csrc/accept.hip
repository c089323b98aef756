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
// How: a short pipeline of launches; the per-index work is spread over
// (sequence, slice of the vocabulary) work-groups and the decisions run on
// one work-group per sequence between them.
//   accept_stats_kernel     per (row, slice): arg max (lowest index on ties),
//                           max, and sum exp((z - max) / tau); rows no decision
//                           can read are skipped
//   accept_decide_kernel    per sequence: combines the slices into each row's
//                           statistics; greedy decisions (final), or the
//                           primary chain's speculative tests
//   accept_fbsum_kernel     per (sequence, quarter slice), only after a first-token
//                           rejection with a fallback: the residual masses
//   accept_fallback_kernel  per sequence: the fallback's tests
//   accept_drawsum_kernel   per (sequence, quarter slice): sums of the final draw's
//                           weights over tiles of 64 indices
//   accept_pick_kernel      per sequence: the tile where the running sum
//                           crosses u * total, then the index inside it
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

__device__ inline double prob(const Dist& d, double inv_tau, int t) { return prob_of(d, inv_tau, d.z[t]); }

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

__device__ inline double fallback_r(const DrawSpec& s, double inv_tau, int t) {
  const double pa = prob(s.a, inv_tau, t);
  return s.Wr > 0.0 ? fmax(pa - prob(s.c, inv_tau, t), 0.0) / s.Wr : pa;
}

__device__ inline double fallback_q(const DrawSpec& s, double inv_tau, int t) {
  return s.Wm > 0.0 ? fmax(prob(s.m, inv_tau, t) - prob(s.c, inv_tau, t), 0.0) / s.Wm : 0.0;
}

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
    default: {  // kDrawRestart: fallback_r - fallback_q, with c's probability computed once
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


__device__ inline Dist dist_of(const AcceptParams& p, int b, int r) {
  const RowStat st = p.stats[size_t(b) * (4 * p.k + 2) + r];
  return Dist{row_ptr(p, b, r), double(st.M), st.S};
}

__device__ inline DrawSpec spec_of(const AcceptParams& p, int b, const SeqState& s) {
  DrawSpec d;
  d.kind = s.kind;
  d.a = dist_of(p, b, s.ra);
  d.c = s.kind == kDrawRow ? d.a : dist_of(p, b, s.rc);
  d.m = (s.kind == kDrawRestart || s.kind == kDrawFallbackR) ? dist_of(p, b, s.rm) : d.a;
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
        if (t0 + int(threadIdx.x) + j * kAcceptThreads < t1) s += exp((double(zv[j]) - M) * p.inv_tau);
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
          if (t + j * kAcceptThreads < t1) s += exp((double(zv[j]) - M) * p.inv_tau);
      }
      s = wg_sum(s);
    }
  }
  if (threadIdx.x == 0) p.part[size_t(br) * p.split + sl] = RowStat{s, mv, mi};
}

// ---------------------------------------------------------------------------
// 2. row statistics, greedy decisions, the primary chain's tests
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kAcceptThreads) void accept_decide_kernel(const AcceptParams p) {
  const int b = blockIdx.x;
  const int k = p.k, V = p.V;
  const int rows = 4 * k + 2;
  const bool fb = p.has_fb[b] != 0;
  // combine the slices: max and arg max, S = sum_i s_i exp((m_i - M) / tau)
  for (int r = threadIdx.x; r < rows; r += kAcceptThreads) {
    if (row_unused(p, r, fb)) continue;
    const RowStat* pr = p.part + (size_t(b) * rows + r) * p.split;
    float M = -INFINITY;
    int arg = 0x7fffffff;
    for (int i = 0; i < p.split; ++i) better(M, arg, pr[i].M, pr[i].arg);
    double S = 0.0;
    if (!p.greedy)
      for (int i = 0; i < p.split; ++i)
        if (pr[i].M > -INFINITY) S += pr[i].S * exp((double(pr[i].M) - double(M)) * p.inv_tau);
    p.stats[size_t(b) * rows + r] = RowStat{S, M, arg};
  }
  __syncthreads();  // (a work-group barrier also orders the global writes above)
  const RowStat* st = p.stats + size_t(b) * rows;
  const int32_t* tok = p.tokens + size_t(b) * 2 * k;
  // the primary chain's p_i(x_i) and q_i(x_i), one thread per position
  __shared__ double s_pt[64], s_qt[64];
  if (!p.greedy && int(threadIdx.x) < k) {
    const int i = threadIdx.x, t = tok[i];
    const bool ok = in_vocab(t, V);
    s_pt[i] = ok ? prob(dist_of(p, b, target_row(k, 0, i)), p.inv_tau, t) : 0.0;
    s_qt[i] = ok ? prob(dist_of(p, b, draft_row(k, 0, i)), p.inv_tau, t) : 0.0;
  }
  __syncthreads();
  if (threadIdx.x != 0) return;
  SeqState ss = {};
  if (p.greedy) {
    int j = 0, n, br, nx;
    while (j < k && in_vocab(tok[j], V) && tok[j] == st[target_row(k, 0, j)].arg) ++j;
    if (j == k || j > 0 || !fb) {
      n = j; br = 0; nx = st[target_row(k, 0, j)].arg;
    } else if (!(in_vocab(tok[k], V) && tok[k] == st[target_row(k, 0, 0)].arg)) {
      n = 0; br = 0; nx = st[target_row(k, 0, 0)].arg;
    } else {
      j = 1;
      while (j < k && in_vocab(tok[k + j], V) && tok[k + j] == st[target_row(k, 1, j)].arg) ++j;
      n = j; br = 1; nx = st[target_row(k, 1, j)].arg;
    }
    p.n_accept[b] = n;
    p.branch[b] = br;
    p.next_token[b] = nx;
    ss.stage = kStageDone;
    p.state[b] = ss;
    return;
  }
  const double it = p.inv_tau;
  const uint32_t* rw = p.rand + size_t(b) * (2 * k + 1);
  auto uni = [&](int w) { return double(rw[w]) * (1.0 / 4294967296.0); };
  // primary chain: accept t iff u q(t) < p(t)
  int j = 0;
  for (; j < k; ++j) {
    if (!in_vocab(tok[j], V)) break;
    if (!(uni(j) * s_qt[j] < s_pt[j])) break;
  }
  (void)it;
  ss.u = uni(2 * k);
  if (j == k) {
    ss.stage = kStageDraw; ss.kind = kDrawRow; ss.ra = target_row(k, 0, k); ss.n = k; ss.branch = 0;
  } else if (j > 0 || !fb) {
    ss.stage = kStageDraw; ss.kind = kDrawResidual; ss.ra = target_row(k, 0, j); ss.rc = draft_row(k, 0, j);
    ss.n = j; ss.branch = 0;
  } else {
    ss.stage = kStageFallback; ss.ra = target_row(k, 0, 0); ss.rc = draft_row(k, 0, 0); ss.rm = draft_row(k, 1, 0);
  }
  p.state[b] = ss;
}

// ---------------------------------------------------------------------------
// 3. the fallback's residual masses, per quarter slice
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kAcceptThreads) void accept_fbsum_kernel(const AcceptParams p) {
  const int n_parts = p.split * kPartsPerSlice;
  const int part = blockIdx.x % n_parts;
  const int b = blockIdx.x / n_parts;
  const SeqState ss = p.state[b];
  if (ss.stage != kStageFallback) return;
  const Dist a = dist_of(p, b, ss.ra), c = dist_of(p, b, ss.rc), m = dist_of(p, b, ss.rm);
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

// ---------------------------------------------------------------------------
// 4. the fallback chain's tests
// ---------------------------------------------------------------------------
__global__ void accept_fallback_kernel(const AcceptParams p) {
  const int b = blockIdx.x;
  SeqState ss = p.state[b];
  if (ss.stage != kStageFallback) return;
  const int k = p.k, V = p.V;
  const double it = p.inv_tau;
  const int32_t* tok = p.tokens + size_t(b) * 2 * k;
  // the fallback chain's p'_i(y_i) and q'_i(y_i) for i >= 1, one lane per position
  __shared__ double s_pt[64], s_qt[64];
  if (threadIdx.x >= 1 && int(threadIdx.x) < k) {
    const int i = threadIdx.x, t = tok[k + i];
    const bool ok = in_vocab(t, V);
    s_pt[i] = ok ? prob(dist_of(p, b, target_row(k, 1, i)), it, t) : 0.0;
    s_qt[i] = ok ? prob(dist_of(p, b, draft_row(k, 1, i)), it, t) : 0.0;
  }
  // the residual masses: the parts' sums, lane i taking parts i, i + 64, ...
  // in order, then a fixed xor tree over the lanes
  double Wr = 0.0, Wm = 0.0;
  const int n_parts = p.split * kPartsPerSlice;
  for (int i = threadIdx.x; i < n_parts; i += 64) {
    Wr += p.sums[(size_t(b) * n_parts + i) * 2];
    Wm += p.sums[(size_t(b) * n_parts + i) * 2 + 1];
  }
  Wr = wave_sum(Wr);
  Wm = wave_sum(Wm);
  __syncthreads();
  if (threadIdx.x != 0) return;
  const uint32_t* rw = p.rand + size_t(b) * (2 * k + 1);
  auto uni = [&](int w) { return double(rw[w]) * (1.0 / 4294967296.0); };
  ss.Wr = Wr;
  ss.Wm = Wm;
  ss.kind = kDrawRestart;
  const DrawSpec d = spec_of(p, b, ss);
  const int y = tok[k];
  const bool acc = in_vocab(y, V) && uni(k) * fallback_q(d, it, y) < fallback_r(d, it, y);
  if (!acc) {
    ss.n = 0; ss.branch = 0;  // restart: draw from max(0, r - q')
  } else {
    int jj = 1;
    for (; jj < k; ++jj) {
      if (!in_vocab(tok[k + jj], V)) break;
      if (!(uni(k + jj) * s_qt[jj] < s_pt[jj])) break;
    }
    ss.n = jj; ss.branch = 1;
    if (jj == k) {
      ss.kind = kDrawRow; ss.ra = target_row(k, 1, k);
    } else {
      ss.kind = kDrawResidual; ss.ra = target_row(k, 1, jj); ss.rc = draft_row(k, 1, jj);
    }
  }
  ss.stage = kStageDraw;
  p.state[b] = ss;
}

// ---------------------------------------------------------------------------
// 5. tile sums of the final draw's weights, per quarter slice
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kAcceptThreads) void accept_drawsum_kernel(const AcceptParams p) {
  __shared__ int s_last;
  // kPartsPerSlice parts per slice, so that a small batch still fills the chip
  const int n_parts = p.split * kPartsPerSlice;
  const int part = blockIdx.x % n_parts;
  const int b = blockIdx.x / n_parts;
  const SeqState ss = p.state[b];
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
      if (lane == 0) p.tiles[size_t(b) * p.n_tiles + tile] = ts;
    }
  }
  atomicMax(&s_last, last);
  __syncthreads();
  if (threadIdx.x == 0) p.last[size_t(b) * n_parts + part] = s_last;
}

// ---------------------------------------------------------------------------
// 6. the index where the running sum crosses u * total
// ---------------------------------------------------------------------------
constexpr int kPickBatch = 16;  // rows of 64 tile sums loaded together
__global__ __launch_bounds__(kAcceptThreads) void accept_pick_kernel(const AcceptParams p) {
  __shared__ double s_total;
  const int b = blockIdx.x;
  SeqState ss = p.state[b];
  if (ss.stage != kStageDraw) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const double* tiles = p.tiles + size_t(b) * p.n_tiles;
  if (wave == 0) {
    // total of the tile sums, in tile order (16 rows of 64 loaded at a time)
    double run = 0.0;
    for (int base = 0; base < p.n_tiles; base += kPickBatch * 64) {
      double ts[kPickBatch];
#pragma unroll
      for (int i = 0; i < kPickBatch; ++i) {
        const int tile = base + i * 64 + lane;
        ts[i] = tile < p.n_tiles ? tiles[tile] : 0.0;
      }
#pragma unroll
      for (int i = 0; i < kPickBatch; ++i) run += __shfl(wave_inclusive_scan(ts[i]), 63);
    }
    if (lane == 0) s_total = run;
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
  if (wave != 0) return;
  const double target = ss.u * total;
  double run = 0.0;
  int hit = -1;
  for (int base = 0; base < p.n_tiles && hit < 0; base += kPickBatch * 64) {
    double ts[kPickBatch];
#pragma unroll
    for (int i = 0; i < kPickBatch; ++i) {
      const int tile = base + i * 64 + lane;
      ts[i] = tile < p.n_tiles ? tiles[tile] : 0.0;
    }
#pragma unroll
    for (int i = 0; i < kPickBatch; ++i) {
      if (hit >= 0) break;
      const int i0 = base + i * 64;
      const double incl = wave_inclusive_scan(ts[i]);
      const unsigned long long over = __ballot(i0 + lane < p.n_tiles && run + incl > target);
      if (over != 0ull) {
        const int l = __ffsll(static_cast<long long>(over)) - 1;
        hit = i0 + l;
        run += __shfl(incl - ts[i], l);
      } else {
        run += __shfl(incl, 63);
      }
    }
  }
  int result = -1;
  if (hit >= 0) {
    const DrawSpec d = spec_of(p, b, ss);
    const int t = hit * kAcceptTile + lane;
    const double w = t < p.V ? weight(d, p.inv_tau, t) : 0.0;
    const double incl = run + wave_inclusive_scan(w);
    const unsigned long long over = __ballot(t < p.V && incl > target);
    if (over != 0ull) result = hit * kAcceptTile + __ffsll(static_cast<long long>(over)) - 1;
  }
  if (result < 0) {  // rounding left no crossing: the last index with weight > 0
    const int n_parts = p.split * kPartsPerSlice;
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
  struct Launch {
    const void* fn;
    int grid, block;
  };
  const Launch all[] = {
      {reinterpret_cast<const void*>(&accept_stats_kernel), p.B * rows * p.split, kAcceptThreads},
      {reinterpret_cast<const void*>(&accept_decide_kernel), p.B, kAcceptThreads},
      {reinterpret_cast<const void*>(&accept_fbsum_kernel), p.B * p.split * kPartsPerSlice, kAcceptThreads},
      {reinterpret_cast<const void*>(&accept_fallback_kernel), p.B, 64},
      {reinterpret_cast<const void*>(&accept_drawsum_kernel), p.B * p.split * kPartsPerSlice, kAcceptThreads},
      {reinterpret_cast<const void*>(&accept_pick_kernel), p.B, kAcceptThreads}};
  const int n = p.greedy ? 2 : 6;  // greedy decisions are final after the second
  for (int i = 0; i < n; ++i) {
    const hipError_t e = hipLaunchKernel(all[i].fn, dim3(all[i].grid), dim3(all[i].block), args, 0, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace ripe
