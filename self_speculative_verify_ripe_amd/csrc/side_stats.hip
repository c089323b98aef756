// side_stats.hip -- per-position plane-substitution error on a FULL cache.
//
// What is computed (RIPE abstract, zhuanzhiai.com paper page: the error of
// storing only the deepest plane, a small set of positions carrying most of
// it, a window of recent positions at full depth removing most of those):
// for a group at depth r (rows i, query heads h of KV head h / G) with FULL
// output O and natural-log LSE, the squared change of the outputs when
// prefix position j alone is read at plane R instead of plane r,
//
//   e_j = sum_{i,h} || (a (v_R - v_r) + g (v_R - O)) / (1 + g) ||^2,
//   a = exp(scale q.k_r - LSE),  g = a expm1(scale q.(k_R - k_r)),
//
// which is the single-term softmax update O^(j) - O written with direct
// differences (no cancellation when planes r and R are close).  Its
// sensitivity to the inputs O and LSE is kappa = a / (1 + g) = a / (1 - a + c):
// at most 1 unless position j holds more than half of a row's attention at
// plane r (at most one such position per row), where O carries too little of
// the other positions' average to recover it in fp32.  kappa_j (max over the
// group's columns and heads) is returned beside e_j so that such positions
// can be told apart.
//
// How: one work-group per (group, KV head, 32 prefix positions).  The tile's
// K and V rows of planes r and R (32 contiguous positions of the FULL
// layout: K rows, V four [D][8] blocks) are staged through LDS -- V transposed to position-major --
// and each thread keeps a 1/8 slice of one position's four rows in
// registers.  The group's query columns and their FULL outputs are staged
// 16 at a time and read back by broadcast; the two dot products per column
// are reduced over the position's 8 lanes with DPP moves.  A second kernel sums the KV
// heads in a fixed order.  The kernel reads 4 rows per (position, KV head),
// but it is bound by VALU issue, not by HBM bandwidth: per query column it
// runs two dot products, their DPP reductions and the single-term update on
// all 8 lanes of a position (measured on c2: about 2 TB/s, the instruction
// count per wave accounting for the time).
#include <hip/hip_runtime.h>
#include <math.h>

#include "side_stats.h"

namespace ripe {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kPeThreads = 256;
constexpr int kParts = kPeThreads / kPeTile;  // threads per position
static_assert(kParts == 8, "the lane reductions below combine 8 consecutive lanes");

// DPP lane moves (VALU, no LDS round trip).  quad_perm(a,b,c,d) encodes
// a | b << 2 | c << 4 | d << 6; row_half_mirror (0x141) reverses each group of
// 8 lanes.
template <int CTRL>
__device__ inline float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int kQuadXor1 = 1 | (0 << 2) | (3 << 4) | (2 << 6);
constexpr int kQuadXor2 = 2 | (3 << 2) | (0 << 4) | (1 << 6);
constexpr int kHalfMirror = 0x141;
template <int L>
constexpr int kQuadBcast = L | (L << 2) | (L << 4) | (L << 6);

// Sum over each aligned group of 8 lanes, the same bits in all 8: after the
// two quad steps every lane of a quad holds the quad's sum, and the mirror
// brings in the other quad's (a + b = b + a, so both quads agree).
__device__ inline float sum8(float x) {
  x += dpp<kQuadXor1>(x);
  x += dpp<kQuadXor2>(x);
  return x + dpp<kHalfMirror>(x);
}

template <typename T, int D>
__global__ __launch_bounds__(kPeThreads) void position_error_kernel(const PosErrParams p) {
  constexpr int E = sizeof(T);
  constexpr int VE = 16 / E;         // elements per 16-byte chunk
  constexpr int DP = D / kParts;     // head-dim slice per thread
  constexpr int RSK = D + VE;        // K rows: one 16-byte chunk of padding
  // V rows: D + 2 elements, so that a transposing store's 4 (bf16) or 8
  // (fp32) position rows start 8 banks apart and its head dimensions fill
  // the rest: 2-way bank conflicts at most, against 8 to 16 with 16-byte rows
  constexpr int RSV = D + 2;
  __shared__ __align__(16) T sk[2][kPeTile][RSK];  // k_r, k_R, position-major
  __shared__ __align__(16) T sv[2][kPeTile][RSV];  // v_r, v_R, position-major
  __shared__ float sq[kPeCols][D];
  __shared__ float so[kPeCols][D];
  __shared__ float sl[kPeCols];

  const int gl = blockIdx.z;
  const PeGroup grp = p.grp[gl];
  const int h = blockIdx.y;
  const int j0 = blockIdx.x * kPeTile;
  if (j0 >= grp.T) return;  // whole work-group

  // ---- stage the tile: rows j0 .. j0 + 31 (in the allocation: t_max is a
  // multiple of 32 and j0 < T <= t_max), and the first chunk of query
  // columns.  Every global load is issued before the first LDS store, so the
  // work-group waits for memory once.
  const int tid = threadIdx.x;
  constexpr int NC = D * E / 128;  // 16-byte chunks per thread per array (32 x D elements)
  constexpr int CR = D / VE;       // K: chunks per row
  u32x4 buf[4][NC];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int plane = (a & 1) ? p.R : grp.depth;
    const size_t head = (size_t(grp.b) * p.R + (plane - 1)) * p.H + h;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int idx = tid + c * kPeThreads;
      if (a < 2) {  // K [t][D]: row-major
        const T* src = static_cast<const T*>(p.cache_k) + (head * p.t_max + j0) * D;
        buf[a][c] = *reinterpret_cast<const u32x4*>(src + size_t(idx / CR) * D + (idx % CR) * VE);
      } else {      // V: the tile is four contiguous blocks [D][8]
        const T* src = static_cast<const T*>(p.cache_v) + (head * p.t_max + j0) * D;
        buf[a][c] = *reinterpret_cast<const u32x4*>(src + size_t(idx) * VE);
      }
    }
  }
  const int nq = grp.n_rows * p.G;
  constexpr int QN = kPeCols * D / kPeThreads;  // staged query values per thread
  // Column loads are unconditional (columns past nq read column nq - 1, in
  // range since nq >= 1) and zeroed when stored, so that no load waits for
  // the one before it.
  T qv[QN];
  float ov[QN], lv;
  auto col_index = [&](int col) {
    col = min(col, nq - 1);
    return size_t(grp.row_start + col / p.G) * p.Hq + size_t(h) * p.G + col % p.G;
  };
  int c_loaded = 0;
  auto load_cols = [&](int c0) {
    c_loaded = c0;
#pragma unroll
    for (int x = 0; x < QN; ++x) {
      const int idx = tid + x * kPeThreads;
      const size_t qi = col_index(c0 + idx / D) * D + idx % D;
      qv[x] = static_cast<const T*>(p.q)[qi];
      ov[x] = p.o[qi];
    }
    lv = p.lse[col_index(c0 + (tid % kPeCols))];
  };
  auto store_cols = [&]() {
#pragma unroll
    for (int x = 0; x < QN; ++x) {
      const int idx = tid + x * kPeThreads;
      const bool ok = c_loaded + idx / D < nq;
      sq[idx / D][idx % D] = ok ? static_cast<float>(qv[x]) : 0.f;
      so[idx / D][idx % D] = ok ? ov[x] : 0.f;
    }
    if (tid < kPeCols) sl[tid] = c_loaded + tid < nq ? lv : 0.f;
  };
  load_cols(0);
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int idx = tid + c * kPeThreads;
      if (a < 2) {
        *reinterpret_cast<u32x4*>(&sk[a][idx / CR][(idx % CR) * VE]) = buf[a][c];
      } else {  // transposed into [t][D]: chunk idx holds slots t0 .. t0 + VE - 1 of dimension d
        const T* e = reinterpret_cast<const T*>(&buf[a][c]);
        const int el = idx * VE;
        const int d = (el % (8 * D)) / 8, t0 = el / (8 * D) * 8 + el % 8;
#pragma unroll
        for (int x = 0; x < VE; ++x) sv[a - 2][t0 + x][d] = e[x];
      }
    }
  store_cols();
  __syncthreads();

  const int jl = tid / kParts, part = tid % kParts;
  const int j = j0 + jl;
  const int d0 = part * DP;
  float kr[DP], dk[DP], dv[DP], vR[DP];
#pragma unroll
  for (int e = 0; e < DP; ++e) {
    kr[e] = static_cast<float>(sk[0][jl][d0 + e]);
    dk[e] = static_cast<float>(sk[1][jl][d0 + e]) - kr[e];
    const float vr = static_cast<float>(sv[0][jl][d0 + e]);
    vR[e] = static_cast<float>(sv[1][jl][d0 + e]);
    dv[e] = vR[e] - vr;
  }

  // ---- query columns (row i, head h*G + x) in chunks of kPeCols ------------
  float acc = 0.f;
  float kappa = 0.f;
  for (int c0 = 0; c0 < nq; c0 += kPeCols) {
    if (c0 > 0) {
      load_cols(c0);
      __syncthreads();  // the previous chunk's readers are done
      store_cols();
      __syncthreads();
    }
    const int nc = min(kPeCols, nq - c0);
    for (int cl = 0; cl < nc; ++cl) {
      float s = 0.f, ds = 0.f;
#pragma unroll
      for (int e = 0; e < DP; ++e) {
        const float qe = sq[cl][d0 + e];
        s = fmaf(qe, kr[e], s);
        ds = fmaf(qe, dk[e], ds);
      }
      s = sum8(s);
      ds = sum8(ds);
      const float a = expf(p.scale * s - sl[cl]);
      const float g = a * expm1f(p.scale * ds);
      float sum = 0.f;
#pragma unroll
      for (int e = 0; e < DP; ++e) {
        const float x = fmaf(a, dv[e], g * (vR[e] - so[cl][d0 + e]));
        sum = fmaf(x, x, sum);
      }
      const float inv = 1.f / (1.f + g);
      acc = fmaf(sum, inv * inv, acc);
      kappa = fmaxf(kappa, a * inv);
    }
  }
  acc = sum8(acc);
  if (part == 0 && j < grp.T) {
    const size_t at = (size_t(p.g0 + gl) * p.H + h) * p.t_max + j;
    p.part[at] = acc;
    p.part_cond[at] = kappa;  // the same in all of the position's lanes
  }
}

// e[g][j] = sum over KV heads, cond[g][j] = their largest kappa (both 0 for
// j >= T).  64 positions per work-group, four lanes per position: lane s
// sums heads s, s + 4, ... in order, then the four sums are added in lane
// order (a fixed order: the result does not depend on the launch).
constexpr int kSumPos = 64;
__global__ __launch_bounds__(256) void position_error_sum_kernel(const PosErrParams p) {
  const int gl = blockIdx.y;
  const int j = blockIdx.x * kSumPos + (threadIdx.x >> 2);
  const int s = threadIdx.x & 3;
  const int g = p.g0 + gl;
  const int T = p.grp[gl].T;
  float e = 0.f, k = 0.f;
  if (j < T) {
    const float* pe = p.part + size_t(g) * p.H * p.t_max + j;
    const float* pk = p.part_cond + size_t(g) * p.H * p.t_max + j;
#pragma unroll 4
    for (int h = s; h < p.H; h += 4) {
      e += pe[size_t(h) * p.t_max];
      k = fmaxf(k, pk[size_t(h) * p.t_max]);
    }
  }
  // the position's four lanes form one DPP quad: broadcast each lane's value
  const float e0 = dpp<kQuadBcast<0>>(e), e1 = dpp<kQuadBcast<1>>(e), e2 = dpp<kQuadBcast<2>>(e),
              e3 = dpp<kQuadBcast<3>>(e);
  const float k0 = dpp<kQuadBcast<0>>(k), k1 = dpp<kQuadBcast<1>>(k), k2 = dpp<kQuadBcast<2>>(k),
              k3 = dpp<kQuadBcast<3>>(k);
  if (s == 0 && j < p.t_max) {
    p.err[size_t(g) * p.t_max + j] = ((e0 + e1) + e2) + e3;
    if (p.cond != nullptr) p.cond[size_t(g) * p.t_max + j] = fmaxf(fmaxf(k0, k1), fmaxf(k2, k3));
  }
}

template <typename T, int D>
hipError_t launch_t(const PosErrParams& p, hipStream_t stream) {
  void* args[] = {const_cast<PosErrParams*>(&p)};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&position_error_kernel<T, D>),
                                 dim3(p.t_max / kPeTile, p.H, p.n_grp), dim3(kPeThreads), args, 0, stream);
  if (e != hipSuccess) return e;
  return hipLaunchKernel(reinterpret_cast<const void*>(&position_error_sum_kernel),
                         dim3((p.t_max + kSumPos - 1) / kSumPos, p.n_grp), dim3(256), args, 0, stream);
}

// ---- tail summary ---------------------------------------------------------
// Per row: the share of sum_j e_j carried by its n largest e_j (ties to the
// lower position), the fraction of those positions in the last W, the share
// of the last W positions, and the positions with cond > 1 and their share.
// The n-th largest value is found by a radix select on the float's bits
// (e >= 0, so the bits order like the values): four passes over the row,
// each a 256-bin histogram of the next byte among the keys that match the
// bytes already chosen, then the byte whose bin holds the n-th largest
// (11 us on a 1024-position row, against 25 us for 32 one-bit counting
// passes).  The tail
// is every position above that value plus the lowest-numbered positions
// equal to it.  Sums are in double, each thread over its positions j = t,
// t + 256, ... in order, then across threads in a fixed order.
constexpr int kTailThreads = 256;

__device__ inline uint32_t tail_key(float x) {
  const uint32_t b = __float_as_uint(x);
  return (b & 0x80000000u) ? 0u : b;  // -0 orders as 0
}

template <typename V>
__device__ inline V block_sum(V x, V* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = x;
  __syncthreads();
  const V r = ((red[0] + red[1]) + red[2]) + red[3];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kTailThreads) void position_error_tail_kernel(const TailParams p) {
  __shared__ double rd[4];
  __shared__ int ri[4];
  const int gl = blockIdx.x;
  const int T = p.T[gl], n = p.n_tail[gl];
  const float* e = p.err + size_t(p.g0 + gl) * p.stride;
  const float* c = p.cond ? p.cond + size_t(p.g0 + gl) * p.stride : nullptr;
  const int w0 = max(0, T - p.window);
  const int t = threadIdx.x;
  double tot = 0.0, win = 0.0, ills = 0.0;
  int illc = 0;
  for (int j = t; j < T; j += kTailThreads) {
    const double x = e[j];
    tot += x;
    if (j >= w0) win += x;
    if (c != nullptr && c[j] > 1.0f) {
      ++illc;
      ills += x;
    }
  }
  tot = block_sum(tot, rd);
  win = block_sum(win, rd);
  ills = block_sum(ills, rd);
  illc = block_sum(illc, ri);
  // the n-th largest key (the largest k with count(key >= k) >= n), a byte
  // at a time from the top: rem is n less the keys above the chosen prefix
  __shared__ int hist[256];
  __shared__ uint32_t s_prefix;
  __shared__ int s_rem;
  uint32_t tau = 0, mask = 0;
  int rem = n;
  for (int shift = 24; shift >= 0 && n > 0; shift -= 8) {
    for (int i = t; i < 256; i += kTailThreads) hist[i] = 0;
    if (t == 0) {  // (kept if no bin were found, which n <= T rules out)
      s_prefix = tau;
      s_rem = rem;
    }
    __syncthreads();
    for (int j = t; j < T; j += kTailThreads) {
      const uint32_t k = tail_key(e[j]);
      if ((k & mask) == tau) atomicAdd(&hist[(k >> shift) & 255u], 1);
    }
    __syncthreads();
    if (t < 64) {
      // lane l: bins 255 - 4l .. 252 - 4l (descending); keys above its bins
      // by an exclusive scan over the lanes
      int c[4], sl = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) sl += (c[i] = hist[255 - 4 * t - i]);
      int incl = sl;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o);
        if (t >= o) incl += y;
      }
      int above = incl - sl;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (above < rem && above + c[i] >= rem) {  // exactly one lane and bin
          s_prefix = tau | (uint32_t(255 - 4 * t - i) << shift);
          s_rem = rem - above;
        }
        above += c[i];
      }
    }
    __syncthreads();
    tau = s_prefix;
    rem = s_rem;
    mask |= 255u << shift;
  }
  int gt = 0, gt_win = 0, tie_low = 0;
  double s_gt = 0.0;
  for (int j = t; j < T && n > 0; j += kTailThreads) {
    const uint32_t k = tail_key(e[j]);
    if (k > tau) {
      ++gt;
      s_gt += e[j];
      if (j >= w0) ++gt_win;
    } else if (k == tau && j < w0) {
      ++tie_low;
    }
  }
  gt = block_sum(gt, ri);
  gt_win = block_sum(gt_win, ri);
  tie_low = block_sum(tie_low, ri);
  s_gt = block_sum(s_gt, rd);
  if (t == 0) {
    const int m = n - gt;                        // positions equal to the n-th largest, lowest first
    const int m_win = m - min(m, tie_low);       // ... of which in the window
    const double tail = s_gt + double(m) * double(__uint_as_float(tau));
    const double nan = __builtin_nan("");
    double* o = p.stats + size_t(p.g0 + gl) * kTailStats;
    o[0] = n;
    o[1] = tot > 0.0 ? tail / tot : nan;
    o[2] = n > 0 ? double(gt_win + m_win) / double(n) : nan;
    o[3] = tot > 0.0 ? win / tot : nan;
    o[4] = c != nullptr ? double(illc) : nan;
    o[5] = c != nullptr && tot > 0.0 ? ills / tot : nan;
    o[6] = tot;
    o[7] = T;
  }
}

}  // namespace

hipError_t launch_position_error_tail(const TailParams& p, hipStream_t stream) {
  if (p.n_rows <= 0) return hipSuccess;
  void* args[] = {const_cast<TailParams*>(&p)};
  return hipLaunchKernel(reinterpret_cast<const void*>(&position_error_tail_kernel), dim3(p.n_rows),
                         dim3(kTailThreads), args, 0, stream);
}

hipError_t launch_position_error(const PosErrParams& p, int dtype, int D, hipStream_t stream) {
  if (p.n_grp <= 0) return hipSuccess;
  if (dtype == 1) return D == 128 ? launch_t<__bf16, 128>(p, stream) : launch_t<__bf16, 64>(p, stream);
  return D == 128 ? launch_t<float, 128>(p, stream) : launch_t<float, 64>(p, stream);
}

}  // namespace ripe
