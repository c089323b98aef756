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
// K and V rows of planes r and R (four contiguous 32-position blocks of the
// FULL layout) are staged through LDS -- V transposed to position-major --
// and each thread keeps a 1/8 slice of one position's four rows in
// registers.  The group's query columns and their FULL outputs are staged
// 16 at a time and read back by broadcast; the two dot products per column
// are reduced over the position's 8 lanes.  A second kernel sums the KV
// heads in a fixed order.  The work is a streaming read of 4 rows per
// (position, KV head): bound by HBM bandwidth.
#include <hip/hip_runtime.h>
#include <math.h>

#include "side_stats.h"

namespace ripe {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kPeThreads = 256;
constexpr int kParts = kPeThreads / kPeTile;  // threads per position

template <typename T, int D>
__global__ __launch_bounds__(kPeThreads) void position_error_kernel(const PosErrParams p) {
  constexpr int E = sizeof(T);
  constexpr int VE = 16 / E;         // elements per 16-byte chunk
  constexpr int DP = D / kParts;     // head-dim slice per thread
  constexpr int RS = D + VE;         // LDS row stride (one chunk of padding)
  __shared__ __align__(16) T skv[4][kPeTile][RS];  // k_r, k_R, v_r, v_R, position-major
  __shared__ float sq[kPeCols][D];
  __shared__ float so[kPeCols][D];
  __shared__ float sl[kPeCols];

  const int gl = blockIdx.z;
  const PeGroup grp = p.grp[gl];
  const int h = blockIdx.y;
  const int j0 = blockIdx.x * kPeTile;
  if (j0 >= grp.T) return;  // whole work-group

  // ---- stage the tile: rows j0 .. j0 + 31 (in the allocation: t_max is a
  // multiple of 32 and j0 < T <= t_max) --------------------------------------
  const int tid = threadIdx.x;
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int plane = (a & 1) ? p.R : grp.depth;
    const size_t head = (size_t(grp.b) * p.R + (plane - 1)) * p.H + h;
    if (a < 2) {  // K [t][D]: row-major, copied as is
      const T* src = static_cast<const T*>(p.cache_k) + (head * p.t_max + j0) * D;
      constexpr int CR = D / VE;  // chunks per row
      for (int c = tid; c < kPeTile * CR; c += kPeThreads) {
        const int row = c / CR, cc = c % CR;
        const u32x4 v = *reinterpret_cast<const u32x4*>(src + size_t(row) * D + cc * VE);
        *reinterpret_cast<u32x4*>(&skv[a][row][cc * VE]) = v;
      }
    } else {  // V [D][32] per block: transposed into [t][D]
      const T* src = static_cast<const T*>(p.cache_v) + (head * (p.t_max / 32) + j0 / 32) * size_t(D) * 32;
      constexpr int CD = 32 / VE;  // chunks per head dimension
      for (int c = tid; c < D * CD; c += kPeThreads) {
        const int d = c / CD, t0 = (c % CD) * VE;
        const u32x4 v = *reinterpret_cast<const u32x4*>(src + size_t(d) * 32 + t0);
        const T* e = reinterpret_cast<const T*>(&v);
#pragma unroll
        for (int x = 0; x < VE; ++x) skv[a][t0 + x][d] = e[x];
      }
    }
  }
  __syncthreads();

  const int jl = tid / kParts, part = tid % kParts;
  const int j = j0 + jl;
  const int d0 = part * DP;
  float kr[DP], dk[DP], dv[DP], vR[DP];
#pragma unroll
  for (int e = 0; e < DP; ++e) {
    kr[e] = static_cast<float>(skv[0][jl][d0 + e]);
    dk[e] = static_cast<float>(skv[1][jl][d0 + e]) - kr[e];
    const float vr = static_cast<float>(skv[2][jl][d0 + e]);
    vR[e] = static_cast<float>(skv[3][jl][d0 + e]);
    dv[e] = vR[e] - vr;
  }

  // ---- query columns (row i, head h*G + x) in chunks of kPeCols ------------
  const int nq = grp.n_rows * p.G;
  float acc = 0.f;
  float kappa = 0.f;
  for (int c0 = 0; c0 < nq; c0 += kPeCols) {
    __syncthreads();  // the previous chunk's readers are done
    for (int idx = tid; idx < kPeCols * D; idx += kPeThreads) {
      const int cl = idx / D, dd = idx % D;
      const int col = c0 + cl;
      float qv = 0.f, ov = 0.f;
      if (col < nq) {
        const size_t qi = (size_t(grp.row_start + col / p.G) * p.Hq + size_t(h) * p.G + col % p.G) * D + dd;
        qv = static_cast<float>(static_cast<const T*>(p.q)[qi]);
        ov = p.o[qi];
      }
      sq[cl][dd] = qv;
      so[cl][dd] = ov;
    }
    if (tid < kPeCols) {
      const int col = c0 + tid;
      sl[tid] = col < nq ? p.lse[size_t(grp.row_start + col / p.G) * p.Hq + size_t(h) * p.G + col % p.G] : 0.f;
    }
    __syncthreads();
    const int nc = min(kPeCols, nq - c0);
    for (int cl = 0; cl < nc; ++cl) {
      float s = 0.f, ds = 0.f;
#pragma unroll
      for (int e = 0; e < DP; ++e) {
        const float qe = sq[cl][d0 + e];
        s = fmaf(qe, kr[e], s);
        ds = fmaf(qe, dk[e], ds);
      }
#pragma unroll
      for (int m = 1; m < kParts; m <<= 1) {
        s += __shfl_xor(s, m);
        ds += __shfl_xor(ds, m);
      }
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
#pragma unroll
  for (int m = 1; m < kParts; m <<= 1) acc += __shfl_xor(acc, m);
  if (part == 0 && j < grp.T) {
    const size_t at = (size_t(p.g0 + gl) * p.H + h) * p.t_max + j;
    p.part[at] = acc;
    p.part_cond[at] = kappa;  // the same in all of the position's lanes
  }
}

// e[g][j] = sum over KV heads in order, cond[g][j] = their largest kappa
// (both 0 for j >= T).
__global__ __launch_bounds__(256) void position_error_sum_kernel(const PosErrParams p) {
  const int gl = blockIdx.y;
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= p.t_max) return;
  const int g = p.g0 + gl;
  const int T = p.grp[gl].T;
  float s = 0.f, k = 0.f;
  if (j < T)
    for (int h = 0; h < p.H; ++h) {
      s += p.part[(size_t(g) * p.H + h) * p.t_max + j];
      k = fmaxf(k, p.part_cond[(size_t(g) * p.H + h) * p.t_max + j]);
    }
  p.err[size_t(g) * p.t_max + j] = s;
  if (p.cond != nullptr) p.cond[size_t(g) * p.t_max + j] = k;
}

template <typename T, int D>
hipError_t launch_t(const PosErrParams& p, hipStream_t stream) {
  void* args[] = {const_cast<PosErrParams*>(&p)};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&position_error_kernel<T, D>),
                                 dim3(p.t_max / kPeTile, p.H, p.n_grp), dim3(kPeThreads), args, 0, stream);
  if (e != hipSuccess) return e;
  return hipLaunchKernel(reinterpret_cast<const void*>(&position_error_sum_kernel),
                         dim3((p.t_max + 255) / 256, p.n_grp), dim3(256), args, 0, stream);
}

}  // namespace

hipError_t launch_position_error(const PosErrParams& p, int dtype, int D, hipStream_t stream) {
  if (p.n_grp <= 0) return hipSuccess;
  if (dtype == 1) return D == 128 ? launch_t<__bf16, 128>(p, stream) : launch_t<__bf16, 64>(p, stream);
  return D == 128 ? launch_t<float, 128>(p, stream) : launch_t<float, 64>(p, stream);
}

}  // namespace ripe
