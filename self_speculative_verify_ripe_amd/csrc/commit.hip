// commit.hip -- scatter accepted draft rows into one recurrent layer's cache.
//
// RIPE abstract (zhuanzhiai.com paper page): RIPE keeps the deepest plane at
// every position and full depth only for a window of recent positions.  A
// commit therefore writes plane R of every accepted row to the deep region
// and planes 1..R-1 of the rows that end up inside the window to ring slot
// j mod We; a position leaving the window needs no copy because its plane R
// is already in the deep region and the position W later reuses its slot.
// FULL writes planes 1..R, DEEPEST plane R.  LoopSpec summary (rit.work):
// rejected rows are simply not committed.
//
// One thread copies 8 consecutive head-dim elements of one (row, plane,
// head): a 16- or 32-byte K row piece, and 8 V elements into the transposed
// V blocks (32 positions each; a RIPE ring whose width We is not a multiple
// of 32 ends with one block of We mod 32 slots).  Paged caches: the host cuts jobs at page boundaries
// and gives each main-region job its page.  Destinations (position, plane, head, element) are
// distinct across threads, so the writes never race.
#include <hip/hip_runtime.h>

#include "plan.h"

namespace ripe {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename T, int D>
__global__ __launch_bounds__(256) void commit_rows(const CommitParams p) {
  const int item = blockIdx.x * 256 + threadIdx.x;
  if (item >= p.n_items) return;
  int lo = 0, hi = p.n_jobs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.job[mid].item0 <= item)
      lo = mid;
    else
      hi = mid - 1;
  }
  const CommitJob& jb = p.job[lo];
  constexpr int CH = D / 8;
  int local = item - jb.item0;
  const int ch = local % CH;
  local /= CH;
  const int h = local % p.H;
  local /= p.H;
  const int pi = local % jb.n_planes;
  const int ri = local / jb.n_planes;
  const int pl = jb.plane_lo + pi;  // 1-based plane
  const int j = jb.j0 + ri;
  const int src = jb.src0 + ri;
  const size_t Hd = size_t(p.H) * D;
  const T* kv = static_cast<const T*>(p.kv_new);
  const T* ks = kv + (size_t(pl - 1) * p.n_rows + src) * Hd + size_t(h) * D + ch * 8;
  const T* vs = kv + (size_t(p.R + pl - 1) * p.n_rows + src) * Hd + size_t(h) * D + ch * 8;
  size_t off;
  int slot;
  int full = 1 << 30;  // slots held in 32-wide V blocks; the rest form one narrower block
  int tail = 0;        // its width
  if (p.layout == 2 && pl < p.R) {
    off = p.ring_off + ((size_t(jb.b) * (p.R - 1) + (pl - 1)) * p.H + h) * size_t(p.We) * D;
    slot = j % p.We;
    full = p.We / 32 * 32;
    tail = p.We - full;
  } else if (p.page_len > 0) {  // paged main region: the job's rows share one page
    off = (((p.layout == 0) ? size_t(jb.page) * p.R + (pl - 1) : size_t(jb.page)) * p.H + h) *
          size_t(p.page_len) * D;
    slot = j % p.page_len;
  } else if (p.layout == 0) {
    off = ((size_t(jb.b) * p.R + (pl - 1)) * p.H + h) * size_t(p.t_max) * D;
    slot = j;
  } else {
    off = (size_t(jb.b) * p.H + h) * size_t(p.t_max) * D;
    slot = j;
  }
  T* kd = static_cast<T*>(p.cache_k) + off + size_t(slot) * D + ch * 8;
  constexpr int NV = 8 * sizeof(T) / 16;  // 16-byte pieces per 8 elements
#pragma unroll
  for (int v = 0; v < NV; ++v)
    reinterpret_cast<u32x4*>(kd)[v] = reinterpret_cast<const u32x4*>(ks)[v];
  T vv[8];
#pragma unroll
  for (int v = 0; v < NV; ++v) reinterpret_cast<u32x4*>(vv)[v] = reinterpret_cast<const u32x4*>(vs)[v];
  T* vd = static_cast<T*>(p.cache_v) + off;
  // element (slot, d) of a [D][w] block that starts at slot b0: b0 * D + d * w + (slot - b0)
  const int b0 = slot < full ? slot / 32 * 32 : full;
  const int w = slot < full ? 32 : tail;
#pragma unroll
  for (int e = 0; e < 8; ++e) vd[size_t(b0) * D + size_t(ch * 8 + e) * w + (slot - b0)] = vv[e];
}

template <typename T, int D>
static hipError_t launch_commit_t(const CommitParams& p, hipStream_t stream) {
  const int blocks = (p.n_items + 255) / 256;
  if (blocks == 0) return hipSuccess;
  void* args[] = {const_cast<CommitParams*>(&p)};
  return hipLaunchKernel(reinterpret_cast<const void*>(&commit_rows<T, D>), dim3(blocks), dim3(256),
                         args, 0, stream);
}

hipError_t launch_commit(const CommitParams& p, int dtype, int D, hipStream_t stream) {
  if (dtype == 1) return D == 128 ? launch_commit_t<__bf16, 128>(p, stream) : launch_commit_t<__bf16, 64>(p, stream);
  return D == 128 ? launch_commit_t<float, 128>(p, stream) : launch_commit_t<float, 64>(p, stream);
}

}  // namespace ripe
