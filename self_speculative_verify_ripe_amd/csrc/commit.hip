// commit.hip -- scatter accepted draft rows into one recurrent layer's cache.
//
// RIPE abstract (zhuanzhiai.com paper page, sentence introducing RIPE): RIPE
// keeps the deepest plane at every position and the other planes only for a
// window of recent positions.  A commit therefore writes plane R of every
// accepted row to the deep region and planes 1..R-1 of the rows that end up
// inside the window to ring slot j mod We; a position leaving the window
// needs no copy because its plane R is already in the deep region and the
// position W later reuses its slot.  FULL writes planes 1..R, DEEPEST plane
// R.  LoopSpec summary (rit.work): rejected rows are simply not committed.
//
// One wavefront per (plane, head, block of 8 slots) writes everything a
// commit puts in that block.  K rows are contiguous per (position, head):
// the wavefront copies the rows of the block's new slots, 16 bytes per lane.
// V is stored transposed in blocks of 8 slots ([D][8]: each head
// dimension's 8 values one 16- or 32-byte run, a block 2 or 4 KB at
// D = 128), so a commit of a few positions touches one or two blocks per
// (plane, head).  The wavefront rewrites the block's runs whole -- a lane
// reads a run unless every slot of it is new, puts the new values in and
// writes the run back; the other slots keep their bytes -- so the stores
// cover whole cache lines.  (The cache lines a commit dirties, not the
// bytes it writes, set what the write-back costs the verify calls that
// stream the cache next; 32-slot blocks would make a commit of 4 positions
// dirty 4 times the lines.)
// The stores are non-temporal: the rows are read again only by later
// calls, and lines left dirty in the caches would be written back while
// those calls stream (c4 loop: the verify call after a commit 60.9 -> 58.8
// us).  Jobs and blocks are planned so that no two tasks of a launch touch
// one block.
// Paged caches: the host cuts jobs at page boundaries and gives each
// main-region job its page.
#include <hip/hip_runtime.h>

#include "plan.h"

namespace ripe {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// element offset of the (plane pl, head h) region of a job: K row of slot s
// at off + s * D; V of slot s, dimension d in its block (see the layout)
__device__ inline size_t region_off(const CommitParams& p, const CommitJob& jb, int pl, int h, int D) {
  if (jb.ring > 0) return p.ring_off + ((size_t(jb.b) * (p.R - 1) + (pl - 1)) * p.H + h) * size_t(p.We) * D;
  if (p.page_len > 0)
    return (((p.layout == 0) ? size_t(jb.page) * p.R + (pl - 1) : size_t(jb.page)) * p.H + h) * size_t(p.page_len) * D;
  if (p.layout == 0) return ((size_t(jb.b) * p.R + (pl - 1)) * p.H + h) * size_t(p.t_max) * D;
  return (size_t(jb.b) * p.H + h) * size_t(p.t_max) * D;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void commit_rows(const CommitParams p) {
  // one wavefront per (job, plane, head, block of kVBlock slots): grid row
  // y is job y (read with one argument load; a search over the job table
  // cost the c4 commit 4 us), and the rows of shorter jobs end early
  const CommitJob& jb = p.job[blockIdx.y];
  int local = int(blockIdx.x) * 4 + int(threadIdx.x >> 6);
  if (local >= jb.n_tasks) return;
  const int lane = threadIdx.x & 63;
  const T* kv = static_cast<const T*>(p.kv_new);
  const size_t Hd = size_t(p.H) * D;
  const int nb = jb.nblk0 + jb.nblk1;
  const int bi = local % nb;
  local /= nb;
  const int blk = bi < jb.nblk0 ? jb.blk0 + bi : jb.blk1 + (bi - jb.nblk0);
  const int h = local % p.H;
  const int pl = jb.plane_lo + local / p.H;                          // 1-based plane
  const int bs = blk * kVBlock;                                     // first slot of the block
  const int w = jb.ring > 0 ? min(kVBlock, jb.ring - bs) : kVBlock;  // its slots
  // row of slot s (or -1): main regions s0 + i, rings (s0 + i) mod We
  auto row_of = [&](int s) -> int {
    int i = s - jb.s0;
    if (jb.ring > 0 && i < 0) i += jb.ring;
    return (i >= 0 && i < jb.n_rows) ? i : -1;
  };
  int n_new = 0;
#pragma unroll
  for (int s = 0; s < kVBlock; ++s) n_new += (s < w && row_of(bs + s) >= 0);
  const size_t reg = region_off(p, jb, pl, h, D);

  // ---- K: the rows of the block's new slots, 16 bytes per lane and step
  constexpr int CPR = D * int(sizeof(T)) / 16;  // 16-byte chunks per row
  const T* ksrc = kv + (size_t(pl - 1) * p.n_rows + jb.src0) * Hd + size_t(h) * D;
  u32x4* const kdst = reinterpret_cast<u32x4*>(static_cast<T*>(p.cache_k) + reg + size_t(bs) * D);
  for (int c = lane; c < n_new * CPR; c += 64) {
    const int r = c / CPR, ch = c % CPR;
    int slot = 0, seen = 0;  // the block's r-th new slot
    for (int s = 0; s < w; ++s)
      if (row_of(bs + s) >= 0 && seen++ == r) {
        slot = s;
        break;
      }
    const u32x4 x = reinterpret_cast<const u32x4*>(ksrc + size_t(row_of(bs + slot)) * Hd)[ch];
    __builtin_nontemporal_store(x, kdst + size_t(slot) * CPR + ch);
  }

  // ---- V: lane l rewrites the runs of head dimensions l, l + 64, ...
  T* vb = static_cast<T*>(p.cache_v) + reg + size_t(bs) * D;
  const T* vsrc = kv + (size_t(p.R + pl - 1) * p.n_rows + jb.src0) * Hd + size_t(h) * D;
  if (w == kVBlock) {
    constexpr int NQ = kVBlock * sizeof(T) / 16;  // 16-byte pieces per run
#pragma unroll
    for (int d = lane; d < D; d += 64) {
      u32x4* run = reinterpret_cast<u32x4*>(vb + size_t(d) * kVBlock);
      T vals[kVBlock];
      if (n_new < kVBlock) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) reinterpret_cast<u32x4*>(vals)[q] = run[q];
      }
#pragma unroll
      for (int s = 0; s < kVBlock; ++s) {
        const int i = row_of(bs + s);
        if (i >= 0) vals[s] = vsrc[size_t(i) * Hd + d];
      }
#pragma unroll
      for (int q = 0; q < NQ; ++q) __builtin_nontemporal_store(reinterpret_cast<const u32x4*>(vals)[q], run + q);
    }
  } else {
    // a ring's narrower last block: element by element (its runs need not
    // be 16-byte aligned)
    for (int d = lane; d < D; d += 64)
      for (int s = 0; s < w; ++s) {
        const int i = row_of(bs + s);
        if (i >= 0) vb[size_t(d) * w + s] = vsrc[size_t(i) * Hd + d];
      }
  }
}

template <typename T, int D>
static hipError_t launch_commit_t(const CommitParams& p, hipStream_t stream) {
  const int blocks = (p.max_tasks + 3) / 4;
  if (blocks == 0 || p.n_jobs == 0) return hipSuccess;
  void* args[] = {const_cast<CommitParams*>(&p)};
  return hipLaunchKernel(reinterpret_cast<const void*>(&commit_rows<T, D>), dim3(blocks, p.n_jobs), dim3(256),
                         args, 0, stream);
}

hipError_t launch_commit(const CommitParams& p, int dtype, int D, hipStream_t stream) {
  if (dtype == 1) return D == 128 ? launch_commit_t<__bf16, 128>(p, stream) : launch_commit_t<__bf16, 64>(p, stream);
  return D == 128 ? launch_commit_t<float, 128>(p, stream) : launch_commit_t<float, 64>(p, stream);
}

}  // namespace ripe
