// verify.hip -- RIPE verification attention kernels for gfx950 (CDNA4).
//
// What is computed (RIPE abstract, zhuanzhiai.com paper page; LoopSpec
// summary, rit.work): for every draft group g (sequence b, depth r, rows
// i < k) and query head h, softmax attention of q[row, h] over
//   * the committed prefix j < T_b, each position read from the plane its
//     layout selects (FULL: r; DEEPEST: R; RIPE: r inside the window of the
//     last W positions, R before it), and
//   * the group's own draft rows 0..i at depth r,
// with KV head h / (Hq / Hkv).
//
// How (split-K / flash-decoding):
//   one work-group (4 wavefronts) per (sequence, KV head, query-column
//   chunk, chunk of <= S key positions of one segment).  Each wavefront
//   streams 32-position steps straight from HBM into VGPRs in MFMA operand
//   order: K rows (row-major [pos][D]) feed the A operand of S^T = K Q^T, and
//   the V blocks (stored transposed, [D][32] per 32 positions) feed the A
//   operand of O^T += V^T P^T, so no LDS staging or shuffles are needed on
//   the hot loop.  The next step's K (V) loads are issued as soon as the
//   current step's K (V) registers are consumed.  Online softmax in the log2
//   domain with one max reduction per step.  The four wavefronts' (m, l, O)
//   are merged through LDS into one fp32 partial per work item.  A second
//   kernel, one work-group per (sequence, KV head, column chunk), merges the
//   partials in split order, normalises, and writes out (storage dtype,
//   round-to-nearest-even), the natural-log LSE and plane_sel.  (The merge
//   is not folded into the first kernel: cross-work-group hand-off on this
//   multi-die part needs a device-scope fence per work-group, i.e. an L2
//   writeback and invalidate each, which costs far more than the launch.)
//
// MFMA shapes: bf16 v_mfma_f32_16x16x32_bf16 (8 bf16 per lane per operand);
// fp32 v_mfma_f32_16x16x4_f32 (no reduced-precision path).  For the
// 16x16 MFMAs, lane l holds A row / B column l%16 and the k-slots of lane
// group l/16; the accumulator lane l holds column l%16, rows 4*(l/16)+j.
#include <hip/hip_runtime.h>
#include <math.h>

#include "plan.h"

namespace ripe {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename T>
struct Op;

// bf16: one 16-byte chunk = 8 elements = one MFMA k-block of 32.
template <>
struct Op<__bf16> {
  static constexpr int VEC = 8;
  static constexpr int VCH = 1;  // 16-byte chunks per lane per V fragment
  typedef bf16x8 P;              // probability fragment (B operand of P.V)
  __device__ static inline floatx4 mma_k(u32x4 a, u32x4 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  __device__ static inline floatx4 mma_v(const u32x4 (&v)[VCH], const P& p, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v[0]), p, c, 0, 0, 0);
  }
  // round p to the MFMA operand precision; the softmax denominator keeps the
  // unrounded value so that the log-sum-exp is not biased by the rounding
  __device__ static inline void pack(P& dst, int e, float x) { dst[e] = static_cast<__bf16>(x); }
  __device__ static inline void zero_tail(u32x4 (&v)[VCH], int nval) {
    // keep elements e < nval of the 8 bf16 values
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int e0 = 2 * w;
      uint32_t m = 0;
      if (e0 < nval) m |= 0x0000FFFFu;
      if (e0 + 1 < nval) m |= 0xFFFF0000u;
      v[0][w] &= m;
    }
  }
  __device__ static inline void store(void* dst, const float* x, int n) {
    __bf16* d = static_cast<__bf16*>(dst);
    for (int i = 0; i < n; ++i) d[i] = static_cast<__bf16>(x[i]);
  }
  __device__ static inline float ld_elem(const void* base, size_t idx) {
    return static_cast<float>(static_cast<const __bf16*>(base)[idx]);
  }
  __device__ static inline void put_elem(u32x4 (&v)[VCH], int e, const void* base, size_t idx) {
    const uint16_t bits = static_cast<const uint16_t*>(base)[idx];
    const int w = e >> 1;
    if (e & 1)
      v[0][w] = (v[0][w] & 0x0000FFFFu) | (uint32_t(bits) << 16);
    else
      v[0][w] = (v[0][w] & 0xFFFF0000u) | uint32_t(bits);
  }
};

// fp32: one 16-byte chunk = 4 elements = four 16x16x4 MFMAs.
template <>
struct Op<float> {
  static constexpr int VEC = 4;
  static constexpr int VCH = 2;
  struct P {
    float v[8];
  };
  __device__ static inline floatx4 mma_k(u32x4 a, u32x4 b, floatx4 c) {
    const floatx4 fa = __builtin_bit_cast(floatx4, a);
    const floatx4 fb = __builtin_bit_cast(floatx4, b);
#pragma unroll
    for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[e], fb[e], c, 0, 0, 0);
    return c;
  }
  __device__ static inline floatx4 mma_v(const u32x4 (&v)[VCH], const P& p, floatx4 c) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const floatx4 fv = __builtin_bit_cast(floatx4, v[h]);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(fv[e], p.v[4 * h + e], c, 0, 0, 0);
    }
    return c;
  }
  __device__ static inline void pack(P& dst, int e, float x) { dst.v[e] = x; }
  __device__ static inline void zero_tail(u32x4 (&v)[VCH], int nval) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (e >= nval) v[e >> 2][e & 3] = 0u;
  }
  __device__ static inline void store(void* dst, const float* x, int n) {
    float* d = static_cast<float*>(dst);
    for (int i = 0; i < n; ++i) d[i] = x[i];
  }
  __device__ static inline float ld_elem(const void* base, size_t idx) {
    return static_cast<const float*>(base)[idx];
  }
  __device__ static inline void put_elem(u32x4 (&v)[VCH], int e, const void* base, size_t idx) {
    v[e >> 2][e & 3] = static_cast<const uint32_t*>(base)[idx];
  }
};

__device__ inline u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

__device__ inline float wave_max_lanegroups(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

__device__ inline float wave_sum_lanegroups(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

// Locate the group, row and head-in-group of query column `col` of sequence
// record `sr`.  Returns the group record index, or -1 for a padding column.
__device__ inline int column_group(const VerifyParams& p, const SeqRec& sr, int col, int& row, int& hh) {
  if (col >= sr.nq) return -1;
  int off = 0;
  for (int i = 0; i < sr.g_count; ++i) {
    const GroupRec& g = p.grp[sr.g_begin + i];
    const int nc = g.n_rows * p.G;
    if (col < off + nc) {
      row = (col - off) / p.G;
      hh = (col - off) % p.G;
      return sr.g_begin + i;
    }
    off += nc;
  }
  return -1;
}

// Raw buffer resource over [base, base + bytes): loads past the end return 0,
// which masks key rows past a segment's end without per-lane branches.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

__device__ inline size_t uniform_u64(size_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(x));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(x >> 32));
  return (size_t(hi) << 32) | lo;
}

__device__ inline u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// The same load with the non-temporal (evict-first) cache policy, sc0 | nt,
// for the V blocks, which are read once.  Measured per call against the
// default policy: c3 -4%, c5 FULL -4%, c5 RIPE -8%, c4 -2%; giving the K rows
// the same hint as well helps c4 (-15%) but costs c3 and c5, and K alone helps
// none.
__device__ inline u32x4 bload16_stream(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 3));
}

// Running softmax state of one wavefront for its NB 16-column blocks.  The
// reference maximum m only moves when a step's maximum exceeds it by more than
// kLazy (log2 units) -- probabilities stay <= 2^kLazy -- so the accumulator
// rescale is rare; the decision is wave-uniform.
constexpr float kLazy = 8.0f;

template <typename T, int D, int NB>
struct Softmax {
  using O = Op<T>;
  static constexpr int DB = D / 16;
  float m[NB], l[NB];
  floatx4 acc[DB][NB];

  __device__ inline void init() {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      m[nb] = -INFINITY;
      l[nb] = 0.f;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db][nb] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
  }

  // scores of one 32-position step: sacc[mb][nb][j] is position 8*lg+4*mb+j
  // of column ln+16*nb; positions >= lim[nb] (step-local) are invisible.
  // When `hole` is set (wave-uniform) the step is a run of ring slots and the
  // slots whose age rank (slot - ring_base mod We) is below hole_len are
  // invisible too; slot0 is this step's first slot.
  __device__ inline void update(const floatx4 (&sacc)[2][NB], const int (&lim)[NB], float sl2,
                                typename O::P (&pf)[NB], bool hole = false, int slot0 = 0, int ring_base = 0,
                                int hole_len = 0, int We = 0) {
    const int lg = (threadIdx.x & 63) >> 4;
    float x[NB][8];
    bool grow = false;
    float mref[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float mx = -INFINITY;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = 4 * mb + j;
          const float v = (8 * lg + e < lim[nb]) ? sacc[mb][nb][j] * sl2 : -INFINITY;
          x[nb][e] = v;
        }
      if (hole) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          int rel = slot0 + 8 * lg + e - ring_base;
          if (rel < 0) rel += We;
          if (rel < hole_len) x[nb][e] = -INFINITY;
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, x[nb][e]);
      mx = wave_max_lanegroups(mx);
      const bool g = (mx > m[nb] + kLazy) || (m[nb] == -INFINITY && mx != -INFINITY);
      mref[nb] = g ? mx : m[nb];
      grow |= g;
    }
    if (__any(grow)) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const float alpha = (mref[nb] == m[nb]) ? 1.f : __builtin_amdgcn_exp2f(m[nb] - mref[nb]);
        l[nb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db][nb] *= alpha;
        m[nb] = mref[nb];
      }
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const float mu = (m[nb] == -INFINITY) ? 0.f : m[nb];
      float ps = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pe = __builtin_amdgcn_exp2f(x[nb][e] - mu);
        O::pack(pf[nb], e, pe);
        ps += pe;
      }
      l[nb] += ps;
    }
  }

  template <int VCH>
  __device__ inline void pv(const u32x4 (&vf)[DB][VCH], const typename O::P (&pf)[NB]) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[db][nb] = O::mma_v(vf[db], pf[nb], acc[db][nb]);
  }
};

template <typename T, int D, int NB>
__device__ inline void qk(const u32x4 (&kf)[2][D / (4 * Op<T>::VEC)],
                          const u32x4 (&qf)[NB][D / (4 * Op<T>::VEC)], floatx4 (&sacc)[2][NB]) {
  constexpr int KC = D / (4 * Op<T>::VEC);
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      floatx4 a = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < KC; ++c) a = Op<T>::mma_k(kf[mb][c], qf[nb][c], a);
      sacc[mb][nb] = a;
    }
}

// Wavefronts per SIMD the register allocation targets: two work-groups per
// CU, each wavefront with one K/V step in flight ahead of the one it computes.
template <typename T, int D, int NB>
constexpr int waves_per_simd() {
  return 2;
}

// LDS bytes of the verify kernel: the four wavefronts' (m, l, O) for the
// merge, which the draft-row path also uses, one slice per wavefront, to
// transpose V rows.
template <typename T, int D, int NB>
constexpr int verify_lds_bytes() {
  constexpr int merge = kWaves * 16 * NB * (D + 4) * 4 + 2 * kWaves * 16 * NB * 4;
  constexpr int draft = kWaves * kStep * D * int(sizeof(T));
  return merge > draft ? merge : draft;
}

// Work items: one piece of one sequence for one KV head and one query-column
// chunk (see plan.h).  A work-group runs either one long item, its steps
// spread over the four wavefronts and merged through LDS, or up to four short
// items, one per wavefront, each wavefront writing its own partial.  The
// host's work-group table says which; the hardware dispatches work-groups in
// grid order.  INF: the launch has in-flight parent blocks (parent segments,
// ring slots hidden by the parent); launches without them use the kernel
// compiled without that code, whose step loop it would otherwise slow down.
// PG, paged caches: 1 when every prefix-plane piece lies inside one page
// (read from that page), 2 when pieces may span pages (such a piece is read
// step by step: each 32-position step lies inside one page); 0 unpaged.  The
// step-by-step code is compiled only into PG = 2, whose loop it slows.
template <typename T, int D, int NB, bool INF, int PG = 0>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(waves_per_simd<T, D, NB>())))
void verify_attn_kernel(const VerifyParams p, const ItemTable tab) {
  using O = Op<T>;
  constexpr int VEC = O::VEC;
  constexpr int VCH = O::VCH;
  constexpr int KC = D / (4 * VEC);  // 16-byte K/Q chunks per lane per 16-row MFMA block
  constexpr int DB = D / 16;         // 16-wide head-dim blocks of the output
  constexpr int CQ = 16 * NB;        // query columns per work-group
  constexpr int E = sizeof(T);
  constexpr int TPC = kThreads / CQ;  // epilogue threads per column
  constexpr int DPT = D / TPC;        // head-dim values per epilogue thread
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ln = lane & 15;
  const int lg = lane >> 4;

  __shared__ __attribute__((aligned(16))) unsigned char lds_raw[verify_lds_bytes<T, D, NB>()];

  // ---- this work item (host-planned; wave-uniform) ----------------------
  // A long item: wavefront w runs steps w, w + 4, ...  A short one: the
  // wavefront runs every step of its own item.
  const uint32_t wge = tab.wg[blockIdx.x];
  const bool solo = (wge & kWgSolo) != 0;
  if (solo && wave > int((wge >> 11) & 3)) return;  // (short items only: no barrier follows)
  const int idx = int(wge & 0x7ffu) + (solo ? wave : 0);
  const int st0 = solo ? 0 : wave;
  const int sstride = solo ? 1 : kWaves;
  const Item it = tab.item[idx];
  const Piece pc = tab.piece[it.piece];
  const int h = it.h;
  const int cc = it.cc;
  const SeqRec sr = p.seq[pc.s];
  const int Wb = min(p.We, sr.T);
  const int nsteps = ceil_div(pc.len, kStep);

  // ---- query columns of this lane ---------------------------------------
  // Straight-line on purpose: every lane loads from a valid address and
  // padding columns are zeroed by selects, with no loads under divergent
  // control flow.  hi[nb]: piece-local end of what the column sees.
  int hi[NB];
  u32x4 qf[NB][KC];
  auto setup_columns = [&]() {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int col = cc * CQ + ln + 16 * nb;
      int row = 0, hh = 0;
      const int gi = column_group(p, sr, col, row, hh);
      const bool valid = gi >= 0;
      const GroupRec& g = p.grp[valid ? gi : sr.g_begin];
      const T* qp = static_cast<const T*>(p.q) + (size_t(g.row_start + row) * p.Hq + size_t(h) * p.G + hh) * D;
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const u32x4 v = ld16(qp + c * 4 * VEC + lg * VEC);
        qf[nb][c] = valid ? v : u32x4{0u, 0u, 0u, 0u};
      }
      const int gd = g.depth;
      int hv;
      if (pc.kind == kSegPlane)
        hv = (p.layout == 0) ? (gd == pc.depth ? sr.T : 0)
             : (p.layout == 1) ? sr.T
                               : (gd == p.R ? sr.T : sr.tw);
      else if (pc.kind == kSegRing)
        hv = (gd == pc.depth) ? Wb : 0;
      else if (!INF || pc.kind == kSegDraft)
        hv = (gi == pc.gidx) ? row + 1 : 0;
      else if (pc.kind == kSegParentDeep)  // in-flight parent rows: all visible
        hv = pc.c0 + pc.len;
      else
        hv = (gd == pc.depth) ? pc.c0 + pc.len : 0;
      hi[nb] = valid ? hv - pc.c0 : 0;
    }
  };

  Softmax<T, D, NB> sm;
  sm.init();
  const float sl2 = p.scale_log2;
  u32x4 kf[2][KC], vf[DB][VCH];

  // Wavefront w runs steps w, w + 4, ... of the piece.
  if (INF ? (pc.kind == kSegPlane || pc.kind == kSegRing) : pc.kind != kSegDraft) {
    // ---- prefix plane or window ring: raw buffer loads ------------------
    // The buffer resources span the piece only: loads past its end return
    // zeros.
    size_t off;
    int bw = kStep;
    // a paged prefix-plane piece inside one page is addressed like an
    // unpaged one; one that spans pages is read step by step (below)
    const int P = PG > 0 ? p.page_len : 1;
    const bool plane_paged = PG > 0 && pc.kind == kSegPlane;
    const bool per_step = PG == 2 && plane_paged && (pc.c0 + pc.len - 1) / P != pc.c0 / P;
    auto page_base = [&](int pos) -> size_t {  // element offset of position pos of the piece's pages
      const int k = pos / P - pc.c0 / P;      // page of the piece
      const size_t pg = size_t(k == 0 ? tab.pages[it.piece] : tab.pages[kMaxPieces + tab.pref[it.piece] + k - 1]);
      return (((p.layout == 0) ? pg * p.R + (pc.depth - 1) : pg) * p.H + h) * size_t(P) * D + size_t(pos % P) * D;
    };
    if (plane_paged) {
      off = page_base(pc.c0);
    } else if (pc.kind == kSegPlane) {
      off = (((p.layout == 0) ? size_t(sr.b) * p.R + (pc.depth - 1) : size_t(sr.b)) * p.H + h) *
                size_t(p.t_max) * D +
            size_t(pc.c0) * D;
    } else {
      off = p.ring_off + ((size_t(sr.b) * (p.R - 1) + (pc.depth - 1)) * p.H + h) * size_t(p.We) * D +
            size_t(pc.c0) * D;  // c0 is a multiple of 32, and of the ring's block width
      bw = p.BW;
    }
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(static_cast<const T*>(p.cache_k) + off, uint32_t(pc.len) * D * E);
    const __amdgpu_buffer_rsrc_t vrs =
        make_rsrc(static_cast<const T*>(p.cache_v) + off, uint32_t(ceil_div(pc.len, bw)) * bw * D * E);
    const uint32_t krow = uint32_t(8 * (ln >> 2) + (ln & 3));
    const uint32_t koff = (krow * D + lg * VEC) * E;
    // A step past the piece maps to an offset beyond the resource's range:
    // those loads return zeros without touching memory, so the prefetch
    // below is unconditional and the wait counts stay exact.
    constexpr uint32_t kOutOfRange = 0x80000000u;
    // A piece spanning pages: the step's K rows are one 32-row run of its
    // page and its V values one [D][32] block, so each step gets resources of
    // its own (a step past the piece reads the piece's last page, out of range).
    auto step_base = [&](int st) -> size_t { return page_base(pc.c0 + min(st, nsteps - 1) * kStep); };
    auto load_k = [&](int st, bool live, u32x4 (&k)[2][KC]) {
      __amdgpu_buffer_rsrc_t rs = krs;
      uint32_t base = live ? uint32_t(st * kStep) * D * E + koff : kOutOfRange;
      if (PG == 2 && per_step) {
        rs = make_rsrc(static_cast<const T*>(p.cache_k) + step_base(st),
                       uint32_t(min(kStep, pc.len - min(st, nsteps - 1) * kStep)) * D * E);
        base = live ? koff : kOutOfRange;
      }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int c = 0; c < KC; ++c) k[mb][c] = bload16(rs, base + (4 * mb * D + c * 4 * VEC) * E);
    };
    auto load_v = [&](int st, bool live, u32x4 (&v)[DB][VCH]) {
      __amdgpu_buffer_rsrc_t rs = vrs;
      const int slot0 = st * kStep + 8 * lg;
      const int blk = slot0 / bw;
      uint32_t base = live ? uint32_t((blk * D + ln) * bw + (slot0 - blk * bw)) * E : kOutOfRange;
      if (PG == 2 && per_step) {  // bw = 32: the step is one whole V block
        rs = make_rsrc(static_cast<const T*>(p.cache_v) + step_base(st), uint32_t(kStep) * D * E);
        base = live ? uint32_t(ln * kStep + 8 * lg) * E : kOutOfRange;
      }
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int c = 0; c < VCH; ++c) v[db][c] = bload16_stream(rs, base + (16 * db * bw + c * VEC) * E);
    };
    const bool hole = INF && pc.kind == kSegRing && sr.hole > 0;
    // first step's loads go out before the query setup
    load_k(st0, st0 < nsteps, kf);
    load_v(st0, st0 < nsteps, vf);
    setup_columns();
    for (int st = st0; st < nsteps; st += sstride) {
      const bool more = st + sstride < nsteps;
      floatx4 sacc[2][NB];
      qk<T, D, NB>(kf, qf, sacc);
      load_k(st + sstride, more, kf);
      int lim[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) lim[nb] = hi[nb] - st * kStep;
      // a ring whose oldest slots now lie before the window (a parent block
      // in flight) does not read those slots
      typename O::P pf[NB];
      if constexpr (INF)
        sm.update(sacc, lim, sl2, pf, hole, pc.c0 + st * kStep, sr.ring_base, sr.hole, p.We);
      else
        sm.update(sacc, lim, sl2, pf);
      // a step reaching past the piece's end: zero the V values of the
      // missing positions (they may hold anything, even NaN)
      if ((st + 1) * kStep > pc.len) {
        const int nval = pc.len - (st * kStep + 8 * lg);
#pragma unroll
        for (int db = 0; db < DB; ++db) O::zero_tail(vf[db], nval);
      }
      sm.pv(vf, pf);
      load_v(st + sstride, more, vf);
    }
  } else {
    // ---- a group's own draft rows (kv_new, row-major): K rows are loaded
    // in MFMA order directly; V rows are staged in this wavefront's LDS slice
    // with 16-byte loads and read back transposed.
    setup_columns();
    // the piece's first row: the group's own rows, or the in-flight parent's
    // (the rows before its window first, then the window's)
    const int Hd = p.H * D;
    const size_t row0 = (!INF || pc.kind == kSegDraft
                             ? size_t(p.grp[pc.gidx].row_start)
                             : size_t(sr.parent_row0) + (pc.kind == kSegParentWin ? sr.nd : 0)) +
                        size_t(pc.c0);
    const T* kb = static_cast<const T*>(p.kv_new) + (size_t(pc.depth - 1) * p.n_rows + row0) * Hd + size_t(h) * D;
    const T* vb = static_cast<const T*>(p.kv_new) + (size_t(p.R + pc.depth - 1) * p.n_rows + row0) * Hd + size_t(h) * D;
    T* stage = reinterpret_cast<T*>(lds_raw) + size_t(wave) * kStep * D;  // [32 rows][D]
    constexpr int CPR = D / VEC;  // 16-byte pieces per row
    const int len = pc.len;
    for (int st = st0; st < nsteps; st += sstride) {
      const int base = st * kStep;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int pos = base + 8 * (ln >> 2) + 4 * mb + (ln & 3);
        const bool ok = pos < len;
        const T* rp = kb + size_t(ok ? pos : 0) * Hd + lg * VEC;
#pragma unroll
        for (int c = 0; c < KC; ++c) {
          const u32x4 v = ld16(rp + c * 4 * VEC);
          kf[mb][c] = ok ? v : u32x4{0u, 0u, 0u, 0u};
        }
      }
      // stage V rows [base, base + 32) of this head: piece i = (row, 16 B)
#pragma unroll
      for (int i = lane; i < kStep * CPR; i += 64) {
        const int r = i / CPR;
        const int c = i - r * CPR;
        const bool ok = base + r < len;
        const u32x4 v = ld16(vb + size_t(ok ? base + r : 0) * Hd + c * VEC);
        *reinterpret_cast<u32x4*>(stage + r * D + c * VEC) = ok ? v : u32x4{0u, 0u, 0u, 0u};
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): staged rows are in LDS
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int v = 0; v < VCH; ++v) vf[db][v] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < 8; ++e) O::put_elem(vf[db], e, stage, size_t(8 * lg + e) * D + 16 * db + ln);
      }
      __builtin_amdgcn_wave_barrier();
      floatx4 sacc[2][NB];
      qk<T, D, NB>(kf, qf, sacc);
      int lim[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) lim[nb] = hi[nb] - base;
      typename O::P pf[NB];
      sm.update(sacc, lim, sl2, pf);
      sm.pv(vf, pf);
    }
  }

  const size_t stride = size_t(CQ) * (D + 2);
  float* const part = p.ws + size_t(it.part) * stride;
  if (solo) {
    // ---- a short item's partial, straight from this wavefront's registers
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const float lt = wave_sum_lanegroups(sm.l[nb]);
      const int col = ln + 16 * nb;
      if (cc * CQ + col < sr.nq) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
          *reinterpret_cast<floatx4*>(part + size_t(col) * D + 16 * db + 4 * lg) = sm.acc[db][nb];
        if (lg == 0) {
          part[size_t(CQ) * D + col] = sm.m[nb];
          part[size_t(CQ) * D + CQ + col] = lt;
        }
      }
    }
    return;
  }

  // ---- merge the four wavefronts through LDS, write one partial ----------
  __syncthreads();  // the draft path's staging slices are reused below
  typedef float OSlice[CQ][D + 4];
  OSlice* lds_o = reinterpret_cast<OSlice*>(lds_raw);
  float (*lds_m)[CQ] = reinterpret_cast<float (*)[CQ]>(lds_raw + kWaves * sizeof(OSlice));
  float (*lds_l)[CQ] = lds_m + kWaves;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const float lt = wave_sum_lanegroups(sm.l[nb]);
    const int col = ln + 16 * nb;
#pragma unroll
    for (int db = 0; db < DB; ++db)
      *reinterpret_cast<floatx4*>(&lds_o[wave][col][16 * db + 4 * lg]) = sm.acc[db][nb];
    if (lg == 0) {
      lds_m[wave][col] = sm.m[nb];
      lds_l[wave][col] = lt;
    }
  }
  __syncthreads();
  const int col = threadIdx.x / TPC;
  const int d0 = (threadIdx.x % TPC) * DPT;
  if (cc * CQ + col < sr.nq) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, lds_m[w][col]);
    float f[kWaves];
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = lds_m[w][col];
      f[w] = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
      L += f[w] * lds_l[w][col];
    }
#pragma unroll
    for (int d = 0; d < DPT; d += 4) {
      floatx4 o = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < kWaves; ++w) o += f[w] * *reinterpret_cast<const floatx4*>(&lds_o[w][col][d0 + d]);
      *reinterpret_cast<floatx4*>(part + size_t(col) * D + d0 + d) = o;
    }
    if (d0 == 0) {
      part[size_t(CQ) * D + col] = M;
      part[size_t(CQ) * D + CQ + col] = L;
    }
  }
}

// Merge: one work-group per (sequence, KV head, query-column chunk) and
// head-dim slice of SLICE values.  It combines the unit's split partials in
// split order, normalises and writes its slice of out; slice 0 also writes
// lse, and (KV head 0, chunk 0, slice 0) the sequence's plane_sel rows.
// 32-wide slices give small batches more work-groups (and room to load up to
// 16 splits in one round); larger batches use 64-wide ones.
constexpr int kMergeThreads = 256;  // threads per merge work-group

template <int N>
struct FloatN {
  typedef float type __attribute__((ext_vector_type(N)));
};

template <typename T, int D, int NB, int SLICE>
__global__ __launch_bounds__(kMergeThreads) void verify_merge_kernel(const VerifyParams p, const UnitTable ut) {
  using O = Op<T>;
  constexpr int CQ = 16 * NB;
  constexpr int TPC = kMergeThreads / CQ;  // threads per column
  constexpr int DPT = SLICE / TPC;         // head-dim values per thread
  constexpr int NS = D / SLICE;            // slices per unit
  typedef typename FloatN<DPT>::type VecT;
  const int slice = blockIdx.x % NS;
  const Unit un = ut.unit[blockIdx.x / NS];
  const int cc = un.cc;
  const int h = un.h;
  const size_t stride = size_t(CQ) * (D + 2);
  const float* const part_base = p.ws + size_t(un.part) * stride;
  const int col = threadIdx.x / TPC;
  const int d0 = slice * SLICE + (threadIdx.x % TPC) * DPT;
  {
    // Every column of the chunk is merged (a padding column's partials exist
    // and are merged harmlessly); only the sequence's columns are stored.
    // The loads need nothing but the unit record, so they go out before the
    // sequence and group records that place the outputs are read.
    const int ns = un.n_split;
    // Global maximum first, then the splits' weighted sums in split order.
    // Up to kFast splits are loaded in one round and kept in registers.
    constexpr int kFast = DPT <= 4 ? 16 : 8;
    float M = -INFINITY;
    float L = 0.f;
    float o[DPT];
#pragma unroll
    for (int d = 0; d < DPT; ++d) o[d] = 0.f;
    if (ns <= kFast) {
      float ms[kFast], ls[kFast];
      VecT ov[kFast];
#pragma unroll
      for (int u = 0; u < kFast; ++u) {
        const bool ok = u < ns;
        const float* part = part_base + size_t(ok ? u : 0) * stride;
        ms[u] = ok ? __builtin_nontemporal_load(part + size_t(CQ) * D + col) : -INFINITY;
        ls[u] = __builtin_nontemporal_load(part + size_t(CQ) * D + CQ + col);
        ov[u] = __builtin_nontemporal_load(reinterpret_cast<const VecT*>(part + size_t(col) * D + d0));
      }
#pragma unroll
      for (int u = 0; u < kFast; ++u) M = fmaxf(M, ms[u]);
#pragma unroll
      for (int u = 0; u < kFast; ++u) {
        const float fs = (ms[u] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ms[u] - M);
        L += fs * ls[u];
#pragma unroll
        for (int e = 0; e < DPT; ++e) o[e] += fs * ov[u][e];
      }
    } else {
      constexpr int U = DPT <= 4 ? 8 : 4;  // splits whose loads are issued together
      for (int sp = 0; sp < ns; sp += U) {
        float mm[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
          mm[u] = (sp + u < ns) ? part_base[size_t(sp + u) * stride + size_t(CQ) * D + col] : -INFINITY;
#pragma unroll
        for (int u = 0; u < U; ++u) M = fmaxf(M, mm[u]);
      }
      for (int sp = 0; sp < ns; sp += U) {
        float ms[U], ls[U];
        VecT ov[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const bool ok = sp + u < ns;
          const float* part = part_base + size_t(ok ? sp + u : 0) * stride;
          ms[u] = ok ? __builtin_nontemporal_load(part + size_t(CQ) * D + col) : -INFINITY;
          ls[u] = __builtin_nontemporal_load(part + size_t(CQ) * D + CQ + col);
          ov[u] = __builtin_nontemporal_load(reinterpret_cast<const VecT*>(part + size_t(col) * D + d0));
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const float fs = (ms[u] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ms[u] - M);
          L += fs * ls[u];
#pragma unroll
          for (int e = 0; e < DPT; ++e) o[e] += fs * ov[u][e];
        }
      }
    }
    const SeqRec sr = p.seq[un.s];
    int row = 0, hh = 0;
    const int gi = column_group(p, sr, cc * CQ + col, row, hh);
    if (gi >= 0) {
      const GroupRec& g = p.grp[gi];
      const size_t orow = size_t(g.row_start + row) * p.Hq + size_t(h) * p.G + hh;
      float res[DPT];
#pragma unroll
      for (int d = 0; d < DPT; ++d) res[d] = o[d] / L;
      if (p.out_f32)
        Op<float>::store(static_cast<float*>(p.out) + orow * D + d0, res, DPT);
      else
        O::store(static_cast<T*>(p.out) + orow * D + d0, res, DPT);
      if (p.lse != nullptr && d0 == 0) p.lse[orow] = (M + log2f(L)) * 0.69314718055994530942f;
    }
  }
  const SeqRec sr = p.seq[un.s];
  // plane_sel of the sequence's groups: written once, by unit (h 0, chunk 0), slice 0
  if (p.plane_sel != nullptr && h == 0 && cc == 0 && slice == 0) {
    for (int gi = sr.g_begin; gi < sr.g_begin + sr.g_count; ++gi) {
      const int r = p.grp[gi].depth;
      int8_t* rowp = p.plane_sel + size_t(p.gorig[gi]) * p.t_max;
      for (int j0 = threadIdx.x * 16; j0 < sr.T; j0 += kMergeThreads * 16) {
        int8_t v[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int j = j0 + e;
          const int pl = (p.layout == 0) ? r : (p.layout == 1) ? p.R : ((j >= sr.tw) ? r : p.R);
          v[e] = int8_t(pl);
        }
        if (j0 + 16 <= sr.T) {
          *reinterpret_cast<u32x4*>(rowp + j0) = *reinterpret_cast<const u32x4*>(v);
        } else {
          for (int e = 0; j0 + e < sr.T; ++e) rowp[j0 + e] = v[e];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------
template <typename T, int D, int NB>
static hipError_t launch_verify_t(const VerifyParams& p, const ItemTable& t, const UnitTable& u,
                                  hipStream_t stream) {
  if (p.n_wg <= 0) return hipSuccess;
  const int grid = p.n_blocks;
  void* args[] = {const_cast<VerifyParams*>(&p), const_cast<ItemTable*>(&t)};
  const void* const kerns[2][3] = {
      {reinterpret_cast<const void*>(&verify_attn_kernel<T, D, NB, false, 0>),
       reinterpret_cast<const void*>(&verify_attn_kernel<T, D, NB, false, 1>),
       reinterpret_cast<const void*>(&verify_attn_kernel<T, D, NB, false, 2>)},
      {reinterpret_cast<const void*>(&verify_attn_kernel<T, D, NB, true, 0>),
       reinterpret_cast<const void*>(&verify_attn_kernel<T, D, NB, true, 1>),
       reinterpret_cast<const void*>(&verify_attn_kernel<T, D, NB, true, 2>)}};
  const void* kern = kerns[p.inflight ? 1 : 0][p.page_mode];
  hipError_t e = hipLaunchKernel(kern, dim3(grid), dim3(kThreads), args, 0, stream);
  if (e != hipSuccess) return e;
  // Merge: 64-wide head-dim slices while they still give one work-group per
  // compute unit, else 32-wide ones (more work-groups for few units).
  // Measured against 32-wide slices up to 1024 work-groups and whole rows
  // beyond: c3 and c4 -0.5 us, c5 RIPE -1.6 us per call, c5 FULL (32 units)
  // unchanged.
  void* margs[] = {const_cast<VerifyParams*>(&p), const_cast<UnitTable*>(&u)};
  if (p.n_units * (D / 64) >= 256)
    return hipLaunchKernel(reinterpret_cast<const void*>(&verify_merge_kernel<T, D, NB, 64>),
                           dim3(p.n_units * (D / 64)), dim3(kMergeThreads), margs, 0, stream);
  return hipLaunchKernel(reinterpret_cast<const void*>(&verify_merge_kernel<T, D, NB, 32>),
                         dim3(p.n_units * (D / 32)), dim3(kMergeThreads), margs, 0, stream);
}

hipError_t launch_verify(const VerifyParams& p, const ItemTable& t, const UnitTable& u, int dtype, int D, int NB,
                         hipStream_t stream) {
  if (dtype == 1) {
    if (D == 128) return NB == 1 ? launch_verify_t<__bf16, 128, 1>(p, t, u, stream) : launch_verify_t<__bf16, 128, 2>(p, t, u, stream);
    return NB == 1 ? launch_verify_t<__bf16, 64, 1>(p, t, u, stream) : launch_verify_t<__bf16, 64, 2>(p, t, u, stream);
  }
  if (D == 128) return NB == 1 ? launch_verify_t<float, 128, 1>(p, t, u, stream) : launch_verify_t<float, 128, 2>(p, t, u, stream);
  return NB == 1 ? launch_verify_t<float, 64, 1>(p, t, u, stream) : launch_verify_t<float, 64, 2>(p, t, u, stream);
}

// Resident verify work-groups per compute unit (0 if the runtime cannot say).
template <typename T, int D, int NB>
static int blocks_per_cu_t() {
  static const int n = [] {
    int b = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, reinterpret_cast<const void*>(&verify_attn_kernel<T, D, NB, false, 0>),
                                                     kThreads, 0) != hipSuccess)
      b = 0;
    return b;
  }();
  return n;
}

int verify_blocks_per_cu(int dtype, int D, int NB) {
  if (dtype == 1) {
    if (D == 128) return NB == 1 ? blocks_per_cu_t<__bf16, 128, 1>() : blocks_per_cu_t<__bf16, 128, 2>();
    return NB == 1 ? blocks_per_cu_t<__bf16, 64, 1>() : blocks_per_cu_t<__bf16, 64, 2>();
  }
  if (D == 128) return NB == 1 ? blocks_per_cu_t<float, 128, 1>() : blocks_per_cu_t<float, 128, 2>();
  return NB == 1 ? blocks_per_cu_t<float, 64, 1>() : blocks_per_cu_t<float, 64, 2>();
}

}  // namespace ripe
