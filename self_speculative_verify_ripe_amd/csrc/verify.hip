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
//   the V blocks (stored transposed, [D][8] per 8 positions, so each lane's
//   8 slots of one head dimension are one 16-byte load) feed the A operand
//   of O^T += V^T P^T, so no LDS staging or shuffles are needed on the hot
//   loop.  The next step's K (V) loads are issued as soon as the current
//   step's K (V) registers are consumed.  Online softmax in the log2 domain
//   with one max reduction per step.  The four wavefronts' (m, l, O) are
//   merged through LDS into one fp32 partial per work item.  The partials
//   of a (sequence, KV head, column chunk) unit are merged in split order,
//   normalised and written out (storage dtype, round-to-nearest-even) with
//   the natural-log LSE and plane_sel: by the unit's last work item to
//   finish when all of the unit's items run on one XCD (the planner places
//   them so when a unit has at most 8 items; the hand-off then stays inside
//   one L2), else by a second kernel, one work-group per unit.
//
// MFMA shapes: bf16 v_mfma_f32_16x16x32_bf16 (8 bf16 per lane per operand);
// fp32 v_mfma_f32_16x16x4_f32 (no reduced-precision path).  For the
// 16x16 MFMAs, lane l holds A row / B column l%16 and the k-slots of lane
// group l/16; the accumulator lane l holds column l%16, rows 4*(l/16)+j.
#include <hip/hip_runtime.h>
#include <type_traits>
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
    put_bits(v, e, static_cast<const uint16_t*>(base)[idx]);
  }
  __device__ static inline void put_bits(u32x4 (&v)[VCH], int e, uint32_t bits) {
    const int w = e >> 1;
    if (e & 1)
      v[0][w] = (v[0][w] & 0x0000FFFFu) | (bits << 16);
    else
      v[0][w] = (v[0][w] & 0xFFFF0000u) | (bits & 0xFFFFu);
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
// default policy: c3 -4%, c5 FULL -4%, c5 RIPE -8%, c4 -2%.  The K rows take
// it only in launches that verify several depths of one sequence (the policy
// bit kPolKStream): in that pattern -- one call per layer and step, each
// right after a commit -- K rows loaded with the default policy evict the
// commit's dirty lines from the caches, and their write-back slows the call
// (c4: 60.6 -> 54.2 us, the same as without a commit); where each call
// verifies one depth it costs c2 (+6%, whose steps reuse the last-level
// cache) and c5 (+3%) and gains c3 2%.
__device__ inline u32x4 bload16_stream(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 3));
}

constexpr int kPolOddRing = 1;
constexpr int kPolKStream = 2;

// Split partial of one work item, bytes from its start: O / L of its CQ
// columns, [CQ][D], then M[CQ] and L[CQ] (fp32), then for 16-bit caches the
// columns' scales[CQ].  16-bit caches keep O / L in fp16, scaled per column
// by a power of two 2^k, k >= 0, that keeps the largest |O / L| below 2^15
// (O / L is a weighted mean of V values, so k > 0 only for |V| >= 2^15);
// fp32 caches keep it in fp32, unscaled.  Normalising before rounding keeps
// the fp16 error relative to the values (2^-11), 8 times below the rounding
// of a BF16 output, and halves the partial bytes: c3 46.1 -> 44.1 us, c4
// 53.8 -> 52.6 us per call (same box).
template <typename T, int D, int CQ>
struct PartLayout {
  static constexpr bool kHalf = sizeof(T) == 2;
  static constexpr uint32_t kO = uint32_t(CQ) * D * (kHalf ? 2 : 4);
  static constexpr uint32_t kM = kO;
  static constexpr uint32_t kL = kO + 4 * CQ;
  static constexpr uint32_t kS = kO + 8 * CQ;
  static constexpr uint32_t kBytes = kO + (kHalf ? 12 : 8) * CQ;
};
typedef _Float16 half4 __attribute__((ext_vector_type(4)));

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

// plane_sel rows of a sequence's groups (positions j < T), written by one
// work-group of nthreads threads: the plane each group's depth reads at j.
__device__ inline void write_plane_sel(const VerifyParams& p, const SeqRec& sr, int tid, int nthreads) {
  if (p.plane_sel == nullptr) return;
  for (int gi = sr.g_begin; gi < sr.g_begin + sr.g_count; ++gi) {
    const int r = p.grp[gi].depth;
    int8_t* rowp = p.plane_sel + size_t(p.gorig[gi]) * p.t_max;
    for (int j0 = tid * 16; j0 < sr.T; j0 += nthreads * 16) {
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

// Work items: one part of one sequence's runs for one KV head and one
// query-column chunk (see plan.h).  The four wavefronts take each run's
// 32-position steps in turn -- wavefront w the run's steps w, w + 4, ...,
// streamed runs first, then draft-row runs -- and merge their softmax states
// through LDS into one partial.  Numbering the steps per run keeps a run's
// steps on the same wavefronts whatever other runs the item holds: runs
// that another group of the sequence adds are masked for this group's
// columns and leave its state bit-identical.  A wavefront keeps two run contexts:
// the run of the step it computes and the run of the step it prefetches, so
// the loads of a step in the next run go out before the current step is done
// and a run boundary costs no pipeline bubble.  The hardware dispatches
// work-groups in grid order.  INF: the launch has in-flight parent blocks
// (parent segments, ring slots hidden by the parent); launches without them
// use the kernel compiled without that code, whose step loop it would
// otherwise slow down.  PG, paged caches: 1 when every prefix-plane run lies
// inside one page (read from that page), 2 when runs may span pages (such a
// run is read step by step: each 32-position step lies inside one page); 0
// unpaged.  The step-by-step code is compiled only into PG = 2, whose loop it
// slows.  POL, BF16 only: load-policy bits.  kPolOddRing: a ring of odd width
// We ends with a V block of odd width (We mod 8 slots) whose runs need not
// start on a dword, so V is read with a shift; the code is compiled only
// into the launches whose window needs it (fp32 runs and even widths start
// on a dword, which is all a 16-byte buffer load needs).  kPolKStream: K rows
// are loaded non-temporally (see bload16_stream).
template <typename T, int D, int NB, bool INF, int PG = 0, int POL = 0>
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
  constexpr bool RT = (POL & kPolOddRing) != 0;
  constexpr bool KNT = (POL & kPolKStream) != 0;
  constexpr int TPC = kThreads / CQ;  // epilogue threads per column
  constexpr int DPT = D / TPC;        // head-dim values per epilogue thread
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ln = lane & 15;
  const int lg = lane >> 4;

  __shared__ __attribute__((aligned(16))) unsigned char lds_raw[verify_lds_bytes<T, D, NB>()];

  // ---- this work item (host-planned; wave-uniform) ----------------------
  // The items are in grid order: the first argument read is this item, as
  // three 32-bit words (scalar loads; its 16-bit fields read one by one
  // would be vector loads).
  Item it;
  {
    const uint32_t* w = reinterpret_cast<const uint32_t*>(&tab.item[blockIdx.x]);
    const uint32_t w0 = w[0], w1 = w[1], w2 = w[2];
    // all three before the empty-slot test: sunk below it, the third would
    // be a dependent read of its own
    asm volatile("" ::"s"(w0), "s"(w1), "s"(w2));
    it.r0 = uint16_t(w0);
    it.n_stream = uint8_t(w0 >> 16);
    it.n_run = uint8_t(w0 >> 24);
    it.part = uint16_t(w1);
    it.h = uint16_t(w1 >> 16);
    it.cc = uint16_t(w2);
    it.s = uint16_t(w2 >> 16);
  }
  if (it.n_run == 0) return;  // a grid position with no item (XCD placement)
  const int h = it.h;
  const int cc = it.cc;
  const int r_draft = it.r0 + it.n_stream;  // first draft-row run
  const int r_end = it.r0 + it.n_run;
  const SeqRec sr = p.seq[it.s];
  const int Wb = min(p.We, sr.T);

  // ---- query columns --------------------------------------------------
  // The sequence's first two group records come with its sequence record;
  // any further ones are read with wave-uniform indices.  Each lane selects
  // its own: a record read with a per-lane index would be a vector load, and
  // waiting for it waits for every vector load issued before it.
  // col_info(cols, ...) finds, for N columns of the chunk at once, the group
  // (-1 for a padding column), the offset within the group's columns, the
  // group's first draft row and its depth; a padding column gets the first
  // group's row_start and depth.
  constexpr int kG = 2;
  GroupRec gr[kG];
#pragma unroll
  for (int i = 0; i < kG; ++i) gr[i] = sr.g01[i];
  auto col_info = [&](const auto& col, auto& gi, auto& cofs, auto& crs, auto& dep) {
    constexpr int N = int(std::extent<std::remove_reference_t<decltype(col)>>::value);
#pragma unroll
    for (int j = 0; j < N; ++j) {
      gi[j] = -1;
      cofs[j] = 0;
      crs[j] = gr[0].row_start;
      dep[j] = gr[0].depth;
    }
    int off = 0;
    auto take = [&](const GroupRec& g, int gidx, bool live) {
      const int nc = live ? g.n_rows * p.G : 0;
#pragma unroll
      for (int j = 0; j < N; ++j) {
        const bool in = gi[j] < 0 && col[j] >= off && col[j] < off + nc;
        gi[j] = in ? gidx : gi[j];
        cofs[j] = in ? col[j] - off : cofs[j];
        crs[j] = in ? g.row_start : crs[j];
        dep[j] = in ? int(g.depth) : dep[j];
      }
      off += nc;
    };
    // no branch on the group count: every record load stays ahead of the
    // first use
#pragma unroll
    for (int i = 0; i < kG; ++i) take(gr[i], sr.g_begin + i, i < sr.g_count);
    for (int i = kG; i < sr.g_count; ++i) take(p.grp[sr.g_begin + i], sr.g_begin + i, true);
  };
  // This lane's MFMA columns ln + 16 nb: group, row and depth, kept to resolve
  // each run's visibility.  A padding column's runs are all invisible
  // (run_hi gives it 0), so every one of its scores is replaced by -inf
  // before use and it adds nothing; the MFMA keeps columns apart, so its
  // query values (the first group's first row) never reach another column.
  int cgi[NB], crow[NB], cdep[NB];
  auto setup_columns = [&]() {
    int col[NB], cofs[NB], crs[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) col[nb] = cc * CQ + ln + 16 * nb;
    col_info(col, cgi, cofs, crs, cdep);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) crow[nb] = cofs[nb] / p.G;
  };
  // The chunk's query rows are read once per work-group: thread t loads the
  // 16-byte pieces t, t + 256, ... of the [CQ][D] chunk (column-major over
  // pieces), which go through LDS to every wavefront's MFMA operands.  Four
  // wavefronts loading the whole chunk each put 4x the bytes in flight at the
  // start of the call, when the first work-group on a compute unit already
  // holds the second one's requests back.
  constexpr int QROW = D * E;                    // bytes of one query row
  constexpr int QPR = QROW / 16;                 // 16-byte pieces per row
  constexpr int QPT = (CQ * QPR + kThreads - 1) / kThreads;  // pieces per thread
  constexpr int QLDS = QROW + 16;                // LDS row stride (padded against bank conflicts)
  static_assert(CQ * QLDS <= verify_lds_bytes<T, D, NB>(), "query chunk must fit the LDS");
  u32x4 qpiece[QPT];
  auto load_q_pieces = [&]() {
    int col[QPT], gi[QPT], cofs[QPT], crs[QPT], dep[QPT];
#pragma unroll
    for (int j = 0; j < QPT; ++j) col[j] = cc * CQ + min((int(threadIdx.x) + j * kThreads) / QPR, CQ - 1);
    col_info(col, gi, cofs, crs, dep);
#pragma unroll
    for (int j = 0; j < QPT; ++j) {
      const int row = cofs[j] / p.G;
      const int hh = cofs[j] - row * p.G;
      const int pc = (int(threadIdx.x) + j * kThreads) % QPR;
      const char* qp = static_cast<const char*>(p.q) +
                       ((size_t(crs[j] + row) * p.Hq + size_t(h) * p.G + hh) * D) * E + size_t(pc) * 16;
      qpiece[j] = ld16(qp);
    }
  };
  u32x4 qf[NB][KC];
  auto stage_q = [&]() {
#pragma unroll
    for (int j = 0; j < QPT; ++j) {
      const int i = int(threadIdx.x) + j * kThreads;
      if (i < CQ * QPR)
        *reinterpret_cast<u32x4*>(lds_raw + (i / QPR) * QLDS + (i % QPR) * 16) = qpiece[j];
    }
    __syncthreads();
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int c = 0; c < KC; ++c)
        qf[nb][c] = *reinterpret_cast<const u32x4*>(lds_raw + (ln + 16 * nb) * QLDS + (c * 4 * VEC + lg * VEC) * E);
    __syncthreads();  // the region is the draft rows' staging area afterwards
  };
  // Run-local end of what each column sees in run `pc` (0: nothing).
  auto run_hi = [&](const Piece& pc, int (&hi)[NB]) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int gd = cdep[nb];
      const int gi = cgi[nb];
      int hv;
      if (pc.kind == kSegPlane)
        hv = (p.layout == 0) ? (gd == pc.depth ? sr.T : 0)
             : (p.layout == 1) ? sr.T
                               : (gd == p.R ? sr.T : sr.tw);
      else if (pc.kind == kSegRing)
        hv = (gd == pc.depth) ? Wb : 0;
      else if (!INF || pc.kind == kSegDraft)
        hv = (gi == pc.gidx) ? crow[nb] + 1 : 0;
      else if (pc.kind == kSegParentDeep)  // in-flight parent rows: all visible
        hv = pc.c0 + pc.len;
      else
        hv = (gd == pc.depth) ? pc.c0 + pc.len : 0;
      hi[nb] = gi >= 0 ? hv - pc.c0 : 0;
    }
  };

  Softmax<T, D, NB> sm;
  sm.init();
  const float sl2 = p.scale_log2;
  u32x4 kf[2][KC], vf[DB][VCH];

  // ---- streamed runs (prefix planes, rings): raw buffer loads ------------
  // A run context: the buffer resources of one run (they span the run only:
  // loads past its end return zeros), its ns steps, and its visibility (set
  // once the columns are known).
  struct Ctx {
    __amdgpu_buffer_rsrc_t krs, vrs;
    int r, ns, len, c0, vlim, depth;
    bool ring, per_step;
    int hi[NB];
  };
  const int P = PG > 0 ? p.page_len : 1;
  // element offset of position pos of run pc's pages (paged caches)
  auto page_base = [&](int r, const Piece& pc, int pos) -> size_t {
    const int k = pos / P - pc.c0 / P;  // page of the run
    const size_t pg = size_t(k == 0 ? tab.pages[r] : tab.pages[kMaxPieces + tab.pref[r] + k - 1]);
    return (((p.layout == 0) ? pg * p.R + (pc.depth - 1) : pg) * p.H + h) * size_t(P) * D + size_t(pos % P) * D;
  };
  auto make_ctx = [&](int r, Ctx& c) {
    const Piece pc = tab.piece[r];
    c.r = r;
    c.ns = ceil_div(pc.len, kStep);
    c.len = pc.len;
    c.c0 = pc.c0;
    c.depth = pc.depth;
    c.ring = pc.kind == kSegRing;
    // slots from the run's start to the end of the region's V blocks: the
    // ring's last block is narrower when We is not a multiple of 8
    c.vlim = c.ring ? p.We - pc.c0 : (1 << 30);
    const bool plane_paged = PG > 0 && !c.ring;
    c.per_step = PG == 2 && plane_paged && (pc.c0 + pc.len - 1) / P != pc.c0 / P;
    size_t off;
    if (plane_paged) {
      off = page_base(r, pc, pc.c0);
    } else if (!c.ring) {
      off = (((p.layout == 0) ? size_t(sr.b) * p.R + (pc.depth - 1) : size_t(sr.b)) * p.H + h) *
                size_t(p.t_max) * D +
            size_t(pc.c0) * D;
    } else {
      off = p.ring_off + ((size_t(sr.b) * (p.R - 1) + (pc.depth - 1)) * p.H + h) * size_t(p.We) * D +
            size_t(pc.c0) * D;  // c0 is a multiple of 32: a V block starts there
    }
    c.krs = make_rsrc(static_cast<const T*>(p.cache_k) + off, uint32_t(pc.len) * D * E);
    c.vrs = make_rsrc(static_cast<const T*>(p.cache_v) + off,
                      uint32_t(min((c.len + 7) / 8 * 8, c.vlim)) * D * E);  // to the run's last V block
  };
  // move (c, st) on to this wavefront's next step: st + 4 in the same run,
  // else step `wave` of the next run that has one; returns false past the
  // item's last streamed run
  auto advance = [&](Ctx& c, int& st) -> bool {
    while (st >= c.ns) {
      if (c.r + 1 >= r_draft) return false;
      make_ctx(c.r + 1, c);
      st = wave;
    }
    return true;
  };
  const uint32_t krow = uint32_t(8 * (ln >> 2) + (ln & 3));
  const uint32_t koff = (krow * D + lg * VEC) * E;
  // A step past the item maps to an offset beyond the resource's range:
  // those loads return zeros without touching memory, so the prefetch below
  // is unconditional and the wait counts stay exact.
  constexpr uint32_t kOutOfRange = 0x80000000u;
  // A run spanning pages: the step's K rows are one 32-row run of its page
  // and its V values four [D][8] blocks, so each step gets resources of its
  // own.
  auto step_base = [&](const Ctx& c, int st) -> size_t {
    const Piece pc = tab.piece[c.r];
    return page_base(c.r, pc, pc.c0 + min(st, c.ns - 1) * kStep);
  };
  auto load_k = [&](const Ctx& c, int st, bool live, u32x4 (&k)[2][KC]) {
    __amdgpu_buffer_rsrc_t rs = c.krs;
    uint32_t base = live ? uint32_t(st * kStep) * D * E + koff : kOutOfRange;
    if (PG == 2 && c.per_step) {
      rs = make_rsrc(static_cast<const T*>(p.cache_k) + step_base(c, st),
                     uint32_t(min(kStep, c.len - min(st, c.ns - 1) * kStep)) * D * E);
      base = live ? koff : kOutOfRange;
    }
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int cch = 0; cch < KC; ++cch) {
        const uint32_t o = base + (4 * mb * D + cch * 4 * VEC) * E;
        if constexpr (KNT)
          k[mb][cch] = bload16_stream(rs, o);
        else
          k[mb][cch] = bload16(rs, o);
      }
  };
  // V is stored in blocks of 8 slots [D][8] (a ring's last block holds
  // We mod 8 slots [D][w]): lane group lg takes the block of the step's slots
  // 8 lg .. 8 lg + 7, head dimension ln + 16 db.  A lane group past the
  // ring's end loads nothing (its values are masked anyway).
  auto load_v = [&](const Ctx& c, int st, bool live, u32x4 (&v)[DB][VCH]) {
    __amdgpu_buffer_rsrc_t rs = c.vrs;
    const int s0 = st * kStep + 8 * lg;
    const int w = min(8, c.vlim - s0);  // differs between lane groups only in a ring's last step
    uint32_t base = live && w > 0 ? uint32_t(s0 * D + ln * w) * E : kOutOfRange;
    if (PG == 2 && c.per_step) {  // w = 8: the step is four whole V blocks
      rs = make_rsrc(static_cast<const T*>(p.cache_v) + step_base(c, st), uint32_t(kStep) * D * E);
      base = live ? uint32_t(8 * lg * D + ln * 8) * E : kOutOfRange;
    }
    if constexpr (RT && sizeof(T) == 2) {
      // A BF16 ring of odd width ends with a narrow block of odd width, whose
      // runs start 2 bytes into a dword for every other head dimension, and
      // a 16-byte buffer load ignores the low two address bits.  So every V
      // load of this variant is taken from the dword boundary below and
      // moved down by (off & 2) bytes (no move for aligned runs); slots past
      // w hold other runs' values and are masked below.  The move is done on
      // every load, without a branch: the same code under a branch taken
      // only for the ring's last step made the kernel compute wrong values
      // in steps that never took it (measured; the cause was not found).
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint32_t off = w > 0 ? base + uint32_t(16 * db * w) * E : kOutOfRange;
        const u32x4 x = bload16_stream(rs, off & ~3u);
        const uint32_t s = (off & 2u) * 8u;
        v[db][0] = u32x4{__builtin_amdgcn_alignbit(x[1], x[0], s), __builtin_amdgcn_alignbit(x[2], x[1], s),
                         __builtin_amdgcn_alignbit(x[3], x[2], s), __builtin_amdgcn_alignbit(0u, x[3], s)};
      }
      return;
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int cch = 0; cch < VCH; ++cch) v[db][cch] = bload16_stream(rs, base + (16 * db * w + cch * VEC) * E);
  };

  Ctx cur;
  int st = wave;
  bool have = it.n_stream > 0;
  if (have) {
    make_ctx(it.r0, cur);
    have = advance(cur, st);
  } else {  // no streamed run: resources of no bytes (every load returns zeros)
    cur.krs = cur.vrs = make_rsrc(p.cache_k, 0);
    cur.r = it.r0;
    cur.ns = cur.len = cur.c0 = 0;
    cur.vlim = 1 << 30;
    cur.depth = 1;
    cur.ring = cur.per_step = false;
  }
  // The query pieces go out first, then the first step's K and V (loads of a
  // wavefront with no step address nothing: past a resource's end they
  // return zeros without touching memory), then the query chunk is staged
  // through LDS while K and V are in flight.
  load_q_pieces();
  load_k(cur, st, have, kf);
  load_v(cur, st, have, vf);
  stage_q();
  setup_columns();
  if (have) {
    run_hi(tab.piece[cur.r], cur.hi);
    for (;;) {
      floatx4 sacc[2][NB];
      qk<T, D, NB>(kf, qf, sacc);
      Ctx nxt = cur;
      int sn = st + kWaves;
      const bool more = advance(nxt, sn);
      if (more && nxt.r != cur.r) run_hi(tab.piece[nxt.r], nxt.hi);
      load_k(nxt, sn, more, kf);
      int lim[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) lim[nb] = cur.hi[nb] - st * kStep;
      typename O::P pf[NB];
      if constexpr (INF) {
        // a ring whose oldest slots now lie before the window (a parent block
        // in flight) does not read those slots
        const bool hole = cur.ring && sr.hole > 0;
        sm.update(sacc, lim, sl2, pf, hole, cur.c0 + st * kStep, sr.ring_base, sr.hole, p.We);
      } else {
        sm.update(sacc, lim, sl2, pf);
      }
      // a step reaching past the run's end: zero the V values of the missing
      // positions (they may hold anything, even NaN)
      if ((st + 1) * kStep > cur.len) {
        const int nval = cur.len - (st * kStep + 8 * lg);
#pragma unroll
        for (int db = 0; db < DB; ++db) O::zero_tail(vf[db], nval);
      }
      sm.pv(vf, pf);
      load_v(nxt, sn, more, vf);
      if (!more) break;
      cur = nxt;
      st = sn;
    }
  }

  // ---- draft-row runs (kv_new, row-major): the group's own rows or the
  // in-flight parent's.  K rows are loaded in MFMA order directly; V rows are
  // staged in this wavefront's LDS slice with 16-byte loads and read back
  // transposed.
  if (r_draft < r_end) {
    const int Hd = p.H * D;
    T* stage = reinterpret_cast<T*>(lds_raw) + size_t(wave) * kStep * D;  // [32 rows][D]
    constexpr int CPR = D / VEC;  // 16-byte pieces per row
    for (int r = r_draft; r < r_end; ++r) {
      const Piece pc = tab.piece[r];
      const int ns = ceil_div(pc.len, kStep);
      // a run's first step goes to the last wavefront: the streamed runs
      // give their steps beyond a multiple of 4 to the first ones.  The start
      // is the same for every draft run, so a group's result does not depend
      // on the other groups of its launch.
      int st = (wave + 1) & (kWaves - 1);
      if (st < ns) {
        int hi[NB];
        run_hi(pc, hi);
        // the run's first row: the group's own rows, or the in-flight
        // parent's (the rows before its window first, then the window's)
        const size_t row0 = (!INF || pc.kind == kSegDraft
                                 ? size_t(p.grp[pc.gidx].row_start)
                                 : size_t(sr.parent_row0) + (pc.kind == kSegParentWin ? sr.nd : 0)) +
                            size_t(pc.c0);
        const T* kb = static_cast<const T*>(p.kv_new) + (size_t(pc.depth - 1) * p.n_rows + row0) * Hd + size_t(h) * D;
        const T* vb = static_cast<const T*>(p.kv_new) + (size_t(p.R + pc.depth - 1) * p.n_rows + row0) * Hd + size_t(h) * D;
        const int len = pc.len;
        for (; st < ns; st += kWaves) {
          const int base = st * kStep;
#pragma unroll
          for (int mb = 0; mb < 2; ++mb) {
            const int pos = base + 8 * (ln >> 2) + 4 * mb + (ln & 3);
            const bool ok = pos < len;
            const T* rp = kb + size_t(ok ? pos : 0) * Hd + lg * VEC;
#pragma unroll
            for (int cch = 0; cch < KC; ++cch) {
              const u32x4 v = ld16(rp + cch * 4 * VEC);
              kf[mb][cch] = ok ? v : u32x4{0u, 0u, 0u, 0u};
            }
          }
          // stage V rows [base, base + 32) of this head: piece i = (row, 16 B)
#pragma unroll
          for (int i = lane; i < kStep * CPR; i += 64) {
            const int rr = i / CPR;
            const int cch = i - rr * CPR;
            const bool ok = base + rr < len;
            const u32x4 v = ld16(vb + size_t(ok ? base + rr : 0) * Hd + cch * VEC);
            *reinterpret_cast<u32x4*>(stage + rr * D + cch * VEC) = ok ? v : u32x4{0u, 0u, 0u, 0u};
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
    }
  }

  using PL = PartLayout<T, D, CQ>;
  char* const part = reinterpret_cast<char*>(p.ws) + size_t(it.part) * PL::kBytes;

  // ---- merge the four wavefronts through LDS ------------------------------
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
  const bool col_ok = cc * CQ + col < sr.nq;
  float M = -INFINITY, L = 0.f;
  float o[DPT];
  if (col_ok) {
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, lds_m[w][col]);
    float f[kWaves];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = lds_m[w][col];
      f[w] = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
      L += f[w] * lds_l[w][col];
    }
#pragma unroll
    for (int d = 0; d < DPT; d += 4) {
      floatx4 a = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < kWaves; ++w) a += f[w] * *reinterpret_cast<const floatx4*>(&lds_o[w][col][d0 + d]);
#pragma unroll
      for (int e = 0; e < 4; ++e) o[d + e] = a[e];
    }
  }
  // the (sequence, KV head, column chunk) unit this item belongs to
  const int unit_local = (h - sr.h0) * sr.n_cc + cc;
  const int n_split = sr.n_split;
  // outputs of a column from its merged (M, L, O) (log2 domain)
  auto write_out = [&](float Mx, float Lx, const float (&ox)[DPT], bool poison) {
    int row = 0, hh = 0;
    const int gi = column_group(p, sr, cc * CQ + col, row, hh);
    if (gi < 0) return;
    const GroupRec& g = p.grp[gi];
    const size_t orow = size_t(g.row_start + row) * p.Hq + size_t(h) * p.G + hh;
    float res[DPT];
#pragma unroll
    for (int d = 0; d < DPT; ++d) res[d] = poison ? __builtin_nanf("") : ox[d] / Lx;
    if (p.out_f32)
      Op<float>::store(static_cast<float*>(p.out) + orow * D + d0, res, DPT);
    else
      O::store(static_cast<T*>(p.out) + orow * D + d0, res, DPT);
    if (p.lse != nullptr && d0 == 0)
      p.lse[orow] = poison ? __builtin_nanf("") : (Mx + log2f(Lx)) * 0.69314718055994530942f;
  };
  if (n_split == 1) {
    // the unit is this one item: its outputs, no partial
    if (col_ok) write_out(M, L, o, false);
    if (h == 0 && cc == 0) write_plane_sel(p, sr, threadIdx.x, kThreads);
    return;
  }
  {
    // the partial (see PartLayout): O / L, and for 16-bit caches the
    // column's scale from the largest |O / L| over its TPC consecutive lanes
    const float il = (col_ok && L > 0.f) ? 1.0f / L : 0.f;
    float on[DPT];
    float amax = 0.f;
#pragma unroll
    for (int d = 0; d < DPT; ++d) {
      on[d] = col_ok ? o[d] * il : 0.f;
      amax = fmaxf(amax, fabsf(on[d]));
    }
    float isc = 1.f, sc = 1.f;
    if constexpr (PL::kHalf) {
#pragma unroll
      for (int s = TPC / 2; s > 0; s >>= 1) amax = fmaxf(amax, __shfl_xor(amax, s));
      int ex = 0;
      frexpf(amax, &ex);  // amax < 2^ex
      const int k = ex > 15 ? ex - 15 : 0;
      sc = ldexpf(1.f, k);
      isc = ldexpf(1.f, -k);
    }
    if (col_ok) {
#pragma unroll
      for (int d = 0; d < DPT; d += 4) {
        if constexpr (PL::kHalf)
          *reinterpret_cast<half4*>(part + (size_t(col) * D + d0 + d) * 2) =
              half4{_Float16(on[d] * isc), _Float16(on[d + 1] * isc), _Float16(on[d + 2] * isc), _Float16(on[d + 3] * isc)};
        else
          *reinterpret_cast<floatx4*>(part + (size_t(col) * D + d0 + d) * 4) = floatx4{on[d], on[d + 1], on[d + 2], on[d + 3]};
      }
      if (d0 == 0) {
        reinterpret_cast<float*>(part + PL::kM)[col] = M;
        reinterpret_cast<float*>(part + PL::kL)[col] = L;
        if constexpr (PL::kHalf) reinterpret_cast<float*>(part + PL::kS)[col] = sc;
      }
    }
  }
  if (!p.fused) return;  // verify_merge_kernel merges the units

  // ---- fused merge: the unit's last item merges it ------------------------
  // Every item of a unit runs on one XCD (the planner places them on grid
  // positions equal mod 8), whose L2 all its compute units share.  Each item
  // waits until its partial stores are acknowledged by that L2, then counts
  // itself in the unit's arrival word: one byte per XCD, so the last arrival
  // also sees whether every item ran on its own XCD.  The last one resets
  // the word for the next call and reads the partials back past its L1; if
  // the items were not all on one XCD its L2 cannot be trusted, and it writes
  // NaN rather than a result.
  __builtin_amdgcn_s_waitcnt(0);  // this wavefront's stores have reached the L2
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  int* const lds_flag = reinterpret_cast<int*>(lds_raw);
  if (threadIdx.x == 0) {
    const uint32_t xcc = __builtin_amdgcn_s_getreg((3 << 11) | 20) & (kXcds - 1);  // HW_REG_XCC_ID
    unsigned long long* const word = p.arrive + (sr.unit0 + unit_local);
    const unsigned long long add = 1ull << (8 * xcc);
    const unsigned long long now =
        __hip_atomic_fetch_add(word, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + add;
    unsigned total = 0;
#pragma unroll
    for (int x = 0; x < kXcds; ++x) total += unsigned(now >> (8 * x)) & 0xFFu;
    int flag = 0;
    if (total == unsigned(n_split)) {
      flag = 1;
      if (now != (static_cast<unsigned long long>(n_split) << (8 * xcc))) flag |= 2;  // items on several XCDs
      __hip_atomic_store(word, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    *lds_flag = flag;
  }
  __syncthreads();
  const int flag = *lds_flag;
  if (!(flag & 1)) return;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  if (col_ok) {
    // The unit's partials in split order, read past the L1 (sc0).  The loads
    // of a batch of splits all go out before any is used (a read past the
    // resource, for splits beyond the unit's, returns 0 and is not used):
    // first every split's maximum, 16 at a time, then the weighted sums, 4
    // splits at a time.  The arithmetic is the merge kernel's, in split order.
    const char* const p0 = reinterpret_cast<const char*>(p.ws) + size_t(sr.part0 + unit_local * n_split) * PL::kBytes;
    const __amdgpu_buffer_rsrc_t prs = make_rsrc(p0, uint32_t(n_split) * PL::kBytes);
    // one float of split s at byte offset off within its partial
    auto ld1 = [&](int s, uint32_t off) -> float {
      return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                           prs, s < n_split ? uint32_t(s) * PL::kBytes + off : 0x80000000u, 0, 1));
    };
    constexpr int U = 4;  // splits whose loads go out together
    float Mx = -INFINITY;
    float Lx = 0.f;
    float ox[DPT];
#pragma unroll
    for (int d = 0; d < DPT; ++d) ox[d] = 0.f;
    float ms[U], ls[U], ss[U];
    floatx4 ov[U][DPT / 4];
    auto load_splits = [&](int s0) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int s = s0 + u;
        ms[u] = ld1(s, PL::kM + 4 * col);
        ls[u] = ld1(s, PL::kL + 4 * col);
        ss[u] = PL::kHalf ? ld1(s, PL::kS + 4 * col) : 1.f;
        const uint32_t base = s < n_split ? uint32_t(s) * PL::kBytes : 0x80000000u;
#pragma unroll
        for (int d = 0; d < DPT; d += 4) {
          if constexpr (PL::kHalf) {
            const half4 hv = __builtin_bit_cast(
                half4, __builtin_amdgcn_raw_buffer_load_b64(prs, base + (uint32_t(col) * D + d0 + d) * 2, 0, 1));
            ov[u][d / 4] = floatx4{float(hv[0]), float(hv[1]), float(hv[2]), float(hv[3])};
          } else {
            ov[u][d / 4] = __builtin_bit_cast(
                floatx4, __builtin_amdgcn_raw_buffer_load_b128(prs, base + (uint32_t(col) * D + d0 + d) * 4, 0, 1));
          }
        }
      }
    };
    auto add_splits = [&](int s0) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (s0 + u >= n_split) break;
        const float fs = (ms[u] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ms[u] - Mx);
        Lx += fs * ls[u];
        const float fo = fs * ls[u] * ss[u];  // O / L stored, scaled
#pragma unroll
        for (int d = 0; d < DPT; d += 4)
#pragma unroll
          for (int e = 0; e < 4; ++e) ox[d + e] += fo * ov[u][d / 4][e];
      }
    };
    if (n_split <= U) {
      // one round trip: every split's (m, l, O), then the maximum, then the sums
      load_splits(0);
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (u < n_split) Mx = fmaxf(Mx, ms[u]);
      add_splits(0);
    } else {
      for (int s0 = 0; s0 < n_split; s0 += 16) {
        float mm[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) mm[u] = ld1(s0 + u, PL::kM + 4 * col);
#pragma unroll
        for (int u = 0; u < 16; ++u)
          if (s0 + u < n_split) Mx = fmaxf(Mx, mm[u]);
      }
      for (int s0 = 0; s0 < n_split; s0 += U) {
        load_splits(s0);
        add_splits(s0);
      }
    }
    write_out(Mx, Lx, ox, (flag & 2) != 0);
  }
  if (h == 0 && cc == 0) write_plane_sel(p, sr, threadIdx.x, kThreads);
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
  if (un.n_split == 1) return;  // the unit's one item wrote its outputs
  const int cc = un.cc;
  const int h = un.h;
  using PL = PartLayout<T, D, CQ>;
  typedef _Float16 HalfV __attribute__((ext_vector_type(DPT)));
  const char* const part_base = reinterpret_cast<const char*>(p.ws) + size_t(un.part) * PL::kBytes;
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
    // Split s's (m, l, scale, O / L slice), see PartLayout.
    auto load = [&](int s, bool ok, float& m, float& l, float& sc, VecT& ov) {
      const char* part = part_base + size_t(ok ? s : 0) * PL::kBytes;
      m = ok ? __builtin_nontemporal_load(reinterpret_cast<const float*>(part + PL::kM) + col) : -INFINITY;
      l = __builtin_nontemporal_load(reinterpret_cast<const float*>(part + PL::kL) + col);
      if constexpr (PL::kHalf) {
        sc = __builtin_nontemporal_load(reinterpret_cast<const float*>(part + PL::kS) + col);
        const HalfV hv = __builtin_nontemporal_load(reinterpret_cast<const HalfV*>(part + (size_t(col) * D + d0) * 2));
#pragma unroll
        for (int e = 0; e < DPT; ++e) ov[e] = float(hv[e]);
      } else {
        sc = 1.f;
        ov = __builtin_nontemporal_load(reinterpret_cast<const VecT*>(part + (size_t(col) * D + d0) * 4));
      }
    };
    constexpr int kFast = DPT <= 4 ? 16 : 8;
    float M = -INFINITY;
    float L = 0.f;
    float o[DPT];
#pragma unroll
    for (int d = 0; d < DPT; ++d) o[d] = 0.f;
    if (ns <= kFast) {
      float ms[kFast], ls[kFast], ss[kFast];
      VecT ov[kFast];
#pragma unroll
      for (int u = 0; u < kFast; ++u) load(u, u < ns, ms[u], ls[u], ss[u], ov[u]);
#pragma unroll
      for (int u = 0; u < kFast; ++u) M = fmaxf(M, ms[u]);
#pragma unroll
      for (int u = 0; u < kFast; ++u) {
        const float fs = (ms[u] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ms[u] - M);
        L += fs * ls[u];
        const float fo = fs * ls[u] * ss[u];
#pragma unroll
        for (int e = 0; e < DPT; ++e) o[e] += fo * ov[u][e];
      }
    } else {
      constexpr int U = DPT <= 4 ? 8 : 4;  // splits whose loads are issued together
      for (int sp = 0; sp < ns; sp += U) {
        float mm[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
          mm[u] = (sp + u < ns) ? reinterpret_cast<const float*>(part_base + size_t(sp + u) * PL::kBytes + PL::kM)[col]
                                : -INFINITY;
#pragma unroll
        for (int u = 0; u < U; ++u) M = fmaxf(M, mm[u]);
      }
      for (int sp = 0; sp < ns; sp += U) {
        float ms[U], ls[U], ss[U];
        VecT ov[U];
#pragma unroll
        for (int u = 0; u < U; ++u) load(sp + u, sp + u < ns, ms[u], ls[u], ss[u], ov[u]);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const float fs = (ms[u] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ms[u] - M);
          L += fs * ls[u];
          const float fo = fs * ls[u] * ss[u];
#pragma unroll
          for (int e = 0; e < DPT; ++e) o[e] += fo * ov[u][e];
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
  if (h == 0 && cc == 0 && slice == 0) write_plane_sel(p, sr, threadIdx.x, kMergeThreads);
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------
// The verify kernel for a launch's in-flight and paging modes and load
// policy bits.  Only BF16 instantiates policies other than 0.
template <typename T, int D, int NB, int POL>
static const void* pick_verify(bool inf, int page_mode) {
  if constexpr (POL != 0 && sizeof(T) != 2) {
    return nullptr;
  } else {
    static const void* const k[2][3] = {
        {reinterpret_cast<const void*>(&verify_attn_kernel<T, D, NB, false, 0, POL>),
         reinterpret_cast<const void*>(&verify_attn_kernel<T, D, NB, false, 1, POL>),
         reinterpret_cast<const void*>(&verify_attn_kernel<T, D, NB, false, 2, POL>)},
        {reinterpret_cast<const void*>(&verify_attn_kernel<T, D, NB, true, 0, POL>),
         reinterpret_cast<const void*>(&verify_attn_kernel<T, D, NB, true, 1, POL>),
         reinterpret_cast<const void*>(&verify_attn_kernel<T, D, NB, true, 2, POL>)}};
    return k[inf ? 1 : 0][page_mode];
  }
}

template <typename T, int D, int NB>
static hipError_t launch_verify_t(const VerifyParams& p, const ItemTable& t, const UnitTable& u,
                                  hipStream_t stream) {
  if (p.n_wg <= 0) return hipSuccess;
  const int grid = p.n_blocks;
  void* args[] = {const_cast<VerifyParams*>(&p), const_cast<ItemTable*>(&t)};
  int pol = 0;
  if constexpr (sizeof(T) == 2) {
    // BF16 rings of odd width: their last V block has runs that start 2
    // bytes into a dword
    if (p.layout == 2 && p.We % 2 != 0) pol |= kPolOddRing;
    if (p.k_stream) pol |= kPolKStream;
  }
  const bool inf = p.inflight != 0;
  const void* kern = pol == 0                 ? pick_verify<T, D, NB, 0>(inf, p.page_mode)
                     : pol == kPolOddRing     ? pick_verify<T, D, NB, kPolOddRing>(inf, p.page_mode)
                     : pol == kPolKStream     ? pick_verify<T, D, NB, kPolKStream>(inf, p.page_mode)
                                              : pick_verify<T, D, NB, kPolOddRing | kPolKStream>(inf, p.page_mode);
  hipError_t e = hipLaunchKernel(kern, dim3(grid), dim3(kThreads), args, 0, stream);
  if (e != hipSuccess || p.fused) return e;
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
