// api.hip -- host side of the C ABI declared in include/ripe.h: argument
// validation, the memory model, the split-K work plan and kernel launches.
//
// Every check runs before the first HIP call, so an invalid call launches
// nothing and modifies nothing.  The plan of a call is packed into the kernel
// arguments (no host-to-device copies); calls with more than 64 sequences or
// 128 groups are cut into several launches that reuse the workspace in
// stream order.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <unordered_set>
#include <vector>

#include "accept.h"
#include "plan.h"
#include "ripe.h"
#include "side_stats.h"

namespace ripe {
hipError_t launch_verify(const VerifyParams& p, const ItemTable& t, const UnitTable& u, int dtype, int D, int NB,
                         hipStream_t stream);
hipError_t launch_commit(const CommitParams& p, int dtype, int D, hipStream_t stream);
int verify_blocks_per_cu(int dtype, int D, int NB);
}  // namespace ripe

namespace {

using namespace ripe;

constexpr int64_t kMaxBytes = int64_t(1) << 50;   // sanity bound on any buffer size
constexpr int64_t kMaxCommitTasks = int64_t(1) << 28;  // commit wavefront tasks per launch
constexpr int kMaxCQ = 32;                        // query columns per verify work-group
constexpr int kMaxSplit = 8192;                   // longest piece (positions)

int elem_bytes(int dtype) { return dtype == RIPE_F32 ? 4 : 2; }

// A failed launch is reported as RIPE_EHIP; with RIPE_DEBUG set in the
// environment the HIP error string is also printed to stderr.
ripe_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return RIPE_OK;
  if (std::getenv("RIPE_DEBUG") != nullptr)
    std::fprintf(stderr, "[ripe] %s: HIP error %d (%s)\n", what, int(e), hipGetErrorString(e));
  return RIPE_EHIP;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// ---- the static scratch of ripe_verify_attn_noalloc ----------------------
// The largest workspace one verify launch uses: the header (with the merge
// units' arrival words, zero before and after every call; a static array
// starts zeroed) and kMaxItems partials of 32 query columns x (D + 2) floats
// at the largest head dimension, D = 128 (the size of an fp32 cache's
// partial; a 16-bit cache's, in fp16, is smaller).
// Calls are cut into launches of at most kMaxItems items, so every verify
// call fits.  Each GPU the library runs on holds its own copy until the
// process ends.
constexpr size_t kStaticWsBytes = size_t(kWsHeader) + size_t(kMaxItems) * 32 * (128 + 2) * 4;
static_assert(kStaticWsBytes == RIPE_NOALLOC_SCRATCH_BYTES, "ripe.h states the scratch size");
static_assert(kWsHeader == RIPE_WORKSPACE_ZERO_BYTES, "ripe.h states the zeroed workspace header");
}  // namespace

static __device__ __align__(256) unsigned char scratch[kStaticWsBytes];

namespace {

// Device address of `scratch` on the current device, looked up once per
// device with that device current (each device holds its own copy; in host
// code the array's name is not a device address).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

ripe_status_t static_scratch(void** ptr) {
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "ripe_verify_attn_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return RIPE_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t s = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (s != hipSuccess) return hip_status(s, "ripe_verify_attn_noalloc: hipGetSymbolAddress");
    if (p == nullptr) return RIPE_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return RIPE_OK;
}

int ring_width(const ripe_desc_t& d) {
  if (d.layout != RIPE_LAYOUT_RIPE) return 0;
  return d.W < d.t_max ? d.W : d.t_max;
}

// Longest piece.  Fixed by the descriptor alone, so that a sequence's plan
// never depends on the rest of the batch.  1024 positions, the best measured
// trade-off between per-piece start-up and balance, unless full sequences
// would then give more than about 1024 pieces per launch (longer pieces) or
// fewer than about 448 (shorter pieces, down to 256 positions): a launch
// runs best when its pieces nearly fill the 512 resident work-group slots of
// the device in one round, and a second round costs more than it balances
// (measured per workload: shorter and longer pieces were slower for c2, c3,
// c4 and c5 but for small margins at c3 960 and c5 FULL 544).
//
// When the descriptor has at least kWholeUnits (sequence, KV head) pairs, one
// piece per segment already nearly fills that round, so segments are not
// split at all (pieces of up to kMaxSplit positions): every unit is then one
// item that writes its outputs directly, with no partial and no merge, and
// there is no second round of work-groups whose argument reads and first
// loads queue behind the first round's streaming (c5 RIPE at B = 64,
// Hkv = 8: 258.3 -> 242.8 us per call; DEEPEST 258.3 -> 239.3 us).
constexpr int64_t kWholeUnits = 448;
int split_len(const ripe_desc_t& d) {
  if (d.split_len > 0) return d.split_len;
  if (int64_t(d.batch) * d.n_kv_heads >= kWholeUnits) return kMaxSplit;
  const int64_t work = int64_t(d.batch) * d.n_kv_heads * d.t_max;  // positions of full sequences
  int64_t s = std::max<int64_t>(1024, (work + 1023) / 1024);
  s = std::min<int64_t>(s, std::max<int64_t>(256, (work + 447) / 448));
  s = (s + 31) / 32 * 32;
  return int(std::min<int64_t>(std::max<int64_t>(s, 256), kMaxSplit));
}

// Near-equal pieces of at most S positions (multiples of 32 but the last).
inline int piece_len(int len, int S) {
  const int n = (len + S - 1) / S;
  return ((len + n - 1) / n + kStep - 1) / kStep * kStep;
}

// Rings of at most this many slots join their depth's anchor part (plan.h).
constexpr int kFold = 4 * kStep;
// Launches whose units have at most this many items merge them in the verify
// kernel (the last item of each unit); others run the merge kernel.
constexpr int kFuseSplits = 8;

// Positions of the main region (FULL: per plane; otherwise the deep plane):
// t_max per sequence, or the page pool of a paged cache.
long double main_positions(const ripe_desc_t& d) {
  return d.page_len > 0 ? (long double)d.n_pages * d.page_len : (long double)d.batch * d.t_max;
}

// Elements from a region's start to its RIPE ring.
uint64_t ring_offset(const ripe_desc_t& d) {
  return uint64_t(main_positions(d)) * uint64_t(d.n_kv_heads) * uint64_t(d.head_dim);
}

// Elements of one region (K or V) of the cache, or -1 on overflow.
int64_t region_elems(const ripe_desc_t& d) {
  const long double main = main_positions(d) * (d.layout == RIPE_LAYOUT_FULL ? d.R : 1);
  const long double ring =
      d.layout == RIPE_LAYOUT_RIPE ? (long double)d.batch * ring_width(d) * (d.R - 1) : 0.0L;
  const long double n = (main + ring) * d.n_kv_heads * d.head_dim;
  if (n * 2 * elem_bytes(d.dtype) > (long double)kMaxBytes) return -1;
  return int64_t(n);
}

ripe_status_t check_desc(const ripe_desc_t* d) {
  if (d == nullptr) return RIPE_EINVAL;
  if (d->layout < RIPE_LAYOUT_FULL || d->layout > RIPE_LAYOUT_RIPE) return RIPE_EINVAL;
  if (d->dtype != RIPE_F32 && d->dtype != RIPE_BF16) return RIPE_EINVAL;
  if (d->R < 1 || d->W < 0 || d->batch < 1 || d->t_max < 1 || d->n_kv_heads < 1 || d->head_dim < 1 ||
      d->n_q_heads < 1 || d->max_rows < 0 || d->max_groups < 0 || d->split_len < 0 || d->page_len < 0 ||
      d->n_pages < 0)
    return RIPE_EINVAL;
  if (d->page_len > 0 && d->n_pages < 1) return RIPE_EINVAL;
  if (d->n_q_heads % d->n_kv_heads != 0) return RIPE_EINVAL;
  // plan records narrow these to 16 bits (sequence index, KV head) and cut
  // pieces of at most split_len positions, whose byte extents feed 32-bit
  // buffer resources
  if (d->R > 127 || d->batch > 65535 || d->n_kv_heads > 65535 || d->split_len > kMaxSplit)
    return RIPE_EUNSUPPORTED;
  if (d->head_dim != 64 && d->head_dim != 128) return RIPE_EUNSUPPORTED;
  if (d->t_max % 32 != 0 || d->split_len % 32 != 0) return RIPE_EUNSUPPORTED;
  if (d->page_len > 0 && (d->page_len % 32 != 0 || d->t_max % d->page_len != 0)) return RIPE_EUNSUPPORTED;
  if (d->n_q_heads / d->n_kv_heads > 65535) return RIPE_EUNSUPPORTED;
  if (region_elems(*d) < 0) return RIPE_EUNSUPPORTED;
  return RIPE_OK;
}

// Upper bound on split partial slots of any verify call within the
// descriptor's max_rows / max_groups bounds: one partial per piece per
// (sequence, KV head, column chunk).
int64_t workspace_bound(const ripe_desc_t& d) {
  const int64_t S = split_len(d);
  const int64_t G = d.n_q_heads / d.n_kv_heads;
  const int64_t We = ring_width(d);
  const int64_t groups = std::max<int64_t>(d.max_groups, 1);
  const int64_t rows = std::max<int64_t>(d.max_rows, groups);
  const int64_t nseq = std::min<int64_t>(d.batch, groups);
  // (a paged cache with pages of at least S positions also cuts at pages)
  const int64_t tpieces = (int64_t(d.t_max) + S - 1) / S + (d.page_len >= S ? d.t_max / d.page_len : 0);
  int64_t per_seq = (d.layout == RIPE_LAYOUT_FULL ? std::min<int64_t>(groups, d.R) : 1) * tpieces;
  if (d.layout == RIPE_LAYOUT_RIPE) per_seq += std::min<int64_t>(groups, d.R - 1) * ((We + S - 1) / S);
  per_seq += groups + (rows + S - 1) / S;  // draft rows
  per_seq += (1 + std::min<int64_t>(groups, d.R)) * ((rows + S - 1) / S);  // an in-flight parent's rows
  const int64_t col_chunks = (rows * G + 15) / 16 + nseq;
  const long double slots = (long double)d.n_kv_heads * col_chunks * per_seq;
  const long double bytes = slots * kMaxCQ * (d.head_dim + 2) * 4 + kWsHeader;
  if (bytes > (long double)kMaxBytes) return -1;
  return int64_t(bytes);
}

int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

// Buffers of ripe_position_error ahead of the verify workspace: the FULL
// output (fp32) and its LSE unless the caller passes them, and the per-KV-head
// sums and condition numbers.  -1 on overflow.
int64_t poserr_extra(const ripe_desc_t& d, int64_t rows, int64_t groups, bool own_out, bool own_lse) {
  const long double o = own_out ? (long double)rows * d.n_q_heads * d.head_dim * 4 : 0;
  const long double l = own_lse ? (long double)rows * d.n_q_heads * 4 : 0;
  const long double s = (long double)groups * d.n_kv_heads * d.t_max * 4;
  if (o + l + 2 * s + 1024 > (long double)kMaxBytes) return -1;
  return align256(int64_t(o)) + align256(int64_t(l)) + 2 * align256(int64_t(s));
}

struct LaunchPlan {
  VerifyParams p;
  ItemTable t;
  UnitTable u;
  int64_t part_bytes;  // split partials
};

// Per-thread planning buffers, reused across calls (no per-call allocation
// once they have grown to the call sizes in use).
struct WgCost {
  int work;        // 32-position steps streamed by the work-group
  uint16_t entry;  // its index among the sorted items
};

// Compute units of the current device (0 if the runtime cannot say).
int compute_units() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  return n;
}

// One part of a sequence's plan: runs [first, first + n_run) of its run
// list, the first n_stream of them streamed from the cache.
struct PartRec {
  int first, n_stream, n_run, steps;
};

struct VerifyScratch {
  std::vector<std::pair<int, int>> spans;
  std::vector<int> count, fill, order, seg_last;
  std::vector<std::vector<Piece>> part_runs;
  std::vector<Seg> segs;
  std::vector<Piece> pieces;
  std::vector<PartRec> parts;
  std::vector<Item> items;
  std::vector<int> cost, by_size;
  std::vector<WgCost> wgs;
  std::vector<uint16_t> grid;  // grid position -> sorted item (kWgEmpty: none)
  std::vector<int64_t> unit_cost;
  std::vector<int> item_unit, unit_order, unit_xcd;
  std::vector<uint16_t> xcd_items[kXcds];
  std::vector<LaunchPlan> plans;
  int n_plans = 0;
  // The inputs the plans above were built from (pointers aside).  A call
  // with the same inputs, e.g. the same verify step on the next recurrent
  // layer's cache, reuses them.
  bool have_key = false;
  ripe_desc_t key_desc;
  int32_t key_rows = 0;
  float key_scale = 0.f;
  int key_NB = 1;
  std::vector<int32_t> key_seq;
  std::vector<ripe_group_t> key_groups;
  std::vector<int32_t> key_parents;  // empty: no parents
  std::vector<int32_t> key_table;    // paged caches: the block table
};

VerifyScratch& verify_scratch() {
  thread_local VerifyScratch sc;
  return sc;
}

}  // namespace

extern "C" int64_t ripe_layout_bytes(const ripe_desc_t* desc, int32_t kind) {
  const ripe_status_t st = check_desc(desc);
  if (st != RIPE_OK) return st;
  if (kind == RIPE_BYTES_CACHE) return 2 * region_elems(*desc) * elem_bytes(desc->dtype);
  if (kind == RIPE_BYTES_WORKSPACE) {
    const int64_t b = workspace_bound(*desc);
    return b < 0 ? int64_t(RIPE_EUNSUPPORTED) : b;
  }
  if (kind == RIPE_BYTES_POSERR_WORKSPACE) {
    const int64_t groups = std::max<int64_t>(desc->max_groups, 1);
    const int64_t rows = std::max<int64_t>(desc->max_rows, groups);
    const int64_t b = workspace_bound(*desc), x = poserr_extra(*desc, rows, groups, true, true);
    return (b < 0 || x < 0 || b + x > kMaxBytes) ? int64_t(RIPE_EUNSUPPORTED) : b + x;
  }
  return RIPE_EINVAL;
}

// Every verify entry point.  parents: host [n_groups][2] (row_start, n_rows)
// of each group's in-flight parent block, or nullptr for none.  table: the
// block table of a paged cache (nullptr for an unpaged one).  static_ws: use
// the static scratch instead of the caller's workspace (looked up after every
// check has passed, right before the first launch).
static ripe_status_t verify_impl(const ripe_desc_t* desc, const void* cache, const int32_t* table,
                          const int32_t* seq_len,
                          const ripe_group_t* groups, const int32_t* parents, int32_t n_groups, int32_t n_rows,
                          float softmax_scale, const void* q, const void* kv_new, void* out, float* lse,
                          int8_t* plane_sel, void* workspace, size_t workspace_bytes, void* stream,
                          bool out_f32 = false, bool static_ws = false) {
  ripe_status_t st = check_desc(desc);
  if (st != RIPE_OK) return st;
  const ripe_desc_t& d = *desc;
  if ((d.page_len > 0) != (table != nullptr)) return RIPE_EINVAL;
  if (n_groups < 0) return RIPE_EINVAL;
  if (n_groups == 0) return RIPE_OK;
  if (groups == nullptr || seq_len == nullptr || n_rows < 1) return RIPE_EINVAL;
  if (n_groups > 65535) return RIPE_EUNSUPPORTED;
  if (!std::isfinite(softmax_scale)) return RIPE_EINVAL;
  if (cache == nullptr || q == nullptr || kv_new == nullptr || out == nullptr) return RIPE_EINVAL;
  if (!aligned(cache, 16) || !aligned(q, 16) || !aligned(kv_new, 16) || !aligned(out, 16)) return RIPE_EINVAL;
  if ((lse && !aligned(lse, 4)) || (plane_sel && !aligned(plane_sel, 16))) return RIPE_EINVAL;
  if (!static_ws && workspace && !aligned(workspace, 256)) return RIPE_EINVAL;
  for (int b = 0; b < d.batch; ++b)
    if (seq_len[b] < 0 || seq_len[b] > d.t_max) return RIPE_ERANGE;
  const int G = d.n_q_heads / d.n_kv_heads;
  const int D = d.head_dim;
  const size_t E = elem_bytes(d.dtype);
  VerifyScratch& sc = verify_scratch();
  hipStream_t hs = static_cast<hipStream_t>(stream);
  auto set_pointers = [&](VerifyParams& p) {
    p.cache_k = cache;
    p.cache_v = static_cast<const char*>(cache) + size_t(region_elems(d)) * E;
    p.q = q;
    p.kv_new = kv_new;
    p.out = out;
    p.out_f32 = out_f32 ? 1 : 0;
    p.lse = lse;
    p.plane_sel = plane_sel;
    p.ws = reinterpret_cast<float*>(static_cast<char*>(workspace) + kWsHeader);
    p.arrive = reinterpret_cast<unsigned long long*>(static_cast<char*>(workspace) + kWsArrive);
  };
  auto launch_all = [&](int NB) -> ripe_status_t {
    if (static_ws) {
      const ripe_status_t s = static_scratch(&workspace);
      if (s != RIPE_OK) return s;
      workspace_bytes = kStaticWsBytes;
    }
    for (int pi = 0; pi < sc.n_plans; ++pi)
      if (workspace == nullptr || size_t(sc.plans[pi].part_bytes) > workspace_bytes) {
        if (static_ws && std::getenv("RIPE_DEBUG") != nullptr)
          std::fprintf(stderr, "[ripe] ripe_verify_attn_noalloc: a launch needs %lld bytes of scratch, more than %zu\n",
                       (long long)sc.plans[pi].part_bytes, kStaticWsBytes);
        return RIPE_EWORKSPACE;
      }
    for (int pi = 0; pi < sc.n_plans; ++pi) {
      LaunchPlan& lp = sc.plans[pi];
      set_pointers(lp.p);
      const ripe_status_t st2 = hip_status(launch_verify(lp.p, lp.t, lp.u, d.dtype, D, NB, hs), "ripe_verify_attn");
      if (st2 != RIPE_OK) return st2;
    }
    return RIPE_OK;
  };
  // same inputs as the plans in hand (already validated): launch them
  if (sc.have_key && std::memcmp(&sc.key_desc, &d, sizeof(d)) == 0 && sc.key_rows == n_rows &&
      std::memcmp(&sc.key_scale, &softmax_scale, sizeof(float)) == 0 && sc.key_groups.size() == size_t(n_groups) &&
      std::memcmp(sc.key_seq.data(), seq_len, sizeof(int32_t) * size_t(d.batch)) == 0 &&
      std::memcmp(sc.key_groups.data(), groups, sizeof(ripe_group_t) * size_t(n_groups)) == 0 &&
      (parents == nullptr ? sc.key_parents.empty()
                          : sc.key_parents.size() == 2 * size_t(n_groups) &&
                                std::memcmp(sc.key_parents.data(), parents, sizeof(int32_t) * 2 * size_t(n_groups)) == 0) &&
      (table == nullptr ||
       std::memcmp(sc.key_table.data(), table, sizeof(int32_t) * sc.key_table.size()) == 0))
    return launch_all(sc.key_NB);
  sc.have_key = false;
  sc.spans.clear();
  for (int i = 0; i < n_groups; ++i) {
    const ripe_group_t& g = groups[i];
    if (g.n_rows < 1) return RIPE_EINVAL;
    if (g.seq < 0 || g.seq >= d.batch || g.depth < 1 || g.depth > d.R || g.row_start < 0 ||
        int64_t(g.row_start) + g.n_rows > n_rows)
      return RIPE_ERANGE;
    if (g.n_rows > 65535) return RIPE_EUNSUPPORTED;
    sc.spans.emplace_back(g.row_start, g.n_rows);
  }
  std::sort(sc.spans.begin(), sc.spans.end());
  for (size_t i = 1; i < sc.spans.size(); ++i)
    if (sc.spans[i - 1].first + sc.spans[i - 1].second > sc.spans[i].first) return RIPE_EINVAL;
  if (parents != nullptr)
    for (int i = 0; i < n_groups; ++i) {
      const int32_t ps = parents[2 * i], kp = parents[2 * i + 1];
      if (kp < 0) return RIPE_EINVAL;
      if (kp > 0 && (ps < 0 || int64_t(ps) + kp > n_rows)) return RIPE_ERANGE;
      if (kp > 65535) return RIPE_EUNSUPPORTED;
      // the ring slots a parent hides are tracked in 16-bit fields
      if (kp > 0 && ring_width(d) > 65535) return RIPE_EUNSUPPORTED;
    }
  const int nblk = d.page_len > 0 ? d.t_max / d.page_len : 0;  // block-table row length
  if (table != nullptr)
    for (int i = 0; i < n_groups; ++i) {  // the pages holding the prefix of every sequence read
      const int b = groups[i].seq;
      for (int k = 0; k * d.page_len < seq_len[b]; ++k)
        if (table[b * nblk + k] < 0 || table[b * nblk + k] >= d.n_pages) return RIPE_ERANGE;
    }

  // groups of each sequence in the caller's order (counting sort by sequence)
  sc.count.assign(d.batch + 1, 0);
  for (int i = 0; i < n_groups; ++i) ++sc.count[groups[i].seq + 1];
  for (int b = 0; b < d.batch; ++b) sc.count[b + 1] += sc.count[b];  // count[b] = first index of b
  sc.order.resize(n_groups);
  sc.fill.assign(sc.count.begin(), sc.count.end() - 1);
  for (int i = 0; i < n_groups; ++i) sc.order[sc.fill[groups[i].seq]++] = i;
  int NB = 1;
  for (int b = 0; b < d.batch; ++b) {
    const int cnt = sc.count[b + 1] - sc.count[b];
    if (cnt > kMaxGroups) return RIPE_EUNSUPPORTED;
    int64_t nq = 0;
    for (int k = sc.count[b]; k < sc.count[b + 1]; ++k) nq += int64_t(groups[sc.order[k]].n_rows) * G;
    if (nq > 65535) return RIPE_EUNSUPPORTED;
    if (nq > 16) NB = 2;  // query-column chunks of 32 if any sequence needs more than 16
  }
  const int CQ = 16 * NB;

  const int We = ring_width(d);
  const int S = split_len(d);

  // Pack (sequence, KV-head range) pieces into launches of <= kMaxItems
  // items, <= kMaxPieces pieces, <= kMaxSeq sequence records and
  // <= kMaxGroups group records.
  sc.n_plans = 0;
  auto new_plan = [&]() -> LaunchPlan& {
    if (sc.plans.size() <= size_t(sc.n_plans)) sc.plans.emplace_back();
    LaunchPlan& lp = sc.plans[sc.n_plans++];
    VerifyParams& p = lp.p;
    p.ring_off = ring_offset(d);
    p.page_len = d.page_len;
    p.page_mode = d.page_len == 0 ? 0 : d.page_len >= S ? 1 : 2;  // see the piece cuts below
    p.layout = d.layout;
    p.R = d.R;
    p.We = We;
    p.t_max = d.t_max;
    p.H = d.n_kv_heads;
    p.Hq = d.n_q_heads;
    p.G = G;
    p.n_rows = n_rows;
    p.n_seq = 0;
    p.n_wg = 0;
    p.n_units = 0;
    p.n_grp = 0;
    p.n_pieces = 0;
    p.n_refs = 0;
    p.inflight = 0;
    p.k_stream = 0;
    p.scale_log2 = float(double(softmax_scale) * 1.4426950408889634);
    return lp;
  };
  LaunchPlan* cur = nullptr;
  GroupRec grp[kMaxGroups];
  for (int b = 0; b < d.batch; ++b) {
    const int g0 = sc.count[b], gc = sc.count[b + 1] - sc.count[b];
    if (gc == 0) continue;
    int nq = 0;
    bool mixed = false;  // groups at several depths
    for (int k = 0; k < gc; ++k) {
      const ripe_group_t& g = groups[sc.order[g0 + k]];
      grp[k].row_start = g.row_start;
      grp[k].n_rows = uint16_t(g.n_rows);
      grp[k].depth = uint8_t(g.depth);
      grp[k].seq = 0;
      nq += g.n_rows * G;
      mixed = mixed || g.depth != groups[sc.order[g0]].depth;
    }
    const int T = seq_len[b];
    // the sequence's in-flight parent block: the same for all its groups
    int ps = 0, kp = 0;
    if (parents != nullptr) {
      const int i0 = sc.order[g0];
      ps = parents[2 * i0];
      kp = parents[2 * i0 + 1];
      for (int k = 1; k < gc; ++k) {
        const int i = sc.order[g0 + k];
        if (parents[2 * i + 1] != kp || (kp > 0 && parents[2 * i] != ps)) return RIPE_EUNSUPPORTED;
      }
      if (kp == 0) ps = 0;
    }
    const InFlight fl = in_flight(d.layout, We, T, kp);
    // Parts of this sequence: every streamed segment (prefix plane, ring) is
    // cut on its own into near-equal pieces of at most S positions (multiples
    // of 32 but the last), each piece a part of its own.  Short rings (at
    // most kFold slots) and the groups' own draft rows are appended to the
    // anchor part of their depth: the last piece of the first segment that
    // a group at that depth reads (RIPE: the deep plane, else the ring; FULL:
    // the plane at that depth; DEEPEST: the plane).  Neither the cuts nor
    // the anchors depend on the other groups of the sequence, so a group's
    // runs fall in the same parts alone or with siblings (whose extra runs
    // are masked for its columns).  An in-flight parent's rows form parts of
    // their own.  Paged caches: with pages of at least S positions a
    // prefix-plane piece is first cut at page boundaries (every run then lies
    // in one page); with shorter pages a run may span pages and the kernel
    // reads each step from its page.
    const bool cut_at_pages = table != nullptr && d.page_len >= S;
    sc.segs.clear();
    enumerate_segments(d.layout, d.R, We, T, grp, 0, gc, kp, [&](const Seg& sg) {
      sc.segs.push_back(sg);
      return false;
    });
    const int n_seg = int(sc.segs.size());
    auto stream = [](const Seg& sg) { return sg.kind == kSegPlane || sg.kind == kSegRing; };
    // the anchor segment of depth r: -1 if none
    auto anchor_seg = [&](int r) {
      int ring = -1;
      for (int i = 0; i < n_seg; ++i) {
        const Seg& sg = sc.segs[i];
        if (sg.kind == kSegPlane && (d.layout != RIPE_LAYOUT_FULL || sg.depth == r)) return i;
        if (sg.kind == kSegRing && sg.depth == r && ring < 0) ring = i;
      }
      return ring;
    };
    auto folded = [&](int i) {  // a short ring that goes into another segment's anchor part
      const Seg& sg = sc.segs[i];
      return sg.kind == kSegRing && sg.len <= kFold && anchor_seg(sg.depth) != i;
    };
    sc.part_runs.resize(std::max<size_t>(sc.part_runs.size(), size_t(n_seg) * 64 + 1));
    int n_part = 0;
    sc.seg_last.assign(n_seg, -1);
    for (int i = 0; i < n_seg; ++i) {
      const Seg& sg = sc.segs[i];
      if (!stream(sg) || folded(i) || sg.len == 0) continue;
      const bool cut = cut_at_pages && sg.kind == kSegPlane;
      for (int a0 = 0; a0 < sg.len;) {
        const int a1 = cut ? std::min(sg.len, (a0 / d.page_len + 1) * d.page_len) : sg.len;
        const int pl = piece_len(a1 - a0, S);
        for (int c0 = a0; c0 < a1; c0 += pl) {
          if (size_t(n_part) >= sc.part_runs.size()) sc.part_runs.resize(2 * sc.part_runs.size());
          sc.part_runs[n_part].clear();
          sc.part_runs[n_part].push_back(Piece{c0, std::min(pl, a1 - c0), uint8_t(sg.kind), uint8_t(sg.depth), 0, 0});
          sc.seg_last[i] = n_part++;
        }
        a0 = a1;
      }
    }
    // the part a short run of depth r joins: its anchor's last piece, or a new part
    auto home = [&](int r) -> int {
      const int a = anchor_seg(r);
      if (a >= 0 && sc.seg_last[a] >= 0) return sc.seg_last[a];
      if (size_t(n_part) >= sc.part_runs.size()) sc.part_runs.resize(2 * sc.part_runs.size());
      sc.part_runs[n_part].clear();
      return n_part++;
    };
    for (int i = 0; i < n_seg; ++i)
      if (folded(i)) {
        const Seg& sg = sc.segs[i];
        sc.part_runs[home(sg.depth)].push_back(Piece{0, sg.len, uint8_t(sg.kind), uint8_t(sg.depth), 0, 0});
      }
    for (int i = 0; i < n_seg; ++i) {
      const Seg& sg = sc.segs[i];
      if (stream(sg) || sg.len == 0) continue;
      const Piece pc{0, sg.len, uint8_t(sg.kind), uint8_t(sg.depth), uint8_t(sg.gidx < 0 ? 0 : sg.gidx), 0};
      if (sg.kind == kSegDraft) {
        sc.part_runs[home(sg.depth)].push_back(pc);
      } else {  // in-flight parent rows: parts of their own, at most S rows each
        const int pl = piece_len(sg.len, S);
        for (int c0 = 0; c0 < sg.len; c0 += pl) {
          if (size_t(n_part) >= sc.part_runs.size()) sc.part_runs.resize(2 * sc.part_runs.size());
          sc.part_runs[n_part].clear();
          sc.part_runs[n_part++].push_back(Piece{c0, std::min(pl, sg.len - c0), pc.kind, pc.depth, 0, 0});
        }
      }
    }
    // flatten: each part's streamed runs first, then its draft-row runs
    sc.pieces.clear();
    sc.parts.clear();
    for (int k = 0; k < n_part; ++k) {
      PartRec pr{int(sc.pieces.size()), 0, 0, 0};
      for (const Piece& pc : sc.part_runs[k])
        if (pc.kind == kSegPlane || pc.kind == kSegRing) {
          sc.pieces.push_back(pc);
          pr.steps += (pc.len + kStep - 1) / kStep;
        }
      pr.n_stream = int(sc.pieces.size()) - pr.first;
      for (const Piece& pc : sc.part_runs[k])
        if (!(pc.kind == kSegPlane || pc.kind == kSegRing)) sc.pieces.push_back(pc);
      pr.n_run = int(sc.pieces.size()) - pr.first;
      if (pr.n_run > 255 || pr.steps > 65535) return RIPE_EUNSUPPORTED;
      sc.parts.push_back(pr);
    }
    const int n_piece = int(sc.pieces.size());
    // page entries past the first that the sequence's prefix-plane runs
    // need (paged caches)
    int n_refs = 0;
    if (table != nullptr)
      for (const Piece& pc : sc.pieces)
        if (pc.kind == kSegPlane) n_refs += (pc.c0 + pc.len - 1) / d.page_len - pc.c0 / d.page_len;
    if (n_refs > kMaxPageRefs) return RIPE_EUNSUPPORTED;  // one sequence's pages must fit a launch
    const int n_split = n_part;
    const int n_cc = (nq + CQ - 1) / CQ;
    const int64_t per_head = int64_t(n_split) * n_cc;
    if (per_head > kMaxItems || n_piece > kMaxPieces) return RIPE_EUNSUPPORTED;  // one KV head must fit a launch
    int h = 0;
    while (h < d.n_kv_heads) {
      if (cur == nullptr || cur->p.n_seq == kMaxSeq || cur->p.n_grp + gc > kMaxGroups ||
          cur->p.n_wg + per_head > kMaxItems || cur->p.n_pieces + n_piece > kMaxPieces ||
          cur->p.n_refs + n_refs > kMaxPageRefs)
        cur = &new_plan();
      VerifyParams& p = cur->p;
      const int hc = int(std::min<int64_t>((kMaxItems - p.n_wg) / per_head, d.n_kv_heads - h));
      SeqRec& sr = p.seq[p.n_seq];
      sr.T = T;
      sr.b = uint16_t(b);
      sr.nq = uint16_t(nq);
      sr.n_cc = uint16_t(n_cc);
      sr.n_split = int32_t(n_split);
      sr.h0 = uint16_t(h);
      sr.h_cnt = uint16_t(hc);
      sr.g_begin = uint8_t(p.n_grp);
      sr.g_count = uint8_t(gc);
      sr.part0 = p.n_wg;  // one partial per item
      sr.unit0 = p.n_units;
      sr.tw = fl.tw;
      sr.parent_row0 = ps;
      sr.kp = uint16_t(kp);
      sr.nd = uint16_t(fl.nd);
      sr.hole = uint16_t(fl.hole);
      sr.ring_base = uint16_t(fl.ring_base);
      if (kp > 0) p.inflight = 1;
      // a launch verifying several depths of one sequence streams its K rows
      // (the one-call-per-step pattern; see the verify kernel's load policy)
      if (mixed) p.k_stream = 1;
      for (int k = 0; k < gc; ++k) {
        p.grp[p.n_grp] = grp[k];
        p.grp[p.n_grp].seq = uint8_t(p.n_seq);
        p.gorig[p.n_grp] = uint16_t(sc.order[g0 + k]);
        ++p.n_grp;
      }
      for (int k = 0; k < 2; ++k) sr.g01[k] = p.grp[sr.g_begin + std::min(k, gc - 1)];
      const int pbase = p.n_pieces;
      for (int k = 0; k < n_piece; ++k) {
        Piece pc = sc.pieces[k];
        pc.s = uint8_t(p.n_seq);
        if (pc.kind == kSegDraft) pc.gidx = uint8_t(sr.g_begin + pc.gidx);
        cur->t.pref[p.n_pieces] = uint16_t(p.n_refs);
        cur->t.pages[p.n_pieces] = 0;
        if (table != nullptr && pc.kind == kSegPlane) {
          const int blk0 = pc.c0 / d.page_len;
          cur->t.pages[p.n_pieces] = table[b * nblk + blk0];
          for (int blk = blk0 + 1; blk * d.page_len < pc.c0 + pc.len; ++blk)
            cur->t.pages[kMaxPieces + p.n_refs++] = table[b * nblk + blk];
        }
        cur->t.piece[p.n_pieces++] = pc;
      }
      // items of unit (h, cc): one per part; partial slot = part0 + unit *
      // n_split + part
      for (int hh = 0; hh < hc; ++hh)
        for (int cc = 0; cc < n_cc; ++cc) {
          const int unit = hh * n_cc + cc;
          for (int k = 0; k < n_split; ++k) {
            const PartRec& pr = sc.parts[k];
            Item& it = cur->t.item[p.n_wg++];
            it.r0 = uint16_t(pbase + pr.first);
            it.n_stream = uint8_t(pr.n_stream);
            it.n_run = uint8_t(pr.n_run);
            it.part = uint16_t(sr.part0 + unit * n_split + k);
            it.h = uint16_t(h + hh);
            it.cc = uint16_t(cc);
            it.s = uint16_t(p.n_seq);
          }
          Unit& un = cur->u.unit[p.n_units + unit];
          un.part = sr.part0 + unit * n_split;
          un.n_split = uint16_t(n_split);
          un.pad = 0;
          un.s = uint16_t(p.n_seq);
          un.h = uint16_t(h + hh);
          un.cc = uint16_t(cc);
          un.hl = uint16_t(hh);
        }
      p.n_units += hc * n_cc;
      ++p.n_seq;
      h += hc;
    }
  }
  // Items run longest first (by 32-position steps; a stable counting sort),
  // one work-group each.
  // The hardware dispatches work-groups in grid order: the first round puts
  // work-group j on compute unit j mod n_cu, and with two resident per unit,
  // j and j + n_cu share one.  A unit's finishing time follows the total
  // work of its pair, so when every work-group fits in that first round the
  // grid pairs the largest with the smallest (the largest ones alone when
  // fewer than 2 n_cu); beyond that, longest-first order lets the
  // work-groups that free up last take the shortest items.  Placement only
  // moves work-groups between compute units: every item writes its own
  // partial and the merge order is fixed, so results do not depend on it.
  const int n_cu = compute_units();
  const int per_cu = verify_blocks_per_cu(d.dtype, D, NB);
  for (int pi = 0; pi < sc.n_plans; ++pi) {
    LaunchPlan& lp = sc.plans[pi];
    lp.part_bytes = kWsHeader + int64_t(lp.p.n_wg) * CQ * (D + 2) * 4;
    Item* items = lp.t.item;
    const int n = lp.p.n_wg;
    // an item's cost: the 32-position steps of its streamed and draft-row runs
    auto cost_of = [&](const Item& it) {
      int c = 0;
      for (int r = it.r0; r < it.r0 + it.n_run; ++r) c += (lp.t.piece[r].len + kStep - 1) / kStep;
      return c;
    };
    int max_steps = 0;
    sc.cost.resize(n);
    for (int i = 0; i < n; ++i) {
      sc.cost[i] = cost_of(items[i]);
      max_steps = std::max(max_steps, sc.cost[i]);
    }
    sc.by_size.assign(max_steps + 2, 0);  // by_size[max_steps - c + 1]: items with more steps than c
    for (int i = 0; i < n; ++i) ++sc.by_size[max_steps - sc.cost[i] + 1];
    for (int c = 1; c <= max_steps + 1; ++c) sc.by_size[c] += sc.by_size[c - 1];
    sc.items.resize(n);
    for (int i = 0; i < n; ++i) sc.items[sc.by_size[max_steps - sc.cost[i]]++] = items[i];
    std::copy(sc.items.begin(), sc.items.end(), items);
    sc.wgs.resize(n);
    for (int i = 0; i < n; ++i) sc.wgs[i] = WgCost{cost_of(items[i]), uint16_t(i)};
    // Fused merge: the items of a unit go on grid positions equal mod 8 (one
    // XCD); units are spread over the XCDs by their total work, largest
    // first, and each XCD's items are placed on its compute units as below.
    // One work-group reads the partials of a unit at the rate of one
    // work-group, so launches with units of more than kFuseSplits items
    // (whose merge is better spread over several work-groups), or a grid past
    // the work-group table, keep the separate merge kernel.
    const int cus_x = n_cu / kXcds;
    bool fused = n_cu > 0 && n_cu % kXcds == 0 && per_cu == 2;
    for (int s = 0; s < lp.p.n_seq && fused; ++s) fused = lp.p.seq[s].n_split <= kFuseSplits;
    sc.grid.assign(size_t(kMaxItems) + 512, kWgEmpty);
    uint16_t* wg = sc.grid.data();
    if (fused) {
      const int nu = lp.p.n_units;
      sc.unit_cost.assign(nu, 0);
      sc.item_unit.resize(n);
      for (int i = 0; i < n; ++i) {
        const SeqRec& sr = lp.p.seq[lp.t.piece[items[i].r0].s];
        const int u = sr.unit0 + (items[i].h - sr.h0) * sr.n_cc + items[i].cc;
        sc.item_unit[i] = u;
        sc.unit_cost[u] += sc.wgs[i].work;
      }
      sc.unit_order.resize(nu);
      for (int u = 0; u < nu; ++u) sc.unit_order[u] = u;
      std::stable_sort(sc.unit_order.begin(), sc.unit_order.end(),
                       [&](int a, int b) { return sc.unit_cost[a] > sc.unit_cost[b]; });
      sc.unit_xcd.assign(nu, 0);
      int64_t load[kXcds] = {};
      for (int u : sc.unit_order) {
        int best = 0;
        for (int x = 1; x < kXcds; ++x)
          if (load[x] < load[best]) best = x;
        sc.unit_xcd[u] = best;
        load[best] += sc.unit_cost[u];
      }
      for (int x = 0; x < kXcds; ++x) sc.xcd_items[x].clear();
      for (int i = 0; i < n; ++i) sc.xcd_items[sc.unit_xcd[sc.item_unit[i]]].push_back(sc.wgs[i].entry);  // decreasing work
      int rows = 0;
      for (int x = 0; x < kXcds; ++x) rows = std::max(rows, int(sc.xcd_items[x].size()));
      if (int64_t(rows) * kXcds > int64_t(kMaxItems) + 512) fused = false;
      if (fused) {
        for (int j = 0; j < rows * kXcds; ++j) wg[j] = kWgEmpty;
        for (int x = 0; x < kXcds; ++x) {
          const std::vector<uint16_t>& v = sc.xcd_items[x];
          const int nx = int(v.size());
          auto put = [&](int k, uint16_t e) { wg[x + kXcds * k] = e; };
          if (nx > cus_x && nx <= 2 * cus_x) {
            const int P = nx - cus_x, S = cus_x - P;
            for (int k = 0; k < P; ++k) {
              put(k, v[S + k]);
              put(cus_x + k, v[nx - 1 - k]);
            }
            for (int k = 0; k < S; ++k) put(P + k, v[k]);
          } else {
            for (int k = 0; k < nx; ++k) put(k, v[k]);
          }
        }
        lp.p.n_blocks = rows * kXcds;
      }
    }
    lp.p.fused = fused ? 1 : 0;
    if (!fused) {
      const int N = n;
      if (per_cu == 2 && n_cu > 0 && N > n_cu && N <= 2 * n_cu) {
        const int P = N - n_cu;  // compute units running two work-groups
        const int S = n_cu - P;  // ... and one
        for (int j = 0; j < P; ++j) {
          wg[j] = sc.wgs[S + j].entry;
          wg[n_cu + j] = sc.wgs[N - 1 - j].entry;
        }
        for (int j = 0; j < S; ++j) wg[P + j] = sc.wgs[j].entry;
      } else {
        for (int j = 0; j < N; ++j) wg[j] = sc.wgs[j].entry;
      }
      lp.p.n_blocks = N;
    }
    // the items in grid order, so that a work-group's first argument read
    // is its own item (sc.items holds them sorted, as wg indexes them)
    for (int j = 0; j < lp.p.n_blocks; ++j) items[j] = wg[j] == kWgEmpty ? Item{} : sc.items[wg[j]];
  }
  sc.key_desc = d;
  sc.key_rows = n_rows;
  sc.key_scale = softmax_scale;
  sc.key_NB = NB;
  sc.key_seq.assign(seq_len, seq_len + d.batch);
  sc.key_groups.assign(groups, groups + n_groups);
  if (parents != nullptr)
    sc.key_parents.assign(parents, parents + 2 * size_t(n_groups));
  else
    sc.key_parents.clear();
  if (table != nullptr)
    sc.key_table.assign(table, table + size_t(d.batch) * nblk);
  else
    sc.key_table.clear();
  sc.have_key = true;
  return launch_all(NB);
}

extern "C" ripe_status_t ripe_verify_attn(const ripe_desc_t* desc, const void* cache, const int32_t* seq_len,
                                          const ripe_group_t* groups, int32_t n_groups, int32_t n_rows,
                                          float softmax_scale, const void* q, const void* kv_new, void* out,
                                          float* lse, int8_t* plane_sel, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  return verify_impl(desc, cache, nullptr, seq_len, groups, nullptr, n_groups, n_rows, softmax_scale, q, kv_new,
                     out, lse, plane_sel, workspace, workspace_bytes, stream);
}

extern "C" ripe_status_t ripe_verify_attn_noalloc(const ripe_desc_t* desc, const void* cache,
                                                  const int32_t* seq_len, const ripe_group_t* groups,
                                                  int32_t n_groups, int32_t n_rows, float softmax_scale,
                                                  const void* q, const void* kv_new, void* out, float* lse,
                                                  int8_t* plane_sel, void* stream) {
  return verify_impl(desc, cache, nullptr, seq_len, groups, nullptr, n_groups, n_rows, softmax_scale, q, kv_new,
                     out, lse, plane_sel, nullptr, 0, stream, false, true);
}

extern "C" ripe_status_t ripe_verify_attn_inflight(const ripe_desc_t* desc, const void* cache,
                                                   const int32_t* seq_len, const ripe_group_t* groups,
                                                   const int32_t* parents, int32_t n_groups, int32_t n_rows,
                                                   float softmax_scale, const void* q, const void* kv_new,
                                                   void* out, float* lse, int8_t* plane_sel, void* workspace,
                                                   size_t workspace_bytes, void* stream) {
  if (parents == nullptr && n_groups > 0) return RIPE_EINVAL;
  return verify_impl(desc, cache, nullptr, seq_len, groups, parents, n_groups, n_rows, softmax_scale, q, kv_new,
                     out, lse, plane_sel, workspace, workspace_bytes, stream);
}

extern "C" ripe_status_t ripe_verify_attn_paged(const ripe_desc_t* desc, const void* cache, const int32_t* block_table,
                                                const int32_t* seq_len, const ripe_group_t* groups,
                                                const int32_t* parents, int32_t n_groups, int32_t n_rows,
                                                float softmax_scale, const void* q, const void* kv_new, void* out,
                                                float* lse, int8_t* plane_sel, void* workspace,
                                                size_t workspace_bytes, void* stream) {
  if (block_table == nullptr) return RIPE_EINVAL;
  return verify_impl(desc, cache, block_table, seq_len, groups, parents, n_groups, n_rows, softmax_scale, q,
                     kv_new, out, lse, plane_sel, workspace, workspace_bytes, stream);
}

// Side statistic on a FULL cache: the FULL outputs at each group's depth
// (a verify pass written in fp32), then the substitution error per prefix
// position and KV head, then the sum over KV heads.
extern "C" ripe_status_t ripe_position_error(const ripe_desc_t* desc, const void* cache, const int32_t* seq_len,
                                             const ripe_group_t* groups, int32_t n_groups, int32_t n_rows,
                                             float softmax_scale, const void* q, const void* kv_new, float* err,
                                             float* cond, float* out_f32, float* lse, void* workspace,
                                             size_t workspace_bytes, void* stream) {
  const ripe_status_t st = check_desc(desc);
  if (st != RIPE_OK) return st;
  const ripe_desc_t& d = *desc;
  if (d.layout != RIPE_LAYOUT_FULL || d.page_len > 0) return RIPE_EUNSUPPORTED;
  if (n_groups < 0) return RIPE_EINVAL;
  if (n_groups == 0) return RIPE_OK;
  if (err == nullptr || !aligned(err, 4) || (cond && !aligned(cond, 4)) || (out_f32 && !aligned(out_f32, 16)) ||
      (lse && !aligned(lse, 4)))
    return RIPE_EINVAL;
  if (groups == nullptr || seq_len == nullptr || n_rows < 1) return RIPE_EINVAL;
  if (workspace == nullptr) return RIPE_EWORKSPACE;
  if (!aligned(workspace, 256)) return RIPE_EINVAL;
  const int64_t extra = poserr_extra(d, n_rows, n_groups, out_f32 == nullptr, lse == nullptr);
  if (extra < 0) return RIPE_EUNSUPPORTED;
  if (size_t(extra) > workspace_bytes) return RIPE_EWORKSPACE;
  char* ws = static_cast<char*>(workspace);
  const int64_t ob = out_f32 ? 0 : align256(int64_t(n_rows) * d.n_q_heads * d.head_dim * 4);
  const int64_t lb = lse ? 0 : align256(int64_t(n_rows) * d.n_q_heads * 4);
  float* O = out_f32 ? out_f32 : reinterpret_cast<float*>(ws);
  float* L = lse ? lse : reinterpret_cast<float*>(ws + ob);
  const int64_t sb = align256(int64_t(n_groups) * d.n_kv_heads * d.t_max * 4);
  float* part = reinterpret_cast<float*>(ws + ob + lb);
  float* part_cond = reinterpret_cast<float*>(ws + ob + lb + sb);
  // verify_impl validates the groups, lengths and pointers before launching
  const ripe_status_t vs = verify_impl(desc, cache, nullptr, seq_len, groups, nullptr, n_groups, n_rows, softmax_scale, q,
                                       kv_new, O, L, nullptr, ws + extra, workspace_bytes - size_t(extra), stream,
                                       true);
  if (vs != RIPE_OK) return vs;
  PosErrParams p;
  p.cache_k = cache;
  p.cache_v = static_cast<const char*>(cache) + size_t(region_elems(d)) * elem_bytes(d.dtype);
  p.q = q;
  p.o = O;
  p.lse = L;
  p.part = part;
  p.part_cond = part_cond;
  p.err = err;
  p.cond = cond;
  p.R = d.R;
  p.H = d.n_kv_heads;
  p.Hq = d.n_q_heads;
  p.G = d.n_q_heads / d.n_kv_heads;
  p.t_max = d.t_max;
  p.scale = softmax_scale;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  for (int g0 = 0; g0 < n_groups; g0 += kPeGroups) {
    p.g0 = g0;
    p.n_grp = std::min(kPeGroups, n_groups - g0);
    for (int k = 0; k < p.n_grp; ++k) {
      const ripe_group_t& g = groups[g0 + k];
      p.grp[k].row_start = g.row_start;
      p.grp[k].n_rows = g.n_rows;
      p.grp[k].T = seq_len[g.seq];
      p.grp[k].b = uint16_t(g.seq);
      p.grp[k].depth = uint16_t(g.depth);
    }
    const ripe_status_t ls = hip_status(launch_position_error(p, d.dtype, d.head_dim, hs), "ripe_position_error");
    if (ls != RIPE_OK) return ls;
  }
  return RIPE_OK;
}

// Both commit entry points (table: the block table of a paged cache, or
// nullptr).
static ripe_status_t commit_impl(const ripe_desc_t* desc, void* cache, const int32_t* table, int32_t* seq_len,
                                 const int32_t* n_accept, const int32_t* src_row, const void* kv_new,
                                 int32_t n_rows, void* stream) {
  ripe_status_t st = check_desc(desc);
  if (st != RIPE_OK) return st;
  const ripe_desc_t& d = *desc;
  if ((d.page_len > 0) != (table != nullptr)) return RIPE_EINVAL;
  if (seq_len == nullptr || n_accept == nullptr || src_row == nullptr || n_rows < 0) return RIPE_EINVAL;
  bool any = false;
  for (int b = 0; b < d.batch; ++b) {
    if (seq_len[b] < 0 || seq_len[b] > d.t_max) return RIPE_ERANGE;
    const int n = n_accept[b];
    if (n < 0) return RIPE_EINVAL;
    if (n == 0) continue;
    any = true;
    if (src_row[b] < 0 || int64_t(src_row[b]) + n > n_rows) return RIPE_ERANGE;
    if (int64_t(seq_len[b]) + n > d.t_max) return RIPE_ECAPACITY;
  }
  if (!any) return RIPE_OK;
  if (cache == nullptr || kv_new == nullptr || !aligned(cache, 16) || !aligned(kv_new, 16)) return RIPE_EINVAL;
  const int P = d.page_len;
  const int nblk = P > 0 ? d.t_max / P : 0;
  if (table != nullptr) {
    // the pages written must exist, and no (page, slot) may be written twice
    struct Span {
      int page, lo, hi;
    };
    std::vector<Span> spans;
    for (int b = 0; b < d.batch; ++b) {
      const int n = n_accept[b];
      if (n == 0) continue;
      const int T = seq_len[b];
      for (int k = T / P; k * P < T + n; ++k) {
        const int pg = table[b * nblk + k];
        if (pg < 0 || pg >= d.n_pages) return RIPE_ERANGE;
        spans.push_back(Span{pg, std::max(T, k * P) - k * P, std::min(T + n, (k + 1) * P) - k * P});
      }
    }
    std::sort(spans.begin(), spans.end(),
              [](const Span& x, const Span& y) { return x.page != y.page ? x.page < y.page : x.lo < y.lo; });
    for (size_t i = 1; i < spans.size(); ++i)
      if (spans[i].page == spans[i - 1].page && spans[i].lo < spans[i - 1].hi) return RIPE_EINVAL;
  }

  const int D = d.head_dim;
  const int We = ring_width(d);
  const size_t E = elem_bytes(d.dtype);
  const int64_t reg = region_elems(d);
  struct Job {
    int b, j0, src0, n, plane_lo, n_planes, page;
  };
  std::vector<Job> jobs;
  auto push = [&](int b, int j0, int src0, int n, int plane_lo, int n_planes, int page) {
    jobs.push_back(Job{b, j0, src0, n, plane_lo, n_planes, page});
  };
  // main-region rows of a paged cache: one job per page touched
  auto add = [&](int b, int j0, int src0, int n, int plane_lo, int n_planes) {
    const bool main_region = !(d.layout == RIPE_LAYOUT_RIPE && plane_lo < d.R);
    if (table == nullptr || !main_region) return push(b, j0, src0, n, plane_lo, n_planes, 0);
    for (int a = j0; a < j0 + n;) {
      const int e = std::min(j0 + n, (a / P + 1) * P);
      push(b, a, src0 + (a - j0), e - a, plane_lo, n_planes, table[b * nblk + a / P]);
      a = e;
    }
  };
  for (int b = 0; b < d.batch; ++b) {
    const int n = n_accept[b];
    if (n == 0) continue;
    const int T = seq_len[b];
    const int s = src_row[b];
    if (d.layout == RIPE_LAYOUT_FULL) {
      add(b, T, s, n, 1, d.R);
    } else {
      add(b, T, s, n, d.R, 1);
      if (d.layout == RIPE_LAYOUT_RIPE && We > 0 && d.R > 1) {
        const int k0 = n > We ? n - We : 0;  // rows that end inside the window
        add(b, T + k0, s + k0, n - k0, 1, d.R - 1);
      }
    }
  }
  // V blocks a job rewrites.  Two tasks of one launch never touch the same
  // block (a job's own ranges are disjoint; a job whose blocks meet those of
  // an earlier job of the launch, such as a sequence sharing a page, starts
  // a new launch), so the read-modify-write of a block never races.
  struct Blocks {
    int s0, ring, blk0, nblk0, blk1, nblk1;
  };
  auto blocks_of = [&](const Job& jb) {
    Blocks k{};
    const bool ring = d.layout == RIPE_LAYOUT_RIPE && jb.plane_lo < d.R;
    k.ring = ring ? We : 0;
    k.s0 = ring ? jb.j0 % We : (table != nullptr ? jb.j0 % P : jb.j0);
    const int e = k.s0 + jb.n;  // one past the last slot, before a ring's wrap
    if (!ring || e <= We) {
      k.blk0 = k.s0 / kVBlock;
      k.nblk0 = (e - 1) / kVBlock - k.blk0 + 1;
    } else {  // slots [s0, We) then [0, e - We)
      const int last = (We - 1) / kVBlock, wrap_last = (e - We - 1) / kVBlock;
      if (wrap_last >= k.s0 / kVBlock) {
        k.blk0 = 0;
        k.nblk0 = last + 1;
      } else {
        k.blk0 = k.s0 / kVBlock;
        k.nblk0 = last - k.blk0 + 1;
        k.blk1 = 0;
        k.nblk1 = wrap_last + 1;
      }
    }
    return k;
  };
  // a launch's blocks: (region, block) with region = page, or sequence and
  // main / ring
  std::unordered_set<int64_t> taken;
  auto key = [&](const Job& jb, const Blocks& k, int blk) {
    const int64_t region = k.ring ? 2 * int64_t(jb.b) + 1 : (table != nullptr ? 2 * (int64_t(d.batch) + jb.page) : 2 * int64_t(jb.b));
    return region * (int64_t(d.t_max) / kVBlock + 1) + blk;
  };
  std::vector<CommitParams> launches;
  size_t i = 0;
  while (i < jobs.size()) {
    CommitParams p;
    std::memset(&p, 0, sizeof(p));
    p.cache_k = cache;
    p.cache_v = static_cast<char*>(cache) + size_t(reg) * E;
    p.kv_new = kv_new;
    p.ring_off = ring_offset(d);
    p.page_len = P;
    p.layout = d.layout;
    p.R = d.R;
    p.We = We;
    p.t_max = d.t_max;
    p.H = d.n_kv_heads;
    p.n_rows = n_rows;
    int64_t tasks = 0, max_nt = 0;
    int nj = 0;
    taken.clear();
    for (; i < jobs.size() && nj < kMaxJobs; ++i) {
      const Job& jb = jobs[i];
      const Blocks k = blocks_of(jb);
      const int64_t nt = int64_t(jb.n_planes) * d.n_kv_heads * (k.nblk0 + k.nblk1);
      // the grid has one row per job, as long as the largest: jobs of very
      // different sizes go to separate launches
      const int64_t mx = std::max(max_nt, nt);
      if (nj > 0 && (tasks + nt > kMaxCommitTasks || mx * (nj + 1) > 2 * (tasks + nt) + (int64_t(1) << 16))) break;
      bool clash = false;
      for (int r = 0; r < 2 && !clash; ++r)
        for (int q = 0; q < (r ? k.nblk1 : k.nblk0) && !clash; ++q)
          clash = taken.count(key(jb, k, (r ? k.blk1 : k.blk0) + q)) != 0;
      if (clash) break;  // (never for a launch's first job: its blocks are still free)
      for (int r = 0; r < 2; ++r)
        for (int q = 0; q < (r ? k.nblk1 : k.nblk0); ++q) taken.insert(key(jb, k, (r ? k.blk1 : k.blk0) + q));
      CommitJob& cj = p.job[nj++];
      cj.n_tasks = int32_t(nt);
      cj.s0 = k.s0;
      cj.src0 = jb.src0;
      cj.n_rows = jb.n;
      cj.page = jb.page;
      cj.ring = k.ring;
      cj.b = uint16_t(jb.b);
      cj.plane_lo = uint8_t(jb.plane_lo);
      cj.n_planes = uint8_t(jb.n_planes);
      cj.blk0 = k.blk0;
      cj.nblk0 = k.nblk0;
      cj.blk1 = k.blk1;
      cj.nblk1 = k.nblk1;
      tasks += nt;
      max_nt = mx;
    }
    p.n_jobs = nj;
    for (int j = 0; j < nj; ++j) p.max_tasks = std::max(p.max_tasks, p.job[j].n_tasks);
    launches.push_back(p);
  }
  hipStream_t hs = static_cast<hipStream_t>(stream);
  for (const CommitParams& p : launches)
    if (hip_status(launch_commit(p, d.dtype, D, hs), "ripe_commit") != RIPE_OK) return RIPE_EHIP;
  for (int b = 0; b < d.batch; ++b) seq_len[b] += n_accept[b];
  return RIPE_OK;
}

extern "C" ripe_status_t ripe_commit(const ripe_desc_t* desc, void* cache, int32_t* seq_len,
                                     const int32_t* n_accept, const int32_t* src_row, const void* kv_new,
                                     int32_t n_rows, void* stream) {
  return commit_impl(desc, cache, nullptr, seq_len, n_accept, src_row, kv_new, n_rows, stream);
}

extern "C" ripe_status_t ripe_commit_paged(const ripe_desc_t* desc, void* cache, const int32_t* block_table,
                                           int32_t* seq_len, const int32_t* n_accept, const int32_t* src_row,
                                           const void* kv_new, int32_t n_rows, void* stream) {
  if (block_table == nullptr) return RIPE_EINVAL;
  return commit_impl(desc, cache, block_table, seq_len, n_accept, src_row, kv_new, n_rows, stream);
}

extern "C" ripe_status_t ripe_position_error_tail(const float* err, const float* cond, const int32_t* T,
                                                  int32_t n_rows, int32_t row_stride, int32_t window,
                                                  double tail_frac, double* stats, void* stream) {
  if (n_rows < 0 || row_stride < 0 || window < 0 || !(tail_frac > 0.0 && tail_frac <= 1.0)) return RIPE_EINVAL;
  if (n_rows == 0) return RIPE_OK;
  if (T == nullptr || err == nullptr || stats == nullptr || !aligned(err, 4) || (cond && !aligned(cond, 4)) ||
      !aligned(stats, 8))
    return RIPE_EINVAL;
  for (int i = 0; i < n_rows; ++i)
    if (T[i] < 0 || T[i] > row_stride) return RIPE_ERANGE;
  TailParams p;
  p.err = err;
  p.cond = cond;
  p.stats = stats;
  p.stride = row_stride;
  p.window = window;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  for (int g0 = 0; g0 < n_rows; g0 += kTailRows) {
    p.g0 = g0;
    p.n_rows = std::min(kTailRows, n_rows - g0);
    for (int k = 0; k < p.n_rows; ++k) {
      const int t = T[g0 + k];
      p.T[k] = t;
      p.n_tail[k] = t == 0 ? 0 : std::max(1, int(std::floor(tail_frac * double(t))));
    }
    if (hip_status(launch_position_error_tail(p, hs), "ripe_position_error_tail") != RIPE_OK) return RIPE_EHIP;
  }
  return RIPE_OK;
}

extern "C" int64_t ripe_accept_workspace_bytes(const ripe_accept_desc_t* desc) {
  if (desc == nullptr) return RIPE_EINVAL;
  const ripe_accept_desc_t& d = *desc;
  if (d.batch < 0 || d.k < 1 || d.vocab < 1 || !std::isfinite(d.temperature) || d.temperature < 0.f)
    return RIPE_EINVAL;
  if (d.k > 64 || d.vocab > (1 << 24)) return RIPE_EUNSUPPORTED;
  if (d.batch == 0) return 0;
  return accept_layout(d.batch, d.k, d.vocab).bytes;
}

extern "C" ripe_status_t ripe_accept(const ripe_accept_desc_t* desc, const float* target_logits,
                                     const float* draft_logits, const int32_t* tokens,
                                     const uint8_t* has_fallback, const uint32_t* rand, int32_t* n_accept,
                                     int32_t* branch, int32_t* next_token, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  const int64_t need = ripe_accept_workspace_bytes(desc);
  if (need < 0) return static_cast<ripe_status_t>(need);
  const ripe_accept_desc_t& d = *desc;
  if (d.batch == 0) return RIPE_OK;
  const bool greedy = d.temperature == 0.f;
  if (target_logits == nullptr || tokens == nullptr || has_fallback == nullptr || n_accept == nullptr ||
      branch == nullptr || next_token == nullptr || (!greedy && (draft_logits == nullptr || rand == nullptr)))
    return RIPE_EINVAL;
  const void* ptrs[] = {target_logits, draft_logits, tokens, has_fallback, rand, n_accept, branch, next_token};
  for (const void* q : ptrs)
    if (q != nullptr && !aligned(q, 16)) return RIPE_EINVAL;
  if (workspace == nullptr || int64_t(workspace_bytes) < need) return RIPE_EWORKSPACE;
  if (!aligned(workspace, 256)) return RIPE_EINVAL;
  AcceptParams p;
  p.target = target_logits;
  p.draft = draft_logits;
  p.tokens = tokens;
  p.has_fb = has_fallback;
  p.rand = rand;
  p.n_accept = n_accept;
  p.branch = branch;
  p.next_token = next_token;
  const AcceptLayout L = accept_layout(d.batch, d.k, d.vocab);
  char* ws = static_cast<char*>(workspace);
  p.part = reinterpret_cast<RowStat*>(ws + L.off_part);
  p.stats = reinterpret_cast<RowStat*>(ws + L.off_stats);
  p.state = reinterpret_cast<SeqState*>(ws + L.off_state);
  p.sums = reinterpret_cast<double*>(ws + L.off_sums);
  p.tiles = reinterpret_cast<double*>(ws + L.off_tiles);
  p.last = reinterpret_cast<int32_t*>(ws + L.off_last);
  p.ptot = reinterpret_cast<double*>(ws + L.off_ptot);
  p.split = L.split;
  p.slice = L.slice;
  p.n_tiles = L.n_tiles;
  p.B = d.batch;
  p.k = d.k;
  p.V = d.vocab;
  p.greedy = greedy ? 1 : 0;
  p.inv_tau = greedy ? 0.0 : 1.0 / double(d.temperature);
  return hip_status(launch_accept(p, static_cast<hipStream_t>(stream)), "ripe_accept");
}
