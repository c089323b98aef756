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
#include <queue>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "plan.h"
#include "ripe.h"

namespace ripe {
hipError_t launch_verify(const VerifyParams& p, const ItemTable& t, const UnitTable& u, int grid, int dtype, int D,
                         int NB, hipStream_t stream);
int verify_slots(int dtype, int D, int NB);
hipError_t launch_commit(const CommitParams& p, int dtype, int D, hipStream_t stream);
}  // namespace ripe

namespace {

using namespace ripe;

constexpr int64_t kMaxBytes = int64_t(1) << 50;   // sanity bound on any buffer size
constexpr int64_t kMaxCommitItems = int64_t(1) << 30;  // commit work items per launch
constexpr int kMaxCQ = 32;                        // query columns per verify work-group

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

int ring_width(const ripe_desc_t& d) {
  if (d.layout != RIPE_LAYOUT_RIPE) return 0;
  return d.W < d.t_max ? d.W : d.t_max;
}

int split_len(const ripe_desc_t& d) {
  if (d.split_len > 0) return d.split_len;
  const int G = d.n_q_heads / d.n_kv_heads;
  // Few query columns per KV head -> small partials -> shorter splits for
  // more parallelism; many columns -> longer splits to amortise the partial.
  return G >= 4 ? 1024 : (G >= 2 ? 512 : 256);
}

// Elements of one region (K or V) of the cache, or -1 on overflow.
int64_t region_elems(const ripe_desc_t& d) {
  const long double per_seq =
      d.layout == RIPE_LAYOUT_FULL ? (long double)d.R * d.t_max
      : d.layout == RIPE_LAYOUT_DEEPEST ? (long double)d.t_max
                                        : (long double)d.t_max + (long double)ring_width(d) * (d.R - 1);
  const long double n = per_seq * d.batch * d.n_kv_heads * d.head_dim;
  if (n * 2 * elem_bytes(d.dtype) > (long double)kMaxBytes) return -1;
  return int64_t(n);
}

ripe_status_t check_desc(const ripe_desc_t* d) {
  if (d == nullptr) return RIPE_EINVAL;
  if (d->layout < RIPE_LAYOUT_FULL || d->layout > RIPE_LAYOUT_RIPE) return RIPE_EINVAL;
  if (d->dtype != RIPE_F32 && d->dtype != RIPE_BF16) return RIPE_EINVAL;
  if (d->R < 1 || d->W < 0 || d->batch < 1 || d->t_max < 1 || d->n_kv_heads < 1 || d->head_dim < 1 ||
      d->n_q_heads < 1 || d->max_rows < 0 || d->max_groups < 0 || d->split_len < 0)
    return RIPE_EINVAL;
  if (d->n_q_heads % d->n_kv_heads != 0) return RIPE_EINVAL;
  if (d->R > 127 || d->batch > 65535) return RIPE_EUNSUPPORTED;
  if (d->head_dim != 64 && d->head_dim != 128) return RIPE_EUNSUPPORTED;
  if (d->t_max % 32 != 0 || d->split_len % 32 != 0) return RIPE_EUNSUPPORTED;
  if (d->n_q_heads / d->n_kv_heads > 65535) return RIPE_EUNSUPPORTED;
  const int We = ring_width(*d);
  if (!(We == 0 || (We < 32 && We % 8 == 0) || We % 32 == 0)) return RIPE_EUNSUPPORTED;
  if (region_elems(*d) < 0) return RIPE_EUNSUPPORTED;
  return RIPE_OK;
}

// Upper bound on split partial slots of any verify call within the
// descriptor's max_rows / max_groups bounds.
int64_t workspace_bound(const ripe_desc_t& d) {
  const int64_t S = split_len(d);
  const int64_t G = d.n_q_heads / d.n_kv_heads;
  const int64_t We = ring_width(d);
  const int64_t groups = std::max<int64_t>(d.max_groups, 1);
  const int64_t rows = std::max<int64_t>(d.max_rows, groups);
  const int64_t nseq = std::min<int64_t>(d.batch, groups);
  const int64_t tchunks = (int64_t(d.t_max) + S - 1) / S;
  int64_t per_seq = (d.layout == RIPE_LAYOUT_FULL ? std::min<int64_t>(groups, d.R) : 1) * tchunks;
  if (d.layout == RIPE_LAYOUT_RIPE) per_seq += std::min<int64_t>(groups, d.R - 1) * ((We + S - 1) / S);
  per_seq += groups + (rows + S - 1) / S;
  const int64_t col_chunks = (rows * G + 15) / 16 + nseq;
  const long double slots = (long double)d.n_kv_heads * col_chunks * per_seq;
  const long double bytes = slots * kMaxCQ * (d.head_dim + 2) * 4 + 256;
  if (bytes > (long double)kMaxBytes) return -1;
  return int64_t(bytes);
}

struct LaunchPlan {
  VerifyParams p;
  ItemTable t;
  UnitTable u;
  int grid;            // persistent work-groups
  int64_t part_bytes;  // split partials
};

// Per-thread planning buffers, reused across calls (no per-call allocation
// once they have grown to the call sizes in use).
struct VerifyScratch {
  std::vector<std::pair<int, int>> spans;
  std::vector<int> count, fill, order;
  std::vector<Seg> segs;
  std::vector<Item> tail;
  std::vector<int> by_size, bin_of, bin_cnt;
  std::vector<LaunchPlan> plans;
  int n_plans = 0;
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
  return RIPE_EINVAL;
}

extern "C" ripe_status_t ripe_verify_attn(const ripe_desc_t* desc, const void* cache, const int32_t* seq_len,
                                          const ripe_group_t* groups, int32_t n_groups, int32_t n_rows,
                                          float softmax_scale, const void* q, const void* kv_new, void* out,
                                          float* lse, int8_t* plane_sel, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  ripe_status_t st = check_desc(desc);
  if (st != RIPE_OK) return st;
  const ripe_desc_t& d = *desc;
  if (n_groups < 0) return RIPE_EINVAL;
  if (n_groups == 0) return RIPE_OK;
  if (groups == nullptr || seq_len == nullptr || n_rows < 1) return RIPE_EINVAL;
  if (n_groups > 65535) return RIPE_EUNSUPPORTED;
  if (!std::isfinite(softmax_scale)) return RIPE_EINVAL;
  if (cache == nullptr || q == nullptr || kv_new == nullptr || out == nullptr) return RIPE_EINVAL;
  if (!aligned(cache, 16) || !aligned(q, 16) || !aligned(kv_new, 16) || !aligned(out, 16)) return RIPE_EINVAL;
  if ((lse && !aligned(lse, 4)) || (plane_sel && !aligned(plane_sel, 16))) return RIPE_EINVAL;
  if (workspace && !aligned(workspace, 256)) return RIPE_EINVAL;
  for (int b = 0; b < d.batch; ++b)
    if (seq_len[b] < 0 || seq_len[b] > d.t_max) return RIPE_ERANGE;
  const int G = d.n_q_heads / d.n_kv_heads;
  VerifyScratch& sc = verify_scratch();
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

  const int D = d.head_dim;
  const int We = ring_width(d);
  const int S = split_len(d);
  const size_t E = elem_bytes(d.dtype);
  const int64_t reg = region_elems(d);
  const char* cache_k = static_cast<const char*>(cache);
  const char* cache_v = cache_k + size_t(reg) * E;

  // Pack (sequence, KV-head range) pieces into launches of <= kMaxItems
  // items, <= kMaxSeq sequence records and <= kMaxGroups group records.
  sc.n_plans = 0;
  auto new_plan = [&]() -> LaunchPlan& {
    if (sc.plans.size() <= size_t(sc.n_plans)) sc.plans.emplace_back();
    LaunchPlan& lp = sc.plans[sc.n_plans++];
    VerifyParams& p = lp.p;
    p.cache_k = cache_k;
    p.cache_v = cache_v;
    p.q = q;
    p.kv_new = kv_new;
    p.out = out;
    p.lse = lse;
    p.plane_sel = plane_sel;
    p.ws = static_cast<float*>(workspace);
    p.ring_off = uint64_t(d.batch) * d.n_kv_heads * uint64_t(d.t_max) * D;
    p.layout = d.layout;
    p.R = d.R;
    p.We = We;
    p.BW = We < 32 ? We : 32;
    p.t_max = d.t_max;
    p.H = d.n_kv_heads;
    p.Hq = d.n_q_heads;
    p.G = G;
    p.n_rows = n_rows;
    p.S = S;
    p.n_seq = 0;
    p.n_wg = 0;
    p.n_units = 0;
    p.n_grp = 0;
    p.scale_log2 = float(double(softmax_scale) * 1.4426950408889634);
    return lp;
  };
  LaunchPlan* cur = nullptr;
  GroupRec grp[kMaxGroups];
  for (int b = 0; b < d.batch; ++b) {
    const int g0 = sc.count[b], gc = sc.count[b + 1] - sc.count[b];
    if (gc == 0) continue;
    int nq = 0;
    for (int k = 0; k < gc; ++k) {
      const ripe_group_t& g = groups[sc.order[g0 + k]];
      grp[k].row_start = g.row_start;
      grp[k].n_rows = uint16_t(g.n_rows);
      grp[k].depth = uint8_t(g.depth);
      grp[k].seq = 0;
      nq += g.n_rows * G;
    }
    const int T = seq_len[b];
    sc.segs.clear();
    int64_t n_split = 0;
    enumerate_segments(d.layout, d.R, We, T, grp, 0, gc, [&](const Seg& sg) {
      sc.segs.push_back(sg);
      n_split += (int64_t(sg.len) + S - 1) / S;
      return false;
    });
    const int n_cc = (nq + CQ - 1) / CQ;
    const int64_t per_head = n_split * n_cc;
    if (per_head > kMaxItems) return RIPE_EUNSUPPORTED;  // one KV head must fit a launch
    int h = 0;
    while (h < d.n_kv_heads) {
      if (cur == nullptr || cur->p.n_seq == kMaxSeq || cur->p.n_grp + gc > kMaxGroups ||
          cur->p.n_wg + per_head > kMaxItems)
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
      for (int k = 0; k < gc; ++k) {
        p.grp[p.n_grp] = grp[k];
        p.grp[p.n_grp].seq = uint8_t(p.n_seq);
        p.gorig[p.n_grp] = uint16_t(sc.order[g0 + k]);
        ++p.n_grp;
      }
      // items: unit (h, cc) and chunk `split` of the sequence's segment list;
      // partial slot = part0 + ((h - h0) * n_cc + cc) * n_split + split
      for (int hh = 0; hh < hc; ++hh)
        for (int cc = 0; cc < n_cc; ++cc) {
          int split = 0;
          for (const Seg& sg : sc.segs) {
            for (int c0 = 0; c0 < sg.len; c0 += S, ++split) {
              Item& it = cur->t.item[p.n_wg++];
              it.c0 = c0;
              it.seg_len = sg.len;
              it.part = sr.part0 + (hh * n_cc + cc) * int(n_split) + split;
              it.h = uint16_t(h + hh);
              it.cc = uint16_t(cc);
              it.s = uint8_t(p.n_seq);
              it.kind = uint8_t(sg.kind);
              it.depth = uint8_t(sg.depth);
              it.gidx = uint8_t(sg.kind == kSegDraft ? sr.g_begin + sg.gidx : 0);
            }
          }
        }
      for (int hh = 0; hh < hc; ++hh)
        for (int cc = 0; cc < n_cc; ++cc) {
          Unit& un = cur->u.unit[p.n_units + hh * n_cc + cc];
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
  // Persistent work-groups: as many as fit on the device at once (at most
  // kMaxSlots).  Items are assigned longest first to the least-loaded
  // work-group (cost = 32-position steps + a fixed per-item latency).
  for (int pi = 0; pi < sc.n_plans; ++pi) {
    LaunchPlan& lp = sc.plans[pi];
    lp.part_bytes = int64_t(lp.p.n_wg) * CQ * (D + 2) * 4;
    if (workspace == nullptr || size_t(lp.part_bytes) > workspace_bytes) return RIPE_EWORKSPACE;
  }
  int slots = sc.n_plans > 0 ? verify_slots(d.dtype, D, NB) : 0;
  if (slots <= 0) slots = 512;
  slots = std::min(slots, kMaxSlots);
  for (int pi = 0; pi < sc.n_plans; ++pi) {
    LaunchPlan& lp = sc.plans[pi];
    Item* items = lp.t.item;
    const int n = lp.p.n_wg;
    auto cost = [&](const Item& it) { return (std::min(S, it.seg_len - it.c0) + kStep - 1) / kStep + 2; };
    sc.by_size.resize(n);
    for (int i = 0; i < n; ++i) sc.by_size[i] = i;
    std::stable_sort(sc.by_size.begin(), sc.by_size.end(),
                     [&](int x, int y) { return cost(items[x]) > cost(items[y]); });
    const int W = std::min(n, slots);
    using Load = std::pair<int64_t, int>;  // (accumulated cost, work-group)
    std::priority_queue<Load, std::vector<Load>, std::greater<Load>> heap;
    for (int w = 0; w < W; ++w) heap.push(Load(0, w));
    sc.bin_of.resize(n);
    sc.bin_cnt.assign(W + 1, 0);
    for (int k = 0; k < n; ++k) {
      Load top = heap.top();
      heap.pop();
      const int i = sc.by_size[k];
      sc.bin_of[i] = top.second;
      ++sc.bin_cnt[top.second + 1];
      top.first += cost(items[i]);
      heap.push(top);
    }
    for (int w = 0; w < W; ++w) sc.bin_cnt[w + 1] += sc.bin_cnt[w];
    for (int w = 0; w <= W; ++w) lp.t.first[w] = uint16_t(sc.bin_cnt[w]);
    // place items by work-group, each work-group's items longest first
    sc.tail.resize(n);
    std::vector<int>& fill = sc.fill;
    fill.assign(sc.bin_cnt.begin(), sc.bin_cnt.end() - 1);
    for (int k = 0; k < n; ++k) {
      const int i = sc.by_size[k];
      sc.tail[fill[sc.bin_of[i]]++] = items[i];
    }
    std::copy(sc.tail.begin(), sc.tail.end(), items);
    lp.grid = W;
  }
  hipStream_t hs = static_cast<hipStream_t>(stream);
  for (int pi = 0; pi < sc.n_plans; ++pi) {
    const LaunchPlan& lp = sc.plans[pi];
    const ripe_status_t st2 = hip_status(launch_verify(lp.p, lp.t, lp.u, lp.grid, d.dtype, D, NB, hs), "ripe_verify_attn");
    if (st2 != RIPE_OK) return st2;
  }
  return RIPE_OK;
}

extern "C" ripe_status_t ripe_commit(const ripe_desc_t* desc, void* cache, int32_t* seq_len,
                                     const int32_t* n_accept, const int32_t* src_row, const void* kv_new,
                                     int32_t n_rows, void* stream) {
  ripe_status_t st = check_desc(desc);
  if (st != RIPE_OK) return st;
  const ripe_desc_t& d = *desc;
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

  const int D = d.head_dim;
  const int We = ring_width(d);
  const size_t E = elem_bytes(d.dtype);
  const int64_t reg = region_elems(d);
  const int64_t per_row_plane = int64_t(d.n_kv_heads) * (D / 8);  // items per (row, plane)

  struct Job {
    int b, j0, src0, n, plane_lo, n_planes;
  };
  std::vector<Job> jobs;
  auto add = [&](int b, int j0, int src0, int n, int plane_lo, int n_planes) {
    // cut rows so that no job exceeds the per-launch item budget
    const int64_t per_row = per_row_plane * n_planes;
    const int max_rows = int(std::max<int64_t>(1, kMaxCommitItems / per_row));
    for (int r0 = 0; r0 < n; r0 += max_rows) {
      const int cnt = std::min(max_rows, n - r0);
      jobs.push_back(Job{b, j0 + r0, src0 + r0, cnt, plane_lo, n_planes});
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
  std::vector<CommitParams> launches;
  size_t i = 0;
  while (i < jobs.size()) {
    CommitParams p;
    std::memset(&p, 0, sizeof(p));
    p.cache_k = cache;
    p.cache_v = static_cast<char*>(cache) + size_t(reg) * E;
    p.kv_new = kv_new;
    p.ring_off = uint64_t(d.batch) * d.n_kv_heads * uint64_t(d.t_max) * D;
    p.layout = d.layout;
    p.R = d.R;
    p.We = We;
    p.BW = We < 32 ? We : 32;
    p.t_max = d.t_max;
    p.H = d.n_kv_heads;
    p.n_rows = n_rows;
    int64_t items = 0;
    int nj = 0;
    for (; i < jobs.size() && nj < kMaxJobs; ++i) {
      const Job& jb = jobs[i];
      const int64_t cnt = int64_t(jb.n) * jb.n_planes * per_row_plane;
      if (nj > 0 && items + cnt > kMaxCommitItems) break;
      CommitJob& cj = p.job[nj++];
      cj.item0 = int32_t(items);
      cj.j0 = jb.j0;
      cj.src0 = jb.src0;
      cj.n_rows = jb.n;
      cj.b = uint16_t(jb.b);
      cj.plane_lo = uint8_t(jb.plane_lo);
      cj.n_planes = uint8_t(jb.n_planes);
      items += cnt;
    }
    p.n_jobs = nj;
    p.n_items = int32_t(items);
    launches.push_back(p);
  }
  hipStream_t hs = static_cast<hipStream_t>(stream);
  for (const CommitParams& p : launches)
    if (hip_status(launch_commit(p, d.dtype, D, hs), "ripe_commit") != RIPE_OK) return RIPE_EHIP;
  for (int b = 0; b < d.batch; ++b) seq_len[b] += n_accept[b];
  return RIPE_OK;
}
