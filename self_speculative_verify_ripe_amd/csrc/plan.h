// plan.h -- work plan shared by the host planner and the gfx950 kernels.
//
// A verify call is split, per sequence, into segments that each read one
// source of keys and values:
//   kind 0  a prefix plane read in position order (FULL: plane r of each
//           distinct depth; DEEPEST: plane R; RIPE: the deep region, plane R,
//           over [0, T - Wb), or over [0, T) when a group sits at depth R);
//   kind 1  a RIPE window ring for each distinct depth r < R, read in ring
//           slot order (slot s holds the one window position j = s mod We);
//   kind 2  one group's own draft rows at its depth (causal within the group).
// The streamed segments of a sequence (prefix planes, then rings) are laid end
// to end and cut into n near-equal parts (n from the split length S, fixed by
// the descriptor), each cut falling on a segment boundary or on a multiple of
// 32 positions inside a segment.  A part is a list of runs (pieces), slices of
// one segment each; the sequence's draft-row segments (kinds 2-4) are
// appended to its last part.  A work item is one part for one KV head and one
// query-column chunk: one work-group reads its runs in order and writes one
// split partial.
//
// Workspace: a 256-byte header, one 64-bit arrival word per merge unit
// (kMaxItems of them; zero between calls), then the partials.
// The plan of a sequence depends only on the descriptor, its committed length
// and its own groups, so a group's result is bit-identical whether it is
// verified alone or batched with other sequences, and RIPE with W >= T (or
// W = 0) runs exactly the pieces of FULL (of DEEPEST).  Groups of one
// sequence share its pieces; a piece that does not apply to a group is masked
// for that group's query columns, which leaves its running softmax state
// bit-identical (factor 1, zero added).
#pragma once
#include <stddef.h>
#include <stdint.h>

#if defined(__HIPCC__)
#define RIPE_HD __host__ __device__
#else
#define RIPE_HD
#endif

namespace ripe {

constexpr int kStep = 32;        // key positions per wavefront step
constexpr int kWaves = 4;        // wavefronts per verify work-group
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxSeq = 64;      // sequences per launch
constexpr int kMaxGroups = 128;  // groups per launch
constexpr int kMaxJobs = 128;    // commit jobs per launch
constexpr int kMaxItems = 2048;  // verify work items (and merge units) per launch
constexpr int kMaxPieces = 512;  // runs (pieces) per launch
constexpr int kMaxPageRefs = 512;   // paged caches: pages after a piece's first, per launch
constexpr int kXcds = 8;         // work-group i of a grid runs on XCD i mod 8 (checked as it runs)
constexpr int64_t kWsArrive = 256;                          // arrival words
constexpr int64_t kWsHeader = kWsArrive + 8 * int64_t(kMaxItems);  // partials

// kinds 3 and 4: the rows of a parent block still in flight, read from the
// draft tensors at the plane they will be read from once committed: rows
// below the window at plane R (every group sees them), rows inside it at
// each group's depth (kind 4, one segment per distinct depth).
enum SegKind { kSegPlane = 0, kSegRing = 1, kSegDraft = 2, kSegParentDeep = 3, kSegParentWin = 4 };

struct GroupRec {      // one group of a launch (8 bytes), sorted by sequence
  int32_t row_start;
  uint16_t n_rows;
  uint8_t depth;
  uint8_t seq;         // launch-local sequence index
};

struct SeqRec {        // one sequence (or a KV-head range of it) in a launch
  int32_t T;           // committed prefix length
  int32_t part0;       // first split partial slot of its units
  int32_t unit0;       // first (KV head, column chunk) unit
  int32_t n_split;     // work items (= partials) per (KV head, column chunk)
  uint16_t b;          // sequence index within the cache
  uint16_t n_cc;       // query-column chunks
  uint16_t h0;         // first KV head of this launch's range
  uint16_t h_cnt;      // KV heads in the range
  uint8_t g_begin;     // first group record of this sequence
  uint8_t g_count;     // its number of groups
  uint16_t nq;         // query columns = sum(rows) * (Hq / Hkv)
  // RIPE window and in-flight parent (see InFlight)
  int32_t tw;          // prefix positions before the window (RIPE, depth < R)
  int32_t parent_row0; // first draft row of the in-flight parent block
  uint16_t kp;         // its rows (0: none)
  uint16_t nd;         // its rows below the window (read at plane R)
  uint16_t hole;       // oldest ring slots not read (now before the window)
  uint16_t ring_base;  // ring slot of the oldest window position
  // copies of its first two group records (the rest: VerifyParams::grp), so
  // that a sequence of at most two groups needs no record load after this one
  GroupRec g01[2];
};

// Where the window falls for a sequence with committed length T, ring width
// We, layout and a parent block of kp rows in flight: the prefix is read as
// it will be once the parent is committed, i.e. with the window covering the
// last We positions of T + kp.  A = first position inside that window.
struct InFlight {
  int tw;    // committed positions read at plane R by groups at depth < R (RIPE)
  int hole;  // ring positions (oldest first) that lie before the window
  int nd;    // parent rows before the window
  int ring_base;
};

RIPE_HD inline InFlight in_flight(int layout, int We, int T, int kp) {
  InFlight f;
  const int Wb = We < T ? We : T;
  const int A0 = T + kp - We;
  const int A = A0 > 0 ? A0 : 0;
  const int ring_lo = T - Wb;  // oldest position held in the ring
  f.ring_base = We > 0 ? ring_lo % We : 0;
  if (layout == 2) {
    f.tw = A < T ? A : T;
    f.hole = f.tw - ring_lo;
    const int nd = A - T;
    f.nd = nd < 0 ? 0 : (nd > kp ? kp : nd);
  } else {
    f.tw = T;
    f.hole = 0;
    f.nd = layout == 1 ? kp : 0;  // DEEPEST reads every parent row at plane R, FULL at depth r
  }
  return f;
}



// A run: positions of one segment of one sequence (12 bytes).
struct Piece {
  int32_t c0;          // first position, segment-local (a multiple of 32)
  int32_t len;         // positions (kind 0), ring slots (kind 1) or rows (kind 2)
  uint8_t kind;        // SegKind
  uint8_t depth;       // plane read (kind 0) or depth r (kinds 1, 2)
  uint8_t gidx;        // group record (kind 2)
  uint8_t s;           // launch-local sequence
};

// One verify work item (12 bytes): runs [r0, r0 + n_stream) streamed from
// the cache (prefix planes, rings), then runs [r0 + n_stream, r0 + n_run)
// read from the draft tensors (draft rows, parent rows), for KV head h and
// query-column chunk cc of launch-local sequence s, written to split
// partial slot `part`.  (s is here so that the sequence record loads beside
// the first run's, not after it.)
struct Item {
  uint16_t r0;
  uint8_t n_stream;
  uint8_t n_run;
  uint16_t part;
  uint16_t h;
  uint16_t cc;
  uint16_t s;          // launch-local sequence (its SeqRec)
};
static_assert(sizeof(Item) == 12 && offsetof(Item, part) == 4 && offsetof(Item, cc) == 8,
              "the verify kernel reads an item as three 32-bit words");

// Runs, work items and work-groups of one launch.  The items are stored in
// grid order (work-group j runs item[j]; see the planner for the placement
// order); the planner marks a grid position with no item kWgEmpty while it
// places them, and stores it as an item with no runs.
constexpr uint16_t kWgEmpty = 0xFFFF;

struct ItemTable {
  Piece piece[kMaxPieces];
  // in grid order: work-group j runs item[j]; an item with no runs marks a
  // grid position with no work (XCD placement leaves gaps)
  Item item[kMaxItems + 512];
  // paged caches: prefix-plane piece i starts in page pages[i] (read with the
  // piece itself); a piece spanning pages continues in pages[kMaxPieces +
  // pref[i]], pages[kMaxPieces + pref[i] + 1], ...
  uint16_t pref[kMaxPieces];
  int32_t pages[kMaxPieces + kMaxPageRefs];
};

// (sequence, KV head, column chunk) of each merge work-group (16 bytes).
// part and n_split let the merge issue its partial loads after this one
// record, before it reads the sequence and group records it needs only to
// place its outputs.
struct Unit {
  int32_t part;        // partial slot of the unit's split 0 (splits are consecutive)
  uint16_t n_split;    // its splits
  uint16_t s;          // launch-local sequence
  uint16_t h;          // KV head
  uint16_t cc;         // query-column chunk
  uint16_t hl;         // KV head within the sequence record's range
  uint16_t pad;
};

struct UnitTable {
  Unit unit[kMaxItems];
};

struct Seg {
  int kind;
  int depth;  // plane read (kind 0), depth r (kinds 1 and 2)
  int gidx;   // group record (kind 2)
  int len;    // positions (kind 0), slots (kind 1) or rows (kind 2)
};

struct VerifyParams {
  const void* cache_k;   // K region of the cache
  const void* cache_v;   // V region of the cache
  const void* q;
  const void* kv_new;
  void* out;
  float* lse;
  int8_t* plane_sel;
  float* ws;             // split partials, one per item (the verify kernel's PartLayout)
  unsigned long long* arrive;  // one arrival word per merge unit (fused merge)
  uint64_t ring_off;     // elements from a region's start to its ring (RIPE)
  int32_t layout, R, We, t_max, H, Hq, G, n_rows, n_seq, n_wg, n_units, n_grp, n_pieces;
  int32_t n_blocks;      // verify work-groups (grid-ordered entries of ItemTable::item)
  float scale_log2;      // softmax scale * log2(e)
  SeqRec seq[kMaxSeq];
  GroupRec grp[kMaxGroups];
  uint16_t gorig[kMaxGroups];  // index of each group in the caller's array
  int32_t inflight;      // some sequence of the launch has a parent block in flight
  int32_t out_f32;       // out is fp32 (else the storage dtype)
  int32_t page_len;      // paged cache: positions per page (0: unpaged)
  int32_t page_mode;     // 0 unpaged, 1 every prefix-plane piece in one page, 2 pieces may span pages
  int32_t n_refs;        // paged cache: entries of ItemTable::pages used past kMaxPieces
  int32_t fused;         // the last item of each unit merges it (else a merge kernel follows)
  int32_t k_stream;      // K rows non-temporal: some sequence has groups at several depths
};

constexpr int kVBlock = 8;  // positions per transposed V block [D][8]

// Rows of one sequence written to one region (44 bytes).  Row i goes to slot
// s0 + i of the region (a position, a page slot), or for a RIPE ring to slot
// (s0 + i) mod We.  One wavefront per (plane, head, block of kVBlock slots;
// a ring's last may be narrower) writes the K rows of the block's new slots
// and rewrites its V runs whole.  The blocks touched form one or two ranges
// [blk0, blk0 + nblk0) and [blk1, blk1 + nblk1) that share no block.
struct CommitJob {
  int32_t n_tasks;     // its wavefront tasks: planes x heads x blocks
  int32_t s0;          // slot of the job's first row
  int32_t src0;        // kv_new row of the job's first row
  int32_t n_rows;
  int32_t page;        // paged cache, main region: the page holding all the job's rows
  int32_t ring;        // We for a RIPE ring job, 0 for the main region
  uint16_t b;
  uint8_t plane_lo;    // first plane written (1-based)
  uint8_t n_planes;
  int32_t blk0, nblk0, blk1, nblk1;
};

struct CommitParams {
  void* cache_k;
  void* cache_v;
  const void* kv_new;
  uint64_t ring_off;
  int32_t layout, R, We, t_max, H, n_rows, n_jobs;
  int32_t max_tasks;        // the largest job's tasks
  int32_t page_len;         // paged cache: positions per page (0: unpaged)
  CommitJob job[kMaxJobs];  // a RIPE job with plane_lo < R writes the ring
};

RIPE_HD inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Visit the segments of one sequence in canonical order (kind 0, then kind 1,
// then kind 2); `visit` returns true to stop.  Distinct depths are visited in
// ascending order.
template <typename Visit>
RIPE_HD inline void enumerate_segments(int layout, int R, int We, int T, const GroupRec* g, int g_begin,
                                       int g_count, int kp, Visit&& visit) {
  const InFlight f = in_flight(layout, We, T, kp);
  const int Wb = We < T ? We : T;
  bool anyR = false;
  for (int i = 0; i < g_count; ++i) anyR |= (g[g_begin + i].depth == R);
  // visit one segment per distinct depth d with lo < d <= hi, in increasing order
  auto per_depth = [&](int kind, int hi, int len) -> bool {
    int cur = 0;
    while (len > 0) {
      int nxt = 1 << 30;
      for (int i = 0; i < g_count; ++i) {
        const int d = g[g_begin + i].depth;
        if (d > cur && d <= hi && d < nxt) nxt = d;
      }
      if (nxt == (1 << 30)) break;
      if (visit(Seg{kind, nxt, -1, len})) return true;
      cur = nxt;
    }
    return false;
  };
  if (layout == 0) {  // FULL: one plane segment per distinct depth
    if (per_depth(kSegPlane, R, T)) return;
  } else if (layout == 1) {  // DEEPEST
    if (T > 0 && visit(Seg{kSegPlane, R, -1, T})) return;
  } else {  // RIPE
    const int deep = anyR ? T : f.tw;
    if (deep > 0 && visit(Seg{kSegPlane, R, -1, deep})) return;
    if (Wb > f.hole && per_depth(kSegRing, R - 1, Wb)) return;
  }
  if (kp > 0) {
    if (f.nd > 0 && visit(Seg{kSegParentDeep, R, -1, f.nd})) return;
    if (kp > f.nd && per_depth(kSegParentWin, R, kp - f.nd)) return;
  }
  for (int i = 0; i < g_count; ++i) {
    const GroupRec& gr = g[g_begin + i];
    if (visit(Seg{kSegDraft, gr.depth, g_begin + i, gr.n_rows})) return;
  }
}

}  // namespace ripe
