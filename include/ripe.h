/*
 * ripe.h -- C ABI of the RIPE self-speculative verification library for
 * AMD Instinct MI355X (gfx950).
 *
 * In a looped (depth-recurrent) language model every token passes R times
 * through the same recurrent block, so the KV cache of a recurrent layer
 * keeps R planes, one per loop.  Self-speculative decoding proposes tokens
 * from a shallow loop count and checks them with all R loops, and that check
 * touches every plane (RIPE abstract, zhuanzhiai.com paper page, opening
 * sentence).  Three cache layouts are supported:
 *
 *   FULL     every plane at every position; depth r reads plane r;
 *   DEEPEST  only the deepest plane R, shared by all depths; every depth
 *            reads plane R;
 *   RIPE     plane R at every position plus planes 1..R-1 for a window of
 *            the W most recent committed positions; depth r reads plane r
 *            inside the window and plane R before it (RIPE abstract,
 *            sentence introducing RIPE).
 *
 * Depths are 1-based; plane R is the deepest.  Several draft groups (draft
 * blocks of different sequences, or LoopSpec-style branches of one sequence
 * at different depths) are verified in one call (LoopSpec summary on
 * rit.work: branches at different recurrent depths in one batched call).
 *
 * Conventions for every entry point:
 *  - Pointers marked "device" are HIP device memory owned by the caller;
 *    pointers marked "host" are read (or, for seq_len in ripe_commit,
 *    updated) before the call returns.  The library allocates no device
 *    memory.  Calls are asynchronous on `stream` (0 = the null stream) and
 *    never synchronise the host.
 *  - State kept between calls: each host thread keeps the work plan of its
 *    last verify call (host memory).  A verify call on the same thread whose
 *    descriptor, lengths, groups, parents, scale and block table equal that
 *    call's reuses the plan with the new buffer pointers.  The plan is a
 *    pure function of those inputs, so results never depend on the cache.
 *  - Every argument is validated on the host before any HIP call.  On an
 *    error nothing is launched and no output (device or host) is modified.
 *  - Device pointers must be 16-byte aligned (workspace: 256-byte aligned).
 *  - Input values must be finite.
 *  - A call launches kernels only (no allocation, no memset, no host
 *    synchronisation), so ripe_verify_attn and ripe_accept can be captured
 *    into a HIP graph; a captured call keeps the host arguments (sequence
 *    lengths, groups) it was captured with.  ripe_commit updates seq_len on
 *    the host, so a captured commit would replay the same positions.
 */
#ifndef RIPE_H_
#define RIPE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RIPE_LAYOUT_FULL = 0,
  RIPE_LAYOUT_DEEPEST = 1,
  RIPE_LAYOUT_RIPE = 2
} ripe_layout_t;

/* Element type shared by the cache, q, kv_new and out. */
typedef enum { RIPE_F32 = 0, RIPE_BF16 = 1 } ripe_dtype_t;

typedef enum {
  RIPE_OK = 0,
  RIPE_EINVAL = -1,        /* malformed argument (null, negative, misaligned) */
  RIPE_ERANGE = -2,        /* a depth, sequence, length or row index out of range */
  RIPE_ECAPACITY = -3,     /* commit would grow a sequence past t_max */
  RIPE_EUNSUPPORTED = -4,  /* well-formed but not supported (head_dim, window width, limits) */
  RIPE_EWORKSPACE = -5,    /* workspace missing or too small */
  RIPE_EHIP = -6           /* a HIP launch failed */
} ripe_status_t;

typedef enum {
  RIPE_BYTES_CACHE = 0,
  RIPE_BYTES_WORKSPACE = 1,
  RIPE_BYTES_POSERR_WORKSPACE = 2
} ripe_bytes_kind_t;

/*
 * One recurrent layer's cache (callers allocate one buffer per layer).
 *
 *  layout      ripe_layout_t
 *  dtype       ripe_dtype_t
 *  R           loops = planes, 1..127
 *  W           RIPE window in positions, any W >= 0 (ignored by FULL /
 *              DEEPEST).  W = 0 keeps only plane R; W >= t_max keeps every
 *              plane everywhere.  The ring holds We = min(W, t_max) slots.
 *  batch       sequences B >= 1
 *  t_max       capacity per sequence, a positive multiple of 32
 *  n_kv_heads  Hkv >= 1
 *  head_dim    D, 64 or 128
 *  n_q_heads   Hq, a multiple of Hkv (query head h reads KV head h / (Hq/Hkv))
 *  max_rows    upper bound on n_rows of a verify call   (workspace sizing)
 *  max_groups  upper bound on n_groups of a verify call (workspace sizing)
 *  split_len   prefix positions per split-K work item: 0 selects the
 *              library default, otherwise a positive multiple of 32.  The
 *              split plan of a sequence depends only on this descriptor and
 *              on that sequence's own groups and length, never on the other
 *              sequences of the call, so a group's results are bit-identical
 *              whether it is verified alone or batched.
 *  page_len    0: one contiguous region per sequence (the layouts below).
 *              Otherwise positions per page of a paged cache, a positive
 *              multiple of 32 dividing t_max: the positions of every
 *              sequence live in pages of a shared pool, found through a
 *              block table (see "Paged caches" below).
 *  n_pages     pages in the pool (page_len > 0), >= 1; ignored otherwise.
 */
typedef struct ripe_desc {
  int32_t layout;
  int32_t dtype;
  int32_t R;
  int32_t W;
  int32_t batch;
  int32_t t_max;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t n_q_heads;
  int32_t max_rows;
  int32_t max_groups;
  int32_t split_len;
  int32_t page_len;
  int32_t n_pages;
} ripe_desc_t;

/*
 * A draft group: rows [row_start, row_start + n_rows) of q / kv_new / out,
 * belonging to sequence `seq`, verified at loop depth `depth` (1..R).  Row i
 * of a group attends to the sequence's committed prefix (planes per layout)
 * and to rows 0..i of its own group at depth `depth`; it never attends to
 * another group's rows.  Row ranges of the groups of one call must not
 * overlap.
 */
typedef struct ripe_group {
  int32_t seq;
  int32_t depth;
  int32_t row_start;
  int32_t n_rows;
} ripe_group_t;

/*
 * Byte layout of one recurrent layer's cache (E = 4 for F32, 2 for BF16;
 * T = t_max; We = min(W, T)).  The K region comes first, then the V region,
 * with no padding:
 *
 *   FULL     K [B][R][Hkv][T][D]            V [B][R][Hkv][T/8][D][8]
 *   DEEPEST  K [B][Hkv][T][D]               V [B][Hkv][T/8][D][8]
 *   RIPE     K deep [B][Hkv][T][D]          V deep [B][Hkv][T/8][D][8]
 *            then K ring [B][R-1][Hkv][We][D], V ring [B][R-1][Hkv][We*D]
 *
 * Plane p lives at index p-1.  V is stored transposed in blocks of 8
 * positions so that each head dimension's 8 values are contiguous (one
 * 16-byte MFMA operand load for BF16; a commit of a few positions rewrites
 * one or two small blocks).  RIPE keeps planes 1..R-1 of position j in ring
 * slot j mod We; the deep region holds plane R of every position.  The V
 * ring of one (sequence, plane, head) stores its We slots as floor(We/8)
 * blocks [D][8], followed, when We is not a multiple of 8, by one block
 * [D][We mod 8] holding the last slots: V of slot s, head dimension d sits
 * at element
 *   (s/8)*8*D + d*8 + s%8                for s < F = floor(We/8)*8,
 *   F*D + d*(We - F) + (s - F)           otherwise.  Hence the cache costs
 *   FULL    2*B*Hkv*D*E * R*T
 *   DEEPEST 2*B*Hkv*D*E * T
 *   RIPE    2*B*Hkv*D*E * (T + We*(R-1))
 * bytes: one plane plus W*(R-1) window slots per sequence (RIPE abstract,
 * memory statement).
 *
 * Paged caches (page_len = P > 0; the block table of a call maps block k of
 * sequence b, positions [kP, kP + P), to a page of the pool).  The main
 * region (FULL: every plane; DEEPEST and RIPE: the deep plane) becomes a pool
 * of N = n_pages pages, with the same order inside a page:
 *
 *   FULL     K [N][R][Hkv][P][D]            V [N][R][Hkv][P/8][D][8]
 *   DEEPEST  K [N][Hkv][P][D]               V [N][Hkv][P/8][D][8]
 *   RIPE     K pool [N][Hkv][P][D]          V pool [N][Hkv][P/8][D][8]
 *            then the ring exactly as above, one per sequence
 *
 * (K pool, K ring, V pool, V ring), costing 2*Hkv*D*E*(N*P*planes +
 * B*We*(R-1)) bytes.  Sequences may share pages, e.g. two LoopSpec branches
 * forked from one confirmed prefix: they read the shared pages and each
 * keeps its own window ring; a commit must not write a page slot that
 * another sequence of the same call writes.  With P = t_max and block 0 of
 * sequence b on page b, the bytes equal those of the unpaged layout.
 *
 * kind = RIPE_BYTES_CACHE returns the cache size above; kind =
 * RIPE_BYTES_WORKSPACE returns a workspace size sufficient for any verify
 * call within the descriptor's max_rows / max_groups bounds; kind =
 * RIPE_BYTES_POSERR_WORKSPACE one sufficient for any ripe_position_error
 * call within them (with out_f32 and lse left to the library).  Returns a
 * negative ripe_status_t on an invalid descriptor or kind.
 */
int64_t ripe_layout_bytes(const ripe_desc_t* desc, int32_t kind);

/*
 * Verification attention for one recurrent layer (RIPE abstract: the verify
 * pass reads the planes the layout keeps; LoopSpec summary: branches at
 * several depths in one batched call).
 *
 *  desc          cache descriptor (host)
 *  cache         device, ripe_layout_bytes(desc, RIPE_BYTES_CACHE) bytes,
 *                laid out as above
 *  seq_len       host [batch]: committed prefix length T_b, 0 <= T_b <= t_max
 *  groups        host [n_groups] (n_groups == 0 is a no-op)
 *  n_rows        rows of q / kv_new / out (>= every group's row_start+n_rows)
 *  softmax_scale scores are softmax_scale * <q, k>
 *  q             device [n_rows][Hq][D]
 *  kv_new        device [2][R][n_rows][Hkv][D]: K then V of every draft row
 *                at every depth; a group at depth r reads slice [.][r-1]
 *  out           device [n_rows][Hq][D]; written for the rows of the groups
 *  lse           device float [n_rows][Hq], natural-log log-sum-exp of each
 *                row's visible scores; may be NULL
 *  plane_sel     device int8 [n_groups][t_max]: plane (1..R) read by group
 *                g at prefix position j, written for j < T_seq; may be NULL
 *  workspace     device scratch of workspace_bytes bytes (256-byte aligned;
 *                ripe_layout_bytes(desc, RIPE_BYTES_WORKSPACE) suffices).
 *                Its first RIPE_WORKSPACE_ZERO_BYTES bytes must be zero
 *                before the first call that uses it (e.g. allocated with a
 *                zero fill); every call leaves them zero, so a workspace is
 *                zeroed once.  They hold the arrival counters through which
 *                the split-K work items of one launch find the last of them,
 *                which merges the partials.  The rest is clobbered.
 *  stream        hipStream_t (as void*) the kernels are launched on
 *
 * Calls that share a workspace must be ordered on one stream.
 */
#define RIPE_WORKSPACE_ZERO_BYTES 16640
ripe_status_t ripe_verify_attn(const ripe_desc_t* desc, const void* cache, const int32_t* seq_len,
                               const ripe_group_t* groups, int32_t n_groups, int32_t n_rows,
                               float softmax_scale, const void* q, const void* kv_new, void* out,
                               float* lse, int8_t* plane_sel, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * ripe_verify_attn for callers that cannot allocate device memory: code
 * under HIP graph capture, serving loops that must not call the allocator,
 * harnesses that forbid allocation.  Arguments, checks and results are those
 * of ripe_verify_attn, without the workspace: the split partials live in a
 * static device array of RIPE_NOALLOC_SCRATCH_BYTES bytes inside the library
 * (about 32.5 MiB), one copy per GPU, held until the process ends.  The
 * call allocates nothing, with no hipMalloc, hipFree or allocating library
 * routine.  The first call on a device looks up that device's copy
 * (hipGetSymbolAddress, with the device current); a failed lookup returns
 * RIPE_EHIP.  The size covers the largest launch any call makes, so no
 * valid call is refused for scratch.  If a launch needed more, the call
 * would return RIPE_EWORKSPACE before launching anything.
 *
 * Every call on one GPU shares that GPU's array, which keeps the last
 * call's partials; nothing in it needs clearing.  Calls that overlap on one
 * GPU, e.g. on two streams without ordering, race on the array and give
 * undefined results.  Order them on one stream, or use ripe_verify_attn
 * with a workspace each.
 */
#define RIPE_NOALLOC_SCRATCH_BYTES 34095360
ripe_status_t ripe_verify_attn_noalloc(const ripe_desc_t* desc, const void* cache, const int32_t* seq_len,
                                       const ripe_group_t* groups, int32_t n_groups, int32_t n_rows,
                                       float softmax_scale, const void* q, const void* kv_new, void* out,
                                       float* lse, int8_t* plane_sel, void* stream);

/*
 * Verification while each group's parent block is still in flight (LoopSpec
 * summary: the computation of the next position starts from an early draft
 * before the current one is confirmed).  As ripe_verify_attn, with
 *
 *  parents   host int32 [n_groups][2]: (row_start, n_rows) of the group's
 *            parent block in q / kv_new; n_rows = 0 means none.  The parent's
 *            rows are the n_rows positions that follow the committed prefix
 *            (T_b .. T_b + n_rows - 1); the group's own rows follow them.
 *            All groups of one sequence name the same parent
 *            (RIPE_EUNSUPPORTED otherwise); rows must lie in [0, n_rows)
 *            (RIPE_ERANGE).
 *
 * Every position is read as it will be once the parent is committed, so the
 * result equals committing the parent first and verifying then: the RIPE
 * window is the last W positions of T_b + n_rows(parent), committed
 * positions before it are read at plane R, and each parent row is read from
 * kv_new at the plane that rule gives it (FULL: the group's depth r;
 * DEEPEST: R; RIPE: r inside the window, R before it).  Every parent row is
 * visible to every row of the group.  plane_sel covers the committed
 * positions only.
 */
ripe_status_t ripe_verify_attn_inflight(const ripe_desc_t* desc, const void* cache, const int32_t* seq_len,
                                        const ripe_group_t* groups, const int32_t* parents, int32_t n_groups,
                                        int32_t n_rows, float softmax_scale, const void* q, const void* kv_new,
                                        void* out, float* lse, int8_t* plane_sel, void* workspace,
                                        size_t workspace_bytes, void* stream);

/*
 * Commit accepted draft rows (RIPE abstract, sentence introducing RIPE: the
 * W most recent positions hold every plane, older ones only the last;
 * LoopSpec summary: rejected continuations are dropped and decoding resumes
 * from the confirmed prefix).
 *
 * For every sequence b with n_accept[b] > 0, draft rows src_row[b] ..
 * src_row[b] + n_accept[b] - 1 of kv_new become positions T_b ..
 * T_b + n_accept[b] - 1, where T_b = seq_len[b]:
 *   FULL     planes 1..R are written;
 *   DEEPEST  plane R is written;
 *   RIPE     plane R is written to the deep region, and planes 1..R-1 of the
 *            positions that are within the new window (j >= T_b + n - We)
 *            are written to ring slot j mod We.  A position leaving the
 *            window needs no copy: its plane R is already in the deep region
 *            and its ring slot is taken over by the position W later.
 * Then seq_len[b] += n_accept[b] (host).  n_accept[b] == 0 leaves sequence b
 * untouched (rollback to the confirmed prefix).
 *
 *  desc       cache descriptor (host)
 *  cache      device, laid out as above (written)
 *  seq_len    host [batch], in/out; T_b + n_accept[b] <= t_max or RIPE_ECAPACITY
 *  n_accept   host [batch], >= 0
 *  src_row    host [batch]; rows src_row[b] + n_accept[b] <= n_rows (ignored
 *             when n_accept[b] == 0)
 *  kv_new     device [2][R][n_rows][Hkv][D] (same layout as for verify)
 *  n_rows     rows of kv_new
 *  stream     hipStream_t (as void*)
 */
ripe_status_t ripe_commit(const ripe_desc_t* desc, void* cache, int32_t* seq_len,
                          const int32_t* n_accept, const int32_t* src_row, const void* kv_new,
                          int32_t n_rows, void* stream);

/*
 * Paged caches (desc->page_len > 0; the calls above return RIPE_EINVAL for
 * such a descriptor, these two RIPE_EINVAL for an unpaged one).  They do what
 * ripe_verify_attn_inflight (parents may be NULL: no parent in flight) and
 * ripe_commit do, reading and writing position j of sequence b in page
 * block_table[b * (t_max / page_len) + j / page_len] at slot j mod page_len.
 *
 *  block_table  host int32 [batch][t_max / page_len].  Verify reads the
 *               entries of blocks holding positions < T_b of every sequence
 *               with groups; commit those of the blocks it writes.  Such an
 *               entry outside [0, n_pages) is RIPE_ERANGE; other entries are
 *               not read.
 *
 * Pages shorter than the split length (desc->split_len, or the library's
 * default): verify uses the unpaged call's work plan and reads each
 * 32-position step from its page, so results are bit-identical to the
 * unpaged call's.  Pages of at least the split length: prefix pieces are
 * cut at page boundaries, so each lies in one page (results equal the
 * unpaged call's where the cut points coincide, e.g. P = t_max).
 * A commit in which two sequences write one (page, slot) is RIPE_EINVAL.
 * The RIPE ring is per sequence and unpaged.  A launch carries the page
 * numbers its pieces read in its kernel arguments: at most 512 pages beyond
 * the first page of each piece, summed over the launch's pieces.  A
 * sequence needing more on its own (pages shorter than the split length and
 * a prefix of about 512 * page_len positions or more) is RIPE_EUNSUPPORTED.
 */
ripe_status_t ripe_verify_attn_paged(const ripe_desc_t* desc, const void* cache, const int32_t* block_table,
                                     const int32_t* seq_len, const ripe_group_t* groups, const int32_t* parents,
                                     int32_t n_groups, int32_t n_rows, float softmax_scale, const void* q,
                                     const void* kv_new, void* out, float* lse, int8_t* plane_sel,
                                     void* workspace, size_t workspace_bytes, void* stream);

ripe_status_t ripe_commit_paged(const ripe_desc_t* desc, void* cache, const int32_t* block_table,
                                int32_t* seq_len, const int32_t* n_accept, const int32_t* src_row,
                                const void* kv_new, int32_t n_rows, void* stream);

/*
 * Accept / rollback after verification (LoopSpec summary, rit.work blog,
 * section on the second branch; RIPE abstract, zhuanzhiai.com paper page: the
 * target distributions come from the verify pass at depth R).
 *
 * Per sequence b there is a primary chain of k draft tokens and, when
 * has_fallback[b] != 0, a fallback chain of k tokens that replaces the
 * primary from position 0 (an alternative first token drawn from the deeper
 * state's distribution after the first proposal is taken out, followed by
 * its own continuation).  The rows:
 *
 *  target_logits device float [batch][2][k+1][vocab]: row [b][c][i] gives
 *                the target distribution softmax(z / temperature) of position
 *                i of chain c (c = 0 primary, 1 fallback); row k scores the
 *                bonus position after a fully accepted chain.  Position 0 of
 *                both chains follows the same committed prefix, so the
 *                fallback's row 0 is not read.
 *  draft_logits  device float [batch][2][k][vocab]: row [b][0][i] is the
 *                distribution q_i the primary's token i was drawn from; row
 *                [b][1][0] is the deeper state's distribution m (the fallback's
 *                first token was drawn from q' = norm(max(0, m - q_0))), rows
 *                [b][1][i >= 1] are the fallback's draft distributions.  Not
 *                read when temperature == 0.
 *  tokens        device int32 [batch][2][k]: the drafted tokens; a token
 *                outside [0, vocab) is never accepted
 *  has_fallback  device uint8 [batch]
 *  rand          device uint32 [batch][2k+1]: random words, u = word / 2^32;
 *                word i for the primary's test i, word k for the fallback's
 *                first test, word k+i for the fallback's test i >= 1, word 2k
 *                for the final draw.  Not read when temperature == 0.
 *  n_accept, branch, next_token   device int32 [batch], written: tokens kept,
 *                the chain they come from (0 when none are kept), and the
 *                token that follows them (a correction, or a bonus token
 *                after a fully accepted chain).  With the verify call's
 *                groups, n_accept and the kept chain's first row are the
 *                n_accept / src_row of ripe_commit.
 *  workspace     device, ripe_accept_workspace_bytes(desc) bytes, 256-byte
 *                aligned; contents need no initialisation and are clobbered
 *
 * Rules (the scheme in full; all arithmetic in double):
 *  - temperature == 0 (greedy): a token is accepted iff it is the arg max of
 *    its target row (lowest index on ties).  The primary chain is checked in
 *    order; if its first token is rejected and a fallback exists, the
 *    fallback's first token is checked against the primary's row 0 and, if
 *    accepted, the fallback chain continues.  The next token is the arg max
 *    of the target row at the position where the kept chain stopped (row 0
 *    of the primary when nothing is kept).
 *  - temperature > 0 (speculative sampling): token t of a row is accepted iff
 *    u * q(t) < p(t), i.e. with probability min(1, p(t)/q(t)).  At the
 *    primary's first rejection j, with no fallback or j > 0, n = j and the
 *    next token is drawn from max(0, p_j - q_j).  At j = 0 with a fallback,
 *    the fallback's first token y is tested against the residual target
 *    r = norm(max(0, p_0 - q_0)) with q': u * q'(y) < r(y); if accepted the
 *    fallback chain continues with the ordinary test (rejection at j':
 *    draw from max(0, p'_j' - q'_j')); if rejected, n = 0 and the next token
 *    is drawn from max(0, r - q') (restart after two rejections).  A fully
 *    accepted chain draws its bonus token from its row k.  A draw from
 *    weights w takes the first index whose running sum exceeds u * sum(w),
 *    or the last index with w > 0 if rounding leaves none; a residual with
 *    no mass is replaced by the row's target distribution (r after a
 *    restart).  Sampling this way keeps each output token's probability
 *    under ordinary decoding.
 *
 * desc->batch >= 0 (0 is a no-op), 1 <= k <= 64, 1 <= vocab <= 2^24,
 * temperature finite and >= 0.  Every row needs at least one finite logit.
 */
typedef struct ripe_accept_desc {
  int32_t batch;
  int32_t k;
  int32_t vocab;
  float temperature;
} ripe_accept_desc_t;

/* Workspace bytes of ripe_accept, or a negative ripe_status_t for an invalid
 * descriptor. */
int64_t ripe_accept_workspace_bytes(const ripe_accept_desc_t* desc);

ripe_status_t ripe_accept(const ripe_accept_desc_t* desc, const float* target_logits,
                          const float* draft_logits, const int32_t* tokens, const uint8_t* has_fallback,
                          const uint32_t* rand, int32_t* n_accept, int32_t* branch, int32_t* next_token,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * ripe_position_error -- side statistic: how much each committed prefix
 * position contributes to the error of storing only the deepest plane.
 *
 * Source: RIPE abstract (zhuanzhiai.com paper page): whether the deepest
 * plane alone suffices depends on how close the late planes are to it; on
 * one model a small set of positions (1%) carries most of its error, and a
 * window of recent positions at full depth removes most of those tail
 * positions.  The pages name this error without defining it; here it is:
 * for group g (sequence b, depth r, rows [row_start, row_start + n_rows)),
 *
 *   err[g][j] = sum over the group's rows and query heads of
 *               || O^(j) - O ||^2,      j < T_b,
 *
 * O being the verify output over the FULL cache (every prefix position at
 * plane r, the group's own rows at depth r, as ripe_verify_attn computes it)
 * and O^(j) the same output with prefix position j alone read at plane R.
 * It is computed from the single-term softmax update, in fp32.  Summed over
 * j it is the first-order estimate of the DEEPEST output's squared error;
 * the sum over j < T_b - W that of RIPE with window W.
 *
 * The update's sensitivity to the FULL output and LSE it starts from is
 * kappa = a / (1 - a + c), a and c being position j's softmax weights at
 * planes r and R in a row.  kappa <= 1 unless position j holds more than half
 * of some row's attention at plane r; there the fp32 result has a relative
 * error up to about kappa times that of the FULL output (1e-4 .. 1e-3 for
 * bf16 caches) and is an estimate only.  cond reports kappa per position.
 *
 *  desc       a FULL descriptor (RIPE_EUNSUPPORTED otherwise); max_rows /
 *             max_groups size RIPE_BYTES_POSERR_WORKSPACE.
 *  cache ... kv_new   as for ripe_verify_attn (plane_sel is not produced).
 *  err        device float [n_groups][t_max]; entries j >= T_b are set to 0.
 *  cond       optional device float [n_groups][t_max]: kappa of each
 *             position, the largest over the group's rows and heads (0 for
 *             j >= T_b); NULL: not written.
 *  out_f32    optional device float [n_rows][Hq][D]: receives the FULL
 *             outputs in fp32 (rows no group covers are not written);
 *             NULL: kept in the workspace.
 *  lse        optional device float [n_rows][Hq]: their natural-log LSE.
 *  workspace  device, 256-byte aligned; at least
 *             ripe_layout_bytes(desc, RIPE_BYTES_POSERR_WORKSPACE) bytes
 *             (RIPE_EWORKSPACE if smaller than the call needs).  Scratch
 *             owned by the caller; zero-filled before its first use (it
 *             holds a verify workspace, whose counters must start at zero),
 *             and every call leaves those counters zero.
 *
 * Validation and errors as for ripe_verify_attn; err, cond and lse must be
 * 4-byte aligned, out_f32 16-byte aligned.  Asynchronous on stream; launches kernels only.
 */
ripe_status_t ripe_position_error(const ripe_desc_t* desc, const void* cache, const int32_t* seq_len,
                                  const ripe_group_t* groups, int32_t n_groups, int32_t n_rows,
                                  float softmax_scale, const void* q, const void* kv_new, float* err,
                                  float* cond, float* out_f32, float* lse, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * ripe_position_error_tail -- the two tail figures of the error rows that
 * ripe_position_error writes, per row.
 *
 * Source: RIPE abstract (zhuanzhiai.com paper page), the sentences on the
 * error's tail: a small share of positions (1%) carries most of the error of
 * the deepest-only cache, and a window of recent positions at full depth
 * removes most of those tail positions.  Read per row (one group) as: the
 * tail is the n = max(1, floor(tail_frac * T)) largest e_j (n = 0 when
 * T = 0), ties going to the lower position; its share of sum_j e_j; the
 * fraction of its positions among the last W; and the share of sum_j e_j
 * that the last W positions carry.
 *
 *  err        device float [n_rows][row_stride]: e_j >= 0 (finite), entries
 *             at j >= T[i] ignored; e.g. ripe_position_error's err with
 *             row_stride = t_max.
 *  cond       optional device float [n_rows][row_stride] (its cond): counts
 *             the positions with cond > 1 (ill-conditioned e_j) and their
 *             share; NULL: those outputs are NaN.
 *  T          host int32 [n_rows]: prefix length of each row, 0..row_stride
 *             (RIPE_ERANGE otherwise).
 *  window     W >= 0.
 *  tail_frac  in (0, 1] (0.01 for the pages' 1%).
 *  stats      device double [n_rows][RIPE_TAIL_STATS], 8-byte aligned:
 *             [0] n, [1] tail share, [2] fraction of the tail positions in
 *             the last W, [3] share of the last W positions, [4] positions
 *             with cond > 1, [5] their share, [6] sum_j e_j, [7] T.  Shares
 *             are NaN when sum_j e_j = 0, [2] when n = 0.
 *
 * Sums are in double over the float inputs.  RIPE_EINVAL for null or
 * misaligned pointers, n_rows < 0, row_stride < 0, W < 0 or tail_frac
 * outside (0, 1].  Asynchronous on stream; launches kernels only.
 */
#define RIPE_TAIL_STATS 8
ripe_status_t ripe_position_error_tail(const float* err, const float* cond, const int32_t* T, int32_t n_rows,
                                       int32_t row_stride, int32_t window, double tail_frac, double* stats,
                                       void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RIPE_H_ */
