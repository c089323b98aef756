// accept.h -- launch record and workspace layout of the accept / rollback
// kernels, shared by the host entry point and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ripe {

constexpr int kAcceptTile = 64;        // vocabulary indices per tile of a draw
constexpr int kAcceptSliceMin = 4096;  // at least this many indices per work-group slice
constexpr int kAcceptMaxSplit = 64;    // slices per row at most
constexpr int kPartsPerSlice = 4;      // parts per slice of the per-sequence sweeps (residual masses, draw weights)

struct RowStat {
  double S;     // sum over the row (or a slice of it) of exp((z - M) * inv_tau)
  float M;      // max logit
  int32_t arg;  // arg max, lowest index on ties
};

// Per-sequence progress between the launches (128 bytes).  It carries the
// statistics of the rows a, c, m it names, so that the launches that follow
// need not look them up before their first logit load.
struct SeqState {
  int32_t stage;      // kStageDone / kStageFallback / kStageDraw
  int32_t kind;       // what the final draw draws from (see accept.hip)
  int32_t ra, rc, rm; // rows of the distributions a, c, m of that draw
  int32_t n, branch;  // tokens kept and their chain
  int32_t pad;
  double Wr, Wm;      // the fallback's residual masses
  double u;           // uniform of the final draw
  double S[3];        // sums of rows ra, rc, rm (RowStat::S)
  float M[3];         // their max logits
  int32_t pad2[9];
};
static_assert(sizeof(SeqState) == 128, "SeqState layout");

struct AcceptParams {
  const float* target;     // [B][2][k+1][V]
  const float* draft;      // [B][2][k][V]
  const int32_t* tokens;   // [B][2][k]
  const uint8_t* has_fb;   // [B]
  const uint32_t* rand;    // [B][2k+1]
  int32_t* n_accept;       // [B]
  int32_t* branch;         // [B]
  int32_t* next_token;     // [B]
  // workspace
  RowStat* part;           // [B][4k+2][split]: per-slice statistics
  RowStat* stats;          // [B][4k+2]
  SeqState* state;         // [2B]: after the primary chain's tests; [B + b]: after a fallback's
  double* sums;            // [B][split * kPartsPerSlice][2]: residual masses per part
  double* tiles;           // [B][n_tiles]: tile sums of the final draw's weights
  int32_t* last;           // [B][split * kPartsPerSlice]: last index with weight > 0 per part
  double* ptot;            // [B][split * kPartsPerSlice]: each part's total weight (its tile sums
                           // added in tile order)
  int32_t B, k, V;
  int32_t greedy;          // temperature == 0
  double inv_tau;          // 1 / temperature
  int32_t split, slice, n_tiles;
};

struct AcceptLayout {
  int32_t split, slice, n_tiles;
  int64_t off_part, off_stats, off_state, off_sums, off_tiles, off_last, off_ptot, bytes;
};

inline int64_t accept_align(int64_t x) { return (x + 255) / 256 * 256; }

// Slices per row and workspace regions (each 256-byte aligned).
inline AcceptLayout accept_layout(int64_t B, int64_t k, int64_t V) {
  AcceptLayout L;
  int64_t split = (V + kAcceptSliceMin - 1) / kAcceptSliceMin;
  split = split < 1 ? 1 : (split > kAcceptMaxSplit ? kAcceptMaxSplit : split);
  int64_t slice = (V + split - 1) / split;
  slice = (slice + kAcceptTile - 1) / kAcceptTile * kAcceptTile;
  L.split = int32_t(split);
  L.slice = int32_t(slice);
  L.n_tiles = int32_t((V + kAcceptTile - 1) / kAcceptTile);
  const int64_t rows = 4 * k + 2;
  int64_t off = 0;
  L.off_part = off;  off += accept_align(B * rows * split * int64_t(sizeof(RowStat)));
  L.off_stats = off; off += accept_align(B * rows * int64_t(sizeof(RowStat)));
  L.off_state = off; off += accept_align(2 * B * int64_t(sizeof(SeqState)));
  L.off_sums = off;  off += accept_align(B * split * kPartsPerSlice * 2 * int64_t(sizeof(double)));
  L.off_tiles = off; off += accept_align(B * L.n_tiles * int64_t(sizeof(double)));
  L.off_last = off;  off += accept_align(B * split * kPartsPerSlice * int64_t(sizeof(int32_t)));
  L.off_ptot = off;  off += accept_align(B * split * kPartsPerSlice * int64_t(sizeof(double)));
  L.bytes = off;
  return L;
}

hipError_t launch_accept(const AcceptParams& p, hipStream_t stream);

}  // namespace ripe
