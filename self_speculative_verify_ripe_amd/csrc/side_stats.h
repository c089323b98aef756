// side_stats.h -- launch record of the per-position substitution-error
// kernels (shared by the host entry point and the kernels).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ripe {

constexpr int kPeGroups = 128;  // groups per launch
constexpr int kPeTile = 32;     // prefix positions per work-group (one V block)
constexpr int kPeCols = 16;     // query columns staged in LDS at a time

struct PeGroup {       // one group (16 bytes)
  int32_t row_start;   // first query row
  int32_t n_rows;      // its rows
  int32_t T;           // committed prefix length of its sequence
  uint16_t b;          // sequence
  uint16_t depth;      // depth r (1-based)
};

struct PosErrParams {
  const void* cache_k;  // FULL K region [B][R][Hkv][t_max][D]
  const void* cache_v;  // FULL V region [B][R][Hkv][t_max/8][D][8]
  const void* q;        // [n_rows][Hq][D], storage dtype
  const float* o;       // FULL output at the group's depth, [n_rows][Hq][D] fp32
  const float* lse;     // its natural-log LSE, [n_rows][Hq]
  float* part;          // per KV head sums, [n_groups][Hkv][t_max]
  float* part_cond;     // per KV head condition numbers, [n_groups][Hkv][t_max]
  float* err;           // result, [n_groups][t_max]
  float* cond;          // max over KV heads of part_cond, [n_groups][t_max] (optional)
  int32_t R, H, Hq, G, t_max;
  int32_t g0;           // index of grp[0] among the call's groups
  int32_t n_grp;        // groups in this launch
  float scale;          // softmax scale
  PeGroup grp[kPeGroups];
};

hipError_t launch_position_error(const PosErrParams& p, int dtype, int D, hipStream_t stream);

// Tail summary of error rows: one work-group per row.
constexpr int kTailRows = 512;   // rows per launch
constexpr int kTailStats = 8;    // doubles per row

struct TailParams {
  const float* err;     // [rows][stride]
  const float* cond;    // [rows][stride] or null
  double* stats;        // [rows][kTailStats]
  int32_t stride;
  int32_t window;       // W: the last W positions of each row's prefix
  int32_t g0;           // index of the launch's first row among the call's rows
  int32_t n_rows;       // rows in this launch
  int32_t T[kTailRows];       // prefix length of each row
  int32_t n_tail[kTailRows];  // tail positions of each row
};

hipError_t launch_position_error_tail(const TailParams& p, hipStream_t stream);

}  // namespace ripe
