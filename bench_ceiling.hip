// bench_ceiling.hip -- streaming-read ceiling of the MI355X for the verify kernel's
// access shape, as a reference for the roofline fraction bench.py reports.
//
// read_kv: each work-group streams one K chunk and one V chunk in 8 KiB steps,
// wavefront w taking steps w, w + 4, ...; the K loads follow the verify
// kernel's MFMA operand pattern (16 rows x 64 bytes per instruction) and the
// V loads read 1 KiB contiguous per instruction.  No arithmetic beyond an
// xor that keeps the loads alive.  Each call reads 200 MiB (100 MiB K +
// 100 MiB V), the size of one c3 verify call.  "rotating" calls walk four
// 256 MiB regions, so the 256 MB last-level cache cannot hold the working
// set (as in bench.py, which rotates four recurrent layers); "same region"
// re-reads one region and is cache-assisted.  read_gs: a grid-stride read of
// 1 GiB.
//
// Build and run:
//   hipcc --offload-arch=gfx950 -O3 -Xclang -target-feature -Xclang -packed-fp32-ops \
//         -o bench_ceiling bench_ceiling.hip && ./bench_ceiling
#include <hip/hip_runtime.h>
#include <cstdio>
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#define CHECK(x) do { hipError_t e = (x); if (e != hipSuccess) { printf("HIP error %s line %d\n", hipGetErrorString(e), __LINE__); return 1; } } while (0)
__device__ inline __amdgpu_buffer_rsrc_t mk(const void* b, uint32_t n) { return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(b), 0, n, 0x00020000); }
// per work-group: K chunk and V chunk (each `chunk` bytes) streamed in 8 KB steps per wave (w, w+4, ...)
__global__ __launch_bounds__(256) void read_kv(const uint8_t* __restrict__ A, const uint8_t* __restrict__ Bv, uint32_t chunk, uint32_t* out) {
  const uint8_t* ka = A + size_t(blockIdx.x) * chunk;
  const uint8_t* va = Bv + size_t(blockIdx.x) * chunk;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, ln = lane & 15, lg = lane >> 4;
  auto kr = mk(ka, chunk); auto vr = mk(va, chunk);
  u32x4 acc = {0, 0, 0, 0};
  for (uint32_t st = wave; st * 8192 < chunk; st += 4) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int pos = 8 * (ln >> 2) + 4 * mb + (ln & 3);
        acc ^= __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(kr, st * 8192 + pos * 256 + c * 64 + lg * 16, 0, 0));
      }
#pragma unroll
    for (int db = 0; db < 8; ++db)
      acc ^= __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vr, st * 8192 + db * 1024 + lane * 16, 0, 0));
  }
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x12345678u) out[0] = 1;
}
__global__ void read_gs(const u32x4* __restrict__ p, size_t n16, uint32_t* out) {
  u32x4 acc = {0, 0, 0, 0};
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x) acc ^= p[i];
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x12345678u) out[0] = 1;
}
int main() {
  const size_t region = size_t(256) << 20;  // 4 regions of 256 MiB: 1 GiB rotation
  uint8_t* buf; uint32_t* out;
  CHECK(hipMalloc(&buf, 4 * region)); CHECK(hipMalloc(&out, 4));
  CHECK(hipMemset(buf, 1, 4 * region));
  hipEvent_t a, b; CHECK(hipEventCreate(&a)); CHECK(hipEventCreate(&b));
  float ms;
  // each call reads K 100 MiB + V 100 MiB from one region; 4 regions rotate
  for (uint32_t chunk : {128u << 10, 256u << 10, 512u << 10}) {
    const int grid = int((size_t(100) << 20) / chunk);
    for (int warm = 0; warm < 8; ++warm) hipLaunchKernelGGL(read_kv, dim3(grid), dim3(256), 0, 0, buf + (warm % 4) * region, buf + (warm % 4) * region + (size_t(128) << 20), chunk, out);
    CHECK(hipDeviceSynchronize());
    const int n = 40;
    CHECK(hipEventRecord(a));
    for (int i = 0; i < n; ++i) hipLaunchKernelGGL(read_kv, dim3(grid), dim3(256), 0, 0, buf + (i % 4) * region, buf + (i % 4) * region + (size_t(128) << 20), chunk, out);
    CHECK(hipEventRecord(b)); CHECK(hipEventSynchronize(b)); CHECK(hipEventElapsedTime(&ms, a, b));
    const double bytes = 2.0 * grid * chunk;
    printf("[ceiling] read_kv rotating 4x256MiB, chunk %u KiB, grid %d: %.1f us per 200 MiB call, %.1f GB/s\n", chunk >> 10, grid, ms * 1e3 / n, bytes * n / (ms * 1e-3) / 1e9);
    // same region every call (cache-warm when it fits)
    CHECK(hipEventRecord(a));
    for (int i = 0; i < n; ++i) hipLaunchKernelGGL(read_kv, dim3(grid), dim3(256), 0, 0, buf, buf + (size_t(128) << 20), chunk, out);
    CHECK(hipEventRecord(b)); CHECK(hipEventSynchronize(b)); CHECK(hipEventElapsedTime(&ms, a, b));
    printf("[ceiling] read_kv same region,        chunk %u KiB, grid %d: %.1f us per call, %.1f GB/s\n", chunk >> 10, grid, ms * 1e3 / n, bytes * n / (ms * 1e-3) / 1e9);
  }
  for (int grid : {2048, 8192}) {
    const size_t n16 = (size_t(1) << 30) / 16;
    hipLaunchKernelGGL(read_gs, dim3(grid), dim3(256), 0, 0, (const u32x4*)buf, n16, out);
    CHECK(hipEventRecord(a));
    for (int i = 0; i < 5; ++i) hipLaunchKernelGGL(read_gs, dim3(grid), dim3(256), 0, 0, (const u32x4*)buf, n16, out);
    CHECK(hipEventRecord(b)); CHECK(hipEventSynchronize(b)); CHECK(hipEventElapsedTime(&ms, a, b));
    printf("[ceiling] read_gs 1 GiB grid %d: %.1f GB/s\n", grid, 5.0 * (size_t(1) << 30) / (ms * 1e-3) / 1e9);
  }
  return 0;
}
