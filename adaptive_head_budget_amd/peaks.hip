// Measured peaks of the MI355X this runs on, next to the published ones the
// rooflines use (dense bf16 MFMA 2.5 PFLOP/s, HBM 8 TB/s):
//   * dense bf16 MFMA: every SIMD runs independent v_mfma_f32_16x16x32_bf16
//     chains (two waves per SIMD, eight accumulators each), with the shader
//     clock read from s_memtime against the 100 MHz s_memrealtime;
//   * HBM read: 1 GiB streamed with 16-byte nontemporal loads;
//   * HBM copy: 1 GiB copied with 16-byte nontemporal loads and stores
//     (read + write bytes counted).
// Prints one JSON object.  Nothing here is part of the eviction path.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define CHECK(x)                                                              \
  do {                                                                        \
    hipError_t e_ = (x);                                                      \
    if (e_ != hipSuccess) {                                                   \
      fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));                 \
      return 1;                                                               \
    }                                                                         \
  } while (0)

__global__ __launch_bounds__(512) void mfma_peak(float* out, uint64_t* clk, int iters, float s) {
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(threadIdx.x * 1e-3f + i);
    b[i] = (__bf16)(s + i);
  }
  f32x4 acc[8];
  for (int i = 0; i < 8; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[i], 0, 0, 0);
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  float t = 0.f;
  for (int i = 0; i < 8; ++i) t += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
  out[blockIdx.x * blockDim.x + threadIdx.x] = t;
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    clk[0] = t1 - t0;
    clk[1] = r1 - r0;
  }
}

__global__ __launch_bounds__(256) void read_peak(const u32x4* __restrict__ a, u32x4* __restrict__ out, size_t n16) {
  const size_t stride = (size_t)gridDim.x * 256 * 8;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (size_t base = (size_t)blockIdx.x * 256 * 8 + threadIdx.x; base < n16; base += stride) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const size_t i = base + (size_t)u * 256;
      if (i < n16) acc += __builtin_nontemporal_load(a + i);
    }
  }
  if (acc.x == 0x9E3779B9u && acc.y == 0x7F4A7C15u) out[threadIdx.x] = acc;   // keeps the loads
}

__global__ __launch_bounds__(256) void copy_peak(const u32x4* __restrict__ a, u32x4* __restrict__ b, size_t n16) {
  const size_t stride = (size_t)gridDim.x * 256 * 4;
  for (size_t base = (size_t)blockIdx.x * 256 * 4 + threadIdx.x; base < n16; base += stride) {
    u32x4 x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const size_t i = base + (size_t)u * 256;
      if (i < n16) x[u] = __builtin_nontemporal_load(a + i);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const size_t i = base + (size_t)u * 256;
      if (i < n16) __builtin_nontemporal_store(x[u], b + i);
    }
  }
}

}  // namespace

int main() {
  int dev = 0, cus = 0;
  CHECK(hipGetDevice(&dev));
  CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));

  // MFMA: one 512-thread workgroup per CU (two waves per SIMD)
  const int blocks = cus, threads = 512, iters = 20000;
  float* out = nullptr;
  uint64_t* clk = nullptr;
  CHECK(hipMalloc(&out, sizeof(float) * blocks * threads));
  CHECK(hipMalloc(&clk, 2 * sizeof(uint64_t)));
  mfma_peak<<<blocks, threads>>>(out, clk, iters / 10, 0.999f);   // warm-up
  CHECK(hipEventRecord(e0));
  mfma_peak<<<blocks, threads>>>(out, clk, iters, 0.999f);
  CHECK(hipEventRecord(e1));
  CHECK(hipEventSynchronize(e1));
  float ms = 0.f;
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  uint64_t h[2];
  CHECK(hipMemcpy(h, clk, sizeof(h), hipMemcpyDeviceToHost));
  const double flops = 2.0 * 16 * 16 * 32 * 8.0 * iters * (threads / 64) * (double)blocks;
  const double mfma_pf = flops / (ms * 1e-3) / 1e15;
  const double ghz = (double)h[0] / ((double)h[1] * 10.0);   // s_memrealtime counts at 100 MHz

  // HBM: 1 GiB read, 1 GiB copy
  const size_t bytes = (size_t)1 << 30, n16 = bytes / 16;
  u32x4 *a = nullptr, *b = nullptr;
  CHECK(hipMalloc(&a, bytes));
  CHECK(hipMalloc(&b, bytes));
  CHECK(hipMemset(a, 1, bytes));
  CHECK(hipMemset(b, 0, bytes));
  auto time5 = [&](auto launch) -> float {
    launch();
    (void)hipEventRecord(e0);
    for (int i = 0; i < 5; ++i) launch();
    (void)hipEventRecord(e1);
    (void)hipEventSynchronize(e1);
    float t = 0.f;
    (void)hipEventElapsedTime(&t, e0, e1);
    return t / 5;
  };
  const float tr = time5([&] { read_peak<<<8 * cus, 256>>>(a, b, n16); });
  const float tc = time5([&] { copy_peak<<<64 * cus, 256>>>(a, b, n16); });
  CHECK(hipGetLastError());
  printf("{\"mfma_bf16_dense_pflops\": %.4f, \"mfma_shader_clock_ghz\": %.3f, \"hbm_read_gbs\": %.1f, "
         "\"hbm_copy_gbs\": %.1f, \"cus\": %d}\n",
         mfma_pf, ghz, bytes / (tr * 1e-3) / 1e9, 2.0 * bytes / (tc * 1e-3) / 1e9, cus);
  return 0;
}
