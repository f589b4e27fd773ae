// Measured ceilings of the device the attention kernels run on (one JSON line on stdout):
//  * bf16 MFMA: v_mfma_f32_32x32x16_bf16 in four independent chains per wave, 2 waves per
//    SIMD, registers only -- the matrix-core rate the prefill kernels are compared with;
//  * the shader clock during that loop, from the shader cycle counter (s_memtime) against the
//    constant 100 MHz real-time counter (s_memrealtime);
//  * HBM streaming read: 2 GiB read once with 16-byte non-temporal loads;
//  * HBM random gather: 2 KB chunks of a 1 GiB buffer in a seeded random order (the pattern a
//    paged KV cache with a permuted block table imposes), after a read of another 1 GiB buffer
//    that evicts the caches.
// Used by bench.py as the "measured" denominators next to the published peaks.
#include <hip/hip_runtime.h>
#include <cstdint>
#include <cstdio>
#include <vector>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define CHECK(x)                                                                          \
  do {                                                                                    \
    hipError_t e_ = (x);                                                                  \
    if (e_ != hipSuccess) {                                                               \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));                      \
      return 1;                                                                           \
    }                                                                                     \
  } while (0)

// clk[0..1]: s_memtime and s_memrealtime at the start of workgroup 0, clk[2..3] at its end
__global__ __launch_bounds__(256) void mfma_loop(float* out, uint64_t* clk, int iters) {
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    clk[0] = __builtin_amdgcn_s_memtime();
    clk[1] = __builtin_amdgcn_s_memrealtime();
  }
  bf16x8 a, b;
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * (threadIdx.x + e));
    b[e] = (__bf16)(0.002f * e);
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  if (s == 12345.f) out[threadIdx.x] = s;  // never true; keeps the chains live
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    clk[2] = __builtin_amdgcn_s_memtime();
    clk[3] = __builtin_amdgcn_s_memrealtime();
  }
}

// every 16-byte word of in[0, n16) read once, 8 loads in flight per lane
__global__ __launch_bounds__(256) void stream_read(const u32x4* __restrict__ in, uint32_t* out,
                                                   int64_t n16) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i + 7 * stride < n16;
       i += 8 * stride) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(in + i + u * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u];
  }
  if (acc[0] == 12345u && acc[1] == 7u) out[threadIdx.x] = acc[2];
}

// one wave per run of chunks: chunk order[c] (2 KB each), 4 chunks in flight per wave
__global__ __launch_bounds__(256) void gather_read(const char* __restrict__ src,
                                                   const int32_t* __restrict__ order, int n,
                                                   uint32_t* out) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6), nw = gridDim.x * 4;
  const int per = (n + nw - 1) / nw;
  const int lo = wave * per, hi = min(n, lo + per);
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int c0 = lo; c0 < hi; c0 += 4) {
    u32x4 v[4][2];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = min(c0 + k, hi - 1);
      const char* p = src + (int64_t)order[c] * 2048 + 16 * lane;
      v[k][0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
      v[k][1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + 1024));
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) acc ^= v[k][0] ^ v[k][1];
  }
  if (acc[0] == 12345u && acc[1] == 7u) out[threadIdx.x] = acc[2];
}

int main() {
  int dev = 0, cus = 0;
  CHECK(hipGetDevice(&dev));
  CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
  float* fout;
  uint32_t* uout;
  uint64_t* clk;
  CHECK(hipMalloc(&fout, 4096));
  CHECK(hipMalloc(&uout, 4096));
  CHECK(hipMalloc(&clk, 64));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  float ms = 0.f;

  // ---- MFMA ---------------------------------------------------------------------------------
  const int mfma_grid = cus * 2, iters = 20000;  // 2 workgroups of 4 waves per CU
  hipLaunchKernelGGL(mfma_loop, dim3(mfma_grid), dim3(256), 0, 0, fout, clk, 100);
  CHECK(hipDeviceSynchronize());
  CHECK(hipEventRecord(e0));
  hipLaunchKernelGGL(mfma_loop, dim3(mfma_grid), dim3(256), 0, 0, fout, clk, iters);
  CHECK(hipEventRecord(e1));
  CHECK(hipEventSynchronize(e1));
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  const double mfma_flops = (double)mfma_grid * 4 * iters * 4 * (32.0 * 32 * 16 * 2);
  const double mfma_tflops = mfma_flops / (ms * 1e-3) / 1e12;
  uint64_t h_clk[4];
  CHECK(hipMemcpy(h_clk, clk, sizeof(h_clk), hipMemcpyDeviceToHost));
  const double sclk_mhz =
      h_clk[3] > h_clk[1] ? (double)(h_clk[2] - h_clk[0]) / (double)(h_clk[3] - h_clk[1]) * 100.0 : 0.0;

  // ---- HBM streaming read -------------------------------------------------------------------
  const int64_t sbytes = 2LL << 30;
  u32x4* sbuf;
  CHECK(hipMalloc(&sbuf, sbytes));
  CHECK(hipMemset(sbuf, 1, sbytes));
  const int sgrid = cus * 16;
  hipLaunchKernelGGL(stream_read, dim3(sgrid), dim3(256), 0, 0, sbuf, uout, sbytes / 16);
  CHECK(hipDeviceSynchronize());
  float best = 1e30f;
  for (int r = 0; r < 5; ++r) {
    CHECK(hipEventRecord(e0));
    hipLaunchKernelGGL(stream_read, dim3(sgrid), dim3(256), 0, 0, sbuf, uout, sbytes / 16);
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    best = ms < best ? ms : best;
  }
  const int64_t read_bytes = (sbytes / 16 / (8LL * sgrid * 256)) * (8LL * sgrid * 256) * 16;
  const double stream_gbs = (double)read_bytes / (best * 1e-3) / 1e9;

  // ---- HBM random 2 KB gather (the first half of sbuf is gathered, the second half evicts) --
  const int n = (int)((sbytes / 2) / 2048);
  std::vector<int32_t> order(n);
  uint64_t x = 0x9E3779B97F4A7C15ull;
  for (int i = 0; i < n; ++i) order[i] = i;
  for (int i = n - 1; i > 0; --i) {  // Fisher-Yates with a 64-bit LCG
    x = x * 6364136223846793005ull + 1442695040888963407ull;
    const int j = (int)((x >> 33) % (uint64_t)(i + 1));
    const int32_t t = order[i];
    order[i] = order[j];
    order[j] = t;
  }
  int32_t* d_order;
  CHECK(hipMalloc(&d_order, (size_t)n * sizeof(int32_t)));
  CHECK(hipMemcpy(d_order, order.data(), (size_t)n * sizeof(int32_t), hipMemcpyHostToDevice));
  const int ggrid = cus * 8;
  best = 1e30f;
  for (int r = 0; r < 4; ++r) {
    hipLaunchKernelGGL(stream_read, dim3(sgrid), dim3(256), 0, 0, sbuf + sbytes / 32, uout,
                       sbytes / 32);  // evict with reads of the other half
    CHECK(hipEventRecord(e0));
    hipLaunchKernelGGL(gather_read, dim3(ggrid), dim3(256), 0, 0, (const char*)sbuf, d_order, n, uout);
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    if (r > 0) best = ms < best ? ms : best;
  }
  const double gather_gbs = (double)n * 2048 / (best * 1e-3) / 1e9;

  printf("{\"mfma_bf16_tflops\": %.1f, \"sclk_mhz_under_mfma\": %.0f, \"hbm_stream_read_gbs\": %.0f, "
         "\"hbm_gather_2k_gbs\": %.0f, \"cus\": %d}\n",
         mfma_tflops, sclk_mhz, stream_gbs, gather_gbs, cus);
  CHECK(hipFree(d_order));
  CHECK(hipFree(sbuf));
  CHECK(hipFree(clk));
  CHECK(hipFree(uout));
  CHECK(hipFree(fout));
  return 0;
}
