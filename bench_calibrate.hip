// Machine calibration for the attention kernels' rooflines on one MI355X
// (gfx950): the rates the kernel designs are judged against, measured rather
// than quoted.  Built and run by `python bench.py --calibrate`.
//
//   1. matrix-core rate: v_mfma_f32_32x32x16_bf16 with independent
//      accumulation chains, 4 or 8 waves per CU;
//   2. LDS read bandwidth: ds_read_b128 rows and ds_read_b64_tr_b16
//      transposed reads at conflict-free addresses;
//   3. products fed from LDS: each 16-byte-per-lane operand read feeds
//      1, 2 or 4 products (1, 0.5, 0.25 KiB of LDS per product);
//   4. vector work under the products: fp32 FMAs and exp2 per product;
//   5. device-wide fp32 global atomic add rate (the dQ accumulation of the
//      tilelang and CK pages' backward) against plain read-modify-write.
//
// Every launch uses 1024 workgroups (four per CU); timings are the best of
// five after one warm-up launch, from hipEvents on the null stream.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

#define CHECK(x)                                                                  \
  do {                                                                            \
    hipError_t err_ = (x);                                                        \
    if (err_ != hipSuccess) {                                                     \
      printf("HIP error %s at line %d\n", hipGetErrorString(err_), __LINE__);     \
      exit(1);                                                                    \
    }                                                                             \
  } while (0)

constexpr int kWords = 8192;  // 16-byte LDS words: 128 KiB
constexpr int kGrid = 1024;   // workgroups per launch
constexpr int kIters = 1000;

__device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

template <int NW>
__device__ __forceinline__ void fill(u32x4* buf) {
  for (int i = threadIdx.x; i < kWords; i += 64 * NW) buf[i] = u32x4{(uint32_t)i, 3u * i, 7u, 9u};
  __syncthreads();
}

// 1. products only: 8 independent chains per wave
template <int NW>
__global__ __launch_bounds__(64 * NW) void k_mfma(f32x16* out, int iters) {
  const int tid = threadIdx.x;
  const u32x4 a = {(uint32_t)tid, 1u, 2u, 3u}, b = {3u, (uint32_t)tid, 1u, 2u};
  f32x16 c[8] = {};
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int k = 0; k < 8; ++k) c[k] = mfma(a, b, c[k]);
  f32x16 t = {};
#pragma unroll
  for (int k = 0; k < 8; ++k) t += c[k];
  out[blockIdx.x * 64 * NW + tid] = t;
}

// 2a. LDS row reads: 16 ds_read_b128 per iteration, consecutive lanes
// consecutive 16-byte words (conflict-free)
__global__ __launch_bounds__(512) void k_lds_b128(u32x4* out, int iters) {
  __shared__ u32x4 buf[kWords];
  fill<8>(buf);
  const int tid = threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  int base = tid;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 16; ++k) acc ^= buf[(base + k * 512) & (kWords - 1)];
    base = (base + 64) & (kWords - 1);
  }
  out[blockIdx.x * 512 + tid] = acc;
}

// 2b. LDS transposed reads: 16 ds_read_b64_tr_b16 per iteration; the 64 lanes
// of a wave cover 512 consecutive bytes (4 rows of 128 bytes)
__global__ __launch_bounds__(512) void k_lds_tr(u32x4* out, int iters) {
  __shared__ u32x4 buf[kWords];
  fill<8>(buf);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int s = lane & 15, g = lane >> 4;
  int base = w * 2048 + (s >> 2) * 128 + 32 * g + 8 * (s & 3);
  u32x2 acc = {0u, 0u};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int off = (base + k * 1024) & (kWords * 16 - 1);
      s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)((__attribute__((address_space(3))) char*)buf + off));
      acc ^= __builtin_bit_cast(u32x2, r);
    }
    base = (base + 128) & (kWords * 16 - 1);
  }
  out[blockIdx.x * 512 + tid] = u32x4{acc[0], acc[1], 0u, 0u};
}

// 3. products whose A operand is read from LDS, each read feeding RE
// products (8 chains per wave), reads issued one iteration ahead
template <int NW, int RE>
__global__ __launch_bounds__(64 * NW) void k_mfma_lds(f32x16* out, int iters) {
  __shared__ u32x4 buf[kWords];
  fill<NW>(buf);
  const int tid = threadIdx.x;
  constexpr int NA = 8 / RE;
  u32x4 b[RE];
#pragma unroll
  for (int r = 0; r < RE; ++r) b[r] = u32x4{3u + r, (uint32_t)tid, 1u, 2u};
  f32x16 c[8] = {};
  int base = tid;
  u32x4 a[NA], n[NA];
#pragma unroll
  for (int k = 0; k < NA; ++k) a[k] = buf[(base + k * 512) & (kWords - 1)];
  for (int it = 0; it < iters; ++it) {
    base = (base + 64) & (kWords - 1);
#pragma unroll
    for (int k = 0; k < NA; ++k) n[k] = buf[(base + k * 512) & (kWords - 1)];
#pragma unroll
    for (int k = 0; k < NA; ++k)
#pragma unroll
      for (int r = 0; r < RE; ++r) c[k * RE + r] = mfma(a[k], b[r], c[k * RE + r]);
#pragma unroll
    for (int k = 0; k < NA; ++k) a[k] = n[k];
  }
  f32x16 t = {};
#pragma unroll
  for (int k = 0; k < 8; ++k) t += c[k];
  out[blockIdx.x * 64 * NW + tid] = t;
}

// 4. 16 products per iteration (4 chains) with NV fp32 FMAs and NE exp2 per
// product in the same wave, independent of the products
template <int NW, int NV, int NE>
__global__ __launch_bounds__(64 * NW) void k_mix(f32x16* out, int iters) {
  const int tid = threadIdx.x;
  const u32x4 a = {(uint32_t)tid, 1u, 2u, 3u}, b = {3u, (uint32_t)tid, 1u, 2u};
  f32x16 c[4] = {};
  float x[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = (float)(tid + i) * 1e-3f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      c[k % 4] = mfma(a, b, c[k % 4]);
#pragma unroll
      for (int v = 0; v < NV; ++v) x[(k * NV + v) % 16] = __builtin_fmaf(x[(k * NV + v) % 16], 0.999f, 1e-4f);
#pragma unroll
      for (int e = 0; e < NE; ++e) x[(k * NE + e + 5) % 16] = __builtin_amdgcn_exp2f(x[(k * NE + e + 5) % 16]) * 0.5f;
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  f32x16 t = {};
#pragma unroll
  for (int k = 0; k < 4; ++k) t += c[k];
#pragma unroll
  for (int i = 0; i < 16; ++i) t[i] += x[i];
  out[blockIdx.x * 64 * NW + tid] = t;
}

// 5. fp32 global atomic add into 64 x 128 fp32 blocks (32 KiB, one per
// workgroup modulo nblk), 32 coalesced adds per thread per pass
__global__ __launch_bounds__(256) void k_atomic(float* acc, int nblk, int passes) {
  float* blk = acc + (size_t)(blockIdx.x % nblk) * 8192;
  const int tid = threadIdx.x;
  for (int p = 0; p < passes; ++p)
#pragma unroll
    for (int i = 0; i < 32; ++i) __builtin_amdgcn_global_atomic_fadd_f32(blk + i * 256 + tid, 1.0f);
}

__global__ __launch_bounds__(256) void k_rmw(float* acc, int nblk, int passes) {
  float* blk = acc + (size_t)(blockIdx.x % nblk) * 8192;
  const int tid = threadIdx.x;
  for (int p = 0; p < passes; ++p)
#pragma unroll
    for (int i = 0; i < 32; ++i) blk[i * 256 + tid] += 1.0f;
}

template <typename F>
float best_ms(F f) {
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  f();
  CHECK(hipDeviceSynchronize());
  float best = 1e30f;
  for (int r = 0; r < 5; ++r) {
    CHECK(hipEventRecord(e0));
    f();
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    if (ms < best) best = ms;
  }
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
  return best;
}

int main() {
  hipDeviceProp_t prop;
  CHECK(hipGetDeviceProperties(&prop, 0));
  printf("device: %s (%s), %d CUs\n", prop.name, prop.gcnArchName, prop.multiProcessorCount);
  const double peak = 2516.6;  // dense bf16 matrix TFLOP/s, published
  void* out;
  CHECK(hipMalloc(&out, (size_t)kGrid * 512 * sizeof(f32x16)));
  f32x16* o16 = (f32x16*)out;
  u32x4* o4 = (u32x4*)out;
  const double prod = 32768.0;  // flop per 32x32x16 product

  printf("\n1. matrix-core rate, v_mfma_f32_32x32x16_bf16\n");
  {
    float ms = best_ms([&] { hipLaunchKernelGGL((k_mfma<4>), dim3(kGrid), dim3(256), 0, 0, o16, kIters); });
    double tf = (double)kGrid * 4 * 8 * kIters * prod / ms / 1e9;
    printf("   4 waves/CU: %8.1f TFLOP/s (%.1f %% of %.1f)\n", tf, 100 * tf / peak, peak);
    ms = best_ms([&] { hipLaunchKernelGGL((k_mfma<8>), dim3(kGrid), dim3(512), 0, 0, o16, kIters); });
    tf = (double)kGrid * 8 * 8 * kIters * prod / ms / 1e9;
    printf("   8 waves/CU: %8.1f TFLOP/s (%.1f %% of %.1f)\n", tf, 100 * tf / peak, peak);
  }

  printf("\n2. LDS read bandwidth (8 waves/CU)\n");
  {
    float ms = best_ms([&] { hipLaunchKernelGGL(k_lds_b128, dim3(kGrid), dim3(512), 0, 0, o4, kIters); });
    double by = (double)kGrid * 512 * 16 * 16 * kIters;
    printf("   ds_read_b128:       %6.1f TB/s device, %6.1f B/clk/CU at 2.4 GHz\n", by / ms / 1e9,
           by / ms / 1e-3 / 256 / 2.4e9);
    ms = best_ms([&] { hipLaunchKernelGGL(k_lds_tr, dim3(kGrid), dim3(512), 0, 0, o4, kIters); });
    by = (double)kGrid * 512 * 8 * 16 * kIters;
    printf("   ds_read_b64_tr_b16: %6.1f TB/s device, %6.1f B/clk/CU at 2.4 GHz\n", by / ms / 1e9,
           by / ms / 1e-3 / 256 / 2.4e9);
  }

  printf("\n3. products with an LDS operand read per RE products\n");
#define RUN_LDS(NW, RE)                                                                                   \
  {                                                                                                     \
    float ms = best_ms([&] { hipLaunchKernelGGL((k_mfma_lds<NW, RE>), dim3(kGrid), dim3(64 * NW), 0, 0, o16, kIters); }); \
    double tf = (double)kGrid * NW * 8 * kIters * prod / ms / 1e9;                                     \
    printf("   %d waves/CU, %.2f KiB/product: %8.1f TFLOP/s\n", NW, 1.0 / RE, tf);                         \
  }
  RUN_LDS(4, 1) RUN_LDS(4, 2) RUN_LDS(4, 4) RUN_LDS(8, 1) RUN_LDS(8, 2) RUN_LDS(8, 4)

  printf("\n4. vector work in the same wave as the products (cycles per product per SIMD at 2.4 GHz)\n");
#define RUN_MIX(NW, NV, NE)                                                                                \
  {                                                                                                      \
    float ms = best_ms([&] { hipLaunchKernelGGL((k_mix<NW, NV, NE>), dim3(kGrid), dim3(64 * NW), 0, 0, o16, kIters); }); \
    double tf = (double)kGrid * NW * 16 * kIters * prod / ms / 1e9;                                     \
    printf("   %d waves/CU, %d fma + %d exp2 per product: %8.1f TFLOP/s, %5.1f cycles\n", NW, NV, NE, tf,      \
           ms * 1e-3 * 2.4e9 / ((double)kGrid / 256.0 * NW / 4 * 16 * kIters));                           \
  }
  RUN_MIX(8, 0, 0) RUN_MIX(8, 2, 0) RUN_MIX(8, 4, 0) RUN_MIX(8, 6, 0) RUN_MIX(8, 8, 0) RUN_MIX(8, 2, 1)
  RUN_MIX(8, 4, 1) RUN_MIX(8, 2, 2) RUN_MIX(4, 4, 1) RUN_MIX(4, 2, 2)

  printf("\n5. fp32 global atomic add vs plain read-modify-write (8192 workgroups x 256 threads x 128 adds)\n");
  {
    float* acc;
    const int nblk_max = 4096;
    CHECK(hipMalloc(&acc, (size_t)nblk_max * 8192 * sizeof(float)));
    CHECK(hipMemset(acc, 0, (size_t)nblk_max * 8192 * sizeof(float)));
    for (int nb : {64, 4096}) {
      const int wgs = 8192, passes = 4;
      const double ops = (double)wgs * 256 * 32 * passes;
      float ms = best_ms([&] { hipLaunchKernelGGL(k_atomic, dim3(wgs), dim3(256), 0, 0, acc, nb, passes); });
      printf("   atomic add, %4d target blocks of 32 KiB: %8.1f G lane-ops/s\n", nb, ops / ms / 1e6);
      ms = best_ms([&] { hipLaunchKernelGGL(k_rmw, dim3(wgs), dim3(256), 0, 0, acc, nb, passes); });
      printf("   plain rmw,  %4d target blocks of 32 KiB: %8.1f G lane-ops/s\n", nb, ops / ms / 1e6);
    }
    CHECK(hipFree(acc));
  }
  CHECK(hipFree(out));
  return 0;
}
