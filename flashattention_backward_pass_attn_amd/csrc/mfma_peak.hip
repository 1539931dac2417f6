// Standalone measurement, not part of libattn.so: the dense matrix-core rate
// an MI355X (gfx950) sustains for v_mfma_f32_32x32x16_{bf16,f16}, and how much
// independent vector-ALU work hides under it on one SIMD.  These two figures
// bound what the attention kernels can reach: the rate sets the practical
// ceiling (the published peak assumes 2.4 GHz under full matrix load), and
// the overlap says whether the softmax arithmetic is free or adds to the
// product time.
//
//   hipcc --offload-arch=gfx950 -O3 -Xclang -target-feature -Xclang -packed-fp32-ops \
//       flashattention_backward_pass_attn_amd/csrc/mfma_peak.hip -o /tmp/mfma_peak && /tmp/mfma_peak
//
// Every launch is 256 workgroups of 512 threads (one per CU, two waves per
// SIMD); each wave runs four independent accumulator chains.  Output: one line
// per case with the kernel time and either TFLOP/s or cycles per loop
// iteration per SIMD at the clock the matrix-only case implies.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

#define CHECK(x)                                                                   \
  do {                                                                             \
    hipError_t e_ = (x);                                                           \
    if (e_ != hipSuccess) {                                                        \
      std::fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));                 \
      std::exit(1);                                                                \
    }                                                                              \
  } while (0)

// MODE 0: products only (bf16); 1: products only (fp16); 2: products plus NV
// independent fp32 FMAs after each product, same wave; 3: the FMAs alone;
// 4: products plus NV/4 exp2 after each product, same wave.
template <int MODE, int NV>
__global__ __launch_bounds__(512) void loop_kernel(float* out, int iters, float seed) {
  f32x16 acc[4];
  for (int c = 0; c < 4; ++c) acc[c] = f32x16{};
  bf16x8 ab, bb;
  f16x8 ah, bh;
  for (int i = 0; i < 8; ++i) {
    ab[i] = (__bf16)(seed * (threadIdx.x + i));
    bb[i] = (__bf16)(seed * i);
    ah[i] = (_Float16)(seed * (threadIdx.x + i));
    bh[i] = (_Float16)(seed * i);
  }
  float x[8];
  for (int i = 0; i < 8; ++i) x[i] = seed * (threadIdx.x + 3 * i);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (MODE == 1) {
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bh, acc[c], 0, 0, 0);
      } else if (MODE != 3) {
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab, bb, acc[c], 0, 0, 0);
      }
      if (MODE == 2 || MODE == 3) {
#pragma unroll
        for (int v = 0; v < NV; ++v) x[v & 7] = __builtin_fmaf(x[v & 7], 0.999f, 0.001f);
      } else if (MODE == 4) {
#pragma unroll
        for (int v = 0; v < NV / 4; ++v) x[v & 7] = __builtin_amdgcn_exp2f(x[v & 7]);
      }
    }
  }
  float s = 0.f;
  for (int c = 0; c < 4; ++c)
    for (int j = 0; j < 16; ++j) s += acc[c][j];
  for (int i = 0; i < 8; ++i) s += x[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

constexpr int kBlocks = 256, kThreads = 512, kIters = 2000;

template <int MODE, int NV>
float time_ms(float* out) {
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  float best = 1e30f;
  for (int rep = 0; rep < 5; ++rep) {
    CHECK(hipEventRecord(e0));
    hipLaunchKernelGGL((loop_kernel<MODE, NV>), dim3(kBlocks), dim3(kThreads), 0, 0, out, kIters, 1e-3f);
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    if (rep > 0 && ms < best) best = ms;  // first launch warms the clock
  }
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
  return best;
}

int main() {
  float* out;
  CHECK(hipMalloc(&out, sizeof(float) * kBlocks * kThreads));
  // 8 waves x 4 chains x 32768 flop per product per iteration, per workgroup
  const double flop = (double)kBlocks * 8 * 4 * 32768.0 * kIters;
  // 2 waves x 4 products per iteration per SIMD, 32 cycles each at the full rate
  const double cyc_per_iter_ideal = 2 * 4 * 32.0;
  const float mb = time_ms<0, 0>(out);
  const float mh = time_ms<1, 0>(out);
  std::printf("products only, bf16: %.3f ms, %.1f TFLOP/s\n", mb, flop / mb / 1e9);
  std::printf("products only, fp16: %.3f ms, %.1f TFLOP/s\n", mh, flop / mh / 1e9);
  // the clock implied by the matrix-only case (32 cycles per product per SIMD)
  const double ghz = cyc_per_iter_ideal * kIters / (mb * 1e-3) / 1e9;
  std::printf("implied clock under matrix load: %.2f GHz\n", ghz);
  auto cyc = [&](float ms) { return ms * 1e-3 * ghz * 1e9 / kIters; };
  std::printf("cycles per iteration per SIMD (2 waves x 4 products = %.0f at the full rate):\n", cyc_per_iter_ideal);
  std::printf("  FMAs alone, 8 per product slot:       %.0f\n", cyc(time_ms<3, 8>(out)));
  std::printf("  FMAs alone, 16 per product slot:      %.0f\n", cyc(time_ms<3, 16>(out)));
  std::printf("  products + 2 FMAs each:               %.0f\n", cyc(time_ms<2, 2>(out)));
  std::printf("  products + 4 FMAs each:               %.0f\n", cyc(time_ms<2, 4>(out)));
  std::printf("  products + 8 FMAs each:               %.0f\n", cyc(time_ms<2, 8>(out)));
  std::printf("  products + 16 FMAs each:              %.0f\n", cyc(time_ms<2, 16>(out)));
  std::printf("  products + 2 exp2 each:               %.0f\n", cyc(time_ms<4, 8>(out)));
  std::printf("  products + 4 exp2 each:               %.0f\n", cyc(time_ms<4, 16>(out)));
  CHECK(hipFree(out));
  return 0;
}
