// Attention backward on gfx950: the preprocess, standalone and as the part of
// it that the dQ kernels run themselves.
//
// Delta_i = sum_d O_id dO_id, in fp32 (tilelang test_tilelang_kernel_mha_bwd.py,
// flashattn_bwd_preprocess; the flash-attention CK mha_bwd.cpp page's
// softmax_d).  Delta equals rowsum(P o dP) and enters dS = P o (dP - Delta) in
// both gradient kernels (attn_bwd_split.h).
#pragma once

#include "attn_device.h"

namespace attn {

constexpr int kPreRows = 64;  // rows per preprocess workgroup

// ---------------------------------------------------------------------------
// Preprocess: Delta = rowsum(O o dO) in fp32 (tilelang
// flashattn_bwd_preprocess).  16 lanes per row, 16 rows per pass.
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(256) void attn_bwd_pre_kernel(Args a) {
  const int z = blockIdx.z, hq = blockIdx.y;
  const Seq s = seq_info(a, z);
  const int r0 = blockIdx.x * kPreRows;
  if (r0 >= s.sq) return;
  const int tid = threadIdx.x, sub = tid & 15, rg = tid >> 4;
  const int hd = a.head_dim;
  const uint16_t* ob = a.o + s.bq * a.o_b + (int64_t)s.q0 * a.o_r + (int64_t)hq * a.o_h;
  const uint16_t* db = a.dout + s.bq * a.do_b + (int64_t)s.q0 * a.do_r + (int64_t)hq * a.do_h;
  const int64_t st0 = s.stat0 + (int64_t)hq * s.stat_h;
#pragma unroll
  for (int pass = 0; pass < kPreRows / 16; ++pass) {
    const int r = r0 + pass * 16 + rg;
    float acc = 0.f;
    if (r < s.sq) {
      for (int c = 8 * sub; c < hd; c += 128) {
        const u32x4 ov = ldg128(ob + (int64_t)r * a.o_r + c);
        const u32x4 dv = ldg128(db + (int64_t)r * a.do_r + c);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc += from_bits<BF16>((uint16_t)(ov[i] & 0xffffu)) * from_bits<BF16>((uint16_t)(dv[i] & 0xffffu));
          acc += from_bits<BF16>((uint16_t)(ov[i] >> 16)) * from_bits<BF16>((uint16_t)(dv[i] >> 16));
        }
      }
    }
    acc += __shfl_xor(acc, 1);
    acc += __shfl_xor(acc, 2);
    acc += __shfl_xor(acc, 4);
    acc += __shfl_xor(acc, 8);
    if (sub == 0 && r < s.sq) {
      // the workspace keeps -Delta: the gradient kernels start the dP
      // accumulator from it, so dP - Delta costs no vector instruction
      a.delta[st0 + r] = -acc;
      if (a.delta_out) a.delta_out[st0 + r] = acc;
    } else if (sub == 1 && r < s.sq) {
      // the exp2-domain LSE the dK/dV kernel stages with Delta
      a.lse2[st0 + r] = a.lse_in[st0 + r] * kLog2e;
    }
  }
}

// ---------------------------------------------------------------------------
// The preprocess fused into the dQ kernels.  A dQ wave holds each of its query
// rows of O and dO as B-operand fragments split over a lane pair: lane c32
// holds the 8-element chunks 16*sd .. +8 and lane c32 + 32 the chunks
// 16*sd + 8 .. +8.  Each lane sums O o dO over its chunks in fp32 and the pair
// adds the two halves, so both lanes end with Delta of the row.
// ---------------------------------------------------------------------------
template <bool BF16, int N>
__device__ __forceinline__ float row_delta_pair(const u32x4 (&o)[N], const u32x4 (&d)[N]) {
  float acc = 0.f;
#pragma unroll
  for (int sd = 0; sd < N; ++sd) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc += from_bits<BF16>((uint16_t)(o[sd][i] & 0xffffu)) * from_bits<BF16>((uint16_t)(d[sd][i] & 0xffffu));
      acc += from_bits<BF16>((uint16_t)(o[sd][i] >> 16)) * from_bits<BF16>((uint16_t)(d[sd][i] >> 16));
    }
  }
  return acc + __shfl_xor(acc, 32);
}

// The workspace entries of one query row, written by lane half 0 of its pair:
// -Delta (the gradient kernels' dP start value) and LSE * log2(e); lane half 1
// writes Delta to delta_out when the caller asked for it.
__device__ __forceinline__ void store_row_stats(float* delta, float* lse2_ws, float* delta_out, int64_t idx, int h,
                                                float lse2, float neg_delta) {
  if (h == 0) {
    delta[idx] = neg_delta;
    lse2_ws[idx] = lse2;
  } else if (delta_out) {
    delta_out[idx] = -neg_delta;
  }
}

}  // namespace attn
