// Device-side building blocks shared by the gfx950 attention kernels:
// matrix-core (MFMA) wrappers, 16-bit conversions, vector load/store helpers
// and the index arithmetic of the tensor layouts.
//
// MFMA layout used throughout (v_mfma_f32_32x32x16_{f16,bf16}, wave64):
//   A (32 x 16, M x K): lane l holds row l%32, k = 8*(l/32) + i, i = 0..7
//   B (16 x 32, K x N): lane l holds col l%32, k = 8*(l/32) + i
//   C (32 x 32):        lane l holds col l%32, rows 8*(j/4) + 4*(l/32) + j%4,
//                        j = 0..15
// The product sums over k, so any relabelling of k that is applied to both A
// and B gives the same C.  The kernels use that freedom: a C tile whose rows
// are the reduction index of the next contraction is fed back as an operand
// directly, with k-slot i of lane-half h standing for row
// 8*(i/4) + 4*h + i%4 of a 16-row step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// Arguments shared by every kernel (passed by value).
// ---------------------------------------------------------------------------
struct Args {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  uint16_t* out_o;  // forward output
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  const float* lse_in;  // backward input (natural log)
  float* lse_out;       // forward output (natural log)
  float* delta;         // workspace, laid out like lse
  float* delta_out;     // optional copy of delta
  float* dq_acc;        // workspace, fp32
  const int32_t* cu_q;
  const int32_t* cu_k;
  // element strides: batch, row, head (dim stride is 1)
  int64_t q_b, q_r, q_h;
  int64_t k_b, k_r, k_h;
  int64_t v_b, v_r, v_h;
  int64_t o_b, o_r, o_h;
  int64_t do_b, do_r, do_h;
  int64_t dq_b, dq_r, dq_h;
  int64_t dk_b, dk_r, dk_h;
  int64_t dv_b, dv_r, dv_h;
  int64_t acc_split;  // elements between deterministic dQ accumulator slices
  int32_t batch, seqlen_q, seqlen_k, heads_q, heads_kv, group, head_dim;
  int32_t total_q;  // varlen: packed rows (stat/accumulator row count per head)
  float scale;       // softmax scale
  float scale_log2;  // scale * log2(e)
  int32_t varlen;
};

// Per-(sequence) geometry: row offsets into packed tensors and lengths.
struct Seq {
  int32_t q0, k0;    // first row of the sequence in the (packed) row axis
  int32_t sq, sk;    // lengths
  int64_t bq, bk;    // batch index used with batch strides (0 in varlen)
  int64_t stat0;     // offset of row 0 of head 0 in lse/delta
  int64_t stat_h;    // head stride in lse/delta
};

__device__ inline Seq seq_info(const Args& a, int z) {
  Seq s;
  if (a.varlen) {
    s.q0 = a.cu_q[z];
    s.k0 = a.cu_k[z];
    s.sq = a.cu_q[z + 1] - s.q0;
    s.sk = a.cu_k[z + 1] - s.k0;
    s.bq = 0;
    s.bk = 0;
    s.stat0 = s.q0;
    s.stat_h = a.total_q;
  } else {
    s.q0 = 0;
    s.k0 = 0;
    s.sq = a.seqlen_q;
    s.sk = a.seqlen_k;
    s.bq = z;
    s.bk = z;
    s.stat0 = (int64_t)z * a.heads_q * a.seqlen_q;
    s.stat_h = a.seqlen_q;
  }
  return s;
}

// Offset (elements) of row 0, head h of the dQ accumulator for sequence z.
// Layout: fixed [B][H][Sq][d], varlen [H][total_q][d] (d = head_dim).
__device__ inline int64_t acc_base(const Args& a, const Seq& s, int h) {
  return (s.stat0 + (int64_t)h * s.stat_h) * a.head_dim;
}

// First q block (of BM rows) that sees any key of KV block n (of BN rows).
// Causal visibility is j <= i + (sk - sq).
template <int BM, int BN, bool CAUSAL>
__device__ inline int first_q_block(int n, int sq, int sk) {
  if (!CAUSAL) return 0;
  int lo = n * BN - (sk - sq);
  return lo <= 0 ? 0 : lo / BM;
}

// ---------------------------------------------------------------------------
// MFMA wrapper: C += A * B on a 32x32x16 tile with 16-bit inputs.
// ---------------------------------------------------------------------------
template <bool BF16>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
}

// fp32 -> 16-bit storage with round-to-nearest-even.
template <bool BF16>
__device__ __forceinline__ uint16_t to_bits(float x) {
  if constexpr (BF16) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
  } else {
    return __builtin_bit_cast(uint16_t, (_Float16)x);
  }
}

template <bool BF16>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return (uint32_t)to_bits<BF16>(lo) | ((uint32_t)to_bits<BF16>(hi) << 16);
}

template <bool BF16>
__device__ __forceinline__ float from_bits(uint16_t b) {
  if constexpr (BF16) {
    return __uint_as_float((uint32_t)b << 16);
  } else {
    return (float)__builtin_bit_cast(_Float16, b);
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ u32x4 ldg128(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ u32x4 lds128(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ u32x2 lds64(const uint16_t* p) {
  return *reinterpret_cast<const u32x2*>(p);
}

__device__ __forceinline__ void sts128(uint16_t* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Scatter the 8 16-bit elements of v into column `r` of a [8][ld] block:
// dst[i * ld] = element i (a transposed store of one 16-byte row chunk).
__device__ __forceinline__ void sts_transposed8(uint16_t* dst, int ld, u32x4 v) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    dst[(2 * i) * ld] = (uint16_t)(v[i] & 0xffffu);
    dst[(2 * i + 1) * ld] = (uint16_t)(v[i] >> 16);
  }
}

// ---------------------------------------------------------------------------
// LDS transpose read (ds_read_b64_tr_b16).  Within each 16-lane group, lane i
// receives element i%4 of the 8-byte chunks addressed by lanes i/4 + 4*r of
// the group, r = 0..3.  If lane s of the group addresses row (s/4) and
// columns 4*(s%4)..+3 of a row-major 16-bit matrix, lane i gets the 4 rows of
// column i: the k-major operand layout the MFMA wants, read straight from a
// row-major tile.
// ---------------------------------------------------------------------------
typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x2 lds_tr4(const uint16_t* p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(u32x2, r);
}

// Per-lane element offset for tr_frag: row (s/4) and column 16*(g%2) + 4*(s%4)
// of a 32-column block, where g is the 16-lane group and s the lane within it.
__device__ __forceinline__ int tr_lane_offset(int lane, int ld) {
  int s = lane & 15;
  int g = lane >> 4;
  return (s >> 2) * ld + 16 * (g & 1) + 4 * (s & 3);
}

// MFMA operand fragment for column (lane%32) of a 32-column block of a
// row-major 16-bit LDS matrix: k-slots 0..3 are rows ra..ra+3, k-slots 4..7
// are rows rb..rb+3.  `p` already includes tr_lane_offset().
__device__ __forceinline__ u32x4 tr_frag(const uint16_t* p, int ld, int ra, int rb) {
  u32x2 x = lds_tr4(p + ra * ld);
  u32x2 y = lds_tr4(p + rb * ld);
  u32x4 r;
  r[0] = x[0];
  r[1] = x[1];
  r[2] = y[0];
  r[3] = y[1];
  return r;
}

}  // namespace attn
