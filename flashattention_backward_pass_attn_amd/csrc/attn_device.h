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

#include <type_traits>

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
  float* lse2;          // workspace: LSE * log2(e), laid out like lse (written by the preprocess)
  float* delta_out;     // optional copy of delta
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
  int32_t batch, seqlen_q, seqlen_k, heads_q, heads_kv, group, head_dim;
  int32_t total_q;  // varlen: packed rows (row count per head of LSE / Delta)
  float scale;       // softmax scale
  float scale_log2;  // scale * log2(e)
  int32_t varlen;
  // Banded mask (kernels instantiated with BANDED = true): key j is visible
  // to query i iff i + off - win_l <= j <= i + off + win_r, off = Sk - Sq
  // (bottom-right aligned).  Causal: win_l = kWinInf, win_r = 0; a local
  // window bounds both sides; kWinInf stands for "no bound".
  int32_t win_l, win_r;
};

// Per-(sequence) geometry: row offsets into packed tensors and lengths.
struct Seq {
  int32_t q0, k0;    // first row of the sequence in the (packed) row axis
  int32_t sq, sk;    // lengths
  int64_t bq, bk;    // batch index used with batch strides (0 in varlen)
  int64_t stat0;     // offset of row 0 of head 0 in lse/delta
  int64_t stat_h;    // head stride in lse/delta
};

// Read-only int32 data (the cu_seqlens arrays, never written while a kernel
// runs) through the constant address space: scalar loads.
__device__ __forceinline__ int32_t ld_const_i32(const int32_t* p, int i) {
  return ((__attribute__((address_space(4))) const int32_t*)p)[i];
}

// The kernel argument block through the constant address space, re-read at
// each use (an opaque copy of its address per call): for arguments used only
// outside a kernel's hot loop, so that they are not held in scalar registers
// across it.
typedef __attribute__((address_space(4))) const Args KArgs;
__device__ __forceinline__ KArgs& kernel_args() {
  const KArgs* p = (const KArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(p));
  return *p;
}

template <class ArgsT>
__device__ inline Seq seq_info(const ArgsT& a, int z) {
  Seq s;
  if (a.varlen) {
    s.q0 = ld_const_i32(a.cu_q, z);
    s.k0 = ld_const_i32(a.cu_k, z);
    s.sq = ld_const_i32(a.cu_q, z + 1) - s.q0;
    s.sk = ld_const_i32(a.cu_k, z + 1) - s.k0;
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

constexpr int kWinInf = 1 << 29;  // "no bound" for a side of the banded mask

// Keys [lo, hi] (inclusive, clamped to [0, sk-1]; hi < lo when empty) seen by
// any of the queries [qa, qb] under the banded mask.
struct Range {
  int lo, hi;
};
__device__ inline Range band_keys(const Args& a, int qa, int qb, int sq, int sk) {
  const int off = sk - sq;
  return Range{max(0, qa + off - a.win_l), min(sk - 1, qb + off + a.win_r)};
}
// Queries [lo, hi] that see any of the keys [ka, kb].
__device__ inline Range band_queries(const Args& a, int ka, int kb, int sq, int sk) {
  const int off = sk - sq;
  return Range{max(0, ka - off - a.win_r), min(sq - 1, kb - off + a.win_l)};
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

// Two fp32 -> one dword of two 16-bit values (round to nearest even), one
// v_cvt_pk_{bf16,f16}_f32.
template <bool BF16>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  const f32x2 v = {lo, hi};
  if constexpr (BF16) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  } else {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  }
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

// ---------------------------------------------------------------------------
// Buffer resources: range-checked global access.  A raw buffer access whose
// byte offset lies at or past num_records is dropped (stores, atomics) or
// reads zero (loads), so tile tails need no branches: rows past the end of a
// sequence and head-dim columns past head_dim are steered out of range.
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // 32-bit data format, raw (untyped) access
constexpr int kOffOOB = 0x7fffff00;           // an offset past every num_records used

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t num_bytes) {
  const int n = num_bytes <= 0 ? 0 : (num_bytes >= 0x7fffff00 ? 0x7fffff00 : (int)num_bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, (int)kRsrcWord3);
}

__device__ __forceinline__ u32x4 buf_load128(rsrc_t r, int off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ __forceinline__ float buf_load_f32(rsrc_t r, int off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

__device__ __forceinline__ void buf_store_u16(rsrc_t r, int off, uint16_t v) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, 0);
}

// ---------------------------------------------------------------------------
// Epilogue store of a wave's 32-row x 32*NT-column fp32 tile held in the MFMA
// C layout (tile t: lane l holds column 32t + l%32 and rows 8(j/4) + 4(l/32) +
// j%4), as 16-bit values into a row-major global matrix.  The tile passes
// through this wave's LDS region `lds` (32*NT*72 bytes): written column-major
// (4 consecutive rows per 8-byte write, columns 72 bytes apart, which spreads
// the 64 lanes over every bank), then read back with the transpose read so
// that each lane holds 8 consecutive columns of one row, stored as one
// 16-byte write.  `dst` covers the matrix from the tile's first row and
// column (row stride `rs` elements); rows >= rows_ok and columns >= cols_ok
// (a multiple of 8) are not written.  Values are multiplied by `mul` and
// rounded to nearest even.
// ---------------------------------------------------------------------------
template <bool BF16, int NT>
__device__ __forceinline__ void store_tile_rows(const f32x16* acc, float mul, uint8_t* lds, rsrc_t dst, int rs,
                                                int rows_ok, int cols_ok, int lane) {
  constexpr int CS = 72;  // bytes per stored column (32 rows + 4 elements of padding)
  const int c32 = lane & 31, h = lane >> 5;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      u32x2 v;
      v[0] = pack2<BF16>(acc[t][4 * jj] * mul, acc[t][4 * jj + 1] * mul);
      v[1] = pack2<BF16>(acc[t][4 * jj + 2] * mul, acc[t][4 * jj + 3] * mul);
      *reinterpret_cast<u32x2*>(lds + (32 * t + c32) * CS + (8 * jj + 4 * h) * 2) = v;
    }
  }
  __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  // 16-lane group g reads 16 rows x 8 columns per step: lane s addresses
  // column d0 + s/4, rows r0 + 4(s%4) .. +3, and receives row r0 + s,
  // columns d0 .. d0+3 (then d0+4 .. d0+7 from the second read).
  const int g = lane >> 4, s = lane & 15;
#pragma unroll
  for (int it = 0; it < 2 * NT; ++it) {
    const int b = 4 * it + g;
    const int r0 = 16 * (b & 1), d0 = 8 * (b >> 1);
    const uint8_t* p = lds + (d0 + (s >> 2)) * CS + (r0 + 4 * (s & 3)) * 2;
    const u32x2 x = lds_tr4(reinterpret_cast<const uint16_t*>(p));
    const u32x2 y = lds_tr4(reinterpret_cast<const uint16_t*>(p + 4 * CS));
    const int row = r0 + s;
    const bool ok = row < rows_ok && d0 < cols_ok;
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{x[0], x[1], y[0], y[1]}, dst,
                                           ok ? (row * rs + d0) * 2 : kOffOOB, 0, 0);
  }
}

// ---------------------------------------------------------------------------
// Direct global -> LDS loads (gfx950 buffer_load ... lds).  Lane t's 16 bytes
// (or 4 bytes) land at LDS byte address m0 + 16*t (4*t); lanes whose offset
// is out of range write zeros.  Issued through inline asm so that the
// compiler does not wait for them before unrelated LDS reads; the caller
// waits with wait_vmcnt<>() and publishes with lds_barrier().
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const void*)p);
}

// Buffer descriptor in scalar registers for the inline-asm loads.
__device__ __forceinline__ u32x4 make_srd(const void* base, int64_t num_bytes) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  const int n = num_bytes <= 0 ? 0 : (num_bytes >= 0x7fffff00 ? 0x7fffff00 : (int)num_bytes);
  u32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((uint32_t)b);
  r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32) & 0xffffu);
  r[2] = __builtin_amdgcn_readfirstlane((uint32_t)n);
  r[3] = kRsrcWord3;
  return r;
}

// The compiler does not see into the asm, so it inserts no wait states for
// it.  An LDS DMA reading M0 one instruction after a scalar write of M0 (the
// compiler sets M0 for the "{m0}" operand right before the asm) needs one:
// the s_nop supplies it.  The descriptor's scalar registers must not have
// been written by a vector instruction (readfirstlane, a spill reload)
// within the five instructions before the load; the build's test of the
// generated assembly checks that for every direct load.
__device__ __forceinline__ void dma16(u32x4 srd, int off, uint32_t lds_byte) {
  __asm__ volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" :: "v"(off), "s"(srd), "{m0}"(lds_byte)
                   : "memory");
}

__device__ __forceinline__ void dma4(u32x4 srd, int off, uint32_t lds_byte) {
  __asm__ volatile("s_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds" :: "v"(off), "s"(srd), "{m0}"(lds_byte)
                   : "memory");
}

// s_waitcnt vmcnt(N) leaving the other counters alone (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ u32x4 lds_rd128(const uint8_t* base, int byte_off) {
  return *reinterpret_cast<const u32x4*>(base + byte_off);
}

__device__ __forceinline__ u32x4 tr_frag_b(const uint8_t* base, int off_a, int off_b) {
  const u32x2 x = lds_tr4(reinterpret_cast<const uint16_t*>(base + off_a));
  const u32x2 y = lds_tr4(reinterpret_cast<const uint16_t*>(base + off_b));
  u32x4 r;
  r[0] = x[0];
  r[1] = x[1];
  r[2] = y[0];
  r[3] = y[1];
  return r;
}

// Workgroup barrier for LDS hand-off: wait for this wave's LDS reads/writes,
// then s_barrier.  Unlike __syncthreads() it does not wait for outstanding
// global memory operations (direct loads of later tiles stay in flight); a
// caller that published data with direct global->LDS loads waits for them
// first with wait_vmcnt<>().  The memory clobber keeps the compiler from
// moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wave index as a scalar (uniform) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// ---------------------------------------------------------------------------
// Instruction-scheduling hints (sched_group_barrier masks: 0x8 MFMA,
// 0x100 DS read, 0x200 DS write, 0x2 VALU).  pipeline_hint<N, R, A>() asks the
// scheduler to issue, for a straight-line section of N MFMAs each fed by R LDS
// reads, the reads A MFMAs ahead of their use, so the matrix core does not
// wait for each read's latency.  Placed at the end of the section.
// ---------------------------------------------------------------------------
template <int N, int R, int A>
__device__ __forceinline__ void pipeline_hint() {
  __builtin_amdgcn_sched_group_barrier(0x100, R * A, 0);
#pragma unroll
  for (int i = 0; i < N - A; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
  }
#pragma unroll
  for (int i = 0; i < A; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
}

__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// Compile-time iteration: f(integral_constant<int, B>), ..., f(<E-1>).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}


// ---------------------------------------------------------------------------
// LDS tile swizzle.  Tiles are row-major with rows of CPR 16-byte chunks;
// chunk c of row r is stored at chunk position c ^ swz(r).  Chosen so that
// the three access patterns of the kernels -- 16 lanes reading 16 consecutive
// rows at one chunk (ds_read_b128), and 32 lanes transposing a 4-row x
// 32-column block from each of two 4-row groups (ds_read_b64_tr_b16) -- each
// touch every bank once (64 banks x 4 bytes).
// ---------------------------------------------------------------------------
template <int CPR>
__device__ __forceinline__ int swz(int r) {
  static_assert(CPR == 8 || CPR == 16 || CPR == 32, "rows of 128, 256 or 512 bytes");
  // 512-byte rows cover the 64 banks twice: permuting the low four chunk
  // bits as for 256-byte rows gives every access pattern the same bank
  // spread (bank group = chunk mod 16).
  if constexpr (CPR == 16 || CPR == 32) {
    return 4 * (r & 3) + ((r >> 2) & 3);
  } else {
    return 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
  }
}

// Byte offset of element column `col` (16-bit elements) of row r.
template <int CPR>
__device__ __forceinline__ int tile_off(int r, int col) {
  return r * CPR * 16 + (((col >> 3) ^ swz<CPR>(r)) << 4) + ((col & 7) << 1);
}

}  // namespace attn
