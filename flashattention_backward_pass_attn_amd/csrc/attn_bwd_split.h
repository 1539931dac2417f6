// Attention backward on gfx950 as two matrix-core kernels that never use
// atomics: a KV-stationary kernel for dK and dV and a Q-stationary kernel for
// dQ.  Both recompute P = exp2(S*scale*log2e - LSE*log2e) from the saved LSE
// (tilelang test_tilelang_kernel_mha_bwd.py, flashattn_bwd) and
// dS = P o (dP - Delta) with Delta from the preprocess.
//
// Why two kernels: the pages accumulate dQ across key blocks with fp32
// atomics (tilelang flashattn_bwd's atomic_add; the CK mha_bwd.cpp page's
// dq_accum).  On MI355X the device-wide fp32 atomic rate is ~330 G lane-ops/s
// for every access shape, which for a causal S=4096, d=128 workload puts a
// floor of ~1.7 ms (128-key blocks) under the dQ accumulation alone.  The
// Q-stationary dQ kernel recomputes S and dP (two extra GEMMs, 7 instead of 5
// per tile pair) but keeps dQ in registers, writes it once, and is
// deterministic by construction (key blocks are summed in ascending order).
//
// Both kernels use 8 wave64s (two per SIMD, so one wave's softmax VALU work
// and LDS reads hide behind the other's matrix-core work).  Each wave owns 32
// rows of the stationary operand and splits the streamed tile with a partner
// wave: the pair computes the two halves of the score tile (no duplicated
// MFMA work), trades their packed probability/gradient operands through LDS,
// and then each wave accumulates one half of the head dimension.
#pragma once

#include <type_traits>

#include "attn_bwd.h"
#include "attn_device.h"

namespace attn {

constexpr int kDkvBM = 64;    // query rows per iteration of the dK/dV kernel
constexpr int kDkvBN = 128;   // key rows per dK/dV workgroup
#ifndef ATTN_DQ_PD
#define ATTN_DQ_PD 6
#endif
constexpr int kDqWaves = 8;              // waves per dQ workgroup (32 queries each)
constexpr int kDqBM = 32 * kDqWaves;     // query rows per dQ workgroup
constexpr int kDqBN = 64;     // key rows per iteration of the dQ kernel

// ---------------------------------------------------------------------------
// dK / dV: one workgroup per (128-key block, KV head, sequence), looping over
// the query blocks (and, for GQA, over the query heads of the KV head).
//   wave w: key rows 32*(w&3) .. +32 of the block; query half (w>>2) of each
//   64-query tile for S = Q K^T and dP = dO V^T; head-dim half (w>>2) for
//   dV += P^T dO and dK += dS^T Q.
// LDS (D = 128): two stages of {Q, dO, LSE, Delta} (2 x 32.5 KiB, swizzled,
// filled by direct global->LDS loads one tile ahead) + the P/dS exchange
// (8 x 4 KiB).
// ---------------------------------------------------------------------------
template <bool BF16, int D, bool CAUSAL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bwd_dkdv_kernel(Args a) {
  constexpr int BM = kDkvBM, BN = kDkvBN;
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int RB = D * 2;                  // bytes per row
  constexpr int TILE = BM * RB;
  constexpr int STAGE = 2 * TILE + 2 * BM * 4;
  constexpr int TD = D / 32;                 // head-dim tiles
  constexpr int TDH = TD / 2;                // head-dim tiles per half
  constexpr int QI = BM * CPR / 512;         // direct loads per wave per Q (or dO) tile
  constexpr int XB = 4 * 16 * 64;            // exchange bytes per wave
  static_assert(TDH >= 1 && QI >= 1, "head dim of 64 or 128");

  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STAGE + 8 * XB];
  const uint32_t smem_lds = lds_addr(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = wave_id();
  const int kvg = w & 3;          // key-row group of this wave
  const int half = w >> 2;        // query half (S, dP) and head-dim half (dV, dK)
  const int h = lane >> 5;
  const int c32 = lane & 31;
  const int sl = lane & 15;
  const int gg = lane >> 4;
  const int rr = sl >> 2;
  const int tcol = 16 * (gg & 1) + 4 * (sl & 3);
  // grid (KV head x sequence, key block): every (head, sequence) pair's
  // blocks of one index go out together, longest (first key block, when
  // causal) first; the blocks of one pair share an XCD and its L2.
  const int nb = blockIdx.y;
  const int g = blockIdx.x % a.heads_kv;
  const int z = blockIdx.x / a.heads_kv;
  const Seq s = seq_info(a, z);
  const int kv0 = nb * BN;
  if (kv0 >= s.sk) return;
  const int hd = a.head_dim;
  const int off_causal = s.sk - s.sq;  // key j visible to query i iff j <= i + off_causal
  const int rows_k = min(BN, s.sk - kv0);

  // ---- K, V of this wave's 32 key rows as B operands of S = Q K^T and
  // dP = dO V^T (column = key, k = head dim).  Rows past the end read as 0.
  u32x4 kf[D / 16], vf[D / 16];
  {
    const uint16_t* kb = a.k + s.bk * a.k_b + (int64_t)(s.k0 + kv0) * a.k_r + (int64_t)g * a.k_h;
    const uint16_t* vb = a.v + s.bk * a.v_b + (int64_t)(s.k0 + kv0) * a.v_r + (int64_t)g * a.v_h;
    const rsrc_t rK = make_rsrc(kb, ((int64_t)(rows_k - 1) * a.k_r + hd) * 2);
    const rsrc_t rV = make_rsrc(vb, ((int64_t)(rows_k - 1) * a.v_r + hd) * 2);
    const int row = 32 * kvg + c32;
#pragma unroll
    for (int sd = 0; sd < D / 16; ++sd) {
      const int d0 = 16 * sd + 8 * h;
      const bool ok = d0 < hd;
      kf[sd] = buf_load128(rK, ok ? (row * (int)a.k_r + d0) * 2 : kOffOOB);
      vf[sd] = buf_load128(rV, ok ? (row * (int)a.v_r + d0) * 2 : kOffOOB);
    }
  }

  f32x16 dk_acc[TDH], dv_acc[TDH];
#pragma unroll
  for (int t = 0; t < TDH; ++t) {
    dk_acc[t] = f32x16{};
    dv_acc[t] = f32x16{};
  }

  // ---- Per-lane LDS byte offsets (swizzle folded in; rows modulo 16).
  int sv[D / 16];  // S/dP A operand: row 32*half + c32, columns 16*sd + 8*h
#pragma unroll
  for (int sd = 0; sd < D / 16; ++sd) sv[sd] = 32 * half * RB + tile_off<CPR>(c32, 16 * sd + 8 * h);
  int ta[TDH], tb[TDH];  // dV/dK B operand: rows 4*h + rr (+8), columns of this wave's head-dim tiles
#pragma unroll
  for (int t = 0; t < TDH; ++t) {
    const int col = 32 * (TDH * half + t) + tcol;
    ta[t] = tile_off<CPR>(4 * h + rr, col);
    tb[t] = tile_off<CPR>(4 * h + rr + 8, col);
  }
  uint8_t* const xown = smem + 2 * STAGE + w * XB + lane * 16;
  const uint8_t* const xpar = smem + 2 * STAGE + (w ^ 4) * XB + lane * 16;

  auto slot_off = [&](int S, int row_stride) {
    const int r = S / CPR;
    const int c = (S % CPR) ^ swz<CPR>(r);
    return 8 * c < hd ? (r * row_stride + 8 * c) * 2 : kOffOOB;
  };
  int qdma[QI], dodma[QI];
#pragma unroll
  for (int i = 0; i < QI; ++i) {
    const int S = (i * 8 + w) * 64 + lane;
    qdma[i] = slot_off(S, (int)a.q_r);
    dodma[i] = slot_off(S, (int)a.do_r);
  }

  const int m_begin = first_q_block<BM, BN, CAUSAL>(nb, s.sq, s.sk);
  const int m_end = (s.sq + BM - 1) / BM;
  const int kv_lane = kv0 + 32 * kvg + c32;  // this lane's key column in S / dP

  for (int hq = g * a.group; hq < (g + 1) * a.group; ++hq) {
    if (m_begin >= m_end) break;
    const uint16_t* qb = a.q + s.bq * a.q_b + (int64_t)s.q0 * a.q_r + (int64_t)hq * a.q_h;
    const uint16_t* db = a.dout + s.bq * a.do_b + (int64_t)s.q0 * a.do_r + (int64_t)hq * a.do_h;
    const int64_t st0 = s.stat0 + (int64_t)hq * s.stat_h;

    // Tile m into stage `st`: Q, dO, LSE, Delta.  Rows past the end read as 0;
    // their P and dS then contribute nothing (Q = dO = 0).
    auto prefetch = [&](int m, int st) {
      const int rows = min(BM, s.sq - m * BM);
      const uint32_t stage = smem_lds + st * STAGE;
      const u32x4 srdQ = make_srd(qb + (int64_t)m * BM * a.q_r, ((int64_t)(rows - 1) * a.q_r + hd) * 2);
      const u32x4 srdO = make_srd(db + (int64_t)m * BM * a.do_r, ((int64_t)(rows - 1) * a.do_r + hd) * 2);
#pragma unroll
      for (int i = 0; i < QI; ++i) {
        const int S0 = (i * 8 + w) * 64;
        dma16(srdQ, qdma[i], stage + S0 * 16);
        dma16(srdO, dodma[i], stage + TILE + S0 * 16);
      }
      if (w == 0) {
        dma4(make_srd(a.lse_in + st0 + m * BM, (int64_t)rows * 4), lane * 4, stage + 2 * TILE);
      } else if (w == 1) {
        dma4(make_srd(a.delta + st0 + m * BM, (int64_t)rows * 4), lane * 4, stage + 2 * TILE + BM * 4);
      }
    };

    // Before refilling stage 0 for a new head, every wave must be done with
    // the previous head's last tile.
    if (hq != g * a.group) lds_barrier();
    prefetch(m_begin, 0);
    for (int m = m_begin; m < m_end; ++m) {
      const int st = (m - m_begin) & 1;
      wait_vmcnt<0>();  // this wave's loads of tile m
      lds_barrier();    // everyone's loads; all reads of the other stage retired
      if (m + 1 < m_end) prefetch(m + 1, st ^ 1);

      const uint8_t* sQ = smem + st * STAGE;
      const uint8_t* sdO = sQ + TILE;
      const float* sL = reinterpret_cast<const float*>(sQ + 2 * TILE);
      const float* sDl = sL + BM;

      // LSE / Delta of this lane's 16 query rows.
      f32x4 Lr[4], Dr[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int qr = 32 * half + 8 * jj + 4 * h;
        Lr[jj] = *reinterpret_cast<const f32x4*>(sL + qr);
        Dr[jj] = *reinterpret_cast<const f32x4*>(sDl + qr);
      }

      // S = Q K^T and dP = dO V^T: 32 queries (this wave's half) x 32 keys.
      f32x16 sacc = f32x16{}, pacc = f32x16{};
      {
        constexpr int NS = D / 16, PD = 3;
        u32x4 fq[PD], fo[PD];
        auto rd = [&](int sd, int slot) {
          fq[slot] = lds_rd128(sQ, sv[sd]);
          fo[slot] = lds_rd128(sdO, sv[sd]);
        };
        sched_fence();
#pragma unroll
        for (int i = 0; i < PD; ++i) rd(i, i);
        sched_fence();
#pragma unroll
        for (int sd = 0; sd < NS; ++sd) {
          const u32x4 a0 = fq[sd % PD], a1 = fo[sd % PD];
          if (sd + PD < NS) rd(sd + PD, sd % PD);
          sacc = mfma32<BF16>(a0, kf[sd], sacc);
          pacc = mfma32<BF16>(a1, vf[sd], pacc);
          sched_fence();
        }
      }

      // P and dS.  C layout: lane = key column kv_lane, rows = queries
      // 32*half + 8*(j/4) + 4*h + j%4.  Tiles crossing the causal diagonal and
      // the partial last key block are masked (zero-filled key rows would
      // otherwise give P = exp(-LSE), which could overflow a 16-bit dS).
      const bool masked = (CAUSAL && (kv0 + BN - 1 > m * BM + off_causal)) || rows_k < BN;
      auto elementwise = [&](auto mask) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int j = 4 * jj + r;
            float p = fast_exp2(__builtin_fmaf(sacc[j], a.scale_log2, -Lr[jj][r] * kLog2e));
            if constexpr (decltype(mask)::value) {
              const int qi = m * BM + 32 * half + 8 * jj + 4 * h + r;
              bool vis = kv_lane < kv0 + rows_k;
              if (CAUSAL) vis = vis && (kv_lane <= qi + off_causal);
              p = vis ? p : 0.f;
            }
            sacc[j] = p;
            pacc[j] = p * (pacc[j] - Dr[jj][r]);
          }
        }
      };
      if (masked) {
        elementwise(std::true_type{});
      } else {
        elementwise(std::false_type{});
      }

      // P^T and dS^T as A operands (row = key, k = query): k-slot i of 16-query
      // step s2 is query 16*s2 + 8*(i/4) + 4*h + i%4 of this wave's half.
      u32x4 pf[2], dsf[2];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pf[s2][e] = pack2<BF16>(sacc[8 * s2 + 2 * e], sacc[8 * s2 + 2 * e + 1]);
          dsf[s2][e] = pack2<BF16>(pacc[8 * s2 + 2 * e], pacc[8 * s2 + 2 * e + 1]);
        }
      }
      // Trade with the partner wave (same keys, other query half).
      *reinterpret_cast<u32x4*>(xown + 0 * 1024) = pf[0];
      *reinterpret_cast<u32x4*>(xown + 1 * 1024) = pf[1];
      *reinterpret_cast<u32x4*>(xown + 2 * 1024) = dsf[0];
      *reinterpret_cast<u32x4*>(xown + 3 * 1024) = dsf[1];
      lds_barrier();
      u32x4 ppf[2], pdsf[2];
      ppf[0] = *reinterpret_cast<const u32x4*>(xpar + 0 * 1024);
      ppf[1] = *reinterpret_cast<const u32x4*>(xpar + 1 * 1024);
      pdsf[0] = *reinterpret_cast<const u32x4*>(xpar + 2 * 1024);
      pdsf[1] = *reinterpret_cast<const u32x4*>(xpar + 3 * 1024);

      // dV += P^T dO and dK += dS^T Q over all 64 queries of the tile, for
      // this wave's head-dim half.  Step = (query half qh, s2, t).
      {
        constexpr int NS = 4 * TDH, PD = 2;
        u32x4 fo[PD], fq[PD];
        auto rd = [&](int i, int slot) {
          const int kstep = i / TDH, t = i % TDH;
          const int qh = (kstep < 2) ? half : (half ^ 1);
          const int ro = (32 * qh + 16 * (kstep & 1)) * RB;
          fo[slot] = tr_frag_b(sdO, ro + ta[t], ro + tb[t]);
          fq[slot] = tr_frag_b(sQ, ro + ta[t], ro + tb[t]);
        };
        sched_fence();
#pragma unroll
        for (int i = 0; i < PD; ++i) rd(i, i);
        sched_fence();
#pragma unroll
        for (int i = 0; i < NS; ++i) {
          const int kstep = i / TDH, t = i % TDH;
          const u32x4 bo = fo[i % PD], bq = fq[i % PD];
          if (i + PD < NS) rd(i + PD, i % PD);
          const u32x4 ap = kstep < 2 ? pf[kstep] : ppf[kstep - 2];
          const u32x4 ad = kstep < 2 ? dsf[kstep] : pdsf[kstep - 2];
          dv_acc[t] = mfma32<BF16>(ap, bo, dv_acc[t]);
          dk_acc[t] = mfma32<BF16>(ad, bq, dk_acc[t]);
          sched_fence();
        }
      }
    }
  }

  // ---- Epilogue: dK * scale, dV; convert (round to nearest even) and store.
  const uint16_t* dkb = a.dk + s.bk * a.dk_b + (int64_t)(s.k0 + kv0) * a.dk_r + (int64_t)g * a.dk_h;
  const uint16_t* dvb = a.dv + s.bk * a.dv_b + (int64_t)(s.k0 + kv0) * a.dv_r + (int64_t)g * a.dv_h;
  const rsrc_t rDK = make_rsrc(dkb, ((int64_t)(rows_k - 1) * a.dk_r + hd) * 2);
  const rsrc_t rDV = make_rsrc(dvb, ((int64_t)(rows_k - 1) * a.dv_r + hd) * 2);
#pragma unroll
  for (int t = 0; t < TDH; ++t) {
    const int d = 32 * (TDH * half + t) + c32;
    const bool ok = d < hd;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int kr = 32 * kvg + 8 * (j >> 2) + 4 * h + (j & 3);
      buf_store_u16(rDK, ok ? (kr * (int)a.dk_r + d) * 2 : kOffOOB, to_bits<BF16>(dk_acc[t][j] * a.scale));
      buf_store_u16(rDV, ok ? (kr * (int)a.dv_r + d) * 2 : kOffOOB, to_bits<BF16>(dv_acc[t][j]));
    }
  }
}

// Compile-time iteration: f(integral_constant<int, B>), ..., f(<E-1>).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Slot layout of one key tile of the dQ kernel and where each softmax
// element's three dependent stages (F, E, M) go.  Slots:
//   [0, SB)   A: S, dP of key half 0 (alternating, head-dim step = slot/2)
//   [SB, SC)  B: dQ += dS K of the previous tile's half 1
//   [SC, SD)  C: S, dP of key half 1
//   [SD, N)   D: dQ += dS K of half 0
// The softmax of half 0 runs during B (the matrix core is then busy with
// the previous tile's dQ, which needs no score registers), that of half 1
// during D; element e's stages sit in slots f, f+1, f+2, so every vector
// instruction reads a value produced one slot earlier.  Stages of half 1
// that fall past the end of the tile run at the start of the next tile's A.
template <int NSD, int TD>
struct DqSchedule {
  static constexpr int SB = 2 * NSD, SC = SB + 2 * TD, SD = SC + 2 * NSD, NSLOT = SD + 2 * TD;
  // element e's first stage; the chain of the last element ends in the
  // last dQ slot of the phase
  static constexpr int spread(int e, int lo, int len) { return lo + (e * (len - 2)) / 16; }
  static constexpr bool is_sdp(int i) { return i < SB || (i >= SC && i < SD); }
  static constexpr bool active(int i, bool first, bool drain) {
    return (i >= SB && i < SC) ? !first : !drain;
  }
  static constexpr int rank(int i, bool first, bool drain) {
    int r = 0;
    for (int k = 0; k < i; ++k) r += active(k, first, drain) ? 1 : 0;
    return r;
  }
  static constexpr int nact(bool first, bool drain) { return rank(NSLOT, first, drain); }
  static constexpr int kth(int k, bool first, bool drain) {
    for (int i = 0; i < NSLOT; ++i)
      if (active(i, first, drain) && rank(i, first, drain) == k) return i;
    return -1;
  }
  static constexpr int fslot_h0(int e) { return spread(e, SB, 2 * TD); }
  static constexpr int fslot_h1(int e) { return spread(e, SD, 2 * TD); }
  static_assert(fslot_h0(15) + 2 < SC, "half 0 must be packed within B");
  static_assert(fslot_h1(15) + 2 < NSLOT, "half 1 must be packed within D");
};

// ---------------------------------------------------------------------------
// dQ: one workgroup per (256-query block, query head, sequence), looping over
// the 64-key tiles it sees in ascending order.  Wave w owns query rows
// 32*w .. +32 and works each key tile alone, as two 32-key halves:
//   S^T = K Q^T and dP^T = V dO^T, P^T = exp2(S^T*scale*log2e - LSE*log2e), dS^T = P^T o (dP^T - Delta),
//   dQ += dS K over the full head dim.
// The transposed score tile puts one query per lane (its column), so LSE and
// Delta are per-lane constants, and dS^T leaves the MFMA in the A-operand
// layout of dQ = dS K.
//
// Schedule.  The matrix-core work of one tile is a stream of slots
//   A: S, dP of half 0      B: dQ of the previous tile's half 1
//   C: S, dP of half 1      D: dQ of half 0
// and the softmax of each half runs in the slots after its S/dP, spread so
// that every vector instruction's input was produced at least one slot
// earlier (no dependency stalls) and the vector work hides under the matrix
// core: half 0 during B and C, half 1 during D and the next tile's A.  The
// K tile of the previous key tile is still needed in B, hence three LDS
// stages.
// LDS (D = 128): three stages of {K, V} (3 x 32 KiB), filled by direct
// global->LDS loads one tile ahead.
// ---------------------------------------------------------------------------
template <bool BF16, int D, bool CAUSAL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bwd_dq_kernel(Args a) {
  constexpr int NW = 8;
  constexpr int BM = kDqBM, BN = kDqBN;
  constexpr int CPR = D / 8;
  constexpr int RB = D * 2;
  constexpr int KT = BN * RB;                // bytes of a K (or V) tile
  constexpr int STAGE = 2 * KT;
  constexpr int NSTAGE = 3;
  constexpr int TD = D / 32;                 // head-dim tiles of dQ
  constexpr int NSD = D / 16;                // k-steps of S^T / dP^T
  constexpr int KI = BN * CPR / (64 * NW);   // direct loads per wave per K (or V) tile
  static_assert(TD >= 2 && KI >= 1, "head dim of 64 or 128");
  static_assert(BM == 32 * NW && BN == 64, "32 queries per wave, two 32-key halves");

  __shared__ __attribute__((aligned(1024))) uint8_t smem[NSTAGE * STAGE];
  const uint32_t smem_lds = lds_addr(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = wave_id();
  const int h = lane >> 5;
  const int c32 = lane & 31;
  const int sl = lane & 15;
  const int gg = lane >> 4;
  const int rr = sl >> 2;
  const int tcol = 16 * (gg & 1) + 4 * (sl & 3);
  // grid (query head x sequence, query block), as in the dK/dV kernel.
  const int hq = blockIdx.x % a.heads_q;
  const int z = blockIdx.x / a.heads_q;
  const Seq s = seq_info(a, z);
  // Causal blocks near the end of a sequence see the most keys: run them first.
  const int mb = CAUSAL ? (int)(gridDim.y - 1 - blockIdx.y) : (int)blockIdx.y;
  const int q0 = mb * BM;
  if (q0 >= s.sq) return;
  const int hd = a.head_dim;
  const int g = hq / a.group;
  const int off_causal = s.sk - s.sq;
  const int qw = q0 + 32 * w;         // first query of this wave
  const int qi = qw + c32;            // this lane's query (a column of S^T)

  // ---- Q and dO of this lane's query as B operands (k = head dim); LSE and
  // Delta of that query.  Rows past the end read as 0.
  u32x4 qf[NSD], df[NSD];
  float L2, Dl;
  {
    const int rows = min(BM, s.sq - q0);
    const uint16_t* qb = a.q + s.bq * a.q_b + (int64_t)(s.q0 + q0) * a.q_r + (int64_t)hq * a.q_h;
    const uint16_t* db = a.dout + s.bq * a.do_b + (int64_t)(s.q0 + q0) * a.do_r + (int64_t)hq * a.do_h;
    const rsrc_t rQ = make_rsrc(qb, ((int64_t)(rows - 1) * a.q_r + hd) * 2);
    const rsrc_t rO = make_rsrc(db, ((int64_t)(rows - 1) * a.do_r + hd) * 2);
    const int row = 32 * w + c32;
#pragma unroll
    for (int sd = 0; sd < NSD; ++sd) {
      const int d0 = 16 * sd + 8 * h;
      const bool ok = d0 < hd;
      qf[sd] = buf_load128(rQ, ok ? (row * (int)a.q_r + d0) * 2 : kOffOOB);
      df[sd] = buf_load128(rO, ok ? (row * (int)a.do_r + d0) * 2 : kOffOOB);
    }
    const int64_t st0 = s.stat0 + (int64_t)hq * s.stat_h + q0;
    L2 = buf_load_f32(make_rsrc(a.lse_in + st0, (int64_t)rows * 4), row * 4) * kLog2e;
    Dl = buf_load_f32(make_rsrc(a.delta + st0, (int64_t)rows * 4), row * 4);
  }

  f32x16 dq_acc[TD];
#pragma unroll
  for (int t = 0; t < TD; ++t) dq_acc[t] = f32x16{};

  // Per-lane LDS offsets, as XOR bases (the swizzle only permutes the chunk
  // bits, so the offset of head-dim step sd is base ^ 32*sd, of dQ tile t
  // base ^ 64*t).  S^T/dP^T A operand: key row c32 of a half, columns
  // 16*sd + 8*h.  dQ B operand (K, transpose read): key rows 4*h + rr (+8)
  // of a 16-key step, columns 32*t + tcol.
  const int svb = tile_off<CPR>(c32, 8 * h);
  const int tab = tile_off<CPR>(4 * h + rr, tcol);
  const int tbb = tile_off<CPR>(4 * h + rr + 8, tcol);

  auto slot_off = [&](int S, int row_stride) {
    const int r = S / CPR;
    const int c = (S % CPR) ^ swz<CPR>(r);
    return 8 * c < hd ? (r * row_stride + 8 * c) * 2 : kOffOOB;
  };
  int kdma[KI], vdma[KI];
#pragma unroll
  for (int i = 0; i < KI; ++i) {
    const int S = (i * NW + w) * 64 + lane;
    kdma[i] = slot_off(S, (int)a.k_r);
    vdma[i] = slot_off(S, (int)a.v_r);
  }

  // Key tiles this query block sees.
  int n_end = (s.sk + BN - 1) / BN;
  if (CAUSAL) {
    const int q_last = min(q0 + BM, s.sq) - 1;
    const int k_lim = q_last + off_causal;
    n_end = k_lim < 0 ? 0 : min(n_end, k_lim / BN + 1);
  }
  const uint16_t* kbase = a.k + s.bk * a.k_b + (int64_t)s.k0 * a.k_r + (int64_t)g * a.k_h;
  const uint16_t* vbase = a.v + s.bk * a.v_b + (int64_t)s.k0 * a.v_r + (int64_t)g * a.v_h;

  auto prefetch = [&](int n) {
    const int rows = min(BN, s.sk - n * BN);
    const uint32_t stage = smem_lds + (n % NSTAGE) * STAGE;
    const u32x4 srdK = make_srd(kbase + (int64_t)n * BN * a.k_r, ((int64_t)(rows - 1) * a.k_r + hd) * 2);
    const u32x4 srdV = make_srd(vbase + (int64_t)n * BN * a.v_r, ((int64_t)(rows - 1) * a.v_r + hd) * 2);
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int S0 = (i * NW + w) * 64;
      dma16(srdK, kdma[i], stage + S0 * 16);
      dma16(srdV, vdma[i], stage + KT + S0 * 16);
    }
  };
  auto tile_masked = [&](int n) {
    return (CAUSAL && (n * BN + BN - 1 > qw + off_causal)) || (n * BN + BN > s.sk);
  };

  // Last key this lane's query sees, minus the lane's row offset 4*h in the
  // C layout (keys past the end or above the diagonal are masked).
  int kv_lim = s.sk - 1;
  if (CAUSAL) kv_lim = min(kv_lim, qi + off_causal);
  kv_lim -= 4 * h;

  // Softmax state: sc/pc = current tile's S^T and (dP^T - Delta) per half;
  // the previous tile's half 1 lives in sp/pp until its dS is packed.
  f32x16 sc0, pc0, sc1, pc1, sp, pp;
  u32x4 ds0[2], ds1[2], dsp[2];
  int n_prev = 0;  // key tile whose half 1 is still pending

  // Elementwise stages on element j of a score/grad pair of key half kh of
  // key tile m.  F: scaled score (masked to -inf), E: exp2, M: dS, packed.
  auto stageF = [&](f32x16& sv, auto jc, int m, int kh, auto mask) {
    constexpr int j = decltype(jc)::value;
    float t = __builtin_fmaf(sv[j], a.scale_log2, -L2);
    if constexpr (decltype(mask)::value) {
      // key m*BN + 32*kh + 8*(j/4) + 4*h + j%4: the wave-uniform part
      // against this lane's limit
      const int ks = m * BN + 32 * kh + 8 * (j >> 2) + (j & 3);
      t = ks <= kv_lim ? t : -__builtin_inff();
    }
    sv[j] = t;
  };
  auto stageE = [&](f32x16& sv, auto jc) {
    constexpr int j = decltype(jc)::value;
    sv[j] = fast_exp2(sv[j]);
  };
  auto stageM = [&](f32x16& sv, f32x16& pv, u32x4* dsv, auto jc) {
    constexpr int j = decltype(jc)::value;
    pv[j] = sv[j] * (pv[j] - Dl);
    // dS as the A operand of dQ = dS K (row = query, k = key): k-slot e of
    // 16-key step s2 is key 16*s2 + 8*(e/4) + 4*h + e%4 of the half.
    if constexpr (j & 1) dsv[j >> 3][(j & 7) >> 1] = pack2<BF16>(pv[j - 1], pv[j]);
  };

  using Sch = DqSchedule<NSD, TD>;
  // One tile: FIRST = no previous tile; DRAIN = only finish the previous
  // tile's half 1 (this wave sees no more keys).
  auto run = [&](int n, auto first_t, auto drain_t, auto mask) {
    constexpr bool FIRST = decltype(first_t)::value;
    constexpr bool DRAIN = decltype(drain_t)::value;
    constexpr int NACT = Sch::nact(FIRST, DRAIN);
    constexpr int PD = ATTN_DQ_PD;  // LDS operand reads in flight ahead of their MFMA
    // loop-variant bases so the per-step XORs are not hoisted out of the loop
    const int svn = svb + (n % NSTAGE) * STAGE;
    const int tan = tab + (n % NSTAGE) * STAGE, tbn = tbb + (n % NSTAGE) * STAGE;
    const int tap = tab + (n_prev % NSTAGE) * STAGE, tbp = tbb + (n_prev % NSTAGE) * STAGE;
    if constexpr (!DRAIN) {
      sc0 = f32x16{};
      pc0 = f32x16{};
    }
    u32x4 buf[PD];
    auto rd = [&](auto kc) {  // LDS operand of the k-th active slot
      constexpr int k = decltype(kc)::value;
      constexpr int i = Sch::kth(k, FIRST, DRAIN);
      if constexpr (Sch::is_sdp(i)) {
        constexpr int kh = i < Sch::SB ? 0 : 1, kq = i < Sch::SB ? i : i - Sch::SC, sd = kq / 2;
        buf[k % PD] = lds_rd128(smem, (svn ^ (32 * sd)) + kh * 32 * RB + ((kq & 1) ? KT : 0));
      } else {
        constexpr bool prev = i < Sch::SC;
        constexpr int kq = prev ? i - Sch::SB : i - Sch::SD, s2 = kq / TD, t = kq % TD;
        constexpr int ro = (32 * (prev ? 1 : 0) + 16 * s2) * RB;
        if constexpr (prev) {
          buf[k % PD] = tr_frag_b(smem, (tap ^ (64 * t)) + ro, (tbp ^ (64 * t)) + ro);
        } else {
          buf[k % PD] = tr_frag_b(smem, (tan ^ (64 * t)) + ro, (tbn ^ (64 * t)) + ro);
        }
      }
    };
    sched_fence();
    static_for<0, (PD < NACT ? PD : NACT)>(rd);
    sched_fence();
    static_for<0, Sch::NSLOT>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if constexpr (i == Sch::SC && !DRAIN) {  // half 1 accumulators start here
        sc1 = f32x16{};
        pc1 = f32x16{};
      }
      if constexpr (Sch::active(i, FIRST, DRAIN)) {
        constexpr int k = Sch::rank(i, FIRST, DRAIN);
        const u32x4 op = buf[k % PD];
        if constexpr (k + PD < NACT) rd(std::integral_constant<int, k + PD>{});
        if constexpr (Sch::is_sdp(i)) {
          constexpr int kq = i < Sch::SB ? i : i - Sch::SC, sd = kq / 2;
          if constexpr (i < Sch::SB) {
            if constexpr (kq & 1) pc0 = mfma32<BF16>(op, df[sd], pc0);
            else sc0 = mfma32<BF16>(op, qf[sd], sc0);
          } else {
            if constexpr (kq & 1) pc1 = mfma32<BF16>(op, df[sd], pc1);
            else sc1 = mfma32<BF16>(op, qf[sd], sc1);
          }
        } else if constexpr (i < Sch::SC) {
          constexpr int kq = i - Sch::SB, s2 = kq / TD, t = kq % TD;
          dq_acc[t] = mfma32<BF16>(dsp[s2], op, dq_acc[t]);
        } else {
          constexpr int kq = i - Sch::SD, s2 = kq / TD, t = kq % TD;
          dq_acc[t] = mfma32<BF16>(ds0[s2], op, dq_acc[t]);
        }
      }
      // softmax stages placed after this slot's matrix-core instruction
      static_for<0, 16>([&](auto ec) {
        constexpr int e = decltype(ec)::value;
        constexpr int f0 = Sch::fslot_h0(e), f1 = Sch::fslot_h1(e);
        if constexpr (!DRAIN) {  // half 0 of this tile
          if constexpr (i == f0) stageF(sc0, ec, n, 0, mask);
          if constexpr (i == f0 + 1) stageE(sc0, ec);
          if constexpr (i == f0 + 2) stageM(sc0, pc0, ds0, ec);
          // half 1 of this tile
          if constexpr (i == f1) stageF(sc1, ec, n, 1, mask);
          if constexpr (i == f1 + 1) stageE(sc1, ec);
          if constexpr (i == f1 + 2) stageM(sc1, pc1, ds1, ec);
        }
        if constexpr (!FIRST) {  // stages of the previous tile's half 1 that spilled over
          if constexpr (i == f1 - Sch::NSLOT) stageF(sp, ec, n_prev, 1, mask);
          if constexpr (i == f1 + 1 - Sch::NSLOT) stageE(sp, ec);
          if constexpr (i == f1 + 2 - Sch::NSLOT) stageM(sp, pp, dsp, ec);
        }
      });
      sched_fence();
    });
    if constexpr (!DRAIN) {
      sp = sc1;
      pp = pc1;
      dsp[0] = ds1[0];
      dsp[1] = ds1[1];
      n_prev = n;
    }
  };

  // Tile loop.  The first tile is peeled (no previous half 1), the tiles
  // that need no mask run in one loop and the masked ones (the diagonal, the
  // ragged last tile) in a second, so the matrix-core accumulators flow
  // through straight loops rather than branches.  A wave keeps running
  // masked tiles past its own last visible key (they add exact zeros) until
  // the block's last tile, so every wave takes the same barriers.
  if (n_end > 0) {
    prefetch(0);
    wait_vmcnt<0>();
    lds_barrier();
    if (1 < n_end) prefetch(1);
    if (tile_masked(0)) {
      run(0, std::true_type{}, std::false_type{}, std::true_type{});
    } else {
      run(0, std::true_type{}, std::false_type{}, std::false_type{});
    }
    int n_um = n_end;  // first tile of this wave that needs the mask
    if (CAUSAL) {
      const int lo = qw + off_causal - (BN - 1);  // tiles n with n*BN + BN-1 <= qw + off need none
      n_um = lo < 0 ? 0 : min(n_um, lo / BN + 1);
    }
    n_um = min(n_um, s.sk / BN);
    n_um = max(n_um, 1);
    int n = 1;
    for (; n < n_um; ++n) {
      wait_vmcnt<0>();
      lds_barrier();
      if (n + 1 < n_end) prefetch(n + 1);
      run(n, std::false_type{}, std::false_type{}, std::false_type{});
    }
    for (; n < n_end; ++n) {
      wait_vmcnt<0>();
      lds_barrier();
      if (n + 1 < n_end) prefetch(n + 1);
      run(n, std::false_type{}, std::false_type{}, std::true_type{});
    }
    run(n_end, std::false_type{}, std::true_type{}, std::false_type{});
  }

  // ---- dQ * scale, converted (round to nearest even).  C layout: lane =
  // head-dim column, rows = queries 32*w + 8*(j/4) + 4*h + j%4.
  {
    const int rows = min(BM, s.sq - q0);
    const uint16_t* dqb = a.dq + s.bq * a.dq_b + (int64_t)(s.q0 + q0) * a.dq_r + (int64_t)hq * a.dq_h;
    const rsrc_t rDQ = make_rsrc(dqb, ((int64_t)(rows - 1) * a.dq_r + hd) * 2);
#pragma unroll
    for (int t = 0; t < TD; ++t) {
      const int d = 32 * t + c32;
      const bool ok = d < hd;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int qr = 32 * w + 8 * (j >> 2) + 4 * h + (j & 3);
        buf_store_u16(rDQ, ok ? (qr * (int)a.dq_r + d) * 2 : kOffOOB, to_bits<BF16>(dq_acc[t][j] * a.scale));
      }
    }
  }
}

}  // namespace attn
