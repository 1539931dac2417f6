// Attention backward on gfx950: preprocess, KV-stationary main kernel and dQ
// postprocess.
//
// The method (tilelang test_tilelang_kernel_mha_bwd.py, flashattn_bwd and its
// preprocess/postprocess; Hopper flash_bwd_launch_template.h, run_flash_bwd):
//   preprocess  Delta_i = sum_d O_id dO_id (fp32); the fp32 dQ accumulator is
//               cleared (the Hopper launcher's Clear_dQaccum preprocess).
//   main        one workgroup per key/value block, looping over query blocks:
//               S = Q K^T, P = exp2(S*scale*log2e - LSE*log2e) recomputed from
//               the saved LSE, dP = dO V^T, dS = P o (dP - Delta),
//               dV += P^T dO, dK += dS^T Q, dQ += dS K (accumulated across
//               workgroups in fp32).  Causal blocks above the diagonal are
//               skipped by starting the query loop at the first block that
//               sees this key block.
//   postprocess dQ = scale * accumulator, converted to fp16/bf16 (the Hopper
//               launcher's ConvertdQ postprocess scaled by scale_softmax).
// dS is kept unscaled; dK is multiplied by the softmax scale in the main
// kernel's epilogue and dQ in the postprocess (the tilelang kernel scales dS
// instead -- the same product).
//
// gfx950 design of the main kernel (not the pages'):
//   * 4 wave64s; wave w owns key rows [32w, 32w+32) of the 128-row key block,
//     so its dK and dV accumulators (32 x d fp32 each) never leave registers,
//     and K and V of those rows sit in registers as MFMA operands.
//   * S and dP are computed as [query x key] tiles; their C layout (lane =
//     key column, 16 query rows per lane) is exactly the operand layout the
//     dV and dK contractions (reduction over queries) need, so P and dS feed
//     the matrix cores without leaving registers.
//   * The other operand of those contractions (dO, Q with the query index as
//     k) is read from the row-major LDS tiles with the LDS transpose read;
//     no transposed copies are stored.
//   * dS goes through LDS once, stored [key][query], for dQ = dS K, whose
//     reduction runs over all 128 keys of the block (all four waves' rows);
//     each wave computes a 32-column slice of dQ and adds it to the fp32
//     accumulator with global float atomics, or, in deterministic mode,
//     stores it to this key block's own accumulator slice (the CK
//     mha_bwd.cpp page's split dq_accum), summed in ascending key-block order
//     by the postprocess.
//   * GQA: the workgroup loops over the query heads of its KV head, so dK/dV
//     come out already summed over the group (the CK page instead expands
//     dK/dV per query head and sums afterwards).
//   * The next Q/dO tile is prefetched into registers during the current one.
#pragma once

#include <type_traits>

#include "attn_device.h"

namespace attn {

constexpr int kBwdBM = 64;   // query rows per iteration of the main kernel
constexpr int kBwdBN = 128;  // key rows per main-kernel workgroup
constexpr int kPreRows = 64; // rows per preprocess / postprocess workgroup (= kBwdBM)

// ---------------------------------------------------------------------------
// Preprocess: Delta = rowsum(O o dO) in fp32, and (atomic mode) a cleared dQ
// accumulator.  16 lanes per row, 16 rows per pass.
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(256) void attn_bwd_pre_kernel(Args a, int clear_acc) {
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
      a.delta[st0 + r] = acc;
      if (a.delta_out) a.delta_out[st0 + r] = acc;
    }
  }
  if (clear_acc) {
    float* accp = a.dq_acc + acc_base(a, s, hq);
    const int rows = min(kPreRows, s.sq - r0);
    const int n4 = rows * hd / 4;
    float4* p4 = reinterpret_cast<float4*>(accp + (int64_t)r0 * hd);
    for (int i = tid; i < n4; i += 256) p4[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

// ---------------------------------------------------------------------------
// Main kernel.
//
// LDS (D = 128): two stages of {Q tile, dO tile, LSE, Delta} (2 x 32.5 KiB)
// and the dS^T tile (16 KiB).  All tiles are row-major with XOR-swizzled
// 16-byte chunks (swz<>), filled by direct global->LDS loads one iteration
// ahead.  The K block is staged once through the second stage to build this
// wave's K fragments for the dQ contraction, which then stay in registers.
// ---------------------------------------------------------------------------
template <bool BF16, int D, bool CAUSAL, bool DET>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_bwd_main_kernel(Args a) {
  constexpr int BM = kBwdBM, BN = kBwdBN;
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int RB = D * 2;                  // bytes per row
  constexpr int TILE = BM * RB;              // bytes of a Q (or dO) tile
  constexpr int STAGE = 2 * TILE + 2 * BM * 4;
  constexpr int DCPR = BM / 8;               // chunks per dS^T row (64 queries)
  constexpr int DRB = BM * 2;
  constexpr int TD = D / 32;                 // head-dim tiles
  constexpr int TQ = BM / 32;                // query sub-tiles per iteration
  constexpr int DQ_TQ = TQ * TD / 4;         // query tiles per wave in the dQ step
  constexpr int QI = BM * CPR / 256;         // direct loads per wave per Q (or dO) tile
  constexpr int KI = BN * CPR / 256;         // ... per K block
  constexpr int NATOM = DQ_TQ * 16;          // vector-memory ops per iteration after the prefetch
  static_assert(TQ * TD % 4 == 0 && DQ_TQ >= 1, "dQ tiles must split over 4 waves");
  static_assert(BN * RB <= STAGE, "the K block is staged in one stage buffer");
  static_assert(DCPR == 8, "dS^T rows of 128 bytes");

  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STAGE + BN * DRB];
  uint8_t* const sdST = smem + 2 * STAGE;
  const uint32_t smem_lds = lds_addr(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = wave_id();
  const int h = lane >> 5;
  const int c32 = lane & 31;
  const int sl = lane & 15;      // lane within its 16-lane group
  const int gg = lane >> 4;      // 16-lane group
  const int rr = sl >> 2;
  const int tcol = 16 * (gg & 1) + 4 * (sl & 3);  // transpose-read column within a 32-column block
  const int nb = blockIdx.x;
  const int g = blockIdx.y;
  const int z = blockIdx.z;
  const Seq s = seq_info(a, z);
  const int kv0 = nb * BN;
  if (kv0 >= s.sk) return;
  const int hd = a.head_dim;
  const int off_causal = s.sk - s.sq;  // key j visible to query i iff j <= i + off_causal

  const int rows_k = min(BN, s.sk - kv0);
  const uint16_t* kb = a.k + s.bk * a.k_b + (int64_t)(s.k0 + kv0) * a.k_r + (int64_t)g * a.k_h;
  const uint16_t* vb = a.v + s.bk * a.v_b + (int64_t)(s.k0 + kv0) * a.v_r + (int64_t)g * a.v_h;

  // Direct loads of swizzled tiles: slot S holds row S / CPR, chunk
  // (S % CPR) ^ swz(row).  Out-of-range rows/columns land as zeros.
  auto slot_off = [&](int S, int row_stride) {
    const int r = S / CPR;
    const int c = (S % CPR) ^ swz<CPR>(r);
    return 8 * c < hd ? (r * row_stride + 8 * c) * 2 : kOffOOB;
  };

  // ---- K block -> stage 1 (staging only), K and V rows of this wave -> registers.
  {
    const u32x4 srdK = make_srd(kb, ((int64_t)(rows_k - 1) * a.k_r + hd) * 2);
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int S0 = (i * 4 + w) * 64;
      dma16(srdK, slot_off(S0 + lane, (int)a.k_r), smem_lds + STAGE + S0 * 16);
    }
  }
  const rsrc_t rK = make_rsrc(kb, ((int64_t)(rows_k - 1) * a.k_r + hd) * 2);
  const rsrc_t rV = make_rsrc(vb, ((int64_t)(rows_k - 1) * a.v_r + hd) * 2);
  // K, V of this wave's 32 key rows as B operands of S = Q K^T, dP = dO V^T
  // (column = key, k = head dim).
  u32x4 kf[D / 16], vf[D / 16];
  {
    const int row = 32 * w + c32;
#pragma unroll
    for (int sd = 0; sd < D / 16; ++sd) {
      const int d0 = 16 * sd + 8 * h;
      const bool ok = d0 < hd;
      kf[sd] = buf_load128(rK, ok ? (row * (int)a.k_r + d0) * 2 : kOffOOB);
      vf[sd] = buf_load128(rV, ok ? (row * (int)a.v_r + d0) * 2 : kOffOOB);
    }
  }
  const int td_w = w % TD;            // head-dim tile of this wave in the dQ step
  const int tq_w = (w / TD) * DQ_TQ;  // first query tile of this wave in the dQ step
  // K as the B operand of dQ = dS K (k = key) for head-dim tile td_w: keys
  // 16*sk + 8*h + rr (k-slots 0..3) and + 4 (k-slots 4..7).
  u32x4 ktf[BN / 16];
  wait_vmcnt<0>();
  lds_barrier();
#pragma unroll
  for (int sk_ = 0; sk_ < BN / 16; ++sk_) {
    const int r0 = 16 * sk_ + 8 * h + rr;
    ktf[sk_] = tr_frag_b(smem + STAGE, tile_off<CPR>(r0, 32 * td_w + tcol), tile_off<CPR>(r0 + 4, 32 * td_w + tcol));
  }

  f32x16 dk_acc[TD], dv_acc[TD];
#pragma unroll
  for (int t = 0; t < TD; ++t) {
    dk_acc[t] = f32x16{};
    dv_acc[t] = f32x16{};
  }

  // ---- Per-lane LDS byte offsets (the swizzle folded in; rows are taken
  // modulo 16, the swizzle period, the rest is an immediate).
  int sv[D / 16];  // S/dP A operand: row c32 (+32*tq), columns 16*sd + 8*h
#pragma unroll
  for (int sd = 0; sd < D / 16; ++sd) sv[sd] = tile_off<CPR>(c32, 16 * sd + 8 * h);
  int ta[TD], tb[TD];  // dV/dK B operand: rows 4*h + rr (+8) (+32*tq + 16*s2), columns 32*t + tcol
#pragma unroll
  for (int t = 0; t < TD; ++t) {
    ta[t] = tile_off<CPR>(4 * h + rr, 32 * t + tcol);
    tb[t] = tile_off<CPR>(4 * h + rr + 8, 32 * t + tcol);
  }
  int dsw[TQ][4];  // dS^T stores: row 32*w + c32, columns 32*tq + 8*jj + 4*h
#pragma unroll
  for (int tq = 0; tq < TQ; ++tq)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) dsw[tq][jj] = tile_off<DCPR>(32 * w + c32, 32 * tq + 8 * jj + 4 * h);
  int dra[DQ_TQ], drb[DQ_TQ];  // dQ A operand (dS from dS^T): rows 8*h + rr (+4) (+16*sk)
#pragma unroll
  for (int k = 0; k < DQ_TQ; ++k) {
    dra[k] = tile_off<DCPR>(8 * h + rr, 32 * (tq_w + k) + tcol);
    drb[k] = tile_off<DCPR>(8 * h + rr + 4, 32 * (tq_w + k) + tcol);
  }

  const int m_begin = first_q_block<BM, BN, CAUSAL>(nb, s.sq, s.sk);
  const int m_end = (s.sq + BM - 1) / BM;
  const int kv_lane = kv0 + 32 * w + c32;  // this lane's key column in S / dP

  int qdma[QI], dodma[QI];
#pragma unroll
  for (int i = 0; i < QI; ++i) {
    const int S = (i * 4 + w) * 64 + lane;
    qdma[i] = slot_off(S, (int)a.q_r);
    dodma[i] = slot_off(S, (int)a.do_r);
  }
  const int dq_col = 32 * td_w + c32;
  const int acc_lane = dq_col < hd ? (4 * h * hd + dq_col) * 4 : kOffOOB;

  for (int hq = g * a.group; hq < (g + 1) * a.group; ++hq) {
    if (m_begin >= m_end) break;
    const uint16_t* qb = a.q + s.bq * a.q_b + (int64_t)s.q0 * a.q_r + (int64_t)hq * a.q_h;
    const uint16_t* db = a.dout + s.bq * a.do_b + (int64_t)s.q0 * a.do_r + (int64_t)hq * a.do_h;
    const int64_t st0 = s.stat0 + (int64_t)hq * s.stat_h;
    float* accp = a.dq_acc + acc_base(a, s, hq) + (DET ? (int64_t)nb * a.acc_split : 0);

    // Tile m into stage `st`: Q, dO, LSE, Delta.  Rows past the end read as 0
    // (their P and dS contribute nothing: Q = dO = 0; their dQ rows are dropped).
    auto prefetch = [&](int m, int st) {
      const int rows = min(BM, s.sq - m * BM);
      const uint32_t stage = smem_lds + st * STAGE;
      const u32x4 srdQ = make_srd(qb + (int64_t)m * BM * a.q_r, ((int64_t)(rows - 1) * a.q_r + hd) * 2);
      const u32x4 srdO = make_srd(db + (int64_t)m * BM * a.do_r, ((int64_t)(rows - 1) * a.do_r + hd) * 2);
#pragma unroll
      for (int i = 0; i < QI; ++i) {
        const int S0 = (i * 4 + w) * 64;
        dma16(srdQ, qdma[i], stage + S0 * 16);
        dma16(srdO, dodma[i], stage + TILE + S0 * 16);
      }
      if (w == 0) {
        dma4(make_srd(a.lse_in + st0 + m * BM, (int64_t)rows * 4), lane * 4, stage + 2 * TILE);
      } else if (w == 1) {
        dma4(make_srd(a.delta + st0 + m * BM, (int64_t)rows * 4), lane * 4, stage + 2 * TILE + BM * 4);
      }
    };

    // The dQ slice of iteration m is added to the accumulator during
    // iteration m + 1, NATOM / (TQ * D/16) atomics per S/dP step, so that the
    // atomic issue overlaps matrix-core work instead of stalling the wave.
    f32x16 qpend[DQ_TQ];
    rsrc_t rPend = make_rsrc(accp, 0);
    auto flush_one = [&](int idx) {
      const int k = idx / 16, j = idx % 16;
      const int rq = 32 * (tq_w + k) + 8 * (j >> 2) + (j & 3);
      const int off = acc_lane == kOffOOB ? kOffOOB : acc_lane + rq * hd * 4;
      if (DET) {
        buf_store_f32(rPend, off, qpend[k][j]);
      } else {
        buf_atomic_add_f32(rPend, off, qpend[k][j]);
      }
    };

    // Every wave has built its K fragments (previous barrier) or finished the
    // previous head's iterations before stage 0 is refilled.
    prefetch(m_begin, 0);
    for (int m = m_begin; m < m_end; ++m) {
      const int st = (m - m_begin) & 1;
      const bool pending = m > m_begin;  // a dQ slice from iteration m - 1 to add
      // This wave's loads of tile m are complete once at most the atomics
      // issued after them (iteration m - 1's, if it had any) are outstanding;
      // the barrier then publishes every wave's part and retires all reads of
      // the other stage.
      if (m >= m_begin + 2) {
        wait_vmcnt<NATOM>();
      } else {
        wait_vmcnt<0>();
      }
      lds_barrier();
      if (m + 1 < m_end) prefetch(m + 1, st ^ 1);

      const uint8_t* sQ = smem + st * STAGE;
      const uint8_t* sdO = sQ + TILE;
      const float* sL = reinterpret_cast<const float*>(sQ + 2 * TILE);
      const float* sDl = sL + BM;

      // One 32-query sub-tile at a time: S = Q K^T and dP = dO V^T for this
      // wave's 32 key columns, then P and dS in registers, then
      // dV += P^T dO and dK += dS^T Q (reduction over the sub-tile's queries).
      // Each MFMA section is software-pipelined by hand: the LDS fragments of
      // step i + PD are read before the MFMAs of step i, and every step is
      // pinned with a scheduling barrier so the reads stay ahead.
      const bool diag = (CAUSAL && (kv0 + BN - 1 > m * BM + off_causal)) || rows_k < BN;
      u32x2 dsT[TQ][4];
#pragma unroll
      for (int tq = 0; tq < TQ; ++tq) {
        f32x16 sacc = f32x16{}, pacc = f32x16{};
        // LSE / Delta of this lane's 16 query rows, read ahead of the MFMAs.
        f32x4 Lr[4], Dr[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int qr = 32 * tq + 8 * jj + 4 * h;
          Lr[jj] = *reinterpret_cast<const f32x4*>(sL + qr);
          Dr[jj] = *reinterpret_cast<const f32x4*>(sDl + qr);
        }
        {
          constexpr int NS = D / 16, PD = 3;
          u32x4 fq[PD], fo[PD];
          auto rd = [&](int sd, int slot) {
            fq[slot] = lds_rd128(sQ, 32 * tq * RB + sv[sd]);
            fo[slot] = lds_rd128(sdO, 32 * tq * RB + sv[sd]);
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
            if (pending) {
              constexpr int PER = NATOM / (TQ * NS);
#pragma unroll
              for (int e = 0; e < PER; ++e) flush_one((tq * NS + sd) * PER + e);
            }
            sched_fence();
          }
        }

        // C layout: lane = key column kv_lane, rows = queries
        // 32*tq + 8*(j/4) + 4*h + j%4.  Only tiles crossing the causal
        // diagonal, and the last (partial) key block, need the mask; masking
        // the zero-filled key rows keeps P = exp(-LSE) there from overflowing.
        auto elementwise = [&](auto masked) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int qr = 32 * tq + 8 * jj + 4 * h;
            const f32x4 L = Lr[jj];
            const f32x4 Dl = Dr[jj];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int j = 4 * jj + r;
              float p = fast_exp2(__builtin_fmaf(sacc[j], a.scale_log2, -L[r] * kLog2e));
              if constexpr (decltype(masked)::value) {
                bool vis = kv_lane < kv0 + rows_k;
                if (CAUSAL) vis = vis && (kv_lane <= m * BM + qr + r + off_causal);
                p = vis ? p : 0.f;
              }
              sacc[j] = p;
              pacc[j] = p * (pacc[j] - Dl[r]);
            }
          }
        };
        if (diag) {
          elementwise(std::true_type{});
        } else {
          elementwise(std::false_type{});
        }
        u32x4 pf[2], dsf[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            pf[s2][e] = pack2<BF16>(sacc[8 * s2 + 2 * e], sacc[8 * s2 + 2 * e + 1]);
            dsf[s2][e] = pack2<BF16>(pacc[8 * s2 + 2 * e], pacc[8 * s2 + 2 * e + 1]);
          }
          dsT[tq][2 * s2] = u32x2{dsf[s2][0], dsf[s2][1]};
          dsT[tq][2 * s2 + 1] = u32x2{dsf[s2][2], dsf[s2][3]};
        }
        {
          constexpr int NS = 2 * TD, PD = 3;  // step = (s2, t)
          u32x4 fo[PD], fq[PD];
          auto rd = [&](int i, int slot) {
            const int s2 = i / TD, t = i % TD;
            const int ro = (32 * tq + 16 * s2) * RB;
            fo[slot] = tr_frag_b(sdO, ro + ta[t], ro + tb[t]);
            fq[slot] = tr_frag_b(sQ, ro + ta[t], ro + tb[t]);
          };
          sched_fence();
#pragma unroll
          for (int i = 0; i < PD; ++i) rd(i, i);
          sched_fence();
#pragma unroll
          for (int i = 0; i < NS; ++i) {
            const int s2 = i / TD, t = i % TD;
            const u32x4 bo = fo[i % PD], bq = fq[i % PD];
            if (i + PD < NS) rd(i + PD, i % PD);
            dv_acc[t] = mfma32<BF16>(pf[s2], bo, dv_acc[t]);
            dk_acc[t] = mfma32<BF16>(dsf[s2], bq, dk_acc[t]);
            sched_fence();
          }
        }
      }

      // dS^T -> LDS as [key][query]: 4 consecutive queries per 8-byte store.
#pragma unroll
      for (int tq = 0; tq < TQ; ++tq) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) *reinterpret_cast<u32x2*>(sdST + dsw[tq][jj]) = dsT[tq][jj];
      }
      lds_barrier();

      // dQ slice = dS K for query tiles tq_w.. and head-dim tile td_w; added
      // to the fp32 accumulator during the next iteration (rows past the end
      // fall out of the descriptor's range).
      const int rows = s.sq - m * BM;
      rPend = make_rsrc(accp + (int64_t)m * BM * hd, (int64_t)min(rows, BM) * hd * 4);
#pragma unroll
      for (int k = 0; k < DQ_TQ; ++k) {
        const int tq = tq_w + k;
        f32x16 qacc = f32x16{};
        {
          constexpr int NS = BN / 16, PD = 4;
          u32x4 fa[PD];
          auto rd = [&](int sk_, int slot) { fa[slot] = tr_frag_b(sdST, 16 * sk_ * DRB + dra[k], 16 * sk_ * DRB + drb[k]); };
          sched_fence();
#pragma unroll
          for (int i = 0; i < PD; ++i) rd(i, i);
          sched_fence();
#pragma unroll
          for (int sk_ = 0; sk_ < NS; ++sk_) {
            const u32x4 af = fa[sk_ % PD];
            if (sk_ + PD < NS) rd(sk_ + PD, sk_ % PD);
            qacc = mfma32<BF16>(af, ktf[sk_], qacc);
            sched_fence();
          }
        }
        qpend[k] = qacc;
      }
    }
    // The last iteration's dQ slice.
    if (m_begin < m_end) {
#pragma unroll
      for (int e = 0; e < NATOM; ++e) flush_one(e);
    }
  }

  // ---- Epilogue: dK * scale, dV; convert (round to nearest even) and store.
  const uint16_t* dkb = a.dk + s.bk * a.dk_b + (int64_t)(s.k0 + kv0) * a.dk_r + (int64_t)g * a.dk_h;
  const uint16_t* dvb = a.dv + s.bk * a.dv_b + (int64_t)(s.k0 + kv0) * a.dv_r + (int64_t)g * a.dv_h;
  const rsrc_t rDK = make_rsrc(dkb, ((int64_t)(rows_k - 1) * a.dk_r + hd) * 2);
  const rsrc_t rDV = make_rsrc(dvb, ((int64_t)(rows_k - 1) * a.dv_r + hd) * 2);
#pragma unroll
  for (int t = 0; t < TD; ++t) {
    const int d = 32 * t + c32;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int kr = 32 * w + 8 * (j >> 2) + 4 * h + (j & 3);
      const int ok = d < hd;
      buf_store_u16(rDK, ok ? (kr * (int)a.dk_r + d) * 2 : kOffOOB, to_bits<BF16>(dk_acc[t][j] * a.scale));
      buf_store_u16(rDV, ok ? (kr * (int)a.dv_r + d) * 2 : kOffOOB, to_bits<BF16>(dv_acc[t][j]));
    }
  }
}

// ---------------------------------------------------------------------------
// Postprocess: dQ = scale * (sum of accumulator slices), converted.
// Deterministic mode sums the slices of the key blocks that visit this query
// block, in ascending key-block order.
// ---------------------------------------------------------------------------
template <bool BF16, bool CAUSAL, bool DET>
__global__ __launch_bounds__(256) void attn_bwd_post_kernel(Args a) {
  const int z = blockIdx.z, hq = blockIdx.y, mb = blockIdx.x;
  const Seq s = seq_info(a, z);
  const int r0 = mb * kPreRows;
  if (r0 >= s.sq) return;
  const int hd = a.head_dim;
  int nsum = 1;
  if (DET) {
    const int nkb = (s.sk + kBwdBN - 1) / kBwdBN;
    nsum = 0;
    while (nsum < nkb && first_q_block<kBwdBM, kBwdBN, CAUSAL>(nsum, s.sq, s.sk) <= mb) ++nsum;
  }
  const float* accp = a.dq_acc + acc_base(a, s, hq);
  uint16_t* dqb = a.dq + s.bq * a.dq_b + (int64_t)s.q0 * a.dq_r + (int64_t)hq * a.dq_h;
  const int c4 = hd / 4;
  const int rows = min(kPreRows, s.sq - r0);
  for (int i = threadIdx.x; i < rows * c4; i += 256) {
    const int r = r0 + i / c4;
    const int c = 4 * (i % c4);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int n = 0; n < nsum; ++n) {
      const float4 v = *reinterpret_cast<const float4*>(accp + (int64_t)n * a.acc_split + (int64_t)r * hd + c);
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    u32x2 pk;
    pk[0] = pack2<BF16>(acc.x * a.scale, acc.y * a.scale);
    pk[1] = pack2<BF16>(acc.z * a.scale, acc.w * a.scale);
    *reinterpret_cast<u32x2*>(dqb + (int64_t)r * a.dq_r + c) = pk;
  }
}

}  // namespace attn
