// Attention backward on gfx950 as two matrix-core kernels that never use
// atomics: a KV-stationary kernel for dK and dV (this file) and a
// Q-stationary kernel for dQ (attn_bwd_dq.h).  Both recompute
// P = exp2(S*scale*log2e - LSE*log2e) from the saved LSE tile by tile
// (tilelang test_tilelang_kernel_mha_bwd.py, flashattn_bwd) and
// dS = P o (dP - Delta) with Delta from the preprocess; nothing of size
// Sq x Sk is ever written to memory.
//
// Why two kernels: the pages accumulate dQ across key blocks with fp32
// atomics (tilelang flashattn_bwd's atomic_add; the CK mha_bwd.cpp page's
// dq_accum).  On MI355X the device-wide fp32 atomic rate measures about
// 340 G lane-ops/s for every access shape (bench_calibrate.hip), which for a
// causal S=4096, d=128 workload puts a floor of about 1.6 ms (128-key blocks)
// under the dQ accumulation alone.  The Q-stationary dQ kernel recomputes S
// and dP (two extra GEMMs, 7 instead of 5 per tile pair) but keeps dQ in
// registers, writes it once, and is deterministic by construction (key
// blocks are summed in ascending order).
//
// The dK/dV kernel runs 8 wave64s, two per SIMD, in two groups half a tile
// apart, so that on every SIMD one wave's softmax and products share each
// interval with the other wave's products.  Each wave owns 32 key rows and
// splits the streamed query tile with a partner wave: the pair computes the
// two halves of the score tile (no duplicated MFMA work); then one wave of
// the pair accumulates dV and the other dK, each over the whole head
// dimension, so each sends its partner only the operand the partner lacks:
// the dV wave sends its dS^T, the dK wave its P^T.
#pragma once

#include <type_traits>

#include "attn_bwd.h"
#include "attn_device.h"

namespace attn {

constexpr int kDkvBM = 64;    // query rows per iteration of the dK/dV kernel
// Key rows per dK/dV workgroup: 16 per wave.  Head dims up to 128 run 8 waves
// (two per SIMD, 128 keys, one workgroup per CU); the 256-wide tile runs 4
// waves (one per SIMD, 64 keys), whose K, V and accumulators take twice the
// registers.  Causal MHA at head dims up to 128 can also run 4 waves (64
// keys) with two workgroups per CU, so that one workgroup's start-up and
// epilogue overlap the other's tile loop (the host picks it; see
// dkdv_small_wg in the launcher).
constexpr int dkdv_waves(int d) { return d > 128 ? 4 : 8; }
constexpr int dkdv_bn(int d) { return 16 * dkdv_waves(d); }
// waves per SIMD of a dK/dV kernel with NW waves per workgroup
constexpr int dkdv_wpe(int d, int nw) { return nw == 8 || d <= 128 ? 2 : 1; }

// ---------------------------------------------------------------------------
// dK / dV: one workgroup per (key block, KV head, sequence) -- 128 keys, or
// 64 for the 256-wide head-dim tile -- looping over the query blocks (and,
// for GQA, over the query heads of the KV head).
//   wave w: key rows 32*(w>>1) .. +32 of the block, shared with its partner
//   w^1; query half R = w&1 of each 64-query tile for S = Q K^T and
//   dP = dO V^T; then R = 0 accumulates dV += P^T dO and R = 1 dK += dS^T Q
//   over all 64 queries and all DC / 32 head-dim tiles.
//   Waves 0-3 and 4-7 (one of each on every SIMD) run half a tile apart.
// The head dim is stored in a D-wide LDS tile (D = 64, 128, 256; columns
// past head_dim are zero) and computed DC wide (a multiple of 32, at most D:
// 96 for head dims 72-96, so a 96-wide head does three quarters of the
// 128-wide tile's products).
// LDS (D = 128): three stages of {Q, dO, LSE*log2(e), -Delta} (3 x 32.5 KiB,
// swizzled, filled by direct global->LDS loads two tiles ahead) + the P or
// dS exchange (8 x 2 KiB); the block's K and V pass through the last stage
// and the bytes after it on their way into registers.
// ---------------------------------------------------------------------------
template <bool BF16, int D, int DC, bool BANDED, int NW = dkdv_waves(D)>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(dkdv_wpe(D, NW), dkdv_wpe(D, NW))))
void attn_bwd_dkdv_kernel(Args a) {
  static_assert(DC % 32 == 0 && DC <= D, "compute width: 32-column tiles within the stored tile");
  static_assert(NW == 8 ? D <= 128 : NW == 4, "8 waves up to head dim 128, else 4");
  constexpr int BM = kDkvBM, BN = 16 * NW;
  // LDS operand reads in flight ahead of their product (two for the 4-wave
  // kernel at two workgroups per CU, which has 256 registers per wave)
  constexpr int PDK = NW == 4 && D <= 128 ? 2 : 3;
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int RB = D * 2;                  // bytes per row
  constexpr int TILE = BM * RB;
  constexpr int STAGE = 2 * TILE + 2 * BM * 4;
  constexpr int TD = DC / 32;                // head-dim tiles of this wave's dV or dK
  constexpr int QI = BM * CPR / (64 * NW);   // direct loads per wave per Q (or dO) tile
  constexpr int NPF = 2 * QI + 1;            // direct loads per wave per tile (Q, dO, one stat row)
  // stages of {Q, dO, LSE, Delta}: three (loads two tiles ahead) when they
  // fit in LDS, else two (one tile ahead)
  constexpr int NSTAGE = NW == 8 ? 3 : 2;
  constexpr int XB = 2 * 16 * 64;            // exchange bytes per wave (two 16-query operands)
  constexpr int KVR = (NSTAGE - 1) * STAGE;  // LDS byte offset of the K tile, V follows
  // 256 bytes the idle waves' stat loads land in, past the stages, the
  // exchange slots and the K/V staging
  constexpr int SINK = NSTAGE * STAGE + NW * XB > KVR + 2 * BN * RB ? NSTAGE * STAGE + NW * XB : KVR + 2 * BN * RB;
  static_assert(TD >= 1 && QI >= 1, "head dim tile of 64, 128 or 256");
  static_assert(SINK + 256 <= 160 * 1024, "LDS");

  __shared__ __attribute__((aligned(1024))) uint8_t smem[SINK + 256];
  const uint32_t smem_lds = lds_addr(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = wave_id();
  const int kvg = w >> 1;         // key-row group of this wave (a pair of waves)
  const int half = w & 1;         // query half (S, dP); 0 accumulates dV, 1 dK
  const int grp = w >> 2;         // pipeline group: 0 runs half a tile ahead of 1
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
  const int off_causal = s.sk - s.sq;  // banded: key j visible to query i iff |j - (i + off)| in the window
  const int rows_k = min(BN, s.sk - kv0);

  // ---- K, V of this wave's 32 key rows as B operands of S = Q K^T and
  // dP = dO V^T (column = key, k = head dim), held in registers for the whole
  // workgroup.  They come through LDS: the block's K and V tiles are loaded
  // with direct global->LDS loads (16 contiguous bytes per lane, each row
  // once) into the region of the last stage and past it, which the loop
  // first touches after the first tile, and each wave then reads its
  // fragments with conflict-free row reads of the swizzled tiles.  Rows past
  // the end read as 0.
  u32x4 kf[DC / 16], vf[DC / 16];
  constexpr int KVI = BN * CPR / (64 * NW);     // direct loads per wave per K (or V) tile
  auto load_kv_lds = [&] {
    KArgs& ka = kernel_args();
    const uint16_t* kb = ka.k + s.bk * ka.k_b + (int64_t)(s.k0 + kv0) * ka.k_r + (int64_t)g * ka.k_h;
    const uint16_t* vb = ka.v + s.bk * ka.v_b + (int64_t)(s.k0 + kv0) * ka.v_r + (int64_t)g * ka.v_h;
    const u32x4 srdK = make_srd(kb, ((int64_t)(rows_k - 1) * ka.k_r + hd) * 2);
    const u32x4 srdV = make_srd(vb, ((int64_t)(rows_k - 1) * ka.v_r + hd) * 2);
#pragma unroll
    for (int i = 0; i < KVI; ++i) {
      const int S = (i * NW + w) * 64 + lane;
      const int r = S / CPR;
      const int c = (S % CPR) ^ swz<CPR>(r);
      const bool ok = 8 * c < hd;
      const uint32_t dst = smem_lds + KVR + (uint32_t)((i * NW + w) * 64) * 16u;
      dma16(srdK, ok ? (r * (int)ka.k_r + 8 * c) * 2 : kOffOOB, dst);
      dma16(srdV, ok ? (r * (int)ka.v_r + 8 * c) * 2 : kOffOOB, dst + BN * RB);
    }
  };
  auto read_kv_regs = [&] {
    const int kvo = KVR + tile_off<CPR>(32 * kvg + c32, 8 * h);
#pragma unroll
    for (int sd = 0; sd < DC / 16; ++sd) {
      kf[sd] = lds_rd128(smem, kvo ^ (32 * sd));
      vf[sd] = lds_rd128(smem, (kvo ^ (32 * sd)) + BN * RB);
    }
  };

  f32x16 acc[TD];  // dV (half 0) or dK (half 1) of this wave's 32 keys
#pragma unroll
  for (int t = 0; t < TD; ++t) acc[t] = f32x16{};

  // ---- Per-lane LDS byte offsets (swizzle folded in; rows modulo 16).
  // S/dP A operand: row 32*half + c32, columns 16*sd + 8*h.  The swizzle
  // only permutes the chunk bits, so step sd is at svb ^ 32*sd.
  const int svb = 32 * half * RB + tile_off<CPR>(c32, 8 * h);
  // dV/dK B operand: rows 4*h + rr (+8), columns 32t + tcol; the column
  // tile only changes chunk bits above those of tcol, so tile t is at
  // ta ^ 64*t (tb ^ 64*t).
  const int ta = tile_off<CPR>(4 * h + rr, tcol);
  const int tb = tile_off<CPR>(4 * h + rr + 8, tcol);
  uint8_t* const xown = smem + NSTAGE * STAGE + w * XB + lane * 16;
  const uint8_t* const xpar = smem + NSTAGE * STAGE + (w ^ 1) * XB + lane * 16;

  auto slot_off = [&](int S, int row_stride) {
    const int r = S / CPR;
    const int c = (S % CPR) ^ swz<CPR>(r);
    return 8 * c < hd ? (r * row_stride + 8 * c) * 2 : kOffOOB;
  };
  int qdma[QI], dodma[QI];
#pragma unroll
  for (int i = 0; i < QI; ++i) {
    const int S = (i * NW + w) * 64 + lane;
    qdma[i] = slot_off(S, (int)a.q_r);
    dodma[i] = slot_off(S, (int)a.do_r);
  }

  // query tiles that see any key of this block
  int m_begin = 0, m_end = (s.sq + BM - 1) / BM;
  if (BANDED) {
    const Range qr = band_queries(a, kv0, kv0 + rows_k - 1, s.sq, s.sk);
    m_begin = qr.lo / BM;
    m_end = qr.hi < qr.lo ? m_begin : qr.hi / BM + 1;
  }
  const int kv_lane = kv0 + 32 * kvg + c32;  // this lane's key column in S / dP

  // The rest runs for a compile-time role R (the wave's half).
  auto body = [&](auto role_t) {
  constexpr int R = decltype(role_t)::value;
  // Packed P^T / dS^T operands of this wave's 32 queries, formed in phase 1
  // of a tile and consumed in its phase 2 (for the second group, across the
  // loop's back edge).
  u32x4 pf[2], dsf[2];

  for (int hq = g * a.group; hq < (g + 1) * a.group; ++hq) {
    if (m_begin >= m_end) break;
    KArgs& ka = kernel_args();
    const uint16_t* qb = ka.q + s.bq * ka.q_b + (int64_t)s.q0 * ka.q_r + (int64_t)hq * ka.q_h;
    const uint16_t* db = ka.dout + s.bq * ka.do_b + (int64_t)s.q0 * ka.do_r + (int64_t)hq * ka.do_h;
    const int64_t st0 = s.stat0 + (int64_t)hq * s.stat_h;

    // Tile m into stage `st`: Q, dO, LSE, Delta.  Rows past the end read as 0;
    // their P and dS then contribute nothing (Q = dO = 0).  Every wave issues
    // exactly NPF loads per call, so the memory-counter waits below are
    // exact: for real == false (no such tile) the loads have an empty range,
    // land zeros in a stage nobody reads again, and the idle waves' stat
    // loads land in the sink.
    // One descriptor per head (the sequence's rows of Q and dO, its LSE or
    // Delta row), built once; a tile is a 32-bit lane offset into it, so the
    // per-tile cost is a few vector adds.  Offsets past the range read as
    // zero: rows past the end, the columns past head_dim (offset kOffOOB)
    // and, for real == false, the whole tile.  Head extents are below 2 GiB
    // (checked on the host), so no offset wraps.
    const u32x4 srdQh = make_srd(qb, ((int64_t)(s.sq - 1) * a.q_r + hd) * 2);
    const u32x4 srdOh = make_srd(db, ((int64_t)(s.sq - 1) * a.do_r + hd) * 2);
    const u32x4 srdSh = make_srd((w == 0 ? ka.lse2 : ka.delta) + st0, w < 2 ? (int64_t)s.sq * 4 : 0);
    auto prefetch = [&](int m, int st, bool real) {
      const uint32_t stage = smem_lds + st * STAGE;
      const uint32_t tq = real ? (uint32_t)(m * BM) * (uint32_t)a.q_r * 2u : (uint32_t)kOffOOB;
      const uint32_t to = real ? (uint32_t)(m * BM) * (uint32_t)a.do_r * 2u : (uint32_t)kOffOOB;
#pragma unroll
      for (int i = 0; i < QI; ++i) {
        const int S0 = (i * NW + w) * 64;
        dma16(srdQh, (int)((uint32_t)qdma[i] + tq), stage + S0 * 16);
        dma16(srdOh, (int)((uint32_t)dodma[i] + to), stage + TILE + S0 * 16);
      }
      const uint32_t sdst = w < 2 ? stage + 2 * TILE + w * BM * 4 : smem_lds + SINK;
      dma4(srdSh, (int)(real ? (uint32_t)(m * BM + lane) * 4u : (uint32_t)kOffOOB), sdst);
    };

    // Phase 1 of tile m (stage st): S and dP for this wave's 32 queries x 32
    // keys, P and dS, and the packed operands into the exchange slot.
    auto phase1_body = [&](int m, int st, auto mask) {
      const uint8_t* sQ = smem + st * STAGE;
      // per-tile base (stage offsets leave the chunk bits alone), so the
      // per-step XORs are not hoisted out of the loop into 8 registers
      const int svn = svb + st * STAGE;
      const float* sL = reinterpret_cast<const float*>(sQ + 2 * TILE);
      const float* sDl = sL + BM;

      // LSE * log2(e) and -Delta of this lane's 16 query rows, in the order
      // of the C layout's rows.  -Delta is the dP accumulator's start value,
      // so the products leave dP - Delta.
      // (Read after the first S products are issued, so that those start on
      // the Q operands alone.)
      f32x4 Lr[4];
      f32x16 pacc;
      auto read_stats = [&] {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          Lr[jj] = *reinterpret_cast<const f32x4*>(sL + 32 * R + 8 * jj + 4 * h);
          const f32x4 nd = *reinterpret_cast<const f32x4*>(sDl + 32 * R + 8 * jj + 4 * h);
#pragma unroll
          for (int r = 0; r < 4; ++r) pacc[4 * jj + r] = nd[r];
        }
      };

      // Visibility of the tile's (query, key) pairs (masked tiles only).
      // C layout of S / dP: lane = key column kv_lane, rows = queries
      // 32*half + 8*(j/4) + 4*h + j%4.  Element (jj, r) is query q_base + e, e = 8*jj + r.  It is visible iff
      // its key (this lane's) is a real row and e_lo <= e <= e_hi, from
      // i + off - win_l <= key <= i + off + win_r.
      const int q_base = m * BM + 32 * R + 4 * h;
      const int d0 = kv_lane - q_base - off_causal;
      const int e_lo = BANDED ? d0 - a.win_r : -kWinInf;
      const int e_hi = BANDED ? d0 + a.win_l : kWinInf;
      const bool key_ok = kv_lane < kv0 + rows_k;

      // S = Q K^T, then dP = dO V^T: 32 queries (this wave's half) x 32
      // keys, one chain after the other, so that P = exp2(S*scale*log2e -
      // LSE2) runs on the vector ALU under the dP products.  The products go
      // out at raised priority: the other wave on this SIMD is in phase 2
      // (matrix-core work only) and fills the gaps.
      f32x16 sacc = f32x16{};
      {
        constexpr int NS = DC / 16, PD = PDK;
        u32x4 fr[PD];
        // operand step i: Q for i < NS (S chain), dO for i >= NS (dP chain)
        auto rd = [&](int i, int slot) {
          const int sd = i % NS;
          fr[slot] = lds_rd128(smem, (svn ^ (32 * sd)) + (i < NS ? 0 : TILE));
        };
        auto p_elem = [&](int j) {
          const int jj = j / 4, r = j % 4;
          float p = fast_exp2(__builtin_fmaf(sacc[j], a.scale_log2, -Lr[jj][r]));
          if constexpr (decltype(mask)::value) {
            const int e = 8 * jj + r;
            p = (key_ok && e >= e_lo && e <= e_hi) ? p : 0.f;
          }
          // keeps the exp between the dP products it is written between:
          // the scheduling fences order only side effects, and the compiler
          // otherwise sinks all 16 exps below the last product
          asm volatile("" : "+v"(p));
          sacc[j] = p;
        };
        sched_fence();
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int i = 0; i < PD; ++i) rd(i, i);
        sched_fence();
#pragma unroll
        for (int i = 0; i < 2 * NS; ++i) {
          const u32x4 op = fr[i % PD];
          if (i + PD < 2 * NS) rd(i + PD, i % PD);
          if (i < NS) {
            sacc = mfma32<BF16>(op, kf[i], sacc);
            if (i == 1) read_stats();
          } else {
            pacc = mfma32<BF16>(op, vf[i - NS], pacc);
            // the 16 elements of P spread over the NS dP products
#pragma unroll
            for (int e = 16 * (i - NS) / NS; e < 16 * (i - NS + 1) / NS; ++e) p_elem(e);
          }
          sched_fence();
        }
        __builtin_amdgcn_s_setprio(0);
        sched_fence();
      }
      // dS = P o (dP - Delta)
#pragma unroll
      for (int j = 0; j < 16; ++j) pacc[j] = sacc[j] * pacc[j];

      // P^T and dS^T as A operands (row = key, k = query): k-slot i of 16-query
      // step s2 is query 16*s2 + 8*(i/4) + 4*h + i%4 of this wave's half.
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pf[s2][e] = pack2<BF16>(sacc[8 * s2 + 2 * e], sacc[8 * s2 + 2 * e + 1]);
          dsf[s2][e] = pack2<BF16>(pacc[8 * s2 + 2 * e], pacc[8 * s2 + 2 * e + 1]);
        }
      }
      // For the partner wave (same keys, other query half): the dV wave needs
      // the dK wave's P^T, the dK wave the dV wave's dS^T.
      *reinterpret_cast<u32x4*>(xown + 0 * 1024) = R == 0 ? dsf[0] : pf[0];
      *reinterpret_cast<u32x4*>(xown + 1 * 1024) = R == 0 ? dsf[1] : pf[1];
    };
    // Tiles crossing an edge of the band and the partial last key block are
    // masked (zero-filled key rows would otherwise give P = exp(-LSE), which
    // could overflow a 16-bit dS); every pair of an unmasked tile is
    // visible: its lowest query sees its highest key and its highest query
    // its lowest key.  One branch per tile, around the whole phase.
    auto phase1 = [&](int m, int st) {
      const bool masked = (BANDED && (kv0 + BN - 1 > m * BM + off_causal + a.win_r ||
                                      kv0 < m * BM + BM - 1 + off_causal - a.win_l)) ||
                          rows_k < BN;
      if (masked) {
        phase1_body(m, st, std::true_type{});
      } else {
        phase1_body(m, st, std::false_type{});
      }
    };

    // Phase 2 of tile m (stage st): dV += P^T dO (R = 0) or dK += dS^T Q
    // (R = 1) over all 64 queries of the tile and every head-dim tile, the
    // other query half's operand from the partner's exchange slot (written
    // before the barrier that ends phase 1).  Step = (query step sq, head-dim
    // tile t), this wave's own query half first.
    auto phase2 = [&](int st) {
      const uint8_t* sB = smem + st * STAGE + (R == 0 ? TILE : 0);  // dO for dV, Q for dK
      u32x4 par[2];
      par[0] = *reinterpret_cast<const u32x4*>(xpar + 0 * 1024);
      par[1] = *reinterpret_cast<const u32x4*>(xpar + 1 * 1024);
      constexpr int NS = 4 * TD, PD = PDK;
      u32x4 fb[PD];
      auto rd = [&](int i, int slot) {
        const int sq = (i / TD + 2 * R) & 3, t = i % TD;
        const int ro = 16 * sq * RB;
        fb[slot] = tr_frag_b(sB, ro + (ta ^ (64 * t)), ro + (tb ^ (64 * t)));
      };
      sched_fence();
#pragma unroll
      for (int i = 0; i < (PD < NS ? PD : NS); ++i) rd(i, i);
      sched_fence();
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const int sq = (i / TD + 2 * R) & 3, t = i % TD;
        const u32x4 bb = fb[i % PD];
        if (i + PD < NS) rd(i + PD, i % PD);
        const u32x4 own = R == 0 ? pf[sq & 1] : dsf[sq & 1];
        const u32x4 av = (sq >> 1) == R ? own : par[sq & 1];
        acc[t] = mfma32<BF16>(av, bb, acc[t]);
        sched_fence();
      }
    };

    if constexpr (NSTAGE == 3) {
      // Two groups of four waves (two pairs each) run half a tile apart: in
      // every interval between barriers one wave of each SIMD is in phase 1
      // (products, then the softmax on the vector ALU) and the other in phase
      // 2 (products only), so the softmax of one overlaps the other's matrix
      // work.  Both groups run the same straight loop body, phase 1, barrier,
      // phase 2, barrier; group 1 enters it one barrier late (s_barrier counts
      // arrivals, not program locations) and group 0 passes one extra barrier
      // at the end, so interval k holds group 0's phase (k & 1) of tile k / 2
      // and group 1's phase ((k - 1) & 1) of tile (k - 1) / 2.
      // Tile j (relative) lives in stage j % 3.  Tile j + 2 is loaded at the
      // start of interval 2j + 1 (group 0's phase 2 of tile j, group 1's phase
      // 1), after the barrier that ends the last read of its stage (group 1's
      // phase 2 of tile j - 1), and this wave's share of tile j + 1 is waited
      // for at the end of interval 2j + 1, before group 0 reads it.
      //
      // Memory-counter accounting: the loads are the only memory operations
      // of the loop and complete in issue order, so waiting until at most
      // NPF are outstanding (the next tile's) means tile j + 1 has landed.
      const int n = m_end - m_begin;
      // The previous head's last interval ended with a barrier: every wave is
      // done with its stages.
      const bool first_head = hq == g * a.group;
      if (first_head) load_kv_lds();
      prefetch(m_begin, 0, true);
      prefetch(m_begin + 1, 1, n > 1);
      wait_vmcnt<NPF>();
      lds_barrier();  // tile 0 (and K/V) landed
      if (first_head) {
        read_kv_regs();
        lds_barrier();  // every wave has its K/V before the staging region is reused
      }
      if (grp) lds_barrier();  // interval 0: group 0's phase 1 of tile 0
      int st = 0, st_load = 2;
      for (int j = 0; j < n; ++j) {
        if (grp) prefetch(m_begin + j + 2, st_load, j + 2 < n);
        phase1(m_begin + j, st);
        if (grp) wait_vmcnt<NPF>();
        lds_barrier();  // exchange slots written
        if (!grp) prefetch(m_begin + j + 2, st_load, j + 2 < n);
        phase2(st);
        if (!grp) wait_vmcnt<NPF>();
        lds_barrier();  // loads published; stage reads retired
        st = st == 2 ? 0 : st + 1;
        st_load = st_load == 2 ? 0 : st_load + 1;
      }
      if (!grp) lds_barrier();  // interval 2n: group 1's phase 2 of the last tile
      } else {
      // One wave per SIMD, one group: phase 1, barrier, phase 2, barrier per
      // tile.  Tile j + 1 is loaded into the other stage at the start of
      // tile j (its stage was last read in phase 2 of tile j - 1) and waited
      // for at the end of tile j.
      const int n = m_end - m_begin;
      const bool first_head = hq == g * a.group;
      if (first_head) load_kv_lds();
      prefetch(m_begin, 0, true);
      wait_vmcnt<0>();
      lds_barrier();  // tile 0 (and K/V) landed
      if (first_head) {
        read_kv_regs();
        lds_barrier();  // every wave has its K/V before the staging region is reused
      }
      int st = 0;
      for (int j = 0; j < n; ++j) {
        prefetch(m_begin + j + 1, st ^ 1, j + 1 < n);
        phase1(m_begin + j, st);
        lds_barrier();  // exchange slots written
        phase2(st);
        wait_vmcnt<0>();
        lds_barrier();  // loads published; stage reads retired
        st ^= 1;
      }
    }
}

  // ---- Epilogue: dV (R = 0) or dK * scale (R = 1), rounded to nearest
  // even, stored as 16-byte row chunks through this wave's LDS region
  // (every wave is past its last stage read -- the loop ended on a barrier --
  // and the empty prefetches of the last tiles have landed once vmcnt
  // reaches 0).
  wait_vmcnt<0>();
  {
    constexpr int REG = 32 * TD * 72;  // LDS bytes per wave
    static_assert(NW * REG <= SINK, "epilogue transpose fits the stages");
    KArgs& ka = kernel_args();
    const int64_t orow = R == 0 ? ka.dv_r : ka.dk_r;
    const uint16_t* ob = R == 0 ? ka.dv + s.bk * ka.dv_b + (int64_t)g * ka.dv_h : ka.dk + s.bk * ka.dk_b + (int64_t)g * ka.dk_h;
    ob += (int64_t)(s.k0 + kv0 + 32 * kvg) * orow;
    const int rows_ok = rows_k - 32 * kvg;
    const rsrc_t rO = make_rsrc(ob, rows_ok > 0 ? ((int64_t)(rows_ok - 1) * orow + hd) * 2 : 0);
    store_tile_rows<BF16, TD>(acc, R == 0 ? 1.f : ka.scale, smem + w * REG, rO, (int)orow, rows_ok, hd, lane);
  }
  };
  if (half) body(std::integral_constant<int, 1>{});
  else body(std::integral_constant<int, 0>{});
}

}  // namespace attn
