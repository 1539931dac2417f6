// Attention backward on gfx950: the dQ kernels.
//
// dQ = scale * dS K (tilelang test_tilelang_kernel_mha_bwd.py, flashattn_bwd:
// the dQ contribution of each key block is dS K; the Hopper
// flash_bwd_launch_template.h page applies the softmax scale to dQ after the
// sum over key blocks).  The kernels are Q-stationary: a wave keeps its
// queries' Q and dO in registers, streams K and V tiles through LDS,
// recomputes S^T = K Q^T and dP^T = V dO^T per key tile, forms
// dS^T = P^T o (dP^T - Delta) with P = exp2(S*scale*log2e - LSE*log2e) from
// the saved LSE, and accumulates dQ in registers over the key tiles in
// ascending order -- no atomics and no dQ accumulator in memory, so the
// result is deterministic and the only workspace is the two row statistics.
// The transposed score tile puts one query per lane, so LSE and Delta are
// per-lane constants, and dS^T leaves the MFMA in the A-operand layout of
// dQ = dS K.  The softmax scale is applied once, in the epilogue, which is
// the pages' dQ postprocess (scale, convert) fused.  Each kernel also runs
// the preprocess for its own query rows first (Delta = rowsum(O o dO) from
// O loaded beside dO, and LSE*log2(e)) and writes both to the workspace for
// the dK/dV kernel, which is launched after it.
#pragma once

#include <type_traits>

#include "attn_device.h"

namespace attn {

constexpr int kDqWaves = 8;              // waves per dQ workgroup (32 queries each), head dim <= 128
constexpr int kDqBM = 32 * kDqWaves;     // query rows per dQ workgroup
constexpr int kDqBN = 64;                // key rows per tile
constexpr int kDqPD = 4;                 // LDS reads in flight ahead of their MFMAs
constexpr int kDqWideBM = 128;           // query rows per dQ workgroup, 256-wide head-dim tile

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
// dQ for head dims up to 128: one workgroup per (query head x sequence,
// 256-query block), 8 waves (two per SIMD), wave w owning queries 32w .. +32
// of the block; each wave works the 64-key tiles its rows see alone, as two
// 32-key halves.
// K and V tiles are stored D wide in LDS (D = 64 or 128) and the products run
// DC wide (96 for head dims 72-96).
//
// Schedule.  The matrix-core work of one tile is a stream of slots
//   A: S, dP of half 0      B: dQ of the previous tile's half 1
//   C: S, dP of half 1      D: dQ of half 0
// and the softmax of each half runs in the dQ slots after it, with one slot
// between dependent vector instructions, so that the vector work of one
// wave overlaps its own matrix-core work.  The K tile of the previous key
// tile is still read in B, hence three LDS stages (3 x 32 KiB at D = 128),
// filled by direct global->LDS loads one tile ahead.
// ---------------------------------------------------------------------------
template <bool BF16, int D, int DC, bool BANDED>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bwd_dq_recompute_kernel(Args a) {
  constexpr int NW = 8;
  constexpr int BM = kDqBM, BN = kDqBN;
  constexpr int CPR = D / 8;
  constexpr int RB = D * 2;
  constexpr int KT = BN * RB;                // bytes of a K (or V) tile
  constexpr int STAGE = 2 * KT;
  constexpr int NSTAGE = 3;
  static_assert(DC % 32 == 0 && DC <= D, "compute width: 32-column tiles within the stored tile");
  constexpr int TD = DC / 32;                // head-dim tiles of dQ
  constexpr int NSD = DC / 16;               // k-steps of S^T / dP^T
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
  const int mb = BANDED ? (int)(gridDim.y - 1 - blockIdx.y) : (int)blockIdx.y;
  const int q0 = mb * BM;
  if (q0 >= s.sq) return;
  const int hd = a.head_dim;
  const int g = hq / a.group;
  const int off_causal = s.sk - s.sq;
  const int qw = q0 + 32 * w;         // first query of this wave
  const int qi = qw + c32;            // this lane's query (a column of S^T)

  // ---- Q and dO of this lane's query as B operands (k = head dim); LSE and
  // Delta of that query.  Rows past the end read as 0.
  // O of the same rows and chunks: the preprocess's input (below).
  u32x4 qf[NSD], df[NSD], of[NSD];
  float L2, Dl;
  int64_t stat_row;  // workspace index of this lane's row, -1 past the end
  {
    const int rows = min(BM, s.sq - q0);
    const uint16_t* qb = a.q + s.bq * a.q_b + (int64_t)(s.q0 + q0) * a.q_r + (int64_t)hq * a.q_h;
    const uint16_t* db = a.dout + s.bq * a.do_b + (int64_t)(s.q0 + q0) * a.do_r + (int64_t)hq * a.do_h;
    const uint16_t* ob = a.o + s.bq * a.o_b + (int64_t)(s.q0 + q0) * a.o_r + (int64_t)hq * a.o_h;
    const rsrc_t rQ = make_rsrc(qb, ((int64_t)(rows - 1) * a.q_r + hd) * 2);
    const rsrc_t rO = make_rsrc(db, ((int64_t)(rows - 1) * a.do_r + hd) * 2);
    const rsrc_t rOut = make_rsrc(ob, ((int64_t)(rows - 1) * a.o_r + hd) * 2);
    const int row = 32 * w + c32;
#pragma unroll
    for (int sd = 0; sd < NSD; ++sd) {
      const int d0 = 16 * sd + 8 * h;
      const bool ok = d0 < hd;
      qf[sd] = buf_load128(rQ, ok ? (row * (int)a.q_r + d0) * 2 : kOffOOB);
      df[sd] = buf_load128(rO, ok ? (row * (int)a.do_r + d0) * 2 : kOffOOB);
      of[sd] = buf_load128(rOut, ok ? (row * (int)a.o_r + d0) * 2 : kOffOOB);
    }
    const int64_t st0 = s.stat0 + (int64_t)hq * s.stat_h + q0;
    L2 = buf_load_f32(make_rsrc(a.lse_in + st0, (int64_t)rows * 4), row * 4) * kLog2e;
    stat_row = row < rows ? st0 + row : -1;
  }

  f32x16 dq_acc[TD];
#pragma unroll
  for (int t = 0; t < TD; ++t) dq_acc[t] = f32x16{};
  f32x16 ndl;  // -Delta of this lane's query in every row (set below)

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
  int n_begin = 0, n_end = (s.sk + BN - 1) / BN;
  if (BANDED) {
    const Range kr = band_keys(a, q0, min(q0 + BM, s.sq) - 1, s.sq, s.sk);
    n_begin = kr.lo / BN;
    n_end = kr.hi < kr.lo ? n_begin : kr.hi / BN + 1;
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
  // a tile needs the mask unless every key of it is visible to every query
  // of this wave
  auto tile_masked = [&](int n) {
    return (BANDED && (n * BN + BN - 1 > qw + off_causal + a.win_r || n * BN < qw + 31 + off_causal - a.win_l)) ||
           (n * BN + BN > s.sk);
  };

  // Keys this lane's query sees, minus the lane's row offset 4*h in the C
  // layout (keys past the end or outside the band are masked).
  int kv_hi = s.sk - 1, kv_lo = -kWinInf;
  if (BANDED) {
    kv_hi = min(kv_hi, qi + off_causal + a.win_r);
    kv_lo = qi + off_causal - a.win_l;
  }
  kv_hi -= 4 * h;
  kv_lo -= 4 * h;

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
      if (BANDED) {
        t = (ks <= kv_hi && ks >= kv_lo) ? t : -__builtin_inff();
      } else {
        t = ks <= kv_hi ? t : -__builtin_inff();
      }
    }
    sv[j] = t;
  };
  auto stageE = [&](f32x16& sv, auto jc) {
    constexpr int j = decltype(jc)::value;
    sv[j] = fast_exp2(sv[j]);
  };
  auto stageM = [&](f32x16& sv, f32x16& pv, u32x4* dsv, auto jc) {
    constexpr int j = decltype(jc)::value;
    pv[j] = sv[j] * pv[j];  // pv holds dP - Delta
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
    constexpr int PD = kDqPD;  // LDS operand reads in flight ahead of their MFMA
    // loop-variant bases so the per-step XORs are not hoisted out of the loop
    const int svn = svb + (n % NSTAGE) * STAGE;
    const int tan = tab + (n % NSTAGE) * STAGE, tbn = tbb + (n % NSTAGE) * STAGE;
    const int tap = tab + (n_prev % NSTAGE) * STAGE, tbp = tbb + (n_prev % NSTAGE) * STAGE;
    if constexpr (!DRAIN) {
      sc0 = f32x16{};
      pc0 = ndl;
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
        pc1 = ndl;
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

  // Tile loop.  The first tile is peeled (no previous half 1); the tiles
  // that need no mask run in one loop and the masked ones (the band's left
  // edge, its right edge or diagonal, the ragged last tile) in loops of
  // their own, so the matrix-core accumulators flow through straight loops
  // rather than branches.  Every wave loads its share of every tile of the
  // block and takes every barrier, also for the tiles it skips (below).
  if (n_begin < n_end) prefetch(n_begin);
  // The preprocess for this wave's rows, under the first tile's loads:
  // -Delta from O and dO, and the workspace rows that the dK/dV kernel
  // stages.  -Delta goes into every row of ndl: the dP^T products start from
  // it, so they leave dP^T - Delta and dS needs one multiply per element.
  Dl = -row_delta_pair<BF16>(of, df);
  if (stat_row >= 0) store_row_stats(a.delta, a.lse2, a.delta_out, stat_row, h, L2, Dl);
#pragma unroll
  for (int j = 0; j < 16; ++j) ndl[j] = Dl;
  // Tiles [n_begin, v_end) hold a key some row of this wave sees; past its
  // last row's diagonal (or band edge), and for a wave whose rows are all
  // past the end, the wave still loads and takes every barrier but issues
  // no products: those tiles would add exact zeros.
  int v_end = n_begin;
  if (qw < s.sq) {
    const int last_key = BANDED ? min(qw + 31, s.sq - 1) + off_causal + a.win_r : s.sk - 1;
    if (last_key >= 0) v_end = min(n_end, max(n_begin, last_key / BN + 1));
  }
  if (n_begin < n_end) {
    wait_vmcnt<0>();
    lds_barrier();
    if (n_begin + 1 < n_end) prefetch(n_begin + 1);
    if (v_end == n_begin) {
      // this wave sees no key of the block: loads and barriers only
    } else if (tile_masked(n_begin)) {
      run(n_begin, std::true_type{}, std::false_type{}, std::true_type{});
    } else {
      run(n_begin, std::true_type{}, std::false_type{}, std::false_type{});
    }
    // this wave's unmasked tiles [u_lo, u_hi): n*BN >= qw + 31 + off - win_l
    // and n*BN + BN-1 <= qw + off + win_r and n*BN + BN <= sk
    int u_lo = n_begin + 1, u_hi = min(n_end, s.sk / BN);
    if (BANDED) {
      const int lo = qw + 31 + off_causal - a.win_l;
      if (lo > 0) u_lo = max(u_lo, (lo + BN - 1) / BN);
      const int hi = qw + off_causal + a.win_r - (BN - 1);
      u_hi = hi < 0 ? 0 : min(u_hi, hi / BN + 1);
    }
    u_hi = min(u_hi, v_end);
    int n = n_begin + 1;
    const int e1 = min(min(u_lo, n_end), v_end);
    for (; n < e1; ++n) {
      wait_vmcnt<0>();
      lds_barrier();
      if (n + 1 < n_end) prefetch(n + 1);
      run(n, std::false_type{}, std::false_type{}, std::true_type{});
    }
    for (; n < u_hi; ++n) {
      wait_vmcnt<0>();
      lds_barrier();
      if (n + 1 < n_end) prefetch(n + 1);
      run(n, std::false_type{}, std::false_type{}, std::false_type{});
    }
    for (; n < v_end; ++n) {
      wait_vmcnt<0>();
      lds_barrier();
      if (n + 1 < n_end) prefetch(n + 1);
      run(n, std::false_type{}, std::false_type{}, std::true_type{});
    }
    // here n == v_end unless the wave saw no tile
    if (v_end > n_begin) {
      if (v_end < n_end) {
        wait_vmcnt<0>();
        lds_barrier();
        if (n + 1 < n_end) prefetch(n + 1);
        run(n, std::false_type{}, std::true_type{}, std::false_type{});
        ++n;
      } else {
        run(n_end, std::false_type{}, std::true_type{}, std::false_type{});
      }
    }
    for (; n < n_end; ++n) {
      wait_vmcnt<0>();
      lds_barrier();
      if (n + 1 < n_end) prefetch(n + 1);
    }
  }

  // ---- dQ * scale, rounded to nearest even: the pages' postprocess, fused.
  // Stored as 16-byte row chunks through this wave's LDS region once every
  // wave is past its last K-tile read.
  if (n_begin < n_end) lds_barrier();
  wait_vmcnt<0>();
  {
    constexpr int REG = 32 * TD * 72;
    static_assert(NW * REG <= NSTAGE * STAGE, "epilogue transpose fits the stages");
    const int rows_ok = min(BM, s.sq - q0) - 32 * w;
    const uint16_t* dqb = a.dq + s.bq * a.dq_b + (int64_t)(s.q0 + q0 + 32 * w) * a.dq_r + (int64_t)hq * a.dq_h;
    const rsrc_t rDQ = make_rsrc(dqb, rows_ok > 0 ? ((int64_t)(rows_ok - 1) * a.dq_r + hd) * 2 : 0);
    store_tile_rows<BF16, TD>(dq_acc, a.scale, smem + w * REG, rDQ, (int)a.dq_r, rows_ok, hd, lane);
  }
}


// ---------------------------------------------------------------------------
// dQ for the 256-wide head-dim tile (head dims 136 .. 256): one workgroup per
// (query head x sequence, 128-query block), 4 waves (one per SIMD), wave w
// owning queries 32w .. +32.  The lane's Q and dO (its column of S^T) stay in
// registers as B operands (128 registers), dQ accumulates in 8 head-dim tiles
// (128 accumulation registers).  Key tiles of 64 keys (K and V, 64 KiB) pass
// through two LDS stages, loaded one tile ahead by direct global->LDS loads.
// Per tile, as two 32-key halves: S^T and dP^T of both halves (alternating
// head-dim steps), dS^T on the vector ALU, then dQ += dS K; the straight-line
// body lets the compiler run half 0's softmax under half 1's products and
// half 1's under half 0's dQ products (with one wave per SIMD nothing else
// fills those gaps; 32-key tiles left them open).  (A software-pipelined
// version that ran the previous tile's dQ products under this tile's softmax
// needed more registers than one wave has and spilled.)
// ---------------------------------------------------------------------------
template <bool BF16, bool BANDED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_bwd_dq_wide_kernel(Args a) {
  constexpr int D = 256, NW = 4, BM = 32 * NW, BN = 64;
  static_assert(BM == kDqWideBM, "grid rows");
  constexpr int CPR = D / 8, RB = D * 2;
  constexpr int KT = BN * RB;                 // bytes of a K (or V) tile
  constexpr int STAGE = 2 * KT;
  constexpr int NSTAGE = 2;
  constexpr int TD = D / 32;                  // head-dim tiles of dQ
  constexpr int NSD = D / 16;                 // k-steps of S^T / dP^T
  constexpr int KI = BN * CPR / (64 * NW);    // direct loads per wave per K (or V) tile
  static_assert(KI >= 1 && NSTAGE * STAGE <= 160 * 1024, "tile shape");

  constexpr int SMEM = NSTAGE * STAGE > NW * 32 * TD * 72 ? NSTAGE * STAGE : NW * 32 * TD * 72;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM];
  const uint32_t smem_lds = lds_addr(smem);

  const int lane = threadIdx.x & 63;
  const int w = wave_id();
  const int h = lane >> 5;
  const int c32 = lane & 31;
  const int sl = lane & 15;
  const int gg = lane >> 4;
  const int rr = sl >> 2;
  const int tcol = 16 * (gg & 1) + 4 * (sl & 3);
  const int hq = blockIdx.x % a.heads_q;
  const int z = blockIdx.x / a.heads_q;
  const Seq s = seq_info(a, z);
  const int mb = BANDED ? (int)(gridDim.y - 1 - blockIdx.y) : (int)blockIdx.y;
  const int q0 = mb * BM;
  if (q0 >= s.sq) return;
  const int hd = a.head_dim;
  const int g = hq / a.group;
  const int off_causal = s.sk - s.sq;
  const int qw = q0 + 32 * w;
  const int qi = qw + c32;

  // O of the same rows and chunks: the preprocess's input (below).
  u32x4 qf[NSD], df[NSD], of[NSD];
  float L2, Dl;
  int64_t stat_row;  // workspace index of this lane's row, -1 past the end
  {
    const int rows = min(BM, s.sq - q0);
    const uint16_t* qb = a.q + s.bq * a.q_b + (int64_t)(s.q0 + q0) * a.q_r + (int64_t)hq * a.q_h;
    const uint16_t* db = a.dout + s.bq * a.do_b + (int64_t)(s.q0 + q0) * a.do_r + (int64_t)hq * a.do_h;
    const uint16_t* ob = a.o + s.bq * a.o_b + (int64_t)(s.q0 + q0) * a.o_r + (int64_t)hq * a.o_h;
    const rsrc_t rQ = make_rsrc(qb, ((int64_t)(rows - 1) * a.q_r + hd) * 2);
    const rsrc_t rO = make_rsrc(db, ((int64_t)(rows - 1) * a.do_r + hd) * 2);
    const rsrc_t rOut = make_rsrc(ob, ((int64_t)(rows - 1) * a.o_r + hd) * 2);
    const int row = 32 * w + c32;
#pragma unroll
    for (int sd = 0; sd < NSD; ++sd) {
      const int d0 = 16 * sd + 8 * h;
      const bool ok = d0 < hd;
      qf[sd] = buf_load128(rQ, ok ? (row * (int)a.q_r + d0) * 2 : kOffOOB);
      df[sd] = buf_load128(rO, ok ? (row * (int)a.do_r + d0) * 2 : kOffOOB);
      of[sd] = buf_load128(rOut, ok ? (row * (int)a.o_r + d0) * 2 : kOffOOB);
    }
    const int64_t st0 = s.stat0 + (int64_t)hq * s.stat_h + q0;
    L2 = buf_load_f32(make_rsrc(a.lse_in + st0, (int64_t)rows * 4), row * 4) * kLog2e;
    stat_row = row < rows ? st0 + row : -1;
  }

  f32x16 dq_acc[TD];
#pragma unroll
  for (int t = 0; t < TD; ++t) dq_acc[t] = f32x16{};

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

  int n_begin = 0, n_end = (s.sk + BN - 1) / BN;
  if (BANDED) {
    const Range kr = band_keys(a, q0, min(q0 + BM, s.sq) - 1, s.sq, s.sk);
    n_begin = kr.lo / BN;
    n_end = kr.hi < kr.lo ? n_begin : kr.hi / BN + 1;
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
  int kv_hi = s.sk - 1, kv_lo = -kWinInf;
  if (BANDED) {
    kv_hi = min(kv_hi, qi + off_causal + a.win_r);
    kv_lo = qi + off_causal - a.win_l;
  }
  kv_hi -= 4 * h;
  kv_lo -= 4 * h;

  // Tile n (stage n % 2): S^T, dP^T, dS^T, then dQ += dS K.  Tile n + 1 is
  // loaded into the other stage at the start of tile n, after the barrier
  // that ends every wave's reads of tile n - 1.
  if (n_begin < n_end) prefetch(n_begin);
  // the preprocess for this wave's rows, under the first tile's loads
  Dl = -row_delta_pair<BF16>(of, df);
  if (stat_row >= 0) store_row_stats(a.delta, a.lse2, a.delta_out, stat_row, h, L2, Dl);
  for (int n = n_begin; n < n_end; ++n) {
    wait_vmcnt<0>();
    lds_barrier();
    if (n + 1 < n_end) prefetch(n + 1);
    const int sv = svb + (n % NSTAGE) * STAGE;
    const int ta = tab + (n % NSTAGE) * STAGE, tb = tbb + (n % NSTAGE) * STAGE;
    const bool masked = (BANDED && (n * BN + BN - 1 > qw + off_causal + a.win_r || n * BN < qw + 31 + off_causal - a.win_l)) ||
                        (n * BN + BN > s.sk);
    // One wave per SIMD: every product's LDS operand is read kDqPD steps
    // ahead through a register ring, and each half's softmax runs one
    // element per product under the next products (half 0 under half 1's
    // S^T/dP^T, half 1 under half 0's dQ); the exps are pinned there (the
    // scheduling fences order only side effects).
    f32x16 sc[2], pc[2];
    u32x4 ds[2][2];
    auto soft = [&](int kh, int j) {  // dS^T element j of half kh, packed in pairs
      float t = __builtin_fmaf(sc[kh][j], a.scale_log2, -L2);
      const int ks = n * BN + 32 * kh + 8 * (j >> 2) + (j & 3);
      if (masked) t = (ks <= kv_hi && ks >= kv_lo) ? t : -__builtin_inff();
      float pv = fast_exp2(t);
      asm volatile("" : "+v"(pv));
      pc[kh][j] = pv * (pc[kh][j] + Dl);  // Dl holds -Delta
      if (j & 1) ds[kh][j >> 3][(j & 7) >> 1] = pack2<BF16>(pc[kh][j - 1], pc[kh][j]);
    };
    {
      // step i: half i / NSD, head-dim step i % NSD; a K and a V fragment
      constexpr int NS = 2 * NSD, PD = kDqPD;
      u32x4 fk[PD], fv[PD];
      auto rd = [&](int i, int slot) {
        const int o = (sv ^ (32 * (i % NSD))) + 32 * (i / NSD) * RB;
        fk[slot] = lds_rd128(smem, o);
        fv[slot] = lds_rd128(smem, o + KT);
      };
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        sc[kh] = f32x16{};
        pc[kh] = f32x16{};
      }
      sched_fence();
#pragma unroll
      for (int i = 0; i < PD; ++i) rd(i, i);
      sched_fence();
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const int kh = i / NSD, sd = i % NSD;
        const u32x4 ka = fk[i % PD], va = fv[i % PD];
        if (i + PD < NS) rd(i + PD, i % PD);
        sc[kh] = mfma32<BF16>(ka, qf[sd], sc[kh]);
        pc[kh] = mfma32<BF16>(va, df[sd], pc[kh]);
        if (kh == 1) soft(0, sd);
        sched_fence();
      }
    }
    {
      // step i: half i / (2*TD), 16-key step (i / TD) % 2, head-dim tile i % TD
      constexpr int NQ = 4 * TD, PD = kDqPD;
      u32x4 fb[PD];
      auto rd = [&](int i, int slot) {
        const int ro = (32 * (i / (2 * TD)) + 16 * ((i / TD) % 2)) * RB;
        const int t = i % TD;
        fb[slot] = tr_frag_b(smem, (ta ^ (64 * t)) + ro, (tb ^ (64 * t)) + ro);
      };
      sched_fence();
#pragma unroll
      for (int i = 0; i < PD; ++i) rd(i, i);
      sched_fence();
#pragma unroll
      for (int i = 0; i < NQ; ++i) {
        const int kh = i / (2 * TD), s2 = (i / TD) % 2;
        const u32x4 kb = fb[i % PD];
        if (i + PD < NQ) rd(i + PD, i % PD);
        dq_acc[i % TD] = mfma32<BF16>(ds[kh][s2], kb, dq_acc[i % TD]);
        if (i < 16) soft(1, i);
        sched_fence();
      }
    }
  }

  // dQ * scale, rounded, as 16-byte row chunks through LDS (every wave is
  // past its last K-tile read once the barrier below is passed).
  if (n_begin < n_end) lds_barrier();
  wait_vmcnt<0>();
  {
    constexpr int REG = 32 * TD * 72;
    static_assert(NW * REG <= sizeof(smem), "epilogue transpose fits");
    const int rows_ok = min(BM, s.sq - q0) - 32 * w;
    const uint16_t* dqb = a.dq + s.bq * a.dq_b + (int64_t)(s.q0 + q0 + 32 * w) * a.dq_r + (int64_t)hq * a.dq_h;
    const rsrc_t rDQ = make_rsrc(dqb, rows_ok > 0 ? ((int64_t)(rows_ok - 1) * a.dq_r + hd) * 2 : 0);
    store_tile_rows<BF16, TD>(dq_acc, a.scale, smem + w * REG, rDQ, (int)a.dq_r, rows_ok, hd, lane);
  }
}

}  // namespace attn
