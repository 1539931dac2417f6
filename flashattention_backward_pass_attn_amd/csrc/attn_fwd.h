// Attention forward on gfx950: O = softmax(scale * Q K^T, masked) V and the
// natural-log LSE the backward pass consumes.
//
// Method: tilelang test_tilelang_kernel_mha_bwd.py, flashattn_fwd -- one
// workgroup per (query block, head, batch), an online softmax over key blocks
// in the exp2 domain with scale*log2(e) folded into one constant, rescaling
// the running output when the row maximum grows, and the final division by
// the row sum.  The stored statistic is converted to natural log, the form the
// flash-attention CK mha_bwd.cpp page's softmax_lse takes.
//
// gfx950 design (not the page's): wave64s each owning 32 query rows (8 per
// workgroup, two per SIMD, up to head dim 128; 4 for the 256-wide tile); the
// score tile is computed transposed, S^T = K Q^T, so that every lane holds one
// query row (its column) -- the row max / row sum need only an in-lane
// reduction plus one exchange between the two lane halves, and the
// probabilities P^T leave the MFMA already in the operand layout of
// O^T += V^T P^T.  V^T is read from the row-major V tile in LDS with the LDS
// transpose read, so no transposed copy is written.  Q stays in registers for
// the whole kernel; K/V blocks come straight from global memory into two LDS
// stages (direct global->LDS loads, one block ahead), laid out with the
// 16-byte-chunk swizzle that keeps both the row reads of K and the transposed
// reads of V free of bank conflicts, and each product's operand is read a
// few products ahead through a ring of registers.
#pragma once

#include "attn_device.h"

namespace attn {

// Waves per workgroup, 32 query rows each: 8 (two per SIMD) up to head dim
// 128, 4 (one per SIMD) for the 256-wide tile.
constexpr int fwd_waves(int d) { return d > 128 ? 4 : 8; }
constexpr int fwd_bm(int d) { return 32 * fwd_waves(d); }  // query rows per workgroup
// Key rows per block: 128 with two waves per SIMD (half the blocks, so half
// the barriers and softmax passes per key; 3 % faster than 64 in an A/B
// run), 64 for the 256-wide tile (its stages would not fit twice as long).
constexpr int fwd_bn(int d) { return d > 128 ? 64 : 128; }
// The running row maximum (log2 units) is moved only when a row grows past it
// by more than this, so P <= 2^8 = 256: exact in fp32 sums, and within the
// fp16 and bf16 range of the P operand.
constexpr float kFwdRescaleSlack = 8.f;
// LDS operand reads in flight ahead of their product
constexpr int kFwdPD = 4;

// Head dims up to 128 run two waves per SIMD; the 256-wide tile (Q and the
// O accumulator in registers) runs one.
constexpr int fwd_waves_per_simd(int d) { return d > 128 ? 1 : 2; }

template <bool BF16, int D, int DC, bool BANDED>
__global__ __launch_bounds__(64 * fwd_waves(D)) __attribute__((amdgpu_waves_per_eu(fwd_waves_per_simd(D), fwd_waves_per_simd(D))))
void attn_fwd_kernel(Args a) {
  static_assert(DC % 32 == 0 && DC <= D, "compute width: 32-column tiles within the stored tile");
  constexpr int NW = fwd_waves(D);
  constexpr int BM = fwd_bm(D), BN = fwd_bn(D);
  constexpr int CPR = D / 8;              // 16-byte chunks per row
  constexpr int RB = D * 2;               // bytes per row
  constexpr int TILE = BN * RB;           // one K (or V) block
  constexpr int STAGE = 2 * TILE;         // K then V
  constexpr int NT = 64 * NW;             // threads
  constexpr int NCH = BN * CPR / NT;      // direct loads per thread per K (or V) block
  constexpr int TK = BN / 32;             // key tiles per block
  constexpr int TD = DC / 32;             // head-dim tiles computed
  static_assert(BN * CPR % NT == 0, "tile/thread mismatch");

  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STAGE];
  const uint32_t smem_lds = lds_addr(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int h = lane >> 5;
  const int c32 = lane & 31;
  // grid (query head x sequence, query block), block index slowest: the
  // longest causal blocks of every head start first, and one head's blocks
  // share an XCD (and its L2 copy of K and V).
  const int hq = blockIdx.x % a.heads_q;
  const int z = blockIdx.x / a.heads_q;
  const Seq s = seq_info(a, z);
  const int qb0 = (BANDED ? (int)(gridDim.y - 1 - blockIdx.y) : (int)blockIdx.y) * BM;
  if (qb0 >= s.sq) return;
  const int g = hq / a.group;
  const int hd = a.head_dim;

  // This lane's query row (a column of S^T); the wave's first query.
  const int qw = qb0 + 32 * w;
  const int qi = qw + c32;
  const int off = s.sk - s.sq;  // bottom-right alignment of the band
  const bool q_ok = qi < s.sq;

  // Q as the B operand of S^T = K Q^T: column qi, k = head dim.
  u32x4 qf[DC / 16];
  {
    const uint16_t* qp = a.q + s.bq * a.q_b + (int64_t)(s.q0 + qi) * a.q_r + (int64_t)hq * a.q_h;
#pragma unroll
    for (int st = 0; st < DC / 16; ++st) {
      const int d0 = 16 * st + 8 * h;
      qf[st] = (q_ok && d0 < hd) ? ldg128(qp + d0) : u32x4{0u, 0u, 0u, 0u};
    }
  }

  // Key blocks this query block sees.
  int n_begin = 0, n_end = (s.sk + BN - 1) / BN;
  if (BANDED) {
    const Range kr = band_keys(a, qb0, min(qb0 + BM, s.sq) - 1, s.sq, s.sk);
    n_begin = kr.lo / BN;
    n_end = kr.hi < kr.lo ? n_begin : kr.hi / BN + 1;
  }

  const uint16_t* kbase = a.k + s.bk * a.k_b + (int64_t)s.k0 * a.k_r + (int64_t)g * a.k_h;
  const uint16_t* vbase = a.v + s.bk * a.v_b + (int64_t)s.k0 * a.v_r + (int64_t)g * a.v_h;
  // One descriptor per tensor over the head's rows; a block is a 32-bit lane
  // offset into it.  Rows past the end and columns past head_dim read as 0.
  const u32x4 srdK = make_srd(kbase, ((int64_t)(s.sk - 1) * a.k_r + hd) * 2);
  const u32x4 srdV = make_srd(vbase, ((int64_t)(s.sk - 1) * a.v_r + hd) * 2);
  // 16-byte slot S of a block's LDS image holds row S / CPR, chunk
  // (S % CPR) ^ swz(row).
  int kdma[NCH], vdma[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int S = (i * NW + w) * 64 + lane;
    const int r = S / CPR;
    const int c = (S % CPR) ^ swz<CPR>(r);
    kdma[i] = 8 * c < hd ? (r * (int)a.k_r + 8 * c) * 2 : kOffOOB;
    vdma[i] = 8 * c < hd ? (r * (int)a.v_r + 8 * c) * 2 : kOffOOB;
  }
  auto prefetch = [&](int nb, int st) {
    const uint32_t stage = smem_lds + st * STAGE;
    const uint32_t tk = (uint32_t)(nb * BN) * (uint32_t)a.k_r * 2u;
    const uint32_t tv = (uint32_t)(nb * BN) * (uint32_t)a.v_r * 2u;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const uint32_t dst = stage + (uint32_t)((i * NW + w) * 64) * 16u;
      dma16(srdK, kdma[i] == kOffOOB ? kOffOOB : (int)((uint32_t)kdma[i] + tk), dst);
      dma16(srdV, vdma[i] == kOffOOB ? kOffOOB : (int)((uint32_t)vdma[i] + tv), dst + TILE);
    }
  };
  // K rows as the A operand of S^T (row = key c32 of a 32-key tile, k = head
  // dim 16*sd + 8*h): step sd is at kvb ^ 32*sd (the swizzle permutes chunk
  // bits only).  V^T for O^T += V^T P^T with the transposed read: key rows
  // 4*h + rr (+8) of a 16-key step, head-dim columns 32*t + tcol.
  const int sl = lane & 15;
  const int kvb = tile_off<CPR>(c32, 8 * h);
  const int rr = sl >> 2;
  const int tcol = 16 * ((lane >> 4) & 1) + 4 * (sl & 3);
  int va[TD], vb[TD];
#pragma unroll
  for (int t = 0; t < TD; ++t) {
    va[t] = tile_off<CPR>(4 * h + rr, 32 * t + tcol);
    vb[t] = tile_off<CPR>(4 * h + rr + 8, 32 * t + tcol);
  }

  f32x16 oacc[TD];
#pragma unroll
  for (int t = 0; t < TD; ++t) oacc[t] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  if (n_begin < n_end) {
    prefetch(n_begin, 0);
    wait_vmcnt<0>();
    lds_barrier();
  }
  int st = 0;
  for (int nb = n_begin; nb < n_end; ++nb) {
    // the other stage was last read in the previous block (barrier below)
    if (nb + 1 < n_end) prefetch(nb + 1, st ^ 1);
    const int sbase = st * STAGE;

    // S^T (keys x queries) for this lane's 32 query columns.
    // The K operands are read kFwdPD products ahead (a ring of registers),
    // so each product waits for a read issued several products earlier.
    f32x16 sc[TK];
#pragma unroll
    for (int tk = 0; tk < TK; ++tk) sc[tk] = f32x16{};
    {
      constexpr int NSD = DC / 16, NS = TK * NSD, PD = kFwdPD;
      u32x4 fr[PD];
      auto rd = [&](int i, int slot) {  // step i: key tile i / NSD, head-dim step i % NSD
        fr[slot] = lds_rd128(smem, (sbase + 32 * (i / NSD) * RB + kvb) ^ (32 * (i % NSD)));
      };
      sched_fence();
#pragma unroll
      for (int i = 0; i < PD; ++i) rd(i, i);
      sched_fence();
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const u32x4 op = fr[i % PD];
        if (i + PD < NS) rd(i + PD, i % PD);
        sc[i / NSD] = mfma32<BF16>(op, qf[i % NSD], sc[i / NSD]);
        sched_fence();
      }
    }
    // The first V^T operands of O^T += V^T P^T do not depend on P: read them
    // now, under the softmax.
    constexpr int NO = TK * 2 * TD, PDO = kFwdPD;
    u32x4 fb[PDO];
    auto rdo = [&](int i, int slot) {  // step i: key tile, 16-key step, head-dim tile
      const int ro = sbase + TILE + (32 * (i / (2 * TD)) + 16 * ((i / TD) % 2)) * RB;
      fb[slot] = tr_frag_b(smem, ro + va[i % TD], ro + vb[i % TD]);
    };
#pragma unroll
    for (int i = 0; i < PDO; ++i) rdo(i, i);

    // Mask (only on tiles crossing an edge of the band or the last key),
    // row max over keys, exp2 with scale*log2(e) folded into the fma.
    // Masked scores become -inf; max(scale*log2e*s) = scale*log2e*max(s).
    const bool masked = (BANDED && (nb * BN + BN - 1 > qw + off + a.win_r || nb * BN < qw + 31 + off - a.win_l)) ||
                        nb * BN + BN > s.sk;
    if (masked) {
      const int kv_hi = min(s.sk - 1, BANDED ? qi + off + a.win_r : s.sk - 1) - 4 * h;
      const int kv_lo = (BANDED ? qi + off - a.win_l : -kWinInf) - 4 * h;
#pragma unroll
      for (int tk = 0; tk < TK; ++tk) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int ks = nb * BN + 32 * tk + 8 * (j >> 2) + (j & 3);  // key minus the lane's 4*h
          sc[tk][j] = (ks <= kv_hi && ks >= kv_lo) ? sc[tk][j] : -INFINITY;
        }
      }
    }
    // Row max.  With one wave per SIMD (the 256-wide tile) nothing else
    // fills the latency of a 32-long dependent chain: a tree of depth 5
    // (measured 10 % faster there); with two waves the chain is as fast.
    float mx = -INFINITY;
    if constexpr (NW == 4) {
      float mt[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        mt[j] = sc[0][j];
#pragma unroll
        for (int tk = 1; tk < TK; ++tk) mt[j] = fmaxf(mt[j], sc[tk][j]);
      }
#pragma unroll
      for (int wdt = 8; wdt >= 1; wdt /= 2) {
#pragma unroll
        for (int j = 0; j < wdt; ++j) mt[j] = fmaxf(mt[j], mt[j + wdt]);
      }
      mx = mt[0];
    } else {
#pragma unroll
      for (int tk = 0; tk < TK; ++tk) {
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sc[tk][j]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32)) * a.scale_log2;
    // Lazy rescaling: the exponent reference m_run moves only when some row
    // of the wave grew by more than kFwdRescaleSlack (log2 units); otherwise
    // P may exceed 1 by up to 2^kFwdRescaleSlack, O and the row sum keep
    // their scale, and the multiply of the O accumulator is skipped.  O / l
    // and the LSE m_run + log2(l) are the same with either reference.
    const bool rescale = __builtin_amdgcn_ballot_w64(mx > m_run + kFwdRescaleSlack) != 0;
    float m_use, alpha = 1.f;
    if (rescale) {
      const float m_new = fmaxf(m_run, mx);
      m_use = (m_new == -INFINITY) ? 0.f : m_new;
      alpha = fast_exp2(m_run - m_use);
      m_run = m_new;
    } else {
      m_use = (m_run == -INFINITY) ? 0.f : m_run;
    }
    float ls = 0.f;
    if constexpr (NW == 4) {
#pragma unroll
      for (int tk = 0; tk < TK; ++tk) {
#pragma unroll
        for (int j = 0; j < 16; ++j) sc[tk][j] = fast_exp2(__builtin_fmaf(sc[tk][j], a.scale_log2, -m_use));
      }
      // row sum as a tree, in a fixed order
      float lt[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        lt[j] = sc[0][j];
#pragma unroll
        for (int tk = 1; tk < TK; ++tk) lt[j] += sc[tk][j];
      }
#pragma unroll
      for (int wdt = 8; wdt >= 1; wdt /= 2) {
#pragma unroll
        for (int j = 0; j < wdt; ++j) lt[j] += lt[j + wdt];
      }
      ls = lt[0];
    } else {
#pragma unroll
      for (int tk = 0; tk < TK; ++tk) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float p = fast_exp2(__builtin_fmaf(sc[tk][j], a.scale_log2, -m_use));
          sc[tk][j] = p;
          ls += p;
        }
      }
    }
    ls += __shfl_xor(ls, 32);
    l_run = l_run * alpha + ls;
    if (rescale) {
#pragma unroll
      for (int t = 0; t < TD; ++t) oacc[t] *= alpha;
    }

    // O^T += V^T P^T: P^T leaves the MFMA in B-operand layout (k = keys).
    u32x4 pf[TK][2];
#pragma unroll
    for (int tk = 0; tk < TK; ++tk) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) pf[tk][s2][e] = pack2<BF16>(sc[tk][8 * s2 + 2 * e], sc[tk][8 * s2 + 2 * e + 1]);
      }
    }
    sched_fence();
#pragma unroll
    for (int i = 0; i < NO; ++i) {
      const u32x4 op = fb[i % PDO];
      if (i + PDO < NO) rdo(i + PDO, i % PDO);
      oacc[i % TD] = mfma32<BF16>(op, pf[i / (2 * TD)][(i / TD) % 2], oacc[i % TD]);
      sched_fence();
    }
    wait_vmcnt<0>();  // block nb + 1 landed (this wave's share)
    lds_barrier();    // everyone's share; every wave is done with stage st
    st ^= 1;
  }

  // Normalise and store.  O^T tile: lane column = query qi, rows = head dim in
  // runs of 4 consecutive elements -> one 8-byte store per run.
  const float inv_l = l_run > 0.f ? 1.f / l_run : 0.f;
  if (q_ok) {
    uint16_t* op = a.out_o + s.bq * a.o_b + (int64_t)(s.q0 + qi) * a.o_r + (int64_t)hq * a.o_h;
#pragma unroll
    for (int t = 0; t < TD; ++t) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d0 = 32 * t + 8 * jj + 4 * h;
        if (d0 < hd) {
          u32x2 pk;
          pk[0] = pack2<BF16>(oacc[t][4 * jj] * inv_l, oacc[t][4 * jj + 1] * inv_l);
          pk[1] = pack2<BF16>(oacc[t][4 * jj + 2] * inv_l, oacc[t][4 * jj + 3] * inv_l);
          *reinterpret_cast<u32x2*>(op + d0) = pk;
        }
      }
    }
    if (h == 0) {
      const float lse = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : INFINITY;
      a.lse_out[s.stat0 + (int64_t)hq * s.stat_h + qi] = lse;
    }
  }
}

}  // namespace attn
