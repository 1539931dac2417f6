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
// ---------------------------------------------------------------------------
template <bool BF16, int D, bool CAUSAL, bool DET>
__global__ __launch_bounds__(256) void attn_bwd_main_kernel(Args a) {
  constexpr int BM = kBwdBM, BN = kBwdBN;
  constexpr int LDQ = D + 8;     // row pitch of the Q / dO tiles (elements)
  constexpr int LDT = BM + 8;    // row pitch of the dS^T tile
  constexpr int TD = D / 32;     // head-dim tiles
  constexpr int TQ = BM / 32;    // query tiles per iteration
  constexpr int DQ_TQ = TQ * TD / 4;  // query tiles per wave in the dQ step
  constexpr int CPR = D / 8;
  constexpr int NCH = BM * CPR / 256;   // 16-byte chunks per thread per Q (or dO) tile
  constexpr int KCH = BN * CPR / 256;   // ... per K block
  static_assert(TQ * TD % 4 == 0 && DQ_TQ >= 1, "dQ tiles must split over 4 waves");
  static_assert(2 * BM >= BN, "K staging reuses the Q/dO tiles");

  __shared__ __attribute__((aligned(16))) uint16_t sQdO[2 * BM * LDQ];
  __shared__ __attribute__((aligned(16))) uint16_t sdST[BN * LDT];
  __shared__ __attribute__((aligned(16))) float sL[BM];
  __shared__ __attribute__((aligned(16))) float sDl[BM];
  uint16_t* sQ = sQdO;
  uint16_t* sdO = sQdO + BM * LDQ;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int h = lane >> 5;
  const int c32 = lane & 31;
  const int nb = blockIdx.x;
  const int g = blockIdx.y;
  const int z = blockIdx.z;
  const Seq s = seq_info(a, z);
  const int kv0 = nb * BN;
  if (kv0 >= s.sk) return;
  const int hd = a.head_dim;

  // ---- K, V of this wave's 32 key rows as B operands (k = head dim).
  const int kv_lane = kv0 + 32 * w + c32;
  const bool kv_ok = kv_lane < s.sk;
  const uint16_t* kbase = a.k + s.bk * a.k_b + (int64_t)s.k0 * a.k_r + (int64_t)g * a.k_h;
  const uint16_t* vbase = a.v + s.bk * a.v_b + (int64_t)s.k0 * a.v_r + (int64_t)g * a.v_h;
  u32x4 kf[D / 16], vf[D / 16];
#pragma unroll
  for (int sd = 0; sd < D / 16; ++sd) {
    const int d0 = 16 * sd + 8 * h;
    const bool ok = kv_ok && d0 < hd;
    kf[sd] = ok ? ldg128(kbase + (int64_t)kv_lane * a.k_r + d0) : u32x4{0u, 0u, 0u, 0u};
    vf[sd] = ok ? ldg128(vbase + (int64_t)kv_lane * a.v_r + d0) : u32x4{0u, 0u, 0u, 0u};
  }

  // ---- K as the B operand of dQ = dS K (k = key), for this wave's head-dim
  // slice: stage the K block in LDS, then read it with the transpose read.
  const int td_w = w % TD;            // head-dim tile of this wave in the dQ step
  const int tq_w = (w / TD) * DQ_TQ;  // first query tile of this wave in the dQ step
  u32x4 ktf[BN / 16];
  {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int id = tid + 256 * i;
      const int r = id / CPR, c = id % CPR;
      const int row = kv0 + r;
      const bool ok = row < s.sk && 8 * c < hd;
      sts128(sQdO + r * LDQ + 8 * c, ok ? ldg128(kbase + (int64_t)row * a.k_r + 8 * c) : u32x4{0u, 0u, 0u, 0u});
    }
    __syncthreads();
    const uint16_t* kp = sQdO + 32 * td_w + tr_lane_offset(lane, LDQ);
#pragma unroll
    for (int sk_ = 0; sk_ < BN / 16; ++sk_) ktf[sk_] = tr_frag(kp, LDQ, 16 * sk_ + 8 * h, 16 * sk_ + 8 * h + 4);
    __syncthreads();
  }

  f32x16 dk_acc[TD], dv_acc[TD];
#pragma unroll
  for (int t = 0; t < TD; ++t) {
    dk_acc[t] = f32x16{};
    dv_acc[t] = f32x16{};
  }

  const int troffQ = tr_lane_offset(lane, LDQ);
  const int troffT = tr_lane_offset(lane, LDT);
  const int m_begin = first_q_block<BM, BN, CAUSAL>(nb, s.sq, s.sk);
  const int m_end = (s.sq + BM - 1) / BM;

  for (int hq = g * a.group; hq < (g + 1) * a.group; ++hq) {
    if (m_begin >= m_end) break;
    const uint16_t* qb = a.q + s.bq * a.q_b + (int64_t)s.q0 * a.q_r + (int64_t)hq * a.q_h;
    const uint16_t* db = a.dout + s.bq * a.do_b + (int64_t)s.q0 * a.do_r + (int64_t)hq * a.do_h;
    const int64_t st0 = s.stat0 + (int64_t)hq * s.stat_h;
    float* accp = a.dq_acc + acc_base(a, s, hq) + (DET ? (int64_t)nb * a.acc_split : 0);

    u32x4 qreg[NCH], doreg[NCH];
    float lreg = 0.f, dlreg = 0.f;
    auto load_tile = [&](int m) {
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int id = tid + 256 * i;
        const int r = id / CPR, c = id % CPR;
        const int row = m * BM + r;
        const bool ok = row < s.sq && 8 * c < hd;
        qreg[i] = ok ? ldg128(qb + (int64_t)row * a.q_r + 8 * c) : u32x4{0u, 0u, 0u, 0u};
        doreg[i] = ok ? ldg128(db + (int64_t)row * a.do_r + 8 * c) : u32x4{0u, 0u, 0u, 0u};
      }
      if (tid < BM) {
        const int row = m * BM + tid;
        const bool ok = row < s.sq;
        lreg = ok ? a.lse_in[st0 + row] * kLog2e : INFINITY;  // P = 0 on rows past the end
        dlreg = ok ? a.delta[st0 + row] : 0.f;
      }
    };

    load_tile(m_begin);
    for (int m = m_begin; m < m_end; ++m) {
      // Tile m into LDS (all waves finished the previous iteration's reads of
      // sQ/sdO before its second barrier, and of sdST before this one).
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int id = tid + 256 * i;
        const int r = id / CPR, c = id % CPR;
        sts128(sQ + r * LDQ + 8 * c, qreg[i]);
        sts128(sdO + r * LDQ + 8 * c, doreg[i]);
      }
      if (tid < BM) {
        sL[tid] = lreg;
        sDl[tid] = dlreg;
      }
      __syncthreads();
      if (m + 1 < m_end) load_tile(m + 1);

      // S = Q K^T and dP = dO V^T for this wave's 32 key columns.
      f32x16 sacc[TQ], pacc[TQ];
#pragma unroll
      for (int tq = 0; tq < TQ; ++tq) {
        sacc[tq] = f32x16{};
        pacc[tq] = f32x16{};
#pragma unroll
        for (int sd = 0; sd < D / 16; ++sd) {
          const int off = (32 * tq + c32) * LDQ + 16 * sd + 8 * h;
          sacc[tq] = mfma32<BF16>(lds128(sQ + off), kf[sd], sacc[tq]);
          pacc[tq] = mfma32<BF16>(lds128(sdO + off), vf[sd], pacc[tq]);
        }
      }

      // P and dS in registers.  C layout: lane = key column kv_lane, rows =
      // queries 32*tq + 8*(j/4) + 4*h + j%4.
#pragma unroll
      for (int tq = 0; tq < TQ; ++tq) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int qr = 32 * tq + 8 * jj + 4 * h;
          const f32x4 L = *reinterpret_cast<const f32x4*>(sL + qr);
          const f32x4 Dl = *reinterpret_cast<const f32x4*>(sDl + qr);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int j = 4 * jj + r;
            const int qi = m * BM + qr + r;
            bool vis = kv_ok;
            if (CAUSAL) vis = vis && (kv_lane <= qi + (s.sk - s.sq));
            const float p = vis ? fast_exp2(sacc[tq][j] * a.scale_log2 - L[r]) : 0.f;
            const float ds = p * (pacc[tq][j] - Dl[r]);
            sacc[tq][j] = p;
            pacc[tq][j] = ds;
          }
        }
      }

      // dV += P^T dO and dK += dS^T Q (reduction over the 64 queries).
#pragma unroll
      for (int tq = 0; tq < TQ; ++tq) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          u32x4 pf, dsf;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            pf[e] = pack2<BF16>(sacc[tq][8 * s2 + 2 * e], sacc[tq][8 * s2 + 2 * e + 1]);
            dsf[e] = pack2<BF16>(pacc[tq][8 * s2 + 2 * e], pacc[tq][8 * s2 + 2 * e + 1]);
          }
          const int ra = 32 * tq + 16 * s2 + 4 * h;
#pragma unroll
          for (int t = 0; t < TD; ++t) {
            const u32x4 bo = tr_frag(sdO + 32 * t + troffQ, LDQ, ra, ra + 8);
            dv_acc[t] = mfma32<BF16>(pf, bo, dv_acc[t]);
            const u32x4 bq = tr_frag(sQ + 32 * t + troffQ, LDQ, ra, ra + 8);
            dk_acc[t] = mfma32<BF16>(dsf, bq, dk_acc[t]);
          }
        }
      }

      // dS^T -> LDS as [key][query]: 4 consecutive queries per 8-byte store.
      {
        uint16_t* row = sdST + (32 * w + c32) * LDT + 4 * h;
#pragma unroll
        for (int tq = 0; tq < TQ; ++tq) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            u32x2 v2;
            v2[0] = pack2<BF16>(pacc[tq][4 * jj], pacc[tq][4 * jj + 1]);
            v2[1] = pack2<BF16>(pacc[tq][4 * jj + 2], pacc[tq][4 * jj + 3]);
            *reinterpret_cast<u32x2*>(row + 32 * tq + 8 * jj) = v2;
          }
        }
      }
      __syncthreads();

      // dQ slice = dS K for query tiles tq_w.. and head-dim tile td_w.
#pragma unroll
      for (int k = 0; k < DQ_TQ; ++k) {
        const int tq = tq_w + k;
        f32x16 qacc = f32x16{};
        const uint16_t* dp = sdST + 32 * tq + troffT;
#pragma unroll
        for (int sk_ = 0; sk_ < BN / 16; ++sk_) {
          const u32x4 af = tr_frag(dp, LDT, 16 * sk_ + 8 * h, 16 * sk_ + 8 * h + 4);
          qacc = mfma32<BF16>(af, ktf[sk_], qacc);
        }
        const int d = 32 * td_w + c32;
        if (d < hd) {
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int qi = m * BM + 32 * tq + 8 * (j >> 2) + 4 * h + (j & 3);
            if (qi < s.sq) {
              float* dst = accp + (int64_t)qi * hd + d;
              if (DET) {
                *dst = qacc[j];
              } else {
                atomicAdd(dst, qacc[j]);
              }
            }
          }
        }
      }
    }
  }

  // ---- Epilogue: dK * scale, dV; convert (round to nearest even) and store.
  uint16_t* dkb = a.dk + s.bk * a.dk_b + (int64_t)s.k0 * a.dk_r + (int64_t)g * a.dk_h;
  uint16_t* dvb = a.dv + s.bk * a.dv_b + (int64_t)s.k0 * a.dv_r + (int64_t)g * a.dv_h;
#pragma unroll
  for (int t = 0; t < TD; ++t) {
    const int d = 32 * t + c32;
    if (d >= hd) continue;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int kv = kv0 + 32 * w + 8 * (j >> 2) + 4 * h + (j & 3);
      if (kv < s.sk) {
        dkb[(int64_t)kv * a.dk_r + d] = to_bits<BF16>(dk_acc[t][j] * a.scale);
        dvb[(int64_t)kv * a.dv_r + d] = to_bits<BF16>(dv_acc[t][j]);
      }
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
