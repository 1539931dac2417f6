// Host side of libattn.so: argument validation, workspace sizing and kernel
// dispatch for the C ABI declared in include/attn.h.
//
// Validation mirrors the flash-attention CK mha_bwd.cpp page's mha_bwd checks
// (fp16/bf16 only and all tensors of one dtype; contiguous last dimension;
// batch > 0; head_dim % 8 == 0 and <= 256; heads_q % heads_kv == 0), returning
// a status code instead of throwing.  Nothing is launched unless every check
// passes.  Launch order follows the Hopper flash_bwd_launch_template.h page's
// run_flash_bwd: the preprocess first, then the gradient kernels, all on the
// caller's stream.  Here the gradients come from two kernels (dK/dV
// KV-stationary, dQ Q-stationary) instead of one kernel with fp32 dQ atomics
// plus a dQ postprocess; see attn_bwd_split.h for why.  The only workspace is
// O(Sq) per head: Delta and LSE * log2(e).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "attn.h"
#include "attn_bwd.h"
#include "attn_bwd_dq.h"
#include "attn_bwd_split.h"
#include "attn_device.h"
#include "attn_fwd.h"

namespace {

using attn::Args;

constexpr size_t kAlign = 256;

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool strides_ok(const attn_strides& s, bool varlen) {
  // 16-byte vector access needs every stride to be a multiple of 8 elements.
  if (s.row <= 0 || s.head <= 0) return false;
  if (s.row % 8 || s.head % 8) return false;
  if (!varlen && (s.batch < 0 || s.batch % 8)) return false;
  return true;
}

attn_status validate_common(const attn_params* p) {
  if (!p) return ATTN_ERR_INVALID_ARGUMENT;
  if (p->dtype != ATTN_FP16 && p->dtype != ATTN_BF16) return ATTN_ERR_INVALID_ARGUMENT;
  if (p->batch <= 0) return ATTN_ERR_INVALID_ARGUMENT;
  if (p->heads_q <= 0 || p->heads_kv <= 0) return ATTN_ERR_INVALID_ARGUMENT;
  if (p->heads_q % p->heads_kv) return ATTN_ERR_INVALID_ARGUMENT;
  if (p->head_dim <= 0 || p->head_dim % 8 || p->head_dim > 256) return ATTN_ERR_INVALID_ARGUMENT;
  if (p->seqlen_q < 0 || p->seqlen_k < 0) return ATTN_ERR_INVALID_ARGUMENT;
  if (p->causal != 0 && p->causal != 1) return ATTN_ERR_INVALID_ARGUMENT;
  if (p->window_left < -1 || p->window_right < -1) return ATTN_ERR_INVALID_ARGUMENT;
  if (p->deterministic != 0 && p->deterministic != 1) return ATTN_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(p->softmax_scale) || !(p->softmax_scale > 0.f)) return ATTN_ERR_INVALID_ARGUMENT;
  const bool vq = p->cu_seqlens_q != nullptr, vk = p->cu_seqlens_k != nullptr;
  if (vq != vk) return ATTN_ERR_INVALID_ARGUMENT;
  if (vq && (p->total_q < 0 || p->total_k < 0)) return ATTN_ERR_INVALID_ARGUMENT;
  // launch-grid limits: head x sequence in grid x, blocks of >= 64 rows in grid y/x
  if (p->heads_q > 65535 || p->batch > 65535) return ATTN_ERR_UNSUPPORTED;
  if ((int64_t)p->heads_q * p->batch > 0x7fffffff) return ATTN_ERR_UNSUPPORTED;
  if (p->seqlen_q > 65535 * 64 || p->seqlen_k > 65535 * 64) return ATTN_ERR_UNSUPPORTED;
  // the kernels address one head of one sequence with 32-bit byte offsets
  // (plus a sentinel just below 2^31): each tensor's per-head extent must
  // stay under 1 GiB
  {
    const attn_strides* qs[] = {&p->q, &p->o, &p->dout, &p->dq};
    const attn_strides* ks[] = {&p->k, &p->v, &p->dk, &p->dv};
    for (const attn_strides* st : qs)
      if ((int64_t)p->seqlen_q * st->row * 2 >= (int64_t)1 << 30) return ATTN_ERR_UNSUPPORTED;
    for (const attn_strides* st : ks)
      if ((int64_t)p->seqlen_k * st->row * 2 >= (int64_t)1 << 30) return ATTN_ERR_UNSUPPORTED;
  }
  return ATTN_OK;
}

bool is_varlen(const attn_params* p) { return p->cu_seqlens_q != nullptr; }

// The banded-mask kernels run for causal and for any bounded window side.
bool banded(const attn_params* p) { return p->causal != 0 || p->window_left >= 0 || p->window_right >= 0; }

// Query-side / key-side tensors may be NULL only when they hold no element.
bool q_empty(const attn_params* p) { return is_varlen(p) ? p->total_q == 0 : p->seqlen_q == 0; }
bool k_empty(const attn_params* p) { return is_varlen(p) ? p->total_k == 0 : p->seqlen_k == 0; }

int64_t stat_count(const attn_params* p) {
  return is_varlen(p) ? (int64_t)p->heads_q * p->total_q
                      : (int64_t)p->batch * p->heads_q * p->seqlen_q;
}

// One fp32 row statistic laid out like lse, and the workspace: Delta, then
// LSE * log2(e) (both written by the preprocess), each rounded up to 256
// bytes.  That is all the backward needs: the gradient kernels recompute P
// and dS tile by tile and keep dQ in registers.
size_t stat_bytes(const attn_params* p) {
  return round_up((size_t)stat_count(p) * sizeof(float), kAlign);
}
size_t workspace_bytes(const attn_params* p) { return 2 * stat_bytes(p); }

Args make_args(const attn_params* p) {
  Args a;
  std::memset(&a, 0, sizeof(a));
  const bool vl = is_varlen(p);
  a.cu_q = p->cu_seqlens_q;
  a.cu_k = p->cu_seqlens_k;
  auto set = [&](const attn_strides& s, int64_t& b, int64_t& r, int64_t& h) {
    b = vl ? 0 : s.batch;
    r = s.row;
    h = s.head;
  };
  set(p->q, a.q_b, a.q_r, a.q_h);
  set(p->k, a.k_b, a.k_r, a.k_h);
  set(p->v, a.v_b, a.v_r, a.v_h);
  set(p->o, a.o_b, a.o_r, a.o_h);
  set(p->dout, a.do_b, a.do_r, a.do_h);
  set(p->dq, a.dq_b, a.dq_r, a.dq_h);
  set(p->dk, a.dk_b, a.dk_r, a.dk_h);
  set(p->dv, a.dv_b, a.dv_r, a.dv_h);
  a.batch = p->batch;
  a.seqlen_q = p->seqlen_q;
  a.seqlen_k = p->seqlen_k;
  a.heads_q = p->heads_q;
  a.heads_kv = p->heads_kv;
  a.group = p->heads_q / p->heads_kv;
  a.head_dim = p->head_dim;
  a.total_q = vl ? p->total_q : 0;
  a.scale = p->softmax_scale;
  a.scale_log2 = p->softmax_scale * attn::kLog2e;
  a.varlen = vl ? 1 : 0;
  // banded mask: causal is (no left bound, right bound 0); a side of the
  // window wider than any offset is no bound
  const int wr = p->causal ? 0 : p->window_right;
  const int wl = p->window_left;
  a.win_l = (wl < 0 || wl >= attn::kWinInf) ? attn::kWinInf : wl;
  a.win_r = (wr < 0 || wr >= attn::kWinInf) ? attn::kWinInf : wr;
  return a;
}

attn_status last_hip_status() {
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

// ---- dispatch helpers ------------------------------------------------------
template <bool BF16, int D, int DC>
void launch_fwd_d(const Args& a, bool causal, dim3 grid, hipStream_t st) {
  if (causal)
    hipLaunchKernelGGL((attn::attn_fwd_kernel<BF16, D, DC, true>), grid, dim3(64 * attn::fwd_waves(D)), 0, st, a);
  else
    hipLaunchKernelGGL((attn::attn_fwd_kernel<BF16, D, DC, false>), grid, dim3(64 * attn::fwd_waves(D)), 0, st, a);
}

template <bool BF16>
void launch_fwd(const Args& a, int dcomp, bool causal, dim3 grid, hipStream_t st) {
  if (dcomp == 64)
    launch_fwd_d<BF16, 64, 64>(a, causal, grid, st);
  else if (dcomp == 96)
    launch_fwd_d<BF16, 128, 96>(a, causal, grid, st);
  else if (dcomp == 128)
    launch_fwd_d<BF16, 128, 128>(a, causal, grid, st);
  else
    launch_fwd_d<BF16, 256, 256>(a, causal, grid, st);
}

template <bool BF16, int D, int DC>
void launch_dkdv_d(const Args& a, bool causal, bool small_wg, dim3 grid_kv, hipStream_t st) {
  if constexpr (D <= 128) {
    if (small_wg) {  // causal only (dkdv_small_wg)
      hipLaunchKernelGGL((attn::attn_bwd_dkdv_kernel<BF16, D, DC, true, 4>), grid_kv, dim3(256), 0, st, a);
      return;
    }
  }
  const dim3 blk(64 * attn::dkdv_waves(D));
  if (causal)
    hipLaunchKernelGGL((attn::attn_bwd_dkdv_kernel<BF16, D, DC, true>), grid_kv, blk, 0, st, a);
  else
    hipLaunchKernelGGL((attn::attn_bwd_dkdv_kernel<BF16, D, DC, false>), grid_kv, blk, 0, st, a);
}

// dQ first: the dQ kernel also writes the workspace rows (-Delta and
// LSE * log2(e)) that the dK/dV kernel reads.
template <bool BF16, int D, int DC>
void launch_grads_d(const Args& a, bool causal, bool small_wg, unsigned phases, dim3 grid_kv, dim3 grid_q,
                    hipStream_t st) {
  if (phases & ATTN_PHASE_DQ) {
    const dim3 blk(64 * attn::kDqWaves);
    if (causal)
      hipLaunchKernelGGL((attn::attn_bwd_dq_recompute_kernel<BF16, D, DC, true>), grid_q, blk, 0, st, a);
    else
      hipLaunchKernelGGL((attn::attn_bwd_dq_recompute_kernel<BF16, D, DC, false>), grid_q, blk, 0, st, a);
  }
  if (phases & ATTN_PHASE_DKDV) launch_dkdv_d<BF16, D, DC>(a, causal, small_wg, grid_kv, st);
}

// Head-dim tiles: stored 64, 128 or 256 wide in LDS (columns past head_dim
// zero-filled); computed 64, 96, 128 or 256 wide (a 96-wide head -- head dims
// 72..96 -- does three quarters of the 128-wide tile's products).
int dtile_for(int head_dim) { return head_dim <= 64 ? 64 : (head_dim <= 128 ? 128 : 256); }
int dcomp_for(int head_dim) { return head_dim <= 64 ? 64 : (head_dim <= 96 ? 96 : (head_dim <= 128 ? 128 : 256)); }

// Query rows per dQ workgroup for a head-dim tile.
int dq_rows(int dtile) { return dtile == 256 ? attn::kDqWideBM : attn::kDqBM; }

// The dK/dV kernel with 4 waves and 64 keys per workgroup, two workgroups per
// CU, instead of 8 waves and 128 keys: for causal (lower-right) attention
// with one query head per KV head and fixed lengths, whose many short
// workgroups gain from one workgroup's start-up and epilogue running under
// the other's tile loop (measured 2-3 % faster on causal B4 H16 S4096 d128).
// GQA (each workgroup loops over the group's query heads), varlen (many
// short sequences) and non-causal attention keep the 8-wave kernel (GQA
// measured 2.5 % and varlen d96 8 % slower with 4 waves).  Windowed bands
// keep it too.
bool dkdv_small_wg(const attn_params* p, int dtile) {
  return dtile <= 128 && p->causal && p->window_left < 0 && p->window_right < 0 && !is_varlen(p) &&
         p->heads_q == p->heads_kv;
}

template <bool BF16>
void launch_grads(const Args& a, int dcomp, bool causal, bool small_wg, unsigned phases, dim3 grid_kv,
                  dim3 grid_q, hipStream_t st) {
  if (dcomp == 64) {
    launch_grads_d<BF16, 64, 64>(a, causal, small_wg, phases, grid_kv, grid_q, st);
  } else if (dcomp == 96) {
    launch_grads_d<BF16, 128, 96>(a, causal, small_wg, phases, grid_kv, grid_q, st);
  } else if (dcomp == 128) {
    launch_grads_d<BF16, 128, 128>(a, causal, small_wg, phases, grid_kv, grid_q, st);
  } else {
    if (phases & ATTN_PHASE_DQ) {
      if (causal)
        hipLaunchKernelGGL((attn::attn_bwd_dq_wide_kernel<BF16, true>), grid_q, dim3(256), 0, st, a);
      else
        hipLaunchKernelGGL((attn::attn_bwd_dq_wide_kernel<BF16, false>), grid_q, dim3(256), 0, st, a);
    }
    if (phases & ATTN_PHASE_DKDV) launch_dkdv_d<BF16, 256, 256>(a, causal, false, grid_kv, st);
  }
}

// ---- the no-allocation entry point's workspace ------------------------------
// attn_bwd_noalloc keeps Delta and LSE * log2(e) in this file-scope device
// array instead of a caller-provided workspace.  Every GPU the library runs
// on holds its own copy until the process ends.  In host code `scratch` is
// only a stand-in for the symbol: its device address comes from
// hipGetSymbolAddress, looked up once per device (with that device current)
// and kept in scratch_ptr[device].
constexpr size_t kScratchBytes = ATTN_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch array (nullptr on a HIP error).
void* scratch_for_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
    scratch_ptr[dev] = ptr;
  }
  return scratch_ptr[dev];
}

}  // namespace

extern "C" {

const char* attn_status_string(attn_status s) {
  switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID_ARGUMENT: return "invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case ATTN_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case ATTN_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* attn_version(void) { return "libattn gfx950 mfma32x32x16 bwd-kvstationary v1"; }

attn_status attn_fwd(const attn_params* p, const void* q, const void* k, const void* v, void* o,
                     float* lse, void* stream) {
  attn_status st = validate_common(p);
  if (st != ATTN_OK) return st;
  const bool qe = q_empty(p), ke = k_empty(p);
  if ((!qe && (!q || !o || !lse)) || (!ke && (!k || !v))) return ATTN_ERR_INVALID_ARGUMENT;
  const bool vl = is_varlen(p);
  if (!strides_ok(p->q, vl) || !strides_ok(p->k, vl) || !strides_ok(p->v, vl) || !strides_ok(p->o, vl))
    return ATTN_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return ATTN_ERR_UNSUPPORTED;
  if (p->seqlen_q == 0 || qe) return ATTN_OK;
  Args a = make_args(p);
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.out_o = static_cast<uint16_t*>(o);
  a.lse_out = lse;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const int dt = dtile_for(p->head_dim);
  const int bm = attn::fwd_bm(dt);
  dim3 grid(p->heads_q * p->batch, (p->seqlen_q + bm - 1) / bm, 1);
  const int dc = dcomp_for(p->head_dim);
  if (p->dtype == ATTN_BF16) launch_fwd<true>(a, dc, banded(p), grid, hs);
  else launch_fwd<false>(a, dc, banded(p), grid, hs);
  return last_hip_status();
}

attn_status attn_bwd_workspace_size(const attn_params* p, size_t* bytes) {
  attn_status st = validate_common(p);
  if (st != ATTN_OK) return st;
  if (!bytes) return ATTN_ERR_INVALID_ARGUMENT;
  *bytes = workspace_bytes(p);
  return ATTN_OK;
}

attn_status attn_bwd_phases(const attn_params* p, const void* q, const void* k, const void* v,
                            const void* o, const float* lse, const void* dout, void* dq, void* dk, void* dv,
                            void* workspace, size_t workspace_bytes_given, float* delta_out, void* stream,
                            unsigned phases) {
  if (phases == 0 || (phases & ~ATTN_PHASE_ALL) != 0) return ATTN_ERR_INVALID_ARGUMENT;
  attn_status st = validate_common(p);
  if (st != ATTN_OK) return st;
  const bool qe = q_empty(p), ke = k_empty(p);
  if ((!qe && (!q || !o || !lse || !dout || !dq)) || (!ke && (!k || !v || !dk || !dv)) || !workspace)
    return ATTN_ERR_INVALID_ARGUMENT;
  const bool vl = is_varlen(p);
  const attn_strides* all[] = {&p->q, &p->k, &p->v, &p->o, &p->dout, &p->dq, &p->dk, &p->dv};
  for (const attn_strides* s : all)
    if (!strides_ok(*s, vl)) return ATTN_ERR_UNSUPPORTED;
  const void* ptrs[] = {q, k, v, o, dout, dq, dk, dv};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return ATTN_ERR_UNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return ATTN_ERR_INVALID_ARGUMENT;
  if (workspace_bytes_given < workspace_bytes(p)) return ATTN_ERR_WORKSPACE_TOO_SMALL;

  Args a = make_args(p);
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<const uint16_t*>(o);
  a.dout = static_cast<const uint16_t*>(dout);
  a.dq = static_cast<uint16_t*>(dq);
  a.dk = static_cast<uint16_t*>(dk);
  a.dv = static_cast<uint16_t*>(dv);
  a.lse_in = lse;
  a.delta_out = delta_out;
  a.delta = static_cast<float*>(workspace);
  a.lse2 = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + stat_bytes(p));

  hipStream_t hs = static_cast<hipStream_t>(stream);
  const bool bf = p->dtype == ATTN_BF16;
  const bool causal = banded(p);  // causal or local window: the banded kernels
  const int dt = dtile_for(p->head_dim);
  const int qblocks = (p->seqlen_q + attn::kPreRows - 1) / attn::kPreRows;
  unsigned grad_phases = phases & (ATTN_PHASE_DKDV | ATTN_PHASE_DQ);
  const bool small_wg = dkdv_small_wg(p, dt);
  const int kvbn = small_wg ? 64 : attn::dkdv_bn(dt);
  const int kvblocks = (p->seqlen_k + kvbn - 1) / kvbn;
  const int dqblocks = (p->seqlen_q + dq_rows(dt) - 1) / dq_rows(dt);
  if (kvblocks == 0) grad_phases &= ~ATTN_PHASE_DKDV;  // no keys: nothing to write in dK/dV
  if (dqblocks == 0) grad_phases &= ~ATTN_PHASE_DQ;    // no queries: no dQ rows

  // The dQ kernel runs the preprocess for its own rows; the standalone
  // preprocess is only needed when the dQ phase does not run.
  if ((phases & ATTN_PHASE_PREPROCESS) && !(grad_phases & ATTN_PHASE_DQ) && qblocks > 0) {
    dim3 grid(qblocks, p->heads_q, p->batch);
    if (bf) hipLaunchKernelGGL((attn::attn_bwd_pre_kernel<true>), grid, dim3(256), 0, hs, a);
    else hipLaunchKernelGGL((attn::attn_bwd_pre_kernel<false>), grid, dim3(256), 0, hs, a);
    if (last_hip_status() != ATTN_OK) return ATTN_ERR_HIP;
  }
  if (grad_phases) {
    // (head x sequence, block): block index slowest, so the longest causal
    // blocks of every head start first and one head's blocks share an XCD.
    dim3 grid_kv(p->heads_kv * p->batch, kvblocks > 0 ? kvblocks : 1, 1);
    dim3 grid_q(p->heads_q * p->batch, dqblocks > 0 ? dqblocks : 1, 1);
    const int dc = dcomp_for(p->head_dim);
    if (bf) launch_grads<true>(a, dc, causal, small_wg, grad_phases, grid_kv, grid_q, hs);
    else launch_grads<false>(a, dc, causal, small_wg, grad_phases, grid_kv, grid_q, hs);
    if (last_hip_status() != ATTN_OK) return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

attn_status attn_bwd(const attn_params* p, const void* q, const void* k, const void* v, const void* o,
                     const float* lse, const void* dout, void* dq, void* dk, void* dv, void* workspace,
                     size_t workspace_bytes_given, float* delta_out, void* stream) {
  return attn_bwd_phases(p, q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes_given, delta_out,
                         stream, ATTN_PHASE_ALL);
}

attn_status attn_bwd_noalloc(const attn_params* p, const void* q, const void* k, const void* v, const void* o,
                             const float* lse, const void* dout, void* dq, void* dk, void* dv, float* delta_out,
                             void* stream) {
  attn_status st = validate_common(p);
  if (st != ATTN_OK) return st;
  if (workspace_bytes(p) > kScratchBytes) return ATTN_ERR_WORKSPACE_TOO_SMALL;
  void* ws = scratch_for_current_device();
  if (ws == nullptr) return ATTN_ERR_HIP;
  return attn_bwd_phases(p, q, k, v, o, lse, dout, dq, dk, dv, ws, kScratchBytes, delta_out, stream,
                         ATTN_PHASE_ALL);
}

}  // extern "C"
