/*
 * attn.h -- C ABI of libattn.so: FlashAttention-style attention forward and
 * backward for AMD Instinct MI355X (gfx950).
 *
 * The backward pass recomputes the softmax probabilities tile by tile from the
 * saved log-sum-exp instead of storing them, and produces dQ, dK, dV in three
 * launches: a preprocess (Delta = rowsum(dO o O)), a KV-stationary kernel for
 * dK and dV and a Q-stationary kernel for dQ (matrix-core contractions with
 * fp32 accumulation).  Nothing of size Sq x Sk is stored: the workspace holds
 * two fp32 row statistics, O(Sq) per head.  The forward produces O and the
 * LSE the backward consumes.
 *
 * Conventions for every entry point
 *  - Every tensor pointer is a DEVICE pointer (hipMalloc'd or equivalent) on
 *    the device that is current when the call is made.  `stream` is a
 *    hipStream_t passed as void* (NULL = the null stream).
 *  - Calls are asynchronous on `stream`; the library never synchronises, never
 *    allocates device memory, never frees, and keeps no mutable global state.
 *    Ownership of every buffer stays with the caller.
 *  - Validation runs on the host before anything is launched; a call that
 *    returns an error has launched nothing and written nothing.  Faults of
 *    launched kernels surface at the caller's next synchronisation.
 *  - Tensors are [batch, seq, heads, head_dim] with element strides given in
 *    attn_params (last dim contiguous), or, in varlen mode, packed
 *    [total, heads, head_dim] with batch stride ignored.  Q, O, dO, dQ have
 *    heads_q heads; K, V, dK, dV have heads_kv heads, and query head h reads
 *    KV head h / (heads_q / heads_kv) (flash-attention CK mha_bwd.cpp, the
 *    GQA reshape to [b, s_k, h_k, h/h_k, d] summed over the group axis).
 *  - LSE is fp32, natural log, contiguous [batch, heads_q, seqlen_q]
 *    (varlen: [heads_q, total_q]), as the CK mha_bwd.cpp page's softmax_lse
 *    and the Hopper flash_bwd_launch_template.h page's softmax_lse_ptr take it.
 *    A query row that sees no key has O = 0 and LSE = +inf.
 */
#ifndef ATTN_H_
#define ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARGUMENT = 1,   /* bad shape, stride, pointer or flag */
  ATTN_ERR_UNSUPPORTED = 2,        /* valid for the method, not built here */
  ATTN_ERR_WORKSPACE_TOO_SMALL = 3,
  ATTN_ERR_HIP = 4                 /* a HIP runtime call or launch failed */
} attn_status;

typedef enum { ATTN_FP16 = 0, ATTN_BF16 = 1 } attn_dtype;

/* Element strides of a 4-D [batch, seq, head, dim] tensor (dim stride is 1). */
typedef struct {
  int64_t batch;
  int64_t row;
  int64_t head;
} attn_strides;

typedef struct {
  attn_dtype dtype;        /* fp16 or bf16; every tensor has this type
                              (CK mha_bwd.cpp: q, k, v, out, dout same dtype) */
  int32_t batch;           /* B > 0, or the number of packed sequences */
  int32_t seqlen_q;        /* fixed-length Sq (>= 0); varlen: max length */
  int32_t seqlen_k;        /* fixed-length Sk (>= 0); varlen: max length */
  int32_t heads_q;         /* H > 0 */
  int32_t heads_kv;        /* Hk > 0, H % Hk == 0 */
  int32_t head_dim;        /* d % 8 == 0, d <= 256 (the CK mha_bwd.cpp
                              page's limit); each head is computed in a 64-,
                              128- or 256-wide tile, zero-padded */
  float softmax_scale;     /* scores are scale * Q K^T, scale > 0 (finite);
                              pass 1/sqrt(d) for the default */
  int32_t causal;          /* 0/1; key j visible to query i iff
                              j <= i + (Sk - Sq) (bottom-right aligned) */
  int32_t deterministic;   /* bwd: 1 = bit-identical run to run (always
                              satisfied: no atomics are used) */
  const int32_t *cu_seqlens_q;  /* device int32[batch+1] prefix sums, or NULL */
  const int32_t *cu_seqlens_k;  /* both NULL (fixed length) or both set */
  int32_t total_q;         /* varlen: cu_seqlens_q[batch] (host copy) */
  int32_t total_k;         /* varlen: cu_seqlens_k[batch] (host copy) */
  attn_strides q, k, v, o, dout, dq, dk, dv;
  int32_t window_left;     /* local (sliding-window) attention, the CK
                              mha_bwd.cpp page's window_size_left/right:
                              key j visible to query i iff
                              i + (Sk - Sq) - window_left <= j <=
                              i + (Sk - Sq) + window_right; -1 = no bound on
                              that side (both -1: no window).  causal = 1
                              sets window_right = 0, as that page does. */
  int32_t window_right;
} attn_params;

/*
 * Limits of this build, reported as ATTN_ERR_UNSUPPORTED before any launch
 * (the arguments are valid for the method):
 *   heads_q or batch above 65535, or heads_q * batch above 2^31 - 1;
 *   seqlen_q or seqlen_k above 65535 * 64;
 *   a per-head extent of 1 GiB or more: seqlen * row stride * 2 bytes, for
 *     any of q, o, dout, dq (seqlen_q) or k, v, dk, dv (seqlen_k) -- the
 *     kernels address one head of one sequence with 32-bit byte offsets;
 *   a row or head stride that is not positive; a batch, row or head
 *     stride, or a tensor address, that is not a multiple of 8 elements
 *     (16 bytes).
 */

/*
 * Forward: O = softmax(scale * Q K^T, masked) V and LSE (natural log).
 * tilelang test_tilelang_kernel_mha_bwd.py, flashattn_fwd (online softmax in
 * the exp2 domain with scale * log2(e) folded into one constant) and
 * ref_program (the definition).
 *   q [.., Sq, H, d], k, v [.., Sk, Hk, d]: inputs, read only.
 *   o [.., Sq, H, d]: output, fully overwritten.
 *   lse fp32 [B, H, Sq] (varlen [H, total_q]): output, fully overwritten.
 * Errors: ATTN_ERR_INVALID_ARGUMENT / ATTN_ERR_UNSUPPORTED before any launch;
 * ATTN_ERR_HIP if a launch fails.
 */
attn_status attn_fwd(const attn_params *p, const void *q, const void *k, const void *v,
                     void *o, float *lse, void *stream);

/*
 * Bytes of device workspace attn_bwd needs: Delta = rowsum(dO o O) (the
 * flash-attention CK mha_bwd.cpp page's softmax_d) and LSE * log2(e), each
 * fp32 laid out like lse and rounded up to 256 bytes -- 8 bytes per
 * (query head, query row), independent of the key length.  The gradient
 * kernels recompute P and dS tile by tile from LSE and Delta (tilelang
 * test_tilelang_kernel_mha_bwd.py, flashattn_bwd) and keep dQ in registers,
 * so nothing else is needed.  Never allocates.
 * Errors: as attn_fwd's validation; ATTN_ERR_INVALID_ARGUMENT for a NULL bytes.
 */
attn_status attn_bwd_workspace_size(const attn_params *p, size_t *bytes);

/*
 * Backward: dQ, dK, dV of sum(O o dO).
 *   tilelang test_tilelang_kernel_mha_bwd.py, flashattn_bwd_preprocess and
 *   flashattn_bwd (the method: P recomputed tile by tile from LSE,
 *   dS = P o (dP - Delta)); flash-attention CK mha_bwd.cpp, mha_bwd (argument
 *   contract); Hopper flash_bwd_launch_template.h, run_flash_bwd (preprocess
 *   first, dQ scaled by scale_softmax).
 *   q, k, v, o, dout, lse: inputs (o, lse from attn_fwd), read only.
 *   dq [.., Sq, H, d], dk, dv [.., Sk, Hk, d]: outputs, fully overwritten; dK
 *   and dV of a KV head are summed over the query heads of its group.
 *   workspace: device buffer, 256-byte aligned, of at least
 *   attn_bwd_workspace_size() bytes, owned by the caller; its contents on
 *   entry do not matter and it is overwritten.
 *   delta_out: NULL, or a device fp32 buffer laid out like lse that receives
 *   Delta = rowsum(dO o O) (for tests).
 * Two launches on `stream`: a Q-stationary kernel for dQ that first runs the
 * preprocess for its own query rows (Delta from O and dO, written to the
 * workspace with LSE * log2(e)), then recomputes dS and sums the key blocks
 * in ascending order in registers (dQ * scale and the conversion are its
 * epilogue: the pages' dQ postprocess, fused); then a KV-stationary kernel
 * for dK and dV that reads the workspace rows.  No atomics
 * are used, so every output is bit-identical from run to run; `deterministic`
 * is accepted and always satisfied.
 * Sq == 0 gives dK = dV = 0; Sk == 0 gives dQ = 0.
 * Errors: as attn_fwd, plus ATTN_ERR_WORKSPACE_TOO_SMALL.
 */
attn_status attn_bwd(const attn_params *p, const void *q, const void *k, const void *v,
                     const void *o, const float *lse, const void *dout,
                     void *dq, void *dk, void *dv,
                     void *workspace, size_t workspace_bytes,
                     float *delta_out, void *stream);

/*
 * The same backward pass, launching only the kernels selected in `phases`
 * (bitwise OR of ATTN_PHASE_*), in the order preprocess, dQ, dK/dV.
 * attn_bwd == attn_bwd_phases(..., ATTN_PHASE_ALL).  Lets a caller time or
 * schedule the kernels separately.  The dQ kernel computes Delta itself and
 * writes Delta and LSE * log2(e) to `workspace`, so ATTN_PHASE_PREPROCESS
 * launches the standalone preprocess only when ATTN_PHASE_DQ is not also
 * selected (then it writes the same workspace rows).  The dK/dV kernel reads
 * them: a dK/dV phase needs the dQ phase or the preprocess to have run on the
 * same workspace first, in this call or an earlier one; otherwise its results
 * are unspecified (but in-bounds).  Arguments, validation and errors as
 * attn_bwd; phases == 0 or an unknown bit is ATTN_ERR_INVALID_ARGUMENT.
 */
#define ATTN_PHASE_PREPROCESS 1u
#define ATTN_PHASE_DKDV 2u
#define ATTN_PHASE_DQ 4u
#define ATTN_PHASE_ALL 7u
attn_status attn_bwd_phases(const attn_params *p, const void *q, const void *k, const void *v,
                            const void *o, const float *lse, const void *dout,
                            void *dq, void *dk, void *dv,
                            void *workspace, size_t workspace_bytes,
                            float *delta_out, void *stream, unsigned phases);

/*
 * attn_bwd without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Delta and LSE * log2(e) live in a static device
 * array of ATTN_NOALLOC_SCRATCH_BYTES inside the library (one copy per GPU,
 * held until the process ends); the call allocates and frees nothing.  The
 * array's device address is looked up with hipGetSymbolAddress on the first
 * call on each device.
 *   Arguments, outputs and errors as attn_bwd (no workspace, workspace_bytes).
 *   A problem whose attn_bwd_workspace_size() exceeds the array -- more than
 *   ATTN_NOALLOC_SCRATCH_BYTES / 8 (query head, query row) pairs, minus
 *   rounding -- returns ATTN_ERR_WORKSPACE_TOO_SMALL before any launch;
 *   ATTN_ERR_HIP if the array's address cannot be obtained.
 *   Every call on one GPU shares that GPU's array: calls that overlap on one
 *   GPU (different streams, or other threads) race on it and must be
 *   serialised by the caller.  Nothing in the array needs to start at zero
 *   (the preprocess writes all of it before it is read).
 */
#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
attn_status attn_bwd_noalloc(const attn_params *p, const void *q, const void *k, const void *v,
                             const void *o, const float *lse, const void *dout,
                             void *dq, void *dk, void *dv, float *delta_out, void *stream);

/*
 * Static, NUL-terminated description of a status code.  The codes stand in
 * for the flash-attention CK mha_bwd.cpp page's error reporting: its
 * TORCH_CHECK argument checks (dtype, contiguity, batch, head_dim, head
 * counts) become ATTN_ERR_INVALID_ARGUMENT or ATTN_ERR_UNSUPPORTED, and its
 * negative kernel time ("invalid argument for fmha_bwd") becomes a status
 * returned before any launch.  Never NULL; unknown codes give
 * "unknown status".
 */
const char *attn_status_string(attn_status s);

/*
 * Library build identifier (static string), e.g. for logs and for matching
 * committed measurements to a build.  Not from the pages.
 */
const char *attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H_ */
