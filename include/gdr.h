/*
 * gdr.h - C ABI of the chunked gated delta rule prefill for AMD MI355X (gfx950).
 *
 * What it computes. Per batch row b and value head h, with key head kh = h / (Hv / Hk)
 * (each key head serves Hv/Hk consecutive value heads, the head sharing of the model page
 * "deg model" / model.py, function _linear_layer, repeat_interleave along the head axis):
 *
 *   q_hat_t = q_t / sqrt(|q_t|^2 + 1e-6) * Dk^-1/2,   k_hat_t = k_t / sqrt(|k_t|^2 + 1e-6)
 *   beta'_t = beta_t * [t < len_b],                    g'_t = g_t * [t < len_b]
 *   S <- s0[s0_row[b], h]  (or zeros)
 *   for t in 0 .. L-1:  S <- exp(g'_t) S;  delta = beta'_t (v_t - S^T k_hat_t);
 *                       S <- S + k_hat_t delta^T;  o_t = S^T q_hat_t
 *   s_final[b, h] = S
 *
 * This is the float64 truth recurrence of the kernel-test page (r15_kernel_test.py, function
 * truth_f64) and the per-token reference of the model page (model.py, function
 * delta_rule_reference, with _l2norm's eps inside the rsqrt), with the exact right-pad guard
 * of model.py's _dn_gates (pads neither write nor decay). The library evaluates it in
 * 64-token chunks (per-chunk UT/WY transform with a 64x64 unit-triangular inverse, then a
 * sequential inter-chunk state scan); the result is the same recurrence up to rounding.
 * The output at a pad position is what the recurrence gives there (the frozen state read
 * with that position's q); it is not zeroed.
 *
 * Layouts (row-major, contiguous, every pointer 16-byte aligned):
 *   q, k      [B, L, Hk, Dk]        qkv_dtype
 *   v, o      [B, L, Hv, Dv]        qkv_dtype
 *   g         [B, L, Hv]            float32 (log decay, expected <= 0; g > 0 is outside the
 *                                   method's domain and its result is unspecified)
 *   beta      [B, L, Hv]            beta_dtype (float32, or qkv_dtype)
 *   lengths   [B]                   int32, right-pad lengths in [0, L]; NULL = all L valid
 *   s0        [n_s0, Hv, Dk, Dv]    float32, key index first; NULL = zero initial state
 *   s0_row    [B]                   int32 rows of s0 each batch row starts from (the fork
 *                                   model's h0 / h0_idx of model.py, _fork_linear_layer);
 *                                   NULL = row b starts from s0[b]
 *   s_final   [B, Hv, Dk, Dv]       float32; NULL = not wanted
 *   workspace gdr_prefill_workspace_size(desc) bytes, 256-byte aligned
 * Dk = Dv = 128 are compiled in. q/k/v/beta/g/lengths/s0/s0_row are device pointers to
 * memory the caller owns and keeps alive until the stream has finished the call; the library
 * keeps no device allocation of its own and does not retain any pointer after returning.
 *
 * Errors. Every argument that can be checked on the host is checked before anything is
 * launched: GDR_EINVAL, GDR_EUNSUPPORTED and GDR_EWORKSPACE mean nothing was launched and no
 * output was touched (GDR_EHIP may come after a first launch). The
 * message of the last non-OK status on the calling thread is gdr_last_error(). Values that
 * live in device memory (lengths, s0_row) are checked by the kernels themselves: a row whose
 * length is outside [0, L], or whose s0_row entry is outside [0, n_s0), gets NaN in all of
 * its o and s_final entries (no memory outside the buffers is ever accessed).
 * gdr_prefill is asynchronous on `stream`; launch failures return GDR_EHIP.
 */
#ifndef GDR_H_
#define GDR_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDR_OK = 0,
  GDR_EINVAL = -1,        /* a null, misaligned, overlapping or inconsistent argument */
  GDR_EUNSUPPORTED = -2,  /* a valid request the library does not implement (Dk, Dv != 128) */
  GDR_EWORKSPACE = -3,    /* workspace missing or smaller than gdr_prefill_workspace_size */
  GDR_EHIP = -4           /* the HIP runtime reported an error while launching */
} gdr_status;

typedef enum { GDR_F32 = 0, GDR_BF16 = 1 } gdr_dtype;

typedef struct {
  int32_t B, L;           /* batch rows, tokens per row (B, L >= 0) */
  int32_t Hk, Hv;         /* key heads, value heads; Hv % Hk == 0 */
  int32_t Dk, Dv;         /* head dims; must be 128 */
  int32_t n_s0;           /* rows in s0 (ignored when s0 is NULL) */
  int32_t qkv_dtype;      /* gdr_dtype of q, k, v and o */
  int32_t beta_dtype;     /* gdr_dtype of beta: GDR_F32 or qkv_dtype */
} gdr_desc;

/* Bytes of device workspace gdr_prefill needs for this shape (0 when B*L == 0), or
 * (size_t)-1 when the descriptor itself is invalid (see gdr_last_error). The workspace holds
 * per-chunk intermediates (the chunk's inverse T*diag(beta), the decayed causal q.k scores
 * and per-token scalars), for bf16 sequences long enough to be cut into segments that are
 * scanned in parallel each segment's state map and entering state, and (bf16) the list of the
 * chunks that hold valid tokens when lengths are given. Every call writes what it reads before
 * reading it. */
size_t gdr_prefill_workspace_size(const gdr_desc* desc);

/* Host-only validation of a gdr_prefill call (same arguments, no stream). Touches no GPU. */
gdr_status gdr_prefill_check(const gdr_desc* desc, const void* q, const void* k, const void* v,
                             const float* g, const void* beta, const int32_t* lengths,
                             const float* s0, const int32_t* s0_row, const void* o,
                             const float* s_final, const void* workspace, size_t workspace_bytes);

/* The chunked gated delta rule prefill. `stream` is a hipStream_t (NULL = the null stream).
 * s_final may be the same pointer as s0 (in-place continuation, as the fork model's store
 * buffer is) only when s0_row is NULL; no other output may overlap any input. */
gdr_status gdr_prefill(const gdr_desc* desc, const void* q, const void* k, const void* v,
                       const float* g, const void* beta, const int32_t* lengths, const float* s0,
                       const int32_t* s0_row, void* o, float* s_final, void* workspace,
                       size_t workspace_bytes, void* stream);

/* gdr_prefill for callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation. Same arguments, layouts, results and errors as
 * gdr_prefill, without the workspace: the library uses a fixed 128 MiB array in device memory
 * instead, one per GPU it runs on, held from the first use of the library on that GPU until the
 * process ends. The first call on a device looks up that device's array (with the device current);
 * no call allocates, frees or creates anything (per-kernel timing events are not recorded).
 * Shapes whose gdr_prefill_workspace_size exceeds 128 MiB (134217728 bytes) are rejected with
 * GDR_EUNSUPPORTED before anything is launched (the long prefill, B = 1, L = 16384, 32 value heads,
 * needs about 101 MB). Every call on a GPU shares that GPU's array, which keeps the last call's
 * contents: calls that overlap on one GPU (on different streams or threads without ordering
 * between them) race and give wrong results; calls in one stream are safe. */
gdr_status gdr_prefill_noalloc(const gdr_desc* desc, const void* q, const void* k, const void* v,
                               const float* g, const void* beta, const int32_t* lengths, const float* s0,
                               const int32_t* s0_row, void* o, float* s_final, void* stream);

/* Work fused into gdr_prefill_ex (model page, model.py, _linear_layer: the gate prologue feeds the
 * delta rule and the gated RMSNorm follows it). Either part may be left out (NULL pointers).
 *   Gate prologue: b_raw, a_raw [B, L, Hv] in desc->beta_dtype (the raw projections) and A_log,
 *     dt_bias [Hv] float32, all four or none. When given, the call's g and beta must be NULL:
 *     beta = sigmoid(b_raw) and g = -exp(A_log) softplus(a_raw + dt_bias) (gdr_gates) are formed
 *     inside the per-chunk kernel, in float32, and never written to memory.
 *   Gated RMSNorm: z [B, L, Hv, 128] in qkv_dtype, 16-byte aligned, and norm_w [128] float32,
 *     16-byte aligned, both or neither; norm_eps finite, >= 0. When given, o holds
 *     norm_w * o / sqrt(mean(o^2) + norm_eps) * silu(z) per (token, head) (gdr_gated_rmsnorm)
 *     instead of the raw output. For bf16 it is applied in registers before o is stored; for
 *     float32 a second kernel normalises o in place after the scan. */
typedef struct {
  const void* b_raw;
  const void* a_raw;
  const float* A_log;
  const float* dt_bias;
  const void* z;
  const float* norm_w;
  float norm_eps;
} gdr_fusion;

/* gdr_prefill with optional fused prologue / epilogue work (fusion may be NULL: then it is
 * gdr_prefill). Same arguments, layouts, workspace and errors as gdr_prefill; g and beta must be
 * NULL when the gate prologue is fused, and non-NULL otherwise (when there are tokens). */
gdr_status gdr_prefill_ex(const gdr_desc* desc, const void* q, const void* k, const void* v, const float* g,
                          const void* beta, const int32_t* lengths, const float* s0, const int32_t* s0_row,
                          const gdr_fusion* fusion, void* o, float* s_final, void* workspace, size_t workspace_bytes,
                          void* stream);

/* The same computation, token by token, for short sequences: decode steps and fork
 * continuations over many rows (the fork model's fork_delta_rule with h0, h0_idx and an in-place
 * store, model.py, _fork_linear_layer). Arguments, layouts, pad guard, s0_row gather, in-place
 * rule and error behaviour are those of gdr_prefill; no workspace is needed. One workgroup per
 * (row, value head) keeps the 128 x 128 state in registers for all L tokens, so the cost is one
 * read of s0 and one write of s_final per (row, head) plus the token rows; any L is accepted, but
 * for long sequences gdr_prefill is far faster. */
gdr_status gdr_decode(const gdr_desc* desc, const void* q, const void* k, const void* v, const float* g,
                      const void* beta, const int32_t* lengths, const float* s0, const int32_t* s0_row,
                      void* o, float* s_final, void* stream);

/* ---- Layer steps on either side of the delta rule (model page, model.py, _linear_layer and
 * _fork_linear_layer). Same conventions as above: device pointers the caller owns, asynchronous
 * on `stream`, every host-checkable argument validated before any launch (a non-OK status
 * means nothing was launched), a row whose device-side length is outside [0, L] gets NaN
 * outputs. Head dimension 128. */

/* Gate prologue (model.py, _dn_gates): per (row b, token t, value head h)
 *   beta[b,t,h] = sigmoid(b_raw[b,t,h]) * [t < len_b]
 *   g[b,t,h]    = -exp(A_log[h]) * softplus(a_raw[b,t,h] + dt_bias[h]) * [t < len_b]
 * b_raw, a_raw [B, L, Hv] in ab_dtype (the raw projections); A_log, dt_bias [Hv] float32;
 * lengths [B] int32 or NULL; outputs beta [B, L, Hv] in ab_dtype and g [B, L, Hv] float32,
 * ready for gdr_prefill / gdr_decode (pads are exact no-ops). Computed in float32, each output
 * rounded once. Outputs must not overlap inputs. */
gdr_status gdr_gates(int32_t B, int32_t L, int32_t Hv, gdr_dtype ab_dtype, const void* b_raw, const void* a_raw,
                     const float* A_log, const float* dt_bias, const int32_t* lengths, void* beta, float* g,
                     void* stream);

/* Causal depthwise convolution + SiLU with conv-tail continuation and the q/k/v split
 * (model.py, _conv_silu, and the tail gather of _linear_layer). With Cm = (2 Hk + Hv) * 128
 * channels and ext = [tail ; mixed] along time (K-1 + L rows):
 *   pre[b,t,c] = sum_{j=0}^{K-1} ext[b, t+j, c] * w[c, j],   out = silu(pre)
 *   q = out[..., 0:Hk*128] -> [B, L, Hk, 128], k = the next Hk*128 channels, v = the last Hv*128
 *   new_tail[b, j] = ext[b, len_b + j], j = 0 .. K-2   (the last K-1 inputs up to the row's length)
 * mixed [B, L, Cm] and tail [B, K-1, Cm] (NULL = zeros) in dtype; w [Cm, K] float32 (the
 * depthwise filter, one row per channel; the last tap multiplies the current token);
 * lengths [B] int32 or NULL; q, k, v in dtype, the layouts gdr_prefill reads; new_tail
 * [B, K-1, Cm] in dtype or NULL (not wanted). new_tail may be tail itself (in-place tail
 * update); no other output may overlap an input. 1 <= K <= 8. Computed in float32. */
gdr_status gdr_conv_silu(int32_t B, int32_t L, int32_t Hk, int32_t Hv, int32_t K, gdr_dtype dtype, const void* mixed,
                         const void* tail, const float* w, const int32_t* lengths, void* q, void* k, void* v,
                         void* new_tail, void* stream);

/* Gated RMSNorm over 128-wide rows (model.py, _gated_rms):
 *   out[r, :] = w * x[r, :] / sqrt(mean(x[r, :]^2) + eps) * silu(z[r, :])
 * x, z, out [rows, 128] in dtype (rows = B * L * Hv for the delta rule's o and the gate z);
 * w [128] float32; eps finite, >= 0. out may be x itself (in place); computed in float32. */
gdr_status gdr_gated_rmsnorm(int64_t rows, gdr_dtype dtype, const void* x, const void* z, const float* w, float eps,
                             void* out, void* stream);

/* gdr_decode with the same optional fused work as gdr_prefill_ex (fusion may be NULL: then it is
 * gdr_decode): a decode step of the fork model's layer (model.py, _fork_linear_layer) that reads the
 * raw gate projections and writes the normalised output. Arguments and errors as gdr_prefill_ex,
 * without the workspace. */
gdr_status gdr_decode_ex(const gdr_desc* desc, const void* q, const void* k, const void* v, const float* g,
                         const void* beta, const int32_t* lengths, const float* s0, const int32_t* s0_row,
                         const gdr_fusion* fusion, void* o, float* s_final, void* stream);

/* Truncated segment starts (bf16 sequences cut into segments). The state map of a run of tokens is
 * S -> Phi S + B with ||Phi||_2 <= exp(sum of g' over the run) whenever every beta' of the run lies in
 * [0, 2] (each token multiplies S by exp(g') (I - beta' k_hat k_hat^T), whose spectral norm is then at
 * most exp(g'), since |k_hat| < 1). When, for every segment boundary of a (row, head), the last few
 * chunks (at most 32) before the boundary decay by at least 2^-40 in that sense, the library takes the
 * state entering the segment from those chunks alone, run from zero, instead of composing the maps of
 * all earlier segments. The dropped term is at most 2^-40 times the norm of the state where the window
 * starts; the kernels measure that norm and, in a last pass, check at every boundary that the error
 * bound carried along the segments stays below 2^-24 of the norm of the state used, and rerun the
 * (row, head) without truncation where it does not. Results therefore agree with the untruncated
 * computation to within that relative bound. On by default; gdr_set_truncation(0) makes every call on
 * any thread take the untruncated path (process-wide setting, not synchronised with calls in flight). */
gdr_status gdr_set_truncation(int on);

/* Byte offset in the workspace of an int32 that the last gdr_prefill call on that workspace sets to
 * the number of (row, head) pairs it recomputed without truncation (valid once the call has finished),
 * or (size_t)-1 when this shape has no segments or the desc is invalid. */
size_t gdr_prefill_status_offset(const gdr_desc* desc);

/* Message of the last non-OK status returned on this thread ("" if none). */
const char* gdr_last_error(void);

/* Kernel timing, for benchmarks. When enabled, gdr_prefill records a HIP event pair on
 * `stream` around each kernel it launches. gdr_timing_read waits for the recorded events,
 * writes per-kernel sums of elapsed milliseconds and launch counts for kernel ids
 * 0 .. n_kernels-1 (GDR_KERNEL_*), and clears the record. Not thread-safe. */
enum {
  GDR_KERNEL_PREP = 0,        /* per-chunk transform: norms, decays, T diag(beta), scores */
  GDR_KERNEL_SCAN = 1,        /* state scan writing o (and s_final) */
  GDR_KERNEL_TRANSITION = 2,  /* bf16 long sequences: per-segment state maps */
  GDR_KERNEL_COMBINE = 3,     /* bf16 long sequences: chains the segment maps */
  GDR_KERNEL_DECODE = 4,      /* gdr_decode */
  GDR_KERNEL_GATES = 5,       /* gdr_gates */
  GDR_KERNEL_CONV = 6,        /* gdr_conv_silu */
  GDR_KERNEL_NORM = 7,        /* gdr_gated_rmsnorm */
  GDR_KERNEL_FINALIZE = 8,    /* bf16 long sequences: checks truncated segment starts, reruns */
  GDR_KERNEL_COUNT = 9
};
gdr_status gdr_timing_enable(int on);
gdr_status gdr_timing_read(double* total_ms, int64_t* launches, int n_kernels);

/* Name of a kernel id ("" if out of range), as it appears in profiler traces. */
const char* gdr_kernel_name(int kernel_id);

#ifdef __cplusplus
}
#endif
#endif /* GDR_H_ */
