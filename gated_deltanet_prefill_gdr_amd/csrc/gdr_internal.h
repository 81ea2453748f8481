// Internal interface between the C ABI (gdr_api.cpp) and the HIP kernels (gdr_prep.hip,
// gdr_scan.hip, gdr_decode.hip, gdr_layer.hip).
#ifndef GDR_INTERNAL_H_
#define GDR_INTERNAL_H_

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace gdr {

constexpr int kChunk = 64;      // tokens per chunk
constexpr int kHeadDim = 128;   // Dk = Dv

// Workspace: one record per (row b, value head h, chunk c), record index (b*Hv + h)*NC + c.
// A record holds, in the element type of q/k/v,
//   Tb = T diag(beta')            (T = (I + A)^-1 of the chunk; zero above the diagonal)
//   P  = (q_hat k_hat^T) (.) E    (decayed causal scores, diagonal included; float32 records
//                                  only: the bf16 output pass forms P itself from Q and K)
// each as 6 blocks in MFMA operand order, one block per (token tile w, token block kb) that
// the lower triangle reaches: (0,0) (1,0) (2,0) (2,1) (3,0) (3,1). A block is 64 lanes x 8
// elements; lane (m = lane % 16, G = lane / 16) holds row 16w + m, columns
// 32kb + {4G..4G+3, 16+4G..16+4G+3}. Then the scalar block, 8 x 64 floats: a_t = e^{gamma_t} rk_t,
// c_t = e^{gamma_t} rq_t, d_t = rk_t e^{gamma_63 - gamma_t}, e^{gamma_63} at [3][0], gamma_t log2(e),
// rk_t, rq_t, then zeros.
constexpr int kFragBlocks = 6;
constexpr int kBlockElems = 64 * 8;
constexpr int kScalarBytes = 8 * kChunk * 4;
constexpr int kScA = 0, kScC = 1, kScD = 2, kScEgC = 3, kScGam2 = 4, kScRk = 5, kScRq = 6;   // rows of 64
// bf16 records order their scalar rows differently: rows 0..3, the first 1 KiB (the only scalar
// block the segment kernels stage), hold a, d, gamma log2 e and rk (e^{gamma_63} is formed from
// gamma_63 where it is used); row 4 holds at [4][0] the contraction flag (1 when every beta' of the
// chunk lies in [0, 2], where each token's map S -> e^{g'} (I - beta' k_hat k_hat^T) S has spectral
// norm at most e^{g'}, and the chunk's decay sum is <= 0, so that the chunk's map has spectral norm
// at most 1; 0 otherwise); rows 5..7 are not used.
constexpr int kBfA = 0, kBfD = 1, kBfGam2 = 2, kBfRk = 3, kBfFlag = 4;

inline size_t record_bytes(size_t elem) {
  return (elem == 2 ? 1 : 2) * size_t(kFragBlocks) * kBlockElems * elem + kScalarBytes;
}

// Segments of the bf16 scan. The chunks of each (row, value head) are split into P runs of
// Ls consecutive chunks (the last run may be shorter) that are scanned in parallel; P = 1 for
// float32 and whenever the rows and heads alone give enough workgroups.
constexpr int kSegTargetWorkgroups = 256;   // one per compute unit
struct SegPlan {
  int P, Ls;
};
inline SegPlan seg_plan(int B, int Hv, int NC, bool bf16) {
  if (!bf16 || NC <= 1) return SegPlan{1, NC};
  const int64_t heads = int64_t(B) * Hv;
  int64_t P = (kSegTargetWorkgroups + heads - 1) / heads;
  if (P > NC) P = NC;
  if (P < 1) P = 1;
  const int Ls = (int)((NC + P - 1) / P);
  return SegPlan{(NC + Ls - 1) / Ls, Ls};
}

// Segment states (bf16 with P > 1), after the records: per (row b, value head h) P slots of
// 128 x 256 floats, slot (b*Hv + h)*P + j. Columns 0..127 of slot j: first the local state
// B_{j-1} that segment j-1 reaches from a zero state, then (after the combine) the true state
// entering segment j. Columns 128..255 of slot j: the transition M_j of segment j (column k
// is the state segment j reaches from e_k with zero values), key index as row.
constexpr size_t kSlotFloats = size_t(kHeadDim) * 2 * kHeadDim;

inline size_t records_bytes(int B, int Hv, int NC, size_t elem) {
  return size_t(B) * Hv * NC * record_bytes(elem);
}

inline size_t seg_bytes(int B, int Hv, int NC, size_t elem) {
  const SegPlan sp = seg_plan(B, Hv, NC, elem == 2);
  return sp.P > 1 ? size_t(B) * Hv * sp.P * kSlotFloats * sizeof(float) : 0;
}

// Chunk list (bf16, after the segment states): the chunks that hold valid tokens when lengths are
// given, row-major: int32 count U, then U entries b NC + c (room for B NC); then the B rows ordered
// by their number of such chunks, longest first (ties in any order).
inline size_t chunk_list_bytes(int B, int NC, size_t elem) { return elem == 2 ? 4 * (1 + size_t(B) * NC + B) : 0; }

// Truncated segment starts (bf16 with P > 1). The state entering segment j >= 1 is
// S_j = Phi S(c_j - W) + S~_j, where S~_j is the state that the last W chunks before c_j reach from
// zero and Phi is the product of those chunks' maps, ||Phi||_2 <= 2^{l2} with l2 the sum of g' log2 e
// over the window (when every beta' there lies in [0, 2]). When a window with l2 <= -kTruncLog2 exists
// for every boundary of a (row, head), the transition pass computes S~_j over that window alone and the
// combine is skipped; the output pass records ||S(c_j - W)||_F, and the finalize pass checks the bound
// eps_j = 2^{l2_j} (||S(c_j - W_j)||_F + eps_{j-1}) <= 2^-24 ||S~_j||_F at every boundary, rerunning the
// (row, head) without truncation where it fails.
constexpr float kTruncLog2 = 40.f;     // a-priori window decay: 2^-40
constexpr float kCertRel = 5.9604645e-8f;   // 2^-24
constexpr int kTruncMaxW = 32;          // longest window, in chunks (at most the segment length)
struct PlanEntry {                      // per (row, head, boundary j), written by the transition pass
  int32_t W;                            // window length in chunks (0: no window, boundary not truncated)
  float l2;                             // sum of g' log2(e) over the window
  int32_t trunc;                        // the (row, head) takes the truncated path (same in every entry)
  int32_t pad;
};
constexpr int kCertFloats = 16;         // [0, 8): per-wave ||S(c_j - W)||^2 parts, [8, 16): ||S~_j||^2 parts
constexpr size_t kTruncHeader = 256;    // int32 status: (row, head) pairs the last call reran

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
inline size_t trunc_offset(int B, int Hv, int NC, size_t elem) {
  return align256(records_bytes(B, Hv, NC, elem) + seg_bytes(B, Hv, NC, elem) + chunk_list_bytes(B, NC, elem));
}
inline size_t trunc_bytes(int B, int Hv, int NC, size_t elem) {
  const SegPlan sp = seg_plan(B, Hv, NC, elem == 2);
  return sp.P > 1 ? kTruncHeader + size_t(B) * Hv * sp.P * (sizeof(PlanEntry) + kCertFloats * sizeof(float)) : 0;
}

inline size_t workspace_bytes(int B, int Hv, int NC, size_t elem) {
  const size_t t = trunc_bytes(B, Hv, NC, elem);
  return t ? trunc_offset(B, Hv, NC, elem) + t
           : records_bytes(B, Hv, NC, elem) + seg_bytes(B, Hv, NC, elem) + chunk_list_bytes(B, NC, elem);
}

// gdr_prefill_noalloc: the workspace lives in a fixed device array of this many bytes (per GPU).
constexpr size_t kNoAllocScratchBytes = size_t(128) << 20;
// Address of this device's array (looked up once per device, with the device current).
hipError_t noalloc_scratch(void** out);

struct PrepParams {
  const void* q;
  const void* k;
  const float* g;
  const void* beta;
  const int32_t* lengths;
  void* ws;          // records, see above
  int B, L, Hk, Hv, NC;
  // fused gate prologue (null b_raw = g and beta as given): beta = sigmoid(b_raw),
  // g = -exp(A_log) softplus(a_raw + dt_bias); b_raw, a_raw [B, L, Hv] in beta's dtype
  const void* b_raw;
  const void* a_raw;
  const float* A_log;     // [Hv]
  const float* dt_bias;   // [Hv]
  int32_t* chunk_list;     // bf16 with lengths: the chunk list and row order (written by the prep launch), else null
};

struct ScanParams {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* lengths;
  const float* s0;
  const int32_t* s0_row;
  void* o;
  float* s_final;
  const void* ws;    // records written by the prep kernel
  float* seg;        // segment states (bf16 with P > 1), see above
  int B, L, Hk, Hv, NC, n_s0;
  int P, Ls;         // segments and chunks per segment
  // truncated segment starts (bf16 with P > 1; see PlanEntry): plan [B Hv P], certificate parts
  // [B Hv P][kCertFloats], the status word; trunc = 0 forces the exact path everywhere
  PlanEntry* plan;
  float* cert;
  int32_t* status;
  int trunc;
  // bf16 without segments, with lengths: the rows by number of chunks, longest first (the chunk
  // list's row order); the output pass takes its rows in this order (null: row index order)
  const int32_t* row_order;
  // fused gated RMSNorm of o (bf16 output pass; null z = plain o): o <- w o / rms(o) silu(z)
  const void* z;     // [B, L, Hv, 128], o's dtype
  const float* norm_w;   // [128]
  float eps;
};

struct DecodeParams {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const void* beta;
  const int32_t* lengths;
  const float* s0;
  const int32_t* s0_row;
  void* o;
  float* s_final;
  int B, L, Hk, Hv, n_s0;
  // fused gate prologue (null b_raw = g and beta as given), as in PrepParams
  const void* b_raw;
  const void* a_raw;
  const float* A_log;
  const float* dt_bias;
  // fused gated RMSNorm of o (null z = plain o), as in ScanParams
  const void* z;
  const float* norm_w;
  float eps;
};

// Layer steps around the delta rule (gdr_layer.hip).
struct GatesParams {
  const void* b;          // [B, L, Hv] raw beta projection
  const void* a;          // [B, L, Hv] raw decay projection
  const float* A_log;     // [Hv]
  const float* dt_bias;   // [Hv]
  const int32_t* lengths;
  void* beta;             // [B, L, Hv], dtype of b
  float* g;               // [B, L, Hv]
  int B, L, Hv;
};

struct ConvParams {
  const void* mixed;      // [B, L, Cm], Cm = (2 Hk + Hv) 128
  const void* tail;       // [B, K-1, Cm] or null (zeros)
  const float* w;         // [Cm, K]
  const int32_t* lengths;
  void* q;                // [B, L, Hk, 128]
  void* k;                // [B, L, Hk, 128]
  void* v;                // [B, L, Hv, 128]
  void* new_tail;         // [B, K-1, Cm] or null; may be tail itself
  int B, L, Hk, Hv, K;
};

struct NormParams {
  const void* x;          // [rows, 128]
  const void* z;          // [rows, 128]
  const float* w;         // [128]
  float eps;
  void* out;              // [rows, 128]; may be x itself
  int64_t rows;
};

constexpr int kMaxConvTaps = 8;

hipError_t launch_gates(const GatesParams& p, int bf16, hipStream_t s);
hipError_t launch_conv_silu(const ConvParams& p, int bf16, hipStream_t s);
hipError_t launch_gated_rmsnorm(const NormParams& p, int bf16, hipStream_t s);

hipError_t launch_prep(const PrepParams& p, int qkv_bf16, int beta_bf16, hipStream_t s);
hipError_t launch_decode(const DecodeParams& p, int qkv_bf16, int beta_bf16, hipStream_t s);
// bf16 with P > 1: segment transitions (all segments but the last), then the combine that
// turns them into the state entering every segment; launch_scan always runs last.
hipError_t launch_transition(const ScanParams& p, hipStream_t s);
hipError_t launch_combine(const ScanParams& p, hipStream_t s);
hipError_t launch_scan(const ScanParams& p, int qkv_bf16, hipStream_t s);
// bf16 with P > 1, after launch_scan: checks the truncation certificates of every (row, head) that
// took the truncated path and reruns those whose bound fails from their entering state.
hipError_t launch_finalize(const ScanParams& p, hipStream_t s);

}  // namespace gdr

#endif  // GDR_INTERNAL_H_
