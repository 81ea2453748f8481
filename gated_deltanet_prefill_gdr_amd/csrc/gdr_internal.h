// Internal interface between the C ABI (gdr_api.cpp) and the HIP kernels (gdr_prep.hip, gdr_scan.hip).
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
//   P  = (q_hat k_hat^T) (.) E    (decayed causal scores, diagonal included)
// each as 6 blocks in MFMA operand order, one block per (token tile w, token block kb) that
// the lower triangle reaches: (0,0) (1,0) (2,0) (2,1) (3,0) (3,1). A block is 64 lanes x 8
// elements; lane (m = lane % 16, G = lane / 16) holds row 16w + m, columns
// 32kb + {4G..4G+3, 16+4G..16+4G+3}. Then 4 x 64 floats: a_t = e^{gamma_t} rk_t,
// c_t = e^{gamma_t} rq_t, d_t = rk_t e^{gamma_63 - gamma_t}, then e^{gamma_63} at [3][0].
constexpr int kFragBlocks = 6;
constexpr int kBlockElems = 64 * 8;

inline size_t record_bytes(size_t elem) {
  return 2 * size_t(kFragBlocks) * kBlockElems * elem + 4 * kChunk * sizeof(float);
}

inline size_t workspace_bytes(int B, int Hv, int NC, size_t elem) {
  return size_t(B) * Hv * NC * record_bytes(elem);
}

struct PrepParams {
  const void* q;
  const void* k;
  const float* g;
  const void* beta;
  const int32_t* lengths;
  void* ws;          // records, see above
  int B, L, Hk, Hv, NC;
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
  int B, L, Hk, Hv, NC, n_s0;
};

hipError_t launch_prep(const PrepParams& p, int qkv_bf16, int beta_bf16, hipStream_t s);
hipError_t launch_scan(const ScanParams& p, int qkv_bf16, hipStream_t s);

}  // namespace gdr

#endif  // GDR_INTERNAL_H_
