// Internal interface between the C ABI (gdr_api.cpp) and the HIP kernels (gdr_kernels.hip).
#ifndef GDR_INTERNAL_H_
#define GDR_INTERNAL_H_

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace gdr {

constexpr int kChunk = 64;      // tokens per chunk
constexpr int kHeadDim = 128;   // Dk = Dv

// Workspace layout, per (row b, value head h, chunk c) block index blk = (b*Hv + h)*NC + c:
//   tb   [blk][64][64]  element type of q/k/v: T diag(beta') of the chunk (zeros above diagonal)
//   p    [blk][64][64]  element type of q/k/v: (q_hat k_hat^T) (.) decay, lower incl. diagonal
//   scal [blk][4][64]   float: a_t, c_t, d_t, then e^{gamma_63} at [3][0]
struct WorkspaceLayout {
  size_t tb_off, p_off, scal_off, total;
};

inline WorkspaceLayout workspace_layout(int B, int Hv, int NC, size_t elem) {
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  const size_t nblk = size_t(B) * Hv * NC;
  WorkspaceLayout w;
  w.tb_off = 0;
  w.p_off = up(nblk * kChunk * kChunk * elem);
  w.scal_off = w.p_off + up(nblk * kChunk * kChunk * elem);
  w.total = w.scal_off + up(nblk * 4 * kChunk * sizeof(float));
  return w;
}

struct PrepParams {
  const void* q;
  const void* k;
  const float* g;
  const void* beta;
  const int32_t* lengths;
  void* ws_tb;
  void* ws_p;
  float* ws_scal;
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
  const void* ws_tb;
  const void* ws_p;
  const float* ws_scal;
  int B, L, Hk, Hv, NC, n_s0;
};

hipError_t launch_prep(const PrepParams& p, int qkv_bf16, int beta_bf16, hipStream_t s);
hipError_t launch_scan(const ScanParams& p, int qkv_bf16, hipStream_t s);

}  // namespace gdr

#endif  // GDR_INTERNAL_H_
