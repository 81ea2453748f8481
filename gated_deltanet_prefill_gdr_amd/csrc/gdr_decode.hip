// Token-by-token gated delta rule for short sequences (decode and fork continuation) (gfx950).
//
// One workgroup (256 threads) per (row b, value head h). The 128 x 128 fp32 state lives in
// registers: thread t holds column n = t % 128 for the 64 key indices 64 (t / 128) .. + 63. Each
// token follows the per-token recurrence of the kernel-test page (r15_kernel_test.py, function
// truth_f64) and of the model page (model.py, delta_rule_reference):
//   S <- e^{g'} S;  delta = beta' (v - S^T k_hat);  S <- S + k_hat delta^T;  o = S^T q_hat
// with q_hat, k_hat from _l2norm (eps inside the rsqrt), q_hat scaled by 128^-1/2, and the
// right-pad guard of _dn_gates (beta' = beta [t < len], g' = g [t < len]). The state is read once
// from s0 (row s0_row[b], the fork model's h0 / h0_idx) and written once to s_final, so the cost
// is the state traffic plus the token rows: the path is bound by HBM.
// Optional fused work (the fork layer's order, model.py, _fork_linear_layer): beta, g formed from
// the raw projections per token (_dn_gates), and the gated RMSNorm of each token's output with its
// gate z (_gated_rms), so that a decode step reads the raw projections and writes the normalised
// output.
#include "gdr_device.h"

namespace gdr {

template <typename T, typename TB>
__global__ __launch_bounds__(256) void gdr_decode_kernel(DecodeParams p) {
  __shared__ float qs[D], ks[D];
  __shared__ float part[2][2][D];   // [kv or o][key half][column] partial sums
  __shared__ float scal[4];         // r_k, r_q of the current token; the norm's two partial sums
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = tid & (D - 1), half = tid >> 7;
  const int h = blockIdx.x % p.Hv, b = blockIdx.x / p.Hv;
  const int kh = h / (p.Hv / p.Hk);
  const T* qg = reinterpret_cast<const T*>(p.q);
  const T* kg = reinterpret_cast<const T*>(p.k);
  const T* vg = reinterpret_cast<const T*>(p.v);
  T* og = reinterpret_cast<T*>(p.o);
  const TB* betag = reinterpret_cast<const TB*>(p.beta);

  const int len = p.lengths ? p.lengths[b] : p.L;
  const int srow = p.s0 ? (p.s0_row ? p.s0_row[b] : b) : 0;
  if ((len < 0 || len > p.L) || (p.s0 && (srow < 0 || srow >= p.n_s0))) {
    const float nan = __builtin_nanf("");
    for (int i = tid; i < p.L * D; i += 256) og[((size_t)b * p.L + i / D) * p.Hv * D + (size_t)h * D + i % D] = from_f<T>(nan);
    if (p.s_final)
      for (int i = tid; i < D * D; i += 256) p.s_final[((size_t)b * p.Hv + h) * D * D + i] = nan;
    return;
  }

  float S[64];
  {
    const float* s0 = p.s0 ? p.s0 + ((size_t)srow * p.Hv + h) * D * D : nullptr;
#pragma unroll
    for (int i = 0; i < 64; ++i) S[i] = s0 ? s0[(64 * half + i) * D + n] : 0.f;
  }
  for (int t = 0; t < p.L; ++t) {
    const size_t tok = (size_t)b * p.L + t;
    const bool valid = t < len;
    // q, k rows of the token into LDS, inverse norms (waves 0 and 1), v of this column
    if (tid < D) {
      ks[tid] = to_f(kg[(tok * p.Hk + kh) * D + tid]);
      qs[tid] = to_f(qg[(tok * p.Hk + kh) * D + tid]);
    }
    const float vn = to_f(vg[(tok * p.Hv + h) * D + n]);
    float gv = 0.f, bv = 0.f;
    if (valid) {
      if (p.b_raw) {   // fused gate prologue (model.py, _dn_gates)
        const float x = to_f(reinterpret_cast<const TB*>(p.a_raw)[tok * p.Hv + h]) + p.dt_bias[h];
        gv = -__expf(p.A_log[h]) * (fmaxf(x, 0.f) + log1pf(__expf(-fabsf(x))));
        bv = __builtin_amdgcn_rcpf(1.0f + __expf(-to_f(reinterpret_cast<const TB*>(p.b_raw)[tok * p.Hv + h])));
      } else {
        gv = p.g[tok * p.Hv + h];
        bv = to_f(betag[tok * p.Hv + h]);
      }
    }
    __syncthreads();
    if (wave < 2) {
      const float* x = wave == 0 ? ks : qs;
      float s2 = x[lane] * x[lane] + x[lane + 64] * x[lane + 64];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) s2 += __shfl_xor(s2, off);
      if (lane == 0) scal[wave] = 1.0f / sqrtf(s2 + 1e-6f) * (wave == 1 ? 0.08838834764831845f : 1.f);
    }
    __syncthreads();
    const float rk = scal[0], rq = scal[1];
    // decay, then k_hat^T S for this column over this half of the keys
    const float eg = expf(gv);
    float kv = 0.f;
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      S[i] *= eg;
      kv += S[i] * ks[64 * half + i];
    }
    part[0][half][n] = kv * rk;
    __syncthreads();
    const float delta = bv * (vn - (part[0][0][n] + part[0][1][n]));
    float ov = 0.f;
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      S[i] += (ks[64 * half + i] * rk) * delta;
      ov += S[i] * qs[64 * half + i];
    }
    part[1][half][n] = ov * rq;
    __syncthreads();
    float on = part[1][0][n] + part[1][1][n];
    if (p.z) {   // fused gated RMSNorm: the sum of squares over the 128 outputs (waves 0, 1)
      if (half == 0) {
        float s2 = on * on;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) s2 += __shfl_xor(s2, off);
        if (lane == 0) scal[2 + wave] = s2;
      }
      __syncthreads();
      const float r = 1.0f / sqrtf((scal[2] + scal[3]) * (1.0f / D) + p.eps);
      const float zf = to_f(reinterpret_cast<const T*>(p.z)[(tok * p.Hv + h) * D + n]);
      on = p.norm_w[n] * (on * r) * (zf * __builtin_amdgcn_rcpf(1.0f + __expf(-zf)));
    }
    if (half == 0) og[(tok * p.Hv + h) * D + n] = from_f<T>(on);
    // the next token's staging waits for every thread's reads of this one
    __syncthreads();
  }
  if (p.s_final) {
    float* sf = p.s_final + ((size_t)b * p.Hv + h) * D * D;
#pragma unroll
    for (int i = 0; i < 64; ++i) sf[(64 * half + i) * D + n] = S[i];
  }
}

hipError_t launch_decode(const DecodeParams& p, int qkv_bf16, int beta_bf16, hipStream_t s) {
  const dim3 grid((unsigned)(p.B * p.Hv));
  if (qkv_bf16) {
    if (beta_bf16)
      hipLaunchKernelGGL((gdr_decode_kernel<__bf16, __bf16>), grid, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL((gdr_decode_kernel<__bf16, float>), grid, dim3(256), 0, s, p);
  } else {
    hipLaunchKernelGGL((gdr_decode_kernel<float, float>), grid, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace gdr
