// The layer steps on either side of the delta rule (gfx950): gate prologue, causal depthwise
// conv + SiLU with tail continuation and the q/k/v split, gated RMSNorm. All three are
// elementwise or short-window work bound by HBM: each reads its inputs once and writes its
// outputs once, with 16-byte accesses coalesced along the channel axis.
//
// Definitions: the model page (model.py), functions _dn_gates, _conv_silu with the tail gather
// of _linear_layer, and _gated_rms. Arithmetic is fp32; results are rounded once to the
// output dtype.
#include "gdr_device.h"

namespace gdr {

// 1 / (1 + e^-x) with the hardware exp2 and reciprocal (about 1 ulp each; an IEEE division would
// cost more than the rest of an element's arithmetic in these memory-bound kernels)
__device__ __forceinline__ float sigmoidf_(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x * -1.4426950408889634f));
}
// log(1 + e^x) without overflow: max(x, 0) + log1p(e^-|x|)
__device__ __forceinline__ float softplusf_(float x) { return fmaxf(x, 0.f) + log1pf(__expf(-fabsf(x))); }

// ---------------------------------------------------------------- gate prologue
// beta = sigmoid(b) [t < len], g = -exp(A_log[h]) softplus(a + dt_bias[h]) [t < len].
// One thread per (row, token, value head); a row with an out-of-range length gets NaN gates.
template <typename T>
__global__ __launch_bounds__(256) void gdr_gates_kernel(GatesParams p) {
  const int64_t n = int64_t(p.B) * p.L * p.Hv;
  const T* bg = reinterpret_cast<const T*>(p.b);
  const T* ag = reinterpret_cast<const T*>(p.a);
  T* beta = reinterpret_cast<T*>(p.beta);
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256) {
    const int h = (int)(i % p.Hv);
    const int64_t bt = i / p.Hv;
    const int t = (int)(bt % p.L), b = (int)(bt / p.L);
    const int len = p.lengths ? p.lengths[b] : p.L;
    float bv, gv;
    if (len < 0 || len > p.L) {
      bv = gv = __builtin_nanf("");
    } else if (t < len) {
      bv = sigmoidf_(to_f(bg[i]));
      gv = -__expf(p.A_log[h]) * softplusf_(to_f(ag[i]) + p.dt_bias[h]);
    } else {
      bv = gv = 0.f;
    }
    beta[i] = from_f<T>(bv);
    p.g[i] = gv;
  }
}

// ---------------------------------------------------------------- conv + SiLU
// pre[t, c] = sum_j ext[t + j, c] w[c, j] over ext = [tail ; mixed] (K-1 + L rows), out = silu(pre),
// channels split into q [0, Hk D), k [Hk D, 2 Hk D), v [2 Hk D, Cm). Thread layout: four channels
// per thread (an 8-byte bf16 or 16-byte fp32 vector; a wave covers 256 consecutive channels of a
// token row), 256 threads per workgroup along the channel axis, kConvTile tokens per workgroup
// along time; each thread slides a window of K-1 rows in registers down its tokens, so every mixed
// element is read once (plus K-1 halo rows per tile, from L2).
// The workgroup of the first tile of each row also writes the new tail; each thread reads the old
// tail entries of its own channels before it writes them, and no other thread reads them (later
// tiles take their halo from mixed), so in-place tail updates (new_tail == tail) are safe.
constexpr int kConvTile = 64;
constexpr int kConvVec = 4;   // channels per thread

template <typename T> struct Vec4;
template <> struct Vec4<__bf16> {
  uint2 raw;
  static __device__ __forceinline__ Vec4 load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    Vec4 v;
    v.raw = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
    return v;
  }
  __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, uint32_t off) const {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, raw), r, off, 0, 0);
  }
};
template <> struct Vec4<float> {
  uint4 raw;
  static __device__ __forceinline__ Vec4 load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    Vec4 v;
    v.raw = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    return v;
  }
  __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, uint32_t off) const {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, raw), r, off, 0, 0);
  }
};
template <typename T> __device__ __forceinline__ float vget(const Vec4<T>& v, int e) {
  return to_f(reinterpret_cast<const T*>(&v.raw)[e]);
}
template <typename T> __device__ __forceinline__ void vset(Vec4<T>& v, int e, float x) {
  reinterpret_cast<T*>(&v.raw)[e] = from_f<T>(x);
}

template <typename T, int K>
__global__ __launch_bounds__(256) void gdr_conv_silu_kernel(ConvParams p) {
  constexpr int VN = kConvVec;
  constexpr int K1 = K - 1;
  const int Cm = (2 * p.Hk + p.Hv) * D;
  const int cv = blockIdx.x * 256 + threadIdx.x;   // channel vector
  if (cv >= Cm / VN) return;
  const int tile = blockIdx.y, b = blockIdx.z;
  const int t0 = tile * kConvTile;
  const int c0 = cv * VN;

  float w[VN][K];
#pragma unroll
  for (int e = 0; e < VN; ++e)
#pragma unroll
    for (int j = 0; j < K; ++j) w[e][j] = p.w[(size_t)(c0 + e) * K + j];

  // range-checked descriptors: loads past the end read zeros, stores past it are dropped
  const uint32_t row_bytes = (uint32_t)Cm * sizeof(T);
  const __amdgpu_buffer_rsrc_t rm =
      make_rsrc(reinterpret_cast<const T*>(p.mixed) + (size_t)b * p.L * Cm, (uint32_t)p.L * row_bytes);
  const __amdgpu_buffer_rsrc_t rt =
      make_rsrc(p.tail ? reinterpret_cast<const T*>(p.tail) + (size_t)b * K1 * Cm : nullptr,
                p.tail ? (uint32_t)K1 * row_bytes : 0u);
  const uint32_t coff = (uint32_t)c0 * sizeof(T);
  auto load_mixed = [&](int t) { return Vec4<T>::load(rm, (uint32_t)t * row_bytes + coff); };
  auto load_tail = [&](int j) { return Vec4<T>::load(rt, (uint32_t)j * row_bytes + coff); };   // ext row j < K-1

  // window: rows t0 - K1 .. t0 - 1 of mixed (from the tail where t < 0)
  float win[K1 > 0 ? K1 : 1][VN];
#pragma unroll
  for (int j = 0; j < K1; ++j) {
    const int t = t0 - K1 + j;
    const Vec4<T> r = t >= 0 ? load_mixed(t) : load_tail(K1 + t);
#pragma unroll
    for (int e = 0; e < VN; ++e) win[j][e] = vget(r, e);
  }

  // destination of this channel vector
  const int kd = p.Hk * D;
  T* dst;
  int dpitch, dc;
  if (c0 < kd) {
    dst = reinterpret_cast<T*>(p.q); dpitch = kd; dc = c0;
  } else if (c0 < 2 * kd) {
    dst = reinterpret_cast<T*>(p.k); dpitch = kd; dc = c0 - kd;
  } else {
    dst = reinterpret_cast<T*>(p.v); dpitch = p.Hv * D; dc = c0 - 2 * kd;
  }
  const uint32_t drow = (uint32_t)dpitch * sizeof(T);
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(dst + (size_t)b * p.L * dpitch, (uint32_t)p.L * drow);
  const uint32_t dcoff = (uint32_t)dc * sizeof(T);

  // tokens loaded together: eight keep 64 bytes per thread in flight (110 -> 104 us at L = 16384,
  // Cm = 8192, also when the gate and norm kernels run around it; sixteen gain nothing more)
  constexpr int U = 8;
#pragma unroll 1
  for (int tt = 0; tt < kConvTile; tt += U) {
    Vec4<T> raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) raw[u] = load_mixed(t0 + tt + u);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      Vec4<T> y;
#pragma unroll
      for (int e = 0; e < VN; ++e) {
        const float cur = vget(raw[u], e);
        float acc = cur * w[e][K1];
#pragma unroll
        for (int j = 0; j < K1; ++j) acc += win[j][e] * w[e][j];
#pragma unroll
        for (int j = 0; j + 1 < K1; ++j) win[j][e] = win[j + 1][e];
        if constexpr (K1 > 0) win[K1 - 1][e] = cur;
        vset(y, e, acc * sigmoidf_(acc));
      }
      y.store(rd, (uint32_t)(t0 + tt + u) * drow + dcoff);
    }
  }

  // new tail = ext rows len .. len + K-2 (ext row r is tail row r for r < K-1, else mixed row r - K+1)
  if constexpr (K1 > 0) {
    if (tile == 0 && p.new_tail) {
      const int len = p.lengths ? p.lengths[b] : p.L;
      const __amdgpu_buffer_rsrc_t rn =
          make_rsrc(reinterpret_cast<T*>(p.new_tail) + (size_t)b * K1 * Cm, (uint32_t)K1 * row_bytes);
      Vec4<T> r[K1];
#pragma unroll
      for (int j = 0; j < K1; ++j) {
        if (len < 0 || len > p.L) {
#pragma unroll
          for (int e = 0; e < VN; ++e) vset(r[j], e, __builtin_nanf(""));
        } else {
          // this thread alone reads and writes these tail entries, so the old tail is still intact
          const int e = len + j;   // ext row
          r[j] = e < K1 ? load_tail(e) : load_mixed(e - K1);
        }
      }
#pragma unroll
      for (int j = 0; j < K1; ++j) r[j].store(rn, (uint32_t)j * row_bytes + coff);
    }
  }
}

// ---------------------------------------------------------------- gated RMSNorm
// y = w x / sqrt(mean(x^2) + eps) silu(z) per 128-wide row. A row is spread over 128 / VN lanes
// of one wave (16-byte vectors); the sum of squares is a butterfly over those lanes. Each lane
// group handles kNormRows rows, all loads issued before any arithmetic.
constexpr int kNormRows = 2;

template <typename T>
__global__ __launch_bounds__(256) void gdr_gated_rmsnorm_kernel(NormParams p) {
  constexpr int VN = 16 / sizeof(T);
  constexpr int LPR = D / VN;          // lanes per row
  constexpr int GPW = 256 / LPR;       // row groups per workgroup
  const int lr = threadIdx.x % LPR;
  // pass i of a workgroup covers GPW consecutive rows: one contiguous run of 4 KiB (bf16)
  const int64_t row0 = int64_t(blockIdx.x) * GPW * kNormRows + threadIdx.x / LPR;
  const T* xg = reinterpret_cast<const T*>(p.x);
  const T* zg = reinterpret_cast<const T*>(p.z);
  T* og = reinterpret_cast<T*>(p.out);
  // rows past the end are skipped as a whole row group (a row's lanes share one wave)
  Vec16<T> x[kNormRows] = {}, z[kNormRows] = {};
#pragma unroll
  for (int i = 0; i < kNormRows; ++i) {
    if (row0 + i * GPW < p.rows) {
      const size_t off = (size_t)(row0 + i * GPW) * D + (size_t)lr * VN;
      x[i].raw = *reinterpret_cast<const uint4*>(xg + off);
      z[i].raw = *reinterpret_cast<const uint4*>(zg + off);
    }
  }
  float w[VN];
#pragma unroll
  for (int e = 0; e < VN; ++e) w[e] = p.w[lr * VN + e];
#pragma unroll
  for (int i = 0; i < kNormRows; ++i) {
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < VN; ++e) {
      const float xf = to_f(x[i].get(e));
      ss += xf * xf;
    }
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) ss += __shfl_xor(ss, m);
    const float r = 1.0f / sqrtf(ss * (1.0f / D) + p.eps);
    Vec16<T> y;
#pragma unroll
    for (int e = 0; e < VN; ++e) {
      const float zf = to_f(z[i].get(e));
      reinterpret_cast<T*>(&y.raw)[e] = from_f<T>(w[e] * (to_f(x[i].get(e)) * r) * (zf * sigmoidf_(zf)));
    }
    if (row0 + i * GPW < p.rows) *reinterpret_cast<uint4*>(og + (size_t)(row0 + i * GPW) * D + (size_t)lr * VN) = y.raw;
  }
}

// ---------------------------------------------------------------- launchers
hipError_t launch_gates(const GatesParams& p, int bf16, hipStream_t s) {
  const int64_t n = int64_t(p.B) * p.L * p.Hv;
  const int64_t want = (n + 255) / 256;
  const unsigned grid = (unsigned)(want < 65536 ? want : 65536);
  if (bf16)
    hipLaunchKernelGGL(gdr_gates_kernel<__bf16>, dim3(grid), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(gdr_gates_kernel<float>, dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_conv_t(const ConvParams& p, hipStream_t s) {
  const int nvec = (2 * p.Hk + p.Hv) * D / kConvVec;
  const int tiles = p.L > 0 ? (p.L + kConvTile - 1) / kConvTile : 1;   // L = 0 still carries the tail
  const dim3 grid((unsigned)((nvec + 255) / 256), (unsigned)tiles, (unsigned)p.B);
  switch (p.K) {
    case 1: hipLaunchKernelGGL((gdr_conv_silu_kernel<T, 1>), grid, dim3(256), 0, s, p); break;
    case 2: hipLaunchKernelGGL((gdr_conv_silu_kernel<T, 2>), grid, dim3(256), 0, s, p); break;
    case 3: hipLaunchKernelGGL((gdr_conv_silu_kernel<T, 3>), grid, dim3(256), 0, s, p); break;
    case 4: hipLaunchKernelGGL((gdr_conv_silu_kernel<T, 4>), grid, dim3(256), 0, s, p); break;
    case 5: hipLaunchKernelGGL((gdr_conv_silu_kernel<T, 5>), grid, dim3(256), 0, s, p); break;
    case 6: hipLaunchKernelGGL((gdr_conv_silu_kernel<T, 6>), grid, dim3(256), 0, s, p); break;
    case 7: hipLaunchKernelGGL((gdr_conv_silu_kernel<T, 7>), grid, dim3(256), 0, s, p); break;
    case 8: hipLaunchKernelGGL((gdr_conv_silu_kernel<T, 8>), grid, dim3(256), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_conv_silu(const ConvParams& p, int bf16, hipStream_t s) {
  return bf16 ? launch_conv_t<__bf16>(p, s) : launch_conv_t<float>(p, s);
}

hipError_t launch_gated_rmsnorm(const NormParams& p, int bf16, hipStream_t s) {
  const int rpw = (bf16 ? 256 / (D / 8) : 256 / (D / 4)) * kNormRows;   // rows per workgroup
  const int64_t blocks = (p.rows + rpw - 1) / rpw;
  if (bf16)
    hipLaunchKernelGGL(gdr_gated_rmsnorm_kernel<__bf16>, dim3((unsigned)blocks), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(gdr_gated_rmsnorm_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace gdr
