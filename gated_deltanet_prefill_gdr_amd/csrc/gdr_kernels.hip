// Chunked gated delta rule prefill: HIP kernels for gfx950 (MI355X).
//
// The recurrence (kernel-test page r15_kernel_test.py, function truth_f64; model page model.py,
// function delta_rule_reference) is evaluated in chunks of C = 64 tokens. Inside a chunk, with
// gamma_t the inclusive cumulative sum of the guarded log decay g'_t, the derivation from the
// per-token recurrence gives (S = state entering the chunk, [Dk, Dv]):
//
//   A[t][i]  = beta'_t e^{gamma_t - gamma_i} k_hat_t . k_hat_i    (i < t)
//   T        = (I + A)^-1
//   Delta    = T diag(beta') (V - diag(e^gamma) K_hat S)          (row t = delta_t)
//   O        = diag(e^gamma) Q_hat S + (Q_hat K_hat^T (.) E) Delta,  E[t][i] = e^{gamma_t - gamma_i}, i <= t
//   S_next   = e^{gamma_63} S + K_hat^T diag(e^{gamma_63 - gamma}) Delta
//
// Two kernels:
//   gdr_prep  - one workgroup per (row, key head, chunk): l2 norms, the Gram K K^T and Q K^T
//               on MFMA (shared by the value heads of the key head), the cumulative decay, the
//               64x64 unit-lower-triangular inverse in LDS (16x16 diagonal blocks by forward
//               substitution, off-diagonal blocks by fp32 MFMA), and it stores per value head
//               and chunk: Tb = T diag(beta'), P = (Q_hat K_hat^T) (.) E, and the per-token
//               scalars a = e^gamma rk, c = e^gamma rq, d = rk e^{gamma_63 - gamma}, e^{gamma_63}.
//   gdr_scan  - one workgroup per (row, value head, 64-column slice of Dv); each wave owns 16
//               state columns (all 128 key rows, fp32 in MFMA accumulators) and walks the chunks
//               in order. The raw (un-normalised) q/k go straight into the MFMAs; the l2 norms
//               and decays enter as per-row scalings of the fp32 accumulators, which commute
//               with the products.
//
// Operand trick. An MFMA sums over k; which physical k index a (lane group, register slot)
// pair stands for does not matter as long as the A and B operands agree. The accumulator of a
// 16x16 tile holds, in lane (n = lane % 16, G = lane / 16), rows 4G .. 4G+3 of column n. Two
// such tiles (rows 0..15 and 16..31) therefore give each lane exactly 8 values of one column,
// which is a full B operand for a 32-deep k block if slot j of lane group G stands for row
// (j < 4 ? 4G + j : 16 + 4G + j - 4). A-operands are loaded from row-major LDS with the same
// slot order (two 4-element reads per lane), so the state, Delta and the residuals feed the
// next product straight from registers, with no LDS round trip.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdr_internal.h"

namespace gdr {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int C = kChunk;   // 64 tokens per chunk
constexpr int D = kHeadDim; // Dk = Dv = 128

// ------------------------------------------------------------------ element helpers
template <typename T> __device__ __forceinline__ float to_f(T x);
template <> __device__ __forceinline__ float to_f<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f<__bf16>(__bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ __bf16 from_f<__bf16>(float x) { return (__bf16)x; }

// 16-byte vector of T (8 bf16 or 4 float), for global <-> LDS staging.
template <typename T> struct Vec16 {
  static constexpr int N = 16 / sizeof(T);
  uint4 raw;
  __device__ __forceinline__ T get(int i) const { return reinterpret_cast<const T*>(&raw)[i]; }
};

// ------------------------------------------------------------------ MFMA fragments
// Eight k-values per lane in the slot order described at the top of this file.
template <typename T> struct Frag;
template <> struct Frag<float> { float v[8]; };
template <> struct Frag<__bf16> { bf16x8 v; };

__device__ __forceinline__ void mma(f4& acc, const Frag<__bf16>& a, const Frag<__bf16>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f4& acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], acc, 0, 0, 0);
}

// A-operand (or B-operand of a transposed product) from row-major LDS: row `row`, k block
// starting at k0; lane group G reads elements k0+4G..k0+4G+3 and k0+16+4G..k0+16+4G+3.
__device__ __forceinline__ Frag<__bf16> lds_frag(const __bf16* base, int pitch, int row, int k0, int G) {
  const __bf16* p = base + row * pitch + k0 + 4 * G;
  bf16x4 lo = *reinterpret_cast<const bf16x4*>(p);
  bf16x4 hi = *reinterpret_cast<const bf16x4*>(p + 16);
  Frag<__bf16> f;
  f.v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return f;
}
__device__ __forceinline__ Frag<float> lds_frag(const float* base, int pitch, int row, int k0, int G) {
  const float* p = base + row * pitch + k0 + 4 * G;
  f4 lo = *reinterpret_cast<const f4*>(p);
  f4 hi = *reinterpret_cast<const f4*>(p + 16);
  Frag<float> f;
#pragma unroll
  for (int j = 0; j < 4; ++j) { f.v[j] = lo[j]; f.v[4 + j] = hi[j]; }
  return f;
}

// B-operand from two accumulator tiles (rows 0..15 and 16..31 of a 32-deep k block), each
// row scaled by s0[i] / s1[i] (the per-row scalars of this lane's rows).
template <typename T>
__device__ __forceinline__ Frag<T> acc_frag(const f4& t0, const f4& t1, const f4& s0, const f4& s1);
template <>
__device__ __forceinline__ Frag<__bf16> acc_frag<__bf16>(const f4& t0, const f4& t1, const f4& s0, const f4& s1) {
  Frag<__bf16> f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f.v[j] = (__bf16)(t0[j] * s0[j]);
    f.v[4 + j] = (__bf16)(t1[j] * s1[j]);
  }
  return f;
}
template <>
__device__ __forceinline__ Frag<float> acc_frag<float>(const f4& t0, const f4& t1, const f4& s0, const f4& s1) {
  Frag<float> f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f.v[j] = t0[j] * s0[j];
    f.v[4 + j] = t1[j] * s1[j];
  }
  return f;
}

__device__ __forceinline__ f4 f4_splat(float x) { return f4{x, x, x, x}; }

// LDS row pitches (elements): 16 extra bytes per row for bf16 tiles keep the two 8-byte
// fragment reads of 16 rows spread over the banks; fp32 gets 16 bytes too (its LDS is tight).
template <typename T> struct Pitch;
template <> struct Pitch<__bf16> { static constexpr int K = D + 16, T64 = C + 16; };
template <> struct Pitch<float> { static constexpr int K = D + 4, T64 = C + 4; };

constexpr int kFP = C + 4;   // pitch of the fp32 64x64 LDS matrices in the prep kernel

// ====================================================================== prep kernel
template <typename T, typename TB>
struct PrepSmem {
  union {
    struct { T k[C * Pitch<T>::K]; T q[C * Pitch<T>::K]; } in;      // phase 1
    struct { float a[C * kFP]; float t[C * kFP]; } inv;            // phase 2
  } u;
  float rk[C], rq[C], gam[C], bet[C];
};

template <typename T, typename TB>
__global__ __launch_bounds__(256) void gdr_prep(PrepParams p) {
  __shared__ __attribute__((aligned(16))) PrepSmem<T, TB> sm;
  constexpr int PK = Pitch<T>::K;
  constexpr int VN = Vec16<T>::N;              // elements per 16-byte vector
  constexpr int VPR = D / VN;                  // vectors per 128-wide row
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n16 = lane & 15, G = lane >> 4;
  const int c = blockIdx.x, kh = blockIdx.y, b = blockIdx.z;
  const int r = p.Hv / p.Hk;
  const int t0 = c * C;
  int len = p.lengths ? p.lengths[b] : p.L;
  len = len < 0 ? 0 : (len > p.L ? p.L : len);

  const T* qg = reinterpret_cast<const T*>(p.q);
  const T* kg = reinterpret_cast<const T*>(p.k);

  // ---- stage q, k of the chunk into LDS; row sums of squares via 16/32-lane reductions
#pragma unroll
  for (int m = 0; m < (C * VPR) / 256; ++m) {
    const int idx = tid + 256 * m, row = idx / VPR, cv = idx % VPR;
    const int t = t0 + row;
    Vec16<T> kv, qv;
    kv.raw = make_uint4(0, 0, 0, 0);
    qv.raw = make_uint4(0, 0, 0, 0);
    if (t < p.L) {
      const size_t off = ((size_t)b * p.L + t) * p.Hk * D + (size_t)kh * D + cv * VN;
      kv.raw = *reinterpret_cast<const uint4*>(kg + off);
      qv.raw = *reinterpret_cast<const uint4*>(qg + off);
    }
    *reinterpret_cast<uint4*>(&sm.u.in.k[row * PK + cv * VN]) = kv.raw;
    *reinterpret_cast<uint4*>(&sm.u.in.q[row * PK + cv * VN]) = qv.raw;
    float sk = 0.f, sq = 0.f;
#pragma unroll
    for (int e = 0; e < VN; ++e) {
      const float x = to_f(kv.get(e)), y = to_f(qv.get(e));
      sk += x * x;
      sq += y * y;
    }
#pragma unroll
    for (int off = 1; off < VPR; off <<= 1) {
      sk += __shfl_xor(sk, off);
      sq += __shfl_xor(sq, off);
    }
    if (cv == 0) {
      sm.rk[row] = 1.0f / sqrtf(sk + 1e-6f);
      sm.rq[row] = (1.0f / sqrtf(sq + 1e-6f)) * 0.08838834764831845f;   // * 128^-1/2
    }
  }
  __syncthreads();

  // ---- lower-triangle 16x16 tiles of K K^T and Q K^T (10 each); wave w owns tiles w, w+4, w+8
  constexpr int kTiles = 10;   // tile ti = I(I+1)/2 + J of the lower triangle, J <= I
  auto tile_i = [](int ti) { return (ti >= 1) + (ti >= 3) + (ti >= 6); };
  auto tile_j = [&](int ti) { const int I = tile_i(ti); return ti - I * (I + 1) / 2; };
  f4 gacc[3], qacc[3];
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    gacc[s] = f4_splat(0.f);
    qacc[s] = f4_splat(0.f);
    const int ti = wave + 4 * s;
    if (ti < kTiles) {
      const int I = tile_i(ti), J = tile_j(ti);
#pragma unroll
      for (int kb = 0; kb < D / 32; ++kb) {
        Frag<T> bk = lds_frag(sm.u.in.k, PK, 16 * J + n16, 32 * kb, G);
        Frag<T> ak = lds_frag(sm.u.in.k, PK, 16 * I + n16, 32 * kb, G);
        Frag<T> aq = lds_frag(sm.u.in.q, PK, 16 * I + n16, 32 * kb, G);
        mma(gacc[s], ak, bk);
        mma(qacc[s], aq, bk);
      }
    }
  }
  __syncthreads();   // q/k staging area is reused below

  T* Tb_all = reinterpret_cast<T*>(p.ws_tb);
  T* P_all = reinterpret_cast<T*>(p.ws_p);
  const TB* betag = reinterpret_cast<const TB*>(p.beta);

  for (int hr = 0; hr < r; ++hr) {
    const int h = kh * r + hr;
    const size_t blk = ((size_t)b * p.Hv + h) * p.NC + c;
    T* Tb = Tb_all + blk * (C * C);
    T* Pm = P_all + blk * (C * C);
    float* sc = p.ws_scal + blk * (4 * C);

    // -- guarded gates and the inclusive cumulative decay (wave 0, lane = token)
    if (wave == 0) {
      const int t = t0 + lane;
      float gv = 0.f, bv = 0.f;
      if (t < len) {
        const size_t off = ((size_t)b * p.L + t) * p.Hv + h;
        gv = p.g[off];
        bv = to_f(betag[off]);
      }
      float x = gv;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off);
        if (lane >= off) x += y;
      }
      const float gC = __shfl(x, 63);
      sm.gam[lane] = x;
      sm.bet[lane] = bv;
      const float eg = expf(x);
      sc[lane] = eg * sm.rk[lane];                      // a_t
      sc[C + lane] = eg * sm.rq[lane];                  // c_t
      sc[2 * C + lane] = sm.rk[lane] * expf(gC - x);    // d_t
      sc[3 * C + lane] = (lane == 0) ? expf(gC) : 0.f;
    }
    __syncthreads();

    // -- A (strictly lower, fp32 in LDS) and P (lower incl. diagonal, to global)
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      const int ti = wave + 4 * s;
      if (ti < kTiles) {
        const int I = tile_i(ti), J = tile_j(ti);
        const int col = 16 * J + n16;
        const float gcol = sm.gam[col], rkcol = sm.rk[col];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = 16 * I + 4 * G + e;
          const float dg = sm.gam[row] - gcol;
          const float dec = expf(row >= col ? dg : 0.f);
          const float av = (row > col) ? sm.bet[row] * dec * sm.rk[row] * rkcol * gacc[s][e] : 0.f;
          const float pv = (row >= col) ? sm.rq[row] * rkcol * dec * qacc[s][e] : 0.f;
          sm.u.inv.a[row * kFP + col] = av;
          Pm[row * C + col] = from_f<T>(pv);
          if (I != J) Pm[col * C + row] = from_f<T>(0.f);   // the mirrored upper tile
        }
      }
    }
    __syncthreads();

    // -- diagonal 16x16 blocks of T by forward substitution (wave w: block w, lane = column)
    if (n16 == lane) {   // lanes 0..15
      const int o = 16 * wave;
      const int kcol = lane;
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float s = (i == kcol) ? 1.f : 0.f;
        const float* arow = &sm.u.inv.a[(o + i) * kFP + o];
#pragma unroll
        for (int j = 0; j < i; ++j) s -= arow[j] * x[j];
        x[i] = s;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) sm.u.inv.t[(o + i) * kFP + o + kcol] = x[i];
    }
    __syncthreads();

    // -- off-diagonal blocks: T_IJ = -T_II sum_{M=J}^{I-1} A_IM T_MJ (wave J: block column J)
    if (wave < 3) {
      const int J = wave;
      for (int I = J + 1; I < 4; ++I) {
        f4 X = f4_splat(0.f);
        for (int M = J; M < I; ++M) {
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const float av = sm.u.inv.a[(16 * I + n16) * kFP + 16 * M + 4 * G + s];
            const float bv = sm.u.inv.t[(16 * M + 4 * G + s) * kFP + 16 * J + n16];
            X = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, X, 0, 0, 0);
          }
        }
        f4 Y = f4_splat(0.f);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const float av = sm.u.inv.t[(16 * I + n16) * kFP + 16 * I + 4 * G + s];
          Y = __builtin_amdgcn_mfma_f32_16x16x4f32(av, X[s], Y, 0, 0, 0);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) sm.u.inv.t[(16 * I + 4 * G + s) * kFP + 16 * J + n16] = -Y[s];
      }
    }
    __syncthreads();

    // -- Tb = T diag(beta'), lower triangle incl. diagonal, zeros above (coalesced rows)
    for (int idx = tid; idx < C * C; idx += 256) {
      const int row = idx / C, col = idx % C;
      const float v = (col <= row) ? sm.u.inv.t[row * kFP + col] * sm.bet[col] : 0.f;
      Tb[idx] = from_f<T>(v);
    }
    __syncthreads();
  }
}

// ====================================================================== scan kernel
template <typename T, int NW>
struct ScanSmem {
  T k[C * Pitch<T>::K];        // K chunk, [token][dk]
  T q[C * Pitch<T>::K];        // Q chunk, [token][dk]
  T kt[D * Pitch<T>::T64];     // K chunk transposed, [dk][token]
  T tb[C * Pitch<T>::T64];     // T diag(beta'), [token][token]
  T pm[C * Pitch<T>::T64];     // decayed causal q.k scores, [token][token]
  T v[C * Pitch<T>::T64];      // this workgroup's 64 value columns, [token][col]
  float sc[4 * C];             // a, c, d, e^{gamma_63}
};

template <typename T, int NW>
__global__ __launch_bounds__(64 * NW) void gdr_scan(ScanParams p) {
  static_assert(NW == 4, "the staging loops assume 4 waves (64 value columns per workgroup)");
  __shared__ __attribute__((aligned(16))) ScanSmem<T, NW> sm;
  constexpr int PK = Pitch<T>::K, PT = Pitch<T>::T64;
  constexpr int VN = Vec16<T>::N;
  constexpr int NT = 64 * NW;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n16 = lane & 15, G = lane >> 4;
  const int cg = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int r = p.Hv / p.Hk, kh = h / r;
  const int col0 = cg * (16 * NW);            // first value column of this workgroup
  const int ncol = col0 + 16 * wave + n16;    // this lane's value column

  const T* qg = reinterpret_cast<const T*>(p.q);
  const T* kg = reinterpret_cast<const T*>(p.k);
  const T* vg = reinterpret_cast<const T*>(p.v);
  T* og = reinterpret_cast<T*>(p.o);
  const T* Tb_all = reinterpret_cast<const T*>(p.ws_tb);
  const T* P_all = reinterpret_cast<const T*>(p.ws_p);

  // ---- device-side argument checks: bad rows get NaN outputs, nothing out of bounds is read
  const int len = p.lengths ? p.lengths[b] : p.L;
  const int srow = p.s0 ? (p.s0_row ? p.s0_row[b] : b) : 0;
  const bool bad = (len < 0 || len > p.L) || (p.s0 && (srow < 0 || srow >= p.n_s0));
  if (bad) {
    const float nan = __builtin_nanf("");
    for (int t = 0; t < p.L; ++t)
      if (wave == 0 && lane < 16 * NW)
        og[((size_t)b * p.L + t) * p.Hv * D + (size_t)h * D + col0 + lane] = from_f<T>(nan);
    if (p.s_final)
      for (int i = tid; i < D * 16 * NW; i += NT)
        p.s_final[(((size_t)b * p.Hv + h) * D + i / (16 * NW)) * D + col0 + i % (16 * NW)] = nan;
    return;
  }

  // ---- state: 8 accumulator tiles of 16 key rows x this wave's 16 columns
  f4 S[8];
  {
    const float* s0 = p.s0 ? p.s0 + ((size_t)srow * p.Hv + h) * D * D : nullptr;
#pragma unroll
    for (int st = 0; st < 8; ++st)
#pragma unroll
      for (int e = 0; e < 4; ++e) S[st][e] = s0 ? s0[(16 * st + 4 * G + e) * D + ncol] : 0.f;
  }

  for (int c = 0; c < p.NC; ++c) {
    const int t0 = c * C;
    const size_t blk = ((size_t)b * p.Hv + h) * p.NC + c;
    __syncthreads();   // the previous chunk is done with LDS
    // -- stage K (both layouts), Q, V slice, Tb, P, scalars
    for (int idx = tid; idx < C * (D / VN); idx += NT) {
      const int row = idx / (D / VN), cv = idx % (D / VN);
      const int t = t0 + row;
      Vec16<T> kv, qv;
      kv.raw = make_uint4(0, 0, 0, 0);
      qv.raw = make_uint4(0, 0, 0, 0);
      if (t < p.L) {
        const size_t off = ((size_t)b * p.L + t) * p.Hk * D + (size_t)kh * D + cv * VN;
        kv.raw = *reinterpret_cast<const uint4*>(kg + off);
        qv.raw = *reinterpret_cast<const uint4*>(qg + off);
      }
      *reinterpret_cast<uint4*>(&sm.k[row * PK + cv * VN]) = kv.raw;
      *reinterpret_cast<uint4*>(&sm.q[row * PK + cv * VN]) = qv.raw;
#pragma unroll
      for (int e = 0; e < VN; ++e) sm.kt[(cv * VN + e) * PT + row] = kv.get(e);
    }
    for (int idx = tid; idx < C * (C / VN); idx += NT) {
      const int row = idx / (C / VN), cv = idx % (C / VN);
      *reinterpret_cast<uint4*>(&sm.tb[row * PT + cv * VN]) =
          *reinterpret_cast<const uint4*>(Tb_all + blk * (C * C) + row * C + cv * VN);
      *reinterpret_cast<uint4*>(&sm.pm[row * PT + cv * VN]) =
          *reinterpret_cast<const uint4*>(P_all + blk * (C * C) + row * C + cv * VN);
    }
    for (int idx = tid; idx < C * (16 * NW / VN); idx += NT) {
      const int row = idx / (16 * NW / VN), cv = idx % (16 * NW / VN);
      const int t = t0 + row;
      uint4 vv = make_uint4(0, 0, 0, 0);
      if (t < p.L)
        vv = *reinterpret_cast<const uint4*>(vg + ((size_t)b * p.L + t) * p.Hv * D + (size_t)h * D + col0 + cv * VN);
      *reinterpret_cast<uint4*>(&sm.v[row * PT + cv * VN]) = vv;
    }
    for (int idx = tid; idx < C; idx += NT)
      *reinterpret_cast<f4*>(&sm.sc[4 * idx]) = *reinterpret_cast<const f4*>(p.ws_scal + blk * (4 * C) + 4 * idx);
    __syncthreads();

    const float* sa = sm.sc;
    const float* scc = sm.sc + C;
    const float* sd = sm.sc + 2 * C;
    const float egC = sm.sc[3 * C];

    // -- state as B operands (4 k blocks of 32 key rows)
    Frag<T> Sf[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) Sf[kb] = acc_frag<T>(S[2 * kb], S[2 * kb + 1], f4_splat(1.f), f4_splat(1.f));

    // -- X = K S and OQ = Q S  (token tiles mt = 0..3)
    f4 X[4], OQ[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      X[mt] = f4_splat(0.f);
      OQ[mt] = f4_splat(0.f);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        mma(X[mt], lds_frag(sm.k, PK, 16 * mt + n16, 32 * kb, G), Sf[kb]);
        mma(OQ[mt], lds_frag(sm.q, PK, 16 * mt + n16, 32 * kb, G), Sf[kb]);
      }
    }
    // -- R = V - diag(a) X (fp32), as B operands over tokens
    f4 R[4], one = f4_splat(1.f);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * mt + 4 * G + e;
        R[mt][e] = to_f(sm.v[t * PT + 16 * wave + n16]) - sa[t] * X[mt][e];
      }
    Frag<T> Rf[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) Rf[kb] = acc_frag<T>(R[2 * kb], R[2 * kb + 1], one, one);

    // -- Delta = Tb R
    f4 Dl[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      Dl[mt] = f4_splat(0.f);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) mma(Dl[mt], lds_frag(sm.tb, PT, 16 * mt + n16, 32 * kb, G), Rf[kb]);
    }
    Frag<T> Df[2], Ddf[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      Df[kb] = acc_frag<T>(Dl[2 * kb], Dl[2 * kb + 1], one, one);
      f4 d0, d1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        d0[e] = sd[32 * kb + 4 * G + e];
        d1[e] = sd[32 * kb + 16 + 4 * G + e];
      }
      Ddf[kb] = acc_frag<T>(Dl[2 * kb], Dl[2 * kb + 1], d0, d1);
    }

    // -- O = diag(c) OQ + P Delta, stored for tokens < L
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f4 O;
#pragma unroll
      for (int e = 0; e < 4; ++e) O[e] = scc[16 * mt + 4 * G + e] * OQ[mt][e];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) mma(O, lds_frag(sm.pm, PT, 16 * mt + n16, 32 * kb, G), Df[kb]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = t0 + 16 * mt + 4 * G + e;
        if (t < p.L) og[((size_t)b * p.L + t) * p.Hv * D + (size_t)h * D + ncol] = from_f<T>(O[e]);
      }
    }

    // -- S <- e^{gamma_63} S + K^T diag(d) Delta
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      S[st] *= egC;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) mma(S[st], lds_frag(sm.kt, PT, 16 * st + n16, 32 * kb, G), Ddf[kb]);
    }
  }

  if (p.s_final) {
    float* sf = p.s_final + ((size_t)b * p.Hv + h) * D * D;
#pragma unroll
    for (int st = 0; st < 8; ++st)
#pragma unroll
      for (int e = 0; e < 4; ++e) sf[(16 * st + 4 * G + e) * D + ncol] = S[st][e];
  }
}

// ====================================================================== launchers
template <typename T, typename TB>
static hipError_t launch_prep_t(const PrepParams& p, hipStream_t s) {
  dim3 grid(p.NC, p.Hk, p.B);
  hipLaunchKernelGGL((gdr_prep<T, TB>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_prep(const PrepParams& p, int qkv_bf16, int beta_bf16, hipStream_t s) {
  if (qkv_bf16) return beta_bf16 ? launch_prep_t<__bf16, __bf16>(p, s) : launch_prep_t<__bf16, float>(p, s);
  return launch_prep_t<float, float>(p, s);
}

hipError_t launch_scan(const ScanParams& p, int qkv_bf16, hipStream_t s) {
  constexpr int NW = 4;
  dim3 grid(D / (16 * NW), p.Hv, p.B);
  if (qkv_bf16)
    hipLaunchKernelGGL((gdr_scan<__bf16, NW>), grid, dim3(64 * NW), 0, s, p);
  else
    hipLaunchKernelGGL((gdr_scan<float, NW>), grid, dim3(64 * NW), 0, s, p);
  return hipGetLastError();
}

}  // namespace gdr
