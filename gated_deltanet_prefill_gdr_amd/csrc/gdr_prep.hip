// Per-chunk preparation for the chunked gated delta rule (gfx950).
//
// One workgroup (4 waves) per (row b, key head kh, chunk c). From the chunk's raw q and k it
// forms, for every value head h served by kh (h = kh*r .. kh*r + r-1):
//   rk_t = (|k_t|^2 + 1e-6)^-1/2,  rq_t = (|q_t|^2 + 1e-6)^-1/2 * 128^-1/2   (model page model.py,
//          function _l2norm, eps inside the rsqrt; q scaled by Dk^-1/2 as in delta_rule_reference)
//   beta'_t, g'_t with the right-pad guard (model.py, _dn_gates: pads neither write nor decay)
//   gamma_t = inclusive cumulative sum of g' within the chunk
//   A[t][i] = beta'_t e^{gamma_t - gamma_i} rk_t rk_i (k_t . k_i)   (i < t)
//   T = (I + A)^-1, Tb = T diag(beta'),  P[t][i] = rq_t rk_i e^{gamma_t - gamma_i} (q_t . k_i)  (i <= t)
// and writes the chunk record (lower-triangle 16x16 tiles of Tb and P, then the per-token scalars
// a = e^gamma rk, c = e^gamma rq, d = rk e^{gamma_63 - gamma} and e^{gamma_63}). The Gram K K^T
// and Q K^T run on MFMA once per key head and serve all r value heads. Exponents are only taken
// of non-positive differences on the kept triangle ("direct" decay from in-chunk differences).
//
// The inverse is blocked: the four 16x16 diagonal blocks by forward substitution (one lane per
// column), then T_IJ = -T_II sum_{M=J}^{I-1} A_IM T_MJ with fp32 MFMA, one wave per block column.
#include "gdr_device.h"

namespace gdr {

template <typename T> struct PrepLayout;
template <> struct PrepLayout<__bf16> { static constexpr int PK = D + 8; };   // 272-byte rows
template <> struct PrepLayout<float> { static constexpr int PK = D + 4; };    // 528-byte rows
constexpr int kFP = C + 4;   // pitch of the fp32 64x64 matrices A and T

template <typename T>
struct PrepSmem {
  static constexpr int PK = PrepLayout<T>::PK;
  union {
    struct { T k[C * PK]; T q[C * PK]; } in;                                   // staging of q, k
    struct { float a[C * kFP]; float t[C * kFP]; float p[C * kFP]; float sc[4 * C]; } out;
  } u;
  float rk[C], rq[C], gam[C], bet[C];
};

template <typename T, typename TB>
__global__ __launch_bounds__(256) void gdr_prep(PrepParams p) {
  __shared__ __attribute__((aligned(16))) PrepSmem<T> sm;
  constexpr int PK = PrepSmem<T>::PK;
  constexpr int VN = Vec16<T>::N;     // elements per 16-byte vector
  constexpr int VPR = D / VN;         // vectors per 128-wide row
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n16 = lane & 15, G = lane >> 4;
  const int c = blockIdx.x, kh = blockIdx.y, b = blockIdx.z;
  const int r = p.Hv / p.Hk;
  const int t0 = c * C;
  int len = p.lengths ? p.lengths[b] : p.L;
  len = len < 0 ? 0 : (len > p.L ? p.L : len);
  const T* qg = reinterpret_cast<const T*>(p.q);
  const T* kg = reinterpret_cast<const T*>(p.k);

  // ---- stage q, k; squared row norms reduced over the VPR lanes that share a row
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

  // ---- lower-triangle tiles of K K^T and Q K^T (10 each); wave w owns tiles w, w+4, w+8
  f4 gacc[3], qacc[3];
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    gacc[s] = f4_splat(0.f);
    qacc[s] = f4_splat(0.f);
    const int ti = wave + 4 * s;
    if (ti < kTiles) {
      const int I = tile_row(ti), J = tile_col(ti);
#pragma unroll
      for (int kb = 0; kb < D / 32; ++kb) {
        const Frag<T> bk = lds_frag(sm.u.in.k, PK, 16 * J + n16, 32 * kb, G);
        mma(gacc[s], lds_frag(sm.u.in.k, PK, 16 * I + n16, 32 * kb, G), bk);
        mma(qacc[s], lds_frag(sm.u.in.q, PK, 16 * I + n16, 32 * kb, G), bk);
      }
    }
  }
  __syncthreads();   // the q/k staging area is reused below

  const TB* betag = reinterpret_cast<const TB*>(p.beta);
  constexpr int kRecBytes = 2 * kFragBlocks * kBlockElems * sizeof(T) + 4 * C * sizeof(float);
  constexpr int kMatVecs = kFragBlocks * kBlockElems / VN;   // 16-byte vectors of Tb (and of P)

  for (int hr = 0; hr < r; ++hr) {
    const int h = kh * r + hr;
    char* rec = reinterpret_cast<char*>(p.ws) + (((size_t)b * p.Hv + h) * p.NC + c) * kRecBytes;

    // -- guarded gates and inclusive cumulative decay (wave 0, lane = token)
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
      sm.u.out.sc[lane] = eg * sm.rk[lane];
      sm.u.out.sc[C + lane] = eg * sm.rq[lane];
      sm.u.out.sc[2 * C + lane] = sm.rk[lane] * expf(gC - x);
      sm.u.out.sc[3 * C + lane] = (lane == 0) ? expf(gC) : 0.f;
    }
    __syncthreads();

    // -- A (strictly lower, fp32) and P (lower incl. diagonal, tile layout), from the Gram tiles
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      const int ti = wave + 4 * s;
      if (ti < kTiles) {
        const int I = tile_row(ti), J = tile_col(ti);
        const int col = 16 * J + n16;
        const float gcol = sm.gam[col], rkcol = sm.rk[col];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = 16 * I + 4 * G + e;
          const float dec = expf(row >= col ? sm.gam[row] - gcol : 0.f);
          sm.u.out.a[row * kFP + col] = (row > col) ? sm.bet[row] * dec * sm.rk[row] * rkcol * gacc[s][e] : 0.f;
          sm.u.out.p[row * kFP + col] = (row >= col) ? sm.rq[row] * rkcol * dec * qacc[s][e] : 0.f;
        }
      }
    }
    __syncthreads();

    // -- diagonal blocks by forward substitution (wave w: block w, lane = column)
    if (lane < 16) {
      const int o = 16 * wave, kcol = lane;
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float s = (i == kcol) ? 1.f : 0.f;
        const float* arow = &sm.u.out.a[(o + i) * kFP + o];
#pragma unroll
        for (int j = 0; j < i; ++j) s -= arow[j] * x[j];
        x[i] = s;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) sm.u.out.t[(o + i) * kFP + o + kcol] = x[i];
    }
    __syncthreads();

    // -- off-diagonal blocks (wave J: block column J)
    if (wave < 3) {
      const int J = wave;
      for (int I = J + 1; I < 4; ++I) {
        f4 X = f4_splat(0.f);
        for (int M = J; M < I; ++M) {
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const float av = sm.u.out.a[(16 * I + n16) * kFP + 16 * M + 4 * G + s];
            const float bv = sm.u.out.t[(16 * M + 4 * G + s) * kFP + 16 * J + n16];
            X = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, X, 0, 0, 0);
          }
        }
        f4 Y = f4_splat(0.f);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const float av = sm.u.out.t[(16 * I + n16) * kFP + 16 * I + 4 * G + s];
          Y = __builtin_amdgcn_mfma_f32_16x16x4f32(av, X[s], Y, 0, 0, 0);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) sm.u.out.t[(16 * I + 4 * G + s) * kFP + 16 * J + n16] = -Y[s];
      }
    }
    __syncthreads();

    // -- the record, in 16-byte stores: Tb (formed here) and P in operand order, then scalars
    for (int v = tid; v < kRecBytes / 16; v += 256) {
      uint4 out;
      if (v < 2 * kMatVecs) {
        const bool is_p = v >= kMatVecs;
        const int s0 = (v - (is_p ? kMatVecs : 0)) * VN;   // first slot of this vector
        const int blk = s0 / kBlockElems, ln = (s0 % kBlockElems) / 8;
        const int row = 16 * block_tile(blk) + (ln & 15), g = ln >> 4, kb = block_kb(blk);
        Vec16<T> pk;
#pragma unroll
        for (int e = 0; e < VN; ++e) {
          const int col = slot_col(kb, g, (s0 + e) % 8);
          float x;
          if (is_p)
            x = col <= row ? sm.u.out.p[row * kFP + col] : 0.f;
          else
            x = col <= row ? sm.u.out.t[row * kFP + col] * sm.bet[col] : 0.f;
          reinterpret_cast<T*>(&pk.raw)[e] = from_f<T>(x);
        }
        out = pk.raw;
      } else {
        out = *reinterpret_cast<const uint4*>(&sm.u.out.sc[(v - 2 * kMatVecs) * 4]);
      }
      *reinterpret_cast<uint4*>(rec + 16 * (size_t)v) = out;
    }
    __syncthreads();   // staging is reused by the next value head
  }
}

hipError_t launch_prep(const PrepParams& p, int qkv_bf16, int beta_bf16, hipStream_t s) {
  dim3 grid(p.NC, p.Hk, p.B);
  if (qkv_bf16) {
    if (beta_bf16)
      hipLaunchKernelGGL((gdr_prep<__bf16, __bf16>), grid, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL((gdr_prep<__bf16, float>), grid, dim3(256), 0, s, p);
  } else {
    hipLaunchKernelGGL((gdr_prep<float, float>), grid, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace gdr
