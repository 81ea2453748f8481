// Per-chunk transform of the chunked gated delta rule (gfx950).
//
// From a chunk's raw k, g and beta (and q for float32) it forms
//   rk_t = (|k_t|^2 + 1e-6)^-1/2,  rq_t = (|q_t|^2 + 1e-6)^-1/2 * 128^-1/2   (model page model.py,
//          function _l2norm, eps inside the rsqrt; q scaled by Dk^-1/2 as in delta_rule_reference)
//   beta'_t, g'_t with the right-pad guard (model.py, _dn_gates: pads neither write nor decay);
//          with the gate prologue fused, beta = sigmoid(b_raw) and g = -exp(A_log) softplus(a_raw +
//          dt_bias) are formed here from the raw projections instead of being read
//   gamma_t = inclusive cumulative sum of g' within the chunk
//   A[t][i] = beta'_t e^{gamma_t - gamma_i} rk_t rk_i (k_t . k_i)   (i < t)
//   T = (I + A)^-1, Tb = T diag(beta'),  P[t][i] = rq_t rk_i e^{gamma_t - gamma_i} (q_t . k_i)  (i <= t)
// and writes the chunk record: Tb (and for float32 P) as MFMA operand blocks (lower triangle
// only), then the per-token scalars a = e^gamma rk, d = rk e^{gamma_63 - gamma}, gamma log2 e and
// rk (float32 also c = e^gamma rq, rq and e^{gamma_63}; bf16 also the chunk's contraction flag).
// Exponents are only taken of non-positive differences on the kept triangle ("direct" decay
// from in-chunk differences), so nothing over- or underflows however strong the decay.
//
// bf16 (gdr_prep_wave): one workgroup of two waves per work item (row b, key head kh, chunk c),
// each wave running the whole transform of one value head of the key head at a time on its own
// (see there). q is not read: the output pass forms the q norms from the Q tile it stages anyway.
// With lengths the items are only the chunks that hold valid tokens (gdr_chunk_list).
//
// float32 (gdr_prep): one workgroup (4 waves) per (row b, value head h, chunk c).
//
// float32 phases (one barrier each; the waves exchange data through LDS only, so the barriers do
// not wait for the global stores of the record; gdr_prep_wave runs the same steps in one wave):
//   1. stage k (and q) rows in LDS, row norms, gates and gamma;
//   2. Gram tiles on MFMA, balanced over the waves: wave w forms its diagonal K K^T tile (3 - w,
//      3 - w) and 2, 2, 1, 1 of the tiles below the diagonal (GramTiles), and (float32) the K Q^T
//      tiles of column w. The K Q^T tile (J, I) is P^T, whose accumulator
//      layout is exactly the operand layout of P, so P goes from registers straight to the record;
//   3. A (fp32) into LDS (float32: over the staging area);
//   4. T of the four 16x16 diagonal blocks by forward substitution, one lane per column, all in
//      registers (one wave per value head), written over A;
//   5. off-diagonal blocks by the 2x2 block rule T_BA = -T_BB A_BA T_AA, first within each
//      32-row half (T_10, T_32), then across the halves, on fp32 MFMA (gdr_prep_wave: on bf16 MFMA
//      with split factors, mma_split), each written over A;
//   6. Tb = T diag(beta') gathered into operand order.
#include <algorithm>

#include "gdr_device.h"

namespace gdr {

template <typename T> struct PrepLayout;
template <> struct PrepLayout<__bf16> { static constexpr int PK = D + 8; };   // 272-byte rows
template <> struct PrepLayout<float> { static constexpr int PK = D + 4; };    // 528-byte rows

// The fp32 64x64 matrices A and T live in LDS as their ten lower 16x16 blocks (I >= J), block (I, J)
// at kBlk (I (I + 1) / 2 + J) floats. In a block, row r = 4a + b, column c sits at
// moff(r, c) = 64 a + 16 ((a + b) & 3) + 4 ((c >> 2) ^ a) + (c & 3): the 16 rows of one operand read
// (four consecutive columns each) and the rows 4G + s of one accumulator-layout access each hit
// the 64 banks once. kBlk = 260 rather than 256 puts the four diagonal blocks, which the forward
// substitution reads at one address per block, in different banks.
constexpr int kBlk = 260;
constexpr int kMatFloats = 10 * kBlk;
__device__ __forceinline__ int moff(int r, int c) {
  const int a = r >> 2, b = r & 3;
  return 64 * a + 16 * ((a + b) & 3) + 4 * ((c >> 2) ^ a) + (c & 3);
}

template <typename T>
struct PrepSmem {
  static constexpr int PK = PrepLayout<T>::PK;
  union {
    struct { T k[C * PK]; T q[C * PK]; } in;   // phases 1-2
    float a[kMatFloats];   // phases 3-6: A, then T over it
  } u;
  float rk[C], rq[C], gam[C], bet[C];
};

// fp32 16x16 tile product with the k index of step s, lane group G standing for 4G + s: the A
// operand av is row n16 of the left tile (tile_row: one 16-byte LDS read per lane), the B operand
// the accumulator layout of the right factor (element s of lane (n, G) is row 4G + s).
__device__ __forceinline__ void mma_acc(f4& acc, const f4& av, const f4& b) {
#pragma unroll
  for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[s], b[s], acc, 0, 0, 0);
}
// The A operand of such a product: row n16, columns 4G .. 4G + 3 of an LDS block.
__device__ __forceinline__ f4 tile_row(const float* a_tile, int n16, int G) {
  return *reinterpret_cast<const f4*>(a_tile + moff(n16, 4 * G));
}
__device__ __forceinline__ void mma_lds_acc(f4& acc, const float* a_tile, int n16, int G, const f4& b) {
  mma_acc(acc, tile_row(a_tile, n16, G), b);
}
// The right factor in accumulator layout, read from an LDS block.
__device__ __forceinline__ f4 tile_acc(const float* tile, int n16, int G) {
  f4 x;
#pragma unroll
  for (int s = 0; s < 4; ++s) x[s] = tile[moff(4 * G + s, n16)];
  return x;
}
__device__ __forceinline__ void store_acc(float* tile, int n16, int G, const f4& x) {
#pragma unroll
  for (int s = 0; s < 4; ++s) tile[moff(4 * G + s, n16)] = x[s];
}
__device__ __forceinline__ const float* blk(const float* m, int I, int J) { return m + kBlk * (I * (I + 1) / 2 + J); }
__device__ __forceinline__ float* blk(float* m, int I, int J) { return m + kBlk * (I * (I + 1) / 2 + J); }

// The same products on bf16 MFMA (bf16 sequences): a 16x16x16 bf16 product takes, per lane, the four
// k values 4G .. 4G + 3 that mma_acc's four fp32 steps take one at a time, so the operands keep their
// layouts. Each fp32 factor is split into bf16 hi + lo: hi is x with its low 16 bits cleared (exact as
// a float, and its bf16 pattern is the upper half of x), lo = x - hi (exact) rounded to bf16. Then
// Ah Bh + Ah Bl + Al Bh drops only Al Bl and lo's rounding (about 2^-15 of the product), far below the
// bf16 rounding the record applies to T afterwards; the fp32 products run at 1/16 of the bf16 rate.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
struct Split4 {
  s16x4 hi, lo;
};
__device__ __forceinline__ Split4 split4(const f4& x) {
  uint32_t u[4];
  float l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float xe = x[e];   // a scalar copy: bit_cast of the vector element x[e] itself compiled to element 0
    u[e] = __builtin_bit_cast(uint32_t, xe);
    l[e] = x[e] - __builtin_bit_cast(float, u[e] & 0xFFFF0000u);
  }
  Split4 r;
  // upper halves of u[0], u[1] (and u[2], u[3]) as one word each: bytes 2, 3 of the low operand, then
  // bytes 2, 3 of the high one
  r.hi = __builtin_bit_cast(s16x4, u32x2{__builtin_amdgcn_perm(u[1], u[0], 0x07060302u),
                                         __builtin_amdgcn_perm(u[3], u[2], 0x07060302u)});
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 l01 = __builtin_convertvector(f2{l[0], l[1]}, bf16x2), l23 = __builtin_convertvector(f2{l[2], l[3]}, bf16x2);
  r.lo = __builtin_bit_cast(s16x4, u32x2{__builtin_bit_cast(uint32_t, l01), __builtin_bit_cast(uint32_t, l23)});
  return r;
}
__device__ __forceinline__ void mma_split(f4& acc, const Split4& a, const Split4& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.hi, b.hi, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.hi, b.lo, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.lo, b.hi, acc, 0, 0, 0);
}

// The lower 16x16 tiles (I, J) of K K^T that wave W forms and scales into A: its diagonal tile
// (3 - W, 3 - W) first (the row norms come from its diagonal), then 2, 2, 1, 1 of the six tiles
// below the diagonal, so that the Gram and A work is spread evenly over the four waves.
template <int W> struct GramTiles;
template <> struct GramTiles<0> { static constexpr int n = 3, I[3] = {3, 3, 3}, J[3] = {3, 0, 1}; };
template <> struct GramTiles<1> { static constexpr int n = 3, I[3] = {2, 3, 2}, J[3] = {2, 2, 0}; };
template <> struct GramTiles<2> { static constexpr int n = 2, I[3] = {1, 2, 0}, J[3] = {1, 1, 0}; };
template <> struct GramTiles<3> { static constexpr int n = 2, I[3] = {0, 1, 0}, J[3] = {0, 0, 0}; };

// Phase 2 of wave W (float32): the Gram tiles of GramTiles<W>, gk[t][e] = (K K^T)[16 I_t + 4G + e]
// [16 J_t + n16], and P into the record (bf16 records carry no P: the output pass forms it from the
// Q and K tiles it stages anyway). Kept a template on W so that every tile choice is fixed at
// compile time.
template <int W, typename T, int PK>
__device__ __forceinline__ void gram_phase(const T* ks, const T* qs, const float* gam2, const float* rk,
                                           const float* rq, int n16, int G, int lane, unsigned char* pbase,
                                           f4 (&gk)[3]) {
  using TL = GramTiles<W>;
  constexpr bool kP = sizeof(T) == 4;
  constexpr int Iq = kP ? W : -1;
  f4 gq[4];
#pragma unroll
  for (int J = 0; J < 4; ++J) gq[J] = f4_splat(0.f);
#pragma unroll
  for (int t = 0; t < 3; ++t) gk[t] = f4_splat(0.f);
#pragma unroll
  for (int kb = 0; kb < D / 32; ++kb) {
    const Frag<T> bq = lds_frag(qs, PK, 16 * (kP ? Iq : 0) + n16, 32 * kb, G);
#pragma unroll
    for (int t = 0; t < TL::n; ++t)
      mma(gk[t], lds_frag(ks, PK, 16 * TL::I[t] + n16, 32 * kb, G), lds_frag(ks, PK, 16 * TL::J[t] + n16, 32 * kb, G));
#pragma unroll
    for (int J = 0; J <= Iq; ++J)   // (K Q^T)[16 J + 4G + e][16 Iq + n16] = P^T
      mma(gq[J], lds_frag(ks, PK, 16 * J + n16, 32 * kb, G), bq);
  }
  if constexpr (!kP) return;
  // P[t][i], t = 16 Iq + n16, i = 16 J + 4G + e; each lane writes its eight slots of block (Iq, kb)
  const int t = 16 * Iq + n16;
  const float gt = gam2[t], rqt = rq[t];
  f4 pv[4];
#pragma unroll
  for (int J = 0; J < 4; ++J) {
    pv[J] = f4_splat(0.f);
    if (J > Iq) continue;
    const f4 gi = *reinterpret_cast<const f4*>(gam2 + 16 * J + 4 * G);
    const f4 ri = *reinterpret_cast<const f4*>(rk + 16 * J + 4 * G);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 16 * J + 4 * G + e;
      const float x = rqt * ri[e] * __builtin_amdgcn_exp2f(fminf(gt - gi[e], 0.f)) * gq[J][e];
      pv[J][e] = (i <= t) ? x : 0.f;
    }
  }
#pragma unroll
  for (int kb = 0; kb <= (Iq >> 1); ++kb) {
    const Frag<T> f = acc_frag<T>(pv[2 * kb], pv[2 * kb + 1], f4_splat(1.f), f4_splat(1.f));
    unsigned char* dst = pbase + (size_t)frag_block(Iq, kb) * kBlockElems * sizeof(T) + (size_t)lane * 8 * sizeof(T);
    if constexpr (sizeof(T) == 2) {
      *reinterpret_cast<bf16x8*>(dst) = f.v;
    } else {
      *reinterpret_cast<f4*>(dst) = f4{f.v[0], f.v[1], f.v[2], f.v[3]};
      *reinterpret_cast<f4*>(dst + 16) = f4{f.v[4], f.v[5], f.v[6], f.v[7]};
    }
  }
}

// Phase 3 of wave W: its K K^T tiles (GramTiles<W>) scaled into A.
template <int W>
__device__ __forceinline__ void a_phase(float* A, const float* gam2, const float* rk, const float* bet, int n16, int G,
                                        const f4 (&gk)[3]) {
  using TL = GramTiles<W>;
#pragma unroll
  for (int t = 0; t < TL::n; ++t) {
    const int I = TL::I[t], J = TL::J[t];
    const f4 gr = *reinterpret_cast<const f4*>(gam2 + 16 * I + 4 * G);
    const f4 rr = *reinterpret_cast<const f4*>(rk + 16 * I + 4 * G);
    const f4 br = *reinterpret_cast<const f4*>(bet + 16 * I + 4 * G);
    const int col = 16 * J + n16;
    const float gc = gam2[col], rc = rk[col];
    float* ab = blk(A, I, J);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * I + 4 * G + e;
      const float x = br[e] * __builtin_amdgcn_exp2f(fminf(gr[e] - gc, 0.f)) * rr[e] * rc * gk[t][e];
      ab[moff(4 * G + e, n16)] = row > col ? x : 0.f;
    }
  }
}

// Phases 3-6 for nh = 1 or 2 value heads at once (the second head's work interleaves with the
// first's, so the pair costs about the latency of one): A of head j from the Gram tiles gk of this
// wave (GramTiles) into M0 or M1 (kMatFloats floats each), the blocked inverse T = (I + A)^-1 in
// place over A, and Tb into the record rec0 or rec1. In place is safe because every block of A is read for the last
// time before the barrier that precedes its overwrite (A_21 and A_31, still needed after the blocks
// of the same phase are written, are read into registers one phase early). While waves 0 and 1
// solve the diagonal blocks, waves 2 and 3 call idle(j) for head j = wave - 2 < nh. Four barriers;
// on return every wave may still be reading M (phase 6), so M may be rewritten only after a barrier.
// (Heads are passed as pointer pairs: a local array of LDS addresses would become a static
// initializer, which the device compiler rejects.)
template <typename T, typename Idle>
__device__ __forceinline__ void inverse_to_records(float* M0, float* M1, const float* gam0, const float* gam1,
                                                   const float* rk, const float* bet0, const float* bet1,
                                                   const f4 (&gk)[3], int nh, int wave, int n16, int G, int lane,
                                                   unsigned char* rec0, unsigned char* rec1, Idle&& idle) {
  auto M = [&](int j) { return j ? M1 : M0; };
  auto gam = [&](int j) { return j ? gam1 : gam0; };
  auto bet = [&](int j) { return j ? bet1 : bet0; };
  // ---- 3. A, strictly lower, fp32
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    if (j >= nh) break;
    switch (wave) {
      case 0: a_phase<0>(M(j), gam(j), rk, bet(j), n16, G, gk); break;
      case 1: a_phase<1>(M(j), gam(j), rk, bet(j), n16, G, gk); break;
      case 2: a_phase<2>(M(j), gam(j), rk, bet(j), n16, G, gk); break;
      default: a_phase<3>(M(j), gam(j), rk, bet(j), n16, G, gk); break;
    }
  }
  lds_barrier();

  // ---- 4. diagonal blocks of head `wave`: lane 16 w' + j solves column j of block w', column k of
  //         the block read from LDS at step k (one address per block, broadcast over its 16
  //         lanes); the column is written over the block once all of its reads are done
  if (wave < nh) {
    float* ablk = blk(M(wave), G, G);
    const int j = n16;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = (i == j) ? 1.f : 0.f;
#pragma unroll
    for (int k = 0; k < 15; ++k) {
#pragma unroll
      for (int i = k + 1; i < 16; ++i) x[i] -= ablk[moff(i, k)] * x[k];
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) ablk[moff(i, j)] = x[i];
  } else if (wave >= 2 && wave - 2 < nh) {
    idle(wave - 2);
  }
  lds_barrier();

  // ---- 5. off-diagonal blocks. Within each 32-row half: T_10 = -T_11 A_10 T_00 (wave 0),
  //         T_32 = -T_33 A_32 T_22 (wave 1); waves 2, 3 meanwhile form A_20 T_00, A_30 T_00.
  //         Across the halves (T_IJ for I in {2,3}, J in {0,1}), with Z = A_[23][01] T_[01][01]:
  //         T_2J = -T_22 Z_2J, T_3J = -(T_32 Z_2J + T_33 Z_3J); wave 2: T_20, wave 3: T_30,
  //         wave 0: T_21, wave 1: T_31.
  const bool row3 = (wave & 1) != 0;   // waves 1, 3 produce row 3 of the second step
  f4 pre0[2], pre1[2], a21[2], a31[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    pre0[j] = pre1[j] = a21[j] = a31[j] = f4_splat(0.f);
    if (j >= nh) break;
    float* Mj = M(j);
    a21[j] = tile_row(blk(Mj, 2, 1), n16, G);            // overwritten in the second step
    if (row3) a31[j] = tile_row(blk(Mj, 3, 1), n16, G);
    if (wave < 2) {
      const int I = 2 * wave + 1, J = 2 * wave;   // (1, 0) or (3, 2)
      f4 x = f4_splat(0.f);
      mma_lds_acc(x, blk(Mj, I, J), n16, G, tile_acc(blk(Mj, J, J), n16, G));
      f4 y = f4_splat(0.f);
      mma_lds_acc(y, blk(Mj, I, I), n16, G, x);
      store_acc(blk(Mj, I, J), n16, G, -y);
    } else {
      const f4 t00 = tile_acc(blk(Mj, 0, 0), n16, G);
      mma_lds_acc(pre0[j], blk(Mj, 2, 0), n16, G, t00);            // A_20 T_00
      if (wave == 3) mma_lds_acc(pre1[j], blk(Mj, 3, 0), n16, G, t00);   // A_30 T_00
    }
  }
  lds_barrier();
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    if (j >= nh) break;
    float* Mj = M(j);
    const int J = (wave >= 2) ? 0 : 1;
    const f4 tj1 = tile_acc(blk(Mj, 1, J), n16, G);   // T_10 (J = 0) or T_11 (J = 1)
    f4 z2 = pre0[j];                                   // Z_2J = A_20 T_0J + A_21 T_1J (T_01 = 0)
    mma_acc(z2, a21[j], tj1);
    f4 out = f4_splat(0.f);
    if (!row3) {
      mma_lds_acc(out, blk(Mj, 2, 2), n16, G, z2);
      store_acc(blk(Mj, 2, J), n16, G, -out);
    } else {
      f4 z3 = pre1[j];                                 // Z_3J = A_30 T_0J + A_31 T_1J
      mma_acc(z3, a31[j], tj1);
      mma_lds_acc(out, blk(Mj, 3, 2), n16, G, z2);
      mma_lds_acc(out, blk(Mj, 3, 3), n16, G, z3);
      store_acc(blk(Mj, 3, J), n16, G, -out);
    }
  }
  lds_barrier();

  // ---- 6. Tb = T diag(beta') in operand order (zero above the diagonal): the nh x 6 blocks
  //         numbered 6 j + bk, wave w writing numbers w, w + 4, w + 8; lane (m, g) of block
  //         (tile I, kb) holds row 16 I + m, columns 32 kb + 4g + {0..3} and 32 kb + 16 + 4g + {0..3}
#pragma unroll
  for (int i3 = 0; i3 < 3; ++i3) {
    const int nb = wave + 4 * i3, j = nb >= kFragBlocks ? 1 : 0, bk = nb - kFragBlocks * j;
    if (j < nh) {
      const int I = block_tile(bk), kb = block_kb(bk);
      const int row = 16 * I + n16, c0 = 32 * kb + 4 * G;
      // columns c0.. lie in block (I, 2 kb), columns c0 + 16.. in block (I, 2 kb + 1), which is
      // above the diagonal (not stored, all zero in T) when 2 kb + 1 > I
      const f4 t_lo = tile_row(blk(M(j), I, 2 * kb), n16, G);
      const f4 t_hi = 2 * kb + 1 <= I ? tile_row(blk(M(j), I, 2 * kb + 1), n16, G) : f4_splat(0.f);
      const f4 b_lo = *reinterpret_cast<const f4*>(&bet(j)[c0]);
      const f4 b_hi = *reinterpret_cast<const f4*>(&bet(j)[c0 + 16]);
      f4 lo, hi;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        lo[e] = (c0 + e <= row) ? t_lo[e] * b_lo[e] : 0.f;
        hi[e] = (c0 + 16 + e <= row) ? t_hi[e] * b_hi[e] : 0.f;
      }
      const Frag<T> f = acc_frag<T>(lo, hi, f4_splat(1.f), f4_splat(1.f));
      unsigned char* dst = (j ? rec1 : rec0) + (size_t)bk * kBlockElems * sizeof(T) + (size_t)lane * 8 * sizeof(T);
      if constexpr (sizeof(T) == 2) {
        *reinterpret_cast<bf16x8*>(dst) = f.v;
      } else {
        *reinterpret_cast<f4*>(dst) = f4{f.v[0], f.v[1], f.v[2], f.v[3]};
        *reinterpret_cast<f4*>(dst + 16) = f4{f.v[4], f.v[5], f.v[6], f.v[7]};
      }
    }
  }
}

template <typename T, typename TB>
__global__ __launch_bounds__(256, 2) void gdr_prep(PrepParams p) {
  __shared__ __attribute__((aligned(16))) PrepSmem<T> sm;
  constexpr int PK = PrepSmem<T>::PK;
  constexpr int VN = Vec16<T>::N;     // elements per 16-byte vector
  constexpr int VPR = D / VN;         // vectors per 128-wide row
  constexpr int NV = (C * VPR) / 256; // 16-byte vectors of q (and of k) per thread
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15, G = lane >> 4;
  // consecutive logical workgroups: the value heads of one key head, then the key heads, then
  // the chunks; kept on one XCD so that the q, k rows they share are read once from HBM
  const int r = p.Hv / p.Hk;
  const int lam = xcd_remap(blockIdx.x, gridDim.x);
  const int hr = lam % r, kh = (lam / r) % p.Hk, c = (lam / p.Hv) % p.NC, b = lam / (p.Hv * p.NC);
  const int h = kh * r + hr;
  const int t0 = c * C;
  int len = p.lengths ? p.lengths[b] : p.L;
  len = len < 0 ? 0 : (len > p.L ? p.L : len);
  constexpr int kMatBytes = kFragBlocks * kBlockElems * (int)sizeof(T);   // Tb (or P) part of a record
  constexpr int kNumMat = sizeof(T) == 4 ? 2 : 1;                         // Tb, and P for float32
  constexpr int kRecBytes = kNumMat * kMatBytes + kScalarBytes;
  unsigned char* rec = reinterpret_cast<unsigned char*>(p.ws) + (((size_t)b * p.Hv + h) * p.NC + c) * kRecBytes;
  constexpr float kLog2e = 1.4426950408889634f;

  // ---- 1. stage q, k (range-checked loads: rows past L read as zeros, all issued at once);
  //         squared row norms over the VPR lanes that share a row; gates and gamma (wave 0)
  {
    const uint32_t row_bytes = (uint32_t)p.Hk * D * sizeof(T);
    const size_t base = (size_t)b * p.L * p.Hk * D;
    const __amdgpu_buffer_rsrc_t rsk = make_rsrc(reinterpret_cast<const T*>(p.k) + base, (uint32_t)p.L * row_bytes);
    const __amdgpu_buffer_rsrc_t rsq = make_rsrc(reinterpret_cast<const T*>(p.q) + base, (uint32_t)p.L * row_bytes);
    uint4 kv[NV], qv[NV];
#pragma unroll
    for (int m = 0; m < NV; ++m) {
      const int idx = tid + 256 * m, row = idx / VPR, cv = idx % VPR;
      const uint32_t off = (uint32_t)(t0 + row) * row_bytes + (uint32_t)(kh * D + cv * VN) * sizeof(T);
      kv[m] = buf_load16(rsk, off);
      qv[m] = buf_load16(rsq, off);
    }
    float gv = 0.f, bv = 0.f;
    if (wave == 0) {
      const int t = t0 + lane;
      const size_t off = ((size_t)b * p.L + t) * p.Hv + h;
      if (t < len) {
        if (p.b_raw) {   // fused gate prologue (model.py, _dn_gates)
          const float x = to_f(reinterpret_cast<const TB*>(p.a_raw)[off]) + p.dt_bias[h];
          const float sp = fmaxf(x, 0.f) + log1pf(__expf(-fabsf(x)));   // softplus without overflow
          gv = -__expf(p.A_log[h]) * sp;
          bv = __builtin_amdgcn_rcpf(1.0f + __expf(-to_f(reinterpret_cast<const TB*>(p.b_raw)[off])));
        } else {
          gv = p.g[off];
          bv = to_f(reinterpret_cast<const TB*>(p.beta)[off]);
        }
      }
    }
#pragma unroll
    for (int m = 0; m < NV; ++m) {
      const int idx = tid + 256 * m, row = idx / VPR, cv = idx % VPR;
      *reinterpret_cast<uint4*>(&sm.u.in.k[row * PK + cv * VN]) = kv[m];
      *reinterpret_cast<uint4*>(&sm.u.in.q[row * PK + cv * VN]) = qv[m];
      Vec16<T> kx, qx;
      kx.raw = kv[m];
      qx.raw = qv[m];
      float sk = 0.f, sq = 0.f;
#pragma unroll
      for (int e = 0; e < VN; ++e) {
        const float x = to_f(kx.get(e)), y = to_f(qx.get(e));
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
    if (wave == 0) {
      float x = gv;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off);
        if (lane >= off) x += y;
      }
      sm.gam[lane] = x * kLog2e;   // gamma in base 2: e^{u - v} = 2^{(u - v) log2 e}
      sm.bet[lane] = bv;
    }
  }
  lds_barrier();

  // ---- 2. Gram tiles: K K^T tiles GramTiles<wave>, K Q^T column wave (P^T); P into the record
  //         straight from the accumulators; the scalars (wave 0)
  f4 gk[3];
  {
    unsigned char* pbase = rec + kMatBytes;
    switch (wave) {
      case 0: gram_phase<0, T, PK>(sm.u.in.k, sm.u.in.q, sm.gam, sm.rk, sm.rq, n16, G, lane, pbase, gk); break;
      case 1: gram_phase<1, T, PK>(sm.u.in.k, sm.u.in.q, sm.gam, sm.rk, sm.rq, n16, G, lane, pbase, gk); break;
      case 2: gram_phase<2, T, PK>(sm.u.in.k, sm.u.in.q, sm.gam, sm.rk, sm.rq, n16, G, lane, pbase, gk); break;
      default: gram_phase<3, T, PK>(sm.u.in.k, sm.u.in.q, sm.gam, sm.rk, sm.rq, n16, G, lane, pbase, gk); break;
    }
    if (wave == 0) {
      const float g2 = sm.gam[lane], g2C = sm.gam[C - 1];
      const float eg = __builtin_amdgcn_exp2f(g2);
      const float rkl = sm.rk[lane], rql = sm.rq[lane];
      float* sc = reinterpret_cast<float*>(rec + kNumMat * kMatBytes);
      sc[kScA * C + lane] = eg * rkl;
      sc[kScC * C + lane] = eg * rql;
      sc[kScD * C + lane] = rkl * __builtin_amdgcn_exp2f(fminf(g2C - g2, 0.f));
      sc[kScEgC * C + lane] = (lane == 0) ? __builtin_amdgcn_exp2f(g2C) : 0.f;
      sc[kScGam2 * C + lane] = g2;   // what the output pass needs to form P
      sc[kScRk * C + lane] = rkl;
      sc[kScRq * C + lane] = rql;
      sc[7 * C + lane] = 0.f;
    }
  }
  lds_barrier();   // the staging area becomes A, then T

  inverse_to_records<T>(sm.u.a, sm.u.a, sm.gam, sm.gam, sm.rk, sm.bet, sm.bet, gk, 1, wave, n16, G, lane, rec, rec,
                        [](int) {});
}

// ====================================================================== bf16
// Gates of value head hr of an item's key head at this lane's token, in two steps so that the loads
// of the next item stay in flight while the current one computes: gates_issue loads the raw words
// (range-checked: tokens past L read zeros, and nothing waits on them), gates_finish applies the
// right-pad guard and, with the fused gate prologue, forms beta = sigmoid(b_raw) and
// g = -exp(A_log) softplus(a_raw + dt_bias) (model.py, _dn_gates).
struct GateRaw {
  uint32_t x0, x1;   // g or a_raw, beta or b_raw (raw bits)
  float dt_bias, A_log;   // with the fused prologue: the head's parameters
  int len, h, t;
};
template <typename TB>
__device__ __forceinline__ GateRaw gates_issue(const PrepParams& p, int b, int kh, int c, int hr, int lane) {
  GateRaw gr;
  gr.h = kh * (p.Hv / p.Hk) + hr;
  gr.t = c * C + lane;
  gr.len = p.lengths ? p.lengths[b] : p.L;
  const size_t row0 = (size_t)b * p.L * p.Hv;
  const uint32_t n = (uint32_t)p.L * p.Hv;   // elements of one batch row
  const uint32_t e = (uint32_t)gr.t * p.Hv + gr.h;
  const void* p0 = p.b_raw ? p.a_raw : static_cast<const void*>(p.g);
  const void* p1 = p.b_raw ? p.b_raw : p.beta;
  const bool w0 = p.b_raw != nullptr && sizeof(TB) == 2;   // element width 2 for raw projections in bf16
  if (p.b_raw) {
    gr.dt_bias = p.dt_bias[gr.h];
    gr.A_log = p.A_log[gr.h];
  }
  if (w0) {
    gr.x0 = (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(make_rsrc(static_cast<const TB*>(p0) + row0, 2 * n), 2 * e, 0, 0);
  } else {
    gr.x0 = __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(static_cast<const float*>(p0) + row0, 4 * n), 4 * e, 0, 0);
  }
  if constexpr (sizeof(TB) == 2)
    gr.x1 = (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(make_rsrc(static_cast<const TB*>(p1) + row0, 2 * n), 2 * e, 0, 0);
  else
    gr.x1 = __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(static_cast<const float*>(p1) + row0, 4 * n), 4 * e, 0, 0);
  return gr;
}
template <typename TB>
__device__ __forceinline__ void gates_finish(const PrepParams& p, const GateRaw& gr, float& gv, float& bv) {
  const int len = gr.len < 0 ? 0 : (gr.len > p.L ? p.L : gr.len);
  auto as_f = [](uint32_t x, bool half) {
    return half ? __builtin_bit_cast(float, x << 16) : __builtin_bit_cast(float, x);   // bf16 -> fp32 is a shift
  };
  const bool half1 = sizeof(TB) == 2;
  const bool half0 = p.b_raw != nullptr && half1;
  const float x0 = as_f(gr.x0, half0), x1 = as_f(gr.x1, half1);
  if (p.b_raw) {
    const float x = x0 + gr.dt_bias;
    const float sp = fmaxf(x, 0.f) + log1pf(__expf(-fabsf(x)));   // softplus without overflow
    gv = -__expf(gr.A_log) * sp;
    bv = __builtin_amdgcn_rcpf(1.0f + __expf(-x1));
  } else {
    gv = x0;
    bv = x1;
  }
  if (gr.t >= len) gv = bv = 0.f;
}

// Inclusive cumulative sum of the gates over the wave's 64 lanes (tokens), in base 2, into LDS.
__device__ __forceinline__ void store_gates(float* gam, float* bet, float gv, float bv, int lane) {
  float x = gv;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  gam[lane] = x * 1.4426950408889634f;   // e^{u - v} = 2^{(u - v) log2 e}
  bet[lane] = bv;
}

// The chunks of a right-padded batch that hold valid tokens, row-major: list[0] = their count U,
// list[1 + u] = b NC + c. Rows whose length is out of range count all their chunks (they are
// computed in full; the output pass turns them into NaN). One workgroup: rows in blocks of 256,
// each with a workgroup-wide inclusive prefix sum of the rows' chunk counts.
__device__ __forceinline__ int row_chunks(const int32_t* lengths, int b, int L, int NC) {
  const int len = lengths[b];
  return (len < 0 || len > L) ? NC : (len + C - 1) / C;
}
__global__ __launch_bounds__(256) void gdr_chunk_list(const int32_t* lengths, int B, int L, int NC, int32_t* list) {
  __shared__ int sc[256];
  const int tid = threadIdx.x;
  int base = 0, nc_first = 0;   // this thread's row of the first block (all rows when B <= 256)
  for (int b0 = 0; b0 < B; b0 += 256) {
    const int b = b0 + tid;
    const int nc = b < B ? row_chunks(lengths, b, L, NC) : 0;
    if (b0 == 0) nc_first = nc;
    sc[tid] = nc;
    __syncthreads();
    for (int d = 1; d < 256; d <<= 1) {
      const int y = tid >= d ? sc[tid - d] : 0;
      __syncthreads();
      sc[tid] += y;
      __syncthreads();
    }
    const int start = base + sc[tid] - nc;
    for (int c = 0; c < nc; ++c) list[1 + start + c] = b * NC + c;
    base += sc[255];
    __syncthreads();
  }
  if (tid == 0) list[0] = base;

  // The rows by number of chunks, longest first, after the list's B NC entries: a counting sort on
  // key 255 - min(chunks, 255) (so that longer rows come first). Equal keys land in the order of the
  // LDS atomics, which decides only which workgroup of the output pass takes a row.
  int32_t* order = list + 1 + (size_t)B * NC;
  auto key = [&](int b) { return 255 - min(b < 256 ? nc_first : row_chunks(lengths, b, L, NC), 255); };
  sc[tid] = 0;
  __syncthreads();
  for (int b = tid; b < B; b += 256) atomicAdd(&sc[key(b)], 1);
  __syncthreads();
  const int cnt = sc[tid];
  __syncthreads();
  for (int d = 1; d < 256; d <<= 1) {   // inclusive prefix sum of the counts
    const int y = tid >= d ? sc[tid - d] : 0;
    __syncthreads();
    sc[tid] += y;
    __syncthreads();
  }
  sc[tid] -= cnt;   // exclusive: the first position of key tid
  __syncthreads();
  for (int b = tid; b < B; b += 256) order[atomicAdd(&sc[key(b)], 1)] = b;
}

// ---- bf16 prep, one wave per value head (gdr_prep_wave)
// One workgroup of kPrepWaves waves per work item (row b, key head kh, chunk c). The waves copy the
// item's K tile HBM -> LDS by DMA (half of the rows each) and meet once; then each wave forms all ten
// lower tiles of the Gram K K^T (bf16 MFMA; rk from their diagonal) and runs, for the value heads
// kh r + j with j = wave, wave + kPrepWaves, ... on its own, the steps of the float32 kernel above in
// sequence: gates and gamma, A, the blocked inverse in its own LDS matrix, and the record. A wave's
// LDS accesses complete in order, so no other barrier is needed; the latency of one wave's steps is
// hidden by the other workgroups on the compute unit rather than split over four waves with a
// barrier between every two steps. With at most kPrepWaves value heads per key head (kOne), each wave
// has at most one head: the waves meet once more after the Gram, the matrices are then written over
// the K tile (22 KiB of LDS per workgroup instead of 38), and the forward substitution is kept from
// loading all of its block ahead, so that three waves fit on a SIMD (six workgroups per CU) instead
// of two.
constexpr int kPrepWaves = 2;
template <bool kOne> struct PrepWaveSmem {
  static constexpr int kKBytes = C * 256, kMBytes = kPrepWaves * kMatFloats * 4;
  // the K tile (rows swizzled, swz) and the waves' matrices (A, then T over it), the latter over the
  // former with kOne
  unsigned char buf[kOne ? (kKBytes > kMBytes ? kKBytes : kMBytes) : kKBytes + kMBytes];
  float rk[kPrepWaves][C], gam[kPrepWaves][C], bet[kPrepWaves][C];
  __device__ unsigned char* k() { return buf; }
  __device__ float* m(int w) { return reinterpret_cast<float*>(buf + (kOne ? 0 : kKBytes)) + w * kMatFloats; }
};

// The ten lower Gram tiles in order t = I (I + 1) / 2 + J (I >= J): tile_i(t), tile_j(t).
__device__ __forceinline__ constexpr int tile_i(int t) { return t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3; }
__device__ __forceinline__ constexpr int tile_j(int t) { return t - tile_i(t) * (tile_i(t) + 1) / 2; }

// Orders this wave's LDS accesses around the statement for the compiler (the hardware keeps a wave's
// LDS accesses in order).
__device__ __forceinline__ void wave_lds_fence() { asm volatile("" ::: "memory"); }

template <typename TB, bool kList, bool kOne>
__global__ __launch_bounds__(64 * kPrepWaves, kOne ? 3 : 2) void gdr_prep_wave(PrepParams p) {
  __shared__ __attribute__((aligned(16))) PrepWaveSmem<kOne> sm;
  constexpr int kRecBytes = kFragBlocks * kBlockElems * 2 + kScalarBytes;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15, G = lane >> 4;
  const int r = p.Hv / p.Hk;
  // work item it: key head fastest (with lengths: kh + Hk u over the chunk list, else kh + Hk (b + B c))
  const int it = blockIdx.x;
  const int kh = it % p.Hk;
  int b, c;
  if constexpr (kList) {
    if (it >= p.chunk_list[0] * p.Hk) return;   // uniform: past the chunks that hold valid tokens
    const int e = p.chunk_list[1 + it / p.Hk];
    b = e / p.NC;
    c = e - b * p.NC;
  } else {
    b = (it / p.Hk) % p.B;
    c = it / (p.Hk * p.B);
  }

  // ---- K tile: rows 32 wave .. 32 wave + 31, eight DMA loads of four rows (rows past L read zeros)
  {
    const uint32_t row_bytes = (uint32_t)p.Hk * D * 2;
    const i32x4 rsk = rsrc_words(reinterpret_cast<const __bf16*>(p.k) + (size_t)b * p.L * p.Hk * D, (uint32_t)p.L * row_bytes);
    constexpr int kRowsPerWave = C / kPrepWaves;
#pragma unroll
    for (int m = 0; m < kRowsPerWave / 4; ++m) {
      const int row = kRowsPerWave * wave + 4 * m + (lane >> 4), pos = lane & 15;
      dma16(rsk, (uint32_t)(c * C + row) * row_bytes + (uint32_t)kh * D * 2 + 16 * (pos ^ swz_f(row)),
            sm.k() + (kRowsPerWave * wave + 4 * m) * 256);
    }
  }
  // the first head's gates, in flight with the tile
  GateRaw graw{};
  if (wave < r) graw = gates_issue<TB>(p, b, kh, c, wave, lane);
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0), as a builtin so that the compiler knows its own loads are done
  lds_barrier();

  // ---- Gram: gk[t][e] = (K K^T)[16 I + 4G + e][16 J + n16] for the ten lower tiles; rk from the diagonal
  float* rk = sm.rk[wave];
  float* gam = sm.gam[wave];
  float* bet = sm.bet[wave];
  float* M = sm.m(wave);
  f4 gk[10];
  auto gram = [&]() {
#pragma unroll
    for (int t = 0; t < 10; ++t) gk[t] = f4_splat(0.f);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      bf16x8 rows[4];
#pragma unroll
      for (int I = 0; I < 4; ++I) rows[I] = lds16(sm.k() + swz(16 * I + n16, 4 * kb + G));
#pragma unroll
      for (int t = 0; t < 10; ++t) gk[t] = mfma(rows[tile_i(t)], rows[tile_j(t)], gk[t]);
    }
#pragma unroll
    for (int I = 0; I < 4; ++I) {   // diagonal element (16 I + n16, 16 I + n16): lane group n16 / 4, slot n16 & 3
      const f4 dg = gk[I * (I + 1) / 2 + I];
      const int e = n16 & 3;
      const float ss = e == 0 ? dg[0] : e == 1 ? dg[1] : e == 2 ? dg[2] : dg[3];
      if ((n16 >> 2) == G) rk[16 * I + n16] = 1.0f / sqrtf(ss + 1e-6f);   // model.py, _l2norm
    }
  };
  if constexpr (kOne) {
    if (wave < r) gram();
    lds_barrier();   // every wave is done with the K tile, which the matrices overwrite
  } else if (wave < r) {
    gram();
  }
  if (wave >= r) return;   // uniform per wave; no barrier follows

  auto head = [&](int j) {
    // ---- gates of value head kh r + j and gamma (the next head's gates are loaded here too)
    float gv, bv;
    gates_finish<TB>(p, j == wave ? graw : gates_issue<TB>(p, b, kh, c, j, lane), gv, bv);
    store_gates(gam, bet, gv, bv, lane);
    wave_lds_fence();

    // ---- A (strictly lower, fp32) from the Gram tiles: A[t][i] = (beta'_t rk_t) rk_i
    //      2^{min(gamma2_t - gamma2_i, 0)} (K K^T)[t][i]; only the diagonal tiles need the mask
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      const f4 gr = *reinterpret_cast<const f4*>(gam + 16 * I + 4 * G);
      const f4 u = *reinterpret_cast<const f4*>(bet + 16 * I + 4 * G) * *reinterpret_cast<const f4*>(rk + 16 * I + 4 * G);
#pragma unroll
      for (int J = 0; J <= I; ++J) {
        const int col = 16 * J + n16;
        const float gc = gam[col], rc = rk[col];
        const f4 g = gk[I * (I + 1) / 2 + J];
        float* ab = blk(M, I, J);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = u[e] * rc * __builtin_amdgcn_exp2f(fminf(gr[e] - gc, 0.f)) * g[e];
          ab[moff(4 * G + e, n16)] = (J < I || 4 * G + e > n16) ? x : 0.f;
        }
      }
    }
    wave_lds_fence();

    // ---- diagonal blocks: lane 16 G + n16 solves column n16 of block G by forward substitution
    {
      float* ablk = blk(M, G, G);
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = (i == n16) ? 1.f : 0.f;
#pragma unroll
      for (int k = 0; k < 15; ++k) {
        if (kOne && (k & 3) == 0) wave_lds_fence();   // loads at most four columns ahead
#pragma unroll
        for (int i = k + 1; i < 16; ++i) x[i] -= ablk[moff(i, k)] * x[k];
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) ablk[moff(i, n16)] = x[i];
    }
    wave_lds_fence();

    // ---- off-diagonal blocks (split bf16 products). A_20, A_21, A_30, A_31 are read before they are
    //      overwritten.
    const Split4 a21 = split4(tile_row(blk(M, 2, 1), n16, G)), a31 = split4(tile_row(blk(M, 3, 1), n16, G));
    f4 pre0 = f4_splat(0.f), pre1 = f4_splat(0.f);
    {
      const Split4 t00 = split4(tile_acc(blk(M, 0, 0), n16, G));
      mma_split(pre0, split4(tile_row(blk(M, 2, 0), n16, G)), t00);   // A_20 T_00
      mma_split(pre1, split4(tile_row(blk(M, 3, 0), n16, G)), t00);   // A_30 T_00
    }
    // within each 32-row half: T_10 = -T_11 A_10 T_00, T_32 = -T_33 A_32 T_22
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int I = 2 * hf + 1, J = 2 * hf;
      f4 x = f4_splat(0.f), y = f4_splat(0.f);
      mma_split(x, split4(tile_row(blk(M, I, J), n16, G)), split4(tile_acc(blk(M, J, J), n16, G)));
      mma_split(y, split4(tile_row(blk(M, I, I), n16, G)), split4(x));
      store_acc(blk(M, I, J), n16, G, -y);
    }
    wave_lds_fence();
    // across the halves: Z_IJ = A_I0 T_0J + A_I1 T_1J (T_01 = 0), T_2J = -T_22 Z_2J,
    // T_3J = -(T_32 Z_2J + T_33 Z_3J), J = 0, 1
    {
      const Split4 t10 = split4(tile_acc(blk(M, 1, 0), n16, G)), t11 = split4(tile_acc(blk(M, 1, 1), n16, G));
      f4 z20 = pre0, z30 = pre1, z21 = f4_splat(0.f), z31 = f4_splat(0.f);
      mma_split(z20, a21, t10);
      mma_split(z30, a31, t10);
      mma_split(z21, a21, t11);
      mma_split(z31, a31, t11);
      const Split4 r22 = split4(tile_row(blk(M, 2, 2), n16, G)), r32 = split4(tile_row(blk(M, 3, 2), n16, G)),
                   r33 = split4(tile_row(blk(M, 3, 3), n16, G));
      const Split4 s20 = split4(z20), s21 = split4(z21), s30 = split4(z30), s31 = split4(z31);
      f4 o20 = f4_splat(0.f), o21 = f4_splat(0.f), o30 = f4_splat(0.f), o31 = f4_splat(0.f);
      mma_split(o20, r22, s20);
      mma_split(o21, r22, s21);
      mma_split(o30, r32, s20);
      mma_split(o30, r33, s30);
      mma_split(o31, r32, s21);
      mma_split(o31, r33, s31);
      store_acc(blk(M, 2, 0), n16, G, -o20);
      store_acc(blk(M, 2, 1), n16, G, -o21);
      store_acc(blk(M, 3, 0), n16, G, -o30);
      store_acc(blk(M, 3, 1), n16, G, -o31);
    }
    wave_lds_fence();

    // ---- the record: Tb = T diag(beta') as the six operand blocks (zero above the diagonal), then
    //      the scalar rows a, d, gamma log2 e, rk and the contraction flag
    unsigned char* rec = reinterpret_cast<unsigned char*>(p.ws) + (((size_t)b * p.Hv + kh * r + j) * p.NC + c) * kRecBytes;
#pragma unroll
    for (int bk = 0; bk < kFragBlocks; ++bk) {
      const int I = block_tile(bk), kb = block_kb(bk);
      const int c0 = 32 * kb + 4 * G;
      // columns c0.. lie in block (I, 2 kb), columns c0 + 16.. in block (I, 2 kb + 1), which is above
      // the diagonal (not stored, all zero in T) when 2 kb + 1 > I
      const f4 t_lo = tile_row(blk(M, I, 2 * kb), n16, G);
      const f4 t_hi = 2 * kb + 1 <= I ? tile_row(blk(M, I, 2 * kb + 1), n16, G) : f4_splat(0.f);
      // T is exactly zero above the diagonal of its stored diagonal blocks (the forward substitution
      // leaves those entries at zero), so no mask is needed
      const f4 lo = t_lo * *reinterpret_cast<const f4*>(&bet[c0]);
      const f4 hi = t_hi * *reinterpret_cast<const f4*>(&bet[c0 + 16]);
      *reinterpret_cast<bf16x8*>(rec + (size_t)bk * kBlockElems * 2 + (size_t)lane * 16) = pack8(lo, hi);
    }
    {
      const float g2 = gam[lane], g2C = gam[C - 1], rkl = rk[lane];
      float* sc = reinterpret_cast<float*>(rec + kFragBlocks * kBlockElems * 2);
      sc[kBfA * C + lane] = __builtin_amdgcn_exp2f(g2) * rkl;
      sc[kBfD * C + lane] = rkl * __builtin_amdgcn_exp2f(fminf(g2C - g2, 0.f));
      sc[kBfGam2 * C + lane] = g2;
      sc[kBfRk * C + lane] = rkl;
      // every beta' of the chunk in [0, 2] (each token's map then has spectral norm <= e^{g'}) and
      // the chunk's decay sum <= 0: the chunk's map has spectral norm <= e^{sum g'} <= 1
      const float bt = bet[lane];
      const bool ok = __all(bt >= 0.f && bt <= 2.f) && g2C <= 0.f;
      sc[kBfFlag * C + lane] = (lane == 0 && ok) ? 1.f : 0.f;
    }
    wave_lds_fence();   // the next head's gates and A are written after this head's last reads
  };
  if constexpr (kOne) {
    head(wave);
  } else {
    for (int j = wave; j < r; j += kPrepWaves) head(j);
  }
}

hipError_t launch_prep(const PrepParams& p, int qkv_bf16, int beta_bf16, hipStream_t s) {
  if (qkv_bf16) {
    // items: an upper bound with a chunk list (the kernel reads the count); <= B Hv NC < 2^31
    // (checked by the caller)
    const int64_t items = int64_t(p.B) * p.Hk * p.NC;
    const dim3 wgrid((unsigned)items), wblock(64 * kPrepWaves);
    if (p.chunk_list) hipLaunchKernelGGL(gdr_chunk_list, dim3(1), dim3(256), 0, s, p.lengths, p.B, p.L, p.NC, p.chunk_list);
    // one instantiation per (gate dtype, chunk list, at most one value head per wave)
    using K = void (*)(PrepParams);
    static const K kernels[2][2][2] = {
        {{gdr_prep_wave<float, false, false>, gdr_prep_wave<float, false, true>},
         {gdr_prep_wave<float, true, false>, gdr_prep_wave<float, true, true>}},
        {{gdr_prep_wave<__bf16, false, false>, gdr_prep_wave<__bf16, false, true>},
         {gdr_prep_wave<__bf16, true, false>, gdr_prep_wave<__bf16, true, true>}}};
    const bool one = p.Hv / p.Hk <= kPrepWaves;
    hipLaunchKernelGGL(kernels[beta_bf16 ? 1 : 0][p.chunk_list ? 1 : 0][one ? 1 : 0], wgrid, wblock, 0, s, p);
  } else {
    const dim3 grid(p.B * p.Hv * p.NC);
    hipLaunchKernelGGL((gdr_prep<float, float>), grid, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace gdr
