// Sequential inter-chunk state scan of the chunked gated delta rule (gfx950).
//
// Per chunk (S = state entering the chunk, [Dk, Dv], fp32; a, c, d, e^{gamma_63}, Tb and P from
// the chunk record written by the prep kernel; K, Q the raw chunk rows):
//   X = K S,  R = V - diag(a) X,  Delta = Tb R,  O = diag(c) Q S + P Delta,
//   S <- e^{gamma_63} S + K^T diag(d) Delta
// which is the per-token recurrence of the kernel-test page (r15_kernel_test.py, function
// truth_f64) unrolled over 64 tokens. The state columns evolve independently, so the value
// dimension is split across workgroups.
//
// gdr_scan_bf16: one workgroup per (row, value head, 16-column slice) = 8 per head. Its four
// waves share each chunk: wave w computes token tile w (rows 16w..16w+15) of X, Q S, R, Delta
// and O, and 32 key rows of the state update. Each wave loads its own operand rows (K and Q
// rows, Tb and P operand blocks, scalars, V) straight into registers two chunks ahead; only K
// goes through LDS (for the transposed K^T operand of the state update) together with bf16
// copies of S, R and Delta, exchanged as ready-made MFMA B operands (three barriers per chunk).
// Workgroups are numbered so that the 8 slices of a head, and the value heads of one key head,
// run on the same XCD and share its L2.
//
// State row order. Wave w holds key rows 32w..32w+31 in two 16x16 accumulator tiles; tile s,
// row r stands for key index 32w + 8(r >> 2) + 4s + (r & 3). With that order the eight B-operand
// slots of lane group G are the eight consecutive key indices 32w + 8G .. 32w + 8G + 7, so every
// A operand along the key index (K and Q rows) is one contiguous 16-byte load per lane.
//
// gdr_scan_f32: float32 inputs; one workgroup per (row, value head, 64-column slice), each wave
// owning 16 columns and walking all chunks on its own (fp32 MFMA, K^T staged in LDS).
#include "gdr_device.h"

namespace gdr {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// ====================================================================== bf16 cooperative scan
constexpr int kSlices = D / 16;                                        // workgroups per (row, head)
constexpr int kRecB = 2 * kFragBlocks * kBlockElems * 2 + 4 * C * 4;   // bf16 record bytes (13312)
constexpr int kScOff = 2 * kFragBlocks * kBlockElems * 2;              // scalars within the record
constexpr int kBufK = C * D * 2;                                       // one 64x128 bf16 K tile

// LDS: two K tiles (64 rows x 256 B; the 16-byte chunk j of row r is stored at position
// j ^ (r & 15), which spreads row reads, row writes and transposing reads over the banks) and
// the operand exchanges.
struct ScanSmemB {
  __attribute__((aligned(16))) unsigned char k[2][kBufK];
  bf16x8 sx[4][64];   // S (bf16) as B operands, k block = 32 key rows
  bf16x8 rx[2][64];   // R, k block = 32 tokens
  bf16x8 dx[2][64];   // Delta
  bf16x8 ddx[2][64];  // diag(d) Delta
};

// One chunk's operands for one lane, loaded three chunks ahead.
struct OperandsB {
  bf16x8 kf[4], qf[4];   // K, Q rows of token tile w, key block kb (8 consecutive key indices)
  bf16x8 tbf[2], pf[2];  // Tb, P operand blocks of token tile w
  f4 a, c, d;            // per-token scalars of this lane's four tokens
  float egc;             // e^{gamma_63}
  uint32_t v[4];         // V of this lane's four tokens: the 4-byte word holding this lane's column
};

__device__ __forceinline__ int swz(int row, int chunk16) { return row * 256 + 16 * (chunk16 ^ (row & 15)); }

// K^T operand for state tile s of wave w (key index 32w + 8(m >> 2) + 4s + (m & 3) in row m),
// k = tokens of block kb, from the swizzled K tile. In each 16-lane group the transposing read
// hands lane j element (j & 3) of the 8 bytes that lanes 4i + (j >> 2) address, i = 0..3; lane
// n therefore points at K[t0 + (n >> 2)][32w + 8(n & 3) + 4s].
__device__ __forceinline__ Frag<__bf16> kt_frag(const unsigned char* tile, int w, int s, int kb, int G, int n16) {
  const int j = 4 * w + (n16 & 3), sub = 8 * s;
  const int r0 = 32 * kb + 4 * G + (n16 >> 2), r1 = r0 + 16;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + swz(r0, j) + sub));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + swz(r1, j) + sub));
  Frag<__bf16> f;
  f.v = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  return f;
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 x) { return __builtin_bit_cast(bf16x8, x); }
__device__ __forceinline__ f4 as_f4(uint4 x) { return __builtin_bit_cast(f4, x); }

// Loop-carried values of one wave between chunks (c = the chunk about to start):
//   Y   = K_c S_{c-1} (token tile w; K_0 S_0 before the first chunk)   fp32 accumulator tile
//   G   = (K_c K_{c-1}^T) rows of token tile w, as A operands over the tokens of chunk c-1
//   Dd  = diag(d_{c-1}) Delta_{c-1}, as B operands over the tokens of chunk c-1
//   eg  = e^{gamma_63} of chunk c-1
// so that X_c = K_c S_c = eg Y + G Dd (S_c = eg S_{c-1} + K_{c-1}^T Dd), i.e. the product with
// the state entering the chunk is formed one chunk early and only the short correction G Dd
// sits on the critical path between chunks.
struct CarryB {
  f4 y;
  bf16x8 g[2], dd[2];
  float eg;
};

__global__ __launch_bounds__(256) void gdr_scan_bf16(ScanParams p) {
  __shared__ __attribute__((aligned(16))) ScanSmemB sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, kept in a scalar register
  const int n16 = lane & 15, G = lane >> 4;
  // XCD-aware numbering: hardware workgroup i runs on XCD i % 8; consecutive logical ids
  // (the slices of one head, then the heads of one key head) are kept on one XCD.
  const int nwg = gridDim.x;                       // B * Hv * kSlices, a multiple of 8
  const int lam = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
  const int slice = lam % kSlices;
  const int h = (lam / kSlices) % p.Hv;
  const int b = lam / (kSlices * p.Hv);
  const int kh = h / (p.Hv / p.Hk);
  const int col0 = 16 * slice, ncol = col0 + n16;
  const __bf16* qg = reinterpret_cast<const __bf16*>(p.q);
  const __bf16* kg = reinterpret_cast<const __bf16*>(p.k);
  const __bf16* vg = reinterpret_cast<const __bf16*>(p.v);
  __bf16* og = reinterpret_cast<__bf16*>(p.o);
  const unsigned char* wsb = reinterpret_cast<const unsigned char*>(p.ws);
  const size_t row_stride_v = (size_t)p.Hv * D;

  const int len = p.lengths ? p.lengths[b] : p.L;
  const int srow = p.s0 ? (p.s0_row ? p.s0_row[b] : b) : 0;
  if ((len < 0 || len > p.L) || (p.s0 && (srow < 0 || srow >= p.n_s0))) {
    const float nan = __builtin_nanf("");
    for (int i = tid; i < p.L * 16; i += 256)
      og[((size_t)b * p.L + i / 16) * row_stride_v + (size_t)h * D + col0 + i % 16] = (__bf16)nan;
    if (p.s_final)
      for (int i = tid; i < D * 16; i += 256)
        p.s_final[(((size_t)b * p.Hv + h) * D + i / 16) * D + col0 + i % 16] = nan;
    return;
  }

  // Range-checked buffer descriptors: rows past L and chunks past the last one read as zeros
  // and output rows past L are dropped, so the loads below are unconditional and branch-free.
  const uint32_t kq_row = (uint32_t)p.Hk * D * 2, vo_row = (uint32_t)p.Hv * D * 2;
  const size_t kq_base = (size_t)b * p.L * p.Hk * D, vo_base = (size_t)b * p.L * p.Hv * D + (size_t)h * D + col0;
  const uint32_t vo_bytes = p.L > 0 ? (uint32_t)(p.L - 1) * vo_row + 32 : 0;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kg + kq_base, (uint32_t)p.L * kq_row);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(qg + kq_base, (uint32_t)p.L * kq_row);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(vg + vo_base, vo_bytes);
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(og + vo_base, vo_bytes);
  const __amdgpu_buffer_rsrc_t rr = make_rsrc(wsb + ((size_t)b * p.Hv + h) * p.NC * kRecB, (uint32_t)p.NC * kRecB);
  const int t4 = 16 * w + 4 * G;                   // first of this lane's four tokens in a chunk
  const uint32_t kq_lane = (uint32_t)(16 * w + n16) * kq_row + (uint32_t)kh * D * 2 + 16 * G;
  const uint32_t blk0 = 1024 * frag_block(w, 0) + 16 * lane;

  auto load = [&](OperandsB& f, int c) {
    const uint32_t kq = (uint32_t)c * C * kq_row + kq_lane;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      f.kf[kb] = as_bf16x8(buf_load16(rk, kq + 64 * kb));
      f.qf[kb] = as_bf16x8(buf_load16(rq, kq + 64 * kb));
    }
    const uint32_t rec = (uint32_t)c * kRecB;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {   // block kb = 1 of tiles 0 and 1 is never used (upper triangle)
      f.tbf[kb] = as_bf16x8(buf_load16(rr, rec + blk0 + 1024 * kb));
      f.pf[kb] = as_bf16x8(buf_load16(rr, rec + kFragBlocks * 1024 + blk0 + 1024 * kb));
    }
    f.a = as_f4(buf_load16(rr, rec + kScOff + 4 * t4));
    f.c = as_f4(buf_load16(rr, rec + kScOff + 4 * (C + t4)));
    f.d = as_f4(buf_load16(rr, rec + kScOff + 4 * (2 * C + t4)));
    f.egc = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rr, rec + kScOff + 4 * 3 * C, 0, 0));
    const uint32_t vrow = ((uint32_t)c * C + t4) * vo_row + 4 * (n16 >> 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) f.v[i] = __builtin_amdgcn_raw_buffer_load_b32(rv, vrow + i * vo_row, 0, 0);
  };

  // ---- state key rows of wave w (order above), this slice's 16 columns
  f4 S[2];
  {
    const float* s0 = p.s0 ? p.s0 + ((size_t)srow * p.Hv + h) * D * D : nullptr;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) S[s][i] = s0 ? s0[(32 * w + 8 * G + 4 * s + i) * D + ncol] : 0.f;
  }
  auto publish_state = [&]() {
    bf16x8 f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = (__bf16)S[0][i];
      f[4 + i] = (__bf16)S[1][i];
    }
    sm.sx[w][lane] = f;
  };

  const int nkb = (w >> 1) + 1;   // token blocks of 32 that reach token tile w (lower triangle)
  // One chunk: f = operands of chunk c, fn = operands of chunk c+1 (only its K rows are used).
  auto chunk = [&](const OperandsB& f, const OperandsB& fn, CarryB& cy, int c) {
    unsigned char* Kt = sm.k[c & 1];
    // -- this wave's K rows into the shared K tile of chunk c
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) *reinterpret_cast<bf16x8*>(Kt + swz(16 * w + n16, 4 * kb + G)) = f.kf[kb];
    // -- critical: X_c = eg Y + G Dd, R = V - diag(a) X  -> exchange
    {
      f4 X = cy.eg * cy.y;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        Frag<__bf16> Ga, Db;
        Ga.v = cy.g[kb];
        Db.v = cy.dd[kb];
        mma(X, Ga, Db);
      }
      bf16x4 rv;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        rv[i] = (__bf16)(__builtin_bit_cast(float, (n16 & 1) ? (f.v[i] & 0xffff0000u) : (f.v[i] << 16)) - f.a[i] * X[i]);
      reinterpret_cast<bf16x4*>(&sm.rx[w >> 1][lane])[w & 1] = rv;
    }
    __syncthreads();
    // -- critical: Delta = Tb R for token tile w  -> exchange Delta and diag(d) Delta
    {
      f4 Dl = f4_splat(0.f);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (kb < nkb) {
          Frag<__bf16> Rf, Tf;
          Rf.v = sm.rx[kb][lane];
          Tf.v = f.tbf[kb];
          mma(Dl, Tf, Rf);
        }
      }
      bf16x4 d1, d2;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        d1[i] = (__bf16)Dl[i];
        d2[i] = (__bf16)(f.d[i] * Dl[i]);
      }
      reinterpret_cast<bf16x4*>(&sm.dx[w >> 1][lane])[w & 1] = d1;
      reinterpret_cast<bf16x4*>(&sm.ddx[w >> 1][lane])[w & 1] = d2;
    }
    // -- off the critical path (state S_c is in sx): OQ = Q_c S_c, Y' = K_{c+1} S_c, and
    //    G' = K_{c+1} K_c^T formed as its transpose K_c K_{c+1}^T, whose accumulator layout is
    //    exactly the A-operand layout G' needs
    f4 OQ = f4_splat(0.f), Yn = f4_splat(0.f);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      Frag<__bf16> Sf, Qa, Kn;
      Sf.v = sm.sx[kb][lane];
      Qa.v = f.qf[kb];
      Kn.v = fn.kf[kb];
      mma(OQ, Qa, Sf);
      mma(Yn, Kn, Sf);
    }
    f4 Gt[4];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      Gt[jt] = f4_splat(0.f);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        Frag<__bf16> Ka, Kn;
        Ka.v = *reinterpret_cast<const bf16x8*>(Kt + swz(16 * jt + n16, 4 * kb + G));
        Kn.v = fn.kf[kb];
        mma(Gt[jt], Ka, Kn);
      }
    }
    __syncthreads();
    // -- O = diag(c) OQ + P Delta (token tile w);  S <- e^{gamma_63} S + K^T diag(d) Delta
    Frag<__bf16> Df[2], Ddf[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      Df[kb].v = sm.dx[kb][lane];
      Ddf[kb].v = sm.ddx[kb][lane];
    }
    {
      f4 O = f.c * OQ;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (kb < nkb) {
          Frag<__bf16> Pf;
          Pf.v = f.pf[kb];
          mma(O, Pf, Df[kb]);
        }
      }
      const uint32_t ob = ((uint32_t)c * C + t4) * vo_row + 2 * n16;
#pragma unroll
      for (int i = 0; i < 4; ++i) buf_store_bf16(ro, ob + i * vo_row, (__bf16)O[i]);
    }
    S[0] *= f.egc;
    S[1] *= f.egc;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      mma(S[0], kt_frag(Kt, w, 0, kb, G, n16), Ddf[kb]);
      mma(S[1], kt_frag(Kt, w, 1, kb, G, n16), Ddf[kb]);
    }
    publish_state();   // read again after the next chunk's first barrier
    cy.y = Yn;
    cy.eg = f.egc;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      cy.dd[kb] = Ddf[kb].v;
      cy.g[kb] = acc_frag<__bf16>(Gt[2 * kb], Gt[2 * kb + 1], f4_splat(1.f), f4_splat(1.f)).v;
    }
  };

  OperandsB f0, f1, f2;
  load(f0, 0);
  load(f1, 1);
  load(f2, 2);
  publish_state();
  // Let the first chunks land before the loop: the loop then starts from the same
  // outstanding-load pattern as its own steady state, so its waits stay exact.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  CarryB cy;
  cy.y = f4_splat(0.f);
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    Frag<__bf16> Sf, Ka;
    Sf.v = sm.sx[kb][lane];
    Ka.v = f0.kf[kb];
    mma(cy.y, Ka, Sf);                 // Y = K_0 S_0
  }
  cy.eg = 1.f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    cy.g[kb] = bf16x8{};
    cy.dd[kb] = bf16x8{};
  }
  int c = 0;
  for (; c + 2 < p.NC; c += 3) {   // straight-line body: three chunks, each set reloaded after use
    chunk(f0, f1, cy, c);
    load(f0, c + 3);
    chunk(f1, f2, cy, c + 1);
    load(f1, c + 4);
    chunk(f2, f0, cy, c + 2);
    load(f2, c + 5);
  }
  if (c < p.NC) chunk(f0, f1, cy, c);
  if (c + 1 < p.NC) chunk(f1, f2, cy, c + 1);

  if (p.s_final) {
    float* sf = p.s_final + ((size_t)b * p.Hv + h) * D * D;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) sf[(32 * w + 8 * G + 4 * s + i) * D + ncol] = S[s][i];
  }
}

// ====================================================================== fp32 scan
constexpr int kRecF = 2 * kFragBlocks * kBlockElems * 4 + 4 * C * 4;   // fp32 record bytes (25600)
constexpr int kPK32 = D + 4, kPT32 = C + 4;

struct ScanSmemF {
  float k[C * kPK32];      // K chunk, [token][dk]
  float q[C * kPK32];      // Q chunk, [token][dk]
  float kt[D * kPT32];     // K chunk transposed, [dk][token]
  float tb[C * kPT32];     // T diag(beta'), [token][token]
  float pm[C * kPT32];     // decayed causal scores, [token][token]
  float v[C * kPT32];      // this workgroup's 64 value columns, [token][col]
  float sc[4 * C];         // a, c, d, e^{gamma_63}
};

__global__ __launch_bounds__(256) void gdr_scan_f32(ScanParams p) {
  __shared__ __attribute__((aligned(16))) ScanSmemF sm;
  constexpr int NW = 4, NT = 256;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n16 = lane & 15, G = lane >> 4;
  const int cg = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int kh = h / (p.Hv / p.Hk);
  const int col0 = cg * (16 * NW);
  const int ncol = col0 + 16 * wave + n16;
  const float* qg = reinterpret_cast<const float*>(p.q);
  const float* kg = reinterpret_cast<const float*>(p.k);
  const float* vg = reinterpret_cast<const float*>(p.v);
  float* og = reinterpret_cast<float*>(p.o);
  const unsigned char* wsb = reinterpret_cast<const unsigned char*>(p.ws);

  const int len = p.lengths ? p.lengths[b] : p.L;
  const int srow = p.s0 ? (p.s0_row ? p.s0_row[b] : b) : 0;
  if ((len < 0 || len > p.L) || (p.s0 && (srow < 0 || srow >= p.n_s0))) {
    const float nan = __builtin_nanf("");
    for (int i = tid; i < p.L * 16 * NW; i += NT)
      og[((size_t)b * p.L + i / (16 * NW)) * p.Hv * D + (size_t)h * D + col0 + i % (16 * NW)] = nan;
    if (p.s_final)
      for (int i = tid; i < D * 16 * NW; i += NT)
        p.s_final[(((size_t)b * p.Hv + h) * D + i / (16 * NW)) * D + col0 + i % (16 * NW)] = nan;
    return;
  }

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
    const unsigned char* rec = wsb + (((size_t)b * p.Hv + h) * p.NC + c) * kRecF;
    const float* recf = reinterpret_cast<const float*>(rec);
    __syncthreads();   // the previous chunk is done with LDS
    for (int idx = tid; idx < C * (D / 4); idx += NT) {
      const int row = idx / (D / 4), cv = idx % (D / 4), t = t0 + row;
      f4 kv = f4_splat(0.f), qv = f4_splat(0.f);
      if (t < p.L) {
        const size_t off = ((size_t)b * p.L + t) * p.Hk * D + (size_t)kh * D + 4 * cv;
        kv = *reinterpret_cast<const f4*>(kg + off);
        qv = *reinterpret_cast<const f4*>(qg + off);
      }
      *reinterpret_cast<f4*>(&sm.k[row * kPK32 + 4 * cv]) = kv;
      *reinterpret_cast<f4*>(&sm.q[row * kPK32 + 4 * cv]) = qv;
#pragma unroll
      for (int e = 0; e < 4; ++e) sm.kt[(4 * cv + e) * kPT32 + row] = kv[e];
    }
    // Tb and P unpacked from operand blocks to full 64x64 (zeros above the stored blocks)
    for (int idx = tid; idx < C * C; idx += NT) {
      const int row = idx / C, col = idx % C;
      const int w = row / 16, kb = col / 32;
      float tv = 0.f, pv = 0.f;
      if (kb <= w / 2) {
        const int cc = col % 32, g = (cc % 16) / 4, j = (cc / 16) * 4 + cc % 4;
        const int e = frag_block(w, kb) * kBlockElems + ((row % 16) + 16 * g) * 8 + j;
        tv = recf[e];
        pv = recf[kFragBlocks * kBlockElems + e];
      }
      sm.tb[row * kPT32 + col] = tv;
      sm.pm[row * kPT32 + col] = pv;
    }
    for (int idx = tid; idx < C * (16 * NW / 4); idx += NT) {
      const int row = idx / (16 * NW / 4), cv = idx % (16 * NW / 4), t = t0 + row;
      f4 vv = f4_splat(0.f);
      if (t < p.L) vv = *reinterpret_cast<const f4*>(vg + ((size_t)b * p.L + t) * p.Hv * D + (size_t)h * D + col0 + 4 * cv);
      *reinterpret_cast<f4*>(&sm.v[row * kPT32 + 4 * cv]) = vv;
    }
    for (int idx = tid; idx < C; idx += NT)
      *reinterpret_cast<f4*>(&sm.sc[4 * idx]) =
          *reinterpret_cast<const f4*>(rec + 2 * kFragBlocks * kBlockElems * 4 + 16 * idx);
    __syncthreads();

    const float* sa = sm.sc;
    const float* scc = sm.sc + C;
    const float* sd = sm.sc + 2 * C;
    const float egC = sm.sc[3 * C];
    const f4 one = f4_splat(1.f);

    Frag<float> Sf[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) Sf[kb] = acc_frag<float>(S[2 * kb], S[2 * kb + 1], one, one);
    f4 X[4], OQ[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      X[mt] = f4_splat(0.f);
      OQ[mt] = f4_splat(0.f);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        mma(X[mt], lds_frag(sm.k, kPK32, 16 * mt + n16, 32 * kb, G), Sf[kb]);
        mma(OQ[mt], lds_frag(sm.q, kPK32, 16 * mt + n16, 32 * kb, G), Sf[kb]);
      }
    }
    f4 R[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * mt + 4 * G + e;
        R[mt][e] = sm.v[t * kPT32 + 16 * wave + n16] - sa[t] * X[mt][e];
      }
    Frag<float> Rf[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) Rf[kb] = acc_frag<float>(R[2 * kb], R[2 * kb + 1], one, one);
    f4 Dl[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      Dl[mt] = f4_splat(0.f);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) mma(Dl[mt], lds_frag(sm.tb, kPT32, 16 * mt + n16, 32 * kb, G), Rf[kb]);
    }
    Frag<float> Df[2], Ddf[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      Df[kb] = acc_frag<float>(Dl[2 * kb], Dl[2 * kb + 1], one, one);
      f4 d0, d1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        d0[e] = sd[32 * kb + 4 * G + e];
        d1[e] = sd[32 * kb + 16 + 4 * G + e];
      }
      Ddf[kb] = acc_frag<float>(Dl[2 * kb], Dl[2 * kb + 1], d0, d1);
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f4 O;
#pragma unroll
      for (int e = 0; e < 4; ++e) O[e] = scc[16 * mt + 4 * G + e] * OQ[mt][e];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) mma(O, lds_frag(sm.pm, kPT32, 16 * mt + n16, 32 * kb, G), Df[kb]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = t0 + 16 * mt + 4 * G + e;
        if (t < p.L) og[((size_t)b * p.L + t) * p.Hv * D + (size_t)h * D + ncol] = O[e];
      }
    }
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      S[st] *= egC;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) mma(S[st], lds_frag(sm.kt, kPT32, 16 * st + n16, 32 * kb, G), Ddf[kb]);
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

hipError_t launch_scan(const ScanParams& p, int qkv_bf16, hipStream_t s) {
  if (qkv_bf16) {
    hipLaunchKernelGGL(gdr_scan_bf16, dim3(p.B * p.Hv * kSlices), dim3(256), 0, s, p);
  } else {
    hipLaunchKernelGGL(gdr_scan_f32, dim3(D / 64, p.Hv, p.B), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace gdr
