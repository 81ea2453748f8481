// Inter-chunk state scan of the chunked gated delta rule (gfx950).
//
// Per chunk (S = state entering the chunk, [Dk, Dv], fp32; a, c, d, e^{gamma_63} and Tb from the
// chunk record written by the prep kernel; P, the decayed and masked scores, from the record too
// (fp32) or formed by the output pass from the staged Q and K tiles as P' (bf16); K, Q the raw
// chunk rows):
//   X = K S,  R = V - diag(a) X,  Delta = Tb R,  O = diag(c) Q S + P Delta,
//   S <- e^{gamma_63} S + K^T diag(d) Delta
// which is the per-token recurrence of the kernel-test page (r15_kernel_test.py, function
// truth_f64) unrolled over 64 tokens. The value columns of the state evolve independently.
//
// bf16: segment-parallel. The map from the state entering a run of chunks to the state leaving
// it is affine, S -> M S + B, with M independent of the values. The chunks of each (row, head)
// are cut into P segments; gdr_transition_bf16 runs every segment but the last from the
// augmented start [0 | identity] (giving B_j and M_j), gdr_combine chains
// S_{j+1} = M_j S_j + B_j over the segments, and gdr_scan_bf16 runs every segment again from
// its true entering state, writing outputs (and, for the last one, the final state). With
// P = 1 only gdr_scan_bf16 runs. Chunks wholly past a row's length (right pads: beta' = g' = 0)
// are the identity map: the transitions skip them and the output pass gives them a short loop of
// their own (O = diag(rq) Q S). Under strong decay a (row, head) takes truncated segment starts
// instead (the transition pass runs only a short window before each boundary from zero, the
// combine returns at once, and gdr_finalize_bf16 checks the error bound afterwards, rerunning the
// (row, head) exactly where it fails; see the truncation plan below).
//
// gdr_scan_f32: float32 inputs; one workgroup per (row, value head, 16-column slice), its four
// waves splitting the slice's state by key blocks and walking all chunks together (fp32 MFMA, each
// chunk loaded into registers one chunk ahead).
#include "gdr_device.h"

namespace gdr {

typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kSlices16 = D / 16;   // 16-column slices of a head
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// ====================================================================== bf16 segment scan
constexpr int kScOff = kFragBlocks * kBlockElems * 2;                  // scalars within a bf16 record
constexpr int kRecB = kScOff + kScalarBytes;                           // bf16 record bytes (8192)
constexpr int kRecBlocks = kFragBlocks + 1;   // 1 KiB loads per chunk: Tb and the first scalar block
constexpr int kBufK = C * D * 2;                                       // one 64x128 bf16 tile

// LDS staging of one chunk (every wave reads every part of it): K, V (and Q) tiles of 64 rows x
// 256 bytes, swizzled as below, and the record as written by the prep kernel. Two buffers: chunk
// c + 1 is loaded while chunk c is computed.
// Right-pad chunks of the output pass without the fused norm are taken kPadGroup at a time: their Q
// tiles fill the Q, K and V regions of one buffer while the next group loads into the other.
constexpr int kPadGroup = 3;
template <bool kOut> struct SegCfg {
  static constexpr int NW = 8;                          // waves per workgroup (two per SIMD)
  static constexpr int NSL = (kOut ? 8 : 16) / NW;      // 16-column slices per wave: 1 (outputs), 2 (transitions)
  static constexpr int kK = 0, kV = kBufK, kRec = 2 * kBufK;
  static constexpr int kQ = kRec + kRecB;               // outputs only
  static constexpr int kZ = kQ + kBufK;                 // outputs only: the fused norm's gate rows
  static constexpr int kBuf = kOut ? kZ + kBufK : kRec + kRecB;
  // outputs only, after the two buffers: P of the current chunk (formed by the waves; one copy,
  // as it is formed and used between the same two barriers), the fused norm's row sums, and the
  // squared norms of the chunk's q rows (formed and used between the same two barriers)
  static constexpr int kP = 2 * kBuf;
  static constexpr int kPart = kP + kFragBlocks * 1024;
  static constexpr int kRq = kPart + 2 * NW * C * 4;    // outputs only: |q_t|^2 of the chunk's tokens
  static constexpr int kLds = kOut ? kRq + kPadGroup * C * 4 : 2 * kBuf;
  static constexpr int kStores = kOut ? 4 * NSL : 0;    // output stores per wave per chunk
  static_assert(NW == 8, "the staging split and the P' block assignment are written for eight waves");
};

// K and Q tiles use the row swizzle swz of the device header. V tiles: position q ^ 2(r & 7), which
// keeps the two chunks of eight consecutive rows read together apart.
__device__ __forceinline__ int swz_v(int row, int chunk16) { return row * 256 + 16 * (chunk16 ^ (2 * (row & 7))); }
// Gate rows of the fused norm: position q ^ (r & 15), so that sixteen consecutive rows read at one
// 16-byte chunk land on sixteen distinct positions (every bank once).
__device__ __forceinline__ int swz_z(int row, int chunk16) { return row * 256 + 16 * (chunk16 ^ (row & 15)); }


// Wait until at most N vector-memory operations of this wave are outstanding and all of its
// LDS accesses are done, then meet the other waves. Memory clobbers keep every LDS access on
// its side of the wait and the barrier.
template <int N> __device__ __forceinline__ void wait_and_barrier() {
  static_assert(N == 0 || N == 4 || N == 8 || N == 12 || N == 24, "extend the list of encodings");   // stores
  if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 24) asm volatile("s_waitcnt vmcnt(24) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 4) asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 8) asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(12) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// 1 / (1 + e^-x) with the hardware exp2 and reciprocal
__device__ __forceinline__ float silu_gate(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x * -1.4426950408889634f));
}

// K^T operand for state tile (key block kb, half s2), k = tokens of token block kb2, from the
// swizzled K tile. In each 16-lane group the transposing read hands lane m element (m & 3) of
// the 8 bytes that lanes 4i + (m >> 2) address, i = 0..3; lane n therefore points at
// K[32 kb2 + 4G + (n >> 2) (+16)][32 kb + 8(n & 3) + 4 s2], and lane m receives key
// 32 kb + 8(m >> 2) + 4 s2 + (m & 3) for the tokens of slots 0..7.
__device__ __forceinline__ bf16x8 kt_frag(const unsigned char* tile, int kb, int s2, int kb2, int G, int n16) {
  const int q = 4 * kb + (n16 & 3), sub = 8 * s2;
  const int r0 = 32 * kb2 + 4 * G + (n16 >> 2), r1 = r0 + 16;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + swz(r0, q) + sub));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + swz(r1, q) + sub));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// V[t0 + i][col0 + n16], i = 0..3, for the 16 columns starting at col0 (a multiple of 16):
// lane n points at V[t0 + (n >> 2)][col0 + 4(n & 3)], and the transposing read gives lane m
// column col0 + m of the four rows.
__device__ __forceinline__ f4 v_col4(const unsigned char* vt, int t0, int col0, int n16) {
  const int t = t0 + (n16 >> 2), col = col0 + 4 * (n16 & 3);
  const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vt + swz_v(t, col >> 3) + 2 * (col & 7)));
  const bf16x4 y = __builtin_bit_cast(bf16x4, x);
  return f4{(float)y[0], (float)y[1], (float)y[2], (float)y[3]};
}

__device__ __forceinline__ bool row_is_bad(const ScanParams& p, int b, int& srow) {
  const int len = p.lengths ? p.lengths[b] : p.L;
  srow = p.s0 ? (p.s0_row ? p.s0_row[b] : b) : 0;
  return (len < 0 || len > p.L) || (p.s0 && (srow < 0 || srow >= p.n_s0));
}

// One segment (chunks [Ls j, Ls j + Ls) of row b, value head h) on one workgroup. Each wave
// owns NSL 16-column slices of the state (all 128 key rows, fp32 accumulators) and runs the
// whole chunk recurrence for them on its own: the accumulator layout of one product is the
// operand layout of the next, so the waves share only the staged chunk, never results.
//
// State layout. Slice sl, key block kb (32 keys), half s2: a 16x16 accumulator tile whose row r
// stands for key 32 kb + 8(r >> 2) + 4 s2 + (r & 3). Lane (n16, G) thus holds keys
// 32 kb + 8G + 4 s2 + i of column n16, and the two halves together are the eight consecutive
// keys 32 kb + 8G .. 32 kb + 8G + 7: one bf16 MFMA operand along the key index, matching a single
// 16-byte read of a K or Q row.
//
// kOut = true (outputs): the value columns seg_col + n16 start from the state entering the
// segment and the chunk outputs are written; the last segment writes the final state.
// kOut = false (transition): the first half of each wave's slices hold value columns from a
// zero state (the local state B_j), the second half identity columns with zero values (the
// transition M_j), 256 columns in all (augmented index seg_col); nothing but the two end states
// is written.
// Column of slice sl of wave w: value columns for the outputs; for the transitions the first
// half of a wave's slices are value columns (local state) and the second half identity columns
// (transition), stored at augmented index 128 + k.
template <bool kOut>
__device__ __forceinline__ int seg_col(int w, int sl) {
  constexpr int NSL = SegCfg<kOut>::NSL, H = NSL / 2;
  if constexpr (kOut) return 16 * (w * NSL + sl);
  else return sl < H ? 16 * (w * H + sl) : D + 16 * (w * H + sl - H);
}
template <bool kOut> __device__ __forceinline__ constexpr bool seg_has_v(int sl) {
  return kOut || sl < SegCfg<kOut>::NSL / 2;
}

// What one workgroup runs: chunks [c_begin, c_end) of (row b, value head h), from an entering state,
// and where its results go.
struct SegRun {
  int c_begin, c_end;
  int src_kind;         // 0: zero (identity for the transitions' M columns), 1: src (pitch 2D), 2: s0 row
  const float* src;     // the entering state in a segment slot, columns 0 .. 127
  bool last;            // outputs: the run ends the row, so it writes s_final
  int cert_chunk;       // outputs: at the top of this chunk (-1: none) each wave writes the sum of
  float* cert;          //   squares of its part of the state into cert[wave]
  float* end_b;         // transitions, windows: the end state of the value columns (slot, pitch 2D)
  float* end_m;         // transitions: the identity columns' state M (slot columns 128.., or null)
  float* n2;            // windows: each wave's sum of squares of the end state (transitions: null)
};

// Sum over the 64 lanes of a wave, in every lane.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// kWin (with kOut): a window, the chunks c_begin .. c_end - 1 run from zero on the value columns in
// the output pass's layout but without its outputs; it leaves the end state and its norm.
// kFuse (with kOut): the gated RMSNorm is fused into the outputs (p.z is set). A separate
// instantiation, so that the plain output pass carries none of the norm's registers or branches.
template <bool kOut, bool kWin = false, bool kFuse = false>
__device__ __forceinline__ void seg_body(const ScanParams& p, unsigned char* lds, int b, int h, const SegRun& run) {
  static_assert(kOut || !kWin, "a window runs in the output pass's layout");
  static_assert(!kFuse || (kOut && !kWin), "the norm is fused into the outputs only");
  using Cfg = SegCfg<kOut>;
  constexpr int NSL = Cfg::NSL, NW = Cfg::NW;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15, G = lane >> 4;
  const int kh = h / (p.Hv / p.Hk);
  const int c_begin = run.c_begin, c_end = run.c_end;
  const __bf16* qg = reinterpret_cast<const __bf16*>(p.q);
  const __bf16* kg = reinterpret_cast<const __bf16*>(p.k);
  const __bf16* vg = reinterpret_cast<const __bf16*>(p.v);
  __bf16* og = reinterpret_cast<__bf16*>(p.o);

  int srow = 0;
  if (kOut && !kWin && row_is_bad(p, b, srow)) {
    const float nan = __builtin_nanf("");
    const int t_end = min(c_end * C, p.L);
    for (int i = c_begin * C * D + tid; i < t_end * D; i += 64 * NW)
      og[((size_t)b * p.L + i / D) * p.Hv * D + (size_t)h * D + i % D] = (__bf16)nan;
    if (p.s_final && run.last)
      for (int i = tid; i < D * D; i += 64 * NW) p.s_final[((size_t)b * p.Hv + h) * D * D + i] = nan;
    return;
  }

  // Chunks entirely past the row's length (right pads: beta' = g' = 0) leave the state unchanged
  // and give O = diag(rq) Q S: only their Q tile (and gate rows) is staged and only the output
  // products run, after the other chunks (three at a time without the fused norm).
  int len_b = p.lengths ? p.lengths[b] : p.L;
  len_b = len_b < 0 ? 0 : (len_b > p.L ? p.L : len_b);
  const uint32_t kq_row = (uint32_t)p.Hk * D * 2, vo_row = (uint32_t)p.Hv * D * 2;
  const size_t kq_base = (size_t)b * p.L * p.Hk * D, vo_base = ((size_t)b * p.L * p.Hv + h) * D;
  const uint32_t vo_bytes = p.L > 0 ? (uint32_t)(p.L - 1) * vo_row + D * 2 : 0;
  const i32x4 rk = rsrc_words(kg + kq_base, (uint32_t)p.L * kq_row);
  const i32x4 rq = rsrc_words(qg + kq_base, (uint32_t)p.L * kq_row);
  const i32x4 rv = rsrc_words(vg + vo_base, vo_bytes);
  const i32x4 rr = rsrc_words(reinterpret_cast<const unsigned char*>(p.ws) + ((size_t)b * p.Hv + h) * p.NC * kRecB,
                              (uint32_t)p.NC * kRecB);
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(og + vo_base, vo_bytes);
  // fused gated RMSNorm (outputs only): gate z in o's layout, weights of this lane's columns
  const i32x4 rz = rsrc_words(kFuse ? reinterpret_cast<const __bf16*>(p.z) + vo_base : nullptr, kFuse ? vo_bytes : 0u);
  f4 nw[NSL];
#pragma unroll
  for (int sl = 0; sl < NSL; ++sl)
    nw[sl] = kFuse ? *reinterpret_cast<const f4*>(p.norm_w + seg_col<kOut>(w, sl) + 4 * G) : f4_splat(0.f);

  // This wave's share of chunk c: K (and Q, and the fused norm's gate rows) and V rows
  // R w .. R w + R - 1 (R = 64 / NW, loads of four rows each) and the 1 KiB record blocks w,
  // w + NW, ... (the Tb blocks 0..5 and the scalar blocks 6, 7); `parts` selects which of them.
  constexpr int R = C / NW;
  enum : int { kStK = 1, kStV = 2, kStRec = 4, kStQ = 8, kStAll = 15 };   // kStQ: Q and gate rows
  auto issue = [&](int c, int parts) {
    unsigned char* Bf = lds + (c & 1) * Cfg::kBuf;
    const uint32_t t0 = (uint32_t)c * C;
#pragma unroll
    for (int m = 0; m < R / 4; ++m) {
      const int r = R * w + 4 * m + (lane >> 4), pos = lane & 15;
      const uint32_t kq = (t0 + r) * kq_row + (uint32_t)kh * D * 2 + 16 * (pos ^ swz_f(r));
      if (parts & kStK) dma16(rk, kq, Bf + Cfg::kK + (R * w + 4 * m) * 256);
      if (kOut && (parts & kStQ)) dma16(rq, kq, Bf + Cfg::kQ + (R * w + 4 * m) * 256);
      if (parts & kStV) dma16(rv, (t0 + r) * vo_row + 16 * (pos ^ (2 * (r & 7))), Bf + Cfg::kV + (R * w + 4 * m) * 256);
      if (kFuse && (parts & kStQ))
        dma16(rz, (t0 + r) * vo_row + 16 * (pos ^ (r & 15)), Bf + Cfg::kZ + (R * w + 4 * m) * 256);
    }
    if (parts & kStRec) {
      const uint32_t rec = (uint32_t)c * kRecB + 16 * lane;
#pragma unroll
      for (int i0 = 0; i0 < kRecBlocks; i0 += NW) {
        const int i = i0 + w;
        if (i < kRecBlocks) dma16(rr, rec + 1024 * i, Bf + Cfg::kRec + 1024 * i);   // wave-uniform
      }
    }
  };
  // a chunk past the row's length (outputs with the fused norm): its Q rows and gate rows
  auto issue_q = [&](int c) {
    unsigned char* Bf = lds + (c & 1) * Cfg::kBuf;
    const uint32_t t0 = (uint32_t)c * C;
#pragma unroll
    for (int m = 0; m < R / 4; ++m) {
      const int r = R * w + 4 * m + (lane >> 4), pos = lane & 15;
      const uint32_t kq = (t0 + r) * kq_row + (uint32_t)kh * D * 2 + 16 * (pos ^ swz_f(r));
      if constexpr (kOut) dma16(rq, kq, Bf + Cfg::kQ + (R * w + 4 * m) * 256);
      if (kFuse) dma16(rz, (t0 + r) * vo_row + 16 * (pos ^ (r & 15)), Bf + Cfg::kZ + (R * w + 4 * m) * 256);
    }
  };
  // Q tiles of the pad chunks c0 .. c0 + kPadGroup - 1 (those before c_end) into the Q, K and V
  // regions of buffer bi (outputs without the fused norm)
  auto issue_qg = [&](int c0, int bi) {
    unsigned char* Bf = lds + bi * Cfg::kBuf;
#pragma unroll
    for (int i = 0; i < kPadGroup; ++i) {
      if (c0 + i >= c_end) break;   // uniform
      const int region = i == 0 ? Cfg::kQ : (i == 1 ? Cfg::kK : Cfg::kV);
      const uint32_t t0 = (uint32_t)(c0 + i) * C;
#pragma unroll
      for (int m = 0; m < R / 4; ++m) {
        const int r = R * w + 4 * m + (lane >> 4), pos = lane & 15;
        const uint32_t kq = (t0 + r) * kq_row + (uint32_t)kh * D * 2 + 16 * (pos ^ swz_f(r));
        if constexpr (kOut) dma16(rq, kq, Bf + region + (R * w + 4 * m) * 256);
      }
    }
  };
  // chunks c_begin .. c_mid - 1 hold valid tokens; c_mid .. c_end - 1 are right pads
  const int c_mid = min(max((len_b + C - 1) / C, c_begin), c_end);

  // ---- state entering the segment
  f4 S[NSL][4][2];
  {
    const float* src = nullptr;
    size_t pitch = 0;
    if (run.src_kind == 1) {
      src = run.src;
      pitch = 2 * D;
    } else if (run.src_kind == 2 && p.s0) {
      src = p.s0 + ((size_t)srow * p.Hv + h) * D * D;
      pitch = D;
    }
    if (src) {
#pragma unroll
      for (int sl = 0; sl < NSL; ++sl)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              S[sl][kb][s2][i] = src[(32 * kb + 8 * G + 4 * s2 + i) * pitch + seg_col<kOut>(w, sl) + n16];
    } else {
#pragma unroll
      for (int sl = 0; sl < NSL; ++sl)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int i = 0; i < 4; ++i)   // zero, or e_k for the identity columns
              S[sl][kb][s2][i] = (seg_col<kOut>(w, sl) + n16 - D == 32 * kb + 8 * G + 4 * s2 + i) ? 1.f : 0.f;
    }
  }

  if constexpr (kWin) {
    // Every chunk of a window holds valid tokens (the plan makes sure): no pads, no Q, no outputs.
    constexpr int kParts = kStK | kStV | kStRec;
    if (c_begin < c_end) issue(c_begin, kParts);
    for (int c = c_begin; c < c_end; ++c) {
      wait_and_barrier<0>();   // chunk c has landed; every wave is done with chunk c - 1's buffer
      if (c + 1 < c_end) issue(c + 1, kParts);
      const unsigned char* Bf = lds + (c & 1) * Cfg::kBuf;
      const unsigned char* Kt = Bf + Cfg::kK;
      const float* sc = reinterpret_cast<const float*>(Bf + Cfg::kRec + kScOff);
      // X = K S, R = V - diag(a) X, Delta = Tb R (lower-triangular blocks only); the window starts
      // from zero, so its first chunk has X = 0 (uniform branch)
      const bool first = c == c_begin;
      f4 X[NSL][4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int sl = 0; sl < NSL; ++sl) X[sl][mt] = f4_splat(0.f);
      if (!first) {
        bf16x8 Sop[NSL][4];
#pragma unroll
        for (int sl = 0; sl < NSL; ++sl)
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) Sop[sl][kb] = pack8(S[sl][kb][0], S[sl][kb][1]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            const bf16x8 kf = lds16(Kt + swz(16 * mt + n16, 4 * kb + G));
#pragma unroll
            for (int sl = 0; sl < NSL; ++sl) X[sl][mt] = mfma(kf, Sop[sl][kb], X[sl][mt]);
          }
      }
      bf16x8 Rop[NSL][2];
#pragma unroll
      for (int sl = 0; sl < NSL; ++sl) {
        f4 R[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          R[mt] = v_col4(Bf + Cfg::kV, 16 * mt + 4 * G, seg_col<kOut>(w, sl), n16) -
                  *reinterpret_cast<const f4*>(sc + 16 * mt + 4 * G) * X[sl][mt];
        Rop[sl][0] = pack8(R[0], R[1]);
        Rop[sl][1] = pack8(R[2], R[3]);
      }
      f4 Dl[NSL][4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int sl = 0; sl < NSL; ++sl) Dl[sl][mt] = f4_splat(0.f);
#pragma unroll
        for (int kb2 = 0; kb2 <= (mt >> 1); ++kb2) {
          const bf16x8 tf = lds16(Bf + Cfg::kRec + 1024 * frag_block(mt, kb2) + 16 * lane);
#pragma unroll
          for (int sl = 0; sl < NSL; ++sl) Dl[sl][mt] = mfma(tf, Rop[sl][kb2], Dl[sl][mt]);
        }
        const f4 d4 = *reinterpret_cast<const f4*>(sc + kBfD * C + 16 * mt + 4 * G);
#pragma unroll
        for (int sl = 0; sl < NSL; ++sl) Dl[sl][mt] *= d4;   // diag(d) Delta
      }
      bf16x8 Ddop[NSL][2];   // the operand K^T diag(d) Delta is formed from
#pragma unroll
      for (int sl = 0; sl < NSL; ++sl) {
        Ddop[sl][0] = pack8(Dl[sl][0], Dl[sl][1]);
        Ddop[sl][1] = pack8(Dl[sl][2], Dl[sl][3]);
      }
      // S <- e^{gamma_63} S + K^T diag(d) Delta (S = 0 before the first chunk)
      const float egc = first ? 0.f : __builtin_amdgcn_exp2f(sc[kBfGam2 * C + C - 1]);   // e^{gamma_63}
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
          for (int sl = 0; sl < NSL; ++sl) S[sl][kb][s2] *= egc;
#pragma unroll
          for (int kb2 = 0; kb2 < 2; ++kb2) {
            const bf16x8 kt = kt_frag(Kt, kb, s2, kb2, G, n16);
#pragma unroll
            for (int sl = 0; sl < NSL; ++sl) S[sl][kb][s2] = mfma(kt, Ddop[sl][kb2], S[sl][kb][s2]);
          }
        }
    }
    __builtin_amdgcn_s_waitcnt(0);   // no load into LDS may still be in flight when the workgroup ends
    float ss = 0.f;
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float x = S[sl][kb][s2][i];
            ss += x * x;
            run.end_b[(32 * kb + 8 * G + 4 * s2 + i) * 2 * D + seg_col<kOut>(w, sl) + n16] = x;
          }
    ss = wave_sum(ss);
    if (lane == 0) run.n2[w] = ss;
    return;
  }

  // Output tiles of a chunk and, with the fused gated RMSNorm, its gate values. The norm needs each
  // token's sum of squares over all 128 columns, i.e. over all waves: every wave leaves its partial
  // sums in LDS (two buffers, by chunk parity) and normalises and stores chunk c - 1 during chunk c,
  // after chunk c + 1's loads are issued and before the P' barrier, so the fusion adds no barrier.
  // Ot: the chunk's outputs; sz: w silu(z) of the same lanes' elements, formed from the gate rows
  // staged with the chunk while the chunk computes.
  f4 Ot[4][NSL], sz[4][NSL];
  float* part = reinterpret_cast<float*>(lds + Cfg::kPart);   // [2][NW][64]
  auto store_tile = [&](int c, int mt) {
    const uint32_t orow = ((uint32_t)c * C + 16 * mt + n16) * vo_row;
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) {
      const bf16x4 ob = {(__bf16)Ot[mt][sl][0], (__bf16)Ot[mt][sl][1], (__bf16)Ot[mt][sl][2], (__bf16)Ot[mt][sl][3]};
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, ob), ro, orow + 2 * (seg_col<kOut>(w, sl) + 4 * G), 0, 0);
    }
  };
  auto store_o = [&](int c) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) store_tile(c, mt);
  };
  auto finish_norm = [&](int c) {   // w o / sqrt(mean(o^2) + eps) silu(z) for chunk c, then store
    const float* pp = part + (c & 1) * NW * C;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      float ss = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) ss += pp[ww * C + 16 * mt + n16];
      const float r = __builtin_amdgcn_rsqf(ss * (1.0f / D) + p.eps);
#pragma unroll
      for (int sl = 0; sl < NSL; ++sl) Ot[mt][sl] *= sz[mt][sl] * r;
    }
    store_o(c);
  };

  constexpr bool fuse = kFuse;
  if (c_begin < c_mid)
    issue(c_begin, kStAll);
  else if (c_begin < c_end && fuse)
    issue_q(c_begin);
  else if (c_begin < c_end)
    issue_qg(c_begin, c_begin & 1);
  wait_and_barrier<0>();
  // The same wait as a builtin the compiler sees: the entering-state loads are then known complete,
  // so it places no wait for them inside the loop (where it would also stall on the next chunk's
  // loads into LDS).
  __builtin_amdgcn_s_waitcnt(0);

  float* rqs = reinterpret_cast<float*>(lds + Cfg::kRq);   // |q_t|^2, t = 0..63 (outputs)
  auto put_qnorms = [&](int mt, const f4& qq) {   // lane (n16, G) holds rows 4G .. 4G + 3 of column n16
    if ((n16 >> 2) == G) {
      const int e = n16 & 3;
      rqs[16 * mt + n16] = e == 0 ? qq[0] : e == 1 ? qq[1] : e == 2 ? qq[2] : qq[3];
    }
  };
  // Row t of O is finished by the q norm factor rq_t; with the fused norm the wave's partial sum
  // of squares of the row goes to LDS and w silu(z) of the lane's elements is formed from the
  // gate rows staged with the chunk.
  auto finish_rows = [&](int mt, int c, const unsigned char* Bf) {
    const float rq = __builtin_amdgcn_rsqf(rqs[16 * mt + n16] + 1e-6f) * 0.08838834764831845f;   // * 128^-1/2
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) Ot[mt][sl] *= rq;
    if (fuse) {
      float ss = 0.f;
#pragma unroll
      for (int sl = 0; sl < NSL; ++sl)
#pragma unroll
        for (int i = 0; i < 4; ++i) ss += Ot[mt][sl][i] * Ot[mt][sl][i];
      ss += __shfl_xor(ss, 16);
      ss += __shfl_xor(ss, 32);
      if (G == 0) part[(c & 1) * NW * C + w * C + 16 * mt + n16] = ss;
      const unsigned char* Zb = Bf + Cfg::kZ;
#pragma unroll
      for (int sl = 0; sl < NSL; ++sl) {
        const int zrow = 16 * mt + n16, zcol = seg_col<kOut>(w, sl) + 4 * G;
        const bf16x4 zb = *reinterpret_cast<const bf16x4*>(Zb + swz_z(zrow, zcol >> 3) + 2 * (zcol & 7));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float zf = (float)zb[i];
          sz[mt][sl][i] = nw[sl][i] * zf * silu_gate(zf);
        }
      }
    }
  };

  for (int c = c_begin; c < c_mid; ++c) {
    // chunk c has landed for every wave, every wave is done with chunk c - 1's buffer, and (fused
    // norm) chunk c - 1's gate rows and partial sums are in LDS. Vector-memory operations issued
    // after chunk c's loads: the output stores of chunk c - 1 (with the fused norm: of chunk c - 2,
    // none in the first iteration).
    if (fuse && c <= c_begin + 1)
      wait_and_barrier<0>();
    else
      wait_and_barrier<Cfg::kStores>();
    if (kOut && c == run.cert_chunk) {   // ||S||_F^2 of the state entering chunk c, this wave's part
      float ss = 0.f;
#pragma unroll
      for (int sl = 0; sl < NSL; ++sl)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int i = 0; i < 4; ++i) ss += S[sl][kb][s2][i] * S[sl][kb][s2][i];
      ss = wave_sum(ss);
      if (lane == 0) run.cert[w] = ss;
    }
    // The next chunk's staging. The output pass spreads it over the iteration: K here, Q after the
    // P' formation, V after X, the record before the P' barrier. Issued all at once, these loads
    // hold up this chunk's first LDS reads and products (about a tenth of the pass at the long
    // prefill). The transitions, which form no P', issue it all here.
    if (c + 1 < c_mid)
      issue(c + 1, kOut ? kStK : kStAll);
    else if (kOut && c + 1 < c_end && fuse)
      issue_q(c + 1);
    else if (kOut && c + 1 < c_end)
      issue_qg(c + 1, (c + 1) & 1);
    const bool stage_next = kOut && c + 1 < c_mid;

    const unsigned char* Bf = lds + (c & 1) * Cfg::kBuf;
    const unsigned char* Kt = Bf + Cfg::kK;
    const unsigned char* Vt = Bf + Cfg::kV;
    const unsigned char* Rc = Bf + Cfg::kRec;
    const float* sc = reinterpret_cast<const float*>(Rc + kScOff);

    // P' of this chunk (outputs): the waves form its six operand blocks (token tile mt, key block
    // kb2; block i by wave i mod NW) from the staged tiles as the tile pair K Q^T (whose
    // accumulator layout is the operand layout of P'), scaled by rk_i 2^{min(gamma2_t - gamma2_i, 0)}
    // on i <= t and zero above the diagonal; read after the barrier that precedes the output
    // products. The q norm of token t,
    // rq_t = (|q_t|^2 + 1e-6)^-1/2 128^-1/2 (model page model.py, _l2norm), is a factor of both
    // output terms of row t (O = diag(rq) (diag(e^gamma) Q S + P' Delta)), so it is applied to the
    // finished row. Its sum of squares is the diagonal of the token tile's Q Q^T, which waves 6 and 7
    // (no P' block) form on MFMA, two tiles each, and leave in LDS.
    if constexpr (kOut) {
      const unsigned char* Qt = Bf + Cfg::kQ;
      // one block each for waves 0..5
      for (int blk = w; blk < w + 1 && blk < kFragBlocks; ++blk) {
        const int mt = block_tile(blk), kb2 = block_kb(blk);
        f4 pt[2] = {f4_splat(0.f), f4_splat(0.f)};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const bf16x8 qf = lds16(Qt + swz(16 * mt + n16, 4 * kb + G));
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) pt[s2] = mfma(lds16(Kt + swz(32 * kb2 + 16 * s2 + n16, 4 * kb + G)), qf, pt[s2]);
        }
        const int t = 16 * mt + n16;
        const float gt = sc[kBfGam2 * C + t];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const int i0 = 32 * kb2 + 16 * s2 + 4 * G;
          const f4 gi = *reinterpret_cast<const f4*>(sc + kBfGam2 * C + i0);
          const f4 ri = *reinterpret_cast<const f4*>(sc + kBfRk * C + i0);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float x = ri[e] * __builtin_amdgcn_exp2f(fminf(gt - gi[e], 0.f)) * pt[s2][e];
            pt[s2][e] = (i0 + e <= t) ? x : 0.f;
          }
        }
        *reinterpret_cast<bf16x8*>(lds + Cfg::kP + 1024 * blk + 16 * lane) = pack8(pt[0], pt[1]);
      }
      // waves 6 and 7, which form no P' block, form the Q Q^T of two token tiles each: its diagonal
      // is |q_t|^2
      if (w >= kFragBlocks) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int mt = 2 * (w - kFragBlocks) + h2;
          f4 qq = f4_splat(0.f);
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            const bf16x8 qf = lds16(Qt + swz(16 * mt + n16, 4 * kb + G));
            qq = mfma(qf, qf, qq);
          }
          put_qnorms(mt, qq);
        }
      }
    }

    bf16x8 Sop[NSL][4];
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) Sop[sl][kb] = pack8(S[sl][kb][0], S[sl][kb][1]);

    if (stage_next) issue(c + 1, kStQ);

    // X = K S
    f4 X[NSL][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int sl = 0; sl < NSL; ++sl) X[sl][mt] = f4_splat(0.f);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const bf16x8 kf = lds16(Kt + swz(16 * mt + n16, 4 * kb + G));
#pragma unroll
        for (int sl = 0; sl < NSL; ++sl) X[sl][mt] = mfma(kf, Sop[sl][kb], X[sl][mt]);
      }
    }
    if (stage_next) issue(c + 1, kStV);
    // R = V - diag(a) X  (zero values for the identity columns)
    bf16x8 Rop[NSL][2];
    {
      f4 a4[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) a4[mt] = *reinterpret_cast<const f4*>(sc + 16 * mt + 4 * G);
#pragma unroll
      for (int sl = 0; sl < NSL; ++sl) {
        const bool has_v = seg_has_v<kOut>(sl);   // compile-time after unrolling
        f4 R[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          R[mt] = -a4[mt] * X[sl][mt];
          if (has_v) R[mt] += v_col4(Vt, 16 * mt + 4 * G, seg_col<kOut>(w, sl), n16);
        }
        Rop[sl][0] = pack8(R[0], R[1]);
        Rop[sl][1] = pack8(R[2], R[3]);
      }
    }
    // Delta = Tb R (lower-triangular blocks only)
    f4 Dl[NSL][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int sl = 0; sl < NSL; ++sl) Dl[sl][mt] = f4_splat(0.f);
#pragma unroll
      for (int kb2 = 0; kb2 <= (mt >> 1); ++kb2) {
        const bf16x8 tf = lds16(Rc + 1024 * frag_block(mt, kb2) + 16 * lane);
#pragma unroll
        for (int sl = 0; sl < NSL; ++sl) Dl[sl][mt] = mfma(tf, Rop[sl][kb2], Dl[sl][mt]);
      }
    }
    bf16x8 Ddop[NSL][2];
    {
      f4 d4[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) d4[mt] = *reinterpret_cast<const f4*>(sc + kBfD * C + 16 * mt + 4 * G);
#pragma unroll
      for (int sl = 0; sl < NSL; ++sl) {
        Ddop[sl][0] = pack8(Dl[sl][0] * d4[0], Dl[sl][1] * d4[1]);
        Ddop[sl][1] = pack8(Dl[sl][2] * d4[2], Dl[sl][3] * d4[3]);
      }
    }
    // O^T = diag(c) (S^T Q^T) + Delta^T P^T: the accumulator lane (token n16, G) holds the four
    // consecutive columns 4G .. 4G + 3 of one token, stored as one 8-byte write.
    if constexpr (kOut) {
      if (stage_next) issue(c + 1, kStRec);
      // the norm of chunk c - 1 and its stores: after all of the next chunk's loads (so that the
      // wait that opens the next chunk leaves only these stores in flight), before this chunk's
      // output products take over Ot
      if (fuse && c > c_begin) finish_norm(c - 1);
      lds_barrier();   // P' is complete
      const unsigned char* Qt = Bf + Cfg::kQ;
      bf16x8 Dop[NSL][2];
#pragma unroll
      for (int sl = 0; sl < NSL; ++sl) {
        Dop[sl][0] = pack8(Dl[sl][0], Dl[sl][1]);
        Dop[sl][1] = pack8(Dl[sl][2], Dl[sl][3]);
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int sl = 0; sl < NSL; ++sl) Ot[mt][sl] = f4_splat(0.f);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const bf16x8 qf = lds16(Qt + swz(16 * mt + n16, 4 * kb + G));
#pragma unroll
          for (int sl = 0; sl < NSL; ++sl) Ot[mt][sl] = mfma(Sop[sl][kb], qf, Ot[mt][sl]);
        }
        const float eg = __builtin_amdgcn_exp2f(sc[kBfGam2 * C + 16 * mt + n16]);   // e^gamma_t
#pragma unroll
        for (int sl = 0; sl < NSL; ++sl) Ot[mt][sl] *= eg;
#pragma unroll
        for (int kb2 = 0; kb2 <= (mt >> 1); ++kb2) {
          const bf16x8 pf = lds16(lds + Cfg::kP + 1024 * frag_block(mt, kb2) + 16 * lane);
#pragma unroll
          for (int sl = 0; sl < NSL; ++sl) Ot[mt][sl] = mfma(Dop[sl][kb2], pf, Ot[mt][sl]);
        }
        finish_rows(mt, c, Bf);
        if (!fuse) store_tile(c, mt);   // each token tile as soon as it is done
      }
    }
    // S <- e^{gamma_63} S + K^T diag(d) Delta
    const float egc = __builtin_amdgcn_exp2f(sc[kBfGam2 * C + C - 1]);   // e^{gamma_63}
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
        for (int sl = 0; sl < NSL; ++sl) S[sl][kb][s2] *= egc;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
          const bf16x8 kt = kt_frag(Kt, kb, s2, kb2, G, n16);
#pragma unroll
          for (int sl = 0; sl < NSL; ++sl) S[sl][kb][s2] = mfma(kt, Ddop[sl][kb2], S[sl][kb][s2]);
        }
      }
  }
  if constexpr (kOut) {
    // Right pads (beta' = g' = 0): the state stays as it is and O = diag(rq) Q S, the only products.
    bf16x8 Sop[NSL][4];
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) Sop[sl][kb] = pack8(S[sl][kb][0], S[sl][kb][1]);
    if (!fuse) {
      // groups of kPadGroup chunks, group g in buffer (c_mid + g) & 1; after a group's loads come
      // the stores of the chunk or group before it (none when the segment starts in the pads: its
      // first group was waited for before the main loop)
      float* rqg = reinterpret_cast<float*>(lds + Cfg::kRq);   // [kPadGroup][64]: |q_t|^2
      for (int c0 = c_mid, g = 0; c0 < c_end; c0 += kPadGroup, ++g) {
        const int bi = (c_mid + g) & 1, n = min(kPadGroup, c_end - c0);
        if (g == 0)
          wait_and_barrier<Cfg::kStores>();
        else
          wait_and_barrier<kPadGroup * Cfg::kStores>();
        if (c0 + kPadGroup < c_end) issue_qg(c0 + kPadGroup, bi ^ 1);
        const unsigned char* Bq = lds + bi * Cfg::kBuf;
        for (int pr = w; pr < 4 * n; pr += NW) {   // q norms of (chunk pr / 4, token tile pr % 4)
          const int i = pr >> 2, mt = pr & 3;
          const unsigned char* Qt = Bq + (i == 0 ? Cfg::kQ : (i == 1 ? Cfg::kK : Cfg::kV));
          f4 qq = f4_splat(0.f);
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            const bf16x8 qf = lds16(Qt + swz(16 * mt + n16, 4 * kb + G));
            qq = mfma(qf, qf, qq);
          }
          if ((n16 >> 2) == G) {
            const int e = n16 & 3;
            rqg[64 * i + 16 * mt + n16] = e == 0 ? qq[0] : e == 1 ? qq[1] : e == 2 ? qq[2] : qq[3];
          }
        }
        lds_barrier();
        for (int i = 0; i < n; ++i) {
          const unsigned char* Qt = Bq + (i == 0 ? Cfg::kQ : (i == 1 ? Cfg::kK : Cfg::kV));
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
            for (int sl = 0; sl < NSL; ++sl) Ot[mt][sl] = f4_splat(0.f);
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
              const bf16x8 qf = lds16(Qt + swz(16 * mt + n16, 4 * kb + G));
#pragma unroll
              for (int sl = 0; sl < NSL; ++sl) Ot[mt][sl] = mfma(Sop[sl][kb], qf, Ot[mt][sl]);
            }
            const float rqv = __builtin_amdgcn_rsqf(rqg[64 * i + 16 * mt + n16] + 1e-6f) * 0.08838834764831845f;
#pragma unroll
            for (int sl = 0; sl < NSL; ++sl) Ot[mt][sl] *= rqv;
            store_tile(c0 + i, mt);
          }
        }
      }
    }
    for (int c = c_mid; fuse && c < c_end; ++c) {
      wait_and_barrier<0>();
      if (c + 1 < c_end) issue_q(c + 1);
      if (c > c_begin) finish_norm(c - 1);
      const unsigned char* Qt = lds + (c & 1) * Cfg::kBuf + Cfg::kQ;
      if (w < 4) {   // q norms of token tile w
        f4 qq = f4_splat(0.f);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const bf16x8 qf = lds16(Qt + swz(16 * w + n16, 4 * kb + G));
          qq = mfma(qf, qf, qq);
        }
        put_qnorms(w, qq);
      }
      lds_barrier();
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int sl = 0; sl < NSL; ++sl) Ot[mt][sl] = f4_splat(0.f);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const bf16x8 qf = lds16(Qt + swz(16 * mt + n16, 4 * kb + G));
#pragma unroll
          for (int sl = 0; sl < NSL; ++sl) Ot[mt][sl] = mfma(Sop[sl][kb], qf, Ot[mt][sl]);
        }
        finish_rows(mt, c, lds + (c & 1) * Cfg::kBuf);
      }
    }
  }
  if (fuse && c_end > c_begin) {   // the last chunk's norm: its partial sums, then store
    lds_barrier();
    finish_norm(c_end - 1);
  }
  __builtin_amdgcn_s_waitcnt(0);   // no load into LDS may still be in flight when the workgroup ends

  // ---- end state
  if (kOut && !(p.s_final && run.last)) return;
#pragma unroll
  for (int sl = 0; sl < NSL; ++sl) {
    float* dst;
    size_t pitch;
    if constexpr (kOut) {
      dst = p.s_final + ((size_t)b * p.Hv + h) * D * D;
      pitch = D;
    } else {
      dst = seg_has_v<kOut>(sl) ? run.end_b : run.end_m;   // B into slot j + 1, M into slot j
      if (!dst) continue;
      pitch = 2 * D;
    }
    const int col = seg_col<kOut>(w, sl) + n16;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[(32 * kb + 8 * G + 4 * s2 + i) * pitch + col] = S[sl][kb][s2][i];
  }
}

__device__ __forceinline__ size_t head_index(const ScanParams& p, int b, int h) { return (size_t)b * p.Hv + h; }
__device__ __forceinline__ float* slot_ptr(const ScanParams& p, int b, int h, int j) {
  return p.seg + (head_index(p, b, h) * p.P + j) * kSlotFloats;
}

// The certificate of a truncated (row, head): eps_j = 2^{l2_j} (||S(c_j - W_j)||_F + eps_{j-1}) <=
// 2^-24 ||S~_j||_F at every boundary j (the norms from the certificate parts the output and transition
// passes left). Called by the whole workgroup: thread j - 1 loads boundary j's parts (all at once), thread
// 0 runs the recurrence over them from LDS. `scratch` holds 3 P floats (P <= 256). Returns 0 for a
// (row, head) on the exact path, 1 when the certificate holds, 2 when it fails (NaN or infinity fail).
static_assert(kSegTargetWorkgroups < 64 * SegCfg<true>::NW, "one boundary per thread: P <= kSegTargetWorkgroups");
__device__ __forceinline__ int certificate_status(const ScanParams& p, size_t hb, float* scratch) {
  // every load first (one memory round trip): whether the (row, head) is truncated, and thread t's
  // boundary t + 1 (P <= 256 < threads)
  const int t = threadIdx.x, jb = t + 1;
  const int truncated = p.plan[hb + 1].trunc;
  float l2 = 0.f, n1 = 0.f, n2 = 0.f;
  if (jb < p.P) {
    const float* ct = p.cert + (hb + jb) * kCertFloats;
    l2 = p.plan[hb + jb].l2;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      n1 += ct[i];
      n2 += ct[8 + i];
    }
    scratch[3 * jb] = __builtin_amdgcn_exp2f(l2);
    scratch[3 * jb + 1] = sqrtf(n1);
    scratch[3 * jb + 2] = sqrtf(n2);
  }
  __syncthreads();
  if (!truncated) return 0;
  int ok = 1;
  if (t == 0) {
    float eps = 0.f;
    for (int j = 1; j < p.P && ok; ++j) {
      eps = scratch[3 * j] * (scratch[3 * j + 1] + eps);
      ok = eps <= kCertRel * scratch[3 * j + 2];
    }
    scratch[0] = ok ? 1.f : 0.f;
  }
  __syncthreads();
  return scratch[0] != 0.f ? 1 : 2;
}


// Outputs: one workgroup per (row, segment, value head), heads fastest; kFuse when p.z is set.
template <bool kFuse>
__global__ __launch_bounds__(64 * SegCfg<true>::NW) void gdr_scan_bf16(ScanParams p) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[SegCfg<true>::kLds];
  // With a row order (rows of unequal lengths, no segments) the workgroups take the rows longest
  // first, in dispatch order, so that the long rows start early on every XCD; otherwise the
  // workgroups of a (row, head) run side by side on one XCD.
  const int lam = p.row_order ? (int)blockIdx.x : xcd_remap(blockIdx.x, gridDim.x);
  const int h = lam % p.Hv, j = (lam / p.Hv) % p.P;
  const int b = p.row_order ? p.row_order[lam / (p.Hv * p.P)] : lam / (p.Hv * p.P);
  SegRun run{};
  run.c_begin = j * p.Ls;
  run.c_end = min(run.c_begin + p.Ls, p.NC);
  // with segments, the combine has put every entering state in its slot (the first one only with s0)
  run.src_kind = p.P > 1 && (j > 0 || p.s0) ? 1 : 2;
  run.src = run.src_kind == 1 ? slot_ptr(p, b, h, j) : nullptr;
  run.last = j == p.P - 1;
  run.cert_chunk = -1;
  if (p.P > 1 && p.trunc && j + 1 < p.P) {
    const PlanEntry e = p.plan[head_index(p, b, h) * p.P + j + 1];
    if (e.trunc) {   // the window of boundary j + 1 starts inside this segment
      run.cert_chunk = (j + 1) * p.Ls - e.W;
      run.cert = p.cert + (head_index(p, b, h) * p.P + j + 1) * kCertFloats;
    }
  }
  seg_body<true, false, kFuse>(p, lds, b, h, run);
}

// ---- Output pass over a pair of value heads (bf16, Hv / Hk even, no fused norm; used without segments
// when the pairs fill the GPU, see use_pair_pass)
// Value heads 2 hp and 2 hp + 1 share one key head, so one workgroup runs both: the K and Q tiles are
// staged once, and each wave holds two 16-column slices (32 columns of one head: waves 0-3 head 2 hp,
// waves 4-7 head 2 hp + 1), so that every K, K^T and Q fragment it reads from LDS feeds two products.
// Per head that halves the LDS reads of the single-head pass above, whose time they bound. Every column
// runs the single-head pass's arithmetic in the same order (the same results, bit for bit).
// A wave's V columns are staged by that wave alone, into an LDS area of its own with one buffer: the
// next chunk's are loaded once this chunk's R has been formed, and no other wave waits for them.
struct PairCfg {
  static constexpr int NW = 8, NSL = 2;
  static constexpr int kK = 0, kQ = kBufK, kRec = 2 * kBufK;   // head e's record at kRec + e kRecB
  static constexpr int kBuf = kRec + 2 * kRecB;                  // one chunk: 48 KiB
  static constexpr int kVWave = C * 64;                          // a wave's V: 64 tokens x 32 columns
  static constexpr int kV = 2 * kBuf;                            // wave w's V at kV + w kVWave
  static constexpr int kP = kV + NW * kVWave;                    // head e's P' at kP + e kFragBlocks KiB
  static constexpr int kRq = kP + 2 * kFragBlocks * 1024;        // |q_t|^2 (kPadGroup chunks in the pads)
  static constexpr int kLds = kRq + kPadGroup * C * 4;
  static constexpr int kStores = 4 * NSL;                        // output stores per wave per chunk
};
static_assert(PairCfg::kLds <= 160 * 1024, "one workgroup's LDS");
static_assert(2 * kRecB == kBufK, "the two records of a chunk hold one Q tile in the pads");

// A wave's V tile in the pair pass: row t (64 bytes: the wave's two 16-column slices) at 64 t, its
// halves swapped when bit 2 of t is set, so that the eight rows one transposing read touches fill
// all 64 banks once.
__device__ __forceinline__ int swz_pv(int row, int half) { return row * 64 + 32 * (half ^ ((row >> 2) & 1)); }

struct PairRun {
  int c_begin, c_end;
  int src_kind;            // as SegRun::src_kind, for both heads
  const float* src[2];     // head e's entering state (segment slot, pitch 2D)
  bool last;               // the run ends the row: s_final is written
  int cert_chunk[2];       // head e: chunk at whose top ||S||_F^2 goes to cert[e] (-1: none)
  float* cert[2];
};

__device__ __forceinline__ void pair_body(const ScanParams& p, unsigned char* lds, int b, int hp, const PairRun& run) {
  using Cfg = PairCfg;
  constexpr int NSL = Cfg::NSL, NW = Cfg::NW;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15, G = lane >> 4;
  const int e = w >> 2, h = 2 * hp + e;           // this wave's head
  const int kh = (2 * hp) / (p.Hv / p.Hk);        // the pair's key head
  const int col0 = 32 * (w & 3);                  // the wave's first column of head h
  const int c_begin = run.c_begin, c_end = run.c_end;
  const __bf16* qg = reinterpret_cast<const __bf16*>(p.q);
  const __bf16* kg = reinterpret_cast<const __bf16*>(p.k);
  const __bf16* vg = reinterpret_cast<const __bf16*>(p.v);
  __bf16* og = reinterpret_cast<__bf16*>(p.o);

  int srow = 0;
  if (row_is_bad(p, b, srow)) {   // NaN outputs for both heads
    const float nan = __builtin_nanf("");
    const int t_end = min(c_end * C, p.L);
    for (int i = c_begin * C * 2 * D + tid; i < t_end * 2 * D; i += 64 * NW) {
      const int t = i / (2 * D), r = i % (2 * D);
      og[((size_t)b * p.L + t) * p.Hv * D + (size_t)(2 * hp + r / D) * D + r % D] = (__bf16)nan;
    }
    if (p.s_final && run.last)
      for (int i = tid; i < 2 * D * D; i += 64 * NW) p.s_final[((size_t)b * p.Hv + 2 * hp) * D * D + i] = nan;
    return;
  }

  int len_b = p.lengths ? p.lengths[b] : p.L;
  len_b = len_b < 0 ? 0 : (len_b > p.L ? p.L : len_b);
  const uint32_t kq_row = (uint32_t)p.Hk * D * 2, vo_row = (uint32_t)p.Hv * D * 2;
  const size_t kq_base = (size_t)b * p.L * p.Hk * D, vo_base = ((size_t)b * p.L * p.Hv + h) * D;
  const uint32_t vo_bytes = p.L > 0 ? (uint32_t)(p.L - 1) * vo_row + D * 2 : 0;
  const i32x4 rk = rsrc_words(kg + kq_base, (uint32_t)p.L * kq_row);
  const i32x4 rq = rsrc_words(qg + kq_base, (uint32_t)p.L * kq_row);
  const i32x4 rv = rsrc_words(vg + vo_base, vo_bytes);   // this wave's head
  // both heads' records: head 2 hp + 1's follow head 2 hp's
  const i32x4 rr = rsrc_words(reinterpret_cast<const unsigned char*>(p.ws) + ((size_t)b * p.Hv + 2 * hp) * p.NC * kRecB,
                              (uint32_t)(2 * p.NC) * kRecB);
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(og + vo_base, vo_bytes);
  unsigned char* Vw = lds + Cfg::kV + w * Cfg::kVWave;

  // Chunk c's shared staging: K and Q rows 8 w .. 8 w + 7 (loads of four rows) and record blocks
  // w, w + 8 of the fourteen (head 2 hp's seven, then head 2 hp + 1's).
  constexpr int R = C / NW;
  enum : int { kStK = 1, kStQ = 2, kStRec = 4, kStAll = 7 };
  auto issue = [&](int c, int parts) {
    unsigned char* Bf = lds + (c & 1) * Cfg::kBuf;
    const uint32_t t0 = (uint32_t)c * C;
#pragma unroll
    for (int m = 0; m < R / 4; ++m) {
      const int r = R * w + 4 * m + (lane >> 4), pos = lane & 15;
      const uint32_t kq = (t0 + r) * kq_row + (uint32_t)kh * D * 2 + 16 * (pos ^ swz_f(r));
      if (parts & kStK) dma16(rk, kq, Bf + Cfg::kK + (R * w + 4 * m) * 256);
      if (parts & kStQ) dma16(rq, kq, Bf + Cfg::kQ + (R * w + 4 * m) * 256);
    }
    if (parts & kStRec) {
#pragma unroll
      for (int i0 = 0; i0 < 2 * kRecBlocks; i0 += NW) {
        const int i = i0 + w;
        if (i < 2 * kRecBlocks) {   // wave-uniform
          const int he = i >= kRecBlocks ? 1 : 0, blk = i - he * kRecBlocks;
          dma16(rr, ((uint32_t)he * p.NC + c) * kRecB + 1024 * blk + 16 * lane,
                Bf + Cfg::kRec + he * kRecB + 1024 * blk);
        }
      }
    }
  };
  // This wave's V columns of chunk c: four loads of 16 rows; lane l lands at byte 16 l of its load's
  // kilobyte, which swz_pv assigns to row 16 m + l / 4 and the piece computed here.
  auto issue_v = [&](int c) {
    const uint32_t t0 = (uint32_t)c * C;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int t = 16 * m + (lane >> 2), qp = lane & 3;
      const int pos = 2 * ((qp >> 1) ^ ((t >> 2) & 1)) + (qp & 1);
      dma16(rv, (t0 + t) * vo_row + 2 * col0 + 16 * pos, Vw + 1024 * m);
    }
  };
  // V[16 mt + 4G + i][col0 + 16 sl + n16], i = 0..3, from this wave's tile (as v_col4)
  auto v_cols = [&](int mt, int sl) {
    const int t = 16 * mt + 4 * G + (n16 >> 2);
    const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Vw + swz_pv(t, sl) + 8 * (n16 & 3)));
    const bf16x4 y = __builtin_bit_cast(bf16x4, x);
    return f4{(float)y[0], (float)y[1], (float)y[2], (float)y[3]};
  };
  // Q tiles of the pad chunks c0 .. c0 + kPadGroup - 1 (those before c_end) into the Q, K and record
  // regions of buffer bi
  auto issue_qg = [&](int c0, int bi) {
    unsigned char* Bf = lds + bi * Cfg::kBuf;
#pragma unroll
    for (int i = 0; i < kPadGroup; ++i) {
      if (c0 + i >= c_end) break;   // uniform
      const int region = i == 0 ? Cfg::kQ : (i == 1 ? Cfg::kK : Cfg::kRec);
      const uint32_t t0 = (uint32_t)(c0 + i) * C;
#pragma unroll
      for (int m = 0; m < R / 4; ++m) {
        const int r = R * w + 4 * m + (lane >> 4), pos = lane & 15;
        const uint32_t kq = (t0 + r) * kq_row + (uint32_t)kh * D * 2 + 16 * (pos ^ swz_f(r));
        dma16(rq, kq, Bf + region + (R * w + 4 * m) * 256);
      }
    }
  };
  const int c_mid = min(max((len_b + C - 1) / C, c_begin), c_end);

  // ---- state entering the segment (this wave's columns of head h)
  f4 S[NSL][4][2];
  {
    const float* src = nullptr;
    size_t pitch = 0;
    if (run.src_kind == 1) {
      src = e ? run.src[1] : run.src[0];
      pitch = 2 * D;
    } else if (run.src_kind == 2 && p.s0) {
      src = p.s0 + ((size_t)srow * p.Hv + h) * D * D;
      pitch = D;
    }
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            S[sl][kb][s2][i] = src ? src[(32 * kb + 8 * G + 4 * s2 + i) * pitch + col0 + 16 * sl + n16] : 0.f;
  }

  f4 Ot[4][NSL];
  auto store_tile = [&](int c, int mt) {
    const uint32_t orow = ((uint32_t)c * C + 16 * mt + n16) * vo_row;
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) {
      const bf16x4 ob = {(__bf16)Ot[mt][sl][0], (__bf16)Ot[mt][sl][1], (__bf16)Ot[mt][sl][2], (__bf16)Ot[mt][sl][3]};
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, ob), ro, orow + 2 * (col0 + 16 * sl + 4 * G), 0, 0);
    }
  };

  if (c_begin < c_mid) {
    issue(c_begin, kStAll);
    issue_v(c_begin);
  } else if (c_begin < c_end) {
    issue_qg(c_begin, c_begin & 1);
  }
  wait_and_barrier<0>();
  __builtin_amdgcn_s_waitcnt(0);   // the entering-state loads are complete (no wait for them in the loop)

  float* rqs = reinterpret_cast<float*>(lds + Cfg::kRq);   // |q_t|^2, t = 0..63
  auto put_qnorms = [&](float* dst, int mt, const f4& qq) {   // lane (n16, G): rows 4G .. 4G + 3 of column n16
    if ((n16 >> 2) == G) {
      const int ee = n16 & 3;
      dst[16 * mt + n16] = ee == 0 ? qq[0] : ee == 1 ? qq[1] : ee == 2 ? qq[2] : qq[3];
    }
  };
  const int cert_chunk = e ? run.cert_chunk[1] : run.cert_chunk[0];
  float* cert = e ? run.cert[1] : run.cert[0];

  for (int c = c_begin; c < c_mid; ++c) {
    // chunk c has landed for every wave (this wave's V too), every wave is done with chunk c - 1's
    // buffer; after chunk c's loads each wave issued only chunk c - 1's output stores
    wait_and_barrier<Cfg::kStores>();
    if (c == cert_chunk) {   // ||S||_F^2 of the state entering chunk c: this wave's part, in slot w & 3
      float ss = 0.f;
#pragma unroll
      for (int sl = 0; sl < NSL; ++sl)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int i = 0; i < 4; ++i) ss += S[sl][kb][s2][i] * S[sl][kb][s2][i];
      ss = wave_sum(ss);
      if (lane == 0) {
        cert[w & 3] = ss;
        cert[4 + (w & 3)] = 0.f;
      }
    }
    if (c + 1 < c_mid)
      issue(c + 1, kStK);
    else if (c + 1 < c_end)
      issue_qg(c + 1, (c + 1) & 1);
    const bool stage_next = c + 1 < c_mid;

    const unsigned char* Bf = lds + (c & 1) * Cfg::kBuf;
    const unsigned char* Kt = Bf + Cfg::kK;
    const unsigned char* Qt = Bf + Cfg::kQ;
    const unsigned char* Rc = Bf + Cfg::kRec + e * kRecB;   // this wave's head's record
    const float* sc = reinterpret_cast<const float*>(Rc + kScOff);

    // P' of this chunk for both heads: waves 0..5 form block w of K Q^T once (the key head's) and
    // scale it by each head's gates; waves 6 and 7 leave |q_t|^2 in LDS (two token tiles each).
    for (int blk = w; blk < w + 1 && blk < kFragBlocks; ++blk) {
      const int mt = block_tile(blk), kb2 = block_kb(blk);
      f4 pt[2] = {f4_splat(0.f), f4_splat(0.f)};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const bf16x8 qf = lds16(Qt + swz(16 * mt + n16, 4 * kb + G));
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) pt[s2] = mfma(lds16(Kt + swz(32 * kb2 + 16 * s2 + n16, 4 * kb + G)), qf, pt[s2]);
      }
      const int t = 16 * mt + n16;
#pragma unroll
      for (int he = 0; he < 2; ++he) {
        const float* sce = reinterpret_cast<const float*>(Bf + Cfg::kRec + he * kRecB + kScOff);
        const float gt = sce[kBfGam2 * C + t];
        f4 x2[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const int i0 = 32 * kb2 + 16 * s2 + 4 * G;
          const f4 gi = *reinterpret_cast<const f4*>(sce + kBfGam2 * C + i0);
          const f4 ri = *reinterpret_cast<const f4*>(sce + kBfRk * C + i0);
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const float x = ri[q4] * __builtin_amdgcn_exp2f(fminf(gt - gi[q4], 0.f)) * pt[s2][q4];
            x2[s2][q4] = (i0 + q4 <= t) ? x : 0.f;
          }
        }
        *reinterpret_cast<bf16x8*>(lds + Cfg::kP + he * kFragBlocks * 1024 + 1024 * blk + 16 * lane) = pack8(x2[0], x2[1]);
      }
    }
    if (w >= kFragBlocks) {   // waves 6 and 7: the Q Q^T of two token tiles each, whose diagonal is |q_t|^2
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int mt = 2 * (w - kFragBlocks) + h2;
        f4 qq = f4_splat(0.f);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const bf16x8 qf = lds16(Qt + swz(16 * mt + n16, 4 * kb + G));
          qq = mfma(qf, qf, qq);
        }
        put_qnorms(rqs, mt, qq);
      }
    }

    bf16x8 Sop[NSL][4];
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) Sop[sl][kb] = pack8(S[sl][kb][0], S[sl][kb][1]);

    if (stage_next) issue(c + 1, kStQ);

    // X = K S
    f4 X[NSL][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int sl = 0; sl < NSL; ++sl) X[sl][mt] = f4_splat(0.f);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const bf16x8 kf = lds16(Kt + swz(16 * mt + n16, 4 * kb + G));
#pragma unroll
        for (int sl = 0; sl < NSL; ++sl) X[sl][mt] = mfma(kf, Sop[sl][kb], X[sl][mt]);
      }
    }
    // R = V - diag(a) X
    bf16x8 Rop[NSL][2];
    {
      f4 a4[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) a4[mt] = *reinterpret_cast<const f4*>(sc + 16 * mt + 4 * G);
#pragma unroll
      for (int sl = 0; sl < NSL; ++sl) {
        f4 Rv[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          Rv[mt] = -a4[mt] * X[sl][mt];
          Rv[mt] += v_cols(mt, sl);
        }
        Rop[sl][0] = pack8(Rv[0], Rv[1]);
        Rop[sl][1] = pack8(Rv[2], Rv[3]);
      }
    }
    // Delta = Tb R (lower-triangular blocks only)
    f4 Dl[NSL][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int sl = 0; sl < NSL; ++sl) Dl[sl][mt] = f4_splat(0.f);
#pragma unroll
      for (int kb2 = 0; kb2 <= (mt >> 1); ++kb2) {
        const bf16x8 tf = lds16(Rc + 1024 * frag_block(mt, kb2) + 16 * lane);
#pragma unroll
        for (int sl = 0; sl < NSL; ++sl) Dl[sl][mt] = mfma(tf, Rop[sl][kb2], Dl[sl][mt]);
      }
    }
    // the next chunk's V into this wave's area: its reads of this chunk's V are complete
    if (stage_next) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      issue_v(c + 1);
    }
    bf16x8 Ddop[NSL][2];
    {
      f4 d4[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) d4[mt] = *reinterpret_cast<const f4*>(sc + kBfD * C + 16 * mt + 4 * G);
#pragma unroll
      for (int sl = 0; sl < NSL; ++sl) {
        Ddop[sl][0] = pack8(Dl[sl][0] * d4[0], Dl[sl][1] * d4[1]);
        Ddop[sl][1] = pack8(Dl[sl][2] * d4[2], Dl[sl][3] * d4[3]);
      }
    }
    if (stage_next) issue(c + 1, kStRec);
    lds_barrier();   // P' (both heads) and the q norms are complete
    // O^T = diag(c) (S^T Q^T) + Delta^T P^T, then the q norm of each row
    {
      bf16x8 Dop[NSL][2];
#pragma unroll
      for (int sl = 0; sl < NSL; ++sl) {
        Dop[sl][0] = pack8(Dl[sl][0], Dl[sl][1]);
        Dop[sl][1] = pack8(Dl[sl][2], Dl[sl][3]);
      }
      const unsigned char* Pe = lds + Cfg::kP + e * kFragBlocks * 1024;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int sl = 0; sl < NSL; ++sl) Ot[mt][sl] = f4_splat(0.f);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const bf16x8 qf = lds16(Qt + swz(16 * mt + n16, 4 * kb + G));
#pragma unroll
          for (int sl = 0; sl < NSL; ++sl) Ot[mt][sl] = mfma(Sop[sl][kb], qf, Ot[mt][sl]);
        }
        const float eg = __builtin_amdgcn_exp2f(sc[kBfGam2 * C + 16 * mt + n16]);   // e^gamma_t
#pragma unroll
        for (int sl = 0; sl < NSL; ++sl) Ot[mt][sl] *= eg;
#pragma unroll
        for (int kb2 = 0; kb2 <= (mt >> 1); ++kb2) {
          const bf16x8 pf = lds16(Pe + 1024 * frag_block(mt, kb2) + 16 * lane);
#pragma unroll
          for (int sl = 0; sl < NSL; ++sl) Ot[mt][sl] = mfma(Dop[sl][kb2], pf, Ot[mt][sl]);
        }
        const float rqv = __builtin_amdgcn_rsqf(rqs[16 * mt + n16] + 1e-6f) * 0.08838834764831845f;   // * 128^-1/2
#pragma unroll
        for (int sl = 0; sl < NSL; ++sl) Ot[mt][sl] *= rqv;
        store_tile(c, mt);
      }
    }
    // S <- e^{gamma_63} S + K^T diag(d) Delta
    const float egc = __builtin_amdgcn_exp2f(sc[kBfGam2 * C + C - 1]);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
        for (int sl = 0; sl < NSL; ++sl) S[sl][kb][s2] *= egc;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
          const bf16x8 kt = kt_frag(Kt, kb, s2, kb2, G, n16);
#pragma unroll
          for (int sl = 0; sl < NSL; ++sl) S[sl][kb][s2] = mfma(kt, Ddop[sl][kb2], S[sl][kb][s2]);
        }
      }
  }

  // Right pads (beta' = g' = 0): the state stays as it is and O = diag(rq) Q S, groups of kPadGroup
  // chunks, group g in buffer (c_mid + g) & 1; after a group's loads come the stores of the chunk or
  // group before it (none when the segment starts in the pads: its first group was waited for above).
  {
    bf16x8 Sop[NSL][4];
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) Sop[sl][kb] = pack8(S[sl][kb][0], S[sl][kb][1]);
    for (int c0 = c_mid, g = 0; c0 < c_end; c0 += kPadGroup, ++g) {
      const int bi = (c_mid + g) & 1, n = min(kPadGroup, c_end - c0);
      if (g == 0)
        wait_and_barrier<Cfg::kStores>();
      else
        wait_and_barrier<kPadGroup * Cfg::kStores>();
      if (c0 + kPadGroup < c_end) issue_qg(c0 + kPadGroup, bi ^ 1);
      const unsigned char* Bq = lds + bi * Cfg::kBuf;
      for (int pr = w; pr < 4 * n; pr += NW) {   // q norms of (chunk pr / 4, token tile pr % 4)
        const int i = pr >> 2, mt = pr & 3;
        const unsigned char* Qt = Bq + (i == 0 ? Cfg::kQ : (i == 1 ? Cfg::kK : Cfg::kRec));
        f4 qq = f4_splat(0.f);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const bf16x8 qf = lds16(Qt + swz(16 * mt + n16, 4 * kb + G));
          qq = mfma(qf, qf, qq);
        }
        put_qnorms(rqs + 64 * i, mt, qq);
      }
      lds_barrier();
      for (int i = 0; i < n; ++i) {
        const unsigned char* Qt = Bq + (i == 0 ? Cfg::kQ : (i == 1 ? Cfg::kK : Cfg::kRec));
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
          for (int sl = 0; sl < NSL; ++sl) Ot[mt][sl] = f4_splat(0.f);
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            const bf16x8 qf = lds16(Qt + swz(16 * mt + n16, 4 * kb + G));
#pragma unroll
            for (int sl = 0; sl < NSL; ++sl) Ot[mt][sl] = mfma(Sop[sl][kb], qf, Ot[mt][sl]);
          }
          const float rqv = __builtin_amdgcn_rsqf(rqs[64 * i + 16 * mt + n16] + 1e-6f) * 0.08838834764831845f;
#pragma unroll
          for (int sl = 0; sl < NSL; ++sl) Ot[mt][sl] *= rqv;
          store_tile(c0 + i, mt);
        }
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);   // no load into LDS may still be in flight when the workgroup ends

  // ---- end state
  if (!(p.s_final && run.last)) return;
  float* dst = p.s_final + ((size_t)b * p.Hv + h) * D * D;
#pragma unroll
  for (int sl = 0; sl < NSL; ++sl)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[(32 * kb + 8 * G + 4 * s2 + i) * D + col0 + 16 * sl + n16] = S[sl][kb][s2][i];
}

// Outputs over value-head pairs: one workgroup per (row, segment, head pair), pairs fastest.
__global__ __launch_bounds__(64 * PairCfg::NW) void gdr_scan_bf16_pair(ScanParams p) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[PairCfg::kLds];
  const int np = p.Hv / 2;
  const int lam = p.row_order ? (int)blockIdx.x : xcd_remap(blockIdx.x, gridDim.x);   // as gdr_scan_bf16
  const int hp = lam % np, j = (lam / np) % p.P;
  const int b = p.row_order ? p.row_order[lam / (np * p.P)] : lam / (np * p.P);
  PairRun run{};
  run.c_begin = j * p.Ls;
  run.c_end = min(run.c_begin + p.Ls, p.NC);
  // with segments, the combine has put every entering state in its slot (the first one only with s0)
  run.src_kind = p.P > 1 && (j > 0 || p.s0) ? 1 : 2;
  run.last = j == p.P - 1;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int h = 2 * hp + e;
    run.src[e] = run.src_kind == 1 ? slot_ptr(p, b, h, j) : nullptr;
    run.cert_chunk[e] = -1;
    run.cert[e] = nullptr;
    if (p.P > 1 && p.trunc && j + 1 < p.P) {
      const PlanEntry pe = p.plan[head_index(p, b, h) * p.P + j + 1];
      if (pe.trunc) {   // the window of boundary j + 1 starts inside this segment
        run.cert_chunk[e] = (j + 1) * p.Ls - pe.W;
        run.cert[e] = p.cert + (head_index(p, b, h) * p.P + j + 1) * kCertFloats;
      }
    }
  }
  pair_body(p, lds, b, hp, run);
}

// Truncation plan of a (row, head), from the chunk records. Its loads are issued first, all of them
// together (one memory round trip), and decided on after: PlanLoads holds what thread t of the
// workgroup reads, decide_window / chunks_contract decide from it. The window candidates come in
// batches of kPlanBatch chunks; a boundary that the first batch does not decide loads the next one.
constexpr int kPlanBatch = 8;
static_assert(kTruncMaxW % kPlanBatch == 0, "whole batches");
struct PlanLoads {
  int len, srow;                                // the row's length and s0 row, as stored
  float flag[kPlanBatch], dec[kPlanBatch];      // boundary t + 1's window candidates cb - 1, cb - 2, ...
  float cflag;                                  // contraction flag of chunk t (1 past the last boundary)
};
__device__ __forceinline__ const float* rec_scalars(const ScanParams& p, int b, int h, int c) {
  return reinterpret_cast<const float*>(reinterpret_cast<const unsigned char*>(p.ws) +
                                        (head_index(p, b, h) * p.NC + c) * kRecB + kScOff);
}
__device__ __forceinline__ PlanLoads plan_loads(const ScanParams& p, int b, int h, int t) {
  PlanLoads pl;
  pl.len = p.lengths ? p.lengths[b] : p.L;
  pl.srow = p.s0 ? (p.s0_row ? p.s0_row[b] : b) : 0;
  // Straight-line loads of in-range records (chunk indices clamped into [0, NC)); candidates past
  // min(Ls, kTruncMaxW) or before chunk 0, and chunks past the last boundary, are ignored later.
  const int cb = min(t + 1, p.P - 1) * p.Ls;   // <= (P - 1) Ls < NC
#pragma unroll
  for (int w = 1; w <= kPlanBatch; ++w) {
    const float* sc = rec_scalars(p, b, h, max(cb - w, 0));
    pl.flag[w - 1] = sc[kBfFlag * C];
    pl.dec[w - 1] = sc[kBfGam2 * C + C - 1];   // the chunk's whole decay, in log2
  }
  pl.cflag = rec_scalars(p, b, h, min(t, p.NC - 1))[kBfFlag * C];
  return pl;
}

// Boundary jb = t + 1 (1 <= jb < P): the shortest window of W <= min(Ls, kTruncMaxW) chunks ending at
// c = jb Ls whose chunks all hold valid tokens, all carry the contraction flag (every beta' in [0, 2],
// decay sum <= 0) and whose decay sums to l2 = sum g' log2 e <= -kTruncLog2. W = 0 when there is none
// (or the row's length or s0 row is out of range).
__device__ __forceinline__ void decide_window(const ScanParams& p, const PlanLoads& pl, int b, int h, int jb,
                                              int& W, float& l2) {
  W = 0;
  l2 = 0.f;
  if (jb >= p.P) return;
  if ((pl.len < 0 || pl.len > p.L) || (p.s0 && (pl.srow < 0 || pl.srow >= p.n_s0))) return;   // a bad row
  const int cb = jb * p.Ls;
  if (cb > (pl.len + C - 1) / C) return;   // the window would reach into the row's pads
  const int wmax = min(min(p.Ls, kTruncMaxW), cb);
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < kPlanBatch; ++i) {   // the first batch, loaded with the plan's other loads
    const int w = i + 1;
    if (w > wmax || !(pl.flag[i] == 1.f)) return;
    acc += pl.dec[i];
    if (acc <= -kTruncLog2) {
      W = w;
      l2 = acc;
      return;
    }
  }
#pragma unroll
  for (int w0 = kPlanBatch; w0 < kTruncMaxW; w0 += kPlanBatch) {
    // the next batch: candidates cb - w0 - 1, ... (clamped to chunk 0; past wmax unused), decided
    // without branches (selects only), so that every load of the batch is used in straight-line code
    // and all of them are in flight together: decided one candidate at a time behind early exits,
    // the loads were sunk to their uses and waited for one by one
    float flag[kPlanBatch], dec[kPlanBatch];
#pragma unroll
    for (int i = 0; i < kPlanBatch; ++i) {
      const float* sc = rec_scalars(p, b, h, max(cb - w0 - 1 - i, 0));
      flag[i] = sc[kBfFlag * C];
      dec[i] = sc[kBfGam2 * C + C - 1];
    }
    bool stop = false;   // a candidate past wmax or without the contraction flag ends the search
    int hit = 0;         // window length found in this batch (0: none yet)
    float hit_l2 = 0.f;
#pragma unroll
    for (int i = 0; i < kPlanBatch; ++i) {
      const int w = w0 + i + 1;
      stop = stop || w > wmax || !(flag[i] == 1.f);
      acc += dec[i];
      const bool take = !stop && hit == 0 && acc <= -kTruncLog2;
      hit = take ? w : hit;
      hit_l2 = take ? acc : hit_l2;
    }
    if (hit > 0) {
      W = hit;
      l2 = hit_l2;
      return;
    }
    if (stop) return;
  }
}

// Every chunk of the (row, head) from start to the last boundary that holds valid tokens contracts (its
// flag: every beta' in [0, 2] and a decay sum <= 0, so that its state map has spectral norm <= 1), checked
// by the workgroup's threads together (thread t: chunk t from the loads, then t + stride, ... for very
// long rows). Then an error in the state at one boundary does not grow on its way to the next window.
__device__ __forceinline__ bool chunks_contract(const ScanParams& p, const PlanLoads& pl, int b, int h, int t,
                                                int stride) {
  const int c_valid = (min(max(pl.len, 0), p.L) + C - 1) / C;
  bool ok = pl.cflag == 1.f || t >= c_valid || t >= (p.P - 1) * p.Ls;
  for (int c = t + stride; c < (p.P - 1) * p.Ls; c += stride)
    ok = ok && (rec_scalars(p, b, h, c)[kBfFlag * C] == 1.f || c >= c_valid);
  return ok;
}

// Transitions: one workgroup per (row, segment j < P - 1, value head). Every workgroup first plans the
// boundaries of its (row, head) (thread t: boundary t + 1; P <= 256 < threads); the (row, head) is
// truncated when every boundary has a window and every chunk up to the last boundary contracts. Then
// segment j's workgroup either runs the window before boundary j + 1 from zero on the value columns
// alone (the output pass's layout, without outputs), leaving the entering state of segment j + 1 in its
// slot and its norm in the certificate (truncated), or runs the whole segment on the augmented start
// [0 | I], leaving B_j and M_j for the combine (exact). The grid is below 256 + B Hv workgroups, so
// the output pass's larger LDS (one workgroup per CU) costs no parallelism.
static_assert(SegCfg<true>::kLds >= SegCfg<false>::kLds && SegCfg<true>::NW == SegCfg<false>::NW, "shared LDS");
__global__ __launch_bounds__(64 * SegCfg<false>::NW) void gdr_transition_bf16(ScanParams p) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[SegCfg<true>::kLds];
  const int lam = xcd_remap(blockIdx.x, gridDim.x);
  const int h = lam % p.Hv, j = (lam / p.Hv) % (p.P - 1), b = lam / (p.Hv * (p.P - 1));
  if (blockIdx.x == 0 && threadIdx.x == 0) *p.status = 0;   // read by the caller only
  const int t = threadIdx.x, jb_t = t + 1;
  int W = 0;
  float l2 = 0.f;
  bool contract = true;
  if (p.trunc) {
    const PlanLoads pl = plan_loads(p, b, h, t);
    decide_window(p, pl, b, h, jb_t, W, l2);
    contract = chunks_contract(p, pl, b, h, t, blockDim.x);
  }
  // every boundary has a window: an AND over the workgroup in the first word of the (not yet used)
  // staging area; the second word passes on the window of boundary j + 1
  int* all_ok = reinterpret_cast<int*>(lds);
  if (t == 0) *all_ok = 1;
  __syncthreads();
  if (!(jb_t >= p.P || W > 0) || !contract) *all_ok = 0;
  if (jb_t == j + 1) all_ok[1] = W;
  __syncthreads();
  const bool trunc = *all_ok != 0 && p.trunc;
  const int w_own = all_ok[1];
  __syncthreads();   // read before the staging area is written
  const size_t hb = head_index(p, b, h) * p.P;
  if (jb_t == j + 1) p.plan[hb + jb_t] = PlanEntry{W, l2, trunc ? 1 : 0, 0};
  if (trunc) {   // (segment 0's entering state, s0 or zero, is copied into slot 0 by the combine)
    SegRun win{};   // chunks (j + 1) Ls - W .. (j + 1) Ls - 1
    win.c_end = (j + 1) * p.Ls;
    win.c_begin = win.c_end - w_own;
    win.src_kind = 0;
    win.cert_chunk = -1;
    win.n2 = p.cert + (hb + j + 1) * kCertFloats + 8;
    win.end_b = slot_ptr(p, b, h, j + 1);
    seg_body<true, true>(p, lds, b, h, win);
    return;
  }
  SegRun run{};
  run.src_kind = 0;
  run.end_b = slot_ptr(p, b, h, j + 1);
  run.c_begin = j * p.Ls;
  run.c_end = min(run.c_begin + p.Ls, p.NC);
  run.end_m = slot_ptr(p, b, h, j);
  run.n2 = nullptr;
  seg_body<false>(p, lds, b, h, run);
}


// Finalize (bf16 with P > 1): one workgroup per (row, value head). For a (row, head) that took the
// truncated path it checks the certificate and, where it fails, counts the (row, head) in the status
// word and runs it again in one piece from its entering state (the copy of s0 the combine put in
// slot 0, or zero), overwriting o and s_final. (Checking in the output pass's last workgroup per head
// instead would need device-scope fences around a per-head counter, which write back and invalidate
// the compute die's L2 once per workgroup and cost far more than this launch.)
__global__ __launch_bounds__(64 * SegCfg<true>::NW) void gdr_finalize_bf16(ScanParams p) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[SegCfg<true>::kLds];
  const int h = blockIdx.x % p.Hv, b = blockIdx.x / p.Hv;
  const size_t hb = head_index(p, b, h) * p.P;
  if (!p.trunc) return;
  // 0: the exact path (nothing to check), 1: the certificate holds
  if (certificate_status(p, hb, reinterpret_cast<float*>(lds)) != 2) return;
  if (threadIdx.x == 0) atomicAdd(p.status, 1);
  __syncthreads();   // the scratch is read before the staging area is written
  SegRun all{};
  all.c_begin = 0;
  all.c_end = p.NC;
  all.src_kind = p.s0 ? 1 : 2;   // the copy of s0 in slot 0, or zero
  all.src = p.s0 ? slot_ptr(p, b, h, 0) : nullptr;
  all.last = true;
  all.cert_chunk = -1;
  if (p.z)
    seg_body<true, false, true>(p, lds, b, h, all);
  else
    seg_body<true, false, false>(p, lds, b, h, all);
}

// Combine: the state entering segment j + 1 is M_j S_j + B_j, S_0 = s0 (or zero). With s0, every
// (row, head) gets a copy of it in slot 0, the truncated ones too (then the kernel stops there). One
// workgroup per (row, value head, 16-column slice); wave w computes key rows 32w .. 32w + 31
// (tiles 2w, 2w + 1, plain row order) and the waves exchange the state each step as bf16
// hi + lo operand pairs, so that with M = Mh + Ml the products Mh Sh + Mh Sl + Ml Sh keep
// about 16 significant bits more than bf16 alone.
//
// Step jj reads this wave's 32 rows of M_jj (all 128 keys) and of the slice of B_jj; neither
// depends on the chained state, so each wave copies them HBM->LDS by DMA two steps ahead into a
// ring of two slots of its own (no other wave reads them, so no barrier guards them). In a slot the
// 16-byte chunk q of M row r sits at position q ^ (r & 15): the sixteen rows that one operand read
// touches then fall on distinct banks.
struct CombineSmem {
  unsigned char m[2][4][32 * 512];   // [slot][wave]: 32 rows of M_jj, 512 bytes each
  unsigned char bs[2][4][32 * 64];   // [slot][wave]: 32 rows of the B_jj slice, 64 bytes each
  bf16x8 sx[2][2][4][64];            // [step parity][hi, lo][wave][lane]: the state exchange
};
// Vector-memory operations this wave issues after the loads of step jj's slot, when that slot is
// waited for: the loads of step jj + 1 (kCombineLoads, if any) and the state stores of the steps
// in between (kCombineStores each).
constexpr int kCombineLoads = 16 + 2, kCombineStores = 8;
template <int N> __device__ __forceinline__ void wait_vm() {
  static_assert(N == 0 || N == 8 || N == 16 || N == 18 || N == 26 || N == 34, "extend the list of encodings");
  if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else if constexpr (N == 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else if constexpr (N == 16) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  else if constexpr (N == 18) asm volatile("s_waitcnt vmcnt(18)" ::: "memory");
  else if constexpr (N == 26) asm volatile("s_waitcnt vmcnt(26)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(34)" ::: "memory");
}

__global__ __launch_bounds__(256) void gdr_combine(ScanParams p) {
  __shared__ __attribute__((aligned(16))) CombineSmem sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15, G = lane >> 4;
  const int lam = xcd_remap(blockIdx.x, gridDim.x);
  const int slice = lam % kSlices16, h = (lam / kSlices16) % p.Hv, b = lam / (kSlices16 * p.Hv);
  int srow = 0;
  if (row_is_bad(p, b, srow)) return;   // the output pass writes NaN for this row
  const bool truncated = p.trunc && p.plan[((size_t)b * p.Hv + h) * p.P + 1].trunc;
  const int col = 16 * slice + n16;
  float* slots = p.seg + ((size_t)b * p.Hv + h) * p.P * kSlotFloats;
  i32x4 rs = rsrc_words(slots, (uint32_t)(p.P * kSlotFloats * sizeof(float)));
#pragma unroll
  for (int i = 0; i < 4; ++i) rs[i] = __builtin_amdgcn_readfirstlane(rs[i]);   // uniform: keep it in SGPRs

  f4 S[2] = {f4_splat(0.f), f4_splat(0.f)};
  if (p.s0) {
    const float* s0 = p.s0 + ((size_t)srow * p.Hv + h) * D * D;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)   // all loads first: the stores below may alias s0 as far as the
#pragma unroll                      // compiler knows, which would otherwise serialise them
      for (int i = 0; i < 4; ++i) S[s2][i] = s0[(32 * w + 16 * s2 + 4 * G + i) * D + col];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int i = 0; i < 4; ++i) slots[(32 * w + 16 * s2 + 4 * G + i) * 2 * D + col] = S[s2][i];
  }
  // Slot 0 now holds s0, where the output pass and a rerun start from (a copy: s_final may be s0
  // itself); without s0 they start from zero and slot 0 is not read. A truncated (row, head) is done:
  // the transition pass has left the entering state of every later segment in its slot.
  if (truncated) return;
  // With no initial state S_1 = B_0, which is already in its slot: the chain starts at step 1.
  const int steps = p.P - 1, first = p.s0 ? 0 : 1;
  if (!p.s0 && steps > 0) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int i = 0; i < 4; ++i) S[s2][i] = slots[kSlotFloats + (32 * w + 16 * s2 + 4 * G + i) * 2 * D + col];
  }
  // This wave's rows of M_jj (slot jj, columns 128..255; two rows per load) and of the B_jj slice
  // (slot jj + 1, columns 16 slice ..; sixteen rows per load) into ring slot u.
  auto issue = [&](int jj, int u) {
    const uint32_t mbase = (uint32_t)jj * kSlotFloats * 4, bbase = (uint32_t)(jj + 1) * kSlotFloats * 4;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 2 * i + (lane >> 5), pos = lane & 31;
      dma16(rs, mbase + ((uint32_t)(32 * w + r) * 2 * D + D) * 4 + 16 * (pos ^ (r & 15)), sm.m[u][w] + 2 * i * 512);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 16 * i + (lane >> 2);
      dma16(rs, bbase + ((uint32_t)(32 * w + r) * 2 * D + 16 * slice + 4 * (lane & 3)) * 4, sm.bs[u][w] + 16 * i * 64);
    }
  };
  // A wait the compiler sees: the state loads above are then known complete, so it places no wait
  // for them inside the loop (where it would also stall on the slot loads in flight).
  __builtin_amdgcn_s_waitcnt(0);
  if (first < steps) issue(first, 0);
  if (first + 1 < steps) issue(first + 1, 1);
  for (int jj = first; jj < steps; ++jj) {
    const int rel = jj - first, u = rel & 1;
    const bool next = jj + 1 < steps;   // step jj + 1's loads were issued after this step's
    if (rel == 0) {
      if (next) wait_vm<kCombineLoads>(); else wait_vm<0>();
    } else if (rel == 1) {
      if (next) wait_vm<kCombineLoads + kCombineStores>(); else wait_vm<kCombineStores>();
    } else {
      if (next) wait_vm<kCombineLoads + 2 * kCombineStores>(); else wait_vm<2 * kCombineStores>();
    }
    bf16x8 mh[2][4], ml[2][4];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const unsigned char* mrow = sm.m[u][w] + (16 * s2 + n16) * 512;
        const f4 m0 = *reinterpret_cast<const f4*>(mrow + 16 * ((8 * kb + G) ^ n16));
        const f4 m1 = *reinterpret_cast<const f4*>(mrow + 16 * ((8 * kb + 4 + G) ^ n16));
        mh[s2][kb] = pack8(m0, m1);
        f4 r0, r1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          r0[i] = m0[i] - (float)mh[s2][kb][i];
          r1[i] = m1[i] - (float)mh[s2][kb][4 + i];
        }
        ml[s2][kb] = pack8(r0, r1);
      }
    f4 Bv[2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        Bv[s2][i] = *reinterpret_cast<const float*>(sm.bs[u][w] + (16 * s2 + 4 * G + i) * 64 + 4 * n16);
    if (jj + 2 < steps) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave is done reading slot u
      issue(jj + 2, u);
    }
    {
      const bf16x8 hi = pack8(S[0], S[1]);
      f4 r0, r1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        r0[i] = S[0][i] - (float)hi[i];
        r1[i] = S[1][i] - (float)hi[4 + i];
      }
      sm.sx[jj & 1][0][w][lane] = hi;
      sm.sx[jj & 1][1][w][lane] = pack8(r0, r1);
    }
    lds_barrier();   // the state exchange is in LDS; the loads of later steps stay in flight
    f4 acc[2] = {f4_splat(0.f), f4_splat(0.f)};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const bf16x8 sh = sm.sx[jj & 1][0][kb][lane], sl = sm.sx[jj & 1][1][kb][lane];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        acc[s2] = mfma(mh[s2][kb], sh, acc[s2]);
        acc[s2] = mfma(mh[s2][kb], sl, acc[s2]);
        acc[s2] = mfma(ml[s2][kb], sh, acc[s2]);
      }
    }
    // the state entering segment jj + 1, over B_jj in slot jj + 1: exactly kCombineStores stores
    float* Bn = slots + (size_t)(jj + 1) * kSlotFloats;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      S[s2] = acc[s2] + Bv[s2];
#pragma unroll
      for (int i = 0; i < 4; ++i) Bn[(32 * w + 16 * s2 + 4 * G + i) * 2 * D + col] = S[s2][i];
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no load into LDS may be in flight at the end
}

// ====================================================================== fp32 scan
constexpr int kRecF = 2 * kFragBlocks * kBlockElems * 4 + kScalarBytes;   // fp32 record bytes (26624)
constexpr int kPK32 = D + 4, kPT32 = C + 4, kPV32 = 16 + 4;

struct ScanSmemF {
  float k[C * kPK32];      // K chunk, [token][dk]
  float q[C * kPK32];      // Q chunk, [token][dk]
  float tb[C * kPT32];     // T diag(beta'), [token][token]
  float pm[C * kPT32];     // decayed causal scores, [token][token]
  float v[C * kPV32];      // this workgroup's 16 value columns, [token][col]
  float sc[4 * C];         // a, c, d, e^{gamma_63}
  f4 xp[4][4][64];         // [wave][token tile][lane]: the waves' partial K S over their 32 keys
  f4 op[4][4][64];         // the same for Q S
};

// One workgroup per (row, value head, 16-column slice); wave w owns keys 32 w .. 32 w + 31 of the
// slice's state (two accumulator tiles) and the chunk's token tile w of the outputs. Per chunk:
// every wave forms its key block's share of X = K S and of Q S (the state's rows split the sum),
// the shares meet in LDS, every wave sums X and forms R = V - diag(a) X and Delta = Tb R in full,
// its output tile O_w = diag(c) (Q S)_w + P_w Delta, and its own key block of
// S <- e^{gamma_63} S + K^T diag(d) Delta, whose K^T operand it reads from the K tile as stored
// (one element per lane and slot, the sixteen keys of a read on distinct banks). The chunk's tiles
// are loaded into registers one chunk ahead and written to LDS after the chunk before it is done.
__global__ __launch_bounds__(256) void gdr_scan_f32(ScanParams p) {
  __shared__ __attribute__((aligned(16))) ScanSmemF sm;
  constexpr int NT = 256;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15, G = lane >> 4;
  const int lam = xcd_remap(blockIdx.x, gridDim.x);   // the slices of a head on one XCD (one L2)
  const int cs = lam % kSlices16, h = (lam / kSlices16) % p.Hv, b = lam / (kSlices16 * p.Hv);
  const int kh = h / (p.Hv / p.Hk);
  const int col0 = 16 * cs;
  const int ncol = col0 + n16;
  const float* qg = reinterpret_cast<const float*>(p.q);
  const float* kg = reinterpret_cast<const float*>(p.k);
  const float* vg = reinterpret_cast<const float*>(p.v);
  float* og = reinterpret_cast<float*>(p.o);
  const unsigned char* wsb = reinterpret_cast<const unsigned char*>(p.ws);

  const int len = p.lengths ? p.lengths[b] : p.L;
  const int srow = p.s0 ? (p.s0_row ? p.s0_row[b] : b) : 0;
  if ((len < 0 || len > p.L) || (p.s0 && (srow < 0 || srow >= p.n_s0))) {
    const float nan = __builtin_nanf("");
    for (int i = tid; i < p.L * 16; i += NT) og[((size_t)b * p.L + i / 16) * p.Hv * D + (size_t)h * D + col0 + i % 16] = nan;
    if (p.s_final)
      for (int i = tid; i < D * 16; i += NT) p.s_final[(((size_t)b * p.Hv + h) * D + i / 16) * D + col0 + i % 16] = nan;
    return;
  }

  // this wave's key block: tiles st = 0, 1 are keys 32 wave + 16 st + 4 G + e, column ncol
  f4 S[2];
  {
    const float* s0 = p.s0 ? p.s0 + ((size_t)srow * p.Hv + h) * D * D : nullptr;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int e = 0; e < 4; ++e) S[st][e] = s0 ? s0[(32 * wave + 16 * st + 4 * G + e) * D + ncol] : 0.f;
  }

  // Chunk staging, one chunk ahead. Per thread: eight 16-byte pieces of K and of Q, six of the
  // record's Tb and P operand blocks (12 blocks of 64 lanes x 8), one of V and (64 threads) one of
  // the scalars.
  f4 kr[8], qr[8], rr[6], vr, sr = f4_splat(0.f);
  auto load = [&](int c) {
    const int t0 = c * C;
    const unsigned char* rec = wsb + (((size_t)b * p.Hv + h) * p.NC + c) * kRecF;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int idx = tid + NT * i, row = idx >> 5, cv = idx & 31, t = t0 + row;
      kr[i] = qr[i] = f4_splat(0.f);
      if (t < p.L) {
        const size_t off = ((size_t)b * p.L + t) * p.Hk * D + (size_t)kh * D + 4 * cv;
        kr[i] = *reinterpret_cast<const f4*>(kg + off);
        qr[i] = *reinterpret_cast<const f4*>(qg + off);
      }
    }
#pragma unroll
    for (int i = 0; i < 6; ++i) {   // block q >> 7 (Tb 0..5, P 6..11), lane (q & 127) >> 1, half q & 1
      const int q = tid + NT * i;
      rr[i] = *reinterpret_cast<const f4*>(reinterpret_cast<const float*>(rec) + (q >> 7) * kBlockElems + ((q & 127) >> 1) * 8 +
                                           4 * (q & 1));
    }
    {
      const int row = tid >> 2, cv = tid & 3, t = t0 + row;
      vr = t < p.L ? *reinterpret_cast<const f4*>(vg + ((size_t)b * p.L + t) * p.Hv * D + (size_t)h * D + col0 + 4 * cv)
                   : f4_splat(0.f);
    }
    if (tid < C) sr = *reinterpret_cast<const f4*>(rec + 2 * kFragBlocks * kBlockElems * 4 + 16 * tid);
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int idx = tid + NT * i, row = idx >> 5, cv = idx & 31;
      *reinterpret_cast<f4*>(&sm.k[row * kPK32 + 4 * cv]) = kr[i];
      *reinterpret_cast<f4*>(&sm.q[row * kPK32 + 4 * cv]) = qr[i];
    }
#pragma unroll
    for (int i = 0; i < 6; ++i) {   // lane (m, g) of block (tile I, kb): row 16 I + m, columns 32 kb + 4g (+16)
      const int q = tid + NT * i, blk = q >> 7, bk = blk % kFragBlocks, ln = (q & 127) >> 1;
      const int row = 16 * block_tile(bk) + (ln & 15), col = 32 * block_kb(bk) + 4 * (ln >> 4) + 16 * (q & 1);
      *reinterpret_cast<f4*>(&(blk < kFragBlocks ? sm.tb : sm.pm)[row * kPT32 + col]) = rr[i];
    }
    *reinterpret_cast<f4*>(&sm.v[(tid >> 2) * kPV32 + 4 * (tid & 3)]) = vr;
    if (tid < C) *reinterpret_cast<f4*>(&sm.sc[4 * tid]) = sr;
  };
  // Tb and P are zero above their stored blocks (rows 0..31, columns 32..63); the blocks never
  // write there
  for (int idx = tid; idx < 32 * 32; idx += NT) {
    const int row = idx >> 5, col = 32 + (idx & 31);
    sm.tb[row * kPT32 + col] = 0.f;
    sm.pm[row * kPT32 + col] = 0.f;
  }
  if (p.NC > 0) load(0);

  const f4 one = f4_splat(1.f);
  for (int c = 0; c < p.NC; ++c) {
    const int t0 = c * C;
    __syncthreads();   // the previous chunk is done with LDS
    store();
    __syncthreads();
    if (c + 1 < p.NC) load(c + 1);

    // this key block's shares of K S and Q S
    const Frag<float> Sf = acc_frag<float>(S[0], S[1], one, one);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f4 x = f4_splat(0.f), o = f4_splat(0.f);
      mma(x, lds_frag(sm.k, kPK32, 16 * mt + n16, 32 * wave, G), Sf);
      mma(o, lds_frag(sm.q, kPK32, 16 * mt + n16, 32 * wave, G), Sf);
      sm.xp[wave][mt][lane] = x;
      sm.op[wave][mt][lane] = o;
    }
    __syncthreads();

    const float* sa = sm.sc;
    const float* scc = sm.sc + C;
    const float* sd = sm.sc + 2 * C;
    const float egC = sm.sc[3 * C];
    // R = V - diag(a) X over the chunk's 64 tokens
    f4 R[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const f4 X = sm.xp[0][mt][lane] + sm.xp[1][mt][lane] + sm.xp[2][mt][lane] + sm.xp[3][mt][lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * mt + 4 * G + e;
        R[mt][e] = sm.v[t * kPV32 + n16] - sa[t] * X[e];
      }
    }
    Frag<float> Rf[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) Rf[kb] = acc_frag<float>(R[2 * kb], R[2 * kb + 1], one, one);
    // Delta = Tb R (the blocks above the diagonal are zero: token tiles 0, 1 need key block 0 only)
    f4 Dl[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      Dl[mt] = f4_splat(0.f);
#pragma unroll
      for (int kb = 0; kb <= (mt >> 1); ++kb) mma(Dl[mt], lds_frag(sm.tb, kPT32, 16 * mt + n16, 32 * kb, G), Rf[kb]);
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
    // output tile `wave`: O = diag(c) Q S + P Delta
    {
      const int mt = wave;
      const f4 qs = sm.op[0][mt][lane] + sm.op[1][mt][lane] + sm.op[2][mt][lane] + sm.op[3][mt][lane];
      f4 O;
#pragma unroll
      for (int e = 0; e < 4; ++e) O[e] = scc[16 * mt + 4 * G + e] * qs[e];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        if (kb <= (mt >> 1)) mma(O, lds_frag(sm.pm, kPT32, 16 * mt + n16, 32 * kb, G), Df[kb]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = t0 + 16 * mt + 4 * G + e;
        if (t < p.L) og[((size_t)b * p.L + t) * p.Hv * D + (size_t)h * D + ncol] = O[e];
      }
    }
    // this key block of S <- e^{gamma_63} S + K^T diag(d) Delta; the K^T operand row (key) is
    // column 32 wave + 16 st + n16 of the K tile, its slots the tokens 32 kb + 4 G + j (+ 16)
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      S[st] *= egC;
      const int key = 32 * wave + 16 * st + n16;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        Frag<float> kt;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          kt.v[j] = sm.k[(32 * kb + 4 * G + j) * kPK32 + key];
          kt.v[4 + j] = sm.k[(32 * kb + 16 + 4 * G + j) * kPK32 + key];
        }
        mma(S[st], kt, Ddf[kb]);
      }
    }
  }

  if (p.s_final) {
    float* sf = p.s_final + ((size_t)b * p.Hv + h) * D * D;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int e = 0; e < 4; ++e) sf[(32 * wave + 16 * st + 4 * G + e) * D + ncol] = S[st][e];
  }
}

hipError_t launch_transition(const ScanParams& p, hipStream_t s) {
  hipLaunchKernelGGL(gdr_transition_bf16, dim3(p.B * p.Hv * (p.P - 1)), dim3(64 * SegCfg<false>::NW), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_combine(const ScanParams& p, hipStream_t s) {
  hipLaunchKernelGGL(gdr_combine, dim3(p.B * p.Hv * kSlices16), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_finalize(const ScanParams& p, hipStream_t s) {
  hipLaunchKernelGGL(gdr_finalize_bf16, dim3(p.B * p.Hv), dim3(64 * SegCfg<true>::NW), 0, s, p);
  return hipGetLastError();
}

// The pair pass needs Hv / Hk even and no fused norm. It is taken when the rows need no segments and
// the pairs alone fill the GPU (B Hv / 2 workgroups, at least one per CU). With segments it would need
// twice as many of them to fill the GPU, so twice the window transitions (two rounds of workgroups)
// and twice the entering-state loads, which cost more than its faster chunks save at the long prefill.
static bool use_pair_pass(const ScanParams& p) {
  return p.z == nullptr && p.Hk > 0 && p.Hv % p.Hk == 0 && (p.Hv / p.Hk) % 2 == 0 && p.P == 1 &&
         int64_t(p.B) * (p.Hv / 2) >= kSegTargetWorkgroups;
}

hipError_t launch_scan(const ScanParams& p, int qkv_bf16, hipStream_t s) {
  if (qkv_bf16) {
    if (p.z)
      hipLaunchKernelGGL(gdr_scan_bf16<true>, dim3(p.B * p.Hv * p.P), dim3(64 * SegCfg<true>::NW), 0, s, p);
    else if (use_pair_pass(p))
      hipLaunchKernelGGL(gdr_scan_bf16_pair, dim3(p.B * (p.Hv / 2) * p.P), dim3(64 * PairCfg::NW), 0, s, p);
    else
      hipLaunchKernelGGL(gdr_scan_bf16<false>, dim3(p.B * p.Hv * p.P), dim3(64 * SegCfg<true>::NW), 0, s, p);
  } else {
    hipLaunchKernelGGL(gdr_scan_f32, dim3(p.B * p.Hv * kSlices16), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace gdr
