// Device-side helpers shared by the prep and scan kernels (gfx950).
//
// MFMA operand convention used throughout. A 16x16 fp32 accumulator tile holds, in lane
// (n = lane % 16, G = lane / 16), rows 4G .. 4G+3 of column n. Two such tiles (rows 0..15 and
// 16..31 of a 32-deep block) give each lane 8 values of one column. We let register slot j of
// lane group G stand for row (j < 4 ? 4G + j : 16 + 4G + j - 4) of the k block; an MFMA only
// needs its A and B operands to agree on which physical k a (lane group, slot) pair stands
// for, so with this order an accumulator pair is directly a B operand, and A operands are two
// 4-element reads per lane from row-major LDS.
#ifndef GDR_DEVICE_H_
#define GDR_DEVICE_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdr_internal.h"

namespace gdr {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int C = kChunk;    // 64 tokens per chunk
constexpr int D = kHeadDim;  // Dk = Dv = 128

template <typename T> __device__ __forceinline__ float to_f(T x);
template <> __device__ __forceinline__ float to_f<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f<__bf16>(__bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ __bf16 from_f<__bf16>(float x) { return (__bf16)x; }

__device__ __forceinline__ f4 f4_splat(float x) { return f4{x, x, x, x}; }

// 16-byte vector of T (8 bf16 or 4 float), for global <-> LDS staging.
template <typename T> struct Vec16 {
  static constexpr int N = 16 / sizeof(T);
  uint4 raw;
  __device__ __forceinline__ T get(int i) const { return reinterpret_cast<const T*>(&raw)[i]; }
};

// Eight k-values per lane in the slot order above.
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

// A operand from row-major LDS: row `row`, k block starting at k0.
__device__ __forceinline__ Frag<__bf16> lds_frag(const __bf16* base, int pitch, int row, int k0, int G) {
  const __bf16* p = base + row * pitch + k0 + 4 * G;
  const bf16x4 lo = *reinterpret_cast<const bf16x4*>(p);
  const bf16x4 hi = *reinterpret_cast<const bf16x4*>(p + 16);
  Frag<__bf16> f;
  f.v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return f;
}
__device__ __forceinline__ Frag<float> lds_frag(const float* base, int pitch, int row, int k0, int G) {
  const float* p = base + row * pitch + k0 + 4 * G;
  const f4 lo = *reinterpret_cast<const f4*>(p);
  const f4 hi = *reinterpret_cast<const f4*>(p + 16);
  Frag<float> f;
#pragma unroll
  for (int j = 0; j < 4; ++j) { f.v[j] = lo[j]; f.v[4 + j] = hi[j]; }
  return f;
}

// A operand whose two halves come from two 16x16 tiles (row-major, pitch 16): slots 0..3 from
// tile t0 row `row` columns 4G..4G+3, slots 4..7 from tile t1 (or zero when t1 is null).
template <typename T>
__device__ __forceinline__ Frag<T> tile_frag(const T* t0, const T* t1, int row, int G);
template <>
__device__ __forceinline__ Frag<__bf16> tile_frag<__bf16>(const __bf16* t0, const __bf16* t1, int row, int G) {
  const bf16x4 lo = *reinterpret_cast<const bf16x4*>(t0 + row * 16 + 4 * G);
  bf16x4 hi = {};
  if (t1) hi = *reinterpret_cast<const bf16x4*>(t1 + row * 16 + 4 * G);
  Frag<__bf16> f;
  f.v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return f;
}

// B operand from two accumulator tiles, each row scaled by s0[i] / s1[i].
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

// Raw buffer access with hardware range checking: loads past `bytes` return zeros and stores
// past it are dropped, so bounds need no branches. Offsets are 32-bit byte offsets from `base`.
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
constexpr int kBufferConfig = 0x00020000;   // descriptor word 3 for the gfx9 family

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferConfig);
}
// The same descriptor as four scalar words, for loads written as inline assembly (made wave-uniform
// explicitly, so that they stay in scalar registers also where the compiler cannot prove it).
__device__ __forceinline__ i32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return i32x4{__builtin_amdgcn_readfirstlane((int)(uint32_t)a), __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32) & 0xffff),
               __builtin_amdgcn_readfirstlane((int)bytes), kBufferConfig};
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ void buf_store_bf16(__amdgpu_buffer_rsrc_t r, uint32_t off, __bf16 x) {
  __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(short, x), r, off, 0, 0);
}

// Lower-triangle 16x16 tile numbering of a 64x64 matrix: tile (I, J), J <= I, is I(I+1)/2 + J.
constexpr int kTiles = 10;
__device__ __forceinline__ int tile_id(int I, int J) { return I * (I + 1) / 2 + J; }
__device__ __forceinline__ int tile_row(int ti) { return (ti >= 1) + (ti >= 3) + (ti >= 6); }
__device__ __forceinline__ int tile_col(int ti) { const int I = tile_row(ti); return ti - I * (I + 1) / 2; }

// Operand blocks of a lower-triangular 64x64 record matrix (see the workspace layout).
__device__ __forceinline__ int frag_block(int w, int kb) { return (w < 2 ? w : 2 * w - 2) + kb; }
__device__ __forceinline__ int block_tile(int blk) { return blk < 2 ? blk : 2 + (blk - 2) / 2; }
__device__ __forceinline__ int block_kb(int blk) { return blk < 2 ? 0 : (blk - 2) % 2; }
// Column (within the 64-token chunk) of slot j of lane group G in token block kb.
__device__ __forceinline__ int slot_col(int kb, int G, int j) { return 32 * kb + (j < 4 ? 4 * G + j : 12 + 4 * G + j); }

// ---- 64 x 128 bf16 tiles staged in LDS by DMA (256-byte rows, no padding)
// The 16-byte chunk q of row r sits at position q ^ f(r mod 16), f the table below (nibble r of the
// constant; as bits: bit 3 of f = bit 0 of r, bit 2 = bit 1, bit 1 = bit 2 xor bit 3, bit 0 = bit 2).
// Measured with the LDS bank-conflict counter over every tile read of the segment kernels, it leaves
// the 16-byte row reads (sixteen consecutive rows of one chunk per lane group: the K, Q operands and
// the Gram) free of bank conflicts, and the transposing 8-byte reads of K^T (four rows by four chunks
// per 16 lanes) at two ways: every lane reads the same half of its chunk, so half of the bank slots
// go unused, and no swizzle tried did better. (The earlier swap of the two 2-bit fields of r gave the
// row reads two ways as well.) A table, because the compiler keeps the operand addresses in fewer
// registers than for the bit form.
__device__ __forceinline__ int swz_f(int row) { return (int)((0xd591e6a2f7b3c480ull >> (4 * (row & 15))) & 15); }
__device__ __forceinline__ int swz(int row, int chunk16) { return row * 256 + 16 * (chunk16 ^ swz_f(row)); }

// 16 bytes per lane from a range-checked buffer straight into LDS at lds + 16 * lane (out of
// range: zeros). Written as inline assembly so that the compiler neither waits for these loads
// at every barrier nor moves LDS accesses across them; the kernel counts them itself (vmcnt).
// The load takes its LDS base from M0, which the compiler may be using for something else: the
// statement saves M0 in an SGPR of its own, sets it, issues the load and puts the old value back,
// so M0 is unchanged when the statement ends and nothing reserved appears in a clobber list.
__device__ __forceinline__ void dma16(const i32x4& r, uint32_t off, const unsigned char* lds) {
  const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(lds));
  uint32_t saved;
  // one wait state separates the write of M0 from the load that reads it
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(base), "v"(off), "s"(r)
      : "memory");
}

__device__ __forceinline__ bf16x8 pack8(const f4& lo, const f4& hi) {
  bf16x8 f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[i] = (__bf16)lo[i];
    f[4 + i] = (__bf16)hi[i];
  }
  return f;
}
__device__ __forceinline__ f4 mfma(const bf16x8& a, const bf16x8& b, const f4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 lds16(const unsigned char* p) { return *reinterpret_cast<const bf16x8*>(p); }

// Workgroup barrier for waves that exchange data through LDS only: waits for this wave's LDS
// accesses, not for its global loads and stores (which a plain __syncthreads would also drain),
// and keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Hardware workgroup i runs on XCD i % 8. Logical workgroup lam = xcd_remap(i, n) numbers them so
// that consecutive logical ids run on one XCD (and share its L2); a bijection on [0, n).
__device__ __forceinline__ int xcd_remap(int id, int n) {
  return (n & 7) ? id : (id & 7) * (n >> 3) + (id >> 3);
}

}  // namespace gdr

#endif  // GDR_DEVICE_H_
