// Device-side building blocks shared by the gfx950 kernels: element types,
// 16-byte vector loads/stores, conversions and the 16x16x32 matrix-core step.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace edit {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// Elements of T in one 16-byte chunk.
template <typename T> struct Chunk;
template <> struct Chunk<bf16> { static constexpr int n = 8; };
template <> struct Chunk<float> { static constexpr int n = 4; };

// A matrix-core operand fragment: 8 consecutive K values of one row (A) or
// one column (B) per lane. bf16: one 16-byte register quad; f32: two quads.
template <typename T> struct Frag;
template <> struct Frag<bf16> { typedef bf16x8 type; };
template <> struct Frag<float> { typedef f32x8 type; };

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }

// ---------------------------------------------------------------------------
// 8-element vectors as fp32 (load, store, zero) for any element type.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void load8(const bf16* p, float (&v)[8]) {
  bf16x8 t = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (float)t[i];
}
__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
  f32x4 a = *reinterpret_cast<const f32x4*>(p);
  f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
}
__device__ __forceinline__ void store8(bf16* p, const float (&v)[8]) {
  bf16x8 t;
#pragma unroll
  for (int i = 0; i < 8; ++i) t[i] = (bf16)v[i];
  *reinterpret_cast<bf16x8*>(p) = t;
}
__device__ __forceinline__ void store8(float* p, const float (&v)[8]) {
  f32x4 a, b;
#pragma unroll
  for (int i = 0; i < 4; ++i) { a[i] = v[i]; b[i] = v[4 + i]; }
  *reinterpret_cast<f32x4*>(p) = a;
  *reinterpret_cast<f32x4*>(p + 4) = b;
}
__device__ __forceinline__ void store4(bf16* p, const float (&v)[4]) {
  bf16x4 t;
#pragma unroll
  for (int i = 0; i < 4; ++i) t[i] = (bf16)v[i];
  *reinterpret_cast<bf16x4*>(p) = t;
}
__device__ __forceinline__ void store4(float* p, const float (&v)[4]) {
  f32x4 a;
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = v[i];
  *reinterpret_cast<f32x4*>(p) = a;
}

// ---------------------------------------------------------------------------
// Fragments
// ---------------------------------------------------------------------------
__device__ __forceinline__ void frag_zero(bf16x8& f) {
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = (bf16)0.0f;
}
__device__ __forceinline__ void frag_zero(f32x8& f) {
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = 0.0f;
}
__device__ __forceinline__ void frag_load(bf16x8& f, const bf16* p) {
  f = *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ void frag_load(f32x8& f, const float* p) {
  f32x4 a = *reinterpret_cast<const f32x4*>(p);
  f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) { f[i] = a[i]; f[4 + i] = b[i]; }
}
// Fragment from a row whose 8 K values sit at element offset o0 (bf16: one
// 16-byte chunk) or at o0 and o1 (f32: two 16-byte chunks, 4 values each).
__device__ __forceinline__ void frag_load2(bf16x8& f, const bf16* row, int o0, int) {
  f = *reinterpret_cast<const bf16x8*>(row + o0);
}
__device__ __forceinline__ void frag_load2(f32x8& f, const float* row, int o0, int o1) {
  f32x4 a = *reinterpret_cast<const f32x4*>(row + o0);
  f32x4 b = *reinterpret_cast<const f32x4*>(row + o1);
#pragma unroll
  for (int i = 0; i < 4; ++i) { f[i] = a[i]; f[4 + i] = b[i]; }
}
__device__ __forceinline__ void frag_from_f32(bf16x8& f, const float (&v)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = (bf16)v[i];
}
__device__ __forceinline__ void frag_from_f32(f32x8& f, const float (&v)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = v[i];
}

// D(16x16) += A(16x32) * B(32x16).
// Lane l supplies A row (l % 16) and B column (l % 16), each with the 8 K
// indices 8*(l/16) .. 8*(l/16)+7. D element (row 4*(l/16)+r, col l%16) is
// acc[r]. The f32 form issues eight 16x16x4 steps, step j taking element j
// of every lane, so it sums the same 32 products.
__device__ __forceinline__ void mma16(f32x4& acc, const bf16x8& a, const bf16x8& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma16(f32x4& acc, const f32x8& a, const f32x8& b) {
#pragma unroll
  for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], acc, 0, 0, 0);
}

__device__ __forceinline__ void acc_zero(f32x4& a) { a[0] = a[1] = a[2] = a[3] = 0.0f; }

// D(32x32) += A(32x16) * B(16x32): the wide matrix-core step, which gfx950
// runs at about twice the flop rate of the 16x16x32 form (2.2 vs 1.2 PF/s
// measured on MI355X with independent accumulators).
// Lane l supplies A row (l % 32) and B column (l % 32), each with the 8 K
// indices 8*(l/32) .. 8*(l/32)+7. D element (row 8*(r/4) + 4*(l/32) + r%4,
// col l%32) is acc[r]. The f32 form issues eight 32x32x2 steps, step j
// taking element j of every lane.
typedef float f32x16 __attribute__((ext_vector_type(16)));
__device__ __forceinline__ void mma32(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma32(f32x16& acc, const f32x8& a, const f32x8& b) {
#pragma unroll
  for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[j], b[j], acc, 0, 0, 0);
}
__device__ __forceinline__ void mma_any(f32x4& acc, const bf16x8& a, const bf16x8& b) { mma16(acc, a, b); }
__device__ __forceinline__ void mma_any(f32x4& acc, const f32x8& a, const f32x8& b) { mma16(acc, a, b); }
__device__ __forceinline__ void mma_any(f32x16& acc, const bf16x8& a, const bf16x8& b) { mma32(acc, a, b); }
__device__ __forceinline__ void mma_any(f32x16& acc, const f32x8& a, const f32x8& b) { mma32(acc, a, b); }
__device__ __forceinline__ void acc_zero(f32x16& a) {
#pragma unroll
  for (int i = 0; i < 16; ++i) a[i] = 0.0f;
}

// Blocks are dealt to the 8 XCDs round-robin (block i runs on XCD i % 8).
// Renumber so that each XCD receives one contiguous range of logical tiles:
// neighbouring tiles then share that XCD's L2.
__device__ __forceinline__ int xcd_swizzle(int bid, int nblocks) {
  const int per = nblocks / 8, rem = nblocks % 8;
  const int x = bid % 8, i = bid / 8;
  return x * per + (x < rem ? x : rem) + i;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

}  // namespace edit
