// Device helpers shared by the gfx950 kernels of libbsa: vector types, matrix
// core (MFMA) wrappers, LDS address casts, bf16 packing and cross-lane moves.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

#define BSA_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D(32x32) += A(32x16) * B(16x32), bf16 inputs, fp32 accumulate.
// Lane l holds A[l%32][8*(l/32)+e], B[8*(l/32)+e][l%32] (e = 0..7) and
// D[8*j + 4*(l/32) + i][l%32] in register 4*j + i.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D(16x16) += A(16x32) * B(32x16), bf16 inputs, fp32 accumulate.
// Lane l holds A[l%16][8*(l/16)+e], B[8*(l/16)+e][l%16] and
// D[4*(l/16) + i][l%16] in register i.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane 4*r + c supplies the address of 4 consecutive 16-bit elements that form
// columns 4c..4c+3 of row r of a 4x16 block; lane i receives column i of that
// block, rows 0..3 in elements 0..3.
__device__ __forceinline__ bf16x4 lds_read_tr16(const void* p) {
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(BSA_LDS(s16x4, p));
  return __builtin_bit_cast(bf16x4, v);
}
// The same read at a byte offset from the start of LDS.
__device__ __forceinline__ bf16x4 lds_read_tr16_at(uint32_t byte_off) {
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)byte_off);
  return __builtin_bit_cast(bf16x4, v);
}

// Asynchronous 16-byte global -> LDS copy.  Every lane supplies its own global
// address; the wave writes 64 consecutive 16-byte slots starting at `lds`
// (wave-uniform), lane L into slot L.
__device__ __forceinline__ void global_to_lds16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, BSA_LDS(void, lds), 16, 0, 0);
}

// Read-only view of an index table in the constant address space: the
// compiler treats it as invariant, so reads at wave-uniform addresses become
// scalar loads (they never count against vmcnt).
template <typename T>
__device__ __forceinline__ const __attribute__((address_space(4))) T* as_const(const T* p) {
  return (const __attribute__((address_space(4))) T*)(p);
}

__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)BSA_LDS(const void, p);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Value held by lane l ^ 32.
__device__ __forceinline__ float xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x), false, false);
  int v = (threadIdx.x & 32) ? r[0] : r[1];
  return __builtin_bit_cast(float, v);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Round two floats to bf16 (one packed conversion, nearest even) and return
// the packed pair; *sum gains the two rounded values and, when EXACT, *exact
// gains the two unrounded ones.
template <bool EXACT = false>
__device__ __forceinline__ uint32_t pack2_bf16_sum(float a, float b, float* sum, float* exact = nullptr) {
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  *sum = __builtin_amdgcn_fdot2_f32_bf16(v, ones, *sum, false);  // exact products, fp32 sum
  if constexpr (EXACT) *exact += a + b;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16x8 pack8(const float* x) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)x[e];
  return r;
}

// Load 8 consecutive elements as bf16 (bf16 source: one 16-byte load; fp32
// source: two 16-byte loads rounded to nearest even).
template <typename T>
__device__ __forceinline__ bf16x8 load8_bf16(const T* p);

template <>
__device__ __forceinline__ bf16x8 load8_bf16<__bf16>(const __bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

template <>
__device__ __forceinline__ bf16x8 load8_bf16<float>(const float* p) {
  f32x4 a = *reinterpret_cast<const f32x4*>(p);
  f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  float t[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return pack8(t);
}

// Order-preserving map of a float to uint32 (larger float -> larger key);
// -0 is folded onto +0 so that the two compare equal.
__device__ __forceinline__ uint32_t float_key(float x) {
  x = x + 0.0f;
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// inverse of float_key (a negative zero comes back as +0)
__device__ __forceinline__ float key_float(uint32_t k) {
  return __builtin_bit_cast(float, (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

}  // namespace bsa
