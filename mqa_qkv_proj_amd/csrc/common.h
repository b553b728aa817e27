// Device helpers shared by the gfx950 kernels: MFMA wrappers, bf16/fp16
// packing, XCD-aware block remapping and wave-level LDS ordering.
//
// MFMA 32x32x16 operand convention used throughout (CDNA4 wave64):
//   A (32 x 16): lane l holds row (l % 32), eight k values "slot j" (j = 0..7)
//                of k-half (l / 32);
//   B (16 x 32): lane l holds column (l % 32), the same eight k slots;
//   D (32 x 32): lane l holds column (l % 32), rows 8*(i/4) + 4*(l/32) + (i%4)
//                for accumulator element i = 0..15.
// Only the row/column placement matters for correctness: A and B always put
// the same k in the same (lane half, slot), so the hardware's k order cancels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace mqkv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16_t mfma32_bf16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16_t mfma32_f16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// 16x16x32: A (16 x 32): lane l holds row l%16, k slots of group l/16; B (32 x 16):
// column l%16, the same k group; D (16 x 16): column l%16, rows 4*(l/16) + i.
__device__ __forceinline__ f32x4_t mfma16_bf16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// 32x32x64 e4m3 x e4m3 -> fp32 (OCP fp8): the same row / column placement as
// 32x32x16, with 32 bytes of k per lane given as two 16-byte fragments.
typedef int i32x8_t __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x16_t mfma32_f8(u32x4_t a0, u32x4_t a1, u32x4_t b0, u32x4_t b1, f32x16_t c) {
  const i32x8_t a = __builtin_bit_cast(i32x8_t, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
  const i32x8_t b = __builtin_bit_cast(i32x8_t, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7));
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// bf16 halves of a packed dword -> exact fp32.
__device__ __forceinline__ float bf16lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Two fp32 -> packed bf16 pair (round to nearest even), first value in the low half.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2_t r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, r);
}

// Two fp32 -> packed fp16 pair (round to nearest even), first value in the low half.
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  f16x2_t r;
  r[0] = (_Float16)a;
  r[1] = (_Float16)b;
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t u) { return __uint_as_float(((uint32_t)u) << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16(float a) {
  bf16x2_t r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)0.0f;
  return (uint16_t)(__builtin_bit_cast(uint32_t, r) & 0xffffu);
}

// Power-of-two exponent s of a tile of V (bf16) for the fp16 P.V products: the
// tile is converted to fp16 as V * 2^-s.  bf16 values with an unbiased exponent in [-17, 15] convert to fp16
// exactly, so a tile whose largest |v| lies in [2^-10, 2^16) keeps s = 0; a tile
// beyond fp16's range (or entirely tiny) takes s = e - 14, which puts its
// largest |v| in [2^14, 2^15).  `em` is the largest exponent field (bits 7..14
// of the bf16 pattern, shifted down) of the tile; 0 = only zeros/subnormals.
__device__ __forceinline__ int v_tile_exp(uint32_t em) {
  const int e = (int)em - 127;
  return (em != 0 && (e > 15 || e < -10)) ? e - 14 : 0;
}
// largest bf16 exponent field of the two halves of a packed pair
__device__ __forceinline__ uint32_t bf16x2_expmax(uint32_t u) {
  return max((u >> 7) & 0xffu, u >> 23 & 0xffu);
}

// Exchange with the lane 32 positions away (the other k-half of an MFMA tile).
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

// max(x, x of the lane 32 away) without a trip through LDS: permlane32_swap on
// two copies of x leaves, in every lane, x and its partner's x in the two
// results (which one is in which depends on the lane half).
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Order a wave's own LDS writes before its later LDS reads (no workgroup barrier).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Workgroups are dispatched round-robin over the 8 XCDs (id % 8).  Remap so that
// each XCD receives a contiguous range of logical ids: neighbouring logical
// blocks (which share K/V or weight tiles) then share one XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  const int full = (nblocks / 8) * 8;
  if (bid >= full) return bid;
  return (bid % 8) * (full / 8) + bid / 8;
}

// f(integral_constant<int, I>) for I = B .. E-1 as straight-line code.  Unlike an
// unrolled loop, this leaves no loop structure for the optimizer to move
// instructions out of, so the written order is the order the scheduler sees.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

__device__ __forceinline__ u32x4_t ld16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }

// Buffer resource over `bytes` bytes from a wave-uniform base: 16-byte loads at
// byte offsets at or beyond `bytes` return zeros instead of touching memory, so
// ragged tile tails need no branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4_t bld16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}
// LDS-DMA: every lane's 16 bytes at buffer offset voff + soff land at
// lds + 16 * lane (lds is wave-uniform).  Lanes whose offset is out of range
// write nothing.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}

__device__ __forceinline__ void st16(void* p, u32x4_t v) { *reinterpret_cast<u32x4_t*>(p) = v; }
__device__ __forceinline__ void st8(void* p, u32x2_t v) { *reinterpret_cast<u32x2_t*>(p) = v; }

}  // namespace mqkv
