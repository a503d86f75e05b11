// Device helpers shared by the gfx950 kernels: bf16 conversion, vector types,
// MFMA wrappers and wavefront reductions. CDNA4 only (64-wide wavefronts).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// fp32 -> bf16 bit pattern, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t f2bf(float f) {
  __bf16 b = (__bf16)f;  // gfx950 lowers this to v_cvt_pk_bf16_f32 (RNE)
  return __builtin_bit_cast(uint16_t, b);
}

// Two fp32 -> packed pair of bf16 (low half = a).
__device__ __forceinline__ uint32_t pack2bf(float a, float b) {
  return (uint32_t)f2bf(a) | ((uint32_t)f2bf(b) << 16);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// 32x32x16 bf16 MFMA, fp32 accumulate. Lane l supplies A[l%32][8*(l/32)+0..7]
// and B[8*(l/32)+0..7][l%32]; C lane l register i holds
// C[(i/4)*8 + (l/32)*4 + i%4][l%32].
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16x16x32 bf16 MFMA. Lane l supplies A[l%16][8*(l/16)+0..7] and
// B[8*(l/16)+0..7][l%16]; C lane l register i holds C[4*(l/16)+i][l%16].
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// fp16 bit pattern <-> fp32 (round to nearest even on the way down).
__device__ __forceinline__ float h2f(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }
__device__ __forceinline__ uint16_t f2h(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }
__device__ __forceinline__ uint32_t pack2h(float a, float b) {
  f16x2 v = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// 16-bit element types of the intermediate key/value tensors and of the
// attention MFMA operands. Both use the same 32x32x16 MFMA rate on gfx950;
// fp16 carries 11 significant bits against bf16's 8 (range |x| < 65504).
struct BF16 {
  static constexpr int code = 0;
  __device__ static __forceinline__ float dec(uint16_t h) { return bf2f(h); }
  __device__ static __forceinline__ uint16_t enc(float f) { return f2bf(f); }
  __device__ static __forceinline__ uint32_t pack2(float a, float b) { return pack2bf(a, b); }
  // low / high element of a packed pair
  __device__ static __forceinline__ float lo(uint32_t w) { return __uint_as_float(w << 16); }
  __device__ static __forceinline__ float hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
  // acc + both elements of a packed pair
  __device__ static __forceinline__ float sum2(uint32_t w, float acc) { return acc + lo(w) + hi(w); }
  __device__ static __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
  }
};

struct F16 {
  static constexpr int code = 1;
  __device__ static __forceinline__ float dec(uint16_t h) { return h2f(h); }
  __device__ static __forceinline__ uint16_t enc(float f) { return f2h(f); }
  __device__ static __forceinline__ uint32_t pack2(float a, float b) { return pack2h(a, b); }
  __device__ static __forceinline__ float lo(uint32_t w) { return h2f((uint16_t)(w & 0xffffu)); }
  __device__ static __forceinline__ float hi(uint32_t w) { return h2f((uint16_t)(w >> 16)); }
  __device__ static __forceinline__ float sum2(uint32_t w, float acc) {
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w), one, acc, false);
  }
  __device__ static __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
  }
};

// Raw buffer resource over [base, base + bytes): loads at byte offsets past
// the end return zeros (the hardware range check), which replaces per-lane
// bounds branches for ragged tiles. Offsets are passed in the vector offset
// (the one the range check covers); the tensor slice must be < 4 GiB.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
}

// LDS operand images for 16-bit MFMA operands loaded by 16-byte LDS-direct
// loads (lane i of a load writes bytes 16i..16i+15 of a 1 KB block).
// A group of SW 1 KB blocks (SW = 1, 2 or 4) holds SW 16-deep k-steps of the
// 32 rows one 32x32 MFMA operand covers. Row r (0..31) lives in block
// r / (32/SW) of the group at byte (r % (32/SW)) * 32*SW (32*SW contiguous
// bytes of the row: with SW = 4 one load instruction brings 8 whole
// 128-byte row segments); its 16-byte chunk x (0..2SW-1) sits at chunk
// position x ^ swz(r). With 16 lanes per LDS cycle (rows r..r+15 of one
// k-step, same chunk), the pairs (row position mod 256 bytes, chunk
// position) are all distinct, so the 16 reads hit 16 different 4-bank groups.
template <int SW>
__device__ __forceinline__ int frag_swz(int r) {
  return (r >> (SW == 4 ? 1 : SW == 2 ? 2 : 3)) & (2 * SW - 1);
}
// Byte offset in the group of the chunk that lane (row r, half g) reads for
// k-step 0; k-step c is at this offset XOR 32c.
template <int SW>
__device__ __forceinline__ int frag_read0(int r, int g) {
  constexpr int RL = 32 / SW;
  return (r / RL) * 1024 + (r % RL) * (32 * SW) + ((frag_swz<SW>(r) ^ g) << 4);
}
// Row r and chunk x that load lane i writes into block rb of a group.
template <int SW>
__device__ __forceinline__ void frag_slot(int rb, int i, int& r, int& x) {
  r = rb * (32 / SW) + i / (2 * SW);
  x = (i % (2 * SW)) ^ frag_swz<SW>(r);
}

}  // namespace mla
