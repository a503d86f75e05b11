// Measurement aids: a streaming HBM read and a dense fp16 MFMA loop, the
// sustained ceilings against which the method's kernels are read beside the
// published MI355X peaks. Neither computes anything of the method.
#include "../../include/mla_ceiling.h"
#include "common.hpp"

namespace mla {
namespace {

constexpr int kReadBlocks = 16384, kReadThreads = 512, kReadUnroll = 8;
constexpr int kMfmaBlocks = 512, kMfmaThreads = 512;  // two 8-wave workgroups per compute unit
constexpr int kFrags = MLA_CEILING_MFMA_OPERAND_BYTES / 1024;  // 1 KB fragments (64 lanes x 16 B)
constexpr uint32_t kNever = 0x9e3779b9u;

__global__ void __launch_bounds__(kReadThreads) hbm_read_kernel(const u32x4* __restrict__ p, size_t n16,
                                                                 uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (kReadUnroll - 1) * stride < n16; i += kReadUnroll * stride) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(p + i);
  const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (x == kNever) sink[0] = x;  // keeps the loads
}

template <bool LDS>
__global__ void __launch_bounds__(kMfmaThreads) mfma_loop_kernel(const u32x4* __restrict__ ops, int iters,
                                                                  float* __restrict__ sink) {
  constexpr int NCH = LDS ? 2 : 4;  // independent accumulation chains per wave
  __shared__ u32x4 frag[kFrags * 64];
  for (int i = threadIdx.x; i < kFrags * 64; i += kMfmaThreads) frag[i] = ops[i];
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const f16x8 a = __builtin_bit_cast(f16x8, frag[lane]);
  const f16x8 b = __builtin_bit_cast(f16x8, frag[64 + lane]);
  f32x16 acc[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
  for (int it = 0; it < iters; ++it) {
    if (!LDS) {
#pragma unroll
      for (int u = 0; u < 12; ++u)
#pragma unroll
        for (int c = 0; c < NCH; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[c], 0, 0, 0);
    } else {
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        f16x8 af[12];
#pragma unroll
        for (int u = 0; u < 12; ++u)
          af[u] = __builtin_bit_cast(f16x8, frag[((c * 12 + u) % kFrags) * 64 + ((lane + it) & 63)]);
#pragma unroll
        for (int u = 0; u < 12; ++u) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[u], b, acc[c], 0, 0, 0);
      }
    }
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[c][e];
  if (__float_as_uint(s) == kNever) sink[0] = s;  // keeps the products
}

}  // namespace
}  // namespace mla

extern "C" mla_status mla_ceiling_hbm_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
  if (!buf || !sink) return MLA_ERR_NULL;
  if (bytes == 0 || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(buf) % 16 != 0) return MLA_ERR_SHAPE;
  (void)hipGetLastError();  // a stale error from earlier work is not this call's
  hipLaunchKernelGGL(mla::hbm_read_kernel, dim3(mla::kReadBlocks), dim3(mla::kReadThreads), 0, stream,
                     static_cast<const mla::u32x4*>(buf), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

extern "C" mla_status mla_ceiling_mfma(const uint16_t* operands, int32_t iters, int32_t lds_operands, float* sink,
                                       double* flops, hipStream_t stream) {
  if (!operands || !sink) return MLA_ERR_NULL;
  if (iters < 1 || (lds_operands != 0 && lds_operands != 1)) return MLA_ERR_SHAPE;
  if (reinterpret_cast<uintptr_t>(operands) % 16 != 0) return MLA_ERR_SHAPE;
  const mla::u32x4* ops = reinterpret_cast<const mla::u32x4*>(operands);
  (void)hipGetLastError();
  if (lds_operands)
    hipLaunchKernelGGL(mla::mfma_loop_kernel<true>, dim3(mla::kMfmaBlocks), dim3(mla::kMfmaThreads), 0, stream, ops,
                       iters, sink);
  else
    hipLaunchKernelGGL(mla::mfma_loop_kernel<false>, dim3(mla::kMfmaBlocks), dim3(mla::kMfmaThreads), 0, stream, ops,
                       iters, sink);
  if (flops) {
    const double per_wave_iter = 12.0 * (lds_operands ? 2 : 4) * 2.0 * 32 * 32 * 16;
    *flops = per_wave_iter * iters * (mla::kMfmaThreads / 64) * (double)mla::kMfmaBlocks;
  }
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

extern "C" mla_status mla_device_info(int32_t device, int32_t* compute_units, int32_t* peak_sclk_khz,
                                      int32_t* peak_mclk_khz) {
  if (!compute_units || !peak_sclk_khz || !peak_mclk_khz) return MLA_ERR_NULL;
  int cu = 0, sclk = 0, mclk = 0;
  if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
      hipDeviceGetAttribute(&sclk, hipDeviceAttributeClockRate, device) != hipSuccess ||
      hipDeviceGetAttribute(&mclk, hipDeviceAttributeMemoryClockRate, device) != hipSuccess)
    return MLA_ERR_HIP;
  *compute_units = cu;
  *peak_sclk_khz = sclk;
  *peak_mclk_khz = mclk;
  return MLA_OK;
}
