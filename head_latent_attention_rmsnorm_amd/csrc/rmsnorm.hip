// RMSNorm (equation page "Read the equation": kv_a_layernorm of the
// compressed latent; GLM-5 "Normalized key-value latent": default epsilon
// 1e-6; Kimi-K2 "Query content heads": q_a_layernorm between the query
// projections). One wavefront per row; 16-byte coalesced bf16 loads; fp32 sum
// of squares reduced across the wavefront; one round-to-nearest-even per
// element into the output type. The latent is written in fp16: kv_b_proj
// multiplies it on fp16 MFMA, and fp16's 11 significant bits keep its
// rounding at the level of the fp16 keys and values themselves (bf16's 8
// bits made it the largest single error of the path). The query RMSNorm
// writes bf16, the input type of q_b_proj.
#include "common.hpp"
#include "launch.hpp"

namespace mla {

// One row whose width R is a multiple of 8 and at most 512*NCH, by one
// wavefront: each lane keeps NCH chunks of 8 elements in registers (chunk c
// of lane l covers columns 8*(l + 64*c) .. +8).
template <int NCH, class OT>
__device__ __forceinline__ void rms_row(const uint16_t* __restrict__ xrow, const uint16_t* __restrict__ w, float eps,
                                        uint16_t* __restrict__ yrow, int R, int lane) {
  const int nch = R >> 3;
  const u32x4* xr = reinterpret_cast<const u32x4*>(xrow);
  u32x4 v[NCH];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int ch = lane + 64 * c;
    if (ch < nch) {
      v[c] = xr[ch];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float a = __uint_as_float(v[c][j] << 16);
        const float b = __uint_as_float(v[c][j] & 0xffff0000u);
        ss += a * a + b * b;
      }
    }
  }
  ss = wave_sum(ss);
  const float r = 1.0f / sqrtf(ss / (float)R + eps);
  const u32x4* wr = reinterpret_cast<const u32x4*>(w);
  u32x4* yr = reinterpret_cast<u32x4*>(yrow);
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int ch = lane + 64 * c;
    if (ch < nch) {
      const u32x4 g = wr[ch];
      u32x4 o;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float a = __uint_as_float(v[c][j] << 16) * r * __uint_as_float(g[j] << 16);
        const float b = __uint_as_float(v[c][j] & 0xffff0000u) * r * __uint_as_float(g[j] & 0xffff0000u);
        o[j] = OT::pack2(a, b);
      }
      yr[ch] = o;
    }
  }
}

template <int NCH, class OT>
__global__ void __launch_bounds__(256) rmsnorm_vec_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                                                          float eps, uint16_t* __restrict__ y, int n, int R) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n) return;
  rms_row<NCH, OT>(x + (size_t)row * R, w, eps, y + (size_t)row * R, R, threadIdx.x & 63);
}

// The latent RMSNorm of a token and the rotation of its shared rotary key in
// one pass (one wavefront per token): the key of token (b, t) is rotated once
// at pos[b*T + t] (t when pos is null) and written to k_rot[b, t, :] in fp16,
// the form the prefill attention reads for every head (Kimi-K2 "Query content
// heads", section "Join query parts": the rotary key is rotated at its
// position; GLM-5 "Normalized key-value latent": one rotary key per token,
// shared by all heads).
template <int NCH>
__global__ void __launch_bounds__(256) latent_prepare_kernel(LatentPrepareArgs a) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= a.n) return;
  rms_row<NCH, F16>(a.x + (size_t)row * a.R, a.w, a.eps, a.y + (size_t)row * a.R, a.R, lane);
  const int half = a.Dr >> 1;
  int p = a.pos ? a.pos[row] : row % a.T;
  p = min(max(p, 0), a.table_len - 1);
  const uint16_t* src = a.k_pe + (size_t)row * a.Dr;
  uint16_t* dst = a.k_rot + (size_t)row * a.Dr;
  for (int i = lane; i < half; i += 64) {
    const int ia = a.pairing ? 2 * i : i;
    const int ib = a.pairing ? 2 * i + 1 : i + half;
    const float c = a.cos[(size_t)p * half + i];
    const float s = a.sin[(size_t)p * half + i];
    const float xa = bf2f(src[ia]), xb = bf2f(src[ib]);
    dst[ia] = f2h(xa * c - xb * s);
    dst[ib] = f2h(xb * c + xa * s);
  }
}

// Any width: two passes over the row with scalar loads.
template <class OT>
__global__ void __launch_bounds__(256) rmsnorm_any_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                                                          float eps, uint16_t* __restrict__ y, int n, int R) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= n) return;
  const uint16_t* xr = x + (size_t)row * R;
  float ss = 0.f;
  for (int i = lane; i < R; i += 64) {
    const float a = bf2f(xr[i]);
    ss += a * a;
  }
  ss = wave_sum(ss);
  const float r = 1.0f / sqrtf(ss / (float)R + eps);
  uint16_t* yr = y + (size_t)row * R;
  for (int i = lane; i < R; i += 64) yr[i] = OT::enc(bf2f(xr[i]) * r * bf2f(w[i]));
}

template <class OT>
static void launch_rmsnorm_t(const uint16_t* x, const uint16_t* w, float eps, uint16_t* y, int n, int R,
                             hipStream_t stream) {
  const dim3 grid((n + 3) / 4), block(256);
  const bool aligned = ((((uintptr_t)x) | ((uintptr_t)w) | ((uintptr_t)y)) & 15) == 0;
  if (aligned && (R % 8) == 0 && R <= 512) {
    hipLaunchKernelGGL((rmsnorm_vec_kernel<1, OT>), grid, block, 0, stream, x, w, eps, y, n, R);
  } else if (aligned && (R % 8) == 0 && R <= 1024) {
    hipLaunchKernelGGL((rmsnorm_vec_kernel<2, OT>), grid, block, 0, stream, x, w, eps, y, n, R);
  } else if (aligned && (R % 8) == 0 && R <= 4096) {
    hipLaunchKernelGGL((rmsnorm_vec_kernel<8, OT>), grid, block, 0, stream, x, w, eps, y, n, R);
  } else {
    hipLaunchKernelGGL(rmsnorm_any_kernel<OT>, grid, block, 0, stream, x, w, eps, y, n, R);
  }
}

hipError_t launch_rmsnorm(const uint16_t* x, const uint16_t* w, float eps, uint16_t* y, int n, int R, int out_dtype,
                          hipStream_t stream) {
  if (out_dtype == BF16::code)
    launch_rmsnorm_t<BF16>(x, w, eps, y, n, R, stream);
  else
    launch_rmsnorm_t<F16>(x, w, eps, y, n, R, stream);
  return hipGetLastError();
}

hipError_t launch_latent_prepare(const LatentPrepareArgs& a, hipStream_t stream) {
  const dim3 grid((a.n + 3) / 4), block(256);
  if (a.R <= 512)
    hipLaunchKernelGGL(latent_prepare_kernel<1>, grid, block, 0, stream, a);
  else if (a.R <= 1024)
    hipLaunchKernelGGL(latent_prepare_kernel<2>, grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL(latent_prepare_kernel<8>, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
