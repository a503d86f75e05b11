// cos/sin table builder (Kimi-K2 "RoPE coefficients", section "Generate RoPE
// coefficients": under YaRN each pair's frequency moves from base^(-2i/Dr)
// towards base^(-2i/Dr)/factor by the linear ramp's fraction r_i over the
// correction band; angles p * frequency; sin/cos scaled by the mscale
// ratio). One thread per (position, pair); ramp, frequencies and angles in
// fp32, as the page computes them.
#include "common.hpp"
#include "launch.hpp"

namespace mla {

__global__ void __launch_bounds__(256) rope_table_kernel(RopeResolved r, int n_pos, float* __restrict__ cos_out,
                                                         float* __restrict__ sin_out) {
  const int half = r.dim >> 1;
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long)n_pos * half) return;
  const int p = (int)(idx / half);
  const int i = (int)(idx - (long)p * half);
  // exponent 2i/dim, as arange(0, dim, 2) / dim in fp32
  const float e = (float)(2 * i) / (float)r.dim;
  const float powb = powf(r.base, e);
  const float theta = 1.0f / powb;  // unscaled frequency
  float inv = theta;
  if (r.yarn) {
    // fraction of the way to the interpolated frequency theta / factor:
    // 0 below the band, 1 above it, linear across it
    const float frac = fminf(fmaxf(((float)i - r.low) / (r.high - r.low), 0.0f), 1.0f);
    inv = theta + (1.0f / (r.factor * powb) - theta) * frac;
  }
  const float ang = (float)p * inv;
  float s, c;
  sincosf(ang, &s, &c);
  cos_out[idx] = c * r.mscale;
  sin_out[idx] = s * r.mscale;
}

hipError_t launch_rope_table(const RopeResolved& r, int n_pos, float* cos_out, float* sin_out,
                             hipStream_t stream) {
  const long total = (long)n_pos * (r.dim / 2);
  const int threads = 256;
  const long blocks = (total + threads - 1) / threads;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream, r, n_pos,
                     cos_out, sin_out);
  return hipGetLastError();
}

}  // namespace mla
