// cos/sin table builder (Kimi-K2 "RoPE coefficients", section "Generate RoPE
// coefficients": frequency blend by the YaRN linear ramp, outer product with
// the positions, sin/cos scaled by the mscale ratio). One thread per
// (position, pair); the ramp, frequencies and angles are fp32 as on the page.
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
  const float extra = 1.0f / powb;  // unscaled frequency
  float inv = extra;
  if (r.yarn) {
    const float inter = 1.0f / (r.factor * powb);  // interpolated frequency
    float ramp = ((float)i - r.low) / (r.high - r.low);
    ramp = fminf(fmaxf(ramp, 0.0f), 1.0f);
    const float keep = 1.0f - ramp;  // weight of the unscaled frequency
    inv = inter * (1.0f - keep) + extra * keep;
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
