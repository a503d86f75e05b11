// Decode attention of one new token per sequence against an expanded per-head
// cache (Kimi-K2 "Query content heads", section "Join query parts": after the
// cache update, scaled scores over every cached key, fp32 softmax, value mix).
//
// The cache stream (K rows of Dn+Dr, V rows of Dv, bf16) dominates: the kernel
// is HBM-bound at about 1 flop per byte, so it uses VALU dot products rather
// than MFMA. Split-K: workgroup (split, head, sequence) handles a contiguous
// range of cached positions in chunks of 512 keys:
//   pass 1  8 lanes per key, 16-byte loads, fp32 dot with the rotated query
//           held in LDS, scores (log2 units) to LDS;
//   softmax chunk maximum and sum, running maximum across chunks;
//   pass 2  each thread owns 8 value columns of 1/KG of the chunk's keys,
//           16-byte loads, fp32 accumulation.
// The cache stream is read once, so its loads are nontemporal (the nt cache
// policy): on this chip that lifts a pure streaming read from about 6.2 to
// about 7 TB/s.
// A split writes (max, sum, unnormalised output) and a combine kernel merges
// the splits with the log-sum-exp rule; a single split writes the output.
#include <mutex>

#include "common.hpp"
#include "launch.hpp"

namespace mla {

namespace {
constexpr int CH = 512;  // keys per chunk
constexpr float kLog2e = 1.4426950408889634f;
}  // namespace

__device__ __forceinline__ float block_reduce(float v, float* red, bool is_max) {
  v = is_max ? wave_max(v) : wave_sum(v);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) r = is_max ? fmaxf(r, red[w]) : r + red[w];
  return r;
}

template <class CT, int DQK, int DV>
__global__ void __launch_bounds__(256) decode_kernel(DecodeArgs a) {
  constexpr int QCH = DQK / 8;         // 16-byte chunks per K row
  constexpr int KPL = (QCH + 7) / 8;   // chunks per lane (8 lanes per key)
  constexpr int VCH = DV / 8;          // 16-byte chunks per V row
  constexpr int KG = 256 / VCH;        // key groups in pass 2
  static_assert(256 % VCH == 0, "DV");

  __shared__ float sq[DQK];
  __shared__ float sc[CH];
  __shared__ float red[4];
  __shared__ float sacc[KG * DV];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int split = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int S = gridDim.x;
  const int Dn = a.Dn, Dr = a.Dr;

  const int L = min(max(a.seq_len[b], 1), a.Tcap);
  const int per = (L + S - 1) / S;
  const int s0 = split * per;
  const int s1 = min(L, s0 + per);

  const size_t bh = (size_t)b * a.H + h;
  const uint16_t* kc = a.k_cache + bh * a.Tcap * DQK;
  const uint16_t* vc = a.v_cache + bh * a.Tcap * DV;

  // rotated query in fp32
  if (tid < DQK) {
    const uint16_t* qr = a.q + bh * DQK;
    float x = bf2f(qr[tid]);
    if (tid >= Dn) {
      int p = min(max(a.q_pos[b], 0), a.table_len - 1);
      const int re = tid - Dn;
      int pi, partner;
      bool first;
      if (a.pairing) {
        pi = re >> 1;
        first = (re & 1) == 0;
        partner = first ? re + 1 : re - 1;
      } else {
        first = re < Dr / 2;
        pi = first ? re : re - Dr / 2;
        partner = first ? re + Dr / 2 : re - Dr / 2;
      }
      const float xp = bf2f(qr[Dn + partner]);
      const float c = a.cos[(size_t)p * (Dr / 2) + pi];
      const float s = a.sin[(size_t)p * (Dr / 2) + pi];
      x = first ? (x * c - xp * s) : (x * c + xp * s);
    }
    sq[tid] = x;
  }
  __syncthreads();

  // this lane's query chunks (pass 1): chunk cc = ll + 8*i
  const int ll = lane & 7;
  float qv[KPL][8];
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int cc = ll + 8 * i;
#pragma unroll
    for (int e = 0; e < 8; ++e) qv[i][e] = (cc < QCH) ? sq[cc * 8 + e] : 0.f;
  }
  const float sl2 = a.scale * kLog2e;

  const int dc = tid % VCH;
  const int kgi = tid / VCH;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  for (int c0 = s0; c0 < s1; c0 += CH) {
    const int n = min(CH, s1 - c0);
    // pass 1: scores
    for (int kb = wave * 8; kb < n; kb += 32 * 4) {
      float dots[4];
      u32x4 kv[4][KPL];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int kk = kb + u * 32 + (lane >> 3);
#pragma unroll
        for (int i = 0; i < KPL; ++i) {
          const int cc = ll + 8 * i;
          u32x4 z = {0u, 0u, 0u, 0u};
          kv[u][i] = (kk < n && cc < QCH)
                         ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kc + (size_t)(c0 + kk) * DQK + cc * 8))
                         : z;
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        float d = 0.f;
#pragma unroll
        for (int i = 0; i < KPL; ++i) {
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            d += CT::lo(kv[u][i][e2]) * qv[i][2 * e2];
            d += CT::hi(kv[u][i][e2]) * qv[i][2 * e2 + 1];
          }
        }
        d += __shfl_xor(d, 1, 64);
        d += __shfl_xor(d, 2, 64);
        d += __shfl_xor(d, 4, 64);
        dots[u] = d;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int kk = kb + u * 32 + (lane >> 3);
        if (ll == 0 && kk < CH) sc[kk] = (kk < n) ? dots[u] * sl2 : -INFINITY;
      }
    }
    __syncthreads();
    // chunk maximum, running maximum, probabilities
    float mx = -INFINITY;
    for (int i = tid; i < n; i += 256) mx = fmaxf(mx, sc[i]);
    mx = block_reduce(mx, red, true);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float ps = 0.f;
    for (int i = tid; i < n; i += 256) {
      const float p = __builtin_amdgcn_exp2f(sc[i] - m_new);
      sc[i] = p;
      ps += p;
    }
    ps = block_reduce(ps, red, false);  // its barriers also publish sc
    l_run = l_run * alpha + ps;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= alpha;
    // pass 2: values
    for (int k0 = kgi; k0 < n; k0 += KG * 4) {
      u32x4 vv[4];
      float pw[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int kk = k0 + u * KG;
        u32x4 z = {0u, 0u, 0u, 0u};
        vv[u] = (kk < n) ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vc + (size_t)(c0 + kk) * DV + dc * 8))
                         : z;
        pw[u] = (kk < n) ? sc[kk] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          acc[2 * e2] += pw[u] * CT::lo(vv[u][e2]);
          acc[2 * e2 + 1] += pw[u] * CT::hi(vv[u][e2]);
        }
      }
    }
    __syncthreads();  // sc is rewritten by the next chunk
  }

  // reduce the KG key groups
#pragma unroll
  for (int e = 0; e < 8; ++e) sacc[kgi * DV + dc * 8 + e] = acc[e];
  __syncthreads();
  if (tid < DV) {
    float o = 0.f;
    for (int k = 0; k < KG; ++k) o += sacc[k * DV + tid];
    if (S == 1) {
      a.out[bh * DV + tid] = f2bf(o / l_run);
    } else {
      const size_t pi = bh * S + split;
      a.part_o[pi * DV + tid] = o;
      if (tid == 0) {
        a.part_ml[pi * 2 + 0] = m_run;
        a.part_ml[pi * 2 + 1] = l_run;
      }
    }
  }
}

// Merge split partials: O = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
__global__ void __launch_bounds__(256) decode_combine_kernel(const float* __restrict__ part_o,
                                                             const float* __restrict__ part_ml, int S, int DV,
                                                             uint16_t* __restrict__ out) {
  const size_t bh = blockIdx.x;
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, part_ml[(bh * S + s) * 2]);
  for (int d = threadIdx.x; d < DV; d += blockDim.x) {
    float num = 0.f, den = 0.f;
    for (int s = 0; s < S; ++s) {
      const float ms = part_ml[(bh * S + s) * 2];
      const float w = (ms == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ms - M);
      num += w * part_o[(bh * S + s) * DV + d];
      den += w * part_ml[(bh * S + s) * 2 + 1];
    }
    out[bh * DV + d] = f2bf(num / den);
  }
}

bool decode_supported(int Dqk, int Dv) {
  return (Dqk == 192 && Dv == 128) || (Dqk == 256 && Dv == 256) || (Dqk == 48 && Dv == 32);
}

int decode_auto_splits(int B, int H, int Tcap) {
  // aim at >= 2048 workgroups (8 per CU) without splits shorter than 256 keys
  const int bh = B * H;
  if (bh <= 0) return 1;  // an empty batch: no launch follows
  int s = (2048 + bh - 1) / bh;
  const int smax = (Tcap + 255) / 256;
  if (s > smax) s = smax;
  if (s < 1) s = 1;
  if (s > 256) s = 256;
  return s;
}

size_t decode_workspace_bytes(int B, int H, int Dv, int splits) {
  if (splits <= 1) return 0;
  const size_t n = (size_t)B * H * splits;
  const size_t o = ((n * Dv * sizeof(float)) + 255) / 256 * 256;
  return o + n * 2 * sizeof(float);
}

template <class CT>
static void launch_decode_t(const DecodeArgs& a, hipStream_t stream, bool& ok) {
  const dim3 grid(a.num_splits, a.H, a.B), block(256);
  const int Dqk = a.Dn + a.Dr;
  ok = true;
  if (Dqk == 192 && a.Dv == 128) {
    hipLaunchKernelGGL((decode_kernel<CT, 192, 128>), grid, block, 0, stream, a);
  } else if (Dqk == 256 && a.Dv == 256) {
    hipLaunchKernelGGL((decode_kernel<CT, 256, 256>), grid, block, 0, stream, a);
  } else if (Dqk == 48 && a.Dv == 32) {
    hipLaunchKernelGGL((decode_kernel<CT, 48, 32>), grid, block, 0, stream, a);
  } else {
    ok = false;
  }
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  bool ok;
  if (a.cache_dtype == F16::code)
    launch_decode_t<F16>(a, stream, ok);
  else
    launch_decode_t<BF16>(a, stream, ok);
  if (!ok) return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.num_splits <= 1) return e;
  hipLaunchKernelGGL(decode_combine_kernel, dim3(a.B * a.H), dim3(128), 0, stream, a.part_o, a.part_ml,
                     a.num_splits, a.Dv, a.out);
  return hipGetLastError();
}

// Scratch of the allocation-free decode entry point: the split partials
// (o [B, H, S, Dv], then (m, l) [B, H, S, 2], as in a caller's workspace)
// live in this array, one copy per GPU, held until the process ends. Every
// split writes all of its partials and the combine reads only those, so
// nothing here needs clearing between calls; calls that overlap on one GPU
// race on it.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

hipError_t decode_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* dev_ptr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!dev_ptr[dev]) {
    // the array's device address on this (current) device; the host-side
    // name is only a stand-in and must never reach a kernel
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    dev_ptr[dev] = p;
  }
  *ptr = dev_ptr[dev];
  return hipSuccess;
}

}  // namespace mla
