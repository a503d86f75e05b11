// kv_b_proj up-projection with the head split fused into the epilogue
// (equation page "Read the equation", "Original context": kv_b_proj of the
// normalised latent, viewed [B, T, H, Dn+Dv], moved head-major and split into
// k_nope and value; GLM-5 "Normalized key-value latent", expand_kv).
//
// GEMM C^T[n][tok] = W[n][:] . c[tok][:] on bf16 MFMA 32x32x16 with fp32
// accumulation. The normalised latent arrives in fp32 and is split on its way
// into LDS into hi = bf16(c) and lo = bf16(c - hi); every W fragment is
// multiplied by both, so the latent enters the product to 16 significant bits
// and the only bf16 rounding left is the one of each output. Both operands
// are K-contiguous (nn.Linear weight [N, R] and latent [M, R]), so each lane
// feeds the MFMA with one 16-byte LDS read per operand. Computing C^T puts
// four consecutive output columns n in one lane, which the epilogue packs
// into one 8-byte store straight into the head-major k_nope / v layout (a
// 4-column group never straddles a head or the k/v boundary because Dn and Dv
// are multiples of 8).
//
// With v_cols set, values are written transposed (V^T [B, H, Dv, v_ld], the
// layout the prefill attention reads): one 2-byte store per value, 32
// consecutive tokens per store instruction.
//
// Workgroup tile 128 n x 128 tokens, 4 waves in 2x2, each 64 x 64 (2x2 MFMA
// tiles); K staged 32 at a time, double-buffered in LDS with a 16-byte row
// pad; global loads for stage s+1 are in flight while stage s is multiplied.
#include "common.hpp"
#include "launch.hpp"

namespace mla {

namespace {
constexpr int TN = 128;       // W rows (output columns) per workgroup
constexpr int TM = 128;       // tokens per workgroup
constexpr int BK = 32;        // reduction depth per LDS stage
constexpr int LDK = BK + 8;   // LDS row stride (bf16 elements), 16-byte pad
}  // namespace

template <class ET>
__global__ void __launch_bounds__(256, 2) kv_expand_kernel(ExpandArgs a, int M, int N) {
  __shared__ __attribute__((aligned(16))) uint16_t sW[2][TN * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t sAh[2][TM * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t sAl[2][TM * LDK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int n0 = blockIdx.x * TN;
  const int m0 = blockIdx.y * TM;
  const int R = a.R;
  const int nstage = (R + BK - 1) / BK;

  // W loader: chunk id = tid + 256*j (j < 2): row = id >> 2, 8 bf16 at kc*8
  // latent loader: chunk id = tid + 256*j (j < 4): row = id >> 3, 4 fp32 at kc*4
  u32x4 rw[2];
  f32x4 ra[4];
  auto gload = [&](int s) {
    const int k0 = s * BK;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int id = tid + 256 * j;
      const int row = id >> 2, kc = id & 3;
      const int k = k0 + kc * 8;
      const int n = n0 + row;
      u32x4 z = {0u, 0u, 0u, 0u};
      rw[j] = (n < N && k < R) ? *reinterpret_cast<const u32x4*>(a.W + (size_t)n * R + k) : z;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int id = tid + 256 * j;
      const int row = id >> 3, kc = id & 7;
      const int k = k0 + kc * 4;
      const int m = m0 + row;
      f32x4 z = {0.f, 0.f, 0.f, 0.f};
      // R is a multiple of 8, so a 4-wide chunk is either all inside or all outside
      ra[j] = (m < M && k < R) ? *reinterpret_cast<const f32x4*>(a.c + (size_t)m * R + k) : z;
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int id = tid + 256 * j;
      const int row = id >> 2, kc = id & 3;
      *reinterpret_cast<u32x4*>(&sW[buf][row * LDK + kc * 8]) = rw[j];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int id = tid + 256 * j;
      const int row = id >> 3, kc = id & 7;
      u32x2 hi, lo;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float x0 = ra[j][2 * e], x1 = ra[j][2 * e + 1];
        const uint16_t h0 = f2bf(x0), h1 = f2bf(x1);
        hi[e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
        lo[e] = pack2bf(x0 - bf2f(h0), x1 - bf2f(h1));
      }
      *reinterpret_cast<u32x2*>(&sAh[buf][row * LDK + kc * 4]) = hi;
      *reinterpret_cast<u32x2*>(&sAl[buf][row * LDK + kc * 4]) = lo;
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  gload(0);
  lstore(0);
  __syncthreads();

  const int lrow = lane & 31;
  const int lk = (lane >> 5) * 8;
  for (int s = 0; s < nstage; ++s) {
    const int buf = s & 1;
    if (s + 1 < nstage) gload(s + 1);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 fw[2], fh[2], fl[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        fw[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(&sW[buf][(wn * 64 + i * 32 + lrow) * LDK + kk * 16 + lk]));
        const int ao = (wm * 64 + i * 32 + lrow) * LDK + kk * 16 + lk;
        fh[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(&sAh[buf][ao]));
        fl[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(&sAl[buf][ao]));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          acc[i][j] = mfma32(fw[i], fl[j], acc[i][j]);
          acc[i][j] = mfma32(fw[i], fh[j], acc[i][j]);
        }
    }
    if (s + 1 < nstage) lstore(buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds C^T rows n = base + (r/4)*8 + (lane/32)*4 + r%4 for
  // token column lane%32 of each 32x32 tile
  const int DnDv = a.Dn + a.Dv;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int tok = m0 + wm * 64 + j * 32 + lrow;
    if (tok >= M) continue;
    const int b = tok / a.T;
    const int t = tok - b * a.T;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * 64 + i * 32 + g * 8 + (lane >> 5) * 4;
        if (n >= N) continue;
        const int h = n / DnDv;
        const int c = n - h * DnDv;
        const size_t rowi = ((size_t)b * a.H + h) * a.Tcap + a.t_off + t;
        if (c >= a.Dn && a.v_cols) {
          // V^T: the four value columns are four rows of [Dv, v_ld]; the lane
          // writing the cache's last column also zeroes the row padding
          const int col = a.t_off + t;
          uint16_t* dst = a.v + (((size_t)b * a.H + h) * a.Dv + (c - a.Dn)) * a.v_ld + col;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            dst[(size_t)e * a.v_ld] = ET::enc(acc[i][j][g * 4 + e]);
            if (col == a.Tcap - 1)
              for (int z = col + 1; z < a.v_ld; ++z) dst[(size_t)e * a.v_ld + (z - col)] = 0;
          }
          continue;
        }
        uint16_t* dst = (c < a.Dn) ? a.k + rowi * a.k_ld + c : a.v + rowi * a.Dv + (c - a.Dn);
        u32x2 o;
        o[0] = ET::pack2(acc[i][j][g * 4 + 0], acc[i][j][g * 4 + 1]);
        o[1] = ET::pack2(acc[i][j][g * 4 + 2], acc[i][j][g * 4 + 3]);
        *reinterpret_cast<u32x2*>(dst) = o;
      }
    }
  }
}

hipError_t launch_kv_expand(const ExpandArgs& a, hipStream_t stream) {
  const int M = a.B * a.T;
  const int N = a.H * (a.Dn + a.Dv);
  const dim3 grid((N + TN - 1) / TN, (M + TM - 1) / TM);
  if (a.kv_dtype == F16::code)
    hipLaunchKernelGGL(kv_expand_kernel<F16>, grid, dim3(256), 0, stream, a, M, N);
  else
    hipLaunchKernelGGL(kv_expand_kernel<BF16>, grid, dim3(256), 0, stream, a, M, N);
  return hipGetLastError();
}

// Rotation of the shared rotary key (Kimi-K2 "Query content heads", "Join
// query parts": the key's rotary part is one rotated key shared by all heads)
// and its broadcast into H head rows. One thread per (token, pair).
template <class ET>
__global__ void __launch_bounds__(256) rotate_key_kernel(RotKeyArgs a) {
  const int half = a.Dr >> 1;
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long)a.B * a.T * half) return;
  const int i = (int)(idx % half);
  const long bt = idx / half;
  const int t = (int)(bt % a.T);
  const int b = (int)(bt / a.T);
  int p = a.pos ? a.pos[bt] : a.t_off + t;
  p = min(max(p, 0), a.table_len - 1);
  const float c = a.cos[(size_t)p * half + i];
  const float s = a.sin[(size_t)p * half + i];
  const int ia = a.pairing ? 2 * i : i;
  const int ib = a.pairing ? 2 * i + 1 : i + half;
  const uint16_t* src = a.k_pe + bt * a.Dr;
  const float xa = bf2f(src[ia]);
  const float xb = bf2f(src[ib]);
  const uint16_t ya = ET::enc(xa * c - xb * s);
  const uint16_t yb = ET::enc(xb * c + xa * s);
  for (int h = 0; h < a.H; ++h) {
    uint16_t* d = a.dst + (((size_t)b * a.H + h) * a.Tcap + a.t_off + t) * a.ld + a.col;
    d[ia] = ya;
    d[ib] = yb;
  }
}

hipError_t launch_rotate_key(const RotKeyArgs& a, hipStream_t stream) {
  const long total = (long)a.B * a.T * (a.Dr / 2);
  const long blocks = (total + 255) / 256;
  if (a.dtype == F16::code)
    hipLaunchKernelGGL(rotate_key_kernel<F16>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(rotate_key_kernel<BF16>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
