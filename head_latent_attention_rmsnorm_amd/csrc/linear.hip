// Linear layers around the latent attention: Y = X W^T (+ bias), the
// nn.Linear form of q_a_proj, q_b_proj, kv_a_proj_with_mqa and o_proj
// (Kimi-K2 "Query content heads" / "Key heads", the MLA constructor: query
// down-projection, query RMSNorm and up-projection, joint key-value
// down-projection that also emits the shared rotary key, output projection;
// GLM-5 "Normalized key-value latent": the same layers). bf16 operands,
// fp32 accumulation, bf16 out.
//
// Layout modes remove the transposes around the attention:
//  - X may be head-major [B, Hx, T, Dx] (o_proj reads the attention output
//    [B, H, T, Dv] as its [B*T, H*Dv] input without a copy);
//  - Y may be head-major [B, Hy, T, Dy] (q_b_proj writes the attention's
//    query layout [B, H, T, Dqk] directly), or split at column ys into two
//    row-major outputs (kv_a_proj_with_mqa writes the latent [B*T, R] and
//    the rotary key [B*T, Dr] separately).
//
// Design (gfx950): 256 x 256 output tile per workgroup, 8 waves of 64 (N) x
// 128 (M); bf16 MFMA 32x32x16 computing C^T = W X^T, so a lane holds 4
// consecutive output columns of one row. X and W move global -> LDS in
// 64-deep stages with 16-byte LDS-direct loads, double-buffered, in the
// swizzled row-segment image (whole 128-byte row segments per load, every
// operand read one conflict-free 16-byte LDS read); the descriptors' range
// checks zero-fill rows past M and N. The epilogue stages each wave's tile
// through LDS so that every global store writes 128 contiguous bytes.
// Tile order: workgroup ids go round-robin over the 8 XCDs, so each XCD is
// given a contiguous range of output tiles, walked in groups of 4 tile rows
// (the 32 workgroups an XCD runs at once then share 4 X tiles and 8 W tiles
// in its L2); 4-8% faster than the plain column-major order on the
// projection shapes.
#include "common.hpp"
#include "launch.hpp"

namespace mla {

namespace {
constexpr int GM = 256, GN = 256, GK = 64;  // workgroup tile: X rows, W rows, depth per stage
constexpr int XG = GM / 32, WG = GN / 32;   // 32-row operand groups per stage
constexpr int NBLK = (XG + WG) * 4;         // 1 KB blocks per stage (4 k-steps per group)
constexpr int STAGE = NBLK * 1024;          // 64 KB
constexpr int LPW = NBLK / 8;               // loads per wave per stage
constexpr int GROUP_ROWS = 4;               // tile rows per group of the tile order

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, voff, 0, 0, 0);
}
}  // namespace

__global__ void __launch_bounds__(512, 2) linear_kernel(LinearArgs a, int nmt, int nnt) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  __builtin_assume(wave >= 0 && wave < 8);
  const int l32 = lane & 31, g = lane >> 5;
  const int ntile = nmt * nnt, per = (ntile + 7) / 8;
  const int L = (blockIdx.x & 7) * per + (blockIdx.x >> 3);  // XCD-contiguous tile index
  if (L >= ntile) return;  // padding workgroup: the whole block exits
  const int gm0 = (L / (GROUP_ROWS * nnt)) * GROUP_ROWS, lg = L % (GROUP_ROWS * nnt);
  const int gsz = min(GROUP_ROWS, nmt - gm0);
  const int mt = gm0 + lg % gsz, nt = lg / gsz;
  const int m0 = mt * GM, n0 = nt * GN;
  const int M = a.M, N = a.N, K = a.K;

  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, (uint32_t)((size_t)M * K * 2));
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.w, (uint32_t)((size_t)N * K * 2));
  // This wave's loads: blocks wave + 8j, X blocks first (group, block in the
  // group). Lane offsets for the stage at k0 = 0; a stage adds a uniform
  // offset (head-major X: the stage's head and column within it).
  uint32_t voff[LPW];
  bool isx[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int bi = wave + 8 * j;
    isx[j] = bi < XG * 4;
    const int gi = (bi % (XG * 4)) / 4, rb = bi % 4;
    int r, x;
    frag_slot<4>(rb, lane, r, x);
    const int kx = 8 * x;  // column within the stage
    if (isx[j]) {
      const int m = m0 + 32 * gi + r;
      if (a.x_mode == 0) {
        voff[j] = (uint32_t)(((size_t)m * K + kx) * 2);
      } else {
        const int b = m / a.xT, t = m - b * a.xT;
        const int Dx = 1 << a.x_dlog2, Hx = K >> a.x_dlog2;
        const size_t e = ((size_t)b * Hx * a.xT + t) * Dx + (size_t)(kx >> a.x_dlog2) * a.xT * Dx + (kx & (Dx - 1));
        voff[j] = (uint32_t)(e * 2);
      }
    } else {
      const int n = n0 + 32 * gi + r;
      voff[j] = (uint32_t)(((size_t)n * K + kx) * 2);
    }
  }
  auto issue = [&](int kt, int buf) __attribute__((always_inline)) {
    const int k0 = kt * GK;
    uint32_t xs;
    if (a.x_mode == 0) {
      xs = (uint32_t)(k0 * 2);
    } else {
      const int Dx = 1 << a.x_dlog2;
      xs = (uint32_t)((((size_t)(k0 >> a.x_dlog2) * a.xT * Dx) + (k0 & (Dx - 1))) * 2);
    }
    const uint32_t ws = (uint32_t)(k0 * 2);
    char* base = smem + buf * STAGE;
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int bi = wave + 8 * j;
      if (isx[j])
        load_lds16(rx, base + bi * 1024, voff[j] + xs);
      else
        load_lds16(rw, base + bi * 1024, voff[j] + ws);
    }
  };

  const int wn = wave & 3, wm = wave >> 2;  // wave tile: W groups 2wn, 2wn+1; X groups 4wm..4wm+3
  const int rd0 = frag_read0<4>(l32, g);
  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int nk = K / GK;
  issue(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) issue(kt + 1, cur ^ 1);
    const char* sb = smem + cur * STAGE;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int off = rd0 ^ (32 * c);
      u32x4 wf[2], xf[4];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        wf[i] = *reinterpret_cast<const u32x4*>(sb + (XG + 2 * wn + i) * 4096 + off);
#pragma unroll
      for (int j = 0; j < 4; ++j) xf[j] = *reinterpret_cast<const u32x4*>(sb + (4 * wm + j) * 4096 + off);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = BF16::mma(wf[i], xf[j], acc[i][j]);
    }
    // the next stage's loads have landed and every wave is done with this one
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // ---- epilogue. C^T lane layout: column m = l32 of X group j, rows
  // n = 8*(e>>2) + 4g + (e&3) of W group i. Stage the wave's 128 (m) x 64 (n)
  // tile in its own 16 KB of LDS: row m, 16-byte chunk q (8 columns) at
  // position q ^ (m & 7).
  char* st = smem + wave * 16384;
  const int nw0 = n0 + 64 * wn, mw0 = m0 + 128 * wm;
  // the bias of this lane's 32 columns, all loads issued together
  float bv[2][4][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
      for (int e = 0; e < 4; ++e) bv[i][q4][e] = 0.f;
  if (a.bias) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int n = nw0 + 32 * i + 8 * q4 + 4 * g;  // 4 columns, N a multiple of 8
        if (n < N) {
          const u32x2 bb = *reinterpret_cast<const u32x2*>(a.bias + n);
          bv[i][q4][0] = __uint_as_float(bb[0] << 16);
          bv[i][q4][1] = __uint_as_float(bb[0] & 0xffff0000u);
          bv[i][q4][2] = __uint_as_float(bb[1] << 16);
          bv[i][q4][3] = __uint_as_float(bb[1] & 0xffff0000u);
        }
      }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = 32 * j + l32;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int nl = 32 * i + 8 * q4 + 4 * g;  // first of the 4 columns, within the wave's 64
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q4 + e] + bv[i][q4][e];
        u32x2 o;
        o[0] = pack2bf(v[0], v[1]);
        o[1] = pack2bf(v[2], v[3]);
        *reinterpret_cast<u32x2*>(st + m * 128 + 16 * ((nl >> 3) ^ (m & 7)) + 8 * ((nl >> 2) & 1)) = o;
      }
    }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's staging writes
  // each store instruction: 8 rows x 128 bytes
  const int cq = lane & 7;
#pragma unroll 4
  for (int rep = 0; rep < 16; ++rep) {
    const int ml = (lane >> 3) + 8 * rep;
    const int m = mw0 + ml, n = nw0 + 8 * cq;
    if (m >= M || n >= N) continue;
    const u32x4 v = *reinterpret_cast<const u32x4*>(st + ml * 128 + 16 * (cq ^ (ml & 7)));
    uint16_t* dst;
    if (a.y_mode == 0) {
      dst = a.y0 + (size_t)m * N + n;
    } else if (a.y_mode == 1) {
      const int b = m / a.yT, t = m - b * a.yT;
      const int h = n / a.yD, d = n - h * a.yD;
      dst = a.y0 + (((size_t)b * (N / a.yD) + h) * a.yT + t) * a.yD + d;
    } else {
      dst = n < a.ys ? a.y0 + (size_t)m * a.ys + n : a.y1 + (size_t)m * (N - a.ys) + (n - a.ys);
    }
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst));  // written once: nontemporal
  }
}

hipError_t launch_linear(const LinearArgs& a, hipStream_t stream) {
  const int nmt = (a.M + GM - 1) / GM, nnt = (a.N + GN - 1) / GN;
  const int per = (nmt * nnt + 7) / 8;
  hipLaunchKernelGGL(linear_kernel, dim3((unsigned)(8 * per)), dim3(512), 0, stream, a, nmt, nnt);
  return hipGetLastError();
}

}  // namespace mla
