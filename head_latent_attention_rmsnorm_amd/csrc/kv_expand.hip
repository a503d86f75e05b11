// kv_b_proj up-projection with the head split fused into the epilogue
// (equation page "Read the equation", "Original context": kv_b_proj of the
// normalised latent, viewed [B, T, H, Dn+Dv], moved head-major and split into
// k_nope and value; GLM-5 "Normalized key-value latent", expand_kv).
//
// GEMM kv[tok][n] = sum_r c[tok][r] W[n][r] on fp16 MFMA 32x32x16 with fp32
// accumulation: the normalised latent arrives in fp16, and W (bf16) is
// widened to fp16 on its way into LDS, which is exact for every bf16 value of
// magnitude >= 2^-24 (smaller ones contribute below fp32 resolution of the
// sum). Both operands are K-contiguous (latent [M, R] and nn.Linear weight
// [N, R]), so each MFMA operand is one 16-byte run of a row. Each output
// column n is one element of head h = n / (Dn+Dv): a key element when
// n mod (Dn+Dv) < Dn, else a value element; the epilogue writes it straight
// into the head-major k_nope / v (or V^T) layout.
//
// Two kernels:
//  - expand_tile_kernel: 256 tokens x 256 columns per workgroup, 8 waves of
//    128 tokens x 64 columns, launched once over the key columns of all heads
//    and once over the value columns (Dn and Dv multiples of 64). The latent
//    tiles move global -> LDS with 16-byte LDS-direct buffer loads gathered
//    into MFMA fragment order; W tiles go through registers for the fp16
//    widening and land in the same fragment order; both double-buffered over
//    the reduction. The value launch with V^T output computes C = c W^T (a
//    lane then holds four consecutive tokens of one value column: one 8-byte
//    store into a V^T row); the others compute C^T = W c^T (four consecutive
//    columns of one token: one 8-byte store into a k_nope / v row). Swapping
//    the two MFMA operands is all it takes: an A and a B fragment have the
//    same lane layout.
//  - expand_skinny_kernel: at most 32 tokens (the decode append): one wave per
//    32 columns, operands loaded from global memory straight into registers.
//  - expand_small_kernel: 128 columns x 128 tokens, 4 waves, everything staged
//    through registers; any other shape (a few hundred tokens, head widths
//    that are not multiples of 64, latent widths that are not multiples of
//    128).
#include "common.hpp"
#include "launch.hpp"

namespace mla {

namespace {
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// 8 bf16 (one 16-byte chunk) widened to 8 fp16
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 w) {
  u32x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = pack2h(__uint_as_float(w[e] << 16), __uint_as_float(w[e] & 0xffff0000u));
  return o;
}

__device__ __forceinline__ f32x16 mma16(u32x4 a, u32x4 b, f32x16 c) { return F16::mma(a, b, c); }

// Destination of output column n (global) of token tok: k or v element.
struct ColInfo {
  int h, c;   // head and column within the head's Dn+Dv
  bool is_v;
};
__device__ __forceinline__ ColInfo col_info(const ExpandArgs& a, int n) {
  const int DnDv = a.Dn + a.Dv;
  ColInfo ci;
  ci.h = n / DnDv;
  ci.c = n - ci.h * DnDv;
  ci.is_v = ci.c >= a.Dn;
  return ci;
}

// Store four consecutive columns n..n+3 (same head, same k/v part) of token
// tok into a row-major k_nope or v row.
template <class ET>
__device__ __forceinline__ void store_row4(const ExpandArgs& a, int tok, int n, float x0, float x1, float x2,
                                           float x3) {
  const ColInfo ci = col_info(a, n);
  const int b = tok / a.T;
  const int t = tok - b * a.T;
  const size_t rowi = ((size_t)b * a.H + ci.h) * a.Tcap + a.t_off + t;
  uint16_t* dst = ci.is_v ? a.v + rowi * a.Dv + (ci.c - a.Dn) : a.k + rowi * a.k_ld + ci.c;
  u32x2 o;
  o[0] = ET::pack2(x0, x1);
  o[1] = ET::pack2(x2, x3);
  *reinterpret_cast<u32x2*>(dst) = o;
}

// Store value column n of token tok into V^T; the write of the cache's last
// column also zeroes the row padding.
template <class ET>
__device__ __forceinline__ void store_vt1(const ExpandArgs& a, int tok, int n, float x) {
  const ColInfo ci = col_info(a, n);
  const int b = tok / a.T;
  const int t = tok - b * a.T;
  const int col = a.t_off + t;
  uint16_t* dst = a.v + (((size_t)b * a.H + ci.h) * a.Dv + (ci.c - a.Dn)) * a.v_ld + col;
  dst[0] = ET::enc(x);
  if (col == a.Tcap - 1) {
#pragma unroll 1
    for (int z = col + 1; z < a.v_ld; ++z) dst[z - col] = 0;
  }
}
}  // namespace

// ---------------------------------------------------------------- tile kernel
namespace {
constexpr int XT_M = 256;  // tokens per workgroup
constexpr int XT_N = 256;  // columns per workgroup
constexpr int XT_K = 32;   // reduction depth per stage
constexpr int XT_NB = 4;   // stages in flight (LDS buffers); loads run XT_NB-1 stages ahead
constexpr int XT_R = 512;  // latent width the tile kernel is built for (fully unrolled stages)
}  // namespace

// One part of the columns: the key columns of every head (VPART false: H*Dn
// columns, written to k_nope rows) or the value columns (VPART true: H*Dv
// columns, written to v rows, or to V^T when COLS). Part column n belongs to
// head n / D (D = Dn or Dv) and is row h*(Dn+Dv) + (VPART ? Dn : 0) + n % D
// of W.
template <class ET, bool VPART, bool COLS>
__global__ void __launch_bounds__(512, 2) expand_tile_kernel(ExpandArgs a, int M) {
  constexpr int KS = XT_K / 16;              // 16-deep MFMA steps per stage
  constexpr int XT_BLK = (XT_M / 32) * KS;   // 1 KB fragment blocks per operand per stage
  constexpr int APW = XT_BLK / 8;            // latent LDS-direct loads per wave per stage
  constexpr int WPT = XT_N * XT_K / 8 / 512; // W 16-byte chunks per thread per stage
  // [stage buffer][A blocks | B blocks], each block 64 lanes x 16 bytes
  __shared__ __attribute__((aligned(16))) u32x4 smem[XT_NB][2 * XT_BLK * 64];

  const int D = VPART ? a.Dv : a.Dn;
  const int N = a.H * D;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2;  // 128-token half of the tile
  const int wn = wave & 3;   // 64-column quarter
  const int l32 = lane & 31, g = lane >> 5;
  const int n0 = blockIdx.x * XT_N;
  const int m0 = blockIdx.y * XT_M;
  constexpr int R = XT_R;
  constexpr int nstage = R / XT_K;

  // latent: LDS-direct loads, APW blocks per wave per stage; block bi =
  // (m-tile bi/KS, k-step bi%KS), lane = (row l32, 8 columns at 8g); rows
  // past the last token read as zeros. The descriptor covers this tile's
  // rows only (at most XT_M * R * 2 bytes), so its 32-bit range never wraps
  // however many tokens the call has.
  const uint32_t rows = (uint32_t)min(M - m0, XT_M);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.c + (size_t)m0 * R, rows * (uint32_t)R * 2u);
  uint32_t voff[APW];
#pragma unroll
  for (int i = 0; i < APW; ++i) {
    const int bi = wave + 8 * i;
    voff[i] = (uint32_t)(((bi / KS) * 32 + l32) * R + (bi % KS) * 16 + 8 * g) * 2u;
  }
  auto issue_a = [&](int s, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < APW; ++i) {
      const int bi = wave + 8 * i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)&smem[buf][bi * 64], 16, voff[i], s * XT_K * 2, 0, 0);
    }
  };
  // W: WPT 16-byte chunks per thread per stage, chunk id = tid + 512j: part
  // column n0 + id/(XT_K/8), 8 reduction elements at 8*(id%(XT_K/8));
  // widened in registers and stored at its fragment slot
  constexpr int CPR = XT_K / 8;  // chunks per W row per stage
  // (columns past the part are read from W row 0: their products only feed
  // waves that store nothing, and every thread issues the same loads, which
  // the vmcnt bookkeeping below relies on)
  const uint16_t* wrow[WPT];
#pragma unroll
  for (int j = 0; j < WPT; ++j) {
    const int n = n0 + (tid + 512 * j) / CPR;
    const int h = n / D;
    const size_t row = n < N ? (size_t)h * (a.Dn + a.Dv) + (VPART ? a.Dn : 0) + (n - h * D) : 0;
    wrow[j] = a.W + row * R + ((tid + 512 * j) % CPR) * 8;
  }
  // W fragment slots are XOR-permuted: slot (row r, 8-element chunk kc of
  // the stage) sits at (r ^ X(kc)) + 32(kc & 1) of its k-step's block, with
  // X = 0, 10, 4, 14. The 16 stores of a 16-lane group (rows 4q..4q+3, chunks
  // 0..3) then land on 16 different bank groups, and so do the 8 of every
  // 8-lane half (without the permutation the four chunks of a row hit one
  // bank group, a 4-way conflict); an operand read (16 lanes, 16
  // consecutive rows, one chunk) still covers all 16.
  auto wslot = [](int r, int kc) __attribute__((always_inline)) { return (r ^ ((2 * kc) ^ (8 * (kc & 1)))) + 32 * (kc & 1); };
  // W chunks of the stages in flight are held in registers, one set per
  // stage buffer (the stage loop is unrolled by XT_NB so the set is static)
  u32x4 wreg[XT_NB][WPT];
  auto load_w = [&](int s, int set) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < WPT; ++j) wreg[set][j] = *reinterpret_cast<const u32x4*>(wrow[j] + s * XT_K);
  };
  auto store_w = [&](int set) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < WPT; ++j) {
      const int id = tid + 512 * j;
      const int nl = id / CPR, kc = id % CPR;
      const int blk = XT_BLK + (nl >> 5) * KS + (kc >> 1);
      smem[set][blk * 64 + wslot(nl & 31, kc)] = bf16x8_to_f16x8(wreg[set][j]);
    }
  };

  const int nw = n0 + wn * 64;  // this wave's first part column
  const bool active = nw < N;

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // vector-memory operations per wave per stage (LDS-direct latent loads and
  // W loads); s_waitcnt vmcnt(n) with n = this times the number of younger
  // stages in flight waits exactly for the oldest stage
  constexpr int PER = APW + WPT;
  static_assert(2 * PER <= 15, "vmcnt field");
#pragma unroll
  for (int u = 0; u < XT_NB - 1; ++u) {
    if (u < nstage) {
      issue_a(u, u);
      load_w(u, u);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  store_w(0);
  __syncthreads();
#pragma unroll
  for (int s0 = 0; s0 < nstage; s0 += XT_NB) {
#pragma unroll
    for (int u = 0; u < XT_NB; ++u) {
    const int s = s0 + u;  // stage s lives in buffer / register set u
    if (s + XT_NB - 1 < nstage) {
      issue_a(s + XT_NB - 1, (u + XT_NB - 1) % XT_NB);
      load_w(s + XT_NB - 1, (u + XT_NB - 1) % XT_NB);
    }
    if (active) {
      const u32x4* blk = &smem[u][lane];
      const u32x4* wblk = &smem[u][0];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u32x4 fa[4], fb[2];
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[i] = blk[((wm * 4 + i) * KS + ks) * 64];
#pragma unroll
        for (int j = 0; j < 2; ++j) fb[j] = wblk[(XT_BLK + (wn * 2 + j) * KS + ks) * 64 + wslot(l32, 2 * ks + g)];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[i][j] = COLS ? mma16(fa[i], fb[j], acc[i][j]) : mma16(fb[j], fa[i], acc[i][j]);
      }
    }
    if (s + 1 < nstage) {
      // stage s+1 has landed (its latent in LDS, its W in registers), the
      // younger stages may still be in flight
      if (s + 3 < nstage)
        __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * PER));
      else if (s + 2 < nstage)
        __builtin_amdgcn_s_waitcnt(0x0F70 | PER);
      else
        __builtin_amdgcn_s_waitcnt(0);
      store_w((u + 1) % XT_NB);
    }
    // workgroup barrier without the fence __syncthreads() carries: that fence
    // would also wait for the LDS-direct loads of the younger stages. The
    // waits above cover stage s+1's loads; this one the LDS stores of its W.
    // The empty asm statements keep the compiler from moving LDS accesses
    // across the barrier.
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    }
  }
  if (!active) return;

  // epilogue, staged through LDS (free after the last stage's barrier) so that
  // every global store writes whole row segments: the wave's 128 x 64 output
  // tile takes exactly its 16 KB share of LDS, unpadded; the 16-byte chunks of
  // a tile row are XOR-swizzled with the row index to spread the banks. The
  // wave's 64 columns belong to one head (D is a multiple of 64).
  const int h = nw / D;
  const int cw = nw - h * D;  // the wave's first column within the head's k or v part
  const int tw = m0 + wm * 128;  // the wave's first token
  uint16_t* stile = reinterpret_cast<uint16_t*>(&smem[0][0]) + wave * (16384 / 2);
  if (!COLS) {
    // C^T tiles: lane holds columns (r/4)*8 + 4g + r%4 of token l32; tile
    // [128 tokens][8 chunks of 8 columns], chunk c of row r stored at
    // c ^ ((r >> 1) & 7): two 128-byte rows share a 256-byte bank window, so
    // the 16 rows 0-15 of a store then cover all 16 chunk positions (with
    // c ^ (r & 7) rows r and r+8 collide: a 4-way conflict)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = i * 32 + l32, chunk = j * 4 + q;
          u32x2 o;
          o[0] = ET::pack2(acc[i][j][4 * q], acc[i][j][4 * q + 1]);
          o[1] = ET::pack2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
          *reinterpret_cast<u32x2*>(stile + row * 64 + ((chunk ^ ((row >> 1) & 7)) * 8) + 4 * g) = o;
        }
    // each lane then writes 8 columns (16 bytes) of one token: 8 tokens x
    // 128 contiguous bytes per store instruction
    const int tl0 = lane >> 3, ch = lane & 7;
    const int tok0 = tw + tl0;
    int b = tok0 / a.T;
    int t = tok0 - b * a.T;
#pragma unroll
    for (int rep = 0; rep < 16; ++rep) {
      const int tl = tl0 + 8 * rep;
      if (tw + tl < M) {
        const size_t rowi = ((size_t)b * a.H + h) * a.Tcap + a.t_off + t;
        uint16_t* dst = (VPART ? a.v + rowi * a.Dv : a.k + rowi * a.k_ld) + cw + ch * 8;
        // nontemporal: the expanded rows are written once (about 3.8% faster)
        __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(stile + tl * 64 + ((ch ^ ((tl >> 1) & 7)) * 8)),
                                    reinterpret_cast<u32x4*>(dst));
      }
      t += 8;
      while (t >= a.T) {
        t -= a.T;
        ++b;
      }
    }
  } else {
    // C tiles: lane holds tokens (r/4)*8 + 4g + r%4 of column l32; tile
    // [64 value columns][16 chunks of 8 tokens], chunk c of row r stored at
    // c ^ (r & 15)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = j * 32 + l32, chunk = i * 4 + q;
          u32x2 o;
          o[0] = ET::pack2(acc[i][j][4 * q], acc[i][j][4 * q + 1]);
          o[1] = ET::pack2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
          *reinterpret_cast<u32x2*>(stile + row * 128 + ((chunk ^ (row & 15)) * 8) + 4 * g) = o;
        }
    // each lane then writes 8 tokens (16 bytes) of one V^T row: 4 rows x
    // 256 contiguous bytes per store instruction, when 8-token groups never
    // straddle a sequence and stay 16-byte aligned (T and t_off multiples of
    // 8); element stores otherwise (kept as compact loops: this path is rare
    // and must not bloat the code)
    const int tc = lane & 15;
    const bool fast = (a.T % 8) == 0 && (a.t_off % 8) == 0;
    const int tok = tw + tc * 8;
    const int b = tok / a.T;
    const int col = a.t_off + (tok - b * a.T);
#pragma unroll 4
    for (int rep = 0; rep < 16; ++rep) {
      const int dl = (lane >> 4) + 4 * rep;
      const int dv = cw + dl;
      const u32x4 x = *reinterpret_cast<const u32x4*>(stile + dl * 128 + ((tc ^ (dl & 15)) * 8));
      if (fast) {
        if (tok < M) {  // M is a multiple of 8 here: the whole group is in range
          uint16_t* row = a.v + (((size_t)b * a.H + h) * a.Dv + dv) * a.v_ld;
          __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(row + col));
          if (col + 7 == a.Tcap - 1) {
#pragma unroll 1
            for (int z = a.Tcap; z < a.v_ld; ++z) row[z] = 0;
          }
        }
      } else {
#pragma unroll 1
        for (int e = 0; e < 8; ++e)
          if (tok + e < M)
            store_vt1<ET>(a, tok + e, h * (a.Dn + a.Dv) + a.Dn + dv,
                          ET::dec((uint16_t)(x[e >> 1] >> (16 * (e & 1)))));
      }
    }
  }
}

// --------------------------------------------------------------- small kernel
namespace {
constexpr int XS_N = 128;      // W rows (output columns) per workgroup
constexpr int XS_M = 128;      // tokens per workgroup
constexpr int XS_K = 32;       // reduction depth per LDS stage
constexpr int XS_LD = XS_K + 8;  // LDS row stride (16-bit elements), 16-byte pad
}  // namespace

template <class ET>
__global__ void __launch_bounds__(256, 2) expand_small_kernel(ExpandArgs a, int M, int N) {
  __shared__ __attribute__((aligned(16))) uint16_t sW[2][XS_N * XS_LD];
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][XS_M * XS_LD];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int n0 = blockIdx.x * XS_N;
  const int m0 = blockIdx.y * XS_M;
  const int R = a.R;
  const int nstage = (R + XS_K - 1) / XS_K;

  // loaders: chunk id = tid + 256*j (j < 2): row = id >> 2, 8 elements at kc*8
  u32x4 rw[2], ra[2];
  auto gload = [&](int s) {
    const int k0 = s * XS_K;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int id = tid + 256 * j;
      const int row = id >> 2, kc = id & 3;
      const int k = k0 + kc * 8;
      const u32x4 z = {0u, 0u, 0u, 0u};
      // R is a multiple of 8, so an 8-wide chunk is either all inside or all outside
      rw[j] = (n0 + row < N && k < R) ? *reinterpret_cast<const u32x4*>(a.W + (size_t)(n0 + row) * R + k) : z;
      ra[j] = (m0 + row < M && k < R) ? *reinterpret_cast<const u32x4*>(a.c + (size_t)(m0 + row) * R + k) : z;
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int id = tid + 256 * j;
      const int row = id >> 2, kc = id & 3;
      *reinterpret_cast<u32x4*>(&sW[buf][row * XS_LD + kc * 8]) = bf16x8_to_f16x8(rw[j]);
      *reinterpret_cast<u32x4*>(&sA[buf][row * XS_LD + kc * 8]) = ra[j];
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
    for (int kk = 0; kk < XS_K / 16; ++kk) {
      u32x4 fw[2], fa[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        fw[i] = *reinterpret_cast<const u32x4*>(&sW[buf][(wn * 64 + i * 32 + lrow) * XS_LD + kk * 16 + lk]);
        fa[i] = *reinterpret_cast<const u32x4*>(&sA[buf][(wm * 64 + i * 32 + lrow) * XS_LD + kk * 16 + lk]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mma16(fw[i], fa[j], acc[i][j]);
    }
    if (s + 1 < nstage) lstore(buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds C^T rows n = base + (r/4)*8 + (lane/32)*4 + r%4 for
  // token column lane%32 of each 32x32 tile
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int tok = m0 + wm * 64 + j * 32 + lrow;
    if (tok >= M) continue;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wn * 64 + i * 32 + q * 8 + (lane >> 5) * 4;
        if (n >= N) continue;
        // a 4-column group never straddles a head or the k/v boundary (Dn and
        // Dv are multiples of 8)
        if (a.v_cols && col_info(a, n).is_v) {
#pragma unroll 1
          for (int e = 0; e < 4; ++e) store_vt1<ET>(a, tok, n + e, acc[i][j][q * 4 + e]);
        } else {
          store_row4<ET>(a, tok, n, acc[i][j][q * 4 + 0], acc[i][j][q * 4 + 1], acc[i][j][q * 4 + 2],
                         acc[i][j][q * 4 + 3]);
        }
      }
    }
  }
}

// -------------------------------------------------------------- skinny kernel
// Few tokens (M <= 32, the decode append): the work is reading W once. One
// wave per 32 output columns computes C^T = W c^T for all (up to 32) tokens;
// every MFMA operand is one 16-byte run of a W or latent row, loaded straight
// from global memory into registers (no LDS), W widened to fp16 on the way.
template <class ET>
__global__ void __launch_bounds__(64) expand_skinny_kernel(ExpandArgs a, int M, int N) {
  const int lane = threadIdx.x;
  const int l32 = lane & 31, g = lane >> 5;
  const int n0 = blockIdx.x * 32;
  const int R = a.R;
  // A operand: W row n0 + l32 (rows past N read row 0: their outputs are not
  // stored); B operand: latent row l32 (tokens past M read as zeros)
  const int wn = n0 + l32 < N ? n0 + l32 : 0;
  const uint16_t* wr = a.W + (size_t)wn * R + 8 * g;
  const bool tok_ok = l32 < M;
  const uint16_t* cr = a.c + (size_t)(tok_ok ? l32 : 0) * R + 8 * g;
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  const u32x4 z = {0u, 0u, 0u, 0u};
  // 8 MFMA steps (128 reduction elements) per round; R is a multiple of 128
  for (int k0 = 0; k0 < R; k0 += 128) {
    u32x4 wf[8], cf[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      wf[ks] = *reinterpret_cast<const u32x4*>(wr + k0 + 16 * ks);
      cf[ks] = tok_ok ? *reinterpret_cast<const u32x4*>(cr + k0 + 16 * ks) : z;
    }
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) acc = mma16(bf16x8_to_f16x8(wf[ks]), cf[ks], acc);
  }
  // lane holds columns n0 + (r/4)*8 + 4g + r%4 of token l32
  if (!tok_ok) return;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int n = n0 + q * 8 + 4 * g;
    if (n >= N) continue;
    // a 4-column group never straddles a head or the k/v boundary (Dn and Dv
    // are multiples of 8)
    if (a.v_cols && col_info(a, n).is_v) {
#pragma unroll 1
      for (int e = 0; e < 4; ++e) store_vt1<ET>(a, l32, n + e, acc[q * 4 + e]);
    } else {
      store_row4<ET>(a, l32, n, acc[q * 4 + 0], acc[q * 4 + 1], acc[q * 4 + 2], acc[q * 4 + 3]);
    }
  }
}

template <class ET>
static hipError_t launch_tile(const ExpandArgs& a, int M, hipStream_t stream) {
  const dim3 gk((a.H * a.Dn + XT_N - 1) / XT_N, (M + XT_M - 1) / XT_M);
  const dim3 gv((a.H * a.Dv + XT_N - 1) / XT_N, (M + XT_M - 1) / XT_M);
  hipLaunchKernelGGL((expand_tile_kernel<ET, false, false>), gk, dim3(512), 0, stream, a, M);
  if (a.v_cols)
    hipLaunchKernelGGL((expand_tile_kernel<ET, true, true>), gv, dim3(512), 0, stream, a, M);
  else
    hipLaunchKernelGGL((expand_tile_kernel<ET, true, false>), gv, dim3(512), 0, stream, a, M);
  return hipGetLastError();
}

hipError_t launch_kv_expand(const ExpandArgs& a, hipStream_t stream) {
  const int M = a.B * a.T;
  const int N = a.H * (a.Dn + a.Dv);
  // the tile kernel needs 64-column groups that are all keys or all values
  // and the latent width it is unrolled for
  if (M >= 512 && (a.Dn % 64) == 0 && (a.Dv % 64) == 0 && a.R == XT_R)
    return a.kv_dtype == F16::code ? launch_tile<F16>(a, M, stream) : launch_tile<BF16>(a, M, stream);
  if (M <= 32 && (a.R % 128) == 0) {
    const dim3 grid((N + 31) / 32);
    if (a.kv_dtype == F16::code)
      hipLaunchKernelGGL(expand_skinny_kernel<F16>, grid, dim3(64), 0, stream, a, M, N);
    else
      hipLaunchKernelGGL(expand_skinny_kernel<BF16>, grid, dim3(64), 0, stream, a, M, N);
    return hipGetLastError();
  }
  const dim3 grid((N + XS_N - 1) / XS_N, (M + XS_M - 1) / XS_M);
  if (a.kv_dtype == F16::code)
    hipLaunchKernelGGL(expand_small_kernel<F16>, grid, dim3(256), 0, stream, a, M, N);
  else
    hipLaunchKernelGGL(expand_small_kernel<BF16>, grid, dim3(256), 0, stream, a, M, N);
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
