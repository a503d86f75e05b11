// Decode against a compressed-latent cache by the absorbed form (equation
// page "Read the equation" and its "Original context": the eager path
// expands the latent into per-head keys and values with kv_b_proj, and the
// absorbed alternative folds the key half of kv_b_proj (W_uk) into the query
// and applies the value half (W_uv) after attention; GLM-5 "Normalized
// key-value latent", section "KV cache": per token the cache keeps the
// normalised latent and the rotated shared rotary key).
//
// Per sequence b and head h, with c_s the cached latent and k_s the rotated
// rotary key of row s:
//   q_lat[h]  = W_uk[h]^T q_nope[h]                       (absorb_q_kernel)
//   s_s       = scale * (q_lat[h] . c_s + rot(q_pe[h]) . k_s)
//   o_lat[h]  = sum_s softmax(s)_s c_s                    (latent_attn_kernel)
//   out[h]    = W_uv[h] o_lat[h]                         (combine_unabsorb_kernel)
// which equals attention over the expanded keys [W_uk c_s | k_s] and values
// W_uv c_s. Every head reads the same 576-wide cache rows, so one workgroup
// serves 64 heads from one copy of each key tile in LDS.
//
// Kernels (gfx950, 64-wide wavefronts):
//  - absorb_prepare_kernel: one-time copy of W_uk transposed per head
//    ([H, R, Dn], Dn contiguous), so that the absorb product reads its MFMA
//    operands as 8 consecutive elements (weights are prepared once, not per
//    step).
//  - latent_append_kernel: the new token's RMSNorm (fp32, fp16 out) and
//    rotary-key rotation, written into cache row q_pos[b].
//  - absorb_q_kernel: q_lat on bf16 MFMA (exact bf16 products, fp32 sums)
//    and the query's rotation; both pre-multiplied by scale*log2(e) and
//    stored as one fp16 row of 576, so scores leave the MFMA in log2 units.
//  - latent_attn_kernel: split-K flash decoding over 64-key tiles, described
//    at the kernel.
//  - combine_unabsorb_kernel: merges the split partials with the
//    log-sum-exp rule into the fp16 latent aggregate o_lat (in LDS) and
//    multiplies it by W_uv on fp16 MFMA, in one launch.
#include "common.hpp"
#include "launch.hpp"

namespace mla {

namespace {
constexpr float kLog2e = 1.4426950408889634f;
constexpr int LR = 512;       // latent width
constexpr int LDR = 64;       // rotary width
constexpr int LW = LR + LDR;  // cache row, elements
constexpr int LT = 64;        // keys per tile
constexpr int NQC = LW / 16;  // 16-deep k-steps of the score product (32 latent + 4 rotary)
constexpr float kRefSlack = 8.0f;  // log2 units a score may exceed the reference by
// LDS map of the attention kernel (bytes)
constexpr int KV_BYTES = LT * LW * 2;               // one tile: latent rows then rotary rows
constexpr int ROPE_OFF = LT * LR * 2;               // rotary rows inside a tile
constexpr int P_OFF = 2 * KV_BYTES;                 // P [64 heads][64 keys] fp16
constexpr int MX_OFF = P_OFF + 64 * LT * 2;         // [2][64] fp32 exchange
constexpr int SMEM_BYTES = MX_OFF + 2 * 64 * 4;

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef short v4s __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, voff, 0, 0, 0);
}

// Chunk swizzles of the LDS images (16-byte chunks XOR-permuted per row).
// Latent rows (1 KB): chunk x of key row k sits at x ^ swz_lat(k). The
// 16 keys 16a..16a+15 get 16 distinct values, so 16 lanes reading one chunk
// of 16 keys hit 16 different bank groups; 4 consecutive keys differ in
// bits 1..3, so the transposed reads (4 keys x 32 bytes) are conflict-free.
__device__ __forceinline__ int swz_lat(int k) { return ((k & 7) << 1) | ((k >> 3) & 1); }
// Rotary rows (128 B) and P rows (128 B): two rows share a 256-byte bank
// window, the swizzle separates the 8 pairs of a 16-row group.
__device__ __forceinline__ int swz_128(int k) { return (k >> 1) & 7; }

__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 w) {
  u32x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = pack2h(__uint_as_float(w[e] << 16), __uint_as_float(w[e] & 0xffff0000u));
  return o;
}

__device__ __forceinline__ f32x16 mma_f16(u32x4 a, u32x4 b, f32x16 c) { return F16::mma(a, b, c); }

// Workgroup barrier for LDS exchanges only: waits for this wave's LDS
// operations, not for its global loads (a fence would also drain the
// prefetch of the next key tile that is meant to stay in flight).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ f32x16 mma_bf16(u32x4 a, u32x4 b, f32x16 c) { return BF16::mma(a, b, c); }

typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
// Eight transposing LDS reads (ds_read_b64_tr_b16: in each group of 16 lanes,
// lane i receives element i%4 of the 4-element rows addressed by lanes
// i/4, i/4+4, i/4+8, i/4+12) and the wait for them, in one block: the
// results are complete when the block ends. (Written out because the
// compiler orders the builtin form after every LDS-direct load in flight,
// which would serialise the next tile's prefetch.)
__device__ __forceinline__ void ds_read_tr8(const uint32_t (&addr)[8], u32x2v (&r)[8]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n"
      "ds_read_b64_tr_b16 %1, %9\n"
      "ds_read_b64_tr_b16 %2, %10\n"
      "ds_read_b64_tr_b16 %3, %11\n"
      "ds_read_b64_tr_b16 %4, %12\n"
      "ds_read_b64_tr_b16 %5, %13\n"
      "ds_read_b64_tr_b16 %6, %14\n"
      "ds_read_b64_tr_b16 %7, %15\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
      : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]), "v"(addr[4]), "v"(addr[5]), "v"(addr[6]),
        "v"(addr[7]));
}

// Key (within a 32-key block) of operand row r of the S^T = K Q^T MFMA: the
// permutation that gives a lane 8 consecutive keys in registers 8*(i>>3)..
__device__ __forceinline__ int krow(int r) {
  return 16 * ((r >> 3) >> 1) + 8 * ((r >> 2) & 1) + 4 * ((r >> 3) & 1) + (r & 3);
}
}  // namespace

// ---------------------------------------------------------------------------
// W_uk^T per head: wt[h][r][j] = W[h*(Dn+Dv) + j][r], j < Dn. 32x32 tiles
// through LDS (coalesced on both sides).
__global__ void __launch_bounds__(256) absorb_prepare_kernel(const uint16_t* __restrict__ W, uint16_t* __restrict__ wt,
                                                             int H, int R, int Dn, int Dv) {
  __shared__ uint16_t tile[32][33];
  const int h = blockIdx.z;
  const int r0 = blockIdx.x * 32, j0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  const uint16_t* src = W + (size_t)h * (Dn + Dv) * R;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int j = j0 + ty + 8 * k, r = r0 + tx;
    tile[ty + 8 * k][tx] = (j < Dn && r < R) ? src[(size_t)j * R + r] : (uint16_t)0;
  }
  __syncthreads();
  uint16_t* dst = wt + (size_t)h * R * Dn;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int r = r0 + ty + 8 * k, j = j0 + tx;
    if (r < R && j < Dn) dst[(size_t)r * Dn + j] = tile[tx][ty + 8 * k];
  }
}

hipError_t launch_absorb_prepare(const uint16_t* W, uint16_t* wt, int H, int R, int Dn, int Dv, hipStream_t stream) {
  const dim3 grid((unsigned)((R + 31) / 32), (unsigned)((Dn + 31) / 32), (unsigned)H);
  hipLaunchKernelGGL(absorb_prepare_kernel, grid, dim3(256), 0, stream, W, wt, H, R, Dn, Dv);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// New token -> cache row t = q_pos[b]: [ rmsnorm(latent[b]) | rot(k_pe[b], t) ]
// in fp16. One wavefront per sequence; with VEC the row moves in 16-byte
// pieces (R a multiple of 8, at most 2048, rows 16-byte aligned).
template <bool VEC>
__global__ void __launch_bounds__(256) latent_append_kernel(LatentAppendArgs a) {
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (b >= a.B) return;
  const int t = min(max(a.t_pos[b], 0), a.Lcap - 1);
  const int p = min(max(a.t_pos[b], 0), a.table_len - 1);
  const uint16_t* x = a.latent + (size_t)b * a.R;
  uint16_t* row = a.cache + ((size_t)b * a.Lcap + t) * (a.R + a.Dr);
  if (VEC) {
    constexpr int NC = 4;  // up to 4 pieces of 8 per lane
    u32x4 v[NC];
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      const int c = lane + 64 * k;
      v[k] = u32x4{0u, 0u, 0u, 0u};
      if (8 * c < a.R) v[k] = *reinterpret_cast<const u32x4*>(x + 8 * c);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = __uint_as_float(v[k][e] << 16), hi = __uint_as_float(v[k][e] & 0xffff0000u);
        ss += lo * lo + hi * hi;
      }
    }
    ss = wave_sum(ss);
    const float rs = 1.0f / sqrtf(ss / (float)a.R + a.eps);
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      const int c = lane + 64 * k;
      if (8 * c >= a.R) continue;
      const u32x4 gw = *reinterpret_cast<const u32x4*>(a.gain + 8 * c);
      u32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        o[e] = pack2h(__uint_as_float(v[k][e] << 16) * rs * __uint_as_float(gw[e] << 16),
                      __uint_as_float(v[k][e] & 0xffff0000u) * rs * __uint_as_float(gw[e] & 0xffff0000u));
      *reinterpret_cast<u32x4*>(row + 8 * c) = o;
    }
  } else {
    float ss = 0.f;
    for (int i = lane; i < a.R; i += 64) {
      const float v = bf2f(x[i]);
      ss += v * v;
    }
    ss = wave_sum(ss);
    const float rs = 1.0f / sqrtf(ss / (float)a.R + a.eps);
    for (int i = lane; i < a.R; i += 64) row[i] = f2h(bf2f(x[i]) * rs * bf2f(a.gain[i]));
  }
  const int half = a.Dr >> 1;
  const uint16_t* kp = a.k_pe + (size_t)b * a.Dr;
  for (int i = lane; i < half; i += 64) {
    const float c = a.cos[(size_t)p * half + i], s = a.sin[(size_t)p * half + i];
    const int ia = a.pairing ? 2 * i : i;
    const int ib = a.pairing ? 2 * i + 1 : i + half;
    const float xa = bf2f(kp[ia]), xb = bf2f(kp[ib]);
    row[a.R + ia] = f2h(xa * c - xb * s);
    row[a.R + ib] = f2h(xb * c + xa * s);
  }
}

hipError_t launch_latent_append(const LatentAppendArgs& a, hipStream_t stream) {
  const bool vec = (a.R % 8) == 0 && a.R <= 2048 && ((a.R + a.Dr) % 8) == 0 &&
                   ((((uintptr_t)a.latent) | ((uintptr_t)a.gain) | ((uintptr_t)a.cache)) & 15) == 0;
  const dim3 grid((unsigned)((a.B + 3) / 4));
  if (vec)
    hipLaunchKernelGGL(latent_append_kernel<true>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(latent_append_kernel<false>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// qa[b][h] = qscale * [ W_uk[h]^T q_nope[b,h] | rot(q_pe[b,h], q_pos[b]) ]
// (fp16, 576 wide). Wave (r-block, h, b-block): a 32x32 tile of q_lat over
// 32 sequences by bf16 MFMA with k = Dn; the same waves also rotate the
// rotary query (one pair per lane).
__global__ void __launch_bounds__(64) absorb_q_kernel(AbsorbArgs a) {
  const int rb = blockIdx.x, h = blockIdx.y, b0 = blockIdx.z * 32;
  const int lane = threadIdx.x, l32 = lane & 31, g = lane >> 5;
  const int Dqk = a.Dn + a.Dr;
  // rotary query: lane (sequence b0 + l32, half g) of wave rb rotates pair
  // 2*rb + g (the 16 waves of a head cover its Dr/2 = 32 pairs). Its loads
  // (position, then table entries) go first, so that their latency overlaps
  // the absorb product below; the results are stored after it.
  const int rbq = b0 + l32, ri = 2 * rb + g, half = a.Dr >> 1;
  const bool rot = rbq < a.B && ri < half;
  const int ia = a.pairing ? 2 * ri : ri;
  const int ib = a.pairing ? 2 * ri + 1 : ri + half;
  float rc = 0.f, rs = 0.f, xa = 0.f, xb = 0.f;
  if (rot) {
    const int p = min(max(a.q_pos[rbq], 0), a.table_len - 1);
    rc = a.cos[(size_t)p * half + ri];
    rs = a.sin[(size_t)p * half + ri];
    const uint16_t* qp = a.q + ((size_t)rbq * a.H + h) * Dqk + a.Dn;
    xa = bf2f(qp[ia]);
    xb = bf2f(qp[ib]);
  }
  {
    const int b = b0 + l32;
    const uint16_t* qrow = a.q + ((size_t)min(b, a.B - 1) * a.H + h) * Dqk;
    const uint16_t* wrow = a.w_ukt + ((size_t)h * LR + rb * 32 + l32) * a.Dn;
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
    const int nc = a.Dn / 16;
    for (int c0 = 0; c0 < nc; c0 += 8) {
      // the group's loads are issued before its MFMAs
      u32x4 qa[8], wb[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        qa[c] = u32x4{0u, 0u, 0u, 0u};
        wb[c] = u32x4{0u, 0u, 0u, 0u};
        if (c0 + c < nc) {
          if (b < a.B) qa[c] = *reinterpret_cast<const u32x4*>(qrow + 16 * (c0 + c) + 8 * g);
          wb[c] = *reinterpret_cast<const u32x4*>(wrow + 16 * (c0 + c) + 8 * g);
        }
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) acc = mma_bf16(qa[c], wb[c], acc);
    }
    // C[b][r]: lane holds column r = l32, rows 8*(i>>2) + 4g + (i&3)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int bb = b0 + 8 * (i >> 2) + 4 * g + (i & 3);
      if (bb < a.B) a.qa[((size_t)bb * a.H + h) * LW + rb * 32 + l32] = f2h(acc[i] * a.qscale);
    }
  }
  if (rot) {
    uint16_t* dst = a.qa + ((size_t)rbq * a.H + h) * LW + LR;
    dst[ia] = f2h((xa * rc - xb * rs) * a.qscale);
    dst[ib] = f2h((xb * rc + xa * rs) * a.qscale);
  }
}

hipError_t launch_absorb_q(const AbsorbArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)(LR / 32), (unsigned)a.H, (unsigned)((a.B + 31) / 32));
  hipLaunchKernelGGL(absorb_q_kernel, grid, dim3(64), 0, stream, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Split-K attention of 64 absorbed query heads over the latent cache.
// Workgroup (split sp, head group hg, sequence b), 4 waves; the split covers
// keys [sp*tps*64, ...) of the sequence in 64-key tiles.
//  - Each key tile (64 rows x 1152 bytes) moves global -> LDS with 16-byte
//    loads that write LDS directly: one load instruction per latent row
//    (1 KB), one per 8 rotary rows; double-buffered.
//  - Scores: wave w computes S^T for heads 32*(w&1).. and keys 32*(w>>1)..
//    of the tile (36 MFMAs 32x32x16, K rows from LDS, the 32 heads' absorbed
//    queries held in registers for the whole split).
//  - Softmax: a per-head reference maximum m. The tile maxima of the two
//    key halves meet in LDS; every wave derives the same reference: set on
//    the first tile, raised only when a tile exceeds it by more than 8
//    (log2 units; exact either way, O and the row sum share m), so the
//    rescale of O is rare. P = 2^(s - m) goes to LDS as fp16 [head][key].
//  - Values: the latent rows themselves. Wave w accumulates O^T for latent
//    columns 128w..128w+127 of all 64 heads: O^T += C^T P^T, where the C^T
//    operand (8 consecutive keys of one column per lane) comes from the
//    key-major LDS rows through transposing LDS reads (ds_read_b64_tr_b16),
//    and P^T from the P rows.
//  - Output per (b, sp, head): O / l in fp16 and the log2-domain
//    log-sum-exp m + log2(l); an empty split writes -inf.
__global__ void __launch_bounds__(256, 1) latent_attn_kernel(LatentAttnArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[SMEM_BYTES];
  const int sp = blockIdx.x, hg = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  __builtin_assume(wave >= 0 && wave < 4);
  const int l32 = lane & 31, g = lane >> 5;
  const int L = min(max(a.seq_len[b], 1), a.Lcap);
  const int kbeg = sp * a.tps * LT;
  const int kend = min(L, kbeg + a.tps * LT);
  const size_t prow = ((size_t)b * a.S + sp) * a.H;  // partial rows of (b, sp)
  const int h0 = hg * 64;
  if (kbeg >= kend) {
    // no rows: weight zero in the merge; zero rows keep its loads finite
    if (tid < 64 && h0 + tid < a.H) a.part_lse[prow + h0 + tid] = -INFINITY;
    for (int hd = tid >> 6; hd < 64 && h0 + hd < a.H; hd += 4)
      *reinterpret_cast<u32x4*>(a.part_o + (prow + h0 + hd) * LR + 8 * lane) = u32x4{0u, 0u, 0u, 0u};
    return;
  }
  const int ntiles = (kend - kbeg + LT - 1) / LT;
  const int hb = wave & 1, kb = wave >> 1;

  // Loads: wave w brings latent rows w, w+4, .. (lane i -> chunk i ^ swz)
  // and rotary instructions w, w+4 (8 rows each; lane i -> row i/8, chunk
  // (i%8) ^ swz). Offsets past the sequence read as zeros.
  const __amdgpu_buffer_rsrc_t rc = make_rsrc(a.cache + (size_t)b * a.Lcap * LW, (uint32_t)L * LW * 2u);
  uint32_t lat_off[4], rope_off[2];
#pragma unroll
  for (int j = 0; j < 4; ++j) lat_off[j] = 16u * (uint32_t)(lane ^ swz_lat((wave + 4 * j) & 15));
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int kk = 8 * (wave + 4 * r) + (lane >> 3);
    rope_off[r] = (uint32_t)kk * (LW * 2) + LR * 2 + 16u * (uint32_t)((lane & 7) ^ swz_128(kk));
  }
  // 64 rows of 576 values starting at row0 of the buffer r -> LDS image at buf
  auto issue_rows = [&](__amdgpu_buffer_rsrc_t r, uint32_t row0, int buf) __attribute__((always_inline)) {
    char* base = smem + buf * KV_BYTES;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int kk = wave + 4 * j;
      load_lds16(r, base + kk * (LR * 2), (row0 + kk) * (LW * 2) + lat_off[j & 3]);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) load_lds16(r, base + ROPE_OFF + (wave + 4 * i) * 1024, row0 * (LW * 2) + rope_off[i]);
  };
  auto issue = [&](int t, int buf) __attribute__((always_inline)) { issue_rows(rc, (uint32_t)(kbeg + t * LT), buf); };

  // score operand addresses (k-step c: latent chunk 2c+g, c < 32; rotary
  // chunk 2(c-32)+g): the chunk XOR becomes an XOR of the byte offset
  const int kk_s = kb * 32 + krow(l32);
  int latA, ropeA;
  {
    const int fz = swz_lat(kk_s & 15), fr = swz_128(kk_s);
    latA = kk_s * (LR * 2) + 16 * ((g ^ fz) & 1) + 32 * (fz >> 1);
    ropeA = ROPE_OFF + kk_s * (LDR * 2) + 16 * ((g ^ fr) & 1) + 32 * (fr >> 1);
  }
  // transposed value reads: in each 16-lane group, lane m supplies the row
  // address of key 8g + m/4 (+4 for the second read), columns 4*(m%4)..+3
  // of the group's 16-column half
  const int m16 = lane & 15, G = lane >> 4;
  int vA0, vA1;
  {
    const int y = 2 * (G & 1) + ((m16 & 3) >> 1);  // chunk within the 32-column block, before 4*dd
    const int k0 = 8 * g + (m16 >> 2), k1 = k0 + 4;
    const int f0 = swz_lat(k0), f1 = swz_lat(k1);
    vA0 = k0 * (LR * 2) + 256 * wave + 16 * (y ^ (f0 & 3)) + 64 * (f0 >> 2) + 8 * (m16 & 1);
    vA1 = k1 * (LR * 2) + 256 * wave + 16 * (y ^ (f1 & 3)) + 64 * (f1 >> 2) + 8 * (m16 & 1);
  }
  // P row addresses (B operand of the value product: head = column)
  int pA[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int hd = hh * 32 + l32;
    pA[hh] = P_OFF + hd * (LT * 2) + 16 * ((g ^ swz_128(hd)) & 1) + 32 * (swz_128(hd) >> 1);
  }
  float* mxs = reinterpret_cast<float*>(smem + MX_OFF);
  // LDS byte address of smem (the transposing reads take raw LDS addresses)
  const uint32_t lds_base = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)smem;

  f32x16 acc[4][2];
#pragma unroll
  for (int dd = 0; dd < 4; ++dd)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[dd][hh][i] = 0.f;
  float m_run[2] = {-1e30f, -1e30f};  // running maximum of heads l32 and 32+l32 (log2 units)
  float lpart = 0.f;                 // this lane's share of the row sum of its score head

  // The 64 heads' absorbed queries move to LDS (buffer 1, free until the
  // first prefetch) in the same row layout as a key tile, rows = heads
  // (rows past H read as zeros), together with key tile 0; each lane then
  // reads its score head's 36 fragments (B operand: head = column).
  {
    const int nh = min(64, a.H - h0);
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.qa + ((size_t)b * a.H + h0) * LW, (uint32_t)nh * LW * 2u);
    issue_rows(rq, 0u, 1);
  }
  issue(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  u32x4 qf[NQC];
  {
    const char* qb = smem + KV_BYTES;
    const int hd = hb * 32 + l32;
    const int fz = swz_lat(hd & 15), fr = swz_128(hd);
    const int qA = hd * (LR * 2) + 16 * ((g ^ fz) & 1) + 32 * (fz >> 1);
    const int qR = ROPE_OFF + hd * (LDR * 2) + 16 * ((g ^ fr) & 1) + 32 * (fr >> 1);
#pragma unroll
    for (int c = 0; c < 32; ++c) qf[c] = *reinterpret_cast<const u32x4*>(qb + ((qA ^ (32 * (c & 7))) + 256 * (c >> 3)));
#pragma unroll
    for (int c = 0; c < 4; ++c) qf[32 + c] = *reinterpret_cast<const u32x4*>(qb + (qR ^ (32 * c)));
  }
  lds_barrier();  // buffer 1 is free again for the first prefetch
  for (int t = 0; t < ntiles; ++t) {
    const int cur = t & 1;
    if (t + 1 < ntiles) issue(t + 1, cur ^ 1);
    const char* kv = smem + cur * KV_BYTES;
    // ---- scores of (32 heads, 32 keys)
    f32x16 s;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
    for (int c0 = 0; c0 < 32; c0 += 8) {
      u32x4 kf[8];
#pragma unroll
      for (int c = 0; c < 8; ++c)
        kf[c] = *reinterpret_cast<const u32x4*>(kv + ((latA ^ (32 * c)) + 256 * (c0 >> 3)));
#pragma unroll
      for (int c = 0; c < 8; ++c) s = mma_f16(kf[c], qf[c0 + c], s);
    }
    {
      u32x4 kf[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) kf[c] = *reinterpret_cast<const u32x4*>(kv + (ropeA ^ (32 * c)));
#pragma unroll
      for (int c = 0; c < 4; ++c) s = mma_f16(kf[c], qf[32 + c], s);
    }
    const int kt0 = kbeg + t * LT + kb * 32;
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = kt0 + 16 * (i >> 3) + 8 * g + (i & 7);
      if (key >= kend) s[i] = -INFINITY;
      mx = fmaxf(mx, s[i]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    if (g == 0) mxs[kb * 64 + hb * 32 + l32] = mx;
    lds_barrier();
    // ---- reference maxima of heads l32 and 32+l32 (identical in every
    // wave). A reference moves only on the first tile or when the tile's
    // maximum exceeds it by more than the slack (P then stays below
    // 2^slack, far inside fp16), so the rescale of O is usually skipped.
    float alpha[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const float tm = fmaxf(mxs[hh * 32 + l32], mxs[64 + hh * 32 + l32]);
      const bool raise = t == 0 || tm > m_run[hh] + kRefSlack;
      const float mn = raise ? fmaxf(m_run[hh], tm) : m_run[hh];
      alpha[hh] = raise ? __builtin_amdgcn_exp2f(m_run[hh] - mn) : 1.0f;
      m_run[hh] = mn;
    }
    {
      const float m = hb ? m_run[1] : m_run[0];
      const float al = hb ? alpha[1] : alpha[0];
      const int hd = hb * 32 + l32;
      float ts = 0.f;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        u32x4 pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = __builtin_amdgcn_exp2f(s[8 * hf + 2 * e] - m);
          const float p1 = __builtin_amdgcn_exp2f(s[8 * hf + 2 * e + 1] - m);
          pk[e] = pack2h(p0, p1);
          ts = F16::sum2(pk[e], ts);
        }
        const int x = 4 * kb + 2 * hf + g;  // 8-key chunk of the 64-key P row
        *reinterpret_cast<u32x4*>(smem + P_OFF + hd * (LT * 2) + 16 * (x ^ swz_128(hd))) = pk;
      }
      lpart = lpart * al + ts;
    }
    if (__any(alpha[0] != 1.0f || alpha[1] != 1.0f)) {
#pragma unroll
      for (int dd = 0; dd < 4; ++dd)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[dd][hh][i] *= alpha[hh];
    }
    lds_barrier();
    // ---- O^T[128 columns][64 heads] += C^T P^T over the tile's 4 key steps
    const uint32_t kvl = lds_base + (uint32_t)(cur * KV_BYTES);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 pb[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) pb[hh] = *reinterpret_cast<const u32x4*>(smem + (pA[hh] ^ (32 * ks)));
      uint32_t ad[8];
#pragma unroll
      for (int dd = 0; dd < 4; ++dd) {
        ad[2 * dd] = kvl + (uint32_t)((vA0 ^ (64 * dd)) + ks * 16 * (LR * 2));
        ad[2 * dd + 1] = kvl + (uint32_t)((vA1 ^ (64 * dd)) + ks * 16 * (LR * 2));
      }
      u32x2v rv[8];
      ds_read_tr8(ad, rv);
#pragma unroll
      for (int dd = 0; dd < 4; ++dd) {
        const u32x4 va = {rv[2 * dd][0], rv[2 * dd][1], rv[2 * dd + 1][0], rv[2 * dd + 1][1]};
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) acc[dd][hh] = mma_f16(va, pb[hh], acc[dd][hh]);
      }
    }
    // the next tile's loads have landed; every wave is done with this
    // tile's buffer and with P
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // ---- row sums: the two key-half waves of each head block meet in LDS
  {
    const float lt = lpart + __shfl_xor(lpart, 32, 64);
    if (g == 0) mxs[kb * 64 + hb * 32 + l32] = lt;
  }
  __syncthreads();
  float inv[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const float l = mxs[hh * 32 + l32] + mxs[64 + hh * 32 + l32];
    inv[hh] = 1.0f / l;
    if (wave == 0 && g == 0 && h0 + hh * 32 + l32 < a.H)
      a.part_lse[prow + h0 + hh * 32 + l32] = m_run[hh] + log2f(l);
  }
  // O^T lane layout: column = head hh*32 + l32, rows 8*(i>>2) + 4g + (i&3).
  // The normalised rows are staged in LDS (buffer 0, free after the loop;
  // 16-byte chunks swizzled per row) and leave as whole 1 KB rows.
  char* stg = smem;
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int hd = hh * 32 + l32;
    const int fz = swz_lat(hd & 15);
#pragma unroll
    for (int dd = 0; dd < 4; ++dd)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        u32x2 o;
        o[0] = pack2h(acc[dd][hh][4 * r4 + 0] * inv[hh], acc[dd][hh][4 * r4 + 1] * inv[hh]);
        o[1] = pack2h(acc[dd][hh][4 * r4 + 2] * inv[hh], acc[dd][hh][4 * r4 + 3] * inv[hh]);
        const int col = 128 * wave + 32 * dd + 8 * r4 + 4 * g;  // 4 columns: 8 bytes
        *reinterpret_cast<u32x2*>(stg + hd * (LR * 2) + 16 * ((col >> 3) ^ fz) + 8 * ((col >> 2) & 1)) = o;
      }
  }
  lds_barrier();
  for (int hd = wave; hd < 64 && h0 + hd < a.H; hd += 4) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(stg + hd * (LR * 2) + 16 * (lane ^ swz_lat(hd & 15)));
    *reinterpret_cast<u32x4*>(a.part_o + (prow + h0 + hd) * LR + 8 * lane) = v;
  }
}

hipError_t launch_latent_attn(const LatentAttnArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)a.S, (unsigned)((a.H + 63) / 64), (unsigned)a.B);
  hipLaunchKernelGGL(latent_attn_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// The merge and the value product in one launch: out[b][h] = W_uv[h] o_lat
// with o_lat[b][h] = sum_s w_s o_s[b][h] / sum_s w_s, w_s = 2^(lse_s - max)
// (the split outputs are normalised, so the weights are the splits' shares
// of the row sum; the first split holds row 0 of every sequence, so the
// largest lse is finite), never stored. Workgroup (h, CU_SEQ sequences),
// 4 waves:
//  1. merge: wave w merges sequences w, w+4 of the block, lane i its latent
//     columns 8i..8i+7; the fp16 rows go to LDS (16-byte chunk x of row b at
//     x ^ b, so the MFMA reads of 8 rows spread over 8 chunk slots);
//  2. product: wave w computes output columns 32 db.. for db = w, w+4, ..
//     < Dv/32 on fp16 MFMA, A = the o_lat rows (rows past the block's
//     sequences are zero), B = W_uv's rows (bf16 -> fp16).
// The 4 workgroups of one head share an XCD (grid x = head), so W_uv[h]
// comes from HBM once.
namespace {
constexpr int CU_SEQ = 8;  // sequences per workgroup
}
__global__ void __launch_bounds__(256) combine_unabsorb_kernel(CombineUnabsorbArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t ol[CU_SEQ * LR];
  const int h = blockIdx.x, b0 = blockIdx.y * CU_SEQ;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int ndb = a.Dv / 32;
  // this wave's first W_uv rows go out first: their latency overlaps the merge
  u32x4 wv[LR / 16];
  if (wave < ndb) {
    const uint16_t* wrow = a.W + ((size_t)h * (a.Dn + a.Dv) + a.Dn + wave * 32 + l32) * LR;
#pragma unroll
    for (int c = 0; c < LR / 16; ++c) wv[c] = *reinterpret_cast<const u32x4*>(wrow + 16 * c + 8 * g);
  }
  // merge, 8 splits per round: all of a round's loads are issued before its
  // arithmetic
  constexpr int SB = 8;
  for (int bl = wave; bl < CU_SEQ; bl += 4) {
    const int b = b0 + bl;
    u32x4 r = {0u, 0u, 0u, 0u};
    if (b < a.B) {
      const float* lse = a.part_lse + (size_t)b * a.S * a.H + h;
      const uint16_t* po = a.part_o + ((size_t)b * a.S * a.H + h) * LR + 8 * lane;
      // running maximum over the rounds (the first split holds row 0 of
      // every sequence, so it is finite after the first round)
      float mx = -INFINITY;
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = 0.f;
      float tot = 0.f;
      for (int s0 = 0; s0 < a.S; s0 += SB) {
        u32x4 o[SB];
        float l[SB];
#pragma unroll
        for (int k = 0; k < SB; ++k) {
          const bool in = s0 + k < a.S;
          o[k] = in ? *reinterpret_cast<const u32x4*>(po + (size_t)(s0 + k) * a.H * LR) : u32x4{0u, 0u, 0u, 0u};
          l[k] = in ? lse[(size_t)(s0 + k) * a.H] : -INFINITY;
        }
        float mr = mx;
#pragma unroll
        for (int k = 0; k < SB; ++k) mr = fmaxf(mr, l[k]);
        const float sc = s0 == 0 ? 0.f : exp2f(mx - mr);
        mx = mr;
        tot *= sc;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] *= sc;
#pragma unroll
        for (int k = 0; k < SB; ++k) {
          // an empty split has lse -inf (weight 0) and zero rows
          const float w = exp2f(l[k] - mx);
          tot += w;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[2 * e] += w * F16::lo(o[k][e]);
            v[2 * e + 1] += w * F16::hi(o[k][e]);
          }
        }
      }
      const float it = 1.0f / tot;
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = pack2h(v[2 * e] * it, v[2 * e + 1] * it);
    }
    *reinterpret_cast<u32x4*>(ol + bl * LR + 8 * (lane ^ bl)) = r;
  }
  __syncthreads();
  for (int db = wave; db < ndb; db += 4) {
    if (db != wave) {
      const uint16_t* wrow = a.W + ((size_t)h * (a.Dn + a.Dv) + a.Dn + db * 32 + l32) * LR;
#pragma unroll
      for (int c = 0; c < LR / 16; ++c) wv[c] = *reinterpret_cast<const u32x4*>(wrow + 16 * c + 8 * g);
    }
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
    for (int c = 0; c < LR / 16; ++c) {
      const int x = 2 * c + g;  // 16-byte chunk of the o_lat row
      const u32x4 av =
          l32 < CU_SEQ ? *reinterpret_cast<const u32x4*>(ol + l32 * LR + 8 * (x ^ l32)) : u32x4{0u, 0u, 0u, 0u};
      acc = mma_f16(av, bf16x8_to_f16x8(wv[c]), acc);
    }
    // C[row][col]: lane holds column db*32 + l32, rows 8*(i>>2) + 4g + (i&3)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int bl = 8 * (i >> 2) + 4 * g + (i & 3);
      if (bl < CU_SEQ && b0 + bl < a.B) a.out[((size_t)(b0 + bl) * a.H + h) * a.Dv + db * 32 + l32] = f2bf(acc[i]);
    }
  }
}

hipError_t launch_combine_unabsorb(const CombineUnabsorbArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)a.H, (unsigned)((a.B + CU_SEQ - 1) / CU_SEQ));
  hipLaunchKernelGGL(combine_unabsorb_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Re-expansion of a latent cache (the GLM-5 page's eager form: every cached
// latent is expanded by kv_b_proj on every call). The expansion itself is
// kv_expand's tile kernel; these two copies adapt the cache rows to it and
// to the expanded-cache decode kernel.

// Latent part of each cache row -> contiguous [rows, R] (kv_expand's input).
__global__ void __launch_bounds__(256) latent_gather_kernel(const uint16_t* __restrict__ cache,
                                                            uint16_t* __restrict__ c, long rows, int R, int RW) {
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const int n8 = R / 8;
  if (idx >= rows * n8) return;
  const long r = idx / n8;
  const int e = (int)(idx % n8) * 8;
  *reinterpret_cast<u32x4*>(c + r * R + e) = *reinterpret_cast<const u32x4*>(cache + r * RW + e);
}

// Rotated rotary key of cache row s of sequence b -> columns Dn..Dn+Dr of
// row s of every head's key cache [B, H, Lcap, Dn+Dr] (the shared key
// broadcast to all heads, GLM-5 expand_kv).
__global__ void __launch_bounds__(256) rope_broadcast_kernel(const uint16_t* __restrict__ cache,
                                                             uint16_t* __restrict__ k, int B, int H, int Lcap, int R,
                                                             int Dr, int Dn) {
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const int n8 = Dr / 8;
  if (idx >= (long)B * Lcap * n8) return;
  const long bs = idx / n8;
  const int e = (int)(idx % n8) * 8;
  const int b = (int)(bs / Lcap), s = (int)(bs % Lcap);
  const u32x4 v = *reinterpret_cast<const u32x4*>(cache + bs * (R + Dr) + R + e);
  const int Dqk = Dn + Dr;
  for (int h = 0; h < H; ++h)
    *reinterpret_cast<u32x4*>(k + (((size_t)b * H + h) * Lcap + s) * Dqk + Dn + e) = v;
}

hipError_t launch_latent_reexpand_copies(const uint16_t* cache, uint16_t* c, uint16_t* k, int B, int H, int Lcap,
                                         int R, int Dr, int Dn, hipStream_t stream) {
  const long rows = (long)B * Lcap;
  const long n1 = rows * (R / 8);
  hipLaunchKernelGGL(latent_gather_kernel, dim3((unsigned)((n1 + 255) / 256)), dim3(256), 0, stream, cache, c, rows,
                     R, R + Dr);
  const long n2 = rows * (Dr / 8);
  hipLaunchKernelGGL(rope_broadcast_kernel, dim3((unsigned)((n2 + 255) / 256)), dim3(256), 0, stream, cache, k, B, H,
                     Lcap, R, Dr, Dn);
  return hipGetLastError();
}

}  // namespace mla
