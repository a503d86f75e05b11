// Causal prefill attention with the rotary step and the nope|rope
// concatenation in the prologue (Kimi-K2 "Query content heads", section "Join
// query parts": rotate the rotary parts, join each head's query and key from
// the non-rotary and rotated parts with the rotary key shared by all heads,
// scale, mask causally, softmax in fp32, mix the values; GLM-5 "Normalized
// key-value latent", expand_kv: the shared rotary key is broadcast to every
// head without being copied).
//
// Design (gfx950, 64-wide wavefronts, 16-bit MFMA 32x32x16 with fp32
// accumulation; operands in the key/value element type, bf16 or fp16):
//  - workgroup = (sequence b, head h, 128 query rows), 4 waves x 32 rows;
//    heaviest (last) query tiles are dispatched first;
//  - each wave keeps its 32 rotated query rows in registers as the B operand
//    of S^T = K Q^T, so the score accumulator has one query per lane and the
//    softmax statistics are per-lane values (lane l and l^32 share a query);
//  - K tiles (k_nope | pre-rotated shared k_pe) and V^T tiles are staged in
//    LDS, single-buffered, with the next tile's global loads in flight while
//    the current one is multiplied;
//  - inside each 32-key sub-tile the K rows are fed to the MFMA in a permuted
//    order, chosen so that the 8 scores a lane holds for one 16-key step of
//    P V are 8 consecutive keys: P goes from the S accumulator to a 16-bit B
//    operand of O^T = V^T P^T with no data movement, and V^T is read with
//    16-byte LDS loads;
//  - fp32 online softmax in the log2 domain (scale * log2 e folded into one
//    multiply), with the running maximum raised only when a score exceeds it
//    by more than 2^8 (the rescale of the O accumulator is skipped otherwise;
//    exact, as O and the row sum share the same reference);
//  - only the diagonal key tiles are masked; tiles above the diagonal are
//    never loaded.
#include "common.hpp"
#include "launch.hpp"

namespace mla {

namespace {
constexpr int BM = 128;          // query rows per workgroup
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.0f;  // log2 units
}  // namespace

template <class ET, int DQK, int DR, int DV, int BN, int MINW>
__global__ void __launch_bounds__(256, MINW) prefill_kernel(PrefillArgs a, int nqt) {
  constexpr int DN = DQK - DR;
  constexpr int QC = DQK / 16;       // 16-deep MFMA steps over the head dim
  constexpr int LDQ = DQK + 8;       // K tile row stride (16-bit elements)
  constexpr int LDV = BN + 8;        // V^T tile row stride (16-bit elements)
  constexpr int KCHUNKS = BN * DQK / 8;        // 16-byte chunks per K tile
  constexpr int KPER = (KCHUNKS + 255) / 256;  // per thread
  constexpr int VUNITS = (BN / 4) * (DV / 8);  // (4 keys x 8 dv) units per V tile
  constexpr int VPER = (VUNITS + 255) / 256;
  constexpr int NSUB = BN / 32;      // 32-key sub-tiles
  constexpr int NPV = BN / 16;       // 16-key PV steps
  constexpr int NO = DV / 32;        // 32-wide dv tiles
  static_assert(DQK % 16 == 0 && DV % 32 == 0 && BN % 32 == 0 && DR % 16 == 0, "tile shape");

  __shared__ __attribute__((aligned(16))) uint16_t sK[BN * LDQ];
  __shared__ __attribute__((aligned(16))) uint16_t sV[DV * LDV];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int HB = a.H * a.B;
  const int qt = nqt - 1 - (int)(blockIdx.x / HB);
  const int hb = blockIdx.x % HB;
  const int h = hb % a.H;
  const int b = hb / a.H;
  const int T = a.T;

  const size_t bh = (size_t)b * a.H + h;
  const uint16_t* qg = a.q + bh * T * DQK;
  const uint16_t* kg = a.k_nope + bh * T * DN;
  const uint16_t* rg = a.k_rot + (size_t)b * T * DR;
  const uint16_t* vg = a.v + bh * T * DV;

  const int l32 = lane & 31;
  const int g = lane >> 5;
  const int qlo = qt * BM + wave * 32;  // first query row of this wave
  const int tq = qlo + l32;             // this lane's query row

  // ---- prologue: rotated query fragments in the operand type (B operand:
  // lane = query, 8 dims); the query arrives in bf16
  u32x4 qf[QC];
  {
    const bool valid = tq < T;
    int p = 0;
    if (valid) {
      p = a.pos ? a.pos[(size_t)b * T + tq] : tq;
      p = min(max(p, 0), a.table_len - 1);
    }
    const uint16_t* qrow = qg + (size_t)(valid ? tq : 0) * DQK;
#pragma unroll
    for (int c = 0; c < QC; ++c) {
      const int d0 = 16 * c + 8 * g;
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (valid) raw = *reinterpret_cast<const u32x4*>(qrow + d0);
      if (d0 >= DN) {
        // rotary part: rotate in fp32, round once to the operand type
        const int re0 = d0 - DN;  // rotary index of the chunk's first element
        u32x4 partner = raw;
        if (!a.pairing) {
          const int pre0 = re0 < DR / 2 ? re0 + DR / 2 : re0 - DR / 2;
          if (valid) partner = *reinterpret_cast<const u32x4*>(qrow + DN + pre0);
        }
        u32x4 outv;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          float y[2];
#pragma unroll
          for (int hl = 0; hl < 2; ++hl) {
            const int e = 2 * e2 + hl;
            const int re = re0 + e;
            const float x = hl ? __uint_as_float(raw[e2] & 0xffff0000u) : __uint_as_float(raw[e2] << 16);
            float xp;
            int pi;
            bool first;
            if (a.pairing) {  // interleaved: partner is the other half of the 32-bit word
              xp = hl ? __uint_as_float(raw[e2] << 16) : __uint_as_float(raw[e2] & 0xffff0000u);
              pi = re >> 1;
              first = (re & 1) == 0;
            } else {
              xp = hl ? __uint_as_float(partner[e2] & 0xffff0000u) : __uint_as_float(partner[e2] << 16);
              pi = re < DR / 2 ? re : re - DR / 2;
              first = re < DR / 2;
            }
            const float cs = a.cos[(size_t)p * (DR / 2) + pi];
            const float sn = a.sin[(size_t)p * (DR / 2) + pi];
            y[hl] = first ? (x * cs - xp * sn) : (x * cs + xp * sn);
          }
          outv[e2] = ET::pack2(y[0], y[1]);
        }
        raw = outv;
      } else if (ET::code != BF16::code) {
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2)
          raw[e2] = ET::pack2(__uint_as_float(raw[e2] << 16), __uint_as_float(raw[e2] & 0xffff0000u));
      }
      qf[c] = raw;
    }
  }

  const int kend = min(T, (qt + 1) * BM);  // keys [0, kend) are visible to some row
  const int nkt = (kend + BN - 1) / BN;

  // ---- tile staging: global -> registers -> LDS
  u32x4 kreg[KPER];
  u32x4 vreg[VPER][4];
  auto gload = [&](int kt) {
    const int key0 = kt * BN;
#pragma unroll
    for (int i = 0; i < KPER; ++i) {
      const int id = tid + 256 * i;
      u32x4 z = {0u, 0u, 0u, 0u};
      kreg[i] = z;
      if (id < KCHUNKS) {
        const int row = id / (DQK / 8);
        const int cc = id - row * (DQK / 8);
        const int s = key0 + row;
        if (s < T) {
          kreg[i] = (cc < DN / 8) ? *reinterpret_cast<const u32x4*>(kg + (size_t)s * DN + cc * 8)
                                  : *reinterpret_cast<const u32x4*>(rg + (size_t)s * DR + (cc - DN / 8) * 8);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < VPER; ++i) {
      const int u = tid + 256 * i;
      const int dc = u % (DV / 8);
      const int kq = u / (DV / 8);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x4 z = {0u, 0u, 0u, 0u};
        vreg[i][j] = z;
        const int s = key0 + kq * 4 + j;
        if (u < VUNITS && s < T) vreg[i][j] = *reinterpret_cast<const u32x4*>(vg + (size_t)s * DV + dc * 8);
      }
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int i = 0; i < KPER; ++i) {
      const int id = tid + 256 * i;
      if (id < KCHUNKS) {
        const int row = id / (DQK / 8);
        const int cc = id - row * (DQK / 8);
        *reinterpret_cast<u32x4*>(&sK[row * LDQ + cc * 8]) = kreg[i];
      }
    }
#pragma unroll
    for (int i = 0; i < VPER; ++i) {
      const int u = tid + 256 * i;
      if (u < VUNITS) {
        const int dc = u % (DV / 8);
        const int kq = u / (DV / 8);
        // transpose 4 keys x 8 dv into 8 rows of 4 consecutive keys
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
#pragma unroll
          for (int hl = 0; hl < 2; ++hl) {
            const int dv = dc * 8 + 2 * e2 + hl;
            uint32_t w0, w1;
            if (hl == 0) {
              w0 = (vreg[i][0][e2] & 0xffffu) | (vreg[i][1][e2] << 16);
              w1 = (vreg[i][2][e2] & 0xffffu) | (vreg[i][3][e2] << 16);
            } else {
              w0 = (vreg[i][0][e2] >> 16) | (vreg[i][1][e2] & 0xffff0000u);
              w1 = (vreg[i][2][e2] >> 16) | (vreg[i][3][e2] & 0xffff0000u);
            }
            u32x2 w = {w0, w1};
            *reinterpret_cast<u32x2*>(&sV[dv * LDV + kq * 4]) = w;
          }
        }
      }
    }
  };

  // ---- running state
  f32x16 oacc[NO];
#pragma unroll
  for (int d = 0; d < NO; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[d][r] = 0.f;
  float m_ref = -INFINITY;  // reference maximum (log2 units)
  float lsum = 0.f;         // this lane's share of the row sum
  const float sl2 = a.scale * kLog2e;

  // K row fed by this lane for the S^T MFMA: the permutation that makes the
  // lane's registers 8*(r>>3) .. hold consecutive keys
  const int krow = 16 * ((l32 >> 3) >> 1) + 8 * ((l32 >> 2) & 1) + 4 * ((l32 >> 3) & 1) + (l32 & 3);

  gload(0);
  for (int kt = 0; kt < nkt; ++kt) {
    lstore();
    __syncthreads();
    if (kt + 1 < nkt) gload(kt + 1);

    const int key0 = kt * BN;
    if (key0 <= qlo + 31) {  // some key of the tile is visible to this wave
      f32x16 sacc[NSUB];
#pragma unroll
      for (int j = 0; j < NSUB; ++j) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[j][r] = 0.f;
        const uint16_t* kr = &sK[(j * 32 + krow) * LDQ + 8 * g];
#pragma unroll
        for (int c = 0; c < QC; ++c) {
          const u32x4 ka = *reinterpret_cast<const u32x4*>(kr + 16 * c);
          sacc[j] = ET::mma(ka, qf[c], sacc[j]);
        }
      }
      // scores -> log2 domain, causal mask on diagonal tiles
      const bool diag = key0 + BN - 1 > qlo;
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < NSUB; ++j) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float s = sacc[j][r] * sl2;
          if (diag) {
            const int key = key0 + j * 32 + 16 * (r >> 3) + 8 * g + (r & 7);
            if (key > tq) s = -INFINITY;
          }
          sacc[j][r] = s;
          mx = fmaxf(mx, s);
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_ref, mx);
      const bool raise = m_new > m_ref + kRescaleSlack;
      if (__any(raise)) {
        float alpha = 1.f;
        if (raise) {
          alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
          m_ref = m_new;
        }
        lsum *= alpha;
#pragma unroll
        for (int d = 0; d < NO; ++d)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[d][r] *= alpha;
      }
      // P = 2^(s - m_ref) as B operands, 8 consecutive keys per lane
      u32x4 pf[NPV];
#pragma unroll
      for (int m = 0; m < NPV; ++m) {
        u32x4 pk;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const float p0 = __builtin_amdgcn_exp2f(sacc[m >> 1][8 * (m & 1) + 2 * e2] - m_ref);
          const float p1 = __builtin_amdgcn_exp2f(sacc[m >> 1][8 * (m & 1) + 2 * e2 + 1] - m_ref);
          lsum += p0 + p1;
          pk[e2] = ET::pack2(p0, p1);
        }
        pf[m] = pk;
      }
      // O^T += V^T P^T
#pragma unroll
      for (int d = 0; d < NO; ++d) {
        const uint16_t* vr = &sV[(d * 32 + l32) * LDV + 8 * g];
#pragma unroll
        for (int m = 0; m < NPV; ++m) {
          const u32x4 va = *reinterpret_cast<const u32x4*>(vr + 16 * m);
          oacc[d] = ET::mma(va, pf[m], oacc[d]);
        }
      }
    }
    __syncthreads();
  }

  // ---- epilogue: normalise, store 4 consecutive dv per 8-byte write
  const float ltot = lsum + __shfl_xor(lsum, 32, 64);
  if (tq < T) {
    const float inv = 1.0f / ltot;
    uint16_t* orow = a.out + (bh * T + tq) * DV;
#pragma unroll
    for (int d = 0; d < NO; ++d) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int dv = d * 32 + r4 * 8 + g * 4;
        u32x2 o;
        o[0] = pack2bf(oacc[d][r4 * 4 + 0] * inv, oacc[d][r4 * 4 + 1] * inv);
        o[1] = pack2bf(oacc[d][r4 * 4 + 2] * inv, oacc[d][r4 * 4 + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + dv) = o;
      }
    }
    if (a.lse && g == 0) a.lse[bh * T + tq] = (m_ref + __log2f(ltot)) * kLn2;
  }
}

bool prefill_supported(int Dqk, int Dr, int Dv) {
  return (Dqk == 48 && Dr == 16 && Dv == 32) || (Dqk == 192 && Dr == 64 && Dv == 128) ||
         (Dqk == 256 && Dr == 64 && Dv == 256);
}

template <class ET>
static hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t stream) {
  const int nqt = (a.T + BM - 1) / BM;
  const dim3 grid((unsigned)nqt * a.H * a.B), block(256);
  const int Dqk = a.Dn + a.Dr;
  if (Dqk == 192 && a.Dv == 128) {
    hipLaunchKernelGGL((prefill_kernel<ET, 192, 64, 128, 64, 2>), grid, block, 0, stream, a, nqt);
  } else if (Dqk == 256 && a.Dv == 256) {
    hipLaunchKernelGGL((prefill_kernel<ET, 256, 64, 256, 32, 1>), grid, block, 0, stream, a, nqt);
  } else if (Dqk == 48 && a.Dv == 32) {
    hipLaunchKernelGGL((prefill_kernel<ET, 48, 16, 32, 64, 2>), grid, block, 0, stream, a, nqt);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  return a.kv_dtype == F16::code ? launch_prefill_t<F16>(a, stream) : launch_prefill_t<BF16>(a, stream);
}

}  // namespace mla
