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
//  - workgroup = (sequence b, head h, NW*32 query rows), NW waves of 32 rows,
//    two waves per SIMD;
//  - each wave keeps its 32 rotated query rows in registers as the B operand
//    of S^T = K Q^T, so the score accumulator has one query per lane and the
//    softmax statistics are per-lane values (lane l and l^32 share a query);
//  - K tiles (k_nope | pre-rotated shared k_pe) and V^T tiles are double-
//    buffered in LDS with one barrier per tile; they are fetched with raw
//    buffer loads whose range check returns zeros past the end of the
//    sequence, so no load is predicated;
//  - inside each 32-key sub-tile the K rows are fed to the MFMA in a permuted
//    order, chosen so that the 8 scores a lane holds for one 16-key step of
//    P V are 8 consecutive keys: P goes from the S accumulator to a 16-bit B
//    operand of O^T = V^T P^T with no data movement, and V^T is read with
//    16-byte LDS loads;
//  - all K fragments of a sub-tile are read from LDS before its MFMAs start
//    (a scheduling fence keeps them in flight together);
//  - MFMA and VALU work hardly overlap on this chip, so the softmax is cut to
//    the bone: in fp16 mode the query is pre-scaled by scale*log2(e) and the
//    first MFMA of every score chain accumulates onto -m (the running
//    reference maximum), so the scores leave the MFMA already as exp2
//    arguments; the reference is raised only when a score exceeds it by more
//    than 2^8 (exact: O and the row sum share the reference);
//  - row sums come from v_dot2 over the packed 16-bit P (the values the PV
//    MFMA consumes), and the transposed V store builds each word with one
//    byte permute;
//  - only the tiles crossing a wave's diagonal are masked; tiles above it are
//    never loaded;
//  - workgroup ids are dealt to the 8 XCDs round-robin; the id -> (b, h,
//    q-tile) map makes XCD x run (b, h) pairs x, x+8, ... one at a time,
//    heaviest query tile first, so a pair's keys and values stay in that
//    XCD's L2.
#include "common.hpp"
#include "launch.hpp"

namespace mla {

namespace {
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.0f;  // log2 units
}  // namespace

template <class ET, int DQK, int DR, int DV, int BN, int NW, int MINW>
__global__ void __launch_bounds__(64 * NW, MINW) prefill_kernel(PrefillArgs a, int nqt) {
  constexpr int NT = 64 * NW;           // threads per workgroup
  constexpr int DN = DQK - DR;
  constexpr int QC = DQK / 16;          // 16-deep MFMA steps over the head dim
  constexpr int LDQ = DQK + 8;          // K tile row stride (16-bit elements)
  constexpr int LDV = BN + 8;           // V^T tile row stride
  constexpr int BMW = NW * 32;          // query rows per workgroup
  constexpr int NCH_N = BN * (DN / 8);  // 16-byte non-rotary chunks per K tile
  constexpr int NCH_R = BN * (DR / 8);  // 16-byte rotary chunks per K tile
  constexpr int PER_N = (NCH_N + NT - 1) / NT;
  constexpr int PER_R = (NCH_R + NT - 1) / NT;
  constexpr int VUNITS = (BN / 4) * (DV / 8);  // (4 keys x 8 values) units
  constexpr int VPER = (VUNITS + NT - 1) / NT;
  constexpr int NSUB = BN / 32;         // 32-key sub-tiles
  constexpr int NPV = BN / 16;          // 16-key PV steps
  constexpr int NO = DV / 32;           // 32-wide value tiles
  constexpr bool FOLD = ET::code == F16::code;  // scores leave the MFMA as exp2 arguments
  static_assert(DN % 8 == 0 && DR % 16 == 0 && DV % 32 == 0 && BN % 32 == 0, "tile shape");

  __shared__ __attribute__((aligned(16))) uint16_t sK[2][BN * LDQ];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][DV * LDV];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int HB = a.H * a.B;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int hb = xcd + 8 * (slot / nqt);
  const int qt = nqt - 1 - slot % nqt;
  if (hb >= HB) return;  // padding workgroup: the whole block exits
  const int h = hb % a.H;
  const int b = hb / a.H;
  const int T = a.T;
  const size_t bh = (size_t)b * a.H + h;

  const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k_nope + bh * T * DN, (uint32_t)T * DN * 2);
  const __amdgpu_buffer_rsrc_t rr = make_rsrc(a.k_rot + (size_t)b * T * DR, (uint32_t)T * DR * 2);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v + bh * T * DV, (uint32_t)T * DV * 2);
  const uint16_t* qg = a.q + bh * T * DQK;

  const int l32 = lane & 31;
  const int g = lane >> 5;
  const int qlo = qt * BMW + wave * 32;  // first query row of this wave
  const int tq = qlo + l32;              // this lane's query row
  const float sl2 = a.scale * kLog2e;
  const float qmul = FOLD ? sl2 : 1.0f;  // query pre-scale

  // ---- prologue: rotated (and in fp16 mode pre-scaled) query fragments
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
            const int re = re0 + 2 * e2 + hl;
            const float x = hl ? __uint_as_float(raw[e2] & 0xffff0000u) : __uint_as_float(raw[e2] << 16);
            float xp;
            int pi;
            bool first;
            if (a.pairing) {  // interleaved: the partner is the other half of the word
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
            y[hl] = (first ? (x * cs - xp * sn) : (x * cs + xp * sn)) * qmul;
          }
          outv[e2] = ET::pack2(y[0], y[1]);
        }
        raw = outv;
      } else if (FOLD || ET::code != BF16::code) {
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2)
          raw[e2] = ET::pack2(__uint_as_float(raw[e2] << 16) * qmul, __uint_as_float(raw[e2] & 0xffff0000u) * qmul);
      }
      qf[c] = raw;
    }
  }

  const int kend = min(T, (qt + 1) * BMW);  // keys [0, kend) are visible to some row
  const int nkt = (kend + BN - 1) / BN;

  // ---- tile staging: global -> registers -> LDS
  u32x4 kn_reg[PER_N], kr_reg[PER_R];
  u32x4 v_reg[VPER][4];
  auto gload = [&](int kt) {
    const int key0 = kt * BN;
#pragma unroll
    for (int i = 0; i < PER_N; ++i) {
      const int id = tid + NT * i;
      const int row = id / (DN / 8), cc = id % (DN / 8);
      if (NCH_N % NT == 0 || id < NCH_N) kn_reg[i] = buf_load16(rk, (uint32_t)((key0 + row) * DN + cc * 8) * 2);
    }
#pragma unroll
    for (int i = 0; i < PER_R; ++i) {
      const int id = tid + NT * i;
      const int row = id / (DR / 8), cc = id % (DR / 8);
      if (NCH_R % NT == 0 || id < NCH_R) kr_reg[i] = buf_load16(rr, (uint32_t)((key0 + row) * DR + cc * 8) * 2);
    }
    // V units: 4 consecutive keys x 8 value columns; the key quad varies
    // fastest across lanes so the transposed 8-byte LDS stores spread over
    // the banks
#pragma unroll
    for (int i = 0; i < VPER; ++i) {
      const int u = tid + NT * i;
      const int kq = u % (BN / 4), dc = u / (BN / 4);
      if (VUNITS % NT == 0 || u < VUNITS) {
#pragma unroll
        for (int j = 0; j < 4; ++j) v_reg[i][j] = buf_load16(rv, (uint32_t)((key0 + kq * 4 + j) * DV + dc * 8) * 2);
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PER_N; ++i) {
      const int id = tid + NT * i;
      const int row = id / (DN / 8), cc = id % (DN / 8);
      if (NCH_N % NT == 0 || id < NCH_N) *reinterpret_cast<u32x4*>(&sK[buf][row * LDQ + cc * 8]) = kn_reg[i];
    }
#pragma unroll
    for (int i = 0; i < PER_R; ++i) {
      const int id = tid + NT * i;
      const int row = id / (DR / 8), cc = id % (DR / 8);
      if (NCH_R % NT == 0 || id < NCH_R) *reinterpret_cast<u32x4*>(&sK[buf][row * LDQ + DN + cc * 8]) = kr_reg[i];
    }
#pragma unroll
    for (int i = 0; i < VPER; ++i) {
      const int u = tid + NT * i;
      const int kq = u % (BN / 4), dc = u / (BN / 4);
      if (VUNITS % NT == 0 || u < VUNITS) {
        // transpose 4 keys x 8 values into 8 rows of 4 keys: one byte
        // permute per 32-bit word (selector 0x05040100 joins the low halves
        // of two words, 0x07060302 the high halves)
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const u32x2 lo = {__builtin_amdgcn_perm(v_reg[i][1][e2], v_reg[i][0][e2], 0x05040100u),
                            __builtin_amdgcn_perm(v_reg[i][3][e2], v_reg[i][2][e2], 0x05040100u)};
          const u32x2 hi = {__builtin_amdgcn_perm(v_reg[i][1][e2], v_reg[i][0][e2], 0x07060302u),
                            __builtin_amdgcn_perm(v_reg[i][3][e2], v_reg[i][2][e2], 0x07060302u)};
          *reinterpret_cast<u32x2*>(&sV[buf][(dc * 8 + 2 * e2) * LDV + kq * 4]) = lo;
          *reinterpret_cast<u32x2*>(&sV[buf][(dc * 8 + 2 * e2 + 1) * LDV + kq * 4]) = hi;
        }
      }
    }
  };

  // ---- running state. Scores are kept relative to a per-query reference
  // m_ref (log2 units); before the first tile the reference is 0 and unset.
  f32x16 oacc[NO];
#pragma unroll
  for (int d = 0; d < NO; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[d][r] = 0.f;
  float m_ref = 0.f;
  bool ref_set = false;
  float lsum = 0.f;  // this lane's share of the row sum
  f32x16 negm;       // -m_ref broadcast: the initial score accumulator
#pragma unroll
  for (int r = 0; r < 16; ++r) negm[r] = 0.f;

  // K row fed by this lane for the S^T MFMA: the permutation that makes the
  // lane's registers 8*(r>>3) .. hold consecutive keys
  const int krow = 16 * ((l32 >> 3) >> 1) + 8 * ((l32 >> 2) & 1) + 4 * ((l32 >> 3) & 1) + (l32 & 3);

  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nkt) gload(kt + 1);
    const int key0 = kt * BN;
    if (key0 <= qlo + 31) {  // some key of the tile is visible to this wave
      // S^T = K Q^T, relative to the reference
      f32x16 sacc[NSUB];
#pragma unroll
      for (int j = 0; j < NSUB; ++j) {
        const uint16_t* kr = &sK[cur][(j * 32 + krow) * LDQ + 8 * g];
        u32x4 kf[QC];
#pragma unroll
        for (int c = 0; c < QC; ++c) kf[c] = *reinterpret_cast<const u32x4*>(kr + 16 * c);
        __builtin_amdgcn_sched_barrier(0);
        sacc[j] = ET::mma(kf[0], qf[0], negm);
#pragma unroll
        for (int c = 1; c < QC; ++c) sacc[j] = ET::mma(kf[c], qf[c], sacc[j]);
      }
      if (!FOLD) {
#pragma unroll
        for (int j = 0; j < NSUB; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[j][r] = fmaf(sacc[j][r], sl2, -m_ref);
      }
      // causal mask on the tiles that cross the diagonal
      if (key0 + BN - 1 > qlo) {
#pragma unroll
        for (int j = 0; j < NSUB; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + j * 32 + 16 * (r >> 3) + 8 * g + (r & 7);
            if (key > tq) sacc[j][r] = -INFINITY;
          }
      }
      // tile maximum relative to the reference; move the reference to it on
      // the first tile and whenever a score exceeds it by more than the slack
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < NSUB; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[j][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const bool raise = !ref_set || mx > kRescaleSlack;
      if (__any(raise)) {
        // the first tile always holds key 0, visible to every row, so mx is
        // finite wherever the reference is still unset
        const float shift = raise ? mx : 0.f;
        const float alpha = (raise && ref_set) ? __builtin_amdgcn_exp2f(-mx) : 1.f;
        m_ref += shift;
        ref_set = true;
        lsum *= alpha;
#pragma unroll
        for (int d = 0; d < NO; ++d)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[d][r] *= alpha;
#pragma unroll
        for (int j = 0; j < NSUB; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[j][r] -= shift;
        if (FOLD) {
#pragma unroll
          for (int r = 0; r < 16; ++r) negm[r] = -m_ref;
        }
      }
      // P = 2^(s - m_ref) as 16-bit B operands, 8 consecutive keys per lane
      u32x4 pf[NPV];
#pragma unroll
      for (int m = 0; m < NPV; ++m) {
        u32x4 pk;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const float p0 = __builtin_amdgcn_exp2f(sacc[m >> 1][8 * (m & 1) + 2 * e2]);
          const float p1 = __builtin_amdgcn_exp2f(sacc[m >> 1][8 * (m & 1) + 2 * e2 + 1]);
          pk[e2] = ET::pack2(p0, p1);
          lsum = ET::sum2(pk[e2], lsum);
        }
        pf[m] = pk;
      }
      // O^T += V^T P^T
#pragma unroll
      for (int d = 0; d < NO; ++d) {
        const uint16_t* vr = &sV[cur][(d * 32 + l32) * LDV + 8 * g];
#pragma unroll
        for (int m = 0; m < NPV; ++m)
          oacc[d] = ET::mma(*reinterpret_cast<const u32x4*>(vr + 16 * m), pf[m], oacc[d]);
      }
    }
    if (kt + 1 < nkt) lstore(cur ^ 1);
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
    // natural-log log-sum-exp of the row's scaled scores
    if (a.lse && g == 0) a.lse[bh * T + tq] = (m_ref + log2f(ltot)) * kLn2;
  }
}

bool prefill_supported(int Dqk, int Dr, int Dv) {
  return (Dqk == 48 && Dr == 16 && Dv == 32) || (Dqk == 192 && Dr == 64 && Dv == 128) ||
         (Dqk == 256 && Dr == 64 && Dv == 256);
}

template <class ET, int DQK, int DR, int DV, int BN, int NW, int MINW>
static hipError_t launch_one(const PrefillArgs& a, hipStream_t stream) {
  constexpr int BMW = NW * 32;
  const int nqt = (a.T + BMW - 1) / BMW;
  const int hb8 = (a.H * a.B + 7) / 8 * 8;  // (b, h) pairs padded to the XCD count
  hipLaunchKernelGGL((prefill_kernel<ET, DQK, DR, DV, BN, NW, MINW>), dim3((unsigned)nqt * hb8), dim3(64 * NW), 0,
                     stream, a, nqt);
  return hipGetLastError();
}

template <class ET>
static hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t stream) {
  const int Dqk = a.Dn + a.Dr;
  if (Dqk == 192 && a.Dv == 128) return launch_one<ET, 192, 64, 128, 32, 8, 2>(a, stream);
  if (Dqk == 256 && a.Dv == 256) return launch_one<ET, 256, 64, 256, 32, 4, 1>(a, stream);
  if (Dqk == 48 && a.Dv == 32) return launch_one<ET, 48, 16, 32, 64, 4, 2>(a, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  return a.kv_dtype == F16::code ? launch_prefill_t<F16>(a, stream) : launch_prefill_t<BF16>(a, stream);
}

}  // namespace mla
