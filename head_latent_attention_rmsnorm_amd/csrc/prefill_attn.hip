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
//  - workgroup = (sequence b, head h, NW*32 query rows), NW waves of 32 rows;
//    with 8 waves the row blocks are dealt so that the two waves sharing a
//    SIMD (w and w+4) get blocks s and 7-s, which evens out the triangular
//    work of the diagonal tiles. When the grid is a single round (at most
//    one 8-wave workgroup per compute unit: short sequences), a workgroup
//    instead takes two 128-row blocks i and nb-1-i (waves 0-3 and 4-7), so
//    every workgroup carries the same causal work;
//  - each wave keeps its 32 rotated query rows in registers as the B operand
//    of S^T = K Q^T, so the score accumulator has one query per lane and the
//    softmax statistics are per-lane values (lane l and l^32 share a query);
//  - values arrive transposed (V^T, keys contiguous per value column), so
//    both products read their A operands as 8 consecutive 16-bit elements;
//  - K and V^T tiles move global -> LDS with 16-byte buffer loads that write
//    LDS directly (no registers, no LDS store instructions): lane i of a load
//    writes bytes 16i..16i+15 of a 1 KB block. A group of SW such blocks
//    holds SW consecutive 16-deep k-steps of the 32 operand rows one MFMA
//    reads (32 keys of K, 32 value columns of V^T): each block carries
//    32/SW whole rows of the group, 32*SW contiguous bytes each, so one load
//    instruction reads 8 full 128-byte lines from memory when SW is 4. The
//    16-byte chunks of a row are stored XOR-permuted by a function of the
//    row, which spreads the 16 lanes of one LDS read cycle over all 64
//    banks: every operand read is one conflict-free 16-byte LDS read, at a
//    per-lane address that only flips bits for the next k-step. The gather
//    into that order happens in the loads' per-lane addresses, which stay
//    fixed over the key loop; the descriptor's range check returns zeros
//    past the end of the sequence. Tiles are double-buffered, one barrier
//    per tile;
//  - the K rows of a 32-key sub-tile are gathered in a permuted order, chosen
//    so that the 8 scores a lane holds for one 16-key step of P V are 8
//    consecutive keys: P goes from the S accumulator to a 16-bit B operand of
//    O^T = V^T P^T with no data movement;
//  - all K fragments of a sub-tile are read from LDS before its MFMAs start
//    (a scheduling fence keeps them in flight together); with a 256-wide
//    head they are read in four batches, which keeps the kernel within 256
//    registers (two waves per SIMD);
//  - each 64-key tile is software-pipelined over its two 32-key sub-tiles:
//    the score MFMAs of sub-tile 1 are issued ahead of the softmax of
//    sub-tile 0, and the PV MFMAs of sub-tile 0 ahead of the softmax of
//    sub-tile 1;
//  - the softmax is cut to the bone: in fp16 mode the query is pre-scaled by scale*log2(e) and the
//    first MFMA of every score chain accumulates onto -m (the running
//    reference maximum), so the scores leave the MFMA as exp2 arguments
//    (for 256-wide values, where registers rather than VALU issue are the
//    limit, -m is subtracted on the VALU instead). The
//    reference only moves when a sub-tile's P would leave a safe range: the
//    per-lane sum of the sub-tile's P (taken anyway, in fp32 adds: a packed
//    fp16 dot product does not co-issue with the MFMAs) bounds every P, and only
//    when it exceeds 2^14 (or on the first sub-tile) is the exact maximum
//    taken and the reference raised to it (exact: O and the row sum share
//    the reference);
//  - only the tiles crossing a wave's diagonal are masked; tiles above it are
//    neither loaded nor multiplied;
//  - the output tile of each wave is staged through LDS (the tile buffers
//    are free after the key loop) and written as whole rows with
//    nontemporal 16-byte stores;
//  - workgroup ids are dealt to the 8 XCDs round-robin; the id -> (b, h,
//    q-tile) map makes XCD x run (b, h) pairs x, x+8, ... one at a time,
//    heaviest query tile first, so a pair's keys and values stay in that
//    XCD's L2.
//
// A second kernel transposes row-major values [B, H, T, Dv] into the V^T
// layout [B, H, Dv, Tv] (Tv = T rounded up to 8, zero-filled) when the caller
// does not already hold them transposed.
#include "common.hpp"
#include "launch.hpp"

namespace mla {

namespace {
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.0f;  // log2 units
constexpr float kSumLimit = 16384.0f;  // per-lane tile sum of P that triggers the exact maximum

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, voff, 0, 0, 0);
}

}  // namespace

template <class ET, int DQK, int DR, int DV, int BN, int NW, int MINW>
__global__ void __launch_bounds__(64 * NW, MINW) prefill_kernel(PrefillArgs a, int nqt, int paired) {
  constexpr int DN = DQK - DR;
  constexpr int QC = DQK / 16;          // 16-deep MFMA steps over the head dim
  constexpr int NSUB = BN / 32;         // 32-key sub-tiles
  constexpr int NPV = BN / 16;          // 16-key PV steps
  constexpr int NO = DV / 32;           // 32-wide value tiles
  constexpr int KBLK = NSUB * QC;       // K operand blocks (1 KB) per tile
  constexpr int NBLK = KBLK + NO * NPV; // K + V^T operand blocks per tile
  constexpr int LPW = (NBLK + NW - 1) / NW;  // LDS-direct loads per wave per tile
  constexpr int BMW = NW * 32;          // query rows per workgroup
  constexpr bool FOLD = ET::code == F16::code;  // scores leave the MFMA in log2 units (query pre-scaled)
  // with FOLD, the score chains accumulate onto -m_ref (no subtraction on the
  // VALU) unless registers are the limit (wide values), where a 16-register
  // broadcast of -m_ref would spill
  constexpr bool NEGM = FOLD && DV < 256;
  // k-steps per operand group (see frag_read0): K groups must not straddle
  // the nope|rope boundary
  constexpr int SWK = (DN % 64 == 0 && DR % 64 == 0) ? 4 : (DN % 32 == 0 && DR % 32 == 0) ? 2 : 1;
  constexpr int SWV = (NPV % 4 == 0) ? 4 : (NPV % 2 == 0) ? 2 : 1;
  static_assert(DN % 16 == 0 && DR % 16 == 0 && DV % 32 == 0 && BN % 32 == 0, "tile shape");

  __shared__ __attribute__((aligned(16))) u32x4 smem[2][NBLK * 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int HB = a.H * a.B;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int hb = xcd + 8 * (slot / nqt);
  const int qt = nqt - 1 - slot % nqt;
  if (hb >= HB) return;  // padding workgroup: the whole block exits
  const int h = hb % a.H;
  const int b = hb / a.H;
  const int T = a.T;                  // query rows
  const int past = a.past;            // cached rows before them: query t sits at position past + t
  const int Tk = past + T;            // key rows
  const size_t kvs = (size_t)a.kv_stride;  // row capacity of the k_nope / rotated-key buffers
  const size_t bh = (size_t)b * a.H + h;
  const uint16_t* qg = a.q + bh * T * DQK;

  const int l32 = lane & 31;
  const int g = lane >> 5;
  // This wave's 32 query rows. Default: work item qt is rows qt*BMW.., and
  // with 8 waves the 32-row blocks are dealt so that the waves sharing a SIMD
  // (w and w+4) get blocks s and 7-s, which evens out the triangular work of
  // the diagonal tiles. Paired mode (8 waves, single-round grids): work item
  // qt holds two 128-row blocks, qt and nb-1-qt; waves 0-3 take the first,
  // waves 4-7 the second, so the two waves sharing a SIMD have complementary
  // causal work and every item the same total. With an odd block count the
  // middle item's second half is empty (no tiles, no stores).
  const int nb128 = (T + 127) / 128;
  bool empty = false;
  int qlo;
  if (NW == 8 && paired) {
    const int blk = wave < 4 ? qt : nb128 - 1 - qt;
    empty = wave >= 4 && blk == qt;
    qlo = empty ? T : blk * 128 + (wave & 3) * 32;
  } else {
    qlo = qt * BMW + ((NW == 8 && wave >= 4) ? 11 - wave : wave) * 32;
  }
  const int tq = qlo + l32;  // this lane's query row
  const float sl2 = a.scale * kLog2e;
  const float qmul = FOLD ? sl2 : 1.0f;  // query pre-scale

  // ---- prologue: rotated (and in fp16 mode pre-scaled) query fragments
  u32x4 qf[QC];
  {
    const bool valid = tq < T;
    int p = 0;
    if (valid) {
      p = a.pos ? a.pos[(size_t)b * T + tq] : past + tq;
      p = min(max(p, 0), a.table_len - 1);
    }
    const uint16_t* qrow = qg + (size_t)(valid ? tq : 0) * DQK;
#pragma unroll
    for (int c = 0; c < QC; ++c) {
      const int d0 = 16 * c + 8 * g;
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (valid) raw = *reinterpret_cast<const u32x4*>(qrow + d0);
      if (d0 >= DN) {
        // rotary part: rotate in fp32, round once to the operand type. The
        // chunk's 8 elements use 8 consecutive pairs (half pairing; the
        // partners are the matching chunk of the other half) or 4 (interleaved:
        // the partner is the other half of each word), so cos and sin arrive
        // as 16-byte loads of the position's table row.
        const int re0 = d0 - DN;  // rotary index of the chunk's first element
        const float* crow = a.cos + (size_t)p * (DR / 2);
        const float* srow = a.sin + (size_t)p * (DR / 2);
        u32x4 outv;
        if (!a.pairing) {
          const bool first = re0 < DR / 2;
          const int pi0 = first ? re0 : re0 - DR / 2;
          u32x4 partner = {0u, 0u, 0u, 0u};
          if (valid) partner = *reinterpret_cast<const u32x4*>(qrow + DN + (first ? re0 + DR / 2 : re0 - DR / 2));
          const f32x4 c0 = *reinterpret_cast<const f32x4*>(crow + pi0);
          const f32x4 c1 = *reinterpret_cast<const f32x4*>(crow + pi0 + 4);
          const f32x4 s0 = *reinterpret_cast<const f32x4*>(srow + pi0);
          const f32x4 s1 = *reinterpret_cast<const f32x4*>(srow + pi0 + 4);
          const float sgn = first ? -1.0f : 1.0f;  // (x cos - x' sin) for the first half, (x cos + x' sin) after
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            const float cs0 = e2 < 2 ? c0[2 * e2] : c1[2 * e2 - 4], cs1 = e2 < 2 ? c0[2 * e2 + 1] : c1[2 * e2 - 3];
            const float sn0 = e2 < 2 ? s0[2 * e2] : s1[2 * e2 - 4], sn1 = e2 < 2 ? s0[2 * e2 + 1] : s1[2 * e2 - 3];
            const float x0 = __uint_as_float(raw[e2] << 16), x1 = __uint_as_float(raw[e2] & 0xffff0000u);
            const float p0 = __uint_as_float(partner[e2] << 16), p1 = __uint_as_float(partner[e2] & 0xffff0000u);
            outv[e2] = ET::pack2((x0 * cs0 + sgn * (p0 * sn0)) * qmul, (x1 * cs1 + sgn * (p1 * sn1)) * qmul);
          }
        } else {
          const f32x4 cs = *reinterpret_cast<const f32x4*>(crow + (re0 >> 1));
          const f32x4 sn = *reinterpret_cast<const f32x4*>(srow + (re0 >> 1));
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            const float x0 = __uint_as_float(raw[e2] << 16), x1 = __uint_as_float(raw[e2] & 0xffff0000u);
            outv[e2] = ET::pack2((x0 * cs[e2] - x1 * sn[e2]) * qmul, (x1 * cs[e2] + x0 * sn[e2]) * qmul);
          }
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


  // keys [0, kend) are visible to some row of the work item
  const int kend = (NW == 8 && paired) ? min(Tk, past + (nb128 - qt) * 128) : min(Tk, past + (qt + 1) * BMW);
  const int nkt = (kend + BN - 1) / BN;

  // Key (within a 32-key sub-tile) of operand row r of the S^T MFMA: the
  // permutation that makes a lane's accumulator registers 8*(i>>3) .. hold
  // consecutive keys
  auto krow = [](int r) { return 16 * ((r >> 3) >> 1) + 8 * ((r >> 2) & 1) + 4 * ((r >> 3) & 1) + (r & 3); };

  // This wave's operand blocks: for each, the buffer descriptor of the whole
  // (b, h) slice it comes from (chosen once here, kept in scalar registers),
  // the lane's byte offset for the tile starting at key 0, and the bytes one
  // key advances it. The tile offset goes into the vector offset, which the
  // descriptor's range check covers: keys past the end of the sequence read
  // as zeros. (Choosing descriptors per tile instead costs tens of scalar
  // instructions per wave, and the 8 waves reach that point together right
  // after the barrier, queueing on the CU's one scalar unit.)
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k_nope + bh * kvs * DN, (uint32_t)Tk * DN * 2u);
  const __amdgpu_buffer_rsrc_t rr = make_rsrc(a.k_rot + (size_t)b * kvs * DR, (uint32_t)Tk * DR * 2u);
  const __amdgpu_buffer_rsrc_t rv =
      make_rsrc(a.v + bh * (size_t)DV * a.v_ld, (uint32_t)DV * (uint32_t)a.v_ld * 2u);
  __amdgpu_buffer_rsrc_t rs[LPW];
  uint32_t voff[LPW], vstep[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int bi = wave + NW * i;
    rs[i] = rv;
    voff[i] = 0;
    vstep[i] = 0;
    if (bi < KBLK) {
      const int j = bi / QC, cq = bi % QC;
      int r, x;
      frag_slot<SWK>(cq % SWK, lane, r, x);
      const int row = 32 * j + krow(r);
      const int col = (cq / SWK) * (16 * SWK) + 8 * x;
      if (col < DN) {
        rs[i] = rk;
        voff[i] = (uint32_t)(row * DN + col) * 2u;
        vstep[i] = DN * 2u;
      } else {
        rs[i] = rr;
        voff[i] = (uint32_t)(row * DR + (col - DN)) * 2u;
        vstep[i] = DR * 2u;
      }
    } else if (bi < NBLK) {
      const int vb = bi - KBLK, d = vb / NPV, s = vb % NPV;
      int r, x;
      frag_slot<SWV>(s % SWV, lane, r, x);
      voff[i] = (uint32_t)((32 * d + r) * a.v_ld + (s / SWV) * (16 * SWV) + 8 * x) * 2u;
      vstep[i] = 2u;
    }
  }

  // queue the LDS-direct loads of key tile kt into buffer buf
  auto issue = [&](int kt, int buf) __attribute__((always_inline)) {
    const uint32_t key0 = (uint32_t)(kt * BN);
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int bi = wave + NW * i;
      if (bi < NBLK) load_lds16(rs[i], &smem[buf][bi * 64], voff[i] + key0 * vstep[i]);
    }
  };

  // ---- running state. Scores are kept relative to a per-query reference
  // m_ref (log2 units); before the first tile the reference is 0 and unset.
  f32x16 oacc[NO];
#pragma unroll
  for (int d = 0; d < NO; ++d)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[d][i] = 0.f;
  float m_ref = 0.f;
  bool ref_set = false;
  float lsum = 0.f;  // this lane's share of the row sum
  f32x16 negm;       // -m_ref broadcast: the initial score accumulator
#pragma unroll
  for (int i = 0; i < 16; ++i) negm[i] = 0.f;

  // One key tile, software-pipelined over its 32-key sub-tiles: the score
  // MFMAs of sub-tile j+1 are issued before the softmax of sub-tile j, and
  // the PV MFMAs of sub-tile j before the softmax of j+1, so the exp and
  // conversion work of one sub-tile can run under the MFMAs of another.
  // this lane's operand read offsets for each k-step position in a group
  int rdk[SWK], rdv[SWV];
#pragma unroll
  for (int c = 0; c < SWK; ++c) rdk[c] = frag_read0<SWK>(l32, g) ^ (32 * c);
#pragma unroll
  for (int c = 0; c < SWV; ++c) rdv[c] = frag_read0<SWV>(l32, g) ^ (32 * c);

  auto tile = [&](int cur, int key0) __attribute__((always_inline)) {
    const char* sb = reinterpret_cast<const char*>(&smem[cur][0]);
    auto kfrag = [&](int j, int c) __attribute__((always_inline)) {
      return *reinterpret_cast<const u32x4*>(sb + (j * QC + (c / SWK) * SWK) * 1024 + rdk[c % SWK]);
    };
    auto vfrag = [&](int d, int s) __attribute__((always_inline)) {
      return *reinterpret_cast<const u32x4*>(sb + (KBLK + d * NPV + (s / SWV) * SWV) * 1024 + rdv[s % SWV]);
    };
    const bool diag = key0 + BN - 1 > past + qlo;  // the tile crosses the wave's diagonal
    f32x16 sacc[NSUB];
    u32x4 pf[NPV];
    auto s_chain = [&](int j) __attribute__((always_inline)) {
      constexpr int KB = QC > 12 ? QC / 4 : QC;  // fragments read ahead of their products
#pragma unroll
      for (int c0 = 0; c0 < QC; c0 += KB) {
        u32x4 kf[KB];
#pragma unroll
        for (int c = 0; c < KB; ++c) kf[c] = kfrag(j, c0 + c);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < KB; ++c) {
          if (c0 + c == 0) {
            if (NEGM) {
              sacc[j] = ET::mma(kf[c], qf[0], negm);
            } else {
              f32x16 z;
#pragma unroll
              for (int i = 0; i < 16; ++i) z[i] = 0.f;
              sacc[j] = ET::mma(kf[c], qf[0], z);
            }
          } else {
            sacc[j] = ET::mma(kf[c], qf[c0 + c], sacc[j]);
          }
        }
      }
    };
    // scale (bf16 mode) and mask the scores of sub-tile j
    auto finish = [&](int j) __attribute__((always_inline)) {
      if (!FOLD) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[j][i] = fmaf(sacc[j][i], sl2, -m_ref);
      } else if (!NEGM) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[j][i] -= m_ref;
      }
      if (diag) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = key0 + j * 32 + 16 * (i >> 3) + 8 * g + (i & 7);
          if (key > past + tq) sacc[j][i] = -INFINITY;
        }
      }
    };
    // P = 2^(s - m_ref) of sub-tile j as 16-bit B operands (8 consecutive
    // keys per lane) and this lane's sum of them
    auto make_p = [&](int j) __attribute__((always_inline)) {
      float t = 0.f;
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        u32x4 pk;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const float p0 = __builtin_amdgcn_exp2f(sacc[j][8 * mm + 2 * e2]);
          const float p1 = __builtin_amdgcn_exp2f(sacc[j][8 * mm + 2 * e2 + 1]);
          pk[e2] = ET::pack2(p0, p1);
          t += p0 + p1;  // fp32 adds: a packed dot product would not overlap the MFMAs
        }
        pf[2 * j + mm] = pk;
      }
      return t;
    };
    s_chain(0);
    finish(0);
#pragma unroll
    for (int j = 0; j < NSUB; ++j) {
      if (j + 1 < NSUB) s_chain(j + 1);
      float ts = make_p(j);
      if (__any(!ref_set || ts > kSumLimit)) {
        // the exact maximum of the sub-tile (relative to the reference);
        // move the reference to it on the first sub-tile and wherever a
        // score exceeds it by more than the slack (the first sub-tile holds
        // key 0, visible to every row, so the maximum is finite where the
        // reference is still unset)
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[j][i]);
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const bool raise = !ref_set || mx > kRescaleSlack;
        const float shift = raise ? mx : 0.f;
        const float alpha = (raise && ref_set) ? __builtin_amdgcn_exp2f(-mx) : 1.f;
        m_ref += shift;
        ref_set = true;
        lsum *= alpha;
#pragma unroll
        for (int d = 0; d < NO; ++d)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[d][i] *= alpha;
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[j][i] -= shift;
        if (NEGM) {
          // the next sub-tile's scores were accumulated onto the old -m_ref
          if (j + 1 < NSUB) {
#pragma unroll
            for (int i = 0; i < 16; ++i) sacc[j + 1][i] -= shift;
          }
#pragma unroll
          for (int i = 0; i < 16; ++i) negm[i] = -m_ref;
        }
        ts = make_p(j);
      }
      lsum += ts;
      if (j + 1 < NSUB) finish(j + 1);
      // O^T += V^T P^T over the sub-tile's two 16-key steps
#pragma unroll
      for (int d = 0; d < NO; ++d)
#pragma unroll
        for (int mm = 0; mm < 2; ++mm)
          oacc[d] = ET::mma(vfrag(d, 2 * j + mm), pf[2 * j + mm], oacc[d]);
    }
  };

  issue(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nkt) issue(kt + 1, cur ^ 1);
    const int key0 = kt * BN;
    if (!empty && key0 <= past + qlo + 31) tile(cur, key0);  // some key of the tile is visible to this wave
    // the next tile's loads have landed in LDS and every wave is done with
    // this tile's buffer
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // ---- epilogue: normalise; each wave stages its 32 x DV output tile in
  // its own part of the (now free) tile buffers, 16-byte chunks XOR-swizzled
  // by row, so that every global store writes whole rows
  const float ltot = lsum + __shfl_xor(lsum, 32, 64);
  {
    constexpr int CPR = DV / 8;  // 16-byte chunks per output row
    static_assert((CPR & (CPR - 1)) == 0 && CPR <= 64, "row swizzle needs a power-of-two chunk count");
    static_assert(NW * 32 * DV * 2 <= (int)sizeof(smem), "the output tiles fit in the tile buffers");
    char* stile = reinterpret_cast<char*>(&smem[0][0]) + wave * (32 * DV * 2);
    const float inv = 1.0f / ltot;
#pragma unroll
    for (int d = 0; d < NO; ++d) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int c = d * 4 + r4;  // chunk of value columns d*32 + r4*8 ..
        u32x2 o;
        o[0] = pack2bf(oacc[d][r4 * 4 + 0] * inv, oacc[d][r4 * 4 + 1] * inv);
        o[1] = pack2bf(oacc[d][r4 * 4 + 2] * inv, oacc[d][r4 * 4 + 3] * inv);
        *reinterpret_cast<u32x2*>(stile + l32 * (DV * 2) + ((c ^ (l32 & (CPR - 1))) * 16) + 8 * g) = o;
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's staging writes
    asm volatile("" ::: "memory");
    constexpr int RPI = 64 / CPR;  // rows per store instruction
    const int ch = lane % CPR;
#pragma unroll
    for (int rep = 0; rep < 32 / RPI; ++rep) {
      const int row = lane / CPR + RPI * rep;
      const u32x4 v = *reinterpret_cast<const u32x4*>(stile + row * (DV * 2) + ((ch ^ (row & (CPR - 1))) * 16));
      // whole rows, written once: nontemporal (8-byte scattered nontemporal
      // stores, without the staging, were 70% slower at short sequences)
      if (qlo + row < T) __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(a.out + (bh * T + qlo + row) * DV + ch * 8));
    }
    // natural-log log-sum-exp of the row's scaled scores
    if (tq < T && a.lse && g == 0) a.lse[bh * T + tq] = (m_ref + log2f(ltot)) * kLn2;
  }
}

// Row-major values [B, H, T, Dv] -> V^T [B, H, Dv, v_ld] (columns T..v_ld-1
// zero). One workgroup per (64 tokens, 64 value columns), looping over b*H+h.
__global__ void __launch_bounds__(256) transpose_v_kernel(const uint16_t* __restrict__ v, uint16_t* __restrict__ vt,
                                                           int BH, int T, int Dv, int v_ld, int ny) {
  constexpr int LD = 64 + 8;  // LDS row stride (16-bit elements)
  __shared__ __attribute__((aligned(16))) uint16_t tile[64 * LD];
  const int tid = threadIdx.x;
  const int t0 = (blockIdx.x / ny) * 64, d0 = (blockIdx.x % ny) * 64;
  for (int bh = blockIdx.y; bh < BH; bh += gridDim.y) {
    const uint16_t* src = v + (size_t)bh * T * Dv;
    uint16_t* dst = vt + (size_t)bh * Dv * v_ld;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int id = tid + 256 * i;
      const int tok = id >> 3, dc = id & 7;
      const int t = t0 + tok, d = d0 + dc * 8;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (t < T && d < Dv) x = *reinterpret_cast<const u32x4*>(src + (size_t)t * Dv + d);
      *reinterpret_cast<u32x4*>(&tile[tok * LD + dc * 8]) = x;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int id = tid + 256 * i;
      const int dr = id >> 3, tc = id & 7;
      const int d = d0 + dr, t = t0 + tc * 8;
      if (d < Dv && t < v_ld) {
        u32x4 y;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2)
          y[e2] = (uint32_t)tile[(tc * 8 + 2 * e2) * LD + dr] | ((uint32_t)tile[(tc * 8 + 2 * e2 + 1) * LD + dr] << 16);
        *reinterpret_cast<u32x4*>(dst + (size_t)d * v_ld + t) = y;
      }
    }
    __syncthreads();
  }
}

hipError_t launch_transpose_v(const uint16_t* v, uint16_t* vt, int BH, int T, int Dv, int v_ld, hipStream_t stream) {
  const int ny = (Dv + 63) / 64;
  const dim3 grid((unsigned)(((v_ld + 63) / 64) * ny), (unsigned)(BH < 65535 ? BH : 65535));
  hipLaunchKernelGGL(transpose_v_kernel, grid, dim3(256), 0, stream, v, vt, BH, T, Dv, v_ld, ny);
  return hipGetLastError();
}

bool prefill_supported(int Dqk, int Dr, int Dv) {
  return (Dqk == 48 && Dr == 16 && Dv == 32) || (Dqk == 192 && Dr == 64 && Dv == 128) ||
         (Dqk == 256 && Dr == 64 && Dv == 256);
}

template <class ET, int DQK, int DR, int DV, int BN, int NW, int MINW>
static hipError_t launch_one(const PrefillArgs& a, hipStream_t stream) {
  constexpr int BMW = NW * 32;
  const int hb8 = (a.H * a.B + 7) / 8 * 8;  // (b, h) pairs padded to the XCD count
  // one round of 8-wave workgroups at most (every workgroup starts at once):
  // pair 128-row blocks so that all work items carry the same causal work;
  // with more rounds the heaviest-first order balances better and loads less
  const int paired = (NW == 8 && (int64_t)a.B * a.H * ((a.T + BMW - 1) / BMW) <= 256) ? 1 : 0;
  const int nqt = paired ? ((a.T + 127) / 128 + 1) / 2 : (a.T + BMW - 1) / BMW;
  hipLaunchKernelGGL((prefill_kernel<ET, DQK, DR, DV, BN, NW, MINW>), dim3((unsigned)nqt * hb8), dim3(64 * NW), 0,
                     stream, a, nqt, paired);
  return hipGetLastError();
}

template <class ET>
static hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t stream) {
  const int Dqk = a.Dn + a.Dr;
  if (Dqk == 192 && a.Dv == 128) return launch_one<ET, 192, 64, 128, 64, 8, 2>(a, stream);
  // wide values: 4-wave workgroups at two waves per SIMD (two workgroups per
  // compute unit); the 256-register budget holds with key fragments read in
  // batches of four and no -m_ref broadcast
  if (Dqk == 256 && a.Dv == 256) return launch_one<ET, 256, 64, 256, 32, 4, 2>(a, stream);
  if (Dqk == 48 && a.Dv == 32) return launch_one<ET, 48, 16, 32, 64, 4, 2>(a, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  // 192/128 heads over more than one round of 256-row work items: two row
  // blocks per wave (prefill_dual.hip); a single round (short sequences)
  // keeps the 8-wave kernel, whose paired 128-row blocks even out the causal
  // work of the one round
  if (prefill_dual_supported(a.Dn + a.Dr, a.Dr, a.Dv) && (int64_t)a.B * a.H * ((a.T + 255) / 256) > 256)
    return launch_prefill_dual(a, stream);
  return launch_prefill_t<F16>(a, stream);
}

}  // namespace mla
