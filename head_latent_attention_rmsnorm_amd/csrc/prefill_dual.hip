// Causal prefill attention for the 192/128 heads of the Kimi-K2 shape (Kimi-K2
// "Query content heads", section "Join query parts": rotate the rotary parts,
// join each head's query and key from the non-rotary and rotated parts with
// the rotary key shared by all heads, scale, mask causally, softmax in fp32,
// mix the values), laid out so that every operand fragment read from LDS
// feeds two MFMAs.
//
// Design (gfx950, one wave per SIMD, 16-bit MFMA 32x32x16 with fp32
// accumulation, operands in the key/value element type):
//  - work item = (sequence b, head h, 256 query rows), one workgroup of 4
//    waves per CU working through a static list of items (persistent; see
//    the item loop for the order); each wave owns
//    64 consecutive query rows as two 32-row blocks, and keeps both blocks'
//    rotated (and, in fp16 mode, pre-scaled) queries in registers as the B
//    operands of S^T = K Q^T. A key fragment (32 keys x 16 dims, 1 KB) is read
//    from LDS once and multiplied into both blocks, and so is a value fragment
//    (32 value columns x 16 keys) for O^T += V^T P^T. That halves the LDS
//    bytes per MFMA against one block per wave, at the price of ~400
//    registers: one wave per SIMD, so latency is hidden inside the wave;
//  - the K / V^T tile image in LDS, the LDS-direct loads that fill it, the key
//    row permutation that lets P feed the PV product straight from the score
//    accumulators and the exp2-domain online softmax with a lazily moved
//    reference are those of the 8-wave kernel in prefill_attn.hip;
//  - a 64-key tile is one flat sequence of 40 steps, each one fragment read
//    from LDS and the two MFMAs that consume it: 12 steps of scores for keys
//    0-31, 12 for keys 32-63, 8 of P V for keys 0-31, 8 for keys 32-63. The
//    read of step i + PF is issued in step i, so each fragment has PF steps
//    (2*PF MFMAs) to arrive. The softmax of keys 0-31 (exp2, conversion,
//    row sums) runs one score at a time between the score MFMAs of keys
//    32-63, and the softmax of keys 32-63 between the P V MFMAs of keys 0-31:
//    a wave's VALU work runs while its own MFMAs execute;
//  - a wave that issues an MFMA while its previous one still occupies the
//    unit stalls until it leaves, so a step's VALU work is split over the
//    gaps after each of its two MFMAs, and no gap gets more than the 32
//    cycles an MFMA takes where that can be helped: one score per half-step,
//    the score accumulators copied out to vector registers 8 at a time over
//    four half-steps (one 16-register copy at the first use would idle the
//    MFMA pipe for ~100 cycles), each P packed where it is computed rather
//    than after the rare-path branch. Scheduling fences around every MFMA
//    keep that order.
#include "common.hpp"
#include "launch.hpp"

namespace mla {

namespace {
constexpr float kLog2eD = 1.4426950408889634f;
constexpr float kLn2D = 0.6931471805599453f;
constexpr float kSlackD = 8.0f;     // log2 units a score may exceed the reference without moving it
constexpr float kSumLimD = 16384.0f;  // per-lane tile sum of P that triggers the exact maximum

typedef __attribute__((address_space(3))) void* lds_ptr_d;

__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_d)lds, 16, voff, 0, 0, 0);
}

__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }

// Register-file placement (no instruction): the value is held in the MFMA
// accumulation registers (AGPRs) or in the ordinary vector registers at this
// point. With ~400 live registers per lane the allocator otherwise shuttles
// the output accumulators and query fragments between the two files on every
// tile.
template <class V>
__device__ __forceinline__ void in_agpr(V& v) {
  asm volatile("" : "+a"(v));
}
template <class V>
__device__ __forceinline__ void in_vgpr(V& v) {
  asm volatile("" : "+v"(v));
}

template <int N>
struct IntC {
  static constexpr int value = N;
};

// f(IntC<I>{}) for I = B .. E-1, unrolled at compile time
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(IntC<B>{});
    static_for<B + 1, E>(f);
  }
}

// Step orders of a 64-key tile (step ids: 0-11 key steps of keys 0-31,
// 12-19 value steps of keys 32-63 of the previous tile, 20-31 key steps of
// keys 32-63, 32-39 value steps of keys 0-31):
//   PIPE: the pipelined tile, ids in order; FIRST: the first pipelined tile
//   (no previous tile); DRAIN: the value steps of the last pipelined tile;
//   DIAG: a whole tile outside the pipeline.
enum StepOrder { kPipe = 0, kFirst = 1, kDrain = 2, kDiag = 3 };
constexpr int order_len(int m) { return m == kFirst ? 32 : m == kDrain ? 8 : 40; }
constexpr int order_id(int m, int k) {
  return m == kPipe ? k : m == kFirst ? (k < 12 ? k : k + 8) : m == kDrain ? 12 + k
                                                                          : (k < 12 ? k : k < 32 ? k + 8 : k - 20);
}

struct TrueT {
  static constexpr bool value = true;
};
struct FalseT {
  static constexpr bool value = false;
};

}  // namespace

template <class ET, int DQK, int DR, int DV, int PF, int NBUF>
__global__ void __launch_bounds__(256, 1) prefill_dual_kernel(PrefillArgs a, int nqt) {
  constexpr int NW = 4;                  // waves
  constexpr int BN = 64;                 // keys per tile
  constexpr int DN = DQK - DR;
  constexpr int QC = DQK / 16;           // 16-deep k-steps over the head dim
  constexpr int NO = DV / 32;            // 32-wide value tiles
  constexpr int KBLK = 2 * QC;           // K operand blocks (1 KB) per tile
  constexpr int NBLK = KBLK + NO * 4;    // K + V^T operand blocks per tile
  constexpr int LPW = NBLK / NW;         // LDS-direct loads per wave per tile
  constexpr int BM = NW * 64;            // query rows per workgroup
  constexpr int NSTEP = KBLK + 2 * 2 * NO;  // fragment reads per tile
  constexpr bool FOLD = ET::code == F16::code;
  constexpr int SWK = (DN % 64 == 0 && DR % 64 == 0) ? 4 : 2;
  constexpr int SWV = 4;
  static_assert(NBLK % NW == 0, "tile blocks split evenly over the waves");
  static_assert(DN % 32 == 0 && DR % 32 == 0 && DV % 32 == 0, "tile shape");
  static_assert(NW * 64 * DV * 2 <= NBLK * 1024 * 2, "the output tiles fit in the tile buffers");

  static_assert(NBUF == 2 || NBUF == 3, "double or triple buffered tiles");
  // NBUF tile buffers and one more: at the start of an item the waves' query
  // rows are staged from buffer 1 on (2 QC KB per wave)
  static_assert(NBLK * 1024 + NW * 2 * QC * 1024 <= (NBUF + 1) * NBLK * 1024, "query staging fits");
  __shared__ __attribute__((aligned(16))) u32x4 smem[NBUF + 1][NBLK * 64];

  const int HB = a.H * a.B;
  // Persistent: one workgroup per CU works through the (b, h, 256-row) items
  // of its XCD (workgroup i runs on XCD i % 8, which takes the (b, h) pairs
  // hb = XCD + 8k). The items of one XCD are listed pair by pair, each pair's
  // row blocks from the last (the longest under the causal mask) to the first;
  // round n hands out the next NC items, to the XCD's workgroups in turn,
  // in reverse order on odd rounds. A workgroup thus alternates long and
  // short items (equal totals when the row blocks per pair match NC), the
  // XCD works on few pairs at a time (their K / V stay in its L2), and no
  // launch gap separates one item from the next.
  const int xcd = blockIdx.x & 7, wg = blockIdx.x >> 3;
  const int NC = gridDim.x >> 3;  // workgroups per XCD
  const int nitems = (HB + 7) / 8 * nqt;
  for (int round = 0; round * NC < nitems; ++round) {
    const int it = round * NC + ((round & 1) ? NC - 1 - wg : wg);
    if (it >= nitems) continue;
    const int hb = xcd + 8 * (it / nqt);
    const int qt = nqt - 1 - it % nqt;
    if (hb >= HB) continue;  // padding pair
    // the lane's index, re-read per item: values derived from it are then
    // recomputed here rather than held in registers across the item loop
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = hb % a.H;
    const int b = hb / a.H;
    const int T = a.T;
    const int past = a.past;
    const int Tk = past + T;
    const size_t kvs = (size_t)a.kv_stride;
    const size_t bh = (size_t)b * a.H + h;
    const uint16_t* qg = a.q + bh * T * DQK;

    const int l32 = lane & 31;
    const int g = lane >> 5;
    const int qlo = qt * BM + wave * 64;  // this wave's first query row; block r holds rows qlo + 32r ..
    const float sl2 = a.scale * kLog2eD;
    const float qmul = FOLD ? sl2 : 1.0f;

    // keys [0, kend) are visible to some row of the workgroup
    const int kend = min(Tk, past + (qt + 1) * BM);
    const int nkt = (kend + BN - 1) / BN;

    // key (within a 32-key sub-tile) of operand row r of the S^T MFMA: a lane's
    // accumulator registers 8m..8m+7 then hold 8 consecutive keys, the B
    // operand layout of the P V product
    auto krow = [](int r) { return 16 * ((r >> 3) >> 1) + 8 * ((r >> 2) & 1) + 4 * ((r >> 3) & 1) + (r & 3); };

    // This wave's share of the tile loads: descriptor of the (b, h) slice, the
    // lane's byte offset for the tile at key 0 and its advance per key. Keys
    // past the end of the sequence read as zeros (range check).
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k_nope + bh * kvs * DN, (uint32_t)Tk * DN * 2u);
    const __amdgpu_buffer_rsrc_t rr = make_rsrc(a.k_rot + (size_t)b * kvs * DR, (uint32_t)Tk * DR * 2u);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v + bh * (size_t)DV * a.v_ld, (uint32_t)DV * (uint32_t)a.v_ld * 2u);
    __amdgpu_buffer_rsrc_t rs[LPW];
    uint32_t voff[LPW], vstep[LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int bi = wave + NW * i;
      if (bi < KBLK) {
        const int j = bi / QC, cq = bi % QC;
        int r, x;
        frag_slot<SWK>(cq % SWK, lane, r, x);
        const int row = 32 * j + krow(r);
        const int gcol = (cq / SWK) * (16 * SWK);  // first column of the group: nope and rope groups never mix
        const int col = gcol + 8 * x;
        if (gcol < DN) {
          rs[i] = rk;
          voff[i] = (uint32_t)(row * DN + col) * 2u;
          vstep[i] = DN * 2u;
        } else {
          rs[i] = rr;
          voff[i] = (uint32_t)(row * DR + (col - DN)) * 2u;
          vstep[i] = DR * 2u;
        }
      } else {
        const int vb = bi - KBLK, d = vb / 4, s = vb % 4;
        int r, x;
        frag_slot<SWV>(s, lane, r, x);
        rs[i] = rv;
        voff[i] = (uint32_t)((32 * d + r) * a.v_ld + 8 * x) * 2u;
        vstep[i] = 2u;
      }
    }
    auto issue = [&](int kt, int buf) __attribute__((always_inline)) {
      const uint32_t key0 = (uint32_t)(kt * BN);
#pragma unroll
      for (int i = 0; i < LPW; ++i) lds_load16(rs[i], &smem[buf][(wave + NW * i) * 64], voff[i] + key0 * vstep[i]);
    };

    // rotary positions of the lane's two query rows. Given positions are
    // looked up and waited for inside their own branch: a load still pending
    // where the branches join would make the other branch wait for every
    // memory operation in flight, the previous item's output stores included.
    int prow[2];
    if (a.pos) {
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int tq = qlo + 32 * r + l32;
        prow[r] = a.pos[(size_t)b * T + (tq < T ? tq : 0)];
      }
#pragma unroll
      for (int r = 0; r < 2; ++r) asm volatile("" : "+v"(prow[r]));
    } else {
#pragma unroll
      for (int r = 0; r < 2; ++r) prow[r] = past + qlo + 32 * r + l32;
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) prow[r] = min(max(prow[r], 0), a.table_len - 1);

    // ---- prologue: rotated (and in fp16 mode pre-scaled) query fragments of
    // both blocks. Every load goes out before any arithmetic, so the whole
    // prologue waits for one memory round trip: the wave's 64 query rows
    // (contiguous in memory) land in LDS as the operand image the key tiles
    // use, each LDS-direct load bringing eight whole 128-byte row segments
    // (rows past the sequence read as zeros); then the cos / sin of the
    // lane's rotary pairs; then the first tile. Rotary chunk cc (16
    // dims, dims 8g..8g+7 in this lane) pairs dims within the chunk
    // (interleaved: 4 pairs) or with chunk cc +- RC/2 (half: 8 pairs, the
    // partner dims in the same lane); either way a lane touches DR/4 pairs,
    // DR/16 runs of four.
    constexpr int RC = DR / 16;
    static_assert(DN % 16 == 0 && DR % 32 == 0, "rotary chunks of 16 dims, two halves");
    static_assert(SWK == 4, "query staging in groups of four k-steps");
    const char* qimg = reinterpret_cast<const char*>(&smem[1][0]) + wave * (2 * QC * 1024);
    {
      const __amdgpu_buffer_rsrc_t rq = make_rsrc(qg, (uint32_t)T * DQK * 2u);
#pragma unroll
      for (int bi = 0; bi < 2 * QC; ++bi) {
        const int r = bi / QC, cq = bi % QC;
        int rr, x;
        frag_slot<SWK>(cq % SWK, lane, rr, x);
        const int col = (cq / SWK) * (16 * SWK) + 8 * x;
        lds_load16(rq, const_cast<char*>(qimg) + bi * 1024, (uint32_t)((qlo + 32 * r + rr) * DQK + col) * 2u);
      }
    }
    u32x4 qf[2][QC];
    f32x4 cw[2][RC], sw[2][RC];
    const int pairing = a.pairing;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int p = prow[r];
#pragma unroll
      for (int k = 0; k < RC; ++k) {
        // first pair of run k: half pairing, chunks k/2 and k/2 + RC/2, its
        // (k&1)-th four pairs; interleaved, chunk k
        const int pi = pairing ? 8 * k + 4 * g : 16 * (k >> 1) + 8 * g + 4 * (k & 1);
        cw[r][k] = *reinterpret_cast<const f32x4*>(a.cos + (size_t)p * (DR / 2) + pi);
        sw[r][k] = *reinterpret_cast<const f32x4*>(a.sin + (size_t)p * (DR / 2) + pi);
      }
    }
    // the first tile's loads go out last: the wait below leaves them in flight
    issue(0, 0);
    // lane's read offsets within an operand group for each k-step position
    int rdk[SWK], rdv[SWV];
#pragma unroll
    for (int c = 0; c < SWK; ++c) rdk[c] = frag_read0<SWK>(l32, g) ^ (32 * c);
#pragma unroll
    for (int c = 0; c < SWV; ++c) rdv[c] = frag_read0<SWV>(l32, g) ^ (32 * c);
    // this wave's staging loads (and the cos / sin) have landed: vmcnt(LPW)
    static_assert(LPW < 16, "vmcnt field");
    __builtin_amdgcn_s_waitcnt(0x0F70 | LPW);
    asm volatile("" ::: "memory");
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int c = 0; c < QC; ++c)
        qf[r][c] = *reinterpret_cast<const u32x4*>(qimg + (r * QC + (c / SWK) * SWK) * 1024 + rdk[c % SWK]);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      auto lo = [](uint32_t w) { return __uint_as_float(w << 16); };
      auto hi = [](uint32_t w) { return __uint_as_float(w & 0xffff0000u); };
      u32x4 rot[RC];
      if (!pairing) {
#pragma unroll
        for (int cc = 0; cc < RC; ++cc) {
          const bool first = cc < RC / 2;
          const u32x4 x = qf[r][DN / 16 + cc], y = qf[r][DN / 16 + (first ? cc + RC / 2 : cc - RC / 2)];
          const int k0 = 2 * (cc % (RC / 2));
          const float sgn = first ? -1.0f : 1.0f;
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            const f32x4 cs = cw[r][k0 + e2 / 2], sn = sw[r][k0 + e2 / 2];
            const int i0 = 2 * (e2 % 2);
            rot[cc][e2] = ET::pack2((lo(x[e2]) * cs[i0] + sgn * (lo(y[e2]) * sn[i0])) * qmul,
                                    (hi(x[e2]) * cs[i0 + 1] + sgn * (hi(y[e2]) * sn[i0 + 1])) * qmul);
          }
        }
      } else {
#pragma unroll
        for (int cc = 0; cc < RC; ++cc) {
          const u32x4 x = qf[r][DN / 16 + cc];
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            const float cs = cw[r][cc][e2], sn = sw[r][cc][e2];
            rot[cc][e2] = ET::pack2((lo(x[e2]) * cs - hi(x[e2]) * sn) * qmul, (hi(x[e2]) * cs + lo(x[e2]) * sn) * qmul);
          }
        }
      }
#pragma unroll
      for (int c = 0; c < QC; ++c) {
        if (c >= DN / 16) {
          qf[r][c] = rot[c - DN / 16];
        } else if (FOLD || ET::code != BF16::code) {
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) qf[r][c][e2] = ET::pack2(lo(qf[r][c][e2]) * qmul, hi(qf[r][c][e2]) * qmul);
        }
      }
    }

    // ---- running state per block
    f32x16 oacc[2][NO];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int d = 0; d < NO; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[r][d][i] = 0.f;
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int d = 0; d < NO; ++d) in_agpr(oacc[r][d]);
    float m_ref[2] = {0.f, 0.f};
    float lsum[2] = {0.f, 0.f};
    bool ref_set = false;
    // fp16 mode: -m_ref broadcast over an accumulator; every score chain starts
    // from it, so the scores leave the MFMA as exp2 arguments
    f32x16 negm[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
#pragma unroll
      for (int i = 0; i < 16; ++i) negm[r][i] = 0.f;
      in_agpr(negm[r]);
    }

    // ---- per-sub-tile state, carried across tiles by the pipeline below
    f32x16 sacc[2][2];  // scores [sub-tile][block]
    u32x4 pf[2][2][2];  // P operands [sub-tile][block][16-key step]
    float ts[2][2];     // per-lane sums of P [sub-tile][block]

    // fragment reads (tile buffer sb): key fragment of sub-tile j, k-step c;
    // value fragment of sub-tile j, value tile d, 16-key step s (0, 1)
    auto kfrag = [&](const char* sb, int j, int c) __attribute__((always_inline)) -> u32x4 {
      return *reinterpret_cast<const u32x4*>(sb + (j * QC + (c / SWK) * SWK) * 1024 + rdk[c % SWK]);
    };
    auto vfrag = [&](const char* sb, int j, int d, int s) __attribute__((always_inline)) -> u32x4 {
      const int st = 2 * j + s;  // 16-key step within the tile
      return *reinterpret_cast<const u32x4*>(sb + (KBLK + d * 4 + (st / SWV) * SWV) * 1024 + rdv[st % SWV]);
    };
    // the two MFMAs of a key step (both blocks) and of a value step
    // the MFMA of block r of a key step and of a value step
    auto s_mfma = [&](int j, int c, int r, u32x4 f) __attribute__((always_inline)) {
      if (c == 0) {
        if (FOLD) {
          sacc[j][r] = ET::mma(f, qf[r][0], negm[r]);
        } else {
          f32x16 z;
#pragma unroll
          for (int e = 0; e < 16; ++e) z[e] = 0.f;
          sacc[j][r] = ET::mma(f, qf[r][0], z);
        }
      } else {
        sacc[j][r] = ET::mma(f, qf[r][c], sacc[j][r]);
      }
    };
    auto pv_mfma = [&](int j, int d, int s, int r, u32x4 f) __attribute__((always_inline)) {
      oacc[r][d] = ET::mma(f, pf[j][r][s], oacc[r][d]);
      in_agpr(oacc[r][d]);
    };

    // Softmax of sub-tile j, one score at a time. Once a block's score chain
    // is complete its 16 accumulators are copied to vector registers in two
    // halves of 8, in successive half-steps (copy_half; one copy of all 16 at
    // the first use would stall the MFMA pipe), and the softmax reads the
    // copies: score v (0..31) is element v % 16 of block v / 16. Each score is
    // scaled (bf16 mode), masked (diagonal tiles) and turned into P; the odd
    // score of a pair packs both (16-bit, the B operand of P V), pinned where
    // it is computed. The lane's row sum takes every P in fp32 adds (a packed
    // dot product would not overlap the MFMAs).
    typedef float f32x8 __attribute__((ext_vector_type(8)));
    f32x8 sv[2][2][2];  // score copies [sub-tile][block][half]
    float pev[2];       // P of the even score of the pair in progress [sub-tile]
    auto copy_half = [&](int j, int r, int hh) __attribute__((always_inline)) {
      in_agpr(sacc[j][r]);  // holds the reads at this point
      f32x8 t;
#pragma unroll
      for (int i = 0; i < 8; ++i) t[i] = sacc[j][r][8 * hh + i];
      in_vgpr(t);
      sv[j][r][hh] = t;
    };
    // score i of block r of sub-tile j as an exp2 argument: scaled (bf16
    // mode) and masked (diagonal tiles)
    auto prepped = [&](int j, int r, int i, int key0, bool diag) __attribute__((always_inline)) -> float {
      float x = sv[j][r][i / 8][i % 8];
      if (!FOLD) x = fmaf(x, sl2, -m_ref[r]);
      if (diag) {
        const int e = i / 2;
        const int kb = key0 + 32 * j + 16 * (e >> 2) + 8 * g + 2 * (e & 3) + (i & 1);
        if (kb > past + qlo + 32 * r + l32) x = -INFINITY;
      }
      return x;
    };
    auto put_p = [&](int j, int r, int e, float p0, float p1) __attribute__((always_inline)) {
      const uint32_t w = ET::pack2(p0, p1);
      asm volatile("" ::"v"(w));  // packed here, not sunk past the rare-path branch
      pf[j][r][e >> 2][e & 3] = w;
    };
    auto score = [&](int j, int v, int key0, bool diag) __attribute__((always_inline)) {
      const int r = v / 16, i = v % 16;
      const float pv = __builtin_amdgcn_exp2f(prepped(j, r, i, key0, diag));
      ts[j][r] = i == 0 ? pv : ts[j][r] + pv;
      if (i % 2 == 0) pev[j] = pv;
      else put_p(j, r, i / 2, pev[j], pv);
    };
    // scores [v0, v1) of sub-tile j
    auto scores = [&](int j, int v0, int v1, int key0, bool diag) __attribute__((always_inline)) {
#pragma unroll
      for (int v = v0; v < v1; ++v) score(j, v, key0, diag);
    };

    // The rare path after the softmax of sub-tile j: the exact maximum of its
    // scores, and the reference moved to it on the first sub-tile or wherever
    // a score exceeds it by more than the slack (exact: O and the row sum share
    // the reference); P and the row sums of sub-tile j are then recomputed
    // from its copies. `pend`: the other sub-tile's scores were already
    // accumulated onto the old -m_ref (fp16 mode, not yet copied) and move
    // with it.
    auto check = [&](int j, bool pend, int key0, bool diag) __attribute__((always_inline)) {
      if (__any(!ref_set || ts[j][0] > kSumLimD || ts[j][1] > kSumLimD)) {
        float shift[2];
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          float mx = -INFINITY;
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, prepped(j, r, i, key0, diag));
          mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
          const bool raise = !ref_set || mx > kSlackD;
          shift[r] = raise ? mx : 0.f;
          const float alpha = (raise && ref_set) ? __builtin_amdgcn_exp2f(-mx) : 1.f;
          m_ref[r] += shift[r];
          lsum[r] *= alpha;
#pragma unroll
          for (int d = 0; d < NO; ++d) {
            // pin the accumulators to their registers on both sides of the
            // rescale, so that their copies for it stay on this rare path
            in_agpr(oacc[r][d]);
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[r][d][i] *= alpha;
            in_agpr(oacc[r][d]);
          }
          if (FOLD) {
            if (pend) {
              // kept in the accumulation registers, as the common path holds it
              in_agpr(sacc[1 - j][r]);
#pragma unroll
              for (int i = 0; i < 16; ++i) sacc[1 - j][r][i] -= shift[r];
              in_agpr(sacc[1 - j][r]);
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) negm[r][i] = -m_ref[r];
            in_agpr(negm[r]);
          }
        }
        ref_set = true;
        // bf16 mode: prepped() now subtracts the moved reference itself
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          float t = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float c = FOLD ? shift[r] : 0.f;
            const float p0 = __builtin_amdgcn_exp2f(prepped(j, r, 2 * e, key0, diag) - c);
            const float p1 = __builtin_amdgcn_exp2f(prepped(j, r, 2 * e + 1, key0, diag) - c);
            pf[j][r][e >> 2][e & 3] = ET::pack2(p0, p1);
            t += p0 + p1;
          }
          ts[j][r] = t;
        }
      }
      lsum[0] += ts[j][0];
      lsum[1] += ts[j][1];
    };

    // A sequence of steps: step k reads ahead the fragment of step k + PF and
    // issues the two MFMAs of step k on its own fragment, then a softmax
    // piece range; a scheduling fence closes every step. Steps are numbered
    // within one pipelined tile (see body below): 0-11 key steps of sub-tile
    // 0, 12-19 value steps of the previous tile's sub-tile 1, 20-31 key steps
    // of sub-tile 1, 32-39 value steps of sub-tile 0.
    auto fetch = [&](const char* cur, const char* prev, int id) __attribute__((always_inline)) -> u32x4 {
      if (id < 12) return kfrag(cur, 0, id);
      if (id < 20) return vfrag(prev, 1, (id - 12) / 2, (id - 12) % 2);
      if (id < 32) return kfrag(cur, 1, id - 20);
      return vfrag(cur, 0, (id - 32) / 2, (id - 32) % 2);
    };
    auto mfma_of = [&](int id, int r, u32x4 f) __attribute__((always_inline)) {
      if (id < 12) s_mfma(0, id, r, f);
      else if (id < 20) pv_mfma(1, (id - 12) / 2, (id - 12) % 2, r, f);
      else if (id < 32) s_mfma(1, id - 20, r, f);
      else pv_mfma(0, (id - 32) / 2, (id - 32) % 2, r, f);
    };
    constexpr int SA = 12;  // scores of a sub-tile whose softmax runs under its own tile's value steps
    // n steps; step k is step order_id(k) of the numbering above. Each step
    // reads ahead the fragment of step k + PF, then issues its two MFMAs (block
    // 0, block 1), each followed by `between(k, h)` for half h: softmax
    // scores, tile loads, the rare-path checks, closed by a scheduling fence.
    // A wave's second MFMA stalls its issue until the first leaves the unit,
    // so VALU work placed after each of the two keeps both gaps busy. The
    // read-ahead runs across the checks, so no step waits for a fresh LDS read.
    auto run = [&](const char* cur, const char* prev, auto order_c, auto&& between) __attribute__((always_inline)) {
      constexpr int M = decltype(order_c)::value;
      constexpr int N = order_len(M);
      u32x4 fr[PF + 1];
      static_for<0, (PF < N ? PF : N)>([&](auto kc) __attribute__((always_inline)) {
        constexpr int k = decltype(kc)::value;
        fr[k] = fetch(cur, prev, order_id(M, k));
      });
      // the copies of a finished score chain (last key step: id 11 or 31 at
      // position kl): block 0 low half after kl's second MFMA, block 0 high
      // half and block 1 low half in the next step, block 1 high half in the
      // one after; each after that half-step's own work
      auto chain_end = [](int kk) { return kk >= 0 && kk < N && (order_id(M, kk) == 11 || order_id(M, kk) == 31); };
      auto chain_of = [](int kk) { return order_id(M, kk) == 11 ? 0 : 1; };
      static_for<0, N>([&](auto kc) __attribute__((always_inline)) {
        constexpr int k = decltype(kc)::value;
        constexpr int id = order_id(M, k);
        if constexpr (k + PF < N) fr[(k + PF) % (PF + 1)] = fetch(cur, prev, order_id(M, k + PF));
        mfma_of(id, 0, fr[k % (PF + 1)]);
        fence();
        between(kc, IntC<0>{});
        if constexpr (chain_end(k - 1)) copy_half(chain_of(k - 1), 0, 1);
        if constexpr (chain_end(k - 2)) copy_half(chain_of(k - 2), 1, 1);
        fence();
        mfma_of(id, 1, fr[k % (PF + 1)]);
        fence();
        between(kc, IntC<1>{});
        if constexpr (chain_end(k)) copy_half(chain_of(k), 0, 0);
        if constexpr (chain_end(k - 1)) copy_half(chain_of(k - 1), 1, 0);
        fence();
      });
    };
    // scores [v0 + n q / m, v0 + n (q+1) / m) of sub-tile j: the q-th of m
    // equal shares of n scores starting at v0
    auto share = [&](int j, int v0, int n, int m, int q, int key0, bool diag) __attribute__((always_inline)) {
      scores(j, v0 + n * q / m, v0 + n * (q + 1) / m, key0, diag);
    };
    // one of this wave's LDS-direct loads of tile kt into buffer bf
    auto issue_one = [&](int i, int kt, int bf) __attribute__((always_inline)) {
      lds_load16(rs[i], &smem[bf][(wave + NW * i) * 64], voff[i] + (uint32_t)(kt * BN) * vstep[i]);
    };

    // One tile in the software pipeline: while the scores of its first 32 keys
    // are multiplied, the softmax of the previous tile's last 32 keys runs on
    // the VALU; then that sub-tile's P V (its values still in the previous
    // buffer) under the first scores of this tile's softmax of keys 0-31; then
    // the scores of keys 32-63 under the rest of it; then the P V of keys 0-31
    // under the first scores of the softmax of keys 32-63, whose remainder and
    // P V are left to the next tile. FIRST: no previous tile. The loads of the
    // next tile (nxt >= 0: its index, into buffer nbf) go into the half-steps
    // whose share of scores is empty, where the VALU has the most slack: the
    // first of every six half-steps of steps 0-11, of every four of steps
    // 12-19, and the last two at step 20 (measured 3.5% fewer cycles per tile
    // than one load in every other step).
    auto body = [&](const char* cur, const char* prev, int key0, int nxt, int nbf, auto first_c)
                    __attribute__((always_inline)) {
      constexpr bool FIRST = decltype(first_c)::value;
      static_assert(LPW == 10, "the load slots below place ten loads per wave");
      auto loads = [&](int k, int h) __attribute__((always_inline)) {
        const int q = k < 12 ? 2 * k + h : 2 * (k - 12) + h;  // half-step within the share group
        const bool empty = k < 12 ? q % 6 == 0 : (k < 20 && q % 4 == 0);
        const int slot = k < 12 ? q / 6 : 4 + q / 4;
        if (empty && nxt >= 0) issue_one(slot, nxt, nbf);
        if (k == 20 && h == 0 && nxt >= 0) {
          issue_one(8, nxt, nbf);
          issue_one(9, nxt, nbf);
        }
      };
      if (!FIRST) {
        run(cur, prev, IntC<kPipe>{}, [&](auto kc, auto hc) __attribute__((always_inline)) {
          constexpr int k = decltype(kc)::value, h = decltype(hc)::value;
          if (k < 12) share(1, SA, 32 - SA, 24, 2 * k + h, 0, false);
          else if (k < 20) share(0, 0, SA, 16, 2 * (k - 12) + h, key0, false);
          else if (k < 32) share(0, SA, 32 - SA, 24, 2 * (k - 20) + h, key0, false);
          else share(1, 0, SA, 16, 2 * (k - 32) + h, key0, false);
          loads(k, h);
          if (h == 1 && k == 11) {
            fence();
            check(1, true, 0, false);
          }
          if (h == 1 && k == 31) {
            fence();
            check(0, true, key0, false);
          }
        });
      } else {
        run(cur, prev, IntC<kFirst>{}, [&](auto kc, auto hc) __attribute__((always_inline)) {
          constexpr int k = decltype(kc)::value, h = decltype(hc)::value;
          constexpr int id = order_id(kFirst, k);
          if (id >= 20 && id < 32) share(0, 0, 32, 24, 2 * (id - 20) + h, key0, false);
          if (id >= 32) share(1, 0, SA, 16, 2 * (id - 32) + h, key0, false);
          loads(k, h);
          if (h == 1 && id == 31) {
            fence();
            check(0, true, key0, false);
          }
        });
      }
    };
    // the pipeline's tail: the rest of the softmax of the last tile's keys
    // 32-63 and their P V (values in buffer prev)
    auto drain = [&](const char* prev) __attribute__((always_inline)) {
      scores(1, SA, 32, 0, false);
      check(1, false, 0, false);
      run(prev, prev, IntC<kDrain>{}, [](auto, auto) {});
    };
    // A whole tile outside the pipeline, for tiles that cross the wave's
    // diagonal: scores of keys 0-31; scores of keys 32-63 under the masked
    // softmax of keys 0-31; P V of keys 0-31 under the softmax of keys 32-63;
    // P V of keys 32-63 (same step numbering, this tile's buffer as the
    // "previous" one).
    auto tile_diag = [&](const char* cur, int key0) __attribute__((always_inline)) {
      run(cur, cur, IntC<kDiag>{}, [&](auto kc, auto hc) __attribute__((always_inline)) {
        constexpr int id = order_id(kDiag, decltype(kc)::value), h = decltype(hc)::value;
        if (id >= 20 && id < 32) share(0, 0, 32, 24, 2 * (id - 20) + h, key0, true);
        if (id >= 32) share(1, 0, 32, 16, 2 * (id - 32) + h, key0, true);
        if (h == 1 && id == 31) {
          fence();
          check(0, true, key0, true);
        }
        if (h == 1 && id == 39) {
          fence();
          check(1, false, key0, true);
        }
      });
    };

    // Tile kt lives in buffer kt % 3; the loads of tile kt+1 are issued at
    // the start of tile kt. Three buffers: the pipelined tile still reads the
    // previous tile's values while the next tile lands. At the end of a tile
    // each wave waits for its own loads, then the barrier makes every wave's
    // loads visible and frees the oldest buffer. The pipelined loop is unrolled
    // three times so that every buffer address is a constant.
    static_assert(NBUF == 3, "the pipeline needs three tile buffers");
    auto buf = [&](int i) __attribute__((always_inline)) {
      return reinterpret_cast<const char*>(&smem[i][0]);
    };
    auto wait_next = [&]() __attribute__((always_inline)) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    };
    // one pipelined tile kt held in buffer B (a constant)
    auto iter = [&](int kt, auto bc) __attribute__((always_inline)) {
      constexpr int B = decltype(bc)::value;
      body(buf(B), buf((B + 2) % 3), kt * BN, kt + 1 < nkt ? kt + 1 : -1, (B + 1) % 3, FalseT{});
      wait_next();
    };
    wait_next();
    // Tiles below the wave's diagonal go through the pipeline; the tiles that
    // cross it are processed whole, after the pipeline is drained. Every wave
    // takes part in the loads and barriers of all nkt tiles; s_barrier counts
    // arrivals, so the loops of different waves meet at the same barriers.
    const int nfull = min(nkt, max(0, (past + qlo + 1) / BN));  // tiles whose last key <= the wave's first row
    if (nfull > 0) {
      body(buf(0), buf(0), 0, 1 < nkt ? 1 : -1, 1, TrueT{});
      wait_next();
    }
    int kt = 1;
    for (; kt + 2 < nfull; kt += 3) {
      iter(kt, IntC<1>{});
      iter(kt + 1, IntC<2>{});
      iter(kt + 2, IntC<0>{});
    }
    if (kt < nfull) iter(kt++, IntC<1>{});
    if (kt < nfull) iter(kt++, IntC<2>{});
    for (kt = nfull; kt < nkt; ++kt) {
      if (kt + 1 < nkt) issue(kt + 1, (kt + 1) % 3);
      if (kt == nfull && nfull > 0) drain(buf((kt - 1) % 3));
      const int key0 = kt * BN;
      if (key0 <= past + qlo + 63) tile_diag(buf(kt % 3), key0);
      wait_next();
    }
    if (nfull > 0 && nfull == nkt) drain(buf((nkt - 1) % 3));

    // ---- epilogue: normalise; each wave stages its 64 x DV output tile in its
    // own part of the free tile buffers (16-byte chunks XOR-swizzled by row) and
    // writes whole rows
    {
      constexpr int CPR = DV / 8;
      static_assert((CPR & (CPR - 1)) == 0 && CPR <= 64, "row swizzle needs a power-of-two chunk count");
      char* stile = reinterpret_cast<char*>(&smem[0][0]) + wave * (64 * DV * 2);
      float ltot[2];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        ltot[r] = lsum[r] + __shfl_xor(lsum[r], 32, 64);
        const float inv = 1.0f / ltot[r];
        const int row = 32 * r + l32;
#pragma unroll
        for (int d = 0; d < NO; ++d) {
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int c = d * 4 + r4;
            u32x2 o;
            o[0] = pack2bf(oacc[r][d][r4 * 4 + 0] * inv, oacc[r][d][r4 * 4 + 1] * inv);
            o[1] = pack2bf(oacc[r][d][r4 * 4 + 2] * inv, oacc[r][d][r4 * 4 + 3] * inv);
            *reinterpret_cast<u32x2*>(stile + row * (DV * 2) + ((c ^ (row & (CPR - 1))) * 16) + 8 * g) = o;
          }
        }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's staging writes
      asm volatile("" ::: "memory");
      constexpr int RPI = 64 / CPR;
      const int ch = lane % CPR;
#pragma unroll
      for (int rep = 0; rep < 64 / RPI; ++rep) {
        const int row = lane / CPR + RPI * rep;
        const u32x4 v = *reinterpret_cast<const u32x4*>(stile + row * (DV * 2) + ((ch ^ (row & (CPR - 1))) * 16));
        if (qlo + row < T)
          __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(a.out + (bh * T + qlo + row) * DV + ch * 8));
      }
      if (a.lse && g == 0) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const int tq = qlo + 32 * r + l32;
          if (tq < T) a.lse[bh * T + tq] = (m_ref[r] + log2f(ltot[r])) * kLn2D;
        }
      }
    }
    // the next item's first tile lands where this one staged its output:
    // every wave's staging reads are done (the output stores may still be
    // in flight)
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
  }
}

bool prefill_dual_supported(int Dqk, int Dr, int Dv) { return Dqk == 192 && Dr == 64 && Dv == 128; }

namespace {
// compute units of the current device (cached per device)
int device_cus() {
  static int cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64 && cache[dev] > 0) return cache[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) cache[dev] = n;
  return n;
}
}  // namespace

hipError_t launch_prefill_dual(const PrefillArgs& a, hipStream_t stream) {
  constexpr int BM = 256;
  const int nqt = (a.T + BM - 1) / BM;
  const int nitems = (a.H * a.B + 7) / 8 * nqt;  // work items per XCD
  // one workgroup per CU (the kernel's LDS and registers fill a CU), eight
  // XCDs; a device reporting fewer CUs still gets one workgroup per XCD
  const int nc = std::max(1, std::min(device_cus() / 8, nitems));
  hipLaunchKernelGGL((prefill_dual_kernel<F16, 192, 64, 128, 3, 3>), dim3((unsigned)(8 * nc)), dim3(256), 0, stream,
                     a, nqt);
  return hipGetLastError();
}

}  // namespace mla
