// Host-side launchers of the gfx950 kernels. Arguments have been validated
// by the C-ABI layer (api.cpp) before any of these is called; each launcher
// only queues work on `stream` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mla {

// Rotary table parameters resolved on the host: the correction band and the
// mscale ratio (double on the host, handed to the device as fp32).
struct RopeResolved {
  int dim;
  int yarn;
  float base;
  float factor;
  float low;
  float high;
  float mscale;
};

hipError_t launch_rope_table(const RopeResolved& r, int n_pos, float* cos_out, float* sin_out,
                             hipStream_t stream);

hipError_t launch_rmsnorm(const uint16_t* x, const uint16_t* w, float eps, uint16_t* y, int n, int R, int out_dtype,
                          hipStream_t stream);

// latent RMSNorm (fp16 out) and the rotation of each token's shared rotary
// key (fp16 out) in one launch; R a multiple of 8 (<= 4096), rows 16-byte
// aligned
struct LatentPrepareArgs {
  const uint16_t* x;     // [n, R] bf16 latent
  const uint16_t* w;     // [R] bf16 gain
  float eps;
  uint16_t* y;           // [n, R] fp16
  const uint16_t* k_pe;  // [n, Dr] bf16, n = B*T
  const float* cos;
  const float* sin;
  int table_len;
  const int32_t* pos;    // [n] or null (= t)
  uint16_t* k_rot;       // [n, Dr] fp16
  int n, T, R, Dr, pairing;
};
hipError_t launch_latent_prepare(const LatentPrepareArgs& a, hipStream_t stream);

struct ExpandArgs {
  const uint16_t* c;  // [B*T, R] normalised latent, fp16
  const uint16_t* W;  // [N, R], N = H*(Dn+Dv)
  uint16_t* k;        // [B, H, Tcap, k_ld]
  uint16_t* v;        // [B, H, Tcap, Dv] (v_cols == 0) or [B, H, Dv, v_ld] (v_cols == 1)
  int B, T, R, H, Dn, Dv, k_ld, Tcap, t_off;
  int kv_dtype;       // element type of k and v: 0 bf16, 1 fp16
  int v_cols;         // values stored transposed (V^T)
  int v_ld;           // row stride of V^T (>= Tcap); columns Tcap..v_ld-1 are zeroed
};
hipError_t launch_kv_expand(const ExpandArgs& a, hipStream_t stream);

// Rotate the shared rotary key of every token (b, t) at pos[b*T+t] (or
// t_off+t) and write it to dst + ((b*H + h)*Tcap + t_off + t)*ld + col for
// every head h in [0, H) (H = 1 with Tcap = T, t_off = 0 gives a compact
// [B, T, Dr] copy).
struct RotKeyArgs {
  const uint16_t* k_pe;  // [B, T, Dr]
  const float* cos;
  const float* sin;
  int table_len;
  const int32_t* pos;  // [B, T] or null
  uint16_t* dst;
  int B, T, H, Dr, Tcap, t_off, ld, col, pairing;
  int dtype;  // element type of dst: 0 bf16, 1 fp16
};
hipError_t launch_rotate_key(const RotKeyArgs& a, hipStream_t stream);

struct PrefillArgs {
  const uint16_t* q;       // [B, H, T, Dqk]
  const uint16_t* k_nope;  // [B, H, kv_stride, Dn] (kv_dtype), rows 0..past+T-1 read
  const uint16_t* k_rot;   // [B, kv_stride, Dr] rotated (kv_dtype)
  const uint16_t* v;       // V^T [B, H, Dv, v_ld] (kv_dtype), columns past+T..v_ld-1 finite
  const float* cos;
  const float* sin;
  int table_len;
  const int32_t* pos;  // [B, T] or null
  uint16_t* out;       // [B, H, T, Dv]
  float* lse;          // [B, H, T] or null
  int B, H, T, Dn, Dr, Dv, pairing;
  float scale;
  int kv_dtype;  // 0 bf16, 1 fp16
  int v_ld;      // row stride of V^T, a multiple of 8, >= past + T
  int past;      // cached rows before the T query rows (0 for a plain prefill)
  int kv_stride; // row capacity of k_nope [B, H, kv_stride, Dn] and k_rot [B, kv_stride, Dr]
};
bool prefill_supported(int Dqk, int Dr, int Dv);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);
// 192/128 heads, two 32-row query blocks per wave (prefill_dual.hip)
bool prefill_dual_supported(int Dqk, int Dr, int Dv);
hipError_t launch_prefill_dual(const PrefillArgs& a, hipStream_t stream);
// row-major values [BH, T, Dv] -> V^T [BH, Dv, v_ld], columns T..v_ld-1 zero
hipError_t launch_transpose_v(const uint16_t* v, uint16_t* vt, int BH, int T, int Dv, int v_ld, hipStream_t stream);

struct DecodeArgs {
  const uint16_t* q;        // [B, H, 1, Dqk]
  const uint16_t* k_cache;  // [B, H, Tcap, Dqk] (cache_dtype)
  const uint16_t* v_cache;  // [B, H, Tcap, Dv]  (cache_dtype)
  const int32_t* seq_len;   // [B]
  const int32_t* q_pos;     // [B]
  const float* cos;
  const float* sin;
  int table_len;
  int B, H, Tcap, Dn, Dr, Dv, pairing, num_splits;
  float scale;
  float* part_o;  // [B, H, S, Dv]
  float* part_ml; // [B, H, S, 2]
  uint16_t* out;  // [B, H, 1, Dv]
  int cache_dtype;  // 0 bf16, 1 fp16
};
bool decode_supported(int Dqk, int Dv);
int decode_auto_splits(int B, int H, int Tcap);
size_t decode_workspace_bytes(int B, int H, int Dv, int splits);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
// the allocation-free decode entry point's scratch: its size, and its device
// address on the current device (looked up once per device)
constexpr size_t kDecodeScratchBytes = (size_t)16 << 20;
hipError_t decode_scratch(void** ptr);

// ---- decode against a compressed-latent cache (absorbed form); the cache
// row is 576 fp16 values: 512 latent then 64 rotated rotary key
constexpr int kLatentR = 512;
constexpr int kLatentDr = 64;
constexpr int kMaxLatentSplits = 64;

hipError_t launch_absorb_prepare(const uint16_t* W, uint16_t* wt, int H, int R, int Dn, int Dv, hipStream_t stream);

struct LatentAppendArgs {
  const uint16_t* latent;  // [B, R] bf16
  const uint16_t* gain;    // [R] bf16
  float eps;
  const uint16_t* k_pe;  // [B, Dr] bf16, not rotated
  const float* cos;
  const float* sin;
  int table_len;
  const int32_t* t_pos;  // [B]: cache row and rotary position
  int pairing, B, R, Dr, Lcap;
  uint16_t* cache;  // [B, Lcap, R+Dr] fp16
};
hipError_t launch_latent_append(const LatentAppendArgs& a, hipStream_t stream);

struct AbsorbArgs {
  const uint16_t* q;      // [B, H, 1, Dn+Dr] bf16
  const uint16_t* w_ukt;  // [H, 512, Dn] bf16
  const int32_t* q_pos;   // [B]
  const float* cos;
  const float* sin;
  int table_len;
  int B, H, Dn, Dr, pairing;
  float qscale;  // scale * log2(e)
  uint16_t* qa;  // [B, H, 576] fp16
};
hipError_t launch_absorb_q(const AbsorbArgs& a, hipStream_t stream);

struct LatentAttnArgs {
  const uint16_t* qa;      // [B, H, 576] fp16
  const uint16_t* cache;   // [B, Lcap, 576] fp16
  const int32_t* seq_len;  // [B]
  uint16_t* part_o;        // [B, S, H, 512] fp16, normalised per split
  float* part_lse;         // [B, S, H] log2 domain, -inf for an empty split
  int B, H, Lcap, S, tps;  // splits, 64-key tiles per split
};
hipError_t launch_latent_attn(const LatentAttnArgs& a, hipStream_t stream);

struct CombineUnabsorbArgs {
  const uint16_t* part_o;  // [B, S, H, 512] fp16 split outputs
  const float* part_lse;   // [B, S, H] log2-domain
  const uint16_t* W;       // [H*(Dn+Dv), 512] bf16
  uint16_t* out;           // [B, H, 1, Dv] bf16
  int B, H, S, Dn, Dv;
};
hipError_t launch_combine_unabsorb(const CombineUnabsorbArgs& a, hipStream_t stream);

// latent cache -> contiguous latent rows [B*Lcap, R] and the rotated key
// broadcast into columns Dn.. of the expanded key cache [B, H, Lcap, Dn+Dr]
// (R and Dr multiples of 8, rows 16-byte aligned)
hipError_t launch_latent_reexpand_copies(const uint16_t* cache, uint16_t* c, uint16_t* k, int B, int H, int Lcap,
                                         int R, int Dr, int Dn, hipStream_t stream);

// ---- linear layer Y = X W^T (+ bias), bf16
struct LinearArgs {
  const uint16_t* x;     // x_mode 0: [M, K]; 1: [B, K/Dx, xT, Dx] with M = B*xT
  const uint16_t* w;     // [N, K]
  const uint16_t* bias;  // [N] or null
  uint16_t* y0;          // y_mode 0: [M, N]; 1: [B, N/yD, yT, yD]; 2: [M, ys]
  uint16_t* y1;          // y_mode 2: [M, N - ys]
  int M, N, K;
  int x_mode, xT, x_dlog2;
  int y_mode, yT, yD, ys;
};
hipError_t launch_linear(const LinearArgs& a, hipStream_t stream);

}  // namespace mla
