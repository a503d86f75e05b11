// C ABI of the library: argument validation on the host, then the kernel
// launchers. Every check runs before any HIP call, so a rejected call queues
// nothing and touches no device state.
#include <math.h>
#include <stdint.h>

#include "../../include/mla.h"
#include "launch.hpp"

namespace {

constexpr int64_t kMaxElems = (int64_t)1 << 40;  // sanity bound on tensor sizes

bool rope_type_ok(int32_t t) { return t == MLA_ROPE_DEFAULT || t == MLA_ROPE_YARN; }
bool pairing_ok(int32_t p) { return p == MLA_PAIR_HALF || p == MLA_PAIR_INTERLEAVED; }
bool dtype_ok(int32_t d) { return d == MLA_DTYPE_BF16 || d == MLA_DTYPE_FP16; }
bool aligned16(const void* p) { return (((uintptr_t)p) & 15) == 0; }

// YaRN magnitude correction (Kimi-K2 "RoPE coefficients": 1 when the scale
// factor is at most 1, else 0.1*mscale*ln(factor) + 1).
double yarn_mscale(double scale, double mscale) {
  if (scale <= 1.0) return 1.0;
  return 0.1 * mscale * log(scale) + 1.0;
}

// Correction dim of a rotation count (same page, yarn_find_correction_dim).
double yarn_corr_dim(double nrot, int dim, double base, double max_pos) {
  return (dim * log(max_pos / (nrot * 2.0 * M_PI))) / (2.0 * log(base));
}

mla_status check_rope(const mla_rope_params* p) {
  if (!p) return MLA_ERR_NULL;
  if (!rope_type_ok(p->type)) return MLA_ERR_ROPE_TYPE;
  if (p->rope_dim < 2 || p->rope_dim > 256 || (p->rope_dim & 1)) return MLA_ERR_SHAPE;
  if (!(p->base > 1.0) || !isfinite(p->base)) return MLA_ERR_SHAPE;
  if (p->type == MLA_ROPE_YARN) {
    if (!(p->factor > 0.0) || !isfinite(p->factor) || p->original_max_pos <= 0 || !(p->beta_fast > 0.0) ||
        !(p->beta_slow > 0.0) || !isfinite(p->mscale) || !isfinite(p->mscale_all_dim))
      return MLA_ERR_SHAPE;
    // the mscale ratio must be finite and non-zero
    const double den = yarn_mscale(p->factor, p->mscale_all_dim);
    if (den == 0.0 || !isfinite(den)) return MLA_ERR_SHAPE;
  }
  return MLA_OK;
}

mla_status hip_status(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_HIP; }

// The launchers report hipGetLastError() after queueing their kernels. Clear
// any error an earlier, unrelated runtime call left behind first, so that it
// is not reported as a failure of this call.
void clear_stale_error() { (void)hipGetLastError(); }

}  // namespace

extern "C" {

const char* mla_status_string(mla_status s) {
  switch (s) {
    case MLA_OK: return "ok";
    case MLA_ERR_NULL: return "null pointer";
    case MLA_ERR_SHAPE: return "invalid shape or size";
    case MLA_ERR_UNSUPPORTED: return "unsupported head dimensions";
    case MLA_ERR_ROPE_TYPE: return "unknown rotary type or pairing";
    case MLA_ERR_WORKSPACE: return "workspace missing or too small";
    case MLA_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

mla_status mla_softmax_scale(const mla_rope_params* p, int32_t qk_head_dim, double* scale_out) {
  mla_status st = check_rope(p);
  if (st != MLA_OK) return st;
  if (!scale_out) return MLA_ERR_NULL;
  if (qk_head_dim < 1) return MLA_ERR_SHAPE;
  double s = pow((double)qk_head_dim, -0.5);
  if (p->type == MLA_ROPE_YARN && p->mscale_all_dim != 0.0) {
    const double g = yarn_mscale(p->factor, p->mscale_all_dim);
    s = s * g * g;
  }
  *scale_out = s;
  return MLA_OK;
}

mla_status mla_rope_table_build(const mla_rope_params* p, int32_t n_pos, float* cos_out, float* sin_out,
                                double* attn_mscale2, hipStream_t stream) {
  mla_status st = check_rope(p);
  if (st != MLA_OK) return st;
  if (!cos_out || !sin_out) return MLA_ERR_NULL;
  if (n_pos < 1 || (int64_t)n_pos * (p->rope_dim / 2) > ((int64_t)1 << 31) - 1) return MLA_ERR_SHAPE;
  mla::RopeResolved r;
  r.dim = p->rope_dim;
  r.base = (float)p->base;
  r.yarn = p->type == MLA_ROPE_YARN;
  r.factor = (float)(r.yarn ? p->factor : 1.0);
  r.low = 0.f;
  r.high = 1.f;
  r.mscale = 1.f;
  double m2 = 1.0;
  if (r.yarn) {
    // correction band in double, as the page computes it with Python floats
    double lo = floor(yarn_corr_dim(p->beta_fast, p->rope_dim, p->base, p->original_max_pos));
    double hi = ceil(yarn_corr_dim(p->beta_slow, p->rope_dim, p->base, p->original_max_pos));
    if (lo < 0) lo = 0;
    if (hi > p->rope_dim - 1) hi = p->rope_dim - 1;
    if (lo == hi) hi += 0.001;  // degenerate band
    r.low = (float)lo;
    r.high = (float)hi;
    r.mscale = (float)(yarn_mscale(p->factor, p->mscale) / yarn_mscale(p->factor, p->mscale_all_dim));
    if (p->mscale_all_dim != 0.0) {
      const double g = yarn_mscale(p->factor, p->mscale_all_dim);
      m2 = g * g;
    }
  }
  if (attn_mscale2) *attn_mscale2 = m2;
  clear_stale_error();
  return hip_status(mla::launch_rope_table(r, n_pos, cos_out, sin_out, stream));
}

mla_status mla_latent_rmsnorm(const mla_bf16* x, const mla_bf16* w, float eps, uint16_t* y, int32_t n, int32_t R,
                              hipStream_t stream) {
  if (n < 0 || R < 1 || R > 8192 || !(eps >= 0.0f) || !isfinite(eps)) return MLA_ERR_SHAPE;
  if ((int64_t)n * R > kMaxElems) return MLA_ERR_SHAPE;
  if (n == 0) return MLA_OK;
  if (!x || !w || !y) return MLA_ERR_NULL;
  clear_stale_error();
  return hip_status(mla::launch_rmsnorm(x, w, eps, y, n, R, MLA_DTYPE_FP16, stream));
}

mla_status mla_latent_prepare(const mla_bf16* latent, const mla_bf16* gain, float eps, const mla_bf16* k_pe,
                              const float* cos, const float* sin, int32_t table_len, const int32_t* pos, int32_t B,
                              int32_t T, int32_t R, int32_t Dr, int32_t pairing, uint16_t* c_norm, uint16_t* k_rot,
                              hipStream_t stream) {
  if (B < 0 || T < 0 || R < 8 || R > 4096 || (R % 8) || Dr < 2 || Dr > 256 || (Dr & 1)) return MLA_ERR_SHAPE;
  if (!(eps >= 0.0f) || !isfinite(eps)) return MLA_ERR_SHAPE;
  if (!pairing_ok(pairing)) return MLA_ERR_ROPE_TYPE;
  if ((int64_t)B * T > ((int64_t)1 << 31) - 1 || (int64_t)B * T * R > kMaxElems) return MLA_ERR_SHAPE;
  if ((int64_t)B * T == 0) return MLA_OK;
  if (!latent || !gain || !k_pe || !cos || !sin || !c_norm || !k_rot) return MLA_ERR_NULL;
  if (table_len < 1 || (!pos && T > table_len)) return MLA_ERR_SHAPE;
  if (!aligned16(latent) || !aligned16(gain) || !aligned16(c_norm)) return MLA_ERR_SHAPE;
  clear_stale_error();
  mla::LatentPrepareArgs a{latent, gain, eps, c_norm, k_pe, cos, sin, table_len, pos, k_rot, B * T, T, R, Dr, pairing};
  return hip_status(mla::launch_latent_prepare(a, stream));
}

mla_status mla_rmsnorm(const mla_bf16* x, const mla_bf16* w, float eps, uint16_t* y, int32_t n, int32_t R,
                       int32_t out_dtype, hipStream_t stream) {
  if (!dtype_ok(out_dtype)) return MLA_ERR_UNSUPPORTED;
  if (n < 0 || R < 1 || R > 8192 || !(eps >= 0.0f) || !isfinite(eps)) return MLA_ERR_SHAPE;
  if ((int64_t)n * R > kMaxElems) return MLA_ERR_SHAPE;
  if (n == 0) return MLA_OK;
  if (!x || !w || !y) return MLA_ERR_NULL;
  clear_stale_error();
  return hip_status(mla::launch_rmsnorm(x, w, eps, y, n, R, out_dtype, stream));
}

mla_status mla_kv_expand(const uint16_t* c_norm, const mla_bf16* W, int32_t B, int32_t T, int32_t R, int32_t H,
                         int32_t Dn, int32_t Dv, uint16_t* k, int32_t k_ld, uint16_t* v, int32_t v_layout,
                         int32_t v_ld, int32_t Tcap, int32_t t_off, int32_t kv_dtype, const mla_bf16* k_pe,
                         const float* cos, const float* sin, int32_t table_len, const int32_t* pos, int32_t Dr,
                         int32_t pairing, hipStream_t stream) {
  if (!dtype_ok(kv_dtype)) return MLA_ERR_UNSUPPORTED;
  if (v_layout != MLA_V_ROWS && v_layout != MLA_V_COLS) return MLA_ERR_SHAPE;
  if (B < 0 || T < 0) return MLA_ERR_SHAPE;
  if ((int64_t)B * T == 0) return MLA_OK;
  if (!c_norm || !W || !k || !v) return MLA_ERR_NULL;
  if (B < 0 || T < 0 || H < 1 || R < 8 || R > 4096 || (R % 8)) return MLA_ERR_SHAPE;
  if (Dn < 8 || Dn > 512 || (Dn % 8) || Dv < 8 || Dv > 512 || (Dv % 8)) return MLA_ERR_SHAPE;
  if (Tcap < 1 || t_off < 0 || (int64_t)t_off + T > Tcap) return MLA_ERR_SHAPE;
  if (k_ld < Dn || (k_ld % 8)) return MLA_ERR_SHAPE;
  if ((int64_t)B * T > ((int64_t)1 << 30) || (int64_t)H * (Dn + Dv) > ((int64_t)1 << 30)) return MLA_ERR_SHAPE;
  if ((int64_t)B * H * Tcap * (int64_t)(k_ld > Dv ? k_ld : Dv) > kMaxElems) return MLA_ERR_SHAPE;
  if (v_layout == MLA_V_COLS && (v_ld < Tcap || (v_ld % 8) || (int64_t)B * H * Dv * v_ld > kMaxElems))
    return MLA_ERR_SHAPE;
  if (!aligned16(c_norm) || !aligned16(W) || !aligned16(k) || !aligned16(v)) return MLA_ERR_SHAPE;
  const bool append = k_pe != nullptr;
  if (append) {
    if (!cos || !sin) return MLA_ERR_NULL;
    if (!pairing_ok(pairing)) return MLA_ERR_ROPE_TYPE;
    if (Dr < 2 || (Dr & 1) || Dr > 256 || k_ld < Dn + Dr || table_len < 1) return MLA_ERR_SHAPE;
    if (!pos && t_off + T > table_len) return MLA_ERR_SHAPE;
  }
  mla::ExpandArgs a{c_norm, W, k, v, B, T, R, H, Dn, Dv, k_ld, Tcap, t_off, kv_dtype, v_layout == MLA_V_COLS,
                    v_layout == MLA_V_COLS ? v_ld : 0};
  clear_stale_error();
  hipError_t e = mla::launch_kv_expand(a, stream);
  if (e != hipSuccess) return MLA_ERR_HIP;
  if (append) {
    mla::RotKeyArgs r{k_pe, cos, sin, table_len, pos, k, B, T, H, Dr, Tcap, t_off, k_ld, Dn, pairing, kv_dtype};
    e = mla::launch_rotate_key(r, stream);
  }
  return hip_status(e);
}

static size_t round256(size_t n) { return (n + 255) / 256 * 256; }

// Workspace of the prefill: the rotated shared rotary key [B, T, Dr], then
// (row-major values only) their transposed copy [B, H, Dv, round8(T)].
static size_t prefill_ws(int32_t B, int32_t H, int32_t T, int32_t Dr, int32_t Dv, int32_t v_layout) {
  size_t n = round256((size_t)B * T * Dr * sizeof(uint16_t));
  if (v_layout == MLA_V_ROWS) n += round256((size_t)B * H * Dv * (size_t)((T + 7) / 8 * 8) * sizeof(uint16_t));
  return n;
}

mla_status mla_prefill_attention(const mla_bf16* q, const uint16_t* k_nope, const mla_bf16* k_pe, const uint16_t* v,
                                 int32_t v_layout, int32_t v_ld, int32_t kv_dtype, const float* cos,
                                 const float* sin, int32_t table_len, const int32_t* pos, int32_t B, int32_t H,
                                 int32_t T, int32_t Dn, int32_t Dr, int32_t Dv, float scale, int32_t pairing,
                                 mla_bf16* out, float* lse, void* workspace, size_t* ws_bytes, hipStream_t stream) {
  if (B < 0 || H < 1 || T < 0 || Dn < 1 || Dr < 2 || (Dr & 1) || Dv < 1) return MLA_ERR_SHAPE;
  if (v_layout != MLA_V_ROWS && v_layout != MLA_V_COLS) return MLA_ERR_SHAPE;
  // fp16 intermediates only: with bf16 keys, values and P the path's error
  // reaches the 2e-2 bound it is held to
  if (!mla::prefill_supported(Dn + Dr, Dr, Dv) || kv_dtype != MLA_DTYPE_FP16) return MLA_ERR_UNSUPPORTED;
  if (!pairing_ok(pairing)) return MLA_ERR_ROPE_TYPE;
  if ((int64_t)B * H * T * (Dn + Dr) > kMaxElems || (int64_t)B * H > ((int64_t)1 << 24) ||
      (int64_t)T > ((int64_t)1 << 26))
    return MLA_ERR_SHAPE;
  const int32_t Tv = v_layout == MLA_V_COLS ? v_ld : (T + 7) / 8 * 8;
  if (v_layout == MLA_V_COLS && (v_ld < T || (v_ld % 8))) return MLA_ERR_SHAPE;
  // one (b, h) slice of every operand is addressed with 32-bit byte offsets
  if ((int64_t)T * (Dn > Dv ? Dn : Dv) * 2 > 0x7fffffff || (int64_t)Dv * Tv * 2 > 0x7fffffff) return MLA_ERR_SHAPE;
  const size_t need = prefill_ws(B, H, T, Dr, Dv, v_layout);
  if (!workspace && ws_bytes) {
    *ws_bytes = need;
    return MLA_OK;
  }
  if (!(scale > 0.0f) || !isfinite(scale)) return MLA_ERR_SHAPE;
  if ((int64_t)B * T == 0) return MLA_OK;
  if (!q || !k_nope || !k_pe || !v || !cos || !sin || !out) return MLA_ERR_NULL;
  if (table_len < 1 || (!pos && T > table_len)) return MLA_ERR_SHAPE;
  if (!workspace || (ws_bytes && *ws_bytes < need)) return MLA_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k_nope) || !aligned16(k_pe) || !aligned16(v) || !aligned16(out) ||
      !aligned16(workspace))
    return MLA_ERR_SHAPE;
  uint16_t* k_rot = static_cast<uint16_t*>(workspace);
  clear_stale_error();
  mla::RotKeyArgs r{k_pe, cos, sin, table_len, pos, k_rot, B, T, 1, Dr, T, 0, Dr, 0, pairing, kv_dtype};
  hipError_t e = mla::launch_rotate_key(r, stream);
  if (e != hipSuccess) return MLA_ERR_HIP;
  const uint16_t* vt = v;
  if (v_layout == MLA_V_ROWS) {
    uint16_t* vt_ws = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) +
                                                  round256((size_t)B * T * Dr * sizeof(uint16_t)));
    e = mla::launch_transpose_v(v, vt_ws, B * H, T, Dv, Tv, stream);
    if (e != hipSuccess) return MLA_ERR_HIP;
    vt = vt_ws;
  }
  mla::PrefillArgs a{q, k_nope, k_rot, vt, cos, sin, table_len, pos, out, lse, B, H, T, Dn, Dr, Dv, pairing, scale,
                     kv_dtype, Tv, 0, T};
  return hip_status(mla::launch_prefill(a, stream));
}

mla_status mla_rotate_rope_key(const mla_bf16* k_pe, const float* cos, const float* sin, int32_t table_len,
                               const int32_t* pos, int32_t B, int32_t T, int32_t Dr, int32_t pairing, uint16_t* dst,
                               int32_t Tcap, int32_t t_off, int32_t kv_dtype, hipStream_t stream) {
  if (B < 0 || T < 0 || Dr < 2 || Dr > 256 || (Dr & 1) || Tcap < 1 || t_off < 0) return MLA_ERR_SHAPE;
  if (!dtype_ok(kv_dtype)) return MLA_ERR_UNSUPPORTED;
  if (!pairing_ok(pairing)) return MLA_ERR_ROPE_TYPE;
  if ((int64_t)t_off + T > Tcap || (int64_t)B * Tcap * Dr > kMaxElems) return MLA_ERR_SHAPE;
  if ((int64_t)B * T == 0) return MLA_OK;
  if (!k_pe || !cos || !sin || !dst) return MLA_ERR_NULL;
  if (table_len < 1 || (!pos && (int64_t)t_off + T > table_len)) return MLA_ERR_SHAPE;
  clear_stale_error();
  mla::RotKeyArgs r{k_pe, cos, sin, table_len, pos, dst, B, T, 1, Dr, Tcap, t_off, Dr, 0, pairing, kv_dtype};
  return hip_status(mla::launch_rotate_key(r, stream));
}

mla_status mla_prefill_attention_cached(const mla_bf16* q, const uint16_t* k_nope, const uint16_t* k_rot,
                                        const uint16_t* vt, int32_t v_ld, int32_t kv_dtype, const float* cos,
                                        const float* sin, int32_t table_len, const int32_t* pos, int32_t B,
                                        int32_t H, int32_t T, int32_t past, int32_t Tcap, int32_t Dn, int32_t Dr,
                                        int32_t Dv, float scale, int32_t pairing, mla_bf16* out, float* lse,
                                        hipStream_t stream) {
  if (B < 0 || H < 1 || T < 0 || past < 0 || Tcap < 1 || Dn < 1 || Dr < 2 || (Dr & 1) || Dv < 1)
    return MLA_ERR_SHAPE;
  if (!mla::prefill_supported(Dn + Dr, Dr, Dv) || kv_dtype != MLA_DTYPE_FP16) return MLA_ERR_UNSUPPORTED;
  if (!pairing_ok(pairing)) return MLA_ERR_ROPE_TYPE;
  if ((int64_t)past + T > Tcap || v_ld < (int64_t)past + T || (v_ld % 8)) return MLA_ERR_SHAPE;
  if ((int64_t)B * H * Tcap * (Dn + Dr) > kMaxElems || (int64_t)B * H * T * (Dn + Dr) > kMaxElems ||
      (int64_t)B * H > ((int64_t)1 << 24) || (int64_t)Tcap > ((int64_t)1 << 26))
    return MLA_ERR_SHAPE;
  // one (b, h) slice of every operand is addressed with 32-bit byte offsets
  if ((int64_t)Tcap * (Dn > Dv ? Dn : Dv) * 2 > 0x7fffffff || (int64_t)Dv * v_ld * 2 > 0x7fffffff)
    return MLA_ERR_SHAPE;
  if (!(scale > 0.0f) || !isfinite(scale)) return MLA_ERR_SHAPE;
  if ((int64_t)B * T == 0) return MLA_OK;
  if (!q || !k_nope || !k_rot || !vt || !cos || !sin || !out) return MLA_ERR_NULL;
  if (table_len < 1 || (!pos && (int64_t)past + T > table_len)) return MLA_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k_nope) || !aligned16(k_rot) || !aligned16(vt) || !aligned16(out))
    return MLA_ERR_SHAPE;
  clear_stale_error();
  mla::PrefillArgs a{q, k_nope, k_rot, vt, cos, sin, table_len, pos, out, lse, B, H, T, Dn, Dr, Dv, pairing, scale,
                     kv_dtype, v_ld, past, Tcap};
  return hip_status(mla::launch_prefill(a, stream));
}

namespace {
// Argument checks shared by the two decode entry points; on MLA_OK, *S and
// *need hold the split count and the bytes of split partials it needs.
mla_status decode_check(const mla_bf16* q, const uint16_t* k_cache, const uint16_t* v_cache, int32_t cache_dtype,
                        const int32_t* seq_len, const int32_t* q_pos, const float* cos, const float* sin,
                        int32_t table_len, int32_t B, int32_t H, int32_t Tcap, int32_t Dn, int32_t Dr, int32_t Dv,
                        float scale, int32_t pairing, int32_t num_splits, const mla_bf16* out, int* S,
                        size_t* need, bool* query_only, bool ws_query) {
  *query_only = false;
  if (B < 0 || H < 1 || Tcap < 1 || Dn < 1 || Dr < 2 || (Dr & 1) || Dv < 1) return MLA_ERR_SHAPE;
  if (!mla::decode_supported(Dn + Dr, Dv) || !dtype_ok(cache_dtype)) return MLA_ERR_UNSUPPORTED;
  if (!pairing_ok(pairing)) return MLA_ERR_ROPE_TYPE;
  if (num_splits < 0 || num_splits > 256 || num_splits > Tcap) return MLA_ERR_SHAPE;
  if ((int64_t)B * H * Tcap * (Dn + Dr) > kMaxElems || B > 65535 || H > 65535) return MLA_ERR_SHAPE;
  *S = num_splits ? num_splits : mla::decode_auto_splits(B, H, Tcap);
  *need = mla::decode_workspace_bytes(B, H, Dv, *S);
  if (ws_query) {
    *query_only = true;
    return MLA_OK;
  }
  if (!(scale > 0.0f) || !isfinite(scale)) return MLA_ERR_SHAPE;
  if (B == 0) return MLA_OK;
  if (!q || !k_cache || !v_cache || !seq_len || !q_pos || !cos || !sin || !out) return MLA_ERR_NULL;
  if (table_len < 1) return MLA_ERR_SHAPE;
  if (!aligned16(k_cache) || !aligned16(v_cache)) return MLA_ERR_SHAPE;
  return MLA_OK;
}

mla_status decode_launch(const mla_bf16* q, const uint16_t* k_cache, const uint16_t* v_cache, int32_t cache_dtype,
                         const int32_t* seq_len, const int32_t* q_pos, const float* cos, const float* sin,
                         int32_t table_len, int32_t B, int32_t H, int32_t Tcap, int32_t Dn, int32_t Dr, int32_t Dv,
                         float scale, int32_t pairing, int S, size_t need, void* workspace, mla_bf16* out,
                         hipStream_t stream) {
  float* part_o = static_cast<float*>(workspace);
  float* part_ml = nullptr;
  if (need > 0) {
    const size_t n = (size_t)B * H * S;
    part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + ((n * Dv * sizeof(float)) + 255) / 256 * 256);
  }
  mla::DecodeArgs a{q, k_cache, v_cache, seq_len, q_pos, cos, sin, table_len, B, H, Tcap, Dn, Dr, Dv, pairing, S,
                    scale, part_o, part_ml, out, cache_dtype};
  return hip_status(mla::launch_decode(a, stream));
}
}  // namespace

mla_status mla_decode_attention(const mla_bf16* q, const uint16_t* k_cache, const uint16_t* v_cache,
                                int32_t cache_dtype, const int32_t* seq_len, const int32_t* q_pos, const float* cos,
                                const float* sin, int32_t table_len, int32_t B, int32_t H, int32_t Tcap, int32_t Dn,
                                int32_t Dr, int32_t Dv, float scale, int32_t pairing, int32_t num_splits,
                                void* workspace, size_t* ws_bytes, mla_bf16* out, hipStream_t stream) {
  int S = 0;
  size_t need = 0;
  bool query_only = false;
  mla_status st = decode_check(q, k_cache, v_cache, cache_dtype, seq_len, q_pos, cos, sin, table_len, B, H, Tcap, Dn,
                               Dr, Dv, scale, pairing, num_splits, out, &S, &need, &query_only,
                               !workspace && ws_bytes);
  if (st != MLA_OK) return st;
  if (query_only) {
    *ws_bytes = need;
    return MLA_OK;
  }
  if (B == 0) return MLA_OK;
  if (need > 0 && (!workspace || (ws_bytes && *ws_bytes < need))) return MLA_ERR_WORKSPACE;
  if (need > 0 && !aligned16(workspace)) return MLA_ERR_SHAPE;
  clear_stale_error();
  return decode_launch(q, k_cache, v_cache, cache_dtype, seq_len, q_pos, cos, sin, table_len, B, H, Tcap, Dn, Dr, Dv,
                       scale, pairing, S, need, workspace, out, stream);
}

mla_status mla_decode_attention_noalloc(const mla_bf16* q, const uint16_t* k_cache, const uint16_t* v_cache,
                                        int32_t cache_dtype, const int32_t* seq_len, const int32_t* q_pos,
                                        const float* cos, const float* sin, int32_t table_len, int32_t B, int32_t H,
                                        int32_t Tcap, int32_t Dn, int32_t Dr, int32_t Dv, float scale,
                                        int32_t pairing, int32_t num_splits, mla_bf16* out, hipStream_t stream) {
  int S = 0;
  size_t need = 0;
  bool query_only = false;
  mla_status st = decode_check(q, k_cache, v_cache, cache_dtype, seq_len, q_pos, cos, sin, table_len, B, H, Tcap, Dn,
                               Dr, Dv, scale, pairing, num_splits, out, &S, &need, &query_only, false);
  if (st != MLA_OK) return st;
  if (B == 0) return MLA_OK;
  if (need > mla::kDecodeScratchBytes) return MLA_ERR_WORKSPACE;  // split partials beyond the static scratch
  void* ws = nullptr;
  clear_stale_error();
  if (need > 0 && mla::decode_scratch(&ws) != hipSuccess) return MLA_ERR_HIP;
  return decode_launch(q, k_cache, v_cache, cache_dtype, seq_len, q_pos, cos, sin, table_len, B, H, Tcap, Dn, Dr, Dv,
                       scale, pairing, S, need, ws, out, stream);
}

// ---- decode against a compressed-latent cache (absorbed form)

mla_status mla_absorb_prepare(const mla_bf16* W, int32_t H, int32_t R, int32_t Dn, int32_t Dv, mla_bf16* w_ukt,
                              hipStream_t stream) {
  if (H < 1 || H > 65535 || R < 1 || R > 8192 || Dn < 1 || Dn > 512 || Dv < 0 || Dv > 512) return MLA_ERR_SHAPE;
  if ((int64_t)H * (Dn + Dv) * R > kMaxElems) return MLA_ERR_SHAPE;
  if (!W || !w_ukt) return MLA_ERR_NULL;
  clear_stale_error();
  return hip_status(mla::launch_absorb_prepare(W, w_ukt, H, R, Dn, Dv, stream));
}

mla_status mla_latent_cache_append(const mla_bf16* latent, const mla_bf16* gain, float eps, const mla_bf16* k_pe,
                                   const float* cos, const float* sin, int32_t table_len, const int32_t* t_pos,
                                   int32_t pairing, int32_t B, int32_t R, int32_t Dr, uint16_t* cache, int32_t Lcap,
                                   hipStream_t stream) {
  if (B < 0 || R < 1 || R > 8192 || Dr < 2 || Dr > 256 || (Dr & 1) || Lcap < 1) return MLA_ERR_SHAPE;
  if (!(eps >= 0.0f) || !isfinite(eps)) return MLA_ERR_SHAPE;
  if (!pairing_ok(pairing)) return MLA_ERR_ROPE_TYPE;
  if ((int64_t)B * Lcap * (R + Dr) > kMaxElems) return MLA_ERR_SHAPE;
  if (B == 0) return MLA_OK;
  if (!latent || !gain || !k_pe || !cos || !sin || !t_pos || !cache) return MLA_ERR_NULL;
  if (table_len < 1) return MLA_ERR_SHAPE;
  clear_stale_error();
  mla::LatentAppendArgs a{latent, gain, eps, k_pe, cos, sin, table_len, t_pos, pairing, B, R, Dr, Lcap, cache};
  return hip_status(mla::launch_latent_append(a, stream));
}

namespace {
struct AbsorbedPlan {
  int S, tps;
  size_t qa_bytes, po_bytes, lse_bytes;
  size_t total() const { return qa_bytes + po_bytes + lse_bytes; }
};
// Splits over the key axis: enough workgroups for the chip (about 256)
// when the batch is small, each split a whole number of 64-key tiles.
AbsorbedPlan absorbed_plan(int32_t B, int32_t H, int32_t Lcap, int32_t num_splits) {
  AbsorbedPlan p{};
  const int tiles = (Lcap + 63) / 64;
  int S = num_splits;
  if (S == 0) {
    const int64_t groups = (int64_t)B * ((H + 63) / 64);
    S = (int)((256 + groups - 1) / (groups > 0 ? groups : 1));
  }
  S = S < 1 ? 1 : S;
  S = S > mla::kMaxLatentSplits ? mla::kMaxLatentSplits : S;
  S = S > tiles ? tiles : S;
  p.tps = (tiles + S - 1) / S;
  p.S = (tiles + p.tps - 1) / p.tps;
  p.qa_bytes = round256((size_t)B * H * (mla::kLatentR + mla::kLatentDr) * 2);
  p.po_bytes = round256((size_t)B * p.S * H * mla::kLatentR * 2);
  p.lse_bytes = round256((size_t)B * p.S * H * 4);
  return p;
}
}  // namespace

mla_status mla_decode_absorbed(const mla_bf16* q, const mla_bf16* W, const mla_bf16* w_ukt, const uint16_t* cache,
                               const int32_t* seq_len, const int32_t* q_pos, const float* cos, const float* sin,
                               int32_t table_len, int32_t B, int32_t H, int32_t Lcap, int32_t R, int32_t Dn,
                               int32_t Dr, int32_t Dv, float scale, int32_t pairing, int32_t num_splits,
                               void* workspace, size_t* ws_bytes, mla_bf16* out, hipStream_t stream) {
  if (B < 0 || B > 65535 || H < 1 || H > 65535 || Lcap < 1) return MLA_ERR_SHAPE;
  if (R != mla::kLatentR || Dr != mla::kLatentDr) return MLA_ERR_UNSUPPORTED;
  if (Dn < 16 || Dn > 512 || (Dn % 16) || Dv < 32 || Dv > 512 || (Dv % 32)) return MLA_ERR_UNSUPPORTED;
  if (!pairing_ok(pairing)) return MLA_ERR_ROPE_TYPE;
  if (num_splits < 0 || num_splits > mla::kMaxLatentSplits) return MLA_ERR_SHAPE;
  if ((int64_t)Lcap * (R + Dr) * 2 >= ((int64_t)1 << 31)) return MLA_ERR_SHAPE;  // one sequence's cache < 2 GiB
  if ((int64_t)B * Lcap * (R + Dr) > kMaxElems || (int64_t)B * H * R > kMaxElems) return MLA_ERR_SHAPE;
  const AbsorbedPlan plan = absorbed_plan(B, H, Lcap, num_splits);
  const size_t need = plan.total();
  if (!workspace && ws_bytes) {
    *ws_bytes = need;
    return MLA_OK;
  }
  if (!(scale > 0.0f) || !isfinite(scale)) return MLA_ERR_SHAPE;
  if (B == 0) return MLA_OK;
  if (!q || !W || !w_ukt || !cache || !seq_len || !q_pos || !cos || !sin || !out) return MLA_ERR_NULL;
  if (table_len < 1) return MLA_ERR_SHAPE;
  if (!workspace || (ws_bytes && *ws_bytes < need)) return MLA_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(W) || !aligned16(w_ukt) || !aligned16(cache) || !aligned16(workspace))
    return MLA_ERR_SHAPE;
  char* ws = static_cast<char*>(workspace);
  uint16_t* qa = reinterpret_cast<uint16_t*>(ws);
  uint16_t* part_o = reinterpret_cast<uint16_t*>(ws + plan.qa_bytes);
  float* part_lse = reinterpret_cast<float*>(ws + plan.qa_bytes + plan.po_bytes);
  clear_stale_error();
  const float kLog2e = 1.4426950408889634f;
  mla::AbsorbArgs aa{q, w_ukt, q_pos, cos, sin, table_len, B, H, Dn, Dr, pairing, scale * kLog2e, qa};
  hipError_t e = mla::launch_absorb_q(aa, stream);
  if (e != hipSuccess) return MLA_ERR_HIP;
  mla::LatentAttnArgs la{qa, cache, seq_len, part_o, part_lse, B, H, Lcap, plan.S, plan.tps};
  e = mla::launch_latent_attn(la, stream);
  if (e != hipSuccess) return MLA_ERR_HIP;
  mla::CombineUnabsorbArgs cu{part_o, part_lse, W, out, B, H, plan.S, Dn, Dv};
  return hip_status(mla::launch_combine_unabsorb(cu, stream));
}

mla_status mla_decode_latent_expanded(const mla_bf16* q, const mla_bf16* W, const uint16_t* cache,
                                      const int32_t* seq_len, const int32_t* q_pos, const float* cos,
                                      const float* sin, int32_t table_len, int32_t B, int32_t H, int32_t Lcap,
                                      int32_t R, int32_t Dn, int32_t Dr, int32_t Dv, float scale, int32_t pairing,
                                      int32_t num_splits, void* workspace, size_t* ws_bytes, mla_bf16* out,
                                      hipStream_t stream) {
  if (B < 0 || B > 65535 || H < 1 || H > 65535 || Lcap < 1) return MLA_ERR_SHAPE;
  if (R < 8 || R > 4096 || (R % 8) || Dr < 8 || Dr > 256 || (Dr % 8)) return MLA_ERR_SHAPE;
  if (!mla::decode_supported(Dn + Dr, Dv)) return MLA_ERR_UNSUPPORTED;
  if (Dn < 8 || (Dn % 8) || Dv < 8 || (Dv % 8)) return MLA_ERR_SHAPE;
  if (!pairing_ok(pairing)) return MLA_ERR_ROPE_TYPE;
  if (num_splits < 0 || num_splits > 256 || num_splits > Lcap) return MLA_ERR_SHAPE;
  if ((int64_t)B * H * Lcap * (Dn + Dr + Dv) > kMaxElems || (int64_t)B * Lcap > ((int64_t)1 << 30)) return MLA_ERR_SHAPE;
  if ((int64_t)H * (Dn + Dv) > ((int64_t)1 << 30)) return MLA_ERR_SHAPE;
  const int S = num_splits ? num_splits : mla::decode_auto_splits(B, H, Lcap);
  const size_t c_bytes = round256((size_t)B * Lcap * R * 2);
  const size_t k_bytes = round256((size_t)B * H * Lcap * (Dn + Dr) * 2);
  const size_t v_bytes = round256((size_t)B * H * Lcap * Dv * 2);
  const size_t need = c_bytes + k_bytes + v_bytes + mla::decode_workspace_bytes(B, H, Dv, S);
  if (!workspace && ws_bytes) {
    *ws_bytes = need;
    return MLA_OK;
  }
  if (!(scale > 0.0f) || !isfinite(scale)) return MLA_ERR_SHAPE;
  if (B == 0) return MLA_OK;
  if (!q || !W || !cache || !seq_len || !q_pos || !cos || !sin || !out) return MLA_ERR_NULL;
  if (table_len < 1) return MLA_ERR_SHAPE;
  if (!workspace || (ws_bytes && *ws_bytes < need)) return MLA_ERR_WORKSPACE;
  if (!aligned16(W) || !aligned16(cache) || !aligned16(workspace)) return MLA_ERR_SHAPE;
  char* ws = static_cast<char*>(workspace);
  uint16_t* c = reinterpret_cast<uint16_t*>(ws);
  uint16_t* k = reinterpret_cast<uint16_t*>(ws + c_bytes);
  uint16_t* v = reinterpret_cast<uint16_t*>(ws + c_bytes + k_bytes);
  float* part_o = reinterpret_cast<float*>(ws + c_bytes + k_bytes + v_bytes);
  float* part_ml = nullptr;
  if (S > 1) {
    const size_t n = (size_t)B * H * S;
    part_ml = reinterpret_cast<float*>(reinterpret_cast<char*>(part_o) + round256(n * Dv * sizeof(float)));
  }
  clear_stale_error();
  hipError_t e = mla::launch_latent_reexpand_copies(cache, c, k, B, H, Lcap, R, Dr, Dn, stream);
  if (e != hipSuccess) return MLA_ERR_HIP;
  // every cached latent row expanded into the per-head key (columns 0..Dn)
  // and value caches: one prefill-size expansion per call
  mla::ExpandArgs xa{c, W, k, v, B, Lcap, R, H, Dn, Dv, Dn + Dr, Lcap, 0, MLA_DTYPE_FP16, 0, 0};
  e = mla::launch_kv_expand(xa, stream);
  if (e != hipSuccess) return MLA_ERR_HIP;
  mla::DecodeArgs da{q, k, v, seq_len, q_pos, cos, sin, table_len, B, H, Lcap, Dn, Dr, Dv, pairing, S,
                     scale, part_o, part_ml, out, MLA_DTYPE_FP16};
  return hip_status(mla::launch_decode(da, stream));
}

mla_status mla_linear(const mla_bf16* x, int32_t x_layout, int32_t x_T, int32_t x_D, const mla_bf16* w,
                      const mla_bf16* bias, int32_t M, int32_t N, int32_t K, mla_bf16* y0, mla_bf16* y1,
                      int32_t y_layout, int32_t y_T, int32_t y_D, int32_t y_split, hipStream_t stream) {
  if (M < 0 || N < 8 || (N % 8) || K < 64 || (K % 64)) return MLA_ERR_SHAPE;
  // byte offsets into X, W and Y are 32-bit
  if ((int64_t)M * K >= ((int64_t)1 << 31) || (int64_t)N * K >= ((int64_t)1 << 31) ||
      (int64_t)M * N >= ((int64_t)1 << 31))
    return MLA_ERR_SHAPE;
  int dlog2 = 0;
  if (x_layout == MLA_LIN_HEADS) {
    if (x_D < 8 || x_D > 4096 || (x_D & (x_D - 1)) || (K % x_D) || x_T < 1 || (M % x_T)) return MLA_ERR_SHAPE;
    while ((1 << dlog2) < x_D) ++dlog2;
  } else if (x_layout != MLA_LIN_ROWS) {
    return MLA_ERR_SHAPE;
  }
  if (y_layout == MLA_LIN_HEADS) {
    if (y_D < 8 || (y_D % 8) || (N % y_D) || y_T < 1 || (M % y_T)) return MLA_ERR_SHAPE;
  } else if (y_layout == MLA_LIN_SPLIT) {
    if (y_split < 8 || y_split >= N || (y_split % 8)) return MLA_ERR_SHAPE;
  } else if (y_layout != MLA_LIN_ROWS) {
    return MLA_ERR_SHAPE;
  }
  if (M == 0) return MLA_OK;
  if (!x || !w || !y0 || (y_layout == MLA_LIN_SPLIT && !y1)) return MLA_ERR_NULL;
  if (!aligned16(x) || !aligned16(w) || !aligned16(y0) || (y1 && !aligned16(y1))) return MLA_ERR_SHAPE;
  if (bias && (((uintptr_t)bias) & 7)) return MLA_ERR_SHAPE;
  clear_stale_error();
  mla::LinearArgs a{x, w, bias, y0, y1, M, N, K, x_layout == MLA_LIN_HEADS ? 1 : 0, x_T, dlog2, y_layout, y_T, y_D,
                    y_split};
  return hip_status(mla::launch_linear(a, stream));
}

}  // extern "C"
