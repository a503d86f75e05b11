/*
 * mla.h - C ABI of the MI355X (gfx950) eager multi-head latent attention
 * forward path: latent RMSNorm -> kv_b_proj expansion -> rotary embedding
 * (default or YaRN) -> causal scaled softmax attention, plus a decode step
 * against an expanded per-head KV cache and one against a compressed-latent
 * cache (absorbed form).
 *
 * Pages cited below:
 *   [eq]        equation page "Read the equation" and its "Original context":
 *               kv = kv_b_proj(kv_a_layernorm(compressed_kv)) viewed into
 *               heads and split into non-rotary key and value.
 *   [K2-query]  Kimi-K2 "Query content heads", sections "Split content
 *               heads" and "Join query parts": query split, rotation of the
 *               rotary parts, nope|rope concatenation, scaled scores, causal
 *               mask, fp32 softmax, value mix, expanded-cache update.
 *   [K2-rope]   Kimi-K2 "RoPE coefficients", section "Generate RoPE
 *               coefficients": YaRN correction range, linear ramp, mscale
 *               ratio, cos/sin cache, class defaults, softmax-scale rule and
 *               the RoPE-type dispatch.
 *   [GLM-kv]    GLM-5 "Normalized key-value latent", sections "Key-value
 *               compression" and "KV cache": latent RMSNorm with default
 *               epsilon 1e-6, kv_b_proj shape, expand_kv, shared rotary key
 *               broadcast to every head, interleaved rotary variant; the
 *               cache keeps the normalised latent and the rotated rotary
 *               key per token and re-expands them on every call.
 *
 * Interface notes (the shapes and scale rules are the pages'; these are the
 * choices made around them, each stated again at its call):
 *   - intermediates in fp16, not the model dtype: the normalised latent
 *     (mla_latent_rmsnorm, mla_latent_prepare), the expanded keys and values
 *     and the attention operands, for three more significant bits at the same
 *     size and MFMA rate (bf16 keys/values remain selectable where the
 *     result stays within bounds: expansion and decode caches);
 *   - values may be handed over transposed (V^T, MLA_V_COLS), the layout the
 *     P.V product reads; the pages' row layout is accepted and transposed;
 *   - every call that reads the cos/sin table takes its length (table_len),
 *     so that device-side positions can be clamped into it;
 *   - calls that need scratch memory take a caller workspace (query its size
 *     with workspace == NULL), except mla_decode_attention_noalloc;
 *   - mla_rope_table_build returns the softmax-scale multiplier in double,
 *     as the host computes it.
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE memory owned by the caller; the library
 *     never allocates, frees or retains them and keeps no global state.
 *   - bf16 tensors are passed as uint16_t bit patterns (bfloat16, round to
 *     nearest even on every write). All layouts are dense row-major in the
 *     order written in brackets, innermost dimension last.
 *   - Calls are asynchronous on `stream` (0 = the null stream). The return
 *     value reports argument validation (checked on the host before any
 *     device work is queued; nothing is launched on error) and launch errors
 *     (MLA_ERR_HIP). Faults during execution surface at the caller's
 *     synchronisation, as with any HIP kernel.
 *   - Positions read from device arrays are not visible to the host; a
 *     position outside [0, table_len) is clamped to the table for memory
 *     safety and its result is unspecified.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t mla_bf16; /* bfloat16 bit pattern */

typedef enum {
  MLA_OK = 0,
  MLA_ERR_NULL = -1,        /* a required pointer is NULL */
  MLA_ERR_SHAPE = -2,       /* sizes inconsistent or out of range */
  MLA_ERR_UNSUPPORTED = -3, /* head dimensions without a compiled kernel */
  MLA_ERR_ROPE_TYPE = -4,   /* unknown rotary type or pairing */
  MLA_ERR_WORKSPACE = -5,   /* workspace missing or smaller than required */
  MLA_ERR_HIP = -6          /* a HIP launch or API call failed */
} mla_status;

/* Rotary types of the RoPE dispatch [K2-rope]: no scaling -> plain rotary
 * embedding; "yarn" -> YaRN. Linear and dynamic-NTK scaling are named on the
 * page without their formulas and are not provided. */
typedef enum { MLA_ROPE_DEFAULT = 0, MLA_ROPE_YARN = 1 } mla_rope_type;

/* Which elements of the rotary part form a rotated pair. HALF: pair i is
 * (x[i], x[i + Dr/2]) (the rotate-half form matching the page's duplicated
 * cos/sin halves, used by the Kimi-K2 call [K2-query]); INTERLEAVED: pair i
 * is (x[2i], x[2i+1]) (GLM-5 calls an interleaved variant [GLM-kv]). Each
 * pair (a, b) becomes (a*cos - b*sin, b*cos + a*sin); element order is
 * unchanged. */
typedef enum { MLA_PAIR_HALF = 0, MLA_PAIR_INTERLEAVED = 1 } mla_rope_pairing;

/* Element type of the expanded keys and values (k_nope, v, the KV cache) and
 * of the attention MFMA operands. The pages keep them in the model dtype
 * (bf16). FP16 has the same size and MFMA rate on gfx950 and three more
 * significant bits, which keeps the whole path inside its error budget; it
 * requires |values| < 65504: a larger key or value becomes inf in the fp16
 * expansion, and the attention outputs that touch it (and the other rows of
 * its 64-key tile, through the zero weight of a masked key times inf) come
 * out inf or NaN, never finite and wrong. The same bound holds for the
 * normalised latent (fp16) and for the query times scale * log2(e).
 * Queries, rotary keys and outputs stay bf16 at the boundary. */
typedef enum { MLA_DTYPE_BF16 = 0, MLA_DTYPE_FP16 = 1 } mla_dtype;

/* Layout of the expanded values. ROWS: [B, H, T, Dv], the layout the pages
 * produce (transpose(1, 2) of the projection, split off after the keys).
 * COLS: V^T [B, H, Dv, v_ld], keys contiguous per value column, with a row
 * stride v_ld that is a multiple of 8 and >= the token count; the padding
 * columns must hold finite values (mla_kv_expand writes zeros there). The
 * prefill attention multiplies P by V with keys as the reduction dimension,
 * so it reads V^T directly; given ROWS it first transposes into its
 * workspace. */
typedef enum { MLA_V_ROWS = 0, MLA_V_COLS = 1 } mla_v_layout;
typedef enum { MLA_LIN_ROWS = 0, MLA_LIN_HEADS = 1, MLA_LIN_SPLIT = 2 } mla_linear_layout;

/* Rotary parameters [K2-rope, YaRN class and rope_scaling keys]. The YaRN
 * class defaults printed on the page are base 10000, factor 1.0,
 * original_max_pos 4096, beta_fast 32, beta_slow 1, mscale 1,
 * mscale_all_dim 0. Fields other than rope_dim and base are ignored for
 * MLA_ROPE_DEFAULT. */
typedef struct {
  int32_t rope_dim;         /* Dr: rotary width, even, 2..256 */
  int32_t type;             /* mla_rope_type */
  double base;              /* rope_theta, > 1 */
  double factor;            /* YaRN scaling factor (> 0) */
  int32_t original_max_pos; /* YaRN original_max_position_embeddings (> 0) */
  double beta_fast;         /* YaRN beta_fast (> 0) */
  double beta_slow;         /* YaRN beta_slow (> 0) */
  double mscale;            /* YaRN mscale */
  double mscale_all_dim;    /* YaRN mscale_all_dim */
} mla_rope_params;

/* Build the cos/sin table [K2-rope, _set_cos_sin_cache].
 *   inv_freq_i = base^(-2i/Dr) for default RoPE; for YaRN, the blend of
 *   base^(-2i/Dr) (below the correction band) and base^(-2i/Dr)/factor (above
 *   it) by the linear ramp over [low, high], where low/high are the floor and
 *   ceiling of the correction dims of beta_fast/beta_slow clamped to
 *   [0, Dr-1] (widened by 0.001 when equal).
 *   m = mscale(factor, mscale) / mscale(factor, mscale_all_dim) for YaRN
 *   (mscale(s, u) = 1 if s <= 1 else 0.1*u*ln(s) + 1), 1 for default.
 *   cos_out[p, i] = m*cos(p*inv_freq_i), sin_out[p, i] = m*sin(p*inv_freq_i)
 *   for p in [0, n_pos), i in [0, Dr/2).
 * The correction range is computed on the host in double (as the page does
 * with Python floats); ramp, frequencies, angles and sin/cos in fp32 on the
 * device. The page's duplicated second half (cat(freqs, freqs)) is not
 * stored.
 * Args: p (host), n_pos >= 1, cos_out/sin_out device fp32 [n_pos, Dr/2].
 *   attn_mscale2 (host, may be NULL) receives mscale(factor, mscale_all_dim)^2
 *   if YaRN and mscale_all_dim != 0, else 1: the softmax-scale multiplier.
 * Errors: MLA_ERR_NULL, MLA_ERR_SHAPE (n_pos < 1, Dr odd/out of range, bad
 *   YaRN numbers), MLA_ERR_ROPE_TYPE (unknown type), MLA_ERR_HIP. */
mla_status mla_rope_table_build(const mla_rope_params* p, int32_t n_pos, float* cos_out,
                                float* sin_out, double* attn_mscale2, hipStream_t stream);

/* Softmax scale rule (host only, no device work) [K2-rope model-args text;
 * GLM-kv yarn_apply_mscale]: qk_head_dim^-0.5, times
 * mscale(factor, mscale_all_dim)^2 when the rotary type is YaRN and
 * mscale_all_dim != 0. Errors: MLA_ERR_NULL, MLA_ERR_SHAPE
 * (qk_head_dim < 1), MLA_ERR_ROPE_TYPE. */
mla_status mla_softmax_scale(const mla_rope_params* p, int32_t qk_head_dim, double* scale_out);

/* Latent RMSNorm [eq; GLM-kv: kv_a_layernorm built without epsilon, i.e.
 * 1e-6]: y[r, :] = w * x[r, :] / sqrt(mean(x[r, :]^2) + eps), computed in
 * fp32 and written in fp16 (one round-to-nearest-even per element; values
 * must stay below 65504 in magnitude). fp16 rather than the model dtype bf16:
 * kv_b_proj multiplies the latent on fp16 MFMA, and fp16's 11 significant
 * bits keep its rounding at the level of the fp16 keys and values, where
 * bf16's 8 would be the largest single error of the whole path.
 * Args: x device bf16 [n, R]; w device bf16 [R]; eps >= 0; y device fp16
 *   [n, R]; n >= 0 rows (0 is a no-op); 1 <= R <= 8192.
 * Errors: MLA_ERR_NULL, MLA_ERR_SHAPE, MLA_ERR_HIP. */
mla_status mla_latent_rmsnorm(const mla_bf16* x, const mla_bf16* w, float eps, uint16_t* y, int32_t n,
                              int32_t R, hipStream_t stream);

/* The latent RMSNorm and the rotation of the shared rotary key in one pass
 * over the tokens [eq; GLM-kv "Key-value compression"; K2-query "Join query
 * parts": the rotary key is rotated at its position, once per token, and
 * shared by all heads]:
 *   c_norm[b, t, :] = mla_latent_rmsnorm of latent[b, t, :] (fp16 out)
 *   k_rot[b, t, :]  = rot(k_pe[b, t, :], pos[b, t]) (pos NULL = t), fp16
 * k_rot is the rotated-key operand of mla_prefill_attention_cached (with
 * past = 0 and Tcap = T, the whole prefill), so the attention needs no
 * rotation pass of its own.
 * Args: latent device bf16 [B, T, R] (R a multiple of 8, 8..4096); gain
 *   device bf16 [R]; eps >= 0; k_pe device bf16 [B, T, Dr] (Dr even,
 *   2..256); cos/sin device fp32 [table_len, Dr/2]; pos device int32
 *   [B, T] or NULL (then table_len >= T); c_norm device fp16 [B, T, R];
 *   k_rot device fp16 [B, T, Dr]. latent, gain and c_norm 16-byte aligned.
 *   B*T == 0 is a no-op.
 * Errors: MLA_ERR_NULL, MLA_ERR_SHAPE, MLA_ERR_ROPE_TYPE, MLA_ERR_HIP. */
mla_status mla_latent_prepare(const mla_bf16* latent, const mla_bf16* gain, float eps,
                              const mla_bf16* k_pe, const float* cos, const float* sin,
                              int32_t table_len, const int32_t* pos, int32_t B, int32_t T,
                              int32_t R, int32_t Dr, int32_t pairing, uint16_t* c_norm,
                              uint16_t* k_rot, hipStream_t stream);

/* kv_b_proj up-projection and head split [eq; GLM-kv expand_kv]:
 *   kv[b, t, :] = c_norm[b, t, :] . W^T, viewed [H, Dn+Dv]; for each head h
 *   k[b, h, t_off + t, 0:Dn]  = kv[b, t, h*(Dn+Dv) + 0 .. Dn)
 *   v[b, h, t_off + t, 0:Dv]  = kv[b, t, h*(Dn+Dv) + Dn .. Dn+Dv)
 * fp16 MFMA with fp32 accumulation, one RNE rounding per output to kv_dtype.
 * W (bf16) is widened to fp16, exact for every bf16 value of magnitude at
 * least 2^-24 (smaller ones round to fp16 subnormals or zero, far below the
 * fp32 resolution of the sums).
 * Append mode (k_pe != NULL), the expanded-cache update of a decode step
 * [K2-query]: additionally the shared rotary key of token (b, t) is rotated
 * at position pos[b*T + t] (or t_off + t when pos is NULL) with the table
 * and written to k[b, h, t_off + t, Dn : Dn+Dr] for every head h.
 * Args: c_norm device fp16 [B, T, R] (from mla_latent_rmsnorm); W device
 *   bf16 [H*(Dn+Dv), R]
 *   (nn.Linear weight layout); k device [B, H, Tcap, k_ld] and v device
 *   [B, H, Tcap, Dv] (v_layout MLA_V_ROWS, v_ld ignored) or V^T
 *   [B, H, Dv, v_ld] (MLA_V_COLS, v_ld >= Tcap and a multiple of 8; the call
 *   that writes column Tcap-1 also zeroes columns Tcap..v_ld-1), both of
 *   element type kv_dtype (mla_dtype);
 *   0 <= t_off, t_off + T <= Tcap;
 *   k_ld >= Dn (>= Dn+Dr in append mode). Append mode only: k_pe device bf16
 *   [B, T, Dr] (not rotated), cos/sin device fp32 [table_len, Dr/2] from
 *   mla_rope_table_build, pos device int32 [B, T] or NULL, pairing.
 *   Dn, Dv multiples of 8 in [8, 512]; R multiple of 8 in [8, 4096];
 *   B*T == 0 is a no-op.
 * Errors: MLA_ERR_NULL, MLA_ERR_SHAPE, MLA_ERR_ROPE_TYPE (pairing),
 *   MLA_ERR_UNSUPPORTED (kv_dtype), MLA_ERR_HIP. */
mla_status mla_kv_expand(const uint16_t* c_norm, const mla_bf16* W, int32_t B, int32_t T,
                         int32_t R, int32_t H, int32_t Dn, int32_t Dv, uint16_t* k, int32_t k_ld,
                         uint16_t* v, int32_t v_layout, int32_t v_ld, int32_t Tcap, int32_t t_off,
                         int32_t kv_dtype,
                         const mla_bf16* k_pe, const float* cos, const float* sin,
                         int32_t table_len, const int32_t* pos, int32_t Dr, int32_t pairing,
                         hipStream_t stream);

/* Causal prefill attention with the rotary step and nope|rope concatenation
 * fused in [K2-query, Join query parts; GLM-kv expand_kv]:
 *   Q[b,h,t]  = [ q[b,h,t,0:Dn] | rot(q[b,h,t,Dn:Dn+Dr], pos[b,t]) ]
 *   K[b,h,s]  = [ k_nope[b,h,s,:] | rot(k_pe[b,s,:], pos[b,s]) ]  (one rotary
 *               key shared by all heads)
 *   S = scale * Q K^T, keys s > t hidden (causal), P = softmax over s in fp32,
 *   out[b,h,t,:] = P V.
 * Flash-style: S and P are never written to memory. Both products run on
 * fp16 MFMA with fp32 accumulation: the rotated query and key parts and P
 * are rounded once to fp16. kv_dtype must be MLA_DTYPE_FP16: with bf16 keys,
 * values and P the path's error reaches its 2e-2 bound (max-abs against the
 * fp64 definition), so MLA_DTYPE_BF16 returns MLA_ERR_UNSUPPORTED.
 * Args: q device bf16 [B, H, T, Dn+Dr] (rotary part not rotated);
 *   k_nope device [B, H, T, Dn] and v device of element type kv_dtype (from
 *   mla_kv_expand), v either [B, H, T, Dv] (v_layout MLA_V_ROWS, v_ld
 *   ignored; transposed into the workspace first) or V^T [B, H, Dv, v_ld]
 *   (MLA_V_COLS, v_ld >= T, a multiple of 8, padding columns finite);
 *   k_pe device bf16 [B, T, Dr] (not rotated); cos/sin device fp32
 *   [table_len, Dr/2]; pos device int32 [B, T] or NULL (= 0..T-1, which
 *   needs table_len >= T); scale from mla_softmax_scale; out device bf16
 *   [B, H, T, Dv]; lse device fp32 [B, H, T] or NULL (natural-log
 *   log-sum-exp of each row's scaled scores).
 *   workspace: device scratch of *ws_bytes bytes (the rotated rotary keys
 *   and, for MLA_V_ROWS, the transposed values). Pass workspace == NULL with
 *   ws_bytes != NULL to query the size (*ws_bytes is set, MLA_OK, nothing
 *   launched).
 *   Supported (Dn+Dr, Dv): (48, 32), (192, 128), (256, 256); Dr in
 *   {16, 64}; T >= 0 (0 is a no-op); one (b, h) slice of k_nope and of V^T
 *   below 2 GiB.
 * Errors: MLA_ERR_NULL, MLA_ERR_SHAPE, MLA_ERR_UNSUPPORTED,
 *   MLA_ERR_ROPE_TYPE, MLA_ERR_WORKSPACE, MLA_ERR_HIP. */
mla_status mla_prefill_attention(const mla_bf16* q, const uint16_t* k_nope, const mla_bf16* k_pe,
                                 const uint16_t* v, int32_t v_layout, int32_t v_ld,
                                 int32_t kv_dtype, const float* cos,
                                 const float* sin, int32_t table_len, const int32_t* pos,
                                 int32_t B, int32_t H,
                                 int32_t T, int32_t Dn, int32_t Dr, int32_t Dv, float scale,
                                 int32_t pairing, mla_bf16* out, float* lse, void* workspace,
                                 size_t* ws_bytes, hipStream_t stream);

/* Rotate rotary keys into a shared rotated-key buffer [K2-query "Join query
 * parts": the rotary key is rotated at its position; GLM-kv: one rotary key
 * per token, shared by every head]: dst[b, t_off+t, :] = rot(k_pe[b, t, :],
 * pos[b, t]) (pos NULL = t_off + t). Together with mla_kv_expand (t_off, V^T
 * layout) this appends a chunk of tokens to the cache that
 * mla_prefill_attention_cached reads.
 * Args: k_pe device bf16 [B, T, Dr] (not rotated); cos/sin device fp32
 *   [table_len, Dr/2]; pos device int32 [B, T] or NULL; dst device
 *   [B, Tcap, Dr] of type kv_dtype (rows t_off..t_off+T-1 written).
 *   B, T >= 0 (an empty call is a no-op); Dr even in [2, 256];
 *   t_off + T <= Tcap.
 * Errors: MLA_ERR_NULL, MLA_ERR_SHAPE, MLA_ERR_UNSUPPORTED,
 *   MLA_ERR_ROPE_TYPE, MLA_ERR_HIP. */
mla_status mla_rotate_rope_key(const mla_bf16* k_pe, const float* cos, const float* sin, int32_t table_len,
                               const int32_t* pos, int32_t B, int32_t T, int32_t Dr, int32_t pairing, uint16_t* dst,
                               int32_t Tcap, int32_t t_off, int32_t kv_dtype, hipStream_t stream);

/* Causal attention of a chunk of T new query tokens against a cache holding
 * `past` earlier tokens and the chunk itself [K2-query "Join query parts":
 * with past key values the cache is updated first and the causal mask is
 * offset by the cached length]:
 *   Q[b,h,t] = [ q[b,h,t,0:Dn] | rot(q[b,h,t,Dn:], pos[b,t]) ]  (pos NULL =
 *              past + t)
 *   K[b,h,s] = [ k_nope[b,h,s,:] | k_rot[b,s,:] ],  V[b,h,s] = V^T[b,h,:,s]
 *   S[t,s] = scale * Q[t] . K[s] for s <= past + t (rows past+t+1.. masked),
 *   P = softmax, out[b,h,t,:] = P V, lse as in mla_prefill_attention.
 * With past = 0 and Tcap = T this is mla_prefill_attention on prepared
 * operands. The cache rows 0..past+T-1 must already hold the chunk's keys
 * and values (mla_kv_expand with t_off = past, mla_rotate_rope_key).
 * Args: q device bf16 [B, H, T, Dn+Dr]; k_nope device [B, H, Tcap, Dn];
 *   k_rot device [B, Tcap, Dr] (rotated); vt device V^T [B, H, Dv, v_ld],
 *   v_ld >= past+T and a multiple of 8, columns past+T..v_ld-1 finite (a
 *   cache allocated zeroed satisfies this); all of type kv_dtype; cos/sin
 *   device fp32 [table_len, Dr/2]; out device bf16 [B, H, T, Dv]; lse device
 *   fp32 [B, H, T] or NULL. past >= 0, past + T <= Tcap; supported (Dn+Dr,
 *   Dv) as for mla_prefill_attention; one (b, h) slice of k_nope and of V^T
 *   below 2 GiB. No workspace. kv_dtype MLA_DTYPE_FP16 only, as for
 *   mla_prefill_attention (MLA_ERR_UNSUPPORTED otherwise).
 * Errors: MLA_ERR_NULL, MLA_ERR_SHAPE, MLA_ERR_UNSUPPORTED,
 *   MLA_ERR_ROPE_TYPE, MLA_ERR_HIP. */
mla_status mla_prefill_attention_cached(const mla_bf16* q, const uint16_t* k_nope, const uint16_t* k_rot,
                                        const uint16_t* vt, int32_t v_ld, int32_t kv_dtype, const float* cos,
                                        const float* sin, int32_t table_len, const int32_t* pos, int32_t B,
                                        int32_t H, int32_t T, int32_t past, int32_t Tcap, int32_t Dn, int32_t Dr,
                                        int32_t Dv, float scale, int32_t pairing, mla_bf16* out, float* lse,
                                        hipStream_t stream);

/* Decode attention of one new token per sequence against an expanded cache
 * [K2-query: expanded cache update then scaled, masked softmax attention]:
 *   Q[b,h] = [ q[b,h,0,0:Dn] | rot(q[b,h,0,Dn:], q_pos[b]) ]
 *   S[s] = scale * Q . k_cache[b,h,s,:] for s < seq_len[b] (the cache's
 *   rotary part is already rotated), P = softmax, out[b,h,0,:] = P V.
 * Split-K: the seq_len[b] rows are cut into num_splits ranges, each giving a
 * partial (max, sum, unnormalised output); a combine kernel merges them with
 * the log-sum-exp rule. The append of the new token is a separate
 * mla_kv_expand call in append mode before this one.
 * Args: q device bf16 [B, H, 1, Dn+Dr]; k_cache device [B, H, Tcap, Dn+Dr]
 *   and v_cache device [B, H, Tcap, Dv] of element type cache_dtype
 *   (mla_dtype); seq_len
 *   device int32 [B] (values clamped to [1, Tcap]); q_pos device int32 [B];
 *   cos/sin device fp32 [table_len, Dr/2]; num_splits 0 = automatic, else
 *   1..256; out device bf16 [B, H, 1, Dv]. workspace/ws_bytes as for
 *   mla_prefill_attention (size depends on B, H, Tcap, Dv and num_splits).
 *   Dn+Dr, Dv multiples of 8, Dn+Dr <= 512, Dv <= 512.
 * Errors: MLA_ERR_NULL, MLA_ERR_SHAPE, MLA_ERR_UNSUPPORTED,
 *   MLA_ERR_ROPE_TYPE, MLA_ERR_WORKSPACE, MLA_ERR_HIP. */
mla_status mla_decode_attention(const mla_bf16* q, const uint16_t* k_cache,
                                const uint16_t* v_cache, int32_t cache_dtype, const int32_t* seq_len,
                                const int32_t* q_pos, const float* cos, const float* sin,
                                int32_t table_len, int32_t B, int32_t H, int32_t Tcap, int32_t Dn,
                                int32_t Dr, int32_t Dv, float scale, int32_t pairing,
                                int32_t num_splits, void* workspace, size_t* ws_bytes,
                                mla_bf16* out, hipStream_t stream);

/* Decode attention that allocates nothing, for callers that cannot allocate
 * or bring a workspace (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). Same arguments, outputs and errors as
 * mla_decode_attention without workspace/ws_bytes: the split partials
 * (B*H*S*(Dv+2)*4 bytes, 256-byte aligned, when S > 1) go to a static device
 * array of MLA_DECODE_SCRATCH_BYTES (16 MiB) inside the library instead, one
 * per GPU, held until the process ends. A call whose partials would exceed
 * it returns MLA_ERR_WORKSPACE and queues nothing (choose fewer splits, or
 * use mla_decode_attention). Calls that overlap on one GPU (different
 * streams or host threads) share that array and race: serialise them. The
 * array's device address is looked up on the first call on each device
 * (MLA_ERR_HIP if that fails). */
#define MLA_DECODE_SCRATCH_BYTES ((size_t)16 << 20)
mla_status mla_decode_attention_noalloc(const mla_bf16* q, const uint16_t* k_cache,
                                        const uint16_t* v_cache, int32_t cache_dtype,
                                        const int32_t* seq_len, const int32_t* q_pos,
                                        const float* cos, const float* sin, int32_t table_len,
                                        int32_t B, int32_t H, int32_t Tcap, int32_t Dn, int32_t Dr,
                                        int32_t Dv, float scale, int32_t pairing,
                                        int32_t num_splits, mla_bf16* out, hipStream_t stream);

/* ---- Decode against a compressed-latent cache ---------------------------
 * Cache layout (the "latent cache"): device fp16 [B, Lcap, R+Dr], row s of
 * sequence b = [ normalised latent of token s (R values) | its rotary key
 * rotated at position s (Dr values) ] [GLM-kv, "KV cache"].
 * The output equals the expanded-cache decode with keys
 * [W_uk[h] c_s | k_s] and values W_uv[h] c_s; the absorbed evaluation
 * [eq: the absorbed path folds W_uk into the query and applies W_uv after
 * attention] never forms them. W_uk[h] / W_uv[h] are rows h*(Dn+Dv) ..
 * +Dn-1 / +Dn .. +Dn+Dv-1 of the kv_b_proj weight W [H*(Dn+Dv), R]. */

/* One-time weight preparation for mla_decode_absorbed: the key half of
 * kv_b_proj transposed per head, w_ukt[h, r, j] = W[h*(Dn+Dv) + j, r] for
 * j < Dn (bf16 copy). Args: W device bf16 [H*(Dn+Dv), R]; w_ukt device bf16
 * [H, R, Dn] (caller-owned, written). 1 <= R <= 8192, 1 <= Dn, Dv <= 512.
 * Errors: MLA_ERR_NULL, MLA_ERR_SHAPE, MLA_ERR_HIP. */
mla_status mla_absorb_prepare(const mla_bf16* W, int32_t H, int32_t R, int32_t Dn, int32_t Dv, mla_bf16* w_ukt,
                              hipStream_t stream);

/* Append the new token of each sequence to a latent cache [GLM-kv: the
 * normalised latent and the rotated key go into the cache]: row t = t_pos[b]
 * of sequence b becomes [ RMSNorm(latent[b]) with gain and eps (fp32, one
 * fp16 rounding) | k_pe[b] rotated at position t (fp16) ].
 * Args: latent device bf16 [B, R]; gain device bf16 [R]; k_pe device bf16
 * [B, Dr] (not rotated); cos/sin device fp32 [table_len, Dr/2]; t_pos
 * device int32 [B] (clamped to [0, Lcap-1] for the row and to the table for
 * the rotation); cache device fp16 [B, Lcap, R+Dr] (only the B rows are
 * written). B >= 0 (0 is a no-op), 1 <= R <= 8192, Dr even in [2, 256].
 * Errors: MLA_ERR_NULL, MLA_ERR_SHAPE, MLA_ERR_ROPE_TYPE, MLA_ERR_HIP. */
mla_status mla_latent_cache_append(const mla_bf16* latent, const mla_bf16* gain, float eps, const mla_bf16* k_pe,
                                   const float* cos, const float* sin, int32_t table_len, const int32_t* t_pos,
                                   int32_t pairing, int32_t B, int32_t R, int32_t Dr, uint16_t* cache, int32_t Lcap,
                                   hipStream_t stream);

/* Decode attention of one new token per sequence against a latent cache, by
 * the absorbed form [eq; K2-query: scaled softmax attention; GLM-kv]:
 *   q_lat[b,h] = W_uk[h]^T q[b,h,0,0:Dn]            (R values)
 *   S[s] = scale * ( q_lat . c_s + rot(q[b,h,0,Dn:], q_pos[b]) . k_s ),
 *          s < seq_len[b]
 *   out[b,h,0,:] = W_uv[h] ( sum_s softmax(S)_s c_s )
 * with (c_s | k_s) = cache[b, s]. Split-K over the key axis: each split
 * gives a normalised partial latent aggregate and its log-sum-exp, merged
 * before the W_uv product. The new token must already be in the cache
 * (mla_latent_cache_append).
 * Args: q device bf16 [B, H, 1, Dn+Dr]; W device bf16 [H*(Dn+Dv), R];
 *   w_ukt device bf16 [H, R, Dn] from mla_absorb_prepare; cache device fp16
 *   [B, Lcap, R+Dr]; seq_len device int32 [B] (clamped to [1, Lcap]); q_pos
 *   device int32 [B]; cos/sin device fp32 [table_len, Dr/2]; scale from
 *   mla_softmax_scale (of Dn+Dr); num_splits 0 = automatic, else 1..64 (at
 *   most one split per 64 cache rows is used); out device bf16 [B, H, 1, Dv].
 *   workspace/ws_bytes as for mla_prefill_attention (size depends on B, H,
 *   Lcap and the split count). Pointers to q, W, w_ukt, cache and workspace
 *   16-byte aligned.
 *   Supported: R = 512, Dr = 64, Dn a multiple of 16 in [16, 512], Dv a
 *   multiple of 32 in [32, 512]; Lcap*(R+Dr)*2 < 2^31.
 * Errors: MLA_ERR_NULL, MLA_ERR_SHAPE, MLA_ERR_UNSUPPORTED,
 *   MLA_ERR_ROPE_TYPE, MLA_ERR_WORKSPACE, MLA_ERR_HIP. */
mla_status mla_decode_absorbed(const mla_bf16* q, const mla_bf16* W, const mla_bf16* w_ukt, const uint16_t* cache,
                               const int32_t* seq_len, const int32_t* q_pos, const float* cos, const float* sin,
                               int32_t table_len, int32_t B, int32_t H, int32_t Lcap, int32_t R, int32_t Dn,
                               int32_t Dr, int32_t Dv, float scale, int32_t pairing, int32_t num_splits,
                               void* workspace, size_t* ws_bytes, mla_bf16* out, hipStream_t stream);

/* The same decode output against a latent cache by re-expansion [GLM-kv
 * "KV cache": every cached latent and rotated key come back and the key and
 * value heads are expanded from all of them on every call; expand_kv]:
 * every cache row 0..Lcap-1 is expanded by kv_b_proj into per-head fp16 keys
 * [W_uk[h] c_s | k_s] and values W_uv[h] c_s in the workspace, then the
 * expanded-cache decode attention (split-K + combine) runs over rows
 * s < seq_len[b]. Costs one prefill-size expansion of Lcap rows per call;
 * mla_decode_absorbed computes the same output without it.
 * Args: q device bf16 [B, H, 1, Dn+Dr]; W device bf16 [H*(Dn+Dv), R]; cache
 *   device fp16 [B, Lcap, R+Dr]; seq_len device int32 [B] (clamped to
 *   [1, Lcap]); q_pos device int32 [B]; cos/sin device fp32
 *   [table_len, Dr/2]; num_splits 0 = automatic, else 1..256; out device
 *   bf16 [B, H, 1, Dv]; workspace/ws_bytes as for mla_prefill_attention
 *   (about B*H*Lcap*(Dn+Dr+Dv)*2 bytes). R and Dr multiples of 8 (R <= 4096,
 *   Dr <= 256), (Dn+Dr, Dv) as for mla_decode_attention.
 * Errors: MLA_ERR_NULL, MLA_ERR_SHAPE, MLA_ERR_UNSUPPORTED,
 *   MLA_ERR_ROPE_TYPE, MLA_ERR_WORKSPACE, MLA_ERR_HIP. */
mla_status mla_decode_latent_expanded(const mla_bf16* q, const mla_bf16* W, const uint16_t* cache,
                                      const int32_t* seq_len, const int32_t* q_pos, const float* cos,
                                      const float* sin, int32_t table_len, int32_t B, int32_t H, int32_t Lcap,
                                      int32_t R, int32_t Dn, int32_t Dr, int32_t Dv, float scale, int32_t pairing,
                                      int32_t num_splits, void* workspace, size_t* ws_bytes, mla_bf16* out,
                                      hipStream_t stream);

/* RMSNorm with a choice of output type [K2-query, the MLA constructor:
 * q_a_layernorm between q_a_proj and q_b_proj; GLM-kv: RMSNorm, default
 * epsilon 1e-6]: y = w * x / sqrt(mean(x^2) + eps) per row of R values, in
 * fp32, rounded once into out_dtype (MLA_DTYPE_BF16 for the query RMSNorm,
 * whose output feeds mla_linear; mla_latent_rmsnorm is this with fp16).
 * Args: x device bf16 [n, R]; w device bf16 [R]; y device [n, R] of type
 *   out_dtype. 1 <= R <= 8192; n >= 0 (0 is a no-op).
 * Errors: MLA_ERR_NULL, MLA_ERR_SHAPE, MLA_ERR_UNSUPPORTED, MLA_ERR_HIP. */
mla_status mla_rmsnorm(const mla_bf16* x, const mla_bf16* w, float eps, uint16_t* y, int32_t n, int32_t R,
                       int32_t out_dtype, hipStream_t stream);

/* ---- Projections around the latent attention ----------------------------
 * Linear layer Y = X W^T (+ bias) [K2-query "Split content heads" and the
 * MLA constructor: q_a_proj, q_b_proj, kv_a_proj_with_mqa and o_proj are
 * nn.Linear layers (weight [out, in]); GLM-kv "Key-value compression": the
 * same layers], bf16 operands, fp32 accumulation, one bf16 rounding (after
 * the bias).
 * Layouts (mla_linear_layout):
 *   X: MLA_LIN_ROWS [M, K], or MLA_LIN_HEADS [B, K/x_D, x_T, x_D] read as
 *      the [M = B*x_T, K] matrix whose row (b, t) is head 0..K/x_D-1 of
 *      token t concatenated (the attention output feeding o_proj);
 *   Y: MLA_LIN_ROWS [M, N]; MLA_LIN_HEADS [B, N/y_D, y_T, y_D] (column n of
 *      row (b, t) goes to head n / y_D, element n % y_D: the query layout
 *      q_b_proj feeds to the attention); MLA_LIN_SPLIT y0 [M, y_split] and
 *      y1 [M, N - y_split] (kv_a_proj_with_mqa's latent and rotary key).
 * Args: x, w device bf16 (w [N, K]); bias device bf16 [N] or NULL; y0/y1
 *   device bf16 as above (y1 only for SPLIT). M >= 0 (0 is a no-op);
 *   N a multiple of 8; K a multiple of 64; M*K, N*K, M*N < 2^31; x_D a
 *   power of two in [8, 4096] dividing K; y_D and y_split multiples of 8;
 *   x_T, y_T dividing M; x, w, y0, y1 16-byte aligned, bias 8-byte aligned.
 * Errors: MLA_ERR_NULL, MLA_ERR_SHAPE, MLA_ERR_HIP. */
mla_status mla_linear(const mla_bf16* x, int32_t x_layout, int32_t x_T, int32_t x_D, const mla_bf16* w,
                      const mla_bf16* bias, int32_t M, int32_t N, int32_t K, mla_bf16* y0, mla_bf16* y1,
                      int32_t y_layout, int32_t y_T, int32_t y_D, int32_t y_split, hipStream_t stream);

/* Human-readable name of a status code (static string, never NULL). */
const char* mla_status_string(mla_status s);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
