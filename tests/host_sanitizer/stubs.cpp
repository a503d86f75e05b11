// Host-only stand-ins for the device-side launchers that the C ABI layer
// (csrc/api.cpp) calls, for a sanitizer build of that layer without a GPU.
// Each records the call and checks that argument validation let through only
// what the real launcher may be given; a broken invariant aborts. The small
// host helpers (supported shapes, split counts, workspace sizes) repeat the
// library's rules.
#include <stdio.h>
#include <stdlib.h>

#include "../../head_latent_attention_rmsnorm_amd/csrc/launch.hpp"

int g_launches = 0;

#define NEED(c)                                                            \
  do {                                                                     \
    if (!(c)) {                                                            \
      fprintf(stderr, "%s:%d: launcher invariant broken: %s\n", __FILE__, __LINE__, #c); \
      abort();                                                             \
    }                                                                      \
  } while (0)

extern "C" hipError_t hipGetLastError(void) { return hipSuccess; }

namespace mla {

hipError_t launch_rope_table(const RopeResolved& r, int n_pos, float* c, float* s, hipStream_t) {
  // the band may come out inverted (low > high) for reversed betas, as the
  // pages compute it; only a zero-width band would divide by zero
  NEED(n_pos >= 1 && c && s && r.dim >= 2 && (r.dim & 1) == 0 && r.high != r.low);
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_rmsnorm(const uint16_t* x, const uint16_t* w, float eps, uint16_t* y, int n, int R, int,
                          hipStream_t) {
  NEED(x && w && y && n >= 1 && R >= 1 && eps >= 0.f);
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_latent_prepare(const LatentPrepareArgs& a, hipStream_t) {
  NEED(a.x && a.w && a.y && a.k_pe && a.k_rot && a.cos && a.sin && a.n >= 1 && a.T >= 1 && a.R % 8 == 0);
  NEED(a.R <= 4096 && a.Dr >= 2 && (a.Dr & 1) == 0 && a.table_len >= 1 && (a.pos || a.T <= a.table_len));
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_kv_expand(const ExpandArgs& a, hipStream_t) {
  NEED(a.c && a.W && a.k && a.v && a.B >= 1 && a.T >= 1 && a.H >= 1 && a.k_ld >= a.Dn);
  NEED(a.t_off >= 0 && a.t_off + a.T <= a.Tcap && (!a.v_cols || a.v_ld >= a.Tcap));
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_rotate_key(const RotKeyArgs& a, hipStream_t) {
  NEED(a.k_pe && a.cos && a.sin && a.dst && a.B >= 1 && a.T >= 1 && a.table_len >= 1 && a.t_off + a.T <= a.Tcap);
  ++g_launches;
  return hipSuccess;
}
bool prefill_supported(int Dqk, int Dr, int Dv) {
  return (Dqk == 48 && Dr == 16 && Dv == 32) || (Dqk == 192 && Dr == 64 && Dv == 128) ||
         (Dqk == 256 && Dr == 64 && Dv == 256);
}
bool prefill_dual_supported(int Dqk, int Dr, int Dv) { return Dqk == 192 && Dr == 64 && Dv == 128; }
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t) {
  NEED(a.q && a.k_nope && a.k_rot && a.v && a.cos && a.sin && a.out && a.B >= 1 && a.T >= 1 && a.H >= 1);
  NEED(a.kv_dtype == 1 && a.v_ld % 8 == 0 && a.v_ld >= a.past + a.T && a.kv_stride >= a.past + a.T);
  NEED(a.table_len >= 1 && (a.pos || a.past + a.T <= a.table_len) && a.scale > 0.f);
  NEED(prefill_supported(a.Dn + a.Dr, a.Dr, a.Dv));
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_prefill_dual(const PrefillArgs& a, hipStream_t s) { return launch_prefill(a, s); }
hipError_t launch_transpose_v(const uint16_t* v, uint16_t* vt, int BH, int T, int Dv, int v_ld, hipStream_t) {
  NEED(v && vt && BH >= 1 && T >= 1 && Dv >= 1 && v_ld >= T && v_ld % 8 == 0);
  ++g_launches;
  return hipSuccess;
}
bool decode_supported(int Dqk, int Dv) {
  return (Dqk == 192 && Dv == 128) || (Dqk == 256 && Dv == 256) || (Dqk == 48 && Dv == 32);
}
int decode_auto_splits(int B, int H, int Tcap) {
  const int bh = B * H;
  if (bh <= 0) return 1;
  int s = (2048 + bh - 1) / bh;
  const int smax = (Tcap + 255) / 256;
  if (s > smax) s = smax;
  if (s < 1) s = 1;
  if (s > 256) s = 256;
  return s;
}
size_t decode_workspace_bytes(int B, int H, int Dv, int splits) {
  if (splits <= 1) return 0;
  const size_t n = (size_t)B * H * splits;
  return ((n * Dv * sizeof(float)) + 255) / 256 * 256 + n * 2 * sizeof(float);
}
hipError_t launch_decode(const DecodeArgs& a, hipStream_t) {
  NEED(a.q && a.k_cache && a.v_cache && a.seq_len && a.q_pos && a.cos && a.sin && a.out);
  NEED(a.B >= 1 && a.H >= 1 && a.num_splits >= 1 && a.num_splits <= 256 && a.table_len >= 1);
  NEED(a.num_splits == 1 || (a.part_o && a.part_ml && a.part_ml > a.part_o));
  ++g_launches;
  return hipSuccess;
}
alignas(256) static unsigned char g_scratch[kDecodeScratchBytes];
hipError_t decode_scratch(void** ptr) {
  *ptr = g_scratch;
  return hipSuccess;
}
hipError_t launch_absorb_prepare(const uint16_t* W, uint16_t* wt, int H, int R, int Dn, int, hipStream_t) {
  NEED(W && wt && H >= 1 && R >= 1 && Dn >= 1);
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_latent_append(const LatentAppendArgs& a, hipStream_t) {
  NEED(a.latent && a.gain && a.k_pe && a.cos && a.sin && a.t_pos && a.cache && a.B >= 1 && a.table_len >= 1);
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_absorb_q(const AbsorbArgs& a, hipStream_t) {
  NEED(a.q && a.w_ukt && a.q_pos && a.cos && a.sin && a.qa && a.B >= 1 && a.H >= 1);
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_latent_attn(const LatentAttnArgs& a, hipStream_t) {
  NEED(a.qa && a.cache && a.seq_len && a.part_o && a.part_lse && a.S >= 1 && a.S <= kMaxLatentSplits && a.tps >= 1);
  NEED((int64_t)a.S * a.tps * 64 >= a.Lcap);
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_combine_unabsorb(const CombineUnabsorbArgs& a, hipStream_t) {
  NEED(a.part_o && a.part_lse && a.W && a.out && a.B >= 1 && a.H >= 1 && a.S >= 1 && a.S <= kMaxLatentSplits);
  NEED(a.Dv >= 32 && a.Dv % 32 == 0);
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_latent_reexpand_copies(const uint16_t* cache, uint16_t* c, uint16_t* k, int B, int H, int Lcap,
                                         int R, int Dr, int, hipStream_t) {
  NEED(cache && c && k && B >= 1 && H >= 1 && Lcap >= 1 && R % 8 == 0 && Dr % 8 == 0);
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_linear(const LinearArgs& a, hipStream_t) {
  NEED(a.x && a.w && a.y0 && a.M >= 1 && a.N % 8 == 0 && a.K % 64 == 0 && (a.y_mode != 2 || a.y1));
  ++g_launches;
  return hipSuccess;
}

}  // namespace mla
