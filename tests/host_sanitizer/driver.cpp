// Drives every entry point of the C ABI (include/mla.h) through its argument
// validation on the host, under AddressSanitizer and UndefinedBehaviorSanitizer:
// rejected calls must return their documented status and launch nothing;
// accepted calls reach the launcher stand-ins (stubs.cpp), whose invariants
// check what validation let through. Device buffers are placeholder
// addresses that nothing on the host may dereference.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "../../include/mla.h"

extern int g_launches;
static int g_fails = 0;

#define EXPECT(call, code)                                                                       \
  do {                                                                                           \
    const int before_ = g_launches;                                                              \
    const mla_status s_ = (call);                                                                \
    if (s_ != (code)) {                                                                          \
      fprintf(stderr, "%s:%d: %s returned %d, expected %d\n", __FILE__, __LINE__, #call, s_, code); \
      ++g_fails;                                                                                 \
    }                                                                                            \
    if ((code) != MLA_OK && g_launches != before_) {                                             \
      fprintf(stderr, "%s:%d: %s launched work although rejected\n", __FILE__, __LINE__, #call); \
      ++g_fails;                                                                                 \
    }                                                                                            \
  } while (0)

static void* const D = reinterpret_cast<void*>(0x100000);  // placeholder device address
#define DP(T) static_cast<T*>(D)

int main() {
  mla_rope_params yarn = {64, MLA_ROPE_YARN, 50000.0, 32.0, 4096, 32.0, 1.0, 1.0, 1.0};
  mla_rope_params def = {64, MLA_ROPE_DEFAULT, 10000.0, 1.0, 4096, 32.0, 1.0, 1.0, 0.0};
  double m2 = 0, scale = 0;
  // rope table and softmax scale
  EXPECT(mla_rope_table_build(&yarn, 8192, DP(float), DP(float), &m2, 0), MLA_OK);
  EXPECT(mla_rope_table_build(&def, 1, DP(float), DP(float), nullptr, 0), MLA_OK);
  EXPECT(mla_rope_table_build(nullptr, 8, DP(float), DP(float), &m2, 0), MLA_ERR_NULL);
  EXPECT(mla_rope_table_build(&yarn, 0, DP(float), DP(float), &m2, 0), MLA_ERR_SHAPE);
  mla_rope_params bad = yarn;
  bad.type = 7;
  EXPECT(mla_rope_table_build(&bad, 8, DP(float), DP(float), &m2, 0), MLA_ERR_ROPE_TYPE);
  bad = yarn;
  bad.rope_dim = 63;
  EXPECT(mla_rope_table_build(&bad, 8, DP(float), DP(float), &m2, 0), MLA_ERR_SHAPE);
  bad = yarn;
  bad.factor = NAN;
  EXPECT(mla_rope_table_build(&bad, 8, DP(float), DP(float), &m2, 0), MLA_ERR_SHAPE);
  bad = yarn;
  bad.beta_fast = bad.beta_slow = 1e-300;  // extreme correction dims: still a finite band
  EXPECT(mla_rope_table_build(&bad, 8, DP(float), DP(float), &m2, 0), MLA_OK);
  EXPECT(mla_softmax_scale(&yarn, 192, &scale), MLA_OK);
  EXPECT(mla_softmax_scale(&yarn, 0, &scale), MLA_ERR_SHAPE);
  EXPECT(mla_softmax_scale(&yarn, 192, nullptr), MLA_ERR_NULL);
  // RMSNorms
  EXPECT(mla_latent_rmsnorm(DP(mla_bf16), DP(mla_bf16), 1e-6f, DP(uint16_t), 16384, 512, 0), MLA_OK);
  EXPECT(mla_latent_rmsnorm(DP(mla_bf16), DP(mla_bf16), -1.f, DP(uint16_t), 4, 512, 0), MLA_ERR_SHAPE);
  EXPECT(mla_latent_rmsnorm(nullptr, DP(mla_bf16), 1e-6f, DP(uint16_t), 4, 512, 0), MLA_ERR_NULL);
  EXPECT(mla_latent_rmsnorm(nullptr, nullptr, 1e-6f, nullptr, 0, 512, 0), MLA_OK);
  EXPECT(mla_rmsnorm(DP(mla_bf16), DP(mla_bf16), 1e-6f, DP(uint16_t), 7, 1536, MLA_DTYPE_BF16, 0), MLA_OK);
  EXPECT(mla_rmsnorm(DP(mla_bf16), DP(mla_bf16), 1e-6f, DP(uint16_t), 7, 1536, 9, 0), MLA_ERR_UNSUPPORTED);
  // latent prepare
  EXPECT(mla_latent_prepare(DP(mla_bf16), DP(mla_bf16), 1e-6f, DP(mla_bf16), DP(float), DP(float), 8192, nullptr, 2,
                            8192, 512, 64, MLA_PAIR_HALF, DP(uint16_t), DP(uint16_t), 0),
         MLA_OK);
  EXPECT(mla_latent_prepare(DP(mla_bf16), DP(mla_bf16), 1e-6f, DP(mla_bf16), DP(float), DP(float), 100, nullptr, 2,
                            8192, 512, 64, MLA_PAIR_HALF, DP(uint16_t), DP(uint16_t), 0),
         MLA_ERR_SHAPE);
  EXPECT(mla_latent_prepare(DP(mla_bf16), DP(mla_bf16), 1e-6f, DP(mla_bf16), DP(float), DP(float), 100,
                            DP(int32_t), 2, 8192, 512, 64, MLA_PAIR_HALF, DP(uint16_t), DP(uint16_t), 0),
         MLA_OK);
  EXPECT(mla_latent_prepare(DP(mla_bf16), DP(mla_bf16), 1e-6f, DP(mla_bf16), DP(float), DP(float), 8192, nullptr, 2,
                            8192, 512, 64, 5, DP(uint16_t), DP(uint16_t), 0),
         MLA_ERR_ROPE_TYPE);
  // kv_b_proj
  EXPECT(mla_kv_expand(DP(uint16_t), DP(mla_bf16), 2, 8192, 512, 64, 128, 128, DP(uint16_t), 128, DP(uint16_t),
                       MLA_V_COLS, 8192, 8192, 0, MLA_DTYPE_FP16, nullptr, nullptr, nullptr, 0, nullptr, 0, 0, 0),
         MLA_OK);
  EXPECT(mla_kv_expand(DP(uint16_t), DP(mla_bf16), 2, 8192, 512, 64, 128, 128, DP(uint16_t), 128, DP(uint16_t),
                       MLA_V_COLS, 8000, 8192, 0, MLA_DTYPE_FP16, nullptr, nullptr, nullptr, 0, nullptr, 0, 0, 0),
         MLA_ERR_SHAPE);
  EXPECT(mla_kv_expand(DP(uint16_t), DP(mla_bf16), 32, 1, 512, 64, 128, 128, DP(uint16_t), 192, DP(uint16_t),
                       MLA_V_ROWS, 0, 1001, 1000, MLA_DTYPE_BF16, DP(mla_bf16), DP(float), DP(float), 1001,
                       DP(int32_t), 64, MLA_PAIR_HALF, 0),
         MLA_OK);
  EXPECT(mla_kv_expand(DP(uint16_t), DP(mla_bf16), 32, 1, 512, 64, 128, 128, DP(uint16_t), 192, DP(uint16_t),
                       MLA_V_ROWS, 0, 1001, 1001, MLA_DTYPE_BF16, nullptr, nullptr, nullptr, 0, nullptr, 0, 0, 0),
         MLA_ERR_SHAPE);
  // prefill
  size_t ws = 0;
  EXPECT(mla_prefill_attention(DP(mla_bf16), DP(uint16_t), DP(mla_bf16), DP(uint16_t), MLA_V_ROWS, 0, MLA_DTYPE_FP16,
                               DP(float), DP(float), 8192, nullptr, 2, 64, 8192, 128, 64, 128, 0.13f, 0,
                               DP(mla_bf16), nullptr, nullptr, &ws, 0),
         MLA_OK);
  if (ws == 0) {
    fprintf(stderr, "prefill workspace query returned 0\n");
    ++g_fails;
  }
  size_t have = ws;
  EXPECT(mla_prefill_attention(DP(mla_bf16), DP(uint16_t), DP(mla_bf16), DP(uint16_t), MLA_V_ROWS, 0, MLA_DTYPE_FP16,
                               DP(float), DP(float), 8192, nullptr, 2, 64, 8192, 128, 64, 128, 0.13f, 0,
                               DP(mla_bf16), nullptr, D, &have, 0),
         MLA_OK);
  have = ws - 1;
  EXPECT(mla_prefill_attention(DP(mla_bf16), DP(uint16_t), DP(mla_bf16), DP(uint16_t), MLA_V_ROWS, 0, MLA_DTYPE_FP16,
                               DP(float), DP(float), 8192, nullptr, 2, 64, 8192, 128, 64, 128, 0.13f, 0,
                               DP(mla_bf16), nullptr, D, &have, 0),
         MLA_ERR_WORKSPACE);
  EXPECT(mla_prefill_attention(DP(mla_bf16), DP(uint16_t), DP(mla_bf16), DP(uint16_t), MLA_V_COLS, 8192,
                               MLA_DTYPE_BF16, DP(float), DP(float), 8192, nullptr, 2, 64, 8192, 128, 64, 128, 0.13f,
                               0, DP(mla_bf16), nullptr, D, &ws, 0),
         MLA_ERR_UNSUPPORTED);
  EXPECT(mla_prefill_attention(DP(mla_bf16), DP(uint16_t), DP(mla_bf16), DP(uint16_t), MLA_V_COLS, 8190,
                               MLA_DTYPE_FP16, DP(float), DP(float), 8192, nullptr, 2, 64, 8192, 128, 64, 128, 0.13f,
                               0, DP(mla_bf16), nullptr, D, &ws, 0),
         MLA_ERR_SHAPE);
  EXPECT(mla_prefill_attention_cached(DP(mla_bf16), DP(uint16_t), DP(uint16_t), DP(uint16_t), 8192, MLA_DTYPE_FP16,
                                      DP(float), DP(float), 8192, nullptr, 2, 64, 1024, 7168, 8192, 128, 64, 128,
                                      0.13f, 0, DP(mla_bf16), nullptr, 0),
         MLA_OK);
  EXPECT(mla_prefill_attention_cached(DP(mla_bf16), DP(uint16_t), DP(uint16_t), DP(uint16_t), 8192, MLA_DTYPE_FP16,
                                      DP(float), DP(float), 8192, nullptr, 2, 64, 1025, 7168, 8192, 128, 64, 128,
                                      0.13f, 0, DP(mla_bf16), nullptr, 0),
         MLA_ERR_SHAPE);
  EXPECT(mla_rotate_rope_key(DP(mla_bf16), DP(float), DP(float), 8192, nullptr, 2, 1024, 64, 0, DP(uint16_t), 8192,
                             7168, MLA_DTYPE_FP16, 0),
         MLA_OK);
  // decode, with and without a workspace
  EXPECT(mla_decode_attention(DP(mla_bf16), DP(uint16_t), DP(uint16_t), MLA_DTYPE_BF16, DP(int32_t), DP(int32_t),
                              DP(float), DP(float), 1001, 32, 64, 1001, 128, 64, 128, 0.13f, 0, 0, nullptr, nullptr,
                              DP(mla_bf16), 0),
         MLA_OK);  // automatic split count 1 at this batch: no workspace needed
  ws = 0;
  EXPECT(mla_decode_attention(DP(mla_bf16), DP(uint16_t), DP(uint16_t), MLA_DTYPE_BF16, DP(int32_t), DP(int32_t),
                              DP(float), DP(float), 1001, 2, 8, 1001, 128, 64, 128, 0.13f, 0, 0, nullptr, &ws,
                              DP(mla_bf16), 0),
         MLA_OK);
  EXPECT(mla_decode_attention(DP(mla_bf16), DP(uint16_t), DP(uint16_t), MLA_DTYPE_BF16, DP(int32_t), DP(int32_t),
                              DP(float), DP(float), 1001, 2, 8, 1001, 128, 64, 128, 0.13f, 0, 0, D, &ws,
                              DP(mla_bf16), 0),
         MLA_OK);
  EXPECT(mla_decode_attention(DP(mla_bf16), DP(uint16_t), DP(uint16_t), MLA_DTYPE_BF16, DP(int32_t), DP(int32_t),
                              DP(float), DP(float), 1001, 2, 8, 1001, 128, 64, 128, 0.13f, 0, 0, nullptr, nullptr,
                              DP(mla_bf16), 0),
         MLA_ERR_WORKSPACE);
  EXPECT(mla_decode_attention_noalloc(DP(mla_bf16), DP(uint16_t), DP(uint16_t), MLA_DTYPE_BF16, DP(int32_t),
                                      DP(int32_t), DP(float), DP(float), 1001, 2, 8, 1001, 128, 64, 128, 0.13f, 0, 0,
                                      DP(mla_bf16), 0),
         MLA_OK);
  EXPECT(mla_decode_attention_noalloc(DP(mla_bf16), DP(uint16_t), DP(uint16_t), MLA_DTYPE_BF16, DP(int32_t),
                                      DP(int32_t), DP(float), DP(float), 1001, 256, 64, 1001, 128, 64, 128, 0.13f, 0,
                                      4, DP(mla_bf16), 0),
         MLA_ERR_WORKSPACE);
  // latent cache
  EXPECT(mla_absorb_prepare(DP(mla_bf16), 64, 512, 128, 128, DP(mla_bf16), 0), MLA_OK);
  EXPECT(mla_latent_cache_append(DP(mla_bf16), DP(mla_bf16), 1e-6f, DP(mla_bf16), DP(float), DP(float), 1001,
                                 DP(int32_t), 0, 32, 512, 64, DP(uint16_t), 1001, 0),
         MLA_OK);
  ws = 0;
  EXPECT(mla_decode_absorbed(DP(mla_bf16), DP(mla_bf16), DP(mla_bf16), DP(uint16_t), DP(int32_t), DP(int32_t),
                             DP(float), DP(float), 1001, 32, 64, 1001, 512, 128, 64, 128, 0.13f, 0, 0, nullptr, &ws,
                             DP(mla_bf16), 0),
         MLA_OK);
  EXPECT(mla_decode_absorbed(DP(mla_bf16), DP(mla_bf16), DP(mla_bf16), DP(uint16_t), DP(int32_t), DP(int32_t),
                             DP(float), DP(float), 1001, 32, 64, 1001, 512, 128, 64, 128, 0.13f, 0, 0, D, &ws,
                             DP(mla_bf16), 0),
         MLA_OK);
  EXPECT(mla_decode_absorbed(DP(mla_bf16), DP(mla_bf16), DP(mla_bf16), DP(uint16_t), DP(int32_t), DP(int32_t),
                             DP(float), DP(float), 1001, 32, 64, 1001, 256, 128, 64, 128, 0.13f, 0, 0, D, &ws,
                             DP(mla_bf16), 0),
         MLA_ERR_UNSUPPORTED);
  ws = 0;
  EXPECT(mla_decode_latent_expanded(DP(mla_bf16), DP(mla_bf16), DP(uint16_t), DP(int32_t), DP(int32_t), DP(float),
                                    DP(float), 1001, 4, 8, 1001, 512, 128, 64, 128, 0.13f, 0, 0, nullptr, &ws,
                                    DP(mla_bf16), 0),
         MLA_OK);
  EXPECT(mla_decode_latent_expanded(DP(mla_bf16), DP(mla_bf16), DP(uint16_t), DP(int32_t), DP(int32_t), DP(float),
                                    DP(float), 1001, 4, 8, 1001, 512, 128, 64, 128, 0.13f, 0, 0, D, &ws,
                                    DP(mla_bf16), 0),
         MLA_OK);
  // linear layers
  EXPECT(mla_linear(DP(mla_bf16), MLA_LIN_ROWS, 0, 0, DP(mla_bf16), nullptr, 16384, 1536, 7168, DP(mla_bf16), nullptr,
                    MLA_LIN_ROWS, 0, 0, 0, 0),
         MLA_OK);
  EXPECT(mla_linear(DP(mla_bf16), MLA_LIN_HEADS, 8192, 128, DP(mla_bf16), nullptr, 16384, 7168, 8192, DP(mla_bf16),
                    nullptr, MLA_LIN_ROWS, 0, 0, 0, 0),
         MLA_OK);
  EXPECT(mla_linear(DP(mla_bf16), MLA_LIN_ROWS, 0, 0, DP(mla_bf16), nullptr, 16384, 576, 7168, DP(mla_bf16), nullptr,
                    MLA_LIN_SPLIT, 0, 0, 512, 0),
         MLA_ERR_NULL);
  EXPECT(mla_linear(DP(mla_bf16), MLA_LIN_ROWS, 0, 0, DP(mla_bf16), nullptr, 1 << 20, 4096, 4096, DP(mla_bf16),
                    nullptr, MLA_LIN_ROWS, 0, 0, 0, 0),
         MLA_ERR_SHAPE);  // M*K beyond 32-bit offsets
  const char* s = mla_status_string(static_cast<mla_status>(-42));
  if (!s || strlen(s) == 0) ++g_fails;
  printf("host sanitizer driver: %d launches, %d failures\n", g_launches, g_fails);
  return g_fails ? 1 : 0;
}
