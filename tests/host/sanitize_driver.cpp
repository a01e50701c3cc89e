// Host-side argument validation of libswiftkv under AddressSanitizer and
// UndefinedBehaviorSanitizer, on a machine without a GPU: every call below
// must return its documented status before touching the device, with no
// sanitizer report.  Built and run by tests/test_host_sanitizers.py.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "../../include/swiftkv.h"

static int failures = 0;

static void expect(const char* what, skv_status got, skv_status want) {
  const char* msg = skv_last_error();
  if (got != want) {
    printf("FAIL %s: status %d, expected %d (%s)\n", what, (int)got, (int)want, msg);
    ++failures;
  } else if (want != SKV_OK && (!msg || !msg[0])) {
    printf("FAIL %s: no message\n", what);
    ++failures;
  } else {
    printf("ok   %s: %d %s\n", what, (int)got, msg ? msg : "");
  }
}

static skv_model_config base() {
  skv_model_config c;
  memset(&c, 0, sizeof c);
  c.n_layers = 32;
  c.d_model = 4096;
  c.n_q_heads = 32;
  c.n_kv_heads = 8;
  c.head_dim = 128;
  c.ffn_dim = 14336;
  c.vocab = 128256;
  c.rope_theta = 500000.f;
  c.rms_eps = 1e-5f;
  c.swiftkv_l = 16;
  c.acrosskv_g = 1;
  c.dtype = SKV_BF16;
  c.max_tokens = 16384;
  c.max_batch = 16;
  c.max_seqlen = 1024;
  c.kv_dtype = SKV_KV_MODEL;
  return c;
}

int main() {
  skv_model* m = (skv_model*)0x1;
  expect("create: NULL config", skv_model_create(NULL, &m), SKV_ERR_INVALID_ARG);
  if (m != NULL) {
    printf("FAIL create: *out not cleared\n");
    ++failures;
  }
  skv_model_config c = base();
  expect("create: NULL out", skv_model_create(&c, NULL), SKV_ERR_INVALID_ARG);

  struct Case {
    const char* what;
    void (*edit)(skv_model_config*);
    skv_status want;
  } cases[] = {
      {"l > L", [](skv_model_config* x) { x->swiftkv_l = 33; }, SKV_ERR_INVALID_ARG},
      {"l < 0", [](skv_model_config* x) { x->swiftkv_l = -1; }, SKV_ERR_INVALID_ARG},
      {"g = 0", [](skv_model_config* x) { x->acrosskv_g = 0; }, SKV_ERR_INVALID_ARG},
      {"kv heads not dividing", [](skv_model_config* x) { x->n_kv_heads = 3; }, SKV_ERR_INVALID_ARG},
      {"zero layers", [](skv_model_config* x) { x->n_layers = 0; }, SKV_ERR_INVALID_ARG},
      {"negative d_model", [](skv_model_config* x) { x->d_model = -4096; }, SKV_ERR_INVALID_ARG},
      {"odd head_dim", [](skv_model_config* x) { x->head_dim = 127; }, SKV_ERR_INVALID_ARG},
      {"bf16 head_dim 64", [](skv_model_config* x) { x->head_dim = 64; }, SKV_ERR_UNSUPPORTED},
      {"bf16 max_batch 33", [](skv_model_config* x) { x->max_batch = 33; }, SKV_ERR_UNSUPPORTED},
      {"bf16 vocab 1000", [](skv_model_config* x) { x->vocab = 1000; }, SKV_ERR_UNSUPPORTED},
      {"max_tokens 0", [](skv_model_config* x) { x->max_tokens = 0; }, SKV_ERR_INVALID_ARG},
      {"rope_theta 0", [](skv_model_config* x) { x->rope_theta = 0.f; }, SKV_ERR_INVALID_ARG},
      {"rms_eps NaN", [](skv_model_config* x) { x->rms_eps = nanf(""); }, SKV_ERR_INVALID_ARG},
      {"unknown dtype", [](skv_model_config* x) { x->dtype = 7; }, SKV_ERR_INVALID_ARG},
      {"unknown kv dtype", [](skv_model_config* x) { x->kv_dtype = 9; }, SKV_ERR_INVALID_ARG},
      {"FP8 cache on fp32", [](skv_model_config* x) { x->dtype = SKV_FP32; x->kv_dtype = SKV_KV_FP8; },
       SKV_ERR_UNSUPPORTED},
      {"max int dims", [](skv_model_config* x) { x->n_q_heads = 2147483647; }, SKV_ERR_INVALID_ARG},
  };
  for (const Case& k : cases) {
    skv_model_config x = base();
    k.edit(&x);
    skv_model* out = (skv_model*)0x1;
    char what[128];
    snprintf(what, sizeof what, "create: %s", k.what);
    expect(what, skv_model_create(&x, &out), k.want);
  }

  double full = 0, swift = 0;
  int32_t lens[3] = {500, 1000, 768};
  expect("flops: valid", skv_flops(&c, lens, 3, &full, &swift), SKV_OK);
  if (!(swift > 0 && swift < full)) {
    printf("FAIL flops: full %g swift %g\n", full, swift);
    ++failures;
  }
  expect("flops: NULL lengths", skv_flops(&c, NULL, 3, &full, &swift), SKV_ERR_INVALID_ARG);
  expect("flops: negative batch", skv_flops(&c, lens, -1, &full, &swift), SKV_ERR_INVALID_ARG);
  expect("flops: NULL output", skv_flops(&c, lens, 3, NULL, &swift), SKV_ERR_INVALID_ARG);
  skv_model_config bad = base();
  bad.acrosskv_g = 0;
  expect("flops: bad config", skv_flops(&bad, lens, 3, &full, &swift), SKV_ERR_INVALID_ARG);

  float logits[4];
  expect("prefill: NULL", skv_prefill(NULL, NULL, NULL, logits, NULL), SKV_ERR_INVALID_ARG);
  expect("step: NULL batch", skv_step(NULL, NULL, NULL, logits, NULL), SKV_ERR_INVALID_ARG);
  expect("step_noalloc: NULL batch", skv_step_noalloc(NULL, NULL, NULL, logits, NULL), SKV_ERR_INVALID_ARG);
  skv_step_batch sb;
  memset(&sb, 0, sizeof sb);
  int32_t ctx = 3;
  sb.ctx_lens_host = &ctx;  // one of the pair only
  expect("step: half a ctx pair", skv_step(NULL, NULL, &sb, logits, NULL), SKV_ERR_INVALID_ARG);
  expect("step_noalloc: half a ctx pair", skv_step_noalloc(NULL, NULL, &sb, logits, NULL), SKV_ERR_INVALID_ARG);
  memset(&sb, 0, sizeof sb);
  expect("step: NULL model", skv_step(NULL, NULL, &sb, logits, NULL), SKV_ERR_INVALID_ARG);

  skv_kv_cache* kc = (skv_kv_cache*)0x1;
  expect("cache create: NULL model", skv_kv_cache_create(NULL, 16, 16, &kc), SKV_ERR_INVALID_ARG);
  skv_tensor_view kv, vv;
  expect("cache view: NULL cache", skv_kv_cache_view(NULL, 1, &kv, &vv), SKV_ERR_INVALID_ARG);
  expect("cache scales: NULL cache", skv_kv_cache_scales(NULL, 1, &kv, &vv), SKV_ERR_INVALID_ARG);
  expect("load globals: NULL model", skv_model_load_globals(NULL, NULL, NULL, NULL), SKV_ERR_INVALID_ARG);
  skv_layer_weights lw;
  memset(&lw, 0, sizeof lw);
  expect("load layer: NULL model", skv_model_load_layer(NULL, 1, &lw), SKV_ERR_INVALID_ARG);
  expect("profile enable: NULL model", skv_profile_enable(NULL, 0, 1), SKV_ERR_INVALID_ARG);
  double ms, fl, by;
  int64_t n;
  expect("profile read: NULL model", skv_profile_read(NULL, &ms, &n, &fl, &by), SKV_ERR_INVALID_ARG);
  double tf, mhz, mx;
  int32_t cus;
  expect("mfma probe: iters 0", skv_mfma_probe(1, 0, NULL, &tf, &mhz, &cus, &mx), SKV_ERR_INVALID_ARG);
  expect("mfma probe: iters 2^23", skv_mfma_probe(1, 1 << 23, NULL, &tf, &mhz, &cus, &mx), SKV_ERR_INVALID_ARG);
  expect("mfma probe: NULL output", skv_mfma_probe(1, 10, NULL, NULL, &mhz, &cus, &mx), SKV_ERR_INVALID_ARG);
  if (skv_num_kv_slots(NULL) != 0) {
    printf("FAIL num_kv_slots(NULL) != 0\n");
    ++failures;
  }
  skv_model_destroy(NULL);
  skv_kv_cache_destroy(NULL);
  printf(failures ? "FAILURES %d\n" : "ALL OK\n", failures);
  return failures ? 1 : 0;
}
