// C ABI of libswiftkv: model and cache objects, load-time repacking,
// host-side validation and the prefill launch sequence.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/swiftkv.h"
#include "kernels.h"

namespace {

thread_local std::string g_err;

skv_status fail(skv_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

#define SKV_HIP(call)                                                                         \
  do {                                                                                        \
    hipError_t e_ = (call);                                                                   \
    if (e_ != hipSuccess)                                                                     \
      return fail(SKV_ERR_HIP, std::string(#call) + ": " + hipGetErrorString(e_));            \
  } while (0)

int ceil_div(int a, int b) { return (a + b - 1) / b; }

// bf16 batches of at most this many new tokens take the row path through
// layers 1..l (run_step).
constexpr int kRowPathMax = kSkinnyMaxRows;
size_t round_up(size_t a, size_t b) { return (a + b - 1) / b * b; }

}  // namespace

// Scratch of skv_step_noalloc: every buffer a row-path call writes besides
// its inputs and outputs (residual rows, bf16 rows, split-K and attention
// partials, per-token metadata) is carved out of this array.  Each device
// holds its own copy for the life of the process.  Host code never passes
// `scratch` itself to a kernel: it uses the device address that
// hipGetSymbolAddress returned on that device (noalloc_scratch below).
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Look up (once per device, with that device current) the device address of
// this device's `scratch`.  Called by skv_model_create.
skv_status noalloc_scratch_init() {
  int dev = 0;
  SKV_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(SKV_ERR_UNSUPPORTED, "device index beyond the scratch table");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    SKV_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return fail(SKV_ERR_HIP, "hipGetSymbolAddress returned NULL for the scratch array");
    g_scratch_ptr[dev] = p;
  }
  return SKV_OK;
}

// The current device's scratch address (NULL if no model was created on it).
void* noalloc_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  return g_scratch_ptr[dev];
}

}  // namespace

// Weights of layers 1..l feed the prompt-token GEMMs and are kept in the
// panel layout with 256-row panels; those of skipped layers (and the LM
// head) feed only the last-token path and use 64-row panels (bf16 models).
// fp32 models keep everything row-major.
struct LayerDev {
  float* attn_norm = nullptr;  // fp32 [d]
  float* ffn_norm = nullptr;
  void* wqkv = nullptr;  // unskipped: [dq + 2 dkv, d]; skipped: [dq, d]
  void* wo = nullptr;    // [d, dq]
  // layer 1 of a bf16 model with a split first layer: [W | W] with twice the
  // columns (panel layout), the B operand of the split-bf16 QKV and O GEMMs
  void* wqkv2 = nullptr;  // [dq + 2 dkv, 2 d]
  void* wo2 = nullptr;    // [d, 2 dq]
  void* wgu = nullptr;   // [2f, d], gate/up interleaved in blocks of P_mlp rows
  void* wdown = nullptr; // [d, f]
  int panel_rows = 0;    // 0: row-major; else the panel height of the layout
  bool loaded = false;
};

struct ProfRec {
  hipEvent_t a, b;
};

struct skv_model {
  skv_model_config cfg;
  bool bf16;
  size_t esz;
  int G;       // AcrossKV groups of skipped layers
  // Prompt tokens run layer 1 in split-bf16 form (bf16 model, l >= 1): the
  // QKV GEMM takes the hi and lo parts of its input (K doubled against
  // [W | W]); with a bf16 cache the attention also computes with both parts
  // of q, K and V, and the O GEMM with both parts of its input.  Layer 1
  // writes the whole residual stream (the embeddings are small), so its
  // rounding dominates what deeper layers inherit.
  bool split1 = false;
  int p_mlp;   // gate/up interleave distance
  int dq, dkv;
  std::vector<void*> allocs;

  void* embed = nullptr;
  void* lm_head = nullptr;
  float* final_norm = nullptr;
  float* rope_cos = nullptr;
  float* rope_sin = nullptr;
  bool globals_loaded = false;
  std::vector<LayerDev> layers;
  void* wkv_skip = nullptr;  // [G * 2 dkv, d] (panel layout for bf16)
  void* staging = nullptr;
  size_t staging_bytes = 0;
  void* gamma_stage = nullptr;

  // workspace
  float* x = nullptr;
  void* act = nullptr;
  void* qbuf = nullptr;
  void* qlo = nullptr;  // split layer 1: low parts of q [T, dq]
  void* obuf = nullptr;
  void* hbuf = nullptr;
  int32_t* pos = nullptr;
  int32_t* slot = nullptr;
  int32_t* seq = nullptr;
  int32_t* last_pos = nullptr;
  int32_t* last_row = nullptr;
  int32_t* iota = nullptr;
  // FP8 KV cache: new K/V rows (bf16) staged in the cache layout with the
  // token index as physical slot, then quantised into the cache
  bool kv8 = false;
  bf16_t* kv_stage = nullptr;
  int64_t stage_group = 0;  // elements per group (K then V)
  int64_t stage_v = 0;      // offset of V within a group
  int32_t* tok_iota = nullptr;
  float* y = nullptr;
  void* ya = nullptr;
  void* yq = nullptr;
  void* yo = nullptr;
  void* yh = nullptr;
  float* partial = nullptr;
  int64_t partial_elems = 0;
  // bf16 prompt-token path: RMSNorm factor per token row, and the partial
  // sums of squares [T, d/16] the residual epilogues leave for it
  float* rrow = nullptr;
  float* ssp = nullptr;
  // bf16 row path: partial sums of squares [RY, d/128] of the rows whose
  // bf16(x * gain) `ya` holds (the skinny products apply the RMSNorm factor)
  float* rss = nullptr;
  float* attn_ws = nullptr;
  int64_t attn_ws_elems = 0;
  float* gemm_ws = nullptr;  // split partial tiles of the GEMMs
  int64_t gemm_ws_elems = 0;

  // profiling
  int prof_class = -1;
  std::vector<ProfRec> prof;
  double prof_flops = 0, prof_bytes = 0;
};

struct skv_kv_cache {
  const skv_model* m;
  int num_blocks, block_size, n_slots;
  void* k;
  void* v;
  int64_t slot_elems;
  bool fp8 = false;
  float* ks = nullptr;  // FP8: per-token scales [n_slots][num_blocks * block_size]
  float* vs = nullptr;
  // split first layer: low parts of layer 1's K and V in the slot layout
  // (written with the slot, read by the split prompt attention)
  void* klo = nullptr;
  void* vlo = nullptr;
};

namespace {

template <typename T>
skv_status dev_alloc(skv_model* m, T** p, size_t bytes) {
  void* q = nullptr;
  if (bytes == 0) bytes = 16;
  if (hipMalloc(&q, bytes) != hipSuccess) {
    (void)hipGetLastError();
    return fail(SKV_ERR_OOM, "hipMalloc of " + std::to_string(bytes) + " bytes failed");
  }
  m->allocs.push_back(q);
  *p = reinterpret_cast<T*>(q);
  return SKV_OK;
}

#define SKV_TRY(x)                  \
  do {                              \
    skv_status s_ = (x);            \
    if (s_ != SKV_OK) return s_;    \
  } while (0)

skv_status validate_config(const skv_model_config* c) {
  if (!c) return fail(SKV_ERR_INVALID_ARG, "config is NULL");
  if (c->n_layers < 1 || c->d_model < 1 || c->n_q_heads < 1 || c->n_kv_heads < 1 || c->head_dim < 2 ||
      c->ffn_dim < 1 || c->vocab < 1)
    return fail(SKV_ERR_INVALID_ARG, "model dimensions must be positive");
  if (c->head_dim % 2) return fail(SKV_ERR_INVALID_ARG, "head_dim must be even (rotate-half RoPE)");
  if (c->n_q_heads % c->n_kv_heads) return fail(SKV_ERR_INVALID_ARG, "n_q_heads must be a multiple of n_kv_heads");
  if (c->swiftkv_l < 0 || c->swiftkv_l > c->n_layers)
    return fail(SKV_ERR_INVALID_ARG, "swiftkv_l must lie in 0..n_layers");
  if (c->acrosskv_g < 1) return fail(SKV_ERR_INVALID_ARG, "acrosskv_g must be >= 1");
  if (c->dtype != SKV_BF16 && c->dtype != SKV_FP32) return fail(SKV_ERR_INVALID_ARG, "unknown dtype");
  if (c->kv_dtype != SKV_KV_MODEL && c->kv_dtype != SKV_KV_FP8) return fail(SKV_ERR_INVALID_ARG, "unknown kv_dtype");
  if (c->kv_dtype == SKV_KV_FP8 && c->dtype != SKV_BF16)
    return fail(SKV_ERR_UNSUPPORTED, "the FP8 KV cache needs a bf16 model");
  if (c->kv_dtype == SKV_KV_FP8 && (int64_t)c->n_kv_heads * c->head_dim > 1024)
    return fail(SKV_ERR_UNSUPPORTED, "the FP8 KV cache needs n_kv_heads * head_dim <= 1024");
  if (c->max_tokens < 1 || c->max_batch < 1 || c->max_seqlen < 1)
    return fail(SKV_ERR_INVALID_ARG, "max_tokens, max_batch and max_seqlen must be positive");
  if (!(c->rope_theta > 0.f) || !(c->rms_eps >= 0.f)) return fail(SKV_ERR_INVALID_ARG, "bad rope_theta or rms_eps");
  if (c->d_model % 4) return fail(SKV_ERR_UNSUPPORTED, "d_model must be a multiple of 4");
  if (c->n_q_heads / c->n_kv_heads > 16) return fail(SKV_ERR_UNSUPPORTED, "at most 16 q heads per kv head");
  if (c->dtype == SKV_BF16) {
    if (c->head_dim != 128) return fail(SKV_ERR_UNSUPPORTED, "bf16 path needs head_dim 128");
    if ((c->n_q_heads / c->n_kv_heads) % 4) return fail(SKV_ERR_UNSUPPORTED, "bf16 path needs hq/hkv % 4 == 0");
    if (c->d_model % 256 || c->ffn_dim % 256)
      return fail(SKV_ERR_UNSUPPORTED, "bf16 path needs d_model and ffn_dim multiples of 256");
    if (c->d_model > 8192) return fail(SKV_ERR_UNSUPPORTED, "bf16 path supports d_model up to 8192");
    if (c->vocab % 128) return fail(SKV_ERR_UNSUPPORTED, "bf16 path needs vocab % 128 == 0");
    if (c->max_batch > 32) return fail(SKV_ERR_UNSUPPORTED, "bf16 path supports at most 32 prompts per call");
  } else {
    if (c->head_dim != 32 && c->head_dim != 64 && c->head_dim != 128)
      return fail(SKV_ERR_UNSUPPORTED, "fp32 path needs head_dim 32, 64 or 128");
    if (c->d_model % 32 || c->ffn_dim % 16 || c->vocab % 32)
      return fail(SKV_ERR_UNSUPPORTED, "fp32 path needs d_model % 32, ffn_dim % 16, vocab % 32 == 0");
    if (c->n_q_heads / c->n_kv_heads > 16) return fail(SKV_ERR_UNSUPPORTED, "at most 16 q heads per kv head");
  }
  return SKV_OK;
}

int slot_of_layer(const skv_model_config& c, int j) {
  return j <= c.swiftkv_l ? j - 1 : c.swiftkv_l + (j - c.swiftkv_l - 1) / c.acrosskv_g;
}
bool is_representative(const skv_model_config& c, int j) {
  return j > c.swiftkv_l && (j - c.swiftkv_l - 1) % c.acrosskv_g == 0;
}

struct Prof {
  skv_model* m;
  bool on;
  hipEvent_t a{}, b{};
  hipStream_t s;
  Prof(skv_model* m_, int cls, hipStream_t s_, double flops, double bytes)
      : m(m_), on(m_ && m_->prof_class == cls), s(s_) {
    if (on) {
      hipEventCreate(&a);
      hipEventCreate(&b);
      hipEventRecord(a, s);
      m->prof_flops += flops;
      m->prof_bytes += bytes;
    }
  }
  ~Prof() {
    if (on) {
      hipEventRecord(b, s);
      m->prof.push_back({a, b});
    }
  }
};

double gemm_bytes(double M, double N, double K, double esz, double out_bytes_per) {
  return (M * K + N * K) * esz + M * N * out_bytes_per;
}

}  // namespace

extern "C" {

const char* skv_last_error(void) { return g_err.c_str(); }

skv_status skv_flops(const skv_model_config* c, const int32_t* seqlens, int32_t batch, double* full, double* swift) {
  SKV_TRY(validate_config(c));
  if (batch < 0 || (batch > 0 && !seqlens) || !full || !swift) return fail(SKV_ERR_INVALID_ARG, "bad arguments");
  const double d = c->d_model, dq = (double)c->n_q_heads * c->head_dim, dkv = (double)c->n_kv_heads * c->head_dim;
  const double f = c->ffn_dim, V = c->vocab, L = c->n_layers, l = c->swiftkv_l, hq = c->n_q_heads,
               dh = c->head_dim;
  const double G = ceil_div(c->n_layers - c->swiftkv_l, c->acrosskv_g);
  const double lin = 2 * d * dq + 2 * dq * d + 6 * d * f + 4 * d * dkv;
  double F = 0, S = 0;
  for (int b = 0; b < batch; ++b) {
    const double n = seqlens[b];
    const double layer_full = n * lin + 2 * n * (n + 1) * dh * hq;
    F += L * layer_full + 2 * d * V;
    S += l * layer_full + G * n * 4 * d * dkv + (L - l) * (2 * d * dq + 2 * dq * d + 6 * d * f + 4 * n * dh * hq) +
         2 * d * V;
  }
  *full = F;
  *swift = S;
  return SKV_OK;
}

skv_status skv_model_create(const skv_model_config* cfg, skv_model** out) {
  if (!out) return fail(SKV_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  SKV_TRY(validate_config(cfg));
  SKV_TRY(noalloc_scratch_init());
  skv_model* m = new skv_model();
  m->cfg = *cfg;
  const auto& c = m->cfg;
  m->bf16 = c.dtype == SKV_BF16;
  m->esz = m->bf16 ? 2 : 4;
  m->G = ceil_div(c.n_layers - c.swiftkv_l, c.acrosskv_g);
  // bf16: the interleave distance of the gate/up GEMM's SwiGLU epilogue
  m->p_mlp = m->bf16 ? EpiSwiGLUPanel::P : 16;
  m->dq = c.n_q_heads * c.head_dim;
  m->dkv = c.n_kv_heads * c.head_dim;
  m->layers.resize(c.n_layers);
  const size_t d = c.d_model, dq = m->dq, dkv = m->dkv, f = c.ffn_dim, V = c.vocab, E = m->esz;
  const size_t T = c.max_tokens, B = c.max_batch;
  auto bail = [&](skv_status s) {
    std::string msg = g_err;
    skv_model_destroy(m);
    g_err = msg;
    return s;
  };
#define ALLOC(p, bytes)                                \
  do {                                                 \
    skv_status s_ = dev_alloc(m, &(p), (bytes));       \
    if (s_ != SKV_OK) return bail(s_);                 \
  } while (0)
  ALLOC(m->embed, V * d * E);
  ALLOC(m->lm_head, V * d * E);
  ALLOC(m->final_norm, d * 4);
  const size_t half = c.head_dim / 2;
  ALLOC(m->rope_cos, (size_t)c.max_seqlen * half * 4);
  ALLOC(m->rope_sin, (size_t)c.max_seqlen * half * 4);
  // panel-layout matrices round their row count up to whole panels
  const size_t R = m->bf16 ? kPanelRows : 1;
  for (int i = 1; i <= c.n_layers; ++i) {
    LayerDev& L = m->layers[i - 1];
    L.panel_rows = !m->bf16 ? 0 : i <= c.swiftkv_l ? kPanelRows : kSkinnyPanelRows;
    const size_t r = L.panel_rows ? L.panel_rows : 1;
    ALLOC(L.attn_norm, d * 4);
    ALLOC(L.ffn_norm, d * 4);
    ALLOC(L.wqkv, round_up(i <= c.swiftkv_l ? dq + 2 * dkv : dq, r) * d * E);
    ALLOC(L.wo, round_up(d, r) * dq * E);
    ALLOC(L.wgu, round_up(2 * f, r) * d * E);
    ALLOC(L.wdown, round_up(d, r) * f * E);
  }
  if (m->G > 0) ALLOC(m->wkv_skip, round_up((size_t)m->G * 2 * dkv, R) * d * E);
  m->split1 = m->bf16 && c.swiftkv_l >= 1;
  m->staging_bytes = std::max({2 * f * d, (dq + 2 * dkv) * d, d * dq, d * f}) * E;
  // split layer 1: W row-major plus [W | W] row-major side by side
  if (m->split1) m->staging_bytes = std::max(m->staging_bytes, std::max(3 * (dq + 2 * dkv) * d, 3 * d * dq) * E);
  ALLOC(m->staging, m->staging_bytes);
  ALLOC(m->gamma_stage, d * E);

  const size_t Tp = round_up(T, R);  // token rows of the panel-layout activations
  ALLOC(m->x, T * d * 4);
  const size_t acols = m->split1 ? 2 * d : d, ocols = m->split1 ? 2 * dq : dq;
  ALLOC(m->act, Tp * acols * E);
  ALLOC(m->qbuf, T * dq * E);
  if (m->split1) {
    ALLOC(m->qlo, T * dq * E);
    LayerDev& L1 = m->layers[0];
    ALLOC(L1.wqkv2, round_up(dq + 2 * dkv, kPanelRows) * 2 * d * E);
    ALLOC(L1.wo2, round_up(d, kPanelRows) * 2 * dq * E);
  }
  ALLOC(m->obuf, Tp * ocols * E);
  ALLOC(m->hbuf, Tp * f * E);
  ALLOC(m->pos, T * 4);
  ALLOC(m->slot, T * 4);
  ALLOC(m->seq, T * 4);
  ALLOC(m->last_pos, B * 4);
  ALLOC(m->last_row, B * 4);
  ALLOC(m->iota, B * 4);
  ALLOC(m->y, B * d * 4);
  // row-major buffers: the last tokens, and (bf16) the new tokens of a
  // batch small enough for the row path
  const size_t RY = m->bf16 ? std::max(B, std::min(T, (size_t)kRowPathMax)) : B;
  ALLOC(m->ya, RY * d * E);
  ALLOC(m->yq, RY * dq * E);
  ALLOC(m->yo, RY * dq * E);
  ALLOC(m->yh, RY * f * E);
  if (m->bf16) ALLOC(m->rss, RY * (d / 128) * 4);
  if (m->bf16) {
    int64_t pe = 0;
    pe = std::max(pe, skinny_partial_elems((int)dq, (int)d));
    pe = std::max(pe, skinny_partial_elems((int)d, (int)dq));
    pe = std::max(pe, skinny_partial_elems((int)(2 * f), (int)d));
    pe = std::max(pe, skinny_partial_elems((int)d, (int)f));
    pe = std::max(pe, skinny_partial_elems((int)V, (int)d));
    pe = std::max(pe, skinny_partial_elems((int)(dq + 2 * dkv), (int)d));
    if (m->G > 0) pe = std::max(pe, skinny_partial_elems((int)(m->G * 2 * dkv), (int)d));
    m->partial_elems = pe;
    ALLOC(m->partial, (size_t)pe * 4);
    m->attn_ws_elems = attn_rows_ws_elems((int)RY, c.max_seqlen, c.n_q_heads, c.head_dim, true);
  } else {
    m->attn_ws_elems = attn_rows_ws_elems((int)std::max(T, B), c.max_seqlen, c.n_q_heads, c.head_dim, false);
  }
  ALLOC(m->attn_ws, (size_t)m->attn_ws_elems * 4);
  if (m->bf16) {
    m->gemm_ws_elems = gemm_bf16_ws_elems();
    ALLOC(m->gemm_ws, (size_t)m->gemm_ws_elems * 4);
    ALLOC(m->rrow, T * 4);
    ALLOC(m->ssp, T * (d / 16) * 4);
  }
  m->kv8 = c.kv_dtype == SKV_KV_FP8;
  if (m->kv8) {
    const size_t T16 = round_up(T, kBlockSize);
    m->stage_v = (int64_t)(T16 * dkv);
    m->stage_group = 2 * m->stage_v;
    ALLOC(m->kv_stage, (size_t)std::max(m->G, 1) * m->stage_group * 2);
    ALLOC(m->tok_iota, T * 4);
  }
#undef ALLOC

  // the panel padding rows of the activations are read (never stored) by
  // the GEMMs: start them at zero so they hold finite values
  if (hipMemset(m->act, 0, Tp * acols * E) != hipSuccess || hipMemset(m->obuf, 0, Tp * ocols * E) != hipSuccess ||
      hipMemset(m->hbuf, 0, Tp * f * E) != hipSuccess || hipDeviceSynchronize() != hipSuccess)
    return bail(fail(SKV_ERR_HIP, "clearing the activation buffers failed"));

  // RoPE tables: angle p * theta^(-2i/dh) in double, cos/sin rounded to fp32
  {
    std::vector<float> cs((size_t)c.max_seqlen * half), sn((size_t)c.max_seqlen * half);
    for (size_t i = 0; i < half; ++i) {
      const double inv = pow((double)c.rope_theta, -2.0 * (double)i / (double)c.head_dim);
      for (size_t p = 0; p < (size_t)c.max_seqlen; ++p) {
        const double a = (double)p * inv;
        cs[p * half + i] = (float)cos(a);
        sn[p * half + i] = (float)sin(a);
      }
    }
    if (hipMemcpy(m->rope_cos, cs.data(), cs.size() * 4, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(m->rope_sin, sn.data(), sn.size() * 4, hipMemcpyHostToDevice) != hipSuccess)
      return bail(fail(SKV_ERR_HIP, "uploading RoPE tables failed"));
    if (m->kv8) {
      std::vector<int32_t> ti(T);
      for (size_t t = 0; t < T; ++t) ti[t] = (int32_t)t;
      if (hipMemcpy(m->tok_iota, ti.data(), T * 4, hipMemcpyHostToDevice) != hipSuccess)
        return bail(fail(SKV_ERR_HIP, "uploading token indices failed"));
    }
    std::vector<int32_t> io(B);
    for (size_t b = 0; b < B; ++b) io[b] = (int32_t)b;
    if (hipMemcpy(m->iota, io.data(), B * 4, hipMemcpyHostToDevice) != hipSuccess)
      return bail(fail(SKV_ERR_HIP, "upload failed"));
  }
  *out = m;
  return SKV_OK;
}

void skv_model_destroy(skv_model* m) {
  if (!m) return;
  for (auto& r : m->prof) {
    hipEventDestroy(r.a);
    hipEventDestroy(r.b);
  }
  for (void* p : m->allocs) (void)hipFree(p);
  delete m;
}

static skv_status copy_in(void* dst, const void* src, size_t bytes, const char* what) {
  if (!src) return fail(SKV_ERR_INVALID_ARG, std::string(what) + " is NULL");
  SKV_HIP(hipMemcpy(dst, src, bytes, hipMemcpyDefault));
  return SKV_OK;
}

static skv_status gain_to_f32(skv_model* m, const void* src, float* dst, const char* what) {
  const size_t d = m->cfg.d_model;
  SKV_TRY(copy_in(m->gamma_stage, src, d * m->esz, what));
  if (m->bf16)
    SKV_HIP(launch_to_f32<bf16_t>((const bf16_t*)m->gamma_stage, (int64_t)d, dst, 0));
  else
    SKV_HIP(launch_to_f32<float>((const float*)m->gamma_stage, (int64_t)d, dst, 0));
  SKV_HIP(hipDeviceSynchronize());
  return SKV_OK;
}

// Copy a row-major host/device matrix into `dst`, either as is
// (panel_rows == 0) or through the staging buffer into the panel layout,
// in chunks of whole panels that fit the staging buffer.  Values are copied
// unchanged.
static skv_status load_matrix(skv_model* m, void* dst, const void* src, size_t rows, size_t cols, int panel_rows,
                              const char* what) {
  const size_t row_bytes = cols * m->esz;
  if (!panel_rows) return copy_in(dst, src, rows * row_bytes, what);
  if (!src) return fail(SKV_ERR_INVALID_ARG, std::string(what) + " is NULL");
  const size_t chunk = m->staging_bytes / row_bytes / panel_rows * panel_rows;
  if (chunk == 0) return fail(SKV_ERR_UNSUPPORTED, "staging buffer smaller than one panel");
  for (size_t r0 = 0; r0 < rows; r0 += chunk) {
    const size_t n = std::min(chunk, rows - r0);
    SKV_TRY(copy_in(m->staging, (const char*)src + r0 * row_bytes, n * row_bytes, what));
    SKV_HIP(launch_to_panels((const bf16_t*)m->staging, (int)n, (int)cols, panel_rows,
                             (bf16_t*)dst + r0 * cols, 0));
    SKV_HIP(hipDeviceSynchronize());
  }
  return SKV_OK;
}

// The panel layout of [W | W] (rows x 2K, the B operand of a split-bf16
// GEMM) from the row-major W (rows x K) at the start of the staging buffer;
// the doubled rows are built in the staging buffer after W.
static skv_status load_doubled(skv_model* m, void* dst, size_t rows, size_t K) {
  const size_t E = m->esz;
  if (3 * rows * K * E > m->staging_bytes) return fail(SKV_ERR_UNSUPPORTED, "staging buffer too small to double W");
  char* src = (char*)m->staging;
  char* dbl = src + rows * K * E;
  SKV_HIP(hipMemcpy2D(dbl, 2 * K * E, src, K * E, K * E, rows, hipMemcpyDeviceToDevice));
  SKV_HIP(hipMemcpy2D(dbl + K * E, 2 * K * E, src, K * E, K * E, rows, hipMemcpyDeviceToDevice));
  SKV_HIP(launch_to_panels((const bf16_t*)dbl, (int)rows, (int)(2 * K), kPanelRows, (bf16_t*)dst, 0));
  SKV_HIP(hipDeviceSynchronize());
  return SKV_OK;
}

skv_status skv_model_load_globals(skv_model* m, const void* embed, const void* final_norm, const void* lm_head) {
  if (!m) return fail(SKV_ERR_INVALID_ARG, "model is NULL");
  const size_t d = m->cfg.d_model, V = m->cfg.vocab;
  SKV_TRY(copy_in(m->embed, embed, V * d * m->esz, "embed"));
  SKV_TRY(gain_to_f32(m, final_norm, m->final_norm, "final_norm"));
  // bf16: the LM head takes bf16(y * final gain) and scales its products by
  // the row's RMSNorm factor
  SKV_TRY(load_matrix(m, m->lm_head, lm_head, V, d, m->bf16 ? kSkinnyPanelRows : 0, "lm_head"));
  m->globals_loaded = true;
  return SKV_OK;
}

skv_status skv_model_load_layer(skv_model* m, int32_t layer, const skv_layer_weights* w) {
  if (!m || !w) return fail(SKV_ERR_INVALID_ARG, "NULL argument");
  const auto& c = m->cfg;
  if (layer < 1 || layer > c.n_layers) return fail(SKV_ERR_INVALID_ARG, "layer outside 1..n_layers");
  LayerDev& L = m->layers[layer - 1];
  const size_t d = c.d_model, dq = m->dq, dkv = m->dkv, f = c.ffn_dim, E = m->esz;
  SKV_TRY(gain_to_f32(m, w->ffn_norm, L.ffn_norm, "ffn_norm"));
  SKV_TRY(gain_to_f32(m, w->attn_norm, L.attn_norm, "attn_norm"));  // leaves gamma_stage = attn gain
  if (layer <= c.swiftkv_l) {
    // [wq; wk; wv] concatenated row-major, then (bf16) into panels
    char* dst = L.panel_rows ? (char*)m->staging : (char*)L.wqkv;
    SKV_TRY(copy_in(dst, w->wq, dq * d * E, "wq"));
    SKV_TRY(copy_in(dst + dq * d * E, w->wk, dkv * d * E, "wk"));
    SKV_TRY(copy_in(dst + (dq + dkv) * d * E, w->wv, dkv * d * E, "wv"));
    if (L.panel_rows) {
      SKV_HIP(launch_to_panels((const bf16_t*)m->staging, (int)(dq + 2 * dkv), (int)d, L.panel_rows,
                               (bf16_t*)L.wqkv, 0));
      SKV_HIP(hipDeviceSynchronize());
      if (layer == 1 && m->split1) SKV_TRY(load_doubled(m, L.wqkv2, dq + 2 * dkv, d));
    }
  } else {
    SKV_TRY(load_matrix(m, L.wqkv, w->wq, dq, d, L.panel_rows, "wq"));
    if (is_representative(c, layer)) {
      // fold this layer's input-RMSNorm gain into its K and V rows (in place
      // in the staging buffer), then store them as this group's block of the
      // skipped-layer projection
      const int grp = (layer - c.swiftkv_l - 1) / c.acrosskv_g;
      SKV_TRY(copy_in(m->staging, w->wk, dkv * d * E, "wk"));
      SKV_TRY(copy_in((char*)m->staging + dkv * d * E, w->wv, dkv * d * E, "wv"));
      if (m->bf16) {
        // 2 dkv = 256 * hkv rows: every group starts on a panel boundary
        bf16_t* dst = (bf16_t*)m->wkv_skip + (size_t)grp * 2 * dkv * d;
        SKV_HIP(launch_fold_rows<bf16_t>((const bf16_t*)m->staging, (const bf16_t*)m->gamma_stage, (int)(2 * dkv),
                                         (int)d, (bf16_t*)m->staging, 0));
        SKV_HIP(launch_to_panels((const bf16_t*)m->staging, (int)(2 * dkv), (int)d, kPanelRows, dst, 0));
      } else {
        float* dst = (float*)m->wkv_skip + (size_t)grp * 2 * dkv * d;
        SKV_HIP(launch_fold_rows<float>((const float*)m->staging, (const float*)m->gamma_stage, (int)(2 * dkv),
                                        (int)d, dst, 0));
      }
      SKV_HIP(hipDeviceSynchronize());
    }
  }
  SKV_TRY(load_matrix(m, L.wo, w->wo, d, dq, L.panel_rows, "wo"));
  if (layer == 1 && m->split1) {
    SKV_TRY(copy_in(m->staging, w->wo, d * dq * E, "wo"));
    SKV_TRY(load_doubled(m, L.wo2, d, dq));
  }
  SKV_TRY(load_matrix(m, L.wdown, w->w_down, d, f, L.panel_rows, "w_down"));
  // gate/up: interleave rows in blocks of P_mlp into L.wgu (row-major), then
  // (bf16) into the layer's panel layout through the staging buffer
  SKV_TRY(copy_in(m->staging, w->w_gate, f * d * E, "w_gate"));
  SKV_TRY(copy_in((char*)m->staging + f * d * E, w->w_up, f * d * E, "w_up"));
  if (m->bf16)
    SKV_HIP(launch_interleave<bf16_t>((const bf16_t*)m->staging, (const bf16_t*)m->staging + f * d, (int)f, (int)d,
                                      m->p_mlp, (bf16_t*)L.wgu, 0));
  else
    SKV_HIP(launch_interleave<float>((const float*)m->staging, (const float*)m->staging + f * d, (int)f, (int)d,
                                     m->p_mlp, (float*)L.wgu, 0));
  if (L.panel_rows) {
    SKV_HIP(launch_to_panels((const bf16_t*)L.wgu, (int)(2 * f), (int)d, L.panel_rows, (bf16_t*)m->staging, 0));
    SKV_HIP(hipMemcpyAsync(L.wgu, m->staging, round_up(2 * f, 256) * d * E, hipMemcpyDeviceToDevice, 0));
  }
  SKV_HIP(hipDeviceSynchronize());
  L.loaded = true;
  return SKV_OK;
}

int32_t skv_num_kv_slots(const skv_model* m) { return m ? m->cfg.swiftkv_l + m->G : 0; }

skv_status skv_kv_cache_create(const skv_model* m, int32_t num_blocks, int32_t block_size, skv_kv_cache** out) {
  if (!m || !out) return fail(SKV_ERR_INVALID_ARG, "NULL argument");
  *out = nullptr;
  if (block_size != kBlockSize) return fail(SKV_ERR_UNSUPPORTED, "block_size must be 16");
  if (num_blocks < 1) return fail(SKV_ERR_INVALID_ARG, "num_blocks must be positive");
  const int n_slots = skv_num_kv_slots(m);
  const int64_t slot_elems = (int64_t)num_blocks * m->cfg.n_kv_heads * block_size * m->cfg.head_dim;
  const bool fp8 = m->kv8;
  const size_t bytes = (size_t)slot_elems * n_slots * (fp8 ? 1 : m->esz);
  const size_t sbytes = fp8 ? (size_t)n_slots * num_blocks * block_size * 4 : 0;
  void *k = nullptr, *v = nullptr;
  if (hipMalloc(&k, bytes) != hipSuccess) {
    (void)hipGetLastError();
    return fail(SKV_ERR_OOM, "KV cache allocation failed");
  }
  if (hipMalloc(&v, bytes) != hipSuccess) {
    (void)hipGetLastError();
    (void)hipFree(k);
    return fail(SKV_ERR_OOM, "KV cache allocation failed");
  }
  float *ks = nullptr, *vs = nullptr;
  if (fp8 && (hipMalloc(&ks, sbytes) != hipSuccess || hipMalloc(&vs, sbytes) != hipSuccess)) {
    (void)hipGetLastError();
    (void)hipFree(k);
    (void)hipFree(v);
    if (ks) (void)hipFree(ks);
    return fail(SKV_ERR_OOM, "KV cache scale allocation failed");
  }
  if (hipMemset(k, 0, bytes) != hipSuccess || hipMemset(v, 0, bytes) != hipSuccess ||
      (fp8 && (hipMemset(ks, 0, sbytes) != hipSuccess || hipMemset(vs, 0, sbytes) != hipSuccess)) ||
      hipDeviceSynchronize() != hipSuccess) {
    (void)hipFree(k);
    (void)hipFree(v);
    if (ks) (void)hipFree(ks);
    if (vs) (void)hipFree(vs);
    return fail(SKV_ERR_HIP, "KV cache clear failed");
  }
  void *klo = nullptr, *vlo = nullptr;
  if (m->split1 && !fp8) {
    const size_t lb = (size_t)slot_elems * m->esz;
    if (hipMalloc(&klo, lb) != hipSuccess || hipMalloc(&vlo, lb) != hipSuccess ||
        hipMemset(klo, 0, lb) != hipSuccess || hipMemset(vlo, 0, lb) != hipSuccess ||
        hipDeviceSynchronize() != hipSuccess) {
      (void)hipGetLastError();
      for (void* p : {k, v, klo, vlo})
        if (p) (void)hipFree(p);
      return fail(SKV_ERR_OOM, "KV cache low-part allocation failed");
    }
  }
  skv_kv_cache* kc = new skv_kv_cache{m, num_blocks, block_size, n_slots, k, v, slot_elems};
  kc->fp8 = fp8;
  kc->ks = ks;
  kc->vs = vs;
  kc->klo = klo;
  kc->vlo = vlo;
  *out = kc;
  return SKV_OK;
}

void skv_kv_cache_destroy(skv_kv_cache* c) {
  if (!c) return;
  (void)hipFree(c->k);
  (void)hipFree(c->v);
  if (c->ks) (void)hipFree(c->ks);
  if (c->vs) (void)hipFree(c->vs);
  if (c->klo) (void)hipFree(c->klo);
  if (c->vlo) (void)hipFree(c->vlo);
  delete c;
}

skv_status skv_kv_cache_view(const skv_kv_cache* c, int32_t layer, skv_tensor_view* k, skv_tensor_view* v) {
  if (!c || !k || !v) return fail(SKV_ERR_INVALID_ARG, "NULL argument");
  const auto& cfg = c->m->cfg;
  if (layer < 1 || layer > cfg.n_layers) return fail(SKV_ERR_INVALID_ARG, "layer outside 1..n_layers");
  const int s = slot_of_layer(cfg, layer);
  const int64_t nb = c->num_blocks, hkv = cfg.n_kv_heads, bs = c->block_size, dh = cfg.head_dim;
  const size_t off = (size_t)s * c->slot_elems * (c->fp8 ? 1 : c->m->esz);
  const int32_t dt = c->fp8 ? SKV_FP8_E4M3 : cfg.dtype;
  *k = skv_tensor_view{(char*)c->k + off, dt, 4, {nb, hkv, bs, dh}, {hkv * bs * dh, bs * dh, dh, 1}};
  *v = skv_tensor_view{(char*)c->v + off, dt, 4, {nb, hkv, bs, dh}, {hkv * bs * dh, bs * dh, dh, 1}};
  return SKV_OK;
}

skv_status skv_kv_cache_scales(const skv_kv_cache* c, int32_t layer, skv_tensor_view* k, skv_tensor_view* v) {
  if (!c || !k || !v) return fail(SKV_ERR_INVALID_ARG, "NULL argument");
  if (!c->fp8) return fail(SKV_ERR_INVALID_ARG, "the cache holds no FP8 scales");
  const auto& cfg = c->m->cfg;
  if (layer < 1 || layer > cfg.n_layers) return fail(SKV_ERR_INVALID_ARG, "layer outside 1..n_layers");
  const int64_t nb = c->num_blocks, bs = c->block_size;
  const size_t off = (size_t)slot_of_layer(cfg, layer) * nb * bs;
  *k = skv_tensor_view{c->ks + off, SKV_FP32, 2, {nb, bs, 0, 0}, {bs, 1, 0, 0}};
  *v = skv_tensor_view{c->vs + off, SKV_FP32, 2, {nb, bs, 0, 0}, {bs, 1, 0, 0}};
  return SKV_OK;
}

skv_status skv_profile_enable(skv_model* m, int32_t kernel_class, int32_t enable) {
  if (!m) return fail(SKV_ERR_INVALID_ARG, "model is NULL");
  if (kernel_class < 0 || kernel_class >= SKV_K_NUM) return fail(SKV_ERR_INVALID_ARG, "unknown kernel class");
  for (auto& r : m->prof) {
    hipEventDestroy(r.a);
    hipEventDestroy(r.b);
  }
  m->prof.clear();
  m->prof_flops = m->prof_bytes = 0;
  m->prof_class = enable ? kernel_class : -1;
  return SKV_OK;
}

skv_status skv_profile_read(skv_model* m, double* total_ms, int64_t* launches, double* flops, double* bytes) {
  if (!m || !total_ms || !launches || !flops || !bytes) return fail(SKV_ERR_INVALID_ARG, "NULL argument");
  double t = 0;
  for (auto& r : m->prof) {
    SKV_HIP(hipEventSynchronize(r.b));
    float ms = 0;
    SKV_HIP(hipEventElapsedTime(&ms, r.a, r.b));
    t += ms;
  }
  *total_ms = t;
  *launches = (int64_t)m->prof.size();
  *flops = m->prof_flops;
  *bytes = m->prof_bytes;
  return SKV_OK;
}

skv_status skv_mfma_probe(int32_t random_operands, int32_t iters, void* stream, double* tflops, double* clock_mhz,
                          int32_t* cus, double* max_clock_mhz) {
  if (iters <= 0 || iters > (1 << 22) || !tflops || !clock_mhz || !cus || !max_clock_mhz)
    return fail(SKV_ERR_INVALID_ARG, "skv_mfma_probe: iters must be in [1, 2^22] and every output non-NULL");
  int dev = 0, n = 0, khz = 0;
  SKV_HIP(hipGetDevice(&dev));
  SKV_HIP(hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev));
  SKV_HIP(hipDeviceGetAttribute(&khz, hipDeviceAttributeClockRate, dev));
  struct DevBuf {
    void* p = nullptr;
    ~DevBuf() {
      if (p) (void)hipFree(p);
    }
  } in, out, clk;
  struct Ev {
    hipEvent_t e = nullptr;
    ~Ev() {
      if (e) (void)hipEventDestroy(e);
    }
  } e0, e1;
  const size_t in_elems = 16 * 64 * 8;  // 16 fragments x 64 lanes x 8 bf16
  SKV_HIP(hipMalloc(&in.p, in_elems * 2));
  SKV_HIP(hipMalloc(&out.p, (size_t)n * 256 * 4));
  SKV_HIP(hipMalloc(&clk.p, (size_t)n * 2 * sizeof(unsigned long long)));
  // random operands: random sign and mantissa bits at magnitudes 2^-7 .. 2^-5
  // (the scale of N(0, 0.02) weights); otherwise one constant value
  std::vector<uint16_t> h(in_elems);
  uint32_t x = 0x2545F491u;
  for (auto& v : h) {
    x = x * 1664525u + 1013904223u;
    v = random_operands ? (uint16_t)(0x3c00u | ((x >> 9) & 0xffu) | ((x >> 8) & 0x8000u)) : (uint16_t)0x3c3c;
  }
  hipStream_t st = (hipStream_t)stream;
  SKV_HIP(hipMemcpyAsync(in.p, h.data(), in_elems * 2, hipMemcpyHostToDevice, st));
  SKV_HIP(hipEventCreate(&e0.e));
  SKV_HIP(hipEventCreate(&e1.e));
  // one untimed launch brings the clock to its steady state
  SKV_HIP(launch_mfma_probe((const bf16x8_t*)in.p, iters, n, (float*)out.p, (unsigned long long*)clk.p, st));
  SKV_HIP(hipEventRecord(e0.e, st));
  SKV_HIP(launch_mfma_probe((const bf16x8_t*)in.p, iters, n, (float*)out.p, (unsigned long long*)clk.p, st));
  SKV_HIP(hipEventRecord(e1.e, st));
  SKV_HIP(hipEventSynchronize(e1.e));
  float ms = 0.f;
  SKV_HIP(hipEventElapsedTime(&ms, e0.e, e1.e));
  std::vector<unsigned long long> c((size_t)n * 2);
  SKV_HIP(hipMemcpy(c.data(), clk.p, c.size() * sizeof(unsigned long long), hipMemcpyDeviceToHost));
  double mhz = 0.0;
  int used = 0;
  for (int g = 0; g < n; ++g)
    if (c[2 * g + 1] > 0) {
      mhz += (double)c[2 * g] / (double)c[2 * g + 1] * 100.0;
      ++used;
    }
  const double flops = (double)mfma_probe_flops_per_mfma() * mfma_probe_per_iter() * (double)iters * 4 * n;
  *tflops = ms > 0.f ? flops / ((double)ms * 1e9) : 0.0;
  *clock_mhz = used ? mhz / used : 0.0;
  *cus = n;
  *max_clock_mhz = khz / 1000.0;
  return SKV_OK;
}

}  // extern "C"

namespace {

// Scratch of one call: the buffers the row path and the last-token path
// write (the model's own workspace, or a caller-independent static array).
struct Work {
  float* x = nullptr;  // fp32 residual stream of the new tokens [T, d]
  float* y = nullptr;  // last tokens' residual stream [B, d]
  void* ya = nullptr;  // row-major bf16 / fp32 rows [RY, d], [RY, dq], [RY, dq], [RY, f]
  void* yq = nullptr;
  void* yo = nullptr;
  void* yh = nullptr;
  float* rss = nullptr;  // bf16: partial sums of squares [RY, d / 128]
  float* partial = nullptr;  // skinny split-K partials
  int64_t partial_elems = 0;
  float* attn_ws = nullptr;  // row attention chunk partials
  int32_t *pos = nullptr, *slot = nullptr, *seq = nullptr;  // [T]
  int32_t *last_pos = nullptr, *last_row = nullptr;          // [B]
  bool profile = true;  // the profiling hook may record events
};

Work model_work(skv_model* m) {
  Work w;
  w.x = m->x;
  w.y = m->y;
  w.ya = m->ya;
  w.yq = m->yq;
  w.yo = m->yo;
  w.yh = m->yh;
  w.rss = m->rss;
  w.partial = m->partial;
  w.partial_elems = m->partial_elems;
  w.attn_ws = m->attn_ws;
  w.pos = m->pos;
  w.slot = m->slot;
  w.seq = m->seq;
  w.last_pos = m->last_pos;
  w.last_row = m->last_row;
  return w;
}

// Host-side facts about one call's batch (validated before anything is enqueued).
struct StepInfo {
  const int32_t* ctx_dev = nullptr;  // device [batch] cached positions per sequence, NULL = none
  int max_new = 0;                   // longest run of new tokens
  int max_total = 0;                 // longest cached + new
  double attn_flops = 0;             // 4 * keys * dh * hq summed over the new tokens
  double ctx_tokens = 0;             // keys attended by the last tokens, summed
  bool need_last = true;             // some sequence needs its next-token logits
};

template <typename T>
skv_status run_step(skv_model* m, skv_kv_cache* kc, const skv_batch* bt, const StepInfo& si, float* logits,
                    hipStream_t s, const Work& w) {
  const auto& c = m->cfg;
  skv_model* pm = w.profile ? m : nullptr;  // the profiling hook's model (NULL: no events)
  const int T_ = bt->total_tokens, B = bt->batch, d = c.d_model, dq = m->dq, dkv = m->dkv, f = c.ffn_dim,
            V = c.vocab, dh = c.head_dim, hq = c.n_q_heads, l = c.swiftkv_l, L = c.n_layers;
  const int P = dh / 2;
  const double E = (double)m->esz;
  T* act = (T*)m->act;
  T* qbuf = (T*)m->qbuf;
  T* obuf = (T*)m->obuf;
  T* hbuf = (T*)m->hbuf;
  T* ya = (T*)w.ya;
  T* yq = (T*)w.yq;
  T* yo = (T*)w.yo;
  T* yh = (T*)w.yh;
  auto slot_of = [&](int s_) {
    return CacheSlot<T>{(T*)kc->k + (int64_t)s_ * kc->slot_elems, (T*)kc->v + (int64_t)s_ * kc->slot_elems,
                        c.n_kv_heads, dh};
  };
  constexpr bool kBf16 = sizeof(T) == 2;
  // FP8 cache: K/V epilogues write the staging area (physical slot = token
  // index), kv_quant moves the rows into the cache, attention reads codes
  const bool kv8 = kc->fp8;
  const int64_t nb16 = (int64_t)kc->num_blocks * kBlockSize;
  auto slot8_of = [&](int s_) {
    return Fp8Slot{(uint8_t*)kc->k + (int64_t)s_ * kc->slot_elems, (uint8_t*)kc->v + (int64_t)s_ * kc->slot_elems,
                   kc->ks + s_ * nb16, kc->vs + s_ * nb16, c.n_kv_heads, dh};
  };
  const CacheSlot<T> stage{(T*)m->kv_stage, (T*)m->kv_stage + m->stage_v, c.n_kv_heads, dh};
  const int32_t* kv_slot = kv8 ? m->tok_iota : w.slot;  // where the K/V epilogues write
  auto quantize = [&](int rows, int ngroups, int first_slot) -> skv_status {
    SKV_HIP(launch_kv_quant(m->kv_stage, m->stage_group, m->stage_v, rows, ngroups, w.slot, slot8_of(first_slot),
                            kc->slot_elems, nb16, s));
    return SKV_OK;
  };
  // bf16 batches of at most kRowPathMax new tokens (decode steps, short
  // chunks) run layers 1..l like the last-token path: row-major
  // activations, the split-K skinny GEMM and per-row attention, instead of
  // 256-row GEMM tiles that would be mostly padding.
  const bool rows_path = kBf16 && T_ <= kRowPathMax;

  // algorithmic work of the attention and last-token rows, for the profiling hook
  const double attn_bytes = (double)T_ * (2.0 * dq + 2.0 * dkv) * E;
  const double n_deep = L - l;
  const double last_flops = n_deep * (B * (4.0 * d * dq + 6.0 * d * f) + 4.0 * si.ctx_tokens * dh * hq) + 2.0 * d * V * B;
  const double last_bytes = n_deep * ((2.0 * dq * d + 3.0 * f * d) * E + si.ctx_tokens * 2.0 * dkv * E) + (double)V * d * E;

  SKV_HIP(launch_meta(bt->cu_seqlens, si.ctx_dev, bt->block_tables, B, bt->max_blocks_per_seq, kc->num_blocks, T_,
                      w.pos, w.slot, w.last_pos, w.last_row, s));
  if (!kBf16 || rows_path) SKV_HIP(launch_token_seq(bt->cu_seqlens, B, T_, w.seq, s));
  SKV_HIP(launch_embed<T>(bt->token_ids, (const T*)m->embed, V, d, T_, w.x, s));
  // bf16: the gain the projections of layer j (1-based) apply to their
  // input, folded into the bf16 copy of x that precedes them (layer L + 1:
  // the final norm); the skipped-layer K/V projection has its gains in its
  // weights, so the input after layer l takes none
  auto gain_before = [&](int j) -> const float* {
    if (j > L) return m->final_norm;
    return m->layers[j - 1].attn_norm;
  };
  if (kBf16 && rows_path)
    SKV_HIP(launch_rows_act_ss(w.x, nullptr, l > 0 ? gain_before(1) : nullptr, T_, d, nullptr, (bf16_t*)ya, w.rss,
                               s));

  // One layer over a few rows held row-major (the last tokens at layers
  // l+1..L; every new token of a short bf16 batch at layers 1..l).  x: the
  // rows' residual stream; with_kv: the QKV product also yields K/V, written
  // to cache slot cs at slot[row]; next_gain: the gain of the RMSNorm that
  // the rows meet after this layer (bf16).
  auto row_layer = [&](const LayerDev& Ly, int cache_slot, int rows, float* x, const int32_t* row_seq,
                       const int32_t* row_pos, bool with_kv, int max_ctx, const float* next_gain) -> skv_status {
    const CacheSlot<T> cs = slot_of(cache_slot);
    const int nq = with_kv ? dq + 2 * dkv : dq;
    EpiQKV<T> eq{yq, kv8 ? stage : cs, row_pos, with_kv ? kv_slot : nullptr, m->rope_cos, m->rope_sin, dq, dkv, dh, P};
    if (with_kv && cache_slot == 0 && kc->klo) {  // keep layer 1's low parts for the split prompt attention
      eq.k_lo = (T*)kc->klo;
      eq.v_lo = (T*)kc->vlo;
    }
    EpiSwiGLU<T> esw{yh, f, m->p_mlp};
    // bf16: ya holds bf16(x * gain) and rss the partial sums of squares of
    // x on entry and on exit; each normalised product scales by 1 / rms(x)
    // in its finalize pass
    SkinnyRowNorm rn_in, rn_out;
    if constexpr (kBf16) {
      rn_in.ss_in = w.rss;
      rn_in.nparts = (int)(d / 128);
      rn_in.inv_d = 1.0f / (float)d;
      rn_in.eps = c.rms_eps;
      rn_out.ss_out = w.rss;
      SKV_HIP(launch_skinny_bf16((const bf16_t*)ya, d, (const bf16_t*)Ly.wqkv, Ly.panel_rows, rows, nq, d, w.partial,
                                 w.partial_elems, eq, s, rn_in));
    } else {
      SKV_HIP(launch_rmsnorm<T>(x, nullptr, Ly.attn_norm, rows, d, c.rms_eps, ya, s));
      if (P == 16) {
        SKV_HIP((launch_gemm_f32<16>((const float*)ya, d, (const float*)Ly.wqkv, d, rows, nq, d, eq, s)));
      } else if (P == 32) {
        SKV_HIP((launch_gemm_f32<32>((const float*)ya, d, (const float*)Ly.wqkv, d, rows, nq, d, eq, s)));
      } else {
        SKV_HIP((launch_gemm_f32<64>((const float*)ya, d, (const float*)Ly.wqkv, d, rows, nq, d, eq, s)));
      }
    }
    if (with_kv && kv8) SKV_TRY(quantize(rows, 1, cache_slot));
    if (kv8) {
      if constexpr (kBf16)
        SKV_HIP(launch_attn_rows_fp8((const bf16_t*)yq, slot8_of(cache_slot), row_seq, row_pos, bt->block_tables,
                                     bt->max_blocks_per_seq, rows, max_ctx, hq, w.attn_ws, (bf16_t*)yo, s));
    } else {
      SKV_HIP(launch_attn_rows<T>(yq, cs, row_seq, row_pos, bt->block_tables, bt->max_blocks_per_seq, rows, max_ctx,
                                  hq, w.attn_ws, yo, s));
    }
    if constexpr (kBf16) {
      EpiResidualRow er_o{x, d, (bf16_t*)ya, Ly.ffn_norm};
      EpiResidualRow er_d{x, d, (bf16_t*)ya, next_gain};
      SKV_HIP(launch_skinny_bf16((const bf16_t*)yo, dq, (const bf16_t*)Ly.wo, Ly.panel_rows, rows, d, dq, w.partial,
                                 w.partial_elems, er_o, s, rn_out));
      SKV_HIP(launch_skinny_bf16((const bf16_t*)ya, d, (const bf16_t*)Ly.wgu, Ly.panel_rows, rows, 2 * f, d, w.partial,
                                 w.partial_elems, esw, s, rn_in));
      SKV_HIP(launch_skinny_bf16((const bf16_t*)yh, f, (const bf16_t*)Ly.wdown, Ly.panel_rows, rows, d, f, w.partial,
                                 w.partial_elems, er_d, s, rn_out));
    } else {
      EpiResidual er{x, d, 16};
      SKV_HIP((launch_gemm_f32<16>((const float*)yo, dq, (const float*)Ly.wo, dq, rows, d, dq, er, s)));
      SKV_HIP(launch_rmsnorm<T>(x, nullptr, Ly.ffn_norm, rows, d, c.rms_eps, ya, s));
      SKV_HIP((launch_gemm_f32<16>((const float*)ya, d, (const float*)Ly.wgu, d, rows, 2 * f, d, esw, s)));
      SKV_HIP((launch_gemm_f32<16>((const float*)yh, f, (const float*)Ly.wdown, f, rows, d, f, er, s)));
    }
    return SKV_OK;
  };

  // bf16 prompt-token GEMMs take bf16(x * gain) (`act`) and apply the row's
  // RMSNorm factor (rrow) in their epilogues.  The residual epilogues write
  // the next act and the partial sums of squares for rrow.  Here: x_1's.
  const bool panel_path = kBf16 && !rows_path;
  auto next_rrow = [&]() -> skv_status {
    Prof p(pm, SKV_K_RMSNORM, s, 0, (double)T_ * d / 16 * 4 + T_ * 4.0);
    SKV_HIP(launch_rms_from_partials(m->ssp, T_, d, c.rms_eps, m->rrow, s));
    return SKV_OK;
  };
  if (panel_path && (l > 0 || m->G > 0)) {
    Prof p(pm, SKV_K_RMSNORM, s, 0, (double)T_ * d * (4 + E));
    SKV_HIP(launch_rows_rms_panel(w.x, l > 0 ? gain_before(1) : nullptr, T_, d, c.rms_eps, m->split1, (bf16_t*)act,
                                  m->rrow, s));
  }
  const float* rrow = panel_path ? m->rrow : nullptr;

  // ---- layers 1..l for every new token
  for (int i = 1; i <= l; ++i) {
    const LayerDev& Ly = m->layers[i - 1];
    CacheSlot<T> cs = slot_of(i - 1);
    if (rows_path) {
      SKV_TRY(row_layer(Ly, i - 1, T_, w.x, w.seq, w.pos, true, si.max_total, i < l ? gain_before(i + 1) : nullptr));
      continue;
    }
    if constexpr (!kBf16) {
      Prof p(pm, SKV_K_RMSNORM, s, 0, (double)T_ * d * (4 + E));
      SKV_HIP(launch_rmsnorm<T>(w.x, nullptr, Ly.attn_norm, T_, d, c.rms_eps, act, s));
    }
    // split-bf16 layer 1: the QKV GEMM contracts over both parts of its
    // input (K doubled); with a bf16 cache the attention computes with both
    // parts and the O GEMM contracts over both parts of the attention output
    const bool split = kBf16 && i == 1 && m->split1;
    const bool split_attn = split && kc->klo != nullptr;
    {
      const int N = dq + 2 * dkv;
      EpiQKV<T> epi{qbuf, kv8 ? stage : cs, w.pos, kv_slot, m->rope_cos, m->rope_sin, dq, dkv, dh, P, rrow};
      if (split_attn) {
        epi.q_lo = (T*)m->qlo;
        epi.k_lo = (T*)kc->klo;
        epi.v_lo = (T*)kc->vlo;
      }
      Prof p(pm, SKV_K_GEMM_QKV, s, 2.0 * T_ * N * d, gemm_bytes(T_, N, d, E, E));
      if constexpr (kBf16)
        SKV_HIP(launch_gemm_bf16((const bf16_t*)act, (const bf16_t*)(split ? Ly.wqkv2 : Ly.wqkv), T_, N,
                                 split ? 2 * d : d, epi, m->gemm_ws, m->gemm_ws_elems, s));
      else if (P == 16)
        SKV_HIP((launch_gemm_f32<16>((const float*)act, d, (const float*)Ly.wqkv, d, T_, N, d, epi, s)));
      else if (P == 32)
        SKV_HIP((launch_gemm_f32<32>((const float*)act, d, (const float*)Ly.wqkv, d, T_, N, d, epi, s)));
      else
        SKV_HIP((launch_gemm_f32<64>((const float*)act, d, (const float*)Ly.wqkv, d, T_, N, d, epi, s)));
    }
    if (kv8) SKV_TRY(quantize(T_, 1, i - 1));
    {
      Prof p(pm, split_attn ? SKV_K_ATTN_PREFILL_SPLIT : SKV_K_ATTN_PREFILL, s, si.attn_flops, attn_bytes);
      if (kv8) {
        if constexpr (kBf16)
          SKV_HIP(launch_attn_prefill_fp8((const bf16_t*)qbuf, slot8_of(i - 1), bt->cu_seqlens, si.ctx_dev,
                                          bt->block_tables, bt->max_blocks_per_seq, B, si.max_new, hq, (bf16_t*)obuf,
                                          s));
      } else if constexpr (kBf16) {
        if (split_attn)
          SKV_HIP(launch_attn_prefill_split((const bf16_t*)qbuf, (const bf16_t*)m->qlo, cs,
                                            CacheSlot<bf16_t>{(bf16_t*)kc->klo, (bf16_t*)kc->vlo, c.n_kv_heads, dh},
                                            bt->cu_seqlens, si.ctx_dev, bt->block_tables, bt->max_blocks_per_seq, B,
                                            si.max_new, hq, (bf16_t*)obuf, s));
        else
          SKV_HIP(launch_attn_prefill_bf16((const bf16_t*)qbuf, cs, bt->cu_seqlens, si.ctx_dev, bt->block_tables,
                                           bt->max_blocks_per_seq, B, si.max_new, hq, (bf16_t*)obuf, s));
      }
      else
        SKV_HIP(launch_attn_rows<T>(qbuf, cs, w.seq, w.pos, bt->block_tables, bt->max_blocks_per_seq, T_,
                                    si.max_total, hq, w.attn_ws, obuf, s));
    }
    {
      EpiResidual epi{w.x, d, kBf16 ? 64 : 16, kBf16 ? (bf16_t*)act : nullptr, kBf16 ? m->ssp : nullptr,
                      kBf16 ? Ly.ffn_norm : nullptr};
      Prof p(pm, SKV_K_GEMM_O, s, 2.0 * T_ * d * dq, gemm_bytes(T_, d, dq, E, kBf16 ? 8 + 2 + 0.25 : 8));
      if constexpr (kBf16)
        SKV_HIP(launch_gemm_bf16((const bf16_t*)obuf, (const bf16_t*)(split_attn ? Ly.wo2 : Ly.wo), T_, d,
                                 split_attn ? 2 * dq : dq, epi, m->gemm_ws, m->gemm_ws_elems, s));
      else
        SKV_HIP((launch_gemm_f32<16>((const float*)obuf, dq, (const float*)Ly.wo, dq, T_, d, dq, epi, s)));
    }
    if constexpr (kBf16) {
      SKV_TRY(next_rrow());
    } else {
      Prof p(pm, SKV_K_RMSNORM, s, 0, (double)T_ * d * (4 + E));
      SKV_HIP(launch_rmsnorm<T>(w.x, nullptr, Ly.ffn_norm, T_, d, c.rms_eps, act, s));
    }
    {
      Prof p(pm, SKV_K_GEMM_GATEUP, s, 2.0 * T_ * 2 * f * d, gemm_bytes(T_, 2.0 * f, d, E, 0) + (double)T_ * f * E);
      if constexpr (kBf16) {
        EpiSwiGLUPanel epi{(bf16_t*)hbuf, f, rrow};
        SKV_HIP(launch_gemm_bf16((const bf16_t*)act, (const bf16_t*)Ly.wgu, T_, 2 * f, d, epi, m->gemm_ws, m->gemm_ws_elems, s));
      } else {
        EpiSwiGLU<T> epi{hbuf, f, m->p_mlp};
        SKV_HIP((launch_gemm_f32<16>((const float*)act, d, (const float*)Ly.wgu, d, T_, 2 * f, d, epi, s)));
      }
    }
    {
      EpiResidual epi{w.x, d, kBf16 ? 64 : 16, kBf16 ? (bf16_t*)act : nullptr, kBf16 ? m->ssp : nullptr,
                      (kBf16 && i < l) ? gain_before(i + 1) : nullptr};
      Prof p(pm, SKV_K_GEMM_DOWN, s, 2.0 * T_ * d * f, gemm_bytes(T_, d, f, E, kBf16 ? 8 + 2 + 0.25 : 8));
      if constexpr (kBf16)
        SKV_HIP(launch_gemm_bf16((const bf16_t*)hbuf, (const bf16_t*)Ly.wdown, T_, d, f, epi, m->gemm_ws, m->gemm_ws_elems, s));
      else
        SKV_HIP((launch_gemm_f32<16>((const float*)hbuf, f, (const float*)Ly.wdown, f, T_, d, f, epi, s)));
    }
    if constexpr (kBf16) SKV_TRY(next_rrow());
  }

  // ---- boundary: KV of every skipped layer / AcrossKV group from x_{l+1}
  if (m->G > 0) {
    if constexpr (!kBf16) {
      // x * r, gains folded into W~ (bf16: act / ya already hold bf16(x_{l+1}) without a gain, with rrow / rss)
      Prof p(pm, SKV_K_RMSNORM, s, 0, (double)T_ * d * (4 + E));
      SKV_HIP(launch_rmsnorm<T>(w.x, nullptr, nullptr, T_, d, c.rms_eps, act, s));
    }
    CacheSlot<T> first = kv8 ? stage : slot_of(l);
    const int N = m->G * 2 * dkv;
    EpiKVSkip<T> epi{first.k, first.v, kv8 ? m->stage_group : kc->slot_elems, w.pos, kv_slot, m->rope_cos,
                     m->rope_sin, dkv, dh, P, c.n_kv_heads, rrow};
    Prof p(pm, SKV_K_GEMM_KVSKIP, s, 2.0 * T_ * N * d, gemm_bytes(T_, N, d, E, E));
    if constexpr (kBf16) {
      if (rows_path) {
        SkinnyRowNorm rn;
        rn.ss_in = w.rss;
        rn.nparts = (int)(d / 128);
        rn.inv_d = 1.0f / (float)d;
        rn.eps = c.rms_eps;
        SKV_HIP(launch_skinny_bf16((const bf16_t*)ya, d, (const bf16_t*)m->wkv_skip, kPanelRows, T_, N, d, w.partial,
                                   w.partial_elems, epi, s, rn));
      }
      else
        SKV_HIP(launch_gemm_bf16((const bf16_t*)act, (const bf16_t*)m->wkv_skip, T_, N, d, epi, m->gemm_ws,
                                 m->gemm_ws_elems, s));
    } else if (P == 16) {
      SKV_HIP((launch_gemm_f32<16>((const float*)act, d, (const float*)m->wkv_skip, d, T_, N, d, epi, s)));
    } else if (P == 32) {
      SKV_HIP((launch_gemm_f32<32>((const float*)act, d, (const float*)m->wkv_skip, d, T_, N, d, epi, s)));
    } else {
      SKV_HIP((launch_gemm_f32<64>((const float*)act, d, (const float*)m->wkv_skip, d, T_, N, d, epi, s)));
    }
    if (kv8) SKV_TRY(quantize(T_, m->G, l));
  }

  // ---- last new token of each sequence through layers l+1..L, then the LM
  // head (only a prompt's last token goes past layer l: a call of unfinished
  // chunks alone stops here)
  if (!si.need_last) return SKV_OK;
  Prof plast(pm, SKV_K_LAST_TOKEN, s, last_flops, last_bytes);
  if constexpr (kBf16)
    SKV_HIP(launch_rows_act_ss(w.x, w.last_row, gain_before(l + 1), B, d, w.y, (bf16_t*)ya, w.rss, s));
  else
    SKV_HIP(launch_gather_rows(w.x, w.last_row, B, d, w.y, s));
  for (int j = l + 1; j <= L; ++j)
    SKV_TRY(row_layer(m->layers[j - 1], slot_of_layer(c, j), B, w.y, m->iota, w.last_pos, false, si.max_total,
                      gain_before(j + 1)));
  EpiStoreF32 el{logits, V, kBf16 ? 64 : 16};
  if constexpr (kBf16) {
    // final RMSNorm: ya = bf16(y * final gain), the partials of y in rss
    SkinnyRowNorm rn;
    rn.ss_in = w.rss;
    rn.nparts = (int)(d / 128);
    rn.inv_d = 1.0f / (float)d;
    rn.eps = c.rms_eps;
    SKV_HIP(launch_skinny_bf16((const bf16_t*)ya, d, (const bf16_t*)m->lm_head, kSkinnyPanelRows, B, V, d, w.partial,
                               w.partial_elems, el, s, rn));
  } else {
    SKV_HIP(launch_rmsnorm<T>(w.y, nullptr, m->final_norm, B, d, c.rms_eps, ya, s));
    SKV_HIP((launch_gemm_f32<16>((const float*)ya, d, (const float*)m->lm_head, d, B, V, d, el, s)));
  }
  return SKV_OK;
}

}  // namespace

namespace {

// Shared argument checks of skv_prefill / skv_step / skv_step_noalloc;
// ctx_host NULL = no cached positions.  Fills si on success.
skv_status check_batch(skv_model* m, skv_kv_cache* kc, const skv_batch* bt, const int32_t* ctx_host,
                       const int32_t* ctx_dev, float* logits, StepInfo& si, const int32_t* need_host = nullptr) {
  if (!m || !kc || !bt) return fail(SKV_ERR_INVALID_ARG, "NULL argument");
  bool need_last = true;
  if (need_host) {
    if (bt->batch < 1 || bt->batch > m->cfg.max_batch)
      return fail(SKV_ERR_INVALID_ARG, "batch must lie in 1..max_batch");
    need_last = false;
    for (int b = 0; b < bt->batch; ++b) need_last = need_last || need_host[b] != 0;
  }
  if (need_last && !logits) return fail(SKV_ERR_INVALID_ARG, "NULL argument");
  if (kc->m != m) return fail(SKV_ERR_INVALID_ARG, "cache was created for another model");
  const auto& c = m->cfg;
  if (!m->globals_loaded) return fail(SKV_ERR_INVALID_ARG, "embedding / LM head not loaded");
  for (int i = 0; i < c.n_layers; ++i)
    if (!m->layers[i].loaded) return fail(SKV_ERR_INVALID_ARG, "layer " + std::to_string(i + 1) + " not loaded");
  const int B = bt->batch;
  if (B < 1 || B > c.max_batch) return fail(SKV_ERR_INVALID_ARG, "batch must lie in 1..max_batch");
  if (bt->total_tokens < 1 || bt->total_tokens > c.max_tokens)
    return fail(SKV_ERR_INVALID_ARG, "total_tokens must lie in 1..max_tokens");
  if (!bt->cu_seqlens_host || !bt->block_tables_host || !bt->token_ids || !bt->cu_seqlens || !bt->block_tables)
    return fail(SKV_ERR_INVALID_ARG, "batch arrays must be non-NULL");
  if (bt->max_blocks_per_seq < 1) return fail(SKV_ERR_INVALID_ARG, "max_blocks_per_seq must be positive");
  const int32_t* cu = bt->cu_seqlens_host;
  if (cu[0] != 0 || cu[B] != bt->total_tokens)
    return fail(SKV_ERR_INVALID_ARG, "cu_seqlens must start at 0 and end at total_tokens");
  const double dh = c.head_dim, hq = c.n_q_heads;
  si = StepInfo{};
  si.ctx_dev = ctx_dev;
  si.need_last = need_last;
  for (int b = 0; b < B; ++b) {
    const int n = cu[b + 1] - cu[b];
    const int cx = ctx_host ? ctx_host[b] : 0;
    if (n < 1) return fail(SKV_ERR_INVALID_ARG, "sequence " + std::to_string(b) + " brings no token");
    if (cx < 0) return fail(SKV_ERR_INVALID_ARG, "negative cached length");
    if ((int64_t)cx + n > c.max_seqlen) return fail(SKV_ERR_INVALID_ARG, "sequence longer than max_seqlen");
    const int tot = cx + n;
    const int nb = ceil_div(tot, kc->block_size);
    if (nb > bt->max_blocks_per_seq) return fail(SKV_ERR_INVALID_ARG, "block table too small");
    for (int i = 0; i < nb; ++i) {
      const int blk = bt->block_tables_host[(int64_t)b * bt->max_blocks_per_seq + i];
      if (blk < 0 || blk >= kc->num_blocks)
        return fail(SKV_ERR_INVALID_ARG, "block table entry outside [0, num_blocks)");
    }
    si.max_new = std::max(si.max_new, n);
    si.max_total = std::max(si.max_total, tot);
    si.attn_flops += 2.0 * dh * hq * ((double)tot * (tot + 1) - (double)cx * (cx + 1));
    si.ctx_tokens += tot;
  }
  if (bt->max_seqlen < si.max_new) return fail(SKV_ERR_INVALID_ARG, "max_seqlen smaller than the longest run");
  return SKV_OK;
}

skv_status check_and_run(skv_model* m, skv_kv_cache* kc, const skv_batch* bt, const int32_t* ctx_host,
                         const int32_t* ctx_dev, float* logits, void* stream, const int32_t* need_host = nullptr) {
  StepInfo si;
  SKV_TRY(check_batch(m, kc, bt, ctx_host, ctx_dev, logits, si, need_host));
  hipStream_t s = (hipStream_t)stream;
  const Work w = model_work(m);
  if (m->bf16) return run_step<bf16_t>(m, kc, bt, si, logits, s, w);
  return run_step<float>(m, kc, bt, si, logits, s, w);
}

}  // namespace

extern "C" skv_status skv_prefill(skv_model* m, skv_kv_cache* kc, const skv_batch* bt, float* logits,
                                  void* stream) {
  return check_and_run(m, kc, bt, nullptr, nullptr, logits, stream);
}

extern "C" skv_status skv_step(skv_model* m, skv_kv_cache* kc, const skv_step_batch* sb, float* logits,
                               void* stream) {
  if (!sb) return fail(SKV_ERR_INVALID_ARG, "NULL argument");
  if (!sb->ctx_lens_host != !sb->ctx_lens)
    return fail(SKV_ERR_INVALID_ARG, "ctx_lens_host and ctx_lens must both be set or both be NULL");
  return check_and_run(m, kc, &sb->tokens, sb->ctx_lens_host, sb->ctx_lens, logits, stream, sb->need_logits_host);
}

extern "C" skv_status skv_step_noalloc(skv_model* m, skv_kv_cache* kc, const skv_step_batch* sb, float* logits,
                                      void* stream) {
  if (!sb) return fail(SKV_ERR_INVALID_ARG, "NULL argument");
  if (!sb->ctx_lens_host != !sb->ctx_lens)
    return fail(SKV_ERR_INVALID_ARG, "ctx_lens_host and ctx_lens must both be set or both be NULL");
  StepInfo si;
  SKV_TRY(check_batch(m, kc, &sb->tokens, sb->ctx_lens_host, sb->ctx_lens, logits, si, sb->need_logits_host));
  if (!m->bf16) return fail(SKV_ERR_UNSUPPORTED, "skv_step_noalloc needs a bf16 model");
  if (kc->fp8) return fail(SKV_ERR_UNSUPPORTED, "skv_step_noalloc does not take an FP8 cache");
  const skv_batch* bt = &sb->tokens;
  if (bt->total_tokens > kRowPathMax)
    return fail(SKV_ERR_INVALID_ARG, "skv_step_noalloc takes at most " + std::to_string(kRowPathMax) +
                                         " new tokens per call");
  char* base = (char*)noalloc_scratch();
  if (!base) return fail(SKV_ERR_INVALID_ARG, "no model was created on the current device");
  const auto& c = m->cfg;
  const size_t T = bt->total_tokens, B = bt->batch, RY = std::max(T, B), d = c.d_model, dq = m->dq, dkv = m->dkv,
               f = c.ffn_dim, V = c.vocab;
  int64_t pe = 0;
  for (const auto& nk : {std::make_pair(dq + 2 * dkv, d), std::make_pair(dq, d), std::make_pair(d, dq),
                         std::make_pair(2 * f, d), std::make_pair(d, f), std::make_pair(V, d),
                         std::make_pair((size_t)std::max(m->G, 1) * 2 * dkv, d)})
    pe = std::max(pe, skinny_partial_elems((int)nk.first, (int)nk.second));
  const int64_t ae = attn_rows_ws_elems((int)RY, si.max_total, c.n_q_heads, c.head_dim, true);
  // carve 256-byte aligned regions
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = round_up(off + std::max(bytes, (size_t)1), 256);
    return base + o;
  };
  Work w;
  w.x = (float*)take(T * d * 4);
  w.y = (float*)take(B * d * 4);
  w.ya = take(RY * d * 2);
  w.yq = take(RY * dq * 2);
  w.yo = take(RY * dq * 2);
  w.yh = take(RY * f * 2);
  w.rss = (float*)take(RY * (d / 128) * 4);
  w.partial = (float*)take((size_t)pe * 4);
  w.partial_elems = pe;
  w.attn_ws = (float*)take((size_t)ae * 4);
  w.pos = (int32_t*)take(T * 4);
  w.slot = (int32_t*)take(T * 4);
  w.seq = (int32_t*)take(T * 4);
  w.last_pos = (int32_t*)take(B * 4);
  w.last_row = (int32_t*)take(B * 4);
  w.profile = false;
  if (off > kNoAllocScratchBytes)
    return fail(SKV_ERR_INVALID_ARG, "skv_step_noalloc needs " + std::to_string(off) + " bytes of scratch, more than its " +
                                         std::to_string(kNoAllocScratchBytes) + " (fewer rows or shorter contexts)");
  return run_step<bf16_t>(m, kc, bt, si, logits, (hipStream_t)stream, w);
}
