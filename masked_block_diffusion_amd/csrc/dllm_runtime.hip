// C ABI of libdllm.so: argument checks, workspace carving and the launch
// sequence of a denoising step / an append pass on the caller's stream.
#include <stdio.h>
#include <string.h>
#include <math.h>

#include <string>
#include <vector>
#include <algorithm>
#include <mutex>

#include "../../include/dllm.h"
#include "dllm_internal.h"

using namespace dllm;

namespace {

constexpr size_t kAlign = 256;
#ifndef DLLM_APPEND_TOKENS
#define DLLM_APPEND_TOKENS 4096
#endif
constexpr int kAppendTokens = DLLM_APPEND_TOKENS;  // model rows x tokens per append chunk

size_t al(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Layout {
  size_t h, x, q, bk, bv, part_o, part_ml, attn, lse, sspart, rlogits, idx, idx_all, gates, masks, off, tok,
      gsort, slot_pos, items, n_items, hmid, ybuf, row_map, entry_pos, seq_off, n_rows, n_entries,
      cpart, conf, xhat, mass, mass_part, kept, n_kept, rem, knorm, pconf, pids, pcpart, kcomp, vcomp, total;
  // derived sizes
  int R, tok_step, tok_append, Mmax, Smax, max_items, n_splits, LBp, Vsub, ntiles, Fmax, es;
  int cap_c;     // rows per (layer, row, head) of the compacted retained K/V (0: not compacted)
};

// Retention with one pool in bf16: the retained prefix K/V are compacted
// once per block and the retained steps stream them (other cases gather the
// kept positions through their index list).
bool compact_retention(const dllm_model_config* c, const dllm_gen_params* g) {
  return g->use_sprint && c->act_dtype == DLLM_BF16 && g->block_length <= 32 && g->image_keep_ratio <= 0.f &&
         g->text_keep_ratio <= 0.f;
}

int elem_size(int dt) { return dt == DLLM_F32 ? 4 : (dt == DLLM_BF16 ? 2 : 1); }

// Model rows per sequence and LM-head rows per masked entry: plain 1 / 1,
// CFG pairs 2 / 2, three-way guidance 3 / 4 (the fourth head row repeats
// the unconditional one so an entry fills one 4-row accumulator group).
int guidance_mode(const dllm_gen_params* g) { return g->cfg_text_scale > 0.f ? 2 : (g->cfg_scale > 0.f ? 1 : 0); }
int rows_per_seq(const dllm_gen_params* g) { return 1 + guidance_mode(g); }
int head_rows_per_entry(const dllm_gen_params* g) {
  const int gm = guidance_mode(g);
  return gm == 2 ? 4 : gm + 1;
}

int pow2_8(int x) {
  int p = 8;
  while (p < x) p <<= 1;
  return p;
}

// Host-side checks of the shapes the kernels assume.  Returns "" if valid.
std::string check_shapes(const dllm_model_config* c, const dllm_gen_params* g) {
  if (!c || !g) return "null config";
  if (c->n_layers < 1 || c->hidden < 256 || c->hidden % 256 || c->hidden > kMaxHidden)
    return "hidden must be a positive multiple of 256, at most 8192";
  if (c->n_heads < 1 || (c->head_dim != 32 && c->head_dim != 64 && c->head_dim != 128))
    return "head_dim must be 32, 64 or 128";
  if ((c->n_heads * c->head_dim) % 256) return "n_heads * head_dim must be a multiple of 256";
  if (c->n_experts < 1 || c->n_experts > 256 || c->n_experts % 16) return "n_experts must be 16..256, multiple of 16";
  if (c->top_k < 1 || c->top_k > 16 || c->top_k > c->n_experts) return "top_k must be 1..min(16, n_experts)";
  if (c->n_shared < 0 || c->n_shared > 1) return "n_shared must be 0 or 1";
  if (c->expert_ffn < 32 || c->expert_ffn % 32) return "expert_ffn must be a multiple of 32";
  if (c->expert_dtype == DLLM_FP8_E4M3 && (c->hidden % 512 || c->expert_ffn % 64))
    return "fp8 experts need hidden a multiple of 512 and expert_ffn a multiple of 64";
  if (c->n_shared && (c->shared_ffn < 32 || c->shared_ffn % 32)) return "shared_ffn must be a multiple of 32";
  if (c->vocab_text < 0 || c->vocab_image < 0 || c->vocab_text + c->vocab_image < 1) return "empty vocabulary";
  if (c->act_dtype != DLLM_F32 && c->act_dtype != DLLM_BF16) return "act_dtype must be F32 or BF16";
  if (c->act_dtype == DLLM_F32 && c->expert_dtype != DLLM_F32) return "F32 activations need F32 experts";
  if (c->act_dtype == DLLM_BF16 && c->expert_dtype != DLLM_BF16 && c->expert_dtype != DLLM_FP8_E4M3)
    return "BF16 activations need BF16 or FP8 experts";
  if (!(c->rms_eps >= 0.f) || !(c->rope_base > 0.f)) return "bad rms_eps / rope_base";
  if (g->block_length < 1 || g->block_length > 64) return "block_length must be 1..64";
  if (pow2_8(g->block_length) * c->head_dim > 4096) return "block_length x head_dim too large for attention tiles";
  if (g->steps < 1) return "steps must be >= 1";
  if (g->n_seq < 1) return "n_seq must be >= 1";
  const int V = c->vocab_text + c->vocab_image;
  const int hi = g->vocab_hi ? g->vocab_hi : V;
  if (g->vocab_lo < 0 || hi > V || hi <= g->vocab_lo) return "bad sub-vocabulary";
  if (g->n_seq * g->block_length > 1024) return "n_seq x block_length must be <= 1024";
  if (g->cfg_text_scale > 0.f && g->cfg_scale > 0.f) return "cfg_scale and cfg_text_scale are exclusive";
  if (g->cfg_text_scale > 0.f && !(g->cfg_image_scale >= 0.f && g->cfg_image_scale < INFINITY))
    return "cfg_image_scale must be finite and >= 0";
  if (g->confidence < 0 || g->confidence > 2) return "bad confidence strategy";
  if (g->use_sprint && !(g->keep_ratio > 0.f && g->keep_ratio <= 1.f)) return "keep_ratio must be in (0, 1]";
  if (g->retention_score != DLLM_RETAIN_MASS && g->retention_score != DLLM_RETAIN_KEYNORM_CONF)
    return "bad retention_score";
  if (g->retention_score == DLLM_RETAIN_KEYNORM_CONF && !(g->retention_alpha >= 0.f && g->retention_alpha <= 1.f))
    return "retention_alpha must be in [0, 1]";
  if (!(g->image_keep_ratio <= 1.f) || !(g->text_keep_ratio <= 1.f)) return "pool keep ratios must be <= 1";
  if (g->use_sprint && g->cache_warmup_steps < 1) return "cache_warmup_steps must be >= 1";
  if (g->use_sprint && g->cache_warmup_steps > g->steps) return "cache_warmup_steps > steps";
  if (g->max_prefix < 0 || g->max_prefix % g->block_length) return "max_prefix must be a multiple of block_length";
  if (g->max_clean_tokens < 0 || g->max_clean_tokens % g->block_length)
    return "max_clean_tokens must be a multiple of block_length";
  // attention combine keeps (m, l) of every partial of a query block in LDS
  if (g->max_prefix > 16384 - 1024) return "max_prefix must be <= 15360";

  return "";
}

Layout make_layout(const dllm_model_config* c, const dllm_gen_params* g) {
  Layout L{};
  L.R = g->n_seq * rows_per_seq(g);
  const int LB = g->block_length;
  L.tok_step = LB;
  int blocks = kAppendTokens / (L.R * LB);
  if (blocks < 1) blocks = 1;
  L.tok_append = blocks * LB;
  if (g->max_clean_tokens > 0 && L.tok_append > g->max_clean_tokens) L.tok_append = g->max_clean_tokens;
  if (L.tok_append < LB) L.tok_append = LB;
  const int ntok = L.tok_step > L.tok_append ? L.tok_step : L.tok_append;
  L.Mmax = L.R * ntok;
  L.Smax = L.Mmax * c->top_k;
  // work items hold at most 32 rows in either kernel family (64 in the
  // work-list kernels): count them at 32
  L.max_items = (c->n_experts < L.Smax ? c->n_experts : L.Smax) + L.Smax / kRowChunk + 1 +
                (L.Mmax + kRowChunk - 1) / kRowChunk;
  // the smaller split; a compacted retained prefix may round up by 31 rows
  L.n_splits = (g->max_prefix + 32 + ntok + kAttnSplitMfma - 1) / kAttnSplitMfma;
  L.LBp = pow2_8(LB);
  const int V = c->vocab_text + c->vocab_image;
  L.Vsub = (g->vocab_hi ? g->vocab_hi : V) - g->vocab_lo;
  L.ntiles = (L.Vsub + 15) / 16;   // confidence partials: at most one per 16 head columns
  L.Fmax = c->expert_ffn > c->shared_ffn ? c->expert_ffn : c->shared_ffn;
  L.es = elem_size(c->act_dtype);
  const size_t D = c->hidden, HD = (size_t)c->n_heads * c->head_dim, E = c->n_experts, k = c->top_k;
  const size_t M = L.Mmax, S = L.Smax, es = L.es;
  const size_t nq = (size_t)L.R * c->n_heads * (ntok / LB);
  const size_t nent = (size_t)g->n_seq * LB;
  const size_t hrows = nent * head_rows_per_entry(g);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t r = o;
    o += al(bytes);
    return r;
  };
  L.h = take(M * D * 4);
  L.x = take(M * D * es);

  L.q = take(M * HD * es);
  L.bk = take((size_t)L.R * HD * LB * es);
  L.bv = take((size_t)L.R * HD * LB * es);
  // one partial per key split, 32 or LBp query rows each
  const size_t qrows = L.LBp > 32 ? L.LBp : 32;
  L.part_o = take(nq * L.n_splits * qrows * c->head_dim * 4);
  L.part_ml = take(nq * L.n_splits * qrows * 2 * 4);
  L.attn = take(M * HD * es);
  L.lse = take((size_t)L.R * c->n_heads * ntok * 4);
  L.sspart = take(M * (D / 16) * 4);   // per-row sums of squares of h, per 16-column tile
  L.rlogits = take(M * E * 4 * kRouterSplit);   // router partial logits per K slice
  L.idx = take(M * k * 4);
  L.masks = take((size_t)c->n_layers * kMaskWords * 4);   // per layer, zeroed by the embedding pass
  L.idx_all = take((size_t)c->n_layers * M * k * 4);
  L.gates = take(M * k * 4);
  L.off = take((E + 2) * 4);
  L.tok = take((S + M) * 4);
  L.gsort = take(S * 4);
  L.slot_pos = take(S * 4);
  L.items = take((size_t)L.max_items * 16);
  L.n_items = take(4);
  L.hmid = take((S + M) * L.Fmax * es);
  L.ybuf = take((S + M) * D * es);   // expert outputs in the activation type
  L.row_map = take(hrows * 4);
  L.entry_pos = take(nent * 4);
  L.seq_off = take(((size_t)g->n_seq + 1) * 4);
  L.n_rows = take(4);
  L.n_entries = take(4);
  L.cpart = take(nent * L.ntiles * 5 * 4);
  L.conf = take(nent * 4);
  L.xhat = take(nent * 4);
  L.mass = take((size_t)L.R * g->max_prefix * 4);
  // per-head attention mass of one layer (retention by attention mass)
  L.mass_part = take(g->use_sprint ? (size_t)c->n_heads * L.R * g->max_prefix * 4 : 0);
  L.kept = take((size_t)L.R * g->max_prefix * 4);
  L.n_kept = take((size_t)L.R * 4);
  L.rem = take((size_t)g->n_seq * 4);
  // prefix state of the retention score: key norms, top-1 probabilities, ids
  L.knorm = take((size_t)L.R * g->max_prefix * 4);
  L.pconf = take((size_t)L.R * g->max_prefix * 4);
  L.pids = take((size_t)L.R * g->max_prefix * 4);
  // LM-head partials of an append chunk (only for the key-norm + confidence score)
  L.pcpart = take(g->retention_score == DLLM_RETAIN_KEYNORM_CONF ? (size_t)L.Mmax * L.ntiles * 5 * 4 : 0);
  // compacted retained K and V: [layers][rows][heads][cap_c][head_dim] each
  L.cap_c = compact_retention(c, g) ? (g->max_prefix + 31) / 32 * 32 : 0;
  const size_t comp = (size_t)c->n_layers * L.R * c->n_heads * L.cap_c * c->head_dim * es;
  L.kcomp = take(comp);
  L.vcomp = take(comp);
  L.total = o;
  return L;
}

// Inspection buffer (caller memory, attached with dllm_debug_attach): router
// logits of every layer of the last forward pass, then the head logits of the
// last step's masked rows.
struct DebugLayout {
  size_t z, logits, total;
};

DebugLayout debug_layout(const dllm_model_config* c, const dllm_gen_params* g, const Layout& L) {
  DebugLayout d{};
  const size_t hrows = (size_t)g->n_seq * g->block_length * head_rows_per_entry(g);
  d.z = 0;
  d.logits = al((size_t)c->n_layers * L.Mmax * c->n_experts * 4);
  d.total = d.logits + al(hrows * L.Vsub * 4);
  return d;
}

int mode_of(const dllm_model_config& c) {
  if (c.act_dtype == DLLM_F32) return MODE_F32;
  return c.expert_dtype == DLLM_FP8_E4M3 ? MODE_FP8 : MODE_BF16;
}

}  // namespace

struct dllm_ctx {
  dllm_model_config cfg;
  dllm_gen_params gp;
  dllm_weights w;
  dllm_kv_cache kv;
  hipStream_t stream;
  char* ws;
  size_t ws_bytes;
  Layout L;
  int P = 0;
  bool block_open = false;
  bool kept_valid = false;
  bool comp_valid = false;   // the compacted retained K/V hold this block's kept set
  int comp_np = 0, comp_pad = 0;   // their rows per (layer, row, head) and leading zero rows
  int last_M = 0;
  AttnPlan last_plan{};
  int n_cu = 256;
  char* dbg = nullptr;   // attached inspection buffer (null: none)
  std::string err;
  // optional launch timing: start/stop event pairs around the kernel groups
  // whose bit is set in prof_mask
  uint32_t prof_mask = 0;
  std::vector<hipEvent_t> ev;
  std::vector<int> ev_cat;
  size_t ev_used = 0;
  double prof_ms[DLLM_PROF_GROUPS] = {0};
  long long prof_n[DLLM_PROF_GROUPS] = {0};

  template <typename T> T* at(size_t off) { return (T*)(ws + off); }
};

// Resolve recorded event pairs into per-group totals (synchronises the events).
static void prof_flush(dllm_ctx* c) {
  for (size_t i = 0; i + 1 < c->ev_used; i += 2) {
    float ms = 0.f;
    if (hipEventSynchronize(c->ev[i + 1]) == hipSuccess &&
        hipEventElapsedTime(&ms, c->ev[i], c->ev[i + 1]) == hipSuccess) {
      c->prof_ms[c->ev_cat[i]] += ms;
      c->prof_n[c->ev_cat[i]] += 1;
    }
  }
  c->ev_used = 0;
}

struct ProfScope {
  dllm_ctx* c;
  int cat;
  bool on;
  ProfScope(dllm_ctx* c_, int cat_) : c(c_), cat(cat_), on((c_->prof_mask >> cat_) & 1u) {
    if (!on) return;
    if (c->ev_used + 2 > c->ev.size()) prof_flush(c);
    c->ev_cat[c->ev_used] = cat;
    (void)hipEventRecord(c->ev[c->ev_used], c->stream);
  }
  ~ProfScope() {
    if (!on) return;
    (void)hipEventRecord(c->ev[c->ev_used + 1], c->stream);
    c->ev_used += 2;
  }
};

static int fail(dllm_ctx* c, int code, const std::string& msg) {
  if (c) c->err = msg;
  return code;
}

#define HIPCHK(expr)                                                                   \
  do {                                                                                 \
    hipError_t e_ = (expr);                                                            \
    if (e_ != hipSuccess)                                                              \
      return fail(ctx, DLLM_ERR_HIP, std::string(#expr ": ") + hipGetErrorString(e_)); \
  } while (0)

extern "C" {

const char* dllm_status_string(int s) {
  switch (s) {
    case DLLM_OK: return "ok";
    case DLLM_ERR_INVALID_ARG: return "invalid argument";
    case DLLM_ERR_OUT_OF_MEMORY: return "workspace or KV capacity too small";
    case DLLM_ERR_HIP: return "HIP error";
    case DLLM_ERR_BAD_STATE: return "call out of order";
    case DLLM_ERR_UNSUPPORTED: return "unsupported combination";
    default: return "unknown status";
  }
}

int dllm_append_tokens(const dllm_model_config* cfg, const dllm_gen_params* gp) {
  if (!check_shapes(cfg, gp).empty()) return 0;
  return make_layout(cfg, gp).tok_append;
}

size_t dllm_workspace_bytes(const dllm_model_config* cfg, const dllm_gen_params* gp) {
  if (!check_shapes(cfg, gp).empty()) return 0;
  Layout L = make_layout(cfg, gp);
  if ((size_t)L.Smax > (size_t)kMaxSlots) return 0;
  return L.total;
}

size_t dllm_kv_bytes(const dllm_model_config* cfg, const dllm_gen_params* gp) {
  if (!check_shapes(cfg, gp).empty()) return 0;
  const int R = gp->n_seq * rows_per_seq(gp);
  return (size_t)cfg->n_layers * R * cfg->n_heads * (size_t)gp->max_prefix * cfg->head_dim *
         elem_size(cfg->act_dtype);
}

// ---- workspace in a static device array (dllm_create_static) ----
// One copy per GPU, alive until the process ends.  Host code reaches it only
// through the address hipGetSymbolAddress returns on each device.
static constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

static constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

// Device address of this GPU's scratch (looked up once per device, with that
// device current).
static int static_scratch(void** out, std::string* why) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *why = "no current HIP device (or device index beyond 63)";
    return DLLM_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      *why = std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e);
      return DLLM_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DLLM_OK;
}

int dllm_create(dllm_ctx** out, const dllm_model_config* cfg, const dllm_gen_params* gp,
                const dllm_weights* w, const dllm_kv_cache* kv, void* d_workspace, size_t ws_bytes,
                void* stream) {
  if (!out) return DLLM_ERR_INVALID_ARG;
  *out = nullptr;
  std::string why = check_shapes(cfg, gp);
  if (!why.empty()) {
    fprintf(stderr, "dllm_create: %s\n", why.c_str());
    return DLLM_ERR_INVALID_ARG;
  }
  if (!w || !kv || !d_workspace) return DLLM_ERR_INVALID_ARG;
  if (((uintptr_t)d_workspace) % kAlign) return DLLM_ERR_INVALID_ARG;
  const bool fp8 = cfg->expert_dtype == DLLM_FP8_E4M3;
  if (!w->embed || !w->attn_norm || !w->w_qkv || !w->w_o || !w->moe_norm || !w->w_router ||
      !w->router_bias || !w->w_gate || !w->w_up || !w->w_down || !w->final_norm || !w->lm_head)
    return DLLM_ERR_INVALID_ARG;
  if (fp8 && (!w->s_gate || !w->s_up || !w->s_down)) return DLLM_ERR_INVALID_ARG;
  if (cfg->n_shared && (!w->ws_gate || !w->ws_up || !w->ws_down)) return DLLM_ERR_INVALID_ARG;
  if (gp->max_prefix > 0 && (!kv->k || !kv->v)) return DLLM_ERR_INVALID_ARG;
  Layout L = make_layout(cfg, gp);
  if ((size_t)L.Smax > (size_t)kMaxSlots) return DLLM_ERR_UNSUPPORTED;
  if (ws_bytes < L.total) return DLLM_ERR_OUT_OF_MEMORY;
  dllm_ctx* c = new dllm_ctx();
  c->cfg = *cfg;
  c->gp = *gp;
  if (c->gp.vocab_hi == 0) c->gp.vocab_hi = cfg->vocab_text + cfg->vocab_image;
  c->w = *w;
  c->kv = *kv;
  c->stream = (hipStream_t)stream;
  c->ws = (char*)d_workspace;
  c->ws_bytes = ws_bytes;
  c->L = L;
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && ncu > 0)
    c->n_cu = ncu;
  *out = c;
  return DLLM_OK;
}

int dllm_create_static(dllm_ctx** out, const dllm_model_config* cfg, const dllm_gen_params* gp,
                       const dllm_weights* w, const dllm_kv_cache* kv, void* stream) {
  if (!out) return DLLM_ERR_INVALID_ARG;
  *out = nullptr;
  std::string why = check_shapes(cfg, gp);
  if (!why.empty()) {
    fprintf(stderr, "dllm_create_static: %s\n", why.c_str());
    return DLLM_ERR_INVALID_ARG;
  }
  const Layout L = make_layout(cfg, gp);
  if (L.total > kStaticScratchBytes) {
    fprintf(stderr, "dllm_create_static: this shape needs %zu bytes of workspace, the static scratch holds %zu\n",
            L.total, kStaticScratchBytes);
    return DLLM_ERR_OUT_OF_MEMORY;
  }
  void* p = nullptr;
  int st = static_scratch(&p, &why);
  if (st != DLLM_OK) {
    fprintf(stderr, "dllm_create_static: %s\n", why.c_str());
    return st;
  }
  st = dllm_create(out, cfg, gp, w, kv, p, kStaticScratchBytes, stream);
  if (st != DLLM_OK) return st;
  // the array keeps whatever the last context on this GPU left in it: clear
  // the part this one uses, with a fill kernel on its stream
  const hipError_t e = launch_fill_f32((float*)p, 0.f, (long long)(L.total / 4), (hipStream_t)stream);
  if (e != hipSuccess) {
    fprintf(stderr, "dllm_create_static: clearing the scratch failed: %s\n", hipGetErrorString(e));
    dllm_destroy(*out);
    *out = nullptr;
    return DLLM_ERR_HIP;
  }
  return DLLM_OK;
}

void dllm_destroy(dllm_ctx* ctx) {
  if (!ctx) return;
  for (hipEvent_t e : ctx->ev) (void)hipEventDestroy(e);
  delete ctx;
}

const char* dllm_last_error(const dllm_ctx* ctx) { return ctx ? ctx->err.c_str() : "null context"; }

int32_t dllm_prefix_length(const dllm_ctx* ctx) { return ctx ? ctx->P : -1; }

}  // extern "C"

// One pass of all layers over n_tok tokens per model row at positions
// P .. P+n_tok-1.  append: K/V go to the cache and the keys of query block b
// are cache positions [0, P + (b+1) L_B); otherwise (a denoising step) the
// keys are the prefix (all of it, or the kept positions) plus the block, and
// the block's K/V stay in scratch.
static int forward(dllm_ctx* ctx, const int32_t* ids, int ids_stride, int n_tok, int rep, bool append,
                   bool use_kept, bool want_mass) {
  const dllm_model_config& c = ctx->cfg;
  const dllm_gen_params& g = ctx->gp;
  const dllm_weights& w = ctx->w;
  const Layout& L = ctx->L;
  hipStream_t s = ctx->stream;
  const int mode = mode_of(c);
  const int dmode = (mode == MODE_F32) ? MODE_F32 : MODE_BF16;
  const int R = L.R, D = c.hidden, H = c.n_heads, dh = c.head_dim, HD = H * dh, E = c.n_experts;
  const int k = c.top_k, LB = g.block_length, es = L.es;
  const int M = R * n_tok;
  const int S = M * k;
  const int P = ctx->P;
  const size_t ees = elem_size(c.expert_dtype);
  const long long kv_row = (long long)H * g.max_prefix * dh;
  const long long kv_head = (long long)g.max_prefix * dh;
  const size_t kv_layer_bytes = (size_t)R * kv_row * es;
  float* h = ctx->at<float>(L.h);
  void* x = ctx->at<void>(L.x);
  void* q = ctx->at<void>(L.q);
  ctx->last_M = M;

  // a denoising step also lists its masked positions (LM-head rows)
  HIPCHK(launch_embed_norm(dmode, ids, ids_stride, R, n_tok, rep, c.vocab_text + c.vocab_image + 1, w.embed,
                           w.attn_norm, c.rms_eps, D, h, x, append ? nullptr : ids, g.n_seq, LB,
                           c.vocab_text + c.vocab_image, guidance_mode(&g), ctx->at<int32_t>(L.row_map),
                           ctx->at<int32_t>(L.entry_pos), ctx->at<int32_t>(L.seq_off), ctx->at<int32_t>(L.n_rows),
                           ctx->at<int32_t>(L.n_entries), ctx->at<uint32_t>(L.masks), c.n_layers * kMaskWords, s));
  // retained steps: the compacted kept rows as a contiguous prefix (np_att
  // rows, the first comp_pad of them masked), else the kept-index gather
  const bool comp = use_kept && ctx->comp_valid;
  const bool gather = use_kept && !comp;
  const int np_att = comp ? ctx->comp_np : P;
  const int nk_max = append ? P + n_tok : np_att + LB;
  const AttnPlan apl = attn_plan(dmode, R, H, n_tok, LB, dh, nk_max, gather ? 1 : 0, np_att, append ? 1 : 0);
  const long long comp_head = (long long)L.cap_c * dh, comp_row = (long long)H * comp_head;
  const size_t comp_layer_bytes = (size_t)R * comp_row * es;
  ctx->last_plan = apl;
  for (int l = 0; l < c.n_layers; ++l) {
    const char* wqkv = (const char*)w.w_qkv + (size_t)l * 3 * HD * D * es;
    const char* wo = (const char*)w.w_o + (size_t)l * D * HD * es;
    const char* wr = (const char*)w.w_router + (size_t)l * E * D * es;
    char* kc = (char*)ctx->kv.k + (size_t)l * kv_layer_bytes;
    char* vc = (char*)ctx->kv.v + (size_t)l * kv_layer_bytes;
    // QKV projection, RoPE, scatter
    {
      ProfScope ps(ctx, DLLM_PROF_QKV);
      // passes of >= 128 rows (prefill, large batches) use the LDS-tiled GEMM
      const bool tiled = qkv_tiled_ok(dmode, M, D, H, dh);
      void* kd = append ? (void*)kc : ctx->at<void>(L.bk);
      void* vd = append ? (void*)vc : ctx->at<void>(L.bv);
      const long long krs = append ? kv_row : (long long)H * LB * dh;
      const long long khs = append ? kv_head : (long long)LB * dh;
      const int kp0 = append ? P : 0;
      if (tiled)
        HIPCHK(launch_qkv_rope_tiled(x, wqkv, R, n_tok, D, H, dh, P, c.rope_base, q, kd, vd, krs, khs, kp0, s));
      else
        HIPCHK(launch_qkv_rope(dmode, x, wqkv, R, n_tok, D, H, dh, P, c.rope_base, q, kd, vd, krs, khs, kp0, s));
      if (append && g.retention_score == DLLM_RETAIN_KEYNORM_CONF)
        HIPCHK(launch_key_norm(dmode, kc, R, n_tok, H, dh, kv_row, kv_head, P, ctx->at<float>(L.knorm),
                               g.max_prefix, l > 0 ? 1 : 0, s));
    }
    // block-wise attention
    const int32_t* kept = gather ? ctx->at<int32_t>(L.kept) : nullptr;
    const int32_t* n_kept = gather ? ctx->at<int32_t>(L.n_kept) : nullptr;
    {
      ProfScope ps(ctx, DLLM_PROF_ATTN);
      const char* ka = comp ? ctx->at<char>(L.kcomp) + (size_t)l * comp_layer_bytes : kc;
      const char* va = comp ? ctx->at<char>(L.vcomp) + (size_t)l * comp_layer_bytes : vc;
      HIPCHK(launch_attn(apl, dmode, q, R, H, dh, n_tok, LB, ka, va, comp ? comp_row : kv_row,
                         comp ? comp_head : kv_head, ctx->at<void>(L.bk), ctx->at<void>(L.bv), kept, n_kept,
                         g.max_prefix, np_att, append ? 1 : 0, P, ctx->at<float>(L.part_o),
                         ctx->at<float>(L.part_ml), ctx->at<void>(L.attn), ctx->at<float>(L.lse), s,
                         comp ? ctx->comp_pad : 0));
    }
    if (want_mass)
      HIPCHK(launch_attn_mass(dmode, q, ctx->at<float>(L.lse), R, H, dh, LB, kc, kv_row, kv_head, P,
                              ctx->at<float>(L.mass), g.max_prefix, s, ctx->at<float>(L.mass_part)));
    // output projection + residual, pre-MoE norm
    if (gemm_tiled_ok(dmode, M, D, HD))
      HIPCHK(launch_gemm_tiled_acc(ctx->at<void>(L.attn), HD, M, wo, HD, D, HD, h, D, ctx->at<float>(L.sspart), s));
    else
      HIPCHK(launch_gemm(dmode, ctx->at<void>(L.attn), HD, nullptr, M, nullptr, wo, HD, D, HD, h, D, 1, s,
                         ctx->at<float>(L.sspart)));
    // router logits, then selection; few tokens route in slot order (each
    // expert workgroup gathers its own slots), more go through the
    // expert-major permutation and its work list
    const bool slot_order = M <= kDirectMaxTokens;
    // pre-MoE RMSNorm folded into the router GEMM, which also writes x
    HIPCHK(launch_router_norm(dmode, h, w.moe_norm + (size_t)l * D, ctx->at<float>(L.sspart), D / 16, c.rms_eps, M,
                              wr, E, D, ctx->at<float>(L.rlogits), x, s));
    int32_t* idx_l = ctx->at<int32_t>(L.idx_all) + (size_t)l * L.Mmax * k;
    const int n_split = router_k_split(D);
    float* z_dbg = ctx->dbg ? (float*)ctx->dbg + (size_t)l * L.Mmax * E : nullptr;
    HIPCHK(launch_router_topk(ctx->at<float>(L.rlogits), n_split, w.router_bias + (size_t)l * E, M, E, k,
                              ctx->at<int32_t>(L.idx), ctx->at<float>(L.gates), idx_l,
                              slot_order ? ctx->at<uint32_t>(L.masks) + (size_t)l * kMaskWords : nullptr, s, z_dbg));
    const int item_rows = expert_item_rows(mode, D, c.expert_ffn, c.n_shared ? c.shared_ffn : c.expert_ffn);
    if (!slot_order)
      HIPCHK(launch_permute(ctx->at<int32_t>(L.idx), ctx->at<float>(L.gates), M, E, k, c.n_shared, item_rows, ctx->at<int32_t>(L.off), ctx->at<int32_t>(L.tok),
                            ctx->at<float>(L.gsort), ctx->at<int32_t>(L.slot_pos), ctx->at<int4>(L.items),
                            ctx->at<int32_t>(L.n_items), s));
    // experts
    ExpertArgs a;
    a.X = x;
    a.items = ctx->at<int4>(L.items);
    a.n_items = ctx->at<int32_t>(L.n_items);
    a.off = ctx->at<int32_t>(L.off);
    a.tok = ctx->at<int32_t>(L.tok);
    a.route = slot_order ? ctx->at<int32_t>(L.idx) : nullptr;
    a.masks = ctx->at<uint32_t>(L.masks) + (size_t)l * kMaskWords;
    a.gate_rows = slot_order ? ctx->at<float>(L.gates) : ctx->at<float>(L.gsort);
    a.M = M;
    a.S = S;
    a.k = k;
    const size_t exp_layer = (size_t)E * c.expert_ffn * D * ees;
    a.wg = (const char*)w.w_gate + l * exp_layer;
    a.wu = (const char*)w.w_up + l * exp_layer;
    a.wd = (const char*)w.w_down + l * exp_layer;
    const size_t sc_layer = (size_t)E * c.expert_ffn;
    a.sg = w.s_gate ? w.s_gate + l * sc_layer : nullptr;
    a.su = w.s_up ? w.s_up + l * sc_layer : nullptr;
    a.sd = w.s_down ? w.s_down + (size_t)l * E * D : nullptr;
    const size_t sh_layer = (size_t)c.shared_ffn * D * es;
    a.swg = c.n_shared ? (const char*)w.ws_gate + l * sh_layer : nullptr;
    a.swu = c.n_shared ? (const char*)w.ws_up + l * sh_layer : nullptr;
    a.swd = c.n_shared ? (const char*)w.ws_down + l * sh_layer : nullptr;
    a.Hmid = ctx->at<void>(L.hmid);
    a.Y = ctx->at<void>(L.ybuf);
    a.D = D;
    a.F = c.expert_ffn;
    a.Fs = c.n_shared ? c.shared_ffn : c.expert_ffn;
    a.E = E;
    a.Fmax = L.Fmax;
    a.n_cu = ctx->n_cu;
    a.gu_packed = w.gate_up_packed ? 1 : 0;
    const int max_items = (E < S ? E : S) + S / item_rows + 1 + (c.n_shared ? (M + item_rows - 1) / item_rows : 0);
    {
      ProfScope ps(ctx, DLLM_PROF_EXPERT_GATEUP);
      HIPCHK(launch_expert_gateup(mode, a, max_items, s));
    }
    {
      ProfScope ps(ctx, DLLM_PROF_EXPERT_DOWN);
      HIPCHK(launch_expert_down(mode, a, max_items, s));
    }
    const float* next_gain = (l + 1 < c.n_layers) ? w.attn_norm + (size_t)(l + 1) * D : w.final_norm;
    HIPCHK(launch_combine_norm(dmode, h, ctx->at<void>(L.ybuf), slot_order ? nullptr : ctx->at<int32_t>(L.slot_pos),
                               M, D, k, S, c.n_shared, next_gain, c.rms_eps, x, s));
  }
  return DLLM_OK;
}

static bool pools_on(const dllm_gen_params& g) { return g.image_keep_ratio > 0.f || g.text_keep_ratio > 0.f; }

extern "C" {

int dllm_block_init(dllm_ctx* ctx, const int32_t* d_clean_ids, int32_t n_clean) {
  if (!ctx) return DLLM_ERR_INVALID_ARG;
  const dllm_gen_params& g = ctx->gp;
  if (n_clean < 0 || n_clean % g.block_length)
    return fail(ctx, DLLM_ERR_INVALID_ARG, "n_clean must be a non-negative multiple of block_length");
  if (n_clean > g.max_clean_tokens)
    return fail(ctx, DLLM_ERR_INVALID_ARG, "n_clean exceeds max_clean_tokens");
  if (n_clean > 0 && !d_clean_ids) return fail(ctx, DLLM_ERR_INVALID_ARG, "null ids");
  if ((long long)ctx->P + n_clean > g.max_prefix)
    return fail(ctx, DLLM_ERR_OUT_OF_MEMORY, "KV cache capacity exceeded");
  const Layout& L = ctx->L;
  const dllm_model_config& c = ctx->cfg;
  hipStream_t s = ctx->stream;
  for (int c0 = 0; c0 < n_clean; c0 += L.tok_append) {
    const int nt = std::min(L.tok_append, n_clean - c0);
    int st = forward(ctx, d_clean_ids + c0, n_clean, nt, 1, true, false, false);
    if (st != DLLM_OK) return st;
    if (g.retention_score == DLLM_RETAIN_KEYNORM_CONF) {
      // top-1 probability of every appended position: LM head over the
      // final-normed rows (identity row map), merged per row
      const int M = L.R * nt;
      const int dmode = c.act_dtype == DLLM_F32 ? MODE_F32 : MODE_BF16;
      const char* head = (const char*)ctx->w.lm_head + (size_t)g.vocab_lo * c.hidden * L.es;
      HIPCHK(launch_head(dmode, ctx->at<void>(L.x), c.hidden, nullptr, nullptr, M, head, L.Vsub, 0, 0.f, 0.f,
                         ctx->at<float>(L.pcpart), s));
      HIPCHK(launch_prefix_conf(ctx->at<float>(L.pcpart), head_partial_tiles(dmode, M, L.Vsub), M, nt, ctx->P,
                                g.max_prefix, ctx->at<float>(L.pconf), s));
    }
    if (pools_on(g))
      HIPCHK(launch_store_ids(d_clean_ids + c0, n_clean, L.R, nt, ctx->P, g.max_prefix, ctx->at<int32_t>(L.pids), s));
    ctx->P += nt;
  }
  ctx->block_open = true;
  ctx->kept_valid = false;
  ctx->comp_valid = false;
  return DLLM_OK;
}

int dllm_denoise_step(dllm_ctx* ctx, int32_t t, const int32_t* d_ids_in, int32_t* d_ids_out,
                      int32_t* d_remaining) {
  if (!ctx) return DLLM_ERR_INVALID_ARG;
  const dllm_model_config& c = ctx->cfg;
  const dllm_gen_params& g = ctx->gp;
  const Layout& L = ctx->L;
  hipStream_t s = ctx->stream;
  if (t < 0 || t >= g.steps) return fail(ctx, DLLM_ERR_INVALID_ARG, "step index out of range");
  if (!d_ids_in || !d_ids_out || !d_remaining) return fail(ctx, DLLM_ERR_INVALID_ARG, "null pointer");
  if (!ctx->block_open) return fail(ctx, DLLM_ERR_BAD_STATE, "no open block: call dllm_block_init first");
  // three-way guidance: SPRINT falls back to the baseline (no retention)
  const bool sprint = g.use_sprint && guidance_mode(&g) != 2;
  const bool warm = !sprint || t < g.cache_warmup_steps;
  if (!warm && !ctx->kept_valid)
    return fail(ctx, DLLM_ERR_BAD_STATE, "retained steps need this block's warm-up step first");
  const bool select_now = sprint && t == g.cache_warmup_steps - 1;
  const bool want_mass = select_now && g.retention_score == DLLM_RETAIN_MASS;
  const int gm = guidance_mode(&g);
  const int LB = g.block_length;
  const int mask_id = c.vocab_text + c.vocab_image;
  if (want_mass) HIPCHK(launch_fill_f32(ctx->at<float>(L.mass), 0.f, (long long)L.R * g.max_prefix, s));
  int st = forward(ctx, d_ids_in, LB, LB, rows_per_seq(&g), false, !warm, want_mass);
  if (st != DLLM_OK) return st;
  const int dmode = c.act_dtype == DLLM_F32 ? MODE_F32 : MODE_BF16;
  const int nent = g.n_seq * LB;
  const int hrows = nent * head_rows_per_entry(&g);
  const float gs_a = gm == 2 ? g.cfg_image_scale : g.cfg_scale, gs_b = g.cfg_text_scale;
  const char* head = (const char*)ctx->w.lm_head + (size_t)g.vocab_lo * c.hidden * L.es;
  {
    ProfScope ps(ctx, DLLM_PROF_HEAD);
    HIPCHK(launch_head(dmode, ctx->at<void>(L.x), c.hidden, ctx->at<int32_t>(L.row_map), ctx->at<int32_t>(L.n_rows),
                       hrows, head, L.Vsub, gm, gs_a, gs_b, ctx->at<float>(L.cpart), s));
  }
  HIPCHK(launch_conf_select(ctx->at<float>(L.cpart), head_partial_tiles(dmode, hrows, L.Vsub),
                            ctx->at<int32_t>(L.seq_off), ctx->at<int32_t>(L.entry_pos),
                            g.vocab_lo, g.confidence, d_ids_in, ctx->at<float>(L.conf), ctx->at<int32_t>(L.xhat),
                            g.n_seq, LB, mask_id, g.steps, t, g.use_threshold, g.threshold, d_ids_out, d_remaining, s));
  if (select_now) {
    if (g.retention_score == DLLM_RETAIN_KEYNORM_CONF)
      HIPCHK(launch_retention_score(ctx->at<float>(L.knorm), ctx->at<float>(L.pconf), L.R, ctx->P, g.max_prefix,
                                    g.retention_alpha, ctx->at<float>(L.mass), s));
    const bool pools = pools_on(g);
    const float r_text = pools && g.text_keep_ratio > 0.f ? g.text_keep_ratio : g.keep_ratio;
    const float r_image = pools && g.image_keep_ratio > 0.f ? g.image_keep_ratio : g.keep_ratio;
    HIPCHK(launch_retention(ctx->at<float>(L.mass), L.R, ctx->P, g.max_prefix,
                            pools ? ctx->at<int32_t>(L.pids) : nullptr, c.vocab_text, c.vocab_text + c.vocab_image,
                            r_text, r_image, ctx->at<int32_t>(L.kept), ctx->at<int32_t>(L.n_kept), s));
    ctx->kept_valid = true;
    if (L.cap_c > 0 && !pools) {
      // one pool: every row keeps ceil(r P) positions (the selection's own
      // count); copy them to the compacted K/V, padded in front to whole tiles
      const int n = keep_count(g.keep_ratio, ctx->P);
      const int np = (n + 31) / 32 * 32;
      const int H = c.n_heads, dh = c.head_dim;
      const long long kv_head = (long long)g.max_prefix * dh, kv_row = (long long)H * kv_head;
      const long long ch = (long long)L.cap_c * dh, cr = (long long)H * ch;
      HIPCHK(launch_kv_compact(ctx->kv.k, ctx->kv.v, (long long)L.R * kv_row, kv_row, kv_head,
                               ctx->at<int32_t>(L.kept), g.max_prefix, n, np - n, L.R, H, dh, c.n_layers,
                               ctx->at<void>(L.kcomp), ctx->at<void>(L.vcomp), (long long)L.R * cr, cr, ch, s));
      ctx->comp_np = np;
      ctx->comp_pad = np - n;
      ctx->comp_valid = true;
    }
  }
  return DLLM_OK;
}

int dllm_generate_block(dllm_ctx* ctx, int32_t* d_ids, int32_t* h_steps_taken) {
  if (!ctx) return DLLM_ERR_INVALID_ARG;
  if (!d_ids || !h_steps_taken) return fail(ctx, DLLM_ERR_INVALID_ARG, "null pointer");
  const dllm_gen_params& g = ctx->gp;
  int32_t* rem = ctx->at<int32_t>(ctx->L.rem);
  std::vector<int32_t> host(g.n_seq);
  *h_steps_taken = 0;
  for (int t = 0; t < g.steps; ++t) {
    int st = dllm_denoise_step(ctx, t, d_ids, d_ids, rem);
    if (st != DLLM_OK) return st;
    HIPCHK(hipMemcpyAsync(host.data(), rem, sizeof(int32_t) * g.n_seq, hipMemcpyDeviceToHost, ctx->stream));
    HIPCHK(hipStreamSynchronize(ctx->stream));
    *h_steps_taken = t + 1;
    long long left = 0;
    for (int v : host) left += v;
    if (left == 0) break;
  }
  return DLLM_OK;
}

int dllm_debug_buffer(dllm_ctx* ctx, int32_t which, int32_t layer, void** d_ptr, size_t* bytes) {
  if (!ctx || !d_ptr || !bytes) return DLLM_ERR_INVALID_ARG;
  const Layout& L = ctx->L;
  const dllm_model_config& c = ctx->cfg;
  const dllm_gen_params& g = ctx->gp;
  const size_t nent = (size_t)g.n_seq * g.block_length;
  const size_t hrows = nent * head_rows_per_entry(&g);
  switch (which) {
    case 0:
      if (layer < 0 || layer >= c.n_layers) return fail(ctx, DLLM_ERR_INVALID_ARG, "bad layer");
      *d_ptr = ctx->at<int32_t>(L.idx_all) + (size_t)layer * L.Mmax * c.top_k;
      *bytes = (size_t)ctx->last_M * c.top_k * 4;
      return DLLM_OK;
    case 1: *d_ptr = ctx->at<void>(L.gates); *bytes = (size_t)ctx->last_M * c.top_k * 4; return DLLM_OK;
    case 2: *d_ptr = ctx->at<void>(L.conf); *bytes = nent * 4; return DLLM_OK;
    case 3: *d_ptr = ctx->at<void>(L.xhat); *bytes = nent * 4; return DLLM_OK;
    case 4: *d_ptr = ctx->at<void>(L.mass); *bytes = (size_t)L.R * g.max_prefix * 4; return DLLM_OK;
    case 5: *d_ptr = ctx->at<void>(L.kept); *bytes = (size_t)L.R * g.max_prefix * 4; return DLLM_OK;
    case 6: *d_ptr = ctx->at<void>(L.n_kept); *bytes = (size_t)L.R * 4; return DLLM_OK;
    case 9: *d_ptr = ctx->at<void>(L.knorm); *bytes = (size_t)L.R * g.max_prefix * 4; return DLLM_OK;
    case 10: *d_ptr = ctx->at<void>(L.pconf); *bytes = (size_t)L.R * g.max_prefix * 4; return DLLM_OK;
    case 11: *d_ptr = ctx->at<void>(L.pids); *bytes = (size_t)L.R * g.max_prefix * 4; return DLLM_OK;
    case 7: *d_ptr = ctx->at<void>(L.h); *bytes = (size_t)ctx->last_M * c.hidden * 4; return DLLM_OK;
    case 13: *d_ptr = ctx->at<void>(L.x); *bytes = (size_t)ctx->last_M * c.hidden * L.es; return DLLM_OK;
    case 8: {
      // the step keeps head logits in registers; recompute them into the
      // inspection buffer with the plain GEMM kernel from the last step's
      // final normed rows and masked-row map
      if (!ctx->dbg) return fail(ctx, DLLM_ERR_BAD_STATE, "no inspection buffer attached (dllm_debug_attach)");
      const DebugLayout dl = debug_layout(&c, &g, L);
      const int dmode = c.act_dtype == DLLM_F32 ? MODE_F32 : MODE_BF16;
      const char* head = (const char*)ctx->w.lm_head + (size_t)g.vocab_lo * c.hidden * L.es;
      float* out = (float*)(ctx->dbg + dl.logits);
      if (launch_gemm(dmode, ctx->at<void>(L.x), c.hidden, ctx->at<int32_t>(L.row_map), (int)hrows,
                      ctx->at<int32_t>(L.n_rows), head, c.hidden, L.Vsub, c.hidden, out, L.Vsub, 0,
                      ctx->stream) != hipSuccess ||
          hipStreamSynchronize(ctx->stream) != hipSuccess)
        return fail(ctx, DLLM_ERR_HIP, "head logits recompute failed");
      *d_ptr = out;
      *bytes = hrows * L.Vsub * 4;
      return DLLM_OK;
    }
    case 12:
      if (!ctx->dbg) return fail(ctx, DLLM_ERR_BAD_STATE, "no inspection buffer attached (dllm_debug_attach)");
      if (layer < 0 || layer >= c.n_layers) return fail(ctx, DLLM_ERR_INVALID_ARG, "bad layer");
      *d_ptr = (float*)ctx->dbg + (size_t)layer * L.Mmax * c.n_experts;
      *bytes = (size_t)ctx->last_M * c.n_experts * 4;
      return DLLM_OK;
    default: return fail(ctx, DLLM_ERR_INVALID_ARG, "unknown buffer");
  }
}

size_t dllm_debug_bytes(const dllm_model_config* cfg, const dllm_gen_params* gp) {
  if (!check_shapes(cfg, gp).empty()) return 0;
  const Layout L = make_layout(cfg, gp);
  return debug_layout(cfg, gp, L).total;
}

int dllm_debug_attach(dllm_ctx* ctx, void* d_buf, size_t bytes) {
  if (!ctx) return DLLM_ERR_INVALID_ARG;
  if (!d_buf) {
    ctx->dbg = nullptr;
    return DLLM_OK;
  }
  if (((uintptr_t)d_buf) % kAlign) return fail(ctx, DLLM_ERR_INVALID_ARG, "inspection buffer must be 256-byte aligned");
  if (bytes < debug_layout(&ctx->cfg, &ctx->gp, ctx->L).total)
    return fail(ctx, DLLM_ERR_OUT_OF_MEMORY, "inspection buffer smaller than dllm_debug_bytes");
  ctx->dbg = (char*)d_buf;
  return DLLM_OK;
}

int dllm_debug_attn_plan(const dllm_ctx* ctx, int32_t* h_plan) {
  if (!ctx || !h_plan) return DLLM_ERR_INVALID_ARG;
  h_plan[0] = ctx->last_plan.kind;
  h_plan[1] = ctx->last_plan.split;
  h_plan[2] = ctx->last_plan.n_splits;
  return DLLM_OK;
}

// ---- block-wise attention on given inputs (test support; allocates its key-
// split partials, synchronises the stream) ----

int dllm_debug_block_attention(int32_t act_dtype, const void* d_q, const void* d_kc, const void* d_vc, int32_t cap,
                               const void* d_bk, const void* d_bv, const int32_t* d_kept, const int32_t* d_n_kept,
                               int32_t rows, int32_t n_heads, int32_t head_dim, int32_t block_length, int32_t P,
                               void* d_out, float* d_lse, int32_t* h_plan, void* stream) {
  if (act_dtype != DLLM_F32 && act_dtype != DLLM_BF16) return DLLM_ERR_INVALID_ARG;
  if (!d_q || !d_bk || !d_bv || !d_out || rows < 1 || n_heads < 1) return DLLM_ERR_INVALID_ARG;
  if (head_dim != 32 && head_dim != 64 && head_dim != 128) return DLLM_ERR_INVALID_ARG;
  if (block_length < 1 || block_length > 64 || pow2_8(block_length) * head_dim > 4096) return DLLM_ERR_INVALID_ARG;
  if (P < 0 || cap < P || P % block_length || (P > 0 && (!d_kc || !d_vc)) || (d_kept && !d_n_kept))
    return DLLM_ERR_INVALID_ARG;
  const int mode = act_dtype == DLLM_F32 ? MODE_F32 : MODE_BF16;
  const int LB = block_length;
  const AttnPlan pl = attn_plan(mode, rows, n_heads, LB, LB, head_dim, P + LB, d_kept ? 1 : 0, P, 0);
  if (h_plan) {
    h_plan[0] = pl.kind;
    h_plan[1] = pl.split;
    h_plan[2] = pl.n_splits;
  }
  const size_t nq = (size_t)rows * n_heads;
  const size_t qrows = pow2_8(LB) > 32 ? pow2_8(LB) : 32;
  float* part = nullptr;
  const size_t n_o = nq * pl.n_splits * qrows * head_dim, n_ml = nq * pl.n_splits * qrows * 2;
  if (hipMalloc(&part, sizeof(float) * (n_o + n_ml)) != hipSuccess) return DLLM_ERR_HIP;
  hipStream_t s = (hipStream_t)stream;
  const long long row_stride = (long long)n_heads * cap * head_dim, head_stride = (long long)cap * head_dim;
  hipError_t e = launch_attn(pl, mode, d_q, rows, n_heads, head_dim, LB, LB, d_kc, d_vc, row_stride, head_stride,
                             d_bk, d_bv, d_kept, d_n_kept, cap, P, 0, P, part, part + n_o, d_out, d_lse, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  (void)hipFree(part);
  return e == hipSuccess ? DLLM_OK : DLLM_ERR_HIP;
}

// ---- decision checks on given inputs (test support; these allocate and free
// temporary device memory and synchronise the stream) ----

int dllm_debug_route(const float* d_logits, const float* d_bias, int32_t n, int32_t n_experts, int32_t top_k,
                     int32_t* d_idx, float* d_gates, void* stream) {
  if (!d_logits || !d_bias || !d_idx || !d_gates || n < 0 || n_experts < 1 || n_experts > 256 || top_k < 1 ||
      top_k > 16 || top_k > n_experts)
    return DLLM_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (launch_router_topk(d_logits, 1, d_bias, n, n_experts, top_k, d_idx, d_gates, nullptr, nullptr, s) != hipSuccess)
    return DLLM_ERR_HIP;
  return hipStreamSynchronize(s) == hipSuccess ? DLLM_OK : DLLM_ERR_HIP;
}

int dllm_debug_unmask(const int32_t* d_ids_in, const float* d_logits, int32_t n_seq, int32_t block_length,
                      int32_t v_sub, int32_t vocab_lo, int32_t mask_id, int32_t steps, int32_t t, int32_t confidence,
                      int32_t use_threshold, float threshold, int32_t* d_ids_out, int32_t* d_remaining,
                      float* d_conf, int32_t* d_xhat, void* stream) {
  if (!d_ids_in || !d_logits || !d_ids_out || !d_remaining || !d_conf || !d_xhat) return DLLM_ERR_INVALID_ARG;
  if (n_seq < 1 || block_length < 1 || block_length > 64 || n_seq * block_length > 1024 || v_sub < 1 ||
      steps < 1 || t < 0 || t >= steps || confidence < 0 || confidence > 2)
    return DLLM_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  const int nent = n_seq * block_length;
  const int ntiles = (v_sub + kHeadCols - 1) / kHeadCols;
  int32_t* tmp = nullptr;
  float* part = nullptr;
  if (hipMalloc(&tmp, sizeof(int32_t) * (4 * nent + 8)) != hipSuccess) return DLLM_ERR_HIP;
  if (hipMalloc(&part, sizeof(float) * (size_t)nent * ntiles * 5) != hipSuccess) {
    (void)hipFree(tmp);
    return DLLM_ERR_HIP;
  }
  int32_t* row_map = tmp;
  int32_t* entry_pos = tmp + 2 * nent;
  int32_t* seq_off = tmp + 3 * nent;
  int32_t* n_rows = seq_off + n_seq + 1;
  int32_t* n_entries = n_rows + 1;
  bool ok = launch_fill_f32(d_conf, -INFINITY, nent, s) == hipSuccess;
  ok = ok && launch_mask_list(d_ids_in, n_seq, block_length, mask_id, 0, row_map, entry_pos, seq_off, n_rows,
                              n_entries, s) == hipSuccess;
  ok = ok && launch_conf_partial(d_logits, n_entries, entry_pos, nent, v_sub, 0, 0.f, part, s) == hipSuccess;
  ok = ok && launch_conf_merge(part, n_entries, nent, v_sub, vocab_lo, entry_pos, confidence, d_conf, d_xhat, nent,
                               s) == hipSuccess;
  ok = ok && launch_select_commit(d_ids_in, d_conf, d_xhat, n_seq, block_length, mask_id, steps, t, use_threshold,
                                  threshold, d_ids_out, d_remaining, s) == hipSuccess;
  ok = ok && hipStreamSynchronize(s) == hipSuccess;
  (void)hipFree(tmp);
  (void)hipFree(part);
  return ok ? DLLM_OK : DLLM_ERR_HIP;
}

int dllm_debug_retention(const float* d_score, int32_t rows, int32_t P, float keep_ratio, const int32_t* d_ids,
                         int32_t vis_lo, int32_t vis_hi, float image_keep_ratio, float text_keep_ratio,
                         int32_t* d_kept, int32_t* d_count, void* stream) {
  auto ratio_ok = [](float r) { return r > 0.f && r <= 1.f; };
  if (!d_score || !d_kept || !d_count || rows < 1 || P < 1) return DLLM_ERR_INVALID_ARG;
  if (d_ids ? !(ratio_ok(image_keep_ratio) && ratio_ok(text_keep_ratio)) : !ratio_ok(keep_ratio))
    return DLLM_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (launch_retention(d_score, rows, P, P, d_ids, vis_lo, vis_hi, d_ids ? text_keep_ratio : keep_ratio,
                       image_keep_ratio, d_kept, d_count, s) != hipSuccess)
    return DLLM_ERR_HIP;
  return hipStreamSynchronize(s) == hipSuccess ? DLLM_OK : DLLM_ERR_HIP;
}

int dllm_pack_gate_up(const dllm_model_config* cfg, const void* d_src, void* d_dst, void* stream) {
  if (!cfg || !d_src || !d_dst || d_src == d_dst) return DLLM_ERR_INVALID_ARG;
  const int kc = cfg->expert_dtype == DLLM_FP8_E4M3 ? 64 : 32;   // reduction elements per fragment
  if (cfg->n_layers < 1 || cfg->n_experts < 1 || cfg->expert_ffn < 16 || cfg->expert_ffn % 16 || cfg->hidden < kc ||
      cfg->hidden % kc)
    return DLLM_ERR_INVALID_ARG;
  if (cfg->expert_dtype != DLLM_F32 && cfg->expert_dtype != DLLM_BF16 && cfg->expert_dtype != DLLM_FP8_E4M3)
    return DLLM_ERR_INVALID_ARG;
  const long long n_mats = (long long)cfg->n_layers * cfg->n_experts;
  const size_t bytes = (size_t)n_mats * cfg->expert_ffn * cfg->hidden * elem_size(cfg->expert_dtype);
  const char* s0 = (const char*)d_src;
  const char* d0 = (const char*)d_dst;
  if (s0 < d0 + bytes && d0 < s0 + bytes) return DLLM_ERR_INVALID_ARG;   // overlap
  if (launch_pack_fragments(d_src, d_dst, n_mats, cfg->expert_ffn, cfg->hidden, elem_size(cfg->expert_dtype),
                            (hipStream_t)stream) != hipSuccess)
    return DLLM_ERR_HIP;
  return DLLM_OK;
}

int dllm_debug_decode_fp8(const uint8_t* d_codes, int32_t n, float* d_out, void* stream) {
  if (!d_codes || !d_out || n < 0) return DLLM_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (launch_decode_fp8(d_codes, n, d_out, s) != hipSuccess) return DLLM_ERR_HIP;
  return hipStreamSynchronize(s) == hipSuccess ? DLLM_OK : DLLM_ERR_HIP;
}

int dllm_profile_enable(dllm_ctx* ctx, int32_t groups) {
  if (!ctx) return DLLM_ERR_INVALID_ARG;
  if (groups & ~DLLM_PROF_ALL) return fail(ctx, DLLM_ERR_INVALID_ARG, "unknown launch timing group");
  if (groups && ctx->ev.empty()) {
    ctx->ev.resize(4096);
    ctx->ev_cat.resize(4096);
    for (auto& e : ctx->ev)
      if (hipEventCreate(&e) != hipSuccess) return fail(ctx, DLLM_ERR_HIP, "hipEventCreate failed");
  }
  ctx->prof_mask = (uint32_t)groups;   // recorded pairs stay pending until read (no wait here)
  return DLLM_OK;
}

int dllm_profile_read(dllm_ctx* ctx, double* h_ms, long long* h_count) {
  if (!ctx || !h_ms || !h_count) return DLLM_ERR_INVALID_ARG;
  prof_flush(ctx);
  for (int i = 0; i < DLLM_PROF_GROUPS; ++i) {
    h_ms[i] = ctx->prof_ms[i];
    h_count[i] = ctx->prof_n[i];
    ctx->prof_ms[i] = 0;
    ctx->prof_n[i] = 0;
  }
  return DLLM_OK;
}

}  // extern "C"
