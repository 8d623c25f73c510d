// Internal declarations shared by the runtime and the kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace dllm {

enum Mode { MODE_F32 = 0, MODE_BF16 = 1, MODE_FP8 = 2 };

// Rows of an expert work item (one launch tile covers up to this many rows;
// 2 MFMA row tiles keep the expert kernels within 128 VGPRs).
#ifndef DLLM_ROWCHUNK
#define DLLM_ROWCHUNK 32
#endif
constexpr int kRowChunk = DLLM_ROWCHUNK;
// Largest hidden size (the combine kernel holds a row in registers).
constexpr int kMaxHidden = 8192;
// Most (token, expert) slots of one forward pass.
constexpr int kMaxSlots = 65536;
// Most tokens of a forward pass that routes in slot order (no permutation).
constexpr int kDirectMaxTokens = 64;
// 32-bit words of an expert bit set (E <= 256).
constexpr int kMaskWords = 8;
// Keys per attention split (one workgroup) and per inner tile.
constexpr int kAttnSplit = 256;       // keys per workgroup, float32 / long-block attention
constexpr int kAttnSplitMfma = 128;   // keys per workgroup, matrix-core attention (4 x 32)
#ifndef DLLM_ATTN_STREAM_UNITS
#define DLLM_ATTN_STREAM_UNITS 256
#endif
constexpr int kAttnStreamUnits = DLLM_ATTN_STREAM_UNITS; // target workgroups of the streaming attention
constexpr int kAttnTile = 64;
// Columns of the LM head handled by one confidence partial.
constexpr int kHeadCols = 256;

// Retained count ceil(r n) of a pool of n positions, with a relative 1e-6
// guard for the float32 representation of decimal ratios (0.8f * 100 =
// 80.0000012 keeps 80), clamped to [0, n].  Same double arithmetic on the
// host and the device.
__host__ __device__ inline int keep_count(float ratio, int n) {
  double v = ceil((double)ratio * (double)n * (1.0 - 1e-6));
  if (v < 0) v = 0;
  if (v > n) v = n;
  return (int)v;
}

struct ExpertArgs {
  const void* X;          // act [M][D] normed inputs (token-major)
  const int4* items;      // work items {expert, first row, rows, 0}
  const int32_t* n_items; // device count
  const int32_t* off;     // [E+2] expert-major row offsets (E = shared)
  const int32_t* tok;     // [S+M] expert-major slot -> token
  const float* gate_rows; // gate weight of each output row (expert-major or slot order)
  const int32_t* route;   // slot-order mode: [S] routed expert of slot s (null: work-list mode)
  const uint32_t* masks;  // slot-order mode: [kMaskWords] bit set of the selected experts
  const void* wg; const void* wu; const void* wd;    // layer base of routed experts
  const float* sg; const float* su; const float* sd; // fp8 row scales (layer base)
  const void* swg; const void* swu; const void* swd; // shared expert (act dtype)
  void* Hmid;             // act [S+M][Fmax]
  void* Y;                // act [S+M][D] expert outputs (float32 in f32 mode, else bf16)
  int D, F, Fs, E, Fmax;
  int M, S, k;            // tokens, slots (M * k), experts per token
  int n_cu;               // compute units of the device (persistent grids)
  int gu_packed;          // routed gate/up weights in the packed fragment layout
};

// ---- launchers (dllm_kernels.hip) ----
hipError_t launch_embed_norm(int mode, const int32_t* ids, int ids_stride, int rows, int n_tok,
                             int rep, int n_embed, const void* embed, const float* gain, float eps,
                             int D, float* h, void* x, const int32_t* ml_ids, int n_seq, int LB, int mask_id,
                             int gm, int32_t* row_map, int32_t* entry_pos, int32_t* seq_off, int32_t* n_rows,
                             int32_t* n_entries, uint32_t* zero_words, int n_zero, hipStream_t s);
// gm: 0 one head row per entry, 1 CFG pairs (gs_a = w), 2 three-way groups of
// 4 rows (gs_a = image scale, gs_b = text scale).
hipError_t launch_head_conf(int mode, const void* X, int D, const int32_t* row_map, const int32_t* n_rows,
                            int max_rows, const void* W, int V, int gm, float gs_a, float gs_b, float* part,
                            hipStream_t s);
// LM head + confidence partials: the streaming kernel above for few head rows,
// the LDS-tiled one (128 columns per partial) for more; head_partial_tiles
// gives the partials per entry of the chosen kernel.
constexpr int kHeadTiledMin = 256;   // 128 x 128 tiles from which the tiled head runs
bool head_tiled_ok(int mode, int max_rows, int V);
int head_partial_tiles(int mode, int max_rows, int V);
hipError_t launch_head(int mode, const void* X, int D, const int32_t* row_map, const int32_t* n_rows, int max_rows,
                       const void* W, int V, int gm, float gs_a, float gs_b, float* part, hipStream_t s);
hipError_t launch_conf_select(const float* part, int ntiles, const int32_t* seq_off, const int32_t* entry_pos,
                              int vocab_lo, int strategy, const int32_t* ids_in, float* conf, int32_t* xhat,
                              int n_seq, int LB, int mask_id, int steps, int t, int use_threshold, float threshold,
                              int32_t* ids_out, int32_t* remaining, hipStream_t s);
// ss_part (optional): per row and 16-column tile, the sum of squares of the
// written C values ([M][ceil(N / 16)]).
hipError_t launch_gemm(int mode, const void* A, int lda, const int32_t* row_map, int M,
                       const int32_t* M_dev, const void* W, int ldw, int N, int K,
                       float* C, int ldc, int accumulate, hipStream_t s, float* ss_part = nullptr);
// Router logits C = RMSNorm(h) W^T, the norm from ss_part ([M][n_part] sums of
// squares of h); also stores the normalized activations x ([M][K]).  The K
// range is split router_k_split(K) ways: C holds [M][N][split] partials.
constexpr int kRouterSplit = 8;
int router_k_split(int K);
hipError_t launch_router_norm(int mode, const float* h, const float* gain, const float* ss_part, int n_part,
                              float eps, int M, const void* W, int N, int K, float* C, void* x, hipStream_t s);
hipError_t launch_qkv_rope(int mode, const void* X, const void* W, int rows, int n_tok, int D, int H, int dh,
                           int pos0, float base, void* q, void* kdst, void* vdst, long long k_row_stride,
                           long long k_head_stride, int k_pos0, hipStream_t s);
// LDS-tiled bf16 GEMMs for passes of at least 128 rows (prefill, large
// batches): C += A W^T with per-16-column sums of squares, and the QKV
// projection with RoPE and the cache scatter.  *_ok: whether the shape fits.
bool gemm_tiled_ok(int mode, int M, int N, int K);
hipError_t launch_gemm_tiled_acc(const void* A, int lda, int M, const void* W, int ldw, int N, int K, float* C,
                                 int ldc, float* ss_part, hipStream_t s);
bool qkv_tiled_ok(int mode, int M, int D, int H, int dh);
hipError_t launch_qkv_rope_tiled(const void* X, const void* W, int rows, int n_tok, int D, int H, int dh, int pos0,
                                 float base, void* q, void* kdst, void* vdst, long long k_row_stride,
                                 long long k_head_stride, int k_pos0, hipStream_t s);
// Attention launch plan of one pass: the kernel, keys per workgroup (one
// partial each) and workgroups per (row, head, query block).
enum { kAttnFloat = 0, kAttnMfma = 1, kAttnStream = 2, kAttnAppend = 3 };
#ifndef DLLM_ATTN_APPEND_MIN_WG
#define DLLM_ATTN_APPEND_MIN_WG 64
#endif
// fewest workgroups for which an append pass shares key tiles across query blocks
constexpr int kAttnAppendMinWg = DLLM_ATTN_APPEND_MIN_WG;
struct AttnPlan {
  int kind, split, n_splits;
};
// gather: keys reached through the retained-prefix index
AttnPlan attn_plan(int mode, int rows, int H, int n_tok, int LB, int dh, int nk_max, int gather, int n_pref,
                   int append);
// Partials (+ merge unless a single streaming split wrote `out` itself);
// out [rows][n_tok][H * dh], lse [rows][H][n_tok] (may be null).
hipError_t launch_attn(const AttnPlan& pl, int mode, const void* q, int rows, int H, int dh, int n_tok, int LB,
                       const void* kc, const void* vc, long long row_stride, long long head_stride, const void* bk,
                       const void* bv, const int32_t* kept, const int32_t* n_kept, int kept_stride, int n_pref,
                       int append, int P, float* part_o, float* part_ml, void* out, float* lse, hipStream_t s,
                       int kbeg = 0);
// Retained prefix K/V (bf16) of `layers` layers -> contiguous rows [0, pad)
// zero, [pad, pad + n) kept positions (strides in elements).
hipError_t launch_kv_compact(const void* kc, const void* vc, long long src_layer, long long src_row,
                             long long src_head, const int32_t* kept, int kept_stride, int n, int pad, int rows, int H,
                             int dh, int layers, void* kd, void* vd, long long dst_layer, long long dst_row,
                             long long dst_head, hipStream_t s);
hipError_t launch_attn_mass(int mode, const void* q, const float* lse, int rows, int H, int dh,
                            int LB, const void* kc, long long row_stride, long long head_stride,
                            int P, float* mass, int mass_stride, hipStream_t s, float* part = nullptr);
// z_out (optional, inspection): the summed router logits [M][E].
hipError_t launch_router_topk(const float* logits, int n_split, const float* bias, int M, int E, int k,
                              int32_t* idx, float* gates, int32_t* idx_copy, uint32_t* masks, hipStream_t s,
                              float* z_out = nullptr);
// Rows of a work item of the expert kernels (work-list mode) for this shape.
int expert_item_rows(int mode, int D, int F, int Fs);
// Items of at most `chunk` rows (expert_item_rows).
hipError_t launch_permute(const int32_t* idx, const float* gates, int M, int E, int k, int shared, int chunk,
                          int32_t* off, int32_t* tok, float* gate_sorted, int32_t* slot_pos, int4* items,
                          int32_t* n_items, hipStream_t s);
hipError_t launch_expert_gateup(int mode, const ExpertArgs& a, int max_items, hipStream_t s);
hipError_t launch_expert_down(int mode, const ExpertArgs& a, int max_items, hipStream_t s);
hipError_t launch_combine_norm(int mode, float* h, const void* Y, const int32_t* slot_pos,
                               int M, int D, int k, int S, int shared, const float* gain,
                               float eps, void* x, hipStream_t s);
hipError_t launch_mask_list(const int32_t* ids, int n_seq, int LB, int mask_id, int gm,
                            int32_t* row_map, int32_t* entry_pos, int32_t* seq_off, int32_t* n_rows,
                            int32_t* n_entries, hipStream_t s);
hipError_t launch_conf_partial(const float* logits, const int32_t* n_entries,
                               const int32_t* row_of_entry, int max_entries, int V, int cfg,
                               float cfg_scale, float* part, hipStream_t s);
hipError_t launch_conf_merge(const float* part, const int32_t* n_entries, int max_entries,
                             int V, int vocab_lo, const int32_t* entry_pos, int strategy,
                             float* conf, int32_t* xhat, int n_pos, hipStream_t s);
hipError_t launch_select_commit(const int32_t* ids_in, const float* conf, const int32_t* xhat,
                                int n_seq, int LB, int mask_id, int steps, int t,
                                int use_threshold, float threshold, int32_t* ids_out,
                                int32_t* remaining, hipStream_t s);
// Kept prefix positions per row: the top keep_count(r_p, P_p) scores of each
// pool (pids null: one pool, r_text), ascending, and their count.
hipError_t launch_retention(const float* score, int rows, int P, int stride, const int32_t* pids, int vis_lo,
                            int vis_hi, float r_text, float r_image, int32_t* kept, int32_t* n_kept,
                            hipStream_t s);
hipError_t launch_key_norm(int mode, const void* kc, int rows, int n_tok, int H, int dh, long long row_stride,
                           long long head_stride, int P0, float* knorm, int stride, int accumulate,
                           hipStream_t s);
hipError_t launch_prefix_conf(const float* part, int ntiles, int M, int n_tok, int P0, int stride, float* pconf,
                              hipStream_t s);
hipError_t launch_store_ids(const int32_t* ids, int ids_stride, int rows, int n_tok, int P0, int stride,
                            int32_t* out, hipStream_t s);
hipError_t launch_retention_score(const float* knorm, const float* pconf, int rows, int P, int stride, float alpha,
                                  float* score, hipStream_t s);
hipError_t launch_fill_f32(float* p, float v, long long n, hipStream_t s);
// Packed fragment layout of n_mats matrices [rows][K] with es-byte elements.
hipError_t launch_pack_fragments(const void* src, void* dst, long long n_mats, int rows, int K, int es,
                                 hipStream_t s);
hipError_t launch_decode_fp8(const uint8_t* codes, int n, float* out, hipStream_t s);

}  // namespace dllm
