// Host side of the C ABI declared in include/csa.h: argument checks (all of
// them before anything is enqueued), workspace layout, and the orchestration
// of the decode step and the prefill chunk of a hybrid CSA / HCA layer.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "csa.h"
#include "kernels.h"
#include "topk.h"

namespace {

thread_local std::string g_err;

csa_status fail(csa_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

csa_status ok() {
  g_err.clear();
  return CSA_OK;
}

csa_status from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(CSA_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

bool is_pow2_in(int v, int lo, int hi) { return v >= lo && v <= hi && (v & (v - 1)) == 0; }

constexpr size_t kAlign = 256;
constexpr int kMaxIndexEntries = 1 << 19;  // top-k keeps a row's selection bitmap in LDS
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

#define REQUIRE(cond, status, ...)                      \
  do {                                                  \
    if (!(cond)) return fail(status, __VA_ARGS__);      \
  } while (0)

#define REQ_PTR(p)                                                                  \
  do {                                                                              \
    REQUIRE((p) != nullptr, CSA_ERR_ARG, "%s must not be NULL", #p);                \
    REQUIRE(((uintptr_t)(p) & 15) == 0, CSA_ERR_ARG, "%s must be 16-byte aligned", #p); \
  } while (0)
// optional pointers: NULL or 16-byte aligned
#define REQ_ALIGNED(p) \
  REQUIRE(((uintptr_t)(p) & 15) == 0, CSA_ERR_ARG, "%s must be 16-byte aligned", #p)

csa_status check_main_dims(int H, int c) {
  REQUIRE(H >= 1, CSA_ERR_ARG, "H must be >= 1 (got %d)", H);
  REQUIRE(c >= 1, CSA_ERR_ARG, "c must be >= 1 (got %d)", c);
  REQUIRE(H <= 128, CSA_ERR_UNSUPPORTED, "H <= 128 supported (got %d)", H);
  REQUIRE(is_pow2_in(c, 64, 512), CSA_ERR_UNSUPPORTED, "c in {64,128,256,512} supported (got %d)", c);
  return CSA_OK;
}

csa_status check_idx_dims(int H_I, int d_I) {
  REQUIRE(H_I >= 1 && d_I >= 1, CSA_ERR_ARG, "H_I and d_I must be >= 1");
  REQUIRE(H_I <= 64, CSA_ERR_UNSUPPORTED, "H_I <= 64 supported (got %d)", H_I);
  REQUIRE(is_pow2_in(d_I, 32, 128), CSA_ERR_UNSUPPORTED, "d_I in {32,64,128} supported (got %d)", d_I);
  return CSA_OK;
}

}  // namespace

namespace csa {
int set_error(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return status;
}
}  // namespace csa

extern "C" {

const char* csa_last_error(void) { return g_err.c_str(); }

int csa_abi_version(void) { return 4; }

int csa_test_set_fused_wait_polls(int polls) { return csa::set_fused_wait_polls(polls); }

static std::atomic<int> g_fold_fusion{1};
int csa_test_set_fold_fusion(int on) { return g_fold_fusion.exchange(on ? 1 : 0, std::memory_order_relaxed); }

// ------------------------------------------------------------------ a1
csa_status csa_compress(csa_dtype dtype, const void* content_a, const void* logits_a,
                        int logit_width, const float* score_w, const float* bias_a,
                        const void* content_b, const void* logits_b, const float* bias_b,
                        const void* prev_content_b, const void* prev_logits_b, int B, int T,
                        int c, int m, void* out, csa_dtype out_dtype, void* out_scale,
                        int E_cap, int64_t out_first_entry, void* stream) {
  REQUIRE(dtype == CSA_F32 || dtype == CSA_BF16, CSA_ERR_UNSUPPORTED, "compressor input dtype must be F32 or BF16");
  REQUIRE(out_dtype == CSA_F32 || out_dtype == CSA_BF16 || out_dtype == CSA_E4M3 || out_dtype == CSA_MXFP4,
          CSA_ERR_ARG, "bad out_dtype");
  REQ_PTR(content_a);
  REQ_PTR(out);
  REQUIRE(logits_a != nullptr || score_w != nullptr, CSA_ERR_ARG, "need logits_a or score_w");
  REQUIRE(!(logits_a && score_w), CSA_ERR_ARG, "give either logits_a or score_w, not both");
  REQUIRE(!(score_w && content_b), CSA_ERR_ARG, "score_w form has one branch only");
  REQUIRE((content_b == nullptr) == (logits_b == nullptr), CSA_ERR_ARG, "content_b and logits_b go together");
  REQUIRE((prev_content_b == nullptr) == (prev_logits_b == nullptr), CSA_ERR_ARG,
          "prev_content_b and prev_logits_b go together");
  REQUIRE(prev_content_b == nullptr || content_b != nullptr, CSA_ERR_ARG, "previous block needs branch b");
  REQUIRE(B >= 1 && T >= 1 && c >= 1 && m >= 1, CSA_ERR_ARG, "B, T, c, m must be >= 1");
  REQUIRE(m <= 128, CSA_ERR_UNSUPPORTED, "m <= 128 supported (got %d)", m);
  REQUIRE(T % m == 0, CSA_ERR_ARG, "T (%d) must be a multiple of m (%d)", T, m);
  REQUIRE(is_pow2_in(c, 32, 512), CSA_ERR_UNSUPPORTED, "c in {32..512}, power of two (got %d)", c);
  REQUIRE(logit_width == 1 || logit_width == c, CSA_ERR_ARG, "logit_width must be 1 or c");
  REQUIRE((out_dtype != CSA_E4M3 && out_dtype != CSA_MXFP4) || out_scale != nullptr, CSA_ERR_ARG,
          "E4M3 and MXFP4 output need out_scale");
  REQUIRE(out_first_entry >= 0 && out_first_entry + T / m <= (int64_t)E_cap, CSA_ERR_ARG,
          "entries [%lld, %lld) do not fit E_cap %d", (long long)out_first_entry,
          (long long)(out_first_entry + T / m), E_cap);
  csa::CompressArgs a{};
  a.dtype = dtype;
  a.ca = content_a; a.za = logits_a; a.cb = content_b; a.zb = logits_b;
  a.prev_cb = prev_content_b; a.prev_zb = prev_logits_b;
  a.logit_width = logit_width; a.score_w = score_w; a.bias_a = bias_a; a.bias_b = bias_b;
  a.B = B; a.T = T; a.c = c; a.m = m;
  a.out = out; a.out_dtype = out_dtype; a.out_scale = out_scale; a.E_cap = E_cap; a.first = out_first_entry;
  return from_hip(csa::launch_compress(a, (hipStream_t)stream), "csa_compress");
}

// ------------------------------------------------------------------ a2 + a3
size_t csa_index_topk_workspace(int B, int Tq, int E_cap, int k) {
  if (B < 1 || Tq < 1 || E_cap < 1 || k < 1) return 0;
  return align_up(csa::index_topk_ws_bytes(B, Tq, E_cap, k));
}

static bool scaled(int dt) { return dt == CSA_E4M3 || dt == CSA_MXFP4; }

static csa_status check_index(csa_dtype idx_dtype, const void* q_idx, const void* q_scale,
                              const float* w_idx, const void* k_idx, const void* k_scale,
                              const int64_t* q_pos, const int32_t* n_entries, int B, int Tq,
                              int H_I, int d_I, int E_cap, int m, int k, int vis,
                              int32_t* topk_idx, int32_t* topk_cnt) {
  REQUIRE(idx_dtype == CSA_F32 || idx_dtype == CSA_BF16 || idx_dtype == CSA_E4M3 || idx_dtype == CSA_MXFP4,
          CSA_ERR_ARG, "bad idx_dtype");
  REQ_PTR(q_idx); REQ_PTR(w_idx); REQ_PTR(k_idx); REQ_PTR(q_pos); REQ_PTR(n_entries);
  REQ_PTR(topk_idx); REQ_PTR(topk_cnt);
  REQUIRE(!scaled(idx_dtype) || (q_scale && k_scale), CSA_ERR_ARG, "E4M3 and MXFP4 need q_scale and k_scale");
  REQUIRE(B >= 1 && Tq >= 1 && E_cap >= 1 && m >= 1, CSA_ERR_ARG, "B, Tq, E_cap, m must be >= 1");
  csa_status st = check_idx_dims(H_I, d_I);
  if (st != CSA_OK) return st;
  REQUIRE(k >= 1, CSA_ERR_ARG, "k must be >= 1");
  REQUIRE(k <= 2048, CSA_ERR_UNSUPPORTED, "k <= 2048 supported (got %d)", k);
  REQUIRE(m <= 128, CSA_ERR_UNSUPPORTED, "m <= 128 supported");
  REQUIRE(vis == 0 || vis == 1, CSA_ERR_ARG, "bad visibility");
  REQUIRE(E_cap <= kMaxIndexEntries, CSA_ERR_UNSUPPORTED, "E_cap <= %d supported (got %d)",
          kMaxIndexEntries, E_cap);
  return CSA_OK;
}

csa_status csa_index_topk(csa_dtype idx_dtype, const void* q_idx, const void* q_scale,
                          const float* w_idx, const void* k_idx, const void* k_scale,
                          const int64_t* q_pos, const int32_t* n_entries, int B, int Tq, int H_I,
                          int d_I, int E_cap, int m, int k, csa_visibility vis, int score_bf16,
                          int32_t* topk_idx,
                          int32_t* topk_cnt, float* scores, void* ws, size_t ws_bytes,
                          void* stream) {
  csa_status st = check_index(idx_dtype, q_idx, q_scale, w_idx, k_idx, k_scale, q_pos, n_entries,
                              B, Tq, H_I, d_I, E_cap, m, k, vis, topk_idx, topk_cnt);
  if (st != CSA_OK) return st;
  REQUIRE(score_bf16 == 0 || score_bf16 == 1, CSA_ERR_ARG, "score_bf16 must be 0 or 1");
  const size_t need = csa_index_topk_workspace(B, Tq, E_cap, k);
  REQUIRE(ws != nullptr && ws_bytes >= need, CSA_ERR_WORKSPACE, "workspace of %zu bytes required (got %zu)",
          need, ws ? ws_bytes : (size_t)0);
  csa::IndexArgs a{};
  a.idx_dtype = idx_dtype; a.q = q_idx; a.q_scale = scaled(idx_dtype) ? q_scale : nullptr;
  a.w = w_idx; a.keys = k_idx; a.k_scale = scaled(idx_dtype) ? k_scale : nullptr;
  a.score_bf16 = score_bf16;
  a.q_pos = q_pos; a.n_entries = n_entries; a.n_add = 0;
  a.B = B; a.Tq = Tq; a.H_I = H_I; a.d_I = d_I; a.E_cap = E_cap; a.m = m; a.k = k; a.vis = vis;
  a.scores = scores; a.topk_idx = topk_idx; a.topk_cnt = topk_cnt; a.ws = ws;
  return from_hip(csa::launch_index_topk(a, (hipStream_t)stream), "csa_index_topk");
}

// ------------------------------------------------------------------ a4 / a5 + a6
size_t csa_attend_workspace(int B, int Tq, int H, int c, int rows_max) {
  if (B < 1 || Tq < 1 || H < 1 || c < 1 || rows_max < 1) return 0;
  return align_up(csa::attend_ws_bytes(B, Tq, H, c, rows_max));
}

static csa_status check_attend_common(csa_dtype dtype, const void* q, const void* kv, int E_cap,
                                      const void* win, int W_cap, int n_win,
                                      const int64_t* q_pos, int B, int Tq, int H, int c, void* out) {
  REQUIRE(dtype == CSA_F32 || dtype == CSA_BF16, CSA_ERR_UNSUPPORTED, "attention dtype must be F32 or BF16");
  REQ_PTR(q); REQ_PTR(kv); REQ_PTR(win); REQ_PTR(q_pos); REQ_PTR(out);
  REQUIRE(B >= 1 && Tq >= 1 && E_cap >= 1, CSA_ERR_ARG, "B, Tq, E_cap must be >= 1");
  csa_status st = check_main_dims(H, c);
  if (st != CSA_OK) return st;
  REQUIRE(n_win >= 1, CSA_ERR_ARG, "n_win must be >= 1");
  REQUIRE(n_win <= 256, CSA_ERR_UNSUPPORTED, "n_win <= 256 supported");
  REQUIRE(W_cap >= n_win, CSA_ERR_ARG, "W_cap (%d) must hold n_win (%d) rows", W_cap, n_win);
  return CSA_OK;
}

csa_status csa_attend(csa_dtype dtype, const void* q, const void* kv, int E_cap,
                      const int32_t* topk_idx, const int32_t* topk_cnt, int k, const void* win,
                      int W_cap, const int64_t* win_pos0, int n_win, const float* sink,
                      const int64_t* q_pos, float scale, int B, int Tq, int H, int c, void* out,
                      float* lse, void* ws, size_t ws_bytes, void* stream) {
  csa_status st = check_attend_common(dtype, q, kv, E_cap, win, W_cap, n_win, q_pos, B, Tq, H, c, out);
  if (st != CSA_OK) return st;
  REQ_PTR(topk_idx); REQ_PTR(topk_cnt);
  REQUIRE(k >= 1, CSA_ERR_ARG, "k must be >= 1");
  REQUIRE(k <= 2048, CSA_ERR_UNSUPPORTED, "k <= 2048 supported");
  const size_t need = csa_attend_workspace(B, Tq, H, c, k + n_win);
  REQUIRE(ws != nullptr && ws_bytes >= need, CSA_ERR_WORKSPACE, "workspace of %zu bytes required", need);
  csa::AttendArgs a{};
  a.dtype = dtype; a.q = q; a.kv = kv; a.E_cap = E_cap;
  a.topk_idx = topk_idx; a.topk_cnt = topk_cnt; a.k = k; a.dense = 0;
  a.win = win; a.W_cap = W_cap; a.win_pos0 = win_pos0; a.win_pos0_const = 0; a.n_win = n_win;
  a.sink = sink; a.q_pos = q_pos; a.scale = scale;
  a.B = B; a.Tq = Tq; a.H = H; a.c = c; a.out = out; a.lse = lse; a.ws = ws; a.ws_bytes = ws_bytes;
  return from_hip(csa::launch_attend(a, (hipStream_t)stream), "csa_attend");
}

csa_status hca_attend(csa_dtype dtype, const void* q, const void* kv, int E_cap,
                      const int32_t* n_entries, int m, csa_visibility vis, const void* win,
                      int W_cap, const int64_t* win_pos0, int n_win, const float* sink,
                      const int64_t* q_pos, float scale, int B, int Tq, int H, int c, void* out,
                      float* lse, void* ws, size_t ws_bytes, void* stream) {
  csa_status st = check_attend_common(dtype, q, kv, E_cap, win, W_cap, n_win, q_pos, B, Tq, H, c, out);
  if (st != CSA_OK) return st;
  REQ_PTR(n_entries);
  REQUIRE(m >= 1, CSA_ERR_ARG, "m must be >= 1");
  REQUIRE(m <= 128, CSA_ERR_UNSUPPORTED, "m <= 128 supported");
  REQUIRE(vis == 0 || vis == 1, CSA_ERR_ARG, "bad visibility");
  const size_t need = csa_attend_workspace(B, Tq, H, c, E_cap + n_win);
  REQUIRE(ws != nullptr && ws_bytes >= need, CSA_ERR_WORKSPACE, "workspace of %zu bytes required", need);
  csa::AttendArgs a{};
  a.dtype = dtype; a.q = q; a.kv = kv; a.E_cap = E_cap;
  a.n_entries = n_entries; a.n_add = 0; a.m = m; a.vis = vis; a.dense = 1;
  a.win = win; a.W_cap = W_cap; a.win_pos0 = win_pos0; a.win_pos0_const = 0; a.n_win = n_win;
  a.sink = sink; a.q_pos = q_pos; a.scale = scale;
  a.B = B; a.Tq = Tq; a.H = H; a.c = c; a.out = out; a.lse = lse; a.ws = ws; a.ws_bytes = ws_bytes;
  return from_hip(csa::launch_attend(a, (hipStream_t)stream), "hca_attend");
}

// ------------------------------------------------------------------ layer
static int n_streams(const csa_layer_desc* d) { return d->overlap ? 4 : 2; }
static int tail_depth(const csa_layer_desc* d) { return d->overlap ? 3 * d->m : 2 * d->m; }

static csa_status check_desc(const csa_layer_desc* d) {
  REQ_PTR(d);
  REQUIRE(d->kind == CSA_LAYER_CSA || d->kind == CSA_LAYER_HCA, CSA_ERR_ARG, "bad layer kind");
  csa_status st = check_main_dims(d->H, d->c);
  if (st != CSA_OK) return st;
  REQUIRE(d->m >= 1, CSA_ERR_ARG, "m must be >= 1");
  REQUIRE(d->m <= 128, CSA_ERR_UNSUPPORTED, "m <= 128 supported");
  REQUIRE(d->n_win >= 1, CSA_ERR_ARG, "n_win must be >= 1");
  REQUIRE(d->n_win <= 256, CSA_ERR_UNSUPPORTED, "n_win <= 256 supported");
  REQUIRE(d->vis == 0 || d->vis == 1, CSA_ERR_ARG, "bad visibility");
  REQUIRE(d->kv_dtype == CSA_F32 || d->kv_dtype == CSA_BF16 || d->kv_dtype == CSA_FP8BF16, CSA_ERR_UNSUPPORTED,
          "kv_dtype must be F32, BF16 or FP8BF16");
  REQUIRE(d->kv_dtype != CSA_FP8BF16 || d->c == csa::kF8Dims + 64, CSA_ERR_UNSUPPORTED,
          "FP8BF16 entries are 448 + 64 coordinates (c = 512, got %d)", d->c);
  REQUIRE(d->overlap == 0 || d->overlap == 1, CSA_ERR_ARG, "overlap must be 0 or 1");
  REQUIRE(d->split_rows >= 0 && d->split_rows % 16 == 0, CSA_ERR_ARG,
          "split_rows must be 0 or a positive multiple of 16 (got %d)", d->split_rows);
  REQUIRE(d->norm_rope == 0 || d->norm_rope == 1, CSA_ERR_ARG, "norm_rope must be 0 or 1");
  if (d->norm_rope) {
    REQUIRE(d->rope_dims >= 2 && d->rope_dims % 2 == 0 && d->rope_dims <= d->c, CSA_ERR_ARG,
            "rope_dims must be even, 2..c (got %d)", d->rope_dims);
    REQUIRE(d->norm_eps >= 0.f && d->norm_eps < 1e30f, CSA_ERR_ARG, "norm_eps must be finite and >= 0");
  }
  if (d->kind == CSA_LAYER_CSA) {
    st = check_idx_dims(d->H_I, d->d_I);
    if (st != CSA_OK) return st;
    REQUIRE(d->k >= 1, CSA_ERR_ARG, "k must be >= 1");
    REQUIRE(d->k <= 2048, CSA_ERR_UNSUPPORTED, "k <= 2048 supported");
    REQUIRE(d->idx_dtype == CSA_F32 || d->idx_dtype == CSA_BF16 || d->idx_dtype == CSA_E4M3 ||
                d->idx_dtype == CSA_MXFP4,
            CSA_ERR_ARG, "bad idx_dtype");
    REQUIRE(d->score_bf16 == 0 || d->score_bf16 == 1, CSA_ERR_ARG, "score_bf16 must be 0 or 1");
    REQUIRE(d->split_rows == 0 || (d->split_rows <= 2304 &&
                                   (d->k + d->n_win + d->split_rows - 1) / d->split_rows <= csa::kMaxRowSplits),
            CSA_ERR_UNSUPPORTED, "split_rows %d: at most 2304 rows and %d splits of k + n_win rows", d->split_rows,
            csa::kMaxRowSplits);
  }
  return CSA_OK;
}

static csa_status check_state(const csa_layer_desc* d, const csa_layer_state* s) {
  REQ_PTR(s);
  REQUIRE(s->B >= 1 && s->E_cap >= 1, CSA_ERR_ARG, "state B and E_cap must be >= 1");
  REQ_PTR(s->kv_cache); REQ_PTR(s->n_entries); REQ_PTR(s->win_ring); REQ_PTR(s->tail);
  REQ_ALIGNED(s->bias_a); REQ_ALIGNED(s->bias_b); REQ_ALIGNED(s->ibias_a); REQ_ALIGNED(s->ibias_b);
  REQ_ALIGNED(s->sink); REQ_ALIGNED(s->idx_scale);
  if (d->kind == CSA_LAYER_CSA) {
    REQ_PTR(s->idx_cache); REQ_PTR(s->idx_tail);
    REQUIRE(s->E_cap <= kMaxIndexEntries, CSA_ERR_UNSUPPORTED, "E_cap <= %d supported for CSA layers",
            kMaxIndexEntries);
    REQUIRE(!scaled(d->idx_dtype) || s->idx_scale != nullptr, CSA_ERR_ARG,
            "E4M3 and MXFP4 indexer caches need idx_scale");
  }
  if (d->norm_rope) {
    REQ_PTR(s->q_norm_w); REQ_PTR(s->kv_norm_w); REQ_PTR(s->rope_inv_freq);
  }
  REQUIRE(d->kv_dtype != CSA_FP8BF16 || s->kv_scale != nullptr, CSA_ERR_ARG, "FP8BF16 entries need kv_scale");
  if (s->block_table) {
    REQ_ALIGNED(s->block_table);
    REQUIRE(is_pow2_in(s->page_entries, 1, 1 << 20), CSA_ERR_ARG,
            "page_entries must be a power of two (got %d)", s->page_entries);
    REQUIRE(s->E_cap % s->page_entries == 0, CSA_ERR_ARG, "page_entries (%d) must divide E_cap (%d)",
            s->page_entries, s->E_cap);
  }
  return CSA_OK;
}

// the rows of the compressed caches: paged (block_table) or per sequence
static csa::PageMap page_map_of(const csa_layer_state* s) {
  csa::PageMap p{};
  p.table = s->block_table;
  p.shift = 0;
  if (s->block_table)
    while ((1 << p.shift) < s->page_entries) ++p.shift;
  return p;
}

// the activations' dtype (queries, window rows, streams, outputs): bf16
// under the FP8 + BF16 cache entry
static int act_dtype(const csa_layer_desc* d) { return d->kv_dtype == CSA_FP8BF16 ? CSA_BF16 : d->kv_dtype; }

// norm_rope: the prepared queries [B][T][H][c] and (prefill) window rows
// [B][n_win-1+T][c], at the start of the workspace after the fold counters
static size_t prep_q_bytes(const csa_layer_desc* d, int B, int T) {
  return d->norm_rope ? align_up((size_t)B * T * d->H * d->c * (d->kv_dtype == CSA_F32 ? 4 : 2)) : 0;
}
static size_t prep_win_bytes(const csa_layer_desc* d, int B, int T) {
  return d->norm_rope ? align_up((size_t)B * (d->n_win - 1 + T) * d->c * (d->kv_dtype == CSA_F32 ? 4 : 2)) : 0;
}
static csa::NormRope norm_rope_of(const csa_layer_desc* d, const csa_layer_state* s) {
  csa::NormRope nr{};
  nr.on = d->norm_rope;
  nr.rope_dims = d->rope_dims;
  nr.eps = d->norm_eps;
  nr.g_q = s->q_norm_w;
  nr.g_kv = s->kv_norm_w;
  nr.inv_freq = s->rope_inv_freq;
  return nr;
}

// variable-length prefill: each query row's position [B][T] and each
// sequence's first window position [B] (int64), after the prepared rows
static size_t varlen_bytes(int B, int T) {
  return align_up((size_t)B * T * sizeof(int64_t)) + align_up((size_t)B * sizeof(int64_t));
}

// the decode fold's whole-entry staging (norm_rope / FP8BF16): [B][c] fp32
static size_t fold_buf_bytes(const csa_layer_desc* d, int B) {
  return (d->norm_rope || d->kv_dtype == CSA_FP8BF16) ? align_up((size_t)B * d->c * sizeof(float)) : 0;
}

size_t hybrid_layer_workspace(const csa_layer_desc* d, int B, int T, int E_cap) {
  if (!d || B < 1 || T < 1 || E_cap < 1) return 0;
  size_t bytes = align_up((size_t)B * sizeof(int32_t)) + prep_q_bytes(d, B, T) + prep_win_bytes(d, B, T) +
                 varlen_bytes(B, T) + fold_buf_bytes(d, B);
  size_t rows = (size_t)E_cap + d->n_win;
  if (d->kind == CSA_LAYER_CSA) {
    bytes += align_up(csa::index_topk_ws_bytes(B, T, E_cap, d->k));
    rows = (size_t)d->k + d->n_win;
  }
  bytes += align_up(csa::attend_ws_bytes(B, T, d->H, d->c, (int)rows, T == 1 ? d->split_rows : 0));
  return bytes;
}

}  // extern "C"

namespace csa {
// every argument check of a decode step but the workspace's (nothing enqueued)
csa_status decode_check(const csa_layer_desc* d, const csa_layer_state* s, const csa_decode_io* io) {
  csa_status st = check_desc(d);
  if (st != CSA_OK) return st;
  st = check_state(d, s);
  if (st != CSA_OK) return st;
  REQUIRE(d->kind == CSA_LAYER_CSA || d->split_rows == 0 ||
              ((int64_t)s->E_cap + d->n_win + d->split_rows - 1) / d->split_rows <= csa::kMaxRowSplits,
          CSA_ERR_UNSUPPORTED, "split_rows %d: more than %d splits of E_cap + n_win rows", d->split_rows,
          csa::kMaxRowSplits);
  REQ_PTR(io);
  REQ_PTR(io->pos); REQ_PTR(io->q); REQ_PTR(io->x_new); REQ_PTR(io->streams); REQ_PTR(io->out);
  if (d->kind == CSA_LAYER_CSA) {
    REQ_PTR(io->q_idx); REQ_PTR(io->w_idx); REQ_PTR(io->idx_streams);
    REQ_PTR(io->topk_idx); REQ_PTR(io->topk_cnt);
    REQUIRE(!scaled(d->idx_dtype) || io->q_scale != nullptr, CSA_ERR_ARG, "E4M3 and MXFP4 indexers need q_scale");
  }
  return CSA_OK;
}
}  // namespace csa

extern "C" {

csa_status hybrid_layer_decode(const csa_layer_desc* d, csa_layer_state* s, const csa_decode_io* io,
                               void* ws, size_t ws_bytes, void* stream) {
  csa_status st = csa::decode_check(d, s, io);
  if (st != CSA_OK) return st;
  const bool is_csa = d->kind == CSA_LAYER_CSA;
  const int B = s->B;
  const size_t need = hybrid_layer_workspace(d, B, 1, s->E_cap);
  REQUIRE(ws != nullptr && ws_bytes >= need, CSA_ERR_WORKSPACE, "workspace of %zu bytes required", need);
  hipStream_t hs = (hipStream_t)stream;
  char* w = (char*)ws;
  int32_t* fold_counters = (int32_t*)w;
  w += align_up((size_t)B * sizeof(int32_t));
  void* q_prep = w;  // norm_rope
  w += prep_q_bytes(d, B, 1) + prep_win_bytes(d, B, 1);
  float* fold_buf = (float*)w;  // norm_rope / FP8BF16: the fold's whole-entry staging
  w += fold_buf_bytes(d, B);

  csa::FoldArgs f{};
  f.counters = fold_counters;
  f.fold_buf = fold_buf;
  f.dtype = act_dtype(d); f.idx_dtype = is_csa ? d->idx_dtype : -1;
  f.kv_fmt = d->kv_dtype == CSA_FP8BF16; f.kv_scale = s->kv_scale;
  f.B = B; f.c = d->c; f.d_I = d->d_I; f.m = d->m; f.R = tail_depth(d); f.n_win = d->n_win;
  f.vis = d->vis; f.overlap = d->overlap;
  f.pos = io->pos; f.n_entries = s->n_entries; f.streams = io->streams; f.idx_streams = io->idx_streams;
  f.x_new = io->x_new; f.tail = s->tail; f.idx_tail = s->idx_tail; f.win_ring = s->win_ring;
  f.kv_cache = s->kv_cache; f.idx_cache = s->idx_cache; f.idx_scale = s->idx_scale; f.E_cap = s->E_cap;
  f.pg = page_map_of(s);
  f.bias_a = s->bias_a; f.bias_b = s->bias_b; f.ibias_a = s->ibias_a; f.ibias_b = s->ibias_b;
  f.nr = norm_rope_of(d, s);
  f.H = d->H; f.q = io->q; f.q_prep = q_prep;
  csa::IndexArgs x{};
  if (is_csa) {
    x.idx_dtype = d->idx_dtype; x.q = io->q_idx; x.q_scale = scaled(d->idx_dtype) ? io->q_scale : nullptr;
    x.w = io->w_idx; x.keys = s->idx_cache; x.k_scale = scaled(d->idx_dtype) ? s->idx_scale : nullptr;
    x.score_bf16 = d->score_bf16;
    x.q_pos = io->pos; x.n_entries = s->n_entries; x.n_add = 0;
    x.B = B; x.Tq = 1; x.H_I = d->H_I; x.d_I = d->d_I; x.E_cap = s->E_cap; x.m = d->m; x.k = d->k;
    x.vis = d->vis; x.scores = nullptr; x.topk_idx = io->topk_idx; x.topk_cnt = io->topk_cnt; x.ws = w;
    x.pg = page_map_of(s);
  }
  csa::AttendArgs a{};
  a.dtype = act_dtype(d); a.q = io->q; a.kv = s->kv_cache; a.E_cap = s->E_cap;
  a.pg = page_map_of(s);
  a.kv_fmt = d->kv_dtype == CSA_FP8BF16; a.kv_scale = s->kv_scale;
  a.win = s->win_ring; a.W_cap = d->n_win; a.win_pos0 = nullptr; a.win_pos0_const = 0; a.n_win = d->n_win;
  a.sink = s->sink; a.q_pos = io->pos; a.scale = d->scale;
  a.B = B; a.Tq = 1; a.H = d->H; a.c = d->c; a.out = io->out; a.lse = io->lse;
  a.split_rows = d->split_rows;
  if (d->norm_rope) {  // the fold kernel prepares the queries; the output is rotated back
    a.q = q_prep;
    a.derot_freq = s->rope_inv_freq;
    a.rope_dims = d->rope_dims;
  }
  if (!is_csa) {
    a.n_entries = s->n_entries; a.n_add = 0; a.m = d->m; a.vis = d->vis; a.dense = 1;
    a.ws = w; a.ws_bytes = ws_bytes - (size_t)(w - (char*)ws);
  }
  // the fold runs first, unless the scoring kernel (CSA) or the attention
  // (HCA) does it (not with norm_rope: the fold kernel also prepares the
  // queries and normalises whole entries)
  const bool fuse = g_fold_fusion.load(std::memory_order_relaxed) != 0;
  const bool fold_in_scan = fuse && is_csa && !d->norm_rope && csa::index_topk_fuses_fold(x, f);
  const bool fold_in_attend = fuse && !is_csa && !d->norm_rope && csa::attend_fuses_fold(a, f);
  hipError_t e = hipSuccess;
  if (!fold_in_scan && !fold_in_attend) {
    e = csa::launch_fold_append(f, hs);
    if (e != hipSuccess) return from_hip(e, "hybrid_layer_decode/fold");
  }

  if (is_csa) {
    e = csa::launch_index_topk(x, hs, fold_in_scan ? &f : nullptr);
    if (e != hipSuccess) return from_hip(e, "hybrid_layer_decode/index");
    w += align_up(csa::index_topk_ws_bytes(B, 1, s->E_cap, d->k));
    a.topk_idx = io->topk_idx; a.topk_cnt = io->topk_cnt; a.k = d->k; a.dense = 0;
    a.ws = w; a.ws_bytes = ws_bytes - (size_t)(w - (char*)ws);
  }
  return from_hip(csa::launch_attend(a, hs), "hybrid_layer_decode/attend");
}

csa_status hybrid_layer_prefill(const csa_layer_desc* d, csa_layer_state* s, const csa_prefill_io* io,
                                void* ws, size_t ws_bytes, void* stream) {
  csa_status st = check_desc(d);
  if (st != CSA_OK) return st;
  st = check_state(d, s);
  if (st != CSA_OK) return st;
  REQ_PTR(io);
  REQ_PTR(io->q); REQ_PTR(io->win); REQ_PTR(io->streams); REQ_PTR(io->out);
  const bool is_csa = d->kind == CSA_LAYER_CSA;
  if (is_csa) {
    REQ_PTR(io->q_idx); REQ_PTR(io->w_idx); REQ_PTR(io->idx_streams);
    REQ_PTR(io->topk_idx); REQ_PTR(io->topk_cnt);
    REQUIRE(!scaled(d->idx_dtype) || io->q_scale != nullptr, CSA_ERR_ARG, "E4M3 and MXFP4 indexers need q_scale");
  }
  const int B = s->B, T = io->T, m = d->m;
  // variable-length chunks: per-sequence starts and lengths on the device
  const bool varlen = io->seq_pos0 != nullptr;
  REQUIRE((io->seq_pos0 == nullptr) == (io->seq_len == nullptr), CSA_ERR_ARG, "seq_pos0 and seq_len go together");
  if (varlen) {
    REQ_PTR(io->seq_pos0); REQ_PTR(io->seq_len);
    REQUIRE(T >= 1, CSA_ERR_ARG, "T must be >= 1");
  } else {
    REQUIRE(T >= 1 && io->pos0 >= 0, CSA_ERR_ARG, "T must be >= 1 and pos0 >= 0");
    REQUIRE(io->pos0 % m == 0 && T % m == 0, CSA_ERR_UNSUPPORTED,
            "prefill chunks must start and end on block boundaries (pos0 %% m == 0, T %% m == 0) "
            "unless given per sequence (seq_pos0, seq_len)");
    REQUIRE((io->pos0 + T) / m <= (int64_t)s->E_cap, CSA_ERR_ARG, "E_cap too small for the chunk's entries");
  }
  const size_t need = hybrid_layer_workspace(d, B, T, s->E_cap);
  REQUIRE(ws != nullptr && ws_bytes >= need, CSA_ERR_WORKSPACE, "workspace of %zu bytes required", need);
  hipStream_t hs = (hipStream_t)stream;
  char* w = (char*)ws + align_up((size_t)B * sizeof(int32_t));
  void* q_prep = w;  // norm_rope: prepared queries, then window rows
  void* win_prep = w + prep_q_bytes(d, B, T);
  w += prep_q_bytes(d, B, T) + prep_win_bytes(d, B, T);
  int64_t* vl_qpos = (int64_t*)w;  // variable-length chunks: query positions, window starts
  int64_t* vl_win0 = (int64_t*)(w + align_up((size_t)B * T * sizeof(int64_t)));
  w += varlen_bytes(B, T);
  const csa::NormRope nr = norm_rope_of(d, s);
  const int S = n_streams(d), R = tail_depth(d);
  const int64_t first = varlen ? 0 : io->pos0 / m;
  const int n_new = varlen ? 0 : T / m;  // (variable-length: the counts are set first)
  const size_t esz = act_dtype(d) == CSA_F32 ? 4 : 2;
  hipError_t e = hipSuccess;
  if (varlen) {
    csa::VarlenArgs v{};
    v.B = B; v.T = T; v.m = m; v.n_win = d->n_win; v.E_cap = s->E_cap;
    v.seq_pos0 = io->seq_pos0; v.seq_len = io->seq_len;
    v.q_pos = vl_qpos; v.win_pos0 = vl_win0; v.n_entries = s->n_entries;
    e = csa::launch_varlen_setup(v, hs);
    if (e != hipSuccess) return from_hip(e, "hybrid_layer_prefill/varlen");
  }

  // compress the chunk's blocks: main entries, then (CSA) indexer keys
  auto compress = [&](const void* streams, int width, const void* tail, void* out, int out_dtype,
                      void* out_scale, const float* ba, const float* bb, bool overlap, bool prep) -> hipError_t {
    csa::CompressArgs c{};
    if (prep) c.nr = nr;
    const int ns = overlap ? 4 : 2;
    const char* base = (const char*)streams;
    const size_t plane = (size_t)T * width * esz;
    c.dtype = act_dtype(d);
    c.ca = base; c.za = base + plane;
    c.cb = overlap ? base + 2 * plane : nullptr;
    c.zb = overlap ? base + 3 * plane : nullptr;
    c.seq_stride = (size_t)ns * T * width;
    if (varlen) {
      c.seq_pos0 = io->seq_pos0; c.seq_len = io->seq_len; c.tail = tail; c.R = R;
    } else if (overlap && io->pos0 > 0) {
      const char* tb = (const char*)tail;
      const size_t slot = (size_t)((io->pos0 - m) % R);
      c.prev_cb = tb + ((size_t)2 * R + slot) * width * esz;
      c.prev_zb = tb + ((size_t)3 * R + slot) * width * esz;
      c.prev_seq_stride = (size_t)ns * R * width;
    }
    c.logit_width = width; c.score_w = nullptr; c.bias_a = ba; c.bias_b = overlap ? bb : nullptr;
    c.B = B; c.T = T; c.c = width; c.m = m;
    c.out = out; c.out_dtype = out_dtype; c.out_scale = out_scale; c.E_cap = s->E_cap; c.first = first;
    c.pg = page_map_of(s);
    return csa::launch_compress(c, hs);
  };
  e = compress(io->streams, d->c, s->tail, s->kv_cache, d->kv_dtype, s->kv_scale, s->bias_a,
                          s->bias_b, d->overlap != 0, d->norm_rope != 0);
  if (e != hipSuccess) return from_hip(e, "hybrid_layer_prefill/compress");
  csa::AttendArgs a{};
  if (is_csa) {
    e = compress(io->idx_streams, d->d_I, s->idx_tail, s->idx_cache, d->idx_dtype, s->idx_scale,
                 s->ibias_a, s->ibias_b, true, false);
    if (e != hipSuccess) return from_hip(e, "hybrid_layer_prefill/compress_idx");
  }
  if (is_csa) {
    csa::IndexArgs x{};
    x.idx_dtype = d->idx_dtype; x.q = io->q_idx; x.q_scale = scaled(d->idx_dtype) ? io->q_scale : nullptr;
    x.w = io->w_idx; x.keys = s->idx_cache; x.k_scale = scaled(d->idx_dtype) ? s->idx_scale : nullptr;
    x.score_bf16 = d->score_bf16;
    x.q_pos = varlen ? vl_qpos : nullptr; x.q_pos0 = io->pos0; x.n_entries = s->n_entries; x.n_add = n_new;
    x.B = B; x.Tq = T; x.H_I = d->H_I; x.d_I = d->d_I; x.E_cap = s->E_cap; x.m = m; x.k = d->k;
    x.vis = d->vis; x.scores = nullptr; x.topk_idx = io->topk_idx; x.topk_cnt = io->topk_cnt; x.ws = w;
    x.pg = page_map_of(s);
    e = csa::launch_index_topk(x, hs);
    if (e != hipSuccess) return from_hip(e, "hybrid_layer_prefill/index");
    w += align_up(csa::index_topk_ws_bytes(B, T, s->E_cap, d->k));
    a.topk_idx = io->topk_idx; a.topk_cnt = io->topk_cnt; a.k = d->k; a.dense = 0;
  } else {
    a.n_entries = s->n_entries; a.n_add = n_new; a.m = m; a.vis = d->vis; a.dense = 1;
  }
  a.dtype = act_dtype(d); a.q = io->q; a.kv = s->kv_cache; a.E_cap = s->E_cap;
  a.kv_fmt = d->kv_dtype == CSA_FP8BF16; a.kv_scale = s->kv_scale;
  a.pg = page_map_of(s);
  a.win = io->win; a.W_cap = d->n_win - 1 + T; a.win_pos0 = varlen ? vl_win0 : nullptr;
  a.win_pos0_const = io->pos0 - (d->n_win - 1); a.n_win = d->n_win;
  a.sink = s->sink; a.q_pos = varlen ? vl_qpos : nullptr; a.q_pos0 = io->pos0; a.scale = d->scale;
  a.B = B; a.Tq = T; a.H = d->H; a.c = d->c; a.out = io->out; a.lse = io->lse;
  a.ws = w; a.ws_bytes = ws_bytes - (size_t)(w - (char*)ws);
  if (d->norm_rope) {
    // the chunk's queries and window rows prepared for the attention
    csa::PrepArgs pa{};
    pa.dtype = act_dtype(d); pa.B = B; pa.T = T; pa.H = d->H; pa.c = d->c; pa.n_win = d->n_win;
    pa.pos0 = io->pos0; pa.seq_pos0 = io->seq_pos0;
    pa.nr = nr; pa.q = io->q; pa.win = io->win; pa.q_prep = q_prep; pa.win_prep = win_prep;
    e = csa::launch_prep_rows(pa, hs);
    if (e != hipSuccess) return from_hip(e, "hybrid_layer_prefill/prep");
    a.q = q_prep;
    a.win = win_prep;
    a.derot_freq = s->rope_inv_freq;
    a.rope_dims = d->rope_dims;
  }
  e = csa::launch_attend(a, hs);
  if (e != hipSuccess) return from_hip(e, "hybrid_layer_prefill/attend");

  csa::PrefillStateArgs p{};
  p.dtype = act_dtype(d); p.B = B; p.T = T; p.c = d->c; p.d_I = d->d_I; p.R = R; p.n_win = d->n_win; p.S = S;
  p.pos0 = io->pos0; p.win = d->norm_rope ? win_prep : io->win;  // the ring holds prepared rows
  p.streams = io->streams; p.idx_streams = is_csa ? io->idx_streams : nullptr;
  p.win_ring = s->win_ring; p.tail = s->tail; p.idx_tail = s->idx_tail; p.n_entries = s->n_entries;
  p.new_entries = n_new;
  p.seq_pos0 = io->seq_pos0; p.seq_len = io->seq_len;
  return from_hip(csa::launch_prefill_state(p, hs), "hybrid_layer_prefill/state");
}

}  // extern "C"
