/*
 * csa.h -- C ABI of the MI355X (gfx950) CSA / HCA hybrid-attention hot path.
 *
 * The method is DeepSeek-V4's hybrid attention layer as described in
 *   [book]  "DeepSeek-V4" (slop-6tp.pages.dev/papers-html/dsv4), ch. 5-8, 13;
 *   [note]  "2026 DeepSeek-V4" (awesome.papernotes.org), "Method Deep Dive",
 *           "Key design 1" (CSA) and "Key design 2" (HCA) with their equations.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers, row-major and contiguous, with
 *   the shapes given per argument, and 16-byte aligned (kernels load rows in
 *   16-byte pieces); a misaligned pointer is CSA_ERR_ARG.  (There are no
 *   strided views: a layer whose compressed caches live in a larger shared
 *   allocation passes it as a paged pool with a block table, see
 *   csa_layer_state.)  The caller owns every buffer (inputs,
 *   outputs, caches, state, workspace); the library never allocates, frees or
 *   keeps a pointer after the call returns.
 * - Work is enqueued asynchronously on `stream` (a hipStream_t passed as
 *   void*; NULL = the default stream).  Buffers must stay alive until the
 *   caller synchronises that stream.
 * - Every entry point returns a csa_status.  All argument checks run on the
 *   host before anything is enqueued, so an error has no side effects.
 *   csa_last_error() returns a thread-local message about the last failure.
 *   Nothing is printed; no C++ exception crosses the ABI.
 * - Positions are 0-based token positions (int64).  Entry ids are int32.
 * - Workspaces ("ws") are caller-allocated device memory of at least the size
 *   the matching *_workspace() function returns.  A workspace must be
 *   zero-filled once when first allocated; every call returns the counters it
 *   uses to zero before it completes.  Calls that share a workspace must be
 *   ordered on one stream, and must be calls of one entry point with one
 *   configuration (the same descriptor and sizes): other calls place other
 *   data where its counters live, so a workspace passed to a different entry
 *   point or configuration must be zero-filled again first.
 * - Supported shapes: c in {64, 128, 256, 512}; d_I in {32, 64, 128};
 *   H <= 128; H_I <= 64; 1 <= m <= 128; k <= 2048; n_win <= 256; at most
 *   2^19 indexer entries per sequence (a 2M-token context at m = 4).  Other
 *   shapes return CSA_ERR_UNSUPPORTED (there is no slow fallback).
 */
#ifndef CSA_H
#define CSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CSA_OK = 0,
  CSA_ERR_ARG = 1,         /* null pointer, bad size, inconsistent arguments  */
  CSA_ERR_UNSUPPORTED = 2, /* valid but outside the supported shapes / dtypes */
  CSA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required      */
  CSA_ERR_DEVICE = 4       /* the HIP runtime reported an error on launch     */
} csa_status;

typedef enum {
  CSA_F32 = 0,  /* IEEE binary32                                            */
  CSA_BF16 = 1, /* bfloat16                                                 */
  CSA_E4M3 = 2, /* OCP FP8 E4M3FN, one float32 scale per vector (v = q * s) */
  CSA_MXFP4 = 3, /* OCP MX FP4: E2M1 values, two per byte (element 2j in the
                   low nibble of byte j), one E8M0 scale byte per block of 32
                   consecutive values (v = e2m1 * 2^(code - 127)); [book]
                   ch. 16 "Why use fine-grained scales?", ch. 8: a 128-dim
                   indexer key is 64 bytes plus four scale bytes            */
  CSA_FP8BF16 = 4 /* the main compressed entry of [book] ch. 8 "The main
                   compressed-entry payload" (c = 512): 448 E4M3FN codes
                   with one float32 scale per entry (max |v[0:448]| / 448)
                   then the 64 rotary coordinates as bf16, 576 bytes; as a
                   layer's kv_dtype the activations (queries, window rows,
                   token streams, outputs) are bf16                          */
} csa_dtype;

/* Which compressed entries a query at position t may read ([book] ch. 5 "When
 * an entry becomes available"; the printed condition is garbled).  The
 * default admits only blocks that end before the query's own block. */
typedef enum {
  CSA_VIS_PRIOR_BLOCKS = 0, /* entry s visible iff s < floor(t / m)       */
  CSA_VIS_COMPLETED = 1     /* entry s visible iff s < floor((t + 1) / m) */
} csa_visibility;

/* Thread-local text of the last error, or "" after a successful call. */
const char* csa_last_error(void);

/* ABI version of this header (bumped on incompatible change; 2 added
 * csa_layer_desc.split_rows; 3 added CSA_MXFP4 with untyped scale pointers,
 * csa_layer_desc.score_bf16, the score_bf16 argument of csa_index_topk, the
 * normalisation / rotary fields of csa_layer_desc and csa_layer_state, and
 * the FP8BF16 main entry with csa_layer_state.kv_scale; 4 added the paged
 * cache, csa_layer_state.block_table and page_entries, and variable-length
 * prefill chunks, csa_prefill_io.seq_pos0 and seq_len). */
int csa_abi_version(void);

/* ------------------------------------------------------------------------
 * a1. Compressor: fold token streams into compressed entries.
 *
 * [note] "Key design 1" equation (CSA, two branches with overlap) and "Key
 * design 2" equation (HCA, one branch); [book] ch. 5 "One weight distribution
 * per coordinate", "Which positions enter a compressed block", and the
 * start-of-sequence rule.
 *
 * For chunk entry i (0 <= i < T/m) and coordinate r, the logits
 *   Za[m*i+j, r] + Ba[j, r]        (j < m, current block, branch a)
 *   Zb[m*(i-1)+j, r] + Bb[j, r]    (j < m, previous block, branch b)
 * go through one softmax across the source positions and the entry is the
 * weighted sum of Ca / Cb.  For i = 0 the previous block is prev_content_b /
 * prev_logits_b; if those are NULL the chunk starts the sequence and entry 0
 * has no branch-b sources.  With content_b == NULL the compressor has one
 * branch (HCA form).
 *
 *   dtype          F32 or BF16: dtype of every content / logit input.
 *   content_a      [B][T][c]
 *   logits_a       [B][T][logit_width]; logit_width is c (per coordinate) or
 *                  1 (one scalar per token, shared by all coordinates).  May
 *                  be NULL when score_w is given.
 *   score_w        [c] float32 or NULL: when logits_a is NULL the scalar
 *                  logit of a token is score_w . content_a[token] (one-branch
 *                  form only).
 *   bias_a         [m][c] float32 or NULL (= 0).
 *   content_b, logits_b, bias_b   branch b, same shapes, or NULL (no overlap).
 *   prev_content_b, prev_logits_b [B][m][c] / [B][m][logit_width] or NULL.
 *   B, T, c, m     T % m == 0.
 *   out            [B][E_cap][c] in out_dtype; entry i of sequence b goes to
 *                  row out_first_entry + i.  out_first_entry + T/m <= E_cap.
 *   out_dtype      F32, BF16, E4M3 (then out_scale, float32 [B][E_cap],
 *                  receives scale = max|entry| / 448 and the codes round to
 *                  nearest even; an all-zero entry gets scale 1) or MXFP4
 *                  (out is [B][E_cap][c/2] bytes and out_scale, uint8
 *                  [B][E_cap][c/32], receives each block's E8M0 code
 *                  floor(log2 max|block|) - 2 + 127, the smallest code for
 *                  an all-zero block; values round to the nearest E2M1
 *                  value, ties to the even code, saturating at 6).
 * ------------------------------------------------------------------------ */
csa_status csa_compress(csa_dtype dtype, const void* content_a, const void* logits_a,
                        int logit_width, const float* score_w, const float* bias_a,
                        const void* content_b, const void* logits_b, const float* bias_b,
                        const void* prev_content_b, const void* prev_logits_b, int B, int T,
                        int c, int m, void* out, csa_dtype out_dtype, void* out_scale,
                        int E_cap, int64_t out_first_entry, void* stream);

/* ------------------------------------------------------------------------
 * a2 + a3. Lightning indexer and per-query top-k.
 *
 * I[t, s] = sum_h w[t, h] * ReLU(q[t, h] . K[s])   ([note] "Key design 1"
 * indexer equation; [book] ch. 6 "The index score": w may be negative), over
 * the entries visible to the query (vis, m, q_pos, n_entries), followed by
 * C_t = TopK_k(I[t, :]) ([note] same equation; [book] ch. 6 "Top-k is a budget
 * over compressed entries": all visible entries are kept when fewer than k).
 * Ties between equal float32 scores go to the lower entry id.
 *
 *   idx_dtype  F32, BF16 or E4M3 for q_idx and k_idx.
 *   q_idx      [B][Tq][H_I][d_I];  q_scale [B][Tq][H_I] float32 iff E4M3,
 *              [B][Tq][H_I][d_I/32] uint8 E8M0 codes iff MXFP4 (an MXFP4
 *              vector is d_I/2 bytes).
 *   w_idx      [B][Tq][H_I] float32 head weights.
 *   k_idx      [B][E_cap][d_I];    k_scale [B][E_cap] float32 iff E4M3,
 *              [B][E_cap][d_I/32] uint8 iff MXFP4; NULL otherwise.
 *   score_bf16 1: every score is rounded to bfloat16 (nearest even) before
 *              the selection ([book] ch. 16 "BF16 index scores"), and the
 *              rounded scores are written; ties, then frequent, still go to
 *              the lower id.  0: float32 scores.
 *   q_pos      [B][Tq] int64 query positions.
 *   n_entries  [B] int32 entries present in the cache.
 *   topk_idx   [B][Tq][k] int32 out: selected ids ascending, -1 padded.
 *   topk_cnt   [B][Tq] int32 out: number selected (= min(k, visible)).
 *   scores     [B][Tq][E_cap] float32 out, or NULL.  Only the visible prefix
 *              of each row is written.
 *   ws         workspace of csa_index_topk_workspace(B, Tq, E_cap, k) bytes.
 * ------------------------------------------------------------------------ */
size_t csa_index_topk_workspace(int B, int Tq, int E_cap, int k);
csa_status csa_index_topk(csa_dtype idx_dtype, const void* q_idx, const void* q_scale,
                          const float* w_idx, const void* k_idx, const void* k_scale,
                          const int64_t* q_pos, const int32_t* n_entries, int B, int Tq, int H_I,
                          int d_I, int E_cap, int m, int k, csa_visibility vis, int score_bf16,
                          int32_t* topk_idx,
                          int32_t* topk_cnt, float* scores, void* ws, size_t ws_bytes,
                          void* stream);

/* ------------------------------------------------------------------------
 * a4 + a6. Sparse attention over the selected entries, the window and the
 * sink, merged in one softmax.
 *
 * Every row serves as both key and value for all H heads (shared-KV MQA,
 * [book] ch. 6 "Shared key-value MQA").  For query (b, t) with position
 * p = q_pos[b][t] the rows are kv[b][topk_idx[b][t][0 .. topk_cnt-1]] and the
 * window rows of positions max(0, p-n_win+1) .. p ([book] ch. 7 "The sliding
 * window"), all in one softmax ([note] concat(selected, local_kv)) whose
 * denominator also holds exp(sink[h]) ([book] ch. 7 "Attention sinks"):
 *   o_h = sum_j exp(l_j - M) row_j / (sum_j exp(l_j - M) + exp(z'_h - M)),
 *   l_j = scale * q_h . row_j.
 *
 *   dtype      F32 or BF16 for q, kv, win and out (float32 accumulation).
 *   q          [B][Tq][H][c]
 *   kv         [B][E_cap][c] compressed entries
 *   topk_idx, topk_cnt   as produced by csa_index_topk (ids must be < E_cap).
 *   win        [B][W_cap][c]: the row of position p is row
 *              (p - win_pos0[b]) mod W_cap (a ring buffer uses win_pos0 = 0; a
 *              linear buffer uses its first position).  All window positions
 *              of every query must be present.
 *   sink       [H] float32 logits, or NULL (no sink).
 *   q_pos      [B][Tq] int64.
 *   out        [B][Tq][H][c];  lse [B][Tq][H] float32 out or NULL
 *              (lse = log of the full softmax denominator incl. the sink).
 *   ws         workspace of csa_attend_workspace(B, Tq, H, c, k + n_win).
 * ------------------------------------------------------------------------ */
size_t csa_attend_workspace(int B, int Tq, int H, int c, int rows_max);
csa_status csa_attend(csa_dtype dtype, const void* q, const void* kv, int E_cap,
                      const int32_t* topk_idx, const int32_t* topk_cnt, int k, const void* win,
                      int W_cap, const int64_t* win_pos0, int n_win, const float* sink,
                      const int64_t* q_pos, float scale, int B, int Tq, int H, int c, void* out,
                      float* lse, void* ws, size_t ws_bytes, void* stream);

/* a5 + a6. Dense HCA attention: as csa_attend, with the rows being every
 * visible compressed entry s < min(n_entries[b], vis-limit(q_pos)) plus the
 * window and the sink ([note] "Key design 2"; [book] ch. 7 "Dense attention
 * over compressed history").  ws: csa_attend_workspace(B, Tq, H, c, E_cap +
 * n_win). */
csa_status hca_attend(csa_dtype dtype, const void* q, const void* kv, int E_cap,
                      const int32_t* n_entries, int m, csa_visibility vis, const void* win,
                      int W_cap, const int64_t* win_pos0, int n_win, const float* sink,
                      const int64_t* q_pos, float scale, int B, int Tq, int H, int c, void* out,
                      float* lse, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * a7 + the whole layer.  A layer is described by csa_layer_desc and keeps its
 * cache and bounded state in csa_layer_state ([book] ch. 5 "What is retained
 * during decode": a classical cache of completed entries plus state for the
 * window and the compression tail; ch. 13 heterogeneous KV cache).
 * ------------------------------------------------------------------------ */
typedef enum { CSA_LAYER_CSA = 1, CSA_LAYER_HCA = 2 } csa_layer_kind;

typedef struct {
  int kind;          /* csa_layer_kind                                        */
  int H, c;          /* query heads, entry / head dim                         */
  int H_I, d_I;      /* indexer heads and dim (CSA)                           */
  int m;             /* compression rate (4 for CSA, 128 for HCA)             */
  int overlap;       /* 1: two-branch overlapping compressor (CSA); 0: one    */
  int k;             /* top-k budget (CSA)                                    */
  int n_win;         /* sliding-window width                                  */
  int vis;           /* csa_visibility                                        */
  int kv_dtype;      /* F32 or BF16: activations, caches, outputs; FP8BF16:  */
                     /* 576-byte cache entries, bf16 activations (c = 512)   */
  int idx_dtype;     /* F32, BF16, E4M3 or MXFP4: indexer queries and keys    */
  float scale;       /* attention logit scale (1/sqrt(c) for the pages)       */
  int split_rows;    /* decode: 0 = the attention's row splits are sized for  */
                     /* the batch; > 0 (a multiple of 16) = every query's     */
                     /* rows are cut into splits of this many rows whatever   */
                     /* the batch, so a token's output is bitwise the same    */
                     /* wherever it sits in a batch ([book] ch. 12 "Batch      */
                     /* invariance"); at most 64 splits per query, and at     */
                     /* most 2304 rows per split for CSA (else               */
                     /* CSA_ERR_UNSUPPORTED).  Prefill chunks ignore it.      */
  int score_bf16;    /* CSA: 1 = index scores rounded to bfloat16 before the  */
                     /* top-k (see csa_index_topk); 0 = float32 scores        */
  int norm_rope;     /* 1: the steps on either side of the core attention     */
                     /* ([book] ch. 7 "Query and KV normalization", "Partial  */
                     /* rotary position embeddings", "Why the output is      */
                     /* de-rotated"): every query head and every produced KV  */
                     /* vector (compressed entry, window row) is RMSNorm-ed,  */
                     /* v * g / sqrt(mean(v^2) + norm_eps), then its last     */
                     /* rope_dims coordinates are rotated in pairs (2i, 2i+1) */
                     /* by pos * inv_freq[i]; the output's last rope_dims     */
                     /* coordinates are rotated back by the query position.   */
                     /* Positions: a query or window row its token's, entry e */
                     /* m * e (its block's first token).  0: off.             */
  int rope_dims;     /* rotated coordinates (even, 2..c) when norm_rope       */
  float norm_eps;    /* RMSNorm epsilon when norm_rope                        */
} csa_layer_desc;

/* Number of compressor streams per token: 4 (ca, za, cb, zb) with overlap,
 * else 2 (ca, za); tail ring depth R = 3m with overlap, else 2m. */
typedef struct {
  int B, E_cap;
  void* kv_cache;        /* [B][E_cap][c] kv_dtype                             */
  void* idx_cache;       /* [B][E_cap][d_I] idx_dtype (CSA; MXFP4: d_I/2 bytes) */
  void* idx_scale;       /* E4M3: float32 [B][E_cap]; MXFP4: uint8             */
                         /* [B][E_cap][d_I/32]; NULL otherwise                 */
  int32_t* n_entries;    /* [B] completed entries in the cache                 */
  void* win_ring;        /* [B][n_win][c]: position p lives in slot p % n_win  */
  void* tail;            /* [B][streams][R][c]: position p in slot p % R       */
  void* idx_tail;        /* [B][4][R][d_I] (CSA): the indexer-key streams      */
  const float* bias_a;   /* [m][c] positional biases of branch a (or NULL)     */
  const float* bias_b;   /* [m][c] branch b (or NULL)                          */
  const float* ibias_a;  /* [m][d_I] indexer-key biases (CSA, or NULL)         */
  const float* ibias_b;
  const float* sink;     /* [H] sink logits or NULL                            */
  const float* q_norm_w;       /* [c] RMSNorm scale of the query heads         */
  const float* kv_norm_w;      /* [c] RMSNorm scale of the KV head             */
  const double* rope_inv_freq; /* [rope_dims/2] inverse frequencies (the      */
                               /* caller's scaling, e.g. base^(-2i/rope_dims)) */
                               /* (the three only read when norm_rope)         */
  float* kv_scale;             /* [B][E_cap] per-entry scales (FP8BF16)        */
  /* Paged compressed cache ([book] ch. 13 "Aligning original-token blocks":
   * an allocation unit of original tokens shared by the layers, e.g. 128
   * tokens = 32 CSA entries (m = 4) = 1 HCA entry (m = 128), so one block
   * table serves a CSA and an HCA layer).  NULL: the per-sequence layout
   * above.  Else kv_cache, kv_scale, idx_cache and idx_scale are pools of
   * pages of page_entries rows each (the row layouts above), shared by the
   * sequences, and entry e of sequence b lives in row
   * block_table[b][e / page_entries] * page_entries + e % page_entries.
   * block_table is int32 [B][E_cap / page_entries] on the device; the pages
   * a sequence's entries reach (the visible ones, and those a call
   * appends) must hold ids of pages inside the pools, each page owned by
   * one sequence (the library does not read the pools' sizes).  Entries
   * of a page are appended in order, so a page is allocated before the
   * step or chunk that writes its first entry.  Window ring and tails
   * stay per sequence (the bounded state cache). */
  const int32_t* block_table;
  int page_entries;            /* power of two, divides E_cap (block_table)   */
} csa_layer_state;

/* One decode step: one new token per sequence at position pos[b]. */
typedef struct {
  const int64_t* pos;       /* [B]                                             */
  const void* q;            /* [B][H][c]                                       */
  const void* q_idx;        /* [B][H_I][d_I] (CSA)                             */
  const void* q_scale;      /* E4M3: float32 [B][H_I]; MXFP4: uint8            */
                            /* [B][H_I][d_I/32]                                */
  const float* w_idx;       /* [B][H_I] (CSA)                                  */
  const void* x_new;        /* [B][c] the new token's window row               */
  const void* streams;      /* [B][streams][c] the new token's compressor rows */
  const void* idx_streams;  /* [B][4][d_I] (CSA)                               */
  void* out;                /* [B][H][c]                                       */
  float* lse;               /* [B][H] or NULL                                  */
  int32_t* topk_idx;        /* [B][k] out (CSA)                                */
  int32_t* topk_cnt;        /* [B] out (CSA)                                   */
} csa_decode_io;

/* A prefill chunk of T tokens per sequence starting at position pos0 (all
 * sequences aligned); pos0 % m == 0 and T % m == 0.  Or, with seq_pos0 and
 * seq_len, a variable-length batch ([book] ch. 11 "Packing and attention
 * boundaries"): sequence b's chunk holds positions seq_pos0[b] ..
 * seq_pos0[b] + seq_len[b] - 1 (0 <= seq_len[b] <= T, seq_pos0[b] >= 0;
 * neither needs to be a multiple of m) in rows 0 .. seq_len[b] - 1 of the
 * [B][T] inputs, and pos0 is not used.  A block becomes an entry when its
 * last token is in the chunk; the block's earlier tokens (and, with
 * overlap, the previous block's) come from the state's tail, as the
 * decode fold takes them, so a trailing fragment shorter than m produces no
 * entry and stays in the tail for the next chunk or decode step, and no
 * block mixes two sequences.  The state must be the one the sequence's
 * earlier calls left: n_entries[b] = floor(seq_pos0[b] / m) completed
 * entries and the tails holding the positions before seq_pos0[b].  Rows
 * >= seq_len[b] are padding: they are read (as queries of the sequence's
 * last position) and their outputs and top-k rows are unspecified; the
 * window rows win[b] are those of positions seq_pos0[b] - (n_win - 1) ..
 * Entries past E_cap are not produced (a chunk must not need them). */
typedef struct {
  int64_t pos0;
  int T;
  const void* q;            /* [B][T][H][c]                                    */
  const void* q_idx;        /* [B][T][H_I][d_I] (CSA)                          */
  const void* q_scale;      /* E4M3: float32 [B][T][H_I]; MXFP4: uint8         */
                            /* [B][T][H_I][d_I/32]                             */
  const float* w_idx;       /* [B][T][H_I] (CSA)                               */
  const void* win;          /* [B][n_win-1+T][c]: rows of positions
                               pos0-n_win+1 .. pos0+T-1                        */
  const void* streams;      /* [B][streams][T][c] the chunk's compressor rows  */
  const void* idx_streams;  /* [B][4][T][d_I] (CSA)                            */
  void* out;                /* [B][T][H][c]                                    */
  float* lse;               /* [B][T][H] or NULL                               */
  int32_t* topk_idx;        /* [B][T][k] out (CSA)                             */
  int32_t* topk_cnt;        /* [B][T] out (CSA)                                */
  const int64_t* seq_pos0;  /* [B] device, or NULL (all chunks start at pos0) */
  const int32_t* seq_len;   /* [B] device (with seq_pos0)                      */
} csa_prefill_io;

/* Workspace for hybrid_layer_decode / hybrid_layer_prefill (T = 1 for decode). */
size_t hybrid_layer_workspace(const csa_layer_desc* desc, int B, int T, int E_cap);

/* Decode step ([note] csa() / hca() in "Key design 1" / "Key design 2"):
 * append the new token to the window ring and the tail; fold the block whose
 * entry becomes visible at this position (at most one per step; the caller
 * steps every position); CSA: score the visible entries, keep the top-k and
 * attend over them + window + sink; HCA: attend over all visible entries +
 * window + sink.  n_entries is updated on the device.  With norm_rope the
 * new token's window row enters the ring prepared (normalised and rotated),
 * as does the folded entry; the ring and the cache hold prepared vectors. */
csa_status hybrid_layer_decode(const csa_layer_desc* desc, csa_layer_state* state,
                               const csa_decode_io* io, void* ws, size_t ws_bytes, void* stream);

/* Prefill chunk: compress the chunk's blocks into the cache (the first uses
 * the previous block's branch b from the tail unless pos0 == 0), answer all T
 * queries causally, then leave the window ring and the tail holding the
 * chunk's last tokens so that decode can continue at pos0 + T.  With
 * norm_rope the chunk's window rows (io->win, raw) and queries are prepared
 * in the workspace, and the ring receives prepared rows. */
csa_status hybrid_layer_prefill(const csa_layer_desc* desc, csa_layer_state* state,
                                const csa_prefill_io* io, void* ws, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): hybrid_layer_decode
 * with its workspace in a device array inside the library, one per device,
 * of hybrid_layer_noalloc_scratch_bytes() bytes (32 MiB: enough for a
 * Pro-shaped CSA layer of 4 sequences x 262,144 entries with k = 1024, or a
 * Flash-shaped HCA layer of 8 x 8,192 entries).  The caller still passes the
 * state, inputs and outputs.  Same arguments, results and errors as
 * hybrid_layer_decode, plus CSA_ERR_WORKSPACE when the call needs more than
 * the array holds.  It allocates and frees nothing.  Calls on one device share
 * its array and must not overlap (calls on different streams of one device, or
 * from several threads at once, race); the array keeps the last call's
 * contents and is cleared by the library (on the call's stream) whenever the
 * configuration (descriptor, B, E_cap) differs from the previous call's. */
size_t hybrid_layer_noalloc_scratch_bytes(void);
csa_status hybrid_layer_decode_noalloc(const csa_layer_desc* desc, csa_layer_state* state,
                                       const csa_decode_io* io, void* stream);

/* ------------------------------------------------------------------------
 * Kernel timing (diagnostics, not part of the method).  While enabled, every
 * kernel the library launches is bracketed by two hipEvents recorded on its
 * stream.  csa_profile_collect waits for the recorded events, fills up to
 * max_entries per-kernel totals (launch count, summed GPU milliseconds) since
 * the previous collect, clears them, and returns the number of kernels seen.
 * ------------------------------------------------------------------------ */
typedef struct {
  char name[48];
  int64_t launches;
  double total_ms;
} csa_kernel_time;

csa_status csa_profile_enable(int on);
int csa_profile_collect(csa_kernel_time* out, int max_entries);

/* Test hook (diagnostics, not part of the method).  In a decode-shaped
 * csa_index_topk / hybrid_layer_decode call, the scoring workgroups of a row
 * wait (polling device memory) for the row's threshold bin, which the last of
 * them publishes; a workgroup that does not see it within `polls` polls gives
 * up, and the row's selection is then rebuilt from its scores by the resolve
 * kernel (same result, slower).  Sets that budget for later calls (rounded
 * down to a multiple of 4; a negative value restores the default of 40000,
 * a few ms) and returns the previous one.  0 makes every waiting workgroup
 * give up at once, so tests can check the fallback against the oracle.
 * Process-wide; not synchronised with calls in flight on other threads. */
int csa_test_set_fused_wait_polls(int polls);

/* Test hook (diagnostics, not part of the method).  Whether a decode step
 * may fold its pending block inside the scoring kernel (CSA) or the dense
 * attention (HCA) rather than in the separate fold kernel (1, the default)
 * or never (0).  The two paths add the new entry's terms in different
 * orders, so they agree within float32 rounding, not bit for bit; a test
 * that compares the two paths' results bit for bit turns fusion off.
 * Returns the previous setting.
 * Process-wide; not synchronised with calls in flight on other threads. */
int csa_test_set_fold_fusion(int on);

#ifdef __cplusplus
}
#endif
#endif /* CSA_H */
