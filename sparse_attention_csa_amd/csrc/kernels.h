// Internal launch interface between the C-ABI host layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "csa.h"

namespace csa {

// sets the thread-local message csa_last_error() returns (api.cpp)
int set_error(int status, const char* fmt, ...);
// argument checks of a decode step, all but the workspace (api.cpp)
csa_status decode_check(const csa_layer_desc* d, const csa_layer_state* s, const csa_decode_io* io);

// kernel timing hook (profile.cpp): records events around a launch when enabled
class ProfScope {
 public:
  ProfScope(const char* name, hipStream_t s);
  ~ProfScope();

 private:
  const char* name_;
  hipStream_t s_;
  void* a_;
};

#define CSA_LAUNCH(name, kern, grid, block, shm, stream, ...)           \
  do {                                                                  \
    ::csa::ProfScope csa_prof_scope_(name, stream);                     \
    hipLaunchKernelGGL(kern, grid, block, shm, stream, __VA_ARGS__);    \
  } while (0)

// storage formats (the csa_dtype codes); MXFP4 vectors are packed E2M1
// pairs with one E8M0 scale byte per 32 values
enum Dt { F32 = 0, BF16 = 1, E4M3 = 2, MXFP4 = 3, FP8BF16 = 4 };
// the 576-byte main entry: 448 e4m3 codes (one float32 scale per entry),
// then 64 bf16
constexpr int kF8Dims = 448, kF8RowB = 576;

// Host-side values that depend on the device (occupancy, LDS attributes set
// on a kernel) are cached per device id, below this bound.
constexpr int kMaxDevices = 64;
// the current device id, or -1 if it cannot be determined (out of range
// too): callers then compute the value without caching it
inline int current_device() {
  int d = 0;
  if (hipGetDevice(&d) != hipSuccess || d < 0 || d >= kMaxDevices) return -1;
  return d;
}

// RMSNorm and partial RoPE of produced KV vectors and queries (norm_rope):
// v * g / sqrt(mean(v^2) + eps), then pairs (2i, 2i+1) of the last
// rope_dims coordinates rotated by pos * inv_freq[i]
struct NormRope {
  int on;
  int rope_dims;
  float eps;
  const float* g_q;         // [c] query heads
  const float* g_kv;        // [c] KV head
  const double* inv_freq;   // [rope_dims / 2]
};

// Paged compressed caches ([book] ch. 13 "Aligning original-token blocks"):
// with a block table, entry e of sequence b lives in row
// table[b][e >> shift] * 2^shift + (e & (2^shift - 1)) of a pool of pages
// shared by all sequences (the main cache, the indexer keys and their
// scales, the entry scales: one row each per entry); without one, in row
// b * E_cap + e.
struct PageMap {
  const int32_t* table;  // [B][E_cap >> shift] page ids, or null
  int shift;             // log2 of the entries per page
};
__host__ __device__ inline size_t page_row(const PageMap& p, int b, int64_t e, int E_cap) {
  if (!p.table) return (size_t)b * E_cap + (size_t)e;
  const int32_t pg = p.table[(size_t)b * (size_t)(E_cap >> p.shift) + (size_t)(e >> p.shift)];
  return ((size_t)(uint32_t)pg << p.shift) + (size_t)(e & ((1 << p.shift) - 1));
}

// ------------------------------------------------------------ compressor
struct CompressArgs {
  int dtype;  // input dtype (F32 / BF16)
  const void *ca, *za, *cb, *zb, *prev_cb, *prev_zb;
  int logit_width;
  const float *score_w, *bias_a, *bias_b;
  int B, T, c, m;
  void* out;
  int out_dtype;
  void* out_scale;  // E4M3: float [B][E_cap]; MXFP4: uint8 [B][E_cap][c/32]
  int E_cap;
  int64_t first;
  size_t seq_stride;       // elements between sequences of ca/za/cb/zb (0: T*c or T*lw)
  size_t prev_seq_stride;  // elements between sequences of prev_cb/prev_zb (0: m*c or m*lw)
  NormRope nr;             // on: entry first + i is prepared at position m * (first + i)
  PageMap pg;              // rows of out / out_scale
  // variable-length chunks (seq_pos0 non-null; first and prev_* unused):
  // sequence b's chunk holds positions seq_pos0[b] .. + seq_len[b] - 1 in
  // rows 0 ..; its entries floor(seq_pos0[b] / m) + blockIdx.x below
  // floor((seq_pos0[b] + seq_len[b]) / m) (and E_cap) are produced, a source
  // token p before the chunk read from slot p % R of its stream in tail
  const int64_t* seq_pos0;
  const int32_t* seq_len;
  const void* tail;  // [B][ns][R][c]: ns = 4 (ca, za, cb, zb) with overlap, else 2
  int R;
};
hipError_t launch_compress(const CompressArgs& a, hipStream_t s);

// decode-step fold of the pending block + append of the new token
struct FoldArgs {
  int dtype;      // kv dtype (F32 / BF16) of streams, tails, caches
  int idx_dtype;  // indexer-cache dtype (F32 / BF16 / E4M3 / MXFP4) or -1 (no indexer)
  int B, c, d_I, m, R, n_win, vis, overlap;
  const int64_t* pos;
  int32_t* n_entries;
  int32_t* counters;        // [B] workspace, zero between calls
  float* fold_buf;          // [B][c] workspace: a whole entry's folded values (norm_rope / FP8BF16)
  const void* streams;      // [B][S][c]
  const void* idx_streams;  // [B][4][d_I]
  const void* x_new;        // [B][c]
  void* tail;               // [B][S][R][c]
  void* idx_tail;           // [B][4][R][d_I]
  void* win_ring;           // [B][n_win][c]
  void* kv_cache;           // [B][E_cap][c]
  void* idx_cache;          // [B][E_cap][d_I] (MXFP4: [B][E_cap][d_I/2] bytes)
  void* idx_scale;          // E4M3: float [B][E_cap]; MXFP4: uint8 [B][E_cap][d_I/32]
  int E_cap;
  const float *bias_a, *bias_b, *ibias_a, *ibias_b;
  // norm_rope: the folded entry and the new window row are prepared, and
  // the step's queries q [B][H][c] are prepared into q_prep
  NormRope nr;
  int H;
  const void* q;
  void* q_prep;
  // main entries stored as FP8BF16 (576 bytes + a float32 scale in kv_scale)
  int kv_fmt;
  float* kv_scale;
  PageMap pg;  // rows of kv_cache, kv_scale, idx_cache, idx_scale
};
hipError_t launch_fold_append(const FoldArgs& a, hipStream_t s);

// norm_rope prefill: queries [B][T][H][c] at positions pos0 + t and window
// rows [B][n_win-1+T][c] at pos0 - (n_win-1) + j, prepared into q_prep and
// win_prep (same layouts)
struct PrepArgs {
  int dtype, B, T, H, c, n_win;
  int64_t pos0;
  const int64_t* seq_pos0;  // [B] or null: per-sequence chunk starts (replace pos0)
  NormRope nr;
  const void* q;
  const void* win;
  void* q_prep;
  void* win_prep;
};
hipError_t launch_prep_rows(const PrepArgs& a, hipStream_t s);

// prefill epilogue: copy the chunk's last tokens into the window ring / tail
struct PrefillStateArgs {
  int dtype, B, T, c, d_I, R, n_win, S;
  int64_t pos0;
  const void* win;          // [B][n_win-1+T][c]
  const void* streams;      // [B][S][T][c]
  const void* idx_streams;  // [B][4][T][d_I] or null
  void* win_ring;
  void* tail;
  void* idx_tail;
  int32_t* n_entries;
  int new_entries;
  // variable-length chunks (replace pos0 and T per sequence; new_entries 0:
  // the counts were set by launch_varlen_setup)
  const int64_t* seq_pos0;
  const int32_t* seq_len;
};
hipError_t launch_prefill_state(const PrefillStateArgs& a, hipStream_t s);

// variable-length prefill: each query row's position (row tq of sequence b
// at seq_pos0[b] + tq, padding rows at the sequence's last position) into
// q_pos [B][T], the window input's first position into win_pos0 [B], and the
// entry counts after the chunk, floor((seq_pos0[b] + seq_len[b]) / m) (at
// most E_cap), into n_entries
struct VarlenArgs {
  int B, T, m, n_win, E_cap;
  const int64_t* seq_pos0;
  const int32_t* seq_len;
  int64_t* q_pos;
  int64_t* win_pos0;
  int32_t* n_entries;
};
hipError_t launch_varlen_setup(const VarlenArgs& a, hipStream_t s);

// ------------------------------------------------------------ indexer + top-k
struct IndexArgs {
  int idx_dtype;
  const void* q;        // [B][Tq][H_I][d_I] (MXFP4: d_I/2 bytes per vector)
  const void* q_scale;  // E4M3: float [B][Tq][H_I]; MXFP4: uint8 [B][Tq][H_I][d_I/32]
  const float* w;       // [B][Tq][H_I]
  const void* keys;     // [B][E_cap][d_I]
  const void* k_scale;  // E4M3: float [B][E_cap]; MXFP4: uint8 [B][E_cap][d_I/32]
  int score_bf16;       // 1: scores are rounded to bfloat16 (nearest-even) before the selection
  const int64_t* q_pos; // [B][Tq], or null: query tq is at q_pos0 + tq
  int64_t q_pos0;
  const int32_t* n_entries;
  int n_add;            // entries appended earlier in the same step
  int B, Tq, H_I, d_I, E_cap, m, k, vis;
  float* scores;        // [B][Tq][E_cap]
  int32_t* topk_idx;    // [B][Tq][k]
  int32_t* topk_cnt;    // [B][Tq]
  void* ws;             // topk scratch
  PageMap pg;           // rows of keys / k_scale
};
size_t index_topk_ws_bytes(int B, int Tq, int E_cap, int k);
// fold: the decode step's fold to run inside the scoring kernel, or null
// (then the caller has already run it); see index_topk_fuses_fold
hipError_t launch_index_topk(const IndexArgs& a, hipStream_t s, const FoldArgs* fold = nullptr);
bool index_topk_fuses_fold(const IndexArgs& a, const FoldArgs& f);

// ------------------------------------------------------------ attention
struct AttendArgs {
  int dtype;
  const void* q;        // [B][Tq][H][c]
  const void* kv;       // [B][E_cap][c]
  int E_cap;
  // sparse (CSA) rows
  const int32_t* topk_idx;
  const int32_t* topk_cnt;
  int k;
  // dense (HCA) rows
  const int32_t* n_entries;
  int n_add;
  int m, vis;
  int dense;
  // window
  const void* win;
  int W_cap;
  const int64_t* win_pos0;  // [B] or null (= 0)
  int64_t win_pos0_const;   // used when win_pos0 is null
  int n_win;
  const float* sink;
  const int64_t* q_pos;  // [B][Tq], or null: query tq is at q_pos0 + tq
  int64_t q_pos0;
  float scale;
  int B, Tq, H, c;
  void* out;
  float* lse;
  void* ws;
  size_t ws_bytes;
  // > 0: every query's rows are cut into splits of this many rows (a multiple
  // of 16) whatever the batch, so a query's result does not depend on the
  // batch it is in; 0: the split size is chosen for the batch
  int split_rows;
  // dense decode with the step's fold inside (see attend_fuses_fold): each
  // split folds fold_cs coordinates of the new entry and writes its share of
  // q . entry and q . token to its slot of fold_s; the merge sums the slots
  // in slice order and adds the new entry and the query's own token as two
  // more rows
  int fold_mode;
  int fold_cs;
  FoldArgs fold;
  float* fold_s;       // [B][H][64 slices][2]: shares of q . new entry, q . own token
  int32_t* fold_row;   // [B]: new entry index + 1, or 0
  uint16_t* fold_new;  // [B][c]: the new entry (bf16), read by the merge
  int fold_nsplit;     // set by the launch: splits that fold (fewer rows each) ...
  int fold_rows;       // ... and their row count
  // norm_rope: the output's last rope_dims coordinates are rotated back by
  // the query position (pairs (2i, 2i+1), angle -t * derot_freq[i]); null: off
  const double* derot_freq;
  int rope_dims;
  // compressed rows stored as FP8BF16 (576 bytes, scale in kv_scale); the
  // window rows and q stay in dtype
  int kv_fmt;
  const float* kv_scale;
  PageMap pg;  // rows of kv / kv_scale
};
// split_rows > 0: rows per split fixed (batch-invariant launch plan), else
// chosen for the batch
size_t attend_ws_bytes(int B, int Tq, int H, int c, int rows_max, int split_rows = 0);
// the largest number of row splits a query's rows may be cut into
constexpr int kMaxRowSplits = 64;
// whether hca decode can fold inside the attention; sets a.fold_mode / fold_cs
bool attend_fuses_fold(AttendArgs& a, const FoldArgs& f);
hipError_t launch_attend(const AttendArgs& a, hipStream_t s);

}  // namespace csa
