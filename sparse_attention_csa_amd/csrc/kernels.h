// Internal launch interface between the C-ABI host layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csa {

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

enum Dt { F32 = 0, BF16 = 1, E4M3 = 2 };

// ------------------------------------------------------------ compressor
struct CompressArgs {
  int dtype;  // input dtype (F32 / BF16)
  const void *ca, *za, *cb, *zb, *prev_cb, *prev_zb;
  int logit_width;
  const float *score_w, *bias_a, *bias_b;
  int B, T, c, m;
  void* out;
  int out_dtype;
  float* out_scale;
  int E_cap;
  int64_t first;
  size_t seq_stride;       // elements between sequences of ca/za/cb/zb (0: T*c or T*lw)
  size_t prev_seq_stride;  // elements between sequences of prev_cb/prev_zb (0: m*c or m*lw)
};
hipError_t launch_compress(const CompressArgs& a, hipStream_t s);

// decode-step fold of the pending block + append of the new token
struct FoldArgs {
  int dtype;      // kv dtype (F32 / BF16) of streams, tails, caches
  int idx_dtype;  // indexer-cache dtype (F32 / BF16 / E4M3) or -1 (no indexer)
  int B, c, d_I, m, R, n_win, vis, overlap;
  const int64_t* pos;
  int32_t* n_entries;
  int32_t* counters;        // [B] workspace, zero between calls
  const void* streams;      // [B][S][c]
  const void* idx_streams;  // [B][4][d_I]
  const void* x_new;        // [B][c]
  void* tail;               // [B][S][R][c]
  void* idx_tail;           // [B][4][R][d_I]
  void* win_ring;           // [B][n_win][c]
  void* kv_cache;           // [B][E_cap][c]
  void* idx_cache;          // [B][E_cap][d_I]
  float* idx_scale;         // [B][E_cap]
  int E_cap;
  const float *bias_a, *bias_b, *ibias_a, *ibias_b;
};
hipError_t launch_fold_append(const FoldArgs& a, hipStream_t s);

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
};
hipError_t launch_prefill_state(const PrefillStateArgs& a, hipStream_t s);

// ------------------------------------------------------------ indexer + top-k
struct IndexArgs {
  int idx_dtype;
  const void* q;        // [B][Tq][H_I][d_I]
  const float* q_scale; // [B][Tq][H_I]
  const float* w;       // [B][Tq][H_I]
  const void* keys;     // [B][E_cap][d_I]
  const float* k_scale; // [B][E_cap]
  const int64_t* q_pos; // [B][Tq], or null: query tq is at q_pos0 + tq
  int64_t q_pos0;
  const int32_t* n_entries;
  int n_add;            // entries appended earlier in the same step
  int B, Tq, H_I, d_I, E_cap, m, k, vis;
  float* scores;        // [B][Tq][E_cap]
  int32_t* topk_idx;    // [B][Tq][k]
  int32_t* topk_cnt;    // [B][Tq]
  void* ws;             // topk scratch
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
  // dense decode with the step's fold inside (see attend_fuses_fold): each
  // split folds fold_cs coordinates of the new entry and adds its share of
  // q . entry and q . token to fold_s; the merge adds the new entry and the
  // query's own token as two more rows
  int fold_mode;
  int fold_cs;
  FoldArgs fold;
  float* fold_s;       // [B][H][2]: q . new entry, q . own token; zero between calls
  int32_t* fold_row;   // [B]: new entry index + 1, or 0
  uint16_t* fold_new;  // [B][c]: the new entry (bf16), read by the merge
  int fold_nsplit;     // set by the launch: splits that fold (fewer rows each) ...
  int fold_rows;       // ... and their row count
};
size_t attend_ws_bytes(int B, int Tq, int H, int c, int rows_max);
// whether hca decode can fold inside the attention; sets a.fold_mode / fold_cs
bool attend_fuses_fold(AttendArgs& a, const FoldArgs& f);
hipError_t launch_attend(const AttendArgs& a, hipStream_t s);

}  // namespace csa
