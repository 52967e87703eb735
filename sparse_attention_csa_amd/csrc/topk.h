// Top-k scratch layout and launchers shared by the scoring and selection kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"
#include "kernels.h"

namespace csa {

constexpr int kTopkBins = 2048;      // histogram of the top 11 key bits
constexpr int kTopkShift = 21;       // key >> 21 = bin
constexpr int kTopkCandCap = 8192;   // threshold-bin candidates resolved in LDS
constexpr int kTopkMaxK = 2048;      // largest k
constexpr int kTopkCollectSlice = 4096;  // entries per collect workgroup
constexpr int kTopkFuseCap = 4096;       // scores a fused scoring workgroup keeps in LDS
constexpr int kTopkMaxWgRow = 1024;      // scoring workgroups per row (fused mode)

// per-row scratch; hist, ctr and sync are zero between calls (the resolving
// workgroups return them to zero)
struct TopkWs {
  int* hist;   // [rows][kTopkBins]
  int* ctr;    // [rows][4]: candidates, certain winners; fused mode: [2] failure flag, [3] threshold bin
  uint2* cand; // [rows][kTopkCandCap] (key, id) of threshold-bin entries (split mode)
  int* sure;   // [rows][kTopkMaxK] ids above the threshold bin (split mode)
  // fused mode (split mode, scores kept by the scoring workgroups)
  unsigned* sync;  // [rows] arrivals of the scoring workgroups (rows <= 64)
  int4* wg_info;   // [rows][kTopkMaxWgRow] per scoring workgroup: certain, candidates, first entry
  int* lsure;      // [rows][list_len] certain winners, workgroup j's at j * list_stride
  uint2* lcand;    // [rows][list_len] candidates (key, id), likewise
  int list_len;    // per row (topk_list_len)
  int list_stride; // set by the scoring launch: the largest per-workgroup entry count
};

// per-row length of the fused lists: room for every workgroup's region of
// list_stride entries, whatever the scan plan
CSA_HOST_DEV inline int topk_list_len(int E_cap) { return E_cap + 64 * kTopkMaxWgRow + kTopkFuseCap; }

// ---- device helpers shared by the scoring and selection kernels

CSA_DEV int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int x = __shfl_up(v, o, 64);
    if (lane >= o) v += x;
  }
  return v;
}

// exclusive prefix of v over the NT threads in thread order; *total = sum.
// s_w: NT/64 ints of scratch.  Contains two barriers.
template <int NT>
CSA_DEV int block_excl_scan(int v, int* s_w, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int inc = wave_incl_scan(v);
  if (lane == 63) s_w[wave] = inc;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int c = s_w[w];
    if (w < wave) off += c;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return off + inc - v;
}

// b1 (bin of the k-th largest key) and the count above it, from each
// thread's kTopkBins / NT bin counts c[i] = count of bin
// kTopkBins - 1 - (PER tid + i) (bins in descending order over the threads);
// every thread gets both.  s_w: NT/64 ints, s_out: 2 ints.
template <int NT>
CSA_DEV void find_bin_counts(const int* c, int k, int* s_w, int* s_out, int* b1, int* above) {
  const int tid = threadIdx.x;
  constexpr int PER = kTopkBins / NT;
  int tot = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) tot += c[i];
  int all;
  const int before = block_excl_scan<NT>(tot, s_w, &all);
  if (before < k && before + tot >= k) {
    int acc = before;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (acc + c[i] >= k) {
        s_out[0] = kTopkBins - 1 - (PER * tid + i);
        s_out[1] = acc;
        break;
      }
      acc += c[i];
    }
  }
  __syncthreads();
  *b1 = s_out[0];
  *above = s_out[1];
  __syncthreads();
}

// the same from a kTopkBins histogram (global or LDS)
template <int NT>
CSA_DEV void find_bin(const int* hist, int k, int* s_w, int* s_out, int* b1, int* above) {
  constexpr int PER = kTopkBins / NT;
  int c[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) c[i] = hist[kTopkBins - 1 - (PER * threadIdx.x + i)];
  find_bin_counts<NT>(c, k, s_w, s_out, b1, above);
}

// Polls a fused scoring workgroup makes for its row's published threshold
// bin before it gives up and leaves the row to the resolve's fallback (a few
// ms at the default).  Settable from the host for tests of that fallback.
int fused_wait_polls();
int set_fused_wait_polls(int polls);

size_t topk_ws_bytes(int rows, int E_cap, bool split);
TopkWs topk_ws_carve(void* base, int rows, int E_cap, bool split);
hipError_t launch_topk_collect(const IndexArgs& a, const TopkWs& ws, int slices, int slice_len,
                               hipStream_t s);
// fused mode: the scoring kernel classified the scores; one workgroup per row
// merges the per-workgroup lists (n_wg scoring workgroups per row)
hipError_t launch_topk_fused_resolve(const IndexArgs& a, const TopkWs& ws, int n_wg, hipStream_t s);
hipError_t launch_topk_rows(const IndexArgs& a, const TopkWs& ws, hipStream_t s);

// MFMA scorer (indexer_mfma.hip); with use_hist it also fills ws.hist.  With
// allow_fuse (split mode) it may also classify the scores against the
// threshold bin (per-row publication); *n_wg_fused is then the number of
// scoring workgroups per row, else 0.  With fold (only when
// index_fold_fusable) it also performs the decode step's fold.
bool index_mfma_supported(const IndexArgs& a);
// paged keys (a.pg.table): whether the scan's paged form takes them
bool index_mfma_pages_fit(const IndexArgs& a);
hipError_t launch_index_score_mfma(const IndexArgs& a, TopkWs& ws, int use_hist, int allow_fuse,
                                   int* n_wg_fused, const FoldArgs* fold, hipStream_t s);
// whether the decode step's fold can run inside the scoring kernel (fold
// workgroups); split: split-mode selection (few rows)
bool index_fold_fusable(const IndexArgs& a, const FoldArgs& f, bool split);

}  // namespace csa
