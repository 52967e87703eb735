// Top-k scratch layout and launchers shared by the scoring and selection kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace csa {

constexpr int kTopkBins = 2048;      // histogram of the top 11 key bits
constexpr int kTopkShift = 21;       // key >> 21 = bin
constexpr int kTopkCandCap = 8192;   // threshold-bin candidates resolved in LDS

// per-row scratch, zero between calls (the finishing workgroup re-zeroes it)
struct TopkWs {
  int* hist;          // [rows][kTopkBins]
  int* ctr;           // [rows][4]: candidates, finished workgroups
  uint32_t* bitmap;   // [rows][bitmap_words]: selected entries
  uint32_t* summary;  // [rows][summary_words]: nonzero bitmap words
  uint2* cand;        // [rows][kTopkCandCap] (key, id), split mode
  int bitmap_words, summary_words;
};

__device__ void topk_resolve_from_row(const float* sc, int nv, int b1, int want, uint32_t* bitmap,
                                      uint32_t* summary, int* s_scan, int* s_hist, int* s_misc);

size_t topk_ws_bytes(int rows, int E_cap, bool with_cand);
// LDS of the split-mode resolve kernel; it must fit one workgroup (160 KB)
size_t topk_split_lds_bytes(int E_cap);
constexpr int kTopkCollectSlice = 4096;  // entries per collect workgroup
TopkWs topk_ws_carve(void* base, int rows, int E_cap, bool with_cand);
hipError_t launch_topk_collect(const IndexArgs& a, const TopkWs& ws, int slices, int slice_len,
                               hipStream_t s);
hipError_t launch_topk_rows(const IndexArgs& a, const TopkWs& ws, hipStream_t s);

// MFMA scorer (indexer_mfma.hip); with use_hist it also fills ws.hist
bool index_mfma_supported(const IndexArgs& a);
hipError_t launch_index_score_mfma(const IndexArgs& a, const TopkWs& ws, int use_hist, hipStream_t s);

}  // namespace csa
