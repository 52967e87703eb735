// Top-k scratch layout and launchers shared by the scoring and selection kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace csa {

constexpr int kTopkBins = 2048;      // histogram of the top 11 key bits
constexpr int kTopkShift = 21;       // key >> 21 = bin
constexpr int kTopkCandCap = 8192;   // threshold-bin candidates resolved in LDS
constexpr int kTopkMaxK = 2048;      // largest k
constexpr int kTopkCollectSlice = 4096;  // entries per collect workgroup

// per-row scratch; hist and ctr are zero between calls (the resolving
// workgroup returns them to zero)
struct TopkWs {
  int* hist;   // [rows][kTopkBins]
  int* ctr;    // [rows][4]: candidates, certain winners
  uint2* cand; // [rows][kTopkCandCap] (key, id) of threshold-bin entries (split mode)
  int* sure;   // [rows][kTopkMaxK] ids above the threshold bin (split mode)
};

size_t topk_ws_bytes(int rows, int E_cap, bool split);
TopkWs topk_ws_carve(void* base, int rows, int E_cap, bool split);
hipError_t launch_topk_collect(const IndexArgs& a, const TopkWs& ws, int slices, int slice_len,
                               hipStream_t s);
hipError_t launch_topk_rows(const IndexArgs& a, const TopkWs& ws, hipStream_t s);

// MFMA scorer (indexer_mfma.hip); with use_hist it also fills ws.hist
bool index_mfma_supported(const IndexArgs& a);
hipError_t launch_index_score_mfma(const IndexArgs& a, const TopkWs& ws, int use_hist, hipStream_t s);

}  // namespace csa
