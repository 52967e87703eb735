// Lightning indexer (row a2) and top-k selection (row a3).
//
// Score: I[t, s] = sum_h w[t, h] * ReLU(q[t, h] . K[s]) over visible entries
// ("2026 DeepSeek-V4" note, "Key design 1" indexer equation; "DeepSeek-V4"
// book ch. 6 "The index score").  For e4m3 the per-vector scales are positive,
// so ReLU(sq*sk*x) = sq*sk*ReLU(x): the query scale folds into w and the key
// scale multiplies the head sum once.
//
// Top-k: C_t = TopK_k(I[t, :]) (same equation; book ch. 6 "Top-k is a budget
// over compressed entries"), ties to the lower entry id, ids ascending.  The
// k-th largest score is found exactly by a radix select on order-preserving
// 32-bit keys (8 bits per pass over the row, LDS histograms), then one
// in-order pass emits every id above the threshold plus the lowest-id ties.

#include "common.h"
#include "kernels.h"
#include "topk.h"

namespace csa {

constexpr int kHMax = 64;  // indexer heads supported

template <typename T>
CSA_DEV float ld_key(const T* p, size_t i) {
  return ld(p, i);
}
CSA_DEV float ld_key(const uint8_t* p, size_t i) { return e4m3_to_f32(p[i]); }

CSA_DEV int64_t n_visible(const IndexArgs& a, int b, int64_t t) {
  const int64_t lim = vis_limit(t, a.m, a.vis);
  const int64_t have = (int64_t)a.n_entries[b] + a.n_add;
  int64_t n = lim < have ? lim : have;
  if (n > a.E_cap) n = a.E_cap;
  return n < 0 ? 0 : n;
}

// --------------------------------------------------------------------------
// scoring: grid (ceil(E_cap/256), B*Tq), one entry per thread (VALU form)
// --------------------------------------------------------------------------
template <typename TK>
__global__ __launch_bounds__(256) void index_score_kernel(IndexArgs a) {
  const int row = blockIdx.y, b = row / a.Tq, tq = row % a.Tq;
  const int tid = threadIdx.x;
  const int H = a.H_I, D = a.d_I;
  const int64_t t = a.q_pos ? a.q_pos[(size_t)b * a.Tq + tq] : a.q_pos0 + tq;
  const int64_t nv = n_visible(a, b, t);
  const int64_t s0 = (int64_t)blockIdx.x * 256;
  if (s0 >= nv) return;

  __shared__ float q_s[kHMax * 128];
  __shared__ float w_s[kHMax];
  const TK* q = reinterpret_cast<const TK*>(a.q) + (size_t)row * H * D;
  for (int i = tid; i < H * D; i += 256) q_s[i] = ld_key(q, i);
  if (tid < H) {
    float w = a.w[(size_t)row * H + tid];
    if (a.q_scale) w *= a.q_scale[(size_t)row * H + tid];
    w_s[tid] = w;
  }
  __syncthreads();

  const int64_t s = s0 + tid;
  if (s >= nv) return;
  const TK* key = reinterpret_cast<const TK*>(a.keys) + ((size_t)b * a.E_cap + s) * D;
  float acc[kHMax];
#pragma unroll
  for (int h = 0; h < kHMax; ++h) acc[h] = 0.f;
  for (int d0 = 0; d0 < D; d0 += 8) {
    float kv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) kv[j] = ld_key(key, d0 + j);
#pragma unroll
    for (int h = 0; h < kHMax; ++h) {
      if (h < H) {
        float x = acc[h];
#pragma unroll
        for (int j = 0; j < 8; ++j) x += q_s[h * D + d0 + j] * kv[j];
        acc[h] = x;
      }
    }
  }
  float score = 0.f;
#pragma unroll
  for (int h = 0; h < kHMax; ++h)
    if (h < H) score += w_s[h] * fmaxf(acc[h], 0.f);
  if (a.k_scale) score *= a.k_scale[(size_t)b * a.E_cap + s];
  a.scores[(size_t)row * a.E_cap + s] = score;
}

// --------------------------------------------------------------------------
// scoring + selection
// --------------------------------------------------------------------------
namespace {
constexpr int kSplitRows = 64;  // at most this many rows: split-mode selection
}

size_t index_topk_ws_bytes(int B, int Tq, int E_cap, int k) {
  (void)k;
  const int rows = B * Tq;
  const size_t sc = ((size_t)rows * E_cap * sizeof(float) + 255) / 256 * 256;
  return sc + topk_ws_bytes(rows, E_cap, rows <= kSplitRows);
}

bool index_topk_fuses_fold(const IndexArgs& a, const FoldArgs& f) {
  return index_fold_fusable(a, f, a.B * a.Tq <= kSplitRows);
}

hipError_t launch_index_topk(const IndexArgs& a0, hipStream_t s, const FoldArgs* fold) {
  IndexArgs a = a0;
  const int rows = a.B * a.Tq;
  char* ws = reinterpret_cast<char*>(a.ws);
  const size_t sc_bytes = ((size_t)rows * a.E_cap * sizeof(float) + 255) / 256 * 256;
  if (!a.scores) a.scores = reinterpret_cast<float*>(ws);
  const bool split = rows <= kSplitRows;
  TopkWs tw = topk_ws_carve(ws + sc_bytes, rows, a.E_cap, split);
  const bool mfma = index_mfma_supported(a) && split;
  hipError_t e;
  int n_wg_fused = 0;
  if (mfma) {
    e = launch_index_score_mfma(a, tw, 1, 1, &n_wg_fused, fold, s);
  } else {
    dim3 g1((a.E_cap + 255) / 256, rows), blk(256);
    if (a.idx_dtype == F32)
      CSA_LAUNCH("index_score", index_score_kernel<float>, g1, blk, 0, s, a);
    else if (a.idx_dtype == BF16)
      CSA_LAUNCH("index_score", index_score_kernel<bf16>, g1, blk, 0, s, a);
    else
      CSA_LAUNCH("index_score", index_score_kernel<uint8_t>, g1, blk, 0, s, a);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  if (mfma) {
    if (n_wg_fused > 0) return launch_topk_fused_resolve(a, tw, n_wg_fused, s);
    const int slice_len = kTopkCollectSlice;
    const int slices = (a.E_cap + slice_len - 1) / slice_len;
    return launch_topk_collect(a, tw, slices, slice_len, s);
  }
  return launch_topk_rows(a, tw, s);
}

}  // namespace csa
