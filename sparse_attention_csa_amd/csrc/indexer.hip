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
#include "mfma_tile.h"
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
// scoring of many queries of one sequence (prefill) on MFMA, bf16, 64 heads
// of dim 128: a workgroup scores four consecutive queries (one per
// wavefront) against a chunk of kPfChunk entries.  The chunk streams through
// LDS in 64-entry key tiles (16 KB, double-buffered, the next tile's loads in
// flight while one is scored) shared by the four queries, so a key crosses
// HBM / L2 once per four queries.  Per wavefront and 16-entry block:
//   D[16 heads x 16 entries] = Q[16 heads x 128] . K^T[128 x 16 entries]
// (v_mfma_f32_16x16x32_bf16, four head tiles, Q in registers); lane (head
// row group g, entry i) holds heads 4g .. 4g+3 of entry i, so ReLU and the
// head weights are in-lane and the head sum takes two lane exchanges.
// --------------------------------------------------------------------------
namespace {
constexpr int kPfTile = 64;     // entries per LDS key tile
constexpr int kPfChunk = 1024;  // entries per workgroup
constexpr int kPfD = 128, kPfH = 64;
}  // namespace

bool index_prefill_mfma_supported(const IndexArgs& a) {
  return a.idx_dtype == BF16 && a.H_I == kPfH && a.d_I == kPfD && a.Tq % 4 == 0;
}

__global__ __launch_bounds__(256) void index_score_prefill_kernel(IndexArgs a) {
  using namespace tile;
  // key tile: row = entry (256 B), its 16-byte chunk c stored at c ^ (row % 16)
  __shared__ __attribute__((aligned(16))) uint4 s_k[2][kPfTile * 16];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, li = l & 15, lg = l >> 4;
  const int row0 = blockIdx.y * 4, row = row0 + w;  // the four rows share their sequence (Tq % 4 == 0)
  const int b = row0 / a.Tq;
  // visible entries of each of the four queries (every thread computes all
  // four: the chunk is needed up to the largest)
  int64_t nv_q = 0, nv_max = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int tq = (row0 + j) % a.Tq;
    const int64_t t = a.q_pos ? a.q_pos[(size_t)b * a.Tq + tq] : a.q_pos0 + tq;
    const int64_t nv = n_visible(a, b, t);
    if (j == w) nv_q = nv;
    nv_max = nv > nv_max ? nv : nv_max;
  }
  const int64_t e0 = (int64_t)blockIdx.x * kPfChunk;
  if (e0 >= nv_max) return;
  const int64_t e1 = e0 + kPfChunk < nv_max ? e0 + kPfChunk : nv_max;
  const int ntiles = (int)((e1 - e0 + kPfTile - 1) / kPfTile);
  const uint16_t* keys = reinterpret_cast<const uint16_t*>(a.keys) + (size_t)b * a.E_cap * kPfD;

  // A operands: Q rows = heads 16 ht + li, d = 32 ks + 8 lg .. +7
  bf16x8_t qa[4][4];
  float wr[4][4];  // weights of heads 16 ht + 4 lg + i
  {
    const uint16_t* q = reinterpret_cast<const uint16_t*>(a.q) + (size_t)row * kPfH * kPfD;
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        qa[ht][ks] = *reinterpret_cast<const bf16x8_t*>(q + (size_t)(16 * ht + li) * kPfD + 32 * ks + 8 * lg);
      const float4 wv = *reinterpret_cast<const float4*>(a.w + (size_t)row * kPfH + 16 * ht + 4 * lg);
      wr[ht][0] = wv.x; wr[ht][1] = wv.y; wr[ht][2] = wv.z; wr[ht][3] = wv.w;
    }
  }
  // thread's share of a tile: chunks tid + 256 u (entry c / 16, chunk c % 16);
  // entries past the last visible one re-read it
  struct Share {
    uint4 v0, v1, v2, v3;
  };
  auto chunk_ptr = [&](int j, int u) -> const uint4* {
    const int c = tid + 256 * u;
    int64_t e = e0 + (int64_t)j * kPfTile + (c >> 4);
    if (e > e1 - 1) e = e1 - 1;
    return reinterpret_cast<const uint4*>(keys + (size_t)e * kPfD + 8 * (c & 15));
  };
  auto load_tile = [&](int j) -> Share {
    return Share{*chunk_ptr(j, 0), *chunk_ptr(j, 1), *chunk_ptr(j, 2), *chunk_ptr(j, 3)};
  };
  auto slot = [&](int buf, int u) -> uint4* {
    const int c = tid + 256 * u, kk = c >> 4;
    return &s_k[buf][kk * 16 + ((c & 15) ^ (kk & 15))];
  };
  auto store_tile = [&](int buf, const Share& r) {
    *slot(buf, 0) = r.v0;
    *slot(buf, 1) = r.v1;
    *slot(buf, 2) = r.v2;
    *slot(buf, 3) = r.v3;
  };
  float* out = a.scores + (size_t)row * a.E_cap;
  store_tile(0, load_tile(0));
  __syncthreads();
  for (int j = 0; j < ntiles; ++j) {
    Share next{};
    if (j + 1 < ntiles) next = load_tile(j + 1);  // in flight while tile j is scored
    const uint4* T = s_k[j & 1];
    const int64_t te = e0 + (int64_t)j * kPfTile;
#pragma unroll
    for (int kb = 0; kb < kPfTile / 16; ++kb) {
      f32x4_t c[4];
#pragma unroll
      for (int ht = 0; ht < 4; ++ht) c[ht] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        // B operand: entry 16 kb + li, d = 32 ks + 8 lg .. +7 (chunk 4 ks + lg)
        const bf16x8_t kf = __builtin_bit_cast(bf16x8_t, T[(16 * kb + li) * 16 + ((4 * ks + lg) ^ li)]);
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) c[ht] = mfma32(qa[ht][ks], kf, c[ht]);
      }
      float part = 0.f;
#pragma unroll
      for (int ht = 0; ht < 4; ++ht)
#pragma unroll
        for (int i = 0; i < 4; ++i) part += wr[ht][i] * fmaxf(c[ht][i], 0.f);
      part += __shfl_xor(part, 16, 64);
      part += __shfl_xor(part, 32, 64);
      const int64_t e = te + 16 * kb + li;
      if (lg == 0 && e < nv_q && e < e1) out[e] = part;
    }
    if (j + 1 < ntiles) store_tile((j + 1) & 1, next);
    __syncthreads();
  }
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
  } else if (index_prefill_mfma_supported(a)) {
    dim3 g1((a.E_cap + kPfChunk - 1) / kPfChunk, rows / 4), blk(256);
    CSA_LAUNCH("index_score", index_score_prefill_kernel, g1, blk, 0, s, a);
    e = hipGetLastError();
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
