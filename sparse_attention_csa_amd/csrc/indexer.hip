// Lightning indexer (row a2) and top-k selection (row a3).
//
// Score: I[t, s] = sum_h w[t, h] * ReLU(q[t, h] . K[s]) over visible entries
// ("2026 DeepSeek-V4" note, "Key design 1" indexer equation; "DeepSeek-V4"
// book ch. 6 "The index score").  For e4m3 the per-vector scales are positive,
// so ReLU(sq*sk*x) = sq*sk*ReLU(x): the query scale folds into w and the key
// scale multiplies the head sum once.  MXFP4 vectors (E2M1 pairs with one
// E8M0 scale per 32 values; "DeepSeek-V4" book ch. 16 "The two main FP4
// targets") are decoded element by element in the VALU form.  With
// score_bf16 the scores are rounded to bfloat16 before the selection (book
// ch. 16 "BF16 index scores"; ties, then frequent, still go to the lower id).
//
// Top-k: C_t = TopK_k(I[t, :]) (same equation; book ch. 6 "Top-k is a budget
// over compressed entries"), ties to the lower entry id, ids ascending.  The
// k-th largest score is found exactly by a radix select on order-preserving
// 32-bit keys (8 bits per pass over the row, LDS histograms), then one
// in-order pass emits every id above the threshold plus the lowest-id ties.

#include <type_traits>

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
// element i of an MXFP4 vector (packed codes p, E8M0 block scales sc)
CSA_DEV float ld_mx4(const uint8_t* p, const uint8_t* sc, int i) {
  const uint32_t byte = p[i >> 1];
  return e2m1_to_f32((i & 1) ? byte >> 4 : byte & 15u) * e8m0_to_f32(sc[i >> 5]);
}

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
  constexpr bool MX = std::is_same<TK, mx4>::value;
  const int row = blockIdx.y, b = row / a.Tq, tq = row % a.Tq;
  const int tid = threadIdx.x;
  const int H = a.H_I, D = a.d_I;
  const int64_t t = a.q_pos ? a.q_pos[(size_t)b * a.Tq + tq] : a.q_pos0 + tq;
  const int64_t nv = n_visible(a, b, t);
  const int64_t s0 = (int64_t)blockIdx.x * 256;
  if (s0 >= nv) return;

  __shared__ float q_s[kHMax * 128];
  __shared__ float w_s[kHMax];
  if constexpr (MX) {
    // the row's H vectors are contiguous: element i of the row at byte i/2,
    // its block scale at i/32 (D is a multiple of 32)
    const uint8_t* q = reinterpret_cast<const uint8_t*>(a.q) + (size_t)row * H * D / 2;
    const uint8_t* qs = reinterpret_cast<const uint8_t*>(a.q_scale) + (size_t)row * H * D / 32;
    for (int i = tid; i < H * D; i += 256) q_s[i] = ld_mx4(q, qs, i);
  } else {
    const TK* q = reinterpret_cast<const TK*>(a.q) + (size_t)row * H * D;
    for (int i = tid; i < H * D; i += 256) q_s[i] = ld_key(q, i);
  }
  if (tid < H) {
    float w = a.w[(size_t)row * H + tid];
    if (!MX && a.q_scale) w *= reinterpret_cast<const float*>(a.q_scale)[(size_t)row * H + tid];
    w_s[tid] = w;
  }
  __syncthreads();

  const int64_t s = s0 + tid;
  if (s >= nv) return;
  const size_t krow = page_row(a.pg, b, s, a.E_cap);  // the key's cache row
  float acc[kHMax];
#pragma unroll
  for (int h = 0; h < kHMax; ++h) acc[h] = 0.f;
  for (int d0 = 0; d0 < D; d0 += 8) {
    float kv[8];
    if constexpr (MX) {
      const uint8_t* key = reinterpret_cast<const uint8_t*>(a.keys) + krow * D / 2;
      const uint8_t* ks = reinterpret_cast<const uint8_t*>(a.k_scale) + krow * D / 32;
#pragma unroll
      for (int j = 0; j < 8; ++j) kv[j] = ld_mx4(key, ks, d0 + j);
    } else {
      const TK* key = reinterpret_cast<const TK*>(a.keys) + krow * D;
#pragma unroll
      for (int j = 0; j < 8; ++j) kv[j] = ld_key(key, d0 + j);
    }
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
  if (!MX && a.k_scale) score *= reinterpret_cast<const float*>(a.k_scale)[krow];
  if (a.score_bf16) score = round_bf16(score);
  a.scores[(size_t)row * a.E_cap + s] = score;
}

// --------------------------------------------------------------------------
// scoring of many queries of one sequence (prefill) on MFMA, bf16, 64 heads
// of dim 128: a workgroup scores QPW consecutive queries (one per
// wavefront) against a chunk of kPfChunk entries.  The chunk streams through
// LDS in 64-entry key tiles (16 KB, double-buffered, the next tile's loads in
// flight while one is scored) shared by the QPW queries, so a key crosses
// HBM / L2 once per QPW queries.  Per wavefront and 16-entry block:
//   D[16 heads x 16 entries] = Q[16 heads x 128] . K^T[128 x 16 entries]
// (v_mfma_f32_16x16x32_bf16, four head tiles, Q in registers); lane (head
// row group g, entry i) holds heads 4g .. 4g+3 of entry i, so ReLU and the
// head weights are in-lane and the head sum takes two lane exchanges.
// --------------------------------------------------------------------------
namespace {
constexpr int kPfTile = 64;     // entries per LDS key tile
// entries per workgroup (the queries' operands are loaded once per chunk):
// measured on the 4096-query chunk 4.91 ms with 1024, 4.78 with 2048, 4.70-4.74
// with 4096 or 8192, 4.75 with 16384; 128-entry key tiles instead of 64 took
// 11.3 ms (twice the LDS per workgroup)
constexpr int kPfChunk = 4096;
constexpr int kPfD = 128, kPfH = 64;
// queries per workgroup (Tq % kPfQpw == 0).  Measured on the 4096-query
// chunk: 8 gave the same time as 4 (the kernel is not bound by the key
// traffic), 16 spilled registers and was slower.
constexpr int kPfQpw = 4;
// MFMA shape of the scorer: 16 (16x16x32) or 32 (32x32x16).  Measured on
// the 4096-query chunk: 4.94 ms with 16, 5.23 ms with 32 (180 VGPRs: two
// wavefronts per SIMD instead of three), 5.12 ms with 32 and 8 queries.
constexpr int kPfMfma = 16;
}  // namespace

bool index_prefill_mfma_supported(const IndexArgs& a) {
  return a.idx_dtype == BF16 && a.H_I == kPfH && a.d_I == kPfD && a.Tq % kPfQpw == 0;
}

template <int QPW, int MF, int PG>
__global__ __launch_bounds__(64 * QPW) void index_score_prefill_kernel(IndexArgs a) {
  using namespace tile;
  constexpr int kT = 64 * QPW;               // threads
  constexpr int kCpt = kPfTile * 16 / kT;    // 16-byte chunks of a key tile per thread
  // key tile: row = entry (256 B), its 16-byte chunk c stored at c ^ (row % 16)
  __shared__ __attribute__((aligned(16))) uint4 s_k[2][kPfTile * 16];
  // PG: page ids of the chunk's entries (paged key cache)
  __shared__ int32_t s_pg[PG ? kPfChunk + 1 : 1];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, li = l & 15, lg = l >> 4;
  const int row0 = blockIdx.y * QPW, row = row0 + w;  // the rows share their sequence (Tq % QPW == 0)
  const int b = row0 / a.Tq;
  // visible entries of each of the four queries (every thread computes all
  // four: the chunk is needed up to the largest)
  int64_t nv_q = 0, nv_max = 0;
#pragma unroll
  for (int j = 0; j < QPW; ++j) {
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
  const uint16_t* keys = reinterpret_cast<const uint16_t*>(a.keys) + (PG ? 0 : (size_t)b * a.E_cap * kPfD);
  const int sh = a.pg.shift;
  const int p_first = (int)(e0 >> sh);
  if constexpr (PG) {
    const int np = (int)((e1 - 1) >> sh) - p_first + 1;  // <= kPfChunk + 1
    const int32_t* tb = a.pg.table + (size_t)b * (a.E_cap >> sh) + p_first;
    for (int i = tid; i < np; i += kT) s_pg[i] = tb[i];
    __syncthreads();
  }

  // A operands.  16x16x32: Q rows = heads 16 ht + li, d = 32 ks + 8 lg ..
  // +7, weights of heads 16 ht + 4 lg + i.  32x32x16: Q rows = heads
  // 32 ht + (l % 32), d = 16 ks + 8 (l / 32) .. +7, weights of heads
  // 32 ht + 8 j + 4 (l / 32) + r (the rows of the lane's accumulator).
  constexpr int kHT = MF == 32 ? 2 : 4, kKS = MF == 32 ? 8 : 4, kNW = MF == 32 ? 16 : 4;
  bf16x8_t qa[kHT][kKS];
  float wr[kHT][kNW];
  {
    const uint16_t* q = reinterpret_cast<const uint16_t*>(a.q) + (size_t)row * kPfH * kPfD;
    const float* wrow = a.w + (size_t)row * kPfH;
#pragma unroll
    for (int ht = 0; ht < kHT; ++ht) {
      if constexpr (MF == 32) {
        const int hi = l & 31, half = l >> 5;
#pragma unroll
        for (int ks = 0; ks < kKS; ++ks)
          qa[ht][ks] = *reinterpret_cast<const bf16x8_t*>(q + (size_t)(32 * ht + hi) * kPfD + 16 * ks + 8 * half);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float4 wv = *reinterpret_cast<const float4*>(wrow + 32 * ht + 8 * j + 4 * half);
          wr[ht][4 * j] = wv.x; wr[ht][4 * j + 1] = wv.y; wr[ht][4 * j + 2] = wv.z; wr[ht][4 * j + 3] = wv.w;
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < kKS; ++ks)
          qa[ht][ks] = *reinterpret_cast<const bf16x8_t*>(q + (size_t)(16 * ht + li) * kPfD + 32 * ks + 8 * lg);
        const float4 wv = *reinterpret_cast<const float4*>(wrow + 16 * ht + 4 * lg);
        wr[ht][0] = wv.x; wr[ht][1] = wv.y; wr[ht][2] = wv.z; wr[ht][3] = wv.w;
      }
    }
  }
  // thread's share of a tile: chunks tid + kT u (entry c / 16, chunk c % 16);
  // entries past the last visible one re-read it
  struct Share {
    uint4 v[kCpt];
  };
  auto chunk_ptr = [&](int j, int u) -> const uint4* {
    const int c = tid + kT * u;
    int64_t e = e0 + (int64_t)j * kPfTile + (c >> 4);
    if (e > e1 - 1) e = e1 - 1;
    size_t r = (size_t)e;
    if constexpr (PG) r = ((size_t)(uint32_t)s_pg[(int)(e >> sh) - p_first] << sh) + (size_t)(e & ((1 << sh) - 1));
    return reinterpret_cast<const uint4*>(keys + r * kPfD + 8 * (c & 15));
  };
  auto load_tile = [&](int j) -> Share {
    Share r;
#pragma unroll
    for (int u = 0; u < kCpt; ++u) r.v[u] = *chunk_ptr(j, u);
    return r;
  };
  auto slot = [&](int buf, int u) -> uint4* {
    const int c = tid + kT * u, kk = c >> 4;
    return &s_k[buf][kk * 16 + ((c & 15) ^ (kk & 15))];
  };
  auto store_tile = [&](int buf, const Share& r) {
#pragma unroll
    for (int u = 0; u < kCpt; ++u) *slot(buf, u) = r.v[u];
  };
  float* out = a.scores + (size_t)row * a.E_cap;
  store_tile(0, load_tile(0));
  __syncthreads();
  for (int j = 0; j < ntiles; ++j) {
    Share next{};
    if (j + 1 < ntiles) next = load_tile(j + 1);  // in flight while tile j is scored
    const uint4* T = s_k[j & 1];
    const int64_t te = e0 + (int64_t)j * kPfTile;
    if constexpr (MF == 32) {
      // 32-entry blocks: D[32 heads x 32 entries] per head tile on
      // v_mfma_f32_32x32x16_bf16; lane (entry l % 32) holds 16 heads of each
      // tile, so the head sum is in-lane plus one exchange (l ^ 32)
#pragma unroll
      for (int kb = 0; kb < kPfTile / 32; ++kb) {
        const int ek = 32 * kb + (l & 31);
        f32x16_t c[kHT];
#pragma unroll
        for (int ht = 0; ht < kHT; ++ht) c[ht] = f32x16_t{};
#pragma unroll
        for (int ks = 0; ks < kKS; ++ks) {
          // B operand: entry ek, d = 16 ks + 8 (l / 32) .. +7 (chunk 2 ks + l / 32)
          const bf16x8_t kf = __builtin_bit_cast(bf16x8_t, T[ek * 16 + ((2 * ks + (l >> 5)) ^ (ek & 15))]);
#pragma unroll
          for (int ht = 0; ht < kHT; ++ht) c[ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[ht][ks], kf, c[ht], 0, 0, 0);
        }
        float part = 0.f;
#pragma unroll
        for (int ht = 0; ht < kHT; ++ht)
#pragma unroll
          for (int i = 0; i < 16; ++i) part += wr[ht][i] * fmaxf(c[ht][i], 0.f);
        part += __shfl_xor(part, 32, 64);
        const int64_t e = te + ek;
        if (l < 32 && e < nv_q && e < e1) out[e] = a.score_bf16 ? round_bf16(part) : part;
      }
    } else
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
      if (lg == 0 && e < nv_q && e < e1) out[e] = a.score_bf16 ? round_bf16(part) : part;
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
  const bool mfma = index_mfma_supported(a) && split && index_mfma_pages_fit(a);
  hipError_t e;
  int n_wg_fused = 0;
  if (mfma) {
    e = launch_index_score_mfma(a, tw, 1, 1, &n_wg_fused, fold, s);
  } else if (index_prefill_mfma_supported(a)) {
    const unsigned gx = (a.E_cap + kPfChunk - 1) / kPfChunk;
    if (a.pg.table)
      CSA_LAUNCH("index_score_prefill", (index_score_prefill_kernel<kPfQpw, kPfMfma, 1>), dim3(gx, rows / kPfQpw),
                 dim3(64 * kPfQpw), 0, s, a);
    else
      CSA_LAUNCH("index_score_prefill", (index_score_prefill_kernel<kPfQpw, kPfMfma, 0>), dim3(gx, rows / kPfQpw),
                 dim3(64 * kPfQpw), 0, s, a);
    e = hipGetLastError();
  } else {
    dim3 g1((a.E_cap + 255) / 256, rows), blk(256);
    if (a.idx_dtype == F32)
      CSA_LAUNCH("index_score", index_score_kernel<float>, g1, blk, 0, s, a);
    else if (a.idx_dtype == BF16)
      CSA_LAUNCH("index_score", index_score_kernel<bf16>, g1, blk, 0, s, a);
    else if (a.idx_dtype == E4M3)
      CSA_LAUNCH("index_score", index_score_kernel<uint8_t>, g1, blk, 0, s, a);
    else
      CSA_LAUNCH("index_score", index_score_kernel<mx4>, g1, blk, 0, s, a);
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
