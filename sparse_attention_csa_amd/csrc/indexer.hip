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
// top-k: grid (B*Tq), 256 threads, one row per WG
// --------------------------------------------------------------------------
// exclusive prefix count of `flag` over the WG in thread order; returns the
// WG total through *total.  s_w holds 4 per-wave counts.
CSA_DEV int block_excl_scan(bool flag, int* s_w, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const unsigned long long mask = __ballot(flag);
  const int in_wave = __popcll(mask & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
  if (lane == 0) s_w[wave] = __popcll(mask);
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int c = s_w[w];
    if (w < wave) off += c;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return off + in_wave;
}

__global__ __launch_bounds__(256) void topk_row_kernel(IndexArgs a) {
  const int row = blockIdx.x, b = row / a.Tq, tq = row % a.Tq;
  const int tid = threadIdx.x;
  const int64_t t = a.q_pos ? a.q_pos[(size_t)b * a.Tq + tq] : a.q_pos0 + tq;
  const int nv = (int)n_visible(a, b, t);
  const float* sc = a.scores + (size_t)row * a.E_cap;
  int32_t* out = a.topk_idx + (size_t)row * a.k;
  const int k = a.k;

  __shared__ int hist[256];
  __shared__ int s_w[4];
  __shared__ uint32_t s_prefix;
  __shared__ int s_krem;

  if (nv <= k) {
    for (int i = tid; i < k; i += 256) out[i] = i < nv ? i : -1;
    if (tid == 0) a.topk_cnt[row] = nv;
    return;
  }
  // radix select of the k-th largest key
  uint32_t prefix = 0;
  int krem = k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    hist[tid] = 0;
    __syncthreads();
    for (int s = tid; s < nv; s += 256) {
      const uint32_t key = f32_key(sc[s]);
      const bool match = pass == 0 || (key >> (shift + 8)) == prefix;
      if (match) atomicAdd(&hist[(key >> shift) & 255], 1);
    }
    __syncthreads();
    if (tid == 0) {
      int above = 0, dsel = 0;
      for (int dgt = 255; dgt >= 0; --dgt) {
        const int h = hist[dgt];
        if (above + h >= krem) {
          dsel = dgt;
          break;
        }
        above += h;
      }
      s_prefix = (prefix << 8) | (uint32_t)dsel;
      s_krem = krem - above;
    }
    __syncthreads();
    prefix = s_prefix;
    krem = s_krem;
    __syncthreads();
  }
  const uint32_t tau = prefix;  // exact key of the k-th largest; take krem ties
  // in-order emission
  int n_out = 0, n_eq = 0;
  for (int base = 0; base < nv; base += 256) {
    const int s = base + tid;
    uint32_t key = 0;
    if (s < nv) key = f32_key(sc[s]);
    const bool eq = s < nv && key == tau;
    int tot_eq;
    const int eq_rank = block_excl_scan(eq, s_w, &tot_eq);
    const bool sel = s < nv && (key > tau || (eq && n_eq + eq_rank < krem));
    int tot_sel;
    const int pos = block_excl_scan(sel, s_w, &tot_sel);
    if (sel) out[n_out + pos] = s;
    n_out += tot_sel;
    n_eq += tot_eq;
  }
  for (int i = n_out + tid; i < k; i += 256) out[i] = -1;
  if (tid == 0) a.topk_cnt[row] = n_out;
}

size_t index_topk_ws_bytes(int B, int Tq, int E_cap, int k) {
  (void)k;
  return (size_t)B * Tq * E_cap * sizeof(float) + 256;
}

hipError_t launch_index_topk(const IndexArgs& a0, hipStream_t s) {
  IndexArgs a = a0;
  if (!a.scores) a.scores = reinterpret_cast<float*>(a.ws);
  dim3 g1((a.E_cap + 255) / 256, a.B * a.Tq), blk(256);
  if (a.idx_dtype == F32)
    CSA_LAUNCH("index_score", index_score_kernel<float>, g1, blk, 0, s, a);
  else if (a.idx_dtype == BF16)
    CSA_LAUNCH("index_score", index_score_kernel<bf16>, g1, blk, 0, s, a);
  else
    CSA_LAUNCH("index_score", index_score_kernel<uint8_t>, g1, blk, 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  CSA_LAUNCH("topk_row", topk_row_kernel, dim3(a.B * a.Tq), blk, 0, s, a);
  return hipGetLastError();
}

}  // namespace csa
