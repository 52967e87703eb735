// Lightning-indexer scoring on MFMA for decode-shaped work (row a2):
// I[t, s] = sum_h w[t, h] * ReLU(q[t, h] . K[s]) ("2026 DeepSeek-V4" note,
// "Key design 1" indexer equation; "DeepSeek-V4" book ch. 6 "The index
// score"), for d_I = 128 and H_I a multiple of 16 (<= 64).
//
// The scan over the visible keys is the HBM stream of a CSA decode step.  A
// wavefront scores 16 keys per step: C[heads x keys] = Q[heads x d] .
// K^T[d x keys] with Q in registers (loaded once) and each lane loading its
// key's 16- or 32-byte slices straight from HBM into the B operand
// (v_mfma_f32_16x16x32_bf16 for bf16 keys, 4 k-steps; the scaled f8f6f4
// v_mfma 16x16x128 with unit scales for e4m3 keys, one step).  The
// accumulator holds 4 heads x 1 key per lane, so ReLU, the head weights and
// the head sum are in-lane, then two cross-lane adds.  For e4m3 the per-head
// query scale is folded into w and the per-key scale multiplies the sum (both
// positive, so they commute with ReLU).  Each wave scores a contiguous run of
// tiles in batches of four, loading the next batch before scoring the current
// one, so eight tiles' keys are in flight per wave.  With use_hist the wave also counts the
// top 11 bits of each score's order-preserving key into an LDS histogram that
// is added to the row's global histogram at the end (stage 1 of the top-k).

#include <type_traits>

#include "common.h"
#include "topk.h"

namespace csa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

namespace {

constexpr int kD = 128;

template <int FP8>
struct KeyOp;

template <>
struct KeyOp<0> {  // bf16 keys: 4 x 16 B per lane
  uint4 v[4];
  CSA_DEV void load(const uint16_t* row, int lg, bool ok) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      v[ks] = ok ? *reinterpret_cast<const uint4*>(row + 32 * ks + 8 * lg) : make_uint4(0, 0, 0, 0);
  }
};

// e4m3 keys: 2 x 16 B per lane.  The reduction index is permuted so that one
// load instruction covers bytes 0..63 (then 64..127) of each key contiguously:
// lane group g supplies d = 16g..16g+15 and 64+16g..64+16g+15 as its 32
// k-slots; the query operand uses the same permutation.
template <>
struct KeyOp<1> {
  uint4 v[2];
  CSA_DEV void load(const uint8_t* row, int lg, bool ok) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      v[i] = ok ? *reinterpret_cast<const uint4*>(row + 64 * i + 16 * lg) : make_uint4(0, 0, 0, 0);
  }
};

CSA_DEV int64_t n_vis(const IndexArgs& a, int b, int64_t t) {
  const int64_t lim = vis_limit(t, a.m, a.vis);
  const int64_t have = (int64_t)a.n_entries[b] + a.n_add;
  int64_t n = lim < have ? lim : have;
  if (n > a.E_cap) n = a.E_cap;
  return n < 0 ? 0 : n;
}

}  // namespace

// grid (n_wg, rows), 256 threads
template <int FP8, int HT>
__global__ __launch_bounds__(256) void index_score_mfma_kernel(IndexArgs a, TopkWs ws, int use_hist) {
  __shared__ int s_hist[kTopkBins];
  const int row = blockIdx.y, b = row / a.Tq, tq = row % a.Tq;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, li = l & 15, lg = l >> 4;
  const int64_t t = a.q_pos ? a.q_pos[(size_t)b * a.Tq + tq] : a.q_pos0 + tq;
  const int64_t nv = n_vis(a, b, t);
  const int H = a.H_I;
  if (use_hist) {
    for (int i = tid; i < kTopkBins; i += 256) s_hist[i] = 0;
    __syncthreads();
  }
  // query operands and effective head weights for this lane's C rows
  bf16x8_t qb[HT][4];
  i32x8_t q8[HT];
  float wr[HT][4];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const int h = 16 * ht + li;
    if constexpr (FP8) {
      const uint8_t* q = reinterpret_cast<const uint8_t*>(a.q) + ((size_t)row * H + h) * kD + 16 * lg;
      const uint4 v0 = *reinterpret_cast<const uint4*>(q), v1 = *reinterpret_cast<const uint4*>(q + 64);
      q8[ht] = i32x8_t{(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w, (int)v1.x, (int)v1.y, (int)v1.z, (int)v1.w};
    } else {
      const uint16_t* q = reinterpret_cast<const uint16_t*>(a.q) + ((size_t)row * H + h) * kD;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qb[ht][ks] = *reinterpret_cast<const bf16x8_t*>(q + 32 * ks + 8 * lg);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int hh = 16 * ht + 4 * lg + r;
      float wv = a.w[(size_t)row * H + hh];
      if (a.q_scale) wv *= a.q_scale[(size_t)row * H + hh];
      wr[ht][r] = wv;
    }
  }
  typedef typename std::conditional<FP8, uint8_t, uint16_t>::type KT;
  const KT* keys = reinterpret_cast<const KT*>(a.keys) + (size_t)b * a.E_cap * kD;
  const float* ksc = a.k_scale ? a.k_scale + (size_t)b * a.E_cap : nullptr;
  float* out = a.scores + (size_t)row * a.E_cap;

  // each wave scores a contiguous range of 16-key tiles, U tiles per batch,
  // with the next batch's loads in flight while the current one is scored
  constexpr int U = 4;
  const int64_t ntile = (nv + 15) / 16;
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  const int64_t per = ((ntile + nwaves - 1) / nwaves + U - 1) / U * U;
  const int64_t t0 = ((int64_t)blockIdx.x * 4 + w) * per;
  const int64_t t1 = t0 + per < ntile ? t0 + per : ntile;
  auto load_batch = [&](KeyOp<FP8>* kb, int64_t tb) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t e = (tb + u) * 16 + li;
      const bool ok = tb + u < t1 && e < nv;
      kb[u].load(keys + (size_t)(ok ? e : 0) * kD, lg, ok);
    }
  };
  KeyOp<FP8> cur[U], nxt[U];
  if (t0 < t1) load_batch(cur, t0);
  for (int64_t tb = t0; tb < t1; tb += U) {
    if (tb + U < t1) load_batch(nxt, tb + U);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t e = (tb + u) * 16 + li;
      const bool ok = tb + u < t1 && e < nv;
      float part = 0.f;
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        f32x4_t c = {0.f, 0.f, 0.f, 0.f};
        if constexpr (FP8) {
          const i32x8_t kb = i32x8_t{(int)cur[u].v[0].x, (int)cur[u].v[0].y, (int)cur[u].v[0].z,
                                     (int)cur[u].v[0].w, (int)cur[u].v[1].x, (int)cur[u].v[1].y,
                                     (int)cur[u].v[1].z, (int)cur[u].v[1].w};
          c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(q8[ht], kb, c, 0, 0, 0, 127, 0, 127);
        } else {
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qb[ht][ks], __builtin_bit_cast(bf16x8_t, cur[u].v[ks]),
                                                        c, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) part += wr[ht][r] * fmaxf(c[r], 0.f);
      }
      part += __shfl_xor(part, 16, 64);
      part += __shfl_xor(part, 32, 64);
      if (ok && lg == 0) {
        if (ksc) part *= ksc[e];
        out[e] = part;
        if (use_hist) atomicAdd(&s_hist[f32_key(part) >> kTopkShift], 1);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) cur[u] = nxt[u];
  }
  if (use_hist) {
    __syncthreads();
    int* gh = ws.hist + (size_t)row * kTopkBins;
    for (int i = tid; i < kTopkBins; i += 256) {
      const int v = s_hist[i];
      if (v) atomicAdd(&gh[i], v);
    }
  }
}

bool index_mfma_supported(const IndexArgs& a) {
  return (a.idx_dtype == BF16 || a.idx_dtype == E4M3) && a.d_I == kD && a.H_I % 16 == 0 && a.H_I <= 64;
}

hipError_t launch_index_score_mfma(const IndexArgs& a, const TopkWs& ws, int use_hist, hipStream_t s) {
  const int rows = a.B * a.Tq;
  // about 1024 workgroups in total, at least 4 tiles (one batch) per wave
  int per_row = (1024 + rows - 1) / rows;
  const int max_wg = (int)((((int64_t)a.E_cap + 15) / 16 + 15) / 16);
  if (per_row > max_wg) per_row = max_wg;
  if (per_row < 1) per_row = 1;
  dim3 grid(per_row, rows), block(256);
  const int HT = a.H_I / 16;
#define CSA_IDX_LAUNCH(F, N)                                                                       \
  CSA_LAUNCH("index_score_mfma", (index_score_mfma_kernel<F, N>), grid, block, 0, s, a, ws, use_hist)
  if (a.idx_dtype == E4M3) {
    if (HT == 4) CSA_IDX_LAUNCH(1, 4); else if (HT == 3) CSA_IDX_LAUNCH(1, 3);
    else if (HT == 2) CSA_IDX_LAUNCH(1, 2); else CSA_IDX_LAUNCH(1, 1);
  } else {
    if (HT == 4) CSA_IDX_LAUNCH(0, 4); else if (HT == 3) CSA_IDX_LAUNCH(0, 3);
    else if (HT == 2) CSA_IDX_LAUNCH(0, 2); else CSA_IDX_LAUNCH(0, 1);
  }
#undef CSA_IDX_LAUNCH
  return hipGetLastError();
}

}  // namespace csa
