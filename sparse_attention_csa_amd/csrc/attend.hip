// Shared-KV attention over compressed rows + sliding window + sink (rows a4,
// a5, a6).  Every row is key and value for all heads ("DeepSeek-V4" book ch. 6
// "Shared key-value MQA"); compressed rows (the top-k set for CSA, every
// visible entry for HCA) and window rows share one softmax whose denominator
// also holds exp(sink_h) (book ch. 7 "The sliding window", "Attention sinks";
// "2026 DeepSeek-V4" note, concat(selected, local_kv)).
//
// Generic VALU kernel: one WG per (query, group of 8 heads); row tiles are
// gathered into LDS (rows padded by one float against bank conflicts), the
// online softmax runs per head, and each thread accumulates 1/32 of a head's
// output row.  It also reads the 576-byte FP8 + BF16 entries ([book] ch. 8
// "The main compressed-entry payload"), decoding each coordinate as it
// gathers the row.

#include "common.h"
#include "kernels.h"

namespace csa {

constexpr int kHG = 8;     // heads per WG
constexpr int kTile = 16;  // rows per LDS tile

CSA_DEV int64_t attend_n_compressed(const AttendArgs& a, int b, int row, int64_t t) {
  if (!a.dense) return a.topk_cnt[row];
  const int64_t lim = vis_limit(t, a.m, a.vis);
  const int64_t have = (int64_t)a.n_entries[b] + a.n_add;
  int64_t n = lim < have ? lim : have;
  if (n > a.E_cap) n = a.E_cap;
  return n < 0 ? 0 : n;
}

template <typename T>
__global__ __launch_bounds__(256) void attend_generic_kernel(AttendArgs a) {
  const int row = blockIdx.x, b = row / a.Tq, tid = threadIdx.x;
  const int h0 = blockIdx.y * kHG;
  const int c = a.c, H = a.H;
  const int64_t t = a.q_pos ? a.q_pos[row] : a.q_pos0 + row % a.Tq;
  const int64_t n_c = attend_n_compressed(a, b, row, t);
  const int64_t n_w = (t + 1) < a.n_win ? (t + 1) : a.n_win;
  const int64_t n_rows = n_c + n_w;
  const int64_t wpos0 = a.win_pos0 ? a.win_pos0[b] : a.win_pos0_const;

  extern __shared__ float smem[];
  float* q_s = smem;                        // [kHG][c]
  float* row_s = q_s + kHG * c;             // [kTile][c+1]
  float* p_s = row_s + kTile * (c + 1);     // [kHG][kTile]
  float* alpha_s = p_s + kHG * kTile;       // [kHG]
  int* valid_s = reinterpret_cast<int*>(alpha_s + kHG);  // [kTile]
  const int ldr = c + 1;

  const T* q = reinterpret_cast<const T*>(a.q) + ((size_t)row * H + h0) * c;
  for (int i = tid; i < kHG * c; i += 256) {
    const int h = i / c;
    q_s[i] = (h0 + h < H) ? ld(q, i) * a.scale : 0.f;
  }
  // compressed rows by their cache row (page_row: paged or per sequence)
  __shared__ size_t s_crow[kTile];
  const T* kv = reinterpret_cast<const T*>(a.kv);
  const uint8_t* kv8 = reinterpret_cast<const uint8_t*>(a.kv);  // (kv_fmt)
  const float* ksc = a.kv_scale;
  const T* win = reinterpret_cast<const T*>(a.win) + (size_t)b * a.W_cap * c;
  const int32_t* ids = a.dense ? nullptr : a.topk_idx + (size_t)row * a.k;

  const int ph = tid / 32;         // head owned in the PV phase
  const int pd = tid % 32;         // dims pd, pd+32, ...
  const int nd = c / 32;
  float acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;  // meaningful in threads tid < kHG

  for (int64_t r0 = 0; r0 < n_rows; r0 += kTile) {
    __syncthreads();
    // gather the tile; an id outside [0, E_cap) contributes no row
    if (tid < kTile) {
      const int64_t j = r0 + tid;
      int okr = j < n_rows;
      if (okr && j < n_c) {
        const int64_t e = a.dense ? j : ids[j];
        okr = e >= 0 && e < a.E_cap;
        if (okr) s_crow[tid] = page_row(a.pg, b, e, a.E_cap);
      }
      valid_s[tid] = okr;
    }
    __syncthreads();
    for (int i = tid; i < kTile * c; i += 256) {
      const int r = i / c, d = i % c;
      const int64_t j = r0 + r;
      float v = 0.f;
      if (valid_s[r]) {
        if (j < n_c) {
          const size_t e = s_crow[r];
          if (a.kv_fmt) {  // the 576-byte entry: scaled e4m3 codes, then bf16
            const uint8_t* er = kv8 + (size_t)e * kF8RowB;
            v = d < kF8Dims ? e4m3_to_f32(er[d]) * ksc[e]
                            : bf16_to_f32(*reinterpret_cast<const uint16_t*>(er + kF8Dims + 2 * (d - kF8Dims)));
          } else {
            v = ld(kv, (size_t)e * c + d);
          }
        } else {
          const int64_t p = t - n_w + 1 + (j - n_c);
          int64_t wr = (p - wpos0) % a.W_cap;
          if (wr < 0) wr += a.W_cap;
          v = ld(win, (size_t)wr * c + d);
        }
      }
      row_s[r * ldr + d] = v;
    }
    __syncthreads();
    // logits: 2 threads per (head, row) pair
    {
      const int pair = tid >> 1, half = tid & 1;
      const int h = pair / kTile, r = pair % kTile;
      const int dh = c / 2;
      float x = 0.f;
      const float* qq = q_s + h * c + half * dh;
      const float* rr = row_s + r * ldr + half * dh;
      for (int d = 0; d < dh; ++d) x += qq[d] * rr[d];
      x += __shfl_xor(x, 1, 64);
      if (half == 0) p_s[h * kTile + r] = (valid_s[r] && h0 + h < H) ? x : -INFINITY;
    }
    __syncthreads();
    if (tid < kHG) {
      float mx = m_run;
      for (int r = 0; r < kTile; ++r) mx = fmaxf(mx, p_s[tid * kTile + r]);
      const float alpha = (m_run == -INFINITY) ? 0.f : __expf(m_run - mx);
      float l = l_run * alpha;
      for (int r = 0; r < kTile; ++r) {
        const float lg = p_s[tid * kTile + r];
        const float p = (lg == -INFINITY) ? 0.f : __expf(lg - mx);
        p_s[tid * kTile + r] = p;
        l += p;
      }
      m_run = mx;
      l_run = l;
      alpha_s[tid] = alpha;
    }
    __syncthreads();
    {
      const float al = alpha_s[ph];
      const float* pp = p_s + ph * kTile;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (j < nd) {
          float x = acc[j] * al;
          const float* col = row_s + pd + 32 * j;
          for (int r = 0; r < kTile; ++r) x += pp[r] * col[r * ldr];
          acc[j] = x;
        }
      }
    }
  }
  __syncthreads();
  // sink and normalisation
  if (tid < kHG) {
    const int h = h0 + tid;
    const float z = (a.sink && h < H) ? a.sink[h] : -INFINITY;
    const float M = fmaxf(m_run, z);
    const float em = __expf(m_run - M);
    const float den = l_run * em + ((z == -INFINITY) ? 0.f : __expf(z - M));
    p_s[tid] = em / den;
    if (a.lse && h < H) a.lse[(size_t)row * H + h] = M + __logf(den);
  }
  __syncthreads();
  {
    const float f = p_s[ph];
    T* o = reinterpret_cast<T*>(a.out) + ((size_t)row * H + h0 + ph) * c;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j < nd) {
        float v = acc[j] * f;
        // norm_rope: rotary coordinates rotated back by the query position;
        // the pair partner of coordinate d is d ^ 1, held by lane tid ^ 1
        const float other = __shfl_xor(v, 1, 64);
        const int d = pd + 32 * j, R = a.rope_dims;
        if (a.derot_freq && d >= c - R) {
          float cs, sn;
          rope_cs(-t, a.derot_freq[(d - (c - R)) >> 1], &cs, &sn);
          v = (d & 1) ? (other * sn + v * cs) : (v * cs - other * sn);
        }
        if (h0 + ph < H) st(o, d, v);
      }
    }
  }
}

bool attend_mfma_shape_ok(int H, int c);
size_t attend_mfma_ws_bytes(int BT, int H, int rows_max, int split_rows);
hipError_t launch_attend_mfma(const AttendArgs& a, int rows_max, hipStream_t s);
bool attend_mfma_sparse_fits(const AttendArgs& a, int rows_max);
bool attend_rows_shape_ok(int H, int c);
void attend_rows_plan(int BT, int H, int rows_max, int split_rows, int* n_split, int* rows_per_split);
hipError_t launch_attend_rows(const AttendArgs& a, int rows_max, hipStream_t s);

// partial (max, sum) pairs and bf16 outputs of the row splits
static size_t split_ws_bytes(int BT, int H, int c, int n_split) {
  if (n_split <= 1) return 0;
  return (size_t)BT * n_split * H * (2 * sizeof(float) + (size_t)c * 2);
}

// split partials, then (dense shapes) the decode fold's q . entry sums and
// entry indices at attend_fold_ws_offset
size_t attend_fold_ws_offset(int B, int Tq, int H, int c, int rows_max, int split_rows) {
  size_t n = 256, extra = 0;
  if (attend_mfma_shape_ok(H, c)) extra = attend_mfma_ws_bytes(B * Tq, H, rows_max, split_rows);
  if (attend_rows_shape_ok(H, c)) {
    int ns, rps;
    attend_rows_plan(B * Tq, H, rows_max, split_rows, &ns, &rps);
    const size_t r = split_ws_bytes(B * Tq, H, c, ns);
    if (r > extra) extra = r;
  }
  return (n + extra + 255) / 256 * 256;
}

size_t attend_ws_bytes(int B, int Tq, int H, int c, int rows_max, int split_rows) {
  size_t n = attend_fold_ws_offset(B, Tq, H, c, rows_max, split_rows);
  if (attend_mfma_shape_ok(H, c))
    n += ((size_t)B * H * 64 * 8 + 255) / 256 * 256 + ((size_t)B * 4 + 255) / 256 * 256 + ((size_t)B * c * 2 + 255) / 256 * 256;
  return n;
}

hipError_t launch_attend(const AttendArgs& a, hipStream_t s) {
  // (576-byte entries: the generic kernel decodes them row by row)
  if (a.dtype == BF16 && !a.kv_fmt && a.dense && attend_mfma_shape_ok(a.H, a.c))
    return launch_attend_mfma(a, a.E_cap + a.n_win, s);
  if (a.dtype == BF16 && !a.kv_fmt && !a.dense && attend_mfma_shape_ok(a.H, a.c) &&
      attend_mfma_sparse_fits(a, a.k + a.n_win))
    return launch_attend_mfma(a, a.k + a.n_win, s);
  if (a.dtype == BF16 && !a.kv_fmt && !a.dense && attend_rows_shape_ok(a.H, a.c))
    return launch_attend_rows(a, a.k + a.n_win, s);
  dim3 grid(a.B * a.Tq, (a.H + kHG - 1) / kHG), block(256);
  const size_t sh = sizeof(float) * ((size_t)kHG * a.c + (size_t)kTile * (a.c + 1) + kHG * kTile + kHG + kTile);
  if (a.dtype == F32)
    CSA_LAUNCH(a.dense ? "attend_dense" : "attend_sparse", attend_generic_kernel<float>, grid, block, sh, s, a);
  else
    CSA_LAUNCH(a.dense ? "attend_dense" : "attend_sparse", attend_generic_kernel<bf16>, grid, block, sh, s, a);
  return hipGetLastError();
}

}  // namespace csa
