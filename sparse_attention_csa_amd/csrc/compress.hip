// Compressor kernels (row a1): the softmax-weighted fold of m (HCA) or 2m
// (CSA, overlapping) source tokens into one compressed entry, one softmax per
// coordinate across the source positions ("2026 DeepSeek-V4" note, "Key
// design 1" and "Key design 2" equations; "DeepSeek-V4" book ch. 5 "One weight
// distribution per coordinate" and the start-of-sequence rule).
//
// Both kernels are HBM-streaming: a wavefront covers 64 consecutive
// coordinates of one source row, so every load is a contiguous 128 B (bf16)
// or 256 B (f32) segment; the per-coordinate softmax is an online max/sum
// across source tokens, split over token groups and merged through LDS.

#include "common.h"
#include "fold.h"
#include "kernels.h"

namespace csa {

template <typename T>
CSA_DEV const T* cptr(const void* p) {
  return reinterpret_cast<const T*>(p);
}

// --------------------------------------------------------------------------
// csa_compress: entries of a chunk.  grid (T/m, B), 256 threads.  Each thread
// owns up to 2 coordinates (c <= 512) and walks all sources of its entry.
// --------------------------------------------------------------------------
template <typename T, typename TO>
__global__ __launch_bounds__(256) void compress_chunk_kernel(CompressArgs a) {
  const int i = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int c = a.c, m = a.m, Tn = a.T, lw = a.logit_width;
  const size_t sc = a.seq_stride ? a.seq_stride : (size_t)Tn * c;
  const size_t sz = a.seq_stride ? a.seq_stride : (size_t)Tn * lw;
  const size_t pc = a.prev_seq_stride ? a.prev_seq_stride : (size_t)m * c;
  const size_t pz = a.prev_seq_stride ? a.prev_seq_stride : (size_t)m * lw;
  const T* ca = cptr<T>(a.ca) + (size_t)b * sc;
  const T* cb = a.cb ? cptr<T>(a.cb) + (size_t)b * sc : nullptr;
  const T* za = a.za ? cptr<T>(a.za) + (size_t)b * sz : nullptr;
  const T* zb = a.zb ? cptr<T>(a.zb) + (size_t)b * sz : nullptr;
  const bool has_b = (cb != nullptr) && (i > 0 || a.prev_cb != nullptr);
  const T* pcb = a.prev_cb ? cptr<T>(a.prev_cb) + (size_t)b * pc : nullptr;
  const T* pzb = a.prev_zb ? cptr<T>(a.prev_zb) + (size_t)b * pz : nullptr;

  __shared__ float s_logit[256];  // scalar logits from score_w, one per source token (m <= 128)
  __shared__ float s_red[8];
  if (a.score_w) {
    // one-branch form: logit_j = score_w . content_a[token j]
    const int wave = tid >> 6, lane = tid & 63;
    for (int j = wave; j < m; j += 4) {
      const size_t row = (size_t)(m * i + j) * c;
      float acc = 0.f;
      for (int r = lane; r < c; r += 64) acc += a.score_w[r] * ld(ca, row + r);
      acc = wave_sum(acc);
      if (lane == 0) s_logit[j] = acc;
    }
    __syncthreads();
  }

  float vals[2];
  int nv = 0;
  for (int r = tid; r < c; r += 256, ++nv) {
    Soft s{-INFINITY, 0.f, 0.f};
    for (int j = 0; j < m; ++j) {
      const int tok = m * i + j;
      float lg;
      if (a.score_w)
        lg = s_logit[j];
      else
        lg = ld(za, (size_t)tok * lw + (lw == 1 ? 0 : r));
      if (a.bias_a) lg += a.bias_a[j * c + r];
      soft_push(s, lg, ld(ca, (size_t)tok * c + r));
    }
    if (has_b) {
      for (int j = 0; j < m; ++j) {
        float lg, v;
        if (i > 0) {
          const int tok = m * (i - 1) + j;
          lg = ld(zb, (size_t)tok * lw + (lw == 1 ? 0 : r));
          v = ld(cb, (size_t)tok * c + r);
        } else {
          lg = ld(pzb, (size_t)j * lw + (lw == 1 ? 0 : r));
          v = ld(pcb, (size_t)j * c + r);
        }
        if (a.bias_b) lg += a.bias_b[j * c + r];
        soft_push(s, lg, v);
      }
    }
    vals[nv] = s.acc / s.l;
  }

  const size_t orow = ((size_t)b * a.E_cap + (size_t)(a.first + i)) * c;
  if constexpr (sizeof(TO) == 1) {
    // e4m3 output: one scale per entry = max|v| / 448
    float amax = 0.f;
    for (int u = 0; u < nv; ++u) amax = fmaxf(amax, fabsf(vals[u]));
    amax = wave_max(amax);
    if ((tid & 63) == 0) s_red[tid >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
    float scale = amax / 448.0f;
    if (!(scale > 0.f)) scale = 1.f;
    uint8_t* o = reinterpret_cast<uint8_t*>(a.out) + orow;
    int u = 0;
    for (int r = tid; r < c; r += 256, ++u) o[r] = f32_to_e4m3(vals[u] / scale);
    if (tid == 0) a.out_scale[(size_t)b * a.E_cap + a.first + i] = scale;
  } else {
    TO* o = reinterpret_cast<TO*>(a.out) + orow;
    int u = 0;
    for (int r = tid; r < c; r += 256, ++u) st(o, r, vals[u]);
  }
}

hipError_t launch_compress(const CompressArgs& a, hipStream_t s) {
  dim3 grid(a.T / a.m, a.B), block(256);
  if (a.dtype == F32) {
    if (a.out_dtype == F32)
      CSA_LAUNCH("compress_chunk", (compress_chunk_kernel<float, float>), grid, block, 0, s, a);
    else if (a.out_dtype == BF16)
      CSA_LAUNCH("compress_chunk", (compress_chunk_kernel<float, bf16>), grid, block, 0, s, a);
    else
      CSA_LAUNCH("compress_chunk", (compress_chunk_kernel<float, uint8_t>), grid, block, 0, s, a);
  } else {
    if (a.out_dtype == F32)
      CSA_LAUNCH("compress_chunk", (compress_chunk_kernel<bf16, float>), grid, block, 0, s, a);
    else if (a.out_dtype == BF16)
      CSA_LAUNCH("compress_chunk", (compress_chunk_kernel<bf16, bf16>), grid, block, 0, s, a);
    else
      CSA_LAUNCH("compress_chunk", (compress_chunk_kernel<bf16, uint8_t>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

// --------------------------------------------------------------------------
// Decode step: fold the block whose entry becomes visible at this position,
// and append the new token to the tail ring and the window ring.
//
// grid (jobs, B), 256 threads.  Job j < c/64 owns coordinates [64j, 64j+64)
// of the main entry and of the new token's appended rows; the last job of a
// CSA layer owns the whole indexer key (its e4m3 scale needs the row
// maximum).  A thread loads 16 contiguous bytes (V coordinates) of each of
// its source rows: the TR = W/V threads of a row cover the job's W
// coordinates, the G = 256/TR thread groups take interleaved source tokens,
// and the per-coordinate online softmaxes of the groups merge through LDS.
//
// The ring holds the last 2m tokens (3m with overlap) and a fold reads at
// most the 2m tokens before t (the new token itself from the step's inputs),
// so the new token's slot is never a source and the appends need no
// ordering against the reads.  Every workgroup of a sequence reads
// n_entries[b]; the last one to finish (a per-sequence counter in the
// workspace, returned to zero) publishes the new count.
// --------------------------------------------------------------------------
template <typename T, typename TI>
__global__ __launch_bounds__(kFoldT) void fold_append_kernel(FoldArgs a) {
  __shared__ Soft s_part[kFoldT * Vec16<T>::V];
  __shared__ float s_red[kFoldT / 64];
  const int job = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int m = a.m, R = a.R, c = a.c;
  const int64_t t = a.pos[b];
  const int n_have = a.n_entries[b];
  __asm__ __volatile__("" ::"s"(t), "s"(n_have));  // both loads in one round trip
  const int64_t lim = vis_limit(t, m, a.vis);
  const bool fold = (lim == (int64_t)n_have + 1) && n_have < a.E_cap;
  const int64_t e = n_have;
  const int nstr = a.overlap ? 4 : 2;
  const int slot = (int)(t % R);

  if (job < c / kFoldCW) {
    const int r0 = job * kFoldCW;
    T* tail = reinterpret_cast<T*>(a.tail) + (size_t)b * nstr * R * c;
    const T* io = reinterpret_cast<const T*>(a.streams) + (size_t)b * nstr * c;
    if (fold) {
      const float val = fold_job<T>(tail, io, c, r0, kFoldCW, m, R, t, e, a.overlap && e > 0, a.bias_a,
                                    a.bias_b, s_part);
      if (tid < kFoldCW) st(reinterpret_cast<T*>(a.kv_cache), ((size_t)b * a.E_cap + e) * c + r0 + tid, val);
    }
    for (int i = tid; i < nstr * kFoldCW; i += kFoldT) {
      const int sc = i / kFoldCW, r = r0 + i % kFoldCW;
      tail[((size_t)sc * R + slot) * c + r] = io[(size_t)sc * c + r];
    }
    if (tid < kFoldCW) {
      T* ring = reinterpret_cast<T*>(a.win_ring) + (size_t)b * a.n_win * c;
      ring[(size_t)(t % a.n_win) * c + r0 + tid] = reinterpret_cast<const T*>(a.x_new)[(size_t)b * c + r0 + tid];
    }
  } else {
    const int d = a.d_I;
    T* itail = reinterpret_cast<T*>(a.idx_tail) + (size_t)b * 4 * R * d;
    const T* iio = reinterpret_cast<const T*>(a.idx_streams) + (size_t)b * 4 * d;
    if (fold) {
      const float iv = fold_job<T>(itail, iio, d, 0, d, m, R, t, e, e > 0, a.ibias_a, a.ibias_b, s_part);
      const size_t row = (size_t)b * a.E_cap + e;
      if constexpr (sizeof(TI) == 1) {
        float am = wave_max(tid < d ? fabsf(iv) : 0.f);
        if ((tid & 63) == 0) s_red[tid >> 6] = am;
        __syncthreads();
        am = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
        float scale = am / 448.0f;
        if (!(scale > 0.f)) scale = 1.f;
        if (tid < d) reinterpret_cast<uint8_t*>(a.idx_cache)[row * d + tid] = f32_to_e4m3(iv / scale);
        if (tid == 0) a.idx_scale[row] = scale;
      } else {
        if (tid < d) st(reinterpret_cast<TI*>(a.idx_cache), row * d + tid, iv);
      }
    }
    for (int i = tid; i < 4 * d; i += kFoldT) {
      const int sc = i / d, r = i % d;
      itail[((size_t)sc * R + slot) * d + r] = iio[(size_t)sc * d + r];
    }
  }
  // the last workgroup of the sequence publishes the count; every
  // workgroup's read of n_entries[b] completed before its increment
  __syncthreads();
  if (tid == 0) {
    const int done = atomicAdd(&a.counters[b], 1);
    if (done == (int)gridDim.x - 1) {
      a.counters[b] = 0;
      if (fold) a.n_entries[b] = n_have + 1;
    }
  }
}

hipError_t launch_fold_append(const FoldArgs& a, hipStream_t s) {
  dim3 grid(a.c / kFoldCW + (a.idx_dtype >= 0 ? 1 : 0), a.B), block(kFoldT);
  if (a.dtype == F32) {
    if (a.idx_dtype == E4M3)
      CSA_LAUNCH("fold_append", (fold_append_kernel<float, uint8_t>), grid, block, 0, s, a);
    else if (a.idx_dtype == BF16)
      CSA_LAUNCH("fold_append", (fold_append_kernel<float, bf16>), grid, block, 0, s, a);
    else
      CSA_LAUNCH("fold_append", (fold_append_kernel<float, float>), grid, block, 0, s, a);
  } else {
    if (a.idx_dtype == E4M3)
      CSA_LAUNCH("fold_append", (fold_append_kernel<bf16, uint8_t>), grid, block, 0, s, a);
    else if (a.idx_dtype == F32)
      CSA_LAUNCH("fold_append", (fold_append_kernel<bf16, float>), grid, block, 0, s, a);
    else
      CSA_LAUNCH("fold_append", (fold_append_kernel<bf16, bf16>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

// --------------------------------------------------------------------------
// Prefill epilogue: the window ring receives the last n_win rows and the tail
// ring the last R tokens' streams, so decode can continue after the chunk.
// grid (B, rows), 256 threads, one row per WG.
// --------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void prefill_state_kernel(PrefillStateArgs a) {
  const int b = blockIdx.x, row = blockIdx.y, tid = threadIdx.x;
  const int n_w = a.n_win < (a.n_win - 1 + a.T) ? a.n_win : (a.n_win - 1 + a.T);
  const int n_t = a.R < a.T ? a.R : a.T;
  if (row < n_w) {
    // window row of position p = pos0 + T - n_w + row
    const int64_t p = a.pos0 + a.T - n_w + row;
    const int64_t src_row = p - (a.pos0 - (a.n_win - 1));
    const T* src = cptr<T>(a.win) + ((size_t)b * (a.n_win - 1 + a.T) + src_row) * a.c;
    T* dst = reinterpret_cast<T*>(a.win_ring) + ((size_t)b * a.n_win + (size_t)(p % a.n_win)) * a.c;
    for (int r = tid; r < a.c; r += 256) dst[r] = src[r];
  } else if (row < n_w + n_t) {
    const int j = row - n_w;
    const int64_t p = a.pos0 + a.T - n_t + j;
    const int64_t tok = p - a.pos0;
    for (int sc = 0; sc < a.S; ++sc) {
      const T* src = cptr<T>(a.streams) + (((size_t)b * a.S + sc) * a.T + tok) * a.c;
      T* dst = reinterpret_cast<T*>(a.tail) + (((size_t)b * a.S + sc) * a.R + (size_t)(p % a.R)) * a.c;
      for (int r = tid; r < a.c; r += 256) dst[r] = src[r];
    }
    if (a.idx_streams) {
      for (int sc = 0; sc < 4; ++sc) {
        const T* src = cptr<T>(a.idx_streams) + (((size_t)b * 4 + sc) * a.T + tok) * a.d_I;
        T* dst = reinterpret_cast<T*>(a.idx_tail) + (((size_t)b * 4 + sc) * a.R + (size_t)(p % a.R)) * a.d_I;
        for (int r = tid; r < a.d_I; r += 256) dst[r] = src[r];
      }
    }
  } else if (row == n_w + n_t && tid == 0) {
    a.n_entries[b] += a.new_entries;
  }
}

hipError_t launch_prefill_state(const PrefillStateArgs& a, hipStream_t s) {
  const int n_w = a.n_win < (a.n_win - 1 + a.T) ? a.n_win : (a.n_win - 1 + a.T);
  const int n_t = a.R < a.T ? a.R : a.T;
  dim3 grid(a.B, n_w + n_t + 1), block(256);
  if (a.dtype == F32)
    CSA_LAUNCH("prefill_state", prefill_state_kernel<float>, grid, block, 0, s, a);
  else
    CSA_LAUNCH("prefill_state", prefill_state_kernel<bf16>, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace csa
