// Compressor kernels (row a1): the softmax-weighted fold of m (HCA) or 2m
// (CSA, overlapping) source tokens into one compressed entry, one softmax per
// coordinate across the source positions ("2026 DeepSeek-V4" note, "Key
// design 1" and "Key design 2" equations; "DeepSeek-V4" book ch. 5 "One weight
// distribution per coordinate" and the start-of-sequence rule).
//
// compress_chunk_kernel (a prefill chunk, csa_compress): one workgroup per
// entry, a thread per coordinate walks the entry's sources with an online
// max / sum (consecutive threads read consecutive coordinates of a source
// row).  fold_append_kernel (a decode step): source tokens split over thread
// groups, the groups' online states merged by lane shuffles and through LDS
// (fold.h).
//
// Produced indexer keys are stored in the cache's format: bf16 / f32, e4m3
// with one float32 scale per key (max |v| / 448), or OCP MXFP4 (E2M1 pairs,
// one E8M0 scale 2^(floor(log2 max |v|) - 2) per block of 32; "DeepSeek-V4"
// book ch. 16 "Why use fine-grained scales?").

#include <type_traits>

#include "common.h"
#include "fold.h"
#include "kernels.h"

namespace csa {

template <typename T>
CSA_DEV const T* cptr(const void* p) {
  return reinterpret_cast<const T*>(p);
}

// the element type a compressor output is stored as when it is not the
// 576-byte entry (the FP8 + BF16 tag maps to bf16, never used for it)
template <typename TO>
struct TIOf {
  typedef TO type;
};
template <>
struct TIOf<f8b16> {
  typedef bf16 type;
};
template <typename TO>
using TI_of = typename TIOf<TO>::type;

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
  // the entry; variable-length chunks: the sequence's chunk starts at vp0,
  // its entries run from floor(vp0 / m) to the last block that ends in it,
  // and sources before vp0 come from the tail ring (blocks never cross
  // sequences: a trailing fragment stays in the tail)
  int64_t e = a.first + i, vp0 = 0;
  const T* vtail = nullptr;
  if (a.seq_pos0) {
    vp0 = a.seq_pos0[b];
    vp0 = vp0 < 0 ? 0 : vp0;
    int64_t len = a.seq_len[b];
    len = len < 0 ? 0 : (len > Tn ? Tn : len);
    e = vp0 / m + i;
    if (e >= (vp0 + len) / m || e >= a.E_cap) return;  // (uniform in the workgroup)
    vtail = cptr<T>(a.tail) + (size_t)b * (a.cb ? 4 : 2) * a.R * c;
  }
  const bool has_b = a.seq_pos0 ? (cb != nullptr && e > 0) : ((cb != nullptr) && (i > 0 || a.prev_cb != nullptr));
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
    // the m sources of a branch in batches whose loads are in flight
    // together (the online softmax takes them in source order; loads past
    // the last source re-read it and are dropped)
    constexpr int kSrcB = 8;
    auto push_branch = [&](auto logit_of, auto value_of) {
      for (int j0 = 0; j0 < m; j0 += kSrcB) {
        float lgs[kSrcB], vs[kSrcB];
#pragma unroll
        for (int u = 0; u < kSrcB; ++u) {
          const int j = j0 + u < m ? j0 + u : m - 1;
          lgs[u] = logit_of(j);
          vs[u] = value_of(j);
        }
#pragma unroll
        for (int u = 0; u < kSrcB; ++u)
          if (j0 + u < m) soft_push(s, lgs[u], vs[u]);
      }
    };
    if (a.seq_pos0) {
      // stream st (0 content a, 1 logits a, 2 content b, 3 logits b) at
      // position p (logit width c)
      auto row = [&](int st, int64_t p) -> const T* {
        const T* ch = st == 0 ? ca : (st == 1 ? za : (st == 2 ? cb : zb));
        return p >= vp0 ? ch + (size_t)(p - vp0) * c : vtail + ((size_t)st * a.R + (size_t)(p % a.R)) * c;
      };
      const int64_t pa = (int64_t)m * e, pb = (int64_t)m * (e - 1);
      push_branch([&](int j) { return ld(row(1, pa + j), r) + (a.bias_a ? a.bias_a[j * c + r] : 0.f); },
                  [&](int j) { return ld(row(0, pa + j), r); });
      if (has_b)
        push_branch([&](int j) { return ld(row(3, pb + j), r) + (a.bias_b ? a.bias_b[j * c + r] : 0.f); },
                    [&](int j) { return ld(row(2, pb + j), r); });
      vals[nv] = s.acc / s.l;
      continue;
    }
    push_branch(
        [&](int j) {
          const int tok = m * i + j;
          const float lg = a.score_w ? s_logit[j] : ld(za, (size_t)tok * lw + (lw == 1 ? 0 : r));
          return lg + (a.bias_a ? a.bias_a[j * c + r] : 0.f);
        },
        [&](int j) { return ld(ca, (size_t)(m * i + j) * c + r); });
    if (has_b) {
      // the previous block: in the chunk, or (first entry) in prev_*
      const T* zsrc = i > 0 ? zb + (size_t)m * (i - 1) * lw : pzb;
      const T* csrc = i > 0 ? cb + (size_t)m * (i - 1) * c : pcb;
      push_branch(
          [&](int j) {
            return ld(zsrc, (size_t)j * lw + (lw == 1 ? 0 : r)) + (a.bias_b ? a.bias_b[j * c + r] : 0.f);
          },
          [&](int j) { return ld(csrc, (size_t)j * c + r); });
    }
    vals[nv] = s.acc / s.l;
  }

  const size_t erow = page_row(a.pg, b, e, a.E_cap);  // the entry's cache row
  const size_t orow = erow * c;
  if constexpr (std::is_same<TO, mx4>::value) {
    // MXFP4 output (c a multiple of 32): the 32 lanes of an aligned lane
    // group hold one block; a pair of neighbouring lanes forms one byte
    uint8_t* o = reinterpret_cast<uint8_t*>(a.out) + orow / 2;
    uint8_t* so = reinterpret_cast<uint8_t*>(a.out_scale) + orow / 32;
    for (int u = 0; u < (c + 255) / 256; ++u) {  // the same trip count in every lane
      const int r = tid + 256 * u;
      uint32_t sc;
      const uint32_t code = mx_quantize_lane(r < c ? vals[u] : 0.f, &sc);
      const uint32_t odd = __shfl_xor(code, 1, 64);
      if (r < c && (r & 1) == 0) o[r / 2] = (uint8_t)(code | (odd << 4));
      if (r < c && (r & 31) == 0) so[r / 32] = (uint8_t)sc;
    }
  } else if constexpr (std::is_same<TO, uint8_t>::value) {
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
    if (tid == 0) reinterpret_cast<float*>(a.out_scale)[erow] = scale;
  } else if (a.nr.on || std::is_same<TO, f8b16>::value) {
    // the entry prepared for the core attention (nr.on): RMSNorm over its c
    // coordinates, then the rotary pairs (neighbouring lanes) at its position,
    // the first token of its block; stored as T or as the 576-byte entry
    const int nu = (c + 255) / 256;  // the same trip count in every lane
    if (!a.nr.on) {
      store_entry<TI_of<TO>>(vals, nu, c, std::is_same<TO, f8b16>::value, a.out,
                             reinterpret_cast<float*>(a.out_scale), erow, s_red);
      return;
    }
    float ss = 0.f;
    for (int u = 0; u < nu; ++u)
      if (tid + 256 * u < c) ss += vals[u] * vals[u];
    ss = wave_sum(ss);
    if ((tid & 63) == 0) s_red[tid >> 6] = ss;
    __syncthreads();
    ss = s_red[0] + s_red[1] + s_red[2] + s_red[3];
    const float inv = 1.0f / sqrtf(ss / (float)c + a.nr.eps);
    const int64_t pos = (int64_t)m * e;
    const int R = a.nr.rope_dims;
    for (int u = 0; u < nu; ++u) {
      const int r = tid + 256 * u;
      float v = r < c ? vals[u] * inv * a.nr.g_kv[r] : 0.f;
      const float other = __shfl_xor(v, 1, 64);
      if (r < c && r >= c - R) {
        float cs, sn;
        rope_cs(pos, a.nr.inv_freq[(r - (c - R)) >> 1], &cs, &sn);
        v = (r & 1) ? (other * sn + v * cs) : (v * cs - other * sn);
      }
      vals[u] = v;
    }
    store_entry<TI_of<TO>>(vals, nu, c, std::is_same<TO, f8b16>::value, a.out, reinterpret_cast<float*>(a.out_scale),
                           erow, s_red);
  } else if constexpr (!std::is_same<TO, f8b16>::value) {
    TO* o = reinterpret_cast<TO*>(a.out) + orow;
    int u = 0;
    for (int r = tid; r < c; r += 256, ++u) st(o, r, vals[u]);
  }
}

template <typename T>
static void launch_compress_to(const CompressArgs& a, dim3 grid, dim3 block, hipStream_t s) {
  if (a.out_dtype == F32)
    CSA_LAUNCH("compress_chunk", (compress_chunk_kernel<T, float>), grid, block, 0, s, a);
  else if (a.out_dtype == BF16)
    CSA_LAUNCH("compress_chunk", (compress_chunk_kernel<T, bf16>), grid, block, 0, s, a);
  else if (a.out_dtype == E4M3)
    CSA_LAUNCH("compress_chunk", (compress_chunk_kernel<T, uint8_t>), grid, block, 0, s, a);
  else if (a.out_dtype == FP8BF16)
    CSA_LAUNCH("compress_chunk", (compress_chunk_kernel<T, f8b16>), grid, block, 0, s, a);
  else
    CSA_LAUNCH("compress_chunk", (compress_chunk_kernel<T, mx4>), grid, block, 0, s, a);
}

// Long one-branch blocks (HCA, m' >= 32 sources per entry) with plain f32 /
// bf16 output: grid (T/m, B, c/64).  A workgroup folds 64 coordinates of
// one entry; wavefront g takes sources g, g + 4, ... of each coordinate with
// its own online softmax state (source loads in batches in flight), and the
// four states merge through LDS in wavefront order.  (The whole-entry
// kernel above walks all m sources of a coordinate in one thread: with
// m = 128 that chain of dependent updates set its time.)
constexpr int kSliceC = 64;
template <typename T, typename TO>
__global__ __launch_bounds__(256) void compress_slices_kernel(CompressArgs a) {
  const int i = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, g = tid >> 6;
  const int c = a.c, m = a.m, lw = a.logit_width;
  const int r = blockIdx.z * kSliceC + (tid & 63);
  const size_t sc = a.seq_stride ? a.seq_stride : (size_t)a.T * c;
  const size_t sz = a.seq_stride ? a.seq_stride : (size_t)a.T * lw;
  const T* ca = cptr<T>(a.ca) + (size_t)b * sc + (size_t)m * i * c + r;
  const T* za = cptr<T>(a.za) + (size_t)b * sz + (size_t)m * i * lw + (lw == 1 ? 0 : r);
  __shared__ Soft s_part[4][kSliceC];
  Soft sf{-INFINITY, 0.f, 0.f};
  constexpr int kB = 8;  // sources per batch and wavefront
  for (int j0 = g; j0 < m; j0 += 4 * kB) {
    float lgs[kB], vs[kB];
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      int j = j0 + 4 * u;
      j = j < m ? j : m - 1;  // (past the last source: re-read it, dropped)
      lgs[u] = ld(za, (size_t)j * lw) + (a.bias_a ? a.bias_a[(size_t)j * c + r] : 0.f);
      vs[u] = ld(ca, (size_t)j * c);
    }
#pragma unroll
    for (int u = 0; u < kB; ++u)
      if (j0 + 4 * u < m) soft_push(sf, lgs[u], vs[u]);
  }
  s_part[g][tid & 63] = sf;
  __syncthreads();
  if (g != 0) return;
  Soft acc = s_part[0][tid];
#pragma unroll
  for (int v = 1; v < 4; ++v) acc = soft_merge(acc, s_part[v][tid]);
  const size_t erow = page_row(a.pg, b, a.first + i, a.E_cap);
  st(reinterpret_cast<TO*>(a.out), erow * c + r, acc.acc / acc.l);
}

hipError_t launch_compress(const CompressArgs& a, hipStream_t s) {
  if (!a.seq_pos0 && !a.score_w && !a.cb && !a.nr.on && a.m >= 32 && a.c % kSliceC == 0 &&
      (a.out_dtype == F32 || a.out_dtype == BF16)) {
    dim3 grid(a.T / a.m, a.B, a.c / kSliceC), block(256);
    if (a.dtype == F32 && a.out_dtype == F32)
      CSA_LAUNCH("compress_chunk", (compress_slices_kernel<float, float>), grid, block, 0, s, a);
    else if (a.dtype == F32)
      CSA_LAUNCH("compress_chunk", (compress_slices_kernel<float, bf16>), grid, block, 0, s, a);
    else if (a.out_dtype == F32)
      CSA_LAUNCH("compress_chunk", (compress_slices_kernel<bf16, float>), grid, block, 0, s, a);
    else
      CSA_LAUNCH("compress_chunk", (compress_slices_kernel<bf16, bf16>), grid, block, 0, s, a);
    return hipGetLastError();
  }
  // (variable-length chunks: a chunk of T tokens ends at most ceil(T/m) blocks)
  dim3 grid(a.seq_pos0 ? (a.T + a.m - 1) / a.m : a.T / a.m, a.B), block(256);
  if (a.dtype == F32)
    launch_compress_to<float>(a, grid, block, s);
  else
    launch_compress_to<bf16>(a, grid, block, s);
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
  const size_t erow = fold ? page_row(a.pg, b, e, a.E_cap) : 0;  // the new entry's cache row
  const int nstr = a.overlap ? 4 : 2;
  const int slot = (int)(t % R);
  const bool has_idx = a.idx_dtype >= 0;
  // whole: the entry's epilogue needs all of it (norm_rope: RMSNorm and the
  // rotary pairs; the 576-byte entry: the scale of its e4m3 part).  The
  // coordinate slices are folded in parallel as always and parked in
  // fold_buf; the last workgroup of the sequence finishes and stores the
  // entry.
  const bool whole = a.nr.on || a.kv_fmt;
  const int main_jobs = c / kFoldCW;
  __shared__ int s_last;

  if (whole && job < main_jobs) {
    const int r0 = job * kFoldCW;
    T* tail = reinterpret_cast<T*>(a.tail) + (size_t)b * nstr * R * c;
    const T* io = reinterpret_cast<const T*>(a.streams) + (size_t)b * nstr * c;
    // the new token's appends first (the fold never reads its slot), so
    // their loads overlap the fold's
    for (int i = tid; i < nstr * kFoldCW; i += kFoldT) {
      const int sc = i / kFoldCW, r = r0 + i % kFoldCW;
      tail[((size_t)sc * R + slot) * c + r] = io[(size_t)sc * c + r];
    }
    if (fold) {
      const float val = fold_job<T>(tail, io, c, r0, kFoldCW, m, R, t, e, a.overlap && e > 0, a.bias_a,
                                    a.bias_b, s_part);
      // (device-coherent stores: the last workgroup reads them)
      if (tid < kFoldCW)
        __hip_atomic_store(a.fold_buf + (size_t)b * c + r0 + tid, val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // the new window row (prepared at t with norm_rope: one wavefront, the
    // whole row)
    T* ring = reinterpret_cast<T*>(a.win_ring) + ((size_t)b * a.n_win + (size_t)(t % a.n_win)) * c;
    const T* xn = reinterpret_cast<const T*>(a.x_new) + (size_t)b * c;
    if (a.nr.on) {
      if (job == 0 && tid < 64) prep_row_wave(xn, ring, c, a.nr, a.nr.g_kv, t);
    } else if (tid < kFoldCW) {
      ring[r0 + tid] = xn[r0 + tid];
    }
  } else if (job >= main_jobs + (has_idx ? 1 : 0)) {
    // the step's queries, prepared at t: one head per wavefront
    const int h = 4 * (job - main_jobs - (has_idx ? 1 : 0)) + (tid >> 6);
    if (h < a.H)
      prep_row_wave(reinterpret_cast<const T*>(a.q) + ((size_t)b * a.H + h) * c,
                    reinterpret_cast<T*>(a.q_prep) + ((size_t)b * a.H + h) * c, c, a.nr, a.nr.g_q, t);
  } else if (job < main_jobs) {
    const int r0 = job * kFoldCW;
    T* tail = reinterpret_cast<T*>(a.tail) + (size_t)b * nstr * R * c;
    const T* io = reinterpret_cast<const T*>(a.streams) + (size_t)b * nstr * c;
    if (fold) {
      const float val = fold_job<T>(tail, io, c, r0, kFoldCW, m, R, t, e, a.overlap && e > 0, a.bias_a,
                                    a.bias_b, s_part);
      if (tid < kFoldCW) st(reinterpret_cast<T*>(a.kv_cache), erow * c + r0 + tid, val);
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
      const size_t row = erow;
      if constexpr (std::is_same<TI, mx4>::value) {
        // MXFP4 (d a multiple of 32, every lane takes part in the block maxima)
        uint32_t sc;
        const uint32_t code = mx_quantize_lane(tid < d ? iv : 0.f, &sc);
        const uint32_t odd = __shfl_xor(code, 1, 64);
        if (tid < d && (tid & 1) == 0)
          reinterpret_cast<uint8_t*>(a.idx_cache)[row * (d / 2) + tid / 2] = (uint8_t)(code | (odd << 4));
        if (tid < d && (tid & 31) == 0) reinterpret_cast<uint8_t*>(a.idx_scale)[row * (d / 32) + tid / 32] = (uint8_t)sc;
      } else if constexpr (sizeof(TI) == 1) {
        float am = wave_max(tid < d ? fabsf(iv) : 0.f);
        if ((tid & 63) == 0) s_red[tid >> 6] = am;
        __syncthreads();
        am = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
        float scale = am / 448.0f;
        if (!(scale > 0.f)) scale = 1.f;
        if (tid < d) reinterpret_cast<uint8_t*>(a.idx_cache)[row * d + tid] = f32_to_e4m3(iv / scale);
        if (tid == 0) reinterpret_cast<float*>(a.idx_scale)[row] = scale;
      } else {
        if (tid < d) st(reinterpret_cast<TI*>(a.idx_cache), row * d + tid, iv);
      }
    }
    for (int i = tid; i < 4 * d; i += kFoldT) {
      const int sc = i / d, r = i % d;
      itail[((size_t)sc * R + slot) * d + r] = iio[(size_t)sc * d + r];
    }
  }
  // the last workgroup of the sequence finishes a whole entry and publishes
  // the count; every workgroup's read of n_entries[b], and its fold_buf
  // stores, completed before its increment
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) s_last = atomicAdd(&a.counters[b], 1) == (int)gridDim.x - 1;
  __syncthreads();
  if (!s_last) return;
  if (whole && fold) {
    const int nu = (c + 255) / 256;  // the same trip count in every lane
    float val[2] = {0.f, 0.f};
    for (int u = 0; u < nu; ++u)
      if (256 * u + tid < c)
        val[u] = __hip_atomic_load(a.fold_buf + (size_t)b * c + 256 * u + tid, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
    if (a.nr.on) {
      // RMSNorm over the c coordinates, then the rotary pairs (neighbouring
      // lanes) at the entry's position m e
      float ss = 0.f;
      for (int u = 0; u < nu; ++u)
        if (256 * u + tid < c) ss += val[u] * val[u];
      ss = wave_sum(ss);
      if ((tid & 63) == 0) s_red[tid >> 6] = ss;
      __syncthreads();
      ss = s_red[0] + s_red[1] + s_red[2] + s_red[3];
      const float inv = 1.0f / sqrtf(ss / (float)c + a.nr.eps);
      const int Rd = a.nr.rope_dims;
      for (int u = 0; u < nu; ++u) {
        const int r = 256 * u + tid;
        float v = r < c ? val[u] * inv * a.nr.g_kv[r] : 0.f;
        const float other = __shfl_xor(v, 1, 64);
        if (r < c && r >= c - Rd) {
          float cs, sn;
          rope_cs((int64_t)m * e, a.nr.inv_freq[(r - (c - Rd)) >> 1], &cs, &sn);
          v = (r & 1) ? (other * sn + v * cs) : (v * cs - other * sn);
        }
        val[u] = v;
      }
    }
    store_entry<T>(val, nu, c, a.kv_fmt, a.kv_cache, a.kv_scale, erow, s_red);
  }
  if (tid == 0) {
    a.counters[b] = 0;
    if (fold) a.n_entries[b] = n_have + 1;
  }
}

template <typename T>
static void launch_fold_to(const FoldArgs& a, dim3 grid, dim3 block, hipStream_t s) {
  if (a.idx_dtype == E4M3)
    CSA_LAUNCH("fold_append", (fold_append_kernel<T, uint8_t>), grid, block, 0, s, a);
  else if (a.idx_dtype == MXFP4)
    CSA_LAUNCH("fold_append", (fold_append_kernel<T, mx4>), grid, block, 0, s, a);
  else if (a.idx_dtype == F32)
    CSA_LAUNCH("fold_append", (fold_append_kernel<T, float>), grid, block, 0, s, a);
  else  // BF16, or no indexer
    CSA_LAUNCH("fold_append", (fold_append_kernel<T, bf16>), grid, block, 0, s, a);
}

hipError_t launch_fold_append(const FoldArgs& a, hipStream_t s) {
  // main-entry jobs (64 coordinates each), the indexer-key job, the query
  // jobs (norm_rope, four heads each)
  const int jobs = a.c / kFoldCW + (a.idx_dtype >= 0 ? 1 : 0) + (a.nr.on ? (a.H + 3) / 4 : 0);
  dim3 grid(jobs, a.B), block(kFoldT);
  if (a.dtype == F32)
    launch_fold_to<float>(a, grid, block, s);
  else
    launch_fold_to<bf16>(a, grid, block, s);
  return hipGetLastError();
}

// --------------------------------------------------------------------------
// norm_rope prefill: the chunk's queries and window rows prepared for the
// core attention (RMSNorm, then the rotary pairs at their positions), one
// wavefront per row.  grid (rows / 4), 256 threads.
// --------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void prep_rows_kernel(PrepArgs a) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t nq = (int64_t)a.B * a.T * a.H;
  const int W = a.n_win - 1 + a.T;
  const int64_t nw = (int64_t)a.B * W;
  const int c = a.c;
  if (row < nq) {
    const int tq = (int)((row / a.H) % a.T);
    const int64_t p0 = a.seq_pos0 ? a.seq_pos0[row / ((int64_t)a.H * a.T)] : a.pos0;
    prep_row_wave(cptr<T>(a.q) + row * c, reinterpret_cast<T*>(a.q_prep) + row * c, c, a.nr, a.nr.g_q, p0 + tq);
  } else if (row < nq + nw) {
    const int64_t r = row - nq;
    const int j = (int)(r % W);
    const int64_t p0 = a.seq_pos0 ? a.seq_pos0[r / W] : a.pos0;
    prep_row_wave(cptr<T>(a.win) + r * c, reinterpret_cast<T*>(a.win_prep) + r * c, c, a.nr, a.nr.g_kv,
                  p0 - (a.n_win - 1) + j);
  }
}

hipError_t launch_prep_rows(const PrepArgs& a, hipStream_t s) {
  const int64_t rows = (int64_t)a.B * a.T * a.H + (int64_t)a.B * (a.n_win - 1 + a.T);
  dim3 grid((unsigned)((rows + 3) / 4)), block(256);
  if (a.dtype == F32)
    CSA_LAUNCH("prep_rows", prep_rows_kernel<float>, grid, block, 0, s, a);
  else
    CSA_LAUNCH("prep_rows", prep_rows_kernel<bf16>, grid, block, 0, s, a);
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
  // the sequence's chunk: positions pos0 .. pos0 + len - 1 (variable-length
  // chunks: its own start and length; rows of the grid past its count exit)
  int64_t pos0 = a.pos0;
  int len = a.T;
  if (a.seq_pos0) {
    pos0 = a.seq_pos0[b] < 0 ? 0 : a.seq_pos0[b];
    len = a.seq_len[b] < 0 ? 0 : (a.seq_len[b] > a.T ? a.T : a.seq_len[b]);
  }
  const int gw = a.n_win < (a.n_win - 1 + a.T) ? a.n_win : (a.n_win - 1 + a.T);  // grid rows of each part
  const int gt = a.R < a.T ? a.R : a.T;
  const int n_w = len == 0 ? 0 : (a.n_win < (a.n_win - 1 + len) ? a.n_win : (a.n_win - 1 + len));
  const int n_t = a.R < len ? a.R : len;
  if (row < gw) {
    if (row >= n_w) return;
    // window row of position p = pos0 + len - n_w + row (none before the
    // sequence's start)
    const int64_t p = pos0 + len - n_w + row;
    if (p < 0) return;
    const int64_t src_row = p - (pos0 - (a.n_win - 1));
    const T* src = cptr<T>(a.win) + ((size_t)b * (a.n_win - 1 + a.T) + src_row) * a.c;
    T* dst = reinterpret_cast<T*>(a.win_ring) + ((size_t)b * a.n_win + (size_t)(p % a.n_win)) * a.c;
    for (int r = tid; r < a.c; r += 256) dst[r] = src[r];
  } else if (row < gw + gt) {
    const int j = row - gw;
    if (j >= n_t) return;
    const int64_t p = pos0 + len - n_t + j;
    const int64_t tok = p - pos0;
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
  } else if (row == gw + gt && tid == 0 && a.new_entries) {
    a.n_entries[b] += a.new_entries;
  }
}

// variable-length prefill set-up: one thread per (sequence, row)
__global__ __launch_bounds__(256) void varlen_setup_kernel(VarlenArgs a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)a.B * a.T) return;
  const int b = (int)(i / a.T), tq = (int)(i % a.T);
  int64_t p0 = a.seq_pos0[b];
  p0 = p0 < 0 ? 0 : p0;
  int len = a.seq_len[b];
  len = len < 0 ? 0 : (len > a.T ? a.T : len);
  // padding rows ask as the last token (or the chunk's start when empty)
  a.q_pos[i] = p0 + (tq < len ? tq : (len > 0 ? len - 1 : 0));
  if (tq == 0) {
    a.win_pos0[b] = p0 - (a.n_win - 1);
    int64_t n = (p0 + len) / a.m;
    a.n_entries[b] = (int32_t)(n < a.E_cap ? n : a.E_cap);
  }
}

hipError_t launch_varlen_setup(const VarlenArgs& a, hipStream_t s) {
  const int64_t n = (int64_t)a.B * a.T;
  CSA_LAUNCH("varlen_setup", varlen_setup_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
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
