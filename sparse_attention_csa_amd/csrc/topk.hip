// Exact per-query top-k over index scores (row a3): the k largest scores of
// the visible entries, ties to the lower entry id, ids emitted in ascending
// order, -1 padded ("2026 DeepSeek-V4" note, "Key design 1": C_t =
// TopK_k(I_t,:); "DeepSeek-V4" book ch. 6: all entries kept when fewer than k
// are visible).
//
// Scores are compared as order-preserving 32-bit keys.  Selection runs in two
// stages:
//  1. coarse: a histogram of the top 11 key bits locates the bin b1 holding
//     the k-th largest key; every entry in a higher bin is selected and is
//     marked in a per-row bitmap; entries in bin b1 are candidates.
//  2. exact: one workgroup resolves the candidates by radix select on the
//     remaining 21 key bits (and, among equal keys, on the entry id), marks
//     the winners, and emits the marked ids in order from the bitmap while
//     clearing it.
// Split mode (few long rows, decode): the histogram is accumulated by the
// scoring kernel, many workgroups scan slices of a row, and the last one to
// finish resolves the row.  Row mode (many rows, prefill): one workgroup per
// row does everything.  Counters, histograms and bitmaps are returned to zero
// by the workgroup that finishes a row.

#include "common.h"
#include "kernels.h"
#include "topk.h"

namespace csa {

namespace {

constexpr int kT = 256;  // threads per workgroup

CSA_DEV uint32_t bin_of(uint32_t key) { return key >> kTopkShift; }

// Locate the bin holding the k-th largest key.  hist: kTopkBins counters.
// Returns b1 and `above` = number of keys in bins > b1 (< k).  kT threads.
CSA_DEV void find_bin(const int* hist, int k, int* s_red, int* b1_out, int* above_out) {
  // each thread owns 8 consecutive bins, counted from the top
  const int tid = threadIdx.x;
  const int hi = kTopkBins - 1 - 8 * tid;  // bins hi, hi-1, ..., hi-7
  int c[8], tot = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    c[i] = hist[hi - i];
    tot += c[i];
  }
  // exclusive prefix over threads (bins above this thread's range)
  s_red[tid] = tot;
  __syncthreads();
  for (int off = 1; off < kT; off <<= 1) {
    const int v = tid >= off ? s_red[tid - off] : 0;
    __syncthreads();
    s_red[tid] += v;
    __syncthreads();
  }
  int before = s_red[tid] - tot;
  __syncthreads();
  if (before < k && before + tot >= k) {
    int acc = before;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (acc + c[i] >= k) {
        s_red[0] = hi - i;
        s_red[1] = acc;
        break;
      }
      acc += c[i];
    }
  }
  __syncthreads();
  *b1_out = s_red[0];
  *above_out = s_red[1];
  __syncthreads();
}

// Radix select among n (key, id) pairs in LDS: the `want` largest by key with
// ties to the lower id.  Marks winners in the row bitmap.  kT threads.
CSA_DEV void select_candidates(const uint32_t* ckey, const int* cid, int n, int want,
                               uint32_t* bitmap, int* s_hist, int* s_misc) {
  const int tid = threadIdx.x;
  // refine the key on bits 20..0 (bin bits already equal): passes of 7 bits
  uint32_t prefix = ckey[0] >> kTopkShift;  // all candidates share the bin
  int rem = want;
  int shift = kTopkShift;
  for (int pass = 0; pass < 3; ++pass) {
    shift -= 7;
    if (tid < 128) s_hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kT) {
      const uint32_t key = ckey[i];
      if ((key >> (shift + 7)) == prefix) atomicAdd(&s_hist[(key >> shift) & 127], 1);
    }
    __syncthreads();
    if (tid == 0) {
      int acc = 0, d = 0;
      for (d = 127; d >= 0; --d) {
        if (acc + s_hist[d] >= rem) break;
        acc += s_hist[d];
      }
      s_misc[0] = d;
      s_misc[1] = rem - acc;
    }
    __syncthreads();
    prefix = (prefix << 7) | (uint32_t)s_misc[0];
    rem = s_misc[1];
    __syncthreads();
  }
  const uint32_t tau = prefix;  // exact key of the last winner; `rem` ties at tau win
  // count ties; if more than rem, pick the rem lowest ids by radix on the id
  if (tid == 0) s_misc[2] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += kT)
    if (ckey[i] == tau) atomicAdd(&s_misc[2], 1);
  __syncthreads();
  const int n_tie = s_misc[2];
  int id_lim = 0x7fffffff;  // ties with id <= id_lim win
  if (n_tie > rem) {
    // rem smallest ids among the ties: 3 passes of 10 bits over a 30-bit id
    uint32_t ipref = 0;
    int r2 = rem;
    for (int pass = 0; pass < 3; ++pass) {
      const int sh = 20 - 10 * pass;
      for (int i = tid; i < 1024; i += kT) s_hist[i] = 0;
      __syncthreads();
      for (int i = tid; i < n; i += kT) {
        const uint32_t id = (uint32_t)cid[i];
        if (ckey[i] == tau && (pass == 0 || (id >> (sh + 10)) == ipref)) atomicAdd(&s_hist[(id >> sh) & 1023], 1);
      }
      __syncthreads();
      if (tid == 0) {
        int acc = 0, d = 0;
        for (d = 0; d < 1024; ++d) {
          if (acc + s_hist[d] >= r2) break;
          acc += s_hist[d];
        }
        s_misc[0] = d;
        s_misc[1] = r2 - acc;
      }
      __syncthreads();
      ipref = (ipref << 10) | (uint32_t)s_misc[0];
      r2 = s_misc[1];
      __syncthreads();
    }
    id_lim = (int)ipref;  // ids are distinct, so exactly rem ties have id <= ipref
  }
  for (int i = tid; i < n; i += kT) {
    const uint32_t key = ckey[i];
    if (key > tau || (key == tau && cid[i] <= id_lim)) atomicOr(&bitmap[cid[i] >> 5], 1u << (cid[i] & 31));
  }
  __syncthreads();
}

// Emit the ids marked in the bitmap in ascending order, clear the bitmap,
// pad with -1 to k.  kT threads; each thread owns 32-word groups in order.
CSA_DEV void emit_bitmap(uint32_t* bitmap, int nwords, int32_t* out, int k, int32_t* cnt_out,
                         int* s_red) {
  const int tid = threadIdx.x;
  int base = 0;
  for (int w0 = 0; w0 < nwords; w0 += kT * 4) {
    // thread owns words w0 + 4 tid .. +3
    uint32_t v[4];
    int c = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int wi = w0 + 4 * tid + i;
      v[i] = wi < nwords ? bitmap[wi] : 0u;
      c += __popc(v[i]);
    }
    s_red[tid] = c;
    __syncthreads();
    for (int off = 1; off < kT; off <<= 1) {
      const int x = tid >= off ? s_red[tid - off] : 0;
      __syncthreads();
      s_red[tid] += x;
      __syncthreads();
    }
    int pos = base + s_red[tid] - c;
    const int total = s_red[kT - 1];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int wi = w0 + 4 * tid + i;
      uint32_t bits = v[i];
      while (bits) {
        const int bpos = __ffs(bits) - 1;
        bits &= bits - 1;
        if (pos < k) out[pos] = wi * 32 + bpos;
        ++pos;
      }
      if (wi < nwords && v[i]) bitmap[wi] = 0u;
    }
    base += total;
  }
  for (int i = base + tid; i < k; i += kT) out[i] = -1;
  if (tid == 0) *cnt_out = base < k ? base : k;
}

CSA_DEV int64_t visible(const IndexArgs& a, int b, int64_t t) {
  const int64_t lim = vis_limit(t, a.m, a.vis);
  const int64_t have = (int64_t)a.n_entries[b] + a.n_add;
  int64_t n = lim < have ? lim : have;
  if (n > a.E_cap) n = a.E_cap;
  return n < 0 ? 0 : n;
}

}  // namespace

// ---------------------------------------------------------------------------
// split mode: grid (n_slices, rows), kT threads.  hist filled by the scorer.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kT) void topk_collect_kernel(IndexArgs a, TopkWs ws, int slice_len) {
  __shared__ int s_red[kT];
  __shared__ int s_flag;
  const int row = blockIdx.y, b = row / a.Tq, tq = row % a.Tq, tid = threadIdx.x;
  const int64_t t = a.q_pos ? a.q_pos[(size_t)b * a.Tq + tq] : a.q_pos0 + tq;
  const int nv = (int)visible(a, b, t);
  const int k = a.k;
  int* hist = ws.hist + (size_t)row * kTopkBins;
  int* ctr = ws.ctr + (size_t)row * 4;
  uint32_t* bitmap = ws.bitmap + (size_t)row * ws.bitmap_words;
  uint2* cand = ws.cand + (size_t)row * kTopkCandCap;
  const float* sc = a.scores + (size_t)row * a.E_cap;

  int b1 = -1, above = 0;
  if (nv > k) find_bin(hist, k, s_red, &b1, &above);
  const int s0 = blockIdx.x * slice_len;
  const int s1 = min(nv, s0 + slice_len);
  if (nv > k) {
    for (int s = s0 + tid; s < s1; s += kT) {
      const uint32_t key = f32_key(sc[s]);
      const int bin = (int)bin_of(key);
      if (bin > b1) {
        atomicOr(&bitmap[s >> 5], 1u << (s & 31));
      } else if (bin == b1) {
        const int slot = atomicAdd(&ctr[0], 1);
        if (slot < kTopkCandCap) cand[slot] = make_uint2(key, (uint32_t)s);
      }
    }
  }
  // last workgroup of the row resolves it
  __threadfence();
  __syncthreads();
  if (tid == 0) s_flag = (atomicAdd(&ctr[1], 1) == (int)gridDim.x - 1);
  __syncthreads();
  if (!s_flag) return;
  __threadfence();
  int32_t* out = a.topk_idx + (size_t)row * k;
  if (nv <= k) {
    for (int i = tid; i < k; i += kT) out[i] = i < nv ? i : -1;
    if (tid == 0) a.topk_cnt[row] = nv;
  } else {
    extern __shared__ unsigned char dyn[];
    uint32_t* ckey = reinterpret_cast<uint32_t*>(dyn);
    int* cid = reinterpret_cast<int*>(ckey + kTopkCandCap);
    int* s_hist = cid + kTopkCandCap;  // 1024
    int* s_misc = s_hist + 1024;       // 4
    const int n_cand = atomicAdd(&ctr[0], 0);
    if (n_cand <= kTopkCandCap) {
      for (int i = tid; i < n_cand; i += kT) {
        const uint2 v = cand[i];
        ckey[i] = v.x;
        cid[i] = (int)v.y;
      }
      __syncthreads();
      select_candidates(ckey, cid, n_cand, k - above, bitmap, s_hist, s_misc);
    } else {
      // too many keys share the threshold bin: resolve from the row itself,
      // scanning it in chunks of kTopkCandCap candidates in id order
      topk_resolve_from_row(sc, nv, b1, k - above, bitmap, ckey, cid, s_hist, s_misc);
    }
    __threadfence();
    __syncthreads();
    emit_bitmap(bitmap, (nv + 31) >> 5, out, k, &a.topk_cnt[row], s_red);
  }
  // reset the row's scratch for the next call
  for (int i = tid; i < kTopkBins; i += kT) hist[i] = 0;
  if (tid == 0) {
    ctr[0] = 0;
    ctr[1] = 0;
  }
}

// ---------------------------------------------------------------------------
// row mode: grid (rows), one workgroup per row, scores already written.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kT) void topk_rowsel_kernel(IndexArgs a, TopkWs ws) {
  extern __shared__ unsigned char dyn[];
  uint32_t* ckey = reinterpret_cast<uint32_t*>(dyn);
  int* cid = reinterpret_cast<int*>(ckey + kTopkCandCap);
  int* s_hist = cid + kTopkCandCap;  // max(1024, kTopkBins) ints
  int* s_misc = s_hist + kTopkBins;  // 4
  int* s_red = s_misc + 4;           // kT
  const int row = blockIdx.x, b = row / a.Tq, tq = row % a.Tq, tid = threadIdx.x;
  const int64_t t = a.q_pos ? a.q_pos[(size_t)b * a.Tq + tq] : a.q_pos0 + tq;
  const int nv = (int)visible(a, b, t);
  const int k = a.k;
  uint32_t* bitmap = ws.bitmap + (size_t)row * ws.bitmap_words;
  const float* sc = a.scores + (size_t)row * a.E_cap;
  int32_t* out = a.topk_idx + (size_t)row * k;
  if (nv <= k) {
    for (int i = tid; i < k; i += kT) out[i] = i < nv ? i : -1;
    if (tid == 0) a.topk_cnt[row] = nv;
    return;
  }
  for (int i = tid; i < kTopkBins; i += kT) s_hist[i] = 0;
  __syncthreads();
  for (int s = tid; s < nv; s += kT) atomicAdd(&s_hist[bin_of(f32_key(sc[s]))], 1);
  __syncthreads();
  int b1, above;
  find_bin(s_hist, k, s_red, &b1, &above);
  if (tid == 0) s_misc[3] = 0;
  __syncthreads();
  for (int s = tid; s < nv; s += kT) {
    const uint32_t key = f32_key(sc[s]);
    const int bin = (int)bin_of(key);
    if (bin > b1) {
      atomicOr(&bitmap[s >> 5], 1u << (s & 31));
    } else if (bin == b1) {
      const int slot = atomicAdd(&s_misc[3], 1);
      if (slot < kTopkCandCap) {
        ckey[slot] = key;
        cid[slot] = s;
      }
    }
  }
  __syncthreads();
  const int n_cand = s_misc[3];
  __syncthreads();
  if (n_cand <= kTopkCandCap)
    select_candidates(ckey, cid, n_cand, k - above, bitmap, s_hist, s_misc);
  else
    topk_resolve_from_row(sc, nv, b1, k - above, bitmap, ckey, cid, s_hist, s_misc);
  __threadfence();
  __syncthreads();
  emit_bitmap(bitmap, (nv + 31) >> 5, out, k, &a.topk_cnt[row], s_red);
}

// Exact resolution when the threshold bin holds more than kTopkCandCap keys:
// radix refine over the row on bits 20..0 restricted to bin b1 (3 passes),
// then one in-order pass marks keys above the threshold and the lowest-id
// ties (the row is scanned in id order, chunk by chunk).
__device__ void topk_resolve_from_row(const float* sc, int nv, int b1, int want, uint32_t* bitmap,
                                      uint32_t* s_flag_key, int* s_scan, int* s_hist, int* s_misc) {
  const int tid = threadIdx.x;
  uint32_t prefix = (uint32_t)b1;
  int rem = want;
  int shift = kTopkShift;
  for (int pass = 0; pass < 3; ++pass) {
    shift -= 7;
    if (tid < 128) s_hist[tid] = 0;
    __syncthreads();
    for (int s = tid; s < nv; s += kT) {
      const uint32_t key = f32_key(sc[s]);
      if ((key >> (shift + 7)) == prefix) atomicAdd(&s_hist[(key >> shift) & 127], 1);
    }
    __syncthreads();
    if (tid == 0) {
      int acc = 0, d = 0;
      for (d = 127; d >= 0; --d) {
        if (acc + s_hist[d] >= rem) break;
        acc += s_hist[d];
      }
      s_misc[0] = d;
      s_misc[1] = rem - acc;
    }
    __syncthreads();
    prefix = (prefix << 7) | (uint32_t)s_misc[0];
    rem = s_misc[1];
    __syncthreads();
  }
  const uint32_t tau = prefix;
  // in-order pass: ties taken while fewer than rem have been taken
  int taken = 0;
  for (int base = 0; base < nv; base += kT) {
    const int s = base + tid;
    const uint32_t key = s < nv ? f32_key(sc[s]) : 0u;
    const bool bin_ok = s < nv && (int)(key >> kTopkShift) == b1;
    const bool eq = bin_ok && key == tau;
    s_scan[tid] = eq ? 1 : 0;
    __syncthreads();
    for (int off = 1; off < kT; off <<= 1) {
      const int x = tid >= off ? s_scan[tid - off] : 0;
      __syncthreads();
      s_scan[tid] += x;
      __syncthreads();
    }
    const int rank = taken + s_scan[tid] - (eq ? 1 : 0);
    const int tot = s_scan[kT - 1];
    __syncthreads();
    if (bin_ok && (key > tau || (eq && rank < rem))) atomicOr(&bitmap[s >> 5], 1u << (s & 31));
    taken += tot;
  }
  (void)s_flag_key;
  __syncthreads();
}

size_t topk_ws_bytes(int rows, int E_cap, bool with_cand) {
  const size_t words = ((size_t)E_cap + 31) / 32;
  return (size_t)rows * (kTopkBins * 4 + 16 + words * 4 + (with_cand ? (size_t)kTopkCandCap * 8 : 0)) + 1024;
}

TopkWs topk_ws_carve(void* base, int rows, int E_cap, bool with_cand) {
  TopkWs w;
  char* p = reinterpret_cast<char*>(base);
  w.bitmap_words = (int)(((size_t)E_cap + 31) / 32);
  w.hist = reinterpret_cast<int*>(p);
  p += (size_t)rows * kTopkBins * 4;
  w.ctr = reinterpret_cast<int*>(p);
  p += (size_t)rows * 16;
  w.bitmap = reinterpret_cast<uint32_t*>(p);
  p += (size_t)rows * w.bitmap_words * 4;
  p = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(p) + 15) & ~uintptr_t(15));
  w.cand = with_cand ? reinterpret_cast<uint2*>(p) : nullptr;
  return w;
}

size_t topk_lds_bytes() { return (size_t)kTopkCandCap * 8 + (kTopkBins + 4 + kT) * 4; }

hipError_t launch_topk_collect(const IndexArgs& a, const TopkWs& ws, int slices, int slice_len,
                               hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&topk_collect_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)topk_lds_bytes());
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  CSA_LAUNCH("topk_collect", topk_collect_kernel, dim3(slices, a.B * a.Tq), dim3(kT), topk_lds_bytes(), s,
             a, ws, slice_len);
  return hipGetLastError();
}

hipError_t launch_topk_rows(const IndexArgs& a, const TopkWs& ws, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&topk_rowsel_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)topk_lds_bytes());
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  CSA_LAUNCH("topk_rows", topk_rowsel_kernel, dim3(a.B * a.Tq), dim3(kT), topk_lds_bytes(), s, a, ws);
  return hipGetLastError();
}

}  // namespace csa
