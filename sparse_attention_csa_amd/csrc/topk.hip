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
//     marked in a two-level per-row bitmap; entries in bin b1 are candidates.
//  2. exact: one workgroup resolves the candidates by radix select on the
//     remaining 21 key bits (and, among equal keys, on the entry id), marks
//     the winners in an LDS copy of the bitmap, and emits the marked ids in
//     order.  The summary level (one bit per nonzero bitmap word) lets the
//     emitter touch only nonzero words in a single prefix pass.
// Split mode (few long rows, decode): the histogram is accumulated by the
// scoring kernel, many workgroups scan slices of a row (candidate slots are
// reserved with one atomic per workgroup), then a second kernel resolves each
// row with one workgroup.  No workgroup waits on another.  Row mode (many rows, prefill): one workgroup per row does
// everything.  Counters, histograms and bitmaps are returned to zero by the
// workgroup that finishes a row.

#include "common.h"
#include "kernels.h"
#include "topk.h"

namespace csa {

namespace {

constexpr int kT = 256;  // threads per workgroup
constexpr int kW = kT / 64;
constexpr int kCollectPer = 16;  // keys per thread in a collect slice
static_assert(kCollectPer * kT == kTopkCollectSlice, "collect slice");

CSA_DEV uint32_t bin_of(uint32_t key) { return key >> kTopkShift; }

CSA_DEV int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int x = __shfl_up(v, o, 64);
    if (lane >= o) v += x;
  }
  return v;
}

// exclusive prefix of v over the workgroup in thread order; *total = sum.
// s_w: kW ints of scratch.  Contains two barriers.
CSA_DEV int block_excl_scan(int v, int* s_w, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int inc = wave_incl_scan(v);
  if (lane == 63) s_w[wave] = inc;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kW; ++w) {
    const int c = s_w[w];
    if (w < wave) off += c;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return off + inc - v;
}

// In a histogram of nb bins (nb = 64 * per), find the bin where the count,
// accumulated from the top (descending) or the bottom, first reaches `want`.
// Executed by wave 0 only; returns (bin, count before it) in s_out[0..1].
template <int PER, bool DESC>
CSA_DEV void wave_find(const int* hist, int want, int* s_out) {
  const int lane = threadIdx.x & 63;
  int c[PER], tot = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int bin = DESC ? (64 * PER - 1 - (PER * lane + i)) : (PER * lane + i);
    c[i] = hist[bin];
    tot += c[i];
  }
  const int inc = wave_incl_scan(tot);
  const int before = inc - tot;
  if (before < want && inc >= want) {
    int acc = before;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (acc + c[i] >= want) {
        s_out[0] = DESC ? (64 * PER - 1 - (PER * lane + i)) : (PER * lane + i);
        s_out[1] = acc;
        break;
      }
      acc += c[i];
    }
  }
}

// mark an id in a two-level bitmap (global or LDS); results are not awaited
CSA_DEV void mark(uint32_t* bitmap, uint32_t* summary, int id) {
  atomicOr(&bitmap[id >> 5], 1u << (id & 31));
  atomicOr(&summary[id >> 10], 1u << ((id >> 5) & 31));
}

// Radix select among n (key, id) pairs in LDS (all in one top-11-bit bin):
// the `want` largest keys, ties to the lower id; winners are marked.
CSA_DEV void select_candidates(const uint32_t* ckey, const int* cid, int n, int want,
                               uint32_t* bitmap, uint32_t* summary, int* s_hist, int* s_misc) {
  const int tid = threadIdx.x;
  uint32_t prefix = ckey[0] >> kTopkShift;
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
    if (tid < 64) wave_find<2, true>(s_hist, rem, s_misc);
    __syncthreads();
    prefix = (prefix << 7) | (uint32_t)s_misc[0];
    rem -= s_misc[1];
    __syncthreads();
  }
  const uint32_t tau = prefix;  // key of the last winner; `rem` keys equal to tau win
  int nt = 0;
  for (int i = tid; i < n; i += kT) nt += ckey[i] == tau;
  int n_tie;
  block_excl_scan(nt, s_misc + 4, &n_tie);
  int id_lim = 0x7fffffff;  // ties with id <= id_lim win
  if (n_tie > rem) {
    // the rem lowest ids among the ties: 3 passes of 10 bits over a 30-bit id
    uint32_t ipref = 0;
    for (int pass = 0; pass < 3; ++pass) {
      const int sh = 20 - 10 * pass;
      for (int i = tid; i < 1024; i += kT) s_hist[i] = 0;
      __syncthreads();
      for (int i = tid; i < n; i += kT) {
        const uint32_t id = (uint32_t)cid[i];
        if (ckey[i] == tau && (pass == 0 || (id >> (sh + 10)) == ipref))
          atomicAdd(&s_hist[(id >> sh) & 1023], 1);
      }
      __syncthreads();
      if (tid < 64) wave_find<16, false>(s_hist, rem, s_misc);
      __syncthreads();
      ipref = (ipref << 10) | (uint32_t)s_misc[0];
      rem -= s_misc[1];
      __syncthreads();
    }
    id_lim = (int)ipref;  // ids are distinct: exactly the wanted ties have id <= ipref
  }
  for (int i = tid; i < n; i += kT) {
    const uint32_t key = ckey[i];
    if (key > tau || (key == tau && cid[i] <= id_lim)) mark(bitmap, summary, cid[i]);
  }
}

// Emit the marked ids in ascending order, clear both bitmap levels, pad with
// -1 to k.  Thread i owns summary words i, i + kT, ... in order.
CSA_DEV void emit_bitmap(uint32_t* bitmap, uint32_t* summary, int nwords, int32_t* out, int k,
                         int32_t* cnt_out, int* s_w) {
  const int tid = threadIdx.x;
  const int nsum = (nwords + 31) >> 5;
  int base = 0;
  for (int s0 = 0; s0 < nsum; s0 += kT) {
    const int si = s0 + tid;
    const uint32_t sw = si < nsum ? summary[si] : 0u;
    int c = 0;
    uint32_t bits = sw;
    while (bits) {
      const int j = __ffs(bits) - 1;
      bits &= bits - 1;
      c += __popc(bitmap[32 * si + j]);
    }
    int total;
    int pos = base + block_excl_scan(c, s_w, &total);
    bits = sw;
    while (bits) {
      const int j = __ffs(bits) - 1;
      bits &= bits - 1;
      const int wi = 32 * si + j;
      uint32_t v = bitmap[wi];
      bitmap[wi] = 0u;
      while (v) {
        const int b = __ffs(v) - 1;
        v &= v - 1;
        if (pos < k) out[pos] = wi * 32 + b;
        ++pos;
      }
    }
    if (sw) summary[si] = 0u;
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

// b1 and the count above it, from a kTopkBins histogram; all threads get them
CSA_DEV void find_bin(const int* hist, int k, int* s_w, int* s_out, int* b1, int* above) {
  const int tid = threadIdx.x;
  constexpr int PER = kTopkBins / kT;  // 8
  int c[PER], tot = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    c[i] = hist[kTopkBins - 1 - (PER * tid + i)];
    tot += c[i];
  }
  int all;
  const int before = block_excl_scan(tot, s_w, &all);
  if (before < k && before + tot >= k) {
    int acc = before;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (acc + c[i] >= k) {
        s_out[0] = kTopkBins - 1 - (PER * tid + i);
        s_out[1] = acc;
        break;
      }
      acc += c[i];
    }
  }
  __syncthreads();
  *b1 = s_out[0];
  *above = s_out[1];
  __syncthreads();
}

struct Lds {
  uint32_t ckey[kTopkCandCap];
  int cid[kTopkCandCap];
  int hist[kTopkBins];
  int misc[16];
};

}  // namespace

// ---------------------------------------------------------------------------
// split mode: grid (n_slices, rows), kT threads.  hist filled by the scorer.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kT) void topk_collect_kernel(IndexArgs a, TopkWs ws, int slice_len) {
  __shared__ int s_misc[16];
  const int row = blockIdx.y, b = row / a.Tq, tq = row % a.Tq, tid = threadIdx.x;
  const int64_t t = a.q_pos ? a.q_pos[(size_t)b * a.Tq + tq] : a.q_pos0 + tq;
  const int nv = (int)visible(a, b, t);
  const int k = a.k;
  int* hist = ws.hist + (size_t)row * kTopkBins;
  int* ctr = ws.ctr + (size_t)row * 4;
  uint32_t* bitmap = ws.bitmap + (size_t)row * ws.bitmap_words;
  uint32_t* summary = ws.summary + (size_t)row * ws.summary_words;
  uint2* cand = ws.cand + (size_t)row * kTopkCandCap;
  const float* sc = a.scores + (size_t)row * a.E_cap;

  int b1 = -1, above = 0;
  if (nv > k) {
    find_bin(hist, k, s_misc, s_misc + 8, &b1, &above);
    const int s0 = blockIdx.x * slice_len;
    const int s1 = min(nv, s0 + slice_len);
    // pass 1: mark winners above the bin, count candidates (keys stay in
    // registers for pass 2; slices are at most kCollectPer * kT long)
    uint32_t keys[kCollectPer];
    int nc = 0;
#pragma unroll
    for (int i = 0; i < kCollectPer; ++i) {
      const int s = s0 + tid + i * kT;
      keys[i] = s < s1 ? f32_key(sc[s]) : 0u;
    }
#pragma unroll
    for (int i = 0; i < kCollectPer; ++i) {
      const int s = s0 + tid + i * kT;
      if (s < s1) {
        const int bin = (int)bin_of(keys[i]);
        if (bin > b1) mark(bitmap, summary, s);
        nc += bin == b1;
      }
    }
    int total;
    int off = block_excl_scan(nc, s_misc, &total);
    if (tid == 0) s_misc[4] = total ? atomicAdd(&ctr[0], total) : 0;
    __syncthreads();
    off += s_misc[4];
    // pass 2: write candidates into the reserved slots
    if (nc) {
#pragma unroll
      for (int i = 0; i < kCollectPer; ++i) {
        const int s = s0 + tid + i * kT;
        if (s < s1 && (int)bin_of(keys[i]) == b1) {
          if (off < kTopkCandCap) cand[off] = make_uint2(keys[i], (uint32_t)s);
          ++off;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// split mode, stage 2: grid (rows), one workgroup resolves a row's
// candidates, emits its ids and clears the row's scratch.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kT) void topk_resolve_kernel(IndexArgs a, TopkWs ws) {
  extern __shared__ unsigned char dyn[];
  Lds& L = *reinterpret_cast<Lds*>(dyn);
  uint32_t* lbit = reinterpret_cast<uint32_t*>(dyn + sizeof(Lds));  // [bitmap_words]
  uint32_t* lsum = lbit + ws.bitmap_words;                           // [summary_words]
  const int row = blockIdx.x, b = row / a.Tq, tq = row % a.Tq, tid = threadIdx.x;
  const int64_t t = a.q_pos ? a.q_pos[(size_t)b * a.Tq + tq] : a.q_pos0 + tq;
  const int nv = (int)visible(a, b, t);
  const int k = a.k;
  int* hist = ws.hist + (size_t)row * kTopkBins;
  int* ctr = ws.ctr + (size_t)row * 4;
  uint32_t* bitmap = ws.bitmap + (size_t)row * ws.bitmap_words;
  uint32_t* summary = ws.summary + (size_t)row * ws.summary_words;
  const uint2* cand = ws.cand + (size_t)row * kTopkCandCap;
  const float* sc = a.scores + (size_t)row * a.E_cap;
  int32_t* out = a.topk_idx + (size_t)row * k;
  if (nv <= k) {
    for (int i = tid; i < k; i += kT) out[i] = i < nv ? i : -1;
    if (tid == 0) a.topk_cnt[row] = nv;
  } else {
    const int nwords = (nv + 31) >> 5, nsum = (nwords + 31) >> 5;
    // the row's winners so far (marked by the collect pass) move to LDS
    for (int i = tid; i < nwords; i += kT) lbit[i] = bitmap[i];
    for (int i = tid; i < nsum; i += kT) lsum[i] = summary[i];
    int b1, above;
    find_bin(hist, k, L.misc, L.misc + 8, &b1, &above);
    const int n_cand = ctr[0];
    if (n_cand <= kTopkCandCap) {
      for (int i = tid; i < n_cand; i += kT) {
        const uint2 v = cand[i];
        L.ckey[i] = v.x;
        L.cid[i] = (int)v.y;
      }
      __syncthreads();
      select_candidates(L.ckey, L.cid, n_cand, k - above, lbit, lsum, L.hist, L.misc);
    } else {
      topk_resolve_from_row(sc, nv, b1, k - above, lbit, lsum, L.cid, L.hist, L.misc);
    }
    __syncthreads();
    // clear the global bitmap words the collect pass may have set
    for (int i = tid; i < nsum; i += kT) {
      uint32_t sw = lsum[i];
      if (sw) summary[i] = 0u;
      while (sw) {
        const int j = __ffs(sw) - 1;
        sw &= sw - 1;
        bitmap[32 * i + j] = 0u;
      }
    }
    emit_bitmap(lbit, lsum, nwords, out, k, &a.topk_cnt[row], L.misc);
  }
  __syncthreads();
  for (int i = tid; i < kTopkBins; i += kT) hist[i] = 0;
  if (tid == 0) ctr[0] = 0;
}

// ---------------------------------------------------------------------------
// row mode: grid (rows), one workgroup per row, scores already written.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kT) void topk_rowsel_kernel(IndexArgs a, TopkWs ws) {
  extern __shared__ unsigned char dyn[];
  Lds& L = *reinterpret_cast<Lds*>(dyn);
  uint32_t* lbit = reinterpret_cast<uint32_t*>(dyn + sizeof(Lds));  // [bitmap_words]
  uint32_t* lsum = lbit + ws.bitmap_words;                           // [summary_words]
  const int row = blockIdx.x, b = row / a.Tq, tq = row % a.Tq, tid = threadIdx.x;
  const int64_t t = a.q_pos ? a.q_pos[(size_t)b * a.Tq + tq] : a.q_pos0 + tq;
  const int nv = (int)visible(a, b, t);
  const int k = a.k;
  const float* sc = a.scores + (size_t)row * a.E_cap;
  int32_t* out = a.topk_idx + (size_t)row * k;
  if (nv <= k) {
    for (int i = tid; i < k; i += kT) out[i] = i < nv ? i : -1;
    if (tid == 0) a.topk_cnt[row] = nv;
    return;
  }
  const int nwords = (nv + 31) >> 5, nsum = (nwords + 31) >> 5;
  for (int i = tid; i < kTopkBins; i += kT) L.hist[i] = 0;
  for (int i = tid; i < nwords; i += kT) lbit[i] = 0u;
  for (int i = tid; i < nsum; i += kT) lsum[i] = 0u;
  __syncthreads();
  for (int s = tid; s < nv; s += kT) atomicAdd(&L.hist[bin_of(f32_key(sc[s]))], 1);
  __syncthreads();
  int b1, above;
  find_bin(L.hist, k, L.misc, L.misc + 8, &b1, &above);
  int nc = 0;
  for (int s = tid; s < nv; s += kT) {
    const int bin = (int)bin_of(f32_key(sc[s]));
    if (bin > b1) mark(lbit, lsum, s);
    nc += bin == b1;
  }
  int n_cand;
  int off = block_excl_scan(nc, L.misc, &n_cand);
  if (n_cand <= kTopkCandCap) {
    if (nc) {
      for (int s = tid; s < nv; s += kT) {
        const uint32_t key = f32_key(sc[s]);
        if ((int)bin_of(key) == b1) {
          L.ckey[off] = key;
          L.cid[off] = s;
          ++off;
        }
      }
    }
    __syncthreads();
    select_candidates(L.ckey, L.cid, n_cand, k - above, lbit, lsum, L.hist, L.misc);
  } else {
    topk_resolve_from_row(sc, nv, b1, k - above, lbit, lsum, L.cid, L.hist, L.misc);
  }
  __syncthreads();
  emit_bitmap(lbit, lsum, nwords, out, k, &a.topk_cnt[row], L.misc);
}

// Exact resolution when the threshold bin holds more than kTopkCandCap keys:
// radix refine over the row on bits 20..0 restricted to bin b1 (3 passes),
// then one in-order pass marks keys above the threshold and the lowest-id
// ties (the row is scanned in id order, chunk by chunk).
__device__ void topk_resolve_from_row(const float* sc, int nv, int b1, int want, uint32_t* bitmap,
                                      uint32_t* summary, int* s_scan, int* s_hist, int* s_misc) {
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
    if (tid < 64) wave_find<2, true>(s_hist, rem, s_misc);
    __syncthreads();
    prefix = (prefix << 7) | (uint32_t)s_misc[0];
    rem -= s_misc[1];
    __syncthreads();
  }
  const uint32_t tau = prefix;
  int taken = 0;
  for (int base = 0; base < nv; base += kT) {
    const int s = base + tid;
    const uint32_t key = s < nv ? f32_key(sc[s]) : 0u;
    const bool bin_ok = s < nv && (int)(key >> kTopkShift) == b1;
    const bool eq = bin_ok && key == tau;
    int tot;
    const int rank = taken + block_excl_scan(eq ? 1 : 0, s_scan, &tot);
    if (bin_ok && (key > tau || (eq && rank < rem))) mark(bitmap, summary, s);
    taken += tot;
  }
  __syncthreads();
}

size_t topk_split_lds_bytes(int E_cap) {
  const size_t words = ((size_t)E_cap + 31) / 32;
  return sizeof(Lds) + (words + (words + 31) / 32) * 4;
}

size_t topk_ws_bytes(int rows, int E_cap, bool with_cand) {
  const size_t words = ((size_t)E_cap + 31) / 32;
  const size_t swords = (words + 31) / 32;
  return (size_t)rows * (kTopkBins * 4 + 16 + (words + swords) * 4 +
                         (with_cand ? (size_t)kTopkCandCap * 8 : 0)) +
         1024;
}

TopkWs topk_ws_carve(void* base, int rows, int E_cap, bool with_cand) {
  TopkWs w;
  char* p = reinterpret_cast<char*>(base);
  w.bitmap_words = (int)(((size_t)E_cap + 31) / 32);
  w.summary_words = (w.bitmap_words + 31) / 32;
  w.hist = reinterpret_cast<int*>(p);
  p += (size_t)rows * kTopkBins * 4;
  w.ctr = reinterpret_cast<int*>(p);
  p += (size_t)rows * 16;
  w.bitmap = reinterpret_cast<uint32_t*>(p);
  p += (size_t)rows * w.bitmap_words * 4;
  w.summary = reinterpret_cast<uint32_t*>(p);
  p += (size_t)rows * w.summary_words * 4;
  p = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(p) + 15) & ~uintptr_t(15));
  w.cand = with_cand ? reinterpret_cast<uint2*>(p) : nullptr;
  return w;
}

static size_t topk_lds_bytes() { return sizeof(Lds); }

hipError_t launch_topk_collect(const IndexArgs& a, const TopkWs& ws, int slices, int slice_len,
                               hipStream_t s) {
  CSA_LAUNCH("topk_collect", topk_collect_kernel, dim3(slices, a.B * a.Tq), dim3(kT), 0, s, a, ws,
             slice_len);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds = topk_lds_bytes() + (size_t)(ws.bitmap_words + ws.summary_words) * 4;
  static int attr2 = 0;
  if (attr2 < (int)lds) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&topk_resolve_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr2 = (int)lds;
  }
  CSA_LAUNCH("topk_resolve", topk_resolve_kernel, dim3(a.B * a.Tq), dim3(kT), lds, s, a, ws);
  return hipGetLastError();
}

hipError_t launch_topk_rows(const IndexArgs& a, const TopkWs& ws, hipStream_t s) {
  const size_t lds = topk_split_lds_bytes(a.E_cap);
  static int attr_set = 0;
  if (attr_set < (int)lds) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&topk_rowsel_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = (int)lds;
  }
  CSA_LAUNCH("topk_rows", topk_rowsel_kernel, dim3(a.B * a.Tq), dim3(kT), lds, s, a, ws);
  return hipGetLastError();
}

}  // namespace csa
