// Exact per-query top-k over index scores (row a3): the k largest scores of
// the visible entries, ties to the lower entry id, ids emitted in ascending
// order, -1 padded ("2026 DeepSeek-V4" note, "Key design 1": C_t =
// TopK_k(I_t,:); "DeepSeek-V4" book ch. 6: all entries kept when fewer than k
// are visible).
//
// Scores are compared as order-preserving 32-bit keys.  Selection runs in two
// stages:
//  1. coarse: a histogram of the top 11 key bits locates the bin b1 holding
//     the k-th largest key.  Every entry in a higher bin is a certain winner
//     (there are fewer than k of them); entries in bin b1 are candidates.
//  2. exact: the (k - #certain) largest candidates are found by radix select
//     on the remaining 21 key bits and, among equal keys, on the entry id.
// If bin b1 holds more candidates than fit in LDS, the threshold is refined
// over the whole row instead and the winners are emitted by one in-order
// scan of the row.
//
// Fused mode (decode, few long rows): the scoring kernel accumulates the
// histogram, publishes b1 per row and leaves each workgroup's certain winners
// and candidates in entry order in its own list region; one workgroup per row
// (topk_fused_resolve_kernel) selects among the candidates keeping their
// order and places every id at its rank in its own list plus its rank in the
// other: a merge of two sorted lists, no sort.  Split mode (the same rows when
// the scorer cannot fuse): collect workgroups append both lists per row, and
// the resolve sorts the winners by id buckets.  Row mode (many rows, prefill):
// one workgroup per row does everything from the row's scores.

#include <atomic>

#include "common.h"
#include "kernels.h"
#include "topk.h"

namespace csa {

namespace {

constexpr int kCT = 256;   // collect workgroup
constexpr int kRT = 1024;  // resolve / row workgroup
constexpr int kSpecL = 16;  // fused resolve: list entries per workgroup loaded with the counts
constexpr int kSpecU = 4;   // ... by this many loads per thread (n_wg * kSpecL <= kSpecU * kRT)
constexpr int kRowU = 16;   // row mode: scores per thread and batch (loads in flight together)
constexpr int kSampleBlk = 16;  // row mode: 256-score blocks sampled for the threshold guess
constexpr int kCollectPer = kTopkCollectSlice / kCT;  // 16 keys per thread

CSA_DEV uint32_t bin_of(uint32_t key) { return key >> kTopkShift; }

// In a histogram of 64 * PER bins, the bin where the count accumulated from
// the top (DESC) or the bottom first reaches `want`.  Executed by one
// wavefront; writes (bin, count before it) to s_out[0..1].
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

CSA_DEV int64_t visible(const IndexArgs& a, int b, int64_t t) {
  const int64_t lim = vis_limit(t, a.m, a.vis);
  const int64_t have = (int64_t)a.n_entries[b] + a.n_add;
  int64_t n = lim < have ? lim : have;
  if (n > a.E_cap) n = a.E_cap;
  return n < 0 ? 0 : n;
}

// LDS of a resolving workgroup.  misc: [0..1] wave_find result, [8..23] and
// [24..39] scan scratch, [40..41] find_bin result, [48..49] list counters.
struct Lds {
  uint32_t ckey[kTopkCandCap];
  int cid[kTopkCandCap];
  int win[kTopkMaxK];   // winner ids (sorted in place)
  int hist[kTopkBins];  // radix histograms / the row histogram
  int sel[kTopkMaxK];   // selected candidates (ordered selection)
  int misc[64];
};

// Radix select among n candidates (keys all in bin b1): the `want` largest,
// ties to the lower id.  Appends the winners' ids to win[*n_win ...].
CSA_DEV void select_candidates(Lds& L, int n, uint32_t b1, int want, int* n_win) {
  const int tid = threadIdx.x;
  uint32_t prefix = b1;
  int rem = want;
  int shift = kTopkShift;
  for (int pass = 0; pass < 3; ++pass) {  // bits 20..14, 13..7, 6..0
    shift -= 7;
    if (tid < 128) L.hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kRT) {
      const uint32_t key = L.ckey[i];
      if ((key >> (shift + 7)) == prefix) atomicAdd(&L.hist[(key >> shift) & 127], 1);
    }
    __syncthreads();
    if (tid < 64) wave_find<2, true>(L.hist, rem, L.misc);
    __syncthreads();
    prefix = (prefix << 7) | (uint32_t)L.misc[0];
    rem -= L.misc[1];
    __syncthreads();
  }
  const uint32_t tau = prefix;  // key of the last winner; `rem` keys equal to tau win
  int nt = 0;
  for (int i = tid; i < n; i += kRT) nt += L.ckey[i] == tau;
  int n_tie;
  block_excl_scan<kRT>(nt, L.misc + 8, &n_tie);
  int id_lim = 0x7fffffff;  // ties with id <= id_lim win
  if (n_tie > rem) {
    // the rem lowest ids among the ties: 2 passes of 10 bits (ids < 2^20)
    uint32_t ipref = 0;
    for (int pass = 0; pass < 2; ++pass) {
      const int sh = 10 - 10 * pass;
      for (int i = tid; i < 1024; i += kRT) L.hist[i] = 0;
      __syncthreads();
      for (int i = tid; i < n; i += kRT) {
        const uint32_t id = (uint32_t)L.cid[i];
        if (L.ckey[i] == tau && (pass == 0 || (id >> (sh + 10)) == ipref))
          atomicAdd(&L.hist[(id >> sh) & 1023], 1);
      }
      __syncthreads();
      if (tid < 64) wave_find<16, false>(L.hist, rem, L.misc);
      __syncthreads();
      ipref = (ipref << 10) | (uint32_t)L.misc[0];
      rem -= L.misc[1];
      __syncthreads();
    }
    id_lim = (int)ipref;  // ids are distinct: exactly the wanted ties have id <= ipref
  }
  if (tid == 0) L.misc[48] = *n_win;
  __syncthreads();
  for (int i = tid; i < n; i += kRT) {
    const uint32_t key = L.ckey[i];
    if (key > tau || (key == tau && L.cid[i] <= id_lim)) {
      const int o = atomicAdd(&L.misc[48], 1);
      if (o < kTopkMaxK) L.win[o] = L.cid[i];
    }
  }
  __syncthreads();
  *n_win = min(L.misc[48], kTopkMaxK);
  __syncthreads();
}

// The same selection for candidates stored in ascending id order, keeping
// that order: the selected ids go to sel[0 ..) (capacity kTopkMaxK).  The
// (up to) three radix passes count into their own 128-bin histograms
// (cleared together up front), so a pass costs two barriers; they stop once
// the boundary bin holds exactly the keys still wanted.  The final filter
// needs one scan: a thread's winners go after the winners above tau (on the
// resolved top bits) of the threads before it and the first rem ties.
// Returns the count selected.
CSA_DEV int select_ordered(Lds& L, int n, uint32_t b1, int want, int* sel) {
  const int tid = threadIdx.x;
  if (tid < 384) L.hist[tid] = 0;
  __syncthreads();
  uint32_t prefix = b1;
  int rem = want;
  int shift = kTopkShift;
  for (int pass = 0; pass < 3; ++pass) {  // bits 20..14, 13..7, 6..0
    shift -= 7;
    int* h = L.hist + 128 * pass;
    for (int i = tid; i < n; i += kRT) {
      const uint32_t key = L.ckey[i];
      if ((key >> (shift + 7)) == prefix) atomicAdd(&h[(key >> shift) & 127], 1);
    }
    __syncthreads();
    if (tid < 64) wave_find<2, true>(h, rem, L.misc + 2 * pass);
    __syncthreads();
    prefix = (prefix << 7) | (uint32_t)L.misc[2 * pass];
    rem -= L.misc[2 * pass + 1];
    // every key with this prefix is taken: the lower bits need no pass
    if (h[L.misc[2 * pass]] == rem) break;
  }
  // the threshold on the resolved top bits of the key (21 bits below b1's)
  const uint32_t tau = prefix;
  const int cpt = (n + kRT - 1) / kRT;
  const int i0 = min(tid * cpt, n), i1 = min(i0 + cpt, n);
  int ng = 0, nt = 0;  // keys above tau, ties
  for (int i = i0; i < i1; ++i) {
    const uint32_t key = L.ckey[i] >> shift;
    ng += key > tau;
    nt += key == tau;
  }
  int tot;
  const int pre = block_excl_scan<kRT>(ng | (nt << 16), L.misc + 8, &tot);
  int tie_rank = pre >> 16;
  int o = (pre & 0xffff) + min(tie_rank, rem);
  for (int i = i0; i < i1; ++i) {
    const uint32_t key = L.ckey[i] >> shift;
    bool take = key > tau;
    if (key == tau) take = tie_rank++ < rem;
    if (take && o < kTopkMaxK) sel[o++] = L.cid[i];
  }
  __syncthreads();
  return (tot & 0xffff) + min(tot >> 16, rem);
}

CSA_DEV int lower_bound_i(const int* v, int n, int x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (v[mid] < x) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

// last j in [0, n) with off[j] <= g (off ascending, off[n] = total > g)
CSA_DEV int owner_of(const int* off, int n, int g) {
  int lo = 0, hi = n;  // off[lo] <= g < off[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (off[mid] <= g) lo = mid;
    else hi = mid;
  }
  return lo;
}

// Ascending sort of the n (<= kTopkMaxK) distinct ids in win[], by buckets
// of the id range [0, nv): bucket counts, their exclusive prefix, a scatter
// into ckey/cid storage (free after the selection), then each thread orders
// its own buckets (about one id per bucket on average) by insertion sort.
// The sorted ids end in L.cid[0..n).
constexpr int kSortBuckets = 2048;
CSA_DEV void sort_ids(Lds& L, int n, int nv) {
  const int tid = threadIdx.x;
  int* cnt = L.hist;                                    // [kSortBuckets]
  int* start = reinterpret_cast<int*>(L.ckey);          // [kSortBuckets] bucket starts
  int* fill = reinterpret_cast<int*>(L.ckey) + kSortBuckets;
  int* dst = L.cid;
  auto bucket = [&](int id) { return (int)(((uint64_t)(uint32_t)id * kSortBuckets) / (uint32_t)nv); };
  for (int i = tid; i < kSortBuckets; i += kRT) cnt[i] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += kRT) atomicAdd(&cnt[bucket(L.win[i])], 1);
  __syncthreads();
  constexpr int PER = kSortBuckets / kRT;
  int c[PER], tot = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    c[j] = cnt[PER * tid + j];
    tot += c[j];
  }
  int all;
  int off = block_excl_scan<kRT>(tot, L.misc + 8, &all);
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    start[PER * tid + j] = off;
    fill[PER * tid + j] = off;
    off += c[j];
  }
  __syncthreads();
  for (int i = tid; i < n; i += kRT) {
    const int id = L.win[i];
    dst[atomicAdd(&fill[bucket(id)], 1)] = id;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int bk = PER * tid + j, b0 = start[bk], b1 = b0 + c[j];
    for (int x = b0 + 1; x < b1; ++x) {
      const int v = dst[x];
      int y = x - 1;
      while (y >= b0 && dst[y] > v) {
        dst[y + 1] = dst[y];
        --y;
      }
      dst[y + 1] = v;
    }
  }
  __syncthreads();
}

// Threshold over the whole row (bin b1 too large for LDS): radix refine on
// bits 20..0 restricted to b1, then one in-order pass writes every winner
// (key above the threshold, or equal to it among the first `rem` in id
// order) to out in ascending id order.  Returns the count written.
CSA_DEV int resolve_from_row(Lds& L, const float* sc, int nv, int b1, int want, int32_t* out) {
  const int tid = threadIdx.x;
  uint32_t prefix = (uint32_t)b1;
  int rem = want;
  int shift = kTopkShift;
  for (int pass = 0; pass < 3; ++pass) {
    shift -= 7;
    if (tid < 128) L.hist[tid] = 0;
    __syncthreads();
    for (int s = tid; s < nv; s += kRT) {
      const uint32_t key = f32_key(sc[s]);
      if ((key >> (shift + 7)) == prefix) atomicAdd(&L.hist[(key >> shift) & 127], 1);
    }
    __syncthreads();
    if (tid < 64) wave_find<2, true>(L.hist, rem, L.misc);
    __syncthreads();
    prefix = (prefix << 7) | (uint32_t)L.misc[0];
    rem -= L.misc[1];
    __syncthreads();
  }
  const uint32_t tau = prefix;
  int taken = 0, pos = 0;
  for (int base = 0; base < nv; base += kRT) {
    const int s = base + tid;
    const uint32_t key = s < nv ? f32_key(sc[s]) : 0u;
    const bool eq = s < nv && key == tau;
    int n_eq;
    const int rank = taken + block_excl_scan<kRT>(eq ? 1 : 0, L.misc + 8, &n_eq);
    const bool win = s < nv && (key > tau || (eq && rank < rem));
    int n_w;
    const int off = block_excl_scan<kRT>(win ? 1 : 0, L.misc + 24, &n_w);
    if (win) out[pos + off] = s;
    taken += n_eq;
    pos += n_w;
  }
  return pos;
}

// write the sorted winners (L.cid) and the -1 padding, and the count
CSA_DEV void emit(const Lds& L, int n, int k, int32_t* out, int32_t* cnt) {
  const int tid = threadIdx.x;
  for (int i = tid; i < k; i += kRT) out[i] = i < n ? L.cid[i] : -1;
  if (tid == 0) *cnt = n < k ? n : k;
}

}  // namespace

// ---------------------------------------------------------------------------
// split mode, stage 1: grid (n_slices, rows), kCT threads.  The row's
// histogram was filled by the scorer.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kCT) void topk_collect_kernel(IndexArgs a, TopkWs ws, int slice_len) {
  __shared__ int s_misc[32];
  const int row = blockIdx.y, b = row / a.Tq, tq = row % a.Tq, tid = threadIdx.x;
  const int64_t t = a.q_pos ? a.q_pos[(size_t)b * a.Tq + tq] : a.q_pos0 + tq;
  const int nv = (int)visible(a, b, t);
  const int k = a.k;
  if (nv <= k) return;
  const int s0 = blockIdx.x * slice_len;
  if (s0 >= nv) return;
  const int s1 = min(nv, s0 + slice_len);
  const float* sc = a.scores + (size_t)row * a.E_cap;
  // the slice's scores first (independent of the threshold bin)
  uint32_t keys[kCollectPer];
#pragma unroll
  for (int i = 0; i < kCollectPer; ++i) {
    const int s = s0 + tid + i * kCT;
    keys[i] = s < s1 ? f32_key(sc[s]) : 0u;
  }
  int b1, above;
  find_bin<kCT>(ws.hist + (size_t)row * kTopkBins, k, s_misc, s_misc + 8, &b1, &above);
  // per thread: certain winners in the low half, candidates in the high half
  // (at most kCollectPer each, so one scan carries both counts)
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < kCollectPer; ++i) {
    const int s = s0 + tid + i * kCT;
    if (s < s1) {
      const int bin = (int)bin_of(keys[i]);
      cnt += (bin > b1 ? 1 : 0) + (bin == b1 ? 1 << 16 : 0);
    }
  }
  int total;
  const int off = block_excl_scan<kCT>(cnt, s_misc, &total);
  // one 64-bit reservation for both lists: candidates in the low word,
  // certain winners in the high word
  unsigned long long* ctr = reinterpret_cast<unsigned long long*>(ws.ctr + (size_t)row * 4);
  if (tid == 0) {
    const unsigned long long ts = total & 0xffff, tc = (unsigned)total >> 16;
    const unsigned long long old = total ? atomicAdd(ctr, tc | (ts << 32)) : 0ull;
    s_misc[16] = (int)(old >> 32);
    s_misc[17] = (int)(old & 0xffffffffull);
  }
  __syncthreads();
  if (cnt == 0) return;
  int os = s_misc[16] + (off & 0xffff), oc = s_misc[17] + (off >> 16);
  int* sure = ws.sure + (size_t)row * kTopkMaxK;
  uint2* cand = ws.cand + (size_t)row * kTopkCandCap;
#pragma unroll
  for (int i = 0; i < kCollectPer; ++i) {
    const int s = s0 + tid + i * kCT;
    if (s < s1) {
      const int bin = (int)bin_of(keys[i]);
      if (bin > b1) {  // fewer than k of them in the row
        if (os < kTopkMaxK) sure[os] = s;
        ++os;
      }
      if (bin == b1) {
        if (oc < kTopkCandCap) cand[oc] = make_uint2(keys[i], (uint32_t)s);
        ++oc;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// split mode, stage 2: grid (rows), kRT threads; resolves a row and returns
// its histogram and counters to zero.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kRT) void topk_resolve_kernel(IndexArgs a, TopkWs ws) {
  extern __shared__ unsigned char dyn[];
  Lds& L = *reinterpret_cast<Lds*>(dyn);
  const int row = blockIdx.x, b = row / a.Tq, tq = row % a.Tq, tid = threadIdx.x;
  const int64_t t = a.q_pos ? a.q_pos[(size_t)b * a.Tq + tq] : a.q_pos0 + tq;
  const int nv = (int)visible(a, b, t);
  const int k = a.k;
  int* hist = ws.hist + (size_t)row * kTopkBins;
  int* ctr = ws.ctr + (size_t)row * 4;
  int32_t* out = a.topk_idx + (size_t)row * k;
  if (nv <= k) {
    for (int i = tid; i < k; i += kRT) out[i] = i < nv ? i : -1;
    if (tid == 0) a.topk_cnt[row] = nv;
  } else {
    const int n_cand = ctr[0], n_sure = min(ctr[1], kTopkMaxK);
    int b1, above;
    find_bin<kRT>(hist, k, L.misc + 8, L.misc + 40, &b1, &above);
    if (n_cand <= kTopkCandCap) {
      const uint2* cand = ws.cand + (size_t)row * kTopkCandCap;
      const int* sure = ws.sure + (size_t)row * kTopkMaxK;
      for (int i = tid; i < n_cand; i += kRT) {
        const uint2 v = cand[i];
        L.ckey[i] = v.x;
        L.cid[i] = (int)v.y;
      }
      for (int i = tid; i < n_sure; i += kRT) L.win[i] = sure[i];
      __syncthreads();
      int n_win = n_sure;  // == above
      select_candidates(L, n_cand, (uint32_t)b1, k - above, &n_win);
      sort_ids(L, n_win, nv);
      emit(L, n_win, k, out, &a.topk_cnt[row]);
    } else {
      const int n = resolve_from_row(L, a.scores + (size_t)row * a.E_cap, nv, b1, k - above, out);
      if (tid == 0) a.topk_cnt[row] = n;
    }
  }
  __syncthreads();
  for (int i = tid; i < kTopkBins; i += kRT) hist[i] = 0;
  if (tid == 0) {
    ctr[0] = 0;
    ctr[1] = 0;
  }
}

// ---------------------------------------------------------------------------
// fused mode, stage 2: grid (rows), kRT threads.  The n_wg scoring
// workgroups of a row left their certain winners and candidates in entry
// order, each in its own region; concatenated in workgroup order both lists
// are sorted by id.  Radix select among the candidates (order kept), then
// each id's output position is its rank in its own list plus its rank in
// the other (a merge of two sorted lists).  A row whose scoring workgroups
// did not all pass the grid barrier is resolved from its scores instead.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kRT) void topk_fused_resolve_kernel(IndexArgs a, TopkWs ws, int n_wg) {
  extern __shared__ unsigned char dyn[];
  Lds& L = *reinterpret_cast<Lds*>(dyn);
  __shared__ int s_os[kTopkMaxWgRow + 1], s_oc[kTopkMaxWgRow + 1];
  const int row = blockIdx.x, b = row / a.Tq, tq = row % a.Tq, tid = threadIdx.x, lane = tid & 63;
  int* hist = ws.hist + (size_t)row * kTopkBins;
  int* ctr = ws.ctr + (size_t)row * 4;
  int32_t* out = a.topk_idx + (size_t)row * a.k;
  const int* lsure = ws.lsure + (size_t)row * ws.list_len;
  const uint2* lcand = ws.lcand + (size_t)row * ws.list_len;
  const int stride = ws.list_stride;
  // all requested at once: the workgroups' counts, the failure flag and the
  // threshold bin the scoring kernel published, the position, and the first
  // kSpecL entries of every workgroup's two lists (at fixed places), which
  // hold whole lists but for rare long ones
  const int4 info = tid < n_wg ? ws.wg_info[(size_t)row * kTopkMaxWgRow + tid] : make_int4(0, 0, 0, 0);
  const int failed = ctr[2], pub = ctr[3];
  const int64_t t = a.q_pos ? a.q_pos[(size_t)b * a.Tq + tq] : a.q_pos0 + tq;
  const bool spec = n_wg * kSpecL <= kSpecU * kRT;
  int sv[kSpecU];
  uint2 cv[kSpecU];
#pragma unroll
  for (int u = 0; u < kSpecU; ++u) {
    const int f = tid + kRT * u, j = f / kSpecL, kk = f % kSpecL;
    const size_t off = (size_t)(j < n_wg ? j : 0) * stride + kk;
    sv[u] = spec ? lsure[off] : 0;
    cv[u] = spec ? lcand[off] : make_uint2(0, 0);
  }
  const int nv = (int)visible(a, b, t);
  const int k = a.k;
  bool from_row = false;
  if (nv <= k) {
    for (int i = tid; i < k; i += kRT) out[i] = i < nv ? i : -1;
    if (tid == 0) a.topk_cnt[row] = nv;
  } else if (failed || pub == 0) {
    from_row = true;
  } else {
    const int b1 = pub & 2047, above = (pub >> 11) & 4095;
    // list offsets: wave 0 scans the workgroups' counts
    if (tid < n_wg) {
      s_os[tid] = info.x;
      s_oc[tid] = info.y;
    }
    // any list longer than the speculative part?
    const int longer = __syncthreads_or(tid < n_wg && (!spec || info.x > kSpecL || info.y > kSpecL));
    if (tid < 64) {
      const int cpw = (n_wg + 63) / 64, j0 = min(lane * cpw, n_wg), j1 = min(j0 + cpw, n_wg);
      int cs = 0, cc = 0;
      for (int j = j0; j < j1; ++j) {
        cs += s_os[j];
        cc += s_oc[j];
      }
      const int is = wave_incl_scan(cs), ic = wave_incl_scan(cc);
      int os = is - cs, oc = ic - cc;
      for (int j = j0; j < j1; ++j) {
        const int ns = s_os[j], nc = s_oc[j];
        s_os[j] = os;
        s_oc[j] = oc;
        os += ns;
        oc += nc;
      }
      if (lane == 63) {
        s_os[n_wg] = is;
        s_oc[n_wg] = ic;
      }
    }
    __syncthreads();
    const int tot_s = s_os[n_wg], tot_c = s_oc[n_wg];
    if (tot_s != above || tot_c > kTopkCandCap) {
      from_row = true;
    } else {
      // place the speculatively loaded entries; the rest of longer lists
      // (each workgroup's entries kSpecL ..) is fetched now, a wavefront per
      // workgroup
      if (spec) {
#pragma unroll
        for (int u = 0; u < kSpecU; ++u) {
          const int f = tid + kRT * u, j = f / kSpecL, kk = f % kSpecL;
          if (j < n_wg) {
            if (kk < s_os[j + 1] - s_os[j]) L.win[s_os[j] + kk] = sv[u];
            if (kk < s_oc[j + 1] - s_oc[j]) {
              L.ckey[s_oc[j] + kk] = cv[u].x;
              L.cid[s_oc[j] + kk] = (int)cv[u].y;
            }
          }
        }
      }
      const int first = spec ? kSpecL : 0;
      for (int j = tid >> 6; longer && j < n_wg; j += kRT / 64) {
        const int ns = s_os[j + 1] - s_os[j], nc = s_oc[j + 1] - s_oc[j];
        for (int kk = first + lane; kk < ns; kk += 64) L.win[s_os[j] + kk] = lsure[(size_t)j * stride + kk];
        for (int kk = first + lane; kk < nc; kk += 64) {
          const uint2 v = lcand[(size_t)j * stride + kk];
          L.ckey[s_oc[j] + kk] = v.x;
          L.cid[s_oc[j] + kk] = (int)v.y;
        }
      }
      __syncthreads();
      const int want = k - above;
      int* sel = L.sel;
      {
        const int n = select_ordered(L, tot_c, (uint32_t)b1, want, sel);
        if (tid == 0) L.misc[50] = n;
        __syncthreads();
      }
      const int n_sel = min(L.misc[50], want);
      // every id at its rank in its own list plus its rank in the other
      // (both lists ascending): one binary search per id, the two lists'
      // ids spread over the threads together
      for (int f = tid; f < tot_s + n_sel; f += kRT) {
        if (f < tot_s) {
          const int id = L.win[f];
          out[f + lower_bound_i(sel, n_sel, id)] = id;
        } else {
          const int id = sel[f - tot_s];
          out[f - tot_s + lower_bound_i(L.win, tot_s, id)] = id;
        }
      }
      for (int i = tot_s + n_sel + tid; i < k; i += kRT) out[i] = -1;
      if (tid == 0) a.topk_cnt[row] = tot_s + n_sel;
    }
  }
  if (from_row) {  // resolve from the row's scores
    int b1, above;
    find_bin<kRT>(hist, k, L.misc + 8, L.misc + 40, &b1, &above);
    const int n = resolve_from_row(L, a.scores + (size_t)row * a.E_cap, nv, b1, k - above, out);
    if (tid == 0) a.topk_cnt[row] = n;
  }
  __syncthreads();
  for (int i = tid; i < kTopkBins; i += kRT) hist[i] = 0;
  if (tid == 0) {
    ctr[0] = 0;
    ctr[1] = 0;
    ctr[2] = 0;
    ctr[3] = 0;
    ws.sync[row] = 0;
  }
}

// ---------------------------------------------------------------------------
// row mode: grid (rows), kRT threads, one workgroup per row, scores already
// written.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kRT) void topk_rowsel_kernel(IndexArgs a, TopkWs ws) {
  extern __shared__ unsigned char dyn[];
  Lds& L = *reinterpret_cast<Lds*>(dyn);
  (void)ws;
  const int row = blockIdx.x, b = row / a.Tq, tq = row % a.Tq, tid = threadIdx.x;
  const int64_t t = a.q_pos ? a.q_pos[(size_t)b * a.Tq + tq] : a.q_pos0 + tq;
  const int nv = (int)visible(a, b, t);
  const int k = a.k;
  const float* sc = a.scores + (size_t)row * a.E_cap;
  int32_t* out = a.topk_idx + (size_t)row * k;
  if (nv <= k) {
    for (int i = tid; i < k; i += kRT) out[i] = i < nv ? i : -1;
    if (tid == 0) a.topk_cnt[row] = nv;
    return;
  }
  for (int i = tid; i < kTopkBins; i += kRT) L.hist[i] = 0;
  if (tid == 0) {
    L.misc[48] = 0;
    L.misc[49] = 0;
  }
  __syncthreads();
  // A guess of the threshold bin from a sample: kSampleBlk blocks of 256
  // consecutive scores spread over the row (their sample's k_s-th largest,
  // k_s a wide margin above the k-th largest's expected count).  The row is
  // then read once: every score into the histogram, and the keys in bins at
  // or above the guess stashed with their ids.  When the row's threshold
  // bin b1 is at or above the guess and the stash did not overflow, the
  // winners (bin > b1) and candidates (bin == b1) are all in the stash;
  // otherwise the row is read a second time for them.
  int lo_bin = 0;
  {
    float v[kSampleBlk * 256 / kRT];
#pragma unroll
    for (int u = 0; u < kSampleBlk * 256 / kRT; ++u) {
      const int q = tid + kRT * u, blk = q / 256;
      const int s = (int)((int64_t)nv * blk / kSampleBlk) + q % 256;
      v[u] = s < nv ? sc[s] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kSampleBlk * 256 / kRT; ++u) {
      const int q = tid + kRT * u, blk = q / 256;
      const int s = (int)((int64_t)nv * blk / kSampleBlk) + q % 256;
      if (s < nv) atomicAdd(&L.hist[bin_of(f32_key(v[u]))], 1);
    }
    if (tid == 0) {
      L.misc[40] = 0;  // (no bin found: stash everything)
      L.misc[41] = 0;
    }
    __syncthreads();
    const int n_samp = nv < kSampleBlk * 256 ? nv : kSampleBlk * 256;
    const int k_s = (int)(2 * (int64_t)k * n_samp / nv) + 64;
    int ab;
    if (k_s < n_samp) find_bin<kRT>(L.hist, k_s, L.misc + 8, L.misc + 40, &lo_bin, &ab);
    for (int i = tid; i < kTopkBins; i += kRT) L.hist[i] = 0;
    __syncthreads();
  }
  // The row in batches of kRowU scores per thread, all of a batch's loads in
  // flight before its first use (one load, wait and LDS atomic per score
  // would make each score a global round trip).
  for (int s0 = 0; s0 < nv; s0 += kRowU * kRT) {
    float v[kRowU];
#pragma unroll
    for (int u = 0; u < kRowU; ++u) {
      const int s = s0 + tid + kRT * u;
      v[u] = s < nv ? sc[s] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kRowU; ++u) {
      const int s = s0 + tid + kRT * u;
      const uint32_t key = f32_key(v[u]);
      const int bin = (int)bin_of(key);
      if (s < nv) {
        atomicAdd(&L.hist[bin], 1);
        if (bin >= lo_bin) {
          const int o = atomicAdd(&L.misc[49], 1);
          if (o < kTopkCandCap) {
            L.ckey[o] = key;
            L.cid[o] = s;
          }
        }
      }
    }
  }
  __syncthreads();
  const int n_st = L.misc[49];
  int b1, above;
  find_bin<kRT>(L.hist, k, L.misc + 8, L.misc + 40, &b1, &above);
  if (b1 >= lo_bin && n_st <= kTopkCandCap) {
    // certain winners to win[], candidates to the front of ckey/cid
    constexpr int kStU = kTopkCandCap / kRT;
    uint32_t key[kStU];
    int id[kStU];
#pragma unroll
    for (int u = 0; u < kStU; ++u) {
      const int i = tid + kRT * u;
      key[u] = i < n_st ? L.ckey[i] : 0u;
      id[u] = i < n_st ? L.cid[i] : -1;
    }
    __syncthreads();
    if (tid == 0) L.misc[49] = 0;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kStU; ++u) {
      const int bin = (int)bin_of(key[u]);
      if (id[u] >= 0 && bin > b1) {
        const int o = atomicAdd(&L.misc[48], 1);
        if (o < kTopkMaxK) L.win[o] = id[u];
      }
      if (id[u] >= 0 && bin == b1) {
        const int o = atomicAdd(&L.misc[49], 1);
        L.ckey[o] = key[u];
        L.cid[o] = id[u];
      }
    }
  } else {
    // the guess missed: certain winners and candidates from a second read
    if (tid == 0) L.misc[49] = 0;
    __syncthreads();
    for (int s0 = 0; s0 < nv; s0 += kRowU * kRT) {
      float v[kRowU];
#pragma unroll
      for (int u = 0; u < kRowU; ++u) {
        const int s = s0 + tid + kRT * u;
        v[u] = s < nv ? sc[s] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < kRowU; ++u) {
        const int s = s0 + tid + kRT * u;
        const uint32_t key = f32_key(v[u]);
        const int bin = (int)bin_of(key);
        if (s < nv && bin > b1) {
          const int o = atomicAdd(&L.misc[48], 1);
          if (o < kTopkMaxK) L.win[o] = s;
        }
        if (s < nv && bin == b1) {
          const int o = atomicAdd(&L.misc[49], 1);
          if (o < kTopkCandCap) {
            L.ckey[o] = key;
            L.cid[o] = s;
          }
        }
      }
    }
  }
  __syncthreads();
  const int n_sure = min(L.misc[48], kTopkMaxK), n_cand = L.misc[49];
  __syncthreads();
  if (n_cand <= kTopkCandCap) {
    int n_win = n_sure;
    select_candidates(L, n_cand, (uint32_t)b1, k - above, &n_win);
    sort_ids(L, n_win, nv);
    emit(L, n_win, k, out, &a.topk_cnt[row]);
  } else {
    const int n = resolve_from_row(L, sc, nv, b1, k - above, out);
    if (tid == 0) a.topk_cnt[row] = n;
  }
}

namespace {
constexpr int kDefaultWaitPolls = 40000;
std::atomic<int> g_wait_polls{kDefaultWaitPolls};
}  // namespace

int fused_wait_polls() { return g_wait_polls.load(std::memory_order_relaxed); }

int set_fused_wait_polls(int polls) {
  if (polls < 0) polls = kDefaultWaitPolls;
  return g_wait_polls.exchange(polls & ~3, std::memory_order_relaxed);
}

size_t topk_ws_bytes(int rows, int E_cap, bool split) {
  size_t per = kTopkBins * 4 + 16;
  if (split)
    per += (size_t)kTopkCandCap * 8 + (size_t)kTopkMaxK * 4 + (size_t)kTopkMaxWgRow * 16 +
           (size_t)topk_list_len(E_cap) * (4 + 8);
  return (size_t)rows * per + 2048;
}

TopkWs topk_ws_carve(void* base, int rows, int E_cap, bool split) {
  TopkWs w{};
  auto align16 = [](char* q) { return reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(q) + 15) & ~uintptr_t(15)); };
  char* p = reinterpret_cast<char*>(base);
  w.hist = reinterpret_cast<int*>(p);
  p += (size_t)rows * kTopkBins * 4;
  w.ctr = reinterpret_cast<int*>(p);
  p += (size_t)rows * 16;
  p = align16(p);
  if (!split) return w;
  w.cand = reinterpret_cast<uint2*>(p);
  p += (size_t)rows * kTopkCandCap * 8;
  w.sure = reinterpret_cast<int*>(p);
  p += (size_t)rows * kTopkMaxK * 4;
  p = align16(p);
  w.sync = reinterpret_cast<unsigned*>(p);
  p += 256;
  w.wg_info = reinterpret_cast<int4*>(p);
  p += (size_t)rows * kTopkMaxWgRow * 16;
  w.list_len = topk_list_len(E_cap);
  w.lcand = reinterpret_cast<uint2*>(p);
  p += (size_t)rows * w.list_len * 8;
  w.lsure = reinterpret_cast<int*>(p);
  return w;
}

// raises the kernel's dynamic LDS limit once per device (done[device])
template <typename K>
static hipError_t allow_lds(K kernel, size_t bytes, std::atomic<size_t>* done) {
  const int dev = current_device();
  if (dev >= 0 && done[dev].load(std::memory_order_relaxed) >= bytes) return hipSuccess;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess && dev >= 0) done[dev].store(bytes, std::memory_order_relaxed);
  return e;
}

hipError_t launch_topk_collect(const IndexArgs& a, const TopkWs& ws, int slices, int slice_len,
                               hipStream_t s) {
  CSA_LAUNCH("topk_collect", topk_collect_kernel, dim3(slices, a.B * a.Tq), dim3(kCT), 0, s, a, ws,
             slice_len);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  static std::atomic<size_t> lds_set[kMaxDevices];
  e = allow_lds(topk_resolve_kernel, sizeof(Lds), lds_set);
  if (e != hipSuccess) return e;
  CSA_LAUNCH("topk_resolve", topk_resolve_kernel, dim3(a.B * a.Tq), dim3(kRT), sizeof(Lds), s, a, ws);
  return hipGetLastError();
}

hipError_t launch_topk_fused_resolve(const IndexArgs& a, const TopkWs& ws, int n_wg, hipStream_t s) {
  static std::atomic<size_t> lds_set[kMaxDevices];
  hipError_t e = allow_lds(topk_fused_resolve_kernel, sizeof(Lds), lds_set);
  if (e != hipSuccess) return e;
  CSA_LAUNCH("topk_resolve", topk_fused_resolve_kernel, dim3(a.B * a.Tq), dim3(kRT), sizeof(Lds), s, a, ws, n_wg);
  return hipGetLastError();
}

hipError_t launch_topk_rows(const IndexArgs& a, const TopkWs& ws, hipStream_t s) {
  static std::atomic<size_t> lds_set[kMaxDevices];
  hipError_t e = allow_lds(topk_rowsel_kernel, sizeof(Lds), lds_set);
  if (e != hipSuccess) return e;
  CSA_LAUNCH("topk_rows", topk_rowsel_kernel, dim3(a.B * a.Tq), dim3(kRT), sizeof(Lds), s, a, ws);
  return hipGetLastError();
}

}  // namespace csa
