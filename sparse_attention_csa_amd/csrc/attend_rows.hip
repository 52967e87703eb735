// Sparse (top-k) attention on MFMA with the rows of a split divided among
// the wavefronts: rows a4 + a6 of the hot path.
//
// What it computes is the generic kernel's result: for a query at position t
// and every head h, one softmax over the query's selected compressed entries
// and its window rows, exp(sink_h) in the denominator ("DeepSeek-V4" book
// ch. 6 "Shared key-value MQA", ch. 7 "The sliding window" and "Attention
// sinks"; "2026 DeepSeek-V4" note, concat(selected, local_kv)).  Every row is
// both key and value.
//
// Work split.  A workgroup owns one query, 16 heads and a contiguous range
// of the query's rows (a "split"; the splits are merged by
// attend_merge_kernel).  The range is cut into 16-row tiles and tile j
// belongs to wavefront j % 4: each wavefront runs its own pipeline (two LDS
// slots, direct global-to-LDS DMA of the gathered rows, no workgroup
// barrier) and the four partial softmax states are combined through LDS at
// the end.  When a split has at most kBufs tiles (144 rows: the Pro-shaped
// decode's splits) every tile has its own LDS buffer and a wavefront issues
// the DMAs of all its tiles at once, so the split waits for one gather round
// trip instead of one per tile; longer splits run a two-slot ring per
// wavefront.  With only 16 heads per workgroup a split's partial output is
// 16 KB, which keeps the merge traffic small next to the gathered rows; the
// head groups of one (query, split) run on the same XCD and share its L2.
//
// Per tile (16 rows):
//   S^T[16 rows x 16 heads] = K . Q^T            16 x v_mfma 16x16x32 bf16
//   weights p = exp2(S sc - m_ref)               fixed reference max, below
//   O^T[512 d x 16 heads] += V^T . P^T           32 x v_mfma 16x16x16 bf16
// The S^T accumulator layout (lane = head, rows 4g..4g+3 in lane group g) is
// the B operand of the 16x16x16 product as it stands; V^T comes from the
// same LDS tile through ds_read_b64_tr_b16.

#include "kernels.h"
#include "mfma_tile.h"

namespace csa {

using namespace tile;

namespace {

constexpr int kTR = 16;                      // rows per tile
constexpr int kTileB = kTR * kRowB;          // 16 KB
constexpr int kSlots = 2;                    // LDS slots per wavefront (ring mode)
constexpr int kBufs = 9;                     // tile buffers in LDS (144 KB)
constexpr int kMaxRows = 2304;               // rows per split (k + n_win <= 2048 + 256)
constexpr int kFill = kMaxRows / 256;        // row-source loads per thread

}  // namespace

// 1-D grid: block L runs on XCD L % 8; the n_hg head groups of one (query,
// split) are blocks L, L + 8, ... so they gather the same rows through one L2.
// DEROT: the output's rotary coordinates are rotated back by the query
// position (norm_rope); PG: the cache is paged (the selected entries' cache
// rows are read from the block table before the row DMAs start).  Separate
// instantiations leave the default one as it was.
template <int DEROT, int PG>
__global__ __launch_bounds__(256, 1) void attend_rows_kernel(AttendArgs a, int n_split, int rows_per_split) {
  // tile buffers: tile j of the split in buffer j when the split has at
  // most kBufs tiles, else buffers 2w, 2w+1 are wavefront w's ring; reused as
  // the epilogue's staging area
  __shared__ __attribute__((aligned(1024))) char bufs[kBufs][kTileB];
  // source of each row of the split: >= 0 cache entry, -1 none (masked),
  // <= -2 window ring row (-2 - ring row)
  __shared__ __attribute__((aligned(16))) int rsrc[kMaxRows];
  __shared__ float s_m[4][16], s_l[4][16];

  const int n_hg = a.H / 16;
  const int L = blockIdx.x;
  const int xcd = L & 7, kk = L >> 3;
  const int hg = kk % n_hg;
  const int rest = (kk / n_hg) * 8 + xcd;
  const int split = rest % n_split, qrow = rest / n_split;
  if (qrow >= a.B * a.Tq) return;

  const int b = qrow / a.Tq;
  const int tid = threadIdx.x, l = tid & 63, li = l & 15, lg = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = a.H;
  const int h0 = hg * 16;

  // the scalar inputs, the split's selected ids (loads kept inside the
  // query's k-entry list) and Q are requested together
  const int64_t* dummy64 = reinterpret_cast<const int64_t*>(a.kv);
  const int64_t t_ld = (a.q_pos ? a.q_pos + qrow : dummy64)[0];
  const int64_t w_ld = (a.win_pos0 ? a.win_pos0 + b : dummy64)[0];
  const int32_t cnt = a.topk_cnt[qrow];
  const int r_begin = split * rows_per_split;
  int32_t v[kFill];
  {
    const int32_t* ids = a.topk_idx + (size_t)qrow * a.k;
#pragma unroll
    for (int u = 0; u < kFill; ++u) {
      const int j = r_begin + tid + 256 * u;
      v[u] = ids[j < a.k ? j : a.k - 1];
    }
  }
  // Q^T operands for the 16 heads: lane (head li, d group lg)
  bf16x8_t qf[16];
  {
    const uint16_t* q = reinterpret_cast<const uint16_t*>(a.q) + ((size_t)qrow * H + h0 + li) * kC + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) qf[ks] = *reinterpret_cast<const bf16x8_t*>(q + 32 * ks);
  }
  // one wait for all of it: no other global load is in flight once the
  // row DMAs start, so the loop's waits count DMAs only
  __builtin_amdgcn_s_waitcnt(0);
  __asm__ __volatile__("" ::"s"(t_ld), "s"(w_ld), "s"(cnt), "v"(qf[0]), "v"(qf[15]), "v"(v[0]), "v"(v[kFill - 1]));
  const int64_t t = a.q_pos ? t_ld : a.q_pos0 + qrow % a.Tq;
  const int64_t wpos0 = a.win_pos0 ? w_ld : a.win_pos0_const;
  const int n_c = cnt < 0 ? 0 : (cnt > a.k ? a.k : cnt);
  const int64_t n_w = (t + 1) < a.n_win ? (t + 1) : a.n_win;
  const int n_rows = n_c + (int)n_w;
  const int r_end = r_begin + rows_per_split < n_rows ? r_begin + rows_per_split : n_rows;
  const int n_tiles = r_end > r_begin ? (r_end - r_begin + kTR - 1) / kTR : 0;
  const uint16_t* kv = reinterpret_cast<const uint16_t*>(a.kv) + (PG ? 0 : (size_t)b * a.E_cap * kC);
  const uint16_t* win = reinterpret_cast<const uint16_t*>(a.win) + (size_t)b * a.W_cap * kC;
  const float sc2 = a.scale * kLog2e;
  // ring row of the first window position (32-bit remainder when it fits)
  const int64_t wofs = t - n_w + 1 - wpos0;
  int wbase;
  if (wofs >= 0 && wofs < 0x7fffffff) {
    wbase = (int)((uint32_t)wofs % (uint32_t)a.W_cap);
  } else {
    int64_t wb = wofs % a.W_cap;
    if (wb < 0) wb += a.W_cap;
    wbase = (int)wb;
  }
  const int wcap = a.W_cap;
  // the query's own window row: always present, the source of masked rows
  int own = wbase + (int)n_w - 1;
  if (own >= wcap) own -= wcap;

  if constexpr (PG) {
    // the selected entries' cache rows (pool rows < 2^31), one round of
    // block-table loads for all of them (an id outside [0, E_cap) reads the
    // sequence's first page id and becomes -1)
    const int sh = a.pg.shift;
    const int32_t* tb = a.pg.table + (size_t)b * (a.E_cap >> sh);
    int32_t pid[kFill];
#pragma unroll
    for (int u = 0; u < kFill; ++u) pid[u] = tb[(v[u] >= 0 && v[u] < a.E_cap) ? (v[u] >> sh) : 0];
#pragma unroll
    for (int u = 0; u < kFill; ++u)
      v[u] = (v[u] >= 0 && v[u] < a.E_cap) ? (int)(((uint32_t)pid[u] << sh) + (uint32_t)(v[u] & ((1 << sh) - 1))) : -1;
  }
  // row sources of the split
  {
#pragma unroll
    for (int u = 0; u < kFill; ++u) {
      const int jr = tid + 256 * u;
      if (jr < rows_per_split) {
        const int j = r_begin + jr;
        int e = -1;
        if (j < n_c) {
          if constexpr (PG)
            e = v[u];  // already the cache row, or -1
          else
            e = (v[u] >= 0 && v[u] < a.E_cap) ? v[u] : -1;
        } else if (j < r_end) {
          int wr = wbase + (j - n_c);
          if (wr >= wcap) wr -= wcap;
          e = -2 - wr;
        }
        rsrc[jr] = e;
      }
    }
  }

  lds_barrier();  // rsrc ready

  const int n_mine = n_tiles > w ? (n_tiles - w + 3) / 4 : 0;  // tiles j = w + 4i
  const bool all_in = n_tiles <= kBufs;  // every tile in its own buffer
  // buffer of this wavefront's i-th tile
  auto buf_of = [&](int i) -> char* { return all_in ? bufs[w + 4 * i] : bufs[kSlots * w + (i & 1)]; };

  const Bases bs = lane_bases(li, lg);
  f32x4_t acc[32];
  float m_run = -INFINITY, l_lane = 0.f;

  // DMA of this wavefront's i-th tile into slot sl.  Lane r (mod 16)
  // computes the source of tile row r; each DMA takes its row's address from
  // that lane (two lane reads) and a per-lane chunk offset fixed for the
  // kernel.
  int dofs[kTR];  // element offset of this lane's 16-byte chunk, per tile row
#pragma unroll
  for (int r = 0; r < kTR; ++r) dofs[r] = 8 * (l ^ swz(r));
  auto issue = [&](int i) {
    const int er = rsrc[(w + 4 * i) * kTR + (l & (kTR - 1))];
    const int row = er >= 0 ? er : (er == -1 ? own : -2 - er);
    const uint16_t* src = (er >= 0 ? kv : win) + (size_t)row * kC;
    const uintptr_t sp = reinterpret_cast<uintptr_t>(src);
    const uint32_t s_lo = (uint32_t)sp, s_hi = (uint32_t)(sp >> 32);
    const uint32_t dst = lds_addr(buf_of(i));
#pragma unroll
    for (int r = 0; r < kTR; ++r) {
      // (readlane returns int: widen through uint32_t, no sign extension)
      const uint64_t ri = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(s_hi, r) << 32) |
                          (uint64_t)(uint32_t)__builtin_amdgcn_readlane(s_lo, r);
      dma16_m0(reinterpret_cast<const uint16_t*>(ri) + dofs[r], dst + r * kRowB);
    }
  };

  auto compute = [&](int i) {
    const char* T = buf_of(i);
    // S^T as two interleaved chains (even / odd k steps); fragment reads
    // run one group of four k steps ahead of the products
    f32x4_t s0 = f32x4_t{0.f, 0.f, 0.f, 0.f}, s1 = s0;
    {
      bf16x8_t kf[2][4];
#pragma unroll
      for (int u = 0; u < 4; ++u) kf[0][u] = lds8(T + bs.s[u]);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        if (g + 1 < 4) {
#pragma unroll
          for (int u = 0; u < 4; ++u) kf[(g + 1) & 1][u] = lds8(T + bs.s[u] + 256 * (g + 1));
        }
        s0 = mfma32(kf[g & 1][0], qf[4 * g], s0);
        s1 = mfma32(kf[g & 1][1], qf[4 * g + 1], s1);
        s0 = mfma32(kf[g & 1][2], qf[4 * g + 2], s0);
        s1 = mfma32(kf[g & 1][3], qf[4 * g + 3], s1);
      }
    }
    // row validity of this lane's rows 4lg .. 4lg+3
    const int jr = (w + 4 * i) * kTR + 4 * lg;
    const int4 ev = *reinterpret_cast<const int4*>(rsrc + jr);
    const int evs[4] = {ev.x, ev.y, ev.z, ev.w};
    // softmax weights against a fixed reference max per head (the first
    // tile's); a tile max above it by more than kSlack (log2 units) raises
    // it and this wavefront redoes its tiles (at most once: the second pass
    // starts from the largest max of the first)
    float x[4];
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool ok = evs[u] != -1 && r_begin + jr + u < r_end;
      x[u] = ok ? (s0[u] + s1[u]) * sc2 : -INFINITY;
      mx = fmaxf(mx, x[u]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const bool jump = m_run != -INFINITY && mx > m_run + kSlack;
    const bool redo = __builtin_amdgcn_ballot_w64(jump) != 0ull;
    if (m_run == -INFINITY || jump) m_run = mx;
    float p[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      p[u] = (x[u] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(x[u] - m_run);
      l_lane += p[u];
    }
    const bf16x4_t pb = bf16x4_t{(__bf16)p[0], (__bf16)p[1], (__bf16)p[2], (__bf16)p[3]};
    const i16x4_t pB = __builtin_bit_cast(i16x4_t, pb);
    // value reads one group of eight d blocks ahead of the products
    {
      i16x4_t vt[2][8];
#pragma unroll
      for (int u = 0; u < 8; ++u) vt[0][u] = ld_tr(T + bs.t[u]);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        if (g + 1 < 4) {
#pragma unroll
          for (int u = 0; u < 8; ++u) vt[(g + 1) & 1][u] = ld_tr(T + bs.t[u] + 256 * (g + 1));
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) acc[8 * g + u] = mfma16(vt[g & 1][u], pB, acc[8 * g + u]);
      }
    }
    return redo;
  };

  // this wavefront's tiles.  All in: every DMA issued up front, tile i
  // computed once its own DMAs (and the older ones) have landed.  Ring: tile
  // i computed while tile i+1 is in flight.  The waits are explicit (the
  // DMAs are the only memory operations in flight here; the empty asm
  // statements keep LDS reads behind them).
  static_assert(kBufs / 4 * kTR <= 63 - kTR, "DMAs in flight must fit the vmcnt counter");
  for (;;) {
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) acc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    l_lane = 0.f;
    bool redo = false;
    if (all_in) {
      for (int i = 0; i < n_mine; ++i) issue(i);
      for (int i = 0; i < n_mine; ++i) {
        const int younger = n_mine - 1 - i;  // tiles issued after tile i (at most 2)
        if (younger >= 2) __builtin_amdgcn_s_waitcnt(wait_vm(2 * kTR));
        else if (younger == 1) __builtin_amdgcn_s_waitcnt(wait_vm(kTR));
        else __builtin_amdgcn_s_waitcnt(wait_vm(0));
        __asm__ __volatile__("" ::: "memory");
        redo |= compute(i);
      }
    } else {
      if (n_mine > 0) issue(0);
      if (n_mine > 1) issue(1);
      for (int i = 0; i < n_mine; ++i) {
        if (i + 1 < n_mine) __builtin_amdgcn_s_waitcnt(wait_vm(kTR));
        else __builtin_amdgcn_s_waitcnt(wait_vm(0));
        __asm__ __volatile__("" ::: "memory");
        redo |= compute(i);
        if (i + 2 < n_mine) {
          __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // this slot's reads are done
          __asm__ __volatile__("" ::: "memory");
          issue(i + 2);
        }
      }
    }
    if (!redo) break;
    // a redo re-fetches this wavefront's tiles into the same buffers: its own
    // reads of them are done (LDS operations complete in order)
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __asm__ __volatile__("" ::: "memory");
  }

  // combine the four wavefronts' states: per head the max of the reference
  // maxima M, each wavefront's O^T scaled by exp2(m_w - M)
  float Lw = l_lane;
  Lw += __shfl_xor(Lw, 16, 64);
  Lw += __shfl_xor(Lw, 32, 64);
  if (lg == 0) {
    s_m[w][li] = m_run;
    s_l[w][li] = Lw;
  }
  __syncthreads();  // every wavefront is done with its slots
  float M = -INFINITY;
#pragma unroll
  for (int v = 0; v < 4; ++v) M = fmaxf(M, s_m[v][li]);
  const float fw = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - M);
  // staging: wavefront v's head row h (512 floats, 2 KB) at
  // red(v) + 2048 h, its 16-byte chunk c at position c ^ h (conflict-free
  // for both access patterns)
  auto red = [&](int v) -> char* { return bufs[2 * v]; };  // 32 KB per wavefront
  {
    char* rw = red(w) + li * 2048;
#pragma unroll
    for (int dt = 0; dt < 32; ++dt)
      *reinterpret_cast<f32x4_t*>(rw + 16 * ((4 * dt + lg) ^ li)) = acc[dt] * fw;
  }
  __syncthreads();

  // wavefront w writes heads 4w .. 4w+3; lane l has d = 8l .. 8l+7
  float* pml = reinterpret_cast<float*>(a.ws);
  uint16_t* po = reinterpret_cast<uint16_t*>(pml + (size_t)a.B * a.Tq * n_split * H * 2);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int hh = 4 * w + j, h = h0 + hh;
    float Mh = -INFINITY;
#pragma unroll
    for (int v = 0; v < 4; ++v) Mh = fmaxf(Mh, s_m[v][hh]);
    float Lh = 0.f;
#pragma unroll
    for (int v = 0; v < 4; ++v)
      if (s_m[v][hh] != -INFINITY) Lh += s_l[v][hh] * __builtin_amdgcn_exp2f(s_m[v][hh] - Mh);
    // lane l: d = 4l .. 4l+3 (chunk l) and 256 + 4l .. (chunk 64 + l)
    f32x4_t o0 = f32x4_t{0.f, 0.f, 0.f, 0.f}, o1 = o0;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const char* rr = red(v) + hh * 2048;
      o0 += *reinterpret_cast<const f32x4_t*>(rr + 16 * (l ^ hh));
      o1 += *reinterpret_cast<const f32x4_t*>(rr + 16 * ((64 + l) ^ hh));
    }
    float f;
    uint16_t* dst;
    if (n_split == 1) {
      const float z2 = a.sink ? a.sink[h] * kLog2e : -INFINITY;
      const float Mf = fmaxf(Mh, z2);
      const float em = Mh == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(Mh - Mf);
      const float den = Lh * em + (z2 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(z2 - Mf));
      f = em / den;
      if (a.lse && l == 0) a.lse[(size_t)qrow * H + h] = (Mf + log2f(den)) * kLn2;
      dst = reinterpret_cast<uint16_t*>(a.out) + ((size_t)qrow * H + h) * kC;
    } else {
      const size_t slot = ((size_t)qrow * n_split + split) * H + h;
      if (l == 0) {
        pml[2 * slot] = Mh;
        pml[2 * slot + 1] = Lh;
      }
      f = Lh > 0.f ? __builtin_amdgcn_rcpf(Lh) : 0.f;
      dst = po + slot * kC;
    }
    float x0[4] = {o0[0] * f, o0[1] * f, o0[2] * f, o0[3] * f};
    float x1[4] = {o1[0] * f, o1[1] * f, o1[2] * f, o1[3] * f};
    if (DEROT) {  // norm_rope: rotary coordinates rotated back by the query position
      rope_pairs<4>(x0, 4, 4 * l, kC, a.rope_dims, a.derot_freq, -t);
      rope_pairs<4>(x1, 4, 256 + 4 * l, kC, a.rope_dims, a.derot_freq, -t);
    }
    uint2 r0, r1;
    r0.x = (uint32_t)f32_to_bf16(x0[0]) | ((uint32_t)f32_to_bf16(x0[1]) << 16);
    r0.y = (uint32_t)f32_to_bf16(x0[2]) | ((uint32_t)f32_to_bf16(x0[3]) << 16);
    r1.x = (uint32_t)f32_to_bf16(x1[0]) | ((uint32_t)f32_to_bf16(x1[1]) << 16);
    r1.y = (uint32_t)f32_to_bf16(x1[2]) | ((uint32_t)f32_to_bf16(x1[3]) << 16);
    *reinterpret_cast<uint2*>(dst + 4 * l) = r0;
    *reinterpret_cast<uint2*>(dst + 256 + 4 * l) = r1;
  }
}

bool attend_rows_shape_ok(int H, int c) { return c == kC && H % 16 == 0; }

// Splits per (query, head group): about one workgroup per CU (256), each a
// multiple of the 16-row tile, at most kMaxRows rows and 64 splits; or
// split_rows rows each whatever the batch.
void attend_rows_plan(int BT, int H, int rows_max, int split_rows, int* n_split, int* rows_per_split) {
  if (split_rows > 0) {
    *rows_per_split = split_rows;
    *n_split = (rows_max + split_rows - 1) / split_rows;
    return;
  }
  const int cols = BT * (H / 16);
  int want = 256 / cols;
  if (want < 1) want = 1;
  if (want > 64) want = 64;
  int rps = (rows_max + want - 1) / want;
  rps = (rps + kTR - 1) / kTR * kTR;
  if (rps > kMaxRows) rps = kMaxRows;
  *rows_per_split = rps;
  *n_split = (rows_max + rps - 1) / rps;
}

hipError_t launch_attend_merge(const AttendArgs& a, int n_split, hipStream_t s);

hipError_t launch_attend_rows(const AttendArgs& a, int rows_max, hipStream_t s) {
  int ns, rps;
  attend_rows_plan(a.B * a.Tq, a.H, rows_max, a.split_rows, &ns, &rps);
  if (ns > 64) return hipErrorInvalidValue;
  const int n_hg = a.H / 16;
  const long long units = (long long)ns * a.B * a.Tq;   // (query, split) pairs
  const long long blocks = (units + 7) / 8 * 8 * n_hg;  // padded to whole XCD rounds
  // norm_rope: with row splits the merge rotates the output back
  const bool derot = a.derot_freq && ns == 1;
  if (a.pg.table && derot)
    CSA_LAUNCH("attend_sparse_rows", (attend_rows_kernel<1, 1>), dim3((unsigned)blocks), dim3(256), 0, s, a, ns, rps);
  else if (a.pg.table)
    CSA_LAUNCH("attend_sparse_rows", (attend_rows_kernel<0, 1>), dim3((unsigned)blocks), dim3(256), 0, s, a, ns, rps);
  else if (derot)
    CSA_LAUNCH("attend_sparse_rows", (attend_rows_kernel<1, 0>), dim3((unsigned)blocks), dim3(256), 0, s, a, ns, rps);
  else
    CSA_LAUNCH("attend_sparse_rows", (attend_rows_kernel<0, 0>), dim3((unsigned)blocks), dim3(256), 0, s, a, ns, rps);
  if (ns > 1) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_attend_merge(a, ns, s);
  }
  return hipGetLastError();
}

}  // namespace csa
