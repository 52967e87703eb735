// Dense (HCA) shared-KV attention on MFMA (bf16, entry dim 512): rows a5 +
// a6 of the hot path.
//
// What it computes is the generic kernel's result: for a query at position t
// and every head h, one softmax over all visible compressed entries and the
// window rows, with exp(sink_h) in the denominator ("DeepSeek-V4" book ch. 6
// "Shared key-value MQA", ch. 7 "The sliding window" and "Attention sinks").
// Every row is both key and value.
//
// Work split.  A workgroup (4 wavefronts, one per SIMD, the whole register
// file) owns one query, 64 heads (16 per wavefront) and a contiguous range of
// its rows ("split"); the splits of one query are merged by
// attend_merge_kernel with the online-softmax rule.  Every wavefront consumes
// every row of a tile, so a row crosses HBM / L2 into LDS once per split, not
// once per head group.  Row tiles of 32 rows (32 KB) are fetched into LDS by
// direct global-to-LDS DMA (one 1 KB row per wave instruction) into a ring of
// four slots: three tiles are in flight while one is computed.
//
// Tied K = V on MFMA.  The score product is computed transposed,
//   S^T[rows x heads] = K[rows x d] . Q^T[d x heads]   (v_mfma 16x16x32 bf16),
// with Q^T held in registers and K read row-major from LDS.  The accumulator
// layout of S^T (lane = head, 4 consecutive rows per lane group) is, after
// exp2 and a bf16 cast, the B operand of
//   O^T[d x heads] += V^T[d x rows] . P^T[rows x heads]  (16x16x32 bf16)
// once the 32 reduction slots of a row pair (two 16-row blocks) are permuted
// consistently: slot 8g+i is row 4g+i of the first block for i < 4 and of
// the second for i >= 4.  V^T comes from the same LDS tile through the gfx950
// transpose read (ds_read_b64_tr_b16), whose per-lane addresses implement
// that permutation.  Softmax runs in base 2.
//
// Decode with the step's fold inside (fold_mode): the splits cover the
// entries that existed before the step; split s of head group 0 also folds
// coordinates [s cs, s cs + cs) of the entry the block ending at the query
// position completes (its sources are loaded after the row loop and arrive
// while the output is written; nothing of the fold stays live across the
// loop), stores them, adds its share of q_h . entry for every head
// to fold_s (device-scope atomics) and appends its share of the token to the
// tail and window rings.  The merge kernel then adds the new entry as one
// more row, weight exp2(scale q . entry - M), and publishes the entry count.
// The query's own window row is read from the step input x_new.

#include "fold.h"
#include "kernels.h"
#include "mfma_tile.h"

namespace csa {

using namespace tile;

namespace {

constexpr int kHW = 64;                // heads per workgroup (16 per wavefront)
constexpr int kTN = 32;                // rows per LDS tile
constexpr int kRing = 4;               // LDS tile slots: kRing - 1 tiles in flight while one is computed
constexpr int kRowsPerWave = kTN / 4;  // DMA instructions per wave and tile
constexpr int kFoldU = 4;              // fold slice: sources per thread (at most)

}  // namespace

// 1-D grid: block L runs on XCD L % 8; the n_hg head groups of one (query,
// split) are blocks L, L + 8, ... so they share that XCD's L2.
__global__ __launch_bounds__(256, 1) void attend_mfma_kernel(AttendArgs a, int n_split, int rows_per_split) {
  __shared__ __attribute__((aligned(1024))) char tiles[kRing][kTN * kRowB];
  __shared__ uint32_t rvalid[kRing][kTN / 4];  // byte r % 4 of word r / 4: row r is a real row
  __shared__ int s_restart;                // a wavefront asks the split to be recomputed
  __shared__ Soft s_fpart[4][64];          // fold: per-wavefront partial states of <= 64 coordinates
  __shared__ float s_fnew[64];             // fold: the new entry's coordinates (bf16-rounded)
  __shared__ float s_fx[64];               // fold: the token's coordinates
  __shared__ int s_fctx[8];                // fold: slice context kept over the row loop

  const int n_hg = a.H / kHW;
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
  const int h0 = hg * kHW + 16 * w;  // this wavefront's first head

  // Everything that depends only on the block index is requested at once
  // and awaited together (one memory round trip): the query operands and
  // the position, entry count and window base.  After that the row DMAs are
  // the only memory operations in flight, so the waits below count DMAs.
  // Q^T operands for this wavefront's 16 heads: lane (head li, d group lg).
  bf16x8_t qf[16];
  {
    const uint16_t* q = reinterpret_cast<const uint16_t*>(a.q) + ((size_t)qrow * H + h0 + li) * kC + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) qf[ks] = *reinterpret_cast<const bf16x8_t*>(q + 32 * ks);
  }
  // (unconditional loads: an absent optional array is replaced by a valid
  // dummy address and the value discarded, so the three loads are in flight
  // together instead of one branch and wait each)
  const int64_t* dummy64 = reinterpret_cast<const int64_t*>(a.kv);
  const int64_t t_ld = (a.q_pos ? a.q_pos + qrow : dummy64)[0];
  const int64_t w_ld = (a.win_pos0 ? a.win_pos0 + b : dummy64)[0];
  const int32_t cnt = a.n_entries[b];
  __builtin_amdgcn_s_waitcnt(0);
  __asm__ __volatile__("" ::"s"(t_ld), "s"(w_ld), "s"(cnt), "v"(qf[0]), "v"(qf[15]));
  const int64_t t = a.q_pos ? t_ld : a.q_pos0 + qrow % a.Tq;
  const int64_t wpos0 = a.win_pos0 ? w_ld : a.win_pos0_const;
  const int64_t lim = vis_limit(t, a.m, a.vis);
  const int64_t have = (int64_t)cnt + a.n_add;
  int64_t n_c = lim < have ? lim : have;
  if (n_c > a.E_cap) n_c = a.E_cap;
  if (n_c < 0) n_c = 0;
  const int64_t n_w = (t + 1) < a.n_win ? (t + 1) : a.n_win;
  // fold_mode: the query's own token is not in the window ring yet; the
  // merge adds it as a row of its own
  const int64_t n_rows = n_c + n_w - (a.fold_mode ? 1 : 0);
  const int r_begin = split * rows_per_split;
  const int r_end = (int)((int64_t)r_begin + rows_per_split < n_rows ? r_begin + rows_per_split : n_rows);
  const int nc32 = (int)n_c;
  const uint16_t* kv = reinterpret_cast<const uint16_t*>(a.kv) + (size_t)b * a.E_cap * kC;
  const uint16_t* win = reinterpret_cast<const uint16_t*>(a.win) + (size_t)b * a.W_cap * kC;
  const float sc2 = a.scale * kLog2e;
  // ring row of the first window position; later window rows follow with
  // one conditional wrap (n_win <= W_cap).  32-bit remainder when the
  // offset fits (always, for positions below 2^31).
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
  // the query's own window row: always present, the source of padding rows
  // (their logits are masked)
  int own = wbase + (int)n_w - 1;
  if (own >= wcap) own -= wcap;
  const uint16_t* pad_row = win + (size_t)own * kC;

  // fold slice (fold_mode, head group 0): coordinates [fr0, fr0 + fW) of
  // the entry completed by the block ending at t (entry lim - 1, stored
  // only if it is the next one: fold_now).  Its context waits in LDS and
  // its loads are issued after the row loop, so that none of it occupies
  // registers during the loop.
  if (a.fold_mode && tid == 0) {
    const int fcs = a.fold_cs, fr0 = split * fcs;
    s_fctx[0] = hg == 0 ? (a.c - fr0 < 0 ? 0 : (a.c - fr0 < fcs ? a.c - fr0 : fcs)) : 0;
    s_fctx[1] = fr0;
    s_fctx[2] = lim == (int64_t)cnt + 1 && cnt < a.E_cap;
    s_fctx[3] = cnt;
    s_fctx[4] = (int)(uint32_t)t;
    s_fctx[5] = (int)(t >> 32);
  }

  if (tid == 0) s_restart = 0;
  __syncthreads();  // s_restart ready

  auto row_src = [&](int j, bool* ok) -> const uint16_t* {
    *ok = false;
    if (j >= r_end) return pad_row;
    if (j < nc32) {
      *ok = true;
      return kv + (size_t)j * kC;
    }
    int wr = wbase + (j - nc32);
    if (wr >= wcap) wr -= wcap;
    *ok = true;
    return win + (size_t)wr * kC;
  };
  // wave w fetches rows kRowsPerWave * w .. of a tile; every wave reads all rows
  auto issue_tile = [&](int r0, int buf) {
    uint32_t vw = 0;
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      const int r = kRowsPerWave * w + i;
      bool ok;
      const uint16_t* src = row_src(r0 + r, &ok);
      dma_row_m0(src, lds_addr(tiles[buf] + r * kRowB), l, swz(r & 15));
      vw |= (uint32_t)ok << (8 * (i & 3));
      if ((i & 3) == 3) {
        if (l == 0) rvalid[buf][r >> 2] = vw;
        vw = 0;
      }
    }
  };

  // the first kRing - 1 tiles
  auto prologue = [&]() {
#pragma unroll
    for (int j = 0; j < kRing - 1; ++j)
      if (r_begin + j * kTN < r_end) issue_tile(r_begin + j * kTN, j);
  };
  prologue();

  // running softmax state: the reference max per head (identical in the 4
  // lane groups), the sum per lane over its own rows, O^T[512 d x 16 heads]
  f32x4_t acc[32];
#pragma unroll
  for (int dt = 0; dt < 32; ++dt) acc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_lane = 0.f;

  // per-lane LDS byte offsets of the score and value reads
  const Bases bs = lane_bases(li, lg);
  const int* s_base = bs.s;
  const int* t_base = bs.t;

  auto compute_tile = [&](int buf) {
    const char* T = tiles[buf];
    // S^T[32 rows x 16 heads] = K . Q^T as two 16-row blocks
    // (the block chains interleave, so consecutive MFMAs are independent)
    constexpr int kRB = kTN / 16;
    f32x4_t s[kRB];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) s[rb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 16; ++ks)
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb)
        s[rb] = mfma32(lds8(T + s_base[ks & 3] + rb * 16 * kRowB + 256 * (ks >> 2)), qf[ks], s[rb]);
    // keep 12 fragment reads in flight ahead of the MFMAs (lgkmcnt counts 15)
    __builtin_amdgcn_sched_group_barrier(0x100, 12, 1);
#pragma unroll
    for (int i = 0; i < 16 * kRB - 12; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 12, 1);
    // softmax weights against a fixed reference max per head; lane holds
    // rows 16rb + 4lg + i of head li.  The reference is the first tile's max
    // and stays put while tile maxima exceed it by at most kSlack (log2
    // units), so weights stay <= 2^kSlack and the accumulator is never
    // rescaled.  A larger jump raises the reference and asks for the split
    // to be recomputed from its first row (at most once: the second pass
    // starts from the largest max of the first).
    float x[kRB][4];
    float mx = -INFINITY;
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      const uint32_t fl = rvalid[buf][4 * rb + lg];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[rb][i] = ((fl >> (8 * i)) & 1u) ? s[rb][i] * sc2 : -INFINITY;
        mx = fmaxf(mx, x[rb][i]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const bool jump = m_run != -INFINITY && mx > m_run + kSlack;
    if (__builtin_amdgcn_ballot_w64(jump) != 0ull && l == 0) s_restart = 1;
    if (m_run == -INFINITY || jump) m_run = mx;  // no weight so far, or a pass to be redone
    bf16x4_t pb[kRB];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = (x[rb][i] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(x[rb][i] - m_run);
        l_lane += p[i];
      }
      pb[rb] = bf16x4_t{(__bf16)p[0], (__bf16)p[1], (__bf16)p[2], (__bf16)p[3]};
    }
    // O^T[d x heads] += V^T[d x 32 rows] . P^T[32 rows x heads] per row pair
#pragma unroll
    for (int pr = 0; pr < kRB / 2; ++pr) {
      const bf16x8_t pB = __builtin_shufflevector(pb[2 * pr], pb[2 * pr + 1], 0, 1, 2, 3, 4, 5, 6, 7);
      const char* vp = T + pr * 32 * kRowB;
#pragma unroll
      for (int dt = 0; dt < 32; ++dt) {
        const char* v0 = vp + t_base[dt & 7] + 256 * (dt >> 3);
        acc[dt] = mfma32(cat8(ld_tr(v0), ld_tr(v0 + 16 * kRowB)), pB, acc[dt]);
      }
    }
    // keep 7 MFMAs' worth of transpose reads in flight
    __builtin_amdgcn_sched_group_barrier(0x100, 14, 2);
#pragma unroll
    for (int i = 0; i < 32 * (kRB / 2) - 7; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 2);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 2);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 7, 2);
  };

  // ring of kRing tile slots, one barrier per tile: a wave first waits for
  // its own DMAs of tile i (the younger tiles i+1, i+2 may stay in flight);
  // after the barrier every wave's DMAs of tile i have landed and every wave
  // has finished tile i-1, so tile i+kRing-1 may be fetched into that slot
  // while tile i is computed.
  static_assert(kRing == 4, "the waits below assume two younger tiles");
  for (;;) {
    int buf = 0;
    for (int r0 = r_begin; r0 < r_end; r0 += kTN) {
      const int younger = (r_end - r0 - 1) / kTN;  // tiles after this one
      if (younger >= 2) __builtin_amdgcn_s_waitcnt(wait_vm(2 * kRowsPerWave));
      else if (younger == 1) __builtin_amdgcn_s_waitcnt(wait_vm(kRowsPerWave));
      else __builtin_amdgcn_s_waitcnt(wait_vm(0));
      lds_barrier();
      const int rn = r0 + (kRing - 1) * kTN;
      if (rn < r_end) issue_tile(rn, (buf + kRing - 1) & (kRing - 1));
      compute_tile(buf);
      buf = (buf + 1) & (kRing - 1);
    }
    lds_barrier();
    const int again = s_restart;
    if (!again) break;
    // recompute the split against the raised reference maxima
    lds_barrier();
    if (tid == 0) s_restart = 0;
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) acc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    l_lane = 0.f;
    prologue();
  }

  // fold slice loads, in flight while the output is written.  The fold's
  // arguments are read through the kernel-argument segment behind a
  // compiler barrier, so they are not held in registers over the loop.
  typedef const __attribute__((address_space(4))) AttendArgs KArgs;
  KArgs* ka = (KArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  __asm__ __volatile__("" : "+s"(ka));
  KArgs& A = *ka;
  const __attribute__((address_space(4))) FoldArgs& F = A.fold;
  const int fW = A.fold_mode ? __builtin_amdgcn_readfirstlane(s_fctx[0]) : 0;
  const int fr0 = __builtin_amdgcn_readfirstlane(s_fctx[1]);
  const bool fold_now = fW > 0 && __builtin_amdgcn_readfirstlane(s_fctx[2]) != 0;
  const int32_t fcnt = __builtin_amdgcn_readfirstlane(s_fctx[3]);
  const int64_t ft = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane(s_fctx[5]) << 32) |
                               (uint32_t)__builtin_amdgcn_readfirstlane(s_fctx[4]));
  // Thread (source group fj, coordinates fr0 + 8 fo ..) takes sources
  // fj + fG u; fq: q_h over 4 coordinates for group g = tid + 256 u (head,
  // 4 coordinates).
  const int fTR = fW > 0 ? A.fold_cs / 8 : 1, fG = 256 / fTR;
  const int fj = tid / fTR, fo = tid % fTR;
  uint4 fz[kFoldU], fx[kFoldU];
  float4 fb[kFoldU][2];
  uint2 fq[4];
  uint4 fapp = uint4{0, 0, 0, 0};
#pragma unroll
  for (int u = 0; u < kFoldU; ++u) {
    fz[u] = fx[u] = uint4{0, 0, 0, 0};
    fb[u][0] = fb[u][1] = float4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) fq[u] = uint2{0, 0};
  const uint16_t* io = reinterpret_cast<const uint16_t*>(F.streams) + (size_t)b * 2 * A.c;
  if (fW > 0) {
    if (fold_now && fo * 8 < fW) {
      const int64_t p0 = (int64_t)fcnt * F.m;  // first source token (entry fcnt)
      const int slot0 = (int)(p0 % F.R);
      const uint16_t* tl = reinterpret_cast<const uint16_t*>(F.tail) + (size_t)b * 2 * F.R * A.c;
      const int cc = fr0 + fo * 8;
#pragma unroll
      for (int u = 0; u < kFoldU; ++u) {
        const int j = fj + fG * u;
        if (j < F.m) {
          int slot = slot0 + j;
          if (slot >= F.R) slot -= F.R;
          const bool cur = p0 + j == ft;  // the current token is not in the tail yet
          fz[u] = *reinterpret_cast<const uint4*>(cur ? io + A.c + cc : tl + ((size_t)F.R + slot) * A.c + cc);
          fx[u] = *reinterpret_cast<const uint4*>(cur ? io + cc : tl + (size_t)slot * A.c + cc);
          if (F.bias_a) {
            fb[u][0] = *reinterpret_cast<const float4*>(F.bias_a + (size_t)j * A.c + cc);
            fb[u][1] = *reinterpret_cast<const float4*>(F.bias_a + (size_t)j * A.c + cc + 4);
          }
        }
      }
    }
    {
      const int ng = H * fW / 4;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int g = tid + 256 * u;
        if (g < ng) {
          const int hh = g / (fW / 4), c4 = g % (fW / 4);
          fq[u] = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(A.q) +
                                                  ((size_t)qrow * H + hh) * kC + fr0 + 4 * c4);
        }
      }
    }
    // the token's share for the rings: x_new, then streams 0 and 1 (8 coordinates each)
    if (tid < 3 * fW / 8) {
      const int which = tid / (fW / 8), cc = fr0 + 8 * (tid % (fW / 8));
      const uint16_t* src = which == 0 ? reinterpret_cast<const uint16_t*>(F.x_new) + (size_t)b * A.c + cc
                                       : io + (size_t)(which - 1) * A.c + cc;
      fapp = *reinterpret_cast<const uint4*>(src);
    }
  }

  // per-head sum over the four lane groups
  float Lh = l_lane;
  Lh += __shfl_xor(Lh, 16, 64);
  Lh += __shfl_xor(Lh, 32, 64);
  const int h = h0 + li;

  // Output rows leave through LDS so that every store instruction writes one
  // contiguous 1 KB row: lane (head li) holds d = 16dt + 4lg + i of O^T; it
  // writes them scaled and rounded to row li of its wavefront's [16][520]
  // bf16 staging block (row stride 1040 B keeps the 8-byte writes of 32
  // lanes on distinct banks), then lane l copies 16 bytes of each row.
  float f;  // output scale for this lane's head
  uint16_t* dst_row0;  // row of this wavefront's first head
  const size_t ostride = kC;
  if (n_split == 1) {
    const float z2 = a.sink ? a.sink[h] * kLog2e : -INFINITY;
    const float M = fmaxf(m_run, z2);
    const float em = m_run == -INFINITY ? 0.f : exp2f(m_run - M);
    const float den = Lh * em + (z2 == -INFINITY ? 0.f : exp2f(z2 - M));
    f = em / den;
    if (a.lse && lg == 0) a.lse[(size_t)qrow * H + h] = (M + log2f(den)) * kLn2;
    dst_row0 = reinterpret_cast<uint16_t*>(a.out) + ((size_t)qrow * H + h0) * kC;
  } else {
    // partial: (m, L) and O / L in bf16
    float* pml = reinterpret_cast<float*>(a.ws);
    uint16_t* po = reinterpret_cast<uint16_t*>(pml + (size_t)a.B * a.Tq * n_split * H * 2);
    const size_t slot = ((size_t)qrow * n_split + split) * H + h;
    if (lg == 0) {
      pml[2 * slot] = m_run;
      pml[2 * slot + 1] = Lh;
    }
    f = Lh > 0.f ? 1.f / Lh : 0.f;
    dst_row0 = po + (((size_t)qrow * n_split + split) * H + h0) * kC;
  }
  constexpr int kOutLD = kC + 8;  // staging row stride (elements)
  uint16_t* stage = reinterpret_cast<uint16_t*>(tiles[0]) + w * 16 * kOutLD;
#pragma unroll
  for (int dt = 0; dt < 32; ++dt) {
    ushort4 v;
    v.x = f32_to_bf16(acc[dt][0] * f);
    v.y = f32_to_bf16(acc[dt][1] * f);
    v.z = f32_to_bf16(acc[dt][2] * f);
    v.w = f32_to_bf16(acc[dt][3] * f);
    *reinterpret_cast<ushort4*>(stage + li * kOutLD + 16 * dt + 4 * lg) = v;
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // this wavefront's LDS writes (lgkmcnt 0)
#pragma unroll
  for (int r = 0; r < 16; ++r)
    *reinterpret_cast<uint4*>(dst_row0 + r * ostride + 8 * l) =
        *reinterpret_cast<const uint4*>(stage + r * kOutLD + 8 * l);

  if (fW > 0) {
    if (fold_now) {
      // merge the G = 256 / fTR source groups of each coordinate: in-thread
      // over its sources, lanes fo, fo + fTR, ... of a wavefront, then the
      // four wavefronts through LDS
      Soft st[8];
      {
        float lg_[kFoldU][8], xv[kFoldU][8];
        float mx[8];
#pragma unroll
        for (int v = 0; v < 8; ++v) mx[v] = -INFINITY;
#pragma unroll
        for (int u = 0; u < kFoldU; ++u) {
          const bool ok = fo * 8 < fW && fj + fG * u < F.m;
          float zz[8];
          unpack16(fz[u], (const bf16*)nullptr, zz);
          unpack16(fx[u], (const bf16*)nullptr, xv[u]);
          const float zb[8] = {fb[u][0].x, fb[u][0].y, fb[u][0].z, fb[u][0].w,
                               fb[u][1].x, fb[u][1].y, fb[u][1].z, fb[u][1].w};
#pragma unroll
          for (int v = 0; v < 8; ++v) {
            lg_[u][v] = ok ? zz[v] + zb[v] : -INFINITY;
            mx[v] = fmaxf(mx[v], lg_[u][v]);
          }
        }
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          float l_ = 0.f, acc_ = 0.f;
#pragma unroll
          for (int u = 0; u < kFoldU; ++u) {
            const float e_ = lg_[u][v] == -INFINITY ? 0.f : __expf(lg_[u][v] - mx[v]);
            l_ += e_;
            acc_ += e_ * xv[u][v];
          }
          st[v] = Soft{mx[v], l_, acc_};
        }
      }
      for (int msk = fTR; msk < 64; msk <<= 1) {
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          const Soft o{__shfl_xor(st[v].mx, msk, 64), __shfl_xor(st[v].l, msk, 64), __shfl_xor(st[v].acc, msk, 64)};
          st[v] = soft_merge(st[v], o);
        }
      }
      if (l < fTR) {
#pragma unroll
        for (int v = 0; v < 8; ++v)
          if (fo * 8 + v < 64) s_fpart[w][fo * 8 + v] = st[v];
      }
      lds_barrier();
      if (tid < fW) {
        Soft acc0 = s_fpart[0][tid];
#pragma unroll
        for (int g = 1; g < 4; ++g) acc0 = soft_merge(acc0, s_fpart[g][tid]);
        const uint16_t vb = f32_to_bf16(acc0.acc / acc0.l);
        s_fnew[tid] = bf16_to_f32(vb);
        reinterpret_cast<uint16_t*>(F.kv_cache)[((size_t)b * A.E_cap + fcnt) * kC + fr0 + tid] = vb;
        A.fold_new[(size_t)b * kC + fr0 + tid] = vb;
      }
    }
    // the token's coordinates (threads 0 .. fW / 8 - 1 hold x_new)
    if (tid < fW / 8) {
      float xv[8];
      unpack16(fapp, (const bf16*)nullptr, xv);
#pragma unroll
      for (int v = 0; v < 8; ++v) s_fx[8 * tid + v] = xv[v];
    }
    lds_barrier();
    // this slice's share of q_h . entry and q_h . token, summed over the
    // fW / 4 groups of a head
    const int gph = fW / 4, ng = H * gph;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int g = tid + 256 * u;
      if (256 * u < ng) {
        float pn = 0.f, po = 0.f;
        if (g < ng) {
          const int c4 = g % gph;
          const uint2 qv = fq[u];
          const float q0 = __uint_as_float(qv.x << 16), q1 = __uint_as_float(qv.x & 0xffff0000u);
          const float q2 = __uint_as_float(qv.y << 16), q3 = __uint_as_float(qv.y & 0xffff0000u);
          po = q0 * s_fx[4 * c4] + q1 * s_fx[4 * c4 + 1] + q2 * s_fx[4 * c4 + 2] + q3 * s_fx[4 * c4 + 3];
          if (fold_now)
            pn = q0 * s_fnew[4 * c4] + q1 * s_fnew[4 * c4 + 1] + q2 * s_fnew[4 * c4 + 2] + q3 * s_fnew[4 * c4 + 3];
        }
        for (int o = 1; o < gph; o <<= 1) {
          po += __shfl_xor(po, o, 64);
          pn += __shfl_xor(pn, o, 64);
        }
        if (g < ng && g % gph == 0) {
          float* fs = A.fold_s + 2 * ((size_t)b * H + g / gph);
          atomicAdd(fs + 1, po);
          if (fold_now) atomicAdd(fs, pn);
        }
      }
    }
    // the token's share of the rings (every step)
    if (tid < 3 * fW / 8) {
      const int which = tid / (fW / 8), cc = fr0 + 8 * (tid % (fW / 8));
      uint16_t* dst = which == 0
                          ? reinterpret_cast<uint16_t*>(F.win_ring) + ((size_t)b * F.n_win + ft % F.n_win) * A.c + cc
                          : reinterpret_cast<uint16_t*>(F.tail) + (((size_t)b * 2 + (which - 1)) * F.R + ft % F.R) * A.c + cc;
      *reinterpret_cast<uint4*>(dst) = fapp;
    }
    if (split == 0 && tid == 0) A.fold_row[b] = fold_now ? fcnt + 1 : 0;
  }
}

// grid (B*Tq, H), 256 threads: wavefront w merges splits w, w+4, ... of one
// head (lane = 8 coordinates), the four wavefronts add up through LDS.
constexpr int kMaxSplit = 64;
constexpr int kMergeU = kMaxSplit / 4;

__global__ __launch_bounds__(256) void attend_merge_kernel(AttendArgs a, int n_split) {
  __shared__ float s_o[4][64 * 8];
  __shared__ float s_den;
  const int qrow = blockIdx.x, h = blockIdx.y, tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int H = a.H;
  const float* pml = reinterpret_cast<const float*>(a.ws);
  const uint16_t* po = reinterpret_cast<const uint16_t*>(pml + (size_t)a.B * a.Tq * n_split * H * 2);
  const float z2 = a.sink ? a.sink[h] * kLog2e : -INFINITY;
  // fold_mode: the query's own token and the step's new entry (if any) as
  // two more rows, weights exp2(s_own - M) and exp2(s_new - M)
  const int b = qrow / a.Tq;
  const int frow = a.fold_mode ? a.fold_row[b] : 0;
  float2 fsv = float2{0.f, 0.f};
  if (a.fold_mode) fsv = *reinterpret_cast<const float2*>(a.fold_s + 2 * ((size_t)b * H + h));
  const float s_new = frow > 0 ? fsv.x * (a.scale * kLog2e) : -INFINITY;
  const float s_own = a.fold_mode ? fsv.y * (a.scale * kLog2e) : -INFINITY;
  // (fixed addresses: every load is issued at once)
  uint4 nrow = uint4{0, 0, 0, 0}, xrow = nrow;
  if (a.fold_mode) {
    nrow = *reinterpret_cast<const uint4*>(a.fold_new + (size_t)b * kC + 8 * l);
    xrow = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.fold.x_new) + (size_t)b * kC + 8 * l);
  }
  // lane s holds split s's statistics
  float ms = -INFINITY, Ls = 0.f;
  if (l < n_split) {
    const float2 v = *reinterpret_cast<const float2*>(pml + 2 * (((size_t)qrow * n_split + l) * H + h));
    ms = v.x;
    Ls = v.y;
  }
  const float M = fmaxf(fmaxf(fmaxf(wave_max(ms), z2), s_new), s_own);
  const float wgt = (ms == -INFINITY || Ls == 0.f) ? 0.f : exp2f(ms - M) * Ls;
  // this wavefront's splits: all loads first
  uint4 raw[kMergeU];
#pragma unroll
  for (int u = 0; u < kMergeU; ++u) {
    const int s = w + 4 * u;
    raw[u] = uint4{0, 0, 0, 0};
    if (s < n_split) {
      const size_t slot = ((size_t)qrow * n_split + s) * H + h;
      raw[u] = *reinterpret_cast<const uint4*>(po + slot * kC + 8 * l);
    }
  }
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < kMergeU; ++u) {
    const int s = w + 4 * u;  // < kMaxSplit = 64
    const float ws = __shfl(wgt, s, 64);
    if (s < n_split) {
      const uint32_t v[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o[2 * i] += ws * bf16_to_f32((uint16_t)(v[i] & 0xffff));
        o[2 * i + 1] += ws * bf16_to_f32((uint16_t)(v[i] >> 16));
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) s_o[w][8 * l + i] = o[i];
  const float w_new = frow > 0 ? exp2f(s_new - M) : 0.f;
  const float w_own = a.fold_mode ? exp2f(s_own - M) : 0.f;
  if (w == 0) {
    const float den = wave_sum(wgt) + (z2 == -INFINITY ? 0.f : exp2f(z2 - M)) + w_new + w_own;
    if (l == 0) s_den = den;
  }
  __syncthreads();
  if (w != 0) return;
  if (a.fold_mode && l == 0) {
    *reinterpret_cast<float2*>(a.fold_s + 2 * ((size_t)b * H + h)) = float2{0.f, 0.f};  // zero for the next call
    if (h == 0 && frow > 0) a.fold.n_entries[b] = frow;  // publish the new entry count
  }
  const float den = s_den;
  const float inv = 1.f / den;
  const uint32_t nw[4] = {nrow.x, nrow.y, nrow.z, nrow.w}, xw[4] = {xrow.x, xrow.y, xrow.z, xrow.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float nv = bf16_to_f32((uint16_t)((nw[i >> 1] >> (16 * (i & 1))) & 0xffff));
    const float xv = bf16_to_f32((uint16_t)((xw[i >> 1] >> (16 * (i & 1))) & 0xffff));
    // (the new entry's row holds old data when no entry was completed)
    o[i] = (s_o[0][8 * l + i] + s_o[1][8 * l + i] + s_o[2][8 * l + i] + s_o[3][8 * l + i] +
            (frow > 0 ? w_new * nv : 0.f) + w_own * xv) *
           inv;
  }
  uint16_t* out = reinterpret_cast<uint16_t*>(a.out) + ((size_t)qrow * H + h) * kC + 8 * l;
  uint4 r;
  r.x = (uint32_t)f32_to_bf16(o[0]) | ((uint32_t)f32_to_bf16(o[1]) << 16);
  r.y = (uint32_t)f32_to_bf16(o[2]) | ((uint32_t)f32_to_bf16(o[3]) << 16);
  r.z = (uint32_t)f32_to_bf16(o[4]) | ((uint32_t)f32_to_bf16(o[5]) << 16);
  r.w = (uint32_t)f32_to_bf16(o[6]) | ((uint32_t)f32_to_bf16(o[7]) << 16);
  *reinterpret_cast<uint4*>(out) = r;
  if (a.lse && l == 0) a.lse[(size_t)qrow * H + h] = (M + log2f(den)) * kLn2;
}

bool attend_mfma_shape_ok(int H, int c) { return c == kC && H % kHW == 0; }

size_t attend_fold_ws_offset(int B, int Tq, int H, int c, int rows_max);
void attend_mfma_plan(int BT, int H, int rows_max, int* n_split, int* rows_per_split);

// HCA decode (one query per sequence, no overlap, bf16) with at least two
// row splits (the merge adds the new entry): the coordinates split into
// power-of-two slices of 8..64, one per split, every source token of a
// block handled by one thread of its slice.
bool attend_fuses_fold(AttendArgs& a, const FoldArgs& f) {
  a.fold_mode = 0;
  if (!a.dense || a.dtype != BF16 || f.dtype != BF16 || !attend_mfma_shape_ok(a.H, a.c) || a.Tq != 1 ||
      a.n_add != 0 || a.win_pos0 != nullptr || a.win_pos0_const != 0 || f.overlap || f.idx_dtype >= 0 ||
      f.B != a.B || f.c != a.c || f.n_win != a.W_cap || f.R < 2 * f.m)
    return false;
  int ns, rps;
  attend_mfma_plan(a.B * a.Tq, a.H, a.E_cap + a.n_win, &ns, &rps);
  if (ns < 2) return false;
  int cs = 8;
  while (cs * ns < a.c) cs *= 2;
  if (cs > 64 || f.m > kFoldU * (256 / (cs / 8)) || a.H * cs > 4096) return false;
  const size_t off = attend_fold_ws_offset(a.B, a.Tq, a.H, a.c, a.E_cap + a.n_win);
  char* base = reinterpret_cast<char*>(a.ws);
  a.fold_s = reinterpret_cast<float*>(base + off);
  const size_t off_row = off + ((size_t)a.B * a.H * 8 + 255) / 256 * 256;
  a.fold_row = reinterpret_cast<int32_t*>(base + off_row);
  a.fold_new = reinterpret_cast<uint16_t*>(base + off_row + ((size_t)a.B * 4 + 255) / 256 * 256);
  a.fold = f;
  a.fold_cs = cs;
  a.fold_mode = 1;
  return true;
}

// Row splits per (query, head group): about one workgroup per CU (256), each
// split a multiple of 16 rows, at most kMaxSplit splits.
void attend_mfma_plan(int BT, int H, int rows_max, int* n_split, int* rows_per_split) {
  const int cols = BT * (H / kHW);
  int want = 256 / cols;
  if (want < 1) want = 1;
  if (want > kMaxSplit) want = kMaxSplit;
  int rps = (rows_max + want - 1) / want;
  rps = (rps + 15) / 16 * 16;
  *rows_per_split = rps;
  *n_split = (rows_max + rps - 1) / rps;
}

size_t attend_mfma_ws_bytes(int BT, int H, int rows_max) {
  int ns, rps;
  attend_mfma_plan(BT, H, rows_max, &ns, &rps);
  if (ns <= 1) return 0;
  return (size_t)BT * ns * H * (2 * sizeof(float) + kC * sizeof(uint16_t));
}

hipError_t launch_attend_merge(const AttendArgs& a, int n_split, hipStream_t s);

hipError_t launch_attend_mfma(const AttendArgs& a, int rows_max, hipStream_t s) {
  int ns, rps;
  attend_mfma_plan(a.B * a.Tq, a.H, rows_max, &ns, &rps);
  const int n_hg = a.H / kHW;
  const long long units = (long long)ns * a.B * a.Tq;       // (query, split) pairs
  const long long blocks = (units + 7) / 8 * 8 * n_hg;      // padded to whole XCD rounds
  CSA_LAUNCH("attend_dense_mfma", attend_mfma_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a, ns, rps);
  if (ns > 1) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_attend_merge(a, ns, s);
  }
  return hipGetLastError();
}

hipError_t launch_attend_merge(const AttendArgs& a, int n_split, hipStream_t s) {
  if (n_split > kMaxSplit) return hipErrorInvalidValue;
  CSA_LAUNCH("attend_merge", attend_merge_kernel, dim3(a.B * a.Tq, a.H), dim3(256), 0, s, a, n_split);
  return hipGetLastError();
}

}  // namespace csa
