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

#include "kernels.h"
#include "mfma_tile.h"

namespace csa {

using namespace tile;

namespace {

constexpr int kHW = 64;                // heads per workgroup (16 per wavefront)
constexpr int kTN = 32;                // rows per LDS tile
constexpr int kRing = 4;               // LDS tile slots: kRing - 1 tiles in flight while one is computed
constexpr int kRowsPerWave = kTN / 4;  // DMA instructions per wave and tile

}  // namespace

// 1-D grid: block L runs on XCD L % 8; the n_hg head groups of one (query,
// split) are blocks L, L + 8, ... so they share that XCD's L2.
__global__ __launch_bounds__(256, 1) void attend_mfma_kernel(AttendArgs a, int n_split, int rows_per_split) {
  __shared__ __attribute__((aligned(1024))) char tiles[kRing][kTN * kRowB];
  __shared__ uint32_t rvalid[kRing][kTN / 4];  // byte r % 4 of word r / 4: row r is a real row
  __shared__ int s_restart;                // a wavefront asks the split to be recomputed

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
  const int64_t n_rows = n_c + n_w;
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
  // lane s holds split s's statistics
  float ms = -INFINITY, Ls = 0.f;
  if (l < n_split) {
    const float2 v = *reinterpret_cast<const float2*>(pml + 2 * (((size_t)qrow * n_split + l) * H + h));
    ms = v.x;
    Ls = v.y;
  }
  const float M = fmaxf(wave_max(ms), z2);
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
  if (w == 0) {
    const float den = wave_sum(wgt) + (z2 == -INFINITY ? 0.f : exp2f(z2 - M));
    if (l == 0) s_den = den;
  }
  __syncthreads();
  if (w != 0) return;
  const float den = s_den;
  const float inv = 1.f / den;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    o[i] = (s_o[0][8 * l + i] + s_o[1][8 * l + i] + s_o[2][8 * l + i] + s_o[3][8 * l + i]) * inv;
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
