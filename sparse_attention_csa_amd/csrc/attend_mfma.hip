// Shared-KV attention on MFMA (bf16, entry dim 512): rows a4 / a5 / a6.
//
// What it computes is the same as the generic kernel: for a query at position
// t and every head h, one softmax over the compressed rows (top-k set or all
// visible entries) and the window rows, with exp(sink_h) in the denominator
// ("DeepSeek-V4" book ch. 6 "Shared key-value MQA", ch. 7 "The sliding
// window" and "Attention sinks"; "2026 DeepSeek-V4" note, concat(selected,
// local_kv)).  Every row is both key and value.
//
// Work split.  A workgroup (4 wavefronts, one per SIMD, the whole register
// file) owns one query, 32 heads and a contiguous range of its rows
// ("split"); several splits of one query are merged by attend_merge_kernel
// with the online-softmax rule.  Row tiles of 64 rows are fetched into LDS by
// direct global-to-LDS DMA (one 1 KB row per wave instruction), double
// buffered so that tile i+1 is in flight while tile i is computed; the LDS
// row stride is 520 elements so 16-byte reads of 16 different rows hit
// distinct banks.  Block order is XCD-aware: the head groups of one split run
// on the same XCD and share its L2.
//
// Tied K = V on MFMA.  The score product is computed transposed,
//   S^T[rows x heads] = K[rows x d] . Q^T[d x heads]   (v_mfma 16x16x32 bf16),
// with Q^T held in registers and K read row-major from LDS; wave w scores
// rows 16w..16w+15 of the tile.  The accumulator layout of S^T (lane = head,
// 4 consecutive rows per lane group) is, after exp2 and a bf16 cast, exactly
// the B operand of
//   O^T[d x heads] += V^T[d x rows] . P^T[rows x heads],
// once the 32-row reduction slots are permuted consistently (slot 8g+t is row
// 4g+t of one 16-row half for t < 4 and of the other half for t >= 4).  V^T is
// fetched from the same LDS tile with the gfx950 transpose read
// (ds_read_b64_tr_b16), whose per-lane addresses implement that permutation.
// Wave w accumulates O^T for d = 128w..128w+127 and all 32 heads, so only P^T
// (4 KB) and per-head maxima cross wavefronts.  Softmax runs in base 2.

#include "common.h"
#include "kernels.h"

namespace csa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

namespace {

constexpr int kC = 512;        // entry / head dim
constexpr int kHT = 1;         // MFMA head tiles per workgroup
constexpr int kHW = 16 * kHT;  // heads per workgroup
constexpr int kTN = 64;        // rows per LDS tile
constexpr int kLD = kC + 8;    // padded LDS row stride (elements)
constexpr int kMaxSparseRows = 2304;  // k + n_win <= 2048 + 256
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kSlack = 8.f;  // log2 headroom before the running max is moved

// s_waitcnt with vmcnt = 16, lgkmcnt / expcnt not waited (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int kWaitVm16 = 0x4F70;
constexpr int kWaitVm0 = 0x0F70;

CSA_DEV f32x4_t mfma(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

CSA_DEV bf16x8_t ld8(const uint16_t* p) { return *reinterpret_cast<const bf16x8_t*>(p); }

CSA_DEV i16x4_t ld_tr(const uint16_t* p) {
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

CSA_DEV bf16x8_t cat8(i16x4_t a, i16x4_t b) {
  i16x8_t v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8_t, v);
}

// one lane's 16 bytes of a 1 KB row, DMA'd to LDS at lds_row + 16 * lane
CSA_DEV void dma_row(const uint16_t* src_row, uint16_t* lds_row, int lane) {
  __builtin_amdgcn_global_load_lds(
      (const void __attribute__((address_space(1)))*)(src_row + 8 * lane),
      (void __attribute__((address_space(3)))*)(lds_row), 16, 0, 0);
}

CSA_DEV int64_t rows_compressed(const AttendArgs& a, int b, int qrow, int64_t t) {
  if (!a.dense) return a.topk_cnt[qrow];
  const int64_t lim = vis_limit(t, a.m, a.vis);
  const int64_t have = (int64_t)a.n_entries[b] + a.n_add;
  int64_t n = lim < have ? lim : have;
  if (n > a.E_cap) n = a.E_cap;
  return n < 0 ? 0 : n;
}

}  // namespace

// 1-D grid: block L runs on XCD L % 8; the n_hg head groups of one (query,
// split) are blocks L, L + 8, ... so they share that XCD's L2.
__global__ __launch_bounds__(256, 1) void attend_mfma_kernel(AttendArgs a, int n_split,
                                                             int rows_per_split) {
  __shared__ uint16_t tile0[kTN * kLD];
  __shared__ uint16_t tile1[kTN * kLD];
  __shared__ float wmax[4][kHW];
  __shared__ float wsum[4][kHW];
  __shared__ int rsrc[kMaxSparseRows];  // sparse: cache entry per row of the split (-1: none)
  __shared__ unsigned char rvalid[2][kTN];

  const int n_hg = a.H / kHW;
  const int L = blockIdx.x;
  const int xcd = L & 7, kk = L >> 3;
  const int hg = kk % n_hg;
  const int rest = (kk / n_hg) * 8 + xcd;
  const int split = rest % n_split, qrow = rest / n_split;
  if (qrow >= a.B * a.Tq) return;

  const int b = qrow / a.Tq;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, li = l & 15, lg = l >> 4;
  const int H = a.H;
  const int h0 = hg * kHW;
  const int64_t t = a.q_pos ? a.q_pos[qrow] : a.q_pos0 + qrow % a.Tq;
  const int64_t n_c = rows_compressed(a, b, qrow, t);
  const int64_t n_w = (t + 1) < a.n_win ? (t + 1) : a.n_win;
  const int64_t n_rows = n_c + n_w;
  const int r_begin = split * rows_per_split;
  const int r_end = (int)((int64_t)r_begin + rows_per_split < n_rows ? r_begin + rows_per_split : n_rows);
  const int nc32 = (int)n_c;
  const int64_t wpos0 = a.win_pos0 ? a.win_pos0[b] : a.win_pos0_const;
  const uint16_t* kv = reinterpret_cast<const uint16_t*>(a.kv) + (size_t)b * a.E_cap * kC;
  const uint16_t* win = reinterpret_cast<const uint16_t*>(a.win) + (size_t)b * a.W_cap * kC;
  const float sc2 = a.scale * kLog2e;
  // ring row of the first window position; later window rows follow with
  // one conditional wrap (n_win <= W_cap)
  int64_t wb = (t - n_w + 1 - wpos0) % a.W_cap;
  if (wb < 0) wb += a.W_cap;
  const int wbase = (int)wb, wcap = a.W_cap;
  // the query's own window row: always present, the source of padding rows
  // (their logits are masked)
  int own = wbase + (int)n_w - 1;
  if (own >= wcap) own -= wcap;
  const uint16_t* pad_row = win + (size_t)own * kC;

  if (!a.dense) {
    const int32_t* ids = a.topk_idx + (size_t)qrow * a.k;
    for (int j = r_begin + tid; j < r_end; j += 256) {
      int e = -1;
      if (j < nc32) {
        const int32_t v = ids[j];
        e = (v >= 0 && v < a.E_cap) ? v : -1;
      }
      rsrc[j - r_begin] = e;
    }
  }

  // Q^T operands for the 32 heads: lane (head li, d group lg)
  bf16x8_t qf[kHT][16];
  {
    const uint16_t* q = reinterpret_cast<const uint16_t*>(a.q) + ((size_t)qrow * H + h0) * kC;
#pragma unroll
    for (int ht = 0; ht < kHT; ++ht)
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) qf[ht][ks] = ld8(q + (size_t)(16 * ht + li) * kC + 32 * ks + 8 * lg);
  }
  __syncthreads();  // rsrc ready

  auto row_src = [&](int j, bool* ok) -> const uint16_t* {
    *ok = false;
    if (j >= r_end) return pad_row;
    if (j < nc32) {
      if (a.dense) {
        *ok = true;
        return kv + (size_t)j * kC;
      }
      const int e = rsrc[j - r_begin];
      if (e < 0) return pad_row;
      *ok = true;
      return kv + (size_t)e * kC;
    }
    int wr = wbase + (j - nc32);
    if (wr >= wcap) wr -= wcap;
    *ok = true;
    return win + (size_t)wr * kC;
  };
  // wave w fetches (and later consumes) rows 16w .. 16w+15 of a tile
  auto issue_tile = [&](int r0, uint16_t* __restrict__ tile, int buf) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 16 * w + i;
      bool ok;
      const uint16_t* src = row_src(r0 + r, &ok);
      dma_row(src, tile + r * kLD, l);
      if (l == 0) rvalid[buf][r] = ok;
    }
  };

  // this wave's running softmax state and O^T[512 d x 32 heads] over its rows
  f32x4_t acc[32][kHT];
#pragma unroll
  for (int dt = 0; dt < 32; ++dt)
#pragma unroll
    for (int ht = 0; ht < kHT; ++ht) acc[dt][ht] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run[kHT], l_run[kHT];
#pragma unroll
  for (int ht = 0; ht < kHT; ++ht) {
    m_run[ht] = -INFINITY;
    l_run[ht] = 0.f;
  }

  auto compute_tile = [&](const uint16_t* __restrict__ tile, int buf) {
    const uint16_t* rows = tile + 16 * w * kLD;  // this wave's 16 rows
    // S^T[16 rows x 32 heads] = K . Q^T
    f32x4_t s[kHT];
#pragma unroll
    for (int ht = 0; ht < kHT; ++ht) s[ht] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      const bf16x8_t kf = ld8(&rows[li * kLD + 32 * ks + 8 * lg]);
#pragma unroll
      for (int ht = 0; ht < kHT; ++ht) s[ht] = mfma(kf, qf[ht][ks], s[ht]);
    }
    // online softmax per head over this wave's rows; lane holds rows 4lg..4lg+3.
    // The reference max m_run only moves when a head's tile max exceeds it by
    // more than kSlack (log2 units), so unnormalised weights stay <= 2^kSlack
    // and the accumulator rescale is a rare, wave-uniform branch.
    bf16x4_t pb[kHT];
    float x[kHT][4], tmax[kHT];
#pragma unroll
    for (int ht = 0; ht < kHT; ++ht) {
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        x[ht][r] = rvalid[buf][16 * w + 4 * lg + r] ? s[ht][r] * sc2 : -INFINITY;
        mx = fmaxf(mx, x[ht][r]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      tmax[ht] = mx;
    }
    bool grow = false;
#pragma unroll
    for (int ht = 0; ht < kHT; ++ht) grow = grow || (tmax[ht] > m_run[ht] + kSlack);
    if (__builtin_amdgcn_ballot_w64(grow) != 0ull) {
#pragma unroll
      for (int ht = 0; ht < kHT; ++ht) {
        const float m_new = fmaxf(m_run[ht], tmax[ht]);
        const float alpha = (m_run[ht] == -INFINITY) ? 0.f : exp2f(m_run[ht] - m_new);
        l_run[ht] *= alpha;
        m_run[ht] = m_new;
#pragma unroll
        for (int dt = 0; dt < 32; ++dt) acc[dt][ht] *= alpha;
      }
    }
#pragma unroll
    for (int ht = 0; ht < kHT; ++ht) {
      float p[4], ps = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[r] = (x[ht][r] == -INFINITY) ? 0.f : exp2f(x[ht][r] - m_run[ht]);
        ps += p[r];
      }
      ps += __shfl_xor(ps, 16, 64);
      ps += __shfl_xor(ps, 32, 64);
      l_run[ht] += ps;
      pb[ht] = bf16x4_t{(__bf16)p[0], (__bf16)p[1], (__bf16)p[2], (__bf16)p[3]};
    }
    // O^T[d x heads] += V^T[d x 16 rows] . P^T[16 rows x heads] (16x16x16):
    // the P^T operand is this lane's own S^T values; V^T comes from one
    // transpose read (lane j of group g addresses row 4g + j/4, d 4(j%4)).
    const uint16_t* vb = &rows[(4 * lg + (li >> 2)) * kLD + 4 * (li & 3)];
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) {
      const bf16x4_t vf = __builtin_bit_cast(bf16x4_t, ld_tr(vb + 16 * dt));
#pragma unroll
      for (int ht = 0; ht < kHT; ++ht)
        acc[dt][ht] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vf, pb[ht], acc[dt][ht], 0, 0, 0);
    }
  };

  // double-buffered loop: tile i computes while tile i+1 is in flight.  Each
  // wave only reads the rows it fetched itself, so waiting for its own DMAs
  // (vmcnt <= 16 leaves the next tile's 16 in flight) suffices before
  // computing; one barrier per tile keeps a buffer from being refilled while
  // another wave could still... (waves never touch each other's rows, the
  // barrier only bounds how far waves drift apart).
  int r0 = r_begin;
  if (r0 < r_end) issue_tile(r0, tile0, 0);
  while (r0 < r_end) {
    const int r1 = r0 + kTN;
    if (r1 < r_end) {
      issue_tile(r1, tile1, 1);
      __builtin_amdgcn_s_waitcnt(kWaitVm16);
    } else {
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
    }
    lds_barrier();
    compute_tile(tile0, 0);
    r0 = r1;
    if (r0 >= r_end) break;
    const int r2 = r0 + kTN;
    if (r2 < r_end) {
      issue_tile(r2, tile0, 0);
      __builtin_amdgcn_s_waitcnt(kWaitVm16);
    } else {
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
    }
    lds_barrier();
    compute_tile(tile1, 1);
    r0 = r2;
  }
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();

  // merge the four wavefronts: common max, rescale, tree-sum O through LDS
  if (lg == 0) {
#pragma unroll
    for (int ht = 0; ht < kHT; ++ht) wmax[w][16 * ht + li] = m_run[ht];
  }
  __syncthreads();
  float Lh[kHT], Mh[kHT];
#pragma unroll
  for (int ht = 0; ht < kHT; ++ht) {
    const int c = 16 * ht + li;
    const float M = fmaxf(fmaxf(wmax[0][c], wmax[1][c]), fmaxf(wmax[2][c], wmax[3][c]));
    const float f = (m_run[ht] == -INFINITY) ? 0.f : exp2f(m_run[ht] - M);
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) acc[dt][ht] *= f;
    Mh[ht] = M;
    Lh[ht] = l_run[ht] * f;
  }
  if (lg == 0) {
#pragma unroll
    for (int ht = 0; ht < kHT; ++ht) wsum[w][16 * ht + li] = Lh[ht];
  }
  f32x4_t* red0 = reinterpret_cast<f32x4_t*>(tile0);  // [32][kHT][64] f32x4
  f32x4_t* red1 = reinterpret_cast<f32x4_t*>(tile1);
  auto put = [&](f32x4_t* R) {
#pragma unroll
    for (int dt = 0; dt < 32; ++dt)
#pragma unroll
      for (int ht = 0; ht < kHT; ++ht) R[(dt * kHT + ht) * 64 + l] = acc[dt][ht];
  };
  auto add = [&](const f32x4_t* R) {
#pragma unroll
    for (int dt = 0; dt < 32; ++dt)
#pragma unroll
      for (int ht = 0; ht < kHT; ++ht) acc[dt][ht] += R[(dt * kHT + ht) * 64 + l];
  };
  if (w == 1) put(red0);
  if (w == 3) put(red1);
  __syncthreads();
  if (w == 0) add(red0);
  if (w == 2) add(red1);
  __syncthreads();
  if (w == 2) put(red0);
  __syncthreads();
  if (w != 0) return;
  add(red0);
#pragma unroll
  for (int ht = 0; ht < kHT; ++ht)
    Lh[ht] = wsum[0][16 * ht + li] + wsum[1][16 * ht + li] + wsum[2][16 * ht + li] + wsum[3][16 * ht + li];

  // wave 0 writes: lane (head li, d rows 4lg..4lg+3 of each 16-wide d tile)
  if (n_split == 1) {
#pragma unroll
    for (int ht = 0; ht < kHT; ++ht) {
      const int h = h0 + 16 * ht + li;
      const float z2 = a.sink ? a.sink[h] * kLog2e : -INFINITY;
      const float M = fmaxf(Mh[ht], z2);
      const float em = exp2f(Mh[ht] - M);
      const float den = Lh[ht] * em + (z2 == -INFINITY ? 0.f : exp2f(z2 - M));
      const float f = em / den;
      if (a.lse && lg == 0) a.lse[(size_t)qrow * H + h] = (M + log2f(den)) * kLn2;
      uint16_t* o = reinterpret_cast<uint16_t*>(a.out) + ((size_t)qrow * H + h) * kC + 4 * lg;
#pragma unroll
      for (int dt = 0; dt < 32; ++dt) {
        ushort4 v;
        v.x = f32_to_bf16(acc[dt][ht][0] * f);
        v.y = f32_to_bf16(acc[dt][ht][1] * f);
        v.z = f32_to_bf16(acc[dt][ht][2] * f);
        v.w = f32_to_bf16(acc[dt][ht][3] * f);
        *reinterpret_cast<ushort4*>(o + 16 * dt) = v;
      }
    }
    return;
  }
  // partial: (m, L) and O / L in bf16
  float* pml = reinterpret_cast<float*>(a.ws);
  uint16_t* po = reinterpret_cast<uint16_t*>(pml + (size_t)a.B * a.Tq * n_split * H * 2);
#pragma unroll
  for (int ht = 0; ht < kHT; ++ht) {
    const int h = h0 + 16 * ht + li;
    const size_t slot = ((size_t)qrow * n_split + split) * H + h;
    if (lg == 0) {
      pml[2 * slot] = Mh[ht];
      pml[2 * slot + 1] = Lh[ht];
    }
    const float f = Lh[ht] > 0.f ? 1.f / Lh[ht] : 0.f;
    uint16_t* o = po + slot * kC + 4 * lg;
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) {
      ushort4 v;
      v.x = f32_to_bf16(acc[dt][ht][0] * f);
      v.y = f32_to_bf16(acc[dt][ht][1] * f);
      v.z = f32_to_bf16(acc[dt][ht][2] * f);
      v.w = f32_to_bf16(acc[dt][ht][3] * f);
      *reinterpret_cast<ushort4*>(o + 16 * dt) = v;
    }
  }
}

// grid (B*Tq, H), 64 threads: each lane merges 8 coordinates of one head.
// All split statistics are loaded first, then all partial rows (independent
// loads in flight together).
constexpr int kMaxSplit = 64;

__global__ __launch_bounds__(64) void attend_merge_kernel(AttendArgs a, int n_split) {
  const int qrow = blockIdx.x, h = blockIdx.y, l = threadIdx.x;
  const int H = a.H;
  const float* pml = reinterpret_cast<const float*>(a.ws);
  const uint16_t* po = reinterpret_cast<const uint16_t*>(pml + (size_t)a.B * a.Tq * n_split * H * 2);
  const float z2 = a.sink ? a.sink[h] * kLog2e : -INFINITY;
  float ms[kMaxSplit], Ls[kMaxSplit];
  float M = z2;
#pragma unroll
  for (int s = 0; s < kMaxSplit; ++s) {
    if (s < n_split) {
      const float2 v = *reinterpret_cast<const float2*>(pml + 2 * (((size_t)qrow * n_split + s) * H + h));
      ms[s] = v.x;
      Ls[s] = v.y;
      M = fmaxf(M, v.x);
    }
  }
  float den = z2 == -INFINITY ? 0.f : exp2f(z2 - M);
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
  for (int s = 0; s < kMaxSplit; ++s) {
    if (s < n_split) {
      const size_t slot = ((size_t)qrow * n_split + s) * H + h;
      const float wgt = (ms[s] == -INFINITY || Ls[s] == 0.f) ? 0.f : exp2f(ms[s] - M) * Ls[s];
      den += wgt;
      const uint4 raw = *reinterpret_cast<const uint4*>(po + slot * kC + 8 * l);
      const uint32_t u[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o[2 * i] += wgt * bf16_to_f32((uint16_t)(u[i] & 0xffff));
        o[2 * i + 1] += wgt * bf16_to_f32((uint16_t)(u[i] >> 16));
      }
    }
  }
  const float inv = 1.f / den;
  uint16_t* out = reinterpret_cast<uint16_t*>(a.out) + ((size_t)qrow * H + h) * kC + 8 * l;
  uint4 r;
  r.x = (uint32_t)f32_to_bf16(o[0] * inv) | ((uint32_t)f32_to_bf16(o[1] * inv) << 16);
  r.y = (uint32_t)f32_to_bf16(o[2] * inv) | ((uint32_t)f32_to_bf16(o[3] * inv) << 16);
  r.z = (uint32_t)f32_to_bf16(o[4] * inv) | ((uint32_t)f32_to_bf16(o[5] * inv) << 16);
  r.w = (uint32_t)f32_to_bf16(o[6] * inv) | ((uint32_t)f32_to_bf16(o[7] * inv) << 16);
  *reinterpret_cast<uint4*>(out) = r;
  if (a.lse && l == 0) a.lse[(size_t)qrow * H + h] = (M + log2f(den)) * kLn2;
}

bool attend_mfma_supported(const AttendArgs& a) {
  return a.dtype == BF16 && a.c == kC && a.H % kHW == 0;
}

// number of row splits per (query, head group) and rows per split
void attend_mfma_plan(int BT, int H, int rows_max, int* n_split, int* rows_per_split) {
  const int cols = BT * (H / kHW);
  const int tiles = (rows_max + kTN - 1) / kTN;
  int want = (256 + cols - 1) / cols;
  if (want < 1) want = 1;
  if (want > kMaxSplit) want = kMaxSplit;
  if (want > tiles) want = tiles;
  const int tiles_per = (tiles + want - 1) / want;
  *rows_per_split = tiles_per * kTN;
  *n_split = (rows_max + *rows_per_split - 1) / *rows_per_split;
}

size_t attend_mfma_ws_bytes(int BT, int H, int rows_max) {
  int ns, rps;
  attend_mfma_plan(BT, H, rows_max, &ns, &rps);
  if (ns <= 1) return 0;
  return (size_t)BT * ns * H * (2 * sizeof(float) + kC * sizeof(uint16_t));
}

hipError_t launch_attend_mfma(const AttendArgs& a, int rows_max, hipStream_t s) {
  int ns, rps;
  attend_mfma_plan(a.B * a.Tq, a.H, rows_max, &ns, &rps);
  const int n_hg = a.H / kHW;
  const long long units = (long long)ns * a.B * a.Tq;       // (query, split) pairs
  const long long blocks = (units + 7) / 8 * 8 * n_hg;      // padded to whole XCD rounds
  CSA_LAUNCH(a.dense ? "attend_dense_mfma" : "attend_sparse_mfma", attend_mfma_kernel, dim3((unsigned)blocks),
             dim3(256), 0, s, a, ns, rps);
  if (ns > 1) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    CSA_LAUNCH("attend_merge", attend_merge_kernel, dim3(a.B * a.Tq, a.H), dim3(64), 0, s, a, ns);
  }
  return hipGetLastError();
}

}  // namespace csa
