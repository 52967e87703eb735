// Shared-KV attention on MFMA (bf16, entry dim 512): rows a4 / a5 / a6.
//
// What it computes is the same as the generic kernel: for a query at position
// t and every head h, one softmax over the compressed rows (top-k set or all
// visible entries) and the window rows, with exp(sink_h) in the denominator
// ("DeepSeek-V4" book ch. 6 "Shared key-value MQA", ch. 7 "The sliding
// window" and "Attention sinks"; "2026 DeepSeek-V4" note, concat(selected,
// local_kv)).  Every row is both key and value.
//
// Work split.  A workgroup (4 wavefronts) owns one query, 32 heads and a
// contiguous range of its rows ("split"); several splits of one query are
// merged by merge_kernel with the online-softmax rule.  Row tiles of 64 rows
// are gathered into LDS (row stride 520 elements, so 16-byte reads of 16
// different rows hit distinct banks).
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

namespace {

constexpr int kC = 512;        // entry / head dim
constexpr int kHW = 32;        // heads per workgroup (2 MFMA head tiles)
constexpr int kTN = 64;        // rows per LDS tile
constexpr int kLD = kC + 8;    // padded LDS row stride (elements)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct Smem {
  uint16_t tile[kTN * kLD];
  uint16_t pt[4][2][64][4];  // P^T halves [wave][head tile][lane][4]
  float wmax[4][kHW];
  float wsum[4][kHW];
  int rowsrc[kTN];  // >= 0: cache entry; <= -2: window row (-2 - r); -1: no row
};

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

CSA_DEV int64_t rows_compressed(const AttendArgs& a, int b, int qrow, int64_t t) {
  if (!a.dense) return a.topk_cnt[qrow];
  const int64_t lim = vis_limit(t, a.m, a.vis);
  const int64_t have = (int64_t)a.n_entries[b] + a.n_add;
  int64_t n = lim < have ? lim : have;
  if (n > a.E_cap) n = a.E_cap;
  return n < 0 ? 0 : n;
}

}  // namespace

// grid (n_split, H/32, B*Tq), 256 threads
__global__ __launch_bounds__(256, 2) void attend_mfma_kernel(AttendArgs a, int n_split,
                                                             int rows_per_split) {
  __shared__ Smem sm;
  const int split = blockIdx.x, hg = blockIdx.y, qrow = blockIdx.z;
  const int b = qrow / a.Tq;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, li = l & 15, lg = l >> 4;
  const int H = a.H;
  const int h0 = hg * kHW;
  const int64_t t = a.q_pos ? a.q_pos[qrow] : a.q_pos0 + qrow % a.Tq;
  const int64_t n_c = rows_compressed(a, b, qrow, t);
  const int64_t n_w = (t + 1) < a.n_win ? (t + 1) : a.n_win;
  const int64_t n_rows = n_c + n_w;
  const int64_t r_begin = (int64_t)split * rows_per_split;
  int64_t r_end = r_begin + rows_per_split;
  if (r_end > n_rows) r_end = n_rows;
  const int64_t wpos0 = a.win_pos0 ? a.win_pos0[b] : a.win_pos0_const;
  const uint16_t* kv = reinterpret_cast<const uint16_t*>(a.kv) + (size_t)b * a.E_cap * kC;
  const uint16_t* win = reinterpret_cast<const uint16_t*>(a.win) + (size_t)b * a.W_cap * kC;
  const int32_t* ids = a.dense ? nullptr : a.topk_idx + (size_t)qrow * a.k;
  const float sc2 = a.scale * kLog2e;

  // Q^T operands for the 32 heads: lane (head li, d group lg)
  bf16x8_t qf[2][16];
  {
    const uint16_t* q = reinterpret_cast<const uint16_t*>(a.q) + ((size_t)qrow * H + h0) * kC;
#pragma unroll
    for (int ht = 0; ht < 2; ++ht)
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) qf[ht][ks] = ld8(q + (size_t)(16 * ht + li) * kC + 32 * ks + 8 * lg);
  }

  f32x4_t acc[8][2];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) acc[dt][ht] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};

  for (int64_t r0 = r_begin; r0 < r_end; r0 += kTN) {
    if (tid < kTN) {
      const int64_t j = r0 + tid;
      int src = -1;
      if (j < r_end) {
        if (j < n_c) {
          const int64_t e = a.dense ? j : (int64_t)ids[j];
          if (e >= 0 && e < a.E_cap) src = (int)e;
        } else {
          const int64_t pos = t - n_w + 1 + (j - n_c);
          int64_t wr = (pos - wpos0) % a.W_cap;
          if (wr < 0) wr += a.W_cap;
          src = -2 - (int)wr;
        }
      }
      sm.rowsrc[tid] = src;
    }
    __syncthreads();
    // gather: wave w copies rows w, w+4, ..., 16 B per lane (one 1 KB row per instruction)
#pragma unroll
    for (int part = 0; part < 4; ++part) {
      uint4 v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int src = sm.rowsrc[w + 4 * (4 * part + i)];
        const uint16_t* p = src >= 0 ? kv + (size_t)src * kC : win + (size_t)(-2 - src) * kC;
        v[i] = src != -1 ? *reinterpret_cast<const uint4*>(p + 8 * l) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<uint4*>(&sm.tile[(w + 4 * (4 * part + i)) * kLD + 8 * l]) = v[i];
    }
    __syncthreads();

    // S^T for rows 16w..16w+15
    f32x4_t s[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      const bf16x8_t kf = ld8(&sm.tile[(16 * w + li) * kLD + 32 * ks + 8 * lg]);
      s[0] = mfma(kf, qf[0][ks], s[0]);
      s[1] = mfma(kf, qf[1][ks], s[1]);
      if ((ks & 3) == 3) __builtin_amdgcn_sched_barrier(0);  // bound hoisted loads
    }
    bool valid[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) valid[r] = sm.rowsrc[16 * w + 4 * lg + r] != -1;
    float alpha[2];
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s[ht][r] = valid[r] ? s[ht][r] * sc2 : -INFINITY;
        mx = fmaxf(mx, s[ht][r]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      if (lg == 0) sm.wmax[w][16 * ht + li] = mx;
    }
    __syncthreads();
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      float tm = fmaxf(fmaxf(sm.wmax[0][16 * ht + li], sm.wmax[1][16 * ht + li]),
                       fmaxf(sm.wmax[2][16 * ht + li], sm.wmax[3][16 * ht + li]));
      const float m_new = fmaxf(m_run[ht], tm);
      alpha[ht] = (m_run[ht] == -INFINITY) ? (m_new == -INFINITY ? 1.f : 0.f) : exp2f(m_run[ht] - m_new);
      float p[4], ps = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[r] = (s[ht][r] == -INFINITY) ? 0.f : exp2f(s[ht][r] - m_new);
        ps += p[r];
      }
      ps += __shfl_xor(ps, 16, 64);
      ps += __shfl_xor(ps, 32, 64);
      l_run[ht] = l_run[ht] * alpha[ht] + ps;
      m_run[ht] = m_new;
      uint16_t* dst = sm.pt[w][ht][l];
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[r] = f32_to_bf16(p[r]);
    }
    __syncthreads();

    // O^T[d 128w.. +128][32 heads] += V^T . P^T
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) acc[dt][ht] *= alpha[ht];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      bf16x8_t pb[2];
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) {
        const i16x4_t lo = *reinterpret_cast<const i16x4_t*>(sm.pt[2 * kc][ht][l]);
        const i16x4_t hi = *reinterpret_cast<const i16x4_t*>(sm.pt[2 * kc + 1][ht][l]);
        pb[ht] = cat8(lo, hi);
      }
      const uint16_t* base = &sm.tile[(32 * kc + 4 * lg + (li >> 2)) * kLD + 128 * w + 4 * (li & 3)];
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const i16x4_t v1 = ld_tr(base + 16 * dt);
        const i16x4_t v2 = ld_tr(base + 16 * kLD + 16 * dt);
        const bf16x8_t vf = cat8(v1, v2);
        acc[dt][0] = mfma(vf, pb[0], acc[dt][0]);
        acc[dt][1] = mfma(vf, pb[1], acc[dt][1]);
        if ((dt & 1) == 1) __builtin_amdgcn_sched_barrier(0);
      }
    }
    __syncthreads();
  }

  // per-head row sums of the four wavefronts
#pragma unroll
  for (int ht = 0; ht < 2; ++ht)
    if (lg == 0) sm.wsum[w][16 * ht + li] = l_run[ht];
  __syncthreads();
  float Lh[2];
#pragma unroll
  for (int ht = 0; ht < 2; ++ht)
    Lh[ht] = sm.wsum[0][16 * ht + li] + sm.wsum[1][16 * ht + li] + sm.wsum[2][16 * ht + li] +
             sm.wsum[3][16 * ht + li];

  if (n_split == 1) {
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      const int h = h0 + 16 * ht + li;
      const float z2 = a.sink ? a.sink[h] * kLog2e : -INFINITY;
      const float M = fmaxf(m_run[ht], z2);
      const float em = exp2f(m_run[ht] - M);
      const float den = Lh[ht] * em + (z2 == -INFINITY ? 0.f : exp2f(z2 - M));
      const float f = em / den;
      if (a.lse && w == 0 && lg == 0) a.lse[(size_t)qrow * H + h] = (M + log2f(den)) * kLn2;
      uint16_t* o = reinterpret_cast<uint16_t*>(a.out) + ((size_t)qrow * H + h) * kC + 128 * w + 4 * lg;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
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
  for (int ht = 0; ht < 2; ++ht) {
    const int h = h0 + 16 * ht + li;
    const size_t slot = ((size_t)qrow * n_split + split) * H + h;
    if (w == 0 && lg == 0) {
      pml[2 * slot] = m_run[ht];
      pml[2 * slot + 1] = Lh[ht];
    }
    const float f = Lh[ht] > 0.f ? 1.f / Lh[ht] : 0.f;
    uint16_t* o = po + slot * kC + 128 * w + 4 * lg;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      ushort4 v;
      v.x = f32_to_bf16(acc[dt][ht][0] * f);
      v.y = f32_to_bf16(acc[dt][ht][1] * f);
      v.z = f32_to_bf16(acc[dt][ht][2] * f);
      v.w = f32_to_bf16(acc[dt][ht][3] * f);
      *reinterpret_cast<ushort4*>(o + 16 * dt) = v;
    }
  }
}

// grid (B*Tq, H), 64 threads: each lane merges 8 coordinates of one head
__global__ __launch_bounds__(64) void attend_merge_kernel(AttendArgs a, int n_split) {
  const int qrow = blockIdx.x, h = blockIdx.y, l = threadIdx.x;
  const int H = a.H;
  const float* pml = reinterpret_cast<const float*>(a.ws);
  const uint16_t* po = reinterpret_cast<const uint16_t*>(pml + (size_t)a.B * a.Tq * n_split * H * 2);
  float M = a.sink ? a.sink[h] * kLog2e : -INFINITY;
  for (int s = 0; s < n_split; ++s) M = fmaxf(M, pml[2 * (((size_t)qrow * n_split + s) * H + h)]);
  float den = a.sink ? exp2f(a.sink[h] * kLog2e - M) : 0.f;
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < n_split; ++s) {
    const size_t slot = ((size_t)qrow * n_split + s) * H + h;
    const float ms = pml[2 * slot], Ls = pml[2 * slot + 1];
    if (ms == -INFINITY || Ls == 0.f) continue;
    const float wgt = exp2f(ms - M) * Ls;
    den += wgt;
    const uint4 raw = *reinterpret_cast<const uint4*>(po + slot * kC + 8 * l);
    const uint32_t u[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] += wgt * bf16_to_f32((uint16_t)(u[i] & 0xffff));
      o[2 * i + 1] += wgt * bf16_to_f32((uint16_t)(u[i] >> 16));
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
  dim3 grid(ns, a.H / kHW, a.B * a.Tq), block(256);
  CSA_LAUNCH(a.dense ? "attend_dense_mfma" : "attend_sparse_mfma", attend_mfma_kernel, grid, block, 0,
             s, a, ns, rps);
  if (ns > 1) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    CSA_LAUNCH("attend_merge", attend_merge_kernel, dim3(a.B * a.Tq, a.H), dim3(64), 0, s, a, ns);
  }
  return hipGetLastError();
}

}  // namespace csa
