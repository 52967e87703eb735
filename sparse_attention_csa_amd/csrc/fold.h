// Compressor fold building blocks shared by the decode fold kernel and the
// scoring kernel's fold workgroup (row a1): the per-coordinate softmax state
// and the fold of one entry's coordinates by a workgroup of kFoldT threads
// ("2026 DeepSeek-V4" note, "Key design 1" and "Key design 2" equations;
// "DeepSeek-V4" book ch. 5 "One weight distribution per coordinate").
#pragma once

#include "common.h"
#include "kernels.h"

namespace csa {

// running softmax state of one coordinate over a subset of sources
struct Soft {
  float mx, l, acc;
};

CSA_DEV void soft_push(Soft& s, float logit, float v) {
  if (logit > s.mx) {
    const float r = __expf(s.mx - logit);
    s.l = s.l * r + 1.f;
    s.acc = s.acc * r + v;
    s.mx = logit;
  } else {
    const float e = __expf(logit - s.mx);
    s.l += e;
    s.acc += e * v;
  }
}

CSA_DEV Soft soft_merge(Soft a, Soft b) {
  if (b.l == 0.f) return a;
  if (a.l == 0.f) return b;
  const float mx = fmaxf(a.mx, b.mx);
  const float ra = __expf(a.mx - mx), rb = __expf(b.mx - mx);
  return Soft{mx, a.l * ra + b.l * rb, a.acc * ra + b.acc * rb};
}

// the same merge with selects instead of branches (no divergent paths in
// the lane-exchange reductions)
CSA_DEV Soft soft_merge_sel(Soft a, Soft b) {
  const float mx = fmaxf(a.mx, b.mx);
  const float ra = a.l == 0.f ? 0.f : __expf(a.mx - mx);
  const float rb = b.l == 0.f ? 0.f : __expf(b.mx - mx);
  return Soft{(a.l == 0.f && b.l == 0.f) ? a.mx : mx, a.l * ra + b.l * rb, a.acc * ra + b.acc * rb};
}

constexpr int kFoldT = 256;
constexpr int kFoldCW = 64;  // main-entry coordinates per workgroup

template <typename T>
struct Vec16 {
  static constexpr int V = 16 / (int)sizeof(T);
};

// V consecutive elements (16 bytes) of T as floats
CSA_DEV void unpack16(const uint4 u, const bf16*, float* o) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = __uint_as_float(w[i] << 16);
    o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
CSA_DEV void unpack16(const uint4 u, const float*, float* o) {
  o[0] = __uint_as_float(u.x); o[1] = __uint_as_float(u.y);
  o[2] = __uint_as_float(u.z); o[3] = __uint_as_float(u.w);
}

// Folds coordinates [r0, r0 + W) of entry e from rows of length d; returns
// the value of coordinate r0 + tid for tid < W.  Sources: branch a is tokens
// e*m .. e*m+m-1 (streams 0, 1), branch b (use_b) tokens (e-1)*m .. e*m-1
// (streams 2, 3); token p is ring slot p % R, the new token t comes from io.
// Each thread folds its U sources per coordinate with one rescale; the G
// partial states of a coordinate then merge across lanes (xor shuffles
// within a wavefront) and across the four wavefronts (LDS).
template <typename T>
CSA_DEV float fold_job(const T* tail, const T* io, int d, int r0, int W, int m, int R, int64_t t,
                       int64_t e, bool use_b, const float* ba, const float* bb, Soft* s_part) {
  constexpr int V = Vec16<T>::V;
  constexpr int U = 4;  // sources in flight per thread
  const int tid = threadIdx.x;
  const int TR = W / V, G = kFoldT / TR;
  const int o = tid % TR, grp = tid / TR;
  const int rr = r0 + o * V;
  const int nsrc = use_b ? 2 * m : m;
  const int64_t p_first = use_b ? (e - 1) * m : e * m;  // earliest source token
  const int slot_first = (int)(p_first % R);
  const int t_off = (int)(t - p_first);
  Soft st[V];
#pragma unroll
  for (int v = 0; v < V; ++v) st[v] = Soft{-INFINITY, 0.f, 0.f};
  for (int j0 = grp; j0 < nsrc; j0 += U * G) {
    uint4 zr[U], xr[U];
    float bz[U][V];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u * G;
      zr[u] = xr[u] = uint4{0, 0, 0, 0};
#pragma unroll
      for (int v = 0; v < V; ++v) bz[u][v] = 0.f;
      if (j < nsrc) {
        const bool a_br = j < m;
        const int jj = a_br ? j : j - m;                 // index within the branch
        const int off = use_b ? (a_br ? m + j : j - m) : j;  // token - p_first
        const int sc = a_br ? 0 : 2;
        const T *pz, *px;
        if (off == t_off) {
          pz = io + (size_t)(sc + 1) * d + rr;
          px = io + (size_t)sc * d + rr;
        } else {
          int slot = slot_first + off;
          while (slot >= R) slot -= R;
          pz = tail + ((size_t)(sc + 1) * R + slot) * d + rr;
          px = tail + ((size_t)sc * R + slot) * d + rr;
        }
        zr[u] = *reinterpret_cast<const uint4*>(pz);
        xr[u] = *reinterpret_cast<const uint4*>(px);
        const float* bias = a_br ? ba : bb;
        if (bias) {
#pragma unroll
          for (int v = 0; v < V; v += 4) {
            const float4 f = *reinterpret_cast<const float4*>(bias + (size_t)jj * d + rr + v);
            bz[u][v] = f.x; bz[u][v + 1] = f.y; bz[u][v + 2] = f.z; bz[u][v + 3] = f.w;
          }
        }
      }
    }
    float z[U][V], x[U][V];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool ok = j0 + u * G < nsrc;
      unpack16(zr[u], (const T*)nullptr, z[u]);
      unpack16(xr[u], (const T*)nullptr, x[u]);
#pragma unroll
      for (int v = 0; v < V; ++v) z[u][v] = ok ? z[u][v] + bz[u][v] : -INFINITY;
    }
#pragma unroll
    for (int v = 0; v < V; ++v) {
      float mx = st[v].mx;
#pragma unroll
      for (int u = 0; u < U; ++u) mx = fmaxf(mx, z[u][v]);
      if (mx == -INFINITY) continue;  // no source here yet
      const float r = __expf(st[v].mx - mx);  // 0 while the state is empty
      float l = st[v].l * r, acc = st[v].acc * r;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float e = __expf(z[u][v] - mx);  // 0 for absent sources
        l += e;
        acc += e * x[u][v];
      }
      st[v] = Soft{mx, l, acc};
    }
  }
  // merge the G groups of every coordinate: the groups of a wavefront are
  // lanes o, o + TR, ...; then the four wavefronts through s_part[w][W]
#pragma unroll
  for (int msk = TR; msk < 64; msk <<= 1) {
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const Soft other{__shfl_xor(st[v].mx, msk, 64), __shfl_xor(st[v].l, msk, 64), __shfl_xor(st[v].acc, msk, 64)};
      st[v] = soft_merge(st[v], other);
    }
  }
  const int wv = tid >> 6;
  if ((tid & 63) < TR) {
#pragma unroll
    for (int v = 0; v < V; ++v) s_part[wv * W + o * V + v] = st[v];
  }
  __syncthreads();
  float val = 0.f;
  if (tid < W) {
    Soft acc = s_part[tid];
#pragma unroll
    for (int g = 1; g < kFoldT / 64; ++g) acc = soft_merge(acc, s_part[g * W + tid]);
    val = acc.acc / acc.l;
  }
  __syncthreads();
  return val;
}

// Stores coordinates 256 u + tid (u < nu) of an entry that a workgroup of
// 256 threads holds (vals[u]) to row `row` of the cache: as T (fmt 0), or as
// the 576-byte FP8 + BF16 entry (fmt 1, c = 512): scale = max |v[0:448]| /
// 448 formed in float32 (1 for an all-zero part), codes e4m3(v / scale),
// then the last 64 coordinates as bf16.  Called by every thread; s_red holds
// four floats.
template <typename T>
CSA_DEV void store_entry(const float* vals, int nu, int c, int fmt, void* cache, float* scales, size_t row,
                         float* s_red) {
  const int tid = threadIdx.x;
  if (!fmt) {
    for (int u = 0; u < nu; ++u) {
      const int r = 256 * u + tid;
      if (r < c) st(reinterpret_cast<T*>(cache), row * c + r, vals[u]);
    }
    return;
  }
  float am = 0.f;
  for (int u = 0; u < nu; ++u)
    if (256 * u + tid < kF8Dims) am = fmaxf(am, fabsf(vals[u]));
  am = wave_max(am);
  __syncthreads();  // s_red is free (earlier reductions' readers are done)
  if ((tid & 63) == 0) s_red[tid >> 6] = am;
  __syncthreads();
  am = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  float scale = am / 448.0f;
  if (!(scale > 0.f)) scale = 1.f;
  uint8_t* o = reinterpret_cast<uint8_t*>(cache) + row * kF8RowB;
  for (int u = 0; u < nu; ++u) {
    const int r = 256 * u + tid;
    if (r < kF8Dims)
      o[r] = f32_to_e4m3(vals[u] / scale);
    else if (r < c)
      *reinterpret_cast<uint16_t*>(o + kF8Dims + 2 * (r - kF8Dims)) = f32_to_bf16(vals[u]);
  }
  if (tid == 0) scales[row] = scale;
}

// One wavefront prepares one vector of length c (64..512, a multiple of 64)
// for the core attention: RMSNorm with scale g, v * g / sqrt(mean(v^2) +
// eps), then the rotary pairs of its last rope_dims coordinates at position
// pos.  Lane l holds coordinates E l .. E l + E - 1, E = c / 64; with E = 1 a
// pair spans lanes l, l ^ 1.  Called by whole wavefronts.
template <typename T>
CSA_DEV void prep_row_wave(const T* src, T* dst, int c, const NormRope& nr, const float* g, int64_t pos) {
  const int l = threadIdx.x & 63, E = c / 64, R = nr.rope_dims;
  float v[8];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    v[j] = j < E ? ld(src, (size_t)l * E + j) : 0.f;
    ss += v[j] * v[j];
  }
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / (float)c + nr.eps);
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (j < E) v[j] *= inv * g[l * E + j];
  if (E >= 2) {
    rope_pairs<8>(v, E, l * E, c, R, nr.inv_freq, pos);
  } else {
    const float o = __shfl_xor(v[0], 1, 64);
    if (l >= c - R) {
      float cs, sn;
      rope_cs(pos, nr.inv_freq[(l - (c - R)) >> 1], &cs, &sn);
      v[0] = (l & 1) ? (o * sn + v[0] * cs) : (v[0] * cs - o * sn);
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (j < E) st(dst, (size_t)l * E + j, v[j]);
}

}  // namespace csa
