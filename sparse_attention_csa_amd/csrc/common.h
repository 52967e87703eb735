// Device helpers shared by the HIP kernels of the CSA/HCA hot path (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define CSA_DEV __device__ __forceinline__
#define CSA_HOST_DEV __host__ __device__

namespace csa {

// ---------------------------------------------------------------- bfloat16
struct bf16 {
  uint16_t bits;
};

CSA_DEV float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// round to nearest even; NaN stays NaN (the gfx950 conversion instruction,
// no branches)
CSA_DEV uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f)); }

// element load / store for the two activation dtypes
CSA_DEV float ld(const float* p, size_t i) { return p[i]; }
CSA_DEV float ld(const bf16* p, size_t i) { return bf16_to_f32(p[i].bits); }
CSA_DEV void st(float* p, size_t i, float v) { p[i] = v; }
CSA_DEV void st(bf16* p, size_t i, float v) { p[i].bits = f32_to_bf16(v); }

// ---------------------------------------------------------------- OCP e4m3fn
// 1 sign, 4 exponent (bias 7), 3 fraction bits; S.1111.111 is NaN; max 448.
CSA_DEV float e4m3_to_f32(uint8_t c) {
  const uint32_t e = (c >> 3) & 0xf, f = c & 7;
  float mag;
  if (e == 0)
    mag = ldexpf((float)f * 0.125f, -6);
  else if (e == 15 && f == 7)
    mag = __builtin_nanf("");
  else
    mag = ldexpf(1.0f + (float)f * 0.125f, (int)e - 7);
  return (c & 0x80) ? -mag : mag;
}

// nearest e4m3fn code of y (|y| clamped to 448), ties to even.
CSA_DEV uint8_t f32_to_e4m3(float y) {
  const uint8_t sign = (y < 0.f) ? 0x80 : 0;
  float a = fminf(fabsf(y), 448.0f);
  if (!(a > 0.f)) return sign;
  int e;
  frexpf(a, &e);                   // a = mant * 2^e, mant in [0.5, 1)
  int sp = e - 4;                  // 4 significant bits
  if (sp < -9) sp = -9;            // subnormal spacing 2^-9
  float r = rintf(ldexpf(a, -sp)); // multiples of the spacing, ties to even
  r = ldexpf(r, sp);
  if (r > 448.f) r = 448.f;
  if (r < ldexpf(1.0f, -6)) {      // subnormal: field 0
    return sign | (uint8_t)(int)rintf(ldexpf(r, 9));
  }
  int er;
  float mr = frexpf(r, &er);       // r = mr * 2^er, mr in [0.5, 1)
  int E = er - 1;                  // r = (2 mr) * 2^E, 2 mr in [1, 2)
  int f = (int)rintf((2.f * mr - 1.f) * 8.f);
  return sign | (uint8_t)(((E + 7) << 3) | f);
}

// ---------------------------------------------------------------- OCP MX FP4
// E2M1 elements (1 sign, 2 exponent bits with bias 1, 1 fraction bit;
// magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6) in blocks of 32 sharing one E8M0
// scale 2^(code - 127).  Two elements per byte, element 2j in the low
// nibble of byte j.
struct mx4 {};   // tag type: MXFP4 storage (a kernel template argument)
struct f8b16 {};  // tag type: the 576-byte FP8 + BF16 main entry

CSA_DEV float e2m1_to_f32(uint32_t c) {
  const uint32_t e = (c >> 1) & 3u, f = c & 1u;
  const float mag = e == 0 ? 0.5f * (float)f : ldexpf(1.0f + 0.5f * (float)f, (int)e - 1);
  return (c & 8u) ? -mag : mag;
}

CSA_DEV float e8m0_to_f32(uint32_t code) { return ldexpf(1.0f, (int)code - 127); }

// E2M1 code of y (already divided by its block scale): the nearest value,
// ties to the even code, saturating at 6
CSA_DEV uint32_t f32_to_e2m1(float y) {
  const float a = fabsf(y);
  const float sp = a < 2.f ? 0.5f : (a < 4.f ? 1.f : 2.f);
  const float r = fminf(rintf(a / sp) * sp, 6.f);  // rintf: half to even on the multiple
  const uint32_t mag = r < 2.f ? (uint32_t)(2.f * r) : (r < 4.f ? 2u + (uint32_t)r : (r == 4.f ? 6u : 7u));
  return (y < 0.f && mag) ? (mag | 8u) : mag;
}

// E8M0 code of a block whose largest magnitude is amax:
// 2^(floor(log2 amax) - 2), the smallest scale for an all-zero block
CSA_DEV uint32_t mx_scale_code(float amax) {
  if (!(amax > 0.f)) return 0u;
  int e;
  frexpf(amax, &e);  // amax = f 2^e, f in [0.5, 1): floor(log2 amax) = e - 1
  const int c = e - 1 - 2 + 127;
  return (uint32_t)(c < 0 ? 0 : (c > 254 ? 254 : c));
}

// The lanes of aligned groups of 32 hold one block's elements (lane
// i of the group: element i).  Returns this lane's E2M1 code; *scale gets
// the block's E8M0 code.
CSA_DEV uint32_t mx_quantize_lane(float v, uint32_t* scale) {
  float am = fabsf(v);
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) am = fmaxf(am, __shfl_xor(am, o, 64));
  const uint32_t sc = mx_scale_code(am);
  *scale = sc;
  return f32_to_e2m1(ldexpf(v, 127 - (int)sc));
}

// ---------------------------------------------------------------- top-k keys
// nearest-even bf16 value of f, as a float (bf16 index scores)
CSA_DEV float round_bf16(float f) { return bf16_to_f32(f32_to_bf16(f)); }

// order-preserving map float -> uint32 (larger float -> larger key)
CSA_DEV uint32_t f32_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------- reductions
CSA_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
CSA_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// ---------------------------------------------------------------- rotary positions
// cos and sin of the angle pos * f: the product and its reduction to
// [-pi, pi] in double (a float angle at position 10^6 would be off by a
// large fraction of a radian), the functions in float
CSA_DEV void rope_cs(int64_t pos, double f, float* cs, float* sn) {
  const double ang = (double)pos * f;
  const double r = ang - 6.283185307179586 * rint(ang * 0.15915494309189535);
  sincosf((float)r, sn, cs);
}

// Rotate the pairs (v[j], v[j+1]), j even and j < n <= N, holding
// coordinates d0 + j of a vector of length c whose last R coordinates are
// rotary (d0 and c - R even), by the angles pos * inv_freq[i] (pair
// i = (d - (c - R)) / 2); the other coordinates stay.
template <int N>
CSA_DEV void rope_pairs(float* v, int n, int d0, int c, int R, const double* inv_freq, int64_t pos) {
#pragma unroll
  for (int j = 0; j < N; j += 2) {
    const int d = d0 + j;
    if (j < n && d >= c - R) {
      float cs, sn;
      rope_cs(pos, inv_freq[(d - (c - R)) >> 1], &cs, &sn);
      const float x = v[j], y = v[j + 1];
      v[j] = x * cs - y * sn;
      v[j + 1] = x * sn + y * cs;
    }
  }
}

// v + the values of lanes l^16, l^32 and l^48 (the four 16-lane rows), with
// the gfx950 lane-swap instructions instead of LDS permutes
CSA_DEV float lane_sum_xor16_32(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// Workgroup barrier that orders LDS only.  __syncthreads() also waits for
// every outstanding global access of the wave (vmcnt(0)), which would drain
// asynchronous global-to-LDS prefetches; callers that need those complete
// wait for them explicitly.
CSA_DEV void lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Workgroup barrier for LDS written by ordinary LDS stores only, while
// global-to-LDS DMAs may still be in flight: waits for this wave's LDS
// operations (lgkmcnt = 0; vmcnt and expcnt are not waited), then s_barrier.
// The empty asm statements keep the compiler from moving memory accesses
// across.  (An LDS-scoped release fence would also wait for the in-flight
// DMAs, since they write LDS.)  DMA'd data is published by waiting for its
// vmcnt explicitly before this barrier.
constexpr int kWaitLgkm0 = 0xC07F;  // gfx9 s_waitcnt: vmcnt 63, expcnt 7, lgkmcnt 0
CSA_DEV void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __asm__ __volatile__("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ __volatile__("" ::: "memory");
}

// LDS atomic add without return.  Issued as inline asm so that the
// compiler's wait insertion does not treat it as possibly overlapping
// in-flight global-to-LDS DMAs into other LDS arrays (it would otherwise
// wait for every outstanding DMA first).  Callers guarantee that p is not in
// any region still being filled by DMA.  No result register, so nothing is
// read before the add completes; later LDS reads wait for it through lgkmcnt
// as usual (LDS operations complete in order).
CSA_DEV void lds_add_noret(int* p, int v) {
  const uint32_t addr = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) int*)p);
  __asm__ __volatile__("ds_add_u32 %0, %1" ::"v"(addr), "v"(v) : "memory");
}

// visible-entry limit for a query at position t
CSA_DEV int64_t vis_limit(int64_t t, int m, int vis) { return vis == 0 ? t / m : (t + 1) / m; }


}  // namespace csa
