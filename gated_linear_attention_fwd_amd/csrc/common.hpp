// common.hpp -- device helpers shared by the HIP kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gla {

// bfloat16 storage type: raw bits. The library never relies on a vendor bf16
// class so that the rounding used for the output is the one written here.
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest, ties to even. Inputs are finite (NaN handling is not needed
// for the outputs of this operation on finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ float relu(float x) { return x > 0.f ? x : 0.f; }

// Logistic sigmoid in fp32; exp overflow to +inf gives exactly 0, as it should.
__device__ __forceinline__ float sigmoid(float x) { return 1.f / (1.f + __expf(-x)); }

// Element access for the two storage dtypes.
template <typename T> struct Elem;

template <> struct Elem<float> {
  __device__ __forceinline__ static float load(const float *p, int64_t i) { return p[i]; }
  __device__ __forceinline__ static void store(float *p, int64_t i, float x) { p[i] = x; }
  // 4 consecutive elements (16-byte aligned when i % 4 == 0)
  __device__ __forceinline__ static float4 load4(const float *p, int64_t i) {
    return *reinterpret_cast<const float4 *>(p + i);
  }
  __device__ __forceinline__ static void store4(float *p, int64_t i, float4 x) {
    *reinterpret_cast<float4 *>(p + i) = x;
  }
};

template <> struct Elem<bf16_t> {
  __device__ __forceinline__ static float load(const bf16_t *p, int64_t i) {
    return bf16_to_f32(p[i].bits);
  }
  __device__ __forceinline__ static void store(bf16_t *p, int64_t i, float x) {
    p[i].bits = f32_to_bf16_rne(x);
  }
  __device__ __forceinline__ static float4 load4(const bf16_t *p, int64_t i) {
    const uint2 w = *reinterpret_cast<const uint2 *>(p + i);
    return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                       __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u));
  }
  __device__ __forceinline__ static void store4(bf16_t *p, int64_t i, float4 x) {
    uint2 w;
    w.x = static_cast<uint32_t>(f32_to_bf16_rne(x.x)) |
          (static_cast<uint32_t>(f32_to_bf16_rne(x.y)) << 16);
    w.y = static_cast<uint32_t>(f32_to_bf16_rne(x.z)) |
          (static_cast<uint32_t>(f32_to_bf16_rne(x.w)) << 16);
    *reinterpret_cast<uint2 *>(p + i) = w;
  }
};

// ---- 3D rotary positions -------------------------------------------------
// (cos a, sin a) for a = pos * freq (freq = theta^(-j/m), m > 0). The angle is
// formed and reduced to [-pi, pi] in double precision, so the fp32 sincosf sees
// a small argument at any position.
__device__ inline float2 rope_cs_at(double pos, double freq) {
  constexpr double kTwoPi = 6.283185307179586476925286766559;
  const double a = pos * freq;
  const double r = a - kTwoPi * rint(a * (1.0 / kTwoPi));
  float s, c;
  sincosf((float)r, &s, &c);
  return make_float2(c, s);
}

// theta^(-j/m), formed in double precision
__device__ inline double rope_freq(int j, int m, double log_theta) {
  return exp(-((double)j / (double)m) * log_theta);
}

// (cos a, sin a) for a = pos * theta^(-j/m)
__device__ inline float2 rope_cs(double pos, int j, int m, double log_theta) {
  return rope_cs_at(pos, rope_freq(j, m, log_theta));
}

// (y, x) = (l / gw, l % gw) for 0 <= l < 2^31: the double quotient is off by
// at most one, which the remainder test corrects.
__device__ __forceinline__ void grid_pos(int l, int gw, double inv_gw, int &y, int &x) {
  int yy = (int)((double)l * inv_gw);
  int xx = l - yy * gw;
  if (xx < 0) {
    --yy;
    xx += gw;
  } else if (xx >= gw) {
    ++yy;
    xx -= gw;
  }
  y = yy;
  x = xx;
}

// (cos, sin) of feature pair p of token l in frame f: the whole turn, temporal
// or spatial, computed directly (the vector-ALU kernels keep no tables, unlike
// the matrix-core path). R is the validated rotation record (RopeK).
template <class R>
__device__ float2 token_rope_cs(const R &r, int f, int l, int p) {
  if (p < r.Pt) return rope_cs((double)r.frame_offset + f, p, r.Pt, r.log_theta);
  int y, x;
  grid_pos(l, r.grid_w, r.inv_gw, y, x);
  if (p < r.Pt + r.Ph) return rope_cs((double)y, p - r.Pt, r.Ph, r.log_theta);
  return rope_cs((double)x, p - r.Pt - r.Ph, r.Pw, r.log_theta);
}

// The frequency theta^(-j/m) of feature pair p (kernels that turn many tokens
// keep these in a table and call token_rope_cs_freq: the same angles).
template <class R>
__device__ double pair_freq(const R &r, int p) {
  if (p < r.Pt) return rope_freq(p, r.Pt, r.log_theta);
  if (p < r.Pt + r.Ph) return rope_freq(p - r.Pt, r.Ph, r.log_theta);
  return rope_freq(p - r.Pt - r.Ph, r.Pw, r.log_theta);
}

template <class R>
__device__ float2 token_rope_cs_freq(const R &r, int f, int l, int p, double freq) {
  if (p < r.Pt) return rope_cs_at((double)r.frame_offset + f, freq);
  int y, x;
  grid_pos(l, r.grid_w, r.inv_gw, y, x);
  return rope_cs_at((double)(p < r.Pt + r.Ph ? y : x), freq);
}

// Rotate the feature pair (a, b) by the angle whose (cos, sin) is cs:
// (a, b) -> (a cos - b sin, a sin + b cos).
__device__ __forceinline__ float2 rotate_pair(float a, float b, float2 cs) {
  return make_float2(fmaf(a, cs.x, -b * cs.y), fmaf(a, cs.y, b * cs.x));
}

}  // namespace gla
