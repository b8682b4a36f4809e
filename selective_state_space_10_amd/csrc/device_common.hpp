// device_common.hpp -- gfx950 device helpers shared by the scan kernels:
// io-type loads/stores (fp32, bf16 with round-to-nearest-even), the step-size
// nonlinearity (softplus) and the SiLU gate, built on the hardware exp2/log2/rcp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct bf16 {
  uint16_t bits;
};

template <typename IO>
struct io_traits;
template <>
struct io_traits<float> {
  static constexpr int bytes = 4;
};
template <>
struct io_traits<bf16> {
  static constexpr int bytes = 2;
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits) { return __uint_as_float(bits << 16); }

// fp32 -> bf16, round to nearest even; NaN stays NaN (quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t x = __float_as_uint(f);
  if ((x & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((x >> 16) | 0x40u);
  x += 0x7fffu + ((x >> 16) & 1u);
  return (uint16_t)(x >> 16);
}

__device__ __forceinline__ float load_io(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float load_io(const bf16* p, int64_t i) { return bf16_bits_to_f32(p[i].bits); }
// the IO type stored at a byte offset from a base
template <typename IO>
__device__ __forceinline__ float load_io_b(const char* p, uint32_t o) { return load_io(reinterpret_cast<const IO*>(p + o), 0); }
__device__ __forceinline__ void store_io(float* p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void store_io(bf16* p, int64_t i, float v) { p[i].bits = f32_to_bf16_bits(v); }

// Four consecutive elements (16 B of fp32, 8 B of bf16); the index is a
// multiple of 4 and the base is 16-byte aligned.
template <typename IO>
struct Vec4;
template <>
struct Vec4<float> {
  typedef float4 raw;
  static __device__ __forceinline__ raw load(const float *p, int64_t i) { return *(const float4 *)(p + i); }
  // at a byte offset from a base
  static __device__ __forceinline__ raw load_b(const char *p, uint32_t o) { return *(const float4 *)(p + o); }
  static __device__ __forceinline__ void store_b(char *p, uint32_t o, float4 v) { *(float4 *)(p + o) = v; }
  static __device__ __forceinline__ raw splat_b(const char *p, uint32_t o) {
    const float v = *(const float *)(p + o);
    return make_float4(v, v, v, v);
  }
  static __device__ __forceinline__ float4 cvt(raw r) { return r; }
  static __device__ __forceinline__ void store(float *p, int64_t i, float4 v) { *(float4 *)(p + i) = v; }
  // one element, repeated four times
  static __device__ __forceinline__ raw splat(const float *p, int64_t i) {
    const float v = p[i];
    return make_float4(v, v, v, v);
  }
};
template <>
struct Vec4<bf16> {
  typedef uint2 raw;
  static __device__ __forceinline__ raw load(const bf16 *p, int64_t i) { return *(const uint2 *)(p + i); }
  static __device__ __forceinline__ raw load_b(const char *p, uint32_t o) { return *(const uint2 *)(p + o); }
  static __device__ __forceinline__ void store_b(char *p, uint32_t o, float4 v) { store(reinterpret_cast<bf16 *>(p + o), 0, v); }
  static __device__ __forceinline__ raw splat_b(const char *p, uint32_t o) {
    const uint32_t b = *(const uint16_t *)(p + o);
    const uint32_t w = b | (b << 16);
    return make_uint2(w, w);
  }
  static __device__ __forceinline__ float4 cvt(raw r) {
    return make_float4(__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u),
                       __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xffff0000u));
  }
  static __device__ __forceinline__ void store(bf16 *p, int64_t i, float4 v) {
    uint2 o;
    o.x = (uint32_t)f32_to_bf16_bits(v.x) | ((uint32_t)f32_to_bf16_bits(v.y) << 16);
    o.y = (uint32_t)f32_to_bf16_bits(v.z) | ((uint32_t)f32_to_bf16_bits(v.w) << 16);
    *(uint2 *)(p + i) = o;
  }
  static __device__ __forceinline__ raw splat(const bf16 *p, int64_t i) {
    const uint32_t b = p[i].bits;
    const uint32_t w = b | (b << 16);
    return make_uint2(w, w);
  }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// softplus(s) = log(1 + e^s) = max(s, 0) + log1p(e^-|s|).
// log1p(w) for w in (0, 1] is log(1 + w) corrected by the rounding error of
// 1 + w: with v = fl(1 + w) and c = (v - 1) - w (exact), log1p(w) = log(v) - c
// up to a relative 2^-24 term.  No branch; for large |s| the log term is e^-|s|.
__device__ __forceinline__ float softplus_f(float s) {
  const float w = fast_exp2(-fabsf(s) * kLog2e);
  const float v = 1.0f + w;
  const float c = (v - 1.0f) - w;
  const float l = fast_log2(v) * kLn2 - c;
  return fmaxf(s, 0.0f) + l;
}

// logistic sigmoid 1 / (1 + e^-x); saturates to 0 / 1 without NaN for finite x.
__device__ __forceinline__ float sigmoid_f(float x) { return fast_rcp(1.0f + fast_exp2(-x * kLog2e)); }

__device__ __forceinline__ float silu_f(float x) { return x * sigmoid_f(x); }

// Input coefficient of the exact zero-order hold, expm1(x) / A with x = dt*A,
// given da = exp(x) and Ainv = 1/A.  For |x| >= 1/4, (da - 1) * Ainv loses at
// most 2^-24 / (1 - e^-1/4) relative; below that, dt * (e^x - 1)/x by its
// Taylor polynomial of degree 5 (remainder below x^6/5040 < 5e-8).  A = 0
// gives x = 0 and so dt.
__device__ __forceinline__ float zoh_coef(float dt, float x, float da, float Ainv) {
  const float phi = fmaf(x, fmaf(x, fmaf(x, fmaf(x, fmaf(x, 1.0f / 720, 1.0f / 120), 1.0f / 24), 1.0f / 6), 0.5f), 1.0f);
  return fabsf(x) < 0.25f ? dt * phi : (da - 1.0f) * Ainv;
}

// d/dA of expm1(dt A)/A = dt^2 psi(x), psi(x) = (x e^x - e^x + 1)/x^2: the
// Taylor polynomial sum_k x^k (k+1)/(k+2)! up to k = 5 for |x| < 1/4, else
// (dt da - coef) * Ainv.
__device__ __forceinline__ float zoh_dcoef_dA(float dt, float x, float da, float coef, float Ainv) {
  const float psi = fmaf(x, fmaf(x, fmaf(x, fmaf(x, fmaf(x, 1.0f / 840, 1.0f / 144), 1.0f / 30), 0.125f), 1.0f / 3), 0.5f);
  return fabsf(x) < 0.25f ? dt * dt * psi : (dt * da - coef) * Ainv;
}

// Step size from the raw input: softplus(raw + bias) or raw + bias.
__device__ __forceinline__ float step_size(float raw, float bias, bool softplus) {
  const float s = raw + bias;
  return softplus ? softplus_f(s) : s;
}

// ---- wave-wide associative scan of affine maps
//
// A step of the recurrence, h -> a h + b, is an affine map; applying (a1, b1)
// and then (a2, b2) gives (a1 a2, a2 b1 + b2), an associative composition with
// identity (1, 0) (the same algebra that lets the scan be split over time and
// recombined).  wave_affine_scan replaces each lane's pair by the composition
// of the pairs of lanes 0 .. lane, in lane order (an inclusive scan over the
// 64 lanes of a wave), in six steps of cross-lane moves: DPP shifts by 1, 2,
// 4 and 8 lanes inside each row of 16, then the last lane of row 0 into row
// 1 and of row 2 into row 3 (row_bcast:15), then lane 31 into rows 2 and 3
// (row_bcast:31).  A lane whose source lies outside the row, or whose row is
// masked off, takes the identity.  Every lane of the wave must be active.

template <int CTRL, int ROWMASK>
__device__ __forceinline__ float dpp_or(float identity, float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, identity),
                                                               __builtin_bit_cast(int, v), CTRL,
                                                               ROWMASK, 0xF, false));
}

// (a, b) <- (a_prev, b_prev) o (a, b) with the pair CTRL brings from another lane
template <int CTRL, int ROWMASK>
__device__ __forceinline__ void affine_step(float &a, float &b) {
  const float ap = dpp_or<CTRL, ROWMASK>(1.0f, a);
  const float bp = dpp_or<CTRL, ROWMASK>(0.0f, b);
  b = fmaf(a, bp, b);
  a = ap * a;
}

__device__ __forceinline__ void wave_affine_scan(float &a, float &b) {
  affine_step<0x111, 0xF>(a, b);  // row_shr:1
  affine_step<0x112, 0xF>(a, b);  // row_shr:2
  affine_step<0x114, 0xF>(a, b);  // row_shr:4
  affine_step<0x118, 0xF>(a, b);  // row_shr:8
  affine_step<0x142, 0xA>(a, b);  // row_bcast:15 into rows 1 and 3
  affine_step<0x143, 0xC>(a, b);  // row_bcast:31 into rows 2 and 3
}

// Returns z (always 0) through an opaque register move that reads every 32-bit
// word of the given values: code whose operands depend on the result cannot be
// scheduled before those values are computed and read.
template <typename... Ts>
__device__ __forceinline__ int after_all(int z, const Ts &...vals) {
  constexpr int W = (0 + ... + (int)(sizeof(Ts) / 4));
  uint32_t w[W];
  int n = 0;
  auto put = [&](const auto &v) {
    static_assert(sizeof(v) % 4 == 0, "whole 32-bit words");
    const auto *p = reinterpret_cast<const uint32_t *>(&v);
#pragma unroll
    for (int i = 0; i < (int)(sizeof(v) / 4); ++i) w[n++] = p[i];
  };
  (put(vals), ...);
#pragma unroll
  for (int i = 0; i < W; i += 8) {  // eight words per move
    auto at = [&](int k) { return w[i + k < W ? i + k : W - 1]; };
    int out;
    asm volatile("v_mov_b32 %0, %1" : "=v"(out)
                 : "v"(z), "v"(at(0)), "v"(at(1)), "v"(at(2)), "v"(at(3)), "v"(at(4)), "v"(at(5)),
                   "v"(at(6)), "v"(at(7))
                 : "memory");
    z = out;
  }
  return z;
}

}  // namespace ssm
