// device_math.h -- float32 numerics of the decoder (gfx950 device code).
//
// The log-domain sum used everywhere is the page's logsumexp ("GPU CTC Prefix
// Beam Search Decoder", sec. 3): max(a,b) + log(1 + exp(-|a-b|)), with
// -FLT_MAX as the additive identity.  exp and log1p are written out as fixed
// float32 operation sequences so that every build of this library computes
// the same bits:
//   exp(x),   x in [-80, 0]: Cody & Waite reduction x = n ln2 + r (ln2 split
//             into a 16-significant-bit head and a tail), degree-7 Taylor
//             polynomial of e^r in Horner form with fused multiply-adds, exact
//             scaling by 2^n;
//   log1p(x), x in [0, 1]: 2 atanh(s), s = x / (2 + x), odd series up to
//             s^15 summed as s + s z q(z), z = s^2, q in Horner form.
// The correction term is dropped when min - max < -80, which keeps every
// intermediate a normal number.  The file must be compiled with
// -ffp-contract=off: each operation written here rounds once.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ctcpb {

constexpr float kNeg = -3.40282346638528859811704183484516925e+38f;  // -FLT_MAX

__device__ __forceinline__ float exp_m80_0(float x) {
  const float n = __builtin_rintf(x * 0x1.715476p+0f);
  float r = __builtin_fmaf(-n, 0x1.62e4p-1f, x);
  r = __builtin_fmaf(-n, 0x1.7f7d1cp-20f, r);
  float p = 0x1.a01a02p-13f;
  p = __builtin_fmaf(p, r, 0x1.6c16c2p-10f);
  p = __builtin_fmaf(p, r, 0x1.111112p-7f);
  p = __builtin_fmaf(p, r, 0x1.555556p-5f);
  p = __builtin_fmaf(p, r, 0x1.555556p-3f);
  p = __builtin_fmaf(p, r, 0x1.0p-1f);
  p = __builtin_fmaf(p, r, 1.0f);
  p = __builtin_fmaf(p, r, 1.0f);
  return __builtin_ldexpf(p, (int)n);
}

// x / (2 + x) for x in [0, 1], correctly rounded: the reciprocal of the
// divisor (in [2, 3]) refined by one Newton step, then the quotient corrected
// once by its exact residual.  Checked bit for bit against the IEEE division
// on every float in [0, 1]; needs none of the general division's scaling.
__device__ __forceinline__ float quot_x_2px(float x) {
  const float d = 2.0f + x;
  const float y0 = __builtin_amdgcn_rcpf(d);
  const float e = __builtin_fmaf(-d, y0, 1.0f);
  const float y1 = __builtin_fmaf(e, y0, y0);
  const float q0 = x * y1;
  const float r = __builtin_fmaf(-d, q0, x);
  return __builtin_fmaf(r, y1, q0);
}

__device__ __forceinline__ float log1p_0_1(float x) {
  const float s = quot_x_2px(x);
  const float z = s * s;
  float q = 0x1.111112p-4f;
  q = __builtin_fmaf(q, z, 0x1.3b13b2p-4f);
  q = __builtin_fmaf(q, z, 0x1.745d18p-4f);
  q = __builtin_fmaf(q, z, 0x1.c71c72p-4f);
  q = __builtin_fmaf(q, z, 0x1.24924ap-3f);
  q = __builtin_fmaf(q, z, 0x1.99999ap-3f);
  q = __builtin_fmaf(q, z, 0x1.555556p-2f);
  const float r = __builtin_fmaf(s * z, q, s);
  return r + r;
}

__device__ __forceinline__ float lse(float a, float b) {
  const bool ge = a >= b;
  const float m = ge ? a : b;
  const float d = (ge ? b : a) - m;
  // without a branch: the correction is computed on an in-range stand-in and
  // discarded when min - max < -80 (or NaN)
  const bool in = d >= -80.0f;
  const float r = m + log1p_0_1(exp_m80_0(in ? d : 0.0f));
  return in ? r : m;
}

// Order-preserving map float -> uint32 (ascending).  -0.0 is first turned
// into +0.0 so that the two zeros, equal as floats, map to one key.
__device__ __forceinline__ uint32_t sortable(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  // negatives: all bits flipped; non-negatives: the sign bit set
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

__device__ __forceinline__ float unsortable(uint32_t s) {
  const uint32_t u = (s & 0x80000000u) ? (s & 0x7fffffffu) : ~s;
  return __uint_as_float(u);
}

// Composite selection key: descending order of the 64-bit value is
// (score descending, id ascending).  0 is below every real key.
__device__ __forceinline__ uint64_t compose(float key, uint32_t id) {
  return ((uint64_t)sortable(key) << 32) | (uint32_t)(~id);
}
__device__ __forceinline__ float comp_key(uint64_t c) { return unsortable((uint32_t)(c >> 32)); }
__device__ __forceinline__ uint32_t comp_id(uint64_t c) { return ~(uint32_t)c; }

// Keys whose score is NEG (or below) are not candidates.
__device__ __forceinline__ uint64_t comp_floor() {
  return ((uint64_t)0x00800000u << 32) | 0xffffffffu;  // sortable(-FLT_MAX), id 0
}

// Mix of a token into a 32-bit prefix hash: xor, multiply by an odd
// constant, xor-shift (each a bijection of the 32-bit state, so prefixes of
// one length that differ in one label never collide).  Used only as a filter
// before an exact token comparison.
__device__ __forceinline__ uint32_t hash_push(uint32_t h, int tok) {
  uint32_t x = (h ^ (uint32_t)(tok + 1)) * 0x9e3779b1u;
  return x ^ (x >> 16);
}
constexpr uint32_t kHashEmpty = 0x4f6cdd1du;

}  // namespace ctcpb
