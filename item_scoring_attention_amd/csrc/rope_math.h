// Rotary embedding arithmetic shared by the rotation pass, the cos/sin table
// and the attention kernels that rotate Q while they load it, so that all of
// them produce the same bits for the same (position, pair).
//
// From Generation to Scoring, §4.1 (position-id rule) fixes the positions:
// prefix token u at u, the token at offset d inside any item at Lq + d. The
// rotation itself is the usual rotary embedding of the decoder families the
// pages use: dims i and i + D/2 of a head row form a pair turned by the
// angle pos * theta^(-2i/D).
#pragma once

#include <hip/hip_runtime.h>

namespace mis {

constexpr double kRopeTwoPi = 6.283185307179586476925286766559;
constexpr double kRopeInvTwoPi = 0.15915494309189533576888376337251;

// cos and sin of pos * inv (inv = theta^(-2i/D)): the product and its
// reduction modulo 2 pi in fp64, sin and cos of the reduced angle in fp32.
__device__ __forceinline__ void rope_cos_sin(double pos, double inv, float &c, float &s) {
  double a = pos * inv;
  a -= kRopeTwoPi * rint(a * kRopeInvTwoPi);
  sincosf(float(a), &s, &c);
}

// (a, b) = dims (i, i + D/2) of one head row, turned by the angle whose cos
// and sin are (c, s). The two products and the fused adds are spelled out so
// every caller rounds the same way.
__device__ __forceinline__ void rope_rotate(float &a, float &b, float c, float s) {
  const float ra = __builtin_fmaf(a, c, -(b * s));
  const float rb = __builtin_fmaf(b, c, a * s);
  a = ra;
  b = rb;
}

// Eight bf16 pairs: lo holds dims i .. i + 7, hi dims i + D/2 .. i + D/2 + 7,
// cs the (cos, sin) of pairs i .. i + 7 as consecutive floats. Results are
// rounded to bf16 (nearest even), as the rotation pass stores them.
template <typename V8>
__device__ __forceinline__ void rope_rotate8(V8 &lo, V8 &hi, const float (&cs)[16]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float a = float(lo[e]), b = float(hi[e]);
    rope_rotate(a, b, cs[2 * e], cs[2 * e + 1]);
    lo[e] = __bf16(a);
    hi[e] = __bf16(b);
  }
}

}  // namespace mis
