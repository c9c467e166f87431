// Rotary position embedding arithmetic shared by the RoPE append kernel
// (rope.hip) and the attention kernel that rotates as it loads
// (attn_stream.hip), so that both produce the same bits.
//
// Channel pair (j, j + d/2) of a row at position pos turns by the angle
// pos * base^(-2j/d) ("rotate half"; SwiftSpec summary, Section 3.3: the
// masked attention takes the position embedding).  The angle is reduced
// modulo 2 pi in double precision (positions reach tens of thousands, where a
// float product would be off by ~1e-3 rad), its cosine and sine rounded to
// float; the rotation is done in float with every product and sum rounded on
// its own (no fused multiply-add), then stored in the tensor's dtype.
#pragma once

#include <hip/hip_runtime.h>

namespace ta {

__device__ __forceinline__ double rope_inv_freq(float base, int j, int d) {
  return pow(static_cast<double>(base), -2.0 * j / d);
}

__device__ __forceinline__ void rope_cos_sin(int pos, double inv_freq, float& c, float& s) {
  const double two_pi = 6.283185307179586476925286766559;
  const double a = fmod(static_cast<double>(pos) * inv_freq, two_pi);
  c = static_cast<float>(cos(a));
  s = static_cast<float>(sin(a));
}

__device__ __forceinline__ void rope_rotate(float x0, float x1, float c, float s, float& y0,
                                            float& y1) {
  y0 = __fsub_rn(__fmul_rn(x0, c), __fmul_rn(x1, s));
  y1 = __fadd_rn(__fmul_rn(x1, c), __fmul_rn(x0, s));
}

}  // namespace ta
