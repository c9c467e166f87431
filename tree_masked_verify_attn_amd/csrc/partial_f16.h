// Partial states of split rows in half precision: what the bf16 MFMA
// attention kernels leave for their combine launches.
//
// A piece of a row's keys (a split, or a piece of a job cut by a range
// boundary) ends with its running maximum m (log2 units), its sum l and its
// output o = sum p v.  o is kept in fp16 after a power-of-two scale 2^-e per
// row: e puts the row's largest magnitude in [2^14, 2^15), so no channel
// passes fp16's largest value and every channel within 2^28 of the largest
// stays a normal fp16 number, rounded to 11 significant bits (relative error
// at most 2^-11, eight times finer than the bf16 output the combine writes).
// The scaling itself is exact.  That halves the bytes written at the end of
// every piece and read back by the combine, against fp32.
//
// Layout: ws_o holds [parts][d] fp16 values, ws_ml [parts] records of
// {m, l, e, 0} (16 bytes).
#pragma once

#include "ta_device.h"

namespace ta {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x3 __attribute__((ext_vector_type(3)));

struct PartialRec {
  float m, l, e, unused;
};

// Scale exponent e of one row held, in the 32x32 MFMA output layout, by lanes
// i and i ^ 32 (acc[mb][r] = channel 32 mb + 8 (r / 4) + 4 (lane / 32) + r % 4).
// Every lane of the wave must execute it (cross-lane swap).
template <int MB>
__device__ __forceinline__ int partial_exp(const f32x16 (&acc)[MB]) {
  float mx[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    mx[mb] = fabsf(acc[mb][0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) mx[mb] = fmaxf(mx[mb], fabsf(acc[mb][r]));
  }
  float amax = mx[0];
#pragma unroll
  for (int mb = 1; mb < MB; ++mb) amax = fmaxf(amax, mx[mb]);
  const uint32_t u = __float_as_uint(amax);
  const auto s = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  amax = fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
  return (amax > 0.f && amax < INFINITY) ? __builtin_amdgcn_frexp_expf(amax) - 15 : 0;
}

// This lane's channels of the row (o scaled by 2^-e) into orow, and the row's
// record from the lane of the lower half.
template <int MB>
__device__ __forceinline__ void store_partial_f16(const f32x16 (&acc)[MB], float m, float l, int e,
                                                  int lhi, uint16_t* orow, PartialRec* rec) {
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      f16x4 h;
#pragma unroll
      for (int i = 0; i < 4; ++i) h[i] = static_cast<_Float16>(ldexpf(acc[mb][4 * q4 + i], -e));
      *reinterpret_cast<f16x4*>(orow + 32 * mb + 8 * q4 + 4 * lhi) = h;
    }
  if (lhi == 0) *reinterpret_cast<f32x4*>(rec) = f32x4{m, l, static_cast<float>(e), 0.f};
}

// Four channels of a stored row and the row's record, as loaded; the
// conversion waits for both loads, so a caller loads a whole batch first.
// (The record's unused fourth word is not loaded: a loaded value that is
// never read frees its register at once, and the next write to it would
// wait for the load.)
struct PartialF16 {
  f32x3 rec;  // m, l, e
  f16x4 h;
};
__device__ __forceinline__ PartialF16 load_partial_f16(const uint16_t* o4, const PartialRec* rec) {
  return PartialF16{*reinterpret_cast<const f32x3*>(rec), *reinterpret_cast<const f16x4*>(o4)};
}
// o += w * (the piece's output) for those channels: 2^e goes into the weight,
// and the products take the fp16 values directly.  (A piece whose weighted
// output lies below 2^-134 contributes nothing: far below any bf16 result.)
__device__ __forceinline__ void add_partial_f16(f32x4& o, const PartialF16& x, float w) {
  const float we = ldexpf(w, static_cast<int>(x.rec[2]));
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = fmaf(static_cast<float>(x.h[i]), we, o[i]);
}

}  // namespace ta
