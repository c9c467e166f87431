// Pieces shared by the streaming attention kernels (attn_stream.hip,
// attn_units.hip): vector types, the XOR-swizzled LDS layout of a K/V stage,
// the LDS-DMA issue and its explicit waits, and the stage geometry.
#pragma once

#include "partial_f16.h"
#include "ta_device.h"

namespace ta {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) uint8_t lds_u8;

constexpr int kThreads = 256;
constexpr int kTile = 32;             // KV positions per ring stage
constexpr float kRescaleSlack = 8.f;  // log2 units: a larger new maximum rescales the state
constexpr float kRescaleMax = 64.f;   // log2 units: p stay below 2^64; a larger jump outweighs the state
constexpr float kLn2 = 0.69314718055994530942f;
constexpr int kMaxSplitBlocks = 512;  // paged: block ids of one split cached in LDS

template <int D>
__device__ __forceinline__ int swz(int t) {
  const int h = ((t & 3) << 1) | ((t >> 2) & 1);
  return D == 128 ? (h | (((t >> 3) & 1) << 3)) : h;
}
template <int D>
__device__ __forceinline__ int lds_off(int t, int chunk) {  // bytes within a K or V stage
  return t * (D * 2) + ((chunk ^ swz<D>(t)) << 4);
}

// x combined with the value of the lane 32 apart, the same in both lanes:
// v_permlane32_swap of x with itself leaves the lower half's values in both
// halves of one result and the upper half's in both halves of the other.
__device__ __forceinline__ float halves_max(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 64 lanes x 16 bytes from `g` (per lane) into LDS [lds_base, lds_base + 1 KiB).
// The KV stream is read once per call: the loads carry the non-temporal (nt)
// cache policy, which on MI355X also raises the rate of this LDS-DMA path
// from about 6.1 to 6.8 TB/s.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt"
               :
               : "s"(lds_base), "v"(g)
               : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
// Workgroup barrier without the fence of __syncthreads (which would wait for
// every outstanding load); the wave's own LDS reads are complete first.
__device__ __forceinline__ void raw_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
}

template <int D, int NRG, int S>
struct SCfg {
  static constexpr int CH = D / 8;                  // 16-byte chunks per row
  static constexpr int ROW = D * 2;                 // bytes per row
  static constexpr int HALF = kTile * ROW;          // K (or V) bytes per stage
  static constexpr int STAGE = 2 * HALF;
  static constexpr int ROWS_PER_INST = 1024 / ROW;  // rows one 1 KiB load covers
  static constexpr int INST_PER_WAVE = HALF / 1024 / 4;  // per wave, for K (same for V)
  static constexpr int NL = 2 * INST_PER_WAVE;      // loads per thread per stage
  static constexpr int KS = D / 16;
  static constexpr int MB = D / 32;
  static constexpr int RPT = 32 * NRG;
  static constexpr int RING = S * STAGE;
  static constexpr int SETUP = kMaxNodes * kMaskWords * 8 + kMaxNodes * 4;  // anc + jump
  static constexpr int LDS = RING > SETUP ? RING : SETUP;
};

template <int N, int NL>
__device__ __forceinline__ void wait_stage(int pending_after) {
  // pending_after = stages issued after the one we need (0 .. N)
  if constexpr (N >= 3) {
    if (pending_after >= 3) { wait_vmcnt<3 * NL>(); return; }
  }
  if constexpr (N >= 2) {
    if (pending_after >= 2) { wait_vmcnt<2 * NL>(); return; }
  }
  if (pending_after >= 1) { wait_vmcnt<NL>(); return; }
  wait_vmcnt<0>();
}

}  // namespace
}  // namespace ta
