// Device helpers shared by the MUSTAFAR kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mustafar {

constexpr int kHeadDim = 128;
constexpr int kWave = 64;
constexpr int kTile = 64;  // rows per tile: one row per lane

// Raw buffer resource word 3 for the gfx9 family (untyped 32-bit dwords).
constexpr int kBufferWord3 = 0x00020000;

typedef __attribute__((address_space(4))) const uint64_t* ConstU64;
typedef __attribute__((address_space(4))) const uint32_t* ConstU32;

__device__ __forceinline__ uint32_t lane_id() {
  return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

// Bounds-checked buffer view: loads past `bytes` return 0 instead of faulting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kBufferWord3);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}
__device__ __forceinline__ void buf_store16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, uint4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) uint32_t, v), r,
                                         byte_off, 0, 0);
}
__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0);
}

// Number of set bits of `mask` below this lane, plus `add`.
__device__ __forceinline__ uint32_t mbcnt64(uint64_t mask, uint32_t add) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, add));
}

// v if this lane's bit of the (wave-uniform) lane mask is set, else 0: one v_cndmask
// with the mask in an SGPR pair.
__device__ __forceinline__ uint32_t keep_if_lane_bit(uint64_t lane_mask, uint32_t v) {
  uint32_t r;
  asm("v_cndmask_b32 %0, 0, %1, %2" : "=v"(r) : "v"(v), "s"(lane_mask));
  return r;
}

// 2^x with the hardware instruction alone (v_exp_f32): no rescaling of
// arguments below -126, whose results only matter as (near-)zero
// probabilities; exp2(-inf) = 0.
__device__ __forceinline__ float exp2_raw(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float half_bits_to_float(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}
__device__ __forceinline__ uint16_t float_to_half_bits(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);  // round to nearest even
}

// Lanes of one wave exchanging data through LDS: the hardware performs one
// wave's LDS operations in issue order, so only the compiler must be kept from
// moving or forwarding memory accesses across the exchange point.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  asm volatile("" ::: "memory");
}

template <class T>
__device__ __forceinline__ T wave_uniform(T x) {
  return __builtin_amdgcn_readfirstlane(x);
}

// Split kernels run two blocks per compute unit, so each SIMD holds one wave of
// each.  The SIMD's issue arbiter prefers the older wave, so the block
// dispatched first finishes its tiles well before the other, which then runs
// its last tiles alone at one wave per SIMD (a sixth of the kernel at the
// Llama-3 layer shape).  A wave's priority therefore falls as its share of
// tiles runs out: 3 while more than half is left, then 2, 1 and 0 below a
// half, a quarter and an eighth.  A wave that has fallen behind then wins
// the arbitration, and the two finish together.  `left` and `share` are
// uniform across the wave.
__device__ __forceinline__ void set_priority_by_tiles_left(int left, int share) {
  if (2 * left > share)
    __builtin_amdgcn_s_setprio(3);
  else if (4 * left > share)
    __builtin_amdgcn_s_setprio(2);
  else if (8 * left > share)
    __builtin_amdgcn_s_setprio(1);
  else
    __builtin_amdgcn_s_setprio(0);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, v),
                                                               __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, false));
}

// Wave-wide max on the vector units: DPP exchanges inside each 16-lane row
// (quad_perm [1,0,3,2], [2,3,0,1], row_ror 4, row_ror 8) leave every lane with
// its row's max; the four row maxima are then read with v_readlane.
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f32<0xB1>(x));
  x = fmaxf(x, dpp_f32<0x4E>(x));
  x = fmaxf(x, dpp_f32<0x124>(x));
  x = fmaxf(x, dpp_f32<0x128>(x));
  const int xi = __builtin_bit_cast(int, x);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}
// Butterflies over lanes l and l ^ 32 (l ^ 16) with the gfx950 lane-swap
// instructions, which run on the vector units (a __shfl_xor is an LDS
// permute with an LDS round trip).  Swapping a register with itself leaves
// x[l] in one result and x[l ^ 32] (x[l ^ 16]) in the other (checked on the
// device), so an order-free combine of the two is the butterfly step.
// The empty asm statement hides the two results from the code generator: it
// otherwise treats a swap of two copies of one value as leaving both equal
// and drops the combine (seen in the generated code after DPP row rotations).
template <bool SWAP32>
__device__ __forceinline__ void lane_swap_pair(float x, float& a, float& b) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  unsigned r0, r1;
  if constexpr (SWAP32) {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    r0 = r[0];
    r1 = r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    r0 = r[0];
    r1 = r[1];
  }
  asm volatile("" : "+v"(r0), "+v"(r1));
  a = __builtin_bit_cast(float, r0);
  b = __builtin_bit_cast(float, r1);
}
__device__ __forceinline__ float max_xor32(float x) {
  float a, b;
  lane_swap_pair<true>(x, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float max_xor16(float x) {
  float a, b;
  lane_swap_pair<false>(x, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float sum_xor32(float x) {
  float a, b;
  lane_swap_pair<true>(x, a, b);
  return a + b;
}
__device__ __forceinline__ float sum_xor16(float x) {
  float a, b;
  lane_swap_pair<false>(x, a, b);
  return a + b;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, kWave);
  return x;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = max(x, (uint32_t)__shfl_xor((int)x, o, kWave));
  return x;
}
// Exclusive prefix sum over the wave's lanes.
__device__ __forceinline__ uint32_t wave_excl_scan(uint32_t x) {
  const uint32_t lane = lane_id();
  uint32_t incl = x;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    uint32_t y = (uint32_t)__shfl_up((int)incl, o, kWave);
    if (lane >= (uint32_t)o) incl += y;
  }
  return incl - x;
}

}  // namespace mustafar
