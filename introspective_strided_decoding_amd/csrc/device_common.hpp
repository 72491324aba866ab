// Device helpers shared by the ISD kernels (gfx950, wave64).
#pragma once

#include <climits>

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace isd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bf16 <-> fp32 on raw bits: a bf16 is the top half of an fp32.
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// Round-to-nearest-even fp32 -> bf16 bits (inputs here are finite).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return uint16_t((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<uint16_t>(uint16_t v) { return bf16_bits_to_f32(v); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ uint16_t from_f32<uint16_t>(float v) { return f32_to_bf16_bits(v); }

// Wave-wide reductions (all 64 lanes receive the result).
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) x += __shfl_xor(x, m);
  return x;
}
__device__ __forceinline__ double wave_max_d(double x) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) x = fmax(x, __shfl_xor(x, m));
  return x;
}
__device__ __forceinline__ double wave_sum_d(double x) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) x += __shfl_xor(x, m);
  return x;
}

// Cross-workgroup hand-off without cache flushes.  Data one workgroup
// publishes for another in the same kernel is written and read with
// device-scope relaxed atomic accesses (coherent across the XCDs' L2 caches
// on their own); the writer waits for its stores to complete before it
// counts its arrival, and only the last arrival reads the data.
template <typename T>
__device__ __forceinline__ void st_coherent(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T ld_coherent(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until this wave's stores have completed (s_waitcnt vmcnt(0)).
__device__ __forceinline__ void wait_stores_done() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// Count this workgroup's arrival; true in the last of `expected` arrivals,
// which also rewinds the counter for the next launch.  Call with all threads.
__device__ __forceinline__ bool arrive_last(uint32_t* counter, uint32_t expected, int* s_flag) {
  wait_stores_done();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = (prev == expected - 1);
    if (last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_flag = last ? 1 : 0;
  }
  __syncthreads();
  return *s_flag != 0;
}

// Smallest `hit` (INT_MAX: none) and largest `last` (-1: none) over the
// workgroup: a ballot per wave, one LDS slot per wave (arrays of at least
// blockDim.x / 64 entries), a barrier, and every thread reads the slots.
// (Divergent LDS atomics would be turned into a loop over the active lanes.)
__device__ __forceinline__ void block_first_last(int hit, int last, int* sm_hit, int* sm_last, int& out_hit,
                                                 int& out_last) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const uint64_t hb = __ballot(hit != INT_MAX);
  const uint64_t lb = __ballot(last >= 0);
  const int wh = __shfl(hit, hb ? __ffsll((unsigned long long)hb) - 1 : 0);
  const int wl = __shfl(last, lb ? 63 - __clzll((long long)lb) : 0);
  if (lane == 0) {
    sm_hit[wave] = hb ? wh : INT_MAX;
    sm_last[wave] = lb ? wl : -1;
  }
  __syncthreads();
  out_hit = INT_MAX;
  out_last = -1;
  for (int w = 0; w < int(blockDim.x) / kWave; ++w) {
    out_hit = min(out_hit, sm_hit[w]);
    out_last = max(out_last, sm_last[w]);
  }
}

// Device flag word (workspace offset 0).
__device__ __forceinline__ void raise_flag(uint32_t* flags, uint32_t bit) {
  if (flags) atomicOr(flags, bit);
}

// ---------------------------------------------------------------------------
// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11): four 64-bit counter words,
// two 64-bit key words; a round multiplies words 0 and 2 by the two round
// multipliers into 128-bit products and mixes their halves with words 1, 3
// and the key; the key advances by two Weyl increments between rounds.
struct Philox4x64Out { uint64_t w[4]; };

__device__ __forceinline__ Philox4x64Out philox4x64_10(uint64_t c0, uint64_t c1, uint64_t c2,
                                                       uint64_t c3, uint64_t k0, uint64_t k1) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += W0; k1 += W1; }
    const uint64_t hi0 = __umul64hi(M0, c0), lo0 = M0 * c0;
    const uint64_t hi1 = __umul64hi(M1, c2), lo1 = M1 * c2;
    const uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
  }
  Philox4x64Out o;
  o.w[0] = c0; o.w[1] = c1; o.w[2] = c2; o.w[3] = c3;
  return o;
}

// 53 top bits -> double in [0, 1).
__device__ __forceinline__ double unit_double(uint64_t w) {
  return double(w >> 11) * (1.0 / 9007199254740992.0);
}

}  // namespace isd
