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

// Lane exchange by DPP (a VALU operand modifier of the gfx9 encoding: no LDS
// crossbar trip).  Lanes whose row is masked off, or whose source lane lies
// outside its row, read 0.
namespace dpp {
constexpr int kQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kShr1 = 0x111, kShr2 = 0x112, kShr4 = 0x114, kShr8 = 0x118;   // row_shr:n
constexpr int kMirror = 0x140;      // row_mirror: lane i of a 16-lane row reads lane 15 - i
constexpr int kHalfMirror = 0x141;  // row_half_mirror: within 8 lanes, 7 - i
constexpr int kBcast15 = 0x142;     // row_bcast:15: lane 15 of each row into the next row
constexpr int kBcast31 = 0x143;     // row_bcast:31: lane 31 into rows 2 and 3
}  // namespace dpp

template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return uint32_t(__builtin_amdgcn_update_dpp(0, int(x), CTRL, ROWS, 0xF, true));
}
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ float dpp_f(float x) {
  return __uint_as_float(dpp_u32<CTRL, ROWS>(__float_as_uint(x)));
}
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ double dpp_d(double x) {
  const uint64_t u = __double_as_longlong(x);
  const uint64_t lo = dpp_u32<CTRL, ROWS>(uint32_t(u)), hi = dpp_u32<CTRL, ROWS>(uint32_t(u >> 32));
  return __longlong_as_double((long long)(lo | (hi << 32)));
}
__device__ __forceinline__ float readlane_f(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}
__device__ __forceinline__ double readlane_d(double x, int lane) {
  const uint64_t u = __double_as_longlong(x);
  const uint64_t lo = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(u)), lane));
  const uint64_t hi = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(u >> 32)), lane));
  return __longlong_as_double((long long)(lo | (hi << 32)));
}

// Wave-wide reduction with an associative, commutative `op` (all 64 lanes
// receive the result): sums within each 16-lane row by quad and mirror
// exchanges, rows combined into lane 63 by the two row broadcasts, then
// read from lane 63 (rows a broadcast skips keep their value).
template <typename T, typename Op>
__device__ __forceinline__ T wave_reduce(T x, Op op) {
  if constexpr (sizeof(T) == 8) {
    x = op(x, dpp_d<dpp::kQuadXor1>(x));
    x = op(x, dpp_d<dpp::kQuadXor2>(x));
    x = op(x, dpp_d<dpp::kHalfMirror>(x));
    x = op(x, dpp_d<dpp::kMirror>(x));
    const T r1 = dpp_d<dpp::kBcast15, 0xA>(x);
    x = ((threadIdx.x & 16) ? op(x, r1) : x);
    const T r2 = dpp_d<dpp::kBcast31, 0xC>(x);
    x = ((threadIdx.x & 32) ? op(x, r2) : x);
    return readlane_d(x, kWave - 1);
  } else {
    x = op(x, dpp_f<dpp::kQuadXor1>(x));
    x = op(x, dpp_f<dpp::kQuadXor2>(x));
    x = op(x, dpp_f<dpp::kHalfMirror>(x));
    x = op(x, dpp_f<dpp::kMirror>(x));
    const T r1 = dpp_f<dpp::kBcast15, 0xA>(x);
    x = ((threadIdx.x & 16) ? op(x, r1) : x);
    const T r2 = dpp_f<dpp::kBcast31, 0xC>(x);
    x = ((threadIdx.x & 32) ? op(x, r2) : x);
    return readlane_f(x, kWave - 1);
  }
}
__device__ __forceinline__ float wave_max(float x) {
  return wave_reduce(x, [](float a, float b) { return fmaxf(a, b); });
}
__device__ __forceinline__ float wave_sum(float x) {
  return wave_reduce(x, [](float a, float b) { return a + b; });
}
__device__ __forceinline__ double wave_max_d(double x) {
  return wave_reduce(x, [](double a, double b) { return fmax(a, b); });
}
__device__ __forceinline__ double wave_sum_d(double x) {
  return wave_reduce(x, [](double a, double b) { return a + b; });
}

// (max, first index) over the wave: the larger value wins, ties go to the
// smaller index (INT_MAX marks "no entry").  Same exchange pattern.
__device__ __forceinline__ void wave_argmax(float& m, int& i) {
  auto take = [&](float om, int oi) {
    if (om > m || (om == m && oi < i)) { m = om; i = oi; }
  };
  take(dpp_f<dpp::kQuadXor1>(m), int(dpp_u32<dpp::kQuadXor1>(uint32_t(i))));
  take(dpp_f<dpp::kQuadXor2>(m), int(dpp_u32<dpp::kQuadXor2>(uint32_t(i))));
  take(dpp_f<dpp::kHalfMirror>(m), int(dpp_u32<dpp::kHalfMirror>(uint32_t(i))));
  take(dpp_f<dpp::kMirror>(m), int(dpp_u32<dpp::kMirror>(uint32_t(i))));
  {
    const float om = dpp_f<dpp::kBcast15, 0xA>(m);
    const int oi = int(dpp_u32<dpp::kBcast15, 0xA>(uint32_t(i)));
    if (threadIdx.x & 16) take(om, oi);
  }
  {
    const float om = dpp_f<dpp::kBcast31, 0xC>(m);
    const int oi = int(dpp_u32<dpp::kBcast31, 0xC>(uint32_t(i)));
    if (threadIdx.x & 32) take(om, oi);
  }
  m = readlane_f(m, kWave - 1);
  i = __builtin_amdgcn_readlane(i, kWave - 1);
}

// Wave-wide inclusive prefix sum in lane order: a Hillis-Steele scan inside
// each 16-lane row by row shifts, then the row totals carried forward by the
// two row broadcasts.  Returns x's exclusive prefix; `total` = the sum.
__device__ __forceinline__ double wave_exclusive_d(double x, double& total) {
  double incl = x;
  incl += dpp_d<dpp::kShr1>(incl);
  incl += dpp_d<dpp::kShr2>(incl);
  incl += dpp_d<dpp::kShr4>(incl);
  incl += dpp_d<dpp::kShr8>(incl);
  incl += dpp_d<dpp::kBcast15, 0xA>(incl);
  incl += dpp_d<dpp::kBcast31, 0xC>(incl);
  total = readlane_d(incl, kWave - 1);
  return incl - x;
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
// 16-byte forms of the same accesses, through a buffer resource over a region
// of `bytes` bytes at `base` (16-byte aligned, bytes < 2^31): buffer loads and
// stores with the sc1 cache policy, the encoding the agent-scope relaxed
// atomics above take on this architecture.  Offsets are in bytes; an offset
// past the region reads 0 and writes nothing.
constexpr int kCachePolicySc1 = 16;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
__device__ __forceinline__ f32x4 ld_coherent16(__amdgpu_buffer_rsrc_t r, int offset) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, offset, 0, kCachePolicySc1));
}
__device__ __forceinline__ void st_coherent16(__amdgpu_buffer_rsrc_t r, int offset, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, offset, 0, kCachePolicySc1);
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
