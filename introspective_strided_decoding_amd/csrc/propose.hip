// Drawing the next N tokens at the MASK rows (isd_propose).
//
// Kernels, in stream order:
//   prop_partial  per (MASK row, 4096-entry vocabulary shard): the shard's
//                 fp32 max and the first index holding it, and (sampling
//                 policy) the float64 sum of exp(l - shard max).  Each thread
//                 owns 16 consecutive entries, read as 16-byte vectors when
//                 the row is aligned.
//   prop_select   one workgroup per MASK row.  Argmax policy: the largest
//                 shard max, ties to the smallest index.  Sampling policy:
//                 shard masses rescaled to the row max, a wave-wide prefix
//                 over them picks the shard holding u * total, and a
//                 workgroup scan inside that shard in vocabulary order picks
//                 the first token whose running mass exceeds u * total.
//                 With a row_norms buffer, the row's (max, sum of exp(l - max))
//                 is written too: the q-row normaliser of the forward that
//                 verifies these proposals.
// Sums and the scan run in float64 (exp by the table-driven exp_nonpos, its
// 64-entry table in LDS), so the draw agrees with a float64 inverse CDF up to
// rounding of the running sums.
#include <climits>

#include "device_common.hpp"
#include "exp64.hpp"
#include "isd_internal.hpp"

namespace isd {
namespace {

constexpr int kPThreads = 256;
constexpr int kPPer = 16;                     // entries per thread
constexpr int kPShard = kPThreads * kPPer;    // entries per shard

// 2^(j/64), j = 0..63, for exp_nonpos; call with all threads of the workgroup.
__device__ __forceinline__ void fill_exp_table(double* tab64) {
  if (threadIdx.x < 64) tab64[threadIdx.x] = exp2(double(threadIdx.x) * (1.0 / 64.0));
  __syncthreads();
}

template <typename T>
__device__ __forceinline__ void load_entries(const T* __restrict__ row, int e0, int e1, bool vec,
                                             float* x) {
  if (vec && e0 + kPPer <= e1) {
    constexpr int EV = 16 / sizeof(T);
#pragma unroll
    for (int v = 0; v < kPPer / EV; ++v) {
      const u32x4 u = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + e0) + v);
      T t[EV];
      __builtin_memcpy(t, &u, 16);
#pragma unroll
      for (int i = 0; i < EV; ++i) x[v * EV + i] = to_f32<T>(t[i]);
    }
  } else {
    // indices clamped into the row so that every load is unconditional and
    // all of them are in flight together
    T t[kPPer];
#pragma unroll
    for (int i = 0; i < kPPer; ++i) t[i] = row[min(e0 + i, e1 - 1)];
#pragma unroll
    for (int i = 0; i < kPPer; ++i) x[i] = (e0 + i < e1) ? to_f32<T>(t[i]) : -INFINITY;
  }
}

// Row-major MASK rows: row = r * N + k.  part[row * shards + sh].
template <typename T>
__global__ __launch_bounds__(kPThreads) void prop_partial(const T* __restrict__ logits, int V, int shards,
                                                          int sample, PropPart* __restrict__ part) {
  __shared__ double tab64[64];
  if (sample) fill_exp_table(tab64);
  const int sh = blockIdx.x;
  const size_t row = blockIdx.y;
  const T* base = logits + row * V;
  constexpr int EV = 16 / sizeof(T);
  const bool vec = ((row * V) % EV) == 0;
  const int e1 = min(V, (sh + 1) * kPShard);
  const int e0 = sh * kPShard + threadIdx.x * kPPer;
  float x[kPPer];
  load_entries<T>(base, e0, e1, vec, x);
  // this thread's max and the first entry holding it
  float mx = x[0];
  int ix = e0;
#pragma unroll
  for (int i = 1; i < kPPer; ++i)
    if (x[i] > mx) { mx = x[i]; ix = e0 + i; }
  if (mx == -INFINITY) ix = INT_MAX;
  // workgroup max, ties to the smallest index
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  wave_argmax(mx, ix);
  __shared__ float smx[kPThreads / 64];
  __shared__ int six[kPThreads / 64];
  __shared__ double ssum[kPThreads / 64];
  if (lane == 0) { smx[wave] = mx; six[wave] = ix; }
  __syncthreads();
  float M = smx[0];
  int I = six[0];
#pragma unroll
  for (int w = 1; w < kPThreads / 64; ++w)
    if (smx[w] > M || (smx[w] == M && six[w] < I)) { M = smx[w]; I = six[w]; }
  double s = 0.0;
  if (sample && M != -INFINITY) {
    const double md = M;
    double e[kPPer];
#pragma unroll
    for (int i = 0; i < kPPer; ++i) e[i] = exp_nonpos(double(x[i]) - md, tab64);
    // pairwise sum of the thread's 16 terms
#pragma unroll
    for (int w = kPPer / 2; w >= 1; w >>= 1)
#pragma unroll
      for (int i = 0; i < w; ++i) e[i] += e[i + w];
    s = wave_sum_d(e[0]);
    if (lane == 0) ssum[wave] = s;
    __syncthreads();
    s = 0.0;
#pragma unroll
    for (int w = 0; w < kPThreads / 64; ++w) s += ssum[w];
  }
  if (threadIdx.x == 0) {
    PropPart p;
    p.sum = s;
    p.max = M;
    p.idx = I;
    part[row * shards + sh] = p;
  }
}

template <typename T>
__global__ __launch_bounds__(kPThreads) void prop_select(const T* __restrict__ logits, int N, int V,
                                                         int shards, int sample,
                                                         const PropPart* __restrict__ part,
                                                         const int32_t* __restrict__ req_ids,
                                                         const int32_t* __restrict__ positions,
                                                         uint64_t seed_lo, uint64_t seed_hi, uint32_t step,
                                                         const int64_t* __restrict__ step_dev,
                                                         int32_t* __restrict__ out,
                                                         float2* __restrict__ row_norms) {
  const int row = blockIdx.x;
  const int r = row / N, k = row % N;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const PropPart* rp = part + size_t(row) * shards;
  __shared__ double tab64[64];
  __shared__ double before_sm, target_sm, scale_sm;
  __shared__ float mshard_sm;
  __shared__ int shard_sm;
  __shared__ int hit_sm[kPThreads / 64], last_sm[kPThreads / 64];
  __shared__ double wsum[kPThreads / 64];
  // lane l of wave 0 owns shards [l*per, (l+1)*per) in vocabulary order; the
  // first of them is requested before the table is built
  const int per = (shards + 63) / 64;
  const int s0 = min(shards, lane * per), s1 = min(shards, s0 + per);
  PropPart first_part;
  first_part.sum = 0.0;
  first_part.max = -INFINITY;
  first_part.idx = INT_MAX;
  if (wave == 0 && s0 < s1) first_part = rp[s0];
  // wave 0: this proposal's uniform, counter (request, position + N + k, step, 1),
  // word 0, drawn while the shard records are in flight (its inputs come by the
  // scalar path); wave 1 fills the exponential's table meanwhile
  double u = 0.0;
  if (wave == 0 && sample) {
    const uint32_t step32 = step_dev ? uint32_t(step_dev[r]) : step;
    const uint64_t pos = uint64_t(uint32_t(positions[r])) + uint64_t(N + k);
    u = unit_double(philox4x64_10(uint64_t(uint32_t(req_ids[r])), pos, uint64_t(step32), 1, seed_lo, seed_hi).w[0]);
  }
  if (sample) {
    if (wave == 1) tab64[lane] = exp2(double(lane) * (1.0 / 64.0));
    __syncthreads();
  }
  if (wave == 0) {
    float mx = -INFINITY;
    int ix = INT_MAX;
    for (int i = s0; i < s1; ++i) {
      const PropPart p = (i == s0) ? first_part : rp[i];
      if (p.max > mx || (p.max == mx && p.idx < ix)) { mx = p.max; ix = p.idx; }
    }
    float M = mx;
    int I = ix;
    wave_argmax(M, I);
    if (!sample) {
      if (lane == 0) out[row] = (I == INT_MAX) ? 0 : I;
    } else {
      // shard masses in units of exp(row max)
      const double Md = M;
      double wsh = 0.0;
      for (int i = s0; i < s1; ++i) {
        const PropPart p = (i == s0) ? first_part : rp[i];
        if (p.max != -INFINITY) wsh += p.sum * exp_nonpos(double(p.max) - Md, tab64);
      }
      double tot;
      const double before_lane = wave_exclusive_d(wsh, tot);
      // the row's normaliser, for the accept test of the forward that verifies these proposals
      if (row_norms && lane == 0) row_norms[row] = make_float2(M, float(tot));
      const double target = u * tot;
      double cum = before_lane;
      int pick = -1, last_nz = -1;
      double pick_before = 0.0, last_before = 0.0;
      float pick_max = -INFINITY, last_max = -INFINITY;
      for (int i = s0; i < s1; ++i) {
        const PropPart p = (i == s0) ? first_part : rp[i];
        const double wi = (p.max == -INFINITY) ? 0.0 : p.sum * exp_nonpos(double(p.max) - Md, tab64);
        if (wi > 0.0) { last_nz = i; last_before = cum; last_max = p.max; }
        if (pick < 0 && cum + wi > target) { pick = i; pick_before = cum; pick_max = p.max; }
        cum += wi;
      }
      const uint64_t hits = __ballot(pick >= 0);
      const uint64_t nz = __ballot(last_nz >= 0);
      int sh;
      double bf;
      float ms;
      if (hits) {
        const int src = __ffsll((unsigned long long)hits) - 1;
        sh = __shfl(pick, src);
        bf = __shfl(pick_before, src);
        ms = __shfl(pick_max, src);
      } else {
        // rounding left the target at or past the total: the last shard with mass
        const int src = nz ? 63 - __clzll((long long)nz) : 0;
        sh = __shfl(last_nz, src);
        bf = __shfl(last_before, src);
        ms = __shfl(last_max, src);
        if (sh < 0) {
          sh = 0;
          ms = -INFINITY;
        }
      }
      if (lane == 0) {
        shard_sm = sh;
        before_sm = bf;
        target_sm = target;
        mshard_sm = ms;
        scale_sm = (ms == -INFINITY) ? 0.0 : exp_nonpos(double(ms) - Md, tab64);
      }
    }
  }
  if (!sample) return;
  __syncthreads();
  // scan the chosen shard in vocabulary order
  const int sh = shard_sm;
  const T* base = logits + size_t(row) * V;
  constexpr int EV = 16 / sizeof(T);
  const bool vec = ((size_t(row) * V) % EV) == 0;
  const int e1 = min(V, (sh + 1) * kPShard);
  const int e0 = sh * kPShard + threadIdx.x * kPPer;
  float x[kPPer];
  load_entries<T>(base, e0, e1, vec, x);
  const double ms = mshard_sm, scale = scale_sm;
  double c[kPPer];
  double run = 0.0;
  int last_here = -1;
#pragma unroll
  for (int i = 0; i < kPPer; ++i) {
    const double v = exp_nonpos(double(x[i]) - ms, tab64) * scale;   // -inf entries give 0
    if (v > 0.0) last_here = e0 + i;
    run += v;
    c[i] = run;
  }
  double wtot;
  const double wbefore = wave_exclusive_d(run, wtot);
  if (lane == 0) wsum[wave] = wtot;
  __syncthreads();
  double before = before_sm + wbefore;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  const double target = target_sm;
  int hit = INT_MAX;
#pragma unroll
  for (int i = kPPer - 1; i >= 0; --i)
    if (e0 + i < e1 && before + c[i] > target) hit = e0 + i;
  int first_hit, last_nz;
  block_first_last(hit, last_here, hit_sm, last_sm, first_hit, last_nz);
  if (threadIdx.x == 0) {
    int y = first_hit;
    if (y == INT_MAX) y = (last_nz >= 0) ? last_nz : max(0, e1 - 1);
    out[row] = y;
  }
}

template <typename T>
hipError_t launch_t(const isd_shape& s, const void* logits, const int32_t* req_ids, const int32_t* positions,
                    uint64_t seed_lo, uint64_t seed_hi, uint32_t step, const int64_t* step_dev, int mode,
                    int32_t* out, float* row_norms, char* ws, const WsLayout& L, hipStream_t stream) {
  const T* lg = static_cast<const T*>(logits);
  const int N = s.stride_n, V = s.vocab, B = s.batch;
  const int shards = prop_shards(V);
  PropPart* part = reinterpret_cast<PropPart*>(ws + L.prop);
  const int sample = (mode == ISD_PROPOSE_SAMPLE) ? 1 : 0;
  hipLaunchKernelGGL((prop_partial<T>), dim3(shards, B * N), dim3(kPThreads), 0, stream, lg, V, shards,
                     sample, part);
  hipLaunchKernelGGL((prop_select<T>), dim3(B * N), dim3(kPThreads), 0, stream, lg, N, V, shards, sample,
                     part, req_ids, positions, seed_lo, seed_hi, step, step_dev, out,
                     reinterpret_cast<float2*>(row_norms));
  return hipGetLastError();
}

}  // namespace

int prop_shards(int vocab) { return (vocab + kPShard - 1) / kPShard; }

hipError_t launch_propose(const isd_shape& s, const void* mask_logits, const int32_t* req_ids,
                          const int32_t* positions, uint64_t seed_lo, uint64_t seed_hi, uint32_t step,
                          const int64_t* step_dev, int mode, int32_t* proposals, float* row_norms, char* ws,
                          const WsLayout& L, hipStream_t stream) {
  if (s.logit_dtype == ISD_BF16)
    return launch_t<uint16_t>(s, mask_logits, req_ids, positions, seed_lo, seed_hi, step, step_dev, mode,
                              proposals, row_norms, ws, L, stream);
  return launch_t<float>(s, mask_logits, req_ids, positions, seed_lo, seed_hi, step, step_dev, mode,
                         proposals, row_norms, ws, L, stream);
}

}  // namespace isd
