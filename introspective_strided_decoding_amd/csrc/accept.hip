// p/q acceptance with residual resampling (isd_accept).
//
// Kernels, in stream order:
//   lse_partial    one read of every p and q row: per (row, vocab shard) the
//                  max and the sum of exp(l - max), fp32, 16-byte vector loads,
//                  wave reductions by lane exchange, then across the 4 waves.
//   accept_decide  one wave per request: combine the shard partials into the
//                  row log-normalisers, gather log p / log q at the proposals,
//                  rho = exp(log p - log q), Philox uniforms, accept iff
//                  u < rho, first rejection by a wave ballot.
//   resid_lse64    rejecting requests only: fp64 (max, sum exp) of the
//                  rejected p and q rows, sharded finely over the vocabulary.
//   resid_mass64   per shard: fp64 sum of r(y) = max(0, p(y) - q(y)) (and of
//                  p(y) for the zero-mass fallback).
//   resid_select   per rejecting request: prefix over shard masses picks the
//                  shard holding u' * S, a workgroup scan inside that shard in
//                  vocabulary order picks y*.
// The residual runs in fp64 so the inverse CDF agrees with a float64
// reference up to rounding of the running sums.
#include <climits>

#include "device_common.hpp"
#include "isd_internal.hpp"

namespace isd {
namespace {

constexpr int kThreads = 256;

template <typename T> struct Vec;
template <> struct Vec<uint16_t> { static constexpr int N = 8; };
template <> struct Vec<float> { static constexpr int N = 4; };

__device__ __forceinline__ void unpack(const u32x4& u, float* x, uint16_t) {
#pragma unroll
  for (int i = 0; i < 4; ++i) { x[2 * i] = bf16_lo(u[i]); x[2 * i + 1] = bf16_hi(u[i]); }
}
__device__ __forceinline__ void unpack(const u32x4& u, float* x, float) {
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(u[i]);
}

// (max, sum) pair merge in natural-log units
__device__ __forceinline__ void ms_merge(float& m, float& s, float m2, float s2) {
  if (m2 == -INFINITY) return;
  if (m == -INFINITY) { m = m2; s = s2; return; }
  if (m2 > m) { s = s * __expf(m - m2) + s2; m = m2; }
  else s += s2 * __expf(m2 - m);
}

template <typename T>
__global__ __launch_bounds__(kThreads) void lse_partial(const T* __restrict__ p_logits,
                                                        const T* __restrict__ q_logits, int rows_half,
                                                        int V, int shard_len, int shards,
                                                        float2* __restrict__ part) {
  constexpr int VN = Vec<T>::N;
  const int sh = blockIdx.x;
  const int row = blockIdx.y;
  const T* base = (row < rows_half) ? p_logits + size_t(row) * V : q_logits + size_t(row - rows_half) * V;
  const int e0 = sh * shard_len;
  const int e1 = min(V, e0 + shard_len);
  float m = -INFINITY, s = 0.f;
  if (e0 < e1) {
    // head up to 16-byte alignment of the absolute element index, vector body, scalar tail
    const size_t abs0 = size_t(row < rows_half ? row : row - rows_half) * V + e0;
    const int head = int((VN - (abs0 % VN)) % VN);
    const int hb = min(e1, e0 + head);
    const int nvec = (e1 - hb) / VN;
    const int tb = hb + nvec * VN;
    for (int e = e0 + threadIdx.x; e < hb; e += kThreads) ms_merge(m, s, to_f32<T>(base[e]), 1.f);
    for (int e = tb + threadIdx.x; e < e1; e += kThreads) ms_merge(m, s, to_f32<T>(base[e]), 1.f);
    const u32x4* vb = reinterpret_cast<const u32x4*>(base + hb);
    int v = threadIdx.x;
    // two vectors per step: one rescale per 2*VN elements
    for (; v + kThreads < nvec; v += 2 * kThreads) {
      const u32x4 a = vb[v], b = vb[v + kThreads];
      float x[2 * VN];
      unpack(a, x, T());
      unpack(b, x + VN, T());
      float mx = x[0];
#pragma unroll
      for (int i = 1; i < 2 * VN; ++i) mx = fmaxf(mx, x[i]);
      if (mx > m) { s *= exp2f((m - mx) * kLog2e); m = mx; }
      const float mb = m * kLog2e;
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < 2 * VN; ++i) acc += exp2f(fmaf(x[i], kLog2e, -mb));
      s += acc;
    }
    if (v < nvec) {
      const u32x4 a = vb[v];
      float x[VN];
      unpack(a, x, T());
      float mx = x[0];
#pragma unroll
      for (int i = 1; i < VN; ++i) mx = fmaxf(mx, x[i]);
      if (mx > m) { s *= exp2f((m - mx) * kLog2e); m = mx; }
      const float mb = m * kLog2e;
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < VN; ++i) acc += exp2f(fmaf(x[i], kLog2e, -mb));
      s += acc;
    }
  }
  // wave reduce of (m, s)
  const float wm = wave_max(m);
  float ws = (m == -INFINITY) ? 0.f : s * __expf(m - wm);
  ws = wave_sum(ws);
  __shared__ float sm[kThreads / 64][2];
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { sm[wave][0] = wm; sm[wave][1] = ws; }
  __syncthreads();
  if (threadIdx.x == 0) {
    float M = -INFINITY, S = 0.f;
    for (int w = 0; w < kThreads / 64; ++w) ms_merge(M, S, sm[w][0], sm[w][1]);
    part[size_t(row) * shards + sh] = make_float2(M, S);
  }
}

__device__ __forceinline__ float row_lse(const float2* part, int shards) {
  float M = -INFINITY, S = 0.f;
  for (int i = 0; i < shards; ++i) ms_merge(M, S, part[i].x, part[i].y);
  return M + __logf(S);
}

template <typename T>
__global__ __launch_bounds__(64) void accept_decide(
    const T* __restrict__ p_logits, const T* __restrict__ q_logits, const int32_t* __restrict__ proposals,
    const int32_t* __restrict__ req_ids, const int32_t* __restrict__ positions, uint64_t seed_lo,
    uint64_t seed_hi, uint32_t step, int N, int V, int shards, const float2* __restrict__ part,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ out_tokens, int32_t* __restrict__ n_out,
    int32_t* __restrict__ n_commit, float* __restrict__ logp_sel, float* __restrict__ logq_sel,
    ReqState* __restrict__ state, uint32_t* __restrict__ flags) {
  const int r = blockIdx.x;
  const int lane = threadIdx.x;
  const int R = N - 1;
  const int B = gridDim.x;
  bool reject = false;
  double u_res = 0.0;
  if (lane < R) {
    const int j = lane;
    const int rp = r * R + j;                  // p row index
    const int rq = B * R + r * R + j;          // q row index (after all p rows)
    const float lse_p = row_lse(part + size_t(rp) * shards, shards);
    const float lse_q = row_lse(part + size_t(rq) * shards, shards);
    const int x = proposals[size_t(r) * N + j + 1];
    float lp, lq;
    if (x < 0 || x >= V) {
      raise_flag(flags, ISD_FLAG_TOKEN_RANGE);
      lp = -INFINITY;
      lq = 0.f;
    } else {
      lp = to_f32<T>(p_logits[size_t(rp) * V + x]) - lse_p;
      lq = to_f32<T>(q_logits[size_t(r * R + j) * V + x]) - lse_q;
    }
    logp_sel[size_t(r) * R + j] = lp;
    logq_sel[size_t(r) * R + j] = lq;
    const float rho = __expf(lp - lq);
    const uint64_t rid = uint64_t(uint32_t(req_ids[r]));
    const uint64_t pos = uint64_t(uint32_t(positions[r])) + uint64_t(j + 1);
    const Philox4x64Out w = philox4x64_10(rid, pos, uint64_t(step), 0, seed_lo, seed_hi);
    const double u = unit_double(w.w[0]);
    u_res = unit_double(w.w[1]);
    reject = !(u < double(rho));
  }
  const uint64_t mask = __ballot(reject);
  const int first = mask ? (__ffsll((unsigned long long)mask) - 1) : -1;
  const int A = (first < 0) ? N : first + 1;
  const double u_first = __shfl(u_res, first < 0 ? 0 : first);
  if (lane < N) {
    const int x = proposals[size_t(r) * N + lane];
    out_tokens[size_t(r) * N + lane] = (lane < A) ? x : -1;
  }
  if (lane == 0) {
    accept_len[r] = A;
    n_out[r] = A + (A < N ? 1 : 0);
    n_commit[r] = min(A, N - 1);
    ReqState st;
    st.accept_len = A;
    st.reject_row = first;
    st.pad0 = st.pad1 = 0;
    st.u_resample = u_first;
    st.pad2 = 0.0;
    state[r] = st;
  }
}

// ---- fp64 residual ----
__device__ __forceinline__ void ms_merge_d(double& m, double& s, double m2, double s2) {
  if (m2 == -INFINITY) return;
  if (m == -INFINITY) { m = m2; s = s2; return; }
  if (m2 > m) { s = s * exp(m - m2) + s2; m = m2; }
  else s += s2 * exp(m2 - m);
}

template <int NT>
__device__ __forceinline__ void block_ms_reduce_d(double& m, double& s, double* sm) {
  const double wm = wave_max_d(m);
  double ws = (m == -INFINITY) ? 0.0 : s * exp(m - wm);
  ws = wave_sum_d(ws);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) { sm[2 * wave] = wm; sm[2 * wave + 1] = ws; }
  __syncthreads();
  double M = -INFINITY, S = 0.0;
  for (int w = 0; w < NT / 64; ++w) ms_merge_d(M, S, sm[2 * w], sm[2 * w + 1]);
  m = M;
  s = S;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void resid_lse64(const T* __restrict__ p_logits,
                                                         const T* __restrict__ q_logits, int N, int V,
                                                         int r_shard_len, int r_shards,
                                                         const ReqState* __restrict__ state,
                                                         double2* __restrict__ lse64) {
  const int sh = blockIdx.x;
  const int r = blockIdx.y;
  const int j = state[r].reject_row;
  if (j < 0) return;
  const size_t row = size_t(r) * (N - 1) + j;
  const T* pr = p_logits + row * V;
  const T* qr = q_logits + row * V;
  const int e0 = sh * r_shard_len, e1 = min(V, e0 + r_shard_len);
  double mp = -INFINITY, sp = 0.0, mq = -INFINITY, sq = 0.0;
  for (int e = e0 + threadIdx.x; e < e1; e += kThreads) {
    ms_merge_d(mp, sp, double(to_f32<T>(pr[e])), 1.0);
    ms_merge_d(mq, sq, double(to_f32<T>(qr[e])), 1.0);
  }
  __shared__ double sm[2 * kThreads / 64];
  block_ms_reduce_d<kThreads>(mp, sp, sm);
  block_ms_reduce_d<kThreads>(mq, sq, sm);
  if (threadIdx.x == 0) {
    lse64[(size_t(r) * r_shards + sh) * 2 + 0] = make_double2(mp, sp);
    lse64[(size_t(r) * r_shards + sh) * 2 + 1] = make_double2(mq, sq);
  }
}

__device__ __forceinline__ void combine_lse64(const double2* __restrict__ lse64, int r, int r_shards,
                                              double& lse_p, double& lse_q) {
  double mp = -INFINITY, sp = 0.0, mq = -INFINITY, sq = 0.0;
  for (int i = 0; i < r_shards; ++i) {
    const double2 a = lse64[(size_t(r) * r_shards + i) * 2 + 0];
    const double2 b = lse64[(size_t(r) * r_shards + i) * 2 + 1];
    ms_merge_d(mp, sp, a.x, a.y);
    ms_merge_d(mq, sq, b.x, b.y);
  }
  lse_p = mp + log(sp);
  lse_q = mq + log(sq);
}

template <typename T>
__global__ __launch_bounds__(kThreads) void resid_mass64(const T* __restrict__ p_logits,
                                                          const T* __restrict__ q_logits, int N, int V,
                                                          int r_shard_len, int r_shards,
                                                          const ReqState* __restrict__ state,
                                                          const double2* __restrict__ lse64,
                                                          double2* __restrict__ mass) {
  const int sh = blockIdx.x;
  const int r = blockIdx.y;
  const int j = state[r].reject_row;
  if (j < 0) return;
  __shared__ double lse_sm[2];
  if (threadIdx.x == 0) combine_lse64(lse64, r, r_shards, lse_sm[0], lse_sm[1]);
  __syncthreads();
  const double lse_p = lse_sm[0], lse_q = lse_sm[1];
  const size_t row = size_t(r) * (N - 1) + j;
  const T* pr = p_logits + row * V;
  const T* qr = q_logits + row * V;
  const int e0 = sh * r_shard_len, e1 = min(V, e0 + r_shard_len);
  double rs = 0.0, ps = 0.0;
  for (int e = e0 + threadIdx.x; e < e1; e += kThreads) {
    const double p = exp(double(to_f32<T>(pr[e])) - lse_p);
    const double q = exp(double(to_f32<T>(qr[e])) - lse_q);
    rs += fmax(0.0, p - q);
    ps += p;
  }
  rs = wave_sum_d(rs);
  ps = wave_sum_d(ps);
  __shared__ double sm[2][kThreads / 64];
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { sm[0][wave] = rs; sm[1][wave] = ps; }
  __syncthreads();
  if (threadIdx.x == 0) {
    double a = 0.0, b = 0.0;
    for (int w = 0; w < kThreads / 64; ++w) { a += sm[0][w]; b += sm[1][w]; }
    mass[size_t(r) * r_shards + sh] = make_double2(a, b);
  }
}

// inclusive scan of one double per thread across the workgroup
__device__ __forceinline__ double block_scan_d(double x, double* sm_w, double& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  __syncthreads();
  if (lane == 63) sm_w[wave] = x;
  __syncthreads();
  double before = 0.0;
  total = 0.0;
  for (int w = 0; w < kThreads / 64; ++w) {
    if (w < wave) before += sm_w[w];
    total += sm_w[w];
  }
  return before + x;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void resid_select(const T* __restrict__ p_logits,
                                                          const T* __restrict__ q_logits, int N, int V,
                                                          int r_shard_len, int r_shards,
                                                          const ReqState* __restrict__ state,
                                                          const double2* __restrict__ lse64,
                                                          const double2* __restrict__ mass,
                                                          int32_t* __restrict__ out_tokens) {
  const int r = blockIdx.x;
  const ReqState st = state[r];
  const int j = st.reject_row;
  if (j < 0) return;
  __shared__ double lse_sm[2];
  __shared__ double target_sm, before_sm;
  __shared__ int shard_sm, fallback_sm;
  if (threadIdx.x == 0) {
    combine_lse64(lse64, r, r_shards, lse_sm[0], lse_sm[1]);
    double S = 0.0;
    for (int i = 0; i < r_shards; ++i) S += mass[size_t(r) * r_shards + i].x;
    int fb = 0;
    if (!(S > 0.0)) {
      fb = 1;
      S = 0.0;
      for (int i = 0; i < r_shards; ++i) S += mass[size_t(r) * r_shards + i].y;
    }
    const double target = st.u_resample * S;
    double cum = 0.0;
    int pick = -1, last_nz = 0;
    double before_last = 0.0;
    for (int i = 0; i < r_shards; ++i) {
      const double mi = fb ? mass[size_t(r) * r_shards + i].y : mass[size_t(r) * r_shards + i].x;
      if (mi > 0.0) { last_nz = i; before_last = cum; }
      if (pick < 0 && cum + mi > target) { pick = i; before_sm = cum; }
      cum += mi;
    }
    if (pick < 0) { pick = last_nz; before_sm = before_last; }
    shard_sm = pick;
    target_sm = target;
    fallback_sm = fb;
  }
  __syncthreads();
  const double lse_p = lse_sm[0], lse_q = lse_sm[1];
  const double target = target_sm;
  const int fb = fallback_sm;
  const size_t row = size_t(r) * (N - 1) + j;
  const T* pr = p_logits + row * V;
  const T* qr = q_logits + row * V;
  const int e0 = shard_sm * r_shard_len, e1 = min(V, e0 + r_shard_len);
  __shared__ double sm_w[kThreads / 64];
  __shared__ int found_sm, last_pos_sm;
  if (threadIdx.x == 0) { found_sm = INT_MAX; last_pos_sm = -1; }
  __syncthreads();
  double before = before_sm;
  for (int c0 = e0; c0 < e1; c0 += kThreads) {
    const int e = c0 + threadIdx.x;
    double rv = 0.0;
    if (e < e1) {
      const double p = exp(double(to_f32<T>(pr[e])) - lse_p);
      if (fb) rv = p;
      else rv = fmax(0.0, p - exp(double(to_f32<T>(qr[e])) - lse_q));
    }
    double total;
    const double incl = block_scan_d(rv, sm_w, total);
    if (e < e1 && rv > 0.0) atomicMax(&last_pos_sm, e);
    if (e < e1 && before + incl > target) atomicMin(&found_sm, e);
    __syncthreads();
    if (found_sm != INT_MAX) break;
    before += total;
  }
  if (threadIdx.x == 0) {
    int y = found_sm;
    if (y == INT_MAX) y = (last_pos_sm >= 0) ? last_pos_sm : e1 - 1;
    out_tokens[size_t(r) * N + st.accept_len] = y;
  }
}

template <typename T>
hipError_t launch_t(const isd_shape& s, const AcceptPlan& p, const void* pl, const void* ql,
                    const int32_t* proposals, const int32_t* req_ids, const int32_t* positions,
                    uint64_t seed_lo, uint64_t seed_hi, uint32_t step, int32_t* accept_len,
                    int32_t* out_tokens, int32_t* n_out, int32_t* n_commit, float* logp_sel,
                    float* logq_sel, char* ws, const WsLayout& L, hipStream_t stream) {
  const T* P = static_cast<const T*>(pl);
  const T* Qp = static_cast<const T*>(ql);
  const int N = s.stride_n, V = s.vocab, B = s.batch;
  uint32_t* flags = reinterpret_cast<uint32_t*>(ws + L.flags);
  float2* part = reinterpret_cast<float2*>(ws + L.lse);
  ReqState* st = reinterpret_cast<ReqState*>(ws + L.req);
  double2* l64 = reinterpret_cast<double2*>(ws + L.lse64);
  double2* mass = reinterpret_cast<double2*>(ws + L.mass);
  hipLaunchKernelGGL((lse_partial<T>), dim3(p.shards, p.rows), dim3(kThreads), 0, stream, P, Qp,
                     B * (N - 1), V, p.shard_len, p.shards, part);
  hipLaunchKernelGGL((accept_decide<T>), dim3(B), dim3(64), 0, stream, P, Qp, proposals, req_ids,
                     positions, seed_lo, seed_hi, step, N, V, p.shards, part, accept_len, out_tokens,
                     n_out, n_commit, logp_sel, logq_sel, st, flags);
  hipLaunchKernelGGL((resid_lse64<T>), dim3(p.r_shards, B), dim3(kThreads), 0, stream, P, Qp, N, V,
                     p.r_shard_len, p.r_shards, st, l64);
  hipLaunchKernelGGL((resid_mass64<T>), dim3(p.r_shards, B), dim3(kThreads), 0, stream, P, Qp, N, V,
                     p.r_shard_len, p.r_shards, st, l64, mass);
  hipLaunchKernelGGL((resid_select<T>), dim3(B), dim3(kThreads), 0, stream, P, Qp, N, V,
                     p.r_shard_len, p.r_shards, st, l64, mass, out_tokens);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_accept(const isd_shape& s, const AcceptPlan& p, const void* p_logits,
                         const void* q_logits, const int32_t* proposals, const int32_t* req_ids,
                         const int32_t* positions, uint64_t seed_lo, uint64_t seed_hi, uint32_t step,
                         int32_t* accept_len, int32_t* out_tokens, int32_t* n_out, int32_t* n_commit,
                         float* logp_sel, float* logq_sel, char* ws, const WsLayout& L,
                         hipStream_t stream) {
  if (s.logit_dtype == ISD_BF16)
    return launch_t<uint16_t>(s, p, p_logits, q_logits, proposals, req_ids, positions, seed_lo, seed_hi,
                              step, accept_len, out_tokens, n_out, n_commit, logp_sel, logq_sel, ws, L,
                              stream);
  return launch_t<float>(s, p, p_logits, q_logits, proposals, req_ids, positions, seed_lo, seed_hi, step,
                         accept_len, out_tokens, n_out, n_commit, logp_sel, logq_sel, ws, L, stream);
}

}  // namespace isd
