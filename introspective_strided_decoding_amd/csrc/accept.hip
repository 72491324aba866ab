// p/q acceptance with residual resampling (isd_accept).
//
// Kernels, in stream order:
//   lse_partial    one read of every p and q row: per (row, vocabulary shard)
//                  the max and the sum of exp(l - max), fp32, 16-byte
//                  streaming loads, wave reductions by lane exchange, then
//                  across the 4 waves; the workgroup whose shard holds the
//                  row's proposal also records the logit there, and the
//                  first workgroup of each request draws its Philox uniforms
//                  (a long dependent chain, hidden under that workgroup's loads).
//   accept_decide  (larger batches) one workgroup per request: its waves
//                  combine the shard partials of the request's rows into
//                  log-normalisers while the first wave loads the recorded
//                  logits at the proposals and the uniforms; rho = exp(log p -
//                  log q), accept iff u < rho, first rejection by a wave
//                  ballot; a rejecting request appends its job to a compact
//                  list.  (A last-arrival hand-off inside the normaliser
//                  launch measured slower: its 60-odd arrivals per request
//                  counter serialise.)
//   resid_pass     (larger batches) rejecting requests only, one pass over
//                  the rejected p and q rows, sharded finely over the
//                  vocabulary: fp64 sums of e_p = exp(l_p - max p) and e_q =
//                  exp(l_q - max q) (the row maxima come exact from the
//                  decision), and the residual's pieces under the decision's
//                  fp32 estimate of the normaliser ratio (see below).
//   decide_resid_pass
//                  (small batches, instead of the two above) grid (residual
//                  shards, requests): every workgroup makes its request's
//                  decision as accept_decide does (the request's first
//                  workgroup stores the results and the job at the request's
//                  slot) and, if the request rejected, serves its shard of
//                  the residual pass; one launch and one dependent read fewer.
//   resid_select   per rejecting request: exact shard masses from those
//                  pieces, a prefix over them picks the shard holding
//                  u' * S, a workgroup scan inside that shard in vocabulary
//                  order picks y*.  With a commit, one more workgroup per
//                  request writes its accepted rows to the KV pages beside the
//                  selections.
// The residual runs in fp64 so the inverse CDF agrees with a float64
// reference up to rounding of the running sums.
#include <climits>

#include "commit_row.hpp"
#include "device_common.hpp"
#include "exp64.hpp"
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

// Everything the accept decision reads and writes.
template <typename T>
struct DecideArgs {
  const T* p_logits;
  const T* q_logits;
  const int32_t* proposals;
  const int32_t* req_ids;
  const int32_t* positions;
  uint64_t seed_lo, seed_hi;
  uint32_t step;
  const int64_t* step_dev;   // per-request step counters in device memory (NULL: `step` for all)
  const float2* q_norms;     // (max, sum exp(l - max)) per MASK row as isd_propose wrote them (NULL: computed here)
  int N, V, shards;
  int32_t *accept_len, *out_tokens, *n_out, *n_commit;
  float *logp_sel, *logq_sel;
  ReqState* jobs;          // jobs: a compact list of rejecting requests (decision launch) or one per request
  uint32_t* rej_count;     // the compact list's length
  float* gath;             // per (request, p/q row): the row's logit at its proposal
  double* unif;            // per (request, stride row j < N-1): Philox uniforms u, u' (two doubles)
  uint32_t* flags;
};

// A shard holds at most kThreads * kLseVec vectors, so every thread issues all
// of its 16-byte loads before it waits on any of them.
constexpr int kLseVec = 8;

// The accept decision for request r, made by each workgroup of the residual
// launch that serves the request (what it reads, the shard partials, the
// logits at the proposals and the uniforms, is a few hundred bytes in L2).
// Every wave combines rows of shard partials into log-normalisers; lane
// j < N-1 of wave 0 tests x_{j+2} against p row j and q row j (their logits
// there were recorded by the normaliser kernel) and a ballot finds the first
// rejection.  With write_out the workgroup also stores the request's results
// and its job: appended to the compact list when it rejected (append), else
// at the request's own slot.  Every thread gets the job (req = -1: nothing
// rejected).
template <typename T>
__device__ __forceinline__ ReqState decide_request(const DecideArgs<T>& a, const float2* __restrict__ part, int r,
                                                   bool write_out, bool append) {
  const int N = a.N, V = a.V, R = N - 1, shards = a.shards;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __shared__ float lse_sm[64], max_sm[64];
  __shared__ ReqState job_sm;
  // every wave: the shard partials of rows wave, wave + 4, ... of the request's
  // 2(N-1) rows (p rows only when the q normalisers are carried); with one
  // shard per lane and at most 4 rows per wave (N <= 9) they are all requested
  // first, otherwise row by row
  const float2* req_part = part + size_t(r) * 2 * R * shards;
  const int n_rows = a.q_norms ? R : 2 * R;
  constexpr int kRowsPerWave = 4;
  const bool one_pass = shards <= 64 && n_rows <= kRowsPerWave * (kThreads / 64);
  float2 pre[kRowsPerWave];
  if (one_pass) {
#pragma unroll
    for (int k = 0; k < kRowsPerWave; ++k) {
      const int row = min(wave + k * (kThreads / 64), n_rows - 1);
      pre[k] = req_part[size_t(row) * shards + min(lane, shards - 1)];
    }
  }
  // wave 0: the proposals and the logits at them, requested before the combine
  int x = 0, xl = 0;
  float raw_p = 0.f, raw_q = 0.f;
  float2 qn = make_float2(0.f, 0.f);
  double u_acc = 0.0, u_res = 0.0;
  if (wave == 0) {
    // indices clamped into range so that every load is unconditional and in flight together
    const int j = min(lane, R - 1);
    xl = a.proposals[size_t(r) * N + min(lane, N - 1)];
    raw_p = a.gath[size_t(r) * 2 * R + j];
    if (a.q_norms) qn = a.q_norms[size_t(r) * N + j + 1];
    else raw_q = a.gath[size_t(r) * 2 * R + R + j];
    // lane j's uniforms, drawn by the normaliser kernel
    const double2 uu = reinterpret_cast<const double2*>(a.unif)[size_t(r) * R + j];
    u_acc = uu.x;
    u_res = uu.y;
    x = __shfl(xl, min(lane + 1, 63));     // lane j < R tests x_{j+2}, proposal j + 1
  }
  const bool in_range = x >= 0 && x < V;
  // carried q normalisers: the q rows' logits at the proposals are gathered here
  // (no normaliser pass over the q rows recorded them)
  if (a.q_norms && wave == 0 && lane < R && in_range)
    raw_q = to_f32<T>(a.q_logits[(size_t(r) * R + lane) * V + x]);
  if (a.q_norms && wave == 0 && lane < R) {
    lse_sm[R + lane] = qn.x + __logf(qn.y);
    max_sm[R + lane] = qn.x;
  }
  auto row_done = [&](int row, float rm, float rs) {
    const float M = wave_max(rm);
    const float S = wave_sum((rm == -INFINITY) ? 0.f : rs * __expf(rm - M));
    if (lane == 0) { lse_sm[row] = M + __logf(S); max_sm[row] = M; }
  };
  if (one_pass) {
#pragma unroll
    for (int k = 0; k < kRowsPerWave; ++k) {
      const int row = wave + k * (kThreads / 64);
      if (row < n_rows) row_done(row, lane < shards ? pre[k].x : -INFINITY, lane < shards ? pre[k].y : 0.f);
    }
  } else {
    for (int row = wave; row < n_rows; row += kThreads / 64) {
      float rm = -INFINITY, rs = 0.f;
      for (int i = lane; i < shards; i += 64) {
        const float2 v = req_part[size_t(row) * shards + i];
        ms_merge(rm, rs, v.x, v.y);
      }
      row_done(row, rm, rs);
    }
  }
  __syncthreads();
  if (wave == 0) {
    bool reject = false;
    if (lane < R) {
      const int j = lane;
      const size_t row = size_t(r) * R + j;
      float lp, lq;
      if (!in_range) {
        if (write_out) raise_flag(a.flags, ISD_FLAG_TOKEN_RANGE);
        lp = -INFINITY;
        lq = 0.f;
      } else {
        lp = raw_p - lse_sm[j];
        lq = raw_q - lse_sm[R + j];
      }
      if (write_out) {
        a.logp_sel[row] = lp;
        a.logq_sel[row] = lq;
      }
      const float rho = __expf(lp - lq);
      reject = !(u_acc < double(rho));
    }
    const uint64_t mask = __ballot(reject);
    const int first = mask ? (__ffsll((unsigned long long)mask) - 1) : -1;
    const int A = (first < 0) ? N : first + 1;
    const double u_first = __shfl(u_res, first < 0 ? 0 : first);
    if (write_out && lane < N) a.out_tokens[size_t(r) * N + lane] = (lane < A) ? xl : -1;
    if (lane == 0) {
      const int fr = first < 0 ? 0 : first;
      ReqState st;
      st.req = first < 0 ? -1 : r;
      st.accept_len = A;
      st.reject_row = fr;
      st.log_kappa = (lse_sm[fr] - max_sm[fr]) - (lse_sm[R + fr] - max_sm[R + fr]);
      st.max_p = max_sm[fr];
      st.max_q = max_sm[R + fr];
      st.u_resample = u_first;
      job_sm = st;
      if (write_out) {
        a.accept_len[r] = A;
        a.n_out[r] = A + (A < N ? 1 : 0);
        a.n_commit[r] = A;                  // rows 0..A-1 hold the accepted prefix
        if (!append)
          a.jobs[r] = st;
        else if (first >= 0)
          a.jobs[atomicAdd(a.rej_count, 1u)] = st;
      }
    }
  }
  __syncthreads();
  // wave-uniform copies (scalar registers), so the caller's branch on req and
  // the addresses it forms from the job stay scalar
  ReqState st;
  st.req = __builtin_amdgcn_readfirstlane(job_sm.req);
  st.accept_len = __builtin_amdgcn_readfirstlane(job_sm.accept_len);
  st.reject_row = __builtin_amdgcn_readfirstlane(job_sm.reject_row);
  st.log_kappa = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, job_sm.log_kappa)));
  st.max_p = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, job_sm.max_p)));
  st.max_q = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, job_sm.max_q)));
  const long long u = __builtin_bit_cast(long long, job_sm.u_resample);
  st.u_resample = __builtin_bit_cast(double, (long long)((unsigned long long)(unsigned)__builtin_amdgcn_readfirstlane(int(u)) |
                                                         ((unsigned long long)(unsigned)__builtin_amdgcn_readfirstlane(int(u >> 32)) << 32)));
  return st;
}

// Grid (n_rows * shards, B), n_rows = 2(N-1) (p rows, then q rows) or N-1
// (p rows only, when the q normalisers are carried): workgroup
// (jj * shards + sh, r) reduces shard sh of row jj of request r; its partial
// lands at part[(r * 2(N-1) + jj) * shards + sh].
template <typename T>
__global__ __launch_bounds__(kThreads) void lse_partial(DecideArgs<T> args, int shard_len, float2* __restrict__ part) {
  constexpr int VN = Vec<T>::N;
  const int V = args.V, shards = args.shards, R = args.N - 1;
  const int r = blockIdx.y;
  const int jj = blockIdx.x / shards, sh = blockIdx.x % shards;
  const bool is_q = jj >= R;
  const size_t row_off = (size_t(r) * R + (is_q ? jj - R : jj)) * V;
  const T* base = (is_q ? args.q_logits : args.p_logits) + row_off;
  const int e0 = sh * shard_len;
  const int e1 = min(V, e0 + shard_len);
  // the proposal this row tests (x_{j+2} for p row and q row j)
  const int xg = args.proposals[size_t(r) * args.N + (is_q ? jj - R : jj) + 1];
  float xv = 0.f;
  bool has_x = false;
  float m = -INFINITY, s = 0.f;
  if (e0 < e1) {
    // scalar head up to 16-byte alignment of the absolute element index, vector body, scalar tail
    const int head = int((VN - ((row_off + e0) % VN)) % VN);
    const int hb = min(e1, e0 + head);
    const int nvec = (e1 - hb) / VN;
    const int tb = hb + nvec * VN;
    const u32x4* vb = reinterpret_cast<const u32x4*>(base + hb);
    u32x4 raw[kLseVec];
    if (nvec > 0) {   // the same for the whole workgroup
      // every load unconditional (indices clamped into the shard) and issued
      // before any is used
#pragma unroll
      for (int k = 0; k < kLseVec; ++k)
        raw[k] = __builtin_nontemporal_load(vb + min(int(threadIdx.x) + k * kThreads, nvec - 1));
    }
    // block (0, r): request r's Philox uniforms (keyed by request, position
    // L + j + 1 and step) for its rows j < N-1, one lane each, drawn while the
    // logits are in flight so the decision does not wait for this long chain
    if (blockIdx.x == 0 && threadIdx.x < 64) {
      const int j = min(int(threadIdx.x), R - 1);
      const uint32_t step32 = args.step_dev ? uint32_t(args.step_dev[r]) : args.step;
      const uint64_t pos = uint64_t(uint32_t(args.positions[r])) + uint64_t(j + 1);
      const Philox4x64Out w =
          philox4x64_10(uint64_t(uint32_t(args.req_ids[r])), pos, uint64_t(step32), 0, args.seed_lo, args.seed_hi);
      if (int(threadIdx.x) < R)
        reinterpret_cast<double2*>(args.unif)[size_t(r) * R + j] = make_double2(unit_double(w.w[0]), unit_double(w.w[1]));
    }
    // pass 1: max over this thread's values (registers, then the scalar head
    // and tail: rows not 16-byte aligned, shard ends)
    float mx = -INFINITY;
    if (nvec > 0) {
#pragma unroll
      for (int k = 0; k < kLseVec; ++k) {
        if (threadIdx.x + k * kThreads < nvec) {
          float x[VN];
          unpack(raw[k], x, T());
#pragma unroll
          for (int i = 0; i < VN; ++i) mx = fmaxf(mx, x[i]);
        }
      }
    }
    bool has_tail = false;
    for (int e = e0 + threadIdx.x; e < hb; e += kThreads) {
      const float x = to_f32<T>(base[e]);
      mx = fmaxf(mx, x);
      has_tail = true;
      if (e == xg) { xv = x; has_x = true; }
    }
    for (int e = tb + threadIdx.x; e < e1; e += kThreads) {
      const float x = to_f32<T>(base[e]);
      mx = fmaxf(mx, x);
      has_tail = true;
      if (e == xg) { xv = x; has_x = true; }
    }
    // pass 2: sum of exp(x - mx) in base 2 by the hardware exp2 (a quarter of the
    // VALU rate; no range fix-up: a term below 2^-126 cannot change a sum that
    // holds the thread's max term, about 1)
    if (mx != -INFINITY) {
      const float mb = mx * kLog2e;
      float acc = 0.f;
      if (nvec > 0) {
#pragma unroll
        for (int k = 0; k < kLseVec; ++k) {
          if (threadIdx.x + k * kThreads < nvec) {
            float x[VN];
            unpack(raw[k], x, T());
#pragma unroll
            for (int i = 0; i < VN; ++i) acc += __builtin_amdgcn_exp2f(fmaf(x[i], kLog2e, -mb));
          }
        }
      }
      if (has_tail) {
        for (int e = e0 + threadIdx.x; e < hb; e += kThreads) acc += exp2f(fmaf(to_f32<T>(base[e]), kLog2e, -mb));
        for (int e = tb + threadIdx.x; e < e1; e += kThreads) acc += exp2f(fmaf(to_f32<T>(base[e]), kLog2e, -mb));
      }
      m = mx;
      s = acc;
    }
    // the logit at the proposal, from the registers of the thread that holds it
    if (nvec > 0 && xg >= hb && xg < tb && (xg - hb) / VN % kThreads == int(threadIdx.x)) {
      const int kx = (xg - hb) / VN / kThreads, ix = (xg - hb) % VN;
#pragma unroll
      for (int k = 0; k < kLseVec; ++k)
        if (k == kx) {
          float x[VN];
          unpack(raw[k], x, T());
#pragma unroll
          for (int i = 0; i < VN; ++i)
            if (i == ix) xv = x[i];
        }
      has_x = true;
    }
  }
  // wave reduce of (m, s)
  const float wm = wave_max(m);
  float ws = (m == -INFINITY) ? 0.f : s * exp2f((m - wm) * kLog2e);
  ws = wave_sum(ws);
  __shared__ float sm[kThreads / 64][2];
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { sm[wave][0] = wm; sm[wave][1] = ws; }
  __syncthreads();
  if (threadIdx.x == 0) {
    float M = -INFINITY, S = 0.f;
    for (int w = 0; w < kThreads / 64; ++w) ms_merge(M, S, sm[w][0], sm[w][1]);
    part[(size_t(r) * 2 * R + jj) * shards + sh] = make_float2(M, S);
    // a decision launch, next in the stream, lists rejecting requests from zero
    if (blockIdx.x == 0 && blockIdx.y == 0) *args.rej_count = 0u;
  }
  // and every list entry it does not fill reads as empty (req = -1), so the
  // residual kernels need only their own entry, not the count
  if (blockIdx.x == 0 && blockIdx.y == 0)
    for (int i = threadIdx.x; i < int(gridDim.y); i += kThreads) args.jobs[i].req = -1;
  if (has_x) args.gath[size_t(r) * 2 * R + jj] = xv;
}

// ---- fp64 residual ----
// Residual workgroup (shard, k) serves job k (the k-th listed rejecting
// request after a decision launch, request k when the decision runs inside
// the pass) and writes its record at k; the selection kernel requests its
// shard records together with the job.  A residual shard is 2048 vocabulary
// entries: 256 threads x 8 consecutive entries.
//
// Every value is e = exp(l - m) in float64 with m the row's exact max (carried
// in the job), by the table-driven exp_nonpos (its 64-entry table in
// LDS), so both kernels recompute exactly the same values.  With
// S_p = sum e_p, S_q = sum e_q and kappa = S_p / S_q, the residual is
// r(y) = max(0, e_p - kappa e_q) / S_p.  kappa is only known once every shard
// is summed, so the pass sorts each entry by the decision's fp32 estimate
// kappa~ (relative error far below the band kResidBand): entries clearly
// inside the support add e_p and e_q to (a, b); entries within the band are
// grouped by their exact logit difference l_p - l_q (equal differences mean
// equal ratios e_p / e_q, so a group lies wholly on one side of any kappa),
// and each group keeps its (sum e_p, sum e_q), for up to kResidAmb groups per
// shard.  The selection kernel then has the exact shard mass
// (a - kappa b + sum over groups of max(0, sum e_p - kappa sum e_q)) / S_p.
// If a shard had more groups, or kappa~ is off by more than half the band,
// the selection kernel recomputes the shard from the logits.
constexpr int kRPer = 8;
constexpr int kRShard = kThreads * kRPer;
constexpr double kResidBand = 1e-4;
constexpr int kAmbSlots = 64;   // boundary entries a pass workgroup lists (more: the shard is recomputed)
constexpr int kSerialAmb = 4;   // up to this many, one thread groups them
static_assert(kSerialAmb <= kResidAmb, "a serial grouping never overflows");

// 2^(j/64), j = 0..63, for exp_nonpos; call with all threads of the workgroup.
__device__ __forceinline__ void fill_exp_table(double* tab64) {
  if (threadIdx.x < 64) tab64[threadIdx.x] = exp2(double(threadIdx.x) * (1.0 / 64.0));
  __syncthreads();
}

// exp(x - m) for x <= m; x = -inf gives 0 without a test (exp_nonpos clamps the
// argument to -746, whose result underflows to 0), and so does an all -inf row (m = -inf:
// the NaN difference is clamped the same way)
__device__ __forceinline__ double exp_shift(float x, float m, const double* tab64) {
  return exp_nonpos(double(x) - double(m), tab64);
}

template <int W = kThreads / 64>
__device__ __forceinline__ double block_sum_d(double x, double* sm) {
  x = wave_sum_d(x);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sm[wave] = x;
  __syncthreads();
  double t = 0.0;
  for (int w = 0; w < W; ++w) t += sm[w];
  return t;
}

// Workgroup sums of K doubles per thread (W waves), with one pair of barriers for all K.
template <int K, int W = kThreads / 64>
__device__ __forceinline__ void block_sum_dk(double* x, double (*sm)[K]) {
#pragma unroll
  for (int i = 0; i < K; ++i) x[i] = wave_sum_d(x[i]);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0)
#pragma unroll
    for (int i = 0; i < K; ++i) sm[wave][i] = x[i];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < K; ++i) {
    double t = 0.0;
    for (int w = 0; w < W; ++w) t += sm[w][i];
    x[i] = t;
  }
}

// P consecutive logits of a p row and of a q row starting at e0 (entries
// >= e1 read as -inf), all loads in flight together.  Whole 16-byte aligned
// runs are vector loads; otherwise the indices are clamped into the shard so
// that every load is unconditional.
template <typename T, int P = kRPer>
__device__ __forceinline__ void load_runs(const T* __restrict__ prow, const T* __restrict__ qrow, int e0,
                                          int e1, float* xp, float* xq) {
  constexpr int VN = Vec<T>::N;
  if constexpr (P % VN == 0) {
    const bool vec = e0 + P <= e1 && ((reinterpret_cast<uintptr_t>(prow + e0) |
                                       reinterpret_cast<uintptr_t>(qrow + e0)) & 15) == 0;
    if (vec) {
      const u32x4* vp = reinterpret_cast<const u32x4*>(prow + e0);
      const u32x4* vq = reinterpret_cast<const u32x4*>(qrow + e0);
      u32x4 rp[P / VN], rq[P / VN];
#pragma unroll
      for (int k = 0; k < P / VN; ++k) {
        rp[k] = vp[k];
        rq[k] = vq[k];
      }
#pragma unroll
      for (int k = 0; k < P / VN; ++k) {
        unpack(rp[k], xp + k * VN, T());
        unpack(rq[k], xq + k * VN, T());
      }
      return;
    }
  }
  T rp[P], rq[P];
#pragma unroll
  for (int k = 0; k < P; ++k) {
    const int e = min(e0 + k, e1 - 1);
    rp[k] = prow[e];
    rq[k] = qrow[e];
  }
#pragma unroll
  for (int k = 0; k < P; ++k) {
    xp[k] = (e0 + k < e1) ? to_f32<T>(rp[k]) : -INFINITY;
    xq[k] = (e0 + k < e1) ? to_f32<T>(rq[k]) : -INFINITY;
  }
}

// Shard sh of job st's residual (k: where its records go); call with all threads.
template <typename T>
__device__ __forceinline__ void resid_shard(const T* __restrict__ p_logits, const T* __restrict__ q_logits, int N,
                                            int V, int r_shards, const ReqState& st, int k, int sh,
                                            ResidShard* __restrict__ shard_out) {
  __shared__ double tab64[64];
  __shared__ double sm4[kThreads / 64][4];
  // entries near the boundary, listed as they are found (rare): exact logit
  // difference, vocabulary index, e_p and e_q
  __shared__ double amb_key[kAmbSlots];
  __shared__ int amb_idx[kAmbSlots];
  __shared__ double amb_e[kAmbSlots][2];
  __shared__ int n_amb_sm;
  __shared__ double cls_key[kResidAmb];
  __shared__ double cls_sum[kResidAmb][2];
  __shared__ int n_cls_sm;
  __shared__ unsigned long long cls_bits[kResidAmb];
  __shared__ float shift_sm[2];
  __shared__ double sm2[kThreads / 64][2];
  const size_t row = size_t(st.req) * (N - 1) + st.reject_row;
  const int e1 = min(V, (sh + 1) * kRShard);
  const int e0 = sh * kRShard + threadIdx.x * kRPer;
  float xp[kRPer], xq[kRPer];
  load_runs<T>(p_logits + row * V, q_logits + row * V, e0, e1, xp, xq);
  if (threadIdx.x == 0) {
    n_amb_sm = 0;
    shift_sm[0] = st.max_p;
    shift_sm[1] = st.max_q;
  }
  fill_exp_table(tab64);
  const double kap = exp(double(st.log_kappa));
  double tot[4] = {0.0, 0.0, 0.0, 0.0};   // S_p, S_q, and (a, b) over the clear part of the support
  unsigned amb = 0;
#pragma unroll
  for (int i = 0; i < kRPer; ++i) {
    const double ep = exp_shift(xp[i], st.max_p, tab64);
    const double eq = exp_shift(xq[i], st.max_q, tab64);
    tot[0] += ep;
    tot[1] += eq;
    const double d = ep - kap * eq, band = kResidBand * kap * eq;
    if (d > band) {
      tot[2] += ep;
      tot[3] += eq;
    } else if (d >= -band && ep > 0.0) {
      amb |= 1u << i;
      const int slot = atomicAdd(&n_amb_sm, 1);
      if (slot < kAmbSlots) {
        amb_key[slot] = double(xp[i]) - double(xq[i]);
        amb_idx[slot] = e0 + i;
        amb_e[slot][0] = ep;
        amb_e[slot][1] = eq;
      }
    }
  }
  block_sum_dk<4>(tot, sm4);   // its barriers also publish the boundary list
  const double sp = tot[0], sq = tot[1], a = tot[2], b = tot[3];
  // Entries near the boundary, grouped by their exact logit difference (equal
  // differences: equal ratios e_p / e_q) and summed in vocabulary order, so the
  // sums do not depend on the order the entries were listed in.
  const int na = n_amb_sm;
  if (na > 0) {
    if (na <= kSerialAmb) {
      // a few entries (most shards that have any): one thread sorts them by
      // vocabulary index, groups them and orders the groups, without barriers
      if (threadIdx.x == 0) {
        for (int c = 1; c < na; ++c)
          for (int j = c; j > 0 && amb_idx[j] < amb_idx[j - 1]; --j) {
            const double tk = amb_key[j], t0 = amb_e[j][0], t1 = amb_e[j][1];
            const int ti = amb_idx[j];
            amb_key[j] = amb_key[j - 1];
            amb_idx[j] = amb_idx[j - 1];
            amb_e[j][0] = amb_e[j - 1][0];
            amb_e[j][1] = amb_e[j - 1][1];
            amb_key[j - 1] = tk;
            amb_idx[j - 1] = ti;
            amb_e[j - 1][0] = t0;
            amb_e[j - 1][1] = t1;
          }
        int n_cls = 0;
        for (int j = 0; j < na; ++j) {
          int c = 0;
          while (c < n_cls && cls_key[c] != amb_key[j]) ++c;
          if (c == n_cls) {
            cls_key[c] = amb_key[j];
            cls_sum[c][0] = 0.0;
            cls_sum[c][1] = 0.0;
            ++n_cls;
          }
          cls_sum[c][0] += amb_e[j][0];
          cls_sum[c][1] += amb_e[j][1];
        }
        for (int c = 1; c < n_cls; ++c)   // the groups in increasing order of their difference
          for (int j = c; j > 0 && cls_key[j] < cls_key[j - 1]; --j) {
            const double tk = cls_key[j], tp = cls_sum[j][0], tq = cls_sum[j][1];
            cls_key[j] = cls_key[j - 1];
            cls_sum[j][0] = cls_sum[j - 1][0];
            cls_sum[j][1] = cls_sum[j - 1][1];
            cls_key[j - 1] = tk;
            cls_sum[j - 1][0] = tp;
            cls_sum[j - 1][1] = tq;
          }
        n_cls_sm = n_cls;
      }
    } else if (na <= kAmbSlots) {
      // One thread per listed entry, each pass O(na): (1) move the entry to its
      // rank by vocabulary index (indices are distinct); (2) mark the first
      // entry of each difference; (3) a first entry's group number is the count
      // of groups with a smaller difference; (4) one thread per group sums its
      // members in vocabulary order.  The same sums, in the same order, as a
      // serial sort and scan.
      const int t = threadIdx.x;
      double key = 0.0, e0v = 0.0, e1v = 0.0;
      int rank = 0;
      if (t < na) {
        key = amb_key[t];
        e0v = amb_e[t][0];
        e1v = amb_e[t][1];
        const int idx = amb_idx[t];
        for (int i = 0; i < na; ++i) rank += amb_idx[i] < idx;
      }
      __syncthreads();
      if (t < na) {
        amb_key[rank] = key;
        amb_e[rank][0] = e0v;
        amb_e[rank][1] = e1v;
      }
      __syncthreads();
      bool first = false;
      if (t < na) {
        key = amb_key[t];
        first = true;
        for (int i = 0; i < t; ++i) first &= amb_key[i] != key;
        amb_idx[t] = first ? 1 : 0;            // the index list is free again: first-of-group marks
      }
      __syncthreads();
      if (t < na && first) {
        int c = 0;
        for (int i = 0; i < na; ++i) c += (amb_idx[i] != 0) && amb_key[i] < key;
        if (c < kResidAmb) cls_key[c] = key;
      }
      if (t == 0) {
        int n = 0;
        for (int i = 0; i < na; ++i) n += amb_idx[i];
        n_cls_sm = n <= kResidAmb ? n : kResidAmb + 1;
      }
      __syncthreads();
      const int n_cls = n_cls_sm;
      if (t < n_cls && n_cls <= kResidAmb) {
        const double ck = cls_key[t];
        double g0 = 0.0, g1 = 0.0;
        for (int i = 0; i < na; ++i)
          if (amb_key[i] == ck) {
            g0 += amb_e[i][0];
            g1 += amb_e[i][1];
          }
        cls_sum[t][0] = g0;
        cls_sum[t][1] = g1;
      }
    } else if (threadIdx.x == 0) {
      n_cls_sm = kResidAmb + 1;
    }
    __syncthreads();
    if (na > kAmbSlots) {
      // More boundary entries than the list holds (many equal logits on both
      // sides, say): the groups' keys are collected with compare-and-swap,
      // then one workgroup sum per group with each entry's exps recomputed.
      constexpr unsigned long long kEmpty = ~0ull;   // a NaN pattern, never a difference
      if (threadIdx.x < kResidAmb) cls_bits[threadIdx.x] = kEmpty;
      __syncthreads();
      bool over = false;
#pragma unroll
      for (int i = 0; i < kRPer; ++i)
        if (amb & (1u << i)) {
          const unsigned long long key = __double_as_longlong(double(xp[i]) - double(xq[i]));
          bool placed = false;
          for (int c = 0; c < kResidAmb && !placed; ++c) {
            const unsigned long long old = atomicCAS(&cls_bits[c], kEmpty, key);
            placed = (old == kEmpty || old == key);
          }
          over |= !placed;
        }
      const bool any_over = __syncthreads_or(over);
      if (threadIdx.x == 0 && !any_over) {   // groups in increasing order of their difference
        for (int c = 1; c < kResidAmb && cls_bits[c] != kEmpty; ++c)
          for (int j = c; j > 0 && __longlong_as_double(cls_bits[j]) < __longlong_as_double(cls_bits[j - 1]); --j) {
            const unsigned long long t = cls_bits[j];
            cls_bits[j] = cls_bits[j - 1];
            cls_bits[j - 1] = t;
          }
      }
      __syncthreads();
      int nc = any_over ? kResidAmb + 1 : 0;
      for (int c = 0; c < kResidAmb && !any_over; ++c) {
        const unsigned long long key = cls_bits[c];
        if (key == kEmpty) break;
        const float mp = shift_sm[0], mq = shift_sm[1];
        double g[2] = {0.0, 0.0};
#pragma unroll
        for (int i = 0; i < kRPer; ++i)
          if ((amb & (1u << i)) && __double_as_longlong(double(xp[i]) - double(xq[i])) == (long long)key) {
            g[0] += exp_shift(xp[i], mp, tab64);
            g[1] += exp_shift(xq[i], mq, tab64);
          }
        block_sum_dk<2>(g, sm2);
        if (threadIdx.x == 0) {
          cls_sum[c][0] = g[0];
          cls_sum[c][1] = g[1];
        }
        nc = c + 1;
      }
      if (threadIdx.x == 0) n_cls_sm = nc;
      __syncthreads();
    }
  }
  const int n_cls = (na > 0) ? n_cls_sm : 0;
  if (threadIdx.x == 0) {
    ResidShard rs;
    rs.sp = sp;
    rs.sq = sq;
    rs.a = a;
    rs.b = b;
    rs.n_amb = n_cls;
    rs.pad = 0;
    for (int j = 0; j < kResidAmb; ++j) {
      rs.amb[j][0] = (j < n_cls && n_cls <= kResidAmb) ? cls_sum[j][0] : 0.0;
      rs.amb[j][1] = (j < n_cls && n_cls <= kResidAmb) ? cls_sum[j][1] : 0.0;
    }
    shard_out[size_t(k) * r_shards + sh] = rs;
  }
}

// The decision launch: one workgroup per request; a rejecting request appends
// its job to the compact list.
template <typename T>
__global__ __launch_bounds__(kThreads) void accept_decide(DecideArgs<T> a, const float2* __restrict__ part) {
  decide_request(a, part, blockIdx.x, true, true);
}

// Grid (residual shards, list length B) after a decision launch: workgroup
// (sh, k) serves the k-th listed rejecting request, so the workgroups with
// work are the first ones dispatched; the rest return after reading their
// empty entry.
template <typename T>
__global__ __launch_bounds__(kThreads) void resid_pass(const T* __restrict__ p_logits, const T* __restrict__ q_logits,
                                                        int N, int V, int r_shards, const ReqState* __restrict__ jobs,
                                                        ResidShard* __restrict__ shard_out) {
  const ReqState st = jobs[blockIdx.y];
  // all of the entry is requested at once, not the gating field first and the
  // rest after the test (the empty asm keeps the compiler from sinking them)
  asm volatile("" ::"s"(st.req), "s"(st.reject_row), "s"(st.log_kappa), "s"(st.max_p), "s"(st.max_q),
               "s"(p_logits), "s"(q_logits));
  if (st.req < 0) return;                        // past the listed rejecting requests
  resid_shard<T>(p_logits, q_logits, N, V, r_shards, st, blockIdx.y, blockIdx.x, shard_out);
}

// Grid (residual shards, requests) with the decision inside: every workgroup
// makes its request's decision (the request's first workgroup stores the
// results and the job at the request's slot), then serves shard sh of the
// residual if the request rejected.  Chosen for small batches, whose grid
// leaves room for the repeated decisions (see plan_accept).
template <typename T>
__global__ __launch_bounds__(kThreads) void decide_resid_pass(DecideArgs<T> args, const float2* __restrict__ part,
                                                               int r_shards, ResidShard* __restrict__ shard_out) {
  const int sh = blockIdx.x, r = blockIdx.y;
  const ReqState st = decide_request(args, part, r, sh == 0, false);
  if (st.req < 0) return;                        // nothing rejected: no residual
  resid_shard<T>(args.p_logits, args.q_logits, args.N, args.V, r_shards, st, r, sh, shard_out);
}

// r(y) = max(0, p(y) - q(y)) and p(y) for P consecutive entries
template <int P>
__device__ __forceinline__ void resid_values(const float* xp, const float* xq, const ReqState& st, double ip,
                                             double iq, const double* tab64, double* rv, double* pv) {
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const double p = exp_shift(xp[i], st.max_p, tab64) * ip;
    rv[i] = fmax(0.0, p - exp_shift(xq[i], st.max_q, tab64) * iq);
    pv[i] = p;
  }
}

// One workgroup of kSelThreads per job (entry k of the compact list, or
// request k; an empty job, req = -1, returns at once): exact shard masses, then
// the inverse-CDF draw.  Wave 0 alone reads the shard records (lane l owns
// the shards [l*per, (l+1)*per), in vocabulary order), sums S_p and S_q by
// lane exchange, turns each record into the shard's exact masses and picks
// the shard holding u' * S by a wave-wide prefix, while wave 1 fills the
// exponential's table; after one barrier every thread scans that shard in
// vocabulary order (kSelPer entries per thread: the few selection workgroups
// have the chip to themselves, so the scan's float64 exponentials are spread
// over 16 waves) and the first crossing is y*.
constexpr int kSelThreads = 1024;
constexpr int kSelPer = kRShard / kSelThreads;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSelRecs = 2;   // records per lane read in one round trip (per <= 2: V <= 262144)
static_assert(kMaxResidShards <= kSelThreads, "one shard record per thread");

// The head of a shard record: its sums and its first kHeadAmb boundary groups
// (seven 16-byte vectors; the other groups are read only when a record has them).
constexpr int kHeadAmb = 4;
struct RecHead {
  double sp, sq, a, b;
  int32_t n_amb, pad;
  double amb[kHeadAmb][2];
};
static_assert(sizeof(ResidShard) % 16 == 0 && (sizeof(RecHead) + 15) / 16 * 16 <= sizeof(ResidShard) &&
                  offsetof(ResidShard, amb) == offsetof(RecHead, amb),
              "record heads are read as 16-byte vectors inside the record");

__device__ __forceinline__ RecHead load_head(const ResidShard* rec) {
  constexpr int NV = (int(sizeof(RecHead)) + 15) / 16;
  const u32x4* src = reinterpret_cast<const u32x4*>(rec);
  u32x4 v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) v[i] = src[i];
  RecHead h;
  __builtin_memcpy(&h, v, sizeof(RecHead));
  return h;
}

template <typename T>
__global__ __launch_bounds__(kSelThreads) void resid_select(const T* __restrict__ p_logits,
                                                          const T* __restrict__ q_logits, int N, int V,
                                                          int r_shards, const ReqState* __restrict__ jobs,
                                                          const ResidShard* __restrict__ shards_in,
                                                          int32_t* __restrict__ out_tokens, int B, CommitArgs cm) {
  __shared__ double tab64[64];
  __shared__ double rmass[kMaxResidShards], pmass[kMaxResidShards];
  __shared__ int redo[kMaxResidShards];
  __shared__ int n_redo_sm;
  __shared__ double red[kSelWaves];
  __shared__ double before_sm, target_sm, ip_sm, iq_sm;
  __shared__ int shard_sm, fb_sm;
  __shared__ int hit_sm[kSelWaves], last_sm[kSelWaves];
  __shared__ double wsum[kSelWaves];
  // workgroups past the first B (isd_accept_commit only): commit request
  // blockIdx.x - B's accepted rows while the selections run
  if (int(blockIdx.x) >= B) {
    if (cm.kv_bf16)
      commit_request<uint16_t, kSelThreads>(cm, blockIdx.x - B);
    else
      commit_request<float, kSelThreads>(cm, blockIdx.x - B);
    return;
  }
  const int k = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const ResidShard* recs = shards_in + size_t(k) * r_shards;
  const int per = (r_shards + 63) / 64;
  const int s0 = min(r_shards, lane * per), s1 = min(r_shards, s0 + per);
  // wave 0: the heads of its lanes' records requested together with the job
  RecHead rec[kSelRecs];
  if (wave == 0 && per <= kSelRecs) {
#pragma unroll
    for (int j = 0; j < kSelRecs; ++j) rec[j] = load_head(recs + min(s0 + j, r_shards - 1));
  }
  const ReqState st = jobs[k];
  // all of the job at once (the empty asm keeps the compiler from requesting the
  // gating field first and the rest after the test)
  asm volatile("" ::"s"(st.req), "s"(st.reject_row), "s"(st.log_kappa), "s"(st.max_p), "s"(st.max_q),
               "s"(st.accept_len), "s"(st.u_resample));
  if (st.req < 0) return;                        // the request rejected nothing
  const int r = st.req;
  const size_t row = size_t(r) * (N - 1) + st.reject_row;
  // wave 0: the inverse CDF over the shard masses held in rmass / pmass (this
  // lane's shards written by this lane, or by every thread after a recompute)
  auto pick_shard = [&](double rsum, double psum, double* rm, double* pm) {
    double rtot, ptot;
    const double rbefore = wave_exclusive_d(rsum, rtot);
    const double pbefore = wave_exclusive_d(psum, ptot);
    const bool fb = !(rtot > 0.0);                 // p and q equal up to rounding: sample p
    const double S = fb ? ptot : rtot;
    const double target = st.u_resample * S;
    double cum = fb ? pbefore : rbefore;
    int pick = -1, last_nz = -1;
    double pick_before = 0.0, last_before = 0.0;
    for (int i = s0; i < s1; ++i) {
      const double mi = fb ? pm[i] : rm[i];
      if (mi > 0.0) { last_nz = i; last_before = cum; }
      if (pick < 0 && cum + mi > target) { pick = i; pick_before = cum; }
      cum += mi;
    }
    // first lane (lowest shards) that holds the crossing
    const uint64_t hits = __ballot(pick >= 0);
    const uint64_t nz = __ballot(last_nz >= 0);
    if (hits) {
      const int src = __ffsll((unsigned long long)hits) - 1;
      const int sh = __shfl(pick, src);
      const double bf = __shfl(pick_before, src);
      if (lane == 0) { shard_sm = sh; before_sm = bf; }
    } else {
      // rounding left the target at or past the total: take the last shard with mass
      const int src = nz ? 63 - __clzll((long long)nz) : 0;
      const int sh = __shfl(last_nz, src);
      const double bf = __shfl(last_before, src);
      if (lane == 0) { shard_sm = sh < 0 ? 0 : sh; before_sm = bf; }
    }
    if (lane == 0) { target_sm = target; fb_sm = fb; }
  };
  if (wave == 0) {
    // exact row sums and kappa
    double psp = 0.0, psq = 0.0;
    if (per <= kSelRecs) {
#pragma unroll
      for (int j = 0; j < kSelRecs; ++j)
        if (s0 + j < s1) {
          psp += rec[j].sp;
          psq += rec[j].sq;
        }
    } else {
      for (int i = s0; i < s1; ++i) {
        psp += recs[i].sp;
        psq += recs[i].sq;
      }
    }
    const double sp = wave_sum_d(psp), sq = wave_sum_d(psq);
    const double kap = sp / sq;
    const bool estimate_ok = fabs(exp(double(st.log_kappa)) / kap - 1.0) < 0.5 * kResidBand;
    const double ip = 1.0 / sp, iq = 1.0 / sq;
    // exact shard masses from the records; shards that cannot be completed are listed
    bool needs_redo = false;
    auto shard_mass = [&](const RecHead& rs, int i, double& rsum, double& psum) {
      const double pm = rs.sp * ip;
      pmass[i] = pm;
      psum += pm;
      if (estimate_ok && rs.n_amb <= kResidAmb) {
        double m = rs.a - kap * rs.b;
#pragma unroll
        for (int j = 0; j < kHeadAmb; ++j)
          if (j < rs.n_amb) m += fmax(0.0, rs.amb[j][0] - kap * rs.amb[j][1]);
        for (int j = kHeadAmb; j < rs.n_amb; ++j)   // groups past the head (rare)
          m += fmax(0.0, recs[i].amb[j][0] - kap * recs[i].amb[j][1]);
        const double rm = fmax(0.0, m) * ip;
        rmass[i] = rm;
        rsum += rm;
      } else {
        needs_redo = true;
      }
    };
    double rsum = 0.0, psum = 0.0;
    if (per <= kSelRecs) {
#pragma unroll
      for (int j = 0; j < kSelRecs; ++j)
        if (s0 + j < s1) shard_mass(rec[j], s0 + j, rsum, psum);
    } else {
      for (int i = s0; i < s1; ++i) shard_mass(load_head(recs + i), i, rsum, psum);
    }
    const uint64_t any_redo = __ballot(needs_redo);
    if (any_redo) {
      // rare: mark the shards to recompute (each lane its own)
      for (int i = s0; i < s1; ++i) {
        const ResidShard* rs = recs + i;
        redo[i] = !(estimate_ok && rs->n_amb <= kResidAmb);
      }
    } else {
      pick_shard(rsum, psum, rmass, pmass);
    }
    if (lane == 0) {
      ip_sm = ip;
      iq_sm = iq;
      n_redo_sm = any_redo ? 1 : 0;
    }
  } else if (wave == 1) {
    tab64[lane] = exp2(double(lane) * (1.0 / 64.0));
  }
  __syncthreads();
  const double ip = ip_sm, iq = iq_sm;
  if (n_redo_sm != 0) {
    // rare: recompute the marked shards' residual masses from the logits, then pick again
    for (int i = 0; i < r_shards; ++i) {
      if (!redo[i]) continue;
      const int e1 = min(V, (i + 1) * kRShard);
      const int e0 = i * kRShard + threadIdx.x * kSelPer;
      float xp[kSelPer], xq[kSelPer];
      load_runs<T, kSelPer>(p_logits + row * V, q_logits + row * V, e0, e1, xp, xq);
      double rv[kSelPer], pv[kSelPer];
      resid_values<kSelPer>(xp, xq, st, ip, iq, tab64, rv, pv);
      double m = 0.0;
#pragma unroll
      for (int j = 0; j < kSelPer; ++j) m += rv[j];
      m = block_sum_d<kSelWaves>(m, red);
      if (threadIdx.x == 0) rmass[i] = m;
      __syncthreads();
    }
    if (wave == 0) {
      double rsum = 0.0, psum = 0.0;
      for (int i = s0; i < s1; ++i) {
        rsum += rmass[i];
        psum += pmass[i];
      }
      pick_shard(rsum, psum, rmass, pmass);
    }
    __syncthreads();
  }
  const int sh = shard_sm;
  const double target = target_sm;
  const int e1 = min(V, (sh + 1) * kRShard);
  const int e0 = sh * kRShard + threadIdx.x * kSelPer;
  float xp[kSelPer], xq[kSelPer];
  load_runs<T, kSelPer>(p_logits + row * V, q_logits + row * V, e0, e1, xp, xq);
  double rv[kSelPer], pv[kSelPer], c[kSelPer];
  resid_values<kSelPer>(xp, xq, st, ip, iq, tab64, rv, pv);
  double run = 0.0;
  int last_here = -1;
#pragma unroll
  for (int i = 0; i < kSelPer; ++i) {
    const double v = fb_sm ? pv[i] : rv[i];
    if (v > 0.0 && e0 + i < e1) last_here = e0 + i;
    run += v;
    c[i] = run;
  }
  // exclusive scan of thread totals (threads in vocabulary order); a wave adds
  // the totals of the waves before it with one lane each
  double wtot;
  const double wbefore = wave_exclusive_d(run, wtot);
  if (lane == 0) wsum[wave] = wtot;
  __syncthreads();
  const double before = before_sm + wbefore + wave_sum_d(lane < wave ? wsum[lane] : 0.0);
  int hit = INT_MAX;
#pragma unroll
  for (int i = kSelPer - 1; i >= 0; --i)
    if (e0 + i < e1 && before + c[i] > target) hit = e0 + i;
  int first_hit, last_nz;
  block_first_last(hit, last_here, hit_sm, last_sm, first_hit, last_nz);
  if (threadIdx.x == 0) {
    int y = first_hit;
    if (y == INT_MAX) y = (last_nz >= 0) ? last_nz : e1 - 1;
    out_tokens[size_t(r) * N + st.accept_len] = y;
  }
}

template <typename T>
hipError_t launch_t(const isd_shape& s, const AcceptPlan& p, const void* pl, const void* ql,
                    const int32_t* proposals, const int32_t* req_ids, const int32_t* positions,
                    uint64_t seed_lo, uint64_t seed_hi, uint32_t step, const int64_t* step_dev,
                    const float* q_norms, int32_t* accept_len, int32_t* out_tokens, int32_t* n_out, int32_t* n_commit,
                    float* logp_sel, float* logq_sel, char* ws, const WsLayout& L, uint32_t* flags,
                    const CommitArgs* commit, hipStream_t stream) {
  const T* P = static_cast<const T*>(pl);
  const T* Qp = static_cast<const T*>(ql);
  const int N = s.stride_n, V = s.vocab, B = s.batch;
  float2* part = reinterpret_cast<float2*>(ws + L.lse);
  ReqState* jobs = reinterpret_cast<ReqState*>(ws + L.jobs);
  ResidShard* rshards = reinterpret_cast<ResidShard*>(ws + L.resid);
  uint32_t* rej_count = reinterpret_cast<uint32_t*>(ws + kRejCountOffset);
  DecideArgs<T> a;
  a.p_logits = P;
  a.q_logits = Qp;
  a.proposals = proposals;
  a.req_ids = req_ids;
  a.positions = positions;
  a.seed_lo = seed_lo;
  a.seed_hi = seed_hi;
  a.step = step;
  a.step_dev = step_dev;
  a.q_norms = reinterpret_cast<const float2*>(q_norms);
  a.N = N;
  a.V = V;
  a.shards = p.shards;
  a.accept_len = accept_len;
  a.out_tokens = out_tokens;
  a.n_out = n_out;
  a.n_commit = n_commit;
  a.logp_sel = logp_sel;
  a.logq_sel = logq_sel;
  a.jobs = jobs;
  a.rej_count = rej_count;
  a.gath = reinterpret_cast<float*>(ws + L.gath);
  a.unif = reinterpret_cast<double*>(ws + L.unif);
  a.flags = flags;
  hipLaunchKernelGGL((lse_partial<T>), dim3((q_norms ? 1 : 2) * (N - 1) * p.shards, B), dim3(kThreads), 0, stream,
                     a, p.shard_len, part);
  if (p.fuse_decision) {
    hipLaunchKernelGGL((decide_resid_pass<T>), dim3(p.r_shards, B), dim3(kThreads), 0, stream, a, part, p.r_shards,
                       rshards);
  } else {
    hipLaunchKernelGGL((accept_decide<T>), dim3(B), dim3(kThreads), 0, stream, a, part);
    hipLaunchKernelGGL((resid_pass<T>), dim3(p.r_shards, B), dim3(kThreads), 0, stream, P, Qp, N, V, p.r_shards,
                       jobs, rshards);
  }
  // with a commit, B more workgroups in the selection launch: one per request
  CommitArgs cm{};
  if (commit) cm = *commit;
  hipLaunchKernelGGL((resid_select<T>), dim3(commit ? 2 * B : B), dim3(kSelThreads), 0, stream, P, Qp, N, V,
                     p.r_shards, jobs, rshards, out_tokens, B, cm);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_accept(const isd_shape& s, const AcceptPlan& p, const void* p_logits,
                         const void* q_logits, const int32_t* proposals, const int32_t* req_ids,
                         const int32_t* positions, uint64_t seed_lo, uint64_t seed_hi, uint32_t step,
                         const int64_t* step_dev, const float* q_norms, int32_t* accept_len, int32_t* out_tokens,
                         int32_t* n_out, int32_t* n_commit, float* logp_sel, float* logq_sel, char* ws,
                         const WsLayout& L, uint32_t* flags, const CommitArgs* commit, hipStream_t stream) {
  if (s.logit_dtype == ISD_BF16)
    return launch_t<uint16_t>(s, p, p_logits, q_logits, proposals, req_ids, positions, seed_lo, seed_hi,
                              step, step_dev, q_norms, accept_len, out_tokens, n_out, n_commit, logp_sel, logq_sel,
                              ws, L, flags, commit, stream);
  return launch_t<float>(s, p, p_logits, q_logits, proposals, req_ids, positions, seed_lo, seed_hi, step,
                         step_dev, q_norms, accept_len, out_tokens, n_out, n_commit, logp_sel, logq_sel, ws, L, flags,
                         commit, stream);
}

}  // namespace isd
