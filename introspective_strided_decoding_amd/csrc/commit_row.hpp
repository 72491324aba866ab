// Appending accepted stride rows to the KV pages: the device code shared by
// the kv_commit kernel and the accept launch that also commits.
//
// One workgroup of kCommitThreads threads per (request r, stride row i),
// i = 0..N-1.  A request commits n rows starting at stride row f: row f + t
// goes to position L + t (L = its length before the commit).  Normally f = 0
// and n = n_commit[r] (the accepted prefix x_1..x_A); a request of the
// decoding loop in re-proposing mode commits row N-1 only (f = N-1, n = 1),
// which carries the token its previous forward resampled.  The workgroup
// requests its row's key and value vectors before the request's length and
// page id arrive, stores them if its row is committed and the pages of the
// positions L..L+t are all mapped (16-byte stores into the key layout,
// element stores into the transposed value layout), and counts its arrival;
// the request's last arrival writes the new length, so ctx_lens_out may
// alias ctx_lens_in.
#pragma once

#include "device_common.hpp"
#include "isd_internal.hpp"

namespace isd {

__device__ __forceinline__ int v_sigma(int s) { return (s & 3) | ((s & 4) << 1) | ((s & 8) >> 1); }

constexpr int kCommitThreads = 256;
constexpr int kCommitPre = 2;   // 16-byte vectors per thread requested up front

// Page id of committed row t of request r (position L + t); -1 when the
// position is past the table, -2 when the table entry is not a pool page.
__device__ __forceinline__ int commit_page(const int32_t* __restrict__ table, int r, int L, int t,
                                           int max_pages, int num_pages) {
  const int pos = L + t;
  if (pos >= max_pages * kPage) return -1;
  const int pid = table[size_t(r) * max_pages + pos / kPage];
  return (pid < 0 || pid >= num_pages) ? -2 : pid;
}

template <typename T>
__device__ __forceinline__ void commit_store(int w, int rvec, int D, int Hkv, int pid, int slot,
                                             const u32x4& v, T* __restrict__ kp, T* __restrict__ vp) {
  constexpr int EV = 16 / sizeof(T);
  if (w < rvec) {
    const int e0 = w * EV, hk = e0 / D, d0 = e0 % D;
    T* dst = kp + ((size_t(pid) * Hkv + hk) * (D / 8) + d0 / 8) * (kPage * 8) + slot * 8 + (d0 & 7);
    *reinterpret_cast<u32x4*>(dst) = v;
  } else {
    const int e0 = (w - rvec) * EV, hk = e0 / D, d0 = e0 % D;
    T* dst = vp + ((size_t(pid) * Hkv + hk) * D + d0) * kPage + v_sigma(slot);
    T x[EV];
    __builtin_memcpy(x, &v, 16);
#pragma unroll
    for (int e = 0; e < EV; ++e) dst[e * kPage] = x[e];
  }
}

// Commit row i of request r; call with all kCommitThreads threads.
template <typename T>
__device__ __forceinline__ void commit_row(const CommitArgs& c, int i, int r, int* s_last) {
  constexpr int EV = 16 / sizeof(T);
  const int N = c.N, Hkv = c.Hkv, D = c.D, max_pages = c.max_pages, num_pages = c.num_pages;
  const int Qn = 2 * N - 1;
  const int rvec = Hkv * D / EV;                 // 16-byte vectors per key (or value) row
  const size_t row_off = (size_t(r) * Qn + i) * Hkv * D;
  const u32x4* ksrc = reinterpret_cast<const u32x4*>(static_cast<const T*>(c.k_new) + row_off);
  const u32x4* vsrc = reinterpret_cast<const u32x4*>(static_cast<const T*>(c.v_new) + row_off);
  T* kp = static_cast<T*>(c.k_pages);
  T* vp = static_cast<T*>(c.v_pages);
  u32x4 pre[kCommitPre];
#pragma unroll
  for (int m = 0; m < kCommitPre; ++m) {
    const int w = threadIdx.x + m * kCommitThreads;
    if (w < 2 * rvec) pre[m] = (w < rvec) ? ksrc[w] : vsrc[w - rvec];
  }
  const int cap = max_pages * kPage;
  int L = c.ctx_in[r], n = c.n_commit[r], f = 0;
  const bool bad_n = n < 0 || n > N, bad_L = L < 0 || L > cap;
  if (bad_n) n = n < 0 ? 0 : N;
  if (c.loop_mode && c.loop_mode[r] == ISD_LOOP_REPROPOSE) {   // the resampled token's row
    n = 1;
    f = N - 1;
  }
  if (bad_L) { L = L < 0 ? 0 : cap; n = 0; }
  // positions L..L+t must all be mapped for row f + t to be stored
  const int t = i - f;
  bool store = t >= 0 && t < n;
  if (store) {
    const int lane = threadIdx.x & 63;
    const int pid_t = (lane <= t) ? commit_page(c.table, r, L, lane, max_pages, num_pages) : 0;
    const uint64_t bad = __ballot(pid_t < 0);
    store = (bad == 0);
  }
  if (store) {
    const int pid = commit_page(c.table, r, L, t, max_pages, num_pages);
    const int slot = (L + t) % kPage;
#pragma unroll
    for (int m = 0; m < kCommitPre; ++m) {
      const int w = threadIdx.x + m * kCommitThreads;
      if (w < 2 * rvec) commit_store<T>(w, rvec, D, Hkv, pid, slot, pre[m], kp, vp);
    }
    for (int w = threadIdx.x + kCommitPre * kCommitThreads; w < 2 * rvec; w += kCommitThreads)
      commit_store<T>(w, rvec, D, Hkv, pid, slot, (w < rvec) ? ksrc[w] : vsrc[w - rvec], kp, vp);
  }
  if (!arrive_last(&c.arrivals[r], uint32_t(N), s_last)) return;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int pid_t = (lane < n) ? commit_page(c.table, r, L, lane, max_pages, num_pages) : 0;
    const uint64_t bad = __ballot(pid_t < 0);
    const int nv = bad ? (__ffsll((unsigned long long)bad) - 1) : n;
    const int first_bad = __shfl(pid_t, bad ? nv : 0);
    if (lane == 0) {
      if (bad_n) raise_flag(c.flags, ISD_FLAG_COMMIT_RANGE);
      if (bad_L) raise_flag(c.flags, ISD_FLAG_CTX_RANGE);
      if (bad) raise_flag(c.flags, first_bad == -1 ? ISD_FLAG_COMMIT_RANGE : ISD_FLAG_PAGE_RANGE);
      c.ctx_out[r] = L + nv;
    }
  }
}

}  // namespace isd
