// Appending accepted stride rows to the KV pages: the device code shared by
// the kv_commit kernel and the accept launch that also commits.
//
// One workgroup of kCommitThreads threads per request r.  The request commits
// n rows starting at stride row f: row f + t goes to position L + t (L = its
// length before the commit).  Normally f = 0 and n = n_commit[r] (the accepted
// prefix x_1..x_A); a request of the decoding loop in re-proposing mode
// commits row N-1 only (f = N-1, n = 1), which carries the token its previous
// forward resampled.  The rows are written only as far as the pages of their
// positions are mapped, and the new length is L plus the rows written, so
// ctx_lens_out may alias ctx_lens_in.
//
// The work is split into cells of (KV head, 8 head dims).  A key cell writes
// its n slot vectors (8 dims each, consecutive slots: contiguous in the key
// layout).  A value cell rewrites, for each of its 8 dims, the dim's whole
// 16-slot row of every page the committed positions touch: it reads the row,
// puts the new values at their (swizzled) slots and writes the row back with
// full 16-byte stores, so no store writes a partial 32-byte sector (a row
// holds one token per slot, 2 bytes each in bf16, and a commit adds only a
// few tokens to it).  One workgroup per request owns every row it rewrites.
#pragma once

#include "device_common.hpp"
#include "isd_internal.hpp"

namespace isd {

__device__ __forceinline__ int v_sigma(int s) { return (s & 3) | ((s & 4) << 1) | ((s & 8) >> 1); }

constexpr int kCommitThreads = 256;
constexpr int kMaxCommitRows = 16;    // N <= 16

// Page id of committed row t of request r (position L + t); -1 when the
// position is past the table, -2 when the table entry is not a pool page.
__device__ __forceinline__ int commit_page(const int32_t* __restrict__ table, int r, int L, int t,
                                           int max_pages, int num_pages) {
  const int pos = L + t;
  if (pos >= max_pages * kPage) return -1;
  const int pid = table[size_t(r) * max_pages + pos / kPage];
  return (pid < 0 || pid >= num_pages) ? -2 : pid;
}

// Element k (0..15) of a value-page row held as 16-byte vectors.
template <typename T, int RV>
__device__ __forceinline__ void row_put(u32x4 (&row)[RV], int k, T v) {
  constexpr int EW = 4 / int(sizeof(T));       // elements per 32-bit word
#pragma unroll
  for (int q = 0; q < RV * 4; ++q) {
    if (q == k / EW) {
      uint32_t bits;
      if constexpr (sizeof(T) == 2) {
        const uint32_t x = uint32_t(v);
        bits = (k & 1) ? ((row[q / 4][q % 4] & 0x0000ffffu) | (x << 16)) : ((row[q / 4][q % 4] & 0xffff0000u) | x);
      } else {
        bits = __float_as_uint(v);
      }
      row[q / 4][q % 4] = bits;
    }
  }
}

// Commit request r's rows; call with all kCommitThreads threads.
template <typename T>
__device__ __forceinline__ void commit_request(const CommitArgs& c, int r) {
  constexpr int EV = 16 / int(sizeof(T));      // elements per 16-byte vector
  constexpr int CV = 8 / EV;                   // vectors per 8-dim cell (1 bf16, 2 fp32)
  constexpr int RV = kPage * int(sizeof(T)) / 16;   // vectors per value-page row (2 bf16, 4 fp32)
  constexpr int JD = (sizeof(T) == 2) ? 8 : 4;      // value rows rewritten together
  __shared__ int s_pid[kMaxCommitRows];
  __shared__ int s_nv;
  const int N = c.N, Hkv = c.Hkv, D = c.D, max_pages = c.max_pages, num_pages = c.num_pages;
  const int Qn = 2 * N - 1;
  const int cap = max_pages * kPage;
  int L = c.ctx_in[r], n = c.n_commit[r], f = 0;
  const bool bad_n = n < 0 || n > N, bad_L = L < 0 || L > cap;
  if (bad_n) n = n < 0 ? 0 : N;
  if (c.loop_mode && c.loop_mode[r] == ISD_LOOP_REPROPOSE) {   // the resampled token's row
    n = 1;
    f = N - 1;
  }
  if (bad_L) { L = L < 0 ? 0 : cap; n = 0; }
  // the pages of positions L..L+n-1; rows are written up to the first unmapped one
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int pid = (lane < n) ? commit_page(c.table, r, L, lane, max_pages, num_pages) : 0;
    const uint64_t bad = __ballot(pid < 0);
    const int nv = bad ? (__ffsll((unsigned long long)bad) - 1) : n;
    const int first_bad = __shfl(pid, bad ? nv : 0);
    if (lane < n) s_pid[lane] = pid;
    if (lane == 0) {
      s_nv = nv;
      if (bad_n) raise_flag(c.flags, ISD_FLAG_COMMIT_RANGE);
      if (bad_L) raise_flag(c.flags, ISD_FLAG_CTX_RANGE);
      if (bad) raise_flag(c.flags, first_bad == -1 ? ISD_FLAG_COMMIT_RANGE : ISD_FLAG_PAGE_RANGE);
    }
  }
  __syncthreads();
  const int nv = s_nv;
  const T* __restrict__ kn = static_cast<const T*>(c.k_new) + size_t(r) * Qn * Hkv * D;
  const T* __restrict__ vn = static_cast<const T*>(c.v_new) + size_t(r) * Qn * Hkv * D;
  T* __restrict__ kp = static_cast<T*>(c.k_pages);
  T* __restrict__ vp = static_cast<T*>(c.v_pages);
  const int cells = Hkv * D / 8;
  for (int u = threadIdx.x; u < 2 * cells && nv > 0; u += kCommitThreads) {
    const bool is_v = u >= cells;
    const int cell = is_v ? u - cells : u;
    const int h = cell / (D / 8), db = cell % (D / 8);
    if (!is_v) {
      // keys: slot vectors of consecutive positions
      for (int t = 0; t < nv; ++t) {
        const u32x4* src = reinterpret_cast<const u32x4*>(kn + (size_t(f + t) * Hkv + h) * D + db * 8);
        u32x4* dst = reinterpret_cast<u32x4*>(
            kp + ((size_t(s_pid[t]) * Hkv + h) * (D / 8) + db) * (kPage * 8) + ((L + t) % kPage) * 8);
#pragma unroll
        for (int q = 0; q < CV; ++q) dst[q] = src[q];
      }
      continue;
    }
    // values: for every page the committed positions touch (one or two: nv <= 16),
    // JD dims at a time, the dims' rows are read, the new tokens put in (four
    // rows' values in registers at a time) and the rows written back
    for (int t0 = 0; t0 < nv;) {
      const int t1 = min(nv, (L + t0) / kPage * kPage + kPage - L);   // positions of this page
      T* rows = vp + ((size_t(s_pid[t0]) * Hkv + h) * D + db * 8) * kPage;   // 8 consecutive dims' rows
#pragma unroll
      for (int j0 = 0; j0 < 8; j0 += JD) {
        u32x4 row[JD][RV];
#pragma unroll
        for (int j = 0; j < JD; ++j)
#pragma unroll
          for (int q = 0; q < RV; ++q) row[j][q] = reinterpret_cast<const u32x4*>(rows + (j0 + j) * kPage)[q];
        for (int tc = t0; tc < t1; tc += 4) {
          T x[4][JD];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (tc + i < t1) {
              const T* src = vn + (size_t(f + tc + i) * Hkv + h) * D + db * 8 + j0;
#pragma unroll
              for (int j = 0; j < JD; ++j) x[i][j] = src[j];
            }
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (tc + i < t1) {
              const int k = v_sigma((L + tc + i) % kPage);
#pragma unroll
              for (int j = 0; j < JD; ++j) row_put<T, RV>(row[j], k, x[i][j]);
            }
        }
#pragma unroll
        for (int j = 0; j < JD; ++j)
#pragma unroll
          for (int q = 0; q < RV; ++q) reinterpret_cast<u32x4*>(rows + (j0 + j) * kPage)[q] = row[j][q];
      }
      t0 = t1;
    }
  }
  // every wave has read the length before it may be overwritten (ctx_lens_out may alias it)
  __syncthreads();
  if (threadIdx.x == 0) c.ctx_out[r] = L + nv;
}

}  // namespace isd
