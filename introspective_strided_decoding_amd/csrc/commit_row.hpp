// Appending accepted stride rows to the KV pages: the device code shared by
// the kv_commit kernel and the accept launch that also commits.
//
// One workgroup per request r.  The request commits n rows starting at
// stride row f: row f + t goes to position L + t (L = its length before the
// commit).  Normally f = 0 and n = n_commit[r] (the accepted
// prefix x_1..x_A); a request of the decoding loop in re-proposing mode
// commits row N-1 only (f = N-1, n = 1), which carries the token its previous
// forward resampled.  The rows are written only as far as the pages of their
// positions are mapped, and the new length is L plus the rows written, so
// ctx_lens_out may alias ctx_lens_in.
//
// Keys: one item per (row t, KV head, 8 head dims), a 16-byte slot vector
// (consecutive slots are contiguous in the key layout), read and written with
// consecutive items on consecutive lanes.  Values: a thread owns value rows
// (KV head, head dim) h*D + d, consecutive rows on consecutive lanes, and
// rewrites each row's whole 16 slots on every page the committed positions
// touch (at most two): it reads the row, puts the new tokens' values at their
// (swizzled) slots and writes the row back with full 16-byte stores, so no
// store writes a partial 32-byte sector (a row holds one token per slot, 2
// bytes each in bf16, and a commit adds only a few tokens to it), and a
// wave's reads and writes of a page are contiguous.  Every wave looks the
// page ids up itself, so no barrier stands between a thread's loads and its
// stores: a request's commit is three memory round trips (its length and
// count; the page ids and the new rows; the value rows).  One workgroup per
// request owns every row it rewrites.
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

// Commit request r's rows; call with all kT threads of the workgroup (256 in
// kv_commit, 1024 inside the selection launch).
constexpr int kCommitPre = 8;        // new tokens whose values a value thread requests with its rows

template <typename T, int kT = kCommitThreads>
__device__ __forceinline__ void commit_request(const CommitArgs& c, int r) {
  constexpr int kCommitRowsPer = kT >= 1024 ? 1 : 1024 / kT;   // value rows a thread rewrites in one pass
  constexpr int kCommitKeyItems = kT >= 512 ? 1 : 512 / kT;    // key items requested before the first store
  constexpr int EV = 16 / int(sizeof(T));      // elements per 16-byte vector
  constexpr int CV = 8 / EV;                   // vectors per 8-dim key cell (1 bf16, 2 fp32)
  constexpr int RV = kPage * int(sizeof(T)) / 16;   // vectors per value-page row (2 bf16, 4 fp32)
  const int N = c.N, Hkv = c.Hkv, D = c.D, max_pages = c.max_pages, num_pages = c.num_pages;
  const int Qn = 2 * N - 1;
  const int cap = max_pages * kPage;
  const int lane = threadIdx.x & 63;
  // the mode is read through a valid address either way, so that the three
  // loads are in flight together
  const int mode = *(c.loop_mode ? c.loop_mode + r : c.ctx_in + r);
  int L = c.ctx_in[r], n = c.n_commit[r], f = 0;
  const bool bad_n = n < 0 || n > N, bad_L = L < 0 || L > cap;
  if (bad_n) n = n < 0 ? 0 : N;
  if (c.loop_mode && mode == ISD_LOOP_REPROPOSE) {   // the resampled token's row
    n = 1;
    f = N - 1;
  }
  if (bad_L) { L = L < 0 ? 0 : cap; n = 0; }
  const T* __restrict__ kn = static_cast<const T*>(c.k_new) + size_t(r) * Qn * Hkv * D;
  const T* __restrict__ vn = static_cast<const T*>(c.v_new) + size_t(r) * Qn * Hkv * D;
  T* __restrict__ kp = static_cast<T*>(c.k_pages);
  T* __restrict__ vp = static_cast<T*>(c.v_pages);
  const int cells = Hkv * D / 8;   // key items per row: (KV head, 8 head dims)
  const int rows = Hkv * D;        // value rows per page: (KV head, head dim)
  const int t_last = max(n, 1) - 1;   // loads past the commit read its last row again (row f when empty)
  auto key_src = [&](int t, int cell) {
    return reinterpret_cast<const u32x4*>(kn + (size_t(f + t) * Hkv + cell / (D / 8)) * D + (cell % (D / 8)) * 8);
  };
  // Requested together with the page ids: this thread's first key items and
  // the new tokens' values of its first value rows (they need only f and n).
  u32x4 kv[kCommitKeyItems][CV];
#pragma unroll
  for (int j = 0; j < kCommitKeyItems; ++j) {
    const int i = min(int(threadIdx.x) + j * kT, cells * (t_last + 1) - 1);
    const u32x4* src = key_src(i / cells, i % cells);
#pragma unroll
    for (int q = 0; q < CV; ++q) kv[j][q] = src[q];
  }
  T x[kCommitRowsPer][kCommitPre];
  auto load_values = [&](int base) {
#pragma unroll
    for (int j = 0; j < kCommitRowsPer; ++j) {
      const int row = min(base + int(threadIdx.x) + j * kT, rows - 1);
#pragma unroll
      for (int t = 0; t < kCommitPre; ++t) x[j][t] = vn[size_t(f + min(t, t_last)) * rows + row];
    }
  };
  load_values(0);
  // the pages of positions L..L+n-1 (lane t: position L + t); rows are written
  // up to the first unmapped one
  const int pid = (lane < n) ? commit_page(c.table, r, L, lane, max_pages, num_pages) : 0;
  const uint64_t bad = __ballot(pid < 0);
  const int nv = bad ? (__ffsll((unsigned long long)bad) - 1) : n;
  const int first_bad = __shfl(pid, bad ? nv : 0);
  if (threadIdx.x == 0) {
    if (bad_n) raise_flag(c.flags, ISD_FLAG_COMMIT_RANGE);
    if (bad_L) raise_flag(c.flags, ISD_FLAG_CTX_RANGE);
    if (bad) raise_flag(c.flags, first_bad == -1 ? ISD_FLAG_COMMIT_RANGE : ISD_FLAG_PAGE_RANGE);
  }
  if (nv > 0) {
    // positions [0, t_split) lie on the first page, the rest (nv <= 16) on the next one
    const int t_split = min(nv, kPage - L % kPage);
    const bool two_pages = t_split < nv;
    const int page_a = __builtin_amdgcn_readlane(pid, 0);
    const int page_b = __builtin_amdgcn_readlane(pid, two_pages ? t_split : 0);
    // value rows (whole 16-slot rows of both pages; the second is the first
    // again when one page holds every position)
    u32x4 ra[kCommitRowsPer][RV], rb[kCommitRowsPer][RV];
    auto load_rows = [&](int base) {
#pragma unroll
      for (int j = 0; j < kCommitRowsPer; ++j) {
        const int row = min(base + int(threadIdx.x) + j * kT, rows - 1);
        const u32x4* a = reinterpret_cast<const u32x4*>(vp + (size_t(page_a) * rows + row) * kPage);
        const u32x4* b = reinterpret_cast<const u32x4*>(vp + (size_t(page_b) * rows + row) * kPage);
#pragma unroll
        for (int q = 0; q < RV; ++q) {
          ra[j][q] = a[q];
          rb[j][q] = b[q];
        }
      }
    };
    // the new tokens' values put at their (swizzled) slots, the rows written back
    auto update_rows = [&](int base) {
#pragma unroll
      for (int t = 0; t < kCommitPre; ++t)
        if (t < nv) {
          const int k = v_sigma((L + t) % kPage);
#pragma unroll
          for (int j = 0; j < kCommitRowsPer; ++j) {
            if (t < t_split)
              row_put<T, RV>(ra[j], k, x[j][t]);
            else
              row_put<T, RV>(rb[j], k, x[j][t]);
          }
        }
      for (int t = kCommitPre; t < nv; ++t) {   // N > 8 only
        const int k = v_sigma((L + t) % kPage);
#pragma unroll
        for (int j = 0; j < kCommitRowsPer; ++j) {
          const int row = min(base + int(threadIdx.x) + j * kT, rows - 1);
          const T v = vn[size_t(f + t) * rows + row];
          if (t < t_split)
            row_put<T, RV>(ra[j], k, v);
          else
            row_put<T, RV>(rb[j], k, v);
        }
      }
#pragma unroll
      for (int j = 0; j < kCommitRowsPer; ++j) {
        const int row = base + int(threadIdx.x) + j * kT;
        if (row < rows) {
          u32x4* a = reinterpret_cast<u32x4*>(vp + (size_t(page_a) * rows + row) * kPage);
          u32x4* b = reinterpret_cast<u32x4*>(vp + (size_t(page_b) * rows + row) * kPage);
#pragma unroll
          for (int q = 0; q < RV; ++q) {
            a[q] = ra[j][q];
            if (two_pages) b[q] = rb[j][q];
          }
        }
      }
    };
    load_rows(0);   // requested before the key stores, which need nothing more
    // ---- keys: slot vectors of consecutive positions ----
    const int items = cells * nv;
    auto key_dst = [&](int t, int cell) {
      const int page = t < t_split ? page_a : page_b;
      return reinterpret_cast<u32x4*>(kp + ((size_t(page) * Hkv + cell / (D / 8)) * (D / 8) + cell % (D / 8)) *
                                               (kPage * 8) + ((L + t) % kPage) * 8);
    };
#pragma unroll
    for (int j = 0; j < kCommitKeyItems; ++j) {
      const int i = int(threadIdx.x) + j * kT;
      if (i < items) {
        u32x4* dst = key_dst(i / cells, i % cells);
#pragma unroll
        for (int q = 0; q < CV; ++q) dst[q] = kv[j][q];
      }
    }
    // more key items than the first passes hold (large heads or many rows)
    for (int i = int(threadIdx.x) + kCommitKeyItems * kT; i < items; i += kT) {
      const u32x4* src = key_src(i / cells, i % cells);
      u32x4* dst = key_dst(i / cells, i % cells);
#pragma unroll
      for (int q = 0; q < CV; ++q) dst[q] = src[q];
    }
    // ---- values ----
    update_rows(0);
    for (int base = kCommitRowsPer * kT; base < rows; base += kCommitRowsPer * kT) {
      load_values(base);   // more value rows than one pass holds (large heads)
      load_rows(base);
      update_rows(base);
    }
  }
  // every wave has read the length before it may be overwritten (ctx_lens_out may alias it)
  __syncthreads();
  if (threadIdx.x == 0) c.ctx_out[r] = L + nv;
}

}  // namespace isd
