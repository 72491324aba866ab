// Stride attention over the paged KV cache (isd_attention).
//
// Work split: a work unit is (request r, KV head hk, split s): a run of
// 32-token tiles (two 16-token pages) of r's context.  One workgroup of W
// waves (four, one per SIMD) serves one unit for all the query columns of
// the GQA group (its G heads x Q stride rows): RB = 1 block of 32 columns
// (two workgroups per CU), or RB = 2 blocks for 33..64 columns, every tile
// then feeding both blocks (one workgroup per CU), so each page is read once.
// The waves take the unit's tiles round-robin, and wave 0 of split 0 also
// takes the stride's own strictly causal block (row i sees stride rows 0..i)
// as one extra, masked tile.  Each wave keeps per column an online softmax
// state (running max m, running sum l, un-normalised output O); the waves
// merge through LDS.  A unit that is the only split of its (r, hk) normalises
// and writes the output directly; otherwise each split publishes a partial
// (m, l, O) with write-through stores and the last split to arrive (an
// atomic count, nobody waits) merges them.
//
// bf16 path (matrix cores): per tile, S^T = K Q^T with
// v_mfma_f32_32x32x16_bf16 (rows = 32 tokens, columns = 32 query columns,
// contraction over the head dim in steps of 16), then O^T += V^T P^T with the
// same instruction (rows = 32 head dims, contraction over the tile's tokens).
// The page layouts (see isd.h) put every MFMA operand in 16 contiguous bytes
// per lane, so K and V go from HBM straight into operand registers with
// fully used 16-byte loads, and P^T goes from the S^T accumulator registers
// into the PV operand without any lane exchange.  Softmax runs in base 2 on
// the VALU; one lane exchange per tile (lane l <-> l^32) shares the column
// max between the two half-waves.
//
// fp32 path: one wave per (request, kv head, split, query column), dot
// products by wave reduction, then a separate combine kernel that merges the
// splits with the stride block.
#include <type_traits>

#include "device_common.hpp"
#include "isd_internal.hpp"

namespace isd {
namespace {

constexpr int kMaxSplits = 64;
constexpr int kRankMax = 256;     // batches up to this size are served longest request first
constexpr int kMaxRows = 64;
constexpr int kMaxQ = 64;

// slot -> storage index inside a V page row: swap bits 2 and 3
__device__ __forceinline__ int v_sigma(int s) { return (s & 3) | ((s & 4) << 1) | ((s & 8) >> 1); }

__device__ __forceinline__ int clamp_ctx(int L, int max_pages, uint32_t* flags) {
  const int cap = max_pages * kPage;
  if (L < 0 || L > cap) {
    raise_flag(flags, ISD_FLAG_CTX_RANGE);
    L = L < 0 ? 0 : cap;
  }
  return L;
}

// Tile range of split s (last split takes the remainder).
__device__ __forceinline__ void split_range(int n_tiles, int s, int n_splits, int tps, int& t0, int& t1) {
  t0 = s * tps;
  t1 = (s == n_splits - 1) ? n_tiles : min(n_tiles, t0 + tps);
}

// Splits that take part for a context of n_tiles tiles: a prefix 0..n-1,
// at least one (an empty context still needs the stride block).
__device__ __forceinline__ int active_splits(int n_tiles, int n_splits, int tps) {
  return max(1, min(n_splits, (n_tiles + tps - 1) / tps));
}

// KV page loads: every page is read exactly once per call, so the loads
// stream past the caches (nontemporal).
__device__ __forceinline__ u32x4 kv_load(const u32x4* p) { return __builtin_nontemporal_load(p); }

// Operand loads of one 32-token tile (pages pid0, pid1; both valid ids).
// One base pointer per lane and page; the unrolled k-steps / dim blocks are
// immediate offsets from it.
template <int D>
__device__ __forceinline__ void load_k(u32x4 (&k)[D / 16], const uint16_t* __restrict__ kp, int pid0,
                                       int pid1, int hk, int Hkv, int lane) {
  const int h = lane >> 5;
  const int i = lane & 31;
  const int pid = (i < 16) ? pid0 : pid1;
  const u32x4* base = reinterpret_cast<const u32x4*>(
      kp + (size_t(pid) * Hkv + hk) * (D * kPage) + (h * kPage + (i & 15)) * 8);
#pragma unroll
  for (int s = 0; s < D / 16; ++s) k[s] = kv_load(base + s * 2 * kPage);
}

template <int D>
__device__ __forceinline__ void load_v(u32x4 (&v)[2][D / 32], const uint16_t* __restrict__ vp, int pid0,
                                       int pid1, int hk, int Hkv, int lane) {
  const int h = lane >> 5;
  const int i = lane & 31;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const u32x4* base = reinterpret_cast<const u32x4*>(
        vp + (size_t(m ? pid1 : pid0) * Hkv + hk) * (D * kPage) + i * kPage + h * 8);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) v[m][db] = kv_load(base + db * 32 * 2);
  }
}

// Page id of logical page lp; an id outside the pool raises the flag and
// reads page 0 instead (the request's result is then unspecified, but no
// access leaves the pool).
__device__ __forceinline__ int page_id(const int32_t* __restrict__ trow, int lp, int num_pages,
                                       uint32_t* flags) {
  const int pid = trow[lp];
  if (pid < 0 || pid >= num_pages) {
    raise_flag(flags, ISD_FLAG_PAGE_RANGE);
    return 0;
  }
  return pid;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// Zero V elements of tokens >= L in a partial tile (page m of tile t).
__device__ __forceinline__ u32x4 mask_v(u32x4 v, int tok_page0, int L, int h) {
  // element e of this lane holds slot (e/4)*8 + h*4 + e%4
  uint32_t w[4] = {v[0], v[1], v[2], v[3]};
#pragma unroll
  for (int e2 = 0; e2 < 4; ++e2) {
    const int e0 = 2 * e2, e1 = 2 * e2 + 1;
    const int s0 = (e0 >> 2) * 8 + h * 4 + (e0 & 3);
    const int s1 = (e1 >> 2) * 8 + h * 4 + (e1 & 3);
    uint32_t keep = 0;
    if (tok_page0 + s0 < L) keep |= 0x0000ffffu;
    if (tok_page0 + s1 < L) keep |= 0xffff0000u;
    w[e2] &= keep;
  }
  return u32x4{w[0], w[1], w[2], w[3]};
}

// Final merge for one (request r, kv head hk), run by a whole 256-thread
// workgroup: the `active` split partials of (r, hk) and the stride's own
// causal block, normalised, written to out.
//   A. every (column c, stride key j <= i(c)) score, one thread per pair;
//   B. per column: global max over split maxima and stride scores, the
//      normaliser, and one coefficient per split / stride key (in LDS);
//   C. every (column, 4 dims) output from the coefficients.
template <typename T, int D>
__device__ __forceinline__ void combine_rk(const T* __restrict__ q, const T* __restrict__ k_new,
                                           const T* __restrict__ v_new, T* __restrict__ out,
                                           const float2* __restrict__ ws_ml, const float* __restrict__ ws_o,
                                           int r, int hk, int Qn, int Hq, int Hkv, int G, int rows,
                                           int rows_pad, int n_splits, int active, float scale_log2,
                                           float (*sc)[kMaxQ], float (*cs)[kMaxSplits]) {
  const int tid = threadIdx.x;
  const int rk = r * Hkv + hk;
  const size_t base0 = size_t(rk) * n_splits * rows_pad;
  const int pairs = rows * Qn;
  for (int pidx = tid; pidx < pairs; pidx += blockDim.x) {
    const int c = pidx / Qn, j = pidx % Qn;
    const int g = c / Qn, i = c % Qn;
    if (j > i) continue;
    const T* qrow = q + ((size_t(r) * Qn + i) * Hq + hk * G + g) * D;
    const T* krow = k_new + ((size_t(r) * Qn + j) * Hkv + hk) * D;
    float acc = 0.f;
#pragma unroll 8
    for (int d = 0; d < D; ++d) acc = fmaf(to_f32<T>(qrow[d]), to_f32<T>(krow[d]), acc);
    sc[c][j] = acc * scale_log2;
  }
  __syncthreads();
  if (tid < rows) {
    const int c = tid, i = c % Qn;
    float M = -INFINITY;
    for (int s = 0; s < active; ++s) M = fmaxf(M, ld_coherent(&ws_ml[base0 + size_t(s) * rows_pad + c].x));
    for (int j = 0; j <= i; ++j) M = fmaxf(M, sc[c][j]);
    float Lsum = 0.f;
    for (int s = 0; s < active; ++s) {
      const float2 ml = make_float2(ld_coherent(&ws_ml[base0 + size_t(s) * rows_pad + c].x),
                                    ld_coherent(&ws_ml[base0 + size_t(s) * rows_pad + c].y));
      const float w = (ml.x == -INFINITY) ? 0.f : exp2f(ml.x - M);
      cs[c][s] = w;
      Lsum += ml.y * w;
    }
    for (int j = 0; j <= i; ++j) {
      const float w = exp2f(sc[c][j] - M);
      sc[c][j] = w;
      Lsum += w;
    }
    const float inv = 1.f / Lsum;
    for (int s = 0; s < active; ++s) cs[c][s] *= inv;
    for (int j = 0; j <= i; ++j) sc[c][j] *= inv;
  }
  __syncthreads();
  constexpr int D4 = D / 4;
  for (int u = tid; u < rows * D4; u += blockDim.x) {
    const int c = u / D4, d0 = (u % D4) * 4;
    const int g = c / Qn, i = c % Qn;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < active; ++s) {
      const float* src = ws_o + (base0 + size_t(s) * rows_pad + c) * D + d0;
      const float w = cs[c][s];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = fmaf(ld_coherent(src + e), w, acc[e]);
    }
    for (int j = 0; j <= i; ++j) {
      const T* vrow = v_new + ((size_t(r) * Qn + j) * Hkv + hk) * D + d0;
      const float w = sc[c][j];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = fmaf(to_f32<T>(vrow[e]), w, acc[e]);
    }
    T* orow = out + ((size_t(r) * Qn + i) * Hq + hk * G + g) * D + d0;
#pragma unroll
    for (int e = 0; e < 4; ++e) orow[e] = from_f32<T>(acc[e]);
  }
}

// RB = row blocks of 32 query columns per wave: 1 (two waves per SIMD, two
// workgroups per CU), or 2 for groups of 33..64 query rows, where every wave
// applies its key and value tiles to both blocks (so a tile crosses from L2
// into the CU once) and takes a whole SIMD's registers.
template <int D, int W, int RB>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(3 - RB, 3 - RB))) void attn_bf16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const uint16_t* __restrict__ kp, const uint16_t* __restrict__ vp, const int32_t* __restrict__ table,
    const int32_t* __restrict__ ctx_lens, uint16_t* __restrict__ out, int Qn, int Hq, int Hkv, int G,
    int rows, int max_pages, int num_pages, int tps, int n_splits, int units, int longest_first,
    float scale_log2,
    float2* __restrict__ ws_ml, float* __restrict__ ws_o, uint32_t* __restrict__ arrivals,
    uint32_t* __restrict__ flags) {
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int COLS = RB * 32;  // query columns of a workgroup
  constexpr int OSTR = D + 4;  // padded LDS row stride
  __shared__ float sm_m[W][COLS];
  __shared__ float sm_l[W][COLS];
  __shared__ __attribute__((aligned(16))) float sm_o0[COLS * OSTR];
  __shared__ __attribute__((aligned(16))) float sm_o1[COLS * OSTR];
  __shared__ __attribute__((aligned(16))) u32x4 sm_q[(D / 8) * COLS];
  __shared__ float sm_ml[COLS][2];
  __shared__ int s_last;

  // Work unit u = blockIdx.x = (request, split, KV head), the head varying
  // fastest; the workgroup serves every query column of its unit.
  const int u = blockIdx.x;
  if (u >= units) return;
  // Workgroup ids equal mod 8 go to one XCD; with the head fastest every XCD
  // gets the same heads of every split of every request (equal work for 8 KV
  // heads), where split-fastest ids would leave the XCDs that hold the later
  // splits idle while short requests, which use one split, run on the others
  const int hk = u % Hkv;
  const int split = (u / Hkv) % n_splits;
  // When the grid takes more than one round of the chip, requests are served
  // longest first (ties in index order): long contexts start early and short
  // ones fill in at the end.  For up to kRankMax requests every workgroup
  // ranks the lengths itself; otherwise, and in a single round, index order.
  const int rank = u / (n_splits * Hkv);
  const int B = units / (n_splits * Hkv);
  int r = rank;
  if (longest_first && B <= kRankMax) {
    __shared__ int sm_len[kRankMax];
    __shared__ int sm_req;
    for (int t = threadIdx.x; t < B; t += blockDim.x) sm_len[t] = ctx_lens[t];
    __syncthreads();
    for (int t = threadIdx.x; t < B; t += blockDim.x) {
      const int lt = sm_len[t];
      int before = 0;
      for (int j = 0; j < B; ++j) {
        const int lj = sm_len[j];
        before += (lj > lt || (lj == lt && j < t)) ? 1 : 0;
      }
      if (before == rank) sm_req = t;
    }
    __syncthreads();
    r = sm_req;
  }
  const int rk = r * Hkv + hk;
  const int row0 = 0;                           // first query row of this workgroup
  const int rows_b = min(COLS, rows);           // query rows of this workgroup
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int h = lane >> 5;
  const int col_l = lane & 31;
  // split 0's wave 0 also takes the stride's own causal block as one extra tile
  const bool stride_tile = (split == 0) && (wave == 0);
  constexpr int CH = D / 8;   // 16-byte chunks per row

  // Requested first, ahead of the context pages (which would otherwise queue
  // in front of them): this thread's Q cells, and for the stride wave the
  // first 32 key rows of the stride block and its first value-row chunks.
  // Indices are clamped so every load is unconditional.
  constexpr int QC = (CH * COLS + 64 * W - 1) / (64 * W);
  u32x4 qc[QC];
#pragma unroll
  for (int j = 0; j < QC; ++j) {
    const int idx = min(int(threadIdx.x) + j * 64 * W, CH * COLS - 1);
    const int ch = idx / COLS, c = min(idx % COLS, rows_b - 1);
    const int g = (row0 + c) / Qn, i = (row0 + c) % Qn;
    qc[j] = *reinterpret_cast<const u32x4*>(q + ((size_t(r) * Qn + i) * Hq + hk * G + g) * D + ch * 8);
  }
  constexpr int kVnEarly = 4;   // value-row chunks per lane requested early (Qn * CH <= 256)
  u32x4 sk[KS], vn[kVnEarly];
  if (stride_tile) {
    const int tic = min(lane & 31, Qn - 1);
#pragma unroll
    for (int s = 0; s < KS; ++s)
      sk[s] = *reinterpret_cast<const u32x4*>(k_new + ((size_t(r) * Qn + tic) * Hkv + hk) * D + (2 * s + h) * 8);
#pragma unroll
    for (int j = 0; j < kVnEarly; ++j) {
      const int c = min(lane + 64 * j, Qn * CH - 1);
      vn[j] = *reinterpret_cast<const u32x4*>(v_new + ((size_t(r) * Qn + c / CH) * Hkv + hk) * D + (c % CH) * 8);
    }
  }
  const int L = clamp_ctx(ctx_lens[r], max_pages, flags);
  const int n_tiles = (L + kTileTokens - 1) / kTileTokens;
  const int active = active_splits(n_tiles, n_splits, tps);
  if (split >= active) return;
  int t0, t1;
  split_range(n_tiles, split, n_splits, tps, t0, t1);

  const int32_t* trow = table + size_t(r) * max_pages;

  // context tiles of this wave: first + W*i for i < n
  const int first = t0 + wave;
  const int n = (first < t1) ? (t1 - first + W - 1) / W : 0;
  // Page ids of this wave's tiles live in one register, 32 tiles at a time:
  // lane 2j+h holds the id of page h of tile j of the current chunk, so the
  // loop reads them with readlane instead of a dependent memory load.
  int pid_reg = 0, pid_chunk = -1;
  auto load_chunk = [&](int chunk) {
    const int j = chunk * 32 + (lane >> 1);
    int pid = 0;
    if (j < n) {
      const int tt = first + W * j;
      // second page past the context: reuse the first (its tokens are masked)
      const int lp = ((lane & 1) && tt * kTileTokens + kPage < L) ? 2 * tt + 1 : 2 * tt;
      pid = page_id(trow, lp, num_pages, flags);
    }
    pid_reg = pid;
    pid_chunk = chunk;
  };
  auto pages_i = [&](int i, int& p0, int& p1) {   // i: index of the tile among this wave's tiles
    if ((i >> 5) != pid_chunk) load_chunk(i >> 5);
    p0 = __builtin_amdgcn_readlane(pid_reg, 2 * (i & 31));
    p1 = __builtin_amdgcn_readlane(pid_reg, 2 * (i & 31) + 1);
  };
  if (n > 0) load_chunk(0);   // page ids of the first tiles, in flight during the staging

  // The stride block's value rows go to LDS (the merge buffer, untouched
  // until the waves combine at the end): lane (h, c) of the PV product needs
  // 8 tokens of dim c, picked from there.
  uint16_t* sm_vn = reinterpret_cast<uint16_t*>(sm_o0);
  if (stride_tile) {
#pragma unroll
    for (int j = 0; j < kVnEarly; ++j) {
      const int c = lane + 64 * j;
      if (c < Qn * CH) *reinterpret_cast<u32x4*>(sm_vn + (c / CH) * D + (c % CH) * 8) = vn[j];
    }
    for (int c = lane + 64 * kVnEarly; c < Qn * CH; c += 64)
      *reinterpret_cast<u32x4*>(sm_vn + (c / CH) * D + (c % CH) * 8) = *reinterpret_cast<const u32x4*>(
          v_new + ((size_t(r) * Qn + c / CH) * Hkv + hk) * D + (c % CH) * 8);
  }
  // Q^T operand B staged in LDS as [dim chunk][column] 16-byte cells: lane
  // (h, column) of k-step ks reads cell (2*ks + h, column); consecutive lanes
  // read consecutive cells.  Columns past the workgroup's rows are zero.
#pragma unroll
  for (int j = 0; j < QC; ++j) {
    const int idx = int(threadIdx.x) + j * 64 * W;
    if (idx < CH * COLS) sm_q[idx] = (idx % COLS < rows_b) ? qc[j] : u32x4{0, 0, 0, 0};
  }
  // The first tile's loads go out after the staging: a wait for the staged
  // values placed after them would also wait for the tile.
  u32x4 ak[KS], av[2][DB], bk[KS], bv[2][DB];
  if (n > 0) {
    int p0, p1;
    pages_i(0, p0, p1);
    load_k<D>(ak, kp, p0, p1, hk, Hkv, lane);
    load_v<D>(av, vp, p0, p1, hk, Hkv, lane);
  }
  __syncthreads();

  f32x16 o[RB][DB];
  float m_run[RB], l_run[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_run[rb] = -INFINITY;
    l_run[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[rb][db] = f32x16{};
  }

  // S^T = K Q^T for one 32-token tile
  auto scores = [&](const u32x4 (&ck)[KS], f32x16 (&s)[RB]) {
    int qcell = h * COLS + col_l;
    asm volatile("" : "+v"(qcell));   // keep the Q operand reads inside the loop
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      s[rb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        s[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ck[ks]),
                                                        as_bf16x8(sm_q[qcell + 2 * ks * COLS + rb * 32]),
                                                        s[rb], 0, 0, 0);
    }
  };
  // online softmax update and O^T += V^T P^T; valid(rb, v) says whether
  // accumulator entry v (token (v/4)*8 + h*4 + v%4 of the tile) counts
  auto consume = [&](f32x16 (&s)[RB], const u32x4 (&cv)[2][DB], auto valid) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float mx = -INFINITY;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float x = s[rb][v] * scale_log2;
        if (!valid(rb, v)) x = -INFINITY;
        s[rb][v] = x;
        mx = fmaxf(mx, x);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run[rb], mx);
      // the hardware exp2 (no range fix-up: arguments are <= 0 and a weight below
      // 2^-126 is negligible against the running sum, which holds a 1); a -inf
      // argument gives 0
      const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run[rb] - m_new);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;   // all masked so far: every s is -inf
      m_run[rb] = m_new;
      float psum = 0.f;
      bf16x8 pb[2];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = __builtin_amdgcn_exp2f(s[rb][v] - m_use);
        psum += p;
        pb[v >> 3][v & 7] = (__bf16)p;
      }
      l_run[rb] = l_run[rb] * alpha + psum;
      // rescale only when some column's running max moved
      if (__ballot(alpha != 1.f)) {
#pragma unroll
        for (int db = 0; db < DB; ++db) o[rb][db] *= alpha;
      }
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int m = 0; m < 2; ++m)
          o[rb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(cv[m][db]), pb[m], o[rb][db], 0, 0, 0);
    }
  };

  // ---- the stride block: keys/values of this pass's rows, masked j <= i ----
  // One 32-token block (Qn <= 31); key rows past Qn were read as row Qn - 1
  // and are zeroed here, value rows past Qn read as zero.
  if (stride_tile) {
#pragma unroll
    for (int s = 0; s < KS; ++s)
      if ((lane & 31) >= Qn) sk[s] = u32x4{0, 0, 0, 0};
    u32x4 sv[2][DB];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint16_t* vcol = sm_vn + db * 32 + (lane & 31);
        uint32_t w[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          uint32_t pair = 0;
#pragma unroll
          for (int hi = 0; hi < 2; ++hi) {
            const int e = 2 * e2 + hi;
            const int t = 16 * m + (e >> 2) * 8 + h * 4 + (e & 3);
            const uint32_t raw = vcol[min(t, Qn - 1) * D];
            const uint32_t bits = (t < Qn) ? raw : 0u;
            pair |= bits << (16 * hi);
          }
          w[e2] = pair;
        }
        sv[m][db] = u32x4{w[0], w[1], w[2], w[3]};
      }
    f32x16 s[RB];
    scores(sk, s);
    consume(s, sv, [&](int rb, int v) {
      const int t = (v >> 2) * 8 + h * 4 + (v & 3);
      const int i = (row0 + rb * 32 + col_l) % Qn;    // stride row of this column
      return t <= i;                           // t < Qn follows from i < Qn
    });
  }

  // ---- context tiles: software pipeline over this wave's tiles ----
  // The next tile's keys are requested before this tile's S^T product and
  // its values right after it.  Two register sets alternate; the last tile is
  // peeled so that every load inside the loop is unconditional.
  auto tile = [&](auto prefetch, u32x4 (&ck)[KS], u32x4 (&cv)[2][DB], u32x4 (&nv)[2][DB], int tt,
                  int np0, int np1) {
    const int tok0 = tt * kTileTokens;
    const bool partial = tok0 + kTileTokens > L;
    f32x16 s[RB];
    scores(ck, s);
    if constexpr (decltype(prefetch)::value) load_v<D>(nv, vp, np0, np1, hk, Hkv, lane);
    if (partial) {
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int db = 0; db < DB; ++db) cv[m][db] = mask_v(cv[m][db], tok0 + 16 * m, L, h);
    }
    consume(s, cv, [&](int, int v) { return !partial || tok0 + (v >> 2) * 8 + h * 4 + (v & 3) < L; });
  };
  using Pre = std::integral_constant<bool, true>;
  using NoPre = std::integral_constant<bool, false>;

  if (n > 0) {
    int p0 = 0, p1 = 0;
    int i = 0;
    for (; i + 2 < n; i += 2) {
      const int ta = first + i * W, tb = ta + W;
      pages_i(i + 1, p0, p1);
      load_k<D>(bk, kp, p0, p1, hk, Hkv, lane);
      tile(Pre{}, ak, av, bv, ta, p0, p1);
      pages_i(i + 2, p0, p1);
      load_k<D>(ak, kp, p0, p1, hk, Hkv, lane);
      tile(Pre{}, bk, bv, av, tb, p0, p1);
    }
    const int ta = first + i * W;
    if (i + 1 < n) {
      pages_i(i + 1, p0, p1);
      load_k<D>(bk, kp, p0, p1, hk, Hkv, lane);
      tile(Pre{}, ak, av, bv, ta, p0, p1);
      tile(NoPre{}, bk, bv, av, ta + W, 0, 0);
    } else {
      tile(NoPre{}, ak, av, bv, ta, 0, 0);
    }
  }

  // ---- merge the W waves of the workgroup ----
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float l_tot = l_run[rb] + __shfl_xor(l_run[rb], 32);
    if (h == 0) {
      sm_m[wave][rb * 32 + col_l] = m_run[rb];
      sm_l[wave][rb * 32 + col_l] = l_tot;
    }
  }
  __syncthreads();
  float wscale[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int c = rb * 32 + col_l;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < W; ++w) M = fmaxf(M, sm_m[w][c]);
    wscale[rb] = (m_run[rb] == -INFINITY) ? 0.f : exp2f(m_run[rb] - M);
  }
  auto put = [&](float* buf, bool add) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int c = rb * 32 + col_l;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          const int d0 = db * 32 + v4 * 8 + h * 4;
          f32x4 val = {o[rb][db][4 * v4 + 0], o[rb][db][4 * v4 + 1], o[rb][db][4 * v4 + 2],
                       o[rb][db][4 * v4 + 3]};
          val *= wscale[rb];
          f32x4* dst = reinterpret_cast<f32x4*>(&buf[c * OSTR + d0]);
          if (add) *dst += val; else *dst = val;
        }
    }
  };
  if (wave < 2) put(wave ? sm_o1 : sm_o0, false);
  if (threadIdx.x < rows_b) {
    const int c = threadIdx.x;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < W; ++w) M = fmaxf(M, sm_m[w][c]);
    float Lsum = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const float mw = sm_m[w][c];
      if (mw != -INFINITY) Lsum += sm_l[w][c] * exp2f(mw - M);
    }
    sm_ml[c][0] = M;
    sm_ml[c][1] = Lsum;
  }
  __syncthreads();
#pragma unroll
  for (int k = 1; k < W / 2; ++k) {
    if (wave == 2 * k || wave == 2 * k + 1) put((wave & 1) ? sm_o1 : sm_o0, true);
    __syncthreads();
  }

  constexpr int V4 = D / 4;
  auto write_out = [&](int c, int d0, f32x4 v) {
    const int g = (row0 + c) / Qn, i = (row0 + c) % Qn;
    uint16_t* dst = out + ((size_t(r) * Qn + i) * Hq + hk * G + g) * D + d0;
    const uint32_t lo = uint32_t(f32_to_bf16_bits(v[0])) | (uint32_t(f32_to_bf16_bits(v[1])) << 16);
    const uint32_t hi = uint32_t(f32_to_bf16_bits(v[2])) | (uint32_t(f32_to_bf16_bits(v[3])) << 16);
    *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
  };
  if (active == 1) {
    // the only split: normalise straight from LDS
    for (int idx = threadIdx.x; idx < rows_b * V4; idx += blockDim.x) {
      const int c = idx / V4, d0 = (idx % V4) * 4;
      const f32x4 a = *reinterpret_cast<const f32x4*>(&sm_o0[c * OSTR + d0]);
      const f32x4 b2 = *reinterpret_cast<const f32x4*>(&sm_o1[c * OSTR + d0]);
      write_out(c, d0, (a + b2) * (1.f / sm_ml[c][1]));
    }
    return;
  }

  // several splits: publish this split's partial, the last to arrive merges
  const int RSTR = COLS;                        // partial rows per (request, KV head, split)
  const size_t base = (size_t(rk) * n_splits + split) * RSTR + row0;
  // Write-through stores, consecutive lanes on consecutive addresses, so each
  // store instruction covers whole cache lines.
  if (threadIdx.x < rows_b) {
    const uint64_t ml = uint64_t(__float_as_uint(sm_ml[threadIdx.x][0])) |
                        (uint64_t(__float_as_uint(sm_ml[threadIdx.x][1])) << 32);
    st_coherent(reinterpret_cast<uint64_t*>(ws_ml + base + threadIdx.x), ml);
  }
  // the O rows of this (request, KV head): [split][RSTR rows][D], as 16-byte pieces
  const size_t base0 = size_t(rk) * n_splits * RSTR + row0;
  const __amdgpu_buffer_rsrc_t o_rsrc =
      coherent_rsrc(ws_o + size_t(rk) * n_splits * RSTR * D, n_splits * RSTR * D * int(sizeof(float)));
  for (int f4 = threadIdx.x; f4 < rows_b * V4; f4 += blockDim.x) {
    const int c = f4 / V4, d0 = (f4 % V4) * 4;
    const f32x4 a = *reinterpret_cast<const f32x4*>(&sm_o0[c * OSTR + d0]);
    const f32x4 b2 = *reinterpret_cast<const f32x4*>(&sm_o1[c * OSTR + d0]);
    st_coherent16(o_rsrc, ((split * RSTR + row0 + c) * D + d0) * int(sizeof(float)), a + b2);
  }
  if (!arrive_last(&arrivals[rk], uint32_t(active), &s_last)) return;
  // The partials were written through to memory before their writers
  // arrived; device-coherent loads read them from there.  (An acquire fence
  // plus plain loads invalidates the XCD's L2 and costs far more.)
#define MERGE_LD(p) ld_coherent(p)
  // per row: global max and the split weights (normaliser folded in); the
  // loads of each batch of splits are all issued before any is used
  __shared__ float sm_w[COLS][kMaxSplits];
  __shared__ float sm_sm[COLS][kMaxSplits];
  if (threadIdx.x < rows_b) {
    const int c = threadIdx.x;
    float M = -INFINITY;
    for (int s0 = 0; s0 < active; s0 += 8) {
      uint64_t v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        v[k] = (s0 + k < active)
                   ? MERGE_LD(reinterpret_cast<const uint64_t*>(ws_ml + base0 + size_t(s0 + k) * RSTR + c))
                   : 0ull;
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (s0 + k < active) {
          const float m = __uint_as_float(uint32_t(v[k]));
          sm_sm[c][s0 + k] = m;
          sm_w[c][s0 + k] = __uint_as_float(uint32_t(v[k] >> 32));
          M = fmaxf(M, m);
        }
    }
    float Lsum = 0.f;
    for (int s = 0; s < active; ++s) {
      const float m = sm_sm[c][s];
      const float w = (m == -INFINITY) ? 0.f : exp2f(m - M);
      Lsum += w * sm_w[c][s];
      sm_w[c][s] = w;
    }
    const float inv = 1.f / Lsum;
    for (int s = 0; s < active; ++s) sm_w[c][s] *= inv;
  }
  __syncthreads();
  // every thread owns up to J 4-float pieces of the output; the 16-byte loads
  // of SB splits at a time go out before their sums (added in split order)
  constexpr int J = (COLS * V4 + 64 * W - 1) / (64 * W);
  constexpr int SB = 4;
  const int n4 = rows_b * V4;
  f32x4 acc[J];
#pragma unroll
  for (int j = 0; j < J; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  int off[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int f4 = min(int(threadIdx.x) + j * 64 * W, n4 - 1);
    off[j] = ((row0 + f4 / V4) * D + (f4 % V4) * 4) * int(sizeof(float));
  }
  const int split_bytes = RSTR * D * int(sizeof(float));
  for (int s0 = 0; s0 < active; s0 += SB) {
    f32x4 v[SB][J];
#pragma unroll
    for (int k = 0; k < SB; ++k)
#pragma unroll
      for (int j = 0; j < J; ++j) v[k][j] = ld_coherent16(o_rsrc, min(s0 + k, active - 1) * split_bytes + off[j]);
#pragma unroll
    for (int k = 0; k < SB; ++k)
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int f4 = threadIdx.x + j * 64 * W;
        if (s0 + k < active && f4 < n4) acc[j] += v[k][j] * sm_w[f4 / V4][s0 + k];
      }
  }
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int f4 = threadIdx.x + j * 64 * W;
    if (f4 < n4) write_out(f4 / V4, (f4 % V4) * 4, acc[j]);
  }
#undef MERGE_LD
}

// fp32 path: one wave per (request, kv head, split) x query column.
template <int D>
__global__ __launch_bounds__(64) void attn_split_f32(
    const float* __restrict__ q, const float* __restrict__ kp, const float* __restrict__ vp,
    const int32_t* __restrict__ table, const int32_t* __restrict__ ctx_lens, int Qn, int Hq, int Hkv,
    int G, int rows, int rows_pad, int max_pages, int num_pages, int tps, int n_splits,
    float scale_log2, float2* __restrict__ ws_ml, float* __restrict__ ws_o,
    uint32_t* __restrict__ flags) {
  constexpr int E = D / 64;  // dims per lane
  const int split = blockIdx.x % n_splits;
  const int rk = blockIdx.x / n_splits;
  const int hk = rk % Hkv;
  const int r = rk / Hkv;
  const int c = blockIdx.y;
  if (c >= rows) return;
  const int L = clamp_ctx(ctx_lens[r], max_pages, flags);
  const int n_tiles = (L + kTileTokens - 1) / kTileTokens;
  if (split >= active_splits(n_tiles, n_splits, tps)) return;
  int t0, t1;
  split_range(n_tiles, split, n_splits, tps, t0, t1);
  const int lane = threadIdx.x;
  const int g = c / Qn, i = c % Qn;
  const float* qrow = q + ((size_t(r) * Qn + i) * Hq + hk * G + g) * D;
  float qv[E], acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) { qv[e] = qrow[lane * E + e]; acc[e] = 0.f; }
  float m = -INFINITY, l = 0.f;
  const int32_t* trow = table + size_t(r) * max_pages;
  const int tok_end = min(L, t1 * kTileTokens);
  for (int tok = t0 * kTileTokens; tok < tok_end; ++tok) {
    const int pid = page_id(trow, tok / kPage, num_pages, flags);
    const int slot = tok % kPage;
    float part = 0.f;
    float vv[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int d = lane * E + e;
      const float kx = kp[((size_t(pid) * Hkv + hk) * (D / 8) + d / 8) * (kPage * 8) + slot * 8 + (d & 7)];
      vv[e] = vp[((size_t(pid) * Hkv + hk) * D + d) * kPage + v_sigma(slot)];
      part = fmaf(qv[e], kx, part);
    }
    const float sc = wave_sum(part) * scale_log2;
    const float m_new = fmaxf(m, sc);
    const float alpha = exp2f(m - m_new);
    const float p = exp2f(sc - m_new);
    l = l * alpha + p;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = acc[e] * alpha + p * vv[e];
    m = m_new;
  }
  const size_t base = (size_t(rk) * n_splits + split) * rows_pad;
  if (lane == 0) ws_ml[base + c] = make_float2(m, l);
#pragma unroll
  for (int e = 0; e < E; ++e) ws_o[(base + c) * D + lane * E + e] = acc[e];
}

template <typename T, int D>
__global__ __launch_bounds__(256) void attn_combine(
    const T* __restrict__ q, const T* __restrict__ k_new, const T* __restrict__ v_new,
    const int32_t* __restrict__ ctx_lens, T* __restrict__ out, const float2* __restrict__ ws_ml,
    const float* __restrict__ ws_o, int Qn, int Hq, int Hkv, int G, int rows, int rows_pad,
    int max_pages, int tps, int n_splits, float scale_log2) {
  __shared__ float sc[kMaxRows][kMaxQ];
  __shared__ float cs[kMaxRows][kMaxSplits];
  const int rk = blockIdx.x;
  const int hk = rk % Hkv;
  const int r = rk / Hkv;
  int L = ctx_lens[r];
  L = (L < 0) ? 0 : min(L, max_pages * kPage);   // flag already raised by the split kernel
  const int n_tiles = (L + kTileTokens - 1) / kTileTokens;
  combine_rk<T, D>(q, k_new, v_new, out, ws_ml, ws_o, r, hk, Qn, Hq, Hkv, G, rows, rows_pad, n_splits,
                   active_splits(n_tiles, n_splits, tps), scale_log2, sc, cs);
}

template <int D>
hipError_t launch_d(const isd_shape& s, const AttnPlan& p, const void* q, const void* k_new,
                    const void* v_new, const void* k_pages, const void* v_pages,
                    const int32_t* table, const int32_t* ctx_lens, float scale, void* out, char* ws,
                    const WsLayout& Lw, hipStream_t stream) {
  const float scale_log2 = scale * kLog2e;
  uint32_t* flags = reinterpret_cast<uint32_t*>(ws + Lw.flags);
  uint32_t* arrivals = reinterpret_cast<uint32_t*>(ws + Lw.attn_cnt);
  float2* ml = reinterpret_cast<float2*>(ws + Lw.attn_ml);
  float* po = reinterpret_cast<float*>(ws + Lw.attn_o);
  const int nwg = s.batch * s.n_kv_heads * p.n_splits;
  // longest requests first once the grid takes more than half a round of the
  // chip (one resident workgroup per CU with two row blocks, two with one)
  const int longest_first = (nwg > device_cus() * (p.row_blocks == 1 ? 2 : 1) / 2) ? 1 : 0;
  if (s.kv_dtype == ISD_BF16) {
    const uint16_t* qq = static_cast<const uint16_t*>(q);
    const uint16_t* kn = static_cast<const uint16_t*>(k_new);
    const uint16_t* vn = static_cast<const uint16_t*>(v_new);
    const uint16_t* kp = static_cast<const uint16_t*>(k_pages);
    const uint16_t* vp = static_cast<const uint16_t*>(v_pages);
    uint16_t* o = static_cast<uint16_t*>(out);
    // one workgroup per (request, KV head, split): its waves cover the 32 query rows,
    // or 64 in two row blocks
    if (p.row_blocks == 1)
      hipLaunchKernelGGL((attn_bf16<D, kAttnWaves, 1>), dim3(nwg), dim3(64 * kAttnWaves), 0, stream,
                         qq, kn, vn, kp, vp, table, ctx_lens, o, p.q_rows, s.n_q_heads, s.n_kv_heads, p.group,
                         p.rows, s.max_pages, s.num_pages, p.tiles_per_split, p.n_splits, nwg, longest_first,
                         scale_log2, ml, po, arrivals, flags);
    else
      hipLaunchKernelGGL((attn_bf16<D, kAttnWaves, 2>), dim3(nwg), dim3(64 * kAttnWaves), 0, stream,
                         qq, kn, vn, kp, vp, table, ctx_lens, o, p.q_rows, s.n_q_heads, s.n_kv_heads, p.group,
                         p.rows, s.max_pages, s.num_pages, p.tiles_per_split, p.n_splits, nwg, longest_first,
                         scale_log2, ml, po, arrivals, flags);
  } else {
    const float* qq = static_cast<const float*>(q);
    hipLaunchKernelGGL((attn_split_f32<D>), dim3(nwg, p.rows), dim3(64), 0, stream, qq,
                       static_cast<const float*>(k_pages), static_cast<const float*>(v_pages), table,
                       ctx_lens, p.q_rows, s.n_q_heads, s.n_kv_heads, p.group, p.rows, p.rows_pad,
                       s.max_pages, s.num_pages, p.tiles_per_split, p.n_splits, scale_log2, ml, po,
                       flags);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attn_combine<float, D>), dim3(s.batch * s.n_kv_heads), dim3(256), 0, stream,
                       qq, static_cast<const float*>(k_new), static_cast<const float*>(v_new),
                       ctx_lens, static_cast<float*>(out), ml, po, p.q_rows, s.n_q_heads,
                       s.n_kv_heads, p.group, p.rows, p.rows_pad, s.max_pages, p.tiles_per_split,
                       p.n_splits, scale_log2);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const isd_shape& s, const AttnPlan& p, const void* q, const void* k_new,
                            const void* v_new, const void* k_pages, const void* v_pages,
                            const int32_t* table, const int32_t* ctx_lens, float scale, void* out,
                            char* ws, const WsLayout& L, hipStream_t stream) {
  if (s.head_dim == 128)
    return launch_d<128>(s, p, q, k_new, v_new, k_pages, v_pages, table, ctx_lens, scale, out, ws, L, stream);
  return launch_d<64>(s, p, q, k_new, v_new, k_pages, v_pages, table, ctx_lens, scale, out, ws, L, stream);
}

}  // namespace isd
