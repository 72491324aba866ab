// Stride attention over the paged KV cache (isd_attention).
//
// Work split: workgroup (r, kv head hk, split s) walks tiles of 32 context
// tokens (two 16-token pages) of request r.  Its four waves take the tiles of
// the split round-robin.  Each wave keeps, for every query column of the GQA
// group (G heads x Q stride rows, padded to 32 or 64 columns), an online
// softmax state (running max m, running sum l, un-normalised output O); the
// four waves merge through LDS and the workgroup writes one partial (m, l, O)
// per column.  The combine kernel merges the partials of all splits with the
// strictly causal block of the stride itself (row i sees stride rows 0..i)
// and normalises.
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
// products by wave reduction; the same partial format and combine kernel.
#include "device_common.hpp"
#include "isd_internal.hpp"

namespace isd {
namespace {

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

template <int D>
struct TileFrag {
  u32x4 k[D / 16];          // S^T operand A per k-step: 8 dims of one token
  u32x4 v[2][D / 32];       // O^T operand A per (page, dim block): 8 tokens of one dim
};

template <int D>
__device__ __forceinline__ void load_tile(TileFrag<D>& f, const uint16_t* __restrict__ kp,
                                          const uint16_t* __restrict__ vp, int pid0, int pid1,
                                          int hk, int Hkv, int lane) {
  const int h = lane >> 5;
  const int i = lane & 31;
  const int pid_k = (i < 16) ? pid0 : pid1;
  const int slot = i & 15;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    if (pid_k >= 0) {
      const size_t off = ((size_t(pid_k) * Hkv + hk) * (D / 8) + (2 * s + h)) * (kPage * 8) + slot * 8;
      f.k[s] = *reinterpret_cast<const u32x4*>(kp + off);
    } else {
      f.k[s] = u32x4{0, 0, 0, 0};
    }
  }
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int pid = m ? pid1 : pid0;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      if (pid >= 0) {
        const int d = db * 32 + i;
        const size_t off = ((size_t(pid) * Hkv + hk) * D + d) * kPage + h * 8;
        f.v[m][db] = *reinterpret_cast<const u32x4*>(vp + off);
      } else {
        f.v[m][db] = u32x4{0, 0, 0, 0};
      }
    }
  }
}

__device__ __forceinline__ int page_id(const int32_t* __restrict__ trow, int lp, int num_pages,
                                       uint32_t* flags) {
  const int pid = trow[lp];
  if (pid < 0 || pid >= num_pages) {
    raise_flag(flags, ISD_FLAG_PAGE_RANGE);
    return -1;
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

template <int D, int RB>
__global__ __launch_bounds__(256) void attn_split_bf16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kp, const uint16_t* __restrict__ vp,
    const int32_t* __restrict__ table, const int32_t* __restrict__ ctx_lens, int Qn, int Hq, int Hkv,
    int G, int rows, int max_pages, int num_pages, int tps, int n_splits, float scale_log2,
    float2* __restrict__ ws_ml, float* __restrict__ ws_o, uint32_t* __restrict__ flags) {
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int COLS = RB * 32;
  constexpr int OSTR = D + 4;  // padded LDS row stride
  __shared__ float sm_m[kAttnWaves][COLS];
  __shared__ float sm_l[kAttnWaves][COLS];
  __shared__ __attribute__((aligned(16))) float sm_o[2][COLS * OSTR];

  const int split = blockIdx.x % n_splits;
  const int rk = blockIdx.x / n_splits;
  const int hk = rk % Hkv;
  const int r = rk / Hkv;
  const int L = clamp_ctx(ctx_lens[r], max_pages, flags);
  const int n_tiles = (L + kTileTokens - 1) / kTileTokens;
  int t0, t1;
  split_range(n_tiles, split, n_splits, tps, t0, t1);
  if (t0 >= t1) return;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int h = lane >> 5;
  const int col_l = lane & 31;
  const int32_t* trow = table + size_t(r) * max_pages;

  // Q^T operand B per (row block, k-step): 8 dims of one query column.
  u32x4 qf[RB][KS];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int c = rb * 32 + col_l;
    if (c < rows) {
      const int g = c / Qn, i = c % Qn;
      const uint16_t* qrow = q + ((size_t(r) * Qn + i) * Hq + hk * G + g) * D;
#pragma unroll
      for (int s = 0; s < KS; ++s) qf[rb][s] = *reinterpret_cast<const u32x4*>(qrow + (2 * s + h) * 8);
    } else {
#pragma unroll
      for (int s = 0; s < KS; ++s) qf[rb][s] = u32x4{0, 0, 0, 0};
    }
  }

  f32x16 o[RB][DB];
  float m_run[RB], l_run[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_run[rb] = -INFINITY;
    l_run[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[rb][db] = f32x16{};
  }

  int t = t0 + wave;
  TileFrag<D> cur, nxt;
  if (t < t1) {
    const int p0 = page_id(trow, 2 * t, num_pages, flags);
    const int p1 = (t * kTileTokens + kPage < L) ? page_id(trow, 2 * t + 1, num_pages, flags) : -1;
    load_tile<D>(cur, kp, vp, p0, p1, hk, Hkv, lane);
  }
  for (; t < t1; t += kAttnWaves) {
    const int tn = t + kAttnWaves;
    if (tn < t1) {
      const int p0 = page_id(trow, 2 * tn, num_pages, flags);
      const int p1 = (tn * kTileTokens + kPage < L) ? page_id(trow, 2 * tn + 1, num_pages, flags) : -1;
      load_tile<D>(nxt, kp, vp, p0, p1, hk, Hkv, lane);
    }
    const int tok0 = t * kTileTokens;
    const bool partial = tok0 + kTileTokens > L;
    if (partial) {
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int db = 0; db < DB; ++db) cur.v[m][db] = mask_v(cur.v[m][db], tok0 + 16 * m, L, h);
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      f32x16 s = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(cur.k[ks]), as_bf16x8(qf[rb][ks]), s, 0, 0, 0);
      float mx = -INFINITY;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int tok = tok0 + (v >> 2) * 8 + h * 4 + (v & 3);
        float x = s[v] * scale_log2;
        if (partial && tok >= L) x = -INFINITY;
        s[v] = x;
        mx = fmaxf(mx, x);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run[rb], mx);
      const float alpha = exp2f(m_run[rb] - m_new);
      m_run[rb] = m_new;
      float psum = 0.f;
      float pv[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        pv[v] = exp2f(s[v] - m_new);
        psum += pv[v];
      }
      l_run[rb] = l_run[rb] * alpha + psum;
      bf16x8 pb[2];
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[m][e] = (__bf16)pv[8 * m + e];
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        o[rb][db] *= alpha;
#pragma unroll
        for (int m = 0; m < 2; ++m)
          o[rb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(cur.v[m][db]), pb[m], o[rb][db], 0, 0, 0);
      }
    }
    cur = nxt;
  }

  // ---- merge the four waves of the workgroup ----
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
    for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, sm_m[w][c]);
    wscale[rb] = (m_run[rb] == -INFINITY) ? 0.f : exp2f(m_run[rb] - M);
  }
  auto put = [&](int buf, bool add) {
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
          f32x4* dst = reinterpret_cast<f32x4*>(&sm_o[buf][c * OSTR + d0]);
          if (add) *dst += val; else *dst = val;
        }
    }
  };
  if (wave < 2) put(wave, false);
  __syncthreads();
  if (wave >= 2) put(wave - 2, true);
  __syncthreads();

  const size_t base = (size_t(rk) * n_splits + split) * (RB * 32);
  if (threadIdx.x < rows) {
    const int c = threadIdx.x;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, sm_m[w][c]);
    float Lsum = 0.f;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) {
      const float mw = sm_m[w][c];
      if (mw != -INFINITY) Lsum += sm_l[w][c] * exp2f(mw - M);
    }
    ws_ml[base + c] = make_float2(M, Lsum);
  }
  constexpr int V4 = D / 4;
  for (int idx = threadIdx.x; idx < rows * V4; idx += blockDim.x) {
    const int c = idx / V4, d0 = (idx % V4) * 4;
    const f32x4 a = *reinterpret_cast<const f32x4*>(&sm_o[0][c * OSTR + d0]);
    const f32x4 b = *reinterpret_cast<const f32x4*>(&sm_o[1][c * OSTR + d0]);
    *reinterpret_cast<f32x4*>(ws_o + (base + c) * D + d0) = a + b;
  }
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
  int t0, t1;
  split_range(n_tiles, split, n_splits, tps, t0, t1);
  if (t0 >= t1) return;
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
    if (pid < 0) continue;
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

// Merge split partials with the stride's own causal block; normalise; write out.
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_combine(
    const T* __restrict__ q, const T* __restrict__ k_new, const T* __restrict__ v_new,
    const int32_t* __restrict__ ctx_lens, T* __restrict__ out, const float2* __restrict__ ws_ml,
    const float* __restrict__ ws_o, int Qn, int Hq, int Hkv, int G, int rows, int rows_pad,
    int max_pages, int tps, int n_splits, float scale_log2) {
  constexpr int E = D / 64;
  const int rk = blockIdx.x;
  const int hk = rk % Hkv;
  const int r = rk / Hkv;
  int L = ctx_lens[r];
  L = (L < 0) ? 0 : min(L, max_pages * kPage);   // flag already raised by the split kernel
  const int n_tiles = (L + kTileTokens - 1) / kTileTokens;
  int active = 0;
  for (int s = 0; s < n_splits; ++s) {
    int t0, t1;
    split_range(n_tiles, s, n_splits, tps, t0, t1);
    if (t0 < t1) active = s + 1;
  }
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  for (int c = wave; c < rows; c += nwaves) {
    const int g = c / Qn, i = c % Qn;
    const int hq = hk * G + g;
    const T* qrow = q + ((size_t(r) * Qn + i) * Hq + hq) * D;
    float qv[E];
#pragma unroll
    for (int e = 0; e < E; ++e) qv[e] = to_f32<T>(qrow[lane * E + e]);
    // split partials first
    const size_t base0 = size_t(rk) * n_splits * rows_pad;
    float M = -INFINITY;
    for (int s = 0; s < active; ++s) {
      int t0, t1;
      split_range(n_tiles, s, n_splits, tps, t0, t1);
      if (t0 < t1) M = fmaxf(M, ws_ml[base0 + size_t(s) * rows_pad + c].x);
    }
    float Lsum = 0.f;
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.f;
    for (int s = 0; s < active; ++s) {
      int t0, t1;
      split_range(n_tiles, s, n_splits, tps, t0, t1);
      if (t0 >= t1) continue;
      const size_t pr = base0 + size_t(s) * rows_pad + c;
      const float2 ml = ws_ml[pr];
      const float w = exp2f(ml.x - M);
      Lsum += ml.y * w;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = fmaf(ws_o[pr * D + lane * E + e], w, acc[e]);
    }
    // then the stride's own rows j <= i, merged online (base-2 scores)
    for (int j = 0; j <= i; ++j) {
      const T* krow = k_new + ((size_t(r) * Qn + j) * Hkv + hk) * D;
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) part = fmaf(qv[e], to_f32<T>(krow[lane * E + e]), part);
      const float sc = wave_sum(part) * scale_log2;
      const float m_new = fmaxf(M, sc);
      const float alpha = exp2f(M - m_new);
      const float p = exp2f(sc - m_new);
      Lsum = Lsum * alpha + p;
      const T* vrow = v_new + ((size_t(r) * Qn + j) * Hkv + hk) * D;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = fmaf(to_f32<T>(vrow[lane * E + e]), p, acc[e] * alpha);
      M = m_new;
    }
    const float inv = 1.f / Lsum;
    T* orow = out + ((size_t(r) * Qn + i) * Hq + hq) * D;
#pragma unroll
    for (int e = 0; e < E; ++e) orow[lane * E + e] = from_f32<T>(acc[e] * inv);
  }
}

template <int D>
hipError_t launch_d(const isd_shape& s, const AttnPlan& p, const void* q, const void* k_new,
                    const void* v_new, const void* k_pages, const void* v_pages,
                    const int32_t* table, const int32_t* ctx_lens, float scale, void* out, char* ws,
                    const WsLayout& Lw, hipStream_t stream) {
  const float scale_log2 = scale * kLog2e;
  uint32_t* flags = reinterpret_cast<uint32_t*>(ws + Lw.flags);
  float2* ml = reinterpret_cast<float2*>(ws + Lw.attn_ml);
  float* po = reinterpret_cast<float*>(ws + Lw.attn_o);
  const int nwg = s.batch * s.n_kv_heads * p.n_splits;
  if (s.kv_dtype == ISD_BF16) {
    const uint16_t* qq = static_cast<const uint16_t*>(q);
    const uint16_t* kp = static_cast<const uint16_t*>(k_pages);
    const uint16_t* vp = static_cast<const uint16_t*>(v_pages);
    if (p.row_blocks == 1)
      hipLaunchKernelGGL((attn_split_bf16<D, 1>), dim3(nwg), dim3(256), 0, stream, qq, kp, vp, table,
                         ctx_lens, p.q_rows, s.n_q_heads, s.n_kv_heads, p.group, p.rows, s.max_pages,
                         s.num_pages, p.tiles_per_split, p.n_splits, scale_log2, ml, po, flags);
    else
      hipLaunchKernelGGL((attn_split_bf16<D, 2>), dim3(nwg), dim3(256), 0, stream, qq, kp, vp, table,
                         ctx_lens, p.q_rows, s.n_q_heads, s.n_kv_heads, p.group, p.rows, s.max_pages,
                         s.num_pages, p.tiles_per_split, p.n_splits, scale_log2, ml, po, flags);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attn_combine<uint16_t, D>), dim3(s.batch * s.n_kv_heads), dim3(256), 0, stream,
                       qq, static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
                       ctx_lens, static_cast<uint16_t*>(out), ml, po, p.q_rows, s.n_q_heads,
                       s.n_kv_heads, p.group, p.rows, p.rows_pad, s.max_pages, p.tiles_per_split,
                       p.n_splits, scale_log2);
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
