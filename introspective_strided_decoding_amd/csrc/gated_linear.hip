// The projections of an R-ISD layer (isd_gated_linear, and
// isd_gated_linear_group for up to four projections of one input):
//
//   Y_p[m] = X[m] W_p^T + gate[m] * scale * (X[m] A_p^T) B_p^T
//
// A group runs as one projection whose output columns are the projections'
// side by side: each launch below covers every projection of the group.
//
// The adapter's second product rides in the base product's k loop: with
// T[m] = bf16(gate[m] * scale * X[m] A^T) (zero on CLEAN rows), Y is one
// product of [X | T] with [W | B] over d_in + rank columns.
//
//   gl_gemm     (gathering) T_part[p][kc][g][r] = sum over a 256-wide k chunk of
//               X[row(g)] A_p^T: the product kernel below with X rows taken
//               through the gate list, k split into chunks, clearing T on the side
//   gl_scatter  T_p[row(g)] = bf16(scale * sum_kc T_part[p][kc][g]) for gated g
//   gl_gemm     the product, bf16 matrix-core operands, fp32 sums; the rank
//               columns come first, so a row whose T is zero enters the base
//               columns with the same +0 accumulators as the base-only call
//               and leaves bit for bit equal to it
//   gl_reduce   only when k is split: Y = bf16(sum of the split partials in
//               split order)
//
// gl_gemm tiling: a workgroup owns a BM x BN tile of Y^T (BM rows of X, BN rows
// of W), WGM x WGN waves, each (BM/WGM) x (BN/WGN) as 32 x 32 blocks of
// v_mfma_f32_32x32x16_bf16.  k advances 64 at a time through a ring of ST LDS
// stages filled by direct-to-LDS loads (no registers in between), so ST - 1
// blocks are in flight while one is multiplied.
#include "device_common.hpp"
#include "isd_internal.hpp"

namespace isd {
namespace {

constexpr int kBK = 64;          // k per block: one 128-byte line of every bf16 row
constexpr int kRank = 128;

__device__ __forceinline__ bf16x8 as_b8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// Byte offset of 16-byte chunk c of row r in a [rows][64] bf16 LDS tile.  The
// chunk index is XORed with (r & 7) ^ ((r >> 3) & 1): a matrix-core operand
// read (16 consecutive rows, one chunk each) and a staging write (the 8 chunks
// of two rows) both touch every bank once.
__device__ __forceinline__ int swz(int r, int c) { return (r * 8 + (c ^ (r & 7) ^ ((r >> 3) & 1))) * 16; }

// vmcnt(N) alone (lgkmcnt and expcnt left at their maximum), gfx9 encoding.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for LDS reuse without a memory fence: a fence would also
// wait for this wave's loads still streaming into later stages.  The wave's
// own LDS reads are complete first; the asm is a compiler memory barrier too.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

typedef const __attribute__((address_space(1))) void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

// The projections of one launch.  Output tiles are numbered across the group:
// projection p owns tile columns tile_end[p-1] .. tile_end[p]-1 (tile_end[-1] = 0).
struct GlGroup {
  int n;
  int tile_end[kGlMaxProj];
  int d_out[kGlMaxProj];
  const uint16_t* W[kGlMaxProj];    // [d_out][K]
  const uint16_t* Bt[kGlMaxProj];   // [d_out][R]
  const uint16_t* T[kGlMaxProj];    // [M][R]
  uint16_t* Y[kGlMaxProj];          // [M][d_out]
  float* part[kGlMaxProj];          // [splits][M][d_out]
};

// Projection owning global tile column ni, and its members (constant indices
// only, so the group stays in the kernel-argument segment).
struct GlProj {
  int first_tile, N;
  const uint16_t *W, *Bt, *T;
  uint16_t* Y;
  float* part;
};
__device__ __forceinline__ GlProj gl_proj(const GlGroup& g, int ni) {
  GlProj q{0, g.d_out[0], g.W[0], g.Bt[0], g.T[0], g.Y[0], g.part[0]};
#pragma unroll
  for (int i = 1; i < kGlMaxProj; ++i)
    if (i < g.n && ni >= g.tile_end[i - 1])
      q = GlProj{g.tile_end[i - 1], g.d_out[i], g.W[i], g.Bt[i], g.T[i], g.Y[i], g.part[i]};
  return q;
}

template <int BM, int BN, int ST, int WGM, int WGN>
__global__ __launch_bounds__(64 * WGM * WGN) void gl_gemm(
    const uint16_t* __restrict__ X, int K, int R, int M, int m_tiles, int splits, const GlGroup g,
    const int32_t* __restrict__ gather, int x_rows, u32x4* __restrict__ zero16, int n16) {
  constexpr int NW = WGM * WGN;                // waves: WGM along X rows, WGN along W rows
  constexpr int WM = BM / WGM, WN = BN / WGN, FM = WM / 32, FN = WN / 32;
  constexpr int IX = BM / (8 * NW), IW = BN / (8 * NW);    // 1 KB direct-to-LDS loads per wave per block
  static_assert(IX * 8 * NW == BM && IW * 8 * NW == BN && FM * 32 == WM && FN * 32 == WN, "tile shape");
  constexpr int kStageBytes = (BM + BN) * kBK * 2;
  __shared__ __align__(16) uint8_t sm[ST * kStageBytes];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Workgroups are handed to the 8 XCDs round robin by id: renumber so that
  // consecutive logical tiles (the m tiles of one W slice) share an XCD's L2.
  const int G = gridDim.x, b = blockIdx.x;
  const int xcd = b & 7, per = G >> 3, extra = G & 7;
  const int l = xcd * per + min(xcd, extra) + (b >> 3);
  const int mi = l % m_tiles, rest = l / m_tiles;
  const int s = rest % splits, ni = rest / splits;
  const GlProj pj = gl_proj(g, ni);
  const uint16_t* __restrict__ W = pj.W;
  const uint16_t* __restrict__ T = pj.T;
  const uint16_t* __restrict__ Bt = pj.Bt;
  const int N = pj.N;
  const int m0 = mi * BM, n0 = (ni - pj.first_tile) * BN;

  const int kb_base = K / kBK;
  const int b0 = s * kb_base / splits, b1 = (s + 1) * kb_base / splits;
  const int n_ext = s == 0 ? R / kBK : 0;
  const int nkb = n_ext + (b1 - b0);

  // A load instruction moves 8 rows of 128 bytes: lane i lands at byte 16 i of
  // the 1 KB it writes, i.e. row i/8, physical chunk i%8, so it fetches the
  // logical chunk that the swizzle puts there.
  const int lrow = lane >> 3;
  // X row of each of this lane's row chunks, fixed over k: output row m reads X
  // row m, or row gather[m] (0 when out of range; that output is never used)
  int xrow[IX];
#pragma unroll
  for (int q = 0; q < IX; ++q) {
    const int m = min(m0 + wave * (BM / NW) + q * 8 + lrow, M - 1);   // rows past M are computed, never stored
    if (gather) {
      const int gr = gather[m];
      xrow[q] = (gr >= 0 && gr < x_rows) ? gr : 0;
    } else {
      xrow[q] = m;
    }
  }
  auto issue = [&](int j) {
    const bool ext = j < n_ext;
    const uint16_t* xs = ext ? T : X;
    const uint16_t* ws = ext ? Bt : W;
    const int ld = ext ? R : K;
    const int k0 = (ext ? j : b0 + j - n_ext) * kBK;
    uint8_t* st = sm + (j % ST) * kStageBytes;
#pragma unroll
    for (int q = 0; q < IX; ++q) {
      const int r = wave * (BM / NW) + q * 8 + lrow;
      const int c = (lane & 7) ^ (r & 7) ^ ((r >> 3) & 1);
      const int row = ext ? min(m0 + r, M - 1) : xrow[q];
      __builtin_amdgcn_global_load_lds((gptr_t)(xs + size_t(row) * ld + k0 + c * 8),
                                       (lptr_t)(st + (wave * (BM / NW) + q * 8) * 128), 16, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < IW; ++q) {
      const int r = wave * (BN / NW) + q * 8 + lrow;
      const int c = (lane & 7) ^ (r & 7) ^ ((r >> 3) & 1);
      __builtin_amdgcn_global_load_lds((gptr_t)(ws + size_t(n0 + r) * ld + k0 + c * 8),
                                       (lptr_t)(st + BM * 128 + (wave * (BN / NW) + q * 8) * 128), 16, 0, 0);
    }
  };

  const int wm = wave % WGM, wn = wave / WGM;
  const int fr = lane & 31, fh = lane >> 5;
  f32x16 acc[FN][FM];
#pragma unroll
  for (int a = 0; a < FN; ++a)
#pragma unroll
    for (int c = 0; c < FM; ++c) acc[a][c] = f32x16{};
  auto compute = [&](int j) {
    const uint8_t* base = sm + (j % ST) * kStageBytes;
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int c = ks * 2 + fh;
      bf16x8 xf[FM], wf[FN];
#pragma unroll
      for (int f = 0; f < FM; ++f) xf[f] = as_b8(*reinterpret_cast<const u32x4*>(base + swz(wm * WM + f * 32 + fr, c)));
#pragma unroll
      for (int f = 0; f < FN; ++f)
        wf[f] = as_b8(*reinterpret_cast<const u32x4*>(base + BM * 128 + swz(wn * WN + f * 32 + fr, c)));
#pragma unroll
      for (int a = 0; a < FN; ++a)
#pragma unroll
        for (int c2 = 0; c2 < FM; ++c2) acc[a][c2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[a], xf[c2], acc[a][c2], 0, 0, 0);
    }
  };

  // ST-stage ring: blocks j+1 .. j+ST-1 are in flight while block j is
  // multiplied.  Per iteration: wait for this wave's loads of block j, barrier
  // (block j visible to all waves, and every wave is done with block j-1),
  // refill block j-1's stage with block j+ST-1, multiply block j.
#pragma unroll
  for (int j = 0; j < ST - 1; ++j)
    if (j < nkb) issue(j);
  for (int j = 0; j < nkb; ++j) {
    const int newer = min(nkb - 1, j + ST - 2) - j;     // blocks issued after j
    if (newer >= ST - 2) wait_vm<(ST - 2) * (IX + IW)>();
    else if (ST > 3 && newer == 1) wait_vm<(IX + IW)>();
    else wait_vm<0>();
    lds_barrier();
    if (j + ST - 1 < nkb) issue(j + ST - 1);
    compute(j);
  }

  // acc[a][c] holds Y^T block (n, m): this lane's column m = fr, rows
  // n = (v/4)*8 + fh*4 + v%4, so each v/4 group is 4 consecutive outputs of one row.
#pragma unroll
  for (int c = 0; c < FM; ++c) {
    const int m = m0 + wm * WM + c * 32 + fr;
    if (m >= M) continue;
#pragma unroll
    for (int a = 0; a < FN; ++a) {
      const int nb = n0 + wn * WN + a * 32 + fh * 4;
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const int n = nb + v4 * 8;
        const float y0 = acc[a][c][4 * v4], y1 = acc[a][c][4 * v4 + 1];
        const float y2 = acc[a][c][4 * v4 + 2], y3 = acc[a][c][4 * v4 + 3];
        if (splits == 1 && !gather) {     // a gathering product always leaves fp32 partials
          *reinterpret_cast<uint2*>(pj.Y + size_t(m) * N + n) =
              make_uint2(uint32_t(f32_to_bf16_bits(y0)) | (uint32_t(f32_to_bf16_bits(y1)) << 16),
                         uint32_t(f32_to_bf16_bits(y2)) | (uint32_t(f32_to_bf16_bits(y3)) << 16));
        } else {
          *reinterpret_cast<f32x4*>(pj.part + (size_t(s) * M + m) * N + n) = f32x4{y0, y1, y2, y3};
        }
      }
    }
  }
  // optional side job: clear n16 16-byte words (the adapter intermediate T)
  if (zero16)
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += gridDim.x * blockDim.x) zero16[i] = u32x4{0, 0, 0, 0};
}

// One thread per 4 outputs of projection blockIdx.y.
__global__ __launch_bounds__(256) void gl_reduce(const GlGroup g, int M, int splits) {
  const int p = blockIdx.y;
  int c4 = M * (g.d_out[0] / 4);
  const f32x4* __restrict__ part = reinterpret_cast<const f32x4*>(g.part[0]);
  uint2* __restrict__ Y = reinterpret_cast<uint2*>(g.Y[0]);
#pragma unroll
  for (int i = 1; i < kGlMaxProj; ++i)
    if (p == i) {
      c4 = M * (g.d_out[i] / 4);
      part = reinterpret_cast<const f32x4*>(g.part[i]);
      Y = reinterpret_cast<uint2*>(g.Y[i]);
    }
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= c4) return;
  f32x4 v = part[i];
  for (int s = 1; s < splits; ++s) v += part[size_t(s) * c4 + i];
  Y[i] = make_uint2(uint32_t(f32_to_bf16_bits(v[0])) | (uint32_t(f32_to_bf16_bits(v[1])) << 16),
                    uint32_t(f32_to_bf16_bits(v[2])) | (uint32_t(f32_to_bf16_bits(v[3])) << 16));
}

// One thread per (gated row, 4 rank columns) of projection blockIdx.y; part is
// [projection][kchunks][m_pad][128], T is [projection][rows][128].  Every
// thread requests the partials of a batch of chunks (16, or 48 for d_in up to
// 12288) before it reads the gate list or adds any: one memory round trip.
constexpr int kScatterThreads = 64;
template <int kScatterBatch>
__global__ __launch_bounds__(kScatterThreads) void gl_scatter(const float* __restrict__ part, int kchunks, int m_pad,
                                                              const int32_t* __restrict__ mask_rows, int n_mask,
                                                              int rows, float scale, uint16_t* __restrict__ T,
                                                              uint32_t* __restrict__ flags) {
  part += size_t(blockIdx.y) * kchunks * m_pad * kRank;
  T += size_t(blockIdx.y) * rows * kRank;
  const int e = blockIdx.x * kScatterThreads + threadIdx.x;
  const int g = e / (kRank / 4), r = (e % (kRank / 4)) * 4;
  if (g >= n_mask) return;
  // eight running sums, chunk kc going to sum kc % 8, chunks in increasing order
  const f32x4* p = reinterpret_cast<const f32x4*>(part + size_t(g) * kRank + r);
  const size_t stride = size_t(m_pad) * (kRank / 4);
  f32x4 t[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) t[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  int row = 0;
  for (int kc = 0; kc < kchunks; kc += kScatterBatch) {
    f32x4 v[kScatterBatch];
#pragma unroll
    for (int u = 0; u < kScatterBatch; ++u) v[u] = p[min(kc + u, kchunks - 1) * stride];   // in bounds, unconditional
    if (kc == 0) row = mask_rows[g];
#pragma unroll
    for (int u = 0; u < kScatterBatch; ++u)
      if (kc + u < kchunks) t[u % 8] += v[u];
  }
  if (row < 0 || row >= rows) {              // skipped, and flagged once per entry
    if (r == 0 && blockIdx.y == 0) raise_flag(flags, ISD_FLAG_ROW_RANGE);
    return;
  }
  const f32x4 sum = ((t[0] + t[1]) + (t[2] + t[3])) + ((t[4] + t[5]) + (t[6] + t[7]));
  *reinterpret_cast<uint2*>(T + size_t(row) * kRank + r) =
      make_uint2(uint32_t(f32_to_bf16_bits(scale * sum[0])) | (uint32_t(f32_to_bf16_bits(scale * sum[1])) << 16),
                 uint32_t(f32_to_bf16_bits(scale * sum[2])) | (uint32_t(f32_to_bf16_bits(scale * sum[3])) << 16));
}

}  // namespace

// Tile shape, waves, stages and k split per shape, from timings on MI355X of
// every instance over the projections of an 8B-class layer at 224 and 896
// rows.  Loads into the CUs bound these kernels: a variant without the
// products takes as long, and plain 16-byte loads into registers stream the
// same tiles no faster than the direct-to-LDS ones (about 45 GB/s per busy CU
// from L2 either way).  So the plan trades bytes per flop (tile size) against
// keeping all 256 CUs busy (tile count, split).
// A group is planned as one projection of the summed width; a tile width
// only when every member's width is a multiple of it (no tile straddles two).
// Between 256 x 256 and 256 x 192 tiles the cost is rounds of the chip times
// the bytes a tile loads per k block: a 256 x 192 tiling that fills whole
// rounds (512 tiles of an 896-row, 24576-wide group, where 256 x 256 leaves
// 384 = 1.5 rounds) loads less per CU.  Likewise 128 x 192 or 128 x 256 tiles
// where they fit one round and 128 x 128 tiles would not (an 896-row q/k/v
// group: 168 tiles of 128 x 256 against 336 of 128 x 128).
GlPlan gl_plan(int32_t rows, int32_t d_in, int32_t d_out, bool all256, bool all192) {
  GlPlan p;
  const int kb = d_in / kBK;
  const long t128 = long((rows + 127) / 128) * (d_out / 128);
  const long t256 = all256 ? long((rows + 255) / 256) * (d_out / 256) : 0;
  const long t192 = all192 ? long((rows + 255) / 256) * (d_out / 192) : 0;
  const long t128x192 = all192 ? long((rows + 127) / 128) * (d_out / 192) : 0;
  const long t128x256 = all256 ? long((rows + 127) / 128) * (d_out / 256) : 0;
  auto one_round = [](long tiles) { return tiles > 0 && tiles <= 256; };
  auto cost = [](long tiles, int bn) { return (tiles + 255) / 256 * (256 + bn); };
  auto split_to = [&](long tiles) {
    while (tiles * p.splits < 256 && kb / (2 * p.splits) >= 8) p.splits *= 2;
  };
  if (rows >= 512 && std::max(t256, t192) >= 160) {
    p.bm = 256;                        // 8 waves: of 128 x 64 (256 x 256) or 64 x 96 (256 x 192)
    p.bn = (t192 >= 160 && (t256 < 160 || cost(t192, 192) < cost(t256, 256))) ? 192 : 256;
    p.stages = 2;
    p.waves = 8;
  } else if (t128 > 256 && (one_round(t128x192) || one_round(t128x256))) {
    // one round of 128 x 192 tiles (4 waves of 64 x 96), else of 128 x 256 tiles
    // (8 waves of 64 x 64), instead of more than one round of 128 x 128
    p.bn = one_round(t128x192) ? 192 : 256;
    p.waves = p.bn == 192 ? 4 : 8;
    p.stages = 3;
  } else if (t128 >= 384) {
    p.stages = 2;                      // two workgroups per CU
  } else if (t128 >= 160) {
    if (d_in >= 8192) {
      p.stages = 2;
      p.splits = 2;
    } else {
      p.waves = 8;                     // 8 waves of 64 x 32
    }
  } else if (d_out <= 2048) {
    p.bm = p.bn = 64;
    split_to(long((rows + 63) / 64) * (d_out / 64));
  } else {
    split_to(t128);
  }
  return p;
}

GlLayout gl_layout(int32_t n_proj, int32_t rows, int32_t d_in, const int32_t* d_out, int32_t rank,
                   int32_t n_mask) {
  GlLayout L;
  long total = 0;
  bool all256 = true, all192 = true;
  for (int p = 0; p < n_proj; ++p) {
    total += d_out[p];
    all256 = all256 && d_out[p] % 256 == 0;
    all192 = all192 && d_out[p] % 192 == 0;
  }
  L.plan = gl_plan(rows, d_in, int32_t(total), all256, all192);
  size_t off = kHeaderBytes;
  if (rank > 0) {
    L.t = off;
    off += (size_t(n_proj) * rows * rank * 2 + 255) / 256 * 256;
    L.down = off;
    off += size_t(n_proj) * size_t(d_in / 256) * size_t(n_mask) * rank * 4;
    off = (off + 255) / 256 * 256;
  }
  if (L.plan.splits > 1) {
    L.split = off;
    off += size_t(L.plan.splits) * rows * size_t(total) * 4;
  }
  L.total = (off + 255) / 256 * 256;
  return L;
}

hipError_t launch_gated_linear(int32_t n_proj, int32_t rows, int32_t d_in, const int32_t* d_out, int32_t rank,
                               const void* X, const void* const* W_t, const void* const* A_t,
                               const void* const* B_t, const int32_t* mask_rows, int32_t n_mask, float scale,
                               void* const* Y, char* ws, hipStream_t stream) {
  if (n_mask == 0) rank = 0;     // no gated row: the base projections, bit for bit
  const GlLayout L = gl_layout(n_proj, rows, d_in, d_out, rank, n_mask);
  const GlPlan& pl = L.plan;
  GlGroup g{};
  g.n = n_proj;
  int max_d = 0;
  for (int p = 0; p < n_proj; ++p) {
    g.d_out[p] = d_out[p];
    g.W[p] = static_cast<const uint16_t*>(W_t[p]);
    g.Y[p] = static_cast<uint16_t*>(Y[p]);
    max_d = d_out[p] > max_d ? d_out[p] : max_d;
  }
  if (rank > 0) {
    uint16_t* t = reinterpret_cast<uint16_t*>(ws + L.t);
    float* down = reinterpret_cast<float*>(ws + L.down);
    // the adapters' down-projection of the gated rows, every adapter of the group in
    // one launch: 64 x 64 tiles of [gathered X rows] x [A_p rows], k split into
    // 256-wide chunks whose partials gl_scatter sums; T is cleared on the side
    const int kchunks = d_in / 256;
    GlGroup gd{};
    gd.n = n_proj;
    for (int p = 0; p < n_proj; ++p) {
      gd.d_out[p] = kRank;
      gd.tile_end[p] = (p + 1) * (kRank / 64);
      gd.W[p] = static_cast<const uint16_t*>(A_t[p]);
      gd.part[p] = down + size_t(p) * kchunks * n_mask * kRank;
    }
    const int mtd = (n_mask + 63) / 64;
    hipLaunchKernelGGL((gl_gemm<64, 64, 4, 2, 2>), dim3(mtd * n_proj * (kRank / 64) * kchunks), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(X), d_in, 0, n_mask, mtd, kchunks, gd, mask_rows, rows,
                       reinterpret_cast<u32x4*>(t), int(size_t(n_proj) * rows * rank * 2 / 16));
    const dim3 sgrid((n_mask * (kRank / 4) + kScatterThreads - 1) / kScatterThreads, n_proj);
    if (kchunks <= 16)
      hipLaunchKernelGGL(gl_scatter<16>, sgrid, dim3(kScatterThreads), 0, stream, down, kchunks, n_mask, mask_rows,
                         n_mask, rows, scale, t, reinterpret_cast<uint32_t*>(ws));
    else
      hipLaunchKernelGGL(gl_scatter<48>, sgrid, dim3(kScatterThreads), 0, stream, down, kchunks, n_mask, mask_rows,
                         n_mask, rows, scale, t, reinterpret_cast<uint32_t*>(ws));
    for (int p = 0; p < n_proj; ++p) {
      g.T[p] = t + size_t(p) * rows * kRank;
      g.Bt[p] = static_cast<const uint16_t*>(B_t[p]);
    }
  }
  if (pl.splits > 1) {
    float* part = reinterpret_cast<float*>(ws + L.split);
    size_t off = 0;
    for (int p = 0; p < n_proj; ++p) {
      g.part[p] = part + off;
      off += size_t(pl.splits) * rows * d_out[p];
    }
  }
  auto tiles = [&](int bn) {
    int end = 0;
    for (int p = 0; p < n_proj; ++p) g.tile_end[p] = end += d_out[p] / bn;
    return end;
  };
  const int R = rank > 0 ? kRank : 0;
  const auto* x = static_cast<const uint16_t*>(X);
  if (pl.bm == 256) {
    const int mt = (rows + 255) / 256;
    if (pl.bn == 192)
      hipLaunchKernelGGL((gl_gemm<256, 192, 2, 4, 2>), dim3(mt * tiles(192) * pl.splits), dim3(512), 0, stream, x,
                         d_in, R, rows, mt, pl.splits, g, nullptr, 0, nullptr, 0);
    else
      hipLaunchKernelGGL((gl_gemm<256, 256, 2, 2, 4>), dim3(mt * tiles(256) * pl.splits), dim3(512), 0, stream, x,
                         d_in, R, rows, mt, pl.splits, g, nullptr, 0, nullptr, 0);
  } else if (pl.bm == 128) {
    const int mt = (rows + 127) / 128;
    const dim3 grid(mt * tiles(pl.bn) * pl.splits);
    if (pl.bn == 192)
      hipLaunchKernelGGL((gl_gemm<128, 192, 3, 2, 2>), grid, dim3(256), 0, stream, x, d_in, R, rows, mt, pl.splits,
                         g, nullptr, 0, nullptr, 0);
    else if (pl.bn == 256)
      hipLaunchKernelGGL((gl_gemm<128, 256, 3, 2, 4>), grid, dim3(512), 0, stream, x, d_in, R, rows, mt, pl.splits,
                         g, nullptr, 0, nullptr, 0);
    else if (pl.stages == 2)
      hipLaunchKernelGGL((gl_gemm<128, 128, 2, 2, 2>), grid, dim3(256), 0, stream, x, d_in, R, rows, mt, pl.splits,
                         g, nullptr, 0, nullptr, 0);
    else if (pl.waves == 8)
      hipLaunchKernelGGL((gl_gemm<128, 128, 4, 2, 4>), grid, dim3(512), 0, stream, x, d_in, R, rows, mt, pl.splits,
                         g, nullptr, 0, nullptr, 0);
    else
      hipLaunchKernelGGL((gl_gemm<128, 128, 4, 2, 2>), grid, dim3(256), 0, stream, x, d_in, R, rows, mt, pl.splits,
                         g, nullptr, 0, nullptr, 0);
  } else {
    const int mt = (rows + 63) / 64;
    hipLaunchKernelGGL((gl_gemm<64, 64, 4, 2, 2>), dim3(mt * tiles(64) * pl.splits), dim3(256), 0, stream, x, d_in,
                       R, rows, mt, pl.splits, g, nullptr, 0, nullptr, 0);
  }
  if (pl.splits > 1) {
    const int count4 = rows * (max_d / 4);
    hipLaunchKernelGGL(gl_reduce, dim3((count4 + 255) / 256, n_proj), dim3(256), 0, stream, g, rows, pl.splits);
  }
  return hipGetLastError();
}

}  // namespace isd
