// Gated low-rank delta of R-ISD (isd_lora_delta): Y[m] += scale * (X[m] A) B
// for the gated (MASK) rows m only.
//
// Weights come in the layouts a linear layer stores them: the down
// projection as A_t[rank][d_in], the up projection as B_t[d_out][rank], so
// every matrix-core operand is 16 contiguous bytes of one row.
//
//   lora_down    T_part[kc][m][n] = sum_{k in chunk kc} X[row(m)][k] A_t[n][k]
//                workgroup = 32 gated rows x 128 ranks (4 waves x 32 ranks),
//                one 256-wide k chunk; v_mfma_f32_32x32x16_bf16, fp32 sums.
//   lora_reduce  T = sum_kc T_part, split into bf16 T_hi + T_lo (T_lo holds
//                the rounding remainder, so T_hi + T_lo carries ~16 bits).
//   lora_up      C^T[o][m] = sum_n B_t[o][n] (T_hi + T_lo)[m][n]; workgroup =
//                32 gated rows x 128 outputs; Y[row(m)][o] += scale * C in a
//                bf16 read-modify-write of the gated rows only.
#include "device_common.hpp"
#include "isd_internal.hpp"

namespace isd {
namespace {

constexpr int kLoraRank = 128;
constexpr int kKChunk = 256;
constexpr int kOBlock = 128;

__device__ __forceinline__ bf16x8 as_b8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

__device__ __forceinline__ int gated_row(const int32_t* __restrict__ mask_rows, int m, int n_mask,
                                         int rows, uint32_t* flags, bool report) {
  if (m >= n_mask) return -1;
  const int row = mask_rows[m];
  if (row < 0 || row >= rows) {
    if (report) raise_flag(flags, ISD_FLAG_ROW_RANGE);
    return -1;
  }
  return row;
}

__global__ __launch_bounds__(256) void lora_down(const uint16_t* __restrict__ X, const uint16_t* __restrict__ At,
                                                 const int32_t* __restrict__ mask_rows, int n_mask, int rows,
                                                 int d_in, int m_pad, float* __restrict__ part,
                                                 uint32_t* __restrict__ flags) {
  const int kc = blockIdx.x, mb = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, col = lane & 31;
  const int n = wave * 32 + col;
  const uint16_t* arow = At + size_t(n) * d_in + kc * kKChunk + h * 8;
  // the adapter rows first: they do not wait for the gated row's index
  u32x4 a[kKChunk / 16], b[kKChunk / 16];
#pragma unroll
  for (int s = 0; s < kKChunk / 16; ++s) a[s] = *reinterpret_cast<const u32x4*>(arow + s * 16);
  const int m = mb * 32 + col;
  const int row = gated_row(mask_rows, m, n_mask, rows, flags, wave == 0 && h == 0 && kc == 0);
  const uint16_t* xrow = X + size_t(row < 0 ? 0 : row) * d_in + kc * kKChunk + h * 8;
  // unconditional loads (a row outside the gate reads row 0 and is zeroed after), so all
  // of them are in flight at once
#pragma unroll
  for (int s = 0; s < kKChunk / 16; ++s) b[s] = *reinterpret_cast<const u32x4*>(xrow + s * 16);
  if (row < 0) {
#pragma unroll
    for (int s = 0; s < kKChunk / 16; ++s) b[s] = u32x4{0, 0, 0, 0};
  }
  f32x16 acc = f32x16{};
#pragma unroll
  for (int s = 0; s < kKChunk / 16; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_b8(a[s]), as_b8(b[s]), acc, 0, 0, 0);
  // C[n][m]: this lane holds m, and n = wave*32 + (v/4)*8 + h*4 + v%4
  float* dst = part + (size_t(kc) * m_pad + m) * kLoraRank + wave * 32 + h * 4;
#pragma unroll
  for (int v4 = 0; v4 < 4; ++v4)
    *reinterpret_cast<f32x4*>(dst + v4 * 8) = f32x4{acc[4 * v4], acc[4 * v4 + 1], acc[4 * v4 + 2], acc[4 * v4 + 3]};
}

// Chunk partials are requested 16 at a time (indices clamped into range, so every
// load is unconditional and in flight together) and added in chunk order.
constexpr int kReduceBatch = 16;
__global__ __launch_bounds__(256) void lora_reduce(const float* __restrict__ part, int kchunks, int count,
                                                   uint16_t* __restrict__ t_hi, uint16_t* __restrict__ t_lo) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= count) return;
  float t = 0.f;
  for (int k0 = 0; k0 < kchunks; k0 += kReduceBatch) {
    float v[kReduceBatch];
#pragma unroll
    for (int u = 0; u < kReduceBatch; ++u) v[u] = part[size_t(min(k0 + u, kchunks - 1)) * count + e];
#pragma unroll
    for (int u = 0; u < kReduceBatch; ++u)
      if (k0 + u < kchunks) t += v[u];
  }
  const uint16_t hi = f32_to_bf16_bits(t);
  t_hi[e] = hi;
  t_lo[e] = f32_to_bf16_bits(t - bf16_bits_to_f32(hi));
}

__global__ __launch_bounds__(256) void lora_up(const uint16_t* __restrict__ Bt, const uint16_t* __restrict__ t_hi,
                                               const uint16_t* __restrict__ t_lo,
                                               const int32_t* __restrict__ mask_rows, int n_mask, int rows,
                                               int d_out, float scale, uint16_t* __restrict__ Y) {
  const int ob = blockIdx.x, mb = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, col = lane & 31;
  const int m = mb * 32 + col;
  const int o = ob * kOBlock + wave * 32 + col;
  const uint16_t* brow = Bt + size_t(o) * kLoraRank + h * 8;
  const uint16_t* hrow = t_hi + size_t(m) * kLoraRank + h * 8;
  const uint16_t* lrow = t_lo + size_t(m) * kLoraRank + h * 8;
  // the gate list, the operands and then the gated row's outputs are all requested
  // before the products, so the read of Y overlaps them (a lane outside the gate
  // reads row 0 and stores nothing)
  const int gr = mask_rows[min(m, n_mask - 1)];                  // unconditional: in flight with the rest
  // every operand load is issued before the first product
  constexpr int KS = kLoraRank / 16;
  u32x4 bv[KS], hv[KS], lv[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    bv[s] = *reinterpret_cast<const u32x4*>(brow + s * 16);
    hv[s] = *reinterpret_cast<const u32x4*>(hrow + s * 16);
    lv[s] = *reinterpret_cast<const u32x4*>(lrow + s * 16);
  }
  __builtin_amdgcn_sched_barrier(0);
  const int row = (m < n_mask && gr >= 0 && gr < rows) ? gr : -1;
  // C^T[o][m]: this lane holds m, and o = ob*128 + wave*32 + (v/4)*8 + h*4 + v%4
  uint16_t* yrow = Y + size_t(row < 0 ? 0 : row) * d_out + ob * kOBlock + wave * 32 + h * 4;
  uint2 yv[4];
#pragma unroll
  for (int v4 = 0; v4 < 4; ++v4) yv[v4] = *reinterpret_cast<const uint2*>(yrow + v4 * 8);
  __builtin_amdgcn_sched_barrier(0);   // keep the loads above ahead of every product
  f32x16 acc = f32x16{};
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_b8(bv[s]), as_b8(hv[s]), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_b8(bv[s]), as_b8(lv[s]), acc, 0, 0, 0);
  }
  // the sums are formed on every lane (so the reads of Y stay where they were
  // issued) and stored only for gated rows
  uint2 out[4];
#pragma unroll
  for (int v4 = 0; v4 < 4; ++v4) {
    const uint2 y = yv[v4];
    const float y0 = bf16_lo(y.x) + scale * acc[4 * v4 + 0];
    const float y1 = bf16_hi(y.x) + scale * acc[4 * v4 + 1];
    const float y2 = bf16_lo(y.y) + scale * acc[4 * v4 + 2];
    const float y3 = bf16_hi(y.y) + scale * acc[4 * v4 + 3];
    out[v4] = make_uint2(uint32_t(f32_to_bf16_bits(y0)) | (uint32_t(f32_to_bf16_bits(y1)) << 16),
                         uint32_t(f32_to_bf16_bits(y2)) | (uint32_t(f32_to_bf16_bits(y3)) << 16));
  }
  if (row < 0) return;
#pragma unroll
  for (int v4 = 0; v4 < 4; ++v4) *reinterpret_cast<uint2*>(yrow + v4 * 8) = out[v4];
}

}  // namespace

LoraLayout lora_layout(int32_t n_mask, int32_t d_in, int32_t rank) {
  LoraLayout L;
  const size_t m_pad = size_t((n_mask + 31) / 32) * 32;
  const size_t kchunks = size_t(d_in / kKChunk);
  size_t off = kHeaderBytes;
  L.part = off;
  off += kchunks * m_pad * rank * 4;
  off = (off + 255) / 256 * 256;
  L.t_hi = off;
  off += m_pad * rank * 2;
  off = (off + 255) / 256 * 256;
  L.t_lo = off;
  off += m_pad * rank * 2;
  L.total = (off + 255) / 256 * 256;
  return L;
}

hipError_t launch_lora(int32_t rows, int32_t d_in, int32_t d_out, int32_t rank, const void* X,
                       const void* A, const void* Bm, const int32_t* mask_rows, int32_t n_mask,
                       float scale, void* Y, char* ws, hipStream_t stream) {
  if (n_mask == 0) return hipSuccess;
  const LoraLayout L = lora_layout(n_mask, d_in, rank);
  const int m_blocks = (n_mask + 31) / 32;
  const int m_pad = m_blocks * 32;
  const int kchunks = d_in / kKChunk;
  float* part = reinterpret_cast<float*>(ws + L.part);
  uint16_t* t_hi = reinterpret_cast<uint16_t*>(ws + L.t_hi);
  uint16_t* t_lo = reinterpret_cast<uint16_t*>(ws + L.t_lo);
  uint32_t* flags = reinterpret_cast<uint32_t*>(ws);
  hipLaunchKernelGGL(lora_down, dim3(kchunks, m_blocks), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(X), static_cast<const uint16_t*>(A), mask_rows, n_mask, rows,
                     d_in, m_pad, part, flags);
  const int count = m_pad * rank;
  hipLaunchKernelGGL(lora_reduce, dim3((count + 255) / 256), dim3(256), 0, stream, part, kchunks, count, t_hi, t_lo);
  hipLaunchKernelGGL(lora_up, dim3(d_out / kOBlock, m_blocks), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(Bm), t_hi, t_lo, mask_rows, n_mask, rows, d_out, scale,
                     static_cast<uint16_t*>(Y));
  return hipGetLastError();
}

}  // namespace isd
