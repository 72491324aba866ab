// Appending accepted CLEAN rows to the KV pages (kv_commit) and the
// workspace header fill.
//
// One workgroup per request: it reads the request's length once, copies
// n_commit rows of k_new / v_new into their page slots (16-byte stores into
// the key layout, element stores into the transposed value layout), and only
// after a barrier writes the new length, so ctx_lens_out may alias
// ctx_lens_in.
#include "device_common.hpp"
#include "isd_internal.hpp"

namespace isd {
namespace {

__device__ __forceinline__ int v_sigma(int s) { return (s & 3) | ((s & 4) << 1) | ((s & 8) >> 1); }

template <typename T>
__global__ __launch_bounds__(256) void kv_commit_kernel(
    const T* __restrict__ k_new, const T* __restrict__ v_new, T* __restrict__ kp, T* __restrict__ vp,
    const int32_t* __restrict__ table, const int32_t* ctx_in, const int32_t* __restrict__ n_commit,
    int32_t* ctx_out, int N, int Hkv, int D, int max_pages, int num_pages, uint32_t* __restrict__ flags) {
  __shared__ int pid_sm[64];
  __shared__ int L_sm, n_sm, nv_sm;
  const int r = blockIdx.x;
  const int Qn = 2 * N - 1;
  const int cap = max_pages * kPage;
  if (threadIdx.x == 0) {
    int L = ctx_in[r];
    int n = n_commit[r];
    if (n < 0 || n > N - 1) {
      raise_flag(flags, ISD_FLAG_COMMIT_RANGE);
      n = n < 0 ? 0 : N - 1;
    }
    if (L < 0 || L > cap) {
      raise_flag(flags, ISD_FLAG_CTX_RANGE);
      L = L < 0 ? 0 : cap;
      n = 0;
    }
    L_sm = L;
    n_sm = n;
  }
  __syncthreads();
  const int L = L_sm, n = n_sm;
  // page of every committed row, resolved in parallel
  if (threadIdx.x < n) {
    const int pos = L + threadIdx.x;
    int pid = -1;
    if (pos < cap) {
      pid = table[size_t(r) * max_pages + pos / kPage];
      if (pid < 0 || pid >= num_pages) pid = -2;
    }
    pid_sm[threadIdx.x] = pid;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int nv = n;
    for (int i = 0; i < n; ++i)
      if (pid_sm[i] < 0) {
        raise_flag(flags, pid_sm[i] == -1 ? ISD_FLAG_COMMIT_RANGE : ISD_FLAG_PAGE_RANGE);
        nv = i;
        break;
      }
    nv_sm = nv;
  }
  __syncthreads();
  const int nv = nv_sm;
  constexpr int EV = 16 / sizeof(T);            // elements per 16-byte vector
  const int kvec = D / EV;                       // 16-byte vectors per key row
  const int kwork = nv * Hkv * kvec;
  for (int w = threadIdx.x; w < kwork; w += blockDim.x) {
    const int c = w % kvec;
    const int hk = (w / kvec) % Hkv;
    const int i = w / (kvec * Hkv);
    const int pid = pid_sm[i];
    const int slot = (L + i) % kPage;
    const int d0 = c * EV;
    const T* src = k_new + ((size_t(r) * Qn + i) * Hkv + hk) * D + d0;
    T* dst = kp + ((size_t(pid) * Hkv + hk) * (D / 8) + d0 / 8) * (kPage * 8) + slot * 8 + (d0 & 7);
    *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
  }
  const int vwork = nv * Hkv * D;
  for (int w = threadIdx.x; w < vwork; w += blockDim.x) {
    const int d = w % D;
    const int hk = (w / D) % Hkv;
    const int i = w / (D * Hkv);
    const int pid = pid_sm[i];
    const int slot = (L + i) % kPage;
    vp[((size_t(pid) * Hkv + hk) * D + d) * kPage + v_sigma(slot)] =
        v_new[((size_t(r) * Qn + i) * Hkv + hk) * D + d];
  }
  __syncthreads();
  if (threadIdx.x == 0) ctx_out[r] = L + nv;
}

__global__ void fill_zero_u32(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// exp of every bf16 bit pattern, float64 (used by the residual sampler)
__global__ void build_exp_table(double* t) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < kExpTableSize) t[b] = exp(double(bf16_bits_to_f32(uint16_t(b))));
}

}  // namespace

hipError_t launch_commit(const isd_shape& s, const void* k_new, const void* v_new, void* k_pages,
                         void* v_pages, const int32_t* table, const int32_t* ctx_in,
                         const int32_t* n_commit, int32_t* ctx_out, uint32_t* flags,
                         hipStream_t stream) {
  if (s.kv_dtype == ISD_BF16)
    hipLaunchKernelGGL((kv_commit_kernel<uint16_t>), dim3(s.batch), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
                       static_cast<uint16_t*>(k_pages), static_cast<uint16_t*>(v_pages), table, ctx_in,
                       n_commit, ctx_out, s.stride_n, s.n_kv_heads, s.head_dim, s.max_pages,
                       s.num_pages, flags);
  else
    hipLaunchKernelGGL((kv_commit_kernel<float>), dim3(s.batch), dim3(256), 0, stream,
                       static_cast<const float*>(k_new), static_cast<const float*>(v_new),
                       static_cast<float*>(k_pages), static_cast<float*>(v_pages), table, ctx_in,
                       n_commit, ctx_out, s.stride_n, s.n_kv_heads, s.head_dim, s.max_pages,
                       s.num_pages, flags);
  return hipGetLastError();
}

hipError_t launch_workspace_init(void* ws, size_t header_bytes, double* exp_table, hipStream_t stream) {
  const int n = int(header_bytes / 4);
  hipLaunchKernelGGL(fill_zero_u32, dim3((n + 255) / 256), dim3(256), 0, stream,
                     static_cast<uint32_t*>(ws), n);
  hipLaunchKernelGGL(build_exp_table, dim3(kExpTableSize / 256), dim3(256), 0, stream, exp_table);
  return hipGetLastError();
}

}  // namespace isd
