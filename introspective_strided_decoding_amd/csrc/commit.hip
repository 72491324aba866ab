// Appending accepted stride rows to the KV pages (kv_commit) and the
// workspace header fill (isd_workspace_init).  The commit itself lives in
// commit_row.hpp: one workgroup per request.
#include "commit_row.hpp"

namespace isd {
namespace {

template <typename T>
__global__ __launch_bounds__(kCommitThreads) void kv_commit_kernel(CommitArgs c) {
  commit_request<T>(c, blockIdx.x);
}

__global__ void fill_zero_u32(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

}  // namespace

CommitArgs commit_args(const isd_shape& s, const void* k_new, const void* v_new, void* k_pages,
                       void* v_pages, const int32_t* table, const int32_t* ctx_in,
                       const int32_t* n_commit, int32_t* ctx_out, uint32_t* flags,
                       const int32_t* loop_mode) {
  CommitArgs c;
  c.k_new = k_new;
  c.v_new = v_new;
  c.k_pages = k_pages;
  c.v_pages = v_pages;
  c.table = table;
  c.ctx_in = ctx_in;
  c.n_commit = n_commit;
  c.ctx_out = ctx_out;
  c.flags = flags;
  c.loop_mode = loop_mode;
  c.N = s.stride_n;
  c.Hkv = s.n_kv_heads;
  c.D = s.head_dim;
  c.max_pages = s.max_pages;
  c.num_pages = s.num_pages;
  c.kv_bf16 = (s.kv_dtype == ISD_BF16) ? 1 : 0;
  return c;
}

hipError_t launch_commit(const isd_shape& s, const CommitArgs& c, hipStream_t stream) {
  const dim3 grid(s.batch);
  if (c.kv_bf16)
    hipLaunchKernelGGL((kv_commit_kernel<uint16_t>), grid, dim3(kCommitThreads), 0, stream, c);
  else
    hipLaunchKernelGGL((kv_commit_kernel<float>), grid, dim3(kCommitThreads), 0, stream, c);
  return hipGetLastError();
}

hipError_t launch_workspace_init(void* ws, size_t header_bytes, hipStream_t stream) {
  const int n = int(header_bytes / 4);
  hipLaunchKernelGGL(fill_zero_u32, dim3((n + 255) / 256), dim3(256), 0, stream,
                     static_cast<uint32_t*>(ws), n);
  return hipGetLastError();
}

}  // namespace isd
