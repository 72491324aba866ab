// Per-request bookkeeping of the multi-step decoding loop (isd_loop_advance).
//
// One thread per request applies one forward's results: committed tokens and
// forwards are counted, the stride's proposals are replaced by this forward's
// proposals unless it rejected one (then the next forward re-proposes from
// the corrected prefix, its row N-1 carrying the resampled token), the
// positions argument of the next forward moves with them, and n_commit
// reports the KV rows the forward committed (a re-proposing forward: one,
// its row N-1).  With a normaliser buffer, the MASK rows' (max, sum exp) pairs
// this forward's proposals wrote move to where the next forward's accept test
// reads its q-row normalisers (every forward's: the next forward verifies the
// proposals this one drew, whatever the mode).
#include "device_common.hpp"
#include "isd_internal.hpp"

namespace isd {
namespace {

__global__ __launch_bounds__(256) void loop_advance_kernel(int B, int N, const int32_t* __restrict__ accept_len,
                                                           const int32_t* __restrict__ n_out,
                                                           const int32_t* __restrict__ next_proposals,
                                                           int32_t* __restrict__ n_commit, int32_t* __restrict__ mode,
                                                           int32_t* __restrict__ proposals,
                                                           int32_t* __restrict__ positions,
                                                           int64_t* __restrict__ tokens,
                                                           int64_t* __restrict__ forwards,
                                                           const float2* __restrict__ norms_in,
                                                           float2* __restrict__ norms_out) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= B) return;
  if (norms_in)
    for (int j = 0; j < N; ++j) norms_out[size_t(r) * N + j] = norms_in[size_t(r) * N + j];
  forwards[r] += 1;
  bool take = true;
  if (mode[r] != ISD_LOOP_REPROPOSE) {
    const int a = accept_len[r], k = n_out[r];
    tokens[r] += k;
    if (a == N) {
      positions[r] += N;
    } else {
      mode[r] = ISD_LOOP_REPROPOSE;
      positions[r] += k - N;
      take = false;
    }
  } else {
    n_commit[r] = 1;
    mode[r] = ISD_LOOP_VERIFY;
    positions[r] += N;
  }
  if (take)
    for (int j = 0; j < N; ++j) proposals[size_t(r) * N + j] = next_proposals[size_t(r) * N + j];
}

}  // namespace

hipError_t launch_loop_advance(int B, int N, const int32_t* accept_len, const int32_t* n_out,
                               const int32_t* next_proposals, int32_t* n_commit, int32_t* mode,
                               int32_t* proposals, int32_t* positions, int64_t* tokens, int64_t* forwards,
                               const float* norms_in, float* norms_out, hipStream_t stream) {
  hipLaunchKernelGGL(loop_advance_kernel, dim3((B + 255) / 256), dim3(256), 0, stream, B, N, accept_len, n_out,
                     next_proposals, n_commit, mode, proposals, positions, tokens, forwards,
                     reinterpret_cast<const float2*>(norms_in), reinterpret_cast<float2*>(norms_out));
  return hipGetLastError();
}

}  // namespace isd
