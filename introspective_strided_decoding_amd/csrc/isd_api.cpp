// C ABI of libisd.so: argument validation, planning, workspace layout and
// dispatch to the HIP kernels.  Everything here runs on the host and returns
// before any launch when an argument is invalid.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "isd.h"
#include "isd_internal.hpp"

// Workgroups the attention aims for: one per CU on 256 CUs (each is 8 waves
// with one 32-column block, or 4 waves with two).
#ifndef ISD_ATTN_TARGET_WGS
#define ISD_ATTN_TARGET_WGS 256
#endif

namespace isd {
namespace {

thread_local char g_last_error[256] = "";

isd_status hip_fail(hipError_t e, const char* where) {
  std::snprintf(g_last_error, sizeof(g_last_error), "%s: %s", where, hipGetErrorString(e));
  return ISD_ERR_HIP;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }   // NULL passes

int ceil_div(long long a, long long b) { return int((a + b - 1) / b); }

isd_status check_dtype(int32_t d) {
  return (d == ISD_F32 || d == ISD_BF16) ? ISD_OK : ISD_ERR_DTYPE;
}

// Checks shared by every step entry point.
isd_status check_shape(const isd_shape* s) {
  if (!s) return ISD_ERR_NULL;
  if (check_dtype(s->kv_dtype) != ISD_OK || check_dtype(s->logit_dtype) != ISD_OK) return ISD_ERR_DTYPE;
  if (s->batch < 1 || s->stride_n < 2 || s->n_q_heads < 1 || s->n_kv_heads < 1 ||
      s->max_pages < 1 || s->num_pages < 1 || s->vocab < 1 || s->max_ctx < 0)
    return ISD_ERR_SHAPE;
  if (s->n_q_heads % s->n_kv_heads) return ISD_ERR_SHAPE;
  if (s->page_size != kPage) return ISD_ERR_UNSUPPORTED;
  if (s->head_dim != 64 && s->head_dim != 128) return ISD_ERR_UNSUPPORTED;
  // the stride's own block is one 32-token attention tile: Q = 2N - 1 <= 31
  if (s->stride_n > 16 || s->batch > 65535) return ISD_ERR_UNSUPPORTED;
  const long long rows = (long long)(s->n_q_heads / s->n_kv_heads) * (2 * s->stride_n - 1);
  if (rows > 64) return ISD_ERR_UNSUPPORTED;
  if ((long long)s->max_pages * kPage > (1LL << 30)) return ISD_ERR_SHAPE;
  return ISD_OK;
}

isd_status check_ws(const isd_shape* s, const void* ws, size_t bytes) {
  if (!ws) return ISD_ERR_NULL;
  if (!aligned16(ws)) return ISD_ERR_ALIGNMENT;
  if (bytes < ws_layout(*s).total) return ISD_ERR_WORKSPACE;
  return ISD_OK;
}

// ---- the scratch of isd_accept_commit_noalloc ----
// One array per device, owned by the library for the life of the process.
// Its header is cleared once per device at set-up; the partials follow, each
// written before it is read within a call, so nothing else needs clearing.  In
// host code `scratch` names a host-side stand-in: the device address comes from
// hipGetSymbolAddress, per device.
constexpr size_t kScratchBytes = size_t(16) << 20;
constexpr size_t kScratchZeroBytes = kHeaderBytes;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
char* g_scratch[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// The current device's scratch address; the first call on a device resolves it
// and clears the counter region on `stream`.
hipError_t device_scratch(char** out, hipStream_t stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [&] {
    void* p = nullptr;
    hipError_t r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (r == hipSuccess) r = launch_workspace_init(p, kScratchZeroBytes, stream);
    g_scratch[dev] = (r == hipSuccess) ? static_cast<char*>(p) : nullptr;
    g_scratch_err[dev] = r;
  });
  if (!g_scratch[dev]) return g_scratch_err[dev] != hipSuccess ? g_scratch_err[dev] : hipErrorNotInitialized;
  *out = g_scratch[dev];
  return hipSuccess;
}

// Regions of isd_accept + commit inside the scratch: the header, then the
// partials.  The flag word is the caller's.
WsLayout scratch_layout(const isd_shape& s) {
  WsLayout L;
  const AcceptPlan c = plan_accept(s);
  L.zero_end = kScratchZeroBytes;
  size_t off = kScratchZeroBytes;
  L.lse = off;
  off = align_up(off + (size_t)c.rows * c.shards * 8, 256);
  L.jobs = off;
  off = align_up(off + (size_t)s.batch * sizeof(ReqState), 256);
  L.gath = off;
  off = align_up(off + (size_t)c.rows * 4, 256);
  L.unif = off;
  off = align_up(off + (size_t)s.batch * (s.stride_n - 1) * 16, 256);
  L.resid = off;
  off = align_up(off + (size_t)s.batch * c.r_shards * sizeof(ResidShard), 256);
  L.total = off;
  return L;
}

// Checks of isd_accept_commit's arguments other than the workspace.
isd_status check_accept_commit(const isd_shape* shape, const void* p_logits, const void* q_logits,
                               const int32_t* proposals, const int32_t* req_ids, const int32_t* positions,
                               const float* q_norms, int32_t* accept_len, int32_t* out_tokens, int32_t* n_out,
                               int32_t* n_commit, float* logp_sel, float* logq_sel, const void* k_new,
                               const void* v_new, void* k_pages, void* v_pages, const int32_t* page_table,
                               const int32_t* ctx_lens_in, int32_t* ctx_lens_out) {
  isd_status st = check_shape(shape);
  if (st != ISD_OK) return st;
  if (!p_logits || !q_logits || !proposals || !req_ids || !positions || !accept_len || !out_tokens ||
      !n_out || !n_commit || !logp_sel || !logq_sel || !k_new || !v_new || !k_pages || !v_pages ||
      !page_table || !ctx_lens_in || !ctx_lens_out)
    return ISD_ERR_NULL;
  if (!aligned16(p_logits) || !aligned16(q_logits) || !aligned16(k_new) || !aligned16(v_new) ||
      !aligned16(k_pages) || !aligned8(q_norms))
    return ISD_ERR_ALIGNMENT;
  if (shape->batch > 65535) return ISD_ERR_UNSUPPORTED;
  if (shape->vocab > 2048 * 1024) return ISD_ERR_UNSUPPORTED;
  return ISD_OK;
}

// isd_accept_commit on validated arguments, its partials at `ws` laid out by `L`.
hipError_t run_accept_commit(const isd_shape& s, const void* p_logits, const void* q_logits,
                             const int32_t* proposals, const int32_t* req_ids, const int32_t* positions,
                             uint64_t seed_lo, uint64_t seed_hi, uint32_t step, const int64_t* step_per_request,
                             const float* q_norms, int32_t* accept_len, int32_t* out_tokens, int32_t* n_out,
                             int32_t* n_commit, float* logp_sel, float* logq_sel, const void* k_new,
                             const void* v_new, void* k_pages, void* v_pages, const int32_t* page_table,
                             const int32_t* ctx_lens_in, int32_t* ctx_lens_out, const int32_t* loop_mode,
                             char* ws, const WsLayout& L, uint32_t* flags, hipStream_t stream) {
  const AcceptPlan p = plan_accept(s);
  const CommitArgs c = commit_args(s, k_new, v_new, k_pages, v_pages, page_table, ctx_lens_in, n_commit,
                                   ctx_lens_out, flags, loop_mode);
  return launch_accept(s, p, p_logits, q_logits, proposals, req_ids, positions, seed_lo, seed_hi, step,
                       step_per_request, q_norms, accept_len, out_tokens, n_out, n_commit, logp_sel, logq_sel, ws,
                       L, flags, &c, stream);
}

}  // namespace

int device_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int cus = cached[dev].load(std::memory_order_relaxed);
  if (cus <= 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    cached[dev].store(cus, std::memory_order_relaxed);
  }
  return cus;
}

AttnPlan plan_attention(const isd_shape& s) {
  AttnPlan p{};
  p.q_rows = 2 * s.stride_n - 1;
  p.group = s.n_q_heads / s.n_kv_heads;
  p.rows = p.group * p.q_rows;
  p.rows_pad = ceil_div(p.rows, 32) * 32;
  p.row_blocks = p.rows_pad / 32;
  const long long cap = (long long)s.max_pages * kPage;
  const long long hint = (s.max_ctx > 0) ? std::min<long long>(s.max_ctx, cap) : cap;
  p.tiles_max = std::max(1, ceil_div(hint, kTileTokens));
  // Splits per (request, KV head): enough workgroups for one per CU, but no
  // more (each extra split costs a partial and a merge).
  const long long pairs = (long long)s.batch * s.n_kv_heads;
  const int target = ISD_ATTN_TARGET_WGS;
  int splits = std::max(1, ceil_div(target, pairs));
  // bf16 workgroups stage Q and fill a load pipeline first, so a split gets at
  // least 8 tiles; the fp32 path (one wave per query column, tokens one at a
  // time) splits down to single tiles.
  const int min_tps = (s.kv_dtype == ISD_BF16) ? 8 : 1;
  p.tiles_per_split = std::max(min_tps, ceil_div(p.tiles_max, splits));
  // the final merge keeps one weight per split in LDS: at most 64 splits
  p.tiles_per_split = std::max(p.tiles_per_split, ceil_div(p.tiles_max, 64));
  p.n_splits = std::max(1, ceil_div(p.tiles_max, p.tiles_per_split));
  return p;
}

AcceptPlan plan_accept(const isd_shape& s) {
  AcceptPlan p{};
  p.rows = 2 * s.batch * (s.stride_n - 1);
  const int V = s.vocab;
  // At most 2048 workgroups in the normaliser pass (what 256 CUs hold at once
  // at its 8 waves per SIMD, so no workgroup waits for a slot), at least 2048
  // entries each, and at most 256 threads x 8 vectors of 16 bytes per shard.
  const int vec = (s.logit_dtype == ISD_BF16) ? 8 : 4;
  int shards = std::max(1, 2048 / p.rows);
  shards = std::min(shards, std::max(1, V / 2048));
  shards = std::max(shards, ceil_div(V, 256 * 8 * vec));
  p.shard_len = ceil_div(ceil_div(V, shards), 8) * 8;
  p.shards = ceil_div(V, p.shard_len);
  // the fp64 residual works on 2048-element shards (256 threads x 8 entries)
  p.r_shard_len = 2048;
  p.r_shards = ceil_div(V, p.r_shard_len);
  // The decision inside the residual pass saves a launch and the pass's dependent
  // read of the job, at the price of every pass workgroup repeating its
  // request's decision (~2 us): measured ahead where the pass grid stays
  // within four workgroups per CU (b8_ctx2k, 600 workgroups: +4 %), behind
  // where it takes more than one resident round (c32_ctx4k -1 %, c128_lora -3.6 %).
  p.fuse_decision = (size_t)s.batch * p.r_shards <= (size_t)4 * device_cus() ? 1 : 0;
  return p;
}

WsLayout ws_layout(const isd_shape& s) {
  WsLayout L;
  const AttnPlan a = plan_attention(s);
  const AcceptPlan c = plan_accept(s);
  size_t off = kHeaderBytes;
  L.attn_cnt = off;
  off = align_up(off + (size_t)s.batch * s.n_kv_heads * 4, 256);
  L.zero_end = off;
  const size_t partial_rows = (size_t)s.batch * s.n_kv_heads * a.n_splits * a.rows_pad;
  L.attn_ml = off;
  off = align_up(off + partial_rows * 8, 256);
  L.attn_o = off;
  off = align_up(off + partial_rows * s.head_dim * 4, 256);
  L.lse = off;
  off = align_up(off + (size_t)c.rows * c.shards * 8, 256);
  L.jobs = off;
  off = align_up(off + (size_t)s.batch * sizeof(ReqState), 256);
  L.gath = off;
  off = align_up(off + (size_t)c.rows * 4, 256);
  L.unif = off;
  off = align_up(off + (size_t)s.batch * (s.stride_n - 1) * 16, 256);
  L.resid = off;
  off = align_up(off + (size_t)s.batch * c.r_shards * sizeof(ResidShard), 256);
  L.prop = off;
  off = align_up(off + (size_t)s.batch * s.stride_n * prop_shards(s.vocab) * sizeof(PropPart), 256);
  L.total = off;
  return L;
}

}  // namespace isd

using namespace isd;

extern "C" {

int32_t isd_abi_version(void) { return 10; }

const char* isd_status_string(int32_t status) {
  switch (status) {
    case ISD_OK: return "ok";
    case ISD_ERR_NULL: return "a required pointer is NULL";
    case ISD_ERR_SHAPE: return "inconsistent or out-of-range sizes";
    case ISD_ERR_DTYPE: return "unknown dtype";
    case ISD_ERR_WORKSPACE: return "workspace smaller than isd_workspace_bytes()";
    case ISD_ERR_UNSUPPORTED: return "valid request not implemented by this build";
    case ISD_ERR_HIP: return "HIP launch or runtime error (see isd_last_error)";
    case ISD_ERR_ALIGNMENT: return "a tensor pointer is not 16-byte aligned";
  }
  return "unknown status";
}

const char* isd_last_error(void) { return g_last_error; }

size_t isd_workspace_bytes(const isd_shape* shape) {
  if (check_shape(shape) != ISD_OK) return 0;
  return ws_layout(*shape).total;
}

isd_status isd_workspace_init(const isd_shape* shape, void* workspace, size_t ws_bytes,
                              hipStream_t stream) {
  isd_status st = check_shape(shape);
  if (st != ISD_OK) return st;
  st = check_ws(shape, workspace, ws_bytes);
  if (st != ISD_OK) return st;
  const WsLayout L = ws_layout(*shape);
  hipError_t e = launch_workspace_init(workspace, L.zero_end, stream);
  return e == hipSuccess ? ISD_OK : hip_fail(e, "isd_workspace_init");
}

isd_status isd_read_flags(const void* workspace, uint32_t* flags, hipStream_t stream) {
  if (!workspace || !flags) return ISD_ERR_NULL;
  hipError_t e = hipMemcpyAsync(flags, workspace, sizeof(uint32_t), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  return e == hipSuccess ? ISD_OK : hip_fail(e, "isd_read_flags");
}

isd_status isd_attention(const isd_shape* shape, const void* q, const void* k_new, const void* v_new,
                         const void* k_pages, const void* v_pages, const int32_t* page_table,
                         const int32_t* ctx_lens, float scale, void* out, void* workspace,
                         size_t ws_bytes, hipStream_t stream) {
  isd_status st = check_shape(shape);
  if (st != ISD_OK) return st;
  if (!q || !k_new || !v_new || !k_pages || !v_pages || !page_table || !ctx_lens || !out)
    return ISD_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_pages) || !aligned16(v_pages) || !aligned16(k_new) ||
      !aligned16(v_new) || !aligned16(out))
    return ISD_ERR_ALIGNMENT;
  if (!(scale >= 0.f) || scale > 1e30f) return ISD_ERR_SHAPE;
  st = check_ws(shape, workspace, ws_bytes);
  if (st != ISD_OK) return st;
  if (scale == 0.f) scale = 1.0f / std::sqrt(float(shape->head_dim));
  const AttnPlan p = plan_attention(*shape);
  const WsLayout L = ws_layout(*shape);
  hipError_t e = launch_attention(*shape, p, q, k_new, v_new, k_pages, v_pages, page_table, ctx_lens,
                                  scale, out, static_cast<char*>(workspace), L, stream);
  return e == hipSuccess ? ISD_OK : hip_fail(e, "isd_attention");
}

isd_status isd_accept(const isd_shape* shape, const void* p_logits, const void* q_logits,
                      const int32_t* proposals, const int32_t* req_ids, const int32_t* positions,
                      uint64_t seed_lo, uint64_t seed_hi, uint32_t step, const int64_t* step_per_request,
                      const float* q_norms, int32_t* accept_len,
                      int32_t* out_tokens, int32_t* n_out, int32_t* n_commit, float* logp_sel,
                      float* logq_sel, void* workspace, size_t ws_bytes, hipStream_t stream) {
  isd_status st = check_shape(shape);
  if (st != ISD_OK) return st;
  if (!p_logits || !q_logits || !proposals || !req_ids || !positions || !accept_len || !out_tokens ||
      !n_out || !n_commit || !logp_sel || !logq_sel)
    return ISD_ERR_NULL;
  if (!aligned16(p_logits) || !aligned16(q_logits) || !aligned8(q_norms)) return ISD_ERR_ALIGNMENT;
  if (shape->batch > 65535) return ISD_ERR_UNSUPPORTED;
  if (shape->vocab > 2048 * 1024) return ISD_ERR_UNSUPPORTED;   // residual shards per row <= 1024
  st = check_ws(shape, workspace, ws_bytes);
  if (st != ISD_OK) return st;
  const AcceptPlan p = plan_accept(*shape);
  const WsLayout L = ws_layout(*shape);
  char* ws = static_cast<char*>(workspace);
  hipError_t e = launch_accept(*shape, p, p_logits, q_logits, proposals, req_ids, positions, seed_lo,
                               seed_hi, step, step_per_request, q_norms, accept_len, out_tokens, n_out, n_commit,
                               logp_sel, logq_sel, ws, L, reinterpret_cast<uint32_t*>(ws + L.flags), nullptr,
                               stream);
  return e == hipSuccess ? ISD_OK : hip_fail(e, "isd_accept");
}

isd_status isd_accept_commit(const isd_shape* shape, const void* p_logits, const void* q_logits,
                             const int32_t* proposals, const int32_t* req_ids, const int32_t* positions,
                             uint64_t seed_lo, uint64_t seed_hi, uint32_t step,
                             const int64_t* step_per_request, const float* q_norms, int32_t* accept_len,
                             int32_t* out_tokens, int32_t* n_out, int32_t* n_commit, float* logp_sel,
                             float* logq_sel, const void* k_new, const void* v_new, void* k_pages,
                             void* v_pages, const int32_t* page_table, const int32_t* ctx_lens_in,
                             int32_t* ctx_lens_out, const int32_t* loop_mode, void* workspace, size_t ws_bytes,
                             hipStream_t stream) {
  isd_status st = check_accept_commit(shape, p_logits, q_logits, proposals, req_ids, positions, q_norms,
                                      accept_len, out_tokens, n_out, n_commit, logp_sel, logq_sel, k_new, v_new,
                                      k_pages, v_pages, page_table, ctx_lens_in, ctx_lens_out);
  if (st != ISD_OK) return st;
  st = check_ws(shape, workspace, ws_bytes);
  if (st != ISD_OK) return st;
  const WsLayout L = ws_layout(*shape);
  char* ws = static_cast<char*>(workspace);
  hipError_t e = run_accept_commit(*shape, p_logits, q_logits, proposals, req_ids, positions, seed_lo, seed_hi,
                                   step, step_per_request, q_norms, accept_len, out_tokens, n_out, n_commit,
                                   logp_sel, logq_sel, k_new, v_new, k_pages, v_pages, page_table, ctx_lens_in,
                                   ctx_lens_out, loop_mode, ws, L, reinterpret_cast<uint32_t*>(ws + L.flags),
                                   stream);
  return e == hipSuccess ? ISD_OK : hip_fail(e, "isd_accept_commit");
}

isd_status isd_accept_commit_noalloc(const isd_shape* shape, const void* p_logits, const void* q_logits,
                                     const int32_t* proposals, const int32_t* req_ids, const int32_t* positions,
                                     uint64_t seed_lo, uint64_t seed_hi, uint32_t step,
                                     const int64_t* step_per_request, const float* q_norms, int32_t* accept_len,
                                     int32_t* out_tokens, int32_t* n_out, int32_t* n_commit, float* logp_sel,
                                     float* logq_sel, const void* k_new, const void* v_new, void* k_pages,
                                     void* v_pages, const int32_t* page_table, const int32_t* ctx_lens_in,
                                     int32_t* ctx_lens_out, const int32_t* loop_mode, uint32_t* flags,
                                     hipStream_t stream) {
  isd_status st = check_accept_commit(shape, p_logits, q_logits, proposals, req_ids, positions, q_norms,
                                      accept_len, out_tokens, n_out, n_commit, logp_sel, logq_sel, k_new, v_new,
                                      k_pages, v_pages, page_table, ctx_lens_in, ctx_lens_out);
  if (st != ISD_OK) return st;
  const WsLayout L = scratch_layout(*shape);
  if (L.total > kScratchBytes) {
    std::snprintf(g_last_error, sizeof(g_last_error),
                  "isd_accept_commit_noalloc: this shape needs %zu bytes of scratch, the library holds %zu",
                  L.total, kScratchBytes);
    return ISD_ERR_WORKSPACE;
  }
  char* ws = nullptr;
  hipError_t e = device_scratch(&ws, stream);
  if (e == hipSuccess)
    e = run_accept_commit(*shape, p_logits, q_logits, proposals, req_ids, positions, seed_lo, seed_hi, step,
                          step_per_request, q_norms, accept_len, out_tokens, n_out, n_commit, logp_sel, logq_sel,
                          k_new, v_new, k_pages, v_pages, page_table, ctx_lens_in, ctx_lens_out, loop_mode, ws, L,
                          flags, stream);
  return e == hipSuccess ? ISD_OK : hip_fail(e, "isd_accept_commit_noalloc");
}

isd_status kv_commit(const isd_shape* shape, const void* k_new, const void* v_new, void* k_pages,
                     void* v_pages, const int32_t* page_table, const int32_t* ctx_lens_in,
                     const int32_t* n_commit, int32_t* ctx_lens_out, void* workspace,
                     size_t ws_bytes, hipStream_t stream) {
  isd_status st = check_shape(shape);
  if (st != ISD_OK) return st;
  if (!k_new || !v_new || !k_pages || !v_pages || !page_table || !ctx_lens_in || !n_commit ||
      !ctx_lens_out)
    return ISD_ERR_NULL;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pages)) return ISD_ERR_ALIGNMENT;
  st = check_ws(shape, workspace, ws_bytes);
  if (st != ISD_OK) return st;
  const WsLayout L = ws_layout(*shape);
  char* ws = static_cast<char*>(workspace);
  const CommitArgs c = commit_args(*shape, k_new, v_new, k_pages, v_pages, page_table, ctx_lens_in, n_commit,
                                   ctx_lens_out, reinterpret_cast<uint32_t*>(ws + L.flags));
  hipError_t e = launch_commit(*shape, c, stream);
  return e == hipSuccess ? ISD_OK : hip_fail(e, "kv_commit");
}

isd_status isd_propose(const isd_shape* shape, const void* mask_logits, const int32_t* req_ids,
                       const int32_t* positions, uint64_t seed_lo, uint64_t seed_hi, uint32_t step,
                       const int64_t* step_per_request, int32_t mode, int32_t* proposals, float* row_norms,
                       void* workspace, size_t ws_bytes, hipStream_t stream) {
  isd_status st = check_shape(shape);
  if (st != ISD_OK) return st;
  if (mode != ISD_PROPOSE_SAMPLE && mode != ISD_PROPOSE_ARGMAX) return ISD_ERR_UNSUPPORTED;
  if (!mask_logits || !proposals || (mode == ISD_PROPOSE_SAMPLE && (!req_ids || !positions)))
    return ISD_ERR_NULL;
  if (!aligned16(mask_logits) || !aligned8(row_norms)) return ISD_ERR_ALIGNMENT;
  if ((long long)shape->batch * shape->stride_n > 65535) return ISD_ERR_UNSUPPORTED;
  if (row_norms && mode != ISD_PROPOSE_SAMPLE) return ISD_ERR_UNSUPPORTED;   // argmax sums nothing
  st = check_ws(shape, workspace, ws_bytes);
  if (st != ISD_OK) return st;
  hipError_t e = launch_propose(*shape, mask_logits, req_ids, positions, seed_lo, seed_hi, step,
                                step_per_request, mode, proposals, row_norms, static_cast<char*>(workspace),
                                ws_layout(*shape), stream);
  return e == hipSuccess ? ISD_OK : hip_fail(e, "isd_propose");
}

isd_status isd_loop_advance(const isd_shape* shape, const int32_t* accept_len, const int32_t* n_out,
                            const int32_t* next_proposals, int32_t* n_commit, int32_t* mode,
                            int32_t* proposals, int32_t* positions, int64_t* tokens, int64_t* forwards,
                            const float* norms_in, float* norms_out, hipStream_t stream) {
  isd_status st = check_shape(shape);
  if (st != ISD_OK) return st;
  if (!accept_len || !n_out || !next_proposals || !n_commit || !mode || !proposals || !positions ||
      !tokens || !forwards || (!norms_in != !norms_out))
    return ISD_ERR_NULL;
  if (!aligned8(norms_in) || !aligned8(norms_out)) return ISD_ERR_ALIGNMENT;
  hipError_t e = launch_loop_advance(shape->batch, shape->stride_n, accept_len, n_out, next_proposals,
                                     n_commit, mode, proposals, positions, tokens, forwards, norms_in, norms_out,
                                     stream);
  return e == hipSuccess ? ISD_OK : hip_fail(e, "isd_loop_advance");
}

size_t isd_lora_workspace_bytes(int32_t n_mask, int32_t d_in, int32_t rank) {
  if (n_mask < 0 || d_in < 256 || d_in % 256 || rank != 128) return 0;
  return lora_layout(n_mask, d_in, rank).total;
}

isd_status isd_lora_delta(int32_t rows, int32_t d_in, int32_t d_out, int32_t rank, const void* X,
                          const void* A_t, const void* B_t, const int32_t* mask_rows, int32_t n_mask,
                          float scale, void* Y, void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (rows < 1 || n_mask < 0 || n_mask > rows || d_in < 1 || d_out < 1 || rank < 1) return ISD_ERR_SHAPE;
  if (rank != 128 || d_in % 256 || d_out % 128) return ISD_ERR_UNSUPPORTED;
  if ((n_mask + 31) / 32 > 65535) return ISD_ERR_UNSUPPORTED;
  if (!(scale == scale)) return ISD_ERR_SHAPE;
  if (!X || !A_t || !B_t || !Y || !workspace || (n_mask > 0 && !mask_rows)) return ISD_ERR_NULL;
  if (!aligned16(X) || !aligned16(A_t) || !aligned16(B_t) || !aligned16(Y) || !aligned16(workspace))
    return ISD_ERR_ALIGNMENT;
  if (ws_bytes < lora_layout(n_mask, d_in, rank).total) return ISD_ERR_WORKSPACE;
  hipError_t e = launch_lora(rows, d_in, d_out, rank, X, A_t, B_t, mask_rows, n_mask, scale, Y,
                             static_cast<char*>(workspace), stream);
  return e == hipSuccess ? ISD_OK : hip_fail(e, "isd_lora_delta");
}

namespace {

// Shape check shared by the gated projection entries: ISD_OK, or the status
// the call returns (the workspace query answers 0 for any failure).
isd_status gl_shape(int32_t n_proj, int32_t rows, int32_t d_in, const int32_t* d_out, int32_t rank,
                    int32_t n_mask) {
  if (!d_out) return ISD_ERR_NULL;
  if (n_proj < 1 || rows < 1 || d_in < 1 || rank < 0 || n_mask < 0 || n_mask > rows) return ISD_ERR_SHAPE;
  if (n_proj > kGlMaxProj || rows > kGlMaxRows || d_in > (1 << 16) || d_in % 256 || (rank != 0 && rank != 128))
    return ISD_ERR_UNSUPPORTED;
  long total = 0;
  for (int p = 0; p < n_proj; ++p) {
    if (d_out[p] < 1) return ISD_ERR_SHAPE;
    if (d_out[p] % 128) return ISD_ERR_UNSUPPORTED;
    total += d_out[p];
  }
  if (long(rows) * total > kGlMaxOut) return ISD_ERR_UNSUPPORTED;
  return ISD_OK;
}

isd_status gated_group(int32_t n_proj, int32_t rows, int32_t d_in, const int32_t* d_out, int32_t rank,
                       const void* X, const void* const* W_t, const void* const* A_t, const void* const* B_t,
                       const int32_t* mask_rows, int32_t n_mask, float scale, void* const* Y, void* workspace,
                       size_t ws_bytes, hipStream_t stream, const char* name) {
  if (isd_status st = gl_shape(n_proj, rows, d_in, d_out, rank, n_mask)) return st;
  if (!(scale == scale) || scale - scale != 0.f) return ISD_ERR_SHAPE;
  if (!X || !W_t || !Y || !workspace) return ISD_ERR_NULL;
  if (rank > 0 && (!A_t || !B_t || (n_mask > 0 && !mask_rows))) return ISD_ERR_NULL;
  if (!aligned16(X) || !aligned16(workspace)) return ISD_ERR_ALIGNMENT;
  for (int p = 0; p < n_proj; ++p) {
    if (!W_t[p] || !Y[p] || (rank > 0 && (!A_t[p] || !B_t[p]))) return ISD_ERR_NULL;
    if (!aligned16(W_t[p]) || !aligned16(Y[p]) || (rank > 0 && (!aligned16(A_t[p]) || !aligned16(B_t[p]))))
      return ISD_ERR_ALIGNMENT;
  }
  if (ws_bytes < gl_layout(n_proj, rows, d_in, d_out, rank, n_mask).total) return ISD_ERR_WORKSPACE;
  hipError_t e = launch_gated_linear(n_proj, rows, d_in, d_out, rank, X, W_t, A_t, B_t, mask_rows, n_mask, scale,
                                     Y, static_cast<char*>(workspace), stream);
  return e == hipSuccess ? ISD_OK : hip_fail(e, name);
}

}  // namespace

size_t isd_gated_linear_workspace_bytes(int32_t rows, int32_t d_in, int32_t d_out, int32_t rank,
                                        int32_t n_mask) {
  return isd_gated_linear_group_workspace_bytes(1, rows, d_in, &d_out, rank, n_mask);
}

isd_status isd_gated_linear(int32_t rows, int32_t d_in, int32_t d_out, int32_t rank, const void* X,
                            const void* W_t, const void* A_t, const void* B_t, const int32_t* mask_rows,
                            int32_t n_mask, float scale, void* Y, void* workspace, size_t ws_bytes,
                            hipStream_t stream) {
  return gated_group(1, rows, d_in, &d_out, rank, X, &W_t, rank > 0 ? &A_t : nullptr, rank > 0 ? &B_t : nullptr,
                     mask_rows, n_mask, scale, &Y, workspace, ws_bytes, stream, "isd_gated_linear");
}

size_t isd_gated_linear_group_workspace_bytes(int32_t n_proj, int32_t rows, int32_t d_in, const int32_t* d_out,
                                              int32_t rank, int32_t n_mask) {
  if (gl_shape(n_proj, rows, d_in, d_out, rank, n_mask) != ISD_OK) return 0;
  return gl_layout(n_proj, rows, d_in, d_out, rank, n_mask).total;
}

isd_status isd_gated_linear_group(int32_t n_proj, int32_t rows, int32_t d_in, const int32_t* d_out, int32_t rank,
                                  const void* X, const void* const* W_t, const void* const* A_t,
                                  const void* const* B_t, const int32_t* mask_rows, int32_t n_mask, float scale,
                                  void* const* Y, void* workspace, size_t ws_bytes, hipStream_t stream) {
  return gated_group(n_proj, rows, d_in, d_out, rank, X, W_t, A_t, B_t, mask_rows, n_mask, scale, Y, workspace,
                     ws_bytes, stream, "isd_gated_linear_group");
}

}  // extern "C"
