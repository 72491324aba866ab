// Host-side planning, workspace layout and kernel launchers of libisd.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "isd.h"

namespace isd {

constexpr int kPage = 16;          // tokens per KV page
constexpr int kTileTokens = 32;    // tokens per attention tile (two pages)
// Waves per attention workgroup (one per SIMD, so two workgroups share a CU
// and one streams while the other stages its operands or writes its output;
// each wave takes 32-token tiles round-robin for one block of 32 query rows).
constexpr int kAttnWaves = 4;
constexpr size_t kHeaderBytes = 256;

// How the KV walk of isd_attention is split across workgroups.
struct AttnPlan {
  int q_rows;           // Q = 2N-1
  int group;            // G = Hq / Hkv
  int rows;             // G * Q query rows per KV head
  int rows_pad;         // rows rounded up to 32
  int row_blocks;       // rows_pad / 32
  int tiles_max;        // tiles of the longest context the plan is sized for
  int tiles_per_split;  // tiles per workgroup (last split takes the remainder)
  int n_splits;         // workgroups per (request, KV head)
};

// How isd_accept shards the vocabulary.
struct AcceptPlan {
  int rows;             // 2 * B * (N-1) logit rows (p rows first, then q rows)
  int shards;           // shards per row for the fp32 normaliser
  int shard_len;        // elements per shard (multiple of 8)
  int r_shards;         // shards per row for the fp64 residual
  int r_shard_len;
  int fuse_decision;    // 1: every residual workgroup makes its request's decision (no decision launch)
};

struct WsLayout {
  size_t flags = 0;          // uint32 device flags
  size_t attn_cnt = 0;       // uint32 per (request, kv head): split arrivals
  size_t zero_end = 0;       // [0, zero_end) is zeroed by isd_workspace_init
  size_t attn_ml = 0;        // float2 (m, l) per partial row
  size_t attn_o = 0;         // float [D] per partial row
  size_t lse = 0;            // float2 (max, sum) per (row, shard)
  size_t jobs = 0;           // ReqState per request (or per listed rejecting request)
  size_t gath = 0;           // float per (request, p/q row): the logit at the row's proposal
  size_t unif = 0;           // double pair per (request, stride row j < N-1): the Philox uniforms (u, u')
  size_t resid = 0;          // ResidShard per (request, residual shard)
  size_t prop = 0;           // PropPart per (MASK row, proposal shard)
  size_t total = 0;
};

// Header word (uint32 at this byte offset of the workspace).
constexpr size_t kRejCountOffset = 4;     // entries in the compact list of rejecting requests

// One request's job, written by the accept decision (req = -1: nothing
// rejected) and read by the residual kernels: either a compact list of the
// rejecting requests (a decision launch of its own) or one slot per request
// (the decision inside the residual pass).
struct ReqState {
  int32_t req;          // request index r
  int32_t accept_len;   // A
  int32_t reject_row;   // j of the rejected row
  float log_kappa;      // fp32 estimate of log(S_p / S_q), S = sum of exp(l - row max)
  float max_p;          // exact max logit of the rejected p row
  float max_q;          // and of its q row
  double u_resample;    // u' of the rejected position
};

// Residual pass output per (request, 2048-entry shard): float64 sums
// of e_p = exp(l_p - max p) and e_q, the same over the entries clearly in the
// residual's support under the estimated ratio, and the same again for each
// group of entries near its boundary that share one exact logit difference.
constexpr int kResidAmb = 8;
constexpr int kMaxResidShards = 1024;   // vocabularies up to 2048 * 1024 entries
struct ResidShard {
  double sp, sq;
  double a, b;
  int32_t n_amb;        // groups near the boundary (kResidAmb + 1: more than fit)
  int32_t pad;
  double amb[kResidAmb][2];
  double pad2;
};

// Per (MASK row, vocabulary shard) summary written by the proposal kernels.
struct PropPart {
  double sum;           // sum of exp(l - max) over the shard (sampling policy)
  float max;            // shard max logit
  int32_t idx;          // first index holding it
};
int prop_shards(int vocab);   // 4096-entry shards of a MASK row

// Compute units of the current device (queried once per device and cached).
int device_cus();

AttnPlan plan_attention(const isd_shape& s);
AcceptPlan plan_accept(const isd_shape& s);
WsLayout ws_layout(const isd_shape& s);

// Everything one KV commit reads and writes (kv_commit, and isd_accept_commit
// whose residual launch also runs the commit's workgroups).
struct CommitArgs {
  const void* k_new;
  const void* v_new;
  void* k_pages;
  void* v_pages;
  const int32_t* table;
  const int32_t* ctx_in;
  const int32_t* n_commit;
  int32_t* ctx_out;
  uint32_t* flags;
  const int32_t* loop_mode;   // per request (NULL: none): a re-proposing request commits its row N-1
  int N, Hkv, D, max_pages, num_pages;
  int kv_bf16;            // 1: bf16 pages, 0: fp32
};
CommitArgs commit_args(const isd_shape& s, const void* k_new, const void* v_new, void* k_pages,
                       void* v_pages, const int32_t* table, const int32_t* ctx_in,
                       const int32_t* n_commit, int32_t* ctx_out, uint32_t* flags,
                       const int32_t* loop_mode = nullptr);

// Launchers (return the first HIP error, hipSuccess otherwise).
hipError_t launch_attention(const isd_shape& s, const AttnPlan& p, const void* q,
                            const void* k_new, const void* v_new, const void* k_pages,
                            const void* v_pages, const int32_t* table, const int32_t* ctx_lens,
                            float scale, void* out, char* ws, const WsLayout& L,
                            hipStream_t stream);

hipError_t launch_accept(const isd_shape& s, const AcceptPlan& p, const void* p_logits,
                         const void* q_logits, const int32_t* proposals, const int32_t* req_ids,
                         const int32_t* positions, uint64_t seed_lo, uint64_t seed_hi,
                         uint32_t step, const int64_t* step_dev, const float* q_norms, int32_t* accept_len,
                         int32_t* out_tokens, int32_t* n_out, int32_t* n_commit, float* logp_sel,
                         float* logq_sel, char* ws,
                         const WsLayout& L, uint32_t* flags, const CommitArgs* commit, hipStream_t stream);

hipError_t launch_commit(const isd_shape& s, const CommitArgs& c, hipStream_t stream);

hipError_t launch_propose(const isd_shape& s, const void* mask_logits, const int32_t* req_ids,
                          const int32_t* positions, uint64_t seed_lo, uint64_t seed_hi, uint32_t step,
                          const int64_t* step_dev, int mode, int32_t* proposals, float* row_norms, char* ws,
                          const WsLayout& L, hipStream_t stream);

hipError_t launch_loop_advance(int B, int N, const int32_t* accept_len, const int32_t* n_out,
                               const int32_t* next_proposals, int32_t* n_commit, int32_t* mode,
                               int32_t* proposals, int32_t* positions, int64_t* tokens, int64_t* forwards,
                               const float* norms_in, float* norms_out, hipStream_t stream);

hipError_t launch_workspace_init(void* ws, size_t header_bytes, hipStream_t stream);

struct LoraLayout {
  size_t part = 0;    // float [d_in/256][n_mask padded to 32][rank]
  size_t t_hi = 0;    // bf16 [n_mask padded][rank]
  size_t t_lo = 0;
  size_t total = 0;
};
LoraLayout lora_layout(int32_t n_mask, int32_t d_in, int32_t rank);

hipError_t launch_lora(int32_t rows, int32_t d_in, int32_t d_out, int32_t rank, const void* X,
                       const void* A, const void* Bm, const int32_t* mask_rows, int32_t n_mask,
                       float scale, void* Y, char* ws, hipStream_t stream);

constexpr int kGlMaxProj = 4;             // projections of one gated group call

constexpr int32_t kGlMaxRows = 1 << 16;   // rows of one gated projection call
constexpr long kGlMaxOut = 1L << 30;      // rows x summed output width of one call

// Gated projection: tile shape and k split, a function of the shape alone so a
// gated call and the base-only call of the same shape sum in the same order.
struct GlPlan {
  int bm = 128;       // tiles of bm rows x bn outputs: 256 x 256 / 192, 128 x 256 / 192 / 128, 64 x 64
  int bn = 128;
  int stages = 4;     // LDS ring depth
  int waves = 4;      // waves per workgroup: 4 or 8
  int splits = 1;     // k split into this many ranges, summed by a second kernel
};
GlPlan gl_plan(int32_t rows, int32_t d_in, int32_t d_out, bool all256, bool all192);

struct GlLayout {
  size_t t = 0;       // bf16 [n_proj][rows][rank]: gated rows' scaled down-projections, zero elsewhere
  size_t down = 0;    // float [n_proj][d_in/256][n_mask][rank]: the down-projection partials
  size_t split = 0;   // float, per projection p in turn: [splits][rows][d_out[p]]
  size_t total = 0;
  GlPlan plan;
};
GlLayout gl_layout(int32_t n_proj, int32_t rows, int32_t d_in, const int32_t* d_out, int32_t rank,
                   int32_t n_mask);

hipError_t launch_gated_linear(int32_t n_proj, int32_t rows, int32_t d_in, const int32_t* d_out, int32_t rank,
                               const void* X, const void* const* W_t, const void* const* A_t,
                               const void* const* B_t, const int32_t* mask_rows, int32_t n_mask, float scale,
                               void* const* Y, char* ws, hipStream_t stream);

}  // namespace isd
