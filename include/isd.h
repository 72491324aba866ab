/*
 * isd.h -- C ABI of libisd.so: one Introspective Strided Decoding (ISD) step
 * on an AMD Instinct MI355X (gfx950).
 *
 * The step (I-DLM project page, ISD card; "I-DLM：扩散模型如何用'自省一致性'
 * 追上自回归模型质量", section "Introspective Strided Decoding（ISD）";
 * "自省扩散语言模型的 token 生成机制与工程实践", section "Token 生成的核心参数与
 * 验收机制"): every request carries a stride of Q = 2N-1 query rows at
 * consecutive positions.  Rows 0..N-2 are CLEAN rows holding the previous
 * pass's proposals x_1..x_{N-1}; rows N-1..2N-2 propose the next N tokens.
 * Under the logit shift (a row's output predicts the next position), row N-1
 * holds x_N, the stride's last token, so its output is the anchor
 * distribution of the token after x_N (the next stride's first proposal,
 * always kept), and rows N..2N-2 hold MASK.  One forward both verifies and
 * proposes:
 *
 *   isd_attention  strictly causal multi-query attention of the stride over
 *                  the request's paged KV cache and the stride itself;
 *   isd_accept     the p/q test: accept x_k with probability min(1, p/q),
 *                  resample from normalize(max(0, p - q)) at the first
 *                  rejection;
 *   kv_commit      append the rows of the accepted prefix to the KV pages
 *                  (isd_accept_commit: both in one call; isd_accept_commit_noalloc:
 *                  the same without a caller workspace);
 *   isd_propose    draw the next N proposals at rows N-1..2N-2 (sampling or
 *                  argmax);
 *   isd_loop_advance  per-request bookkeeping of the multi-step decoding loop;
 *   isd_lora_delta the gated low-rank delta of Residual ISD (R-ISD), added at
 *                  MASK rows only.
 *   isd_gated_linear  a whole R-ISD projection: base weights on every row,
 *                  the adapter fused in on the MASK rows.
 *   isd_gated_linear_group  up to four such projections of one input (the
 *                  q, k and v projections; gate and up) in one set of launches.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor arguments are DEVICE pointers owned by the caller, dense,
 *   row-major in the index order written next to them.  The library never
 *   allocates, frees or synchronises on these calls; the work is enqueued on
 *   `stream` and the call returns at once.  Calls on one stream run in order;
 *   the intended order per step is attention -> accept -> commit (a decoding
 *   loop: attention -> accept_commit and propose -> loop_advance).  Calls
 *   enqueue kernels only (no memset, no allocation), so they may be recorded
 *   into a HIP graph.  The only state kept between calls is each device's
 *   compute-unit count, queried once.
 * - Arguments are validated on the host before anything is enqueued.  A bad
 *   argument returns an isd_status != ISD_OK and enqueues nothing.  Values
 *   that live in device memory (context lengths, page-table entries, token
 *   ids, commit counts) cannot be checked on the host: the kernels bound-check
 *   them, skip the offending access, and OR a bit into the device flag word
 *   (ISD_FLAG_*) at byte offset 0 of the workspace.  Results for a request
 *   that raised a flag are unspecified, but no access leaves the buffers.
 * - The workspace is caller-owned device memory of at least
 *   isd_workspace_bytes() bytes, prepared once by isd_workspace_init().  It
 *   holds scratch partials and the flag word and may be reused by every call
 *   on the same stream; concurrent calls must use distinct workspaces.
 * - A launch failure returns ISD_ERR_HIP; isd_last_error() gives the text.
 *   Nothing crosses the ABI as a C++ exception.
 */
#ifndef ISD_H
#define ISD_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum isd_status {
  ISD_OK = 0,
  ISD_ERR_NULL = 1,         /* a required pointer is NULL */
  ISD_ERR_SHAPE = 2,        /* inconsistent or out-of-range sizes */
  ISD_ERR_DTYPE = 3,        /* unknown dtype */
  ISD_ERR_WORKSPACE = 4,    /* workspace smaller than isd_workspace_bytes() */
  ISD_ERR_UNSUPPORTED = 5,  /* valid request this build does not implement */
  ISD_ERR_HIP = 6,          /* a HIP launch or runtime call failed */
  ISD_ERR_ALIGNMENT = 7     /* a tensor pointer is not 16-byte aligned */
} isd_status;

typedef enum isd_dtype {
  ISD_F32 = 0,   /* IEEE binary32 */
  ISD_BF16 = 1   /* bfloat16 */
} isd_dtype;

/* Device flag bits (workspace byte offset 0, uint32). */
#define ISD_FLAG_CTX_RANGE 0x1u    /* ctx_lens[r] < 0 or > max_pages * page_size */
#define ISD_FLAG_PAGE_RANGE 0x2u   /* a needed page_table entry is outside [0, num_pages) */
#define ISD_FLAG_TOKEN_RANGE 0x4u  /* a proposal id is outside [0, vocab) */
#define ISD_FLAG_COMMIT_RANGE 0x8u /* n_commit[r] outside [0, N], or no page for a commit slot */
#define ISD_FLAG_ROW_RANGE 0x10u   /* a LoRA mask row is outside [0, rows) */

/*
 * Sizes of one step.
 *   Q = 2 * stride_n - 1 query rows per request; G = n_q_heads / n_kv_heads.
 *   Supported: 1 <= batch <= 65535, stride_n in [2, 16] (Q <= 31: the stride
 *   block is one 32-token attention tile), head_dim in {64, 128},
 *   page_size == 16,
 *   G * Q <= 64 (query rows per KV head), n_q_heads % n_kv_heads == 0.
 *   max_ctx is a hint (an upper bound of the context lengths, used to split
 *   the KV walk across workgroups); 0 means max_pages * page_size.  A context
 *   longer than max_ctx is still processed correctly, only less evenly.
 */
typedef struct isd_shape {
  int32_t batch;        /* B: requests in the step */
  int32_t stride_n;     /* N: proposals per stride */
  int32_t n_q_heads;    /* Hq */
  int32_t n_kv_heads;   /* Hkv */
  int32_t head_dim;     /* D */
  int32_t page_size;    /* tokens per KV page (16) */
  int32_t max_pages;    /* columns of page_table */
  int32_t num_pages;    /* pages in the pool */
  int32_t vocab;        /* V */
  int32_t max_ctx;      /* hint, see above */
  int32_t kv_dtype;     /* an isd_dtype: q, k_new, v_new, pages, out */
  int32_t logit_dtype;  /* an isd_dtype: p_logits, q_logits */
} isd_shape;

/*
 * KV page pool layout (both pools hold num_pages pages; e = element size):
 *
 *   k_pages[page][kv_head][d / 8][slot][d % 8]
 *   v_pages[page][kv_head][d][sigma(slot)]
 *
 * sigma swaps bits 2 and 3 of the slot index (sigma(s) = (s & 3) |
 * ((s & 4) << 1) | ((s & 8) >> 1)); it is its own inverse.  Token position t
 * of request r lives in page page_table[r * max_pages + t / page_size],
 * slot t % page_size.  Both layouts let one 64-lane wavefront read a page's
 * keys or values as fully used 16-byte vectors that feed the matrix cores
 * directly.
 */

/* Workspace bytes needed by isd_attention, isd_accept, kv_commit and isd_propose for `shape`. */
size_t isd_workspace_bytes(const isd_shape* shape);

/*
 * Prepare a workspace for `shape` on `stream`: zero the header (flag word and
 * internal counters).  Call once per workspace before its first use; the
 * calls below keep the header consistent after.
 */
isd_status isd_workspace_init(const isd_shape* shape, void* workspace, size_t ws_bytes,
                              hipStream_t stream);

/*
 * Read the device flag word of `workspace` into *flags.  This call copies
 * to the host and synchronises `stream`; it is meant for checks, not for the
 * per-step path.
 */
isd_status isd_read_flags(const void* workspace, uint32_t* flags, hipStream_t stream);

/*
 * isd_attention -- strictly causal stride attention over the paged KV cache.
 *
 * Definition ("I-DLM：扩散模型如何用'自省一致性'追上自回归模型质量", section
 * "三项关键训练创新", item 1: one causal mask over MASK and clean tokens;
 * I-DLM project page, ISD card): stride row i of request r sits at absolute
 * position L_r + i (L_r = ctx_lens[r]) and query head h reads KV head h / G.
 * Row i attends to the cached positions 0..L_r-1 (from the pages) and to the
 * stride's own rows 0..i (k_new / v_new), never to later rows:
 *
 *   out[r][i][h] = sum_t softmax_t(scale * q[r][i][h] . k_t) v_t
 *
 *   q      [B][Q][Hq][D]    kv_dtype
 *   k_new  [B][Q][Hkv][D]   kv_dtype (keys of this pass's stride rows)
 *   v_new  [B][Q][Hkv][D]   kv_dtype
 *   k_pages, v_pages        pool layout above, kv_dtype
 *   page_table [B][max_pages] int32; entries past a request's pages are ignored
 *   ctx_lens   [B] int32    cached positions per request, 0 allowed
 *   scale      softmax scale; 0 selects 1/sqrt(D)
 *   out    [B][Q][Hq][D]    kv_dtype, written
 *
 * Accumulation is fp32 (bf16 inputs run on the matrix cores).  Flags:
 * CTX_RANGE, PAGE_RANGE.
 */
isd_status isd_attention(const isd_shape* shape, const void* q, const void* k_new,
                         const void* v_new, const void* k_pages, const void* v_pages,
                         const int32_t* page_table, const int32_t* ctx_lens, float scale,
                         void* out, void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * isd_accept -- the p/q acceptance test with residual resampling.
 *
 * Definition ("I-DLM：扩散模型如何用'自省一致性'追上自回归模型质量", section
 * "Introspective Strided Decoding（ISD）"; "自省扩散语言模型的 token 生成机制与
 * 工程实践", sections "从质量差距到自省机制" and "Token 生成的核心参数与验收机制";
 * I-DLM project page, caption on geometric acceptance):
 *   - x_1 = proposals[r][0] was decided before this step and is always kept.
 *   - For k = 2..N, row j = k-2 of p_logits is the anchor distribution p
 *     (from CLEAN row j, logit-shifted) and row j of q_logits the proposal
 *     distribution q that produced x_k.  Logits are used as given
 *     (temperature already applied).
 *   - rho_k = exp(log p(x_k) - log q(x_k)); accept iff u_k < rho_k; stop at
 *     the first rejection.  accept_len = A = 1 + leading accepts, in [1, N].
 *   - If A < N, the token at position A+1 is y* = the first y (in vocabulary
 *     order) whose running sum of max(0, p - q) exceeds u'_k * sum(max(0, p - q)),
 *     computed in float64; if that sum is 0, p itself is sampled the same way.
 *   - u_k and u'_k are words 0 and 1 of the Philox4x64-10 block (Salmon et
 *     al., SC'11) with key (seed_lo, seed_hi) and counter
 *     (req_ids[r], positions[r] + k - 1, step, 0), each mapped to
 *     (w >> 11) * 2^-53.  positions[r] is the absolute position of x_1.
 *     step is the `step` argument, or, when step_per_request is not NULL,
 *     the low 32 bits of step_per_request[r] (a device array, so a recorded
 *     graph of a decoding loop draws afresh on every replay).
 *
 *   p_logits, q_logits [B][N-1][V]  logit_dtype
 *   proposals  [B][N] int32          x_1..x_N
 *   req_ids    [B] int32 (>= 0)      stable request ids (Philox counter word 0)
 *   positions  [B] int32 (>= 0)
 *   accept_len [B] int32             written: A
 *   out_tokens [B][N] int32          written: x_1..x_A, then y* if A < N, then -1
 *   n_out      [B] int32             written: A + (A < N)
 *   n_commit   [B] int32             written: A, the stride rows 0..A-1 that hold
 *                                    the accepted prefix and are committed
 *   logp_sel, logq_sel [B][N-1] fp32 written: log p(x_k), log q(x_k) for every row
 *   q_norms    [B][N] float pairs (max, sum of exp(l - max)), 8-byte aligned,
 *              or NULL.  The q rows are the previous forward's MASK rows
 *              that proposed x_2..x_N, and isd_propose already normalised
 *              them: pass the pairs it wrote (its row_norms) and the q rows'
 *              normalisers are taken from there instead of a second pass
 *              over q_logits; pair (r, k) belongs to the MASK row that
 *              proposed x_{k+1}, pair (r, 0) is not read.  q_logits is still
 *              read at the proposals.  NULL: computed here.
 *
 * The log-normalisers behind logp_sel / logq_sel and rho are fp32; the
 * residual is fp64.  Flags: TOKEN_RANGE (an out-of-range proposal is
 * rejected).
 */
isd_status isd_accept(const isd_shape* shape, const void* p_logits, const void* q_logits,
                      const int32_t* proposals, const int32_t* req_ids, const int32_t* positions,
                      uint64_t seed_lo, uint64_t seed_hi, uint32_t step,
                      const int64_t* step_per_request, const float* q_norms, int32_t* accept_len,
                      int32_t* out_tokens,
                      int32_t* n_out, int32_t* n_commit, float* logp_sel, float* logq_sel,
                      void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * kv_commit -- append the accepted prefix of every stride to the KV pages.
 *
 * Definition (paged KV cache reused from the AR serving stack:
 * "I-DLM：扩散模型如何用'自省一致性'追上自回归模型质量", section "推理：复用 AR
 * 推理栈"; the accepted prefix is committed, and a row's key/value is valid
 * iff its token and every token before it were accepted): rows
 * 0..n_commit[r]-1 of k_new[r] / v_new[r] (the rows holding x_1..x_A) are
 * written to positions ctx_lens_in[r] + i, and ctx_lens_out[r] =
 * ctx_lens_in[r] + n_commit[r].
 *
 *   k_new, v_new  [B][Q][Hkv][D] kv_dtype
 *   k_pages, v_pages  pool layout above, written in the committed slots only
 *   page_table    [B][max_pages] int32; the caller maps pages for every slot
 *                 it may commit (positions up to ctx_len + N - 1)
 *   ctx_lens_in   [B] int32
 *   n_commit      [B] int32 in [0, N] (isd_accept's output)
 *   ctx_lens_out  [B] int32, written; may alias ctx_lens_in
 *
 * Flags: CTX_RANGE, COMMIT_RANGE, PAGE_RANGE (the row is skipped and the
 * length still advances by the valid prefix only).
 */
isd_status kv_commit(const isd_shape* shape, const void* k_new, const void* v_new,
                     void* k_pages, void* v_pages, const int32_t* page_table,
                     const int32_t* ctx_lens_in, const int32_t* n_commit,
                     int32_t* ctx_lens_out, void* workspace, size_t ws_bytes,
                     hipStream_t stream);

/*
 * isd_accept_commit -- isd_accept, then kv_commit of the rows it accepted, in
 * one call with one launch fewer.
 *
 * Same definitions, arguments and outputs as isd_accept followed by
 * kv_commit(shape, k_new, v_new, k_pages, v_pages, page_table, ctx_lens_in,
 * n_commit, ctx_lens_out, ...) on the same stream, with n_commit the
 * isd_accept output; results are identical to those two calls.  The commit's
 * workgroups run inside the residual launch, next to the residual work,
 * once the accept decision is known.
 *
 *   loop_mode [B] int32 or NULL: the decoding loop's per-request mode before
 *             this forward's isd_loop_advance (ISD_LOOP_VERIFY /
 *             ISD_LOOP_REPROPOSE, below).  A verifying request commits its
 *             accepted prefix as above; a re-proposing request commits one
 *             row, its stride row N-1 (which carries the token the forward
 *             before resampled), at position ctx_lens_in[r], and its length
 *             grows by one.  A loop forward commits here; there is no
 *             kv_commit after the bookkeeping.  NULL: every request verifies.
 *
 * Flags: those of both calls.
 */
isd_status isd_accept_commit(const isd_shape* shape, const void* p_logits, const void* q_logits,
                             const int32_t* proposals, const int32_t* req_ids,
                             const int32_t* positions, uint64_t seed_lo, uint64_t seed_hi,
                             uint32_t step, const int64_t* step_per_request, const float* q_norms,
                             int32_t* accept_len, int32_t* out_tokens, int32_t* n_out, int32_t* n_commit,
                             float* logp_sel, float* logq_sel,
                             const void* k_new, const void* v_new, void* k_pages, void* v_pages,
                             const int32_t* page_table, const int32_t* ctx_lens_in,
                             int32_t* ctx_lens_out, const int32_t* loop_mode, void* workspace,
                             size_t ws_bytes, hipStream_t stream);

/*
 * isd_accept_commit_noalloc -- isd_accept_commit for callers that cannot
 * allocate device memory or pass a workspace: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.
 *
 * Same definitions, arguments, outputs and launches as isd_accept_commit,
 * without `workspace` / `ws_bytes`: the partials live in a scratch array the
 * library holds on each device (16 MiB, held until the process ends; its
 * counter region is cleared by the first call on the device, and the kernels
 * rewind every counter they use).  The call allocates nothing and calls no
 * allocating routine.
 *
 *   flags  device pointer to one uint32 the caller owns (or NULL: not
 *          reported), into which the kernels OR the ISD_FLAG_* bits that
 *          isd_accept_commit would raise in its workspace.
 *
 * Returns ISD_ERR_WORKSPACE when the shape needs more than the 16 MiB
 * (batch * ceil(vocab / 2048) * 176 bytes of residual partials dominate:
 * e.g. 128 requests at a 1.2M-entry vocabulary fit).  Every call on one
 * device shares that device's scratch: calls that overlap in time on one
 * device (two streams, two threads) race; issue them in one stream's order.
 */
isd_status isd_accept_commit_noalloc(const isd_shape* shape, const void* p_logits, const void* q_logits,
                                     const int32_t* proposals, const int32_t* req_ids,
                                     const int32_t* positions, uint64_t seed_lo, uint64_t seed_hi,
                                     uint32_t step, const int64_t* step_per_request, const float* q_norms,
                                     int32_t* accept_len, int32_t* out_tokens, int32_t* n_out,
                                     int32_t* n_commit, float* logp_sel, float* logq_sel,
                                     const void* k_new, const void* v_new, void* k_pages, void* v_pages,
                                     const int32_t* page_table, const int32_t* ctx_lens_in,
                                     int32_t* ctx_lens_out, const int32_t* loop_mode, uint32_t* flags,
                                     hipStream_t stream);

/*
 * isd_propose -- draw the next N proposals at the MASK rows.
 *
 * Definition ("I-DLM：扩散模型如何用'自省一致性'追上自回归模型质量", section
 * "Introspective Strided Decoding（ISD）": every forward pass draws N new
 * tokens at the MASK positions from the proposal distribution q;
 * "自省扩散语言模型的 token 生成机制与工程实践", section "从质量差距到自省机制",
 * and section "服务部署与 SGLang 集成" for the argmax proposal policy):
 *
 *   ISD_PROPOSE_SAMPLE  proposals[r][k] = the first y (vocabulary order)
 *                       whose running sum of q = softmax(mask_logits[r][k])
 *                       exceeds u * (total), sums in float64; u is word 0 of
 *                       the Philox4x64-10 block with key (seed_lo, seed_hi)
 *                       and counter (req_ids[r], positions[r] + N + k, step,
 *                       1), mapped to (w >> 11) * 2^-53.  positions[r] is the
 *                       absolute position of x_1, so MASK row k proposes the
 *                       token at positions[r] + N + k.  step is the `step`
 *                       argument or, when step_per_request is not NULL, the
 *                       low 32 bits of step_per_request[r] (device array).
 *   ISD_PROPOSE_ARGMAX  proposals[r][k] = the smallest index of the largest
 *                       logit (req_ids, positions, seed, step and
 *                       step_per_request unused and may be NULL / 0).
 *
 *   mask_logits [B][N][V] logit_dtype, 16-byte aligned; every row holds at
 *               least one finite logit
 *   proposals   [B][N] int32, written
 *   row_norms   [B][N] float pairs, 8-byte aligned, or NULL: written with
 *               each MASK row's (max logit, sum of exp(l - max)) for the
 *               isd_accept of the forward that verifies these proposals
 *               (its q_norms).  ISD_PROPOSE_SAMPLE only (the argmax policy
 *               sums nothing: ISD_ERR_UNSUPPORTED).
 *
 * Uses the same workspace as the calls above (isd_workspace_bytes()).
 * Supported: batch * stride_n <= 65535.
 */
typedef enum isd_propose_mode {
  ISD_PROPOSE_SAMPLE = 0,
  ISD_PROPOSE_ARGMAX = 1
} isd_propose_mode;

isd_status isd_propose(const isd_shape* shape, const void* mask_logits, const int32_t* req_ids,
                       const int32_t* positions, uint64_t seed_lo, uint64_t seed_hi,
                       uint32_t step, const int64_t* step_per_request, int32_t mode,
                       int32_t* proposals, float* row_norms, void* workspace, size_t ws_bytes,
                       hipStream_t stream);

/*
 * isd_loop_advance -- per-request bookkeeping of the multi-step decoding loop.
 *
 * Definition (every forward verifies the previous proposals and proposes N
 * new ones: "I-DLM：扩散模型如何用'自省一致性'追上自回归模型质量", section
 * "Introspective Strided Decoding（ISD）"; each request advances on its own:
 * I-DLM project page, caption on SDAR synchronisation; a rejection costs one
 * more forward that proposes again from the corrected prefix, the reading
 * that reproduces the TPF column of "自省扩散语言模型的 token 生成机制与工程
 * 实践", section "Token 生成的核心参数与验收机制").  A forward of the batch is
 * isd_attention (with ctx_lens = positions) -> isd_accept_commit (with
 * loop_mode = mode) and isd_propose -> isd_loop_advance on one stream (or
 * the two middle calls on two streams, joined before the bookkeeping), with
 * isd_accept_commit and isd_propose called with `proposals` and `positions`
 * below.  Per request r:
 *
 *   forwards[r] += 1, and
 *   mode VERIFY, accept_len A = N: tokens += N, proposals <- next_proposals,
 *                                   positions += N;
 *   mode VERIFY, A < N:            tokens += n_out (= A + 1), proposals kept,
 *                                   mode <- REPROPOSE, positions += n_out - N
 *                                   (so the re-proposing forward's row N-1 sits
 *                                   at the resampled token's position and
 *                                   carries it, and its proposing row k
 *                                   proposes the token right after the
 *                                   committed prefix, plus k);
 *   mode REPROPOSE:                its accept result is ignored, n_commit <- 1
 *                                   (its row N-1 was committed), proposals <-
 *                                   next_proposals, mode <- VERIFY,
 *                                   positions += N.
 *
 * Every committed token's key and value are then written exactly once, at
 * its own position: between forwards the committed length is positions[r]
 * in VERIFY mode and positions[r] + N - 1 in REPROPOSE mode (the resampled
 * token still waits for its row), and positions[r] is the context length the
 * next forward's attention reads.
 *
 *   accept_len, n_out [B] int32   this forward's isd_accept outputs
 *   next_proposals [B][N] int32   this forward's isd_propose output
 *   n_commit  [B] int32           isd_accept's output; set to 1 for a
 *                                 re-proposing request (rows committed)
 *   mode      [B] int32           ISD_LOOP_VERIFY / ISD_LOOP_REPROPOSE, in/out
 *   proposals [B][N] int32        the stride's x_1..x_N, in/out
 *   positions [B] int32           positions argument of the next forward, in/out;
 *                                 start at >= N - 1 so it stays non-negative
 *   tokens, forwards [B] int64    running counts, in/out (start at 0)
 *   norms_in, norms_out [B][N] float pairs, 8-byte aligned, both or neither
 *                                 NULL: norms_out <- norms_in, for every
 *                                 request and mode.  norms_in is this
 *                                 forward's isd_propose row_norms (written
 *                                 while its accept test ran beside it), and
 *                                 norms_out the q_norms of the next forward's
 *                                 isd_accept, which verifies the proposals
 *                                 this forward drew.
 *
 * TPF of a request = tokens / forwards.  No workspace; no flags.
 * `forwards` can serve as the step_per_request array of isd_accept and
 * isd_propose: it advances by one per forward on the device, so one forward
 * recorded into a HIP graph draws fresh uniforms on every replay (for a
 * batch whose requests all start together it equals the forward index).
 */
#define ISD_LOOP_VERIFY 0
#define ISD_LOOP_REPROPOSE 1
isd_status isd_loop_advance(const isd_shape* shape, const int32_t* accept_len, const int32_t* n_out,
                            const int32_t* next_proposals, int32_t* n_commit, int32_t* mode,
                            int32_t* proposals, int32_t* positions, int64_t* tokens,
                            int64_t* forwards, const float* norms_in, float* norms_out,
                            hipStream_t stream);

/*
 * isd_lora_delta -- the gated rank-r delta of Residual ISD (R-ISD).
 *
 * Definition ("自省扩散语言模型的 token 生成机制与工程实践", section "Token 生成
 * 的核心参数与验收机制"; I-DLM project page, R-ISD card): an adapter is active
 * at MASK rows only; CLEAN (verifying) rows keep the base weights:
 *
 *   Y[m][:] += scale * (X[m][:] @ A) @ B   for m in mask_rows[0..n_mask-1]
 *
 * The adapter weights are taken in the layouts a linear layer stores them:
 *   X    [rows][d_in]    bf16   input activations of the adapted projection
 *   A_t  [rank][d_in]    bf16   down projection (A transposed)
 *   B_t  [d_out][rank]   bf16   up projection (B transposed)
 *   Y    [rows][d_out]   bf16   base projection output, updated in place at
 *                               the gated rows only (other rows untouched)
 *   mask_rows [n_mask] int32    distinct row indices in [0, rows)
 *
 * bf16 operands on the matrix cores with fp32 accumulation; the rank-r
 * intermediate is summed in fp32 and enters the second product as two bf16
 * terms (value and rounding remainder).  Supported: rank == 128,
 * d_in % 256 == 0, d_out % 128 == 0.  Workspace: at least
 * isd_lora_workspace_bytes() bytes; its first 4 bytes are a flag word
 * (ISD_FLAG_ROW_RANGE: a gated row outside [0, rows) is skipped) that the
 * caller zeroes before the first call.  Rows listed twice race.
 */
size_t isd_lora_workspace_bytes(int32_t n_mask, int32_t d_in, int32_t rank);
isd_status isd_lora_delta(int32_t rows, int32_t d_in, int32_t d_out, int32_t rank, const void* X,
                          const void* A_t, const void* B_t, const int32_t* mask_rows,
                          int32_t n_mask, float scale, void* Y, void* workspace, size_t ws_bytes,
                          hipStream_t stream);

/*
 * isd_gated_linear -- one whole projection of an R-ISD layer: the base
 * weights on every row, plus the rank-r adapter on the MASK rows.
 *
 * Definition ("自省扩散语言模型的 token 生成机制与工程实践", section "Token 生成
 * 的核心参数与验收机制"; I-DLM project page, R-ISD card): the verifying
 * (CLEAN) rows run the base weights alone, which is what keeps their output
 * equal to the base model's; the MASK rows add the gated adapter:
 *
 *   Y[m][:] = X[m][:] @ W + gate[m] * scale * (X[m][:] @ A) @ B
 *
 * with gate[m] = 1 for m in mask_rows[0..n_mask-1], else 0.  Layouts are those
 * a linear layer stores:
 *   X    [rows][d_in]    bf16   input activations
 *   W_t  [d_out][d_in]   bf16   base weight (W transposed)
 *   A_t  [rank][d_in]    bf16   adapter down projection (A transposed)
 *   B_t  [d_out][rank]   bf16   adapter up projection (B transposed)
 *   Y    [rows][d_out]   bf16   output, every element written; must not
 *                               overlap X
 *   mask_rows [n_mask] int32    row indices in [0, rows)
 *
 * rank == 0 runs the base projection alone (A_t, B_t and mask_rows are not
 * read and may be NULL); rank == 128 runs the gated one.  Arithmetic: bf16
 * operands on the matrix cores, fp32 sums, one rounding to bf16 at the end;
 * the adapter's rank-r intermediate is summed in fp32, scaled, and rounded
 * once to bf16 before the second product.  A row outside the gate comes out
 * bit for bit equal to the rank == 0 call's row of the same shape (the sums
 * over W run in an order fixed by (rows, d_in, d_out) alone), provided B_t is
 * finite.
 *
 * Supported: 1 <= rows <= 65536, 256 <= d_in <= 65536 with d_in % 256 == 0,
 * d_out % 128 == 0, rows * d_out <= 2^30, rank in {0, 128}, 0 <= n_mask <=
 * rows, scale not NaN or infinite.  Workspace: at
 * least isd_gated_linear_workspace_bytes() bytes (0 for an unsupported
 * shape); its first 4 bytes are a flag word that the caller zeroes before
 * the first call (ISD_FLAG_ROW_RANGE: a gated row outside [0, rows) is
 * skipped).  A row listed twice is
 * adapted once.  Errors: ISD_ERR_SHAPE, ISD_ERR_UNSUPPORTED, ISD_ERR_NULL,
 * ISD_ERR_ALIGNMENT (every pointer 16-byte aligned), ISD_ERR_WORKSPACE,
 * ISD_ERR_HIP.
 */
size_t isd_gated_linear_workspace_bytes(int32_t rows, int32_t d_in, int32_t d_out, int32_t rank,
                                        int32_t n_mask);
isd_status isd_gated_linear(int32_t rows, int32_t d_in, int32_t d_out, int32_t rank, const void* X,
                            const void* W_t, const void* A_t, const void* B_t, const int32_t* mask_rows,
                            int32_t n_mask, float scale, void* Y, void* workspace, size_t ws_bytes,
                            hipStream_t stream);

/*
 * isd_gated_linear_group -- n_proj (1..4) projections of the same input X
 * and the same gated rows, each as isd_gated_linear defines it:
 *
 *   Y_p[m][:] = X[m][:] @ W_p + gate[m] * scale * (X[m][:] @ A_p) @ B_p
 *
 * (source as isd_gated_linear's).  In a transformer layer the q, k and v
 * projections read the same normed hidden state, and so do the MLP's gate
 * and up projections; one call reads X's gated rows once for all adapters
 * and runs every projection's product in one launch whose output tiles span
 * the group, so narrow members (k, v) fill the chip together with the wide
 * one instead of each splitting its k range alone.
 *
 * d_out, W_t, A_t, B_t and Y are HOST arrays of n_proj entries, read during
 * the call only; the pointers they hold are device pointers with the
 * layouts of isd_gated_linear ([d_out[p]][d_in], [rank][d_in],
 * [d_out[p]][rank], [rows][d_out[p]]).  A_t and B_t may be NULL when
 * rank == 0.  The outputs Y[p] must not overlap each other or X.  With one
 * projection the call is isd_gated_linear (same kernels, same results).
 * The tiling follows the summed width sum_p d_out[p]; a row outside the gate
 * equals the rank == 0 group call's row bit for bit (not necessarily the
 * single-projection call's, whose k split may differ).
 *
 * Supported: 1 <= n_proj <= 4, each d_out[p] % 128 == 0, rows * sum_p
 * d_out[p] <= 2^30, and the limits of isd_gated_linear.  Workspace: at least
 * isd_gated_linear_group_workspace_bytes() bytes (0 for an unsupported
 * shape), flag word as isd_gated_linear's.  Errors: as isd_gated_linear's.
 */
size_t isd_gated_linear_group_workspace_bytes(int32_t n_proj, int32_t rows, int32_t d_in, const int32_t* d_out,
                                              int32_t rank, int32_t n_mask);
isd_status isd_gated_linear_group(int32_t n_proj, int32_t rows, int32_t d_in, const int32_t* d_out, int32_t rank,
                                  const void* X, const void* const* W_t, const void* const* A_t,
                                  const void* const* B_t, const int32_t* mask_rows, int32_t n_mask, float scale,
                                  void* const* Y, void* workspace, size_t ws_bytes, hipStream_t stream);

/* Text for a status code (static storage); `status` is an isd_status value,
 * taken as a plain integer so that any code a caller holds, valid or not, is
 * safe to pass (one outside the enumeration gives "unknown status"). */
const char* isd_status_string(int32_t status);

/* Text of the last ISD_ERR_HIP on the calling thread ("" if none). */
const char* isd_last_error(void);

/* ABI version: bumped on any change of a signature or a layout above. */
int32_t isd_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ISD_H */
