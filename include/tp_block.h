/*
 * tp_block.h - one rank's share of a Megatron-style tensor-parallel transformer block on one
 * AMD Instinct MI355X (gfx950), with the N-way partial-sum reduce done locally.
 *
 * The operations follow these passages of the source pages:
 *   [TS-HOW]   TensorSharp "Multi-GPU & Multi-Node", section "How tensor parallelism works":
 *              column-parallel QKV and gate/up split the output dim (heads, FFN columns); attention
 *              and the activation run per rank over the owned heads against that rank's own KV
 *              cache; row-parallel o_proj and down split the input dim and emit partial sums; one
 *              all-reduce per block half leaves every rank with the identical hidden state; norms
 *              are replicated.
 *   [TS-REQ]   same page, section "Requirements & constraints": head counts, KV-head counts and
 *              the FFN width must divide by the degree; a block-quantised row-parallel split needs
 *              its input dim divisible by degree x block size.
 *   [ML-PROB]  mlxcel issue #488, section "Problem": the one-device runtime builds every rank's
 *              shard from the full weights, runs the ranks in sequence and sums the partials
 *              locally (reduce_sum).
 *   [ML-ACC]   same issue, section "Acceptance criteria": running tp>1 on one device is legitimate
 *              if it is explicit, and must never give silently wrong results.
 *   [NN-CHG]   nnsight PR #677, section "Change": row-parallel layers split the input dim, the
 *              others the output dim; fused weights keep their rows grouped by rank.
 *   [TS-REP]   TensorSharp, section "How tensor parallelism works", after its three steps: the
 *              norms, the token embeddings and the LM head are not sharded but held whole by every
 *              rank, so they add no collective.
 *   [ML-OOS]   mlxcel issue #488, section "Out of scope": embeddings and LM head stay replicated
 *              (a vocabulary-parallel split is left out).
 *   [TS-MOE]   TensorSharp, section "Supported architectures": with expert slicing each expert
 *              is itself sharded the column/row way (its gate and up projections by output
 *              columns, its down projection by input columns), so a rank keeps 1/N of every
 *              expert, the router is the same on every rank, and the expert ids chosen for a
 *              token mean the same thing everywhere; section "Requirements & constraints": under
 *              tensor parallelism MoE models take one sequence at a time.
 *
 * Conventions for every call:
 *   - All tensors are caller-owned device memory unless stated. The library allocates nothing,
 *     keeps no state between calls and never synchronises the host, except tp_rope_table_init.
 *   - `stream` is a hipStream_t (NULL = the default stream); every launch is asynchronous on it.
 *   - Weights are [out, in] row-major (y = x * W^T). Activations are [tokens, features] row-major.
 *   - Every argument is validated on the host before any launch; a failed call launches nothing
 *     and returns a non-zero tp_status, with details in tp_last_error() (per calling thread).
 *     Unsupported combinations are refused, never silently approximated [ML-ACC].
 *   - Device-side indices (positions, block tables, page ids) are trusted; out-of-range values are
 *     clamped into the buffers they index, so they cannot fault, but give unspecified results.
 */
#ifndef TP_BLOCK_H
#define TP_BLOCK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t tp_status;
enum {
  TP_OK = 0,
  TP_ERR_INVALID_ARG = 1,      /* null pointer, bad enum, non-positive size                    */
  TP_ERR_RANK = 2,             /* rank outside [0, tp_degree)                                  */
  TP_ERR_NOT_DIVISIBLE = 3,    /* heads / kv heads / ffn not divisible by the degree [TS-REQ]  */
  TP_ERR_QUANT_ALIGN = 4,      /* Q8_0 split not on a 32-weight block boundary [TS-REQ]        */
  TP_ERR_BUFFER_TOO_SMALL = 5, /* a caller buffer is smaller than the size query reports       */
  TP_ERR_UNSUPPORTED = 6,      /* a dtype / shape / mode combination this build does not run   */
  TP_ERR_HIP = 7               /* a HIP runtime or launch error                                */
};

enum { TP_DTYPE_F32 = 0, TP_DTYPE_BF16 = 1, TP_DTYPE_Q8_0 = 2 };
enum { TP_ACT_SILU = 0, TP_ACT_GELU_TANH = 1 };
enum { TP_HALF_ATTN = 0, TP_HALF_FFN = 1 };
enum { TP_MODE_DECODE = 0, TP_MODE_PREFILL = 1 };

/* Block shape and numeric formats. Plain data, no pointers.
 * Supported (w_dtype, act_dtype): (F32, F32), (BF16, BF16), (Q8_0, BF16). The KV cache uses the
 * activation dtype. partial_dtype: F32 (default) or BF16. head_dim: 64, 128 or 256.
 * n_heads / n_kv_heads: 1, 2, 4 or 8. rms_eps is added inside the square root; rope_base is the
 * rotary base. max_position bounds every position (size of the rotary table). */
typedef struct {
  int32_t d_model, n_heads, n_kv_heads, head_dim, ffn_dim, tp_degree, page_size, max_position;
  float rms_eps, rope_base;
  int32_t w_dtype, act_dtype, partial_dtype, ffn_act;
} tp_block_desc;

typedef struct {
  uint64_t offset, bytes;
} tp_region;

/* Where rank r's slices live inside its packed shard buffer (offsets 256-byte aligned).
 *   qkv     [(Hq/N + 2 Hkv/N) * hd, d]: Wq rows of the owned query heads, then Wk rows, then Wv
 *           rows of the owned KV heads (column-parallel, rows grouped by rank [NN-CHG]).
 *   o       [d, Hq/N * hd]: the Wo columns of the owned query heads (row-parallel).
 *   gate_up [2 F/N, d]: the Wg rows of the owned FFN columns, then the Wu rows.
 *   down    [d, F/N]: the Wd columns of the owned FFN columns (row-parallel).
 * For Q8_0 these regions hold the int8 codes ([out, in], one byte per weight) and the *_scale
 * regions the fp16 block scales ([out, in/32]); for other dtypes *_scale.bytes is 0.
 * payload_bytes is exactly 1/N of the full block's weight bytes; alloc_bytes adds alignment. */
typedef struct {
  tp_region qkv, o, gate_up, down;
  tp_region qkv_scale, o_scale, gate_up_scale, down_scale;
  uint64_t payload_bytes, alloc_bytes;
} tp_shard_layout;

/* Full (unsharded) weights, device pointers, [out, in] row-major:
 * wq [Hq*hd, d], wk and wv [Hkv*hd, d], wo [d, Hq*hd], wg and wu [F, d], wd [d, F].
 * F32 / BF16: plain elements. Q8_0: per row, in/32 blocks of 34 bytes (fp16 scale, 32 int8). */
typedef struct {
  const void *wq, *wk, *wv, *wo, *wg, *wu, *wd;
} tp_full_weights;

/* One step's token batch. Device arrays: positions [n_tokens]; seq_lens [n_seqs] (keys attended by
 * the sequence's last token, new tokens included); block_table [n_seqs, max_pages] (physical page
 * of every page_size-token page). rope_table: the table tp_rope_table_init filled.
 * DECODE: one new token per sequence, token b belongs to sequence b (n_tokens == n_seqs).
 * PREFILL: n_seqs == 1; all tokens belong to sequence 0.
 * Token t attends the keys at positions 0..positions[t] of its sequence (causal).
 * max_seq_len (host value): an upper bound of positions[t] + 1 over the batch, at most
 * max_pages * page_size and max_position; it sizes the split-KV grid. */
typedef struct {
  int32_t mode, n_tokens, n_seqs, max_pages, max_seq_len;
  const int32_t* positions;
  const int32_t* seq_lens;
  const int32_t* block_table;
  const float* rope_table;
} tp_batch;

/* Rank r's paged KV cache, holding only the KV heads rank r owns [TS-HOW], activation dtype:
 * k_pages [n_pages][Hkv/N][page_size][hd] (after the rotary embedding) and v_pages stored
 * transposed, [n_pages][Hkv/N][hd][page_size], so that 8 consecutive keys of one hd column are
 * contiguous (the B operand layout of the P.V matrix-core step). Slots no key has been written to
 * (past a sequence's last position, pages a block-table entry points at beyond a sequence's own)
 * may hold anything, NaN and Inf included: the attention kernels never let such a slot reach the
 * output [ML-ACC], so recycled pages need no clearing. */
typedef struct {
  void* k_pages;
  void* v_pages;
  int32_t n_pages;
} tp_kv_cache;

/* Fill `out` with rank r's packed-shard layout. Host only; runs the full shape validation
 * ([TS-REQ] divisibility and Q8_0 block alignment). */
tp_status tp_shard_weights_size(const tp_block_desc* desc, int32_t rank, tp_shard_layout* out);

/* Build rank r's shard from the full weights (the from_full_weights step of [ML-PROB]): copy its
 * slices [TS-HOW] into `dst` (device, dst_bytes >= alloc_bytes) in the layout above. Q8_0 blocks
 * are split into codes and scales. Norm weights are not sharded: callers pass the replicated
 * gamma directly to tp_partial_reduce. */
tp_status tp_shard_weights(const tp_block_desc* desc, int32_t rank, const tp_full_weights* src,
                           void* dst, uint64_t dst_bytes, void* stream);

/* Bytes of workspace tp_block_shard_forward needs for this batch (either half). */
tp_status tp_workspace_size(const tp_block_desc* desc, const tp_batch* batch, uint64_t* bytes);

/* How tp_block_step (and the attention half of tp_moe_block_step) runs a batch. */
enum {
  TP_SCHEDULE_STAGED = 0,     /* the separate calls, rank after rank */
  TP_SCHEDULE_PER_RANK = 1,   /* norms and reduces folded into each rank's decode GEMVs */
  TP_SCHEDULE_ALL_RANKS = 2   /* as PER_RANK, each projection / attention one launch for all */
};
tp_status tp_step_schedule(const tp_block_desc* desc, const tp_batch* batch, int32_t* schedule);

/* Bytes of workspace tp_block_step and tp_moe_block_step need for this batch:
 * tp_workspace_size, times tp_degree (each copy 256-byte aligned) under TP_SCHEDULE_ALL_RANKS. */
tp_status tp_step_workspace_size(const tp_block_desc* desc, const tp_batch* batch,
                                 uint64_t* bytes);

/* Bytes of the rotary table: max_position * head_dim/2 pairs of fp32 (cos, sin). */
tp_status tp_rope_table_bytes(const tp_block_desc* desc, uint64_t* bytes);

/* Fill the rotary table: entry [p][i] = (cos, sin)(p * rope_base^(-2i/head_dim)), computed on the
 * host in fp64, rounded to fp32 and copied to `dev_table`. Synchronises `stream`. */
tp_status tp_rope_table_init(const tp_block_desc* desc, void* dev_table, uint64_t table_bytes,
                             void* stream);

/* One rank's share of one block half [TS-HOW], given the replicated normed input xn [T, d]
 * (activation dtype):
 *   ATTN: qkv_r = xn W_qkv,r^T; rotary embedding of q and k at the token positions; K and V of the
 *         new tokens written into rank r's cache `kv`; causal attention of every owned query head
 *         over its KV head (group = head / (Hq/Hkv)); partial_out = a_r W_o,r^T.
 *   FFN:  [g ; u] = xn W_gu,r^T; m_r = act(g) * u; partial_out = m_r W_down,r^T.
 * partial_out is [T, d] in partial_dtype; only it, the workspace and (ATTN) `kv` are written.
 * workspace: device, at least tp_workspace_size bytes. n_tokens == 0 is a no-op. */
tp_status tp_block_shard_forward(const tp_block_desc* desc, int32_t rank, int32_t half,
                                 const void* shard, const tp_batch* batch, const void* xn,
                                 const tp_kv_cache* kv, void* partial_out, void* workspace,
                                 uint64_t workspace_bytes, void* stream);

/* Measurement variant of tp_block_shard_forward: the same work, with the kernels of the half's
 * dominant weight stream (ATTN: the QKV projection; FFN: the gate/up projection) launched through
 * hipExtLaunchKernel so that ev_begin is recorded when the first of them starts executing and
 * ev_end when the last of them finishes: hipEventElapsedTime(ev_begin, ev_end) is that
 * projection's kernel time, as a profiler's kernel trace would report it, without the stream's
 * dispatch gaps. The events are caller-created hipEvent_t handles (ev_end NULL: no timing).
 * Not for graph capture. */
tp_status tp_block_shard_forward_timed(const tp_block_desc* desc, int32_t rank, int32_t half,
                                       const void* shard, const tp_batch* batch, const void* xn,
                                       const tp_kv_cache* kv, void* partial_out, void* workspace,
                                       uint64_t workspace_bytes, void* stream, void* ev_begin,
                                       void* ev_end);

/* For callers that cannot allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): tp_block_shard_forward with its workspace taken from a static
 * device array of the library, 16 MiB per GPU (enough for every decode and 64-token batched-decode
 * shape of the workloads here), obtained once per device on the first call there and held until
 * the process ends. The call allocates nothing. A batch whose workspace (tp_workspace_size) is
 * larger returns TP_ERR_BUFFER_TOO_SMALL before anything is launched. Every call on one GPU
 * shares that array: calls that may overlap on one GPU (several streams, several threads) race
 * and must be serialised by the caller. No part of the array needs to start at zero. */
tp_status tp_block_shard_forward_noalloc(const tp_block_desc* desc, int32_t rank, int32_t half,
                                         const void* shard, const tp_batch* batch, const void* xn,
                                         const tp_kv_cache* kv, void* partial_out, void* stream);

/* One whole block step for all N ranks in one call [ML-PROB] [TS-HOW]:
 *   xn = RMSNorm(x) gamma1;  P_r = ATTN half of rank r (r = 0..N-1);
 *   h1 = x + (((P_0 + P_1) + ...) + P_{N-1});  xn2 = RMSNorm(h1) gamma2;
 *   P_r = FFN half of rank r;  out = h1 + (((P_0 + P_1) + ...) + P_{N-1}),
 * as tp_partial_reduce and tp_block_shard_forward called in that order compute it. When every
 * projection of the step is one decode GEMV launch (at most four tokens, and no more than the
 * GEMV takes at each row length), the call saves three launches per step: each rank's QKV and
 * gate/up projections normalise the residual stream themselves (the projection takes
 * gamma * x and scales its sums by 1/sqrt(mean(x^2) + eps), so the normed input is not rounded
 * to the activation dtype first, as the separate calls round it; xn and xn2 are still stored,
 * rounded), and the last rank's o_proj and down projections add all ranks' partials in rank
 * order plus the residual, with the reduce's arithmetic. Every rank's partial is still stored.
 * When, in addition, every rank's inputs of a projection fit one workgroup's LDS (1 < N <= 4), each
 * projection and the attention run as one launch for all ranks (TP_SCHEDULE_ALL_RANKS: six
 * launches per step, seven with the attention's split merge counted): every block of a
 * column-parallel launch works for one rank with that rank's slice and cache, and every block
 * of a row-parallel launch computes its rows for rank 0, 1, ... in turn, each rank's sums exactly
 * as in that rank's own launch, then adds the partials in rank order and the residual. The
 * results equal the per-rank schedule's bit for bit. Batched decode (5 to 64 tokens) whose
 * projections all take the split-K QKV and the band GEMMs (bf16) or the Q8_0 matrix-core GEMM
 * (Q8_0, whose QKV has at most 16 K ranges), bf16 prefill whose QKV takes the split-K wide
 * tiles and whose other projections take the 256 x 256 wide tiles, and Q8_0 prefill on the
 * matrix-core GEMM (head dims the prefill attention takes), also get
 * TP_SCHEDULE_ALL_RANKS: the separate calls' sequence with each projection (with its split-K
 * epilogue), the rotary / KV append and the attention as one launch for all ranks (under one
 * launch the causal prefill's long and short row blocks of all ranks share the chip). The
 * launches are sized for all ranks' work together, so three choices differ from the separate
 * calls': a prefill QKV whose tiles of all ranks fill the chip is not split over K; the bf16
 * batched QKV splits K into fewer ranges; the batched attention splits each sequence's keys into
 * fewer ranges (often none). (The Q8_0 projections keep each rank's K ranges; their QKV tiles are
 * summed in the same order by the rotary kernel.) Each changes only the order of fp32 additions
 * before a rounding: q, k, v, the attention output and so the rest of the step equal the separate
 * calls' to rounding, not bit for bit.
 * Otherwise (TP_SCHEDULE_STAGED)
 * the call issues exactly the separate calls above. tp_step_schedule reports which schedule a
 * batch gets.
 * shards, kv: host arrays of N entries (rank r's packed shard, device pointer; rank r's cache).
 * x, gamma1, gamma2 (inputs) and xn, h1, xn2, out: activation dtype, [T, d] ([d] for the gammas);
 * partials: [N, T, d] in partial_dtype (holds the FFN partials on return). workspace: at least
 * tp_step_workspace_size bytes (TP_ERR_BUFFER_TOO_SMALL otherwise; under the all-ranks schedule
 * it holds one copy of the per-rank workspace per rank). n_tokens == 0 is a no-op. */
tp_status tp_block_step(const tp_block_desc* desc, const void* const* shards, const tp_batch* batch,
                        const tp_kv_cache* kv, const void* x, const void* gamma1,
                        const void* gamma2, void* partials, void* xn, void* h1, void* xn2,
                        void* out, void* workspace, uint64_t workspace_bytes, void* stream);

/* tp_block_step with the schedule chosen by the caller (TP_SCHEDULE_*; -1: the call's own
 * choice, as tp_block_step). A schedule the batch does not allow (any above what
 * tp_step_schedule reports) returns TP_ERR_UNSUPPORTED before anything is launched. The staged
 * and per-rank schedules need only tp_workspace_size bytes of workspace. */
tp_status tp_block_step_with_schedule(const tp_block_desc* desc, int32_t schedule,
                                      const void* const* shards, const tp_batch* batch,
                                      const tp_kv_cache* kv, const void* x, const void* gamma1,
                                      const void* gamma2, void* partials, void* xn, void* h1,
                                      void* xn2, void* out, void* workspace,
                                      uint64_t workspace_bytes, void* stream);

/* Measurement variant of tp_block_step: ev_begin / ev_end bracket the gate/up projection of rank
 * timed_rank as in tp_block_shard_forward_timed (under TP_SCHEDULE_ALL_RANKS: the one gate/up
 * launch of all ranks, for any timed_rank in [0, N)). Not for graph capture. */
tp_status tp_block_step_timed(const tp_block_desc* desc, const void* const* shards,
                              const tp_batch* batch, const tp_kv_cache* kv, const void* x,
                              const void* gamma1, const void* gamma2, void* partials, void* xn,
                              void* h1, void* xn2, void* out, void* workspace,
                              uint64_t workspace_bytes, void* stream, int32_t timed_rank,
                              void* ev_begin, void* ev_end);

/* The local copy-and-reduce step [ML-PROB] that stands in for the all-reduce [TS-HOW]:
 *   residual_out[t] = residual_in[t] + (((P_0[t] + P_1[t]) + ...) + P_{n-1}[t])
 * summed in fp32 in rank order (the partials first, then the residual) and rounded once to the
 * activation dtype; then, if gamma is not NULL, normed_out = RMSNorm(residual_out) * gamma over
 * d_model (fp32 math on the stored, rounded values).
 * partials: [n_partials, n_tokens, d] in partial_dtype. residual_in/out, gamma, normed_out:
 * activation dtype, [n_tokens, d] ([d] for gamma). residual_out may alias residual_in.
 * n_partials == 0 gives a pure RMSNorm of residual_in (partials and residual_out may be NULL).
 * n_tokens == 0 is a no-op. */
tp_status tp_partial_reduce(const tp_block_desc* desc, int32_t n_tokens, const void* partials,
                            int32_t n_partials, const void* residual_in, void* residual_out,
                            const void* gamma, void* normed_out, void* stream);

/* ---- the replicated model head around a stack of blocks [TS-REP] [ML-OOS] ----
 * One packed table of vocab rows x d_model serves the token-embedding lookup and the LM head
 * (tied embeddings; untied models pack two tables). Its layout, 256-byte aligned regions:
 *   table        [vocab, d] in w_dtype; for Q8_0 the int8 codes, one byte per weight;
 *   table_scale  Q8_0 only: the fp16 block scales [vocab, d/32] (bytes = 0 otherwise). */
typedef struct {
  tp_region table, table_scale;
  uint64_t payload_bytes, alloc_bytes;
} tp_head_layout;

/* Fill `out` with the packed head layout for `vocab` rows (vocab > 0). Host only. */
tp_status tp_head_size(const tp_block_desc* desc, int32_t vocab, tp_head_layout* out);

/* Pack a full table `src` (device, [vocab, d] row-major in w_dtype; Q8_0: d/32 blocks of 34 bytes
 * per row, fp16 scale then 32 int8) into `dst` (device, dst_bytes >= alloc_bytes). */
tp_status tp_head_pack(const tp_block_desc* desc, int32_t vocab, const void* src, void* dst,
                       uint64_t dst_bytes, void* stream);

/* Token-embedding lookup: x_out[t] = row token_ids[t] of the packed table, in the activation
 * dtype ([n_tokens, d], 16-byte aligned). F32 / BF16 rows are copied bit for bit; Q8_0 rows are
 * dequantised (scale * code, exact in fp32) and rounded once to bf16 (nearest even).
 * token_ids: device int32 [n_tokens]; ids outside [0, vocab) are clamped. n_tokens == 0 is a
 * no-op. */
tp_status tp_embed_lookup(const tp_block_desc* desc, int32_t vocab, const void* head,
                          const int32_t* token_ids, int32_t n_tokens, void* x_out, void* stream);

/* LM head: logits[t, v] = sum_k xn[t, k] * table[v, k] (fp32 accumulation, fp32 logits
 * [n_tokens, vocab]). xn is the final RMSNorm of the stack's output (tp_partial_reduce with no
 * partials), activation dtype [n_tokens, d]. Few tokens stream the table through the GEMV; BF16
 * with more tokens runs the matrix-core GEMM. n_tokens == 0 is a no-op. */
tp_status tp_lm_head(const tp_block_desc* desc, int32_t vocab, const void* head, const void* xn,
                     int32_t n_tokens, float* logits, void* stream);

/* ---- expert-sliced mixture-of-experts FFN half [TS-MOE] ----
 * Replaces the dense FFN half: n_experts experts of width expert_ffn, each gated like the dense
 * FFN (desc->ffn_act), top_k of them per token (1 <= top_k <= min(n_experts, 16),
 * n_experts <= 1024). expert_ffn must divide by tp_degree, expert_ffn / tp_degree by 8, and for
 * Q8_0 expert_ffn by 32 * tp_degree (the row-parallel down split on block boundaries [TS-REQ]).
 * desc->ffn_dim is not used by these calls. */
typedef struct {
  int32_t n_experts, top_k, expert_ffn;
} tp_moe_desc;

/* Full expert weights, device, w_dtype as tp_full_weights: wg and wu [n_experts * expert_ffn, d]
 * (expert-major rows), wd [n_experts * d, expert_ffn]. */
typedef struct {
  const void *wg, *wu, *wd;
} tp_moe_full_weights;

/* Rank r's expert shard, 256-byte aligned regions: gate and up [n_experts][expert_ffn/N][d] (the
 * rank's gate and up rows of every expert), down [n_experts][d][expert_ffn/N] (its columns of every
 * expert's down rows); Q8_0 code planes, with the fp16 scale planes in *_scale. payload_bytes is
 * exactly 1/N of the experts' weight bytes (the router is replicated, not sharded). */
typedef struct {
  tp_region gate, up, down, gate_scale, up_scale, down_scale;
  uint64_t payload_bytes, alloc_bytes;
} tp_moe_layout;

tp_status tp_moe_shard_size(const tp_block_desc* desc, const tp_moe_desc* moe, int32_t rank,
                            tp_moe_layout* out);

/* Pack rank r's expert slices from the full expert weights into `dst` (device). */
tp_status tp_moe_shard_weights(const tp_block_desc* desc, const tp_moe_desc* moe, int32_t rank,
                               const tp_moe_full_weights* src, void* dst, uint64_t dst_bytes,
                               void* stream);

/* The replicated router, computed once for all ranks: logits [T, n_experts] (fp32) =
 * xn . router^T with router [n_experts, d] in the activation dtype; then per token the top_k
 * experts by logit, largest first (equal logits: lower index first), into topk_ids [T, top_k]
 * (int32), and their weights, the softmax of the selected logits, into topk_weights [T, top_k]
 * (fp32). A NaN logit ranks as -inf, below every number (so it is chosen only when fewer than
 * top_k logits are numbers, with weight 0 unless every selected logit is -inf or NaN).
 * n_tokens == 0 is a no-op. */
tp_status tp_moe_route(const tp_block_desc* desc, const tp_moe_desc* moe, const void* router,
                       const void* xn, int32_t n_tokens, float* logits, int32_t* topk_ids,
                       float* topk_weights, void* stream);

/* Workspace bytes of tp_moe_shard_forward for n_tokens tokens. */
tp_status tp_moe_workspace_size(const tp_block_desc* desc, const tp_moe_desc* moe,
                                int32_t n_tokens, uint64_t* bytes);

/* Rank r's MoE FFN half: for every token t and selected expert j (e = topk_ids[t, j]),
 * m = act(xn[t] . Wg_e[F_r]^T) * (xn[t] . Wu_e[F_r]^T) over the rank's slice F_r of the expert,
 * partial_out[t] = sum_j topk_weights[t, j] * (m . Wd_e[:, F_r]^T) ([T, d], partial_dtype). Expert
 * ids outside [0, n_experts) are clamped. n_tokens == 0 is a no-op. */
tp_status tp_moe_shard_forward(const tp_block_desc* desc, const tp_moe_desc* moe, int32_t rank,
                               const void* shard, const void* xn, int32_t n_tokens,
                               const int32_t* topk_ids, const float* topk_weights,
                               void* partial_out, void* workspace, uint64_t workspace_bytes,
                               void* stream);

/* Measurement variant: ev_begin / ev_end span the two expert kernels, as for
 * tp_block_shard_forward_timed. Not for graph capture. */
tp_status tp_moe_shard_forward_timed(const tp_block_desc* desc, const tp_moe_desc* moe,
                                     int32_t rank, const void* shard, const void* xn,
                                     int32_t n_tokens, const int32_t* topk_ids,
                                     const float* topk_weights, void* partial_out,
                                     void* workspace, uint64_t workspace_bytes, void* stream,
                                     void* ev_begin, void* ev_end);

/* One whole MoE block step for all N ranks in one call: the attention halves as in
 * tp_block_step, h1 and xn2 = RMSNorm(h1) gamma2, the replicated router (tp_moe_route), every
 * rank's expert half (tp_moe_shard_forward) and out = h1 + (((P_0 + P_1) + ...) + P_{N-1}).
 * For decode batches whose dense projections are single GEMV launches the norms and reduces are
 * folded into the neighbouring projections as in tp_block_step (the router's input is the
 * unrounded norm of h1; xn2 is stored rounded for the experts), saving three launches, and the
 * attention halves run as one launch per projection for all ranks under TP_SCHEDULE_ALL_RANKS;
 * otherwise the separate calls run. shards (dense attention shards), moe_shards, kv: host arrays
 * of N entries. Buffers as in tp_block_step and tp_moe_route; workspace: tp_step_workspace_size
 * bytes, moe_workspace: at least tp_moe_workspace_size bytes (16-byte aligned); with N times
 * that, a decode step whose norms and reduces are folded runs every rank's expert gate/up
 * projection as one launch (rank r's activations in the r-th share; with at most 64 experts
 * that launch also selects the experts from the logits, by tp_moe_route's rule and with the same
 * ids and weights, so no separate top-k launch runs), and, for at most four
 * ranks whose activations fit one workgroup's LDS, every rank's expert down as one launch whose
 * workgroups add the ranks' partials in rank order and the residual; each rank's sums are those
 * of its own launch and every partial is still stored, so the results are the same bits.
 * n_tokens == 0 is a no-op. */
tp_status tp_moe_block_step(const tp_block_desc* desc, const tp_moe_desc* moe,
                            const void* const* shards, const void* const* moe_shards,
                            const tp_batch* batch, const tp_kv_cache* kv, const void* x,
                            const void* gamma1, const void* gamma2, const void* router,
                            void* partials, void* xn, void* h1, void* xn2, void* out,
                            float* logits, int32_t* topk_ids, float* topk_weights,
                            void* workspace, uint64_t workspace_bytes, void* moe_workspace,
                            uint64_t moe_workspace_bytes, void* stream);

/* Measurement variant of tp_moe_block_step (the same launches and results): ev_begin / ev_end
 * (hipEvent_t, non-NULL, else TP_ERR_INVALID_ARG) bracket the expert gate/up launch of every
 * rank when the step takes the all-ranks expert launches described above, and otherwise rank 0's
 * expert half as in tp_moe_shard_forward_timed. Not for graph capture. */
tp_status tp_moe_block_step_timed(const tp_block_desc* desc, const tp_moe_desc* moe,
                                  const void* const* shards, const void* const* moe_shards,
                                  const tp_batch* batch, const tp_kv_cache* kv, const void* x,
                                  const void* gamma1, const void* gamma2, const void* router,
                                  void* partials, void* xn, void* h1, void* xn2, void* out,
                                  float* logits, int32_t* topk_ids, float* topk_weights,
                                  void* workspace, uint64_t workspace_bytes, void* moe_workspace,
                                  uint64_t moe_workspace_bytes, void* stream, void* ev_begin,
                                  void* ev_end);

const char* tp_status_str(tp_status status);
/* Detail of the calling thread's last failure ("" if none). */
const char* tp_last_error(void);

/* ---- test helpers: they run the same device index and dequant code as the hot path ---- */

/* Scatter rank r's packed shard back to full-size logical matrices (device, same formats as
 * tp_shard_weights' input); every element outside rank r's slices is left untouched. */
tp_status tp_shard_unpack(const tp_block_desc* desc, int32_t rank, const void* shard,
                          const tp_full_weights* dst, void* stream);

/* Dequantise n_blocks Q8_0 blocks held as codes [n_blocks*32] int8 and scales [n_blocks] fp16
 * into out [n_blocks*32] fp32: out = float(scale) * code. */
tp_status tp_dequant_q8_0(const void* codes, const void* scales, float* out, uint64_t n_blocks,
                          void* stream);

/* One projection of rank r's packed shard exactly as tp_block_shard_forward runs it, with the fp32
 * output epilogue of the row-parallel partials: out[t, o] = sum_k x[t, k] W[o, k], fp32
 * [n_tokens, rows], for W the region `which` of `shard` taken as a plain [rows, K] matrix:
 * 0 = qkv [(Hq/N + 2 Hkv/N) hd, d], 1 = o [d, Hq/N hd], 2 = gate_up [2 F/N, d] (gate rows, then
 * up rows), 3 = down [d, F/N]. x is [n_tokens, K] in the activation dtype. The token count picks
 * the kernel as in the forward path (for Q8_0: the dequantising GEMV up to four tokens, the
 * matrix-core Q8_0 GEMM beyond, split over K when its tiles do not fill the chip). With one-hot
 * rows of x the result is the region's weights as the kernels dequantise them, which a test
 * compares bit for bit with d * q ([TS-REQ], block-quantised weights). workspace: device, at
 * least tp_shard_project_workspace_size bytes (may be NULL when that size is 256 or less). */
tp_status tp_shard_project(const tp_block_desc* desc, int32_t which, const void* shard,
                           const void* x, int32_t n_tokens, float* out, void* workspace,
                           uint64_t workspace_bytes, void* stream);
tp_status tp_shard_project_workspace_size(const tp_block_desc* desc, int32_t which,
                                          int32_t n_tokens, uint64_t* bytes);

/* Byte offsets, inside the workspace, of the intermediates of the last forward call with this
 * desc/batch: post-rotary q [T, Hq/N*hd], attention output a_r [T, Hq/N*hd] (activation dtype),
 * and the FFN activation m_r [T, F/N] (activation dtype). */
tp_status tp_workspace_offsets(const tp_block_desc* desc, const tp_batch* batch,
                               uint64_t* q_offset, uint64_t* attn_offset, uint64_t* ffn_offset);

#ifdef __cplusplus
}
#endif
#endif /* TP_BLOCK_H */
