// Host-side launchers of the libtpblock kernels. Each enqueues on `st` and returns the launch
// status; shapes are validated by the caller (tp_api.hip) before any of these run.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpk {

enum ActType { ACT_F32 = 0, ACT_BF16 = 1 };
enum WType { W_F32 = 0, W_BF16 = 1, W_Q8 = 2 };
enum Epilogue { EPI_ACT = 0, EPI_F32 = 1, EPI_BF16 = 2, EPI_GATED = 3, EPI_ROPE = 4,
                EPI_REDUCE = 5, EPI_REDUCE_BF = 6, EPI_RED_ALL = 7, EPI_RED_ALL_BF = 8 };

// Optional timing of one projection by kernel execution (not by stream events): while `stop` is
// set, every launch below goes through hipExtLaunchKernelGGL, the first one also recording
// `start` when it begins and each one recording `stop` when it ends, so the pair spans exactly the
// projection's kernels. Per calling thread; the API sets it around the timed projection only.
struct LaunchTiming {
  hipEvent_t start = nullptr, stop = nullptr;
};
extern thread_local LaunchTiming g_timing;

template <typename F, typename... Args>
inline void launch(F kernel, const dim3& grid, const dim3& block, uint32_t lds, hipStream_t st,
                   Args... args) {
  if (g_timing.stop) {
    hipExtLaunchKernelGGL(kernel, grid, block, lds, st, g_timing.start, g_timing.stop, 0u,
                          args...);
    g_timing.start = nullptr;
  } else {
    hipLaunchKernelGGL(kernel, grid, block, lds, st, args...);
  }
}

// Arguments of the fused QKV epilogue (rotary embedding + paged KV append), passed by value.
struct RopeEpi {
  const int* positions;
  const int* block_table;
  const float* rope;  // [pos_limit or more][hd/2] (cos, sin) pairs
  void* q_out;        // [T][hq * hd]
  void* k_pages;
  void* v_pages;
  int t0;             // first token of this launch's token group
  int mode, max_pages, ps, n_pages, pos_limit, hq, hk, hd;
};

// The replicated work of the one-call block step, folded into the decode GEMVs that border it.
//   Prologue (gamma != NULL; the QKV and gate/up projections): the token rows X are the residual
//     stream and the projection's input is RMSNorm(X) * gamma (fp32, not rounded to the
//     activation dtype); workgroup 0 also stores it, rounded, to normed_out when that is not NULL.
//   EPI_REDUCE / EPI_REDUCE_BF (the o_proj and down projections of the last rank): the partial is
//     stored as with the fp32 / bf16 partial epilogue, and res_out = res_in + (((P_0 + P_1) + ...)
//     + P_{n_prev}) in fp32 with one rounding, P_0..P_{n_prev-1} read from `prev`.
struct FuseArgs {
  const void* gamma;
  float eps;
  void* normed_out;
  const void* prev;
  size_t part_stride;  // elements from one rank's partial to the next
  int n_prev;
  const void* res_in;
  void* res_out;
};

// One launch that covers every rank's share of a step (the one-call decode step), with each
// rank's own pointers. Column-parallel projections (and the decode attention): blocks
// [r * bpr, (r + 1) * bpr) work for rank r with w[r], s[r], y[r] and, under the rotary epilogue,
// the rank's q buffer and KV pool. Row-parallel projections with EPI_RED_ALL / EPI_RED_ALL_BF
// (at most four ranks): every block computes its output rows for all ranks, rank r from its
// input rows x[r] and weight slice w[r]; each rank's partial is stored at y[r] and the partials
// are added in rank order (then the residual, FuseArgs::res_in / res_out), the arithmetic of the
// reduce kernel.
constexpr int kMaxRanks = 8;
struct RankPtrs {
  int n;    // ranks in the launch; 0: a single rank's launch (the plain pointer arguments)
  int bpr;  // blocks per rank of a column-parallel launch
  const void* w[kMaxRanks];
  const uint16_t* s[kMaxRanks];
  const void* x[kMaxRanks];
  void* y[kMaxRanks];
  void* q_out[kMaxRanks];
  void* k_pages[kMaxRanks];
  void* v_pages[kMaxRanks];
  int n_pages[kMaxRanks];
};

// Per-rank operands of a matrix-core GEMM launch over all ranks (grid.z = rank): activations a,
// weights b (gated: b2 the up rows), output c. n = 0: a single rank's launch.
struct GemmRanks {
  int n;
  const void* a[kMaxRanks];
  const void* b[kMaxRanks];
  const void* b2[kMaxRanks];
  void* c[kMaxRanks];
};

// Per-rank buffers of the rotary / KV-append kernel over all ranks (grid.y = rank).
struct RopeRanks {
  int n;
  const float* parts[kMaxRanks];
  void* q_out[kMaxRanks];
  void* k_pages[kMaxRanks];
  void* v_pages[kMaxRanks];
  int n_pages[kMaxRanks];
};

// Per-rank pointers of a decode attention launch over all ranks (blockIdx.y = rank * hk + kv
// head); n = 0: a single rank's launch (the plain pointer arguments).
struct AttnRanks {
  int n;
  const void* q[kMaxRanks];
  const void* k_pages[kMaxRanks];
  const void* v_pages[kMaxRanks];
  int n_pages[kMaxRanks];
  float* part_o[kMaxRanks];
  float* part_ml[kMaxRanks];
  void* out[kMaxRanks];
};

// Raise `kernel`'s dynamic-LDS limit to `bytes` on the current device; done once per (kernel,
// device) and remembered, so launchers may call it before every launch.
hipError_t allow_lds(const void* kernel, int bytes);

// k_pack.hip
hipError_t copy2d(void* dst, size_t dst_ld, const void* src, size_t src_ld, int64_t rows,
                  size_t row_bytes, hipStream_t st);
hipError_t q8_split(const void* aos, size_t aos_ld, int64_t rows, int64_t nblk, void* codes,
                    void* scales, hipStream_t st);
hipError_t q8_join(void* aos, size_t aos_ld, int64_t rows, int64_t nblk, const void* codes,
                   const void* scales, hipStream_t st);
hipError_t q8_dequant_buf(const void* codes, const void* scales, float* out, int64_t n_blocks,
                          hipStream_t st);
hipError_t launch_embed(int wt, const void* table, const void* scales, const int32_t* ids,
                        int T, int vocab, int d, void* x, hipStream_t st);

// k_moe.hip
hipError_t launch_moe_topk(const float* logits, int T, int E, int top_k, int32_t* ids,
                           float* weights, hipStream_t st);
// fuse: the down kernel also adds the earlier ranks' partials and the residual (EPI_REDUCE's
// arithmetic) into fuse->res_out.
hipError_t launch_moe_ffn(int wt, int at, int actf, int pt, const void* Wg, const void* Sg,
                          const void* Wu, const void* Su, const void* Wd, const void* Sd, int d,
                          int Fr, int E, int top_k, int T, const int32_t* ids, const float* wts,
                          const void* X, void* M, void* P, hipStream_t st,
                          const FuseArgs* fuse = nullptr);
// Per-rank operands of the MoE expert projections of every rank in one launch: the rank's gate,
// up and down slices (wg, wu, wd; Q8_0 scales sg, su, sd), its expert activations m
// [T][top_k * Fr] and its partial p [T][d].
struct MoeRanks {
  int n;
  const void* wg[kMaxRanks];
  const void* sg[kMaxRanks];
  const void* wu[kMaxRanks];
  const void* su[kMaxRanks];
  const void* wd[kMaxRanks];
  const void* sd[kMaxRanks];
  void* m[kMaxRanks];
  void* p[kMaxRanks];
};
// The two halves of launch_moe_ffn on their own: the gate/up of every rank in mr (blockIdx.z =
// rank; each block's work exactly that of the rank's own launch) and one rank's down (with the
// reduce epilogue when `fuse` is given). logits (optional, E <= 64): the gate/up selects each
// token's experts from the router logits itself (launch_moe_topk's rule and results) and stores
// the selection in ids and its weights in weights.
hipError_t launch_moe_gate_up_ranks(int wt, int at, int actf, int d, int Fr, int E, int top_k,
                                    int T, const int32_t* ids, const void* X, const MoeRanks& mr,
                                    hipStream_t st, const float* logits = nullptr,
                                    float* weights = nullptr);
hipError_t launch_moe_down(int wt, int at, int pt, const void* Wd, const void* Sd, int d, int Fr,
                           int E, int top_k, int T, const int32_t* ids, const float* wts,
                           const void* M, void* P, hipStream_t st, const FuseArgs* fuse);
// The down of every rank in mr (at most four, dividing four) in one launch with the reduce in
// it: a workgroup's waves take the same output rows for different ranks, each wave's sums
// exactly as in its rank's own launch; every partial is stored at mr.p[r], and out = res +
// (((P_0 + P_1) + ...) + P_{n-1}) with the partials at their stored precision, the reduce
// kernel's arithmetic. moe_down_ranks_fit: whether every rank's activations fit the LDS.
bool moe_down_ranks_fit(int n_ranks, int top_k, int Fr);
hipError_t launch_moe_down_ranks(int wt, int at, int pt, int d, int Fr, int E, int top_k, int T,
                                 const int32_t* ids, const float* wts, const MoeRanks& mr,
                                 const void* res, void* out, hipStream_t st);

// k_reduce.hip
hipError_t launch_partial_reduce(int act, int part, int T, int d, const void* partials, int n,
                                 const void* res_in, void* res_out, const void* gamma,
                                 void* normed, float eps, hipStream_t st);

// k_gemv.hip
int gemv_max_tokens(int K);
hipError_t launch_gemv(int wt, int at, int epi, int actf, int T, const void* W, const void* S,
                       int K, int n_out, int gate_off, const void* X, void* Y, int ldy,
                       const RopeEpi* rope, hipStream_t st, const FuseArgs* fuse = nullptr);
// The same projection for every rank in one launch (RankPtrs; T within one token group):
// column-parallel epilogues (EPI_ROPE, EPI_GATED) with the norm prologue, or the row-parallel
// EPI_RED_ALL / EPI_RED_ALL_BF. gemv_ranks_fit: whether the launch's staged inputs fit the LDS.
bool gemv_ranks_fit(int wt, int epi, int n_ranks, int T, int K);
hipError_t launch_gemv_ranks(int wt, int at, int epi, int actf, int T, const RankPtrs& rp, int K,
                             int n_out, int gate_off, const void* X, int ldy, const RopeEpi* rope,
                             hipStream_t st, const FuseArgs& fuse);

// k_gemm.hip
// Split-K projection of M <= 64 tokens; `part` holds the fp32 split tiles
// (splitk_workspace_bytes), summed in split order by a small epilogue kernel.
size_t splitk_workspace_bytes(int M, int N, int K, bool dual);
// Sum of S fp32 partial tiles [S][M][N] (gated: [S][M][2N], gate then up) in split order, then the
// epilogue into C. gr (optional): every rank in one launch, rank r's tiles at gr->a[r] and its
// output at gr->c[r].
hipError_t launch_splitk_epilogue(int epi, int actf, const float* part, int S, int M, int N,
                                  void* C, int ldc, hipStream_t st, const GemmRanks* gr = nullptr);
// Q8_0 weights (codes [N, K] int8, scales [N, K/32] fp16; gated: B2 = the up rows) for more tokens
// than the GEMV takes; `part` (q8_gemm_workspace_bytes, may be NULL) holds split-K partial tiles.
size_t q8_gemm_workspace_bytes(int M, int N, int K, bool dual);
hipError_t launch_gemm_q8(int epi, int actf, int M, int N, int K, const void* A, const void* Bq,
                          const void* Bs, const void* B2q, const void* B2s, void* C, int ldc,
                          float* part, hipStream_t st);
// The Q8_0 projection of every rank in one launch (grid.z = rank * S + K range): rank r's
// activations a[r], codes and scales q[r], s[r] (gated: the up rows' q2[r], s2[r]), output c[r]
// and partial-tile workspace part[r] (q8_gemm_workspace_bytes; with parts_only at least
// S * M * N floats). Each rank's K ranges are those of its own launch_gemm_q8, so its results are
// the same bits. parts_only: leave the fp32 partial tiles [S][M][N] in part[r] (even for S == 1)
// and return S in *S_out, for the caller to sum; else the all-ranks epilogue runs when S > 1.
struct Q8Ranks {
  int n;
  const void* a[kMaxRanks];
  const void* q[kMaxRanks];
  const void* s[kMaxRanks];
  const void* q2[kMaxRanks];
  const void* s2[kMaxRanks];
  void* c[kMaxRanks];
  float* part[kMaxRanks];
};
int q8_gemm_splits(int M, int N, int K);
hipError_t launch_gemm_q8_ranks(int epi, int actf, int M, int N, int K, const Q8Ranks& gr, int ldc,
                                hipStream_t st, bool parts_only, int* S_out);
// parts_only: launch the GEMM alone, leaving the fp32 partial tiles [S][M][N] (dual: gate then
// up per row) in `part`, and return S there; the caller then sums them.
hipError_t launch_gemm_splitk(int epi, int actf, int M, int N, int K, const void* A,
                              const void* B, const void* B2, void* C, int ldc, float* part,
                              hipStream_t st, int* parts_only = nullptr);
// The direct-to-LDS split-K GEMM of every rank in one launch, partial tiles only (K % 64 == 0):
// rank r reads gr.a[r], gr.b[r] (gr.b2[r]) and writes its S tiles to (float*)gr.c[r]; returns S.
hipError_t launch_gemm_splitk_ranks(int epi, int M, int N, int K, const GemmRanks& gr,
                                    hipStream_t st, int* parts);
hipError_t launch_gemm_bf16(int epi, int actf, int M, int N, int K, const void* A, const void* B,
                            const void* B2, void* C, int ldc, hipStream_t st);
// k_gemm_band.hip: M <= 64 tokens, a 16-column band of the output per workgroup over the whole
// K (no split, epilogue in the kernel); K % 128 == 0 and at least 192 bands.
bool gemm_band_supported(int epi, int M, int N, int K);
hipError_t launch_gemm_band(int epi, int actf, int M, int N, int K, const void* A, const void* B,
                            const void* B2, void* C, int ldc, hipStream_t st,
                            const GemmRanks* gr = nullptr);
// The bf16 QKV projection of M tokens with the rotary embedding and the KV append in its epilogue
// (the 128 or 256-row direct-to-LDS tiles; q goes to re.q_out, k and v into the pages). Supported
// when N % 128 == 0, hd is 64 or 128, K % 64 == 0, M >= 128 and the shape is not one for the
// wide-tile kernel; otherwise the caller projects and then runs launch_rope_append.
bool gemm_rope_supported(int M, int N, int K, int hd);
hipError_t launch_gemm_qkv_rope(int M, int N, int K, const void* A, const void* B,
                                const RopeEpi& re, hipStream_t st);

// k_gemm_wide.hip: 256 x 256 tiles over eight waves (gated: 112 output columns); M >= 256,
// N >= the tile width, K % 64 == 0. gemm_wide_tiles returns the tile count, 0 when the shape
// does not fit.
long gemm_wide_tiles(int epi, int M, int N);
hipError_t launch_gemm_wide(int epi, int actf, int M, int N, int K, const void* A, const void* B,
                            const void* B2, void* C, int ldc, hipStream_t st,
                            const GemmRanks* gr = nullptr);
// Split-K bf16 projection on 256 x 160 tiles writing ksplit fp32 partial products
// ([ksplit][M][N]) for shapes too narrow to fill the chip with whole-K tiles;
// gemm_split_count returns the K ranges to use (1: not worth it).
int gemm_split_count(int M, int N, int K);
hipError_t launch_gemm_split_f32(int M, int N, int K, const void* A, const void* B, float* parts,
                                 int ksplit, hipStream_t st, const GemmRanks* gr = nullptr);

// k_attn.hip
// Rotary embedding + KV append from np (1..16) fp32 partials of the QKV projection (bf16 cache).
hipError_t launch_rope_append_parts(const float* parts, int np, int T, int hq, int hk, int hd,
                                    void* q_out, const int* positions, int mode,
                                    const int* block_table, int max_pages, int ps, int n_pages,
                                    int pos_limit, void* kp, void* vp, const float* rope,
                                    hipStream_t st, const RopeRanks* rr = nullptr);
hipError_t launch_rope_append(int at, const void* qkv, int T, int hq, int hk, int hd, void* q_out,
                              const int* positions, int mode, const int* block_table,
                              int max_pages, int ps, int n_pages, int pos_limit, void* kp,
                              void* vp, const float* rope, hipStream_t st);
// k_attn_prefill.hip: bf16 causal prefill of one sequence, KV tiles shared by a GQA group.
bool attn_prefill_supported(int hd, int G, int ps);
// ar: every rank in one launch (grid.z = rank; q, pages, n_pages, out per rank).
hipError_t launch_attn_prefill(int hd, int G, int T, int hk, const void* q, const void* kp,
                               const void* vp, const int* positions, const int* bt,
                               int max_pages, int n_pages, int pos_limit, void* out,
                               hipStream_t st, const AttnRanks* ar = nullptr);
hipError_t launch_attn_decode(int at, int hd, int G, int T, int hk, const void* q, const void* kp,
                              const void* vp, const int* positions, int mode, const int* bt,
                              int max_pages, int ps, int n_pages, int chunk, int n_split,
                              int pos_limit, float* part_o, float* part_ml, void* out,
                              hipStream_t st);
// Decode attention (mode 0) of every rank in one launch, and one merge launch for all ranks.
hipError_t launch_attn_decode_ranks(int at, int hd, int G, int T, int hk, const AttnRanks& ar,
                                    const int* positions, const int* bt, int max_pages, int ps,
                                    int chunk, int n_split, int pos_limit, hipStream_t st);

}  // namespace tpk
