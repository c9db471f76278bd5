// libtpblock C ABI: validation, shard and workspace layouts, and the launch sequences of one rank's
// block half and of the local partial-sum reduce. See include/tp_block.h for the contract.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/tp_block.h"
#include "tp_kernels.h"

namespace tpk {
thread_local LaunchTiming g_timing;

hipError_t allow_lds(const void* kernel, int bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static std::mutex mu;
  static std::map<std::pair<const void*, int>, int> done;  // (kernel, device) -> bytes allowed
  std::lock_guard<std::mutex> lock(mu);
  auto it = done.find({kernel, dev});
  if (it != done.end() && it->second >= bytes) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done[{kernel, dev}] = bytes;
  return e;
}
}

namespace {

thread_local std::string g_err;

tp_status fail(tp_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

tp_status hip_fail(hipError_t e, const char* where) {
  return fail(TP_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

constexpr uint64_t kAlign = 256;
uint64_t align_up(uint64_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Dims {
  int d, Hq, Hkv, hd, F, N, ps, maxpos;
  int hq, hk, fr, qdim, qkv_rows;
  int wt, at, pt, actf;
  float eps, base;
  int wb;  // bytes per weight element (Q8_0: one code byte; scales are separate)
  int ab;  // bytes per activation element
};

tp_status check_desc(const tp_block_desc* desc, Dims* o) {
  if (!desc) return fail(TP_ERR_INVALID_ARG, "desc is NULL");
  const tp_block_desc& D = *desc;
  if (D.d_model <= 0 || D.n_heads <= 0 || D.n_kv_heads <= 0 || D.head_dim <= 0 ||
      D.ffn_dim <= 0 || D.tp_degree <= 0 || D.page_size <= 0 || D.max_position <= 0)
    return fail(TP_ERR_INVALID_ARG,
                "dimensions must be positive (d_model=%d n_heads=%d n_kv_heads=%d head_dim=%d "
                "ffn_dim=%d tp_degree=%d page_size=%d max_position=%d)",
                D.d_model, D.n_heads, D.n_kv_heads, D.head_dim, D.ffn_dim, D.tp_degree,
                D.page_size, D.max_position);
  if (!(D.rms_eps >= 0.f) || !std::isfinite(D.rms_eps))
    return fail(TP_ERR_INVALID_ARG, "rms_eps must be finite and >= 0");
  if (!(D.rope_base > 0.f) || !std::isfinite(D.rope_base))
    return fail(TP_ERR_INVALID_ARG, "rope_base must be finite and > 0");
  if (D.w_dtype < TP_DTYPE_F32 || D.w_dtype > TP_DTYPE_Q8_0)
    return fail(TP_ERR_INVALID_ARG, "unknown w_dtype %d", D.w_dtype);
  if (D.act_dtype != TP_DTYPE_F32 && D.act_dtype != TP_DTYPE_BF16)
    return fail(TP_ERR_INVALID_ARG, "act_dtype must be F32 or BF16 (got %d)", D.act_dtype);
  if (D.partial_dtype != TP_DTYPE_F32 && D.partial_dtype != TP_DTYPE_BF16)
    return fail(TP_ERR_INVALID_ARG, "partial_dtype must be F32 or BF16 (got %d)", D.partial_dtype);
  if (D.ffn_act != TP_ACT_SILU && D.ffn_act != TP_ACT_GELU_TANH)
    return fail(TP_ERR_INVALID_ARG, "unknown ffn_act %d", D.ffn_act);
  const bool combo_ok = (D.w_dtype == TP_DTYPE_F32 && D.act_dtype == TP_DTYPE_F32) ||
                        (D.w_dtype == TP_DTYPE_BF16 && D.act_dtype == TP_DTYPE_BF16) ||
                        (D.w_dtype == TP_DTYPE_Q8_0 && D.act_dtype == TP_DTYPE_BF16);
  if (!combo_ok)
    return fail(TP_ERR_UNSUPPORTED,
                "weight/activation dtypes (%d, %d) are not built; supported: (F32, F32), "
                "(BF16, BF16), (Q8_0, BF16)",
                D.w_dtype, D.act_dtype);
  const int N = D.tp_degree;
  if (D.n_heads % N || D.n_kv_heads % N || D.ffn_dim % N)
    return fail(TP_ERR_NOT_DIVISIBLE,
                "n_heads=%d, n_kv_heads=%d and ffn_dim=%d must all divide by tp_degree=%d",
                D.n_heads, D.n_kv_heads, D.ffn_dim, N);
  if (D.n_heads % D.n_kv_heads)
    return fail(TP_ERR_NOT_DIVISIBLE, "n_heads=%d must be a multiple of n_kv_heads=%d", D.n_heads,
                D.n_kv_heads);
  if (D.w_dtype == TP_DTYPE_Q8_0) {
    if (D.d_model % 32)
      return fail(TP_ERR_QUANT_ALIGN, "Q8_0 needs d_model %% 32 == 0 (d_model=%d)", D.d_model);
    if ((D.n_heads * D.head_dim) % (N * 32))
      return fail(TP_ERR_QUANT_ALIGN,
                  "Q8_0 row-parallel o_proj split needs n_heads*head_dim=%d divisible by "
                  "tp_degree*32=%d",
                  D.n_heads * D.head_dim, N * 32);
    if (D.ffn_dim % (N * 32))
      return fail(TP_ERR_QUANT_ALIGN,
                  "Q8_0 row-parallel down split needs ffn_dim=%d divisible by tp_degree*32=%d",
                  D.ffn_dim, N * 32);
  }
  const int G = D.n_heads / D.n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(TP_ERR_UNSUPPORTED, "n_heads/n_kv_heads=%d: built for 1, 2, 4 or 8", G);
  if (D.head_dim != 64 && D.head_dim != 128 && D.head_dim != 256)
    return fail(TP_ERR_UNSUPPORTED, "head_dim=%d: built for 64, 128 or 256", D.head_dim);
  if (D.page_size % 16)
    return fail(TP_ERR_UNSUPPORTED, "page_size=%d: must be a multiple of 16", D.page_size);
  const int fr = D.ffn_dim / N;
  if (D.d_model % 8 || fr % 8)
    return fail(TP_ERR_UNSUPPORTED,
                "d_model=%d and ffn_dim/tp_degree=%d must be multiples of 8 (16-byte vectors)",
                D.d_model, fr);
  if (D.d_model > 16384)
    return fail(TP_ERR_UNSUPPORTED, "d_model=%d: built for at most 16384", D.d_model);
  Dims& x = *o;
  x.d = D.d_model; x.Hq = D.n_heads; x.Hkv = D.n_kv_heads; x.hd = D.head_dim; x.F = D.ffn_dim;
  x.N = N; x.ps = D.page_size; x.maxpos = D.max_position;
  x.hq = D.n_heads / N; x.hk = D.n_kv_heads / N; x.fr = fr;
  x.qdim = x.hq * x.hd; x.qkv_rows = (x.hq + 2 * x.hk) * x.hd;
  x.wt = D.w_dtype; x.at = D.act_dtype; x.pt = D.partial_dtype; x.actf = D.ffn_act;
  x.eps = D.rms_eps; x.base = D.rope_base;
  x.wb = D.w_dtype == TP_DTYPE_F32 ? 4 : (D.w_dtype == TP_DTYPE_BF16 ? 2 : 1);
  x.ab = D.act_dtype == TP_DTYPE_F32 ? 4 : 2;
  return TP_OK;
}

void make_layout(const Dims& x, tp_shard_layout* L) {
  *L = tp_shard_layout{};
  uint64_t off = 0, payload = 0;
  auto put = [&](tp_region& r, uint64_t rows, uint64_t cols, tp_region& sc) {
    r.offset = off;
    r.bytes = rows * cols * (uint64_t)x.wb;
    off = align_up(off + r.bytes);
    payload += r.bytes;
    if (x.wt == TP_DTYPE_Q8_0) {
      sc.offset = off;
      sc.bytes = rows * (cols / 32) * 2;
      off = align_up(off + sc.bytes);
      payload += sc.bytes;
    }
  };
  put(L->qkv, x.qkv_rows, x.d, L->qkv_scale);
  put(L->o, x.d, x.qdim, L->o_scale);
  put(L->gate_up, 2 * (uint64_t)x.fr, x.d, L->gate_up_scale);
  put(L->down, x.d, x.fr, L->down_scale);
  L->payload_bytes = payload;
  L->alloc_bytes = off;
}

struct WsLayout {
  uint64_t qkv, q, attn, part_o, part_ml, ffn, gemm, gemm_bytes, qkvp, total;
  int n_split, chunk, pos_limit;
};

tp_status check_batch(const Dims& x, const tp_batch* b, bool need_attn) {
  if (!b) return fail(TP_ERR_INVALID_ARG, "batch is NULL");
  if (b->mode != TP_MODE_DECODE && b->mode != TP_MODE_PREFILL)
    return fail(TP_ERR_INVALID_ARG, "unknown batch mode %d", b->mode);
  if (b->n_tokens < 0 || b->n_seqs < 0)
    return fail(TP_ERR_INVALID_ARG, "n_tokens=%d and n_seqs=%d must be >= 0", b->n_tokens,
                b->n_seqs);
  if (b->mode == TP_MODE_DECODE && b->n_seqs != b->n_tokens)
    return fail(TP_ERR_INVALID_ARG, "decode batches carry one token per sequence (n_tokens=%d, "
                "n_seqs=%d)", b->n_tokens, b->n_seqs);
  if (b->mode == TP_MODE_PREFILL && b->n_tokens > 0 && b->n_seqs != 1)
    return fail(TP_ERR_INVALID_ARG, "prefill batches carry one sequence (n_seqs=%d)", b->n_seqs);
  if (b->max_pages <= 0) return fail(TP_ERR_INVALID_ARG, "max_pages=%d must be > 0", b->max_pages);
  const int64_t cap = (int64_t)b->max_pages * x.ps;
  if (b->max_seq_len < 0 || b->max_seq_len > cap || b->max_seq_len > x.maxpos)
    return fail(TP_ERR_INVALID_ARG,
                "max_seq_len=%d must be in [0, min(max_pages*page_size=%lld, max_position=%d)]",
                b->max_seq_len, (long long)cap, x.maxpos);
  if (need_attn && b->n_tokens > 0 && (!b->positions || !b->block_table || !b->rope_table))
    return fail(TP_ERR_INVALID_ARG, "positions, block_table and rope_table must be non-NULL");
  return TP_OK;
}

// One projection of T tokens: bf16 weights with more tokens than the GEMV holds go to the MFMA
// GEMM; everything else streams through the GEMV (in groups of up to 4 tokens).
bool use_gemm(const Dims& x, int T, int K) {
  return x.wt == TP_DTYPE_BF16 && T > tpk::gemv_max_tokens(K);
}

// Q8_0 projections of more than four tokens run on the matrix cores (k_gemm_q8) instead of
// streaming the weights once per group of four tokens through the GEMV.
bool use_q8_gemm(const Dims& x, int T) { return x.wt == TP_DTYPE_Q8_0 && T > 4; }

// K ranges of the split-K QKV projection (bf16 prefill shapes too narrow to fill the chip with
// whole-K tiles); 1: the projection runs unsplit.
int qkv_ksplit(const Dims& x, int T) {
  if (x.at != TP_DTYPE_BF16 || T <= 64 || !use_gemm(x, T, x.d)) return 1;
  return tpk::gemm_split_count(T, x.qkv_rows, x.d);
}

// ranks: how many ranks' attention shares one launch (the all-ranks batched schedule: the key
// range is split only as far as all ranks' workgroups together need).
WsLayout ws_layout(const Dims& x, const tp_batch& b, int ranks = 1) {
  WsLayout w{};
  const uint64_t T = (uint64_t)b.n_tokens;
  int L = b.max_seq_len > 0 ? b.max_seq_len : b.max_pages * x.ps;
  if (L > x.maxpos) L = x.maxpos;
  if (L < 1) L = 1;
  w.pos_limit = L;
  // Key splits of the attention: about 256 workgroups in total, in multiples of 32 keys, each at
  // least one 32-key tile per wave (128 keys) or, for heads of 256 and more, whose tiles carry
  // twice the bytes, two of the four waves busy (64 keys).
  const int per_split = x.hk * (int)(T > 0 ? T : 1) * ranks;
  const int want = (256 + per_split - 1) / per_split;
  const int min_chunk = x.hd >= 256 ? 64 : 128;
  int chunk = (L + want - 1) / want;
  chunk = (chunk + 31) / 32 * 32;
  if (chunk < min_chunk) chunk = min_chunk;
  w.chunk = chunk;
  w.n_split = (L + chunk - 1) / chunk;
  uint64_t off = 0;
  auto put = [&](uint64_t& o, uint64_t bytes) {
    o = off;
    off = align_up(off + bytes);
  };
  const bool splitk = x.wt == TP_DTYPE_BF16 && T > 0 && T <= 64;
  put(w.qkv, T * x.qkv_rows * x.ab);
  put(w.q, T * x.qdim * x.ab);
  put(w.attn, T * x.qdim * x.ab);
  put(w.part_o, T * x.hq * (uint64_t)w.n_split * x.hd * 4);
  put(w.part_ml, T * x.hq * (uint64_t)w.n_split * 2 * 4);
  put(w.ffn, T * x.fr * x.ab);
  // fp32 split-K partial tiles of the batched-decode projections (bf16 weights, 4 < T <= 64)
  // and of the Q8_0 matrix-core projections (more than four tokens, narrow shapes).
  uint64_t gemm = 0;
  if (splitk) {
    const uint64_t cand[4] = {
        tpk::splitk_workspace_bytes((int)T, x.qkv_rows, x.d, false),
        tpk::splitk_workspace_bytes((int)T, x.d, x.qdim, false),
        tpk::splitk_workspace_bytes((int)T, x.fr, x.d, true),
        tpk::splitk_workspace_bytes((int)T, x.d, x.fr, false)};
    for (uint64_t c : cand) gemm = c > gemm ? c : gemm;
  } else if (use_q8_gemm(x, (int)T)) {
    // (The QKV's: its K ranges' tiles, which the all-ranks batched step leaves for the rotary
    // kernel to sum, even when there is one range.)
    const uint64_t cand[4] = {
        (uint64_t)tpk::q8_gemm_splits((int)T, x.qkv_rows, x.d) * T * x.qkv_rows * 4,
        tpk::q8_gemm_workspace_bytes((int)T, x.d, x.qdim, false),
        tpk::q8_gemm_workspace_bytes((int)T, x.fr, x.d, true),
        tpk::q8_gemm_workspace_bytes((int)T, x.d, x.fr, false)};
    for (uint64_t c : cand) gemm = c > gemm ? c : gemm;
  }
  put(w.gemm, gemm);
  w.gemm_bytes = gemm;
  // fp32 partial products of the split-K QKV projection.
  const uint64_t ks = (uint64_t)qkv_ksplit(x, (int)T);
  put(w.qkvp, ks > 1 ? ks * T * x.qkv_rows * 4 : 0);
  w.total = off > 0 ? off : kAlign;
  return w;
}

// Kernel-execution timing of one projection (see tpk::LaunchTiming); cleared on every exit path.
struct TimedScope {
  TimedScope(hipEvent_t b, hipEvent_t e) { tpk::g_timing = {b, e}; }
  ~TimedScope() { tpk::g_timing = {}; }
};

hipError_t project(const Dims& x, int epi, int T, const char* W, const char* S, int K, int n_out,
                   int gate_off, const void* X, void* Y, int ldy, hipStream_t st,
                   const tpk::RopeEpi* rope = nullptr, float* splitk_ws = nullptr,
                   const tpk::FuseArgs* fuse = nullptr) {
  // The fused norm prologue and reduce epilogue exist on the decode GEMV only.
  if (fuse && (use_q8_gemm(x, T) || use_gemm(x, T, K) || T > tpk::gemv_max_tokens(K)))
    return hipErrorInvalidValue;
  if (use_q8_gemm(x, T) && epi != tpk::EPI_ROPE) {
    const bool gated = epi == tpk::EPI_GATED;
    const char* B2 = gated ? W + (size_t)gate_off * K : nullptr;
    const char* S2 = gated ? S + (size_t)gate_off * (K / 32) * 2 : nullptr;
    return tpk::launch_gemm_q8(epi, x.actf, T, n_out, K, X, W, S, B2, S2, Y, ldy, splitk_ws, st);
  }
  if (use_gemm(x, T, K)) {
    const char* B2 = (epi == tpk::EPI_GATED) ? W + (size_t)gate_off * K * 2 : nullptr;
    if (T <= 64 && tpk::gemm_band_supported(epi, T, n_out, K))
      return tpk::launch_gemm_band(epi, x.actf, T, n_out, K, X, W, B2, Y, ldy, st);
    if (T <= 64 && splitk_ws)
      return tpk::launch_gemm_splitk(epi, x.actf, T, n_out, K, X, W, B2, Y, ldy, splitk_ws, st);
    return tpk::launch_gemm_bf16(epi, x.actf, T, n_out, K, X, W, B2, Y, ldy, st);
  }
  const int wt = x.wt == TP_DTYPE_F32 ? tpk::W_F32 : (x.wt == TP_DTYPE_BF16 ? tpk::W_BF16 : tpk::W_Q8);
  return tpk::launch_gemv(wt, x.at == TP_DTYPE_F32 ? tpk::ACT_F32 : tpk::ACT_BF16, epi, x.actf, T,
                          W, S, K, n_out, gate_off, X, Y, ldy, rope, st, fuse);
}

// The one-call block step folds the replicated norms and the local reduces into the decode GEMVs
// around them; that needs every projection of the step to be a single GEMV launch.
bool fused_step_ok(const Dims& x, int T) {
  if (T < 1 || T > 4 || x.N > 8) return false;
  const int ks[3] = {x.d, x.qdim, x.fr};
  for (int K : ks)
    if (T > tpk::gemv_max_tokens(K) || use_gemm(x, T, K)) return false;
  return !use_q8_gemm(x, T);
}

int gemv_wt(const Dims& x) {
  return x.wt == TP_DTYPE_F32 ? tpk::W_F32 : (x.wt == TP_DTYPE_BF16 ? tpk::W_BF16 : tpk::W_Q8);
}

// ... and, with at most four ranks whose inputs fit one workgroup's LDS, each projection and the attention
// run as one launch for all ranks (the row-parallel ones adding the partials in rank order), so
// the decode step is six launches. Each rank then needs its own copy of the workspace.
bool ranks_step_ok(const Dims& x, int T) {
  if (!fused_step_ok(x, T) || x.N < 2) return false;
  const int wt = gemv_wt(x);
  return tpk::gemv_ranks_fit(wt, tpk::EPI_ROPE, x.N, T, x.d) &&
         tpk::gemv_ranks_fit(wt, tpk::EPI_RED_ALL, x.N, T, x.qdim) &&
         tpk::gemv_ranks_fit(wt, tpk::EPI_RED_ALL, x.N, T, x.fr);
}

// Batched decode (5 to 64 tokens) whose projections all take the split-K QKV and the band GEMMs
// (bf16) or the Q8_0 matrix-core GEMM: the staged sequence with each projection, the rotary / KV
// append and the attention as one launch for all ranks (the reduces are one launch for all ranks
// already).
bool ranks_staged_ok(const Dims& x, const tp_batch& b) {
  const int T = b.n_tokens;
  if (x.N < 2 || x.N > tpk::kMaxRanks || T < 1 || T > 64 || b.mode != TP_MODE_DECODE) return false;
  if (x.at != TP_DTYPE_BF16) return false;
  // Q8_0: the rotary kernel sums the QKV's K ranges (at most 16).
  if (x.wt == TP_DTYPE_Q8_0)
    return use_q8_gemm(x, T) && tpk::q8_gemm_splits(T, x.qkv_rows, x.d) <= 16;
  if (x.wt != TP_DTYPE_BF16) return false;
  if (!use_gemm(x, T, x.d) || !use_gemm(x, T, x.qdim) || !use_gemm(x, T, x.fr)) return false;
  if (x.d % 64 != 0) return false;  // the direct-to-LDS split-K QKV
  return tpk::gemm_band_supported(tpk::EPI_F32, T, x.d, x.qdim) &&
         tpk::gemm_band_supported(tpk::EPI_GATED, T, x.fr, x.d) &&
         tpk::gemm_band_supported(tpk::EPI_F32, T, x.d, x.fr);
}

// Prefill whose QKV takes the split-K wide tiles and whose o_proj, gate/up and down take the
// 256 x 256 wide tiles (bf16), or whose projections take the Q8_0 matrix-core GEMM (Q8_0, at
// most 16 K ranges for the QKV): the staged sequence with one launch per stage for all ranks.
bool ranks_prefill_ok(const Dims& x, const tp_batch& b) {
  const int T = b.n_tokens;
  if (x.N < 2 || x.N > tpk::kMaxRanks || T < 256 || b.mode != TP_MODE_PREFILL) return false;
  if (x.at != TP_DTYPE_BF16) return false;
  if (x.wt == TP_DTYPE_Q8_0)
    return use_q8_gemm(x, T) && tpk::attn_prefill_supported(x.hd, x.Hq / x.Hkv, x.ps) &&
           tpk::q8_gemm_splits(T, x.qkv_rows, x.d) <= 16;
  if (x.wt != TP_DTYPE_BF16) return false;
  if (qkv_ksplit(x, T) <= 1 || !tpk::attn_prefill_supported(x.hd, x.Hq / x.Hkv, x.ps))
    return false;
  auto wide = [&](int epi, int n_out, int K) {
    return K % 64 == 0 && tpk::gemm_wide_tiles(epi, T, n_out) >= 192;
  };
  return wide(tpk::EPI_F32, x.d, x.qdim) && wide(tpk::EPI_GATED, x.fr, x.d) &&
         wide(tpk::EPI_F32, x.d, x.fr);
}

bool all_ranks_ok(const Dims& x, const tp_batch& b) {
  return ranks_step_ok(x, b.n_tokens) || ranks_staged_ok(x, b) || ranks_prefill_ok(x, b);
}

// Workspace layout of one rank under the step's schedule (the all-ranks staged schedule plans
// the attention's key splits for all ranks' workgroups together).
WsLayout step_ws_layout(const Dims& x, const tp_batch& b) {
  const bool staged_all = !ranks_step_ok(x, b.n_tokens) &&
                          (ranks_staged_ok(x, b) || ranks_prefill_ok(x, b));
  return ws_layout(x, b, staged_all ? x.N : 1);
}

uint64_t step_ws_bytes(const Dims& x, const tp_batch& b) {
  if (!all_ranks_ok(x, b)) return ws_layout(x, b).total;
  return (uint64_t)x.N * align_up(step_ws_layout(x, b).total);
}

}  // namespace

extern "C" {

const char* tp_status_str(tp_status s) {
  switch (s) {
    case TP_OK: return "TP_OK";
    case TP_ERR_INVALID_ARG: return "TP_ERR_INVALID_ARG";
    case TP_ERR_RANK: return "TP_ERR_RANK";
    case TP_ERR_NOT_DIVISIBLE: return "TP_ERR_NOT_DIVISIBLE";
    case TP_ERR_QUANT_ALIGN: return "TP_ERR_QUANT_ALIGN";
    case TP_ERR_BUFFER_TOO_SMALL: return "TP_ERR_BUFFER_TOO_SMALL";
    case TP_ERR_UNSUPPORTED: return "TP_ERR_UNSUPPORTED";
    case TP_ERR_HIP: return "TP_ERR_HIP";
  }
  return "TP_ERR_UNKNOWN";
}

const char* tp_last_error(void) { return g_err.c_str(); }

tp_status tp_shard_weights_size(const tp_block_desc* desc, int32_t rank, tp_shard_layout* out) {
  Dims x;
  if (tp_status s = check_desc(desc, &x)) return s;
  if (rank < 0 || rank >= x.N) return fail(TP_ERR_RANK, "rank %d not in [0, %d)", rank, x.N);
  if (!out) return fail(TP_ERR_INVALID_ARG, "out is NULL");
  make_layout(x, out);
  g_err.clear();
  return TP_OK;
}

static tp_status check_full(const tp_full_weights* w) {
  if (!w || !w->wq || !w->wk || !w->wv || !w->wo || !w->wg || !w->wu || !w->wd)
    return fail(TP_ERR_INVALID_ARG, "full weights: every pointer must be non-NULL");
  return TP_OK;
}

// Pack (to_shard = true) or unpack rank r's slices. The slice geometry is the same both ways.
static tp_status shard_copy(const Dims& x, int r, const tp_full_weights* full, char* shard,
                            bool to_shard, hipStream_t st) {
  tp_shard_layout L;
  make_layout(x, &L);
  struct Piece {
    const void* full;
    int64_t row0, rows;      // rows taken from the full matrix
    int64_t col0, cols;      // columns taken (elements)
    int64_t full_cols;       // row length of the full matrix (elements)
    uint64_t dst_row0;       // first row inside the packed region
    const tp_region* reg;
    const tp_region* sreg;
    int64_t reg_cols;        // row length inside the packed region (elements)
  };
  const int64_t hd = x.hd, d = x.d;
  const std::vector<Piece> pieces = {
      {full->wq, r * x.hq * hd, x.hq * hd, 0, d, d, 0, &L.qkv, &L.qkv_scale, d},
      {full->wk, r * x.hk * hd, x.hk * hd, 0, d, d, (uint64_t)(x.hq * hd), &L.qkv, &L.qkv_scale, d},
      {full->wv, r * x.hk * hd, x.hk * hd, 0, d, d, (uint64_t)((x.hq + x.hk) * hd), &L.qkv,
       &L.qkv_scale, d},
      {full->wo, 0, d, (int64_t)r * x.qdim, x.qdim, (int64_t)x.Hq * hd, 0, &L.o, &L.o_scale, x.qdim},
      {full->wg, (int64_t)r * x.fr, x.fr, 0, d, d, 0, &L.gate_up, &L.gate_up_scale, d},
      {full->wu, (int64_t)r * x.fr, x.fr, 0, d, d, (uint64_t)x.fr, &L.gate_up, &L.gate_up_scale, d},
      {full->wd, 0, d, (int64_t)r * x.fr, x.fr, (int64_t)x.F, 0, &L.down, &L.down_scale, x.fr},
  };
  for (const Piece& p : pieces) {
    hipError_t e;
    if (x.wt == TP_DTYPE_Q8_0) {
      const size_t full_ld = (size_t)(p.full_cols / 32) * 34;
      char* src = (char*)p.full + (size_t)p.row0 * full_ld + (size_t)(p.col0 / 32) * 34;
      char* codes = shard + p.reg->offset + p.dst_row0 * (uint64_t)p.reg_cols;
      char* scales = shard + p.sreg->offset + p.dst_row0 * (uint64_t)(p.reg_cols / 32) * 2;
      e = to_shard ? tpk::q8_split(src, full_ld, p.rows, p.cols / 32, codes, scales, st)
                   : tpk::q8_join(src, full_ld, p.rows, p.cols / 32, codes, scales, st);
    } else {
      const size_t full_ld = (size_t)p.full_cols * x.wb;
      char* fptr = (char*)p.full + (size_t)p.row0 * full_ld + (size_t)p.col0 * x.wb;
      char* sptr = shard + p.reg->offset + p.dst_row0 * (uint64_t)p.reg_cols * x.wb;
      const size_t sld = (size_t)p.reg_cols * x.wb, row_bytes = (size_t)p.cols * x.wb;
      e = to_shard ? tpk::copy2d(sptr, sld, fptr, full_ld, p.rows, row_bytes, st)
                   : tpk::copy2d(fptr, full_ld, sptr, sld, p.rows, row_bytes, st);
    }
    if (e != hipSuccess) return hip_fail(e, to_shard ? "tp_shard_weights" : "tp_shard_unpack");
  }
  g_err.clear();
  return TP_OK;
}

tp_status tp_shard_weights(const tp_block_desc* desc, int32_t rank, const tp_full_weights* src,
                           void* dst, uint64_t dst_bytes, void* stream) {
  Dims x;
  if (tp_status s = check_desc(desc, &x)) return s;
  if (rank < 0 || rank >= x.N) return fail(TP_ERR_RANK, "rank %d not in [0, %d)", rank, x.N);
  if (tp_status s = check_full(src)) return s;
  if (!dst) return fail(TP_ERR_INVALID_ARG, "dst is NULL");
  tp_shard_layout L;
  make_layout(x, &L);
  if (dst_bytes < L.alloc_bytes)
    return fail(TP_ERR_BUFFER_TOO_SMALL, "dst_bytes=%llu < alloc_bytes=%llu",
                (unsigned long long)dst_bytes, (unsigned long long)L.alloc_bytes);
  return shard_copy(x, rank, src, (char*)dst, true, (hipStream_t)stream);
}

tp_status tp_shard_unpack(const tp_block_desc* desc, int32_t rank, const void* shard,
                          const tp_full_weights* dst, void* stream) {
  Dims x;
  if (tp_status s = check_desc(desc, &x)) return s;
  if (rank < 0 || rank >= x.N) return fail(TP_ERR_RANK, "rank %d not in [0, %d)", rank, x.N);
  if (tp_status s = check_full(dst)) return s;
  if (!shard) return fail(TP_ERR_INVALID_ARG, "shard is NULL");
  return shard_copy(x, rank, dst, (char*)shard, false, (hipStream_t)stream);
}

// ---- replicated head: one packed [vocab, d] table for the embedding lookup and the LM head
static tp_status check_head(const tp_block_desc* desc, int32_t vocab, Dims* x) {
  if (tp_status s = check_desc(desc, x)) return s;
  if (vocab <= 0) return fail(TP_ERR_INVALID_ARG, "vocab=%d must be > 0", vocab);
  return TP_OK;
}

static void make_head_layout(const Dims& x, int32_t vocab, tp_head_layout* L) {
  *L = tp_head_layout{};
  L->table.offset = 0;
  L->table.bytes = (uint64_t)vocab * x.d * x.wb;
  uint64_t off = align_up(L->table.bytes);
  if (x.wt == TP_DTYPE_Q8_0) {
    L->table_scale.offset = off;
    L->table_scale.bytes = (uint64_t)vocab * (x.d / 32) * 2;
    off = align_up(off + L->table_scale.bytes);
  }
  L->payload_bytes = L->table.bytes + L->table_scale.bytes;
  L->alloc_bytes = off;
}

tp_status tp_head_size(const tp_block_desc* desc, int32_t vocab, tp_head_layout* out) {
  Dims x;
  if (tp_status s = check_head(desc, vocab, &x)) return s;
  if (!out) return fail(TP_ERR_INVALID_ARG, "out is NULL");
  make_head_layout(x, vocab, out);
  g_err.clear();
  return TP_OK;
}

tp_status tp_head_pack(const tp_block_desc* desc, int32_t vocab, const void* src, void* dst,
                       uint64_t dst_bytes, void* stream) {
  Dims x;
  if (tp_status s = check_head(desc, vocab, &x)) return s;
  if (!src || !dst) return fail(TP_ERR_INVALID_ARG, "src and dst must be non-NULL");
  tp_head_layout L;
  make_head_layout(x, vocab, &L);
  if (dst_bytes < L.alloc_bytes)
    return fail(TP_ERR_BUFFER_TOO_SMALL, "dst_bytes=%llu < alloc_bytes=%llu",
                (unsigned long long)dst_bytes, (unsigned long long)L.alloc_bytes);
  hipStream_t st = (hipStream_t)stream;
  char* d = (char*)dst;
  hipError_t e;
  if (x.wt == TP_DTYPE_Q8_0)
    e = tpk::q8_split(src, (size_t)(x.d / 32) * 34, vocab, x.d / 32, d + L.table.offset,
                      d + L.table_scale.offset, st);
  else
    e = tpk::copy2d(d + L.table.offset, (size_t)x.d * x.wb, src, (size_t)x.d * x.wb, vocab,
                    (size_t)x.d * x.wb, st);
  if (e != hipSuccess) return hip_fail(e, "tp_head_pack");
  g_err.clear();
  return TP_OK;
}

tp_status tp_embed_lookup(const tp_block_desc* desc, int32_t vocab, const void* head,
                          const int32_t* token_ids, int32_t n_tokens, void* x_out, void* stream) {
  Dims x;
  if (tp_status s = check_head(desc, vocab, &x)) return s;
  if (n_tokens < 0) return fail(TP_ERR_INVALID_ARG, "n_tokens=%d must be >= 0", n_tokens);
  if (n_tokens == 0) return TP_OK;
  if (!head || !token_ids || !x_out)
    return fail(TP_ERR_INVALID_ARG, "head, token_ids and x_out must be non-NULL");
  if (!aligned16(head) || !aligned16(x_out))
    return fail(TP_ERR_INVALID_ARG, "head and x_out must be 16-byte aligned");
  tp_head_layout L;
  make_head_layout(x, vocab, &L);
  const char* h = (const char*)head;
  const int wt = x.wt == TP_DTYPE_F32 ? tpk::W_F32 : (x.wt == TP_DTYPE_BF16 ? tpk::W_BF16 : tpk::W_Q8);
  hipError_t e = tpk::launch_embed(wt, h + L.table.offset, h + L.table_scale.offset, token_ids,
                                   n_tokens, vocab, x.d, x_out, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "tp_embed_lookup");
  g_err.clear();
  return TP_OK;
}

tp_status tp_lm_head(const tp_block_desc* desc, int32_t vocab, const void* head, const void* xn,
                     int32_t n_tokens, float* logits, void* stream) {
  Dims x;
  if (tp_status s = check_head(desc, vocab, &x)) return s;
  if (n_tokens < 0) return fail(TP_ERR_INVALID_ARG, "n_tokens=%d must be >= 0", n_tokens);
  if (n_tokens == 0) return TP_OK;
  if (!head || !xn || !logits)
    return fail(TP_ERR_INVALID_ARG, "head, xn and logits must be non-NULL");
  if (!aligned16(head) || !aligned16(xn) || !aligned16(logits))
    return fail(TP_ERR_INVALID_ARG, "head, xn and logits must be 16-byte aligned");
  tp_head_layout L;
  make_head_layout(x, vocab, &L);
  const char* h = (const char*)head;
  hipError_t e;
  const size_t one_split = (size_t)n_tokens * vocab * sizeof(float);
  if (use_gemm(x, n_tokens, x.d) && n_tokens <= 64 &&
      tpk::splitk_workspace_bytes(n_tokens, vocab, x.d, false) == one_split) {
    // A vocabulary wide enough to fill the chip with whole-K column tiles: the batched-decode
    // GEMM (activation tile shared through LDS) writes its single fp32 tile straight into the
    // logits, which have the partial-tile layout [T, vocab].
    int parts = 0;
    e = tpk::launch_gemm_splitk(tpk::EPI_F32, 0, n_tokens, vocab, x.d, xn, h + L.table.offset,
                                nullptr, logits, vocab, logits, (hipStream_t)stream, &parts);
    if (e == hipSuccess && parts != 1) e = hipErrorInvalidValue;
  } else {
    e = project(x, tpk::EPI_F32, n_tokens, h + L.table.offset, h + L.table_scale.offset, x.d,
                vocab, 0, xn, logits, vocab, (hipStream_t)stream);
  }
  if (e != hipSuccess) return hip_fail(e, "tp_lm_head");
  g_err.clear();
  return TP_OK;
}

// ---- expert-sliced MoE FFN half
struct MoeDims {
  int E, k, F, fr;
};

static tp_status check_moe(const tp_block_desc* desc, const tp_moe_desc* moe, Dims* x,
                           MoeDims* m) {
  if (tp_status s = check_desc(desc, x)) return s;
  if (!moe) return fail(TP_ERR_INVALID_ARG, "moe is NULL");
  if (moe->n_experts < 1 || moe->n_experts > 1024)
    return fail(TP_ERR_INVALID_ARG, "n_experts=%d must be in [1, 1024]", moe->n_experts);
  if (moe->top_k < 1 || moe->top_k > 16 || moe->top_k > moe->n_experts)
    return fail(TP_ERR_INVALID_ARG, "top_k=%d must be in [1, min(n_experts, 16)]", moe->top_k);
  if (moe->expert_ffn <= 0) return fail(TP_ERR_INVALID_ARG, "expert_ffn must be > 0");
  if (moe->expert_ffn % x->N)
    return fail(TP_ERR_NOT_DIVISIBLE, "expert_ffn=%d must divide by tp_degree=%d",
                moe->expert_ffn, x->N);
  if ((moe->expert_ffn / x->N) % 8)
    return fail(TP_ERR_UNSUPPORTED, "expert_ffn/tp_degree=%d must be a multiple of 8",
                moe->expert_ffn / x->N);
  if (x->wt == TP_DTYPE_Q8_0 && moe->expert_ffn % (x->N * 32))
    return fail(TP_ERR_QUANT_ALIGN,
                "Q8_0 row-parallel expert down split needs expert_ffn=%d divisible by "
                "tp_degree*32=%d",
                moe->expert_ffn, x->N * 32);
  *m = MoeDims{moe->n_experts, moe->top_k, moe->expert_ffn, moe->expert_ffn / x->N};
  return TP_OK;
}

static void make_moe_layout(const Dims& x, const MoeDims& m, tp_moe_layout* L) {
  *L = tp_moe_layout{};
  uint64_t off = 0, payload = 0;
  auto put = [&](tp_region& r, uint64_t rows, uint64_t cols, tp_region& sc) {
    r.offset = off;
    r.bytes = rows * cols * (uint64_t)x.wb;
    off = align_up(off + r.bytes);
    payload += r.bytes;
    if (x.wt == TP_DTYPE_Q8_0) {
      sc.offset = off;
      sc.bytes = rows * (cols / 32) * 2;
      off = align_up(off + sc.bytes);
      payload += sc.bytes;
    }
  };
  put(L->gate, (uint64_t)m.E * m.fr, x.d, L->gate_scale);
  put(L->up, (uint64_t)m.E * m.fr, x.d, L->up_scale);
  put(L->down, (uint64_t)m.E * x.d, m.fr, L->down_scale);
  L->payload_bytes = payload;
  L->alloc_bytes = off;
}

tp_status tp_moe_shard_size(const tp_block_desc* desc, const tp_moe_desc* moe, int32_t rank,
                            tp_moe_layout* out) {
  Dims x;
  MoeDims m;
  if (tp_status s = check_moe(desc, moe, &x, &m)) return s;
  if (rank < 0 || rank >= x.N) return fail(TP_ERR_RANK, "rank %d not in [0, %d)", rank, x.N);
  if (!out) return fail(TP_ERR_INVALID_ARG, "out is NULL");
  make_moe_layout(x, m, out);
  g_err.clear();
  return TP_OK;
}

tp_status tp_moe_shard_weights(const tp_block_desc* desc, const tp_moe_desc* moe, int32_t rank,
                               const tp_moe_full_weights* src, void* dst, uint64_t dst_bytes,
                               void* stream) {
  Dims x;
  MoeDims m;
  if (tp_status s = check_moe(desc, moe, &x, &m)) return s;
  if (rank < 0 || rank >= x.N) return fail(TP_ERR_RANK, "rank %d not in [0, %d)", rank, x.N);
  if (!src || !src->wg || !src->wu || !src->wd || !dst)
    return fail(TP_ERR_INVALID_ARG, "src->wg, wu, wd and dst must be non-NULL");
  tp_moe_layout L;
  make_moe_layout(x, m, &L);
  if (dst_bytes < L.alloc_bytes)
    return fail(TP_ERR_BUFFER_TOO_SMALL, "dst_bytes=%llu < alloc_bytes=%llu",
                (unsigned long long)dst_bytes, (unsigned long long)L.alloc_bytes);
  hipStream_t st = (hipStream_t)stream;
  char* d = (char*)dst;
  const int64_t dm = x.d, fr = m.fr, F = m.F, E = m.E, r = rank;
  hipError_t e = hipSuccess;
  if (x.wt == TP_DTYPE_Q8_0) {
    const size_t ld_in = (size_t)(dm / 32) * 34;  // one full row of d, in 34-byte blocks
    for (int64_t ex = 0; ex < E && e == hipSuccess; ++ex) {
      const size_t row0 = (size_t)(ex * F + r * fr);
      e = tpk::q8_split((const char*)src->wg + row0 * ld_in, ld_in, fr, dm / 32,
                        d + L.gate.offset + (size_t)ex * fr * dm,
                        d + L.gate_scale.offset + (size_t)ex * fr * (dm / 32) * 2, st);
      if (e == hipSuccess)
        e = tpk::q8_split((const char*)src->wu + row0 * ld_in, ld_in, fr, dm / 32,
                          d + L.up.offset + (size_t)ex * fr * dm,
                          d + L.up_scale.offset + (size_t)ex * fr * (dm / 32) * 2, st);
    }
    if (e == hipSuccess)
      e = tpk::q8_split((const char*)src->wd + (size_t)(r * fr / 32) * 34, (size_t)(F / 32) * 34,
                        E * dm, fr / 32, d + L.down.offset, d + L.down_scale.offset, st);
  } else {
    const size_t wb = x.wb;
    e = tpk::copy2d(d + L.gate.offset, fr * dm * wb, (const char*)src->wg + r * fr * dm * wb,
                    F * dm * wb, E, fr * dm * wb, st);
    if (e == hipSuccess)
      e = tpk::copy2d(d + L.up.offset, fr * dm * wb, (const char*)src->wu + r * fr * dm * wb,
                      F * dm * wb, E, fr * dm * wb, st);
    if (e == hipSuccess)
      e = tpk::copy2d(d + L.down.offset, fr * wb, (const char*)src->wd + r * fr * wb, F * wb,
                      E * dm, fr * wb, st);
  }
  if (e != hipSuccess) return hip_fail(e, "tp_moe_shard_weights");
  g_err.clear();
  return TP_OK;
}

tp_status tp_moe_route(const tp_block_desc* desc, const tp_moe_desc* moe, const void* router,
                       const void* xn, int32_t n_tokens, float* logits, int32_t* topk_ids,
                       float* topk_weights, void* stream) {
  Dims x;
  MoeDims m;
  if (tp_status s = check_moe(desc, moe, &x, &m)) return s;
  if (n_tokens < 0) return fail(TP_ERR_INVALID_ARG, "n_tokens=%d must be >= 0", n_tokens);
  if (n_tokens == 0) return TP_OK;
  if (!router || !xn || !logits || !topk_ids || !topk_weights)
    return fail(TP_ERR_INVALID_ARG, "router, xn, logits, topk_ids and topk_weights must be non-NULL");
  if (!aligned16(router) || !aligned16(xn))
    return fail(TP_ERR_INVALID_ARG, "router and xn must be 16-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  const int at = x.at == TP_DTYPE_F32 ? tpk::ACT_F32 : tpk::ACT_BF16;
  const int wt = x.at == TP_DTYPE_F32 ? tpk::W_F32 : tpk::W_BF16;
  hipError_t e = tpk::launch_gemv(wt, at, tpk::EPI_F32, 0, n_tokens, router, nullptr, x.d, m.E, 0,
                                  xn, logits, m.E, nullptr, st);
  if (e == hipSuccess) e = tpk::launch_moe_topk(logits, n_tokens, m.E, m.k, topk_ids, topk_weights, st);
  if (e != hipSuccess) return hip_fail(e, "tp_moe_route");
  g_err.clear();
  return TP_OK;
}

tp_status tp_moe_workspace_size(const tp_block_desc* desc, const tp_moe_desc* moe,
                                int32_t n_tokens, uint64_t* bytes) {
  Dims x;
  MoeDims m;
  if (tp_status s = check_moe(desc, moe, &x, &m)) return s;
  if (n_tokens < 0) return fail(TP_ERR_INVALID_ARG, "n_tokens=%d must be >= 0", n_tokens);
  if (!bytes) return fail(TP_ERR_INVALID_ARG, "bytes is NULL");
  const uint64_t b = (uint64_t)n_tokens * m.k * m.fr * x.ab;
  *bytes = b > 0 ? align_up(b) : kAlign;
  return TP_OK;
}

static tp_status moe_forward_impl(const tp_block_desc* desc, const tp_moe_desc* moe,
                                  int32_t rank, const void* shard, const void* xn,
                                  int32_t n_tokens, const int32_t* topk_ids,
                                  const float* topk_weights, void* partial_out, void* workspace,
                                  uint64_t workspace_bytes, void* stream, hipEvent_t evb,
                                  hipEvent_t eve, const tpk::FuseArgs* fout = nullptr) {
  Dims x;
  MoeDims m;
  if (tp_status s = check_moe(desc, moe, &x, &m)) return s;
  if (rank < 0 || rank >= x.N) return fail(TP_ERR_RANK, "rank %d not in [0, %d)", rank, x.N);
  if (n_tokens < 0) return fail(TP_ERR_INVALID_ARG, "n_tokens=%d must be >= 0", n_tokens);
  if (n_tokens == 0) {
    g_err.clear();
    return TP_OK;
  }
  if (!shard || !xn || !topk_ids || !topk_weights || !partial_out || !workspace)
    return fail(TP_ERR_INVALID_ARG,
                "shard, xn, topk_ids, topk_weights, partial_out and workspace must be non-NULL");
  if (!aligned16(shard) || !aligned16(xn) || !aligned16(workspace))
    return fail(TP_ERR_INVALID_ARG, "shard, xn and workspace must be 16-byte aligned");
  uint64_t need = 0;
  tp_moe_workspace_size(desc, moe, n_tokens, &need);
  if (workspace_bytes < need)
    return fail(TP_ERR_BUFFER_TOO_SMALL, "workspace_bytes=%llu < %llu",
                (unsigned long long)workspace_bytes, (unsigned long long)need);
  tp_moe_layout L;
  make_moe_layout(x, m, &L);
  const char* sh = (const char*)shard;
  const int wt = x.wt == TP_DTYPE_F32 ? tpk::W_F32 : (x.wt == TP_DTYPE_BF16 ? tpk::W_BF16 : tpk::W_Q8);
  const int at = x.at == TP_DTYPE_F32 ? tpk::ACT_F32 : tpk::ACT_BF16;
  const int pt = x.pt == TP_DTYPE_F32 ? tpk::ACT_F32 : tpk::ACT_BF16;
  hipError_t e;
  {
    TimedScope ts(evb, eve);
    e = tpk::launch_moe_ffn(wt, at, x.actf, pt, sh + L.gate.offset, sh + L.gate_scale.offset,
                            sh + L.up.offset, sh + L.up_scale.offset, sh + L.down.offset,
                            sh + L.down_scale.offset, x.d, m.fr, m.E, m.k, n_tokens, topk_ids,
                            topk_weights, xn, workspace, partial_out, (hipStream_t)stream, fout);
  }
  if (e != hipSuccess) return hip_fail(e, "moe ffn");
  g_err.clear();
  return TP_OK;
}

tp_status tp_moe_shard_forward(const tp_block_desc* desc, const tp_moe_desc* moe, int32_t rank,
                               const void* shard, const void* xn, int32_t n_tokens,
                               const int32_t* topk_ids, const float* topk_weights,
                               void* partial_out, void* workspace, uint64_t workspace_bytes,
                               void* stream) {
  return moe_forward_impl(desc, moe, rank, shard, xn, n_tokens, topk_ids, topk_weights,
                          partial_out, workspace, workspace_bytes, stream, nullptr, nullptr);
}

tp_status tp_moe_shard_forward_timed(const tp_block_desc* desc, const tp_moe_desc* moe,
                                     int32_t rank, const void* shard, const void* xn,
                                     int32_t n_tokens, const int32_t* topk_ids,
                                     const float* topk_weights, void* partial_out,
                                     void* workspace, uint64_t workspace_bytes, void* stream,
                                     void* ev_begin, void* ev_end) {
  return moe_forward_impl(desc, moe, rank, shard, xn, n_tokens, topk_ids, topk_weights,
                          partial_out, workspace, workspace_bytes, stream, (hipEvent_t)ev_begin,
                          (hipEvent_t)ev_end);
}

tp_status tp_dequant_q8_0(const void* codes, const void* scales, float* out, uint64_t n_blocks,
                          void* stream) {
  if (n_blocks == 0) return TP_OK;
  if (!codes || !scales || !out)
    return fail(TP_ERR_INVALID_ARG, "codes, scales and out must be non-NULL");
  hipError_t e = tpk::q8_dequant_buf(codes, scales, out, (int64_t)n_blocks, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "tp_dequant_q8_0");
  return TP_OK;
}

// One region of a rank's packed shard as a plain [rows, K] matrix: the projection the forward
// path runs on it, for the test helpers below.
struct Region {
  const tp_region *w, *s;
  int K, rows;
};

static tp_status shard_region(const Dims& x, const tp_shard_layout& L, int32_t which, Region* r) {
  switch (which) {
    case 0: *r = Region{&L.qkv, &L.qkv_scale, x.d, x.qkv_rows}; return TP_OK;
    case 1: *r = Region{&L.o, &L.o_scale, x.qdim, x.d}; return TP_OK;
    case 2: *r = Region{&L.gate_up, &L.gate_up_scale, x.d, 2 * x.fr}; return TP_OK;
    case 3: *r = Region{&L.down, &L.down_scale, x.fr, x.d}; return TP_OK;
  }
  return fail(TP_ERR_INVALID_ARG, "which=%d must be 0 (qkv), 1 (o), 2 (gate_up) or 3 (down)",
              which);
}

static uint64_t project_ws_bytes(const Dims& x, int T, const Region& g) {
  if (x.wt == TP_DTYPE_BF16 && T <= 64 && use_gemm(x, T, g.K))
    return tpk::splitk_workspace_bytes(T, g.rows, g.K, false);
  if (use_q8_gemm(x, T)) return tpk::q8_gemm_workspace_bytes(T, g.rows, g.K, false);
  return 0;
}

tp_status tp_shard_project_workspace_size(const tp_block_desc* desc, int32_t which,
                                          int32_t n_tokens, uint64_t* bytes) {
  Dims x;
  if (tp_status s = check_desc(desc, &x)) return s;
  if (n_tokens < 0) return fail(TP_ERR_INVALID_ARG, "n_tokens=%d must be >= 0", n_tokens);
  if (!bytes) return fail(TP_ERR_INVALID_ARG, "bytes is NULL");
  tp_shard_layout L;
  make_layout(x, &L);
  Region g;
  if (tp_status s = shard_region(x, L, which, &g)) return s;
  const uint64_t b = project_ws_bytes(x, n_tokens, g);
  *bytes = b > 0 ? align_up(b) : kAlign;
  return TP_OK;
}

tp_status tp_shard_project(const tp_block_desc* desc, int32_t which, const void* shard,
                           const void* x_in, int32_t n_tokens, float* out, void* workspace,
                           uint64_t workspace_bytes, void* stream) {
  Dims x;
  if (tp_status s = check_desc(desc, &x)) return s;
  if (n_tokens < 0) return fail(TP_ERR_INVALID_ARG, "n_tokens=%d must be >= 0", n_tokens);
  tp_shard_layout L;
  make_layout(x, &L);
  Region g;
  if (tp_status s = shard_region(x, L, which, &g)) return s;
  if (n_tokens == 0) return TP_OK;
  if (!shard || !x_in || !out) return fail(TP_ERR_INVALID_ARG, "shard, x and out must be non-NULL");
  if (!aligned16(shard) || !aligned16(x_in) || !aligned16(out))
    return fail(TP_ERR_INVALID_ARG, "shard, x and out must be 16-byte aligned");
  if (tpk::gemv_max_tokens(g.K) < 1 && !use_gemm(x, n_tokens, g.K) && !use_q8_gemm(x, n_tokens))
    return fail(TP_ERR_UNSUPPORTED, "projection with K=%d exceeds the GEMV's 16384", g.K);
  const uint64_t need = project_ws_bytes(x, n_tokens, g);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(TP_ERR_BUFFER_TOO_SMALL, "workspace_bytes=%llu < %llu",
                (unsigned long long)workspace_bytes, (unsigned long long)need);
  const char* sh = (const char*)shard;
  hipError_t e = project(x, tpk::EPI_F32, n_tokens, sh + g.w->offset, sh + g.s->offset, g.K,
                         g.rows, 0, x_in, out, g.rows, (hipStream_t)stream, nullptr,
                         need > 0 ? (float*)workspace : nullptr);
  if (e != hipSuccess) return hip_fail(e, "tp_shard_project");
  g_err.clear();
  return TP_OK;
}

tp_status tp_workspace_size(const tp_block_desc* desc, const tp_batch* batch, uint64_t* bytes) {
  Dims x;
  if (tp_status s = check_desc(desc, &x)) return s;
  if (tp_status s = check_batch(x, batch, false)) return s;
  if (!bytes) return fail(TP_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = ws_layout(x, *batch).total;
  return TP_OK;
}

tp_status tp_step_workspace_size(const tp_block_desc* desc, const tp_batch* batch,
                                 uint64_t* bytes) {
  Dims x;
  if (tp_status s = check_desc(desc, &x)) return s;
  if (tp_status s = check_batch(x, batch, false)) return s;
  if (!bytes) return fail(TP_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = step_ws_bytes(x, *batch);
  return TP_OK;
}

tp_status tp_step_schedule(const tp_block_desc* desc, const tp_batch* batch, int32_t* schedule) {
  Dims x;
  if (tp_status s = check_desc(desc, &x)) return s;
  if (tp_status s = check_batch(x, batch, false)) return s;
  if (!schedule) return fail(TP_ERR_INVALID_ARG, "schedule is NULL");
  const int T = batch->n_tokens;
  *schedule = all_ranks_ok(x, *batch) ? TP_SCHEDULE_ALL_RANKS
                                      : (fused_step_ok(x, T) ? TP_SCHEDULE_PER_RANK
                                                             : TP_SCHEDULE_STAGED);
  return TP_OK;
}

tp_status tp_workspace_offsets(const tp_block_desc* desc, const tp_batch* batch,
                               uint64_t* q_offset, uint64_t* attn_offset, uint64_t* ffn_offset) {
  Dims x;
  if (tp_status s = check_desc(desc, &x)) return s;
  if (tp_status s = check_batch(x, batch, false)) return s;
  if (!q_offset || !attn_offset || !ffn_offset)
    return fail(TP_ERR_INVALID_ARG, "offset outputs must be non-NULL");
  const WsLayout w = ws_layout(x, *batch);
  *q_offset = w.q;
  *attn_offset = w.attn;
  *ffn_offset = w.ffn;
  return TP_OK;
}

tp_status tp_rope_table_bytes(const tp_block_desc* desc, uint64_t* bytes) {
  Dims x;
  if (tp_status s = check_desc(desc, &x)) return s;
  if (!bytes) return fail(TP_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = (uint64_t)x.maxpos * (x.hd / 2) * 2 * sizeof(float);
  return TP_OK;
}

tp_status tp_rope_table_init(const tp_block_desc* desc, void* dev_table, uint64_t table_bytes,
                             void* stream) {
  Dims x;
  if (tp_status s = check_desc(desc, &x)) return s;
  if (!dev_table) return fail(TP_ERR_INVALID_ARG, "dev_table is NULL");
  const uint64_t need = (uint64_t)x.maxpos * (x.hd / 2) * 2 * sizeof(float);
  if (table_bytes < need)
    return fail(TP_ERR_BUFFER_TOO_SMALL, "table_bytes=%llu < %llu", (unsigned long long)table_bytes,
                (unsigned long long)need);
  const int half = x.hd / 2;
  std::vector<float> host((size_t)x.maxpos * half * 2);
  for (int i = 0; i < half; ++i) {
    const double theta = std::pow((double)x.base, -2.0 * i / x.hd);
    for (int p = 0; p < x.maxpos; ++p) {
      const double a = (double)p * theta;
      host[((size_t)p * half + i) * 2] = (float)std::cos(a);
      host[((size_t)p * half + i) * 2 + 1] = (float)std::sin(a);
    }
  }
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(dev_table, host.data(), need, hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e, "tp_rope_table_init");
  return TP_OK;
}

// fin: norm prologue of the half's first projection (xn is then the residual stream, not its
// norm); fout: reduce epilogue of its row-parallel projection. Both only on the decode GEMVs.
static tp_status forward_impl(const tp_block_desc* desc, int32_t rank, int32_t half,
                              const void* shard, const tp_batch* batch, const void* xn,
                              const tp_kv_cache* kv, void* partial_out, void* workspace,
                              uint64_t workspace_bytes, void* stream, hipEvent_t evb,
                              hipEvent_t eve, const tpk::FuseArgs* fin = nullptr,
                              const tpk::FuseArgs* fout = nullptr) {
  Dims x;
  if (tp_status s = check_desc(desc, &x)) return s;
  if (rank < 0 || rank >= x.N) return fail(TP_ERR_RANK, "rank %d not in [0, %d)", rank, x.N);
  if (half != TP_HALF_ATTN && half != TP_HALF_FFN)
    return fail(TP_ERR_INVALID_ARG, "unknown half %d", half);
  const bool attn = half == TP_HALF_ATTN;
  if (tp_status s = check_batch(x, batch, attn)) return s;
  const int T = batch->n_tokens;
  if (T == 0) {
    g_err.clear();
    return TP_OK;
  }
  if (!shard || !xn || !partial_out || !workspace)
    return fail(TP_ERR_INVALID_ARG, "shard, xn, partial_out and workspace must be non-NULL");
  if (!aligned16(shard) || !aligned16(xn) || !aligned16(partial_out) || !aligned16(workspace))
    return fail(TP_ERR_INVALID_ARG, "shard, xn, partial_out and workspace must be 16-byte aligned");
  if (attn) {
    if (!kv || !kv->k_pages || !kv->v_pages || kv->n_pages <= 0)
      return fail(TP_ERR_INVALID_ARG, "ATTN needs a KV cache with non-NULL pages and n_pages > 0");
    if (!aligned16(kv->k_pages) || !aligned16(kv->v_pages))
      return fail(TP_ERR_INVALID_ARG, "KV pages must be 16-byte aligned");
  }
  const WsLayout w = ws_layout(x, *batch);
  if (workspace_bytes < w.total)
    return fail(TP_ERR_BUFFER_TOO_SMALL, "workspace_bytes=%llu < %llu",
                (unsigned long long)workspace_bytes, (unsigned long long)w.total);
  const bool gemm = x.wt == TP_DTYPE_BF16;
  const int kmax = attn ? (x.d > x.qdim ? x.d : x.qdim) : (x.d > x.fr ? x.d : x.fr);
  if (tpk::gemv_max_tokens(kmax) < 1 && !(gemm && T > 4))
    return fail(TP_ERR_UNSUPPORTED, "decode projection with K=%d exceeds the GEMV's 16384", kmax);

  tp_shard_layout L;
  make_layout(x, &L);
  hipStream_t st = (hipStream_t)stream;
  const char* sh = (const char*)shard;
  char* ws = (char*)workspace;
  if ((fin || fout) && !fused_step_ok(x, T))
    return fail(TP_ERR_UNSUPPORTED, "fused norm / reduce need single-launch decode GEMVs");
  const int epi_part = fout ? (x.pt == TP_DTYPE_F32 ? tpk::EPI_REDUCE : tpk::EPI_REDUCE_BF)
                            : (x.pt == TP_DTYPE_F32 ? tpk::EPI_F32 : tpk::EPI_BF16);
  const int at = x.at == TP_DTYPE_F32 ? tpk::ACT_F32 : tpk::ACT_BF16;
  float* skw = w.gemm_bytes > 0 ? (float*)(ws + w.gemm) : nullptr;
  hipError_t e;
  if (attn) {
    void* qkv = ws + w.qkv;
    tpk::RopeEpi re{};
    re.positions = batch->positions;
    re.block_table = batch->block_table;
    re.rope = batch->rope_table;
    re.q_out = ws + w.q;
    re.k_pages = kv->k_pages;
    re.v_pages = kv->v_pages;
    re.mode = batch->mode;
    re.max_pages = batch->max_pages;
    re.ps = x.ps;
    re.n_pages = kv->n_pages;
    re.pos_limit = w.pos_limit;
    re.hq = x.hq;
    re.hk = x.hk;
    re.hd = x.hd;
    const int ks = qkv_ksplit(x, T);
    int sk_parts = 0;
    if (use_gemm(x, T, x.d) && skw && at == tpk::ACT_BF16) {
      // Batched decode: the split-K projection's partial tiles go straight to the rotary / KV
      // append, which sums them (no separate epilogue launch).
      {
        TimedScope ts(evb, eve);
        e = tpk::launch_gemm_splitk(tpk::EPI_ACT, x.actf, T, x.qkv_rows, x.d, xn,
                                    sh + L.qkv.offset, nullptr, qkv, x.qkv_rows, skw, st, &sk_parts);
      }
      if (e != hipSuccess) return hip_fail(e, "qkv projection");
      e = tpk::launch_rope_append_parts(skw, sk_parts, T, x.hq, x.hk, x.hd, ws + w.q,
                                        batch->positions, batch->mode, batch->block_table,
                                        batch->max_pages, x.ps, kv->n_pages, w.pos_limit,
                                        kv->k_pages, kv->v_pages, batch->rope_table, st);
      if (e != hipSuccess) return hip_fail(e, "rotary embedding / KV append");
    } else if (ks > 1) {
      // Split-K projection on tiles that fill the chip, then the rotary embedding and the KV
      // append from the summed partials.
      float* parts = (float*)(ws + w.qkvp);
      {
        TimedScope ts(evb, eve);
        e = tpk::launch_gemm_split_f32(T, x.qkv_rows, x.d, xn, sh + L.qkv.offset, parts, ks, st);
      }
      if (e != hipSuccess) return hip_fail(e, "qkv projection");
      e = tpk::launch_rope_append_parts(parts, ks, T, x.hq, x.hk, x.hd, ws + w.q, batch->positions,
                                        batch->mode, batch->block_table, batch->max_pages, x.ps,
                                        kv->n_pages, w.pos_limit, kv->k_pages, kv->v_pages,
                                        batch->rope_table, st);
      if (e != hipSuccess) return hip_fail(e, "rotary embedding / KV append");
    } else if (use_gemm(x, T, x.d) && !skw && at == tpk::ACT_BF16 &&
               tpk::gemm_rope_supported(T, x.qkv_rows, x.d, x.hd)) {
      // Multi-token MFMA path with the rotary embedding and the KV append in the GEMM epilogue.
      {
        TimedScope ts(evb, eve);
        e = tpk::launch_gemm_qkv_rope(T, x.qkv_rows, x.d, xn, sh + L.qkv.offset, re, st);
      }
      if (e != hipSuccess) return hip_fail(e, "qkv projection");
    } else if (use_gemm(x, T, x.d) || use_q8_gemm(x, T)) {
      // Multi-token MFMA path: projection, then rotary embedding + KV append.
      {
        TimedScope ts(evb, eve);
        e = project(x, tpk::EPI_ACT, T, sh + L.qkv.offset, sh + L.qkv_scale.offset, x.d,
                    x.qkv_rows, 0, xn, qkv, x.qkv_rows, st, nullptr, skw);
      }
      if (e != hipSuccess) return hip_fail(e, "qkv projection");
      e = tpk::launch_rope_append(at, qkv, T, x.hq, x.hk, x.hd, ws + w.q, batch->positions,
                                  batch->mode, batch->block_table, batch->max_pages, x.ps,
                                  kv->n_pages, w.pos_limit, kv->k_pages, kv->v_pages,
                                  batch->rope_table, st);
      if (e != hipSuccess) return hip_fail(e, "rotary embedding / KV append");
    } else {
      // Decode path: the GEMV applies the rotary embedding and appends K/V in its epilogue.
      {
        TimedScope ts(evb, eve);
        e = project(x, tpk::EPI_ROPE, T, sh + L.qkv.offset, sh + L.qkv_scale.offset, x.d,
                    x.qkv_rows, 0, xn, qkv, x.qkv_rows, st, &re, nullptr, fin);
      }
      if (e != hipSuccess) return hip_fail(e, "qkv projection");
    }
    e = tpk::launch_attn_decode(at, x.hd, x.Hq / x.Hkv, T, x.hk, ws + w.q, kv->k_pages,
                                kv->v_pages, batch->positions, batch->mode, batch->block_table,
                                batch->max_pages, x.ps, kv->n_pages, w.chunk, w.n_split,
                                w.pos_limit, (float*)(ws + w.part_o), (float*)(ws + w.part_ml),
                                ws + w.attn, st);
    if (e != hipSuccess) return hip_fail(e, "attention");
    // bf16 o_proj of a batch (short rows, K = Hq/N * hd): the skinny GEMM reduces its K split
    // inside the workgroup, which measured faster than the split-K form and its epilogue launch.
    e = project(x, epi_part, T, sh + L.o.offset, sh + L.o_scale.offset, x.qdim, x.d, 0,
                ws + w.attn, partial_out, x.d, st, nullptr, x.wt == TP_DTYPE_BF16 ? nullptr : skw,
                fout);
    if (e != hipSuccess) return hip_fail(e, "o projection");
  } else {
    {
      TimedScope ts(evb, eve);
      e = project(x, tpk::EPI_GATED, T, sh + L.gate_up.offset, sh + L.gate_up_scale.offset, x.d,
                  x.fr, x.fr, xn, ws + w.ffn, x.fr, st, nullptr, skw, fin);
    }
    if (e != hipSuccess) return hip_fail(e, "gate/up projection");
    e = project(x, epi_part, T, sh + L.down.offset, sh + L.down_scale.offset, x.fr, x.d, 0,
                ws + w.ffn, partial_out, x.d, st, nullptr, skw, fout);
    if (e != hipSuccess) return hip_fail(e, "down projection");
  }
  g_err.clear();
  return TP_OK;
}

tp_status tp_block_shard_forward(const tp_block_desc* desc, int32_t rank, int32_t half,
                                 const void* shard, const tp_batch* batch, const void* xn,
                                 const tp_kv_cache* kv, void* partial_out, void* workspace,
                                 uint64_t workspace_bytes, void* stream) {
  return forward_impl(desc, rank, half, shard, batch, xn, kv, partial_out, workspace,
                      workspace_bytes, stream, nullptr, nullptr);
}

tp_status tp_block_shard_forward_timed(const tp_block_desc* desc, int32_t rank, int32_t half,
                                       const void* shard, const tp_batch* batch, const void* xn,
                                       const tp_kv_cache* kv, void* partial_out, void* workspace,
                                       uint64_t workspace_bytes, void* stream, void* ev_begin,
                                       void* ev_end) {
  return forward_impl(desc, rank, half, shard, batch, xn, kv, partial_out, workspace,
                      workspace_bytes, stream, (hipEvent_t)ev_begin, (hipEvent_t)ev_end);
}

}  // extern "C"

// Workspace of tp_block_shard_forward_noalloc: one array per GPU, loaded with the library and held
// until the process ends. Host code never passes `scratch` itself (its host-side name is not a
// device address); it uses the device address hipGetSymbolAddress returns for the current device.
static constexpr uint64_t kScratchBytes = 16ull << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

tp_status scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "tp_block_shard_forward_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(TP_ERR_UNSUPPORTED, "device %d: the static scratch is tracked for %d devices", dev,
                kMaxDevices);
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {};
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol,
                      "tp_block_shard_forward_noalloc: hipGetSymbolAddress(scratch)");
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return TP_OK;
}

}  // namespace

extern "C" {

tp_status tp_block_shard_forward_noalloc(const tp_block_desc* desc, int32_t rank, int32_t half,
                                         const void* shard, const tp_batch* batch, const void* xn,
                                         const tp_kv_cache* kv, void* partial_out, void* stream) {
  Dims x;
  if (tp_status s = check_desc(desc, &x)) return s;
  if (rank < 0 || rank >= x.N) return fail(TP_ERR_RANK, "rank %d not in [0, %d)", rank, x.N);
  if (half != TP_HALF_ATTN && half != TP_HALF_FFN)
    return fail(TP_ERR_INVALID_ARG, "unknown half %d", half);
  if (tp_status s = check_batch(x, batch, half == TP_HALF_ATTN)) return s;
  const uint64_t need = ws_layout(x, *batch).total;
  if (need > kScratchBytes)
    return fail(TP_ERR_BUFFER_TOO_SMALL,
                "this batch needs %llu bytes of workspace; the static scratch of "
                "tp_block_shard_forward_noalloc holds %llu (pass a workspace to "
                "tp_block_shard_forward instead)",
                (unsigned long long)need, (unsigned long long)kScratchBytes);
  if (batch->n_tokens == 0) {
    g_err.clear();
    return TP_OK;
  }
  void* ws = nullptr;
  if (tp_status s = scratch_ptr(&ws)) return s;
  return forward_impl(desc, rank, half, shard, batch, xn, kv, partial_out, ws, kScratchBytes,
                      stream, nullptr, nullptr);
}

// The attention halves of every rank with the fused norm and reduce (the decode GEMV path):
// rank r's QKV projection normalises x itself (rank 0 also stores xn) and the last rank's o_proj
// leaves h1 = x + (((P_0 + P_1) + ...) + P_{N-1}).
static tp_status attn_halves_fused(const tp_block_desc* desc, const Dims& x,
                                   const void* const* shards, const tp_batch* batch,
                                   const tp_kv_cache* kv, const void* x_in, const void* gamma1,
                                   void* partials, void* xn, void* h1, void* workspace,
                                   uint64_t workspace_bytes, void* stream) {
  const int T = batch->n_tokens, N = x.N;
  const size_t pstride = (size_t)T * x.d;
  const size_t pbytes = x.pt == TP_DTYPE_F32 ? 4 : 2;
  tpk::FuseArgs fin{};
  fin.eps = x.eps;
  fin.gamma = gamma1;
  tpk::FuseArgs fout{};
  fout.prev = partials;
  fout.part_stride = pstride;
  fout.n_prev = N - 1;
  fout.res_in = x_in;
  fout.res_out = h1;
  for (int r = 0; r < N; ++r) {
    fin.normed_out = r == 0 ? xn : nullptr;
    void* pr = (char*)partials + (size_t)r * pstride * pbytes;
    if (tp_status s = forward_impl(desc, r, TP_HALF_ATTN, shards[r], batch, x_in, &kv[r], pr,
                                   workspace, workspace_bytes, stream, nullptr, nullptr, &fin,
                                   r == N - 1 ? &fout : nullptr))
      return s;
  }
  return TP_OK;
}

// The attention halves of all ranks as three launches: every rank's QKV projection (with the norm
// prologue; rank 0's block also stores xn), every rank's attention and split merge, and every
// rank's o_proj with the rank-ordered reduce into h1. Rank r uses workspace copy r.
static tp_status attn_halves_ranks(const tp_block_desc* desc, const Dims& x,
                                   const void* const* shards, const tp_batch* batch,
                                   const tp_kv_cache* kv, const void* x_in, const void* gamma1,
                                   void* partials, void* xn, void* h1, void* workspace,
                                   uint64_t workspace_bytes, void* stream) {
  const int T = batch->n_tokens, N = x.N;
  const WsLayout w = ws_layout(x, *batch);
  const uint64_t wstride = align_up(w.total);
  if (workspace_bytes < (uint64_t)N * wstride)
    return fail(TP_ERR_BUFFER_TOO_SMALL, "workspace_bytes=%llu < %llu (one copy per rank)",
                (unsigned long long)workspace_bytes, (unsigned long long)N * wstride);
  if (!aligned16(workspace)) return fail(TP_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  for (int r = 0; r < N; ++r) {
    if (!shards[r] || !aligned16(shards[r]))
      return fail(TP_ERR_INVALID_ARG, "shard %d is NULL or not 16-byte aligned", r);
    if (!kv[r].k_pages || !kv[r].v_pages || kv[r].n_pages <= 0)
      return fail(TP_ERR_INVALID_ARG, "ATTN needs a KV cache with non-NULL pages and n_pages > 0");
    if (!aligned16(kv[r].k_pages) || !aligned16(kv[r].v_pages))
      return fail(TP_ERR_INVALID_ARG, "KV pages must be 16-byte aligned");
  }
  tp_shard_layout L;
  make_layout(x, &L);
  hipStream_t st = (hipStream_t)stream;
  const int wt = gemv_wt(x);
  const int at = x.at == TP_DTYPE_F32 ? tpk::ACT_F32 : tpk::ACT_BF16;
  const size_t pstride = (size_t)T * x.d, pbytes = x.pt == TP_DTYPE_F32 ? 4 : 2;
  auto wsr = [&](int r) { return (char*)workspace + (size_t)r * wstride; };
  auto shard = [&](int r) { return (const char*)shards[r]; };

  tpk::RankPtrs rq{};
  rq.n = N;
  for (int r = 0; r < N; ++r) {
    rq.w[r] = shard(r) + L.qkv.offset;
    rq.s[r] = (const uint16_t*)(shard(r) + L.qkv_scale.offset);
    rq.y[r] = wsr(r) + w.qkv;
    rq.q_out[r] = wsr(r) + w.q;
    rq.k_pages[r] = kv[r].k_pages;
    rq.v_pages[r] = kv[r].v_pages;
    rq.n_pages[r] = kv[r].n_pages;
  }
  tpk::RopeEpi re{};
  re.positions = batch->positions;
  re.block_table = batch->block_table;
  re.rope = batch->rope_table;
  re.mode = batch->mode;
  re.max_pages = batch->max_pages;
  re.ps = x.ps;
  re.pos_limit = w.pos_limit;
  re.hq = x.hq;
  re.hk = x.hk;
  re.hd = x.hd;
  tpk::FuseArgs fin{};
  fin.gamma = gamma1;
  fin.eps = x.eps;
  fin.normed_out = xn;
  hipError_t e = tpk::launch_gemv_ranks(wt, at, tpk::EPI_ROPE, x.actf, T, rq, x.d, x.qkv_rows, 0,
                                        x_in, x.qkv_rows, &re, st, fin);
  if (e != hipSuccess) return hip_fail(e, "qkv projection (all ranks)");

  tpk::AttnRanks ar{};
  ar.n = N;
  for (int r = 0; r < N; ++r) {
    ar.q[r] = wsr(r) + w.q;
    ar.k_pages[r] = kv[r].k_pages;
    ar.v_pages[r] = kv[r].v_pages;
    ar.n_pages[r] = kv[r].n_pages;
    ar.part_o[r] = (float*)(wsr(r) + w.part_o);
    ar.part_ml[r] = (float*)(wsr(r) + w.part_ml);
    ar.out[r] = wsr(r) + w.attn;
  }
  e = tpk::launch_attn_decode_ranks(at, x.hd, x.Hq / x.Hkv, T, x.hk, ar, batch->positions,
                                    batch->block_table, batch->max_pages, x.ps, w.chunk, w.n_split,
                                    w.pos_limit, st);
  if (e != hipSuccess) return hip_fail(e, "attention (all ranks)");

  tpk::RankPtrs ro{};
  ro.n = N;
  for (int r = 0; r < N; ++r) {
    ro.w[r] = shard(r) + L.o.offset;
    ro.s[r] = (const uint16_t*)(shard(r) + L.o_scale.offset);
    ro.x[r] = wsr(r) + w.attn;
    ro.y[r] = (char*)partials + (size_t)r * pstride * pbytes;
  }
  tpk::FuseArgs fo{};
  fo.res_in = x_in;
  fo.res_out = h1;
  e = tpk::launch_gemv_ranks(wt, at, x.pt == TP_DTYPE_F32 ? tpk::EPI_RED_ALL : tpk::EPI_RED_ALL_BF,
                             0, T, ro, x.qdim, x.d, 0, nullptr, x.d, nullptr, st, fo);
  if (e != hipSuccess) return hip_fail(e, "o projection and reduce (all ranks)");
  return TP_OK;
}

// The FFN half of all ranks as two launches: every rank's gate/up (norm prologue; rank 0's block
// stores xn2) and every rank's down projection with the rank-ordered reduce into out.
static tp_status ffn_halves_ranks(const tp_block_desc* desc, const Dims& x,
                                  const void* const* shards, const tp_batch* batch,
                                  const void* h1, const void* gamma2, void* partials, void* xn2,
                                  void* out, void* workspace, void* stream, hipEvent_t evb,
                                  hipEvent_t eve) {
  (void)desc;
  const int T = batch->n_tokens, N = x.N;
  const WsLayout w = ws_layout(x, *batch);
  const uint64_t wstride = align_up(w.total);
  tp_shard_layout L;
  make_layout(x, &L);
  hipStream_t st = (hipStream_t)stream;
  const int wt = gemv_wt(x);
  const int at = x.at == TP_DTYPE_F32 ? tpk::ACT_F32 : tpk::ACT_BF16;
  const size_t pstride = (size_t)T * x.d, pbytes = x.pt == TP_DTYPE_F32 ? 4 : 2;
  auto wsr = [&](int r) { return (char*)workspace + (size_t)r * wstride; };
  auto shard = [&](int r) { return (const char*)shards[r]; };
  tpk::RankPtrs rg{};
  rg.n = N;
  for (int r = 0; r < N; ++r) {
    rg.w[r] = shard(r) + L.gate_up.offset;
    rg.s[r] = (const uint16_t*)(shard(r) + L.gate_up_scale.offset);
    rg.y[r] = wsr(r) + w.ffn;
  }
  tpk::FuseArgs fin{};
  fin.gamma = gamma2;
  fin.eps = x.eps;
  fin.normed_out = xn2;
  hipError_t e;
  {
    TimedScope ts(evb, eve);
    e = tpk::launch_gemv_ranks(wt, at, tpk::EPI_GATED, x.actf, T, rg, x.d, x.fr, x.fr, h1, x.fr,
                               nullptr, st, fin);
  }
  if (e != hipSuccess) return hip_fail(e, "gate/up projection (all ranks)");
  tpk::RankPtrs rd{};
  rd.n = N;
  for (int r = 0; r < N; ++r) {
    rd.w[r] = shard(r) + L.down.offset;
    rd.s[r] = (const uint16_t*)(shard(r) + L.down_scale.offset);
    rd.x[r] = wsr(r) + w.ffn;
    rd.y[r] = (char*)partials + (size_t)r * pstride * pbytes;
  }
  tpk::FuseArgs fo{};
  fo.res_in = h1;
  fo.res_out = out;
  e = tpk::launch_gemv_ranks(wt, at, x.pt == TP_DTYPE_F32 ? tpk::EPI_RED_ALL : tpk::EPI_RED_ALL_BF,
                             0, T, rd, x.fr, x.d, 0, nullptr, x.d, nullptr, st, fo);
  if (e != hipSuccess) return hip_fail(e, "down projection and reduce (all ranks)");
  return TP_OK;
}

// The batched-decode or prefill block step with one launch per stage for all ranks
// (ranks_staged_ok, ranks_prefill_ok): xn = norm(x); every rank's split-K QKV, then its sum +
// rotary + KV append; every rank's attention (decode: and split merge); every rank's o_proj
// partial; h1, xn2 = reduce; every rank's gate/up; every rank's down partial; out = reduce. Each
// rank's work is exactly that of its own launches.
static tp_status staged_ranks(const tp_block_desc* desc, const Dims& x, const void* const* shards,
                              const tp_batch* batch, const tp_kv_cache* kv, const void* x_in,
                              const void* gamma1, const void* gamma2, void* partials, void* xn,
                              void* h1, void* xn2, void* out, void* workspace,
                              uint64_t workspace_bytes, void* stream, hipEvent_t evb,
                              hipEvent_t eve) {
  const int T = batch->n_tokens, N = x.N;
  const WsLayout w = step_ws_layout(x, *batch);
  const uint64_t wstride = align_up(w.total);
  if (workspace_bytes < (uint64_t)N * wstride)
    return fail(TP_ERR_BUFFER_TOO_SMALL, "workspace_bytes=%llu < %llu (one copy per rank)",
                (unsigned long long)workspace_bytes, (unsigned long long)N * wstride);
  if (!aligned16(workspace)) return fail(TP_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  for (int r = 0; r < N; ++r) {
    if (!shards[r] || !aligned16(shards[r]))
      return fail(TP_ERR_INVALID_ARG, "shard %d is NULL or not 16-byte aligned", r);
    if (!kv[r].k_pages || !kv[r].v_pages || kv[r].n_pages <= 0)
      return fail(TP_ERR_INVALID_ARG, "ATTN needs a KV cache with non-NULL pages and n_pages > 0");
    if (!aligned16(kv[r].k_pages) || !aligned16(kv[r].v_pages))
      return fail(TP_ERR_INVALID_ARG, "KV pages must be 16-byte aligned");
  }
  const bool prefill = batch->mode == TP_MODE_PREFILL;
  const bool q8 = x.wt == TP_DTYPE_Q8_0;
  if ((!prefill || q8) && w.gemm_bytes == 0)
    return fail(TP_ERR_UNSUPPORTED, "no split-K workspace for this batch");
  tp_shard_layout L;
  make_layout(x, &L);
  hipStream_t st = (hipStream_t)stream;
  const size_t pstride = (size_t)T * x.d, pbytes = x.pt == TP_DTYPE_F32 ? 4 : 2;
  const int epi_part = x.pt == TP_DTYPE_F32 ? tpk::EPI_F32 : tpk::EPI_BF16;
  auto wsr = [&](int r) { return (char*)workspace + (size_t)r * wstride; };
  auto shard = [&](int r) { return (const char*)shards[r]; };
  auto part = [&](int r) { return (void*)((char*)partials + (size_t)r * pstride * pbytes); };

  if (tp_status s = tp_partial_reduce(desc, T, nullptr, 0, x_in, nullptr, gamma1, xn, stream))
    return s;
  // QKV partial products: split-K tiles (batched, and Q8_0) or the wide split-K tiles (prefill).
  const uint64_t pofs = prefill && !q8 ? w.qkvp : w.gemm;
  tpk::GemmRanks gq{};
  gq.n = N;
  for (int r = 0; r < N; ++r) {
    gq.a[r] = xn;
    gq.b[r] = shard(r) + L.qkv.offset;
    gq.c[r] = wsr(r) + pofs;
  }
  int S = 0;
  hipError_t e;
  // Q8_0 projections: rank r's codes and block scales of one region (gated: gate rows, then the up
  // rows at row gate_off).
  auto q8ranks = [&](const tp_region& codes, const tp_region& scales, int K, int gate_off,
                     const void* const* in, void* const* outp, bool with_part) {
    tpk::Q8Ranks g{};
    g.n = N;
    for (int r = 0; r < N; ++r) {
      g.a[r] = in[r];
      g.q[r] = shard(r) + codes.offset;
      g.s[r] = shard(r) + scales.offset;
      if (gate_off > 0) {
        g.q2[r] = shard(r) + codes.offset + (size_t)gate_off * K;
        g.s2[r] = shard(r) + scales.offset + (size_t)gate_off * (K / 32) * 2;
      }
      g.c[r] = outp[r];
      g.part[r] = with_part ? (float*)(wsr(r) + w.gemm) : nullptr;
    }
    return g;
  };
  if (q8) {
    const void* in[tpk::kMaxRanks];
    void* outp[tpk::kMaxRanks];
    for (int r = 0; r < N; ++r) {
      in[r] = xn;
      outp[r] = wsr(r) + w.qkv;  // (unused: the tiles stay in the workspace)
    }
    const tpk::Q8Ranks g = q8ranks(L.qkv, L.qkv_scale, x.d, 0, in, outp, true);
    e = tpk::launch_gemm_q8_ranks(tpk::EPI_ACT, 0, T, x.qkv_rows, x.d, g, x.qkv_rows, st, true, &S);
  } else if (prefill) {
    // One rank's QKV tiles are too few to fill the chip, which is why the separate calls split K;
    // all ranks' tiles together usually are enough, and then each tile takes the whole K (one
    // fp32 sum per output, rounded once: the separate calls' q, k, v to rounding).
    const long tiles = (long)((T + 255) / 256) * ((x.qkv_rows + 159) / 160);
    S = tiles * N >= 192 ? 1 : qkv_ksplit(x, T);
    e = tpk::launch_gemm_split_f32(T, x.qkv_rows, x.d, nullptr, nullptr, nullptr, S, st, &gq);
  } else {
    e = tpk::launch_gemm_splitk_ranks(tpk::EPI_ACT, T, x.qkv_rows, x.d, gq, st, &S);
  }
  if (e != hipSuccess) return hip_fail(e, "qkv projection (all ranks)");
  tpk::RopeRanks rr{};
  rr.n = N;
  for (int r = 0; r < N; ++r) {
    rr.parts[r] = (const float*)(wsr(r) + pofs);
    rr.q_out[r] = wsr(r) + w.q;
    rr.k_pages[r] = kv[r].k_pages;
    rr.v_pages[r] = kv[r].v_pages;
    rr.n_pages[r] = kv[r].n_pages;
  }
  e = tpk::launch_rope_append_parts(rr.parts[0], S, T, x.hq, x.hk, x.hd, rr.q_out[0],
                                    batch->positions, batch->mode, batch->block_table,
                                    batch->max_pages, x.ps, rr.n_pages[0], w.pos_limit,
                                    rr.k_pages[0], rr.v_pages[0], batch->rope_table, st, &rr);
  if (e != hipSuccess) return hip_fail(e, "rotary embedding / KV append (all ranks)");
  tpk::AttnRanks ar{};
  ar.n = N;
  for (int r = 0; r < N; ++r) {
    ar.q[r] = wsr(r) + w.q;
    ar.k_pages[r] = kv[r].k_pages;
    ar.v_pages[r] = kv[r].v_pages;
    ar.n_pages[r] = kv[r].n_pages;
    ar.part_o[r] = (float*)(wsr(r) + w.part_o);
    ar.part_ml[r] = (float*)(wsr(r) + w.part_ml);
    ar.out[r] = wsr(r) + w.attn;
  }
  if (prefill)
    e = tpk::launch_attn_prefill(x.hd, x.Hq / x.Hkv, T, x.hk, nullptr, nullptr, nullptr,
                                 batch->positions, batch->block_table, batch->max_pages, 1,
                                 w.pos_limit, nullptr, st, &ar);
  else
    e = tpk::launch_attn_decode_ranks(tpk::ACT_BF16, x.hd, x.Hq / x.Hkv, T, x.hk, ar,
                                      batch->positions, batch->block_table, batch->max_pages,
                                      x.ps, w.chunk, w.n_split, w.pos_limit, st);
  if (e != hipSuccess) return hip_fail(e, "attention (all ranks)");
  // The projections: band GEMMs (batched) or wide tiles (prefill), as the separate calls pick.
  auto gemm = [&](int epi, int actf, int n_out, int K, int ldc, const tpk::GemmRanks* g) {
    return prefill ? tpk::launch_gemm_wide(epi, actf, T, n_out, K, nullptr, nullptr, nullptr,
                                           nullptr, ldc, st, g)
                   : tpk::launch_gemm_band(epi, actf, T, n_out, K, nullptr, nullptr, nullptr,
                                           nullptr, ldc, st, g);
  };
  int S8 = 0;
  auto q8gemm = [&](int epi, int actf, int n_out, int K, int ldc, const tp_region& codes,
                    const tp_region& scales, int gate_off, const void* const* in,
                    void* const* outp) {
    const tpk::Q8Ranks g = q8ranks(codes, scales, K, gate_off, in, outp, true);
    return tpk::launch_gemm_q8_ranks(epi, actf, T, n_out, K, g, ldc, st, false, &S8);
  };
  const void* in_o[tpk::kMaxRanks];
  void* out_p[tpk::kMaxRanks];
  for (int r = 0; r < N; ++r) {
    in_o[r] = wsr(r) + w.attn;
    out_p[r] = part(r);
  }
  tpk::GemmRanks go{};
  go.n = N;
  for (int r = 0; r < N; ++r) {
    go.a[r] = wsr(r) + w.attn;
    go.b[r] = shard(r) + L.o.offset;
    go.c[r] = part(r);
  }
  e = q8 ? q8gemm(epi_part, 0, x.d, x.qdim, x.d, L.o, L.o_scale, 0, in_o, out_p)
         : gemm(epi_part, 0, x.d, x.qdim, x.d, &go);
  if (e != hipSuccess) return hip_fail(e, "o projection (all ranks)");
  if (tp_status s = tp_partial_reduce(desc, T, partials, N, x_in, h1, gamma2, xn2, stream))
    return s;
  tpk::GemmRanks gg{};
  gg.n = N;
  for (int r = 0; r < N; ++r) {
    gg.a[r] = xn2;
    gg.b[r] = shard(r) + L.gate_up.offset;
    gg.b2[r] = shard(r) + L.gate_up.offset + (size_t)x.fr * x.d * 2;
    gg.c[r] = wsr(r) + w.ffn;
  }
  {
    TimedScope ts(evb, eve);
    if (q8) {
      const void* in[tpk::kMaxRanks];
      void* outp[tpk::kMaxRanks];
      for (int r = 0; r < N; ++r) {
        in[r] = xn2;
        outp[r] = wsr(r) + w.ffn;
      }
      e = q8gemm(tpk::EPI_GATED, x.actf, x.fr, x.d, x.fr, L.gate_up, L.gate_up_scale, x.fr, in,
                 outp);
    } else {
      e = gemm(tpk::EPI_GATED, x.actf, x.fr, x.d, x.fr, &gg);
    }
  }
  if (e != hipSuccess) return hip_fail(e, "gate/up projection (all ranks)");
  tpk::GemmRanks gd{};
  gd.n = N;
  for (int r = 0; r < N; ++r) {
    gd.a[r] = wsr(r) + w.ffn;
    gd.b[r] = shard(r) + L.down.offset;
    gd.c[r] = part(r);
  }
  if (q8) {
    const void* in[tpk::kMaxRanks];
    for (int r = 0; r < N; ++r) in[r] = wsr(r) + w.ffn;
    e = q8gemm(epi_part, 0, x.d, x.fr, x.d, L.down, L.down_scale, 0, in, out_p);
  } else {
    e = gemm(epi_part, 0, x.d, x.fr, x.d, &gd);
  }
  if (e != hipSuccess) return hip_fail(e, "down projection (all ranks)");
  return tp_partial_reduce(desc, T, partials, N, h1, out, nullptr, nullptr, stream);
}

static tp_status step_impl(const tp_block_desc* desc, const void* const* shards,
                           const tp_batch* batch, const tp_kv_cache* kv, const void* x_in,
                           const void* gamma1, const void* gamma2, void* partials, void* xn,
                           void* h1, void* xn2, void* out, void* workspace,
                           uint64_t workspace_bytes, void* stream, int32_t timed_rank,
                           hipEvent_t evb, hipEvent_t eve, int32_t schedule = -1) {
  Dims x;
  if (tp_status s = check_desc(desc, &x)) return s;
  if (tp_status s = check_batch(x, batch, true)) return s;
  const int T = batch->n_tokens, N = x.N;
  if (schedule < -1 || schedule > TP_SCHEDULE_ALL_RANKS)
    return fail(TP_ERR_INVALID_ARG, "unknown schedule %d", schedule);
  const bool can_fuse = fused_step_ok(x, T), can_all = all_ranks_ok(x, *batch);
  const int best = can_all ? TP_SCHEDULE_ALL_RANKS
                           : (can_fuse ? TP_SCHEDULE_PER_RANK : TP_SCHEDULE_STAGED);
  if ((schedule == TP_SCHEDULE_PER_RANK && !can_fuse) ||
      (schedule == TP_SCHEDULE_ALL_RANKS && !can_all))
    return fail(TP_ERR_UNSUPPORTED, "schedule %d is not available for this batch", schedule);
  const int sched = schedule < 0 ? best : schedule;
  if (T == 0) {
    g_err.clear();
    return TP_OK;
  }
  if (!shards || !kv) return fail(TP_ERR_INVALID_ARG, "shards and kv must be non-NULL arrays");
  if (!x_in || !gamma1 || !gamma2 || !partials || !xn || !h1 || !xn2 || !out)
    return fail(TP_ERR_INVALID_ARG,
                "x, gamma1, gamma2, partials, xn, h1, xn2 and out must be non-NULL");
  const void* bufs[8] = {x_in, gamma1, gamma2, partials, xn, h1, xn2, out};
  for (const void* b : bufs)
    if (!aligned16(b)) return fail(TP_ERR_INVALID_ARG, "step buffers must be 16-byte aligned");
  const size_t pstride = (size_t)T * x.d;
  const size_t pbytes = x.pt == TP_DTYPE_F32 ? 4 : 2;
  char* P = (char*)partials;
  auto part = [&](int r) { return (void*)(P + (size_t)r * pstride * pbytes); };
  auto timing = [&](int r) -> std::pair<hipEvent_t, hipEvent_t> {
    return r == timed_rank ? std::make_pair(evb, eve) : std::make_pair(hipEvent_t{}, hipEvent_t{});
  };
  if (sched == TP_SCHEDULE_ALL_RANKS && !can_fuse) {
    const bool timed = timed_rank >= 0 && timed_rank < N;
    if (tp_status s = staged_ranks(desc, x, shards, batch, kv, x_in, gamma1, gamma2, partials, xn,
                                   h1, xn2, out, workspace, workspace_bytes, stream,
                                   timed ? evb : nullptr, timed ? eve : nullptr))
      return s;
    g_err.clear();
    return TP_OK;
  }
  if (sched == TP_SCHEDULE_STAGED) {
    // The staged sequence of the same library calls.
    if (tp_status s = tp_partial_reduce(desc, T, nullptr, 0, x_in, nullptr, gamma1, xn, stream))
      return s;
    for (int r = 0; r < N; ++r)
      if (tp_status s = forward_impl(desc, r, TP_HALF_ATTN, shards[r], batch, xn, &kv[r], part(r),
                                     workspace, workspace_bytes, stream, nullptr, nullptr))
        return s;
    if (tp_status s = tp_partial_reduce(desc, T, partials, N, x_in, h1, gamma2, xn2, stream))
      return s;
    for (int r = 0; r < N; ++r) {
      const auto ev = timing(r);
      if (tp_status s = forward_impl(desc, r, TP_HALF_FFN, shards[r], batch, xn2, nullptr, part(r),
                                     workspace, workspace_bytes, stream, ev.first, ev.second))
        return s;
    }
    return tp_partial_reduce(desc, T, partials, N, h1, out, nullptr, nullptr, stream);
  }
  if (sched == TP_SCHEDULE_ALL_RANKS) {
    // One launch per projection and for the attention, covering every rank.
    if (tp_status s = attn_halves_ranks(desc, x, shards, batch, kv, x_in, gamma1, partials, xn,
                                        h1, workspace, workspace_bytes, stream))
      return s;
    const bool timed = timed_rank >= 0 && timed_rank < N;
    if (tp_status s = ffn_halves_ranks(desc, x, shards, batch, h1, gamma2, partials, xn2, out,
                                       workspace, stream, timed ? evb : nullptr,
                                       timed ? eve : nullptr))
      return s;
    g_err.clear();
    return TP_OK;
  }
  // Fused schedule: every rank's first projection normalises the residual stream itself, and
  // the last rank's row-parallel projection adds all ranks' partials (rank order) and the
  // residual. The partials are still stored per rank.
  if (tp_status s = attn_halves_fused(desc, x, shards, batch, kv, x_in, gamma1, partials, xn, h1,
                                      workspace, workspace_bytes, stream))
    return s;
  tpk::FuseArgs fin{};
  fin.eps = x.eps;
  tpk::FuseArgs fout{};
  fout.prev = partials;
  fout.part_stride = pstride;
  fout.n_prev = N - 1;
  for (int r = 0; r < N; ++r) {
    fin.gamma = gamma2;
    fin.normed_out = r == 0 ? xn2 : nullptr;
    fout.res_in = h1;
    fout.res_out = out;
    const auto ev = timing(r);
    if (tp_status s = forward_impl(desc, r, TP_HALF_FFN, shards[r], batch, h1, nullptr, part(r),
                                   workspace, workspace_bytes, stream, ev.first, ev.second, &fin,
                                   r == N - 1 ? &fout : nullptr))
      return s;
  }
  g_err.clear();
  return TP_OK;
}

// evb / eve (optional): bracket the expert gate/up launch of every rank when the step takes the
// all-ranks expert launches, else rank 0's expert half.
static tp_status moe_step_impl(const tp_block_desc* desc, const tp_moe_desc* moe,
                               const void* const* shards, const void* const* moe_shards,
                               const tp_batch* batch, const tp_kv_cache* kv, const void* x_in,
                               const void* gamma1, const void* gamma2, const void* router,
                               void* partials, void* xn, void* h1, void* xn2, void* out,
                               float* logits, int32_t* topk_ids, float* topk_weights,
                               void* workspace, uint64_t workspace_bytes, void* moe_workspace,
                               uint64_t moe_workspace_bytes, void* stream, hipEvent_t evb,
                               hipEvent_t eve) {
  Dims x;
  MoeDims m;
  if (tp_status s = check_moe(desc, moe, &x, &m)) return s;
  if (tp_status s = check_batch(x, batch, true)) return s;
  const int T = batch->n_tokens, N = x.N;
  if (T == 0) {
    g_err.clear();
    return TP_OK;
  }
  if (!shards || !moe_shards || !kv)
    return fail(TP_ERR_INVALID_ARG, "shards, moe_shards and kv must be non-NULL arrays");
  if (!x_in || !gamma1 || !gamma2 || !router || !partials || !xn || !h1 || !xn2 || !out ||
      !logits || !topk_ids || !topk_weights)
    return fail(TP_ERR_INVALID_ARG, "every buffer of the MoE block step must be non-NULL");
  const void* bufs[10] = {x_in, gamma1, gamma2, router, partials, xn, h1, xn2, out, logits};
  for (const void* b : bufs)
    if (!aligned16(b)) return fail(TP_ERR_INVALID_ARG, "step buffers must be 16-byte aligned");
  const size_t pstride = (size_t)T * x.d;
  const size_t pbytes = x.pt == TP_DTYPE_F32 ? 4 : 2;
  auto part = [&](int r) { return (void*)((char*)partials + (size_t)r * pstride * pbytes); };
  const bool fused = fused_step_ok(x, T);
  // With room for every rank's expert activations in moe_workspace, a decode step runs the
  // ranks' expert gate/up projections as one launch (each block's work that of its rank's own
  // launch), and with at most 64 experts that launch also selects the experts (no top-k launch).
  uint64_t mws = 0;
  tp_moe_workspace_size(desc, moe, T, &mws);
  const bool ranks_experts = fused && N > 1 && moe_workspace && aligned16(moe_workspace) &&
                             moe_workspace_bytes >= (uint64_t)N * mws;
  const bool fold_topk = ranks_experts && m.E <= 64;
  if (fused) {
    if (ranks_step_ok(x, T)) {
      if (tp_status s = attn_halves_ranks(desc, x, shards, batch, kv, x_in, gamma1, partials, xn,
                                          h1, workspace, workspace_bytes, stream))
        return s;
    } else if (tp_status s = attn_halves_fused(desc, x, shards, batch, kv, x_in, gamma1, partials,
                                               xn, h1, workspace, workspace_bytes, stream)) {
      return s;
    }
    // The router normalises h1 itself and stores xn2 for the experts.
    tpk::FuseArgs fin{};
    fin.eps = x.eps;
    fin.gamma = gamma2;
    fin.normed_out = xn2;
    hipStream_t st = (hipStream_t)stream;
    const int at = x.at == TP_DTYPE_F32 ? tpk::ACT_F32 : tpk::ACT_BF16;
    const int wt = x.at == TP_DTYPE_F32 ? tpk::W_F32 : tpk::W_BF16;
    hipError_t e = tpk::launch_gemv(wt, at, tpk::EPI_F32, 0, T, router, nullptr, x.d, m.E, 0, h1,
                                    logits, m.E, nullptr, st, &fin);
    if (e == hipSuccess && !fold_topk)
      e = tpk::launch_moe_topk(logits, T, m.E, m.k, topk_ids, topk_weights, st);
    if (e != hipSuccess) return hip_fail(e, "tp_moe_block_step: router");
  } else {
    if (tp_status s = tp_partial_reduce(desc, T, nullptr, 0, x_in, nullptr, gamma1, xn, stream))
      return s;
    for (int r = 0; r < N; ++r)
      if (tp_status s = forward_impl(desc, r, TP_HALF_ATTN, shards[r], batch, xn, &kv[r], part(r),
                                     workspace, workspace_bytes, stream, nullptr, nullptr))
        return s;
    if (tp_status s = tp_partial_reduce(desc, T, partials, N, x_in, h1, gamma2, xn2, stream))
      return s;
    if (tp_status s = tp_moe_route(desc, moe, router, xn2, T, logits, topk_ids, topk_weights,
                                   stream))
      return s;
  }
  tpk::FuseArgs fout{};
  fout.prev = partials;
  fout.part_stride = pstride;
  fout.n_prev = N - 1;
  fout.res_in = h1;
  fout.res_out = out;
  // The all-ranks expert launches: the gate/up of every rank (selecting the experts when the
  // top-k launch was skipped), then the down of every rank or each rank's down, the last one
  // adding the partials and the residual.
  if (ranks_experts) {
    for (int r = 0; r < N; ++r)
      if (!moe_shards[r] || !aligned16(moe_shards[r]))
        return fail(TP_ERR_INVALID_ARG, "moe shard %d is NULL or not 16-byte aligned", r);
    tp_moe_layout L;
    make_moe_layout(x, m, &L);
    const int wt = x.wt == TP_DTYPE_F32 ? tpk::W_F32 : (x.wt == TP_DTYPE_BF16 ? tpk::W_BF16 : tpk::W_Q8);
    const int at = x.at == TP_DTYPE_F32 ? tpk::ACT_F32 : tpk::ACT_BF16;
    const int pt = x.pt == TP_DTYPE_F32 ? tpk::ACT_F32 : tpk::ACT_BF16;
    hipStream_t st = (hipStream_t)stream;
    tpk::MoeRanks mr{};
    mr.n = N;
    for (int r = 0; r < N; ++r) {
      const char* sh = (const char*)moe_shards[r];
      mr.wg[r] = sh + L.gate.offset;
      mr.sg[r] = sh + L.gate_scale.offset;
      mr.wu[r] = sh + L.up.offset;
      mr.su[r] = sh + L.up_scale.offset;
      mr.m[r] = (char*)moe_workspace + (size_t)r * mws;
    }
    hipError_t e;
    {
      TimedScope ts(evb, eve);
      e = tpk::launch_moe_gate_up_ranks(wt, at, x.actf, x.d, m.fr, m.E, m.k, T, topk_ids, xn2, mr,
                                        st, fold_topk ? logits : nullptr, topk_weights);
    }
    if (e != hipSuccess) return hip_fail(e, "moe gate/up (all ranks)");
    if (tpk::moe_down_ranks_fit(N, m.k, m.fr)) {
      // Every rank's down in one launch, the reduce in it (as the last rank's down adds it).
      for (int r = 0; r < N; ++r) {
        const char* sh = (const char*)moe_shards[r];
        mr.wd[r] = sh + L.down.offset;
        mr.sd[r] = sh + L.down_scale.offset;
        mr.p[r] = part(r);
      }
      e = tpk::launch_moe_down_ranks(wt, at, pt, x.d, m.fr, m.E, m.k, T, topk_ids, topk_weights,
                                     mr, h1, out, st);
      if (e != hipSuccess) return hip_fail(e, "moe down (all ranks)");
      g_err.clear();
      return TP_OK;
    }
    for (int r = 0; r < N; ++r) {
      const char* sh = (const char*)moe_shards[r];
      e = tpk::launch_moe_down(wt, at, pt, sh + L.down.offset, sh + L.down_scale.offset, x.d,
                               m.fr, m.E, m.k, T, topk_ids, topk_weights, mr.m[r], part(r), st,
                               r == N - 1 ? &fout : nullptr);
      if (e != hipSuccess) return hip_fail(e, "moe down");
    }
    g_err.clear();
    return TP_OK;
  }
  for (int r = 0; r < N; ++r) {
    if (tp_status s = moe_forward_impl(desc, moe, r, moe_shards[r], xn2, T, topk_ids, topk_weights,
                                       part(r), moe_workspace, moe_workspace_bytes, stream,
                                       r == 0 ? evb : nullptr, r == 0 ? eve : nullptr,
                                       fused && r == N - 1 ? &fout : nullptr))
      return s;
  }
  if (!fused) return tp_partial_reduce(desc, T, partials, N, h1, out, nullptr, nullptr, stream);
  g_err.clear();
  return TP_OK;
}

tp_status tp_moe_block_step(const tp_block_desc* desc, const tp_moe_desc* moe,
                            const void* const* shards, const void* const* moe_shards,
                            const tp_batch* batch, const tp_kv_cache* kv, const void* x_in,
                            const void* gamma1, const void* gamma2, const void* router,
                            void* partials, void* xn, void* h1, void* xn2, void* out,
                            float* logits, int32_t* topk_ids, float* topk_weights,
                            void* workspace, uint64_t workspace_bytes, void* moe_workspace,
                            uint64_t moe_workspace_bytes, void* stream) {
  return moe_step_impl(desc, moe, shards, moe_shards, batch, kv, x_in, gamma1, gamma2, router,
                       partials, xn, h1, xn2, out, logits, topk_ids, topk_weights, workspace,
                       workspace_bytes, moe_workspace, moe_workspace_bytes, stream, nullptr,
                       nullptr);
}

tp_status tp_moe_block_step_timed(const tp_block_desc* desc, const tp_moe_desc* moe,
                                  const void* const* shards, const void* const* moe_shards,
                                  const tp_batch* batch, const tp_kv_cache* kv, const void* x_in,
                                  const void* gamma1, const void* gamma2, const void* router,
                                  void* partials, void* xn, void* h1, void* xn2, void* out,
                                  float* logits, int32_t* topk_ids, float* topk_weights,
                                  void* workspace, uint64_t workspace_bytes, void* moe_workspace,
                                  uint64_t moe_workspace_bytes, void* stream, void* ev_begin,
                                  void* ev_end) {
  if (!ev_begin || !ev_end) return fail(TP_ERR_INVALID_ARG, "ev_begin and ev_end must be non-NULL");
  return moe_step_impl(desc, moe, shards, moe_shards, batch, kv, x_in, gamma1, gamma2, router,
                       partials, xn, h1, xn2, out, logits, topk_ids, topk_weights, workspace,
                       workspace_bytes, moe_workspace, moe_workspace_bytes, stream,
                       (hipEvent_t)ev_begin, (hipEvent_t)ev_end);
}

tp_status tp_block_step(const tp_block_desc* desc, const void* const* shards, const tp_batch* batch,
                        const tp_kv_cache* kv, const void* x, const void* gamma1,
                        const void* gamma2, void* partials, void* xn, void* h1, void* xn2,
                        void* out, void* workspace, uint64_t workspace_bytes, void* stream) {
  return step_impl(desc, shards, batch, kv, x, gamma1, gamma2, partials, xn, h1, xn2, out,
                   workspace, workspace_bytes, stream, -1, nullptr, nullptr);
}

tp_status tp_block_step_with_schedule(const tp_block_desc* desc, int32_t schedule,
                                      const void* const* shards, const tp_batch* batch,
                                      const tp_kv_cache* kv, const void* x, const void* gamma1,
                                      const void* gamma2, void* partials, void* xn, void* h1,
                                      void* xn2, void* out, void* workspace,
                                      uint64_t workspace_bytes, void* stream) {
  return step_impl(desc, shards, batch, kv, x, gamma1, gamma2, partials, xn, h1, xn2, out,
                   workspace, workspace_bytes, stream, -1, nullptr, nullptr, schedule);
}

tp_status tp_block_step_timed(const tp_block_desc* desc, const void* const* shards,
                              const tp_batch* batch, const tp_kv_cache* kv, const void* x,
                              const void* gamma1, const void* gamma2, void* partials, void* xn,
                              void* h1, void* xn2, void* out, void* workspace,
                              uint64_t workspace_bytes, void* stream, int32_t timed_rank,
                              void* ev_begin, void* ev_end) {
  return step_impl(desc, shards, batch, kv, x, gamma1, gamma2, partials, xn, h1, xn2, out,
                   workspace, workspace_bytes, stream, timed_rank, (hipEvent_t)ev_begin,
                   (hipEvent_t)ev_end);
}

tp_status tp_partial_reduce(const tp_block_desc* desc, int32_t n_tokens, const void* partials,
                            int32_t n_partials, const void* residual_in, void* residual_out,
                            const void* gamma, void* normed_out, void* stream) {
  Dims x;
  if (tp_status s = check_desc(desc, &x)) return s;
  if (n_tokens < 0 || n_partials < 0)
    return fail(TP_ERR_INVALID_ARG, "n_tokens=%d and n_partials=%d must be >= 0", n_tokens,
                n_partials);
  if (n_tokens == 0) return TP_OK;
  if (!residual_in) return fail(TP_ERR_INVALID_ARG, "residual_in is NULL");
  if (n_partials > 0 && (!partials || !residual_out))
    return fail(TP_ERR_INVALID_ARG, "n_partials=%d needs non-NULL partials and residual_out",
                n_partials);
  if (gamma && !normed_out) return fail(TP_ERR_INVALID_ARG, "gamma given but normed_out is NULL");
  if (!gamma && n_partials == 0)
    return fail(TP_ERR_INVALID_ARG, "nothing to do: no partials and no gamma");
  if (!aligned16(residual_in) || (residual_out && !aligned16(residual_out)) ||
      (partials && !aligned16(partials)) || (gamma && !aligned16(gamma)) ||
      (normed_out && !aligned16(normed_out)))
    return fail(TP_ERR_INVALID_ARG, "reduce buffers must be 16-byte aligned");
  const int at = x.at == TP_DTYPE_F32 ? tpk::ACT_F32 : tpk::ACT_BF16;
  const int pt = x.pt == TP_DTYPE_F32 ? tpk::ACT_F32 : tpk::ACT_BF16;
  hipError_t e = tpk::launch_partial_reduce(at, pt, n_tokens, x.d, partials, n_partials,
                                            residual_in, residual_out, gamma, normed_out, x.eps,
                                            (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "tp_partial_reduce");
  g_err.clear();
  return TP_OK;
}

}  // extern "C"
