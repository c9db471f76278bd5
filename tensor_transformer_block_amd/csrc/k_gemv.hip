// Host dispatch of the decode projections (K2 / K3): token groups of at most four per launch.
#include "k_gemv_impl.h"

namespace tpk {

int gemv_max_tokens(int K) {
  int nt = 16384 / K;
  return nt > 4 ? 4 : nt;
}

hipError_t launch_gemv(int wt, int at, int epi, int actf, int T, const void* W, const void* S,
                       int K, int n_out, int gate_off, const void* X, void* Y, int ldy,
                       const RopeEpi* rope, hipStream_t st, const FuseArgs* fuse) {
  const int ntmax = gemv_max_tokens(K);
  if (ntmax < 1) return hipErrorInvalidValue;
  if (epi == EPI_ROPE && !rope) return hipErrorInvalidValue;
  const size_t xb = (at == ACT_F32) ? 4 : 2;
  const size_t yb = (epi == EPI_F32) ? 4 : ((epi == EPI_BF16) ? 2 : xb);
  if ((epi == EPI_REDUCE || epi == EPI_REDUCE_BF) && (!fuse || !fuse->res_in || !fuse->res_out || fuse->n_prev < 0 ||
                            fuse->n_prev > kMaxPrevPartials || (fuse->n_prev > 0 && !fuse->prev)))
    return hipErrorInvalidValue;
  // The fused prologue and reduce handle one token group (their rows must stay whole).
  if (fuse && T > ntmax) return hipErrorInvalidValue;
  if (epi == EPI_RED_ALL || epi == EPI_RED_ALL_BF) return hipErrorInvalidValue;
  const FuseArgs fa = fuse ? *fuse : FuseArgs{};
  RopeEpi re = rope ? *rope : RopeEpi{};
  if (!rope) re.hd = 2;  // unused by non-rotary epilogues; keeps the row mapping well defined
  const RankPtrs rp{};  // a single rank's launch
  for (int t0 = 0; t0 < T; t0 += ntmax) {
    const int nt = (T - t0) < ntmax ? (T - t0) : ntmax;
    const void* Xt = (const char*)X + (size_t)t0 * K * xb;
    void* Yt = (char*)Y + (size_t)t0 * ldy * yb;
    re.t0 = t0;
    hipError_t e;
    const uint16_t* s16 = (const uint16_t*)S;
    if (wt == W_F32 && at == ACT_F32)
      e = gemv_f32(epi, actf, nt, W, s16, K, n_out, gate_off, Xt, Yt, ldy, re, fa, rp, st);
    else if (wt == W_BF16 && at == ACT_BF16)
      e = gemv_bf16(epi, actf, nt, W, s16, K, n_out, gate_off, Xt, Yt, ldy, re, fa, rp, st);
    else if (wt == W_Q8 && at == ACT_BF16)
      e = gemv_q8(epi, actf, nt, W, s16, K, n_out, gate_off, Xt, Yt, ldy, re, fa, rp, st);
    else
      return hipErrorInvalidValue;
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Staged bytes of a launch over all ranks: EPI_RED_ALL* stages every rank's input rows.
static size_t ranks_lds(int wt, int epi, int n_ranks, int T, int K) {
  const bool allr = epi == EPI_RED_ALL || epi == EPI_RED_ALL_BF;
  const size_t xb = (allr && wt != W_F32) ? 2 : 4;  // bf16 rows stay bf16 there
  // Q8_0: fp16 rows and an (offset, 1 / scale) pair per 16 values.
  const size_t one = wt == W_Q8 ? (size_t)T * K * 2 + (size_t)T * (K / 16) * 8 : (size_t)T * K * xb;
  return (allr ? (size_t)n_ranks : 1) * one;
}

bool gemv_ranks_fit(int wt, int epi, int n_ranks, int T, int K) {
  const bool allr = epi == EPI_RED_ALL || epi == EPI_RED_ALL_BF;
  return n_ranks >= 1 && n_ranks <= (allr ? 4 : kMaxRanks) && T >= 1 &&
         T <= gemv_max_tokens(K) && ranks_lds(wt, epi, n_ranks, T, K) <= 160 * 1024;
}

hipError_t launch_gemv_ranks(int wt, int at, int epi, int actf, int T, const RankPtrs& rp, int K,
                             int n_out, int gate_off, const void* X, int ldy, const RopeEpi* rope,
                             hipStream_t st, const FuseArgs& fuse) {
  const bool allr = epi == EPI_RED_ALL || epi == EPI_RED_ALL_BF;
  if (!gemv_ranks_fit(wt, epi, rp.n, T, K)) return hipErrorInvalidValue;
  if (!(allr || epi == EPI_ROPE || epi == EPI_GATED)) return hipErrorInvalidValue;
  if (epi == EPI_ROPE && !rope) return hipErrorInvalidValue;
  if (allr && (!fuse.res_in || !fuse.res_out || fuse.gamma)) return hipErrorInvalidValue;
  for (int r = 0; r < rp.n; ++r)
    if (!rp.w[r] || !rp.y[r] || (allr && !rp.x[r]) || (wt == W_Q8 && !rp.s[r]))
      return hipErrorInvalidValue;
  RopeEpi re = rope ? *rope : RopeEpi{};
  if (!rope) re.hd = 2;
  re.t0 = 0;
  const uint16_t* s16 = (const uint16_t*)rp.s[0];
  // Rank 0's pointers also go in the plain arguments (used as they are when rp.n == 1).
  if (rope) {
    re.q_out = rp.q_out[0];
    re.k_pages = rp.k_pages[0];
    re.v_pages = rp.v_pages[0];
    re.n_pages = rp.n_pages[0];
  }
  if (wt == W_F32 && at == ACT_F32)
    return gemv_f32(epi, actf, T, rp.w[0], s16, K, n_out, gate_off, X, rp.y[0], ldy, re, fuse, rp, st);
  if (wt == W_BF16 && at == ACT_BF16)
    return gemv_bf16(epi, actf, T, rp.w[0], s16, K, n_out, gate_off, X, rp.y[0], ldy, re, fuse, rp, st);
  if (wt == W_Q8 && at == ACT_BF16)
    return gemv_q8(epi, actf, T, rp.w[0], s16, K, n_out, gate_off, X, rp.y[0], ldy, re, fuse, rp, st);
  return hipErrorInvalidValue;
}

}  // namespace tpk
