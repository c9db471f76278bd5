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
  const FuseArgs fa = fuse ? *fuse : FuseArgs{};
  RopeEpi re = rope ? *rope : RopeEpi{};
  if (!rope) re.hd = 2;  // unused by non-rotary epilogues; keeps the row mapping well defined
  for (int t0 = 0; t0 < T; t0 += ntmax) {
    const int nt = (T - t0) < ntmax ? (T - t0) : ntmax;
    const void* Xt = (const char*)X + (size_t)t0 * K * xb;
    void* Yt = (char*)Y + (size_t)t0 * ldy * yb;
    re.t0 = t0;
    hipError_t e;
    const uint16_t* s16 = (const uint16_t*)S;
    if (wt == W_F32 && at == ACT_F32)
      e = gemv_f32(epi, actf, nt, W, s16, K, n_out, gate_off, Xt, Yt, ldy, re, fa, st);
    else if (wt == W_BF16 && at == ACT_BF16)
      e = gemv_bf16(epi, actf, nt, W, s16, K, n_out, gate_off, Xt, Yt, ldy, re, fa, st);
    else if (wt == W_Q8 && at == ACT_BF16)
      e = gemv_q8(epi, actf, nt, W, s16, K, n_out, gate_off, Xt, Yt, ldy, re, fa, st);
    else
      return hipErrorInvalidValue;
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace tpk
