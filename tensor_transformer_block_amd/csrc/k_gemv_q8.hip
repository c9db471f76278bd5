// Decode projections for one weight format; the kernel template is in k_gemv_impl.h.
#include "k_gemv_impl.h"

namespace tpk {

hipError_t gemv_q8(int epi, int actf, int nt, const void* W, const uint16_t* S, int K, int n_out,
                   int gate_off, const void* X, void* Y, int ldy, const RopeEpi& re, const FuseArgs& fa,
                   const RankPtrs& rp,
                   hipStream_t st) {
  return gemv_format<W_Q8, ACT_BF16>(epi, actf, nt, W, S, K, n_out, gate_off, X, Y, ldy, re, fa, rp, st);
}

}  // namespace tpk
