// Decode projections for one weight format; the kernel template is in k_gemv_impl.h.
#include "k_gemv_impl.h"

namespace tpk {

hipError_t gemv_f32(int epi, int actf, int nt, const void* W, const uint16_t* S, int K, int n_out,
                   int gate_off, const void* X, void* Y, int ldy, const RopeEpi& re, const FuseArgs& fa,
                   const RankPtrs& rp,
                   hipStream_t st) {
  return gemv_format<W_F32, ACT_F32>(epi, actf, nt, W, S, K, n_out, gate_off, X, Y, ldy, re, fa, rp, st);
}

}  // namespace tpk
