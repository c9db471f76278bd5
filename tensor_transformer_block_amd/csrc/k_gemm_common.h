// Types and helpers shared by the MFMA GEMM kernels (k_gemm.hip, k_gemm_wide.hip, k_attn_prefill.hip).
#pragma once
#include "tp_common.h"

namespace tpk {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// Cache-policy bits of a direct-to-LDS load: kStreamAux is the non-temporal bit. The band GEMM's
// weight stream takes it (the 64-sequence batched step 206.3 -> 201.4 us); the split-K QKV's
// weights measured faster without it (198.6 us against 201.4), and the prefill tiles re-read
// their operands.
constexpr int kStreamAux = 2;

template <int N_OUT>
__device__ __forceinline__ void wait_vmcnt() {
  // s_waitcnt with vmcnt = N_OUT (6-bit, split field), expcnt and lgkmcnt left at "no wait".
  __builtin_amdgcn_s_waitcnt((N_OUT & 15) | (7 << 4) | (15 << 8) | ((N_OUT >> 4) << 14));
}

}  // namespace tpk
