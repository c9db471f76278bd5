// K4b: bf16 projections of up to 64 tokens (batched decode) without a K split.
//
// With 64 tokens a projection still streams its weights from HBM (64 FLOP per weight byte), and
// the output is small, so the work is split over output columns only: a workgroup owns a band of
// 16 output columns (gated: the 16 gate columns and the matching 16 up columns) for every token
// and the whole K range. The epilogue (activation-dtype store, fp32 / bf16 row-parallel partial,
// or act(g) * u) therefore runs in the same kernel, and no fp32 partial tiles go through memory.
//
// Stages of BK columns of K: the tokens' activation rows (16 MT) and the band's weight rows go
// straight from global memory into an RS-slot LDS ring by direct-to-LDS loads, RS - 1 stages in
// flight. One wave-load moves 1 KB: 1024 / (2 BK) whole rows of the stage, so each weight row is
// read as one 2 BK-byte segment per stage. 16-byte chunks are XOR-swizzled by row % 16 so that
// the MFMA operand reads (16 rows, one chunk each) spread over the banks.
//
// Wave w multiplies token tile w (tokens 16w .. 16w + 15) by the band, k-step after k-step, so
// each output element is a single fp32 accumulation in k order and the waves never exchange
// partial sums. MFMA operand layout as in k_gemm.hip (16x16x32 bf16).
#include "k_gemm_common.h"
#include "tp_kernels.h"

namespace tpk {

template <int MT, int EPI, int ACTF, int BK, int RS, int NRK, bool XR>
__global__ __launch_bounds__(256) void k_gemm_band(const uint16_t* __restrict__ A,
                                                   const uint16_t* __restrict__ B,
                                                   const uint16_t* __restrict__ B2, int M, int N,
                                                   int K, void* __restrict__ C, int ldc,
                                                   GemmRanks gr) {
  constexpr bool DUAL = (EPI == EPI_GATED);
  constexpr int NB = DUAL ? 2 : 1;
  constexpr int AR = MT * 16, BR = 16 * NB;  // staged activation rows, weight rows per group
  constexpr int BRA = NRK * BR;              // weight rows of the NRK groups sharing A
  constexpr int CPR = BK / 8;                // 16-byte chunks per staged row
  constexpr int RPL = 64 / CPR;              // rows per wave-load
  constexpr int SWZ = (CPR < 16 ? CPR : 16) - 1;
  constexpr int STAGE = (AR + BRA) * BK;     // bf16 elements per ring slot
  constexpr int A_WL = AR / RPL, B_WL = BRA / RPL;
  constexpr int A_PW = (A_WL + 3) / 4, B_PW = (B_WL + 3) / 4;  // per wave; surplus ones repeat
  constexpr int LPW = A_PW + B_PW;
  static_assert(BK % 32 == 0 && 64 % CPR == 0 && AR % RPL == 0 && BR % RPL == 0, "stage shape");
  static_assert((RS - 2) * LPW <= 63, "vmcnt range");
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];

  // The workgroup's NRK groups of 16 columns share its activation stages, group i in staged rows
  // [i * BR, (i + 1) * BR). XR: the groups are NRK ranks' same 16 columns (a column-parallel
  // projection of one input, every rank in one launch; blockIdx.z picks the ranks r0 ..
  // r0 + NRK - 1). Otherwise: NRK adjacent 16-column bands of one rank (blockIdx.z = rank when
  // every rank is in the launch), so each activation stage serves 16 NRK columns.
  const int r0 = gr.n > 1 ? (int)blockIdx.z * (XR ? NRK : 1) : 0;
  if (gr.n > 1) A = (const uint16_t*)gr.a[r0];
  auto wsrc = [&](int i, bool up) -> const uint16_t* {
    const int r = XR ? r0 + i : r0;
    if (gr.n > 1) return (const uint16_t*)(up ? gr.b2[r] : gr.b[r]);
    return up ? B2 : B;
  };
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = blockIdx.x * 16 * (XR ? 1 : NRK);
  auto cbase = [&](int i) { return XR ? n0 : n0 + 16 * i; };
  const int nst = K / BK;  // K % BK == 0 (checked by the launcher)

  // Lane l of a wave-load stores its 16 bytes at chunk l % CPR of row l / CPR of the wave-load's
  // rows, so it loads the row's global chunk (l % CPR) ^ (row % 16). Rows past M or N load a
  // clamped (valid) row whose results are never stored.
  const int lrow = lane / CPR, lpc = lane % CPR;
  auto issue = [&](int slot, int stg) {
    uint16_t* st = smem + slot * STAGE;
    const size_t kb = (size_t)min(stg, nst - 1) * BK;
#pragma unroll
    for (int i = 0; i < A_PW; ++i) {
      const int g = (wave * A_PW + i) % A_WL;  // a repeated group writes identical bytes
      const int row = g * RPL + lrow;
      const uint16_t* src = A + (size_t)min(row, M - 1) * K + kb + ((lpc ^ (row & SWZ)) << 3);
      __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)(st + g * RPL * BK), 16, 0,
                                       0);
    }
#pragma unroll
    for (int i = 0; i < B_PW; ++i) {
      const int g = (wave * B_PW + i) % B_WL;
      const int row = g * RPL + lrow;  // rank row / BR: gate rows, then (gated) the up rows
      const int lr = row % BR;
      const uint16_t* base = wsrc(row / BR, DUAL && lr >= 16);
      const int col = min(cbase(row / BR) + (lr & 15), N - 1);
      const uint16_t* src = base + (size_t)col * K + kb + ((lpc ^ (row & SWZ)) << 3);
      __builtin_amdgcn_global_load_lds((glb_void_t*)src,
                                       (lds_void_t*)(st + (AR + g * RPL) * BK), 16, 0,
                                       kStreamAux);
    }
  };

  floatx4 acc[NRK][NB];
#pragma unroll
  for (int i = 0; i < NRK; ++i)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[i][b] = floatx4{0.f, 0.f, 0.f, 0.f};
  const int fr = lane & 15, fq = lane >> 4;
  const bool mma_wave = MT == 4 || wave < MT;  // wave-uniform

#pragma unroll
  for (int s = 0; s < RS - 1; ++s) issue(s, s);
  for (int stg = 0; stg < nst; ++stg) {
    // Stage stg has landed for this wave once only the RS - 2 newer stages remain in flight;
    // after the barrier for every wave, and every wave is done reading slot (stg - 1) % RS.
    wait_vmcnt<(RS - 2) * LPW>();
    __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    issue((stg + RS - 1) % RS, stg + RS - 1);
    if (mma_wave) {
      const uint16_t* a_s = smem + (stg % RS) * STAGE + (wave * 16 + fr) * BK;
      const uint16_t* b_s = smem + (stg % RS) * STAGE + (AR + fr) * BK;
#pragma unroll
      for (int kk = 0; kk < BK / 32; ++kk) {
        const int sw = ((kk * 4 + fq) ^ (fr & SWZ)) << 3;
        const bf16x8 af = *(const bf16x8*)(a_s + sw);
#pragma unroll
        for (int i = 0; i < NRK; ++i)
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            const bf16x8 bf = *(const bf16x8*)(b_s + (i * BR + b * 16) * BK + sw);
            acc[i][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf, acc[i][b], 0, 0, 0);
          }
      }
    }
  }
  // The clamped loads past the last stage may still be in flight.
  wait_vmcnt<0>();
  if (!mma_wave) return;
#pragma unroll
  for (int i = 0; i < NRK; ++i) {
    void* Ci = gr.n > 1 ? gr.c[XR ? r0 + i : r0] : C;
    const int col = cbase(i) + fr;
    if (col >= N) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = wave * 16 + fq * 4 + r;
      if (row >= M) continue;
      const size_t o = (size_t)row * ldc + col;
      if constexpr (EPI == EPI_GATED) {
        ((uint16_t*)Ci)[o] = f32_to_bf16(gated<ACTF>(acc[i][0][r], acc[i][NB - 1][r]));
      } else if constexpr (EPI == EPI_F32) {
        ((float*)Ci)[o] = acc[i][0][r];
      } else {
        ((uint16_t*)Ci)[o] = f32_to_bf16(acc[i][0][r]);
      }
    }
  }
}

namespace {

// Stage depth and ring size: 256-byte weight row segments and a ring of at most five slots (four
// stages in flight) that fits the 160 KB of LDS and the wait counter's range. Deeper rings, or
// separate rings that keep more weight stages than activation stages in flight, measured slower
// inside the batched step (64 sequences, 4 ranks: 201.1 us with five slots, 202.2 with six,
// 203.3 with up to eight, 205.9 with four, 216.6 with 23 weight stages in flight); so did
// 512-byte segments.
constexpr int BD_BK = 128;
template <int MT, bool DUAL, int BK, int NRK>
constexpr int band_slots() {
  constexpr int stage = (MT * 16 + NRK * 16 * (DUAL ? 2 : 1)) * BK * 2;
  constexpr int rpl = 64 / (BK / 8);
  constexpr int lpw = (MT * 16 / rpl + 3) / 4 + (NRK * 16 * (DUAL ? 2 : 1) / rpl + 3) / 4;
  constexpr int s = (160 * 1024) / stage;
  constexpr int smax = 63 / lpw + 2;
  constexpr int r = s < smax ? s : smax;
  return r > 5 ? 5 : r;
}

template <int MT, int EPI, int ACTF, int NRK, bool XR>
hipError_t band_launch_n(int M, int N, int K, const uint16_t* a, const uint16_t* b,
                         const uint16_t* b2, void* C, int ldc, hipStream_t st,
                         const GemmRanks& gr) {
  constexpr bool DUAL = EPI == EPI_GATED;
  // Groups of ranks sharing A stage more weight rows per slot: 128-byte row segments keep the
  // ring deep enough there.
  constexpr int BK = NRK > 1 ? 64 : BD_BK;
  constexpr int RS = band_slots<MT, DUAL, BK, NRK>();
  constexpr size_t lds = (size_t)RS * (MT * 16 + NRK * 16 * (DUAL ? 2 : 1)) * BK * 2;
  if (K % BK != 0) return hipErrorInvalidValue;
  auto kern = k_gemm_band<MT, EPI, ACTF, BK, RS, NRK, XR>;
  hipError_t e = allow_lds((const void*)kern, (int)lds);
  if (e != hipSuccess) return e;
  const int nz = gr.n > 1 ? (XR ? gr.n / NRK : gr.n) : 1;
  const int cols = 16 * (XR ? 1 : NRK);
  launch(kern, dim3((N + cols - 1) / cols, 1, nz), dim3(256), lds, st, a, b, b2, M, N, K, C, ldc,
         gr);
  return hipGetLastError();
}

// share > 0: groups of `share` ranks of one input; share < 0: -share adjacent bands of one rank.
template <int MT, int EPI, int ACTF>
hipError_t band_launch(int M, int N, int K, const uint16_t* a, const uint16_t* b,
                       const uint16_t* b2, void* C, int ldc, hipStream_t st, const GemmRanks& gr,
                       int share) {
  if (share == 4) return band_launch_n<MT, EPI, ACTF, 4, true>(M, N, K, a, b, b2, C, ldc, st, gr);
  if (share == 2) return band_launch_n<MT, EPI, ACTF, 2, true>(M, N, K, a, b, b2, C, ldc, st, gr);
  if (share == -4) return band_launch_n<MT, EPI, ACTF, 4, false>(M, N, K, a, b, b2, C, ldc, st, gr);
  if (share == -2) return band_launch_n<MT, EPI, ACTF, 2, false>(M, N, K, a, b, b2, C, ldc, st, gr);
  return band_launch_n<MT, EPI, ACTF, 1, true>(M, N, K, a, b, b2, C, ldc, st, gr);
}

template <int MT>
hipError_t band_mt(int epi, int actf, int M, int N, int K, const uint16_t* a, const uint16_t* b,
                   const uint16_t* b2, void* C, int ldc, hipStream_t st, const GemmRanks& gr,
                   int share) {
  switch (epi) {
    case EPI_ACT: return band_launch<MT, EPI_ACT, 0>(M, N, K, a, b, b2, C, ldc, st, gr, share);
    case EPI_F32: return band_launch<MT, EPI_F32, 0>(M, N, K, a, b, b2, C, ldc, st, gr, share);
    case EPI_BF16: return band_launch<MT, EPI_BF16, 0>(M, N, K, a, b, b2, C, ldc, st, gr, share);
    case EPI_GATED:
      return actf == 0 ? band_launch<MT, EPI_GATED, 0>(M, N, K, a, b, b2, C, ldc, st, gr, share)
                       : band_launch<MT, EPI_GATED, 1>(M, N, K, a, b, b2, C, ldc, st, gr, share);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool gemm_band_supported(int epi, int M, int N, int K) {
  return M >= 1 && M <= 64 && K % BD_BK == 0 && (N + 15) / 16 >= 192 &&
         (epi == EPI_ACT || epi == EPI_F32 || epi == EPI_BF16 || epi == EPI_GATED);
}

hipError_t launch_gemm_band(int epi, int actf, int M, int N, int K, const void* A, const void* B,
                            const void* B2, void* C, int ldc, hipStream_t st,
                            const GemmRanks* gr) {
  if (M == 0 || N == 0) return hipSuccess;
  if (!gemm_band_supported(epi, M, N, K)) return hipErrorInvalidValue;
  const GemmRanks one{};
  if (gr) {
    if (gr->n < 1 || gr->n > kMaxRanks) return hipErrorInvalidValue;
    for (int r = 0; r < gr->n; ++r)
      if (!gr->a[r] || !gr->b[r] || !gr->c[r] || (epi == EPI_GATED && !gr->b2[r]))
        return hipErrorInvalidValue;
    A = gr->a[0];
    B = gr->b[0];
    B2 = gr->b2[0];
    C = gr->c[0];
  }
  const GemmRanks& g = gr ? *gr : one;
  // Every rank in one launch: a gated projection of one input shares each workgroup's
  // activation stages among groups of four (or two) ranks; other projections (each rank its own
  // input) give a workgroup four (or two) adjacent bands of one rank while the launch still has
  // 256 workgroups, so each activation stage serves more weight rows.
  int share = 1;
  if (gr && gr->n > 1 && K % 64 == 0) {
    const int n = gr->n;
    bool same_a = true;
    for (int r = 1; r < n; ++r)
      if (gr->a[r] != gr->a[0]) same_a = false;
    if (epi == EPI_GATED && same_a) {
      share = n % 4 == 0 ? 4 : (n % 2 == 0 ? 2 : 1);
    } else if (epi != EPI_GATED) {
      const long bands = (N + 15) / 16;
      share = (bands / 4) * n >= 256 ? -4 : ((bands / 2) * n >= 256 ? -2 : 1);
    }
  }
  const uint16_t *a = (const uint16_t*)A, *b = (const uint16_t*)B, *b2 = (const uint16_t*)B2;
  switch ((M + 15) / 16) {
    case 1: return band_mt<1>(epi, actf, M, N, K, a, b, b2, C, ldc, st, g, share);
    case 2: return band_mt<2>(epi, actf, M, N, K, a, b, b2, C, ldc, st, g, share);
    case 3: return band_mt<3>(epi, actf, M, N, K, a, b, b2, C, ldc, st, g, share);
    default: return band_mt<4>(epi, actf, M, N, K, a, b, b2, C, ldc, st, g, share);
  }
}

}  // namespace tpk
