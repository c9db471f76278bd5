// Q8_0 projections of more tokens than the decode GEMV takes (batched decode, prefill) on the
// bf16 matrix cores.
//
// C[m, n] = sum_k A[m, k] w[n, k] with w = d[n, k/32] * q[n, k]: activations A [M, K] bf16, codes
// q [N, K] int8 and block scales d [N, K/32] fp16 (the code and scale planes of the packed shard).
// One 32-wide k-step of v_mfma_f32_16x16x32_bf16 is exactly one Q8_0 block, so the codes enter the
// matrix core unscaled (every int8 is exact in bf16) and each block's 16 x 16 product is scaled by
// its column's block scale and added in fp32: acc += d[n][b] * (A[:, b] . q[n, b]). That is the
// product with the dequantised weights up to the order of fp32 additions; the dequantised weights
// are never rounded. (TensorSharp "Multi-GPU & Multi-Node", section "Requirements & constraints",
// block-quantised weights split on block boundaries; the row-parallel slices start on a block.)
//
// Workgroup tile 64 x 64 x 64, four waves in a 2 x 2 grid, each 32 x 32 = 2 x 2 MFMA tiles (two
// for gate and up in the gated epilogue). A and the codes are staged through double-buffered LDS,
// the codes widened to bf16 on the way in; the next tile's global loads are issued before the
// current tile's MFMAs. Narrow shapes split K over grid.z: each split writes an fp32 partial tile
// and the split-K epilogue adds them in split order.
#include "k_gemm_common.h"
#include "tp_kernels.h"

namespace tpk {

constexpr int Q8_BM = 64, Q8_BN = 64, Q8_BK = 64;
constexpr int Q8_LD = Q8_BK + 8;  // bf16 per LDS row (16-byte pad against bank conflicts)

__device__ __forceinline__ uint32_t q8_pair_bf16(uint32_t w, int sh) {
  // two int8 codes (bytes sh/8 and sh/8 + 1 of w) -> two bf16 patterns (exact)
  const float a = (float)(int8_t)((w >> sh) & 0xffu);
  const float b = (float)(int8_t)((w >> (sh + 8)) & 0xffu);
  return (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xffff0000u);
}

template <int EPI, int ACTF>
__global__ __launch_bounds__(256) void k_gemm_q8(const uint16_t* __restrict__ A,
                                                 const int8_t* __restrict__ Bq,
                                                 const uint16_t* __restrict__ Bs,
                                                 const int8_t* __restrict__ B2q,
                                                 const uint16_t* __restrict__ B2s, int M, int N,
                                                 int K, int kt_per, void* __restrict__ C, int ldc,
                                                 float* __restrict__ part, int nsplit, Q8Ranks gr) {
  constexpr bool DUAL = (EPI == EPI_GATED);
  // Every rank in one launch: blockIdx.z = rank * nsplit + K range.
  int split = blockIdx.z;
  if (gr.n > 1) {
    const int r = blockIdx.z / nsplit;
    split = blockIdx.z - r * nsplit;
    A = (const uint16_t*)gr.a[r];
    Bq = (const int8_t*)gr.q[r];
    Bs = (const uint16_t*)gr.s[r];
    B2q = (const int8_t*)gr.q2[r];
    B2s = (const uint16_t*)gr.s2[r];
    C = gr.c[r];
    part = gr.part[r];
  }
  constexpr int NB = DUAL ? 2 : 1;
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][Q8_BM * Q8_LD];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][NB][Q8_BN * Q8_LD];
  __shared__ float sS[2][NB][Q8_BN][2];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * Q8_BM, n0 = blockIdx.x * Q8_BN;
  const int nkt = (K + Q8_BK - 1) / Q8_BK;
  const int kt0 = split * kt_per, kt1 = min(nkt, kt0 + kt_per);
  const int nblk = K / 32;

  // Staging assignment: A as two rows of 8 bf16 per thread; the codes as 16 bytes of one weight
  // row per thread; the scales (two blocks per row and tile) by the first 128 threads.
  const int lr = tid >> 3, lc = (tid & 7) * 8;
  const int br = tid >> 2, bc = (tid & 3) * 16;
  const int sr = tid >> 1, sb = tid & 1;
  uint4 ra[2], rq[NB];
  uint16_t rs[NB];
  auto gload = [&](int k0) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = lr + 32 * h, k = k0 + lc;
      ra[h] = (m0 + r < M && k < K) ? *(const uint4*)(A + (size_t)(m0 + r) * K + k)
                                    : make_uint4(0, 0, 0, 0);
    }
    const bool bin = n0 + br < N && k0 + bc < K;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int8_t* q = b == 0 ? Bq : B2q;
      rq[b] = bin ? *(const uint4*)(q + (size_t)(n0 + br) * K + k0 + bc) : make_uint4(0, 0, 0, 0);
    }
    if (tid < 2 * Q8_BN) {
      const int blk = k0 / 32 + sb;
      const bool sin = n0 + sr < N && blk < nblk;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const uint16_t* s = b == 0 ? Bs : B2s;
        rs[b] = sin ? s[(size_t)(n0 + sr) * nblk + blk] : (uint16_t)0;
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int h = 0; h < 2; ++h) *(uint4*)(&sA[buf][(lr + 32 * h) * Q8_LD + lc]) = ra[h];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const uint32_t w[4] = {rq[b].x, rq[b].y, rq[b].z, rq[b].w};
      uint4 lo, hi;
      lo.x = q8_pair_bf16(w[0], 0);  lo.y = q8_pair_bf16(w[0], 16);
      lo.z = q8_pair_bf16(w[1], 0);  lo.w = q8_pair_bf16(w[1], 16);
      hi.x = q8_pair_bf16(w[2], 0);  hi.y = q8_pair_bf16(w[2], 16);
      hi.z = q8_pair_bf16(w[3], 0);  hi.w = q8_pair_bf16(w[3], 16);
      *(uint4*)(&sB[buf][b][br * Q8_LD + bc]) = lo;
      *(uint4*)(&sB[buf][b][br * Q8_LD + bc + 8]) = hi;
      if (tid < 2 * Q8_BN) sS[buf][b][sr][sb] = f16_to_f32(rs[b]);
    }
  };

  floatx4 acc[NB][2][2];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[b][i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int fr = lane & 15, fk = (lane >> 4) * 8;
  if (kt0 < kt1) {
    gload(kt0 * Q8_BK);
    sstore(0);
  }
  __syncthreads();
  for (int kt = kt0; kt < kt1; ++kt) {
    const int cur = (kt - kt0) & 1;
    if (kt + 1 < kt1) gload((kt + 1) * Q8_BK);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int kk = kb * 32;
      bf16x8 af[2], bfr[NB][2];
      float sc[NB][2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *(const bf16x8*)(&sA[cur][(wm * 32 + i * 16 + fr) * Q8_LD + kk + fk]);
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int n = wn * 32 + j * 16 + fr;
          bfr[b][j] = *(const bf16x8*)(&sB[cur][b][n * Q8_LD + kk + fk]);
          sc[b][j] = sS[cur][b][n][kb];
        }
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const floatx4 p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                af[i], bfr[b][j], floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[b][i][j][r] = fmaf(sc[b][j], p[r], acc[b][i][j][r]);
          }
    }
    if (kt + 1 < kt1) sstore(cur ^ 1);
    __syncthreads();
  }

  // Lane holds C[row0 + r][col] for r = 0..3 (the MFMA output layout).
  const int ncols = DUAL ? 2 * N : N;
  float* pbase = part ? part + (size_t)split * M * ncols : nullptr;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wn * 32 + j * 16 + fr;
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + wm * 32 + i * 16 + (lane >> 4) * 4 + r;
        if (row >= M) continue;
        const float v = acc[0][i][j][r];
        if (pbase) {
          pbase[(size_t)row * ncols + col] = v;
          if constexpr (DUAL) pbase[(size_t)row * ncols + N + col] = acc[NB - 1][i][j][r];
          continue;
        }
        const size_t o = (size_t)row * ldc + col;
        if constexpr (EPI == EPI_GATED) {
          ((uint16_t*)C)[o] = f32_to_bf16(gated<ACTF>(v, acc[NB - 1][i][j][r]));
        } else if constexpr (EPI == EPI_F32) {
          ((float*)C)[o] = v;
        } else {
          ((uint16_t*)C)[o] = f32_to_bf16(v);  // EPI_ACT (bf16 activations) and EPI_BF16
        }
      }
    }
  }
}

// K splits: one per workgroup tile when the tiles nearly fill the chip, else enough splits for
// about 256 workgroups with at least four 64-wide k-tiles each.
static void q8_plan(int M, int N, int K, int* S, int* kt_per) {
  const int nkt = (K + Q8_BK - 1) / Q8_BK;
  const long tiles = (long)((N + Q8_BN - 1) / Q8_BN) * ((M + Q8_BM - 1) / Q8_BM);
  int s = 1;
  if (tiles < 192) {
    s = (int)((256 + tiles - 1) / tiles);
    const int smax = nkt / 4 > 1 ? nkt / 4 : 1;
    if (s > smax) s = smax;
  }
  const int per = (nkt + s - 1) / s;
  *kt_per = per;
  *S = (nkt + per - 1) / per;
}

int q8_gemm_splits(int M, int N, int K) {
  int S, per;
  q8_plan(M, N, K, &S, &per);
  return S;
}

size_t q8_gemm_workspace_bytes(int M, int N, int K, bool dual) {
  int S, per;
  q8_plan(M, N, K, &S, &per);
  return S > 1 ? (size_t)S * M * (dual ? 2 * (size_t)N : (size_t)N) * sizeof(float) : 0;
}

hipError_t launch_gemm_q8(int epi, int actf, int M, int N, int K, const void* A, const void* Bq,
                          const void* Bs, const void* B2q, const void* B2s, void* C, int ldc,
                          float* part, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  if (K % 32) return hipErrorInvalidValue;
  if (epi == EPI_GATED && (!B2q || !B2s)) return hipErrorInvalidValue;
  int S, per;
  q8_plan(M, N, K, &S, &per);
  if (S > 1 && !part) {  // no room for partial tiles: one K range per tile
    S = 1;
    per = (K + Q8_BK - 1) / Q8_BK;
  }
  float* p = S > 1 ? part : nullptr;
  const Q8Ranks nr{};
  const dim3 g((N + Q8_BN - 1) / Q8_BN, (M + Q8_BM - 1) / Q8_BM, S), b(256);
  const uint16_t* a = (const uint16_t*)A;
  const int8_t *q = (const int8_t*)Bq, *q2 = (const int8_t*)B2q;
  const uint16_t *s = (const uint16_t*)Bs, *s2 = (const uint16_t*)B2s;
  switch (epi) {
    case EPI_ACT:
      launch((k_gemm_q8<EPI_ACT, 0>), g, b, 0, st, a, q, s, q2, s2, M, N, K, per, C, ldc, p, S, nr);
      break;
    case EPI_F32:
      launch((k_gemm_q8<EPI_F32, 0>), g, b, 0, st, a, q, s, q2, s2, M, N, K, per, C, ldc, p, S, nr);
      break;
    case EPI_BF16:
      launch((k_gemm_q8<EPI_BF16, 0>), g, b, 0, st, a, q, s, q2, s2, M, N, K, per, C, ldc, p, S, nr);
      break;
    case EPI_GATED:
      if (actf == 0)
        launch((k_gemm_q8<EPI_GATED, 0>), g, b, 0, st, a, q, s, q2, s2, M, N, K, per, C, ldc, p, S, nr);
      else
        launch((k_gemm_q8<EPI_GATED, 1>), g, b, 0, st, a, q, s, q2, s2, M, N, K, per, C, ldc, p, S, nr);
      break;
    default:
      return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || S == 1) return e;
  return launch_splitk_epilogue(epi, actf, part, S, M, N, C, ldc, st);
}

hipError_t launch_gemm_q8_ranks(int epi, int actf, int M, int N, int K, const Q8Ranks& gr, int ldc,
                                hipStream_t st, bool parts_only, int* S_out) {
  if (gr.n < 1 || gr.n > kMaxRanks || K % 32 || !S_out) return hipErrorInvalidValue;
  const bool dual = epi == EPI_GATED;
  int S, per;
  q8_plan(M, N, K, &S, &per);
  *S_out = S;
  for (int r = 0; r < gr.n; ++r)
    if (!gr.a[r] || !gr.q[r] || !gr.s[r] || !gr.c[r] || (dual && (!gr.q2[r] || !gr.s2[r])) ||
        ((S > 1 || parts_only) && !gr.part[r]))
      return hipErrorInvalidValue;
  if (M == 0 || N == 0) return hipSuccess;
  if (parts_only && dual) return hipErrorInvalidValue;
  Q8Ranks g = gr;
  if (S == 1 && !parts_only)
    for (int r = 0; r < gr.n; ++r) g.part[r] = nullptr;  // one K range: the epilogue in the tiles
  const dim3 grid((N + Q8_BN - 1) / Q8_BN, (M + Q8_BM - 1) / Q8_BM, S * gr.n), b(256);
  const uint16_t* a = (const uint16_t*)g.a[0];
  const int8_t *q = (const int8_t*)g.q[0], *q2 = (const int8_t*)g.q2[0];
  const uint16_t *s = (const uint16_t*)g.s[0], *s2 = (const uint16_t*)g.s2[0];
  float* p = g.part[0];
  void* C = g.c[0];
  if (gr.n == 1) g.n = 0;  // a single rank takes the plain arguments
  switch (epi) {
    case EPI_ACT:
      launch((k_gemm_q8<EPI_ACT, 0>), grid, b, 0, st, a, q, s, q2, s2, M, N, K, per, C, ldc, p, S, g);
      break;
    case EPI_F32:
      launch((k_gemm_q8<EPI_F32, 0>), grid, b, 0, st, a, q, s, q2, s2, M, N, K, per, C, ldc, p, S, g);
      break;
    case EPI_BF16:
      launch((k_gemm_q8<EPI_BF16, 0>), grid, b, 0, st, a, q, s, q2, s2, M, N, K, per, C, ldc, p, S, g);
      break;
    case EPI_GATED:
      if (actf == 0)
        launch((k_gemm_q8<EPI_GATED, 0>), grid, b, 0, st, a, q, s, q2, s2, M, N, K, per, C, ldc, p, S, g);
      else
        launch((k_gemm_q8<EPI_GATED, 1>), grid, b, 0, st, a, q, s, q2, s2, M, N, K, per, C, ldc, p, S, g);
      break;
    default:
      return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || parts_only || S == 1) return e;
  GemmRanks ge{};
  ge.n = gr.n;
  for (int r = 0; r < gr.n; ++r) {
    ge.a[r] = gr.part[r];
    ge.c[r] = gr.c[r];
  }
  return launch_splitk_epilogue(epi, actf, gr.part[0], S, M, N, gr.c[0], ldc, st,
                                gr.n > 1 ? &ge : nullptr);
}

}  // namespace tpk
