// K4: bf16 projections for many tokens (batched decode, prefill) on the CDNA4 matrix cores.
//
// C[m, n] = sum_k A[m, k] B[n, k]: A = activations [M, K], B = weights [N, K], both K-contiguous,
// so both MFMA operands are plain 16-byte loads of 8 consecutive k. Workgroup tile 64 x 64 x 64,
// four waves in a 2 x 2 grid, each wave 32 x 32 = 2 x 2 tiles of v_mfma_f32_16x16x32_bf16.
// A and B tiles are staged through LDS (double-buffered, rows padded by 16 bytes against bank
// conflicts); the next tile's global loads are issued before the current tile's MFMAs.
//
// MFMA 16x16x32 operand layout (gfx950): lane l supplies row (l % 16) of A and column (l % 16) of
// B, each as 8 consecutive k starting at 8 * (l / 16); the 16 x 16 fp32 result lands with lane l
// holding rows 4 * (l / 16) + r, r = 0..3, of column l % 16. A and B use the same k assignment, so
// the contraction over k does not depend on how the hardware orders k within the instruction.
//
// Epilogues as in the GEMV: activation-dtype store (QKV), fp32 / bf16 partial store (row-parallel
// o_proj and down), and the fused gate/up pair: B2 holds the up rows, act(g) * u is stored.
#include "tp_common.h"
#include "tp_kernels.h"

namespace tpk {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4;

constexpr int GB_M = 64, GB_N = 64, GB_K = 64;
constexpr int G_LDS_LD = GB_K + 8;  // bf16 elements per LDS row

template <int EPI, int ACTF>
__global__ __launch_bounds__(256) void k_gemm_bf16(const uint16_t* __restrict__ A,
                                                   const uint16_t* __restrict__ B,
                                                   const uint16_t* __restrict__ B2, int M, int N,
                                                   int K, void* __restrict__ C, int ldc) {
  constexpr bool DUAL = (EPI == EPI_GATED);
  constexpr int NB = DUAL ? 2 : 1;
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][GB_M * G_LDS_LD];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][NB][GB_N * G_LDS_LD];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * GB_M, n0 = blockIdx.x * GB_N;

  // Global -> register staging: each thread moves 2 chunks of 8 bf16 per operand tile.
  const int lr = tid >> 3, lc = (tid & 7) * 8;
  uint4 ra[2], rb[NB][2];
  auto gload = [&](int k0) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = lr + 32 * h, k = k0 + lc;
      const bool kin = k < K;
      ra[h] = (m0 + r < M && kin) ? *(const uint4*)(A + (size_t)(m0 + r) * K + k)
                                  : make_uint4(0, 0, 0, 0);
      const bool nin = (n0 + r < N) && kin;
      rb[0][h] = nin ? *(const uint4*)(B + (size_t)(n0 + r) * K + k) : make_uint4(0, 0, 0, 0);
      if constexpr (DUAL)
        rb[NB - 1][h] = nin ? *(const uint4*)(B2 + (size_t)(n0 + r) * K + k)
                            : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = lr + 32 * h;
      *(uint4*)(&sA[buf][r * G_LDS_LD + lc]) = ra[h];
#pragma unroll
      for (int b = 0; b < NB; ++b) *(uint4*)(&sB[buf][b][r * G_LDS_LD + lc]) = rb[b][h];
    }
  };

  floatx4 acc[NB][2][2];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[b][i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int nk = (K + GB_K - 1) / GB_K;
  gload(0);
  sstore(0);
  __syncthreads();
  const int fr = lane & 15, fk = (lane >> 4) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * GB_K);
#pragma unroll
    for (int kk = 0; kk < GB_K; kk += 32) {
      bf16x8 af[2], bfr[NB][2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *(const bf16x8*)(&sA[cur][(wm * 32 + i * 16 + fr) * G_LDS_LD + kk + fk]);
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          bfr[b][j] = *(const bf16x8*)(&sB[cur][b][(wn * 32 + j * 16 + fr) * G_LDS_LD + kk + fk]);
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[b][i][j] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[b][j], acc[b][i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) {
      sstore(cur ^ 1);
    }
    __syncthreads();
  }

  // Epilogue: lane holds C[row0 + r][col] for r = 0..3.
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wn * 32 + j * 16 + (lane & 15);
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + wm * 32 + i * 16 + (lane >> 4) * 4 + r;
        if (row >= M) continue;
        const size_t o = (size_t)row * ldc + col;
        const float v = acc[0][i][j][r];
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

// Large-tile variant for prefill-sized M (>= 256 rows): workgroup tile BM x 128 x 64 (BM = 256 or
// 128), four waves in a 2 x 2 grid, each holding a (BM/2) x 64 accumulator tile (up to 32 MFMA
// tiles), so every 16-byte LDS fragment feeds several MFMAs. A and B stage through two LDS buffers
// (rows padded by 16 bytes: conflict-free ds_read_b128); the next K-tile's global loads are in
// flight during the current tile's MFMAs. Workgroups are ordered so that consecutive tiles of one
// output row band run on the same XCD (blocks are dealt to the 8 XCDs round-robin), keeping the
// shared A band in that XCD's L2. Dual-B (gate/up): the 128 B columns are 64 gate + 64 up rows of
// the same 64 output columns; each wave holds 32 gate and the matching 32 up columns.
constexpr int BG_N = 128, BG_K = 64, BG_LD = BG_K + 8;

template <int EPI, int ACTF, int BM>
__global__ __launch_bounds__(256) void k_gemm_big(const uint16_t* __restrict__ A,
                                                  const uint16_t* __restrict__ B,
                                                  const uint16_t* __restrict__ B2, int M, int N,
                                                  int K, void* __restrict__ C, int ldc,
                                                  int tiles_m, int tiles_n) {
  constexpr bool DUAL = (EPI == EPI_GATED);
  constexpr int WM = BM / 2;        // rows per wave
  constexpr int TM = WM / 16;       // 16-row MFMA tiles per wave
  constexpr int TN = 4;             // 16-col MFMA tiles per wave (64 B columns)
  constexpr int ACH = BM * BG_K / 8 / 256;   // 16-byte chunks of A per thread per K-tile
  constexpr int BCH = BG_N * BG_K / 8 / 256; // ... of B
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  uint16_t* sA = smem;                          // [2][BM * BG_LD]
  uint16_t* sB = smem + 2 * BM * BG_LD;         // [2][BG_N * BG_LD]

  // XCD-aware tile order: block b runs on XCD b % 8; give each XCD a contiguous run of tiles.
  // The first 8 * floor(n / 8) blocks are remapped (a bijection on that range); the rest keep
  // their index.
  const int nblk = gridDim.x;
  const int b = blockIdx.x;
  const int full = nblk / 8 * 8;
  const int lt = (b < full) ? (b % 8) * (full / 8) + b / 8 : b;
  const int tm = lt / tiles_n, tn = lt % tiles_n;
  const int m0 = tm * BM;
  // Columns of B this block stages: plain: n0 .. n0+127; dual: 64 output columns n0 .. n0+63 of
  // both the gate (B) and up (B2) matrices.
  const int n0 = DUAL ? tn * 64 : tn * BG_N;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  uint4 ra[ACH], rb[BCH];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const int c = tid + i * 256, r = c >> 3, k = k0 + (c & 7) * 8;
      ra[i] = (m0 + r < M && k < K) ? *(const uint4*)(A + (size_t)(m0 + r) * K + k)
                                    : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < BCH; ++i) {
      const int c = tid + i * 256, r = c >> 3, k = k0 + (c & 7) * 8;
      const uint16_t* src;
      int col;
      if constexpr (DUAL) {
        col = n0 + (r & 63);
        src = (r < 64) ? B : B2;
      } else {
        col = n0 + r;
        src = B;
      }
      rb[i] = (col < N && k < K) ? *(const uint4*)(src + (size_t)col * K + k)
                                 : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const int c = tid + i * 256;
      *(uint4*)(sA + buf * BM * BG_LD + (c >> 3) * BG_LD + (c & 7) * 8) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < BCH; ++i) {
      const int c = tid + i * 256;
      *(uint4*)(sB + buf * BG_N * BG_LD + (c >> 3) * BG_LD + (c & 7) * 8) = rb[i];
    }
  };

  floatx4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  // B rows (in the staged 128-row tile) read by this wave's column tile j.
  auto brow = [&](int j) -> int {
    if constexpr (DUAL) return (j < 2 ? 0 : 64) + wn * 32 + (j & 1) * 16;  // gate j=0,1; up j=2,3
    else return wn * 64 + j * 16;
  };
  const int fr = lane & 15, fk = (lane >> 4) * 8;
  const int nk = (K + BG_K - 1) / BG_K;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BG_K);
    const uint16_t* a_s = sA + cur * BM * BG_LD;
    const uint16_t* b_s = sB + cur * BG_N * BG_LD;
#pragma unroll
    for (int kk = 0; kk < BG_K; kk += 32) {
      bf16x8 bf[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bf[j] = *(const bf16x8*)(b_s + (brow(j) + fr) * BG_LD + kk + fk);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const bf16x8 af = *(const bf16x8*)(a_s + (wm * WM + i * 16 + fr) * BG_LD + kk + fk);
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[j], acc[i][j], 0, 0, 0);
      }
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  // Epilogue: lane holds C[row][col] for rows 4 (lane / 16) + r of each 16-row tile.
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = m0 + wm * WM + i * 16 + (lane >> 4) * 4 + r;
      if (row >= M) continue;
      if constexpr (DUAL) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = n0 + wn * 32 + j * 16 + fr;
          if (col < N)
            ((uint16_t*)C)[(size_t)row * ldc + col] =
                f32_to_bf16(gated<ACTF>(acc[i][j][r], acc[i][j + 2][r]));
        }
      } else {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int col = n0 + wn * 64 + j * 16 + fr;
          if (col >= N) continue;
          const size_t o = (size_t)row * ldc + col;
          if constexpr (EPI == EPI_F32) ((float*)C)[o] = acc[i][j][r];
          else ((uint16_t*)C)[o] = f32_to_bf16(acc[i][j][r]);
        }
      }
    }
  }
}

template <int BM>
static hipError_t big_bm(int epi, int actf, int M, int N, int K, const uint16_t* a,
                         const uint16_t* b, const uint16_t* b2, void* C, int ldc, hipStream_t st) {
  const int tiles_m = (M + BM - 1) / BM;
  const int tiles_n = (epi == EPI_GATED) ? (N + 63) / 64 : (N + BG_N - 1) / BG_N;
  dim3 g(tiles_m * tiles_n), blk(256);
  const size_t lds = (size_t)2 * (BM + BG_N) * BG_LD * sizeof(uint16_t);
#define TPK_BIG(E, AF)                                                                          \
  do {                                                                                          \
    static bool attr_set = false;                                                               \
    if (!attr_set) {                                                                            \
      hipFuncSetAttribute((const void*)k_gemm_big<E, AF, BM>,                                   \
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);                \
      attr_set = true;                                                                          \
    }                                                                                           \
    hipLaunchKernelGGL((k_gemm_big<E, AF, BM>), g, blk, lds, st, a, b, b2, M, N, K, C, ldc,    \
                       tiles_m, tiles_n);                                                       \
  } while (0)
  switch (epi) {
    case EPI_ACT: TPK_BIG(EPI_ACT, 0); break;
    case EPI_F32: TPK_BIG(EPI_F32, 0); break;
    case EPI_BF16: TPK_BIG(EPI_BF16, 0); break;
    case EPI_GATED:
      if (actf == 0) TPK_BIG(EPI_GATED, 0);
      else TPK_BIG(EPI_GATED, 1);
      break;
    default:
      return hipErrorInvalidValue;
  }
#undef TPK_BIG
  return hipGetLastError();
}

// Skinny variant for batched decode (M <= 64 tokens): the weight stream dominates, so a
// workgroup owns only 16 output columns (16 weight rows) for all M tokens and its four waves
// split K four ways; each wave keeps MT (<= 4) 16 x 16 tiles in registers, loads both operands
// straight from global memory (the small activation matrix is served by L2), and the four
// partial tiles are added in LDS in wave order before the epilogue.
constexpr int SK_U = 2;  // k-steps of 32 per register set; two sets alternate

template <int EPI, int ACTF, int MT>
__global__ __launch_bounds__(256) void k_gemm_skinny(const uint16_t* __restrict__ A,
                                                     const uint16_t* __restrict__ B,
                                                     const uint16_t* __restrict__ B2, int M,
                                                     int N, int K, void* __restrict__ C,
                                                     int ldc) {
  constexpr bool DUAL = (EPI == EPI_GATED);
  constexpr int NB = DUAL ? 2 : 1;
  __shared__ floatx4 s_acc[4][NB][MT][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * 16;
  const int fr = lane & 15, fk = (lane >> 4) * 8;
  const int ksteps = (K + 31) / 32;
  const int per = (ksteps + 3) / 4;
  const int ks0 = wave * per, ks1 = min(ksteps, ks0 + per);
  const bool nin = n0 + fr < N;
  const uint16_t* brow = B + (size_t)(nin ? n0 + fr : 0) * K;
  const uint16_t* brow2 = DUAL ? B2 + (size_t)(nin ? n0 + fr : 0) * K : nullptr;

  floatx4 acc[NB][MT];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int i = 0; i < MT; ++i) acc[b][i] = floatx4{0.f, 0.f, 0.f, 0.f};

  auto load = [&](int ks, bf16x8 (&af)[SK_U][MT], bf16x8 (&bfr)[SK_U][NB]) {
#pragma unroll
    for (int u = 0; u < SK_U; ++u) {
      const int k = (ks + u) * 32 + fk;
      const bool kin = (ks + u < ks1) && (k < K);
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const int row = i * 16 + fr;
        uint4 v = (kin && row < M) ? *(const uint4*)(A + (size_t)row * K + k) : make_uint4(0, 0, 0, 0);
        af[u][i] = __builtin_bit_cast(bf16x8, v);
      }
      uint4 w = (kin && nin) ? ld_stream16(brow + k) : make_uint4(0, 0, 0, 0);
      bfr[u][0] = __builtin_bit_cast(bf16x8, w);
      if constexpr (DUAL) {
        uint4 w2 = (kin && nin) ? ld_stream16(brow2 + k) : make_uint4(0, 0, 0, 0);
        bfr[u][NB - 1] = __builtin_bit_cast(bf16x8, w2);
      }
    }
  };
  auto mma = [&](const bf16x8 (&af)[SK_U][MT], const bf16x8 (&bfr)[SK_U][NB]) {
#pragma unroll
    for (int u = 0; u < SK_U; ++u)
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < MT; ++i)
          acc[b][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[u][i], bfr[u][b], acc[b][i], 0, 0, 0);
  };
  bf16x8 a0[SK_U][MT], b0[SK_U][NB], a1[SK_U][MT], b1[SK_U][NB];
  if (ks0 < ks1) load(ks0, a0, b0);
  for (int ks = ks0; ks < ks1; ks += 2 * SK_U) {
    if (ks + SK_U < ks1) load(ks + SK_U, a1, b1);
    mma(a0, b0);
    if (ks + 2 * SK_U < ks1) load(ks + 2 * SK_U, a0, b0);
    if (ks + SK_U < ks1) mma(a1, b1);
  }
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int i = 0; i < MT; ++i) s_acc[wave][b][i][lane] = acc[b][i];
  __syncthreads();
  if (wave != 0) return;
  const int col = n0 + (lane & 15);
  if (col >= N) return;
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    floatx4 tot[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      tot[b] = s_acc[0][b][i][lane];
#pragma unroll
      for (int w = 1; w < 4; ++w) tot[b] += s_acc[w][b][i][lane];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = i * 16 + (lane >> 4) * 4 + r;
      if (row >= M) continue;
      const size_t o = (size_t)row * ldc + col;
      if constexpr (EPI == EPI_GATED) {
        ((uint16_t*)C)[o] = f32_to_bf16(gated<ACTF>(tot[0][r], tot[NB - 1][r]));
      } else if constexpr (EPI == EPI_F32) {
        ((float*)C)[o] = tot[0][r];
      } else {
        ((uint16_t*)C)[o] = f32_to_bf16(tot[0][r]);
      }
    }
  }
}

template <int MT>
static hipError_t skinny_mt(int epi, int actf, int M, int N, int K, const uint16_t* a,
                            const uint16_t* b, const uint16_t* b2, void* C, int ldc,
                            hipStream_t st) {
  dim3 g((N + 15) / 16), blk(256);
  switch (epi) {
    case EPI_ACT:
      hipLaunchKernelGGL((k_gemm_skinny<EPI_ACT, 0, MT>), g, blk, 0, st, a, b, b2, M, N, K, C, ldc);
      break;
    case EPI_F32:
      hipLaunchKernelGGL((k_gemm_skinny<EPI_F32, 0, MT>), g, blk, 0, st, a, b, b2, M, N, K, C, ldc);
      break;
    case EPI_BF16:
      hipLaunchKernelGGL((k_gemm_skinny<EPI_BF16, 0, MT>), g, blk, 0, st, a, b, b2, M, N, K, C, ldc);
      break;
    case EPI_GATED:
      if (actf == 0)
        hipLaunchKernelGGL((k_gemm_skinny<EPI_GATED, 0, MT>), g, blk, 0, st, a, b, b2, M, N, K, C, ldc);
      else
        hipLaunchKernelGGL((k_gemm_skinny<EPI_GATED, 1, MT>), g, blk, 0, st, a, b, b2, M, N, K, C, ldc);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_bf16(int epi, int actf, int M, int N, int K, const void* A, const void* B,
                            const void* B2, void* C, int ldc, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  const uint16_t *a = (const uint16_t*)A, *bb = (const uint16_t*)B, *b2 = (const uint16_t*)B2;
  if (M <= 64) {
    switch ((M + 15) / 16) {
      case 1: return skinny_mt<1>(epi, actf, M, N, K, a, bb, b2, C, ldc, st);
      case 2: return skinny_mt<2>(epi, actf, M, N, K, a, bb, b2, C, ldc, st);
      case 3: return skinny_mt<3>(epi, actf, M, N, K, a, bb, b2, C, ldc, st);
      default: return skinny_mt<4>(epi, actf, M, N, K, a, bb, b2, C, ldc, st);
    }
  }
  if (M >= 256) {
    // Enough row bands for 256-row tiles to fill the chip, else 128-row tiles.
    const long t256 = (long)((M + 255) / 256) * ((epi == EPI_GATED) ? (N + 63) / 64 : (N + 127) / 128);
    if (t256 >= 256) return big_bm<256>(epi, actf, M, N, K, a, bb, b2, C, ldc, st);
    return big_bm<128>(epi, actf, M, N, K, a, bb, b2, C, ldc, st);
  }
  dim3 g((N + GB_N - 1) / GB_N, (M + GB_M - 1) / GB_M), b(256);
  switch (epi) {
    case EPI_ACT:
      hipLaunchKernelGGL((k_gemm_bf16<EPI_ACT, 0>), g, b, 0, st, a, bb, b2, M, N, K, C, ldc);
      break;
    case EPI_F32:
      hipLaunchKernelGGL((k_gemm_bf16<EPI_F32, 0>), g, b, 0, st, a, bb, b2, M, N, K, C, ldc);
      break;
    case EPI_BF16:
      hipLaunchKernelGGL((k_gemm_bf16<EPI_BF16, 0>), g, b, 0, st, a, bb, b2, M, N, K, C, ldc);
      break;
    case EPI_GATED:
      if (actf == 0)
        hipLaunchKernelGGL((k_gemm_bf16<EPI_GATED, 0>), g, b, 0, st, a, bb, b2, M, N, K, C, ldc);
      else
        hipLaunchKernelGGL((k_gemm_bf16<EPI_GATED, 1>), g, b, 0, st, a, bb, b2, M, N, K, C, ldc);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace tpk
