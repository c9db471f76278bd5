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
#include "k_gemm_common.h"
#include "tp_kernels.h"

namespace tpk {

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

  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
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
    hipError_t ea = allow_lds((const void*)k_gemm_big<E, AF, BM>, (int)lds);                     \
    if (ea != hipSuccess) return ea;                                                            \
    launch((k_gemm_big<E, AF, BM>), g, blk, lds, st, a, b, b2, M, N, K, C, ldc,    \
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

// Split-K variant for batched decode (M <= 64 tokens). A workgroup owns 64 output columns
// (dual: 64 gate and the matching 64 up columns) for all M tokens and one K range; its four waves
// take 16 columns each and share the activation tile through LDS (double-buffered, 128-wide K
// stages), so the activations are read once per 64 columns instead of once per 16. The weight
// stream of each wave goes straight to registers, one stage ahead. Each split writes its fp32
// partial tile to workspace; k_splitk_epilogue adds the splits in split order (deterministic)
// and applies the epilogue.
constexpr int SP_BK = 128, SP_LD = SP_BK + 8;

template <int MT, bool DUAL>
__global__ __launch_bounds__(256) void k_gemm_splitk(const uint16_t* __restrict__ A,
                                                     const uint16_t* __restrict__ B,
                                                     const uint16_t* __restrict__ B2, int M,
                                                     int N, int K, int kchunk,
                                                     float* __restrict__ part) {
  constexpr int NB = DUAL ? 2 : 1;
  constexpr int AR = MT * 16;                  // activation rows staged
  constexpr int ACH = AR * SP_BK / 8 / 256;    // 16-byte A chunks per thread per stage
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][AR * SP_LD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 15, fk = (lane >> 4) * 8;
  const int n0 = blockIdx.x * 64, sidx = blockIdx.y;
  const int k0 = sidx * kchunk, k1 = min(K, k0 + kchunk);
  const int col = n0 + wave * 16 + fr;
  const bool cin = col < N;
  const uint16_t* brow = B + (size_t)(cin ? col : 0) * K;
  const uint16_t* brow2 = DUAL ? B2 + (size_t)(cin ? col : 0) * K : nullptr;

  uint4 ra[ACH > 0 ? ACH : 1];
  uint4 rb[SP_BK / 32][NB];
  auto gload = [&](int ks) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const int c = tid + i * 256, r = c / (SP_BK / 8), k = ks + (c % (SP_BK / 8)) * 8;
      ra[i] = (r < M && k < k1) ? *(const uint4*)(A + (size_t)r * K + k) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < SP_BK / 32; ++u) {
      const int k = ks + u * 32 + fk;
      const bool ok = cin && k < k1;
      rb[u][0] = ok ? ld_stream16(brow + k) : make_uint4(0, 0, 0, 0);
      if constexpr (DUAL) rb[u][NB - 1] = ok ? ld_stream16(brow2 + k) : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const int c = tid + i * 256, r = c / (SP_BK / 8), kc = (c % (SP_BK / 8)) * 8;
      *(uint4*)(&sA[buf][r * SP_LD + kc]) = ra[i];
    }
  };

  floatx4 acc[NB][MT];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int i = 0; i < MT; ++i) acc[b][i] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int nst = (k1 > k0) ? (k1 - k0 + SP_BK - 1) / SP_BK : 0;
  if (nst > 0) {
    gload(k0);
    sstore(0);
  }
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    const int cur = st & 1;
    uint4 bcur[SP_BK / 32][NB];
#pragma unroll
    for (int u = 0; u < SP_BK / 32; ++u)
#pragma unroll
      for (int b = 0; b < NB; ++b) bcur[u][b] = rb[u][b];
    if (st + 1 < nst) gload(k0 + (st + 1) * SP_BK);
#pragma unroll
    for (int u = 0; u < SP_BK / 32; ++u) {
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const bf16x8 af = *(const bf16x8*)(&sA[cur][(i * 16 + fr) * SP_LD + u * 32 + fk]);
#pragma unroll
        for (int b = 0; b < NB; ++b)
          acc[b][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              af, __builtin_bit_cast(bf16x8, bcur[u][b]), acc[b][i], 0, 0, 0);
      }
    }
    if (st + 1 < nst) sstore(cur ^ 1);
    __syncthreads();
  }
  // Partial tile: part[sidx][row][col] (dual: gate at col, up at N + col).
  const int ncols = DUAL ? 2 * N : N;
  if (!cin) return;
  float* pbase = part + (size_t)sidx * M * ncols;
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = i * 16 + (lane >> 4) * 4 + r;
      if (row >= M) continue;
      pbase[(size_t)row * ncols + col] = acc[0][i][r];
      if constexpr (DUAL) pbase[(size_t)row * ncols + N + col] = acc[NB - 1][i][r];
    }
}

// The same split-K GEMM with both operands fed through a six-slot LDS ring by direct-to-LDS
// loads (used when K % 64 == 0). The weight tile of a stage is read as 8 rows x 128 bytes per
// wave instruction (the register-fed form above reads 16 rows x 64 bytes, which the HBM serves at
// well under half the rate of longer row segments), and five stages stay in flight per
// workgroup, so a few hundred workgroups keep enough bytes outstanding to stream the weights at
// HBM rate. Stage layout: the activation rows (AR = 16 MT) then the weight rows (64, gated: 64
// gate then 64 up), 64 bf16 each, 16-byte chunks XOR-swizzled by row % 8.
constexpr int SD_BK = 64, SD_ST = 6;

template <int MT, bool DUAL>
__global__ __launch_bounds__(256) void k_gemm_splitk_dma(const uint16_t* __restrict__ A,
                                                         const uint16_t* __restrict__ B,
                                                         const uint16_t* __restrict__ B2, int M,
                                                         int N, int K, int kchunk,
                                                         float* __restrict__ part, GemmRanks gr) {
  if (gr.n > 1) {  // every rank in one launch (blockIdx.z = rank)
    const int r = blockIdx.z;
    A = (const uint16_t*)gr.a[r];
    B = (const uint16_t*)gr.b[r];
    B2 = (const uint16_t*)gr.b2[r];
    part = (float*)gr.c[r];
  }
  constexpr int NB = DUAL ? 2 : 1;
  constexpr int AR = MT * 16;                       // activation rows staged
  constexpr int BR = 64 * NB;                       // weight rows staged
  constexpr int STAGE = (AR + BR) * SD_BK;          // bf16 elements per slot
  constexpr int A_WL = AR / 8;                      // 1 KB wave-loads of A per stage
  constexpr int A_PW = (A_WL + 3) / 4;              // per wave (surplus loads repeat one)
  constexpr int B_PW = BR / 8 / 4;                  // per wave
  constexpr int LPW = A_PW + B_PW;                  // loads per wave per stage
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = blockIdx.x * 64, sidx = blockIdx.y;
  const int k0 = sidx * kchunk, k1 = min(K, k0 + kchunk);
  const int nst = (k1 - k0) / SD_BK;  // K % 64 == 0 and kchunk % 64 == 0: whole stages

  // Lane l of a wave-load covers row l / 8 of an 8-row group and stores its 16 bytes at chunk
  // l % 8 of that row in LDS, so it loads global chunk (l % 8) ^ (row % 8). Rows past M or N load
  // a clamped (valid) row and are never stored.
  const int lrow = lane >> 3, lpc = lane & 7;
  const int lchunk = (lpc ^ lrow) << 4;
  auto issue = [&](int slot, int stg) {
    uint16_t* st = smem + slot * STAGE;
    const uint32_t kb = (uint32_t)(k0 + min(stg, nst - 1) * SD_BK) * 2;
#pragma unroll
    for (int i = 0; i < A_PW; ++i) {
      const int g = (wave * A_PW + i) % A_WL;  // a repeated group writes identical bytes
      const int row = min(g * 8 + lrow, M - 1);
      const char* src = (const char*)(A + (size_t)row * K) + kb + lchunk;
      __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)(st + g * 8 * SD_BK), 16,
                                       0, 0);
    }
#pragma unroll
    for (int i = 0; i < B_PW; ++i) {
      const int g = wave * B_PW + i;  // 8-row group of the staged weight rows
      const uint16_t* base;
      int col;
      if constexpr (DUAL) {
        base = (g < 8) ? B : B2;
        col = n0 + (g & 7) * 8 + lrow;
      } else {
        base = B;
        col = n0 + g * 8 + lrow;
      }
      const char* src = (const char*)(base + (size_t)min(col, N - 1) * K) + kb + lchunk;
      __builtin_amdgcn_global_load_lds((glb_void_t*)src,
                                       (lds_void_t*)(st + (AR + g * 8) * SD_BK), 16, 0, 0);
    }
  };

  floatx4 acc[NB][MT];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int i = 0; i < MT; ++i) acc[b][i] = floatx4{0.f, 0.f, 0.f, 0.f};
  const int fr = lane & 15, fq = lane >> 4;

#pragma unroll
  for (int s = 0; s < SD_ST - 1; ++s) issue(s, s);
  for (int stg = 0; stg < nst; ++stg) {
    // Stage stg has landed for this wave once only the SD_ST - 2 newer stages remain in flight;
    // after the barrier for every wave, and every wave is done reading slot (stg - 1) % SD_ST.
    wait_vmcnt<(SD_ST - 2) * LPW>();
    __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    issue((stg + SD_ST - 1) % SD_ST, stg + SD_ST - 1);
    const uint16_t* a_s = smem + (stg % SD_ST) * STAGE;
    const uint16_t* b_s = a_s + AR * SD_BK;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int sw = 8 * ((kk * 4 + fq) ^ (fr & 7));
      bf16x8 bf[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b)
        bf[b] = *(const bf16x8*)(b_s + (b * 64 + wave * 16 + fr) * SD_BK + sw);
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const bf16x8 af = *(const bf16x8*)(a_s + (i * 16 + fr) * SD_BK + sw);
#pragma unroll
        for (int b = 0; b < NB; ++b)
          acc[b][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[b], acc[b][i], 0, 0, 0);
      }
    }
  }
  // The clamped loads past the last stage may still be in flight.
  wait_vmcnt<0>();
  const int col = n0 + wave * 16 + fr;
  if (col >= N) return;
  const int ncols = DUAL ? 2 * N : N;
  float* pbase = part + (size_t)sidx * M * ncols;
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = i * 16 + fq * 4 + r;
      if (row >= M) continue;
      pbase[(size_t)row * ncols + col] = acc[0][i][r];
      if constexpr (DUAL) pbase[(size_t)row * ncols + N + col] = acc[NB - 1][i][r];
    }
}

// Sum of the S split-K partial tiles, in split order, then the epilogue. A thread owns four
// consecutive columns of one row (V4: N % 4 == 0, C and ldc 16-byte / 4-element aligned; else
// one column) and issues the loads of four splits before it adds them, so the split loads
// overlap instead of forming a chain of dependent round trips. Every rank in one launch
// (gr.n > 1): blockIdx.y = rank, its partial tiles at gr.a[rank] and its output at gr.c[rank].
template <int EPI, int ACTF, bool V4>
__global__ __launch_bounds__(256) void k_splitk_epilogue(const float* __restrict__ part, int S,
                                                         int M, int N, void* __restrict__ C,
                                                         int ldc, GemmRanks gr) {
  constexpr bool DUAL = (EPI == EPI_GATED);
  if (gr.n > 1) {
    part = (const float*)gr.a[blockIdx.y];
    C = gr.c[blockIdx.y];
  }
  constexpr int W = V4 ? 4 : 1;
  typedef __attribute__((__vector_size__(W * sizeof(float)))) float vec;
  const int ncols = DUAL ? 2 * N : N;
  const int nv = N / W;
  const size_t total = (size_t)M * nv;
  const size_t slab = (size_t)M * ncols;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total;
       i += (size_t)gridDim.x * blockDim.x) {
    const int row = (int)(i / nv), col = (int)(i % nv) * W;
    const float* p = part + (size_t)row * ncols + col;
    vec g = {}, u = {};
    int s = 0;
    for (; s + 4 <= S; s += 4) {
      vec a[4], b[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        a[k] = *(const vec*)(p + (s + k) * slab);
        if constexpr (DUAL) b[k] = *(const vec*)(p + (s + k) * slab + N);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        g += a[k];
        if constexpr (DUAL) u += b[k];
      }
    }
    for (; s < S; ++s) {
      g += *(const vec*)(p + s * slab);
      if constexpr (DUAL) u += *(const vec*)(p + s * slab + N);
    }
    const size_t o = (size_t)row * ldc + col;
    if constexpr (EPI == EPI_F32) {
      *(vec*)((float*)C + o) = g;
    } else {
      uint16_t h[W];
#pragma unroll
      for (int k = 0; k < W; ++k)
        h[k] = f32_to_bf16(EPI == EPI_GATED ? gated<ACTF>(g[k], u[k]) : g[k]);
      if constexpr (V4)
        *(uint2*)((uint16_t*)C + o) = make_uint2(h[0] | ((uint32_t)h[1] << 16),
                                                 h[2] | ((uint32_t)h[3] << 16));
      else
        ((uint16_t*)C)[o] = h[0];
    }
  }
}

template <bool V4>
static hipError_t splitk_epilogue(int epi, int actf, const float* part, int S, int M, int N,
                                  void* C, int ldc, hipStream_t st, const GemmRanks& gr) {
  const size_t total = (size_t)M * N / (V4 ? 4 : 1);
  dim3 eg((unsigned)((total + 255) / 256 < 8192 ? (total + 255) / 256 : 8192),
          gr.n > 1 ? gr.n : 1),
      eb(256);
#define TPK_EPI(E, A) launch((k_splitk_epilogue<E, A, V4>), eg, eb, 0, st, part, S, M, N, C, ldc, gr)
  switch (epi) {
    case EPI_ACT: TPK_EPI(EPI_ACT, 0); break;
    case EPI_F32: TPK_EPI(EPI_F32, 0); break;
    case EPI_BF16: TPK_EPI(EPI_BF16, 0); break;
    case EPI_GATED:
      if (actf == 0) TPK_EPI(EPI_GATED, 0);
      else TPK_EPI(EPI_GATED, 1);
      break;
    default: return hipErrorInvalidValue;
  }
#undef TPK_EPI
  return hipGetLastError();
}

hipError_t launch_splitk_epilogue(int epi, int actf, const float* part, int S, int M, int N,
                                  void* C, int ldc, hipStream_t st, const GemmRanks* gr) {
  const GemmRanks one{};
  const GemmRanks& g = gr ? *gr : one;
  if (gr && (gr->n < 1 || gr->n > kMaxRanks)) return hipErrorInvalidValue;
  bool v4 = N % 4 == 0 && ldc % 4 == 0 && (uintptr_t)C % 16 == 0 && (uintptr_t)part % 16 == 0;
  for (int r = 0; gr && r < gr->n; ++r)
    v4 = v4 && (uintptr_t)gr->c[r] % 16 == 0 && (uintptr_t)gr->a[r] % 16 == 0;
  return v4 ? splitk_epilogue<true>(epi, actf, part, S, M, N, C, ldc, st, g)
            : splitk_epilogue<false>(epi, actf, part, S, M, N, C, ldc, st, g);
}

// Split count for the split-K variants: enough workgroups to cover the chip, K ranges a multiple
// of the 128-wide stage and at least 256 long. The direct-to-LDS form (K % 64 == 0) holds one
// workgroup per CU (its ring takes most of the LDS), so it stays within one round of 256.
void splitk_plan(int N, int K, bool dual, int* S, int* kchunk) {
  const int tiles = (N + 63) / 64;
  int s = (K % SD_BK == 0) ? 256 / tiles : (256 + tiles - 1) / tiles;
  const int smax = (K + 255) / 256;
  if (s > smax) s = smax;
  if (s < 1) s = 1;
  int kc = (K + s - 1) / s;
  kc = (kc + SP_BK - 1) / SP_BK * SP_BK;
  *kchunk = kc;
  *S = (K + kc - 1) / kc;
  (void)dual;
}

size_t splitk_workspace_bytes(int M, int N, int K, bool dual) {
  int S, kc;
  splitk_plan(N, K, dual, &S, &kc);
  return (size_t)S * M * (dual ? 2 * N : N) * sizeof(float);
}

static hipError_t splitk_impl(int epi, int actf, int M, int N, int K, const void* A,
                              const void* B, const void* B2, void* C, int ldc, float* part,
                              hipStream_t st, int* parts_only, const GemmRanks& gr) {
  if (M == 0 || N == 0) return hipSuccess;
  if (M > 64) return hipErrorInvalidValue;
  const bool dual = (epi == EPI_GATED);
  int S, kc;
  // A launch over all ranks counts every rank's tiles toward filling the chip.
  const int nr = gr.n > 1 ? gr.n : 1;
  splitk_plan(N * nr, K, dual, &S, &kc);
  dim3 g((N + 63) / 64, S, nr), blk(256);
  const uint16_t *a = (const uint16_t*)A, *b = (const uint16_t*)B, *b2 = (const uint16_t*)B2;
  const int mt = (M + 15) / 16;
  if (K % SD_BK == 0) {
    // Direct-to-LDS form; the dynamic LDS of a six-slot ring exceeds the default 64 KB.
#define TPK_SD(MTV, DV)                                                                          \
  do {                                                                                           \
    constexpr size_t lds = (size_t)SD_ST * (MTV * 16 + 64 * (DV ? 2 : 1)) * SD_BK * 2;          \
    hipError_t ea = allow_lds((const void*)k_gemm_splitk_dma<MTV, DV>, (int)lds);                \
    if (ea != hipSuccess) return ea;                                                             \
    launch((k_gemm_splitk_dma<MTV, DV>), g, blk, lds, st, a, b, b2, M, N, K, kc, part, gr);     \
  } while (0)
#define TPK_SDM(MTV) \
  if (dual) TPK_SD(MTV, true); else TPK_SD(MTV, false)
    switch (mt) {
      case 1: TPK_SDM(1); break;
      case 2: TPK_SDM(2); break;
      case 3: TPK_SDM(3); break;
      default: TPK_SDM(4); break;
    }
#undef TPK_SDM
#undef TPK_SD
  } else {
#define TPK_SK(MTV)                                                                              \
  if (dual) launch((k_gemm_splitk<MTV, true>), g, blk, 0, st, a, b, b2, M, N, K, kc, part); \
  else launch((k_gemm_splitk<MTV, false>), g, blk, 0, st, a, b, b2, M, N, K, kc, part)
    switch (mt) {
      case 1: TPK_SK(1); break;
      case 2: TPK_SK(2); break;
      case 3: TPK_SK(3); break;
      default: TPK_SK(4); break;
    }
#undef TPK_SK
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (parts_only) {  // the caller sums the S partial tiles itself
    *parts_only = S;
    return hipSuccess;
  }
  return launch_splitk_epilogue(epi, actf, part, S, M, N, C, ldc, st);
}

hipError_t launch_gemm_splitk(int epi, int actf, int M, int N, int K, const void* A,
                              const void* B, const void* B2, void* C, int ldc, float* part,
                              hipStream_t st, int* parts_only) {
  return splitk_impl(epi, actf, M, N, K, A, B, B2, C, ldc, part, st, parts_only, GemmRanks{});
}

hipError_t launch_gemm_splitk_ranks(int epi, int M, int N, int K, const GemmRanks& gr,
                                    hipStream_t st, int* parts) {
  if (gr.n < 1 || gr.n > kMaxRanks || K % SD_BK != 0 || !parts) return hipErrorInvalidValue;
  for (int r = 0; r < gr.n; ++r)
    if (!gr.a[r] || !gr.b[r] || !gr.c[r] || (epi == EPI_GATED && !gr.b2[r]))
      return hipErrorInvalidValue;
  return splitk_impl(epi, 0, M, N, K, gr.a[0], gr.b[0], gr.b2[0], nullptr, 0, (float*)gr.c[0],
                     st, parts, gr);
}

// Prefill GEMM with a three-stage LDS ring filled by direct-to-LDS loads (global_load_lds_dwordx4,
// gfx950): a wave-wide load drops 64 x 16 bytes straight into LDS, so no registers hold staged
// data and two K-tiles stay in flight while the third is multiplied. Rows of 64 bf16 are stored
// with their eight 16-byte chunks XOR-swizzled by (row & 7): the DMA writes stay contiguous and
// the MFMA operand reads (16 rows, one chunk each) hit distinct banks. Tiles and epilogues as in
// k_gemm_big. Needs K % 64 == 0; rows and columns past M and N load clamped (valid) addresses and
// their results are never stored.

constexpr int LG_BK = 64, LG_ST = 3;

template <int EPI, int ACTF, int BM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, BM == 256 ? 1 : 2))) void k_gemm_lds(const uint16_t* __restrict__ A,
                                                  const uint16_t* __restrict__ B,
                                                  const uint16_t* __restrict__ B2, int M, int N,
                                                  int K, void* __restrict__ C, int ldc,
                                                  int tiles_m, int tiles_n, RopeEpi re) {
  constexpr bool DUAL = (EPI == EPI_GATED);
  constexpr int WM = BM / 2, TM = WM / 16, TN = 4;
  constexpr int A_LOADS = BM / 8 / 4;   // 1 KB wave-loads of A per wave per stage
  constexpr int B_LOADS = 128 / 8 / 4;  // ... of B
  constexpr int LPS = A_LOADS + B_LOADS;
  constexpr int STAGE = (BM + 128) * LG_BK;  // bf16 elements per stage
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];

  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
  // The last tile in M (and in N) is shifted back to end at the matrix edge, so every load is in
  // bounds without per-row clamps; rows and columns before ms0 / ns0 belong to the previous tile
  // and are not stored twice. The launcher guarantees M >= BM and N >= the tile width.
  constexpr int NW = DUAL ? 64 : 128;
  const int ms0 = tm * BM, ns0 = tn * NW;
  const int m0 = min(ms0, M - BM), n0 = min(ns0, N - NW);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  // Rotary epilogue: lane k of wave w holds the position and KV page of tile row w + 4 k, loaded
  // now so that the epilogue's loads do not wait on them.
  int pos_l = 0, page_l = 0;
  if constexpr (EPI == EPI_ROPE) {
    if (lane < BM / 4) {
      const int t = m0 + wave + 4 * lane;
      pos_l = min(max(re.positions[t], 0), re.pos_limit - 1);
      const int seq = (re.mode == 0) ? t : 0;
      page_l = min(max(re.block_table[(size_t)seq * re.max_pages + pos_l / re.ps], 0),
                   re.n_pages - 1);
    }
  }

  // Wave-load i of A covers tile rows (wave * A_LOADS + i) * 8 + lane / 8, 16 bytes each; since
  // those row groups start at multiples of 8, the swizzled chunk (lane % 8) ^ (row % 8) and thus
  // the lane's byte offset inside a group is the same for every load, A and B alike. Bases stay
  // wave-uniform (scalar registers); only that one 32-bit offset lives in a vector register.
  const int lrow = lane >> 3, lpc = lane & 7;
  const uint32_t lane_off = (uint32_t)((lrow * K + ((lpc ^ lrow) << 3)) * 2);
  const char* a_base = (const char*)(A + (size_t)(m0 + wave * A_LOADS * 8) * K);
  const size_t grp_stride = (size_t)8 * K * 2;  // bytes between consecutive 8-row groups
  auto issue = [&](int stage_slot, int k0) {
    uint16_t* st = smem + stage_slot * STAGE;
    const size_t kb = (size_t)k0 * 2;
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i)
      __builtin_amdgcn_global_load_lds((glb_void_t*)(a_base + i * grp_stride + kb + lane_off),
                                       (lds_void_t*)(st + (wave * A_LOADS + i) * 8 * LG_BK), 16,
                                       0, 0);
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) {
      const int g = wave * B_LOADS + i;  // 8-row group of the 128 staged B rows
      const char* src;
      if constexpr (DUAL)
        src = (const char*)((g < 8 ? B : B2) + (size_t)(n0 + (g & 7) * 8) * K);
      else
        src = (const char*)(B + (size_t)(n0 + g * 8) * K);
      __builtin_amdgcn_global_load_lds((glb_void_t*)(src + kb + lane_off),
                                       (lds_void_t*)(st + BM * LG_BK + g * 8 * LG_BK), 16, 0, 0);
    }
  };

  floatx4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  auto brow = [&](int j) -> int {
    if constexpr (DUAL) return (j < 2 ? 0 : 64) + wn * 32 + (j & 1) * 16;
    else return wn * 64 + j * 16;
  };
  const int fr = lane & 15, fq = lane >> 4;
  const int nk = K / LG_BK;
  // Operand fragments of one 32-deep k-step: TN of B, TM of A, read from a swizzled stage.
  struct Frag {
    bf16x8 a[TM], b[TN];
  };
  auto load_frag = [&](Frag& f, int slot, int kk) {
    const uint16_t* a_s = smem + slot * STAGE;
    const uint16_t* b_s = a_s + BM * LG_BK;
    const int kc = kk * 4 + fq;  // logical 16-byte chunk of this lane's 8 k values
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int r = brow(j) + fr;
      f.b[j] = *(const bf16x8*)(b_s + r * LG_BK + 8 * (kc ^ (r & 7)));
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int r = wm * WM + i * 16 + fr;
      f.a[i] = *(const bf16x8*)(a_s + r * LG_BK + 8 * (kc ^ (r & 7)));
    }
  };
  auto mma = [&](const Frag& f) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
  };

  // Schedule per K-tile kt (BK = 64, two k-steps): the second k-step's fragments are read while
  // the first k-step's MFMAs run; the barrier that publishes tile kt + 1 sits between the two
  // halves, and the next tile's first fragments are read while the second half's MFMAs run. So
  // LDS read latency and the barrier wait overlap matrix work instead of adding to it.
  issue(0, 0);
  if (nk > 1) issue(1, LG_BK);
  if (nk > 1) wait_vmcnt<LPS>();
  else wait_vmcnt<0>();
  // Bare barrier: the memory clobber keeps the compiler from moving LDS accesses across it.
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if (nk > 2) issue(2, 2 * LG_BK);
  Frag cur, nxt;
  load_frag(cur, 0, 0);
  int kt = 0;
  // Steady state, free of branches between the two MFMA halves (a branch there makes the register
  // allocator copy accumulators around): tiles kt + 1 and kt + 2 are in flight, kt + 3 is issued.
  constexpr int NF = TM + TN, NMMA = TM * TN;
  static_assert(NMMA >= 2 * NF && NMMA >= LPS + NF, "MFMA count must cover the interleaved reads");
  for (; kt + 3 < nk; ++kt) {
    const int slot = kt % LG_ST;
    load_frag(nxt, slot, 1);
    mma(cur);
    // Scheduling hints: two MFMAs, then one fragment read, so the reads hide under matrix work.
#pragma unroll
    for (int g = 0; g < NF; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
    }
    if constexpr (NMMA > 2 * NF) __builtin_amdgcn_sched_group_barrier(0x008, NMMA - 2 * NF, 0);
    // Nothing crosses the wait + barrier below (MFMAs touch no memory, so the asm alone would not
    // stop the scheduler from moving them over it).
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<LPS>();
    // After this barrier every wave has finished reading tile kt (its reads completed before
    // the barrier), so tile kt + 3 may overwrite that slot.
    __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    issue(slot, (kt + 3) * LG_BK);
    load_frag(cur, (kt + 1) % LG_ST, 0);
    mma(nxt);
    // Hint: the global->LDS loads, then the next tile's first reads, each after one MFMA.
#pragma unroll
    for (int g = 0; g < LPS; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);  // VMEM (direct-to-LDS load)
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
#pragma unroll
    for (int g = 0; g < NF; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    if constexpr (NMMA > LPS + NF) __builtin_amdgcn_sched_group_barrier(0x008, NMMA - LPS - NF, 0);
  }
  // The last (at most three) tiles: nothing more to issue.
  for (; kt < nk; ++kt) {
    load_frag(nxt, kt % LG_ST, 1);
    mma(cur);
    if (kt + 1 < nk) {
      if (kt + 2 < nk) wait_vmcnt<LPS>();
      else wait_vmcnt<0>();
      __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      load_frag(cur, (kt + 1) % LG_ST, 0);
    }
    mma(nxt);
  }

  if constexpr (EPI == EPI_ROPE) {
    // Fused rotary embedding + KV append (launcher: N % 128 == 0 and hd of 64 or 128, so the
    // tile's 128 columns are whole heads and never shifted). The tile, rounded to bf16 as the
    // plain QKV output would be, goes through LDS (free once every wave is past its last reads)
    // with each row's position and KV page; rows are padded to 130 elements so that 16 rows of
    // one column sit in distinct banks.
    constexpr int TS = 130;
    __syncthreads();
    uint16_t* tile = smem;                           // [BM][TS] bf16
    int* s_pp = (int*)(smem + ((BM * TS + 7) & ~7));  // [BM][2]: position, page
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          tile[(wm * WM + i * 16 + fq * 4 + r) * TS + wn * 64 + j * 16 + fr] =
              f32_to_bf16(acc[i][j][r]);
    if (lane < BM / 4) {
      s_pp[2 * (wave + 4 * lane)] = pos_l;
      s_pp[2 * (wave + 4 * lane) + 1] = page_l;
    }
    __syncthreads();
    const int hd = re.hd, half = hd >> 1;
    const float2* rope = (const float2*)re.rope;
    // q and k heads: thread (wave w, lane p) owns rotation pair p of the tile's 64 (head hh,
    // element e) and rows w, w + 4, ...; a row's position and page are lane reads of the
    // registers loaded at the start, so the unrolled rows' loads are independent.
    {
      const int p = lane;
      const int hh = p / half, e = p - hh * half;
      const int head = (n0 + hh * hd) / hd;
      const int col = hh * hd + e;
      if (head < re.hq + re.hk) {
#pragma unroll
        for (int k = 0; k < BM / 4; ++k) {
          const int rl = wave + 4 * k;
          const int t = m0 + rl;
          if (t < ms0) continue;  // stored by the previous tile
          const int pos = __builtin_amdgcn_readlane(pos_l, k);
          const int page = __builtin_amdgcn_readlane(page_l, k);
          const float a = bf16_to_f32(tile[rl * TS + col]), b = bf16_to_f32(tile[rl * TS + col + half]);
          const float2 cs = rope[(size_t)pos * half + e];
          const uint16_t ra = f32_to_bf16(a * cs.x - b * cs.y), rb = f32_to_bf16(b * cs.x + a * cs.y);
          uint16_t* d = head < re.hq
              ? (uint16_t*)re.q_out + ((size_t)t * re.hq + head) * hd
              : (uint16_t*)re.k_pages + (((size_t)page * re.hk + (head - re.hq)) * re.ps + pos % re.ps) * hd;
          d[e] = ra;
          d[e + half] = rb;
        }
      }
    }
    // v heads, into the transposed pages ([page][kv head][hd][slot]): lanes take 16 consecutive
    // rows of one hd element, so consecutive positions land in one 32-byte page row.
    for (int hh = 0; hh < 128 / hd; ++hh) {
      const int head = (n0 + hh * hd) / hd;
      if (head < re.hq + re.hk) continue;  // uniform
      const int g = head - re.hq - re.hk;
      const int rs = tid & 15, e0 = tid >> 4;
#pragma unroll 2
      for (int rb = 0; rb < BM / 16; ++rb) {
        const int rl = 16 * rb + rs;
        if (m0 + rl < ms0) continue;
        const int pos = s_pp[2 * rl], page = s_pp[2 * rl + 1];
        uint16_t* dv = (uint16_t*)re.v_pages + ((size_t)page * re.hk + g) * hd * re.ps + pos % re.ps;
#pragma unroll
        for (int e = e0; e < 128; e += 16)
          if (e < hd) dv[(size_t)e * re.ps] = tile[rl * TS + hh * hd + e];
      }
    }
    return;
  }

#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = m0 + wm * WM + i * 16 + fq * 4 + r;
      if (row < ms0) continue;  // stored by the previous tile
      if constexpr (DUAL) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = n0 + wn * 32 + j * 16 + fr;
          if (col >= ns0)
            ((uint16_t*)C)[(size_t)row * ldc + col] =
                f32_to_bf16(gated<ACTF>(acc[i][j][r], acc[i][j + 2][r]));
        }
      } else {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int col = n0 + wn * 64 + j * 16 + fr;
          if (col < ns0) continue;
          const size_t o = (size_t)row * ldc + col;
          if constexpr (EPI == EPI_F32) ((float*)C)[o] = acc[i][j][r];
          else ((uint16_t*)C)[o] = f32_to_bf16(acc[i][j][r]);
        }
      }
    }
  }
}

template <int BM>
static hipError_t lds_bm(int epi, int actf, int M, int N, int K, const uint16_t* a,
                         const uint16_t* b, const uint16_t* b2, void* C, int ldc, hipStream_t st,
                         const RopeEpi* re = nullptr) {
  const int tiles_m = (M + BM - 1) / BM;
  const int tiles_n = (epi == EPI_GATED) ? (N + 63) / 64 : (N + 127) / 128;
  if (M < BM || N < ((epi == EPI_GATED) ? 64 : 128) || K % LG_BK != 0) return hipErrorInvalidValue;
  dim3 g(tiles_m * tiles_n), blk(256);
  const size_t lds = (size_t)LG_ST * (BM + 128) * LG_BK * sizeof(uint16_t);
#define TPK_LDS(E, AF)                                                                          \
  do {                                                                                          \
    hipError_t ea = allow_lds((const void*)k_gemm_lds<E, AF, BM>, (int)lds);                     \
    if (ea != hipSuccess) return ea;                                                            \
    launch((k_gemm_lds<E, AF, BM>), g, blk, lds, st, a, b, b2, M, N, K, C, ldc, tiles_m,        \
           tiles_n, rope_arg);                                                                  \
  } while (0)
  RopeEpi rope_arg{};
  if (re) rope_arg = *re;
  switch (epi) {
    case EPI_ACT: TPK_LDS(EPI_ACT, 0); break;
    case EPI_F32: TPK_LDS(EPI_F32, 0); break;
    case EPI_BF16: TPK_LDS(EPI_BF16, 0); break;
    case EPI_GATED:
      if (actf == 0) TPK_LDS(EPI_GATED, 0);
      else TPK_LDS(EPI_GATED, 1);
      break;
    case EPI_ROPE:
      if (!re) return hipErrorInvalidValue;
      TPK_LDS(EPI_ROPE, 0);
      break;
    default:
      return hipErrorInvalidValue;
  }
#undef TPK_LDS
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
      launch((k_gemm_skinny<EPI_ACT, 0, MT>), g, blk, 0, st, a, b, b2, M, N, K, C, ldc);
      break;
    case EPI_F32:
      launch((k_gemm_skinny<EPI_F32, 0, MT>), g, blk, 0, st, a, b, b2, M, N, K, C, ldc);
      break;
    case EPI_BF16:
      launch((k_gemm_skinny<EPI_BF16, 0, MT>), g, blk, 0, st, a, b, b2, M, N, K, C, ldc);
      break;
    case EPI_GATED:
      if (actf == 0)
        launch((k_gemm_skinny<EPI_GATED, 0, MT>), g, blk, 0, st, a, b, b2, M, N, K, C, ldc);
      else
        launch((k_gemm_skinny<EPI_GATED, 1, MT>), g, blk, 0, st, a, b, b2, M, N, K, C, ldc);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

bool gemm_rope_supported(int M, int N, int K, int hd) {
  return M >= 128 && N >= 128 && N % 128 == 0 && K % LG_BK == 0 && (hd == 64 || hd == 128) &&
         gemm_wide_tiles(EPI_ACT, M, N) < 192;
}

hipError_t launch_gemm_qkv_rope(int M, int N, int K, const void* A, const void* B,
                                const RopeEpi& re, hipStream_t st) {
  if (!gemm_rope_supported(M, N, K, re.hd) || re.hd * (re.hq + 2 * re.hk) != N)
    return hipErrorInvalidValue;
  const uint16_t *a = (const uint16_t*)A, *b = (const uint16_t*)B;
  const long t256 = (long)((M + 255) / 256) * ((N + 127) / 128);
  if (M >= 256 && t256 >= 256) return lds_bm<256>(EPI_ROPE, 0, M, N, K, a, b, nullptr, nullptr, 0, st, &re);
  return lds_bm<128>(EPI_ROPE, 0, M, N, K, a, b, nullptr, nullptr, 0, st, &re);
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
    // Wide tiles when they alone nearly fill the chip (LDS traffic per MFMA is lowest there).
    if (K % LG_BK == 0 && gemm_wide_tiles(epi, M, N) >= 192)
      return launch_gemm_wide(epi, actf, M, N, K, A, B, B2, C, ldc, st);
    // The direct-to-LDS kernel needs whole K-tiles and at least one full tile in N.
    if (K % LG_BK == 0 && N >= ((epi == EPI_GATED) ? 64 : 128)) {
      if (t256 >= 256) return lds_bm<256>(epi, actf, M, N, K, a, bb, b2, C, ldc, st);
      return lds_bm<128>(epi, actf, M, N, K, a, bb, b2, C, ldc, st);
    }
    if (t256 >= 256) return big_bm<256>(epi, actf, M, N, K, a, bb, b2, C, ldc, st);
    return big_bm<128>(epi, actf, M, N, K, a, bb, b2, C, ldc, st);
  }
  dim3 g((N + GB_N - 1) / GB_N, (M + GB_M - 1) / GB_M), b(256);
  switch (epi) {
    case EPI_ACT:
      launch((k_gemm_bf16<EPI_ACT, 0>), g, b, 0, st, a, bb, b2, M, N, K, C, ldc);
      break;
    case EPI_F32:
      launch((k_gemm_bf16<EPI_F32, 0>), g, b, 0, st, a, bb, b2, M, N, K, C, ldc);
      break;
    case EPI_BF16:
      launch((k_gemm_bf16<EPI_BF16, 0>), g, b, 0, st, a, bb, b2, M, N, K, C, ldc);
      break;
    case EPI_GATED:
      if (actf == 0)
        launch((k_gemm_bf16<EPI_GATED, 0>), g, b, 0, st, a, bb, b2, M, N, K, C, ldc);
      else
        launch((k_gemm_bf16<EPI_GATED, 1>), g, b, 0, st, a, bb, b2, M, N, K, C, ldc);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace tpk
