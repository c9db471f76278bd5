// Prefill GEMM, wide tile: 256 x 256 per workgroup (gated: 256 rows x 112 output columns), for
// projections with enough rows and columns to fill the chip with such tiles (the 70B shard's
// gate/up, o_proj and down). Same operand layout and epilogues as the 256 x 128 kernel in
// k_gemm.hip. Eight waves of 64 x 128 (gated 64 x 112), two per SIMD: while one waits (at the
// barrier that publishes a K-tile, on a burst of direct-to-LDS loads, on a fragment read) the
// other keeps the matrix core busy. A wave reads 4 + 8 fragments per 32 MFMAs; the big tile keeps
// the direct-to-LDS writes at 128 bytes per MFMA.
//
// Two LDS slots, each a 64-deep K-tile of A (256 rows) and B (256 rows; gated: 224 rows, 8 gate
// rows then the 8 matching up rows, 14 times), 16-byte chunks XOR-swizzled by row % 8, filled by
// global_load_lds_dwordx4. A gated tile has 112 output columns, so that the 70B shard's 3584 FFN
// columns make 32 tile columns and 256 tiles, one per CU; each 16-column MFMA block holds 8 gate
// and the 8 matching up columns, which meet in one lane through a DPP row rotation. Each K-tile
// is two 32-deep k-steps whose fragment reads are double-buffered in registers; the barrier that
// publishes the next K-tile sits between the steps. Accumulators live in VGPRs (112 or 128 per
// lane).
#include <type_traits>

#include "k_gemm_common.h"
#include "tp_kernels.h"

namespace tpk {

constexpr int WD_BK = 64;  // k per LDS slot

// Staged B rows and output columns per tile (BR: a narrower non-gated tile, 160 columns).
constexpr int wd_brows(int epi, int br = 0) { return br ? br : (epi == EPI_GATED ? 224 : 256); }
constexpr int wd_ncols(int epi, int br = 0) {
  return epi == EPI_GATED ? wd_brows(epi, br) / 2 : wd_brows(epi, br);
}

// Grid: tiles_m * tiles_n tiles times ksplit K ranges. Block b is renumbered so each XCD's share
// is a contiguous run (K range major, then tiles); inside a K range a run walks GM = 4 m-bands
// down before stepping across n, so the tiles one XCD holds at a time reuse both operands in its
// L2. With ksplit > 1 each K range writes its own fp32 partial product, C + range * M * ldc.
template <int EPI, int ACTF, int BR>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_gemm_wide(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
    const uint16_t* __restrict__ B2, int M, int N, int K, void* __restrict__ C, int ldc,
    int tiles_m, int tiles_n, int ksplit, GemmRanks gr) {
  constexpr bool DUAL = (EPI == EPI_GATED);
  constexpr int NBR = wd_brows(EPI, BR);      // staged B rows
  constexpr int NW = wd_ncols(EPI, BR);       // output columns per tile
  constexpr int STAGE = (256 + NBR) * WD_BK;  // bf16 elements per slot
  constexpr int TM = 4, TN = NBR / 32;        // 16 x 16 blocks per wave (4 x 2 waves)
  constexpr int LA = 4;                       // 1 KB wave-loads of A per wave per slot
  constexpr int NGB = NBR / 8;                // 8-row groups of B per slot
  constexpr int LB = (NGB + 7) / 8;           // B wave-loads per wave
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  if (gr.n > 1) {  // every rank in one launch (blockIdx.z = rank)
    const int r = blockIdx.z;
    A = (const uint16_t*)gr.a[r];
    B = (const uint16_t*)gr.b[r];
    B2 = (const uint16_t*)gr.b2[r];
    C = gr.c[r];
  }

  int tm, tn, split;
  {
    constexpr int GM = 4;
    const int b = blockIdx.x, nblk = gridDim.x, tiles = tiles_m * tiles_n;
    const int full = nblk / 8 * 8;
    const int lt = (b < full) ? (b % 8) * (full / 8) + b / 8 : b;
    split = lt / tiles;
    const int t = lt % tiles;
    const int g = t / (GM * tiles_n), r = t % (GM * tiles_n);
    const int gm = min(GM, tiles_m - g * GM);
    tm = g * GM + r % gm;
    tn = r / gm;
  }
  // This block's K range, in 64-deep K-tiles.
  const int nk_all = K / WD_BK, kbase = nk_all / ksplit, krem = nk_all % ksplit;
  const int kt0 = split * kbase + min(split, krem);
  const int nk = kbase + (split < krem ? 1 : 0);
  // Edge tiles shift back inside the matrix (the launcher guarantees M >= 256 and N >= NW); what
  // the previous tile already covers is not stored again.
  const int ms0 = tm * 256, ns0 = tn * NW;
  const int m0 = min(ms0, M - 256), n0 = min(ns0, N - NW);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  __builtin_assume(wave >= 0 && wave < 8);
  // Waves w and w + 4 share a SIMD: same 64-row band, the two column halves.
  const int wm = wave & 3, wn = wave >> 2;

  // Wave-load i covers 8 rows; the lane's swizzled chunk (lane % 8) ^ (row % 8) is the same for
  // every load, so addresses are a wave-uniform base plus one 32-bit lane offset.
  const int lrow = lane >> 3, lpc = lane & 7;
  const uint32_t lane_off = (uint32_t)((lrow * K + ((lpc ^ lrow) << 3)) * 2);
  const char* a_base = (const char*)(A + (size_t)(m0 + wave * LA * 8) * K);
  const size_t grp = (size_t)8 * K * 2;
  auto issue_a = [&](int slot, int kt) {
    uint16_t* st = smem + slot * STAGE;
    const uint32_t off = lane_off + (uint32_t)(kt0 + kt) * (WD_BK * 2);
#pragma unroll
    for (int i = 0; i < LA; ++i)
      __builtin_amdgcn_global_load_lds((glb_void_t*)(a_base + i * grp + off),
                                       (lds_void_t*)(st + (wave * LA + i) * 8 * WD_BK), 16, 0, 0);
  };
  auto issue_b = [&](int slot, int kt) {
    uint16_t* st = smem + slot * STAGE + 256 * WD_BK;
    const uint32_t off = lane_off + (uint32_t)(kt0 + kt) * (WD_BK * 2);
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      // 8-row group of the staged B rows (wave-uniform). Where NGB is not a multiple of 8 the
      // spare waves repeat the last group: the same bytes to the same LDS place, branch-free.
      const int g = min(wave + 8 * i, NGB - 1);
      const char* src;
      if constexpr (DUAL)
        src = (const char*)(((g & 1) ? B2 : B) + (size_t)(n0 + (g >> 1) * 8) * K);
      else
        src = (const char*)(B + (size_t)(n0 + g * 8) * K);
      __builtin_amdgcn_global_load_lds((glb_void_t*)(src + off),
                                       (lds_void_t*)(st + g * 8 * WD_BK), 16, 0, 0);
    }
  };

  floatx4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  // Staged B row of block j (gated: 8 output columns, gate in lanes fr < 8, up above).
  auto brow = [&](int j) -> int { return wn * (NBR / 2) + j * 16; };
  const int fr = lane & 15, fq = lane >> 4;
  struct Frag {
    bf16x8 a[TM], b[TN];
  };
  auto load = [&](Frag& f, int slot, int kk) {
    const uint16_t* a_s = smem + slot * STAGE;
    const uint16_t* b_s = a_s + 256 * WD_BK;
    const int sw = 8 * ((kk * 4 + fq) ^ (fr & 7));
#pragma unroll
    for (int j = 0; j < TN; ++j) f.b[j] = *(const bf16x8*)(b_s + (brow(j) + fr) * WD_BK + sw);
#pragma unroll
    for (int i = 0; i < TM; ++i)
      f.a[i] = *(const bf16x8*)(a_s + (wm * 64 + i * 16 + fr) * WD_BK + sw);
  };
  // MFMAs of block rows [I0, I0 + TM / 2).
  auto mma_rows = [&](const Frag& f, auto i0) {
#pragma unroll
    for (int i = decltype(i0)::value; i < decltype(i0)::value + TM / 2; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
  };
  auto mma = [&](const Frag& f) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
  };
  // Scheduling hints for one region: its global loads first, two MFMAs, then one fragment read
  // per two MFMAs.
  auto hints = [&](auto nvmem) {
    if constexpr (decltype(nvmem)::value > 0)
      __builtin_amdgcn_sched_group_barrier(0x010, decltype(nvmem)::value, 0);  // VMEM
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                          // MFMA
#pragma unroll
    for (int g = 0; g < TM + TN; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                        // LDS read
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, TM * TN - 2 - 2 * (TM + TN), 0);
  };

  Frag x, y;
  issue_a(0, 0);
  issue_b(0, 0);
  wait_vmcnt<0>();
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  issue_a(1, min(1, nk - 1));
  issue_b(1, min(1, nk - 1));
  load(x, 0, 0);
  int kt = 0;
  // Steady state, branch-free so the hints see whole regions. The tile issued two ahead is
  // clamped to the last one (in bounds; its slot is never read again).
  for (; kt + 1 < nk; ++kt) {
    __builtin_amdgcn_sched_barrier(0);
    load(y, kt & 1, 1);
    mma(x);
    hints(std::integral_constant<int, 0>{});
    __builtin_amdgcn_sched_barrier(0);
    // Tile kt + 1 has landed for this wave; after the barrier for every wave, and every wave is
    // done reading slot kt & 1 (its reads completed before the barrier), which then refills.
    wait_vmcnt<0>();
    __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    // The refill goes out in two halves, A with the first half of the MFMAs and the fragment
    // reads, B with the second half (one burst of all loads from every wave at once right after
    // the barrier holds up the fragment reads).
    issue_a(kt & 1, min(kt + 2, nk - 1));
    load(x, (kt + 1) & 1, 0);
    mma_rows(y, std::integral_constant<int, 0>{});
    __builtin_amdgcn_sched_group_barrier(0x010, LA, 0);                          // VMEM
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                           // MFMA
#pragma unroll
    for (int g = 0; g < TM + TN; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                         // LDS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    issue_b(kt & 1, min(kt + 2, nk - 1));
    mma_rows(y, std::integral_constant<int, TM / 2>{});
    __builtin_amdgcn_sched_group_barrier(0x010, LB, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, TM * TN / 2, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  load(y, kt & 1, 1);
  mma(x);
  mma(y);
  // The clamped loads may still be in flight; they must land before the LDS is released.
  wait_vmcnt<0>();

#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = m0 + wm * 64 + i * 16 + fq * 4 + r;
      if (row < ms0) continue;  // stored by the previous tile
      if constexpr (DUAL) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          // Lanes fr and fr ^ 8 swap values (rotation by 8 within each row of 16 lanes).
          const float v = acc[i][j][r];
          const float w = __int_as_float(
              __builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xf, 0xf, false));
          const int col = n0 + wn * (NW / 2) + j * 8 + fr;
          if (fr < 8 && col >= ns0)
            ((uint16_t*)C)[(size_t)row * ldc + col] = f32_to_bf16(gated<ACTF>(v, w));
        }
      } else {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int col = n0 + wn * (NW / 2) + j * 16 + fr;
          if (col < ns0) continue;
          const size_t o = (size_t)row * ldc + col;
          if constexpr (EPI == EPI_F32) ((float*)C + (size_t)split * M * ldc)[o] = acc[i][j][r];
          else ((uint16_t*)C)[o] = f32_to_bf16(acc[i][j][r]);
        }
      }
    }
  }
}

long gemm_wide_tiles(int epi, int M, int N) {
  const int nw = wd_ncols(epi);
  if (M < 256 || N < nw) return 0;
  return (long)((M + 255) / 256) * ((N + nw - 1) / nw);
}

static bool ranks_ok(const GemmRanks* gr, bool dual) {
  if (!gr) return true;
  if (gr->n < 1 || gr->n > kMaxRanks) return false;
  for (int r = 0; r < gr->n; ++r)
    if (!gr->a[r] || !gr->b[r] || !gr->c[r] || (dual && !gr->b2[r])) return false;
  return true;
}

hipError_t launch_gemm_wide(int epi, int actf, int M, int N, int K, const void* A, const void* B,
                          const void* B2, void* C, int ldc, hipStream_t st,
                          const GemmRanks* gr) {
  const int nw = wd_ncols(epi);
  if (M < 256 || N < nw || K % WD_BK != 0) return hipErrorInvalidValue;
  if (!ranks_ok(gr, epi == EPI_GATED)) return hipErrorInvalidValue;
  const GemmRanks one{};
  const GemmRanks& grr = gr ? *gr : one;
  if (gr) {
    A = gr->a[0];
    B = gr->b[0];
    B2 = gr->b2[0];
    C = gr->c[0];
  }
  const int tiles_m = (M + 255) / 256, tiles_n = (N + nw - 1) / nw;
  dim3 g(tiles_m * tiles_n, 1, grr.n > 1 ? grr.n : 1), blk(512);
  const size_t lds = (size_t)2 * (256 + wd_brows(epi)) * WD_BK * sizeof(uint16_t);
  const uint16_t *a = (const uint16_t*)A, *b = (const uint16_t*)B, *b2 = (const uint16_t*)B2;
#define TPK_WIDE(E, AF)                                                                           \
  do {                                                                                          \
    hipError_t ea = allow_lds((const void*)k_gemm_wide<E, AF, 0>, (int)lds);                     \
    if (ea != hipSuccess) return ea;                                                            \
    launch((k_gemm_wide<E, AF, 0>), g, blk, lds, st, a, b, b2, M, N, K, C, ldc, tiles_m,        \
           tiles_n, 1, grr);                                                                    \
  } while (0)
  switch (epi) {
    case EPI_ACT: TPK_WIDE(EPI_ACT, 0); break;
    case EPI_F32: TPK_WIDE(EPI_F32, 0); break;
    case EPI_BF16: TPK_WIDE(EPI_BF16, 0); break;
    case EPI_GATED:
      if (actf == 0) TPK_WIDE(EPI_GATED, 0);
      else TPK_WIDE(EPI_GATED, 1);
      break;
    default:
      return hipErrorInvalidValue;
  }
#undef TPK_WIDE
  return hipGetLastError();
}

// Split-K projection on 256 x 160 tiles: enough tiles times K ranges to give every CU one block,
// for projections too narrow to fill the chip with whole-K tiles (the 70B shard's QKV: 64 tiles,
// four K ranges). Returns 1 when the shape does not gain from it.
int gemm_split_count(int M, int N, int K) {
  if (M < 256 || N < 160 || K % WD_BK != 0) return 1;
  const long tiles = (long)((M + 255) / 256) * ((N + 159) / 160);
  if (tiles >= 128) return 1;
  int s = (int)(256 / tiles);
  if (s > 8) s = 8;
  while (s > 1 && K / WD_BK < 2 * s) --s;
  return s;
}

hipError_t launch_gemm_split_f32(int M, int N, int K, const void* A, const void* B, float* parts,
                                 int ksplit, hipStream_t st, const GemmRanks* gr) {
  constexpr int BR = 160;
  if (M < 256 || N < BR || K % WD_BK != 0 || ksplit < 1 || K / WD_BK < ksplit)
    return hipErrorInvalidValue;
  if (!ranks_ok(gr, false)) return hipErrorInvalidValue;
  const GemmRanks one{};
  const GemmRanks& grr = gr ? *gr : one;
  if (gr) {
    A = gr->a[0];
    B = gr->b[0];
    parts = (float*)gr->c[0];
  }
  const int tiles_m = (M + 255) / 256, tiles_n = (N + BR - 1) / BR;
  dim3 g(tiles_m * tiles_n * ksplit, 1, grr.n > 1 ? grr.n : 1), blk(512);
  const size_t lds = (size_t)2 * (256 + BR) * WD_BK * sizeof(uint16_t);
  hipError_t ea = allow_lds((const void*)k_gemm_wide<EPI_F32, 0, BR>, (int)lds);
  if (ea != hipSuccess) return ea;
  launch((k_gemm_wide<EPI_F32, 0, BR>), g, blk, lds, st, (const uint16_t*)A, (const uint16_t*)B,
         (const uint16_t*)nullptr, M, N, K, (void*)parts, N, tiles_m, tiles_n, ksplit, grr);
  return hipGetLastError();
}

}  // namespace tpk
