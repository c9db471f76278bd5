// Causal prefill attention for one rank's heads, bf16, MFMA, with the KV tiles shared by all the
// query heads of a GQA group (TensorSharp "Multi-GPU & Multi-Node", section "How tensor
// parallelism works": every rank attends with its own heads against its own KV cache).
//
// A workgroup takes four 16-row blocks (16 tokens of four query heads of one KV head, or more
// tokens of fewer heads when the group is smaller), one per wave. Key tiles of 64 keys (four
// 16-token pages) come into a double-buffered LDS ring by direct-to-LDS loads (K rows with their
// 16-byte chunks XOR-swizzled by key, V as stored: transposed per page), so the K/V bytes leave L2
// once per workgroup rather than once per (token block, head). Scores and output are computed
// transposed, S^T = K Q^T and O^T += V^T P^T (16x16x32 MFMA): each lane then owns one query row,
// the row's online softmax (exp2 domain, causal mask on edge tiles only) needs two cross-lane
// steps, and P goes from the score registers straight into the next MFMA without an LDS trip.
#include "k_gemm_common.h"
#include "tp_kernels.h"

namespace tpk {

typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;

constexpr int AP_KT = 64;   // keys per tile (four 16-slot pages)
constexpr int AP_ST = 4;    // K/V tile slots in LDS: three tiles in flight while one is used

__device__ __forceinline__ int ap_clamp(int v, int lo, int hi) {
  return v < lo ? lo : (v > hi ? hi : v);
}

// Reductions over the four lanes l % 16 + 16 i (same row of the transposed tiles) with the
// gfx950 lane-swap instructions (VALU, no LDS round trip): swapping a value with itself leaves
// the lane's own value in one result and its partner's (lane ^ 16, then lane ^ 32) in the other.
__device__ __forceinline__ float ap_rowmax(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float ap_rowsum(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <int HD, int G>
__global__ __launch_bounds__(256) void k_attn_prefill(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kpages,
    const uint16_t* __restrict__ vpages, const int* __restrict__ positions,
    const int* __restrict__ block_table, int max_pages, int n_pages, int hk, int T, int pos_limit,
    uint16_t* __restrict__ out, float scale_log2) {
  constexpr int KS = HD / 32;              // k-steps over hd in Q K^T
  constexpr int NO = HD / 16;              // hd blocks of O
  constexpr int NHW = G < 4 ? G : 4;       // query heads per workgroup
  constexpr int TB = 4 / NHW;              // 16-token blocks per workgroup
  constexpr int CH = HD / 8;               // 16-byte chunks per key row of K
  constexpr int TILE = AP_KT * HD;         // bf16 elements of a K (or V) tile
  constexpr int WLW = TILE * 2 / 1024 / 4; // 1 KB wave-loads per wave per K (or V) tile
  constexpr int KPL = 1024 / (HD * 2);     // keys per K wave-load
  constexpr int VWP = HD * 32 / 1024;      // V wave-loads per page (32 bytes per hd row)
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  __shared__ int s_kmax;

  const int g = blockIdx.y / (G / NHW), hgrp = blockIdx.y % (G / NHW);
  const int t0 = (gridDim.x - 1 - blockIdx.x) * (16 * TB);  // latest tokens first
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fr = lane & 15, fq = lane >> 4;
  const int hq = hk * G;

  // Keys this workgroup needs: up to the largest position among its tokens.
  if (tid == 0) s_kmax = 0;
  __syncthreads();
  if (tid < 16 * TB && t0 + tid < T)
    atomicMax(&s_kmax, ap_clamp(positions[t0 + tid], 0, pos_limit - 1) + 1);
  __syncthreads();
  const int ntiles = (s_kmax + AP_KT - 1) / AP_KT;

  // This wave's 16-row block: token block wave / NHW, head wave % NHW of the group. Lane l works
  // on row (token) l % 16 throughout: S and O are kept transposed (keys or hd along the MFMA
  // rows), so the softmax of a row lives in the four lanes l % 16 + 16 i and P feeds the P V
  // product straight from registers.
  const int tk = t0 + (wave / NHW) * 16 + fr;
  const int head = g * G + hgrp * NHW + wave % NHW;
  const bool row_ok = tk < T;
  const int lim = row_ok ? ap_clamp(positions[row_ok ? tk : 0], 0, pos_limit - 1) + 1 : 1;
  // Tiles ending at or below every row's limit need no causal mask.
  int wmin = row_ok ? lim : 0x7fffffff;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) wmin = min(wmin, __shfl_xor(wmin, off, 64));

  bf16x8 qf[KS];  // Q^T operand: lane row fr, hd chunk fq of each 32-wide step
  {
    const uint16_t* qrow = q + ((size_t)(row_ok ? tk : 0) * hq + head) * HD + fq * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = row_ok ? *(const bf16x8*)(qrow + ks * 32) : bf16x8{};
  }

  // LDS: AP_ST slots, each a K tile [64 keys][HD] then a V tile [4 pages][HD][16].
  auto issue = [&](int slot, int t) {
    uint16_t* ks_ = smem + slot * 2 * TILE;
    uint16_t* vs_ = ks_ + TILE;
#pragma unroll
    for (int i = 0; i < WLW; ++i) {
      const int w = wave * WLW + i;
      // K: keys KPL w ..; lane -> key KPL w + l / CH, LDS chunk l % CH holding global chunk
      // (l % CH) ^ (key % CH).
      {
        const int key = KPL * w + lane / CH, pos = lane % CH;
        const int pg = min(4 * t + key / 16, max_pages - 1);
        const int pid = ap_clamp(block_table[pg], 0, n_pages - 1);
        const uint16_t* src = kpages + (((size_t)pid * hk + g) * 16 + key % 16) * HD +
                              ((pos ^ (key & (CH - 1))) << 3);
        __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)(ks_ + w * 512), 16, 0,
                                         0);
      }
      // V: wave-load w covers 32 hd rows of page w / VWP, as stored ([hd][16 keys] per page).
      {
        const int pi = w / VWP, row = (w % VWP) * 32 + lane / 2;
        const int pg = min(4 * t + pi, max_pages - 1);
        const int pid = ap_clamp(block_table[pg], 0, n_pages - 1);
        const uint16_t* src = vpages + (((size_t)pid * hk + g) * HD + row) * 16 + (lane & 1) * 8;
        __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)(vs_ + w * 512), 16, 0,
                                         0);
      }
    }
  };

  float m = -INFINITY, lsum = 0.f;
  floatx4 o[NO];  // O^T: lane holds O[row fr][hd 16 n + 4 fq + r]
#pragma unroll
  for (int n = 0; n < NO; ++n) o[n] = floatx4{0.f, 0.f, 0.f, 0.f};

  // Tiles past the last one are clamped onto it (in bounds, never used), so every iteration
  // waits for the same count: loads return in issue order.
  constexpr int LPT = 2 * WLW;  // loads per wave per tile
  if (ntiles > 0) {
#pragma unroll
    for (int i = 0; i < AP_ST - 1; ++i) issue(i, min(i, ntiles - 1));
  }
  for (int t = 0; t < ntiles; ++t) {
    // Tile t has landed for this wave once only the AP_ST - 2 newer tiles are in flight; after
    // the barrier for all waves, which have also finished tile t - 1, whose slot then refills.
    wait_vmcnt<(AP_ST - 2) * LPT>();
    __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    issue((t + AP_ST - 1) % AP_ST, min(t + AP_ST - 1, ntiles - 1));
    const uint16_t* ks_ = smem + (t % AP_ST) * 2 * TILE;
    const uint16_t* vs_ = ks_ + TILE;

    // S^T = K Q^T per 16-key block kb: lane holds S[row fr][key 16 kb + 4 fq + r]. All of the
    // tile's K fragments are read first (one LDS round trip), then the four MFMA chains run
    // interleaved.
    bf16x8 kf[4][KS];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int key = 16 * kb + fr;
#pragma unroll
      for (int kc = 0; kc < KS; ++kc)
        kf[kb][kc] = *(const bf16x8*)(ks_ + key * HD + (((kc * 4 + fq) ^ (key & (CH - 1))) << 3));
    }
    floatx4 s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) s[kb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < KS; ++kc)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kb][kc], qf[kc], s[kb], 0, 0, 0);
    // V^T fragments of the tile, read now so the softmax below hides their latency: lane
    // supplies V^T[hd 16 n + fr] at keys 32 kk + 4 fq + r and 32 kk + 16 + 4 fq + r (slots
    // 4 fq .. 4 fq + 3 of pages 2 kk and 2 kk + 1), the key order of P^T below.
    bf16x8 vf[2][NO];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const uint16_t* va = vs_ + (2 * kk) * HD * 16 + fr * 16 + 4 * fq;
#pragma unroll
      for (int n = 0; n < NO; ++n) {
        // Read as bf16 vectors: typed this way the compiler does not order these reads behind
        // the tile loads still in flight (the explicit wait and barrier above already do).
        const bf16x4 lo = *(const bf16x4*)(va + n * 256);
        const bf16x4 hi = *(const bf16x4*)(va + HD * 16 + n * 256);
        vf[kk][n] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
    }
    // Causal mask (edge tiles only: a wave-uniform branch), online softmax in the exp2 domain
    // with the hardware exp2 (its flush of results below 2^-126 to zero is immaterial here).
    float mx = -INFINITY;
    if ((t + 1) * AP_KT > wmin) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool out = t * AP_KT + 16 * kb + 4 * fq + r >= lim;
          s[kb][r] = out ? -INFINITY : s[kb][r] * scale_log2;
          mx = fmaxf(mx, s[kb][r]);
        }
    } else {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          s[kb][r] *= scale_log2;
          mx = fmaxf(mx, s[kb][r]);
        }
    }
    mx = ap_rowmax(mx);
    // Tile 0 holds key 0, which every row attends, so mn is finite from there on.
    const float mn = fmaxf(m, mx);
    const float alpha = __builtin_amdgcn_exp2f(m - mn);
    m = mn;
    float ps = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = __builtin_amdgcn_exp2f(s[kb][r] - mn);
        ps += p;
        s[kb][r] = p;
      }
    lsum = lsum * alpha + ps;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int n = 0; n < NO; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[n][r] *= alpha;
    }
    // P^T operand of the 32-key step kk: this lane's keys 32 kk + 4 fq + r, then 32 kk + 16 +
    // 4 fq + r (any fixed order of the 8 keys works, as V^T above uses the same one).
    bf16x8 pf[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pf[kk][r] = (__bf16)s[2 * kk][r];
        pf[kk][4 + r] = (__bf16)s[2 * kk + 1][r];
      }
    // O^T += V^T P^T.
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int n = 0; n < NO; ++n)
        o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[kk][n], pf[kk], o[n], 0, 0, 0);
    // Scheduling hints: the K reads, the S MFMAs, then the V reads ahead of the softmax.
    __builtin_amdgcn_sched_group_barrier(0x100, 4 * KS, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 4 * KS, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 4 * NO, 0);
  }
  wait_vmcnt<0>();

  lsum = ap_rowsum(lsum);
  if (!row_ok) return;
  const float inv = 1.0f / lsum;
  uint16_t* orow = out + ((size_t)tk * hq + head) * HD + 4 * fq;
#pragma unroll
  for (int n = 0; n < NO; ++n) {
    const uint32_t lo = (uint32_t)f32_to_bf16(o[n][0] * inv) | ((uint32_t)f32_to_bf16(o[n][1] * inv) << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16(o[n][2] * inv) | ((uint32_t)f32_to_bf16(o[n][3] * inv) << 16);
    *(uint2*)(orow + 16 * n) = make_uint2(lo, hi);
  }
}

template <int HD, int G>
static hipError_t prefill_hg(int T, int hk, hipStream_t st, const void* q, const void* kp,
                             const void* vp, const int* positions, const int* bt, int max_pages,
                             int n_pages, int pos_limit, void* out, float sl2) {
  constexpr int NHW = G < 4 ? G : 4, TB = 4 / NHW;
  const size_t lds = (size_t)AP_ST * 2 * AP_KT * HD * sizeof(uint16_t);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)k_attn_prefill<HD, G>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  dim3 grid((T + 16 * TB - 1) / (16 * TB), hk * (G / NHW));
  hipLaunchKernelGGL((k_attn_prefill<HD, G>), grid, dim3(256), lds, st, (const uint16_t*)q,
                     (const uint16_t*)kp, (const uint16_t*)vp, positions, bt, max_pages, n_pages,
                     hk, T, pos_limit, (uint16_t*)out, sl2);
  return hipGetLastError();
}

bool attn_prefill_supported(int hd, int G, int ps) {
  return (hd == 64 || hd == 128) && (G == 1 || G == 2 || G == 4 || G == 8) && ps == 16;
}

hipError_t launch_attn_prefill(int hd, int G, int T, int hk, const void* q, const void* kp,
                               const void* vp, const int* positions, const int* bt,
                               int max_pages, int n_pages, int pos_limit, void* out,
                               hipStream_t st) {
  if (T <= 0) return hipSuccess;
  const float sl2 = 1.4426950408889634f / sqrtf((float)hd);
#define TPK_AP(HDV, GV) \
  return prefill_hg<HDV, GV>(T, hk, st, q, kp, vp, positions, bt, max_pages, n_pages, pos_limit, out, sl2)
  if (hd == 128) {
    switch (G) {
      case 1: TPK_AP(128, 1);
      case 2: TPK_AP(128, 2);
      case 4: TPK_AP(128, 4);
      case 8: TPK_AP(128, 8);
    }
  } else if (hd == 64) {
    switch (G) {
      case 1: TPK_AP(64, 1);
      case 2: TPK_AP(64, 2);
      case 4: TPK_AP(64, 4);
      case 8: TPK_AP(64, 8);
    }
  }
#undef TPK_AP
  return hipErrorInvalidValue;
}

}  // namespace tpk
