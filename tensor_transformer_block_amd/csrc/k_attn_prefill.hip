// Causal prefill attention for one rank's heads, bf16, MFMA, with the KV tiles shared by all the
// query heads of a GQA group (TensorSharp "Multi-GPU & Multi-Node", section "How tensor
// parallelism works": every rank attends with its own heads against its own KV cache).
//
// A workgroup takes four 16-row blocks of one KV head (16 tokens of four query heads, or more
// tokens of fewer heads when the group is smaller) and splits their keys over four key groups of
// two waves: super-tile j (128 keys, eight 16-token pages) gives group kg the 32 keys 128 j + 32 kg,
// so the long causal rows are spread over all eight waves (two per SIMD, one hiding the other's
// softmax) and the groups' partial softmax states are merged through LDS at the end. Each wave
// computes two of the row blocks against its keys with the same K and V fragments, which halves
// the LDS reads per MFMA. The super-tiles come into a double-buffered LDS ring by direct-to-LDS
// loads (K rows with their 16-byte chunks XOR-swizzled by key, V as stored: transposed per page),
// so the K/V bytes leave L2 once per workgroup. Scores and output are computed transposed,
// S^T = K Q^T and O^T += V^T P^T (16x16x32 MFMA): each lane then owns one query row of each of
// its two row blocks, a row's online softmax (exp2 domain, causal mask on edge tiles only) needs
// two cross-lane steps, and P goes from the score registers straight into the next MFMA.
#include "k_gemm_common.h"
#include "tp_kernels.h"

namespace tpk {

typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;

constexpr int AP_SUB = 32;  // keys per key group per step (two 16-token pages)
constexpr int AP_KG = 4;    // key groups per workgroup (two waves each)

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
__global__ __launch_bounds__(512) void k_attn_prefill(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kpages,
    const uint16_t* __restrict__ vpages, const int* __restrict__ positions,
    const int* __restrict__ block_table, int max_pages, int n_pages, int hk, int T, int pos_limit,
    uint16_t* __restrict__ out, float scale_log2) {
  constexpr int KS = HD / 32;               // k-steps over hd in Q K^T
  constexpr int NO = HD / 16;               // hd blocks of O
  constexpr int NHW = G < 4 ? G : 4;        // query heads per workgroup
  constexpr int TB = 4 / NHW;               // 16-token blocks per workgroup
  constexpr int CH = HD / 8;                // 16-byte chunks per key row of K
  constexpr int SUBE = AP_SUB * HD;         // bf16 elements of a group's K (or V) sub-tile
  constexpr int SLOT = AP_KG * 2 * SUBE;    // bf16 elements of one super-tile (K and V)
  constexpr int KPL = 1024 / (HD * 2);      // keys per K wave-load (1 KB)
  constexpr int PWL = HD * 32 / 1024;       // wave-loads per 16-key page of K (and of V)
  constexpr int NPG = NO / AP_KG;           // hd blocks of O each key group writes out
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  __shared__ float2 s_ml[AP_KG][2][2][64];  // merge: (m, l) per key group, wave, row block, lane
  __shared__ int s_kmax;

  const int g = blockIdx.y / (G / NHW), hgrp = blockIdx.y % (G / NHW);
  const int t0 = (gridDim.x - 1 - blockIdx.x) * (16 * TB);  // latest tokens first
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = wave >> 1, wp = wave & 1;  // key group, wave within the group
  const int fr = lane & 15, fq = lane >> 4;
  const int hq = hk * G;

  // Keys this workgroup needs: up to the largest position among its tokens.
  if (tid == 0) s_kmax = 0;
  __syncthreads();
  if (tid < 16 * TB && t0 + tid < T)
    atomicMax(&s_kmax, ap_clamp(positions[t0 + tid], 0, pos_limit - 1) + 1);
  __syncthreads();
  const int nsup = (s_kmax + 4 * AP_SUB - 1) / (4 * AP_SUB);

  // The wave's row blocks rb = 2 wp + h (h = 0, 1): token block rb / NHW, head rb % NHW of the
  // workgroup's heads. Lane l works on row (token) l % 16 of both throughout: S and O are kept
  // transposed (keys or hd along the MFMA rows), so the softmax of a row lives in the four lanes
  // l % 16 + 16 i and P feeds the P V product straight from registers.
  int tk[2], head[2], lim[2];
  bf16x8 qf[2][KS];  // Q^T operands: lane row fr, hd chunk fq of each 32-wide step
  int wmin = 0x7fffffff, wmax = 0;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int rb = 2 * wp + h;
    tk[h] = t0 + (rb / NHW) * 16 + fr;
    head[h] = g * G + hgrp * NHW + rb % NHW;
    const bool ok = tk[h] < T;
    lim[h] = ok ? ap_clamp(positions[tk[h]], 0, pos_limit - 1) + 1 : 1;
    if (ok) wmin = min(wmin, lim[h]);
    wmax = max(wmax, lim[h]);
    const uint16_t* qrow = q + ((size_t)(ok ? tk[h] : 0) * hq + head[h]) * HD + fq * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[h][ks] = ok ? *(const bf16x8*)(qrow + ks * 32) : bf16x8{};
  }
  // Sub-tiles ending at or below every row's limit need no causal mask; those starting at or
  // past every row's limit need no work.
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    wmin = min(wmin, __shfl_xor(wmin, off, 64));
    wmax = max(wmax, __shfl_xor(wmax, off, 64));
  }

  // Super-tile j in LDS slot j % 2: group kg's K sub-tile [32 keys][HD] at (2 kg) SUBE, its V
  // sub-tile [2 pages][HD][16] at (2 kg + 1) SUBE. Wave wp of group kg loads page 2 kg + wp of
  // the super-tile (K rows 16 wp .. 16 wp + 15 and V page wp of the group's sub-tile). The page
  // ids of the next super-tile are read a step ahead into a register (lane i: page 8 j + i % 8).
  auto page_ids = [&](int j) {
    return block_table[min(8 * j + (lane & 7), max_pages - 1)];
  };
  auto issue = [&](int slot, int ptab) {
    const int pid = ap_clamp(__builtin_amdgcn_readlane(ptab, 2 * kg + wp), 0, n_pages - 1);
    uint16_t* ks_ = smem + slot * SLOT + 2 * kg * SUBE + 16 * wp * HD;
    uint16_t* vs_ = smem + slot * SLOT + (2 * kg + 1) * SUBE + wp * HD * 16;
    const uint16_t* kpg = kpages + ((size_t)pid * hk + g) * 16 * HD;
    const uint16_t* vpg = vpages + ((size_t)pid * hk + g) * HD * 16;
#pragma unroll
    for (int i = 0; i < PWL; ++i) {
      // K: keys KPL i .. of the page; lane -> key KPL i + l / CH, LDS chunk l % CH holding
      // global chunk (l % CH) ^ (key % CH).
      const int key = KPL * i + lane / CH, pos = lane % CH;
      __builtin_amdgcn_global_load_lds(
          (glb_void_t*)(kpg + key * HD + ((pos ^ ((16 * wp + key) & (CH - 1))) << 3)),
          (lds_void_t*)(ks_ + i * 512), 16, 0, 0);
      // V: 32 hd rows of the page per wave-load, as stored ([hd][16 keys]).
      __builtin_amdgcn_global_load_lds(
          (glb_void_t*)(vpg + (i * 32 + lane / 2) * 16 + (lane & 1) * 8),
          (lds_void_t*)(vs_ + i * 512), 16, 0, 0);
    }
  };

  float m[2] = {-INFINITY, -INFINITY}, lsum[2] = {0.f, 0.f};
  floatx4 o[2][NO];  // O^T: lane holds O[row fr of block h][hd 16 n + 4 fq + r]
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int n = 0; n < NO; ++n) o[h][n] = floatx4{0.f, 0.f, 0.f, 0.f};

  int ptab = 0;
  if (nsup > 0) {
    issue(0, page_ids(0));
    ptab = page_ids(1);
  }
  for (int j = 0; j < nsup; ++j) {
    // Super-tile j has landed for every wave, and every wave is done with super-tile j - 1,
    // whose slot then takes super-tile j + 1.
    wait_vmcnt<0>();
    __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (j + 1 < nsup) {
      issue((j + 1) & 1, ptab);
      ptab = page_ids(j + 2);
    }
    const int kb0 = (4 * j + kg) * AP_SUB;  // first key of this group's sub-tile
    if (kb0 >= wmax) continue;
    const uint16_t* ks_ = smem + (j & 1) * SLOT + 2 * kg * SUBE;
    const uint16_t* vs_ = ks_ + SUBE;

    // S^T = K Q^T per 16-key block kb and row block h: lane holds S[row fr][key 16 kb + 4 fq + r].
    bf16x8 kf[2][KS];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = 16 * kb + fr;
#pragma unroll
      for (int kc = 0; kc < KS; ++kc)
        kf[kb][kc] = *(const bf16x8*)(ks_ + key * HD + (((kc * 4 + fq) ^ (key & (CH - 1))) << 3));
    }
    floatx4 s[2][2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) s[h][kb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < KS; ++kc)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          s[h][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kb][kc], qf[h][kc], s[h][kb], 0, 0, 0);
    // V^T fragments, read now so the softmax below hides their latency: lane supplies V^T[hd
    // 16 n + fr] at keys 4 fq + r and 16 + 4 fq + r (slots 4 fq .. 4 fq + 3 of the two pages),
    // the key order of P^T below.
    bf16x8 vf[NO];
#pragma unroll
    for (int n = 0; n < NO; ++n) {
      // Read as bf16 vectors: typed this way the compiler does not order these reads behind
      // the tile loads still in flight (the explicit wait and barrier above already do).
      const bf16x4 lo = *(const bf16x4*)(vs_ + (16 * n + fr) * 16 + 4 * fq);
      const bf16x4 hi = *(const bf16x4*)(vs_ + (HD + 16 * n + fr) * 16 + 4 * fq);
      vf[n] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    // Causal mask (edge sub-tiles only: a wave-uniform branch), online softmax in the exp2
    // domain with the hardware exp2 (its flush of results below 2^-126 to zero is immaterial
    // here). A row whose keys so far are all masked keeps m = -inf and contributes nothing.
    const bool edge = kb0 + AP_SUB > wmin;
    bf16x8 pf[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (edge) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (kb0 + 16 * kb + 4 * fq + r >= lim[h]) s[h][kb][r] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[h][kb][r]);
      const float mn = fmaxf(m[h], ap_rowmax(mx) * scale_log2);
      const float mref = mn == -INFINITY ? 0.f : mn;
      const float alpha = __builtin_amdgcn_exp2f(m[h] - mref);
      m[h] = mn;
      float ps = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[h][kb][r], scale_log2, -mref));
          ps += p;
          pf[h][4 * kb + r] = (__bf16)p;
        }
      lsum[h] = lsum[h] * alpha + ps;
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int n = 0; n < NO; ++n)
#pragma unroll
          for (int r = 0; r < 4; ++r) o[h][n][r] *= alpha;
      }
    }
    // O^T += V^T P^T.
#pragma unroll
    for (int n = 0; n < NO; ++n)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        o[h][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[n], pf[h], o[h][n], 0, 0, 0);
  }

  // Merge the four key groups' states (m, l, O) of each row: every group publishes its state,
  // then group kg combines hd blocks NPG kg .. NPG kg + NPG - 1 of all four and writes them out.
  // The tile ring is free once every wave has passed the barrier (nothing is in flight).
  wait_vmcnt<0>();
  float* mo = (float*)smem;  // [kg][wp][h][n][lane][4]
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    lsum[h] = ap_rowsum(lsum[h]);
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    s_ml[kg][wp][h][lane] = make_float2(m[h], lsum[h]);
#pragma unroll
    for (int n = 0; n < NO; ++n)
      if (n / NPG != kg)
        *(floatx4*)(mo + ((((kg * 2 + wp) * 2 + h) * NO + n) * 64 + lane) * 4) = o[h][n];
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (tk[h] >= T) continue;
    float mk[AP_KG], M = -INFINITY;
#pragma unroll
    for (int c = 0; c < AP_KG; ++c) {
      mk[c] = s_ml[c][wp][h][lane].x;
      M = fmaxf(M, mk[c]);
    }
    float w[AP_KG], L = 0.f;
#pragma unroll
    for (int c = 0; c < AP_KG; ++c) {
      w[c] = __builtin_amdgcn_exp2f(mk[c] - M);
      L += w[c] * s_ml[c][wp][h][lane].y;
    }
    const float inv = 1.0f / L;
    uint16_t* orow = out + ((size_t)tk[h] * hq + head[h]) * HD + 4 * fq;
#pragma unroll
    for (int n = 0; n < NO; ++n) {
      if (n / NPG != kg) continue;  // wave-uniform; keeps o[][] statically indexed
      floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < AP_KG; ++c) {
        const floatx4 oc = c == kg ? o[h][n]
                                   : *(const floatx4*)(mo + ((((c * 2 + wp) * 2 + h) * NO + n) * 64 + lane) * 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] += w[c] * oc[r];
      }
      const uint32_t lo = (uint32_t)f32_to_bf16(acc[0] * inv) | ((uint32_t)f32_to_bf16(acc[1] * inv) << 16);
      const uint32_t hi = (uint32_t)f32_to_bf16(acc[2] * inv) | ((uint32_t)f32_to_bf16(acc[3] * inv) << 16);
      *(uint2*)(orow + 16 * n) = make_uint2(lo, hi);
    }
  }
}

template <int HD, int G>
static hipError_t prefill_hg(int T, int hk, hipStream_t st, const void* q, const void* kp,
                             const void* vp, const int* positions, const int* bt, int max_pages,
                             int n_pages, int pos_limit, void* out, float sl2) {
  constexpr int NHW = G < 4 ? G : 4, TB = 4 / NHW;
  // Two super-tile slots; the merge at the end reuses the same bytes.
  const size_t lds = (size_t)2 * AP_KG * 2 * AP_SUB * HD * sizeof(uint16_t);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)k_attn_prefill<HD, G>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  dim3 grid((T + 16 * TB - 1) / (16 * TB), hk * (G / NHW));
  hipLaunchKernelGGL((k_attn_prefill<HD, G>), grid, dim3(512), lds, st, (const uint16_t*)q,
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
