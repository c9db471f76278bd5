// Causal prefill attention for one rank's heads, bf16, MFMA, with the KV tiles shared by all the
// query heads of a GQA group (TensorSharp "Multi-GPU & Multi-Node", section "How tensor
// parallelism works": every rank attends with its own heads against its own KV cache).
//
// A workgroup takes four 16-row blocks of one KV head (16 tokens of four query heads, or more
// tokens of fewer heads when the group is smaller) and splits their keys over four key groups of
// two waves: super-tile j (128 keys, eight 16-token pages) gives group kg the 32 keys 128 j + 32 kg,
// so the long causal rows are spread over all eight waves (two per SIMD) and the groups' partial
// softmax states are merged through LDS at the end. Each wave computes two of the row blocks
// against its keys with the same K and V fragments, which halves the LDS reads per MFMA.
//
// Scores and output are computed transposed, S^T = K Q^T and O^T += V^T P^T (16x16x32 MFMA):
// each lane then owns one query row of each of its two row blocks, a row's online softmax needs
// two cross-lane steps, and P goes from the score registers straight into the next MFMA. The
// MFMA rows of K are permuted so that a lane's eight scores are eight consecutive keys, which
// makes its V^T operand one 16-byte LDS read of the page as stored. The scores of the group's
// next sub-tile are computed while the softmax of the current one runs (the matrix cores and
// the vector ALUs work side by side), so K and V live one super-tile apart in two rings: K of
// super-tiles j + 1 and j + 2, V of j and j + 1, each loaded by direct-to-LDS transfers with its
// 16-byte chunks XOR-swizzled against LDS bank conflicts.
#include "k_gemm_common.h"
#include "tp_kernels.h"

namespace tpk {

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

// K row swizzle: the 16-byte chunk c of sub-tile key `key` sits at chunk c ^ ap_kswz(key). The
// eight keys one 16-lane K fragment read takes per bank window (keys 8 a + 4 kb + b, b < 4, two
// consecutive a) then hit eight different chunk positions.
template <int CH>
__device__ __forceinline__ int ap_kswz(int key) {
  return ((key & 3) | ((key >> 1) & 12)) & (CH - 1);
}

template <int HD, int G>
__global__ __launch_bounds__(512) void k_attn_prefill(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kpages,
    const uint16_t* __restrict__ vpages, const int* __restrict__ positions,
    const int* __restrict__ block_table, int max_pages, int n_pages, int hk, int T, int pos_limit,
    uint16_t* __restrict__ out, float scale_log2, AttnRanks ar) {
  constexpr int KS = HD / 32;               // k-steps over hd in Q K^T
  constexpr int NO = HD / 16;               // hd blocks of O
  constexpr int NHW = G < 4 ? G : 4;        // query heads per workgroup
  constexpr int TB = 4 / NHW;               // 16-token blocks per workgroup
  constexpr int CH = HD / 8;                // 16-byte chunks per key row of K
  constexpr int SUBE = AP_SUB * HD;         // bf16 elements of a group's K (or V) sub-tile
  constexpr int KPL = 1024 / (HD * 2);      // keys per K wave-load (1 KB)
  constexpr int PWL = HD * 32 / 1024;       // wave-loads per 16-key page of K (and of V)
  constexpr int NPG = NO / AP_KG;           // hd blocks of O each key group writes out
  constexpr float TAU = 8.f;                // lazy running max: scores reach at most 2^TAU
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  __shared__ float2 s_ml[AP_KG][2][2][64];  // merge: (m, l) per key group, wave, row block, lane
  __shared__ int s_kmax;
  // Every rank in one launch: consecutive workgroups, which the dispatcher deals round-robin to
  // the XCDs, take consecutive ranks, so each XCD's L2 holds the KV of few ranks; the longest
  // token tiles of every rank still go first.
  int bx = blockIdx.x, by = blockIdx.y;
  if (ar.n > 1) {
    const int lin = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    const int r = lin % ar.n, rest = lin / ar.n;
    by = rest % gridDim.y;
    bx = rest / gridDim.y;
    q = (const uint16_t*)ar.q[r];
    kpages = (const uint16_t*)ar.k_pages[r];
    vpages = (const uint16_t*)ar.v_pages[r];
    n_pages = ar.n_pages[r];
    out = (uint16_t*)ar.out[r];
  }

  const int g = by / (G / NHW), hgrp = by % (G / NHW);
  const int t0 = (gridDim.x - 1 - bx) * (16 * TB);  // latest tokens first
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
  const int kmax = s_kmax;  // keys below this were written (prior cache or this step)
  const int nsup = (kmax + 4 * AP_SUB - 1) / (4 * AP_SUB);

  // The wave's row blocks rb = 2 wp + h (h = 0, 1): token block rb / NHW, head rb % NHW of the
  // workgroup's heads. Lane l works on row (token) l % 16 of both throughout.
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

  // LDS: K ring [2][AP_KG][32 keys][HD] (swizzled rows), V ring [2][AP_KG][2 pages][HD][16].
  // Wave wp of group kg loads page 2 kg + wp of a super-tile: K keys 16 wp .. 16 wp + 15 and V
  // page wp of the group's sub-tile. Page ids are read ahead into a register (lane i: page
  // 8 j + i % 8 of super-tile j) and picked out with a lane read.
  uint16_t* const kring = smem;
  uint16_t* const vring = smem + 2 * AP_KG * SUBE;
  auto page_ids = [&](int j) { return block_table[min(8 * j + (lane & 7), max_pages - 1)]; };
  auto page_of = [&](int ptab) {
    const int pid = ap_clamp(__builtin_amdgcn_readlane(ptab, 2 * kg + wp), 0, n_pages - 1);
    return (size_t)pid * hk + g;
  };
  auto issue_k = [&](int slot, int ptab) {
    const uint16_t* kpg = kpages + page_of(ptab) * 16 * HD;
    uint16_t* dst = kring + (slot * AP_KG + kg) * SUBE + 16 * wp * HD;
#pragma unroll
    for (int i = 0; i < PWL; ++i) {
      const int key = KPL * i + lane / CH, pos = lane % CH;  // key of the page; LDS chunk pos
      __builtin_amdgcn_global_load_lds(
          (glb_void_t*)(kpg + key * HD + ((pos ^ ap_kswz<CH>(16 * wp + key)) << 3)),
          (lds_void_t*)(dst + i * 512), 16, 0, 0);
    }
  };
  auto issue_v = [&](int slot, int ptab) {
    const uint16_t* vpg = vpages + page_of(ptab) * HD * 16;
    uint16_t* dst = vring + (slot * AP_KG + kg) * SUBE + wp * HD * 16;
#pragma unroll
    for (int i = 0; i < PWL; ++i) {
      // 32 hd rows as stored ([hd][16 keys]); the two 16-byte halves of a row swap places on
      // rows with bit 2 set.
      const int row = i * 32 + lane / 2, half = (lane & 1) ^ ((row >> 2) & 1);
      __builtin_amdgcn_global_load_lds((glb_void_t*)(vpg + row * 16 + half * 8),
                                       (lds_void_t*)(dst + i * 512), 16, 0, 0);
    }
  };
  // S^T = K Q^T of the sub-tile in K slot `slot`, per 16-key block kb and row block h. MFMA row
  // 4 a + b of block kb takes key 8 a + 4 kb + b, so lane (fr, fq) ends up holding
  // S[row fr][key 8 fq + 4 kb + r].
  auto scores = [&](int slot, floatx4 (&sc)[2][2]) {
    const uint16_t* ks_ = kring + (slot * AP_KG + kg) * SUBE;
    bf16x8 kf[2][KS];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = 8 * (fr >> 2) + 4 * kb + (fr & 3);
#pragma unroll
      for (int kc = 0; kc < KS; ++kc)
        kf[kb][kc] = *(const bf16x8*)(ks_ + key * HD + (((kc * 4 + fq) ^ ap_kswz<CH>(key)) << 3));
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) sc[h][kb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < KS; ++kc)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          sc[h][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kb][kc], qf[h][kc], sc[h][kb], 0, 0, 0);
  };

  float m[2] = {-INFINITY, -INFINITY}, lsum[2] = {0.f, 0.f};
  floatx4 o[2][NO];  // O^T: lane holds O[row fr of block h][hd 16 n + 4 fq + r]
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int n = 0; n < NO; ++n) o[h][n] = floatx4{0.f, 0.f, 0.f, 0.f};
  float mref[2];
  bf16x8 pf[2];
  // Online softmax of one sub-tile's scores in the exp2 domain, in two phases so that the rare
  // O rescale (a branch) sits between them and the exponentials share one basic block with the
  // MFMAs. The running max only moves when a tile's max exceeds it by more than TAU; a row whose
  // keys so far are all masked keeps m = -inf and contributes nothing.
  auto new_max = [&](floatx4 (&sc)[2][2]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[h][kb][r]);
      mx = ap_rowmax(mx) * scale_log2;
      const float mn = mx > m[h] + TAU ? mx : m[h];
      mref[h] = mn == -INFINITY ? 0.f : mn;
      const float alpha = __builtin_amdgcn_exp2f(m[h] - mref[h]);
      m[h] = mn;
      lsum[h] *= alpha;
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int n = 0; n < NO; ++n)
#pragma unroll
          for (int r = 0; r < 4; ++r) o[h][n][r] *= alpha;
      }
    }
  };
  // P = exp2(s scale - m) with the hardware exp2 (its flush of results below 2^-126 to zero is
  // immaterial here), packed to bf16 as the B operand of the P V step.
  auto exps = [&](floatx4 (&sc)[2][2]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float ps = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[h][kb][r], scale_log2, -mref[h]));
          ps += p;
          pf[h][4 * kb + r] = (__bf16)p;
        }
      lsum[h] += ps;
    }
  };
  // V^T of the sub-tile in V slot `slot` (lane: hd row 16 n + fr, keys kb0 + 8 fq .. kb0 + 8 fq
  // + 7, one 16-byte read), then O^T += V^T P^T. Keys at or past kmax have P = 0, but their slots
  // may never have been written and hold a NaN or an Inf (0 times either is a NaN), so the
  // sub-tile that crosses kmax clears their V elements first. (`edge` is a constant at each call:
  // the overlapped branch below only runs sub-tiles that end below every row's limit.)
  auto accumulate = [&](int slot, int kb0, bool edge) {
    const uint16_t* vs_ = vring + (slot * AP_KG + kg) * SUBE + (fq >> 1) * HD * 16;
    bf16x8 vf[NO];
#pragma unroll
    for (int n = 0; n < NO; ++n)
      vf[n] = *(const bf16x8*)(vs_ + (16 * n + fr) * 16 + (((fq & 1) ^ ((fr >> 2) & 1)) << 3));
    if (edge && kb0 + AP_SUB > kmax) {
      const uint4 keep = v_keep_mask(kmax - (kb0 + 8 * fq));
#pragma unroll
      for (int n = 0; n < NO; ++n) {
        uint4 u = __builtin_bit_cast(uint4, vf[n]);
        u.x &= keep.x;
        u.y &= keep.y;
        u.z &= keep.z;
        u.w &= keep.w;
        vf[n] = __builtin_bit_cast(bf16x8, u);
      }
    }
#pragma unroll
    for (int n = 0; n < NO; ++n)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        o[h][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[n], pf[h], o[h][n], 0, 0, 0);
  };
  // Causal mask of the scores of the sub-tile starting at key kb0 (edge sub-tiles only).
  auto mask = [&](floatx4 (&sc)[2][2], int kb0) {
    if (kb0 + AP_SUB > wmin) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (kb0 + 8 * fq + 4 * kb + r >= lim[h]) sc[h][kb][r] = -INFINITY;
    }
  };

  floatx4 scur[2][2], snxt[2][2];
  int pb = 0, pc = 0;  // page ids of super-tiles j + 1 and j + 2
  if (nsup > 0) {
    const int pa = page_ids(0);
    issue_k(0, pa);
    issue_v(0, pa);
    pb = page_ids(1);
    if (nsup > 1) issue_k(1, pb);
    pc = page_ids(2);
    wait_vmcnt<0>();
    __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    scores(0, scur);
  }
  for (int j = 0; j < nsup; ++j) {
    // K of super-tile j + 1 and V of j have landed for every wave, and every wave is done with
    // K of j and V of j - 1, whose slots then take K of j + 2 and V of j + 1.
    wait_vmcnt<0>();
    __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (j + 2 < nsup) issue_k(j & 1, pc);
    if (j + 1 < nsup) issue_v((j + 1) & 1, pb);
    pb = pc;
    pc = page_ids(j + 3);
    const int kb0 = (4 * j + kg) * AP_SUB;  // first key of this group's current sub-tile
    if (kb0 >= wmax) continue;
    mask(scur, kb0);
    new_max(scur);
    if (j + 1 < nsup && kb0 + 4 * AP_SUB < wmax) {
      // Scores of the next sub-tile on the matrix cores while the exponentials run on the VALUs.
      scores((j + 1) & 1, snxt);
      exps(scur);
      accumulate(j & 1, kb0, false);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) scur[h][kb] = snxt[h][kb];
      // Scheduling hints: the K reads, then each score MFMA followed by a few VALU operations
      // of the exponentials, then the V reads and the P V MFMAs.
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * KS, 0);
#pragma unroll
      for (int i = 0; i < 4 * KS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, NO, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * NO, 0);
    } else {
      exps(scur);
      accumulate(j & 1, kb0, true);
    }
  }

  // Merge the four key groups' states (m, l, O) of each row: every group publishes its state,
  // then group kg combines hd blocks NPG kg .. NPG kg + NPG - 1 of all four and writes them out.
  // The rings are free once every wave has passed the barrier (nothing is in flight).
  wait_vmcnt<0>();
  float* mo = (float*)smem;  // [kg][wp][h][n][lane][4]
#pragma unroll
  for (int h = 0; h < 2; ++h) lsum[h] = ap_rowsum(lsum[h]);
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
                             int n_pages, int pos_limit, void* out, float sl2,
                             const AttnRanks& ar) {
  constexpr int NHW = G < 4 ? G : 4, TB = 4 / NHW;
  // Two super-tile slots; the merge at the end reuses the same bytes.
  const size_t lds = (size_t)2 * AP_KG * 2 * AP_SUB * HD * sizeof(uint16_t);
  hipError_t e = allow_lds((const void*)k_attn_prefill<HD, G>, (int)lds);
  if (e != hipSuccess) return e;
  dim3 grid((T + 16 * TB - 1) / (16 * TB), hk * (G / NHW), ar.n > 1 ? ar.n : 1);
  hipLaunchKernelGGL((k_attn_prefill<HD, G>), grid, dim3(512), lds, st, (const uint16_t*)q,
                     (const uint16_t*)kp, (const uint16_t*)vp, positions, bt, max_pages, n_pages,
                     hk, T, pos_limit, (uint16_t*)out, sl2, ar);
  return hipGetLastError();
}

bool attn_prefill_supported(int hd, int G, int ps) {
  return (hd == 64 || hd == 128) && (G == 1 || G == 2 || G == 4 || G == 8) && ps == 16;
}

hipError_t launch_attn_prefill(int hd, int G, int T, int hk, const void* q, const void* kp,
                               const void* vp, const int* positions, const int* bt,
                               int max_pages, int n_pages, int pos_limit, void* out,
                               hipStream_t st, const AttnRanks* ar) {
  if (T <= 0) return hipSuccess;
  const AttnRanks one{};
  if (ar) {
    if (ar->n < 1 || ar->n > kMaxRanks) return hipErrorInvalidValue;
    for (int r = 0; r < ar->n; ++r)
      if (!ar->q[r] || !ar->k_pages[r] || !ar->v_pages[r] || !ar->out[r] || ar->n_pages[r] < 1)
        return hipErrorInvalidValue;
    q = ar->q[0];
    kp = ar->k_pages[0];
    vp = ar->v_pages[0];
    n_pages = ar->n_pages[0];
    out = ar->out[0];
  }
  const AttnRanks& arr = ar ? *ar : one;
  const float sl2 = 1.4426950408889634f / sqrtf((float)hd);
#define TPK_AP(HDV, GV) \
  return prefill_hg<HDV, GV>(T, hk, st, q, kp, vp, positions, bt, max_pages, n_pages, pos_limit, out, sl2, arr)
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
