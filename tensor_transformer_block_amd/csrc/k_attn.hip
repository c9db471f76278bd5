// K8 (rotary embedding + paged KV append) and K5 (owned-head causal attention over the rank's
// paged KV cache, split along the keys, then merged).
//
// TensorSharp "How tensor parallelism works", step 2: attention runs per rank over only the heads
// that rank owns, against that rank's own KV cache. With grouped KV heads, query head h of the
// rank reads KV head h / (Hq/Hkv); Hkv divisible by N keeps each group inside one rank.
//
// Rotary embedding (Su et al., RoFormer), rotate-half form: the pair (x_i, x_{i+hd/2}) is rotated by
// position * base^(-2i/hd); cos/sin come from a host-computed table. The cache stores rotated K.
//
// Attention is split over the keys (flash-decoding): workgroup (split, kv head, token) scores its
// key range for the Hq/Hkv query heads of one group, so every key and value is read once per group,
// and keeps a running max / sum (the online softmax of Milakov & Gimelshein 2018). A second kernel
// merges the splits: o = sum_s o_s 2^(m_s - M) / sum_s l_s 2^(m_s - M).
#include "tp_common.h"
#include "tp_kernels.h"

namespace tpk {

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

template <int AT>
__global__ void k_rope_append(const void* __restrict__ qkv, int T, int hq, int hk, int hd,
                              void* __restrict__ q_out, const int* __restrict__ positions,
                              int mode, const int* __restrict__ block_table, int max_pages, int ps,
                              int n_pages, int pos_limit, void* __restrict__ kp,
                              void* __restrict__ vp, const float2* __restrict__ rope) {
  const int half = hd >> 1;
  const int heads = hq + 2 * hk;
  const int64_t total = (int64_t)T * heads * half;
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int e = (int)(i % half);
  const int head = (int)((i / half) % heads);
  const int t = (int)(i / ((int64_t)half * heads));
  const int pos = clampi(positions[t], 0, pos_limit - 1);
  const size_t src = (size_t)t * heads * hd + (size_t)head * hd;
  const float a = ld_act<AT>(qkv, src + e), b = ld_act<AT>(qkv, src + e + half);
  if (head < hq + hk) {
    const float2 cs = rope[(size_t)pos * half + e];
    const float ra = a * cs.x - b * cs.y, rb = b * cs.x + a * cs.y;
    if (head < hq) {
      const size_t dq = (size_t)t * hq * hd + (size_t)head * hd;
      st_act<AT>(q_out, dq + e, ra);
      st_act<AT>(q_out, dq + e + half, rb);
      return;
    }
  }
  const int seq = (mode == 0) ? t : 0;
  const int page = clampi(block_table[(size_t)seq * max_pages + pos / ps], 0, n_pages - 1);
  const int slot = pos % ps;
  if (head < hq + hk) {
    const float2 cs = rope[(size_t)pos * half + e];
    const int g = head - hq;
    const size_t dk = (((size_t)page * hk + g) * ps + slot) * hd;
    st_act<AT>(kp, dk + e, a * cs.x - b * cs.y);
    st_act<AT>(kp, dk + e + half, b * cs.x + a * cs.y);
  } else {
    const int g = head - hq - hk;
    const size_t dv = (((size_t)page * hk + g) * ps + slot) * hd;
    st_act<AT>(vp, dv + e, a);
    st_act<AT>(vp, dv + e + half, b);
  }
}

hipError_t launch_rope_append(int at, const void* qkv, int T, int hq, int hk, int hd, void* q_out,
                              const int* positions, int mode, const int* block_table,
                              int max_pages, int ps, int n_pages, int pos_limit, void* kp,
                              void* vp, const float* rope, hipStream_t st) {
  const int64_t total = (int64_t)T * (hq + 2 * hk) * (hd / 2);
  if (total == 0) return hipSuccess;
  dim3 g((unsigned)((total + 255) / 256)), b(256);
  if (at == ACT_F32)
    hipLaunchKernelGGL(k_rope_append<ACT_F32>, g, b, 0, st, qkv, T, hq, hk, hd, q_out, positions,
                       mode, block_table, max_pages, ps, n_pages, pos_limit, kp, vp,
                       (const float2*)rope);
  else
    hipLaunchKernelGGL(k_rope_append<ACT_BF16>, g, b, 0, st, qkv, T, hq, hk, hd, q_out, positions,
                       mode, block_table, max_pages, ps, n_pages, pos_limit, kp, vp,
                       (const float2*)rope);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Split-KV attention. Lane layout inside a wavefront: a key's HD elements are spread over
// LPK = HD / E lanes (E = elements per 16-byte load), so one wave-wide load covers KPP = 64 / LPK
// keys. Lanes with the same key form a "subgroup"; dot products reduce across its LPK lanes.
// The four waves of a workgroup take pages round-robin and merge through LDS at the end.
template <int AT, int HD, int G>
__global__ __launch_bounds__(256) void k_attn_split(
    const void* __restrict__ q, const void* __restrict__ kpages, const void* __restrict__ vpages,
    const int* __restrict__ positions, int mode, const int* __restrict__ block_table,
    int max_pages, int ps, int n_pages, int hk, int chunk, int n_split, int pos_limit,
    float* __restrict__ part_o, float* __restrict__ part_ml, float scale_log2) {
  constexpr int E = Vec16<AT>::N;
  constexpr int LPK = HD / E;
  constexpr int KPP = 64 / LPK;
  constexpr int EB = (AT == ACT_F32) ? 4 : 2;
  static_assert(LPK <= 64 && KPP >= 1, "head_dim too large for one wavefront");
  __shared__ float s_m[4][G], s_l[4][G];
  __shared__ float s_o[4][G][HD];

  const int split = blockIdx.x, g = blockIdx.y, t = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane / LPK, e0 = (lane % LPK) * E;
  const int hq = hk * G;
  const int pos = clampi(positions[t], 0, pos_limit - 1);
  const int n_keys = pos + 1;
  const int k0 = split * chunk;
  const int k1 = min(n_keys, k0 + chunk);
  const int seq = (mode == 0) ? t : 0;

  float qv[G][E];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    Vec16<AT>::load((const char*)q + ((size_t)t * hq * HD + (size_t)(g * G + h) * HD + e0) * EB,
                    qv[h]);
#pragma unroll
    for (int e = 0; e < E; ++e) qv[h][e] *= scale_log2;
  }
  float m[G], l[G], acc[G][E];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[h][e] = 0.f;
  }

  // Passes over one page, handled in groups of at most PG passes.
  const int passes = ps / KPP;
  constexpr int PG = 4;
  if (k0 < k1) {
    for (int pg = k0 / ps + wave; pg * ps < k1; pg += 4) {
      const int phys = clampi(block_table[(size_t)seq * max_pages + pg], 0, n_pages - 1);
      const char* kb = (const char*)kpages + (((size_t)phys * hk + g) * ps) * HD * EB;
      const char* vb = (const char*)vpages + (((size_t)phys * hk + g) * ps) * HD * EB;
      for (int p0 = 0; p0 < passes; p0 += PG) {
        float kf[PG][E], vf[PG][E];
        int key[PG];
#pragma unroll
        for (int j = 0; j < PG; ++j) {
          const int kin = (p0 + j) * KPP + sub;
          key[j] = pg * ps + kin;
          if (p0 + j < passes) {
            Vec16<AT>::load(kb + ((size_t)kin * HD + e0) * EB, kf[j]);
            Vec16<AT>::load(vb + ((size_t)kin * HD + e0) * EB, vf[j]);
          } else {
            key[j] = k1;  // no such pass: masked below
#pragma unroll
            for (int e = 0; e < E; ++e) kf[j][e] = vf[j][e] = 0.f;
          }
        }
        float s[PG][G];
#pragma unroll
        for (int j = 0; j < PG; ++j) {
#pragma unroll
          for (int h = 0; h < G; ++h) {
            float d = 0.f;
#pragma unroll
            for (int e = 0; e < E; ++e) d = fmaf(qv[h][e], kf[j][e], d);
#pragma unroll
            for (int o = LPK / 2; o > 0; o >>= 1) d += __shfl_xor(d, o, 64);
            s[j][h] = (key[j] >= k0 && key[j] < k1) ? d : -INFINITY;
          }
          // Slots past the sequence may hold anything (even NaN); keep them out of p * v.
          if (!(key[j] >= k0 && key[j] < k1)) {
#pragma unroll
            for (int e = 0; e < E; ++e) vf[j][e] = 0.f;
          }
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float mx = s[0][h];
#pragma unroll
          for (int j = 1; j < PG; ++j) mx = fmaxf(mx, s[j][h]);
#pragma unroll
          for (int o = LPK; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
          const float mn = fmaxf(m[h], mx);
          if (mn == -INFINITY) continue;  // nothing valid seen yet by this wave
          const float alpha = exp2f(m[h] - mn);
          m[h] = mn;
          l[h] *= alpha;
#pragma unroll
          for (int e = 0; e < E; ++e) acc[h][e] *= alpha;
#pragma unroll
          for (int j = 0; j < PG; ++j) {
            const float p = exp2f(s[j][h] - mn);
            l[h] += p;
#pragma unroll
            for (int e = 0; e < E; ++e) acc[h][e] = fmaf(p, vf[j][e], acc[h][e]);
          }
        }
      }
    }
  }
  // Sum the subgroups' partial l and o (they share m).
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int o = LPK; o < 64; o <<= 1) {
      l[h] += __shfl_xor(l[h], o, 64);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[h][e] += __shfl_xor(acc[h][e], o, 64);
    }
  }
  if (sub == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < E; ++e) s_o[wave][h][e0 + e] = acc[h][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      s_m[wave][h] = m[h];
      s_l[wave][h] = l[h];
    }
  }
  __syncthreads();
  for (int idx = tid; idx < G * HD; idx += 256) {
    const int h = idx / HD, e = idx % HD;
    float M = fmaxf(fmaxf(s_m[0][h], s_m[1][h]), fmaxf(s_m[2][h], s_m[3][h]));
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f = exp2f(s_m[w][h] - M);
        L += s_l[w][h] * f;
        O += s_o[w][h][e] * f;
      }
    }
    const size_t row = ((size_t)t * hq + g * G + h) * n_split + split;
    part_o[row * HD + e] = O;
    if (e == 0) {
      part_ml[row * 2] = M;
      part_ml[row * 2 + 1] = L;
    }
  }
}

template <int AT>
__global__ void k_attn_combine(const float* __restrict__ part_o, const float* __restrict__ part_ml,
                               int n_split, int hd, int hq, void* __restrict__ out) {
  const int t = blockIdx.x, h = blockIdx.y;
  const size_t row0 = ((size_t)t * hq + h) * n_split;
  float M = -INFINITY;
  for (int s = 0; s < n_split; ++s) M = fmaxf(M, part_ml[(row0 + s) * 2]);
  for (int e = threadIdx.x; e < hd; e += blockDim.x) {
    float L = 0.f, O = 0.f;
    for (int s = 0; s < n_split; ++s) {
      const float mv = part_ml[(row0 + s) * 2];
      if (mv == -INFINITY) continue;
      const float f = exp2f(mv - M);
      L += part_ml[(row0 + s) * 2 + 1] * f;
      O += part_o[(row0 + s) * hd + e] * f;
    }
    st_act<AT>(out, ((size_t)t * hq + h) * hd + e, O / L);
  }
}

template <int AT, int HD>
static hipError_t attn_g(int G, dim3 grid, hipStream_t st, const void* q, const void* kp,
                         const void* vp, const int* positions, int mode, const int* bt,
                         int max_pages, int ps, int n_pages, int hk, int chunk, int n_split,
                         int pos_limit, float* po, float* pml, float sl2) {
#define TPK_ATT(GV)                                                                           \
  hipLaunchKernelGGL((k_attn_split<AT, HD, GV>), grid, dim3(256), 0, st, q, kp, vp, positions, \
                     mode, bt, max_pages, ps, n_pages, hk, chunk, n_split, pos_limit, po, pml, sl2)
  switch (G) {
    case 1: TPK_ATT(1); break;
    case 2: TPK_ATT(2); break;
    case 4: TPK_ATT(4); break;
    case 8: TPK_ATT(8); break;
    default: return hipErrorInvalidValue;
  }
#undef TPK_ATT
  return hipGetLastError();
}

hipError_t launch_attn_decode(int at, int hd, int G, int T, int hk, const void* q, const void* kp,
                              const void* vp, const int* positions, int mode, const int* bt,
                              int max_pages, int ps, int n_pages, int chunk, int n_split,
                              int pos_limit, float* part_o, float* part_ml, void* out,
                              hipStream_t st) {
  if (T == 0) return hipSuccess;
  const float sl2 = 1.4426950408889634f / sqrtf((float)hd);
  dim3 grid(n_split, hk, T);
  hipError_t e;
#define TPK_HD(ATV, HDV)                                                                        \
  e = attn_g<ATV, HDV>(G, grid, st, q, kp, vp, positions, mode, bt, max_pages, ps, n_pages, hk, \
                       chunk, n_split, pos_limit, part_o, part_ml, sl2)
  if (at == ACT_F32) {
    if (hd == 64) TPK_HD(ACT_F32, 64);
    else if (hd == 128) TPK_HD(ACT_F32, 128);
    else if (hd == 256) TPK_HD(ACT_F32, 256);
    else return hipErrorInvalidValue;
  } else {
    if (hd == 64) TPK_HD(ACT_BF16, 64);
    else if (hd == 128) TPK_HD(ACT_BF16, 128);
    else if (hd == 256) TPK_HD(ACT_BF16, 256);
    else return hipErrorInvalidValue;
  }
#undef TPK_HD
  if (e != hipSuccess) return e;
  const int hq = hk * G;
  dim3 cg(T, hq), cb(hd < 256 ? hd : 256);
  if (at == ACT_F32)
    hipLaunchKernelGGL(k_attn_combine<ACT_F32>, cg, cb, 0, st, part_o, part_ml, n_split, hd, hq, out);
  else
    hipLaunchKernelGGL(k_attn_combine<ACT_BF16>, cg, cb, 0, st, part_o, part_ml, n_split, hd, hq, out);
  return hipGetLastError();
}

}  // namespace tpk
