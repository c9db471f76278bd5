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
    // V pages are stored transposed: [page][kv head][hd][slot].
    const int g = head - hq - hk;
    const size_t dv = ((size_t)page * hk + g) * hd;
    st_act<AT>(vp, (dv + e) * ps + slot, a);
    st_act<AT>(vp, (dv + e + half) * ps + slot, b);
  }
}

// The same rotary embedding + KV append from NP fp32 partial products of the QKV projection
// (a split-K GEMM's K ranges, [NP][T][heads * hd]): the partials are summed in range order and
// rounded once to bf16, the value the unsplit projection would have stored, then rotated.
// Workgroup: one token (blockIdx.x) of one rank (blockIdx.y); its position and KV page are read
// once, and the threads walk the token's heads in groups of four rotation pairs.
template <int NP>
__global__ void k_rope_append_parts(const float* __restrict__ parts, int T, int hq, int hk, int hd,
                                    uint16_t* __restrict__ q_out,
                                    const int* __restrict__ positions, int mode,
                                    const int* __restrict__ block_table, int max_pages, int ps,
                                    int n_pages, int pos_limit, uint16_t* __restrict__ kp,
                                    uint16_t* __restrict__ vp, const float2* __restrict__ rope,
                                    RopeRanks rr) {
  if (rr.n > 1) {  // every rank in one launch (blockIdx.y = rank)
    const int r = blockIdx.y;
    parts = rr.parts[r];
    q_out = (uint16_t*)rr.q_out[r];
    kp = (uint16_t*)rr.k_pages[r];
    vp = (uint16_t*)rr.v_pages[r];
    n_pages = rr.n_pages[r];
  }
  const int t = blockIdx.x;
  const int half = hd >> 1, q4 = half >> 2;
  const int heads = hq + 2 * hk;
  const int pos = clampi(positions[t], 0, pos_limit - 1);
  const int seq = (mode == 0) ? t : 0;
  const int page = clampi(block_table[(size_t)seq * max_pages + pos / ps], 0, n_pages - 1);
  const size_t pstride = (size_t)T * heads * hd;
  // Thread j: four consecutive rotation pairs (e .. e + 3 with e + half .. e + half + 3) of one
  // head, so every partial read and every q / k store is a 16- or 8-byte access.
  for (int j = threadIdx.x; j < heads * q4; j += blockDim.x) {
    const int head = j / q4, e = (j - head * q4) * 4;
    const size_t src = ((size_t)t * heads + head) * hd;
    float4 sa = *(const float4*)(parts + src + e), sb = *(const float4*)(parts + src + e + half);
#pragma unroll
    for (int p = 1; p < NP; ++p) {
      const float4 xa = *(const float4*)(parts + p * pstride + src + e);
      const float4 xb = *(const float4*)(parts + p * pstride + src + e + half);
      sa.x += xa.x; sa.y += xa.y; sa.z += xa.z; sa.w += xa.w;
      sb.x += xb.x; sb.y += xb.y; sb.z += xb.z; sb.w += xb.w;
    }
    const uint16_t ua[4] = {f32_to_bf16(sa.x), f32_to_bf16(sa.y), f32_to_bf16(sa.z), f32_to_bf16(sa.w)};
    const uint16_t ub[4] = {f32_to_bf16(sb.x), f32_to_bf16(sb.y), f32_to_bf16(sb.z), f32_to_bf16(sb.w)};
    if (head < hq + hk) {
      const float4 c01 = *(const float4*)(rope + (size_t)pos * half + e);      // (cos, sin) of e, e+1
      const float4 c23 = *(const float4*)(rope + (size_t)pos * half + e + 2);  // of e+2, e+3
      const float cs[4][2] = {{c01.x, c01.y}, {c01.z, c01.w}, {c23.x, c23.y}, {c23.z, c23.w}};
      uint16_t ra[4], rb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = bf16_to_f32(ua[i]), b = bf16_to_f32(ub[i]);
        ra[i] = f32_to_bf16(a * cs[i][0] - b * cs[i][1]);
        rb[i] = f32_to_bf16(b * cs[i][0] + a * cs[i][1]);
      }
      const uint2 pa = make_uint2(ra[0] | ((uint32_t)ra[1] << 16), ra[2] | ((uint32_t)ra[3] << 16));
      const uint2 pb = make_uint2(rb[0] | ((uint32_t)rb[1] << 16), rb[2] | ((uint32_t)rb[3] << 16));
      uint16_t* d = head < hq ? q_out + ((size_t)t * hq + head) * hd
                              : kp + (((size_t)page * hk + (head - hq)) * ps + pos % ps) * hd;
      *(uint2*)(d + e) = pa;
      *(uint2*)(d + e + half) = pb;
    } else {
      // V pages are stored transposed: [page][kv head][hd][slot].
      uint16_t* dv = vp + ((size_t)page * hk + (head - hq - hk)) * hd * ps + pos % ps;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dv[(size_t)(e + i) * ps] = ua[i];
        dv[(size_t)(e + half + i) * ps] = ub[i];
      }
    }
  }
}

hipError_t launch_rope_append_parts(const float* parts, int np, int T, int hq, int hk, int hd,
                                    void* q_out, const int* positions, int mode,
                                    const int* block_table, int max_pages, int ps, int n_pages,
                                    int pos_limit, void* kp, void* vp, const float* rope,
                                    hipStream_t st, const RopeRanks* rr) {
  if (hd % 8) return hipErrorInvalidValue;
  const int per_token = (hq + 2 * hk) * (hd / 8);  // threads' work items per token
  if (T == 0 || per_token == 0) return hipSuccess;
  const RopeRanks one{};
  const RopeRanks& rk = rr ? *rr : one;
  if (rr && (rr->n < 1 || rr->n > kMaxRanks)) return hipErrorInvalidValue;
  if (rr) {
    parts = rr->parts[0];
    q_out = rr->q_out[0];
    kp = rr->k_pages[0];
    vp = rr->v_pages[0];
    n_pages = rr->n_pages[0];
  }
  const int threads = per_token > 1024 - 63 ? 1024 : (per_token + 63) / 64 * 64;
  dim3 g((unsigned)T, rr && rr->n > 1 ? rr->n : 1), b(threads);
#define TPK_RAP(NPV)                                                                            \
  hipLaunchKernelGGL(k_rope_append_parts<NPV>, g, b, 0, st, parts, T, hq, hk, hd,               \
                     (uint16_t*)q_out, positions, mode, block_table, max_pages, ps, n_pages,    \
                     pos_limit, (uint16_t*)kp, (uint16_t*)vp, (const float2*)rope, rk)
  switch (np) {
    case 1: TPK_RAP(1); break;
    case 2: TPK_RAP(2); break;
    case 3: TPK_RAP(3); break;
    case 4: TPK_RAP(4); break;
    case 5: TPK_RAP(5); break;
    case 6: TPK_RAP(6); break;
    case 7: TPK_RAP(7); break;
    case 8: TPK_RAP(8); break;
    case 9: TPK_RAP(9); break;
    case 10: TPK_RAP(10); break;
    case 11: TPK_RAP(11); break;
    case 12: TPK_RAP(12); break;
    case 13: TPK_RAP(13); break;
    case 14: TPK_RAP(14); break;
    case 15: TPK_RAP(15); break;
    case 16: TPK_RAP(16); break;
    default: return hipErrorInvalidValue;
  }
#undef TPK_RAP
  return hipGetLastError();
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
// A wave walks its pages in 16-key tiles with the next tile's K and V loads in flight while the
// current tile is scored; the physical page ids of all its pages are fetched up front, in
// parallel with q. The four waves of a workgroup merge through LDS; with one split the result is
// final, otherwise k_attn_combine merges the splits.
constexpr int kMaxSplit = 1024;

template <int AT, int HD>
struct AttnTile {
  static constexpr int E = Vec16<AT>::N;
  static constexpr int LPK = HD / E;
  static constexpr int KPP = 64 / LPK;
  static constexpr int NP = 16 / KPP;  // passes per 16-key tile
};

template <int AT, int HD, int G>
__global__ __launch_bounds__(256) void k_attn_split(
    const void* __restrict__ q, const void* __restrict__ kpages, const void* __restrict__ vpages,
    const int* __restrict__ positions, int mode, const int* __restrict__ block_table,
    int max_pages, int ps, int n_pages, int hk, int chunk, int n_split, int pos_limit,
    float* __restrict__ part_o, float* __restrict__ part_ml, void* __restrict__ out,
    float scale_log2, AttnRanks ar) {
  using TL = AttnTile<AT, HD>;
  constexpr int E = TL::E, LPK = TL::LPK, KPP = TL::KPP, NP = TL::NP;
  constexpr int EB = (AT == ACT_F32) ? 4 : 2;
  static_assert(LPK <= 64 && KPP >= 1 && NP >= 1, "head_dim too large for one wavefront");
  __shared__ float s_m[4][G], s_l[4][G];
  __shared__ float s_o[4][G][HD];

  const int split = blockIdx.x, t = blockIdx.z;
  int g = blockIdx.y;
  if (ar.n > 1) {  // every rank in one launch: this block's rank and its buffers
    const int rank = g / hk;
    g -= rank * hk;
    q = ar.q[rank];
    kpages = ar.k_pages[rank];
    vpages = ar.v_pages[rank];
    n_pages = ar.n_pages[rank];
    part_o = ar.part_o[rank];
    part_ml = ar.part_ml[rank];
    out = ar.out[rank];
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane / LPK, e0 = (lane % LPK) * E;
  const int hq = hk * G;
  const int pos = clampi(positions[t], 0, pos_limit - 1);
  const int n_keys = pos + 1;
  const int k0 = split * chunk;
  const int k1 = min(n_keys, k0 + chunk);
  const int seq = (mode == 0) ? t : 0;

  // This wave's 16-key tiles: tile j covers keys k0 + (wave + 4 j) * 16 + [0, 16).
  const int tiles = (k1 > k0) ? (k1 - k0 + 15) / 16 : 0;
  const int ntw = tiles > wave ? (tiles - wave + 3) / 4 : 0;
  // Physical page of tile j, fetched by lane j % 64 (for j < 64; later blocks refetch).
  auto fetch_page = [&](int j) -> int {
    const int key = k0 + (wave + 4 * j) * 16;
    const int pg = min(key / ps, max_pages - 1);
    return clampi(block_table[(size_t)seq * max_pages + pg], 0, n_pages - 1);
  };
  int pid_reg = (lane < ntw) ? fetch_page(lane) : 0;

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

  auto tile_base = [&](int j, int pid) -> size_t {
    const int key = k0 + (wave + 4 * j) * 16;
    return (((size_t)pid * hk + g) * ps + (key % ps)) * HD;  // key % ps is a multiple of 16
  };
  auto load_tile = [&](int j, uint4 (&kbuf)[NP], uint4 (&vbuf)[NP]) {
    if (j >= 64 && (j & 63) == 0) pid_reg = (lane < ntw - j) ? fetch_page(j + lane) : 0;
    const int pid = __shfl(pid_reg, j & 63, 64);
    const size_t base = tile_base(j, pid);
    const size_t vbase = ((size_t)pid * hk + g) * HD;  // V^T: [page][head][hd][slot]
    const int slot0 = (k0 + (wave + 4 * j) * 16) % ps;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const size_t off = (base + (size_t)(p * KPP + sub) * HD + e0) * EB;
      kbuf[p] = *(const uint4*)((const char*)kpages + off);
      const int slot = slot0 + p * KPP + sub;
      uint32_t w[4];
      if constexpr (AT == ACT_F32) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          w[i] = ((const uint32_t*)vpages)[(vbase + e0 + i) * ps + slot];
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          w[i] = (uint32_t)((const uint16_t*)vpages)[(vbase + e0 + 2 * i) * ps + slot] |
                 ((uint32_t)((const uint16_t*)vpages)[(vbase + e0 + 2 * i + 1) * ps + slot] << 16);
      }
      vbuf[p] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  };
  auto score_tile = [&](int j, const uint4 (&kbuf)[NP], const uint4 (&vbuf)[NP]) {
    const int kbase = k0 + (wave + 4 * j) * 16;
    float s[NP][G];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      float kf[E];
      unpack16<AT>(kbuf[p], kf);
      const bool valid = kbase + p * KPP + sub < k1;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) d = fmaf(qv[h][e], kf[e], d);
#pragma unroll
        for (int o = LPK / 2; o > 0; o >>= 1) d += __shfl_xor(d, o, 64);
        s[p][h] = valid ? d : -INFINITY;
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = s[0][h];
#pragma unroll
      for (int p = 1; p < NP; ++p) mx = fmaxf(mx, s[p][h]);
#pragma unroll
      for (int o = LPK; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
      const float mn = fmaxf(m[h], mx);  // finite: key kbase < k1 is always valid
      const float alpha = exp2f(m[h] - mn);
      m[h] = mn;
      l[h] *= alpha;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[h][e] *= alpha;
    }
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      float vf[E];
      unpack16<AT>(vbuf[p], vf);
      if (!(kbase + p * KPP + sub < k1)) {
#pragma unroll
        for (int e = 0; e < E; ++e) vf[e] = 0.f;  // slots past the sequence may hold anything
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float pr = exp2f(s[p][h] - m[h]);
        l[h] += pr;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[h][e] = fmaf(pr, vf[e], acc[h][e]);
      }
    }
  };
  // Two named register buffers: tile j + 1 loads while tile j is scored.
  uint4 ka[NP], va[NP], kc[NP], vc[NP];
  if (ntw > 0) load_tile(0, ka, va);
  for (int j = 0; j < ntw; j += 2) {
    if (j + 1 < ntw) load_tile(j + 1, kc, vc);
    score_tile(j, ka, va);
    if (j + 2 < ntw) load_tile(j + 2, ka, va);
    if (j + 1 < ntw) score_tile(j + 1, kc, vc);
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
  const size_t tg = (size_t)t * hq + (size_t)g * G;  // first query head row of this group
  for (int idx = tid; idx < G * HD; idx += 256) {
    const int h = idx / HD, e = idx % HD;
    const float M = fmaxf(fmaxf(s_m[0][h], s_m[1][h]), fmaxf(s_m[2][h], s_m[3][h]));
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f = exp2f(s_m[w][h] - M);
        L += s_l[w][h] * f;
        O += s_o[w][h][e] * f;
      }
    }
    if (n_split == 1) {
      st_act<AT>(out, (tg + h) * HD + e, O / L);
    } else {
      const size_t row = (tg + h) * n_split + split;
      part_o[row * HD + e] = O;
      if (e == 0) {
        part_ml[row * 2] = M;
        part_ml[row * 2 + 1] = L;
      }
    }
  }
}

// bf16 attention on the matrix cores, for decode (split over keys) and prefill (causal).
//
// A wavefront owns 16 query rows. Decode: the G query heads of one token's KV group (rows G..15
// idle), and the four waves of a workgroup split the key range, then merge through LDS. Prefill:
// 16 consecutive tokens of one query head, each wave its own rows, keys up to the rows' causal
// limit. Per 32-key tile (two 16-key n-tiles, each inside one page):
//   S = Q K^T   v_mfma_f32_16x16x32_bf16, A = q rows (16 B of hd per lane), B = K rows (16 B);
//   online softmax on the 16 x 32 tile in registers (rows live in the same lanes as O's rows);
//   O += P V    P goes through LDS (bf16) into the A layout; B = 8 consecutive keys of one hd
//               column, a contiguous 16 B because V pages are stored transposed, [hd][slot].
// The next tile's K loads are issued once the scores are done and its V loads once P V is done.
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_a;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4_a;

constexpr int kPLd = 40;  // bf16 per LDS row of P (32 keys + padding)

// A decode launch reads each key and value once: streaming (non-temporal) loads, which keep the
// caches from filling with lines nothing reads again (64 sequences of 2048 keys, 4 ranks: 95.2 ->
// 83.2 us; one 4096-key sequence, 2 ranks: 2.3 us less per step). Heads of 256 measured 0.45 us
// faster per step with plain loads for one sequence but not for batches (the launcher picks), and
// prefill tiles re-read K and V from cache.
template <bool PLAIN>
__device__ __forceinline__ uint4 kv_ld(const uint16_t* p) {
  if constexpr (PLAIN) return *(const uint4*)p;
  else return ld_stream16(p);
}

// Decode with heads of up to 128 fits three waves per SIMD (168 registers) without spilling; more
// waves keep more key tiles in flight (64 sequences of 2048 keys, 4 ranks: 84.9 -> 83.4 us).
// NTW: streaming loads for heads wider than 128 too (the batched launches; see the launcher).
template <int HD, bool PREFILL, bool NTW = false>
__global__ __launch_bounds__(256, (HD <= 128 && !PREFILL) ? 3 : 1) void k_attn_mfma(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kpages,
    const uint16_t* __restrict__ vpages, const int* __restrict__ positions, int mode,
    const int* __restrict__ block_table, int max_pages, int ps, int n_pages, int hk, int G,
    int T, int chunk, int n_split, int pos_limit, float* __restrict__ part_o,
    float* __restrict__ part_ml, uint16_t* __restrict__ out, float scale_log2, AttnRanks ar) {
  constexpr int KS = HD / 32;  // MFMA k-steps over hd in Q K^T
  constexpr int NO = HD / 16;  // 16-wide hd n-tiles of O
  __shared__ __attribute__((aligned(16))) uint16_t s_pb[4][16 * kPLd];
  __shared__ float s_m[4][8], s_l[4][8];
  __shared__ float s_o[PREFILL ? 1 : 4][PREFILL ? 1 : 8][HD];

  int g = blockIdx.y;
  if (!PREFILL && ar.n > 1) {  // every rank in one launch: this block's rank and its buffers
    const int rank = g / hk;
    g -= rank * hk;
    q = (const uint16_t*)ar.q[rank];
    kpages = (const uint16_t*)ar.k_pages[rank];
    vpages = (const uint16_t*)ar.v_pages[rank];
    n_pages = ar.n_pages[rank];
    part_o = ar.part_o[rank];
    part_ml = ar.part_ml[rank];
    out = (uint16_t*)ar.out[rank];
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 15, fq = lane >> 4;
  const int hq = hk * G;

  // ---- rows of this wave and the key range
  int tok_fr, head_fr;   // the row this lane feeds into the A operand (row fr)
  bool row_ok_fr;
  int lim[4];            // per S/O row 4 fq + r: keys < lim are attended
  int kstart, kend, tstep, toff, seq, split = 0;
  if constexpr (PREFILL) {
    const int ntt = (T + 15) / 16;
    const int gi = blockIdx.x * 4 + wave;                // group: (token tile, head in group)
    const bool gok = gi < ntt * G;
    const int tt = gok ? (ntt - 1) - gi / G : 0;         // latest tokens first
    const int hh = gok ? gi % G : 0;
    tok_fr = tt * 16 + fr;
    row_ok_fr = gok && tok_fr < T;
    head_fr = g * G + hh;
    int kmax = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tk = tt * 16 + 4 * fq + r;
      const bool ok = gok && tk < T;
      lim[r] = ok ? clampi(positions[tk], 0, pos_limit - 1) + 1 : pos_limit;
    }
    for (int r = 0; r < 16; ++r) {
      const int tk = tt * 16 + r;
      if (gok && tk < T) kmax = max(kmax, clampi(positions[tk], 0, pos_limit - 1) + 1);
    }
    kstart = 0;
    kend = kmax;
    tstep = 1;
    toff = 0;
    seq = 0;
  } else {
    split = blockIdx.x;
    const int t = blockIdx.z;
    tok_fr = t;
    row_ok_fr = fr < G;
    head_fr = g * G + (fr < G ? fr : 0);
    const int nk = clampi(positions[t], 0, pos_limit - 1) + 1;
    kstart = split * chunk;
    kend = min(nk, kstart + chunk);
#pragma unroll
    for (int r = 0; r < 4; ++r) lim[r] = kend;
    tstep = 4;
    toff = wave;
    seq = (mode == 0) ? t : 0;
  }
  const int tiles = (kend > kstart) ? (kend - kstart + 31) / 32 : 0;
  const int ntw = tiles > toff ? (tiles - toff + tstep - 1) / tstep : 0;

  // Page ids: lane i of pid_reg holds the page of n-tile 64 * block + i of this wave.
  auto tile_key = [&](int j) { return kstart + (toff + tstep * j) * 32; };
  auto fetch_page = [&](int nt) -> int {
    const int key = tile_key(nt >> 1) + 16 * (nt & 1);
    const int pg = min(key / ps, max_pages - 1);
    return clampi(block_table[(size_t)seq * max_pages + pg], 0, n_pages - 1);
  };
  int pid_reg = (lane < 2 * ntw) ? fetch_page(lane) : 0;
  auto page_of = [&](int j, int h) -> int { return __shfl(pid_reg, (2 * j + h) & 63, 64); };

  bf16x8_a qf[KS];
  {
    const uint16_t* qrow = q + ((size_t)(row_ok_fr ? tok_fr : 0) * hq + head_fr) * HD;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 v = row_ok_fr ? *(const uint4*)(qrow + ks * 32 + fq * 8) : make_uint4(0, 0, 0, 0);
      qf[ks] = __builtin_bit_cast(bf16x8_a, v);
    }
  }
  float m[4], lsum[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m[r] = -INFINITY;
    lsum[r] = 0.f;
  }
  floatx4_a o[NO];
#pragma unroll
  for (int n = 0; n < NO; ++n) o[n] = floatx4_a{0.f, 0.f, 0.f, 0.f};

  uint4 kf[2][KS], vf[NO];
  auto load_k = [&](int j) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int pid = page_of(j, h);
      const int key = tile_key(j) + 16 * h + fr;
      const uint16_t* base = kpages + (((size_t)pid * hk + g) * ps + (key % ps)) * HD + fq * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kf[h][ks] = kv_ld<PREFILL || (HD > 128 && !NTW)>(base + ks * 32);
    }
  };
  auto load_v = [&](int j) {
    // lane: hd column n * 16 + fr, keys 8 fq .. 8 fq + 7 of the tile (n-tile fq / 2)
    const int pid = page_of(j, fq >> 1);
    const int slot = (tile_key(j) + 16 * (fq >> 1)) % ps + 8 * (fq & 1);
    const uint16_t* base = vpages + (((size_t)pid * hk + g) * HD + fr) * ps + slot;
#pragma unroll
    for (int n = 0; n < NO; ++n) vf[n] = kv_ld<PREFILL || (HD > 128 && !NTW)>(base + (size_t)n * 16 * ps);
  };
  auto refresh_pages = [&](int j) {
    if ((j & 31) == 0) {
      const int nt = 2 * j + lane;
      pid_reg = (nt < 2 * ntw) ? fetch_page(nt) : 0;
    }
  };
  uint16_t* pb = s_pb[wave];
  if (ntw > 0) {
    load_k(0);
    load_v(0);
  }
  for (int j = 0; j < ntw; ++j) {
    const int kb0 = tile_key(j);
    floatx4_a sc[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      sc[h] = floatx4_a{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        sc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[ks], __builtin_bit_cast(bf16x8_a, kf[h][ks]),
                                                        sc[h], 0, 0, 0);
    }
    if (j + 1 < ntw) {
      refresh_pages(j + 1);
      load_k(j + 1);
    }
    // Lane holds S[row 4 fq + r][key kb0 + 16 h + fr].
    float tmax[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int key = kb0 + 16 * h + fr;
        sc[h][r] = (key < lim[r] && key < kend) ? sc[h][r] * scale_log2 : -INFINITY;
      }
      tmax[r] = fmaxf(sc[0][r], sc[1][r]);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) tmax[r] = row16_max(tmax[r]);
    float alpha[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      // Every row has a valid key in its first tile, so mn is finite from there on.
      const float mn = fmaxf(m[r], tmax[r]);
      alpha[r] = exp2f(m[r] - mn);
      m[r] = mn;
      const float p0 = exp2f(sc[0][r] - mn), p1 = exp2f(sc[1][r] - mn);
      lsum[r] = lsum[r] * alpha[r] + p0 + p1;
      const int row = 4 * fq + r;
      pb[row * kPLd + fr] = f32_to_bf16(p0);
      pb[row * kPLd + 16 + fr] = f32_to_bf16(p1);
    }
#pragma unroll
    for (int n = 0; n < NO; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) o[n][r] *= alpha[r];
    // Keys at or past kend get P = 0, but a slot no key was written to may hold a NaN or an Inf,
    // and 0 times either is a NaN: the last tile zeroes its V elements past kend (this lane's
    // eight keys are kb0 + 8 fq .. kb0 + 8 fq + 7 in every hd column).
    if (kb0 + 32 > kend) {
      const uint4 keep = v_keep_mask(kend - (kb0 + 8 * fq));
#pragma unroll
      for (int n = 0; n < NO; ++n) {
        vf[n].x &= keep.x;
        vf[n].y &= keep.y;
        vf[n].z &= keep.z;
        vf[n].w &= keep.w;
      }
    }
    // The wave's own P writes must land before its lanes read them back in the A layout.
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    const bf16x8_a pa = *(const bf16x8_a*)(pb + fr * kPLd + fq * 8);
#pragma unroll
    for (int n = 0; n < NO; ++n)
      o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, __builtin_bit_cast(bf16x8_a, vf[n]), o[n],
                                                     0, 0, 0);
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    if (j + 1 < ntw) load_v(j + 1);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) lsum[r] = row16_sum(lsum[r]);

  if constexpr (PREFILL) {
    // Lane holds O[row 4 fq + r][hd n * 16 + fr]; write the finished rows.
    const int ntt = (T + 15) / 16;
    const int gi = blockIdx.x * 4 + wave;
    if (gi >= ntt * G) return;
    const int tt = (ntt - 1) - gi / G, hh = gi % G;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tk = tt * 16 + 4 * fq + r;
      if (tk >= T) continue;
      const float inv = 1.0f / lsum[r];
      uint16_t* orow = out + ((size_t)tk * hq + g * G + hh) * HD;
#pragma unroll
      for (int n = 0; n < NO; ++n) orow[n * 16 + fr] = f32_to_bf16(o[n][r] * inv);
    }
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * fq + r;
      if (row < G) {
        if (fr == 0) {
          s_m[wave][row] = m[r];
          s_l[wave][row] = lsum[r];
        }
#pragma unroll
        for (int n = 0; n < NO; ++n) s_o[wave][row][n * 16 + fr] = o[n][r];
      }
    }
    __syncthreads();
    const int t = blockIdx.z;
    const size_t tg = (size_t)t * hq + (size_t)g * G;
    for (int idx = tid; idx < G * HD; idx += 256) {
      const int h = idx / HD, e = idx % HD;
      const float M = fmaxf(fmaxf(s_m[0][h], s_m[1][h]), fmaxf(s_m[2][h], s_m[3][h]));
      float L = 0.f, O = 0.f;
      if (M != -INFINITY) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float f = exp2f(s_m[w][h] - M);
          L += s_l[w][h] * f;
          O += s_o[w][h][e] * f;
        }
      }
      if (n_split == 1) {
        out[(tg + h) * HD + e] = f32_to_bf16(O / L);
      } else {
        const size_t row = (tg + h) * n_split + split;
        part_o[row * HD + e] = O;
        if (e == 0) {
          part_ml[row * 2] = M;
          part_ml[row * 2 + 1] = L;
        }
      }
    }
  }
}

// Merge of the key splits: workgroup (token, query head, 64-element slice of hd). Every split's
// (m, l) is loaded in parallel, the weights 2^(m_s - M) go through LDS, four threads per element
// each sum a quarter of the splits with independent loads, and the quarters are added in order.
template <int AT>
__global__ __launch_bounds__(256) void k_attn_combine(const float* __restrict__ part_o,
                                                      const float* __restrict__ part_ml,
                                                      int n_split, int hd, int hq,
                                                      void* __restrict__ out, AttnRanks ar) {
  __shared__ float s_w[kMaxSplit];
  __shared__ float s_red[2][4];
  __shared__ float s_acc[4][64];
  const int t = blockIdx.x, tid = threadIdx.x;
  int h = blockIdx.y;
  if (ar.n > 1) {  // every rank in one launch (blockIdx.y = rank * hq + head)
    const int rank = h / hq;
    h -= rank * hq;
    part_o = ar.part_o[rank];
    part_ml = ar.part_ml[rank];
    out = ar.out[rank];
  }
  const int e = blockIdx.z * 64 + (tid & 63), part = tid >> 6;
  const size_t row0 = ((size_t)t * hq + h) * n_split;
  float mx = -INFINITY;
  for (int sp = tid; sp < n_split; sp += 256) {
    const float m = part_ml[(row0 + sp) * 2];
    s_w[sp] = m;
    mx = fmaxf(mx, m);
  }
  mx = wave_max(mx);
  if ((tid & 63) == 0) s_red[0][tid >> 6] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(s_red[0][0], s_red[0][1]), fmaxf(s_red[0][2], s_red[0][3]));
  float lsum = 0.f;
  for (int sp = tid; sp < n_split; sp += 256) {
    const float m = s_w[sp];
    const float w = (m == -INFINITY) ? 0.f : exp2f(m - M);
    s_w[sp] = w;
    lsum += part_ml[(row0 + sp) * 2 + 1] * w;
  }
  lsum = wave_sum(lsum);
  if ((tid & 63) == 0) s_red[1][tid >> 6] = lsum;
  __syncthreads();
  const float L = (s_red[1][0] + s_red[1][1]) + (s_red[1][2] + s_red[1][3]);
  float acc = 0.f;
  if (e < hd) {
#pragma unroll 8
    for (int sp = part; sp < n_split; sp += 4) acc += part_o[(row0 + sp) * hd + e] * s_w[sp];
  }
  s_acc[part][tid & 63] = acc;
  __syncthreads();
  if (part == 0 && e < hd) {
    const float o = ((s_acc[0][tid] + s_acc[1][tid]) + s_acc[2][tid]) + s_acc[3][tid];
    st_act<AT>(out, ((size_t)t * hq + h) * hd + e, o / L);
  }
}

template <int HD>
static hipError_t attn_mfma_g(bool prefill, int G, int T, int hk, hipStream_t st, const void* q,
                              const void* kp, const void* vp, const int* positions, int mode,
                              const int* bt, int max_pages, int ps, int n_pages, int chunk,
                              int n_split, int pos_limit, float* po, float* pml, void* out,
                              float sl2, const AttnRanks& ar) {
  if (G > 8) return hipErrorInvalidValue;
  if (prefill) {
    const int groups = (T + 15) / 16 * G;
    dim3 grid((groups + 3) / 4, hk, 1);
    hipLaunchKernelGGL((k_attn_mfma<HD, true>), grid, dim3(256), 0, st, (const uint16_t*)q,
                       (const uint16_t*)kp, (const uint16_t*)vp, positions, mode, bt, max_pages,
                       ps, n_pages, hk, G, T, chunk, 1, pos_limit, po, pml, (uint16_t*)out, sl2,
                       AttnRanks{});
  } else {
    dim3 grid(n_split, hk * (ar.n > 1 ? ar.n : 1), T);
    // Heads wider than 128: plain loads for a few sequences (the Gemma-like decode, 0.5 us per
    // step faster than streaming loads), streaming loads for batches (the Gemma-like 64-sequence
    // batch streams 255 MB of K and V: 153.1 -> 146.8 us per step).
    if (HD > 128 && T > 4)
      hipLaunchKernelGGL((k_attn_mfma<HD, false, true>), grid, dim3(256), 0, st,
                         (const uint16_t*)q, (const uint16_t*)kp, (const uint16_t*)vp, positions,
                         mode, bt, max_pages, ps, n_pages, hk, G, T, chunk, n_split, pos_limit,
                         po, pml, (uint16_t*)out, sl2, ar);
    else
      hipLaunchKernelGGL((k_attn_mfma<HD, false>), grid, dim3(256), 0, st, (const uint16_t*)q,
                         (const uint16_t*)kp, (const uint16_t*)vp, positions, mode, bt,
                         max_pages, ps, n_pages, hk, G, T, chunk, n_split, pos_limit, po, pml,
                         (uint16_t*)out, sl2, ar);
  }
  return hipGetLastError();
}

template <int AT, int HD>
static hipError_t attn_g(int G, dim3 grid, hipStream_t st, const void* q, const void* kp,
                         const void* vp, const int* positions, int mode, const int* bt,
                         int max_pages, int ps, int n_pages, int hk, int chunk, int n_split,
                         int pos_limit, float* po, float* pml, void* out, float sl2,
                         const AttnRanks& ar) {
#define TPK_ATT(GV)                                                                           \
  hipLaunchKernelGGL((k_attn_split<AT, HD, GV>), grid, dim3(256), 0, st, q, kp, vp, positions, \
                     mode, bt, max_pages, ps, n_pages, hk, chunk, n_split, pos_limit, po, pml,   \
                     out, sl2, ar)
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

static hipError_t attn_decode_impl(int at, int hd, int G, int T, int hk, const void* q,
                                   const void* kp, const void* vp, const int* positions, int mode,
                                   const int* bt, int max_pages, int ps, int n_pages, int chunk,
                                   int n_split, int pos_limit, float* part_o, float* part_ml,
                                   void* out, const AttnRanks& ar, hipStream_t st) {
  if (T == 0) return hipSuccess;
  if (n_split > kMaxSplit || chunk % 16 || ps % 16) return hipErrorInvalidValue;
  const int nr = ar.n > 1 ? ar.n : 1;
  const float sl2 = 1.4426950408889634f / sqrtf((float)hd);
  dim3 grid(n_split, hk * nr, T);
  hipError_t e;
#define TPK_HD(ATV, HDV)                                                                        \
  e = attn_g<ATV, HDV>(G, grid, st, q, kp, vp, positions, mode, bt, max_pages, ps, n_pages, hk, \
                       chunk, n_split, pos_limit, part_o, part_ml, out, sl2, ar)
  if (at == ACT_F32) {
    if (hd == 64) TPK_HD(ACT_F32, 64);
    else if (hd == 128) TPK_HD(ACT_F32, 128);
    else if (hd == 256) TPK_HD(ACT_F32, 256);
    else return hipErrorInvalidValue;
  } else {
    if (chunk % 32) return hipErrorInvalidValue;
    const bool prefill = (mode == 1);
    if (prefill && nr > 1) return hipErrorInvalidValue;
    if (prefill && attn_prefill_supported(hd, G, ps))
      return launch_attn_prefill(hd, G, T, hk, q, kp, vp, positions, bt, max_pages, n_pages,
                                 pos_limit, out, st);
#define TPK_HDM(HDV)                                                                          \
  e = attn_mfma_g<HDV>(prefill, G, T, hk, st, q, kp, vp, positions, mode, bt, max_pages, ps, \
                       n_pages, chunk, n_split, pos_limit, part_o, part_ml, out, sl2, ar)
    if (hd == 64) TPK_HDM(64);
    else if (hd == 128) TPK_HDM(128);
    else if (hd == 256) TPK_HDM(256);
    else return hipErrorInvalidValue;
#undef TPK_HDM
    if (prefill) return e;
  }
#undef TPK_HD
  if (e != hipSuccess || n_split == 1) return e;
  const int hq = hk * G;
  dim3 cg(T, hq * nr, (hd + 63) / 64), cb(256);
  if (at == ACT_F32)
    hipLaunchKernelGGL(k_attn_combine<ACT_F32>, cg, cb, 0, st, part_o, part_ml, n_split, hd, hq,
                       out, ar);
  else
    hipLaunchKernelGGL(k_attn_combine<ACT_BF16>, cg, cb, 0, st, part_o, part_ml, n_split, hd, hq,
                       out, ar);
  return hipGetLastError();
}

hipError_t launch_attn_decode(int at, int hd, int G, int T, int hk, const void* q, const void* kp,
                              const void* vp, const int* positions, int mode, const int* bt,
                              int max_pages, int ps, int n_pages, int chunk, int n_split,
                              int pos_limit, float* part_o, float* part_ml, void* out,
                              hipStream_t st) {
  return attn_decode_impl(at, hd, G, T, hk, q, kp, vp, positions, mode, bt, max_pages, ps,
                          n_pages, chunk, n_split, pos_limit, part_o, part_ml, out, AttnRanks{},
                          st);
}

hipError_t launch_attn_decode_ranks(int at, int hd, int G, int T, int hk, const AttnRanks& ar,
                                    const int* positions, const int* bt, int max_pages, int ps,
                                    int chunk, int n_split, int pos_limit, hipStream_t st) {
  if (ar.n < 1 || ar.n > kMaxRanks) return hipErrorInvalidValue;
  for (int r = 0; r < ar.n; ++r)
    if (!ar.q[r] || !ar.k_pages[r] || !ar.v_pages[r] || !ar.part_o[r] || !ar.part_ml[r] ||
        !ar.out[r] || ar.n_pages[r] < 1)
      return hipErrorInvalidValue;
  return attn_decode_impl(at, hd, G, T, hk, ar.q[0], ar.k_pages[0], ar.v_pages[0], positions, 0,
                          bt, max_pages, ps, ar.n_pages[0], chunk, n_split, pos_limit,
                          ar.part_o[0], ar.part_ml[0], ar.out[0], ar, st);
}

}  // namespace tpk
