// K2 / K3: decode projections, y[t, o] = sum_k x[t, k] W[o, k], for a handful of tokens.
//
// Decode reads every byte of a rank's 1/N weight slice once per step and does ~1 FLOP per byte,
// so these kernels are HBM-streaming GEMVs, not GEMMs. A wavefront owns R weight rows and streams
// them with 16-byte loads, U per row and lane in flight (R * U = 16 loads per lane, 12 for Q8_0),
// R chosen by row length so short rows (o_proj, Q8_0) still keep enough bytes in flight. The first
// batch of loads is issued before the token vectors are staged in LDS, so the two latencies
// overlap. Dot products finish with DPP row reductions.
//
// Weight formats: fp32, bf16, and Q8_0 split into an int8 code plane [out, in] plus an fp16 scale
// plane [out, in/32]. For Q8_0 the token rows are staged as fp16, each chunk of 16 values scaled
// by its own power of two (largest magnitude in [2^14, 2^15)): bf16 values fit fp16's 11-bit
// significand exactly, and the prologue's gamma * x is rounded once to it. A code c becomes the
// fp16 number 1152 + c with one byte permute per two codes (its sign bit flipped gives the byte
// c + 128, placed under the exponent of 1024), and the chunk is
// sum_k c_k x_k = sum_k (1152 + c_k) x_k - 1152 sum_k x_k, eight two-term fp16 dot products with
// fp32 accumulation (the products are exact in fp32) and the staged offset. A code costs one
// instruction instead of a conversion and an FMA, which matters here: the weight bytes are a
// quarter of fp32's per value, so the arithmetic per byte is four times the fp32 path's.
// Epilogues:
//   EPI_F32 / EPI_BF16   store a partial sum (row-parallel o_proj and down, TensorSharp "How
//             tensor parallelism works", step 3);
//   EPI_GATED act(g) * u of the column-parallel gate/up pair (row slots 2k, 2k + 1 hold rows p
//             and p + gate_off);
//   EPI_ROPE  the fused QKV epilogue: slots 2k, 2k + 1 hold rows i and i + hd/2 of one head, so
//             the rotary embedding of q and k is applied in registers, q is stored and k and v are
//             appended to the rank's paged cache (step 2 of the same section: its own KV cache);
//   EPI_REDUCE, EPI_REDUCE_BF  the last rank's row-parallel projection in the one-call block
//             step: the partial (fp32, or bf16) plus the local reduce (earlier ranks' partials in
//             rank order, then the residual);
//   EPI_RED_ALL, EPI_RED_ALL_BF  every rank's row-parallel projection in one launch (N <= 4): the
//             waves of a workgroup take the same rows for different ranks (N waves per row group,
//             each rank's inputs staged side by side, each rank's dot products exactly as in that
//             rank's own launch), store each partial, and one wave per row group adds them in
//             rank order from LDS, then the residual.
// Column-parallel epilogues can also cover every rank in one launch (RankPtrs): each block
// picks its rank's weight slice and outputs by its index.
// With PRO (FuseArgs::gamma set) the projection's input is RMSNorm(X) * gamma of the residual rows
// X: the workgroup stages gamma * x (exact in fp32) and the row's sum of squares from the same
// loads, and scales the finished dot products by 1/sqrt(mean(x^2) + eps), so the norm costs no
// extra pass, barrier or memory trip.
#pragma once
#include "tp_common.h"
#include "tp_kernels.h"

namespace tpk {

template <int WT> struct WFmt;
template <> struct WFmt<W_F32> { static constexpr int VE = 4, WB = 4; };
template <> struct WFmt<W_BF16> { static constexpr int VE = 8, WB = 2; };
template <> struct WFmt<W_Q8> { static constexpr int VE = 16, WB = 1; };

// Decode one 16-byte weight chunk into VE fp32 values (Q8_0: for the MoE expert kernels; the
// decode GEMV's main loop takes fp16 dot products of Q8_0 chunks instead).
template <int WT>
__device__ __forceinline__ void decode_chunk(const uint4& raw, float scale, float* w) {
  const uint32_t r[4] = {raw.x, raw.y, raw.z, raw.w};
  if constexpr (WT == W_F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = __uint_as_float(r[i]);
  } else if constexpr (WT == W_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w[2 * i] = __uint_as_float(r[i] << 16);
      w[2 * i + 1] = __uint_as_float(r[i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int32_t code = (int32_t)(int8_t)((r[i] >> (8 * b)) & 0xffu);
        w[4 * i + b] = q8_dequant(scale, code);
      }
    }
  }
}

typedef _Float16 q8h2 __attribute__((ext_vector_type(2)));

// Stage one chunk of 16 activations for the Q8_0 inner product: the values times a power of two
// that puts the largest magnitude in [2^14, 2^15) (2^127 for an all-zero or subnormal chunk, so
// the scale stays a finite float), rounded to fp16, and the pair (1152 * sum of the fp16 values,
// 1 / scale) that turns a chunk's dot product with the codes' 1152 + c back into sum c x.
__device__ __forceinline__ void q8_stage_chunk(const float* v, uint16_t* dst, float2* meta) {
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(v[e]));
  const int eb = (int)((__float_as_uint(amax) >> 23) & 0xffu);  // amax in [2^(eb-127), 2^(eb-126))
  const int sb = 268 - eb > 254 ? 254 : 268 - eb;                // scale 2^(141 - eb)
  const float sc = __uint_as_float((uint32_t)sb << 23), inv = 1.0f / sc;
  uint32_t h[8];
  float sum = 0.f;
#pragma unroll
  for (int e = 0; e < 16; e += 2) {
    const _Float16 a = (_Float16)(v[e] * sc), b = (_Float16)(v[e + 1] * sc);
    sum += (float)a + (float)b;
    h[e / 2] = (uint32_t)__builtin_bit_cast(uint16_t, a) |
               ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
  }
  *(uint4*)dst = make_uint4(h[0], h[1], h[2], h[3]);
  *(uint4*)(dst + 8) = make_uint4(h[4], h[5], h[6], h[7]);
  *meta = make_float2(1152.f * sum * inv, inv);
}

__device__ __forceinline__ int clampi_g(int v, int lo, int hi) {
  return v < lo ? lo : (v > hi ? hi : v);
}

// Rows per wave: by the number of 16-byte chunks per row, so that each wave streams a few KB, but
// no more than leaves about 1024 waves (one per SIMD) when the matrix has few rows.
inline int gemv_rows_per_wave(int nch, bool paired, long rows) {
  int r = nch > 512 ? 1 : (nch > 256 ? 2 : (nch > 128 ? 4 : 8));
  while (r > 1 && rows / r < 1024) r >>= 1;
  return (paired && r < 2) ? 2 : r;
}

constexpr int kMaxPrevPartials = 7;  // EPI_REDUCE: tp_degree <= 8

// PRO: the norm prologue; PV: the reduce epilogues' room for earlier partials (1, 3 or 7: every
// one is fetched ahead of the weight stream and held in registers, so it is sized to the degree).
template <int WT, int AT, int EPI, int NT, int ACTF, int R, bool PRO, int PV>
__global__ __launch_bounds__(256) void k_gemv(const void* __restrict__ W,
                                              const uint16_t* __restrict__ S, int K, int n_out,
                                              int gate_off, const void* __restrict__ X,
                                              void* __restrict__ Y, int ldy, RopeEpi re,
                                              FuseArgs fa, RankPtrs rp) {
  // [NR][NT][K] staged token rows (NR ranks' inputs under EPI_RED_ALL*, else one): fp32, or as
  // stored when EPI_RED_ALL* takes bf16 rows (which halves the workgroup's LDS); Q8_0 weights
  // take fp16 rows and then [NR][NT][K / 16] (offset, 1 / scale) pairs
  extern __shared__ float xs[];
  __shared__ float red[PRO ? NT : 1][4];  // prologue norm: each wave's sum of squares per token
  constexpr int VE = WFmt<WT>::VE;
  constexpr int WB = WFmt<WT>::WB;
  constexpr int AV = Vec16<AT>::N;
  // Q8_0, measured on the Gemma-like shard: at four rows per wave one chunk per row in flight
  // (gate/up 13.0 -> 11.3 us against three: more waves per SIMD, and the staging of one wave
  // overlaps the others' streams); at one or two rows twelve chunks in all, so that a batch
  // covers a 5120-wide down row (9.7 us, against 10.4-11.0 with two to four per row).
  constexpr int U = WT == W_Q8 ? (R == 4 ? 1 : (R >= 8 ? 2 : 12 / R)) : 16 / R;
  static_assert(WT != W_Q8 || AT == ACT_BF16, "Q8_0 weights take bf16 activations");
  constexpr bool PAIRED = (EPI == EPI_GATED || EPI == EPI_ROPE);
  static_assert(!PAIRED || R % 2 == 0, "paired epilogues need an even number of rows");
  constexpr bool ALLR = (EPI == EPI_RED_ALL || EPI == EPI_RED_ALL_BF);
  constexpr bool XS16 = ALLR && AT == ACT_BF16;  // bf16 rows in LDS, widened (exactly) on use
  uint16_t* const xs16 = (uint16_t*)xs;
  // The wave index is uniform: with it in a scalar register, each weight row's base address is
  // too, and the loads take a 32-bit lane offset instead of a 64-bit address per lane.
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // A column-parallel launch over all ranks: this block's rank and its pointers.
  int blk = blockIdx.x;
  if constexpr (!ALLR) {
    if (rp.n > 1) {
      const int rank = blockIdx.x / rp.bpr;
      blk -= rank * rp.bpr;
      W = rp.w[rank];
      S = rp.s[rank];
      Y = rp.y[rank];
      re.q_out = rp.q_out[rank];
      re.k_pages = rp.k_pages[rank];
      re.v_pages = rp.v_pages[rank];
      re.n_pages = rp.n_pages[rank];
    }
  }
  const int NR = ALLR ? rp.n : 1;
  // EPI_RED_ALL* (N <= 4): WPR = N waves per row group (wave w serves rank w % N), RW row
  // groups per workgroup.
  const int WPR = NR < 4 ? NR : 4, RW = 4 / WPR;
  const int w = ALLR ? blk * RW + wave / WPR : blk * 4 + wave;

  // Rows of this wavefront's slots.
  int row[R];
  bool ok[R];
  const int half = re.hd >> 1;
#pragma unroll
  for (int s = 0; s < R; ++s) {
    if constexpr (EPI == EPI_GATED) {
      const int p = w * (R / 2) + s / 2;
      ok[s] = p < n_out;
      row[s] = (s & 1) ? p + gate_off : p;
    } else if constexpr (EPI == EPI_ROPE) {
      const int p = w * (R / 2) + s / 2;
      ok[s] = p < (n_out >> 1);
      row[s] = (p / half) * re.hd + (p % half) + ((s & 1) ? half : 0);
    } else {
      row[s] = w * R + s;
      ok[s] = row[s] < n_out && (!ALLR || wave / WPR < RW);
    }
    if (!ok[s]) row[s] = 0;  // loads stay in bounds; results are dropped
  }
  const bool active = ok[0];
  const int nch = K / VE;

  // EPI_REDUCE: the earlier ranks' partials and the residual of this lane's token (lane t stores
  // token t) are requested first and kept as raw bits until the epilogue, so no wait for them
  // sits in front of the weight stream.
  constexpr bool RED = (EPI == EPI_REDUCE || EPI == EPI_REDUCE_BF);
  constexpr bool RES = RED || ALLR;
  constexpr int RV = RES ? R : 1;
  static_assert(PV >= 1 && PV <= kMaxPrevPartials, "earlier partials held per row");
  // The loads are unconditional (a lane past the launch's tokens reads token 0, a partial past
  // n_prev reads partial 0, rows out of range read row 0): guarded loads would be merged with
  // their defaults at the branch joins, and each merge waits for its load.
  uint32_t e_prev[RED ? RV : 1][PV], e_res[RV];
  if constexpr (RES) {
    const int tl = lane < NT ? lane : 0;
    const bool any_prev = fa.n_prev > 0;
#pragma unroll
    for (int s = 0; s < R; ++s) {
      const size_t idx = (size_t)tl * ldy + row[s];
      if constexpr (AT == ACT_F32) e_res[s] = ((const uint32_t*)fa.res_in)[idx];
      else e_res[s] = ((const uint16_t*)fa.res_in)[idx];
      if constexpr (RED) {
#pragma unroll
      for (int k = 0; k < PV; ++k) {
        const size_t pi = any_prev ? (size_t)(k < fa.n_prev ? k : 0) * fa.part_stride + idx : 0;
        const void* base = any_prev ? fa.prev : fa.res_in;
        if constexpr (EPI == EPI_REDUCE_BF) e_prev[s][k] = ((const uint16_t*)base)[pi];
        else e_prev[s][k] = ((const uint32_t*)base)[any_prev ? pi : 0];
      }
      }
    }
  }

  const char* wp[R];
  const uint16_t* sp[R];
  auto set_rows = [&](const void* Wr, const uint16_t* Sr) {
#pragma unroll
    for (int s = 0; s < R; ++s) {
      wp[s] = (const char*)Wr + (size_t)row[s] * K * WB;
      sp[s] = Sr + (size_t)row[s] * (K / 32);
    }
  };
  if constexpr (!ALLR) set_rows(W, S);
  uint4 b[R][U];
  float sc[R][U];
  auto load_batch = [&](int c0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * 64 + lane;
      if (c < nch) {
#pragma unroll
        for (int s = 0; s < R; ++s) {
          b[s][u] = ld_stream16(wp[s] + (size_t)c * 16);
          if constexpr (WT == W_Q8) sc[s][u] = f16_to_f32(sp[s][c >> 1]);
          else sc[s][u] = 0.f;
        }
      } else {
#pragma unroll
        for (int s = 0; s < R; ++s) {
          b[s][u] = make_uint4(0, 0, 0, 0);
          sc[s][u] = 0.f;
        }
      }
    }
  };
  // In flight while the token vectors are staged (EPI_RED_ALL*: the first batch of the wave's
  // first rank).
  const int rk0 = ALLR ? wave % WPR : 0;
  if constexpr (ALLR) set_rows(rp.w[rk0], rp.s[rk0]);  // rk0 < NR; idle waves read row 0
  load_batch(0);

  // Rotary epilogue inputs (each token's position and KV page, the cos/sin of this wave's pairs)
  // do not depend on the projection, so they are fetched here, under the weight stream, instead
  // of as two dependent round trips after it.
  constexpr int EN = (EPI == EPI_ROPE) ? NT : 1, EP = (EPI == EPI_ROPE) ? R / 2 : 1;
  int e_pos[EN], e_page[EN];
  float2 e_cs[EP][EN];
  if constexpr (EPI == EPI_ROPE) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int tok = re.t0 + t;
      e_pos[t] = clampi_g(re.positions[tok], 0, re.pos_limit - 1);
      const int seq = (re.mode == 0) ? tok : 0;
      const int pg = min(e_pos[t] / re.ps, re.max_pages - 1);
      e_page[t] = clampi_g(re.block_table[(size_t)seq * re.max_pages + pg], 0, re.n_pages - 1);
#pragma unroll
      for (int s = 0; s < R; s += 2) {
        const int p = w * (R / 2) + s / 2;
        e_cs[s / 2][t] = make_float2(1.f, 0.f);
        if (ok[s] && p / half < re.hq + re.hk)
          e_cs[s / 2][t] = ((const float2*)re.rope)[(size_t)e_pos[t] * half + p % half];
      }
    }
  }

  // Q8_0: [NR][NT][K] fp16 token rows, then [NR][NT][K / 16] (offset, 1 / scale) per chunk.
  uint16_t* const xh = (uint16_t*)xs;
  float2* const xc = (float2*)(xh + (size_t)NR * NT * K);
  if constexpr (WT == W_Q8) {
    float ssq[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) ssq[t] = 0.f;
    for (int i = tid; i < NR * NT * nch; i += 256) {
      const int rt = i / nch, c = i - rt * nch;  // chunk c of token row rt = r * NT + t
      const int r = rt / NT, t = rt - r * NT;
      const uint16_t* xr = (const uint16_t*)(ALLR ? rp.x[r] : X) + (size_t)t * K + (size_t)c * 16;
      float v[16];
      Vec16<ACT_BF16>::load(xr, v);
      Vec16<ACT_BF16>::load(xr + 8, v + 8);
      if constexpr (PRO) {
        float g[16];
        Vec16<ACT_BF16>::load((const uint16_t*)fa.gamma + (size_t)c * 16, g);
        Vec16<ACT_BF16>::load((const uint16_t*)fa.gamma + (size_t)c * 16 + 8, g + 8);
        float q = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          q = fmaf(v[e], v[e], q);
          v[e] *= g[e];
        }
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
          if (tt == t) ssq[tt] += q;
      }
      q8_stage_chunk(v, xh + (size_t)i * 16, xc + i);
    }
    if constexpr (PRO) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const float w = wave_sum(ssq[t]);
        if (lane == 0) red[t][wave] = w;
      }
    }
  } else if constexpr (PRO) {
    // gamma * x and the squares of x from one load of each; per token, a wave sum per wave.
    constexpr int EB = AT == ACT_F32 ? 4 : 2;
    float ssq[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) ssq[t] = 0.f;
    for (int k = tid * AV; k < K; k += 256 * AV) {
      float g[AV];
      Vec16<AT>::load((const char*)fa.gamma + (size_t)k * EB, g);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        float xv[AV];
        Vec16<AT>::load((const char*)X + ((size_t)t * K + k) * EB, xv);
#pragma unroll
        for (int e = 0; e < AV; ++e) {
          ssq[t] = fmaf(xv[e], xv[e], ssq[t]);
          xv[e] *= g[e];
        }
#pragma unroll
        for (int e = 0; e < AV; e += 4)
          *(float4*)(xs + (size_t)t * K + k + e) = make_float4(xv[e], xv[e + 1], xv[e + 2], xv[e + 3]);
      }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float w = wave_sum(ssq[t]);
      if (lane == 0) red[t][wave] = w;
    }
  } else if constexpr (XS16) {
    for (int r = 0; r < NR; ++r) {
      const uint16_t* xr = (const uint16_t*)rp.x[r];
      uint16_t* xd = xs16 + (size_t)r * NT * K;
      for (int i = tid * 8; i < NT * K; i += 256 * 8) *(uint4*)(xd + i) = *(const uint4*)(xr + i);
    }
  } else {
    for (int r = 0; r < NR; ++r) {
      const char* xr = (const char*)(ALLR ? rp.x[r] : X);
      float* xd = xs + (size_t)r * NT * K;
      for (int i = tid * AV; i < NT * K; i += 256 * AV)
        Vec16<AT>::load(xr + (size_t)i * (AT == ACT_F32 ? 4 : 2), xd + i);
    }
  }
  // Eight staged values of row `row` (rank-major) from element e0, as fp32.
  auto xget8 = [&](size_t e0, float* v) {
    if constexpr (XS16) {
      const uint4 u = *(const uint4*)(xs16 + e0);
      const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w4[i] << 16);
        v[2 * i + 1] = __uint_as_float(w4[i] & 0xffff0000u);
      }
    } else {
      const float4 a = *(const float4*)(xs + e0), b = *(const float4*)(xs + e0 + 4);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
  };
  __syncthreads();
  float inv[PRO ? NT : 1];
  if constexpr (PRO) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float tot = (red[t][0] + red[t][1]) + (red[t][2] + red[t][3]);
      inv[t] = 1.0f / sqrtf(tot / (float)K + fa.eps);
    }
    if (fa.normed_out != nullptr && blockIdx.x == 0) {  // the normed rows, for the caller
#pragma unroll
      for (int t = 0; t < NT; ++t)
        for (int k = tid; k < K; k += 256) {
          // (Q8_0 staged fp16: gamma * x again from its inputs, in the same fp32 product.)
          const float v = WT == W_Q8 ? ld_act<AT>(X, (size_t)t * K + k) * ld_act<AT>(fa.gamma, k)
                                     : xs[(size_t)t * K + k];
          st_act<AT>(fa.normed_out, (size_t)t * K + k, v * inv[t]);
        }
    }
  }
  if (!ALLR && !active) return;

  float acc[R][NT];
  // EPI_RED_ALL*: every rank's partial of this workgroup's rows, for the rank-ordered sum.
  __shared__ float s_part[ALLR ? kMaxRanks : 1][ALLR ? 2 : 1][ALLR ? R : 1][ALLR ? NT : 1];
  // EPI_RED_ALL* (at most four ranks): each wave serves exactly one rank, rk0.
  if (!ALLR || active) {
  const int rk = rk0;
  const float* const xsr = xs + (size_t)rk * NT * K;
#pragma unroll
  for (int s = 0; s < R; ++s)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[s][t] = 0.f;

  for (int c0 = 0; c0 < nch; c0 += 64 * U) {
    if (c0 > 0) load_batch(c0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * 64 + lane;
      if (c < nch) {
#pragma unroll
        for (int s = 0; s < R; ++s) {
          if constexpr (WT == W_Q8) {
            // Codes as fp16 1152 + c, two per word: sign bits flipped, then each byte under 0x64.
            const uint32_t r4[4] = {b[s][u].x ^ 0x80808080u, b[s][u].y ^ 0x80808080u,
                                    b[s][u].z ^ 0x80808080u, b[s][u].w ^ 0x80808080u};
            q8h2 wh[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              wh[2 * i] = __builtin_bit_cast(q8h2, __builtin_amdgcn_perm(0x64646464u, r4[i], 0x04010400u));
              wh[2 * i + 1] =
                  __builtin_bit_cast(q8h2, __builtin_amdgcn_perm(0x64646464u, r4[i], 0x04030402u));
            }
#pragma unroll
            for (int t = 0; t < NT; ++t) {
              const size_t e0 = ((size_t)rk * NT + t) * K + (size_t)c * 16;
              const uint4 xa = *(const uint4*)(xh + e0), xb = *(const uint4*)(xh + e0 + 8);
              const uint32_t xw[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
              float d = 0.f;
#pragma unroll
              for (int i = 0; i < 8; ++i)
                d = __builtin_amdgcn_fdot2(wh[i], __builtin_bit_cast(q8h2, xw[i]), d, false);
              const float2 m = xc[((size_t)rk * NT + t) * nch + c];
              acc[s][t] = fmaf(sc[s][u], fmaf(d, m.y, -m.x), acc[s][t]);
            }
          } else {
            float f[VE];
            decode_chunk<WT>(b[s][u], sc[s][u], f);
#pragma unroll
            for (int t = 0; t < NT; ++t) {
              if constexpr (XS16) {
                float xv[8];  // VE == 8: bf16 weights
                xget8(((size_t)rk * NT + t) * K + (size_t)c * VE, xv);
#pragma unroll
                for (int e = 0; e < VE; ++e) acc[s][t] = fmaf(f[e], xv[e], acc[s][t]);
              } else {
                const float* xp = xsr + t * K + c * VE;
#pragma unroll
                for (int e = 0; e < VE; e += 4) {
                  const float4 xv = *(const float4*)(xp + e);
                  acc[s][t] = fmaf(f[e], xv.x, acc[s][t]);
                  acc[s][t] = fmaf(f[e + 1], xv.y, acc[s][t]);
                  acc[s][t] = fmaf(f[e + 2], xv.z, acc[s][t]);
                  acc[s][t] = fmaf(f[e + 3], xv.w, acc[s][t]);
                }
              }
            }
          }
        }
      }
    }
  }
#pragma unroll
  for (int s = 0; s < R; ++s)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[s][t] = wave_sum(acc[s][t]);
  if constexpr (ALLR) {
    // Rank rk's partial at its stored precision: to memory (lane t stores token t) and to LDS.
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int s = 0; s < R; ++s) {
        float p = acc[s][t];
        if constexpr (EPI == EPI_RED_ALL_BF) p = bf16_to_f32(f32_to_bf16(p));
        if (lane == t && ok[s]) {
          const size_t idx = (size_t)t * ldy + row[s];
          if constexpr (EPI == EPI_RED_ALL_BF) ((uint16_t*)rp.y[rk])[idx] = f32_to_bf16(p);
          else ((float*)rp.y[rk])[idx] = p;
        }
        if (lane == 0) s_part[rk][wave / WPR][s][t] = p;
      }
    }
  }
  }  // the wave's rank
  float tot[ALLR ? R : 1][ALLR ? NT : 1];  // EPI_RED_ALL*: ((P_0 + P_1) + ...) + P_{N-1}
  if constexpr (ALLR) {
    __syncthreads();
    if (!active || wave % WPR != 0) return;
#pragma unroll
    for (int s = 0; s < R; ++s)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        tot[s][t] = s_part[0][wave / WPR][s][t];
        for (int r = 1; r < NR; ++r) tot[s][t] += s_part[r][wave / WPR][s][t];
      }
  }
  if constexpr (PRO) {
#pragma unroll
    for (int s = 0; s < R; ++s)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[s][t] *= inv[t];
  }

  // Lane t stores token t's results.
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (lane != t) continue;
    const size_t yo = (size_t)t * ldy;
    if constexpr (EPI == EPI_GATED) {
#pragma unroll
      for (int s = 0; s < R; s += 2)
        if (ok[s]) st_act<AT>(Y, yo + row[s], gated<ACTF>(acc[s][t], acc[s + 1][t]));
    } else if constexpr (EPI == EPI_F32) {
#pragma unroll
      for (int s = 0; s < R; ++s)
        if (ok[s]) ((float*)Y)[yo + row[s]] = acc[s][t];
    } else if constexpr (RED) {
      auto part = [&](uint32_t raw) {
        return EPI == EPI_REDUCE_BF ? bf16_to_f32(raw) : __uint_as_float(raw);
      };
#pragma unroll
      for (int s = 0; s < R; ++s) {
        if (!ok[s]) continue;
        const size_t idx = yo + row[s];
        float p = acc[s][t];
        if constexpr (EPI == EPI_REDUCE_BF) {
          const uint16_t b = f32_to_bf16(p);
          ((uint16_t*)Y)[idx] = b;
          p = bf16_to_f32(b);
        } else {
          ((float*)Y)[idx] = p;
        }
        // ((P_0 + P_1) + ...) + P_last, then the residual: the reduce kernel's order.
        float sum = p;
        if (fa.n_prev > 0) {
          sum = part(e_prev[s][0]);
#pragma unroll
          for (int k = 1; k < PV; ++k)
            if (k < fa.n_prev) sum += part(e_prev[s][k]);
          sum += p;
        }
        const float res = AT == ACT_F32 ? __uint_as_float(e_res[s]) : bf16_to_f32(e_res[s]);
        st_act<AT>(fa.res_out, idx, res + sum);
      }
    } else if constexpr (ALLR) {
#pragma unroll
      for (int s = 0; s < R; ++s) {
        if (!ok[s]) continue;
        const float res = AT == ACT_F32 ? __uint_as_float(e_res[s]) : bf16_to_f32(e_res[s]);
        st_act<AT>(fa.res_out, yo + row[s], res + tot[s][t]);
      }
    } else if constexpr (EPI == EPI_BF16 || EPI == EPI_ACT) {
#pragma unroll
      for (int s = 0; s < R; ++s)
        if (ok[s]) st_act<EPI == EPI_BF16 ? ACT_BF16 : AT>(Y, yo + row[s], acc[s][t]);
    } else if constexpr (EPI == EPI_ROPE) {
      const int tok = re.t0 + t;
      const int pos = e_pos[t], page = e_page[t];
#pragma unroll
      for (int s = 0; s < R; s += 2) {
        if (!ok[s]) continue;
        const int p = w * (R / 2) + s / 2;
        const int head = p / half, i = p % half;
        const float a = acc[s][t], bv = acc[s + 1][t];
        if (head < re.hq + re.hk) {
          const float2 cs = e_cs[s / 2][t];
          const float ra = a * cs.x - bv * cs.y, rb = bv * cs.x + a * cs.y;
          if (head < re.hq) {
            const size_t dq = (size_t)tok * re.hq * re.hd + (size_t)head * re.hd + i;
            st_act<AT>(re.q_out, dq, ra);
            st_act<AT>(re.q_out, dq + half, rb);
          } else {
            const size_t dk =
                (((size_t)page * re.hk + (head - re.hq)) * re.ps + pos % re.ps) * re.hd + i;
            st_act<AT>(re.k_pages, dk, ra);
            st_act<AT>(re.k_pages, dk + half, rb);
          }
        } else {
          // V pages are stored transposed: [page][kv head][hd][slot].
          const size_t dv = ((size_t)page * re.hk + (head - re.hq - re.hk)) * re.hd + i;
          const int slot = pos % re.ps;
          st_act<AT>(re.v_pages, dv * re.ps + slot, a);
          st_act<AT>(re.v_pages, (dv + half) * re.ps + slot, bv);
        }
      }
    }
  }
}

template <int WT, int AT, int EPI, int NT, int ACTF, int R, bool PRO, int PV>
static hipError_t gemv_launch(dim3 g, size_t lds, const void* W, const uint16_t* S, int K,
                              int n_out, int gate_off, const void* X, void* Y, int ldy,
                              const RopeEpi& re, const FuseArgs& fa, const RankPtrs& rp,
                              hipStream_t st) {
  // (Q8_0 with 64 KB of staged tokens goes past the default dynamic-LDS limit.)
  if (lds > 65536) {
    hipError_t ea = allow_lds((const void*)k_gemv<WT, AT, EPI, NT, ACTF, R, PRO, PV>, (int)lds);
    if (ea != hipSuccess) return ea;
  }
  launch((k_gemv<WT, AT, EPI, NT, ACTF, R, PRO, PV>), g, dim3(256), (uint32_t)lds, st, W, S, K,
         n_out, gate_off, X, Y, ldy, re, fa, rp);
  return hipGetLastError();
}

// The kernel variant for the fusion arguments: the norm prologue only for the projections that
// consume the normed state, the reduce epilogues sized to the number of earlier partials.
template <int WT, int AT, int EPI, int NT, int ACTF, int R>
static hipError_t gemv_variant(dim3 g, size_t lds, const void* W, const uint16_t* S, int K,
                               int n_out, int gate_off, const void* X, void* Y, int ldy,
                               const RopeEpi& re, const FuseArgs& fa, const RankPtrs& rp, hipStream_t st) {
  // (EPI_F32 with the prologue: the MoE router on the block's residual stream.)
  constexpr bool CAN_PRO = (EPI == EPI_ROPE || EPI == EPI_GATED || EPI == EPI_F32);
  constexpr bool RED = (EPI == EPI_REDUCE || EPI == EPI_REDUCE_BF);
  if constexpr (CAN_PRO) {
    if (fa.gamma)
      return gemv_launch<WT, AT, EPI, NT, ACTF, R, true, 1>(g, lds, W, S, K, n_out, gate_off, X,
                                                             Y, ldy, re, fa, rp, st);
  } else if (fa.gamma) {
    return hipErrorInvalidValue;
  }
  if constexpr (RED) {
    if (fa.n_prev > 3)
      return gemv_launch<WT, AT, EPI, NT, ACTF, R, false, 7>(g, lds, W, S, K, n_out, gate_off, X,
                                                              Y, ldy, re, fa, rp, st);
    if (fa.n_prev > 1)
      return gemv_launch<WT, AT, EPI, NT, ACTF, R, false, 3>(g, lds, W, S, K, n_out, gate_off, X,
                                                              Y, ldy, re, fa, rp, st);
  }
  return gemv_launch<WT, AT, EPI, NT, ACTF, R, false, 1>(g, lds, W, S, K, n_out, gate_off, X, Y,
                                                          ldy, re, fa, rp, st);
}

template <int WT, int AT, int EPI, int ACTF, int R>
static hipError_t gemv_nt(int nt, const void* W, const uint16_t* S, int K, int n_out, int gate_off,
                          const void* X, void* Y, int ldy, const RopeEpi& re, const FuseArgs& fa,
                          const RankPtrs& rp, hipStream_t st) {
  int waves;
  if constexpr (EPI == EPI_GATED) waves = (n_out + R / 2 - 1) / (R / 2);
  else if constexpr (EPI == EPI_ROPE) waves = (n_out / 2 + R / 2 - 1) / (R / 2);
  else waves = (n_out + R - 1) / R;
  constexpr bool ALLR = (EPI == EPI_RED_ALL || EPI == EPI_RED_ALL_BF);
  // Column-parallel launches over all ranks repeat the grid once per rank; the row-parallel
  // EPI_RED_ALL* launches stage every rank's inputs.
  const int nr = rp.n > 1 ? rp.n : 1;
  // EPI_RED_ALL*: each row group takes min(N, 4) waves, 4 / min(N, 4) row groups per block.
  const int rw = 4 / (nr < 4 ? nr : 4);
  const int bpr = ALLR ? (waves + rw - 1) / rw : (waves + 3) / 4;
  const dim3 g(ALLR ? bpr : bpr * nr);
  // (EPI_RED_ALL* with bf16 rows keeps them as bf16; Q8_0 stages fp16 rows and a pair of floats
  // per 16 values.)
  const size_t xb = (ALLR && AT == ACT_BF16) ? 2 : sizeof(float);
  const size_t lds = (size_t)(ALLR ? nr : 1) *
                     (WT == W_Q8 ? (size_t)nt * K * 2 + (size_t)nt * (K / 16) * 8
                                 : (size_t)nt * K * xb);
  RankPtrs rq = rp;
  rq.bpr = bpr;
  switch (nt) {
    case 1:
      return gemv_variant<WT, AT, EPI, 1, ACTF, R>(g, lds, W, S, K, n_out, gate_off, X, Y, ldy,
                                                    re, fa, rq, st);
    case 2:
      return gemv_variant<WT, AT, EPI, 2, ACTF, R>(g, lds, W, S, K, n_out, gate_off, X, Y, ldy,
                                                    re, fa, rq, st);
    case 3:
      return gemv_variant<WT, AT, EPI, 3, ACTF, R>(g, lds, W, S, K, n_out, gate_off, X, Y, ldy,
                                                    re, fa, rq, st);
    case 4:
      return gemv_variant<WT, AT, EPI, 4, ACTF, R>(g, lds, W, S, K, n_out, gate_off, X, Y, ldy,
                                                    re, fa, rq, st);
  }
  return hipErrorInvalidValue;
}

template <int WT, int AT, int EPI, int ACTF>
static hipError_t gemv_r(int r, int nt, const void* W, const uint16_t* S, int K, int n_out,
                         int gate_off, const void* X, void* Y, int ldy, const RopeEpi& re,
                         const FuseArgs& fa, const RankPtrs& rp, hipStream_t st) {
  constexpr bool PAIRED = (EPI == EPI_GATED || EPI == EPI_ROPE);
  switch (r) {
    case 1:
      if constexpr (!PAIRED)
        return gemv_nt<WT, AT, EPI, ACTF, 1>(nt, W, S, K, n_out, gate_off, X, Y, ldy, re, fa, rp, st);
      return hipErrorInvalidValue;
    case 2: return gemv_nt<WT, AT, EPI, ACTF, 2>(nt, W, S, K, n_out, gate_off, X, Y, ldy, re, fa, rp, st);
    case 4: return gemv_nt<WT, AT, EPI, ACTF, 4>(nt, W, S, K, n_out, gate_off, X, Y, ldy, re, fa, rp, st);
    case 8: return gemv_nt<WT, AT, EPI, ACTF, 8>(nt, W, S, K, n_out, gate_off, X, Y, ldy, re, fa, rp, st);
  }
  return hipErrorInvalidValue;
}

// All epilogues for one weight / activation format (one translation unit per format).
template <int WT, int AT>
hipError_t gemv_format(int epi, int actf, int nt, const void* W, const uint16_t* S, int K,
                       int n_out, int gate_off, const void* X, void* Y, int ldy, const RopeEpi& re,
                       const FuseArgs& fa, const RankPtrs& rp, hipStream_t st) {
  const int nch = K / WFmt<WT>::VE;
  const bool paired = (epi == EPI_GATED || epi == EPI_ROPE);
  // (EPI_RED_ALL*: a row group takes one wave per rank, up to four.)
  const long wrows = (epi == EPI_RED_ALL || epi == EPI_RED_ALL_BF)
                         ? (long)n_out * (rp.n < 4 ? (rp.n > 1 ? rp.n : 1) : 4)
                         : (epi == EPI_GATED ? 2L * n_out : (long)n_out);
  int r = gemv_rows_per_wave(nch, paired, wrows);
  // Two ranks' row-parallel launch of 16-bit or Q8_0 weights: two rows per wave. Every workgroup
  // stages both ranks' input rows, so fewer, larger workgroups stage less; two rows measured best
  // or level on the 8B-shaped down (K 7168: 22.9 -> 20.5 us with one row) and o_proj and the
  // Gemma-like Q8_0 down and o_proj.
  if ((epi == EPI_RED_ALL || epi == EPI_RED_ALL_BF) && rp.n == 2 && WT != W_F32) r = 2;
  switch (epi) {
    case EPI_F32:
      return gemv_r<WT, AT, EPI_F32, 0>(r, nt, W, S, K, n_out, gate_off, X, Y, ldy, re, fa, rp, st);
    case EPI_BF16:
      return gemv_r<WT, AT, EPI_BF16, 0>(r, nt, W, S, K, n_out, gate_off, X, Y, ldy, re, fa, rp, st);
    case EPI_ACT:
      return gemv_r<WT, AT, EPI_ACT, 0>(r, nt, W, S, K, n_out, gate_off, X, Y, ldy, re, fa, rp, st);
    case EPI_REDUCE:
      return gemv_r<WT, AT, EPI_REDUCE, 0>(r, nt, W, S, K, n_out, gate_off, X, Y, ldy, re, fa, rp, st);
    case EPI_REDUCE_BF:
      return gemv_r<WT, AT, EPI_REDUCE_BF, 0>(r, nt, W, S, K, n_out, gate_off, X, Y, ldy, re, fa, rp,
                                              st);
    case EPI_RED_ALL:
      return gemv_r<WT, AT, EPI_RED_ALL, 0>(r, nt, W, S, K, n_out, gate_off, X, Y, ldy, re, fa, rp,
                                            st);
    case EPI_RED_ALL_BF:
      return gemv_r<WT, AT, EPI_RED_ALL_BF, 0>(r, nt, W, S, K, n_out, gate_off, X, Y, ldy, re, fa,
                                               rp, st);
    case EPI_ROPE:
      return gemv_r<WT, AT, EPI_ROPE, 0>(r, nt, W, S, K, n_out, gate_off, X, Y, ldy, re, fa, rp, st);
    case EPI_GATED:
      if (actf == 0)
        return gemv_r<WT, AT, EPI_GATED, 0>(r, nt, W, S, K, n_out, gate_off, X, Y, ldy, re, fa, rp, st);
      return gemv_r<WT, AT, EPI_GATED, 1>(r, nt, W, S, K, n_out, gate_off, X, Y, ldy, re, fa, rp, st);
  }
  return hipErrorInvalidValue;
}

hipError_t gemv_f32(int epi, int actf, int nt, const void* W, const uint16_t* S, int K, int n_out,
                    int gate_off, const void* X, void* Y, int ldy, const RopeEpi& re,
                    const FuseArgs& fa, const RankPtrs& rp,
                    hipStream_t st);
hipError_t gemv_bf16(int epi, int actf, int nt, const void* W, const uint16_t* S, int K, int n_out,
                     int gate_off, const void* X, void* Y, int ldy, const RopeEpi& re,
                    const FuseArgs& fa, const RankPtrs& rp,
                     hipStream_t st);
hipError_t gemv_q8(int epi, int actf, int nt, const void* W, const uint16_t* S, int K, int n_out,
                   int gate_off, const void* X, void* Y, int ldy, const RopeEpi& re,
                    const FuseArgs& fa, const RankPtrs& rp,
                   hipStream_t st);

}  // namespace tpk
