// K2 / K3: decode projections, y[t, o] = sum_k x[t, k] W[o, k], for a handful of tokens.
//
// Decode reads every byte of a rank's 1/N weight slice once per step and does ~1 FLOP per byte,
// so these kernels are HBM-streaming GEMVs, not GEMMs: each wavefront owns two weight rows and
// streams them with 16-byte loads, eight loads per row in flight per lane; the first batch of loads
// is issued before the token vectors are staged in LDS (as fp32), so the two latencies overlap; a
// cross-lane sum finishes each dot product.
//
// Weight formats: fp32, bf16, and Q8_0 split into an int8 code plane [out, in] plus an fp16 scale
// plane [out, in/32] (dequantised in registers, exactly, by q8_dequant).
// Epilogues:
//   EPI_ACT   store in the activation dtype;
//   EPI_F32 / EPI_BF16   store a partial sum (row-parallel o_proj and down, TensorSharp "How
//             tensor parallelism works", step 3);
//   EPI_GATED act(g) * u of the column-parallel gate/up pair (rows o and o + gate_off);
//   EPI_ROPE  the fused QKV epilogue: a wavefront owns rows i and i + hd/2 of one head, so it
//             applies the rotary embedding to q and k in registers, stores q, and appends k and v
//             to the rank's paged cache (step 2 of the same section: the rank's own KV cache).
#include "tp_common.h"
#include "tp_kernels.h"

namespace tpk {

template <int WT> struct WFmt;
template <> struct WFmt<W_F32> { static constexpr int VE = 4, WB = 4; };
template <> struct WFmt<W_BF16> { static constexpr int VE = 8, WB = 2; };
template <> struct WFmt<W_Q8> { static constexpr int VE = 16, WB = 1; };

// Decode one 16-byte weight chunk into VE fp32 values.
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

constexpr int GEMV_UNROLL = 8;

__device__ __forceinline__ int clampi_g(int v, int lo, int hi) {
  return v < lo ? lo : (v > hi ? hi : v);
}

template <int WT, int AT, int EPI, int NT, int ACTF>
__global__ __launch_bounds__(256) void k_gemv(const void* __restrict__ W,
                                              const uint16_t* __restrict__ S, int K, int n_out,
                                              int gate_off, const void* __restrict__ X,
                                              void* __restrict__ Y, int ldy, RopeEpi re) {
  extern __shared__ float xs[];  // [NT][K]
  constexpr int VE = WFmt<WT>::VE;
  constexpr int WB = WFmt<WT>::WB;
  constexpr int AV = Vec16<AT>::N;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // Rows of this wavefront.
  const int w = blockIdx.x * 4 + wave;
  int r0, r1;
  bool active, v1 = true;
  if constexpr (EPI == EPI_GATED) {
    active = w < n_out;
    r0 = w;
    r1 = w + gate_off;
  } else if constexpr (EPI == EPI_ROPE) {
    const int half = re.hd >> 1;
    active = w < (n_out >> 1);
    r0 = (w / half) * re.hd + (w % half);
    r1 = r0 + half;
  } else {
    r0 = 2 * w;
    active = r0 < n_out;
    r1 = r0 + 1;
    v1 = r1 < n_out;
    if (!v1) r1 = r0;
  }
  if (!active) r0 = r1 = 0;  // loads stay in bounds; results are dropped
  const int nch = K / VE;
  const char* w0 = (const char*)W + (size_t)r0 * K * WB;
  const char* w1 = (const char*)W + (size_t)r1 * K * WB;
  const uint16_t* s0 = S + (size_t)r0 * (K / 32);
  const uint16_t* s1 = S + (size_t)r1 * (K / 32);

  uint4 b0[GEMV_UNROLL], b1[GEMV_UNROLL];
  float sc0[GEMV_UNROLL], sc1[GEMV_UNROLL];
  auto load_batch = [&](int c0) {
#pragma unroll
    for (int u = 0; u < GEMV_UNROLL; ++u) {
      const int c = c0 + u * 64 + lane;
      if (c < nch) {
        b0[u] = ld_stream16(w0 + (size_t)c * 16);
        b1[u] = ld_stream16(w1 + (size_t)c * 16);
        if constexpr (WT == W_Q8) {
          sc0[u] = f16_to_f32(s0[c >> 1]);
          sc1[u] = f16_to_f32(s1[c >> 1]);
        } else {
          sc0[u] = sc1[u] = 0.f;
        }
      } else {
        b0[u] = b1[u] = make_uint4(0, 0, 0, 0);
        sc0[u] = sc1[u] = 0.f;
      }
    }
  };
  load_batch(0);  // in flight while the token vectors are staged

  for (int i = tid * AV; i < NT * K; i += 256 * AV)
    Vec16<AT>::load((const char*)X + (size_t)i * (AT == ACT_F32 ? 4 : 2), xs + i);
  __syncthreads();
  if (!active) return;

  float acc0[NT], acc1[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc0[t] = acc1[t] = 0.f;

  for (int c0 = 0; c0 < nch; c0 += 64 * GEMV_UNROLL) {
    if (c0 > 0) load_batch(c0);
#pragma unroll
    for (int u = 0; u < GEMV_UNROLL; ++u) {
      const int c = c0 + u * 64 + lane;
      if (c < nch) {
        float f0[VE], f1[VE];
        decode_chunk<WT>(b0[u], sc0[u], f0);
        decode_chunk<WT>(b1[u], sc1[u], f1);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const float* xp = xs + t * K + c * VE;
#pragma unroll
          for (int e = 0; e < VE; e += 4) {
            const float4 xv = *(const float4*)(xp + e);
            acc0[t] = fmaf(f0[e], xv.x, acc0[t]);
            acc0[t] = fmaf(f0[e + 1], xv.y, acc0[t]);
            acc0[t] = fmaf(f0[e + 2], xv.z, acc0[t]);
            acc0[t] = fmaf(f0[e + 3], xv.w, acc0[t]);
            acc1[t] = fmaf(f1[e], xv.x, acc1[t]);
            acc1[t] = fmaf(f1[e + 1], xv.y, acc1[t]);
            acc1[t] = fmaf(f1[e + 2], xv.z, acc1[t]);
            acc1[t] = fmaf(f1[e + 3], xv.w, acc1[t]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    acc0[t] = wave_sum(acc0[t]);
    acc1[t] = wave_sum(acc1[t]);
  }
  // Lane t stores token t's results.
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (lane != t) continue;
    const size_t yo = (size_t)t * ldy;
    if constexpr (EPI == EPI_GATED) {
      st_act<AT>(Y, yo + w, gated<ACTF>(acc0[t], acc1[t]));
    } else if constexpr (EPI == EPI_ACT) {
      st_act<AT>(Y, yo + r0, acc0[t]);
      if (v1) st_act<AT>(Y, yo + r1, acc1[t]);
    } else if constexpr (EPI == EPI_F32) {
      ((float*)Y)[yo + r0] = acc0[t];
      if (v1) ((float*)Y)[yo + r1] = acc1[t];
    } else if constexpr (EPI == EPI_BF16) {
      ((uint16_t*)Y)[yo + r0] = f32_to_bf16(acc0[t]);
      if (v1) ((uint16_t*)Y)[yo + r1] = f32_to_bf16(acc1[t]);
    } else {  // EPI_ROPE
      const int tok = re.t0 + t;
      const int half = re.hd >> 1;
      const int head = w / half, i = w % half;
      const int pos = clampi_g(re.positions[tok], 0, re.pos_limit - 1);
      const float a = acc0[t], b = acc1[t];
      if (head < re.hq + re.hk) {
        const float2 cs = ((const float2*)re.rope)[(size_t)pos * half + i];
        const float ra = a * cs.x - b * cs.y, rb = b * cs.x + a * cs.y;
        if (head < re.hq) {
          const size_t dq = (size_t)tok * re.hq * re.hd + (size_t)head * re.hd + i;
          st_act<AT>(re.q_out, dq, ra);
          st_act<AT>(re.q_out, dq + half, rb);
        } else {
          const int seq = (re.mode == 0) ? tok : 0;
          const int page = clampi_g(re.block_table[(size_t)seq * re.max_pages + pos / re.ps], 0,
                                    re.n_pages - 1);
          const size_t dk =
              (((size_t)page * re.hk + (head - re.hq)) * re.ps + pos % re.ps) * re.hd + i;
          st_act<AT>(re.k_pages, dk, ra);
          st_act<AT>(re.k_pages, dk + half, rb);
        }
      } else {
        const int seq = (re.mode == 0) ? tok : 0;
        const int page = clampi_g(re.block_table[(size_t)seq * re.max_pages + pos / re.ps], 0,
                                  re.n_pages - 1);
        // V pages are stored transposed: [page][kv head][hd][slot].
        const size_t dv = ((size_t)page * re.hk + (head - re.hq - re.hk)) * re.hd + i;
        const int slot = pos % re.ps;
        st_act<AT>(re.v_pages, dv * re.ps + slot, a);
        st_act<AT>(re.v_pages, (dv + half) * re.ps + slot, b);
      }
    }
  }
}

template <int WT, int AT, int EPI, int ACTF>
static hipError_t gemv_nt(int nt, const void* W, const uint16_t* S, int K, int n_out, int gate_off,
                          const void* X, void* Y, int ldy, const RopeEpi& re, hipStream_t st) {
  const int waves = (EPI == EPI_GATED) ? n_out : (n_out + 1) / 2;
  dim3 g((waves + 3) / 4), b(256);
  const size_t lds = (size_t)nt * K * sizeof(float);
#define TPK_GEMV(NTV)                                                                       \
  hipLaunchKernelGGL((k_gemv<WT, AT, EPI, NTV, ACTF>), g, b, lds, st, W, S, K, n_out,      \
                     gate_off, X, Y, ldy, re)
  switch (nt) {
    case 1: TPK_GEMV(1); break;
    case 2: TPK_GEMV(2); break;
    case 3: TPK_GEMV(3); break;
    case 4: TPK_GEMV(4); break;
    default: return hipErrorInvalidValue;
  }
#undef TPK_GEMV
  return hipGetLastError();
}

template <int WT, int AT>
static hipError_t gemv_epi(int epi, int actf, int nt, const void* W, const uint16_t* S, int K,
                           int n_out, int gate_off, const void* X, void* Y, int ldy,
                           const RopeEpi& re, hipStream_t st) {
  switch (epi) {
    case EPI_ACT:
      return gemv_nt<WT, AT, EPI_ACT, 0>(nt, W, S, K, n_out, gate_off, X, Y, ldy, re, st);
    case EPI_F32:
      return gemv_nt<WT, AT, EPI_F32, 0>(nt, W, S, K, n_out, gate_off, X, Y, ldy, re, st);
    case EPI_BF16:
      return gemv_nt<WT, AT, EPI_BF16, 0>(nt, W, S, K, n_out, gate_off, X, Y, ldy, re, st);
    case EPI_ROPE:
      return gemv_nt<WT, AT, EPI_ROPE, 0>(nt, W, S, K, n_out, gate_off, X, Y, ldy, re, st);
    case EPI_GATED:
      if (actf == 0)
        return gemv_nt<WT, AT, EPI_GATED, 0>(nt, W, S, K, n_out, gate_off, X, Y, ldy, re, st);
      return gemv_nt<WT, AT, EPI_GATED, 1>(nt, W, S, K, n_out, gate_off, X, Y, ldy, re, st);
  }
  return hipErrorInvalidValue;
}

int gemv_max_tokens(int K) {
  int nt = 16384 / K;
  return nt > 4 ? 4 : nt;
}

hipError_t launch_gemv(int wt, int at, int epi, int actf, int T, const void* W, const void* S,
                       int K, int n_out, int gate_off, const void* X, void* Y, int ldy,
                       const RopeEpi* rope, hipStream_t st) {
  const int ntmax = gemv_max_tokens(K);
  if (ntmax < 1) return hipErrorInvalidValue;
  if (epi == EPI_ROPE && !rope) return hipErrorInvalidValue;
  const size_t xb = (at == ACT_F32) ? 4 : 2;
  const size_t yb = (epi == EPI_F32) ? 4 : ((epi == EPI_BF16) ? 2 : xb);
  RopeEpi re = rope ? *rope : RopeEpi{};
  for (int t0 = 0; t0 < T; t0 += ntmax) {
    const int nt = (T - t0) < ntmax ? (T - t0) : ntmax;
    const void* Xt = (const char*)X + (size_t)t0 * K * xb;
    void* Yt = (char*)Y + (size_t)t0 * ldy * yb;
    re.t0 = t0;
    hipError_t e;
    if (wt == W_F32 && at == ACT_F32)
      e = gemv_epi<W_F32, ACT_F32>(epi, actf, nt, W, (const uint16_t*)S, K, n_out, gate_off, Xt,
                                   Yt, ldy, re, st);
    else if (wt == W_BF16 && at == ACT_BF16)
      e = gemv_epi<W_BF16, ACT_BF16>(epi, actf, nt, W, (const uint16_t*)S, K, n_out, gate_off, Xt,
                                     Yt, ldy, re, st);
    else if (wt == W_Q8 && at == ACT_BF16)
      e = gemv_epi<W_Q8, ACT_BF16>(epi, actf, nt, W, (const uint16_t*)S, K, n_out, gate_off, Xt,
                                   Yt, ldy, re, st);
    else
      return hipErrorInvalidValue;
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace tpk
