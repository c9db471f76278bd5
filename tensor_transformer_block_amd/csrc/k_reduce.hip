// K7: the local copy-and-reduce step that replaces the cross-GPU all-reduce on one device
// (mlxcel issue #488, "Problem": ranks run in sequence and their partials are summed locally;
// TensorSharp "How tensor parallelism works", step 3: the reduce leaves the identical hidden
// state on every rank), fused with the residual add and the replicated RMSNorm that follows it.
//
// One workgroup per token row; each thread owns up to MAXC chunks of 8 features, kept in
// registers between the sum and the normalisation, so the row is read and written once.
// Summation order is fixed: ((P_0 + P_1) + ...) + P_{n-1} in fp32, then + residual, then a single
// rounding to the activation dtype. The norm is computed from the stored (rounded) residual.
#include "tp_common.h"
#include "tp_kernels.h"

namespace tpk {

template <int T>
__device__ __forceinline__ void load8(const void* base, size_t idx, float* v) {
  if constexpr (T == ACT_F32) {
    Vec16<ACT_F32>::load((const float*)base + idx, v);
    Vec16<ACT_F32>::load((const float*)base + idx + 4, v + 4);
  } else {
    Vec16<ACT_BF16>::load((const uint16_t*)base + idx, v);
  }
}

// The partials are read exactly once: streaming (non-temporal) loads keep them from displacing
// the residual and the weights in the caches and measure faster on large reads.
template <int T>
__device__ __forceinline__ void load8_stream(const void* base, size_t idx, float* v) {
  if constexpr (T == ACT_F32) {
    const uint4 a = ld_stream16((const float*)base + idx), b = ld_stream16((const float*)base + idx + 4);
    v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y);
    v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
    v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y);
    v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
  } else {
    const uint4 a = ld_stream16((const uint16_t*)base + idx);
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
}

template <int T>
__device__ __forceinline__ void store8(void* base, size_t idx, const float* v) {
  if constexpr (T == ACT_F32) {
    float4* p = (float4*)((float*)base + idx);
    p[0] = make_float4(v[0], v[1], v[2], v[3]);
    p[1] = make_float4(v[4], v[5], v[6], v[7]);
  } else {
    uint4 o;
    o.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
    o.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
    o.z = (uint32_t)f32_to_bf16(v[4]) | ((uint32_t)f32_to_bf16(v[5]) << 16);
    o.w = (uint32_t)f32_to_bf16(v[6]) | ((uint32_t)f32_to_bf16(v[7]) << 16);
    *(uint4*)((uint16_t*)base + idx) = o;
  }
}

template <int T>
__device__ __forceinline__ float round_to(float v) {
  if constexpr (T == ACT_F32) return v;
  else return bf16_to_f32(f32_to_bf16(v));
}

// Up to kPre partials per chunk are loaded before any is added, so their latencies overlap;
// the sum is still taken strictly in rank order.
constexpr int kPre = 8;

template <int AT, int PT, int MAXC>
__global__ __launch_bounds__(256) void k_partial_reduce(int d, const void* __restrict__ partials,
                                                        int n_part, size_t part_stride,
                                                        const void* res_in, void* res_out,
                                                        const void* __restrict__ gamma,
                                                        void* __restrict__ normed, float eps) {
  __shared__ float red[4];
  const int t = blockIdx.x, tid = threadIdx.x;
  const int nchunk = d >> 3;
  const size_t row = (size_t)t * d;
  float v[MAXC][8], gm[MAXC][8];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int ci = tid + c * 256;
    if (ci < nchunk) {
      const size_t idx = row + (size_t)ci * 8;
      float r[8];
      load8<AT>(res_in, idx, r);
      if (gamma != nullptr) load8<AT>(gamma, (size_t)ci * 8, gm[c]);
      if (n_part > 0) {
        float p[kPre][8];
#pragma unroll
        for (int k = 0; k < kPre; ++k)
          if (k < n_part) load8_stream<PT>(partials, (size_t)k * part_stride + idx, p[k]);
        float sum[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) sum[e] = p[0][e];
#pragma unroll
        for (int k = 1; k < kPre; ++k)
          if (k < n_part) {
#pragma unroll
            for (int e = 0; e < 8; ++e) sum[e] += p[k][e];
          }
        for (int k = kPre; k < n_part; ++k) {
          float q[8];
          load8_stream<PT>(partials, (size_t)k * part_stride + idx, q);
#pragma unroll
          for (int e = 0; e < 8; ++e) sum[e] += q[e];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) r[e] = round_to<AT>(r[e] + sum[e]);
        store8<AT>(res_out, idx, r);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[c][e] = r[e];
        ss += r[e] * r[e];
      }
    }
  }
  if (gamma == nullptr) return;
  ss = wave_sum(ss);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  const float tot = (red[0] + red[1]) + (red[2] + red[3]);
  const float inv = 1.0f / sqrtf(tot / (float)d + eps);
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int ci = tid + c * 256;
    if (ci < nchunk) {
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = gm[c][e] * (v[c][e] * inv);
      store8<AT>(normed, row + (size_t)ci * 8, o);
    }
  }
}

template <int AT, int PT>
static hipError_t launch_reduce_t(int T, int d, const void* partials, int n, const void* res_in,
                                  void* res_out,
                                  const void* gamma, void* normed, float eps, hipStream_t st) {
  const int nchunk = d / 8;
  const int maxc = (nchunk + 255) / 256;
  const size_t stride = (size_t)T * d;
  dim3 g(T), b(256);
#define TPK_RED(MC)                                                                          \
  hipLaunchKernelGGL((k_partial_reduce<AT, PT, MC>), g, b, 0, st, d, partials, n, stride, \
                     res_in, res_out, gamma, normed, eps)
  switch (maxc) {
    case 1: TPK_RED(1); break;
    case 2: TPK_RED(2); break;
    case 3: TPK_RED(3); break;
    case 4: TPK_RED(4); break;
    case 5: TPK_RED(5); break;
    case 6: TPK_RED(6); break;
    case 7: TPK_RED(7); break;
    case 8: TPK_RED(8); break;
    default: return hipErrorInvalidValue;
  }
#undef TPK_RED
  return hipGetLastError();
}

hipError_t launch_partial_reduce(int act, int part, int T, int d, const void* partials, int n,
                                 const void* res_in, void* res_out, const void* gamma,
                                 void* normed, float eps, hipStream_t st) {
  if (act == ACT_F32 && part == ACT_F32)
    return launch_reduce_t<ACT_F32, ACT_F32>(T, d, partials, n, res_in, res_out, gamma, normed, eps, st);
  if (act == ACT_F32 && part == ACT_BF16)
    return launch_reduce_t<ACT_F32, ACT_BF16>(T, d, partials, n, res_in, res_out, gamma, normed, eps, st);
  if (act == ACT_BF16 && part == ACT_F32)
    return launch_reduce_t<ACT_BF16, ACT_F32>(T, d, partials, n, res_in, res_out, gamma, normed, eps, st);
  return launch_reduce_t<ACT_BF16, ACT_BF16>(T, d, partials, n, res_in, res_out, gamma, normed, eps, st);
}

}  // namespace tpk
