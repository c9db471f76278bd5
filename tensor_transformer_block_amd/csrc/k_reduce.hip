// K7: the local copy-and-reduce step that replaces the cross-GPU all-reduce on one device
// (mlxcel issue #488, "Problem": ranks run in sequence and their partials are summed locally;
// TensorSharp "How tensor parallelism works", step 3: the reduce leaves the identical hidden
// state on every rank), fused with the residual add and the replicated RMSNorm that follows it.
//
// One workgroup per token row; each thread owns one or two chunks of 8 features, kept in
// registers between the sum and the normalisation, so the row is read and written once.
// Summation order is fixed: ((P_0 + P_1) + ...) + P_{n-1} in fp32, then + residual, then a single
// rounding to the activation dtype. The norm is computed from the stored (rounded) residual.
#include "tp_common.h"
#include "tp_kernels.h"

namespace tpk {

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

// Register image of 8 consecutive values (two 16-byte vectors of fp32 or one of bf16), loaded
// without conversion so that every load of a row can be in flight before the first is used.
template <int T>
struct Raw8 {
  uint4 v[T == ACT_F32 ? 2 : 1];
};

template <int T>
__device__ __forceinline__ void ld_raw8(const void* base, size_t idx, Raw8<T>& r) {
  if constexpr (T == ACT_F32) {
    r.v[0] = *(const uint4*)((const float*)base + idx);
    r.v[1] = *(const uint4*)((const float*)base + idx + 4);
  } else {
    r.v[0] = *(const uint4*)((const uint16_t*)base + idx);
  }
}

// The partials are read exactly once: streaming (non-temporal) loads keep them from displacing
// the residual and the weights in the caches and measure faster on large reads.
template <int T>
__device__ __forceinline__ void ld_raw8_stream(const void* base, size_t idx, Raw8<T>& r) {
  if constexpr (T == ACT_F32) {
    r.v[0] = ld_stream16((const float*)base + idx);
    r.v[1] = ld_stream16((const float*)base + idx + 4);
  } else {
    r.v[0] = ld_stream16((const uint16_t*)base + idx);
  }
}

template <int T>
__device__ __forceinline__ void unpack8(const Raw8<T>& r, float* v) {
  unpack16<T>(r.v[0], v);
  if constexpr (T == ACT_F32) unpack16<T>(r.v[1], v + 4);
}

// Partials are loaded in groups of kGroup / MAXC per chunk: a group's loads are all issued before
// any of them is added, so their latencies overlap; the sum is still taken strictly in rank order.
// Groups of four measured faster than eight on the eight-rank prefill reduce (70B step 15-40 us
// less) and level elsewhere; two were level.
constexpr int kGroup = 4;
constexpr int kMaxThreads = 1024;

// One workgroup per token row, one chunk of 8 features per thread (two when the row has more than
// 1024 chunks). Decode rows are a single workgroup whose time is memory latency, so the row's
// residual, gamma and first partial group are all requested before the first wait, and the
// stores come after the last load.
template <int AT, int PT, int MAXC>
__global__ __launch_bounds__(kMaxThreads) void k_partial_reduce(
    int d, const void* __restrict__ partials, int n_part, size_t part_stride, const void* res_in,
    void* res_out, const void* __restrict__ gamma, void* __restrict__ normed, float eps) {
  constexpr int G = kGroup / MAXC;
  __shared__ float red[kMaxThreads / 64];
  const int t = blockIdx.x, tid = threadIdx.x, nt = blockDim.x;
  const int nchunk = d >> 3;
  const size_t row = (size_t)t * d;
  float v[MAXC][8], gm[MAXC][8];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    // Threads past the row's end re-read its last chunk and store nothing.
    const int ci = min(tid + c * nt, nchunk - 1);
    const size_t idx = row + (size_t)ci * 8;
    Raw8<AT> rr, gr;
    Raw8<PT> pr[G];
    ld_raw8<AT>(res_in, idx, rr);
    if (gamma != nullptr) ld_raw8<AT>(gamma, (size_t)ci * 8, gr);
#pragma unroll
    for (int k = 0; k < G; ++k)
      if (k < n_part) ld_raw8_stream<PT>(partials, (size_t)k * part_stride + idx, pr[k]);
    unpack8<AT>(rr, v[c]);
    if (gamma != nullptr) unpack8<AT>(gr, gm[c]);
    if (n_part > 0) {
      float sum[8], q[8];
      unpack8<PT>(pr[0], sum);
#pragma unroll
      for (int k = 1; k < G; ++k)
        if (k < n_part) {
          unpack8<PT>(pr[k], q);
#pragma unroll
          for (int e = 0; e < 8; ++e) sum[e] += q[e];
        }
      for (int k0 = G; k0 < n_part; k0 += G) {
#pragma unroll
        for (int k = 0; k < G; ++k)
          if (k0 + k < n_part)
            ld_raw8_stream<PT>(partials, (size_t)(k0 + k) * part_stride + idx, pr[k]);
#pragma unroll
        for (int k = 0; k < G; ++k)
          if (k0 + k < n_part) {
            unpack8<PT>(pr[k], q);
#pragma unroll
            for (int e = 0; e < 8; ++e) sum[e] += q[e];
          }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) v[c][e] = round_to<AT>(v[c][e] + sum[e]);
    }
    if (tid + c * nt < nchunk) {
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf(v[c][e], v[c][e], ss);
    }
  }
  if (n_part > 0) {
#pragma unroll
    for (int c = 0; c < MAXC; ++c)
      if (tid + c * nt < nchunk) store8<AT>(res_out, row + (size_t)(tid + c * nt) * 8, v[c]);
  }
  if (gamma == nullptr) return;
  ss = wave_sum(ss);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
  for (int w = 0; w < (nt >> 6); ++w) tot += red[w];
  const float inv = 1.0f / sqrtf(tot / (float)d + eps);
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int ci = tid + c * nt;
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
                                  void* res_out, const void* gamma, void* normed, float eps,
                                  hipStream_t st) {
  const int nchunk = d / 8;
  const int maxc = (nchunk + kMaxThreads - 1) / kMaxThreads;
  const int threads = ((nchunk + maxc - 1) / maxc + 63) / 64 * 64;
  const size_t stride = (size_t)T * d;
  dim3 g(T), b(threads);
  if (maxc == 1)
    hipLaunchKernelGGL((k_partial_reduce<AT, PT, 1>), g, b, 0, st, d, partials, n, stride, res_in,
                       res_out, gamma, normed, eps);
  else if (maxc == 2)
    hipLaunchKernelGGL((k_partial_reduce<AT, PT, 2>), g, b, 0, st, d, partials, n, stride, res_in,
                       res_out, gamma, normed, eps);
  else
    return hipErrorInvalidValue;
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
