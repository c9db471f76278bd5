// K1: building a rank's packed shard from the full weights, and the inverse scatter used by the
// tests to prove the index maps bit-exact. One-time work, bound by HBM copies.
//
// Column-parallel slices are whole rows of the full matrix, row-parallel slices are column ranges
// of every row (TensorSharp, "How tensor parallelism works", steps 1 and 3). Q8_0 rows are split
// into a code plane (one int8 per weight, 16-byte aligned rows for vector loads) and a scale plane
// (one fp16 per 32-weight block), so the payload stays 34 bytes per 32 weights.
#include "tp_common.h"
#include "tp_kernels.h"

namespace tpk {

template <typename U>
__global__ void k_copy2d(char* __restrict__ dst, size_t dst_ld, const char* __restrict__ src,
                         size_t src_ld, int64_t rows, int64_t units_per_row) {
  const int64_t total = rows * units_per_row;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / units_per_row, c = i - r * units_per_row;
    *(U*)(dst + r * dst_ld + c * sizeof(U)) = *(const U*)(src + r * src_ld + c * sizeof(U));
  }
}

static int grid_for(int64_t n) {
  int64_t g = (n + 255) / 256;
  if (g > 8192) g = 8192;
  return (int)(g < 1 ? 1 : g);
}

hipError_t copy2d(void* dst, size_t dst_ld, const void* src, size_t src_ld, int64_t rows,
                  size_t row_bytes, hipStream_t st) {
  if (rows <= 0 || row_bytes == 0) return hipSuccess;
  const uintptr_t all = (uintptr_t)dst | (uintptr_t)src | dst_ld | src_ld | row_bytes;
  const int64_t n16 = rows * (int64_t)(row_bytes / 16), n4 = rows * (int64_t)(row_bytes / 4);
  const int64_t n2 = rows * (int64_t)(row_bytes / 2), n1 = rows * (int64_t)row_bytes;
  if ((all & 15) == 0)
    hipLaunchKernelGGL(k_copy2d<uint4>, dim3(grid_for(n16)), dim3(256), 0, st, (char*)dst, dst_ld,
                       (const char*)src, src_ld, rows, (int64_t)(row_bytes / 16));
  else if ((all & 3) == 0)
    hipLaunchKernelGGL(k_copy2d<uint32_t>, dim3(grid_for(n4)), dim3(256), 0, st, (char*)dst, dst_ld,
                       (const char*)src, src_ld, rows, (int64_t)(row_bytes / 4));
  else if ((all & 1) == 0)
    hipLaunchKernelGGL(k_copy2d<uint16_t>, dim3(grid_for(n2)), dim3(256), 0, st, (char*)dst, dst_ld,
                       (const char*)src, src_ld, rows, (int64_t)(row_bytes / 2));
  else
    hipLaunchKernelGGL(k_copy2d<uint8_t>, dim3(grid_for(n1)), dim3(256), 0, st, (char*)dst, dst_ld,
                       (const char*)src, src_ld, rows, (int64_t)row_bytes);
  return hipGetLastError();
}

// One thread per 34-byte block: AoS block (scale, 32 codes) <-> (codes plane, scale plane).
// `aos` points at the first block of the slice in row 0; `aos_ld` is the full row stride (bytes).
__global__ void k_q8_split(const uint8_t* __restrict__ aos, size_t aos_ld, int64_t rows,
                           int64_t nblk, int8_t* __restrict__ codes, uint16_t* __restrict__ scales) {
  const int64_t total = rows * nblk;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / nblk, b = i - r * nblk;
    const uint16_t* blk = (const uint16_t*)(aos + r * aos_ld + b * 34);  // 2-byte aligned
    scales[r * nblk + b] = blk[0];
    uint16_t* dst = (uint16_t*)(codes + (r * nblk + b) * 32);
#pragma unroll
    for (int k = 0; k < 16; ++k) dst[k] = blk[1 + k];
  }
}

__global__ void k_q8_join(uint8_t* __restrict__ aos, size_t aos_ld, int64_t rows, int64_t nblk,
                          const int8_t* __restrict__ codes, const uint16_t* __restrict__ scales) {
  const int64_t total = rows * nblk;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / nblk, b = i - r * nblk;
    uint16_t* blk = (uint16_t*)(aos + r * aos_ld + b * 34);
    blk[0] = scales[r * nblk + b];
    const uint16_t* src = (const uint16_t*)(codes + (r * nblk + b) * 32);
#pragma unroll
    for (int k = 0; k < 16; ++k) blk[1 + k] = src[k];
  }
}

hipError_t q8_split(const void* aos, size_t aos_ld, int64_t rows, int64_t nblk, void* codes,
                    void* scales, hipStream_t st) {
  if (rows <= 0 || nblk <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_q8_split, dim3(grid_for(rows * nblk)), dim3(256), 0, st,
                     (const uint8_t*)aos, aos_ld, rows, nblk, (int8_t*)codes, (uint16_t*)scales);
  return hipGetLastError();
}

hipError_t q8_join(void* aos, size_t aos_ld, int64_t rows, int64_t nblk, const void* codes,
                   const void* scales, hipStream_t st) {
  if (rows <= 0 || nblk <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_q8_join, dim3(grid_for(rows * nblk)), dim3(256), 0, st, (uint8_t*)aos,
                     aos_ld, rows, nblk, (const int8_t*)codes, (const uint16_t*)scales);
  return hipGetLastError();
}

__global__ void k_q8_dequant(const int8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
                             float* __restrict__ out, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    out[i] = q8_dequant(f16_to_f32(scales[i >> 5]), codes[i]);
}

hipError_t q8_dequant_buf(const void* codes, const void* scales, float* out, int64_t n_blocks,
                          hipStream_t st) {
  if (n_blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_q8_dequant, dim3(grid_for(n_blocks * 32)), dim3(256), 0, st,
                     (const int8_t*)codes, (const uint16_t*)scales, out, n_blocks * 32);
  return hipGetLastError();
}

// Token-embedding lookup (the replicated input layer around the block stack): row ids[t] of the
// packed table becomes x[t] in the activation dtype. F32 and BF16 rows are copied as stored; a
// Q8_0 row is dequantised (scale * code is exact in fp32) and rounded once to bf16. A thread moves
// one 16-byte chunk of the stored row; ids outside [0, vocab) are clamped into the table.
template <int WT>
__global__ void k_embed(const char* __restrict__ table, const uint16_t* __restrict__ scales,
                        const int32_t* __restrict__ ids, int vocab, int d,
                        char* __restrict__ x) {
  constexpr int WB = WT == W_F32 ? 4 : (WT == W_BF16 ? 2 : 1);
  const int t = blockIdx.x;
  int id = ids[t];
  id = id < 0 ? 0 : (id >= vocab ? vocab - 1 : id);
  const int nch = d * WB / 16;
  const char* row = table + (size_t)id * d * WB;
  for (int c = threadIdx.x; c < nch; c += blockDim.x) {
    const uint4 v = *(const uint4*)(row + (size_t)c * 16);
    if constexpr (WT != W_Q8) {
      *(uint4*)(x + ((size_t)t * d * WB) + (size_t)c * 16) = v;
    } else {
      const float sc = f16_to_f32(scales[(size_t)id * (d / 32) + c / 2]);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      uint32_t o[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int32_t b0 = (int8_t)(w[i] & 0xffu), b1 = (int8_t)((w[i] >> 8) & 0xffu);
        const int32_t b2 = (int8_t)((w[i] >> 16) & 0xffu), b3 = (int8_t)(w[i] >> 24);
        o[2 * i] = f32_to_bf16(q8_dequant(sc, b0)) | ((uint32_t)f32_to_bf16(q8_dequant(sc, b1)) << 16);
        o[2 * i + 1] =
            f32_to_bf16(q8_dequant(sc, b2)) | ((uint32_t)f32_to_bf16(q8_dequant(sc, b3)) << 16);
      }
      uint4* dst = (uint4*)(x + ((size_t)t * d + (size_t)c * 16) * 2);
      dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
      dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
    }
  }
}

hipError_t launch_embed(int wt, const void* table, const void* scales, const int32_t* ids,
                        int T, int vocab, int d, void* x, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  const dim3 g(T), b(256);
  if (wt == W_F32)
    hipLaunchKernelGGL(k_embed<W_F32>, g, b, 0, st, (const char*)table, nullptr, ids, vocab, d,
                       (char*)x);
  else if (wt == W_BF16)
    hipLaunchKernelGGL(k_embed<W_BF16>, g, b, 0, st, (const char*)table, nullptr, ids, vocab, d,
                       (char*)x);
  else if (wt == W_Q8)
    hipLaunchKernelGGL(k_embed<W_Q8>, g, b, 0, st, (const char*)table, (const uint16_t*)scales,
                       ids, vocab, d, (char*)x);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace tpk
