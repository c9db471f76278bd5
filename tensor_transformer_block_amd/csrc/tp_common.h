// Device-side helpers shared by the kernels of libtpblock (gfx950 / CDNA4, 64-wide wavefronts).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tp_kernels.h"

namespace tpk {

constexpr int kWave = 64;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load (non-temporal hint: data read once, keep it out of the way in cache).
__device__ __forceinline__ uint4 ld_stream16(const void* p) {
  const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Round to nearest even (the gfx950 conversion instruction); NaN stays a NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// Q8_0 dequantisation of one weight: fp16 scale times the signed code. The product of an 11-bit
// significand and an 8-bit integer is exact in fp32.
__device__ __forceinline__ float q8_dequant(float scale, int32_t code) {
  return scale * (float)code;
}

// Bit mask keeping the first `n` (clamped to [0, 8]) of eight bf16 values packed in 16 bytes:
// V elements of keys no one has written to are cleared with it before a P.V product.
__device__ __forceinline__ uint4 v_keep_mask(int n) {
  n = n < 0 ? 0 : (n > 8 ? 8 : n);
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = (2 * i < n ? 0x0000ffffu : 0u) | (2 * i + 1 < n ? 0xffff0000u : 0u);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

template <int AT>
__device__ __forceinline__ float ld_act(const void* p, size_t i) {
  if constexpr (AT == ACT_F32) return ((const float*)p)[i];
  else return bf16_to_f32(((const uint16_t*)p)[i]);
}

template <int AT>
__device__ __forceinline__ void st_act(void* p, size_t i, float v) {
  if constexpr (AT == ACT_F32) ((float*)p)[i] = v;
  else ((uint16_t*)p)[i] = f32_to_bf16(v);
}

template <int T>
__device__ __forceinline__ float round_to(float v) {
  if constexpr (T == ACT_F32) return v;
  else return bf16_to_f32(f32_to_bf16(v));
}

// 16-byte vector of activations widened to fp32: 4 (fp32) or 8 (bf16) values.
template <int AT> struct Vec16;
template <> struct Vec16<ACT_F32> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void load(const void* p, float* out) {
    float4 v = *(const float4*)p;
    out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
  }
};
template <> struct Vec16<ACT_BF16> {
  static constexpr int N = 8;
  __device__ __forceinline__ static void load(const void* p, float* out) {
    uint4 v = *(const uint4*)p;
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};

// Widen a 16-byte register vector of activations to fp32 (4 fp32 or 8 bf16 values).
template <int AT>
__device__ __forceinline__ void unpack16(const uint4& v, float* out) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  if constexpr (AT == ACT_F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(w[i]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
}

// Cross-lane reductions. Inside a row of 16 lanes they use DPP lane swizzles (quad_perm, then
// row_half_mirror, then row_mirror): after the four steps every lane of the row holds the row
// total. Rows are combined with two lane permutes through the LDS crossbar.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, true));
}
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1, 0, 3, 2]
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2, 3, 0, 1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<kQuadXor1>(v);
  v += dpp_f<kQuadXor2>(v);
  v += dpp_f<kRowHalfMirror>(v);
  v += dpp_f<kRowMirror>(v);
  return v;
}

__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<kQuadXor1>(v));
  v = fmaxf(v, dpp_f<kQuadXor2>(v));
  v = fmaxf(v, dpp_f<kRowHalfMirror>(v));
  v = fmaxf(v, dpp_f<kRowMirror>(v));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  v += __shfl_xor(v, 16, kWave);
  v += __shfl_xor(v, 32, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  v = fmaxf(v, __shfl_xor(v, 16, kWave));
  v = fmaxf(v, __shfl_xor(v, 32, kWave));
  return v;
}

// SiLU(z) = z / (1 + e^-z)  and  GELU-tanh(z) = z/2 (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))).
__device__ __forceinline__ float act_silu(float z) { return z / (1.0f + __expf(-z)); }
__device__ __forceinline__ float act_gelu_tanh(float z) {
  const float k = 0.7978845608028654f;  // sqrt(2/pi)
  float u = k * (z + 0.044715f * z * z * z);
  // tanh(u) = 1 - 2 / (e^{2u} + 1), saturating correctly for large |u|.
  float t = 1.0f - 2.0f / (__expf(2.0f * u) + 1.0f);
  return 0.5f * z * (1.0f + t);
}

template <int ACTF>
__device__ __forceinline__ float gated(float g, float u) {
  if constexpr (ACTF == 0) return act_silu(g) * u;
  else return act_gelu_tanh(g) * u;
}

// Workgroup -> output tile for the GEMMs. Workgroups are dealt round-robin to the 8 XCDs, so
// the first 8 * floor(n / 8) of them are renumbered to make each XCD's share a contiguous run of
// tile indices; a run then walks GM m-bands down before stepping across n, so the tiles one XCD
// holds at a time form a GM x k block and both operands are reused in that XCD's L2.
__device__ __forceinline__ void tile_coords(int b, int nblk, int tiles_m, int tiles_n, int& tm,
                                            int& tn) {
  constexpr int GM = 4;
  const int full = nblk / 8 * 8;
  const int lt = (b < full) ? (b % 8) * (full / 8) + b / 8 : b;
  const int g = lt / (GM * tiles_n), r = lt % (GM * tiles_n);
  const int gm = min(GM, tiles_m - g * GM);
  tm = g * GM + r % gm;
  tn = r / gm;
}

}  // namespace tpk
