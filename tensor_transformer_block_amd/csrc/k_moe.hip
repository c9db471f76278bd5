// Expert-sliced mixture-of-experts FFN for one rank (TensorSharp "Multi-GPU & Multi-Node",
// section "Supported architectures": each expert is sharded like the dense FFN, its gate and up
// rows by output column and its down rows by input column, and the router is identical on all
// ranks; a rank therefore keeps 1/N of every expert, and the expert ids picked for a token are
// valid on each of them).
//
//   router:  logits [T, E] = xn . Wr^T (the decode GEMV), then k_moe_topk: per token the top_k
//            experts by logit (largest first, equal logits: lower index first) and their weights,
//            the softmax of the selected logits;
//   gate/up: k_moe_gate_up: m[t, j*Fr + i] = act(xn[t] . Wg[e][i]) * (xn[t] . Wu[e][i]) for the
//            token's j-th expert e, over the rank's Fr = F_e/N gate and up rows of that expert;
//   down:    k_moe_down: partial[t, n] = sum_j w[t, j] * (m[t, j*Fr : (j+1)*Fr] . Wd[e][n]) over
//            the rank's Fr columns of expert e's down rows.
// The expert kernels stream only the selected experts' slices: one token's k experts are a small
// subset of the table, so they are GEMVs over indirectly addressed rows (16-byte loads, the token
// vector staged in LDS as fp32, dot products reduced across the wave). MoE blocks run token by
// token (grid.y = token), as the page notes MoE models do under tensor parallelism.
#include "k_gemv_impl.h"

namespace tpk {

// ---------------------------------------------------------------------------- top-k routing
// One wave per token: each lane holds PER >= E/64 logits (PER a power of two; routers of at most
// 64 experts take k_moe_topk64 below instead); top_k rounds of a wave-wide (value, index) maximum
// pick the experts in order, then the selected logits' softmax gives the weights.
constexpr int kMoeMaxExperts = 1024, kMoeMaxTopK = 16;

template <int PER>
__global__ __launch_bounds__(256) void k_moe_topk(const float* __restrict__ logits, int T, int E,
                                                  int top_k, int32_t* __restrict__ ids,
                                                  float* __restrict__ weights) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = i * 64 + lane;
    const float z = e < E ? logits[(size_t)t * E + e] : -INFINITY;
    v[i] = z != z ? -INFINITY : z;  // a NaN logit ranks as -inf (below every number)
  }
  bool taken[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) taken[i] = (i * 64 + lane) >= E;
  // round r's winner is kept by lane r
  float my_v = -INFINITY;
  int my_i = 0;
  for (int r = 0; r < top_k; ++r) {
    // lane-local best untaken entry: larger value, then lower index (indices grow with i)
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = i * 64 + lane;
      if (!taken[i] && (v[i] > bv || (v[i] == bv && e < bi))) {
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    // every lane now holds the winner; its owner marks it taken
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (i * 64 + lane == bi) taken[i] = true;
    if (lane == r) {
      my_v = bv;
      my_i = bi;
    }
  }
  // softmax of the selected logits (the first winner is their maximum)
  const float top = __shfl(my_v, 0, 64);
  const float ex = lane < top_k ? expf(my_v - top) : 0.f;
  const float den = wave_sum(ex);
  if (lane < top_k) {
    ids[(size_t)t * top_k + lane] = my_i;
    weights[(size_t)t * top_k + lane] = ex / den;
  }
}

// At most 64 experts: each lane holds one logit and counts the entries ranked above it (larger,
// or equal with a lower index), which places every selected expert directly: one pass over the
// wave's logits in LDS instead of top_k rounds of wave-wide maxima. The winners are then moved to
// lane = rank, the layout the softmax above uses, so ids and weights come out the same.
// One wave selects token t's top_k of E <= 64 logits (as above) into s_i / s_v (the wave's own
// LDS rows, kMoeMaxTopK entries each) and returns, in lanes < top_k, the selection's id and
// softmax weight.
__device__ __forceinline__ void moe_topk64_wave(const float* __restrict__ zt, int E, int top_k,
                                                float* s_z, float* s_v, int* s_i, int lane,
                                                int* id_out, float* w_out) {
  const float z = lane < E ? zt[lane] : -INFINITY;
  const float v = z != z ? -INFINITY : z;  // a NaN logit ranks as -inf (below every number)
  s_z[lane] = v;
  // The wave's own LDS writes must land before its lanes read each other's entries.
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  int rank = 0;
#pragma unroll
  for (int j = 0; j < 64; j += 4) {
    const float4 z = *(const float4*)&s_z[j];
    rank += (z.x > v || (z.x == v && j < lane)) + (z.y > v || (z.y == v && j + 1 < lane)) +
            (z.z > v || (z.z == v && j + 2 < lane)) + (z.w > v || (z.w == v && j + 3 < lane));
  }
  if (lane < E && rank < top_k) {  // padding lanes (-inf, highest indices) never rank this high
    s_v[rank] = v;
    s_i[rank] = lane;
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  const float my_v = lane < top_k ? s_v[lane] : -INFINITY;
  const int my_i = lane < top_k ? s_i[lane] : 0;
  const float top = __shfl(my_v, 0, 64);
  const float ex = lane < top_k ? expf(my_v - top) : 0.f;
  const float den = wave_sum(ex);
  *id_out = my_i;
  *w_out = ex / den;
}

__global__ __launch_bounds__(256) void k_moe_topk64(const float* __restrict__ logits, int T,
                                                    int E, int top_k, int32_t* __restrict__ ids,
                                                    float* __restrict__ weights) {
  __shared__ __attribute__((aligned(16))) float s_z[4][64];
  __shared__ float s_v[4][kMoeMaxTopK];
  __shared__ int s_i[4][kMoeMaxTopK];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  int id;
  float w;
  moe_topk64_wave(logits + (size_t)t * E, E, top_k, s_z[wave], s_v[wave], s_i[wave], lane, &id,
                  &w);
  if (lane < top_k) {
    ids[(size_t)t * top_k + lane] = id;
    weights[(size_t)t * top_k + lane] = w;
  }
}

hipError_t launch_moe_topk(const float* logits, int T, int E, int top_k, int32_t* ids,
                           float* weights, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  if (E < 1 || E > kMoeMaxExperts || top_k < 1 || top_k > kMoeMaxTopK || top_k > E)
    return hipErrorInvalidValue;
  const dim3 g((T + 3) / 4), b(256);
  const int per = (E + 63) / 64;
  if (per <= 1) launch(k_moe_topk64, g, b, 0, st, logits, T, E, top_k, ids, weights);
  else if (per <= 2) launch(k_moe_topk<2>, g, b, 0, st, logits, T, E, top_k, ids, weights);
  else if (per <= 4) launch(k_moe_topk<4>, g, b, 0, st, logits, T, E, top_k, ids, weights);
  else if (per <= 8) launch(k_moe_topk<8>, g, b, 0, st, logits, T, E, top_k, ids, weights);
  else launch(k_moe_topk<kMoeMaxExperts / 64>, g, b, 0, st, logits, T, E, top_k, ids, weights);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------- expert GEMVs
// Dot product of one 16-byte weight chunk with VE staged fp32 inputs.
template <int WT>
__device__ __forceinline__ float moe_dot(const uint4& raw, float scale, const float* xp) {
  constexpr int VE = WFmt<WT>::VE;
  float f[VE];
  decode_chunk<WT>(raw, scale, f);
  float a = 0.f;
#pragma unroll
  for (int e = 0; e < VE; e += 4) {
    const float4 xv = *(const float4*)(xp + e);
    a = fmaf(f[e], xv.x, a);
    a = fmaf(f[e + 1], xv.y, a);
    a = fmaf(f[e + 2], xv.z, a);
    a = fmaf(f[e + 3], xv.w, a);
  }
  return a;
}

template <int WT>
__device__ __forceinline__ float moe_scale(const uint16_t* S, size_t row, int nblk, int chunk) {
  if constexpr (WT == W_Q8) return f16_to_f32(S[row * nblk + (chunk >> 1)]);
  else return 0.f;
}

// gate/up: a wave owns PW (gate, up) row pairs of the token's selected experts.
constexpr int MOE_PW = 2;

template <int WT, int AT, int ACTF>
__global__ __launch_bounds__(256) void k_moe_gate_up(const char* __restrict__ Wg,
                                                     const uint16_t* __restrict__ Sg,
                                                     const char* __restrict__ Wu,
                                                     const uint16_t* __restrict__ Su, int K,
                                                     int Fr, int E, int top_k,
                                                     const int32_t* __restrict__ ids,
                                                     const void* __restrict__ X,
                                                     void* __restrict__ Mout, MoeRanks mr,
                                                     const float* __restrict__ logits,
                                                     int32_t* __restrict__ ids_out,
                                                     float* __restrict__ w_out) {
  extern __shared__ float xs[];  // [K]
  // logits (E <= 64): the workgroup selects the token's experts itself (wave 0, the router's
  // top-k rule) instead of reading ids; the first workgroup of rank 0 stores the selection and
  // its weights for the down projection and the caller.
  __shared__ __attribute__((aligned(16))) float s_z[64];
  __shared__ float s_v[kMoeMaxTopK];
  __shared__ int s_i[kMoeMaxTopK], s_ids[kMoeMaxTopK];
  const bool sel = logits != nullptr;
  constexpr int VE = WFmt<WT>::VE, WB = WFmt<WT>::WB, AV = Vec16<AT>::N;
  if (mr.n > 1) {  // every rank in one launch (blockIdx.z = rank): that rank's slices and output
    const int r = blockIdx.z;
    Wg = (const char*)mr.wg[r];
    Sg = (const uint16_t*)mr.sg[r];
    Wu = (const char*)mr.wu[r];
    Su = (const uint16_t*)mr.su[r];
    Mout = mr.m[r];
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = blockIdx.y;
  const int nch = K / VE, nblk = K / 32;
  const int np = top_k * Fr;
  size_t grow[MOE_PW];
  bool ok[MOE_PW];
  auto rows = [&](const int32_t* id_src) {
#pragma unroll
    for (int s = 0; s < MOE_PW; ++s) {
      const int p = (blockIdx.x * 4 + wave) * MOE_PW + s;
      ok[s] = p < np;
      const int pp = ok[s] ? p : 0;
      int e = id_src[pp / Fr];
      e = e < 0 ? 0 : (e >= E ? E - 1 : e);
      grow[s] = (size_t)e * Fr + pp % Fr;
    }
  };
  if (!sel) {
    rows(ids + (size_t)t * top_k);
  } else if (wave == 0) {
    int id;
    float w;
    moe_topk64_wave(logits + (size_t)t * E, E, top_k, s_z, s_v, s_i, lane, &id, &w);
    if (lane < top_k) {
      s_ids[lane] = id;
      if (blockIdx.x == 0 && blockIdx.z == 0) {
        ids_out[(size_t)t * top_k + lane] = id;
        w_out[(size_t)t * top_k + lane] = w;
      }
    }
  }
  for (int i = tid * AV; i < K; i += 256 * AV)
    Vec16<AT>::load((const char*)X + ((size_t)t * K + i) * (AT == ACT_F32 ? 4 : 2), xs + i);
  __syncthreads();
  if (sel) rows(s_ids);
  if (!ok[0]) return;
  float g[MOE_PW], u[MOE_PW];
#pragma unroll
  for (int s = 0; s < MOE_PW; ++s) g[s] = u[s] = 0.f;
  for (int c0 = 0; c0 < nch; c0 += 64 * 4) {
    uint4 bg[MOE_PW][4], bu[MOE_PW][4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = c0 + q * 64 + lane;
#pragma unroll
      for (int s = 0; s < MOE_PW; ++s) {
        bg[s][q] = c < nch ? ld_stream16(Wg + (grow[s] * K + (size_t)c * VE) * WB)
                           : make_uint4(0, 0, 0, 0);
        bu[s][q] = c < nch ? ld_stream16(Wu + (grow[s] * K + (size_t)c * VE) * WB)
                           : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = c0 + q * 64 + lane;
      if (c >= nch) continue;
#pragma unroll
      for (int s = 0; s < MOE_PW; ++s) {
        g[s] += moe_dot<WT>(bg[s][q], moe_scale<WT>(Sg, grow[s], nblk, c * VE / 16), xs + c * VE);
        u[s] += moe_dot<WT>(bu[s][q], moe_scale<WT>(Su, grow[s], nblk, c * VE / 16), xs + c * VE);
      }
    }
  }
#pragma unroll
  for (int s = 0; s < MOE_PW; ++s) {
    g[s] = wave_sum(g[s]);
    u[s] = wave_sum(u[s]);
  }
  if (lane == 0) {
#pragma unroll
    for (int s = 0; s < MOE_PW; ++s) {
      const int p = (blockIdx.x * 4 + wave) * MOE_PW + s;
      if (p < np) st_act<AT>(Mout, (size_t)t * np + p, gated<ACTF>(g[s], u[s]));
    }
  }
}

// down: a wave owns MOE_DR output rows. Its lanes walk the concatenation of the token's k
// segments (expert j's Fr columns of the row), 16 bytes each, so every lane has a load in flight
// whatever Fr is, and add w_j times each chunk's dot product with m.
constexpr int MOE_DR = 2, MOE_DU = 8;  // rows per wave, chunks per lane in flight per row

// PV > 0: the last rank of the one-call MoE block also adds the earlier ranks' partials (up to PV
// of them, in rank order) and the residual, as the reduce kernel would (FuseArgs as for the
// decode GEMV's reduce epilogue); their values are requested before the weight stream.
template <int WT, int AT, int PT, int PV>
__global__ __launch_bounds__(256) void k_moe_down(const char* __restrict__ Wd,
                                                  const uint16_t* __restrict__ Sd, int d, int Fr,
                                                  int E, int top_k,
                                                  const int32_t* __restrict__ ids,
                                                  const float* __restrict__ wts,
                                                  const void* __restrict__ Min,
                                                  void* __restrict__ P, FuseArgs fa) {
  extern __shared__ float ms[];  // [top_k * Fr]
  __shared__ int s_e[kMoeMaxTopK];
  __shared__ float s_w[kMoeMaxTopK];
  constexpr int VE = WFmt<WT>::VE, WB = WFmt<WT>::WB, AV = Vec16<AT>::N;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = blockIdx.y;
  const int np = top_k * Fr, chF = Fr / VE, nblk = Fr / 32, nq = top_k * chF;
  for (int i = tid * AV; i < np; i += 256 * AV)
    Vec16<AT>::load((const char*)Min + ((size_t)t * np + i) * (AT == ACT_F32 ? 4 : 2), ms + i);
  if (tid < top_k) {
    int e = ids[(size_t)t * top_k + tid];
    s_e[tid] = e < 0 ? 0 : (e >= E ? E - 1 : e);
    s_w[tid] = wts[(size_t)t * top_k + tid];
  }
  __syncthreads();
  const int n0 = (blockIdx.x * 4 + wave) * MOE_DR;
  if (n0 >= d) return;
  int nrow[MOE_DR];
#pragma unroll
  for (int s = 0; s < MOE_DR; ++s) nrow[s] = n0 + s < d ? n0 + s : d - 1;
  constexpr int PR = PV > 0 ? PV : 1, RR = PV > 0 ? MOE_DR : 1;
  uint32_t e_prev[RR][PR], e_res[RR];
  if constexpr (PV > 0) {  // unconditional, clamped loads (no waits at branch joins)
    const bool any_prev = fa.n_prev > 0;
#pragma unroll
    for (int s = 0; s < MOE_DR; ++s) {
      const size_t o = (size_t)t * d + nrow[s];
      if constexpr (AT == ACT_F32) e_res[s] = ((const uint32_t*)fa.res_in)[o];
      else e_res[s] = ((const uint16_t*)fa.res_in)[o];
#pragma unroll
      for (int k = 0; k < PV; ++k) {
        const size_t pi = any_prev ? (size_t)(k < fa.n_prev ? k : 0) * fa.part_stride + o : 0;
        const void* base = any_prev ? fa.prev : fa.res_in;
        if constexpr (PT == ACT_BF16) e_prev[s][k] = ((const uint16_t*)base)[pi];
        else e_prev[s][k] = ((const uint32_t*)base)[any_prev ? pi : 0];
      }
    }
  }
  float acc[MOE_DR];
#pragma unroll
  for (int s = 0; s < MOE_DR; ++s) acc[s] = 0.f;
  for (int q0 = 0; q0 < nq; q0 += 64 * MOE_DU) {
    uint4 b[MOE_DU][MOE_DR];
    int jj[MOE_DU], cc[MOE_DU];
#pragma unroll
    for (int u = 0; u < MOE_DU; ++u) {
      const int q = q0 + u * 64 + lane;
      const bool in = q < nq;
      jj[u] = in ? q / chF : 0;
      cc[u] = in ? q - jj[u] * chF : 0;
#pragma unroll
      for (int s = 0; s < MOE_DR; ++s) {
        const size_t row = (size_t)s_e[jj[u]] * d + nrow[s];
        b[u][s] = in ? ld_stream16(Wd + (row * Fr + (size_t)cc[u] * VE) * WB)
                     : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < MOE_DU; ++u) {
      const int q = q0 + u * 64 + lane;
      if (q >= nq) continue;
      const float wj = s_w[jj[u]];
      const float* mp = ms + jj[u] * Fr + cc[u] * VE;
#pragma unroll
      for (int s = 0; s < MOE_DR; ++s) {
        const size_t row = (size_t)s_e[jj[u]] * d + nrow[s];
        acc[s] = fmaf(wj, moe_dot<WT>(b[u][s], moe_scale<WT>(Sd, row, nblk, cc[u] * VE / 16), mp),
                      acc[s]);
      }
    }
  }
#pragma unroll
  for (int s = 0; s < MOE_DR; ++s) acc[s] = wave_sum(acc[s]);
  if (lane == 0) {
#pragma unroll
    for (int s = 0; s < MOE_DR; ++s) {
      if (n0 + s >= d) continue;
      const size_t o = (size_t)t * d + n0 + s;
      float p = acc[s];
      if constexpr (PT == ACT_F32) {
        ((float*)P)[o] = p;
      } else {
        const uint16_t b = f32_to_bf16(p);
        ((uint16_t*)P)[o] = b;
        p = bf16_to_f32(b);
      }
      if constexpr (PV > 0) {
        auto part = [&](uint32_t raw) {
          return PT == ACT_BF16 ? bf16_to_f32(raw) : __uint_as_float(raw);
        };
        float sum = p;
        if (fa.n_prev > 0) {
          sum = part(e_prev[s][0]);
#pragma unroll
          for (int k = 1; k < PV; ++k)
            if (k < fa.n_prev) sum += part(e_prev[s][k]);
          sum += p;
        }
        const float res = AT == ACT_F32 ? __uint_as_float(e_res[s]) : bf16_to_f32(e_res[s]);
        st_act<AT>(fa.res_out, o, res + sum);
      }
    }
  }
}

// The down of every rank in one launch (at most four ranks, NR dividing four): wave w serves
// rank w % NR for the MOE_DR rows of row group w / NR, with the rank's activations staged in LDS
// beside the other ranks'; the partials go to memory at their stored precision and to LDS, and
// the rank-0 wave of each row group adds them in rank order, then the residual.
template <int WT, int AT, int PT>
__global__ __launch_bounds__(256) void k_moe_down_ranks(int d, int Fr, int E, int top_k,
                                                        const int32_t* __restrict__ ids,
                                                        const float* __restrict__ wts,
                                                        MoeRanks mr,
                                                        const void* __restrict__ res,
                                                        void* __restrict__ out) {
  extern __shared__ float ms[];  // [NR][top_k * Fr]
  __shared__ int s_e[kMoeMaxTopK];
  __shared__ float s_w[kMoeMaxTopK];
  __shared__ float s_part[4][MOE_DR];  // [wave][row]
  constexpr int VE = WFmt<WT>::VE, WB = WFmt<WT>::WB, AV = Vec16<AT>::N;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = blockIdx.y;
  const int NR = mr.n, RG = 4 / NR;
  const int np = top_k * Fr, chF = Fr / VE, nblk = Fr / 32, nq = top_k * chF;
  for (int r = 0; r < NR; ++r)
    for (int i = tid * AV; i < np; i += 256 * AV)
      Vec16<AT>::load((const char*)mr.m[r] + ((size_t)t * np + i) * (AT == ACT_F32 ? 4 : 2),
                      ms + (size_t)r * np + i);
  if (tid < top_k) {
    int e = ids[(size_t)t * top_k + tid];
    s_e[tid] = e < 0 ? 0 : (e >= E ? E - 1 : e);
    s_w[tid] = wts[(size_t)t * top_k + tid];
  }
  __syncthreads();
  const int rk = wave % NR, g = wave / NR;
  const bool active = g < RG;  // NR = 3 leaves the fourth wave idle
  const int n0 = (blockIdx.x * RG + (active ? g : 0)) * MOE_DR;
  const char* Wd = (const char*)mr.wd[rk];
  const uint16_t* Sd = (const uint16_t*)mr.sd[rk];
  const float* msr = ms + (size_t)rk * np;
  int nrow[MOE_DR];
#pragma unroll
  for (int s = 0; s < MOE_DR; ++s) nrow[s] = n0 + s < d ? n0 + s : d - 1;
  float acc[MOE_DR];
#pragma unroll
  for (int s = 0; s < MOE_DR; ++s) acc[s] = 0.f;
  if (active && n0 < d) {
    for (int q0 = 0; q0 < nq; q0 += 64 * MOE_DU) {
      uint4 b[MOE_DU][MOE_DR];
      int jj[MOE_DU], cc[MOE_DU];
#pragma unroll
      for (int u = 0; u < MOE_DU; ++u) {
        const int q = q0 + u * 64 + lane;
        const bool in = q < nq;
        jj[u] = in ? q / chF : 0;
        cc[u] = in ? q - jj[u] * chF : 0;
#pragma unroll
        for (int s = 0; s < MOE_DR; ++s) {
          const size_t row = (size_t)s_e[jj[u]] * d + nrow[s];
          b[u][s] = in ? ld_stream16(Wd + (row * Fr + (size_t)cc[u] * VE) * WB)
                       : make_uint4(0, 0, 0, 0);
        }
      }
#pragma unroll
      for (int u = 0; u < MOE_DU; ++u) {
        const int q = q0 + u * 64 + lane;
        if (q >= nq) continue;
        const float wj = s_w[jj[u]];
        const float* mp = msr + jj[u] * Fr + cc[u] * VE;
#pragma unroll
        for (int s = 0; s < MOE_DR; ++s) {
          const size_t row = (size_t)s_e[jj[u]] * d + nrow[s];
          acc[s] = fmaf(wj, moe_dot<WT>(b[u][s], moe_scale<WT>(Sd, row, nblk, cc[u] * VE / 16), mp),
                        acc[s]);
        }
      }
    }
#pragma unroll
    for (int s = 0; s < MOE_DR; ++s) acc[s] = wave_sum(acc[s]);
    if (lane == 0) {
#pragma unroll
      for (int s = 0; s < MOE_DR; ++s) {
        float p = acc[s];
        if (n0 + s < d) {
          const size_t o = (size_t)t * d + n0 + s;
          if constexpr (PT == ACT_F32) {
            ((float*)mr.p[rk])[o] = p;
          } else {
            const uint16_t bb = f32_to_bf16(p);
            ((uint16_t*)mr.p[rk])[o] = bb;
            p = bf16_to_f32(bb);
          }
        }
        s_part[wave][s] = p;
      }
    }
  }
  __syncthreads();
  if (active && rk == 0 && lane == 0 && n0 < d) {
#pragma unroll
    for (int s = 0; s < MOE_DR; ++s) {
      if (n0 + s >= d) continue;
      const size_t o = (size_t)t * d + n0 + s;
      float sum = s_part[wave][s];
      for (int r = 1; r < NR; ++r) sum += s_part[wave + r][s];
      st_act<AT>(out, o, ld_act<AT>(res, o) + sum);
    }
  }
}

bool moe_down_ranks_fit(int n_ranks, int top_k, int Fr) {
  return n_ranks >= 1 && n_ranks <= 4 && (size_t)n_ranks * top_k * Fr * sizeof(float) <= 160 * 1024;
}

template <int WT, int AT, int PT, int PV>
static hipError_t moe_down_launch(dim3 g, size_t lds, hipStream_t st, const char* wd,
                                  const uint16_t* sd, int d, int Fr, int E, int top_k,
                                  const int32_t* ids, const float* wts, const void* M, void* P,
                                  const FuseArgs& fa) {
  if (lds > 65536) {
    hipError_t ea = allow_lds((const void*)k_moe_down<WT, AT, PT, PV>, (int)lds);
    if (ea != hipSuccess) return ea;
  }
  launch((k_moe_down<WT, AT, PT, PV>), g, dim3(256), (uint32_t)lds, st, wd, sd, d, Fr, E, top_k,
         ids, wts, M, P, fa);
  return hipGetLastError();
}

// The down kernel for the partial dtype, with the reduce epilogue when `fuse` is given.
template <int WT, int AT, int PT>
static hipError_t moe_down_variant(dim3 g, size_t lds, hipStream_t st, const char* wd,
                                   const uint16_t* sd, int d, int Fr, int E, int top_k,
                                   const int32_t* ids, const float* wts, const void* M, void* P,
                                   const FuseArgs* fuse) {
  const FuseArgs fa = fuse ? *fuse : FuseArgs{};
  if (!fuse)
    return moe_down_launch<WT, AT, PT, 0>(g, lds, st, wd, sd, d, Fr, E, top_k, ids, wts, M, P, fa);
  if (fa.n_prev > 3)
    return moe_down_launch<WT, AT, PT, 7>(g, lds, st, wd, sd, d, Fr, E, top_k, ids, wts, M, P, fa);
  if (fa.n_prev > 1)
    return moe_down_launch<WT, AT, PT, 3>(g, lds, st, wd, sd, d, Fr, E, top_k, ids, wts, M, P, fa);
  return moe_down_launch<WT, AT, PT, 1>(g, lds, st, wd, sd, d, Fr, E, top_k, ids, wts, M, P, fa);
}

// The gate/up kernel of one rank (mr.n == 0) or of every rank (grid.z = rank).
template <int WT, int AT>
static hipError_t moe_gate_up_fmt(int actf, const void* Wg, const void* Sg, const void* Wu,
                                  const void* Su, int d, int Fr, int E, int top_k, int T,
                                  const int32_t* ids, const void* X, void* M, const MoeRanks& mr,
                                  hipStream_t st, const float* logits = nullptr,
                                  int32_t* ids_out = nullptr, float* w_out = nullptr) {
  const int np = top_k * Fr;
  const dim3 gu((np + 4 * MOE_PW - 1) / (4 * MOE_PW), T, mr.n > 1 ? mr.n : 1), b(256);
  const size_t lds_gu = (size_t)d * sizeof(float);
  const char *wg = (const char*)Wg, *wu = (const char*)Wu;
  const uint16_t *sg = (const uint16_t*)Sg, *su = (const uint16_t*)Su;
  if (lds_gu > 65536) {
    hipError_t ea = allow_lds((const void*)(actf ? k_moe_gate_up<WT, AT, 1> : k_moe_gate_up<WT, AT, 0>),
                              (int)lds_gu);
    if (ea != hipSuccess) return ea;
  }
  if (actf == 0)
    launch((k_moe_gate_up<WT, AT, 0>), gu, b, lds_gu, st, wg, sg, wu, su, d, Fr, E, top_k, ids, X, M,
           mr, logits, ids_out, w_out);
  else
    launch((k_moe_gate_up<WT, AT, 1>), gu, b, lds_gu, st, wg, sg, wu, su, d, Fr, E, top_k, ids, X, M,
           mr, logits, ids_out, w_out);
  return hipGetLastError();
}

template <int WT, int AT>
static hipError_t moe_down_fmt(int pt, const void* Wd, const void* Sd, int d, int Fr, int E,
                               int top_k, int T, const int32_t* ids, const float* wts,
                               const void* M, void* P, hipStream_t st, const FuseArgs* fuse) {
  const int np = top_k * Fr;
  const dim3 gd((d + 4 * MOE_DR - 1) / (4 * MOE_DR), T);
  const size_t lds_d = (size_t)np * sizeof(float);
  const char* wd = (const char*)Wd;
  const uint16_t* sd = (const uint16_t*)Sd;
  if (pt == ACT_F32)
    return moe_down_variant<WT, AT, ACT_F32>(gd, lds_d, st, wd, sd, d, Fr, E, top_k, ids, wts, M,
                                             P, fuse);
  return moe_down_variant<WT, AT, ACT_BF16>(gd, lds_d, st, wd, sd, d, Fr, E, top_k, ids, wts, M, P,
                                            fuse);
}

template <int WT, int AT>
static hipError_t moe_ffn_fmt(int actf, int pt, const void* Wg, const void* Sg, const void* Wu,
                              const void* Su, const void* Wd, const void* Sd, int d, int Fr, int E,
                              int top_k, int T, const int32_t* ids, const float* wts,
                              const void* X, void* M, void* P, hipStream_t st,
                              const FuseArgs* fuse) {
  hipError_t e = moe_gate_up_fmt<WT, AT>(actf, Wg, Sg, Wu, Su, d, Fr, E, top_k, T, ids, X, M,
                                         MoeRanks{}, st);
  if (e != hipSuccess) return e;
  return moe_down_fmt<WT, AT>(pt, Wd, Sd, d, Fr, E, top_k, T, ids, wts, M, P, st, fuse);
}

hipError_t launch_moe_gate_up_ranks(int wt, int at, int actf, int d, int Fr, int E, int top_k,
                                    int T, const int32_t* ids, const void* X, const MoeRanks& mr,
                                    hipStream_t st, const float* logits, float* weights) {
  if (T <= 0) return hipSuccess;
  if (mr.n < 1 || mr.n > kMaxRanks) return hipErrorInvalidValue;
  if (logits && (E > 64 || top_k < 1 || top_k > kMoeMaxTopK || top_k > E || !weights || !ids))
    return hipErrorInvalidValue;
  int32_t* ids_out = logits ? const_cast<int32_t*>(ids) : nullptr;
  for (int r = 0; r < mr.n; ++r)
    if (!mr.wg[r] || !mr.wu[r] || !mr.m[r] || (wt == W_Q8 && (!mr.sg[r] || !mr.su[r])))
      return hipErrorInvalidValue;
  if (wt == W_F32 && at == ACT_F32)
    return moe_gate_up_fmt<W_F32, ACT_F32>(actf, mr.wg[0], mr.sg[0], mr.wu[0], mr.su[0], d, Fr, E,
                                           top_k, T, ids, X, mr.m[0], mr, st, logits, ids_out, weights);
  if (wt == W_BF16 && at == ACT_BF16)
    return moe_gate_up_fmt<W_BF16, ACT_BF16>(actf, mr.wg[0], mr.sg[0], mr.wu[0], mr.su[0], d, Fr,
                                             E, top_k, T, ids, X, mr.m[0], mr, st, logits, ids_out, weights);
  if (wt == W_Q8 && at == ACT_BF16)
    return moe_gate_up_fmt<W_Q8, ACT_BF16>(actf, mr.wg[0], mr.sg[0], mr.wu[0], mr.su[0], d, Fr, E,
                                           top_k, T, ids, X, mr.m[0], mr, st, logits, ids_out, weights);
  return hipErrorInvalidValue;
}

hipError_t launch_moe_down(int wt, int at, int pt, const void* Wd, const void* Sd, int d, int Fr,
                           int E, int top_k, int T, const int32_t* ids, const float* wts,
                           const void* M, void* P, hipStream_t st, const FuseArgs* fuse) {
  if (T <= 0) return hipSuccess;
  if (fuse && (!fuse->res_in || !fuse->res_out || fuse->n_prev < 0 ||
               fuse->n_prev > kMaxPrevPartials || (fuse->n_prev > 0 && !fuse->prev)))
    return hipErrorInvalidValue;
  if (wt == W_F32 && at == ACT_F32)
    return moe_down_fmt<W_F32, ACT_F32>(pt, Wd, Sd, d, Fr, E, top_k, T, ids, wts, M, P, st, fuse);
  if (wt == W_BF16 && at == ACT_BF16)
    return moe_down_fmt<W_BF16, ACT_BF16>(pt, Wd, Sd, d, Fr, E, top_k, T, ids, wts, M, P, st,
                                          fuse);
  if (wt == W_Q8 && at == ACT_BF16)
    return moe_down_fmt<W_Q8, ACT_BF16>(pt, Wd, Sd, d, Fr, E, top_k, T, ids, wts, M, P, st, fuse);
  return hipErrorInvalidValue;
}

template <int WT, int AT>
static hipError_t moe_down_ranks_fmt(int pt, int d, int Fr, int E, int top_k, int T,
                                     const int32_t* ids, const float* wts, const MoeRanks& mr,
                                     const void* res, void* out, hipStream_t st) {
  const int rg = 4 / mr.n;
  const dim3 g((d + rg * MOE_DR - 1) / (rg * MOE_DR), T), b(256);
  const size_t lds = (size_t)mr.n * top_k * Fr * sizeof(float);
  const void* kern = pt == ACT_F32 ? (const void*)k_moe_down_ranks<WT, AT, ACT_F32>
                                   : (const void*)k_moe_down_ranks<WT, AT, ACT_BF16>;
  if (lds > 65536) {
    hipError_t ea = allow_lds(kern, (int)lds);
    if (ea != hipSuccess) return ea;
  }
  if (pt == ACT_F32)
    launch((k_moe_down_ranks<WT, AT, ACT_F32>), g, b, (uint32_t)lds, st, d, Fr, E, top_k, ids,
           wts, mr, res, out);
  else
    launch((k_moe_down_ranks<WT, AT, ACT_BF16>), g, b, (uint32_t)lds, st, d, Fr, E, top_k, ids,
           wts, mr, res, out);
  return hipGetLastError();
}

hipError_t launch_moe_down_ranks(int wt, int at, int pt, int d, int Fr, int E, int top_k, int T,
                                 const int32_t* ids, const float* wts, const MoeRanks& mr,
                                 const void* res, void* out, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  if (!moe_down_ranks_fit(mr.n, top_k, Fr) || !res || !out) return hipErrorInvalidValue;
  for (int r = 0; r < mr.n; ++r)
    if (!mr.wd[r] || !mr.m[r] || !mr.p[r] || (wt == W_Q8 && !mr.sd[r])) return hipErrorInvalidValue;
  if (wt == W_F32 && at == ACT_F32)
    return moe_down_ranks_fmt<W_F32, ACT_F32>(pt, d, Fr, E, top_k, T, ids, wts, mr, res, out, st);
  if (wt == W_BF16 && at == ACT_BF16)
    return moe_down_ranks_fmt<W_BF16, ACT_BF16>(pt, d, Fr, E, top_k, T, ids, wts, mr, res, out, st);
  if (wt == W_Q8 && at == ACT_BF16)
    return moe_down_ranks_fmt<W_Q8, ACT_BF16>(pt, d, Fr, E, top_k, T, ids, wts, mr, res, out, st);
  return hipErrorInvalidValue;
}

hipError_t launch_moe_ffn(int wt, int at, int actf, int pt, const void* Wg, const void* Sg,
                          const void* Wu, const void* Su, const void* Wd, const void* Sd, int d,
                          int Fr, int E, int top_k, int T, const int32_t* ids, const float* wts,
                          const void* X, void* M, void* P, hipStream_t st,
                          const FuseArgs* fuse) {
  if (T <= 0) return hipSuccess;
  if (fuse && (!fuse->res_in || !fuse->res_out || fuse->n_prev < 0 ||
               fuse->n_prev > kMaxPrevPartials || (fuse->n_prev > 0 && !fuse->prev)))
    return hipErrorInvalidValue;
  if (wt == W_F32 && at == ACT_F32)
    return moe_ffn_fmt<W_F32, ACT_F32>(actf, pt, Wg, Sg, Wu, Su, Wd, Sd, d, Fr, E, top_k, T, ids,
                                       wts, X, M, P, st, fuse);
  if (wt == W_BF16 && at == ACT_BF16)
    return moe_ffn_fmt<W_BF16, ACT_BF16>(actf, pt, Wg, Sg, Wu, Su, Wd, Sd, d, Fr, E, top_k, T,
                                         ids, wts, X, M, P, st, fuse);
  if (wt == W_Q8 && at == ACT_BF16)
    return moe_ffn_fmt<W_Q8, ACT_BF16>(actf, pt, Wg, Sg, Wu, Su, Wd, Sd, d, Fr, E, top_k, T, ids,
                                       wts, X, M, P, st, fuse);
  return hipErrorInvalidValue;
}

}  // namespace tpk
