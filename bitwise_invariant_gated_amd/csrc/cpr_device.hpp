// Device routines of the CPR Gated DeltaNet layer for gfx950.
//
// Every quantity that must round identically in prefill and decode is
// computed by exactly one routine in this file:
//   token_step        the per-token recurrence on one state column
//                     (prefill's in-chunk scan and decode both call it)
//   chunk_local_f32   chunk products W, U, K~^T, Gamma_n of one chunk
//                     (prefill's chunk pass and decode's resync call it)
//   chain_step_f32    boundary advance S' = Gamma_n S + K~^T (U - W S)
//                     (prefill's boundary chain and decode's resync call it)
// The pages that describe the method (IsoExec, section "Chunkwise-Parallel
// Recurrent (CPR) Gated DeltaNet"; the Chinese page's section on a third way
// for Gated DeltaNet) fix only the structure: boundary states by the chunk
// form, then the recurrence inside every chunk from those boundaries, and
// decode resynchronising every C tokens.  The rounding choices below are this
// library's own; they are fixed (explicit FMAs, no contraction, fixed loop
// orders) so that every caller reproduces them bit for bit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cpr {

constexpr int kChunk = 64;  // C
constexpr int kWave = 64;

typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
// Wave-uniform, read-only row pointer: loads through it become scalar loads
// into SGPRs, which every lane's VALU instruction can read directly.
typedef const __attribute__((address_space(4))) u32x8* UniformRow;

// ---------------------------------------------------------------------------
// storage dtypes

struct Bf16 {
  typedef uint16_t T;
  static constexpr int kRowGroup = 16;  // values per 32-byte scalar load
  __device__ static __forceinline__ float load(const T* p, size_t i) {
    return __uint_as_float((uint32_t)p[i] << 16);
  }
  __device__ static __forceinline__ void store(T* p, size_t i, float x) { p[i] = round(x); }
  // fp32 -> bf16, round to nearest even; NaN stays NaN.
  __device__ static __forceinline__ uint16_t round(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
  }
  __device__ static __forceinline__ float elem(const u32x8& w, int e) {
    return (e & 1) ? __uint_as_float(w[e >> 1] & 0xffff0000u) : __uint_as_float(w[e >> 1] << 16);
  }
};

struct F32 {
  typedef float T;
  static constexpr int kRowGroup = 8;
  __device__ static __forceinline__ float load(const T* p, size_t i) { return p[i]; }
  __device__ static __forceinline__ void store(T* p, size_t i, float x) { p[i] = x; }
  __device__ static __forceinline__ float elem(const u32x8& w, int e) { return __uint_as_float(w[e]); }
};

// Hides a pointer's value from the optimiser so that each use issues its own
// scalar load (bounding SGPR live ranges instead of hoisting every load).
__device__ __forceinline__ UniformRow fresh(UniformRow p) {
  asm volatile("" : "+s"(p));
  return p;
}

__device__ __forceinline__ float lane_bcast(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

// ---------------------------------------------------------------------------
// The per-token step (one state column per lane).
//
// Lane j holds column j of S (S[i][j] = M[j][i], i = 0..DK-1) in s[].  With
// k, q wave-uniform (scalar registers), the step is, in this exact order:
//   pass A, i ascending:  s[i] = alpha * s[i];  p_(i mod 2) = fma(s[i], k[i], p_(i mod 2))
//   p = p_0 + p_1;  u = beta * (v_j - p)
//   pass B, i ascending:  s[i] = fma(k[i], u, s[i]);  o_(i mod 2) = fma(s[i], q[i], o_(i mod 2))
//   return o_0 + o_1
// which is M' = alpha M, p = M' k, u = beta (v - p), M = M' + u k^T, o = M q.
template <class D, int DK>
__device__ __forceinline__ float token_step(float (&s)[DK], UniformRow krow, UniformRow qrow,
                                            float alpha, float beta, float v) {
  constexpr int G = D::kRowGroup;
  static_assert(DK % G == 0, "key dim must be a multiple of the scalar load group");
  float p0 = 0.f, p1 = 0.f;
#pragma unroll
  for (int gi = 0; gi < DK / G; ++gi) {
    const u32x8 w = *fresh(krow + gi);
#pragma unroll
    for (int e = 0; e < G; e += 2) {
      const int i = gi * G + e;
      s[i] = alpha * s[i];
      p0 = __builtin_fmaf(s[i], D::elem(w, e), p0);
      s[i + 1] = alpha * s[i + 1];
      p1 = __builtin_fmaf(s[i + 1], D::elem(w, e + 1), p1);
    }
  }
  const float u = beta * (v - (p0 + p1));
  float o0 = 0.f, o1 = 0.f;
#pragma unroll
  for (int gi = 0; gi < DK / G; ++gi) {
    const u32x8 w = *fresh(krow + gi);
    const u32x8 x = *fresh(qrow + gi);
#pragma unroll
    for (int e = 0; e < G; e += 2) {
      const int i = gi * G + e;
      s[i] = __builtin_fmaf(D::elem(w, e), u, s[i]);
      o0 = __builtin_fmaf(s[i], D::elem(x, e), o0);
      s[i + 1] = __builtin_fmaf(D::elem(w, e + 1), u, s[i + 1]);
      o1 = __builtin_fmaf(s[i + 1], D::elem(x, e + 1), o1);
    }
  }
  return o0 + o1;
}

// alpha = exp(g); one definition for the scan and for decode.
__device__ __forceinline__ float decay_of(float g) { return expf(g); }

// ---------------------------------------------------------------------------
// Chunk-local products, fp32 VALU (one full chunk of C tokens, one head).
//
// With gamma_t = g_0 + ... + g_t (left to right), Gamma_t = exp(gamma_t),
// e_t = exp(gamma_{C-1} - gamma_t):
//   L[t][s] = (beta_t * exp(gamma_t - gamma_s)) * (k_t . k_s)   for s < t
//   T = (I + L)^{-1} diag(beta)       (forward substitution, column by column)
//   W[t][i]  = sum_{r<=t} (T[t][r] * Gamma_r) * K[r][i]
//   U[t][j]  = sum_{r<=t} T[t][r] * V[r][j]
//   KtT[i][r] = e_r * K[r][i]
//   Gamma_n  = Gamma_{C-1}
// Every sum runs in ascending index order from 0 with explicit FMAs.
template <int DK, int DV>
struct ChunkLds {
  float K[kChunk][DK];
  float V[kChunk][DV];
  float A[kChunk][kChunk];   // L
  float Tm[kChunk][kChunk];  // T
  float g[kChunk], beta[kChunk], gam[kChunk], Gam[kChunk], e[kChunk];
};

// Caller has staged K, V, g, beta into sm and synchronised.  Writes W [C][DK],
// U [C][DV], KtT [DK][C] and *gamn (global memory).
template <int DK, int DV>
__device__ void chunk_local_f32(ChunkLds<DK, DV>& sm, float* __restrict__ W, float* __restrict__ U,
                                float* __restrict__ KtT, float* __restrict__ gamn) {
  constexpr int C = kChunk;
  const int tid = threadIdx.x;
  const int nt = blockDim.x;
  if (tid == 0) {
    float acc = sm.g[0];
    sm.gam[0] = acc;
    for (int t = 1; t < C; ++t) {
      acc = acc + sm.g[t];
      sm.gam[t] = acc;
    }
  }
  __syncthreads();
  for (int t = tid; t < C; t += nt) {
    sm.Gam[t] = expf(sm.gam[t]);
    sm.e[t] = expf(sm.gam[C - 1] - sm.gam[t]);
  }
  for (int idx = tid; idx < C * C; idx += nt) {
    const int t = idx / C, s = idx % C;
    float val = 0.f;
    if (s < t) {
      const float y = sm.beta[t] * expf(sm.gam[t] - sm.gam[s]);
      float d = 0.f;
      for (int i = 0; i < DK; ++i) d = __builtin_fmaf(sm.K[t][i], sm.K[s][i], d);
      val = y * d;
    }
    sm.A[t][s] = val;
  }
  __syncthreads();
  for (int s = tid; s < C; s += nt) {
    for (int t = 0; t < C; ++t) {
      float acc;
      if (t < s) {
        acc = 0.f;
      } else if (t == s) {
        acc = sm.beta[s];
      } else {
        acc = 0.f;
        for (int r = s; r < t; ++r) acc = __builtin_fmaf(-sm.A[t][r], sm.Tm[r][s], acc);
      }
      sm.Tm[t][s] = acc;
    }
  }
  __syncthreads();
  for (int idx = tid; idx < C * DK; idx += nt) {
    const int t = idx / DK, i = idx % DK;
    float acc = 0.f;
    for (int r = 0; r <= t; ++r) acc = __builtin_fmaf(sm.Tm[t][r] * sm.Gam[r], sm.K[r][i], acc);
    W[idx] = acc;
  }
  for (int idx = tid; idx < C * DV; idx += nt) {
    const int t = idx / DV, j = idx % DV;
    float acc = 0.f;
    for (int r = 0; r <= t; ++r) acc = __builtin_fmaf(sm.Tm[t][r], sm.V[r][j], acc);
    U[idx] = acc;
  }
  for (int idx = tid; idx < DK * C; idx += nt) {
    const int i = idx / C, r = idx % C;
    KtT[idx] = sm.e[r] * sm.K[r][i];
  }
  if (tid == 0) *gamn = sm.Gam[C - 1];
}

// ---------------------------------------------------------------------------
// Boundary advance, fp32 VALU, for a block of NB state columns.
//   Delta[t][j] = U[t][j] - sum_i W[t][i] S[i][j]     (acc starts at U, i ascending)
//   S'[i][j]    = Gamma_n * S[i][j] + sum_t KtT[i][t] Delta[t][j]   (t ascending)
// The value of each S' entry depends only on its own column, so any column
// blocking gives the same bits.
template <int DK, int NB>
struct ChainLds {
  float S[DK][NB];
  float W[kChunk][DK];
  float KtT[DK][kChunk];
  float U[kChunk][NB];
  float D[kChunk][NB];
  float gamn;
};

// Caller has staged W, KtT, U (columns of this block), gamn and S; synchronised.
template <int DK, int NB>
__device__ void chain_step_f32(ChainLds<DK, NB>& sm) {
  constexpr int C = kChunk;
  constexpr int kPer = (DK * NB + 255) / 256;
  const int tid = threadIdx.x;
  const int nt = blockDim.x;
  for (int idx = tid; idx < C * NB; idx += nt) {
    const int t = idx / NB, j = idx % NB;
    float acc = sm.U[t][j];
    for (int i = 0; i < DK; ++i) acc = __builtin_fmaf(-sm.W[t][i], sm.S[i][j], acc);
    sm.D[t][j] = acc;
  }
  __syncthreads();
  float out[kPer];
  const float gn = sm.gamn;
#pragma unroll
  for (int m = 0; m < kPer; ++m) {
    const int idx = tid + m * nt;
    if (idx < DK * NB) {
      const int i = idx / NB, j = idx % NB;
      float acc = gn * sm.S[i][j];
      for (int t = 0; t < C; ++t) acc = __builtin_fmaf(sm.KtT[i][t], sm.D[t][j], acc);
      out[m] = acc;
    }
  }
  __syncthreads();
#pragma unroll
  for (int m = 0; m < kPer; ++m) {
    const int idx = tid + m * nt;
    if (idx < DK * NB) sm.S[idx / NB][idx % NB] = out[m];
  }
  __syncthreads();
}

}  // namespace cpr
