// Backward of the CPR Gated DeltaNet layer (gradient of the exact recurrence,
// evaluated per chunk from the forward's boundary states).
//
// The pages give the trainer forward+backward only as a stage timing
// (IsoExec, "Chunkwise-Parallel Recurrent (CPR) Gated DeltaNet", table row
// "Trainer Fwd+Bwd"); any exact gradient of the recurrence is correct.  This
// one differentiates the chunk (WY / UT) form.  Per chunk of n <= C tokens
// with start state B (S layout, d_k x d_v) and local positions t:
//   gamma = cumsum(g), Gamma = exp(gamma), e_t = exp(gamma_{C-1} - gamma_t),
//   D[t][s] = exp(gamma_t - gamma_s) (s <= t),  G = K K^T,
//   A = strict lower of beta_t D G,  X = (I + A)^{-1},  T = X diag(beta),
//   W = T diag(Gamma) K,  U = T V,  Delta = U - W B,  Kt = diag(e) K,
//   P = (Q K^T) .* D (lower, diagonal included),
//   O  = diag(Gamma) Q B + P Delta,      B' = Gamma_{C-1} B + Kt^T Delta.
// A chunk shorter than C is padded with g = beta = 0 and k = q = v = dO = 0,
// which leaves every quantity of its real tokens unchanged.
// Given dO and dB' (adjoint of B'):
//   dDelta = P^T dO + Kt dB'
//   dB     = Gamma_{C-1} dB' + (diag(Gamma) Q)^T dO - W^T dDelta   (reverse chain)
//   dQ = diag(Gamma) dO B^T + (dP .* D) K,            dP = dO Delta^T
//   dW = -dDelta B^T,  dV = T^T dDelta,  dKt = Delta dB'^T
//   dT = dDelta V^T + dW (diag(Gamma) K)^T,  dX = dT diag(beta),
//   dbeta_s += sum_t X[t][s] dT[t][s],  dA = -X^T dX X^T (strict lower)
//   dbeta_t += sum_s dA D G,  dG = dA .* beta_t D
//   dK = (dP .* D)^T Q + diag(e) dKt + diag(Gamma) T^T dW + (dG + dG^T) K
//   dgamma_t = rowsum(Z)_t - colsum(Z)_t + dGamma_t Gamma_t - de_t e_t
//              (+ dGamma_n Gamma_n + sum de e at t = C-1),
//     Z = (dP .* QK^T + dA .* beta G) .* D,
//     dGamma_t = <dO_t, (Q B)_t> + <(T^T dW)_t, K_t>, de_t = <dKt_t, K_t>,
//     dGamma_n = <dB', B>
//   dg = reverse cumsum of dgamma within the chunk.
// Products run on MFMA (fp32 operands, v_mfma_f32_16x16x4_f32) except the
// reverse chain, which uses the forward chain's bf16 operands.  Reductions
// run in a fixed order (no atomics), so reruns give identical bits.
#pragma once

#include "cpr_device.hpp"

namespace cpr {
namespace bwd {

using mfma::f32x4;
constexpr int C = kChunk;

using mfma::mma4;

// 16 x 16 output tile at (m0, n0) of sum_k A(m, k) B(k, n), k < K (K % 4 == 0).
// fp32 operand layout: lane holds A[m0 + c][k0 + g] and B[k0 + g][n0 + c].
template <int K, class FA, class FB>
__device__ __forceinline__ f32x4 tile(FA&& A, FB&& B, int m0, int n0, f32x4 acc) {
  const int lane = threadIdx.x & 63, lr = lane & 15, g = lane >> 4;
#pragma unroll 8
  for (int k0 = 0; k0 < K; k0 += 4) acc = mma4(A(m0 + lr, k0 + g), B(k0 + g, n0 + lr), acc);
  return acc;
}

// visit the 4 elements a lane holds in an accumulator tile: f(row, col, value)
template <class F>
__device__ __forceinline__ void tile_each(const f32x4& acc, int m0, int n0, F&& f) {
  const int lane = threadIdx.x & 63, lr = lane & 15, g = lane >> 4;
#pragma unroll
  for (int r = 0; r < 4; ++r) f(m0 + 4 * g + r, n0 + lr, acc[r]);
}

// Matrices of R (DK x DV) and dDelta (C x DV) per chunk slot are stored in
// accumulator tiles grouped by 16-column block: element (row, col) of a
// matrix with NR rows lives at
//   (((col / 16) * (NR / 16) + row / 16) * 64 + 16 ((row % 16) / 4) + col % 16) * 4 + row % 4.
template <int NR>
__device__ __forceinline__ size_t tile_index(int row, int col) {
  const int lane = 16 * ((row & 15) >> 2) + (col & 15);
  return ((size_t)((col >> 4) * (NR / 16) + (row >> 4)) * 64 + lane) * 4 + (row & 3);
}

// per-slot backward workspace (bytes); Kt and -W^T are the reverse chain's
// operands, stored in ESZ-byte elements (bf16 for bf16 inputs, fp32 for fp32)
template <int DK, int DV, int ESZ>
struct BwdSlot {
  static constexpr size_t kKt = (size_t)C * DK * ESZ;   // Kt [C][DK]
  static constexpr size_t kWnT = (size_t)DK * C * ESZ;  // -W^T [DK][C]
  static constexpr size_t kR = (size_t)DK * DV * 4;   // R, fp32 tiles
  static constexpr size_t kDd = (size_t)C * DV * 4;   // dDelta, fp32 tiles
  static constexpr size_t kX = (size_t)C * C * 4;     // X, fp32 [C][C]
  static constexpr size_t kDbp = (size_t)DK * DV * 4; // dB', fp32 [DK][DV]
  // d > 128 (bf16 inputs at d_k = d_v = 256): the C x d fp32 arrays of the
  // local and gradient kernels (and the gradient kernel's G) do not fit the
  // LDS and live here instead, one region of C x max(DK, DV) per array, each
  // written once per launch
  static constexpr bool kWide = DK > 128 || DV > 128;
  static constexpr int DM = DK > DV ? DK : DV;
  static constexpr size_t kArr = (size_t)C * DM * 4;
  static constexpr int kArrays = 7;
  static constexpr size_t kScr = kWide ? kArrays * kArr : 0;
  static constexpr size_t oKt = 0, oWnT = oKt + kKt, oR = oWnT + kWnT, oDd = oR + kR, oX = oDd + kDd,
                          oDbp = oX + kX, oScr = oDbp + kDbp, bytes = oScr + kScr;
};

// Chunk scalars shared by the two per-chunk kernels.
struct ChunkScalars {
  float g[C], beta[C], gam[C], Gam[C], e[C];
};

// gamma, Gamma, e from token tid's g and beta (threads tid < C; padding
// tokens pass 0), loaded by the caller ahead of its other staging.
__device__ __forceinline__ void chunk_scalars_from(ChunkScalars& cs, float g_t, float beta_t) {
  const int tid = threadIdx.x;
  if (tid < C) {
    cs.g[tid] = g_t;
    cs.beta[tid] = beta_t;
  }
  __syncthreads();
  if (tid == 0) {
    float acc = cs.g[0];
    cs.gam[0] = acc;
    for (int t = 1; t < C; ++t) {
      acc = acc + cs.g[t];
      cs.gam[t] = acc;
    }
  }
  __syncthreads();
  if (tid < C) {
    cs.Gam[tid] = expf(cs.gam[tid]);
    cs.e[tid] = expf(cs.gam[C - 1] - cs.gam[tid]);
  }
  __syncthreads();
}

// g, beta of the chunk's n real tokens (padding: 0), gamma, Gamma, e.
template <class D>
__device__ __forceinline__ void chunk_scalars(ChunkScalars& cs, const typename D::T* g, const typename D::T* beta,
                                              size_t row0, int H, int n) {
  const int tid = threadIdx.x;
  if (tid < C) {
    cs.g[tid] = tid < n ? D::load(g, row0 + (size_t)tid * H) : 0.f;
    cs.beta[tid] = tid < n ? D::load(beta, row0 + (size_t)tid * H) : 0.f;
  }
  __syncthreads();
  if (tid == 0) {
    float acc = cs.g[0];
    cs.gam[0] = acc;
    for (int t = 1; t < C; ++t) {
      acc = acc + cs.g[t];
      cs.gam[t] = acc;
    }
  }
  __syncthreads();
  if (tid < C) {
    cs.Gam[tid] = expf(cs.gam[tid]);
    cs.e[tid] = expf(cs.gam[C - 1] - cs.gam[tid]);
  }
  __syncthreads();
}

// X = (I + A)^{-1} for strictly lower A, one wave, lane = column s; the same
// blocked right-looking substitution as the forward, from the identity.
// A is read from At[s][t] = A[t][s]; X is written to Xo[t][s] (full matrix).
template <int LDA, int LDX>
__device__ __forceinline__ void unit_lower_inverse(const float (*At)[LDA], float (*Xo)[LDX]) {
  const int s = threadIdx.x & 63;
#pragma unroll
  for (int Bk = 0; Bk < C / 16; ++Bk) {
    float x[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) x[q] = (16 * Bk + q == s) ? 1.f : 0.f;
#pragma unroll 2
    for (int r = 0; r < 16 * Bk; ++r) {
      const float xr = Xo[r][s];
#pragma unroll
      for (int q = 0; q < 16; ++q) x[q] = __builtin_fmaf(-At[r][16 * Bk + q], xr, x[q]);
    }
#pragma unroll
    for (int r = 0; r < 15; ++r) {
#pragma unroll
      for (int q = r + 1; q < 16; ++q) x[q] = __builtin_fmaf(-At[16 * Bk + r][16 * Bk + q], x[r], x[q]);
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) Xo[16 * Bk + q][s] = x[q];
  }
}

}  // namespace bwd
}  // namespace cpr
