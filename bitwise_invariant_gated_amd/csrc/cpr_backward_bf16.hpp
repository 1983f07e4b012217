// Backward of the CPR Gated DeltaNet layer for bf16 inputs: per-chunk stages
// with every operand staged in LDS or read as 16-byte lane vectors.
//
// The gradient is the one written out in cpr_backward.hpp (chunk / WY form,
// exact in exact arithmetic).  For a chunk of n <= C tokens (padded to C with
// k = q = v = dO = 0, g = beta = 0), start state B (d_k x d_v) and end-state
// adjoint dB':
//   local     (before the reverse chain)
//     L = strict lower(beta_t D G), X = (I + L)^{-1}, P = (Q K^T) .* D
//     W = X diag(beta Gamma) K,  Kt = diag(e) K
//     Ddl = P^T dO,  R = (diag(Gamma) Q)^T dO - W^T Ddl
//   reverse chain   dB = Gamma_n dB' + R + (-W^T) Kt dB'   (bf16 operands)
//   state     (after it)
//     Dd = Ddl + diag(e) (K dB'),  Delta = X diag(beta) (V - diag(Gamma) K B)  (= X diag(beta) V - W B)
//     QB = dO B^T,  dWn = Dd B^T (= -dW),  dKt = Delta dB'^T,  dGamma_n = <dB', B>
//   local gradients
//     dPD = (dO Delta^T) .* D,  dQ = diag(Gamma) QB + dPD K
//     dV = diag(beta) X^T Dd,  TW = T^T dW = -diag(beta) X^T dWn
//     dT = Dd V^T - (dWn K^T) diag(Gamma),  dX = dT diag(beta)
//     dA = -X^T (dX X^T) (strict lower),  dG = dA .* beta_t D
//     dK = dPD^T Q + (dG + dG^T) K + diag(e) dKt + diag(Gamma) TW
//     dbeta = colsum(X .* dT) + rowsum(dA .* D .* G)
//     dgamma = rowsum(Z) - colsum(Z) + (dGamma_out + dGamma_W) Gamma - de e
//              (+ dGamma_n Gamma_n + sum(de e) at t = C - 1),
//       Z = dPD .* QK + beta_t dA .* D .* G,  dGamma_out = <QB, Q> per row,
//       dGamma_W = <TW, K> per row,  de = <dKt, K> per row
//     dg = reverse cumsum of dgamma.
// Products with an fp32 operand run on v_mfma_f32_16x16x16_bf16 with that
// operand split into bf16 hi + lo parts (three products per 16-wide k block,
// two where the other operand is the layer's bf16 k, q, v or dO; mma16s
// below); G and Q K^T take their exact bf16 operands on
// v_mfma_f32_16x16x32_bf16, the reverse chain bf16 operands as the forward
// chain, and the inverse's blocks below the diagonal the forward's fp32
// routine.  Every reduction has a fixed order, so reruns give identical bits.
#pragma once

#include "cpr_backward.hpp"
#include "cpr_device.hpp"

namespace cpr {
namespace bwdb {

using namespace mfma;
constexpr int C = kChunk;

// Per (chunk slot, head) workspace.  TL = accumulator-tile order (element
// (r, c) of a matrix with NR rows at (((c/16) (NR/16) + r/16) 64 + 16 ((r%16)/4)
// + c%16) 4 + r%4); RM = row-major.
template <int DK, int DV>
struct Slot {
  static constexpr size_t oKTF = 0;                                 // Kt fragments (chain phase 1)
  static constexpr size_t oWNF = oKTF + (size_t)C * DK * 2;         // -W^T fragments (chain phase 2)
  static constexpr size_t oR = oWNF + (size_t)DK * C * 2;           // R, TL (DK rows)
  static constexpr size_t oDbp = oR + (size_t)DK * DV * 4;          // dB', TL (DK rows)
  static constexpr size_t oX = oDbp + (size_t)DK * DV * 4;          // X, RM
  static constexpr size_t oDdl = oX + (size_t)C * C * 4;            // Ddl, TL (C rows)
  static constexpr size_t oDd = oDdl + (size_t)C * DV * 4;          // Dd, RM
  static constexpr size_t oDe = oDd + (size_t)C * DV * 4;           // Delta, RM
  static constexpr size_t oQB = oDe + (size_t)C * DV * 4;           // QB, RM
  static constexpr size_t oDWn = oQB + (size_t)C * DK * 4;          // dWn, RM
  static constexpr size_t oDKt = oDWn + (size_t)C * DK * 4;         // dKt, RM
  static constexpr size_t oDGn = oDKt + (size_t)C * DK * 4;         // dGamma_n
  static constexpr size_t bytes = oDGn + 256;
};

// ---------------------------------------------------------------------------
// operand helpers (lane l = 16 g + c)


// fp32 products at the bf16 MFMA rate.  A lane's operand x (four values of a
// 16-wide k block: lane 16 g + c holds index 4 g + {0..3}) is split as x = hi + lo with
// hi = bf16(x) and lo = bf16(x - hi) (x - hi is exact in fp32), which holds x
// to about 2^-17 |x|; a product then takes hi*hi + hi*lo + lo*hi, in that
// order, on v_mfma_f32_16x16x16_bf16 (the dropped lo*lo term is about 2^-17
// of the product).  An operand that is already bf16 (the layer's k, q, v,
// dO) has lo = 0 and takes two terms.  One bf16 MFMA of k = 16 stands for
// four fp32 ones and costs a quarter of one of them.
typedef short s16x4 __attribute__((ext_vector_type(4)));
struct Split4 {
  s16x4 hi, lo;
};

__device__ __forceinline__ Split4 split4(const f32x4& x) {
  const uint32_t h0 = pack2(x[0], x[1]), h1 = pack2(x[2], x[3]);
  const uint32_t l0 = pack2(x[0] - __uint_as_float(h0 << 16), x[1] - __uint_as_float(h0 & 0xffff0000u));
  const uint32_t l1 = pack2(x[2] - __uint_as_float(h1 << 16), x[3] - __uint_as_float(h1 & 0xffff0000u));
  return Split4{__builtin_bit_cast(s16x4, u32x2{h0, h1}), __builtin_bit_cast(s16x4, u32x2{l0, l1})};
}

__device__ __forceinline__ f32x4 mfma_bf16_k16(s16x4 a, s16x4 b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mma16s(const Split4& a, const Split4& b, f32x4 acc) {
  acc = mfma_bf16_k16(a.hi, b.hi, acc);
  acc = mfma_bf16_k16(a.hi, b.lo, acc);
  return mfma_bf16_k16(a.lo, b.hi, acc);
}

// a exact in bf16
__device__ __forceinline__ f32x4 mma16s(s16x4 a, const Split4& b, f32x4 acc) {
  acc = mfma_bf16_k16(a, b.hi, acc);
  return mfma_bf16_k16(a, b.lo, acc);
}

// b exact in bf16
__device__ __forceinline__ f32x4 mma16s(const Split4& a, s16x4 b, f32x4 acc) {
  acc = mfma_bf16_k16(a.hi, b, acc);
  return mfma_bf16_k16(a.lo, b, acc);
}

__device__ __forceinline__ float bfv(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

// the bits of M[r][k0 + 4 g + {0..3}] of a row-major bf16 matrix (8-byte aligned rows)
__device__ __forceinline__ s16x4 row4_bits(const uint16_t* M, int ld, int r, int k0, int g) {
  return __builtin_bit_cast(s16x4, *reinterpret_cast<const u32x2*>(M + (size_t)r * ld + k0 + 4 * g));
}

// the bits of M[k0 + 4 g + {0..3}][col] of a row-major bf16 matrix
__device__ __forceinline__ s16x4 col4_bits(const uint16_t* M, int ld, int k0, int col, int g) {
  const uint16_t* p = M + (size_t)(k0 + 4 * g) * ld + col;
  return s16x4{(short)p[0], (short)p[ld], (short)p[2 * ld], (short)p[3 * ld]};
}

// M[k0 + 4 g + {0..3}][col] of a row-major bf16 matrix
__device__ __forceinline__ f32x4 col4_bf(const uint16_t* M, int ld, int k0, int col, int g) {
  const uint16_t* p = M + (size_t)(k0 + 4 * g) * ld + col;
  return f32x4{bfv(p[0]), bfv(p[ld]), bfv(p[2 * ld]), bfv(p[3 * ld])};
}

// M[r][k0 + 4 g + {0..3}] of a row-major fp32 matrix (16-byte aligned rows)
__device__ __forceinline__ f32x4 row4_f(const float* M, int ld, int r, int k0, int g) {
  return *reinterpret_cast<const f32x4*>(M + (size_t)r * ld + k0 + 4 * g);
}

// M[k0 + 4 g + {0..3}][col] of a row-major fp32 matrix
__device__ __forceinline__ f32x4 col4_f(const float* M, int ld, int k0, int col, int g) {
  const float* p = M + (size_t)(k0 + 4 * g) * ld + col;
  return f32x4{p[0], p[ld], p[2 * ld], p[3 * ld]};
}

// this lane's 16 bytes of TL tile (row block rb, column block cb) of a matrix with NR rows
template <int NR>
__device__ __forceinline__ f32x4 tl4(const float* T, int rb, int cb, int lane) {
  return *reinterpret_cast<const f32x4*>(T + ((size_t)(cb * (NR / 16) + rb) * 64 + lane) * 4);
}

template <int NR>
__device__ __forceinline__ void st_tl(float* T, int rb, int cb, const f32x4& acc, int lane) {
  *reinterpret_cast<f32x4*>(T + ((size_t)(cb * (NR / 16) + rb) * 64 + lane) * 4) = acc;
}

// accumulator tile (rows r0 + 4 g + i, column c0 + c) into a row-major fp32 matrix
__device__ __forceinline__ void st_rm(float* M, int ld, int r0, int c0, const f32x4& acc, int lane) {
  const int c = lane & 15, g = lane >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) M[(size_t)(r0 + 4 * g + i) * ld + c0 + c] = acc[i];
}

// sum over the 16 lanes of a lane group by DPP row rotations (8, 4, 2, 1);
// callers use the value in lane c = 0, whose addition order is fixed
template <int R>
__device__ __forceinline__ float row_ror(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 + R, 0xf, 0xf, false));
}
__device__ __forceinline__ float sum16(float x) {
  x += row_ror<8>(x);
  x += row_ror<4>(x);
  x += row_ror<2>(x);
  x += row_ror<1>(x);
  return x;
}

// Staging in two halves, so that a stage issues all of its global loads
// before its first LDS write (one memory round trip, not one per piece).
// Rows t < n of a [T, H, D] bf16 tensor (row t at src + (row0 + t H) D) over
// NT threads; rows t >= n load row n - 1 (n >= 1) and are stored as zeros.
template <int D, int NT>
struct RowLoads {
  static constexpr int M = C * D / 8 / NT;
  static_assert(M * NT == C * D / 8, "rows split over the threads");
  u32x4 w[M];
  __device__ __forceinline__ void load(const uint16_t* __restrict__ src, size_t row0, int H, int n) {
    const int last = n > 0 ? n - 1 : 0;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const int idx = threadIdx.x + m * NT, t = min(idx / (D / 8), last), c8 = (idx % (D / 8)) * 8;
      w[m] = *reinterpret_cast<const u32x4*>(src + (row0 + (size_t)t * H) * D + c8);
    }
  }
  template <int LD>
  __device__ __forceinline__ void store(uint16_t (*dst)[LD], int n) const {
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const int idx = threadIdx.x + m * NT, t = idx / (D / 8), c8 = (idx % (D / 8)) * 8;
      *reinterpret_cast<u32x4*>(&dst[t][c8]) = t < n ? w[m] : zero;
    }
  }
};

// The slot's X (C x C fp32, row-major) over NT threads.
template <int NT>
struct XLoads {
  static constexpr int M = C * C / 4 / NT;
  static_assert(M * NT == C * C / 4, "X split over the threads");
  f32x4 w[M];
  __device__ __forceinline__ void load(const float* __restrict__ Xg) {
#pragma unroll
    for (int m = 0; m < M; ++m) w[m] = reinterpret_cast<const f32x4*>(Xg)[threadIdx.x + m * NT];
  }
  template <int LD>
  __device__ __forceinline__ void store(float (*X)[LD]) const {
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const int idx = threadIdx.x + m * NT, t = idx / (C / 4), s4 = (idx % (C / 4)) * 4;
      *reinterpret_cast<f32x4*>(&X[t][s4]) = w[m];
    }
  }
};

// token threadIdx.x's g and beta (threads < C), 0 past the chunk's n tokens
__device__ __forceinline__ void load_scalars(const uint16_t* gp, const uint16_t* bp, size_t row0, int H, int n,
                                             float& g_t, float& b_t) {
  const int last = n > 0 ? n - 1 : 0, t = min((int)threadIdx.x, last);
  const float g = Bf16::load(gp, row0 + (size_t)t * H), b = Bf16::load(bp, row0 + (size_t)t * H);
  const bool real = (int)threadIdx.x < n;
  g_t = real ? g : 0.f;
  b_t = real ? b : 0.f;
}

// tiles on or below the diagonal of a C x C matrix: index q in [0, 10)
__device__ __forceinline__ void lower_tile(int q, int& tm, int& tn) {
  tm = q < 1 ? 0 : q < 3 ? 1 : q < 6 ? 2 : 3;
  tn = q - tm * (tm + 1) / 2;
}

// ===========================================================================
// local stage (64 W threads): L, X, P, W, Kt and -W^T fragments, Ddl, R
template <int DK, int DV>
struct LocalLds {
  static constexpr int kLK = DK + 8, kLV = DV + 8, kLA = C + 4;
  uint16_t K[C][kLK];
  uint16_t Q[C][kLK];
  uint16_t dO[C][kLV];
  float A[C][kLA];  // L, then X^T on and above the diagonal
  float P[C][kLA];  // P[t][s]
  float Ddl[C * DV];  // TL
  bwd::ChunkScalars cs;
};

template <int DK, int DV, int W>
__device__ __forceinline__ void local_stage(LocalLds<DK, DV>& sm, const uint16_t* q, const uint16_t* k,
                                            const uint16_t* d_o, const uint16_t* gp, const uint16_t* bp,
                                            size_t row0, int H, size_t kq0, int Hk, int n,
                                            uint8_t* __restrict__ slot, float* __restrict__ gamn) {
  typedef Slot<DK, DV> Sl;
  typedef LocalLds<DK, DV> Lds;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 15, g = lane >> 4;
  // d-wide products: wave w makes the 16-wide tiles w, w + W, ...
  static_assert((DK / 16) % W == 0 && (DV / 16) % W == 0 && W >= 4, "tiles per wave");
  {
    RowLoads<DK, 64 * W> rk, rq;
    RowLoads<DV, 64 * W> rd;
    float g_t, b_t;
    rk.load(k, kq0, Hk, n);
    rq.load(q, kq0, Hk, n);
    rd.load(d_o, row0, H, n);
    load_scalars(gp, bp, row0, H, n, g_t, b_t);
    rk.store(sm.K, n);
    rq.store(sm.Q, n);
    rd.store(sm.dO, n);
    bwd::chunk_scalars_from(sm.cs, g_t, b_t);  // synchronises
  }
  const bwd::ChunkScalars& cs = sm.cs;
  // L (strictly lower) and P (lower, diagonal included) from the 10 lower tiles each
  for (int q2 = wave; q2 < 20; q2 += W) {
    int tm, tn;
    lower_tile(q2 % 10, tm, tn);
    const bool isP = q2 >= 10;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < DK / 32; ++kb)
      acc = mma(frag_row(isP ? &sm.Q[16 * tm + lr][0] : &sm.K[16 * tm + lr][0], 32 * kb, g),
                frag_row(&sm.K[16 * tn + lr][0], 32 * kb, g), acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * tm + 4 * g + r, s = 16 * tn + lr;
      if (!isP) {
        if (s < t) sm.A[t][s] = (cs.beta[t] * expf(cs.gam[t] - cs.gam[s])) * acc[r];
      } else {
        sm.P[t][s] = (s <= t) ? acc[r] * expf(cs.gam[t] - cs.gam[s]) : 0.f;
      }
    }
  }
  for (int idx = tid; idx < C * C; idx += 64 * W) {
    const int t = idx / C, s = idx % C;
    if ((s >> 4) > (t >> 4)) sm.P[t][s] = 0.f;
  }
  __syncthreads();
  if (wave == 0) {
    inverse_diag_blocks(sm.A, lane);
  } else {
    // Kt fragments (chain phase 1, the slot's first 16 KB): fragment (kb, tm)
    for (int f = wave - 1; f < (DK / 32) * (C / 16); f += W - 1) {
      const int kb = f / (C / 16), tm = f % (C / 16), t = 16 * tm + lr;
      const u32x4 raw = frag_row(&sm.K[t][0], 32 * kb, g);
      const float et = cs.e[t];
      u32x4 out;
#pragma unroll
      for (int w = 0; w < 4; ++w)
        out[w] = pack2(et * __uint_as_float(raw[w] << 16), et * __uint_as_float(raw[w] & 0xffff0000u));
      *reinterpret_cast<u32x4*>(slot + Sl::oKTF + ((size_t)f * 64 + lane) * 16) = out;
    }
  }
  __syncthreads();
  inverse_below_diag(sm.A, wave, lane);
  // W tiles (tm, it), it = wave + W p; X[t][s] = A[s][t] for s <= t.  The
  // K column block is shared by the four row tiles, whose accumulations
  // interleave.
  constexpr int NI = DK / (16 * W), NJ = DV / (16 * W), NB = C / 16;
  f32x4 Wt[NI][NB];
#pragma unroll
  for (int p = 0; p < NI; ++p) {
    const int it = wave + W * p;
#pragma unroll
    for (int tm = 0; tm < NB; ++tm) Wt[p][tm] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sb = 0; sb < NB; ++sb) {
      const s16x4 b = col4_bits(&sm.K[0][0], Lds::kLK, 16 * sb, 16 * it + lr, g);
      f32x4 bg;
#pragma unroll
      for (int m = 0; m < 4; ++m) bg[m] = cs.beta[16 * sb + 4 * g + m] * cs.Gam[16 * sb + 4 * g + m];
#pragma unroll
      for (int tm = sb; tm < NB; ++tm) {
        const int t = 16 * tm + lr;
        f32x4 a;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int s = 16 * sb + 4 * g + m;
          a[m] = (s <= t) ? sm.A[s][t] * bg[m] : 0.f;
        }
        Wt[p][tm] = mma16s(split4(a), b, Wt[p][tm]);
      }
    }
    // -W^T fragments (chain phase 2): fragment (kb, it)
#pragma unroll
    for (int kb = 0; kb < C / 32; ++kb) {
      const f32x4& x = Wt[p][2 * kb];
      const f32x4& y = Wt[p][2 * kb + 1];
      const u32x4 out = {pack2(-x[0], -x[1]), pack2(-x[2], -x[3]), pack2(-y[0], -y[1]), pack2(-y[2], -y[3])};
      *reinterpret_cast<u32x4*>(slot + Sl::oWNF + ((size_t)(kb * (DK / 16) + it) * 64 + lane) * 16) = out;
    }
  }
  // Ddl = P^T dO, tiles (sb, jt), jt = wave + W p; P[t][s] = 0 for t < s
  float* Ddlg = reinterpret_cast<float*>(slot + Sl::oDdl);
#pragma unroll
  for (int p = 0; p < NJ; ++p) {
    const int jt = wave + W * p;
    f32x4 acc[NB];
#pragma unroll
    for (int sb = 0; sb < NB; ++sb) acc[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int tb = 0; tb < NB; ++tb) {
      const s16x4 b = col4_bits(&sm.dO[0][0], Lds::kLV, 16 * tb, 16 * jt + lr, g);
#pragma unroll
      for (int sb = 0; sb <= tb; ++sb) {
        f32x4 a;
#pragma unroll
        for (int m = 0; m < 4; ++m) a[m] = sm.P[16 * tb + 4 * g + m][16 * sb + lr];
        acc[sb] = mma16s(split4(a), b, acc[sb]);
      }
    }
#pragma unroll
    for (int sb = 0; sb < NB; ++sb) {
      st_tl<C>(sm.Ddl, sb, jt, acc[sb], lane);
      st_tl<C>(Ddlg, sb, jt, acc[sb], lane);
    }
  }
  __syncthreads();
  // R = (diag(Gamma) Q)^T dO - W^T Ddl, tiles (it, jt) with this wave's it;
  // the eight column tiles accumulate together
  float* Rg = reinterpret_cast<float*>(slot + Sl::oR);
#pragma unroll
  for (int p = 0; p < NI; ++p) {
    const int it = wave + W * p;
    f32x4 acc[DV / 16];
#pragma unroll
    for (int jt = 0; jt < DV / 16; ++jt) acc[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int tb = 0; tb < NB; ++tb) {
      f32x4 a = col4_bf(&sm.Q[0][0], Lds::kLK, 16 * tb, 16 * it + lr, g);
#pragma unroll
      for (int m = 0; m < 4; ++m) a[m] *= cs.Gam[16 * tb + 4 * g + m];
      const f32x4& w = Wt[p][tb];
      const Split4 as = split4(a), wn = split4(f32x4{-w[0], -w[1], -w[2], -w[3]});
#pragma unroll
      for (int jt = 0; jt < DV / 16; ++jt) {
        acc[jt] = mma16s(as, col4_bits(&sm.dO[0][0], Lds::kLV, 16 * tb, 16 * jt + lr, g), acc[jt]);
        acc[jt] = mma16s(wn, split4(tl4<C>(sm.Ddl, tb, jt, lane)), acc[jt]);
      }
    }
#pragma unroll
    for (int jt = 0; jt < DV / 16; ++jt) st_tl<DK>(Rg, it, jt, acc[jt], lane);
  }
  // X (row-major, zero above the diagonal) and Gamma_n
  float* Xg = reinterpret_cast<float*>(slot + Sl::oX);
  for (int idx = tid; idx < C * C; idx += 64 * W) {
    const int t = idx / C, s = idx % C;
    Xg[idx] = (s <= t) ? sm.A[s][t] : 0.f;
  }
  if (tid == 0) *gamn = cs.Gam[C - 1];
}

// ===========================================================================
// state stage (64 W threads): Dd, Delta, QB, dWn, dKt, dGamma_n
//
// Columns 32 jb .. 32 jb + 31 of a TL state (DK rows), over NT threads: load()
// issues the reads into registers, store() writes them into Bs row-major, so
// a block's reads can be in flight while the previous block is consumed.
template <int DK, int NT>
struct ColLoads {
  static constexpr int M = 2 * (DK / 16) * 64 / NT;
  static_assert(M * NT == 2 * (DK / 16) * 64, "columns split over the threads");
  f32x4 w[M];
  __device__ __forceinline__ void load(const float* __restrict__ T, int jb) {
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const int pc = threadIdx.x + m * NT, tt = pc >> 6, l = pc & 63;
      w[m] = tl4<DK>(T, tt % (DK / 16), 2 * jb + tt / (DK / 16), l);
    }
  }
  template <int LB>
  __device__ __forceinline__ void store(float (*Bs)[LB]) const {
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const int pc = threadIdx.x + m * NT, tt = pc >> 6, l = pc & 63;
      const int ct = tt / (DK / 16), im = tt % (DK / 16), c = l & 15, g = l >> 4;
#pragma unroll
      for (int r = 0; r < 4; ++r) Bs[16 * im + 4 * g + r][16 * ct + c] = w[m][r];
    }
  }
};

template <int DK, int DV, int W, class SM>
__device__ __forceinline__ void state_stage(SM& sm, const uint16_t* k, const uint16_t* v,
                                            const uint16_t* d_o, const uint16_t* gp, const uint16_t* bp,
                                            size_t row0, int H, size_t kq0, int Hk, int n,
                                            const float* __restrict__ B, uint8_t* __restrict__ slot) {
  typedef Slot<DK, DV> Sl;
  typedef SM Lds;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 15, g = lane >> 4;
  // wave w makes the 16-wide row / column tiles w, w + W, ...
  static_assert((DK / 16) % W == 0 && (DV / 16) % W == 0, "tiles per wave");
  constexpr int NI = DK / (16 * W), NJ = DV / (16 * W);
  const float* Xg = reinterpret_cast<const float*>(slot + Sl::oX);
  const float* Ddlg = reinterpret_cast<const float*>(slot + Sl::oDdl);
  const float* dBp = reinterpret_cast<const float*>(slot + Sl::oDbp);
  constexpr int NB = C / 16;
  // the first column tile's dB', B and Ddl tiles are loaded with the staging
  // (a barrier waits only for LDS, so they stay in flight across it)
  f32x4 d0[DK / 16], b0[DK / 16], l0[NB];
#pragma unroll
  for (int ib = 0; ib < DK / 16; ++ib) {
    d0[ib] = tl4<DK>(dBp, ib, wave, lane);
    b0[ib] = tl4<DK>(B, ib, wave, lane);
  }
  {
    RowLoads<DK, 64 * W> rk;
    RowLoads<DV, 64 * W> rv, rd;
    XLoads<64 * W> rx;
    float g_t, b_t;
    rk.load(k, kq0, Hk, n);
    rv.load(v, row0, H, n);
    rd.load(d_o, row0, H, n);
    rx.load(Xg);
    load_scalars(gp, bp, row0, H, n, g_t, b_t);
#pragma unroll
    for (int tm = 0; tm < NB; ++tm) l0[tm] = tl4<C>(Ddlg, tm, wave, lane);
    rk.store(sm.K, n);
    rv.store(sm.V, n);
    rd.store(sm.dO, n);
    rx.store(sm.X);
    bwd::chunk_scalars_from(sm.cs, g_t, b_t);  // synchronises
  }
  const bwd::ChunkScalars& cs = sm.cs;
  float* Ddg = reinterpret_cast<float*>(slot + Sl::oDd);
  float* Deg = reinterpret_cast<float*>(slot + Sl::oDe);
  // Column tile jt = wave + W p: the dB' and B tiles of the column block are
  // loaded once; the four row tiles accumulate together.
  //   Dd    = Ddl + Kt dB'
  //   KB    = K B                                   (kept in registers)
  //   Delta = X diag(beta) (V - diag(Gamma) KB)     (= X diag(beta) V - W B)
  // the QB phase's first 32 columns of B
  ColLoads<DK, 64 * W> cols;
  cols.load(B, 0);
  // <dB', B>: this lane's share (the tiles it loads below, p, ib, element
  // ascending), summed over the threads at the end in a fixed order
  float gdot = 0.f;
#pragma unroll
  for (int p = 0; p < NJ; ++p) {
    const int jt = wave + W * p;
    Split4 bD[DK / 16], bB[DK / 16];
#pragma unroll
    for (int ib = 0; ib < DK / 16; ++ib) {
      const f32x4 d = p == 0 ? d0[ib] : tl4<DK>(dBp, ib, jt, lane), b = p == 0 ? b0[ib] : tl4<DK>(B, ib, jt, lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) gdot = __builtin_fmaf(b[r], d[r], gdot);
      bD[ib] = split4(d);
      bB[ib] = split4(b);
    }
    // Kt dB' as diag(e) (K dB'): K is exact in bf16
    f32x4 kd[NB], kb[NB];
#pragma unroll
    for (int tm = 0; tm < NB; ++tm) kd[tm] = kb[tm] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ib = 0; ib < DK / 16; ++ib)
#pragma unroll
      for (int tm = 0; tm < NB; ++tm) {
        const s16x4 a = row4_bits(&sm.K[0][0], Lds::kLK, 16 * tm + lr, 16 * ib, g);
        kd[tm] = mma16s(a, bD[ib], kd[tm]);
        kb[tm] = mma16s(a, bB[ib], kb[tm]);
      }
    f32x4 dd[NB];
#pragma unroll
    for (int tm = 0; tm < NB; ++tm) {
      const f32x4 ddl = p == 0 ? l0[tm] : tl4<C>(Ddlg, tm, jt, lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) dd[tm][r] = __builtin_fmaf(cs.e[16 * tm + 4 * g + r], kd[tm][r], ddl[r]);
      st_rm(&sm.Dd[0][0], Lds::kLD, 16 * tm, 16 * jt, dd[tm], lane);
      st_rm(Ddg, DV, 16 * tm, 16 * jt, dd[tm], lane);
    }
    f32x4 de[NB];
#pragma unroll
    for (int tm = 0; tm < NB; ++tm) de[tm] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sb = 0; sb < NB; ++sb) {
      // B operand: rows s = 16 sb + 4 g + m of V - diag(Gamma) KB, column 16 jt + c
      const f32x4 v = col4_bf(&sm.V[0][0], Lds::kLV, 16 * sb, 16 * jt + lr, g);
      f32x4 b;
#pragma unroll
      for (int m = 0; m < 4; ++m) b[m] = __builtin_fmaf(-cs.Gam[16 * sb + 4 * g + m], kb[sb][m], v[m]);
      const Split4 bs = split4(b);
#pragma unroll
      for (int tm = sb; tm < NB; ++tm) {
        f32x4 a = row4_f(&sm.X[0][0], Lds::kLX, 16 * tm + lr, 16 * sb, g);
#pragma unroll
        for (int m = 0; m < 4; ++m) a[m] *= cs.beta[16 * sb + 4 * g + m];
        de[tm] = mma16s(split4(a), bs, de[tm]);
      }
    }
#pragma unroll
    for (int tm = 0; tm < NB; ++tm) {
      st_rm(&sm.De[0][0], Lds::kLD, 16 * tm, 16 * jt, de[tm], lane);
      st_rm(Deg, DV, 16 * tm, 16 * jt, de[tm], lane);
    }
  }
  sm.red[tid] = gdot;
  __syncthreads();
  // QB = dO B^T and dWn = Dd B^T, then dKt = Delta dB'^T, 32 columns of B / dB' at a time
  f32x4 QB[NI][C / 16], DW[NI][C / 16];
#pragma unroll
  for (int p = 0; p < NI; ++p)
#pragma unroll
    for (int tm = 0; tm < C / 16; ++tm) QB[p][tm] = DW[p][tm] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int jb = 0; jb < DV / 32; ++jb) {
    cols.store(sm.Bs);
    __syncthreads();
    cols.load(jb + 1 < DV / 32 ? B : dBp, jb + 1 < DV / 32 ? jb + 1 : 0);  // next block (or dB's first)
#pragma unroll
    for (int p = 0; p < NI; ++p) {
      const int it = wave + W * p;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const Split4 b = split4(row4_f(&sm.Bs[0][0], Lds::kLB, 16 * it + lr, 16 * kk, g));
#pragma unroll
        for (int tm = 0; tm < C / 16; ++tm) {
          QB[p][tm] = mma16s(row4_bits(&sm.dO[0][0], Lds::kLV, 16 * tm + lr, 32 * jb + 16 * kk, g), b, QB[p][tm]);
          DW[p][tm] =
              mma16s(split4(row4_f(&sm.Dd[0][0], Lds::kLD, 16 * tm + lr, 32 * jb + 16 * kk, g)), b, DW[p][tm]);
        }
      }
    }
    __syncthreads();
  }
  float* QBg = reinterpret_cast<float*>(slot + Sl::oQB);
  float* DWg = reinterpret_cast<float*>(slot + Sl::oDWn);
#pragma unroll
  for (int p = 0; p < NI; ++p)
#pragma unroll
    for (int tm = 0; tm < C / 16; ++tm) {
      st_rm(QBg, DK, 16 * tm, 16 * (wave + W * p), QB[p][tm], lane);
      st_rm(DWg, DK, 16 * tm, 16 * (wave + W * p), DW[p][tm], lane);
      QB[p][tm] = f32x4{0.f, 0.f, 0.f, 0.f};  // reused for dKt
    }
  for (int jb = 0; jb < DV / 32; ++jb) {
    cols.store(sm.Bs);  // block jb of dB', loaded during the previous block's products
    __syncthreads();
    if (jb + 1 < DV / 32) cols.load(dBp, jb + 1);
#pragma unroll
    for (int p = 0; p < NI; ++p) {
      const int it = wave + W * p;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const Split4 b = split4(row4_f(&sm.Bs[0][0], Lds::kLB, 16 * it + lr, 16 * kk, g));
#pragma unroll
        for (int tm = 0; tm < C / 16; ++tm)
          QB[p][tm] =
              mma16s(split4(row4_f(&sm.De[0][0], Lds::kLD, 16 * tm + lr, 32 * jb + 16 * kk, g)), b, QB[p][tm]);
      }
    }
    __syncthreads();
  }
  float* KTg = reinterpret_cast<float*>(slot + Sl::oDKt);
#pragma unroll
  for (int p = 0; p < NI; ++p)
#pragma unroll
    for (int tm = 0; tm < C / 16; ++tm) st_rm(KTg, DK, 16 * tm, 16 * (wave + W * p), QB[p][tm], lane);
  // dGamma_n = <dB', B> from the threads' shares (written to red before the
  // barriers above), in a fixed order
  {
    if (tid < 64) {  // lane l sums red[W l .. W l + W - 1], then the lanes in order
      float part = 0.f;
      for (int r = 0; r < W; ++r) part += sm.red[W * tid + r];
      float s = 0.f;
      for (int l = 0; l < 64; ++l) s += lane_bcast(part, l);
      if (tid == 0) *reinterpret_cast<float*>(slot + Sl::oDGn) = s;
    }
  }
}

// ===========================================================================
// local gradients (64 W threads): dq, dk, dv, dg, dbeta of the chunk's tokens
// The state and gradient stages of one (chunk slot, head) in one work-group:
// K, V, dO, X and the chunk scalars, staged by the state stage, stay in the
// LDS for the gradient stage; the two stages' other arrays share the rest.
template <int DK, int DV, int W>
struct StateGradLds {
  static constexpr int kLK = DK + 8, kLV = DV + 8, kLX = C + 4, kLD = DV + 4, kLB = 32 + 4;
  uint16_t K[C][kLK];
  uint16_t V[C][kLV];
  uint16_t dO[C][kLV];
  float X[C][kLX];
  bwd::ChunkScalars cs;
  union alignas(16) {
    struct {  // state stage
      float Dd[C][kLD];
      float De[C][kLD];
      float Bs[DK][kLB];
      float red[64 * W];
    };
    struct {  // gradient stage
      uint16_t Q[C][kLK];
      float dPD[C][kLX];
      float M2[C][kLX];
      float M3[C][kLX];
      float pGO[C][DK / 16], pGW[C][DK / 16], pDE[C][DK / 16];
      float rzP[C], czP[C], dbc[C], dbr[C], rzA[C], czA[C], dgo[C], de[C], dgam[C];
      float sum_de;
    };
  };
};

// K, V, dO, X and the chunk scalars are already in the LDS (the state stage
// of the same work-group put them there); only Q is loaded.
template <int DK, int DV, int W, class SM>
// dq and dk go to rows kq0 + t Hk of [T, Hk, DK] in bf16 or, when the key
// heads are shared (dq_part non-null), to the value head's rows row0 + t H of
// fp32 [T, H, DK] partials that a later pass sums over the group.
__device__ __forceinline__ void grad_stage(SM& sm, const uint16_t* q, const uint16_t* k,
                                           const uint16_t* v, const uint16_t* d_o, const uint16_t* gp,
                                           const uint16_t* bp, size_t row0, int H, size_t kq0, int Hk, int n,
                                           const uint8_t* __restrict__ slot, uint16_t* __restrict__ dq,
                                           uint16_t* __restrict__ dk, float* __restrict__ dq_part,
                                           float* __restrict__ dk_part, uint16_t* __restrict__ dv,
                                           float* __restrict__ dg, float* __restrict__ dbeta) {
  typedef Slot<DK, DV> Sl;
  typedef SM Lds;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 15, g = lane >> 4;
  // d-wide products: wave w makes the 16-wide tiles w, w + W, ...; C x C
  // products: wave w < C / 16 makes row or column block w
  static_assert((DK / 16) % W == 0 && (DV / 16) % W == 0 && W >= C / 16, "tiles per wave");
  constexpr int NI = DK / (16 * W), NJ = DV / (16 * W);
  const float* Xg = reinterpret_cast<const float*>(slot + Sl::oX);
  const float* Ddg = reinterpret_cast<const float*>(slot + Sl::oDd);
  const float* Deg = reinterpret_cast<const float*>(slot + Sl::oDe);
  const float* QBg = reinterpret_cast<const float*>(slot + Sl::oQB);
  const float* DWg = reinterpret_cast<const float*>(slot + Sl::oDWn);
  const float* KTg = reinterpret_cast<const float*>(slot + Sl::oDKt);
  constexpr int NB = C / 16;
  // Every global operand is loaded one phase ahead of its use (a barrier
  // waits only for LDS, so the loads stay in flight across it).
  const float dGn = *reinterpret_cast<const float*>(slot + Sl::oDGn);
  const int tn_p = wave % NB;  // the dPD phase's column block
  f32x4 bde_raw[DV / 16];
  {
    RowLoads<DK, 64 * W> rq;
    rq.load(q, kq0, Hk, n);
#pragma unroll
    for (int jb = 0; jb < DV / 16; ++jb) bde_raw[jb] = row4_f(Deg, DV, 16 * tn_p + lr, 16 * jb, g);
    rq.store(sm.Q, n);
    __syncthreads();
  }
  const bwd::ChunkScalars& cs = sm.cs;

  // the next phase's operands: QB (dQ), Dd and dWn columns (dV, TW)
  float qb[NI][NB][4];
  f32x4 bd_raw[NJ][NB], bw_raw[NI][NB];
#pragma unroll
  for (int p = 0; p < NI; ++p)
#pragma unroll
    for (int tm = 0; tm < NB; ++tm)
#pragma unroll
      for (int r = 0; r < 4; ++r) qb[p][tm][r] = QBg[(size_t)(16 * tm + 4 * g + r) * DK + 16 * (wave + W * p) + lr];
#pragma unroll
  for (int p = 0; p < NJ; ++p)
#pragma unroll
    for (int tb = 0; tb < NB; ++tb) bd_raw[p][tb] = col4_f(Ddg, DV, 16 * tb, 16 * (wave + W * p) + lr, g);
#pragma unroll
  for (int p = 0; p < NI; ++p)
#pragma unroll
    for (int tb = 0; tb < NB; ++tb) bw_raw[p][tb] = col4_f(DWg, DK, 16 * tb, 16 * (wave + W * p) + lr, g);

  // dPD = (dO Delta^T) .* D (lower, diagonal included), Z_P = dPD .* QK^T;
  // wave w makes the tiles (w / NB + (W / NB) j, w % NB) (zero above the diagonal)
  {
    constexpr int NT2 = NB * NB / W;
    const int tn = tn_p;
    Split4 bde[DV / 16];
#pragma unroll
    for (int jb = 0; jb < DV / 16; ++jb) bde[jb] = split4(bde_raw[jb]);
    f32x4 acc[NT2], qk[NT2];
#pragma unroll
    for (int j = 0; j < NT2; ++j) acc[j] = qk[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jb = 0; jb < DV / 16; ++jb)
#pragma unroll
      for (int j = 0; j < NT2; ++j) {
        const int tm = wave / NB + (W / NB) * j;
        if (tm >= tn) acc[j] = mma16s(row4_bits(&sm.dO[0][0], Lds::kLV, 16 * tm + lr, 16 * jb, g), bde[jb], acc[j]);
      }
#pragma unroll
    for (int kb = 0; kb < DK / 32; ++kb) {
      const u32x4 kf = frag_row(&sm.K[16 * tn + lr][0], 32 * kb, g);
#pragma unroll
      for (int j = 0; j < NT2; ++j) {
        const int tm = wave / NB + (W / NB) * j;
        if (tm >= tn) qk[j] = mma(frag_row(&sm.Q[16 * tm + lr][0], 32 * kb, g), kf, qk[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < NT2; ++j) {
      const int tm = wave / NB + (W / NB) * j;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * tm + 4 * g + r, s2 = 16 * tn + lr;
        const float dpd = (tm >= tn && s2 <= t) ? acc[j][r] * expf(cs.gam[t] - cs.gam[s2]) : 0.f;
        sm.dPD[t][s2] = dpd;
        sm.M2[t][s2] = dpd * qk[j][r];
      }
    }
  }
  __syncthreads();
  if (tid < C) {
    float acc = 0.f;
    for (int s2 = 0; s2 < C; ++s2) acc += sm.M2[tid][s2];
    sm.rzP[tid] = acc;
  } else if (tid < 2 * C) {
    const int s2 = tid - C;
    float acc = 0.f;
    for (int t = 0; t < C; ++t) acc += sm.M2[t][s2];
    sm.czP[s2] = acc;
  }
  // the dT phase's rows of Dd and dWn (row block wave % NB)
  f32x4 ad_raw[DV / 16], aw_raw[DK / 16];
#pragma unroll
  for (int jb = 0; jb < DV / 16; ++jb) ad_raw[jb] = row4_f(Ddg, DV, 16 * (wave % NB) + lr, 16 * jb, g);
#pragma unroll
  for (int ib = 0; ib < DK / 16; ++ib) aw_raw[ib] = row4_f(DWg, DK, 16 * (wave % NB) + lr, 16 * ib, g);
  // dQ = diag(Gamma) QB + dPD K;  <QB, Q> per row
#pragma unroll
  for (int p = 0; p < NI; ++p) {
    const int it = wave + W * p, i = 16 * it + lr;
    f32x4 acc[NB];
#pragma unroll
    for (int tm = 0; tm < NB; ++tm) acc[tm] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sb = 0; sb < NB; ++sb) {
      const s16x4 b = col4_bits(&sm.K[0][0], Lds::kLK, 16 * sb, i, g);
#pragma unroll
      for (int tm = sb; tm < NB; ++tm)
        acc[tm] = mma16s(split4(row4_f(&sm.dPD[0][0], Lds::kLX, 16 * tm + lr, 16 * sb, g)), b, acc[tm]);
    }
#pragma unroll
    for (int tm = 0; tm < NB; ++tm)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * tm + 4 * g + r;
        const float part = sum16(qb[p][tm][r] * bfv(sm.Q[t][i]));
        if (lr == 0) sm.pGO[t][it] = part;
        if (t < n) {
          const float val = __builtin_fmaf(cs.Gam[t], qb[p][tm][r], acc[tm][r]);
          if (dq_part)
            dq_part[(row0 + (size_t)t * H) * DK + i] = val;
          else
            Bf16::store(dq, (kq0 + (size_t)t * Hk) * DK + i, val);
        }
      }
  }
  // dV = diag(beta) X^T Dd
#pragma unroll
  for (int p = 0; p < NJ; ++p) {
    const int jt = wave + W * p;
    Split4 bd[NB];
    f32x4 acc[NB];
#pragma unroll
    for (int tb = 0; tb < NB; ++tb) {
      bd[tb] = split4(bd_raw[p][tb]);
      acc[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int tb = 0; tb < NB; ++tb)
#pragma unroll
      for (int sb = 0; sb <= tb; ++sb)
        acc[sb] = mma16s(split4(col4_f(&sm.X[0][0], Lds::kLX, 16 * tb, 16 * sb + lr, g)), bd[tb], acc[sb]);
#pragma unroll
    for (int sb = 0; sb < NB; ++sb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int s2 = 16 * sb + 4 * g + r;
        if (s2 < n) Bf16::store(dv, (row0 + (size_t)s2 * H) * DV + 16 * jt + lr, cs.beta[s2] * acc[sb][r]);
      }
  }
  // TW = T^T dW = -diag(beta) X^T dWn (kept for dK)
  f32x4 TW[NI][NB];
#pragma unroll
  for (int p = 0; p < NI; ++p) {
    const int it = wave + W * p;
    Split4 bw[NB];
#pragma unroll
    for (int tb = 0; tb < NB; ++tb) {
      bw[tb] = split4(bw_raw[p][tb]);
      TW[p][tb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int tb = 0; tb < NB; ++tb)
#pragma unroll
      for (int sb = 0; sb <= tb; ++sb)
        TW[p][sb] = mma16s(split4(col4_f(&sm.X[0][0], Lds::kLX, 16 * tb, 16 * sb + lr, g)), bw[tb], TW[p][sb]);
#pragma unroll
    for (int sb = 0; sb < NB; ++sb)
#pragma unroll
      for (int r = 0; r < 4; ++r) TW[p][sb][r] = -cs.beta[16 * sb + 4 * g + r] * TW[p][sb][r];
  }
  __syncthreads();  // Z_P sums done: M2 is free
  // the dK phase's dKt values
  float kt[NI][NB][4];
#pragma unroll
  for (int p = 0; p < NI; ++p)
#pragma unroll
    for (int sb = 0; sb < NB; ++sb)
#pragma unroll
      for (int r = 0; r < 4; ++r) kt[p][sb][r] = KTg[(size_t)(16 * sb + 4 * g + r) * DK + 16 * (wave + W * p) + lr];
  // dT = Dd V^T - (dWn K^T) diag(Gamma); wave w makes row block w % NB,
  // column blocks (w / NB) NT2 .. + NT2 - 1
  {
    constexpr int NT2 = NB * NB / W;
    const int tm = wave % NB, tn0 = (wave / NB) * NT2;
    f32x4 acc[NT2], acw[NT2];
#pragma unroll
    for (int u = 0; u < NT2; ++u) acc[u] = acw[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jb = 0; jb < DV / 16; ++jb) {
      const Split4 ad = split4(ad_raw[jb]);
#pragma unroll
      for (int u = 0; u < NT2; ++u)
        acc[u] = mma16s(ad, row4_bits(&sm.V[0][0], Lds::kLV, 16 * (tn0 + u) + lr, 16 * jb, g), acc[u]);
    }
#pragma unroll
    for (int ib = 0; ib < DK / 16; ++ib) {
      const Split4 aw = split4(aw_raw[ib]);
#pragma unroll
      for (int u = 0; u < NT2; ++u)
        acw[u] = mma16s(aw, row4_bits(&sm.K[0][0], Lds::kLK, 16 * (tn0 + u) + lr, 16 * ib, g), acw[u]);
    }
#pragma unroll
    for (int u = 0; u < NT2; ++u) {
      const float gs = cs.Gam[16 * (tn0 + u) + lr];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        sm.M2[16 * tm + 4 * g + r][16 * (tn0 + u) + lr] = __builtin_fmaf(-gs, acw[u][r], acc[u][r]);
    }
  }
  __syncthreads();
  if (tid < C) {  // dbeta, column part: sum_t X[t][s] dT[t][s]
    float acc = 0.f;
    for (int t = 0; t < C; ++t) acc = __builtin_fmaf(sm.X[t][tid], sm.M2[t][tid], acc);
    sm.dbc[tid] = acc;
  }
  __syncthreads();
  for (int idx = tid; idx < C * C; idx += 64 * W) sm.M2[idx / C][idx % C] *= cs.beta[idx % C];  // dX
  __syncthreads();
  // Y = dX X^T -> M3; wave w makes row block w % NB, column blocks
  // tn_y(w, u): all of them (W = NB), or {h, NB - 1 - h} with h = w / NB
  // (W = 2 NB), which gives every wave the same number of products
  {
    constexpr int NT2 = NB * NB / W;
    const int tm = wave % NB, h = wave / NB;
    auto tn_y = [&](int u) { return NT2 == NB ? u : (u == 0 ? h : NB - 1 - h); };
    f32x4 acc[NT2];
#pragma unroll
    for (int u = 0; u < NT2; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int rb = 0; rb < NB; ++rb) {
      const Split4 a = split4(row4_f(&sm.M2[0][0], Lds::kLX, 16 * tm + lr, 16 * rb, g));
#pragma unroll
      for (int u = 0; u < NT2; ++u) {
        const int tn = tn_y(u);
        if (tn >= rb) acc[u] = mma16s(a, split4(row4_f(&sm.X[0][0], Lds::kLX, 16 * tn + lr, 16 * rb, g)), acc[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < NT2; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.M3[16 * tm + 4 * g + r][16 * tn_y(u) + lr] = acc[u][r];
  }
  __syncthreads();
  // dA = -X^T Y (strict lower); dA .* D -> M2, Z_A = dA .* D .* G -> M3 after a
  // barrier; wave w makes the tiles (w / NB + (W / NB) j, w % NB)
  constexpr int NTA = NB * NB / W;
  f32x4 ZA[NTA];
  {
    const int tn = wave % NB;
    f32x4 acc[NTA], gk[NTA];
#pragma unroll
    for (int j = 0; j < NTA; ++j) acc[j] = gk[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int rb = 0; rb < NB; ++rb) {
      const Split4 b = split4(col4_f(&sm.M3[0][0], Lds::kLX, 16 * rb, 16 * tn + lr, g));
#pragma unroll
      for (int j = 0; j < NTA; ++j) {
        const int tm = wave / NB + (W / NB) * j;
        if (tm <= rb && tm >= tn)
          acc[j] = mma16s(split4(col4_f(&sm.X[0][0], Lds::kLX, 16 * rb, 16 * tm + lr, g)), b, acc[j]);
      }
    }
#pragma unroll
    for (int kb = 0; kb < DK / 32; ++kb) {
      const u32x4 kf = frag_row(&sm.K[16 * tn + lr][0], 32 * kb, g);
#pragma unroll
      for (int j = 0; j < NTA; ++j) {
        const int tm = wave / NB + (W / NB) * j;
        if (tm >= tn) gk[j] = mma(frag_row(&sm.K[16 * tm + lr][0], 32 * kb, g), kf, gk[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < NTA; ++j) {
      const int tm = wave / NB + (W / NB) * j;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * tm + 4 * g + r, s2 = 16 * tn + lr;
        float dad = 0.f, z = 0.f;
        if (tm >= tn && s2 < t) {
          dad = -acc[j][r] * expf(cs.gam[t] - cs.gam[s2]);
          z = dad * gk[j][r];
        }
        sm.M2[t][s2] = dad;
        ZA[j][r] = z;
      }
    }
  }
  __syncthreads();  // Y no longer read
#pragma unroll
  for (int j = 0; j < NTA; ++j) {
    const int tm = wave / NB + (W / NB) * j;
#pragma unroll
    for (int r = 0; r < 4; ++r) sm.M3[16 * tm + 4 * g + r][16 * (wave % NB) + lr] = ZA[j][r];
  }
  __syncthreads();
  if (tid < C) {
    float acc = 0.f;
    for (int s2 = 0; s2 < C; ++s2) acc += sm.M3[tid][s2];
    sm.dbr[tid] = acc;
    sm.rzA[tid] = cs.beta[tid] * acc;
  } else if (tid < 2 * C) {
    const int s2 = tid - C;
    float acc = 0.f;
    for (int t = 0; t < C; ++t) acc = __builtin_fmaf(cs.beta[t], sm.M3[t][s2], acc);
    sm.czA[s2] = acc;
  }
  // dK = dPD^T Q + (dG + dG^T) K + diag(e) dKt + diag(Gamma) TW, dG = beta_t (dA .* D)
#pragma unroll
  for (int p = 0; p < NI; ++p) {
    const int it = wave + W * p, i = 16 * it + lr;
    f32x4 acc[NB];
#pragma unroll
    for (int sb = 0; sb < NB; ++sb) acc[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int tb = 0; tb < NB; ++tb) {
      const s16x4 bq = col4_bits(&sm.Q[0][0], Lds::kLK, 16 * tb, i, g);
      const s16x4 bk = col4_bits(&sm.K[0][0], Lds::kLK, 16 * tb, i, g);
#pragma unroll
      for (int sb = 0; sb < NB; ++sb) {
        if (sb <= tb)
          acc[sb] = mma16s(split4(col4_f(&sm.dPD[0][0], Lds::kLX, 16 * tb, 16 * sb + lr, g)), bq, acc[sb]);
        const f32x4 lo = row4_f(&sm.M2[0][0], Lds::kLX, 16 * sb + lr, 16 * tb, g);   // dA D [s][t]
        const f32x4 hi = col4_f(&sm.M2[0][0], Lds::kLX, 16 * tb, 16 * sb + lr, g);  // dA D [t][s]
        const float bs = cs.beta[16 * sb + lr];
        f32x4 a;
#pragma unroll
        for (int m = 0; m < 4; ++m) a[m] = __builtin_fmaf(bs, lo[m], cs.beta[16 * tb + 4 * g + m] * hi[m]);
        acc[sb] = mma16s(split4(a), bk, acc[sb]);
      }
    }
#pragma unroll
    for (int sb = 0; sb < NB; ++sb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int s2 = 16 * sb + 4 * g + r;
        const float ks = bfv(sm.K[s2][i]);
        const float tw = TW[p][sb][r];
        const float pw = sum16(tw * ks), pe = sum16(kt[p][sb][r] * ks);
        if (lr == 0) {
          sm.pGW[s2][it] = pw;
          sm.pDE[s2][it] = pe;
        }
        const float val = acc[sb][r] + cs.e[s2] * kt[p][sb][r] + cs.Gam[s2] * tw;
        if (s2 < n) {
          if (dk_part)
            dk_part[(row0 + (size_t)s2 * H) * DK + i] = val;
          else
            Bf16::store(dk, (kq0 + (size_t)s2 * Hk) * DK + i, val);
        }
      }
  }
  __syncthreads();
  if (tid < C) {
    float a = 0.f, b = 0.f, c = 0.f;
    for (int it = 0; it < DK / 16; ++it) {
      a += sm.pGO[tid][it];
      b += sm.pGW[tid][it];
      c += sm.pDE[tid][it];
    }
    sm.dgo[tid] = a + b;
    sm.de[tid] = c;
  }
  __syncthreads();
  // each token's dgamma term and dbeta in parallel; one thread then forms the
  // reverse cumulative sum (t = C - 1 down to 0) and the de e sum in order
  if (tid < C) {
    const int t = tid;
    sm.dgam[t] = (sm.rzP[t] + sm.rzA[t]) - (sm.czP[t] + sm.czA[t]) + sm.dgo[t] * cs.Gam[t] - sm.de[t] * cs.e[t];
    if (t < n) dbeta[row0 + (size_t)t * H] = sm.dbc[t] + sm.dbr[t];
  } else if (tid == C) {
    float sum_de = 0.f;
    for (int t = 0; t < C; ++t) sum_de = __builtin_fmaf(sm.de[t], cs.e[t], sum_de);
    sm.sum_de = sum_de;
  }
  __syncthreads();
  if (tid == 0) {
    float acc = 0.f;
    for (int t = C - 1; t >= 0; --t) {
      float dgam = sm.dgam[t];
      if (t == C - 1) dgam += dGn * cs.Gam[C - 1] + sm.sum_de;
      acc += dgam;
      sm.dgam[t] = acc;
    }
  }
  __syncthreads();
  if (tid < n) dg[row0 + (size_t)tid * H] = sm.dgam[tid];
}

}  // namespace bwdb
}  // namespace cpr
