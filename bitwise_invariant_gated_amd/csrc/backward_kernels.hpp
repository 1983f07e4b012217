// Backward kernels (fwd_bwd): local terms, reverse chain, state and gradient
// stages, fp32 and bf16 paths.
//
// Part of libgdn_cpr (included by gdn_cpr.hip, in this order: prefill_kernels.hpp,
// decode_kernels.hpp, comparator_kernels.hpp, backward_kernels.hpp).
#pragma once

#include "comparator_kernels.hpp"
#include "cpr_backward.hpp"
#include "cpr_backward_bf16.hpp"

namespace {

// ---------------------------------------------------------------------------
// backward (fwd_bwd): per-chunk local terms, reverse boundary chain, gradients

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* g;
  const void* beta;
  const void* d_o;
  const int32_t* cu;
  const int32_t* all_base;
  const float* bnd;   // forward state at the start of every chunk slot
  const float* d_hT;  // [N,H,DK,DV] or null
  uint8_t* ws;        // [A_max*H] backward slots
  float* gamn;        // [A_max*H]
  void* dq;
  void* dk;
  void* dv;
  float* dg;
  float* dbeta;
  float* dh0;
  float* dq_part;  // [T, H, DK] fp32 per value head when key heads are shared, else null
  float* dk_part;
  int32_t N;
  int32_t H;
  int32_t Hk;  // heads of q and k
  int32_t G;   // value heads per key head, H / Hk
  int32_t Cl;  // chunk length
};

// Barrier after writes to the slot's scratch (the C x d arrays of the local
// and gradient kernels when d > 128): each wave waits for its stores to
// complete first, so every wave of the work-group reads them after it.
template <bool kWide>
__device__ __forceinline__ void sync_scratch() {
  if constexpr (kWide) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

template <int DK, int DV, bool kStage = false>
struct BwdLocalLds {
  static constexpr bool kWide = DK > 128 || DV > 128;  // W and Dd in the slot's scratch
  float At[C][C + 1];  // At[s][t] = A[t][s]
  float X[C][C + 1];
  float Pt[C][C + 1];  // Pt[s][t] = P[t][s]
  float W[C][kWide ? 1 : DK + 1];
  float Dd[C][kWide ? 1 : DV + 1];
  bwd::ChunkScalars cs;
  // kStage (bf16 inputs, d > 128): the chunk's K, Q and dO rows, which every
  // product reads, as bf16 bits (rows past the chunk's tokens are zero)
  alignas(16) uint16_t Ks[kStage ? C : 1][kStage ? DK + 8 : 1];
  alignas(16) uint16_t Qs[kStage ? C : 1][kStage ? DK + 8 : 1];
  alignas(16) uint16_t dOs[kStage ? C : 1][kStage ? DV + 8 : 1];
};

// B1: per chunk slot (full or partial) and head: X, W, Kt, -W^T, dDelta_local
// = P^T dO and R = (diag(Gamma) Q)^T dO - W^T dDelta_local.
template <class D, int DK, int DV>
__global__ __launch_bounds__(256) void k_bwd_local(const BwdArgs a) {
  using namespace bwd;
  using T = typename D::T;
  typedef BwdSlot<DK, DV, sizeof(T)> Slot;
  constexpr bool kWide = Slot::kWide;
  // d > 128 on bf16 inputs: the LDS has room for the chunk's K, Q and dO
  // (about 150 KB with the C x C arrays, one work-group per CU), which the
  // products would otherwise fetch element by element from global memory
  constexpr bool kStage = kWide && std::is_same<D, Bf16>::value;
  __shared__ BwdLocalLds<DK, DV, kStage> sm;
  const int slot = blockIdx.x, h = blockIdx.y, H = a.H;
  if (slot >= a.all_base[a.N]) return;
  const int i = find_seq(a.all_base, a.N, slot);
  const int c = slot - a.all_base[i];
  const int L = a.cu[i + 1] - a.cu[i];
  const int n = min(a.Cl, L - c * a.Cl);
  const size_t row0 = ((size_t)a.cu[i] + (size_t)c * a.Cl) * H + h;
  const int tid = threadIdx.x, wave = tid >> 6;
  const T* kp = (const T*)a.k;
  const T* qp = (const T*)a.q;
  const T* dop = (const T*)a.d_o;
  const size_t kq0 = kq_row((size_t)a.cu[i] + (size_t)c * a.Cl, h, a.Hk, a.G);
  if constexpr (kStage) {
    // 16-byte pieces (8 elements); chunk_scalars' barriers publish them
    typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
    const u32x4v zero = {0u, 0u, 0u, 0u};
    for (int idx = tid; idx < C * (DK / 8); idx += 256) {
      const int t = idx / (DK / 8), m = idx % (DK / 8);
      u32x4v kv = zero, qv = zero;
      if (t < n) {  // rows past the chunk's tokens are not read
        const size_t off = (kq0 + (size_t)t * a.Hk) * DK + 8 * m;
        kv = *reinterpret_cast<const u32x4v*>(kp + off);
        qv = *reinterpret_cast<const u32x4v*>(qp + off);
      }
      *reinterpret_cast<u32x4v*>(&sm.Ks[t][8 * m]) = kv;
      *reinterpret_cast<u32x4v*>(&sm.Qs[t][8 * m]) = qv;
    }
    for (int idx = tid; idx < C * (DV / 8); idx += 256) {
      const int t = idx / (DV / 8), m = idx % (DV / 8);
      u32x4v dv = zero;
      if (t < n) dv = *reinterpret_cast<const u32x4v*>(dop + (row0 + (size_t)t * H) * DV + 8 * m);
      *reinterpret_cast<u32x4v*>(&sm.dOs[t][8 * m]) = dv;
    }
  }
  chunk_scalars<D>(sm.cs, (const T*)a.g, (const T*)a.beta, row0, H, n);
  const ChunkScalars& cs = sm.cs;
  auto Kx = [&](int t, int e) {
    if constexpr (kStage) return __uint_as_float((uint32_t)sm.Ks[t][e] << 16);
    else return t < n ? D::load(kp, (kq0 + (size_t)t * a.Hk) * DK + e) : 0.f;
  };
  auto Qx = [&](int t, int e) {
    if constexpr (kStage) return __uint_as_float((uint32_t)sm.Qs[t][e] << 16);
    else return t < n ? D::load(qp, (kq0 + (size_t)t * a.Hk) * DK + e) : 0.f;
  };
  auto dOx = [&](int t, int j) {
    if constexpr (kStage) return __uint_as_float((uint32_t)sm.dOs[t][j] << 16);
    else return t < n ? D::load(dop, (row0 + (size_t)t * H) * DV + j) : 0.f;
  };
  uint8_t* ws = a.ws + ((size_t)slot * H + h) * Slot::bytes;
  // W [C][DK] and Dd [C][DV]: in the LDS, or in the slot's scratch when d > 128
  float* const scr = reinterpret_cast<float*>(ws + Slot::oScr);
  float* const Wm = kWide ? scr : &sm.W[0][0];
  float* const Dm = kWide ? scr + Slot::kArr / 4 : &sm.Dd[0][0];
  constexpr int LW = kWide ? DK : DK + 1, LDd = kWide ? DV : DV + 1;

  // A = strict lower(beta_t D G) and P = lower(QK^T .* D): 16 + 16 tiles
  for (int q = 0; q < 8; ++q) {
    const int id = wave * 8 + q, tl = id & 15, tm = tl >> 2, tn = tl & 3;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (id < 16) {
      acc = tile<DK>([&](int m, int k) { return Kx(m, k); }, [&](int k, int nn) { return Kx(nn, k); }, 16 * tm,
                     16 * tn, acc);
      tile_each(acc, 16 * tm, 16 * tn, [&](int t, int s, float v) {
        sm.At[s][t] = (s < t) ? (cs.beta[t] * expf(cs.gam[t] - cs.gam[s])) * v : 0.f;
      });
    } else {
      acc = tile<DK>([&](int m, int k) { return Qx(m, k); }, [&](int k, int nn) { return Kx(nn, k); }, 16 * tm,
                     16 * tn, acc);
      tile_each(acc, 16 * tm, 16 * tn,
                [&](int t, int s, float v) { sm.Pt[s][t] = (s <= t) ? v * expf(cs.gam[t] - cs.gam[s]) : 0.f; });
    }
  }
  __syncthreads();
  if (wave == 0) unit_lower_inverse<C + 1, C + 1>(sm.At, sm.X);
  __syncthreads();
  float* Dd = reinterpret_cast<float*>(ws + Slot::oDd);
  constexpr int nW = 4 * (DK / 16), nD = 4 * (DV / 16);
  for (int id = wave; id < nW + nD; id += 4) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (id < nW) {
      const int tm = id / (DK / 16), it = id % (DK / 16);
      acc = tile<C>([&](int t, int r) { return sm.X[t][r] * (cs.beta[r] * cs.Gam[r]); },
                    [&](int r, int e) { return Kx(r, e); }, 16 * tm, 16 * it, acc);
      tile_each(acc, 16 * tm, 16 * it, [&](int t, int e, float v) { Wm[t * LW + e] = v; });
    } else {
      const int u = id - nW, tm = u / (DV / 16), jt = u % (DV / 16);
      acc = tile<C>([&](int t, int s) { return sm.Pt[t][s]; }, [&](int s, int j) { return dOx(s, j); }, 16 * tm,
                    16 * jt, acc);
      tile_each(acc, 16 * tm, 16 * jt, [&](int t, int j, float v) { Dm[t * LDd + j] = v; });
      *reinterpret_cast<f32x4*>(Dd + ((size_t)(jt * (C / 16) + tm) * 64 + (tid & 63)) * 4) = acc;
    }
  }
  sync_scratch<kWide>();
  T* Kt = reinterpret_cast<T*>(ws + Slot::oKt);
  T* WnT = reinterpret_cast<T*>(ws + Slot::oWnT);
  float* Xs = reinterpret_cast<float*>(ws + Slot::oX);
  for (int idx = tid; idx < C * DK; idx += 256) {
    const int t = idx / DK, e = idx % DK;
    D::store(Kt, idx, cs.e[t] * Kx(t, e));
    D::store(WnT, (size_t)e * C + t, -Wm[t * LW + e]);
  }
  for (int idx = tid; idx < C * C; idx += 256) Xs[idx] = sm.X[idx / C][idx % C];
  float* R = reinterpret_cast<float*>(ws + Slot::oR);
  constexpr int nR = (DK / 16) * (DV / 16);
  for (int id = wave; id < nR; id += 4) {
    const int im = id / (DV / 16), jt = id % (DV / 16);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = tile<C>([&](int e, int t) { return cs.Gam[t] * Qx(t, e); }, [&](int t, int j) { return dOx(t, j); },
                  16 * im, 16 * jt, acc);
    acc = tile<C>([&](int e, int t) { return -Wm[t * LW + e]; }, [&](int t, int j) { return Dm[t * LDd + j]; },
                  16 * im, 16 * jt, acc);
    *reinterpret_cast<f32x4*>(R + ((size_t)(jt * (DK / 16) + im) * 64 + (tid & 63)) * 4) = acc;
  }
  if (tid == 0) a.gamn[(size_t)slot * H + h] = cs.Gam[C - 1];
}

// B2 for fp32 inputs: the same reverse chain with fp32 operands on
// v_mfma_f32_16x16x4_f32.  The k index of step m in a 16-row tile is
// 16 tile + 4 g + m, so accumulator tiles (lane group g holds rows 4 g .. 4 g
// + 3) are B operands as they stand.
template <int DK, int DV>
__global__ __launch_bounds__(DV * 4) void k_bwd_chain_f32(const BwdArgs a) {
  using namespace bwd;
  typedef BwdSlot<DK, DV, 4> Slot;
  const int i = blockIdx.x, h = blockIdx.y, H = a.H;
  const int tid = threadIdx.x, jb = tid >> 6, lane = tid & 63, lr = lane & 15, g = lane >> 4;
  const int L = a.cu[i + 1] - a.cu[i];
  const int nall = (L + a.Cl - 1) / a.Cl;
  const size_t sh = (size_t)i * H + h;
  const size_t SS = (size_t)DK * DV;
  const int abase = a.all_base[i];
  f32x4 S1[DK / 16][1];
  load_state_tiles<DK, DV, 1>(S1, a.d_hT ? a.d_hT + sh * SS : nullptr, jb, lane);
  f32x4(&S)[DK / 16] = *reinterpret_cast<f32x4(*)[DK / 16]>(&S1);
  for (int c = nall - 1; c >= 0; --c) {
    const size_t sl = (size_t)(abase + c) * H + h;
    uint8_t* ws = a.ws + sl * Slot::bytes;
    store_state_tiles<DK, DV, 1>(reinterpret_cast<float*>(ws + Slot::oDbp), S1, jb, lane);
    const float* Kt = reinterpret_cast<const float*>(ws + Slot::oKt);
    const float* WnT = reinterpret_cast<const float*>(ws + Slot::oWnT);
    const float* R = reinterpret_cast<const float*>(ws + Slot::oR);
    float* Dd = reinterpret_cast<float*>(ws + Slot::oDd);
    f32x4 E[C / 16];
#pragma unroll
    for (int tm = 0; tm < C / 16; ++tm) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int it = 0; it < DK / 16; ++it)
#pragma unroll
        for (int m = 0; m < 4; ++m) acc = mma4(Kt[(16 * tm + lr) * DK + 16 * it + 4 * g + m], S[it][m], acc);
      E[tm] = acc;
      f32x4* dd = reinterpret_cast<f32x4*>(Dd + ((size_t)(jb * (C / 16) + tm) * 64 + lane) * 4);
      *dd = *dd + acc;
    }
    const float gn = a.gamn[sl];
#pragma unroll
    for (int im = 0; im < DK / 16; ++im) {
      const f32x4 r = *reinterpret_cast<const f32x4*>(R + ((size_t)(jb * (DK / 16) + im) * 64 + lane) * 4);
      f32x4 acc = {gn * S[im][0] + r[0], gn * S[im][1] + r[1], gn * S[im][2] + r[2], gn * S[im][3] + r[3]};
#pragma unroll
      for (int tm = 0; tm < C / 16; ++tm)
#pragma unroll
        for (int m = 0; m < 4; ++m) acc = mma4(WnT[(16 * im + lr) * C + 16 * tm + 4 * g + m], E[tm][m], acc);
      S[im] = acc;
    }
  }
  if (a.dh0) store_state_tiles<DK, DV, 1>(a.dh0 + sh * SS, S1, jb, lane);
}

// B2 for bf16 inputs at d_k = d_v = 256 (the slot of the kernels above, Kt
// and -W^T in bf16): the same step with each product on
// v_mfma_f32_16x16x16_bf16, Kt or -W^T exact as the A operand and the fp32
// adjoint (or E) split into bf16 hi + lo parts as the B operand (two products
// per 16-wide k block; the accumulator tiles are B operands as they stand).
// Work-groups of 4 waves own 64 state columns, a wave 16 of them.  Each
// chunk's Kt and -W^T (64 KiB) pass through the LDS: they are fetched into
// registers with 16-byte loads one chunk ahead and written to the LDS at the
// start of the chunk's step.
template <int DK, int DV>
__global__ __launch_bounds__(256) void k_bwd_chain_wide(const BwdArgs a) {
  using namespace bwd;
  using mfma::u32x4;
  typedef BwdSlot<DK, DV, 2> Slot;
  constexpr int kLK = DK + 8, kLC = C + 8;  // LDS rows (bf16), padded against bank conflicts
  constexpr int kPieces = (int)((Slot::kKt + Slot::kWnT) / 16), kPer = kPieces / 256;
  static_assert(kPer * 256 == kPieces && Slot::oWnT == Slot::kKt, "Kt and -W^T are adjacent, split over the threads");
  __shared__ __attribute__((aligned(16))) uint16_t sKt[C][kLK];
  __shared__ __attribute__((aligned(16))) uint16_t sWn[DK][kLC];
  const int i = blockIdx.x, h = blockIdx.y, H = a.H;
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, g = lane >> 4;
  const int jb = blockIdx.z * 4 + (tid >> 6);
  const int L = a.cu[i + 1] - a.cu[i];
  const int nall = (L + a.Cl - 1) / a.Cl;
  const size_t sh = (size_t)i * H + h;
  const size_t SS = (size_t)DK * DV;
  const int abase = a.all_base[i];
  auto slot_of = [&](int c) { return a.ws + ((size_t)(abase + c) * H + h) * Slot::bytes; };
  // piece p (16 bytes) of the slot's Kt (then -W^T) bytes
  u32x4 pre[kPer];
  auto fetch = [&](int c) {
    const u32x4* src = reinterpret_cast<const u32x4*>(slot_of(c) + Slot::oKt);
#pragma unroll
    for (int m = 0; m < kPer; ++m) pre[m] = src[tid + 256 * m];
  };
  auto stage = [&] {
#pragma unroll
    for (int m = 0; m < kPer; ++m) {
      const int p = tid + 256 * m;
      if (p < (int)(Slot::kKt / 16)) {
        const int r = p / (DK / 8), c8 = (p % (DK / 8)) * 8;
        *reinterpret_cast<u32x4*>(&sKt[r][c8]) = pre[m];
      } else {
        const int q = p - (int)(Slot::kKt / 16), r = q / (C / 8), c8 = (q % (C / 8)) * 8;
        *reinterpret_cast<u32x4*>(&sWn[r][c8]) = pre[m];
      }
    }
  };
  f32x4 S1[DK / 16][1];
  load_state_tiles<DK, DV, 1>(S1, a.d_hT ? a.d_hT + sh * SS : nullptr, jb, lane);
  if (nall > 0) fetch(nall - 1);
  for (int c = nall - 1; c >= 0; --c) {
    uint8_t* ws = slot_of(c);
    __syncthreads();  // the previous chunk's LDS operands are no longer read
    stage();
    __syncthreads();
    if (c > 0) fetch(c - 1);
    store_state_tiles<DK, DV, 1>(reinterpret_cast<float*>(ws + Slot::oDbp), S1, jb, lane);
    const float* R = reinterpret_cast<const float*>(ws + Slot::oR);
    float* Dd = reinterpret_cast<float*>(ws + Slot::oDd);
    bwdb::Split4 Sp[DK / 16];
#pragma unroll
    for (int it = 0; it < DK / 16; ++it) Sp[it] = bwdb::split4(S1[it][0]);
    bwdb::Split4 Ep[C / 16];
#pragma unroll
    for (int tm = 0; tm < C / 16; ++tm) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int it = 0; it < DK / 16; ++it)
        acc = bwdb::mma16s(bwdb::row4_bits(&sKt[0][0], kLK, 16 * tm + lr, 16 * it, g), Sp[it], acc);
      Ep[tm] = bwdb::split4(acc);
      f32x4* dd = reinterpret_cast<f32x4*>(Dd + ((size_t)(jb * (C / 16) + tm) * 64 + lane) * 4);
      *dd = *dd + acc;
    }
    const float gn = a.gamn[(size_t)(abase + c) * H + h];
#pragma unroll
    for (int im = 0; im < DK / 16; ++im) {
      const f32x4 r = *reinterpret_cast<const f32x4*>(R + ((size_t)(jb * (DK / 16) + im) * 64 + lane) * 4);
      f32x4 acc = {__builtin_fmaf(gn, S1[im][0][0], r[0]), __builtin_fmaf(gn, S1[im][0][1], r[1]),
                   __builtin_fmaf(gn, S1[im][0][2], r[2]), __builtin_fmaf(gn, S1[im][0][3], r[3])};
#pragma unroll
      for (int tm = 0; tm < C / 16; ++tm)
        acc = bwdb::mma16s(bwdb::row4_bits(&sWn[0][0], kLC, 16 * im + lr, 16 * tm, g), Ep[tm], acc);
      S1[im][0] = acc;
    }
  }
  if (a.dh0) store_state_tiles<DK, DV, 1>(a.dh0 + sh * SS, S1, jb, lane);
}

template <int DK, int DV, bool kStage = false>
struct BwdGradLds {
  static constexpr int DM = DK > DV ? DK : DV;
  static constexpr bool kWide = DK > 128 || DV > 128;  // N1, M1 and M2 in the slot's scratch
  float N1[C][kWide ? 1 : C + 1];  // G
  float N2[C][C + 1];   // dT -> dX -> dA -> dG
  float N3[C][C + 1];   // X
  float N4[C][C + 1];   // dPD = (dO Delta^T) .* D, lower incl.
  float N5[C][C + 1];   // Z_P, then Y, then dA D G
  float M1[C][kWide ? 1 : DM + 1];  // W -> dO B^T -> dW -> T^T dW
  float M2[C][kWide ? 1 : DM + 1];  // U -> Delta -> dKt
  bwd::ChunkScalars cs;
  float rzP[C], czP[C], dGamO[C], dGamW[C], de[C], dbc[C], dbr[C], rzA[C], czA[C];
  float red[256];
  // kStage (bf16 inputs, d > 128): the chunk's K and Q rows as bf16 bits
  // (rows past the chunk's tokens are zero)
  alignas(16) uint16_t Ks[kStage ? C : 1][kStage ? DK + 8 : 1];
  alignas(16) uint16_t Qs[kStage ? C : 1][kStage ? DK + 8 : 1];
};

// B3: per chunk slot and head: dq, dk, dv, dg, dbeta of the chunk's tokens.
template <class D, int DK, int DV>
__global__ __launch_bounds__(256) void k_bwd_grads(const BwdArgs a) {
  using namespace bwd;
  using T = typename D::T;
  typedef BwdSlot<DK, DV, sizeof(T)> Slot;
  // d > 128 on bf16 inputs: the chunk's K and Q, the most-read operands, in
  // the LDS (about 140 KB with the C x C arrays, one work-group per CU)
  // instead of element by element from global memory
  constexpr bool kStage = Slot::kWide && std::is_same<D, Bf16>::value;
  __shared__ BwdGradLds<DK, DV, kStage> sm;
  const int slot = blockIdx.x, h = blockIdx.y, H = a.H;
  if (slot >= a.all_base[a.N]) return;
  const int i = find_seq(a.all_base, a.N, slot);
  const int c = slot - a.all_base[i];
  const int L = a.cu[i + 1] - a.cu[i];
  const int n = min(a.Cl, L - c * a.Cl);
  const size_t row0 = ((size_t)a.cu[i] + (size_t)c * a.Cl) * H + h;
  const int tid = threadIdx.x, wave = tid >> 6;
  const T* kp = (const T*)a.k;
  const T* qp = (const T*)a.q;
  const T* vp = (const T*)a.v;
  const T* dop = (const T*)a.d_o;
  const size_t kq0 = kq_row((size_t)a.cu[i] + (size_t)c * a.Cl, h, a.Hk, a.G);
  if constexpr (kStage) {
    // 16-byte pieces (8 elements); chunk_scalars' barriers publish them
    typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
    for (int idx = tid; idx < C * (DK / 8); idx += 256) {
      const int t = idx / (DK / 8), m = idx % (DK / 8);
      u32x4v kv = {0u, 0u, 0u, 0u}, qv = {0u, 0u, 0u, 0u};
      if (t < n) {  // rows past the chunk's tokens are not read
        const size_t off = (kq0 + (size_t)t * a.Hk) * DK + 8 * m;
        kv = *reinterpret_cast<const u32x4v*>(kp + off);
        qv = *reinterpret_cast<const u32x4v*>(qp + off);
      }
      *reinterpret_cast<u32x4v*>(&sm.Ks[t][8 * m]) = kv;
      *reinterpret_cast<u32x4v*>(&sm.Qs[t][8 * m]) = qv;
    }
  }
  chunk_scalars<D>(sm.cs, (const T*)a.g, (const T*)a.beta, row0, H, n);
  const ChunkScalars& cs = sm.cs;
  auto Kx = [&](int t, int e) {
    if constexpr (kStage) return __uint_as_float((uint32_t)sm.Ks[t][e] << 16);
    else return t < n ? D::load(kp, (kq0 + (size_t)t * a.Hk) * DK + e) : 0.f;
  };
  auto Qx = [&](int t, int e) {
    if constexpr (kStage) return __uint_as_float((uint32_t)sm.Qs[t][e] << 16);
    else return t < n ? D::load(qp, (kq0 + (size_t)t * a.Hk) * DK + e) : 0.f;
  };
  auto Vx = [&](int t, int j) { return t < n ? D::load(vp, (row0 + (size_t)t * H) * DV + j) : 0.f; };
  auto dOx = [&](int t, int j) { return t < n ? D::load(dop, (row0 + (size_t)t * H) * DV + j) : 0.f; };
  const uint8_t* ws = a.ws + ((size_t)slot * H + h) * Slot::bytes;
  const float* Bst = a.bnd + ((size_t)slot * H + h) * DK * DV;
  const float* dBp = reinterpret_cast<const float*>(ws + Slot::oDbp);
  const float* Ddg = reinterpret_cast<const float*>(ws + Slot::oDd);
  const float* Xs = reinterpret_cast<const float*>(ws + Slot::oX);
  auto dDx = [&](int t, int j) { return Ddg[tile_index<C>(t, j)]; };
  constexpr int nK = 4 * (DK / 16), nV = 4 * (DV / 16);
  // the C x d arrays: W, dO B^T, dW, T^T dW share the LDS array M1 and U ->
  // Delta, dKt share M2; when d > 128 each has a region of the slot's scratch
  constexpr bool kWide = Slot::kWide;
  constexpr int LM = kWide ? Slot::DM : Slot::DM + 1;
  float* const scr = reinterpret_cast<float*>(const_cast<uint8_t*>(ws) + Slot::oScr);
  constexpr size_t kA = Slot::kArr / 4;
  float* const mW = kWide ? scr : &sm.M1[0][0];
  float* const mU = kWide ? scr + kA : &sm.M2[0][0];
  float* const mQB = kWide ? scr + 2 * kA : &sm.M1[0][0];
  float* const mdW = kWide ? scr + 3 * kA : &sm.M1[0][0];
  float* const mTW = kWide ? scr + 4 * kA : &sm.M1[0][0];
  float* const mKt = kWide ? scr + 5 * kA : &sm.M2[0][0];
  // G (C x C) as well, so that two work-groups fit a CU's LDS
  float* const nG = kWide ? scr + 6 * kA : &sm.N1[0][0];
  constexpr int LG = kWide ? C : C + 1;

  // G and X
  for (int q = 0; q < 4; ++q) {
    const int tl = wave * 4 + q, tm = tl >> 2, tn = tl & 3;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = tile<DK>([&](int m, int k) { return Kx(m, k); }, [&](int k, int nn) { return Kx(nn, k); }, 16 * tm, 16 * tn,
                   acc);
    tile_each(acc, 16 * tm, 16 * tn, [&](int t, int s, float v) { nG[t * LG + s] = v; });
  }
  for (int idx = tid; idx < C * C; idx += 256) sm.N3[idx / C][idx % C] = Xs[idx];
  sync_scratch<kWide>();
  // W = X diag(beta Gamma) K -> M1,  U = X diag(beta) V -> M2
  for (int id = wave; id < nK + nV; id += 4) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (id < nK) {
      const int tm = id / (DK / 16), it = id % (DK / 16);
      acc = tile<C>([&](int t, int r) { return sm.N3[t][r] * (cs.beta[r] * cs.Gam[r]); },
                    [&](int r, int e) { return Kx(r, e); }, 16 * tm, 16 * it, acc);
      tile_each(acc, 16 * tm, 16 * it, [&](int t, int e, float v) { mW[t * LM + e] = v; });
    } else {
      const int u = id - nK, tm = u / (DV / 16), jt = u % (DV / 16);
      acc = tile<C>([&](int t, int r) { return sm.N3[t][r] * cs.beta[r]; }, [&](int r, int j) { return Vx(r, j); },
                    16 * tm, 16 * jt, acc);
      tile_each(acc, 16 * tm, 16 * jt, [&](int t, int j, float v) { mU[t * LM + j] = v; });
    }
  }
  sync_scratch<kWide>();
  // Delta = U - W B (in place in M2; every tile is read and written by one wave)
  for (int id = wave; id < nV; id += 4) {
    const int tm = id / (DV / 16), jt = id % (DV / 16);
    f32x4 acc;
    {
      const int lane = tid & 63, lr = lane & 15, g = lane >> 4;
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = mU[(16 * tm + 4 * g + r) * LM + 16 * jt + lr];
    }
    acc = tile<DK>([&](int t, int e) { return -mW[t * LM + e]; }, [&](int e, int j) { return Bst[bnd_index<DK>(e, j)]; },
                   16 * tm, 16 * jt, acc);
    tile_each(acc, 16 * tm, 16 * jt, [&](int t, int j, float v) { mU[t * LM + j] = v; });
  }
  sync_scratch<kWide>();
  // dP .* D (N4), Z_P = dPD .* QK (N5); dV = T^T dDelta
  for (int q = 0; q < 4; ++q) {
    const int tl = wave * 4 + q, tm = tl >> 2, tn = tl & 3;
    f32x4 accP = {0.f, 0.f, 0.f, 0.f}, accQ = {0.f, 0.f, 0.f, 0.f};
    accP = tile<DV>([&](int t, int j) { return dOx(t, j); }, [&](int j, int s) { return mU[s * LM + j]; }, 16 * tm,
                    16 * tn, accP);
    accQ = tile<DK>([&](int t, int e) { return Qx(t, e); }, [&](int e, int s) { return Kx(s, e); }, 16 * tm, 16 * tn,
                    accQ);
    const int lane = tid & 63, lr = lane & 15, g = lane >> 4;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * tm + 4 * g + r, s = 16 * tn + lr;
      const float dpd = (s <= t) ? accP[r] * expf(cs.gam[t] - cs.gam[s]) : 0.f;
      sm.N4[t][s] = dpd;
      sm.N5[t][s] = dpd * accQ[r];
    }
  }
  T* dvp = (T*)a.dv;
  for (int id = wave; id < nV; id += 4) {
    const int tm = id / (DV / 16), jt = id % (DV / 16);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = tile<C>([&](int t, int s) { return sm.N3[s][t]; }, [&](int s, int j) { return dDx(s, j); }, 16 * tm,
                  16 * jt, acc);
    tile_each(acc, 16 * tm, 16 * jt, [&](int t, int j, float v) {
      if (t < n) D::store(dvp, (row0 + (size_t)t * H) * DV + j, cs.beta[t] * v);
    });
  }
  sync_scratch<kWide>();
  // row / column sums of Z_P; dO B^T -> M1
  if (tid < C) {
    float acc = 0.f;
    for (int s = 0; s < C; ++s) acc += sm.N5[tid][s];
    sm.rzP[tid] = acc;
  } else if (tid < 2 * C) {
    const int s = tid - C;
    float acc = 0.f;
    for (int t = 0; t < C; ++t) acc += sm.N5[t][s];
    sm.czP[s] = acc;
  }
  for (int id = wave; id < nK; id += 4) {
    const int tm = id / (DK / 16), it = id % (DK / 16);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = tile<DV>([&](int t, int j) { return dOx(t, j); }, [&](int j, int e) { return Bst[bnd_index<DK>(e, j)]; },
                   16 * tm, 16 * it, acc);
    tile_each(acc, 16 * tm, 16 * it, [&](int t, int e, float v) { mQB[t * LM + e] = v; });
  }
  sync_scratch<kWide>();
  // dQ = diag(Gamma) dO B^T + dPD K;  dGamma (output part) = <dO B^T, Q> per row
  T* dqp = (T*)a.dq;
  for (int id = wave; id < nK; id += 4) {
    const int tm = id / (DK / 16), it = id % (DK / 16);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = tile<C>([&](int t, int s) { return sm.N4[t][s]; }, [&](int s, int e) { return Kx(s, e); }, 16 * tm, 16 * it,
                  acc);
    tile_each(acc, 16 * tm, 16 * it, [&](int t, int e, float v) {
      if (t < n) {
        const float val = cs.Gam[t] * mQB[t * LM + e] + v;
        if (a.dq_part)
          a.dq_part[(row0 + (size_t)t * H) * DK + e] = val;
        else
          D::store(dqp, (kq0 + (size_t)t * a.Hk) * DK + e, val);
      }
    });
  }
  if (tid < C) {
    float acc = 0.f;
    for (int e = 0; e < DK; ++e) acc = __builtin_fmaf(mQB[tid * LM + e], Qx(tid, e), acc);
    sm.dGamO[tid] = acc;
  }
  sync_scratch<kWide>();
  // dW = -dDelta B^T -> M1
  for (int id = wave; id < nK; id += 4) {
    const int tm = id / (DK / 16), it = id % (DK / 16);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = tile<DV>([&](int t, int j) { return dDx(t, j); }, [&](int j, int e) { return Bst[bnd_index<DK>(e, j)]; },
                   16 * tm, 16 * it, acc);
    tile_each(acc, 16 * tm, 16 * it, [&](int t, int e, float v) { mdW[t * LM + e] = -v; });
  }
  sync_scratch<kWide>();
  // T^T dW and dKt = Delta dB'^T (kept in registers), dT -> N2
  f32x4 TW[(nK + 3) / 4], KW[(nK + 3) / 4];
  for (int q = 0, id = wave; id < nK; id += 4, ++q) {
    const int tm = id / (DK / 16), it = id % (DK / 16);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    TW[q] = tile<C>([&](int t, int s) { return cs.beta[t] * sm.N3[s][t]; },
                    [&](int s, int e) { return mdW[s * LM + e]; }, 16 * tm, 16 * it, acc);
    KW[q] = tile<DV>([&](int t, int j) { return mU[t * LM + j]; }, [&](int j, int e) { return dBp[(size_t)e * DV + j]; },
                     16 * tm, 16 * it, acc);
  }
  for (int q = 0; q < 4; ++q) {
    const int tl = wave * 4 + q, tm = tl >> 2, tn = tl & 3;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = tile<DV>([&](int t, int j) { return dDx(t, j); }, [&](int j, int s) { return Vx(s, j); }, 16 * tm, 16 * tn,
                   acc);
    acc = tile<DK>([&](int t, int e) { return mdW[t * LM + e]; }, [&](int e, int s) { return cs.Gam[s] * Kx(s, e); },
                   16 * tm, 16 * tn, acc);
    tile_each(acc, 16 * tm, 16 * tn, [&](int t, int s, float v) { sm.N2[t][s] = v; });
  }
  sync_scratch<kWide>();
  for (int q = 0, id = wave; id < nK; id += 4, ++q) {
    const int tm = id / (DK / 16), it = id % (DK / 16);
    tile_each(TW[q], 16 * tm, 16 * it, [&](int t, int e, float v) { mTW[t * LM + e] = v; });
    tile_each(KW[q], 16 * tm, 16 * it, [&](int t, int e, float v) { mKt[t * LM + e] = v; });
  }
  sync_scratch<kWide>();
  // dGamma (W part), de, dbeta (column part)
  if (tid < C) {
    float acc = 0.f;
    for (int e = 0; e < DK; ++e) acc = __builtin_fmaf(mTW[tid * LM + e], Kx(tid, e), acc);
    sm.dGamW[tid] = acc;
  } else if (tid < 2 * C) {
    const int t = tid - C;
    float acc = 0.f;
    for (int e = 0; e < DK; ++e) acc = __builtin_fmaf(mKt[t * LM + e], Kx(t, e), acc);
    sm.de[t] = acc;
  } else if (tid < 3 * C) {
    const int s = tid - 2 * C;
    float acc = 0.f;
    for (int t = 0; t < C; ++t) acc = __builtin_fmaf(sm.N3[t][s], sm.N2[t][s], acc);
    sm.dbc[s] = acc;
  }
  sync_scratch<kWide>();
  for (int idx = tid; idx < C * C; idx += 256) sm.N2[idx / C][idx % C] *= sm.cs.beta[idx % C];  // dX
  sync_scratch<kWide>();
  // Y = dX X^T -> N5
  for (int q = 0; q < 4; ++q) {
    const int tl = wave * 4 + q, tm = tl >> 2, tn = tl & 3;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = tile<C>([&](int t, int r) { return sm.N2[t][r]; }, [&](int r, int s) { return sm.N3[s][r]; }, 16 * tm,
                  16 * tn, acc);
    tile_each(acc, 16 * tm, 16 * tn, [&](int t, int s, float v) { sm.N5[t][s] = v; });
  }
  sync_scratch<kWide>();
  // dA = -X^T Y, strict lower -> N2
  {
    f32x4 accs[4];
    for (int q = 0; q < 4; ++q) {
      const int tl = wave * 4 + q, tm = tl >> 2, tn = tl & 3;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      accs[q] = tile<C>([&](int t, int r) { return sm.N3[r][t]; }, [&](int r, int s) { return sm.N5[r][s]; }, 16 * tm,
                        16 * tn, acc);
    }
    sync_scratch<kWide>();
    for (int q = 0; q < 4; ++q) {
      const int tl = wave * 4 + q, tm = tl >> 2, tn = tl & 3;
      tile_each(accs[q], 16 * tm, 16 * tn, [&](int t, int s, float v) { sm.N2[t][s] = (s < t) ? -v : 0.f; });
    }
  }
  sync_scratch<kWide>();
  // dA D G -> N5, dG = dA beta_t D -> N2
  for (int idx = tid; idx < C * C; idx += 256) {
    const int t = idx / C, s = idx % C;
    const float dA = sm.N2[t][s];
    float zb = 0.f, dG = 0.f;
    if (s < t) {
      const float Dv = expf(cs.gam[t] - cs.gam[s]);
      zb = dA * Dv * nG[t * LG + s];
      dG = dA * cs.beta[t] * Dv;
    }
    sm.N5[t][s] = zb;
    sm.N2[t][s] = dG;
  }
  sync_scratch<kWide>();
  if (tid < C) {
    float acc = 0.f;
    for (int s = 0; s < C; ++s) acc += sm.N5[tid][s];
    sm.dbr[tid] = acc;
    sm.rzA[tid] = cs.beta[tid] * acc;
  } else if (tid < 2 * C) {
    const int s = tid - C;
    float acc = 0.f;
    for (int t = 0; t < C; ++t) acc = __builtin_fmaf(cs.beta[t], sm.N5[t][s], acc);
    sm.czA[s] = acc;
  }
  {
    float acc = 0.f;
    for (int idx = tid; idx < DK * DV; idx += 256)
      acc = __builtin_fmaf(dBp[idx], Bst[bnd_index<DK>(idx / DV, idx % DV)], acc);
    sm.red[tid] = acc;
  }
  sync_scratch<kWide>();
  if (tid == 0) {
    float dGn = 0.f;
    for (int r = 0; r < 256; ++r) dGn += sm.red[r];
    float sum_de = 0.f;
    for (int t = 0; t < C; ++t) sum_de = __builtin_fmaf(sm.de[t], cs.e[t], sum_de);
    float acc = 0.f;
    for (int t = C - 1; t >= 0; --t) {
      float dgam = (sm.rzP[t] + sm.rzA[t]) - (sm.czP[t] + sm.czA[t]) + (sm.dGamO[t] + sm.dGamW[t]) * cs.Gam[t] -
                   sm.de[t] * cs.e[t];
      if (t == C - 1) dgam += dGn * cs.Gam[C - 1] + sum_de;
      acc += dgam;
      if (t < n) {
        a.dg[row0 + (size_t)t * H] = acc;
        a.dbeta[row0 + (size_t)t * H] = sm.dbc[t] + sm.dbr[t];
      }
    }
  }
  // dK = dPD^T Q + (dG + dG^T) K + diag(e) dKt + diag(Gamma) T^T dW
  T* dkp = (T*)a.dk;
  for (int id = wave; id < nK; id += 4) {
    const int tm = id / (DK / 16), it = id % (DK / 16);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = tile<C>([&](int t, int s) { return sm.N4[s][t]; }, [&](int s, int e) { return Qx(s, e); }, 16 * tm, 16 * it,
                  acc);
    acc = tile<C>([&](int t, int s) { return sm.N2[t][s] + sm.N2[s][t]; }, [&](int s, int e) { return Kx(s, e); },
                  16 * tm, 16 * it, acc);
    tile_each(acc, 16 * tm, 16 * it, [&](int t, int e, float v) {
      if (t < n) {
        const float val = v + cs.e[t] * mKt[t * LM + e] + cs.Gam[t] * mTW[t * LM + e];
        if (a.dk_part)
          a.dk_part[(row0 + (size_t)t * H) * DK + e] = val;
        else
          D::store(dkp, (kq0 + (size_t)t * a.Hk) * DK + e, val);
      }
    });
  }
}

// ---------------------------------------------------------------------------
// backward, bf16 path: local stage, reverse chain, state stage, gradients
// (cpr_backward_bf16.hpp); one work-group per (chunk slot, head) except the chain

struct SlotPos {
  int n;        // real tokens of the chunk
  size_t row0;  // row of its first token in [T, H, ...]
  size_t kq0;   // its row in [T, Hk, DK] (q, k)
  size_t sl;    // slot * H + h
};

__device__ __forceinline__ bool slot_pos(const BwdArgs& a, SlotPos& p) {
  const int slot = blockIdx.x, h = blockIdx.y, H = a.H;
  if (slot >= a.all_base[a.N]) return false;
  const int i = find_seq(a.all_base, a.N, slot);
  const int c = slot - a.all_base[i];
  const int L = a.cu[i + 1] - a.cu[i];
  p.n = min(a.Cl, L - c * a.Cl);
  const size_t tok0 = (size_t)a.cu[i] + (size_t)c * a.Cl;
  p.row0 = tok0 * H + h;
  p.kq0 = kq_row(tok0, h, a.Hk, a.G);
  p.sl = (size_t)slot * H + h;
  return true;
}

// waves per work-group of the local, state and gradient stages: their
// d-wide products split into 16-wide tiles over the waves, so two waves per
// SIMD where d_k and d_v give 8 tiles each (the LDS holds one work-group per CU)
template <int DK, int DV>
constexpr int kBwdWaves = (DK / 16) % 8 == 0 && (DV / 16) % 8 == 0 ? 8 : 4;

template <int DK, int DV>
__global__ __launch_bounds__((kBwdWaves<DK, DV> * 64)) void k_bwd_local_bf16(const BwdArgs a) {
  typedef bwdb::Slot<DK, DV> Sl;
  __shared__ bwdb::LocalLds<DK, DV> sm;
  SlotPos p;
  if (!slot_pos(a, p)) return;
  bwdb::local_stage<DK, DV, kBwdWaves<DK, DV>>(sm, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.d_o,
                            (const uint16_t*)a.g, (const uint16_t*)a.beta, p.row0, a.H, p.kq0, a.Hk, p.n,
                            a.ws + p.sl * Sl::bytes, a.gamn + p.sl);
}

// The state and gradient stages of one (chunk slot, head) in one work-group,
// the state stage's slot results (Dd, Delta, QB, dWn, dKt, dGamma_n) read back
// by the gradient stage once every wave's stores are complete.
template <int DK, int DV>
__global__ __launch_bounds__((kBwdWaves<DK, DV> * 64)) void k_bwd_state_grads_bf16(const BwdArgs a) {
  typedef bwdb::Slot<DK, DV> Sl;
  constexpr int W = kBwdWaves<DK, DV>;
  __shared__ bwdb::StateGradLds<DK, DV, W> sm;
  SlotPos p;
  if (!slot_pos(a, p)) return;
  uint8_t* slot = a.ws + p.sl * Sl::bytes;
  bwdb::state_stage<DK, DV, W>(sm, (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.d_o,
                               (const uint16_t*)a.g, (const uint16_t*)a.beta, p.row0, a.H, p.kq0, a.Hk, p.n,
                               a.bnd + p.sl * DK * DV, slot);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  bwdb::grad_stage<DK, DV, W>(sm, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                              (const uint16_t*)a.d_o, (const uint16_t*)a.g, (const uint16_t*)a.beta, p.row0, a.H,
                              p.kq0, a.Hk, p.n, slot, (uint16_t*)a.dq, (uint16_t*)a.dk, a.dq_part, a.dk_part,
                              (uint16_t*)a.dv, a.dg, a.dbeta);
}

// Reverse chain, bf16 path: the forward chain's structure run from the last
// chunk to the first.  Per chunk (dS = adjoint of the chunk's end state):
//   store dB' = dS;  E = Kt bf16(dS);  dS = fma(Gamma_n, dS, R) + (-W^T) bf16(E)
// Work-groups own CB = WAVES * NT * 16 state columns; the chunk's Kt / -W^T
// fragments and its R tiles for those columns go through a two-buffer LDS
// stage with loads two chunks ahead.
template <int DK, int DV, int WAVES, int NT>
__global__ __launch_bounds__(WAVES * 64) void k_bwd_chain_bf16(const BwdArgs a) {
  using namespace mfma;
  typedef bwdb::Slot<DK, DV> Sl;
  constexpr int kThreads = WAVES * 64;
  constexpr int CB = WAVES * NT * 16;
  constexpr int kFragPieces = (int)(Sl::oR / 16);
  constexpr int kRPieces = DK * CB * 4 / 16;
  constexpr int kPieces = kFragPieces + kRPieces;
  constexpr int kPer = kPieces / kThreads;
  constexpr int kPerFrag = kFragPieces / kThreads;
  static_assert(kPieces % kThreads == 0 && kFragPieces % kThreads == 0, "staging split");
  static_assert(DV % CB == 0, "column blocks tile d_v");
  __shared__ u32x4 stage[2][kPieces];
  __shared__ float gn_stage[2];
  const int i = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int jbg = blockIdx.z * (CB / 16), jb0 = jbg + wave * NT;
  const int H = a.H;
  const int L = a.cu[i + 1] - a.cu[i];
  const int nall = (L + a.Cl - 1) / a.Cl;
  const size_t sh = (size_t)i * H + h;
  const size_t SS = (size_t)DK * DV;
  const int abase = a.all_base[i];
  // step u visits chunk nall - 1 - u
  auto slot_of = [&](int u) { return a.ws + ((size_t)(abase + nall - 1 - u) * H + h) * Sl::bytes; };
  auto gamn_of = [&](int u) { return a.gamn[(size_t)(abase + nall - 1 - u) * H + h]; };
  auto fetch = [&](int u, u32x4 (&r)[kPer]) {
    const uint8_t* s = slot_of(u);
    const u32x4* f = reinterpret_cast<const u32x4*>(s);
    const u32x4* rr = reinterpret_cast<const u32x4*>(s + Sl::oR) + (size_t)jbg * (DK / 16) * 64;
#pragma unroll
    for (int m = 0; m < kPer; ++m) {
      const int p = tid + m * kThreads;
      r[m] = m < kPerFrag ? f[p] : rr[p - kFragPieces];
    }
  };
  auto put = [&](int buf, const u32x4 (&r)[kPer]) {
#pragma unroll
    for (int m = 0; m < kPer; ++m) stage[buf][tid + m * kThreads] = r[m];
  };
  auto barrier = [] { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };

  f32x4 S[DK / 16][NT];
  load_state_tiles<DK, DV, NT>(S, a.d_hT ? a.d_hT + sh * SS : nullptr, jb0, lane);
  u32x4 R0[kPer], R1[kPer];
  float G0 = 1.f, G1 = 1.f;
  if (nall > 0) {
    fetch(0, R0);
    G0 = gamn_of(0);
    put(0, R0);
    if (tid == 0) gn_stage[0] = G0;
    const int u1 = min(1, nall - 1);
    fetch(u1, R1);
    G1 = gamn_of(u1);
  }
  __syncthreads();
  auto step = [&](auto par, auto is_last, int u) {
    constexpr int P = decltype(par)::value;
    constexpr bool kLast = decltype(is_last)::value;
    u32x4(&RP)[kPer] = P ? R1 : R0;
    u32x4(&RQ)[kPer] = P ? R0 : R1;
    float& GP = P ? G1 : G0;
    float& GQ = P ? G0 : G1;
    if constexpr (!kLast) {
      const int uf = min(u + 2, nall - 1);
      fetch(uf, RP);
      GP = gamn_of(uf);
    }
    const u32x4* st = stage[P];
    const float gn = gn_stage[P];
    store_bnd_tiles<DK, NT>(reinterpret_cast<float*>(slot_of(u) + Sl::oDbp), S, jb0, lane);
    f32x4 Ut[C / 16][NT];
#pragma unroll
    for (int tm = 0; tm < C / 16; ++tm)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) Ut[tm][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    chain_step_bf16_init<DK, NT>(
        S, [&](int kb, int tm) { return st[(kb * (C / 16) + tm) * 64 + lane]; },
        [&](int kb, int im) { return st[(int)(Sl::oWNF / 16) + (kb * (DK / 16) + im) * 64 + lane]; }, Ut,
        [&](int im, int nt, const f32x4& x) {
          const f32x4 r =
              __builtin_bit_cast(f32x4, st[kFragPieces + ((wave * NT + nt) * (DK / 16) + im) * 64 + lane]);
          return f32x4{__builtin_fmaf(gn, x[0], r[0]), __builtin_fmaf(gn, x[1], r[1]), __builtin_fmaf(gn, x[2], r[2]),
                       __builtin_fmaf(gn, x[3], r[3])};
        });
    if constexpr (!kLast) {
      put(P ^ 1, RQ);
      if (tid == 0) gn_stage[P ^ 1] = GQ;
      barrier();
    }
  };
  typedef std::integral_constant<int, 0> P0;
  typedef std::integral_constant<int, 1> P1;
  typedef std::integral_constant<bool, false> Mid;
  typedef std::integral_constant<bool, true> Last;
  int u = 0;
  for (; u + 2 < nall; u += 2) {
    step(P0{}, Mid{}, u);
    step(P1{}, Mid{}, u + 1);
  }
  if (u + 1 < nall) {
    step(P0{}, Mid{}, u);
    step(P1{}, Last{}, u + 1);
  } else if (u < nall) {
    step(P0{}, Last{}, u);
  }
  if (a.dh0) store_state_tiles<DK, DV, NT>(a.dh0 + sh * SS, S, jb0, lane);
}


}  // namespace
