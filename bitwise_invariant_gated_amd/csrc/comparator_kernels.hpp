// Comparator kernels (not CPR): recurrent everywhere, chunkwise prefill with
// recurrent decode, chunkwise-everywhere decode.
//
// Part of libgdn_cpr (included by gdn_cpr.hip, in this order: prefill_kernels.hpp,
// decode_kernels.hpp, comparator_kernels.hpp, backward_kernels.hpp).
#pragma once

#include "decode_kernels.hpp"

namespace {

// ---------------------------------------------------------------------------
// comparators (not CPR): the two evaluation orders whose mismatch the pages
// describe, built from this library's routines (English page, CPR section
// and its table; Chinese page, third-way section):
//   recurrent everywhere   the token step over each whole sequence, and the
//                          same step for decode (no chunk boundaries)
//   chunkwise everywhere   boundary states over every chunk (the last,
//                          partial chunk zero-padded) and the outputs from the
//                          chunk form O = diag(Gamma) Q B + (Q K^T .* D) Delta,
//                          with no per-token scan
// "Native mixed" serving is the chunkwise prefill followed by the recurrent
// decode: both are exact in exact arithmetic, but they round differently.

struct CmpArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* g;
  const void* beta;
  const int32_t* cu;
  const float* h0;
  float* state;  // [N, H, DK, DV] final state (prefill) / running state (decode)
  void* o;
  int32_t* all_base;
  uint8_t* prod;
  float* gamn;
  float* bnd;
  int32_t N;
  int32_t H;
  int32_t Hk;  // heads of q and k
  int32_t G;   // value heads per key head, H / Hk
};

// recurrent prefill: one wave per (sequence, head, 64 state columns), the
// scan's operand delivery (DPP row broadcast) over every token in order
template <class D, int DK, int DV>
__global__ __launch_bounds__(64, 3) void k_cmp_rec_prefill(const CmpArgs a) {
  using T = typename D::T;
  const int i = blockIdx.x, h = blockIdx.y, H = a.H;
  const int lane = threadIdx.x, col = blockIdx.z * kWave + lane;
  const int L = a.cu[i + 1] - a.cu[i];
  const size_t sh = (size_t)i * H + h;
  const size_t SS = (size_t)DK * DV;
  float s[DK];
#pragma unroll
  for (int ii = 0; ii < DK; ++ii) s[ii] = a.h0 ? a.h0[sh * SS + (size_t)ii * DV + col] : 0.f;
  const T* gp = (const T*)a.g;
  const T* bp = (const T*)a.beta;
  const T* kp = (const T*)a.k;
  const T* qp = (const T*)a.q;
  const T* vp = (const T*)a.v;
  T* op = (T*)a.o;
  for (int c0 = 0; c0 < L; c0 += kWave) {
    const int n = min(kWave, L - c0);
    const size_t tok0 = (size_t)a.cu[i] + c0;
    float alpha_l = 1.f, beta_l = 0.f;
    if (lane < n) {
      const size_t r = (tok0 + lane) * H + h;
      alpha_l = decay_of(D::load(gp, r));
      beta_l = D::load(bp, r);
    }
    scan_tokens_plain<D, DK, DV>(s, kp, qp, vp, op, tok0 * H + h, H, kq_row(tok0, h, a.Hk, a.G), a.Hk, n, col,
                                 lane, alpha_l, beta_l);
  }
#pragma unroll
  for (int ii = 0; ii < DK; ++ii) a.state[sh * SS + (size_t)ii * DV + col] = s[ii];
}

// recurrent decode: the per-token step on the running state, nothing else
template <class D, int DK, int DV>
__global__ __launch_bounds__(DV) void k_cmp_rec_decode(const CmpArgs a) {
  using T = typename D::T;
  const size_t sh = (size_t)blockIdx.x * a.H + blockIdx.y;
  const int col = threadIdx.x;
  float* R = a.state + sh * (size_t)DK * DV;
  float s[DK];
#pragma unroll
  for (int ii = 0; ii < DK; ++ii) s[ii] = R[(size_t)ii * DV + col];
  const T* kp = (const T*)a.k;
  const T* qp = (const T*)a.q;
  const float alpha = decay_of(D::load((const T*)a.g, sh));
  const float bt = D::load((const T*)a.beta, sh);
  const float vv = D::load((const T*)a.v, sh * DV + col);
  const size_t kr = kq_row(blockIdx.x, blockIdx.y, a.Hk, a.G);
  KQRaw<D> raw;
  load_kq<D, DK>(raw, kp + kr * DK, qp + kr * DK, col);
  float kf[8], qf[8];
  unpack_kq<D>(raw, kf, qf);
  const float out = token_step_plain<DK>(s, kf, qf, alpha, bt, vv);
  D::store((T*)a.o, sh * DV + col, out);
#pragma unroll
  for (int ii = 0; ii < DK; ++ii) R[(size_t)ii * DV + col] = s[ii];
}

// chunkwise: chunk products of every chunk slot, a partial chunk padded with
// k = v = 0, g = beta = 0 (identity steps)
template <int DK, int DV>
__global__ __launch_bounds__(256, 3) void k_cmp_chunk_local_bf16(const CmpArgs a) {
  typedef SlotB<DK, DV> Sl;
  __shared__ ChunkLdsB<DK, DV> sm;
  const int slot = blockIdx.x, h = blockIdx.y, H = a.H;
  if (slot >= a.all_base[a.N]) return;
  const int i = find_seq(a.all_base, a.N, slot);
  const int c = slot - a.all_base[i];
  const int n = min(C, a.cu[i + 1] - a.cu[i] - c * C);
  const size_t tok0 = (size_t)a.cu[i] + (size_t)c * C;
  const size_t row0 = tok0 * H + h, kq0 = kq_row(tok0, h, a.Hk, a.G);
  stage_chunk_bf16<DK, DV>(sm, (const uint16_t*)a.k, kq0, a.Hk, (const uint16_t*)a.v, row0, H,
                           (const uint16_t*)a.g, (const uint16_t*)a.beta, row0, H, n);
  const size_t ps = (size_t)slot * H + h;
  chunk_local_bf16<DK, DV>(sm, a.prod + ps * Sl::bytes, a.gamn + ps);
}

// chunkwise outputs: per (chunk slot, head), 4 waves x 32 state columns
//   Delta = U + Wneg bf16(B)                       (as the chain's first phase)
//   O     = diag(Gamma) (Q bf16(B)) + bf16(P) bf16(Delta),  P = (Q K^T) .* D
template <int DK, int DV>
struct CmpOutLds {
  uint16_t Q[C][DK + 8];
  uint16_t K[C][DK + 8];
  uint16_t P[C][C + 8];
  float g[C], gam[C], Gam[C];
};

// gamma, Gamma and P = bf16((Q K^T) .* D) of a chunk staged in sm (Q, K, g)
template <int DK, int DV>
__device__ __forceinline__ void cmp_out_prepare(CmpOutLds<DK, DV>& sm) {
  using namespace mfma;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 15, g = lane >> 4;
  if (tid == 0) {
    float acc = sm.g[0];
    sm.gam[0] = acc;
    for (int t = 1; t < C; ++t) {
      acc = acc + sm.g[t];
      sm.gam[t] = acc;
    }
  }
  __syncthreads();
  if (tid < C) sm.Gam[tid] = expf(sm.gam[tid]);
  for (int q2 = wave; q2 < 16; q2 += 4) {
    const int tm = q2 >> 2, tn = q2 & 3;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (tn <= tm) {
#pragma unroll
      for (int kb = 0; kb < DK / 32; ++kb)
        acc = mma(frag_row(&sm.Q[16 * tm + lr][0], 32 * kb, g), frag_row(&sm.K[16 * tn + lr][0], 32 * kb, g), acc);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * tm + 4 * g + r, s2 = 16 * tn + lr;
      sm.P[t][s2] = Bf16::round(s2 <= t ? acc[r] * expf(sm.gam[t] - sm.gam[s2]) : 0.f);
    }
  }
  __syncthreads();
}

// Chunkwise outputs of the 16-row tiles tm0 <= tm < tm1 of one chunk, this
// wave's DV / 4 state columns: S = the chunk's start state (accumulator
// tiles), sl = its product slot.  out(row, column, value) receives each.
template <int DK, int DV, class Out>
__device__ __forceinline__ void cmp_out_rows(const CmpOutLds<DK, DV>& sm, const mfma::f32x4 (&S)[DK / 16][DV / 64],
                                             const uint8_t* sl, int tm0, int tm1, Out&& out) {
  using namespace mfma;
  typedef SlotB<DK, DV> Sl;
  constexpr int NT = DV / 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, lr = lane & 15, g = lane >> 4;
  const int jb0 = wave * NT;
  const u32x4* WF = reinterpret_cast<const u32x4*>(sl + Sl::oWF);
  const f32x4* UT = reinterpret_cast<const f32x4*>(sl + Sl::oU);
  u32x4 Sb[DK / 32][NT];
#pragma unroll
  for (int kb = 0; kb < DK / 32; ++kb)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) Sb[kb][nt] = frag_from_acc(S[2 * kb][nt], S[2 * kb + 1][nt]);
  f32x4 Dl[C / 16][NT];
#pragma unroll
  for (int tm = 0; tm < C / 16; ++tm)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) Dl[tm][nt] = UT[((jb0 + nt) * (C / 16) + tm) * 64 + lane];
#pragma unroll
  for (int kb = 0; kb < DK / 32; ++kb)
#pragma unroll
    for (int tm = 0; tm < C / 16; ++tm) {
      const u32x4 w = WF[(kb * (C / 16) + tm) * 64 + lane];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) Dl[tm][nt] = mma(w, Sb[kb][nt], Dl[tm][nt]);
    }
  u32x4 Db[C / 32][NT];
#pragma unroll
  for (int kb = 0; kb < C / 32; ++kb)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) Db[kb][nt] = frag_from_acc(Dl[2 * kb][nt], Dl[2 * kb + 1][nt]);
#pragma unroll
  for (int tm = 0; tm < C / 16; ++tm) {
    if (tm < tm0 || tm >= tm1) continue;
    f32x4 O[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) O[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < DK / 32; ++kb) {
      const u32x4 qf = frag_row(&sm.Q[16 * tm + lr][0], 32 * kb, g);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) O[nt] = mma(qf, Sb[kb][nt], O[nt]);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) O[nt][r] *= sm.Gam[16 * tm + 4 * g + r];
#pragma unroll
    for (int kb = 0; kb < C / 32; ++kb) {
      const u32x4 pf = frag_row(&sm.P[16 * tm + lr][0], 32 * kb, g);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) O[nt] = mma(pf, Db[kb][nt], O[nt]);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) out(16 * tm + 4 * g + r, 16 * (jb0 + nt) + lr, O[nt][r]);
  }
}

template <int DK, int DV>
__global__ __launch_bounds__(256) void k_cmp_chunk_out_bf16(const CmpArgs a) {
  typedef SlotB<DK, DV> Sl;
  constexpr int NT = DV / 64;  // 16-column tiles per wave
  __shared__ CmpOutLds<DK, DV> sm;
  const int slot = blockIdx.x, h = blockIdx.y, H = a.H;
  if (slot >= a.all_base[a.N]) return;
  const int i = find_seq(a.all_base, a.N, slot);
  const int c = slot - a.all_base[i];
  const int n = min(C, a.cu[i + 1] - a.cu[i] - c * C);
  const size_t tok0 = (size_t)a.cu[i] + (size_t)c * C;
  const size_t row0 = tok0 * H + h, kq0 = kq_row(tok0, h, a.Hk, a.G);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const uint16_t* qp = (const uint16_t*)a.q;
  const uint16_t* kp = (const uint16_t*)a.k;
  typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
  for (int idx = tid; idx < C * DK / 8; idx += 256) {
    const int t = idx / (DK / 8), i0 = (idx % (DK / 8)) * 8;
    u32x4v wq = {0u, 0u, 0u, 0u}, wk = {0u, 0u, 0u, 0u};
    if (t < n) {
      wq = *reinterpret_cast<const u32x4v*>(qp + (kq0 + (size_t)t * a.Hk) * DK + i0);
      wk = *reinterpret_cast<const u32x4v*>(kp + (kq0 + (size_t)t * a.Hk) * DK + i0);
    }
    *reinterpret_cast<u32x4v*>(&sm.Q[t][i0]) = wq;
    *reinterpret_cast<u32x4v*>(&sm.K[t][i0]) = wk;
  }
  if (tid < C) sm.g[tid] = tid < n ? Bf16::load((const uint16_t*)a.g, row0 + (size_t)tid * H) : 0.f;
  __syncthreads();
  cmp_out_prepare(sm);
  const size_t ps = (size_t)slot * H + h;
  const float* B = a.bnd + ps * (size_t)DK * DV;
  const int jb0 = wave * NT;
  mfma::f32x4 S[DK / 16][NT];
#pragma unroll
  for (int im = 0; im < DK / 16; ++im)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      S[im][nt] = *reinterpret_cast<const mfma::f32x4*>(B + ((size_t)((jb0 + nt) * (DK / 16) + im) * 64 + lane) * 4);
  uint16_t* op = (uint16_t*)a.o;
  cmp_out_rows(sm, S, a.prod + ps * Sl::bytes, 0, C / 16, [&](int t, int col, float val) {
    if (t < n) op[(row0 + (size_t)t * H) * DV + col] = Bf16::round(val);
  });
}

// chunkwise-everywhere decode (comparator): every token recomputes the chunk
// products of its partial chunk -- the cached tail, then the token, then zero
// padding -- and takes its output from the chunk form on the cache's boundary
// state, as the chunkwise prefill does for the same token.  When the token
// completes the chunk, k_chain_resync_bf16 moves the boundary (s_run follows
// it then; between boundaries this comparator leaves s_run alone).
template <int DK, int DV>
__global__ __launch_bounds__(256, 3) void k_cmp_cdec_local_bf16(const DecodeArgs a) {
  __shared__ ChunkLdsB<DK, DV> sm;
  const size_t sh = (size_t)blockIdx.x * a.H + blockIdx.y;
  const size_t ch = cache_row(a.slot, blockIdx.x) * a.H + blockIdx.y;
  const int tl = a.tail_len[ch];
  if ((unsigned)tl >= (unsigned)C) return;
  const int tid = threadIdx.x;
  const size_t kr = kq_row(blockIdx.x, blockIdx.y, a.Hk, a.G);
  const uint16_t* tk = (const uint16_t*)a.tail_k;
  const uint16_t* tv = (const uint16_t*)a.tail_v;
  const uint16_t* kp = (const uint16_t*)a.k;
  const uint16_t* vp = (const uint16_t*)a.v;
  typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
  // rows t < tl from the tail, row tl the token, rows past it zero: every
  // load is issued (rows past tl load the token again) before the LDS writes
  constexpr int MK = C * DK / 8 / 256, MV = C * DV / 8 / 256;
  u32x4v lk[MK], lv[MV];
#pragma unroll
  for (int m = 0; m < MK; ++m) {
    const int idx = tid + 256 * m, t = idx / (DK / 8), i0 = (idx % (DK / 8)) * 8;
    const uint16_t* src = t < tl ? tk + (ch * C + t) * DK : kp + kr * DK;
    lk[m] = *reinterpret_cast<const u32x4v*>(src + i0);
  }
#pragma unroll
  for (int m = 0; m < MV; ++m) {
    const int idx = tid + 256 * m, t = idx / (DV / 8), j0 = (idx % (DV / 8)) * 8;
    const uint16_t* src = t < tl ? tv + (ch * C + t) * DV : vp + sh * DV;
    lv[m] = *reinterpret_cast<const u32x4v*>(src + j0);
  }
  const int ts = min(tid, C - 1);
  const uint16_t* gs = ts < tl ? (const uint16_t*)a.tail_g : (const uint16_t*)a.g;
  const uint16_t* bs = ts < tl ? (const uint16_t*)a.tail_beta : (const uint16_t*)a.beta;
  const size_t r = ts < tl ? ch * C + ts : sh;
  const float gl = Bf16::load(gs, r), bl = Bf16::load(bs, r);
  const u32x4v zero = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int m = 0; m < MK; ++m) {
    const int idx = tid + 256 * m, t = idx / (DK / 8);
    *reinterpret_cast<u32x4v*>(&sm.K[t][(idx % (DK / 8)) * 8]) = t <= tl ? lk[m] : zero;
  }
#pragma unroll
  for (int m = 0; m < MV; ++m) {
    const int idx = tid + 256 * m, t = idx / (DV / 8);
    *reinterpret_cast<u32x4v*>(&sm.V[t][(idx % (DV / 8)) * 8]) = t <= tl ? lv[m] : zero;
  }
  if (tid < C) {
    sm.gam[tid] = tid <= tl ? gl : 0.f;
    sm.beta[tid] = tid <= tl ? bl : 0.f;
  }
  __syncthreads();
  chunk_local_bf16<DK, DV>(sm, a.prod + sh * prod_slot_bytes(true, DK, DV), a.gamn + sh);
  // append the token to the tail (row tl of the tail is read by no kernel of this step)
  uint16_t* wk = (uint16_t*)a.tail_k + (ch * C + tl) * DK;
  uint16_t* wv = (uint16_t*)a.tail_v + (ch * C + tl) * DV;
  for (int e = tid; e < DK; e += 256) wk[e] = kp[kr * DK + e];
  for (int e = tid; e < DV; e += 256) wv[e] = vp[sh * DV + e];
  if (tid == 0) {
    ((uint16_t*)a.tail_g)[ch * C + tl] = ((const uint16_t*)a.g)[sh];
    ((uint16_t*)a.tail_beta)[ch * C + tl] = ((const uint16_t*)a.beta)[sh];
  }
}

// its output row, then tail_len and the resynchronisation flag
template <int DK, int DV>
__global__ __launch_bounds__(256) void k_cmp_cdec_out_bf16(const DecodeArgs a) {
  constexpr int NT = DV / 64;
  __shared__ CmpOutLds<DK, DV> sm;
  const size_t sh = (size_t)blockIdx.x * a.H + blockIdx.y;
  const size_t ch = cache_row(a.slot, blockIdx.x) * a.H + blockIdx.y;
  const int tl = a.tail_len[ch];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  __syncthreads();  // every wave has read tail_len before it is rewritten below
  if ((unsigned)tl >= (unsigned)C) {
    if (tid == 0) a.flag[sh] = 0;
    return;
  }
  const uint16_t* tk = (const uint16_t*)a.tail_k;
  const uint16_t* qp = (const uint16_t*)a.q;
  const uint16_t* kp = (const uint16_t*)a.k;
  typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
  for (int idx = tid; idx < C * DK / 8; idx += 256) {
    const int t = idx / (DK / 8), i0 = (idx % (DK / 8)) * 8;
    u32x4v wq = {0u, 0u, 0u, 0u}, wk = {0u, 0u, 0u, 0u};
    if (t < tl) wk = *reinterpret_cast<const u32x4v*>(tk + (ch * C + t) * DK + i0);
    if (t == tl) {
      wq = *reinterpret_cast<const u32x4v*>(qp + kq_row(blockIdx.x, blockIdx.y, a.Hk, a.G) * DK + i0);
      wk = *reinterpret_cast<const u32x4v*>(kp + kq_row(blockIdx.x, blockIdx.y, a.Hk, a.G) * DK + i0);
    }
    *reinterpret_cast<u32x4v*>(&sm.Q[t][i0]) = wq;
    *reinterpret_cast<u32x4v*>(&sm.K[t][i0]) = wk;
  }
  if (tid < C)
    sm.g[tid] = tid < tl ? Bf16::load((const uint16_t*)a.tail_g, ch * C + tid)
                         : (tid == tl ? Bf16::load((const uint16_t*)a.g, sh) : 0.f);
  __syncthreads();
  cmp_out_prepare(sm);
  mfma::f32x4 S[DK / 16][NT];
  load_state_tiles<DK, DV, NT>(S, a.s_bnd + ch * (size_t)DK * DV, wave * NT, lane);
  uint16_t* op = (uint16_t*)a.o;
  cmp_out_rows(sm, S, a.prod + sh * prod_slot_bytes(true, DK, DV), tl / 16, tl / 16 + 1,
               [&](int t, int col, float val) {
                 if (t == tl) op[sh * DV + col] = Bf16::round(val);
               });
  if (tid == 0) {
    const bool full = (tl + 1 == C);
    a.tail_len[ch] = full ? 0 : tl + 1;
    a.flag[sh] = full ? 1 : 0;
  }
}


}  // namespace
