// Prefill kernels: kernel arguments, the varlen plan, chunk products, the
// boundary chain, the in-chunk scan and the one-launch prefill.
//
// Part of libgdn_cpr (included by gdn_cpr.hip, in this order: prefill_kernels.hpp,
// decode_kernels.hpp, comparator_kernels.hpp, backward_kernels.hpp).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "cpr_device.hpp"

// private to the library: the kernels name cpr's routines unqualified
using namespace cpr;

namespace {


// C is the row count of the chunk machinery (chunk-product slots, MFMA tiles,
// LDS arrays): 64.  The layer's chunk length Cl (the boundary and
// resynchronisation period, 16, 32 or 64) is a runtime argument: a chunk of
// Cl tokens fills the first Cl rows of a 64-row slot and the other rows are
// identity padding (k = v = 0, g = beta = 0), which adds exact zeros to every
// product and leaves the cumulative decay unchanged, so the real rows'
// values are those of a Cl-row computation.
constexpr int C = kChunk;
constexpr int kChainCols = 32;  // state columns per boundary-chain work item
// cache-policy bits of a buffer access with agent (device) scope coherence
// (SC1): the access is coherent with every other work-group of the launch
// whatever its XCD, with no cache-wide write-back or invalidate
constexpr int kAuxAgent = 16;

// ---------------------------------------------------------------------------
// kernel arguments

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* g;
  const void* beta;
  const int32_t* start;  // [N] first token row of each sequence
  const int32_t* end;    // [N] one past its last token row (cu_seqlens + 1 for a plain prefill)
  int32_t skip_empty;    // 1: a sequence with no tokens leaves its cache untouched
  const int32_t* slot;   // [N] cache row of sequence i, or null (row i)
  int32_t h0_slotted;    // 1: h0 is indexed by cache row (h0 = the cache's s_bnd)
  int32_t all_chunks;    // 1 (comparator): products exist for every chunk slot, partial ones zero-padded;
                         // the chain runs over all of them and writes only the final state to s_bnd
  const float* h0;
  float* s_bnd;
  float* s_run;
  void* tail_k;
  void* tail_v;
  void* tail_g;
  void* tail_beta;
  int32_t* tail_len;
  float* lgs;  // [rows, H] log-scale of s_run (the cache's run_log_scale), or null
  float* hT;   // [N, H, DK, DV] final state exp(lg) N of every sequence (batch order), or null
  void* o;
  int32_t* full_base;  // [N+1] prefix sums of full chunks per sequence
  int32_t* all_base;   // [N+1] prefix sums of all chunks (full + partial)
  uint8_t* prod;       // [F_max*H] chunk-product slots of prod_slot_bytes
  float* gamn;         // [F_max*H]
  float* bnd;          // [A_max*H][DK][DV] state at the start of every chunk
  int32_t* order;      // [A_max] fused launch: chunk-major slot order (workspace)
  int32_t* ready;      // [N*H*NZ*kReadyStride] fused launch: published boundary counts (workspace)
  int32_t* counters;   // [2] fused launch: ticket, timeout (workspace)
  int32_t N;
  int32_t H;
  int32_t Hk;  // heads of q and k
  int32_t G;   // value heads per key head, H / Hk
  int32_t Cl;  // chunk length
};

struct DecodeArgs {
  const int32_t* slot;  // [N] cache row of sequence i, or null (row i)
  const void* q;
  const void* k;
  const void* v;
  const void* g;
  const void* beta;
  float* s_bnd;
  float* s_run;
  void* tail_k;
  void* tail_v;
  void* tail_g;
  void* tail_beta;
  int32_t* tail_len;
  float* lgs;  // [rows, H] log-scale of s_run, or null (written 0 when s_run becomes a boundary)
  float* hT;   // [N, H, DK, DV] state after the step (batch order), or null
  void* o;
  int32_t* flag;  // [N*H] bit 0: this pair resynchronises in this step; bit 1: the resync also writes hT
  uint8_t* prod;  // chunk-product slots of prod_slot_bytes, one per pair of a resync launch
  float* gamn;    // one per product slot
  int32_t seq0;   // resync launches: the grid's sequence 0 is sequence seq0 of the batch
  int32_t N;
  int32_t H;
  int32_t Hk;  // heads of q and k
  int32_t G;   // value heads per key head, H / Hk
  int32_t Cl;  // chunk length (rows per cache tail)
};

template <int DK, int DV>
__host__ __device__ constexpr size_t prod_floats() {
  return (size_t)C * DK + (size_t)C * DV + (size_t)DK * C;
}

// bytes of one chunk-product slot: fp32 W, U, K~^T on the fp32 path; bf16
// Wneg and K~^T plus fp32 U on the bf16 (MFMA) path
__host__ __device__ constexpr size_t prod_slot_bytes(bool bf16, int DK, int DV) {
  return bf16 ? (size_t)C * DK * 2 + (size_t)DK * C * 2 + (size_t)C * DV * 4
              : ((size_t)C * DK + (size_t)C * DV + (size_t)DK * C) * 4;
}

// largest i in [0, N) with base[i] <= slot (slot < base[N] assumed)
__device__ __forceinline__ int find_seq(const int32_t* __restrict__ base, int N, int slot) {
  int lo = 0, hi = N;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (base[mid] <= slot)
      lo = mid;
    else
      hi = mid;
  }
  return lo;
}

// cache row of batch entry i (slot-indexed caches)
__device__ __forceinline__ size_t cache_row(const int32_t* __restrict__ slot, int i) {
  return slot ? (size_t)slot[i] : (size_t)i;
}

// row of q and k ([rows, Hk, d_k]) that value head h of token row tok reads:
// key head h / G (value heads jG .. jG + G - 1 share key head j)
__device__ __forceinline__ size_t kq_row(size_t tok, int h, int Hk, int G) { return tok * Hk + h / G; }

// ---------------------------------------------------------------------------
// varlen plan: exclusive prefix sums of full and of all chunks per sequence

// Bookkeeping of the fused boundary-chain + scan launch (k_chain_scan_bf16),
// prepared by the plan kernel of the same call.
struct FusedPlan {
  int32_t* order;   // [A] chunk slots in chunk-major order (chunk 0 of every sequence, then chunk 1, ...),
                    // or null: no fused launch follows
  int32_t* ticket;  // [2] work-item counter of the fused launch, then its wait-timeout word
                    // (cleared by every plan that is given them, fused launch or not)
  int32_t* ready;   // [n_ready] boundaries published so far by each chain item
  int32_t n_ready;
};
constexpr int kFusedMaxSeqs = 128;  // sequences per call for which the plan builds the chunk-major order

__global__ __launch_bounds__(1024) void k_plan(const int32_t* __restrict__ start, const int32_t* __restrict__ end,
                                               int32_t N, int32_t Cl, int32_t* __restrict__ full_base,
                                               int32_t* __restrict__ all_base, const FusedPlan fp) {
  // 1024 sequences per pass: an inclusive scan inside each wave (shuffles),
  // the 16 wave totals through LDS, and the running totals of earlier passes
  // (integers, so the order of the sums does not matter)
  __shared__ int32_t wf[16], wa[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int cf = 0, ca = 0;
  for (int base = 0; base < N; base += 1024) {
    const int i = base + tid;
    int nf = 0, na = 0;
    if (i < N) {
      const int L = end[i] - start[i];
      nf = L / Cl;
      na = (L + Cl - 1) / Cl;
    }
    int sf = nf, sa = na;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int xf = __shfl_up(sf, off), xa = __shfl_up(sa, off);
      if (lane >= off) {
        sf += xf;
        sa += xa;
      }
    }
    if (lane == 63) {
      wf[wave] = sf;
      wa[wave] = sa;
    }
    __syncthreads();
    int pf = 0, pa = 0, tf = 0, ta = 0;
    for (int w = 0; w < 16; ++w) {
      if (w < wave) {
        pf += wf[w];
        pa += wa[w];
      }
      tf += wf[w];
      ta += wa[w];
    }
    if (i < N) {
      full_base[i] = cf + pf + sf - nf;
      all_base[i] = ca + pa + sa - na;
    }
    cf += tf;
    ca += ta;
    __syncthreads();  // wf, wa are rewritten by the next pass
  }
  if (tid == 0) {
    full_base[N] = cf;
    all_base[N] = ca;
  }
  if (tid == 0 && fp.ticket) fp.ticket[1] = 0;  // no wait of this call has given up (yet)
  if (fp.order == nullptr) return;
  // fused launch: clear its counters, and order the chunk slots by chunk
  // index (then by sequence): slot (i, c) goes to position
  //   sum_j min(nall_j, c) + #{j < i : nall_j > c}
  // so that the scan units of early chunks, whose boundaries the chain
  // publishes first, are taken first.  The order only schedules work; no
  // result depends on it.
  __shared__ int32_t nall_s[kFusedMaxSeqs];
  for (int j = tid; j < fp.n_ready; j += 1024) fp.ready[j] = 0;
  if (tid == 0) *fp.ticket = 0;
  for (int j = tid; j < N; j += 1024) nall_s[j] = (end[j] - start[j] + Cl - 1) / Cl;
  __syncthreads();  // nall_s and all_base complete
  for (int sl = tid; sl < ca; sl += 1024) {
    const int i = find_seq(all_base, N, sl);
    const int c = sl - all_base[i];
    int pos = 0;
    for (int j = 0; j < N; ++j) {
      const int nj = nall_s[j];
      pos += min(nj, c) + ((j < i && nj > c) ? 1 : 0);
    }
    fp.order[pos] = sl;
  }
}

// ---------------------------------------------------------------------------
// chunk products

template <class D, int DK, int DV>
__device__ __forceinline__ void stage_chunk(ChunkLds<DK, DV>& sm, const typename D::T* __restrict__ k,
                                            size_t k_row0, size_t k_stride,
                                            const typename D::T* __restrict__ v, size_t v_row0,
                                            size_t v_stride, const typename D::T* __restrict__ g,
                                            const typename D::T* __restrict__ beta, size_t gb0,
                                            size_t gb_stride, int n) {
  // rows t >= n (a chunk shorter than the slot) are identity padding
  const int tid = threadIdx.x, nt = blockDim.x;
  for (int idx = tid; idx < C * DK; idx += nt) {
    const int t = idx / DK, i = idx % DK;
    sm.K[t][i] = t < n ? D::load(k, (k_row0 + (size_t)t * k_stride) * DK + i) : 0.f;
  }
  for (int idx = tid; idx < C * DV; idx += nt) {
    const int t = idx / DV, j = idx % DV;
    sm.V[t][j] = t < n ? D::load(v, (v_row0 + (size_t)t * v_stride) * DV + j) : 0.f;
  }
  for (int t = tid; t < C; t += nt) {
    sm.g[t] = t < n ? D::load(g, gb0 + (size_t)t * gb_stride) : 0.f;
    sm.beta[t] = t < n ? D::load(beta, gb0 + (size_t)t * gb_stride) : 0.f;
  }
  __syncthreads();
}

template <class D, int DK, int DV>
__global__ __launch_bounds__(256) void k_chunk_local_prefill(const PrefillArgs a) {
  using T = typename D::T;
  __shared__ ChunkLds<DK, DV> sm;
  const int f = blockIdx.x, h = blockIdx.y;
  const int N = a.N, H = a.H;
  if (f >= a.full_base[N]) return;
  const int i = find_seq(a.full_base, N, f);
  const int c = f - a.full_base[i];
  const size_t tok0 = (size_t)a.start[i] + (size_t)c * a.Cl;
  const size_t row0 = tok0 * H + h;  // row index into [T, H, ...]
  stage_chunk<D, DK, DV>(sm, (const T*)a.k, kq_row(tok0, h, a.Hk, a.G), a.Hk, (const T*)a.v, row0, H,
                         (const T*)a.g, (const T*)a.beta, row0, H, a.Cl);
  const size_t slot = (size_t)f * H + h;
  float* P = (float*)(a.prod + slot * prod_slot_bytes(false, DK, DV));
  chunk_local_f32<DK, DV>(sm, P, P + C * DK, P + C * DK + C * DV, a.gamn + slot);
}

template <class D, int DK, int DV>
__global__ __launch_bounds__(256) void k_chunk_local_resync(const DecodeArgs a) {
  using T = typename D::T;
  __shared__ ChunkLds<DK, DV> sm;
  const int i = a.seq0 + blockIdx.x;
  const size_t sh = (size_t)i * a.H + blockIdx.y;
  if (a.flag[sh] == 0) return;
  const size_t ps = (size_t)blockIdx.x * a.H + blockIdx.y;  // product slot
  const size_t ch = cache_row(a.slot, i) * a.H + blockIdx.y;
  // tail rows of this (sequence, head): [Cl, DK], [Cl, DV], [Cl]
  const size_t tr = ch * a.Cl;
  stage_chunk<D, DK, DV>(sm, (const T*)a.tail_k, tr, 1, (const T*)a.tail_v, tr, 1, (const T*)a.tail_g,
                         (const T*)a.tail_beta, tr, 1, a.Cl);
  float* P = (float*)(a.prod + ps * prod_slot_bytes(false, DK, DV));
  chunk_local_f32<DK, DV>(sm, P, P + C * DK, P + C * DK + C * DV, a.gamn + ps);
}

// bf16 path: MFMA chunk products
template <int DK, int DV>
__global__ __launch_bounds__(256, 3) void k_chunk_local_prefill_bf16(const PrefillArgs a) {
  __shared__ ChunkLdsB<DK, DV> sm;
  const int f = blockIdx.x, h = blockIdx.y;
  const int N = a.N, H = a.H;
  if (f >= a.full_base[N]) return;
  const int i = find_seq(a.full_base, N, f);
  const int c = f - a.full_base[i];
  const size_t tok0 = (size_t)a.start[i] + (size_t)c * a.Cl;
  const size_t row0 = tok0 * H + h;
  stage_chunk_bf16<DK, DV>(sm, (const uint16_t*)a.k, kq_row(tok0, h, a.Hk, a.G), a.Hk, (const uint16_t*)a.v, row0,
                           H, (const uint16_t*)a.g, (const uint16_t*)a.beta, row0, H, a.Cl);
  const size_t slot = (size_t)f * H + h;
  chunk_local_bf16<DK, DV>(sm, a.prod + slot * prod_slot_bytes(true, DK, DV), a.gamn + slot);
}


// ---------------------------------------------------------------------------
// boundary chain

template <int DK, int DV, int NB>
__device__ __forceinline__ void stage_products(ChainLds<DK, NB>& sm, const float* __restrict__ P,
                                               const float* __restrict__ gamn, int col0) {
  const int tid = threadIdx.x, nt = blockDim.x;
  const float* W = P;
  const float* U = P + C * DK;
  const float* KtT = P + C * DK + C * DV;
  for (int idx = tid; idx < C * DK; idx += nt) (&sm.W[0][0])[idx] = W[idx];
  for (int idx = tid; idx < DK * C; idx += nt) (&sm.KtT[0][0])[idx] = KtT[idx];
  for (int idx = tid; idx < C * NB; idx += nt) {
    const int t = idx / NB, j = idx % NB;
    sm.U[t][j] = U[t * DV + col0 + j];
  }
  if (tid == 0) sm.gamn = *gamn;
  __syncthreads();
}

template <int DK, int DV, int NB>
__device__ __forceinline__ void put_block(float* __restrict__ dst, const ChainLds<DK, NB>& sm, int col0) {
  for (int idx = threadIdx.x; idx < DK * NB; idx += blockDim.x) {
    const int i = idx / NB, j = idx % NB;
    dst[(size_t)i * DV + col0 + j] = sm.S[i][j];
  }
}

// the same block into a boundary slot (accumulator-tile order, bnd_index)
template <int DK, int DV, int NB>
__device__ __forceinline__ void put_block_bnd(float* __restrict__ dst, const ChainLds<DK, NB>& sm, int col0) {
  for (int idx = threadIdx.x; idx < DK * NB; idx += blockDim.x) {
    const int i = idx / NB, j = idx % NB;
    dst[bnd_index<DK>(i, col0 + j)] = sm.S[i][j];
  }
}

template <int DK, int DV, int NB>
__device__ __forceinline__ void get_block(ChainLds<DK, NB>& sm, const float* __restrict__ src, int col0) {
  for (int idx = threadIdx.x; idx < DK * NB; idx += blockDim.x) {
    const int i = idx / NB, j = idx % NB;
    sm.S[i][j] = src ? src[(size_t)i * DV + col0 + j] : 0.f;
  }
  __syncthreads();
}

template <int DK, int DV>
__global__ __launch_bounds__(256) void k_chain_prefill(const PrefillArgs a) {
  constexpr int NB = kChainCols;
  __shared__ ChainLds<DK, NB> sm;
  const int i = blockIdx.x, h = blockIdx.y, col0 = blockIdx.z * NB;
  const int H = a.H;
  const int L = a.end[i] - a.start[i];
  if (a.skip_empty && L == 0) return;
  const int Cl = a.Cl;
  const int nfull = L / Cl, nall = (L + Cl - 1) / Cl;
  const size_t sh = (size_t)i * H + h;
  const size_t SS = (size_t)DK * DV;
  const size_t ch = cache_row(a.slot, i) * H + h;
  get_block<DK, DV, NB>(sm, a.h0 ? a.h0 + (a.h0_slotted ? ch : sh) * SS : nullptr, col0);
  const int abase = a.all_base[i], fbase = a.full_base[i];
  if (nall > 0) put_block_bnd<DK, DV, NB>(a.bnd + ((size_t)abase * H + h) * SS, sm, col0);
  for (int c = 0; c < nfull; ++c) {
    const size_t slot = (size_t)(fbase + c) * H + h;
    stage_products<DK, DV, NB>(sm, (const float*)(a.prod + slot * prod_slot_bytes(false, DK, DV)), a.gamn + slot,
                               col0);
    chain_step_f32<DK, NB>(sm);
    if (c + 1 < nall) put_block_bnd<DK, DV, NB>(a.bnd + ((size_t)(abase + c + 1) * H + h) * SS, sm, col0);
  }
  put_block<DK, DV, NB>(a.s_bnd + ch * SS, sm, col0);
  if (L % Cl == 0) {
    put_block<DK, DV, NB>(a.s_run + ch * SS, sm, col0);
    if (a.hT) put_block<DK, DV, NB>(a.hT + sh * SS, sm, col0);
  }
  if (blockIdx.z == 0 && threadIdx.x == 0) {
    a.tail_len[ch] = L % Cl;
    if (L % Cl == 0 && a.lgs) a.lgs[ch] = 0.f;
  }
}

template <int DK, int DV>
__global__ __launch_bounds__(256) void k_chain_resync(const DecodeArgs a) {
  constexpr int NB = kChainCols;
  __shared__ ChainLds<DK, NB> sm;
  const int i = a.seq0 + blockIdx.x;
  const size_t sh = (size_t)i * a.H + blockIdx.y;
  if (a.flag[sh] == 0) return;
  const size_t ps = (size_t)blockIdx.x * a.H + blockIdx.y;  // product slot
  const int col0 = blockIdx.z * NB;
  const size_t SS = (size_t)DK * DV;
  const size_t ch = cache_row(a.slot, i) * a.H + blockIdx.y;
  get_block<DK, DV, NB>(sm, a.s_bnd + ch * SS, col0);
  stage_products<DK, DV, NB>(sm, (const float*)(a.prod + ps * prod_slot_bytes(false, DK, DV)), a.gamn + ps, col0);
  chain_step_f32<DK, NB>(sm);
  put_block<DK, DV, NB>(a.s_bnd + ch * SS, sm, col0);
  put_block<DK, DV, NB>(a.s_run + ch * SS, sm, col0);
  if (a.hT && (a.flag[sh] & 2)) put_block<DK, DV, NB>(a.hT + sh * SS, sm, col0);
  if (blockIdx.z == 0 && threadIdx.x == 0 && a.lgs) a.lgs[ch] = 0.f;
}

// bf16 path: one work-group per (sequence, head, block of CB = WAVES * NT * 16
// state columns); each wave keeps NT 16-column tiles of the state in MFMA
// accumulator tiles for the whole chain.  A chunk's WF / KF fragments (shared
// by the work-group) and the U tiles of its columns go through a two-buffer
// LDS stage; the loads run two chunks ahead in registers, so each step only
// waits on loads issued a full step earlier.  The column split is bit-neutral
// (every state column's arithmetic depends only on that column), so the
// launch picks WAVES and NT by the number of (sequence, head) pairs.
template <int DK, int DV, int WAVES, int NT>
__global__ __launch_bounds__(WAVES * 64) void k_chain_prefill_bf16(const PrefillArgs a) {
  using namespace mfma;
  typedef SlotB<DK, DV> Sl;
  constexpr int kThreads = WAVES * 64;
  constexpr int CB = WAVES * NT * 16;
  constexpr int kFragPieces = (int)(Sl::oU / 16);  // WF + KF, 16-byte pieces
  constexpr int kUPieces = C * CB * 4 / 16;        // U tiles of this block's columns
  constexpr int kPieces = kFragPieces + kUPieces;
  constexpr int kPer = kPieces / kThreads;
  constexpr int kPerFrag = kFragPieces / kThreads;
  static_assert(kPieces % kThreads == 0 && kFragPieces % kThreads == 0, "staging split");
  static_assert(DV % CB == 0, "column blocks tile d_v");
  __shared__ u32x4 stage[2][kPieces];
  const int i = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int jbg = blockIdx.z * (CB / 16), jb0 = jbg + wave * NT;
  const int H = a.H;
  const int L = a.end[i] - a.start[i];
  if (a.skip_empty && L == 0) return;
  const int Cl = a.Cl;
  int nfull = L / Cl;
  const int nall = (L + Cl - 1) / Cl;
  const size_t sh = (size_t)i * H + h;
  const size_t SS = (size_t)DK * DV;
  const int abase = a.all_base[i];
  const int fbase = a.all_chunks ? abase : a.full_base[i];
  if (a.all_chunks) nfull = nall;
  auto slot_of = [&](int c) { return a.prod + ((size_t)(fbase + c) * H + h) * Sl::bytes; };
  auto gamn_of = [&](int c) { return a.gamn[(size_t)(fbase + c) * H + h]; };
  // piece p of chunk c: WF/KF piece p, or U piece p - kFragPieces of this block's tiles
  auto fetch = [&](int c, u32x4 (&r)[kPer]) {
    const uint8_t* s = slot_of(c);
    const u32x4* f = reinterpret_cast<const u32x4*>(s);
    const u32x4* u = reinterpret_cast<const u32x4*>(s + Sl::oU) + (size_t)jbg * (C / 16) * 64;
#pragma unroll
    for (int m = 0; m < kPer; ++m) {
      const int p = tid + m * kThreads;
      r[m] = m < kPerFrag ? f[p] : u[p - kFragPieces];
    }
  };
  auto put = [&](int buf, const u32x4 (&r)[kPer]) {
#pragma unroll
    for (int m = 0; m < kPer; ++m) stage[buf][tid + m * kThreads] = r[m];
  };
  auto barrier = [] { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };

  f32x4 S[DK / 16][NT];
  const size_t ch = cache_row(a.slot, i) * H + h;
  load_state_tiles<DK, DV, NT>(S, a.h0 ? a.h0 + (a.h0_slotted ? ch : sh) * SS : nullptr, jb0, lane);
  if (nall > 0) store_bnd_tiles<DK, NT>(a.bnd + ((size_t)abase * H + h) * SS, S, jb0, lane);
  // Gamma_n travels with its chunk: every thread loads it, thread 0 stages it
  __shared__ float gn_stage[2];
  u32x4 R0[kPer], R1[kPer];
  float G0 = 1.f, G1 = 1.f;
  if (nfull > 0) {
    fetch(0, R0);
    G0 = gamn_of(0);
    put(0, R0);
    if (tid == 0) gn_stage[0] = G0;
    const int c1 = min(1, nfull - 1);
    fetch(c1, R1);
    G1 = gamn_of(c1);
  }
  __syncthreads();
  // Step c: chunk c is in stage buffer P = c & 1; its registers RP are free
  // and receive chunk c + 2 (clamped: the loads stay unconditional, so the
  // compiler's wait counts cover exactly the loads a put needs); chunk c + 1
  // sits in the other registers RQ and goes to the other buffer.  All steps
  // but the last store their boundary unconditionally, for the same reason.
  auto step = [&](auto par, auto is_last, int c) {
    constexpr int P = decltype(par)::value;
    constexpr bool kLast = decltype(is_last)::value;
    u32x4(&RP)[kPer] = P ? R1 : R0;
    u32x4(&RQ)[kPer] = P ? R0 : R1;
    float& GP = P ? G1 : G0;
    float& GQ = P ? G0 : G1;
    if constexpr (!kLast) {
      const int cf = min(c + 2, nfull - 1);
      fetch(cf, RP);
      GP = gamn_of(cf);
    }
    const u32x4* st = stage[P];
    const float gn = gn_stage[P];
    f32x4 Ut[C / 16][NT];
#pragma unroll
    for (int tm = 0; tm < C / 16; ++tm)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        Ut[tm][nt] = __builtin_bit_cast(f32x4, st[kFragPieces + ((wave * NT + nt) * (C / 16) + tm) * 64 + lane]);
    chain_step_bf16<DK, NT>(
        S, [&](int kb, int tm) { return st[(kb * (C / 16) + tm) * 64 + lane]; },
        [&](int kb, int im) { return st[(int)(Sl::oKF / 16) + (kb * (DK / 16) + im) * 64 + lane]; }, Ut, gn);
    float* bnd_next = a.bnd + ((size_t)(abase + c + 1) * H + h) * SS;
    if constexpr (kLast) {
      if (c + 1 < nall) store_bnd_tiles<DK, NT>(bnd_next, S, jb0, lane);
    } else {
      store_bnd_tiles<DK, NT>(bnd_next, S, jb0, lane);
      put(P ^ 1, RQ);
      if (tid == 0) gn_stage[P ^ 1] = GQ;
      barrier();
    }
  };
  typedef std::integral_constant<int, 0> P0;
  typedef std::integral_constant<int, 1> P1;
  typedef std::integral_constant<bool, false> Mid;
  typedef std::integral_constant<bool, true> Last;
  int c = 0;
  for (; c + 2 < nfull; c += 2) {
    step(P0{}, Mid{}, c);
    step(P1{}, Mid{}, c + 1);
  }
  if (c + 1 < nfull) {
    step(P0{}, Mid{}, c);
    step(P1{}, Last{}, c + 1);
  } else if (c < nfull) {
    step(P0{}, Last{}, c);
  }
  store_state_tiles<DK, DV, NT>(a.s_bnd + ch * SS, S, jb0, lane);
  if (a.all_chunks) return;
  if (L % Cl == 0) {
    store_state_tiles<DK, DV, NT>(a.s_run + ch * SS, S, jb0, lane);
    if (a.hT) store_state_tiles<DK, DV, NT>(a.hT + sh * SS, S, jb0, lane);
  }
  if (blockIdx.z == 0 && tid == 0) {
    a.tail_len[ch] = L % Cl;
    if (L % Cl == 0 && a.lgs) a.lgs[ch] = 0.f;
  }
}

// chain step of a filled tail, bf16 path, from a product slot the decode
// workspace already holds (the chunkwise-everywhere comparator's decode):
// one wave per (sequence, head, 32 state columns), the waves of a (sequence,
// head) in one work-group
constexpr int kResyncNT = 2;
template <int DV>
constexpr int kResyncWaves = DV / (16 * kResyncNT) < 4 ? DV / (16 * kResyncNT) : 4;

template <int DK, int DV>
__global__ __launch_bounds__(kResyncWaves<DV> * 64) void k_chain_resync_bf16(const DecodeArgs a) {
  constexpr int NT = kResyncNT;
  const size_t sh = (size_t)blockIdx.x * a.H + blockIdx.y;
  if (a.flag[sh] == 0) return;
  const int lane = threadIdx.x & 63;
  const int jb0 = (blockIdx.z * kResyncWaves<DV> + (threadIdx.x >> 6)) * NT;
  const size_t SS = (size_t)DK * DV;
  mfma::f32x4 S[DK / 16][NT];
  const size_t ch = cache_row(a.slot, blockIdx.x) * a.H + blockIdx.y;
  load_state_tiles<DK, DV, NT>(S, a.s_bnd + ch * SS, jb0, lane);
  chain_step_bf16_global<DK, DV, NT>(S, a.prod + sh * prod_slot_bytes(true, DK, DV), a.gamn[sh], jb0, lane);
  store_state_tiles<DK, DV, NT>(a.s_bnd + ch * SS, S, jb0, lane);
  store_state_tiles<DK, DV, NT>(a.s_run + ch * SS, S, jb0, lane);
  if (blockIdx.z == 0 && threadIdx.x == 0 && a.lgs) a.lgs[ch] = 0.f;
}

// decode resync, bf16 path, in one launch: one work-group per (sequence,
// head).  A pair whose tail filled forms the tail's chunk products into the
// decode workspace's product slot (as the prefill's chunk-product kernel
// does for a chunk) and then, wave w for state columns 32 w .. 32 w + 31,
// takes the chain step from s_bnd with them (k_chain_resync_bf16's
// arithmetic); every other pair exits at once, so a step in which no tail
// fills costs one launch of early-exit work-groups.  The grid covers
// sequences seq0 .. seq0 + gridDim.x - 1 of the batch (all of them, except
// in the fixed-scratch decode, which resynchronises the batch in groups);
// product slots are indexed within the grid.
template <int DK, int DV>
__global__ __launch_bounds__(256, DK > 128 ? 1 : 3) void k_resync_bf16(const DecodeArgs a) {
  // 32 columns per wave pass (16 at d_k = 256, where a 16-column block's
  // state is already 64 accumulator registers); four waves take the passes
  constexpr int NT = DK > 128 ? 1 : kResyncNT, NW = DV / (16 * NT);
  __shared__ ChunkLdsB<DK, DV> sm;
  const int i = a.seq0 + blockIdx.x;
  const size_t sh = (size_t)i * a.H + blockIdx.y;
  const int flag = a.flag[sh];
  if (flag == 0) return;
  const size_t ps = (size_t)blockIdx.x * a.H + blockIdx.y;  // product slot
  const size_t ch = cache_row(a.slot, i) * a.H + blockIdx.y;
  const size_t tr = ch * a.Cl;
  uint8_t* const prod = a.prod + ps * prod_slot_bytes(true, DK, DV);
  stage_chunk_bf16<DK, DV>(sm, (const uint16_t*)a.tail_k, tr, 1, (const uint16_t*)a.tail_v, tr, 1,
                           (const uint16_t*)a.tail_g, (const uint16_t*)a.tail_beta, tr, 1, a.Cl);
  chunk_local_bf16<DK, DV>(sm, prod, a.gamn + ps);
  __syncthreads();  // the slot and Gamma_n, written by every wave, are read below
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  auto pass = [&](int jw) {
    const int jb0 = jw * NT;
    const size_t SS = (size_t)DK * DV;
    mfma::f32x4 S[DK / 16][NT];
    load_state_tiles<DK, DV, NT>(S, a.s_bnd + ch * SS, jb0, lane);
    chain_step_bf16_global<DK, DV, NT>(S, prod, a.gamn[ps], jb0, lane);
    store_state_tiles<DK, DV, NT>(a.s_bnd + ch * SS, S, jb0, lane);
    store_state_tiles<DK, DV, NT>(a.s_run + ch * SS, S, jb0, lane);
    if (a.hT && (flag & 2)) store_state_tiles<DK, DV, NT>(a.hT + sh * SS, S, jb0, lane);
  };
  if constexpr (NW <= 4) {
    if (wave < NW) pass(wave);
  } else {
#pragma unroll 1
    for (int jw = wave; jw < NW; jw += 4) pass(jw);
  }
  if (threadIdx.x == 0 && a.lgs) a.lgs[ch] = 0.f;
}

// ---------------------------------------------------------------------------
// in-chunk scan (prefill): one wave per (chunk, head, 64 state columns; 32
// at d_k = 256)

// One scan unit: chunk slot `slot` (chunk c of sequence i), head h, state
// columns WC z .. WC z + WC - 1 (one wave; WC = KeySplit<DK>::kCols; lane =
// column, and at d_k = 256 lanes j and j + 32 the two key halves of column
// j).  kAgentBnd: the boundary state is read with agent-scope loads, because
// the boundary chain wrote it during the same launch (k_chain_scan_bf16).
template <class D, int DK, int DV, bool kAgentBnd>
__device__ __forceinline__ void scan_unit(const PrefillArgs& a, int slot, int i, int h, int z, int lane) {
  using T = typename D::T;
  constexpr int KL = KeySplit<DK>::kKeys, WC = KeySplit<DK>::kCols;
  const int H = a.H;
  const int c = slot - a.all_base[i];
  const int L = a.end[i] - a.start[i];
  const int Cl = a.Cl;
  const int n = min(Cl, L - c * Cl);
  const size_t tok0 = (size_t)a.start[i] + (size_t)c * Cl;
  const int col = z * WC + lane % WC;
  const int k0 = (lane / WC) * KL;  // this lane's first key row
  const size_t SS = (size_t)DK * DV;

  const float* B = a.bnd + ((size_t)slot * H + h) * SS;
  float s[KL];
  {
    // rows 4q .. 4q+3 of column col sit 256 q bytes after rows 0 .. 3
    static_assert(bnd_index<DK>(4, 0) == 64 && bnd_index<DK>(16, 0) == 256, "row groups 256 bytes apart");
    const BufRsrc rb = buf_rsrc(B, (uint32_t)(SS * sizeof(float)));
    const uint32_t col_off = (uint32_t)(bnd_index<DK>(k0, col) * 4);
#pragma unroll
    for (int q = 0; q < KL / 4; ++q) {  // rows k0 + 4q .. k0 + 4q+3 of column col: one 16-byte load
      const mfma::f32x4 x = __builtin_bit_cast(
          mfma::f32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, col_off, 256 * q, kAgentBnd ? kAuxAgent : 0));
      s[4 * q] = x[0];
      s[4 * q + 1] = x[1];
      s[4 * q + 2] = x[2];
      s[4 * q + 3] = x[3];
    }
  }

  const T* gp = (const T*)a.g;
  const T* bp = (const T*)a.beta;
  float g_l = 0.f, beta_l = 0.f;
  if (lane < n) {
    const size_t r = (tok0 + lane) * H + h;
    g_l = D::load(gp, r);
    beta_l = D::load(bp, r);
  }
  // the scale steps of the chunk's tokens in token order from the boundary
  // (lg = 0), lane t keeping token t's; then every lane takes its token's
  // step scalars (the same helpers as the decode step)
  float lg = 0.f;
  TokenScale ts_l{0.f, false};
  for (int t = 0; t < n; ++t) {
    const TokenScale ts = token_scale(lg, lane_bcast(g_l, t));
    if (lane == t) ts_l = ts;
    lg = scale_after(ts);
  }
  float c_l, b_l;
  step_factors(ts_l, beta_l, c_l, b_l);
  const uint64_t renorm = __ballot(ts_l.renorm && lane < n);
  const T* kp = (const T*)a.k;
  const T* qp = (const T*)a.q;
  const T* vp = (const T*)a.v;
  scan_tokens<D, DK, DV>(s, kp, qp, vp, (T*)a.o, tok0 * H + h, H, kq_row(tok0, h, a.Hk, a.G), a.Hk, n, col, lane,
                         c_l, b_l, renorm);
  const int nall = (L + Cl - 1) / Cl;
  if (c == nall - 1 && (L % Cl) != 0) {
    // last, partial chunk: its end state is the running state (N with
    // log-scale lg), its tokens the tail
    const size_t ch = cache_row(a.slot, i) * H + h;
    float* R = a.s_run + ch * SS;
    store_state_col<KL, DV>(R, (uint32_t)(SS * 4), s, k0, col, 1.f);
    if (z == 0 && lane == 0 && a.lgs) a.lgs[ch] = lg;
    if (a.hT)  // the state itself, exp(lg) N (gdn_cpr_cache_state's product)
      store_state_col<KL, DV>(a.hT + ((size_t)i * H + h) * SS, (uint32_t)(SS * 4), s, k0, col, scale_of_log(lg));
    T* tv = (T*)a.tail_v + ch * Cl * DV;
    if (lane < WC)
      for (int t = 0; t < n; ++t) tv[(size_t)t * DV + col] = vp[((tok0 + t) * H + h) * DV + col];
    if (z == 0) {
      T* tk = (T*)a.tail_k + ch * Cl * DK;
      for (int idx = lane; idx < n * DK; idx += kWave) {
        const int t = idx / DK, e = idx % DK;
        tk[idx] = kp[kq_row(tok0 + t, h, a.Hk, a.G) * DK + e];
      }
      if (lane < n) {
        ((T*)a.tail_g)[ch * Cl + lane] = gp[(tok0 + lane) * H + h];
        ((T*)a.tail_beta)[ch * Cl + lane] = bp[(tok0 + lane) * H + h];
      }
    }
  }
}

template <class D, int DK, int DV>
__global__ __launch_bounds__(64, 3) void k_scan(const PrefillArgs a) {
  const int slot = blockIdx.x;
  if (slot >= a.all_base[a.N]) return;
  scan_unit<D, DK, DV, false>(a, slot, find_seq(a.all_base, a.N, slot), blockIdx.y, blockIdx.z, threadIdx.x);
}

// ---------------------------------------------------------------------------
// chunk products, boundary chain and in-chunk scan in one launch (bf16 inputs)
//
// The chain step of chunk c needs only chunk c's products, and the scan of
// chunk c only the boundary B_c, so each can start as soon as its input is
// in memory instead of after the whole stage before it.  Every work-group
// takes a ticket from an atomic counter when it starts, so ticket order is
// start order.  Tickets 0 .. n_cp-1 are chunk-product items, one per (chunk
// slot in chunk-major order, head; partial chunks have none), which publish
// a flag once their product slot has reached memory.  The next n_chain
// tickets are chain items, one per (sequence, head, 64-column block): the
// chain of k_chain_prefill_bf16 with 4 waves x 16 columns and a one-buffer
// LDS stage, which waits for each chunk's flag before loading its products
// and publishes, after each step, how many boundaries of its columns have
// reached memory.  Later tickets are scan items: 4 waves, each one (chunk,
// head, 64-column half) unit, units in chunk-major order, each waiting until
// its chain item has published its boundary.  Every item waits only on items
// with lower tickets, which started before it and never wait on it, so every
// wait ends; the waits are bounded all the same.  Products and boundaries
// travel with agent-scope stores and loads (coherent across the XCDs, no
// cache-wide maintenance); a flag or count is published only after the
// stores are complete.  No value depends on the order in which items run.
struct FusedArgs {
  const int32_t* order;  // [A] chunk slots, chunk-major
  int32_t* ticket;       // zeroed by the plan kernel
  int32_t* ready;        // [N * H * NZ * kReadyStride] boundaries published per chain item (one per
                         // kReadyStride words), zeroed by the plan kernel
  int32_t* cp_ready;     // [F * H] 1 once a (full chunk, head)'s products are in memory (zeroed by the
                         // plan kernel), or null: the products come from an earlier launch
  int32_t* timeout;      // set to 1 if a wait ever gives up (never expected)
  int32_t n_cp;          // chunk-product items (tickets 0 .. n_cp - 1)
  int32_t n_chain;       // chain items (the next n_chain tickets)
};

constexpr int kFusedChainCols = 64;  // state columns per chain item (= per scan unit)
// each chain item's count sits on a cache line of its own: thousands of
// waiting waves poll the counts, and packed counts would send all those polls
// to a handful of lines (one memory channel), which then slows the chain's
// own traffic
constexpr int kReadyStride = 32;  // int32 words

__device__ __forceinline__ void publish_count(int32_t* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ int read_count(const int32_t* p) {
  return __hip_atomic_load(const_cast<int32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Test hook: a positive value replaces the waits' poll bound (so that a test
// can make them give up while every work-group still exits); 0, the
// default, keeps it.  Set by gdn_cpr_debug_set_wait_polls.
__device__ int32_t g_wait_polls = 0;

// waits (bounded) until *p >= need; false if it gave up.  The default polls
// every ~8,000 cycles (3 to 4 us; a chain step takes about as long), so that
// thousands of waiting scan waves add little memory traffic; the chain's wait
// for chunk products (a few waves, on its critical path) polls every ~200
// cycles.  Either way the bound is about a second.
template <int kSleep = 127>
__device__ __forceinline__ bool wait_count(const int32_t* p, int need) {
  constexpr int kMaxPolls = kSleep >= 127 ? 1 << 18 : 1 << 21;
  if (__builtin_amdgcn_readfirstlane(read_count(p)) >= need) return true;  // no wait: no further load
  const int32_t over = g_wait_polls;
  const int polls = over > 0 ? min((int)over, kMaxPolls) : kMaxPolls;
  for (int it = 1; it < polls; ++it) {
    __builtin_amdgcn_s_sleep(kSleep);
    if (__builtin_amdgcn_readfirstlane(read_count(p)) >= need) return true;
  }
  return false;
}

template <int DK, int DV>
__global__ __launch_bounds__(256, DK > 128 ? 2 : 3) void k_chain_scan_bf16(const PrefillArgs a, const FusedArgs f) {
  using namespace mfma;
  typedef SlotB<DK, DV> Sl;
  constexpr int kThreads = 256, CB = kFusedChainCols, NZ = DV / CB;
  constexpr int kFragPieces = (int)(Sl::oU / 16);  // WF + KF, 16-byte pieces
  constexpr int kUPieces = C * CB * 4 / 16;        // U tiles of this item's columns
  constexpr int kPieces = kFragPieces + kUPieces;
  constexpr int kPer = kPieces / kThreads;
  constexpr int kPerFrag = kFragPieces / kThreads;
  static_assert(kPieces % kThreads == 0 && kFragPieces % kThreads == 0, "staging split");
  static_assert(DV % CB == 0, "column blocks tile d_v");
  // one LDS block: a chain item's stage or a chunk-product item's arrays (at
  // d_k = 256 the launch has chain items only)
  constexpr bool kCP = KeySplit<DK>::kParts == 1;
  constexpr size_t kStageBytes = (size_t)kPieces * 16, kCpBytes = kCP ? sizeof(ChunkLdsB<DK, DV>) : 0;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kStageBytes > kCpBytes ? kStageBytes : kCpBytes];
  u32x4* const stage = reinterpret_cast<u32x4*>(lds);
  __shared__ float gn_stage;
  __shared__ int32_t ticket_s;
  // the ticket and the wave index are uniform over each wave: reading them
  // into scalar registers keeps every index derived from them scalar
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (tid == 0) ticket_s = atomicAdd(f.ticket, 1);
  __syncthreads();
  const int t = __builtin_amdgcn_readfirstlane(ticket_s);
  const int H = a.H;
  if (t < f.n_cp) {
    // ---- chunk-product item: full chunk slot order[t / H], head t % H
    if constexpr (kCP) {
      const int pos = t / H, h = t % H;
      if (pos >= a.all_base[a.N]) return;
      const int slot = f.order[pos];
      if (slot < 0 || slot >= a.all_base[a.N]) return;  // (the plan writes every position in range)
      const int i = find_seq(a.all_base, a.N, slot);
      const int c = slot - a.all_base[i];
      if (c >= (a.end[i] - a.start[i]) / a.Cl) return;  // a partial chunk has no products
      const size_t tok0 = (size_t)a.start[i] + (size_t)c * a.Cl;
      const size_t row0 = tok0 * H + h;
      ChunkLdsB<DK, DV>& sm = *reinterpret_cast<ChunkLdsB<DK, DV>*>(lds);
      stage_chunk_bf16<DK, DV>(sm, (const uint16_t*)a.k, kq_row(tok0, h, a.Hk, a.G), a.Hk, (const uint16_t*)a.v,
                               row0, H, (const uint16_t*)a.g, (const uint16_t*)a.beta, row0, H, a.Cl);
      const size_t ps = (size_t)(a.full_base[i] + c) * H + h;
      chunk_local_bf16<DK, DV, kAuxAgent>(sm, a.prod + ps * Sl::bytes, a.gamn + ps);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's slot stores are complete
      __syncthreads();                                  // and every wave's
      if (tid == 0) publish_count(f.cp_ready + ps, 1);
    }
    return;
  }
  if (t >= f.n_cp + f.n_chain) {
    // ---- scan item: one unit per wave (launches at d_k = 256 have chain items only)
    if constexpr (KeySplit<DK>::kParts == 1) {
      const long u = (long)(t - f.n_cp - f.n_chain) * 4 + wave;
      const long per_slot = (long)H * NZ;
      if (u >= (long)a.all_base[a.N] * per_slot) return;
      const int pos = (int)(u / per_slot), r = (int)(u % per_slot), h = r / NZ, z = r % NZ;
      const int slot = f.order[pos];
      if (slot < 0 || slot >= a.all_base[a.N]) return;  // (the plan writes every position in range)
      const int i = find_seq(a.all_base, a.N, slot);
      const int c = slot - a.all_base[i];
      if (!wait_count(f.ready + (((size_t)i * H + h) * NZ + z) * kReadyStride, c + 1) && lane == 0)
        atomicExch(f.timeout, 1);
      scan_unit<Bf16, DK, DV, true>(a, slot, i, h, z, lane);
    }
    return;
  }
  // ---- chain item
  const int tc = t - f.n_cp;
  const int i = tc / (H * NZ), r = tc % (H * NZ), h = r / NZ, z = r % NZ;
  const int jbg = z * (CB / 16), jb0 = jbg + wave;  // one 16-column tile per wave
  const int L = a.end[i] - a.start[i];
  if (a.skip_empty && L == 0) return;
  const int Cl = a.Cl;
  const int nfull = L / Cl, nall = (L + Cl - 1) / Cl;
  const size_t sh = (size_t)i * H + h;
  const size_t SS = (size_t)DK * DV;
  const int abase = a.all_base[i], fbase = a.full_base[i];
  int32_t* const rdy = f.ready + (sh * NZ + z) * kReadyStride;
  auto slot_of = [&](int c) { return a.prod + ((size_t)(fbase + c) * H + h) * Sl::bytes; };
  // chunk c's products, once its chunk-product item has published them; read
  // at agent scope, since that item may have run on another XCD
  auto gamn_of = [&](int c) {
    return __hip_atomic_load(a.gamn + (size_t)(fbase + c) * H + h, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  auto fetch = [&](int c, u32x4 (&rg)[kPer]) {
    if (f.cp_ready && !wait_count<2>(f.cp_ready + (size_t)(fbase + c) * H + h, 1) && lane == 0)
      atomicExch(f.timeout, 1);
    const BufRsrc sr = buf_rsrc(slot_of(c), (uint32_t)Sl::bytes);
    const uint32_t u0 = (uint32_t)(Sl::oU + (size_t)jbg * (C / 16) * 64 * 16);
#pragma unroll
    for (int m = 0; m < kPer; ++m) {
      const int p = tid + m * kThreads;
      const uint32_t off = m < kPerFrag ? (uint32_t)p * 16u : u0 + (uint32_t)(p - kFragPieces) * 16u;
      rg[m] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(sr, off, 0, kAuxAgent));
    }
  };
  f32x4 S[DK / 16][1];
  const size_t ch = cache_row(a.slot, i) * H + h;
  load_state_tiles<DK, DV, 1>(S, a.h0 ? a.h0 + (a.h0_slotted ? ch : sh) * SS : nullptr, jb0, lane);
  // boundary c of this wave's tile, agent scope (bnd_index layout)
  auto store_bnd = [&](int c) {
    const BufRsrc rb = buf_rsrc(a.bnd + ((size_t)(abase + c) * H + h) * SS, (uint32_t)(SS * sizeof(float)));
#pragma unroll
    for (int im = 0; im < DK / 16; ++im)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, S[im][0]), rb,
                                             (uint32_t)(((jb0 * (DK / 16) + im) * 64 + lane) * 16), 0, kAuxAgent);
  };
  auto all_stores_done = [] { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };
  if (nall > 0) store_bnd(0);
  u32x4 R[kPer];
  float G = 1.f;
  if (nfull > 0) {
    fetch(0, R);
    G = gamn_of(0);
  }
  all_stores_done();
  if (nfull > 0) {
    for (int m = 0; m < kPer; ++m) stage[tid + m * kThreads] = R[m];
    if (tid == 0) gn_stage = G;
    const int c1 = min(1, nfull - 1);
    fetch(c1, R);
    G = gamn_of(c1);
  }
  __syncthreads();
  if (tid == 0 && nall > 0) publish_count(rdy, 1);
  // Step c: the stage holds chunk c's products, R chunk c+1's.  After the
  // step's products every wave waits for its outstanding memory operations
  // (the boundary B_c stored and the fetch issued one step earlier), so once
  // all waves are past the barrier B_0 .. B_c are complete and published.
  for (int c = 0; c < nfull; ++c) {
    f32x4 Ut[C / 16][1];
#pragma unroll
    for (int tm = 0; tm < C / 16; ++tm)
      Ut[tm][0] = __builtin_bit_cast(f32x4, stage[kFragPieces + (wave * (C / 16) + tm) * 64 + lane]);
    chain_step_bf16<DK, 1>(
        S, [&](int kb, int tm) { return stage[(kb * (C / 16) + tm) * 64 + lane]; },
        [&](int kb, int im) { return stage[(int)(Sl::oKF / 16) + (kb * (DK / 16) + im) * 64 + lane]; }, Ut,
        gn_stage);
    all_stores_done();
    __syncthreads();  // every wave is done with the stage; B_c is complete
    if (tid == 0) publish_count(rdy, c + 1);
    if (c + 1 < nall) store_bnd(c + 1);
    if (c + 1 < nfull) {
#pragma unroll
      for (int m = 0; m < kPer; ++m) stage[tid + m * kThreads] = R[m];
      if (tid == 0) gn_stage = G;
      const int cf = min(c + 2, nfull - 1);
      fetch(cf, R);
      G = gamn_of(cf);
    }
    __syncthreads();  // the stage holds chunk c+1
  }
  all_stores_done();
  __syncthreads();
  if (tid == 0 && nall > 0) publish_count(rdy, nall);
  store_state_tiles<DK, DV, 1>(a.s_bnd + ch * SS, S, jb0, lane);
  if (L % Cl == 0) {
    store_state_tiles<DK, DV, 1>(a.s_run + ch * SS, S, jb0, lane);
    if (a.hT) store_state_tiles<DK, DV, 1>(a.hT + sh * SS, S, jb0, lane);
  }
  if (z == 0 && tid == 0) {
    a.tail_len[ch] = L % Cl;
    if (L % Cl == 0 && a.lgs) a.lgs[ch] = 0.f;
  }
}


}  // namespace
