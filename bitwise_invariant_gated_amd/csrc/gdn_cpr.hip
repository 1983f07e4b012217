// CPR Gated DeltaNet layer: HIP kernels for gfx950 and the C ABI (gdn_cpr.h).
//
// Prefill (per call, all on the caller's stream):
//   k_plan            per-sequence chunk counts -> prefix sums (varlen plan)
//   k_chunk_local     chunk products of every full chunk, all in parallel
//   k_chain           boundary states: sequential over each sequence's full
//                     chunks, parallel over sequences x heads x column blocks
//   k_scan            per-token recurrence inside every chunk, all chunks in
//                     parallel, each from its boundary state; writes o, the
//                     final state and the decode tail
// Decode step:
//   k_decode          per-token step on the running state (one work item per
//                     sequence x head), tail append, resync flag
//   k_resync_bf16 (bf16; fp32: k_chunk_local_resync, k_chain_resync)
//                     for the (sequence, head) pairs whose tail just filled:
//                     the same chunk products and boundary advance as prefill
//                     over the C tail tokens, from the boundary state
// The structure follows the pages (IsoExec, "Chunkwise-Parallel Recurrent
// (CPR) Gated DeltaNet"; Chinese page, third-way section): boundary states
// first, then a parallel in-chunk recurrent scan; decode resynchronises every
// C tokens.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <type_traits>

#include "../../include/gdn_cpr.h"
#include "cpr_backward.hpp"
#include "cpr_backward_bf16.hpp"
#include "cpr_device.hpp"

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
  int32_t* ticket;  // work-item counter of the fused launch
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

// waits (bounded) until *p >= need; false if it gave up.  The default polls
// every ~8,000 cycles (3 to 4 us; a chain step takes about as long), so that
// thousands of waiting scan waves add little memory traffic; the chain's wait
// for chunk products (a few waves, on its critical path) polls every ~200
// cycles.  Either way the bound is about a second.
template <int kSleep = 127>
__device__ __forceinline__ bool wait_count(const int32_t* p, int need) {
  constexpr int kMaxPolls = kSleep >= 127 ? 1 << 18 : 1 << 21;
  for (int it = 0; it < kMaxPolls; ++it) {
    if (__builtin_amdgcn_readfirstlane(read_count(p)) >= need) return true;
    __builtin_amdgcn_s_sleep(kSleep);
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

// ---------------------------------------------------------------------------
// decode: one work-group per (sequence, head); a thread per state column (two
// per column at d_k = 256, one per key half: ColumnLanes)

// Where thread `tid` of a work-group of DV * kParts threads sits: its state
// column, its first key row, and whether it writes the column's per-column
// outputs (the lower key half does).
template <int DK>
struct ColumnLanes {
  int lane, col, k0;
  bool writer;
  __device__ explicit ColumnLanes(int tid) {
    constexpr int WC = KeySplit<DK>::kCols;
    lane = tid & 63;
    col = (tid >> 6) * WC + lane % WC;
    k0 = (lane / WC) * KeySplit<DK>::kKeys;
    writer = lane < WC;
  }
};

template <int DK, int DV>
constexpr int kColumnThreads = DV * KeySplit<DK>::kParts;

template <class D, int DK, int DV>
__global__ __launch_bounds__(DV * KeySplit<DK>::kParts) void k_decode(const DecodeArgs a) {
  using T = typename D::T;
  constexpr int KL = KeySplit<DK>::kKeys, NTH = kColumnThreads<DK, DV>;
  const size_t sh = (size_t)blockIdx.x * a.H + blockIdx.y;
  const size_t ch = cache_row(a.slot, blockIdx.x) * a.H + blockIdx.y;
  const int tid = threadIdx.x;
  const ColumnLanes<DK> cl(tid);
  const int col = cl.col;
  const size_t SS = (size_t)DK * DV;
  const int tl = a.tail_len[ch];
  const float lg = a.lgs[ch];
  __syncthreads();  // every wave has read tail_len and lgs before they are rewritten below
  const int Cl = a.Cl;
  if ((unsigned)tl >= (unsigned)Cl) {  // not a valid cache: touch nothing
    if (tid == 0) a.flag[sh] = 0;
    return;
  }
  const T* kp = (const T*)a.k;
  const T* qp = (const T*)a.q;
  const size_t kr = kq_row(blockIdx.x, blockIdx.y, a.Hk, a.G);
  // the token's k, v, g, beta as stored, for the tail append at the end
  // (loaded here, before any store, so the append needs no second read)
  constexpr int KE = (DK + NTH - 1) / NTH;
  T k_app[KE];
#pragma unroll
  for (int m = 0; m < KE; ++m) k_app[m] = tid + m * NTH < DK ? kp[kr * DK + tid + m * NTH] : T();
  const T v_app = ((const T*)a.v)[sh * DV + col];
  const T g_app = ((const T*)a.g)[sh], b_app = ((const T*)a.beta)[sh];
  float* R = a.s_run + ch * SS;
  float s[KL];
  load_state_col<KL, DV>(s, R, (uint32_t)(SS * 4), cl.k0, col);
  float lg_next = lg;
  const float out = token_step_at<D, DK>(s, lg_next, kp + kr * DK, qp + kr * DK, D::load(&g_app, 0),
                                         D::load(&b_app, 0), D::load(&v_app, 0), cl.lane);
  if (cl.writer) D::store((T*)a.o, sh * DV + col, out);
  // append the token to the tail
  T* tk = (T*)a.tail_k + (ch * Cl + tl) * DK;
#pragma unroll
  for (int m = 0; m < KE; ++m)
    if (tid + m * NTH < DK) tk[tid + m * NTH] = k_app[m];
  if (cl.writer) ((T*)a.tail_v)[(ch * Cl + tl) * DV + col] = v_app;
  if (tid == 0) {
    ((T*)a.tail_g)[ch * Cl + tl] = g_app;
    ((T*)a.tail_beta)[ch * Cl + tl] = b_app;
  }
  const bool full = (tl + 1 == Cl);
  if (!full) {
    store_state_col<KL, DV>(R, (uint32_t)(SS * 4), s, cl.k0, col, 1.f);
    if (a.hT)  // the state itself, exp(lg) N (gdn_cpr_cache_state's product)
      store_state_col<KL, DV>(a.hT + sh * SS, (uint32_t)(SS * 4), s, cl.k0, col, scale_of_log(lg_next));
  }
  if (tid == 0) {
    a.tail_len[ch] = full ? 0 : tl + 1;
    a.lgs[ch] = full ? 0.f : lg_next;  // a full tail resynchronises to a boundary (scale 1)
    a.flag[sh] = full ? 3 : 0;         // the resync then also writes hT (if asked for)
  }
}

// ---------------------------------------------------------------------------
// the running state of every (sequence, head) from its scaled form:
// out = exp(lg) * s_run, row-major [d_k][d_v] (the same product the scan
// uses when it writes a final state itself)

__global__ __launch_bounds__(256) void k_cache_state(const float* __restrict__ s_run, const float* __restrict__ lgs,
                                                    const int32_t* __restrict__ slot, float* __restrict__ out,
                                                    int H, int SS4) {
  const size_t sh = (size_t)blockIdx.x * H + blockIdx.y;
  const size_t ch = cache_row(slot, blockIdx.x) * H + blockIdx.y;
  const float e = scale_of_log(lgs[ch]);
  const float4* src = reinterpret_cast<const float4*>(s_run) + ch * SS4;
  float4* dst = reinterpret_cast<float4*>(out) + sh * SS4;
  for (int i = threadIdx.x; i < SS4; i += 256) {
    const float4 x = src[i];
    dst[i] = make_float4(e * x.x, e * x.y, e * x.z, e * x.w);
  }
}

// ---------------------------------------------------------------------------
// prefill continued from a cache: the head of each sequence (the tokens that
// complete the cache's partial chunk) runs the decode step token by token;
// the resynchronisation kernels then close that chunk, and the rest of the
// sequence (which starts on a chunk boundary) goes through the prefill
// kernels from the new boundary state.

struct ContArgs {
  const int32_t* slot;  // [N] cache row of sequence i, or null (row i)
  const void* q;
  const void* k;
  const void* v;
  const void* g;
  const void* beta;
  const int32_t* cu;
  float* s_run;
  void* tail_k;
  void* tail_v;
  void* tail_g;
  void* tail_beta;
  int32_t* tail_len;
  float* lgs;  // [rows, H] log-scale of s_run
  float* hT;   // [N, H, DK, DV] final state (batch order), or null
  void* o;
  int32_t* flag;        // [N*H] as DecodeArgs::flag: bit 0 the head closes the chunk, bit 1 the resync writes hT
  int32_t* body_start;  // [N] first token row after the head
  int32_t N;
  int32_t H;
  int32_t Hk;  // heads of q and k
  int32_t G;   // value heads per key head, H / Hk
  int32_t Cl;  // chunk length
};

template <class D, int DK, int DV>
__global__ __launch_bounds__(DV * KeySplit<DK>::kParts) void k_cont_head(const ContArgs a) {
  using T = typename D::T;
  constexpr int KL = KeySplit<DK>::kKeys, NTH = kColumnThreads<DK, DV>;
  const int i = blockIdx.x, h = blockIdx.y, H = a.H;
  const size_t sh = (size_t)i * H + h;
  const size_t ch = cache_row(a.slot, i) * H + h;
  const int tid = threadIdx.x;
  const ColumnLanes<DK> cl(tid);
  const int col = cl.col;
  const size_t SS = (size_t)DK * DV;
  const int tl = a.tail_len[ch];
  float lg = a.lgs[ch];
  __syncthreads();  // every wave has read tail_len and lgs before they are rewritten below
  const int L = a.cu[i + 1] - a.cu[i];
  const int Cl = a.Cl;
  const int nh = ((unsigned)tl < (unsigned)Cl && tl > 0) ? min(Cl - tl, L) : 0;
  if (h == 0 && tid == 0) a.body_start[i] = a.cu[i] + nh;
  if (tid == 0) a.flag[sh] = 0;
  float* R = a.s_run + ch * SS;
  if (L == 0) {  // nothing new: the final state is the cached one
    if (a.hT) {
      float x[KL];
      load_state_col<KL, DV>(x, R, (uint32_t)(SS * 4), cl.k0, col);
      store_state_col<KL, DV>(a.hT + sh * SS, (uint32_t)(SS * 4), x, cl.k0, col, scale_of_log(lg));
    }
    return;
  }
  if (nh == 0) return;  // the body prefill writes the final state
  float s[KL];
  load_state_col<KL, DV>(s, R, (uint32_t)(SS * 4), cl.k0, col);
  const T* kp = (const T*)a.k;
  const T* qp = (const T*)a.q;
  const T* vp = (const T*)a.v;
  const T* gp = (const T*)a.g;
  const T* bp = (const T*)a.beta;
  constexpr int KE = (DK + NTH - 1) / NTH;
  for (int t = 0; t < nh; ++t) {
    const size_t row = (size_t)(a.cu[i] + t) * H + h;
    const size_t kr = kq_row((size_t)(a.cu[i] + t), h, a.Hk, a.G);
    // the token's k, v, g, beta as stored, for the tail append below (read
    // before the output store, so the append needs no second read)
    T k_app[KE];
#pragma unroll
    for (int m = 0; m < KE; ++m) k_app[m] = tid + m * NTH < DK ? kp[kr * DK + tid + m * NTH] : T();
    const T v_app = vp[row * DV + col], g_app = gp[row], b_app = bp[row];
    const float out = token_step_at<D, DK>(s, lg, kp + kr * DK, qp + kr * DK, D::load(&g_app, 0),
                                           D::load(&b_app, 0), D::load(&v_app, 0), cl.lane);
    if (cl.writer) D::store((T*)a.o, row * DV + col, out);
    const size_t tr = ch * Cl + tl + t;  // tail row
    T* tk = (T*)a.tail_k + tr * DK;
#pragma unroll
    for (int m = 0; m < KE; ++m)
      if (tid + m * NTH < DK) tk[tid + m * NTH] = k_app[m];
    if (cl.writer) ((T*)a.tail_v)[tr * DV + col] = v_app;
    if (tid == 0) {
      ((T*)a.tail_g)[tr] = g_app;
      ((T*)a.tail_beta)[tr] = b_app;
    }
  }
  const bool full = (tl + nh == Cl);
  if (!full) {
    store_state_col<KL, DV>(R, (uint32_t)(SS * 4), s, cl.k0, col, 1.f);
    if (a.hT)  // the head is the whole segment (nh == L): exp(lg) N is the final state
      store_state_col<KL, DV>(a.hT + sh * SS, (uint32_t)(SS * 4), s, cl.k0, col, scale_of_log(lg));
  }
  if (tid == 0) {
    a.tail_len[ch] = full ? 0 : tl + nh;
    a.lgs[ch] = full ? 0.f : lg;
    // a closed chunk resynchronises; with no body after it, that boundary is the final state
    a.flag[sh] = full ? (nh == L ? 3 : 1) : 0;
  }
}

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

template <int DK, int DV>
struct BwdLocalLds {
  float At[C][C + 1];  // At[s][t] = A[t][s]
  float X[C][C + 1];
  float Pt[C][C + 1];  // Pt[s][t] = P[t][s]
  float W[C][DK + 1];
  float Dd[C][DV + 1];
  bwd::ChunkScalars cs;
};

// B1: per chunk slot (full or partial) and head: X, W, Kt, -W^T, dDelta_local
// = P^T dO and R = (diag(Gamma) Q)^T dO - W^T dDelta_local.
template <class D, int DK, int DV>
__global__ __launch_bounds__(256) void k_bwd_local(const BwdArgs a) {
  using namespace bwd;
  using T = typename D::T;
  typedef BwdSlot<DK, DV, sizeof(T)> Slot;
  __shared__ BwdLocalLds<DK, DV> sm;
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
  chunk_scalars<D>(sm.cs, (const T*)a.g, (const T*)a.beta, row0, H, n);
  const ChunkScalars& cs = sm.cs;
  const size_t kq0 = kq_row((size_t)a.cu[i] + (size_t)c * a.Cl, h, a.Hk, a.G);
  auto Kx = [&](int t, int e) { return t < n ? D::load(kp, (kq0 + (size_t)t * a.Hk) * DK + e) : 0.f; };
  auto Qx = [&](int t, int e) { return t < n ? D::load(qp, (kq0 + (size_t)t * a.Hk) * DK + e) : 0.f; };
  auto dOx = [&](int t, int j) { return t < n ? D::load(dop, (row0 + (size_t)t * H) * DV + j) : 0.f; };
  uint8_t* ws = a.ws + ((size_t)slot * H + h) * Slot::bytes;

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
      tile_each(acc, 16 * tm, 16 * it, [&](int t, int e, float v) { sm.W[t][e] = v; });
    } else {
      const int u = id - nW, tm = u / (DV / 16), jt = u % (DV / 16);
      acc = tile<C>([&](int t, int s) { return sm.Pt[t][s]; }, [&](int s, int j) { return dOx(s, j); }, 16 * tm,
                    16 * jt, acc);
      tile_each(acc, 16 * tm, 16 * jt, [&](int t, int j, float v) { sm.Dd[t][j] = v; });
      *reinterpret_cast<f32x4*>(Dd + ((size_t)(jt * (C / 16) + tm) * 64 + (tid & 63)) * 4) = acc;
    }
  }
  __syncthreads();
  T* Kt = reinterpret_cast<T*>(ws + Slot::oKt);
  T* WnT = reinterpret_cast<T*>(ws + Slot::oWnT);
  float* Xs = reinterpret_cast<float*>(ws + Slot::oX);
  for (int idx = tid; idx < C * DK; idx += 256) {
    const int t = idx / DK, e = idx % DK;
    D::store(Kt, idx, cs.e[t] * Kx(t, e));
    D::store(WnT, (size_t)e * C + t, -sm.W[t][e]);
  }
  for (int idx = tid; idx < C * C; idx += 256) Xs[idx] = sm.X[idx / C][idx % C];
  float* R = reinterpret_cast<float*>(ws + Slot::oR);
  constexpr int nR = (DK / 16) * (DV / 16);
  for (int id = wave; id < nR; id += 4) {
    const int im = id / (DV / 16), jt = id % (DV / 16);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = tile<C>([&](int e, int t) { return cs.Gam[t] * Qx(t, e); }, [&](int t, int j) { return dOx(t, j); },
                  16 * im, 16 * jt, acc);
    acc = tile<C>([&](int e, int t) { return -sm.W[t][e]; }, [&](int t, int j) { return sm.Dd[t][j]; }, 16 * im,
                  16 * jt, acc);
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

template <int DK, int DV>
struct BwdGradLds {
  static constexpr int DM = DK > DV ? DK : DV;
  float N1[C][C + 1];   // G
  float N2[C][C + 1];   // dT -> dX -> dA -> dG
  float N3[C][C + 1];   // X
  float N4[C][C + 1];   // dPD = (dO Delta^T) .* D, lower incl.
  float N5[C][C + 1];   // Z_P, then Y, then dA D G
  float M1[C][DM + 1];  // W -> dO B^T -> dW -> T^T dW
  float M2[C][DM + 1];  // U -> Delta -> dKt
  bwd::ChunkScalars cs;
  float rzP[C], czP[C], dGamO[C], dGamW[C], de[C], dbc[C], dbr[C], rzA[C], czA[C];
  float red[256];
};

// B3: per chunk slot and head: dq, dk, dv, dg, dbeta of the chunk's tokens.
template <class D, int DK, int DV>
__global__ __launch_bounds__(256) void k_bwd_grads(const BwdArgs a) {
  using namespace bwd;
  using T = typename D::T;
  typedef BwdSlot<DK, DV, sizeof(T)> Slot;
  __shared__ BwdGradLds<DK, DV> sm;
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
  chunk_scalars<D>(sm.cs, (const T*)a.g, (const T*)a.beta, row0, H, n);
  const ChunkScalars& cs = sm.cs;
  const size_t kq0 = kq_row((size_t)a.cu[i] + (size_t)c * a.Cl, h, a.Hk, a.G);
  auto Kx = [&](int t, int e) { return t < n ? D::load(kp, (kq0 + (size_t)t * a.Hk) * DK + e) : 0.f; };
  auto Qx = [&](int t, int e) { return t < n ? D::load(qp, (kq0 + (size_t)t * a.Hk) * DK + e) : 0.f; };
  auto Vx = [&](int t, int j) { return t < n ? D::load(vp, (row0 + (size_t)t * H) * DV + j) : 0.f; };
  auto dOx = [&](int t, int j) { return t < n ? D::load(dop, (row0 + (size_t)t * H) * DV + j) : 0.f; };
  const uint8_t* ws = a.ws + ((size_t)slot * H + h) * Slot::bytes;
  const float* Bst = a.bnd + ((size_t)slot * H + h) * DK * DV;
  const float* dBp = reinterpret_cast<const float*>(ws + Slot::oDbp);
  const float* Ddg = reinterpret_cast<const float*>(ws + Slot::oDd);
  const float* Xs = reinterpret_cast<const float*>(ws + Slot::oX);
  auto dDx = [&](int t, int j) { return Ddg[tile_index<C>(t, j)]; };
  constexpr int nK = 4 * (DK / 16), nV = 4 * (DV / 16);

  // G and X
  for (int q = 0; q < 4; ++q) {
    const int tl = wave * 4 + q, tm = tl >> 2, tn = tl & 3;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = tile<DK>([&](int m, int k) { return Kx(m, k); }, [&](int k, int nn) { return Kx(nn, k); }, 16 * tm, 16 * tn,
                   acc);
    tile_each(acc, 16 * tm, 16 * tn, [&](int t, int s, float v) { sm.N1[t][s] = v; });
  }
  for (int idx = tid; idx < C * C; idx += 256) sm.N3[idx / C][idx % C] = Xs[idx];
  __syncthreads();
  // W = X diag(beta Gamma) K -> M1,  U = X diag(beta) V -> M2
  for (int id = wave; id < nK + nV; id += 4) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (id < nK) {
      const int tm = id / (DK / 16), it = id % (DK / 16);
      acc = tile<C>([&](int t, int r) { return sm.N3[t][r] * (cs.beta[r] * cs.Gam[r]); },
                    [&](int r, int e) { return Kx(r, e); }, 16 * tm, 16 * it, acc);
      tile_each(acc, 16 * tm, 16 * it, [&](int t, int e, float v) { sm.M1[t][e] = v; });
    } else {
      const int u = id - nK, tm = u / (DV / 16), jt = u % (DV / 16);
      acc = tile<C>([&](int t, int r) { return sm.N3[t][r] * cs.beta[r]; }, [&](int r, int j) { return Vx(r, j); },
                    16 * tm, 16 * jt, acc);
      tile_each(acc, 16 * tm, 16 * jt, [&](int t, int j, float v) { sm.M2[t][j] = v; });
    }
  }
  __syncthreads();
  // Delta = U - W B (in place in M2; every tile is read and written by one wave)
  for (int id = wave; id < nV; id += 4) {
    const int tm = id / (DV / 16), jt = id % (DV / 16);
    f32x4 acc;
    {
      const int lane = tid & 63, lr = lane & 15, g = lane >> 4;
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = sm.M2[16 * tm + 4 * g + r][16 * jt + lr];
    }
    acc = tile<DK>([&](int t, int e) { return -sm.M1[t][e]; }, [&](int e, int j) { return Bst[bnd_index<DK>(e, j)]; },
                   16 * tm, 16 * jt, acc);
    tile_each(acc, 16 * tm, 16 * jt, [&](int t, int j, float v) { sm.M2[t][j] = v; });
  }
  __syncthreads();
  // dP .* D (N4), Z_P = dPD .* QK (N5); dV = T^T dDelta
  for (int q = 0; q < 4; ++q) {
    const int tl = wave * 4 + q, tm = tl >> 2, tn = tl & 3;
    f32x4 accP = {0.f, 0.f, 0.f, 0.f}, accQ = {0.f, 0.f, 0.f, 0.f};
    accP = tile<DV>([&](int t, int j) { return dOx(t, j); }, [&](int j, int s) { return sm.M2[s][j]; }, 16 * tm,
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
  __syncthreads();
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
    tile_each(acc, 16 * tm, 16 * it, [&](int t, int e, float v) { sm.M1[t][e] = v; });
  }
  __syncthreads();
  // dQ = diag(Gamma) dO B^T + dPD K;  dGamma (output part) = <dO B^T, Q> per row
  T* dqp = (T*)a.dq;
  for (int id = wave; id < nK; id += 4) {
    const int tm = id / (DK / 16), it = id % (DK / 16);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = tile<C>([&](int t, int s) { return sm.N4[t][s]; }, [&](int s, int e) { return Kx(s, e); }, 16 * tm, 16 * it,
                  acc);
    tile_each(acc, 16 * tm, 16 * it, [&](int t, int e, float v) {
      if (t < n) {
        const float val = cs.Gam[t] * sm.M1[t][e] + v;
        if (a.dq_part)
          a.dq_part[(row0 + (size_t)t * H) * DK + e] = val;
        else
          D::store(dqp, (kq0 + (size_t)t * a.Hk) * DK + e, val);
      }
    });
  }
  if (tid < C) {
    float acc = 0.f;
    for (int e = 0; e < DK; ++e) acc = __builtin_fmaf(sm.M1[tid][e], Qx(tid, e), acc);
    sm.dGamO[tid] = acc;
  }
  __syncthreads();
  // dW = -dDelta B^T -> M1
  for (int id = wave; id < nK; id += 4) {
    const int tm = id / (DK / 16), it = id % (DK / 16);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = tile<DV>([&](int t, int j) { return dDx(t, j); }, [&](int j, int e) { return Bst[bnd_index<DK>(e, j)]; },
                   16 * tm, 16 * it, acc);
    tile_each(acc, 16 * tm, 16 * it, [&](int t, int e, float v) { sm.M1[t][e] = -v; });
  }
  __syncthreads();
  // T^T dW and dKt = Delta dB'^T (kept in registers), dT -> N2
  f32x4 TW[(nK + 3) / 4], KW[(nK + 3) / 4];
  for (int q = 0, id = wave; id < nK; id += 4, ++q) {
    const int tm = id / (DK / 16), it = id % (DK / 16);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    TW[q] = tile<C>([&](int t, int s) { return cs.beta[t] * sm.N3[s][t]; }, [&](int s, int e) { return sm.M1[s][e]; },
                    16 * tm, 16 * it, acc);
    KW[q] = tile<DV>([&](int t, int j) { return sm.M2[t][j]; }, [&](int j, int e) { return dBp[(size_t)e * DV + j]; },
                     16 * tm, 16 * it, acc);
  }
  for (int q = 0; q < 4; ++q) {
    const int tl = wave * 4 + q, tm = tl >> 2, tn = tl & 3;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = tile<DV>([&](int t, int j) { return dDx(t, j); }, [&](int j, int s) { return Vx(s, j); }, 16 * tm, 16 * tn,
                   acc);
    acc = tile<DK>([&](int t, int e) { return sm.M1[t][e]; }, [&](int e, int s) { return cs.Gam[s] * Kx(s, e); },
                   16 * tm, 16 * tn, acc);
    tile_each(acc, 16 * tm, 16 * tn, [&](int t, int s, float v) { sm.N2[t][s] = v; });
  }
  __syncthreads();
  for (int q = 0, id = wave; id < nK; id += 4, ++q) {
    const int tm = id / (DK / 16), it = id % (DK / 16);
    tile_each(TW[q], 16 * tm, 16 * it, [&](int t, int e, float v) { sm.M1[t][e] = v; });
    tile_each(KW[q], 16 * tm, 16 * it, [&](int t, int e, float v) { sm.M2[t][e] = v; });
  }
  __syncthreads();
  // dGamma (W part), de, dbeta (column part)
  if (tid < C) {
    float acc = 0.f;
    for (int e = 0; e < DK; ++e) acc = __builtin_fmaf(sm.M1[tid][e], Kx(tid, e), acc);
    sm.dGamW[tid] = acc;
  } else if (tid < 2 * C) {
    const int t = tid - C;
    float acc = 0.f;
    for (int e = 0; e < DK; ++e) acc = __builtin_fmaf(sm.M2[t][e], Kx(t, e), acc);
    sm.de[t] = acc;
  } else if (tid < 3 * C) {
    const int s = tid - 2 * C;
    float acc = 0.f;
    for (int t = 0; t < C; ++t) acc = __builtin_fmaf(sm.N3[t][s], sm.N2[t][s], acc);
    sm.dbc[s] = acc;
  }
  __syncthreads();
  for (int idx = tid; idx < C * C; idx += 256) sm.N2[idx / C][idx % C] *= sm.cs.beta[idx % C];  // dX
  __syncthreads();
  // Y = dX X^T -> N5
  for (int q = 0; q < 4; ++q) {
    const int tl = wave * 4 + q, tm = tl >> 2, tn = tl & 3;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = tile<C>([&](int t, int r) { return sm.N2[t][r]; }, [&](int r, int s) { return sm.N3[s][r]; }, 16 * tm,
                  16 * tn, acc);
    tile_each(acc, 16 * tm, 16 * tn, [&](int t, int s, float v) { sm.N5[t][s] = v; });
  }
  __syncthreads();
  // dA = -X^T Y, strict lower -> N2
  {
    f32x4 accs[4];
    for (int q = 0; q < 4; ++q) {
      const int tl = wave * 4 + q, tm = tl >> 2, tn = tl & 3;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      accs[q] = tile<C>([&](int t, int r) { return sm.N3[r][t]; }, [&](int r, int s) { return sm.N5[r][s]; }, 16 * tm,
                        16 * tn, acc);
    }
    __syncthreads();
    for (int q = 0; q < 4; ++q) {
      const int tl = wave * 4 + q, tm = tl >> 2, tn = tl & 3;
      tile_each(accs[q], 16 * tm, 16 * tn, [&](int t, int s, float v) { sm.N2[t][s] = (s < t) ? -v : 0.f; });
    }
  }
  __syncthreads();
  // dA D G -> N5, dG = dA beta_t D -> N2
  for (int idx = tid; idx < C * C; idx += 256) {
    const int t = idx / C, s = idx % C;
    const float dA = sm.N2[t][s];
    float zb = 0.f, dG = 0.f;
    if (s < t) {
      const float Dv = expf(cs.gam[t] - cs.gam[s]);
      zb = dA * Dv * sm.N1[t][s];
      dG = dA * cs.beta[t] * Dv;
    }
    sm.N5[t][s] = zb;
    sm.N2[t][s] = dG;
  }
  __syncthreads();
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
  __syncthreads();
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
        const float val = v + cs.e[t] * sm.M2[t][e] + cs.Gam[t] * sm.M1[t][e];
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

template <int DK, int DV>
__global__ __launch_bounds__((kBwdWaves<DK, DV> * 64)) void k_bwd_state_bf16(const BwdArgs a) {
  typedef bwdb::Slot<DK, DV> Sl;
  constexpr int W = kBwdWaves<DK, DV>;
  __shared__ bwdb::StateLds<DK, DV, W> sm;
  SlotPos p;
  if (!slot_pos(a, p)) return;
  bwdb::state_stage<DK, DV, W>(sm, (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.d_o,
                            (const uint16_t*)a.g, (const uint16_t*)a.beta, p.row0, a.H, p.kq0, a.Hk, p.n,
                            a.bnd + p.sl * DK * DV, a.ws + p.sl * Sl::bytes);
}

template <int DK, int DV>
__global__ __launch_bounds__((kBwdWaves<DK, DV> * 64)) void k_bwd_grads_bf16(const BwdArgs a) {
  typedef bwdb::Slot<DK, DV> Sl;
  __shared__ bwdb::GradLds<DK, DV> sm;
  SlotPos p;
  if (!slot_pos(a, p)) return;
  bwdb::grad_stage<DK, DV, kBwdWaves<DK, DV>>(sm, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                           (const uint16_t*)a.d_o, (const uint16_t*)a.g, (const uint16_t*)a.beta, p.row0, a.H, p.kq0,
                           a.Hk, p.n, a.ws + p.sl * Sl::bytes, (uint16_t*)a.dq, (uint16_t*)a.dk, a.dq_part,
                           a.dk_part, (uint16_t*)a.dv, a.dg, a.dbeta);
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

// ---------------------------------------------------------------------------
// host side

thread_local std::string g_last_error;
thread_local void* const* g_events = nullptr;
thread_local int32_t g_n_events = 0;

// records stage event i (instrumentation hook; no-op unless set)
inline void mark(int i, hipStream_t st) {
  if (g_events && i < g_n_events && g_events[i]) (void)hipEventRecord((hipEvent_t)g_events[i], st);
}

gdn_status fail(gdn_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

// wide_ok: the call serves d_k = d_v = 256 (bf16 prefill, decode,
// continuation and the cache read-out; not fwd_bwd or the comparators)
bool shape_ok(const gdn_cpr_shape* s, std::string* why, bool wide_ok = false) {
  if (!s) {
    *why = "shape is NULL";
    return false;
  }
  if (s->num_heads < 1) {
    *why = "num_heads must be >= 1";
    return false;
  }
  const bool wide = s->head_dim_k == 256 && s->head_dim_v == 256;
  if (!((s->head_dim_k == 64 || s->head_dim_k == 128) && (s->head_dim_v == 64 || s->head_dim_v == 128)) && !wide) {
    *why = "head dims must be 64 or 128 (or both 256)";
    return false;
  }
  if (wide && !wide_ok) {
    *why = "head dims of 256 serve prefill, decode and continuation only";
    return false;
  }
  if (wide && s->dtype != GDN_DTYPE_BF16) {
    *why = "head dims of 256 take bf16 inputs";
    return false;
  }
  if (s->chunk != 16 && s->chunk != 32 && s->chunk != C) {
    *why = "chunk must be 16, 32 or 64";
    return false;
  }
  if (s->dtype != GDN_DTYPE_F32 && s->dtype != GDN_DTYPE_BF16) {
    *why = "dtype must be GDN_DTYPE_F32 or GDN_DTYPE_BF16";
    return false;
  }
  if (s->num_key_heads < 0 || s->num_key_heads > s->num_heads ||
      (s->num_key_heads > 0 && s->num_heads % s->num_key_heads != 0)) {
    *why = "num_key_heads must be 0 or divide num_heads";
    return false;
  }
  return true;
}

// heads of q and k (0 in the shape means one per value head)
int key_heads(const gdn_cpr_shape& s) { return s.num_key_heads > 0 ? s.num_key_heads : s.num_heads; }

struct PrefillLayout {
  size_t full_base, all_base, prod, slot, gamn, bnd, order, ready, counters, total;
};

PrefillLayout prefill_layout(const gdn_cpr_shape& s, int32_t N, int64_t T) {
  const size_t H = s.num_heads, DK = s.head_dim_k, DV = s.head_dim_v;
  const size_t Fmax = (size_t)(T / s.chunk);
  const size_t Amax = Fmax + (size_t)N;
  PrefillLayout L;
  size_t off = 0;
  L.full_base = off;
  off = align_up(off + sizeof(int32_t) * (N + 1));
  L.all_base = off;
  off = align_up(off + sizeof(int32_t) * (N + 1));
  L.prod = off;
  L.slot = prod_slot_bytes(s.dtype == GDN_DTYPE_BF16, (int)DK, (int)DV);
  off = align_up(off + Fmax * H * L.slot);
  L.gamn = off;
  off = align_up(off + sizeof(float) * Fmax * H);
  L.bnd = off;
  off = align_up(off + sizeof(float) * Amax * H * DK * DV);
  // fused launch: chunk-major slot order, per-chain-item counts and
  // chunk-product flags, ticket and timeout words
  L.order = off;
  off = align_up(off + sizeof(int32_t) * Amax);
  L.ready = off;  // then one chunk-product flag per (full chunk, head)
  off = align_up(off + sizeof(int32_t) * ((size_t)N * H * (DV / kFusedChainCols) * kReadyStride + Fmax * H));
  L.counters = off;
  off = align_up(off + 2 * sizeof(int32_t));
  L.total = off;
  return L;
}

struct DecodeLayout {
  size_t flag, prod, slot, gamn, total;
};

DecodeLayout decode_layout(const gdn_cpr_shape& s, int32_t N) {
  const size_t H = s.num_heads, DK = s.head_dim_k, DV = s.head_dim_v;
  DecodeLayout L;
  size_t off = 0;
  L.flag = off;
  off = align_up(off + sizeof(int32_t) * (size_t)N * H);
  L.prod = off;
  L.slot = prod_slot_bytes(s.dtype == GDN_DTYPE_BF16, (int)DK, (int)DV);
  off = align_up(off + (size_t)N * H * L.slot);
  L.gamn = off;
  off = align_up(off + sizeof(float) * (size_t)N * H);
  L.total = off;
  return L;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

#define CHECK_PTR(p, name)                                                                 \
  do {                                                                                     \
    if (!(p)) return fail(GDN_ERR_INVALID_ARG, "%s: %s is NULL", fn, name);                \
    if (!aligned16(p)) return fail(GDN_ERR_INVALID_ARG, "%s: %s is not 16-byte aligned", fn, name); \
  } while (0)

#define CHECK_OPT_PTR(p, name)                                                             \
  do {                                                                                     \
    if ((p) && !aligned16(p))                                                              \
      return fail(GDN_ERR_INVALID_ARG, "%s: %s is not 16-byte aligned", fn, name);         \
  } while (0)

gdn_status launch_status(const char* fn) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(GDN_ERR_HIP, "%s: kernel launch failed: %s", fn, hipGetErrorString(e));
  g_last_error.clear();
  return GDN_OK;
}

// A second stream for the overlapped stages of bf16 gdn_cpr_fwd_bwd, with the
// events that fork work onto it and join it back.  Streams come from a
// bounded pool per device (at most kSidePool, each created on first need at
// the default priority and kept until the process ends): a call holds one
// while it enqueues, so concurrent callers never share a stream's events,
// and the number of streams stays bounded however many threads call.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};

constexpr int kSidePool = 8;
constexpr int kMaxDevices = 64;

struct SidePool {
  std::mutex m;
  SideStream made[kSidePool];
  bool busy[kSidePool] = {};
  int n = 0;
};

SidePool& side_pool(int dev) {
  static SidePool pools[kMaxDevices];
  return pools[dev];
}

// creates a side stream and its events on device dev (the current device is
// restored); false if any of them cannot be made
bool make_side_stream(int dev, SideStream& y) {
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return false;
  if (cur != dev && hipSetDevice(dev) != hipSuccess) return false;
  bool ok = hipStreamCreateWithFlags(&y.s, hipStreamNonBlocking) == hipSuccess;
  hipEvent_t* ev[2] = {&y.fork, &y.join};
  for (int i = 0; i < 2 && ok; ++i) ok = hipEventCreateWithFlags(ev[i], hipEventDisableTiming) == hipSuccess;
  if (cur != dev) (void)hipSetDevice(cur);
  if (!ok) {
    for (int i = 0; i < 2; ++i)
      if (*ev[i]) (void)hipEventDestroy(*ev[i]);
    if (y.s) (void)hipStreamDestroy(y.s);
    (void)hipGetLastError();
    y = SideStream{};
  }
  return ok;
}

// A side stream on the device of st, held for the lease's lifetime; get()
// is nullptr when none can be had (every pooled stream in use and the pool
// full, or creation failed): the caller then runs on st alone.
class SideLease {
 public:
  explicit SideLease(hipStream_t st) {
    hipDevice_t dev = 0;
    if (hipStreamGetDevice(st, &dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
      (void)hipGetLastError();
      return;
    }
    SidePool& p = side_pool(dev);
    std::lock_guard<std::mutex> lock(p.m);
    for (int i = 0; i < p.n; ++i)
      if (!p.busy[i]) {
        take(p, i, dev);
        return;
      }
    if (p.n < kSidePool && make_side_stream(dev, p.made[p.n])) take(p, p.n++, dev);
  }
  ~SideLease() {
    if (slot_ < 0) return;
    SidePool& p = side_pool(dev_);
    std::lock_guard<std::mutex> lock(p.m);
    p.busy[slot_] = false;
  }
  SideLease(const SideLease&) = delete;
  SideLease& operator=(const SideLease&) = delete;
  const SideStream* get() const { return slot_ < 0 ? nullptr : &side_pool(dev_).made[slot_]; }

 private:
  void take(SidePool& p, int i, int dev) {
    p.busy[i] = true;
    slot_ = i;
    dev_ = dev;
  }
  int slot_ = -1, dev_ = 0;
};

// bf16 boundary chain: the fewer (sequence, head) pairs, the more work-groups
// per pair (the column split is bit-neutral)
template <int DK, int DV>
void launch_chain_bf16(const PrefillArgs& a, hipStream_t st) {
  const long pairs = (long)a.N * a.H;
  if constexpr (DV >= 128) {
    if (pairs * (DV / 128) >= 128) {
      hipLaunchKernelGGL((k_chain_prefill_bf16<DK, DV, 4, 2>), dim3(a.N, a.H, DV / 128), dim3(256), 0, st, a);
      return;
    }
  }
  if (pairs * (DV / 64) >= 96)
    hipLaunchKernelGGL((k_chain_prefill_bf16<DK, DV, 4, 1>), dim3(a.N, a.H, DV / 64), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((k_chain_prefill_bf16<DK, DV, 2, 1>), dim3(a.N, a.H, DV / 32), dim3(128), 0, st, a);
}

template <int DK, int DV>
void launch_resync_bf16(const DecodeArgs& a, int n_seqs, hipStream_t st) {
  hipLaunchKernelGGL((k_resync_bf16<DK, DV>), dim3(n_seqs, a.H), dim3(256), 0, st, a);
}

// The fused boundary chain + scan launch (k_chain_scan_bf16) serves bf16
// prefills of up to kFusedMaxSeqs sequences whose chain items leave most of
// the chip's work-group slots to the scan; other prefills run the chain and
// the scan as two launches.  Both give the same bits.
constexpr long kFusedMaxChainItems = 512;
// and whose longest chain (at most T / C steps of a few microseconds) ends well
// inside the bounded waits of its scan units (about a second)
constexpr long kFusedMaxChainSteps = 1L << 16;

template <int DK, int DV>
bool use_fused(const PrefillArgs& a, int64_t T) {
  return KeySplit<DK>::kParts == 1 && a.order && a.all_chunks == 0 && a.N <= kFusedMaxSeqs &&
         (long)a.N * a.H * (DV / kFusedChainCols) <= kFusedMaxChainItems && T / a.Cl <= kFusedMaxChainSteps;
}

template <class D, int DK, int DV>
gdn_status run_prefill(const PrefillArgs& a, int64_t T, hipStream_t st, const char* fn) {
  const int Fmax = (int)(T / a.Cl);
  const int Amax = Fmax + a.N;
  constexpr bool kBf16 = std::is_same<D, Bf16>::value;
  const bool fused = kBf16 && use_fused<DK, DV>(a, T);
  // at d_k = 256 the chain runs as the chain items of the fused kernel alone
  // (its one-buffer stage fits the LDS where the two-buffer chain's does not),
  // then the scan
  constexpr bool kChainOnly = KeySplit<DK>::kParts > 1;
  static_assert(!kChainOnly || kBf16, "d_k = 256 runs on the bf16 path");
  constexpr int NZ = DV / kFusedChainCols;
  // the fused launch's counts: the chain items', then the chunk-product flags
  const int n_counts = a.N * a.H * NZ * kReadyStride;
  FusedPlan fp{};
  if (fused || kChainOnly) fp = FusedPlan{a.order, a.counters, a.ready, n_counts + (fused ? Fmax * a.H : 0)};
  mark(0, st);
  hipLaunchKernelGGL(k_plan, dim3(1), dim3(1024), 0, st, a.start, a.end, a.N, a.Cl, a.full_base, a.all_base, fp);
  mark(1, st);
  if (fused) {
    // chunk products, chain and scan as one launch: events 2, 3 and 4 follow it
    const FusedArgs f{a.order, a.counters, a.ready, a.ready + n_counts, a.counters + 1, Amax * a.H,
                      a.N * a.H * NZ};
    const long units = (long)Amax * a.H * NZ;
    const unsigned groups = (unsigned)(f.n_cp + f.n_chain + (units + 3) / 4);
    if constexpr (kBf16) hipLaunchKernelGGL((k_chain_scan_bf16<DK, DV>), dim3(groups), dim3(256), 0, st, a, f);
    mark(2, st);
    mark(3, st);
    mark(4, st);
    return launch_status(fn);
  }
  if (Fmax > 0) {
    if constexpr (kBf16)
      hipLaunchKernelGGL((k_chunk_local_prefill_bf16<DK, DV>), dim3(Fmax, a.H), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((k_chunk_local_prefill<D, DK, DV>), dim3(Fmax, a.H), dim3(256), 0, st, a);
  }
  mark(2, st);
  if (a.N > 0) {
    if constexpr (kChainOnly) {
      const FusedArgs f{a.order, a.counters, a.ready, nullptr, a.counters + 1, 0, a.N * a.H * NZ};
      hipLaunchKernelGGL((k_chain_scan_bf16<DK, DV>), dim3(f.n_chain), dim3(256), 0, st, a, f);
    } else if constexpr (kBf16) {
      launch_chain_bf16<DK, DV>(a, st);
    } else {
      hipLaunchKernelGGL((k_chain_prefill<DK, DV>), dim3(a.N, a.H, DV / kChainCols), dim3(256), 0, st, a);
    }
  }
  mark(3, st);
  if (Amax > 0 && T > 0)
    hipLaunchKernelGGL((k_scan<D, DK, DV>), dim3(Amax, a.H, DV / KeySplit<DK>::kCols), dim3(kWave), 0, st, a);
  mark(4, st);
  return launch_status(fn);
}

// The resync runs over groups of `group` sequences, one launch (bf16) or
// two (fp32) per group, each group's pairs using product slots 0 ..
// group * H - 1; the workspace decode takes the whole batch as one group.
template <class D, int DK, int DV>
gdn_status run_decode(const DecodeArgs& a, int group, hipStream_t st, const char* fn) {
  mark(0, st);
  hipLaunchKernelGGL((k_decode<D, DK, DV>), dim3(a.N, a.H), dim3(kColumnThreads<DK, DV>), 0, st, a);
  mark(1, st);
  for (int s0 = 0; s0 < a.N; s0 += group) {
    DecodeArgs r = a;
    r.seq0 = s0;
    const int n = std::min(group, a.N - s0);
    if constexpr (std::is_same<D, Bf16>::value) {
      launch_resync_bf16<DK, DV>(r, n, st);
    } else {
      hipLaunchKernelGGL((k_chunk_local_resync<D, DK, DV>), dim3(n, r.H), dim3(256), 0, st, r);
      hipLaunchKernelGGL((k_chain_resync<DK, DV>), dim3(n, r.H, DV / kChainCols), dim3(256), 0, st, r);
    }
  }
  mark(2, st);
  return launch_status(fn);
}

// Calls that also serve d_k = d_v = 256 on bf16 inputs (specialised below)
template <template <class, int, int> class Fn>
struct WideFn : std::false_type {};

template <template <class, int, int> class Fn, class... Args>
gdn_status dispatch(const gdn_cpr_shape& s, Args&&... args) {
  const bool bf = s.dtype == GDN_DTYPE_BF16;
  const int dk = s.head_dim_k, dv = s.head_dim_v;
  if constexpr (WideFn<Fn>::value) {
    if (bf && dk == 256 && dv == 256) return Fn<Bf16, 256, 256>::run(std::forward<Args>(args)...);
  }
#define GDN_CASE(DKv, DVv)                                                         \
  if (dk == DKv && dv == DVv)                                                      \
    return bf ? Fn<Bf16, DKv, DVv>::run(std::forward<Args>(args)...)               \
              : Fn<F32, DKv, DVv>::run(std::forward<Args>(args)...);
  GDN_CASE(64, 64)
  GDN_CASE(64, 128)
  GDN_CASE(128, 64)
  GDN_CASE(128, 128)
#undef GDN_CASE
  return fail(GDN_ERR_UNSUPPORTED, "unsupported head dims");
}

template <class D, int DK, int DV>
struct PrefillFn {
  static gdn_status run(const PrefillArgs& a, int64_t T, hipStream_t st, const char* fn) {
    return run_prefill<D, DK, DV>(a, T, st, fn);
  }
};

template <class D, int DK, int DV>
struct DecodeFn {
  static gdn_status run(const DecodeArgs& a, int group, hipStream_t st, const char* fn) {
    return run_decode<D, DK, DV>(a, group, st, fn);
  }
};

struct ContLayout {
  PrefillLayout pre;
  DecodeLayout dec;
  size_t dec_off, body_start, total;
};

ContLayout cont_layout(const gdn_cpr_shape& s, int32_t N, int64_t T) {
  ContLayout L;
  L.pre = prefill_layout(s, N, T);
  L.dec = decode_layout(s, N);
  L.dec_off = L.pre.total;
  L.body_start = align_up(L.dec_off + L.dec.total);
  L.total = align_up(L.body_start + sizeof(int32_t) * (size_t)N);
  return L;
}

template <class D, int DK, int DV>
struct ContFn {
  static gdn_status run(const ContArgs& ca, const DecodeArgs& da, const PrefillArgs& pa, int64_t T, hipStream_t st,
                        const char* fn) {
    hipLaunchKernelGGL((k_cont_head<D, DK, DV>), dim3(ca.N, ca.H), dim3(kColumnThreads<DK, DV>), 0, st, ca);
    if constexpr (std::is_same<D, Bf16>::value) {
      launch_resync_bf16<DK, DV>(da, da.N, st);
    } else {
      hipLaunchKernelGGL((k_chunk_local_resync<D, DK, DV>), dim3(da.N, da.H), dim3(256), 0, st, da);
      hipLaunchKernelGGL((k_chain_resync<DK, DV>), dim3(da.N, da.H, DV / kChainCols), dim3(256), 0, st, da);
    }
    gdn_status r = launch_status(fn);
    if (r != GDN_OK) return r;
    return run_prefill<D, DK, DV>(pa, T, st, fn);
  }
};

template <>
struct WideFn<PrefillFn> : std::true_type {};
template <>
struct WideFn<DecodeFn> : std::true_type {};
template <>
struct WideFn<ContFn> : std::true_type {};

// comparators: chunkwise layout = plan, one product slot and one boundary
// state per (chunk slot incl. partial, head)
struct CmpLayout {
  size_t full_base, all_base, prod, gamn, bnd, total;
};

CmpLayout cmp_layout(const gdn_cpr_shape& s, int32_t N, int64_t T) {
  const size_t H = s.num_heads, DK = s.head_dim_k, DV = s.head_dim_v;
  const size_t Amax = (size_t)(T / C) + (size_t)N;
  CmpLayout L;
  size_t off = 0;
  L.full_base = off;
  off = align_up(off + sizeof(int32_t) * (N + 1));
  L.all_base = off;
  off = align_up(off + sizeof(int32_t) * (N + 1));
  L.prod = off;
  off = align_up(off + Amax * H * prod_slot_bytes(true, (int)DK, (int)DV));
  L.gamn = off;
  off = align_up(off + sizeof(float) * Amax * H);
  L.bnd = off;
  off = align_up(off + sizeof(float) * Amax * H * DK * DV);
  L.total = off;
  return L;
}

template <class D, int DK, int DV>
struct CmpPrefillFn {
  static gdn_status run(int mode, const CmpArgs& ca, const PrefillArgs& pa, int64_t T, hipStream_t st,
                        const char* fn) {
    if constexpr (!std::is_same<D, Bf16>::value) {
      return fail(GDN_ERR_UNSUPPORTED, "%s: the comparators take bf16 inputs", fn);
    } else {
      const int Amax = (int)(T / C) + ca.N;
      if (mode == GDN_CMP_RECURRENT) {
        hipLaunchKernelGGL((k_cmp_rec_prefill<D, DK, DV>), dim3(ca.N, ca.H, DV / kWave), dim3(kWave), 0, st, ca);
        return launch_status(fn);
      }
      hipLaunchKernelGGL(k_plan, dim3(1), dim3(1024), 0, st, pa.start, pa.end, pa.N, pa.Cl, pa.full_base,
                         pa.all_base, FusedPlan{});
      if (T > 0) hipLaunchKernelGGL((k_cmp_chunk_local_bf16<DK, DV>), dim3(Amax, ca.H), dim3(256), 0, st, ca);
      launch_chain_bf16<DK, DV>(pa, st);
      if (T > 0) hipLaunchKernelGGL((k_cmp_chunk_out_bf16<DK, DV>), dim3(Amax, ca.H), dim3(256), 0, st, ca);
      return launch_status(fn);
    }
  }
};

template <class D, int DK, int DV>
struct CmpDecodeFn {
  static gdn_status run(const CmpArgs& ca, hipStream_t st, const char* fn) {
    hipLaunchKernelGGL((k_cmp_rec_decode<D, DK, DV>), dim3(ca.N, ca.H), dim3(DV), 0, st, ca);
    return launch_status(fn);
  }
};

template <class D, int DK, int DV>
struct CmpChunkDecodeFn {
  static gdn_status run(const DecodeArgs& a, hipStream_t st, const char* fn) {
    if constexpr (!std::is_same<D, Bf16>::value) {
      return fail(GDN_ERR_UNSUPPORTED, "%s: the comparators take bf16 inputs", fn);
    } else {
      hipLaunchKernelGGL((k_cmp_cdec_local_bf16<DK, DV>), dim3(a.N, a.H), dim3(256), 0, st, a);
      hipLaunchKernelGGL((k_cmp_cdec_out_bf16<DK, DV>), dim3(a.N, a.H), dim3(256), 0, st, a);
      hipLaunchKernelGGL((k_chain_resync_bf16<DK, DV>), dim3(a.N, a.H, DV / (16 * kResyncNT) / kResyncWaves<DV>),
                       dim3(64 * kResyncWaves<DV>), 0, st, a);
      return launch_status(fn);
    }
  }
};

// dq, dk of key heads shared by G value heads: out[tok][j][e] = sum over
// g = 0 .. G-1 (ascending) of part[tok][j G + g][e], rounded once to dtype.
// One work-group of DK threads per (token, key head).
template <class D, int DK>
__global__ __launch_bounds__(DK) void k_key_head_sum(const float* __restrict__ part, typename D::T* __restrict__ out,
                                                     int Hk, int G) {
  const size_t r = blockIdx.x;  // token * Hk + j
  const int e = threadIdx.x;
  const size_t tok = r / Hk, j = r % Hk;
  const float* p = part + ((tok * Hk + j) * G) * DK + e;  // rows tok * H + j G + g, H = Hk G
  float acc = p[0];
  for (int g = 1; g < G; ++g) acc = acc + p[(size_t)g * DK];
  D::store(out, r * DK + e, acc);
}

struct FwdBwdLayout {
  PrefillLayout pre;
  size_t s_bnd, s_run, tail_k, tail_v, tail_g, tail_b, tail_len, bgamn, bslots, slot, dq_part, dk_part, total;
};

FwdBwdLayout fwd_bwd_layout(const gdn_cpr_shape& s, int32_t N, int64_t T) {
  const size_t H = s.num_heads, DK = s.head_dim_k, DV = s.head_dim_v;
  const size_t esz = s.dtype == GDN_DTYPE_BF16 ? 2 : 4;
  const size_t Amax = (size_t)(T / s.chunk) + (size_t)N;
  FwdBwdLayout L;
  L.pre = prefill_layout(s, N, T);
  size_t off = L.pre.total;
  const size_t NH = (size_t)N * H;
  L.s_bnd = off;
  off = align_up(off + NH * DK * DV * 4);
  L.s_run = off;
  off = align_up(off + NH * DK * DV * 4);
  L.tail_k = off;
  off = align_up(off + NH * C * DK * esz);
  L.tail_v = off;
  off = align_up(off + NH * C * DV * esz);
  L.tail_g = off;
  off = align_up(off + NH * C * esz);
  L.tail_b = off;
  off = align_up(off + NH * C * esz);
  L.tail_len = off;
  off = align_up(off + NH * 4);
  L.bgamn = off;
  off = align_up(off + Amax * H * 4);
  if (s.dtype == GDN_DTYPE_BF16)  // bwdb::Slot
    L.slot = 2 * (size_t)C * DK * 2 + 2 * DK * DV * 4 + (size_t)C * C * 4 + 3 * (size_t)C * DK * 4 +
             3 * (size_t)C * DV * 4 + 256;
  else
    L.slot = (size_t)C * DK * esz + DK * (size_t)C * esz + DK * DV * 4 + (size_t)C * DV * 4 + (size_t)C * C * 4 +
             DK * DV * 4;
  L.bslots = off;
  off = align_up(off + Amax * H * L.slot);
  L.dq_part = L.dk_part = 0;
  if (key_heads(s) != (int)H) {  // per-value-head dq, dk partials
    L.dq_part = off;
    off = align_up(off + (size_t)T * H * DK * 4);
    L.dk_part = off;
    off = align_up(off + (size_t)T * H * DK * 4);
  }
  L.total = off;
  return L;
}

template <class D, int DK, int DV>
struct FwdBwdFn {
  static void launch_key_head_sums(const BwdArgs& ba, int64_t T, hipStream_t st) {
    if (!ba.dq_part) return;
    const unsigned rows = (unsigned)(T * ba.Hk);
    hipLaunchKernelGGL((k_key_head_sum<D, DK>), dim3(rows), dim3(DK), 0, st, ba.dq_part, (typename D::T*)ba.dq, ba.Hk,
                       ba.G);
    hipLaunchKernelGGL((k_key_head_sum<D, DK>), dim3(rows), dim3(DK), 0, st, ba.dk_part, (typename D::T*)ba.dk, ba.Hk,
                       ba.G);
  }
  static void launch_bwd_chain_bf16(const BwdArgs& ba, hipStream_t st) {
    const long pairs = (long)ba.N * ba.H;
    if (pairs * (DV / 64) >= 96)
      hipLaunchKernelGGL((k_bwd_chain_bf16<DK, DV, 4, 1>), dim3(ba.N, ba.H, DV / 64), dim3(256), 0, st, ba);
    else
      hipLaunchKernelGGL((k_bwd_chain_bf16<DK, DV, 2, 1>), dim3(ba.N, ba.H, DV / 32), dim3(128), 0, st, ba);
  }
  // bf16 path on two streams.  The backward's local terms and reverse chain
  // read only the inputs, d_o, d_hT and the plan, so they run on the side
  // stream beside the forward chunk products, boundary chain and in-chunk
  // scan; the state and gradient stages, which need both chains, follow on
  // the caller's stream after the join.  (Running the scan beside the state
  // and gradient stages instead measured the same.)  Every kernel computes
  // what it computes in the one-stream order, so the bits are the same.
  static gdn_status run_overlapped(const PrefillArgs& pa, const BwdArgs& ba, int64_t T, hipStream_t st,
                                   const SideStream& x, const char* fn) {
    const int Fmax = (int)(T / pa.Cl), Amax = Fmax + pa.N;
    auto ev = [&](hipError_t e) { return e == hipSuccess; };
    mark(0, st);
    hipLaunchKernelGGL(k_plan, dim3(1), dim3(1024), 0, st, pa.start, pa.end, pa.N, pa.Cl, pa.full_base, pa.all_base,
                       FusedPlan{});
    mark(1, st);
    if (!ev(hipEventRecord(x.fork, st)) || !ev(hipStreamWaitEvent(x.s, x.fork, 0)))
      return fail(GDN_ERR_HIP, "%s: stream fork failed: %s", fn, hipGetErrorString(hipGetLastError()));
    hipLaunchKernelGGL((k_bwd_local_bf16<DK, DV>), dim3(Amax, pa.H), dim3(kBwdWaves<DK, DV> * 64), 0, x.s, ba);
    launch_bwd_chain_bf16(ba, x.s);
    if (!ev(hipEventRecord(x.join, x.s))) return fail(GDN_ERR_HIP, "%s: event record failed", fn);
    if (Fmax > 0)
      hipLaunchKernelGGL((k_chunk_local_prefill_bf16<DK, DV>), dim3(Fmax, pa.H), dim3(256), 0, st, pa);
    mark(2, st);
    if (pa.N > 0) launch_chain_bf16<DK, DV>(pa, st);
    mark(3, st);
    hipLaunchKernelGGL((k_scan<D, DK, DV>), dim3(Amax, pa.H, DV / kWave), dim3(kWave), 0, st, pa);
    mark(4, st);
    if (!ev(hipStreamWaitEvent(st, x.join, 0)))
      return fail(GDN_ERR_HIP, "%s: stream join failed: %s", fn, hipGetErrorString(hipGetLastError()));
    mark(5, st);
    hipLaunchKernelGGL((k_bwd_state_bf16<DK, DV>), dim3(Amax, pa.H), dim3(kBwdWaves<DK, DV> * 64), 0, st, ba);
    hipLaunchKernelGGL((k_bwd_grads_bf16<DK, DV>), dim3(Amax, pa.H), dim3(kBwdWaves<DK, DV> * 64), 0, st, ba);
    launch_key_head_sums(ba, T, st);
    mark(6, st);
    return launch_status(fn);
  }
  static gdn_status run(const PrefillArgs& pa, const BwdArgs& ba, int64_t T, size_t slot_bytes, hipStream_t st,
                        const char* fn) {
    constexpr bool kBf16 = std::is_same<D, Bf16>::value;
    const size_t want = kBf16 ? bwdb::Slot<DK, DV>::bytes : bwd::BwdSlot<DK, DV, sizeof(typename D::T)>::bytes;
    if (slot_bytes != want) return fail(GDN_ERR_HIP, "%s: internal slot size mismatch", fn);
    if constexpr (kBf16) {
      if (T > 0) {
        // one stream only if no side stream can be had
        SideLease lease(st);
        if (const SideStream* x = lease.get()) return run_overlapped(pa, ba, T, st, *x, fn);
      }
    }
    gdn_status r = run_prefill<D, DK, DV>(pa, T, st, fn);
    if (r != GDN_OK) return r;
    const int Amax = (int)(T / pa.Cl) + pa.N;
    if constexpr (kBf16) {
      if (T > 0)
        hipLaunchKernelGGL((k_bwd_local_bf16<DK, DV>), dim3(Amax, pa.H), dim3(kBwdWaves<DK, DV> * 64), 0, st, ba);
      launch_bwd_chain_bf16(ba, st);
      mark(5, st);
      if (T > 0) {
        hipLaunchKernelGGL((k_bwd_state_bf16<DK, DV>), dim3(Amax, pa.H), dim3(kBwdWaves<DK, DV> * 64), 0, st, ba);
        hipLaunchKernelGGL((k_bwd_grads_bf16<DK, DV>), dim3(Amax, pa.H), dim3(kBwdWaves<DK, DV> * 64), 0, st, ba);
        launch_key_head_sums(ba, T, st);
      }
      mark(6, st);
    } else {
      // fp32 inputs: local terms, reverse chain and gradients on fp32 operands
      if (T > 0) hipLaunchKernelGGL((k_bwd_local<D, DK, DV>), dim3(Amax, pa.H), dim3(256), 0, st, ba);
      hipLaunchKernelGGL((k_bwd_chain_f32<DK, DV>), dim3(pa.N, pa.H), dim3(DV * 4), 0, st, ba);
      mark(5, st);
      if (T > 0) {
        hipLaunchKernelGGL((k_bwd_grads<D, DK, DV>), dim3(Amax, pa.H), dim3(256), 0, st, ba);
        launch_key_head_sums(ba, T, st);
      }
      mark(6, st);
    }
    return launch_status(fn);
  }
};

}  // namespace

// ===========================================================================
// C ABI

extern "C" size_t gdn_cpr_workspace_size(const gdn_cpr_shape* shape, int32_t num_seqs,
                                         int64_t total_tokens, int32_t op) {
  std::string why;
  if (!shape_ok(shape, &why, op != GDN_OP_FWD_BWD) || num_seqs < 0 || total_tokens < 0) return 0;
  if (op == GDN_OP_PREFILL) return prefill_layout(*shape, num_seqs, total_tokens).total;
  if (op == GDN_OP_FWD_BWD) return fwd_bwd_layout(*shape, num_seqs, total_tokens).total;
  if (op == GDN_OP_DECODE) return decode_layout(*shape, num_seqs).total;
  if (op == GDN_OP_PREFILL_CONTINUE) return cont_layout(*shape, num_seqs, total_tokens).total;
  return 0;
}

extern "C" gdn_status gdn_cpr_prefill(const gdn_cpr_shape* shape, int32_t num_seqs, int64_t total_tokens,
                                      const void* q, const void* k, const void* v, const void* g,
                                      const void* beta, const int32_t* cu_seqlens, const float* h0, float* hT,
                                      const gdn_cpr_cache* cache_out, void* o, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  const char* fn = "gdn_cpr_prefill";
  std::string why;
  if (!shape_ok(shape, &why, true)) return fail(GDN_ERR_UNSUPPORTED, "%s: %s", fn, why.c_str());
  if (num_seqs < 0 || total_tokens < 0) return fail(GDN_ERR_INVALID_ARG, "%s: negative size", fn);
  if (total_tokens > (int64_t)INT32_MAX / 2) return fail(GDN_ERR_UNSUPPORTED, "%s: too many tokens", fn);
  if (!cache_out) return fail(GDN_ERR_INVALID_ARG, "%s: cache_out is NULL", fn);
  CHECK_PTR(cu_seqlens, "cu_seqlens");
  CHECK_OPT_PTR(h0, "h0");
  CHECK_OPT_PTR(hT, "hT");
  if (hT && (hT == cache_out->s_bnd || hT == cache_out->s_run))
    return fail(GDN_ERR_INVALID_ARG, "%s: hT aliases the cache", fn);
  CHECK_PTR(cache_out->s_bnd, "cache.s_bnd");
  CHECK_PTR(cache_out->s_run, "cache.s_run");
  CHECK_PTR(cache_out->tail_k, "cache.tail_k");
  CHECK_PTR(cache_out->tail_v, "cache.tail_v");
  CHECK_PTR(cache_out->tail_g, "cache.tail_g");
  CHECK_PTR(cache_out->tail_beta, "cache.tail_beta");
  CHECK_PTR(cache_out->tail_len, "cache.tail_len");
  CHECK_PTR(cache_out->run_log_scale, "cache.run_log_scale");
  CHECK_OPT_PTR(cache_out->slot_index, "cache.slot_index");
  if (total_tokens > 0) {
    CHECK_PTR(q, "q");
    CHECK_PTR(k, "k");
    CHECK_PTR(v, "v");
    CHECK_PTR(g, "g");
    CHECK_PTR(beta, "beta");
    CHECK_PTR(o, "o");
  }
  if (num_seqs == 0) {
    g_last_error.clear();
    return GDN_OK;
  }
  const PrefillLayout L = prefill_layout(*shape, num_seqs, total_tokens);
  if (!workspace || workspace_bytes < L.total)
    return fail(GDN_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, L.total,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(GDN_ERR_INVALID_ARG, "%s: workspace is not 16-byte aligned", fn);
  char* ws = (char*)workspace;
  PrefillArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.start = cu_seqlens;
  a.end = cu_seqlens + 1;
  a.skip_empty = 0;
  a.slot = cache_out->slot_index;
  a.h0_slotted = 0;
  a.all_chunks = 0;
  a.h0 = h0;
  a.s_bnd = cache_out->s_bnd;
  a.s_run = cache_out->s_run;
  a.tail_k = cache_out->tail_k;
  a.tail_v = cache_out->tail_v;
  a.tail_g = cache_out->tail_g;
  a.tail_beta = cache_out->tail_beta;
  a.tail_len = cache_out->tail_len;
  a.lgs = cache_out->run_log_scale;
  a.hT = hT;
  a.o = o;
  a.full_base = (int32_t*)(ws + L.full_base);
  a.all_base = (int32_t*)(ws + L.all_base);
  a.prod = (uint8_t*)(ws + L.prod);
  a.gamn = (float*)(ws + L.gamn);
  a.bnd = (float*)(ws + L.bnd);
  a.order = (int32_t*)(ws + L.order);
  a.ready = (int32_t*)(ws + L.ready);
  a.counters = (int32_t*)(ws + L.counters);
  a.N = num_seqs;
  a.H = shape->num_heads;
  a.Hk = key_heads(*shape);
  a.G = a.H / a.Hk;
  a.Cl = shape->chunk;
  return dispatch<PrefillFn>(*shape, a, total_tokens, (hipStream_t)stream, fn);
}

// Checks shared by the two decode entry points; fills every field of `a`
// except the scratch pointers.  *done: nothing to enqueue (num_seqs == 0).
gdn_status decode_prepare(const char* fn, const gdn_cpr_shape* shape, int32_t num_seqs, const void* q, const void* k,
                          const void* v, const void* g, const void* beta, const gdn_cpr_cache* cache, float* hT,
                          void* o, DecodeArgs& a, bool* done) {
  *done = false;
  std::string why;
  if (!shape_ok(shape, &why, true)) return fail(GDN_ERR_UNSUPPORTED, "%s: %s", fn, why.c_str());
  if (num_seqs < 0) return fail(GDN_ERR_INVALID_ARG, "%s: negative size", fn);
  if (!cache) return fail(GDN_ERR_INVALID_ARG, "%s: cache is NULL", fn);
  if (num_seqs == 0) {
    g_last_error.clear();
    *done = true;
    return GDN_OK;
  }
  CHECK_PTR(q, "q");
  CHECK_PTR(k, "k");
  CHECK_PTR(v, "v");
  CHECK_PTR(g, "g");
  CHECK_PTR(beta, "beta");
  CHECK_PTR(o, "o");
  CHECK_PTR(cache->s_bnd, "cache.s_bnd");
  CHECK_PTR(cache->s_run, "cache.s_run");
  CHECK_PTR(cache->tail_k, "cache.tail_k");
  CHECK_PTR(cache->tail_v, "cache.tail_v");
  CHECK_PTR(cache->tail_g, "cache.tail_g");
  CHECK_PTR(cache->tail_beta, "cache.tail_beta");
  CHECK_PTR(cache->tail_len, "cache.tail_len");
  CHECK_PTR(cache->run_log_scale, "cache.run_log_scale");
  CHECK_OPT_PTR(cache->slot_index, "cache.slot_index");
  CHECK_OPT_PTR(hT, "hT");
  if (hT && (hT == cache->s_bnd || hT == cache->s_run)) return fail(GDN_ERR_INVALID_ARG, "%s: hT aliases the cache", fn);
  a = DecodeArgs{};
  a.slot = cache->slot_index;
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.s_bnd = cache->s_bnd;
  a.s_run = cache->s_run;
  a.tail_k = cache->tail_k;
  a.tail_v = cache->tail_v;
  a.tail_g = cache->tail_g;
  a.tail_beta = cache->tail_beta;
  a.tail_len = cache->tail_len;
  a.lgs = cache->run_log_scale;
  a.hT = hT;
  a.o = o;
  a.N = num_seqs;
  a.H = shape->num_heads;
  a.Hk = key_heads(*shape);
  a.G = a.H / a.Hk;
  a.Cl = shape->chunk;
  return GDN_OK;
}

extern "C" gdn_status gdn_cpr_decode_step(const gdn_cpr_shape* shape, int32_t num_seqs, const void* q,
                                          const void* k, const void* v, const void* g, const void* beta,
                                          const gdn_cpr_cache* cache, float* hT, void* o, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  const char* fn = "gdn_cpr_decode_step";
  DecodeArgs a;
  bool done = false;
  const gdn_status r = decode_prepare(fn, shape, num_seqs, q, k, v, g, beta, cache, hT, o, a, &done);
  if (r != GDN_OK || done) return r;
  const DecodeLayout L = decode_layout(*shape, num_seqs);
  if (!workspace || workspace_bytes < L.total)
    return fail(GDN_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, L.total,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(GDN_ERR_INVALID_ARG, "%s: workspace is not 16-byte aligned", fn);
  char* ws = (char*)workspace;
  a.flag = (int32_t*)(ws + L.flag);
  a.prod = (uint8_t*)(ws + L.prod);
  a.gamn = (float*)(ws + L.gamn);
  return dispatch<DecodeFn>(*shape, a, (int)num_seqs, (hipStream_t)stream, fn);
}

// ---------------------------------------------------------------------------
// The decode step for callers that cannot allocate device memory: its
// scratch (per-pair resync flags, then per-slot Gamma_n and chunk products)
// is one fixed array per device, resolved once per device with
// hipGetSymbolAddress.  Host code uses only the resolved address; the
// array's name is not a device address on the host.

constexpr size_t kNoAllocMaxPairs = size_t(1) << 16;             // (sequence, head) pairs per call
constexpr size_t kNoAllocFlagBytes = kNoAllocMaxPairs * sizeof(int32_t);
constexpr size_t kNoAllocProdBytes = size_t(64) << 20;            // product slots of one resync group
constexpr size_t kNoAllocScratchBytes = 2 * kNoAllocFlagBytes + kNoAllocProdBytes;
static_assert(kNoAllocMaxPairs == GDN_NOALLOC_MAX_PAIRS && kNoAllocScratchBytes == GDN_NOALLOC_SCRATCH_BYTES,
              "the header states the fixed scratch's limits");
static_assert(kNoAllocProdBytes / prod_slot_bytes(true, 64, 64) * sizeof(float) <= kNoAllocFlagBytes,
              "the Gamma_n region holds one float per product slot of the smallest shape");

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
uint8_t* g_scratch_ptr[kMaxScratchDevices];

// The device that work enqueued on `stream` runs on.
gdn_status stream_device(hipStream_t stream, int* dev, const char* fn) {
  const hipError_t e = stream ? hipStreamGetDevice(stream, dev) : hipGetDevice(dev);
  if (e != hipSuccess) return fail(GDN_ERR_HIP, "%s: device of the stream: %s", fn, hipGetErrorString(e));
  if (*dev < 0 || *dev >= kMaxScratchDevices) return fail(GDN_ERR_UNSUPPORTED, "%s: device %d", fn, *dev);
  return GDN_OK;
}

// This device's copy of `scratch`, looked up on first use with the device current.
gdn_status scratch_of(int dev, uint8_t** out, const char* fn) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "%s: selecting device %d: %s", fn, dev, hipGetErrorString(e));
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || !p)
      return fail(GDN_ERR_HIP, "%s: address of the scratch array on device %d: %s", fn, dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = (uint8_t*)p;
  }
  *out = g_scratch_ptr[dev];
  return GDN_OK;
}

extern "C" gdn_status gdn_cpr_decode_step_noalloc(const gdn_cpr_shape* shape, int32_t num_seqs, const void* q,
                                                  const void* k, const void* v, const void* g, const void* beta,
                                                  const gdn_cpr_cache* cache, float* hT, void* o, void* stream) {
  const char* fn = "gdn_cpr_decode_step_noalloc";
  DecodeArgs a;
  bool done = false;
  gdn_status r = decode_prepare(fn, shape, num_seqs, q, k, v, g, beta, cache, hT, o, a, &done);
  if (r != GDN_OK || done) return r;
  const size_t pairs = (size_t)num_seqs * (size_t)shape->num_heads;
  if (pairs > kNoAllocMaxPairs)
    return fail(GDN_ERR_UNSUPPORTED, "%s: %zu (sequence, head) pairs; the fixed scratch holds flags for at most %zu",
                fn, pairs, kNoAllocMaxPairs);
  const size_t slots = kNoAllocProdBytes / prod_slot_bytes(shape->dtype == GDN_DTYPE_BF16, shape->head_dim_k,
                                                           shape->head_dim_v);
  const size_t group = slots / (size_t)shape->num_heads;  // sequences per resync launch
  if (group == 0)
    return fail(GDN_ERR_UNSUPPORTED, "%s: %d heads; the fixed scratch holds chunk products for at most %zu", fn,
                shape->num_heads, slots);
  int dev = -1;
  r = stream_device((hipStream_t)stream, &dev, fn);
  if (r != GDN_OK) return r;
  uint8_t* base = nullptr;
  r = scratch_of(dev, &base, fn);
  if (r != GDN_OK) return r;
  a.flag = (int32_t*)base;
  a.gamn = (float*)(base + kNoAllocFlagBytes);
  a.prod = base + 2 * kNoAllocFlagBytes;
  return dispatch<DecodeFn>(*shape, a, (int)std::min<size_t>(group, (size_t)num_seqs), (hipStream_t)stream, fn);
}

extern "C" gdn_status gdn_cpr_prefill_continue(const gdn_cpr_shape* shape, int32_t num_seqs, int64_t total_tokens,
                                               const void* q, const void* k, const void* v, const void* g,
                                               const void* beta, const int32_t* cu_seqlens, const gdn_cpr_cache* cache,
                                               float* hT, void* o, void* workspace, size_t workspace_bytes,
                                               void* stream) {
  const char* fn = "gdn_cpr_prefill_continue";
  std::string why;
  if (!shape_ok(shape, &why, true)) return fail(GDN_ERR_UNSUPPORTED, "%s: %s", fn, why.c_str());
  if (num_seqs < 0 || total_tokens < 0) return fail(GDN_ERR_INVALID_ARG, "%s: negative size", fn);
  if (total_tokens > (int64_t)INT32_MAX / 2) return fail(GDN_ERR_UNSUPPORTED, "%s: too many tokens", fn);
  if (!cache) return fail(GDN_ERR_INVALID_ARG, "%s: cache is NULL", fn);
  CHECK_PTR(cu_seqlens, "cu_seqlens");
  CHECK_PTR(cache->s_bnd, "cache.s_bnd");
  CHECK_PTR(cache->s_run, "cache.s_run");
  CHECK_PTR(cache->tail_k, "cache.tail_k");
  CHECK_PTR(cache->tail_v, "cache.tail_v");
  CHECK_PTR(cache->tail_g, "cache.tail_g");
  CHECK_PTR(cache->tail_beta, "cache.tail_beta");
  CHECK_PTR(cache->tail_len, "cache.tail_len");
  CHECK_PTR(cache->run_log_scale, "cache.run_log_scale");
  CHECK_OPT_PTR(cache->slot_index, "cache.slot_index");
  CHECK_OPT_PTR(hT, "hT");
  if (hT && (hT == cache->s_bnd || hT == cache->s_run)) return fail(GDN_ERR_INVALID_ARG, "%s: hT aliases the cache", fn);
  if (total_tokens > 0) {
    CHECK_PTR(q, "q");
    CHECK_PTR(k, "k");
    CHECK_PTR(v, "v");
    CHECK_PTR(g, "g");
    CHECK_PTR(beta, "beta");
    CHECK_PTR(o, "o");
  }
  if (num_seqs == 0) {
    g_last_error.clear();
    return GDN_OK;
  }
  const ContLayout L = cont_layout(*shape, num_seqs, total_tokens);
  if (!workspace || workspace_bytes < L.total)
    return fail(GDN_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, L.total,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(GDN_ERR_INVALID_ARG, "%s: workspace is not 16-byte aligned", fn);
  char* ws = (char*)workspace;
  char* wd = ws + L.dec_off;
  int32_t* body_start = (int32_t*)(ws + L.body_start);
  ContArgs ca{};
  ca.slot = cache->slot_index;
  ca.q = q;
  ca.k = k;
  ca.v = v;
  ca.g = g;
  ca.beta = beta;
  ca.cu = cu_seqlens;
  ca.s_run = cache->s_run;
  ca.tail_k = cache->tail_k;
  ca.tail_v = cache->tail_v;
  ca.tail_g = cache->tail_g;
  ca.tail_beta = cache->tail_beta;
  ca.tail_len = cache->tail_len;
  ca.lgs = cache->run_log_scale;
  ca.hT = hT;
  ca.o = o;
  ca.flag = (int32_t*)(wd + L.dec.flag);
  ca.body_start = body_start;
  ca.N = num_seqs;
  ca.H = shape->num_heads;
  ca.Hk = key_heads(*shape);
  ca.G = ca.H / ca.Hk;
  ca.Cl = shape->chunk;
  DecodeArgs da{};
  memset(&da, 0, sizeof(da));
  da.s_bnd = cache->s_bnd;
  da.s_run = cache->s_run;
  da.tail_k = cache->tail_k;
  da.tail_v = cache->tail_v;
  da.tail_g = cache->tail_g;
  da.tail_beta = cache->tail_beta;
  da.tail_len = cache->tail_len;
  da.lgs = cache->run_log_scale;
  da.hT = hT;
  da.flag = ca.flag;
  da.prod = (uint8_t*)(wd + L.dec.prod);
  da.gamn = (float*)(wd + L.dec.gamn);
  da.N = num_seqs;
  da.H = shape->num_heads;
  da.Hk = key_heads(*shape);
  da.G = da.H / da.Hk;
  da.Cl = shape->chunk;
  da.slot = cache->slot_index;
  PrefillArgs pa{};
  pa.q = q;
  pa.k = k;
  pa.v = v;
  pa.g = g;
  pa.beta = beta;
  pa.start = body_start;
  pa.end = cu_seqlens + 1;
  pa.skip_empty = 1;
  pa.slot = cache->slot_index;
  pa.h0_slotted = 1;
  pa.all_chunks = 0;
  pa.h0 = cache->s_bnd;  // the boundary the body starts from (aliases the output, as allowed)
  pa.s_bnd = cache->s_bnd;
  pa.s_run = cache->s_run;
  pa.tail_k = cache->tail_k;
  pa.tail_v = cache->tail_v;
  pa.tail_g = cache->tail_g;
  pa.tail_beta = cache->tail_beta;
  pa.tail_len = cache->tail_len;
  pa.lgs = cache->run_log_scale;
  pa.hT = hT;
  pa.o = o;
  pa.full_base = (int32_t*)(ws + L.pre.full_base);
  pa.all_base = (int32_t*)(ws + L.pre.all_base);
  pa.prod = (uint8_t*)(ws + L.pre.prod);
  pa.gamn = (float*)(ws + L.pre.gamn);
  pa.bnd = (float*)(ws + L.pre.bnd);
  pa.order = (int32_t*)(ws + L.pre.order);
  pa.ready = (int32_t*)(ws + L.pre.ready);
  pa.counters = (int32_t*)(ws + L.pre.counters);
  pa.N = num_seqs;
  pa.H = shape->num_heads;
  pa.Hk = key_heads(*shape);
  pa.G = pa.H / pa.Hk;
  pa.Cl = shape->chunk;
  return dispatch<ContFn>(*shape, ca, da, pa, total_tokens, (hipStream_t)stream, fn);
}

extern "C" gdn_status gdn_cpr_fwd_bwd(const gdn_cpr_shape* shape, int32_t num_seqs, int64_t total_tokens,
                                      const void* q, const void* k, const void* v, const void* g,
                                      const void* beta, const int32_t* cu_seqlens, const float* h0,
                                      const void* d_o, const float* d_hT, void* o, float* hT, void* dq,
                                      void* dk, void* dv, float* dg, float* dbeta, float* dh0,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "gdn_cpr_fwd_bwd";
  std::string why;
  if (!shape_ok(shape, &why)) return fail(GDN_ERR_UNSUPPORTED, "%s: %s", fn, why.c_str());
  if (num_seqs < 0 || total_tokens < 0) return fail(GDN_ERR_INVALID_ARG, "%s: negative size", fn);
  if (total_tokens > (int64_t)INT32_MAX / 2) return fail(GDN_ERR_UNSUPPORTED, "%s: too many tokens", fn);
  CHECK_PTR(cu_seqlens, "cu_seqlens");
  CHECK_OPT_PTR(h0, "h0");
  CHECK_OPT_PTR(d_hT, "d_hT");
  CHECK_OPT_PTR(hT, "hT");
  CHECK_OPT_PTR(dh0, "dh0");
  if (total_tokens > 0) {
    CHECK_PTR(q, "q");
    CHECK_PTR(k, "k");
    CHECK_PTR(v, "v");
    CHECK_PTR(g, "g");
    CHECK_PTR(beta, "beta");
    CHECK_PTR(d_o, "d_o");
    CHECK_PTR(o, "o");
    CHECK_PTR(dq, "dq");
    CHECK_PTR(dk, "dk");
    CHECK_PTR(dv, "dv");
    CHECK_PTR(dg, "dg");
    CHECK_PTR(dbeta, "dbeta");
  }
  if (num_seqs == 0) {
    g_last_error.clear();
    return GDN_OK;
  }
  const FwdBwdLayout L = fwd_bwd_layout(*shape, num_seqs, total_tokens);
  if (!workspace || workspace_bytes < L.total)
    return fail(GDN_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, L.total,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(GDN_ERR_INVALID_ARG, "%s: workspace is not 16-byte aligned", fn);
  char* ws = (char*)workspace;
  PrefillArgs pa{};
  pa.q = q;
  pa.k = k;
  pa.v = v;
  pa.g = g;
  pa.beta = beta;
  pa.start = cu_seqlens;
  pa.end = cu_seqlens + 1;
  pa.skip_empty = 0;
  pa.slot = nullptr;
  pa.h0_slotted = 0;
  pa.all_chunks = 0;
  pa.h0 = h0;
  pa.s_bnd = (float*)(ws + L.s_bnd);
  pa.s_run = (float*)(ws + L.s_run);
  pa.tail_k = ws + L.tail_k;
  pa.tail_v = ws + L.tail_v;
  pa.tail_g = ws + L.tail_g;
  pa.tail_beta = ws + L.tail_b;
  pa.tail_len = (int32_t*)(ws + L.tail_len);
  pa.lgs = nullptr;
  pa.hT = hT;
  pa.o = o;
  pa.full_base = (int32_t*)(ws + L.pre.full_base);
  pa.all_base = (int32_t*)(ws + L.pre.all_base);
  pa.prod = (uint8_t*)(ws + L.pre.prod);
  pa.gamn = (float*)(ws + L.pre.gamn);
  pa.bnd = (float*)(ws + L.pre.bnd);
  pa.order = (int32_t*)(ws + L.pre.order);
  pa.ready = (int32_t*)(ws + L.pre.ready);
  pa.counters = (int32_t*)(ws + L.pre.counters);
  pa.N = num_seqs;
  pa.H = shape->num_heads;
  pa.Hk = key_heads(*shape);
  pa.G = pa.H / pa.Hk;
  pa.Cl = shape->chunk;
  BwdArgs ba;
  ba.q = q;
  ba.k = k;
  ba.v = v;
  ba.g = g;
  ba.beta = beta;
  ba.d_o = d_o;
  ba.cu = cu_seqlens;
  ba.all_base = pa.all_base;
  ba.bnd = pa.bnd;
  ba.d_hT = d_hT;
  ba.ws = (uint8_t*)(ws + L.bslots);
  ba.gamn = (float*)(ws + L.bgamn);
  ba.dq = dq;
  ba.dk = dk;
  ba.dv = dv;
  ba.dg = dg;
  ba.dbeta = dbeta;
  ba.dh0 = dh0;
  ba.dq_part = L.dq_part ? (float*)(ws + L.dq_part) : nullptr;
  ba.dk_part = L.dk_part ? (float*)(ws + L.dk_part) : nullptr;
  ba.N = num_seqs;
  ba.H = shape->num_heads;
  ba.Hk = key_heads(*shape);
  ba.G = ba.H / ba.Hk;
  ba.Cl = shape->chunk;
  return dispatch<FwdBwdFn>(*shape, pa, ba, total_tokens, L.slot, (hipStream_t)stream, fn);
}

extern "C" size_t gdn_cmp_workspace_size(const gdn_cpr_shape* shape, int32_t mode, int32_t num_seqs,
                                         int64_t total_tokens) {
  std::string why;
  if (!shape_ok(shape, &why) || num_seqs < 0 || total_tokens < 0 || shape->chunk != C) return 0;
  if (mode == GDN_CMP_RECURRENT) return 256;
  if (mode == GDN_CMP_CHUNKWISE) return cmp_layout(*shape, num_seqs, total_tokens).total;
  return 0;
}

extern "C" gdn_status gdn_cmp_prefill(const gdn_cpr_shape* shape, int32_t mode, int32_t num_seqs, int64_t total_tokens,
                                      const void* q, const void* k, const void* v, const void* g, const void* beta,
                                      const int32_t* cu_seqlens, const float* h0, float* state_out, void* o,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "gdn_cmp_prefill";
  std::string why;
  if (!shape_ok(shape, &why)) return fail(GDN_ERR_UNSUPPORTED, "%s: %s", fn, why.c_str());
  if (shape->chunk != C) return fail(GDN_ERR_UNSUPPORTED, "%s: the comparators take chunk = 64 only", fn);
  if (shape->dtype != GDN_DTYPE_BF16) return fail(GDN_ERR_UNSUPPORTED, "%s: the comparators take bf16 inputs", fn);
  if (mode != GDN_CMP_RECURRENT && mode != GDN_CMP_CHUNKWISE) return fail(GDN_ERR_INVALID_ARG, "%s: mode", fn);
  if (num_seqs < 0 || total_tokens < 0) return fail(GDN_ERR_INVALID_ARG, "%s: negative size", fn);
  if (total_tokens > (int64_t)INT32_MAX / 2) return fail(GDN_ERR_UNSUPPORTED, "%s: too many tokens", fn);
  CHECK_PTR(cu_seqlens, "cu_seqlens");
  CHECK_OPT_PTR(h0, "h0");
  CHECK_PTR(state_out, "state_out");
  if (total_tokens > 0) {
    CHECK_PTR(q, "q");
    CHECK_PTR(k, "k");
    CHECK_PTR(v, "v");
    CHECK_PTR(g, "g");
    CHECK_PTR(beta, "beta");
    CHECK_PTR(o, "o");
  }
  if (num_seqs == 0) {
    g_last_error.clear();
    return GDN_OK;
  }
  const size_t need = gdn_cmp_workspace_size(shape, mode, num_seqs, total_tokens);
  if (!workspace || workspace_bytes < need)
    return fail(GDN_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(GDN_ERR_INVALID_ARG, "%s: workspace is not 16-byte aligned", fn);
  char* ws = (char*)workspace;
  const CmpLayout L = cmp_layout(*shape, num_seqs, total_tokens);
  CmpArgs ca;
  memset(&ca, 0, sizeof(ca));
  ca.q = q;
  ca.k = k;
  ca.v = v;
  ca.g = g;
  ca.beta = beta;
  ca.cu = cu_seqlens;
  ca.h0 = h0;
  ca.state = state_out;
  ca.o = o;
  ca.N = num_seqs;
  ca.H = shape->num_heads;
  ca.Hk = key_heads(*shape);
  ca.G = ca.H / ca.Hk;
  PrefillArgs pa{};
  memset(&pa, 0, sizeof(pa));
  if (mode == GDN_CMP_CHUNKWISE) {
    ca.all_base = (int32_t*)(ws + L.all_base);
    ca.prod = (uint8_t*)(ws + L.prod);
    ca.gamn = (float*)(ws + L.gamn);
    ca.bnd = (float*)(ws + L.bnd);
    pa.start = cu_seqlens;
    pa.end = cu_seqlens + 1;
    pa.all_chunks = 1;
    pa.h0 = h0;
    pa.s_bnd = state_out;
    pa.full_base = (int32_t*)(ws + L.full_base);
    pa.all_base = ca.all_base;
    pa.prod = ca.prod;
    pa.gamn = ca.gamn;
    pa.bnd = ca.bnd;
    pa.N = num_seqs;
    pa.H = shape->num_heads;
    pa.Hk = key_heads(*shape);
    pa.G = pa.H / pa.Hk;
    pa.Cl = shape->chunk;
  }
  return dispatch<CmpPrefillFn>(*shape, (int)mode, ca, pa, total_tokens, (hipStream_t)stream, fn);
}

extern "C" gdn_status gdn_cmp_decode_step(const gdn_cpr_shape* shape, int32_t num_seqs, const void* q,
                                          const void* k, const void* v, const void* g, const void* beta,
                                          float* state, void* o, void* stream) {
  const char* fn = "gdn_cmp_decode_step";
  std::string why;
  if (!shape_ok(shape, &why)) return fail(GDN_ERR_UNSUPPORTED, "%s: %s", fn, why.c_str());
  if (shape->chunk != C) return fail(GDN_ERR_UNSUPPORTED, "%s: the comparators take chunk = 64 only", fn);
  if (num_seqs < 0) return fail(GDN_ERR_INVALID_ARG, "%s: negative size", fn);
  if (num_seqs == 0) {
    g_last_error.clear();
    return GDN_OK;
  }
  CHECK_PTR(q, "q");
  CHECK_PTR(k, "k");
  CHECK_PTR(v, "v");
  CHECK_PTR(g, "g");
  CHECK_PTR(beta, "beta");
  CHECK_PTR(o, "o");
  CHECK_PTR(state, "state");
  CmpArgs ca;
  memset(&ca, 0, sizeof(ca));
  ca.q = q;
  ca.k = k;
  ca.v = v;
  ca.g = g;
  ca.beta = beta;
  ca.state = state;
  ca.o = o;
  ca.N = num_seqs;
  ca.H = shape->num_heads;
  ca.Hk = key_heads(*shape);
  ca.G = ca.H / ca.Hk;
  return dispatch<CmpDecodeFn>(*shape, ca, (hipStream_t)stream, fn);
}

extern "C" gdn_status gdn_cmp_chunk_decode_step(const gdn_cpr_shape* shape, int32_t num_seqs, const void* q,
                                                const void* k, const void* v, const void* g, const void* beta,
                                                const gdn_cpr_cache* cache, void* o, void* workspace,
                                                size_t workspace_bytes, void* stream) {
  const char* fn = "gdn_cmp_chunk_decode_step";
  std::string why;
  if (!shape_ok(shape, &why)) return fail(GDN_ERR_UNSUPPORTED, "%s: %s", fn, why.c_str());
  if (shape->chunk != C) return fail(GDN_ERR_UNSUPPORTED, "%s: the comparators take chunk = 64 only", fn);
  if (shape->dtype != GDN_DTYPE_BF16) return fail(GDN_ERR_UNSUPPORTED, "%s: the comparators take bf16 inputs", fn);
  if (num_seqs < 0) return fail(GDN_ERR_INVALID_ARG, "%s: negative size", fn);
  if (!cache) return fail(GDN_ERR_INVALID_ARG, "%s: cache is NULL", fn);
  if (num_seqs == 0) {
    g_last_error.clear();
    return GDN_OK;
  }
  CHECK_PTR(q, "q");
  CHECK_PTR(k, "k");
  CHECK_PTR(v, "v");
  CHECK_PTR(g, "g");
  CHECK_PTR(beta, "beta");
  CHECK_PTR(o, "o");
  CHECK_PTR(cache->s_bnd, "cache.s_bnd");
  CHECK_PTR(cache->s_run, "cache.s_run");
  CHECK_PTR(cache->tail_k, "cache.tail_k");
  CHECK_PTR(cache->tail_v, "cache.tail_v");
  CHECK_PTR(cache->tail_g, "cache.tail_g");
  CHECK_PTR(cache->tail_beta, "cache.tail_beta");
  CHECK_PTR(cache->tail_len, "cache.tail_len");
  CHECK_PTR(cache->run_log_scale, "cache.run_log_scale");
  CHECK_OPT_PTR(cache->slot_index, "cache.slot_index");
  const DecodeLayout L = decode_layout(*shape, num_seqs);
  if (!workspace || workspace_bytes < L.total)
    return fail(GDN_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, L.total,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(GDN_ERR_INVALID_ARG, "%s: workspace is not 16-byte aligned", fn);
  char* ws = (char*)workspace;
  DecodeArgs a{};
  a.slot = cache->slot_index;
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.s_bnd = cache->s_bnd;
  a.s_run = cache->s_run;
  a.tail_k = cache->tail_k;
  a.tail_v = cache->tail_v;
  a.tail_g = cache->tail_g;
  a.tail_beta = cache->tail_beta;
  a.tail_len = cache->tail_len;
  a.lgs = cache->run_log_scale;
  a.o = o;
  a.flag = (int32_t*)(ws + L.flag);
  a.prod = (uint8_t*)(ws + L.prod);
  a.gamn = (float*)(ws + L.gamn);
  a.N = num_seqs;
  a.H = shape->num_heads;
  a.Hk = key_heads(*shape);
  a.G = a.H / a.Hk;
  a.Cl = shape->chunk;
  return dispatch<CmpChunkDecodeFn>(*shape, a, (hipStream_t)stream, fn);
}

extern "C" gdn_status gdn_cpr_cache_state(const gdn_cpr_shape* shape, int32_t num_seqs, const gdn_cpr_cache* cache,
                                          float* state_out, void* stream) {
  const char* fn = "gdn_cpr_cache_state";
  std::string why;
  if (!shape_ok(shape, &why, true)) return fail(GDN_ERR_UNSUPPORTED, "%s: %s", fn, why.c_str());
  if (num_seqs < 0) return fail(GDN_ERR_INVALID_ARG, "%s: negative size", fn);
  if (!cache) return fail(GDN_ERR_INVALID_ARG, "%s: cache is NULL", fn);
  if (num_seqs == 0) {
    g_last_error.clear();
    return GDN_OK;
  }
  CHECK_PTR(cache->s_run, "cache.s_run");
  CHECK_PTR(cache->run_log_scale, "cache.run_log_scale");
  CHECK_OPT_PTR(cache->slot_index, "cache.slot_index");
  CHECK_PTR(state_out, "state_out");
  if (state_out == cache->s_run) return fail(GDN_ERR_INVALID_ARG, "%s: state_out aliases cache.s_run", fn);
  const int SS4 = shape->head_dim_k * shape->head_dim_v / 4;
  hipLaunchKernelGGL(k_cache_state, dim3(num_seqs, shape->num_heads), dim3(256), 0, (hipStream_t)stream,
                     cache->s_run, cache->run_log_scale, cache->slot_index, state_out, shape->num_heads, SS4);
  return launch_status(fn);
}

extern "C" void gdn_cpr_set_stage_events(void* const* events, int32_t n_events) {
  g_events = (events && n_events > 0) ? events : nullptr;
  g_n_events = g_events ? n_events : 0;
}

extern "C" const char* gdn_cpr_last_error(void) { return g_last_error.c_str(); }

extern "C" const char* gdn_cpr_numerics_id(void) {
  return "gdn_cpr numerics v7: "
         "per-token step (one routine for the prefill scan, decode and the continuation head; k and q by DPP "
         "row broadcast) in fp32 on a scaled running state M = exp(lg) N: x = lg + g (fp32 add); "
         "renorm = x < -32; c = exp(x); b = beta * r with r = exp(-x), r = 1 when renorm; renorm: N = c N, "
         "c = 1; lg after the token = 0 when renorm, else x; lane j (state column j); every accumulator "
         "starts with the product of its first term (p_i = k[i] * N[i] for i < 4, o_i = q[i] * N[i] for "
         "i < 2), then "
         "pass A, i ascending: p_(i mod 4) = fma(k[i], N[i], p_(i mod 4)); "
         "w = b * (v - c * ((p_0 + p_1) + (p_2 + p_3))); "
         "pass B, i ascending: N[i] = fma(k[i], w, N[i]); o_(i mod 2) = fma(q[i], N[i], o_(i mod 2)); "
         "o = c * (o_0 + o_1); "
         "d_k = 256 (bf16 inputs): lanes j and j + 32 hold keys 0..127 and 128..255 of column j and run the "
         "passes over their half with P = (p_0 + p_1) + (p_2 + p_3) and O = o_0 + o_1 per half; "
         "w = b * (v - c * (P_lo + P_hi)); o = c * (O_lo + O_hi); "
         "final state = exp(lg) * N elementwise; exp = ocml expf; "
         "gamma = left-to-right fp32 cumsum of g; "
         "fp32 inputs: chunk products and boundary chain fp32 VALU with ascending explicit-fma sums and "
         "column-wise forward substitution; bf16 inputs: G, W^T, U and the boundary chain on "
         "v_mfma_f32_16x16x32_bf16 (k slots k0+4g+{0..3}, k0+16+4g+{0..3}; k steps ascending) with bf16 "
         "T diag(Gamma), T, K~, S, Delta operands and fp32 accumulation; (I+L)^-1 by 16x16 blocks: "
         "diagonal blocks by fp32 forward substitution (ascending pivots), blocks below by "
         "v_mfma_f32_16x16x4_f32 (Y = sum_k L_Bk X_kj, k ascending; X_Bj = -X_BB Y); T = X diag(beta) "
         "rounded once per product; bf16 outputs round-to-nearest-even; "
         "C in {16, 32, 64}: a chunk of C < 64 tokens is a 64-row chunk whose rows past C are identity "
         "steps (k = v = 0, g = beta = 0)";
}
