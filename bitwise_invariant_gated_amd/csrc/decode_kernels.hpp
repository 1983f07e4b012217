// Decode kernels: the decode step, the cache read-out and the continuation head.
//
// Part of libgdn_cpr (included by gdn_cpr.hip, in this order: prefill_kernels.hpp,
// decode_kernels.hpp, comparator_kernels.hpp, backward_kernels.hpp).
#pragma once

#include "prefill_kernels.hpp"

namespace {

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


}  // namespace
