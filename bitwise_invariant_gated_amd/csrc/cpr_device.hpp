// Device routines of the CPR Gated DeltaNet layer for gfx950.
//
// Every quantity that must round identically in prefill and decode is
// computed by exactly one routine in this file:
//   token_step        the per-token recurrence on one state column of the
//                     scaled running state (with its scalars from
//                     token_scale, step_factors and scale_after); the
//                     prefill scan (scan_tokens), the decode step and the
//                     continuation head all call this one function, each
//                     delivering k and q to it the same way (DPP row
//                     broadcast from a 16-byte slice per lane)
//   chunk_local_bf16  chunk products W, U, K~^T, Gamma_n of one chunk
//   chunk_local_f32   (prefill's chunk pass and decode's resync call them)
//   chain_step_bf16   boundary advance S' = Gamma_n S + K~^T (U - W S)
//   chain_step_f32    (prefill's boundary chain and decode's resync call them)
// The pages that describe the method (IsoExec, section "Chunkwise-Parallel
// Recurrent (CPR) Gated DeltaNet"; the Chinese page's section on a third way
// for Gated DeltaNet) fix only the structure: boundary states by the chunk
// form, then the recurrence inside every chunk from those boundaries, and
// decode resynchronising every C tokens, so that the three stages share one
// rounding rhythm.  The rounding choices below are this library's own; they
// are fixed (explicit FMAs, no contraction, fixed loop orders) so that every
// caller reproduces them bit for bit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace cpr {

constexpr int kChunk = 64;  // C
constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// storage dtypes

struct Bf16 {
  typedef uint16_t T;
  __device__ static __forceinline__ float load(const T* p, size_t i) {
    return __uint_as_float((uint32_t)p[i] << 16);
  }
  __device__ static __forceinline__ void store(T* p, size_t i, float x) { p[i] = round(x); }
  // fp32 -> bf16, round to nearest even (gfx950 v_cvt_pk_bf16_f32: branch
  // free, IEEE RNE for every non-NaN input; NaN stays NaN).
  __device__ static __forceinline__ uint16_t round(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
  // the element's bits as loaded, decoded later (load() = from_bits(load_bits()))
  __device__ static __forceinline__ uint32_t load_bits(const T* p, size_t i) { return p[i]; }
  __device__ static __forceinline__ float from_bits(uint32_t b) { return __uint_as_float(b << 16); }
};

struct F32 {
  typedef float T;
  __device__ static __forceinline__ float load(const T* p, size_t i) { return p[i]; }
  __device__ static __forceinline__ void store(T* p, size_t i, float x) { p[i] = x; }
  __device__ static __forceinline__ uint32_t load_bits(const T* p, size_t i) { return __float_as_uint(p[i]); }
  __device__ static __forceinline__ float from_bits(uint32_t b) { return __uint_as_float(b); }
};

// Buffer resource over [base, base + bytes) for raw (unformatted) buffer
// loads and stores: the address is the wave-uniform base plus a 32-bit
// scalar offset plus a 32-bit lane offset, so a per-lane access pattern
// costs one VGPR, and the hardware drops any access past `bytes`.
// Dword 3 is the gfx9 raw-buffer format word.
typedef __amdgpu_buffer_rsrc_t BufRsrc;
__device__ __forceinline__ BufRsrc buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// A lane's part of one state column of a [rows][DV] fp32 state at `base`:
// rows k0 .. k0 + KL - 1 of column col, through one buffer resource, so the
// lane offset is one VGPR and every row offset is a wave-uniform constant
// (no 64-bit address per row).
template <int KL, int DV>
__device__ __forceinline__ void load_state_col(float (&s)[KL], const float* base, uint32_t bytes, int k0, int col) {
  const BufRsrc r = buf_rsrc(base, bytes);
  const uint32_t off = (uint32_t)(k0 * DV + col) * 4u;
#pragma unroll
  for (int ii = 0; ii < KL; ++ii)
    s[ii] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, ii * DV * 4, 0));
}

// stores scale * s (scale = 1: s itself; the product is exact then)
template <int KL, int DV>
__device__ __forceinline__ void store_state_col(float* base, uint32_t bytes, const float (&s)[KL], int k0, int col,
                                                float scale) {
  const BufRsrc r = buf_rsrc(base, bytes);
  const uint32_t off = (uint32_t)(k0 * DV + col) * 4u;
#pragma unroll
  for (int ii = 0; ii < KL; ++ii)
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(scale * s[ii]), r, off, ii * DV * 4, 0);
}

__device__ __forceinline__ float lane_bcast(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

// ---------------------------------------------------------------------------
// Operand delivery of the per-token steps: DPP row broadcast.
//
// Every lane 16 r + c holds elements 8c .. 8c+7 of the token's k and q rows
// (each 16-lane row of the wave holds a full copy; for d_k = 64 lanes c >= 8
// repeat slot c - 8), and v_fmac_f32_dpp with row_newbcast:c reads element
// 8c + e from lane c of the lane's own row.  So every lane (one state column)
// sees every element of k and q without scalar loads, whose cache misses
// stall the wave.
//
// Hazard: a DPP instruction must not read, as its DPP source, a VGPR written
// by a VALU instruction in the two preceding cycles.  The unpacked k and q
// values pass through an s_nop 1 before each pass, and the build checks the
// ISA for any remaining DPP-source write within two instructions.
#define CPR_FMAC_BCAST_CASE(N)                                                                  \
  if constexpr (I == N)                                                                          \
    asm volatile("v_fmac_f32_dpp %0, %1, %2 row_newbcast:" #N " row_mask:0xf bank_mask:0xf"      \
                 : "+v"(acc)                                                                     \
                 : "v"(src), "v"(x));
// acc += src[lane 16 r + I of this lane's row] * x
template <int I>
__device__ __forceinline__ void fmac_bcast(float& acc, float src, float x) {
  static_assert(I >= 0 && I < 16, "row_newbcast selects one of 16 lanes");
  CPR_FMAC_BCAST_CASE(0) CPR_FMAC_BCAST_CASE(1) CPR_FMAC_BCAST_CASE(2) CPR_FMAC_BCAST_CASE(3)
  CPR_FMAC_BCAST_CASE(4) CPR_FMAC_BCAST_CASE(5) CPR_FMAC_BCAST_CASE(6) CPR_FMAC_BCAST_CASE(7)
  CPR_FMAC_BCAST_CASE(8) CPR_FMAC_BCAST_CASE(9) CPR_FMAC_BCAST_CASE(10) CPR_FMAC_BCAST_CASE(11)
  CPR_FMAC_BCAST_CASE(12) CPR_FMAC_BCAST_CASE(13) CPR_FMAC_BCAST_CASE(14) CPR_FMAC_BCAST_CASE(15)
}
#undef CPR_FMAC_BCAST_CASE

#define CPR_MUL_BCAST_CASE(N)                                                                   \
  if constexpr (I == N)                                                                          \
    asm volatile("v_mul_f32_dpp %0, %1, %2 row_newbcast:" #N " row_mask:0xf bank_mask:0xf"       \
                 : "=v"(acc)                                                                     \
                 : "v"(src), "v"(x));
// acc = src[lane 16 r + I of this lane's row] * x (an accumulator's first term)
template <int I>
__device__ __forceinline__ void mul_bcast(float& acc, float src, float x) {
  static_assert(I >= 0 && I < 16, "row_newbcast selects one of 16 lanes");
  CPR_MUL_BCAST_CASE(0) CPR_MUL_BCAST_CASE(1) CPR_MUL_BCAST_CASE(2) CPR_MUL_BCAST_CASE(3)
  CPR_MUL_BCAST_CASE(4) CPR_MUL_BCAST_CASE(5) CPR_MUL_BCAST_CASE(6) CPR_MUL_BCAST_CASE(7)
  CPR_MUL_BCAST_CASE(8) CPR_MUL_BCAST_CASE(9) CPR_MUL_BCAST_CASE(10) CPR_MUL_BCAST_CASE(11)
  CPR_MUL_BCAST_CASE(12) CPR_MUL_BCAST_CASE(13) CPR_MUL_BCAST_CASE(14) CPR_MUL_BCAST_CASE(15)
}
#undef CPR_MUL_BCAST_CASE

// The two passes of token_step as asm statements of 16 keys each.  They hold
// the same DPP multiply-adds, in the same order, as one statement per
// instruction would, but the compiler brackets every inline-asm statement
// that reads a register another one wrote since its last own instruction
// with an s_nop (it cannot see that no 16-bit destination select is
// involved), which cost one issue slot per four multiply-adds.  Within a
// statement no instruction reads, as its DPP source, a register written in
// the statement (the sources are k and q), and an accumulator or state
// element is read at the earliest four instructions after it is written.
#define CPR_DPP(OP, A, S, X, N) #OP " %" #A ", %" #S ", %" #X " row_newbcast:" #N " row_mask:0xf bank_mask:0xf\n"
// pass A, keys 8N .. 8N+7: p_(e mod 4) += k[8N+e] * N[8N+e]; operands
// %0..%3 p_0..p_3, %4..%11 k elements 0..7 of the lane's slot, S0..S7 the keys' N
#define CPR_PA_GROUP(N, S0, S1, S2, S3, S4, S5, S6, S7)                                               \
  CPR_DPP(v_fmac_f32_dpp, 0, 4, S0, N) CPR_DPP(v_fmac_f32_dpp, 1, 5, S1, N)                              \
  CPR_DPP(v_fmac_f32_dpp, 2, 6, S2, N) CPR_DPP(v_fmac_f32_dpp, 3, 7, S3, N)                              \
  CPR_DPP(v_fmac_f32_dpp, 0, 8, S4, N) CPR_DPP(v_fmac_f32_dpp, 1, 9, S5, N)                              \
  CPR_DPP(v_fmac_f32_dpp, 2, 10, S6, N) CPR_DPP(v_fmac_f32_dpp, 3, 11, S7, N)
// keys 0 .. 7: the first four terms start the accumulators
#define CPR_PA_FIRST                                                                                     \
  CPR_DPP(v_mul_f32_dpp, 0, 4, 12, 0) CPR_DPP(v_mul_f32_dpp, 1, 5, 13, 0)                                \
  CPR_DPP(v_mul_f32_dpp, 2, 6, 14, 0) CPR_DPP(v_mul_f32_dpp, 3, 7, 15, 0)                                \
  CPR_DPP(v_fmac_f32_dpp, 0, 8, 16, 0) CPR_DPP(v_fmac_f32_dpp, 1, 9, 17, 0)                              \
  CPR_DPP(v_fmac_f32_dpp, 2, 10, 18, 0) CPR_DPP(v_fmac_f32_dpp, 3, 11, 19, 0)
#define CPR_PA_IN(B)                                                                                     \
  "v"(kf[0]), "v"(kf[1]), "v"(kf[2]), "v"(kf[3]), "v"(kf[4]), "v"(kf[5]), "v"(kf[6]), "v"(kf[7]),        \
      "v"(s[16 * B]), "v"(s[16 * B + 1]), "v"(s[16 * B + 2]), "v"(s[16 * B + 3]), "v"(s[16 * B + 4]),    \
      "v"(s[16 * B + 5]), "v"(s[16 * B + 6]), "v"(s[16 * B + 7]), "v"(s[16 * B + 8]), "v"(s[16 * B + 9]), \
      "v"(s[16 * B + 10]), "v"(s[16 * B + 11]), "v"(s[16 * B + 12]), "v"(s[16 * B + 13]),                \
      "v"(s[16 * B + 14]), "v"(s[16 * B + 15])
#define CPR_PA_CASE(B, N0, N1)                                                                           \
  if constexpr (I == B)                                                                                  \
    asm volatile(CPR_PA_GROUP(N0, 12, 13, 14, 15, 16, 17, 18, 19) CPR_PA_GROUP(N1, 20, 21, 22, 23, 24, 25, 26, 27) \
                 : "+v"(p[0]), "+v"(p[1]), "+v"(p[2]), "+v"(p[3])                                        \
                 : CPR_PA_IN(B));
// pass A over keys 16 I .. 16 I + 15 (the accumulators start at I = 0)
template <int I, int DK>
__device__ __forceinline__ void pass_a_keys16(float (&p)[4], const float (&kf)[8], const float (&s)[DK]) {
  static_assert(I >= 0 && I < 8 && 16 * I + 16 <= DK, "16-key groups of at most 128 keys");
  if constexpr (I == 0)
    asm volatile(CPR_PA_FIRST CPR_PA_GROUP(1, 20, 21, 22, 23, 24, 25, 26, 27)
                 : "=&v"(p[0]), "=&v"(p[1]), "=&v"(p[2]), "=&v"(p[3])
                 : CPR_PA_IN(0));
  CPR_PA_CASE(1, 2, 3) CPR_PA_CASE(2, 4, 5) CPR_PA_CASE(3, 6, 7) CPR_PA_CASE(4, 8, 9)
  CPR_PA_CASE(5, 10, 11) CPR_PA_CASE(6, 12, 13) CPR_PA_CASE(7, 14, 15)
}
#undef CPR_PA_CASE
#undef CPR_PA_IN
#undef CPR_PA_FIRST
#undef CPR_PA_GROUP

// pass B over keys 16 I .. 16 I + 15: for each pair of keys the update
// N[i] += k[i] w, N[i+1] += k[i+1] w, then the output terms of the pair
// before it, o_0 += q[i-2] N[i-2], o_1 += q[i-1] N[i-1].  Operands: %0..%15
// the keys' N, %16 %17 o_0 o_1, %18 %19 N of the two keys before the group,
// %20..%27 k, %28..%35 q elements 0..7 of the lane's slot, %36 w.
#define CPR_PB_U(A, K, N) CPR_DPP(v_fmac_f32_dpp, A, K, 36, N)
#define CPR_PB_O(A, Q, S, N) CPR_DPP(v_fmac_f32_dpp, A, Q, S, N)
#define CPR_PB_TAIL(N0, N1)                                                                              \
  CPR_PB_U(2, 22, N0) CPR_PB_U(3, 23, N0) CPR_PB_O(16, 28, 0, N0) CPR_PB_O(17, 29, 1, N0)               \
  CPR_PB_U(4, 24, N0) CPR_PB_U(5, 25, N0) CPR_PB_O(16, 30, 2, N0) CPR_PB_O(17, 31, 3, N0)               \
  CPR_PB_U(6, 26, N0) CPR_PB_U(7, 27, N0) CPR_PB_O(16, 32, 4, N0) CPR_PB_O(17, 33, 5, N0)               \
  CPR_PB_U(8, 20, N1) CPR_PB_U(9, 21, N1) CPR_PB_O(16, 34, 6, N0) CPR_PB_O(17, 35, 7, N0)               \
  CPR_PB_U(10, 22, N1) CPR_PB_U(11, 23, N1) CPR_PB_O(16, 28, 8, N1) CPR_PB_O(17, 29, 9, N1)             \
  CPR_PB_U(12, 24, N1) CPR_PB_U(13, 25, N1) CPR_PB_O(16, 30, 10, N1) CPR_PB_O(17, 31, 11, N1)           \
  CPR_PB_U(14, 26, N1) CPR_PB_U(15, 27, N1) CPR_PB_O(16, 32, 12, N1) CPR_PB_O(17, 33, 13, N1)
#define CPR_PB_OUT(B)                                                                                    \
  "+v"(s[16 * B]), "+v"(s[16 * B + 1]), "+v"(s[16 * B + 2]), "+v"(s[16 * B + 3]), "+v"(s[16 * B + 4]),   \
      "+v"(s[16 * B + 5]), "+v"(s[16 * B + 6]), "+v"(s[16 * B + 7]), "+v"(s[16 * B + 8]),                \
      "+v"(s[16 * B + 9]), "+v"(s[16 * B + 10]), "+v"(s[16 * B + 11]), "+v"(s[16 * B + 12]),             \
      "+v"(s[16 * B + 13]), "+v"(s[16 * B + 14]), "+v"(s[16 * B + 15])
#define CPR_PB_IN                                                                                        \
  "v"(kf[0]), "v"(kf[1]), "v"(kf[2]), "v"(kf[3]), "v"(kf[4]), "v"(kf[5]), "v"(kf[6]), "v"(kf[7]),        \
      "v"(qf[0]), "v"(qf[1]), "v"(qf[2]), "v"(qf[3]), "v"(qf[4]), "v"(qf[5]), "v"(qf[6]), "v"(qf[7]), "v"(w)
#define CPR_PB_CASE(B, NP, N0, N1)                                                                       \
  if constexpr (I == B)                                                                                  \
    asm volatile(CPR_PB_U(0, 20, N0) CPR_PB_U(1, 21, N0) CPR_PB_O(16, 34, 18, NP) CPR_PB_O(17, 35, 19, NP) \
                     CPR_PB_TAIL(N0, N1)                                                                 \
                 : CPR_PB_OUT(B), "+v"(o[0]), "+v"(o[1])                                                  \
                 : "v"(s[16 * B - 2]), "v"(s[16 * B - 1]), CPR_PB_IN);
template <int I, int DK>
__device__ __forceinline__ void pass_b_keys16(float (&s)[DK], float (&o)[2], const float (&kf)[8], const float (&qf)[8],
                                              float w) {
  static_assert(I >= 0 && I < 8 && 16 * I + 16 <= DK, "16-key groups of at most 128 keys");
  // keys 0, 1 have no pair before them; keys 2, 3's output terms start o_0, o_1
  // (%18 %19 are unused here)
  if constexpr (I == 0)
    asm volatile(CPR_PB_U(0, 20, 0) CPR_PB_U(1, 21, 0) CPR_PB_U(2, 22, 0) CPR_PB_U(3, 23, 0)
                     CPR_DPP(v_mul_f32_dpp, 16, 28, 0, 0) CPR_DPP(v_mul_f32_dpp, 17, 29, 1, 0)
                         CPR_PB_U(4, 24, 0) CPR_PB_U(5, 25, 0) CPR_PB_O(16, 30, 2, 0) CPR_PB_O(17, 31, 3, 0)
                             CPR_PB_U(6, 26, 0) CPR_PB_U(7, 27, 0) CPR_PB_O(16, 32, 4, 0) CPR_PB_O(17, 33, 5, 0)
                                 CPR_PB_U(8, 20, 1) CPR_PB_U(9, 21, 1) CPR_PB_O(16, 34, 6, 0) CPR_PB_O(17, 35, 7, 0)
                                     CPR_PB_U(10, 22, 1) CPR_PB_U(11, 23, 1) CPR_PB_O(16, 28, 8, 1)
                                         CPR_PB_O(17, 29, 9, 1) CPR_PB_U(12, 24, 1) CPR_PB_U(13, 25, 1)
                                             CPR_PB_O(16, 30, 10, 1) CPR_PB_O(17, 31, 11, 1) CPR_PB_U(14, 26, 1)
                                                 CPR_PB_U(15, 27, 1) CPR_PB_O(16, 32, 12, 1) CPR_PB_O(17, 33, 13, 1)
                 : CPR_PB_OUT(0), "=&v"(o[0]), "=&v"(o[1])
                 : "v"(kf[0]), "v"(kf[1]), CPR_PB_IN);
  CPR_PB_CASE(1, 1, 2, 3) CPR_PB_CASE(2, 3, 4, 5) CPR_PB_CASE(3, 5, 6, 7) CPR_PB_CASE(4, 7, 8, 9)
  CPR_PB_CASE(5, 9, 10, 11) CPR_PB_CASE(6, 11, 12, 13) CPR_PB_CASE(7, 13, 14, 15)
}
#undef CPR_PB_CASE
#undef CPR_PB_IN
#undef CPR_PB_OUT
#undef CPR_PB_TAIL
#undef CPR_PB_O
#undef CPR_PB_U
#undef CPR_DPP

template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// Raw k and q elements 8c .. 8c+7 of one token (c = lane mod 16).
template <class D>
struct KQRaw {
  uint32_t w[sizeof(typename D::T) == 2 ? 8 : 16];  // k then q: 4 + 4 dwords (bf16) or 8 + 8 (fp32)
};

// How a state column's keys sit on the lanes.  Up to d_k = 128 a lane holds
// its column's whole key range and a wave covers 64 columns.  At d_k = 256
// the keys of column j are split over lanes j and j + 32 (rows 0-1 of the
// wave hold keys 0 .. 127, rows 2-3 keys 128 .. 255), a wave covers 32
// columns, and the two halves' partial sums are combined across the lane
// halves (halves_sum).
template <int DK>
struct KeySplit {
  static constexpr int kParts = DK > 128 ? 2 : 1;
  static constexpr int kKeys = DK / kParts;  // state elements per lane
  static constexpr int kCols = 64 / kParts;  // state columns per wave
  static_assert(DK % 16 == 0 && DK <= 256, "head dims up to 256");
};

// this lane's 16-byte slot of a k or q row of DK elements: elements 8c ..
// 8c+7 of its half of the row, c = lane mod 16
template <int DK>
__device__ __forceinline__ int kq_slot(int lane) {
  if constexpr (KeySplit<DK>::kParts == 2) return (lane & 15) + 16 * (lane >> 5);
  return (lane & 15) & (DK / 8 - 1);  // lanes past the row repeat an in-bounds slot
}

// x of lanes 0-31 plus x of lanes 32-63 (lane l pairs with l +- 32), the same
// value in every lane: v_permlane32_swap exchanges the two lane halves, so
// the two values meet in one fp32 add, which is exact in either order
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// k and q of one token from plain row pointers (decode, continuation head)
template <class D, int DK>
__device__ __forceinline__ void load_kq(KQRaw<D>& r, const typename D::T* krow, const typename D::T* qrow, int lane) {
  typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
  const int c = kq_slot<DK>(lane);
  constexpr int n = sizeof(typename D::T) == 2 ? 1 : 2;  // 16-byte loads per 8 elements
#pragma unroll
  for (int m = 0; m < n; ++m) {
    const u32x4v a = *reinterpret_cast<const u32x4v*>(krow + 8 * c + 4 * m);
    const u32x4v b = *reinterpret_cast<const u32x4v*>(qrow + 8 * c + 4 * m);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      r.w[4 * m + e] = a[e];
      r.w[4 * n + 4 * m + e] = b[e];
    }
  }
}

template <class D>
__device__ __forceinline__ void unpack_kq(const KQRaw<D>& r, float (&kf)[8], float (&qf)[8]) {
  if constexpr (sizeof(typename D::T) == 2) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t wk = r.w[e >> 1], wq = r.w[4 + (e >> 1)];
      kf[e] = (e & 1) ? __uint_as_float(wk & 0xffff0000u) : __uint_as_float(wk << 16);
      qf[e] = (e & 1) ? __uint_as_float(wq & 0xffff0000u) : __uint_as_float(wq << 16);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      kf[e] = __uint_as_float(r.w[e]);
      qf[e] = __uint_as_float(r.w[8 + e]);
    }
  }
}

// ---------------------------------------------------------------------------
// The plain per-token step (one state column per lane), used only by the
// comparators that stand for the orders CPR replaces (recurrent everywhere,
// and the recurrent decode of "native mixed" serving): the state is decayed
// element by element at every token.  The CPR path uses token_step below.
//
// Lane j holds column j of S (S[i][j] = M[j][i], i = 0..DK-1) in s[].  The
// step is, in this exact order:
//   pass A, i ascending:  s[i] = alpha * s[i];  p_(i mod 2) = fma(s[i], k[i], p_(i mod 2))
//   p = p_0 + p_1;  u = beta * (v_j - p)
//   pass B, i ascending:  s[i] = fma(k[i], u, s[i]);  o_(i mod 2) = fma(s[i], q[i], o_(i mod 2))
//   return o_0 + o_1
// which is M' = alpha M, p = M' k, u = beta (v - p), M = M' + u k^T, o = M q.

// alpha = exp(g) (comparators)
__device__ __forceinline__ float decay_of(float g) { return expf(g); }

template <int DK>
__device__ __forceinline__ float token_step_plain(float (&s)[DK], const float (&kf)[8], const float (&qf)[8],
                                                  float alpha, float beta, float v) {
  static_assert(DK % 16 == 0 && DK <= 128, "one 16-lane row holds the key row");
  asm volatile("s_nop 1" ::"v"(kf[0]), "v"(kf[1]), "v"(kf[2]), "v"(kf[3]), "v"(kf[4]), "v"(kf[5]), "v"(kf[6]),
               "v"(kf[7]));
  float p0 = 0.f, p1 = 0.f;
  static_for<0, DK / 8>([&](auto nc) {
    constexpr int n = decltype(nc)::value;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const int i = 8 * n + e;
      s[i] = alpha * s[i];
      fmac_bcast<n>(p0, kf[e], s[i]);
      s[i + 1] = alpha * s[i + 1];
      fmac_bcast<n>(p1, kf[e + 1], s[i + 1]);
    }
  });
  const float u = beta * (v - (p0 + p1));
  asm volatile("s_nop 1" ::"v"(qf[0]), "v"(qf[1]), "v"(qf[2]), "v"(qf[3]), "v"(qf[4]), "v"(qf[5]), "v"(qf[6]),
               "v"(qf[7]));
  float o0 = 0.f, o1 = 0.f;
  // software-pipelined: the updates of elements 2j, 2j+1 are followed by the
  // output terms of elements 2j-2, 2j-1, so every state register and output
  // accumulator is read at least four instructions after its last write and
  // the DPP hazard needs no wait (each accumulator still takes its terms in
  // ascending order)
  static_for<0, DK / 2 + 1>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    if constexpr (j < DK / 2) {
      constexpr int i = 2 * j, n = i / 8, e = i % 8;
      fmac_bcast<n>(s[i], kf[e], u);
      fmac_bcast<n>(s[i + 1], kf[e + 1], u);
    }
    if constexpr (j >= 1) {
      constexpr int i = 2 * j - 2, n = i / 8, e = i % 8;
      fmac_bcast<n>(o0, qf[e], s[i]);
      fmac_bcast<n>(o1, qf[e + 1], s[i + 1]);
    }
  });
  return o0 + o1;
}

// ---------------------------------------------------------------------------
// The CPR per-token step, on a scaled running state.
//
// Between chunk boundaries the running state is held as M = exp(lg) N: the
// state registers (and the cache's s_run) hold N, and lg, one fp32 per
// sequence and head, is the log of its scale.  A boundary state has lg = 0
// and N = M.  Token t, with log-decay g, first advances the scale
// (token_scale):
//   x = lg + g                                        (one fp32 add)
//   renorm = x < kRenormLog
// then takes its scalars (step_factors):
//   c = exp(x),  b = beta * r  with  r = exp(-x)  (r = 1 when renorm)
// and steps N (token_step):
//   renorm:  N = c N element by element, then c = 1
//   p = c (N k)      w = b (v - p)      (= u r with u = beta (v - p))
//   N = N + w k^T    o = c (N q)
// and the log-scale after the token is x, or 0 when renorm (scale_after).
// In exact arithmetic this is M' = alpha M = c N, p = M' k,
// M = M' + u k^T = exp(lg') N and o = M q: the update of the pages'
// recurrence.  The per-element decay multiply of the plain step becomes the
// scalar c, so a state element costs three FMAs per token (N k, the update,
// N q) instead of a multiply and three FMAs.  Renormalising keeps |N| within
// a factor exp(-kRenormLog) of the state's scale, far inside fp32's range;
// the decision depends only on the sequence's own log-decays since the last
// boundary, so prefill and decode renormalise at the same tokens.
//
// Order (pinned), lane j (state column j).  Every accumulator starts with
// the product of its first term -- p_i = k[i] * N[i] for i < 4, o_i = q[i] * N[i] for i < 2 --
// (the o terms taken after the update) and then takes fused multiply-adds in
// ascending i:
//   pass A, i ascending:  p_(i mod 4) = fma(k[i], N[i], p_(i mod 4))
//   w = b * (v - c * ((p_0 + p_1) + (p_2 + p_3)))
//   pass B, i ascending:  N[i] = fma(k[i], w, N[i]);  o_(i mod 2) = fma(q[i], N[i], o_(i mod 2))
//   o = c * (o_0 + o_1)
//
// At d_k = 256 (KeySplit) each lane runs these passes over its half of the
// keys, i = 0 .. 127 of the half, with P = (p_0 + p_1) + (p_2 + p_3) and
// O = o_0 + o_1 per half, and the halves meet in one add:
//   w = b * (v - c * (P_lo + P_hi)),  o = c * (O_lo + O_hi).
constexpr float kRenormLog = -32.f;

struct TokenScale {
  float x;      // lg + g
  bool renorm;  // x < kRenormLog: the token renormalises
};

// the scale step of a token with log-decay g on a running state of log-scale lg
__device__ __forceinline__ TokenScale token_scale(float lg, float g) {
  const float x = lg + g;
  return TokenScale{x, x < kRenormLog};
}

// log-scale of the running state after the token
__device__ __forceinline__ float scale_after(TokenScale t) { return t.renorm ? 0.f : t.x; }

// the token's step scalars: c = exp(x) (for a renormalising token, the factor
// applied to N before a step with c = 1) and b = beta * r with r = exp(-x)
// (r = 1 when renormalising)
__device__ __forceinline__ void step_factors(TokenScale t, float beta, float& c, float& b) {
  c = expf(t.x);
  b = beta * (t.renorm ? 1.f : expf(-t.x));
}

// N = c N before a renormalising token's step
template <int DK>
__device__ __forceinline__ void renormalise(float (&s)[DK], float c) {
#pragma unroll
  for (int i = 0; i < DK; ++i) s[i] = c * s[i];
}

// state element of a scaled running state: exp(lg) * n (exactly n when lg = 0)
__device__ __forceinline__ float scale_of_log(float lg) { return expf(lg); }

// The per-token step.  s: this lane's state column (N; its half at
// d_k = 256); kf, qf: this lane's unpacked k and q elements 8c .. 8c+7 (DPP
// delivery above); c, b, renorm: the token's scalars (step_factors,
// token_scale); v: the lane's value element.  Returns the output element o.
template <int DKF>
__device__ __forceinline__ float token_step(float (&s)[KeySplit<DKF>::kKeys], const float (&kf)[8],
                                            const float (&qf)[8], float c, float b, bool renorm, float v) {
  constexpr int DK = KeySplit<DKF>::kKeys;  // keys of this lane
  static_assert(DK % 16 == 0 && DK <= 128, "one 16-lane row holds the lane's keys");
  if (renorm) {
    renormalise<DK>(s, c);
    c = 1.f;
  }
  asm volatile("s_nop 1" ::"v"(kf[0]), "v"(kf[1]), "v"(kf[2]), "v"(kf[3]), "v"(kf[4]), "v"(kf[5]), "v"(kf[6]),
               "v"(kf[7]));
  float p[4];
  static_for<0, DK / 16>([&](auto bc) { pass_a_keys16<decltype(bc)::value, DK>(p, kf, s); });
  float P = (p[0] + p[1]) + (p[2] + p[3]);
  if constexpr (KeySplit<DKF>::kParts == 2) P = halves_sum(P);
  const float w = b * (v - c * P);
  asm volatile("s_nop 1" ::"v"(qf[0]), "v"(qf[1]), "v"(qf[2]), "v"(qf[3]), "v"(qf[4]), "v"(qf[5]), "v"(qf[6]),
               "v"(qf[7]));
  float o[2];
  // software-pipelined as in token_step_plain: the updates of elements 2j,
  // 2j+1 are followed by the output terms of elements 2j-2, 2j-1
  static_for<0, DK / 16>([&](auto bc) { pass_b_keys16<decltype(bc)::value, DK>(s, o, kf, qf, w); });
  fmac_bcast<DK / 8 - 1>(o[0], qf[6], s[DK - 2]);
  fmac_bcast<DK / 8 - 1>(o[1], qf[7], s[DK - 1]);
  float O = o[0] + o[1];
  if constexpr (KeySplit<DKF>::kParts == 2) O = halves_sum(O);
  return c * O;
}

// One token of a single-token caller (decode, continuation head): the token's
// k and q rows, g, beta and value element; the state column s (N) and the
// log-scale lg are updated in place.  Returns the output element.
template <class D, int DK>
__device__ __forceinline__ float token_step_at(float (&s)[KeySplit<DK>::kKeys], float& lg, const typename D::T* krow,
                                               const typename D::T* qrow, float g, float beta, float v, int lane) {
  KQRaw<D> raw;
  load_kq<D, DK>(raw, krow, qrow, lane);
  const TokenScale ts = token_scale(lg, g);
  float c, b;
  step_factors(ts, beta, c, b);
  float kf[8], qf[8];
  unpack_kq<D>(raw, kf, qf);
  const float out = token_step<DK>(s, kf, qf, c, b, ts.renorm, v);
  lg = scale_after(ts);
  return out;
}

// The CPR scan's loop over tokens t = 0 .. n-1 (n >= 1) of one stretch of a
// sequence that starts on a chunk boundary: token t at row row0 + t * H of v
// and o and at row kq0 + t * Hk of q and k; output o_t to column col of its
// row of o; the state (N, from scale 1) updated in place.  Lane t holds token
// t's step scalars c_l and b_l (step_factors); bit t of renorm is set when
// token t renormalises.  k, q and v of token t+1 are fetched as soon as
// token t's have been unpacked; every fetch is issued (its index is clamped
// to token n-1), so the wait before a token's first use of its operands
// covers that token's loads only.  Rows are addressed as a wave-uniform base
// plus a 32-bit lane offset (one VGPR per operand kind).  At d_k = 256 the
// lanes of the upper half hold the same columns' upper keys and store the
// same outputs as the lower half.
template <class D, int DK, int DV>
__device__ __forceinline__ void scan_tokens(float (&s)[KeySplit<DK>::kKeys], const typename D::T* __restrict__ kp,
                                            const typename D::T* __restrict__ qp, const typename D::T* __restrict__ vp,
                                            typename D::T* __restrict__ op, size_t row0, int H, size_t kq0, int Hk,
                                            int n, int col, int lane, float c_l, float b_l, uint64_t renorm) {
  typedef typename D::T T;
  typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
  constexpr int nq = sizeof(T) == 2 ? 1 : 2;  // 16-byte loads per 8 elements
  const uint32_t kq_stride = (uint32_t)(Hk * DK * sizeof(T)), v_stride = (uint32_t)(H * DV * sizeof(T));
  const BufRsrc rk = buf_rsrc(kp + kq0 * DK, (uint32_t)(n - 1) * kq_stride + DK * sizeof(T));
  const BufRsrc rq = buf_rsrc(qp + kq0 * DK, (uint32_t)(n - 1) * kq_stride + DK * sizeof(T));
  const BufRsrc rv = buf_rsrc(vp + row0 * DV, (uint32_t)(n - 1) * v_stride + DV * sizeof(T));
  const BufRsrc ro = buf_rsrc(op + row0 * DV, (uint32_t)(n - 1) * v_stride + DV * sizeof(T));
  const uint32_t kq_off = (uint32_t)(kq_slot<DK>(lane) * 8 * sizeof(T));
  const uint32_t v_off = (uint32_t)(col * sizeof(T));
  KQRaw<D> raw;
  uint32_t vb;
  auto fetch = [&](int t) {
    const uint32_t tt = (uint32_t)min(t, n - 1);
#pragma unroll
    for (int m = 0; m < nq; ++m) {
      const u32x4v a =
          __builtin_bit_cast(u32x4v, __builtin_amdgcn_raw_buffer_load_b128(rk, kq_off + 16 * m, tt * kq_stride, 0));
      const u32x4v b =
          __builtin_bit_cast(u32x4v, __builtin_amdgcn_raw_buffer_load_b128(rq, kq_off + 16 * m, tt * kq_stride, 0));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        raw.w[4 * m + e] = a[e];
        raw.w[4 * nq + 4 * m + e] = b[e];
      }
    }
    if constexpr (sizeof(T) == 2)
      vb = __builtin_amdgcn_raw_buffer_load_b16(rv, v_off, tt * v_stride, 0);
    else
      vb = __builtin_amdgcn_raw_buffer_load_b32(rv, v_off, tt * v_stride, 0);
  };
  // token t's operands are unpacked (and token t+1's fetch issued) at the end
  // of iteration t-1, so the loop carries the unpacked values and the fetch
  // writes the registers the unpack has just read
  float kf[8], qf[8];
  float vcur;
  auto take = [&](int t) {
    unpack_kq<D>(raw, kf, qf);
    uint32_t vbits = vb;
    asm volatile("" : "+v"(vbits));  // decode v here, not next to its load
    vcur = D::from_bits(vbits);
    // the next fetch is issued after the unpack, so that its registers are
    // not live beside both tokens' raw words (before the first token the
    // compiler would otherwise issue both fetches back to back)
    asm volatile("" ::"v"(kf[0]), "v"(kf[1]), "v"(kf[2]), "v"(kf[3]), "v"(kf[4]), "v"(kf[5]), "v"(kf[6]),
                 "v"(kf[7]), "v"(qf[0]), "v"(qf[1]), "v"(qf[2]), "v"(qf[3]), "v"(qf[4]), "v"(qf[5]), "v"(qf[6]),
                 "v"(qf[7])
                 : "memory");
    fetch(t + 1);
  };
  fetch(0);
  take(0);
  for (int t = 0; t < n; ++t) {
    const float out =
        token_step<DK>(s, kf, qf, lane_bcast(c_l, t), lane_bcast(b_l, t), (renorm >> t) & 1, vcur);
    auto store = [&] {
      if constexpr (sizeof(T) == 2)
        __builtin_amdgcn_raw_buffer_store_b16(D::round(out), ro, v_off, (uint32_t)t * v_stride, 0);
      else
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(out), ro, v_off, (uint32_t)t * v_stride, 0);
    };
    // every lane stores, with no branch around the store, so the wait
    // before the next token's operands can leave the store in flight (a
    // store under an exec branch makes it wait for all).  At d_k = 256 the
    // two lanes of a column hold the same bits (halves_sum adds the lower
    // half to the upper in both) and store them to the same address.
    store();
    if (t + 1 < n) take(t + 1);
  }
}

// The plain scan loop (comparators): tokens t = 0 .. n-1 (n >= 1) of one
// stretch of a sequence, laid out as for scan_tokens, with the plain step;
// alpha_l / beta_l hold token t's decay and beta in lane t.  k, q and v of
// token t+1 are fetched into the other of two register buffers as token t
// starts.
template <class D, int DK, int DV>
__device__ __forceinline__ void scan_tokens_plain(float (&s)[DK], const typename D::T* __restrict__ kp,
                                                  const typename D::T* __restrict__ qp,
                                                  const typename D::T* __restrict__ vp, typename D::T* __restrict__ op,
                                                  size_t row0, int H, size_t kq0, int Hk, int n, int col, int lane,
                                                  float alpha_l, float beta_l) {
  KQRaw<D> r0, r1;
  uint32_t v0, v1;
  auto fetch = [&](KQRaw<D>& r, uint32_t& vb, int t) {
    const size_t tt = (size_t)min(t, n - 1);
    const size_t row = row0 + tt * H, kr = kq0 + tt * Hk;
    load_kq<D, DK>(r, kp + kr * DK, qp + kr * DK, lane);
    vb = D::load_bits(vp + row * DV, col);
  };
  auto step = [&](KQRaw<D>& r, uint32_t& vb, KQRaw<D>& rn, uint32_t& vn, int t) {
    float kf[8], qf[8];
    unpack_kq<D>(r, kf, qf);
    uint32_t vbits = vb;
    asm volatile("" : "+v"(vbits));  // decode v here, not next to its load
    const float vcur = D::from_bits(vbits);
    fetch(rn, vn, t + 1);
    const float out = token_step_plain<DK>(s, kf, qf, lane_bcast(alpha_l, t), lane_bcast(beta_l, t), vcur);
    D::store(op + (row0 + (size_t)t * H) * DV, col, out);
  };
  fetch(r0, v0, 0);
  int t = 0;
  for (; t + 1 < n; t += 2) {
    step(r0, v0, r1, v1, t);
    step(r1, v1, r0, v0, t + 1);
  }
  if (t < n) step(r0, v0, r1, v1, t);
}

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
__device__ __forceinline__ void chunk_local_f32(ChunkLds<DK, DV>& sm, float* __restrict__ W, float* __restrict__ U,
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
__device__ __forceinline__ void chain_step_f32(ChainLds<DK, NB>& sm) {
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

// ===========================================================================
// bf16 inputs: chunk products and boundary advance on MFMA
// (v_mfma_f32_16x16x32_bf16: bf16 operands, fp32 accumulation).
//
// Operand layout (16x16 output tiles, 64 lanes, lane = 16 g + c):
//   accumulator: lane holds D[4g + r][c], r = 0..3
//   A fragment:  lane holds A[c][k slots of group g], 8 bf16
//   B fragment:  lane holds B[k slots of group g][c], 8 bf16
// The k slots of group g for a 32-wide k step starting at k0 are
//   k0 + 4g + {0,1,2,3}  and  k0 + 16 + 4g + {0,1,2,3}
// (the same mapping for A and B, so every product pairs matching k).  With
// this mapping two accumulator tiles that cover rows k0..k0+31 ARE a B
// fragment, so the boundary state and the corrections Delta feed the next
// product straight from registers.
namespace mfma {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mma(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// two fp32 -> packed bf16 (lo in bits 0..15), one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}

// B fragment from the accumulator tiles holding rows k0..k0+15 (a) and k0+16..k0+31 (b)
__device__ __forceinline__ u32x4 frag_from_acc(const f32x4& a, const f32x4& b) {
  return u32x4{pack2(a[0], a[1]), pack2(a[2], a[3]), pack2(b[0], b[1]), pack2(b[2], b[3])};
}

// fragment from one row of a row-major bf16 matrix (8-byte aligned rows)
__device__ __forceinline__ u32x4 frag_row(const uint16_t* row, int k0, int g) {
  const u32x2 x = *reinterpret_cast<const u32x2*>(row + k0 + 4 * g);
  const u32x2 y = *reinterpret_cast<const u32x2*>(row + k0 + 16 + 4 * g);
  return u32x4{x[0], x[1], y[0], y[1]};
}

}  // namespace mfma

// Chunk-product slot of the bf16 path.  It is written in the order the
// boundary chain consumes it: every 1 KB block is one wave-wide MFMA operand
// with lane l's 16 bytes at byte 16 l, so the chain reads it with contiguous
// 16-byte loads.  Lane l = 16 g + c:
//   WF  A fragments of Wneg = -W (C x DK); fragment (kb, tm) is block
//       kb * C/16 + tm; lane holds Wneg[16 tm + c][32 kb + 4 g + {0..3}] and
//       Wneg[16 tm + c][32 kb + 16 + 4 g + {0..3}]
//   KF  A fragments of K~^T (DK x C); fragment (kb, im) is block kb * DK/16 + im;
//       lane holds KtT[16 im + c][32 kb + 4 g + {0..3}] and [32 kb + 16 + 4 g + {0..3}]
//   UT  U (C x DV) fp32 in accumulator tiles; tile (jt, tm) is block
//       jt * C/16 + tm; lane holds U[16 tm + 4 g + r][16 jt + c], r = 0..3
template <int DK, int DV>
struct SlotB {
  static constexpr size_t oWF = 0;
  static constexpr size_t oKF = (size_t)kChunk * DK * 2;
  static constexpr size_t oU = oKF + (size_t)DK * kChunk * 2;
  static constexpr size_t bytes = oU + (size_t)kChunk * DV * 4;
};

// Chunk products, bf16 path (one full chunk, one head, 256 threads = 4 waves).
//   gamma = left-to-right fp32 cumsum of g; Gamma_t = exp(gamma_t);
//   e_t = exp(gamma_{C-1} - gamma_t)
//   G = K K^T                             (MFMA, bf16 K exact, fp32 sums)
//   L[t][s] = (beta_t * exp(gamma_t - gamma_s)) * G[t][s], s < t   (fp32)
//   X = (I + L)^{-1} by 16 x 16 blocks (fp32):
//     diagonal blocks X_BB = (I + L_BB)^{-1} by forward substitution: lane =
//       column s, rows q ascending, acc = (q == s), then
//       acc = fma(-L[q][r], X[r][s], acc) for r = 0 .. q-1 ascending;
//     below the diagonal, block rows B = 1, 2, 3 in turn, for j < B:
//       Y = sum_{k=j}^{B-1} L_Bk X_kj,  X_Bj = -X_BB Y
//       (v_mfma_f32_16x16x4_f32, blocks k ascending; step m of a 16-wide
//       block contracts index 4 g + m in lane group g)
//   T = X diag(beta);  TB = bf16(T);  TG = bf16(T diag(Gamma))
//   W^T = K^T TG^T  -> Wneg fragments (MFMA bf16; W rounded to bf16, negated)
//   U   = TB V                         (MFMA bf16; fp32 tiles)
//   KtT = bf16(e_r * K[r][i])
//   Gamma_n = Gamma_{C-1}
// 53,248 bytes for d_k = d_v = 128: three work-groups fit in one CU's LDS.
template <int DK, int DV>
struct alignas(16) ChunkLdsB {
  static constexpr int kLK = DK + 8, kLV = DV + 8, kLA = kChunk + 4, kLT = kChunk + 4;
  uint16_t K[kChunk][kLK];  // row-major K
  uint16_t V[kChunk][kLV];  // row-major V
  // A[t][s] = L[t][s] (s < t); A[s][t] = X[t][s] (s <= t).  Once X is read,
  // the same bytes hold bf16(T diag(Gamma)) and bf16(T), row-major (TG, TB).
  float A[kChunk][kLA];
  float beta[kChunk], gam[kChunk], Gam[kChunk], e[kChunk];  // gam holds g until the cumsum
  __device__ uint16_t (*TG())[kLT] { return reinterpret_cast<uint16_t (*)[kLT]>(&A[0][0]); }
  __device__ uint16_t (*TB())[kLT] { return reinterpret_cast<uint16_t (*)[kLT]>(&A[0][0]) + kChunk; }
  static_assert(2 * kChunk * kLT * 2 <= kChunk * kLA * 4, "TG and TB fit in A's bytes");
};

// Stage one chunk (bf16 rows) into LDS: K and V row-major, g (into gam), beta.
// Row t of k starts at k + (k_row0 + t * k_stride) * DK (likewise v); g and
// beta at gb0 + t * gb_stride.  Rows t >= n (a chunk shorter than the slot)
// are identity padding: k = v = 0, g = beta = 0.
template <int DK, int DV>
__device__ __forceinline__ void stage_chunk_bf16(ChunkLdsB<DK, DV>& sm, const uint16_t* __restrict__ k,
                                                 size_t k_row0, size_t k_stride,
                                                 const uint16_t* __restrict__ v, size_t v_row0,
                                                 size_t v_stride, const uint16_t* __restrict__ g,
                                                 const uint16_t* __restrict__ beta, size_t gb0,
                                                 size_t gb_stride, int n) {
  // 256 threads (every caller's work-group): all of a thread's loads are
  // issued before its first LDS write, so the staging costs one memory
  // round trip rather than one per 16-byte piece
  constexpr int NT = 256, MK = kChunk * DK / 8 / NT, MV = kChunk * DV / 8 / NT;
  static_assert(MK * NT == kChunk * DK / 8 && MV * NT == kChunk * DV / 8 && kChunk <= NT, "staging split");
  const int tid = threadIdx.x;
  typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
  // rows past n load row n - 1 (callers have n >= 1) and are zeroed after
  // the loads, so no load sits behind a branch
  const int last = n > 0 ? n - 1 : 0;
  u32x4v wk[MK], wv[MV];
#pragma unroll
  for (int m = 0; m < MK; ++m) {
    const int idx = tid + m * NT, t = min(idx / (DK / 8), last), i0 = (idx % (DK / 8)) * 8;
    wk[m] = *reinterpret_cast<const u32x4v*>(k + (k_row0 + (size_t)t * k_stride) * DK + i0);
  }
#pragma unroll
  for (int m = 0; m < MV; ++m) {
    const int idx = tid + m * NT, t = min(idx / (DV / 8), last), j0 = (idx % (DV / 8)) * 8;
    wv[m] = *reinterpret_cast<const u32x4v*>(v + (v_row0 + (size_t)t * v_stride) * DV + j0);
  }
  const int tg = min(tid, last);
  const float gl = Bf16::load(g, gb0 + (size_t)tg * gb_stride);
  const float bl = Bf16::load(beta, gb0 + (size_t)tg * gb_stride);
  const u32x4v zero = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int m = 0; m < MK; ++m) {
    const int idx = tid + m * NT, t = idx / (DK / 8);
    *reinterpret_cast<u32x4v*>(&sm.K[t][(idx % (DK / 8)) * 8]) = t < n ? wk[m] : zero;
  }
#pragma unroll
  for (int m = 0; m < MV; ++m) {
    const int idx = tid + m * NT, t = idx / (DV / 8);
    *reinterpret_cast<u32x4v*>(&sm.V[t][(idx % (DV / 8)) * 8]) = t < n ? wv[m] : zero;
  }
  if (tid < kChunk) {
    sm.gam[tid] = tid < n ? gl : 0.f;
    sm.beta[tid] = tid < n ? bl : 0.f;
  }
  __syncthreads();
}

namespace mfma {
// Fragment whose k index runs down the rows of a row-major bf16 matrix M
// (leading dimension ld): lane 16 g + c gets M[k0 + 4 g + e][col] and
// M[k0 + 16 + 4 g + e][col], e = 0..3 (col already includes c).
__device__ __forceinline__ u32x4 frag_col(const uint16_t* M, int ld, int k0, int col, int g) {
  const uint16_t* p = M + (k0 + 4 * g) * ld + col;
  const uint16_t* q = p + 16 * ld;
  return u32x4{(uint32_t)p[0] | ((uint32_t)p[ld] << 16), (uint32_t)p[2 * ld] | ((uint32_t)p[3 * ld] << 16),
               (uint32_t)q[0] | ((uint32_t)q[ld] << 16), (uint32_t)q[2 * ld] | ((uint32_t)q[3 * ld] << 16)};
}

__device__ __forceinline__ f32x4 mma4(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
}  // namespace mfma

// X = (I + L)^{-1} for a strictly lower C x C matrix L, by 16 x 16 blocks.
// A holds L below the diagonal (A[t][s] = L[t][s], s < t); the routines
// write X^T into the diagonal and upper triangle (A[s][t] = X[t][s], s <= t,
// the diagonal blocks' lower halves receiving X's zeros).
//   diagonal blocks (inverse_diag_blocks, one wave, lane 16 B + s solves
//   column s of block B): rows q ascending, acc = (q == s), then
//   acc = fma(-L[q][r], X[r][s], acc) for r = 0 .. q-1 ascending;
//   below the diagonal (inverse_below_diag, all 4 waves of the work-group,
//   block rows B = 1, 2, 3 in turn, wave j < B makes block (B, j)):
//   Y = sum_{k=j}^{B-1} L_Bk X_kj (k ascending), X_Bj = -X_BB Y
//   (v_mfma_f32_16x16x4_f32; step m of a 16-wide block contracts index
//   4 g + m in lane group g).
template <int LDA>
__device__ __forceinline__ void inverse_diag_blocks(float (*A)[LDA], int lane) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  const int o = 16 * (lane >> 4), s = lane & 15;
  float x[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    float acc = (q == s) ? 1.f : 0.f;
#pragma unroll
    for (int r = 0; r < q; ++r) acc = __builtin_fmaf(-A[o + q][o + r], x[r], acc);
    x[q] = acc;  // exactly +0 for q < s
  }
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4)
    *reinterpret_cast<f4*>(&A[o + s][o + 4 * q4]) = f4{x[4 * q4], x[4 * q4 + 1], x[4 * q4 + 2], x[4 * q4 + 3]};
}

// Caller synchronised after inverse_diag_blocks; ends synchronised.
template <int LDA>
__device__ __forceinline__ void inverse_below_diag(float (*A)[LDA], int wave, int lane) {
  using namespace mfma;
  const int lr = lane & 15, g = lane >> 4;
#pragma unroll
  for (int B = 1; B < kChunk / 16; ++B) {
    if (wave < B) {
      const int j = wave;
      f32x4 Y = {0.f, 0.f, 0.f, 0.f};
      for (int kk = j; kk < B; ++kk)
#pragma unroll
        for (int m = 0; m < 4; ++m)
          Y = mma4(A[16 * B + lr][16 * kk + 4 * g + m], A[16 * j + lr][16 * kk + 4 * g + m], Y);
      f32x4 Xb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < 4; ++m) Xb = mma4(-A[16 * B + 4 * g + m][16 * B + lr], Y[m], Xb);
      *reinterpret_cast<f32x4*>(&A[16 * j + lr][16 * B + 4 * g]) = Xb;
    }
    __syncthreads();
  }
}

// Caller staged the chunk and synchronised; 256 threads.  Writes the slot
// (SlotB layout) and *gamn.
// kAux: the cache policy of the slot stores.  0: plain stores, for a slot
// that a later launch reads.  Otherwise the buffer instructions' cache-policy
// bits (and Gamma_n an atomic store) at agent scope, for a slot that another
// work-group of the same launch reads, possibly on another XCD.
template <int DK, int DV, int kAux = 0>
__device__ __forceinline__ void chunk_local_bf16(ChunkLdsB<DK, DV>& sm, uint8_t* __restrict__ slot,
                                                 float* __restrict__ gamn) {
  using namespace mfma;
  constexpr int C = kChunk;
  typedef SlotB<DK, DV> Sl;
  static_assert(DK % 32 == 0 && DV % 32 == 0, "head dims are multiples of 32");
  const BufRsrc slot_r = buf_rsrc(slot, (uint32_t)Sl::bytes);
  auto put = [&](size_t off, u32x4 x) {
    if constexpr (kAux == 0)
      *reinterpret_cast<u32x4*>(slot + off) = x;
    else
      __builtin_amdgcn_raw_buffer_store_b128(x, slot_r, (uint32_t)off, 0, kAux);
  };
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, lr = lane & 15, g = lane >> 4;
  // gamma = left-to-right fp32 cumsum of g (wave 0, in registers), while
  // waves 1-3 form the 10 tiles of G = K K^T on or below the diagonal
  // (wave w: tiles w - 1, w + 2, w + 5, w + 8 of the row-major order)
  f32x4 Gt[4];
  if (wave == 0) {
    const float gl = sm.gam[lane];
    float acc = lane_bcast(gl, 0), mine = acc;
    for (int t = 1; t < C; ++t) {
      acc = acc + lane_bcast(gl, t);
      if (lane == t) mine = acc;
    }
    sm.gam[lane] = mine;
    sm.Gam[lane] = expf(mine);
    sm.e[lane] = expf(acc - mine);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int q = wave - 1 + 3 * j;
      Gt[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (q < 10) {
        const int tm = q < 1 ? 0 : q < 3 ? 1 : q < 6 ? 2 : 3;
        const int tn = q - tm * (tm + 1) / 2;
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb)
          Gt[j] = mma(frag_row(&sm.K[16 * tm + lr][0], 32 * kb, g), frag_row(&sm.K[16 * tn + lr][0], 32 * kb, g),
                      Gt[j]);
      }
    }
  }
  __syncthreads();
  // L[t][s] = (beta_t exp(gamma_t - gamma_s)) G[t][s], s < t
  if (wave > 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int q = wave - 1 + 3 * j;
      if (q < 10) {
        const int tm = q < 1 ? 0 : q < 3 ? 1 : q < 6 ? 2 : 3;
        const int tn = q - tm * (tm + 1) / 2;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * tm + 4 * g + r, s = 16 * tn + lr;
          if (s < t) sm.A[t][s] = (sm.beta[t] * expf(sm.gam[t] - sm.gam[s])) * Gt[j][r];
        }
      }
    }
  }
  __syncthreads();
  if (wave == 0) {
    inverse_diag_blocks(sm.A, lane);
  } else {
    // K~^T fragments meanwhile
    for (int f = wave - 1; f < (C / 32) * (DK / 16); f += 3) {
      const int kb = f / (DK / 16), im = f % (DK / 16);
      const u32x4 raw = frag_col(&sm.K[0][0], ChunkLdsB<DK, DV>::kLK, 32 * kb, 16 * im + lr, g);
      u32x4 out;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int r = 32 * kb + 16 * (w >> 1) + 4 * g + 2 * (w & 1);
        out[w] = pack2(sm.e[r] * __uint_as_float(raw[w] << 16), sm.e[r + 1] * __uint_as_float(raw[w] & 0xffff0000u));
      }
      put(Sl::oKF + ((size_t)f * 64 + lane) * 16, out);
    }
  }
  __syncthreads();
  inverse_below_diag(sm.A, wave, lane);
  // T = X diag(beta) -> TB = bf16(T), TG = bf16(T diag(Gamma)), written over
  // A once every thread holds its part of X: thread items (t, 8 columns r0..)
  float Tv[C * C / 8 / 256][8];
#pragma unroll
  for (int m = 0; m < C * C / 8 / 256; ++m) {
    const int item = tid + 256 * m, t = item >> 3, r0 = (item & 7) * 8;
#pragma unroll
    for (int e2 = 0; e2 < 8; ++e2) {
      const int r = r0 + e2;
      Tv[m][e2] = (r <= t) ? sm.A[r][t] * sm.beta[r] : 0.f;
    }
  }
  __syncthreads();
#pragma unroll
  for (int m = 0; m < C * C / 8 / 256; ++m) {
    const int item = tid + 256 * m, t = item >> 3, r0 = (item & 7) * 8;
    u32x2 b[2], gg[2];
#pragma unroll
    for (int e2 = 0; e2 < 8; e2 += 2) {
      b[e2 >> 2][(e2 >> 1) & 1] = pack2(Tv[m][e2], Tv[m][e2 + 1]);
      gg[e2 >> 2][(e2 >> 1) & 1] = pack2(Tv[m][e2] * sm.Gam[r0 + e2], Tv[m][e2 + 1] * sm.Gam[r0 + e2 + 1]);
    }
    *reinterpret_cast<u32x2*>(&sm.TB()[t][r0]) = b[0];
    *reinterpret_cast<u32x2*>(&sm.TB()[t][r0 + 4]) = b[1];
    *reinterpret_cast<u32x2*>(&sm.TG()[t][r0]) = gg[0];
    *reinterpret_cast<u32x2*>(&sm.TG()[t][r0 + 4]) = gg[1];
  }
  __syncthreads();
  // Wneg fragments: W^T tiles (2 p, tm) and (2 p + 1, tm) form fragment (p, tm)
  for (int p = wave; p < DK / 32; p += 4) {
    u32x4 Kt[2][C / 32];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int kb = 0; kb < C / 32; ++kb)
        Kt[h][kb] = frag_col(&sm.K[0][0], ChunkLdsB<DK, DV>::kLK, 32 * kb, 32 * p + 16 * h + lr, g);
#pragma unroll
    for (int tm = 0; tm < C / 16; ++tm) {
      f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int kb = 0; kb < C / 32; ++kb) {
        const u32x4 tg = frag_row(&sm.TG()[16 * tm + lr][0], 32 * kb, g);
        acc[0] = mma(Kt[0][kb], tg, acc[0]);
        acc[1] = mma(Kt[1][kb], tg, acc[1]);
      }
      const u32x4 out = {pack2(-acc[0][0], -acc[0][1]), pack2(-acc[0][2], -acc[0][3]), pack2(-acc[1][0], -acc[1][1]),
                         pack2(-acc[1][2], -acc[1][3])};
      put(Sl::oWF + ((size_t)(p * (C / 16) + tm) * 64 + lane) * 16, out);
    }
  }
  // U tiles (tm, jt), jt = 2 p, 2 p + 1
  for (int p = wave; p < DV / 32; p += 4) {
    u32x4 Vt[2][C / 32];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int kb = 0; kb < C / 32; ++kb)
        Vt[h][kb] = frag_col(&sm.V[0][0], ChunkLdsB<DK, DV>::kLV, 32 * kb, 32 * p + 16 * h + lr, g);
#pragma unroll
    for (int tm = 0; tm < C / 16; ++tm) {
      f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int kb = 0; kb < C / 32; ++kb) {
        const u32x4 tb = frag_row(&sm.TB()[16 * tm + lr][0], 32 * kb, g);
        acc[0] = mma(tb, Vt[0][kb], acc[0]);
        acc[1] = mma(tb, Vt[1][kb], acc[1]);
      }
#pragma unroll
      for (int h = 0; h < 2; ++h)
        put(Sl::oU + ((size_t)((2 * p + h) * (C / 16) + tm) * 64 + lane) * 16, __builtin_bit_cast(u32x4, acc[h]));
    }
  }
  if (tid == 0) {
    if constexpr (kAux == 0)
      *gamn = sm.Gam[C - 1];
    else
      __hip_atomic_store(gamn, sm.Gam[C - 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Boundary advance on the bf16 path for NT 16-column blocks of the state,
// one wave.  S[im][nt] is the accumulator tile of state rows 16 im .. 16 im + 15.
//   Sb    = bf16(S)                            (B fragments)
//   Delta = U + Wneg Sb                        (acc starts at U, k ascending)
//   S'    = Gamma_n * S + KtT bf16(Delta)      (acc starts at Gamma_n * S)
// wf(kb, tm) and kf(kb, im) return the slot's WF / KF fragments (from LDS or
// global memory).  k steps run outermost so consecutive MFMAs are
// independent; each tile accumulates its k steps in ascending order from its
// initial value, so the result depends neither on NT nor on where the
// operands come from.
// The general form: init2(im, nt, S[im][nt]) gives phase 2's initial tile
// (Gamma_n * S for the forward; the reverse chain adds its R term).
template <int DK, int NT, class FW, class FK, class FI>
__device__ __forceinline__ void chain_step_bf16_init(mfma::f32x4 (&S)[DK / 16][NT], FW&& wf, FK&& kf,
                                                     const mfma::f32x4 (&Ut)[kChunk / 16][NT], FI&& init2) {
  using namespace mfma;
  constexpr int C = kChunk;
  u32x4 Wf[DK / 32][C / 16], Kf[C / 32][DK / 16];
#pragma unroll
  for (int kb = 0; kb < DK / 32; ++kb)
#pragma unroll
    for (int tm = 0; tm < C / 16; ++tm) Wf[kb][tm] = wf(kb, tm);
#pragma unroll
  for (int kb = 0; kb < C / 32; ++kb)
#pragma unroll
    for (int im = 0; im < DK / 16; ++im) Kf[kb][im] = kf(kb, im);
  u32x4 Sb[DK / 32][NT];
#pragma unroll
  for (int kb = 0; kb < DK / 32; ++kb)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) Sb[kb][nt] = frag_from_acc(S[2 * kb][nt], S[2 * kb + 1][nt]);
  f32x4 D[C / 16][NT];
#pragma unroll
  for (int tm = 0; tm < C / 16; ++tm)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) D[tm][nt] = Ut[tm][nt];
#pragma unroll
  for (int kb = 0; kb < DK / 32; ++kb)
#pragma unroll
    for (int tm = 0; tm < C / 16; ++tm)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) D[tm][nt] = mma(Wf[kb][tm], Sb[kb][nt], D[tm][nt]);
  u32x4 Db[C / 32][NT];
#pragma unroll
  for (int kb = 0; kb < C / 32; ++kb)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) Db[kb][nt] = frag_from_acc(D[2 * kb][nt], D[2 * kb + 1][nt]);
#pragma unroll
  for (int im = 0; im < DK / 16; ++im)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) S[im][nt] = init2(im, nt, S[im][nt]);
#pragma unroll
  for (int kb = 0; kb < C / 32; ++kb)
#pragma unroll
    for (int im = 0; im < DK / 16; ++im)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) S[im][nt] = mma(Kf[kb][im], Db[kb][nt], S[im][nt]);
}

template <int DK, int NT, class FW, class FK>
__device__ __forceinline__ void chain_step_bf16(mfma::f32x4 (&S)[DK / 16][NT], FW&& wf, FK&& kf,
                                                const mfma::f32x4 (&Ut)[kChunk / 16][NT], float gn) {
  chain_step_bf16_init<DK, NT>(S, wf, kf, Ut, [gn](int, int, const mfma::f32x4& x) {
    return mfma::f32x4{gn * x[0], gn * x[1], gn * x[2], gn * x[3]};
  });
}

// One step straight from a global chunk-product slot (decode resync), for
// the NT 16-column blocks starting at block jb0.
template <int DK, int DV, int NT>
__device__ __forceinline__ void chain_step_bf16_global(mfma::f32x4 (&S)[DK / 16][NT],
                                                       const uint8_t* __restrict__ slot, float gn, int jb0, int lane) {
  typedef SlotB<DK, DV> Sl;
  typedef mfma::u32x4 F;
  const F* W = reinterpret_cast<const F*>(slot + Sl::oWF);
  const F* K = reinterpret_cast<const F*>(slot + Sl::oKF);
  const mfma::f32x4* U = reinterpret_cast<const mfma::f32x4*>(slot + Sl::oU);
  mfma::f32x4 Ut[kChunk / 16][NT];
#pragma unroll
  for (int tm = 0; tm < kChunk / 16; ++tm)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) Ut[tm][nt] = U[((jb0 + nt) * (kChunk / 16) + tm) * 64 + lane];
  chain_step_bf16<DK, NT>(
      S, [&](int kb, int tm) { return W[(kb * (kChunk / 16) + tm) * 64 + lane]; },
      [&](int kb, int im) { return K[(kb * (DK / 16) + im) * 64 + lane]; }, Ut, gn);
}

// State tile I/O for NT 16-column blocks from block jb0 (row-major [DK][DV]
// states): rows 16 im + 4 g + r, column 16 (jb0 + nt) + c.
template <int DK, int DV, int NT>
__device__ __forceinline__ void load_state_tiles(mfma::f32x4 (&S)[DK / 16][NT], const float* __restrict__ src,
                                                 int jb0, int lane) {
  const int lr = lane & 15, g = lane >> 4;
#pragma unroll
  for (int im = 0; im < DK / 16; ++im)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        S[im][nt][r] = src ? src[(size_t)(16 * im + 4 * g + r) * DV + 16 * (jb0 + nt) + lr] : 0.f;
}

template <int DK, int DV, int NT>
__device__ __forceinline__ void store_state_tiles(float* __restrict__ dst, const mfma::f32x4 (&S)[DK / 16][NT],
                                                  int jb0, int lane) {
  const int lr = lane & 15, g = lane >> 4;
#pragma unroll
  for (int im = 0; im < DK / 16; ++im)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[(size_t)(16 * im + 4 * g + r) * DV + 16 * (jb0 + nt) + lr] = S[im][nt][r];
}

// Boundary states inside the workspace are kept in accumulator-tile order:
// element (row, col) of a [DK][DV] state at
//   (((col / 16) * (DK / 16) + row / 16) * 64 + 16 ((row % 16) / 4) + col % 16) * 4 + row % 4,
// so the chain writes one 16-byte store per tile and the scan reads each
// lane's column with 16-byte loads.
template <int DK>
__host__ __device__ constexpr size_t bnd_index(int row, int col) {
  return ((size_t)((col >> 4) * (DK / 16) + (row >> 4)) * 64 + 16 * ((row & 15) >> 2) + (col & 15)) * 4 + (row & 3);
}

template <int DK, int NT>
__device__ __forceinline__ void store_bnd_tiles(float* __restrict__ dst, const mfma::f32x4 (&S)[DK / 16][NT], int jb0,
                                                int lane) {
#pragma unroll
  for (int im = 0; im < DK / 16; ++im)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      *reinterpret_cast<mfma::f32x4*>(dst + ((size_t)((jb0 + nt) * (DK / 16) + im) * 64 + lane) * 4) = S[im][nt];
}

// the same layout from a row-major [DK][DV] state (or zeros), for chunk 0
template <int DK, int DV, int NT>
__device__ __forceinline__ void store_bnd_tiles_from_rows(float* __restrict__ dst, const float* __restrict__ src,
                                                          int jb0, int lane) {
  mfma::f32x4 S[DK / 16][NT];
  load_state_tiles<DK, DV, NT>(S, src, jb0, lane);
  store_bnd_tiles<DK, NT>(dst, S, jb0, lane);
}

}  // namespace cpr
