// CPR Gated DeltaNet layer for gfx950: host side and the C ABI (gdn_cpr.h).
// The kernels live in prefill_kernels.hpp, decode_kernels.hpp,
// comparator_kernels.hpp and backward_kernels.hpp.
//
// Prefill (per call, all on the caller's stream):
//   k_plan            per-sequence chunk counts -> prefix sums (varlen plan)
//   k_chain_scan_bf16 bf16 batches of up to 128 sequences: one launch whose
//                     work-groups are, in ticket order, the chunk products
//                     of every full chunk, the boundary chains and the
//                     in-chunk scans, each starting when its input is ready
//   otherwise         k_chunk_local (chunk products of every full chunk, all
//                     in parallel), k_chain (boundary states: sequential over
//                     each sequence's full chunks, parallel over sequences x
//                     heads x column blocks), k_scan (per-token recurrence
//                     inside every chunk from its boundary state; writes o,
//                     the final state and the decode tail)
// Decode step:
//   k_decode          per-token step on the running state (one work-group
//                     per sequence x head), tail append, resync flag
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
#include "backward_kernels.hpp"

namespace {

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
// continuation, fwd_bwd and the cache read-out; not the comparators)
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
    *why = "head dims of 256 serve prefill, decode, continuation and fwd_bwd only";
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
  hipEvent_t fork = nullptr, join = nullptr, fchain = nullptr;
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
  hipEvent_t* ev[3] = {&y.fork, &y.join, &y.fchain};
  for (int i = 0; i < 3 && ok; ++i) ok = hipEventCreateWithFlags(ev[i], hipEventDisableTiming) == hipSuccess;
  if (cur != dev) (void)hipSetDevice(cur);
  if (!ok) {
    for (int i = 0; i < 3; ++i)
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
  FusedPlan fp{nullptr, a.counters, nullptr, 0};  // the plan clears the timeout word either way
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
  const bool wide = DK > 128 || DV > 128;
  if (s.dtype == GDN_DTYPE_BF16 && !wide)  // bwdb::Slot
    L.slot = 2 * (size_t)C * DK * 2 + 2 * DK * DV * 4 + (size_t)C * C * 4 + 3 * (size_t)C * DK * 4 +
             3 * (size_t)C * DV * 4 + 256;
  else  // bwd::BwdSlot (fp32 inputs, and bf16 at d = 256 with its scratch arrays)
    L.slot = (size_t)C * DK * esz + DK * (size_t)C * esz + DK * DV * 4 + (size_t)C * DV * 4 + (size_t)C * C * 4 +
             DK * DV * 4 + (wide ? 7 * (size_t)C * std::max(DK, DV) * 4 : 0);
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
  // stream beside the forward boundary chain and in-chunk scan (after the
  // forward's chunk products); the state and gradient stages, which need both
  // chains, follow on the caller's stream after the join.  Every kernel
  // computes what it computes in the one-stream order, so the bits are the
  // same.
  static gdn_status run_overlapped(const PrefillArgs& pa, const BwdArgs& ba, int64_t T, hipStream_t st,
                                   const SideStream& x, const char* fn) {
    const int Fmax = (int)(T / pa.Cl), Amax = Fmax + pa.N;
    auto ev = [&](hipError_t e) { return e == hipSuccess; };
    mark(0, st);
    hipLaunchKernelGGL(k_plan, dim3(1), dim3(1024), 0, st, pa.start, pa.end, pa.N, pa.Cl, pa.full_base, pa.all_base,
                       FusedPlan{nullptr, pa.counters, nullptr, 0});
    mark(1, st);
    // the forward's chunk products first, on the whole chip: launched beside
    // the backward's local stage, whose work-groups take a CU each, they would
    // wait for CUs to free up and delay the forward chain behind them
    if (Fmax > 0)
      hipLaunchKernelGGL((k_chunk_local_prefill_bf16<DK, DV>), dim3(Fmax, pa.H), dim3(256), 0, st, pa);
    mark(2, st);
    if (!ev(hipEventRecord(x.fork, st)) || !ev(hipStreamWaitEvent(x.s, x.fork, 0)))
      return fail(GDN_ERR_HIP, "%s: stream fork failed: %s", fn, hipGetErrorString(hipGetLastError()));
    hipLaunchKernelGGL((k_bwd_local_bf16<DK, DV>), dim3(Amax, pa.H), dim3(kBwdWaves<DK, DV> * 64), 0, x.s, ba);
    launch_bwd_chain_bf16(ba, x.s);
    if (pa.N > 0) launch_chain_bf16<DK, DV>(pa, st);
    mark(3, st);
    // the forward boundary states are complete here; the state and gradient
    // stages need them and the reverse chain's, not the scan's outputs, so they
    // follow the reverse chain on the side stream and take CUs as the scan's
    // waves drain (the event is recorded before the side stream waits on it)
    if (!ev(hipEventRecord(x.fchain, st)))
      return fail(GDN_ERR_HIP, "%s: event record failed: %s", fn, hipGetErrorString(hipGetLastError()));
    hipLaunchKernelGGL((k_scan<D, DK, DV>), dim3(Amax, pa.H, DV / kWave), dim3(kWave), 0, st, pa);
    mark(4, st);
    if (!ev(hipStreamWaitEvent(x.s, x.fchain, 0)))
      return fail(GDN_ERR_HIP, "%s: stream wait failed: %s", fn, hipGetErrorString(hipGetLastError()));
    mark(5, x.s);
    hipLaunchKernelGGL((k_bwd_state_grads_bf16<DK, DV>), dim3(Amax, pa.H), dim3(kBwdWaves<DK, DV> * 64), 0, x.s, ba);
    if (!ev(hipEventRecord(x.join, x.s)) || !ev(hipStreamWaitEvent(st, x.join, 0)))
      return fail(GDN_ERR_HIP, "%s: stream join failed: %s", fn, hipGetErrorString(hipGetLastError()));
    launch_key_head_sums(ba, T, st);
    mark(6, st);
    return launch_status(fn);
  }
  static gdn_status run(const PrefillArgs& pa, const BwdArgs& ba, int64_t T, size_t slot_bytes, hipStream_t st,
                        const char* fn) {
    constexpr bool kBf16 = std::is_same<D, Bf16>::value;
    // d_k = d_v = 256 (bf16 only) runs the fp32-product kernels with their C x d
    // arrays in the slot and the bf16-operand reverse chain
    constexpr bool kWide = DK > 128 || DV > 128;
    static_assert(!kWide || kBf16, "d = 256 takes bf16 inputs");
    const size_t want = kBf16 && !kWide ? bwdb::Slot<DK, DV>::bytes
                                        : bwd::BwdSlot<DK, DV, sizeof(typename D::T)>::bytes;
    if (slot_bytes != want) return fail(GDN_ERR_HIP, "%s: internal slot size mismatch", fn);
    if constexpr (kBf16 && !kWide) {
      if (T > 0) {
        // one stream only if no side stream can be had
        SideLease lease(st);
        if (const SideStream* x = lease.get()) return run_overlapped(pa, ba, T, st, *x, fn);
      }
    }
    gdn_status r = run_prefill<D, DK, DV>(pa, T, st, fn);
    if (r != GDN_OK) return r;
    const int Amax = (int)(T / pa.Cl) + pa.N;
    if constexpr (kWide) {
      if (T > 0) hipLaunchKernelGGL((k_bwd_local<D, DK, DV>), dim3(Amax, pa.H), dim3(256), 0, st, ba);
      hipLaunchKernelGGL((k_bwd_chain_wide<DK, DV>), dim3(pa.N, pa.H, DV / 64), dim3(256), 0, st, ba);
      mark(5, st);
      if (T > 0) {
        hipLaunchKernelGGL((k_bwd_grads<D, DK, DV>), dim3(Amax, pa.H), dim3(256), 0, st, ba);
        launch_key_head_sums(ba, T, st);
      }
      mark(6, st);
    } else if constexpr (kBf16) {
      if (T > 0)
        hipLaunchKernelGGL((k_bwd_local_bf16<DK, DV>), dim3(Amax, pa.H), dim3(kBwdWaves<DK, DV> * 64), 0, st, ba);
      launch_bwd_chain_bf16(ba, st);
      mark(5, st);
      if (T > 0) {
        hipLaunchKernelGGL((k_bwd_state_grads_bf16<DK, DV>), dim3(Amax, pa.H), dim3(kBwdWaves<DK, DV> * 64), 0,
                           st, ba);
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

template <>
struct WideFn<FwdBwdFn> : std::true_type {};

}  // namespace

// ===========================================================================
// C ABI

extern "C" size_t gdn_cpr_workspace_size(const gdn_cpr_shape* shape, int32_t num_seqs,
                                         int64_t total_tokens, int32_t op) {
  std::string why;
  if (!shape_ok(shape, &why, true) || num_seqs < 0 || total_tokens < 0) return 0;
  if (op == GDN_OP_PREFILL) return prefill_layout(*shape, num_seqs, total_tokens).total;
  if (op == GDN_OP_FWD_BWD) return fwd_bwd_layout(*shape, num_seqs, total_tokens).total;
  if (op == GDN_OP_DECODE) return decode_layout(*shape, num_seqs).total;
  if (op == GDN_OP_PREFILL_CONTINUE) return cont_layout(*shape, num_seqs, total_tokens).total;
  return 0;
}

extern "C" gdn_status gdn_cpr_debug_set_wait_polls(int32_t polls) {
  const char* fn = "gdn_cpr_debug_set_wait_polls";
  if (polls < 0) return fail(GDN_ERR_INVALID_ARG, "%s: negative poll count", fn);
  if (hipMemcpyToSymbol(HIP_SYMBOL(g_wait_polls), &polls, sizeof(polls)) != hipSuccess)
    return fail(GDN_ERR_HIP, "%s: %s", fn, hipGetErrorString(hipGetLastError()));
  g_last_error.clear();
  return GDN_OK;
}

extern "C" gdn_status gdn_cpr_wait_status(const gdn_cpr_shape* shape, int32_t num_seqs, int64_t total_tokens,
                                          const void* workspace, size_t workspace_bytes, int32_t* status,
                                          void* stream) {
  const char* fn = "gdn_cpr_wait_status";
  std::string why;
  if (!shape_ok(shape, &why, true)) return fail(GDN_ERR_UNSUPPORTED, "%s: %s", fn, why.c_str());
  if (num_seqs < 0 || total_tokens < 0) return fail(GDN_ERR_INVALID_ARG, "%s: negative size", fn);
  CHECK_PTR(status, "status");
  // prefill, continuation and fwd_bwd place the prefill layout at the start
  // of their workspace: the timeout word follows the fused launch's ticket
  const PrefillLayout L = prefill_layout(*shape, num_seqs, total_tokens);
  if (!workspace || workspace_bytes < L.total)
    return fail(GDN_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, L.total,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(GDN_ERR_INVALID_ARG, "%s: workspace is not 16-byte aligned", fn);
  const char* word = (const char*)workspace + L.counters + sizeof(int32_t);
  if (hipMemcpyAsync(status, word, sizeof(int32_t), hipMemcpyDeviceToDevice, (hipStream_t)stream) != hipSuccess)
    return fail(GDN_ERR_HIP, "%s: copy failed: %s", fn, hipGetErrorString(hipGetLastError()));
  g_last_error.clear();
  return GDN_OK;
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
  if (!shape_ok(shape, &why, true)) return fail(GDN_ERR_UNSUPPORTED, "%s: %s", fn, why.c_str());
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
