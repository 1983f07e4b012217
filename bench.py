"""Benchmark of the CPR Gated DeltaNet layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step is one pass of the layer's hot path over synthetic inputs already
resident in HBM:
  - prefill of 5 packed sequences x 2,048 tokens (H=16, d_k=d_v=128, C=64,
    bf16 q/k/v/g/beta, fp32 state): varlen plan, chunk products, boundary
    chain, in-chunk scan;
  - one decode step for 256 sequences whose state holds a 2,048-token prefix
    (per-token step on the running state; the resynchronisation pass runs
    every call and does the chunk computation when a tail fills).
Prints one JSON line.  `value` is tokens per second over the whole step
(5*2048 + 256 tokens).  The dominant kernel is the in-chunk scan; its
duration is measured with HIP events recorded by the library on its own
stream (gdn_cpr_set_stage_events).  The CPU baseline is the float64 oracle
on a bounded sample of the same workload.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN layer tokens/s (prefill 5x2048, decode 256x1) + bitwise prefill/decode parity"
# MI355X published peaks: fp32 vector 157.3 TFLOP/s (256 CUs x 4 SIMDs x 16
# lanes x 2 flop x 2 (packed fp32) x 2.4 GHz), fp32 matrix (MFMA) 157.3
# TFLOP/s, HBM 8 TB/s.  This library does not issue packed fp32 instructions,
# so its vector-fp32 issue limit is half the published figure (78.6 TFLOP/s);
# fractions of both are reported, the published one first.
PEAK_F32 = 157.3
PEAK_VALU_F32_NONPACKED = 256 * 4 * 16 * 2 * 2.4e9 / 1e12
PEAK_MFMA_F32 = 157.3
PEAK_MFMA_BF16 = 2500.0  # dense
PEAK_HBM = 8000.0  # GB/s


def bwd_state_grads_flop(C: int, dk: int, dv: int) -> int:
    """MFMA flops of the backward's state and gradient stages for one chunk-head:
    the products of the chunk-form gradient, each taken over the 16 x 16 tiles
    where its triangular C x C operand (X, the causal mask of P and dPD, dA) is
    nonzero, as the kernels issue them (the instruction counters of one
    fwd_bwd call record the same count: 19,365,888 at C = 64, d = 128).
      state:  Kt dB', K B, dO B^T, Dd B^T, Delta dB'^T (C x d x d each); X diag(beta) (.)
      grads:  dO Delta^T (lower), dPD K, X^T Dd, X^T dWn, dPD^T Q (triangular operand);
              Dd V^T and dWn (Gamma K)^T, (dG + dG^T) K (full); dX X^T; X^T Y (strict lower);
              Q K^T and K K^T (bf16, lower)"""
    nb = C // 16
    tile = 2 * 16 * 16 * 16
    tri = nb * (nb + 1) // 2
    state = 5 * 2 * C * dk * dv + tri * (dv // 16) * tile
    grads = (tri * (dv // 16) * 2 + tri * (dk // 16) * 3) * tile       # dPD, dV; dPD K, TW, dPD^T Q
    grads += nb * nb * (dv // 16 + dk // 16) * tile                    # dT
    grads += nb * nb * (dk // 16) * tile                               # (dG + dG^T) K
    grads += nb * tri * tile + sum((i + 1) * (nb - i) for i in range(nb)) * tile  # dX X^T, X^T Y
    grads += 2 * tri * (dk // 16) * tile                               # Q K^T, K K^T
    return state + grads


def bwd_state_grads_bf16_exec_flop(C: int, dk: int, dv: int) -> int:
    """bf16 MFMA flops the state and gradient stages execute for one chunk-head.
    A product with an fp32 operand runs as bf16 hi/lo parts: three products
    (hi hi, hi lo, lo hi) when both operands are fp32, two when the other is
    the layer's bf16 k, q, v or dO; Q K^T and K K^T take one.  Over the same
    tiles as `bwd_state_grads_flop` (the instruction counters of one fwd_bwd
    call record the same count: 44,072,960 at C = 64, d = 128)."""
    nb = C // 16
    tile = 2 * 16 * 16 * 16
    tri = nb * (nb + 1) // 2
    tri_y = sum((i + 1) * (nb - i) for i in range(nb))
    # K dB', K B, dO B^T: 2 each; Dd B^T, Delta dB'^T: 3 each; X diag(beta) (.): 3
    state = (2 + 2 + 2 + 3 + 3) * 2 * C * dk * dv + 3 * tri * (dv // 16) * tile
    grads = (2 * tri * (dv // 16) + 2 * tri * (dk // 16)) * tile        # dO Delta^T, dPD K
    grads += (3 * tri * (dv // 16) + 3 * tri * (dk // 16)) * tile       # X^T Dd, X^T dWn
    grads += 2 * tri * (dk // 16) * tile                               # dPD^T Q
    grads += 2 * nb * nb * (dv // 16 + dk // 16) * tile                # Dd V^T, dWn K^T
    grads += 2 * nb * nb * (dk // 16) * tile                           # (dG + dG^T) K
    grads += 3 * (nb * tri + tri_y) * tile                             # dX X^T, X^T Y
    grads += 2 * tri * (dk // 16) * tile                               # Q K^T, K K^T
    return state + grads


def _oracle_forward_heads(args):
    """CPU baseline worker: the fp64 oracle forward on a slice of heads
    (runs in a child process with one BLAS thread)."""
    import oracle
    q, k, v, g, beta, cu, h0 = args
    oracle.recurrent_forward(q, k, v, g, beta, cu, h0)
    return True


def _oracle_fwd_bwd_heads(args):
    """CPU baseline worker: the fp64 oracle forward and analytic backward on a slice of heads."""
    import oracle
    q, k, v, g, beta, cu, d_o = args
    oracle.recurrent_forward(q, k, v, g, beta, cu, None)
    oracle.recurrent_backward(q, k, v, g, beta, cu, None, d_o, None)
    return True


def cpu_baseline(b_pre_sets, H, D, make_batch, workload):
    """The fp64 oracle (the test oracle, unchanged) on bounded samples of the
    three workloads, timed on the host's cores: heads are independent, so the
    work is split by head over a process pool of one process per core; a
    one-core figure is kept beside it.  Returns the cpu_baseline object."""
    import concurrent.futures as cf
    import multiprocessing as mp

    import oracle
    from threadpoolctl import threadpool_limits

    cores = min(len(os.sched_getaffinity(0)), 16)
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"  # inherited by the pool's processes

    def split(b, with_do=False):
        per = [slice(h, h + 1) for h in range(b.num_heads)]
        out = []
        for sl in per:
            tail = (b.d_o[:, sl],) if with_do else ((None if b.h0 is None else b.h0[:, sl]),)
            out.append((b.q[:, sl], b.k[:, sl], b.v[:, sl], b.g[:, sl], b.beta[:, sl], b.cu_seqlens) + tail)
        return out

    ctx = mp.get_context("spawn")  # fresh interpreters: nothing of this GPU process is shared
    with cf.ProcessPoolExecutor(max_workers=cores, mp_context=ctx) as pool:
        list(pool.map(_oracle_forward_heads, split(b_pre_sets[0])[:cores]))  # start the workers
        # prefill: the three 5 x 2,048 input sets the GPU rotates through
        t0 = time.perf_counter()
        jobs = [j for bs in b_pre_sets for j in split(bs)]
        list(pool.map(_oracle_forward_heads, jobs))
        t_pre = time.perf_counter() - t0
        n_pre = sum(bs.total_tokens for bs in b_pre_sets)
        # one decode step of 256 sequences x 16 heads from nonzero states
        bd = make_batch(3, [1] * 256, H, D, D, "bf16", h0_std=0.1)
        t0 = time.perf_counter()
        list(pool.map(_oracle_forward_heads, split(bd)))
        t_dec = time.perf_counter() - t0
        # trainer forward + backward: the first 512 tokens of the 1 x 10,240 workload
        bt, _, _, _ = workload("train_1x10240")
        bt = bt.truncate([512])
        t0 = time.perf_counter()
        list(pool.map(_oracle_fwd_bwd_heads, split(bt, with_do=True)))
        t_fb = time.perf_counter() - t0
    # one core: the first prefill set
    with threadpool_limits(limits=1):
        b0 = b_pre_sets[0]
        t0 = time.perf_counter()
        oracle.recurrent_forward(b0.q, b0.k, b0.v, b0.g, b0.beta, b0.cu_seqlens, None)
        t_one = time.perf_counter() - t0
    return {"value": round(n_pre / t_pre, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"fp64 token recurrence (NumPy; heads split over {cores} single-threaded processes) over the "
                      f"three 5 x 2048 prefill input sets the GPU rotates through ({n_pre} tokens, 16 heads, d=128): "
                      f"{t_pre:.1f} s; host has {len(os.sched_getaffinity(0))} cores available",
            "one_core": {"value": round(b0.total_tokens / t_one, 2), "unit": "tokens/s", "cores": 1,
                         "sample": f"the first 5 x 2048 set on one thread: {t_one:.1f} s"},
            "decode_step": {"value": round(256 / t_dec, 2), "unit": "tokens/s", "cores": cores,
                            "sample": f"one decode step, 256 sequences x 16 heads from N(0, 0.1) states: {t_dec:.2f} s"},
            "fwd_bwd": {"value": round(bt.total_tokens / t_fb, 2), "unit": "tokens/s", "cores": cores,
                        "sample": f"oracle forward + analytic backward on the first {bt.total_tokens} tokens of the "
                                  f"1 x 10240 trainer workload (16 heads): {t_fb:.2f} s"}}


def kernel_source_digest():
    """sha256 over the HIP sources and the C header (the code the counters were taken on)."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "bitwise_invariant_gated_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".hpp", ".h")):
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    with open(os.path.join(ROOT, "include", "gdn_cpr.h"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM-side bytes per launch of `kernel` from the committed PMC summary, or None when the
    kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic_counters.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != kernel_source_digest():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k.get("bytes_per_launch")


def stats(xs):
    """mean, median, p90 and min of per-step HIP-event times (ms)"""
    a = np.asarray(xs, dtype=np.float64)
    return {"mean": round(float(a.mean()), 5), "median": round(float(np.median(a)), 5),
            "p90": round(float(np.percentile(a, 90)), 5), "min": round(float(a.min()), 5)}


def _gfx_clock_from(data):
    """First graphics-clock reading (MHz) in amd-smi or rocm-smi JSON output."""
    import re
    if isinstance(data, dict):
        for key, val in data.items():
            k = str(key).lower()
            if k.startswith("gfx") and isinstance(val, dict):
                clk = val.get("clk", val)
                v = clk.get("value") if isinstance(clk, dict) else None
                if isinstance(v, (int, float)) and v > 0:
                    return float(v)
            if k.startswith("sclk clock speed") and isinstance(val, str):
                m = re.search(r"(\d+)\s*mhz", val.lower())
                if m:
                    return float(m.group(1))
        for val in data.values():
            r = _gfx_clock_from(val)
            if r:
                return r
    elif isinstance(data, list):
        for val in data:
            r = _gfx_clock_from(val)
            if r:
                return r
    return None


def read_gfx_clock():
    """(MHz, command) of GPU 0's current graphics clock from amd-smi, else
    rocm-smi (child processes), or (None, None)."""
    import subprocess
    for cmd in (["amd-smi", "metric", "--clock", "--json"], ["rocm-smi", "--showclocks", "--json"]):
        try:
            out = subprocess.run(cmd, capture_output=True, text=True, timeout=20).stdout
            v = _gfx_clock_from(json.loads(out))
        except Exception:
            continue
        if v:
            return v, " ".join(cmd)
    return None, None


def clock_under_load(run, max_s=30.0):
    """Read the graphics clock once while run() is issued back to back."""
    import threading

    import torch
    res = []
    th = threading.Thread(target=lambda: res.append(read_gfx_clock()), daemon=True)
    th.start()
    t_end = time.perf_counter() + max_s
    n = 0
    while th.is_alive() and time.perf_counter() < t_end:
        run()
        n += 1
        if n % 32 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    th.join(timeout=1.0)
    return res[0] if res else (None, None)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the graphics-clock reading (about a second of extra prefills), e.g. under a profiler")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="before timing, run one plain device copy of this many MiB (a known-size "
                         "kernel that scales the FETCH_SIZE / WRITE_SIZE counters of a --pmc run)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this layer's work is sharded by sequence/head with "
              "no exchange, so there is no multi-GPU step to time (run with --gpus 1)", file=sys.stderr)
        return 2

    import torch

    import bitwise_invariant_gated_amd as gdn
    from gdn_synth import make_batch, workload

    dev = "cuda"
    torch.cuda.set_device(0)
    H, D, C = 16, 128, 64
    shape = gdn.LayerShape(H, D, D, C, torch.bfloat16)

    def to_dev(b):
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(torch.bfloat16)
        return dict(q=t(b.q), k=t(b.k), v=t(b.v), g=t(b.g), beta=t(b.beta),
                    cu=torch.from_numpy(b.cu_seqlens).to(dev))

    # ---- prefill inputs: three draws of the 5 x 2,048 workload, rotated so
    # that repeats are not served from the 256 MB last-level cache
    log("generating prefill inputs")
    b_pre, _, _, _ = workload("prefill_5x2048")
    sets = [to_dev(b_pre)] + [to_dev(make_batch(200 + r, [2048] * 5, H, D, D, "bf16")) for r in range(2)]
    T = b_pre.total_tokens
    N_pre = b_pre.num_seqs
    caches = [gdn.alloc_cache(shape, N_pre, dev) for _ in sets]
    outs = [torch.empty((T, H, D), dtype=torch.bfloat16, device=dev) for _ in sets]
    ws_pre = gdn.alloc_workspace(shape, N_pre, T, gdn.GDN_OP_PREFILL, dev)

    # ---- decode: 256 sequences with a 2,048-token prefix, then decode tokens
    log("generating decode inputs (256 x 2,048-token prefixes)")
    n_dec_tok = args.warmup + args.steps + 64
    b_dec = make_batch(3, [2048 + n_dec_tok] * 256, H, D, D, "bf16")
    dd = to_dev(b_dec)
    N_dec = 256
    rows_all = (torch.from_numpy(b_dec.cu_seqlens[:-1].astype(np.int64)).to(dev)[None, :]
                + torch.arange(2048, 2048 + n_dec_tok, device=dev)[:, None])  # [steps, N]
    dec_in = {n: dd[n][rows_all].contiguous() for n in ("q", "k", "v", "g", "beta")}
    b_prefix = b_dec.truncate([2048] * 256)
    dp = to_dev(b_prefix)
    cache_dec = gdn.alloc_cache(shape, N_dec, dev)
    o_prefix = torch.empty((b_prefix.total_tokens, H, D), dtype=torch.bfloat16, device=dev)
    ws_big = gdn.alloc_workspace(shape, N_dec, b_prefix.total_tokens, gdn.GDN_OP_PREFILL, dev)
    log("prefilling the decode prefix")
    gdn.gdn_cpr_prefill(shape, dp["q"], dp["k"], dp["v"], dp["g"], dp["beta"], dp["cu"], None,
                        cache_dec, o_prefix, ws_big)
    del ws_big, o_prefix, dp
    ws_dec = gdn.alloc_workspace(shape, N_dec, 0, gdn.GDN_OP_DECODE, dev)
    o_dec = torch.empty((N_dec, H, D), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)  # reads and writes copy_probe_mib MiB
        torch.cuda.synchronize()
        del src, dst

    stream = torch.cuda.current_stream()
    pre_ev = gdn.StageEvents(5)
    dec_ev = gdn.StageEvents(3)
    scan_ms, chain_ms, local_ms, prefill_ms, decode_ms = [], [], [], [], []
    dstep_ms, dres_ms = [], []
    dstep = [0]

    def step(timed):
        r = dstep[0] % len(sets)
        s = sets[r]
        with pre_ev:
            gdn.gdn_cpr_prefill(shape, s["q"], s["k"], s["v"], s["g"], s["beta"], s["cu"], None,
                                caches[r], outs[r], ws_pre)
        i = dstep[0]
        with dec_ev:
            gdn.gdn_cpr_decode_step(shape, dec_in["q"][i], dec_in["k"][i], dec_in["v"][i],
                                    dec_in["g"][i], dec_in["beta"][i], cache_dec, o_dec, ws_dec)
        dstep[0] += 1
        if timed:
            torch.cuda.synchronize()  # per-step event readout; the step total is timed separately
            local_ms.append(pre_ev.stage_ms(2))
            chain_ms.append(pre_ev.stage_ms(3))
            scan_ms.append(pre_ev.stage_ms(4))
            prefill_ms.append(pre_ev.events[0].elapsed_time(pre_ev.events[4]))
            decode_ms.append(dec_ev.events[0].elapsed_time(dec_ev.events[2]))
            dstep_ms.append(dec_ev.stage_ms(1))
            dres_ms.append(dec_ev.stage_ms(2))

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    # timed region 1: K steps back to back (whole-step wall time)
    start_step = dstep[0]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        r = dstep[0] % len(sets)
        s = sets[r]
        gdn.gdn_cpr_prefill(shape, s["q"], s["k"], s["v"], s["g"], s["beta"], s["cu"], None,
                            caches[r], outs[r], ws_pre)
        i = dstep[0]
        gdn.gdn_cpr_decode_step(shape, dec_in["q"][i], dec_in["k"][i], dec_in["v"][i],
                                dec_in["g"][i], dec_in["beta"][i], cache_dec, o_dec, ws_dec)
        dstep[0] += 1
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = e0.elapsed_time(e1)
    log(f"timed {args.steps} steps: {total_ms:.3f} ms (host wall {wall * 1e3:.3f} ms)")
    # timed region 2: per-stage events (same work, one step at a time)
    dstep[0] = start_step  # decode tokens advance regardless; keep rows in range
    dstep[0] = args.warmup + args.steps
    for _ in range(min(args.steps, 32)):
        if dstep[0] >= n_dec_tok:
            break
        step(True)
    ms_per_step = total_ms / args.steps
    toks = T + N_dec
    value = toks / (ms_per_step / 1e3)
    clk_mhz, clk_src = None, None
    if not args.no_clock:
        log("graphics clock under the prefill (amd-smi)")
        s0c = sets[0]
        clk_mhz, clk_src = clock_under_load(
            lambda: gdn.gdn_cpr_prefill(shape, s0c["q"], s0c["k"], s0c["v"], s0c["g"], s0c["beta"], s0c["cu"], None,
                                        caches[0], outs[0], ws_pre))

    # ---- decode over 64 consecutive steps (one chunk: exactly one resync per
    # sequence) on a fresh copy of the 2,048-token-prefix cache
    log("decode: 64 consecutive steps (one resynchronisation)")
    b_dec64 = make_batch(3, [2048 + 64] * 256, H, D, D, "bf16")
    d64 = to_dev(b_dec64)
    rows64 = (torch.from_numpy(b_dec64.cu_seqlens[:-1].astype(np.int64)).to(dev)[None, :]
              + torch.arange(2048, 2048 + 64, device=dev)[:, None])
    dec64 = {n: d64[n][rows64].contiguous() for n in ("q", "k", "v", "g", "beta")}
    c64 = gdn.alloc_cache(shape, N_dec, dev)
    bp64 = b_dec64.truncate([2048] * 256)
    dp64 = to_dev(bp64)
    ws_big = gdn.alloc_workspace(shape, N_dec, bp64.total_tokens, gdn.GDN_OP_PREFILL, dev)
    o_big = torch.empty((bp64.total_tokens, H, D), dtype=torch.bfloat16, device=dev)
    gdn.gdn_cpr_prefill(shape, dp64["q"], dp64["k"], dp64["v"], dp64["g"], dp64["beta"], dp64["cu"], None,
                        c64, o_big, ws_big)
    del ws_big, o_big, dp64, d64
    torch.cuda.synchronize()
    e2, e3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e2.record(stream)
    for i in range(64):
        gdn.gdn_cpr_decode_step(shape, dec64["q"][i], dec64["k"][i], dec64["v"][i], dec64["g"][i],
                                dec64["beta"][i], c64, o_dec, ws_dec)
    e3.record(stream)
    torch.cuda.synchronize()
    dec64_ms = e2.elapsed_time(e3) / 64

    # ---- the same decode call recorded in a HIP graph and replayed (as a
    # serving loop would run it): a step in which no tail fills, then the
    # replays' mean over a whole chunk (one resync per sequence)
    log("decode: one call recorded in a graph, replayed")
    c_gr = c64.clone()
    x_gr = {n: dec64[n][0].clone() for n in dec64}
    run_gr = lambda: gdn.gdn_cpr_decode_step(shape, x_gr["q"], x_gr["k"], x_gr["v"], x_gr["g"], x_gr["beta"], c_gr,
                                             o_dec, ws_dec)
    s_side = torch.cuda.Stream()
    s_side.wait_stream(stream)
    with torch.cuda.stream(s_side):
        run_gr()
    stream.wait_stream(s_side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run_gr()
    torch.cuda.synchronize()
    graph.replay()  # the cache's tails now hold 2 tokens: the next 62 replays resync nothing
    torch.cuda.synchronize()
    e2.record(stream)
    for _ in range(32):
        graph.replay()
    e3.record(stream)
    torch.cuda.synchronize()
    dec_graph_ms = e2.elapsed_time(e3) / 32
    e2.record(stream)
    for _ in range(64):
        graph.replay()
    e3.record(stream)
    torch.cuda.synchronize()
    dec_graph64_ms = e2.elapsed_time(e3) / 64
    del graph, c_gr

    # ---- multi-token decode through the continuation call: 4 tokens for each
    # of the 256 cached sequences per call (from the cache after the 64-step
    # series), against 4 single-token decode steps on a copy of that cache
    log("continuation: 256 sequences x 4 tokens per call")
    n_tok = 4
    c_cont = c64.clone()
    c_dec = c64.clone()
    b_c = make_batch(3, [2048 + 64 + n_tok] * 256, H, D, D, "bf16")
    dc = to_dev(b_c)
    rows_c = (torch.from_numpy(b_c.cu_seqlens[:-1].astype(np.int64)).to(dev)[:, None]
              + torch.arange(2048 + 64, 2048 + 64 + n_tok, device=dev)[None, :]).reshape(-1)
    cont_in = {n: dc[n][rows_c].contiguous() for n in ("q", "k", "v", "g", "beta")}
    dec_in4 = {n: cont_in[n].view(256, n_tok, *cont_in[n].shape[1:]).transpose(0, 1).contiguous()
               for n in cont_in}
    cu_c = torch.arange(0, 256 * n_tok + 1, n_tok, dtype=torch.int32, device=dev)
    ws_c = gdn.alloc_workspace(shape, N_dec, 256 * n_tok, gdn.GDN_OP_PREFILL_CONTINUE, dev)
    o_c = torch.empty((256 * n_tok, H, D), dtype=torch.bfloat16, device=dev)
    o_d4 = torch.empty((n_tok, N_dec, H, D), dtype=torch.bfloat16, device=dev)
    del dc
    e4, e5, e6 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    torch.cuda.synchronize()
    e4.record(stream)
    gdn.gdn_cpr_prefill_continue(shape, cont_in["q"], cont_in["k"], cont_in["v"], cont_in["g"],
                                 cont_in["beta"], cu_c, c_cont, o_c, ws_c)
    e5.record(stream)
    for j in range(n_tok):
        gdn.gdn_cpr_decode_step(shape, dec_in4["q"][j], dec_in4["k"][j], dec_in4["v"][j], dec_in4["g"][j],
                                dec_in4["beta"][j], c_dec, o_d4[j], ws_dec)
    e6.record(stream)
    torch.cuda.synchronize()
    cont_ms, dec4_ms = e4.elapsed_time(e5), e5.elapsed_time(e6)
    cont_bitwise = bool(torch.equal(o_c.view(256, n_tok, H, D).transpose(0, 1).contiguous().view(torch.int16),
                                    o_d4.view(torch.int16))
                        and torch.equal(c_cont.s_run.view(torch.int32), c_dec.s_run.view(torch.int32))
                        and torch.equal(c_cont.run_log_scale.view(torch.int32), c_dec.run_log_scale.view(torch.int32)))

    # ---- head dim 256 (bf16): the 5 x 2,048 prefill at H = 16, and a decode
    # step of 64 sequences x 16 heads from a 256-token prefix (no tail fills)
    log("head dim 256: prefill 5 x 2,048 and a 64-sequence decode step")
    D2, N2 = 256, 64
    shape2 = gdn.LayerShape(H, D2, D2, C, torch.bfloat16)
    s2 = to_dev(make_batch(210, [2048] * 5, H, D2, D2, "bf16"))
    ws2 = gdn.alloc_workspace(shape2, N_pre, T, gdn.GDN_OP_PREFILL, dev)
    c2 = gdn.alloc_cache(shape2, N_pre, dev)
    o2 = torch.empty((T, H, D2), dtype=torch.bfloat16, device=dev)
    run2 = lambda: gdn.gdn_cpr_prefill(shape2, s2["q"], s2["k"], s2["v"], s2["g"], s2["beta"], s2["cu"], None,
                                       c2, o2, ws2)
    run2()
    torch.cuda.synchronize()
    ta, tb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ta.record(stream)
    for _ in range(5):
        run2()
    tb.record(stream)
    torch.cuda.synchronize()
    pre2_ms = ta.elapsed_time(tb) / 5
    del ws2, c2, o2, s2
    b2d = make_batch(211, [256 + 8] * N2, H, D2, D2, "bf16")
    d2 = to_dev(b2d)
    rows2 = (torch.from_numpy(b2d.cu_seqlens[:-1].astype(np.int64)).to(dev)[None, :]
             + torch.arange(256, 264, device=dev)[:, None])
    dec2 = {n: d2[n][rows2].contiguous() for n in ("q", "k", "v", "g", "beta")}
    p2 = to_dev(b2d.truncate([256] * N2))
    c2d = gdn.alloc_cache(shape2, N2, dev)
    ws2 = gdn.alloc_workspace(shape2, N2, 256 * N2, gdn.GDN_OP_PREFILL, dev)
    o2 = torch.empty((256 * N2, H, D2), dtype=torch.bfloat16, device=dev)
    gdn.gdn_cpr_prefill(shape2, p2["q"], p2["k"], p2["v"], p2["g"], p2["beta"], p2["cu"], None, c2d, o2, ws2)
    del ws2, o2, p2, d2
    ws2d = gdn.alloc_workspace(shape2, N2, 0, gdn.GDN_OP_DECODE, dev)
    o2d = torch.empty((N2, H, D2), dtype=torch.bfloat16, device=dev)
    dec2_call = lambda j: gdn.gdn_cpr_decode_step(shape2, dec2["q"][j], dec2["k"][j], dec2["v"][j], dec2["g"][j],
                                                  dec2["beta"][j], c2d, o2d, ws2d)
    dec2_call(0)
    torch.cuda.synchronize()
    ta.record(stream)
    for j in range(1, 8):
        dec2_call(j)
    tb.record(stream)
    torch.cuda.synchronize()
    dec2_ms = ta.elapsed_time(tb) / 7
    dec2_bytes = N2 * H * (2 * D2 * D2 * 4 + 2 * 4 + 3 * D2 * 2 + 2 * 2 + D2 * 2 + (2 * D2 + 2) * 2)
    del c2d, ws2d, dec2
    # fwd_bwd at d = 256 on the trainer shape: the prefill's forward, the
    # fp32-product backward kernels and the bf16-operand reverse chain
    log("head dim 256: fwd_bwd 1 x 10,240")
    b2t = make_batch(212, [10240], H, D2, D2, "bf16", with_do=True)
    t2 = to_dev(b2t)
    t2_do = torch.from_numpy(b2t.d_o).to(dev).to(torch.bfloat16)
    T2 = b2t.total_tokens
    ws2f = gdn.alloc_workspace(shape2, 1, T2, gdn.GDN_OP_FWD_BWD, dev)
    o2f = torch.empty((T2, H, D2), dtype=torch.bfloat16, device=dev)
    g2f = [torch.empty((T2, H, D2), dtype=torch.bfloat16, device=dev) for _ in range(3)]
    dg2f, db2f = (torch.empty((T2, H), dtype=torch.float32, device=dev) for _ in range(2))
    fb2_ev = gdn.StageEvents(7)

    def fb2():
        gdn.gdn_cpr_fwd_bwd(shape2, t2["q"], t2["k"], t2["v"], t2["g"], t2["beta"], t2["cu"], None, t2_do, None,
                            o2f, None, g2f[0], g2f[1], g2f[2], dg2f, db2f, None, ws2f)

    fb2()
    torch.cuda.synchronize()
    fb2_ms, fb2_fwd, fb2_grads = [], [], []
    for _ in range(3):
        with fb2_ev:
            fb2()
        torch.cuda.synchronize()
        fb2_ms.append(fb2_ev.events[0].elapsed_time(fb2_ev.events[6]))
        fb2_fwd.append(fb2_ev.events[0].elapsed_time(fb2_ev.events[4]))
        fb2_grads.append(fb2_ev.stage_ms(6))
    del ws2f, o2f, g2f, dg2f, db2f, t2, t2_do
    fb2_t = float(np.median(fb2_ms))
    fb2_g = float(np.median(fb2_grads))
    fb2_flop = bwd_state_grads_flop(C, D2, D2) * (T2 // C) * H
    flops2 = 7.0 * D2 * D2 * T * H
    head_dim_256 = {
        "prefill": {"workload": "5 x 2048 tokens, H = 16, d_k = d_v = 256, bf16", "ms": round(pre2_ms, 4),
                    "tokens_per_s": round(T / (pre2_ms / 1e3), 1),
                    "roofline": {"what": "the whole prefill call against the scan's fp32 work (7 d^2 per token-head)",
                                 "bound": "alu", "algorithmic_flop": flops2,
                                 "achieved": round(flops2 / (pre2_ms / 1e3) / 1e12, 3), "peak": PEAK_F32,
                                 "unit": "TFLOP/s",
                                 "frac": round(flops2 / (pre2_ms / 1e3) / 1e12 / PEAK_F32, 4),
                                 "frac_vs_nonpacked_issue_peak":
                                     round(flops2 / (pre2_ms / 1e3) / 1e12 / PEAK_VALU_F32_NONPACKED, 4)}},
        "decode": {"workload": "64 sequences x 1 token, H = 16, d_k = d_v = 256, 256-token prefix (no resync)",
                   "ms": round(dec2_ms, 5), "tokens_per_s": round(N2 / (dec2_ms / 1e3), 1),
                   "roofline": {"bound": "hbm", "algorithmic_bytes_per_call": dec2_bytes,
                                "achieved": round(dec2_bytes / (dec2_ms / 1e3) / 1e9, 1), "peak": PEAK_HBM,
                                "unit": "GB/s", "frac": round(dec2_bytes / (dec2_ms / 1e3) / 1e9 / PEAK_HBM, 4),
                                "note": "whole decode call (the empty resync pass included)"}},
        "fwd_bwd": {"workload": "1 x 10240 tokens, H = 16, d_k = d_v = 256, bf16", "ms": round(fb2_t, 4),
                    "tokens_per_s": round(T2 / (fb2_t / 1e3), 1),
                    "stage_ms": {"forward": round(float(np.median(fb2_fwd)), 4),
                                 "local_and_reverse_chain": round(float(np.median(fb2_ms)) - float(np.median(fb2_fwd))
                                                                  - fb2_g, 4),
                                 "state_and_gradients": round(fb2_g, 4)},
                    "roofline": {"what": "the state and gradient kernel (k_bwd_grads, fp32 MFMA) against the "
                                         "chunk-form gradient's products over their nonzero tiles",
                                 "bound": "mfma", "algorithmic_flop": fb2_flop,
                                 "achieved": round(fb2_flop / (fb2_g / 1e3) / 1e12, 3), "peak": PEAK_MFMA_F32,
                                 "unit": "TFLOP/s", "frac": round(fb2_flop / (fb2_g / 1e3) / 1e12 / PEAK_MFMA_F32, 4)}}}

    # ---- trainer forward + backward, 1 x 10,240 tokens
    log("fwd_bwd: 1 x 10,240 tokens")
    # three input draws (each with its own dO) and output sets, rotated as for
    # the prefill so that repeats are not served from the last-level cache
    b_tr, _, _, _ = workload("train_1x10240")
    b_trs = [b_tr] + [make_batch(400 + r, [10240], H, D, D, "bf16", with_do=True) for r in range(2)]
    trs = [to_dev(b) for b in b_trs]
    for b, x in zip(b_trs, trs):
        x["do"] = torch.from_numpy(b.d_o).to(dev).to(torch.bfloat16)
    T4 = b_tr.total_tokens
    ws_tr = gdn.alloc_workspace(shape, 1, T4, gdn.GDN_OP_FWD_BWD, dev)
    bf = dict(dtype=torch.bfloat16, device=dev)
    outs4 = []
    for _ in trs:
        outs4.append(dict(o=torch.empty((T4, H, D), **bf), dq=torch.empty((T4, H, D), **bf),
                          dk=torch.empty((T4, H, D), **bf), dv=torch.empty((T4, H, D), **bf),
                          dg=torch.empty((T4, H), dtype=torch.float32, device=dev),
                          db=torch.empty((T4, H), dtype=torch.float32, device=dev)))
    fb_ev = gdn.StageEvents(7)
    fb_i = [0]

    def fwd_bwd():
        r = fb_i[0] % len(trs)
        fb_i[0] += 1
        x, y = trs[r], outs4[r]
        gdn.gdn_cpr_fwd_bwd(shape, x["q"], x["k"], x["v"], x["g"], x["beta"], x["cu"], None, x["do"],
                            None, y["o"], None, y["dq"], y["dk"], y["dv"], y["dg"], y["db"], None, ws_tr)

    # warm-up: the calls before this block (head dim 256, 24 ms each) leave the
    # chip in another state; ten calls settle it
    for _ in range(10):
        fwd_bwd()
    torch.cuda.synchronize()
    # the bf16 call runs the backward local terms, reverse chain and state and
    # gradient stages on a second stream beside the forward (see
    # gdn_cpr_fwd_bwd): events 0 -> 4 span the forward, 0 -> 5 end when the
    # reverse chain and the forward chain are both done (event 5 is recorded on
    # the second stream), 5 -> 6 is the state and gradient stages (and the
    # join back)
    fb_ms, fb_fwd, fb_bchain, fb_grads = [], [], [], []
    for _ in range(48):
        with fb_ev:
            fwd_bwd()
        torch.cuda.synchronize()
        fb_ms.append(fb_ev.events[0].elapsed_time(fb_ev.events[6]))
        fb_fwd.append(fb_ev.events[0].elapsed_time(fb_ev.events[4]))
        fb_bchain.append(fb_ev.events[0].elapsed_time(fb_ev.events[5]))
        fb_grads.append(fb_ev.stage_ms(6))
    del ws_tr, trs, outs4

    # ---- comparators (not CPR) on the same inputs: prefill 5 x 2,048 and the
    # 256-sequence decode step, plus the prefill/decode agreement on the last
    # token of each prefill sequence
    log("comparators: recurrent-everywhere and chunkwise (native) prefill, recurrent decode")
    s0 = sets[0]
    cmp_res = {}
    st_cmp = torch.empty((N_pre, H, D, D), dtype=torch.float32, device=dev)
    o_cmp = torch.empty((T, H, D), dtype=torch.bfloat16, device=dev)
    last = torch.from_numpy(b_pre.cu_seqlens[1:].astype(np.int64) - 1).to(dev)
    bpre_1 = b_pre.truncate([2047] * 5)
    p1 = to_dev(bpre_1)
    x_last = {n: s0[n][last].contiguous() for n in ("q", "k", "v", "g", "beta")}
    for name, mode in (("recurrent_everywhere", gdn.GDN_CMP_RECURRENT), ("chunkwise_native", gdn.GDN_CMP_CHUNKWISE)):
        ws_cmp = gdn.gdn_cmp_workspace(shape, mode, N_pre, T, dev)
        run = lambda: gdn.gdn_cmp_prefill(shape, mode, s0["q"], s0["k"], s0["v"], s0["g"], s0["beta"], s0["cu"],
                                          None, st_cmp, o_cmp, ws_cmp)
        run()
        torch.cuda.synchronize()
        ta, tb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 3
        ta.record(stream)
        for _ in range(reps):
            run()
        tb.record(stream)
        torch.cuda.synchronize()
        pre_ms = ta.elapsed_time(tb) / reps
        o_full = o_cmp[last].clone()
        st1 = torch.empty_like(st_cmp)
        o1 = torch.empty((bpre_1.total_tokens, H, D), dtype=torch.bfloat16, device=dev)
        gdn.gdn_cmp_prefill(shape, mode, p1["q"], p1["k"], p1["v"], p1["g"], p1["beta"], p1["cu"], None, st1, o1,
                            gdn.gdn_cmp_workspace(shape, mode, N_pre, bpre_1.total_tokens, dev))
        o_dl = torch.empty((N_pre, H, D), dtype=torch.bfloat16, device=dev)
        gdn.gdn_cmp_decode_step(shape, x_last["q"], x_last["k"], x_last["v"], x_last["g"], x_last["beta"], st1, o_dl)
        torch.cuda.synchronize()
        cmp_res[name] = {"prefill_ms": round(pre_ms, 5),
                         "prefill_tokens_per_s": round(T / (pre_ms / 1e3), 1),
                         "decode_after_prefill_equals_prefill_bitwise":
                             bool(torch.equal(o_dl.view(torch.int16), o_full.view(torch.int16))),
                         "max_abs_decode_minus_prefill": float(torch.max(torch.abs(o_dl.float() - o_full.float())))}
        del ws_cmp
    # recurrent decode step (no tail, no resync) on the 256-sequence state
    st_dec = cache_dec.s_run.clone()
    o_rd = torch.empty((N_dec, H, D), dtype=torch.bfloat16, device=dev)
    i0 = 0
    gdn.gdn_cmp_decode_step(shape, dec_in["q"][i0], dec_in["k"][i0], dec_in["v"][i0], dec_in["g"][i0],
                            dec_in["beta"][i0], st_dec, o_rd)
    torch.cuda.synchronize()
    ta, tb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ta.record(stream)
    for j in range(8):
        gdn.gdn_cmp_decode_step(shape, dec_in["q"][j], dec_in["k"][j], dec_in["v"][j], dec_in["g"][j],
                                dec_in["beta"][j], st_dec, o_rd)
    tb.record(stream)
    torch.cuda.synchronize()
    cmp_res["recurrent_decode_step_ms"] = round(ta.elapsed_time(tb) / 8, 5)
    del st_dec, p1
    # chunkwise-everywhere decode: 64 consecutive steps (one chunk, one boundary
    # move per sequence) from the 2,112-token cache, beside CPR's 64-step mean
    c_cd = c64.clone()
    o_cd = torch.empty((N_dec, H, D), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    ta.record(stream)
    for i in range(64):
        gdn.gdn_cmp_chunk_decode_step(shape, dec64["q"][i], dec64["k"][i], dec64["v"][i], dec64["g"][i],
                                      dec64["beta"][i], c_cd, o_cd, ws_dec)
    tb.record(stream)
    torch.cuda.synchronize()
    cmp_res["chunkwise_decode_mean_over_64_steps_ms"] = round(ta.elapsed_time(tb) / 64, 5)
    cmp_res["cpr_decode_mean_over_64_steps_ms"] = round(dec64_ms, 5)
    del c_cd

    # ---- parity: decode the last token of every prefill sequence == prefill output
    log("parity check: prefill vs decode on the 5 x 2,048 workload")
    s = sets[0]
    bpre_1 = b_pre.truncate([2047] * 5)
    p1 = to_dev(bpre_1)
    cache_p = gdn.alloc_cache(shape, N_pre, dev)
    o_p = torch.empty((bpre_1.total_tokens, H, D), dtype=torch.bfloat16, device=dev)
    gdn.gdn_cpr_prefill(shape, p1["q"], p1["k"], p1["v"], p1["g"], p1["beta"], p1["cu"], None,
                        cache_p, o_p, ws_pre)
    last = torch.from_numpy(b_pre.cu_seqlens[1:].astype(np.int64) - 1).to(dev)
    ws_d5 = gdn.alloc_workspace(shape, N_pre, 0, gdn.GDN_OP_DECODE, dev)
    o_d5 = torch.empty((N_pre, H, D), dtype=torch.bfloat16, device=dev)
    gdn.gdn_cpr_decode_step(shape, s["q"][last].contiguous(), s["k"][last].contiguous(),
                            s["v"][last].contiguous(), s["g"][last].contiguous(),
                            s["beta"][last].contiguous(), cache_p, o_d5, ws_d5)
    c_full = gdn.alloc_cache(shape, N_pre, dev)
    o_full = torch.empty((T, H, D), dtype=torch.bfloat16, device=dev)
    gdn.gdn_cpr_prefill(shape, s["q"], s["k"], s["v"], s["g"], s["beta"], s["cu"], None,
                        c_full, o_full, ws_pre)
    torch.cuda.synchronize()
    parity_o = bool(torch.equal(o_d5.view(torch.int16), o_full[last].contiguous().view(torch.int16)))
    parity_s = bool(torch.equal(cache_p.s_run.view(torch.int32), c_full.s_run.view(torch.int32))
                    and torch.equal(cache_p.run_log_scale.view(torch.int32), c_full.run_log_scale.view(torch.int32)))

    # the chunk products, the boundary chain and the in-chunk scan run as one
    # launch for this batch (k_chain_scan_bf16): events 1 -> 4 span it, and
    # stages 3 and 4 alone are empty
    fused = float(np.mean(scan_ms)) < 0.02 and float(np.mean(chain_ms)) < 0.02
    launch_ms = np.asarray(local_ms) + np.asarray(chain_ms) + np.asarray(scan_ms) if fused else np.asarray(scan_ms)
    scan_avg = float(np.mean(launch_ms))
    flops_scan = 7.0 * D * D * T * H  # algorithmic: 7 flop per state entry per token-head
    achieved = flops_scan / (scan_avg / 1e3) / 1e12
    roofline = {
        "kernel": ("k_chain_scan_bf16 (chunk products + boundary chain + in-chunk recurrent scan, one launch; "
                   "the scan's fp32 flops counted)") if fused else "k_scan (in-chunk recurrent scan)",
        "bound": "alu",
        "achieved": round(achieved, 3),
        "peak": PEAK_F32,
        "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_F32, 4),
        "frac_vs_nonpacked_issue_peak": round(achieved / PEAK_VALU_F32_NONPACKED, 4),
        "nonpacked_issue_peak": round(PEAK_VALU_F32_NONPACKED, 1),
        "traffic": measured_traffic("k_chain_scan_bf16" if fused else "k_scan"),
        "algorithmic_flop_per_launch": flops_scan,
        "avg_launch_ms": round(scan_avg, 5),
    }
    pre_avg = float(np.mean(prefill_ms))
    prefill_roofline = {
        "what": "the whole prefill call (plan, chunk products, chain, scan) against the scan's fp32 work",
        "bound": "alu", "achieved": round(flops_scan / (pre_avg / 1e3) / 1e12, 3), "peak": PEAK_F32,
        "unit": "TFLOP/s", "frac": round(flops_scan / (pre_avg / 1e3) / 1e12 / PEAK_F32, 4),
        "roofline_us": round(flops_scan / (PEAK_F32 * 1e12) * 1e6, 1),
        "frac_vs_nonpacked_issue_peak": round(flops_scan / (pre_avg / 1e3) / 1e12 / PEAK_VALU_F32_NONPACKED, 4)}
    # the backward's state and gradient stages (one kernel, k_bwd_state_grads_bf16)
    # run after the join: their algorithmic fp32 product flops against the fp32
    # matrix peak, and the bf16 MFMA flops they execute against the bf16 peak
    n_chunk_heads = (T4 // C) * H
    fb_flop_ch = bwd_state_grads_flop(C, D, D)
    fb_flop = fb_flop_ch * n_chunk_heads
    fb_t = float(np.median(fb_grads))
    fb_exec_ch = bwd_state_grads_bf16_exec_flop(C, D, D)
    fb_roofline = {"kernels": "k_bwd_state_grads_bf16", "bound": "mfma",
                   "achieved": round(fb_flop / (fb_t / 1e3) / 1e12, 3), "peak": PEAK_MFMA_F32, "unit": "TFLOP/s",
                   "frac": round(fb_flop / (fb_t / 1e3) / 1e12 / PEAK_MFMA_F32, 4),
                   "algorithmic_flop_per_chunk_head": fb_flop_ch, "chunk_heads": n_chunk_heads,
                   "note": "fp32-class products taken as bf16 hi/lo parts on the bf16 MFMA; the fraction above is "
                           "the algorithmic fp32 work against the fp32 MFMA peak",
                   "executed_bf16_flop_per_chunk_head": fb_exec_ch,
                   "executed_bf16_tflops": round(fb_exec_ch * n_chunk_heads / (fb_t / 1e3) / 1e12, 2),
                   "executed_bf16_frac": round(fb_exec_ch * n_chunk_heads / (fb_t / 1e3) / 1e12 / PEAK_MFMA_BF16, 4)}
    dec_avg = float(np.mean(decode_ms))
    # per (sequence, head): state read + write, log-scale read + write, q/k/v, g/beta, o, tail append
    dec_bytes = N_dec * H * (2 * D * D * 4 + 2 * 4 + 3 * D * 2 + 2 * 2 + D * 2 + (2 * D + 2) * 2)
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "io_dtype": "bf16",
        "data": "synthetic (seeded GDN-shaped inputs; see gdn_synth)",
        "config": {"workload": "prefill 5x2048 tokens + decode 256 seqs x 1 token (2048-token prefix)",
                   "heads": H, "d_k": D, "d_v": D, "chunk": C, "state": "fp32"},
        "gpu_clock_mhz": {"gfx_under_prefill": clk_mhz, "source": clk_src},
        "timing_stats_ms": {"prefill": stats(prefill_ms),
                            "products_chain_and_scan" if fused else "scan": stats(launch_ms),
                            "decode_token_step": stats(dstep_ms), "decode_call": stats(decode_ms),
                            "samples": len(prefill_ms)},
        "prefill": {"ms": round(pre_avg, 5),
                    "tokens_per_s": round(T / (pre_avg / 1e3), 1),
                    "stage_ms": ({"plan": round(float(np.mean(prefill_ms)) - scan_avg, 5),
                                  "chunk_products_chain_and_scan": round(scan_avg, 5)} if fused else
                                 {"chunk_products": round(float(np.mean(local_ms)), 5),
                                  "boundary_chain": round(float(np.mean(chain_ms)), 5),
                                  "scan": round(scan_avg, 5)}),
                    "roofline": prefill_roofline},
        "decode": {"ms": round(dec_avg, 5), "tokens_per_s": round(N_dec / (dec_avg / 1e3), 1),
                   "stage_ms": {"token_step": round(float(np.mean(dstep_ms)), 5),
                                "resync_pass": round(float(np.mean(dres_ms)), 5)},
                   "roofline": {"kernel": "k_decode (per-token step, state read-modify-write)",
                                "bound": "hbm", "algorithmic_bytes_per_launch": dec_bytes,
                                "achieved": round(dec_bytes / (float(np.mean(dstep_ms)) / 1e3) / 1e9, 1),
                                "peak": PEAK_HBM, "unit": "GB/s",
                                "traffic": measured_traffic("k_decode"),
                                "frac": round(dec_bytes / (float(np.mean(dstep_ms)) / 1e3) / 1e9 / PEAK_HBM, 4)},
                   "whole_call_GBps": round(dec_bytes / (dec_avg / 1e3) / 1e9, 1),
                   "mean_over_64_steps_ms": round(dec64_ms, 5),
                   "mean_over_64_steps_tokens_per_s": round(N_dec / (dec64_ms / 1e3), 1),
                   "graph_replay": {"what": "one decode call captured in a HIP graph and replayed",
                                    "ms_no_resync": round(dec_graph_ms, 5),
                                    "mean_over_64_replays_ms": round(dec_graph64_ms, 5),
                                    "no_resync_tokens_per_s": round(N_dec / (dec_graph_ms / 1e3), 1)}},
        "fwd_bwd": {"workload": "1 x 10240 tokens", "ms": round(float(np.median(fb_ms)), 4),
                    "tokens_per_s": round(T4 / (float(np.median(fb_ms)) / 1e3), 1),
                    "streams": 2,
                    "stage_ms": {"forward": round(float(np.median(fb_fwd)), 4),
                                 "to_reverse_chain_joined": round(float(np.median(fb_bchain)), 4),
                                 "state_and_gradients": round(float(np.median(fb_grads)), 4)},
                    "roofline": fb_roofline},
        "continuation": {"workload": "256 cached sequences x 4 tokens in one gdn_cpr_prefill_continue call",
                         "ms": round(cont_ms, 5), "tokens_per_s": round(256 * n_tok / (cont_ms / 1e3), 1),
                         "four_decode_steps_ms": round(dec4_ms, 5),
                         "equals_four_decode_steps_bitwise": cont_bitwise},
        "head_dim_256": head_dim_256,
        "comparators": cmp_res,
        "parity": {"decode_o_equals_prefill_o_bitwise": parity_o,
                   "decode_state_equals_prefill_state_bitwise": parity_s},
        "roofline": roofline,
    }

    if not args.no_cpu_baseline:
        log("CPU baseline: fp64 oracle on the host's cores (prefill sets, a decode step, a fwd+bwd sample)")
        sample = [b_pre] + [make_batch(200 + r, [2048] * 5, H, D, D, "bf16") for r in range(2)]
        result["cpu_baseline"] = cpu_baseline(sample, H, D, make_batch, workload)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
