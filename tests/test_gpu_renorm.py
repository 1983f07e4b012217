"""GPU: gates that decay hard enough to renormalise the scaled running state.

The per-token step keeps the running state as exp(lg) N, lg being the
cumulative log-decay since the chunk boundary; when lg would fall below -32
the token first multiplies N by exp(lg) and lg restarts at 0.  Synthetic gates
with g around -2.5 per token (and, separately, rare spikes of g = -20 or -40
in the usual gates) cross that threshold inside chunks.  Prefill must still
match the fp64 oracle, decode must still equal prefill bit for bit, and the
cache's run_log_scale must be the value the rule gives when replayed on the
host in fp32.
"""

import numpy as np
import pytest
import torch

import oracle
from gdn_synth import make_batch, round_to_bf16

from gpu_util import DevBatch, as_f64, bits, decode_rows, note, prefill, state_of, tol_for

pytestmark = pytest.mark.gpu

LENS = [1, 40, 63, 64, 65, 130, 200]
C = 64
RENORM_LOG = np.float32(-32.0)


def with_gates(b, seed, mode):
    """Replace b.g by strongly decaying gates (values exact in b's dtype)."""
    rng = np.random.default_rng(seed)
    if mode == "strong":
        g = -2.5 - 0.5 * np.abs(rng.standard_normal(b.g.shape))
    else:  # "spikes": the usual gates with rare large drops
        g = b.g.astype(np.float64).copy()
        u = rng.random(b.g.shape)
        g[u < 0.03] = -20.0
        g[u > 0.97] = -40.0
    g = g.astype(np.float32)
    b.g[:] = round_to_bf16(g) if b.dtype == "bf16" else g
    return b


def replay_log_scale(b):
    """lg after each sequence's last token under the renormalisation rule,
    in fp32, and the number of renormalising tokens: [N, H], int."""
    N, H = b.num_seqs, b.num_heads
    out = np.zeros((N, H), np.float32)
    n_ren = 0
    for i in range(N):
        L = int(b.cu_seqlens[i + 1] - b.cu_seqlens[i])
        r = L % C
        gs = b.g[int(b.cu_seqlens[i]) + L - r:int(b.cu_seqlens[i + 1])]  # the open chunk's tokens
        for h in range(H):
            lg = np.float32(0.0)
            for t in range(r):
                x = np.float32(lg + gs[t, h])
                if x < RENORM_LOG:
                    lg = np.float32(0.0)
                    n_ren += 1
                else:
                    lg = x
            out[i, h] = lg
    return out, n_ren


@pytest.mark.parametrize("mode", ["strong", "spikes"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_renormalising_prefill_matches_oracle(dtype, mode):
    note(f"renormalising prefill {dtype} {mode}")
    b = with_gates(make_batch(801, LENS, 2, 128, 128, dtype=dtype, h0_std=0.1), 901, mode)
    lg_ref, n_ren = replay_log_scale(b)
    assert n_ren > 0  # the data does cross the threshold inside open chunks
    db = DevBatch(b)
    o, c = prefill(db)
    torch.cuda.synchronize()
    assert np.array_equal(bits(c.run_log_scale), lg_ref.view(np.int32))
    o_ref, h_ref = oracle.recurrent_forward(b.q, b.k, b.v, b.g, b.beta, b.cu_seqlens, b.h0)
    err_o = float(np.max(np.abs(as_f64(o) - o_ref)))
    err_s = float(np.max(np.abs(as_f64(state_of(db.shape, c)) - h_ref)))
    assert err_o <= tol_for(b, float(np.max(np.abs(o_ref)))), err_o
    assert err_s <= tol_for(b, float(np.max(np.abs(h_ref)))), err_s


@pytest.mark.parametrize("mode", ["strong", "spikes"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_renormalising_decode_equals_prefill_bitwise(dtype, mode):
    note(f"renormalising decode == prefill {dtype} {mode}")
    full = np.array([140, 134, 200, 75, 261])
    steps = 70
    b = with_gates(make_batch(802, list(full), 2, 128, 128, dtype=dtype, h0_std=0.1), 902, mode)
    pre = full - steps
    db = DevBatch(b)
    o_full, c_full = prefill(db)
    _, c_dec = prefill(DevBatch(b.truncate(list(pre))))
    o_dec = decode_rows(db, pre, steps, c_dec)
    torch.cuda.synchronize()
    ob, od = bits(o_full), bits(o_dec)
    for i, L in enumerate(full):
        a = int(b.cu_seqlens[i])
        assert np.array_equal(od[:, i], ob[a + pre[i]:a + L]), i
    for name in ("s_run", "run_log_scale", "s_bnd", "tail_len"):
        assert np.array_equal(bits(getattr(c_full, name)), bits(getattr(c_dec, name))), name
