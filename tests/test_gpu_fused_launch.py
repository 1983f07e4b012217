"""GPU: the one-launch prefill (chunk products, boundary chain and scan as the
tickets of one kernel) against the three-launch prefill.

A bf16 batch of at most 128 sequences whose chain items number at most 512
runs as one launch; one sequence more takes the three launches.  Since every
sequence's bits depend only on its own tokens, the 128 sequences of the first
batch must come out bit-identical in both runs: outputs, boundary and running
states, tails.  The lengths cover empty sequences, sequences shorter than one
chunk (no chunk-product item), exact multiples of the chunk and long ones.
"""

import numpy as np
import pytest
import torch

import oracle
from gdn_synth import make_batch

from gpu_util import DevBatch, as_f64, bits, note, prefill, state_of

pytestmark = pytest.mark.gpu


def lengths(seed, n):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 63, 64, 65, 128, 200, 0, 257]
    return fixed + [int(x) for x in rng.integers(0, 330, n - len(fixed))]


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128)])
def test_one_launch_equals_three_launches_bitwise(dk, dv):
    note(f"one-launch vs three-launch prefill dk={dk} dv={dv}")
    lens = lengths(930 + dk + dv, 129)  # 129 sequences: the last one only in the second batch
    b = make_batch(931 + dk, lens, 2, dk, dv, dtype="bf16", h0_std=0.1)
    b128 = b.select(range(128))
    o1, c1 = prefill(DevBatch(b128))   # 128 x 2 heads x dv/64 chain items <= 512: one launch
    o2, c2 = prefill(DevBatch(b))      # 129 sequences: three launches
    torch.cuda.synchronize()
    n128 = int(b128.cu_seqlens[-1])
    assert np.array_equal(bits(o1), bits(o2)[:n128])
    for name, t1, t2 in zip(("s_bnd", "s_run", "tail_k", "tail_v", "tail_g", "tail_beta", "tail_len",
                             "run_log_scale"), c1.tensors(), c2.tensors()):
        a1, a2 = bits(t1), bits(t2)[:128]
        if name.startswith("tail_") and name != "tail_len":
            tl = bits(c1.tail_len)
            for i in range(128):
                assert np.array_equal(a1[i, :, :tl[i, 0]], a2[i, :, :tl[i, 0]]), (name, i)
        else:
            assert np.array_equal(a1, a2), name
    # and a sample of the sequences against the oracle
    pick = [0, 1, 2, 3, 4, 5, 6, 8, 40, 127]
    bs = b128.select(pick)
    o_ref, h_ref = oracle.recurrent_forward(bs.q, bs.k, bs.v, bs.g, bs.beta, bs.cu_seqlens, bs.h0)
    rows = np.concatenate([np.arange(b128.cu_seqlens[i], b128.cu_seqlens[i + 1]) for i in pick])
    assert float(np.max(np.abs(as_f64(o1)[rows] - o_ref))) <= 2e-2
    st = as_f64(state_of(DevBatch(b128).shape, c1))[pick]
    assert float(np.max(np.abs(st - h_ref))) <= 2e-2
