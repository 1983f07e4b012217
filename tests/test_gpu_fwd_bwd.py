"""GPU fwd_bwd: gradients against the CPU oracle's analytic backward (itself
pinned by autograd and finite differences in test_oracle.py), the forward
bit-identical to prefill, and reruns bit-identical.

Tolerances per gradient tensor (the output tolerances carried over to the
gradients): fp32 inputs max|err| <= 1e-5 * max|ref|; bf16 inputs
max|err| <= 2e-2 * max(1, max|ref|).  Each test prints the measured
max|err| / max|ref| per tensor.
"""

import numpy as np
import pytest
import torch

import bitwise_invariant_gated_amd as gdn
import oracle
from gdn_synth import make_batch, workload

from gpu_util import DEV, DevBatch, as_f64, bits, note, prefill, state_of, torch_dtype

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dh0")


def run_fwd_bwd(db, d_hT=None):
    b = db.b
    N, T, H = b.num_seqs, b.total_tokens, b.num_heads
    dt = torch_dtype(b)
    out = dict(
        o=torch.empty((T, H, b.d_v), dtype=dt, device=DEV),
        hT=torch.empty((N, H, b.d_k, b.d_v), dtype=torch.float32, device=DEV),
        dq=torch.empty((T, b.num_key_heads, b.d_k), dtype=dt, device=DEV),
        dk=torch.empty((T, b.num_key_heads, b.d_k), dtype=dt, device=DEV),
        dv=torch.empty((T, H, b.d_v), dtype=dt, device=DEV),
        dg=torch.empty((T, H), dtype=torch.float32, device=DEV),
        dbeta=torch.empty((T, H), dtype=torch.float32, device=DEV),
        dh0=torch.empty((N, H, b.d_k, b.d_v), dtype=torch.float32, device=DEV),
    )
    ws = gdn.alloc_workspace(db.shape, N, T, gdn.GDN_OP_FWD_BWD)
    dh = None if d_hT is None else torch.from_numpy(d_hT).to(DEV)
    gdn.gdn_cpr_fwd_bwd(db.shape, db.q, db.k, db.v, db.g, db.beta, db.cu, db.h0, db.d_o, dh,
                        out["o"], out["hT"], out["dq"], out["dk"], out["dv"], out["dg"],
                        out["dbeta"], out["dh0"], ws)
    return out


def check_grads(b, out, d_hT):
    ref = oracle.recurrent_backward(b.q, b.k, b.v, b.g, b.beta, b.cu_seqlens, b.h0, b.d_o, d_hT)
    errs = {}
    for n in NAMES:
        got = as_f64(out[n])
        r = ref[n]
        m = float(np.max(np.abs(r))) if r.size else 0.0
        err = float(np.max(np.abs(got - r))) if r.size else 0.0
        if b.dtype == "f32":
            tol = 1e-5 * m
        else:
            tol = 2e-2 * max(1.0, m)
        errs[n] = (err, tol, m)
    bad = {n: e for n, e in errs.items() if not e[0] <= e[1]}
    assert not bad, bad
    return errs


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (64, 128)])
def test_fwd_bwd_matches_oracle(dtype, dk, dv):
    note(f"fwd_bwd ragged {dtype} dk={dk} dv={dv}")
    lens = [1, 63, 64, 65, 130, 0, 200]
    b = make_batch(301, lens, 2, dk, dv, dtype=dtype, h0_std=0.1, with_do=True)
    rng = np.random.default_rng(5)
    d_hT = rng.standard_normal((len(lens), 2, dk, dv)).astype(np.float32)
    db = DevBatch(b)
    out = run_fwd_bwd(db, d_hT)
    torch.cuda.synchronize()
    errs = check_grads(b, out, d_hT)
    print({n: f"{e[0]:.2e}/{e[2]:.2e}" for n, e in errs.items()})


def test_fwd_bwd_forward_is_prefill_bitwise_and_rerun_identical():
    note("fwd_bwd forward == prefill, rerun")
    b = make_batch(302, [300, 64, 17], 3, 128, 128, dtype="bf16", h0_std=0.1, with_do=True)
    db = DevBatch(b)
    out1 = run_fwd_bwd(db)
    out2 = run_fwd_bwd(db)
    o_p, c_p = prefill(db)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out1["o"]), bits(o_p))
    assert np.array_equal(bits(out1["hT"]), bits(state_of(db.shape, c_p)))
    for n in ("o", "hT") + NAMES:
        assert np.array_equal(bits(out1[n]), bits(out2[n])), n


def test_fwd_bwd_zero_dO_gives_state_only_gradient():
    """dO = 0, dhT = 0: every gradient is exactly zero."""
    note("fwd_bwd zero upstream")
    b = make_batch(303, [70, 5], 2, 64, 64, dtype="bf16", h0_std=0.1, with_do=True)
    b.d_o[:] = 0.0
    out = run_fwd_bwd(DevBatch(b))
    torch.cuda.synchronize()
    for n in NAMES:
        assert float(torch.max(torch.abs(out[n].float()))) == 0.0, n


def test_train_1x10240_matches_oracle():
    """1 x 10,240 tokens, H=16, d=128, bf16, dO ~ N(0,1): the trainer shape."""
    note("fwd_bwd train 1x10240 vs oracle")
    b, _, _, _ = workload("train_1x10240")
    db = DevBatch(b)
    out = run_fwd_bwd(db)
    o_p, _ = prefill(db)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out["o"]), bits(o_p))
    errs = check_grads(b, out, None)
    print("train_1x10240:", {n: f"{e[0]:.2e}/{e[2]:.2e}" for n, e in errs.items()})
