"""GPU: bf16 fwd_bwd called from two host threads at once.

Each calling thread gets its own second stream and events inside the
library, so two threads that call gdn_cpr_fwd_bwd concurrently, each on its
own stream with its own workspace and outputs, must get the same bits as one
call made alone.
"""

import threading

import pytest
import torch

import bitwise_invariant_gated_amd as gdn
from gdn_synth import make_batch

from gpu_util import DEV, DevBatch, note

pytestmark = pytest.mark.gpu

CALLS = 4


def _outputs(T, N, H, d):
    bf = dict(dtype=torch.bfloat16, device=DEV)
    f32 = dict(dtype=torch.float32, device=DEV)
    return dict(o=torch.empty((T, H, d), **bf), hT=torch.empty((N, H, d, d), **f32),
                dq=torch.empty((T, H, d), **bf), dk=torch.empty((T, H, d), **bf), dv=torch.empty((T, H, d), **bf),
                dg=torch.empty((T, H), **f32), dbeta=torch.empty((T, H), **f32), dh0=torch.empty((N, H, d, d), **f32))


def _bits(x):
    return x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32)


def test_two_threads_fwd_bwd_bitwise_equal_to_one_call():
    note("threads: two concurrent bf16 fwd_bwd callers")
    d = 128
    b = make_batch(711, [900, 300, 77], 4, d, d, dtype="bf16", h0_std=0.1, with_do=True)
    db = DevBatch(b)
    shape, N, T, H = db.shape, b.num_seqs, b.total_tokens, b.num_heads

    def call(x, ws, stream):
        gdn.gdn_cpr_fwd_bwd(shape, db.q, db.k, db.v, db.g, db.beta, db.cu, db.h0, db.d_o, None, x["o"], x["hT"],
                            x["dq"], x["dk"], x["dv"], x["dg"], x["dbeta"], x["dh0"], ws, stream=stream)

    ref = _outputs(T, N, H, d)
    call(ref, gdn.alloc_workspace(shape, N, T, gdn.GDN_OP_FWD_BWD), torch.cuda.current_stream())
    torch.cuda.synchronize()

    results, errors = [], []
    work = [(_outputs(T, N, H, d), gdn.alloc_workspace(shape, N, T, gdn.GDN_OP_FWD_BWD), torch.cuda.Stream())
            for _ in range(2)]
    torch.cuda.synchronize()
    start = threading.Barrier(2)

    def worker(x, ws, stream):
        try:
            with torch.cuda.stream(stream):
                start.wait()
                for _ in range(CALLS):
                    call(x, ws, stream)
            stream.synchronize()
            results.append(x)
        except Exception as e:  # reported below, on the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=w) for w in work]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    assert len(results) == 2
    for x in results:
        for name in ref:
            assert torch.equal(_bits(x[name]), _bits(ref[name])), name
