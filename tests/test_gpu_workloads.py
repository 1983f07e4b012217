"""Full-size workloads on the GPU: the decode case (256 sequences with a
2,048-token prefix, then 128 decode steps) and the varlen packed batch (64
sequences, lengths U[1, 8192], nonzero initial states, then 100 decode
steps).  Bitwise checks run on every sequence; the fp64 oracle (too slow for
the whole batch) checks a seeded sample of sequences.
"""

import numpy as np
import pytest
import torch

import oracle
from gdn_synth import workload

from gpu_util import DevBatch, as_f64, bits, decode_rows, note, prefill, state_of

pytestmark = pytest.mark.gpu


def _oracle_check(b, seqs, o_full, state_full, tol=2e-2):
    sub = b.select(seqs)
    o_ref, h_ref = oracle.recurrent_forward(sub.q, sub.k, sub.v, sub.g, sub.beta, sub.cu_seqlens, sub.h0)
    ob = as_f64(o_full)
    got = np.concatenate([ob[b.seq_slice(i)] for i in seqs], axis=0)
    err_o = float(np.max(np.abs(got - o_ref)))
    err_s = float(np.max(np.abs(as_f64(state_full)[seqs] - h_ref)))
    assert err_o <= tol and err_s <= tol, (err_o, err_s)
    return err_o, err_s


def test_decode_256_sequences_bitwise_equal_to_prefill():
    note("decode_256x1: 256 x (2048 prefill + 128 decode) vs 256 x 2176 prefill")
    b, pre, n_dec, _ = workload("decode_256x1")
    db = DevBatch(b)
    o_full, c_full = prefill(db)  # 256 x 2,176 tokens in one prefill
    dp = DevBatch(b.truncate(pre))
    _, c_dec = prefill(dp)
    del dp
    o_dec = decode_rows(db, pre, n_dec, c_dec)  # two resynchronisations per sequence
    torch.cuda.synchronize()
    ob, od = bits(o_full), bits(o_dec)
    for i in range(b.num_seqs):
        a0 = int(b.cu_seqlens[i]) + int(pre[i])
        assert np.array_equal(od[:, i], ob[a0:a0 + n_dec]), i
    for name in ("s_run", "run_log_scale", "s_bnd", "tail_len"):
        assert np.array_equal(bits(getattr(c_full, name)), bits(getattr(c_dec, name))), name
    err = _oracle_check(b, [0, 97, 255], o_full, state_of(db.shape, c_full))
    print(f"decode_256x1 sampled oracle error: o {err[0]:.2e}, state {err[1]:.2e}")


def test_varlen_64_alone_equals_packed_through_prefill_and_decode():
    note("varlen_64: packed vs alone, prefill + 100 decode steps")
    b, pre, n_dec, _ = workload("varlen_64")
    db = DevBatch(b)
    N = b.num_seqs
    # packed: prefill the prefixes, decode 100 steps
    _, c_pack = prefill(DevBatch(b.truncate(pre)))
    o_pack_dec = decode_rows(db, pre, n_dec, c_pack)
    # packed: one prefill over prefix + decode tokens (the reference for decode)
    o_full, c_full = prefill(db)
    torch.cuda.synchronize()
    ob = bits(o_full)
    od = bits(o_pack_dec)
    for i in range(N):
        a0 = int(b.cu_seqlens[i]) + int(pre[i])
        assert np.array_equal(od[:, i], ob[a0:a0 + n_dec]), i
    for name in ("s_run", "run_log_scale", "s_bnd", "tail_len"):
        assert np.array_equal(bits(getattr(c_full, name)), bits(getattr(c_pack, name))), name
    # alone: every sequence by itself, prefill of its prefix then 100 decode steps
    s_run_pack = bits(c_pack.s_run)
    lgs_pack = bits(c_pack.run_log_scale)
    s_bnd_pack = bits(c_pack.s_bnd)
    for i in range(N):
        bi = b.select([i])
        dbi = DevBatch(bi)
        oi, ci = prefill(DevBatch(bi.truncate([int(pre[i])])))
        oi_dec = decode_rows(dbi, np.array([pre[i]]), n_dec, ci)
        torch.cuda.synchronize()
        sl = b.seq_slice(i)
        full_i = ob[sl]
        assert np.array_equal(bits(oi), full_i[:int(pre[i])]), i
        assert np.array_equal(bits(oi_dec)[:, 0], full_i[int(pre[i]):]), i
        assert np.array_equal(bits(ci.s_run)[0], s_run_pack[i]), i
        assert np.array_equal(bits(ci.run_log_scale)[0], lgs_pack[i]), i
        assert np.array_equal(bits(ci.s_bnd)[0], s_bnd_pack[i]), i
    lengths = b.lengths
    sample = [int(np.argmin(lengths)), int(np.argmax(lengths)), 17]
    err = _oracle_check(b, sample, o_full, state_of(db.shape, c_full))
    print(f"varlen_64 sampled oracle error: o {err[0]:.2e}, state {err[1]:.2e}; "
          f"tokens {int(lengths.sum())}, lengths {int(lengths.min())}..{int(lengths.max())}")
