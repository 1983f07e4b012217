"""Pins for the CPU fp64 oracle (CPU only).

Each check ties the oracle to something other than itself: the literal matrix
form of the update, a hand-worked example, closed forms of special cases,
exact store/retrieve, agreement of two independently written evaluation
orders, an independent autodiff, and finite differences.  A final group plants
plausible mistakes in copies of the oracle and asserts that the pins catch
them.
"""

import os

import numpy as np
import pytest

import oracle
from oracle import chunkwise as ocw
from oracle import recurrent as orec
from gdn_synth import make_batch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
_REAL_STEP = orec.token_step


def _rand_problem(seed, lengths, H=2, dk=5, dv=3, h0=True):
    b = make_batch(seed, lengths, H, dk, dv, dtype="f32", h0_std=0.5 if h0 else None,
                   with_do=True)
    return b


def _run_rec(b, step=None):
    return orec.recurrent_forward(b.q, b.k, b.v, b.g, b.beta, b.cu_seqlens, b.h0)


# ----------------------------------------------------------------------------
# the update rule itself


def _literal_step(M, q, k, v, g, beta):
    """M_t = alpha M (I - beta k k^T) + beta v k^T ; o = M_t q (one head)."""
    a = np.exp(g)
    dk = k.shape[0]
    Mn = a * M @ (np.eye(dk) - beta * np.outer(k, k)) + beta * np.outer(v, k)
    return Mn, Mn @ q


def check_step_against_literal(step_fn):
    rng = np.random.default_rng(7)
    err = 0.0
    for _ in range(20):
        dv, dk = 3, 5
        M = rng.standard_normal((1, dv, dk))
        q, k = rng.standard_normal((1, dk)), rng.standard_normal((1, dk))
        v = rng.standard_normal((1, dv))
        g = -np.abs(rng.standard_normal(1))
        beta = rng.uniform(0.05, 0.95, 1)
        Mn, o = step_fn(M, q, k, v, g, beta)
        Ml, ol = _literal_step(M[0], q[0], k[0], v[0], g[0], beta[0])
        err = max(err, np.max(np.abs(Mn[0] - Ml)), np.max(np.abs(o[0] - ol)))
    return err


def test_token_step_matches_literal_matrix_form():
    assert check_step_against_literal(oracle.token_step) < 1e-13


def _read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            vals[parts[0]] = np.array([float(x) for x in parts[1:]])
    return vals


def check_hand_example(forward_fn):
    gv = _read_golden("hand_two_token.txt")
    q = gv["q"].reshape(2, 1, 2)
    k = gv["k"].reshape(2, 1, 2)
    v = gv["v"].reshape(2, 1, 2)
    g = gv["g"].reshape(2, 1)
    beta = gv["beta"].reshape(2, 1)
    cu = np.array([0, 2], np.int32)
    o, hT = forward_fn(q, k, v, g, beta, cu, None)
    return max(np.max(np.abs(o.reshape(-1) - gv["o"])),
               np.max(np.abs(hT.reshape(-1) - gv["S_final"])))


def test_hand_worked_two_token_example():
    assert check_hand_example(oracle.recurrent_forward) < 1e-14
    f = lambda *a: oracle.chunkwise_forward(*a, chunk=2)
    assert check_hand_example(f) < 1e-14
    f1 = lambda *a: oracle.chunkwise_forward(*a, chunk=1)
    assert check_hand_example(f1) < 1e-14


# ----------------------------------------------------------------------------
# closed forms and exact special cases


def check_pure_decay(forward_fn):
    """beta = 0: S_t = exp(sum_{s<=t} g_s) S_0 and o_t = S_t^T q_t."""
    b = _rand_problem(11, [7, 5], H=2, dk=4, dv=3)
    b.beta[:] = 0.0
    o, hT = forward_fn(b.q, b.k, b.v, b.g, b.beta, b.cu_seqlens, b.h0)
    err = 0.0
    for i in range(b.num_seqs):
        sl = b.seq_slice(i)
        decay = np.exp(np.cumsum(b.g[sl].astype(np.float64), axis=0))  # [L,H]
        S0 = b.h0[i].astype(np.float64)  # [H,dk,dv]
        o_ref = decay[:, :, None] * np.einsum("hij,thi->thj", S0, b.q[sl].astype(np.float64))
        err = max(err, np.max(np.abs(o[sl] - o_ref)))
        err = max(err, np.max(np.abs(hT[i] - decay[-1][:, None, None] * S0)))
    return err


def test_beta_zero_is_pure_decay():
    assert check_pure_decay(oracle.recurrent_forward) < 1e-13
    assert check_pure_decay(lambda *a: oracle.chunkwise_forward(*a, chunk=3)) < 1e-13


def test_beta_zero_zero_state_gives_zero_output():
    b = _rand_problem(12, [9], h0=False)
    b.beta[:] = 0.0
    o, hT = oracle.recurrent_forward(b.q, b.k, b.v, b.g, b.beta, b.cu_seqlens, None)
    assert np.all(o == 0.0) and np.all(hT == 0.0)


def check_store_retrieve(forward_fn):
    """alpha = 1, beta = 1, orthonormal keys: writing v_j under k_j, then
    reading with q = k_j (beta = 0 so nothing is written) returns v_j."""
    rng = np.random.default_rng(3)
    d, n = 8, 6
    Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
    keys = Qm[:, :n].T  # n orthonormal rows
    vals = rng.standard_normal((n, 4))
    T = 2 * n
    q = np.zeros((T, 1, d))
    k = np.zeros((T, 1, d))
    v = np.zeros((T, 1, 4))
    g = np.zeros((T, 1))
    beta = np.zeros((T, 1))
    for j in range(n):
        k[j, 0] = keys[j]
        v[j, 0] = vals[j]
        beta[j, 0] = 1.0
        q[j, 0] = keys[j]  # reading right after writing also returns v_j
    for j in range(n):
        q[n + j, 0] = keys[j]
        k[n + j, 0] = keys[(j + 1) % n]
    o, _ = forward_fn(q, k, v, g, beta, np.array([0, T]), None)
    return max(np.max(np.abs(o[:n, 0] - vals)), np.max(np.abs(o[n:, 0] - vals)))


def test_store_and_retrieve_with_orthonormal_keys():
    assert check_store_retrieve(oracle.recurrent_forward) < 1e-13
    assert check_store_retrieve(lambda *a: oracle.chunkwise_forward(*a, chunk=4)) < 1e-13


def test_scalar_case_first_order_recurrence():
    """d_k = d_v = 1: s_t = alpha (1 - beta k^2) s_{t-1} + beta k v, o = s q."""
    b = _rand_problem(5, [13], H=1, dk=1, dv=1)
    o, hT = oracle.recurrent_forward(b.q, b.k, b.v, b.g, b.beta, b.cu_seqlens, b.h0)
    s = float(b.h0[0, 0, 0, 0])
    for t in range(13):
        a = np.exp(float(b.g[t, 0]))
        kk, vv, bb = float(b.k[t, 0, 0]), float(b.v[t, 0, 0]), float(b.beta[t, 0])
        s = a * (1 - bb * kk * kk) * s + bb * kk * vv
        assert abs(o[t, 0, 0] - s * float(b.q[t, 0, 0])) < 1e-14
    assert abs(hT[0, 0, 0, 0] - s) < 1e-14


# ----------------------------------------------------------------------------
# two independently written evaluation orders agree (brute force, tiny inputs)


@pytest.mark.parametrize("chunk", [1, 2, 3, 8, 64])
def test_chunkwise_equals_recurrent(chunk):
    b = _rand_problem(21, [1, 17, 64, 70, 0, 129], H=2, dk=6, dv=4)
    o_r, h_r = _run_rec(b)
    o_c, h_c = oracle.chunkwise_forward(b.q, b.k, b.v, b.g, b.beta, b.cu_seqlens, b.h0,
                                        chunk=chunk)
    assert np.max(np.abs(o_r - o_c)) < 1e-12
    assert np.max(np.abs(h_r - h_c)) < 1e-12


def test_chunk_boundaries_equal_recurrent_states():
    b = _rand_problem(22, [50], H=1, dk=5, dv=3)
    o, hT, states = orec.recurrent_forward(b.q, b.k, b.v, b.g, b.beta, b.cu_seqlens, b.h0,
                                           return_all_states=True)
    _, _, bounds = oracle.chunkwise_forward(b.q, b.k, b.v, b.g, b.beta, b.cu_seqlens, b.h0,
                                            chunk=16, return_boundaries=True)
    for c, t in enumerate([0, 16, 32, 48, 50]):
        assert np.max(np.abs(bounds[0][c] - np.swapaxes(states[0][t], -1, -2))) < 1e-12


def test_identity_padding_rows_leave_chunk_products_unchanged():
    """A token with k = v = 0, g = beta = 0 is the identity step (alpha = 1, no
    write), so padding a chunk of n < 64 tokens with such rows leaves the real
    rows of W, U, K~ and Gamma_n, and the chunk's boundary map, unchanged.
    This is the reading behind chunk lengths shorter than the 64-row slot."""
    rng = np.random.default_rng(31)
    for n in (16, 32, 47):
        K = rng.standard_normal((n, 6))
        K /= np.linalg.norm(K, axis=1, keepdims=True)
        V = rng.standard_normal((n, 4))
        g = -np.abs(rng.standard_normal(n)) * 0.2
        beta = 1.0 / (1.0 + np.exp(-rng.standard_normal(n)))
        pad = 64 - n
        Kp = np.vstack([K, np.zeros((pad, 6))])
        Vp = np.vstack([V, np.zeros((pad, 4))])
        gp = np.concatenate([g, np.zeros(pad)])
        bp = np.concatenate([beta, np.zeros(pad)])
        W, U, Kt, Gn, T, _, _ = oracle.chunk_products(K, V, g, beta)
        Wp, Up, Ktp, Gnp, Tp, _, _ = oracle.chunk_products(Kp, Vp, gp, bp)
        assert np.max(np.abs(Wp[:n] - W)) < 1e-13 and np.max(np.abs(Wp[n:])) == 0.0
        assert np.max(np.abs(Up[:n] - U)) < 1e-13 and np.max(np.abs(Up[n:])) == 0.0
        assert np.max(np.abs(Ktp[:n] - Kt)) < 1e-13 and np.max(np.abs(Ktp[n:])) == 0.0
        assert abs(Gnp - Gn) < 1e-15
        # the boundary map B' = Gamma_n B + (U - W B^T)^T K~ is the same
        B = rng.standard_normal((4, 6))
        Bn = Gn * B + (U - W @ B.T).T @ Kt
        Bnp = Gnp * B + (Up - Wp @ B.T).T @ Ktp
        assert np.max(np.abs(Bnp - Bn)) < 1e-13
    # the recurrence: identity tokens after a sequence leave its final state as it is
    b = _rand_problem(32, [40], H=1, dk=5, dv=3)
    _, h = _run_rec(b)
    z = np.zeros((24,) + b.q.shape[1:])
    o2, h2 = orec.recurrent_forward(np.concatenate([b.q, z]), np.concatenate([b.k, z]),
                                    np.concatenate([b.v, np.zeros((24,) + b.v.shape[1:])]),
                                    np.concatenate([b.g, np.zeros((24,) + b.g.shape[1:])]),
                                    np.concatenate([b.beta, np.zeros((24,) + b.beta.shape[1:])]),
                                    np.array([0, 64], np.int32), b.h0)
    assert np.array_equal(h2, h)


def test_chunk_products_T_is_inverse():
    rng = np.random.default_rng(4)
    n, dk, dv = 10, 6, 4
    K = rng.standard_normal((n, dk))
    K /= np.linalg.norm(K, axis=1, keepdims=True)
    V = rng.standard_normal((n, dv))
    g = -np.abs(rng.standard_normal(n)) * 0.1
    beta = rng.uniform(0.1, 0.9, n)
    W, U, Kt, Gn, T, D, Gam = ocw.chunk_products(K, V, g, beta)
    # T (I+L) structure: T diag(beta)^-1 inverts I + L, built here by hand
    L = np.zeros((n, n))
    for t in range(n):
        for s in range(t):
            L[t, s] = beta[t] * np.exp(np.sum(g[s + 1:t + 1])) * K[t] @ K[s]
    Tinv = np.linalg.inv(np.eye(n) + L)
    assert np.max(np.abs(T - Tinv * beta[None, :])) < 1e-13
    assert np.allclose(np.triu(T, 1), 0.0)
    assert abs(Gn - np.exp(np.sum(g))) < 1e-15


# ----------------------------------------------------------------------------
# structural invariants


def test_value_permutation_permutes_output():
    b = _rand_problem(31, [20, 9], H=2, dk=4, dv=5)
    o, hT = _run_rec(b)
    perm = np.array([3, 0, 4, 1, 2])
    b2 = make_batch(31, [20, 9], 2, 4, 5, dtype="f32", h0_std=0.5)
    b2.v = b.v[:, :, perm]
    b2.h0 = b.h0[:, :, :, perm]
    o2, hT2 = _run_rec(b2)
    assert np.max(np.abs(o2 - o[:, :, perm])) < 1e-13
    assert np.max(np.abs(hT2 - hT[:, :, :, perm])) < 1e-13


def test_sequences_and_heads_independent():
    b = _rand_problem(32, [11, 30, 4], H=3, dk=4, dv=4)
    o, hT = _run_rec(b)
    for i in range(3):
        bi = b.select([i])
        oi, hi = _run_rec(bi)
        assert np.array_equal(oi, o[b.seq_slice(i)])
        assert np.array_equal(hi[0], hT[i])
    # heads: reverse the head order
    bh = b.select([0, 1, 2])
    for name in ("q", "k", "v", "g", "beta"):
        setattr(bh, name, getattr(b, name)[:, ::-1].copy())
    bh.h0 = b.h0[:, ::-1].copy()
    oh, hh = _run_rec(bh)
    assert np.max(np.abs(oh[:, ::-1] - o)) < 1e-14


def test_linearity_in_values():
    b = _rand_problem(33, [25], h0=False)
    o1, _ = _run_rec(b)
    b.v = b.v.astype(np.float64) * 3.0
    o3, _ = _run_rec(b)
    assert np.max(np.abs(o3 - 3.0 * o1)) < 1e-12
    b2 = _rand_problem(33, [25], h0=True)
    o, h = _run_rec(b2)
    b2.v = b2.v.astype(np.float64) * -2.0
    b2.h0 = b2.h0.astype(np.float64) * -2.0
    o2, h2 = _run_rec(b2)
    assert np.max(np.abs(o2 + 2.0 * o)) < 1e-12


def test_chunk_size_independence():
    b = _rand_problem(34, [100, 37], H=2, dk=8, dv=8)
    o16, h16 = oracle.chunkwise_forward(b.q, b.k, b.v, b.g, b.beta, b.cu_seqlens, b.h0, chunk=16)
    o64, h64 = oracle.chunkwise_forward(b.q, b.k, b.v, b.g, b.beta, b.cu_seqlens, b.h0, chunk=64)
    assert np.max(np.abs(o16 - o64)) < 1e-12 and np.max(np.abs(h16 - h64)) < 1e-12


# ----------------------------------------------------------------------------
# backward: independent autodiff and finite differences


def _torch_literal_loss(q, k, v, g, beta, h0, d_o, d_hT, cu):
    import torch
    L = 0.0
    for i in range(len(cu) - 1):
        H = q.shape[1]
        for h in range(H):
            M = h0[i, h].T.clone()
            for t in range(int(cu[i]), int(cu[i + 1])):
                a = torch.exp(g[t, h])
                kt = k[t, h]
                M = a * M @ (torch.eye(kt.shape[0], dtype=torch.float64)
                             - beta[t, h] * torch.outer(kt, kt)) + beta[t, h] * torch.outer(v[t, h], kt)
                L = L + torch.dot(M @ q[t, h], d_o[t, h])
            L = L + torch.sum(M.T * d_hT[i, h])
    return L


def test_backward_matches_torch_autograd():
    import torch
    b = _rand_problem(41, [9, 14], H=2, dk=4, dv=3)
    rng = np.random.default_rng(5)
    d_hT = rng.standard_normal(b.h0.shape)
    ref = oracle.recurrent_backward(b.q, b.k, b.v, b.g, b.beta, b.cu_seqlens, b.h0, b.d_o, d_hT,
                                    checkpoint=4)
    ts = {n: torch.tensor(np.asarray(getattr(b, n), np.float64), requires_grad=True)
          for n in ("q", "k", "v", "g", "beta", "h0")}
    L = _torch_literal_loss(ts["q"], ts["k"], ts["v"], ts["g"], ts["beta"], ts["h0"],
                            torch.tensor(b.d_o, dtype=torch.float64),
                            torch.tensor(d_hT, dtype=torch.float64), b.cu_seqlens)
    L.backward()
    for n, key in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"), ("beta", "dbeta"),
                   ("h0", "dh0")):
        assert np.max(np.abs(ts[n].grad.numpy() - ref[key])) < 1e-12, n


def test_backward_matches_finite_differences():
    """64 tokens, one head, d = 16 (the trainer case shrunk); h = 1e-6 central
    differences agree with the analytic gradient to 1e-6 * max|grad|."""
    b = make_batch(4, [64], 1, 16, 16, dtype="bf16", h0_std=0.3, with_do=True)
    rng = np.random.default_rng(9)
    d_hT = rng.standard_normal(b.h0.shape)
    ref = oracle.recurrent_backward(b.q, b.k, b.v, b.g, b.beta, b.cu_seqlens, b.h0, b.d_o, d_hT)
    inputs = {n: np.asarray(getattr(b, n), np.float64) for n in ("q", "k", "v", "g", "beta", "h0")}
    # every entry of g and beta, a seeded sample of the others (full sweeps
    # take minutes; the sample still touches every token)
    fd = oracle.fd_gradients(inputs, b.cu_seqlens, b.d_o, d_hT, names=("g", "beta"))
    for n, key in (("g", "dg"), ("beta", "dbeta")):
        scale = np.max(np.abs(ref[key]))
        assert np.max(np.abs(fd[n] - ref[key])) <= 1e-6 * scale, n
    pick = np.random.default_rng(10)
    for n, key in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("h0", "dh0")):
        x = inputs[n]
        flat_idx = pick.choice(x.size, size=min(96, x.size), replace=False)
        scale = np.max(np.abs(ref[key]))
        for j in flat_idx:
            idx = np.unravel_index(j, x.shape)
            old = x[idx]
            x[idx] = old + 1e-6
            lp = oracle.loss_value(inputs, b.cu_seqlens, b.d_o, d_hT)
            x[idx] = old - 1e-6
            lm = oracle.loss_value(inputs, b.cu_seqlens, b.d_o, d_hT)
            x[idx] = old
            assert abs((lp - lm) / 2e-6 - ref[key][idx]) <= 1e-6 * scale, (n, idx)


# ----------------------------------------------------------------------------
# key and query heads shared by groups of value heads (oracle/heads.py)
def test_shared_key_heads_equal_one_head_runs():
    """Value head h of a grouped batch equals a one-head run on its own v, g,
    beta and state with key head h // G's query and key rows; the chunk form
    agrees with the token form on the grouped batch."""
    b = make_batch(51, [13, 40, 7], 6, 5, 3, dtype="f32", h0_std=0.5, num_key_heads=2)  # G = 3
    assert b.q.shape[1] == 2 and b.v.shape[1] == 6
    o, hT = oracle.recurrent_forward(b.q, b.k, b.v, b.g, b.beta, b.cu_seqlens, b.h0)
    oc, hc = oracle.chunkwise_forward(b.q, b.k, b.v, b.g, b.beta, b.cu_seqlens, b.h0, chunk=8)
    assert np.max(np.abs(oc - o)) < 1e-12 and np.max(np.abs(hc - hT)) < 1e-12
    for h in range(6):
        j = h // 3
        oh, hh = oracle.recurrent_forward(b.q[:, j:j + 1], b.k[:, j:j + 1], b.v[:, h:h + 1], b.g[:, h:h + 1],
                                          b.beta[:, h:h + 1], b.cu_seqlens, b.h0[:, h:h + 1])
        assert np.max(np.abs(oh[:, 0] - o[:, h])) < 1e-13, h
        assert np.max(np.abs(hh[:, 0] - hT[:, h])) < 1e-13, h


def test_shared_key_head_gradients_sum_over_the_group():
    """dq and dk of a shared key head are the sums of the one-head gradients
    of its value heads; every per-value-head gradient is that head's own."""
    b = make_batch(52, [9, 12], 4, 4, 3, dtype="f32", h0_std=0.5, with_do=True, num_key_heads=2)
    d_hT = np.random.default_rng(6).standard_normal(b.h0.shape)
    ref = oracle.recurrent_backward(b.q, b.k, b.v, b.g, b.beta, b.cu_seqlens, b.h0, b.d_o, d_hT, checkpoint=4)
    assert ref["dq"].shape == b.q.shape and ref["dk"].shape == b.k.shape
    for j in range(2):
        dq_sum = np.zeros_like(ref["dq"][:, j])
        dk_sum = np.zeros_like(ref["dk"][:, j])
        for h in (2 * j, 2 * j + 1):
            r = oracle.recurrent_backward(b.q[:, j:j + 1], b.k[:, j:j + 1], b.v[:, h:h + 1], b.g[:, h:h + 1],
                                          b.beta[:, h:h + 1], b.cu_seqlens, b.h0[:, h:h + 1], b.d_o[:, h:h + 1],
                                          d_hT[:, h:h + 1], checkpoint=4)
            dq_sum += r["dq"][:, 0]
            dk_sum += r["dk"][:, 0]
            for key in ("dv", "dg", "dbeta", "dh0"):
                assert np.max(np.abs(r[key][:, 0] - ref[key][:, h])) < 1e-12, (key, h)
        assert np.max(np.abs(dq_sum - ref["dq"][:, j])) < 1e-12
        assert np.max(np.abs(dk_sum - ref["dk"][:, j])) < 1e-12


def test_shared_key_head_gradients_match_finite_differences():
    """One key head shared by two value heads: central differences of the
    loss agree with the analytic dq and dk (h = 1e-6, 1e-6 * max|grad|)."""
    b = make_batch(53, [10], 2, 3, 3, dtype="f32", h0_std=0.3, with_do=True, num_key_heads=1)
    d_hT = np.random.default_rng(7).standard_normal(b.h0.shape)
    ref = oracle.recurrent_backward(b.q, b.k, b.v, b.g, b.beta, b.cu_seqlens, b.h0, b.d_o, d_hT)
    inputs = {n: np.asarray(getattr(b, n), np.float64) for n in ("q", "k", "v", "g", "beta", "h0")}
    fd = oracle.fd_gradients(inputs, b.cu_seqlens, b.d_o, d_hT, names=("q", "k"))
    for n, key in (("q", "dq"), ("k", "dk")):
        scale = np.max(np.abs(ref[key]))
        assert np.max(np.abs(fd[n] - ref[key])) <= 1e-6 * scale, n


# ----------------------------------------------------------------------------
# planted mistakes: each must be caught by at least one pin above


def _mut_sign(M, q, k, v, g, beta):
    a = np.exp(g)[:, None, None]
    Mp = a * M
    p = np.einsum("bji,bi->bj", Mp, k)
    u = beta[:, None] * (v + p)  # wrong sign
    Mn = Mp + u[:, :, None] * k[:, None, :]
    return Mn, np.einsum("bji,bi->bj", Mn, q)


def _mut_no_decay_in_p(M, q, k, v, g, beta):
    a = np.exp(g)[:, None, None]
    p = np.einsum("bji,bi->bj", M, k)  # projection before the decay
    u = beta[:, None] * (v - p)
    Mn = a * M + u[:, :, None] * k[:, None, :]
    return Mn, np.einsum("bji,bi->bj", Mn, q)


def _mut_output_before_update(M, q, k, v, g, beta):
    Mn, _ = _REAL_STEP(M, q, k, v, g, beta)
    return Mn, np.einsum("bji,bi->bj", np.exp(g)[:, None, None] * M, q)


def _mut_transposed_output(M, q, k, v, g, beta):
    Mn, _ = _REAL_STEP(M, q, k, v, g, beta)
    if Mn.shape[1] != Mn.shape[2]:
        # only defined for square states; make the mismatch visible anyway
        return Mn, np.einsum("bji,bi->bj", Mn, q) * 0.5
    return Mn, np.einsum("bij,bi->bj", Mn, q)


@pytest.mark.parametrize("mut", [_mut_sign, _mut_no_decay_in_p, _mut_output_before_update,
                                 _mut_transposed_output])
def test_pins_catch_planted_step_mistakes(mut, monkeypatch):
    assert check_step_against_literal(mut) > 1e-6
    monkeypatch.setattr(orec, "token_step", mut)
    caught = check_hand_example(orec.recurrent_forward) > 1e-6
    caught = caught or check_pure_decay(orec.recurrent_forward) > 1e-6
    caught = caught or check_store_retrieve(orec.recurrent_forward) > 1e-6
    assert caught


def test_pins_catch_planted_chunk_mistakes(monkeypatch):
    real = ocw.chunk_products

    def no_gamma_in_W(K, V, g, beta):
        W, U, Kt, Gn, T, D, Gam = real(K, V, g, beta)
        return T @ K, U, Kt, Gn, T, D, Gam  # dropped diag(Gamma) in W

    def wrong_e(K, V, g, beta):
        W, U, Kt, Gn, T, D, Gam = real(K, V, g, beta)
        return W, U, Gam[:, None] * K, Gn, T, D, Gam  # Gamma instead of e

    b = _rand_problem(21, [17, 64], H=2, dk=6, dv=4)
    o_r, h_r = _run_rec(b)
    for bad in (no_gamma_in_W, wrong_e):
        monkeypatch.setattr(ocw, "chunk_products", bad)
        o_c, h_c = ocw.chunkwise_forward(b.q, b.k, b.v, b.g, b.beta, b.cu_seqlens, b.h0, chunk=8)
        assert np.max(np.abs(o_r - o_c)) > 1e-6 or np.max(np.abs(h_r - h_c)) > 1e-6
    monkeypatch.setattr(ocw, "chunk_products", real)
