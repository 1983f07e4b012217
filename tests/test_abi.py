"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, sizes workspaces, and rejects bad arguments on the host
before enqueueing anything (no call here reaches a kernel launch)."""

import ctypes
import os
import re

import pytest

from bitwise_invariant_gated_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib_or_skip():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("library not built")
    return _lib.load()


def test_header_declares_exactly_the_bound_symbols():
    with open(os.path.join(ROOT, "include", "gdn_cpr.h")) as f:
        text = f.read()
    declared = set(re.findall(r"\b(gdn_(?:cpr|cmp)_[a-z_]+)\s*\(", text))
    assert declared == set(_lib.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = _lib_or_skip()
    for name in _lib.EXPORTED:
        assert hasattr(lib, name), name


def _shape(H=2, dk=64, dv=64, C=64, dtype=_lib.GDN_DTYPE_BF16):
    return _lib.Shape(H, dk, dv, C, dtype)


def test_workspace_size_shapes():
    lib = _lib_or_skip()
    s = _shape(16, 128, 128)
    n_pre = lib.gdn_cpr_workspace_size(ctypes.byref(s), 5, 10240, _lib.GDN_OP_PREFILL)
    n_dec = lib.gdn_cpr_workspace_size(ctypes.byref(s), 256, 0, _lib.GDN_OP_DECODE)
    assert n_pre > 5 * 16 * 32 * 128 * 128 * 4  # at least one fp32 boundary state per chunk
    assert n_dec > 256 * 16 * 4
    assert n_pre % 256 == 0 and n_dec % 256 == 0
    # shorter chunks: more chunk slots and boundary states for the same tokens
    n32 = lib.gdn_cpr_workspace_size(ctypes.byref(_shape(16, 128, 128, C=32)), 5, 10240, _lib.GDN_OP_PREFILL)
    n16 = lib.gdn_cpr_workspace_size(ctypes.byref(_shape(16, 128, 128, C=16)), 5, 10240, _lib.GDN_OP_PREFILL)
    assert n16 > n32 > n_pre
    assert lib.gdn_cmp_workspace_size(ctypes.byref(_shape(16, 128, 128, C=32)), _lib.GDN_CMP_CHUNKWISE, 5, 10240) == 0
    bad = _shape(16, 96, 128)
    assert lib.gdn_cpr_workspace_size(ctypes.byref(bad), 5, 10240, _lib.GDN_OP_PREFILL) == 0
    assert lib.gdn_cpr_workspace_size(ctypes.byref(s), -1, 10240, _lib.GDN_OP_PREFILL) == 0


def test_head_dim_256_serves_bf16_prefill_decode_continuation_and_fwd_bwd_only():
    lib = _lib_or_skip()
    s = _shape(16, 256, 256)
    for op in (_lib.GDN_OP_PREFILL, _lib.GDN_OP_DECODE, _lib.GDN_OP_PREFILL_CONTINUE, _lib.GDN_OP_FWD_BWD):
        assert lib.gdn_cpr_workspace_size(ctypes.byref(s), 4, 4096, op) > 0, op
    # fwd_bwd at d = 256: per (chunk slot, head) Kt and -W^T (bf16), R, dDelta,
    # X, dB' and seven C x 256 fp32 arrays of the local and gradient kernels
    f1 = lib.gdn_cpr_workspace_size(ctypes.byref(s), 1, 64, _lib.GDN_OP_FWD_BWD)
    f2 = lib.gdn_cpr_workspace_size(ctypes.byref(s), 1, 128, _lib.GDN_OP_FWD_BWD)
    slot = 2 * 64 * 256 * 2 + 2 * 256 * 256 * 4 + 64 * 256 * 4 + 64 * 64 * 4 + 7 * 64 * 256 * 4
    assert f2 - f1 >= 16 * slot
    assert lib.gdn_cpr_workspace_size(ctypes.byref(_shape(16, 256, 256, dtype=_lib.GDN_DTYPE_F32)), 4, 4096,
                                      _lib.GDN_OP_PREFILL) == 0
    assert lib.gdn_cpr_workspace_size(ctypes.byref(_shape(16, 128, 256)), 4, 4096, _lib.GDN_OP_PREFILL) == 0
    assert lib.gdn_cmp_workspace_size(ctypes.byref(s), _lib.GDN_CMP_CHUNKWISE, 4, 4096) == 0
    # a d = 256 chunk-product slot: W and K~^T fragments in bf16, U in fp32 (128 KiB)
    n1 = lib.gdn_cpr_workspace_size(ctypes.byref(s), 1, 0, _lib.GDN_OP_DECODE)
    n2 = lib.gdn_cpr_workspace_size(ctypes.byref(s), 2, 0, _lib.GDN_OP_DECODE)
    assert n2 - n1 >= 16 * 128 * 1024


FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation fails first


def _cache(ptr=FAKE, slots=None, lgs=None):
    return _lib.Cache(ptr, ptr, ptr, ptr, ptr, ptr, ptr, slots, ptr if lgs is None else lgs)


def _prefill(lib, shape, N=2, T=128, cache=None, cu=FAKE, q=FAKE, ws=FAKE, ws_bytes=0, h0=None, hT=None):
    cache = cache if cache is not None else _cache()
    return lib.gdn_cpr_prefill(ctypes.byref(shape), N, T, q, FAKE, FAKE, FAKE, FAKE, cu, h0, hT,
                               ctypes.byref(cache), FAKE, ws, ws_bytes, None)


def test_prefill_rejects_unsupported_shapes():
    lib = _lib_or_skip()
    for s in (_shape(dk=96), _shape(dv=32), _shape(C=48), _shape(C=128), _shape(H=0), _shape(dtype=7),
              _shape(dk=256), _shape(dk=256, dv=256, dtype=_lib.GDN_DTYPE_F32)):
        assert _prefill(lib, s) == _lib.GDN_ERR_UNSUPPORTED
        assert lib.gdn_cpr_last_error()


def test_prefill_rejects_null_and_misaligned_pointers():
    lib = _lib_or_skip()
    s = _shape()
    assert _prefill(lib, s, cu=None) == _lib.GDN_ERR_INVALID_ARG
    assert b"cu_seqlens" in lib.gdn_cpr_last_error()
    assert _prefill(lib, s, q=None) == _lib.GDN_ERR_INVALID_ARG
    assert _prefill(lib, s, q=FAKE + 4) == _lib.GDN_ERR_INVALID_ARG
    assert b"aligned" in lib.gdn_cpr_last_error()
    assert _prefill(lib, s, h0=FAKE + 8) == _lib.GDN_ERR_INVALID_ARG
    assert _prefill(lib, s, hT=FAKE + 8) == _lib.GDN_ERR_INVALID_ARG
    assert b"hT" in lib.gdn_cpr_last_error()
    assert _prefill(lib, s, hT=FAKE) == _lib.GDN_ERR_INVALID_ARG  # the fake cache's s_bnd
    assert b"aliases" in lib.gdn_cpr_last_error()
    assert _prefill(lib, s, cache=_cache(0)) == _lib.GDN_ERR_INVALID_ARG
    assert _prefill(lib, s, cache=_cache(lgs=0)) == _lib.GDN_ERR_INVALID_ARG
    assert b"run_log_scale" in lib.gdn_cpr_last_error()
    assert _prefill(lib, s, N=-1) == _lib.GDN_ERR_INVALID_ARG


def test_prefill_rejects_small_workspace():
    lib = _lib_or_skip()
    s = _shape()
    need = lib.gdn_cpr_workspace_size(ctypes.byref(s), 2, 128, _lib.GDN_OP_PREFILL)
    assert _prefill(lib, s, ws_bytes=need - 1) == _lib.GDN_ERR_WORKSPACE
    assert _prefill(lib, s, ws=None, ws_bytes=need) == _lib.GDN_ERR_WORKSPACE
    assert b"workspace" in lib.gdn_cpr_last_error()


def test_prefill_empty_batch_is_a_no_op():
    lib = _lib_or_skip()
    assert _prefill(lib, _shape(), N=0, T=0) == _lib.GDN_OK
    assert lib.gdn_cpr_last_error() == b""


def test_decode_rejects_bad_arguments():
    lib = _lib_or_skip()
    s = _shape()
    cache = _cache()

    def dec(shape=s, N=4, q=FAKE, ws=FAKE, ws_bytes=0, c=cache, hT=None):
        return lib.gdn_cpr_decode_step(ctypes.byref(shape), N, q, FAKE, FAKE, FAKE, FAKE,
                                       ctypes.byref(c), hT, FAKE, ws, ws_bytes, None)

    assert dec(shape=_shape(dk=32)) == _lib.GDN_ERR_UNSUPPORTED
    assert dec(q=None) == _lib.GDN_ERR_INVALID_ARG
    assert dec(c=_cache(FAKE + 2)) == _lib.GDN_ERR_INVALID_ARG
    assert dec(c=_cache(FAKE, FAKE + 4)) == _lib.GDN_ERR_INVALID_ARG
    assert b"slot_index" in lib.gdn_cpr_last_error()
    assert dec(c=_cache(lgs=0)) == _lib.GDN_ERR_INVALID_ARG
    assert b"run_log_scale" in lib.gdn_cpr_last_error()
    assert dec(hT=FAKE + 4) == _lib.GDN_ERR_INVALID_ARG
    assert dec(hT=FAKE) == _lib.GDN_ERR_INVALID_ARG
    assert b"aliases" in lib.gdn_cpr_last_error()
    assert dec(ws_bytes=16) == _lib.GDN_ERR_WORKSPACE
    assert dec(N=0) == _lib.GDN_OK


def test_noalloc_decode_rejects_bad_arguments_and_sizes():
    lib = _lib_or_skip()
    s = _shape()

    def dec(shape=s, N=4, q=FAKE, c=_cache(), hT=None):
        return lib.gdn_cpr_decode_step_noalloc(ctypes.byref(shape), N, q, FAKE, FAKE, FAKE, FAKE,
                                               ctypes.byref(c), hT, FAKE, None)

    assert dec(shape=_shape(dk=32)) == _lib.GDN_ERR_UNSUPPORTED
    assert dec(q=None) == _lib.GDN_ERR_INVALID_ARG
    assert dec(c=_cache(FAKE, FAKE + 4)) == _lib.GDN_ERR_INVALID_ARG
    assert b"slot_index" in lib.gdn_cpr_last_error()
    assert dec(hT=FAKE) == _lib.GDN_ERR_INVALID_ARG
    assert b"aliases" in lib.gdn_cpr_last_error()
    # the fixed scratch: flags for 65,536 (sequence, head) pairs ...
    assert dec(N=32769) == _lib.GDN_ERR_UNSUPPORTED
    assert b"pairs" in lib.gdn_cpr_last_error()
    # ... and chunk products for 1,024 heads at d = 128 bf16 (64 KiB each)
    assert dec(shape=_shape(H=1025, dk=128, dv=128), N=1) == _lib.GDN_ERR_UNSUPPORTED
    assert b"heads" in lib.gdn_cpr_last_error()
    assert dec(N=0) == _lib.GDN_OK


def test_cache_state_rejects_bad_arguments():
    lib = _lib_or_skip()
    s = _shape()

    def st(shape=s, N=2, c=_cache(), out=FAKE + 256):
        return lib.gdn_cpr_cache_state(ctypes.byref(shape), N, ctypes.byref(c) if c is not None else None, out, None)

    assert st(shape=_shape(dk=96)) == _lib.GDN_ERR_UNSUPPORTED
    assert st(c=None) == _lib.GDN_ERR_INVALID_ARG
    assert st(out=None) == _lib.GDN_ERR_INVALID_ARG
    assert st(out=FAKE + 260) == _lib.GDN_ERR_INVALID_ARG
    assert st(c=_cache(lgs=0)) == _lib.GDN_ERR_INVALID_ARG
    assert b"run_log_scale" in lib.gdn_cpr_last_error()
    assert st(out=FAKE) == _lib.GDN_ERR_INVALID_ARG  # aliases s_run
    assert b"aliases" in lib.gdn_cpr_last_error()
    assert st(N=-1) == _lib.GDN_ERR_INVALID_ARG
    assert st(N=0) == _lib.GDN_OK


def test_prefill_continue_rejects_bad_arguments():
    lib = _lib_or_skip()
    s = _shape()

    def cont(shape=s, N=2, T=128, q=FAKE, cu=FAKE, ws=FAKE, ws_bytes=0, c=_cache(), hT=None):
        return lib.gdn_cpr_prefill_continue(ctypes.byref(shape), N, T, q, FAKE, FAKE, FAKE, FAKE, cu,
                                            ctypes.byref(c), hT, FAKE, ws, ws_bytes, None)

    assert cont(shape=_shape(C=8)) == _lib.GDN_ERR_UNSUPPORTED
    assert cont(cu=None) == _lib.GDN_ERR_INVALID_ARG
    assert cont(q=FAKE + 2) == _lib.GDN_ERR_INVALID_ARG
    assert cont(c=_cache(0)) == _lib.GDN_ERR_INVALID_ARG
    assert cont(hT=FAKE + 4) == _lib.GDN_ERR_INVALID_ARG
    assert cont(hT=FAKE) == _lib.GDN_ERR_INVALID_ARG
    assert b"aliases" in lib.gdn_cpr_last_error()
    need = lib.gdn_cpr_workspace_size(ctypes.byref(s), 2, 128, _lib.GDN_OP_PREFILL_CONTINUE)
    assert need >= lib.gdn_cpr_workspace_size(ctypes.byref(s), 2, 128, _lib.GDN_OP_PREFILL)
    assert cont(ws_bytes=need - 1) == _lib.GDN_ERR_WORKSPACE
    assert cont(N=0, T=0) == _lib.GDN_OK


def test_numerics_id_is_stable_text():
    lib = _lib_or_skip()
    a = lib.gdn_cpr_numerics_id()
    assert a and a == lib.gdn_cpr_numerics_id()


def _pinned_order_lines():
    """The formulas of the per-token step's pinned order, as the comment above
    token_step in cpr_device.hpp states them."""
    with open(os.path.join(ROOT, "bitwise_invariant_gated_amd", "csrc", "cpr_device.hpp")) as f:
        text = f.read()
    block = text[text.index("// Order (pinned), lane j (state column j)."):].splitlines()
    lines = [next(ln for ln in block if "--" in ln).split("--")[1].strip()]  # the first-term products
    start = next(k for k, ln in enumerate(block) if ln.startswith("//   pass A"))
    for ln in block[start:]:
        if not ln.startswith("//   "):
            break
        lines.extend(part.strip() for part in ln[2:].split(";  "))
    return [" ".join(x.split()) for x in lines if x]


def test_numerics_id_states_the_pinned_token_step_order():
    """The identity text must name the per-token step's order exactly as the
    device code's comment pins it (equal text is meant to mean equal bits)."""
    lib = _lib_or_skip()
    ident = " ".join(lib.gdn_cpr_numerics_id().decode().split())
    lines = _pinned_order_lines()
    assert len(lines) == 6, lines
    for ln in lines:
        assert ln in ident, ln
    assert "C in {16, 32, 64}" in ident
    # the key split at d_k = 256, as the device code's comment states it
    with open(os.path.join(ROOT, "bitwise_invariant_gated_amd", "csrc", "cpr_device.hpp")) as f:
        dev = " ".join(f.read().split())
    for formula in ("w = b * (v - c * (P_lo + P_hi))", "o = c * (O_lo + O_hi)"):
        assert formula in dev and formula in ident, formula


def test_wait_status_rejects_bad_arguments():
    lib = _lib_or_skip()
    s = _shape()
    need = lib.gdn_cpr_workspace_size(ctypes.byref(s), 2, 300, _lib.GDN_OP_PREFILL)

    def ws(shape=s, N=2, T=300, w=FAKE + 4096, nbytes=need, status=FAKE + 256):
        return lib.gdn_cpr_wait_status(ctypes.byref(shape), N, T, w, nbytes, status, None)

    assert ws(shape=_shape(dk=96)) == _lib.GDN_ERR_UNSUPPORTED
    assert ws(N=-1) == _lib.GDN_ERR_INVALID_ARG
    assert ws(T=-1) == _lib.GDN_ERR_INVALID_ARG
    assert ws(status=None) == _lib.GDN_ERR_INVALID_ARG
    assert ws(status=FAKE + 260) == _lib.GDN_ERR_INVALID_ARG
    assert ws(w=None) == _lib.GDN_ERR_WORKSPACE
    assert ws(nbytes=need - 1) == _lib.GDN_ERR_WORKSPACE
    assert b"workspace" in lib.gdn_cpr_last_error()
    assert ws(w=FAKE + 4100) == _lib.GDN_ERR_INVALID_ARG


def test_debug_wait_polls_rejects_a_negative_count():
    lib = _lib_or_skip()
    assert lib.gdn_cpr_debug_set_wait_polls(-1) == _lib.GDN_ERR_INVALID_ARG
