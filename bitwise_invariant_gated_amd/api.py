"""Python binding of the CPR Gated DeltaNet C ABI (include/gdn_cpr.h).

Argument marshalling only: torch tensors provide device memory and the HIP
stream; every step of the layer runs in the library's HIP kernels.  The
function names are the C names.
"""

from __future__ import annotations

import ctypes
import dataclasses
from typing import Optional

import torch

from . import _lib

_DTYPES = {torch.float32: _lib.GDN_DTYPE_F32, torch.bfloat16: _lib.GDN_DTYPE_BF16}


@dataclasses.dataclass(frozen=True)
class LayerShape:
    num_heads: int
    head_dim_k: int
    head_dim_v: int
    chunk: int = 64
    dtype: torch.dtype = torch.bfloat16
    num_key_heads: int = 0  # heads of q and k; 0 = num_heads

    def c(self) -> _lib.Shape:
        if self.dtype not in _DTYPES:
            raise ValueError(f"unsupported dtype {self.dtype}")
        return _lib.Shape(self.num_heads, self.head_dim_k, self.head_dim_v, self.chunk,
                          _DTYPES[self.dtype], self.num_key_heads)


@dataclasses.dataclass
class CprCache:
    """Device tensors of a gdn_cpr_cache (layouts in gdn_cpr.h).  s_run holds
    the running state in scaled form (the state is exp(run_log_scale) * s_run;
    gdn_cpr_cache_state writes it out).  slot_index (int32 [N] or None)
    selects the cache rows of a call's batch entries."""

    s_bnd: torch.Tensor
    s_run: torch.Tensor
    tail_k: torch.Tensor
    tail_v: torch.Tensor
    tail_g: torch.Tensor
    tail_beta: torch.Tensor
    tail_len: torch.Tensor
    run_log_scale: torch.Tensor
    slot_index: Optional[torch.Tensor] = None

    def c(self) -> _lib.Cache:
        si = None if self.slot_index is None else _ptr(self.slot_index)
        return _lib.Cache(_ptr(self.s_bnd), _ptr(self.s_run), _ptr(self.tail_k), _ptr(self.tail_v),
                          _ptr(self.tail_g), _ptr(self.tail_beta), _ptr(self.tail_len), si,
                          _ptr(self.run_log_scale))

    def clone(self) -> "CprCache":
        return CprCache(*(t.clone() for t in self.tensors()), self.slot_index)

    def with_slots(self, slot_index: Optional[torch.Tensor]) -> "CprCache":
        """The same cache arrays addressed through another row map."""
        return CprCache(*self.tensors(), slot_index)

    def tensors(self):
        """Every array of the cache (slot_index aside), in field order."""
        return (self.s_bnd, self.s_run, self.tail_k, self.tail_v, self.tail_g, self.tail_beta, self.tail_len,
                self.run_log_scale)


def alloc_cache(shape: LayerShape, num_seqs: int, device="cuda") -> CprCache:
    N, H, dk, dv, C = num_seqs, shape.num_heads, shape.head_dim_k, shape.head_dim_v, shape.chunk
    f32 = dict(dtype=torch.float32, device=device)
    dt = dict(dtype=shape.dtype, device=device)
    return CprCache(torch.zeros((N, H, dk, dv), **f32), torch.zeros((N, H, dk, dv), **f32),
                    torch.zeros((N, H, C, dk), **dt), torch.zeros((N, H, C, dv), **dt),
                    torch.zeros((N, H, C), **dt), torch.zeros((N, H, C), **dt),
                    torch.zeros((N, H), dtype=torch.int32, device=device), torch.zeros((N, H), **f32))


def gdn_cpr_cache_state(shape: LayerShape, cache: CprCache, num_seqs: Optional[int] = None, out=None,
                        stream=None) -> torch.Tensor:
    """The state after each cached sequence's last token, exp(run_log_scale) * s_run,
    as a new [N, H, d_k, d_v] fp32 tensor (or into `out`)."""
    lib = _lib.load()
    if num_seqs is None:
        num_seqs = int(cache.slot_index.numel()) if cache.slot_index is not None else int(cache.s_run.shape[0])
    if out is None:
        out = torch.empty((num_seqs, shape.num_heads, shape.head_dim_k, shape.head_dim_v), dtype=torch.float32,
                          device=cache.s_run.device)
    cc = cache.c()
    _lib.check(lib.gdn_cpr_cache_state(ctypes.byref(shape.c()), num_seqs, ctypes.byref(cc), _ptr(out),
                                       _stream(stream)))
    return out


def gdn_cpr_wait_status(shape: LayerShape, num_seqs: int, total_tokens: int, workspace: torch.Tensor,
                        status: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """The wait status of the last prefill / continuation / fwd_bwd call on `workspace`
    (called with that call's sizes) as a one-element int32 device tensor (or into
    `status`): 0 if every bounded wait ended normally, 1 if one gave up."""
    lib = _lib.load()
    if status is None:
        status = torch.empty(1, dtype=torch.int32, device=workspace.device)
    _lib.check(lib.gdn_cpr_wait_status(ctypes.byref(shape.c()), num_seqs, total_tokens, _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), _ptr(status), _stream(stream)))
    return status


def gdn_cpr_workspace_size(shape: LayerShape, num_seqs: int, total_tokens: int, op: int) -> int:
    return int(_lib.load().gdn_cpr_workspace_size(ctypes.byref(shape.c()), num_seqs, total_tokens, op))


def alloc_workspace(shape: LayerShape, num_seqs: int, total_tokens: int, op: int,
                    device="cuda") -> torch.Tensor:
    n = gdn_cpr_workspace_size(shape, num_seqs, total_tokens, op)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def gdn_cpr_prefill(shape: LayerShape, q, k, v, g, beta, cu_seqlens, h0, cache: CprCache, o,
                    workspace: torch.Tensor, stream=None, hT=None) -> None:
    """hT (optional, [N, H, d_k, d_v] fp32) receives every sequence's final state."""
    lib = _lib.load()
    N = int(cu_seqlens.numel()) - 1
    T = int(q.shape[0])
    cc = cache.c()
    _lib.check(lib.gdn_cpr_prefill(ctypes.byref(shape.c()), N, T, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                   _ptr(beta), _ptr(cu_seqlens), _ptr(h0), _ptr(hT), ctypes.byref(cc),
                                   _ptr(o), _ptr(workspace), workspace.numel(), _stream(stream)))


def gdn_cpr_decode_step(shape: LayerShape, q, k, v, g, beta, cache: CprCache, o,
                        workspace: torch.Tensor, stream=None, hT=None) -> None:
    """hT (optional, [N, H, d_k, d_v] fp32) receives the state after the token."""
    lib = _lib.load()
    N = int(q.shape[0])
    cc = cache.c()
    _lib.check(lib.gdn_cpr_decode_step(ctypes.byref(shape.c()), N, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                       _ptr(beta), ctypes.byref(cc), _ptr(hT), _ptr(o), _ptr(workspace),
                                       workspace.numel(), _stream(stream)))


def gdn_cpr_decode_step_noalloc(shape: LayerShape, q, k, v, g, beta, cache: CprCache, o, stream=None,
                                hT=None) -> None:
    """gdn_cpr_decode_step with the library's fixed per-device scratch instead
    of a workspace (allocates nothing; calls that overlap on one device race)."""
    lib = _lib.load()
    N = int(q.shape[0])
    cc = cache.c()
    _lib.check(lib.gdn_cpr_decode_step_noalloc(ctypes.byref(shape.c()), N, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                               _ptr(beta), ctypes.byref(cc), _ptr(hT), _ptr(o), _stream(stream)))


def gdn_cpr_prefill_continue(shape: LayerShape, q, k, v, g, beta, cu_seqlens, cache: CprCache, o,
                             workspace: torch.Tensor, stream=None, hT=None) -> None:
    """hT (optional, [N, H, d_k, d_v] fp32) receives every sequence's final state."""
    lib = _lib.load()
    N = int(cu_seqlens.numel()) - 1
    T = int(q.shape[0])
    cc = cache.c()
    _lib.check(lib.gdn_cpr_prefill_continue(ctypes.byref(shape.c()), N, T, _ptr(q), _ptr(k), _ptr(v),
                                            _ptr(g), _ptr(beta), _ptr(cu_seqlens), ctypes.byref(cc),
                                            _ptr(hT), _ptr(o), _ptr(workspace), workspace.numel(),
                                            _stream(stream)))


def gdn_cpr_fwd_bwd(shape: LayerShape, q, k, v, g, beta, cu_seqlens, h0, d_o, d_hT, o, hT, dq, dk,
                    dv, dg, dbeta, dh0, workspace: torch.Tensor, stream=None) -> None:
    lib = _lib.load()
    N = int(cu_seqlens.numel()) - 1
    T = int(q.shape[0])
    _lib.check(lib.gdn_cpr_fwd_bwd(ctypes.byref(shape.c()), N, T, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                   _ptr(beta), _ptr(cu_seqlens), _ptr(h0), _ptr(d_o), _ptr(d_hT),
                                   _ptr(o), _ptr(hT), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg),
                                   _ptr(dbeta), _ptr(dh0), _ptr(workspace), workspace.numel(),
                                   _stream(stream)))


def gdn_cmp_workspace(shape: LayerShape, mode: int, num_seqs: int, total_tokens: int,
                      device="cuda") -> torch.Tensor:
    n = int(_lib.load().gdn_cmp_workspace_size(ctypes.byref(shape.c()), mode, num_seqs, total_tokens))
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def gdn_cmp_prefill(shape: LayerShape, mode: int, q, k, v, g, beta, cu_seqlens, h0, state_out, o,
                    workspace: torch.Tensor, stream=None) -> None:
    """Comparator prefill (GDN_CMP_RECURRENT or GDN_CMP_CHUNKWISE), not CPR."""
    lib = _lib.load()
    N = int(cu_seqlens.numel()) - 1
    T = int(q.shape[0])
    _lib.check(lib.gdn_cmp_prefill(ctypes.byref(shape.c()), mode, N, T, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                   _ptr(beta), _ptr(cu_seqlens), _ptr(h0), _ptr(state_out), _ptr(o),
                                   _ptr(workspace), workspace.numel(), _stream(stream)))


def gdn_cmp_decode_step(shape: LayerShape, q, k, v, g, beta, state, o, stream=None) -> None:
    """Comparator decode: the per-token step on `state`, no tail, no resynchronisation."""
    lib = _lib.load()
    N = int(q.shape[0])
    _lib.check(lib.gdn_cmp_decode_step(ctypes.byref(shape.c()), N, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                       _ptr(beta), _ptr(state), _ptr(o), _stream(stream)))


def gdn_cmp_chunk_decode_step(shape: LayerShape, q, k, v, g, beta, cache: CprCache, o,
                              workspace: torch.Tensor, stream=None) -> None:
    """Comparator decode, chunkwise everywhere: the token's output from the chunk
    form over its partial chunk (cache tail + the token) on cache.s_bnd."""
    lib = _lib.load()
    N = int(q.shape[0])
    cc = cache.c()
    _lib.check(lib.gdn_cmp_chunk_decode_step(ctypes.byref(shape.c()), N, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                             _ptr(beta), ctypes.byref(cc), _ptr(o), _ptr(workspace),
                                             workspace.numel(), _stream(stream)))


class StageEvents:
    """Per-stage HIP events recorded by the library's measurement hook
    (gdn_cpr_set_stage_events), as torch events on the call's stream."""

    def __init__(self, n: int):
        self.events = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in self.events:
            e.record()  # materialise the underlying hipEvent_t
        torch.cuda.synchronize()
        self._arr = (ctypes.c_void_p * n)(*(e.cuda_event for e in self.events))

    def __enter__(self):
        _lib.load().gdn_cpr_set_stage_events(self._arr, len(self.events))
        return self

    def __exit__(self, *exc):
        _lib.load().gdn_cpr_set_stage_events(None, 0)
        return False

    def stage_ms(self, i: int) -> float:
        """Milliseconds between event i-1 and event i (after synchronisation)."""
        return self.events[i - 1].elapsed_time(self.events[i])


def gdn_cpr_last_error() -> str:
    return _lib.load().gdn_cpr_last_error().decode()


def gdn_cpr_numerics_id() -> str:
    return _lib.load().gdn_cpr_numerics_id().decode()
