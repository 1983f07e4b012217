"""CPU fp64 oracle for the chunkwise-parallel recurrent (CPR) Gated DeltaNet layer.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The HIP library never calls it, and
it shares no code, constants or helpers with the HIP path.

What it computes (from the IsoExec pages, section "Chunkwise-Parallel
Recurrent (CPR) Gated DeltaNet", and the Chinese page's section on the
"third way" for Gated DeltaNet): the Gated DeltaNet recurrence itself.  CPR
evaluates that recurrence in a particular order so that training, prefill and
decode round identically; in exact arithmetic every evaluation order gives the
same numbers, so the oracle is the plain definition, run in float64 on the
inputs already rounded to the kernel's storage dtype.

Modules:
  recurrent  -- token-by-token recurrence (the definition), forward only
  chunkwise  -- the chunk (WY/UT) form, written separately, same results
  backward   -- analytic reverse-mode gradient of the recurrence
  fd         -- central finite differences of a scalar loss, for pinning
  heads      -- key/query heads shared by groups of value heads

Notation (one head): state M (d_v x d_k), key/query k, q (d_k), value v (d_v),
log-decay g <= 0 with alpha = exp(g), write strength beta in (0, 1).
  M_t = alpha_t M_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
  o_t = M_t q_t
States cross the oracle's interface in the storage layout S = M^T, i.e.
[..., d_k, d_v] (key dimension first).

Parity pins: see tests/test_oracle.py.  Every function here is pinned by at
least one check that does not re-run its own formula.
"""

from .recurrent import recurrent_forward, token_step
from .chunkwise import chunkwise_forward, chunk_products
from .backward import recurrent_backward
from .fd import fd_gradients, loss_value
from .heads import expand_key_heads, sum_key_heads

__all__ = [
    "recurrent_forward",
    "token_step",
    "chunkwise_forward",
    "chunk_products",
    "recurrent_backward",
    "fd_gradients",
    "loss_value",
    "expand_key_heads",
    "sum_key_heads",
]
