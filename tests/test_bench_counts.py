"""bench.py's flop counts for the backward's state and gradient stages against
the MFMA instruction counters of one fwd_bwd call (1 x 10,240 tokens, 16
heads, d = 128, C = 64: 2,560 chunk-heads), as recorded in
profiles/prefill_5x2048_decode_256x1_counters.md:
  - the algorithmic products over their nonzero 16 x 16 tiles, 19,365,888
    flops per chunk-head (what the stages executed when their products ran on
    fp32 MFMA, SQ_INSTS_VALU_MFMA_MOPS_F32 x 512 / 2,560);
  - the bf16 MFMA flops they execute with the fp32-operand products split
    into bf16 hi/lo parts, 44,072,960 per chunk-head
    (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 / 2,560: state 27,131,904,
    gradients 16,941,056)."""

import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_algorithmic_count_matches_counters():
    assert bench.bwd_state_grads_flop(64, 128, 128) == 19_365_888


def test_executed_bf16_count_matches_counters():
    assert bench.bwd_state_grads_bf16_exec_flop(64, 128, 128) == 44_072_960


def test_split_costs_between_two_and_three_products():
    # every fp32-operand product takes two or three bf16 products; Q K^T and
    # K K^T (one each) are a small share, so the ratio lies inside (2, 3)
    for d in (64, 128):
        a = bench.bwd_state_grads_flop(64, d, d)
        e = bench.bwd_state_grads_bf16_exec_flop(64, d, d)
        assert 2 * a < e < 3 * a
