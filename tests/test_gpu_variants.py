"""Drafter variants against the oracle through the C ABI: block sizes other
than 16 (the LLaMA drafters' 10, and 8), depths 1, 3 and 8, and sliding-window
layers (window below and above the block size, W = 1, several sliding layers,
ragged contexts with and without history older than the window). Each case is
the same prefill + forward + fused accept flow as the main parity tests, every
stage compared element by element with the oracle."""
import pytest

from gpu_harness import log
from synth import SMALL_BF16, TINY_FP32
from test_gpu_parity import run_flow

pytestmark = pytest.mark.gpu


def test_gpu_block10_ragged():
    run_flow(SMALL_BF16.with_(block_size=10), [0, 45, 130, 290, 7], "small-b10")


def test_gpu_block10_fp32_three_layers():
    run_flow(TINY_FP32.with_(block_size=10, n_layers=3), [33, 64], "tiny-b10-d3")


@pytest.mark.parametrize("depth", [1, 3, 8])
def test_gpu_depth(depth):
    log(f"case: depth {depth}")
    run_flow(SMALL_BF16.with_(n_layers=depth), [61, 200], f"small-d{depth}")


def test_gpu_sliding_window_bf16():
    # layers 0 and 2 slide with a 40-key window, layer 1 attends to everything
    cfg = SMALL_BF16.with_(n_layers=3, sliding_window=40, sliding_layers=(0, 2))
    run_flow(cfg, [0, 37, 100, 301, 5, 64], "small-swa40")


def test_gpu_sliding_window_narrower_than_block_fp32():
    # window 3 < block 4: later queries lose the block's first keys too
    cfg = TINY_FP32.with_(n_layers=2, sliding_window=3, sliding_layers=(1,))
    run_flow(cfg, [40, 2, 0], "tiny-swa3")


def test_gpu_sliding_window_of_one():
    # W = 1: a query sees its own and later block positions only
    cfg = TINY_FP32.with_(n_layers=2, sliding_window=1, sliding_layers=(1,))
    run_flow(cfg, [17, 70, 40], "tiny-swa1b")


def test_gpu_sliding_window_of_one_every_layer():
    # every layer at W = 1: the mask slots see only mask slots, so their logits
    # are near ties (margins ~0.002); hidden states and logits are still
    # compared everywhere, drafts where the margin allows
    cfg = TINY_FP32.with_(n_layers=2, sliding_window=1, sliding_layers=(0, 1))
    run_flow(cfg, [17, 70], "tiny-swa1", degenerate=True)


def test_gpu_sliding_window_wide_long_context():
    # 1000-key window over contexts of up to 3000: most history outside it
    cfg = SMALL_BF16.with_(sliding_window=1000, sliding_layers=(1,))
    run_flow(cfg, [3000, 999, 1500], "small-swa1000")
