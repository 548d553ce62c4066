"""The allocation-free drafting call (dflash_sample_drafts_static) against the
workspace call it is a variant of (dflash_sample_drafts), through the C ABI:
same inputs, bit-identical tokens and log q, on two calls in a row, the second
with a smaller input (the static scratch keeps the first call's contents)."""
import numpy as np
import pytest
import torch

from block_diffusion_drafter_amd import binding as B
from gpu_harness import log
from synth import inputs as I

pytestmark = pytest.mark.gpu


def _run_both(rows, V, T, seed, rnd, tag):
    lg = torch.from_numpy(I.normal(41, tag, (rows, V), 2.0, False).reshape(rows, V)).cuda()
    tok_ws = torch.full((rows,), -1, dtype=torch.int32, device="cuda")
    lq_ws = torch.full((rows,), np.nan, dtype=torch.float32, device="cuda")
    ws = B.sampling_workspace(rows, 2, V)
    B.sample_drafts(lg, T, seed, rnd, tok_ws, ws, lq_ws)
    tok_st = torch.full((rows,), -1, dtype=torch.int32, device="cuda")
    lq_st = torch.full((rows,), np.nan, dtype=torch.float32, device="cuda")
    B.sample_drafts_static(lg, T, seed, rnd, tok_st, lq_st)
    torch.cuda.synchronize()
    return tok_ws.cpu(), lq_ws.cpu(), tok_st.cpu(), lq_st.cpu()


def test_gpu_sample_drafts_static_matches_workspace_call():
    # first call: 480 rows at vocab 151936 (the batch-32 drafting shape, 9120
    # of the scratch's 16384 split entries); second: fewer rows, another vocab
    for rows, V, T, tag in ((480, 151936, 1.0, "na1"), (45, 1000, 0.7, "na2")):
        log(f"case: sample_drafts_static rows {rows} vocab {V} T {T}")
        tw, lw, ts, ls = _run_both(rows, V, T, 99, 3, tag)
        assert ((ts >= 0) & (ts < V)).all()
        assert torch.equal(tw, ts), f"tokens differ at {torch.nonzero(tw != ts)[:5].tolist()}"
        assert torch.equal(lw, ls), "log q differs"
        log(f"  {rows} tokens and log q bit-identical to the workspace call")


def test_gpu_sample_drafts_static_rejects_oversized_request():
    # 16385 split entries needed: refused before anything is enqueued
    V = 8192 * 2
    rows = 8193
    lg = torch.zeros((rows, V), dtype=torch.float32, device="cuda")
    tok = torch.full((rows,), -7, dtype=torch.int32, device="cuda")
    with pytest.raises(B.DFlashError, match="-9"):
        B.sample_drafts_static(lg, 1.0, 1, 0, tok)
    torch.cuda.synchronize()
    assert bool((tok == -7).all())
