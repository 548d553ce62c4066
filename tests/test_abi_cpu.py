"""The C-ABI library without a GPU: it loads, exports every function that
include/dflash.h declares, and rejects bad arguments on the host before it
enqueues anything (no call here reaches a HIP launch)."""
import ctypes
import os
import re

import pytest

from block_diffusion_drafter_amd import binding as B
from synth import TINY_FP32, QWEN3_8B_SHAPED

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "dflash.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dflash_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_function():
    names = header_functions()
    assert len(names) >= 12, names
    lib = B.lib()
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def test_status_strings():
    lib = B.lib()
    for code in range(0, -10, -1):
        s = lib.dflash_status_string(code).decode()
        assert s and s != "unknown status", code
    assert lib.dflash_status_string(-99).decode() == "unknown status"


FAKE = 1 << 20  # a 16-byte-aligned non-null address; never dereferenced here


def fake_weights(n_layers):
    layers = (B.LayerWeights * n_layers)()
    for l in range(n_layers):
        for f in B.LAYER_FIELDS:
            setattr(layers[l], f, FAKE)
    w = B.WeightsStruct(FAKE, FAKE, FAKE, FAKE, FAKE,
                        ctypes.cast(layers, ctypes.POINTER(B.LayerWeights)), FAKE, 1 << 40)
    return w, layers


def create(cfg_struct, n_layers=None):
    w, layers = fake_weights(n_layers if n_layers is not None else max(1, cfg_struct.n_layers))
    h = ctypes.c_void_p()
    rc = B.lib().dflash_create(ctypes.byref(cfg_struct), ctypes.byref(w), ctypes.byref(h))
    return rc, h


@pytest.mark.parametrize("cfg", [TINY_FP32, QWEN3_8B_SHAPED], ids=lambda c: c.name)
def test_create_and_workspace(cfg):
    rc, h = create(B.make_config(cfg))
    assert rc == 0 and h.value
    lib = B.lib()
    n1 = lib.dflash_workspace_bytes(h, 1, 2080, 16)
    n32 = lib.dflash_workspace_bytes(h, 32, 8224, 512)
    assert 0 < n1 < n32
    assert lib.dflash_workspace_bytes(h, 0, 64, 0) == -2
    assert lib.dflash_workspace_bytes(None, 1, 64, 0) == -1
    lib.dflash_destroy(h)


@pytest.mark.parametrize("field,value,code", [
    ("dtype", 7, -3), ("head_dim", 96, -6), ("block_size", 17, -6), ("block_size", 0, -6),
    ("n_kv_heads", 3, -2), ("hidden", 250, -2), ("mask_token_id", 1000, -2),
    ("n_layers", 17, -6), ("vocab", 1, -2)])
def test_create_rejects_bad_config(field, value, code):
    c = B.make_config(TINY_FP32)
    setattr(c, field, value)
    rc, h = create(c, n_layers=1)
    assert rc == code and not h.value


def test_create_rejects_null_and_misaligned_weights():
    c = B.make_config(TINY_FP32)
    w, layers = fake_weights(1)
    h = ctypes.c_void_p()
    create_ = lambda: B.lib().dflash_create(ctypes.byref(c), ctypes.byref(w), ctypes.byref(h))
    layers[0].q_norm = None
    assert create_() == -1
    layers[0].q_norm = FAKE + 4
    assert create_() == -4
    layers[0].q_norm = FAKE
    # the row-major projections are only read by dflash_pack_weights
    layers[0].wq = None
    w.lm_head = None
    assert create_() == 0 and h.value
    B.lib().dflash_destroy(h)
    w.packed = None
    assert create_() == -1
    w.packed = FAKE + 8
    assert create_() == -4
    w.packed = FAKE
    w.packed_bytes = B.lib().dflash_packed_weight_bytes(ctypes.byref(c)) - 1
    assert create_() == -5
    assert B.lib().dflash_create(ctypes.byref(c), ctypes.byref(w), None) == -1


def tiled_bytes(rows, k, es):
    kc = 256 // es
    return -(-rows // 16) * 16 * (-(-k // kc) * kc) * es


def expected_packed_bytes(cfg):
    """Sizes of the tiled copies, each on a 256-byte boundary, in the order the
    header lists them."""
    es = 2 if cfg.dtype == "bf16" else 4
    d, q, kv, i = cfg.hidden, cfg.n_heads * cfg.head_dim, cfg.n_kv_heads * cfg.head_dim, cfg.intermediate
    parts = []
    for _ in range(cfg.n_layers):
        parts += [tiled_bytes(q + 2 * kv, d, es), tiled_bytes(d, q, es), tiled_bytes(i, d, es),
                  tiled_bytes(i, d, es), tiled_bytes(d, i, es)]
    parts += [tiled_bytes(d, cfg.n_target_feats * cfg.target_hidden, es),
              tiled_bytes(cfg.n_layers * 2 * kv, d, es), tiled_bytes(cfg.vocab, d, es)]
    return sum(-(-p // 256) * 256 for p in parts)


@pytest.mark.parametrize("cfg", [TINY_FP32, QWEN3_8B_SHAPED], ids=lambda c: c.name)
def test_packed_weight_bytes(cfg):
    lib = B.lib()
    c = B.make_config(cfg)
    n = lib.dflash_packed_weight_bytes(ctypes.byref(c))
    assert n == expected_packed_bytes(cfg)
    assert lib.dflash_packed_weight_bytes(None) == -1
    c.head_dim = 96
    assert lib.dflash_packed_weight_bytes(ctypes.byref(c)) == -6


def test_pack_weights_rejects_bad_arguments_before_launching():
    lib = B.lib()
    c = B.make_config(TINY_FP32)
    w, layers = fake_weights(1)
    n = lib.dflash_packed_weight_bytes(ctypes.byref(c))
    pack = lambda dst=FAKE, nb=n: lib.dflash_pack_weights(ctypes.byref(c), ctypes.byref(w), dst,
                                                          nb, None)
    assert pack(dst=None) == -1
    assert pack(dst=FAKE + 4) == -4
    assert pack(nb=n - 1) == -5
    layers[0].w_down = None
    assert pack() == -1
    layers[0].w_down = FAKE + 2
    assert pack() == -4
    layers[0].w_down = FAKE
    w.fc = None
    assert pack() == -1
    assert lib.dflash_pack_weights(None, ctypes.byref(w), FAKE, n, None) == -1


def test_calls_reject_bad_arguments_before_launching():
    lib = B.lib()
    rc, h = create(B.make_config(TINY_FP32))
    assert rc == 0
    cache = B.KVCacheStruct(FAKE, FAKE, FAKE, 2, 64)
    bad_cap = B.KVCacheStruct(FAKE, FAKE, FAKE, 2, 48)
    no_k = B.KVCacheStruct(None, FAKE, FAKE, 2, 64)
    ws_need = lib.dflash_workspace_bytes(h, 1, 64, 0)
    fwd = lambda c, batch=1, ws=FAKE, wsb=ws_need, drafts=FAKE: lib.dflash_draft_forward(
        h, ctypes.byref(c), FAKE, batch, drafts, None, None, None, None, None, None, ws, wsb, None)
    assert fwd(bad_cap) == -2
    assert fwd(no_k) == -1
    assert fwd(cache, batch=3) == -2
    assert fwd(cache, batch=0) == -2
    assert fwd(cache, wsb=ws_need - 1) == -5
    assert fwd(cache, ws=FAKE + 8) == -4
    assert fwd(cache, drafts=None) == -1
    # fused accept needs both outputs
    assert lib.dflash_draft_forward(h, ctypes.byref(cache), FAKE, 1, FAKE, None, None, FAKE,
                                    None, FAKE, None, FAKE, ws_need, None) == -1
    # append: misaligned ctx, too-small workspace, negative rows
    assert lib.dflash_ctx_kv_append(h, ctypes.byref(cache), FAKE + 2, FAKE, 4, None, FAKE,
                                    1 << 30, None) == -4
    assert lib.dflash_ctx_kv_append(h, ctypes.byref(cache), FAKE, FAKE, 4, None, FAKE, 16,
                                    None) == -5
    assert lib.dflash_ctx_kv_append(h, ctypes.byref(cache), FAKE, FAKE, -1, None, FAKE, 16,
                                    None) == -2
    # project: bad stride, null feature pointer
    feats = (ctypes.c_void_p * 3)(FAKE, FAKE, None)
    assert lib.dflash_ctx_project(h, feats, 256, 4, FAKE, FAKE, 1 << 30, None) == -1
    feats = (ctypes.c_void_p * 3)(FAKE, FAKE, FAKE)
    assert lib.dflash_ctx_project(h, feats, 100, 4, FAKE, FAKE, 1 << 30, None) == -2
    assert lib.dflash_ctx_project(h, feats, 256, 0, None, None, 0, None) == 0  # no-op
    # accept
    assert lib.dflash_accept(FAKE, None, 2, 4, FAKE, FAKE, None, None) == -1
    assert lib.dflash_accept(FAKE, FAKE, -1, 4, FAKE, FAKE, None, None) == -2
    assert lib.dflash_accept(None, None, 0, 4, None, None, None, None) == 0
    lib.dflash_destroy(h)


def test_profiler_state_machine():
    lib = B.lib()
    assert lib.dflash_profiler_read(99, None, None, None, None) == -2
    n = ctypes.c_int64()
    d = ctypes.c_double()
    assert lib.dflash_profiler_read(0, ctypes.byref(n), ctypes.byref(d), ctypes.byref(d),
                                    ctypes.byref(d)) == 0
    assert n.value == 0


def test_sampling_calls_reject_bad_arguments_before_launching():
    lib = B.lib()
    assert lib.dflash_sampling_workspace_bytes(4, 16, 1000) > 0
    assert lib.dflash_sampling_workspace_bytes(4, 1, 1000) == -2
    assert lib.dflash_sampling_workspace_bytes(4, 16, 1) == -2
    need = lib.dflash_sampling_workspace_bytes(2, 16, 1000)
    samp = lambda logits=FAKE, stride=1000, rows=30, T=0.8, tokens=FAKE, ws=FAKE, wsb=need: \
        lib.dflash_sample_drafts(logits, stride, rows, 1000, T, 7, 0, tokens, None, ws, wsb, None)
    assert samp(T=0.0) == -2
    assert samp(T=float("nan")) == -2
    assert samp(T=float("inf")) == -2
    assert samp(stride=999) == -2
    assert samp(rows=-1) == -2
    assert samp(rows=0, logits=None) == 0  # no-op
    assert samp(logits=None) == -1
    assert samp(tokens=FAKE + 4) == -4
    assert samp(wsb=16) == -5
    ver = lambda block=16, T=1.0, drafts=FAKE, ws=FAKE, wsb=need, batch=2, logq=None: \
        lib.dflash_verify_sampled(drafts, FAKE, logq, FAKE, batch, block, 1000, T, 1, 0, FAKE,
                                  FAKE, None, ws, wsb, None)
    assert ver(block=1) == -2
    assert ver(block=18) == -2
    assert ver(T=-1.0) == -2
    assert ver(batch=0, drafts=None) == 0
    assert ver(drafts=None) == -1
    assert ver(ws=FAKE + 8) == -4
    assert ver(logq=FAKE + 4) == -4
    assert ver(wsb=need // 4) == -5


def test_block_append_and_round_graph_reject_bad_arguments_before_launching():
    lib = B.lib()
    rc, h = create(B.make_config(TINY_FP32))
    assert rc == 0
    cache = B.KVCacheStruct(FAKE, FAKE, FAKE, 2, 64)
    need = lib.dflash_workspace_bytes(h, 2, 64, 2 * TINY_FP32.block_size)
    app = lambda ctx=FAKE, acc=FAKE, ws=FAKE, wsb=need, c=cache: \
        lib.dflash_ctx_kv_append_accepted(h, ctypes.byref(c), ctx, acc, None, ws, wsb, None)
    assert app(acc=None) == -1
    assert app(acc=FAKE + 4) == -4
    assert app(ctx=None) == -1
    assert app(ctx=FAKE + 2) == -4
    assert app(wsb=16) == -5
    assert app(c=B.KVCacheStruct(FAKE, FAKE, FAKE, 2, 48)) == -2
    assert lib.dflash_ctx_kv_append_accepted(None, ctypes.byref(cache), FAKE, FAKE, None, FAKE,
                                             need, None) == -1

    feats = (ctypes.c_void_p * 3)(FAKE, FAKE, FAKE)
    io = B.RoundIOStruct(2, ctypes.cast(feats, ctypes.POINTER(ctypes.c_void_p)), 256, FAKE, FAKE,
                         FAKE, FAKE, FAKE, None, None, FAKE, need)
    g = ctypes.c_void_p(FAKE)
    create_g = lambda stream=FAKE, io_=io: lib.dflash_round_graph_create(
        h, ctypes.byref(cache), ctypes.byref(io_), stream, ctypes.byref(g))
    # the NULL stream cannot be captured: refused before any HIP call
    assert create_g(stream=None) == -1
    assert g.value is None  # *out cleared on failure
    io.batch = 3  # must match the cache's batch
    assert create_g() == -2
    io.batch = 2
    assert lib.dflash_round_graph_create(h, ctypes.byref(cache), None, FAKE, ctypes.byref(g)) == -1
    assert lib.dflash_round_graph_create(h, ctypes.byref(cache), ctypes.byref(io), FAKE,
                                         None) == -1
    assert lib.dflash_round_graph_launch(None, None) == -1
    lib.dflash_round_graph_destroy(None)  # no-op
    lib.dflash_destroy(h)


def test_sliding_window_config_is_validated():
    lib = B.lib()
    c = B.make_config(TINY_FP32.with_(n_layers=2, sliding_window=8, sliding_layers=(1,)))
    rc, h = create(c)
    assert rc == 0
    lib.dflash_destroy(h)
    c.sliding_window = 0          # a sliding layer needs a window >= 1
    assert create(c)[0] == -2
    c.sliding_window = 8
    c.sliding_layer_mask = 1 << 2  # no layer 2 in a 2-layer drafter
    assert create(c)[0] == -2
    c.sliding_layer_mask = 0       # no sliding layer: the window is ignored
    c.sliding_window = -5
    rc, h = create(c)
    assert rc == 0
    lib.dflash_destroy(h)


def test_packed_block_attention_rejects_bad_arguments_before_launching():
    lib = B.lib()
    rc, h = create(B.make_config(TINY_FP32))
    assert rc == 0
    cache = B.KVCacheStruct(FAKE, FAKE, FAKE, 2, 64)
    call = lib.dflash_packed_block_attention
    # no handle, no cache
    assert call(None, ctypes.byref(cache), 0, 1, 2, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == -1
    assert call(h, None, 0, 1, 2, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == -1
    # layer outside the drafter, negative counts, more sequences than the cache holds
    assert call(h, ctypes.byref(cache), 1, 1, 2, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == -2
    assert call(h, ctypes.byref(cache), 0, -1, 2, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == -2
    assert call(h, ctypes.byref(cache), 0, 3, 2, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == -2
    # missing or misaligned buffers
    assert call(h, ctypes.byref(cache), 0, 1, 2, None, FAKE, FAKE, FAKE, FAKE, None, None) == -1
    assert call(h, ctypes.byref(cache), 0, 1, 2, FAKE, FAKE + 8, FAKE, FAKE, FAKE, None,
                None) == -4
    # nothing to do: no launch, no pointer needed
    assert call(h, ctypes.byref(cache), 0, 1, 0, None, None, None, None, None, None, None) == 0
    lib.dflash_destroy(h)


def test_sample_drafts_static_checks_on_the_host():
    """The allocation-free drafting call refuses, before touching any device
    state, a request larger than its static scratch (16384 split entries of
    8192 logits), and bad shapes; an empty request is a no-op."""
    lib = B.lib()
    f = lib.dflash_sample_drafts_static
    assert f(FAKE, 16384, 8193, 16384, 1.0, 1, 0, FAKE, None, None) == -9      # 16386 entries
    assert f(FAKE, 8192 * 32, 513, 8192 * 32, 1.0, 1, 0, FAKE, None, None) == -9
    assert f(FAKE, 1000, 4, 1000, 0.0, 1, 0, FAKE, None, None) == -2           # T <= 0
    assert f(FAKE, 999, 4, 1000, 1.0, 1, 0, FAKE, None, None) == -2            # stride < vocab
    assert f(None, 1000, 4, 1000, 1.0, 1, 0, FAKE, None, None) == -1
    assert f(FAKE + 4, 1000, 4, 1000, 1.0, 1, 0, FAKE, None, None) == -4
    assert f(FAKE, 1000, 0, 1000, 1.0, 1, 0, None, None, None) == 0            # nothing to do
