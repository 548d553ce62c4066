"""Thin Python binding of libdflash.so (the C ABI in include/dflash.h).

Argument marshalling only: torch tensors are passed as device pointers with
the current HIP stream; every step of the drafter pass runs in the library's
kernels. The library must have been built (``python -m
block_diffusion_drafter_amd.build``); loading fails loudly otherwise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, List, Optional, Sequence

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdflash.so")
_lib = None

DFLASH_FP32, DFLASH_BF16 = 0, 1
DEV_CAPACITY, DEV_TOKEN, DEV_OFFSETS = 1, 2, 4
KERNEL_CLASSES = ["gemm_f32out", "gemm_resid", "gemm_swiglu", "lm_head", "attention",
                  "attention_combine", "norm_rope", "rmsnorm", "small", "sampling",
                  "attention_packed"]

LAYER_FIELDS = ["in_norm", "wq", "wk", "wv", "q_norm", "k_norm", "wo", "post_norm",
                "w_gate", "w_up", "w_down"]


class Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("hidden", "n_heads", "n_kv_heads", "head_dim", "n_layers", "intermediate",
                 "n_target_feats", "target_hidden", "vocab", "block_size", "mask_token_id",
                 "dtype")] + [("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
                              ("sliding_window", ctypes.c_int32),
                              ("sliding_layer_mask", ctypes.c_uint32)]


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in LAYER_FIELDS]


class WeightsStruct(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("lm_head", ctypes.c_void_p),
                ("fc", ctypes.c_void_p), ("fc_norm", ctypes.c_void_p),
                ("final_norm", ctypes.c_void_p), ("layers", ctypes.POINTER(LayerWeights)),
                ("packed", ctypes.c_void_p), ("packed_bytes", ctypes.c_int64)]


class KVCacheStruct(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("ctx_len", ctypes.c_void_p),
                ("batch", ctypes.c_int32), ("capacity", ctypes.c_int32)]


class RoundIOStruct(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("feats", ctypes.POINTER(ctypes.c_void_p)),
                ("feat_row_stride", ctypes.c_int64), ("target_tokens", ctypes.c_void_p),
                ("draft_tokens", ctypes.c_void_p), ("accept_len", ctypes.c_void_p),
                ("anchor", ctypes.c_void_p), ("ctx", ctypes.c_void_p), ("logits", ctypes.c_void_p),
                ("dev_status", ctypes.c_void_p), ("ws", ctypes.c_void_p),
                ("ws_bytes", ctypes.c_int64)]


class DFlashError(RuntimeError):
    pass


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise DFlashError(f"{_LIB_PATH} is missing: build it with "
                              "`python -m block_diffusion_drafter_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        L.dflash_status_string.restype = ctypes.c_char_p
        L.dflash_status_string.argtypes = [i32]
        L.dflash_create.restype = i32
        L.dflash_create.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(WeightsStruct),
                                    ctypes.POINTER(vp)]
        L.dflash_packed_weight_bytes.restype = i64
        L.dflash_packed_weight_bytes.argtypes = [ctypes.POINTER(Config)]
        L.dflash_pack_weights.restype = i32
        L.dflash_pack_weights.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(WeightsStruct),
                                          vp, i64, vp]
        L.dflash_destroy.restype = None
        L.dflash_destroy.argtypes = [vp]
        L.dflash_workspace_bytes.restype = i64
        L.dflash_workspace_bytes.argtypes = [vp, i32, i32, i32]
        L.dflash_ctx_project.restype = i32
        L.dflash_ctx_project.argtypes = [vp, ctypes.POINTER(vp), i64, i32, vp, vp, i64, vp]
        L.dflash_ctx_kv_append.restype = i32
        L.dflash_ctx_kv_append.argtypes = [vp, ctypes.POINTER(KVCacheStruct), vp, vp, i32, vp,
                                           vp, i64, vp]
        L.dflash_ctx_kv_append_accepted.restype = i32
        L.dflash_ctx_kv_append_accepted.argtypes = [vp, ctypes.POINTER(KVCacheStruct), vp, vp, vp,
                                                    vp, i64, vp]
        L.dflash_round_graph_create.restype = i32
        L.dflash_round_graph_create.argtypes = [vp, ctypes.POINTER(KVCacheStruct),
                                                ctypes.POINTER(RoundIOStruct), vp,
                                                ctypes.POINTER(vp)]
        L.dflash_round_graph_launch.restype = i32
        L.dflash_round_graph_launch.argtypes = [vp, vp]
        L.dflash_round_graph_destroy.restype = None
        L.dflash_round_graph_destroy.argtypes = [vp]
        L.dflash_draft_forward.restype = i32
        L.dflash_draft_forward.argtypes = [vp, ctypes.POINTER(KVCacheStruct), vp, i32, vp, vp,
                                           vp, vp, vp, vp, vp, vp, i64, vp]
        L.dflash_accept.restype = i32
        L.dflash_accept.argtypes = [vp, vp, i32, i32, vp, vp, vp, vp]
        L.dflash_packed_block_attention.restype = i32
        L.dflash_packed_block_attention.argtypes = [vp, ctypes.POINTER(KVCacheStruct), i32, i32,
                                                    i32, vp, vp, vp, vp, vp, vp, vp]
        L.dflash_sampling_workspace_bytes.restype = i64
        L.dflash_sampling_workspace_bytes.argtypes = [i32, i32, i32]
        L.dflash_sample_drafts.restype = i32
        L.dflash_sample_drafts.argtypes = [vp, i64, i32, i32, ctypes.c_float, ctypes.c_uint64, i32,
                                           vp, vp, vp, i64, vp]
        L.dflash_sample_drafts_static.restype = i32
        L.dflash_sample_drafts_static.argtypes = [vp, i64, i32, i32, ctypes.c_float,
                                                  ctypes.c_uint64, i32, vp, vp, vp]
        L.dflash_verify_sampled.restype = i32
        L.dflash_verify_sampled.argtypes = [vp, vp, vp, vp, i32, i32, i32, ctypes.c_float,
                                            ctypes.c_uint64, i32, vp, vp, vp, vp, i64, vp]
        L.dflash_profiler_start.restype = i32
        L.dflash_profiler_start.argtypes = [i32, ctypes.c_uint32]
        L.dflash_profiler_stop.restype = i32
        L.dflash_profiler_read.restype = i32
        L.dflash_profiler_read.argtypes = [i32, ctypes.POINTER(i64),
                                           ctypes.POINTER(ctypes.c_double),
                                           ctypes.POINTER(ctypes.c_double),
                                           ctypes.POINTER(ctypes.c_double)]
        L.dflash_profiler_reset.restype = i32
        L.dflash_probe_mfma_bf16.restype = i32
        L.dflash_probe_mfma_bf16.argtypes = [i32, i32, vp, ctypes.POINTER(ctypes.c_double), vp]
        _lib = L
    return _lib


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise DFlashError(f"{what}: {lib().dflash_status_string(rc).decode()} ({rc})")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise DFlashError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise DFlashError("tensor must be contiguous")
    return t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def torch_dtype(dtype: int) -> torch.dtype:
    return torch.bfloat16 if dtype == DFLASH_BF16 else torch.float32


def make_config(cfg) -> Config:
    """Config struct from a shape description with the usual field names."""
    return Config(hidden=cfg.hidden, n_heads=cfg.n_heads, n_kv_heads=cfg.n_kv_heads,
                  head_dim=cfg.head_dim, n_layers=cfg.n_layers, intermediate=cfg.intermediate,
                  n_target_feats=cfg.n_target_feats, target_hidden=cfg.target_hidden,
                  vocab=cfg.vocab, block_size=cfg.block_size, mask_token_id=cfg.mask_token_id,
                  dtype=DFLASH_BF16 if cfg.dtype == "bf16" else DFLASH_FP32,
                  rms_eps=cfg.rms_eps,
                  rope_theta=float(cfg.rope_theta) if cfg.rope_theta is not None else 0.0,
                  sliding_window=int(getattr(cfg, "sliding_window", 0) or 0),
                  sliding_layer_mask=sum(1 << int(l) for l in getattr(cfg, "sliding_layers", ())))


class KVCache:
    """Caller-owned per-layer context K/V cache (see dflash_kv_cache)."""

    BLOCK = 32

    def __init__(self, n_layers: int, batch: int, n_kv_heads: int, capacity: int, head_dim: int,
                 dtype: torch.dtype, device="cuda"):
        if capacity % self.BLOCK:
            raise DFlashError("capacity must be a multiple of 32")
        self.n_layers, self.batch, self.n_kv_heads = n_layers, batch, n_kv_heads
        self.capacity, self.head_dim, self.dtype = capacity, head_dim, dtype
        self.k = torch.zeros((n_layers, batch, n_kv_heads, capacity, head_dim), dtype=dtype,
                             device=device)
        self.v = torch.zeros((n_layers, batch, n_kv_heads, capacity // self.BLOCK, head_dim,
                              self.BLOCK), dtype=dtype, device=device)
        self.ctx_len = torch.zeros(batch, dtype=torch.int32, device=device)

    def struct(self) -> KVCacheStruct:
        return KVCacheStruct(self.k.data_ptr(), self.v.data_ptr(), self.ctx_len.data_ptr(),
                             self.batch, self.capacity)

    # Layout marshalling for setting up and inspecting cache contents.
    def write_positions(self, layer: int, seq: int, start: int, k: torch.Tensor,
                        v: torch.Tensor) -> None:
        """Store k, v [n_kv_heads, n, head_dim] at positions start..start+n-1."""
        n = k.shape[1]
        self.k[layer, seq, :, start:start + n] = k.to(self.dtype)
        pos = torch.arange(start, start + n, device=self.k.device)
        vv = self.v[layer, seq]                       # [H, nb, hd, 32]
        vv[:, pos // self.BLOCK, :, pos % self.BLOCK] = v.to(self.dtype).permute(1, 0, 2)

    def read_positions(self, layer: int, seq: int, start: int, n: int):
        """(k, v) [n_kv_heads, n, head_dim] at positions start..start+n-1."""
        k = self.k[layer, seq, :, start:start + n]
        pos = torch.arange(start, start + n, device=self.k.device)
        v = self.v[layer, seq][:, pos // self.BLOCK, :, pos % self.BLOCK].permute(1, 0, 2)
        return k, v


class DraftModel:
    """A dflash_handle over caller-provided device weights.

    weights: name -> device tensor in the model dtype, with the names
    embed, lm_head, fc, fc_norm, final_norm and layers.{l}.{field}.
    The projections are copied once into the library's tiled layout (a device
    buffer this object owns, written by dflash_pack_weights on the current
    stream); the row-major tensors stay referenced for the embedding and gains.
    """

    def __init__(self, cfg, weights: Dict[str, torch.Tensor]):
        self.cfg = cfg
        self.c = make_config(cfg)
        self.weights = weights  # keep the buffers alive for the handle's lifetime
        n = cfg.n_layers
        self._layers = (LayerWeights * n)()
        for l in range(n):
            for f in LAYER_FIELDS:
                setattr(self._layers[l], f, _ptr(weights[f"layers.{l}.{f}"]))
        lm = weights.get("lm_head", weights["embed"])
        n_packed = lib().dflash_packed_weight_bytes(ctypes.byref(self.c))
        if n_packed < 0:
            _check(int(n_packed), "dflash_packed_weight_bytes")
        self.packed = torch.empty(int(n_packed), dtype=torch.uint8, device="cuda")
        self._w = WeightsStruct(_ptr(weights["embed"]), _ptr(lm), _ptr(weights["fc"]),
                                _ptr(weights["fc_norm"]), _ptr(weights["final_norm"]),
                                ctypes.cast(self._layers, ctypes.POINTER(LayerWeights)),
                                _ptr(self.packed), int(n_packed))
        _check(lib().dflash_pack_weights(ctypes.byref(self.c), ctypes.byref(self._w),
                                         _ptr(self.packed), int(n_packed), _stream()),
               "dflash_pack_weights")
        h = ctypes.c_void_p()
        _check(lib().dflash_create(ctypes.byref(self.c), ctypes.byref(self._w), ctypes.byref(h)),
               "dflash_create")
        self.handle = h

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and _lib is not None:
            _lib.dflash_destroy(h)
            self.handle = None

    @property
    def dtype(self) -> torch.dtype:
        return torch_dtype(self.c.dtype)

    def workspace_bytes(self, max_batch: int, capacity: int, max_tokens: int) -> int:
        n = lib().dflash_workspace_bytes(self.handle, max_batch, capacity, max_tokens)
        if n < 0:
            _check(int(n), "dflash_workspace_bytes")
        return int(n)

    def new_workspace(self, max_batch: int, capacity: int, max_tokens: int) -> torch.Tensor:
        return torch.empty(self.workspace_bytes(max_batch, capacity, max_tokens),
                           dtype=torch.uint8, device="cuda")

    def new_cache(self, batch: int, capacity: int) -> KVCache:
        c = self.cfg
        return KVCache(c.n_layers, batch, c.n_kv_heads, capacity, c.head_dim, self.dtype)

    def ctx_project(self, feats: Sequence[torch.Tensor], out: torch.Tensor,
                    ws: torch.Tensor) -> torch.Tensor:
        n_tok = feats[0].shape[0]
        stride = feats[0].stride(0)
        arr = (ctypes.c_void_p * len(feats))(*[f.data_ptr() for f in feats])
        for f in feats:
            if f.stride(0) != stride or f.stride(1) != 1 or not f.is_cuda:
                raise DFlashError("features must be row-major device tensors with one row stride")
        _check(lib().dflash_ctx_project(self.handle, arr, stride, n_tok, _ptr(out), _ptr(ws),
                                        ws.numel(), _stream()), "dflash_ctx_project")
        return out

    def ctx_kv_append(self, cache: KVCache, ctx: torch.Tensor, cu_new: torch.Tensor,
                      ws: torch.Tensor, dev_status: Optional[torch.Tensor] = None) -> None:
        st = cache.struct()
        _check(lib().dflash_ctx_kv_append(self.handle, ctypes.byref(st), _ptr(ctx), _ptr(cu_new),
                                          ctx.shape[0], _ptr(dev_status), _ptr(ws), ws.numel(),
                                          _stream()), "dflash_ctx_kv_append")

    def ctx_kv_append_accepted(self, cache: KVCache, ctx: torch.Tensor, accept_len: torch.Tensor,
                               ws: torch.Tensor, dev_status: Optional[torch.Tensor] = None) -> None:
        """ctx: the block positions of every sequence [batch * B, hidden];
        rows 0..accept_len[s] of sequence s join its context."""
        if ctx.shape[0] != cache.batch * self.cfg.block_size:
            raise DFlashError("ctx must hold batch * block_size rows")
        st = cache.struct()
        _check(lib().dflash_ctx_kv_append_accepted(self.handle, ctypes.byref(st), _ptr(ctx),
                                                   _ptr(accept_len), _ptr(dev_status), _ptr(ws),
                                                   ws.numel(), _stream()),
               "dflash_ctx_kv_append_accepted")

    def draft_forward(self, cache: KVCache, anchor: torch.Tensor, draft_tokens: torch.Tensor,
                      ws: torch.Tensor, logits: Optional[torch.Tensor] = None,
                      hidden_out: Optional[torch.Tensor] = None,
                      target_tokens: Optional[torch.Tensor] = None,
                      accept_len: Optional[torch.Tensor] = None,
                      bonus: Optional[torch.Tensor] = None,
                      dev_status: Optional[torch.Tensor] = None) -> None:
        st = cache.struct()
        _check(lib().dflash_draft_forward(
            self.handle, ctypes.byref(st), _ptr(anchor), anchor.shape[0], _ptr(draft_tokens),
            _ptr(logits), _ptr(hidden_out), _ptr(target_tokens), _ptr(accept_len), _ptr(bonus),
            _ptr(dev_status), _ptr(ws), ws.numel(), _stream()), "dflash_draft_forward")


    def packed_block_attention(self, cache: KVCache, layer: int, anchors: torch.Tensor,
                               q: torch.Tensor, k_blk: torch.Tensor, v_blk: torch.Tensor,
                               out: torch.Tensor,
                               dev_status: Optional[torch.Tensor] = None) -> None:
        """Training-pattern attention of packed blocks (one layer): anchors
        [n_seq, nb] int32; q, out [n_seq, nb, B, Hq, hd]; k_blk, v_blk
        [n_seq, nb, B, Hkv, hd]; the context K/V come from `cache`."""
        st = cache.struct()
        n_seq, nb = anchors.shape
        _check(lib().dflash_packed_block_attention(
            self.handle, ctypes.byref(st), layer, n_seq, nb, _ptr(anchors), _ptr(q), _ptr(k_blk),
            _ptr(v_blk), _ptr(out), _ptr(dev_status), _stream()), "dflash_packed_block_attention")


class RoundGraph:
    """A decoding round captured once by dflash_round_graph_create and replayed
    with dflash_round_graph_launch: accept the verified block, fuse its
    features, inject the accepted rows, draft the next block. The tensors are
    the graph's fixed buffers: refill feats and target_tokens between replays.
    Capture runs on a side stream (the default stream cannot be captured)."""

    def __init__(self, model: DraftModel, cache: KVCache, feats: Sequence[torch.Tensor],
                 target_tokens: torch.Tensor, draft_tokens: torch.Tensor,
                 accept_len: torch.Tensor, anchor: torch.Tensor, ctx: torch.Tensor,
                 ws: torch.Tensor, logits: Optional[torch.Tensor] = None,
                 dev_status: Optional[torch.Tensor] = None):
        stride = feats[0].stride(0)
        for f in feats:
            if f.stride(0) != stride or f.stride(1) != 1 or not f.is_cuda:
                raise DFlashError("features must be row-major device tensors with one row stride")
        # keep every buffer the graph points at alive as long as the graph
        self._keep = (model, cache, list(feats), target_tokens, draft_tokens, accept_len, anchor,
                      ctx, ws, logits, dev_status)
        self._cache = cache.struct()
        self._feat_ptrs = (ctypes.c_void_p * len(feats))(*[f.data_ptr() for f in feats])
        self._io = RoundIOStruct(cache.batch, ctypes.cast(self._feat_ptrs,
                                                          ctypes.POINTER(ctypes.c_void_p)),
                                 stride, _ptr(target_tokens), _ptr(draft_tokens), _ptr(accept_len),
                                 _ptr(anchor), _ptr(ctx), _ptr(logits), _ptr(dev_status), _ptr(ws),
                                 ws.numel())
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        g = ctypes.c_void_p()
        _check(lib().dflash_round_graph_create(model.handle, ctypes.byref(self._cache),
                                               ctypes.byref(self._io), side.cuda_stream,
                                               ctypes.byref(g)), "dflash_round_graph_create")
        self.graph = g

    def replay(self) -> None:
        _check(lib().dflash_round_graph_launch(self.graph, _stream()), "dflash_round_graph_launch")

    def close(self) -> None:
        if getattr(self, "graph", None) is not None and _lib is not None:
            _lib.dflash_round_graph_destroy(self.graph)
            self.graph = None

    def __del__(self):
        self.close()


def accept(draft_tokens: torch.Tensor, target_tokens: torch.Tensor, block_size: int,
           accept_len: torch.Tensor, bonus: torch.Tensor,
           anchor_out: Optional[torch.Tensor] = None) -> None:
    _check(lib().dflash_accept(_ptr(draft_tokens), _ptr(target_tokens), target_tokens.shape[0],
                               block_size, _ptr(accept_len), _ptr(bonus), _ptr(anchor_out),
                               _stream()), "dflash_accept")


def sampling_workspace(batch: int, block_size: int, vocab: int) -> torch.Tensor:
    n = lib().dflash_sampling_workspace_bytes(batch, block_size, vocab)
    if n < 0:
        _check(int(n), "dflash_sampling_workspace_bytes")
    return torch.empty(int(n), dtype=torch.uint8, device="cuda")


def sample_drafts(logits: torch.Tensor, temperature: float, seed: int, rnd: int,
                  tokens: torch.Tensor, ws: torch.Tensor,
                  logq: Optional[torch.Tensor] = None) -> None:
    """tokens[r] ~ softmax(logits[r] / T) (fp32 logits [rows, >= vocab])."""
    rows, vocab = logits.shape
    if logits.dtype != torch.float32 or logits.stride(1) != 1:
        raise DFlashError("logits must be fp32 with unit column stride")
    _check(lib().dflash_sample_drafts(logits.data_ptr(), logits.stride(0), rows, vocab,
                                      float(temperature), int(seed), int(rnd), _ptr(tokens),
                                      _ptr(logq), _ptr(ws), ws.numel(), _stream()),
           "dflash_sample_drafts")


def sample_drafts_static(logits: torch.Tensor, temperature: float, seed: int, rnd: int,
                         tokens: torch.Tensor, logq: Optional[torch.Tensor] = None) -> None:
    """sample_drafts without a workspace (the library's static scratch): for
    callers that cannot allocate; rows * ceil(vocab / 8192) <= 16384."""
    rows, vocab = logits.shape
    if logits.dtype != torch.float32 or logits.stride(1) != 1:
        raise DFlashError("logits must be fp32 with unit column stride")
    _check(lib().dflash_sample_drafts_static(logits.data_ptr(), logits.stride(0), rows, vocab,
                                             float(temperature), int(seed), int(rnd),
                                             _ptr(tokens), _ptr(logq), _stream()),
           "dflash_sample_drafts_static")


def verify_sampled(drafts: torch.Tensor, draft_logits: torch.Tensor,
                   target_logits: torch.Tensor, temperature: float, seed: int, rnd: int,
                   accept_len: torch.Tensor, out_token: torch.Tensor, ws: torch.Tensor,
                   anchor_out: Optional[torch.Tensor] = None,
                   draft_logq: Optional[torch.Tensor] = None) -> None:
    """drafts [b, B-1], draft logits [b, B-1, V], target logits [b, B, V];
    draft_logq [b, B-1] (optional): log q of the drawn candidates, as
    sample_drafts returned it at this temperature."""
    b, Bk, vocab = target_logits.shape
    _check(lib().dflash_verify_sampled(_ptr(drafts), _ptr(draft_logits), _ptr(draft_logq),
                                       _ptr(target_logits), b,
                                       Bk, vocab, float(temperature), int(seed), int(rnd),
                                       _ptr(accept_len), _ptr(out_token), _ptr(anchor_out),
                                       _ptr(ws), ws.numel(), _stream()), "dflash_verify_sampled")


def profiler_start(max_launches: int = 100000, classes: Optional[List[str]] = None) -> None:
    """Bracket library launches with HIP events; ``classes`` limits it to some
    kernel classes (names from KERNEL_CLASSES), None means all."""
    mask = 0
    for c in (classes or []):
        mask |= 1 << KERNEL_CLASSES.index(c)
    _check(lib().dflash_profiler_start(max_launches, mask), "dflash_profiler_start")


def profiler_stop() -> None:
    _check(lib().dflash_profiler_stop(), "dflash_profiler_stop")


def profiler_read() -> Dict[str, dict]:
    out = {}
    for i, name in enumerate(KERNEL_CLASSES):
        n = ctypes.c_int64()
        ms, by, fl = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
        _check(lib().dflash_profiler_read(i, ctypes.byref(n), ctypes.byref(ms), ctypes.byref(by),
                                          ctypes.byref(fl)), "dflash_profiler_read")
        out[name] = dict(launches=n.value, ms=ms.value, bytes=by.value, flops=fl.value)
    return out


def profiler_reset() -> None:
    _check(lib().dflash_profiler_reset(), "dflash_profiler_reset")


def probe_mfma_bf16(n_workgroups: int, iters: int, sink: torch.Tensor) -> float:
    """Enqueue the MFMA calibration loop on the current stream; returns its flops.
    sink: device fp32 tensor of at least n_workgroups * 8 entries."""
    if sink.numel() < n_workgroups * 8 or sink.dtype != torch.float32 or not sink.is_cuda:
        raise DFlashError("sink must be a device fp32 tensor of n_workgroups * 8 entries")
    fl = ctypes.c_double()
    _check(lib().dflash_probe_mfma_bf16(n_workgroups, iters, _ptr(sink), ctypes.byref(fl),
                                        _stream()), "dflash_probe_mfma_bf16")
    return fl.value
