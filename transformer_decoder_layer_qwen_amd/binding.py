"""Thin Python binding of the C ABI in ``include/qlayer.h`` (ctypes).

Argument marshalling only: every step of the layer runs in the HIP kernels of
``libqlayer.so``. PyTorch is used for device memory and streams. If the
library has not been built this module raises on first use; there is no
fallback path.

The module-level functions carry the C names (``qlayer_create``,
``qlayer_prefill``, ``qlayer_decode``, ``qlayer_moe_ffn``, ...) and take raw
pointers; ``QLayer`` wraps them for torch tensors.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqlayer.so")

QL_OK, QL_EINVAL, QL_EUNSUPPORTED, QL_ENOMEM, QL_EHIP, QL_ECACHE_FULL = 0, -1, -2, -3, -4, -5
QL_BF16, QL_F32 = 0, 1
STATUS_NAMES = {0: "QL_OK", -1: "QL_EINVAL", -2: "QL_EUNSUPPORTED", -3: "QL_ENOMEM",
                -4: "QL_EHIP", -5: "QL_ECACHE_FULL"}

# every function include/qlayer.h declares
EXPORTS = ("qlayer_create", "qlayer_destroy", "qlayer_workspace_bytes", "qlayer_prefill",
           "qlayer_prefill_varlen", "qlayer_decode", "qlayer_decode_stack", "qlayer_decode_noalloc", "qlayer_moe_ffn", "qlayer_set_taps",
           "qlayer_set_stage_events", "qlayer_last_error", "qlayer_abi_version")
NOALLOC_MAX_WORKSPACE = 64 << 20

# ql_stage
STAGES = {"rmsnorm1": 1, "qkv": 2, "qkv_post": 3, "attention": 4, "o_proj": 5, "rmsnorm2": 6,
          "gate_up": 7, "down": 8, "router": 9, "permute": 10, "expert_gate_up": 11,
          "expert_down": 12, "combine": 13, "shared_gate_up": 14, "shared_down": 15}


class QlConfig(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int), ("n_q_heads", ctypes.c_int), ("n_kv_heads", ctypes.c_int),
                ("head_dim", ctypes.c_int), ("ffn_dim", ctypes.c_int),
                ("n_experts", ctypes.c_int), ("top_k", ctypes.c_int),
                ("norm_topk_prob", ctypes.c_int), ("qkv_bias", ctypes.c_int),
                ("qk_norm", ctypes.c_int), ("rms_eps", ctypes.c_float),
                ("rope_theta", ctypes.c_float), ("dtype", ctypes.c_int),
                ("max_tokens", ctypes.c_int), ("max_batch", ctypes.c_int),
                ("shared_ffn_dim", ctypes.c_int)]


WEIGHT_FIELDS = ("ln1_g", "ln2_g", "wq", "wk", "wv", "wo", "bq", "bk", "bv", "q_norm_g",
                 "k_norm_g", "w_gate", "w_up", "w_down", "w_router", "we_gate", "we_up",
                 "we_down", "ws_gate", "ws_up", "ws_down", "w_shared_gate")


class QlWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in WEIGHT_FIELDS]


class QlTaps(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("attn", ctypes.c_void_p), ("r", ctypes.c_void_p),
                ("z", ctypes.c_void_p), ("h", ctypes.c_void_p), ("logits", ctypes.c_void_p)]


class QLayerError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    # HIP runtime: make sure torch's copy is the one in the process before the
    # library resolves its libamdhip64 dependency (one runtime per process)
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m transformer_decoder_layer_qwen_amd.build`")
    lib = ctypes.CDLL(path)
    vp, ci = ctypes.c_void_p, ctypes.c_int
    lib.qlayer_create.argtypes = [ctypes.POINTER(QlConfig), ctypes.POINTER(QlWeights),
                                  ctypes.POINTER(vp)]
    lib.qlayer_destroy.argtypes = [vp]
    lib.qlayer_workspace_bytes.argtypes = [vp]
    lib.qlayer_workspace_bytes.restype = ctypes.c_size_t
    lib.qlayer_prefill.argtypes = [vp, vp, ci, ci, ci, vp, vp, ci, vp, vp]
    lib.qlayer_decode.argtypes = [vp, vp, ci, vp, vp, ci, vp, vp, ci, vp, vp]
    lib.qlayer_prefill_varlen.argtypes = [vp, vp, ci, vp, vp, vp, vp, ci, vp, vp, ci, vp, vp]
    lib.qlayer_decode_stack.argtypes = [vp, ci, vp, ci, vp, vp, ci, vp, vp, ci, vp, vp, vp]
    lib.qlayer_decode_noalloc.argtypes = [ctypes.POINTER(QlConfig), ctypes.POINTER(QlWeights), vp,
                                          ci, vp, vp, ci, vp, vp, ci, vp, vp]
    lib.qlayer_moe_ffn.argtypes = [vp, vp, ci, vp, vp, vp, vp]
    lib.qlayer_set_taps.argtypes = [vp, ctypes.POINTER(QlTaps)]
    lib.qlayer_set_stage_events.argtypes = [vp, ci, vp, vp]
    lib.qlayer_last_error.restype = ctypes.c_char_p
    lib.qlayer_last_error.argtypes = []
    lib.qlayer_abi_version.restype = ci
    for name in ("qlayer_create", "qlayer_destroy", "qlayer_prefill", "qlayer_prefill_varlen",
                 "qlayer_decode", "qlayer_decode_stack",
                 "qlayer_decode_noalloc", "qlayer_moe_ffn", "qlayer_set_taps",
                 "qlayer_set_stage_events"):
        getattr(lib, name).restype = ci
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != QL_OK:
        msg = load_library().qlayer_last_error().decode(errors="replace")
        raise QLayerError(status, msg)


# ------------------------------------------------------ C-named wrappers ----

def qlayer_abi_version() -> int:
    return load_library().qlayer_abi_version()


def qlayer_last_error() -> str:
    return load_library().qlayer_last_error().decode(errors="replace")


def qlayer_create(cfg: QlConfig, w: QlWeights) -> int:
    h = ctypes.c_void_p()
    _check(load_library().qlayer_create(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(h)))
    return h.value


def qlayer_destroy(h: int) -> None:
    _check(load_library().qlayer_destroy(h))


def qlayer_workspace_bytes(h: int) -> int:
    return load_library().qlayer_workspace_bytes(h)


def qlayer_prefill(h, x, B, S, pos_offset, k_cache, v_cache, T_max, y, stream) -> None:
    _check(load_library().qlayer_prefill(h, x, B, S, pos_offset, k_cache, v_cache, T_max, y,
                                         stream))


def qlayer_prefill_varlen(h, x, B, seq_start, cache_len, seq_start_host, cache_len_host,
                          pos_offset, k_cache, v_cache, T_max, y, stream) -> None:
    _check(load_library().qlayer_prefill_varlen(h, x, B, seq_start, cache_len, seq_start_host,
                                                cache_len_host, pos_offset, k_cache, v_cache,
                                                T_max, y, stream))


def qlayer_decode(h, x, B, cache_len, cache_len_host, pos_offset, k_cache, v_cache, T_max, y,
                  stream) -> None:
    _check(load_library().qlayer_decode(h, x, B, cache_len, cache_len_host, pos_offset, k_cache,
                                        v_cache, T_max, y, stream))


def qlayer_decode_stack(layers, L, x, B, cache_len, cache_len_host, pos_offset, k_caches,
                        v_caches, T_max, y, tmp, stream) -> None:
    _check(load_library().qlayer_decode_stack(layers, L, x, B, cache_len, cache_len_host,
                                              pos_offset, k_caches, v_caches, T_max, y, tmp,
                                              stream))


def decode_stack(layers, x, cache_len, k_caches, v_caches, y=None, tmp=None, pos_offset=0,
                 cache_len_host=None, stream=None):
    """One decode step through QLayer objects `layers` (their handles and the
    per-layer caches marshalled into pointer arrays)."""
    torch = _torch()
    L, Bn = len(layers), x.shape[0]
    hs = (ctypes.c_void_p * L)(*[ly.handle for ly in layers])
    ks = (ctypes.c_void_p * L)(*[k.data_ptr() for k in k_caches])
    vs = (ctypes.c_void_p * L)(*[v.data_ptr() for v in v_caches])
    host = None
    if cache_len_host is not None:
        arr = (ctypes.c_int * Bn)(*[int(v) for v in cache_len_host])
        host = ctypes.cast(arr, ctypes.c_void_p).value
    y = torch.empty_like(x) if y is None else y
    tmp = torch.empty_like(x) if tmp is None else tmp
    qlayer_decode_stack(ctypes.cast(hs, ctypes.c_void_p).value, L, x.data_ptr(), Bn,
                        cache_len.data_ptr(), host, pos_offset,
                        ctypes.cast(ks, ctypes.c_void_p).value,
                        ctypes.cast(vs, ctypes.c_void_p).value, k_caches[0].shape[1],
                        y.data_ptr(), tmp.data_ptr(), _stream(stream))
    return y


def qlayer_decode_noalloc(cfg: QlConfig, w: QlWeights, x, B, cache_len, cache_len_host,
                          pos_offset, k_cache, v_cache, T_max, y, stream) -> None:
    _check(load_library().qlayer_decode_noalloc(ctypes.byref(cfg), ctypes.byref(w), x, B,
                                                cache_len, cache_len_host, pos_offset, k_cache,
                                                v_cache, T_max, y, stream))


def qlayer_moe_ffn(h, r, N, y, topk_idx, topk_w, stream) -> None:
    _check(load_library().qlayer_moe_ffn(h, r, N, y, topk_idx, topk_w, stream))


def qlayer_set_stage_events(h, stage: int, start_event, stop_event) -> None:
    _check(load_library().qlayer_set_stage_events(h, stage, start_event, stop_event))


def qlayer_set_taps(h, taps: Optional[QlTaps]) -> None:
    _check(load_library().qlayer_set_taps(h, ctypes.byref(taps) if taps is not None else None))


# ------------------------------------------------------------ torch side ----

def _torch():
    import torch
    return torch


def to_device(arr: np.ndarray, device="cuda"):
    """Stored tensor (bf16 bits as uint16, or float32) -> torch tensor on device."""
    torch = _torch()
    if arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(
            torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)


def to_host_f32(t) -> np.ndarray:
    """Device tensor -> float32 numpy (bf16 widened exactly)."""
    torch = _torch()
    return t.detach().to(torch.float32).cpu().numpy()


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


class QLayer:
    """One layer's handle: weights (device tensors) + library workspace."""

    def __init__(self, cfg, weights: Dict[str, "object"], max_tokens: int = 0,
                 max_batch: int = 0):
        torch = _torch()
        self.cfg = cfg
        self.dtype = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        for name, t in weights.items():
            if t is None:
                continue
            if t.dtype != self.dtype or not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"weight {name}: need a contiguous {self.dtype} CUDA tensor")
        self._weights = dict(weights)   # keep the memory alive for the handle's lifetime
        c = QlConfig(d=cfg.d, n_q_heads=cfg.n_q_heads, n_kv_heads=cfg.n_kv_heads,
                     head_dim=cfg.head_dim, ffn_dim=cfg.ffn_dim, n_experts=cfg.n_experts,
                     top_k=cfg.top_k, norm_topk_prob=int(cfg.norm_topk_prob),
                     qkv_bias=int(cfg.qkv_bias), qk_norm=int(cfg.qk_norm),
                     rms_eps=cfg.rms_eps, rope_theta=cfg.rope_theta,
                     dtype=QL_BF16 if cfg.dtype == "bf16" else QL_F32,
                     max_tokens=max_tokens, max_batch=max_batch,
                     shared_ffn_dim=getattr(cfg, "shared_ffn_dim", 0))
        w = QlWeights(**{n: _ptr(weights.get(n)) for n in WEIGHT_FIELDS})
        self.c_config, self.c_weights = c, w
        self.handle = qlayer_create(c, w)
        self.max_tokens, self.max_batch = max_tokens, max_batch
        self._taps = None

    # -- entry points ------------------------------------------------------
    def prefill(self, x, k_cache, v_cache, pos_offset: int = 0, y=None, stream=None):
        torch = _torch()
        B, S, d = x.shape
        self._check_act(x, (B, S, self.cfg.d))
        self._check_cache(k_cache, v_cache, B)
        if y is None:
            y = torch.empty_like(x)
        qlayer_prefill(self.handle, x.data_ptr(), B, S, pos_offset, k_cache.data_ptr(),
                       v_cache.data_ptr(), k_cache.shape[1], y.data_ptr(), _stream(stream))
        return y

    def decode(self, x, cache_len, k_cache, v_cache, pos_offset: int = 0, cache_len_host=None,
               y=None, stream=None):
        torch = _torch()
        B = x.shape[0]
        self._check_act(x, (B, self.cfg.d))
        self._check_cache(k_cache, v_cache, B)
        if cache_len.dtype != torch.int32 or not cache_len.is_cuda or cache_len.numel() != B:
            raise ValueError("cache_len: need a CUDA int32 tensor of B entries")
        host = None
        if cache_len_host is not None:
            arr = (ctypes.c_int * B)(*[int(v) for v in cache_len_host])
            host = ctypes.cast(arr, ctypes.c_void_p).value
        if y is None:
            y = torch.empty_like(x)
        qlayer_decode(self.handle, x.data_ptr(), B, cache_len.data_ptr(), host, pos_offset,
                      k_cache.data_ptr(), v_cache.data_ptr(), k_cache.shape[1], y.data_ptr(),
                      _stream(stream))
        return y

    def prefill_varlen(self, x, seq_start, cache_len, k_cache, v_cache, pos_offset: int = 0,
                       y=None, stream=None):
        """x [N, d]; seq_start [B + 1] and cache_len [B] as Python int lists (the
        device copies are made here)."""
        torch = _torch()
        N = x.shape[0]
        B = len(cache_len)
        self._check_act(x, (N, self.cfg.d))
        self._check_cache(k_cache, v_cache, B)
        if len(seq_start) != B + 1 or seq_start[-1] != N:
            raise ValueError("seq_start: need B + 1 offsets ending at N")
        ss_d = torch.tensor(seq_start, dtype=torch.int32, device=x.device)
        cl_d = torch.tensor(cache_len, dtype=torch.int32, device=x.device)
        ss_h = (ctypes.c_int * (B + 1))(*[int(v) for v in seq_start])
        cl_h = (ctypes.c_int * B)(*[int(v) for v in cache_len])
        self._varlen_keep = (ss_d, cl_d)   # alive until the stream has used them
        if y is None:
            y = torch.empty_like(x)
        qlayer_prefill_varlen(self.handle, x.data_ptr(), B, ss_d.data_ptr(), cl_d.data_ptr(),
                              ctypes.cast(ss_h, ctypes.c_void_p).value,
                              ctypes.cast(cl_h, ctypes.c_void_p).value, pos_offset,
                              k_cache.data_ptr(), v_cache.data_ptr(), k_cache.shape[1],
                              y.data_ptr(), _stream(stream))
        return y

    def moe_ffn(self, r, y=None, topk_idx=None, topk_w=None, stream=None):
        torch = _torch()
        N = r.shape[0]
        self._check_act(r, (N, self.cfg.d))
        if y is None:
            y = torch.empty_like(r)
        qlayer_moe_ffn(self.handle, r.data_ptr(), N, y.data_ptr(), _ptr(topk_idx), _ptr(topk_w),
                       _stream(stream))
        return y

    def set_taps(self, q=None, attn=None, r=None, z=None, h=None, logits=None):
        self._taps_tensors = (q, attn, r, z, h, logits)
        self._taps = QlTaps(q=_ptr(q), attn=_ptr(attn), r=_ptr(r), z=_ptr(z), h=_ptr(h),
                            logits=_ptr(logits))
        qlayer_set_taps(self.handle, self._taps)

    def set_stage_events(self, stage: str, start_event, stop_event):
        """Record raw hipEvent_t handles around one stage of every later call."""
        qlayer_set_stage_events(self.handle, STAGES[stage] if stage else 0, start_event,
                                stop_event)

    def clear_taps(self):
        self._taps = None
        qlayer_set_taps(self.handle, None)

    @property
    def workspace_bytes(self) -> int:
        return qlayer_workspace_bytes(self.handle)

    def close(self):
        if getattr(self, "handle", None):
            qlayer_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- checks ------------------------------------------------------------
    def _check_act(self, t, shape):
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"expected shape {shape}, got {tuple(t.shape)}")
        if t.dtype != self.dtype or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"need a contiguous {self.dtype} CUDA tensor")

    def _check_cache(self, k, v, B):
        shp = (B, k.shape[1], self.cfg.n_kv_heads, self.cfg.head_dim)
        for t in (k, v):
            self._check_act(t, shp)


def device_weights(w_np: Dict[str, np.ndarray], device="cuda"):
    """Stored weights (from ``synth.make_weights``) -> dict of device tensors."""
    return {k: to_device(v, device) for k, v in w_np.items()}
