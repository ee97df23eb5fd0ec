"""Python binding of librdt: the recurrent-depth transformer block on MI355X.

Argument marshalling only -- every step of the T-loop runs in the HIP kernels of
librdt.so (built in-tree by ``recurrent_depth_transformer_amd.build``). PyTorch
provides device memory and streams. Importing this module never falls back to
anything: if librdt.so is missing, ``load_library`` raises.

    blk = RecurrentBlock(cfg)                 # cfg: dict of rdt_config fields
    W = device_weights(inputs, cfg, "cuda")   # numpy arrays -> device tensors
    out = blk.forward(W["h0"], W["e"], W, T=cfg["T"])
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["RdtConfig", "RdtWeights", "RdtAux", "RdtError", "RecurrentBlock", "load_library",
           "device_weights", "make_config", "EXPORTED_SYMBOLS", "LIB_PATH", "router_bias_update",
           "expert_depths"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "librdt.so")

EXPORTED_SYMBOLS = [
    "rdt_config_default", "rdt_config_validate", "rdt_create", "rdt_destroy",
    "rdt_workspace_size", "rdt_spectral_radius", "rdt_set_graph_mode",
    "rdt_recurrent_forward", "rdt_profile_forward", "rdt_stage_name", "rdt_last_error", "rdt_version",
    "rdt_cache_size", "rdt_prefill", "rdt_decode_workspace_size", "rdt_decode_step",
    "rdt_router_bias_update", "rdt_expert_depths", "rdt_recurrent_forward_noalloc",
]
NOALLOC_SCRATCH_BYTES = 32 << 20   # RDT_NOALLOC_SCRATCH_BYTES
N_STAGES = 13

RDT_OK, RDT_E_INVALID, RDT_E_UNSUPPORTED, RDT_E_UNSTABLE, RDT_E_WORKSPACE, RDT_E_HIP = 0, -1, -2, -3, -4, -5
_STATUS = {RDT_E_INVALID: "RDT_E_INVALID", RDT_E_UNSUPPORTED: "RDT_E_UNSUPPORTED",
           RDT_E_UNSTABLE: "RDT_E_UNSTABLE", RDT_E_WORKSPACE: "RDT_E_WORKSPACE", RDT_E_HIP: "RDT_E_HIP"}

_i32, _f32, _vp = ctypes.c_int32, ctypes.c_float, ctypes.c_void_p


class RdtConfig(ctypes.Structure):
    _fields_ = [("batch", _i32), ("seq", _i32), ("dim", _i32), ("attn_type", _i32),
                ("n_heads", _i32), ("n_kv_heads", _i32), ("head_dim", _i32),
                ("q_lora_rank", _i32), ("kv_lora_rank", _i32), ("qk_rope_head_dim", _i32),
                ("qk_nope_head_dim", _i32), ("v_head_dim", _i32),
                ("rope_base", _f32), ("norm_eps", _f32),
                ("n_experts", _i32), ("n_shared_experts", _i32), ("top_k", _i32), ("expert_dim", _i32),
                ("n_bias_rows", _i32), ("lora_rank", _i32), ("n_lora", _i32),
                ("act_enabled", _i32), ("act_threshold", _f32), ("dtype", _i32), ("max_T", _i32),
                ("parallel_block", _i32), ("shared_scale", _i32),
                ("da_heads", _i32), ("da_kv_heads", _i32), ("da_head_dim", _i32)]


WEIGHT_FIELDS = ["g1", "g2", "Wq", "Wk", "Wv", "Wdq", "gq", "Wuq", "Wdkv", "gkv", "Wuk", "Wuv",
                 "Wo", "Wr", "router_bias", "Wg", "Wu", "Wd", "Wsg", "Wsu", "Wsd",
                 "lora_down", "lora_up", "w_halt", "A", "B", "Wq_da", "Wk_da", "Wv_da", "Wo_da", "g_da"]
AUX_FIELDS = ["loops", "route_idx", "route_gap", "expert_counts", "act_cum", "n2_dump", "a_dump", "h_dump"]


class RdtWeights(ctypes.Structure):
    _fields_ = [(n, _vp) for n in WEIGHT_FIELDS]


class RdtAux(ctypes.Structure):
    _fields_ = [(n, _vp) for n in AUX_FIELDS]


class RdtError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH):
    """Load librdt.so (raises when it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"librdt.so not found at {path}; build it with "
                           "`python -m recurrent_depth_transformer_amd.build`")
    lib = ctypes.CDLL(path)
    lib.rdt_config_default.argtypes = [ctypes.POINTER(RdtConfig)]
    lib.rdt_config_validate.argtypes = [ctypes.POINTER(RdtConfig)]
    lib.rdt_create.argtypes = [ctypes.POINTER(RdtConfig), ctypes.POINTER(_vp)]
    lib.rdt_destroy.argtypes = [_vp]
    lib.rdt_destroy.restype = None
    lib.rdt_workspace_size.argtypes = [_vp, _i32]
    lib.rdt_workspace_size.restype = ctypes.c_size_t
    lib.rdt_spectral_radius.argtypes = [ctypes.POINTER(_f32), _i32, ctypes.POINTER(_f32)]
    lib.rdt_set_graph_mode.argtypes = [_vp, _i32]
    lib.rdt_recurrent_forward.argtypes = [_vp, _vp, _vp, ctypes.POINTER(RdtWeights), _i32, _vp,
                                          ctypes.POINTER(RdtAux), _vp, ctypes.c_size_t, _vp]
    lib.rdt_recurrent_forward_noalloc.argtypes = [_vp, _vp, _vp, ctypes.POINTER(RdtWeights), _i32, _vp,
                                                  ctypes.POINTER(RdtAux), _vp]
    lib.rdt_profile_forward.argtypes = [_vp, _vp, _vp, ctypes.POINTER(RdtWeights), _i32, _vp,
                                        ctypes.POINTER(RdtAux), _vp, ctypes.c_size_t, _vp,
                                        ctypes.POINTER(_f32), ctypes.POINTER(_i32), _i32]
    lib.rdt_cache_size.argtypes = [ctypes.POINTER(RdtConfig), _i32, _i32]
    lib.rdt_cache_size.restype = ctypes.c_size_t
    lib.rdt_prefill.argtypes = [_vp, _vp, _vp, ctypes.POINTER(RdtWeights), _i32, _vp, ctypes.POINTER(RdtAux),
                                _vp, _i32, _vp, ctypes.c_size_t, _vp]
    lib.rdt_decode_workspace_size.argtypes = [_vp, _i32, _i32]
    lib.rdt_decode_workspace_size.restype = ctypes.c_size_t
    lib.rdt_decode_step.argtypes = [_vp, _vp, _vp, ctypes.POINTER(RdtWeights), _i32, _i32, _vp, _i32, _vp,
                                    ctypes.POINTER(RdtAux), _vp, ctypes.c_size_t, _vp]
    lib.rdt_router_bias_update.argtypes = [_vp, _i32, _i32, _vp, _i32, _f32, _vp]
    lib.rdt_expert_depths.argtypes = [_vp, _i32, _i32, _vp, _vp]
    lib.rdt_stage_name.argtypes = [_i32]
    lib.rdt_stage_name.restype = ctypes.c_char_p
    lib.rdt_last_error.restype = ctypes.c_char_p
    lib.rdt_version.restype = ctypes.c_char_p
    for name in ["rdt_config_default", "rdt_config_validate", "rdt_create", "rdt_spectral_radius",
                 "rdt_set_graph_mode", "rdt_recurrent_forward", "rdt_profile_forward", "rdt_prefill",
                 "rdt_decode_step", "rdt_router_bias_update", "rdt_expert_depths",
                 "rdt_recurrent_forward_noalloc"]:
        getattr(lib, name).restype = _i32
    _lib = lib
    return lib


def _check(status: int):
    if status != RDT_OK:
        raise RdtError(status, load_library().rdt_last_error().decode())


def make_config(cfg: dict) -> RdtConfig:
    """rdt_config from a workload dict (field names as in rdt.h)."""
    lib = load_library()
    c = RdtConfig()
    _check(lib.rdt_config_default(ctypes.byref(c)))
    mla = cfg.get("attn", "gqa") == "mla"
    c.batch, c.seq, c.dim = cfg["batch"], cfg["seq"], cfg["dim"]
    c.attn_type = 1 if mla else 0
    c.n_heads = cfg["n_heads"]
    c.n_kv_heads = cfg.get("n_kv_heads", cfg["n_heads"])
    c.head_dim = cfg.get("head_dim", 0) if not mla else 0
    for f in ("q_lora_rank", "kv_lora_rank", "qk_rope_head_dim", "qk_nope_head_dim", "v_head_dim"):
        setattr(c, f, int(cfg.get(f, 0)) if mla else 0)
    c.rope_base = float(cfg.get("rope_base", 10000.0))
    c.norm_eps = float(cfg.get("norm_eps", 1e-6))
    c.n_experts, c.top_k, c.expert_dim = cfg["n_experts"], cfg["top_k"], cfg["expert_dim"]
    c.n_shared_experts = cfg.get("n_shared_experts", 0)
    c.n_bias_rows = cfg.get("n_bias_rows", 1)
    c.lora_rank, c.n_lora = cfg.get("lora_rank", 0), cfg.get("n_lora", 0)
    c.act_enabled = 1 if cfg.get("act", False) else 0
    c.act_threshold = float(cfg.get("act_threshold", 0.99))
    c.dtype = 0 if cfg.get("dtype", "bf16") == "f32" else 1
    c.max_T = int(cfg.get("max_T", max(16, int(cfg.get("T", 16)))))
    c.parallel_block = int(cfg.get("parallel", 0))
    c.shared_scale = int(cfg.get("shared_scale", 0))
    c.da_heads = int(cfg.get("da_heads", 0))
    c.da_kv_heads = int(cfg.get("da_kv_heads", 0))
    c.da_head_dim = int(cfg.get("da_head_dim", 0))
    return c


def device_weights(inputs: dict, cfg: dict, device="cuda") -> dict:
    """Copy drawn inputs to the device in the storage type librdt expects.

    Projection weights become bfloat16 (bf16 workloads; the values are already
    bf16-exact so the conversion is lossless) or stay float32; gains, A, B,
    router bias, halting vector, h0 and e stay float32.
    """
    import torch
    f32_names = {"g1", "g2", "gq", "gkv", "router_bias", "w_halt", "A", "B", "e", "h0", "g_da"}
    store = torch.float32 if cfg.get("dtype", "bf16") == "f32" else torch.bfloat16
    out = {}
    for k, v in inputs.items():
        t = torch.from_numpy(v)
        dt = torch.float32 if k in f32_names else store
        out[k] = t.to(device=device, dtype=dt).contiguous()
    return out


def _ptr(t):
    if t is None:
        return None
    return t.data_ptr()


class RecurrentBlock:
    """One rdt_handle: shapes fixed at construction, T chosen per call."""

    def __init__(self, cfg: dict, graph: bool = True):
        self.lib = load_library()
        self.cfg = dict(cfg)
        self.c = make_config(cfg)
        h = _vp()
        _check(self.lib.rdt_create(ctypes.byref(self.c), ctypes.byref(h)))
        self.h = h
        _check(self.lib.rdt_set_graph_mode(self.h, 1 if graph else 0))
        self._ws = None

    def close(self):
        if getattr(self, "h", None):
            self.lib.rdt_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def set_graph_mode(self, enabled: bool):
        _check(self.lib.rdt_set_graph_mode(self.h, 1 if enabled else 0))

    def workspace_size(self, T: int) -> int:
        return int(self.lib.rdt_workspace_size(self.h, int(T)))

    def workspace(self, T: int, device="cuda"):
        """A cached workspace tensor large enough for T loops."""
        import torch
        need = self.workspace_size(T)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
        return self._ws

    def forward(self, h0, e, weights: dict, T: int | None = None, out=None, aux: dict | None = None,
                workspace=None, stream=None):
        """out = h_T. Tensors live on the GPU; aux maps rdt_aux field names to
        preallocated device tensors. In graph mode the library replays the graph
        it captured for the same pointers and T: pass the same out (and
        workspace) on every call to replay it; a fresh out per call (out=None)
        captures a new graph whenever the allocator returns a new address."""
        return self._run(False, h0, e, weights, T, out, aux, workspace, stream)[0]

    def forward_noalloc(self, h0, e, weights: dict, T: int | None = None, out=None, aux: dict | None = None,
                        stream=None):
        """forward through rdt_recurrent_forward_noalloc: the library's static
        per-device scratch instead of a workspace; kernels launched one by one.
        `out` must be preallocated by the caller when nothing may allocate."""
        import torch
        T = int(self.cfg.get("T", 1) if T is None else T)
        if out is None:
            out = torch.empty_like(h0)
        w, a = self._structs(weights, aux)
        if stream is None:
            stream = torch.cuda.current_stream(h0.device).cuda_stream
        _check(self.lib.rdt_recurrent_forward_noalloc(self.h, _ptr(h0), _ptr(e), ctypes.byref(w), T, _ptr(out),
                                                      ctypes.byref(a), stream))
        return out

    def profile_forward(self, h0, e, weights: dict, T: int | None = None, out=None, aux: dict | None = None,
                        workspace=None, stream=None):
        """Kernel-by-kernel forward with HIP events around every launch.
        Returns (out, {stage name: (device ms, launches)}); waits for the GPU."""
        return self._run(True, h0, e, weights, T, out, aux, workspace, stream)

    # ---------------------------------------------------------------- decode
    def cache_size(self, T: int, max_seq: int) -> int:
        """Bytes of the per-loop K/V (MLA: latent) cache."""
        return int(self.lib.rdt_cache_size(ctypes.byref(self.c), int(T), int(max_seq)))

    def new_cache(self, T: int, max_seq: int, device="cuda"):
        import torch
        n = self.cache_size(T, max_seq)
        if n == 0:
            raise RdtError(RDT_E_INVALID, "invalid cache shape")
        return torch.empty(n, dtype=torch.uint8, device=device)

    def prefill(self, h0, e, weights: dict, T: int, cache, max_seq: int, out=None, aux: dict | None = None,
                workspace=None, stream=None):
        """Forward over the prompt that also fills the per-loop cache."""
        import torch
        if out is None:
            out = torch.empty_like(h0)
        w, a = self._structs(weights, aux)
        ws = self.workspace(T, h0.device) if workspace is None else workspace
        stream = torch.cuda.current_stream(h0.device).cuda_stream if stream is None else stream
        _check(self.lib.rdt_prefill(self.h, _ptr(h0), _ptr(e), ctypes.byref(w), int(T), _ptr(out), ctypes.byref(a),
                                    _ptr(cache), int(max_seq), _ptr(ws), ws.numel(), stream))
        return out

    def decode_workspace_size(self, T: int, max_seq: int) -> int:
        return int(self.lib.rdt_decode_workspace_size(self.h, int(T), int(max_seq)))

    def decode_step(self, h0, e, weights: dict, T: int, pos: int, cache, max_seq: int, out=None,
                    aux: dict | None = None, workspace=None, stream=None):
        """One new token per sequence ([batch, dim] state) at position pos."""
        import torch
        if out is None:
            out = torch.empty_like(h0)
        w, a = self._structs(weights, aux)
        if workspace is None:
            need = self.decode_workspace_size(T, max_seq)
            if getattr(self, "_dws", None) is None or self._dws.numel() < need:
                self._dws = torch.empty(max(need, 256), dtype=torch.uint8, device=h0.device)
            workspace = self._dws
        stream = torch.cuda.current_stream(h0.device).cuda_stream if stream is None else stream
        _check(self.lib.rdt_decode_step(self.h, _ptr(h0), _ptr(e), ctypes.byref(w), int(T), int(pos), _ptr(cache),
                                        int(max_seq), _ptr(out), ctypes.byref(a), _ptr(workspace),
                                        workspace.numel(), stream))
        return out

    def _structs(self, weights, aux):
        w = RdtWeights()
        for name in WEIGHT_FIELDS:
            setattr(w, name, _ptr(weights.get(name)))
        a = RdtAux()
        for name in AUX_FIELDS:
            setattr(a, name, _ptr((aux or {}).get(name)))
        return w, a

    def _run(self, profile, h0, e, weights, T, out, aux, workspace, stream):
        import torch
        T = int(self.cfg.get("T", 1) if T is None else T)
        if out is None:
            out = torch.empty_like(h0)
        w = RdtWeights()
        for name in WEIGHT_FIELDS:
            t = weights.get(name)
            setattr(w, name, _ptr(t))
        a = RdtAux()
        for name in AUX_FIELDS:
            setattr(a, name, _ptr((aux or {}).get(name)))
        ws = self.workspace(T, h0.device) if workspace is None else workspace
        if stream is None:
            stream = torch.cuda.current_stream(h0.device).cuda_stream
        if not profile:
            _check(self.lib.rdt_recurrent_forward(self.h, _ptr(h0), _ptr(e), ctypes.byref(w), T, _ptr(out),
                                                  ctypes.byref(a), _ptr(ws), ws.numel(), stream))
            return out, None
        ms = (_f32 * N_STAGES)()
        cnt = (_i32 * N_STAGES)()
        _check(self.lib.rdt_profile_forward(self.h, _ptr(h0), _ptr(e), ctypes.byref(w), T, _ptr(out),
                                            ctypes.byref(a), _ptr(ws), ws.numel(), stream, ms, cnt, N_STAGES))
        stages = {self.lib.rdt_stage_name(i).decode(): (float(ms[i]), int(cnt[i])) for i in range(N_STAGES)}
        return out, stages


def router_bias_update(expert_counts, router_bias, gamma: float, stream=None):
    """In-place balancing step on device tensors: expert_counts int32 [T, E],
    router_bias float32 [rows, E]."""
    import torch
    lib = load_library()
    T, E = expert_counts.shape
    rows = router_bias.shape[0]
    if router_bias.shape[1] != E or expert_counts.dtype != torch.int32 or router_bias.dtype != torch.float32:
        raise RdtError(RDT_E_INVALID, "expert_counts int32 [T, E] and router_bias float32 [rows, E] expected")
    stream = torch.cuda.current_stream(router_bias.device).cuda_stream if stream is None else stream
    _check(lib.rdt_router_bias_update(_ptr(expert_counts.contiguous()), T, E, _ptr(router_bias), rows,
                                      float(gamma), stream))
    return router_bias


def expert_depths(expert_counts, stream=None):
    """Loops in which each expert received tokens: int32 [E] device tensor."""
    import torch
    lib = load_library()
    T, E = expert_counts.shape
    out = torch.empty(E, dtype=torch.int32, device=expert_counts.device)
    stream = torch.cuda.current_stream(out.device).cuda_stream if stream is None else stream
    _check(lib.rdt_expert_depths(_ptr(expert_counts.contiguous()), T, E, _ptr(out), stream))
    return out
