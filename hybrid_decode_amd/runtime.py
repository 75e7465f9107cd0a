"""Device-side plumbing around the C-ABI: torch allocates, the library computes.

Builds the C structs of ``binding`` from host arrays (the synthetic generator's
output), owns the device tensors behind every pointer, and offers the layer
loop of a decode stack.  Nothing here does any of the decode arithmetic.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as B

_KERNELS = {}


def kernels(device: int = 0) -> int:
    """Resolve the kernel table once per device (fails without a gfx950 GPU)."""
    if device not in _KERNELS:
        _KERNELS[device] = B.q35_kernels_resolve(device)
    return _KERNELS[device]


def cfg_struct(cfg) -> B.Qwen35ForwardConfig:
    c = B.Qwen35ForwardConfig()
    for name, _ in B.Qwen35ForwardConfig._fields_:
        if name == "act_dtype":
            c.act_dtype = B.Q35_ACT_F32 if cfg.act_dtype == "f32" else B.Q35_ACT_BF16
        else:
            setattr(c, name, getattr(cfg, name))
    return c


def stream_ptr(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def to_dev(arr: np.ndarray, device="cuda") -> torch.Tensor:
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


def ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def act_dtype(cfg):
    return torch.float32 if cfg.act_dtype == "f32" else torch.int16


def act_empty(cfg, n: int, device="cuda") -> torch.Tensor:
    return torch.zeros(n, dtype=act_dtype(cfg), device=device)


def act_to_host(t: torch.Tensor, cfg) -> np.ndarray:
    a = t.detach().cpu().numpy()
    return a.view(np.uint16) if cfg.act_dtype == "bf16" else a


def act_to_f32(t: torch.Tensor, cfg) -> np.ndarray:
    a = act_to_host(t, cfg)
    if cfg.act_dtype == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32)
    return a


class QuantWeightDev:
    def __init__(self, w: dict, device="cuda"):
        self.codes = to_dev(w["codes"], device)
        self.scales = to_dev(w["scales"], device)
        self.biases = to_dev(w["biases"], device)
        n, k = w["codes"].shape
        self.n, self.k = n, k
        self.struct = B.Q35QuantWeight(ptr(self.codes), ptr(self.scales), ptr(self.biases), n, k)

    @property
    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.codes, self.scales, self.biases))


class GdnLayerDev:
    QUANT = ("in_proj_a", "in_proj_b", "in_proj_qkv", "in_proj_z", "out_proj", "gate_proj",
             "up_proj", "down_proj")
    VEC = ("input_ln", "a_log", "dt_bias", "conv1d_weight", "norm_weight", "post_ln")

    def __init__(self, layer: dict, device="cuda"):
        self.t = {k: to_dev(layer[k], device) for k in self.VEC}
        self.q = {k: QuantWeightDev(layer[k], device) for k in self.QUANT}
        s = B.LinearAttentionLayer()
        for k in self.VEC:
            setattr(s, k, ptr(self.t[k]))
        for k in self.QUANT:
            setattr(s, k, self.q[k].struct)
        self.struct = s

    @property
    def weight_bytes(self) -> int:
        return sum(q.nbytes for q in self.q.values())


class FullLayerDev:
    QUANT = ("q_proj", "k_proj", "v_proj", "o_proj", "gate_proj", "up_proj", "down_proj")
    VEC = ("input_ln", "q_norm", "k_norm", "post_ln")

    def __init__(self, layer: dict, device="cuda"):
        self.t = {k: to_dev(layer[k], device) for k in self.VEC}
        self.q = {k: QuantWeightDev(layer[k], device) for k in self.QUANT}
        s = B.FullAttentionLayer()
        for k in self.VEC:
            setattr(s, k, ptr(self.t[k]))
        for k in self.QUANT:
            setattr(s, k, self.q[k].struct)
        self.struct = s

    @property
    def weight_bytes(self) -> int:
        return sum(q.nbytes for q in self.q.values())


class GdnStateDev:
    def __init__(self, state: dict, device="cuda"):
        self.conv1d_state = to_dev(state["conv1d_state"], device)
        self.gdn_state = to_dev(state["gdn_state"], device)
        self.struct = B.LinearAttentionState(ptr(self.conv1d_state), ptr(self.gdn_state))

    def to_host(self) -> dict:
        return {"conv1d_state": self.conv1d_state.cpu().numpy(),
                "gdn_state": self.gdn_state.cpu().numpy()}


class KvCacheDev:
    """One layer's KV cache in device memory, its format read from the arrays:
    bf16: {"k", "v"} uint16 bits [cap, Hkv, D]; Turbo8 ("k_scales" present):
    "k", "v" uint8 E4M3 codes [cap, Hkv, D], "k_scales", "v_scales" bf16 bits
    [cap, Hkv, D/16]; a Lloyd-Max format (named by "kv_dtype"; "v_scales" only
    means Bf16K + Turbo4V): packed indices uint8 [cap, Hkv, D*bits/8] and E4M3
    scale bytes [cap, Hkv, D/16] for each quantised side, "k" bf16 bits
    [cap, Hkv, D] for the asymmetric ones."""

    # the sparse-V threshold the pages' Turbo branch uses unless overridden
    SPARSE_V_DEFAULT = 1e-3

    def __init__(self, kv: dict, device="cuda", sparse_v: float = SPARSE_V_DEFAULT):
        if "kv_dtype" in kv:
            self.dtype = B.KV_DTYPES.index(kv["kv_dtype"])
        elif "k_scales" in kv:
            self.dtype = B.Q35_KV_TURBO8
        elif "v_scales" in kv:
            self.dtype = B.Q35_KV_BF16K_TURBO4V
        else:
            self.dtype = B.Q35_KV_BF16
        self.turbo8 = self.dtype == B.Q35_KV_TURBO8
        self.k = to_dev(kv["k"], device)
        self.v = to_dev(kv["v"], device)
        self.capacity = int(kv["k"].shape[0])
        self.k_scales = to_dev(kv["k_scales"], device) if "k_scales" in kv else None
        self.v_scales = to_dev(kv["v_scales"], device) if "v_scales" in kv else None
        self.sparse_v = float(sparse_v)
        self.struct = B.LayerKvCache(ptr(self.k), ptr(self.v), self.capacity, self.dtype,
                                     ptr(self.k_scales), ptr(self.v_scales), self.sparse_v)

    def to_host(self) -> dict:
        """The arrays as NumPy, in the dtypes the generators use."""
        def host(t):
            a = t.cpu().numpy()
            return a.view(np.uint16) if a.dtype == np.int16 else a
        out = {"k": host(self.k), "v": host(self.v)}
        if self.k_scales is not None:
            out["k_scales"] = host(self.k_scales)
        if self.v_scales is not None:
            out["v_scales"] = host(self.v_scales)
        return out


def _f32(n, device):
    return torch.zeros(n, dtype=torch.float32, device=device)


class GdnScratchDev:
    TAPS = ("x_norm", "dt_raw", "b_raw", "qkv", "qkv_smooth", "y_norm", "out", "x_norm2",
            "gate_act", "up_act")

    def __init__(self, cfg, taps: bool = False, device="cuda"):
        H, I, Hv = cfg.hidden, cfg.intermediate, cfg.num_v_heads_lin
        qt, zd = cfg.qkv_total_lin, cfg.z_dim_lin
        sizes = {"qkv_conv": qt, "z": zd, "gate": Hv, "beta": Hv, "y": zd, "x_resid": H,
                 "mlp_act": I, "x_norm": H, "dt_raw": Hv, "b_raw": Hv, "qkv": qt,
                 "qkv_smooth": qt, "y_norm": zd, "out": H, "x_norm2": H, "gate_act": I,
                 "up_act": I}
        self.t = {}
        s = B.LinearAttentionScratch()
        for name, n in sizes.items():
            if name in self.TAPS and not taps:
                continue
            self.t[name] = _f32(n, device)
            setattr(s, name, ptr(self.t[name]))
        if taps:
            self.t["x_final"] = act_empty(cfg, H, device)
            s.x_final = ptr(self.t["x_final"])
        self.struct = s


class FullScratchDev:
    TAPS = ("x_norm", "q_norm_out", "k_norm_out", "attn_out", "o", "x_norm2", "gate_act", "up_act")

    def __init__(self, cfg, capacity: int, taps: bool = False, device="cuda"):
        H, I = cfg.hidden, cfg.intermediate
        sizes = {"q_full": cfg.q_total, "k": cfg.kv_dim, "v": cfg.kv_dim, "gated_attn": cfg.q_only,
                 "x_resid": H, "mlp_act": I, "x_norm": H, "q_norm_out": cfg.q_only,
                 "k_norm_out": cfg.kv_dim, "attn_out": cfg.q_only, "o": H, "x_norm2": H,
                 "gate_act": I, "up_act": I}
        self.t = {}
        s = B.FullAttentionScratch()
        for name, n in sizes.items():
            if name in self.TAPS and not taps:
                continue
            self.t[name] = _f32(n, device)
            setattr(s, name, ptr(self.t[name]))
        self.t["x_out"] = act_empty(cfg, H, device)
        s.x_out = ptr(self.t["x_out"])
        nbytes = B.q35_full_attention_workspace_bytes(cfg_struct(cfg), capacity)
        self.t["workspace"] = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        s.workspace = ptr(self.t["workspace"])
        s.workspace_bytes = nbytes
        self.t["status"] = torch.zeros(1, dtype=torch.int32, device=device)
        s.status = ptr(self.t["status"])
        self.struct = s


# --------------------------------------------------------------------------- layer calls

def forward_linear_attention(cfg, layer: GdnLayerDev, state: GdnStateDev, scratch: GdnScratchDev,
                             x_in: torch.Tensor, x_buf: torch.Tensor, device: int = 0,
                             stream=None, dump=None) -> int:
    return B.q35_forward_linear_attention(kernels(device), cfg_struct(cfg), layer.struct,
                                          state.struct, scratch.struct, ptr(x_in), ptr(x_buf),
                                          stream_ptr(stream), dump)


def forward_full_attention(cfg, layer: FullLayerDev, scratch: FullScratchDev, kv: KvCacheDev,
                           inv_freq: torch.Tensor, positions: torch.Tensor, x_in: torch.Tensor,
                           cache_pos: int | None, device: int = 0, stream=None) -> int:
    """cache_pos None: the position is read on the device from positions[0]."""
    if cache_pos is None:
        return B.q35_forward_full_attention_devpos(kernels(device), cfg_struct(cfg), layer.struct,
                                                   scratch.struct, kv.struct, ptr(inv_freq),
                                                   ptr(positions), ptr(x_in), stream_ptr(stream))
    return B.q35_forward_full_attention(kernels(device), cfg_struct(cfg), layer.struct,
                                        scratch.struct, kv.struct, ptr(inv_freq), ptr(positions),
                                        ptr(x_in), cache_pos, cache_pos + 1, stream_ptr(stream))


def inv_freq_dev(cfg, device="cuda") -> torch.Tensor:
    return torch.from_numpy(B.q35_rope_inv_freq(cfg_struct(cfg))).to(device)


# --------------------------------------------------------------------------- persistent decode

def _stack_desc(kinds, layers, states, kvs, inv_freq, positions, tail):
    """Q35DecodeStackDesc of a stack (and the host array it points into)."""
    import ctypes as C
    n = len(kinds)
    arr = (B.Q35StackLayer * n)()
    for i, kind in enumerate(kinds):
        if kind == "gdn":
            arr[i].kind = B.Q35_LAYER_LINEAR
            arr[i].linear = C.pointer(layers[i].struct)
            arr[i].state = C.pointer(states[i].struct)
        else:
            arr[i].kind = B.Q35_LAYER_FULL
            arr[i].full = C.pointer(layers[i].struct)
            arr[i].kv = C.pointer(kvs[i].struct)
    d = B.Q35DecodeStackDesc()
    d.n_layers = n
    d.layers = arr
    d.inv_freq = ptr(inv_freq)
    d.positions = ptr(positions)
    if tail is not None:
        d.lm_head = C.pointer(tail["lm_head"].struct)
        d.final_norm = ptr(tail["final_norm"])
        d.embed = ptr(tail["embed"])
        d.tokens = ptr(tail["tokens"])
        d.logits = ptr(tail.get("logits"))
        d.history = ptr(tail.get("history"))
        d.history_len = tail.get("history_len", 0)
        d.history_base = tail.get("history_base", 0)
    return arr, d


class DecodePlan:
    """A stack's layers (and optionally its tail) run by the persistent decode
    kernel: ``step()`` is one cooperative launch per token."""

    def __init__(self, cfg, kinds, layers, states, kvs, inv_freq, positions, tail=None,
                 device: int = 0):
        self.cfg, self.kinds, self.device = cfg, list(kinds), device
        self.c = cfg_struct(cfg)
        self.k = kernels(device)
        n = len(kinds)
        arr, d = _stack_desc(kinds, layers, states, kvs, inv_freq, positions, tail)
        self.tail = tail
        self._keep = (arr, d, layers, states, kvs, inv_freq, positions)
        nbytes = B.q35_decode_workspace_bytes(self.k, self.c, d)
        self.ws = torch.zeros(nbytes + 256, dtype=torch.uint8, device=f"cuda:{device}")
        off = (-self.ws.data_ptr()) % 256
        self.ws_off = off
        self.plan = B.q35_decode_plan_create(self.k, self.c, d, self.ws.data_ptr() + off, nbytes)
        self.n_stages, self.first_stage = B.q35_decode_stage_layout(self.plan, n)

    def step(self, stream=None) -> None:
        B.q35_decode_step(self.plan, stream_ptr(stream))

    def check(self) -> int:
        """Error word of the plan (0: every inter-block wait completed)."""
        return B.q35_decode_check(self.plan)

    def layer_input(self, layer: int) -> torch.Tensor:
        """View of layer `layer`'s input residual stream (layer == n: the last output)."""
        p = B.q35_decode_layer_input(self.plan, layer)
        o = p - self.ws.data_ptr()
        nb = self.cfg.hidden * (4 if self.cfg.act_dtype == "f32" else 2)
        return self.ws[o:o + nb].view(act_dtype(self.cfg))

    def stage_times_us(self):
        ticks, hz = B.q35_decode_stage_times(self.plan, self.n_stages)
        return ticks, hz

    def __del__(self):
        try:
            B.q35_decode_plan_release(self.plan)
        except Exception:
            pass


# --------------------------------------------------------------------------- XCD-split decode

class XcdPlan:
    """A stack's layers (and optionally its tail) with the steps that split over
    the eight XCDs joined per launch: ``step()`` enqueues one token (two launches
    per GDN layer, four per full-attention layer, then the tail)."""

    def __init__(self, cfg, kinds, layers, states, kvs, inv_freq, positions, tail=None,
                 device: int = 0):
        self.cfg, self.kinds, self.device = cfg, list(kinds), device
        self.c = cfg_struct(cfg)
        self.k = kernels(device)
        arr, d = _stack_desc(kinds, layers, states, kvs, inv_freq, positions, tail)
        self.tail = tail
        self._keep = (arr, d, layers, states, kvs, inv_freq, positions)
        nbytes = B.q35_xcd_workspace_bytes(self.k, self.c, d)
        self.ws = torch.zeros(nbytes + 256, dtype=torch.uint8, device=f"cuda:{device}")
        off = (-self.ws.data_ptr()) % 256
        self.plan = B.q35_xcd_plan_create(self.k, self.c, d, self.ws.data_ptr() + off, nbytes)
        self._bufs = B.q35_xcd_buffers(self.plan)

    def step(self, stream=None) -> None:
        B.q35_xcd_step(self.plan, stream_ptr(stream))

    def check(self) -> int:
        """Error word of the plan (0: every wait completed, every block on its XCD)."""
        return B.q35_xcd_check(self.plan)

    def _view(self, p: int, n: int, dtype) -> torch.Tensor:
        o = p - self.ws.data_ptr()
        nb = n * torch.empty((), dtype=dtype).element_size()
        return self.ws[o:o + nb].view(dtype)

    def layer_input(self, layer: int) -> torch.Tensor:
        """The first layer's input (0) or the last layer's output (n_layers), act [hidden]."""
        return self._view(B.q35_xcd_layer_input(self.plan, layer), self.cfg.hidden, act_dtype(self.cfg))

    def buffer(self, name: str, n: int, dtype=torch.float32) -> torch.Tensor:
        """View of one of the plan's shared buffers (Q35XcdBuffers field `name`)."""
        return self._view(getattr(self._bufs, name), n, dtype)

    def __del__(self):
        try:
            B.q35_xcd_plan_release(self.plan)
        except Exception:
            pass


# --------------------------------------------------------------------------- decode stack

class DecodeStack:
    """A stack of GDN / full-attention layers plus embedding and int8 lm_head.

    One ``step()`` is one greedy decode token entirely on the device: the
    layer loop, final RMSNorm, lm_head GEMV, argmax, the next token's
    embedding, and the position increment, so it can be captured once into a
    HIP graph and replayed.
    """

    def __init__(self, cfg, kinds, layers, states, kvs, embed, final_norm, lm_head, start_pos: int,
                 start_token: int, history_len: int = 0, device: int = 0, taps: bool = False,
                 persistent: bool = False, xcd: bool = False):
        dev = f"cuda:{device}"
        self.cfg, self.kinds, self.device = cfg, list(kinds), device
        self.c = cfg_struct(cfg)
        B.q35_config_validate(self.c)
        self.layers = [GdnLayerDev(l, dev) if k == "gdn" else FullLayerDev(l, dev)
                       for k, l in zip(kinds, layers)]
        self.states = [GdnStateDev(s, dev) if s is not None else None for s in states]
        self.kvs = [KvCacheDev(kv, dev) if kv is not None else None for kv in kvs]
        cap = max([kv.capacity for kv in self.kvs if kv is not None] or [1])
        self.gdn_scratch = GdnScratchDev(cfg, taps, dev)
        self.full_scratch = FullScratchDev(cfg, cap, taps, dev)
        self.embed = to_dev(embed, dev)
        self.final_norm = to_dev(final_norm, dev)
        self.lm_head = QuantWeightDev(lm_head, dev)
        self.inv_freq = inv_freq_dev(cfg, dev)
        self.positions = torch.tensor([start_pos], dtype=torch.int32, device=dev)
        self.tokens = torch.tensor([start_token], dtype=torch.int32, device=dev)
        self.history_len = history_len
        self.history_base = start_pos
        self.history = torch.full((max(history_len, 1),), -1, dtype=torch.int32, device=dev)
        self.x_embed = act_empty(cfg, cfg.hidden, dev)
        self.x_main = act_empty(cfg, cfg.hidden, dev)
        self.logits = torch.zeros(cfg.vocab, dtype=torch.float32, device=dev)
        nb = B.q35_lm_head_workspace_bytes(self.c)
        self.lm_ws = torch.zeros(nb, dtype=torch.uint8, device=dev)
        self.k = kernels(device)
        B.q35_embed_lookup(self.k, self.c, ptr(self.embed), ptr(self.tokens), ptr(self.x_embed),
                           stream_ptr())
        self.plan = None
        if persistent or xcd:
            tail = {"lm_head": self.lm_head, "final_norm": self.final_norm, "embed": self.embed,
                    "tokens": self.tokens, "logits": self.logits,
                    "history": self.history if history_len else None,
                    "history_len": history_len, "history_base": self.history_base}
            cls = XcdPlan if xcd else DecodePlan
            self.plan = cls(cfg, self.kinds, self.layers, self.states, self.kvs,
                            self.inv_freq, self.positions, tail, device)

    @property
    def weight_bytes(self) -> int:
        return sum(l.weight_bytes for l in self.layers) + self.lm_head.nbytes

    def step(self, stream=None, write_logits: bool = True) -> None:
        if self.plan is not None:  # the plan's launches (logits always written when held)
            self.plan.step(stream)
            return
        s = stream_ptr(stream)
        x = ptr(self.x_embed)
        for li, kind in enumerate(self.kinds):
            if kind == "gdn":
                x = B.q35_forward_linear_attention(self.k, self.c, self.layers[li].struct,
                                                   self.states[li].struct, self.gdn_scratch.struct,
                                                   x, ptr(self.x_main), s)
            else:
                x = B.q35_forward_full_attention_devpos(self.k, self.c, self.layers[li].struct,
                                                        self.full_scratch.struct,
                                                        self.kvs[li].struct, ptr(self.inv_freq),
                                                        ptr(self.positions), x, s)
        self.last_x = x
        B.q35_lm_head_argmax(self.k, self.c, ptr(self.final_norm), self.lm_head.struct, x,
                             ptr(self.logits) if write_logits else None, ptr(self.lm_ws),
                             self.lm_ws.numel(), ptr(self.tokens), ptr(self.positions),
                             ptr(self.history) if self.history_len else None, self.history_len,
                             self.history_base, ptr(self.embed), ptr(self.x_embed), s)
