"""CPU oracle for single-token decode of Qwen3.5 hybrid decoder layers.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The
product path (the HIP library and its Python binding) never does, and this
module imports nothing from it.

What it computes: the decode step of the ``qwen3_5`` forward module described
by four documentation pages (the rustdoc index "Module qwen3_5", and the
source pages ``mod.rs``, ``full_attention.rs`` and ``linear_attention.rs``).
Each function names the item of those pages it follows.  Everything is plain
NumPy in float64, with the storage formats the pages fix honoured exactly:

* weights are 8-bit affine codes with one bf16 scale and bias per 64 inputs;
* the conv state and the GDN state are fp32 (``LinearAttentionState``);
* the KV cache is bf16 (``MetalKvDtype::Bf16``);
* gate and beta are fp32 vectors;
* the residual stream between layers is held in the activation dtype
  (the GDN forward copies ``hidden * 2`` bytes into the caller's buffer).

All other intermediates stay unrounded (float64).  Where the pages leave a
step open, the reading taken is stated at that function.

Parity pins for every function live in ``tests/test_oracle_pins.py``; none
of those pins re-types a formula from here.
"""
from __future__ import annotations

import math

import numpy as np

# --------------------------------------------------------------------------- storage formats


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 (exact: bf16 is a truncated fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round to bf16 bit patterns, nearest-even, from the exact value.

    Reading: the pages never say how a value is rounded into a bf16 buffer;
    round-to-nearest-even on the unrounded value is taken.  The value is first
    rounded to fp32 (a bf16 store is fed fp32 data), then to bf16.
    """
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    nan = np.isnan(f)
    r = ((u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16))
    out = r.astype(np.uint16)
    out[nan] = np.uint16(0x7FC0)
    return out


def act_to_f64(x: np.ndarray, act_dtype: str) -> np.ndarray:
    """Activation buffer (bf16 bits or fp32 values) -> float64."""
    if act_dtype == "bf16":
        return bf16_to_f64(x)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def f64_to_act(x: np.ndarray, act_dtype: str) -> np.ndarray:
    """Store a float64 vector in the activation dtype."""
    if act_dtype == "bf16":
        return f64_to_bf16(x)
    return np.asarray(x, dtype=np.float64).astype(np.float32)


# --------------------------------------------------------------------------- quantised weights


def dequant(w: dict) -> np.ndarray:
    """Dense fp32 weights of an 8-bit affine, 64-group matrix.

    The pages show the weight trait only by name; the preset constructor of
    ``Qwen35ForwardConfig`` (``mod.rs``) names an "MLX-8bit" checkpoint with
    ``group_size`` 64.  Reading: MLX affine quantisation,
    ``W[n, k] = scale[n, k // 64] * code[n, k] + bias[n, k // 64]``, evaluated in
    fp32 (the product of a bf16 scale and a code below 256 is exact in fp32, so
    the only rounding is the single one of the sum).
    """
    codes = np.asarray(w["codes"])
    n, k = codes.shape
    s = bf16_to_f64(w["scales"]).astype(np.float32)
    b = bf16_to_f64(w["biases"]).astype(np.float32)
    s_full = np.repeat(s, 64, axis=1)
    b_full = np.repeat(b, 64, axis=1)
    prod = s_full * codes.astype(np.float32)          # exact in fp32
    return (prod + b_full).astype(np.float32)          # one fp32 rounding


class QuantMatrix:
    """A quantised matrix with its dequantised form cached on first use.

    ``dtype`` float64 (the default) evaluates the GEMV in float64.  float32 keeps
    the dense weights in fp32 (they are exact fp32 values either way) and forms
    the product with fp32 BLAS and fp32 accumulation, x rounded to fp32: the
    exception the oracle allows for the stack-sized matrices, where it halves
    the memory of the cached weights at a relative error of about 1e-6.
    """

    def __init__(self, w: dict, dtype=np.float64):
        self.w = w
        self.dtype = np.dtype(dtype)
        assert self.dtype in (np.float64, np.float32)
        self._dense = None

    @property
    def shape(self):
        return np.asarray(self.w["codes"]).shape

    def dense(self) -> np.ndarray:
        if self._dense is None:
            self._dense = dequant(self.w).astype(self.dtype)
        return self._dense

    def __matmul__(self, x: np.ndarray) -> np.ndarray:
        """y = W x (the weight trait's plain GEMV), returned as float64."""
        return (self.dense() @ np.asarray(x, dtype=self.dtype)).astype(np.float64)


def as_qm(w) -> QuantMatrix:
    return w if isinstance(w, QuantMatrix) else QuantMatrix(w)


def stored(x, mode: str):
    """A buffer the pages keep in bf16: unchanged in Mode A (the parity
    authority, intermediates unrounded), rounded to bf16 in Mode B (diagnostic:
    the residual stream, the smoothed qkv and every GEMV output are rounded where
    the pages store them as bf16)."""
    if mode == "A":
        return np.asarray(x, dtype=np.float64)
    if mode == "B":
        return bf16_to_f64(f64_to_bf16(np.asarray(x, dtype=np.float64)))
    raise ValueError(f"mode {mode!r} (A or B)")


# --------------------------------------------------------------------------- elementwise / norms


def rms_norm(x: np.ndarray, w_bf16: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm of the last axis with a bf16 weight vector.

    Follows the ``rms_norm`` kernel the pages launch with ``(n, eps, x, w, out)``
    for the input, post-attention, per-head q/k and GDN output norms.  Reading:
    ``x * w / sqrt(mean(x^2) + eps)`` with the weight used as stored (no ``1+w``
    offset), ``eps = rms_eps``.
    """
    x = np.asarray(x, dtype=np.float64)
    w = bf16_to_f64(w_bf16)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * w


def l2_norm(x: np.ndarray, eps: float) -> np.ndarray:
    """Per-row L2 normalisation used on the GDN Q and K heads.

    Reading of the ``l2_eps`` argument of ``causal_conv1d_update_l2norm``:
    ``x / sqrt(sum(x^2) + eps)``.
    """
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def sigmoid(x):
    x = np.asarray(x, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-x))


def silu(x):
    x = np.asarray(x, dtype=np.float64)
    return x * sigmoid(x)


def softplus(x):
    """log(1 + e^x); identity above 20 (reading: the usual threshold)."""
    x = np.asarray(x, dtype=np.float64)
    return np.where(x > 20.0, x, np.log1p(np.exp(np.minimum(x, 20.0))))


# --------------------------------------------------------------------------- GDN pieces


def conv_update_silu(conv_state: np.ndarray, x: np.ndarray, w_bf16: np.ndarray):
    """One decode step of the causal depthwise conv, then SiLU, per channel.

    ``LinearAttentionState.conv1d_state`` is fp32 ``[channels, K]`` and the conv
    weight bf16 ``[channels, K]`` (``mod.rs``).  Reading: the state keeps the last
    K raw inputs of each channel with the newest in slot K-1; a step shifts the
    state left by one, puts the new input in slot K-1, and the output is the
    dot product of that window with the channel's K taps (no bias), then SiLU.

    Returns (new fp32 state, float64 outputs).
    """
    st = np.asarray(conv_state, dtype=np.float32).astype(np.float64)
    x = np.asarray(x, dtype=np.float64)
    w = bf16_to_f64(w_bf16)
    window = np.concatenate([st[:, 1:], x[:, None]], axis=1)
    u = np.sum(window * w, axis=1)
    new_state = window.astype(np.float32)   # the state is stored in fp32
    return new_state, silu(u)


def gdn_gate(a: np.ndarray, dt_bias_bf16: np.ndarray, a_log_f32: np.ndarray) -> np.ndarray:
    """Decay gate per v-head: exp(-exp(A_log) * softplus(a + dt_bias)), stored fp32.

    From the comment before the ``gdn_compute_gate`` launch of
    ``forward_linear_attention``; the gate buffer is fp32 ``[num_state_heads]``.
    """
    a = np.asarray(a, dtype=np.float64)
    A = np.asarray(a_log_f32, dtype=np.float32).astype(np.float64)
    g = np.exp(-np.exp(A) * softplus(a + bf16_to_f64(dt_bias_bf16)))
    return g.astype(np.float32)


def gdn_beta(b: np.ndarray) -> np.ndarray:
    """beta = sigmoid(b), stored fp32 (comment before the ``sigmoid_bf16_to_f32`` launch)."""
    return sigmoid(b).astype(np.float32)


def gated_delta_step(S: np.ndarray, q: np.ndarray, k: np.ndarray, v: np.ndarray,
                     g: float, beta: float):
    """One step of the gated delta rule for one head, state in [dk, dv] orientation.

    Reading of ``gated_delta_rule_decode``: the state first decays by the gate,
    then is corrected towards v along k with step size beta (the delta rule),
    and the read-out uses the corrected state; the 1/sqrt(dk) query scale is
    applied to the output (comment before the gate launch).

        S <- g * S
        delta = beta * (v - S^T k)
        S <- S + k delta^T
        y = S^T q / sqrt(dk)

    Returns (new state as fp32, y float64).
    """
    S = np.asarray(S, dtype=np.float32).astype(np.float64)
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = float(g)
    beta = float(beta)
    dk = S.shape[0]
    S = g * S
    delta = beta * (v - S.T @ k)
    S = S + np.outer(k, delta)
    y = (S.T @ q) / math.sqrt(dk)
    return S.astype(np.float32), y


# --------------------------------------------------------------------------- attention pieces


def rope_inv_freq(theta: float, rotary_dim: int) -> np.ndarray:
    """inv_freq[i] = theta^(-2i/R) for i < R/2, computed in float64, stored fp32.

    Reading: the caller-owned ``inv_freq`` buffer consumed by ``rope_apply`` holds
    the standard RoPE frequencies of ``rope_theta`` over the rotary width.
    """
    i = np.arange(rotary_dim // 2, dtype=np.float64)
    return (float(theta) ** (-2.0 * i / rotary_dim)).astype(np.float32)


def rope_partial(x: np.ndarray, pos: int, inv_freq_f32: np.ndarray, rotary_dim: int) -> np.ndarray:
    """Rotate the first ``rotary_dim`` entries of each head row; the rest pass through.

    From the ``rotary_dim`` field comment of ``Qwen35ForwardConfig`` and the two
    ``rope_apply`` launches of ``forward_full_attention``.  Reading: rotate-half
    pairing ``(i, i + R/2)``; the angle is the fp32 product ``pos * inv_freq[i]``
    (the kernel gets fp32 ``inv_freq`` and integer positions); sin and cos of
    that angle are taken in float64.
    """
    x = np.array(x, dtype=np.float64, copy=True)
    half = rotary_dim // 2
    ang = (np.float32(pos) * np.asarray(inv_freq_f32, dtype=np.float32)).astype(np.float64)
    c, s = np.cos(ang), np.sin(ang)
    x1 = x[..., :half].copy()
    x2 = x[..., half:rotary_dim].copy()
    x[..., :half] = x1 * c - x2 * s
    x[..., half:rotary_dim] = x2 * c + x1 * s
    return x


def attention_decode(q: np.ndarray, k_cache_bf16: np.ndarray, v_cache_bf16: np.ndarray,
                     seq_len: int) -> np.ndarray:
    """Single-query GQA softmax attention over cache rows [0, seq_len).

    ``attention_decode`` launch of ``forward_full_attention``: scale
    ``1/sqrt(head_dim)``, one query per q-head.  Reading: q-head h reads kv-head
    ``h // (Hq/Hkv)``; the cache is token-major ``[capacity, Hkv, D]``.

    q: [Hq, D] float64.  Returns [Hq, D] float64.
    """
    Hq, D = q.shape
    Hkv = k_cache_bf16.shape[1]
    rep = Hq // Hkv
    K = bf16_to_f64(k_cache_bf16[:seq_len])
    V = bf16_to_f64(v_cache_bf16[:seq_len])
    out = np.empty((Hq, D))
    for h in range(Hq):
        kvh = h // rep
        s = K[:, kvh, :] @ q[h] / math.sqrt(D)
        p = np.exp(s - s.max())
        p /= p.sum()
        out[h] = p @ V[:, kvh, :]
    return out


# --------------------------------------------------------------------------- layers


def mlp_residual(cfg, layer: dict, r: np.ndarray, mode: str = "A"):
    """Post-norm, SwiGLU MLP and residual: the tail shared by both layer forwards.

    ``add_rms_norm`` then ``gate_proj.gemv_gate_up_with(up_proj)`` then
    ``down_proj.gemv_silu_gate_resid``:
    x_out = r + W_down (silu(W_gate xn2) * (W_up xn2)),  xn2 = RMSNorm(r; post_ln).
    """
    xn2 = rms_norm(r, layer["post_ln"], cfg.rms_eps)
    ga = stored(as_qm(layer["gate_proj"]) @ xn2, mode)
    up = stored(as_qm(layer["up_proj"]) @ xn2, mode)
    h = silu(ga) * up
    x_out = r + stored(as_qm(layer["down_proj"]) @ h, mode)
    return stored(x_out, mode), {"x_norm2": xn2, "gate_act": ga, "up_act": up}


def forward_linear_attention(cfg, layer: dict, state: dict, x_in: np.ndarray, mode: str = "A"):
    """One token through one GDN layer (``forward_linear_attention``).

    state: {"conv1d_state": fp32 [C, K], "gdn_state": fp32 [Hv, dk, dv]}; a new
    dict is returned, the input is not modified.
    x_in: the residual stream in the activation dtype.
    mode: "A" (default, the parity authority) or "B" (bf16 at the buffers the
    pages store as bf16, see ``stored``).

    Returns (x_out float64, new_state, taps) where taps holds the named
    intermediates the page's dump hook exposes.
    """
    Hk, Hv = cfg.num_k_heads_lin, cfg.num_v_heads_lin
    dk, dv = cfg.k_head_dim_lin, cfg.v_head_dim_lin
    x = act_to_f64(x_in, cfg.act_dtype)

    xn = rms_norm(x, layer["input_ln"], cfg.rms_eps)
    a = stored(as_qm(layer["in_proj_a"]) @ xn, mode)
    b = stored(as_qm(layer["in_proj_b"]) @ xn, mode)
    qkv = stored(as_qm(layer["in_proj_qkv"]) @ xn, mode)
    z = stored(as_qm(layer["in_proj_z"]) @ xn, mode)

    conv_state, s = conv_update_silu(state["conv1d_state"], qkv, layer["conv1d_weight"])
    qk = 2 * Hk * dk
    s = s.copy()
    s[:qk] = l2_norm(s[:qk].reshape(2 * Hk, dk), 1e-6).reshape(-1)
    s = stored(s, mode)

    g = gdn_gate(a, layer["dt_bias"], layer["a_log"])
    beta = gdn_beta(b)

    q = s[:Hk * dk].reshape(Hk, dk)
    k = s[Hk * dk:qk].reshape(Hk, dk)
    v = s[qk:].reshape(Hv, dv)
    rep = Hv // Hk
    S_all = np.asarray(state["gdn_state"], dtype=np.float32)
    S_new = np.empty_like(S_all)
    y = np.empty((Hv, dv))
    for j in range(Hv):
        i = j // rep
        S_new[j], y[j] = gated_delta_step(S_all[j], q[i], k[i], v[j], g[j], beta[j])

    yn = rms_norm(y, layer["norm_weight"], cfg.rms_eps)
    out = stored(as_qm(layer["out_proj"]) @ (silu(z) * yn.reshape(-1)), mode)
    r = stored(x + out, mode)
    x_final, mt = mlp_residual(cfg, layer, r, mode)

    taps = {"gdn_x_norm": xn, "gdn_qkv_pre": qkv, "gdn_qkv_smooth": s, "gdn_y": y.reshape(-1),
            "gdn_y_norm": yn.reshape(-1), "gdn_out": out, "gdn_x_resid": r,
            "gdn_x_final": x_final, "dt_raw": a, "b_raw": b, "z": z, "gate": g, "beta": beta}
    taps.update(mt)
    return x_final, {"conv1d_state": conv_state, "gdn_state": S_new}, taps


def forward_full_attention(cfg, layer: dict, kv: dict, inv_freq: np.ndarray, x_in: np.ndarray,
                           cache_pos: int, seq_len_attn: int | None = None, mode: str = "A"):
    """One token through one gated full-attention layer (``forward_full_attention``).

    kv: {"k": bf16 [cap, Hkv, D], "v": bf16 [cap, Hkv, D]}; a new dict with row
    ``cache_pos`` written is returned, the input is not modified.
    mode: "A" (default) or "B" (bf16 at the pages' bf16 buffers, see ``stored``).
    Returns (x_out float64, new_kv, taps).
    """
    Hq, Hkv, D, R = cfg.num_heads, cfg.num_kv_heads, cfg.head_dim, cfg.rotary_dim
    if seq_len_attn is None:
        seq_len_attn = cache_pos + 1
    x = act_to_f64(x_in, cfg.act_dtype)

    xn = rms_norm(x, layer["input_ln"], cfg.rms_eps)
    q_full = stored(as_qm(layer["q_proj"]) @ xn, mode)
    k = stored(as_qm(layer["k_proj"]) @ xn, mode)
    v = stored(as_qm(layer["v_proj"]) @ xn, mode)

    # per head [Q_h | gate_h]  (q_total comment, qwen35_qkv_split launch)
    qh = q_full.reshape(Hq, 2 * D)
    q = qh[:, :D]
    gate = qh[:, D:]

    qn = rms_norm(q, layer["q_norm"], cfg.rms_eps)
    kn = rms_norm(k.reshape(Hkv, D), layer["k_norm"], cfg.rms_eps)
    qr = rope_partial(qn, cache_pos, inv_freq, R)
    kr = rope_partial(kn, cache_pos, inv_freq, R)

    kc = np.array(kv["k"], copy=True)
    vc = np.array(kv["v"], copy=True)
    kc[cache_pos] = f64_to_bf16(kr)
    vc[cache_pos] = f64_to_bf16(v.reshape(Hkv, D))

    attn = attention_decode(qr, kc, vc, seq_len_attn)
    ga = attn * sigmoid(gate)
    o = stored(as_qm(layer["o_proj"]) @ ga.reshape(-1), mode)
    r = stored(x + o, mode)
    x_out, mt = mlp_residual(cfg, layer, r, mode)

    taps = {"x_norm": xn, "q_full": q_full, "k": k, "v": v, "q_norm_out": qr.reshape(-1),
            "k_norm_out": kr.reshape(-1), "attn_out": attn.reshape(-1),
            "gated_attn": ga.reshape(-1), "o": o, "x_resid": r, "x_out": x_out}
    taps.update(mt)
    return x_out, {"k": kc, "v": vc}, taps


# --------------------------------------------------------------------------- stack tail


def lm_head_logits(cfg, final_norm_bf16: np.ndarray, lm_head, x: np.ndarray) -> np.ndarray:
    """Final RMSNorm then the quantised lm_head GEMV (caller-owned tail; reading:
    the standard decoder tail, since the pages leave it to the caller)."""
    h = rms_norm(np.asarray(x, dtype=np.float64), final_norm_bf16, cfg.rms_eps)
    return as_qm(lm_head) @ h


def greedy(logits: np.ndarray) -> int:
    """Index of the largest logit; the lowest index wins a tie."""
    return int(np.argmax(logits))


def decode_stack_step(cfg, kinds: list, layers: list, states: list, kvs: list,
                      inv_freq: np.ndarray, x_in: np.ndarray, cache_pos: int):
    """One token through a stack of layers (the caller's layer loop).

    The residual stream passed between layers is stored in the activation
    dtype, as the GDN forward's copy into the caller's buffer implies.
    Returns (x_out float64, new_states, new_kvs).
    """
    x = x_in
    new_states, new_kvs = list(states), list(kvs)
    x64 = act_to_f64(x, cfg.act_dtype)
    for li, kind in enumerate(kinds):
        if kind == "gdn":
            x64, new_states[li], _ = forward_linear_attention(cfg, layers[li], states[li], x)
        else:
            x64, new_kvs[li], _ = forward_full_attention(cfg, layers[li], kvs[li], inv_freq, x,
                                                         cache_pos)
        x = f64_to_act(x64, cfg.act_dtype)
    return x64, x, new_states, new_kvs
