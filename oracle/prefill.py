"""CPU oracle for multi-token prefill of the two Qwen3.5 layer kinds.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The
product path never does, and this module imports nothing from it.

The pages document the decode step only; the overview of the ``qwen3_5``
module (rustdoc index, first paragraph) leaves the prompt pass to the caller.
Reading taken here: a prefill of T tokens into a layer is T decode steps in
token order, token t running at cache position ``cache_pos + t`` (its RoPE
position and its KV row) and attending to cache rows ``[0, cache_pos + t]``;
conv and GDN states are carried from one token to the next.  So the oracle is
that loop over the per-token functions of ``qwen35``, which are pinned
themselves; how a GPU groups the tokens (chunks of the delta rule, tiles of
the causal attention) changes only the rounding.  With a quantised KV cache
(the Turbo branches of the full_attention.rs page) the per-token function is
that format's forward in ``turbo8`` or ``turbo_lm``: every prompt token
appends its quantised row and attends to the rows as stored, the sparse-V
gate included.

Every function returns float64 per-token outputs and the updated state or
cache; nothing given to it is modified.
"""
from __future__ import annotations

import numpy as np

from . import qwen35 as Q
from . import turbo8 as T8
from . import turbo_lm as TL

_WEIGHTS = ("in_proj_a", "in_proj_b", "in_proj_qkv", "in_proj_z", "out_proj", "q_proj", "k_proj",
            "v_proj", "o_proj", "gate_proj", "up_proj", "down_proj")


def _dense_once(layer: dict) -> dict:
    """The layer with its quantised matrices wrapped once, so each is dequantised
    a single time for the whole token loop (values unchanged)."""
    out = dict(layer)
    for name in _WEIGHTS:
        if name in out:
            out[name] = Q.as_qm(out[name])
    return out


def prefill_linear_attention(cfg, layer: dict, state: dict, x_in: np.ndarray, taps=()):
    """T tokens through one GDN layer (``forward_linear_attention`` per token).

    x_in: [T, hidden] in the activation dtype.  Returns (x_out float64
    [T, hidden], new_state, {name: [T, ...]} for each name in ``taps``).
    """
    lay = _dense_once(layer)
    T = x_in.shape[0]
    out = np.empty((T, cfg.hidden))
    got = {n: [] for n in taps}
    st = state
    for t in range(T):
        out[t], st, tp = Q.forward_linear_attention(cfg, lay, st, x_in[t])
        for n in taps:
            got[n].append(np.asarray(tp[n]))
    return out, st, {n: np.stack(v) for n, v in got.items()}


def _full_step(fmt: str, sparse_v: float):
    """The per-token full-attention forward for a KV cache format."""
    if fmt == "bf16":
        return Q.forward_full_attention
    if fmt == "turbo8":
        return lambda cfg, lay, kv, inv, x, pos: T8.forward_full_attention_turbo8(cfg, lay, kv, inv, x, pos,
                                                                                  sparse_v=sparse_v)
    if fmt in TL.FORMATS:
        return lambda cfg, lay, kv, inv, x, pos: TL.forward_full_attention(fmt, cfg, lay, kv, inv, x, pos,
                                                                           sparse_v=sparse_v)
    raise ValueError(f"unknown KV cache format {fmt!r}")


def prefill_full_attention(cfg, layer: dict, kv: dict, inv_freq: np.ndarray, x_in: np.ndarray,
                           cache_pos: int, taps=(), fmt: str = "bf16",
                           sparse_v: float = T8.SPARSE_V_DEFAULT):
    """T tokens through one gated full-attention layer (``forward_full_attention``
    per token, or the Turbo branch of ``fmt``'s cache with the sparse-V
    threshold ``sparse_v``), token t at cache position ``cache_pos + t`` with
    ``seq_len_attn = cache_pos + t + 1``.

    Returns (x_out float64 [T, hidden], new_kv, {name: [T, ...]}).
    """
    lay = _dense_once(layer)
    step = _full_step(fmt, sparse_v)
    T = x_in.shape[0]
    out = np.empty((T, cfg.hidden))
    got = {n: [] for n in taps}
    cur = kv
    for t in range(T):
        out[t], cur, tp = step(cfg, lay, cur, inv_freq, x_in[t], cache_pos + t)
        for n in taps:
            got[n].append(np.asarray(tp[n]))
    new = dict(kv)
    new.update(cur)
    return out, new, {n: np.stack(v) for n, v in got.items()}
