"""The synthetic workloads, built from named seeded draws (no decode arithmetic).

* ``tiny_stack``      two-layer hybrid (GDN then full attention), fp32 activations,
                      hidden 256, zero states, 16 decode tokens from N(0,1) inputs;
* ``gdn_layer_4b``    one GDN layer at the 4B dims, bf16 activations, GDN state
                      N(0, 0.1), conv state N(0, 1), 256 single-token steps;
* ``full_layer_4b``   one full-attention layer at the 4B dims, bf16 KV cache with
                      rows [0, 4096) prefilled N(0, 1), 64 steps from position 4096;
* ``full_layer_4b_turbo8``  the same layer over a Turbo8 cache whose rows
                      [0, 4096) hold uniformly drawn finite E4M3 codes and bf16
                      scales U(1e-3, 1e-2);
* ``full_layer_4b_lm``  the same layer over a Lloyd-Max format cache (uniformly
                      drawn indices and E4M3 scales; bf16 keys N(0, 1) for the
                      asymmetric formats);
* ``stack_4b``        the 4B-shaped stack (every 4th layer full attention), int8
                      lm_head over the 248 320-token vocabulary, bf16 embedding table
                      N(0, 1), zero GDN states, KV rows [0, ctx) prefilled N(0, 1)
                      (bf16) or with uniformly drawn codes and scales (Turbo8).
"""
from __future__ import annotations

from . import (LM_FORMATS, Gen, gdn_layer, full_layer, gdn_state, kv_cache, kv_cache_lm,
               kv_cache_turbo8, layer_kinds, qwen3_5_4b, tiny)


def tiny_stack(gen: Gen, steps: int = 16, capacity: int = 16):
    cfg = tiny("f32")
    kinds = layer_kinds(2)
    layers = [gdn_layer(gen, cfg, "tiny.L0"), full_layer(gen, cfg, "tiny.L1")]
    states = [gdn_state(gen, cfg, "tiny.L0"), None]
    kvs = [None, kv_cache(gen, cfg, "tiny.L1", capacity, 0)]
    xs = [gen.act(f"tiny.x{t}", (cfg.hidden,), cfg.act_dtype) for t in range(steps)]
    return {"cfg": cfg, "kinds": kinds, "layers": layers, "states": states, "kvs": kvs, "xs": xs}


def gdn_layer_4b(gen: Gen, steps: int = 256):
    cfg = qwen3_5_4b("bf16")
    layer = gdn_layer(gen, cfg, "c2.L")
    state = gdn_state(gen, cfg, "c2.L", gdn_std=0.1, conv_std=1.0)
    xs = [gen.act(f"c2.x{t}", (cfg.hidden,), cfg.act_dtype) for t in range(steps)]
    return {"cfg": cfg, "layer": layer, "state": state, "xs": xs}


def full_layer_4b(gen: Gen, steps: int = 64, prefill: int = 4096):
    cfg = qwen3_5_4b("bf16")
    layer = full_layer(gen, cfg, "c3.L")
    kv = kv_cache(gen, cfg, "c3.L", prefill + steps, prefill)
    xs = [gen.act(f"c3.x{t}", (cfg.hidden,), cfg.act_dtype) for t in range(steps)]
    return {"cfg": cfg, "layer": layer, "kv": kv, "xs": xs, "start": prefill}


def full_layer_4b_turbo8(gen: Gen, steps: int = 12, prefill: int = 4096):
    cfg = qwen3_5_4b("bf16")
    layer = full_layer(gen, cfg, "c3t8.L")
    kv = kv_cache_turbo8(gen, cfg, "c3t8.L", prefill + steps, prefill)
    xs = [gen.act(f"c3t8.x{t}", (cfg.hidden,), cfg.act_dtype) for t in range(steps)]
    return {"cfg": cfg, "layer": layer, "kv": kv, "xs": xs, "start": prefill}


def full_layer_4b_lm(gen: Gen, fmt: str, steps: int = 12, prefill: int = 4096):
    """The 4B full-attention layer over a Lloyd-Max format cache (``kv_cache_lm``)."""
    cfg = qwen3_5_4b("bf16")
    layer = full_layer(gen, cfg, f"c3{fmt}.L")
    kv = kv_cache_lm(gen, cfg, f"c3{fmt}.L", prefill + steps, prefill, fmt)
    xs = [gen.act(f"c3{fmt}.x{t}", (cfg.hidden,), cfg.act_dtype) for t in range(steps)]
    return {"cfg": cfg, "layer": layer, "kv": kv, "xs": xs, "start": prefill}


def stack_4b(gen: Gen, num_layers: int = 32, ctx: int = 8192, extra: int = 256, progress=None,
             kv: str = "bf16"):
    """The 4B-shaped stack.  ``capacity = ctx + extra`` tokens per KV cache; ``kv``
    "bf16" (rows N(0, 1)), "turbo8" (rows of uniformly drawn finite E4M3 codes
    and bf16 scales U(1e-3, 1e-2)) or a Lloyd-Max format (``kv_cache_lm``)."""
    cfg = qwen3_5_4b("bf16")
    kinds = layer_kinds(num_layers)
    layers, states, kvs = [], [], []
    for i, kind in enumerate(kinds):
        if kind == "gdn":
            layers.append(gdn_layer(gen, cfg, f"c4.L{i}"))
            states.append(gdn_state(gen, cfg, f"c4.L{i}"))
            kvs.append(None)
        else:
            layers.append(full_layer(gen, cfg, f"c4.L{i}"))
            states.append(None)
            if kv in LM_FORMATS:
                kvs.append(kv_cache_lm(gen, cfg, f"c4.L{i}", ctx + extra, ctx, kv))
            else:
                make = {"bf16": kv_cache, "turbo8": kv_cache_turbo8}[kv]
                kvs.append(make(gen, cfg, f"c4.L{i}", ctx + extra, ctx))
        if progress:
            progress(i)
    embed = gen.normal_bf16("c4.embed", (cfg.vocab, cfg.hidden))
    final_norm = gen.norm_weight("c4.final_norm", cfg.hidden)
    lm_head = gen.quant("c4.lm_head", cfg.vocab, cfg.hidden)
    start_token = int(gen.uniform_f32("c4.t0", (1,), 0.0, float(cfg.vocab))[0])
    return {"cfg": cfg, "kinds": kinds, "layers": layers, "states": states, "kvs": kvs,
            "embed": embed, "final_norm": final_norm, "lm_head": lm_head, "ctx": ctx,
            "start_token": start_token}
