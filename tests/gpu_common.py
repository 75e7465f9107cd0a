"""Shared helpers for the GPU parity tests (imported only by tests)."""
import numpy as np

import oracle as O

# Tolerances (relative L2 error per compared tensor):
TOL_BF16 = 2e-2    # bf16 activations
TOL_F32 = 1e-3     # fp32 activations (tiny config) and the fp32 GDN state after 64 steps
TOL_GEMV = 2e-5    # one fp32 GEMV against float64
# one GEMV whose x is rounded to f16 (11 significant bits) before exact products:
# the error is that rounding, ~2^-12 relative per element, averaged over the dot
TOL_GEMV_F16 = 1e-3


def rel(gpu, ref) -> float:
    gpu = np.asarray(gpu, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(gpu - ref) / (den if den > 0 else 1.0))


def say(msg: str) -> None:
    print(msg, flush=True)


def act_in(cfg, gen, name):
    """A per-step layer input in the activation dtype."""
    return gen.act(name, (cfg.hidden,), cfg.act_dtype)


def oracle_act(x, cfg):
    return O.act_to_f64(x, cfg.act_dtype)
