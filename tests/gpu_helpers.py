"""Helpers shared by the GPU tests (not collected: no test_ prefix).

The HIP path runs through the C ABI (prefix_shared_decode_amd); the expected
values always come from the fp64 oracle on host copies of the same inputs.
"""

from __future__ import annotations

import math

import numpy as np

import oracle
import prefix_shared_decode_amd as P
from workloads import make_values

# parity tolerances (bf16 inputs; fp32 inputs), over the whole output tensor
TOL = {"bf16": {"max_abs": 1e-2, "rel_l2": 5e-3}, "f32": {"max_abs": 1e-5, "rel_l2": 1e-5}}


def log(msg):
    print(msg, flush=True)


def to_host64(t):
    return t.float().cpu().numpy().astype(np.float64)


def cfg_for(wl, out_dtype="f32", sm_scale=0.0):
    return P.make_config(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_pages, wl.dtype, out_dtype,
                         sm_scale=sm_scale)


def values(wl, seed=None):
    return make_values(wl, "cuda", seed)


def run(wl, batch, q, k, v, out_dtype="f32", want_ml=True, sm_scale=0.0, **plan_kw):
    import torch

    step = P.DecodeStep(cfg_for(wl, out_dtype, sm_scale), batch, **plan_kw)
    n = len(batch["query_group"])
    ot = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    out = torch.full((n, wl.num_q_heads, wl.head_dim), float("nan"), dtype=ot, device="cuda")
    m = torch.full((n, wl.num_q_heads), float("nan"), dtype=torch.float32, device="cuda") if want_ml else None
    l = torch.full((n, wl.num_q_heads), float("nan"), dtype=torch.float32, device="cuda") if want_ml else None
    step(q, k, v, out, m, l)
    torch.cuda.synchronize()
    return step, out, m, l


def oracle_all(wl, batch, q, k, v, sm_scale=None):
    return oracle.decode_attention(to_host64(q), to_host64(k), to_host64(v), batch, scale=sm_scale)


def errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = got - ref
    return float(np.abs(d).max()) if d.size else 0.0, float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300))


def assert_close(got, ref, dtype, what=""):
    mx, rel = errors(got, ref)
    tol = TOL[dtype]
    log(f"  {what}: max_abs={mx:.3e} rel_l2={rel:.3e} (tol {tol['max_abs']:.0e}/{tol['rel_l2']:.0e})")
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert mx <= tol["max_abs"] and rel <= tol["rel_l2"], f"{what}: max_abs={mx} rel_l2={rel}"


def assert_lse_close(m, l, M, L, tol):
    """Compare log-sum-exp m + ln l (the statistics' one scale-free combination)."""
    got = to_host64(m) + np.log(to_host64(l))
    ref = M + np.log(L)
    err = float(np.abs(got - ref).max())
    log(f"  lse max err {err:.3e}")
    assert err <= tol


def scale_default(d):
    return 1.0 / math.sqrt(d)
