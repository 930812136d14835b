"""psa_decode_attention_noalloc: the entry point that allocates nothing.

It runs the kernels of psa_decode_attention with their scratch (merge
counters and fp32 partials) in the library's static device array, given only
the uploaded plan image.  Its output must equal psa_decode_attention's bit
for bit (same kernels, same deterministic merge order) and the oracle's
within the bf16 tolerance, on consecutive calls that share the array (the
second with a smaller batch), and again after that.
"""

import numpy as np
import pytest

import prefix_shared_decode_amd as P
from workloads import build_single_level

from gpu_helpers import assert_close, assert_lse_close, log, oracle_all, to_host64, values


def test_scratch_limit_is_checked_before_any_device_call():
    """A plan whose counters and partials exceed the 64 MiB array is refused
    (host-side check, no GPU needed); so is an image buffer smaller than the
    plan image."""
    import ctypes as C

    wl = build_single_level("noalloc_big", 32, 8, 128, "bf16", [], [1024] * 64, seed=1)
    cfg = P.make_config(32, 8, 128, wl.num_pages, "bf16")
    plan = P.psa_build_plan(cfg, wl.batch, distinct_chunk_tokens=16)
    info = plan.info()
    assert info["workspace_bytes"] - info["image_bytes"] > 64 << 20
    L = P.lib()
    host = (C.c_uint8 * 64)()
    st = L.psa_decode_attention_noalloc(plan.handle, C.addressof(host), C.addressof(host), C.addressof(host),
                                        C.addressof(host), None, None, C.addressof(host), info["image_bytes"], None)
    assert P._lib.STATUS[st] == "PSA_ERR_WORKSPACE_TOO_SMALL"
    assert b"static array" in L.psa_last_error()
    small = P.psa_build_plan(cfg, build_single_level("noalloc_s", 32, 8, 128, "bf16", [], [40], seed=1).batch)
    st = L.psa_decode_attention_noalloc(small.handle, C.addressof(host), C.addressof(host), C.addressof(host),
                                        C.addressof(host), None, None, C.addressof(host),
                                        small.info()["image_bytes"] - 1, None)
    assert P._lib.STATUS[st] == "PSA_ERR_WORKSPACE_TOO_SMALL"


@pytest.mark.gpu
def test_noalloc_equals_workspace_entry_point():
    import torch

    big = build_single_level("noalloc_1", 32, 8, 128, "bf16", [(400, 30, (0, 300)), (90, 7, (1, 60))],
                             (6, (1, 900)), seed=31)
    small = build_single_level("noalloc_2", 32, 8, 128, "bf16", [(150, 5, (1, 40))], (2, (1, 100)), seed=32)
    # call 1: small chunks (many partials, merges by the last arriver and in registers);
    # call 2: a smaller batch with default chunks; call 3: the first plan again
    cases = [(big, dict(prefix_chunk_tokens=128, distinct_chunk_tokens=64, mfma_tile_rows=32)), (small, {}),
             (big, dict(prefix_chunk_tokens=128, distinct_chunk_tokens=64, mfma_tile_rows=32))]
    for call, (wl, opts) in enumerate(cases):
        log(f"case noalloc call {call + 1}: {wl.name} {opts}")
        q, k, v = values(wl)
        cfg = P.make_config(32, 8, 128, wl.num_pages, "bf16")
        plan = P.psa_build_plan(cfg, wl.batch, **opts)
        info = plan.info()
        n = len(wl.batch["query_group"])
        shape, mshape = (n, 32, 128), (n, 32)
        ws = torch.empty(info["workspace_bytes"], dtype=torch.uint8, device="cuda")
        P.psa_plan_upload(plan, ws)
        ref = torch.full(shape, float("nan"), device="cuda")
        mref = torch.full(mshape, float("nan"), device="cuda")
        lref = torch.full(mshape, float("nan"), device="cuda")
        P.psa_decode_attention(plan, q, k, v, ref, ws, mref, lref)
        image = torch.empty(info["image_bytes"], dtype=torch.uint8, device="cuda")  # the image only
        P.psa_plan_upload(plan, image)
        with pytest.raises(P.PsaError):  # too small for the workspace entry point
            P.psa_decode_attention(plan, q, k, v, ref.clone(), image)
        for rep in range(2):
            out = torch.full(shape, float("nan"), device="cuda")
            m = torch.full(mshape, float("nan"), device="cuda")
            l = torch.full(mshape, float("nan"), device="cuda")
            P.psa_decode_attention_noalloc(plan, q, k, v, out, image, m, l)
            torch.cuda.synchronize()
            assert torch.equal(out, ref) and torch.equal(m, mref) and torch.equal(l, lref), (call, rep)
        O, M, L = oracle_all(wl, wl.batch, q, k, v)
        assert_close(to_host64(out), O, "bf16", f"noalloc call {call + 1}")
        assert_lse_close(m, l, M, L, 2e-4)
        assert np.isfinite(to_host64(out)).all()
