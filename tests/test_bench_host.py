"""Host-side checks of bench.py (no GPU): the one-GPU contract."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_kernel_source_hash_is_stable():
    sys.path.insert(0, ROOT)
    import bench

    h = bench.kernel_source_hash()
    assert len(h) == 16 and h == bench.kernel_source_hash()


def test_tile_flops_of_the_work_list_equal_the_prefix_flops():
    """components.prefix_tiles_in_fused counts each MFMA tile's flops as
    4 d x rows x chunk tokens from the work list; without prefix limits and
    with every group at or above the MFMA threshold, their sum is the plan's
    algorithmic prefix flops (each prefix token of each row once)."""
    import numpy as np

    sys.path.insert(0, ROOT)
    import prefix_shared_decode_amd as P
    from workloads import make_workload

    for name in ("llama3_8b_8x100", "longchat13b_1x256"):
        wl = make_workload(name)
        cfg = P.make_config(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_pages, wl.dtype, "f32")
        plan = P.psa_build_plan(cfg, wl.batch)
        info = plan.info()
        it = np.asarray(plan.items()).reshape(int(info["num_items"]), 4, 8)
        tile = (it[:, 0, 0] & 0xFF) == 2
        flops = (4.0 * wl.head_dim * it[:, 0, 7] * (it[:, 0, 4] - it[:, 0, 3]))[tile].sum()
        assert tile.sum() == info["num_prefix_items"]
        assert flops == info["prefix_flops"]
