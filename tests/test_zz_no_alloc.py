"""mk_build_schedule_static (the schedule build with its scratch in a fixed
device array, for callers that cannot allocate) against mk_build_schedule on
a workspace: every table bit for bit, on two calls in a row, the second with
a smaller input (the scratch keeps the first call's contents), and both
against the oracle's schedule."""
import numpy as np
import pytest
import torch

import workloads
from oracle import schedule
from tests.helpers import dev, say

pytestmark = pytest.mark.gpu

from mixture_experts_layer_device_amd import binding as B  # noqa: E402
from mixture_experts_layer_device_amd.layer import MoELayer  # noqa: E402


def _static_tables(re, R, E, MB, cap):
    nb = -(-R // MB) if R else 0
    z = lambda n: torch.full((max(n, 1),), -7, dtype=torch.int32, device="cuda")     # noqa: E731
    t = {"counts": z(E), "offsets": z(E + 1), "mb_counts": z(nb * E), "mb_offsets": z(nb * (E + 1)),
         "sorted_pos": z(R), "inv": z(nb * MB), "items": z(4 * cap), "mb_items": z(nb + 1), "err": z(1)}
    B.mk_build_schedule_static(re, R, E, MB, cap, t["counts"], t["offsets"], t["mb_counts"], t["mb_offsets"],
                               t["sorted_pos"], t["inv"], t["items"], t["mb_items"], t["err"],
                               torch.cuda.current_stream())
    return t


@pytest.mark.parametrize("E,MB", [(128, 4096), (8, 1000), (1024, 256)])
def test_static_schedule_matches_workspace_schedule(E, MB):
    rng = np.random.default_rng(E + MB)
    R1, R2 = 16384, 3001
    L = MoELayer(H=256, I=128, E=E, k=1, max_rows=R1, minibatch_rows=MB)
    cap = L.query("item_capacity")
    for R in (R1, R2):                       # the second call is smaller
        say(f"[no-alloc schedule] E={E} MB={MB} R={R}")
        re = rng.choice(E, size=R, p=workloads.zipf_local_weights(E, 1.2)).astype(np.int32)
        if R == R2:
            re[[5, 77]] = [-1, E]            # two ids out of range: flagged, rows dropped
        re_d = dev(re)
        st = _static_tables(re_d, R, E, MB, cap)
        L.build_schedule(re_d, R)
        torch.cuda.synchronize()
        nb = -(-R // MB)
        ref = schedule.build(re, E, MB, L.query("ring_rows"), L.query("tile_m"))
        n_items = len(ref.items)
        for name, n in (("counts", E), ("offsets", E + 1), ("mb_counts", nb * E), ("mb_offsets", nb * (E + 1)),
                        ("sorted_pos", R), ("inv", nb * MB), ("mb_items", nb + 1), ("items", 4 * n_items)):
            got = st[name][:n].cpu().numpy()
            want = L.table(name, n).cpu().numpy()
            assert np.array_equal(got, want), name
            assert np.array_equal(got, getattr(ref, name).reshape(-1)[:n]), name
        err = int(st["err"].cpu().item()) & 0xFFFFFFFF
        assert err == L.device_error()
        assert err == (B.MK_DEVERR_EXPERT_RANGE if R == R2 else 0)
    L.close()


def test_static_schedule_refuses_beyond_its_scratch():
    # nb * (c4 * E + c) * 4 bytes above 4 MiB (c = ceil(MB / 256) chunks, c4 = c rounded up to 4)
    with pytest.raises(B.MkError) as ei:
        B.mk_build_schedule_static(1, 1 << 20, 1024, 4096, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, None)
    assert ei.value.status == B.MK_ERR_LIMIT
