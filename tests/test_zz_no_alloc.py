"""GPU: gdn_layer_tail_noalloc (the library's static per-GPU scratch in place
of a workspace) against gdn_layer_tail with a caller's workspace, through the
C ABI: two calls in a row, the second with a smaller batch, on the
three-launch path that stages in the scratch, and on the single launch.
Both entry points run the same kernels, so the results must agree bitwise;
the oracle checks the first call too."""
import numpy as np
import pytest

import gdn_inputs as gi
import ref

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import gated_deltanet_decode_amd as g
    return g


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run(g, ti, M, params, noalloc):
    import torch
    B, C = ti["x"].shape
    t = {n: dev(x) for n, x in ti.items()}
    Md = dev(M)
    y = torch.empty((B, 4096), device="cuda")
    if noalloc:
        g.layer_tail_noalloc(t["x"], t["conv_w"], t["conv_state"], t["beta"], t["gate"], Md,
                             t["z"], t["norm_w"], y, params=params)
    else:
        ws = torch.empty(g.layer_tail_workspace_bytes(B), dtype=torch.uint8, device="cuda")
        g.layer_tail(t["x"], t["conv_w"], t["conv_state"], t["beta"], t["gate"], Md, t["z"],
                     t["norm_w"], y, workspace=ws, params=params)
    torch.cuda.synchronize()
    return dict(y=y.cpu().numpy(), state=Md.cpu().numpy(),
                conv_state=t["conv_state"].cpu().numpy())


@pytest.mark.parametrize("unfused", [1, 0])
def test_noalloc_tail_matches_workspace_tail(g, orc, unfused):
    params = g.TailParams(4, 128, 1e-6, unfused)
    for call, B in enumerate((32, 5)):
        print(f"\n  gdn_layer_tail_noalloc call {call + 1}: B={B} three launches={unfused}",
              flush=True)
        ti = gi.tail_inputs(6100 + B, B)
        M = gi.state(6100 + B, 0, B)
        got = run(g, ti, M, params, noalloc=True)
        want = run(g, ti, M, params, noalloc=False)
        for n in ("y", "state", "conv_state"):
            assert np.array_equal(got[n], want[n]), f"{n} differs from gdn_layer_tail (B={B})"
        if call == 0:
            cs = ti["conv_state"].copy()
            Mo = M.copy()
            y, _, _ = orc.layer_tail(ti["x"], ti["conv_w"], cs, ti["beta"], ti["gate"], Mo,
                                     ti["z"], ti["norm_w"], 16, 128)
            ref.assert_close("y", got["y"], y, 1e-5)
            ref.assert_close("state", got["state"], Mo, 1e-6)
            assert np.array_equal(got["conv_state"], cs), "conv cache not bitwise"


def test_noalloc_tail_refuses_staging_beyond_the_scratch(g):
    """B = 342 on the three-launch path needs more than the 16 MiB scratch:
    refused before anything is enqueued, buffers untouched."""
    import torch
    B = 342
    C = 8192
    x = torch.zeros((B, C), device="cuda")
    cw = torch.zeros((C, 4), device="cuda")
    cs = torch.full((B, 3, C), 2.0, device="cuda")
    bt = torch.zeros((B, 32), device="cuda")
    M = torch.full((B, 32, 128, 128), 3.0, device="cuda")
    z = torch.zeros((B, 4096), device="cuda")
    nw = torch.ones(128, device="cuda")
    y = torch.full((B, 4096), 5.0, device="cuda")
    with pytest.raises(g.GdnError) as e:
        g.layer_tail_noalloc(x, cw, cs, bt, bt, M, z, nw, y, params=g.TailParams(4, 128, 1e-6, 1))
    assert e.value.code == -5 and "static scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((cs == 2.0).all()) and bool((M == 3.0).all()) and bool((y == 5.0).all())
