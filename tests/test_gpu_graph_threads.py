"""GPU: every entry point can be captured into a HIP graph (through torch's
graph capture) and replayed, and may be called from several host threads on
their own streams at once; results are bitwise those of eager calls."""
import threading

import numpy as np
import pytest

import gdn_inputs as gi

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


def _replay_matches_eager(make_call, state_names, outs):
    """make_call(bufs) launches one call on the current stream.  Capture it on
    copies, then alternate graph replays with eager calls on other copies and
    compare every replay bit for bit."""
    import torch
    eager = {n: t.clone() for n, t in state_names.items()}
    graph = {n: t.clone() for n, t in state_names.items()}
    outs_e = {n: torch.empty_like(t) for n, t in outs.items()}
    outs_g = {n: torch.empty_like(t) for n, t in outs.items()}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr, stream=side):
        make_call(graph, outs_g)
    torch.cuda.synchronize()
    for rep in range(3):
        gr.replay()
        make_call(eager, outs_e)
        torch.cuda.synchronize()
        for n in state_names:
            assert torch.equal(graph[n], eager[n]), f"replay {rep}: {n} differs"
        for n in outs:
            assert torch.equal(outs_g[n], outs_e[n]), f"replay {rep}: {n} differs"


def test_graph_capture_step_seq_pair_tail(g):
    import torch
    print("\n  graph capture: step, seq, pair, tail", flush=True)
    B = 4
    si = {n: dev(x) for n, x in gi.step_inputs(6000, 0, B).items()}
    M = dev(gi.state(6000, 0, B))
    _replay_matches_eager(
        lambda st, o: g.step(si["q"], si["k"], si["v"], si["beta"], si["gate"], st["M"], o["out"]),
        {"M": M}, {"out": torch.empty((B, 32, 128), device="cuda")})

    ss = {n: dev(x) for n, x in gi.step_inputs(6001, 0, B, T=21).items()}
    _replay_matches_eager(
        lambda st, o: g.seq(ss["q"], ss["k"], ss["v"], ss["beta"], ss["gate"], st["M"], o["out"]),
        {"M": M}, {"out": torch.empty((B, 21, 32, 128), device="cuda")})

    sp = {n: dev(x) for n, x in gi.step_inputs(6002, 0, B, T=2).items()}
    _replay_matches_eager(
        lambda st, o: g.pair(sp["q"], sp["k"], sp["v"], sp["beta"], sp["gate"], st["M"],
                             o["next"], o["out"]),
        {"M": M}, {"out": torch.empty((B, 2, 32, 128), device="cuda"),
                   "next": torch.empty_like(M)})

    ti = {n: dev(x) for n, x in gi.tail_inputs(6003, B).items()}
    ws = torch.empty(g.layer_tail_workspace_bytes(B), dtype=torch.uint8, device="cuda")
    for fu in (0, 1):
        p = g.TailParams(4, 128, 1e-6, fu)
        _replay_matches_eager(
            lambda st, o: g.layer_tail(ti["x"], ti["conv_w"], st["cs"], ti["beta"], ti["gate"],
                                       st["M"], ti["z"], ti["norm_w"], o["y"], workspace=ws,
                                       params=p),
            {"M": M, "cs": ti["conv_state"]}, {"y": torch.empty((B, 4096), device="cuda")})


def test_graph_capture_large_launch_shapes(g):
    """The launch shapes that only large calls take: gdn_seq with more half
    heads than fit two per CU (the 16-token kernel held to three workgroups
    per CU, which spills a few registers to scratch) and gdn_step's staged
    kernel (two tiles per workgroup through LDS)."""
    import torch
    print("\n  graph capture: seq B=24 T=20, step B=300 (staged)", flush=True)
    B = 24
    ss = {n: dev(x) for n, x in gi.step_inputs(6004, 0, B, T=20).items()}
    M = dev(gi.state(6004, 0, B))
    _replay_matches_eager(
        lambda st, o: g.seq(ss["q"], ss["k"], ss["v"], ss["beta"], ss["gate"], st["M"], o["out"]),
        {"M": M}, {"out": torch.empty((B, 20, 32, 128), device="cuda")})
    del M
    B = 300                                   # 300 x 32 x 16 = 153,600 tiles
    si = {n: dev(x) for n, x in gi.step_inputs(6005, 0, B).items()}
    M = dev(gi.state(6005, 0, B))
    _replay_matches_eager(
        lambda st, o: g.step(si["q"], si["k"], si["v"], si["beta"], si["gate"], st["M"], o["out"]),
        {"M": M}, {"out": torch.empty((B, 32, 128), device="cuda")})


def test_graph_capture_gate_transform_and_tail_ba(g):
    import torch
    print("\n  graph capture: gate transform, tail from raw gates", flush=True)
    B = 4
    gin = {n: dev(x) for n, x in gi.gate_inputs(6004, B).items()}
    _replay_matches_eager(
        lambda st, o: g.gate_transform(gin["ba"], gin["a_log"], gin["dt_bias"], o["beta"],
                                       o["gate"]),
        {}, {"beta": torch.empty((B, 32), device="cuda"),
             "gate": torch.empty((B, 32), device="cuda")})
    ti = {n: dev(x) for n, x in gi.tail_inputs(6004, B).items()}
    M = dev(gi.state(6004, 0, B))
    ws = torch.empty(g.layer_tail_ba_workspace_bytes(B), dtype=torch.uint8, device="cuda")
    for fu in (0, 1):
        p = g.TailParams(4, 128, 1e-6, fu)
        _replay_matches_eager(
            lambda st, o: g.layer_tail_ba(ti["x"], ti["conv_w"], st["cs"], gin["ba"],
                                          gin["a_log"], gin["dt_bias"], st["M"], ti["z"],
                                          ti["norm_w"], o["y"], workspace=ws, params=p),
            {"M": M, "cs": ti["conv_state"]}, {"y": torch.empty((B, 4096), device="cuda")})


def test_graph_capture_cached_step_tail_pair_noalloc(g):
    """gdn_step_ex with GDN_STATE_CACHED (one wave per tile at B = 1, the
    one-shot cached layout at B = 64), gdn_layer_tail_pair, and
    gdn_layer_tail_noalloc on both launch paths (after one call outside the
    capture, which looks up the static scratch's address)."""
    import torch
    print("\n  graph capture: cached step, tail pair, no-alloc tail", flush=True)
    for B in (1, 64):
        si = {n: dev(x) for n, x in gi.step_inputs(6010 + B, 0, B).items()}
        M = dev(gi.state(6010 + B, 0, B))
        _replay_matches_eager(
            lambda st, o: g.step(si["q"], si["k"], si["v"], si["beta"], si["gate"], st["M"],
                                 o["out"], cached=True),
            {"M": M}, {"out": torch.empty((B, 32, 128), device="cuda")})
        del M
    B = 4
    t1 = {n: dev(x) for n, x in gi.tail_inputs(6020, B, slot=0).items()}
    t2 = {n: dev(x) for n, x in gi.tail_inputs(6020, B, slot=1).items()}
    pr = {n: torch.stack([t1[n], t2[n]], dim=1).contiguous() for n in ("x", "beta", "gate", "z")}
    M = dev(gi.state(6020, 0, B))
    _replay_matches_eager(
        lambda st, o: g.layer_tail_pair(pr["x"], t1["conv_w"], st["cs"], o["csn"], pr["beta"],
                                        pr["gate"], st["M"], o["Mn"], pr["z"], t1["norm_w"],
                                        o["y"]),
        {"M": M, "cs": t1["conv_state"]},
        {"y": torch.empty((B, 2, 4096), device="cuda"), "Mn": torch.empty_like(M),
         "csn": torch.empty_like(t1["conv_state"])})
    for fu in (0, 1):
        p = g.TailParams(4, 128, 1e-6, fu)
        warm = (M.clone(), t1["conv_state"].clone(), torch.empty((B, 4096), device="cuda"))
        g.layer_tail_noalloc(t1["x"], t1["conv_w"], warm[1], t1["beta"], t1["gate"], warm[0],
                             t1["z"], t1["norm_w"], warm[2], params=p)
        torch.cuda.synchronize()
        _replay_matches_eager(
            lambda st, o: g.layer_tail_noalloc(t1["x"], t1["conv_w"], st["cs"], t1["beta"],
                                               t1["gate"], st["M"], t1["z"], t1["norm_w"],
                                               o["y"], params=p),
            {"M": M, "cs": t1["conv_state"]}, {"y": torch.empty((B, 4096), device="cuda")})


def test_concurrent_host_threads(g):
    """Four host threads, each on its own stream and buffers, call gdn_step
    and gdn_seq repeatedly at the same time."""
    import torch
    print("\n  concurrent host threads", flush=True)
    n_threads, reps, B = 4, 12, 3
    cases = []
    for i in range(n_threads):
        si = {n: dev(x) for n, x in gi.step_inputs(6100 + i, 0, B).items()}
        ss = {n: dev(x) for n, x in gi.step_inputs(6200 + i, 0, B, T=9).items()}
        M = dev(gi.state(6100 + i, 0, B))
        cases.append((si, ss, M))

    def work(i, M, out, out_s, stream):
        si, ss, _ = cases[i]
        with torch.cuda.stream(stream):
            for _ in range(reps):
                g.step(si["q"], si["k"], si["v"], si["beta"], si["gate"], M, out)
                g.seq(ss["q"], ss["k"], ss["v"], ss["beta"], ss["gate"], M, out_s)

    serial = []
    for i in range(n_threads):
        M = cases[i][2].clone()
        out = torch.empty((B, 32, 128), device="cuda")
        out_s = torch.empty((B, 9, 32, 128), device="cuda")
        work(i, M, out, out_s, torch.cuda.current_stream())
        serial.append((M, out, out_s))
    torch.cuda.synchronize()

    res, errors = [], []
    streams = [torch.cuda.Stream() for _ in range(n_threads)]
    for i in range(n_threads):
        res.append((cases[i][2].clone(), torch.empty((B, 32, 128), device="cuda"),
                    torch.empty((B, 9, 32, 128), device="cuda")))
    torch.cuda.synchronize()

    def run(i):
        try:
            work(i, *res[i], streams[i])
        except Exception as e:  # report in the main thread
            errors.append(e)
    ths = [threading.Thread(target=run, args=(i,)) for i in range(n_threads)]
    for t in ths:
        t.start()
    for t in ths:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(n_threads):
        for a, b in zip(res[i], serial[i]):
            assert torch.equal(a, b), f"thread {i} differs from the serial run"
