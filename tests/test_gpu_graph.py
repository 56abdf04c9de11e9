"""The fused decode step of several layers captured as a HIP graph, as a
serving loop may run it: every replay, with eager library calls and torch
work run between replays, gives the eager step's outputs and cache bit for
bit and leaves the workspace zero (the library records no memset; its calls
return the workspace to zero themselves)."""

import numpy as np
import pytest

import workloads as wl
from kvq_testlib import bf16_dev, dev_tensor, kv_dev, log, to_host_bits

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("D,H,KVH,recent", [(128, 32, 8, 0), (96, 8, 2, 0), (128, 16, 4, 64), (256, 16, 4, 0)])
def test_graph_replays_equal_eager(kvq, D, H, KVH, recent):
    import torch
    B, T, layers = 3, 1500, 3
    log(f"graph: D={D} H={H} KVH={KVH} recent={recent}")
    s = torch.cuda.Stream()
    rng = np.random.default_rng(D + H + recent)
    lays = []
    for _ in range(layers):
        x = wl.random_kv(int(rng.integers(1 << 30)), (B, KVH, T, D), "bf16")
        qb, _ = wl.random_q(int(rng.integers(1 << 30)), (B, H, D))
        c = kvq.Int8KVCache(B, H, KVH, D, max_len=T, fill=0, recent_window=recent)
        c.append(kv_dev(np.ascontiguousarray(x["k_raw"][:, :, :T - 1])),
                 kv_dev(np.ascontiguousarray(x["v_raw"][:, :, :T - 1])), dev_tensor(np.zeros(B, np.int32)))
        lays.append({"c": c, "k": kv_dev(np.ascontiguousarray(x["k_raw"][:, :, T - 1:])),
                     "v": kv_dev(np.ascontiguousarray(x["v_raw"][:, :, T - 1:])), "q": bf16_dev(qb),
                     "out": torch.zeros((B, H, D), dtype=torch.bfloat16, device="cuda")})
    torch.cuda.synchronize()
    lens = dev_tensor(np.full(B, T, np.int32))
    ws = lays[0]["c"].workspace(T)
    scale = 1.0 / np.sqrt(D)

    def step():
        for ly in lays:
            ly["c"].append_decode(ly["k"], ly["v"], ly["q"], lens, scale, T, out=ly["out"], workspace=ws, stream=s)

    with torch.cuda.stream(s):
        step()
    s.synchronize()
    want = [to_host_bits(ly["out"]) for ly in lays]
    state = [{n: getattr(ly["c"], n).clone() for n in ("k_codes", "v_codes", "k_scales", "v_scales")} for ly in lays]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    s.synchronize()
    other_ws = lays[0]["c"].workspace(T)
    for r in range(4):
        for ly in lays:
            ly["out"].zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g.replay()
        s.synchronize()
        for i, ly in enumerate(lays):
            assert np.array_equal(to_host_bits(ly["out"]), want[i]), f"replay {r}, layer {i}: output"
            for n, t in state[i].items():
                assert torch.equal(getattr(ly["c"], n), t), f"replay {r}, layer {i}: {n}"
        assert int(torch.count_nonzero(ws).item()) == 0, f"replay {r}: workspace left nonzero"
        # eager work between replays: a library call on its own workspace and torch ops
        eager = lays[r % layers]["c"].decode(lays[0]["q"], lens, scale, T, workspace=other_ws)
        _ = (eager.float().sum() + torch.randn(1000, device="cuda").abs().sum()).item()
        torch.cuda.synchronize()
