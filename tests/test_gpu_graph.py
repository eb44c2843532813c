"""The whole call (quantize, forward, backward through the C ABI) captured in
one HIP graph and replayed.

The library only enqueues kernels on the caller's stream (no allocation, no
host synchronisation, no memset nodes), so a captured step must replay to the
eager result: every replay is checked against an eager step run before it,
with eager work and synchronisations between replays (the fp16 dQ atomics
make dQ's summation order free in the default mode, so there dQ is held to
accumulation-order noise and everything else to bit equality; the
deterministic mode is bitwise throughout).  The pages capture the call in a
CUDA graph for timing ([Reading, 5.1] benchmark method; appendix on pitfalls).
"""

import pytest
import torch

from precision_causal_attention_hadamard_amd import workloads as W

pytestmark = pytest.mark.gpu


def make_call(lib, wl, deterministic):
    dev = torch.device("cuda")
    q, k, v, do = (t.to(dev) for t in (wl.q, wl.k, wl.v, wl.do))
    return lib.TrainingCall(q, k, v, do, wl.cu_seqlens, hadamard=wl.hadamard, path=wl.path,
                            deterministic=deterministic)


def outputs(call):
    return {n: getattr(call, n).clone() for n in ("o", "dq", "dk", "dv", "row_max", "row_sum")}


CASES = {
    "ragged_d128_h4": lambda: W.small_packed(71, [129, 64, 31, 250], heads=4, head_dim=128),
    "hadamard_outliers_d128": lambda: W.small_packed(72, [300, 211], heads=2, head_dim=128,
                                                     outlier_scale=20.0, hadamard=True),
    "mixed_d64": lambda: W.small_packed(73, [1, 70, 33, 130], heads=3, head_dim=64, path=1),
}


@pytest.mark.parametrize("deterministic", [False, True], ids=["atomic", "deterministic"])
@pytest.mark.parametrize("case", list(CASES))
def test_graph_replays_match_eager(gpu_lib, case, deterministic):
    print(f"[graph] case={case} deterministic={deterministic}", flush=True)
    wl = CASES[case]()
    call = make_call(gpu_lib, wl, deterministic)
    call.step()                       # warm-up outside the capture
    torch.cuda.synchronize()
    eager = outputs(call)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call.step()
    torch.cuda.synchronize()
    for rep in range(3):
        # eager work between replays: overwrite every output, then replay
        for t in (call.o, call.dq, call.dk, call.dv, call.row_sum):
            t.fill_(7.0)
        call.row_max.fill_(-5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = outputs(call)
        for n, ref in eager.items():
            if n == "dq" and not deterministic:
                rel = float((got[n].float() - ref.float()).abs().max() / ref.float().abs().max())
                assert rel <= 2e-3, (rep, n, rel)
            else:
                assert torch.equal(got[n], ref), (rep, n)
        # an eager step between replays gives the same result again
        call.step()
        torch.cuda.synchronize()
        for n in ("o", "dk", "dv", "row_max", "row_sum"):
            assert torch.equal(getattr(call, n), eager[n]), (rep, "eager", n)
