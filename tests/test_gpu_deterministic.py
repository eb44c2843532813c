"""Deterministic dQ (descriptor field `deterministic` = 1): each (key tile,
query tile) step stores its fp16 dQ partial in its own slot, and the
finaliser adds the slots of a query in fp16 in ascending key-tile order.

Checked here, on the GPU through the C ABI:
- parity with the oracle to the same bar as the atomic mode;
- bitwise repeatability of every output across steps and across calls;
- O, dK, dV bitwise equal to the atomic mode (they do not touch dQ), and dQ
  within fp16 accumulation-order noise of it;
- the dQ causality probe that the atomic mode cannot run bitwise: with the
  causal dQ prescale, scaling the keys and values of tokens more than 32
  positions after i0 leaves the dQ rows up to i0 bit-identical.
"""

import pytest
import torch

from precision_causal_attention_hadamard_amd import workloads as W
from test_gpu_parity import CASES, check_outputs, run_oracle

pytestmark = pytest.mark.gpu

DET_CASES = {
    "ragged_d64_h3": CASES["ragged_d64_h3"],
    "hadamard_outliers_d128": CASES["hadamard_outliers_d128"],
    "ragged_d128_h4": CASES["ragged_d128_h4"],
    "mixed_d128_h2": lambda: W.small_packed(42, [256, 100], heads=2, head_dim=128, path=1),
    # the finaliser's rotation at d = 64 (one butterfly stage across a lane's chunks)
    "hadamard_ragged_d64_h3": lambda: W.small_packed(43, [1, 17, 45, 100, 33, 64, 130, 2, 200], heads=3,
                                                     head_dim=64, hadamard=True),
}


def run_det(flamia, wl, deterministic=True, causal_dq_scale=False, steps=1):
    dev = torch.device("cuda")
    q, k, v, do = (t.to(dev) for t in (wl.q, wl.k, wl.v, wl.do))
    call = flamia.TrainingCall(q, k, v, do, wl.cu_seqlens, hadamard=wl.hadamard, path=wl.path,
                               causal_dq_scale=causal_dq_scale, deterministic=deterministic)
    for _ in range(steps):
        call.step()
    torch.cuda.synchronize()
    return call


@pytest.mark.parametrize("case", list(DET_CASES))
def test_deterministic_parity(gpu_lib, case):
    print(f"[det] case={case}", flush=True)
    wl = DET_CASES[case]()
    call = run_det(gpu_lib, wl)
    assert call.plan_error_word() == 0
    m = check_outputs(call, run_oracle(wl))
    print(f"[det] {case}: " + ", ".join(f"{k} rel={v[0]:.2e} cos={v[1]:.6f}" for k, v in m.items()), flush=True)


@pytest.mark.parametrize("case", ["ragged_d128_h4", "mixed_d128_h2"])
def test_deterministic_bitwise_repeat_and_atomic_agreement(gpu_lib, case):
    wl = DET_CASES[case]()
    a = run_det(gpu_lib, wl)
    first = {n: getattr(a, n).clone() for n in ("o", "dq", "dk", "dv")}
    a.step()
    torch.cuda.synchronize()
    b = run_det(gpu_lib, wl, steps=2)
    for n, ref in first.items():
        assert torch.equal(getattr(a, n), ref), n
        assert torch.equal(getattr(b, n), ref), n
    c = run_det(gpu_lib, wl, deterministic=False)
    for n in ("o", "dk", "dv"):
        assert torch.equal(getattr(c, n), first[n]), n
    dq_a, dq_c = first["dq"].float(), c.dq.float()
    rel = float((dq_a - dq_c).abs().max() / dq_c.abs().max())
    print(f"[det] {case}: dq deterministic vs atomic max rel diff {rel:.2e}", flush=True)
    assert rel <= 2e-3


def test_deterministic_dq_causality_probe(gpu_lib):
    wl = W.small_packed(35, [400], heads=2, head_dim=128)
    a = run_det(gpu_lib, wl, causal_dq_scale=True)
    i0 = 150
    k2, v2 = wl.k.clone(), wl.v.clone()
    k2[i0 + 33:] *= 256.0
    v2[i0 + 33:] *= 256.0
    wl2 = W.Workload(wl.name, wl.q, k2, v2, wl.do, wl.cu_seqlens, wl.heads, wl.head_dim)
    b = run_det(gpu_lib, wl2, causal_dq_scale=True)
    assert torch.equal(b.o[: i0 + 1], a.o[: i0 + 1])
    assert torch.equal(b.dq[: i0 + 1], a.dq[: i0 + 1])
    assert not torch.equal(b.dq, a.dq)


def test_deterministic_overflow_is_loud(gpu_lib):
    """max_doc_len under-promised (100 tokens for two 2000-token documents):
    the partials that do not fit are dropped, every dQ row that lost one is
    NaN, the plan's error word is 1, and everything else -- O, dK, dV and the
    dQ rows that kept all their partials -- equals the call with the true
    bound bit for bit."""
    wl = W.small_packed(38, [2000, 2000], heads=1, head_dim=64)
    dev = torch.device("cuda")
    q, k, v, do = (t.to(dev) for t in (wl.q, wl.k, wl.v, wl.do))
    bad = gpu_lib.TrainingCall(q, k, v, do, wl.cu_seqlens, deterministic=True, max_doc_len=100)
    good = gpu_lib.TrainingCall(q, k, v, do, wl.cu_seqlens, deterministic=True)
    bad.step()
    good.step()
    torch.cuda.synchronize()
    assert bad.plan_error_word() == 1 and good.plan_error_word() == 0
    for n in ("o", "dk", "dv"):
        assert torch.equal(getattr(bad, n), getattr(good, n)), n
    nan_rows = torch.isnan(bad.dq.float()).any(dim=-1).squeeze(1).cpu()
    assert torch.isnan(bad.dq.float()[nan_rows]).all()
    assert 0 < int(nan_rows.sum()) < wl.total_tokens
    assert int(nan_rows[2000:].sum()) == 2000             # the second document's steps all lie beyond the cap
    keep = ~nan_rows
    assert torch.equal(bad.dq[keep], good.dq[keep])
