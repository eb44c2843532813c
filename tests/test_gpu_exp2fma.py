"""The training call with part of the exponentials on the FMA pipe
(``exp2_fma = 1``; [Reading, 4.4] second bullet: a polynomial emulates part
of the exp work on the FMA units): the 32 x 32 blocks whose query-block and
key-block indices have an odd sum take a degree-5 polynomial for exp2, in
both passes.

* Parity with the oracle (exact P) within the bar of R15 applied by the
  decision rule of R21: the polynomial's error (2.4 ulp) lies inside the
  ±4-ulp exp2 allowance of the decision bounds.
* The backward replays the forward's probability codes (same block choice,
  same instruction sequence), checked as for the plain call.
* The row sums differ from the plain call's (the polynomial is really used),
  and the calls it is not built for are refused.
"""

import numpy as np
import pytest
import torch

import decision_compare as DCMP
from oracle import attention as A
from oracle import decisions as DC
from precision_causal_attention_hadamard_amd import workloads as W
from test_gpu_diag import check_replay, run_diag

pytestmark = pytest.mark.gpu

CASES = {
    "ragged_d64_h3": lambda: W.small_packed(51, [1, 17, 45, 100, 33, 64, 130, 2], heads=3, head_dim=64),
    "hadamard_outliers_d128": lambda: W.small_packed(52, [300, 211], heads=2, head_dim=128,
                                                     outlier_scale=20.0, hadamard=True),
    "extreme_rows_d128": lambda: W.extreme_rows(5, [230, 100], head_dim=128),
}


def np_inputs(wl):
    return [t.float().numpy().astype(np.float64) for t in (wl.q, wl.k, wl.v, wl.do)]


def run(lib, wl, exp2_fma):
    dev = torch.device("cuda")
    q, k, v, do = (t.to(dev) for t in (wl.q, wl.k, wl.v, wl.do))
    call = lib.TrainingCall(q, k, v, do, wl.cu_seqlens, hadamard=wl.hadamard, exp2_fma=exp2_fma)
    call.step()
    torch.cuda.synchronize()
    return call


@pytest.mark.parametrize("case", list(CASES))
def test_exp2_fma_parity(gpu_lib, case):
    wl = CASES[case]()
    print(f"[exp2fma] {case}", flush=True)
    call = run(gpu_lib, wl, True)
    qn, kn, vn, don = np_inputs(wl)
    num = A.Numerics(hadamard=wl.hadamard)
    ref = A.training_call(qn, kn, vn, don, wl.cu_seqlens, num)
    al = DC.allowances(qn, kn, vn, don, wl.cu_seqlens, num)
    names = ("o", "dq", "dk", "dv")
    outs = {n: getattr(call, n).float().cpu().numpy() for n in names}
    m = DCMP.check_outputs(outs, ref, al, f"exp2fma {case}", names)
    rm = call.row_max.cpu().numpy().astype(np.int64)
    assert np.all(np.abs(rm - ref["row_max"]) <= 1)
    np.testing.assert_allclose(call.row_sum.cpu().numpy(), ref["row_sum"], rtol=1e-3)
    # P^ codes rarely move under a few-ulp change of P, but l sums the fp32
    # probabilities: it shows that the polynomial ran
    plain = run(gpu_lib, wl, False)
    assert not torch.equal(call.row_sum, plain.row_sum)
    print(f"[exp2fma] {case}: " + ", ".join(f"{k} rel={v[1]:.2e} cos={v[2]:.6f}" for k, v in m.items()),
          flush=True)


@pytest.mark.parametrize("case", list(CASES))
def test_exp2_fma_backward_replays_forward_codes(gpu_lib, case):
    wl = CASES[case]()
    print(f"[exp2fma diag] {case}", flush=True)
    call, fwd, fmax, bwd, _ = run_diag(gpu_lib, wl, exp2_fma=True)
    checked, below, differ_below = check_replay(wl, call, fwd, fmax, bwd, case)
    print(f"[exp2fma diag] {case}: {checked} codes in the normal range equal; "
          f"{differ_below} of {below} below it differ", flush=True)
    assert checked > 0
    # the diagnostic instantiation gives the plain entry points' results
    got = {n: getattr(call, n).clone() for n in ("o", "dk", "dv", "row_max", "row_sum")}
    call.step()
    torch.cuda.synchronize()
    for n, t in got.items():
        assert torch.equal(t, getattr(call, n)), n


def test_exp2_fma_refuses_unsupported_calls(gpu_lib):
    wl = W.small_packed(53, [64, 40], heads=2, head_dim=64)
    dev = torch.device("cuda")
    q, k, v, do = (t.to(dev) for t in (wl.q, wl.k, wl.v, wl.do))
    for kw in (dict(path=1), dict(exact=True), dict(causal=False), dict(deterministic=True)):
        with pytest.raises(gpu_lib.FlamiaError):
            call = gpu_lib.TrainingCall(q, k, v, do, wl.cu_seqlens, exp2_fma=True, **kw)
            call.quantize()
    kg, vg = k[:, :1].contiguous(), v[:, :1].contiguous()          # grouped query attention
    with pytest.raises(gpu_lib.FlamiaError):
        call = gpu_lib.TrainingCall(q, kg, vg, do, wl.cu_seqlens, exp2_fma=True)
        call.quantize()
    call = gpu_lib.TrainingCall(q, k, v, do, wl.cu_seqlens, exp2_fma=True)
    call.quantize()
    with pytest.raises(gpu_lib.FlamiaError, match="flamia_attn_fwd_p4"):
        gpu_lib.attn_fwd_p4(call.desc, call.qt, call.o, call.row_max, call.row_sum, call.fws)
