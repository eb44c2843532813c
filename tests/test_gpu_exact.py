"""The exact option on the GPU (per-token operand scales, the V fold on every
tile, per-row / per-key dS exponents, the per-token causal dQ prescale),
through the C ABI.

* Parity with the oracle's exact option: per-token codes and exponents bit
  for bit (V's per-key codes equal its codes; K's in-block prefix maximum),
  outputs to the decision-aware bar (decision_compare.py), atomic and
  deterministic dQ.
* The pages' leak probe on the GPU: inputs at positions >= j0 perturbed so
  their scale groups' maxima rise, deterministic dQ; O and dQ of every
  earlier position come back bit for bit, also inside j0's own 32-token block.
"""

import numpy as np
import pytest
import torch

import decision_compare as DCMP
from oracle import attention as A
from oracle import decisions as DC
from precision_causal_attention_hadamard_amd import workloads as W

pytestmark = pytest.mark.gpu


def np_inputs(wl):
    return [t.float().numpy().astype(np.float64) for t in (wl.q, wl.k, wl.v, wl.do)]


def run_gpu(lib, wl, deterministic=False, tensors=None):
    dev = torch.device("cuda")
    q, k, v, do = (t.to(dev) for t in (tensors or (wl.q, wl.k, wl.v, wl.do)))
    call = lib.TrainingCall(q, k, v, do, wl.cu_seqlens, hadamard=wl.hadamard, deterministic=deterministic,
                            exact=True)
    call.step()
    torch.cuda.synchronize()
    return call


CASES = {
    "ragged_d64_h3": lambda: W.small_packed(71, [1, 17, 45, 100, 33, 64, 130, 2], heads=3, head_dim=64),
    "ragged_d128_h2": lambda: W.small_packed(72, [129, 64, 31, 250], heads=2, head_dim=128),
    "hadamard_outliers_d128": lambda: W.small_packed(73, [300, 211], heads=2, head_dim=128,
                                                     outlier_scale=20.0, hadamard=True),
    "gqa_h6_kv2_d128": lambda: W.small_packed(75, [129, 64, 31, 250], heads=6, head_dim=128, kv_heads=2),
    "gqa_h4_kv1_d64": lambda: W.small_packed(76, [1, 17, 45, 100, 33, 64, 130, 2], heads=4, head_dim=64,
                                             kv_heads=1),
}


@pytest.mark.parametrize("det", [False, True], ids=["atomic", "deterministic"])
@pytest.mark.parametrize("case", list(CASES))
def test_exact_parity(gpu_lib, case, det):
    print(f"[exact] case={case} deterministic={det}", flush=True)
    wl = CASES[case]()
    call = run_gpu(gpu_lib, wl, det)
    q, k, v, do = np_inputs(wl)
    num = A.Numerics(hadamard=wl.hadamard, exact=True)
    ref = A.training_call(q, k, v, do, wl.cu_seqlens, num)
    for f in ("q_codes", "k_codes", "v_codes", "v_key_codes"):
        np.testing.assert_array_equal(call.codes(f).cpu().numpy(), ref[f], err_msg=f)
    np.testing.assert_array_equal(ref["v_codes"], ref["v_key_codes"])
    for f in ("q_exp", "k_exp", "v_exp", "v_key_exp", "v_ref_exp"):
        np.testing.assert_array_equal(call.exps(f).cpu().numpy().astype(np.int64), ref[f] + 127, err_msg=f)
    # K's in-block prefix maximum of the per-token exponents
    kref = np.zeros_like(ref["k_exp"])
    for s, e in zip(wl.cu_seqlens, wl.cu_seqlens[1:]):
        for b0 in range(s, e, 32):
            kref[:, b0:min(b0 + 32, e)] = np.maximum.accumulate(ref["k_exp"][:, b0:min(b0 + 32, e)], axis=1)
    np.testing.assert_array_equal(call.exps("k_ref_exp").cpu().numpy().astype(np.int64), kref + 127)
    al = DC.allowances(q, k, v, do, wl.cu_seqlens, num)
    outs = {n: getattr(call, n).float().cpu().numpy() for n in ("o", "dq", "dk", "dv")}
    DCMP.check_outputs(outs, ref, al, f"exact {case}")
    rm = call.row_max.cpu().numpy().astype(np.int64)
    assert np.all(np.abs(rm - ref["row_max"]) <= 1) and (rm != ref["row_max"]).mean() <= 1e-3
    if det:
        assert call.plan_error_word() == 0


@pytest.mark.parametrize("j0", [40, 33, 64, 97])
def test_exact_leak_probe_is_zero_on_the_gpu(gpu_lib, j0):
    print(f"[exact] probe j0={j0}", flush=True)
    wl = W.small_packed(74, [130, 70], heads=2, head_dim=128)
    base = run_gpu(gpu_lib, wl, deterministic=True)
    pert = []
    g = torch.Generator().manual_seed(5)
    for t in (wl.q, wl.k, wl.v, wl.do):
        x = t.float().clone()
        x[j0:130] = x[j0:130] * 300.0 + torch.round(torch.randn(x[j0:130].shape, generator=g) * 4) / 4
        pert.append(x.to(torch.bfloat16))
    moved = run_gpu(gpu_lib, wl, deterministic=True, tensors=pert)
    for n in ("o", "dq"):
        a, b = getattr(base, n)[:j0], getattr(moved, n)[:j0]
        assert torch.equal(a, b), (n, j0, float((a.float() - b.float()).abs().max()))
    assert torch.equal(base.o[130:], moved.o[130:])            # the other document
    assert not torch.equal(base.o[j0:130], moved.o[j0:130])     # the perturbation reached the call


def test_exact_fullsize_sampled(gpu_lib):
    """The 2 x 4096-token, 16-head, d = 128 outlier workload with the exact
    option, whole call on the GPU; the oracle recomputes document 1, heads 0
    and 9."""
    wl = W.config(2)
    print(f"[exact] fullsize {wl.name}: GPU call", flush=True)
    call = run_gpu(gpu_lib, wl)
    doc, heads = 1, [0, 9]
    s, e = wl.cu_seqlens[doc], wl.cu_seqlens[doc + 1]
    arrs = [t[s:e][:, heads].float().numpy().astype(np.float64) for t in (wl.q, wl.k, wl.v, wl.do)]
    num = A.Numerics(hadamard=wl.hadamard, exact=True)
    print("[exact] fullsize: oracle slice", flush=True)
    ref = A.training_call(*arrs, [0, e - s], num)
    print("[exact] fullsize: decision bounds", flush=True)
    al = DC.allowances(*arrs, [0, e - s], num)
    hs = torch.tensor(heads)
    for f in ("q_codes", "k_codes", "v_codes"):
        np.testing.assert_array_equal(call.codes(f)[s:e].cpu()[:, hs].numpy(), ref[f], err_msg=f)
    for f in ("q_exp", "k_exp", "v_exp", "v_ref_exp"):
        np.testing.assert_array_equal(call.exps(f).cpu()[hs][:, s:e].numpy().astype(np.int64), ref[f] + 127,
                                      err_msg=f)
    outs = {n: getattr(call, n)[s:e].cpu()[:, hs].float().numpy() for n in ("o", "dq", "dk", "dv")}
    DCMP.check_outputs(outs, ref, al, "exact fullsize")
    rm = call.row_max.cpu()[hs][:, s:e].numpy().astype(np.int64)
    assert np.all(np.abs(rm - ref["row_max"]) <= 1) and (rm != ref["row_max"]).mean() <= 1e-3
