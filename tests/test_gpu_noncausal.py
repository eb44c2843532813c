"""GPU parity of the non-causal call (descriptor field causal = 0) against the
oracle, through the C ABI.

Without the mask every key of a document is visible to every query of it;
the quantization rules are those of the causal call, and the diagonal per-key
V fold takes the whole 32-token block as visible, so its reference is the
block exponent.  Checked here:
- codes and exponent bytes bit for bit, the fold reference equal to the block
  exponent;
- O, dQ, dK, dV to the bar of the causal cases (decision_compare.py), the
  integer row maximum and l as there; MHA, Hadamard with outliers, grouped
  query heads, deterministic dQ, the mixed NVFP4-score path;
- the work lists equal the oracle's non-causal lists;
- the last token of each document sees the same keys with and without the
  mask, so its O row, row maximum and l are bitwise those of the causal call;
- document isolation, bit for bit;
- the packed lognormal workload at full size (sampled document/head slices).
"""

import numpy as np
import pytest
import torch

import decision_compare as DCMP
from oracle import attention as A
from oracle import decisions as DC
from oracle import worklist as WL
from precision_causal_attention_hadamard_amd import workloads as W
from test_gpu_fullsize import doc_choice, report

pytestmark = pytest.mark.gpu


def np_inputs(wl):
    return [t.float().numpy().astype(np.float64) for t in (wl.q, wl.k, wl.v, wl.do)]


def run_nc(flamia, wl, deterministic=False, causal=False, steps=1):
    dev = torch.device("cuda")
    q, k, v, do = (t.to(dev) for t in (wl.q, wl.k, wl.v, wl.do))
    call = flamia.TrainingCall(q, k, v, do, wl.cu_seqlens, hadamard=wl.hadamard, causal=causal,
                               deterministic=deterministic, path=wl.path)
    for _ in range(steps):
        call.step()
    torch.cuda.synchronize()
    return call


def oracle_nc(arrs, cu, hadamard, path=0):
    num = A.Numerics(hadamard=hadamard, causal=False, path="mixed" if path else "mxfp8")
    ref = A.training_call(*arrs, cu, num)
    ref["_allow"] = DC.allowances(*arrs, cu, num)
    return ref


def check_codes(call, ref, sl=slice(None), heads=None):
    hs = torch.tensor(heads) if heads is not None else slice(None)
    for f in ("q_codes", "k_codes", "v_codes", "v_key_codes"):
        np.testing.assert_array_equal(call.codes(f)[sl].cpu()[:, hs].numpy(), ref[f], err_msg=f)
    for f in ("q_exp", "k_exp", "v_exp", "v_key_exp"):
        got = call.exps(f).cpu()[hs][:, sl].numpy().astype(np.int64)
        np.testing.assert_array_equal(got, ref[f] + 127, err_msg=f)
    # no mask: the fold reference is the block exponent
    got = call.exps("v_ref_exp").cpu()[hs][:, sl].numpy().astype(np.int64)
    np.testing.assert_array_equal(got, ref["v_exp"] + 127, err_msg="v_ref_exp")


def check_outputs(outs, call_rm, call_rs, ref, tag):
    m = DCMP.check_outputs(outs, ref, ref["_allow"], tag, ("o", "dq", "dk", "dv"))
    rm = call_rm.astype(np.int64)
    assert np.all(np.abs(rm - ref["row_max"]) <= 1)
    assert (rm != ref["row_max"]).mean() <= 1e-3
    np.testing.assert_allclose(call_rs, ref["row_sum"], rtol=1e-3)
    return {n: (v[1], v[2]) for n, v in m.items()}


CASES = {
    "ragged_d64_h3": lambda: W.small_packed(51, [1, 17, 45, 100, 33, 64, 130, 2], heads=3, head_dim=64),
    "hadamard_outliers_d128": lambda: W.small_packed(52, [300, 211], heads=2, head_dim=128,
                                                     outlier_scale=20.0, hadamard=True),
    "ragged_d128_h4": lambda: W.small_packed(53, [129, 64, 31, 250], heads=4, head_dim=128),
    "long_doc_d128": lambda: W.small_packed(54, [1000], heads=2, head_dim=128),
    "gqa_d128_h4_kv2": lambda: W.small_packed(55, [129, 64, 31, 250], heads=4, head_dim=128, kv_heads=2),
    "gqa_d64_h6_kv2": lambda: W.small_packed(56, [50, 1, 177], heads=6, head_dim=64, kv_heads=2),
    "mixed_ragged_d64": lambda: W.small_packed(63, [1, 70, 33, 130], heads=3, head_dim=64, path=1),
    "mixed_d128_h2": lambda: W.small_packed(64, [256, 100], heads=2, head_dim=128, path=1),
}


def parity(lib, case, deterministic=False):
    wl = CASES[case]()
    call = run_nc(lib, wl, deterministic=deterministic)
    if deterministic:
        assert call.plan_error_word() == 0
    ref = oracle_nc(np_inputs(wl), wl.cu_seqlens, wl.hadamard, wl.path)
    check_codes(call, ref)
    outs = {n: getattr(call, n).float().cpu().numpy() for n in ("o", "dq", "dk", "dv")}
    m = check_outputs(outs, call.row_max.cpu().numpy(), call.row_sum.cpu().numpy(), ref, "noncausal")
    print(f"[noncausal] {case} det={deterministic}: "
          + ", ".join(f"{k} rel={v[0]:.2e} cos={v[1]:.6f}" for k, v in m.items()), flush=True)
    return call


@pytest.mark.parametrize("case", list(CASES))
def test_noncausal_parity(gpu_lib, case):
    print(f"[noncausal] case={case}", flush=True)
    parity(gpu_lib, case)


@pytest.mark.parametrize("case", ["ragged_d128_h4", "gqa_d128_h4_kv2", "hadamard_outliers_d128", "mixed_d128_h2"])
def test_noncausal_deterministic_parity_repeat_and_atomic_agreement(gpu_lib, case):
    print(f"[noncausal] deterministic case={case}", flush=True)
    a = parity(gpu_lib, case, deterministic=True)
    first = {n: getattr(a, n).clone() for n in ("o", "dq", "dk", "dv")}
    a.step()
    torch.cuda.synchronize()
    for n, ref in first.items():
        assert torch.equal(getattr(a, n), ref), n
    c = run_nc(gpu_lib, CASES[case]())
    for n in ("o", "dk", "dv"):
        assert torch.equal(getattr(c, n), first[n]), n
    rel = float((first["dq"].float() - c.dq.float()).abs().max() / c.dq.float().abs().max())
    print(f"[noncausal] {case}: dq deterministic vs atomic max rel diff {rel:.2e}", flush=True)
    assert rel <= 2e-3


def test_noncausal_worklists_match_oracle(gpu_lib):
    docs = [int(x) for x in np.random.default_rng(57).integers(0, 700, size=40)] + [2500, 0, 33]
    for d in ([1, 300, 0, 129, 128, 1000, 17, 64], docs):
        wl = W.small_packed(58, d, heads=1, head_dim=64)
        call = run_nc(gpu_lib, wl)
        fbq, fbk, bbq, bbk = gpu_lib.tile_config(64)
        fwd, bwd = call.plan_lists()
        want_f = [(dd, t) for dd, t, h, c in WL.fwd_items(wl.cu_seqlens, 1, fbq, fbk, causal=False)]
        want_b = [(dd, t) for dd, t, h, c in WL.bwd_items(wl.cu_seqlens, 1, bbq, bbk, causal=False)]
        assert [tuple(x) for x in fwd.tolist()] == want_f
        assert [tuple(x) for x in bwd.tolist()] == want_b


def test_noncausal_last_token_equals_causal_bitwise(gpu_lib):
    wl = CASES["ragged_d128_h4"]()
    a = run_nc(gpu_lib, wl, causal=True)
    b = run_nc(gpu_lib, wl, causal=False)
    last = torch.tensor([e - 1 for e in wl.cu_seqlens[1:]], device="cuda")
    assert torch.equal(a.o[last], b.o[last])
    assert torch.equal(a.row_max[:, last], b.row_max[:, last])
    assert torch.equal(a.row_sum[:, last], b.row_sum[:, last])
    assert not torch.equal(a.o, b.o) and not torch.equal(a.dk, b.dk)


def test_noncausal_document_isolation_gpu(gpu_lib):
    wl = W.small_packed(59, [90, 200, 70], heads=2, head_dim=64)
    a = run_nc(gpu_lib, wl)
    base = {n: getattr(a, n).clone() for n in ("o", "dq", "dk", "dv")}
    s, e = wl.cu_seqlens[1], wl.cu_seqlens[2]
    pert = [t.clone() for t in (wl.q, wl.k, wl.v, wl.do)]
    for t in pert:
        t[s:e] = (t[s:e].float() * 1e4).to(torch.bfloat16)
    wl2 = W.Workload(wl.name, *pert, wl.cu_seqlens, wl.heads, wl.head_dim)
    b = run_nc(gpu_lib, wl2)
    other = torch.cat([torch.arange(0, s), torch.arange(e, wl.total_tokens)]).cuda()
    for n in ("o", "dk", "dv"):
        assert torch.equal(getattr(b, n)[other], base[n][other]), n
    # dQ rows of other documents: the fp16 atomic order may differ, the values may not move beyond it
    dq_a, dq_b = base["dq"][other].float(), b.dq[other].float()
    assert float((dq_a - dq_b).abs().max()) <= 2e-3 * float(dq_a.abs().max())


def test_noncausal_fullsize_packed_lognormal(gpu_lib):
    """The packed lognormal workload (4 x 16384 tokens, 16 heads, d = 128) as
    one non-causal call; oracle slices of three documents."""
    wl = W.config(3)
    print("[noncausal] config3 shape: GPU call", flush=True)
    call = run_nc(gpu_lib, wl)
    for which, heads in (("ragged", [13]), ("shortest", [4]), ("0", [0, 9])):
        doc = doc_choice(wl.cu_seqlens, which)
        s, e = wl.cu_seqlens[doc], wl.cu_seqlens[doc + 1]
        arrs = [t[s:e][:, heads].float().numpy().astype(np.float64) for t in (wl.q, wl.k, wl.v, wl.do)]
        print(f"[noncausal]   oracle slice doc {doc} (L={e - s}) heads {heads}", flush=True)
        ref = oracle_nc(arrs, [0, e - s], wl.hadamard)
        check_codes(call, ref, slice(s, e), heads)
        hs = torch.tensor(heads)
        outs = {n: getattr(call, n)[s:e].cpu()[:, hs].float().numpy() for n in ("o", "dq", "dk", "dv")}
        m = check_outputs(outs, call.row_max.cpu()[hs][:, s:e].numpy(), call.row_sum.cpu()[hs][:, s:e].numpy(),
                          ref, "noncausal fullsize")
        report("config3 non-causal", wl, doc, heads, m)
