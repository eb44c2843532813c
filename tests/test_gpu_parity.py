"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Bit-exact: E4M3 codes, exponent bytes, per-key V codes, the fold reference,
the work lists.  Within tolerance (max-abs relative error <= 2e-2 and cosine
>= 0.999 per output tensor, applied to what is unique where admissible fp32
evaluations can take a quantized decision either way -- decision_compare.py):
O, dQ, dK, dV.  The integer row maximum must agree except where a score lies
within fp32 accumulation rounding of an integer boundary.
"""

import numpy as np
import pytest
import torch

import decision_compare as DCMP
from oracle import attention as A
from oracle import decisions as DC
from oracle import formats, nvfp4, quant
from oracle import worklist as WL
from precision_causal_attention_hadamard_amd import workloads as W

pytestmark = pytest.mark.gpu


def np_inputs(wl):
    return [t.float().numpy().astype(np.float64) for t in (wl.q, wl.k, wl.v, wl.do)]


def run_gpu(flamia, wl, causal_dq_scale=False):
    dev = torch.device("cuda")
    q, k, v, do = (t.to(dev) for t in (wl.q, wl.k, wl.v, wl.do))
    call = flamia.TrainingCall(q, k, v, do, wl.cu_seqlens, hadamard=wl.hadamard,
                               causal_dq_scale=causal_dq_scale, path=wl.path)
    call.step()
    torch.cuda.synchronize()
    return call


def run_oracle(wl):
    """The oracle's result, with its decision bounds attached for check_outputs."""
    q, k, v, do = np_inputs(wl)
    num = A.Numerics(hadamard=wl.hadamard, path="mixed" if wl.path else "mxfp8")
    ref = A.training_call(q, k, v, do, wl.cu_seqlens, num)
    ref["_allow"] = DC.allowances(q, k, v, do, wl.cu_seqlens, num)
    return ref


def check_codes(call, ref):
    for f in ("q_codes", "k_codes", "v_codes", "v_key_codes"):
        np.testing.assert_array_equal(call.codes(f).cpu().numpy(), ref[f], err_msg=f)
    for f in ("q_exp", "k_exp", "v_exp", "v_key_exp", "v_ref_exp"):
        np.testing.assert_array_equal(call.exps(f).cpu().numpy().astype(np.int64), ref[f] + 127, err_msg=f)


def check_outputs(call, ref, names=("o", "dq", "dk", "dv"), tag="parity"):
    outs = {n: getattr(call, n).float().cpu().numpy() for n in names}
    m = DCMP.check_outputs(outs, ref, ref["_allow"], tag, names)
    rm = call.row_max.cpu().numpy().astype(np.int64)
    diff = rm != ref["row_max"]
    assert np.all(np.abs(rm - ref["row_max"]) <= 1)
    assert diff.mean() <= 1e-3, diff.mean()
    np.testing.assert_allclose(call.row_sum.cpu().numpy(), ref["row_sum"], rtol=1e-3)
    return {n: (v[1], v[2]) for n, v in m.items()}


CASES = {
    "tiny_config1": lambda: W.config(1),
    "ragged_d64_h3": lambda: W.small_packed(31, [1, 17, 45, 100, 33, 64, 130, 2], heads=3, head_dim=64),
    "hadamard_outliers_d128": lambda: W.small_packed(32, [300, 211], heads=2, head_dim=128,
                                                     outlier_scale=20.0, hadamard=True),
    "ragged_d128_h4": lambda: W.small_packed(33, [129, 64, 31, 250], heads=4, head_dim=128),
    # zero-length documents at the start, in the middle and at the end of the packed batch
    "empty_docs_d64": lambda: W.small_packed(37, [0, 45, 0, 0, 100, 33, 0], heads=2, head_dim=64),
    # documents on tile and block boundaries (multiples of 32, 64 and 128 tokens), one head
    "aligned_d128_h1": lambda: W.small_packed(38, [128, 256, 64, 32, 384], heads=1, head_dim=128),
    # one long document at d = 64 with the rotation: many key tiles per query tile
    "long_d64_hadamard": lambda: W.small_packed(39, [1999], heads=2, head_dim=64, hadamard=True),
    # row maxima near +150 and -150 beside ordinary rows: both probability forms
    "extreme_rows_d64": lambda: W.extreme_rows(1, [200, 97]),
    "extreme_rows_d128": lambda: W.extreme_rows(2, [160, 130], head_dim=128),
}


@pytest.mark.parametrize("case", list(CASES))
def test_parity_small(gpu_lib, case):
    print(f"[parity] case={case}", flush=True)
    wl = CASES[case]()
    call = run_gpu(gpu_lib, wl)
    ref = run_oracle(wl)
    check_codes(call, ref)
    m = check_outputs(call, ref)
    print(f"[parity] {case}: " + ", ".join(f"{k} rel={v[0]:.2e} cos={v[1]:.6f}" for k, v in m.items()), flush=True)


def test_parity_causal_dq_scale(gpu_lib):
    wl = CASES["hadamard_outliers_d128"]()
    call = run_gpu(gpu_lib, wl, causal_dq_scale=True)
    ref = run_oracle(wl)
    check_outputs(call, ref)


WORKLIST_DOCS = {
    # under 64 tiles per list: the one-wave sort
    "small": [1, 300, 0, 129, 128, 1000, 17, 64],
    # above 64 tiles per list: the workgroup sort
    "many": [int(x) for x in np.random.default_rng(36).integers(0, 700, size=40)] + [2500, 0, 33],
}


def check_dispatch(bwd, disp):
    """The backward's launch order is a permutation of the backward list
    that keeps each document's key tiles together, in tile order, with the
    documents in the order their first tiles take in the backward list."""
    b, s_ = np.asarray(bwd, np.int64), np.asarray(disp, np.int64)
    assert b.shape == s_.shape
    kb, ks = b[:, 0] * (1 << 20) + b[:, 1], s_[:, 0] * (1 << 20) + s_[:, 1]
    assert np.array_equal(np.sort(kb), np.sort(ks)) and len(np.unique(ks)) == len(ks)
    if not len(b):
        return
    _, first = np.unique(b[:, 0], return_index=True)
    doc_order = b[np.sort(first), 0]
    starts = np.r_[True, s_[1:, 0] != s_[:-1, 0]]
    assert np.array_equal(s_[starts, 0], doc_order)          # contiguous, in first-appearance order
    run_start = np.flatnonzero(starts)
    pos = np.arange(len(s_)) - run_start[np.cumsum(starts) - 1]
    assert np.array_equal(s_[:, 1], pos)                      # tiles 0, 1, ... inside each document


@pytest.mark.parametrize("docs", list(WORKLIST_DOCS))
def test_worklists_match_oracle(gpu_lib, docs):
    heads = 3 if docs == "small" else 1
    wl = W.small_packed(34, WORKLIST_DOCS[docs], heads=heads, head_dim=64)
    call = run_gpu(gpu_lib, wl)
    fbq, fbk, bbq, bbk = gpu_lib.tile_config(64)
    fwd, bwd = call.plan_lists()
    want_f = [(d, t) for d, t, h, c in WL.fwd_items(wl.cu_seqlens, 1, fbq, fbk)]
    want_b = [(d, t) for d, t, h, c in WL.bwd_items(wl.cu_seqlens, 1, bbq, bbk)]
    assert [tuple(x) for x in fwd.tolist()] == want_f
    assert [tuple(x) for x in bwd.tolist()] == want_b
    check_dispatch(bwd, call.plan_dispatch())


def test_repeatable_bitwise(gpu_lib):
    wl = CASES["ragged_d128_h4"]()
    a = run_gpu(gpu_lib, wl)
    o1, dk1, dv1 = a.o.clone(), a.dk.clone(), a.dv.clone()
    a.step()
    torch.cuda.synchronize()
    assert torch.equal(a.o, o1) and torch.equal(a.dk, dk1) and torch.equal(a.dv, dv1)


def test_causality_probe_gpu(gpu_lib):
    """Scaling K and V of keys j > i0 + 32 leaves every earlier output bit-identical."""
    wl = W.small_packed(35, [400], heads=2, head_dim=128)
    a = run_gpu(gpu_lib, wl)
    o_a = a.o.clone()
    i0 = 150
    k2, v2 = wl.k.clone(), wl.v.clone()
    k2[i0 + 33:] *= 256.0
    v2[i0 + 33:] *= 256.0
    wl2 = W.Workload(wl.name, wl.q, k2, v2, wl.do, wl.cu_seqlens, wl.heads, wl.head_dim)
    b = run_gpu(gpu_lib, wl2)
    assert torch.equal(b.o[: i0 + 1], o_a[: i0 + 1])
    assert not torch.equal(b.o, o_a)


def test_document_isolation_gpu(gpu_lib):
    wl = W.small_packed(36, [90, 200, 70], heads=2, head_dim=64)
    a = run_gpu(gpu_lib, wl)
    base = {n: getattr(a, n).clone() for n in ("o", "dk", "dv")}
    codes = {f: a.codes(f).clone() for f in ("q_codes", "k_codes", "v_codes")}
    s, e = wl.cu_seqlens[1], wl.cu_seqlens[2]
    pert = [t.clone() for t in (wl.q, wl.k, wl.v, wl.do)]
    for t in pert:
        t[s:e] = (t[s:e].float() * 1e4).to(torch.bfloat16)
    wl2 = W.Workload(wl.name, *pert, wl.cu_seqlens, wl.heads, wl.head_dim)
    b = run_gpu(gpu_lib, wl2)
    other = torch.cat([torch.arange(0, s), torch.arange(e, wl.total_tokens)]).cuda()
    for n in base:
        assert torch.equal(getattr(b, n)[other], base[n][other]), n
    for f in codes:
        assert torch.equal(b.codes(f)[other], codes[f][other]), f


MIXED_CASES = {
    "mixed_ragged_d64": lambda: W.small_packed(41, [1, 70, 33, 130], heads=3, head_dim=64, path=1),
    "mixed_d128_h2": lambda: W.small_packed(42, [256, 100], heads=2, head_dim=128, path=1),
    "mixed_hadamard_outliers_d128": lambda: W.small_packed(43, [200, 57], heads=2, head_dim=128,
                                                           outlier_scale=20.0, hadamard=True, path=1),
}


def check_nvfp4(call, wl):
    """NVFP4 codes (packed, even element in the low nibble), E4M3 group-scale
    bytes and tensor scales equal the oracle's, bit for bit."""
    q, k, v, _ = np_inputs(wl)
    qt = quant.quantize_qkv(q, k, v, wl.cu_seqlens, wl.hadamard)
    for which, rot in (("q", qt["q_rot"]), ("k", qt["k_rot"])):
        codes, scales, t, _ = nvfp4.quantize_nvfp4(rot)
        packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
        g_codes, g_sf, g_t = call.nvfp4(which)
        np.testing.assert_array_equal(g_codes.cpu().numpy(), packed, err_msg=f"{which} codes")
        np.testing.assert_array_equal(g_sf.cpu().numpy(), formats.e4m3_bits(scales), err_msg=f"{which} scales")
        assert float(g_t) == float(t), which


@pytest.mark.parametrize("case", list(MIXED_CASES))
def test_parity_mixed_path(gpu_lib, case):
    print(f"[parity] case={case}", flush=True)
    wl = MIXED_CASES[case]()
    call = run_gpu(gpu_lib, wl)
    ref = run_oracle(wl)
    check_codes(call, ref)
    check_nvfp4(call, wl)
    m = check_outputs(call, ref)
    print(f"[parity] {case}: " + ", ".join(f"{k} rel={v[0]:.2e} cos={v[1]:.6f}" for k, v in m.items()), flush=True)


def test_empty_call(gpu_lib):
    """No tokens at all (one or several empty documents): every entry point
    succeeds with the empty tensors torch hands over, and the work lists are
    empty."""
    dev = torch.device("cuda")
    for cu in ([0, 0], [0, 0, 0, 0]):
        z = torch.empty(0, 2, 64, dtype=torch.bfloat16, device=dev)
        call = gpu_lib.TrainingCall(z, z, z, z, cu)
        call.step()
        torch.cuda.synchronize()
        fwd, bwd = call.plan_lists()
        assert len(fwd) == 0 and len(bwd) == 0
        assert call.o.numel() == 0 and call.dq.numel() == 0
