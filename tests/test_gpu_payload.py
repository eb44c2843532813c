"""GPU payloads the pages make exact, compared with the oracle bit for bit.

* The backward's preparation stage (flamia_attn_bwd_prep) on stand-in saved
  forward state (seeded O, integer row maximum and row sum, so both sides see
  the same inputs): the dO token-block codes and exponent bytes, the dQ
  accumulator prescale exponent and 2^-8 / l bit for bit; G = dO~ 2^-8 / l
  (bf16 of the fp32 product) bit for bit; D = sum_d dO~ O within the bound of
  an fp32 sum of d exact products ([Summary, §3.3]: D comes from the same
  quantized dO as dP).
* The dQ finaliser (flamia_attn_bwd_finish, atomic mode): dq equals
  bf16(acc 2^sigma * softmax_scale) bit for bit from the fp16 accumulator and
  the prescale exponent the workspace holds after the main stage (with the
  rotation: that value rotated back by the fp32 butterflies of the oracle's
  transform, bit for bit).
* The E4M3 conversion of the quantizer: every finite bf16 value times every
  power of two 2^k, k = -20..20, that lies in a block's E4M3 range, through
  flamia_quantize; the Q, K, V block codes and the per-key V codes and
  exponents equal the oracle's.
"""

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import formats
from oracle.quant import quantize_per_key, quantize_qkv, quantize_token_blocks
from precision_causal_attention_hadamard_amd import workloads as W

pytestmark = pytest.mark.gpu

U = 2.0 ** -24

CASES = {
    "ragged_d64_h3": dict(wl=lambda: W.small_packed(81, [1, 17, 45, 100, 33, 64, 130, 2], heads=3, head_dim=64)),
    "outliers_d128_causal_scale": dict(wl=lambda: W.small_packed(82, [300, 211], heads=2, head_dim=128,
                                                                 outlier_scale=20.0, hadamard=True),
                                       causal_dq_scale=True),
    "gqa_d128_h4_kv2": dict(wl=lambda: W.small_packed(83, [129, 64, 31, 250], heads=4, head_dim=128, kv_heads=2)),
    "exact_d128": dict(wl=lambda: W.small_packed(84, [200, 70], heads=2, head_dim=128), exact=True),
    "noncausal_d64": dict(wl=lambda: W.small_packed(85, [90, 33, 160], heads=2, head_dim=64), causal=False),
    "config2_fullsize": dict(wl=lambda: W.config(2)),
}


@pytest.mark.parametrize("case", list(CASES))
def test_bwd_prep_payload(gpu_lib, case):
    spec = CASES[case]
    wl = spec["wl"]()
    exact, cds, causal = spec.get("exact", False), spec.get("causal_dq_scale", False), spec.get("causal", True)
    print(f"[payload] {case}: T={wl.total_tokens} H={wl.heads} Hk={wl.kv_heads} d={wl.head_dim}", flush=True)
    T, H, d = wl.total_tokens, wl.heads, wl.head_dim
    o, row_max, row_sum = W.saved_forward_state(list(CASES).index(case), T, H, d)
    dev = torch.device("cuda")
    q, k, v, do = (t.to(dev) for t in (wl.q, wl.k, wl.v, wl.do))
    call = gpu_lib.TrainingCall(q, k, v, do, wl.cu_seqlens, hadamard=wl.hadamard, causal_dq_scale=cds,
                                exact=exact, causal=causal)
    call.quantize()
    gpu_lib.attn_bwd_prep(call.desc, call.qt, o.to(dev), row_max.to(dev), row_sum.to(dev), do, call.bws)
    torch.cuda.synchronize()
    got = {n_: t.cpu() for n_, t in call.bwd_payload().items()}

    # oracle side, from the same inputs
    gran = "token" if exact else "block"
    dof = wl.do.float().numpy().astype(np.float64)
    codes, exps, dod = quantize_token_blocks(dof, wl.cu_seqlens, granularity=gran)
    np.testing.assert_array_equal(got["do_codes"].numpy(), codes, err_msg="dO codes")
    np.testing.assert_array_equal(got["do_exp"].numpy().astype(np.int64), exps + 127, err_msg="dO exponents")
    qt = quantize_qkv(wl.q.float().numpy(), wl.k.float().numpy(), wl.v.float().numpy(), wl.cu_seqlens,
                      wl.hadamard, granularity=gran)
    sig = A.dq_prescale(exps, qt["k_exp"], qt["v_exp"], wl.cu_seqlens, d, cds, exact)
    np.testing.assert_array_equal(got["dq_sigma"].numpy().astype(np.int64), sig, err_msg="dQ prescale")
    l = row_sum.numpy().astype(np.float64)
    inv_l = np.ldexp(formats.fp32_round(1.0 / l), -8)
    np.testing.assert_array_equal(got["inv_l"].numpy().astype(np.float64), inv_l, err_msg="2^-8 / l")
    g = formats.bf16_round(formats.fp32_round(dod * inv_l.T[:, :, None]))
    np.testing.assert_array_equal(got["g"].float().numpy().astype(np.float64), g, err_msg="G")
    of = o.float().numpy().astype(np.float64)
    D = np.sum(dod * of, axis=2).T
    bound = (d * U / (1 - d * U)) * np.sum(np.abs(dod * of), axis=2).T + U * np.abs(D)
    err = np.abs(got["D"].numpy().astype(np.float64) - D)
    assert np.all(err <= bound), float(np.max(err - bound))
    print(f"[payload] {case}: codes, exponents, sigma, 2^-8/l, G bit-exact; "
          f"D max error {float(np.max(err / np.maximum(bound, 1e-300))):.3f} of its fp32 bound", flush=True)


def test_e4m3_conversion_sweep(gpu_lib):
    wl = W.e4m3_sweep()
    print(f"[payload] e4m3 sweep: {wl.total_tokens} tokens, {len(wl.doc_lens)} shifts", flush=True)
    dev = torch.device("cuda")
    q, k, v, do = (t.to(dev) for t in (wl.q, wl.k, wl.v, wl.do))
    call = gpu_lib.TrainingCall(q, k, v, do, wl.cu_seqlens)
    call.quantize()
    torch.cuda.synchronize()
    x = wl.q.float().numpy().astype(np.float64)
    codes, exps, _ = quantize_token_blocks(x, wl.cu_seqlens)
    for n, (s, e) in enumerate(zip(wl.cu_seqlens[:-1], wl.cu_seqlens[1:])):
        assert np.all(exps[:, s:e] == n - 20)           # document n is the shift 2^(n - 20)
    for f in ("q_codes", "k_codes", "v_codes"):
        np.testing.assert_array_equal(call.codes(f).cpu().numpy(), codes, err_msg=f)
    for f in ("q_exp", "k_exp", "v_exp"):
        np.testing.assert_array_equal(call.exps(f).cpu().numpy().astype(np.int64), exps + 127, err_msg=f)
    kc, ke, _ = quantize_per_key(x)
    np.testing.assert_array_equal(call.codes("v_key_codes").cpu().numpy(), kc, err_msg="per-key codes")
    np.testing.assert_array_equal(call.exps("v_key_exp").cpu().numpy().astype(np.int64), ke + 127)
    # the sweep reaches every E4M3 code (both signs, subnormals, zero)
    assert len(np.unique(codes)) == 254


@pytest.mark.parametrize("case", ["ragged_d64_h3", "noncausal_d64", "gqa_d128_h4_kv2", "config2_fullsize"])
def test_dq_finaliser_applies_the_prescale(gpu_lib, case):
    spec = CASES[case]
    wl = spec["wl"]()
    causal = spec.get("causal", True)
    print(f"[finalise] {case}", flush=True)
    dev = torch.device("cuda")
    q, k, v, do = (t.to(dev) for t in (wl.q, wl.k, wl.v, wl.do))
    call = gpu_lib.TrainingCall(q, k, v, do, wl.cu_seqlens, hadamard=wl.hadamard, causal=causal)
    call.step()
    torch.cuda.synchronize()
    pay = call.bwd_payload()
    sig = pay["dq_sigma"].t().contiguous().unsqueeze(-1).float()          # [T, H, 1]
    scale = np.float32(1.0 / np.sqrt(wl.head_dim))
    x = pay["dq_acc"].float() * torch.exp2(sig)                           # exact: a power of two
    want = (x * torch.tensor(scale, device=dev)).to(torch.bfloat16)      # fp32 product, then RNE
    if wl.hadamard:
        # rotated back with the forward rotation's fp32 butterflies, in its order
        from oracle.hadamard import fwht_fp32
        xs = (x * torch.tensor(scale, device=dev)).cpu().numpy().astype(np.float32)
        want = torch.from_numpy(fwht_fp32(xs)).to(torch.bfloat16).to(dev)
    assert torch.equal(call.dq, want)
