"""Forward/backward consistency and the dS zero fraction on the GPU
([Summary, §3.3 Forward-Backward Numerical Consistency]; its second bullet
for the dS blocks), through the diagnostic entry points.

* The backward recomputes the probability codes the forward produced: for
  every (query, key) pair the query sees, the forward's E4M3 code of
  P 2^8 (times the diagonal fold), taken against the running integer row
  maximum of its key step and rescaled by 2^(running - final maximum), equals
  the backward's code taken against the stored final maximum wherever both
  lie in E4M3's normal range (P 2^8 f >= 2^-6, i.e. P f >= 2^-14).  Below it
  the two may differ (a rescale by a power of two moves subnormal codes, and
  a value just under 2^-6 can round up to 2^-6 on the final scale's
  subnormal grid); the count is reported.
* The diagnostic calls give the plain calls' results bit for bit (dK, dV; O,
  the row statistics) and dQ within atomic-order noise.
* The GPU's fraction of nonzero dS whose E4M3 code is zero agrees with the
  oracle's to within the few codes decisions can move.
"""

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import formats
from precision_causal_attention_hadamard_amd import workloads as W

pytestmark = pytest.mark.gpu

CASES = {
    "tiny_config1": lambda: W.config(1),
    "ragged_d64_h3": lambda: W.small_packed(31, [1, 17, 45, 100, 33, 64, 130, 2], heads=3, head_dim=64),
    "hadamard_outliers_d128": lambda: W.small_packed(32, [300, 211], heads=2, head_dim=128,
                                                     outlier_scale=20.0, hadamard=True),
    "long_d128_h2": lambda: W.small_packed(95, [1500, 700], heads=2, head_dim=128),
    # row maxima near +150 and -150 (both probability forms, both passes)
    "extreme_rows_d128": lambda: W.extreme_rows(3, [230, 100], head_dim=128),
}

E4M3_VALUES = formats.e4m3_decode(np.arange(256, dtype=np.uint8))


def run_diag(lib, wl, **kw):
    dev = torch.device("cuda")
    q, k, v, do = (t.to(dev) for t in (wl.q, wl.k, wl.v, wl.do))
    call = lib.TrainingCall(q, k, v, do, wl.cu_seqlens, hadamard=wl.hadamard, **kw)
    T, H, d = call.shape
    Lmax = max(wl.doc_lens)
    nkt = -(-Lmax // 64)
    fwd = torch.full((H, T, Lmax), 0xFF, dtype=torch.uint8, device=dev)       # 0xFF: never a P^ code (NaN)
    fmax = torch.full((H, T, nkt), -(1 << 30), dtype=torch.int32, device=dev)
    bwd = torch.full((H, T, Lmax), 0xFF, dtype=torch.uint8, device=dev)
    counts = torch.zeros(2, dtype=torch.int64, device=dev)
    call.quantize()
    lib.attn_fwd_diag(call.desc, call.qt, call.o, call.row_max, call.row_sum, fwd, fmax, Lmax)
    lib.attn_bwd_prep(call.desc, call.qt, call.o, call.row_max, call.row_sum, call.do, call.bws)
    lib.attn_bwd_main_diag(call.desc, call.qt, call.dk, call.dv, call.bws, bwd, Lmax, counts)
    lib.attn_bwd_finish(call.desc, call.qt, call.dq, call.dk, call.bws)
    torch.cuda.synchronize()
    return call, fwd.cpu().numpy(), fmax.cpu().numpy(), bwd.cpu().numpy(), counts.cpu().numpy()


def check_replay(wl, call, fwd, fmax, bwd, case):
    """Every visible pair written by both kernels, none of the masked ones;
    the codes equal in E4M3's normal range.  Returns (checked, below,
    differ_below)."""
    m_final = call.row_max.cpu().numpy().astype(np.int64)
    checked = below = differ_below = 0
    for s, e in zip(wl.cu_seqlens[:-1], wl.cu_seqlens[1:]):
        L = e - s
        if L == 0:
            continue
        i = np.arange(L)
        vis = i[None, :] <= i[:, None]                      # query i sees key j <= i
        kt = np.arange(L) // 64
        for h in range(wl.heads):
            cf, cb = fwd[h, s:e, :L], bwd[h, s:e, :L]
            assert np.all(cf[vis] != 0xFF) and np.all(cb[vis] != 0xFF), "a visible pair was not written"
            assert np.all(cf[~vis] == 0xFF) and np.all(cb[~vis] == 0xFF), "a masked pair was written"
            run = fmax[h, s:e][:, kt].astype(np.int64)       # running max of each key's step
            shift = run - m_final[h, s:e][:, None]           # <= 0
            assert np.all(shift[vis] <= 0)
            vf = np.ldexp(E4M3_VALUES[cf].astype(np.float64), shift)
            vb = E4M3_VALUES[cb].astype(np.float64)
            # in E4M3's normal range at both maxima (a value just below 2^-6 can
            # round up to 2^-6 on the final scale's subnormal grid: excluded)
            normal = vis & (np.abs(vb) >= 2.0 ** -6) & (np.abs(vf) >= 2.0 ** -6)
            np.testing.assert_array_equal(vf[normal], vb[normal], err_msg=f"{case} head {h} doc at {s}")
            checked += int(normal.sum())
            sub = vis & ~normal
            below += int(sub.sum())
            differ_below += int(np.count_nonzero(vf[sub] != vb[sub]))
    return checked, below, differ_below


@pytest.mark.parametrize("case", list(CASES))
def test_backward_replays_forward_codes(gpu_lib, case):
    wl = CASES[case]()
    print(f"[diag] {case}", flush=True)
    call, fwd, fmax, bwd, counts = run_diag(gpu_lib, wl)
    checked, below, differ_below = check_replay(wl, call, fwd, fmax, bwd, case)
    print(f"[diag] {case}: {checked} codes in the normal range equal; {differ_below} of {below} below it differ",
          flush=True)
    assert checked > 0


@pytest.mark.parametrize("case", ["ragged_d64_h3", "hadamard_outliers_d128", "extreme_rows_d128"])
def test_diag_calls_give_the_plain_results(gpu_lib, case):
    wl = CASES[case]()
    call, *_ = run_diag(gpu_lib, wl)
    got = {n: getattr(call, n).clone() for n in ("o", "dk", "dv", "dq", "row_max", "row_sum")}
    call.step()
    torch.cuda.synchronize()
    for n in ("o", "dk", "dv", "row_max", "row_sum"):
        assert torch.equal(got[n], getattr(call, n)), n
    a, b = got["dq"].float(), call.dq.float()
    assert float((a - b).abs().max() / b.abs().max()) <= 2e-3


@pytest.mark.parametrize("case", ["tiny_config1", "hadamard_outliers_d128", "long_d128_h2"])
def test_ds_zero_fraction_matches_oracle(gpu_lib, case):
    wl = CASES[case]()
    call, *_, counts = run_diag(gpu_lib, wl)
    q, k, v, do = [t.float().numpy().astype(np.float64) for t in (wl.q, wl.k, wl.v, wl.do)]
    ref = A.training_call(q, k, v, do, wl.cu_seqlens, A.Numerics(hadamard=wl.hadamard))
    nz, zero = int(counts[0]), int(counts[1])
    frac = zero / nz
    print(f"[diag] {case}: GPU dS zero fraction {frac:.5f} ({zero} of {nz} nonzero dS), "
          f"oracle {ref['ds_zero_fraction']:.5f}", flush=True)
    pairs = sum(L * (L + 1) // 2 for L in wl.doc_lens) * wl.heads
    assert 0.97 * pairs <= nz <= pairs               # almost every visible dS is nonzero
    assert abs(frac - ref["ds_zero_fraction"]) <= 2e-3
