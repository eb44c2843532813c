"""fp64 brute-force attention (torch CPU) -- the textbook routine that the
oracle's attention core must reduce to when quantization is switched off."""

import numpy as np
import torch


def causal_attention_fp64(q, k, v, do, cu_seqlens, scale=None, causal=True):
    """Per-document causal softmax attention in float64 with autograd.
    k, v may have fewer heads Hk (grouped query attention: query head h uses
    head h // (H / Hk); autograd sums the repeated heads' gradients).
    Returns O, dQ ([T, H, d]) and dK, dV ([T, Hk, d]) as float64 numpy arrays."""
    q = torch.as_tensor(np.asarray(q, np.float64))
    k = torch.as_tensor(np.asarray(k, np.float64))
    v = torch.as_tensor(np.asarray(v, np.float64))
    do = torch.as_tensor(np.asarray(do, np.float64))
    T, H, d = q.shape
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    Hk = k.shape[1]
    outs = [torch.zeros(T, h_, d, dtype=torch.float64) for h_ in (H, H, Hk, Hk)]
    for s, e in zip(cu_seqlens[:-1], cu_seqlens[1:]):
        if e == s:
            continue
        qs = q[s:e].transpose(0, 1).clone().requires_grad_(True)   # [H, L, d]
        ks = k[s:e].transpose(0, 1).clone().requires_grad_(True)   # [Hk, L, d]
        vs = v[s:e].transpose(0, 1).clone().requires_grad_(True)
        g = H // ks.shape[0]                                       # grouped query attention
        kr, vr = ks.repeat_interleave(g, dim=0), vs.repeat_interleave(g, dim=0)
        sc = (qs @ kr.transpose(1, 2)) * scale
        if causal:
            L = e - s
            mask = torch.ones(L, L, dtype=torch.bool).tril()
            sc = sc.masked_fill(~mask, float("-inf"))
        o = torch.softmax(sc, dim=-1) @ vr
        o.backward(do[s:e].transpose(0, 1))
        for dst, src in zip(outs, (o, qs.grad, ks.grad, vs.grad)):
            dst[s:e] = src.detach().transpose(0, 1)
    return [x.numpy() for x in outs]
