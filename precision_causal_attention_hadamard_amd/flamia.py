"""Thin Python binding of libflamia.so (ctypes).

Same names as the C ABI in ``include/flamia.h``; this module only marshals
arguments.  PyTorch supplies device memory and the stream; every step of the
call runs in the library's HIP kernels.  There is no fallback: if the
library is missing, ``load()`` raises.
"""

from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libflamia.so")

FLAMIA_OK = 0
_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported configuration",
           3: "size exceeds the library's index limits", 4: "HIP kernel launch failed"}


class FlamiaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {_STATUS.get(status, status)} (status {status})")
        self.status = status


class AttnDesc(ctypes.Structure):
    _fields_ = [("total_tokens", ctypes.c_int32), ("num_docs", ctypes.c_int32),
                ("max_doc_len", ctypes.c_int32), ("cu_seqlens", ctypes.c_void_p),
                ("num_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("causal", ctypes.c_int32), ("path", ctypes.c_int32),
                ("hadamard", ctypes.c_int32), ("causal_dq_scale", ctypes.c_int32),
                ("deterministic", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("num_kv_heads", ctypes.c_int32), ("exact", ctypes.c_int32),
                ("exp2_fma", ctypes.c_int32)]


class QTensors(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in
                ("q_codes", "k_codes", "v_codes", "v_key_codes", "q_exp", "k_exp", "v_exp",
                 "v_key_exp", "v_ref_exp", "plan", "q_fp4", "k_fp4", "q_sf", "k_sf",
                 "qk_tensor_scale", "q_fp4_bf16", "k_fp4_bf16", "k_ref_exp")]


class BwdWsOffsets(ctypes.Structure):
    _fields_ = [(name, ctypes.c_size_t) for name in ("do_codes", "do_exp", "neg_delta", "inv_l", "g", "dq_sigma",
                                                     "dq_acc")]


EXPORTS = ("flamia_buffer_sizes", "flamia_qtensors_layout", "flamia_plan_build", "flamia_quantize", "flamia_attn_fwd",
           "flamia_attn_fwd_p4", "flamia_attn_bwd", "flamia_attn_bwd_noalloc", "flamia_attn_bwd_prep", "flamia_attn_bwd_main",
           "flamia_attn_bwd_finish", "flamia_attn_fwd_diag", "flamia_attn_bwd_main_diag", "flamia_bwd_ws_layout", "flamia_tile_config", "flamia_plan_view", "flamia_status_string")

_lib = None


def load(path: str = LIB_PATH):
    """Load libflamia.so (raises when it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with precision_causal_attention_hadamard_amd/build.py")
    lib = ctypes.CDLL(path)
    P, S, I = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
    dp, qp = ctypes.POINTER(AttnDesc), ctypes.POINTER(QTensors)
    sig = {
        "flamia_buffer_sizes": [dp, ctypes.POINTER(S), ctypes.POINTER(S), ctypes.POINTER(S)],
        "flamia_qtensors_layout": [dp, P, qp],
        "flamia_plan_build": [dp, qp, P],
        "flamia_quantize": [dp, P, P, P, qp, P],
        "flamia_attn_fwd": [dp, qp, P, P, P, P, P],
        "flamia_attn_fwd_p4": [dp, qp, P, P, P, P, P],
        "flamia_attn_bwd": [dp, qp, P, P, P, P, P, P, P, P, P],
        "flamia_attn_bwd_noalloc": [dp, qp, P, P, P, P, P, P, P, P],
        "flamia_attn_bwd_prep": [dp, qp, P, P, P, P, P, P],
        "flamia_attn_bwd_main": [dp, qp, P, P, P, P],
        "flamia_attn_bwd_finish": [dp, qp, P, P, P, P],
        "flamia_attn_fwd_diag": [dp, qp, P, P, P, P, P, P, I, P],
        "flamia_attn_bwd_main_diag": [dp, qp, P, P, P, P, I, P, P],
        "flamia_bwd_ws_layout": [dp, ctypes.POINTER(BwdWsOffsets)],
        "flamia_tile_config": [I, ctypes.POINTER(I), ctypes.POINTER(I), ctypes.POINTER(I), ctypes.POINTER(I)],
        "flamia_plan_view": [dp, ctypes.POINTER(S), ctypes.POINTER(I), ctypes.POINTER(S), ctypes.POINTER(I),
                             ctypes.POINTER(S)],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.flamia_status_string.argtypes = [ctypes.c_int]
    lib.flamia_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int, where: str):
    if status != FLAMIA_OK:
        raise FlamiaError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def make_desc(cu_seqlens_dev: torch.Tensor, total_tokens: int, num_docs: int, max_doc_len: int,
              num_heads: int, head_dim: int, hadamard: bool = False, causal_dq_scale: bool = False,
              softmax_scale: float = 0.0, path: int = 0, causal: int = 1, deterministic: int = 0,
              num_kv_heads: int = 0, exact: int = 0, exp2_fma: int = 0) -> AttnDesc:
    return AttnDesc(total_tokens, num_docs, max_doc_len,
                    cu_seqlens_dev.data_ptr() if cu_seqlens_dev is not None else None,
                    num_heads, head_dim, causal, path, int(hadamard), int(causal_dq_scale),
                    deterministic, softmax_scale, num_kv_heads, exact, exp2_fma)


def buffer_sizes(desc: AttnDesc):
    q, f, b = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(load().flamia_buffer_sizes(ctypes.byref(desc), ctypes.byref(q), ctypes.byref(f), ctypes.byref(b)),
           "flamia_buffer_sizes")
    return q.value, f.value, b.value


def qtensors_layout(desc: AttnDesc, base: torch.Tensor) -> QTensors:
    qt = QTensors()
    _check(load().flamia_qtensors_layout(ctypes.byref(desc), _ptr(base), ctypes.byref(qt)),
           "flamia_qtensors_layout")
    return qt


def plan_build(desc, qt: QTensors, stream=None):
    _check(load().flamia_plan_build(ctypes.byref(desc), ctypes.byref(qt), _stream(stream)), "flamia_plan_build")


def quantize(desc, q, k, v, qt: QTensors, stream=None):
    _check(load().flamia_quantize(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), ctypes.byref(qt),
                                  _stream(stream)), "flamia_quantize")


def attn_fwd(desc, qt: QTensors, o, row_max, row_sum, ws=None, stream=None):
    _check(load().flamia_attn_fwd(ctypes.byref(desc), ctypes.byref(qt), _ptr(o), _ptr(row_max),
                                  _ptr(row_sum), _ptr(ws), _stream(stream)), "flamia_attn_fwd")


def attn_fwd_p4(desc, qt: QTensors, o, row_max, row_sum, ws=None, stream=None):
    _check(load().flamia_attn_fwd_p4(ctypes.byref(desc), ctypes.byref(qt), _ptr(o), _ptr(row_max),
                                     _ptr(row_sum), _ptr(ws), _stream(stream)), "flamia_attn_fwd_p4")


def attn_bwd(desc, qt: QTensors, o, row_max, row_sum, dout, dq, dk, dv, ws, stream=None):
    _check(load().flamia_attn_bwd(ctypes.byref(desc), ctypes.byref(qt), _ptr(o), _ptr(row_max),
                                  _ptr(row_sum), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws),
                                  _stream(stream)), "flamia_attn_bwd")


def attn_bwd_noalloc(desc, qt: QTensors, o, row_max, row_sum, dout, dq, dk, dv, stream=None):
    _check(load().flamia_attn_bwd_noalloc(ctypes.byref(desc), ctypes.byref(qt), _ptr(o), _ptr(row_max),
                                          _ptr(row_sum), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                                          _stream(stream)), "flamia_attn_bwd_noalloc")


def attn_bwd_prep(desc, qt: QTensors, o, row_max, row_sum, dout, ws, stream=None):
    _check(load().flamia_attn_bwd_prep(ctypes.byref(desc), ctypes.byref(qt), _ptr(o), _ptr(row_max),
                                       _ptr(row_sum), _ptr(dout), _ptr(ws), _stream(stream)),
           "flamia_attn_bwd_prep")


def attn_bwd_main(desc, qt: QTensors, dk, dv, ws, stream=None):
    _check(load().flamia_attn_bwd_main(ctypes.byref(desc), ctypes.byref(qt), _ptr(dk), _ptr(dv), _ptr(ws),
                                       _stream(stream)), "flamia_attn_bwd_main")


def attn_bwd_finish(desc, qt: QTensors, dq, dk, ws, stream=None):
    _check(load().flamia_attn_bwd_finish(ctypes.byref(desc), ctypes.byref(qt), _ptr(dq), _ptr(dk), _ptr(ws),
                                         _stream(stream)), "flamia_attn_bwd_finish")


def attn_fwd_diag(desc, qt: QTensors, o, row_max, row_sum, phat, phat_max, row_len: int, ws=None, stream=None):
    _check(load().flamia_attn_fwd_diag(ctypes.byref(desc), ctypes.byref(qt), _ptr(o), _ptr(row_max),
                                       _ptr(row_sum), _ptr(ws), _ptr(phat), _ptr(phat_max), row_len,
                                       _stream(stream)), "flamia_attn_fwd_diag")


def attn_bwd_main_diag(desc, qt: QTensors, dk, dv, ws, phat, row_len: int, ds_counts, stream=None):
    _check(load().flamia_attn_bwd_main_diag(ctypes.byref(desc), ctypes.byref(qt), _ptr(dk), _ptr(dv), _ptr(ws),
                                            _ptr(phat), row_len, _ptr(ds_counts), _stream(stream)),
           "flamia_attn_bwd_main_diag")


def bwd_ws_layout(desc: AttnDesc) -> BwdWsOffsets:
    out = BwdWsOffsets()
    _check(load().flamia_bwd_ws_layout(ctypes.byref(desc), ctypes.byref(out)), "flamia_bwd_ws_layout")
    return out


def tile_config(head_dim: int):
    v = [ctypes.c_int32() for _ in range(4)]
    _check(load().flamia_tile_config(head_dim, *[ctypes.byref(x) for x in v]), "flamia_tile_config")
    return tuple(x.value for x in v)


def plan_view(desc: AttnDesc):
    fo, bo, do_ = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    cf, cb = ctypes.c_int32(), ctypes.c_int32()
    _check(load().flamia_plan_view(ctypes.byref(desc), ctypes.byref(fo), ctypes.byref(cf), ctypes.byref(bo),
                                   ctypes.byref(cb), ctypes.byref(do_)), "flamia_plan_view")
    return fo.value, cf.value, bo.value, cb.value, do_.value


def status_string(status: int) -> str:
    return load().flamia_status_string(status).decode()


class TrainingCall:
    """Device buffers and the three calls of one packed attention training
    step (quantize, forward, backward).  Inputs are bf16 CUDA tensors, q and
    do ``[T, H, d]``, k and v ``[T, Hk, d]`` (Hk dividing H: grouped query
    attention when Hk < H); ``cu_seqlens`` a list of ints; ``causal`` False
    drops the j <= i mask (every key of a document is visible); ``exp2_fma``
    puts the exponentials of half of the 32 x 32 blocks on the FMA-pipe
    polynomial in both passes."""

    def __init__(self, q, k, v, do, cu_seqlens, hadamard=False, causal_dq_scale=False,
                 softmax_scale=0.0, path=0, deterministic=False, exact=False, causal=True, max_doc_len=None,
                 exp2_fma=False):
        dev = q.device
        self.q, self.k, self.v, self.do = q, k, v, do
        T, H, d = q.shape
        Hk = k.shape[1]
        self.cu_list = [int(c) for c in cu_seqlens]
        self.cu = torch.tensor(self.cu_list, dtype=torch.int32, device=dev)
        lens = [b - a for a, b in zip(self.cu_list, self.cu_list[1:])]
        mdl = (max(lens) if lens else 0) if max_doc_len is None else max_doc_len
        self.desc = make_desc(self.cu, T, len(lens), mdl, H, d, hadamard,
                              causal_dq_scale, softmax_scale, path, causal=int(causal),
                              deterministic=int(deterministic),
                              num_kv_heads=Hk, exact=int(exact), exp2_fma=int(exp2_fma))
        qb, fb, bb = buffer_sizes(self.desc)
        self.qbuf = torch.empty(qb, dtype=torch.uint8, device=dev)
        self.qt = qtensors_layout(self.desc, self.qbuf)
        self.bws = torch.empty(max(bb, 1), dtype=torch.uint8, device=dev)
        self.fws = torch.empty(fb, dtype=torch.uint8, device=dev) if fb else None
        self.o = torch.empty_like(q)
        self.row_max = torch.empty(H, T, dtype=torch.int32, device=dev)
        self.row_sum = torch.empty(H, T, dtype=torch.float32, device=dev)
        self.dq = torch.empty_like(q)
        self.dk = torch.empty_like(k)
        self.dv = torch.empty_like(v)
        self.shape = (T, H, d)
        self.kv_heads = Hk

    def quantize(self, stream=None):
        quantize(self.desc, self.q, self.k, self.v, self.qt, stream)

    def forward(self, stream=None):
        attn_fwd(self.desc, self.qt, self.o, self.row_max, self.row_sum, self.fws, stream)

    def backward(self, stream=None):
        attn_bwd(self.desc, self.qt, self.o, self.row_max, self.row_sum, self.do, self.dq, self.dk,
                 self.dv, self.bws, stream)

    def backward_staged(self, stream=None):
        attn_bwd_prep(self.desc, self.qt, self.o, self.row_max, self.row_sum, self.do, self.bws, stream)
        attn_bwd_main(self.desc, self.qt, self.dk, self.dv, self.bws, stream)
        attn_bwd_finish(self.desc, self.qt, self.dq, self.dk, self.bws, stream)

    def step(self, stream=None):
        self.quantize(stream)
        self.forward(stream)
        self.backward(stream)

    # views of the quantized payload (for tests)
    def _view(self, field: str, nbytes: int) -> torch.Tensor:
        off = getattr(self.qt, field) - self.qbuf.data_ptr()
        return self.qbuf[off:off + nbytes]

    def _heads(self, field: str) -> int:
        return self.shape[1] if field.startswith("q") else self.kv_heads

    def codes(self, field: str) -> torch.Tensor:
        T, _, d = self.shape
        H = self._heads(field)
        return self._view(field, T * H * d).view(T, H, d)

    def exps(self, field: str) -> torch.Tensor:
        T = self.shape[0]
        H = self._heads(field)
        return self._view(field, T * H).view(H, T)

    def nvfp4(self, which: str):
        """Mixed path: (packed E2M1 codes [T,H,d/2], E4M3 group-scale bytes
        [T,H,d/16], tensor scale) of 'q' or 'k'."""
        T, H, d = self.shape
        codes = self._view(f"{which}_fp4", T * H * d // 2).view(T, H, d // 2)
        sf = self._view(f"{which}_sf", T * H * d // 16).view(T, H, d // 16)
        ts = self._view("qk_tensor_scale", 16).view(torch.float32)
        return codes, sf, ts[2 if which == "q" else 3]

    def plan_lists(self):
        """(forward, backward) work lists as (doc, tile) rows, longest first."""
        fo, cf, bo, cb, _ = plan_view(self.desc)
        base = self.qt.plan - self.qbuf.data_ptr()
        raw = self.qbuf[base:base + bo + 8 * cb]
        counts = raw[:16].view(torch.int32).cpu()
        fwd = raw[fo:fo + 8 * cf].view(torch.int32).view(cf, 2).cpu()
        bwd = raw[bo:bo + 8 * cb].view(torch.int32).view(cb, 2).cpu()
        return fwd[: int(counts[0])], bwd[: int(counts[1])]

    def plan_dispatch(self):
        """The backward kernel's launch order (doc, tile), a permutation of
        the backward list grouped by document."""
        _, _, _, cb, so = plan_view(self.desc)
        base = self.qt.plan - self.qbuf.data_ptr()
        raw = self.qbuf[base:base + so + 8 * cb]
        n = int(raw[12:16].view(torch.int32).cpu()[0])
        return raw[so:so + 8 * cb].view(torch.int32).view(cb, 2).cpu()[:n]

    def bwd_payload(self):
        """What the backward's prep stage left in the workspace: dO codes
        [T,H,d], dO exponent bytes [H,T], D [H,T] (fp32), 2^-8 / l [H,T], G
        [T,H,d] (bf16), the dQ prescale exponent [H,T] (int32) and the fp16
        dQ accumulator [T,H,d] (summed by the main stage)."""
        T, H, d = self.shape
        o = bwd_ws_layout(self.desc)
        w = self.bws
        return dict(do_codes=w[o.do_codes:o.do_codes + T * H * d].view(T, H, d),
                    do_exp=w[o.do_exp:o.do_exp + T * H].view(H, T),
                    D=-w[o.neg_delta:o.neg_delta + 4 * T * H].view(torch.float32).view(H, T),
                    inv_l=w[o.inv_l:o.inv_l + 4 * T * H].view(torch.float32).view(H, T),
                    g=w[o.g:o.g + 2 * T * H * d].view(torch.bfloat16).view(T, H, d),
                    dq_sigma=w[o.dq_sigma:o.dq_sigma + 4 * T * H].view(torch.int32).view(H, T),
                    dq_acc=w[o.dq_acc:o.dq_acc + 2 * T * H * d].view(torch.float16).view(T, H, d))

    def plan_error_word(self) -> int:
        """Word 2 of the plan: 1 when deterministic mode ran out of dQ partial slots."""
        base = self.qt.plan - self.qbuf.data_ptr()
        return int(self.qbuf[base + 8:base + 12].view(torch.int32).cpu()[0])
