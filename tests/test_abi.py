"""The C-ABI library loads, exports every function include/flamia.h declares,
and rejects bad host arguments before launching anything (no GPU needed)."""

import ctypes
import os
import re

import pytest

from precision_causal_attention_hadamard_amd import flamia

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flamia.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(flamia_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return flamia.load()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 8
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(flamia.EXPORTS)


def base_desc(**kw):
    fake_cu = ctypes.c_void_p(0x1000)   # never dereferenced by host-side validation
    d = flamia.AttnDesc(256, 1, 256, fake_cu.value, 2, 64, 1, 0, 0, 0, 0, 0.0, 0)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def sizes_status(lib, d):
    q, f, b = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    return lib.flamia_buffer_sizes(ctypes.byref(d), ctypes.byref(q), ctypes.byref(f), ctypes.byref(b)), q.value, b.value


def test_buffer_sizes_valid(lib):
    st, q, b = sizes_status(lib, base_desc())
    assert st == 0
    T, H, d = 256, 2, 64
    assert q >= 4 * T * H * d + 5 * T * H           # codes + exponent bytes + plan
    assert b >= T * H * d * (1 + 2 + 2)              # dO codes, G, dQ acc
    st_m, _, b_m = sizes_status(lib, base_desc(path=1))
    assert st_m == 0 and b_m >= b + 4 * T * H * d    # the mixed path also stages fp32 dK


@pytest.mark.parametrize("field,value,want", [
    ("head_dim", 96, 1), ("head_dim", 256, 1), ("num_heads", 0, 1), ("num_docs", 0, 1),
    ("total_tokens", -1, 1), ("max_doc_len", 300, 1), ("hadamard", 2, 1),
    ("causal", 2, 1), ("deterministic", 2, 1), ("path", 7, 1),
    ("num_kv_heads", -1, 1), ("num_kv_heads", 3, 1),
])
def test_invalid_and_unsupported_descriptors(lib, field, value, want):
    st, _, _ = sizes_status(lib, base_desc(**{field: value}))
    assert st == want, (field, value, st)


def test_grouped_query_heads_validation_and_layout(lib):
    """num_kv_heads: 0 or H is MHA; a proper divisor of H shrinks the K-side
    buffers to Hk heads; a non-divisor is invalid; the mixed path takes
    grouping with one query head per backward item."""
    T, d = 256, 64
    full = sizes_status(lib, base_desc(num_heads=6))
    assert sizes_status(lib, base_desc(num_heads=6, num_kv_heads=6))[1:] == full[1:]
    assert sizes_status(lib, base_desc(num_heads=6, num_kv_heads=4))[0] == 1
    st, q, b = sizes_status(lib, base_desc(num_heads=6, num_kv_heads=2))
    # 6 backward items (3 key tiles x 2 key/value heads) are far below two per CU,
    # so each group of 3 query heads is split over 3 items whose fp32 dK and
    # dV partials need staging: the fp32 dK region (T x 6 x d, which holds the
    # 3 x T x 2 x d dK partials) and a dV region of its own
    assert st == 0 and b == full[2] + 4 * T * 6 * d + 4 * 3 * T * 2 * d
    assert full[1] - q >= 3 * T * 4 * d + 4 * T * 4   # three K-side code tensors, four exponent planes
    # the mixed path runs one query head per item: fp32 dK, dV partials of each group's 3 heads
    st_m, _, b_m = sizes_status(lib, base_desc(num_heads=6, num_kv_heads=2, path=1))
    assert st_m == 0 and b_m == sizes_status(lib, base_desc(num_heads=6, path=1))[2] + 4 * 3 * T * 2 * d
    assert sizes_status(lib, base_desc(num_heads=6, num_kv_heads=6, path=1))[0] == 0
    qt = flamia.QTensors()
    dg = base_desc(num_heads=6, num_kv_heads=2)
    assert lib.flamia_qtensors_layout(ctypes.byref(dg), ctypes.c_void_p(0x100000), ctypes.byref(qt)) == 0
    assert qt.k_codes - qt.q_codes >= T * 6 * d and qt.v_codes - qt.k_codes == T * 2 * d
    assert qt.k_exp - qt.q_exp == T * 6 and qt.v_exp - qt.k_exp == T * 2


def causal_steps(L, bq=64, bk=128):
    """(key tile, query tile) pairs of a causal document: key tile u visits query tiles 2u .. Q-1."""
    n, q = -(-L // bk), -(-L // bq)
    return sum(q - (u * bk) // bq for u in range(n))


def test_deterministic_workspace_holds_every_partition():
    """Deterministic mode adds one 64 x d fp16 slot per (step, head).  The
    host's bound must cover the causal steps of any split of T tokens into
    documents of at most max_doc_len tokens; check it against brute-force
    step counts of extreme and random splits."""
    import random
    lib = flamia.load()
    rng = random.Random(5)
    for T, M, ndocs_hint in ((256, 256, 1), (4096, 64, 64), (8192, 4096, 2), (5000, 1000, 9), (3000, 1, 3000)):
        for trial in range(6):
            if trial == 0:
                lens = [M] * (T // M) + ([T % M] if T % M else [])
            elif trial == 1:
                lens = [1] * T if T <= 4096 else [M] * (T // M) + ([T % M] if T % M else [])
            else:
                lens, left = [], T
                while left:
                    L = min(left, rng.randint(1, M))
                    lens.append(L)
                    left -= L
            d0 = base_desc(total_tokens=T, max_doc_len=M, num_docs=len(lens), num_heads=3, head_dim=64)
            d1 = base_desc(total_tokens=T, max_doc_len=M, num_docs=len(lens), num_heads=3, head_dim=64,
                           deterministic=1)
            st0, _, b0 = sizes_status(lib, d0)
            st1, _, b1 = sizes_status(lib, d1)
            assert st0 == 0 and st1 == 0
            cap_steps = (b1 - b0) // (3 * 64 * 64 * 2)
            need = sum(causal_steps(L) for L in lens)
            assert cap_steps >= need, (T, M, len(lens), cap_steps, need)
    # the bound is tight enough for long documents (within 10 % of two 4096-token documents)
    d0 = base_desc(total_tokens=8192, max_doc_len=4096, num_docs=2, num_heads=1, head_dim=128)
    d1 = base_desc(total_tokens=8192, max_doc_len=4096, num_docs=2, num_heads=1, head_dim=128, deterministic=1)
    cap = (sizes_status(lib, d1)[2] - sizes_status(lib, d0)[2]) // (64 * 128 * 2)
    assert 2 * causal_steps(4096) <= cap <= 1.1 * 2 * causal_steps(4096)


def test_under_promised_max_doc_len_leaves_too_few_slots():
    """The deterministic workspace is sized from max_doc_len, which the host
    cannot check (the lengths live on the GPU).  Promising 100 tokens for two
    2000-token documents sizes it for fewer causal steps than they need, so
    the backward must flag the overflow (the GPU test checks that the rows
    that lose a partial come out as NaN and the plan's word 2 is set)."""
    lib = flamia.load()
    def cap(M):
        d0 = base_desc(total_tokens=4000, max_doc_len=M, num_docs=2, num_heads=1, head_dim=64)
        d1 = base_desc(total_tokens=4000, max_doc_len=M, num_docs=2, num_heads=1, head_dim=64, deterministic=1)
        return (sizes_status(lib, d1)[2] - sizes_status(lib, d0)[2]) // (64 * 64 * 2)
    need = 2 * causal_steps(2000)
    assert cap(2000) >= need
    assert cap(100) < need // 2
    assert all(cap(m) <= cap(m + 100) for m in range(100, 2000, 100))      # grows with the promise


def test_null_arguments_rejected_without_launch(lib):
    assert lib.flamia_buffer_sizes(None, None, None, None) == 1
    d = base_desc(cu_seqlens=None)
    assert sizes_status(lib, d)[0] == 1
    d = base_desc()
    qt = flamia.QTensors()
    # NULL inputs / incomplete qtensors: rejected before any kernel is launched
    assert lib.flamia_quantize(ctypes.byref(d), None, None, None, ctypes.byref(qt), None) == 1
    assert lib.flamia_attn_fwd(ctypes.byref(d), ctypes.byref(qt), None, None, None, None, None) == 1
    assert lib.flamia_attn_bwd(ctypes.byref(d), ctypes.byref(qt), *([None] * 9)) == 1
    assert lib.flamia_attn_bwd_main(ctypes.byref(d), ctypes.byref(qt), None, None, None, None) == 1
    assert lib.flamia_attn_bwd_finish(ctypes.byref(d), None, None, None, None, None) == 1


def test_layout_alignment_and_carving(lib):
    d = base_desc()
    qt = flamia.QTensors()
    assert lib.flamia_qtensors_layout(ctypes.byref(d), ctypes.c_void_p(0x10010), ctypes.byref(qt)) == 1
    assert lib.flamia_qtensors_layout(ctypes.byref(d), ctypes.c_void_p(0x100000), ctypes.byref(qt)) == 0
    ptrs = [getattr(qt, f) for f, _ in flamia.QTensors._fields_ if getattr(qt, f)]
    assert all(p % 256 == 0 for p in ptrs) and len(set(ptrs)) == len(ptrs) == 10
    assert qt.k_codes - qt.q_codes >= 256 * 2 * 64
    assert not qt.q_fp4 and not qt.qk_tensor_scale          # MXFP8 path: no NVFP4 operands
    # the mixed path carves the NVFP4 operands too, and needs a bigger buffer
    d1 = base_desc(path=1)
    qt1 = flamia.QTensors()
    assert lib.flamia_qtensors_layout(ctypes.byref(d1), ctypes.c_void_p(0x100000), ctypes.byref(qt1)) == 0
    ptrs1 = [getattr(qt1, f) for f, _ in flamia.QTensors._fields_ if f != "k_ref_exp"]
    assert all(ptrs1) and len(set(ptrs1)) == len(ptrs1) and not qt1.k_ref_exp
    # the exact option adds K's in-block prefix maximum, [H, T] bytes
    de = base_desc(exact=1)
    qte = flamia.QTensors()
    assert lib.flamia_qtensors_layout(ctypes.byref(de), ctypes.c_void_p(0x100000), ctypes.byref(qte)) == 0
    assert qte.k_ref_exp and qte.k_ref_exp % 256 == 0 and qte.k_ref_exp not in ptrs
    assert sizes_status(lib, de)[1] >= sizes_status(lib, d)[1] + 256 * 2
    assert sizes_status(lib, base_desc(exact=1, path=1))[0] == 2
    assert sizes_status(lib, base_desc(exact=1, num_heads=4, num_kv_heads=2))[0] == 0
    assert sizes_status(lib, base_desc(exact=2))[0] == 1
    assert sizes_status(lib, d1)[1] >= sizes_status(lib, d)[1] + 256 * 2 * 64 * (2 * 0.5 + 2 / 16)


def test_tile_config_and_status_strings(lib):
    assert flamia.tile_config(128) == (128, 64, 64, 128)
    assert flamia.tile_config(64) == (128, 64, 64, 128)
    with pytest.raises(flamia.FlamiaError):
        flamia.tile_config(32)
    for s in range(5):
        assert flamia.status_string(s)
    assert flamia.status_string(99) == "unknown status"


def test_large_worklists_get_a_key_area_and_launch_limits_are_reported(lib):
    """Lists beyond one workgroup's LDS sort (8192 tiles of 128 tokens) take
    the multi-workgroup path, whose padded keys (two buffers of the three
    lists, rounded up to runs of 2048) live in the plan; a call whose launches
    would exceed 32-bit work-item counts is reported, not launched."""
    def plan_bytes(d):
        off, cap, boff, bcap = ctypes.c_size_t(), ctypes.c_int32(), ctypes.c_size_t(), ctypes.c_int32()
        doff = ctypes.c_size_t()
        assert lib.flamia_plan_view(ctypes.byref(d), ctypes.byref(off), ctypes.byref(cap),
                                    ctypes.byref(boff), ctypes.byref(bcap), ctypes.byref(doff)) == 0
        assert doff.value >= boff.value + 8 * bcap.value        # the dispatch list follows the backward list
        return cap.value, bcap.value
    small = base_desc(total_tokens=8192 * 128 - 128, max_doc_len=8192 * 128 - 128, num_docs=1)
    big = base_desc(total_tokens=1 << 20, max_doc_len=1 << 20, num_docs=1)
    many = base_desc(total_tokens=131072, max_doc_len=1, num_docs=131072)
    st_s, q_s, _ = sizes_status(lib, small)
    st_b, q_b, _ = sizes_status(lib, big)
    st_m, q_m, _ = sizes_status(lib, many)
    assert st_s == st_b == st_m == 0
    assert plan_bytes(small) == (8192, 8192) and plan_bytes(big) == (8193, 8193)
    assert plan_bytes(many) == (132096, 132096)
    runs = -(-132096 // 2048) * 2048
    assert q_m >= 6 * 8 * runs
    # codes grow by 4 bytes per element, the key area by 6 x 8 bytes per padded slot
    assert q_b - q_s >= 4 * 128 * 2 * 64 + 6 * 8 * 10240
    huge = base_desc(total_tokens=(1 << 23), max_doc_len=1, num_docs=(1 << 23), head_dim=64)
    assert sizes_status(lib, huge)[0] == 3


def test_noncausal_descriptor_rules(lib):
    """causal = 0 is accepted on both paths (also grouped and deterministic);
    the causal dQ prescale and the exact option, both defined by which keys a
    query may see, are invalid without the mask."""
    assert sizes_status(lib, base_desc(causal=0))[0] == 0
    assert sizes_status(lib, base_desc(causal=0, deterministic=1))[0] == 0
    assert sizes_status(lib, base_desc(causal=0, num_heads=4, num_kv_heads=2))[0] == 0
    assert sizes_status(lib, base_desc(causal=0, causal_dq_scale=1))[0] == 1
    assert sizes_status(lib, base_desc(causal=0, exact=1))[0] == 1
    assert sizes_status(lib, base_desc(causal=0, path=1))[0] == 0


def test_exp2_fma_descriptor_rules(lib):
    """exp2_fma is 0 or 1; 1 is built for the default MXFP8 call only (causal,
    one key/value head per query head, atomic dQ, no exact option)."""
    assert sizes_status(lib, base_desc(exp2_fma=1))[0] == 0
    assert sizes_status(lib, base_desc(exp2_fma=1, hadamard=1, causal_dq_scale=1))[0] == 0
    assert sizes_status(lib, base_desc(exp2_fma=2))[0] == 1
    assert sizes_status(lib, base_desc(exp2_fma=-1))[0] == 1
    for kw in (dict(path=1), dict(exact=1), dict(causal=0), dict(deterministic=1),
               dict(num_heads=4, num_kv_heads=2)):
        assert sizes_status(lib, base_desc(exp2_fma=1, **kw))[0] == 2, kw
    # the layouts do not depend on it
    assert sizes_status(lib, base_desc(exp2_fma=1))[1:] == sizes_status(lib, base_desc())[1:]


def noncausal_steps(L, bq=64, bk=128):
    """Every key tile of a document visits every query tile without the mask."""
    return (-(-L // bk)) * (-(-L // bq))


def test_noncausal_deterministic_workspace_bound():
    import random
    lib = flamia.load()
    rng = random.Random(6)
    for T, M in ((256, 256), (4096, 64), (8192, 4096), (5000, 1000), (3000, 1), (1000, 129)):
        for trial in range(5):
            if trial == 0:
                lens = [M] * (T // M) + ([T % M] if T % M else [])
            else:
                lens, left = [], T
                while left:
                    L = min(left, rng.randint(1, M))
                    lens.append(L)
                    left -= L
            kw = dict(total_tokens=T, max_doc_len=M, num_docs=len(lens), num_heads=3, head_dim=64, causal=0)
            st0, _, b0 = sizes_status(lib, base_desc(**kw))
            st1, _, b1 = sizes_status(lib, base_desc(deterministic=1, **kw))
            assert st0 == 0 and st1 == 0
            cap_steps = (b1 - b0) // (3 * 64 * 64 * 2)
            need = sum(noncausal_steps(L) for L in lens)
            assert cap_steps >= need, (T, M, len(lens), cap_steps, need)
