"""The C-ABI library on the CPU: exported symbols, metadata fields, and every
argument check (no GPU needed, no kernel is ever launched).

Every error-path call below starts from a valid call whose metadata has a
core count of 0, which the library rejects as its last check before a
launch; so even a missing check could not launch a kernel on the dummy
pointers used here.
"""

import ctypes
import json
import os
import re
import subprocess

import numpy as np
import pytest

import sparse_mla_attention_02_amd as smla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "smla.h")
PAGE = json.load(open(os.path.join(ROOT, "tests", "golden", "page_example.json")))

LIB = smla._lib
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call fails validation


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(smla_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = header_functions()
    assert {"smla_l1norm_metadata", "smla_softmax_l1norm"} <= set(names)
    lib = ctypes.CDLL(smla.library_path())
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", smla.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r" T (\w+)$", out, flags=re.M))
    assert set(names) <= exported


def test_status_codes_match_page():
    assert smla.SMLA_ERR_PARAM_NULLPTR == PAGE["error_codes"]["ACLNN_ERR_PARAM_NULLPTR"]
    assert smla.SMLA_ERR_PARAM_INVALID == PAGE["error_codes"]["ACLNN_ERR_PARAM_INVALID"]
    assert smla.SMLA_METADATA_SIZE == PAGE["metadata_size"]
    hdr = open(HEADER).read()
    for name, val in [("SMLA_ERR_PARAM_NULLPTR", 161001), ("SMLA_ERR_PARAM_INVALID", 161002),
                      ("SMLA_METADATA_SIZE", 64)]:
        assert re.search(rf"{name}\s*=?\s*{val}\b", hdr), name


def test_output_numel_page_example():
    ex = PAGE["tnd_example"]
    T1, N1, D = ex["q_shape"]
    T2, N2, _ = ex["k_shape"]
    assert LIB.smla_output_numel(1, 1, T1, N2, T2) == int(np.prod(ex["softmax_l1_norm_shape"]))
    assert LIB.smla_output_numel(0, 2, 3, 1, 5) == 30
    assert LIB.smla_output_numel(7, 1, 1, 1, 1) == -1
    assert LIB.smla_output_numel(0, -1, 1, 1, 1) == -1


def test_output_shape_helper_page_example():
    import torch
    ex = PAGE["tnd_example"]
    q = torch.empty(ex["q_shape"], device="meta")
    k = torch.empty(ex["k_shape"], device="meta")
    assert smla.output_shape(q, k, "TND") == tuple(ex["softmax_l1_norm_shape"])
    qb = torch.empty(2, 7, 16, 512, device="meta")
    kb = torch.empty(2, 9, 1, 512, device="meta")
    assert smla.output_shape(qb, kb, "BSND") == (2, 7, 1, 9)


def test_python_defaults_match_page():
    import inspect
    sig = inspect.signature(smla.sparse_flash_mla_softmax_l1_norm)
    for name, val in PAGE["attribute_defaults"].items():
        assert sig.parameters[name].default == val, name


# ---------------------------------------------------------------- metadata

def meta(**kw):
    args = dict(num_heads_q=128, num_heads_k=1, head_dim=512, batch_size=1,
                max_seqlen_q=4096, max_seqlen_k=4096, topk=2048, mask_mode=3,
                core_budget=36)
    args.update(kw)
    return smla.smla_l1norm_metadata(**args)


@pytest.mark.parametrize("total,budget", [(4096, 36), (35, 36), (36, 36), (37, 36),
                                          (100, 7), (1, 512), (8192, 512), (11536, 512)])
def test_metadata_fields_follow_page_formulas(total, budget):
    m = meta(batch_size=1, max_seqlen_q=total, core_budget=budget).numpy()
    cores = min(total, budget)
    assert m[0] == total
    assert m[4] == cores
    assert m[1] == -(-total // cores)          # ceil
    assert m[2] == total // cores              # floor
    # tail workgroups run floor(total/cores) rows, the rest ceil
    assert m[1] * (m[4] - m[3]) + m[2] * m[3] == m[0]
    assert 0 <= m[3] < max(m[4], 1)
    assert m[5] == 0x534D4C41 and m[8] == 128 and m[9] == 1 and m[10] == 512
    assert m[24] == 1                          # 128 heads, topk 2048: pipelined kernel
    assert m[25] == 4096                       # the longest key sequence (S2)
    assert (m[26:] == 0).all()


@pytest.mark.parametrize("heads,topk,variant", [(128, 2048, 1), (65, 64, 1), (64, 2048, 2),
                                                (128, 2049, 0), (1, 16, 2), (64, 5000, 2),
                                                (16, 0, 2), (100, 0, 1)])
def test_metadata_names_the_kernel_variant(heads, topk, variant):
    m = meta(num_heads_q=heads, topk=topk).numpy()
    assert m[24] == variant
    assert m[20] == (1 if heads <= 32 else 2 if heads <= 64 else 4)


def test_metadata_page_example_tnd():
    import torch
    ex = PAGE["tnd_example"]
    cq = torch.tensor([0, ex["q_shape"][0]], dtype=torch.int32)
    ck = torch.tensor([0, ex["k_shape"][0]], dtype=torch.int32)
    m = smla.smla_l1norm_metadata(
        ex["q_shape"][1], ex["k_shape"][1], ex["q_shape"][2], cu_seqlens_q=cq,
        cu_seqlens_k=ck, cmp_residual_k=torch.zeros(1, dtype=torch.int32),
        max_seqlen_q=16, max_seqlen_k=ex["max_seqlen_k"], topk=2048,
        cmp_ratio=ex["cmp_ratio"], mask_mode=ex["mask_mode"], layout_q="TND",
        layout_k="TND", core_budget=PAGE["page_max_core_num"]).numpy()
    assert tuple(m.shape) == tuple(ex["metadata_shape"])
    assert m[0] == 16 and m[4] == 16 and m[1] == 1 and m[2] == 1 and m[3] == 0
    assert m[7] == 1 and m[11] == 1 and m[17] == 16 and m[18] == 2048


def test_metadata_tnd_derives_lengths():
    import torch
    cq = torch.tensor([0, 1024, 4024, 4536, 11536], dtype=torch.int32)
    m = smla.smla_l1norm_metadata(64, 1, 512, cu_seqlens_q=cq, cu_seqlens_k=cq, topk=2048,
                                  mask_mode=3, layout_q="TND", layout_k="TND",
                                  core_budget=512).numpy()
    assert m[0] == 11536 and m[11] == 4 and m[12] == 7000 and m[13] == 7000
    assert m[17] == 11536 and m[18] == 11536 and m[20] == 2


@pytest.mark.parametrize("kw,code", [
    (dict(num_heads_k=2), 161002), (dict(num_heads_q=0), 161002),
    (dict(num_heads_q=129), 161002), (dict(head_dim=256), 161002),
    (dict(mask_mode=1), 161002), (dict(cmp_ratio=0), 161002), (dict(cmp_ratio=129), 161002),
    (dict(layout_q="TND"), 161002), (dict(layout_q="XYZ", layout_k="XYZ"), 161002),
    (dict(topk=-3), 161002), (dict(max_seqlen_q=0), 161002),
    (dict(batch_size=0), 161002), (dict(core_budget=-1), 161002),
])
def test_metadata_errors(kw, code):
    with pytest.raises(smla.SmlaError) as e:
        meta(**kw)
    assert e.value.status == code


def test_metadata_error_paths_raw():
    import torch
    m = np.zeros(64, dtype=np.int32)
    f = LIB.smla_l1norm_metadata
    # metadata pointer NULL
    assert f(128, 1, 512, None, None, None, None, None, None, 1, 8, 8, 4, 0, 0, 0, 1, 0, 36,
             None) == 161001
    # seqused given: accepted (the split does not use it)
    one = np.zeros(1, dtype=np.int32)
    assert f(128, 1, 512, None, None, one.ctypes.data, one.ctypes.data, None, None, 1, 8, 8,
             4, 0, 0, 0, 1, 0, 36, m.ctypes.data) == 0
    # TND without cu_seqlens
    assert f(128, 1, 512, None, None, None, None, None, None, 1, 0, 0, 4, 1, 1, 0, 1, 0, 36,
             m.ctypes.data) == 161001
    # cu_seqlens not starting at 0 / decreasing
    bad0 = np.array([1, 5], dtype=np.int32)
    good = np.array([0, 5], dtype=np.int32)
    assert f(128, 1, 512, bad0.ctypes.data, good.ctypes.data, None, None, None, None, 1, 0, 0,
             4, 1, 1, 0, 1, 0, 36, m.ctypes.data) == 161002
    dec = np.array([0, 5, 3], dtype=np.int32)
    assert f(128, 1, 512, dec.ctypes.data, dec.ctypes.data, None, None, None, None, 2, 0, 0,
             4, 1, 1, 0, 1, 0, 36, m.ctypes.data) == 161002
    assert b"non-decreasing" in LIB.smla_last_error()


def test_metadata_device_query_without_gpu():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    with pytest.raises(smla.SmlaError) as e:
        meta(core_budget=0)
    assert e.value.status == 561001


# ---------------------------------------------------------------- main call

def base_args(layout=0, G=128, K=2048, mask=3, ratio=1, B=1, S1=64, S2=64):
    """A call that passes every check except the final core-count check."""
    md = np.zeros(64, dtype=np.int32)
    R = B * S1 if layout == 0 else S1
    rows_k = B * S2 if layout == 0 else S2
    md[[0, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16, 17, 18, 19, 25]] = [
        R, 0, 0x534D4C41, 2, layout, G, 1, 512, B, S1, S2, K, mask, ratio, R, rows_k, 1, S2]
    a = dict(q=FAKE, k=FAKE, lse=FAKE, idx=FAKE, cu_q=None, cu_k=None, sq=None, sk=None,
             res=None, tlen=FAKE, meta=md, dtype=1, B=B, S1=S1, S2=S2, N1=G, N2=1, D=512,
             K=K, scale=0.044, maxk=0, ratio=ratio, mask=mask, lq=layout, lk=layout,
             out=FAKE, stream=None)
    if layout == 1:
        a["cu_q"] = FAKE
        a["cu_k"] = FAKE
    return a


def call(a):
    md = a["meta"]
    mp = md.ctypes.data if md is not None else None
    return LIB.smla_softmax_l1norm(
        a["q"], a["k"], a["lse"], a["idx"], a["cu_q"], a["cu_k"], a["sq"], a["sk"], a["res"],
        a["tlen"], mp, a["dtype"], a["B"], a["S1"], a["S2"], a["N1"], a["N2"], a["D"], a["K"],
        a["scale"], a["maxk"], a["ratio"], a["mask"], a["lq"], a["lk"], a["out"], a["stream"])


def test_base_call_stops_at_core_count():
    for layout in (0, 1):
        assert call(base_args(layout)) == 161002
        assert b"core count" in LIB.smla_last_error()


def _with(**kw):
    a = base_args(**{k: v for k, v in kw.items() if k in ("layout", "mask", "ratio", "G")})
    for k, v in kw.items():
        if k not in ("layout", "mask", "ratio", "G"):
            a[k] = v
    return a


@pytest.mark.parametrize("kw,code,msg", [
    (dict(q=None), 161002, b"required"), (dict(k=None), 161002, b"required"),
    (dict(lse=None), 161002, b"required"), (dict(out=None), 161002, b"required"),
    (dict(dtype=2), 161002, b"dtype"), (dict(lk=1), 161002, b"equal"),
    (dict(lq=4, lk=4), 161002, b"layout"), (dict(N2=2), 161002, b"N2"),
    (dict(N1=0), 161002, b"N1"), (dict(N1=129), 161002, b"N1"), (dict(D=256), 161002, b"512"),
    (dict(mask=1), 161002, b"mask_mode"), (dict(ratio=0), 161002, b"cmp_ratio"),
    (dict(ratio=129), 161002, b"cmp_ratio"), (dict(maxk=-1), 161002, b"max_seqlen_k"),
    (dict(sq=FAKE), 161002, b"core count"), (dict(sk=FAKE), 161002, b"core count"),
    (dict(idx=None), 161002, b"topk must be 0"), (dict(K=0), 161002, b"topk"),
    (dict(meta=None), 161001, b"metadata"),
    (dict(layout=1, cu_q=None), 161001, b"cu_seqlens"),
    (dict(layout=1, cu_k=None), 161001, b"cu_seqlens"),
    (dict(mask=3, ratio=4, res=None), 161001, b"cmp_residual_k"),
    (dict(mask=0, tlen=None), 161001, b"topk_length"),
    (dict(B=-1), 161002, b"sizes"), (dict(layout=1, B=0), 161002, b"batch_size"),
])
def test_main_call_errors(kw, code, msg):
    a = _with(**kw)
    assert call(a) == code, LIB.smla_last_error()
    assert msg in LIB.smla_last_error()


def test_dense_metadata_and_call_checks():
    # topk 0 (no sparse_indices) is the dense case: planned like any other
    m = meta(topk=0).numpy()
    assert m[14] == 0 and m[4] >= 1
    # a dense call must carry topk 0 in its metadata too
    a = base_args()
    a["idx"] = None
    a["K"] = 0
    assert call(a) == 161002
    assert b"does not match" in LIB.smla_last_error()


def test_tnd_max_seqlen_k_below_the_longest_sequence_is_rejected():
    import torch
    cu = torch.tensor([0, 5, 12], dtype=torch.int32)
    with pytest.raises(smla.SmlaError) as e:
        smla.smla_l1norm_metadata(128, 1, 512, cu_seqlens_q=cu, cu_seqlens_k=cu, batch_size=2,
                                  max_seqlen_k=6, topk=4, layout_q="TND", layout_k="TND",
                                  core_budget=64)
    assert e.value.status == 161002


@pytest.mark.parametrize("field,value", [(5, 0), (6, 9), (7, 1), (8, 64), (9, 2), (10, 128),
                                         (11, 2), (12, 65), (13, 63), (14, 16), (15, 0),
                                         (16, 2), (17, 1), (18, 1), (0, 3)])
def test_metadata_mismatch_is_rejected(field, value):
    a = base_args()
    a["meta"][field] = value
    assert call(a) == 161002
    err = LIB.smla_last_error()
    assert b"does not match" in err or b"not made by" in err, err


def test_empty_q_returns_without_looking_at_pointers():
    a = base_args(S1=0)
    for k in ("q", "k", "lse", "idx", "tlen", "out"):
        a[k] = None
    a["meta"] = None
    assert call(a) == 0
    a = base_args(layout=1, S1=0)
    for k in ("q", "k", "lse", "idx", "tlen", "out", "cu_q", "cu_k"):
        a[k] = None
    a["meta"] = None
    assert call(a) == 0
    # empty output (no keys)
    a = base_args(S2=0)
    a["meta"] = None
    assert call(a) == 0
    # still checks attributes first
    a = base_args(S1=0)
    a["N2"] = 2
    assert call(a) == 161002


# ---------------------------------------------------------------- lse call

def call_lse(a):
    md = a["meta"]
    mp = md.ctypes.data if md is not None else None
    return LIB.smla_softmax_lse(
        a["q"], a["k"], a["idx"], a["cu_q"], a["cu_k"], a["sq"], a["sk"], a["res"],
        a["tlen"], mp, a["dtype"], a["B"], a["S1"], a["S2"], a["N1"], a["N2"], a["D"], a["K"],
        a["scale"], a["maxk"], a["ratio"], a["mask"], a["lq"], a["lk"], a["out"], a["stream"])


def test_lse_call_is_declared_and_stops_at_core_count():
    assert "smla_softmax_lse" in header_functions()
    for layout in (0, 1):
        assert call_lse(base_args(layout)) == 161002
        assert b"core count" in LIB.smla_last_error()


@pytest.mark.parametrize("kw,code,msg", [
    (dict(q=None), 161002, b"required"), (dict(k=None), 161002, b"required"),
    (dict(out=None), 161002, b"required"),
    (dict(dtype=2), 161002, b"dtype"), (dict(lk=1), 161002, b"equal"),
    (dict(N2=2), 161002, b"N2"), (dict(N1=129), 161002, b"N1"), (dict(D=256), 161002, b"512"),
    (dict(mask=1), 161002, b"mask_mode"), (dict(ratio=129), 161002, b"cmp_ratio"),
    (dict(sq=FAKE), 161002, b"core count"),
    (dict(idx=None), 161002, b"topk must be 0"), (dict(K=0), 161002, b"topk"),
    (dict(meta=None), 161001, b"metadata"),
    (dict(layout=1, cu_q=None), 161001, b"cu_seqlens"),
    (dict(mask=3, ratio=4, res=None), 161001, b"cmp_residual_k"),
    (dict(mask=0, tlen=None), 161001, b"topk_length"),
])
def test_lse_call_errors(kw, code, msg):
    a = _with(**kw)
    assert call_lse(a) == code, LIB.smla_last_error()
    assert msg in LIB.smla_last_error()


def test_lse_call_checks_the_metadata_and_empty_q():
    a = base_args()
    a["meta"][14] = 16
    assert call_lse(a) == 161002
    assert b"does not match" in LIB.smla_last_error()
    a = base_args(S1=0)
    for k in ("q", "k", "idx", "tlen", "out"):
        a[k] = None
    a["meta"] = None
    assert call_lse(a) == 0
    # without keys the rows are still written (-inf), so the call goes on to
    # the metadata check
    a = base_args(layout=1, S2=0)
    a["k"] = None
    assert call_lse(a) == 161002
    assert b"core count" in LIB.smla_last_error()


# ---------------------------------------------------------------- K-wide call

def call_kwide(a):
    md = a["meta"]
    mp = md.ctypes.data if md is not None else None
    return LIB.smla_softmax_l1norm_kwide(
        a["q"], a["k"], a["lse"], a["idx"], a["cu_q"], a["cu_k"], a["sq"], a["sk"], a["res"],
        a["tlen"], mp, a["dtype"], a["B"], a["S1"], a["S2"], a["N1"], a["N2"], a["D"], a["K"],
        a["scale"], a["maxk"], a["ratio"], a["mask"], a["lq"], a["lk"], a["out"], a["stream"])


def test_kwide_call_is_declared_and_checked_like_the_main_call():
    assert "smla_softmax_l1norm_kwide" in header_functions()
    for layout in (0, 1):
        assert call_kwide(base_args(layout)) == 161002
        assert b"core count" in LIB.smla_last_error()
    for kw, code in [(dict(lse=None), 161002), (dict(out=None), 161002), (dict(N2=2), 161002),
                     (dict(meta=None), 161001), (dict(mask=0, tlen=None), 161001)]:
        assert call_kwide(_with(**kw)) == code, (kw, LIB.smla_last_error())


def test_kwide_dense_tnd_width_is_max_seqlen_k():
    # dense TND K-wide rows are max_seqlen_k wide, which must be the metadata's
    a = base_args(layout=1, K=0)
    a["idx"] = None
    a["meta"][13] = 64
    a["maxk"] = 63
    assert call_kwide(a) == 161002
    assert b"max_seqlen_k" in LIB.smla_last_error()
    a["maxk"] = 64
    assert call_kwide(a) == 161002
    assert b"core count" in LIB.smla_last_error()
    # width 0: nothing to do, no pointer looked at
    a["maxk"] = 0
    a["out"] = None
    assert call_kwide(a) == 0


# ---------------------------------------------------------------- limits

def test_metadata_rejects_sizes_past_the_32bit_offsets():
    """Key rows are addressed as key * 1024 bytes, index lists as entry * 4
    bytes and output rows as column * 4 bytes, all in 32 bits: the metadata
    call refuses what would overflow them, with SMLA_ERR_UNSUPPORTED."""
    import torch
    for kw in (dict(max_seqlen_k=(1 << 21) + 1), dict(topk=(1 << 24) + 1)):
        with pytest.raises(smla.SmlaError) as e:
            meta(**kw)
        assert e.value.status == smla.SMLA_ERR_UNSUPPORTED, kw
    # exactly 2^21 keys per sequence is still addressable
    m = meta(max_seqlen_k=1 << 21).numpy()
    assert m[25] == 1 << 21
    # TND: the longest sequence decides, not the total
    cu_q = torch.tensor([0, 3, 6], dtype=torch.int32)
    ok_k = torch.tensor([0, 1 << 20, (1 << 21) + (1 << 20)], dtype=torch.int32)
    m = smla.smla_l1norm_metadata(128, 1, 512, cu_seqlens_q=cu_q, cu_seqlens_k=ok_k,
                                  topk=16, layout_q="TND", layout_k="TND",
                                  core_budget=8).numpy()
    assert m[25] == 1 << 21 and m[18] == (1 << 21) + (1 << 20)
    bad_k = torch.tensor([0, 5, (1 << 21) + 6], dtype=torch.int32)
    with pytest.raises(smla.SmlaError) as e:
        smla.smla_l1norm_metadata(128, 1, 512, cu_seqlens_q=cu_q, cu_seqlens_k=bad_k,
                                  topk=16, layout_q="TND", layout_k="TND", core_budget=8)
    assert e.value.status == smla.SMLA_ERR_UNSUPPORTED
    assert "2097152" in str(e.value)


@pytest.mark.parametrize("kw,msg", [
    (dict(S2=0x1FFFFFFD), b"output rows"), (dict(K=(1 << 24) + 1), b"topk"),
])
def test_main_call_rejects_sizes_past_the_32bit_offsets(kw, msg):
    a = _with(**kw)
    assert call(a) == smla.SMLA_ERR_UNSUPPORTED, LIB.smla_last_error()
    assert msg in LIB.smla_last_error()


def test_main_call_checks_the_longest_key_sequence_field():
    a = base_args()
    a["meta"][4] = 1            # a valid core count: the field 25 check is the last
    a["meta"][25] = 65          # S2 is 64
    assert call(a) == 161002
    assert b"longest key sequence" in LIB.smla_last_error()


# ---------------------------------------------------------------- index check

def test_check_indices_accepts_distinct_rows_and_padding():
    idx = np.array([[3, 1, -1, -1], [0, 2, 5, -1], [7, 7, 7, 7]], dtype=np.int32)
    tl = np.array([2, 3, 1], dtype=np.int32)   # row 2 looks at one entry only
    smla.smla_check_indices(idx, tl)
    # without topk_length every entry is looked at: row 2 repeats key 7
    with pytest.raises(smla.SmlaError) as e:
        smla.smla_check_indices(idx)
    assert e.value.status == 161002 and "row 2" in str(e.value)


def test_check_indices_names_the_first_bad_row_and_entries():
    idx = np.zeros((4, 6), dtype=np.int32)
    idx[:] = np.arange(6)
    idx[1, 4] = 1                       # row 1 repeats key 1 at entries 1 and 4
    idx[3, 5] = 0
    bad = ctypes.c_int64(0)
    st = LIB.smla_check_indices(idx.ctypes.data, None, 4, 6, ctypes.byref(bad))
    assert st == 161002 and bad.value == 1
    err = LIB.smla_last_error()
    assert b"row 1" in err and b"key 1" in err and b"entries 1 and 4" in err
    # a repeat past the row's entry count is never used
    tl = np.array([6, 4, 6, 5], dtype=np.int32)
    assert LIB.smla_check_indices(idx.ctypes.data, tl.ctypes.data, 4, 6,
                                  ctypes.byref(bad)) == 0
    assert bad.value == -1
    # sizes and null pointers
    assert LIB.smla_check_indices(None, None, 0, 6, None) == 0
    assert LIB.smla_check_indices(None, None, 2, 6, None) == 161001
    assert LIB.smla_check_indices(idx.ctypes.data, None, -1, 6, None) == 161002


def test_check_indices_on_a_generated_workload():
    import workloads
    p = workloads.generate("bsnd_causal", batch=1, seqlen_q=64)
    smla.smla_check_indices(p.sparse_indices, p.topk_length)


def test_log_lines_on_stderr():
    code = ("import sparse_mla_attention_02_amd as s;"
            "s.smla_l1norm_metadata(128, 1, 512, batch_size=1, max_seqlen_q=8, "
            "max_seqlen_k=8, topk=4, core_budget=4)")
    env = dict(os.environ, SMLA_LOG="1")
    r = subprocess.run([os.sys.executable, "-c", code], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert "smla: metadata layout=BSND R=8 N1=128 K=4" in r.stderr
    assert "cores=4" in r.stderr
    env["SMLA_LOG"] = "0"
    r = subprocess.run([os.sys.executable, "-c", code], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=120)
    assert "smla:" not in r.stderr


def test_build_reads_scratch_use_from_the_compiler_remarks():
    """The build refuses pipelined kernels that the compiler gave scratch
    memory; the remark parser finds each kernel's ScratchSize line."""
    from sparse_mla_attention_02_amd import _build
    text = "\n".join([
        "a.hip:1:1: remark: Function Name: kern_a [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:1:1: remark:     VGPRs: 256 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: remark: Function Name: kern_b [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: remark:     ScratchSize [bytes/lane]: 12 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:3:9: warning: something else",
    ])
    assert _build.scratch_users(text) == [("kern_b", 12)]
    compiles, _ = _build.commands("/tmp/libx.so", "/tmp")
    guarded = {os.path.basename(c[c.index("-c") + 1]) for c in compiles
               if _build.RESOURCE_REMARKS[0] in c}
    assert guarded == _build.NO_SCRATCH
