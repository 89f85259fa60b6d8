"""libqsa.so loads, exports what include/qsa.h declares, and rejects calls
outside the packed-decode contract on the host (no GPU needed: validation
reads descriptors only and runs before any HIP call).

Contract: page "fix(qsa): restore SM121 correctness with Humanize and Kernel
Design Agent", section "Changes" -- bf16, head dim 256, 12:1 GQA as
24Q/2KV or 12Q/1KV, 1 <= bs <= 128, unsupported calls fail with a
descriptive error.
"""
import ctypes
import os
import re
import subprocess

import pytest

import sparse_index_paged_amd as qsa
from sparse_index_paged_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qsa.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qsa_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = qsa.load_library()
    declared = _declared_functions()
    assert "qsa_decode" in declared and len(declared) >= 10
    for name in declared:
        assert hasattr(lib, name), f"{name} declared in qsa.h but not exported"
    assert set(declared) == set(B.EXPORTS)
    nm = subprocess.run(["nm", "-D", "--defined-only", qsa.lib_path()], capture_output=True,
                        text=True, check=True).stdout
    exported = set(re.findall(r"\bT (qsa_\w+)", nm))
    assert exported == set(declared)


def test_header_compiles_as_c():
    src = "#include \"qsa.h\"\nint main(void) { return qsa_abi_version() != QSA_ABI_VERSION; }\n"
    res = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", "-I",
                          os.path.join(ROOT, "include"), "-x", "c", "-"], input=src, text=True,
                         capture_output=True)
    assert res.returncode == 0, res.stderr


def test_abi_version():
    assert qsa.abi_version() == B.ABI_VERSION == 5


def test_plan_and_options():
    assert qsa.get_option("split_target") == 0          # cost model
    # one workgroup per CU when the pairs fill the chip; below that, splits
    # until the gather is bound by HBM, weighed against the merge per split
    assert qsa.plan(128, 2) == (1, 256)
    assert qsa.plan(64, 2) == (2, 256)
    assert qsa.plan(32, 2) == (3, 192)        # HBM-bound already at 3 splits: more only add merge
    assert qsa.plan(16, 1) == (9, 144)         # at most ceil(2055 / 256) splits are ever active
    assert qsa.plan(17, 2) == (5, 200)         # 5 pairs x 5 splits = 25 workgroups on the busiest XCD
    assert qsa.plan(85, 2) == (1, 176)         # 22 pairs per XCD: unsplit beats a second workgroup per CU
    assert qsa.plan(48, 2) == (2, 192)
    assert qsa.plan(96, 2) == (1, 192)
    assert qsa.plan(96, 1) == (2, 192)
    for bs in range(1, 129):
        for hkv in (1, 2):
            s, w = qsa.plan(bs, hkv)
            assert 1 <= s <= 9 and w == ((bs * hkv + 7) // 8) * 8 * s
    # all splits of pair p run on XCD p % 8 (32 CUs each): no plan puts more
    # than two workgroups on a CU of the busiest XCD
    for bs in range(1, 129):
        for hkv in (1, 2):
            s, _ = qsa.plan(bs, hkv)
            assert -(-bs * hkv // 8) * s <= 2 * 32, (bs, hkv, s)
    # the cap follows min_split_keys: with 128 keys per split up to 16 can be
    # active, and a single row then takes more than 9
    qsa.set_option("min_split_keys", 128)
    try:
        assert 9 < qsa.plan(1, 2)[0] <= 16
    finally:
        qsa.set_option("min_split_keys", 256)
    # "splits" fixes the split count (bounded by max_splits)
    qsa.set_option("splits", 5)
    try:
        assert qsa.plan(128, 2) == (5, 1280)
        assert qsa.get_option("splits") == 5
    finally:
        qsa.set_option("splits", 0)
    assert qsa.plan(128, 2) == (1, 256)
    with pytest.raises(qsa.QsaError, match="unknown option"):
        qsa.set_option("nope", 3)
    with pytest.raises(qsa.QsaError, match="bs must be"):
        qsa.plan(0, 2)
    qsa.set_option("split_target", 2048)
    try:
        assert qsa.plan(128, 2)[0] == 8
    finally:
        qsa.set_option("split_target", 0)
    # placement of bf16 workgroups by their XCD: on (1, the default) or off (0)
    assert qsa.get_option("xcc_lanes") == 1
    qsa.set_option("xcc_lanes", 0)
    try:
        assert qsa.get_option("xcc_lanes") == 0
    finally:
        qsa.set_option("xcc_lanes", 1)
    with pytest.raises(qsa.QsaError, match="xcc_lanes must be 0 or 1"):
        qsa.set_option("xcc_lanes", 2)


# ---- contract rejection with fake (never dereferenced) device pointers ----

FAKE = 1 << 20  # 16-byte aligned, never dereferenced on the host


def _t(shape, dtype, strides=None, data=FAKE):
    d = B.QsaTensor()
    d.data = data
    d.dtype = dtype
    d.ndim = len(shape)
    if strides is None:
        strides, acc = [], 1
        for n in reversed(shape):
            strides.insert(0, acc)
            acc *= n
    for i, (n, s) in enumerate(zip(shape, strides)):
        d.shape[i] = n
        d.stride[i] = s
    return d


def _call(bs=4, hq=24, hkv=2, d=256, slots=64, pool_dtype=B.BF16, v_dtype=None, scales=None,
          q_dtype=B.BF16, cu_len=None, pool_data=FAKE, q_strides=None, out_shape=None,
          lse_shape=None, sel_dtype=B.I32, pool_strides=None, out_data=FAKE, out_strides=None):
    lib = qsa.load_library()
    row = d if pool_dtype != B.U4X2 else d // 2
    q = _t((bs, hq, d), q_dtype, q_strides)
    k = _t((slots, hkv, row), pool_dtype, pool_strides, data=pool_data)
    v = _t((slots, hkv, row), v_dtype or pool_dtype, pool_strides)
    sel = _t((100,), sel_dtype)
    cu = _t(((cu_len if cu_len is not None else bs + 1),), B.I32)
    out = _t(out_shape or (bs, hq, d), B.BF16, out_strides, data=out_data)
    lse = _t(lse_shape or (bs, hq), B.F32)
    st = lib.qsa_decode(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v),
                        ctypes.byref(scales) if scales is not None else None, ctypes.byref(sel),
                        ctypes.byref(cu), ctypes.byref(out), ctypes.byref(lse), None)
    return st, lib.qsa_last_error().decode()


def _scales(slots=64, hkv=2, group=256, dtype=B.F32):
    return B.QsaKvScales(_t((slots, hkv, 256 // group), dtype), _t((slots, hkv, 256 // group), dtype),
                         group)


@pytest.mark.parametrize("kwargs,match", [
    (dict(d=128), "head dim must be 256"),
    (dict(bs=129), r"bs must be in \[1, 128\]"),
    (dict(hq=16), r"\(Hq, Hkv\) must be \(24, 2\) or \(12, 1\)"),
    (dict(hq=12, hkv=2), r"\(Hq, Hkv\)"),
    (dict(hq=24, hkv=1), r"\(Hq, Hkv\)"),
    (dict(q_dtype=B.F16), "q must be bf16"),
    (dict(pool_dtype=B.F32), "is not bf16, fp8_e4m3fn, i8 or u4x2"),
    (dict(pool_dtype=B.I8, v_dtype=B.FP8_E4M3FN, scales=None), "must share a format"),
    (dict(pool_dtype=B.I8), "pools need kv_scales"),
    (dict(scales="bf16"), "take no scales"),
    (dict(pool_dtype=B.I8, scales="g48"), "group_size 48 is not supported"),
    (dict(pool_dtype=B.U4X2, scales="g256"), "group_size 256 is not supported"),
    (dict(pool_dtype=B.I8, scales="bf16s"), "k_scale must be f32 or f16"),
    (dict(cu_len=3), "cu_seqlens must have bs \\+ 1"),
    (dict(pool_data=FAKE + 8), "16-byte boundaries"),
    (dict(q_strides=(24 * 256, 256, 2)), "contiguous in its last dimension"),
    (dict(out_shape=(4, 24, 128)), "out must be"),
    (dict(out_data=FAKE + 8), "out rows must start on 16-byte boundaries"),
    (dict(out_strides=(24 * 260, 260, 1)), "out rows must start on 16-byte boundaries"),
    (dict(lse_shape=(4, 12)), "lse must be"),
    (dict(sel_dtype=B.F32), "sel_indices must be i32"),
])
def test_contract_rejections(kwargs, match):
    sc = kwargs.pop("scales", None)
    if sc == "bf16":
        kwargs["scales"] = _scales()
    elif sc == "g48":
        kwargs["scales"] = B.QsaKvScales(_t((64, 2, 5), B.F32), _t((64, 2, 5), B.F32), 48)
    elif sc == "g256":
        kwargs["scales"] = _scales(group=256)
    elif sc == "bf16s":
        kwargs["scales"] = _scales(dtype=B.BF16)
    st, msg = _call(**kwargs)
    assert st == 1, (st, msg)
    assert re.search(match, msg), msg


def test_null_arguments_are_arg_errors():
    lib = qsa.load_library()
    st = lib.qsa_decode(None, None, None, None, None, None, None, None, None)
    assert st == 2
    assert "q is NULL" in lib.qsa_last_error().decode()


def test_workspace_calls_without_a_device():
    """Without a HIP device the workspace calls fail cleanly (nothing is
    launched); with none attached there is nothing to free or count."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a HIP device is present")
    lib = qsa.load_library()
    for name in ("qsa_workspace_attach", "qsa_workspace_detach"):
        assert getattr(lib, name)(None) == 4
        assert "no HIP device" in lib.qsa_last_error().decode()
    assert lib.qsa_workspace_bytes() == 0
    assert lib.qsa_workspace_release() == 0
    ptr, n = ctypes.c_void_p(), ctypes.c_int()
    assert lib.qsa_debug_counters(ctypes.byref(ptr), ctypes.byref(n), None) == 4


def _store(n=8, hkv=2, slots=64, pool_dtype=B.BF16, scales=None, new_dtype=B.BF16,
           new_shape=None, loc_dtype=B.I32, loc_len=None, new_data=FAKE, new_strides=None,
           v_pool_shape=None):
    lib = qsa.load_library()
    row = 256 if pool_dtype != B.U4X2 else 128
    k_new = _t(new_shape or (n, hkv, 256), new_dtype, new_strides, data=new_data)
    v_new = _t(new_shape or (n, hkv, 256), new_dtype, new_strides)
    loc = _t((n if loc_len is None else loc_len,), loc_dtype)
    kp = _t((slots, hkv, row), pool_dtype)
    vp = _t(v_pool_shape or (slots, hkv, row), pool_dtype)
    st = lib.qsa_kv_store(ctypes.byref(k_new), ctypes.byref(v_new), ctypes.byref(loc),
                          ctypes.byref(kp), ctypes.byref(vp),
                          ctypes.byref(scales) if scales is not None else None, None)
    return st, lib.qsa_last_error().decode()


@pytest.mark.parametrize("kwargs,match", [
    (dict(new_dtype=B.F32), "k_new must be bf16"),
    (dict(new_shape=(8, 1, 256)), r"k_new and v_new must be \[n, Hkv, 256\]"),
    (dict(new_shape=(8, 2, 128)), r"k_new and v_new must be \[n, Hkv, 256\]"),
    (dict(loc_dtype=B.F32), "loc must be i32 or i64"),
    (dict(loc_len=7), "loc must have n = 8 entries"),
    (dict(new_data=FAKE + 8), "rows must start on 16-byte boundaries"),
    (dict(new_strides=(2 * 260, 260, 1)), "rows must start on 16-byte boundaries"),
    (dict(pool_dtype=B.I8), "qsa_kv_store: i8 pools need kv_scales"),
    (dict(scales="g256"), "qsa_kv_store: bf16 pools take no scales"),
    (dict(pool_dtype=B.U4X2, scales="g256"), "group_size 256 is not supported"),
    (dict(pool_dtype=B.I8, scales="bf16s"), "k_scale must be f32 or f16"),
    (dict(v_pool_shape=(32, 2, 256)), "k_pool and v_pool shapes differ"),
    (dict(hkv=3), "pools must hold 1 or 2 KV heads"),
])
def test_store_contract_rejections(kwargs, match):
    sc = kwargs.pop("scales", None)
    if sc == "g256":
        kwargs["scales"] = _scales(group=256)
    elif sc == "bf16s":
        kwargs["scales"] = _scales(dtype=B.BF16)
    st, msg = _store(**kwargs)
    assert st == 1, (st, msg)
    assert re.search(match, msg), msg


# ---- tiered pool (int8 ring + int4 pool) ----

def _tiered(r=64, slots=256, hkv=2, ring_dtype=B.I8, cold_dtype=B.U4X2, scale_dtype=B.F16,
            ring_scale_groups=4, cold_scale_groups=8, owner_len=None, claim_len=None,
            claim_dtype=B.I32, ring_data=FAKE, cold_hkv=None):
    ch = cold_hkv or hkv
    return B.QsaTieredPool(
        _t((r, hkv, 256), ring_dtype, data=ring_data), _t((r, hkv, 256), ring_dtype),
        _t((r, hkv, ring_scale_groups), scale_dtype), _t((r, hkv, ring_scale_groups), scale_dtype),
        _t((owner_len or r,), B.I32), _t((claim_len or r,), claim_dtype),
        _t((slots, ch, 128), cold_dtype), _t((slots, ch, 128), cold_dtype),
        _t((slots, ch, cold_scale_groups), scale_dtype),
        _t((slots, ch, cold_scale_groups), scale_dtype))


def _decode_tiered(pool, bs=4, hq=24):
    lib = qsa.load_library()
    q = _t((bs, hq, 256), B.BF16)
    sel = _t((100,), B.I32)
    cu = _t((bs + 1,), B.I32)
    out = _t((bs, hq, 256), B.BF16)
    lse = _t((bs, hq), B.F32)
    st = lib.qsa_decode_tiered(ctypes.byref(q), ctypes.byref(pool), ctypes.byref(sel),
                               ctypes.byref(cu), ctypes.byref(out), ctypes.byref(lse), None)
    return st, lib.qsa_last_error().decode()


def _store_tiered(pool, n=8, hkv=2):
    lib = qsa.load_library()
    k_new = _t((n, hkv, 256), B.BF16)
    v_new = _t((n, hkv, 256), B.BF16)
    loc = _t((n,), B.I32)
    st = lib.qsa_kv_store_tiered(ctypes.byref(k_new), ctypes.byref(v_new), ctypes.byref(loc),
                                 ctypes.byref(pool), None)
    return st, lib.qsa_last_error().decode()


@pytest.mark.parametrize("kwargs,match", [
    (dict(r=48), "power of two rows"),
    (dict(ring_dtype=B.FP8_E4M3FN), "ring_k / ring_v must be i8"),
    (dict(cold_dtype=B.I8), "cold_k / cold_v must be u4x2"),
    (dict(scale_dtype=B.F32), "tiered pool scales must be f16"),
    (dict(ring_scale_groups=8), r"scales must be \[slots, Hkv, 256/group\]"),
    (dict(cold_scale_groups=4), r"scales must be \[slots, Hkv, 256/group\]"),
    (dict(owner_len=32), "owner must have one entry per ring row"),
    (dict(ring_data=FAKE + 8), "16-byte boundaries"),
    (dict(hkv=2, cold_hkv=1), "different KV head counts"),
])
def test_tiered_contract_rejections(kwargs, match):
    st, msg = _decode_tiered(_tiered(**kwargs))
    assert st == 1, (st, msg)
    assert re.search(match, msg), msg
    assert msg.startswith("qsa_decode_tiered")


@pytest.mark.parametrize("kwargs,match", [
    (dict(claim_len=32), "claim must have one entry per ring row"),
    (dict(claim_dtype=B.I64), "claim must be i32"),
    (dict(r=12), "power of two rows"),
])
def test_tiered_store_contract_rejections(kwargs, match):
    st, msg = _store_tiered(_tiered(**kwargs))
    assert st == 1, (st, msg)
    assert re.search(match, msg), msg
    assert msg.startswith("qsa_kv_store_tiered")


def test_tiered_query_and_store_shape_rejections():
    st, msg = _decode_tiered(_tiered(hkv=1), hq=24)
    assert st == 1 and re.search(r"\(Hq, Hkv\)", msg), msg
    st, msg = _store_tiered(_tiered(hkv=2), hkv=1)
    assert st == 1 and "k_new and v_new must be [n, Hkv, 256]" in msg, msg
    lib = qsa.load_library()
    assert lib.qsa_decode_tiered(None, None, None, None, None, None, None) == 2
    assert "q is NULL" in lib.qsa_last_error().decode()
    assert lib.qsa_kv_store_tiered(None, None, None, None, None) == 2
    assert "pool is NULL" in lib.qsa_last_error().decode()


# ---- indexer ----

def _index(bs=2, hi=4, di=64, n_k=100, max_blocks=32, max_tokens=128, budget=64, c=4,
           q_dtype=B.BF16, weights="f32", sel_len=None, cu_len=None, k_di=None, bt_rows=None,
           q_data=FAKE):
    lib = qsa.load_library()
    q = _t((bs, hi, di), q_dtype, data=q_data)
    w = _t((bs, hi), B.F32 if weights == "f32" else B.BF16) if weights else None
    k = _t((n_k, k_di or di), B.BF16)
    bt = _t((bt_rows or bs, max_blocks), B.I32)
    r2t = _t((bs, max_tokens), B.I32)
    cl = _t((bs,), B.I32)
    sel = _t((sel_len if sel_len is not None else bs * (budget + c - 1),), B.I32)
    cu = _t((cu_len or bs + 1,), B.I32)
    st = lib.qsa_index(ctypes.byref(q), ctypes.byref(w) if w is not None else None, ctypes.byref(k),
                       ctypes.byref(bt), ctypes.byref(r2t), ctypes.byref(cl), budget, c,
                       ctypes.byref(sel), ctypes.byref(cu), None)
    return st, lib.qsa_last_error().decode()


@pytest.mark.parametrize("kwargs,match", [
    (dict(bs=129), r"bs must be in \[1, 128\]"),
    (dict(hi=65), r"index heads must be in \[1, 64\]"),
    (dict(di=96), "index head dim must be 64 or 128"),
    (dict(q_dtype=B.F16), "q_index must be bf16"),
    (dict(weights="bf16"), "head_weights must be f32"),
    (dict(k_di=128), "k_index_pool rows must hold 64 elements"),
    (dict(bt_rows=3), "one row per q_index row"),
    (dict(max_tokens=262145), "more than 262144 tokens"),
    (dict(c=0), r"compress_ratio must be in \[1, 64\]"),
    (dict(budget=66, c=4), "budget must be a positive multiple"),
    (dict(budget=2048, c=16), r"budget \+ compress_ratio - 1 <= 2055"),
    (dict(sel_len=10), "sel_out must hold"),
    (dict(cu_len=5), "cu_out must have bs \\+ 1"),
    (dict(q_data=FAKE + 8), "16-byte boundaries"),
])
def test_index_contract_rejections(kwargs, match):
    st, msg = _index(**kwargs)
    assert st == 1, (st, msg)
    assert re.search(match, msg), msg
    assert msg.startswith("qsa_index")



def test_kv_pool_checks_before_any_launch():
    """KvPool needs scales for quantized pools, and its no-allocation decode
    needs out and lse; both are refused on the host."""
    import torch
    import sparse_index_paged_amd as qsa
    k = torch.zeros(16, 2, 256, dtype=torch.uint8)
    with pytest.raises(ValueError, match="need k_scale and v_scale"):
        qsa.KvPool(k, k, kv_format="fp8")
    pool = qsa.KvPool(torch.zeros(16, 2, 256, dtype=torch.bfloat16),
                      torch.zeros(16, 2, 256, dtype=torch.bfloat16))
    q = torch.zeros(1, 24, 256, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="needs out and lse"):
        pool.decode(q, torch.zeros(1, dtype=torch.int32), torch.zeros(2, dtype=torch.int32), noalloc=True)


def test_stamps_build_exports_the_api_and_its_call():
    """libqsa_stamps.so (include/qsa_stamps.h) exports everything qsa.h
    declares plus qsa_debug_set_phase_stamps, which libqsa.so does not."""
    path = os.path.join(os.path.dirname(qsa.lib_path()), "libqsa_stamps.so")
    nm = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True,
                        check=True).stdout
    exported = set(re.findall(r"\bT (qsa_\w+)", nm))
    assert exported == set(_declared_functions()) | {"qsa_debug_set_phase_stamps"}
    lib = B.load_stamps_library()
    assert lib.qsa_debug_set_phase_stamps(None, 0) == 0


def test_pool_objects_refuse_reallocated_tensors():
    """KvPool / TieredPool keep descriptors built once; a held tensor whose
    storage was replaced (resize_) is refused on the host before any call."""
    import torch
    import sparse_index_paged_amd as qsa
    k = torch.zeros(16, 2, 256, dtype=torch.bfloat16)
    v = torch.zeros(16, 2, 256, dtype=torch.bfloat16)
    pool = qsa.KvPool(k, v)
    pool.check()
    k.resize_(4096, 2, 256)
    with pytest.raises(ValueError, match="reallocated"):
        pool.check()
    ks = torch.ones(16, 2, 1)
    qp = qsa.KvPool(torch.zeros(16, 2, 256, dtype=torch.uint8), torch.zeros(16, 2, 256, dtype=torch.uint8),
                    kv_format="fp8", k_scale=ks, v_scale=ks.clone())
    qp.check()
    ks.resize_(8192, 2, 1)
    with pytest.raises(ValueError, match="reallocated"):
        qp.check()
    r, slots = 64, 256
    arrays = dict(ring_k=torch.zeros(r, 2, 256, dtype=torch.int8), ring_v=torch.zeros(r, 2, 256, dtype=torch.int8),
                  ring_k_scale=torch.zeros(r, 2, 4, dtype=torch.float16),
                  ring_v_scale=torch.zeros(r, 2, 4, dtype=torch.float16),
                  owner=torch.zeros(r, dtype=torch.int32), claim=torch.zeros(r, dtype=torch.int32),
                  cold_k=torch.zeros(slots, 2, 128, dtype=torch.uint8),
                  cold_v=torch.zeros(slots, 2, 128, dtype=torch.uint8),
                  cold_k_scale=torch.zeros(slots, 2, 8, dtype=torch.float16),
                  cold_v_scale=torch.zeros(slots, 2, 8, dtype=torch.float16))
    tp = qsa.TieredPool(arrays)
    tp.check()
    arrays["owner"].resize_(1 << 16)
    with pytest.raises(ValueError, match="reallocated"):
        tp.check()


def test_probe_library_exports_what_its_header_declares():
    """libqsa_probe.so (measurement helpers, include/qsa_probe.h) exports
    exactly the calls its header declares, and its argument checks reject
    bad calls on the host without a device."""
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "qsa_probe.h")).read(), flags=re.S)
    declared = set(re.findall(r"\b(qsa_probe_[a-z_]+)\s*\(", text))
    assert declared == {"qsa_probe_gather", "qsa_probe_line_reads"}
    path = os.path.join(os.path.dirname(qsa.lib_path()), "libqsa_probe.so")
    nm = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True,
                        check=True).stdout
    assert set(re.findall(r"\bT (qsa_\w+)", nm)) == declared
    lib = ctypes.CDLL(path)
    P, I64 = ctypes.c_void_p, ctypes.c_int64
    f = lib.qsa_probe_line_reads
    f.restype = ctypes.c_int
    f.argtypes = [P, I64, I64, ctypes.c_int, ctypes.c_uint32, P, I64, P]
    fake = ctypes.c_void_p(1 << 20)  # 128-byte aligned, never dereferenced on these paths
    assert f(None, 1 << 20, 1024, 0, 1, fake, 1, None) == 1          # no buffer
    assert f(fake, 1 << 20, 1024, 4, 1, fake, 1, None) == 1          # unknown load form
    assert f(fake, 1 << 20, 1000, 0, 1, fake, 1, None) == 1          # not a multiple of 1024
    assert f(fake, 1 << 20, 4096, 0, 1, fake, 3, None) == 1          # sink too small
    assert f(fake, 64, 1024, 0, 1, fake, 1, None) == 1               # less than one line
    assert f(ctypes.c_void_p((1 << 20) + 4), 1 << 20, 1024, 0, 1, fake, 1, None) == 1  # misaligned
