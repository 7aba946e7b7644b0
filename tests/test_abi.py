"""CPU checks of the C ABI: the library loads, exports every function include/fa.h
declares, and rejects bad arguments with the documented status before launching.

Every call here fails argument validation, so no kernel is launched (the fake
device pointers are never dereferenced); that is the property under test.
"""

import math
import os
import re
import subprocess

import pytest

import exact_io_aware_43_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3
A = 0x10000  # fake, 16-byte aligned "device" addresses: never dereferenced
PTR = [A + 0x1000 * i for i in range(12)]


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_expected_api():
    assert declared_functions() == sorted(
        ["fa_fwd", "fa_fwd_dropout", "fa_fwd_ext", "fa_bwd", "fa_bwd_dropout", "fa_bwd_ext", "fa_bwd_stages",
         "fa_bwd_workspace_size",
         "fa_bwd_noalloc", "fa_bwd_noalloc_max_bytes", "fa_fwd_kvcache", "fa_kvcache_workspace_size",
         "fa_fp8_v_keys", "fa_quantize_fp8_qk", "fa_quantize_fp8_v", "fa_fwd_fp8",
         "fa_strerror", "fa_version"])


def test_library_exports_every_declared_symbol():
    lib = fa.lib()
    out = subprocess.run(["nm", "-D", "--defined-only", fa.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\s[TW]\s+(\S+)", out))
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in exported, f"{name} not exported with C linkage"


def test_version_and_strerror():
    assert fa.fa_version() == 10000
    for code in (OK, INVALID, UNSUPPORTED, WORKSPACE, -4, -5):
        s = fa.fa_strerror(code)
        assert s and s != "unknown status"
    assert fa.fa_strerror(123) == "unknown status"


def _fwd(**kw):
    a = dict(q=PTR[0], k=PTR[1], v=PTR[2], o=PTR[3], lse=PTR[4], B=1, H=4, Hkv=2, N=64, d=128, scale=0.125,
             causal=0, alibi=None, cu=None, dtype=fa.FA_BF16, stream=None)
    a.update(kw)
    return fa.fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Hkv"], a["N"], a["d"], a["scale"],
                     a["causal"], a["alibi"], a["cu"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), INVALID), (dict(k=None), INVALID), (dict(v=None), INVALID), (dict(o=None), INVALID),
    (dict(lse=None), INVALID), (dict(B=0), INVALID), (dict(H=0), INVALID), (dict(Hkv=0), INVALID),
    (dict(N=0), INVALID), (dict(N=-5), INVALID), (dict(H=6, Hkv=4), INVALID), (dict(causal=2), INVALID),
    (dict(scale=math.nan), INVALID), (dict(scale=math.inf), INVALID), (dict(dtype=3), INVALID),
    (dict(d=96), UNSUPPORTED), (dict(d=8), UNSUPPORTED), (dict(d=48), UNSUPPORTED), (dict(d=512), UNSUPPORTED), (dict(d=0), INVALID),
    (dict(q=PTR[0] + 8), INVALID), (dict(o=PTR[3] + 2), INVALID), (dict(lse=PTR[4] + 4), INVALID),
    (dict(alibi=PTR[5] + 4), INVALID), (dict(cu=PTR[6] + 4), INVALID),
    (dict(B=1 << 16, N=1 << 16, H=2, Hkv=2), INVALID),
    # grid limits: at most 65535 tiles of 128 rows (64 for fp32) and 65535 sequences
    (dict(B=1, N=65535 * 128 + 1, H=1, Hkv=1), INVALID), (dict(B=65536, N=1, H=1, Hkv=1), INVALID),
    (dict(B=1, N=65535 * 64 + 1, H=1, Hkv=1, dtype=fa.FA_FP32), INVALID),
])
def test_fwd_rejects(kw, expect):
    assert _fwd(**kw) == expect


def _bwd(stages=None, **kw):
    a = dict(q=PTR[0], k=PTR[1], v=PTR[2], o=PTR[3], do=PTR[4], lse=PTR[5], dq=PTR[6], dk=PTR[7], dv=PTR[8],
             B=2, H=4, Hkv=2, N=64, d=64, scale=0.125, causal=1, alibi=None, cu=None, dtype=fa.FA_BF16,
             ws=PTR[9], ws_bytes=1 << 20, stream=None)
    a.update(kw)
    args = [a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"], a["B"], a["H"], a["Hkv"],
            a["N"], a["d"], a["scale"], a["causal"], a["alibi"], a["cu"], a["dtype"], a["ws"], a["ws_bytes"]]
    if stages is None:
        return fa.fa_bwd(*args, a["stream"])
    return fa.fa_bwd_stages(*args, stages, a["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), INVALID), (dict(do=None), INVALID), (dict(lse=None), INVALID), (dict(dq=None), INVALID),
    (dict(dk=None), INVALID), (dict(dv=None), INVALID), (dict(H=3), INVALID), (dict(causal=-1), INVALID),
    (dict(dtype=fa.FA_FP32), UNSUPPORTED), (dict(d=96), UNSUPPORTED), (dict(d=512), UNSUPPORTED),
    (dict(dk=PTR[7] + 8), INVALID), (dict(ws=None), WORKSPACE), (dict(ws=PTR[9] + 8), WORKSPACE),
    (dict(ws_bytes=2 * 2 * 4 * 64 * 4 - 1), WORKSPACE),
])
def test_bwd_rejects(kw, expect):
    assert _bwd(**kw) == expect
    assert _bwd(stages=fa.FA_BWD_ALL, **kw) == expect


@pytest.mark.parametrize("stages", [0, 8, 9, 0xFF])
def test_bwd_stage_mask_rejected(stages):
    assert _bwd(stages=stages) == INVALID


def test_workspace_size():
    # two fp32 values (D and the log2-scaled statistic) per (sequence, head, position),
    # positions padded to a multiple of 64, total rounded up to 256 bytes
    assert fa.fa_bwd_workspace_size(2, 4, 2, 64, 64, 1, 0, fa.FA_BF16) == 2 * 2 * 4 * 64 * 4
    assert fa.fa_bwd_workspace_size(1, 32, 32, 16384, 128, 1, 0, fa.FA_BF16) == 2 * 32 * 16384 * 4
    assert fa.fa_bwd_workspace_size(1, 1, 1, 3, 64, 0, 0, fa.FA_BF16) == 2 * 64 * 4
    assert fa.fa_bwd_workspace_size(3, 2, 1, 65, 64, 0, 0, fa.FA_BF16) == 2 * 3 * 2 * 128 * 4
    assert fa.fa_bwd_workspace_size(0, 4, 2, 64, 64, 1, 0, fa.FA_BF16) == 0
    assert fa.fa_bwd_workspace_size(1, 4, 3, 64, 64, 1, 0, fa.FA_BF16) == 0
    assert fa.fa_bwd_workspace_size(1, 4, 2, 64, 80, 1, 0, fa.FA_BF16) == 0


def test_binding_shape_errors():
    import torch

    q = torch.zeros(2, 8, 4, 64)
    with pytest.raises(ValueError):
        fa.attention(q, q, q)  # host tensors are refused before any call
    with pytest.raises(ValueError):
        fa._binding._shape(torch.zeros(8, 4, 64), torch.zeros(8, 2, 64), torch.zeros(3, dtype=torch.int32), None)
    assert fa._binding._shape(q, torch.zeros(2, 8, 2, 64), None, None) == (2, 4, 2, 8, 64)


def test_no_undefined_kernel_stubs():
    """Every kernel's host launch stub is defined in the library (a host-pass
    diagnostic that is deferred for device code can silently drop them)."""
    out = subprocess.run(["nm", "-D", "--undefined-only", fa.LIB_PATH], capture_output=True, text=True).stdout
    assert "__device_stub__" not in out, [l for l in out.splitlines() if "__device_stub__" in l][:3]


def _val_case(**over):
    """Keyword arguments of a valid dense (or packed) call on host tensors, with overrides."""
    import torch

    bf = torch.bfloat16
    base = dict(q=torch.zeros(2, 8, 4, 64, dtype=bf), k=torch.zeros(2, 8, 2, 64, dtype=bf),
                v=torch.zeros(2, 8, 2, 64, dtype=bf), cu_seqlens=None, max_seqlen=None, alibi_slopes=None,
                q_like=(), lse=None)
    base.update(over)
    return base


def _validate(**kw):
    q, k, v = kw.pop("q"), kw.pop("k"), kw.pop("v")
    return fa._binding.validate(q, k, v, require_device=False, **kw)


def test_binding_validation_accepts_valid_calls():
    import torch

    assert _validate(**_val_case()) == (2, 4, 2, 8, 64)
    c = _val_case(alibi_slopes=torch.zeros(4), lse=torch.zeros(2, 4, 8),
                  q_like=(("o", torch.zeros(2, 8, 4, 64, dtype=torch.bfloat16)),))
    assert _validate(**c) == (2, 4, 2, 8, 64)
    bf = torch.bfloat16
    packed = dict(q=torch.zeros(30, 4, 128, dtype=bf), k=torch.zeros(30, 1, 128, dtype=bf),
                  v=torch.zeros(30, 1, 128, dtype=bf), cu_seqlens=torch.tensor([0, 10, 30], dtype=torch.int32),
                  max_seqlen=20, lse=torch.zeros(2, 4, 20))
    assert _validate(**_val_case(**packed)) == (2, 4, 1, 20, 128)


def _bad_cases():
    import torch

    bf, f16 = torch.bfloat16, torch.float16
    cu = torch.tensor([0, 10, 30], dtype=torch.int32)
    packed = dict(q=torch.zeros(30, 4, 128, dtype=bf), k=torch.zeros(30, 2, 128, dtype=bf),
                  v=torch.zeros(30, 2, 128, dtype=bf), cu_seqlens=cu, max_seqlen=20)
    return {
        "k_wrong_N": dict(k=torch.zeros(2, 7, 2, 64, dtype=bf)),
        "k_wrong_B": dict(k=torch.zeros(1, 8, 2, 64, dtype=bf)),
        "k_wrong_d": dict(k=torch.zeros(2, 8, 2, 32, dtype=bf)),
        "v_differs_from_k": dict(v=torch.zeros(2, 8, 1, 64, dtype=bf)),
        "k_dtype": dict(k=torch.zeros(2, 8, 2, 64, dtype=f16)),
        "q_dtype_int": dict(q=torch.zeros(2, 8, 4, 64, dtype=torch.int16)),
        "heads_not_multiple": dict(k=torch.zeros(2, 8, 3, 64, dtype=bf), v=torch.zeros(2, 8, 3, 64, dtype=bf)),
        "noncontiguous_v": dict(v=torch.zeros(2, 8, 64, 2, dtype=bf).transpose(2, 3)),
        "slopes_dtype": dict(alibi_slopes=torch.zeros(4, dtype=torch.float64)),
        "slopes_shape": dict(alibi_slopes=torch.zeros(2)),
        "lse_shape": dict(lse=torch.zeros(2, 4, 9)),
        "lse_dtype": dict(lse=torch.zeros(2, 4, 8, dtype=bf)),
        "out_shape": dict(q_like=(("out", torch.zeros(2, 8, 4, 32, dtype=bf)),)),
        "dout_dtype": dict(q_like=(("dout", torch.zeros(2, 8, 4, 64, dtype=f16)),)),
        "o_missing": dict(q_like=(("o", None),)),
        "packed_cu_int64": dict(packed, cu_seqlens=cu.to(torch.int64)),
        "packed_cu_2d": dict(packed, cu_seqlens=cu.reshape(1, 3)),
        "packed_no_max": dict(packed, max_seqlen=None),
        "packed_zero_max": dict(packed, max_seqlen=0),
        "packed_k_rows": dict(packed, k=torch.zeros(29, 2, 128, dtype=bf)),
        "packed_lse_shape": dict(packed, lse=torch.zeros(4, 2, 20)),
        "dense_given_3d": dict(q=torch.zeros(8, 4, 64, dtype=bf)),
    }


@pytest.mark.parametrize("name", sorted(_bad_cases()))
def test_binding_validation_rejects(name):
    with pytest.raises(ValueError):
        _validate(**_val_case(**_bad_cases()[name]))


def test_binding_refuses_host_tensors():
    import torch

    q = torch.zeros(1, 8, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device"):
        fa.attention(q, q, q)
    with pytest.raises(ValueError, match="device"):
        fa.attention_bwd(q, q, q, q, q, torch.zeros(1, 2, 8))


def _noalloc(**kw):
    a = dict(q=PTR[0], k=PTR[1], v=PTR[2], o=PTR[3], do=PTR[4], lse=PTR[5], dq=PTR[6], dk=PTR[7], dv=PTR[8],
             B=2, H=4, Hkv=2, N=64, d=64, scale=0.125, causal=1, alibi=None, cu=None, dtype=fa.FA_BF16, stream=None)
    a.update(kw)
    return fa.fa_bwd_noalloc(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"], a["B"],
                             a["H"], a["Hkv"], a["N"], a["d"], a["scale"], a["causal"], a["alibi"], a["cu"],
                             a["dtype"], a["stream"])


def test_noalloc_scratch_size():
    assert fa.fa_bwd_noalloc_max_bytes() == 16 << 20


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), INVALID), (dict(dv=None), INVALID), (dict(H=3), INVALID), (dict(causal=2), INVALID),
    (dict(dtype=fa.FA_FP32), UNSUPPORTED), (dict(d=96), UNSUPPORTED), (dict(dk=PTR[7] + 8), INVALID),
    # 8 bytes per (sequence, head, position) above the 16 MiB scratch: rejected before any device call
    (dict(B=1, H=64, Hkv=64, N=32768 + 1), -5), (dict(B=4, H=32, Hkv=8, N=16384 + 64), -5),
])
def test_noalloc_rejects(kw, expect):
    assert _noalloc(**kw) == expect


@pytest.mark.parametrize("p_drop,expect", [
    (-0.1, INVALID), (1.0, INVALID), (1.5, INVALID), (float("nan"), INVALID), (0.999, INVALID),
])
def test_dropout_rejects_probability(p_drop, expect):
    a = [PTR[0], PTR[1], PTR[2], PTR[3], PTR[4], 1, 4, 2, 64, 128, 0.125, 0, None, None, fa.FA_BF16]
    assert fa.fa_fwd_dropout(*a, p_drop, 1, 0, None) == expect
    b = [PTR[0], PTR[1], PTR[2], PTR[3], PTR[4], PTR[5], PTR[6], PTR[7], PTR[8], 2, 4, 2, 64, 64, 0.125, 1, None,
         None, fa.FA_BF16]
    assert fa.fa_bwd_dropout(*b, p_drop, 1, 0, PTR[9], 1 << 20, None) == expect


def test_dropout_rejects_like_plain_calls():
    assert fa.fa_fwd_dropout(None, PTR[1], PTR[2], PTR[3], PTR[4], 1, 4, 2, 64, 128, 0.125, 0, None, None,
                             fa.FA_BF16, 0.1, 1, 0, None) == INVALID
    assert fa.fa_fwd_dropout(PTR[0], PTR[1], PTR[2], PTR[3], PTR[4], 1, 4, 2, 64, 128, 0.125, 0, None, None,
                             fa.FA_FP32, 0.1, 1, 0, None) == UNSUPPORTED
    b = [PTR[0], PTR[1], PTR[2], PTR[3], PTR[4], PTR[5], PTR[6], PTR[7], PTR[8], 2, 4, 2, 64, 64, 0.125, 1, None,
         None, fa.FA_BF16, 0.1, 1, 0]
    assert fa.fa_bwd_dropout(*b, None, 1 << 20, None) == WORKSPACE
    assert fa.fa_bwd_dropout(*b, PTR[9], 16, None) == WORKSPACE


@pytest.mark.parametrize("wl,wr,cap,p_drop,dtype,expect", [
    (-2, -1, 0.0, 0.0, fa.FA_BF16, INVALID), (-1, -5, 0.0, 0.0, fa.FA_BF16, INVALID),
    (4, 0, -1.0, 0.0, fa.FA_BF16, INVALID), (4, 0, float("inf"), 0.0, fa.FA_BF16, INVALID),
    (4, 0, float("nan"), 0.0, fa.FA_BF16, INVALID), (-1, -1, 0.0, 1.0, fa.FA_BF16, INVALID),
    (16, 16, 30.0, 0.1, fa.FA_BF16, UNSUPPORTED), (-1, -1, 0.0, 0.1, fa.FA_FP32, UNSUPPORTED),
])
def test_ext_rejects(wl, wr, cap, p_drop, dtype, expect):
    """Window below -1, a negative or non-finite cap and out-of-range dropout are
    invalid; dropout with softcapping (or with fp32) is unsupported. No device call
    is made: every check runs before the first launch."""
    a = [PTR[0], PTR[1], PTR[2], PTR[3], PTR[4], 1, 4, 2, 64, 128, 0.125, 0, None, None, dtype]
    assert fa.fa_fwd_ext(*a, wl, wr, cap, p_drop, 1, 0, None) == expect
    if dtype == fa.FA_FP32:
        return
    b = [PTR[0], PTR[1], PTR[2], PTR[3], PTR[4], PTR[5], PTR[6], PTR[7], PTR[8], 2, 4, 2, 64, 64, 0.125, 1, None,
         None, dtype]
    assert fa.fa_bwd_ext(*b, wl, wr, cap, p_drop, 1, 0, PTR[9], 1 << 20, None) == expect


def test_ext_rejects_like_plain_calls():
    assert fa.fa_fwd_ext(None, PTR[1], PTR[2], PTR[3], PTR[4], 1, 4, 2, 64, 128, 0.125, 0, None, None,
                         fa.FA_BF16, 8, 0, 10.0, 0.0, 1, 0, None) == INVALID
    assert fa.fa_fwd_ext(PTR[0], PTR[1], PTR[2], PTR[3], PTR[4], 1, 4, 2, 64, 96, 0.125, 0, None, None,
                         fa.FA_BF16, 8, 0, 10.0, 0.0, 1, 0, None) == UNSUPPORTED
    b = [PTR[0], PTR[1], PTR[2], PTR[3], PTR[4], PTR[5], PTR[6], PTR[7], PTR[8], 2, 4, 2, 64, 64, 0.125, 1, None,
         None, fa.FA_BF16, 8, 0, 10.0, 0.0, 1, 0]
    assert fa.fa_bwd_ext(*b, None, 1 << 20, None) == WORKSPACE
    b32 = b[:18] + [fa.FA_FP32] + b[19:]
    assert fa.fa_bwd_ext(*b32, PTR[9], 1 << 20, None) == UNSUPPORTED


def test_kvcache_workspace_size():
    # one split: nothing needed
    assert fa.fa_kvcache_workspace_size(1, 8, 8, 1, 100, 128, 1) == 0
    # explicit splits: fp32 O and lse per (sequence, head, query, split)
    assert fa.fa_kvcache_workspace_size(2, 8, 2, 3, 4096, 128, 4) == ((2 * 8 * 3 * 4 * 129 * 4 + 255) & ~255)
    # at most one split per 128 keys of the capacity
    assert fa.fa_kvcache_workspace_size(1, 4, 4, 1, 300, 64, 64) == ((1 * 4 * 1 * 3 * 65 * 4 + 255) & ~255)
    # auto: one workgroup per compute unit, at least 512 keys per range; with several ranges per sequence they
    # are balanced over the caches laid end to end: B * S = 8 * 4 = 32 ranges per kv head, a partial per range
    assert fa.fa_kvcache_workspace_size(8, 32, 8, 1, 16384, 128, 0) == ((8 * 32 * 1 * 32 * 129 * 4 + 255) & ~255)
    assert fa.fa_kvcache_workspace_size(1, 8, 1, 1, 2048, 128, 0) == ((1 * 8 * 1 * 4 * 129 * 4 + 255) & ~255)
    # auto: a deterministic choice; a large batch of heads needs no split
    assert fa.fa_kvcache_workspace_size(64, 64, 64, 1, 4096, 128, 0) == 0
    assert fa.fa_kvcache_workspace_size(1, 8, 1, 1, 65536, 128, 0) > 0
    for bad in [(0, 8, 8, 1, 100, 128, 0), (1, 8, 3, 1, 100, 128, 0), (1, 8, 8, 0, 100, 128, 0),
                (1, 8, 8, 1, 0, 128, 0), (1, 8, 8, 1, 100, 96, 0), (1, 8, 8, 1, 100, 128, -1)]:
        assert fa.fa_kvcache_workspace_size(*bad) == 0


def _kv(**kw):
    a = dict(q=PTR[0], k=PTR[1], v=PTR[2], o=PTR[3], lse=PTR[4], cl=PTR[5], B=2, H=8, Hkv=2, Nq=1, Nk=4096, d=128,
             scale=0.125, causal=1, alibi=None, dtype=fa.FA_BF16, splits=4, ws=PTR[6], ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return fa.fa_fwd_kvcache(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cl"], a["B"], a["H"], a["Hkv"], a["Nq"],
                             a["Nk"], a["d"], a["scale"], a["causal"], a["alibi"], a["dtype"], a["splits"], a["ws"],
                             a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), INVALID), (dict(cl=None), INVALID), (dict(lse=None), INVALID), (dict(H=6, Hkv=4), INVALID),
    (dict(Nq=0), INVALID), (dict(Nk=0), INVALID), (dict(causal=3), INVALID), (dict(splits=-2), INVALID),
    (dict(scale=math.nan), INVALID), (dict(d=256), UNSUPPORTED), (dict(d=32), UNSUPPORTED),
    (dict(dtype=fa.FA_FP32), UNSUPPORTED), (dict(k=PTR[1] + 4), INVALID), (dict(cl=PTR[5] + 4), INVALID),
    (dict(ws=None), WORKSPACE), (dict(ws_bytes=100), WORKSPACE), (dict(ws=PTR[6] + 8), WORKSPACE),
])
def test_kvcache_rejects(kw, expect):
    assert _kv(**kw) == expect


def test_fp8_v_keys():
    """Transposed V codes are padded to whole 128-key tiles."""
    assert [fa.fa_fp8_v_keys(n) for n in (1, 127, 128, 129, 1000, 16384)] == [128, 128, 128, 256, 1024, 16384]
    assert fa.fa_fp8_v_keys(0) == 0 and fa.fa_fp8_v_keys(-3) == 0


def _q8(**kw):
    a = dict(x=PTR[0], codes=PTR[1], scales=PTR[2], B=1, N=300, H=4, d=128, signs=None, dtype=fa.FA_BF16)
    a.update(kw)
    return fa.fa_quantize_fp8_qk(a["x"], a["codes"], a["scales"], a["B"], a["N"], a["H"], a["d"], a["signs"],
                                 a["dtype"], None)


def _v8(**kw):
    a = dict(v=PTR[0], codes=PTR[1], scales=PTR[2], B=1, N=300, Hkv=2, d=64, dtype=fa.FA_FP16)
    a.update(kw)
    return fa.fa_quantize_fp8_v(a["v"], a["codes"], a["scales"], a["B"], a["N"], a["Hkv"], a["d"], a["dtype"], None)


def _f8(**kw):
    a = dict(q=PTR[0], k=PTR[1], v=PTR[2], qs=PTR[3], ks=PTR[4], vs=PTR[5], o=PTR[6], lse=PTR[7], B=1, H=4, Hkv=2,
             N=300, d=128, scale=0.1, causal=1, rotated=0, dtype=fa.FA_BF16)
    a.update(kw)
    return fa.fa_fwd_fp8(a["q"], a["k"], a["v"], a["qs"], a["ks"], a["vs"], a["o"], a["lse"], a["B"], a["H"],
                         a["Hkv"], a["N"], a["d"], a["scale"], a["causal"], a["rotated"], a["dtype"], None)


@pytest.mark.parametrize("call,kw,expect", [
    (_q8, dict(x=None), INVALID), (_q8, dict(codes=PTR[1] + 4), INVALID), (_q8, dict(N=0), INVALID),
    (_q8, dict(H=0), INVALID), (_q8, dict(d=32), UNSUPPORTED), (_q8, dict(d=256), UNSUPPORTED),
    (_q8, dict(dtype=fa.FA_FP32), UNSUPPORTED), (_q8, dict(dtype=7), INVALID),
    (_q8, dict(B=1 << 12, N=1 << 12, H=1 << 8), INVALID), (_q8, dict(N=65535 * 128 + 1, H=1), INVALID),
    (_v8, dict(B=65536, N=1, Hkv=1), INVALID), (_f8, dict(N=65535 * 128 + 1, H=1, Hkv=1), INVALID),
    (_v8, dict(scales=None), INVALID), (_v8, dict(v=PTR[0] + 2), INVALID), (_v8, dict(Hkv=-1), INVALID),
    (_v8, dict(d=96), UNSUPPORTED), (_v8, dict(dtype=fa.FA_FP32), UNSUPPORTED),
    (_f8, dict(vs=None), INVALID), (_f8, dict(lse=PTR[7] + 4), INVALID), (_f8, dict(H=6, Hkv=4), INVALID),
    (_f8, dict(causal=2), INVALID), (_f8, dict(rotated=5), INVALID), (_f8, dict(scale=math.inf), INVALID),
    (_f8, dict(d=256), UNSUPPORTED), (_f8, dict(dtype=fa.FA_FP32), UNSUPPORTED), (_f8, dict(dtype=-1), INVALID),
    (_f8, dict(N=0), INVALID),
])
def test_fp8_rejects(call, kw, expect):
    """FP8 entry points check every argument before any launch (no device call here)."""
    assert call(**kw) == expect


def test_hadamard_sign_words():
    signs = [1.0] * 128
    for i in (0, 5, 63, 64, 127):
        signs[i] = -1.0
    w = fa.hadamard_sign_words(signs, 128)
    assert list(w) == [(1 << 0) | (1 << 5) | (1 << 63), (1 << 0) | (1 << 63)]
    with pytest.raises(ValueError):
        fa.hadamard_sign_words([1.0] * 127 + [0.5], 128)
    with pytest.raises(ValueError):
        fa.hadamard_sign_words([1.0] * 64, 128)


def test_fp8_binding_validation():
    """The FP8 helpers refuse host tensors, 32-bit inputs and mismatched shapes
    before any call into the library."""
    import torch

    x = torch.zeros(1, 8, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device"):
        fa.quantize_fp8_qk(x)
    with pytest.raises(ValueError, match="device"):
        fa.quantize_fp8_v(x)
    codes = torch.zeros(1, 8, 2, 64, dtype=torch.uint8)
    sc = torch.zeros(1, 2, 1)
    with pytest.raises(ValueError, match="device"):
        fa.attention_fp8_quantized(codes, sc, codes, sc, torch.zeros(1, 2, 64, 128, dtype=torch.uint8),
                                   torch.zeros(1, 2, 64))
    with pytest.raises(ValueError):
        fa.hadamard_sign_words([1.0, -1.0] * 32, 128)
