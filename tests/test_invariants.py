"""GPU checks of what the definition fixes independently of the oracle's arithmetic,
of the kernels' rarely taken branches, and of the output bounds.

* V = 1 gives O = 1 (rows of P sum to 1) and dQ = dK = 0 (dP_ij = D_i).
* Identical keys give a uniform P: O_i is the mean of the visible V rows,
  lse_i = s_i + ln n_i and dQ = 0.
* A dominant score placed in a late key tile, and inputs with a large score
  range, make the forward raise its running reference maximum after the first
  tile, which ordinary N(0, 1) inputs almost never do.
* Canary bands: every output is written through pointers into the middle of a
  larger buffer whose margins hold a sentinel; nothing outside the documented
  extent may change, including the lse entries past a packed sequence's end.

Sources: "FlashAttention: Faster Attention Without Dropping a Single
Interaction", Method Deep Dive, Key designs 1-3 (definition, mergeable state,
backward) and Limitations, "Numerical exactness, low precision, and
reproducibility".
"""

import numpy as np
import pytest
import torch

import exact_io_aware_43_amd as fa
import oracle.attention as OA
from gpu_util import (TOL_O_MAX, TOL_ZERO_GRAD_RMS, check_bwd_full, check_fwd_full, f64, gpu_bwd, gpu_fwd,
                      make_inputs, record, to_dev)
from exact_io_aware_43_amd.workloads import Workload

pytestmark = pytest.mark.gpu
TORCH_DT = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}


def _banner(msg):
    print(f"[invariants] {msg}", flush=True)


def _abs_rms(x):
    return float(np.sqrt(np.mean(x ** 2))) if x.size else 0.0


@pytest.mark.parametrize("dt", ["bf16", "fp16"])
@pytest.mark.parametrize("causal,alibi", [(False, False), (True, False), (True, True), (False, True)])
def test_v_ones(dt, causal, alibi):
    w = Workload(f"v_ones_{dt}_c{int(causal)}_a{int(alibi)}", dt, 2, 4, 2, 333, 128, causal=causal, alibi=alibi)
    _banner(str(w))
    inp = make_inputs(w, 21, with_grad=True)
    inp["v"] = torch.ones_like(inp["v"])
    dinp = to_dev(inp)
    o, lse = gpu_fwd(w, dinp)
    og = f64(o)
    err = float(np.abs(og - 1.0).max())
    dq, dk, dv = (f64(g) for g in gpu_bwd(w, dinp, o, lse))
    ref_dv = OA.attention_bwd(inp["q"], inp["k"], inp["v"], inp["do"], scale=inp["scale"], causal=causal,
                              alibi_slopes=inp["alibi_slopes"])[2]
    m = dict(o_minus_1_maxabs=err, dq_abs_rms=_abs_rms(dq), dk_abs_rms=_abs_rms(dk),
             dv_relrms=float(np.linalg.norm(dv - ref_dv) / np.linalg.norm(ref_dv)))
    record("invariant", w, m, note="V = 1: O = 1, dQ = dK = 0")
    _banner(str(m))
    assert err <= TOL_O_MAX
    assert m["dq_abs_rms"] <= TOL_ZERO_GRAD_RMS and m["dk_abs_rms"] <= TOL_ZERO_GRAD_RMS
    assert m["dv_relrms"] <= 1e-2


@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys(causal):
    w = Workload(f"same_keys_c{int(causal)}", "bf16", 1, 4, 4, 300, 128, causal=causal)
    _banner(str(w))
    inp = make_inputs(w, 22, with_grad=True)
    inp["k"] = inp["k"][:, :1].expand_as(inp["k"]).contiguous()
    dinp = to_dev(inp)
    o, lse = gpu_fwd(w, dinp)
    og, lg = f64(o), f64(lse)
    v, q, k = (OA._f64(inp[x]) for x in ("v", "q", "k"))
    n_i = np.arange(1, w.N + 1) if causal else np.full(w.N, w.N)
    mean_v = (np.cumsum(v, axis=1) / n_i[None, :, None, None]) if causal else \
        np.broadcast_to(v.mean(axis=1, keepdims=True), v.shape)
    s_i = inp["scale"] * np.einsum("bnhc,bhc->bhn", q, k[:, 0])
    lse_cf = s_i + np.log(n_i)[None, None, :]
    dq = f64(gpu_bwd(w, dinp, o, lse)[0])
    m = dict(o_vs_mean_v_maxabs=float(np.abs(og - mean_v).max()), lse_vs_closed_form=float(np.abs(lg - lse_cf).max()),
             dq_abs_rms=_abs_rms(dq))
    record("invariant", w, m, note="identical keys: O = mean V, lse = s + ln n, dQ = 0")
    _banner(str(m))
    assert m["o_vs_mean_v_maxabs"] <= TOL_O_MAX
    assert m["lse_vs_closed_form"] <= 1e-3
    assert m["dq_abs_rms"] <= TOL_ZERO_GRAD_RMS


def _spiked(w, seed, spikes):
    """Inputs whose keys at the given positions score far above the rest for
    every query: q_i gets a common component c along dimension 0 and key j a
    weight a_j along it, so score(i, j) = scale (c a_j + noise)."""
    inp = make_inputs(w, seed, with_grad=False)
    dt = TORCH_DT[w.dtype]
    q = inp["q"].float()
    k = inp["k"].float()
    q[..., 0] = 8.0
    for j, a in spikes:
        k[:, j, :, :] = 0.0
        k[:, j, :, 0] = a
    inp["q"], inp["k"] = q.to(dt), k.to(dt)
    return inp


@pytest.mark.parametrize("dt", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_dominant_score_late_tile(dt, causal, d):
    """Keys far apart in the sequence score 8*(10, 20, 40)*scale above a row's
    baseline, the largest in the last key tile: every row that sees them raises
    its reference maximum in a late tile and ends with O close to that key's V."""
    N = 700
    w = Workload(f"spike_{dt}_d{d}_c{int(causal)}", dt, 1, 2, 1, N, d, causal=causal)
    _banner(str(w))
    inp = _spiked(w, 23, [(130, 10.0), (390, 20.0), (N - 3, 40.0)])
    dinp = to_dev(inp)
    o, lse = gpu_fwd(w, dinp)
    r = check_fwd_full(w, inp, o, lse)
    _banner(str(r))
    # rows past the last spike copy its V row up to O(e^-delta)
    v = OA._f64(inp["v"])
    og = f64(o)
    tail = og[:, N - 3:] if causal else og
    assert np.abs(tail - v[:, N - 3:N - 2]).max() <= 2 * TOL_O_MAX


@pytest.mark.parametrize("dt", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
def test_large_score_range(dt, causal):
    """Q and K with standard deviation 4: scores spread over tens of natural-log
    units, so later tiles regularly exceed the running maximum by more than the
    lazy-rescale threshold. V and dO are brought back to unit scale (an exact
    division by 4), so the absolute bar on O means what it means elsewhere."""
    w = Workload(f"wide_{dt}_c{int(causal)}", dt, 2, 4, 2, 600, 128, causal=causal, std=4.0)
    _banner(str(w))
    inp = make_inputs(w, 24, with_grad=True)
    inp["v"] = inp["v"] / 4
    inp["do"] = inp["do"] / 4
    dinp = to_dev(inp)
    o, lse = gpu_fwd(w, dinp)
    _banner(str(check_fwd_full(w, inp, o, lse)))
    _banner(str(check_bwd_full(w, inp, gpu_bwd(w, dinp, o, lse))))


# ------------------------------------------------------------------ canary bands

GUARD = 4096  # bytes of sentinel on each side of every output (keeps 16-byte alignment)


class Guarded:
    """A device buffer of `nbytes` between two GUARD-byte margins, all filled with
    the byte `fill`; `ptr` is the address of the inner region."""

    def __init__(self, nbytes, fill=0x7B):
        self.n = nbytes
        self.buf = torch.full((nbytes + 2 * GUARD,), fill, dtype=torch.uint8, device="cuda")
        self.fill = fill
        self.ptr = self.buf.data_ptr() + GUARD

    def margins_intact(self):
        b = self.buf.cpu()
        return bool((b[:GUARD] == self.fill).all() and (b[GUARD + self.n:] == self.fill).all())

    def inner(self, dtype, shape):
        return self.buf[GUARD:GUARD + self.n].view(dtype).view(shape)


@pytest.mark.parametrize("varlen", [False, True])
def test_canary_bands(varlen):
    dt = torch.bfloat16
    if varlen:
        lengths = [300, 1, 0, 129, 64]
        w = Workload("canary_varlen", "bf16", len(lengths), 4, 2, 300, 128, causal=True, alibi=True,
                     varlen=(1, 300))
        inp = make_inputs(w, 25, lengths=lengths, with_grad=True)
    else:
        lengths = None
        w = Workload("canary_dense", "bf16", 2, 4, 2, 333, 128, causal=True, alibi=True)
        inp = make_inputs(w, 25, with_grad=True)
    _banner(str(w))
    dinp = to_dev(inp)
    B, H, Hkv, d = w.B, w.H, w.Hkv, w.d
    N = inp["max_seqlen"]
    qn, kn = inp["q"].numel(), inp["k"].numel()
    o_g = Guarded(qn * 2)
    lse_g = Guarded(B * H * N * 4, fill=0x7F)  # 0x7f7f7f7f: a finite sentinel float
    P = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    sh = torch.cuda.current_stream().cuda_stream
    st = fa.fa_fwd(P(dinp["q"]), P(dinp["k"]), P(dinp["v"]), o_g.ptr, lse_g.ptr, B, H, Hkv, N, d, inp["scale"], 1,
                   P(dinp["alibi_slopes"]), P(dinp["cu_seqlens"]), fa.FA_BF16, sh)
    assert st == 0
    torch.cuda.synchronize()
    assert o_g.margins_intact() and lse_g.margins_intact()
    o = o_g.inner(dt, inp["q"].shape)
    lse = lse_g.inner(torch.float32, (B, H, N))
    check_fwd_full(w, inp, o, lse)
    if varlen:
        sentinel = torch.full((1,), 0x7F, dtype=torch.uint8).repeat(4).view(torch.float32)[0].item()
        lc = lse.cpu()
        for b, n in enumerate(lengths):
            assert (lc[b, :, n:] == sentinel).all(), f"lse past the end of sequence {b} was written"

    ws_bytes = fa.fa_bwd_workspace_size(B, H, Hkv, N, d, 1, int(varlen), fa.FA_BF16)
    ws_g = Guarded(ws_bytes)
    dq_g, dk_g, dv_g = Guarded(qn * 2), Guarded(kn * 2), Guarded(kn * 2)
    st = fa.fa_bwd(P(dinp["q"]), P(dinp["k"]), P(dinp["v"]), P(o), P(dinp["do"]), P(lse), dq_g.ptr, dk_g.ptr,
                   dv_g.ptr, B, H, Hkv, N, d, inp["scale"], 1, P(dinp["alibi_slopes"]), P(dinp["cu_seqlens"]),
                   fa.FA_BF16, ws_g.ptr, ws_bytes, sh)
    assert st == 0
    torch.cuda.synchronize()
    for g in (ws_g, dq_g, dk_g, dv_g, o_g, lse_g):
        assert g.margins_intact()
    grads = (dq_g.inner(dt, inp["q"].shape), dk_g.inner(dt, inp["k"].shape), dv_g.inner(dt, inp["v"].shape))
    check_bwd_full(w, inp, grads)
    # a rejected call writes nothing
    before = [g.buf.clone() for g in (dq_g, dk_g, dv_g)]
    st = fa.fa_bwd(P(dinp["q"]), P(dinp["k"]), P(dinp["v"]), P(o), P(dinp["do"]), P(lse), dq_g.ptr, dk_g.ptr,
                   dv_g.ptr, B, H, Hkv, N, d, inp["scale"], 1, P(dinp["alibi_slopes"]), P(dinp["cu_seqlens"]),
                   fa.FA_BF16, ws_g.ptr, ws_bytes - 256, sh)
    assert st == -3
    torch.cuda.synchronize()
    for g, b0 in zip((dq_g, dk_g, dv_g), before):
        assert torch.equal(g.buf, b0)


def test_past_one_million_rows():
    """N = 1,100,000 (one head, d = 128, causal): more rows than 65535 blocks of
    16, which the backward pre-pass once put along grid z. The whole path runs;
    sampled forward rows match the oracle; the backward keeps sum_j dV_j =
    sum_i dO_i (every row of P sums to 1) and sum_j dK_j = 0 (every row of dS
    sums to 0), measured against the sizes of the terms."""
    N, d = 1_100_000, 128
    w = Workload("million", "bf16", 1, 1, 1, N, d, causal=True)
    g = torch.Generator().manual_seed(11)
    q, k, v, do = (torch.randn(1, N, 1, d, generator=g).to(torch.bfloat16).cuda() for _ in range(4))
    scale = d ** -0.5
    _banner(f"N={N} forward")
    o, lse = fa.attention(q, k, v, causal=True, softmax_scale=scale)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 777, 65535 * 16 - 1, 65535 * 16, 1_049_000, N - 1])
    o_ref, l_ref = OA.head_rows_fwd(f64(q[0, :, 0]), f64(k[0, :, 0]), f64(v[0, :, 0]), rows, scale, causal=True)
    err_o = float(np.abs(f64(o[0, rows, 0]) - o_ref).max())
    err_l = float(np.abs(f64(lse[0, 0, rows]) - l_ref).max())
    _banner(f"sampled rows: O max-abs {err_o:.3e}, lse max-abs {err_l:.3e}")
    assert err_o <= TOL_O_MAX and err_l <= 1e-3
    _banner(f"N={N} backward")
    dq, dk, dv = fa.attention_bwd(do, q, k, v, o, lse, causal=True, softmax_scale=scale)
    torch.cuda.synchronize()
    for x in (dq, dk, dv):
        assert torch.isfinite(x.float()).all()
    sv, so = dv[0, :, 0].double().sum(0), do[0, :, 0].double().sum(0)
    rel_v = float((sv - so).norm() / so.norm())
    sk = dk[0, :, 0].double().sum(0)
    rel_k = float(sk.norm() / dk[0, :, 0].double().abs().sum(0).norm())
    _banner(f"sum dV vs sum dO rel {rel_v:.3e}; |sum dK| / sum |dK| {rel_k:.3e}")
    record("million_rows", w, dict(o_maxabs=err_o, lse_maxabs=err_l, sum_dv_rel=rel_v, sum_dk_rel=rel_k))
    assert rel_v <= 1e-2 and rel_k <= 1e-2
