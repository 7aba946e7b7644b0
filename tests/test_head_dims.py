"""GPU parity at head dims 16, 32 and 256, forward and backward, against the fp64 oracle.

Head dim 16 runs in the head-dim-32 kernels with the upper 16 columns of every
staged tile and register fragment zero (the direct loads of those chunks fall
outside the buffer range and store zeros) and only 16 columns stored, so the
cases below also check that nothing past a row's 16 elements is read or
written. The same kernels as head dims 64 and 128, instanced for these sizes: 32 needs
fewer 1 KB direct-load instructions per tile than there are waves (the first
ones issue them); at 256 the forward runs 4 waves per workgroup on 64-key
tiles (its O accumulator alone takes 128 registers per lane), the dK/dV pass 4
waves on 32-query steps and the dQ pass 4 waves.

Whole-tensor comparisons at the usual bars over lengths that span several
tiles with a ragged tail, causal and not, ALiBi, GQA, packed sequences, a
window, softcapping and dropout; the fp32 forward at both sizes. Source of the
head-dim list: "FlashAttention: Faster Attention Without Dropping a Single
Interaction", Usage contract (head-dimension row).
"""

import numpy as np
import pytest
import torch

import exact_io_aware_43_amd as fa
import oracle.attention as OA
import oracle.philox as PX
from gpu_util import _compare_bwd, _compare_fwd, f64, make_inputs, seq_lengths, to_dev
from exact_io_aware_43_amd.workloads import Workload

pytestmark = pytest.mark.gpu


def _banner(msg):
    print(f"[hdim] {msg}", flush=True)


CASES = [
    # (workload, extra kwargs for attention / the oracle)
    (Workload("d16_bf16_c1", "bf16", 2, 4, 2, 700, 16, causal=True), {}),
    (Workload("d16_fp16_c0_mqa", "fp16", 1, 8, 1, 333, 16), {}),
    (Workload("d16_bf16_c1_alibi_varlen", "bf16", 3, 4, 4, 600, 16, causal=True, alibi=True, varlen=(1, 600)), {}),
    (Workload("d16_bf16_c0_window_cap", "bf16", 2, 4, 2, 520, 16, std=2.0), dict(window=(70, 30), softcap=8.0)),
    (Workload("d16_bf16_c1_dropout", "bf16", 1, 4, 2, 300, 16, causal=True), dict(dropout=(0.2, 77, 1))),
    (Workload("d32_bf16_c1", "bf16", 2, 4, 2, 700, 32, causal=True), {}),
    (Workload("d32_fp16_c0", "fp16", 1, 8, 2, 333, 32), {}),
    (Workload("d32_bf16_c1_alibi_varlen", "bf16", 3, 4, 4, 600, 32, causal=True, alibi=True, varlen=(1, 600)), {}),
    (Workload("d32_bf16_c0_window_cap", "bf16", 2, 4, 2, 520, 32, std=2.0), dict(window=(70, 30), softcap=8.0)),
    (Workload("d32_bf16_c1_dropout", "bf16", 1, 4, 2, 300, 32, causal=True), dict(dropout=(0.2, 77, 1))),
    (Workload("d256_bf16_c1", "bf16", 2, 4, 2, 450, 256, causal=True), {}),
    (Workload("d256_fp16_c0", "fp16", 1, 4, 1, 333, 256), {}),
    (Workload("d256_bf16_c1_alibi_varlen", "bf16", 3, 4, 2, 400, 256, causal=True, alibi=True, varlen=(1, 400)),
     {}),
    (Workload("d256_bf16_c0_window_cap", "bf16", 1, 4, 4, 300, 256, std=2.0), dict(window=(50, 90), softcap=12.0)),
    (Workload("d256_bf16_c1_dropout", "bf16", 1, 2, 1, 260, 256, causal=True), dict(dropout=(0.3, 5, 2))),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0].name for c in CASES])
def test_head_dim_parity(case):
    w, extra = case
    _banner(f"{w} {extra}")
    lengths = [w.N, 1, w.N // 3] if w.varlen else None
    inp = make_inputs(w, 95, lengths=lengths, with_grad=w.backward)
    if w.std != 1.0:  # wide scores from Q, K; V and dO back to unit spread (exact division)
        inp["v"] = inp["v"] / w.std
        if inp["do"] is not None:
            inp["do"] = inp["do"] / w.std
    d = to_dev(inp)
    drop = extra.get("dropout")
    akw = dict(window_size=extra.get("window", (-1, -1)), softcap=extra.get("softcap", 0.0))
    if drop:
        akw.update(dropout_p=drop[0], seed=drop[1], offset=drop[2])
    o, lse = fa.attention(d["q"], d["k"], d["v"], causal=w.causal, softmax_scale=d["scale"],
                          alibi_slopes=d["alibi_slopes"], cu_seqlens=d["cu_seqlens"], max_seqlen=d["max_seqlen"],
                          **akw)
    torch.cuda.synchronize()
    okw = dict(scale=inp["scale"], causal=w.causal, alibi_slopes=inp["alibi_slopes"], cu_seqlens=inp["cu_seqlens"],
               window=extra.get("window"), softcap=extra.get("softcap", 0.0), dropout=drop)
    o_ref, lse_ref = OA.attention_fwd(inp["q"], inp["k"], inp["v"], **okw)
    lg = f64(lse)
    mask = np.zeros(lg.shape, dtype=bool)
    for b, n in enumerate(seq_lengths(inp, w)):
        mask[b, :, :n] = True
    bar = 256.0 / PX.keep_threshold(drop[0]) if drop else 1.0
    _banner(str(_compare_fwd(w, f64(o), o_ref, lg[mask], lse_ref[mask], note=f"head dim {w.d}", o_bar_scale=bar)))
    if not w.backward:
        return
    g = fa.attention_bwd(d["do"], d["q"], d["k"], d["v"], o, lse, causal=w.causal, softmax_scale=d["scale"],
                         alibi_slopes=d["alibi_slopes"], cu_seqlens=d["cu_seqlens"], max_seqlen=d["max_seqlen"],
                         **akw)
    torch.cuda.synchronize()
    ref = OA.attention_bwd(inp["q"], inp["k"], inp["v"], inp["do"], **okw)
    _banner(str(_compare_bwd(w, [f64(x) for x in g], ref, note=f"head dim {w.d}")))


@pytest.mark.parametrize("dd", [16, 32, 256])
def test_fp32_head_dims(dd):
    w = Workload(f"fp32_d{dd}", "fp32", 1, 2, 1, 150, dd, causal=True, alibi=True, backward=False)
    inp = make_inputs(w, 96, with_grad=False)
    d = to_dev(inp)
    o, lse = fa.attention(d["q"], d["k"], d["v"], causal=True, softmax_scale=d["scale"],
                          alibi_slopes=d["alibi_slopes"])
    torch.cuda.synchronize()
    o_ref, lse_ref = OA.attention_fwd(inp["q"], inp["k"], inp["v"], scale=inp["scale"], causal=True,
                                      alibi_slopes=inp["alibi_slopes"])
    _banner(str(_compare_fwd(w, f64(o), o_ref, f64(lse).ravel(), lse_ref.ravel(), note=f"fp32 head dim {dd}")))


def test_head_dim_16_leaves_neighbours_alone():
    """Head dim 16 reads and writes only its own 16 columns. The outputs sit in
    buffers with canaries right after their last element, which survive the
    forward and the backward. Then kv head 1 of K and V and query head 3 of Q
    and dO are NaN: a read past a row's 16 elements would reach them from the
    heads before, so query heads 0 and 1 (kv head 0) must still match the oracle
    in O, lse, dQ and kv head 0's dK, dV."""
    w = Workload("d16_guard", "bf16", 1, 4, 2, 257, 16, causal=True)
    inp = make_inputs(w, 97, with_grad=True)
    canary = -12345.0
    sh = torch.cuda.current_stream().cuda_stream

    def padded_like(t):
        buf = torch.full((t.numel() + 64,), canary, dtype=t.dtype, device=t.device)
        return buf, buf[: t.numel()].view(t.shape)

    def run(q, k, v, do):
        ob, o = padded_like(q)
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
        assert fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), w.B, w.H, w.Hkv, w.N,
                         w.d, inp["scale"], 1, None, None, fa.FA_BF16, sh) == 0
        bufs = [padded_like(x) for x in (q, k, v)]
        ws = torch.empty(fa.fa_bwd_workspace_size(w.B, w.H, w.Hkv, w.N, w.d, 1, 0, fa.FA_BF16), dtype=torch.uint8,
                         device="cuda")
        assert fa.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                         bufs[0][1].data_ptr(), bufs[1][1].data_ptr(), bufs[2][1].data_ptr(), w.B, w.H, w.Hkv, w.N,
                         w.d, inp["scale"], 1, None, None, fa.FA_BF16, ws.data_ptr(), ws.numel(), sh) == 0
        torch.cuda.synchronize()
        for buf, view in [(ob, o)] + bufs:
            assert torch.all(buf[view.numel():] == canary), "a write past the last head-dim-16 row"
        return o, lse, [b[1] for b in bufs]

    d = to_dev(inp)
    o, lse, g = run(d["q"], d["k"], d["v"], d["do"])
    o_ref, lse_ref = OA.attention_fwd(inp["q"], inp["k"], inp["v"], scale=inp["scale"], causal=True)
    _banner(str(_compare_fwd(w, f64(o), o_ref, f64(lse).ravel(), lse_ref.ravel(), note="head dim 16 canaries")))
    ref = OA.attention_bwd(inp["q"], inp["k"], inp["v"], inp["do"], scale=inp["scale"], causal=True)
    _banner(str(_compare_bwd(w, [f64(x) for x in g], ref, note="head dim 16 canaries")))

    q2, k2, v2, do2 = (d[x].clone() for x in ("q", "k", "v", "do"))
    k2[:, :, 1] = float("nan")
    v2[:, :, 1] = float("nan")
    q2[:, :, 3] = float("nan")
    do2[:, :, 3] = float("nan")
    o2, lse2, g2 = run(q2, k2, v2, do2)
    w0 = Workload("d16_guard_head0", "bf16", 1, 2, 1, 257, 16, causal=True)
    sub = {x: inp[x][:, :, :2] for x in ("q", "do")}
    sub.update({x: inp[x][:, :, :1] for x in ("k", "v")})
    o_ref0, lse_ref0 = OA.attention_fwd(sub["q"], sub["k"], sub["v"], scale=inp["scale"], causal=True)
    _banner(str(_compare_fwd(w0, f64(o2[:, :, :2]), o_ref0, f64(lse2[:, :2]).ravel(), lse_ref0.ravel(),
                             note="head dim 16 beside NaN heads")))
    ref0 = OA.attention_bwd(sub["q"], sub["k"], sub["v"], sub["do"], scale=inp["scale"], causal=True)
    _banner(str(_compare_bwd(w0, [f64(g2[0][:, :, :2]), f64(g2[1][:, :, :1]), f64(g2[2][:, :, :1])], ref0,
                             note="head dim 16 beside NaN heads")))


@pytest.mark.parametrize("H,Hkv,packed", [(1, 1, False), (4, 1, True), (1, 1, True)],
                         ids=["mha1_dense", "mqa_packed", "mha1_packed"])
def test_head_dim_16_reads_no_row_past_the_end(H, Hkv, packed):
    """Head dim 16 with a single kv head (or a single query head): a 16-bit row
    of the tensor is 32 bytes, less than a row of the 32-wide staged tiles. The
    tiles that hold a tensor's last row must not take in the row after it. Each
    input sits at the start of a buffer whose next row is NaN; a read of that
    row would reach O, dQ, dK or dV through a zero weight (0 x NaN), so forward
    and backward must still match the oracle on every element."""
    w = Workload(f"d16_end_{H}_{Hkv}_{int(packed)}", "bf16", 3 if packed else 2, H, Hkv, 300, 16, causal=True,
                 varlen=(1, 300) if packed else None)
    lengths = [300, 17, 129] if packed else None
    inp = make_inputs(w, 11, lengths=lengths, with_grad=True)
    d = to_dev(inp)

    def before_nan_row(t):
        rows = t.shape[0]
        buf = torch.full((rows + 1,) + tuple(t.shape[1:]), float("nan"), dtype=t.dtype, device=t.device)
        buf[:rows] = t
        return buf[:rows]

    q, k, v, do = (before_nan_row(d[x]) for x in ("q", "k", "v", "do"))
    args = dict(causal=True, softmax_scale=inp["scale"], cu_seqlens=d["cu_seqlens"], max_seqlen=inp["max_seqlen"])
    o, lse = fa.attention(q, k, v, **args)
    g = fa.attention_bwd(do, q, k, v, o, lse, **args)
    torch.cuda.synchronize()
    o_ref, lse_ref = OA.attention_fwd(inp["q"], inp["k"], inp["v"], scale=inp["scale"], causal=True,
                                      cu_seqlens=inp["cu_seqlens"])
    lens = seq_lengths(inp, w)
    mask = np.zeros(tuple(lse.shape), dtype=bool)
    for b, n in enumerate(lens):
        mask[b, :, :n] = True
    _banner(str(_compare_fwd(w, f64(o), o_ref, f64(lse)[mask], lse_ref[mask], note="head dim 16 before a NaN row")))
    ref = OA.attention_bwd(inp["q"], inp["k"], inp["v"], inp["do"], scale=inp["scale"], causal=True,
                           cu_seqlens=inp["cu_seqlens"])
    _banner(str(_compare_bwd(w, [f64(x) for x in g], ref, note="head dim 16 before a NaN row")))
