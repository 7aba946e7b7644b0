"""GPU parity at head dims 32 and 256, forward and backward, against the fp64 oracle.

The same kernels as head dims 64 and 128, instanced for these sizes: 32 needs
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


@pytest.mark.parametrize("dd", [32, 256])
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
