"""fa_bwd_noalloc (the backward with the library's static per-GPU scratch) gives
the same dQ, dK, dV as fa_bwd with a caller workspace: two calls in a row, the
second on a smaller problem, so the scratch holds the first call's values when
the second starts, and a problem beyond the scratch is refused without writing.

The kernels are the ones fa_bwd launches and are deterministic, so the results
must agree bit for bit; they are also held to the backward bar (relative RMS
<= 1e-2) against the fp64 oracle.
"""

import pytest
import torch

import exact_io_aware_43_amd as fa
from gpu_util import check_bwd_full, gpu_fwd, make_inputs, to_dev
from exact_io_aware_43_amd.workloads import Workload

pytestmark = pytest.mark.gpu


def _ptr(t):
    return None if t is None else t.data_ptr()


def _both(w, inp):
    """(grads from fa_bwd with a workspace, grads from fa_bwd_noalloc)."""
    d = to_dev(inp)
    o, lse = gpu_fwd(w, d)
    N = inp["max_seqlen"]
    dt = fa.FA_BF16 if w.dtype == "bf16" else fa.FA_FP16
    sh = torch.cuda.current_stream().cuda_stream
    args = (_ptr(d["q"]), _ptr(d["k"]), _ptr(d["v"]), _ptr(o), _ptr(d["do"]), _ptr(lse))
    tail = (w.B, w.H, w.Hkv, N, w.d, d["scale"], int(w.causal), _ptr(d["alibi_slopes"]), _ptr(d["cu_seqlens"]), dt)
    ref = [torch.full_like(d[x], float("nan")) for x in ("q", "k", "v")]
    ws_bytes = fa.fa_bwd_workspace_size(w.B, w.H, w.Hkv, N, w.d, int(w.causal), int(d["cu_seqlens"] is not None), dt)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    assert fa.fa_bwd(*args, *[_ptr(t) for t in ref], *tail, ws.data_ptr(), ws_bytes, sh) == 0
    got = [torch.full_like(d[x], float("nan")) for x in ("q", "k", "v")]
    assert fa.fa_bwd_noalloc(*args, *[_ptr(t) for t in got], *tail, sh) == 0
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_matches_fa_bwd_twice_shrinking():
    big = Workload("noalloc_big", "bf16", 2, 8, 2, 700, 128, causal=True, alibi=True)
    small = Workload("noalloc_small", "bf16", 1, 4, 4, 150, 64, causal=False)
    for w, seed in ((big, 31), (small, 32)):
        print(f"[noalloc] {w}", flush=True)
        inp = make_inputs(w, seed, with_grad=True)
        ref, got = _both(w, inp)
        for r, g in zip(ref, got):
            assert torch.equal(r, g)
        check_bwd_full(w, inp, got)


def test_noalloc_varlen():
    w = Workload("noalloc_varlen", "bf16", 4, 4, 2, 300, 128, causal=True, varlen=(1, 300))
    print(f"[noalloc] {w}", flush=True)
    inp = make_inputs(w, 33, lengths=[300, 1, 129, 64], with_grad=True)
    ref, got = _both(w, inp)
    for r, g in zip(ref, got):
        assert torch.equal(r, g)
    check_bwd_full(w, inp, got)


def test_noalloc_refuses_oversize_without_writing():
    # 8 * B * H * N64 bytes of scratch: B=1, H=64, N=32832 needs 16.03 MiB > 16 MiB
    B, H, N, d = 1, 64, 32832, 64
    x = torch.zeros(B, N, H, d, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros(B, H, N, device="cuda")
    outs = [torch.full_like(x, 7.0) for _ in range(3)]
    st = fa.fa_bwd_noalloc(x.data_ptr(), x.data_ptr(), x.data_ptr(), x.data_ptr(), x.data_ptr(), lse.data_ptr(),
                           *[t.data_ptr() for t in outs], B, H, H, N, d, 0.125, 1, None, None, fa.FA_BF16,
                           torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == -5, fa.fa_strerror(st)
    for t in outs:
        assert bool((t == 7.0).all())
