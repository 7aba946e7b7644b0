"""Both workgroup shapes of the backward kernels at ragged lengths.

The dK/dV kernel runs 8-wave workgroups on 256-key tiles at head dims 64 and
128, except that grids of at most 2 x 256 (head dim 64) or 256 (head dim 128)
such workgroups (sequences x kv heads x 256-key tiles) run 4-wave workgroups on
128-key tiles. The causal dQ kernel likewise keeps 8-wave workgroups only for
grids of more than 256 (sequences x query heads x 256-query tiles). Every
small-shape test takes the 4-wave forms, so the cases here sit just above those
bounds, with lengths that end inside a tile, and compare the results with the
fp64 oracle on whole (sequence, kv head) groups. Each case is paired with the
same inputs cut to the first sequence, which falls under the bounds and runs
the 4-wave forms on the same rows.
"""

import numpy as np
import pytest

import gpu_util as G
from exact_io_aware_43_amd.workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu

# (name, dtype, d, causal, H, Hkv, N, packed lengths or None)
CASES = [
    ("d128_causal_dense", "bf16", 128, True, 24, 24, 1000, None),
    ("d128_noncausal_packed_gqa", "fp16", 128, False, 48, 24, 1000, [1000, 517, 3]),
    ("d64_causal_packed", "bf16", 64, True, 48, 48, 1000, [1000, 300, 777]),
    ("d64_noncausal_dense", "fp16", 64, False, 48, 48, 999, None),
]


def _grid(B, heads, N):
    return B * heads * ((N + 255) // 256)


def _workload(name, dt, d, causal, H, Hkv, N, lengths):
    return Workload(name, dt, len(lengths) if lengths else 3, H, Hkv, N, d, causal=causal,
                    varlen=(1, N) if lengths else None)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_large_grid_shapes(case):
    name, dt, d, causal, H, Hkv, N, lengths = case
    w = _workload(*case)
    # the grids are above the 4-wave bounds (so the 8-wave forms run)
    assert _grid(w.B, Hkv, N) > (512 if d == 64 else 256)
    if causal:
        assert _grid(w.B, H, N) > 256
    print(f"[shapes] {name} B {w.B} H {H}/{Hkv} N {N} d {d}", flush=True)
    inp = make_inputs(w, 31, lengths=lengths, with_grad=True)
    dinp = G.to_dev(inp)
    o, lse = G.gpu_fwd(w, dinp)
    grads = G.gpu_bwd(w, dinp, o, lse)
    last = w.B - 1
    pairs = [(0, 0), (last, Hkv - 1), (last, Hkv // 2)]
    rows = list(range(0, N, 37)) + [N - 1]
    G.check_fwd_sampled(w, inp, o, lse, [(b, g * (H // Hkv), rows) for b, g in pairs])
    G.check_bwd_heads(w, inp, grads, pairs, note="8-wave grid")

    # the first sequence alone: a grid under the bounds (4-wave forms), same rows
    n0 = lengths[0] if lengths else N
    w1 = w.with_(name=name + "_first", B=1, N=n0, varlen=None)
    assert _grid(1, Hkv, n0) <= (512 if d == 64 else 256) and _grid(1, H, n0) <= 256
    inp1 = dict(inp)
    if lengths is None:
        for key in ("q", "k", "v", "do"):
            inp1[key] = inp[key][:1].contiguous()
    else:
        for key in ("q", "k", "v", "do"):
            inp1[key] = inp[key][:n0].unsqueeze(0).contiguous()
        inp1["cu_seqlens"] = None
        inp1["max_seqlen"] = n0
    dinp1 = G.to_dev(inp1)
    o1, lse1 = G.gpu_fwd(w1, dinp1)
    grads1 = G.gpu_bwd(w1, dinp1, o1, lse1)
    G.check_bwd_heads(w1, inp1, grads1, [(0, 0), (0, Hkv - 1)], note="4-wave grid")
    # the forward has one shape for both grids: bit-identical rows
    of = o[:1] if lengths is None else o[:n0].unsqueeze(0)
    assert np.array_equal(G.f64(of), G.f64(o1))
    assert np.array_equal(G.f64(lse[:1, :, :n0]), G.f64(lse1))
