"""Helpers for the GPU parity tests: run libfa through its binding, run the oracle, compare.

Tolerances (fixed for this path): fp32 forward O max-abs <= 1e-5; 16-bit
forward O max-abs <= 1e-2 and relative RMS <= 5e-3, lse max-abs <= 1e-3;
16-bit backward relative RMS <= 1e-2 on each of dQ, dK, dV.

A 16-bit O is stored in its own type. Where half a unit in the last place of
that type at |O_ref| is below 1e-2 (|O_ref| < 4 in bf16, < 32 in fp16) a
correctly rounded output meets the 1e-2 bound, and the raw max-abs
|o - o_ref| is gated there. Only where half an ulp is 1e-2 or more can no
value of the type meet it; on those elements the gate is the error beyond that
rounding, |o - o_ref| - ulp(o_ref)/2 <= 1e-2. Both maxima are recorded.

Every comparison is appended to RECORDS (test id, workload, metrics); the test
session writes them out when FA_PARITY_REPORT names a file (see conftest.py).
"""

from __future__ import annotations

import numpy as np
import torch

import exact_io_aware_43_amd as fa
import oracle.attention as OA
from exact_io_aware_43_amd.workloads import Workload, make_inputs, seq_lengths

TOL_F32_O = 1e-5
TOL_O_MAX = 1e-2
TOL_O_RMS = 5e-3
TOL_LSE = 1e-3
TOL_GRAD_RMS = 1e-2


def rel_rms(x: np.ndarray, ref: np.ndarray) -> float:
    return float(np.linalg.norm((x - ref).ravel()) / max(np.linalg.norm(ref.ravel()), 1e-300))


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def to_dev(inp: dict) -> dict:
    out = dict(inp)
    for key in ("q", "k", "v", "do", "cu_seqlens", "alibi_slopes"):
        if out.get(key) is not None:
            out[key] = out[key].to("cuda")
    return out


def gpu_fwd(w: Workload, dinp: dict):
    o, lse = fa.attention(dinp["q"], dinp["k"], dinp["v"], causal=w.causal, softmax_scale=dinp["scale"],
                          alibi_slopes=dinp["alibi_slopes"], cu_seqlens=dinp["cu_seqlens"],
                          max_seqlen=dinp["max_seqlen"])
    torch.cuda.synchronize()
    return o, lse


def gpu_bwd(w: Workload, dinp: dict, o, lse):
    g = fa.attention_bwd(dinp["do"], dinp["q"], dinp["k"], dinp["v"], o, lse, causal=w.causal,
                         softmax_scale=dinp["scale"], alibi_slopes=dinp["alibi_slopes"],
                         cu_seqlens=dinp["cu_seqlens"], max_seqlen=dinp["max_seqlen"])
    torch.cuda.synchronize()
    return g


def check_fwd_full(w: Workload, inp: dict, o, lse):
    """Whole-tensor comparison with the fp64 oracle (small shapes)."""
    o_ref, lse_ref = OA.attention_fwd(inp["q"], inp["k"], inp["v"], scale=inp["scale"], causal=w.causal,
                                      alibi_slopes=inp["alibi_slopes"], cu_seqlens=inp["cu_seqlens"])
    og, lg = f64(o), f64(lse)
    lens = seq_lengths(inp, w)
    mask = np.zeros(lg.shape, dtype=bool)
    for b, n in enumerate(lens):
        mask[b, :, :n] = True
    return _compare_fwd(w, og, o_ref, lg[mask], lse_ref[mask], note="whole tensors")


_SIG_BITS = {"bf16": 8, "fp16": 11, "fp32": 24}
_MIN_SPACING = {"bf16": 2.0 ** -133, "fp16": 2.0 ** -24, "fp32": 2.0 ** -149}


def half_ulp(x: np.ndarray, dtype: str) -> np.ndarray:
    """Half the spacing of ``dtype`` values at |x| (normal range; subnormal spacing below)."""
    ax = np.abs(x)
    _, e = np.frexp(ax)  # ax = f * 2**e with f in [0.5, 1)
    ulp = np.ldexp(1.0, (e - _SIG_BITS[dtype]).astype(np.int64))
    ulp = np.where(ax == 0, _MIN_SPACING[dtype], np.maximum(ulp, _MIN_SPACING[dtype]))
    return 0.5 * ulp


RECORDS: list = []
CURRENT_TEST = {"id": None}


def record(kind: str, w: Workload, metrics: dict, **extra) -> None:
    RECORDS.append(dict(test=CURRENT_TEST["id"], kind=kind, workload=w.name, dtype=w.dtype, B=w.B, H=w.H,
                        Hkv=w.Hkv, N=w.N, d=w.d, causal=bool(w.causal), alibi=bool(w.alibi), **extra, **metrics))


def _compare_fwd(w, og, o_ref, lg, lref, note="", o_bar_scale=1.0):
    """Gate O, lse against the references. ``o_bar_scale`` multiplies the O
    max-abs bar: with dropout the kept probabilities are scaled by 256 / K, and
    every rounding error of the 16-bit probabilities with them."""
    assert np.isfinite(og).all() and np.isfinite(lg).all(), "non-finite output"
    diff = np.abs(og - o_ref)
    hu = half_ulp(o_ref, w.dtype)
    reach = hu < TOL_O_MAX  # a correctly rounded output can meet the bound here
    err_o = float(diff.max()) if og.size else 0.0
    err_reach = float(diff[reach].max()) if reach.any() else 0.0
    excess = float((diff - hu)[~reach].max()) if (~reach).any() else 0.0
    err_l = float(np.abs(lg - lref).max()) if lg.size else 0.0
    rms = rel_rms(og, o_ref) if og.size else 0.0
    out = dict(o_maxabs=err_o, o_maxabs_gated=err_reach, o_beyond_rounding=excess, n_beyond=int((~reach).sum()),
               o_relrms=rms, lse_maxabs=err_l, n_rows=int(lg.size))
    if o_bar_scale != 1.0:
        out["o_bar"] = TOL_O_MAX * o_bar_scale
    record("fwd", w, out, note=note)
    bar = TOL_O_MAX * o_bar_scale
    if w.dtype == "fp32":
        assert err_o <= TOL_F32_O, f"O max-abs {err_o:.3e} > {TOL_F32_O}"
    else:
        assert err_reach <= bar, f"O max-abs {err_reach:.3e} > {bar}"
        assert excess <= bar, f"O max-abs beyond output rounding {excess:.3e} > {bar} (|O| large)"
        assert rms <= TOL_O_RMS, f"O rel-RMS {rms:.3e} > {TOL_O_RMS}"
        assert err_l <= TOL_LSE, f"lse max-abs {err_l:.3e} > {TOL_LSE}"
    return out


def _head_view(inp, w, b, h):
    """fp64 arrays (q_h, k_g, v_g) of sequence b, query head h, and the sequence length."""
    G = w.H // w.Hkv
    g = h // G
    if inp["cu_seqlens"] is None:
        sl = (b, slice(None))
        n = w.N
    else:
        cu = inp["cu_seqlens"].tolist()
        sl = (slice(cu[b], cu[b + 1]),)
        n = cu[b + 1] - cu[b]
    q = inp["q"][sl][:, h]
    k = inp["k"][sl][:, g]
    v = inp["v"][sl][:, g]
    return q, k, v, n, sl


def check_fwd_sampled(w: Workload, inp: dict, o, lse, samples, note="sampled rows"):
    """Compare sampled rows of O and lse: ``samples`` is a list of (b, h, rows)."""
    ogs, orefs, lgs, lrefs = [], [], [], []
    og_all, lg_all = o.cpu(), lse.cpu()
    for b, h, rows in samples:
        q, k, v, n, sl = _head_view(inp, w, b, h)
        rows = np.array([r for r in rows if 0 <= r < n], dtype=np.int64)
        if rows.size == 0:
            continue
        slope = None if inp["alibi_slopes"] is None else float(inp["alibi_slopes"][h])
        o_ref, l_ref = OA.head_rows_fwd(OA._f64(q), OA._f64(k), OA._f64(v), rows, inp["scale"], w.causal, slope)
        ogs.append(f64(og_all[sl][:, h][rows]))
        orefs.append(o_ref)
        lgs.append(f64(lg_all[b, h])[rows])
        lrefs.append(l_ref)
    return _compare_fwd(w, np.concatenate(ogs), np.concatenate(orefs), np.concatenate(lgs), np.concatenate(lrefs),
                        note=note)


def check_bwd_full(w: Workload, inp: dict, grads):
    ref = OA.attention_bwd(inp["q"], inp["k"], inp["v"], inp["do"], scale=inp["scale"], causal=w.causal,
                           alibi_slopes=inp["alibi_slopes"], cu_seqlens=inp["cu_seqlens"])
    return _compare_bwd(w, [f64(g) for g in grads], ref, note="whole tensors")


TOL_ZERO_GRAD_RMS = 1e-3


def _compare_bwd(w, got, ref, note=""):
    """Relative RMS per gradient. A reference that is exactly zero (one key per
    row: P = 1 and dS = 0, so dQ = dK = 0) has no relative error; there the
    absolute RMS of the result must be below 1e-3 instead."""
    out = {}
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        assert np.isfinite(g).all(), f"non-finite {name}"
        if not np.any(r):
            out[name + "_abs_rms"] = float(np.sqrt(np.mean(g ** 2))) if g.size else 0.0
        else:
            out[name] = rel_rms(g, r)
    record("bwd", w, out, note=note)
    for name in ("dq", "dk", "dv"):
        if name in out:
            assert out[name] <= TOL_GRAD_RMS, f"{name} rel-RMS {out[name]:.3e} > {TOL_GRAD_RMS}"
        else:
            e = out[name + "_abs_rms"]
            assert e <= TOL_ZERO_GRAD_RMS, f"{name} abs-RMS {e:.3e} > {TOL_ZERO_GRAD_RMS} (zero reference)"
    return out


def check_bwd_heads(w: Workload, inp: dict, grads, pairs, note="whole (sequence, kv head) groups"):
    """Full-size backward check on whole (b, kv head) groups: every query head of
    the group is recomputed by the oracle, so dK and dV of that kv head and dQ of
    those query heads are exact references."""
    dq, dk, dv = (g.cpu() for g in grads)
    G = w.H // w.Hkv
    got, ref = [[], [], []], [[], [], []]
    for b, g in pairs:
        dk_sum = dv_sum = None
        for h in range(g * G, (g + 1) * G):
            q, k, v, n, sl = _head_view(inp, w, b, h)
            do = inp["do"][sl][:, h]
            slope = None if inp["alibi_slopes"] is None else float(inp["alibi_slopes"][h])
            rq, rk, rv = OA.head_bwd(OA._f64(q), OA._f64(k), OA._f64(v), OA._f64(do), inp["scale"], w.causal, slope)
            got[0].append(f64(dq[sl][:, h]))
            ref[0].append(rq)
            dk_sum = rk if dk_sum is None else dk_sum + rk
            dv_sum = rv if dv_sum is None else dv_sum + rv
        got[1].append(f64(dk[sl][:, g]))
        ref[1].append(dk_sum)
        got[2].append(f64(dv[sl][:, g]))
        ref[2].append(dv_sum)
    return _compare_bwd(w, [np.concatenate(x) for x in got], [np.concatenate(x) for x in ref],
                        note=f"{note} {pairs}")


def small(w_name_or_w, **kw) -> Workload:
    from exact_io_aware_43_amd.workloads import WORKLOADS

    w = WORKLOADS[w_name_or_w] if isinstance(w_name_or_w, str) else w_name_or_w
    return w.with_(**kw)


__all__ = [name for name in dir() if not name.startswith("_")] + ["make_inputs"]


_NAMED = ("fp32_small", "gpt2m", "long_causal", "varlen_alibi", "gqa")


def _fmt(x):
    return "—" if x is None else (f"{x:.2e}" if isinstance(x, float) else str(x))


def _in_grid(r) -> bool:
    return "::test_sweep_" in (r.get("test") or "")


def write_report(path: str) -> None:
    """RECORDS as JSON at ``path`` and as Markdown tables at ``path + '.md'``: the
    named workloads at full size first (worst value of each metric over their
    checks), then every comparison of the session."""
    import json
    import os

    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "w") as f:
        json.dump(RECORDS, f, indent=1)
    fwd_keys = ("o_maxabs_gated", "o_beyond_rounding", "o_maxabs", "o_relrms", "lse_maxabs")
    bwd_keys = ("dq", "dk", "dv")
    lines = ["# GPU parity against the fp64 oracle", "",
             "Bars: fp32 O max-abs <= 1e-5; 16-bit O max-abs <= 1e-2 (raw, on elements where half an ulp of the",
             "output type is below 1e-2; beyond that rounding elsewhere), O relative RMS <= 5e-3, lse max-abs <= 1e-3;",
             "dQ, dK, dV relative RMS <= 1e-2. FP8 forward (against the FP8 oracle's exact attention of the",
             "dequantized inputs): lse max-abs <= 1e-3, O relative RMS <= 0.05 and <= 0.15 per query row; RMSE",
             "against fp64 within 1.3x the oracle's own (kind fp8_rmse).", "",
             "## Named workloads at full size (worst over their checks)", "",
             "| workload | pass | checks | " + " | ".join(fwd_keys) + " | " + " | ".join(b + " rel-RMS" for b in bwd_keys)
             + " |",
             "|" + "---|" * (3 + len(fwd_keys) + len(bwd_keys))]
    for name in _NAMED:
        for kind in ("fwd", "bwd"):
            rs = [r for r in RECORDS if r["workload"] == name and r["kind"] == kind]
            if not rs:
                continue
            keys = fwd_keys if kind == "fwd" else bwd_keys
            vals = {k: max((r[k] for r in rs if k in r), default=None) for k in keys}
            cells = [_fmt(vals.get(k)) if k in keys else "" for k in fwd_keys + bwd_keys]
            lines.append(f"| {name} | {kind} | {len(rs)} | " + " | ".join(cells) + " |")
    # the randomized grid: one row per pass, worst value over its cases
    grid = [r for r in RECORDS if _in_grid(r)]
    if grid:
        lines += ["", "## Randomized instance grids (tests/test_sweep.py: plain, and window / softcap / dropout; worst over their cases)", "",
                  "| pass | cases | " + " | ".join(fwd_keys) + " | " + " | ".join(b + " rel-RMS" for b in bwd_keys) + " |",
                  "|" + "---|" * (2 + len(fwd_keys) + len(bwd_keys))]
        for kind in ("fwd", "bwd"):
            rs = [r for r in grid if r["kind"] == kind]
            keys = fwd_keys if kind == "fwd" else bwd_keys
            vals = {k: max((r[k] for r in rs if k in r), default=None) for k in keys}
            cells = [_fmt(vals.get(k)) if k in keys else "" for k in fwd_keys + bwd_keys]
            lines.append(f"| {kind} | {len(rs)} | " + " | ".join(cells) + " |")
    lines += ["", "## Every other comparison", "",
              "| test | workload | pass | note | metrics |", "|---|---|---|---|---|"]
    skip = {"test", "kind", "workload", "note", "dtype", "B", "H", "Hkv", "N", "d", "causal", "alibi"}
    for r in RECORDS:
        if _in_grid(r):
            continue
        shape = f"{r['dtype']} B{r['B']} H{r['H']}/{r['Hkv']} N{r['N']} d{r['d']} c{int(r['causal'])} a{int(r['alibi'])}"
        m = ", ".join(f"{k}={_fmt(v)}" for k, v in r.items() if k not in skip)
        lines.append(f"| {r['test']} | {r['workload']} ({shape}) | {r['kind']} | {r.get('note', '')} | {m} |")
    with open(path + ".md", "w") as f:
        f.write("\n".join(lines) + "\n")
