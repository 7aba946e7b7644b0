"""GPU decode over a key/value cache (fa_fwd_kvcache) against the fp64 oracle
(oracle.attention.decode_fwd), at the forward bars: O max-abs <= 1e-2 (raw where
a correctly rounded 16-bit value can meet it), O relative RMS <= 5e-3, lse
max-abs <= 1e-3; queries that see no key must give O = 0 and lse = -inf.

Covers one and several key splits (auto, 1, 3, 8 ranges), GQA groups whose
G * Nq query rows span several 32-row groups, per-sequence cache lengths
(including 1, lengths below Nq and an empty cache), ALiBi, both 16-bit types,
and the decode of the last tokens of a sequence against the GPU's own
prefill forward. Source: "FlashAttention: Faster Attention Without Dropping a
Single Interaction", Key design 2 (merging the states of disjoint key sets)
and Limitations (long context and inference).
"""

import numpy as np
import pytest
import torch

import exact_io_aware_43_amd as fa
import oracle.attention as OA
from gpu_util import _compare_fwd, f64
from exact_io_aware_43_amd.workloads import Workload, alibi_slopes, make_decode_inputs

pytestmark = pytest.mark.gpu


def _banner(msg):
    print(f"[decode] {msg}", flush=True)


def _run(w, inp, num_splits, causal=True):
    dev = {k: (v.to("cuda") if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    o, lse = fa.attention_kvcache(dev["q"], dev["k_cache"], dev["v_cache"], dev["cache_seqlens"], causal=causal,
                                  softmax_scale=inp["scale"], alibi_slopes=dev["alibi_slopes"],
                                  num_splits=num_splits)
    torch.cuda.synchronize()
    return o, lse


def _check(w, inp, o, lse, causal=True, note=""):
    o_ref, lse_ref = OA.decode_fwd(inp["q"], inp["k_cache"], inp["v_cache"], inp["cache_seqlens"].numpy(),
                                   scale=inp["scale"], causal=causal, alibi_slopes=inp["alibi_slopes"])
    og, lg = f64(o), f64(lse)
    seen = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lg), seen), "queries that see no key must have lse = -inf, others finite"
    assert np.all(og.transpose(0, 2, 1, 3)[~seen] == 0.0), "O of a query that sees no key must be 0"
    return _compare_fwd(w, og, o_ref, lg[seen], lse_ref[seen], note=note)


CASES = [
    # (B, H, Hkv, Nq, Nk, d, lengths, alibi, dtype)
    (3, 8, 2, 1, 1000, 128, [1000, 1, 517], False, "bf16"),
    (3, 8, 2, 4, 1000, 128, [1000, 3, 517], True, "bf16"),
    (2, 4, 4, 1, 700, 64, [700, 129], False, "fp16"),
    (2, 32, 1, 2, 600, 128, [600, 256], False, "bf16"),   # 64 query rows per kv head: two row groups
    (2, 16, 16, 3, 300, 64, [0, 300], True, "bf16"),      # an empty cache
]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}H{c[1]}kv{c[2]}q{c[3]}k{c[4]}d{c[5]}a{int(c[7])}{c[8]}"
                                             for c in CASES])
@pytest.mark.parametrize("num_splits", [0, 1, 3, 8])
@pytest.mark.parametrize("causal", [True, False])
def test_decode_parity(case, num_splits, causal):
    B, H, Hkv, Nq, Nk, d, lengths, alibi, dt = case
    w = Workload(f"decode_{dt}_d{d}", dt, B, H, Hkv, Nk, d, causal=causal, alibi=alibi)
    inp = make_decode_inputs(w, Nq, lengths, seed=70 + num_splits)
    _banner(f"{w} Nq={Nq} lengths={lengths} splits={num_splits}")
    o, lse = _run(w, inp, num_splits, causal)
    _banner(str(_check(w, inp, o, lse, causal, note=f"decode Nq={Nq} splits={num_splits}")))


def test_decode_matches_prefill_rows():
    """The last Nq tokens of a sequence decoded against its cache equal those rows of
    the (GPU) causal forward over the whole sequence, within the forward bars."""
    w = Workload("prefill", "bf16", 1, 8, 2, 777, 128, causal=True, alibi=True)
    from exact_io_aware_43_amd.workloads import make_inputs
    full = make_inputs(w, 71, with_grad=False)
    Nq = 5
    dev = {k: (v.to("cuda") if isinstance(v, torch.Tensor) else v) for k, v in full.items()}
    o_full, lse_full = fa.attention(dev["q"], dev["k"], dev["v"], causal=True, softmax_scale=full["scale"],
                                    alibi_slopes=dev["alibi_slopes"])
    q = dev["q"][:, -Nq:].contiguous()
    cl = torch.tensor([w.N], dtype=torch.int32, device="cuda")
    o, lse = fa.attention_kvcache(q, dev["k"], dev["v"], cl, causal=True, softmax_scale=full["scale"],
                                  alibi_slopes=dev["alibi_slopes"], num_splits=3)
    torch.cuda.synchronize()
    diff = (o.float() - o_full[:, -Nq:].float()).abs().max().item()
    ldiff = (lse - lse_full[:, :, -Nq:]).abs().max().item()
    _banner(f"decode vs prefill rows: O max-abs {diff:.3e}, lse max-abs {ldiff:.3e}")
    assert diff <= 1e-2 and ldiff <= 1e-3


def test_decode_full_size():
    """The decode workload at full size: B=8, H=32, Hkv=8, one new query per
    sequence, 16384 cached keys, d=128, causal, bf16, every output row checked."""
    from exact_io_aware_43_amd.workloads import DECODE
    w, Nq, lengths = DECODE
    inp = make_decode_inputs(w, Nq, lengths, seed=0)
    _banner(f"full size {w} Nq={Nq}")
    o, lse = _run(w, inp, 0, True)
    _banner(str(_check(w, inp, o, lse, True, note="decode workload, every row")))


@pytest.mark.parametrize("causal", [True, False])
def test_decode_balanced_ranges_over_many_short_caches(causal):
    """The automatic split's balanced ranges lay the caches of a kv head end to
    end, so one workgroup can cover several short caches (and the end and start
    of two long ones). Sixteen caches of 0 to 40 keys between two long ones, with
    empty and one-key caches among them, against the oracle; queries of empty
    caches get O = 0 and lse = -inf."""
    rng = np.random.default_rng(31)
    lengths = [1500] + [int(x) for x in rng.integers(0, 41, size=16)] + [2048]
    lengths[3], lengths[7] = 0, 1
    w = Workload("decode_many_short", "bf16", len(lengths), 8, 2, 2048, 128, causal=causal, alibi=True)
    inp = make_decode_inputs(w, 2, lengths, seed=33)
    _banner(f"{w} lengths={lengths}")
    o, lse = _run(w, inp, 0, causal)
    _banner(str(_check(w, inp, o, lse, causal, note="balanced ranges, many short caches")))
