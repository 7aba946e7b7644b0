"""Host-side checks of the GPU parity gate (no GPU): which errors the 16-bit O
gate lets through, on hand-made arrays.

The bar is O max-abs <= 1e-2 against the fp64 reference. A correctly rounded
bf16 value is within half an ulp of the reference: 2^-9 = 0.00195 for
|O| in [1, 2), 0.0039 in [2, 4) and 0.0078 in [4, 8). So for |O_ref| < 4 the
raw error is gated; only where half an ulp reaches 1e-2 (|O_ref| >= 4 in
bf16) is the error beyond rounding gated instead.
"""

import numpy as np
import pytest

import gpu_util as gu
from exact_io_aware_43_amd.workloads import Workload

W16 = Workload("gate", "bf16", 1, 1, 1, 4, 64)
W32 = Workload("gate32", "fp32", 1, 1, 1, 4, 64)


def _fwd(w, o, o_ref):
    o, o_ref = np.asarray(o, dtype=np.float64), np.asarray(o_ref, dtype=np.float64)
    z = np.zeros(1)
    return gu._compare_fwd(w, o, o_ref, z, z)


def test_half_ulp_values():
    assert gu.half_ulp(np.array([1.0]), "bf16")[0] == 2.0 ** -8
    assert gu.half_ulp(np.array([1.5]), "bf16")[0] == 2.0 ** -8
    assert gu.half_ulp(np.array([3.0]), "bf16")[0] == 2.0 ** -7
    assert gu.half_ulp(np.array([0.75]), "bf16")[0] == 2.0 ** -9
    assert gu.half_ulp(np.array([40.0]), "fp16")[0] == 2.0 ** -6


@pytest.mark.parametrize("ref,err,ok", [
    (3.0, 0.0099, True),    # |O| in [2, 4): raw error gated, just inside
    (3.0, 0.0101, False),   # the old excess-over-rounding gate allowed up to 0.0178 here
    (1.5, 0.0101, False),
    (0.2, 0.0099, True),
    (5.0, 0.0150, True),    # |O| >= 4: half an ulp is 0.0156 > 1e-2; gate the excess (0.015 - 0.0156 < 0)
    (5.0, 0.0260, False),   # excess 0.0104
    (-3.5, -0.0101, False),
])
def test_bf16_gate(ref, err, ok):
    # other elements exact; enough of them that the relative RMS stays far below its bar
    o_ref = np.concatenate([[ref], np.full(100000, 1.0)])
    o = o_ref.copy()
    o[0] += err
    if ok:
        _fwd(W16, o, o_ref)
    else:
        with pytest.raises(AssertionError):
            _fwd(W16, o, o_ref)


def test_fp32_gate_is_raw():
    _fwd(W32, [1.0 + 9e-6], [1.0])
    with pytest.raises(AssertionError):
        _fwd(W32, [1.0 + 1.1e-5], [1.0])


def test_records_and_report(tmp_path):
    n0 = len(gu.RECORDS)
    _fwd(W16, [1.0], [1.0])
    assert len(gu.RECORDS) == n0 + 1 and gu.RECORDS[-1]["workload"] == "gate"
    gu.write_report(str(tmp_path / "parity.json"))
    assert (tmp_path / "parity.json.md").read_text().startswith("# GPU parity")
    del gu.RECORDS[n0:]


def test_report_folds_the_randomized_grid(tmp_path):
    n0 = len(gu.RECORDS)
    saved = gu.CURRENT_TEST["id"]
    try:
        gu.CURRENT_TEST["id"] = "tests/test_sweep.py::test_sweep_case[s1_case]"
        _fwd(W16, [1.0], [1.0])
        gu.CURRENT_TEST["id"] = "tests/test_other.py::test_one"
        _fwd(W16, [1.0], [1.0])
    finally:
        gu.CURRENT_TEST["id"] = saved
    gu.write_report(str(tmp_path / "parity.json"))
    text = (tmp_path / "parity.json.md").read_text()
    assert "## Randomized instance grids" in text and "| fwd | 1 |" in text
    assert "test_sweep_case[s1_case]" not in text and "tests/test_other.py::test_one" in text
    del gu.RECORDS[n0:]
