"""The comparison helper the GPU parity tests use, checked on the CPU: a NaN
in a result must never pass a tolerance."""
import math

import numpy as np

from gpu_util import max_abs_err


def test_nan_is_an_infinite_error():
    assert max_abs_err([0.0, math.nan], [0.0, 0.0]) == math.inf
    assert max_abs_err([0.0, 1.0], [math.nan, 1.0]) == math.inf
    # Python's max() would drop the NaN; the helper must not
    assert max(0.0, math.nan) == 0.0
    assert not max_abs_err([[1.0, math.nan]], [[1.0, 2.0]]) <= 1e9


def test_equal_infinities_are_no_error():
    assert max_abs_err([-math.inf, 1.0], [-math.inf, 1.25]) == 0.25
    assert max_abs_err([-math.inf], [math.inf]) == math.inf
    assert max_abs_err([-math.inf], [0.0]) == math.inf


def test_plain_difference_and_empty():
    assert max_abs_err(np.array([1.0, -2.0]), np.array([1.5, -2.0])) == 0.5
    assert max_abs_err(np.zeros((0, 3)), np.zeros((0, 3))) == 0.0


def test_build_rejects_kernels_with_scratch():
    """The build fails when a kernel spills to scratch memory: the parser of
    the compiler's resource-usage remarks names each such kernel."""
    from exact_attention_16_amd import build
    remarks = "\n".join([
        "x.h:1:1: remark: Function Name: _ZN2fa9fa_fwd_ppIDF16bLi128ELb1ELi8ELb0EEEvNS_7ProblemE",
        "x.h:1:1: remark:     VGPRs: 220",
        "x.h:1:1: remark:     ScratchSize [bytes/lane]: 0",
        "x.h:1:1: remark: Function Name: _ZN2fa9fa_fwd_k4IDF16_Li64ELb0ELi8ELb0EEEvNS_7ProblemE",
        "x.h:1:1: remark:     VGPRs: 256",
        "x.h:1:1: remark:     ScratchSize [bytes/lane]: 12",
    ])
    assert build.scratch_use(remarks) == [("_ZN2fa9fa_fwd_k4IDF16_Li64ELb0ELi8ELb0EEEvNS_7ProblemE", 12)]
    assert build.scratch_use(remarks.replace(": 12", ": 0")) == []
