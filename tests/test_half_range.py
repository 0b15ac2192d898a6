"""Host check of the IEEE half range limits that include/qt.h documents for the
GEMM operands (weights packed as half in bf16 mode; inputs half(x * gain)): the
thresholds quoted there must be what round-to-nearest-even half conversion does.
The GPU side of the same limits (a refused weight, the QT_STATUS_FP16_RANGE bit)
is tests/test_gpu_kernels.py."""
import os
import re

import numpy as np
import pytest

pytestmark = pytest.mark.filterwarnings("ignore:overflow encountered in cast:RuntimeWarning")

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "qt.h")


def _bf16(bits):
    return float(np.array([bits << 16], dtype=np.uint32).view(np.float32)[0])


def test_quoted_limits_match_half_rounding():
    text = open(HEADER).read()
    # the weight limit: the largest finite half; the input limit: the first value
    # that rounds to infinity
    assert re.search(r"\|w\| > 65504", text)
    assert re.search(r"\|x \* gain\| >= 65520", text)
    assert np.isfinite(np.float16(65504.0)) and np.float16(65504.0) == 65504.0
    assert np.isfinite(np.float16(np.float32(65519.996)))
    assert np.float16(np.float32(65519.996)) == 65504.0
    assert np.isinf(np.float16(np.float32(65520.0)))
    assert np.isinf(np.float16(np.float32(-65520.0)))


def test_values_the_gpu_tests_plant_are_beyond_the_range():
    # bf16 0x47C3 (the weight planted in the refusal test) exceeds the largest half
    w = _bf16(0x47C3)
    assert w == 99840.0 and w > 65504.0
    # bf16 0x4843 (the Talker input planted in the status test) overflows half(x * g)
    # for every gain above 65520 / 199680
    x = _bf16(0x4843)
    assert x == 199680.0
    g = 65520.0 / x
    assert 0.32 < g < 0.33
    assert np.isinf(np.float16(np.float32(x * 0.34)))
    assert np.isfinite(np.float16(np.float32(x * 0.32)))
