"""gfx950's hardware f32 -> e4m3 pair conversion equals the e4m3 rounding
formula (nearest, ties to even; the format of "Enabling trillion-parameter
models on AWS EFA", section "Evaluation": block-scaled fp8 dispatch) on every
fp32 value of magnitude at most 448, both signs and both halves of the
packed result: the quantising sender encodes with it after clamping to 448.
The check runs in a test helper kernel (tests/native/fp8_convert_check.hip),
not in the library."""
import ctypes
import os

import pytest
import torch

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "native",
                   "libfp8_convert_check.so")


def test_hardware_conversion_matches_the_formula():
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} is missing: build first (__graft_entry__.build())")
    lib = ctypes.CDLL(LIB)
    lib.fp8_convert_check.argtypes = [ctypes.c_void_p] * 3
    lib.fp8_convert_check.restype = ctypes.c_int
    counts = torch.zeros(2, dtype=torch.int64, device="cuda")
    first_bad = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    rc = lib.fp8_convert_check(counts.data_ptr(), first_bad.data_ptr(),
                               torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    checked, bad = counts.tolist()
    assert checked == 0x43E00000 + 1          # every bit pattern from +0 to 448
    assert bad == 0, f"first mismatch at bits {first_bad.item() & 0xffffffff:#010x}"
