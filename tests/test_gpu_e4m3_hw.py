"""The fp8 quantiser's fast path, checked exhaustively on the GPU (tests/e4m3_hw_check.hip):
the hardware e4m3 conversion against an encoder written from the format definition for every fp32
pattern below 464 in magnitude and every NaN, and the reciprocal-and-correction quotient against
the correctly rounded one for every pair of bf16 values (v, block maximum) that takes that path and
for 2^32 pseudo-random fp32 pairs.
The quantiser's codes themselves are compared with the oracle in test_gpu_parity.py
(test_fp8_quantiser_sweep and the fp8 workloads)."""
import ctypes
import os

import pytest
import torch

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libe4m3_hw_check.so")


def test_e4m3_hardware_conversion_and_quotient_exhaustive():
    print("[gpu] e4m3 hardware conversion and quotient, exhaustive", flush=True)
    assert os.path.exists(LIB), "tests/libe4m3_hw_check.so is not built; run __graft_entry__.build()"
    lib = ctypes.CDLL(LIB)
    lib.e4m3_hw_check.argtypes = [ctypes.POINTER(ctypes.c_ulonglong)]
    torch.cuda.init()
    counts = (ctypes.c_ulonglong * 6)()
    assert lib.e4m3_hw_check(counts) == 0
    enc_inputs, enc_bad, pairs, pair_bad, rnd_pairs, rnd_bad = list(counts)
    # |d| < 464: 2 * (0x43E80000) patterns; NaN: 2 * (2^23 - 1)
    assert enc_inputs == 2 * 0x43E80000 + 2 * ((1 << 23) - 1)
    assert enc_bad == 0
    assert pairs > 2_000_000_000
    assert pair_bad == 0
    assert rnd_pairs > 4_000_000_000
    assert rnd_bad == 0
