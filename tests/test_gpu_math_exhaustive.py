"""Exhaustive equality of the producers' scalar math: every one of the 2^32 f32 inputs.

The GLU producers inline fixed f32 operation sequences for e^x and erfc (the pages give the
activation formulas, SwiGLU and GeGLU-erf, but no exp or erf); the RMS producer and the
quantizer rely on correctly rounded f32 square root and division. Bit-exact producer parity on
sampled workloads does not show that the device and the host oracle agree on every input, so
here the device evaluates each function on all 2^32 bit patterns (qimg_eval_math, chunk by
chunk) and the host compares each chunk with the oracle's evaluation, bit for bit; a NaN
output only has to be NaN on both sides (payloads are not part of the contract).
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import helpers as H
from oracle import oracle as O
from q8_activation_quant_amd import qimg

CHUNK = 1 << 27
THREADS = 16 if (os.cpu_count() or 1) >= 16 else 8  # divides CHUNK

ORACLE = {
    "exp": lambda x, out: O.exp_q(x, out),
    "erfc": lambda x, out: O.erfc_q(x, out),
    "swiglu": lambda x, out: O.glu_act(x, "swiglu", out),
    "geglu_erf": lambda x, out: O.glu_act(x, "geglu_erf", out),
    "rsqrt": lambda x, out: O.rms_scale(x, out),
    "qscale": lambda x, out: O.quant_recip(x, out),
    "qdiv": lambda x, out: O.quant_scale(x, out),
    "f2h": lambda x, out: O.f32_to_f16_words(x, out),
    "reglu": lambda x, out: O.glu_act(x, "reglu", out),
    "geglu": lambda x, out: O.glu_act(x, "geglu", out),
    "geglu_quick": lambda x, out: O.glu_act(x, "geglu_quick", out),
    "swiglu_oai_gate": lambda x, out: O.glu_pair(x, "swiglu_oai", 0.0, out=out),
}


def _is_nan(fn, bits):
    """NaN results (any payload): f32 NaNs, or binary16 NaNs for the f16 conversion."""
    if fn == "f2h":
        return ((bits & 0x7C00) == 0x7C00) & ((bits & 0x3FF) != 0)
    return np.isnan(bits.view(np.float32))


class _Slot:
    """Reusable host buffers of one worker (first-touch page faults dominate otherwise)."""

    def __init__(self, n):
        self.base = np.arange(n, dtype=np.uint32)
        self.x = np.empty(n, dtype=np.uint32)
        self.want = np.empty(n, dtype=np.float32)
        self.bad = np.empty(n, dtype=bool)

    def compare(self, fn, first, got_bits):
        """Oracle on bit patterns first + i (mod 2^32); returns (mismatches, first few cases)."""
        np.add(self.base, np.uint32(first & 0xFFFFFFFF), out=self.x)
        ORACLE[fn](self.x.view(np.float32), self.want)
        wb = self.want.view(np.uint32)
        np.not_equal(wb, got_bits, out=self.bad)
        if not self.bad.any():
            return 0, []
        self.bad &= ~(_is_nan(fn, wb) & _is_nan(fn, got_bits))
        idx = np.flatnonzero(self.bad)
        return idx.size, [(int(self.x[i]), int(wb[i]), int(got_bits[i])) for i in idx[:4]]


def test_chunk_compare_finds_planted_mismatches():
    """Host side only: one flipped bit is found, a different NaN payload is not a mismatch."""
    n, first = 4096, 0x7F7FF800  # runs from finite values through +inf into NaN patterns
    slot = _Slot(n)
    x = (np.arange(n, dtype=np.uint32) + np.uint32(first)).view(np.float32)
    got = O.glu_act(x, "swiglu").view(np.uint32).copy()
    assert slot.compare("swiglu", first, got) == (0, [])
    nan_at = int(np.flatnonzero(np.isnan(got.view(np.float32)))[0])
    got[nan_at] ^= 1  # another quiet NaN
    got[17] ^= 1 << 3
    nb, cases = slot.compare("swiglu", first, got)
    assert nb == 1 and cases[0][0] == first + 17


@pytest.mark.gpu
@pytest.mark.parametrize("fn", list(ORACLE))
def test_activation_math_all_f32_inputs(fn):
    torch = H.torch()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    out = torch.empty(CHUNK, dtype=torch.float32, device="cuda")
    host = torch.empty(CHUNK, dtype=torch.float32, pin_memory=True)
    host_bits = host.numpy().view(np.uint32)
    step = CHUNK // THREADS
    slots = [_Slot(step) for _ in range(THREADS)]
    total_bad, examples = 0, []
    with ThreadPoolExecutor(THREADS) as pool:
        for first in range(0, 1 << 32, CHUNK):
            qimg.eval_math(fn, first, out)
            host.copy_(out, non_blocking=True)
            torch.cuda.synchronize()
            jobs = [pool.submit(slots[k].compare, fn, first + k * step, host_bits[k * step:(k + 1) * step])
                    for k in range(THREADS)]
            for j in jobs:
                nb, cases = j.result()
                total_bad += nb
                examples.extend(cases)
    assert total_bad == 0, "%s: %d of 2^32 inputs differ; (x bits, oracle bits, device bits): %s" % (
        fn, total_bad, [tuple(hex(v) for v in c) for c in examples[:8]])


@pytest.mark.gpu
def test_eval_math_rejects_bad_arguments():
    torch = H.torch()
    out = torch.empty(16, dtype=torch.float32, device="cuda")
    with pytest.raises(qimg.QimgError):
        qimg.eval_math(12, 0, out)
    st = qimg.lib().qimg_eval_math(0, 0, (1 << 32) + 1, qimg._ptr(out), None)
    assert st == qimg.EINVAL
    assert qimg.lib().qimg_eval_math(0, 0, 0, None, None) == qimg.OK
