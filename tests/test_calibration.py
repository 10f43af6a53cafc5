"""The measurement calibration library (include/ttt_peak.h, libttt_peak.so):
it exports every declared symbol and rejects bad arguments on the host (CPU);
on the GPU its copy kernel copies exactly, the device reports the expected
geometry and the MFMA loop produces finite output."""
import ctypes
import os
import re

import pytest

from weights_ttt_layer_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ttt_peak.h")


@pytest.fixture(scope="module")
def plib():
    return binding.load_peak_library()


def test_exports_every_declared_symbol(plib):
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(ttt_peak_[a-z0-9_]+)\s*\(", text)))
    assert names == ["ttt_peak_copy", "ttt_peak_device_info", "ttt_peak_mfma", "ttt_peak_mfma_flops"]
    for n in names:
        assert hasattr(plib, n), f"libttt_peak.so does not export {n}"


def test_rejects_bad_arguments_before_any_hip_call(plib):
    buf = ctypes.create_string_buffer(64)
    p = ctypes.cast(buf, ctypes.c_void_p)
    q = ctypes.c_void_p(p.value + 32)
    assert plib.ttt_peak_copy(None, q, 16, None) == 1
    assert plib.ttt_peak_copy(p, q, 0, None) == 1
    assert plib.ttt_peak_copy(p, q, 24, None) == 1                         # not a multiple of 16
    assert plib.ttt_peak_copy(p, ctypes.c_void_p(p.value + 16), 32, None) == 1   # overlap
    assert plib.ttt_peak_mfma(None, 1, 1, None) == 1
    assert plib.ttt_peak_mfma(p, 0, 1, None) == 1
    assert plib.ttt_peak_mfma(p, 1, 0, None) == 1


def test_mfma_flop_count(plib):
    # four waves per workgroup, four 32x32x16 products per iteration
    assert plib.ttt_peak_mfma_flops(3, 7) == 3 * 4 * 7 * 4 * 2 * 32 * 32 * 16


@pytest.mark.gpu
def test_peak_kernels_on_device():
    import torch
    info = binding.peak_device_info(0)
    print(f"device: {info}", flush=True)
    assert info["wavefront_size"] == 64 and info["compute_units"] >= 1 and info["clock_khz"] > 0
    src = torch.randint(-2**31, 2**31 - 1, (3 * 4096 + 4,), dtype=torch.int32, device="cuda")
    dst = torch.zeros_like(src)
    binding.peak_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    out = torch.full((2 * 256,), float("nan"), dtype=torch.float32, device="cuda")
    flops = binding.peak_mfma(out, 2, 10)
    torch.cuda.synchronize()
    assert flops == 2 * 4 * 10 * 4 * 32768 and bool(torch.isfinite(out).all())
