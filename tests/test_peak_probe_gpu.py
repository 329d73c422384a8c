"""GPU check of the benchmark's ceiling probes (libbsa_peak.so): small launches of both probes
return success and leave finite, expected outputs.  The probes are not part of the attention
path; the benchmark uses them to report roofline fractions against measured ceilings."""

import ctypes
import os

import pytest
import torch

from block_sparse_attention_landmark_amd import build as B

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def peak(gpu):
    if not os.path.exists(B.PEAK_LIB):
        pytest.fail("libbsa_peak.so is not built; run `python -m block_sparse_attention_landmark_amd.build`")
    lib = ctypes.CDLL(B.PEAK_LIB)
    lib.bsa_peak_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.bsa_peak_mfma.restype = ctypes.c_int
    lib.bsa_peak_gather.argtypes = [ctypes.c_void_p, ctypes.c_uint32, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_void_p, ctypes.c_void_p]
    lib.bsa_peak_gather.restype = ctypes.c_int
    return lib


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def test_peak_mfma_small(peak):
    n_wg, iters = 8, 10
    out = torch.full((n_wg * 256,), float("nan"), dtype=torch.float32, device="cuda")
    assert peak.bsa_peak_mfma(ctypes.c_void_p(out.data_ptr()), n_wg, iters, _stream()) == 0
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    # invalid arguments are rejected before any launch
    assert peak.bsa_peak_mfma(ctypes.c_void_p(out.data_ptr()), 0, iters, _stream()) != 0


def test_peak_gather_small(peak):
    n_blocks, n_wg, bpw = 4096, 8, 16                 # a 64 MiB buffer of 16 KB blocks
    src = torch.full((n_blocks * 16384,), 7, dtype=torch.uint8, device="cuda")
    out = torch.zeros(n_wg * 256, dtype=torch.int32, device="cuda")
    assert peak.bsa_peak_gather(ctypes.c_void_p(src.data_ptr()), n_blocks, n_wg, bpw,
                                ctypes.c_void_p(out.data_ptr()), _stream()) == 0
    torch.cuda.synchronize()
    # every gathered byte is 7, so every word read back from the LDS ring is 0x07070707
    assert (out == 0x07070707).all()
    assert peak.bsa_peak_gather(ctypes.c_void_p(src.data_ptr()), 0, n_wg, bpw,
                                ctypes.c_void_p(out.data_ptr()), _stream()) != 0
