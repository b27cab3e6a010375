"""Exhaustive check of the kernels' bf16 reciprocal against IEEE division
(the refit's bit-exactness depends on it being correctly rounded)."""
import ctypes

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def test_rcp_bf16_exhaustive():
    import torch
    import quantized_linear_attention_amd as stq
    lib = ctypes.CDLL(stq.library_path())
    lib.stq_debug_rcp_bf16.restype = ctypes.c_int32
    out = torch.empty(65536, dtype=torch.float32, device="cuda")
    assert lib.stq_debug_rcp_bf16(ctypes.c_void_p(out.data_ptr()),
                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    b = np.arange(65536, dtype=np.uint32)
    x = (b << 16).view(np.float32)
    with np.errstate(divide="ignore", over="ignore"):
        ref = (np.float32(1.0) / x).astype(np.float32)      # IEEE binary32 division
    # positive normal bf16 whose reciprocal is normal: exponent field 1..252
    e = (b >> 7) & 0xFF
    ok = (b < 0x8000) & (e >= 1) & (e <= 252)
    assert ok.sum() == 252 * 128
    bad = np.nonzero(got[ok].view(np.uint32) != ref[ok].view(np.uint32))[0]
    assert bad.size == 0, "first mismatches at bf16 %s" % b[ok][bad[:5]]
