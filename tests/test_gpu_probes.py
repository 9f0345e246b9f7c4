"""The measurement probes of kvc_tools.h on the GPU: each launches and ends,
the copy probe's destination equals its source byte for byte, and sizes that
do not split into whole loads are rejected before any launch."""
import ctypes as C

import pytest

pytestmark = pytest.mark.gpu


def _lib():
    from block_causal_kv_amd import _lib
    return _lib, _lib.load()


def test_copy_probe_copies_every_byte():
    import torch
    _l, lib = _lib()
    src = torch.randint(0, 256, (3 << 20,), dtype=torch.uint8, device="cuda")
    dst = torch.zeros_like(src)
    assert lib.kvc_probe_copy(C.c_void_p(src.data_ptr()), C.c_void_p(dst.data_ptr()), src.numel(), None) == 0
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


@pytest.mark.parametrize("nbytes", [4096, 3 * 4096, 1 << 20, (5 << 20) + 4096, 1 << 28])
def test_lds_load_probe_runs_and_ends(nbytes):
    import torch
    _l, lib = _lib()
    src = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    assert lib.kvc_probe_lds_load(C.c_void_p(src.data_ptr()), nbytes, None) == 0, lib.kvc_last_error()
    torch.cuda.synchronize()
    assert lib.kvc_probe_lds_load(C.c_void_p(src.data_ptr()), nbytes + 16, None) == _l.KVC_ERR_INVALID


def test_mfma_probe_runs_and_ends():
    import torch
    _l, lib = _lib()
    sink = torch.full((2 * 256,), float("nan"), dtype=torch.float32, device="cuda")
    assert lib.kvc_probe_mfma_bf16(C.c_void_p(sink.data_ptr()), 2, 8, None) == 0
    torch.cuda.synchronize()
    assert torch.isfinite(sink).all()
