"""The CPU wave model (wave64.py) held against the GPU.

tests/hip/lane_probe.hip runs single wave64 operations on per-lane inputs:
v_permlane32_swap through its compiler builtin (which result is which),
ds_bpermute, the transposing LDS read ds_read_b64_tr_b16 and the bf16 matrix
core v_mfma_f32_32x32x16_bf16. Each result is compared with the model: exactly
for the data movements, to fp32 accumulation rounding for the product.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

import wave64 as w
from gpu_util import say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hip", "liblane_probe.so")
RNG = np.random.default_rng(17)


@pytest.fixture(scope="module")
def probe():
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} is not built (python tests/hip/build.py)")
    lib = ctypes.CDLL(LIB)
    for name in ("lane_probe_swap", "lane_probe_bpermute", "lane_probe_tr16"):
        getattr(lib, name).argtypes = [ctypes.c_void_p] * 4
        getattr(lib, name).restype = ctypes.c_int
    lib.lane_probe_mfma.argtypes = [ctypes.c_void_p] * 5
    lib.lane_probe_mfma.restype = ctypes.c_int
    return lib


def call(fn, *tensors):
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = fn(*[ctypes.c_void_p(t.data_ptr()) for t in tensors], stream)
    assert rc == 0, f"launch status {rc}"
    torch.cuda.synchronize()


def dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dtype).to(DEV)


def test_permlane32_swap_results(probe):
    say("lane probe: permlane32_swap")
    x = RNG.integers(0, 2**31, 64)
    y = RNG.integers(0, 2**31, 64)
    out = torch.zeros(128, dtype=torch.int32, device=DEV)
    call(probe.lane_probe_swap, dev(x, torch.int32), dev(y, torch.int32), out)
    got = out.cpu().numpy().reshape(2, 64)
    want0, want1 = w.permlane32_swap(x, y)
    np.testing.assert_array_equal(got[0], want0)
    np.testing.assert_array_equal(got[1], want1)


def test_bpermute(probe):
    say("lane probe: ds_bpermute")
    for addr in (4 * RNG.integers(0, 64, 64), RNG.integers(0, 1024, 64) & ~3,
                 np.array([4 * (8 * (i >> 2) + (i & 3)) for i in range(64)])):
        data = RNG.integers(-2**30, 2**30, 64)
        out = torch.zeros(64, dtype=torch.int32, device=DEV)
        call(probe.lane_probe_bpermute, dev(addr, torch.int32), dev(data, torch.int32), out)
        np.testing.assert_array_equal(out.cpu().numpy(), w.ds_bpermute(addr, data))


def _tr16_addresses():
    """The flash kernels' transposing-read addresses (both head dims, every
    channel tile, both 8-row sections, both 16-key steps), and random ones."""
    import test_lane_maps as t
    sets = []
    for D in (64, 128):
        off = t.v_offsets(D)
        for mt in range(D // 32):
            for sec in range(2):
                for st in range(2):
                    sets.append(off[mt, sec] + st * 16 * 2 * D)
    sets.append(8 * RNG.integers(0, 1024, 64))
    return sets


def test_transposing_read(probe):
    say("lane probe: ds_read_b64_tr_b16")
    init = np.arange(4096)  # element index as the value
    lds = w.Lds(8192)
    lds.write16(0, init.astype(np.float64))
    for addr in _tr16_addresses():
        assert addr.min() >= 0 and addr.max() + 8 <= 8192 and (addr % 8 == 0).all()
        out = torch.zeros(256, dtype=torch.int16, device=DEV)
        call(probe.lane_probe_tr16, dev(init, torch.int16), dev(addr, torch.int32), out)
        got = out.cpu().numpy().astype(np.int64).reshape(64, 4)
        np.testing.assert_array_equal(got, w.ds_read_tr16_b64(lds, addr).astype(np.int64))


def _bf16_bits(x):
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def test_mfma_layout(probe):
    say("lane probe: v_mfma_f32_32x32x16_bf16")
    a_bits = _bf16_bits(RNG.standard_normal((64, 8)))
    b_bits = _bf16_bits(RNG.standard_normal((64, 8)))
    c = RNG.standard_normal((64, 16)).astype(np.float32)
    d = torch.zeros(64 * 16, dtype=torch.float32, device=DEV)
    call(probe.lane_probe_mfma, dev(a_bits.view(np.int16), torch.int16), dev(b_bits.view(np.int16), torch.int16),
         dev(c, torch.float32), d)
    to_f = lambda bits: (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    want = w.mfma_32x32x16(to_f(a_bits), to_f(b_bits), c.astype(np.float64))
    np.testing.assert_allclose(d.cpu().numpy().reshape(64, 16), want, rtol=1e-5, atol=1e-5)
