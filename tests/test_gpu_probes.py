"""Register and memory layouts that the gfx950 kernels rely on, checked on the device.

Each probe (libattn_probes.so, test-only) runs one wave on fixed-size buffers
and the expected result is computed here on the host from the documented
CDNA3/CDNA4 operand layouts:

* v_mfma_f32_32x32x16_bf16: lane l holds A[l % 32][8*(l // 32) + i] and
  B[8*(l // 32) + i][l % 32] (i = 0..7); accumulator register r of lane l is
  C[8*(r // 4) + 4*(l // 32) + r % 4][l % 32].
* v_permlane32_swap: swaps the upper half of the first operand with the lower
  half of the second.
* 16-byte direct-to-LDS loads: lane l's 16 bytes land at LDS base + 16*l.
* the packed fp32 -> bf16 convert rounds to nearest even.
"""

import ctypes
import os

import numpy as np
import pytest

from gpu_util import cuda_ok, log

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not cuda_ok(), reason="needs a GPU")]

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROBES = os.path.join(ROOT, "exact_attention_forward_tiled_amd", "libattn_probes.so")


@pytest.fixture(scope="module")
def lib():
    lib = ctypes.CDLL(PROBES)
    P, I = ctypes.c_void_p, ctypes.c_int
    for name, args in {"probe_mfma_bf16": [P, P, P, P], "probe_permlane32": [P, P],
                       "probe_lds_dma": [P, P, P], "probe_cvt_dot": [P, P, P, P],
                       "probe_mfma_fp4": [P, P, P, P, P, P]}.items():
        fn = getattr(lib, name)
        fn.restype = I
        fn.argtypes = args
    return lib


def _dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _sync():
    import torch
    torch.cuda.synchronize()


def test_mfma_bf16_layout(lib):
    import torch
    rng = np.random.default_rng(0)
    A = rng.integers(-4, 5, size=(32, 16)).astype(np.float32)   # exact in bf16
    B = rng.integers(-4, 5, size=(16, 32)).astype(np.float32)
    a_lane = np.zeros((64, 8), np.float32)
    b_lane = np.zeros((64, 8), np.float32)
    for l in range(64):
        for i in range(8):
            a_lane[l, i] = A[l % 32, 8 * (l // 32) + i]
            b_lane[l, i] = B[8 * (l // 32) + i, l % 32]
    a = torch.from_numpy(a_lane).to(torch.bfloat16).cuda()
    b = torch.from_numpy(b_lane).to(torch.bfloat16).cuda()
    c = torch.zeros((64, 16), dtype=torch.float32, device="cuda")
    log("probe mfma_bf16")
    assert lib.probe_mfma_bf16(a.data_ptr(), b.data_ptr(), c.data_ptr(), None) == 0
    _sync()
    C = A @ B
    got = c.cpu().numpy()
    want = np.zeros((64, 16), np.float32)
    for l in range(64):
        for r in range(16):
            want[l, r] = C[8 * (r // 4) + 4 * (l // 32) + r % 4, l % 32]
    assert np.array_equal(got, want)


def test_permlane32_swap(lib):
    import torch
    out = torch.zeros((64, 2), dtype=torch.int32, device="cuda")
    log("probe permlane32")
    assert lib.probe_permlane32(out.data_ptr(), None) == 0
    _sync()
    got = out.cpu().numpy()
    lanes = np.arange(64)
    first = np.where(lanes < 32, lanes, lanes - 32 + 100)      # upper half takes src's lower half
    second = np.where(lanes < 32, lanes + 32, lanes + 100)     # src's lower half takes old's upper
    assert np.array_equal(got[:, 0], first), got[:, 0]
    assert np.array_equal(got[:, 1], second), got[:, 1]
    # with both operands equal, each lane sees its own value and lane l ^ 32's
    x = lanes
    pair = np.sort(np.stack([np.where(lanes < 32, x, x - 32), np.where(lanes < 32, x + 32, x)]),
                   axis=0)
    assert np.array_equal(pair, np.sort(np.stack([x, x ^ 32]), axis=0))


def test_direct_to_lds_lane_map(lib):
    import torch
    src = _dev(np.arange(256, dtype=np.uint32).view(np.int32))
    out = torch.zeros(256, dtype=torch.int32, device="cuda")
    log("probe lds_dma")
    assert lib.probe_lds_dma(src.data_ptr(), out.data_ptr(), None) == 0
    _sync()
    got = out.cpu().numpy().view(np.uint32).reshape(64, 4)
    want = np.array([[4 * (63 - l) + i for i in range(4)] for l in range(64)], np.uint32)
    assert np.array_equal(got, want)


def test_bf16_convert_rounds_to_nearest_even(lib):
    import torch
    rng = np.random.default_rng(5)
    x = rng.standard_normal(128).astype(np.float32)
    x[:6] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -(1.0 + 2 ** -8), 0.0, 300.5]
    acc = np.zeros(64, np.float32)
    out = torch.zeros(128, dtype=torch.int32, device="cuda")
    log("probe cvt_dot")
    assert lib.probe_cvt_dot(_dev(x).data_ptr(), _dev(acc).data_ptr(), out.data_ptr(), None) == 0
    _sync()
    got = out.cpu().numpy().view(np.uint32).reshape(64, 2)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    want = ref[0::2].astype(np.uint32) | (ref[1::2].astype(np.uint32) << 16)
    assert np.array_equal(got[:, 0], want)
