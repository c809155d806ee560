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
* ds_read_b64_tr_b16 (the transposing read of the backward kernels): within each
  group of 16 lanes, lane t returns element t % 4 of the 8-byte words addressed
  by lanes t // 4, t // 4 + 4, t // 4 + 8, t // 4 + 12 of the group.
* the packed fp32 -> bf16 convert rounds to nearest even.
* v_mfma_scale_f32_32x32x64_f8f6f4 with fp4 (E2M1) operands: lane l holds row
  (A) or column (B) l % 32 and the 32 k-elements 32*(l // 32) .. +31, element i
  in nibble i of its 16 bytes (low nibble first); lane l's E8M0 scale byte,
  picked from its 32-bit scale register by op_sel, scales exactly those 32
  elements; the accumulator layout is that of the bf16 product.
* v_cvt_scalef32_pk_fp4_f32 writes RNE(x / scale) onto the E2M1 grid (ties to
  the even code, saturating at +-6) into the selected byte, keeping the others;
  v_cvt_scalef32_pk_f32_fp4 decodes a selected byte times the scale.
* the same MFMA with fp8 (E4M3) operands: lane l holds row (A) or column (B)
  l % 32 in 32 bytes (8 registers); bytes 0-15 belong to k-block 0 (k 0..31)
  and bytes 16-31 to k-block 1 (k 32..63), each k-block being the 16-byte
  halves of lanes l % 32 and l % 32 + 32; the E8M0 byte of lane
  (l % 32) + 32*b scales k-block b of that row or column.  (The order of the
  elements inside a k-block is the same for A and B, so it does not show in
  the product; the model below takes byte i of lane half h as k = 16h + i.)
  The product of E4M3 operands is not rounded once in fp32: its error reaches
  about 2^-11 of the largest single product.
* v_cvt_scalef32_pk_fp8_f32 with scale 1 rounds to the nearest E4M3 value
  (ties to even, subnormals kept) and writes the two codes into the selected
  16-bit half, keeping the other.
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
                       "probe_mfma_fp4": [P, P, P, P, P, P],
                       "probe_mfma_fp4_sel2": [P, P, P, P, P, P],
                       "probe_cvt_fp4": [P, P, P, P], "probe_dec_fp4": [P, P, P, P],
                       "probe_mfma_fp8": [P, P, P, P, P, P], "probe_cvt_fp8": [P, P, P],
                       "probe_wave_place": [P, ctypes.c_int, P], "probe_tr16": [P, P, P]}.items():
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


@pytest.mark.parametrize("pattern", ["contiguous", "rows_of_a_tile"])
def test_transposing_lds_read_lane_map(lib, pattern):
    import torch
    lanes = np.arange(64)
    if pattern == "contiguous":
        addr = 4 * lanes
    else:
        # as the backward kernels address a tile of 64-word rows: lane a of a 16-lane group
        # reads row a // 4 (plus 8 per lane half), column quad a % 4 (plus 16 for odd groups)
        g, t = lanes // 16, lanes % 16
        addr = (8 * (g // 2) + t // 4) * 64 + 16 * (g % 2) + 4 * (t % 4)
    assert (addr % 4 == 0).all() and addr.min() >= 0 and addr.max() <= 1020
    a = _dev(addr.astype(np.int32))
    out = torch.zeros(256, dtype=torch.int16, device="cuda")
    log(f"probe tr16 {pattern}")
    assert lib.probe_tr16(a.data_ptr(), out.data_ptr(), None) == 0
    _sync()
    got = out.cpu().numpy().view(np.uint16).reshape(64, 4).astype(np.int64)
    want = np.zeros((64, 4), np.int64)
    for l in range(64):
        g, t = l // 16, l % 16
        for j in range(4):
            want[l, j] = addr[16 * g + 4 * j + t // 4] + t % 4
    assert np.array_equal(got, want)
    if pattern == "rows_of_a_tile":
        # lane t of each group gets column 16 (g % 2) + t of four consecutive rows
        for l in range(64):
            g, t = l // 16, l % 16
            rows = got[l] // 64
            cols = got[l] % 64
            assert (cols == 16 * (g % 2) + t).all() and (rows == 8 * (g // 2) + np.arange(4)).all()


def test_bf16_convert_rounds_to_nearest_even(lib):
    import torch
    rng = np.random.default_rng(5)
    x = rng.standard_normal(128).astype(np.float32)
    x[:6] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -(1.0 + 2 ** -8), 0.0, 300.5]
    acc = np.zeros(64, np.float32)
    out = torch.zeros(128, dtype=torch.int32, device="cuda")
    log("probe cvt_dot")
    xd, accd = _dev(x), _dev(acc)       # keep the device buffers alive across the launch
    assert lib.probe_cvt_dot(xd.data_ptr(), accd.data_ptr(), out.data_ptr(), None) == 0
    _sync()
    got = out.cpu().numpy().view(np.uint32).reshape(64, 2)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    want = ref[0::2].astype(np.uint32) | (ref[1::2].astype(np.uint32) << 16)
    assert np.array_equal(got[:, 0], want)


E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _fp4_value(code):
    return (-1.0 if code & 8 else 1.0) * E2M1[code & 7]


def _fp4_case(seed):
    rng = np.random.default_rng(seed)
    ca = rng.integers(0, 16, size=(64, 32)).astype(np.uint8)
    cb = rng.integers(0, 16, size=(64, 32)).astype(np.uint8)
    sa = rng.integers(124, 131, size=64).astype(np.uint32)
    sb = rng.integers(124, 131, size=64).astype(np.uint32)
    A = np.zeros((32, 64))
    B = np.zeros((64, 32))
    for l in range(64):
        for i in range(32):
            A[l % 32, 32 * (l // 32) + i] = _fp4_value(ca[l, i]) * 2.0 ** (int(sa[l]) - 127)
            B[32 * (l // 32) + i, l % 32] = _fp4_value(cb[l, i]) * 2.0 ** (int(sb[l]) - 127)
    C = A @ B
    want = np.array([[C[8 * (r // 4) + 4 * (l // 32) + r % 4, l % 32] for r in range(16)]
                     for l in range(64)])
    pack = lambda c: np.ascontiguousarray(c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
    return pack(ca), pack(cb), sa, sb, want, rng


def test_mfma_fp4_layout_and_scales(lib):
    import torch
    a, b, sa, sb, want, rng = _fp4_case(7)
    bufs = [_dev(a), _dev(b), _dev(sa.astype(np.uint8)), _dev(sb.astype(np.uint8))]
    c = torch.zeros((64, 16), dtype=torch.float32, device="cuda")
    log("probe mfma_fp4")
    assert lib.probe_mfma_fp4(*[t.data_ptr() for t in bufs], c.data_ptr(), None) == 0
    _sync()
    assert np.array_equal(c.cpu().numpy().astype(np.float64), want)
    # scale byte 2 of a 32-bit register (other bytes hold noise)
    wa = (rng.integers(0, 256, 64) | (sa << 16) | (rng.integers(0, 256, 64) << 24)).astype(np.uint32)
    wb = (rng.integers(0, 256, 64) | (sb << 16) | (rng.integers(0, 256, 64) << 8)).astype(np.uint32)
    bufs2 = [_dev(a), _dev(b), _dev(wa.view(np.int32)), _dev(wb.view(np.int32))]
    c2 = torch.zeros((64, 16), dtype=torch.float32, device="cuda")
    log("probe mfma_fp4_sel2")
    assert lib.probe_mfma_fp4_sel2(*[t.data_ptr() for t in bufs2], c2.data_ptr(), None) == 0
    _sync()
    assert np.array_equal(c2.cpu().numpy().astype(np.float64), want)


def _rne_e2m1(y):
    """Nearest E2M1 magnitude code of y >= 0 (ties to the even code, saturating at 6)."""
    best = None
    for code in range(8):
        dist = abs(E2M1[code] - y)
        if best is None or dist < best[0] - 1e-12 or (abs(dist - best[0]) <= 1e-12 and code % 2 == 0):
            best = (dist, code)
    return best[1] if y <= 6.0 else 7


def test_fp4_convert_rounding_saturation_and_byte_select(lib):
    import torch
    grid = np.array([0.0, 0.25, 0.26, 0.5, 0.74, 0.75, 0.76, 1.0, 1.25, 1.3, 1.5, 1.75, 1.8, 2.0,
                     2.5, 2.6, 3.0, 3.5, 3.6, 4.0, 5.0, 5.1, 6.0, 7.0, 100.0, 1e-30, 0.124, 0.126],
                    np.float32)
    x = np.resize(grid, 128).astype(np.float32)
    x[100:] = -x[100:]
    scale = np.where(np.arange(64) % 3 == 0, 1.0, np.where(np.arange(64) % 3 == 1, 2.0, 0.5))
    scale = scale.astype(np.float32)
    bufs = [_dev(x), _dev(scale)]
    out = torch.zeros(256, dtype=torch.int32, device="cuda")
    log("probe cvt_fp4")
    assert lib.probe_cvt_fp4(bufs[0].data_ptr(), bufs[1].data_ptr(), out.data_ptr(), None) == 0
    _sync()
    got = out.cpu().numpy().view(np.uint32).reshape(64, 4)
    for l in range(64):
        codes = []
        for v in (x[2 * l], x[2 * l + 1]):
            y = float(v) / float(scale[l])
            mag = _rne_e2m1(abs(y))
            codes.append(mag | (8 if np.signbit(v) else 0))
        byte = codes[0] | (codes[1] << 4)
        for sel in range(4):
            want = (0xFFFFFFFF & ~(0xFF << (8 * sel))) | (byte << (8 * sel))
            assert got[l, sel] == want, (l, sel, x[2 * l], x[2 * l + 1], scale[l], hex(got[l, sel]))


def test_fp4_decode(lib):
    import torch
    src = np.arange(256, dtype=np.uint32).reshape(64, 4)
    word = (src[:, 0] | (src[:, 1] << 8) | (src[:, 2] << 16) | (src[:, 3] << 24)).astype(np.uint32)
    scale = np.where(np.arange(64) % 2 == 0, 1.0, 0.25).astype(np.float32)
    bufs = [_dev(word.view(np.int32)), _dev(scale)]
    out = torch.zeros(64 * 8, dtype=torch.float32, device="cuda")
    log("probe dec_fp4")
    assert lib.probe_dec_fp4(bufs[0].data_ptr(), bufs[1].data_ptr(), out.data_ptr(), None) == 0
    _sync()
    got = out.cpu().numpy().reshape(64, 4, 2)
    for l in range(64):
        for sel in range(4):
            byte = int(src[l, sel])
            assert got[l, sel, 0] == _fp4_value(byte & 15) * scale[l]
            assert got[l, sel, 1] == _fp4_value(byte >> 4) * scale[l]


def test_wave_placement_pairs_waves_on_simds(lib):
    """Wave placement of a 512-thread workgroup: waves w and w + 4 share a SIMD and
    waves 0-3 sit on four different SIMDs.  The bf16 kernel's two waves of a SIMD
    (w and w + 4) therefore compete for one matrix unit and one VALU, which is what
    its per-SIMD instruction budget assumes (a speed, not a correctness, property:
    every LDS hand-over in the kernel crosses a workgroup barrier)."""
    import torch
    blocks = 1024
    out = torch.zeros(blocks * 8, dtype=torch.int32, device="cuda")
    log("probe wave_place")
    assert lib.probe_wave_place(out.data_ptr(), blocks, None) == 0
    _sync()
    hw = out.cpu().numpy().astype(np.uint32).reshape(blocks, 8)
    simd = (hw >> 4) & 3
    cu = (hw >> 8) & 15
    log(f"  simd ids of the first blocks: {simd[:4].tolist()}")
    assert np.all(cu == cu[:, :1]), "all waves of a workgroup on one CU"
    assert np.all(simd[:, :4] == simd[:, 4:]), "wave w and w + 4 share a SIMD"
    assert np.all(np.sort(simd[:, :4], axis=1) == np.arange(4)), "waves 0-3 on distinct SIMDs"


def _e4m3_decode(codes):
    """E4M3 byte -> value through torch's float8_e4m3fn (an independent decoder)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).float().numpy().astype(np.float64)


def test_mfma_fp8_layout_and_scales(lib):
    import torch
    rng = np.random.default_rng(8)
    ca = rng.integers(0, 256, size=(64, 32)).astype(np.uint8)
    cb = rng.integers(0, 256, size=(64, 32)).astype(np.uint8)
    ca[(ca & 0x7F) == 0x7F] = 0x12          # no NaN codes
    cb[(cb & 0x7F) == 0x7F] = 0x34
    sa = rng.integers(120, 135, size=64).astype(np.uint8)
    sb = rng.integers(120, 135, size=64).astype(np.uint8)
    va, vb = _e4m3_decode(ca), _e4m3_decode(cb)

    def k_of(l, i):
        h = l // 32
        return 16 * h + i if i < 16 else 32 + 16 * h + (i - 16)

    A = np.zeros((32, 64))
    B = np.zeros((64, 32))
    for l in range(64):
        for i in range(32):
            k = k_of(l, i)
            blk = k // 32          # the scale of k-block blk comes from lane (l % 32) + 32*blk
            A[l % 32, k] = va[l, i] * 2.0 ** (int(sa[l % 32 + 32 * blk]) - 127)
            B[k, l % 32] = vb[l, i] * 2.0 ** (int(sb[l % 32 + 32 * blk]) - 127)
    C = A @ B
    want = np.array([[C[8 * (r // 4) + 4 * (l // 32) + r % 4, l % 32] for r in range(16)]
                     for l in range(64)])
    # bound of the hardware's accumulation error: 2^-10 of the largest product
    pmax = np.array([[np.max(np.abs(A[8 * (r // 4) + 4 * (l // 32) + r % 4] *
                                    B[:, l % 32])) for r in range(16)] for l in range(64)])
    bufs = [_dev(ca), _dev(cb), _dev(sa), _dev(sb)]
    c = torch.zeros((64, 16), dtype=torch.float32, device="cuda")
    log("probe mfma_fp8")
    assert lib.probe_mfma_fp8(*[t.data_ptr() for t in bufs], c.data_ptr(), None) == 0
    _sync()
    got = c.cpu().numpy().astype(np.float64)
    # a scale misapplied to a k-block (e.g. each lane's own byte for all its 32 elements)
    # is off by far more than this on these inputs
    assert np.all(np.abs(got - want) <= 2.0 ** -10 * pmax)


def test_fp8_convert_rounding_and_half_select(lib):
    import torch
    rng = np.random.default_rng(9)
    mags = _e4m3_decode(np.arange(127))
    mids = ((mags[:-1] + mags[1:]) / 2)[rng.permutation(126)[:40]]     # exact ties
    x = np.concatenate([mags[rng.integers(0, 127, 24)], mids,
                        np.exp2(rng.uniform(-12, 8.7, 40)), rng.uniform(0, 300, 24)])
    x = x.astype(np.float32)
    assert x.shape == (128,)             # the probe reads 64 lanes x 2 floats
    x[::3] = -x[::3]
    bufs = [_dev(x)]
    out = torch.zeros(128, dtype=torch.int32, device="cuda")
    log("probe cvt_fp8")
    assert lib.probe_cvt_fp8(bufs[0].data_ptr(), out.data_ptr(), None) == 0
    _sync()
    got = out.cpu().numpy().view(np.uint32).reshape(64, 2)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy().astype(np.uint32)
    for l in range(64):
        pair = ref[2 * l] | (ref[2 * l + 1] << 8)
        assert got[l, 0] == (0xFFFF0000 | pair), (l, x[2 * l], x[2 * l + 1], hex(got[l, 0]))
        assert got[l, 1] == (0x0000FFFF | (pair << 16)), (l, hex(got[l, 1]))
