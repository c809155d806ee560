"""Host-side checks of the C ABI (no GPU needed: nothing here launches a kernel).

* libattn.so loads and exports every function declared in include/attn.h;
* argument validation returns the documented codes before any launch;
* the cubic used by the VALU exp2 meets its error bound.
"""

import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "exact_attention_forward_tiled_amd")


@pytest.fixture(scope="module")
def fa():
    if not os.path.exists(os.path.join(PKG, "libattn.so")):
        from exact_attention_forward_tiled_amd.build import build
        build()
    import exact_attention_forward_tiled_amd as fa
    return fa


def _declared():
    text = open(os.path.join(ROOT, "include", "attn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(fa):
    names = _declared()
    assert "attn_fwd" in names and "attn_fwd_mxfp4" in names
    lib = ctypes.CDLL(os.path.join(PKG, "libattn.so"))
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(fa.EXPORTS)


FAKE = 4096  # a 16-byte aligned non-null address; never dereferenced on these paths


@pytest.mark.parametrize("args,code", [
    (dict(q=0), -1),
    (dict(o=0), -1),
    (dict(q=FAKE + 8), -1),            # misaligned
    (dict(B=0), -1),
    (dict(N=0), -1),
    (dict(Hq=6, Hkv=4), -1),
    (dict(causal=2), -1),
    (dict(scale=float("nan")), -1),
    (dict(scale=float("inf")), -1),
    (dict(d=96), -2),
    (dict(d=256), -2),
    (dict(N=1 << 23, d=128, Hq=1), -2),        # one head's K reaches 2 GiB
    (dict(B=1 << 16, N=1 << 15, Hq=1), -2),    # 2^31 rows
])
def test_fwd_validation(fa, args, code):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, Hq=2, Hkv=1, N=16, d=64, causal=0,
             scale=0.125)
    a.update(args)
    st = fa.attn_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["N"],
                     a["d"], a["causal"], a["scale"])
    assert st == code


def test_opts_validation(fa):
    for tau, mode, frac in [(-1.0, "hw", None), (float("nan"), "hw", None), (8.0, 7, None),
                            (8.0, "mix", -0.1), (8.0, "mix", 1.5), (8.0, "mix", float("nan"))]:
        opts = fa.make_opts(tau, mode, poly_frac=frac)
        st = fa.attn_fwd_ex(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 1, 16, 64, 0, 0.1, opts, None)
        assert st == -1
    # a negative window is invalid for both forwards
    opts = fa.make_opts(8.0, "hw", window=-1)
    assert fa.attn_fwd_ex(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 1, 16, 64, 0, 0.1, opts, None) == -1
    assert fa.attn_fwd_mxfp4_ex(*[FAKE] * 8, 1, 1, 1, 64, 128, 0, 0.1, opts, None) == -1
    # soft-capping: C must be finite and >= 0; score modifications need the hardware exp
    # and the bf16 forward
    for cap in (-1.0, float("nan"), float("inf")):
        opts = fa.make_opts(8.0, "hw", softcap=cap)
        assert fa.attn_fwd_ex(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 1, 16, 64, 0, 0.1, opts,
                              None) == -1
    for kw in (dict(softcap=5.0), dict(alibi_ptr=FAKE)):
        opts = fa.make_opts(8.0, "poly", **kw)
        assert fa.attn_fwd_ex(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 1, 16, 64, 0, 0.1, opts,
                              None) == -2
        opts = fa.make_opts(8.0, "hw", **kw)
        assert fa.attn_fwd_mxfp4_ex(*[FAKE] * 8, 1, 1, 1, 64, 128, 0, 0.1, opts, None) == -2
    # documents: at least one, at most N (documents are non-empty), for every forward
    for nd in (0, -1, 17):
        opts = fa.make_opts(8.0, "hw", doc_ptr=FAKE, n_docs=nd)
        assert fa.attn_fwd_ex(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 1, 16, 64, 0, 0.1, opts,
                              None) == -1
    for nd in (0, -1, 65):
        opts = fa.make_opts(8.0, "hw", doc_ptr=FAKE, n_docs=nd)
        assert fa.attn_fwd_mxfp4_ex(*[FAKE] * 8, 1, 1, 1, 64, 128, 0, 0.1, opts, None) == -1


def test_tau_bound(fa):
    """tau above ATTN_TAU_MAX (64) is rejected by every forward and the backward; 64 itself
    passes the option check (the call then stops at the unsupported head dimension)."""
    for tau in (64.5, 200.0, float("inf")):
        opts = fa.make_opts(tau, "hw")
        assert fa.attn_fwd_ex(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 1, 16, 64, 0, 0.1, opts,
                              None) == -1
        assert fa.attn_fwd_mxfp4_ex(*[FAKE] * 8, 1, 1, 1, 64, 128, 0, 0.1, opts, None) == -1
        assert fa.attn_fwd_mxfp8_ex(*[FAKE] * 8, 1, 1, 1, 64, 128, 0, 0.1, opts, None) == -1
        assert fa.attn_bwd_ex(*[FAKE] * 10, 1, 1, 1, 16, 64, 0, 0.1, opts, None) == -1
    opts = fa.make_opts(64.0, "hw")
    assert fa.attn_fwd_ex(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 1, 16, 96, 0, 0.1, opts,
                          None) == -2
    assert fa.attn_fwd_mxfp4_ex(*[FAKE] * 8, 1, 1, 1, 64, 64, 0, 0.1, opts, None) == -2


def test_bwd_noalloc_validation(fa):
    """The allocation-free backward validates like attn_bwd_ex before touching the device,
    and rejects problems whose D does not fit its static workspace (B*Hq*N > 2^21)."""
    base = [FAKE] * 9
    assert fa.attn_bwd_noalloc(0, *base[1:], 1, 2, 1, 16, 64, 0, 0.1) == -1
    assert fa.attn_bwd_noalloc(*base, 1, 2, 1, 0, 64, 0, 0.1) == -1
    assert fa.attn_bwd_noalloc(*base, 1, 2, 1, 16, 96, 0, 0.1) == -2
    assert fa.attn_bwd_noalloc(*base, 1, 2, 1, 16, 64, 0, 0.1, fa.make_opts(tau=-1.0)) == -1
    assert fa.attn_bwd_noalloc(*base, 1, 64, 8, (1 << 21) // 64 + 1, 128, 0, 0.1) == -2
    assert fa.attn_bwd_noalloc(*base, 2, 16, 16, 65537, 128, 1, 0.1) == -2


def test_default_opts_layout(fa):
    """attn_default_opts fills every field of the C struct; reading them back through the
    binding's mirror checks that the two layouts agree."""
    from exact_attention_forward_tiled_amd.binding import AttnOpts, lib
    o = AttnOpts()
    o.tau, o.exp_mode, o.poly_frac, o.stats, o.window = -3.0, 9, -3.0, FAKE, -7
    o.alibi_slopes, o.softcap, o.doc_offsets, o.n_docs = FAKE, -2.0, FAKE, -5
    lib.attn_default_opts(ctypes.byref(o))
    assert (o.tau, o.exp_mode, o.poly_frac, o.stats, o.window) == (8.0, 0, 0.5, None, 0)
    assert (o.alibi_slopes, o.softcap, o.doc_offsets, o.n_docs) == (None, 0.0, None, 0)


def test_mxfp4_validation(fa):
    base = [FAKE] * 8
    assert fa.attn_fwd_mxfp4(*base, 1, 2, 2, 64, 64, 0, 0.1) == -2      # d must be 128
    assert fa.attn_fwd_mxfp4(*base, 1, 2, 2, 48, 128, 0, 0.1) == -2     # N % 32
    assert fa.attn_fwd_mxfp4(0, *base[1:], 1, 2, 2, 64, 128, 0, 0.1) == -1
    assert fa.attn_quantize_mxfp4_rows(FAKE, FAKE, FAKE, 4, 48) == -1
    assert fa.attn_quantize_mxfp4_cols_t(FAKE, FAKE, FAKE, 1, 40, 8) == -1


def test_mxfp8_validation(fa):
    base = [FAKE] * 8
    assert fa.attn_fwd_mxfp8(*base, 1, 2, 2, 64, 64, 0, 0.1) == -2      # d must be 128
    assert fa.attn_fwd_mxfp8(*base, 1, 2, 2, 48, 128, 0, 0.1) == -2     # N % 32
    assert fa.attn_fwd_mxfp8(*base, 1, 3, 2, 64, 128, 0, 0.1) == -1     # Hq % Hkv
    assert fa.attn_fwd_mxfp8(*base, 1, 2, 2, 64, 128, 2, 0.1) == -1     # causal in {0, 1}
    assert fa.attn_fwd_mxfp8(0, *base[1:], 1, 2, 2, 64, 128, 0, 0.1) == -1
    # masks are taken, but still validated before any launch; score modifications are not
    assert fa.attn_fwd_mxfp8_ex(*base, 1, 2, 2, 64, 64, 0, 0.1, fa.make_opts(window=16),
                                None) == -2
    assert fa.attn_fwd_mxfp8_ex(*base, 1, 2, 2, 64, 128, 0, 0.1, fa.make_opts(window=-1),
                                None) == -1
    assert fa.attn_fwd_mxfp8_ex(*base, 1, 2, 2, 64, 128, 0, 0.1,
                                fa.make_opts(doc_ptr=FAKE, n_docs=65), None) == -1
    assert fa.attn_fwd_mxfp8_ex(*base, 1, 2, 2, 64, 128, 0, 0.1, fa.make_opts(alibi_ptr=FAKE),
                                None) == -2
    assert fa.attn_fwd_mxfp8_ex(*base, 1, 2, 2, 64, 128, 0, 0.1, fa.make_opts(softcap=2.0),
                                None) == -2
    # the MXFP4 forward takes the masks too, validated the same way before any launch
    assert fa.attn_fwd_mxfp4_ex(*base, 1, 2, 2, 64, 128, 0, 0.1, fa.make_opts(window=-1),
                                None) == -1
    assert fa.attn_fwd_mxfp4_ex(*base, 1, 2, 2, 64, 128, 0, 0.1,
                                fa.make_opts(doc_ptr=FAKE, n_docs=65), None) == -1
    assert fa.attn_fwd_mxfp4_ex(*base, 1, 2, 2, 64, 128, 0, 0.1, fa.make_opts(alibi_ptr=FAKE),
                                None) == -2
    assert fa.attn_quantize_mxfp8_rows(FAKE, FAKE, FAKE, 4, 48) == -1
    assert fa.attn_quantize_mxfp8_cols_t(FAKE, FAKE, FAKE, 1, 40, 8) == -1


def test_bwd_validation(fa):
    base = [FAKE] * 10
    assert fa.attn_bwd(*base, 1, 2, 2, 64, 96, 0, 0.1) == -2            # d in {64, 128}
    assert fa.attn_bwd(*base, 1, 3, 2, 64, 128, 0, 0.1) == -1           # Hq % Hkv
    assert fa.attn_bwd(*base, 1, 2, 2, 0, 128, 0, 0.1) == -1            # N >= 1
    assert fa.attn_bwd(*base, 1, 2, 2, 64, 128, 3, 0.1) == -1           # causal in {0, 1}
    assert fa.attn_bwd(*base, 1, 2, 2, 64, 128, 0, float("inf")) == -1  # finite scale
    for i in range(10):                                                 # every pointer
        args = list(base)
        args[i] = 0
        assert fa.attn_bwd(*args, 1, 2, 2, 64, 128, 0, 0.1) == -1
    args = list(base)
    args[6] = FAKE + 4                                                  # dq 16-byte aligned
    assert fa.attn_bwd(*args, 1, 2, 2, 64, 128, 0, 0.1) == -1


def test_bwd_ex_validation(fa):
    """The masking options of the backward: rejected before any launch."""
    base = [FAKE] * 10
    shape = (1, 2, 2, 64, 128, 0, 0.1)
    assert fa.attn_bwd_ex(*base, *shape, fa.make_opts(window=-1)) == -1
    assert fa.attn_bwd_ex(*base, *shape, fa.make_opts(doc_ptr=FAKE, n_docs=0)) == -1
    assert fa.attn_bwd_ex(*base, *shape, fa.make_opts(doc_ptr=FAKE, n_docs=65)) == -1
    assert fa.attn_bwd_ex(*base, *shape, fa.make_opts(softcap=-1.0)) == -1
    assert fa.attn_bwd_ex(*base, *shape, fa.make_opts(softcap=float("inf"))) == -1
    assert fa.attn_bwd_ex(*base, 1, 2, 2, 64, 96, 0, 0.1, fa.make_opts(softcap=5.0)) == -2
    assert fa.attn_bwd_ex(*base, *shape, fa.make_opts(tau=-1.0)) == -1
    assert fa.attn_bwd_ex(*base, 1, 2, 2, 64, 96, 0, 0.1, fa.make_opts(window=8)) == -2
    args = list(base)
    args[9] = 0                                                         # delta
    assert fa.attn_bwd_ex(*args, *shape, fa.make_opts(window=8)) == -1


def test_strerror(fa):
    from exact_attention_forward_tiled_amd.binding import lib
    assert lib.attn_strerror(0) == b"success"
    assert lib.attn_strerror(-2) == b"unsupported shape or format"
    assert lib.attn_strerror(12345) == b"unknown status"
    with pytest.raises(ValueError):
        fa.check(-1)
    with pytest.raises(NotImplementedError):
        fa.check(-2)


def _poly_coeffs():
    text = open(os.path.join(PKG, "csrc", "exp2_poly.h")).read()
    return [np.float32(float(re.search(rf"ATTN_EXP2_{n} ([-0-9.e+]+)f", text).group(1)))
            for n in ("C1", "C2", "C3")]


def test_exp2_cubic_error_bound():
    """The committed cubic, evaluated in fp32 as the kernel does, stays within 1.2e-4 relative
    error of 2^x over the whole range the kernel feeds it (x in [-126, 8])."""
    c1, c2, c3 = _poly_coeffs()
    x = np.concatenate([np.linspace(-126.0, 8.0, 2_000_003, dtype=np.float32),
                        np.float32(np.arange(-126, 9)),
                        np.nextafter(np.float32(np.arange(-125, 9)), np.float32(-200))])
    n = np.floor(x)
    f = (x - n).astype(np.float32)
    p = (f * (f * (f * c3 + c2) + c1) + np.float32(1.0)).astype(np.float32)
    bits = p.view(np.int32) + (n.astype(np.int32) << 23)
    got = bits.view(np.float32).astype(np.float64)
    rel = np.abs(got / np.exp2(x.astype(np.float64)) - 1.0)
    assert rel.max() < 1.2e-4


def test_exp2_cubic_exhaustive_scan(tmp_path):
    """Every fp32 x in [-126, 8] (2,214,330,370 values) through the kernel's fp32 steps of the
    cubic (fused multiply-adds, exponent-bit add), against 2^x in double: the largest
    relative error stays at the fit's 1.03e-4 (the fp32 evaluation adds under 1e-6)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    exe = str(tmp_path / "exp2_scan")
    subprocess.run([gcc, "-O2", "-fopenmp", "-ffp-contract=off", "-I",
                    os.path.join(PKG, "csrc"), os.path.join(ROOT, "tests", "exp2_scan.c"),
                    "-lm", "-o", exe], check=True)
    count, worst = subprocess.run([exe], check=True, capture_output=True,
                                  text=True).stdout.split()
    assert int(count) == 0x41000000 + 1 + 0x42FC0000 + 1
    assert float(worst) <= 1.04e-4


def test_abi_under_address_sanitizer(fa, tmp_path):
    """The host code of the C ABI built with AddressSanitizer and UndefinedBehaviorSanitizer
    (g++, host code only; the kernels' objects are linked unchanged), driven through every
    entry point's argument checks by tests/abi_asan.c.  Nothing is launched."""
    import glob
    import shutil
    import subprocess
    gxx, gcc = shutil.which("g++"), shutil.which("gcc")
    if gxx is None or gcc is None:
        pytest.skip("no host C/C++ compiler")
    objs = sorted(glob.glob(os.path.join(ROOT, "_build", "obj", "attn_*.hip.o")))
    if len(objs) < 4:
        from exact_attention_forward_tiled_amd.build import build
        build()
        objs = sorted(glob.glob(os.path.join(ROOT, "_build", "obj", "attn_*.hip.o")))
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    san = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-g", "-O1"]
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
           "-I", os.path.join(rocm, "include"), "-D__HIP_PLATFORM_AMD__"]
    api_o = str(tmp_path / "attn_api_asan.o")
    drv_o = str(tmp_path / "abi_asan.o")
    exe = str(tmp_path / "abi_asan")
    subprocess.run([gxx, "-std=c++17", "-fPIC", "-c", *san, *inc,
                    os.path.join(PKG, "csrc", "attn_api.cpp"), "-o", api_o], check=True)
    subprocess.run([gcc, "-c", *san, *inc, os.path.join(ROOT, "tests", "abi_asan.c"), "-o",
                    drv_o], check=True)
    subprocess.run([gxx, *san, drv_o, api_o, *objs, "-L", os.path.join(rocm, "lib"),
                    "-Wl,-rpath," + os.path.join(rocm, "lib"), "-lamdhip64", "-o", exe],
                   check=True)
    # verify_asan_link_order=0: the environment may preload a library of its own ahead of
    # the sanitizer runtime
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([exe], capture_output=True, text=True, env=env)
    assert res.returncode == 0 and res.stdout.strip() == "ok", res.stdout + res.stderr
