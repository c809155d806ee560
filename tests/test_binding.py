"""The Python binding's buffer checks (CPU only, nothing is launched).

The C ABI sees only pointers and sizes, so the binding checks every caller tensor (inputs,
caller-given outputs, the backward's workspace) for shape, dtype, device and contiguity
and raises ValueError before any launch.  These tests use CPU tensors: every check runs
before the one that requires the operands on the GPU."""

import pytest
import torch

import exact_attention_forward_tiled_amd as fa
from exact_attention_forward_tiled_amd import binding

BF, F32, U8 = torch.bfloat16, torch.float32, torch.uint8
B, HQ, HKV, N, D = 1, 4, 2, 64, 128


def _qkv():
    return (torch.zeros(B, HQ, N, D, dtype=BF), torch.zeros(B, HKV, N, D, dtype=BF),
            torch.zeros(B, HKV, N, D, dtype=BF))


def _raises(fn, match):
    with pytest.raises(ValueError, match=match):
        fn()


def test_require():
    t = torch.zeros(2, 3, dtype=F32)
    binding.require(t, "t", (2, 3), F32, t.device)
    _raises(lambda: binding.require(t, "t", (3, 2), F32, t.device), "shape")
    _raises(lambda: binding.require(t, "t", (2, 3), BF, t.device), "must be torch.bfloat16")
    _raises(lambda: binding.require(t.t(), "t", (3, 2), F32, t.device), "contiguous")


def test_fwd_checks_inputs_and_outputs():
    q, k, v = _qkv()
    good = (torch.zeros(B, HQ, N, D, dtype=F32), torch.zeros(B, HQ, N, dtype=F32))
    _raises(lambda: fa.fwd(q, k, v, out=good), "CUDA")           # all shapes fine
    _raises(lambda: fa.fwd(q, k[:, :, :32], v), "k must have shape")
    _raises(lambda: fa.fwd(q, k, v.float()), "v must be torch.bfloat16")
    _raises(lambda: fa.fwd(q, k, v, out=(good[0][:, :, :32], good[1])), "o must have shape")
    _raises(lambda: fa.fwd(q, k, v, out=(good[0], good[1].double())), "lse must be")
    _raises(lambda: fa.fwd(q, k, v, out=(good[0].transpose(2, 3).contiguous()
                                         .transpose(2, 3), good[1])), "contiguous")
    _raises(lambda: fa.fwd(q, k, v, out=(good[0],)), "out must hold 2")


def test_fwd_mxfp4_checks_operands_and_outputs():
    q4 = torch.zeros(B, HQ, N, D // 2, dtype=U8)
    qs = torch.zeros(B, HQ, N, D // 32, dtype=U8)
    k4 = torch.zeros(B, HKV, N, D // 2, dtype=U8)
    ks = torch.zeros(B, HKV, N, D // 32, dtype=U8)
    vt4 = torch.zeros(B, HKV, D, N // 2, dtype=U8)
    vts = torch.zeros(B, HKV, D, N // 32, dtype=U8)
    ops = [q4, qs, k4, ks, vt4, vts]
    _raises(lambda: fa.fwd_mxfp4(*ops), "CUDA")
    for i, name in enumerate(("q4", "qs", "k4", "ks", "vt4", "vts")):
        bad = list(ops)
        bad[i] = bad[i][..., :-1].contiguous()
        if i == 0:
            continue        # q4 defines the problem's shape
        _raises(lambda: fa.fwd_mxfp4(*bad), f"{name} must have shape")
    bad = list(ops)
    bad[1] = qs.to(torch.int8)
    _raises(lambda: fa.fwd_mxfp4(*bad), "qs must be torch.uint8")
    _raises(lambda: fa.fwd_mxfp4(*ops, out=(torch.zeros(B, HQ, N, D), torch.zeros(B, HQ))),
            "lse must have shape")


def test_fwd_mxfp8_checks_operands_and_outputs():
    ops = [torch.zeros(B, HQ, N, D, dtype=U8), torch.zeros(B, HQ, N, D // 32, dtype=U8),
           torch.zeros(B, HKV, N, D, dtype=U8), torch.zeros(B, HKV, N, D // 32, dtype=U8),
           torch.zeros(B, HKV, D, N, dtype=U8), torch.zeros(B, HKV, D, N // 32, dtype=U8)]
    _raises(lambda: fa.fwd_mxfp8(*ops), "CUDA")
    bad = list(ops)
    bad[4] = torch.zeros(B, HKV, N, D, dtype=U8)[..., :64].contiguous()
    _raises(lambda: fa.fwd_mxfp8(*bad), "vt8 must have shape")
    _raises(lambda: fa.fwd_mxfp8(*ops, out=(torch.zeros(B, HQ, N, D, dtype=BF),
                                           torch.zeros(B, HQ, N))), "o must be torch.float32")


def test_bwd_checks_everything():
    q, k, v = _qkv()
    o = torch.zeros(B, HQ, N, D, dtype=F32)
    lse = torch.zeros(B, HQ, N, dtype=F32)
    g = torch.zeros(B, HQ, N, D, dtype=BF)
    grads = (torch.zeros(B, HQ, N, D), torch.zeros(B, HKV, N, D), torch.zeros(B, HKV, N, D))
    _raises(lambda: fa.bwd(q, k, v, o, lse, g, out=grads), "CUDA")
    _raises(lambda: fa.bwd(q, k, v, o, lse[:, :, :10], g), "lse must have shape")
    _raises(lambda: fa.bwd(q, k, v, o, lse, g.float()), "dout must be torch.bfloat16")
    _raises(lambda: fa.bwd(q, k, v, o, lse, g, out=(grads[0], grads[0], grads[2])),
            "dk must have shape")
    _raises(lambda: fa.bwd(q, k, v, o, lse, g, delta=torch.zeros(B * HQ * N - 1)), "delta")
    _raises(lambda: fa.bwd(q, k, v, o, lse, g, delta=torch.zeros(2 * B * HQ * N)[::2]),
            "delta")
