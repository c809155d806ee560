"""The allocation-free backward (attn_bwd_noalloc) against the workspace form (attn_bwd_ex).

Both run the same kernels; only D's buffer differs (the library's static device array
instead of a caller workspace), so the gradients must agree bit for bit, and both meet the
backward's parity gates against the oracle.  Two calls in a row, the second on a smaller
problem, show that nothing from the first call leaks into the second."""

import math

import numpy as np
import pytest

import oracle
import synth
from oracle import backward as bw
from gpu_util import (BWD_DQK_RELRMS, BWD_DQK_ROW, BWD_DV_RELRMS, BWD_DV_ROW, cuda_ok, gate, log,
                      to_dev_bf16)

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not cuda_ok(), reason="needs a GPU")]

CASES = [
    # B, Hq, Hkv, N, causal
    (2, 4, 2, 700, True),
    (1, 2, 1, 190, False),
]


def test_noalloc_matches_workspace_form_two_calls():
    import torch
    import exact_attention_forward_tiled_amd as fa
    from exact_attention_forward_tiled_amd import binding
    for i, (B, Hq, Hkv, N, causal) in enumerate(CASES):
        d = 128
        scale = 1.0 / math.sqrt(d)
        qb, kb, vb = synth.configs.random_case(90 + i, B, Hq, Hkv, N, d)
        gb = synth.normal_bf16((B, Hq, N, d), 990 + i, 1.0)
        q, k, v, g = (to_dev_bf16(x) for x in (qb, kb, vb, gb))
        log(f"noalloc call {i}: {(B, Hq, Hkv, N, causal)}")
        o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
        want = fa.bwd(q, k, v, o, lse, g, causal=causal, scale=scale)
        got = [torch.full(t.shape, float("nan"), dtype=torch.float32, device="cuda")
               for t in want]
        st = binding.attn_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                      lse.data_ptr(), g.data_ptr(), got[0].data_ptr(),
                                      got[1].data_ptr(), got[2].data_ptr(), B, Hq, Hkv, N, d,
                                      int(causal), scale, None,
                                      torch.cuda.current_stream().cuda_stream)
        assert st == 0, binding.lib.attn_strerror(st)
        torch.cuda.synchronize()
        for a, b_ in zip(got, want):
            assert torch.equal(a, b_)
        ref = bw.attention_backward(*(synth.bf16_bits_to_f64(x) for x in (qb, kb, vb, gb)),
                                    causal, scale)
        dq, dk, dv = (t.cpu().numpy() for t in got)
        gate(dq, ref[0], BWD_DQK_RELRMS, BWD_DQK_ROW, "dQ")
        gate(dk, ref[1], BWD_DQK_RELRMS, BWD_DQK_ROW, "dK")
        gate(dv, ref[2], BWD_DV_RELRMS, BWD_DV_ROW, "dV")
