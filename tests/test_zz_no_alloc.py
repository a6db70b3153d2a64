"""flare_forward_noalloc (the forward with the library's static scratch, for
callers that cannot allocate) against flare_forward, through the C ABI.

Two calls in a row on one stream, the second with a smaller input, so that
the second runs on what the first left in the shared scratch; each output must
equal flare_forward's bit for bit (same kernels, same plan) and meet the bf16
bar against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from flare_inputs import make_inputs
from rank_latent_attention_flare_amd import flare as F
from tests.gpu_util import assert_parity, sample_rows, to_dev, to_host64

pytestmark = pytest.mark.gpu

CASES = [
    # B, H, N, M, D: the larger first (workspace 9 MB), then a smaller one
    # with ragged tokens and latents
    (2, 8, 65536, 128, 32),
    (1, 2, 3001, 100, 64),
]


def test_noalloc_matches_forward_on_two_calls():
    ins, outs = [], []
    for i, (B, H, N, M, D) in enumerate(CASES):
        Q, K, V = make_inputs(B, H, N, M, D, "bf16", q_scale=0.5, seed=500 + i)
        need = F.flare_workspace_size(F.FLARE_OP_FORWARD, B, H, N, M, D, torch.bfloat16)
        print(f"[noalloc] call {i}: B={B} H={H} N={N} M={M} D={D} workspace {need} bytes", flush=True)
        assert 0 < need <= (64 << 20)
        d = tuple(to_dev(x) for x in (Q, K, V))
        ins.append(((Q, K, V), d))
        outs.append(F.flare_forward_noalloc(*d, out=torch.empty_like(d[1])))
    torch.cuda.synchronize()
    for i, (((Q, K, V), d), y) in enumerate(zip(ins, outs)):
        ref = F.flare_forward(*d)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), f"call {i} differs from flare_forward"
        B, H, N, M, D = CASES[i]
        rows = sample_rows(N, 1024, seed=i)
        heads = [(0, 0), (B - 1, H - 1)]
        yo = oracle.forward(Q, K, V, rows=rows, heads=heads)[0]
        yg = to_host64(y[:, :, torch.from_numpy(rows).cuda()])
        for b, h in heads:
            assert_parity(yg[b, h], yo[b, h], "bf16", f"noalloc call {i} head ({b},{h})")


def test_noalloc_repeated_calls_are_bitwise_equal():
    # the same input again after another call has used the scratch
    B, H, N, M, D = CASES[1]
    d = tuple(to_dev(x) for x in make_inputs(B, H, N, M, D, "bf16", q_scale=0.5, seed=600))
    a = F.flare_forward_noalloc(*d)
    F.flare_forward_noalloc(*(to_dev(x) for x in make_inputs(1, 1, 5000, 256, 32, "bf16", 0.5, seed=601)))
    b = F.flare_forward_noalloc(*d)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
