"""GPU parity of flare_attend (the FLARE skill page's token-query decode:
token queries attend to the latent states Z as keys and values) against the
fp64 oracle, in both layouts, at small ragged shapes and, on sampled tokens,
at the 65k-mesh size."""
import zlib

import numpy as np
import pytest
import torch

import oracle
from flare_inputs import WORKLOADS, f32_to_bf16_bits, make_inputs, workload_inputs
from rank_latent_attention_flare_amd import flare as F
from tests.gpu_util import assert_parity, sample_rows, to_dev, to_host64

pytestmark = pytest.mark.gpu

CASES = [
    (2, 3, 1000, 64, 64, "bf16"),
    (1, 2, 4097, 100, 32, "bf16"),
    (1, 1, 1, 1, 32, "bf16"),
    (2, 2, 777, 33, 128, "bf16"),
    # exact latent counts with token-major queries: head groups per workgroup
    (1, 4, 3001, 128, 32, "bf16"),
    (2, 2, 1999, 64, 64, "bf16"),
    (1, 2, 1200, 320, 128, "bf16"),  # split decode (D = 128, M > 256)
    (1, 3, 3000, 40, 8, "f32"),
    (1, 2, 500, 300, 32, "f32"),
]


def case_id(c):
    return "B{}H{}N{}M{}D{}-{}".format(*c)


def stored(x64: np.ndarray, dt: str) -> np.ndarray:
    x = x64.astype(np.float32)
    return x if dt == "f32" else f32_to_bf16_bits(x)


@pytest.mark.parametrize("layout", [F.FLARE_LAYOUT_BHND, F.FLARE_LAYOUT_BNHD], ids=["bhnd", "bnhd"])
@pytest.mark.parametrize("case", CASES, ids=case_id)
def test_attend_matches_oracle(case, layout):
    B, H, N, M, D, dt = case
    seed = zlib.crc32(repr(("attend",) + case).encode()) % 100000
    Q, K, V = make_inputs(B, H, N, M, D, dt, q_scale=0.5, seed=seed)
    Zs = stored(oracle.encode(Q, K, V), dt)  # realistic latent states
    q = K                                    # token queries with the statistics of keys
    print(f"[attend] case={case_id(case)} layout={layout} seed={seed}", flush=True)
    qd = to_dev(q)
    if layout == F.FLARE_LAYOUT_BNHD:
        qd = qd.transpose(1, 2).contiguous()
    Y = F.flare_attend(qd, to_dev(Zs), layout)
    torch.cuda.synchronize()
    if layout == F.FLARE_LAYOUT_BNHD:
        Y = Y.transpose(1, 2)
    assert_parity(to_host64(Y.contiguous()), oracle.attend(q, Zs), dt, f"attend {case_id(case)}")


def test_skill_page_layer_matches_oracle():
    # the page's layer: Z = encode(latents, k, v), then Y = attend(q, Z)
    B, H, N, M, D, dt = 2, 4, 3000, 64, 64, "bf16"
    Q, K, V = make_inputs(B, H, N, M, D, dt, q_scale=0.5, seed=7)
    q = make_inputs(B, H, N, M, D, dt, q_scale=0.5, seed=8)[1]
    Z = F.flare_encode(to_dev(Q), to_dev(K), to_dev(V))
    Y = F.flare_attend(to_dev(q), Z)
    torch.cuda.synchronize()
    Zr = oracle.encode(Q, K, V)
    assert_parity(to_host64(Y), oracle.attend(q, Zr), dt, "encode then attend")


def test_attend_full_size_sampled_tokens():
    w = WORKLOADS[2]
    Qh, Kh, Vh = workload_inputs(w)
    heads = [(0, 0), (w.B - 1, w.H - 1)]
    Zr = oracle.encode(Qh, Kh, Vh, heads=heads)
    Zs = np.zeros(Zr.shape, np.uint16)
    for b, h in heads:
        Zs[b, h] = f32_to_bf16_bits(Zr[b, h].astype(np.float32))
    print(f"[attend] full size {w.name}", flush=True)
    Y = F.flare_attend(to_dev(Kh), to_dev(Zs))
    torch.cuda.synchronize()
    rows = sample_rows(w.N, 512, seed=3)
    ref = oracle.attend(Kh, Zs, rows=rows, heads=heads)
    Yh = to_host64(Y[:, :, torch.from_numpy(rows).cuda()])
    for b, h in heads:
        assert_parity(Yh[b, h], ref[b, h], "bf16", f"attend {w.name} head ({b},{h})")
