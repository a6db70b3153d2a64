"""Seeded random sweep of shapes: every entry point against the fp64 oracle
on shapes drawn at random (fixed seed) from the supported ranges, beside the
hand-picked cases of the other files.

Each case draws the storage type, the head width D, the latent count M, the
token count N, the batch B and the head count H, the entry point and the
layout; N is then shrunk so that the oracle finishes in about a second. The
forward entry points are held to the bars of tests/gpu_util.py, the
gradients to those of tests/test_backward_gpu.py. A case whose shape is out
of the supported ranges cannot be drawn; the list printed by
`pytest --collect-only` names every shape.
"""
import numpy as np
import pytest
import torch

import oracle
from flare_inputs import f32_to_bf16_bits, make_inputs
from rank_latent_attention_flare_amd import flare as F
from tests.gpu_util import assert_parity, to_dev, to_host64
from tests.test_backward_gpu import check

pytestmark = pytest.mark.gpu

OPS = ("encode", "decode", "forward", "pp_forward")
PLAIN = {"encode": F.flare_encode, "decode": F.flare_decode, "forward": F.flare_forward,
         "pp_forward": F.flare_pp_forward}
EX = {"encode": F.flare_encode_ex, "decode": F.flare_decode_ex, "forward": F.flare_forward_ex,
      "pp_forward": F.flare_pp_forward_ex}


def _draw(count: int, seed: int, budget: float, backward: bool):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        dt = "f32" if i % 3 == 0 else "bf16"
        if dt == "bf16":
            D = int(rng.choice([32, 64, 128]))
            M = int(rng.integers(1, 513))
        else:
            D = int(rng.choice([8, 16, 24, 32, 48, 64, 96, 128]))
            M = int(rng.integers(1, 700))
        B, H = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        N = int(rng.integers(1, 6001))
        N = max(1, min(N, int(budget / (B * H * M * D))))
        op = ("backward", "pp_backward")[i % 2] if backward else OPS[i % 4]
        layout = "bnhd" if (i // 4) % 2 else "bhnd"
        out.append((op, layout, B, H, N, M, D, dt))
    return out


FWD = _draw(32, 20261203, 1.5e8, backward=False)
BWD = _draw(12, 20261204, 2.5e7, backward=True)


def case_id(c):
    return "{}-{}-B{}H{}N{}M{}D{}-{}".format(*c)


def token_major(t: torch.Tensor) -> torch.Tensor:
    return t.transpose(1, 2).contiguous()


@pytest.mark.parametrize("case", FWD, ids=case_id)
def test_random_forward_shapes(case):
    op, layout, B, H, N, M, D, dt = case
    seed = sum(case[2:7]) * 7 + OPS.index(op)
    Q, K, V = make_inputs(B, H, N, M, D, dt, q_scale=0.5, seed=seed)
    if op == "decode":
        Zr = oracle.encode(Q, K, V)
        V = Zr.astype(np.float32) if dt == "f32" else f32_to_bf16_bits(Zr.astype(np.float32))
    print(f"[random] {case_id(case)} seed={seed}", flush=True)
    q, k, v = to_dev(Q), to_dev(K), to_dev(V)
    if layout == "bhnd":
        out = PLAIN[op](q, k, v)
    else:
        out = EX[op](q, token_major(k), v if op == "decode" else token_major(v), F.FLARE_LAYOUT_BNHD)
        if op != "encode":
            out = out.transpose(1, 2)
    torch.cuda.synchronize()
    want = {"encode": lambda: oracle.encode(Q, K, V), "decode": lambda: oracle.decode(Q, K, V),
            "forward": lambda: oracle.forward(Q, K, V)[0], "pp_forward": lambda: oracle.pp_forward(Q, K, V)[0]}[op]()
    assert_parity(to_host64(out.contiguous()), want, dt, case_id(case))


@pytest.mark.parametrize("case", BWD, ids=case_id)
def test_random_backward_shapes(case):
    op, layout, B, H, N, M, D, dt = case
    seed = sum(case[2:7]) * 11 + (op == "pp_backward")
    Q, K, V = make_inputs(B, H, N, M, D, dt, q_scale=0.5, seed=seed)
    dY = make_inputs(B, H, N, M, D, dt, seed=seed + 1)[2]
    print(f"[random] {case_id(case)} seed={seed}", flush=True)
    q, k, v, g = to_dev(Q), to_dev(K), to_dev(V), to_dev(dY)
    pp = op == "pp_backward"
    if layout == "bhnd":
        got = (F.flare_pp_backward if pp else F.flare_backward)(q, k, v, g)
    else:
        ex = F.flare_pp_backward_ex if pp else F.flare_backward_ex
        dq, dk, dv = ex(q, token_major(k), token_major(v), token_major(g), F.FLARE_LAYOUT_BNHD)
        got = (dq, dk.transpose(1, 2).contiguous(), dv.transpose(1, 2).contiguous())
    torch.cuda.synchronize()
    want = (oracle.pp_backward if pp else oracle.backward)(Q, K, V, dY)
    check(got, want, dt, case_id(case))
