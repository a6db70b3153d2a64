"""GPU checks of the token-major layout ([B][N][H][D] for K, V and Y).

The *_ex entry points with FLARE_LAYOUT_BNHD run the same kernels as the plain
entry points, with token rows addressed through a head-interleaved stride, so
their outputs must equal the plain results on the same values bit for bit
(after moving the layout back), and therefore meet the oracle bar too.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
from flare_inputs import f32_to_bf16_bits, make_inputs
from rank_latent_attention_flare_amd import flare as F
from tests.gpu_util import assert_parity, to_dev, to_host64

pytestmark = pytest.mark.gpu

PLAIN = {"encode": F.flare_encode, "decode": F.flare_decode, "forward": F.flare_forward,
         "pp_forward": F.flare_pp_forward}
EX = {"encode": F.flare_encode_ex, "decode": F.flare_decode_ex, "forward": F.flare_forward_ex,
      "pp_forward": F.flare_pp_forward_ex}
CASES = [
    # B, H, N, M, D, dtype: several tiles, ragged token and latent tails
    (2, 3, 1000, 64, 64, "bf16"),
    (1, 2, 4097, 100, 32, "bf16"),
    (2, 2, 777, 33, 128, "bf16"),
    (3, 8, 2049, 128, 32, "bf16"),
    (1, 3, 3000, 40, 8, "f32"),
    (2, 2, 999, 17, 64, "f32"),
]


def case_id(c):
    return "B{}H{}N{}M{}D{}-{}".format(*c)


def token_major(t: torch.Tensor) -> torch.Tensor:
    return t.transpose(1, 2).contiguous()


@pytest.mark.parametrize("op", list(PLAIN))
@pytest.mark.parametrize("case", CASES, ids=case_id)
def test_token_major_equals_plain_layout(op, case):
    B, H, N, M, D, dt = case
    seed = zlib.crc32(repr(("layout", op) + case).encode()) % 100000
    Q, K, V = make_inputs(B, H, N, M, D, dt, q_scale=0.5, seed=seed)
    if op == "decode":
        Zr = oracle.encode(Q, K, V)
        V = Zr.astype(np.float32) if dt == "f32" else f32_to_bf16_bits(Zr.astype(np.float32))
    print(f"[layout] op={op} case={case_id(case)} seed={seed}", flush=True)
    q, k, v = to_dev(Q), to_dev(K), to_dev(V)
    ref = PLAIN[op](q, k, v)
    kt = token_major(k)
    vt = v if op == "decode" else token_major(v)
    out = EX[op](q, kt, vt, F.FLARE_LAYOUT_BNHD)
    # with a caller workspace, and the plain layout through the same entry point
    ws = F.workspace_for({"encode": F.FLARE_OP_ENCODE, "decode": F.FLARE_OP_DECODE, "forward": F.FLARE_OP_FORWARD,
                          "pp_forward": F.FLARE_OP_PP_FORWARD}[op], q, k)
    out_ws = EX[op](q, kt, vt, F.FLARE_LAYOUT_BNHD, workspace=ws)
    same = EX[op](q, k, v, F.FLARE_LAYOUT_BHND)
    torch.cuda.synchronize()
    if op != "encode":
        assert tuple(out.shape) == (B, N, H, D)
        out, out_ws = out.transpose(1, 2), out_ws.transpose(1, 2)
    assert torch.equal(out.contiguous().view(torch.int16 if dt == "bf16" else torch.int32),
                       ref.view(torch.int16 if dt == "bf16" else torch.int32))
    assert torch.equal(out_ws.contiguous(), out.contiguous())
    assert torch.equal(same, ref)
    want = {"encode": lambda: oracle.encode(Q, K, V), "decode": lambda: oracle.decode(Q, K, V),
            "forward": lambda: oracle.forward(Q, K, V)[0], "pp_forward": lambda: oracle.pp_forward(Q, K, V)[0]}[op]()
    assert_parity(to_host64(out.contiguous()), want, dt, f"{op} token-major {case_id(case)}")
