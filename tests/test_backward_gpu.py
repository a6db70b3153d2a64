"""GPU parity of flare_backward and flare_pp_backward (gradients of the FLARE and FLARE++ forwards) against the
fp64 oracle's backward, which is pinned to torch fp64 autograd and to central
differences of the oracle forward.

Bars. fp32 storage: the kernels work in fp32 and sum in a different order
than the oracle; the gradients contain differences of nearly equal terms
(<dZ, V> - <dZ, Z>), so the bar is relative to the largest gradient entry:
max |gpu - oracle| <= 1e-4 * max |oracle| per tensor. bf16 storage: inputs,
outputs and the forward's probabilities are bf16, as in the forward's bar:
rel-L2 <= 1e-2 and max |gpu - oracle| <= 2e-2 * max |oracle| per tensor.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
from flare_inputs import WORKLOADS, f32_to_bf16_bits, make_inputs, workload_inputs
from rank_latent_attention_flare_amd import flare as F
from tests.gpu_util import errors, to_dev, to_host64

pytestmark = pytest.mark.gpu

CASES = [
    # B, H, N, M, D, dtype
    (1, 2, 300, 40, 32, "f32"),
    (2, 2, 500, 17, 16, "f32"),
    (1, 3, 2049, 64, 8, "f32"),
    (2, 3, 1000, 64, 64, "bf16"),
    (1, 2, 777, 33, 32, "bf16"),
    (1, 2, 4097, 100, 64, "bf16"),
    (1, 1, 1, 1, 32, "bf16"),
    (1, 1, 3000, 300, 32, "bf16"),
    # many heads: two token blocks per wave in the token-side kernels, the
    # second one ragged (next-block loads clamped to the last block)
    (2, 128, 777, 33, 32, "bf16"),
    # the same at D = 64 with padded latents (the statistics kernel forms the
    # dZ partials there)
    (2, 128, 777, 50, 64, "bf16"),
    # D = 64 with more than 256 latents: the matrix-core kernels over latent
    # ranges of at most 256 (the second ragged, or a full 256, or padded)
    (1, 1, 600, 300, 64, "bf16"),
    (2, 1, 700, 480, 64, "bf16"),
    (1, 1, 500, 512, 64, "bf16"),
    # D = 64 with 256 latents (padded from 250): the latent kernels with four
    # latent blocks per wave and two token streams
    (1, 2, 1500, 250, 64, "bf16"),
    # D = 96 and 128 in fp32: the fp32 VALU kernels, token tiles of 32 in the
    # latent kernels, two columns per lane in the dZ merge; bf16 at D = 128:
    # the matrix core (M = 400 over latent and statistics ranges)
    (1, 2, 500, 40, 128, "f32"),
    (2, 1, 333, 70, 96, "f32"),
    (1, 2, 700, 64, 128, "bf16"),
    (1, 1, 300, 400, 128, "bf16"),
    # bf16 at D = 128 on the matrix core: a whole head of 128 latents, and
    # latent ranges of 128 (two full, or the second ragged)
    (1, 2, 800, 128, 128, "bf16"),
    (1, 1, 500, 256, 128, "bf16"),
    (2, 1, 600, 200, 128, "bf16"),
    # D = 128 above 256 latents: the per-token statistics over two ranges of
    # up to 256 too, merged per token
    (1, 1, 400, 512, 128, "bf16"),
]


def case_id(c):
    return "B{}H{}N{}M{}D{}-{}".format(*c)


def check_one(g, w, dt, what):
    e = errors(to_host64(g), w)
    print(f"[backward] {what} {e}", flush=True)
    assert e["finite"], f"{what}: non-finite"
    if e["ref_max"] == 0.0:
        # an identically zero gradient (N = M = 1: both softmaxes are the
        # constant 1): no scale to be relative to; the inputs are unit-scale,
        # so rounding residue must stay far below it
        assert e["max_abs"] <= 1e-5, f"{what}: {e}"
        return
    if dt == "f32":
        assert e["rel_max"] <= 1e-4, f"{what}: {e}"
    else:
        assert e["rel_l2"] <= 1e-2 and e["rel_max"] <= 2e-2, f"{what}: {e}"


def check(got, want, dt, what):
    for g, w, name in zip(got, want, ("dQ", "dK", "dV")):
        check_one(g, w, dt, f"{what} {name}")


@pytest.mark.parametrize("case", CASES, ids=case_id)
def test_backward_matches_oracle(case):
    B, H, N, M, D, dt = case
    seed = zlib.crc32(repr(("backward",) + case).encode()) % 100000
    Q, K, V = make_inputs(B, H, N, M, D, dt, q_scale=0.5, seed=seed)
    dY = make_inputs(B, H, N, M, D, dt, seed=seed + 1)[2]
    print(f"[backward] case={case_id(case)} seed={seed}", flush=True)
    got = F.flare_backward(to_dev(Q), to_dev(K), to_dev(V), to_dev(dY))
    torch.cuda.synchronize()
    check(got, oracle.backward(Q, K, V, dY), dt, case_id(case))


SHARP = [
    # B, H, N, M, D, q_scale, kv_scale: logits spread over hundreds of log2
    # units, so most tokens' largest logit lies far below the head's largest
    # and the statistics take their exact-maximum path for whole waves; at
    # q_scale 8 waves of both kinds occur
    (1, 2, 2000, 64, 32, 12.0, 2.0),
    (1, 1, 3000, 100, 64, 8.0, 2.0),
    # D = 64 with M <= 64 (the statistics kernel forms the dZ partials itself)
    # and padded latents (M = 50 of 64)
    (1, 2, 2000, 50, 64, 8.0, 2.0),
    # padded last latent block whose logits start from -1e30 in the dK/dV
    # kernel: the eight-wave form (D = 64, M > 128), the four-wave form at
    # D = 32 with separate latent passes, and the D = 32 form with dQ and dZ
    # fused in
    (1, 1, 2500, 250, 64, 8.0, 2.0),
    (1, 1, 2000, 300, 32, 12.0, 2.0),
    (1, 2, 2000, 100, 32, 12.0, 2.0),
    # latent ranges at D = 64 (256 + 44, the second padded) and D = 128
    # (128 + 72)
    (1, 1, 1500, 300, 64, 8.0, 2.0),
    (1, 1, 1500, 200, 128, 8.0, 2.0),
    (1, 1, 1000, 300, 128, 8.0, 2.0),  # and statistics over two ranges
]


@pytest.mark.parametrize("case", SHARP, ids=lambda c: "B{}H{}N{}M{}D{}-q{}kv{}".format(*c))
def test_backward_sharp_logits(case):
    B, H, N, M, D, qs, ks = case
    seed = zlib.crc32(repr(("sharp",) + case).encode()) % 100000
    Q, K, V = make_inputs(B, H, N, M, D, "bf16", q_scale=qs, kv_scale=ks, seed=seed)
    dY = make_inputs(B, H, N, M, D, "bf16", seed=seed + 1)[2]
    print(f"[backward] sharp case={case} seed={seed}", flush=True)
    got = F.flare_backward(to_dev(Q), to_dev(K), to_dev(V), to_dev(dY))
    torch.cuda.synchronize()
    check(got, oracle.backward(Q, K, V, dY), "bf16", f"sharp {case}")


@pytest.mark.parametrize("D,M", [(32, 50), (64, 50), (64, 100)])
def test_backward_negative_logits(D, M):
    # Every logit near -200 in log2 units (a common component of Q and K
    # pointing in opposite directions), with padded latents: the exponentials
    # against the encode's offsets underflow unless every kernel takes its
    # offsets from the statistics of this head; (64, 50) runs the fused dZ
    # path, (64, 100) the separate latent pass.
    rng = np.random.default_rng(1000 + D + M)
    B, H, N = 1, 2, 1500
    q = 0.3 * rng.standard_normal((H, M, D), dtype=np.float32)
    k = 0.3 * rng.standard_normal((B, H, N, D), dtype=np.float32)
    v = rng.standard_normal((B, H, N, D), dtype=np.float32)
    g = rng.standard_normal((B, H, N, D), dtype=np.float32)
    q[..., 0] -= 33.0
    k[..., 0] += 33.0
    Q, K, V, dY = (f32_to_bf16_bits(x) for x in (q, k, v, g))
    print(f"[backward] negative logits D={D} M={M}", flush=True)
    got = F.flare_backward(to_dev(Q), to_dev(K), to_dev(V), to_dev(dY))
    torch.cuda.synchronize()
    want = oracle.backward(Q, K, V, dY)
    for g, w, name in zip(got, want, ("dQ", "dK", "dV")):
        print(f"[backward] negative D={D} M={M} {name} {errors(to_host64(g), w)}", flush=True)
    check_one(got[1], want[1], "bf16", f"negative D={D} M={M} dK")
    check_one(got[2], want[2], "bf16", f"negative D={D} M={M} dV")
    # dQ = s dl K. Along d = 0, the direction every key shares (K[n][0] near
    # 33), the entries are sums whose terms cancel: the encode part of each
    # row of dl sums to zero exactly, and on this input sum_n |dl[m][n]| is
    # 100-400 times |sum_n dl[m][n]|. One bf16 rounding of each dl term
    # (relative 2^-9, the matrix-core operand) then leaves an error up to
    # s 2^-9 sum_n |dl[m][n]| |K[n][0]| (0.2-0.7 on these inputs, measured
    # 0.02-0.17), which no element bar on that column can hold. The other
    # columns carry no shared component and meet the bar; column 0 must be
    # finite.
    dq = to_host64(got[0])
    assert np.isfinite(dq).all()
    check_one(got[0][..., 1:], want[0][..., 1:], "bf16", f"negative D={D} M={M} dQ[..., 1:]")


def test_backward_workspace_variant_is_identical():
    B, H, N, M, D, dt = 2, 2, 900, 64, 32, "bf16"
    Q, K, V = make_inputs(B, H, N, M, D, dt, q_scale=0.5, seed=11)
    dY = make_inputs(B, H, N, M, D, dt, seed=12)[2]
    q, k, v, g = to_dev(Q), to_dev(K), to_dev(V), to_dev(dY)
    a = F.flare_backward(q, k, v, g)
    ws = torch.empty(F.flare_workspace_size(F.FLARE_OP_BACKWARD, B, H, N, M, D, q.dtype), dtype=torch.uint8,
                     device="cuda")
    b = F.flare_backward(q, k, v, g, workspace=ws)
    c = F.flare_backward(q, k, v, g, workspace=ws)
    torch.cuda.synchronize()
    for x, y, z in zip(a, b, c):
        assert torch.equal(x, y) and torch.equal(y, z)


def test_backward_full_size_one_head_group():
    # the 65k-mesh workload: every gradient of head 0 (dQ[0] sums its four
    # batch entries) against the oracle
    w = WORKLOADS[2]
    Qh, Kh, Vh = workload_inputs(w)
    dY = make_inputs(w.B, w.H, w.N, w.M, w.D, w.dtype, seed=99)[2]
    print(f"[backward] full size {w.name}", flush=True)
    dQ, dK, dV = F.flare_backward(to_dev(Qh), to_dev(Kh), to_dev(Vh), to_dev(dY))
    torch.cuda.synchronize()
    dq_ref = np.zeros((w.M, w.D))
    for b in range(w.B):
        dq, dk, dv = oracle.backward_head(oracle.widen(Qh[0]), oracle.widen(Kh[b, 0]), oracle.widen(Vh[b, 0]),
                                          oracle.widen(dY[b, 0]))
        dq_ref += dq
        check_one(dK[b, 0], dk, "bf16", f"{w.name} dK b={b}")
        check_one(dV[b, 0], dv, "bf16", f"{w.name} dV b={b}")
    check_one(dQ[0], dq_ref, "bf16", f"{w.name} dQ")


PP_CASES = [
    # B, H, N, M, D, dtype
    (2, 1, 600, 400, 64, "bf16"),  # latent ranges in both stages (the first with dZ given)
    (1, 1, 500, 250, 128, "bf16"),  # the same at D = 128
    (1, 1, 300, 400, 128, "bf16"),  # and with statistics over ranges (second stage)
    (2, 2, 300, 40, 32, "f32"),
    (1, 1, 500, 17, 16, "f32"),
    (2, 2, 1000, 64, 64, "bf16"),
    (1, 2, 777, 33, 32, "bf16"),
    (2, 1, 3000, 128, 32, "bf16"),
    (1, 1, 1, 1, 32, "bf16"),
    (2, 1, 400, 48, 128, "bf16"),
    (1, 2, 300, 20, 96, "f32"),
    (1, 1, 900, 256, 64, "bf16"),  # encode-only latent kernel with four latent blocks per wave
]


@pytest.mark.parametrize("case", PP_CASES, ids=case_id)
def test_pp_backward_matches_oracle(case):
    B, H, N, M, D, dt = case
    seed = zlib.crc32(repr(("pp_backward",) + case).encode()) % 100000
    Q, K, V = make_inputs(B, H, N, M, D, dt, q_scale=0.5, seed=seed)
    dY = make_inputs(B, H, N, M, D, dt, seed=seed + 1)[2]
    print(f"[pp_backward] case={case_id(case)} seed={seed}", flush=True)
    got = F.flare_pp_backward(to_dev(Q), to_dev(K), to_dev(V), to_dev(dY))
    torch.cuda.synchronize()
    check(got, oracle.pp_backward(Q, K, V, dY), dt, "pp " + case_id(case))


def test_pp_backward_workspace_variant_is_identical():
    B, H, N, M, D, dt = 2, 2, 900, 64, 32, "bf16"
    Q, K, V = make_inputs(B, H, N, M, D, dt, q_scale=0.5, seed=31)
    dY = make_inputs(B, H, N, M, D, dt, seed=32)[2]
    q, k, v, g = to_dev(Q), to_dev(K), to_dev(V), to_dev(dY)
    a = F.flare_pp_backward(q, k, v, g)
    ws = torch.empty(F.flare_workspace_size(F.FLARE_OP_PP_BACKWARD, B, H, N, M, D, q.dtype), dtype=torch.uint8,
                     device="cuda")
    b = F.flare_pp_backward(q, k, v, g, workspace=ws)
    c = F.flare_pp_backward(q, k, v, g, workspace=ws)
    torch.cuda.synchronize()
    for x, y, z in zip(a, b, c):
        assert torch.equal(x, y) and torch.equal(y, z)


def test_pp_backward_full_size_one_head_group():
    # FLARE++ at the 65k-mesh size: every gradient of head 0 (dQ[0] sums its
    # four batch entries) against the oracle
    w = WORKLOADS[2]
    Qh, Kh, Vh = workload_inputs(w)
    dY = make_inputs(w.B, w.H, w.N, w.M, w.D, w.dtype, seed=98)[2]
    print(f"[pp_backward] full size {w.name}", flush=True)
    dQ, dK, dV = F.flare_pp_backward(to_dev(Qh), to_dev(Kh), to_dev(Vh), to_dev(dY))
    torch.cuda.synchronize()
    dq_ref = np.zeros((w.M, w.D))
    for b in range(w.B):
        dq, dk, dv = oracle.pp_backward_head(oracle.widen(Qh[0]), oracle.widen(Kh[b, 0]), oracle.widen(Vh[b, 0]),
                                             oracle.widen(dY[b, 0]))
        dq_ref += dq
        check_one(dK[b, 0], dk, "bf16", f"pp {w.name} dK b={b}")
        check_one(dV[b, 0], dv, "bf16", f"pp {w.name} dV b={b}")
    check_one(dQ[0], dq_ref, "bf16", f"pp {w.name} dQ")
