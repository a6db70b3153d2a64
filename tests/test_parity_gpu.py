"""GPU parity of libflare (through the C ABI) against the fp64 CPU oracle.

* small and ragged shapes: every output element against the oracle, for all
  four entry points and both storage types (several tiles, tails of tokens
  and of latents, N = 1, M = 1);
* the five workloads at full size, in the launch configuration the benchmark
  times (caller workspace): sampled tokens of two heads against the oracle,
  computed one by one;
* properties that hold at any size: constant V, zero queries, scaling and
  permutation of the tokens, determinism, chunk-count invariance, and the
  composition identities between the entry points.
"""
import json
import os
import zlib

import numpy as np
import pytest
import torch

import oracle
from flare_inputs import WORKLOADS, f32_to_bf16_bits, make_inputs, workload_inputs
from rank_latent_attention_flare_amd import flare as F
from tests.gpu_util import assert_parity, errors, sample_rows, to_dev, to_host64

pytestmark = pytest.mark.gpu

OPS = {"encode": F.flare_encode, "decode": F.flare_decode, "forward": F.flare_forward, "pp_forward": F.flare_pp_forward}
OPCODE = {"encode": F.FLARE_OP_ENCODE, "decode": F.FLARE_OP_DECODE, "forward": F.FLARE_OP_FORWARD,
          "pp_forward": F.FLARE_OP_PP_FORWARD}

SMALL = [
    # B, H, N, M, D, dtype
    (1, 4, 1024, 32, 16, "f32"),
    (1, 3, 3000, 40, 8, "f32"),
    (2, 2, 1, 1, 64, "f32"),
    (1, 1, 2500, 300, 32, "f32"),
    # fp32 lanes per latent / token: 2 and 4 lanes (few latents or tokens),
    # D = 24 (2 lanes at most), D = 96 and 128, and one lane per token in a
    # decode of more than 2^18 token rows
    (2, 1, 900, 12, 24, "f32"),
    (1, 2, 600, 16, 128, "f32"),
    (1, 1, 500, 70, 48, "f32"),
    (1, 1, 300, 20, 96, "f32"),
    (1, 2, 140000, 24, 32, "f32"),
    (2, 3, 1000, 64, 64, "bf16"),
    (1, 2, 4097, 100, 32, "bf16"),
    (1, 1, 1, 1, 32, "bf16"),
    (1, 2, 7, 17, 64, "bf16"),
    (1, 1, 300, 256, 128, "bf16"),
    (2, 1, 5000, 200, 64, "bf16"),
    (1, 2, 777, 33, 128, "bf16"),
    (3, 1, 2049, 128, 32, "bf16"),
    (1, 2, 640, 64, 128, "bf16"),
    # more than 8 latent blocks (D <= 64): the decode's grouped latent loop,
    # with and without a padded last block
    (1, 2, 1500, 300, 64, "bf16"),
    (1, 1, 1000, 512, 32, "bf16"),
    (2, 1, 700, 480, 64, "bf16"),
    # D = 64 with exactly 256 latents (twelve-wave decode workgroups) and with
    # 512 (eight-wave workgroups), ragged tokens
    (1, 2, 3001, 256, 64, "bf16"),
    (1, 1, 2500, 512, 64, "bf16"),
    # D = 128 beyond 256 latents: encode workgroups over two latent groups,
    # decode in two launches over the latent ranges (the second ragged at 300)
    (1, 2, 1500, 512, 128, "bf16"),
    (2, 1, 777, 300, 128, "bf16"),
]


def small_id(c):
    return "B{}H{}N{}M{}D{}-{}".format(*c)


def oracle_for(op, Q, K, V):
    if op == "encode":
        return oracle.encode(Q, K, V)
    if op == "decode":
        return oracle.decode(Q, K, V)
    if op == "forward":
        return oracle.forward(Q, K, V)[0]
    return oracle.pp_forward(Q, K, V)[0]


@pytest.mark.parametrize("op", list(OPS))
@pytest.mark.parametrize("case", SMALL, ids=small_id)
def test_small_shapes_match_oracle(op, case):
    B, H, N, M, D, dt = case
    seed = zlib.crc32(repr((op,) + case).encode()) % 100000
    Q, K, V = make_inputs(B, H, N, M, D, dt, q_scale=0.5, seed=seed)
    if op == "decode":
        Zr = oracle.encode(Q, K, V)
        V = Zr.astype(np.float32) if dt == "f32" else f32_to_bf16_bits(Zr.astype(np.float32))
    print(f"[small] op={op} case={small_id(case)} seed={seed}", flush=True)
    out = OPS[op](to_dev(Q), to_dev(K), to_dev(V))
    torch.cuda.synchronize()
    assert_parity(to_host64(out), oracle_for(op, Q, K, V), dt, f"{op} {small_id(case)}")


@pytest.mark.parametrize("op", ["forward", "pp_forward"])
def test_ws_variant_equals_allocating_variant(op):
    Q, K, V = (to_dev(x) for x in make_inputs(2, 2, 3000, 96, 64, "bf16", 0.5, seed=11))
    a = OPS[op](Q, K, V)
    b = OPS[op](Q, K, V, workspace=F.workspace_for(OPCODE[op], Q, K))
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# ------------------------------------------------------------ full workloads
_cache = {}


def workload(i):
    if i not in _cache:
        _cache.clear()
        w = WORKLOADS[i]
        print(f"[workload] generating {w.name}", flush=True)
        Q, K, V = workload_inputs(w)
        _cache[i] = (w, Q, K, V, to_dev(Q), to_dev(K), to_dev(V))
    return _cache[i]


def heads_to_check(w):
    return [(0, 0), (w.B - 1, w.H - 1)] if w.B * w.H > 1 else [(0, 0)]


@pytest.mark.parametrize("i", [1, 2, 3, 4, 5, 6, 7])
def test_workload_matches_oracle_on_sampled_tokens(i):
    w, Q, K, V, Qd, Kd, Vd = workload(i)
    op = w.op
    print(f"[workload] {w.name} op={op} plan: {F.flare_describe_plan(OPCODE[op], w.B, w.H, w.N, w.M, w.D, Qd.dtype)}",
          flush=True)
    ws = F.workspace_for(OPCODE[op], Qd, Kd)
    Y = OPS[op](Qd, Kd, Vd, workspace=ws)
    torch.cuda.synchronize()
    rows = sample_rows(w.N, 2048, seed=i)
    heads = heads_to_check(w) if i != 1 else None
    rows_arg = rows if i != 1 else None
    if op == "forward":
        Yo, Zo = oracle.forward(Q, K, V, rows=rows_arg, heads=heads)
    else:
        Yo, _, Zo = oracle.pp_forward(Q, K, V, rows=rows_arg, heads=heads)
    Yg = to_host64(Y[:, :, torch.from_numpy(rows).cuda()] if rows_arg is not None else Y)
    report = {"workload": w.name, "op": op, "tokens_checked": int(len(rows) if rows_arg is not None else w.N),
              "heads": heads or "all", "Y": {}, "Z": {}}
    for (b, h) in (heads or [(b, h) for b in range(w.B) for h in range(w.H)]):
        e = assert_parity(Yg[b, h], Yo[b, h], w.dtype, f"{w.name} Y head ({b},{h})")
        report["Y"][f"{b},{h}"] = e
    if op == "forward":
        Z = F.flare_encode(Qd, Kd, Vd, workspace=F.workspace_for(F.FLARE_OP_ENCODE, Qd, Kd))
        Zg = to_host64(Z)
        for (b, h) in (heads or [(b, h) for b in range(w.B) for h in range(w.H)]):
            report["Z"][f"{b},{h}"] = assert_parity(Zg[b, h], Zo[b, h], w.dtype, f"{w.name} Z head ({b},{h})")
    out_dir = os.environ.get("FLARE_REPORT_DIR")
    if out_dir:
        os.makedirs(out_dir, exist_ok=True)
        with open(os.path.join(out_dir, f"parity_{w.name}.json"), "w") as f:
            json.dump(report, f, indent=1)


# --------------------------------------------------------------- properties
@pytest.mark.parametrize("i", [2, 3, 4, 5])
def test_constant_values_give_exact_constant(i):
    w, Q, K, V, Qd, Kd, Vd = workload(i)
    g = torch.Generator(device="cuda").manual_seed(100 + i)
    c = torch.randn(w.B, w.H, 1, w.D, device="cuda", generator=g).to(Vd.dtype)
    Vc = c.expand_as(Vd).contiguous()
    Y = OPS[w.op](Qd, Kd, Vc)
    torch.cuda.synchronize()
    assert torch.equal(Y, c.expand_as(Y)), f"max dev {(Y.float() - c.float()).abs().max().item()}"


@pytest.mark.parametrize("i", [2, 3, 4])
def test_values_scale_exactly(i):
    w, Q, K, V, Qd, Kd, Vd = workload(i)
    Y1 = F.flare_forward(Qd, Kd, Vd)
    Y2 = F.flare_forward(Qd, Kd, (Vd.float() * 2).to(Vd.dtype))
    torch.cuda.synchronize()
    assert torch.equal((Y1.float() * 2).to(Y1.dtype), Y2)


@pytest.mark.parametrize("i", [2, 3, 4])
def test_zero_queries_give_token_means(i):
    w, Q, K, V, Qd, Kd, Vd = workload(i)
    Y = F.flare_forward(torch.zeros_like(Qd), Kd, Vd)
    mean = Vd.double().mean(dim=2, keepdim=True)
    torch.cuda.synchronize()
    e = errors(Y.double().cpu().numpy(), mean.expand(Y.shape).cpu().numpy())
    assert e["rel_l2"] <= 1e-2 and e["max_abs"] <= 3e-2, e


@pytest.mark.parametrize("i", [2, 3, 5])
def test_token_permutation_permutes_output(i):
    w, Q, K, V, Qd, Kd, Vd = workload(i)
    g = torch.Generator(device="cuda").manual_seed(7)
    perm = torch.randperm(w.N, device="cuda", generator=g)
    Y = OPS[w.op](Qd, Kd, Vd)
    Yp = OPS[w.op](Qd, Kd[:, :, perm].contiguous(), Vd[:, :, perm].contiguous())
    torch.cuda.synchronize()
    e = errors(Yp.double().cpu().numpy(), Y[:, :, perm].double().cpu().numpy())
    assert e["rel_l2"] <= 1e-2 and e["max_abs"] <= 3e-2, e


@pytest.mark.parametrize("i", [2, 4, 5])
def test_bitwise_repeatable(i):
    w, Q, K, V, Qd, Kd, Vd = workload(i)
    ws = F.workspace_for(OPCODE[w.op], Qd, Kd)
    a = OPS[w.op](Qd, Kd, Vd, workspace=ws)
    b = OPS[w.op](Qd, Kd, Vd, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.fixture
def tuning():
    """flare_set_tuning for one test; every key is restored to the library's choice afterwards."""
    yield F.flare_set_tuning
    for key in range(F.FLARE_TUNE_KEYS):
        F.flare_set_tuning(key, 0)


@pytest.mark.parametrize("i", [2, 3])
def test_chunk_count_invariance(i, tuning):
    w, Q, K, V, Qd, Kd, Vd = workload(i)
    a = F.flare_forward(Qd, Kd, Vd)
    tuning(F.FLARE_TUNE_CHUNKS, 1)
    b = F.flare_forward(Qd, Kd, Vd)
    tuning(F.FLARE_TUNE_CHUNKS, 5)
    c = F.flare_forward(Qd, Kd, Vd)
    tuning(F.FLARE_TUNE_CHUNKS, 40)  # more than 16 chunks: the combine splits each entry over four lanes
    d = F.flare_forward(Qd, Kd, Vd)
    torch.cuda.synchronize()
    for x in (b, c, d):
        e = errors(x.double().cpu().numpy(), a.double().cpu().numpy())
        assert e["rel_l2"] <= 5e-3, e


@pytest.mark.parametrize("i", [2, 3, 4])
def test_forward_matches_decode_of_encode(i):
    # Same Z (rounded once to bf16 in both); the fused forward's decode uses
    # one offset per (b, h) from the encode, the standalone decode per-token
    # offsets, so the two agree to rounding, not bit for bit.
    w, Q, K, V, Qd, Kd, Vd = workload(i)
    Y = F.flare_forward(Qd, Kd, Vd)
    Z = F.flare_encode(Qd, Kd, Vd)
    Y2 = F.flare_decode(Qd, Kd, Z)
    torch.cuda.synchronize()
    e = errors(Y.double().cpu().numpy(), Y2.double().cpu().numpy())
    assert e["rel_l2"] <= 2e-3 and e["max_abs"] <= 3e-2, e


def test_pp_forward_is_forward_with_corrected_queries():
    # B = 1: Q' = Q + encode(Q) is per-head, so the public calls can compose it.
    Q, K, V = (to_dev(x) for x in make_inputs(1, 4, 20000, 128, 64, "bf16", 0.5, seed=21))
    Y = F.flare_pp_forward(Q, K, V)
    Qp = (Q.float() + F.flare_encode(Q, K, V)[0].float()).to(torch.bfloat16)
    Y2 = F.flare_forward(Qp.contiguous(), K, V)
    torch.cuda.synchronize()
    e = errors(Y.double().cpu().numpy(), Y2.double().cpu().numpy())
    assert e["rel_l2"] <= 1e-2 and e["max_abs"] <= 3e-2, e


@pytest.mark.parametrize("D", [32, 64])
def test_two_token_block_decode_matches_oracle(D, tuning):
    # The decode built for two 32-token blocks per wave and step (a tuning
    # alternative to the default one) against the oracle, forward and
    # standalone decode, with ragged tokens and latents.
    tuning(F.FLARE_TUNE_DEC_TB, 2)
    Q, K, V = make_inputs(1, 2, 3001, 100, D, "bf16", 0.5, seed=30 + D)
    Zb = f32_to_bf16_bits(oracle.encode(Q, K, V).astype(np.float32))
    print(f"[tb2] D={D}", flush=True)
    Y = F.flare_forward(to_dev(Q), to_dev(K), to_dev(V))
    Y2 = F.flare_decode(to_dev(Q), to_dev(K), to_dev(Zb))
    torch.cuda.synchronize()
    assert_parity(to_host64(Y), oracle.forward(Q, K, V)[0], "bf16", f"forward D={D}")
    assert_parity(to_host64(Y2), oracle.decode(Q, K, Zb), "bf16", f"decode D={D}")


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    """Half the spacing of bf16 numbers at |x| (8 significand bits): the most
    that rounding a real x to nearest bf16 can move it (normal range)."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return 2.0 ** (e - 8)


@pytest.mark.parametrize("shape", [(1, 2, 3001, 100, 64), (1, 2, 3001, 300, 128)], ids=["D64", "D128-split"])
@pytest.mark.parametrize("kind", ["large", "negative"])
def test_extreme_logits_match_oracle(kind, shape):
    # Logits far from zero, so that the offsets leave the zero-offset regime
    # of both kernels: large positive logits (c*S up to about 45 in log2
    # units), or every logit near -200 in log2 units (a common component of
    # Q and K pointing in opposite directions; about -140 at D = 128). At
    # D = 128 with 300 latents the decode runs in two launches over the
    # latent ranges; on the negative input the standalone decode's per-token
    # bound is loose enough that both launches fall back to exact maxima
    # before their merge.
    rng = np.random.default_rng(71 if kind == "large" else 72)
    B, H, N, M, D = shape
    q = rng.standard_normal((H, M, D), dtype=np.float32)
    k = rng.standard_normal((B, H, N, D), dtype=np.float32)
    v = rng.standard_normal((B, H, N, D), dtype=np.float32)
    if kind == "large":
        q *= 8.0
    else:
        q = 0.3 * q
        k = 0.3 * k
        q[..., 0] -= 33.0
        k[..., 0] += 33.0
    Q, K, V = (f32_to_bf16_bits(x) for x in (q, k, v))
    print(f"[extreme] {kind} {shape}", flush=True)
    Qd, Kd, Vd = to_dev(Q), to_dev(K), to_dev(V)
    Y = F.flare_forward(Qd, Kd, Vd)
    Yp = F.flare_pp_forward(Qd, Kd, Vd)
    Qp = F.flare_pp_queries(Qd, Kd, Vd)
    Zb = f32_to_bf16_bits(oracle.encode(Q, K, V).astype(np.float32))
    Yd = F.flare_decode(Qd, Kd, to_dev(Zb))
    torch.cuda.synchronize()
    assert_parity(to_host64(Y), oracle.forward(Q, K, V)[0], "bf16", f"forward {kind}")
    assert_parity(to_host64(Yd), oracle.decode(Q, K, Zb), "bf16", f"decode {kind}")
    # FLARE++ stores its corrected queries Q' = Q + Z0 in bf16 before the
    # second pass. At these logits that rounding alone moves Y by more than the
    # element bound (oracle against oracle: forward at bf16(Q'), pp_forward at
    # fp64 Q', about 6e-2 on the "large" input), so the pass is checked in its
    # two stages:
    #  1. the library's own Q' (flare_pp_queries, the Q' flare_pp_forward uses)
    #     against the oracle's fp64 Q': within the bf16 rounding of the stored
    #     value (half a bf16 spacing) plus the Z bar, element by element;
    Yo_pp, Qp_or, _ = oracle.pp_forward(Q, K, V)
    Qp_g = to_host64(Qp)
    bound = bf16_half_ulp(Qp_or) * (1 + 2.0 ** -14) + 3e-2  # (fp32 sum, then bf16)
    worst = float(np.max(np.abs(Qp_g - Qp_or) - bound))
    assert worst <= 0.0, f"Q' outside rounding + Z bar by {worst:.3e}"
    #  2. flare_pp_forward is flare_forward at that Q' (B = 1, same plan), bit
    #     for bit, and meets the standard bar against the oracle's forward at
    #     that same Q'.
    Yf = F.flare_forward(Qp[0].contiguous(), Kd, Vd)
    torch.cuda.synchronize()
    assert torch.equal(Yp.view(torch.int16), Yf.view(torch.int16))
    Yo_at_qp = oracle.forward(Qp_g[0], K, V)[0]
    e = assert_parity(to_host64(Yp), Yo_at_qp, "bf16", f"pp_forward {kind}")
    # Recorded, not asserted: the whole pass against the oracle's fp64-Q'
    # pass, and the part of that difference the bf16 Q' alone makes (oracle
    # against oracle); by the triangle inequality the first is at most the
    # second plus the stage-2 error asserted above.
    print(f"[extreme] {kind} pp_forward at the library's Q': {e}; against fp64 Q': "
          f"{errors(to_host64(Yp), Yo_pp)}; bf16 Q' alone: {errors(Yo_at_qp, Yo_pp)}", flush=True)
