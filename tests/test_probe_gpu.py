"""GPU checks of the peak probes bench.py reports beside the published peaks:
they run over the whole chip, their outputs are finite, and the rates they
give lie below the published dense peaks (2.5 PFLOP/s bf16 MFMA) and above a
floor that only a broken probe would miss."""
import numpy as np
import pytest
import torch

from rank_latent_attention_flare_amd import flare as F

pytestmark = pytest.mark.gpu


def timed(launch):
    launch()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    work = launch()
    e1.record()
    torch.cuda.synchronize()
    return work, e0.elapsed_time(e1) * 1e-3


def test_mfma_probe_rate_is_plausible():
    out = torch.empty(F.flare_probe_lanes(), dtype=torch.float32, device="cuda")
    work, t = timed(lambda: F.flare_probe_peak(F.FLARE_PROBE_MFMA_BF16, 1000, out))
    assert work == F.flare_probe_lanes() / 64 * 1000 * 4 * 32768
    assert torch.isfinite(out).all()
    rate = work / t
    print(f"[probe] bf16 MFMA {rate / 1e12:.0f} TFLOP/s", flush=True)
    assert 1e14 < rate <= 2.5e15 * 1.02


def test_exp_probe_rate_is_plausible():
    out = torch.empty(F.flare_probe_lanes(), dtype=torch.float32, device="cuda")
    work, t = timed(lambda: F.flare_probe_peak(F.FLARE_PROBE_EXP, 2000, out))
    assert work == F.flare_probe_lanes() * 2000 * 16
    # x <- 2^(-x) from [0.5, 1] stays in [0.5, 1]
    assert bool(((out >= 8.0) & (out <= 16.0)).all())
    rate = work / t
    print(f"[probe] v_exp_f32 {rate / 1e12:.2f} T/s", flush=True)
    # 256 CUs x 4 SIMDs x 16 lanes per clock at 2.4 GHz is 39e12 lane-ops/s
    assert 1e11 < rate < 4e13


def test_read_kernel_folds_every_vector():
    # XOR of every 32-bit word of the buffer, folded per lane, then over
    # lanes: each word appears once, so the lane results XOR to the XOR of
    # all words (low 16 bits, as the kernel stores them)
    g = torch.Generator(device="cuda").manual_seed(5)
    src = torch.randint(0, 2**31 - 1, ((1 << 22) + 4,), dtype=torch.int32, device="cuda", generator=g)
    out = torch.empty(F.flare_probe_lanes(), dtype=torch.float32, device="cuda")
    F.flare_read_kernel(src, out)
    torch.cuda.synchronize()
    got = int(np.bitwise_xor.reduce(out.cpu().numpy().astype(np.int64)))
    want = int(np.bitwise_xor.reduce(src.cpu().numpy().astype(np.int64))) & 0xffff
    assert got == want
