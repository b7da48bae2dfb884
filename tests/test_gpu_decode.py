"""Bit-exact parity of the HIP trellis decode (moe_exl3_decode) with the oracle.

Each output mode runs the fragment decoder of one kernel of the layer, so the
values checked here are the values those kernels compute with:
F16 (gate/up MFMA), BF16 (down MFMA), FP8 (fp8 MFMA), GEMV_F16 (the
decode-fused GEMV's fp16 operand 128 c + 1532), MFMA_BIASED_F16 (the gate/up
MFMA's operand on one-block tiles, mcg codebook, 128 c + 1532) and F32."""
import numpy as np
import pytest
import torch

import oracle
import trellis_quantized_moe_exl3_amd as M
from gpu_util import dev

pytestmark = pytest.mark.gpu

MCG = 0x9E3779B1
MODES = [M.DT_F32, M.DT_F16, M.DT_BF16, M.DT_FP8, M.DT_GEMV_F16, M.DT_MFMA_BIASED_F16]
BIASED = (M.DT_GEMV_F16, M.DT_MFMA_BIASED_F16)


def _gpu_decode(codes, n_in, n_out, K, cb, dt, mcg=MCG):
    dtype = {M.DT_F32: torch.float32, M.DT_F16: torch.int16, M.DT_BF16: torch.int16,
             M.DT_FP8: torch.uint8, M.DT_GEMV_F16: torch.int16, M.DT_MFMA_BIASED_F16: torch.int16}[dt]
    # poisoned: every element must be written
    dst = torch.full((n_in, n_out), -1, dtype=dtype, device="cuda")
    M.decode(dev(codes), n_in, n_out, K, mcg, cb, dst, dt)
    torch.cuda.synchronize()
    return dst.cpu()


def _expect(ref: np.ndarray, dt, cb):
    """The exact value each mode must hold, from the oracle's fp32 c values."""
    if dt == M.DT_FP8 and cb == 0:
        # the MCG codebook is rounded to E4M3 by the oracle's own routine
        ref = np.vectorize(oracle.e4m3_rne)(ref.astype(np.float64)).astype(np.float32)
    t = torch.from_numpy(ref)
    if dt == M.DT_F32:
        return t
    if dt == M.DT_F16:
        return t.to(torch.float16).view(torch.int16)
    if dt == M.DT_BF16:
        return t.to(torch.bfloat16).view(torch.int16)
    if dt in BIASED:
        biased = ref.astype(np.float64) * 128.0 + 1532.0
        assert (biased == np.round(biased)).all() and biased.min() >= 1020 and biased.max() <= 2044
        return torch.from_numpy(biased).to(torch.float16).view(torch.int16)
    return t.to(torch.float8_e4m3fn).view(torch.uint8)


@pytest.mark.parametrize("K", [2, 3, 4])
@pytest.mark.parametrize("cb", [0, 1])
@pytest.mark.parametrize("dt", MODES)
def test_decode_small_bit_exact(K, cb, dt):
    if dt == M.DT_MFMA_BIASED_F16 and cb == 1:
        pytest.skip("the one-block MFMA tiles use the F16 decoder with the E4M3 codebook")
    n_in, n_out = 48, 96
    rng = np.random.default_rng(100 * K + 10 * cb + dt)
    codes = rng.integers(0, 1 << 16, (n_in // 16) * (n_out // 16) * 16 * K, dtype=np.uint16)
    ref = oracle.decode_matrix(codes, n_in, n_out, K, MCG, cb)
    got = _gpu_decode(codes, n_in, n_out, K, cb, dt)
    exp = _expect(ref, dt, cb)
    assert torch.equal(got, exp), f"mismatches: {(got != exp).sum().item()}"


@pytest.mark.parametrize("K", [2, 3, 4])
@pytest.mark.parametrize("cb", [0, 1])
def test_decode_full_projection_bit_exact(K, cb):
    # one expert's gate projection at the real shape [4096][2048], every mode
    n_in, n_out = 4096, 2048
    rng = np.random.default_rng(7 + K + 10 * cb)
    codes = rng.integers(0, 1 << 16, (n_in // 16) * (n_out // 16) * 16 * K, dtype=np.uint16)
    ref = oracle.decode_matrix(codes, n_in, n_out, K, MCG, cb)
    for dt in MODES:
        if dt == M.DT_FP8 and cb == 0:
            continue   # the E4M3 rounding of the plain codebook is covered at the small size
        if dt == M.DT_MFMA_BIASED_F16 and cb == 1:
            continue   # mcg only
        got = _gpu_decode(codes, n_in, n_out, K, cb, dt)
        exp = _expect(ref, dt, cb)
        assert torch.equal(got, exp), f"dt={dt} mismatches: {(got != exp).sum().item()}"
    again = _gpu_decode(codes, n_in, n_out, K, cb, M.DT_GEMV_F16)
    assert torch.equal(again, _expect(ref, M.DT_GEMV_F16, cb))


@pytest.mark.parametrize("mcg", [1, 0xFFFFFFFF, 0x12345679])
@pytest.mark.parametrize("dt", [M.DT_F32, M.DT_F16, M.DT_GEMV_F16, M.DT_MFMA_BIASED_F16])
def test_decode_other_multipliers(mcg, dt):
    K, n_in, n_out = 3, 32, 32
    rng = np.random.default_rng(mcg & 0xFFFF)
    codes = rng.integers(0, 1 << 16, 4 * 16 * K, dtype=np.uint16)
    ref = oracle.decode_matrix(codes, n_in, n_out, K, mcg, 0)
    got = _gpu_decode(codes, n_in, n_out, K, 0, dt, mcg=mcg)
    assert torch.equal(got, _expect(ref, dt, 0))


def test_decode_mfma_biased_rejects_e4m3_codebook():
    codes = torch.zeros(16 * 2, dtype=torch.int16, device="cuda")
    dst = torch.zeros((16, 16), dtype=torch.int16, device="cuda")
    with pytest.raises(M.MoeError) as e:
        M.decode(codes, 16, 16, 2, MCG, 1, dst, M.DT_MFMA_BIASED_F16)
    assert e.value.code == M.ERR_UNSUPPORTED
