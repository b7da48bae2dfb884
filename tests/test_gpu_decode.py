"""Bit-exact parity of the HIP trellis decode (moe_exl3_decode) with the oracle."""
import numpy as np
import pytest
import torch

import oracle
import trellis_quantized_moe_exl3_amd as M
from gpu_util import dev

pytestmark = pytest.mark.gpu

MCG = 0x9E3779B1


def _gpu_decode(codes, n_in, n_out, K, cb, dt, mcg=MCG):
    dtype = {M.DT_F32: torch.float32, M.DT_F16: torch.int16, M.DT_BF16: torch.int16,
             M.DT_FP8: torch.uint8}[dt]
    dst = torch.empty((n_in, n_out), dtype=dtype, device="cuda")
    M.decode(dev(codes), n_in, n_out, K, mcg, cb, dst, dt)
    torch.cuda.synchronize()
    return dst.cpu()


def _expect(ref: np.ndarray, dt):
    t = torch.from_numpy(ref)
    if dt == M.DT_F32:
        return t
    if dt == M.DT_F16:
        return t.to(torch.float16).view(torch.int16)
    if dt == M.DT_BF16:
        return t.to(torch.bfloat16).view(torch.int16)
    return t.to(torch.float8_e4m3fn).view(torch.uint8)


@pytest.mark.parametrize("K", [2, 3, 4])
@pytest.mark.parametrize("cb", [0, 1])
@pytest.mark.parametrize("dt", [M.DT_F32, M.DT_F16, M.DT_BF16, M.DT_FP8])
def test_decode_small_bit_exact(K, cb, dt):
    n_in, n_out = 48, 96
    rng = np.random.default_rng(100 * K + 10 * cb + dt)
    codes = rng.integers(0, 1 << 16, (n_in // 16) * (n_out // 16) * 16 * K, dtype=np.uint16)
    ref = oracle.decode_matrix(codes, n_in, n_out, K, MCG, cb)
    if dt == M.DT_FP8 and cb == 0:
        ref = np.vectorize(oracle.e4m3_rne)(ref.astype(np.float64)).astype(np.float32)
    got = _gpu_decode(codes, n_in, n_out, K, cb, dt)
    exp = _expect(ref, dt)
    assert torch.equal(got, exp), f"mismatches: {(got != exp).sum().item()}"


@pytest.mark.parametrize("K", [2, 3, 4])
def test_decode_full_projection_bit_exact(K):
    # one expert's gate projection at the real shape [4096][2048]
    n_in, n_out = 4096, 2048
    rng = np.random.default_rng(7 + K)
    codes = rng.integers(0, 1 << 16, (n_in // 16) * (n_out // 16) * 16 * K, dtype=np.uint16)
    ref = oracle.decode_matrix(codes, n_in, n_out, K, MCG, 0)
    got = _gpu_decode(codes, n_in, n_out, K, 0, M.DT_F32).numpy()
    np.testing.assert_array_equal(got, ref)
    again = _gpu_decode(codes, n_in, n_out, K, 0, M.DT_F32).numpy()
    np.testing.assert_array_equal(again, got)


@pytest.mark.parametrize("mcg", [1, 0xFFFFFFFF, 0x12345679])
def test_decode_other_multipliers(mcg):
    K, n_in, n_out = 3, 32, 32
    rng = np.random.default_rng(mcg & 0xFFFF)
    codes = rng.integers(0, 1 << 16, 4 * 16 * K, dtype=np.uint16)
    ref = oracle.decode_matrix(codes, n_in, n_out, K, mcg, 0)
    got = _gpu_decode(codes, n_in, n_out, K, 0, M.DT_F32, mcg=mcg).numpy()
    np.testing.assert_array_equal(got, ref)
