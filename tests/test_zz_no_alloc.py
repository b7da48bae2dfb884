"""moe_exl3_layer_noalloc (the library's per-GPU scratch array as workspace)
against moe_exl3_layer with a caller workspace, through the C ABI: two calls in
a row, the second with fewer tokens, each bit-identical to the workspace
entry point (the two share every kernel); and the size limit."""
import numpy as np
import pytest
import torch

import trellis_quantized_moe_exl3_amd as M
import workloads as W
from gpu_util import DevLayer

pytestmark = pytest.mark.gpu


def _both(dl, x):
    ref = torch.empty_like(x)
    ws = dl.workspace(x.shape[0])
    M.layer(dl.desc, dl.weights, x, ref, ws)
    got = torch.full_like(x, -1)
    M.layer_noalloc(dl.desc, dl.weights, x, got)
    torch.cuda.synchronize()
    return got.cpu(), ref.cpu()


@pytest.mark.parametrize("name,T1,T2", [("tiny", 300, 37), ("decode", 64, 8)])
def test_noalloc_matches_workspace_entry_two_calls(name, T1, T2):
    inp = W.gen_layer(W.BY_NAME[name].replace(tokens=T1))
    dl = DevLayer(inp)
    for T in (T1, T2):
        x = dl.x[:T].contiguous()
        got, ref = _both(dl, x)
        assert torch.equal(got, ref), f"T={T}: {(got != ref).sum().item()} elements differ"
        assert np.isfinite(W.act_bits_to_f32(got.numpy().view(np.uint16), inp.cfg.act_dtype)).all()


def test_noalloc_rejects_calls_beyond_its_array():
    inp = W.gen_layer(W.BY_NAME["decode"].replace(tokens=8))
    dl = DevLayer(inp)
    T = 2048
    assert M.workspace_size(dl.desc, T) > M.SCRATCH_BYTES
    x = torch.zeros((T, inp.cfg.hidden), dtype=torch.int16, device="cuda")
    out = torch.empty_like(x)
    with pytest.raises(M.MoeError) as ei:
        M.layer_noalloc(dl.desc, dl.weights, x, out)
    assert ei.value.code == M.ERR_WORKSPACE
