"""Helpers for the GPU parity tests: move seeded inputs to the device, call the
layer through the C ABI, compare with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import trellis_quantized_moe_exl3_amd as M
import workloads as W


def dev(a: np.ndarray) -> torch.Tensor:
    """Device tensor with the same bytes (16-bit types travel as int16)."""
    a = np.ascontiguousarray(a)
    if a.dtype in (np.uint16, np.float16):
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


class DevLayer:
    """Device copies of a LayerInputs plus the descriptor/weights structs."""

    def __init__(self, inp: W.LayerInputs, shared: bool = True, flags: int = 0,
                 gemv_max_rows: int = 0):
        cfg = inp.cfg
        self.inp = inp
        # codes drawn for a subset of experts (a dict) are not needed on the
        # device by routing-only tests
        self.code_tab = self.k_tab = None
        if inp.ktab is not None and not isinstance(inp.codes[0], dict):
            # one pool per projection, each tensor at its own width; the
            # table holds every tensor's device address
            self.codes = [dev(np.concatenate([np.asarray(t, dtype=np.uint16) for t in c])) for c in inp.codes]
            addr = np.zeros((3, cfg.n_trellis), dtype=np.int64)
            for p in range(3):
                off = 0
                for e in range(cfg.n_trellis):
                    addr[p, e] = self.codes[p].data_ptr() + 2 * off
                    off += cfg.words_of(p, e, inp.ktab)
            self.code_tab = dev(addr)
            self.k_tab = dev(np.ascontiguousarray(inp.ktab, dtype=np.int32))
            flags |= M.PER_TENSOR_K
        else:
            self.codes = [None if isinstance(c, dict) else dev(c) for c in inp.codes]
        self.signs = dev(inp.signs) if inp.signs is not None else None
        if self.signs is not None:
            flags |= M.HADAMARD
        if cfg.shared_trellis:
            flags |= M.SHARED_TRELLIS
        self.suh = [dev(s) for s in inp.suh]
        self.svh = [dev(s) for s in inp.svh]
        self.router_w = dev(inp.router_w)
        self.bias = dev(inp.router_bias) if inp.router_bias is not None else None
        self.shared = [dev(s) for s in inp.shared] if (inp.shared is not None and shared) else None
        f = flags
        if self.shared is not None:
            f |= M.HAS_SHARED
        if self.bias is not None:
            f |= M.HAS_ROUTER_BIAS
        self.desc = M.make_desc(cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k, cfg.K,
                                cfg.codebook, cfg.mcg, cfg.act_dtype, f, gemv_max_rows)
        self.weights = M.make_weights(self.codes, self.suh, self.svh, self.router_w, self.bias,
                                      self.shared, self.signs, self.code_tab, self.k_tab)
        self.x = dev(inp.x)

    def workspace(self, T: int) -> torch.Tensor:
        return poisoned_workspace(self.desc, T)

    def run(self, x: torch.Tensor = None) -> np.ndarray:
        """Layer output as fp32 numpy [T][H]."""
        x = self.x if x is None else x
        out = torch.empty_like(x)
        ws = self.workspace(x.shape[0])
        M.layer(self.desc, self.weights, x, out, ws)
        torch.cuda.synchronize()
        return W.act_bits_to_f32(host_bits(out), self.inp.cfg.act_dtype)

    def route(self, x: torch.Tensor = None):
        x = self.x if x is None else x
        T = x.shape[0]
        cfg = self.inp.cfg
        k, E = cfg.top_k, cfg.n_experts
        idx = torch.empty(T * k, dtype=torch.int32, device="cuda")
        w = torch.empty(T * k, dtype=torch.float32, device="cuda")
        counts = torch.empty(E, dtype=torch.int32, device="cuda")
        offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
        sorted_ids = torch.empty(T * k, dtype=torch.int32, device="cuda")
        pos = torch.empty(T * k, dtype=torch.int32, device="cuda")
        ws = self.workspace(T)
        M.route(self.desc, self.weights, x, idx, w, counts, offsets, sorted_ids, pos, ws)
        torch.cuda.synchronize()
        return (idx.cpu().numpy().reshape(T, k), w.cpu().numpy().reshape(T, k),
                counts.cpu().numpy(), offsets.cpu().numpy(), sorted_ids.cpu().numpy(),
                pos.cpu().numpy())


def poisoned_workspace(desc, T: int) -> torch.Tensor:
    """A workspace filled with 0xFF bytes (NaN in every float type, -1 in every
    int32), so that a read of a slot the call never wrote shows up."""
    return torch.full((M.workspace_size(desc, T),), 0xFF, dtype=torch.uint8, device="cuda")


def rel_err(out: np.ndarray, ref: np.ndarray) -> float:
    """max |out - ref| / max |ref| over the whole array."""
    den = float(np.abs(ref).max())
    assert den > 0
    return float(np.abs(out.astype(np.float64) - ref).max()) / den
