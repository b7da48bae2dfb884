"""Benchmark of the EXL3 trellis-coded MoE layer on one MI355X.

Workload (one step = one whole layer, every launch of the hot path): the
7168-token prefill chunk at GLM-5.3-Flash shapes (hidden 4096, expert
intermediate 2048, 288 experts top-8 with a skewing router bias, K = 2 mcg
codes, fp16 shared expert), seeded synthetic inputs already resident in HBM.
`value` is tokens per second of that layer.  Also timed, each in an object of
the same JSON line: the 8-token decode step at K = 2, 3, 4 (code HBM GB/s, us
per layer and the VALU-implied bound, with rotating copies of the codes so the
256 MB last-level cache cannot hold them); the 1-, 2-, 4- and 8-token verify
batches replayed from HIP graphs; the 2048-token prefill at K = 3 and K = 4;
the 16384-token E4M3-codebook layer on fp16 and fp8 MFMA; the format variants
(per-tensor K3/K4 widths, and the rotated exlr8 layout with a trellis shared
expert); the achievable HBM read bandwidth; and the CPU oracle per workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Helpers for rocprofv3 counter passes (each does one thing and exits):

    python bench.py --profile-layer prefill --reps 2   # the layer, N times
    python bench.py --profile-layer decode --profile-tokens 1 --copies 4 --reps 100 --profile-graph
    python bench.py --copy-calibration 1024            # a plain 1 GiB copy, 4 times

The roofline's `traffic` (HBM bytes per launch of the dominant kernel) is read
from profiles/pmc_traffic_mfma_gateup_prefill.md, which records the FETCH_SIZE /
WRITE_SIZE readings, the copy-kernel scale factors and a hash of the kernel
sources they were taken with; when the sources have changed since, `traffic`
is null.
"""
from __future__ import annotations

import argparse
import ctypes as C
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP16_TFLOPS = 2500.0      # MI355X dense fp16/bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA
PEAK_HBM_GBPS = 8000.0
# VALU lane operations per second: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz
PEAK_VALU_LANE_OPS = 256 * 4 * 16 * 2.4e9
VALU_FILE = os.path.join(ROOT, "profiles", "pmc_valu_gemv_decode.md")
GEMV_ROWS = 2                  # default per-expert row count up to which the GEMV path runs
SHARED_GEMV_TOKENS = 16        # above this many tokens the shared expert's 16-bit MFMA tiles run inside
                               # the routed gate/up and down launches
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic_mfma_gateup_prefill.md")
KERNEL_SOURCES = ["mfma.hip", "gemm.h", "trellis.h", "common.h", "internal.h"]


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for n in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "trellis_quantized_moe_exl3_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic():
    """HBM bytes per launch of the gate/up MFMA kernel from the committed counter
    summary, or None when it is missing or was taken with other kernel sources."""
    try:
        kv = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if ":" in line and line.startswith("- "):
                    k, v = line[2:].split(":", 1)
                    kv[k.strip()] = v.strip().strip("`")
        if kv.get("kernel_sources_sha256") != kernel_source_hash():
            return None
        return float(kv["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def _dev(a):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype in (np.uint16, np.float16):
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


class Hip:
    """hipEvent helpers through the HIP runtime (events on the library's stream)."""

    def __init__(self):
        self.l = C.CDLL("libamdhip64.so")
        self.l.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.l.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.l.hipEventDestroy.argtypes = [C.c_void_p]
        # events and streams are pointers: without the declaration ctypes
        # would pass the handles as 32-bit ints
        self.l.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]

    def event(self):
        e = C.c_void_p()
        assert self.l.hipEventCreate(C.byref(e)) == 0
        return e.value

    def ms(self, a, b) -> float:
        f = C.c_float()
        assert self.l.hipEventElapsedTime(C.byref(f), a, b) == 0
        return f.value

    def destroy(self, e):
        self.l.hipEventDestroy(e)


def setup(cfg, copies=1, shared=True, extra_flags=0, gemv_rows=0):
    """Device inputs of a workload: `copies` copies of the codes (rotated by
    the decode legs), the descriptor and one weights struct per copy.  Format
    variants: per-tensor widths (one code pool per projection and a table of
    tensor addresses), sign vectors, a trellis shared expert."""
    import trellis_quantized_moe_exl3_amd as M
    import workloads as W
    inp = W.gen_layer(cfg)
    flags = extra_flags
    tabs = []
    if inp.ktab is not None:
        flags |= M.PER_TENSOR_K
        codes = []
        for _ in range(copies):
            pools = [_dev(np.concatenate(c)) for c in inp.codes]
            addr = np.zeros((3, cfg.n_trellis), dtype=np.int64)
            for p in range(3):
                off = 0
                for e in range(cfg.n_trellis):
                    addr[p, e] = pools[p].data_ptr() + 2 * off
                    off += cfg.words_of(p, e, inp.ktab)
            codes.append(pools)
            tabs.append(_dev(addr))
        ktab = _dev(np.ascontiguousarray(inp.ktab, dtype=np.int32))
    else:
        codes = [[_dev(c) for c in inp.codes] for _ in range(copies)]
        ktab = None
    suh = [_dev(s) for s in inp.suh]
    svh = [_dev(s) for s in inp.svh]
    rw = _dev(inp.router_w)
    bias = _dev(inp.router_bias) if inp.router_bias is not None else None
    sh = [_dev(s) for s in inp.shared] if (shared and inp.shared is not None) else None
    signs = _dev(inp.signs) if inp.signs is not None else None
    flags |= (M.HAS_SHARED if sh is not None else 0) | (M.HAS_ROUTER_BIAS if bias is not None else 0)
    flags |= (M.HADAMARD if signs is not None else 0) | (M.SHARED_TRELLIS if cfg.shared_trellis else 0)
    desc = M.make_desc(cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k, cfg.K, cfg.codebook,
                       cfg.mcg, cfg.act_dtype, flags, gemv_rows)
    weights = [M.make_weights(c, suh, svh, rw, bias, sh, signs, tabs[i] if tabs else None, ktab)
               for i, c in enumerate(codes)]
    keep = (codes, suh, svh, rw, bias, sh, signs, tabs, ktab)
    return inp, desc, weights, keep


def time_layer_graph(desc, weights_list, x, steps, hip):
    """Device ms per layer when each layer call is replayed from a HIP graph,
    as a serving loop would run a decode step: one graph per weight copy
    (captured after an eager warm-up call on the capture stream), replayed in
    the same rotation as the eager run, between two events on the replay
    stream."""
    import torch
    import trellis_quantized_moe_exl3_amd as M
    out = torch.empty_like(x)
    ws = torch.empty(M.workspace_size(desc, x.shape[0]), dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for w in weights_list:
            M.layer(desc, w, x, out, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for w in weights_list:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            M.layer(desc, w, x, out, ws)
        graphs.append(g)
    torch.cuda.synchronize()
    for i in range(len(graphs)):
        graphs[i].replay()
    stream = torch.cuda.current_stream().cuda_stream
    a, b = hip.event(), hip.event()
    torch.cuda.synchronize()
    assert hip.l.hipEventRecord(a, stream) == 0
    for i in range(steps):
        graphs[i % len(graphs)].replay()
    assert hip.l.hipEventRecord(b, stream) == 0
    torch.cuda.synchronize()
    dev_ms = hip.ms(a, b) / steps
    hip.destroy(a)
    hip.destroy(b)
    del graphs
    return dev_ms


def time_layer(desc, weights_list, x, steps, warmup, hip):
    """Times `steps` layers through moe_exl3_layer (no timing hooks inside the
    timed region) between two device synchronisations, then runs the same
    number of layers through moe_exl3_layer_profiled for the per-step split.
    Returns (ms per step from host clocks, per-step event ms [steps][STEP_END],
    device ms per step from two events around the plain run, out, workspace).
    Each event recorded between steps adds a few microseconds of its own, so
    only the plain run gives the layer time."""
    import torch
    import trellis_quantized_moe_exl3_amd as M
    out = torch.empty_like(x)
    ws = torch.empty(M.workspace_size(desc, x.shape[0]), dtype=torch.uint8, device="cuda")
    nw = len(weights_list)
    stream = torch.cuda.current_stream().cuda_stream
    for i in range(warmup):
        M.layer(desc, weights_list[i % nw], x, out, ws)
    a, b = hip.event(), hip.event()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    assert hip.l.hipEventRecord(a, stream) == 0
    for i in range(steps):
        M.layer(desc, weights_list[i % nw], x, out, ws)
    assert hip.l.hipEventRecord(b, stream) == 0
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    dev_ms = hip.ms(a, b) / steps
    hip.destroy(a)
    hip.destroy(b)
    evs = [[hip.event() for _ in range(M.STEP_END + 1)] for _ in range(steps)]
    for i in range(steps):
        M.layer_profiled(desc, weights_list[i % nw], x, out, ws, evs[i])
    torch.cuda.synchronize()
    per = np.array([[hip.ms(e[j], e[j + 1]) for j in range(M.STEP_END)] for e in evs])
    for e in evs:
        for x_ in e:
            hip.destroy(x_)
    return (t1 - t0) * 1000.0 / steps, per, dev_ms, out, ws


def routing_counts(desc, weights, x, cfg):
    import torch
    import trellis_quantized_moe_exl3_amd as M
    T = x.shape[0]
    idx = torch.empty(T * cfg.top_k, dtype=torch.int32, device="cuda")
    counts = torch.empty(cfg.n_experts, dtype=torch.int32, device="cuda")
    ws = torch.empty(M.workspace_size(desc, T), dtype=torch.uint8, device="cuda")
    M.route(desc, weights, x, idx, None, counts, None, None, None, ws)
    torch.cuda.synchronize()
    return counts.cpu().numpy()


def per_layer_percentiles(desc, weights_list, x, steps, hip):
    """Median, p10 and p90 of the device time of single layers: each layer of
    a separate pass sits between two events of its own (an event adds a few
    microseconds, which the plain pass's mean does not contain)."""
    import torch
    import trellis_quantized_moe_exl3_amd as M
    out = torch.empty_like(x)
    ws = torch.empty(M.workspace_size(desc, x.shape[0]), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    evs = [hip.event() for _ in range(steps + 1)]
    torch.cuda.synchronize()
    assert hip.l.hipEventRecord(evs[0], stream) == 0
    for i in range(steps):
        M.layer(desc, weights_list[i % len(weights_list)], x, out, ws)
        assert hip.l.hipEventRecord(evs[i + 1], stream) == 0
    torch.cuda.synchronize()
    t = np.array([hip.ms(evs[i], evs[i + 1]) for i in range(steps)])
    for e in evs:
        hip.destroy(e)
    return {"median_ms": float(np.median(t)), "p10_ms": float(np.percentile(t, 10)),
            "p90_ms": float(np.percentile(t, 90)), "layers": steps}


def expert_flops(cfg, T):
    """Algorithmic flops of the expert contractions: gate, up and down of every
    routed row (T * k) and of the shared expert (T rows when there is one)."""
    rows = T * cfg.top_k + (T if (cfg.shared or cfg.shared_trellis) else 0)
    return 6.0 * cfg.hidden * cfg.inter * rows


def recorded_valu_per_weight():
    """VALU lane instructions per routed weight of the decode GEMVs, from the
    committed counter summary (None when missing)."""
    try:
        with open(VALU_FILE) as f:
            for line in f:
                if line.startswith("VALU lane instructions per routed weight"):
                    return float(line.split("=")[-1].split(",")[0].strip())
    except (OSError, ValueError):
        pass
    return None


def decode_leg(W, M, hip, K, steps, copies=4):
    """The 8-token decode step at width K with `copies` rotating code copies:
    us per layer (plain and graph replay), the routed kernels' code GB/s and
    the VALU-implied bound of those kernels."""
    import torch
    dcfg = W.BY_NAME["decode"].replace(K=K)
    dinp, ddesc, dweights, dkeep = setup(dcfg, copies=copies)
    dx = _dev(dinp.x)
    dms, dper, ddev, _, _ = time_layer(ddesc, dweights, dx, steps, 5, hip)
    dgraph = time_layer_graph(ddesc, dweights, dx, steps, hip)
    pct = per_layer_percentiles(ddesc, dweights, dx, steps, hip)
    dcounts = routing_counts(ddesc, dweights[0], dx, dcfg)
    touched = int((dcounts > 0).sum())
    weights_n = touched * 3 * dcfg.hidden * dcfg.inter
    code_bytes = weights_n * K // 8
    dstep = {n: float(dper[:, i].mean()) for i, n in enumerate(M.STEPS)}
    routed_ms = dstep["gemv_gateup"] + dstep["mfma_gateup"] + dstep["gemv_down"] + dstep["mfma_down"]
    code_gbps = code_bytes / (routed_ms * 1e-3) / 1e9
    vpw = recorded_valu_per_weight()
    bound_us = weights_n * vpw / PEAK_VALU_LANE_OPS * 1e6 if vpw else None
    print(f"[bench] decode K={K} {ddev * 1000:.1f} us/layer ({dgraph * 1000:.1f} from graph replays), "
          f"code {code_gbps:.0f} GB/s; steps {json.dumps({k: round(v * 1000, 1) for k, v in dstep.items()})}",
          file=sys.stderr, flush=True)
    del dkeep, dweights
    torch.cuda.empty_cache()
    return {"workload": f"decode-8: T=8, K={K}, no router bias, {copies} rotating code copies",
            "us_per_layer": ddev * 1000, "us_per_layer_graph_replay": dgraph * 1000,
            "us_median": pct["median_ms"] * 1000, "us_p10": pct["p10_ms"] * 1000, "us_p90": pct["p90_ms"] * 1000,
            "host_ms_per_step": dms, "touched_experts": touched, "routed_weights": weights_n,
            "code_bytes": code_bytes, "routed_kernels_us": routed_ms * 1000, "code_GBps": code_gbps,
            "code_hbm_frac": code_gbps / PEAK_HBM_GBPS,
            "valu_per_weight": vpw, "valu_per_weight_source": "profiles/pmc_valu_gemv_decode.md (K=2)",
            "valu_bound_us": bound_us,
            "valu_bound_frac": (bound_us / (routed_ms * 1000)) if bound_us else None,
            "step_us": {k: v * 1000 for k, v in dstep.items()}}


def verify_batches(W, M, hip, steps):
    """us per layer of the 1-, 2-, 4- and 8-token verify batches, each layer
    replayed from a HIP graph with 4 rotating code copies (the decode-latency
    regime of speculative decoding)."""
    import torch
    res = {}
    for T in (1, 2, 4, 8):
        cfg = W.BY_NAME["decode"].replace(tokens=T)
        inp, desc, weights, keep = setup(cfg, copies=4)
        x = _dev(inp.x)
        res[str(T)] = time_layer_graph(desc, weights, x, steps, hip) * 1000
        del keep, weights
        torch.cuda.empty_cache()
    print(f"[bench] verify batches us/layer (graph replay) {json.dumps({k: round(v, 1) for k, v in res.items()})}",
          file=sys.stderr, flush=True)
    return {"workload": "decode shapes at T = 1, 2, 4, 8, K=2, graph replay, 4 rotating code copies",
            "us_per_layer_graph_replay": res}


def prefill_leg(W, M, hip, name, steps, flags=0, label=None):
    """One prefill-sized workload: ms per layer, per-step split, layer-level
    expert MFMA utilisation and expert weights decoded per second."""
    import torch
    cfg = W.BY_NAME[name]
    inp, desc, weights, keep = setup(cfg, extra_flags=flags)
    x = _dev(inp.x)
    ms, per, dev_ms, _, _ = time_layer(desc, weights, x, steps, 2, hip)
    step = {n: float(per[:, i].mean()) for i, n in enumerate(M.STEPS)}
    counts = routing_counts(desc, weights[0], x, cfg)
    touched = int((counts > 0).sum()) + (1 if cfg.shared_trellis else 0)
    fl = expert_flops(cfg, cfg.tokens)
    res = {"ms_per_step": ms, "device_ms_per_step": dev_ms, "tokens_per_s": cfg.tokens / (ms * 1e-3),
           "expert_tflop": fl / 1e12, "mfma_util_fp16_peak": fl / (ms * 1e-3) / (PEAK_FP16_TFLOPS * 1e12),
           "touched_trellis_experts": touched,
           "expert_weights_per_s": touched * 3 * cfg.hidden * cfg.inter / (ms * 1e-3), "step_ms": step}
    print(f"[bench] {label or name} flags={flags} {ms:.3f} ms/step; steps "
          f"{json.dumps({k: round(v, 4) for k, v in step.items()})}", file=sys.stderr, flush=True)
    del keep, weights, x
    torch.cuda.empty_cache()
    return cfg, res


def gemv_threshold_sweep(W, M, hip, steps):
    """Layer time against the per-expert row threshold between the GEMV and
    the MFMA paths (the descriptor's gemv_max_rows, at most 8; 0 is the
    default: 8 up to 8 tokens, else 2), on the 7168-token prefill layer and
    the 8-token step (4 rotating code copies)."""
    import torch
    res = {}
    for name, copies, rows in (("prefill", 1, (1, 2, 4, 8)), ("decode", 4, (1, 2, 4, 8))):
        cfg = W.BY_NAME[name]
        out = {}
        for g in rows:
            inp, desc, weights, keep = setup(cfg, copies=copies, gemv_rows=g)
            x = _dev(inp.x)
            _, _, dev_ms, _, _ = time_layer(desc, weights, x, steps, 2, hip)
            out[str(g)] = dev_ms
            del keep, weights, x
            torch.cuda.empty_cache()
        res[name] = {"ms_per_layer_by_gemv_max_rows": out}
        print(f"[bench] gemv threshold {name}: {json.dumps({k: round(v, 4) for k, v in out.items()})}",
              file=sys.stderr, flush=True)
    return res


def tile_classes(W, M, hip, steps):
    """Expert MFMA rates per row-tile class: the gate/up and down launches'
    event-timed TFLOP/s on routings whose tiles are all full (256 rows), mostly
    33-96 rows, or all at most 32 rows (no shared expert, every expert on the
    MFMA kernels)."""
    import torch
    res = {}
    for name in ("tiles_full", "tiles_mid", "tiles_small"):
        cfg = W.BY_NAME[name]
        inp, desc, weights, keep = setup(cfg)
        x = _dev(inp.x)
        ms, per, _, _, _ = time_layer(desc, weights, x, steps, 2, hip)
        step = {n: float(per[:, i].mean()) for i, n in enumerate(M.STEPS)}
        counts = routing_counts(desc, weights[0], x, cfg)
        on = counts[counts > GEMV_ROWS]
        rows, tiles = int(on.sum()), int(((on + 255) // 256).sum())
        gu, dn = step["mfma_gateup"], step["mfma_down"]
        fl = 2.0 * cfg.hidden * cfg.inter * rows
        res[name] = {"tokens": cfg.tokens, "rows_on_mfma": rows, "row_tiles": tiles,
                     "rows_per_tile": rows / tiles, "layer_ms": ms,
                     "gateup_ms": gu, "gateup_tflops": 2 * fl / (gu * 1e-3) / 1e12,
                     "gateup_us_per_tile": gu * 1000 / tiles,
                     "down_ms": dn, "down_tflops": fl / (dn * 1e-3) / 1e12,
                     "down_us_per_tile": dn * 1000 / tiles}
        print(f"[bench] {name}: {json.dumps({k: round(v, 3) for k, v in res[name].items()})}",
              file=sys.stderr, flush=True)
        del keep, weights, x
        torch.cuda.empty_cache()
    return res


def stream_read_bandwidth(hip, gib=4, reps=10):
    """Achievable HBM read bandwidth: the probe kernel streaming `gib` GiB,
    timed with events (best of `reps` passes)."""
    import torch
    path = os.path.join(ROOT, "trellis_quantized_moe_exl3_amd", "libmoe_exl3_bw.so")
    if not os.path.exists(path):
        return None
    l = C.CDLL(path)
    l.moe_exl3_bw_stream_read.argtypes = [C.c_void_p, C.c_int64, C.c_void_p, C.c_int, C.c_void_p]
    n = gib << 30
    buf = torch.ones(n // 4, dtype=torch.int32, device="cuda")
    blocks = 256 * 64
    sink = torch.zeros(blocks, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    best = 0.0
    for _ in range(reps):
        a, b = hip.event(), hip.event()
        assert hip.l.hipEventRecord(a, stream) == 0
        assert l.moe_exl3_bw_stream_read(buf.data_ptr(), n, sink.data_ptr(), blocks, stream) == 0
        assert hip.l.hipEventRecord(b, stream) == 0
        torch.cuda.synchronize()
        best = max(best, n / (hip.ms(a, b) * 1e-3) / 1e9)
        hip.destroy(a)
        hip.destroy(b)
    del buf
    torch.cuda.empty_cache()
    print(f"[bench] streaming read {best:.0f} GB/s", file=sys.stderr, flush=True)
    return best


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(cfg, n_tokens, threads=None):
    import oracle
    import workloads as W
    threads = threads or int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    inp = W.gen_layer(cfg, experts=[])
    sample = list(range(n_tokens))
    idx, _ = oracle.route_tokens(inp, sample)
    ex = sorted(set(idx.ravel().tolist()) | ({cfg.n_experts} if cfg.shared_trellis else set()))
    codes = [W.gen_codes(cfg, p, ex, inp.ktab) for p in range(3)]
    t0 = time.perf_counter()
    oracle.layer(inp, sample, nthreads=threads, codes=codes, present=set(ex))
    dt = time.perf_counter() - t0
    return {"value": n_tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n_tokens} tokens of the {cfg.tokens}-token {cfg.name} layer "
                      f"({len(ex)} distinct experts decoded), fp64 oracle, {dt:.1f} s"}


def oracle_per_config():
    """The oracle on a bounded sample of each workload (all host threads, and
    one thread for the two small ones): tokens/s and ms per sampled layer."""
    import workloads as W
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    plan = [("tiny", 64, True), ("decode", 8, True), ("mixed_k3", 8, False), ("mixed_k4", 8, False),
            ("fp8", 8, False)]
    out = {"cpu_model": cpu_model(), "threads": threads}
    for name, n, single in plan:
        cfg = W.BY_NAME[name]
        r = cpu_baseline(cfg, n, threads)
        ent = {"tokens_per_s": r["value"], "sample": r["sample"]}
        if single:
            ent["tokens_per_s_1_thread"] = cpu_baseline(cfg, n, 1)["value"]
        out[name] = ent
        print(f"[bench] oracle {name}: {json.dumps(ent)}", file=sys.stderr, flush=True)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=50)
    ap.add_argument("--cpu-tokens", type=int, default=80)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fp8", action="store_true", help="skip the 16384-token E4M3 workload")
    ap.add_argument("--quick", action="store_true",
                    help="headline prefill and K=2 decode only (no other legs, no oracle)")
    ap.add_argument("--profile-layer", default=None, help="run this workload's layer --reps times and exit")
    ap.add_argument("--profile-flags", type=int, default=0, help="extra descriptor flags for --profile-layer")
    ap.add_argument("--copies", type=int, default=1,
                    help="--profile-layer: rotate this many copies of the codes (the decode leg uses 4)")
    ap.add_argument("--profile-tokens", type=int, default=0,
                    help="--profile-layer: this many tokens instead of the workload's own")
    ap.add_argument("--profile-graph", action="store_true",
                    help="--profile-layer: replay the layers from HIP graphs, as the verify-batch leg does")
    ap.add_argument("--reps", type=int, default=2)
    ap.add_argument("--copy-calibration", type=int, default=0, help="copy this many MiB 4 times and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: the benchmark runs the layer on one GPU only; multi-GPU scaling is not "
              "part of it", file=sys.stderr)
        sys.exit(2)

    import torch
    import trellis_quantized_moe_exl3_amd as M
    import workloads as W
    torch.cuda.set_device(0)
    hip = Hip()

    if args.copy_calibration:
        n = args.copy_calibration << 20
        a = torch.ones(n, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(4):
            b.copy_(a)
        torch.cuda.synchronize()
        print(f"[bench] copied {n} bytes 4 times", file=sys.stderr, flush=True)
        return
    if args.profile_layer:
        pcfg = W.BY_NAME[args.profile_layer]
        if args.profile_tokens > 0:
            pcfg = pcfg.replace(tokens=args.profile_tokens)
        pinp, pdesc, pweights, pkeep = setup(pcfg, copies=args.copies, extra_flags=args.profile_flags)
        px = _dev(pinp.x)
        if args.profile_graph:
            us = time_layer_graph(pdesc, pweights, px, args.reps, hip) * 1000
            print(f"[bench] replayed the {args.profile_layer} layer (T={pcfg.tokens}) {args.reps} times "
                  f"from graphs: {us:.1f} us/layer", file=sys.stderr, flush=True)
            return
        pout = torch.empty_like(px)
        pws = torch.empty(M.workspace_size(pdesc, px.shape[0]), dtype=torch.uint8, device="cuda")
        for i in range(args.reps):
            M.layer(pdesc, pweights[i % len(pweights)], px, pout, pws)
        torch.cuda.synchronize()
        print(f"[bench] ran the {args.profile_layer} layer (T={pcfg.tokens}) {args.reps} times", file=sys.stderr,
              flush=True)
        return

    # ---- prefill: the headline workload
    cfg = W.BY_NAME["prefill"]
    inp, desc, weights, keep = setup(cfg)
    x = _dev(inp.x)
    print(f"[bench] prefill inputs ready (T={cfg.tokens})", file=sys.stderr, flush=True)
    ms, per, total, _, _ = time_layer(desc, weights, x, args.steps, args.warmup, hip)
    pct = per_layer_percentiles(desc, weights, x, args.steps, hip)
    counts = routing_counts(desc, weights[0], x, cfg)
    mfma_rows = int(counts[counts > GEMV_ROWS].sum())
    step_ms = {n: float(per[:, i].mean()) for i, n in enumerate(M.STEPS)}
    gu_ms = step_ms["mfma_gateup"]
    # the gate/up launch also carries the shared expert's T rows (same H x 2I shape)
    shared_rows = cfg.tokens if (cfg.shared and cfg.tokens > SHARED_GEMV_TOKENS) else 0
    gu_flops = 2.0 * 2 * cfg.hidden * cfg.inter * (mfma_rows + shared_rows)
    achieved = gu_flops / (gu_ms * 1e-3) / 1e12
    layer_flops = expert_flops(cfg, cfg.tokens)
    print(f"[bench] prefill {ms:.3f} ms/step; steps {json.dumps({k: round(v, 4) for k, v in step_ms.items()})}",
          file=sys.stderr, flush=True)
    del keep, weights, x
    torch.cuda.empty_cache()

    # ---- decode: 8 tokens, rotating copies, K = 2 (and 3, 4)
    decode = decode_leg(W, M, hip, 2, args.decode_steps)
    extra = {}
    if not args.quick:
        extra["decode_k3"] = decode_leg(W, M, hip, 3, args.decode_steps)
        extra["decode_k4"] = decode_leg(W, M, hip, 4, args.decode_steps)
        extra["verify_batches"] = verify_batches(W, M, hip, args.decode_steps)
        # config 4: the 2048-token prefill at K = 3 and K = 4
        mixed = {"workload": "prefill-2048 at K=3 and K=4 (same seeds), router bias, fp16 shared expert"}
        for name in ("mixed_k3", "mixed_k4"):
            _, mixed[name] = prefill_leg(W, M, hip, name, min(args.steps, 10))
        extra["mixed_width"] = mixed
        # format variants
        var = {}
        _, var["per_tensor_k34"] = prefill_leg(W, M, hip, "mixed_k34", min(args.steps, 10))
        var["per_tensor_k34"]["workload"] = "prefill-2048, every tensor K3 or K4 (per-tensor widths)"
        _, var["exlr8_prefill"] = prefill_leg(W, M, hip, "exlr8_prefill", min(args.steps, 10))
        var["exlr8_prefill"]["workload"] = ("prefill-2048, K4 E4M3 codebook, rotated experts, trellis shared "
                                            "expert (exlr8 layout)")
        _, var["exlr8_prefill_fp8"] = prefill_leg(W, M, hip, "exlr8_prefill", min(args.steps, 10), M.FP8_MFMA,
                                                  "exlr8_prefill fp8")
        extra["format_variants"] = var
        extra["tile_classes"] = tile_classes(W, M, hip, min(args.steps, 10))
        extra["gemv_threshold"] = gemv_threshold_sweep(W, M, hip, min(args.steps, 10))
        # one tensor-parallel rank's share of the prefill layer (I split in two)
        _, extra["tp2_rank_prefill"] = prefill_leg(W, M, hip, "prefill_tp2", min(args.steps, 10))
        extra["tp2_rank_prefill"]["workload"] = ("prefill-7168 at I = 1024: the intermediate half that one of "
                                                 "two tensor-parallel ranks holds")
        # the 64-token correctness layer, for its latency
        tcfg = W.BY_NAME["tiny"]
        tinp, tdesc, tweights, tkeep = setup(tcfg)
        _, _, tdev, _, _ = time_layer(tdesc, tweights, _dev(tinp.x), args.decode_steps, 5, hip)
        extra["tiny"] = {"workload": "tiny: T=64, H=256, I=128, E=8, top-2, K=2", "us_per_layer": tdev * 1000}
        print(f"[bench] tiny {tdev * 1000:.1f} us/layer", file=sys.stderr, flush=True)
        del tkeep, tweights
        extra["hbm_read_GBps_achievable"] = stream_read_bandwidth(hip)

    # ---- 16384-token prefill with the E4M3 codebook: fp16 and fp8 MFMA
    fp8 = None
    if not args.no_fp8 and not args.quick:
        fp8 = {"workload": "prefill-16384: T=16384, K=4, E4M3-rounded mcg codebook, bf16 activations"}
        for name, fl in (("fp16_mfma", 0), ("fp8_mfma", M.FP8_MFMA)):
            fcfg, fp8[name] = prefill_leg(W, M, hip, "fp8", min(args.steps, 10), fl, f"fp8 workload {name}")
        # layer-level utilisation: routed flops on the fp8 peak, shared on fp16
        routed = 6.0 * fcfg.hidden * fcfg.inter * fcfg.tokens * fcfg.top_k
        shared = 6.0 * fcfg.hidden * fcfg.inter * fcfg.tokens
        t = fp8["fp8_mfma"]["ms_per_step"] * 1e-3
        fp8["fp8_mfma"]["mfma_util_mixed_peak"] = (routed / (PEAK_FP8_TFLOPS * 1e12) +
                                                   shared / (PEAK_FP16_TFLOPS * 1e12)) / t

    cpu = None
    oracle_cfgs = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, args.cpu_tokens)
        cpu["cpu_model"] = cpu_model()
        if not args.quick:
            oracle_cfgs = oracle_per_config()

    hbm = extra.get("hbm_read_GBps_achievable")
    decode["code_frac_of_achievable"] = decode["code_GBps"] / hbm if hbm else None
    rec = {
        "metric": "MoE-layer tokens/s @7168-tok prefill; us/layer @8-tok decode; code HBM GB/s",
        "value": cfg.tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16/bf16 MFMA, fp32 accumulate (K=2 trellis codes)",
        "data": "synthetic (seeded; uniform random codes, N(0,1) activations)",
        "config": {"workload": "prefill-7168: one MoE layer, T=7168, H=4096, I=2048, E=288, top-8, "
                               "K=2 mcg, router bias N(0,1), fp16 shared expert",
                   "tokens": cfg.tokens, "parallelism": "single GPU"},
        "roofline": {"kernel": "mfma_gateup (group_gemm_kernel<0,2,0>)", "bound": "mfma",
                     "achieved": achieved, "peak": PEAK_FP16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_FP16_TFLOPS, "traffic": recorded_traffic(),
                     "traffic_source": "recorded: profiles/pmc_traffic_mfma_gateup_prefill.md "
                                       "(null when the kernel sources changed since)",
                     "launch_ms": gu_ms, "flops_per_launch": gu_flops},
        "layer_mfma_util": {"expert_tflop": layer_flops / 1e12,
                            "frac_of_fp16_peak": layer_flops / (ms * 1e-3) / (PEAK_FP16_TFLOPS * 1e12)},
        "prefill_percentiles": pct,
        "step_ms": step_ms,
        "decode": decode,
        **extra,
        "e4m3_prefill": fp8,
        "cpu_baseline": cpu,
        "oracle_per_config": oracle_cfgs,
    }
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
