"""Throughput of the fused varlen / GQA attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--pass forward|backward|decode|pack|unpack] [--no-cpu-baseline]
                    [--cpu-heads N]

One step = one call of the forward entry point over the whole workload (the
complete hot path: a single fused kernel launch; the FP8 forward adds the
launch that widens V to bf16), inputs already resident in HBM, outputs
preallocated.  The default workload is the long-context packed
batch: lengths [8192, 4096, 2048, 2048] (16384 tokens), H=64, Hkv=8, D=128,
bf16, causal.

Prints ONE JSON line.  FLOPs are algorithmic: 4*D per visible (query, key)
pair per head, counted exactly from the sequence lengths and the mask.  Time
comes from HIP events recorded on the stream the kernel runs on (torch's
current stream), bracketed by device synchronisation.

``--pass decode`` times the split-KV decode entry point on the KV-cache
workload (one query per sequence against 8192 cached keys) in GB/s against
HBM; ``--pass pack|unpack`` the padded <-> packed copies.

``--pass backward`` times one backward call instead (its three kernels; O
and LSE from the GPU forward, computed once beforehand) and reports its own
metric with 2.5x the forward's FLOPs (five products per visible pair).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "varlen causal GQA attn fwd TFLOP/s on 1 MI355X; % of bf16 MFMA peak"
METRIC_BWD = "varlen causal GQA attn bwd TFLOP/s on 1 MI355X; % of bf16 MFMA peak"
HEADLINE_WORKLOAD = "varlen_bf16_long"


def metric_name(cfg: dict, bwd: bool, dtype: str) -> str:
    """The headline metric for the long-context workload; for the others the
    same form, naming their layout, mask, head grouping and peak."""
    if cfg.get("workload") == HEADLINE_WORKLOAD:
        return METRIC_BWD if bwd else METRIC
    layout = "varlen" if cfg.get("layout") == "packed varlen" else "dense"
    mask = "windowed " if cfg.get("window") else ("causal " if cfg.get("causal") else "")
    group = "GQA" if cfg.get("kv_heads", 0) < cfg.get("heads", 0) else "MHA"
    return (f"{layout} {mask}{group} attn {'bwd' if bwd else 'fwd'} TFLOP/s on 1 MI355X; "
            f"% of {dtype} MFMA peak")


METRIC_PACK = "padded <-> packed varlen copy GB/s on 1 MI355X; % of HBM peak"
METRIC_DECODE = "KV-cache decode attn fwd GB/s on 1 MI355X; % of HBM peak"
PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "fp8": 5000.0, "f32": 157.3}
HBM_PEAK_GBS = 8000.0
KERNEL_SOURCES = {
    "forward": ["variable_length_gqa_amd/csrc/attn_fwd.hip",
                "variable_length_gqa_amd/csrc/fwd_params.h",
                "variable_length_gqa_amd/csrc/kernel_common.h",
                "variable_length_gqa_amd/csrc/ticket.h",
                "variable_length_gqa_amd/csrc/pack.hip"],
    "backward": ["variable_length_gqa_amd/csrc/attn_bwd.hip",
                 "variable_length_gqa_amd/csrc/bwd_params.h",
                 "variable_length_gqa_amd/csrc/kernel_common.h"],
    "pack": ["variable_length_gqa_amd/csrc/pack.hip"],
    "unpack": ["variable_length_gqa_amd/csrc/pack.hip"],
    "decode": ["variable_length_gqa_amd/csrc/decode.hip",
               "variable_length_gqa_amd/csrc/decode_params.h",
               "variable_length_gqa_amd/csrc/kernel_common.h"],
}


def kernel_source_digest(which: str = "forward") -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[which]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, which: str = "forward"):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when it is missing or was taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    rec = t.get(workload if which == "forward" else f"{workload}:{which}")
    if not rec or rec.get("kernel_source_digest") != kernel_source_digest(which):
        return None
    return rec.get("hbm_bytes_per_launch")


def make_step(name, dev):
    import torch

    import variable_length_gqa_amd as vg
    from variable_length_gqa_amd import flops as F
    from variable_length_gqa_amd import workloads as W

    x = W.workload(name)
    if isinstance(x, W.Varlen):
        xd = x.to(dev)
        out = torch.empty_like(xd.q)
        lse = torch.empty((xd.q.shape[0], x.num_heads), dtype=torch.float32, device=dev)

        def step():
            vg.varlen_attention_fwd(xd.q, xd.k, xd.v, xd.cu_q, xd.cu_k, x.batch_size,
                                    x.num_heads, x.num_kv_heads, x.max_seqlen_q, x.max_seqlen_k,
                                    x.head_dim, x.causal, out=out, lse=lse)

        flops = F.attention_flops(x.lengths_q, x.lengths_k, x.num_heads, x.head_dim, x.causal)
        eb = x.q.element_size()
        io = F.io_bytes(sum(x.lengths_q), sum(x.lengths_k), x.num_heads, x.num_kv_heads,
                        x.head_dim, eb)
        cfg = {"workload": name, "layout": "packed varlen", "lengths": x.lengths_q,
               "total_tokens": sum(x.lengths_q), "heads": x.num_heads,
               "kv_heads": x.num_kv_heads, "head_dim": x.head_dim, "causal": x.causal}
        dt = {torch.bfloat16: "bf16", torch.float16: "f16", torch.float32: "f32"}[x.q.dtype]
        return x, step, flops, io, cfg, dt
    dd = x.to(dev)
    B, H, Sq, D = x.q.shape
    n = x.kv_seq_len if x.kv_seq_len is not None else x.k.shape[2]
    flops = F.attention_flops([Sq] * B, [n] * B, H, D, x.causal, x.window)
    if x.scales:
        out = torch.empty(dd.q.shape, dtype=torch.uint8, device=dev)
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=dev)
        o_scale = _fp8_o_scale()
        s = x.scales

        def step():
            vg.flash_attention_fwd_fp8(dd.q, dd.k, dd.v, H, x.num_kv_heads, D, x.causal,
                                       s["q_scale"], s["k_scale"], s["v_scale"], o_scale,
                                       out=out, lse=lse)
        dt, eb = "fp8", 1
    else:
        out = torch.empty_like(dd.q)
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=dev)

        def step():
            vg.flash_attention_fwd(dd.q, dd.k, dd.v, H, x.num_kv_heads, D, x.causal, x.window,
                                   x.kv_seq_len, out=out, lse=lse)
        dt = {torch.bfloat16: "bf16", torch.float16: "f16", torch.float32: "f32"}[x.q.dtype]
        eb = x.q.element_size()
    io = F.io_bytes(B * Sq, B * n, H, x.num_kv_heads, D, eb)
    cfg = {"workload": name, "layout": "dense", "batch": B, "seqlen_q": Sq, "kv_seq_len": n,
           "kv_capacity": x.k.shape[2], "heads": H, "kv_heads": x.num_kv_heads, "head_dim": D,
           "causal": x.causal, "window": x.window}
    return x, step, flops, io, cfg, dt


def make_step_bwd(name, dev):
    """One backward pass over the workload: dO seeded, O and LSE from the GPU
    forward (computed once, outside the timed region), outputs preallocated."""
    import torch

    import variable_length_gqa_amd as vg
    from variable_length_gqa_amd import flops as F
    from variable_length_gqa_amd import workloads as W

    x = W.workload(name)
    if isinstance(x, W.Varlen):
        xd = x.to(dev)
        out, lse = vg.varlen_attention_fwd(xd.q, xd.k, xd.v, xd.cu_q, xd.cu_k, x.batch_size,
                                           x.num_heads, x.num_kv_heads, x.max_seqlen_q,
                                           x.max_seqlen_k, x.head_dim, x.causal)
        dO = W.make_dout(x.q, 400).to(dev)
        dq, dk, dv = torch.empty_like(xd.q), torch.empty_like(xd.k), torch.empty_like(xd.v)
        ws = torch.empty(vg.attention.bwd_workspace_floats(xd.q.shape[0], xd.k.shape[0],
                                                            x.num_heads, x.num_kv_heads,
                                                            x.head_dim),
                         dtype=torch.float32, device=dev)

        def step():
            vg.varlen_attention_bwd(dO, xd.q, xd.k, xd.v, out, lse, xd.cu_q, xd.cu_k,
                                    x.batch_size, x.num_heads, x.num_kv_heads, x.max_seqlen_q,
                                    x.max_seqlen_k, x.head_dim, x.causal, dq=dq, dk=dk, dv=dv,
                                    workspace=ws)

        flops = 2.5 * F.attention_flops(x.lengths_q, x.lengths_k, x.num_heads, x.head_dim,
                                        x.causal)
        cfg = {"workload": name, "pass": "backward", "layout": "packed varlen",
               "lengths": x.lengths_q, "total_tokens": sum(x.lengths_q), "heads": x.num_heads,
               "kv_heads": x.num_kv_heads, "head_dim": x.head_dim, "causal": x.causal}
    elif x.scales:
        # E4M3: O (codes) and LSE from the GPU FP8 forward, dout quantised from
        # N(0,1) draws; the gradient scales only set the codes' range
        dd = x.to(dev)
        B, H, Sq, D = x.q.shape
        sc = x.scales
        o_scale = _fp8_o_scale()
        out, lse = vg.flash_attention_fwd_fp8(dd.q, dd.k, dd.v, H, x.num_kv_heads, D, x.causal,
                                              sc["q_scale"], sc["k_scale"], sc["v_scale"],
                                              o_scale)
        do8, do_scale = W.quantize_e4m3(W.make_dout(torch.empty(x.q.shape), 400))
        do8 = do8.to(dev)
        dq, dk, dv = torch.empty_like(dd.q), torch.empty_like(dd.k), torch.empty_like(dd.v)
        ws = torch.empty(vg.attention.bwd_workspace_floats(B * Sq, B * x.k.shape[2], H,
                                                            x.num_kv_heads, D, e4m3=True),
                         dtype=torch.float32, device=dev)
        gs = 1e-3

        def step():
            vg.flash_attention_bwd_fp8(do8, dd.q, dd.k, dd.v, out, lse, H, x.num_kv_heads, D,
                                       x.causal, sc["q_scale"], sc["k_scale"], sc["v_scale"],
                                       do_scale, o_scale, gs, gs, gs, dq=dq, dk=dk, dv=dv,
                                       workspace=ws)

        n = x.k.shape[2]
        flops = 2.5 * F.attention_flops([Sq] * B, [n] * B, H, D, x.causal)
        cfg = {"workload": name, "pass": "backward", "layout": "dense", "batch": B,
               "seqlen_q": Sq, "seqlen_k": n, "heads": H, "kv_heads": x.num_kv_heads,
               "head_dim": D, "causal": x.causal, "inputs": "E4M3 codes, per-tensor scales",
               "outputs": "E4M3 codes", "products": "bf16 matrix cores (exact widening)"}
        return x, step, int(flops), None, cfg, "bf16"
    else:
        if x.kv_seq_len not in (None, x.k.shape[2]):
            raise SystemExit("the backward pass runs on workloads without a kv_seq_len "
                             "shorter than the K/V buffer")
        dd = x.to(dev)
        B, H, Sq, D = x.q.shape
        out, lse = vg.flash_attention_fwd(dd.q, dd.k, dd.v, H, x.num_kv_heads, D, x.causal,
                                          x.window)
        dO = W.make_dout(x.q, 400).to(dev)
        dq, dk, dv = torch.empty_like(dd.q), torch.empty_like(dd.k), torch.empty_like(dd.v)
        ws = torch.empty(vg.attention.bwd_workspace_floats(B * Sq, B * x.k.shape[2], H,
                                                            x.num_kv_heads, D),
                         dtype=torch.float32, device=dev)

        def step():
            vg.flash_attention_bwd(dO, dd.q, dd.k, dd.v, out, lse, H, x.num_kv_heads, D,
                                   x.causal, x.window, dq=dq, dk=dk, dv=dv, workspace=ws)

        n = x.k.shape[2]
        flops = 2.5 * F.attention_flops([Sq] * B, [n] * B, H, D, x.causal, x.window)
        cfg = {"workload": name, "pass": "backward", "layout": "dense", "batch": B,
               "seqlen_q": Sq, "seqlen_k": n, "heads": H, "kv_heads": x.num_kv_heads,
               "head_dim": D, "causal": x.causal, "window": x.window}
    dt = {torch.bfloat16: "bf16", torch.float16: "f16"}[x.q.dtype]
    return x, step, int(flops), None, cfg, dt


def make_step_pack(name, dev, which):
    """Pack (padded [B, S, H, D] -> packed) or unpack of the workload's q: the
    step before / after the varlen forward.  Bytes are the algorithmic ones:
    each valid row read and written once (unpack also writes the padding)."""
    import torch

    from variable_length_gqa_amd import packing
    from variable_length_gqa_amd import workloads as W

    x = W.workload(name)
    if not isinstance(x, W.Varlen):
        raise SystemExit("pack / unpack run on the packed workloads")
    B, S = x.batch_size, x.max_seqlen_q
    padded = torch.zeros((B, S) + tuple(x.q.shape[1:]), dtype=x.q.dtype)
    cu = x.cu_q.tolist()
    for b in range(B):
        padded[b, :cu[b + 1] - cu[b]] = x.q[cu[b]:cu[b + 1]]
    padded = padded.to(dev)
    cud = x.cu_q.to(dev)
    total = cu[-1]
    packed = torch.empty((total,) + tuple(x.q.shape[1:]), dtype=x.q.dtype, device=dev)
    row = x.q[0].numel() * x.q.element_size()
    if which == "pack":
        def step():
            packing.pack(padded, cud, total=total, out=packed)
        nbytes = 2 * total * row
    else:
        packing.pack(padded, cud, total=total, out=packed)
        out = torch.empty_like(padded)

        def step():
            packing.unpack(packed, cud, S, out=out)
        nbytes = total * row + B * S * row
    cfg = {"workload": name, "pass": which, "batch": B, "max_seqlen": S,
           "total_tokens": total, "row_bytes": row}
    dt = {torch.bfloat16: "bf16", torch.float16: "f16", torch.float32: "f32"}[x.q.dtype]
    return x, step, nbytes, padded, cfg, dt


def cpu_baseline_pack(x, which, padded_dev):
    """The NumPy packing oracle on the whole workload (one process)."""
    import numpy as np

    from oracle import pack as P

    padded = padded_dev.cpu().view(torch_int16()).numpy()
    lengths = [int(n) for n in np.diff(x.cu_q.numpy())]
    t0 = time.perf_counter()
    packed = P.pack(padded, lengths)
    if which == "unpack":
        t0 = time.perf_counter()
        P.unpack(packed, x.cu_q.numpy(), padded.shape[1])
    secs = time.perf_counter() - t0
    row = padded[0, 0].nbytes
    nbytes = 2 * packed.shape[0] * row if which == "pack" else \
        packed.shape[0] * row + padded.shape[0] * padded.shape[1] * row
    return {"value": nbytes / secs / 1e9, "unit": "GB/s", "cores": 1, "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": f"the whole workload's q ({nbytes / 1e6:.0f} MB moved, {secs:.2f} s, "
                      f"NumPy, one thread)"}


def torch_int16():
    import torch

    return torch.int16


def cpu_baseline_bwd(name, x, n_heads, unit_scale):
    """The f64 backward oracle on the first ``n_heads`` query heads (a bounded
    sample of the same workload), all worker processes."""
    import oracle
    from oracle.attention import default_workers
    from variable_length_gqa_amd import flops as F
    from variable_length_gqa_amd import workloads as W

    workers = default_workers()
    heads = list(range(n_heads))
    dO = W.make_dout(x.q, 400)
    t0 = time.perf_counter()
    if isinstance(x, W.Varlen):
        oracle.varlen_attention_bwd(dO, x.q, x.k, x.v, x.cu_q, x.cu_k, x.num_heads,
                                    x.num_kv_heads, x.causal, workers=workers, heads=heads)
        fl = 2.5 * F.attention_flops(x.lengths_q, x.lengths_k, n_heads, x.head_dim, x.causal)
    elif x.scales:
        import torch

        B, H, Sq, D = x.q.shape
        sc = x.scales
        do8, do_scale = W.quantize_e4m3(W.make_dout(torch.empty(x.q.shape), 400))
        # the work does not depend on the stored output's values: q's codes
        # stand in for them
        # (first batch entry only: the f64 oracle needs ~4 s per head of it)
        oracle.flash_attention_bwd_fp8(do8[:1], x.q[:1], x.k[:1], x.v[:1], x.q[:1], H,
                                       x.num_kv_heads, x.causal, sc["q_scale"], sc["k_scale"],
                                       sc["v_scale"], do_scale, sc["v_scale"], 1.0, 1.0, 1.0,
                                       workers=workers, heads=heads)
        fl = 2.5 * F.attention_flops([Sq], [x.k.shape[2]], n_heads, D, x.causal)
    else:
        B, H, Sq, D = x.q.shape
        oracle.flash_attention_bwd(dO, x.q, x.k, x.v, H, x.num_kv_heads, x.causal, x.window,
                                   workers=workers, heads=heads)
        fl = 2.5 * F.attention_flops([Sq] * B, [x.k.shape[2]] * B, n_heads, D, x.causal,
                                     x.window)
    secs = time.perf_counter() - t0
    which = "of batch entry 0" if x.scales else "of every sequence"
    return secs, {"value": fl / secs / unit_scale, "unit": "TFLOP/s", "cores": workers,
                  "cpu_model": cpu_model(), "kind": "oracle",
                  "sample": f"backward of query heads 0..{n_heads - 1} of {x.num_heads} {which} "
                            f"({fl:.3e} algorithmic FLOPs, {secs:.1f} s wall, f64 "
                            f"NumPy, one process per core, masked scores computed too)"}


def cpu_model() -> str:
    """The host CPU's model name from /proc/cpuinfo, with its family / model /
    stepping numbers (a virtualised host may report only a generic name), or
    the platform's processor string."""
    info = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if not line.strip():
                    break  # the first processor's block
                k, _, v = line.partition(":")
                info.setdefault(k.strip().lower(), v.strip())
    except OSError:
        pass
    if "model name" in info:
        ids = [f"{k} {info[k]}" for k in ("cpu family", "model", "stepping") if k in info]
        return info["model name"] + (f" ({', '.join(ids)})" if ids else "")
    import platform

    return platform.processor() or "unknown"


def _fp8_o_scale():
    with open(os.path.join(ROOT, "tests", "golden", "fp8_o_scale.json")) as f:
        return json.load(f)["o_scale"]


def cpu_baseline(name, x, n_heads, unit_scale):
    """The f64 oracle, as it stands, on a bounded sample of the same workload:
    the first ``n_heads`` query heads of every sequence, all worker processes."""
    import oracle
    from oracle.attention import default_workers
    from variable_length_gqa_amd import flops as F
    from variable_length_gqa_amd import workloads as W

    workers = default_workers()
    heads = list(range(n_heads))
    t0 = time.perf_counter()
    if isinstance(x, W.Varlen):
        oracle.varlen_attention_fwd(x.q, x.k, x.v, x.cu_q, x.cu_k, x.num_heads, x.num_kv_heads,
                                    x.causal, workers=workers, heads=heads)
        fl = F.attention_flops(x.lengths_q, x.lengths_k, n_heads, x.head_dim, x.causal)
    else:
        B, H, Sq, D = x.q.shape
        n = x.kv_seq_len if x.kv_seq_len is not None else x.k.shape[2]
        if x.scales:
            s = x.scales
            oracle.flash_attention_fwd_fp8(x.q, x.k, x.v, H, x.num_kv_heads, x.causal,
                                           s["q_scale"], s["k_scale"], s["v_scale"], 1.0,
                                           workers=workers, heads=heads)
        else:
            oracle.flash_attention_fwd(x.q, x.k, x.v, H, x.num_kv_heads, x.causal, x.window,
                                       x.kv_seq_len, workers=workers, heads=heads)
        fl = F.attention_flops([Sq] * B, [n] * B, n_heads, D, x.causal, x.window)
    secs = time.perf_counter() - t0
    return secs, {"value": fl / secs / unit_scale, "unit": "TFLOP/s", "cores": workers,
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"query heads 0..{n_heads - 1} of {x.num_heads} of every sequence "
                      f"({fl:.3e} algorithmic FLOPs, {secs:.1f} s wall, f64 NumPy, "
                      f"one process per core, masked scores computed too)"}


# the other forward workloads timed beside the headline one (every config the
# metric's target names: f32 MHA, the 16-sequence GQA mix, the dense window
# over a capacity buffer, FP8)
OTHER_FORWARD_WORKLOADS = ("varlen_f32_mha", "varlen_bf16_gqa", "dense_bf16_window", "dense_fp8")


def W_workload(name):
    from variable_length_gqa_amd import workloads as W

    return W.workload(name)


SETTLE = {"steps": 0, "ms": 0.0}


def settle(torch, step, settle_ms):
    """Untimed steps until the GPU has run the step for about ``settle_ms`` of
    wall time: from idle its clocks take some 50-100 ms of sustained load to
    reach their steady state (measured: the long-context forward runs 1.57 ms
    per step in its first five launches, 1.355 in the next twenty, 1.32 after
    ~60 ms), which a few warm-up steps do not cover.  Recorded in the JSON line
    ("settle") beside the W warm-up steps."""
    n, t0 = 0, time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < settle_ms:
        for _ in range(4):
            step()
        n += 4
        torch.cuda.synchronize()
    SETTLE["steps"] += n
    SETTLE["ms"] += (time.perf_counter() - t0) * 1e3
    return n


def time_steps(torch, step, steps, warmup, dev, settle_ms=150.0):
    """Clock settle (untimed), W untimed warm-up steps, then K steps between HIP
    events recorded on torch's current stream (the stream every entry point
    launches on), bracketed by device synchronisation.  Returns (ms per step,
    wall s)."""
    if settle_ms > 0:
        settle(torch, step, settle_ms)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / steps, time.perf_counter() - t0


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--settle-ms", type=float, default=150.0,
                    help="untimed steps for about this long before the warm-up steps, so "
                         "the GPU clocks reach their steady state under load (0: none)")
    ap.add_argument("--no-workloads", action="store_true",
                    help="time only the named workload (by default the long-context forward "
                         "run also times the other forward workloads)")
    ap.add_argument("--cpu-heads", type=int, default=0,
                    help="query heads in the CPU-baseline sample (0: sized to ~15 s)")
    ap.add_argument("--pass", dest="which",
                    choices=("forward", "backward", "pack", "unpack", "decode"),
                    default="forward",
                    help="the forward (the headline metric), the backward pass, the "
                         "padded <-> packed copies, or the split-KV decode path")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the forward shards across GPUs by heads or by "
              "sequences with no exchange; the benchmark runs on and reports one GPU.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(max(1, args.steps)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n,
                          "launches": max(1, args.steps)}), flush=True)
        return
    bwd = args.which == "backward"
    if args.which in ("pack", "unpack"):
        return bench_pack(args, dev)
    if args.which == "decode":
        return bench_decode(args, dev)
    x, step, flops, io, cfg, dt = (make_step_bwd if bwd else make_step)(args.workload, dev)
    ms, wall = time_steps(torch, step, args.steps, args.warmup, dev, args.settle_ms)
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[dt]
    traffic = measured_traffic(args.workload, args.which)

    res = {
        "metric": metric_name(cfg, bwd, dt), "value": round(tflops, 2), "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dt,
        "data": "synthetic (seeded N(0,1) inputs of the workload's shapes)",
        "config": cfg,
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(tflops / peak, 4), "traffic": traffic},
        "flops_per_step": flops, "wall_s_timed": round(wall, 3),
        "settle": {"steps": SETTLE["steps"], "ms": round(SETTLE["ms"], 1),
                   "note": "untimed steps before the warm-up ones, for steady GPU clocks"},
        "kernel_source_digest": kernel_source_digest(args.which),
    }
    if io is not None:
        res["io_bytes_per_step"] = io
        res["io_gbs"] = round(io / (ms * 1e-3) / 1e9, 1)
    if not bwd and not args.no_workloads and args.workload == "varlen_bf16_long":
        # the other forward workloads, each timed exactly as the headline one
        # (its own W warm-up steps, then K timed steps on the kernel's stream)
        del x, step
        torch.cuda.empty_cache()
        res["workloads"] = {}
        for name in OTHER_FORWARD_WORKLOADS:
            xo, so, fo, _, co, do = make_step(name, dev)
            mso, _ = time_steps(torch, so, args.steps, args.warmup, dev, args.settle_ms)
            tf = fo / (mso * 1e-3) / 1e12
            pk = PEAK_TFLOPS[do]
            res["workloads"][name] = {
                "ms_per_step": round(mso, 4), "tflops": round(tf, 2), "dtype": do,
                "peak_tflops": pk, "frac": round(tf / pk, 4), "flops_per_step": fo,
                "traffic": measured_traffic(name, "forward"), "config": co}
            del xo, so
            torch.cuda.empty_cache()
        x = W_workload(args.workload)
    if not args.no_cpu_baseline:
        base = cpu_baseline_bwd if bwd else cpu_baseline
        n_heads = args.cpu_heads
        if n_heads <= 0:
            # size the sample to about 15 s: time one head group, then scale up
            G = x.num_heads // x.num_kv_heads
            secs, _ = base(args.workload, x, min(G, x.num_heads), 1e12)
            n_heads = int(min(x.num_heads, max(G, G * round(15.0 / max(secs, 1e-3)))))
        _, res["cpu_baseline"] = base(args.workload, x, min(n_heads, x.num_heads), 1e12)
    print(json.dumps(res), flush=True)


def bench_pack(args, dev):
    import torch

    x, step, nbytes, padded, cfg, dt = make_step_pack(args.workload, dev, args.which)
    ms, _ = time_steps(torch, step, args.steps, args.warmup, dev, args.settle_ms)
    gbs = nbytes / (ms * 1e-3) / 1e9
    stream = torch.cuda.current_stream(dev)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    # reference: a plain device-to-device copy moving the same bytes (half read, half written)
    src = torch.empty(nbytes // 2, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    ev0.record(stream)
    for _ in range(args.steps):
        dst.copy_(src)
    ev1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = nbytes / (ev0.elapsed_time(ev1) / args.steps * 1e-3) / 1e9
    del src, dst
    res = {
        "metric": METRIC_PACK, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dt,
        "data": "synthetic (seeded N(0,1) inputs of the workload's shapes)", "config": cfg,
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(args.workload, args.which)},
        "bytes_per_step": nbytes, "copy_reference_gbs": round(copy_gbs, 1),
        "settle": {"steps": SETTLE["steps"], "ms": round(SETTLE["ms"], 1)},
        "kernel_source_digest": kernel_source_digest("pack"),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_pack(x, args.which, padded)
    print(json.dumps(res), flush=True)


def decode_bytes(x):
    """Algorithmic HBM bytes of one decode call: every visible K and V row of
    each (batch, kv head) read once, q read and out written once, lse written."""
    from variable_length_gqa_amd import flops as F

    B, H, Sq, D = x.q.shape
    n = x.kv_seq_len if x.kv_seq_len is not None else x.k.shape[2]
    eb = x.q.element_size()
    keys = F.visible_key_span(Sq, n, x.causal, x.window)
    return 2 * B * x.num_kv_heads * keys * D * eb + 2 * B * H * Sq * D * eb + B * H * Sq * 4


def cpu_baseline_decode(x):
    """The f64 dense-forward oracle on the whole decode workload, all worker
    processes, reported in the GPU metric's unit (the workload's algorithmic
    bytes over the oracle's wall time)."""
    import oracle
    from oracle.attention import default_workers

    workers = default_workers()
    t0 = time.perf_counter()
    oracle.flash_attention_fwd(x.q, x.k, x.v, x.num_heads, x.num_kv_heads, x.causal, x.window,
                               x.kv_seq_len, workers=workers)
    secs = time.perf_counter() - t0
    nb = decode_bytes(x)
    return {"value": nb / secs / 1e9, "unit": "GB/s", "cores": workers, "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": f"the whole workload ({nb / 1e6:.0f} MB of algorithmic traffic, "
                      f"{secs:.1f} s wall, f64 NumPy, one process per core)"}


def bench_decode(args, dev):
    import torch

    import variable_length_gqa_amd as vg
    from variable_length_gqa_amd import flops as F
    from variable_length_gqa_amd import workloads as W

    name = args.workload if args.workload != "varlen_bf16_long" else "dense_bf16_decode"
    x = W.workload(name)
    if not isinstance(x, W.Dense) or x.scales:
        raise SystemExit("--pass decode runs on a dense 16-bit workload")
    dd = x.to(dev)
    B, H, Sq, D = x.q.shape
    cap = x.k.shape[2]
    n = x.kv_seq_len if x.kv_seq_len is not None else cap
    out = torch.empty_like(dd.q)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=dev)
    ws = torch.empty(vg.decode_workspace_floats(B, x.num_kv_heads, D, cap), dtype=torch.float32,
                     device=dev)

    def step():
        vg.flash_attention_decode(dd.q, dd.k, dd.v, H, x.num_kv_heads, D, x.causal, x.window,
                                  x.kv_seq_len, out=out, lse=lse, workspace=ws)

    ms, wall = time_steps(torch, step, args.steps, args.warmup, dev, args.settle_ms)
    nb = decode_bytes(x)
    gbs = nb / (ms * 1e-3) / 1e9
    flops = F.attention_flops([Sq] * B, [n] * B, H, D, x.causal, x.window)
    dt = {torch.bfloat16: "bf16", torch.float16: "f16"}[x.q.dtype]
    cfg = {"workload": name, "layout": "dense", "batch": B, "seqlen_q": Sq, "kv_seq_len": n,
           "kv_capacity": cap, "heads": H, "kv_heads": x.num_kv_heads, "head_dim": D,
           "causal": x.causal, "window": x.window}
    res = {
        "metric": METRIC_DECODE, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dt,
        "data": "synthetic (seeded N(0,1) inputs of the workload's shapes)", "config": cfg,
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(name, "decode")},
        "bytes_per_step": nb, "tflops": round(flops / (ms * 1e-3) / 1e12, 3),
        "wall_s_timed": round(wall, 3),
        "settle": {"steps": SETTLE["steps"], "ms": round(SETTLE["ms"], 1)},
        "kernel_source_digest": kernel_source_digest("decode"),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_decode(x)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
