"""Benchmark of the BSA forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config ns128] [--no-cpu-baseline]

One step = one mosaic_bsa_forward call (pool -> compressed + top-n selection
-> fused selected/local fine attention with the gated sum) over one batch of
synthetic HEALPix-NESTED fields already resident in HBM.  The default
workload is Nside = 128 (24 ensemble members x 8 heads x head_dim 64, block
64, top-n 16, window 512); the Nside = 256 workload (2 x 16 heads, block 256,
top-n 8, window 1024) is measured in the same run and reported under
"secondary".  The training forward (mosaic_bsa_forward_train) and the
backward from its saved state (mosaic_bsa_backward, float32 upstream
gradient), and the backward that recomputes that state, are timed after each
forward and reported under "backward"; they are not part of the step.  So is
a stack of encoder layers on the primary workload (512 channels, 4 layers,
synthetic weights: input projection, BSA, output projection with the
residual, plus one level of HEALPix coarsening of its input), reported
under "encoder_layer", and the lat-lon -> HEALPix interpolation (0.25-degree
grid onto Nside 256), reported under "interpolation".  Prints one JSON line.

Roofline of the dominant kernel (the fine-attention kernel, bf16 MFMA):
algorithmic FLOPs per launch = sum over queries of 4*d*(n*block + |window(t)|)
(edge windows clipped), divided by the kernel's mean duration measured with
HIP events on the stream it runs on.  The oracle (float64 numpy) is timed on
host cores on a bounded sample of (batch, head) slices of the same inputs.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from spherical_block_sparse_amd import CONFIGS, BSAConfig, make_inputs  # noqa: E402
from spherical_block_sparse_amd import _lib  # noqa: E402

TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")
DURATION_JSON = os.path.join(ROOT, "profiles", "kernel_durations.json")

PEAK_BF16_TFLOPS = 2500.0
PEAK_FP64_TFLOPS = 78.6
PEAK_HBM_GBS = 8000.0


def window_keys_total(n_tok: int, window: int) -> int:
    t = np.arange(n_tok, dtype=np.int64)
    lo = np.maximum(t - window // 2, 0)
    hi = np.minimum(t + (window + 1) // 2, n_tok)
    return int((hi - lo).sum())


def fine_flops(cfg: BSAConfig) -> float:
    """Algorithmic FLOPs of one fine-kernel launch: QK^T and PV of both branches."""
    d = cfg.head_dim
    per_slice = 4 * d * (cfg.n_tokens * cfg.topn * cfg.block + window_keys_total(cfg.n_tokens, cfg.window))
    return float(per_slice) * cfg.slices


def backward_flops(cfg: BSAConfig) -> float:
    """Algorithmic FLOPs of the backward's fine branches: per (query, key) pair
    of the selected and local sets, five products of 2*d FLOPs (S = QK^T
    recomputed, dP = dO V^T, dV += P^T dO, dQ += dS K, dK += dS^T Q), i.e.
    2.5x the forward's two; the pooled branch's m^2 share is left out."""
    return 2.5 * fine_flops(cfg)


def compress_flops(cfg: BSAConfig) -> float:
    m, d = cfg.n_blocks, cfg.head_dim
    return 4.0 * m * m * d * cfg.slices          # logits + ā·v̄


def compress_bound_ms(cfg: BSAConfig) -> float:
    """Matrix-core time of one compress+select launch at the published peaks, in the
    precision the forward computes it: for top-n <= 16 the logits as three bf16 piece
    products (3 * 2*m^2*d bf16 FLOPs) and ā·v̄ (2*m^2*d bf16) per slice; above that,
    float64 logits plus bf16 ā·v̄."""
    half = 2.0 * cfg.n_blocks ** 2 * cfg.head_dim * cfg.slices
    if cfg.topn <= 16:
        return 4.0 * half / (PEAK_BF16_TFLOPS * 1e12) * 1e3
    return (half / (PEAK_FP64_TFLOPS * 1e12) + half / (PEAK_BF16_TFLOPS * 1e12)) * 1e3


def pool_bytes(cfg: BSAConfig) -> float:
    """q, k, v read once; q̄, k̄ (float64), v̄ (float32), k̄'s two bf16 pieces, and the
    per-block key norm and |k̄|^2 (float32) written."""
    e_in = cfg.slices * cfg.n_tokens * cfg.head_dim
    e_out = cfg.slices * cfg.n_blocks * cfg.head_dim
    return 3.0 * e_in * 2 + e_out * (8 + 8 + 4 + 4) + cfg.slices * cfg.n_blocks * 8


def measured_traffic(key: str):
    """HBM bytes per launch of a kernel from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE passes (copy-calibrated), or None when they are
    missing or the kernel source has changed since they were taken."""
    import hashlib
    try:
        rec = json.load(open(TRAFFIC_JSON))[key]
        src = os.path.join(ROOT, rec["source"])
        if hashlib.sha256(open(src, "rb").read()).hexdigest() != rec["source_sha256"]:
            return None
        return rec["hbm_bytes"]
    except (OSError, KeyError, ValueError):
        return None


def profiled_ms(key: str):
    """Mean duration (ms) of a kernel in the committed rocprofv3 kernel trace of
    the bench command, or None when it is missing or the kernel source has
    changed since it was taken."""
    import hashlib
    try:
        rec = json.load(open(DURATION_JSON))[key]
        src = os.path.join(ROOT, rec["source"])
        if hashlib.sha256(open(src, "rb").read()).hexdigest() != rec["source_sha256"]:
            return None
        return rec["avg_ms"]
    except (OSError, KeyError, ValueError):
        return None


def time_stream(fn, steps: int) -> float:
    """Mean milliseconds of fn() over `steps` calls, HIP events on the current stream."""
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        fn()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps


def time_steps(fn, steps: int) -> tuple:
    """Mean milliseconds of fn() over `steps` calls, as time_stream, plus each
    call's own duration: an event is recorded between consecutive calls on the
    same stream (no synchronisation inside the timed region)."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(steps):
        fn()
        ev[i + 1].record()
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    return ev[0].elapsed_time(ev[steps]) / steps, per


def host_cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def measure(cfg: BSAConfig, steps: int, warmup: int, backward: bool = True) -> dict:
    print(f"[bench] {cfg.name}: generating inputs", file=sys.stderr, flush=True)
    q, k, v, g = make_inputs(cfg, device="cuda", dtype=torch.bfloat16)
    b, h, n, d = cfg.batch, cfg.heads, cfg.n_tokens, cfg.head_dim
    m = cfg.n_blocks
    dev = q.device
    out = torch.empty((b, h, n, d), dtype=torch.float32, device=dev)
    sel = torch.empty((b, h, m, cfg.topn), dtype=torch.int32, device=dev)
    ws = torch.empty(_lib.mosaic_bsa_workspace_bytes(b, h, d, cfg.nside, cfg.block, cfg.topn),
                     dtype=torch.uint8, device=dev)
    fwd = lambda: _lib.mosaic_bsa_forward(q, k, v, g, cfg.nside, cfg.block, cfg.topn, cfg.window,
                                          out=out, sel_idx=sel, workspace=ws)
    print(f"[bench] {cfg.name}: warmup {warmup}", file=sys.stderr, flush=True)
    for _ in range(warmup):
        fwd()
    torch.cuda.synchronize()
    print(f"[bench] {cfg.name}: timing {steps} steps", file=sys.stderr, flush=True)
    ms, per_step = time_steps(fwd, steps)

    # per-kernel durations through the stage entry points (same kernels)
    qbar = torch.empty((b, h, m, d), dtype=torch.float64, device=dev)
    kbar = torch.empty_like(qbar)
    vbar = torch.empty((b, h, m, d), dtype=torch.float32, device=dev)
    o_cg = torch.empty_like(vbar)
    knorm = torch.empty((b, h, m), dtype=torch.float32, device=dev)
    kpieces = torch.empty((b, h, m, 2, d), dtype=torch.bfloat16, device=dev)
    kbn2 = torch.empty((b, h, m), dtype=torch.float32, device=dev)
    sel2 = torch.empty_like(sel)
    out2 = torch.empty_like(out)
    pool = lambda: _lib.mosaic_bsa_pool(q, k, v, cfg.nside, cfg.block, qbar, kbar, vbar, knorm=knorm,
                                        kpieces=kpieces, kbn2=kbn2)
    cs = lambda: _lib.mosaic_bsa_compress_select(qbar, kbar, vbar, cfg.nside, cfg.block, cfg.topn, o_cg, sel2,
                                                 kpieces=kpieces, kbn2=kbn2)
    sb = torch.empty((cfg.batch, cfg.heads, cfg.n_blocks), dtype=torch.float32, device=dev)
    bound = lambda: _lib.mosaic_bsa_select_bound(sel2, knorm, cfg.nside, cfg.block, cfg.topn, cfg.head_dim, sb)
    fine = lambda: _lib.mosaic_bsa_fine(q, k, v, g, o_cg, sel2, cfg.nside, cfg.block, cfg.topn, cfg.window, out2,
                                        knorm=knorm, sel_bound=sb)
    pool(); cs(); bound(); fine()
    kt = max(3, steps // 2)
    pool_ms = time_stream(pool, kt)
    cs_ms = time_stream(cs, kt)
    bound_ms = time_stream(bound, kt)
    fine_ms = time_stream(fine, kt)
    torch.cuda.synchronize()
    same = bool(torch.equal(sel, sel2) and torch.equal(out, out2))

    ff = fine_flops(cfg)
    bwd = None
    if backward:
        gen = torch.Generator(device=dev).manual_seed(cfg.seed + 7)
        dout = torch.randn((b, h, n, d), generator=gen, device=dev, dtype=torch.float32)
        grads = [torch.empty((b, h, n, d), dtype=torch.float32, device=dev) for _ in range(3)]
        dgates = torch.empty((b, h, n, 3), dtype=torch.float32, device=dev)
        bws = torch.empty(_lib.mosaic_bsa_backward_workspace_bytes(b, h, d, cfg.nside, cfg.block, cfg.topn),
                          dtype=torch.uint8, device=dev)
        saved = torch.empty(_lib.mosaic_bsa_saved_bytes(b, h, d, cfg.nside, cfg.block), dtype=torch.uint8,
                            device=dev)
        out_t, sel_t = torch.empty_like(out), torch.empty_like(sel)
        fwd_t = lambda: _lib.mosaic_bsa_forward_train(q, k, v, g, cfg.nside, cfg.block, cfg.topn, cfg.window,
                                                      out=out_t, sel_idx=sel_t, saved=saved)
        print(f"[bench] {cfg.name}: training forward + backward", file=sys.stderr, flush=True)
        fwd_t()
        kb = max(3, steps // 4)
        fwd_t_ms = time_stream(fwd_t, kb)
        bw = lambda: _lib.mosaic_bsa_backward(q, k, v, g, sel_t, dout, cfg.nside, cfg.block, cfg.topn, cfg.window,
                                              *grads, dgates, workspace=bws, saved=saved)
        bw_r = lambda: _lib.mosaic_bsa_backward(q, k, v, g, sel_t, dout, cfg.nside, cfg.block, cfg.topn,
                                                cfg.window, *grads, dgates, workspace=bws)
        bw()
        bwd_ms = time_stream(bw, kb)
        bw_r()
        bwd_r_ms = time_stream(bw_r, kb)
        bf = backward_flops(cfg)
        bwd = {"ms": bwd_ms, "tokens_per_s": cfg.tokens / (bwd_ms * 1e-3), "algorithmic_flops": bf,
               "achieved_TFLOPs": bf / (bwd_ms * 1e-3) / 1e12,
               "frac_bf16_peak": bf / (bwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
               "from": "mosaic_bsa_forward_train state",
               "training_forward_ms": fwd_t_ms, "recompute_ms": bwd_r_ms,
               "training_step_tokens_per_s": cfg.tokens / ((fwd_t_ms + bwd_ms) * 1e-3),
               "traffic": {"dq": measured_traffic(f"dq_{cfg.name}"), "dkdv": measured_traffic(f"dkdv_{cfg.name}")}}
        del dout, grads, dgates, bws, saved, out_t, sel_t
    res = dict(backward=bwd,
        cfg=cfg, ms=ms, tokens_per_s=cfg.tokens / (ms * 1e-3),
        step_ms={"median": float(np.median(per_step)), "min": min(per_step), "max": max(per_step)},
        pool_ms=pool_ms, cs_ms=cs_ms, bound_ms=bound_ms, fine_ms=fine_ms, stages_match_forward=same,
        fine_tflops=ff / (fine_ms * 1e-3) / 1e12, fine_flops=ff,
        pool_gbs=pool_bytes(cfg) / (pool_ms * 1e-3) / 1e9, pool_bytes=pool_bytes(cfg),
        cs_tflops=compress_flops(cfg) / (cs_ms * 1e-3) / 1e12,
        inputs=(q, k, v, g, sel),
    )
    return res


def measure_layer(cfg: BSAConfig, channels: int, layers: int, steps: int) -> dict:
    """A stack of encoder layers (input projection, BSA, output projection with
    the residual) on the workload's mesh with synthetic weights: ms per layer,
    and each projection GEMM timed through its stage entry point."""
    from spherical_block_sparse_amd import make_layer_inputs
    print(f"[bench] {cfg.name}: encoder layers ({layers} x {channels} channels)", file=sys.stderr, flush=True)
    x, w_in, w_out = make_layer_inputs(cfg, channels, layers, device="cuda")
    b, n, h, d = cfg.batch, cfg.n_tokens, cfg.heads, cfg.head_dim
    ws = torch.empty(_lib.mosaic_bsa_layer_workspace_bytes(b, h, d, channels, cfg.nside, cfg.block, cfg.topn),
                     dtype=torch.uint8, device="cuda")
    ys = [torch.empty_like(x), torch.empty_like(x)]
    sel = torch.empty((b, h, cfg.n_blocks, cfg.topn), dtype=torch.int32, device="cuda")

    def stack():
        cur = x
        for li in range(layers):
            nxt = ys[li % 2]
            _lib.mosaic_bsa_layer_forward(cur, w_in[li], w_out[li], h, d, cfg.nside, cfg.block, cfg.topn,
                                          cfg.window, y=nxt, sel_idx=sel, workspace=ws)
            cur = nxt
    stack()
    ms = time_stream(stack, max(2, steps // 5)) / layers
    q, k, v, g = _lib.mosaic_bsa_layer_in(x, w_in[0], h, d, cfg.nside)
    attn = torch.randn((b, h, n, d), device="cuda", dtype=torch.float32)
    lin = lambda: _lib.mosaic_bsa_layer_in(x, w_in[0], h, d, cfg.nside, q, k, v, g)
    lout = lambda: _lib.mosaic_bsa_layer_out(attn, w_out[0], x, cfg.nside, ys[0])
    merged = attn.to(torch.bfloat16).permute(0, 2, 1, 3).contiguous().view(b, n, h * d)
    lmerged = lambda: _lib.mosaic_bsa_layer_out_merged(merged, w_out[0], x, cfg.nside, h, ys[0])
    in_ms, out_ms, merged_ms = time_stream(lin, 5), time_stream(lout, 5), time_stream(lmerged, 5)
    # HEALPix coarsening of the layer input by one level (Nside 128 -> 64)
    xc = _lib.mosaic_healpix_coarsen(x, cfg.nside, 1)
    co = lambda: _lib.mosaic_healpix_coarsen(x, cfg.nside, 1, y=xc)
    co_ms = time_stream(co, 5)
    co_bytes = float(x.numel() * 2 + xc.numel() * 4)
    del xc
    m_tok = b * n
    in_fl = 2.0 * m_tok * channels * (3 * h * d + 3 * h)
    out_fl = 2.0 * m_tok * (h * d) * channels
    del x, w_in, w_out, ws, ys, q, k, v, g, attn, merged
    return {"channels": channels, "layers": layers, "ms_per_layer": ms,
            "tokens_per_s_per_layer": cfg.tokens / (ms * 1e-3),
            "in_proj": {"ms": in_ms, "TFLOPs": in_fl / (in_ms * 1e-3) / 1e12,
                        "frac_bf16_peak": in_fl / (in_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS},
            # the output projection the layer runs: attention output merged in bf16
            # [b][N][H*d], as the layer's fine kernel writes it
            "out_proj": {"ms": merged_ms, "TFLOPs": out_fl / (merged_ms * 1e-3) / 1e12,
                         "frac_bf16_peak": out_fl / (merged_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS},
            # the float32 stage entry point: takes the attention output in float32
            # [b][H][N][d] and rounds it while staging through registers
            "out_proj_from_f32": {"ms": out_ms, "TFLOPs": out_fl / (out_ms * 1e-3) / 1e12,
                                  "frac_bf16_peak": out_fl / (out_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS},
            "weights": "synthetic N(0, 1/fan_in), bf16",
            "coarsen_1_level": {"ms": co_ms, "bytes": co_bytes, "GBs": co_bytes / (co_ms * 1e-3) / 1e9,
                                "frac_hbm_peak": co_bytes / (co_ms * 1e-3) / 1e9 / PEAK_HBM_GBS}}


def measure_ceilings() -> dict:
    """Measured ceilings of this GPU beside the published peaks, from the
    probes of libmosaic_probe.so: a streaming read of a 4 GiB buffer (the
    pooling kernel's access pattern without its arithmetic) and back-to-back
    bf16 MFMAs on register operands; plus the runtime's device copy of the
    same buffer (bytes read + written)."""
    from spherical_block_sparse_amd import probe
    print("[bench] measured ceilings", file=sys.stderr, flush=True)
    props = torch.cuda.get_device_properties(0)
    cus = props.multi_processor_count
    n = 1 << 30   # float32 elements: 4 GiB
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    sink = torch.zeros(8 * cus * 64, dtype=torch.float32, device="cuda")
    rblocks = 8 * cus * 8
    read_ms = time_stream(lambda: probe.probe_read(src, sink, rblocks), 10)
    dst = torch.empty_like(src)
    copy_ms = time_stream(lambda: dst.copy_(src), 10)
    del src, dst
    mblocks, iters = 2 * cus * 4, 4096
    flops = probe.probe_mfma(sink, mblocks, iters)
    mfma_ms = time_stream(lambda: probe.probe_mfma(sink, mblocks, iters), 10)
    clk = torch.zeros((mblocks, 2), dtype=torch.int64, device="cuda")
    probe.probe_mfma(sink, mblocks, iters, clk)
    c = clk.double().sum(0).cpu()
    mfma_ghz = float(c[0] / c[1]) * 0.1   # shader clocks per 100 MHz tick
    torch.cuda.empty_cache()
    nbytes = 4.0 * n
    return {"read_GBs": nbytes / (read_ms * 1e-3) / 1e9, "copy_GBs": 2 * nbytes / (copy_ms * 1e-3) / 1e9,
            "bf16_mfma_TFLOPs": flops / (mfma_ms * 1e-3) / 1e12, "mfma_probe_clock_GHz": mfma_ghz,
            "bf16_mfma_TFLOPs_per_GHz": flops / (mfma_ms * 1e-3) / 1e12 / mfma_ghz,
            "published": {"hbm_GBs": PEAK_HBM_GBS, "bf16_TFLOPs": PEAK_BF16_TFLOPS},
            "how": (f"mosaic_probe_read over 4 GiB ({rblocks} workgroups), the runtime's 4 GiB device copy "
                    f"(read + written bytes), mosaic_probe_mfma ({mblocks} workgroups x 4 waves x {iters} x 8 "
                    f"v_mfma_f32_16x16x32_bf16)")}


def measure_interp(steps: int) -> dict:
    """The lat-lon -> HEALPix interpolation: the 0.25-degree grid (721 x 1440)
    onto Nside 256 for 2 members x 16 heads (d = dv = 64, a 4 x 4 stencil)."""
    from spherical_block_sparse_amd.synth import make_interp_inputs
    print("[bench] interpolation 721x1440 -> Nside 256, 32 slices", file=sys.stderr, flush=True)
    s_, n_lat, n_lon, nside = 32, 721, 1440, 256
    k, v, w_q, nbr, rel = make_interp_inputs(nside, n_lat, n_lon, s_, device="cuda", seed=nside)
    out = _lib.mosaic_interp_attention(k, v, w_q, nbr, rel)
    ws = torch.empty(_lib.mosaic_interp_workspace_bytes(s_, n_lat * n_lon), dtype=torch.uint8, device="cuda")
    fn = lambda: _lib.mosaic_interp_attention(k, v, w_q, nbr, rel, out=out, workspace=ws)
    ms = time_stream(fn, max(3, steps // 2))
    n_src, n_dst, kk = n_lat * n_lon, nbr.shape[0], nbr.shape[1]
    # each source row once (k, v), the stencil once, each output once
    byts = float(s_ * n_src * (64 + 64) * 2 + n_dst * kk * 16 + s_ * n_dst * 64 * 4)
    del k, v, w_q, nbr, rel, out, ws
    return {"workload": "0.25-degree lat-lon (721 x 1440) -> HEALPix Nside 256, 2 members x 16 heads, "
                        "d = dv = 64, 4 x 4 stencil", "ms": ms, "targets_per_s": s_ * n_dst / (ms * 1e-3),
            "algorithmic_bytes": byts, "GBs": byts / (ms * 1e-3) / 1e9,
            "frac_hbm_peak": byts / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}


def cpu_baseline(cfg: BSAConfig, inputs, budget_s: float) -> dict:
    """The float64 oracle as it stands, on whole (batch, head) slices of the
    same inputs, until `budget_s` seconds of work are done (at least one)."""
    import oracle
    from spherical_block_sparse_amd.synth import to_f64
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:   # pragma: no cover - threadpoolctl is optional
        threads = os.cpu_count() or 1
    q, k, v, g, _ = inputs
    done, t_total = 0, 0.0
    rng = np.random.default_rng(0)
    order = rng.permutation(cfg.slices)
    for s in order:
        b, h = divmod(int(s), cfg.heads)
        args = [to_f64(x[b, h]) for x in (q, k, v, g)]
        t0 = time.perf_counter()
        oracle.bsa_slice_ref(*args, cfg.block, cfg.topn, cfg.window)
        t_total += time.perf_counter() - t0
        done += 1
        print(f"[bench] oracle slice ({b},{h}) done, {t_total:.1f} s", file=sys.stderr, flush=True)
        if t_total >= budget_s:
            break
    # tokens/s in the metric's unit: one token = one pixel of one member across all heads
    tok_s = done * cfg.n_tokens / cfg.heads / t_total
    return {"value": tok_s, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} of {cfg.slices} (batch, head) slices of the {cfg.name} inputs, "
                      f"{t_total:.1f} s, scaled by 1/heads to whole tokens",
            "host_cpus": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)), "cpu_model": host_cpu_model()}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="ns128", choices=sorted(CONFIGS))
    ap.add_argument("--secondary", default="ns256", help="second workload reported alongside ('' for none)")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true", help="skip the (secondary) backward timing")
    ap.add_argument("--layer-channels", type=int, default=512, help="encoder-layer width (0: skip the layer timing)")
    ap.add_argument("--layers", type=int, default=4)
    ap.add_argument("--no-interp", action="store_true", help="skip the interpolation timing")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the BSA slices are independent and the library has no "
              "multi-GPU path (batch/head slices would shard across GPUs with no communication). "
              "Run with --gpus 1.", file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    _lib.lib()

    cfg = CONFIGS[args.config]
    r = measure(cfg, args.steps, args.warmup, backward=not args.no_backward)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, r["inputs"], args.cpu_budget)
    del r["inputs"]
    torch.cuda.empty_cache()
    layer = None
    if args.layer_channels:
        layer = measure_layer(cfg, args.layer_channels, args.layers, args.steps)
        torch.cuda.empty_cache()
    ceilings = measure_ceilings()
    interp = None
    if not args.no_interp:
        interp = measure_interp(args.steps)
        torch.cuda.empty_cache()

    secondary = None
    if args.secondary and args.secondary != args.config:
        s = measure(CONFIGS[args.secondary], max(5, args.steps // 2), max(2, args.warmup // 2),
                    backward=not args.no_backward)
        cpu2 = None
        if not args.no_cpu_baseline:
            cpu2 = cpu_baseline(s["cfg"], s["inputs"], args.cpu_budget)
        del s["inputs"]
        secondary = {
            "workload": s["cfg"].name, "value": s["tokens_per_s"], "unit": "tokens/s", "ms_per_step": s["ms"],
            "step_ms": s["step_ms"],
            "kernels_ms": {"pool": s["pool_ms"], "compress_select": s["cs_ms"], "select_bound": s["bound_ms"],
                           "fine": s["fine_ms"]},
            "fine_mfma_frac": s["fine_tflops"] / PEAK_BF16_TFLOPS,
            "compress_select_frac": compress_bound_ms(s["cfg"]) / s["cs_ms"],
            "pool_hbm_frac": s["pool_gbs"] / PEAK_HBM_GBS,
            "backward": s["backward"],
            "cpu_baseline": cpu2,
        }

    c = r["cfg"]
    line = {
        "metric": "BSA fwd tokens/s at Nside=128 & 256; % bf16 MFMA peak, % HBM peak",
        "value": r["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms"],
        # each timed call's own duration (events between consecutive calls)
        "step_ms": r["step_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{c.name}: HEALPix Nside={c.nside} NESTED, N={c.n_tokens}, batch {c.batch}, "
                        f"{c.heads} heads x {c.head_dim}, block {c.block} ({c.n_blocks} blocks), "
                        f"top-n {c.topn}, window {c.window}, {c.field} field",
            "global_batch": c.batch, "seq_len": c.n_tokens, "heads": c.heads, "head_dim": c.head_dim,
            "block": c.block, "topn": c.topn, "window": c.window, "tokens_per_step": c.tokens,
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "mfma", "kernel": "bsa_fine (fine_kernel<64, WAVES, kPlain>)",
            "achieved": r["fine_tflops"], "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": r["fine_tflops"] / PEAK_BF16_TFLOPS, "traffic": measured_traffic(f"fine_{c.name}"),
            "flops_per_launch": r["fine_flops"], "ms_per_launch": r["fine_ms"],
            # the same kernel's mean duration in the committed rocprofv3 trace of this command
            "profiled_ms_per_launch": profiled_ms(f"fine_{c.name}"),
            "frac_profiled": (None if profiled_ms(f"fine_{c.name}") is None else
                              r["fine_flops"] / (profiled_ms(f"fine_{c.name}") * 1e-3) / 1e12 / PEAK_BF16_TFLOPS),
        },
        "kernels": {
            "pool": {"ms": r["pool_ms"], "bound": "hbm", "achieved_GBs": r["pool_gbs"],
                     "frac": r["pool_gbs"] / PEAK_HBM_GBS, "bytes_per_launch": r["pool_bytes"],
                     "traffic": measured_traffic(f"pool_{c.name}")},
            "compress_select": {"ms": r["cs_ms"],
                                "bound": "bf16 matrix (3 piece products + ā·v̄)" if c.topn <= 16
                                         else "fp64 + bf16 matrix",
                                "bound_ms": compress_bound_ms(c), "frac": compress_bound_ms(c) / r["cs_ms"],
                                "achieved_TFLOPs": r["cs_tflops"],
                                "traffic": measured_traffic(f"select_{c.name}")},
            "select_bound": {"ms": r["bound_ms"]},
            "fine": {"ms": r["fine_ms"], "frac_bf16_peak": r["fine_tflops"] / PEAK_BF16_TFLOPS},
            "stages_match_forward": r["stages_match_forward"],
        },
        "backward": r["backward"],
        "encoder_layer": layer,
        "interpolation": interp,
        # the fine kernel and the pool against measured ceilings (context; the roofline
        # above uses the published peaks)
        "measured_ceilings": dict(ceilings,
                                  fine_frac_of_mfma=r["fine_tflops"] / ceilings["bf16_mfma_TFLOPs"],
                                  pool_frac_of_read=r["pool_gbs"] / ceilings["read_GBs"]),
        "cpu_baseline": cpu,
        "secondary": secondary,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
