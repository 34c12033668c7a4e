#!/usr/bin/env python3
"""Benchmark of one VMoBA attention layer, forward + backward, on one MI355X.

A step is the whole hot path over one batch of synthetic input already resident in
HBM: block-mean pooling -> global threshold selection -> block-sparse attention
forward -> backward (delta, dK/dV, dQ).  The default workload is the 3D layer at the
93x576x1024 training length: latent 24x36x64 = 55,296 tokens, 12 heads of 128, blocks
(4, 6, 8), tau = 0.25.

Prints one JSON line.  value = algorithmic TFLOP/s over the selected pairs,
(4 + 8) * d * P per step with P the selected token pairs (forward: Q K^T and P V;
backward: dV, dP, dQ, dK), divided by the measured step time.

Timing: W untimed warm-up steps, then K steps between two device synchronisations
(ms_per_step, the mean of the wall time, which gives `value`), with HIP events around
every stage of every step on the launch stream (stage means for the roofline, medians in
`timing`).  Then, unless --no-flush, the same K steps again, each after a 512 MiB scratch
write that evicts the L2 caches and the Infinity Cache (medians in `timing`, suffix
_flushed).  Then, unless --no-clock, 1.5 s of back-to-back steps while a second thread
samples the shader clock; `sclk` holds its median and the bf16 peak scaled to it.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_SCLK_MHZ = 2400.0      # the shader clock the bf16 peak is quoted at
FLUSH_BYTES = 512 << 20     # scratch written before each flushed repeat


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-flush", action="store_true",
                    help="skip the repeats with a 512 MiB scratch write before each step")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip sampling the shader clock during a 1.5 s run of steps")
    ap.add_argument("--workload", default="l3d_55k")
    ap.add_argument("--layer", type=int, default=0, help="layer of the workload's cycle")
    ap.add_argument("--tau", type=float, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--select-mode", default="threshold_global",
                    choices=["threshold_global", "topk_global", "threshold_local", "topk_local"],
                    help="selection strategy (the method's is threshold_global)")
    ap.add_argument("--topk", type=int, default=None, help="k of the top-k strategies")
    ap.add_argument("--dit", action="store_true",
                    help="time one synthetic DiT block (projections, MLP) around the layer")
    ap.add_argument("--granularity", default="block", choices=["block", "token"],
                    help="token: the token-granular query pool (prints its own line)")
    ap.add_argument("--sweep", action="store_true",
                    help="time every bf16 workload, layer and tau (one JSON line each)")
    ap.add_argument("--sweep-workloads", default=None,
                    help="comma-separated workloads for --sweep (default: all)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (counter scale)")
    ap.add_argument("--summarize-profile", metavar="DIR", default=None,
                    help="write the profiles/ summaries from the rocprofv3 runs under DIR "
                         "(kt: kernel trace; fetch, write, mops: counter runs of the step; "
                         "calf, calw: counter runs of --calibrate-copy; sq*: other counter "
                         "passes); no GPU is used")
    return ap.parse_args()


def calibrate_copy():
    """A plain copy of known size: 2^28 fp32 elements (1 GiB) read and written, 3 times.

    Under rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE its per-dispatch readings give the
    scale between the counters and algorithmic bytes."""
    import torch
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes_read": n * 4, "calibrate_copy_bytes_written": n * 4,
                      "launches": 3}), flush=True)


def cpu_baseline(inp, cfg, spec, tau, min_seconds=10.0, max_heads=4, mode="threshold_global",
                 topk=None):
    """The fp64 oracle on the host cores, on whole heads of the same layer: head 0, then
    further heads while less than `min_seconds` have passed (at most `max_heads`)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max(int(i.get("num_threads", 1)) for i in threadpool_info())
    except Exception:
        threads = os.cpu_count()
    T, H, W = cfg["T"], cfg["H"], cfg["W"]
    mem = oracle.block_members(T, H, W, spec.block)
    S = mem.shape[1]
    dt, flops, heads = 0.0, 0.0, 0
    while heads < min(max_heads, cfg["heads"]) and (heads == 0 or dt < min_seconds):
        h = slice(heads, heads + 1)
        q, k, v, do = (inp[x][:, :, h].float().numpy() for x in ("q", "k", "v", "do"))
        t0 = time.perf_counter()
        qp, kp = oracle.block_means(q, mem), oracle.block_means(k, mem)
        mask, _, _ = oracle.select_all_heads(qp, kp, tau, mode=mode, k=topk)
        o, lse = oracle.sparse_attention_fwd(q, k, v, mem, mask)
        oracle.sparse_attention_bwd(q, k, v, o, lse, do, mem, mask)
        dt += time.perf_counter() - t0
        flops += 12.0 * cfg["head_dim"] * float(mask.sum()) * S * S
        heads += 1
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"whole heads 0-{heads - 1} of {cfg['heads']} of the same layer (pool, "
                      f"select, sparse fwd+bwd in fp64): {dt:.1f} s wall for "
                      f"{flops / 1e12:.3f} TFLOP algorithmic; the rate is extrapolated to "
                      f"the layer's other heads (heads are independent problems of "
                      f"similar size)",
            "heads_timed": heads, "heads_in_layer": cfg["heads"], "seconds": dt}


def _kernel_source_hash(kernel):
    import hashlib
    src = {"attn_fwd_bf16_kernel": "attn_fwd.hip", "attn_fwd16_bf16_kernel": "attn_fwd.hip",
           "attn_bwd_dkdv_bf16_kernel": "attn_bwd.hip",
           "attn_bwd_dkdv_split_bf16_kernel": "attn_bwd.hip",
           "attn_bwd_dq_split_bf16_kernel": "attn_bwd.hip",
           "attn_bwd_dq_bf16_kernel": "attn_bwd.hip"}[kernel]
    h = hashlib.sha256()
    for fn in (src, "attn_common.h", "device_common.h"):
        with open(os.path.join(ROOT, "block_sparse_attention_layer_amd", "csrc", fn), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_counters(kernel, workload):
    """Per-launch counter record of `kernel` (sparse instance) from the committed summary,
    or None when there is none for this workload or the kernel's source changed since."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    want = _kernel_source_hash(kernel)
    for entry in rec["kernels"].values():   # the counter runs launch no dense baseline
        if entry["kernel"] == kernel and entry["source_sha"] == want:
            return entry
    return None


def recorded_traffic(kernel, workload):
    """HBM bytes per launch of `kernel`, copy-calibrated FETCH_SIZE + WRITE_SIZE, or None."""
    entry = recorded_counters(kernel, workload)
    return None if entry is None else entry["traffic_bytes"]


def fwd_kernel_name(qlim, head_dim, bf16):
    """The forward kernel the library launches: 48 queries per wave (16x16x32 MFMA) at
    d = 128 when 192-query tiles pad no more than 128-query ones."""
    if bf16 and head_dim == 128 and -(-qlim // 192) * 192 <= -(-qlim // 128) * 128:
        return "attn_fwd16_bf16_kernel"
    return "attn_fwd_bf16_kernel"


def dkdv_kernel_name(klim, head_dim, bf16):
    """The dK/dV kernel the library launches: 192 keys a workgroup in key groups of 48, each
    split over two waves (16x16x32 MFMA), at d = 128 when 192-key tiles pad no more than
    128-key ones."""
    if bf16 and head_dim == 128 and -(-klim // 192) * 192 <= -(-klim // 128) * 128:
        return "attn_bwd_dkdv_split_bf16_kernel"
    return "attn_bwd_dkdv_bf16_kernel"


def dq_kernel_name(qlim, head_dim, bf16, rows):
    """The dQ kernel the library launches: 192 queries a workgroup in query groups of 48,
    each split over two waves, at d = 128 when 192-query tiles pad no more than 128-query
    ones and either 128-query tiles would leave more than an eighth of their slots empty or
    the launch has at least 1,024 such workgroups (`rows`: head groups times query
    blocks)."""
    p128 = -(-qlim // 128) * 128
    t192 = -(-qlim // 192)
    if (bf16 and head_dim == 128 and t192 * 192 <= p128
            and ((p128 - qlim) * 8 > p128 or rows * t192 >= 1024)):
        return "attn_bwd_dq_split_bf16_kernel"
    return "attn_bwd_dq_bf16_kernel"


def _event_medians(evs, names, suffix):
    """Median over repeats of the step time and of each stage (HIP events)."""
    import statistics
    n = len(names)
    step = [e[0].elapsed_time(e[n]) for e in evs]
    stages = {nm: round(statistics.median(e[j].elapsed_time(e[j + 1]) for e in evs), 4)
              for j, nm in enumerate(names)}
    return {f"ms_per_step_median{suffix}": round(statistics.median(step), 4),
            f"ms_per_step_min{suffix}": round(min(step), 4),
            f"stage_ms_median{suffix}": stages}


def sample_sclk(step, seconds=1.5):
    """Shader clock (MHz, amd-smi's current GFX clock through torch) sampled every 10 ms
    from a second thread while `step` runs back to back for `seconds`."""
    import statistics
    import threading
    import torch
    try:
        torch.cuda.clock_rate(0)
    except Exception as e:   # no amd-smi access on this host
        return {"error": f"{type(e).__name__}: {e}"[:200]}
    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            try:
                c = torch.cuda.clock_rate(0)
                if c:
                    samples.append(float(c))
            except Exception:
                pass
            time.sleep(0.01)
    th = threading.Thread(target=sampler, daemon=True)
    t0 = time.perf_counter()
    th.start()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            step()
        torch.cuda.synchronize()
    stop.set()
    th.join()
    if not samples:
        return {"error": "no samples"}
    med = statistics.median(samples)
    return {"median_mhz": med, "min_mhz": min(samples), "max_mhz": max(samples),
            "samples": len(samples), "seconds": seconds,
            "bf16_peak_at_median_tflops": round(PEAK_BF16_TFLOPS * med / PEAK_SCLK_MHZ, 1)}


def run_config(workload, layer, tau, steps, warmup, dense_reps, cpu_sample,
               mode="threshold_global", topk=None, flush=False, clock=False):
    """Time the hot path of one layer of a workload; returns a dict of measurements.
    mode / topk choose the selection strategy (threshold_global, the method's, by default)."""
    import torch
    from synthetic import CONFIGS, make_layer_inputs
    import block_sparse_attention_layer_amd as vm

    cfg = CONFIGS[workload]
    spec = cfg["layers"][layer]
    if tau is None:
        tau = 0.25 if 0.25 in cfg["taus"] else cfg["taus"][0]
    dev = torch.device("cuda:0")
    inp = make_layer_inputs(workload, layer, backward=True)
    dtype = torch.bfloat16 if cfg["dtype"] == "bf16" else torch.float32
    p = vm.Problem(cfg["batch"], cfg["heads"], cfg["head_dim"], cfg["T"], cfg["H"], cfg["W"],
                   spec.layer_idx, tuple(spec.block), dtype, dtype)
    q, k, v, do = (inp[x].to(dev) for x in ("q", "k", "v", "do"))
    nb = vm.vmoba_num_blocks(p)
    S = p.L // nb
    d = p.head_dim
    names = ["pool", "select", "fwd", "delta", "dkdv", "dq"]

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record()
        mark(0)
        qp, kp = vm.vmoba_partition_pool(p, q, k)
        mark(1)
        sel = vm.vmoba_select(p, qp, kp, tau, mode=mode, k=topk)
        mark(2)
        o, lse = vm.vmoba_sparse_attn_fwd(p, q, k, v, sel.row_ptr, sel.col_idx)
        mark(3)
        delta = vm.vmoba_sparse_attn_bwd_delta(p, o, do)
        mark(4)
        vm.vmoba_sparse_attn_bwd_dkdv(p, q, k, v, lse, delta, do, sel.col_ptr, sel.row_idx)
        mark(5)
        vm.vmoba_sparse_attn_bwd_dq(p, q, k, v, lse, delta, do, sel.row_ptr, sel.col_idx)
        mark(6)
        return sel

    for _ in range(warmup):
        sel = step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        sel = step(evs[i])
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / steps
    stage_ms = {n: sum(e[j].elapsed_time(e[j + 1]) for e in evs) / steps
                for j, n in enumerate(names)}
    timing = {"repeats": steps, "ms_per_step_mean_wall": round(ms_step, 4)}
    timing.update(_event_medians(evs, names, ""))
    if flush:
        # the same steps with a 512 MiB scratch write before each (evicts L2 and the
        # 256 MB Infinity Cache); events bracket the step only
        scratch = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
        fevs = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(steps)]
        for i in range(steps):
            scratch.fill_(float(i))
            step(fevs[i])
        torch.cuda.synchronize()
        del scratch
        timing["flush_bytes"] = FLUSH_BYTES
        timing.update(_event_medians(fevs, names, "_flushed"))
    sclk = sample_sclk(step) if clock else None

    nnz = float(sel.head_stats[:, 1].double().sum().item())
    pairs = nnz * S * S
    fl = {"fwd": 4.0 * d * pairs, "dkdv": 6.0 * d * pairs, "dq": 2.0 * d * pairs}
    executed = {"fwd": 4.0 * d * pairs, "dkdv": 8.0 * d * pairs, "dq": 6.0 * d * pairs}
    esz = 2 if dtype == torch.bfloat16 else 4
    pool_bytes = 2.0 * p.L * p.groups * d * esz + 2.0 * p.groups * nb * d * 4
    select_bytes = 2.0 * p.groups * nb * d * 4 + 6.0 * p.groups * nb * nb * 4
    kernel_names = {"fwd": fwd_kernel_name(S, d, dtype == torch.bfloat16),
                    "dkdv": dkdv_kernel_name(S, d, dtype == torch.bfloat16),
                    "dq": dq_kernel_name(S, d, dtype == torch.bfloat16, p.groups * nb)}

    dense = None
    if dense_reps > 0:
        o_d, lse_d = vm.vmoba_dense_attn_fwd(p, q, k, v)
        vm.vmoba_dense_attn_bwd(p, q, k, v, o_d, lse_d, do)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(dense_reps):
            o_d, lse_d = vm.vmoba_dense_attn_fwd(p, q, k, v)
            vm.vmoba_dense_attn_bwd(p, q, k, v, o_d, lse_d, do)
        torch.cuda.synchronize()
        dense = (time.perf_counter() - t1) * 1e3 / dense_reps

    cpu = None
    if cpu_sample:
        cpu = cpu_baseline(inp, cfg, spec, tau, mode=mode, topk=topk)
        cpu.pop("seconds")
    return dict(cfg=cfg, spec=spec, tau=tau, mode=mode, topk=topk, p=p, nb=nb, S=S, d=d,
                dtype=dtype,
                ms_step=ms_step, stage_ms=stage_ms, pairs=pairs,
                density=nnz / (p.groups * nb * nb), fl=fl, executed=executed,
                pool_bytes=pool_bytes, select_bytes=select_bytes, kernel_names=kernel_names,
                dense=dense, cpu=cpu, timing=timing, sclk=sclk)


def run_tokens(workload, layer, tau, steps, warmup):
    """Time the token-granular path of one layer (pool, token selection, forward under the
    token mask, backward) and print one JSON line."""
    import torch
    from synthetic import CONFIGS, make_layer_inputs
    import block_sparse_attention_layer_amd as vm

    cfg = CONFIGS[workload]
    spec = cfg["layers"][layer]
    if tau is None:
        tau = 0.25 if 0.25 in cfg["taus"] else cfg["taus"][0]
    dev = torch.device("cuda:0")
    inp = make_layer_inputs(workload, layer, backward=True)
    p = vm.Problem(cfg["batch"], cfg["heads"], cfg["head_dim"], cfg["T"], cfg["H"], cfg["W"],
                   spec.layer_idx, tuple(spec.block), torch.bfloat16, torch.bfloat16)
    q, k, v, do = (inp[x].to(dev) for x in ("q", "k", "v", "do"))
    nb = vm.vmoba_num_blocks(p)
    S = p.L // nb
    d = p.head_dim
    names = ["pool", "select_tokens", "fwd", "bwd"]

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record()
        mark(0)
        _, kp = vm.vmoba_partition_pool(p, q, k)
        mark(1)
        sel = vm.vmoba_select_tokens(p, q, kp, tau)
        mark(2)
        o, lse = vm.vmoba_token_attn_fwd(p, q, k, v, sel.row_ptr, sel.col_idx, sel.token_mask)
        mark(3)
        vm.vmoba_token_attn_bwd(p, q, k, v, o, lse, do, sel.row_ptr, sel.col_idx, sel.col_ptr,
                                sel.row_idx, sel.token_mask)
        mark(4)
        return sel

    for _ in range(warmup):
        sel = step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        sel = step(evs[i])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    st = {n: sum(e[j].elapsed_time(e[j + 1]) for e in evs) / steps for j, n in enumerate(names)}
    tok_pairs = float(sel.head_stats[:, 1].double().sum().item())     # (token, block) pairs
    union_pairs = float(sel.row_ptr[:, -1].double().sum().item())      # listed block pairs
    pairs = tok_pairs * S                        # (query token, key token) pairs attended
    walked = union_pairs * S * S                 # pairs the kernels walk (masked ones too)
    line = {
        "metric": "VMoBA token-granular pool: attn fwd+bwd TFLOP/s at 55K tokens",
        "value": round(12.0 * d * pairs / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
        "ms_per_step": round(ms, 4), "steps": steps, "warmup": warmup,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{workload} layer {layer} (blocks {tuple(spec.block)}, "
                               f"{nb} of {S}), tau {tau}, token-granular query pool"},
        "stages_ms": {n: round(st[n], 4) for n in names},
        "selected_token_pairs": pairs, "walked_token_pairs": walked,
        "kept_fraction_of_walked": round(pairs / walked, 4),
        "token_pair_density": round(pairs / (p.groups * float(p.L) ** 2), 5),
        "fwd_tflops_walked": round(4.0 * d * walked / (st["fwd"] * 1e-3) / 1e12, 2),
        "select_gbs": round(p.groups * float(p.L) * nb * 4 * 6 / (st["select_tokens"] * 1e-3)
                            / 1e9, 1),
    }
    print(json.dumps(line), flush=True)


def run_dit(workload, layer, tau, steps, warmup, mlp_hidden=8960):
    """One pre-norm DiT block at Wan 2.1 1.3B's sizes (dim = heads * d = 1536, MLP 8960)
    around the layer, forward + backward in bf16 on the workload's latent: the sparse step
    and the dense (warm-up) step, with the attention calls timed apart from the rest.
    Prints one JSON line."""
    import torch
    from synthetic import CONFIGS, make_dit_input, make_dit_params
    import block_sparse_attention_layer_amd as vm

    cfg = CONFIGS[workload]
    spec = cfg["layers"][layer]
    if tau is None:
        tau = 0.25 if 0.25 in cfg["taus"] else cfg["taus"][0]
    dev = torch.device("cuda:0")
    heads, d = cfg["heads"], cfg["head_dim"]
    dim = heads * d
    latent = (cfg["T"], cfg["H"], cfg["W"])
    blocks = [None, None, None]
    blocks[spec.layer_idx % 3] = tuple(spec.block)
    T, H, W = latent
    defaults = [(1, H, W), (T, H, W), (T, H, W)]   # unused modes: any valid shape
    cyc = vm.LayerCycle(latent, *[b or defaults[i] for i, b in enumerate(blocks)])
    blk = vm.SyntheticDiTBlock(dim, heads, mlp_hidden, spec.layer_idx, cyc, tau=tau,
                               dtype=torch.bfloat16, device=dev)
    blk.load_params({n: t.to(torch.bfloat16) for n, t in
                     make_dit_params(dim, mlp_hidden, 1, seed=7000)[0].items()})
    x, g = (t.to(dev, torch.bfloat16) for t in make_dit_input(cfg["batch"], latent, dim))

    # time the attention calls inside the block with events around the library entry points
    attn_ms = []
    import block_sparse_attention_layer_amd.layer as lay
    orig = {}
    for name in ("vmoba_sparse_attn_fwd", "vmoba_sparse_attn_bwd", "vmoba_dense_attn_fwd",
                 "vmoba_dense_attn_bwd", "select_blocks"):
        fn = getattr(lay, name)
        orig[name] = fn

        def wrapped(*a, _fn=fn, **kw):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            out = _fn(*a, **kw)
            e1.record()
            attn_ms.append((e0, e1))
            return out
        setattr(lay, name, wrapped)

    def run(full):
        xg = x.detach().requires_grad_()
        y = blk(xg, full=full)
        y.backward(g)

    out = {}
    try:
        for full in (False, True):
            for _ in range(warmup):
                run(full)
            torch.cuda.synchronize()
            attn_ms.clear()
            t0 = time.perf_counter()
            for _ in range(steps):
                run(full)
            torch.cuda.synchronize()
            ms = (time.perf_counter() - t0) * 1e3 / steps
            a = sum(e0.elapsed_time(e1) for e0, e1 in attn_ms) / steps
            out["dense" if full else "sparse"] = (ms, a)
    finally:
        for name, fn in orig.items():
            setattr(lay, name, fn)
    (ms_s, a_s), (ms_d, a_d) = out["sparse"], out["dense"]
    line = {
        "metric": "DiT block fwd+bwd ms (VMoBA layer vs full attention)",
        "config": {"workload": f"{workload} layer {layer}: latent {T}x{H}x{W} = {T * H * W} "
                               f"tokens, dim {dim} ({heads} x {d}), MLP {mlp_hidden}, blocks "
                               f"{tuple(spec.block)}, tau {tau}, bf16, synthetic weights"},
        "steps": steps, "warmup": warmup,
        "sparse_block_ms": round(ms_s, 3), "sparse_attention_ms": round(a_s, 3),
        "dense_block_ms": round(ms_d, 3), "dense_attention_ms": round(a_d, 3),
        "rest_of_block_ms": round(ms_s - a_s, 3),
        "attention_share_sparse": round(a_s / ms_s, 3),
        "attention_share_dense": round(a_d / ms_d, 3),
        "block_speedup": round(ms_d / ms_s, 3),
    }
    print(json.dumps(line), flush=True)


def describe(workload, r):
    p, spec = r["p"], r["spec"]
    sel = ("" if r.get("mode", "threshold_global") == "threshold_global"
           else f", selection {r['mode']} k {r['topk']}")
    return (f"{workload}: layer_idx {spec.layer_idx} (l mod 3 = {spec.layer_idx % 3}), latent "
            f"{p.T}x{p.H}x{p.W} = {p.L} tokens, {p.heads} heads x {r['d']}, blocks "
            f"{tuple(spec.block)} ({r['nb']} blocks of {r['S']}), tau {r['tau']}{sel}, "
            f"pool+select+sparse fwd+bwd")


def summary(r):
    """Per-stage figures shared by the contract line and the sweep lines."""
    sm, fl, pairs, d = r["stage_ms"], r["fl"], r["pairs"], r["d"]
    attn = ["fwd", "dkdv", "dq"]
    ms = r["ms_step"]
    return {
        "stages_ms": {n: round(sm[n], 4) for n in sm},
        "attn_ms": round(sum(sm[n] for n in ("fwd", "delta", "dkdv", "dq")), 4),
        "stage_tflops": {n: round(fl[n] / (sm[n] * 1e-3) / 1e12, 2) for n in attn},
        "stage_frac_bf16_peak": {n: round(fl[n] / (sm[n] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
                                 for n in attn},
        "tflops_fa_convention": round((4.0 + 10.0) * d * pairs / (ms * 1e-3) / 1e12, 2),
        "pool_gbs": round(r["pool_bytes"] / (sm["pool"] * 1e-3) / 1e9, 1),
        "pool_frac_hbm": round(r["pool_bytes"] / (sm["pool"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "select_gbs": round(r["select_bytes"] / (sm["select"] * 1e-3) / 1e9, 1),
        "select_frac_hbm": round(r["select_bytes"] / (sm["select"] * 1e-3) / 1e9 /
                                 PEAK_HBM_GBS, 5),
        "kept_pair_density": round(r["density"], 5),
        "selected_token_pairs": pairs,
        "dense_ms_per_step": None if r["dense"] is None else round(r["dense"], 3),
        "speedup_vs_dense": None if r["dense"] is None else round(r["dense"] / ms, 3),
    }


def _short_kernel(name):
    """'void vmoba::k<unsigned short, 128>(vmoba::Geom, ...)' -> 'k<bf16, 128>'."""
    n = name.replace("void ", "").replace("vmoba::", "")
    depth, out = 0, []
    for ch in n:   # drop the argument list: the first '(' outside template brackets
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            break
        out.append(ch)
    return "".join(out).replace("unsigned short", "bf16").strip()


def _csv_rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def _find(dirpath, suffix):
    for root, _, files in os.walk(dirpath):
        for fn in files:
            if fn.endswith(suffix):
                return os.path.join(root, fn)
    raise FileNotFoundError(f"no *{suffix} under {dirpath}")


def _per_dispatch(dirpath, counter):
    """Mean per dispatch of `counter` for every kernel of one rocprofv3 --pmc run."""
    acc = {}
    for r in _csv_rows(_find(dirpath, "counter_collection.csv")):
        if r["Counter_Name"] != counter:
            continue
        k = _short_kernel(r["Kernel_Name"])
        acc.setdefault(k, []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}, {k: len(v) for k, v in acc.items()}


def summarize_profile(d, workload="l3d_55k", steps=20, warmup=5):
    """profiles/ summaries from rocprofv3 output directories under d (see --help)."""
    out_dir = os.path.join(ROOT, "profiles")
    hot = ["pool_kernel", "block_scores_kernel", "attn_fwd16_bf16_kernel",
           "attn_fwd_bf16_kernel", "delta_kernel", "attn_bwd_dkdv_split_bf16_kernel",
           "attn_bwd_dkdv_bf16_kernel", "attn_bwd_dq_split_bf16_kernel",
           "attn_bwd_dq_bf16_kernel"]
    bench_cmd = "python3 <repo>/bench.py"
    pmc_cmd = ("python3 <repo>/bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-dense "
               "--no-flush --no-clock")
    # kernel trace: all launches, and the timed launches of the sparse instances
    stats = _csv_rows(_find(os.path.join(d, "kt"), "kernel_stats.csv"))
    trace = _csv_rows(_find(os.path.join(d, "kt"), "kernel_trace.csv"))
    trace.sort(key=lambda r: int(r["Start_Timestamp"]))
    by_kernel = {}
    for r in trace:
        k = _short_kernel(r["Kernel_Name"])
        by_kernel.setdefault(k, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6)
    lines = [f"# rocprofv3 kernel trace: 3D layer, 55,296 tokens ({workload}), pool + select + "
             "sparse fwd + bwd", "",
             "Command (run from /tmp, with TMPDIR=/tmp; `<repo>` is the repository root):", "",
             f"    rocprofv3 --kernel-trace --stats -d <out>/kt -o kt --output-format csv -- {bench_cmd}",
             "", f"bench.py with its defaults: {warmup} warm-up steps, {steps} timed steps, the "
             f"same {steps} steps after a 512 MiB scratch write each, 1.5 s of steps while the "
             "clock is sampled, then the dense baseline (1 warm-up + 2 timed forward+backward "
             "passes) and the CPU oracle sample (host only).  Per-kernel statistics of "
             "`kt_kernel_stats.csv` (every launch of the run):", "",
             "| kernel | launches | avg ms | min ms | max ms | share |", "|---|---|---|---|---|---|"]
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"]))[:22]:
        kname = _short_kernel(r["Name"])
        kname = kname if len(kname) <= 90 else kname[:87] + "..."
        lines.append(f"| {kname} | {r['Calls']} | "
                     f"{float(r['AverageNs']) / 1e6:.3f} | {float(r['MinNs']) / 1e6:.3f} | "
                     f"{float(r['MaxNs']) / 1e6:.3f} | {float(r['Percentage']):.1f}% |")
    lines += ["", f"Averages over the {steps} timed launches of each sparse instance (launches "
              f"{warmup + 1} to {warmup + steps} in time order, the ones bench.py times with "
              "events):", ""]
    timed = {}
    for k, ds in by_kernel.items():
        base = k.split("<")[0]
        if base in hot and ("false" in k or "<bf16, 128>" in k or base in ("pool_kernel", "block_scores_kernel")):
            if "true, false" in k and base.startswith("attn"):   # dense instances
                continue
            sel = ds[warmup:warmup + steps]
            if sel:
                timed[k] = sum(sel) / len(sel)
                lines.append(f"- {k}: {timed[k]:.4f} ms")
    # bench.py's own line from the profiled run: its event-timed stage means must agree
    try:
        with open(os.path.join(d, "kt.log")) as f:
            bl = next(json.loads(x) for x in f if x.startswith('{"metric"'))
        sm = bl["stages_ms"]
        lines += ["", f"bench.py's own HIP-event means over the same {steps} timed steps of the "
                  "profiled run: " + ", ".join(f"{k} {v:.4f} ms" for k, v in sm.items()) +
                  f"; {bl['ms_per_step']:.3f} ms a step, {bl['value']:.1f} TFLOP/s "
                  "algorithmic (the profiler's own overhead included)."]
    except (OSError, StopIteration, KeyError, ValueError):
        pass
    lines += ["", "Written by `python3 bench.py --summarize-profile <out>` from the run above."]
    with open(os.path.join(out_dir, f"kernel_trace_{workload}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    # HBM traffic and MFMA work per dispatch
    fetch, n_f = _per_dispatch(os.path.join(d, "fetch"), "FETCH_SIZE")
    write, _ = _per_dispatch(os.path.join(d, "write"), "WRITE_SIZE")
    mops, _ = _per_dispatch(os.path.join(d, "mops"), "SQ_INSTS_VALU_MFMA_MOPS_BF16")
    calf, _ = _per_dispatch(os.path.join(d, "calf"), "FETCH_SIZE")
    calw, _ = _per_dispatch(os.path.join(d, "calw"), "WRITE_SIZE")
    copy_bytes = float(1 << 30)
    cf = copy_bytes / (max(calf.values()) * 1024.0)
    cw = copy_bytes / (max(calw.values()) * 1024.0)
    rec = {"workload": workload, "fetch_scale": cf, "write_scale": cw, "kernels": {}}
    rows = []
    for k in fetch:
        base = k.split("<")[0]
        if base not in hot:
            continue
        try:
            sha = _kernel_source_hash(base)
        except KeyError:
            sha = None
        rb, wb = fetch[k] * 1024.0 * cf, write.get(k, 0.0) * 1024.0 * cw
        rec["kernels"][k] = {"kernel": base, "fetch_kib": fetch[k], "write_kib": write.get(k, 0.0),
                             "read_bytes": rb, "write_bytes": wb, "traffic_bytes": rb + wb,
                             "mfma_mops": mops.get(k, 0.0), "source_sha": sha}
        rows.append(f"| {k} | {n_f[k]} | {fetch[k]:.0f} | {write.get(k, 0.0):.0f} | "
                    f"{rb / 1e9:.3f} | {wb / 1e9:.3f} | {(rb + wb) / 1e9:.3f} | "
                    f"{mops.get(k, 0.0):.4g} |")
    with open(os.path.join(out_dir, f"hbm_traffic_{workload}.json"), "w") as f:
        json.dump(rec, f, indent=1)
    lines = [f"# HBM traffic per launch: 3D layer, 55,296 tokens ({workload})", "",
             "Commands (run from /tmp, with TMPDIR=/tmp; `<repo>` is the repository root), one "
             "counter per run:", ""]
    for name, ctr, cmd in (("fetch", "FETCH_SIZE", pmc_cmd), ("write", "WRITE_SIZE", pmc_cmd),
                           ("mops", "SQ_INSTS_VALU_MFMA_MOPS_BF16", pmc_cmd),
                           ("calf", "FETCH_SIZE", "python3 <repo>/bench.py --calibrate-copy"),
                           ("calw", "WRITE_SIZE", "python3 <repo>/bench.py --calibrate-copy")):
        lines.append(f"    rocprofv3 --pmc {ctr} -d <out>/{name} -o {name} --output-format csv -- {cmd}")
    lines += ["", f"Calibration: a plain device copy of 1 GiB reads {max(calf.values()):.0f} KiB "
              f"of FETCH_SIZE and {max(calw.values()):.0f} KiB of WRITE_SIZE per dispatch, so "
              f"bytes = FETCH_SIZE x 1024 x {cf:.3f} and WRITE_SIZE x 1024 x {cw:.3f}.", "",
              "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | read GB | written GB | "
              "traffic GB | MFMA MOPs (512 flop) |", "|---|---|---|---|---|---|---|---|"] + rows
    lines += ["", "`source_sha` in the JSON beside this file hashes the kernel's source file "
              "with the two shared headers; bench.py reports `roofline.traffic` only while it "
              "still matches.", "",
              "Written by `python3 bench.py --summarize-profile <out>` from the runs above."]
    with open(os.path.join(out_dir, f"hbm_traffic_{workload}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    # further counter passes (sq*): every counter of every pass, per dispatch
    passes = sorted(x for x in os.listdir(d) if x.startswith("sq") and os.path.isdir(os.path.join(d, x)))
    if passes:
        lines = [f"# Counters of the attention kernels: 3D layer, 55,296 tokens ({workload})", "",
                 "One rocprofv3 --pmc pass per row group below, each as", "",
                 f"    rocprofv3 --pmc <counters> -d <out>/<pass> -o <pass> --output-format csv -- {pmc_cmd}",
                 "", "Values are means per dispatch of the sparse instances, summed over the "
                 "chip as rocprofv3 reports them (SQ_WAVE_CYCLES, SQ_WAIT_*, SQ_ACTIVE_* are in "
                 "quad-cycles; GRBM_GUI_ACTIVE is summed over the 8 XCDs).", ""]
        bases = ["attn_fwd16_bf16_kernel", "attn_bwd_dkdv_split_bf16_kernel",
                 "attn_bwd_dq_split_bf16_kernel"]
        all_vals = {}
        for ps in passes:
            vals = {}
            for r in _csv_rows(_find(os.path.join(d, ps), "counter_collection.csv")):
                k = _short_kernel(r["Kernel_Name"])
                vals.setdefault((r["Counter_Name"], k), []).append(float(r["Counter_Value"]))
            all_vals[ps] = vals
        # the sparse instance of each kernel (the dense ones carry "true, false")
        seen = {k for vals in all_vals.values() for (_, k) in vals}
        kernels = [next((k for k in sorted(seen) if k.split("<")[0] == b and "true, false" not in k),
                        b) for b in bases]
        lines.append("| pass | counter | " + " | ".join(k.split("<")[0] for k in kernels) + " |")
        lines.append("|---|---|" + "---|" * len(kernels))
        for ps in passes:
            vals = all_vals[ps]
            for ctr in sorted({c for c, _ in vals}):
                cells = []
                for k in kernels:
                    v = vals.get((ctr, k))
                    cells.append(f"{sum(v) / len(v):.4g}" if v else "")
                lines.append(f"| {ps} | {ctr} | " + " | ".join(cells) + " |")
        with open(os.path.join(out_dir, f"counters_{workload}.md"), "w") as f:
            f.write("\n".join(lines) + "\n")
    print(json.dumps({"timed_avg_ms": timed, "traffic_gb": {
        k: round(v["traffic_bytes"] / 1e9, 3) for k, v in rec["kernels"].items()}}))


def main():
    args = parse()
    if args.summarize_profile:
        summarize_profile(args.summarize_profile)
        return
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported (the layer "
              f"would shard over heads, see the design notes).", file=sys.stderr)
        sys.exit(2)
    if args.sweep:
        sweep(args)
        return
    if args.dit:
        run_dit(args.workload, args.layer, args.tau, args.steps, args.warmup)
        return
    if args.granularity == "token":
        run_tokens(args.workload, args.layer, args.tau, args.steps, args.warmup)
        return

    r = run_config(args.workload, args.layer, args.tau, args.steps, args.warmup,
                   0 if args.no_dense else 2, not args.no_cpu_baseline,
                   args.select_mode, args.topk, flush=not args.no_flush,
                   clock=not args.no_clock)
    ms_step, stage_ms, fl = r["ms_step"], r["stage_ms"], r["fl"]
    value = 12.0 * r["d"] * r["pairs"] / (ms_step * 1e-3) / 1e12
    dom = max(["fwd", "dkdv", "dq"], key=lambda n: stage_ms[n])
    kname = r["kernel_names"][dom]
    achieved = fl[dom] / (stage_ms[dom] * 1e-3) / 1e12
    counters = recorded_counters(kname, args.workload)
    mfma_util = None
    if counters is not None and counters.get("mfma_mops") is not None:
        # executed MFMA work (512 flops per MOP) over the live launch time at peak
        mfma_util = counters["mfma_mops"] * 512.0 / (stage_ms[dom] * 1e-3) / (
            PEAK_BF16_TFLOPS * 1e12)
    line = {
        "metric": "VMoBA attn fwd+bwd ms/layer & TFLOP/s (% bf16 MFMA peak) at 55K tokens",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if str(r["dtype"]) == "torch.bfloat16" else "fp32",
        "data": "synthetic",
        "config": {"workload": describe(args.workload, r), "global_batch": r["p"].batch,
                   "seq_len": r["p"].L, "parallelism": "none (1 GPU)"},
        "roofline": {
            "kernel": kname, "bound": "mfma",
            "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": None if counters is None else counters["traffic_bytes"],
            "traffic_unit": "HBM bytes per launch (FETCH_SIZE and WRITE_SIZE, copy-calibrated)",
            "avg_ms": round(stage_ms[dom], 4),
            "algorithmic_flops_per_launch": fl[dom],
            "executed_flops_per_launch": r["executed"][dom],
            "mfma_util_counter": None if mfma_util is None else round(mfma_util, 4)},
        "cpu_baseline": r["cpu"],
        "timing": r["timing"],
        "sclk": r["sclk"],
    }
    sc = r["sclk"]
    if sc and "median_mhz" in sc:
        # the same work against the peak at the clock the chip held while running it
        line["roofline"]["peak_at_sclk"] = sc["bf16_peak_at_median_tflops"]
        line["roofline"]["frac_at_sclk"] = round(achieved / sc["bf16_peak_at_median_tflops"], 4)
    line.update(summary(r))
    print(json.dumps(line), flush=True)


def sweep(args):
    """One JSON line per workload layer and tau (the per-config report; not the contract
    line).  Fewer steps, no CPU sample."""
    from synthetic import CONFIGS, CONFIG_ORDER
    names = args.sweep_workloads.split(",") if args.sweep_workloads else CONFIG_ORDER
    for name in names:
        cfg = CONFIGS[name]
        if cfg["dtype"] != "bf16":
            continue
        for layer in range(len(cfg["layers"])):
            for tau in cfg["taus"]:
                r = run_config(name, layer, tau, args.steps, args.warmup,
                               0 if args.no_dense else 1, False)
                line = {"workload": describe(name, r), "ms_per_step": round(r["ms_step"], 4),
                        "tflops": round(12.0 * r["d"] * r["pairs"] / (r["ms_step"] * 1e-3) /
                                        1e12, 2)}
                line.update(summary(r))
                print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
