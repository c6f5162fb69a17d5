"""Throughput of the MoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload full_t512]

One step = one moe_layer_forward (router, selection, permute, gate/up +
SwiGLU, down, combine; shared expert included) over one batch of synthetic
tokens already resident in HBM.  Prints one JSON line.  `value` comes from K
steps captured in one HIP graph and replayed (the same kernels as an eager
call, without the per-launch host and dispatch cost; --eager times steps
launched one by one instead).  Besides tokens/s it reports the roofline of the
dominant kernel (its algorithmic bytes or flops per launch over its average
duration, timed with HIP events recorded on the library's stream around that
kernel in every step of an eager timed loop of K steps), the layer's fraction
of the HBM and bf16 MFMA peaks against its target, and the CPU oracle timed on
this host (`cpu_baseline`).

The default workload (512 tokens: the weight-streaming, HBM-bound regime) is
the headline; the same run measures the 16384-token layer with an expert bias
(`large_batch`) and the 65536-token layer with skewed routing (`skew`), the
MFMA regime, and the 256-token fp32 layer (`fp32`), each with its own
roofline, target and CPU baseline.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/sec (2048h, 256e top-8) on 1 MI355X; % MFMA / HBM peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MALL_BYTES = 256 * 2 ** 20     # MI355X Infinity Cache
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s


def algorithmic_work(shape, counts):
    """Per-launch algorithmic bytes (and flops) of the kernels and the layer.

    Bytes count what the method must move at least once: the weights of every
    expert that received a token, the shared expert, the router weight, x, y
    and the routing outputs.  Intermediates (hidden activations, per-pair
    outputs) are excluded everywhere: the gate/up figure (the roofline's
    dominant kernel at small T) is its weights and x, the down figure its
    weights only."""
    T, H, I, Is, K, E = shape.T, shape.H, shape.I, shape.I_shared, shape.top_k, shape.E
    elt = 2 if shape.dtype == "bf16" else 4
    hit = int((counts > 0).sum())
    P = T * K
    gate_up_w = (hit * 2 * I * H + 2 * Is * H) * elt
    down_w = (hit * I * H + Is * H) * elt
    k_gate_up = gate_up_w + T * H * elt
    k_down = down_w
    layer = (gate_up_w + down_w + E * H * 4 + 2 * T * H * elt + P * 8)
    flops_gate_up = 2.0 * 2 * (P * I + T * Is) * H
    flops_down = 2.0 * (P * I + T * Is) * H
    flops_router = 2.0 * T * E * H
    return dict(hit=hit, k_gate_up=k_gate_up, k_down=k_down, layer=layer,
                flops_gate_up=flops_gate_up, flops_down=flops_down,
                flops_layer=flops_gate_up + flops_down + flops_router)


class HipEvents:
    """Timing events created directly through the HIP runtime, without the
    system-scope fence torch's events carry (that fence costs several
    microseconds per record between two kernels)."""
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, n):
        import ctypes
        try:
            self.hip = ctypes.CDLL("libamdhip64.so")
        except OSError:
            self.hip = ctypes.CDLL("/opt/rocm/lib/libamdhip64.so")
        self.c = ctypes
        self.ev = []
        for _ in range(n):
            h = ctypes.c_void_p()
            rc = self.hip.hipEventCreateWithFlags(ctypes.byref(h),
                                                  ctypes.c_uint(self.DISABLE_SYSTEM_FENCE))
            if rc != 0:
                raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
            self.ev.append(h.value)

    def elapsed_ms(self, a, b):
        ms = self.c.c_float()
        rc = self.hip.hipEventElapsedTime(self.c.byref(ms), self.c.c_void_p(a), self.c.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def close(self):
        for h in self.ev:
            self.hip.hipEventDestroy(self.c.c_void_p(h))


KERNEL_SOURCES = ("experts.hip", "experts_gemm.hip", "experts_stream.hip", "expert_tiles.h",
                  "ring.h", "device.h", "kernels.h")


def kernel_source_hash():
    import hashlib
    csrc = os.path.join(ROOT, "group_limited_top_amd", "csrc")
    return hashlib.sha256(b"".join(open(os.path.join(csrc, f), "rb").read()
                                   for f in KERNEL_SOURCES)).hexdigest()


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter runs
    (profiles/traffic.json), or None when the kernel sources changed since."""
    try:
        rec = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))[workload][kernel]
    except (OSError, KeyError, ValueError):
        return None
    if kernel_source_hash() != rec["source_sha256"]:
        return None
    return rec["hbm_bytes_per_launch"]


def _counter_means(run_dir, counter):
    """Per kernel (short name): mean of `counter` per dispatch in a rocprofv3
    --pmc csv run directory."""
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    tot, disp = {}, {}
    for f in files:
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            k = r["Kernel_Name"].split("(")[0].replace("void ", "").replace("moe::", "").strip()
            tot[k] = tot.get(k, 0.0) + float(r["Counter_Value"])
            disp.setdefault(k, set()).add(r["Dispatch_Id"])
    return {k: tot[k] / len(disp[k]) for k in tot}


def write_traffic(workload, fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, copy_mib, note):
    """profiles/traffic.json entries for every libmoe kernel of `workload`: HBM
    bytes per launch = FETCH_SIZE x f + WRITE_SIZE x w (KiB), with f and w set
    so that a plain device copy of copy_mib MiB reads and writes its size."""
    fetch = _counter_means(fetch_dir, "FETCH_SIZE")
    write = _counter_means(write_dir, "WRITE_SIZE")
    cf = _counter_means(copy_fetch_dir, "FETCH_SIZE")
    cw = _counter_means(copy_write_dir, "WRITE_SIZE")
    copy_k = [k for k in cf if "copyBuffer" in k]
    if not copy_k:
        raise SystemExit("no copy kernel in the calibration runs")
    kib = copy_mib * 1024.0
    fscale = round(kib / cf[copy_k[0]], 4)
    wscale = round(kib / cw[copy_k[0]], 4)
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        data = json.load(open(path))
    except (OSError, ValueError):
        data = {}
    entry = {}
    for k in sorted(fetch):
        if not k.startswith("k_") or k not in write:
            continue
        entry[k] = {"hbm_bytes_per_launch": int(round((fetch[k] * fscale + write[k] * wscale) * 1024)),
                    "fetch_kib": round(fetch[k], 1), "write_kib": round(write[k], 1),
                    "fetch_scale": fscale, "write_scale": wscale,
                    "source_sha256": kernel_source_hash(), "profile": note}
    data[workload] = entry
    with open(path, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps({workload: entry}, indent=1))


def measure_peaks():
    """What this GPU reaches on a pure streaming read of 4 GiB (global -> LDS
    loads) and on a loop of register-operand bf16 MFMAs (libmoe_probe,
    include/moe_probe.h): the best of a few launches each, timed with HIP
    events."""
    import ctypes
    import torch
    so = os.path.join(ROOT, "group_limited_top_amd", "libmoe_probe.so")
    lib = ctypes.CDLL(so)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    nbytes = 4 << 30
    buf = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    blocks, iters = 1024, 256
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def best(fn, reps):
        fn()
        torch.cuda.synchronize()
        ms = []
        for _ in range(reps):
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(b))
        return min(ms)

    def read():
        rc = lib.moe_probe_stream_read(ctypes.c_void_p(buf.data_ptr()), ctypes.c_size_t(nbytes),
                                       ctypes.c_void_p(sink.data_ptr()), 4096, stream)
        if rc != 0:
            raise RuntimeError(f"moe_probe_stream_read failed ({rc})")

    def mfma():
        rc = lib.moe_probe_mfma_bf16(ctypes.c_void_p(out.data_ptr()), blocks, iters, stream)
        if rc != 0:
            raise RuntimeError(f"moe_probe_mfma_bf16 failed ({rc})")

    gbs = nbytes / (best(read, 5) * 1e-3) / 1e9
    tflops = blocks * 4 * iters * 8 * 16384 / (best(mfma, 3) * 1e-3) / 1e12
    del buf
    return {"hbm_read_GBs": round(gbs, 1), "bf16_mfma_TFLOPs": round(tflops, 1),
            "how": "libmoe_probe: global->LDS DMA reads of 4 GiB (4 KiB a wave a round), best of 5; "
                   "8 independent v_mfma_f32_16x16x32_bf16 chains per wave, 4096 waves, best of 3"}


def gpu_clocks():
    """sclk / mclk levels (the current one is marked) and average power of this
    GPU, read from its sysfs files right after the timed region (no child
    process: reading files only); None where a file is not there."""
    import glob
    import torch
    try:
        pr = torch.cuda.get_device_properties(0)
        bdf = f"{pr.pci_domain_id:04x}:{pr.pci_bus_id:02x}:{pr.pci_device_id:02x}.0"
    except Exception:
        return None
    base = f"/sys/bus/pci/devices/{bdf}"
    out = {"pci": bdf}

    def current(name):
        try:
            for line in open(f"{base}/{name}"):
                if line.rstrip().endswith("*"):
                    return line.split(":", 1)[1].replace("*", "").strip()
        except OSError:
            return None
        return None

    out["sclk"] = current("pp_dpm_sclk")
    out["mclk"] = current("pp_dpm_mclk")
    for f in glob.glob(f"{base}/hwmon/hwmon*/power1_average") + glob.glob(f"{base}/hwmon/hwmon*/power1_input"):
        try:
            out["power_W"] = round(int(open(f).read()) / 1e6, 1)
            break
        except (OSError, ValueError):
            pass
    return out if (out.get("sclk") or out.get("power_W")) else None


def verify_logits_run(L, d, shape, xd, weights, ws, y_timed, counts_timed):
    """A forward that also writes the router logits must give the timed run's
    y and counts bit for bit (and the same choices as a plain forward)."""
    import torch
    dev = xd.device
    T, E, k = shape.T, shape.E, shape.top_k
    y0 = torch.empty_like(y_timed)
    y1 = torch.empty_like(y_timed)
    i0 = torch.empty(T, k, dtype=torch.int32, device=dev)
    i1 = torch.empty(T, k, dtype=torch.int32, device=dev)
    c1 = torch.empty_like(counts_timed)
    lg = torch.empty(T, E, dtype=torch.float32, device=dev)
    L.moe_layer_forward(d, xd, weights, y0, topk_idx_out=i0, ws=ws)
    d.flags |= L.MOE_F_WRITE_LOGITS
    L.moe_layer_forward(d, xd, weights, y1, topk_idx_out=i1, logits_out=lg, counts_out=c1, ws=ws)
    d.flags &= ~L.MOE_F_WRITE_LOGITS
    torch.cuda.synchronize()
    same = (torch.equal(y1.view(torch.int16), y_timed.view(torch.int16))
            and torch.equal(y0.view(torch.int16), y_timed.view(torch.int16))
            and torch.equal(i0, i1) and torch.equal(c1, counts_timed))
    return {"logits_run_bit_identical": bool(same),
            "what": "y, counts of a forward writing logits vs the timed run's; idx vs a plain forward"}


def bench_stack(L, shape, K, W):
    """The residual stack workload (independent layers, x <- RN(x + layer(
    RN(RMSNorm(x))))): K passes through all layers captured in one HIP graph,
    each pass starting from the same x (a 2-byte-per-element device copy
    inside the graph, ~0.5% of a pass).  Per-layer fractions use the layer's
    algorithmic FLOP and bytes with the counts of each layer's routing."""
    import torch
    dev = "cuda"
    nl = shape.layers
    layers = []
    for l in range(nl):
        _, wr, bias = synth_router(shape, l)
        w = synth_weights(shape, l)
        layers.append(dict(w, w_router=wr.to(dev), expert_bias=None if bias is None else bias.to(dev)))
    x0 = synth_router(shape, 0)[0].to(dev)
    d = L.desc_from_shape(shape)
    ws = L.alloc_workspace(d, dev)
    x = torch.empty_like(x0)
    counts = torch.empty(nl, shape.E, dtype=torch.int32, device=dev)
    for _ in range(max(W, 1)):
        x.copy_(x0)
        L.moe_stack_forward(d, x, layers, ws, counts_out=counts)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(K):
            x.copy_(x0)
            L.moe_stack_forward(d, x, layers, ws)
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    g.replay()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / K
    c = counts.cpu().numpy()
    work = [algorithmic_work(shape, c[l]) for l in range(nl)]
    flops = sum(wk["flops_layer"] for wk in work)
    nbytes = sum(wk["layer"] for wk in work)
    tf = flops / (ms * 1e-3) / 1e12
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"metric": METRIC, "value": round(shape.T / (ms * 1e-3), 1), "unit": "tokens/s",
            "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": round(ms, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": shape.dtype, "data": "synthetic",
            "config": {"workload": shape.name, "tokens": shape.T, "layers": nl, "hidden": shape.H,
                       "experts": shape.E, "top_k": shape.top_k, "moe_intermediate": shape.I,
                       "shared_intermediate": shape.I_shared},
            "step": f"one pass through {nl} layers (RMSNorm, MoE layer, residual each)",
            "ms_per_layer": round(ms / nl, 4),
            "layer_avg": {"tflops": round(tf, 2), "mfma_frac": round(tf / BF16_PEAK_TFLOPS, 4),
                          "hbm_GBs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                          "algorithmic_flops_per_layer": round(flops / nl),
                          "algorithmic_bytes_per_layer": round(nbytes / nl)}}


def synth_router(shape, layer):
    from group_limited_top_amd import synth
    return synth.router_inputs(shape, layer)


def synth_weights(shape, layer):
    from group_limited_top_amd import synth
    return synth.expert_weights(shape, device="cuda", layer=layer)


def cpu_baseline(shape, x, wr, bias, w, max_tokens):
    """The oracle as it stands: routing for every token, experts + combine for
    a bounded sample of tokens; throughput scaled to tokens/s.  The sample is
    the first `max_tokens` tokens, or for more than 16384 tokens the first
    `max_tokens` tokens t = 0 (mod 8) (an extrapolation from that sample).
    Up to 4096 tokens the same sample is also timed on one thread."""
    import numpy as np
    import oracle
    from group_limited_top_amd import synth

    nb = synth.to_numpy_bits
    xb, wrb = nb(x), wr.numpy()
    b = None if bias is None else bias.numpy()
    ow = [None if w[k] is None else nb(w[k])
          for k in ("w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down")]
    threads = oracle.default_threads()
    t0 = time.perf_counter()
    idx, tw, _, _ = oracle.route(xb, wrb, b, shape.n_group, shape.topk_group, shape.top_k,
                                 shape.scale, threads)
    t_route = time.perf_counter() - t0
    stride = 8 if shape.T > 16384 else 1
    tok = np.arange(0, shape.T, stride, dtype=np.int32)[:max_tokens]
    n = tok.size
    t0 = time.perf_counter()
    oracle.experts(xb, idx, tw, *ow, tokens=tok, nthreads=threads)
    t_exp = time.perf_counter() - t0
    per_token = t_route / shape.T + t_exp / n
    which = f"the first {n} tokens" if stride == 1 else f"{n} tokens t = 0 (mod 8), extrapolated"
    sample = (f"routing of all {shape.T} tokens ({t_route:.2f} s) + experts and combine of "
              f"{which} ({t_exp:.2f} s), scaled per token")
    cpu = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    out = {"value": round(1.0 / per_token, 2), "unit": "tokens/s", "cores": threads,
           "kind": "oracle", "sample": sample, "cpu_model": cpu, "nproc": os.cpu_count()}
    if shape.T <= 4096:
        # the same sample on one thread
        t0 = time.perf_counter()
        oracle.route(xb, wrb, b, shape.n_group, shape.topk_group, shape.top_k, shape.scale, 1)
        t_route1 = time.perf_counter() - t0
        n1 = min(n, 64)
        t0 = time.perf_counter()
        oracle.experts(xb, idx, tw, *ow, tokens=tok[:n1], nthreads=1)
        t_exp1 = time.perf_counter() - t0
        out["value_1thread"] = round(1.0 / (t_route1 / shape.T + t_exp1 / n1), 2)
        out["sample_1thread"] = f"routing of all {shape.T} tokens + experts and combine of {n1} tokens"
    return out


def bench_balance(L, d, shape, xd, weights, ws, K):
    """Load-balancing kernels at this workload: the auxiliary loss over the
    forward's router logits and counts, the expert-bias update, and the
    load statistics of a 19-layer tracking table (the model's MoE layers).
    Each is timed over K back-to-back calls with events on the stream the
    binding launches on; algorithmic bytes are what each call must read and
    write once."""
    import torch
    dev = xd.device
    T, E = shape.T, shape.E
    y = torch.empty(T, shape.H, dtype=shape.torch_dtype, device=dev)
    logits = torch.empty(T, E, dtype=torch.float32, device=dev)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    d.flags |= L.MOE_F_WRITE_LOGITS
    L.moe_layer_forward(d, xd, weights, y, logits_out=logits, counts_out=counts, ws=ws)
    d.flags &= ~L.MOE_F_WRITE_LOGITS
    aux_ws = L.aux_loss_workspace(T, E, dev)
    tracking = counts.to(torch.int64).repeat(19, 1).contiguous()
    load = torch.empty(19, E, dtype=torch.float32, device=dev)
    summ = torch.empty(19, L.MOE_NSTAT, dtype=torch.float64, device=dev)
    bias = torch.zeros(E, dtype=torch.float32, device=dev)
    aux_out = (torch.empty(E, dtype=torch.float64, device=dev),
               torch.empty(E, dtype=torch.float64, device=dev),
               torch.empty(1, dtype=torch.float64, device=dev))
    calls = {
        "aux_loss": (lambda: L.moe_aux_loss(logits, counts, aux_ws, aux_out),
                     T * E * 4 + E * 4 + 2 * E * 8 + 8),
        "bias_update": (lambda: L.moe_bias_update(counts, bias, bias, 1e-3), E * 4 * 3),
        "expert_stats_19_layers": (lambda: L.moe_expert_stats(tracking, shape.n_group, load, summ),
                                   19 * E * (8 + 4) + 19 * L.MOE_NSTAT * 8),
    }
    out = {}
    for name, (fn, nbytes) in calls.items():
        fn()
        torch.cuda.synchronize()
        # K calls captured in one HIP graph, so that host launch cost does not
        # space out kernels of a few microseconds
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(K):
                fn()
        g.replay()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) / K * 1e3
        gbs = nbytes / (us * 1e-6) / 1e9
        out[name] = {"us_per_call": round(us, 2), "algorithmic_bytes": nbytes,
                     "GBs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    return out


def bench_backward(L, d, shape, xd, weights, K):
    """The layer backward (moe_layer_backward) at this workload, for the
    routing the forward chose and a random bf16 upstream gradient: K calls
    captured in a HIP graph.  Algorithmic FLOP: the data and weight gradients
    of the three projections over all R = T*(k+1) expert rows (with the shared
    expert), 6 * 2*R*H*I; the kernels also recompute g and u (2 * 2*R*H*I more)
    instead of keeping them from the forward.  Bytes: the fp32 weight gradients
    written (every expert's, the shared expert's and the router's)."""
    import torch
    dev = xd.device
    T, H, E, I, Is, k = shape.T, shape.H, shape.E, shape.I, shape.I_shared, shape.top_k
    y = torch.empty(T, H, dtype=shape.torch_dtype, device=dev)
    logits = torch.empty(T, E, dtype=torch.float32, device=dev)
    idx = torch.empty(T, k, dtype=torch.int32, device=dev)
    ws = L.alloc_workspace(d, dev)
    d.flags |= L.MOE_F_WRITE_LOGITS
    L.moe_layer_forward(d, xd, weights, y, topk_idx_out=idx, logits_out=logits, ws=ws)
    d.flags &= ~L.MOE_F_WRITE_LOGITS
    g = torch.Generator(device="cpu").manual_seed(shape.seed + 77)
    dy = torch.randn(T, H, generator=g).to(shape.torch_dtype).to(dev)
    bws = L.backward_workspace(d, dev)
    out = L.moe_layer_backward(d, xd, weights, idx, logits, dy, ws=bws)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(K):
            L.moe_layer_backward(d, xd, weights, idx, logits, dy, ws=bws, out=out)
    graph.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    graph.replay()
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) / K * 1e3
    R = T * (k + (1 if Is else 0))
    flops = 6 * 2 * R * H * I
    flops_run = 8 * 2 * R * H * I
    grad_bytes = (3 * E * I * H + (3 * Is * H) + E * H) * 4
    tf = flops / (us * 1e-6) / 1e12
    return {"us_per_call": round(us, 1), "tokens_per_s": round(T / (us * 1e-6), 1),
            "algorithmic_flops": flops, "tflops": round(tf, 2),
            "mfma_frac": round(tf / BF16_PEAK_TFLOPS, 4),
            "executed_flops_incl_recompute": flops_run,
            "grad_bytes_written": grad_bytes,
            "grad_write_GBs": round(grad_bytes / (us * 1e-6) / 1e9, 1)}


TARGETS = {  # the layer fraction each regime is held to
    "hbm": ("layer_hbm_frac", 0.65),
    "mfma": ("layer_mfma_frac", 0.50),
}


def layer_inputs(L, shape, dev):
    """Seeded synthetic inputs of a single-layer workload, on the GPU."""
    from group_limited_top_amd import synth
    x, wr, bias = synth.router_inputs(shape)
    if shape.bias == "skew":
        bias = synth.skew_bias()
    w = synth.expert_weights(shape, device=dev)
    weights = dict(w, w_router=wr.to(dev), expert_bias=None if bias is None else bias.to(dev))
    return x, wr, bias, w, weights


def bench_layer(L, shape, K, W, eager=False, balance=True, backward=True, cpu=True,
                cpu_tokens=512, peaks=None):
    """One single-layer workload: K timed steps (see the module docstring).
    Returns the JSON object of that workload (the bench line's fields)."""
    import torch
    dev = "cuda"
    x, wr, bias, w, weights = layer_inputs(L, shape, dev)
    d = L.desc_from_shape(shape)
    xd = x.to(dev)
    # Weights that fit the 256 MB Infinity Cache would be read from it from the
    # second step on: such a layer's timed steps rotate over copies whose total
    # exceeds it (step i uses copy i mod n), so every step reads its weights
    # from HBM as the first one does.
    wbytes = sum(t.numel() * t.element_size() for t in weights.values() if t is not None)
    ncopy = 1 if wbytes >= MALL_BYTES else -(-3 * MALL_BYTES // (2 * wbytes)) + 1
    wsets = [weights] + [{k: (None if t is None else t.clone()) for k, t in weights.items()}
                         for _ in range(ncopy - 1)]
    y = torch.empty(shape.T, shape.H, dtype=shape.torch_dtype, device=dev)
    counts = torch.empty(shape.E, dtype=torch.int32, device=dev)
    ws = L.alloc_workspace(d, dev)
    stage = "gate_up"
    hev = HipEvents(2 * K)
    pairs = [(hev.ev[2 * i], hev.ev[2 * i + 1]) for i in range(K)]

    for i in range(W):
        L.moe_layer_forward(d, xd, wsets[i % ncopy], y, counts_out=counts, ws=ws)
    torch.cuda.synchronize()
    # timed region: K steps, each recording an event pair around the dominant
    # kernel on the library's stream
    t_start = torch.cuda.Event(enable_timing=True)
    t_stop = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t_start.record()
    for i in range(K):
        L.moe_layer_forward(d, xd, wsets[i % ncopy], y, counts_out=counts, ws=ws, timed_stage=stage,
                            events=pairs[i])
    t_stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t_start.elapsed_time(t_stop) / K
    kern_ms = sum(hev.elapsed_ms(a, b) for a, b in pairs) / K
    hev.close()
    # the same K steps with no event inside a step, for reference
    u0 = torch.cuda.Event(enable_timing=True)
    u1 = torch.cuda.Event(enable_timing=True)
    u0.record()
    for i in range(K):
        L.moe_layer_forward(d, xd, wsets[i % ncopy], y, counts_out=counts, ws=ws)
    u1.record()
    torch.cuda.synchronize()
    ms_step_plain = u0.elapsed_time(u1) / K
    ms_step_graph = None
    if not eager:
        # the K steps captured in one HIP graph and replayed: the same kernels,
        # without the per-launch host and dispatch cost
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(K):
                L.moe_layer_forward(d, xd, wsets[i % ncopy], y, counts_out=counts, ws=ws)
        g.replay()  # first replay uploads the graph
        torch.cuda.synchronize()
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        g0.record()
        g.replay()
        g1.record()
        torch.cuda.synchronize()
        ms_step_graph = g0.elapsed_time(g1) / K
        del g
    assert L.moe_status(ws) == 0
    clocks = gpu_clocks()
    verification = verify_logits_run(L, d, shape, xd, weights, ws, y, counts)

    work = algorithmic_work(shape, counts.cpu().numpy())
    ms_value = ms_step_graph if ms_step_graph is not None else ms_step
    tokens_per_s = shape.T / (ms_value * 1e-3)
    if shape.T >= 4096:
        achieved = work["flops_gate_up"] / (kern_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": None}
    else:
        achieved = work["k_gate_up"] / (kern_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None}
    if peaks:
        mp = peaks["bf16_mfma_TFLOPs"] if roof["bound"] == "mfma" else peaks["hbm_read_GBs"]
        roof["measured_peak"] = mp
        roof["frac_vs_measured"] = round(roof["achieved"] / mp, 4)
    kname = L.moe_stage_kernel(d, stage)
    roof["traffic"] = measured_traffic(shape.name, kname)
    roof.update(kernel=kname,
                kernel_ms=round(kern_ms, 4), algorithmic_bytes=work["k_gate_up"],
                algorithmic_flops=work["flops_gate_up"])
    layer_hbm = work["layer"] / (ms_value * 1e-3) / 1e9
    layer_tflops = work["flops_layer"] / (ms_value * 1e-3) / 1e12
    layer = {"algorithmic_bytes": work["layer"], "algorithmic_flops": work["flops_layer"],
             "hbm_GBs": round(layer_hbm, 1), "hbm_frac": round(layer_hbm / HBM_PEAK_GBS, 4),
             "tflops": round(layer_tflops, 2),
             "mfma_frac": round(layer_tflops / BF16_PEAK_TFLOPS, 4),
             "experts_hit": work["hit"], "max_expert_rows": int(counts.max().item())}
    tname, tval = TARGETS[roof["bound"]]
    got = layer["mfma_frac"] if roof["bound"] == "mfma" else layer["hbm_frac"]
    out = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": K, "warmup": W, "ms_per_step": round(ms_value, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": shape.dtype, "data": "synthetic",
        "config": {"workload": shape.name, "tokens": shape.T, "hidden": shape.H,
                   "experts": shape.E, "n_group": shape.n_group, "topk_group": shape.topk_group,
                   "top_k": shape.top_k, "moe_intermediate": shape.I,
                   "shared_intermediate": shape.I_shared, "expert_bias": shape.bias,
                   "weight_copies": ncopy},
        "roofline": roof,
        "layer": layer,
        "target": {tname: tval, "achieved": got, "met": bool(got >= tval),
                   "ms_per_step_at_target": round(
                       (work["flops_layer"] / (tval * BF16_PEAK_TFLOPS * 1e12) if roof["bound"] == "mfma"
                        else work["layer"] / (tval * HBM_PEAK_GBS * 1e9)) * 1e3, 4)},
        "clocks_after_timed_region": clocks,
        "verification": verification,
        "wall_s_timed": round(wall, 4),
        "timing": {"value_from": "graph" if ms_step_graph is not None else "eager",
                   "ms_per_step_graph": None if ms_step_graph is None else round(ms_step_graph, 4),
                   "ms_per_step_eager_with_kernel_events": round(ms_step, 4),
                   "ms_per_step_eager": round(ms_step_plain, 4)},
    }
    if balance:
        out["balance"] = bench_balance(L, d, shape, xd, weights, ws, K)
    if backward and shape.dtype == "bf16":
        out["backward"] = bench_backward(L, d, shape, xd, weights, min(K, 10))
    del ws, wsets, y
    torch.cuda.empty_cache()
    if cpu:
        out["cpu_baseline"] = cpu_baseline(shape, x, wr, bias, w, cpu_tokens)
    return out


# The default run: the 512-token layer (HBM-bound weight stream) is the
# headline; the 16384-token layer with bias and the 65536-token skewed layer
# (the MFMA regime) and the small fp32 layer are measured in the same run,
# each with its own roofline and CPU baseline (all cores, plus one thread for
# the fp32 layer).
EXTRA_WORKLOADS = (("large_batch", "full_t16k_bias"), ("skew", "skew_t64k"), ("fp32", "tiny_f32"))


def library_gemm(L, synth, reps=20):
    """Context for the 16384-token layer's MFMA fraction: what the platform's
    BLAS (torch bf16 matmul / bmm, i.e. hipBLASLt) reaches on this GPU on a
    dense 8192^3 product and on the per-expert products of a perfectly
    balanced routing (256 experts x 512 rows, contiguous rows, operands in the
    library's preferred layout, no gather, no SwiGLU, no combine), beside
    libmoe's moe_permute + moe_experts on that same balanced routing (gathered
    rows, SwiGLU, shared expert and combine included).  Event-timed mean of
    `reps` calls after 3 untimed ones."""
    import torch
    dev = "cuda"

    # operands drawn like the layer's own inputs (synth): token rows N(0, 1)
    # from the CPU generator, weights N(0, 0.02) from the GPU generator (the
    # MFMA rate under load depends on the operand bits: the clock is power
    # limited, and zero operands run faster)
    def tokens(*s):
        return synth._normal(s, 1.0, 11, "cpu", torch.bfloat16).to(dev)

    def weights(*s):
        return synth._normal(s, 0.02, 12, dev, torch.bfloat16)

    def mean_ms(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    def entry(flop, ms):
        return {"us": round(ms * 1e3, 1), "tflops": round(flop / (ms * 1e-3) / 1e12, 1),
                "mfma_frac": round(flop / (ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12), 4)}

    out = {"what": "bf16; library = torch.matmul / torch.bmm (hipBLASLt), "
                   "libmoe = moe_permute + moe_experts through the C ABI"}
    n = 8192
    A, B = tokens(n, n), weights(n, n)
    out["library_dense_8192"] = entry(2 * n ** 3, mean_ms(lambda: torch.matmul(A, B)))
    del A, B
    shape = synth.WORKLOADS["full_t16k_bias"]
    T, H, E, K, I, Is = shape.T, shape.H, shape.E, shape.top_k, shape.I, shape.I_shared
    M = T * K // E
    xe, wgu = tokens(E, M, H), weights(E, H, 2 * I)  # gate and up side by side
    flop_gu = 2 * E * M * H * 2 * I
    out["library_bmm_gate_up"] = entry(flop_gu, mean_ms(lambda: torch.bmm(xe, wgu)))
    xe.zero_()
    wgu.zero_()
    out["library_bmm_gate_up_zero_operands"] = entry(flop_gu, mean_ms(lambda: torch.bmm(xe, wgu)))
    del xe, wgu
    he, wd = tokens(E, M, I), weights(E, I, H)
    out["library_bmm_down"] = entry(2 * E * M * I * H, mean_ms(lambda: torch.bmm(he, wd)))
    del he, wd
    # libmoe on the balanced routing: pair p = t K + j goes to expert p mod E
    # (E divides T K: every expert gets T K / E rows, a token's K experts differ)
    d = L.desc_from_shape(shape)
    w = synth.expert_weights(shape, device=dev)
    x = synth.router_inputs(shape)[0].to(dev)
    idx = (torch.arange(T * K, dtype=torch.int32, device=dev) % E).view(T, K)
    topk_w = torch.full((T, K), 1.0 / K, dtype=torch.float32, device=dev)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    sp = torch.empty(T * K, dtype=torch.int32, device=dev)
    ps = torch.empty(T * K, dtype=torch.int32, device=dev)
    y = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    ws = L.alloc_workspace(d, dev)

    def ours():
        L.moe_permute(d, idx, counts, offsets, sp, ps, None, ws)
        L.moe_experts(d, x, topk_w, offsets, sp, ps, w, y, ws)

    flop = 2 * 3 * H * (T * K * I + T * Is)
    out["libmoe_experts_balanced"] = entry(flop, mean_ms(ours))
    out["libmoe_experts_balanced"]["rows_per_expert"] = int(counts.min().item())
    out["libmoe_experts_balanced"]["kernels"] = [L.moe_stage_kernel(d, s) for s in ("gate_up", "down")]
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None,
                    help="one workload only (default: the 512-token headline plus the "
                         "16384- and 65536-token layers and the fp32 layer)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="time steps launched one by one instead of a HIP graph of K steps")
    ap.add_argument("--cpu-tokens", type=int, default=512)
    ap.add_argument("--no-backward", action="store_true", help="skip timing the layer backward")
    ap.add_argument("--no-extra-workloads", action="store_true",
                    help="with the default workload: skip the 16384- and 65536-token and fp32 layers")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip measuring the streaming-read and MFMA rates of this GPU")
    ap.add_argument("--backward-only", action="store_true",
                    help="only time the layer backward (prints its JSON object, not the bench line)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (3 times), to scale the "
                         "FETCH_SIZE / WRITE_SIZE counters of a profiler run")
    ap.add_argument("--write-traffic", nargs=4, default=None,
                    metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="no GPU: turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs of this "
                         "workload and of --copy-calibration into profiles/traffic.json")
    ap.add_argument("--profile-note", default="", help="with --write-traffic: the summary file")
    ap.add_argument("--library-gemm", action="store_true",
                    help="only compare torch's bf16 GEMMs (hipBLASLt) with libmoe's experts on a "
                         "balanced 16384-token routing (prints its JSON object)")
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(args.workload or "full_t512", *args.write_traffic,
                      args.copy_calibration or 1024, args.profile_note)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this layer's data-parallel share needs no "
              f"exchange); --gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        n = args.copy_calibration * 2 ** 20
        a = torch.ones(n, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)
        return
    from group_limited_top_amd import _lib as L
    from group_limited_top_amd import synth

    torch.cuda.set_device(0)
    if args.library_gemm:
        print(json.dumps({"library_gemm": library_gemm(L, synth)}), flush=True)
        return
    shape = synth.WORKLOADS[args.workload or "full_t512"]
    if shape.layers != 1:
        print(json.dumps(bench_stack(L, shape, min(args.steps, 10), min(args.warmup, 2))), flush=True)
        return
    if args.backward_only:
        _, _, _, _, weights = layer_inputs(L, shape, "cuda")
        x = synth.router_inputs(shape)[0].to("cuda")
        d = L.desc_from_shape(shape)
        print(json.dumps({"workload": shape.name,
                          "backward": bench_backward(L, d, shape, x, weights, min(args.steps, 10))}),
              flush=True)
        return
    peaks = None if args.no_peaks else measure_peaks()
    out = bench_layer(L, shape, args.steps, args.warmup, eager=args.eager,
                      backward=not args.no_backward, cpu=not args.no_cpu_baseline,
                      cpu_tokens=args.cpu_tokens, peaks=peaks)
    out["peaks_measured"] = peaks
    if args.workload is None and not args.no_extra_workloads:
        for key, name in EXTRA_WORKLOADS:
            out[key] = bench_layer(L, synth.WORKLOADS[name], min(args.steps, 20),
                                   min(args.warmup, 5), eager=args.eager, balance=False,
                                   backward=False,
                                   cpu=not args.no_cpu_baseline, cpu_tokens=args.cpu_tokens,
                                   peaks=peaks)
            for k in ("metric", "unit", "n_gpus", "higher_is_better", "scaling", "vs_baseline",
                      "data"):
                out[key].pop(k)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
