"""Throughput of the MoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload full_t512]

One step = one moe_layer_forward (router, selection, permute, gate/up +
SwiGLU, down, combine; shared expert included) over one batch of synthetic
tokens already resident in HBM.  Prints one JSON line.  Besides tokens/s it
reports the roofline of the dominant kernel (its algorithmic bytes or flops per
launch over its average duration, timed with HIP events recorded on the
library's stream around that kernel in every timed step) and the CPU oracle
timed on this host (`cpu_baseline`).
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
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s


def algorithmic_work(shape, counts):
    """Per-launch algorithmic bytes (and flops) of the kernels and the layer.

    Bytes count what the method must move at least once: the weights of every
    expert that received a token, the shared expert, the router weight, x, y
    and the routing outputs.  Intermediates (hidden activations, per-pair
    outputs) are excluded from the layer figure; the kernel figures count the
    kernel's own inputs and outputs once."""
    T, H, I, Is, K, E = shape.T, shape.H, shape.I, shape.I_shared, shape.top_k, shape.E
    elt = 2 if shape.dtype == "bf16" else 4
    hit = int((counts > 0).sum())
    P = T * K
    gate_up_w = (hit * 2 * I * H + 2 * Is * H) * elt
    down_w = (hit * I * H + Is * H) * elt
    k_gate_up = gate_up_w + T * H * elt + (P * I + T * Is) * elt
    k_down = down_w + (P * I + T * Is) * elt + (P + (T if Is else 0)) * H * elt
    layer = (gate_up_w + down_w + E * H * 4 + 2 * T * H * elt + P * 8)
    flops_gate_up = 2.0 * 2 * (P * I + T * Is) * H
    flops_down = 2.0 * (P * I + T * Is) * H
    flops_router = 2.0 * T * E * H
    return dict(hit=hit, k_gate_up=k_gate_up, k_down=k_down, layer=layer,
                flops_gate_up=flops_gate_up, flops_down=flops_down,
                flops_layer=flops_gate_up + flops_down + flops_router)


def cpu_baseline(shape, x, wr, bias, w, max_tokens):
    """The oracle as it stands: routing for every token, experts + combine for
    the first `max_tokens` tokens; throughput scaled to tokens/s."""
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
    n = min(max_tokens, shape.T)
    tok = np.arange(n, dtype=np.int32)
    t0 = time.perf_counter()
    oracle.experts(xb, idx, tw, *ow, tokens=tok, nthreads=threads)
    t_exp = time.perf_counter() - t0
    per_token = t_route / shape.T + t_exp / n
    sample = (f"routing of all {shape.T} tokens ({t_route:.2f} s) + experts and combine of "
              f"{n} tokens ({t_exp:.2f} s), scaled per token")
    return {"value": round(1.0 / per_token, 2), "unit": "tokens/s", "cores": threads,
            "kind": "oracle", "sample": sample}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="full_t512")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=512)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this layer's data-parallel share needs no "
              f"exchange); --gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    from group_limited_top_amd import _lib as L
    from group_limited_top_amd import synth

    shape = synth.WORKLOADS[args.workload]
    if shape.layers != 1:
        raise SystemExit("bench.py times single-layer workloads")
    dev = "cuda"
    torch.cuda.set_device(0)
    x, wr, bias = synth.router_inputs(shape)
    if shape.bias == "skew":
        bias_path = os.path.join(ROOT, "tests", "golden", "skew_t64k_expert_bias.txt")
        import numpy as np
        bias = torch.from_numpy(np.loadtxt(bias_path, dtype=np.float32))
    w = synth.expert_weights(shape, device=dev)
    d = L.desc_from_shape(shape)
    weights = dict(w, w_router=wr.to(dev), expert_bias=None if bias is None else bias.to(dev))
    xd = x.to(dev)
    y = torch.empty(shape.T, shape.H, dtype=shape.torch_dtype, device=dev)
    counts = torch.empty(shape.E, dtype=torch.int32, device=dev)
    ws = L.alloc_workspace(d, dev)
    stage = "gate_up"
    K, W = args.steps, args.warmup
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(K)]
    for a, b in evs:  # create the underlying HIP events before handing them over
        a.record()
        b.record()
    torch.cuda.synchronize()

    for _ in range(W):
        L.moe_layer_forward(d, xd, weights, y, counts_out=counts, ws=ws)
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_stop = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t_start.record()
    for i in range(K):
        L.moe_layer_forward(d, xd, weights, y, counts_out=counts, ws=ws, timed_stage=stage,
                            events=evs[i])
    t_stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = t_start.elapsed_time(t_stop)
    ms_step = ms_total / K
    kern_ms = sum(a.elapsed_time(b) for a, b in evs) / K
    assert L.moe_status(ws) == 0

    work = algorithmic_work(shape, counts.cpu().numpy())
    tokens_per_s = shape.T / (ms_step * 1e-3)
    if shape.T >= 4096:
        achieved = work["flops_gate_up"] / (kern_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": None}
    else:
        achieved = work["k_gate_up"] / (kern_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None}
    roof.update(kernel="k_gateup_bf16" if shape.dtype == "bf16" else "k_gateup_f32",
                kernel_ms=round(kern_ms, 4), algorithmic_bytes=work["k_gate_up"],
                algorithmic_flops=work["flops_gate_up"])
    layer_hbm = work["layer"] / (ms_step * 1e-3) / 1e9
    layer_tflops = work["flops_layer"] / (ms_step * 1e-3) / 1e12
    out = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": K, "warmup": W, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": shape.dtype, "data": "synthetic",
        "config": {"workload": shape.name, "tokens": shape.T, "hidden": shape.H,
                   "experts": shape.E, "n_group": shape.n_group, "topk_group": shape.topk_group,
                   "top_k": shape.top_k, "moe_intermediate": shape.I,
                   "shared_intermediate": shape.I_shared, "expert_bias": shape.bias},
        "roofline": roof,
        "layer": {"algorithmic_bytes": work["layer"], "hbm_GBs": round(layer_hbm, 1),
                  "hbm_frac": round(layer_hbm / HBM_PEAK_GBS, 4), "tflops": round(layer_tflops, 2),
                  "mfma_frac": round(layer_tflops / BF16_PEAK_TFLOPS, 4),
                  "experts_hit": work["hit"]},
        "wall_s_timed": round(wall, 4),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(shape, x, wr, bias, w, args.cpu_tokens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
