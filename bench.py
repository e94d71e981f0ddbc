"""Benchmark: biased grouped top-k routing on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step = one call of route_biased_grouped_topk over the whole batch of
router logits (sigmoid + correction bias, 8 groups of 32 of 256 experts,
top-4 groups, top-8 experts, renormalised; bf16 logits, M = 65536 tokens).
Inputs are seeded synthetic data already resident in device memory.  The
call rotates over several identical input/output sets whose total size is
far larger than the 256 MB last-level cache, so each call reads its logits
from HBM.  Prints one JSON line on stdout; details go to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

METRIC = "routed tokens/s + HBM GB/s at M=64K E=256 K=8; µs/call at M=64"
HBM_PEAK_GBPS = 8000.0
WORKLOAD = "biased_grouped_e256"


# HBM bytes per launch of the headline kernel, from rocprofv3 FETCH_SIZE and
# WRITE_SIZE runs scaled by a plain copy of known size; valid only for the
# kernel sources they were taken on.
TRAFFIC_FILE = os.path.join(HERE, "profiles", "route_fast_biased_grouped_e256_m65536_traffic.txt")
KERNEL_SOURCES = ("route_fast.hip", "route_tile.hpp", "route_common.hpp")


def kernel_source_digest():
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(HERE, "moe_expert_routing_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """Bytes per launch (fetch + write) if the stored counters match these sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            kv = dict(l.split("=", 1) for l in f if "=" in l and not l.startswith("#"))
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv.get("source_sha256") != kernel_source_digest():
        return None
    return float(kv["fetch_bytes_per_launch"]) + float(kv["write_bytes_per_launch"])


def copy_calibration(nbytes=1 << 30, reps=5):
    """A plain device copy of known size, for scaling the HBM byte counters."""
    import torch
    dev = torch.device("cuda", 0)
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "reps": reps}),
          flush=True)


def eprint(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(M, E, K, logit_bytes, bias=True):
    """One read of the logits (and the bias), one write of weights + ids."""
    return M * E * logit_bytes + M * K * 8 + (E * 4 if bias else 0)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_cores():
    """Cores this process may run on, at most 16 (the host share of one GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(wl, budget_s=12.0, gpu_out=None):
    """The oracle as it stands on the same workload, timed on the host: one
    core, then the rows split over every core (one thread per core, each
    calling the oracle on its rows; the oracle's C routine releases the GIL).
    With gpu_out = (weights, ids) of the GPU on this batch, an untimed oracle
    pass is also compared with it row by row, and the counts (exact rows,
    near-tie rows by class, failures) are returned."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle
    from workloads import make_bias, make_logits

    x = make_logits(wl)
    b = make_bias(wl)
    M = x.shape[0]
    args = dict(scoring=oracle.SIGMOID, bias=b, num_expert_group=wl.G, topk_group=wl.TG,
                group_rule=oracle.GROUP_TOP2SUM, renormalize=wl.renormalize)

    def run_rows(lo, hi):
        return oracle.route(x[lo:hi], wl.K, **args)

    # one core: full passes over the batch for half the budget
    t0 = time.perf_counter()
    reps = 0
    while True:
        run_rows(0, M)
        reps += 1
        if time.perf_counter() - t0 >= budget_s / 2:
            break
    one = reps * M / (time.perf_counter() - t0)
    # every core: the batch split into one row range per thread
    n = host_cores()
    bounds = [(M * i // n, M * (i + 1) // n) for i in range(n)]
    t0 = time.perf_counter()
    reps_all = 0
    with ThreadPoolExecutor(n) as ex:
        while True:
            list(ex.map(lambda r: run_rows(*r), bounds))
            reps_all += 1
            if time.perf_counter() - t0 >= budget_s / 2:
                break
    dt_all = time.perf_counter() - t0
    res = {"value": reps_all * M / dt_all, "unit": "tokens/s", "cores": n, "kind": "oracle",
           "sample": f"{reps_all} full passes over the {M}-token batch split over {n} threads "
                     f"({dt_all:.1f} s); one core: {reps} passes at {one:.0f} tokens/s "
                     f"(C oracle in double precision)",
           "one_core_value": one, "cpu_model": cpu_model(), "host_cpus": os.cpu_count()}
    parity = None
    if gpu_out is not None:
        sys.path.insert(0, os.path.join(HERE, "tests"))
        from parity_check import compare
        rep = compare(x, gpu_out[0], gpu_out[1], scoring=oracle.SIGMOID, bias=b, G=wl.G,
                      TG=wl.TG, rule=oracle.GROUP_TOP2SUM, K=wl.K, renorm=wl.renormalize)
        parity = {"rows": rep.rows, "exact": rep.exact, "near_tie_k": rep.near_tie_k,
                  "near_tie_order": rep.near_tie_order, "near_tie_group": rep.near_tie_group,
                  "failures": len(rep.failures)}
    del np
    return res, parity


def _events(n):
    import torch
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


def time_calls(launch, n_sets, stream, steps=400, warmup=40):
    """Mean per-call time (us) of back-to-back launches, and mean kernel time
    (us) from an event pair around each launch; launch(i) runs set i % n_sets."""
    import numpy as np
    import torch
    for i in range(warmup):
        launch(i % n_sets)
    torch.cuda.synchronize()
    e0, e1 = _events(2)
    e0.record(stream)
    for i in range(steps):
        launch(i % n_sets)
    e1.record(stream)
    torch.cuda.synchronize()
    per_call = e0.elapsed_time(e1) * 1e3 / steps
    ev = _events(2 * min(steps, 200))
    for i in range(len(ev) // 2):
        ev[2 * i].record(stream)
        launch(i % n_sets)
        ev[2 * i + 1].record(stream)
    torch.cuda.synchronize()
    kern = float(np.mean([ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(len(ev) // 2)]))
    return per_call, kern * 1e3


def measure_all(out_path=None):
    """Every workload: each config, the biased-grouped M sweep, the fused
    routers (7168-wide at 8192 and few tokens, 8 experts), dispatch metadata
    and the post-routing steps."""
    import numpy as np
    import torch

    import moe_expert_routing_amd as mr
    from workloads import (BIASED_GROUPED_M_SWEEP, WORKLOADS, make_bias, make_logits,
                           make_router_inputs)
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream(dev)

    def dev_tensor(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    results = []

    def routing_case(name, M=None):
        wl = WORKLOADS[name]
        x = dev_tensor(make_logits(wl, M))
        M = x.shape[0]
        b = make_bias(wl)
        b = None if b is None else dev_tensor(b)
        lb = 4 if wl.dtype == "f32" else 2
        nbytes = algorithmic_bytes(M, wl.E, wl.K, lb, bias=b is not None)
        n_sets = max(1, min(64, -(-512 * 2**20 // (M * (wl.E * lb + 8 * wl.K)))))
        xs = [x] + [x.clone() for _ in range(n_sets - 1)]
        outs = [(torch.empty(M, wl.K, device=dev), torch.empty(M, wl.K, dtype=torch.int32,
                                                               device=dev)) for _ in range(n_sets)]

        def launch(i):
            w, ids = outs[i]
            if wl.entry == "route_topk_softmax":
                mr.route_topk_softmax(xs[i], wl.K, wl.renormalize, w, ids, stream=stream)
            elif wl.entry == "route_grouped_topk":
                mr.route_grouped_topk(xs[i], wl.K, wl.G, wl.TG, wl.renormalize, wl.scoring, w, ids,
                                      stream=stream)
            else:
                mr.route_biased_grouped_topk(xs[i], b, wl.K, wl.G, wl.TG, wl.renormalize, w, ids,
                                             stream=stream)
        per_call, kern = time_calls(launch, n_sets, stream)
        r = {"workload": name, "entry": wl.entry, "M": M, "E": wl.E, "K": wl.K, "G": wl.G,
             "TG": wl.TG, "logits": wl.dtype, "rotating_sets": n_sets,
             "us_per_call": per_call, "kernel_us": kern, "tokens_per_s": M / (per_call * 1e-6),
             "alg_bytes": nbytes, "GBps_kernel": nbytes / (kern * 1e-6) / 1e9,
             "frac_hbm_kernel": nbytes / (kern * 1e-6) / 1e9 / HBM_PEAK_GBPS}
        results.append(r)
        eprint(json.dumps(r))

    routing_case("softmax_e8_k2")
    routing_case("sigmoid_bias_e256_k8")
    routing_case("grouped_softmax_e160")
    for M in BIASED_GROUPED_M_SWEEP:
        routing_case("biased_grouped_e256", M)
    results.append(steady_state_case(stream))
    eprint(json.dumps(results[-1]))

    wl = WORKLOADS["fused_router_h7168"]
    hidden, w = make_router_inputs(wl)
    hd, wd = dev_tensor(hidden), dev_tensor(w)
    bd = dev_tensor(make_bias(wl))
    M, H, E = wl.M, wl.hidden_dim, wl.E
    n_sets = 5
    hs = [hd] + [hd.clone() for _ in range(n_sets - 1)]
    outs = [(torch.empty(M, wl.K, device=dev), torch.empty(M, wl.K, dtype=torch.int32,
                                                           device=dev)) for _ in range(n_sets)]

    ws_fr = torch.empty(max(mr.route_fused_router_workspace_size(M, H, E), 16),
                        dtype=torch.uint8, device=dev)

    def launch_fr(i, ws_arg=ws_fr):
        mr.route_fused_router(hs[i], wd, wl.K, wl.G, wl.TG, wl.renormalize, "sigmoid", bd,
                              "top2sum", outs[i][0], outs[i][1], stream=stream,
                              workspace=ws_arg)
    # the library's default for this shape (four hidden splits of 128-row
    # tiles with partial logits in the workspace), then the single fused kernel
    per_call, kern = time_calls(launch_fr, n_sets, stream, steps=200, warmup=20)
    per_call_one, kern_one = time_calls(lambda i: launch_fr(i, False), n_sets, stream,
                                        steps=200, warmup=20)
    # context: the unfused pair, torch's bf16 matmul (hipBLASLt) to bf16
    # logits, then the routing kernel
    lgs = [torch.empty(M, E, dtype=torch.bfloat16, device=dev) for _ in range(n_sets)]

    def launch_unfused(i):
        with torch.cuda.stream(stream):
            torch.matmul(hs[i], wd, out=lgs[i])
        mr.route_biased_grouped_topk(lgs[i], bd, wl.K, wl.G, wl.TG, wl.renormalize,
                                     outs[i][0], outs[i][1], stream=stream)
    per_call_unfused, _ = time_calls(launch_unfused, n_sets, stream, steps=100, warmup=10)
    nbytes = M * H * 2 + H * E * 2 + E * 4 + M * wl.K * 8
    flops = 2.0 * M * H * E
    r = {"workload": wl.name, "entry": wl.entry, "M": M, "H": H, "E": E, "K": wl.K,
         "rotating_sets": n_sets, "us_per_call": per_call, "kernel_us": kern,
         "us_per_call_one_kernel": per_call_one, "kernel_us_one_kernel": kern_one,
         "us_per_call_torch_matmul_then_routing": per_call_unfused,
         "tokens_per_s": M / (per_call * 1e-6), "alg_bytes": nbytes,
         "GBps_kernel": nbytes / (kern * 1e-6) / 1e9,
         "frac_hbm_kernel": nbytes / (kern * 1e-6) / 1e9 / HBM_PEAK_GBPS,
         "TFLOPs_kernel": flops / (kern * 1e-6) / 1e12,
         "frac_mfma_bf16_kernel": flops / (kern * 1e-6) / 2.5e15}
    results.append(r)
    eprint(json.dumps(r))
    def graph_us(fn, n=20, reps=5):
        """Per-call time (us) of fn from a replayed HIP graph of n calls:
        kernel time plus the gaps between kernels, without host launch cost."""
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for _ in range(3):
                fn(side)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                for _ in range(n):
                    fn(side)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = _events(2)
            e0.record(stream)
            g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3 / n)
        return float(np.median(ts))

    # few tokens through the 7168-wide router: split path (workspace) and
    # the single fused kernel, graph replay
    for Ms in (1, 64, 1024, 2048, 4096):
        xs_ = hd[:Ms].contiguous()
        o_ = (torch.empty(Ms, wl.K, device=dev), torch.empty(Ms, wl.K, dtype=torch.int32,
                                                            device=dev))
        need = mr.route_fused_router_workspace_size(Ms, H, E)
        wsp = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)

        def fr_call(st, ws_arg):
            mr.route_fused_router(xs_, wd, wl.K, wl.G, wl.TG, wl.renormalize, "sigmoid", bd,
                                  "top2sum", o_[0], o_[1], stream=st, workspace=ws_arg)
        t_split = graph_us(lambda st: fr_call(st, wsp))
        t_one = graph_us(lambda st: fr_call(st, False))
        lg_ = torch.empty(Ms, E, dtype=torch.bfloat16, device=dev)

        def unfused_few(st):
            torch.matmul(xs_, wd, out=lg_)
            mr.route_biased_grouped_topk(lg_, bd, wl.K, wl.G, wl.TG, wl.renormalize, o_[0],
                                         o_[1], stream=st)
        t_unfused = graph_us(unfused_few)
        r = {"workload": "fused_router_h7168_few_tokens", "entry": wl.entry, "M": Ms, "H": H,
             "E": E, "K": wl.K, "splits": need // (4 * E * Ms) if need else 1,
             "tile_rows": 64 if Ms > 2048 else 32,
             "us_per_call_graph_split": t_split, "us_per_call_graph_one_kernel": t_one,
             "us_per_call_graph_torch_matmul_then_routing": t_unfused}
        results.append(r)
        eprint(json.dumps(r))

    # few experts: 8-expert router (hidden 4096, top-2 softmax, cap 30) and
    # 16-expert router (hidden 6144, top-4 softmax, renormalised)
    for wl8, Ms in [(WORKLOADS[n], m) for n in ("fused_router_e8_h4096", "fused_router_e16_h6144")
                    for m in (1, 64, 2048, 8192)]:
        if Ms == 1:
            h8, w8 = make_router_inputs(wl8)
            h8d, w8d = dev_tensor(h8), dev_tensor(w8)
        xs_ = h8d[:Ms].contiguous()
        o_ = (torch.empty(Ms, wl8.K, device=dev), torch.empty(Ms, wl8.K, dtype=torch.int32,
                                                             device=dev))

        def sr_call(st):
            mr.route_fused_router(xs_, w8d, wl8.K, 1, 1, wl8.renormalize, wl8.scoring, None,
                                  "max", o_[0], o_[1], stream=st, logit_softcap=wl8.softcap)
        t = graph_us(sr_call)
        # context: the unfused pair, torch's bf16 matmul (hipBLASLt) then the
        # routing kernel, without the cap
        lg = torch.empty(Ms, wl8.E, dtype=torch.bfloat16, device=dev)

        def unfused(st):
            torch.matmul(xs_, w8d, out=lg)
            mr.route_topk_softmax(lg, wl8.K, wl8.renormalize, o_[0], o_[1], stream=st)
        t_unfused = graph_us(unfused)
        nbytes = Ms * wl8.hidden_dim * 2 + wl8.hidden_dim * wl8.E * 2 + Ms * wl8.K * 8
        r = {"workload": wl8.name, "entry": wl8.entry, "M": Ms, "H": wl8.hidden_dim,
             "E": wl8.E, "K": wl8.K, "softcap": wl8.softcap, "us_per_call_graph": t,
             "us_per_call_graph_torch_matmul_then_routing": t_unfused,
             "alg_bytes": nbytes, "GBps": nbytes / (t * 1e-6) / 1e9,
             "note": "warm (graph replay of one input set)"}
        if Ms == wl8.M:
            sets8 = [xs_] + [xs_.clone() for _ in range(4)]
            outs8 = [(torch.empty(Ms, wl8.K, device=dev),
                      torch.empty(Ms, wl8.K, dtype=torch.int32, device=dev)) for _ in range(5)]

            def launch8(i):
                mr.route_fused_router(sets8[i], w8d, wl8.K, 1, 1, wl8.renormalize, wl8.scoring,
                                      None, "max", outs8[i][0], outs8[i][1], stream=stream,
                                      logit_softcap=wl8.softcap)
            per_call, kern = time_calls(launch8, 5, stream, steps=200, warmup=20)
            r.update({"rotating_sets": 5, "us_per_call_cold": per_call,
                      "GBps_cold": nbytes / (per_call * 1e-6) / 1e9,
                      "frac_hbm_cold": nbytes / (per_call * 1e-6) / 1e9 / HBM_PEAK_GBPS})
        results.append(r)
        eprint(json.dumps(r))

    # dispatch metadata of the 65536-token biased grouped routing output
    wl = WORKLOADS["biased_grouped_e256"]
    xb = dev_tensor(make_logits(wl))
    bb = dev_tensor(make_bias(wl))
    rw, rids = mr.route_biased_grouped_topk(xb, bb, wl.K, wl.G, wl.TG, wl.renormalize)
    n_sets = 8
    ids_sets = [rids] + [rids.clone() for _ in range(n_sets - 1)]
    w_sets = [rw] + [rw.clone() for _ in range(n_sets - 1)]
    ws = torch.empty(mr.route_dispatch_workspace_size(wl.M, wl.K, wl.E), dtype=torch.uint8,
                     device=dev)

    n = wl.M * wl.K
    outs = [(torch.empty(wl.E, dtype=torch.int32, device=dev),
             torch.empty(wl.E + 1, dtype=torch.int32, device=dev),
             torch.empty(n, dtype=torch.int32, device=dev),
             torch.empty(n, dtype=torch.int32, device=dev),
             torch.empty(n, dtype=torch.float32, device=dev)) for _ in range(n_sets)]

    def launch_disp(i):
        mr.route_dispatch_metadata(ids_sets[i], wl.E, w_sets[i], workspace=ws, stream=stream,
                                   out=outs[i])
    per_call, kern = time_calls(launch_disp, n_sets, stream, steps=200, warmup=20)
    nbytes = 2 * n * 4 + n * 4 + 3 * n * 4 + 2 * wl.E * 4  # ids twice, weights; 3 outputs
    r = {"workload": "dispatch_metadata_e256_m65536", "entry": "route_dispatch_metadata",
         "M": wl.M, "K": wl.K, "E": wl.E, "rotating_sets": n_sets, "us_per_call": per_call,
         "kernel_us": kern, "alg_bytes": nbytes, "GBps_kernel": nbytes / (kern * 1e-6) / 1e9,
         "note": "two kernels per call at this size (three when the coarse count matrix "
                 "exceeds 16384 counts); outputs and workspace preallocated"}
    results.append(r)
    eprint(json.dumps(r))
    # post-routing steps on the 65536 x 8 routing output (in place)
    n_sets = 16
    shared = torch.randint(0, wl.E, (wl.M,), dtype=torch.int32, device=dev)
    w_sets = [rw.clone() for _ in range(n_sets)]
    id_sets = [rids.clone() for _ in range(n_sets)]

    def launch_shared(i):
        mr.route_fuse_shared_expert(w_sets[i], id_sets[i], shared, 2.5, stream=stream)
    per_call, kern = time_calls(launch_shared, n_sets, stream, steps=400, warmup=20)
    nbytes = wl.M * wl.K * 8 + wl.M * 4 + wl.M * 8  # read w, ids; shared ids; write last slot
    r = {"workload": "fuse_shared_expert_m65536_k8", "entry": "route_fuse_shared_expert",
         "M": wl.M, "K": wl.K, "rotating_sets": n_sets, "us_per_call": per_call,
         "kernel_us": kern, "alg_bytes": nbytes, "GBps_kernel": nbytes / (kern * 1e-6) / 1e9}
    results.append(r)
    eprint(json.dumps(r))

    def launch_sort(i):
        mr.route_sort_ids(w_sets[i], id_sets[i], stream=stream)
    per_call, kern = time_calls(launch_sort, n_sets, stream, steps=400, warmup=20)
    nbytes = 2 * wl.M * wl.K * 8  # read and write weights and ids
    r = {"workload": "sort_ids_m65536_k8", "entry": "route_sort_ids", "M": wl.M, "K": wl.K,
         "rotating_sets": n_sets, "us_per_call": per_call, "kernel_us": kern,
         "alg_bytes": nbytes, "GBps_kernel": nbytes / (kern * 1e-6) / 1e9}
    results.append(r)
    eprint(json.dumps(r))
    if out_path:
        with open(out_path, "w") as f:
            json.dump(results, f, indent=1)
    return results


STEADY_REPEAT = 32  # 32 x 65536 tokens in one launch


def steady_inputs():
    """The 65536-token headline logits repeated 32 times on the device (1 GiB
    of bf16, more than the last-level cache), the bias and output buffers."""
    import numpy as np
    import torch

    from workloads import WORKLOADS, make_bias, make_logits
    wl = WORKLOADS[WORKLOAD]
    dev = torch.device("cuda", 0)
    x = torch.from_numpy(make_logits(wl).view(np.int16)).view(torch.bfloat16).to(dev)
    x = x.repeat(STEADY_REPEAT, 1)
    b = torch.from_numpy(make_bias(wl)).to(dev)
    M = x.shape[0]
    w = torch.empty(M, wl.K, device=dev)
    ids = torch.empty(M, wl.K, dtype=torch.int32, device=dev)
    return wl, x, b, w, ids


def steady_state_case(stream):
    """The headline kernel on 32x the headline tokens in one launch: the
    per-65536-token cost once the launch's start-up and tail are spread
    over many tiles."""
    import moe_expert_routing_amd as mr
    wl, x, b, w, ids = steady_inputs()
    M = x.shape[0]

    def launch(i):
        mr.route_biased_grouped_topk(x, b, wl.K, wl.G, wl.TG, wl.renormalize, w, ids,
                                     stream=stream)
    per_call, kern = time_calls(launch, 1, stream, steps=40, warmup=4)
    nbytes = algorithmic_bytes(M, wl.E, wl.K, 2)
    return {"workload": wl.name, "case": "steady state: one launch of 32 x 65536 tokens",
            "M": M, "us_per_call": per_call, "kernel_us": kern,
            "us_per_65536_tokens": kern * 65536 / M, "tokens_per_s": M / (kern * 1e-6),
            "alg_bytes": nbytes, "GBps_kernel": nbytes / (kern * 1e-6) / 1e9,
            "frac_hbm_kernel": nbytes / (kern * 1e-6) / 1e9 / HBM_PEAK_GBPS}


def steady_run(calls=3):
    """A few launches of the headline kernel on 32x its tokens: the program
    profiled for the steady-state clock and VALU counters."""
    import torch

    import moe_expert_routing_amd as mr
    wl, x, b, w, ids = steady_inputs()
    for _ in range(calls):
        mr.route_biased_grouped_topk(x, b, wl.K, wl.G, wl.TG, wl.renormalize, w, ids)
    torch.cuda.synchronize()
    print(json.dumps({"steady_run": "done", "calls": calls, "tokens": x.shape[0]}), flush=True)


def profile_run(calls=5):
    """A few calls of every workload's kernels, each on its own input set
    where it reads enough to leave the last-level cache, with no timing
    loops: the program profiled by the committed rocprofv3 summaries
    (kernel traces and counter passes)."""
    import numpy as np
    import torch

    import moe_expert_routing_amd as mr
    from workloads import WORKLOADS, make_bias, make_logits, make_router_inputs
    dev = torch.device("cuda", 0)

    def dev_tensor(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    def sets(t, n):
        return [t] + [t.clone() for _ in range(n - 1)]

    for name in ("biased_grouped_e256", "sigmoid_bias_e256_k8", "grouped_softmax_e160",
                 "softmax_e8_k2"):
        wl = WORKLOADS[name]
        xs = sets(dev_tensor(make_logits(wl)), calls)
        b = make_bias(wl)
        b = None if b is None else dev_tensor(b)
        for x in xs:
            if wl.entry == "route_topk_softmax":
                mr.route_topk_softmax(x, wl.K, wl.renormalize)
            elif wl.entry == "route_grouped_topk":
                mr.route_grouped_topk(x, wl.K, wl.G, wl.TG, wl.renormalize, wl.scoring)
            else:
                out = mr.route_biased_grouped_topk(x, b, wl.K, wl.G, wl.TG, wl.renormalize)
                if name == "biased_grouped_e256":
                    w, ids = out
        torch.cuda.synchronize()
        eprint(f"[profile] {name}: {calls} calls")
    # the 64-token case (one wavefront per row)
    wl = WORKLOADS["biased_grouped_e256"]
    b64 = dev_tensor(make_bias(wl))
    for x in sets(dev_tensor(make_logits(wl, 64)), calls):
        mr.route_biased_grouped_topk(x, b64, wl.K, wl.G, wl.TG, wl.renormalize)
    torch.cuda.synchronize()
    eprint(f"[profile] {wl.name} M=64: {calls} calls")
    # dispatch metadata of the 65536-token routing output
    for _ in range(calls):
        mr.route_dispatch_metadata(ids, wl.E, w)
    torch.cuda.synchronize()
    eprint(f"[profile] dispatch metadata: {calls} calls")
    # fused routers: the 7168-wide one on its default split path and as one
    # kernel, then the few-expert ones
    wl = WORKLOADS["fused_router_h7168"]
    hidden, wr = make_router_inputs(wl)
    hs = sets(dev_tensor(hidden), min(calls, 3))
    wd, bd = dev_tensor(wr), dev_tensor(make_bias(wl))
    for ws in (None, False):
        for h in hs:
            mr.route_fused_router(h, wd, wl.K, wl.G, wl.TG, wl.renormalize, "sigmoid", bd,
                                  "top2sum", workspace=ws)
        torch.cuda.synchronize()
        eprint(f"[profile] {wl.name} ({'split path' if ws is None else 'one kernel'})")
    del hs
    for name in ("fused_router_e8_h4096", "fused_router_e16_h6144"):
        wl = WORKLOADS[name]
        hidden, wr = make_router_inputs(wl)
        hs = sets(dev_tensor(hidden), min(calls, 3))
        wd = dev_tensor(wr)
        for h in hs:
            mr.route_fused_router(h, wd, wl.K, 1, 1, wl.renormalize, wl.scoring, None, "max",
                                  logit_softcap=wl.softcap)
        torch.cuda.synchronize()
        eprint(f"[profile] {name}")
        del hs
    print(json.dumps({"profile_run": "done", "calls": calls}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--sets", type=int, default=0, help="rotating input sets (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--all-configs", action="store_true",
                    help="also time every workload (stderr, and --all-out FILE as JSON)")
    ap.add_argument("--all-out", default=None)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (for HBM byte counter scaling)")
    ap.add_argument("--profile-run", action="store_true",
                    help="only run a few calls of every workload (for rocprofv3 passes)")
    ap.add_argument("--steady-run", action="store_true",
                    help="only run a few headline launches of 32x its tokens (for rocprofv3)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU: routing is per token and needs no collective; "
              f"--gpus {args.gpus} is not supported (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.profile_run:
        profile_run()
        return
    if args.steady_run:
        steady_run()
        return

    import numpy as np
    import torch

    import moe_expert_routing_amd as mr
    from workloads import WORKLOADS, make_bias, make_logits

    wl = WORKLOADS[WORKLOAD]
    dev = torch.device("cuda", 0)
    x_np = make_logits(wl)
    b_np = make_bias(wl)
    M, E, K = x_np.shape[0], wl.E, wl.K
    bytes_per_call = algorithmic_bytes(M, E, K, 2)
    set_bytes = M * E * 2 + M * K * 8
    sets = args.sets or max(2, -(-1024 * 2**20 // set_bytes))  # >= 1 GiB in rotation
    x0 = torch.from_numpy(x_np.view(np.int16)).view(torch.bfloat16).to(dev)
    bias = torch.from_numpy(b_np).to(dev)
    xs = [x0] + [x0.clone() for _ in range(sets - 1)]
    ws = [torch.empty((M, K), dtype=torch.float32, device=dev) for _ in range(sets)]
    ids = [torch.empty((M, K), dtype=torch.int32, device=dev) for _ in range(sets)]
    stream = torch.cuda.current_stream(dev)

    def step(i):
        s = i % sets
        mr.route_biased_grouped_topk(xs[s], bias, K, wl.G, wl.TG, wl.renormalize,
                                     topk_weights=ws[s], topk_ids=ids[s], stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: K back-to-back calls; events on the launch stream
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    value = M / (ms_per_step * 1e-3)

    # an event pair around each single launch (adds the event overhead)
    n_pair = min(args.steps, 400)
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(n_pair)]
    for i, (a, b) in enumerate(pairs):
        a.record(stream)
        step(i)
        b.record(stream)
    torch.cuda.synchronize()
    kern_ms = float(np.mean([a.elapsed_time(b) for a, b in pairs]))
    # The timed region holds nothing but back-to-back launches of the routing
    # kernel on this stream, so its average launch duration is ms_per_step
    # (event pairs around single launches add the event overhead to each).
    achieved = bytes_per_call / (ms_per_step * 1e-3) / 1e9

    # Independent batches alternating over two streams (default priority), so
    # that the start-up and tail of one launch overlap the next: context for
    # how much of the step time is launch structure.  The step time above
    # (one stream, one launch per step) is the figure reported as value.
    side2 = torch.cuda.Stream(dev)

    def two_streams(n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        side2.wait_stream(stream)
        for i in range(n):
            s = i % sets
            mr.route_biased_grouped_topk(xs[s], bias, K, wl.G, wl.TG, wl.renormalize,
                                         topk_weights=ws[s], topk_ids=ids[s],
                                         stream=stream if i % 2 == 0 else side2)
        stream.wait_stream(side2)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    two_streams(args.warmup)
    two_ms = two_streams(args.steps)

    # warm (cache-resident) figure for context
    for i in range(50):
        mr.route_biased_grouped_topk(x0, bias, K, wl.G, wl.TG, wl.renormalize,
                                     topk_weights=ws[0], topk_ids=ids[0], stream=stream)
    e2, e3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e2.record(stream)
    for i in range(200):
        mr.route_biased_grouped_topk(x0, bias, K, wl.G, wl.TG, wl.renormalize,
                                     topk_weights=ws[0], topk_ids=ids[0], stream=stream)
    e3.record(stream)
    torch.cuda.synchronize()
    warm_ms = e2.elapsed_time(e3) / 200

    # decode-size latency: M = 64, back-to-back enqueue and HIP-graph replay
    x64 = x0[:64].contiguous()
    w64 = torch.empty((64, K), dtype=torch.float32, device=dev)
    i64 = torch.empty((64, K), dtype=torch.int32, device=dev)
    for _ in range(100):
        mr.route_biased_grouped_topk(x64, bias, K, wl.G, wl.TG, wl.renormalize, w64, i64,
                                     stream=stream)
    torch.cuda.synchronize()
    e4, e5 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e4.record(stream)
    for _ in range(1000):
        mr.route_biased_grouped_topk(x64, bias, K, wl.G, wl.TG, wl.renormalize, w64, i64,
                                     stream=stream)
    e5.record(stream)
    torch.cuda.synchronize()
    m64_loop_us = e4.elapsed_time(e5)
    pairs64 = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(200)]
    for a, b in pairs64:
        a.record(stream)
        mr.route_biased_grouped_topk(x64, bias, K, wl.G, wl.TG, wl.renormalize, w64, i64,
                                     stream=stream)
        b.record(stream)
    torch.cuda.synchronize()
    m64_kernel_us = float(np.mean([a.elapsed_time(b) for a, b in pairs64])) * 1e3
    graph_us = None
    try:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            mr.route_biased_grouped_topk(x64, bias, K, wl.G, wl.TG, wl.renormalize, w64, i64,
                                         stream=side)
            with torch.cuda.graph(g, stream=side):
                for _ in range(100):
                    mr.route_biased_grouped_topk(x64, bias, K, wl.G, wl.TG, wl.renormalize,
                                                 w64, i64, stream=side)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        e6, e7 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e6.record(stream)
        for _ in range(10):
            g.replay()
        e7.record(stream)
        torch.cuda.synchronize()
        graph_us = e6.elapsed_time(e7) * 1e3 / 1000
    except Exception as exc:  # graph capture is optional context
        eprint(f"[bench] graph replay skipped: {exc}")

    # every set holds the same inputs, so every set must hold identical results
    for i in range(sets):
        step(i)
    torch.cuda.synchronize()
    for s in range(1, sets):
        if not (torch.equal(ws[s], ws[0]) and torch.equal(ids[s], ids[0])):
            raise SystemExit("rotating sets disagree")

    result = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "biased grouped top-k routing (DeepSeek-V3 shape)",
                   "tokens": M, "experts": E, "top_k": K, "num_expert_group": wl.G,
                   "topk_group": wl.TG, "scoring": "sigmoid+correction_bias",
                   "group_score": "top-2 sum", "renormalize": wl.renormalize,
                   "logits": "bf16 N(0, var 2)", "bias": "fp32 N(0, var 0.02)",
                   "rotating_sets": sets, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": measured_traffic()},
        "hbm_GBps_whole_step": bytes_per_call / (ms_per_step * 1e-3) / 1e9,
        "kernel_us_timed_region": ms_per_step * 1e3,
        "kernel_us_event_pairs": kern_ms * 1e3,
        "warm_cache_us_per_call": warm_ms * 1e3,
        "M64": {"kernel_us_event_pairs": m64_kernel_us, "loop_us_per_call": m64_loop_us,
                "graph_us_per_call": graph_us},
        "wall_s_timed": wall,
        "two_streams": {"us_per_step": two_ms * 1e3, "tokens_per_s": M / (two_ms * 1e-3),
                        "hbm_GBps": bytes_per_call / (two_ms * 1e-3) / 1e9,
                        "note": "independent batches alternating over two streams; one "
                                "launch's start-up and tail overlap the next (context, "
                                "not the step time)"},
    }
    # The goals set for this workload: >= 70% of HBM peak at 65536 tokens and
    # <= 5 us per call at 64 tokens.  The first is not met: the kernel is
    # bound by VALU issue (about 570 instructions per 8-row tile), not by
    # HBM bytes (its traffic is 1.007x the algorithmic bytes).
    frac = achieved / HBM_PEAK_GBPS
    result["targets"] = {
        "hbm_frac": {"target": 0.70, "measured": frac, "met": frac >= 0.70,
                     "note": "not met: VALU-issue bound, traffic 1.007x algorithmic"
                     if frac < 0.70 else "met"},
        "m64_us": {"target": 5.0, "measured_graph": graph_us,
                   "met": graph_us is not None and graph_us <= 5.0},
    }
    if args.all_configs:
        measure_all(args.all_out)
    if not args.no_cpu_baseline:
        result["cpu_baseline"], result["oracle_parity"] = cpu_baseline(
            wl, args.cpu_seconds, (ws[0].cpu().numpy(), ids[0].cpu().numpy()))
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
