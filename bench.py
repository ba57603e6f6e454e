"""Benchmark: FFN-side tokens/s per MoE layer on one MI355X.

A step is one afd_ffn_run -- the whole FFN-side hot path (wait + fan-in,
top-k routing, dispatch permutation, gate/up SwiGLU grouped GEMM, down grouped
GEMM with the shared expert, weighted combine + split + return publish) over
one work item of P peers.  Before each step the peers pack their messages on
their own streams and are synchronized, so the inputs are resident in HBM
when the step starts; after it they unpack.  Each step is timed with HIP
events on the FFN stream; inside the timed steps two more events bracket the
gate/up GEMM (the longest kernel in every workload), whose average duration
gives the roofline figure.  (Every event record costs a few microseconds
between two launches, so the timed steps carry only those two.)  An untimed
pass afterwards, with an event between every two kernels, gives the
per-kernel breakdown.

Prints one JSON line.  Default workload: the largest one, skewed routing
over large experts (2 peers x 4096 tokens, H=7168, 256 experts, top-8,
I=2048, one shared expert of 2048, a Zipf(1.1) per-expert logit bias).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
MFMA_FP8_PEAK_TFLOPS = 5000.0    # MI355X dense fp8 MFMA, published
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def algorithmic(wl, counts):
    """Algorithmic flops and bytes of one FFN step and of its kernels."""
    T, H, E, K, I, Is = (wl.total_tokens, wl.hidden, wl.num_experts, wl.top_k, wl.intermediate,
                         wl.shared_intermediate)
    pairs = T * K
    touched = int((np.asarray(counts) > 0).sum())
    g1_flops = 4.0 * H * I * pairs + 4.0 * H * Is * T
    g2_flops = 2.0 * H * I * pairs + 2.0 * H * Is * T
    wb = 1 if wl.w1_fp8 else 2  # bytes per gate/up weight (e4m3 codes, or bf16)
    w13_bytes = touched * 2 * I * H * wb + (2 * Is * H * wb if Is else 0)
    w2_bytes = touched * H * I * 2 + (H * Is * 2 if Is else 0)
    io_bytes = T * H * 2 + T * E * 4 + T * H * 2
    return {
        "flops": g1_flops + g2_flops,
        "bytes": w13_bytes + w2_bytes + io_bytes,
        "gemm_gate_up_swiglu": {"flops": g1_flops, "bytes": w13_bytes + T * H * wb * (K + 1) + 2 * pairs * I},
        "gemm_down": {"flops": g2_flops, "bytes": w2_bytes + 2 * pairs * I + 2 * T * Is},
        "touched_experts": touched,
    }


def _variant(wl):
    return ("_attention_routed" if wl.attention_routes else "") + ("_w1_fp8" if wl.w1_fp8 else "")


def measured_traffic(wl, kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary of this workload (profiles/hbm_bytes_<workload>.json), or None
    if there is none or it was measured on a kernel source other than the
    one built now."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"hbm_bytes_{wl.name}{_variant(wl)}.json")
    src = os.path.join(ROOT, "combine_afd_slot_amd", "csrc", "afd_kernels.hip")
    try:
        side = json.load(open(path))
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    except OSError:
        return None
    if side.get("workload") != wl.name or side.get("kernel_source_sha256") != sha:
        return None
    b = side["bytes_per_launch"].get(kernel)
    return None if b is None else int(b["read"] + b["written"])


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# workloads whose whole oracle run fits the baseline's time budget on the
# measurement host's cores (about 3 s for decode, 9 s for prefill)
FULL_ORACLE = ("tiny", "decode", "prefill")


def _oracle_run(oracle, wl, inp, n):
    """One timed oracle pass (steady clock) over the first n[p] tokens of each peer."""
    x = [inp["x"][p][:n[p]] for p in range(wl.num_peers)]
    l = [inp["l"][p][:n[p]] for p in range(wl.num_peers)]
    t0 = time.perf_counter()
    if wl.w1_fp8:
        oracle.ffn_fp8(x, l, inp["W13"], inp["W2"], inp.get("Ws13"), inp.get("Ws2"), K=wl.top_k,
                       rsf=wl.routed_scaling_factor, renorm=wl.renormalize)
    else:
        oracle.ffn(x, l, inp["W13"], inp["W2"], inp.get("Ws13"), inp.get("Ws2"), K=wl.top_k,
                   rsf=wl.routed_scaling_factor, renorm=wl.renormalize)
    return time.perf_counter() - t0


def cpu_baseline(wl, inp, target_s=8.0):
    """The oracle as it stands (float64 C, OpenMP over the host's threads),
    timed on this workload's inputs: the median of 3 runs, over every token
    where that fits the budget, else over a labelled prefix sample of each
    peer; plus 1-thread times of the whole oracle on the tiny and decode
    workloads."""
    from oracle import oracle
    from combine_afd_slot_amd.inputs import WORKLOADS, make_inputs
    oracle.lib()
    T = wl.total_tokens
    threads = oracle.num_threads()
    if wl.name in FULL_ORACLE and not wl.w1_fp8:
        n = list(wl.seq_lens)
        label = f"every token ({T}), whole oracle path a1-a7 in float64"
    else:
        frac = min(1.0, 32.0 / T)
        n = [max(1, int(round(v * frac))) if v else 0 for v in wl.seq_lens]
        dt = _oracle_run(oracle, wl, inp, n)
        if dt < target_s and frac < 1.0:
            frac = min(1.0, frac * target_s / max(dt, 1e-3))
            n = [max(1, int(round(v * frac))) if v else 0 for v in wl.seq_lens]
        label = (f"first {sum(n)} of {T} tokens (each peer's leading {frac:.4f} share), whole oracle path "
                 f"a1-a7 in float64" + (" with the fp8 W1 operands" if wl.w1_fp8 else ""))
    runs = sorted(_oracle_run(oracle, wl, inp, n) for _ in range(3))
    med = runs[1]
    one = {}
    oracle.set_threads(1)
    try:
        for name in ("tiny", "decode"):
            w1 = WORKLOADS[name]
            i1 = inp if w1.name == wl.name and not wl.w1_fp8 else make_inputs(w1)
            reps = 3 if name == "tiny" else 1
            ts = sorted(_oracle_run(oracle, w1, i1, list(w1.seq_lens)) for _ in range(reps))
            one[name] = {"tokens_per_s": round(w1.total_tokens / ts[len(ts) // 2], 2),
                         "runs": reps, "s": round(ts[len(ts) // 2], 4)}
    finally:
        oracle.set_threads(threads)
    return {"value": round(sum(n) / med, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": label, "runs_s": [round(r, 3) for r in runs], "stat": "median of 3",
            "nproc": os.cpu_count(), "cpu_model": _cpu_model(), "one_thread_whole_oracle": one}


def peer_side_ms(torch, sess, n):
    """Untimed pass: per step, the slowest peer's pack and unpack (HIP events
    on each peer's stream; not part of the FFN step)."""
    P = sess.wl.num_peers
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(P)]
    pk, up = [], []
    for _ in range(n):
        for p in range(P):
            ev[p][0].record(sess.peer_streams[p])
            sess.pack(p)
            ev[p][1].record(sess.peer_streams[p])
        for ps in sess.peer_streams:
            ps.synchronize()
        sess.run()
        sess.ffn_stream.synchronize()
        for p in range(P):
            ev[p][2].record(sess.peer_streams[p])
            sess.unpack(p)
            ev[p][3].record(sess.peer_streams[p])
        for ps in sess.peer_streams:
            ps.synchronize()
        pk.append(max(ev[p][0].elapsed_time(ev[p][1]) for p in range(P)))
        up.append(max(ev[p][2].elapsed_time(ev[p][3]) for p in range(P)))
    return {"pack": round(float(np.mean(pk)), 4), "unpack": round(float(np.mean(up)), 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="skew",
                    help="tiny | prefill | fanin4 | skew | decode (default: skew, the largest workload)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-profile", action="store_true", help="no per-kernel events (pure step timing)")
    ap.add_argument("--attention-routes", action="store_true",
                    help="attention-routed window: the peers route, group and combine; the FFN side merges "
                         "their group lists")
    ap.add_argument("--w1-fp8", action="store_true",
                    help="gate/up GEMMs on e4m3 operands (token and W13 rows quantised per row); down GEMM bf16")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain 1 GiB device-to-device copy, 10 times (scale for HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the FFN-rank path here runs on a single MI355X "
              "(no collectives); run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.calibrate_copy:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": n, "calibrate_copy_bytes_written": n, "launches": 10}))
        return
    from combine_afd_slot_amd import afd
    from combine_afd_slot_amd.driver import FfnSession
    from combine_afd_slot_amd.inputs import WORKLOADS, make_inputs

    wl = WORKLOADS[args.workload]
    if args.attention_routes or args.w1_fp8:
        import dataclasses
        wl = dataclasses.replace(wl, attention_routes=int(args.attention_routes), w1_fp8=int(args.w1_fp8))
    log(f"[bench] workload {wl.name}: seq_lens={wl.seq_lens} H={wl.hidden} E={wl.num_experts} "
        f"K={wl.top_k} I={wl.intermediate} Is={wl.shared_intermediate}")
    t0 = time.time()
    inp = make_inputs(wl)
    log(f"[bench] inputs drawn in {time.time() - t0:.1f} s")

    sess = FfnSession(wl, inp)
    for i in range(args.warmup):
        sess.step()
    st = sess.status()
    if st.status != 0:
        raise RuntimeError(f"warmup run failed: {afd.status_string(st.status)}")
    counts = sess.routing()["counts"]
    log(f"[bench] warmup done ({args.warmup} steps); expert counts min/max {counts.min()}/{counts.max()}")

    if not args.no_profile:
        # timed steps: events only around the gate/up GEMM, so the other
        # kernels run back to back exactly as without profiling
        afd.afd_profile_enable(sess.win, 3)
        afd.afd_profile_read(sess.win, reset=True)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    step_ms = []
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(args.steps):
        sess.pack_all()
        ev0.record(sess.ffn_stream)
        sess.run()
        ev1.record(sess.ffn_stream)
        sess.ffn_stream.synchronize()
        step_ms.append(ev0.elapsed_time(ev1))
        sess.unpack_all()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    st = sess.status()
    if st.status != 0:
        raise RuntimeError(f"timed run failed: {afd.status_string(st.status)}")
    kern, kern_all = {}, {}
    if not args.no_profile:
        tot, runs = afd.afd_profile_read(sess.win, reset=True)
        kern = {k: v / max(runs, 1) for k, v in tot.items() if k == "gemm_gate_up_swiglu"}
        # an untimed pass with an event between every two kernels, for the
        # per-kernel breakdown (the events add small gaps between launches)
        afd.afd_profile_enable(sess.win, 1)
        for i in range(min(args.steps, 10)):
            sess.step()
        tot, runs = afd.afd_profile_read(sess.win, reset=True)
        afd.afd_profile_enable(sess.win, 0)
        kern_all = {k: round(v / max(runs, 1), 4) for k, v in tot.items()}
        if wl.attention_routes:  # the slots hold the attention-routed run's kernels
            ren = {"route_topk": "merge_group_lists", "permute": "dispatch_plan",
                   "combine_split_publish": "return_copy_publish"}
            kern_all = {ren.get(k, k): v for k, v in kern_all.items() if k != "scan_offsets"}
    peer_ms = peer_side_ms(torch, sess, min(args.steps, 10))
    sess.close()

    ms = float(np.mean(step_ms))
    T = wl.total_tokens
    alg = algorithmic(wl, counts)
    value = T / (ms * 1e-3)
    line = {
        "metric": "FFN-side tokens/sec per MoE layer (dispatch+GEMM+combine); % of MFMA/HBM roofline",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_step_p10_p50_p90": [round(float(np.percentile(step_ms, q)), 4) for q in (10, 50, 90)],
        "wall_ms_per_step_incl_pack_unpack": round(wall * 1e3 / args.steps, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 gate/up, bf16 down" if wl.w1_fp8 else "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "peers": wl.num_peers, "seq_lens": list(wl.seq_lens),
                   "total_tokens": T, "hidden": wl.hidden, "experts": wl.num_experts, "top_k": wl.top_k,
                   "intermediate": wl.intermediate, "shared_intermediate": wl.shared_intermediate,
                   "token_cap": wl.token_cap, "parallelism": "single GPU"},
        "mfma_frac_step": round(alg["flops"] / (ms * 1e-3) / (MFMA_BF16_PEAK_TFLOPS * 1e12), 4),
        "hbm_frac_step": round(alg["bytes"] / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
        "expert_counts_min_max": [int(counts.min()), int(counts.max())],
        "peer_side_ms_max_over_peers": peer_ms,
    }
    if wl.attention_routes:
        line["config"]["attention_routes"] = 1
    if wl.w1_fp8:
        line["config"]["w1_fp8"] = 1
    peak = MFMA_FP8_PEAK_TFLOPS if wl.w1_fp8 else MFMA_BF16_PEAK_TFLOPS  # the dominant GEMM's operand type
    if kern:
        line["kernel_ms"] = {k: round(v, 4) for k, v in kern.items()}
        line["kernel_ms_all_separate_pass"] = kern_all
        dom = "gemm_gate_up_swiglu"  # twice the down GEMM's weights and flops
        # decode-shaped steps stream weights: bound by HBM; prefill steps by MFMA
        ai = alg[dom]["flops"] / alg[dom]["bytes"]
        ridge = peak * 1e12 / (HBM_PEAK_GBS * 1e9)
        if ai >= ridge:
            ach = alg[dom]["flops"] / (kern[dom] * 1e-3) / 1e12
            line["roofline"] = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 1),
                                "peak": peak, "unit": "TFLOP/s",
                                "frac": round(ach / peak, 4), "traffic": measured_traffic(wl, dom)}
        else:
            ach = alg[dom]["bytes"] / (kern[dom] * 1e-3) / 1e9
            line["roofline"] = {"kernel": dom, "bound": "hbm", "achieved": round(ach, 1),
                                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": measured_traffic(wl, dom)}
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle (median of 3)")
        line["cpu_baseline"] = cpu_baseline(wl, inp)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
