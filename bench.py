#!/usr/bin/env python3
"""Decode-step bench of the W4A16 GEMV on one MI355X.

One step = the 128 GEMVs of 32 Llama-3-8B-shaped decoder layers at M = 1
(fused QKV 4096->6144, O 4096->4096, fused gate-up 4096->28672, down
14336->4096), each with its own seeded 4-bit group-32 weights, all resident in
HBM (4.37 GB packed). Products run in order, each one starting only after
every earlier one's results are written (the ordering a decode loop needs).
Two launch forms of the same step are timed:

* chain: one w4a16_gemv_chain launch per step, the products ordered on the
  device, the next product's weights streamed while that ordering point is
  reached;
* separate: 128 w4a16_gemv launches on one stream, replayed from a HIP graph.

The faster one is the reported value. Printed: one JSON line with the whole-step
throughput in algorithmic GB/s (N*K/2 code bytes + 4 bytes of scale/min per 32
weights + x + y, per GEMV), the roofline entry of the dominant kernel of the
reported form (its launches event-timed on the launch stream) and the fp64
oracle timed on this host's cores as a reported CPU baseline. The roofline
entry is taken against the roof the kernel would hit first: the HBM peak, or,
when its 2*M*N*K flops take longer at the fp32 vector peak than its bytes at
the HBM peak (M >= 7), that vector peak; the other roof's fraction is given
beside it.

--workload gemv4096|llama8b_layer|llama8b_verify|llama70b_step (with --m for
the activation rows of the verify and 70B workloads) times one of the other
configurations the same way, with separate launches: the single 4096 x 4096
GEMV, one 8B layer, the M = 4 / 8 verify batches and the 80-layer 70B step.
Workloads that fit the 256 MB MALL walk independently seeded copies of their
weights, at least 512 MB per timed step, and report the time per copy.

--only chain|separate times one form (for counter runs); --copy-calibration
runs only a plain device copy of 1 GiB three times (the FETCH_SIZE /
WRITE_SIZE scale of a kernel of known traffic). --codec q4_sym|q5|q8_sym runs
the same step with one of the weight-code variants (separate launches only:
the chain streams the 4-bit code) and reports it the same way. --kv 8|4 runs
the other bandwidth-bound operation of the decode step instead: attention of
one new token over the INT8 / INT4 KV cache of all 32 layers of the 8B shape
(32 query heads, 8 KV heads, head size 128) at the context the core-modules
page's KV budget allows (38,863 / 77,726 tokens), one w4a16_kv_attention call
per layer replayed from a HIP graph.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workload  # noqa: E402

METRIC = "W4A16 decode GEMV µs/step and effective HBM GB/s (% of peak), 8B shapes"
HBM_PEAK_GBS = 8000.0
# fp32 vector peak: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz x 4 flops per lane
# per v_dot2_f32_f16 (two products and two adds), the same as packed fp32 FMA
VALU_PEAK_TFLOPS = 157.3
WORKLOAD = "llama8b_step"
WORKLOAD_TEXT = {
    "gemv4096": "gemv4096: one GEMV 4096->4096, plain N(0,1) activations",
    "llama8b_layer": "llama8b_layer: one Llama-3-8B-shaped layer (qkv 4096->6144, o 4096->4096, "
                     "gate_up 4096->28672, down 14336->4096)",
    "llama8b_step": "llama8b_step: 32 Llama-3-8B-shaped layers x (qkv 4096->6144, o 4096->4096, "
                    "gate_up 4096->28672, down 14336->4096)",
    "llama8b_verify": "llama8b_verify: one Llama-3-8B-shaped layer, speculative-verify rows, "
                      "plain N(0,1) activations",
    "llama70b_step": "llama70b_step: 80 Llama-3-70B-shaped layers x (qkv 8192->10240, o 8192->8192, "
                     "gate_up 8192->57344, down 28672->8192)",
    "llama70b_tp8": "llama70b_tp8: one GPU's share of the 80-layer 70B step under 8-way tensor parallelism "
                    "(qkv 8192->1280, o 1024->8192, gate_up 8192->7168, down 3584->8192)",
}


# code bits per weight and parameter bytes per group of 32 weights, per codec
CODEC_BITS = {"q4": (4, 4), "q4_sym": (4, 2), "q5": (5, 4), "q8_sym": (8, 2), "pal4": (4, 0)}
CODEC_DTYPE = {"q4": "u4xf16->f32", "q4_sym": "u4xf16->f32", "q5": "u5xf16->f32", "q8_sym": "i8xf16->f32",
               "pal4": "u4xf16->f32"}
CODEC_TEXT = {"q4": "4-bit codes, group 32, fp16 scale+min",
              "q4_sym": "symmetric 4-bit codes (s*(q-8)), group 32, fp16 scale",
              "q5": "5-bit codes, group 32, fp16 scale+min",
              "q8_sym": "symmetric 8-bit codes (s*q, int8), group 32, fp16 scale",
              "pal4": "palettised 4-bit codes (a 16-entry fp16 palette per row)"}


def gemv_bytes(M, N, K, codec="q4"):
    """Algorithmic bytes of one GEMV: codes, per-group parameters, x and y."""
    bits, par = CODEC_BITS[codec]
    palettes = 32 * N if codec == "pal4" else 0  # 16 binary16 entries per row
    return N * K * bits // 8 + par * N * (K // 32) + palettes + 2 * M * K + 4 * M * N


# HBM traffic per launch of a kernel on a workload, keyed (workload, M, kernel),
# from rocprofv3 FETCH_SIZE and WRITE_SIZE runs scaled by the same counters on
# a 1 GiB device copy; kept only while the kernel is unchanged since the
# counters were taken.
TRAFFIC = {
    # (16,750.70 KiB FETCH_SIZE x 2.000 + 52.0 KiB WRITE_SIZE x 1.000) per dispatch
    ("llama8b_step", 1, "gemv_kernel<1, 1, 1>"): 34_358_684,
    # (2,137,088.35 KiB x 2.000 + 11,904.06 KiB x 1.000) per dispatch
    ("llama8b_step", 1, "chain_kernel<1, 24, 8>"): 4_388_946_709,
    # the 70B step: (65,464.03 KiB x 2.000 + 84.0 KiB x 1.000) per dispatch
    ("llama70b_step", 1, "gemv_kernel<1, 1, 1>"): 134_156_358,
    # weight-code variants: (15,084.23 / 20,094.84 / 28,408.95 KiB x 2.000 + 52.0 KiB x 1.000)
    ("llama8b_step", 1, "codec_kernel<1, 1, 1, 1>"): 30_945_743,
    ("llama8b_step", 1, "codec_kernel<2, 1, 1, 1>"): 41_207_479,
    ("llama8b_step", 1, "codec_kernel<3, 1, 1, 1>"): 58_234_777,
    # verify batches: (16,946.12 / 17,196.90 KiB x 2.000 + 200.0 / 400.0 KiB x 1.000)
    ("llama8b_verify", 4, "gemv_kernel<4, 1, 1>"): 34_910_459,
    ("llama8b_verify", 8, "gemv_kernel<8, 1, 1>"): 35_628_853,
    # one GPU's share of the 70B step at 8-way tensor parallelism: (10,126.34 KiB x 2.000 + 35.33 KiB x 1.000)
    ("llama70b_tp8", 1, "gemv_kernel<1, 1, 1>"): 20_774_930,
    # the 70B step at M = 8: (63,843.49 KiB x 2.000 + 810.67 KiB x 1.000)
    ("llama70b_step", 8, "gemv_kernel<8, 1, 1>"): 131_581_595,
    # palettised codes: (13,617.78 KiB x 2.000 + 52.0 KiB x 1.000)
    ("llama8b_step", 1, "codec_kernel<4, 1, 1, 1>"): 27_942_458,
    # KV-cache attention, split pass: (41,442.61 / 48,739.67 KiB x 2.000 + 1,235.0 / 828.75 KiB x 1.000)
    ("llama8b_kv_int8", 1, "kv_attn_kernel<8, 4>"): 86_139_115,
    ("llama8b_kv_int4", 1, "kv_attn_kernel<4, 4>"): 100_667_484,
}


KV_METRIC = "KV-cache decode attention µs/step and effective HBM GB/s (% of peak), 8B shapes"


def kv_layer_bytes(bits, T, Hq, Hkv):
    """Algorithmic bytes of one layer's attention: the codes and group
    parameters of T tokens (keys and values), q and o."""
    per_value = {8: 1 + 2 / 32, 4: 0.5 + 4 / 32}[bits]
    return int(round(T * Hkv * 128 * 2 * per_value)) + Hq * 128 * 2 + Hq * 128 * 4


def copy_calibration(torch, dev):
    """Three plain device copies of 1 GiB (known traffic: 1 GiB read, 1 GiB written)."""
    a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    log("[bench] copy calibration: 3 copies of 1 GiB done")


def host_cpu_model():
    """The host CPU's model name from /proc/cpuinfo (None where it is not readable)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def system_info(torch, w4, dev):
    """What the line was measured on: device, runtime and library versions, host CPU."""
    props = torch.cuda.get_device_properties(dev)
    return {
        "device": props.name,
        "arch": getattr(props, "gcnArchName", None),
        "compute_units": props.multi_processor_count,
        "hip": torch.version.hip,
        "torch": torch.__version__,
        "library_abi": w4.w4a16_abi_version(),
        "host_cpu": host_cpu_model(),
        "host_threads": len(os.sched_getaffinity(0)),
    }


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def rotation_sets(wl, M, codec):
    """Independently seeded copies of a workload's weights that one timed step
    walks through, so that at least ~512 MB is streamed per step and the data
    cannot be served from the 256 MB MALL."""
    step = sum(gemv_bytes(m, p.N, p.K, codec) for _, _, p, m in workload.workload_gemvs(wl, M))
    return max(1, -(-512_000_000 // step))


def build_inputs(torch, w4, M, dev, threads, codec="q4", wl=WORKLOAD, sets=1):
    """Generate, pack and upload every GEMV of the step (times `sets` seeded
    copies: copy s of a one-layer workload uses layer index s); returns a list
    of dicts."""
    base = list(workload.workload_gemvs(wl, M))
    if sets > 1 and workload.WORKLOADS[wl].layers != 1:
        raise ValueError("rotation copies are for one-layer workloads")
    items = [(s if sets > 1 else layer, pi, p, m) for s in range(sets) for layer, pi, p, m in base]

    def make(item):
        layer, pi, p, m = item
        x, codes, scale, mn = workload.codec_gemv_inputs(codec, wl, layer, pi, m)
        blob = w4.w4a16_codec_pack(codec, codes, scale, mn)
        return item, x, blob

    out = []
    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        for i, ((layer, pi, p, m), x, blob) in enumerate(ex.map(make, items)):
            if len(items) > 64 and (i + 1) % 64 == 0:
                log(f"[bench] {i + 1} of {len(items)} GEMVs packed and uploaded")
            packed = w4.upload_packed(blob, dev)
            xd = torch.from_numpy(x).to(dev)
            y = torch.zeros((m, p.N), dtype=torch.float32, device=dev)
            out.append(dict(layer=layer, proj=pi, name=p.name, M=m, N=p.N, K=p.K, x=xd, packed=packed, y=y,
                            bytes=gemv_bytes(m, p.N, p.K, codec),
                            kernel=w4.w4a16_codec_launch_shape(codec, m, p.N, p.K)["kernel"]))
            del blob
    return out


def launch_step(w4, gemvs, stream_handle, codec="q4"):
    cid = w4.codec_id(codec)
    for g in gemvs:
        st = w4.w4a16_codec_gemv_raw(cid, g["xp"], g["pp"], g["yp"], g["M"], g["N"], g["K"], stream_handle)
        if st != 0:
            raise w4.W4A16Error(st, "w4a16_codec_gemv")


def spot_check(w4, gemvs, torch, codec="q4", wl=WORKLOAD):
    """Sampled rows of two GEMVs of the step against the oracle (sanity only)."""
    import oracle

    for g in gemvs[2:4] if len(gemvs) >= 4 else gemvs[:2]:
        x, codes, scale, mn = workload.codec_gemv_inputs(codec, wl, g["layer"], g["proj"], g["M"])
        rows = np.arange(0, g["N"], max(1, g["N"] // 64))
        y_ref, B = oracle.codecs_ref.gemv_rows(codec, x, codes, scale, mn, rows)
        y = g["y"].cpu().numpy()[:, rows].astype(np.float64)
        if not oracle.within_tolerance(y, y_ref, B).all():
            raise AssertionError(f"bench spot check failed on {g['name']} layer {g['layer']}")


def cpu_baseline(budget_s=12.0, codec="q4", wl=WORKLOAD, M=1):
    """The fp64 oracle on whole GEMVs of the same step until ~budget_s of work."""
    import threadpoolctl

    import oracle

    threads = len(os.sched_getaffinity(0))
    done_bytes = 0
    done = []
    t_total = 0.0
    step = list(workload.workload_gemvs(wl, M))
    with threadpoolctl.threadpool_limits(1):
        for layer, pi, p, m in step:
            x, codes, scale, mn = workload.codec_gemv_inputs(codec, wl, layer, pi, m)
            t0 = time.perf_counter()
            if codec == "q4":
                oracle.gemv(x, codes, scale, mn, threads=threads)
            else:
                oracle.codecs_ref.gemv(codec, x, codes, scale, mn, threads=threads)
            t_total += time.perf_counter() - t0
            done_bytes += gemv_bytes(m, p.N, p.K, codec)
            done.append(f"L{layer}.{p.name}")
            if t_total >= budget_s:
                break
    return {
        "value": round(done_bytes / t_total / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "host_cpu": host_cpu_model(),
        "kind": "oracle",
        "sample": f"fp64 oracle on the first {len(done)} of the step's {len(step)} GEMVs (layer order, "
                  f"{done[0]} .. {done[-1]}), "
                  f"{done_bytes / 1e6:.1f} MB algorithmic, {t_total:.1f} s wall, "
                  f"{threads} worker threads, BLAS threads limited to 1",
        "us_per_step_extrapolated": round(t_total / done_bytes * sum(
            gemv_bytes(m, p.N, p.K, codec) for _, _, p, m in step) * 1e6, 1),
    }


def time_loop(torch, stream, fn, warmup, steps):
    """Wall-clock seconds per call of fn() over `steps` calls after `warmup`."""
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        for _ in range(steps):
            fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def kv_cpu_baseline(bits, T, budget_s):
    """The fp64 attention oracle on whole layers of the same step until ~budget_s."""
    import threadpoolctl

    import oracle

    done, t_total, nbytes = 0, 0.0, 0
    Hq, Hkv = workload.KV_HQ, workload.KV_HKV
    while t_total < budget_s and done < workload.KV_LAYERS:
        cache = workload.kv_cache(bits, 3, done, T, Hkv)
        q = workload.kv_query(3, done, Hq)
        t0 = time.perf_counter()
        with threadpoolctl.threadpool_limits(1):
            oracle.kv_attention_ref.attention(bits, q, *cache)
        t_total += time.perf_counter() - t0
        nbytes += kv_layer_bytes(bits, T, Hq, Hkv)
        done += 1
    return {
        "value": round(nbytes / t_total / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "host_cpu": host_cpu_model(),
        "kind": "oracle",
        "sample": f"fp64 attention oracle (numpy) on the first {done} of the step's {workload.KV_LAYERS} layers "
                  f"(T = {T}), {nbytes / 1e6:.1f} MB algorithmic, {t_total:.1f} s wall, one thread",
    }


def main_kv(args, torch, w4, dev):
    bits = args.kv
    T = workload.KV_CONTEXT[bits]
    Hq, Hkv, L = workload.KV_HQ, workload.KV_HKV, workload.KV_LAYERS
    t0 = time.time()
    layers = []
    for layer in range(L):
        cache = workload.kv_cache(bits, 3, layer, T, Hkv)
        q = workload.kv_query(3, layer, Hq)
        kv = w4.upload_packed(w4.w4a16_kv_pack(bits, *cache), dev)
        qd = torch.from_numpy(q).to(dev)
        o = torch.zeros((Hq, 128), dtype=torch.float32, device=dev)
        layers.append(dict(kv=kv, q=qd, o=o))
        del cache
    ws = torch.empty(w4.w4a16_kv_workspace_bytes(T, Hq) // 4, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    layer_bytes = kv_layer_bytes(bits, T, Hq, Hkv)
    step_bytes = L * layer_bytes
    log(f"[bench] KV attention: {L} layers, INT{bits}, T={T}, {step_bytes / 1e9:.3f} GB/step, "
        f"inputs ready in {time.time() - t0:.1f} s")
    stream = torch.cuda.Stream(device=dev)
    sh = stream.cuda_stream
    ptrs = [(g["q"].data_ptr(), g["kv"].data_ptr(), g["o"].data_ptr()) for g in layers]
    wsp, wsb = ws.data_ptr(), ws.numel() * 4

    def step(handle=sh):
        for qp, kp, op in ptrs:
            st = w4.w4a16_kv_attention_raw(bits, qp, kp, op, T, Hq, Hkv, wsp, wsb, handle)
            if st != 0:
                raise w4.W4A16Error(st, "w4a16_kv_attention")

    with torch.cuda.stream(stream):
        step()
    stream.synchronize()
    import oracle

    for layer in (0, L - 1):  # sanity: sampled heads against the oracle
        cache = workload.kv_cache(bits, 3, layer, T, Hkv)
        heads = [0, 13, Hq - 1]
        o_ref, B = oracle.kv_attention_ref.attention(bits, workload.kv_query(3, layer, Hq), *cache, heads=heads)
        if not oracle.kv_attention_ref.within_tolerance(layers[layer]["o"].cpu().numpy()[heads], o_ref, B).all():
            raise AssertionError(f"bench spot check failed on layer {layer}")
    log("[bench] spot checks ok")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        step(stream.cuda_stream)
    torch.cuda.synchronize()
    sec = time_loop(torch, stream, graph.replay, args.warmup, args.steps)
    log(f"[bench] KV attention step: {sec * 1e6:.1f} us")
    marks = []
    with torch.cuda.stream(stream):
        for _ in range(max(1, args.steps // 4)):
            for qp, kp, op in ptrs:
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                b.record(stream)
                st = w4.w4a16_kv_attention_timed_raw(bits, qp, kp, op, T, Hq, Hkv, wsp, wsb, sh, a.cuda_event,
                                                     b.cuda_event)
                if st != 0:
                    raise w4.W4A16Error(st, "w4a16_kv_attention_timed")
                marks.append((a, b))
    torch.cuda.synchronize()
    avg_us = sum(a.elapsed_time(b) for a, b in marks) / len(marks) * 1e3
    shape = w4.w4a16_kv_launch_shape(bits, T, Hq, Hkv)
    kernel = shape["kernel"]
    achieved = layer_bytes / (avg_us * 1e-6) / 1e9
    log(f"[bench] {kernel}: avg {avg_us:.2f} us per launch, {layer_bytes / 1e6:.2f} MB, {achieved:.1f} GB/s")
    value = step_bytes / sec / 1e9
    line = {
        "metric": KV_METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sec * 1e3, 5),
        "us_per_step": round(sec * 1e6, 2),
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"i{bits}xf16->f32" if bits == 8 else "u4xf16->f32",
        "data": "synthetic",
        "config": {
            "workload": f"llama8b_kv_int{bits}: one new token's attention over 32 layers x (32 query heads, "
                        f"8 KV heads, head size 128), INT{bits} KV cache of {T} tokens, group-32 fp16 parameters",
            "layers": L,
            "tokens": T,
            "bytes_per_step": step_bytes,
            "launch": f"{L} w4a16_kv_attention calls per step ({kernel} + {shape['merge_kernel']}), "
                      f"replayed from a HIP graph",
        },
        "system": system_info(torch, w4, dev),
        "roofline": {
            "bound": "hbm",
            "kernel": kernel,
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": TRAFFIC.get((f"llama8b_kv_int{bits}", 1, kernel)),
            "avg_launch_us": round(avg_us, 3),
            "bytes_per_launch": layer_bytes,
        },
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the fp64 oracle on host cores ...")
        line["cpu_baseline"] = kv_cpu_baseline(bits, T, args.cpu_budget)
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--only", choices=["chain", "separate"], default=None)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time separate launches eagerly (counter runs)")
    ap.add_argument("--codec", choices=list(CODEC_BITS), default="q4",
                    help="weight code of the step (the chain runs the 4-bit code only)")
    ap.add_argument("--workload", choices=list(workload.WORKLOADS), default=WORKLOAD,
                    help="configuration to time (default: the 32-layer 8B decode step)")
    ap.add_argument("--m", type=int, default=None, help="activation rows (default: the workload's first)")
    ap.add_argument("--kv", type=int, choices=[8, 4], default=None,
                    help="bench decode attention over an INT8 / INT4 KV cache instead of the GEMVs")
    args = ap.parse_args()
    codec = args.codec
    wl = args.workload
    M = args.m if args.m is not None else workload.WORKLOADS[wl].ms[0]
    if M not in workload.WORKLOADS[wl].ms:
        ap.error(f"--m {M}: {wl} runs M in {workload.WORKLOADS[wl].ms}")
    if codec != "q4" or wl != WORKLOAD:
        if args.only == "chain":
            ap.error("the chain form is timed on the 4-bit 8B decode step only")
        args.only = "separate"

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the W4A16 GEMV path has no multi-GPU code "
              "(a sharded run would split N across GPUs with no exchange); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import bit_weight_quantized_w4a16_amd as w4

    if not os.path.exists(w4.LIB_PATH):
        from bit_weight_quantized_w4a16_amd import _build
        _build.build()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        copy_calibration(torch, dev)
        return
    if args.kv is not None:
        main_kv(args, torch, w4, dev)
        return
    t0 = time.time()
    sets = rotation_sets(wl, M, codec) if workload.WORKLOADS[wl].layers == 1 else 1
    gemvs = build_inputs(torch, w4, M, dev, threads=min(16, len(os.sched_getaffinity(0))), codec=codec, wl=wl,
                         sets=sets)
    torch.cuda.synchronize()
    for g in gemvs:
        g["xp"], g["pp"], g["yp"] = g["x"].data_ptr(), g["packed"].data_ptr(), g["y"].data_ptr()
    step_bytes = sum(g["bytes"] for g in gemvs) // sets  # one copy of the workload
    log(f"[bench] {wl} M={M}: {len(gemvs) // sets} GEMVs, {step_bytes / 1e9:.3f} GB/step"
        f"{f', {sets} seeded copies walked per timed pass' if sets > 1 else ''}, "
        f"inputs ready in {time.time() - t0:.1f} s")

    stream = torch.cuda.Stream(device=dev)
    sh = stream.cuda_stream

    # separate launches first (their outputs are the chain's reference)
    with torch.cuda.stream(stream):
        launch_step(w4, gemvs, sh, codec)
    stream.synchronize()
    spot_check(w4, gemvs, torch, codec, wl)

    if codec == "q4" and wl == WORKLOAD:
        # the decode step as one chained launch: plan and workspace made once
        plan = torch.from_numpy(w4.w4a16_chain_plan(
            [(g["x"], g["packed"], g["y"], g["N"], g["K"]) for g in gemvs], M)).to(dev)
        workspace = torch.zeros(w4.W4A16_CHAIN_WORKSPACE_BYTES // 4, dtype=torch.int32, device=dev)
        plan_p, ws_p, count = plan.data_ptr(), workspace.data_ptr(), len(gemvs)
        ws_bytes = workspace.numel() * workspace.element_size()

        def chain_step():
            st = w4.w4a16_gemv_chain_raw(plan_p, count, M, ws_p, ws_bytes, sh)
            if st != 0:
                raise w4.W4A16Error(st, "w4a16_gemv_chain")

        separate = [g["y"].clone() for g in gemvs]
        for g in gemvs:
            g["y"].fill_(float("nan"))
        # the plan and workspace uploads, the clones and the NaN fills ran on
        # the current stream; the chain runs on `stream`
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            chain_step()
        stream.synchronize()
        st, bits = w4.w4a16_chain_status_raw(ws_p, ws_bytes, sh, False)
        if st != w4.W4A16_OK:
            raise w4.W4A16Error(st, f"first chain call (error word {bits:#x})")
        spot_check(w4, gemvs, torch)
        worst = max(float(((g["y"] - r).abs() / (r.abs() + 1e-3)).max()) for g, r in zip(gemvs, separate))
        if workspace.cpu().numpy().any():
            raise AssertionError("chain workspace not clean after a call (counters, flags or error word)")
        log(f"[bench] spot checks ok; chain vs separate launches: max rel diff {worst:.2e}")
    else:
        log(f"[bench] spot checks ok ({codec})")

    forms = {}
    if args.only in (None, "separate"):
        # separate launches, replayed from a HIP graph
        if args.no_graph:
            replay = lambda: launch_step(w4, gemvs, sh, codec)  # noqa: E731
        else:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=stream):
                launch_step(w4, gemvs, stream.cuda_stream, codec)
            torch.cuda.synchronize()
            replay = graph.replay
        forms["separate"] = time_loop(torch, stream, replay, args.warmup, args.steps) / sets
        log(f"[bench] separate launches ({'eager' if args.no_graph else 'graph'}): "
            f"{forms['separate'] * 1e6:.1f} us/step")
    if args.only in (None, "chain"):
        forms["chain"] = time_loop(torch, stream, chain_step, args.warmup, args.steps)
        # the error word is sticky: zero after the timed calls means every one was valid
        st, bits = w4.w4a16_chain_status_raw(ws_p, ws_bytes, sh, False)
        if st != w4.W4A16_OK:
            raise w4.W4A16Error(st, f"timed chain calls (error word {bits:#x})")
        log(f"[bench] chain: {forms['chain'] * 1e6:.1f} us/step")
    form = min(forms, key=forms.get)
    sec = forms[form]
    ms_per_step = sec * 1e3

    # The dominant kernel of the reported form: the chain kernel, or the
    # w4a16_gemv instantiation that moves the most bytes per step. Its launches
    # go through the *_timed entry points, which record the kernel's own start
    # and end into two HIP events on the launch stream: the average of their
    # elapsed times is the per-launch duration rocprofv3 reports for it.
    def timed_events():
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)   # creates the underlying HIP events
        b.record(stream)
        return a, b

    marks = []
    if form == "chain":
        kernel = w4.chain_launch_shape(M)["kernel"]
        launch_bytes = [step_bytes]
        launch_flops = [sum(2 * g["M"] * g["N"] * g["K"] for g in gemvs) // sets]
        with torch.cuda.stream(stream):
            for _ in range(args.steps):
                a, b = timed_events()
                st = w4.w4a16_gemv_chain_timed_raw(plan_p, count, M, ws_p, ws_bytes, sh, a.cuda_event, b.cuda_event)
                if st != 0:
                    raise w4.W4A16Error(st, "w4a16_gemv_chain_timed")
                marks.append((a, b))
    else:
        by_kernel = {}
        for g in gemvs:
            by_kernel[g["kernel"]] = by_kernel.get(g["kernel"], 0) + g["bytes"]
        kernel = max(by_kernel, key=by_kernel.get)
        launch_bytes = [g["bytes"] for g in gemvs if g["kernel"] == kernel]
        launch_flops = [2 * g["M"] * g["N"] * g["K"] for g in gemvs if g["kernel"] == kernel]
        with torch.cuda.stream(stream):
            for _ in range(max(1, args.steps // 4)):
                for g in gemvs:
                    if g["kernel"] == kernel:
                        a, b = timed_events()
                        st = w4.w4a16_codec_gemv_timed_raw(codec, g["xp"], g["pp"], g["yp"], g["M"], g["N"], g["K"],
                                                           sh, a.cuda_event, b.cuda_event)
                        if st != 0:
                            raise w4.W4A16Error(st, "w4a16_codec_gemv_timed")
                        marks.append((a, b))
                    else:
                        launch_step(w4, [g], sh, codec)
    torch.cuda.synchronize()
    avg_us = sum(a.elapsed_time(b) for a, b in marks) / len(marks) * 1e3
    per_launch = sum(launch_bytes) / len(launch_bytes)
    achieved = per_launch / (avg_us * 1e-6) / 1e9
    flops_per_launch = sum(launch_flops) / len(launch_flops)
    achieved_tflops = flops_per_launch / (avg_us * 1e-6) / 1e12
    # the roof the launch would hit first: streaming its bytes at the HBM peak,
    # or its 2*M*N*K flops at the vector peak (from M = 7 on)
    alu_bound = flops_per_launch / (VALU_PEAK_TFLOPS * 1e12) > per_launch / (HBM_PEAK_GBS * 1e9)
    hbm_view = {"achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    alu_view = {"achieved": round(achieved_tflops, 3), "peak": VALU_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved_tflops / VALU_PEAK_TFLOPS, 4)}
    log(f"[bench] {kernel}: avg {avg_us:.2f} us per launch, {per_launch / 1e6:.2f} MB per launch, "
        f"{achieved:.1f} GB/s")

    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": CODEC_DTYPE[codec],
        "data": "synthetic",
        "config": {
            "workload": f"{WORKLOAD_TEXT[wl]}, M={M}, " + CODEC_TEXT[codec],
            "gemvs_per_step": len(gemvs) // sets,
            "bytes_per_step": step_bytes,
            "launch": {"chain": "one w4a16_gemv_chain launch per step, products ordered on the device",
                       "separate": "%d %s launches per step, replayed from a HIP graph%s"
                                   % (len(gemvs) // sets, "w4a16_gemv" if codec == "q4" else "w4a16_codec_gemv",
                                      f" over {sets} seeded copies of the weights (time per copy)"
                                      if sets > 1 else "")}[form],
            "us_per_step_by_launch_form": {k: round(v * 1e6, 2) for k, v in forms.items()},
        },
        "system": system_info(torch, w4, dev),
        "roofline": {
            "bound": "alu" if alu_bound else "hbm",
            "kernel": kernel,
            **(alu_view if alu_bound else hbm_view),
            "traffic": TRAFFIC.get((wl, M, kernel)),
            "avg_launch_us": round(avg_us, 3),
            "bytes_per_launch": round(per_launch),
            "flops_per_launch": round(flops_per_launch),
            # the same launches against the other roof
            ("hbm" if alu_bound else "alu"): hbm_view if alu_bound else alu_view,
        },
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the fp64 oracle on host cores ...")
        line["cpu_baseline"] = cpu_baseline(args.cpu_budget, codec, wl, M)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
