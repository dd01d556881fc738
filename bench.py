#!/usr/bin/env python3
"""Benchmark of the fused-attention hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

Headline (``value``): causal GQA prefill, B=1, Hq=32, Hkv=8, Sq=Skv=2048,
d=128, bf16 -- algorithmic TFLOP/s over exactly K back-to-back calls of
fa_prefill (inputs resident in HBM, bracketed by device synchronisation),
after --settle-s seconds of untimed calls (the GPU clocks ramp up over about
half a second of load) and W untimed warmup calls.
Also reported on the same JSON line:
  - roofline of the prefill kernel: algorithmic FLOP per launch / mean launch
    duration (HIP events on the launch stream) against the bf16 dense MFMA peak;
    HBM traffic from the committed rocprofv3 counter summary when it was taken
    on the current kernel source, else null;
  - decode: contiguous 32k (B=4), paged mixed lengths (B=8) and long-context
    256k (B=1), over bf16, FP8 E4M3 and int8 caches: us/call (both kernels)
    and algorithmic HBM GB/s against 8 TB/s, two ways: each call timed alone
    after a 1 GiB read that evicts the 256 MB last-level cache (a read leaves
    no dirty lines behind), and sustained (calls back to back between one
    event pair, rotating over copies of the cache that hold at least 768 MiB
    together, so the cache comes from HBM); the decode roofline takes the
    sustained figure and shows the isolated one beside it;
  - us/call at B=1 for the fp32 single-head prefill and the bf16 prefill;
  - launch modes for the fp32 single-head prefill and the long-context decode:
    eager isolated, eager back-to-back and HIP-graph replay us/call;
  - ceilings: a plain streaming-read kernel's GB/s and an MFMA-loop kernel's
    bf16 TFLOP/s on the same GPU, the practical limits next to the peaks;
  - cpu_baseline: the fp64 oracle on the full prefill workload, host cores,
    repeated for about 10 s.
Only one GPU is used; --gpus above 1 exits with a message.
--prefill-only, --decode-only and --only LEG run one leg (for profiler passes).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (256 CU x 4096 FLOP/clk x 2.4 GHz)
PEAK_FP32_TFLOPS = 157.3  # MI355X dense fp32 (matrix and vector)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "prefill attn TFLOP/s + decode HBM GB/s (% of peak); µs/call at B=1"
PREFILL_KERNEL_SRC = os.path.join(ROOT, "attention_fa_prefill_amd", "csrc", "prefill_bf16.hip")
DECODE_KERNEL_SRC = os.path.join(ROOT, "attention_fa_prefill_amd", "csrc", "decode.hip")
COUNTERS = os.path.join(ROOT, "profiles", "hbm_counters.json")


def prefill_flops(B, Hq, Sq, Skv, d, causal):
    """Algorithmic FLOPs: 2*d for q.k plus 2*d for p*v per visible (query, key)."""
    if causal:
        off = Skv - Sq
        vis = sum(min(Skv, i + off + 1) for i in range(Sq))
    else:
        vis = Sq * Skv
    return 4 * d * Hq * B * vis


def prefill_bytes(B, Hq, Hkv, Sq, Skv, d, elt=2):
    return elt * (2 * B * Hq * Sq * d + 2 * B * Hkv * Skv * d)


def decode_bytes(case):
    """Algorithmic bytes: every cached K and V row once, q and o, seqlens, and the
    block-table entries of the pages used."""
    import numpy as np

    lens = np.clip(case.seqlens, 0, case.max_kv_len).astype(np.int64)
    es = 1 if (getattr(case, "fp8", False) or getattr(case, "int8", False)) else 2  # bytes per cached element
    b = es * 2 * case.Hkv * case.d * int(lens.sum()) + 2 * 2 * case.B * case.Hq * case.d + 4 * case.B
    if case.paged:
        b += 4 * int(((lens + 15) // 16).sum())
    return b


def sha(path):
    """Fingerprint of a kernel source's code: comments and blank space are
    dropped first, so that editing a comment does not void the counter data."""
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    code = "\n".join(" ".join(line.split()) for line in text.splitlines() if line.strip())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def traffic_for(kernel_key, src_path):
    """HBM bytes per launch from the committed counter summary, if it was taken on
    the current kernel source; else None."""
    try:
        with open(COUNTERS) as f:
            data = json.load(f)
        ent = data[kernel_key]
    except (OSError, KeyError, ValueError):
        return None
    if ent.get("source_sha") != sha(src_path):
        return None
    return ent.get("bytes_per_launch")


def smi_clocks_under_load(step, torch, samples=3, max_s=20.0):
    """Run `amd-smi metric -c --json` in a child process `samples` times while
    `step` is issued back to back; return the graphics clocks (per XCD, per
    sample, and their median over samples) and the memory clock it reports,
    or the error. The tool reads the clocks at one instant, so one sample can
    land in a short idle gap; the median over samples is the figure to use."""
    import subprocess
    import threading

    res = {"data": []}

    def query():
        try:
            for _ in range(samples):
                out = subprocess.run(["amd-smi", "metric", "-c", "--json"], capture_output=True, text=True,
                                     timeout=max_s).stdout
                res["data"].append(json.loads(out))
        except Exception as e:  # noqa: BLE001 - reported, never fatal
            res["error"] = repr(e)[:200]

    th = threading.Thread(target=query)
    t0 = time.perf_counter()
    th.start()
    while th.is_alive() and time.perf_counter() - t0 < samples * max_s:
        for _ in range(200):
            step()
        torch.cuda.synchronize()
    th.join()
    if not res["data"]:
        return {"source": "amd-smi metric -c --json", "error": res.get("error", "no output")}
    try:
        per_sample, mx, mem = [], [], []
        for d in res["data"]:
            clk = d["gpu_data"][0]["clock"]
            per_sample.append([v["clk"]["value"] for k, v in sorted(clk.items())
                               if k.startswith("gfx") and isinstance(v, dict)])
            mx += [v["max_clk"]["value"] for k, v in clk.items() if k.startswith("gfx") and isinstance(v, dict)]
            mem += [v["clk"]["value"] for k, v in clk.items() if k.startswith("mem") and isinstance(v, dict)
                    and isinstance(v.get("clk"), dict)]
        med = [statistics.median(x) for x in zip(*per_sample)]
        return {"source": "amd-smi metric -c --json, sampled during back-to-back headline calls",
                "gfx_mhz_per_xcd_median": med, "gfx_mhz_per_xcd_samples": per_sample,
                "gfx_max_mhz": max(mx) if mx else None, "mem_mhz": mem[0] if mem else None}
    except (KeyError, IndexError, TypeError, ValueError) as e:
        return {"source": "amd-smi metric -c --json", "error": "unexpected format: " + repr(e)[:100]}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-s", type=float, default=0.5,
                    help="untimed prefill calls for at least this long before the warmup steps, so that the "
                         "GPU clocks have left their idle state (they ramp up over ~0.5 s of load)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill-only", action="store_true", help="skip the decode and latency legs")
    ap.add_argument("--decode-only", action="store_true",
                    help="run only the decode leg and print its results (not the headline line)")
    ap.add_argument("--decode-reps", type=int, default=50)
    ap.add_argument("--only", choices=["prefill_cache", "head_dims", "f32_large", "decode_head_dims", "decode_d256"],
                    help="run only this leg and print its results (not the headline line); for profiler passes")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run 5 plain 256 MiB device-to-device copies (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (this path does not "
              f"shard across GPUs).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import attention_fa_prefill_amd as fa
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    if args.copy_calibration:
        # a plain copy of known size: 256 MiB read + 256 MiB written per dispatch
        src = torch.ones(1 << 28, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": 1 << 28, "dispatches": 5}), flush=True)
        return

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    def i32(x):
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(dev)

    import ctypes

    L = fa.lib()
    ctypes_stream = ctypes.c_void_p(stream.cuda_stream)

    # Eviction buffer: 1 GiB, four times the 256 MB last-level (Infinity)
    # cache. It is READ before each cold call: a write here would leave
    # dirty lines whose write-back would then compete with the timed
    # kernel's reads and understate its bandwidth.
    flush = None

    def timed_calls(fn, reps, evict):
        nonlocal flush
        if evict and flush is None:
            flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        times = []
        for _ in range(3):
            fn()
        for _ in range(reps):
            if evict:
                torch.amax(flush)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            b.synchronize()
            times.append(a.elapsed_time(b) * 1e3)
        return times

    def decode_leg(makers=(workloads.decode_contig_32k, workloads.decode_paged_mixed, workloads.decode_long_256k)):
        dec = {}
        cases = ([m() for m in makers] + [workloads.as_fp8(m()) for m in makers] +
                 [workloads.as_int8(m()) for m in makers])
        for dc in cases:
            if dc.fp8 or dc.int8:  # FP8 E4M3 or int8 codes, one byte per element
                dk = torch.from_numpy(np.ascontiguousarray(dc.kcache)).to(dev)
                dv = torch.from_numpy(np.ascontiguousarray(dc.vcache)).to(dev)
                dq = bf16(dc.q)
            else:
                dq, dk, dv = bf16(dc.q), bf16(dc.kcache), bf16(dc.vcache)
            lens = i32(dc.seqlens)
            bt = i32(dc.block_table) if dc.paged else None
            od = torch.empty_like(dq)
            # the default split size (0): the library may enlarge it on the device
            # from seqlens and reports the size it used at the end of the workspace
            need = fa.decode_workspace_bytes(dc.B, dc.Hq, dc.Hkv, dc.d, dc.max_kv_len, 0)
            ws = torch.empty(need, dtype=torch.uint8, device=dev)
            dargs = (ctypes.c_void_p(dq.data_ptr()), ctypes.c_void_p(dk.data_ptr()), ctypes.c_void_p(dv.data_ptr()),
                     ctypes.c_void_p(bt.data_ptr()) if bt is not None else None, ctypes.c_void_p(lens.data_ptr()),
                     ctypes.c_void_p(od.data_ptr()), dc.B, dc.Hq, dc.Hkv, dc.d, dc.max_kv_len,
                     16 if dc.paged else 0, 0, dc.scale, ctypes.c_void_p(ws.data_ptr()), need, ctypes_stream)

            def dcall(dargs=dargs, fp8=dc.fp8, int8=dc.int8, ks=dc.k_scale, vs=dc.v_scale):
                if fp8:
                    st = L.fa_decode_fp8(*dargs[:14], ks, vs, *dargs[14:])
                elif int8:
                    st = L.fa_decode_int8(*dargs[:14], ks, vs, *dargs[14:])
                else:
                    st = L.fa_decode(*dargs)
                if st != 0:
                    raise RuntimeError(fa.status_string(st))

            t = timed_calls(dcall, args.decode_reps, evict=True)
            t_warm = timed_calls(dcall, 20, evict=False)
            nbytes = decode_bytes(dc)
            # Sustained rate, as a serving loop issues decode steps: calls back
            # to back between one event pair, rotating over copies of the cache
            # that together hold at least 768 MiB (three times the 256 MB
            # last-level cache), so that every call reads a cache the previous
            # calls have pushed out of it.
            cache_bytes = dk.numel() * dk.element_size() + dv.numel() * dv.element_size()
            n_copy = max(2, -(-(768 << 20) // cache_bytes))
            copies = [(dk, dv)] + [(dk.clone(), dv.clone()) for _ in range(n_copy - 1)]
            rot = [dargs[:1] + (ctypes.c_void_p(ck.data_ptr()), ctypes.c_void_p(cv.data_ptr())) + dargs[3:]
                   for ck, cv in copies]
            n_sus = 10 * n_copy
            sus = []
            for _ in range(5):
                for ra in rot:
                    dcall(dargs=ra)
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                for i in range(n_sus):
                    dcall(dargs=rot[i % n_copy])
                b.record(stream)
                b.synchronize()
                sus.append(a.elapsed_time(b) * 1e3 / n_sus)
            us_sus = statistics.median(sus)
            del copies, rot
            p50 = statistics.median(t)
            tps = int(ws[need - 256:need - 252].view(torch.int32).item())
            dec[dc.name] = {"us_per_call_p50": round(p50, 2), "us_p10": round(float(np.percentile(t, 10)), 2),
                            "us_p90": round(float(np.percentile(t, 90)), 2),
                            "GB_per_s": round(nbytes / (p50 * 1e-6) / 1e9, 1),
                            "frac_of_hbm_peak": round(nbytes / (p50 * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                            "algorithmic_bytes": nbytes, "cache_evicted": "read 1 GiB before each call",
                            "us_per_call_p50_warm": round(statistics.median(t_warm), 2),
                            "us_per_call_sustained": round(us_sus, 2),
                            "GB_per_s_sustained": round(nbytes / (us_sus * 1e-6) / 1e9, 1),
                            "frac_of_hbm_peak_sustained": round(nbytes / (us_sus * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                            "sustained": f"{n_sus} calls back to back, rotating over {n_copy} copies of the cache "
                                         f"({n_copy * cache_bytes / 2**20:.0f} MiB), median of 5 runs",
                            "B": dc.B, "Hq": dc.Hq, "Hkv": dc.Hkv, "d": dc.d, "tokens": dc.total_tokens(),
                            "paged": dc.paged, "tokens_per_split": tps,
                            "splits_per_kv_head": int(sum(-(-min(int(x), dc.max_kv_len) // tps) for x in dc.seqlens)),
                            "kv_cache": "fp8_e4m3" if dc.fp8 else ("int8" if dc.int8 else "bf16")}
            if dc.fp8 or dc.int8:
                base = dec[dc.name[: -len("_fp8" if dc.fp8 else "_int8")]]
                dec[dc.name]["k_scale"], dec[dc.name]["v_scale"] = dc.k_scale, dc.v_scale
                dec[dc.name]["speedup_vs_bf16_cache"] = round(base["us_per_call_p50"] / p50, 3)
            del dq, dk, dv, ws, od, lens, bt
            torch.cuda.empty_cache()
        return dec

    def leg_prefill_cache():
        """chunked prefill over the paged cache of the chunk workload"""
        # chunked prefill over a paged KV cache (fa_prefill_cache): back-to-back
        # calls with the cache resident, the same timing as the headline
        pc = workloads.prefill_cache_chunk512()
        pq, pk, pv = bf16(pc.q), bf16(pc.kcache), bf16(pc.vcache)
        plens, pbt = i32(pc.seqlens), i32(pc.block_table)
        po = torch.empty_like(pq)
        pargs = (ctypes.c_void_p(pq.data_ptr()), ctypes.c_void_p(pk.data_ptr()), ctypes.c_void_p(pv.data_ptr()),
                 ctypes.c_void_p(pbt.data_ptr()), ctypes.c_void_p(plens.data_ptr()), ctypes.c_void_p(po.data_ptr()),
                 pc.B, pc.Hq, pc.Hkv, pc.Sq, pc.d, pc.max_kv_len, 16, pc.scale, 1, ctypes_stream)

        def pcall():
            st = L.fa_prefill_cache(*pargs)
            if st != 0:
                raise RuntimeError(fa.status_string(st))
        for _ in range(200):
            pcall()
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for _ in range(100):
            pcall()
        ev1.record(stream)
        ev1.synchronize()
        pc_us = ev0.elapsed_time(ev1) * 1e3 / 100
        pc_flop = sum(prefill_flops(1, pc.Hq, pc.Sq, int(L_), pc.d, True) for L_ in pc.seqlens)
        return {
            "workload": pc.name, "us_per_call_mean": round(pc_us, 2),
            "TFLOP_per_s": round(pc_flop / (pc_us * 1e-6) / 1e12, 1),
            "frac_of_bf16_peak": round(pc_flop / (pc_us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "algorithmic_flop_per_call": pc_flop, "B": pc.B, "Hq": pc.Hq, "Hkv": pc.Hkv, "Sq": pc.Sq, "d": pc.d,
            "cached_lengths": [int(x) for x in pc.seqlens], "paged": True, "causal": True,
            "note": "chunk of Sq new queries per sequence over its paged cache (chunk included); 100 back-to-back calls"}

    def leg_head_dims():
        """head dims 256, 96 and 32"""
        # head dims 256, 96 and 32: back-to-back calls, as above
        n_cus = torch.cuda.get_device_properties(0).multi_processor_count

        def hd_kernel_name(hc):
            # d = 32 takes the key-split kernel (four key parts on causal grids of at most 8 * CUs
            # 64-row tiles, else two); d = 256 takes it on causal grids under two rounds of 128-row
            # tiles with at least 10 tiles per head
            tiles = -(-hc.Sq // 128) * hc.Hq * hc.B
            if hc.d == 96:
                return "prefill_bf16_kernel<96, false>"
            if hc.d == 32:
                return "prefill_hd_ks_kernel<32, 4, false>" if -(-hc.Sq // 64) * hc.Hq * hc.B <= 8 * n_cus else \
                    "prefill_hd_ks_kernel<32, 2, false>"
            return ("prefill_hd_ks_kernel<256, 2, false>"
                    if hc.d == 256 and hc.causal and -(-hc.Sq // 128) >= 10 and tiles < 2 * n_cus
                    else f"prefill_hd_kernel<{hc.d}, false>")
        hd = {}
        for hc in (workloads.prefill_gqa_d256(), workloads.prefill_mha_d96(), workloads.prefill_gqa_d32()):
            hq_, hk_, hv_ = bf16(hc.q), bf16(hc.k), bf16(hc.v)
            ho = torch.empty_like(hq_)
            hargs = (ctypes.c_void_p(hq_.data_ptr()), ctypes.c_void_p(hk_.data_ptr()), ctypes.c_void_p(hv_.data_ptr()),
                     ctypes.c_void_p(ho.data_ptr()), hc.B, hc.Hq, hc.Hkv, hc.Sq, hc.Skv, hc.d, hc.scale, 1,
                     ctypes_stream)

            def hcall(hargs=hargs):
                st = L.fa_prefill(*hargs)
                if st != 0:
                    raise RuntimeError(fa.status_string(st))
            for _ in range(200):
                hcall()
            torch.cuda.synchronize()
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record(stream)
            for _ in range(100):
                hcall()
            ev1.record(stream)
            ev1.synchronize()
            h_us = ev0.elapsed_time(ev1) * 1e3 / 100
            h_flop = prefill_flops(hc.B, hc.Hq, hc.Sq, hc.Skv, hc.d, True)
            hd[hc.name] = {"us_per_call_mean": round(h_us, 2), "TFLOP_per_s": round(h_flop / (h_us * 1e-6) / 1e12, 1),
                           "frac_of_bf16_peak": round(h_flop / (h_us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4),
                           "algorithmic_flop_per_call": h_flop, "B": hc.B, "Hq": hc.Hq, "Hkv": hc.Hkv, "Sq": hc.Sq,
                           "d": hc.d, "causal": True, "kernel": hd_kernel_name(hc)}
            del hq_, hk_, hv_, ho
        return hd

    def leg_f32_large():
        """fp32 prefill at the C2 shape"""
        # fp32 prefill at the C2 shape (the matrix-core fp32 kernel), timed like
        # the head-dim legs, against the fp32 matrix peak
        fc = workloads.prefill_case(1, 32, 8, 2048, 2048, 128, True, "f32", seed=1002, scale=128 ** -0.5,
                                    name="prefill_f32_gqa_b1h32x8s2048d128")
        fq, fk, fv = (torch.from_numpy(x).to(dev) for x in (fc.q, fc.k, fc.v))
        fo = torch.empty_like(fq)
        fargs = (ctypes.c_void_p(fq.data_ptr()), ctypes.c_void_p(fk.data_ptr()), ctypes.c_void_p(fv.data_ptr()),
                 ctypes.c_void_p(fo.data_ptr()), 1, 32, 8, 2048, 2048, 128, fc.scale, 1, ctypes_stream)

        def fcall():
            st = L.fa_prefill_f32(*fargs)
            if st != 0:
                raise RuntimeError(fa.status_string(st))
        for _ in range(30):
            fcall()
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for _ in range(30):
            fcall()
        ev1.record(stream)
        ev1.synchronize()
        f_us = ev0.elapsed_time(ev1) * 1e3 / 30
        f_flop = prefill_flops(1, 32, 2048, 2048, 128, True)
        return {
            "workload": fc.name, "us_per_call_mean": round(f_us, 2),
            "TFLOP_per_s": round(f_flop / (f_us * 1e-6) / 1e12, 2),
            "frac_of_fp32_peak": round(f_flop / (f_us * 1e-6) / 1e12 / PEAK_FP32_TFLOPS, 4),
            "kernel": "prefill_f32_mfma_kernel<128>", "note": "30 back-to-back calls after 30 warm-up calls"}

    def leg_decode_head_dims():
        """decode at head dims 96 and 32 (padded LDS stage rows), the shape and lengths of the d = 256 leg"""
        return decode_leg(makers=(lambda: workloads.decode_paged_hd(96), lambda: workloads.decode_paged_hd(32)))

    def leg_decode_d256():
        """decode at head dim 256 (one split work-group per CU), bf16 and one-byte caches"""
        return decode_leg(makers=(workloads.decode_paged_d256,))

    if args.decode_only:
        print(json.dumps({"decode": decode_leg()}), flush=True)
        return
    if args.only:
        leg = {"prefill_cache": leg_prefill_cache, "head_dims": leg_head_dims, "f32_large": leg_f32_large,
               "decode_head_dims": leg_decode_head_dims, "decode_d256": leg_decode_d256}[args.only]
        print(json.dumps({args.only: leg()}), flush=True)
        return

    # ------------------------------------------------------------------ headline: GQA causal prefill
    case = workloads.prefill_gqa_2k()
    q, k, v = bf16(case.q), bf16(case.k), bf16(case.v)
    o = torch.empty_like(q)
    B, Hq, Hkv, Sq, Skv, d = case.B, case.Hq, case.Hkv, case.Sq, case.Skv, case.d
    argv = (ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
            ctypes.c_void_p(o.data_ptr()), B, Hq, Hkv, Sq, Skv, d, case.scale, 1, ctypes_stream)

    def step():
        st = L.fa_prefill(*argv)
        if st != 0:
            raise RuntimeError(fa.status_string(st))

    t_settle = time.perf_counter()
    n_settle = 0
    while time.perf_counter() - t_settle < args.settle_s:
        for _ in range(50):
            step()
        torch.cuda.synchronize()
        n_settle += 50
    # GPU clocks as the driver reports them, sampled (amd-smi, a child
    # process) while the headline call runs back to back
    clocks = smi_clocks_under_load(step, torch)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    # Timed region: K back-to-back calls between one pair of events on the
    # launch stream (no events in between, which would add their own gaps).
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for _ in range(K):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / K
    flops = prefill_flops(B, Hq, Sq, Skv, d, True)
    value = flops / (ms_per_step * 1e-3) / 1e12
    mean_launch_ms = ms_per_step  # one kernel per call: the mean launch duration over the timed region
    achieved = flops / (mean_launch_ms * 1e-3) / 1e12
    # separately: isolated calls, each between its own pair of events (latency per call)
    launch_ms = []
    for _ in range(min(K, 50)):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step()
        b.record(stream)
        b.synchronize()
        launch_ms.append(a.elapsed_time(b))
    traffic = traffic_for("prefill_bf16_kernel<128>@prefill_gqa_b1h32x8s2048d128", PREFILL_KERNEL_SRC)
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                "kernel": "prefill_bf16_kernel<128, false>", "mean_launch_us": round(mean_launch_ms * 1e3, 2),
                "algorithmic_flop_per_launch": flops,
                "algorithmic_bytes_per_launch": prefill_bytes(B, Hq, Hkv, Sq, Skv, d)}

    result = {"metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": K,
              "warmup": args.warmup, "settle_calls": n_settle, "ms_per_step": round(ms_per_step, 5),
              "higher_is_better": True,
              "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
              "config": {"workload": case.name, "B": B, "Hq": Hq, "Hkv": Hkv, "Sq": Sq, "Skv": Skv, "d": d,
                         "causal": True, "scale": case.scale, "seed": 1002},
              "roofline": roofline,
              "prefill_us_per_call_p50": round(statistics.median(launch_ms) * 1e3, 2),
              "gpu_clocks_under_load": clocks}

    # ------------------------------------------------------------------ decode and latency legs
    if not args.prefill_only:
        dec = decode_leg()
        result["decode"] = dec
        traffic_dec = traffic_for("decode_split_kernel<128>@decode_long_b1h16x2kv256kd128", DECODE_KERNEL_SRC)
        long = dec["decode_long_b1h16x2kv256kd128"]
        # achieved: the call's bytes over its mean duration in a timed region of
        # back-to-back calls whose caches come from HBM (the sustained figure);
        # the isolated call (its own event pair, caches evicted before it) is
        # reported beside it.
        result["roofline_decode"] = {"bound": "hbm", "achieved": long["GB_per_s_sustained"], "peak": PEAK_HBM_GBS,
                                     "unit": "GB/s", "frac": long["frac_of_hbm_peak_sustained"], "traffic": traffic_dec,
                                     "workload": "decode_long_b1h16x2kv256kd128",
                                     "isolated_call_GB_per_s": long["GB_per_s"],
                                     "isolated_call_frac": long["frac_of_hbm_peak"],
                                     "note": "split + merge kernels per call: " + long["sustained"] +
                                             "; isolated: one call between its own event pair after a 1 GiB read"}
        long8 = dec["decode_long_b1h16x2kv256kd128_fp8"]
        result["roofline_decode_fp8"] = {
            "bound": "hbm", "achieved": long8["GB_per_s_sustained"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": long8["frac_of_hbm_peak_sustained"],
            "traffic": traffic_for("decode_split_kernel<128, fp8>@decode_long_b1h16x2kv256kd128_fp8", DECODE_KERNEL_SRC),
            "workload": "decode_long_b1h16x2kv256kd128_fp8",
            "isolated_call_GB_per_s": long8["GB_per_s"], "isolated_call_frac": long8["frac_of_hbm_peak"],
            "note": "FP8 E4M3 cache (1 byte per element); split + merge kernels per call: " + long8["sustained"] +
                    "; isolated: one call between its own event pair after a 1 GiB read"}

        result["prefill_cache"] = leg_prefill_cache()
        result["prefill_head_dims"] = leg_head_dims()
        result["prefill_f32_large"] = leg_f32_large()

        # decode at head dim 256 (one split work-group per CU), bf16 and
        # one-byte caches, timed like the decode legs above
        result["decode_head_dim_256"] = leg_decode_d256()
        # decode at head dims 96 and 32 (padded LDS stage rows), the same shape
        result["decode_head_dims_96_32"] = leg_decode_head_dims()

        # fp32 single-head causal prefill at B=1 (launch-latency bound)
        c1 = workloads.prefill_f32_small()
        q1 = torch.from_numpy(c1.q).to(dev)
        k1 = torch.from_numpy(c1.k).to(dev)
        v1 = torch.from_numpy(c1.v).to(dev)
        o1 = torch.empty_like(q1)
        a1 = (ctypes.c_void_p(q1.data_ptr()), ctypes.c_void_p(k1.data_ptr()), ctypes.c_void_p(v1.data_ptr()),
              ctypes.c_void_p(o1.data_ptr()), 1, 1, 1, 128, 128, 64, c1.scale, 1, ctypes_stream)

        def c1call():
            st = L.fa_prefill_f32(*a1)
            if st != 0:
                raise RuntimeError(fa.status_string(st))

        t1 = timed_calls(c1call, 200, evict=False)
        # empty-work floor: the same stream, a 1-element fill (one trivial kernel)
        tiny = torch.empty(1, device=dev)
        tf = timed_calls(lambda: tiny.fill_(0.0), 200, evict=False)
        # decode of one chat-length sequence (B = 1, 4096 tokens), warm and cold
        cc = workloads.decode_b1_chat()
        qc, kcc, vcc = bf16(cc.q), bf16(cc.kcache), bf16(cc.vcache)
        lc, btc = i32(cc.seqlens), i32(cc.block_table)
        oc = torch.empty_like(qc)
        needc = fa.decode_workspace_bytes(cc.B, cc.Hq, cc.Hkv, cc.d, cc.max_kv_len, 0)
        wsc = torch.empty(needc, dtype=torch.uint8, device=dev)

        def cccall():
            st = L.fa_decode(ctypes.c_void_p(qc.data_ptr()), ctypes.c_void_p(kcc.data_ptr()),
                             ctypes.c_void_p(vcc.data_ptr()), ctypes.c_void_p(btc.data_ptr()),
                             ctypes.c_void_p(lc.data_ptr()), ctypes.c_void_p(oc.data_ptr()), cc.B, cc.Hq, cc.Hkv,
                             cc.d, cc.max_kv_len, 16, 0, cc.scale, ctypes.c_void_p(wsc.data_ptr()), needc,
                             ctypes_stream)
            if st != 0:
                raise RuntimeError(fa.status_string(st))

        tcw = timed_calls(cccall, 200, evict=False)
        tcc = timed_calls(cccall, args.decode_reps, evict=True)
        del qc, kcc, vcc, lc, btc, oc, wsc

        result["latency_b1"] = {
            c1.name: {"us_per_call_p50": round(statistics.median(t1), 2),
                      "us_p10": round(float(np.percentile(t1, 10)), 2)},
            "single_trivial_kernel_floor_us_p50": round(statistics.median(tf), 2),
            case.name: {"us_per_call_p50": result["prefill_us_per_call_p50"]},
            "decode_long_b1h16x2kv256kd128": {"us_per_call_p50": long["us_per_call_p50"]},
            cc.name: {"us_per_call_p50_warm": round(statistics.median(tcw), 2),
                      "us_per_call_p50_cold": round(statistics.median(tcc), 2),
                      "tokens_per_split": fa.decode_split_tokens(cc.B, cc.Hq, cc.Hkv, cc.max_kv_len, 0),
                      "algorithmic_bytes": decode_bytes(cc)},
        }

        # ------------------------------------------------------------------ launch modes (C1 and C5)
        # The same call issued three ways, all with inputs resident and caches
        # warm: eager and isolated (an event pair around each call), eager and
        # back-to-back (N calls between one event pair), and replayed from a HIP
        # graph that holds N back-to-back calls (the FlashRT summary's capture-
        # once, replay-per-token mechanism), plus a one-call graph replayed in
        # isolation.
        c5 = workloads.decode_long_256k()
        q5, k5, v5 = bf16(c5.q), bf16(c5.kcache), bf16(c5.vcache)
        lens5, bt5 = i32(c5.seqlens), i32(c5.block_table)
        o5 = torch.empty_like(q5)
        need5 = fa.decode_workspace_bytes(c5.B, c5.Hq, c5.Hkv, c5.d, c5.max_kv_len, 0)
        ws5 = torch.empty(need5, dtype=torch.uint8, device=dev)

        def c5call(st_handle):
            st = L.fa_decode(ctypes.c_void_p(q5.data_ptr()), ctypes.c_void_p(k5.data_ptr()),
                             ctypes.c_void_p(v5.data_ptr()), ctypes.c_void_p(bt5.data_ptr()),
                             ctypes.c_void_p(lens5.data_ptr()), ctypes.c_void_p(o5.data_ptr()), c5.B, c5.Hq, c5.Hkv,
                             c5.d, c5.max_kv_len, 16, 0, c5.scale, ctypes.c_void_p(ws5.data_ptr()), need5, st_handle)
            if st != 0:
                raise RuntimeError(fa.status_string(st))

        def c1call_on(st_handle):
            st = L.fa_prefill_f32(*a1[:-1], st_handle)
            if st != 0:
                raise RuntimeError(fa.status_string(st))

        def launch_modes(call, n=20, reps=100):
            cur = lambda: ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)  # noqa: E731
            iso = timed_calls(lambda: call(ctypes_stream), reps, evict=False)
            for _ in range(n):
                call(ctypes_stream)
            torch.cuda.synchronize()
            b2b = []
            for _ in range(5):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(reps):
                    call(ctypes_stream)
                e1.record(stream)
                e1.synchronize()
                b2b.append(e0.elapsed_time(e1) * 1e3 / reps)
            side = torch.cuda.Stream(device=dev)
            side.wait_stream(stream)
            with torch.cuda.stream(side):  # warm-up on a side stream before capture
                call(cur())
            stream.wait_stream(side)
            torch.cuda.synchronize()
            g_n, g_1 = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
            with torch.cuda.graph(g_n):
                for _ in range(n):
                    call(cur())
            with torch.cuda.graph(g_1):
                call(cur())
            torch.cuda.synchronize()
            for _ in range(3):
                g_n.replay()
            torch.cuda.synchronize()
            rep_n = []
            for _ in range(5):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(reps // n):
                    g_n.replay()
                e1.record(stream)
                e1.synchronize()
                rep_n.append(e0.elapsed_time(e1) * 1e3 / (n * (reps // n)))
            rep_1 = timed_calls(lambda: g_1.replay(), reps, evict=False)
            del g_n, g_1
            return {"eager_isolated_us_p50": round(statistics.median(iso), 2),
                    "eager_back_to_back_us_per_call": round(statistics.median(b2b), 2),
                    "graph_replay_back_to_back_us_per_call": round(statistics.median(rep_n), 2),
                    "graph_replay_one_call_isolated_us_p50": round(statistics.median(rep_1), 2),
                    "graph_calls_per_replay": n}

        # a short-context serving batch: one split per sequence, so fa_decode
        # is one launch (no merge kernel)
        cb = workloads.decode_batch_short()
        qb, kb, vb = bf16(cb.q), bf16(cb.kcache), bf16(cb.vcache)
        lensb, btb = i32(cb.seqlens), i32(cb.block_table)
        ob = torch.empty_like(qb)
        needb = fa.decode_workspace_bytes(cb.B, cb.Hq, cb.Hkv, cb.d, cb.max_kv_len, 0)
        wsb = torch.empty(needb, dtype=torch.uint8, device=dev)
        assert fa.decode_split_tokens(cb.B, cb.Hq, cb.Hkv, cb.max_kv_len, 0) >= cb.max_kv_len

        def cbcall(st_handle):
            st = L.fa_decode(ctypes.c_void_p(qb.data_ptr()), ctypes.c_void_p(kb.data_ptr()),
                             ctypes.c_void_p(vb.data_ptr()), ctypes.c_void_p(btb.data_ptr()),
                             ctypes.c_void_p(lensb.data_ptr()), ctypes.c_void_p(ob.data_ptr()), cb.B, cb.Hq, cb.Hkv,
                             cb.d, cb.max_kv_len, 16, 0, cb.scale, ctypes.c_void_p(wsb.data_ptr()), needb, st_handle)
            if st != 0:
                raise RuntimeError(fa.status_string(st))

        result["launch_modes"] = {
            c1.name: launch_modes(c1call_on),
            c5.name: launch_modes(c5call),
            cb.name: launch_modes(cbcall),
            "note": "inputs resident, caches warm; back-to-back figures are the mean over 100 calls (median of 5 "
                    "runs); the graph holds 20 calls and is replayed 5 times per run; isolated figures are the "
                    "median of 100 calls, each between its own event pair"}
        # the same batch through split kernel + merge kernel: a block table
        # twice as wide (capacity 2048, split size 1024) gives two splits per
        # sequence, the second always empty, i.e. the same work plus the merge
        btw = torch.zeros((cb.B, 2 * btb.shape[1]), dtype=torch.int32, device=dev)
        btw[:, : btb.shape[1]] = btb
        needw = fa.decode_workspace_bytes(cb.B, cb.Hq, cb.Hkv, cb.d, 2 * cb.max_kv_len, cb.max_kv_len)
        wsw = torch.empty(needw, dtype=torch.uint8, device=dev)

        def cbcall_two():
            st = L.fa_decode(ctypes.c_void_p(qb.data_ptr()), ctypes.c_void_p(kb.data_ptr()),
                             ctypes.c_void_p(vb.data_ptr()), ctypes.c_void_p(btw.data_ptr()),
                             ctypes.c_void_p(lensb.data_ptr()), ctypes.c_void_p(ob.data_ptr()), cb.B, cb.Hq, cb.Hkv,
                             cb.d, 2 * cb.max_kv_len, 16, cb.max_kv_len, cb.scale, ctypes.c_void_p(wsw.data_ptr()),
                             needw, ctypes_stream)
            if st != 0:
                raise RuntimeError(fa.status_string(st))

        nb = decode_bytes(cb)
        one_c = statistics.median(timed_calls(lambda: cbcall(ctypes_stream), args.decode_reps, evict=True))
        two_c = statistics.median(timed_calls(cbcall_two, args.decode_reps, evict=True))
        one_w = statistics.median(timed_calls(lambda: cbcall(ctypes_stream), 50, evict=False))
        two_w = statistics.median(timed_calls(cbcall_two, 50, evict=False))
        result["decode_one_launch"] = {
            "workload": cb.name, "algorithmic_bytes": nb,
            "one_launch_us_p50": round(one_c, 2), "split_plus_merge_us_p50": round(two_c, 2),
            "one_launch_GB_per_s": round(nb / (one_c * 1e-6) / 1e9, 1),
            "one_launch_us_p50_warm": round(one_w, 2), "split_plus_merge_us_p50_warm": round(two_w, 2),
            "note": "one split per sequence: the split kernel writes o (one launch); the comparison runs the same "
                    "splits through split kernel + merge kernel; caches evicted before each call (warm: not)"}
        del q5, k5, v5, lens5, bt5, o5, ws5, qb, kb, vb, lensb, btb, ob, wsb, btw, wsw
        torch.cuda.empty_cache()

        # ------------------------------------------------------------------ practical ceilings
        C = ctypes.CDLL(os.path.join(ROOT, "attention_fa_prefill_amd", "libfa_ceiling.so"))
        C.fa_ceiling_read.argtypes = [ctypes.c_void_p, ctypes.c_long, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
        C.fa_ceiling_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        rbuf = torch.ones(1 << 27, dtype=torch.float32, device=dev)  # 512 MiB
        rbytes = rbuf.numel() * 4
        sink = torch.zeros(1 << 16, dtype=torch.int32, device=dev)

        def read_call():
            if C.fa_ceiling_read(ctypes.c_void_p(rbuf.data_ptr()), rbytes, ctypes.c_void_p(sink.data_ptr()), 2048,
                                 ctypes_stream) != 0:
                raise RuntimeError("ceiling read kernel launch failed")

        mm_grid, mm_rounds = 512, 1000
        mm_flop = mm_grid * 4 * 8 * mm_rounds * 32768

        def mfma_call(normal):
            if C.fa_ceiling_mfma(ctypes.c_void_p(sink.data_ptr()), mm_grid, mm_rounds, normal, ctypes_stream) != 0:
                raise RuntimeError("ceiling mfma kernel launch failed")

        t_rd = statistics.median(timed_calls(read_call, 20, evict=True))
        t_mm = statistics.median(timed_calls(lambda: mfma_call(0), 10, evict=False))
        t_mn = statistics.median(timed_calls(lambda: mfma_call(1), 10, evict=False))
        del rbuf
        torch.cuda.empty_cache()
        result["ceilings"] = {
            "stream_read_GB_per_s": round(rbytes / (t_rd * 1e-6) / 1e9, 1),
            "stream_read_frac_of_hbm_peak": round(rbytes / (t_rd * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "mfma_loop_bf16_TFLOP_per_s": round(mm_flop / (t_mm * 1e-6) / 1e12, 1),
            "mfma_loop_frac_of_bf16_peak": round(mm_flop / (t_mm * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "mfma_loop_bf16_normal_data_TFLOP_per_s": round(mm_flop / (t_mn * 1e-6) / 1e12, 1),
            "mfma_loop_normal_data_frac_of_bf16_peak": round(mm_flop / (t_mn * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "note": "plain 512 MiB streaming read (caches evicted) and an 8-chain v_mfma_f32_32x32x16_bf16 loop on "
                    "small integer operands and on N(0,1)-like bf16 operands (the matrix core's power, and so the "
                    "clock, depends on the operand bits), timed per call with HIP events like the attention calls"}

    # ------------------------------------------------------------------ CPU baseline: the oracle
    if not args.no_cpu_baseline:
        import oracle

        qf, kf, vf = case.as_f64()
        runs = []
        t_all = time.perf_counter()
        while not runs or time.perf_counter() - t_all < 10.0:
            t0 = time.perf_counter()
            oracle.attention(qf, kf, vf, case.scale, True)
            runs.append(time.perf_counter() - t0)
        dt = statistics.median(runs)
        result["cpu_baseline"] = {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s",
                                  "cores": oracle.num_threads(), "kind": "oracle",
                                  "sample": f"the whole {case.name} workload (fp64), {len(runs)} runs in "
                                            f"{sum(runs):.1f} s, median {dt:.3f} s per run"}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
