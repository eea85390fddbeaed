#!/usr/bin/env python3
"""Benchmark of the ATMA global-layer hot path on one MI355X.

One step = the gated-delta memory prefill plus the causal Polar attention prefill over
one batch of the 378M-class layer at the 2K training length (B=8, T=2048; memory: 8 heads
of width 128; Polar: 16 heads of width 64; bf16 operands, fp32 state and statistics),
inputs resident in HBM (three input sets used in turn, so no step reads inputs the previous
step left in the last-level cache).  Throughput = B*T tokens per step.

Also reported (secondary, fewer steps): the 64K prefill and one decode step against a
262144-token KV cache at batch 1 and 16 (Polar decode + memory decode step).

Prints one JSON line.  ``--gpus`` above 1 is refused: the library runs on one GPU.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tokens/sec gated-delta+Polar fwd at T=2K/64K/256K; % MFMA or HBM roofline"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
NSETS = 3  # input sets the headline step rotates through
PEAK_FP32_MFMA_TFLOPS = 157.3


def polar_flops(B, T, Hq, D=64):
    # QK^T and PV multiply-adds over the causal pairs (diagonal included), 2 flops each
    return 4.0 * D * B * Hq * T * (T + 1) / 2


def gdn_bytes(B, T, H, D=128, es=2):
    # q, k, v read + o written (es bytes each) and alpha, beta (fp32) per token and head,
    # plus the final fp32 state
    return B * H * T * (4 * D * es + 8) + B * H * D * D * 4


def gdn_fwd_flops(B, T, H, D=128, C=64):
    # chunked forward's products per token and head: C(3 Dk + 2 Dv) + 6 Dk Dv + C^2/3 (Dk = Dv = D;
    # triangular halves counted once)
    return B * H * T * (C * 5 * D + 6 * D * D + C * C / 3)


def gdn_bwd_flops(B, T, H, D=128, C=64):
    # every forward product has two operand gradients of its own size: twice the forward
    return 2 * gdn_fwd_flops(B, T, H, D, C)


def decode_bytes(B, L, Hkv=16, D=64, H=8, Dg=128):
    # K and V cache read once (bf16) + memory state read and written (fp32)
    return 2 * B * L * Hkv * D * 2 + 2 * B * H * Dg * Dg * 4


# HBM traffic of the dominant kernel per launch, from two rocprofv3 --pmc runs of this script
# (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch) scaled by what the same counters read for a
# device copy of known size; keyed by the SHA-256 of the kernel's sources at the time the
# counters were taken, so an edited kernel reports null until it is measured again.
MEASURED_TRAFFIC = {
    # layer_b8_t2k: FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0 KiB per dispatch (profiles/polar_fwd_layer_b8_t2k.txt)
    "polar_fwd_kernel": {"sha": "e5540cc82bc0cca1", "bytes": 185649366},
    # layer_b8_t2k, prep + carry (one segment at this shape; the carry forms the output)
    "atma_gdn_fwd (prep+carry+out)": {"sha": "402753ebac569130", "bytes": 444711826},
    # layer_b8_t2k backward: prep + both walks + pre + post (profiles/gdn_bwd_layer_b8_t2k.txt)
    "atma_gdn_bwd (all kernels)": {"sha": "435838d3e9475fec", "bytes": 3556505114},
}


def _sources_sha(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "gated_delta_memory_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


KERNEL_SOURCES = {"polar_fwd_kernel": ["polar_fwd.hip", "atma_device.hpp"],
                  "atma_gdn_bwd (all kernels)": ["gdn_bwd.hip", "gdn_common.hpp", "atma_device.hpp"],
                  "atma_gdn_fwd (prep+carry+out)": ["gdn_fwd.hip", "gdn_fwd_bf16.hip", "gdn_common.hpp",
                                                    "atma_device.hpp"]}


def measured_traffic(kernel):
    m = MEASURED_TRAFFIC.get(kernel)
    if m is None or m["sha"] != _sources_sha(KERNEL_SOURCES[kernel]):
        return None
    return m["bytes"]


def calibration_copy(torch, mib):
    """A plain device-to-device copy of `mib` MiB, three times: the reference dispatch that
    scales the FETCH_SIZE / WRITE_SIZE counters to bytes."""
    n = mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


class Timer:
    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def __call__(self, fn):
        e0 = self.torch.cuda.Event(enable_timing=True)
        e1 = self.torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        self.pairs.append((e0, e1))

    def mean_ms(self):
        return sum(a.elapsed_time(b) for a, b in self.pairs) / max(1, len(self.pairs))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # about 0.1 s of untimed steps: the GPU's clocks reach their steady state under load only after
    # that (with 5 warm-up steps the same step measured about 8% slower)
    ap.add_argument("--warmup", type=int, default=400)
    ap.add_argument("--no-secondary", action="store_true", help="skip the 64K prefill and 256K decode lines")
    ap.add_argument("--sections", default=",".join(SECTIONS),
                    help="comma-separated secondary sections to run (default: all): " + ", ".join(SECTIONS))
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--calib-copy", type=int, default=0, metavar="MIB",
                    help="first run a plain device copy of MIB MiB three times (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: the library runs on one GPU only; --gpus must be 1 (sharding across GPUs "
              "is not built)", file=sys.stderr)
        sys.exit(2)

    import torch

    import gated_delta_memory_amd as atma
    import workloads

    dev = "cuda"
    if args.calib_copy:
        calibration_copy(torch, args.calib_copy)
    w = workloads.WORKLOADS["layer_b8_t2k"]
    B, T = w.B, w.T
    # NSETS independent input/output sets (seeds w.seed + i), step s using set s % NSETS: their
    # ~400 MB exceed the 256 MB last-level cache, so a step cannot be served from the previous
    # step's cached inputs.
    sets = []
    for i in range(NSETS):
        inp = workloads.make_workload(dataclasses.replace(w, seed=w.seed + i), device=dev)
        g, p = inp["gdn"], inp["polar"]
        sets.append({"g": g, "p": p, "o_g": torch.empty_like(g["v"]), "o_p": torch.empty_like(p["q"]),
                     "S_g": torch.empty(B, w.gdn_H, w.gdn_D, w.gdn_D, dtype=torch.float32, device=dev)})
    ws_g = torch.empty(atma.atma_gdn_fwd_workspace_bytes(B, T, w.gdn_H, w.gdn_D, w.gdn_D), dtype=torch.uint8,
                       device=dev)
    cur = [0]

    def gdn(stream=None):
        st = sets[cur[0] % NSETS]
        g = st["g"]
        atma.atma_gdn_fwd(g["q"], g["k"], g["v"], g["alpha"], g["beta"], o=st["o_g"], final_state=st["S_g"],
                          workspace=ws_g, stream=stream)

    def polar(stream=None):
        st = sets[cur[0] % NSETS]
        p = st["p"]
        atma.atma_polar_attn_fwd(p["q"], p["k"], p["v"], p["params"], o=st["o_p"], stream=stream)

    for i in range(args.warmup):
        cur[0] = i
        gdn()
        polar()
    torch.cuda.synchronize()

    # timed region: exactly `steps` steps, synchronised on both sides.  Events bracket every launch
    # of the Polar kernel (the roofline kernel) and nothing else: each recorded event costs the
    # step a few microseconds (events around both calls made the step about 6% slower, around the
    # Polar call alone about 2%), so the memory call's own time is taken in a second event-timed
    # pass over the same steps after the timed region.
    tg, tp = Timer(torch), Timer(torch)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        cur[0] = i
        gdn()
        tp(polar)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / args.steps
    value = B * T * args.steps / elapsed
    polar_ms = tp.mean_ms()
    for i in range(args.steps):
        cur[0] = i
        tg(gdn)
        polar()
    torch.cuda.synchronize()
    gdn_ms = tg.mean_ms()

    pf = polar_flops(B, T, w.polar_Hq)
    gb = gdn_bytes(B, T, w.gdn_H, w.gdn_D)
    polar_tflops = pf / (polar_ms * 1e-3) / 1e12
    gdn_gbs = gb / (gdn_ms * 1e-3) / 1e9
    # The step's longest single kernel is the Polar prefill kernel (the memory call is three
    # shorter kernels: prep, carry, output; see the rocprofv3 summaries), so it carries the
    # roofline object; the memory call's HBM fraction is reported beside it.
    roofline = {"kernel": "polar_fwd_kernel", "bound": "mfma", "achieved": round(polar_tflops, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(polar_tflops / PEAK_BF16_TFLOPS, 4),
                "traffic": measured_traffic("polar_fwd_kernel"), "launch_ms": round(polar_ms, 4),
                "per_launch": f"{pf:.4e} flop = 4*64*B*Hq*T(T+1)/2, B={B} T={T} Hq={w.polar_Hq}"}
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "B": B, "T": T, "gdn_heads": w.gdn_H, "gdn_head_dim": w.gdn_D,
                   "polar_heads": w.polar_Hq, "polar_kv_heads": w.polar_Hkv, "polar_head_dim": w.polar_D,
                   "chunk": w.chunk, "state": "fp32"},
        "roofline": roofline,
        "breakdown_ms": {"gdn_fwd": round(gdn_ms, 4), "polar_fwd": round(polar_ms, 4),
                         "gdn_hbm_GBps": round(gdn_gbs, 1), "gdn_hbm_frac": round(gdn_gbs / PEAK_HBM_GBS, 4),
                         "gdn_bytes_per_call": f"{gb:.4e} B = B*H*T*(4*D*2+8) + B*H*D*D*4",
                         "gdn_traffic": measured_traffic("atma_gdn_fwd (prep+carry+out)"),
                         "polar_TFLOPs": round(polar_tflops, 2)},
    }
    # The memory and Polar calls are independent given their inputs: the same step with the memory
    # call on a second stream (default priority) overlapping the Polar call.
    if not args.no_secondary:
        side = torch.cuda.Stream()
        main_s = torch.cuda.current_stream()

        def step2():
            side.wait_stream(main_s)
            gdn(stream=side)
            polar(stream=main_s)
            main_s.wait_stream(side)

        for i in range(args.warmup):
            cur[0] = i
            step2()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            cur[0] = i
            step2()
        torch.cuda.synchronize()
        el2 = time.perf_counter() - t0
        out["two_streams"] = {"tokens_per_s": round(B * T * args.steps / el2, 1),
                              "ms_per_step": round(el2 * 1e3 / args.steps, 4),
                              "note": "memory call on a second stream overlapping the Polar call"}
    del inp, g, p, sets, ws_g
    torch.cuda.empty_cache()

    if not args.no_secondary:
        out["secondary"] = secondary(torch, atma, workloads, sections=args.sections.split(","))
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


SECTIONS = ("cores", "polar_d128", "canon", "polar_train", "gdn_train", "prefill_64k", "prefill_256k", "decode")


def secondary(torch, atma, workloads, sections=SECTIONS):
    res = {}

    def want(name):
        return name in sections

    if want("cores"):
        # the matched control cores (NoPE / RoPE causal softmax attention) beside Polar, 2K layer shape
        w = workloads.WORKLOADS["layer_b8_t2k"]
        p = workloads.make_workload(w, device="cuda")["polar"]
        o_p = torch.empty_like(p["q"])
        ws_r = torch.empty(int(atma.lib.atma_softmax_attn_workspace_bytes(w.B, w.T, w.polar_Hq, w.polar_Hkv, 64,
                                                                           10000.0)), dtype=torch.uint8, device="cuda")
        tpo, tno, tro = Timer(torch), Timer(torch), Timer(torch)
        for it in range(21):
            (tpo if it else (lambda f: f()))(lambda: atma.atma_polar_attn_fwd(p["q"], p["k"], p["v"], p["params"], o=o_p))
            (tno if it else (lambda f: f()))(lambda: atma.atma_softmax_attn_fwd(p["q"], p["k"], p["v"], 0.0, o=o_p))
            (tro if it else (lambda f: f()))(lambda: atma.atma_softmax_attn_fwd(p["q"], p["k"], p["v"], 10000.0, o=o_p,
                                                                                workspace=ws_r))
        torch.cuda.synchronize()
        pf = polar_flops(w.B, w.T, w.polar_Hq)
        res["cores_" + w.name] = {"polar_ms": round(tpo.mean_ms(), 4), "nope_ms": round(tno.mean_ms(), 4),
                                  "rope_ms": round(tro.mean_ms(), 4),
                                  "nope_mfma_frac": round(pf / (tno.mean_ms() * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        del p, o_p, ws_r
        torch.cuda.empty_cache()
    if want("polar_d128"):
        # the real model's attention layout: 8 query / 2 kv heads at head width 128
        for (B, T, name, reps) in ((8, 2048, "polar_d128_gqa_b8_t2k", 21), (1, 65536, "polar_d128_gqa_b1_t64k", 4)):
            p = workloads.make_polar_inputs(B, T, 8, 2, 128, device="cuda")
            o_p = torch.empty_like(p["q"])
            tq = Timer(torch)
            for it in range(reps):
                (tq if it else (lambda f: f()))(lambda: atma.atma_polar_attn_fwd(p["q"], p["k"], p["v"], p["params"], o=o_p))
            torch.cuda.synchronize()
            fl = 4 * 128 * B * 8 * T * (T + 1) / 2
            res[name] = {"polar_ms": round(tq.mean_ms(), 4),
                         "polar_mfma_frac": round(fl / (tq.mean_ms() * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
            del p, o_p
            torch.cuda.empty_cache()
    if want("canon"):
        # Canon prologue (depthwise causal convolution, 4 taps, residual, per-head unit norm) on the
        # query projection of the 8/2-head, D = 128 layout at the 2K shape: algorithmic bytes are one
        # read of x and one write of y (bf16), the taps and the carried state are negligible
        B, T, Cq, K = 8, 2048, 8 * 128, 4
        gen = torch.Generator(device="cuda").manual_seed(5)
        x = torch.randn(B, T, Cq, device="cuda", generator=gen).to(torch.bfloat16)
        wc = torch.randn(K, Cq, device="cuda", generator=gen) * 0.5
        st = torch.zeros(B, K - 1, Cq, device="cuda", dtype=torch.bfloat16)
        yc = torch.empty_like(x)
        # the kernel is shorter than the binding's host-side checks, so 50 calls are queued back to
        # back between one pair of events (an event pair around a single call would time the host)
        call = lambda: atma.atma_canon(x, wc, st, residual=True, heads=8, update_state=False, y=yc)
        call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(50):
            call()
        e1.record()
        torch.cuda.synchronize()
        cms = e0.elapsed_time(e1) / 50
        cb = 2 * B * T * Cq * 2
        res["canon_q_d128_b8_t2k"] = {"canon_us": round(cms * 1e3, 2), "bytes": cb,
                                      "hbm_frac": round(cb / (cms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        del x, wc, st, yc
        torch.cuda.empty_cache()
    if want("polar_train"):
        # training step of the Polar core (training forward + backward) at the 2K layer shapes; the
        # backward's algorithmic work is the usual five products per visible (query, key) pair
        # (S recomputed, dP, dV, dK, dQ): 10 D flop per pair per head
        for (B, T, Hq, Hkv, D, name) in ((8, 2048, 16, 16, 64, "polar_train_layer_b8_t2k"),
                                         (8, 2048, 8, 2, 128, "polar_train_d128_gqa_b8_t2k")):
            p = workloads.make_polar_inputs(B, T, Hq, Hkv, D, device="cuda")
            do = torch.randn(B, T, Hq, D, device="cuda").to(torch.bfloat16)
            f = dict(dtype=torch.float32, device="cuda")
            gout = {"dq": torch.empty_like(p["q"]), "dk": torch.empty_like(p["k"]), "dv": torch.empty_like(p["v"]),
                    "d_temp_raw": torch.empty(Hq, **f), "d_null_slope_raw": torch.empty(Hq, **f),
                    "d_null_bias": torch.empty(Hq, **f), "d_mag_beta": torch.empty(Hq, **f),
                    "d_v_null": torch.empty(Hq, D, **f)}
            ws_b = torch.empty(int(atma.lib.atma_polar_attn_bwd_workspace_bytes(B, T, Hq, Hkv, D)), dtype=torch.uint8,
                               device="cuda")
            fw = {}
            tf, tb = Timer(torch), Timer(torch)

            def fwd_train():
                fw["o"], fw["mu"], fw["st"], fw["dir"] = atma.atma_polar_attn_fwd_train(p["q"], p["k"], p["v"],
                                                                                        p["params"])

            def bwd():
                atma.atma_polar_attn_bwd(p["q"], p["k"], p["v"], p["params"], fw["mu"], fw["st"], fw["dir"], do,
                                         out=gout, workspace=ws_b)

            for it in range(11):
                (tf if it else (lambda fn: fn()))(fwd_train)
                (tb if it else (lambda fn: fn()))(bwd)
            torch.cuda.synchronize()
            pairs = B * Hq * T * (T + 1) / 2
            res[name] = {"fwd_train_ms": round(tf.mean_ms(), 4), "bwd_ms": round(tb.mean_ms(), 4),
                         "bwd_TFLOPs": round(10 * D * pairs / (tb.mean_ms() * 1e-3) / 1e12, 2),
                         "bwd_mfma_frac": round(10 * D * pairs / (tb.mean_ms() * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                         "tokens_per_s": round(B * T / ((tf.mean_ms() + tb.mean_ms()) * 1e-3), 1)}
            del p, do, gout, ws_b, fw
            torch.cuda.empty_cache()
    if want("gdn_train"):
        # memory backward at the 2K layer shape (B=8, H=8, d=128, bf16 inputs, fp32 arithmetic)
        w = workloads.WORKLOADS["layer_b8_t2k"]
        g = workloads.make_workload(w, device="cuda")["gdn"]
        do = torch.randn_like(g["v"])
        ws_gb = torch.empty(int(atma.lib.atma_gdn_bwd_workspace_bytes(w.B, w.T, w.gdn_H, w.gdn_D, w.gdn_D, 64, 1)),
                            dtype=torch.uint8, device="cuda")
        tgb = Timer(torch)
        for it in range(6):
            (tgb if it else (lambda fn: fn()))(lambda: atma.atma_gdn_bwd(g["q"], g["k"], g["v"], g["alpha"], g["beta"], do,
                                                                         workspace=ws_gb))
        torch.cuda.synchronize()
        bf = gdn_bwd_flops(w.B, w.T, w.gdn_H, w.gdn_D)
        tf = bf / (tgb.mean_ms() * 1e-3) / 1e12
        res["gdn_train_" + w.name] = {
            "bwd_ms": round(tgb.mean_ms(), 4), "workspace_MB": round(ws_gb.numel() / 2 ** 20, 1),
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_FP32_MFMA_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / PEAK_FP32_MFMA_TFLOPS, 4),
                         "traffic": measured_traffic("atma_gdn_bwd (all kernels)"),
                         "per_launch": f"{bf:.4e} flop = 2 x B*H*T*(C(3D+2D) + 6D^2 + C^2/3), B={w.B} T={w.T} "
                                       f"H={w.gdn_H} D={w.gdn_D} C=64 (twice the chunked forward's products)"}}
        del g, do, ws_gb
        torch.cuda.empty_cache()
    if want("prefill_64k"):
        # 64K prefill
        w = workloads.WORKLOADS["prefill_b1_t64k"]
        inp = workloads.make_workload(w, device="cuda")
        g, p = inp["gdn"], inp["polar"]
        o_g = torch.empty_like(g["v"])
        ws_g = torch.empty(atma.atma_gdn_fwd_workspace_bytes(w.B, w.T, w.gdn_H, w.gdn_D, w.gdn_D), dtype=torch.uint8,
                           device="cuda")
        S_g = torch.empty(w.B, w.gdn_H, w.gdn_D, w.gdn_D, device="cuda")
        o_p = torch.empty_like(p["q"])
        tg, tp = Timer(torch), Timer(torch)
        for it in range(4):
            (tg if it else (lambda f: f()))(lambda: atma.atma_gdn_fwd(g["q"], g["k"], g["v"], g["alpha"], g["beta"],
                                                                      o=o_g, final_state=S_g, workspace=ws_g))
            (tp if it else (lambda f: f()))(lambda: atma.atma_polar_attn_fwd(p["q"], p["k"], p["v"], p["params"], o=o_p))
        torch.cuda.synchronize()
        gm, pm = tg.mean_ms(), tp.mean_ms()
        pf = polar_flops(w.B, w.T, w.polar_Hq)
        res[w.name] = {"tokens_per_s": round(w.B * w.T / ((gm + pm) * 1e-3), 1), "gdn_ms": round(gm, 3),
                       "polar_ms": round(pm, 3), "polar_mfma_frac": round(pf / (pm * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                       "gdn_hbm_frac": round(gdn_bytes(w.B, w.T, w.gdn_H) / (gm * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        del inp, g, p, o_g, ws_g, S_g, o_p
        torch.cuda.empty_cache()
    if want("prefill_256k"):
        # 256K prefill, once (one warm-up, one timed call of each)
        w = workloads.WORKLOADS["prefill_b1_t256k"]
        inp = workloads.make_workload(w, device="cuda")
        g, p = inp["gdn"], inp["polar"]
        o_g = torch.empty_like(g["v"])
        ws_g = torch.empty(atma.atma_gdn_fwd_workspace_bytes(w.B, w.T, w.gdn_H, w.gdn_D, w.gdn_D), dtype=torch.uint8,
                           device="cuda")
        S_g = torch.empty(w.B, w.gdn_H, w.gdn_D, w.gdn_D, device="cuda")
        o_p = torch.empty_like(p["q"])
        tg, tp = Timer(torch), Timer(torch)
        for it in range(2):
            (tg if it else (lambda f: f()))(lambda: atma.atma_gdn_fwd(g["q"], g["k"], g["v"], g["alpha"], g["beta"],
                                                                      o=o_g, final_state=S_g, workspace=ws_g))
            (tp if it else (lambda f: f()))(lambda: atma.atma_polar_attn_fwd(p["q"], p["k"], p["v"], p["params"], o=o_p))
        torch.cuda.synchronize()
        gm, pm = tg.mean_ms(), tp.mean_ms()
        pf = polar_flops(w.B, w.T, w.polar_Hq)
        res[w.name] = {"tokens_per_s": round(w.B * w.T / ((gm + pm) * 1e-3), 1), "gdn_ms": round(gm, 3),
                       "polar_ms": round(pm, 3), "polar_mfma_frac": round(pf / (pm * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                       "gdn_hbm_frac": round(gdn_bytes(w.B, w.T, w.gdn_H) / (gm * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        del inp, g, p, o_g, ws_g, S_g, o_p
        torch.cuda.empty_cache()
    if want("decode"):
        # 256K decode, batch 1 and 16; two state / query buffers alternate so caches cannot serve them
        L = workloads.DECODE_CONTEXT
        for B in (1, 16):
            d = workloads.make_decode_inputs(B, L, device="cuda")
            ws = torch.empty(atma.atma_polar_attn_decode_workspace_bytes(B, 16, L), dtype=torch.uint8, device="cuda")
            gd = d["gdn"]
            states = [gd["state"].clone(), gd["state"].clone()]
            qs = [d["q"], d["q"].clone()]
            od = torch.empty_like(d["q"])
            og = torch.empty(B, 8, 128, dtype=torch.bfloat16, device="cuda")
            tpd, tgd = Timer(torch), Timer(torch)
            for it in range(23):
                i = it & 1
                fp = lambda: atma.atma_polar_attn_decode(qs[i], d["k_cache"], d["v_cache"], L, d["params"], o=od,
                                                         workspace=ws)
                fg = lambda: atma.atma_gdn_decode_step(gd["q"], gd["k"], gd["v"], gd["alpha"], gd["beta"], states[i],
                                                       o=og)
                if it < 3:
                    fp(), fg()
                else:
                    tpd(fp)
                    tgd(fg)
            torch.cuda.synchronize()
            pm, gm = tpd.mean_ms(), tgd.mean_ms()
            # the same step with the memory step on a second stream (default priority), overlapping
            # the Polar decode: the step's time is then the longer of the two
            side, main_s = torch.cuda.Stream(), torch.cuda.current_stream()
            t2 = Timer(torch)
            for it in range(23):
                i = it & 1

                def step2():
                    side.wait_stream(main_s)
                    atma.atma_gdn_decode_step(gd["q"], gd["k"], gd["v"], gd["alpha"], gd["beta"], states[i], o=og,
                                              stream=side)
                    atma.atma_polar_attn_decode(qs[i], d["k_cache"], d["v_cache"], L, d["params"], o=od, workspace=ws)
                    main_s.wait_stream(side)

                (t2 if it >= 3 else (lambda f: f()))(step2)
            torch.cuda.synchronize()
            sm = t2.mean_ms()
            byts = decode_bytes(B, L)
            res[f"decode_262k_b{B}"] = {"tokens_per_s": round(B / ((pm + gm) * 1e-3), 1), "polar_us": round(pm * 1e3, 1),
                                        "gdn_us": round(gm * 1e3, 1),
                                        "hbm_frac": round(byts / ((pm + gm) * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                                        "two_streams": {"step_us": round(sm * 1e3, 1),
                                                        "tokens_per_s": round(B / (sm * 1e-3), 1),
                                                        "hbm_frac": round(byts / (sm * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}}
            del d, ws, states, qs, od, og
            torch.cuda.empty_cache()
    return res


def cpu_model():
    """The host CPU's model name (first "model name" line of /proc/cpuinfo), or the platform's."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or platform.machine()


def cpu_baseline(w):
    """The fp64 oracle, as it stands, on this host's cores: full memory recurrence and full causal
    Polar attention for the workload's sequences (same shapes, same seed recipe)."""
    import numpy as np

    import oracle
    import workloads

    nseq = w.B  # the whole batch: no extrapolation
    inp = workloads.make_workload(w, device="cpu")
    g, p = inp["gdn"], inp["polar"]
    sl = slice(0, nseq)
    gq, gk, gv, ga, gb = (g[x][sl] for x in ("q", "k", "v", "alpha", "beta"))
    pq, pk, pv = (p[x][sl] for x in ("q", "k", "v"))
    cores = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    oracle.gdn_sequential(gq, gk, gv, ga, gb, threads=cores)
    oracle.polar_fwd(pq, pk, pv, p["params"], threads=cores)
    dt = time.perf_counter() - t0
    used = max(oracle.threads_used(cores, nseq * w.gdn_H), oracle.threads_used(cores, nseq * w.T * w.polar_Hq))
    del np
    return {"value": round(nseq * w.T / dt, 2), "unit": "tokens/s", "cores": used, "kind": "oracle",
            "cpu_model": cpu_model(),
            "seconds": round(dt, 2),
            "sample": f"{nseq} of {w.B} sequences of {w.name} (T={w.T}): full fp64 memory recurrence "
                      f"({w.gdn_H} heads x d={w.gdn_D}) + full causal Polar attention ({w.polar_Hq} heads x d=64)"}


if __name__ == "__main__":
    main()
