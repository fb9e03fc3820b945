#!/usr/bin/env python3
"""Benchmark of the fused LM-head + exact-sampling decode step on one MI355X.

Workload (the FlashSampling page's main micro-benchmark shape, "reproduction"):
a Qwen3-8B-shaped LM head, H [B, 4096] bf16 ~ N(0, 1), W [151936, 4096] bf16 ~
N(0, 0.02), per-row temperature ~ U[0.5, 1.2], seeded per row, exact
sampling with float32 noise (no filtering); B = 64 is the headline, B = 1, 8, 32 are reported
beside it.  Inputs are synthetic and already resident in HBM when timing starts.

One step = one fs_sample_fused call: a single kernel launch, Stage 1 with
Stage 2 in the last workgroup of each batch tile, offset advancing each step.
Before anything is timed the headline step runs for a fixed wall time
(--prewarm-ms, reported), so the first timed pass does not meet a cold GPU.
Prints one JSON line: `value` is microseconds per decode step at B = 64, the
mean over one timed pass of K steps; the p10/p50/p90 of that same pass's
per-step times and the kernel's average duration come from HIP events the
library records around each launch on the stream it runs on, inside that
pass.  `roofline` prices the kernel's algorithmic HBM bytes against that
duration; `stream_ceiling` is a plain streaming read of the same number of
bytes (what an HBM-bound kernel can practically reach); `standalone_sampler`
does the same for fs_sample_logits, `filtered_sampler` for
fs_sample_logits_filtered (top-k, top-p, min-p) beside the eager transformers
chain, `large_batch` the B = 256 head with bias and `wide_head` the D = 8192,
V = 262144 head with float64 noise, each beside the unfused GEMM + sampler,
`verify` fs_verify (speculative-decoding rejection sampling, K = 4) beside an
eager PyTorch rejection sampler; `cpu_baseline` is the float64 CPU oracle
computing the same steps on this host's cores.
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

METRIC = ("µs/decode-step & achieved HBM GB/s (fused LM-head+sample), "
          "D=4096 V=151936 B=1–64")
D_MODEL, VOCAB = 4096, 151936
LOGITS_CHUNK = 2048             # smallest chunk of the standalone sampler (bounds its candidate count)
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, published
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "fused_stage1_qwen3_8b_b64_traffic.txt")
KERNEL_SOURCES = ["decode_exact_categorical_amd/csrc/fs_fused.hip",
                  "decode_exact_categorical_amd/csrc/fs_device.hpp",
                  "decode_exact_categorical_amd/csrc/fs_launch.hpp"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per Stage 1 launch from the committed rocprofv3 counter summary,
    if it was taken on the current kernel source (else None)."""
    if not os.path.exists(PROFILE_TRAFFIC):
        return None
    vals = {}
    with open(PROFILE_TRAFFIC) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def kernel_alg_bytes(B: int, D: int, V: int, n_tiles: int, bias: bool = False, cand: int = 8,
                     fp8: bool = False) -> int:
    """What one fused sampling launch must move (Stage 1 and Stage 2 in one kernel):
    W once (bf16, or FP8 codes plus one float32 scale per row), H once,
    temperatures, [bias], candidates written and read back once, the sampled
    indices written."""
    w_bytes = V * D + 4 * V if fp8 else V * D * 2
    return (w_bytes + B * D * 2 + 4 * B + (4 * B * V if bias else 0)
            + 2 * cand * B * n_tiles + 8 * B)


def mxfp4_alg_bytes(B: int, D: int, V: int, n_tiles: int, cand: int = 8) -> int:
    """kernel_alg_bytes for MXFP4 weights: D/2 bytes of codes and D/32 of scales a row."""
    return V * D // 2 + V * D // 32 + B * D * 2 + 4 * B + 2 * cand * B * n_tiles + 8 * B


def mxfp4_from_bf16(torch, W, chunk_rows: int = 16384):
    """MXFP4 copy of a bf16 [V, D] weight on its device: per block of 32, scale
    2^X with X = floor(log2 max|w|) - 2, elements rounded to the nearest E2M1
    value (ties to the even code, saturating at 6); element 2j in the low
    nibble of byte j.  Returns (W4 uint8 [V, D/2], S uint8 [V, D/32])."""
    V, D = W.shape
    dev = W.device
    mids = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], device=dev)
    W4 = torch.empty((V, D // 2), dtype=torch.uint8, device=dev)
    S = torch.empty((V, D // 32), dtype=torch.uint8, device=dev)
    for r0 in range(0, V, chunk_rows):
        r1 = min(V, r0 + chunk_rows)
        blk = W[r0:r1].float().view(r1 - r0, D // 32, 32)
        amax = blk.abs().amax(dim=2)
        X = torch.where(amax > 0, torch.floor(torch.log2(amax.clamp_min(1e-38))) - 2,
                        torch.full_like(amax, -127.0)).clamp(-127, 127)
        x = blk * torch.exp2(-X)[..., None]
        mag = x.abs()
        code = torch.bucketize(mag, mids, right=True)
        prev = mids[(code - 1).clamp_min(0)]
        tie = (code > 0) & (mag == prev)
        code = torch.where(tie & (code % 2 == 1), code - 1, code)
        code = code | ((x < 0) & (code > 0)).long() << 3
        code = code.view(r1 - r0, D).to(torch.uint8)
        W4[r0:r1] = code[:, 0::2] | (code[:, 1::2] << 4)
        S[r0:r1] = (X + 127).to(torch.uint8)
    return W4, S


def logits_alg_bytes(B: int, V: int, cand: int = 8) -> int:
    """What one standalone sampling launch must move: the float32 logits once,
    temperatures, candidates written and read back once, the indices written."""
    n_tiles = (V + LOGITS_CHUNK - 1) // LOGITS_CHUNK
    return 4 * B * V + 4 * B + 2 * cand * B * n_tiles + 8 * B


def verify_alg_bytes(B: int, K: int, V: int, residual_rows: int) -> int:
    """What one verification call must move: every float32 target and draft row
    once (the softmax normalisers and the bonus draw), the two rows of the
    rejected position again for each row whose residual draw runs (its scores
    need both normalisers), the draft tokens, temperatures and outputs; the
    small per-chunk partials are left out."""
    return 4 * B * (2 * K + 1) * V + 8 * V * residual_rows + 8 * B * K + 4 * B + 8 * B * (K + 2)


def cpu_time_subset(oracle, H_rows, W_h, temp_rows, bias_rows, B_full: int, *, seed: int,
                    fp64: bool, what: str):
    """The float64 oracle on a few rows of a step (host tensors), timed and scaled
    by B_full / rows to the whole step: rows are independent, so the full step
    costs that many times as much (reported as extrapolated)."""
    n = H_rows.shape[0]
    t0 = time.perf_counter()
    oracle.sample_fused(H_rows, W_h, temp_rows, bias_rows, seed=seed, offset=1,
                        fp64_noise=fp64)
    dt = time.perf_counter() - t0
    return {"us_per_step": round(dt * 1e6 * B_full / n, 1), "rows": n, "rows_in_step": B_full,
            "measured_s": round(dt, 3), "measured": f"extrapolated from {n} rows ({what})"}


def percentiles(xs, qs=(10, 50, 90)):
    ys = sorted(xs)
    out = {}
    for q in qs:
        k = min(len(ys) - 1, max(0, int(round(q / 100 * (len(ys) - 1)))))
        out[f"p{q}"] = ys[k]
    return out


def time_calls(torch, fs, call, steps, warmup):
    """Time `steps` calls of call(s) after `warmup` untimed ones, in one pass.
    Returns (mean ms per step, mean kernel ms, per-step ms percentiles).  Two
    torch events on the current stream (the stream the library launches on)
    bracket the pass for the mean; the HIP events the library records around
    each launch in the same pass give each kernel's duration and, from one
    launch's start to the next, the per-step times."""
    for s in range(warmup):
        call(s)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with fs.KernelTimer(per_call=True) as kt:
        e0.record()
        for s in range(steps):
            call(warmup + s)
        e1.record()
        torch.cuda.synchronize()
    mean_step = e0.elapsed_time(e1) / steps
    per_step = kt.start_to_start_ms or [mean_step]
    return mean_step, kt.kernel_ms / max(1, kt.calls), percentiles(per_step)


def prewarm(torch, call, ms: float):
    """Run call(s) back to back for `ms` of wall time; returns (ms spent, calls)."""
    t0 = time.perf_counter()
    n = 0
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(8):
            call(n)
            n += 1
        torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3, n


def time_region(torch, fn, steps, warmup):
    for s in range(warmup):
        fn(s)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for s in range(steps):
        fn(warmup + s)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=25)
    ap.add_argument("--batch", type=int, default=64)
    ap.add_argument("--prewarm-ms", type=float, default=1500.0,
                    help="wall time of back-to-back headline steps run before any timing")
    ap.add_argument("--sweep", default="1,8,32", help="extra batch sizes reported beside B")
    ap.add_argument("--only-fused", action="store_true",
                    help="time the fused step only (no sweep, baselines or CPU oracle)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--standalone-sweep", action="store_true",
                    help="only time fs_sample_logits at the row counts and vocabulary sizes of "
                         "the Megatron fp64-noise page's cost table, float32 and float64 noise")
    ap.add_argument("--stream-ceiling", action="store_true",
                    help="only time the plain streaming read (fs_debug_stream_read) of the headline "
                         "step's algorithmic byte count, --steps times")
    ap.add_argument("--large-batch", action="store_true",
                    help="only time the large-batch head (B = 256, D = 4096, V = 128256, fp32 bias "
                         "with 10%% of each row masked), --steps times: the command profiled for "
                         "the wide kernel's MFMA counters")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a device-to-device copy of 1 GiB, --steps times (the known-size "
                         "reference for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this path has no multi-GPU mode "
              "(sharding the vocabulary across GPUs is not built).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0")
        src.fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": args.steps}), flush=True)
        return 0

    import decode_exact_categorical_amd as fs
    import synthetic

    if args.stream_ceiling:
        dev = torch.device("cuda:0")
        n = kernel_alg_bytes(args.batch, D_MODEL, VOCAB, fs.fused_tiles(args.batch, D_MODEL, VOCAB))
        buf = torch.empty(n // 16 * 16, dtype=torch.uint8, device=dev)
        buf.fill_(7)
        sink = torch.zeros(1, dtype=torch.int64, device=dev)
        ms, kms, pc = time_calls(torch, fs, lambda s: fs.debug_stream_read(buf, sink), args.steps,
                                 args.warmup)
        gbs = buf.numel() / (kms * 1e-3) / 1e9
        print(json.dumps({"stream_ceiling_bytes": buf.numel(), "avg_launch_us": round(kms * 1e3, 2),
                          "achieved_gbs": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
                          "steps": args.steps}), flush=True)
        return 0

    if args.large_batch:
        dev = torch.device("cuda:0")
        gl = torch.Generator(device=dev).manual_seed(7)
        VL, BL = 128256, 256
        WL = (torch.randn(VL, D_MODEL, generator=gl, device=dev) * 0.02).to(torch.bfloat16)
        HL = torch.randn(BL, D_MODEL, generator=gl, device=dev).to(torch.bfloat16)
        TL = 0.5 + 0.7 * torch.rand(BL, generator=gl, device=dev)
        biasL = torch.randn(BL, VL, generator=gl, device=dev)
        biasL.masked_fill_(torch.rand(BL, VL, generator=gl, device=dev) < 0.1, float("-inf"))
        ms, kms, pc = time_calls(
            torch, fs, lambda s: fs.sample_fused(HL, WL, TL, biasL, seed=77, offset=s),
            args.steps, args.warmup)
        flops = 2 * BL * VL * D_MODEL
        print(json.dumps({"large_batch_us": round(ms * 1e3, 2), "kernel_us": round(kms * 1e3, 2),
                          "tflops": round(flops / (kms * 1e-3) / 1e12, 1),
                          "mfma_frac": round(flops / (kms * 1e-3) / (MFMA_BF16_PEAK_TFLOPS * 1e12), 4),
                          "steps": args.steps}), flush=True)
        return 0

    if args.standalone_sweep:
        dev = torch.device("cuda:0")
        rows = {}
        for (vl, bl) in ((131072, 1), (131072, 8), (131072, 64), (131072, 256), (131072, 1024),
                         (262144, 64), (262144, 256)):
            g = torch.Generator(device=dev).manual_seed(5)
            X = torch.randn(bl, vl, generator=g, dtype=torch.float32, device=dev)
            Tl = torch.full((bl,), 0.8, dtype=torch.float32, device=dev)
            for f64 in (False, True):
                ms, kms, pc = time_calls(
                    torch, fs, lambda s: fs.sample_logits(X, Tl, seed=99, offset=s, fp64_noise=f64),
                    args.steps, args.warmup)
                rows[f"V{vl}_B{bl}_{'fp64' if f64 else 'fp32'}"] = {
                    "us_per_call": round(ms * 1e3, 2), "p50_us": round(pc["p50"] * 1e3, 2),
                    "kernel_us": round(kms * 1e3, 2)}
                log(f"  V={vl} B={bl} fp64={f64}: {rows[list(rows)[-1]]}")
            del X
        print(json.dumps({"standalone_sweep": rows, "unit": "us"}), flush=True)
        return 0

    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    cus = props.multi_processor_count
    B = args.batch
    sweep = [int(x) for x in args.sweep.split(",") if x] if not args.only_fused else []
    Bmax = max([B] + sweep)

    log(f"device {props.name} ({cus} CUs); generating W [{VOCAB}, {D_MODEL}] bf16 on the host")
    W_h = synthetic.weight(VOCAB, D_MODEL, std=0.02)
    H_h = synthetic.hidden(Bmax, D_MODEL)
    T_h = synthetic.temperatures(Bmax)
    W = W_h.to(dev)
    H = H_h.to(dev)
    temp = T_h.to(dev)
    torch.cuda.synchronize()

    nT = fs.fused_tiles(B, D_MODEL, VOCAB)
    Hb, Tb = H[:B].contiguous(), temp[:B].contiguous()
    step = lambda s: fs.sample_fused(Hb, W, Tb, seed=1234, offset=s)  # noqa: E731
    pw_ms, pw_calls = prewarm(torch, step, args.prewarm_ms)
    log(f"pre-warm: {pw_calls} fused steps in {pw_ms:.0f} ms")
    log(f"timing fused step B={B}: {args.warmup} warmup + {args.steps} timed steps")
    t0 = time.perf_counter()
    ms_step, k_ms, pct = time_calls(torch, fs, lambda s: step(10**7 + s), args.steps, args.warmup)
    wall = time.perf_counter() - t0
    us_step = ms_step * 1e3
    k_bytes = kernel_alg_bytes(B, D_MODEL, VOCAB, nT)
    k_gbs = k_bytes / (k_ms * 1e-3) / 1e9
    traffic = measured_traffic()
    result = {
        "metric": METRIC,
        "value": round(us_step, 2),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) H, N(0,0.02) W, U[0.5,1.2] temperatures)",
        "config": {
            "workload": "fused LM-head matmul + exact Gumbel-max sampling, one decode step",
            "global_batch": B, "D": D_MODEL, "V": VOCAB, "noise": "fp32 (23-bit Philox uniforms)",
            "temperature": "per row U[0.5,1.2]", "bias": None, "seed": 1234,
            "offset": "advances every step",
        },
        "prewarm_ms": round(pw_ms, 1),
        "prewarm_steps": pw_calls,
        "tokens_per_s": round(B / (ms_step * 1e-3), 1),
        "hbm_gbs_step": round(k_bytes / (ms_step * 1e-3) / 1e9, 1),
        "step_us_percentiles": {k: round(v * 1e3, 2) for k, v in pct.items()},
        "roofline": {
            "kernel": "fused_stage1_kernel (matmul + transform + noise + tile argmax; "
                      "Stage 2 in the last workgroup of each batch tile)",
            "bound": "hbm",
            "achieved": round(k_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(k_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "alg_bytes_per_launch": k_bytes,
            "avg_launch_us": round(k_ms * 1e3, 2),
            "vocab_tiles": nT,
        },
        "timed_wall_s": round(wall, 3),
    }
    # The same steps without the library's per-launch timing events (what a
    # caller that does not profile sees; those events widen the gap between
    # launches by a few microseconds), right after the timed pass.
    ef_ms = time_region(torch, lambda s: step(2 * 10**7 + s), args.steps, args.warmup)
    result["event_free_us_per_step"] = round(ef_ms * 1e3, 2)

    # The practical read ceiling: a plain streaming read of as many bytes as
    # the headline kernel's algorithmic bytes, timed the same way.
    buf = torch.empty(k_bytes // 16 * 16, dtype=torch.uint8, device=dev)
    buf.fill_(7)
    sink = torch.zeros(1, dtype=torch.int64, device=dev)
    _, r_ms, _ = time_calls(torch, fs, lambda s: fs.debug_stream_read(buf, sink), args.steps,
                            args.warmup)
    r_gbs = buf.numel() / (r_ms * 1e-3) / 1e9
    result["stream_ceiling"] = {
        "kernel": "stream_read_kernel (plain 16-byte-load read of the same byte count)",
        "bytes": buf.numel(), "avg_launch_us": round(r_ms * 1e3, 2),
        "achieved": round(r_gbs, 1), "unit": "GB/s", "frac_of_peak": round(r_gbs / HBM_PEAK_GBS, 4),
        "fused_frac_of_ceiling": round(k_gbs / r_gbs, 4),
    }
    log(f"  stream ceiling: {result['stream_ceiling']}")
    del buf

    want_cpu = not args.only_fused and not args.no_cpu_baseline
    cpu_extra = {}
    if want_cpu:
        import oracle
    if not args.only_fused:
        per = {}
        for b in sweep:
            Hs, Ts = H[:b].contiguous(), temp[:b].contiguous()
            ms, kms, pc = time_calls(
                torch, fs, lambda s: fs.sample_fused(Hs, W, Ts, seed=1234, offset=10**6 + s),
                max(20, args.steps // 2), args.warmup)
            kb = kernel_alg_bytes(b, D_MODEL, VOCAB, fs.fused_tiles(b, D_MODEL, VOCAB))
            per[str(b)] = {"us_per_step": round(ms * 1e3, 2),
                           "p50_us": round(pc["p50"] * 1e3, 2),
                           "kernel_us": round(kms * 1e3, 2),
                           "kernel_gbs": round(kb / (kms * 1e-3) / 1e9, 1),
                           "kernel_frac": round(kb / (kms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                           "tokens_per_s": round(b / (ms * 1e-3), 1)}
            log(f"  B={b}: {per[str(b)]}")
        result["batch_sweep"] = per

        # FP8 weights: the same head quantised per row to OCP E4M3 codes with one
        # float32 scale per row (the row's largest magnitude over 448), on the GPU.
        log("timing the FP8-weight fused step")
        amax = W.float().abs().amax(dim=1)
        W_scale = (amax / 448.0).clamp_min(1e-30).contiguous()
        W8 = torch.empty((VOCAB, D_MODEL), dtype=torch.uint8, device=dev)
        for r0 in range(0, VOCAB, 16384):
            r1 = min(VOCAB, r0 + 16384)
            W8[r0:r1] = (W[r0:r1].float() / W_scale[r0:r1, None]).to(torch.float8_e4m3fn).view(
                torch.uint8)
        f8 = {"workload": "W [151936, 4096] OCP E4M3 + float32 row scales, fp32 noise"}
        for b in sorted(set(sweep + [B])):
            Hs, Ts = H[:b].contiguous(), temp[:b].contiguous()
            ms, kms, pc = time_calls(
                torch, fs,
                lambda s: fs.sample_fused_w8(Hs, W8, W_scale, Ts, seed=1234, offset=2 * 10**6 + s),
                max(20, args.steps // 2), args.warmup)
            kb = kernel_alg_bytes(b, D_MODEL, VOCAB, fs.fused_tiles(b, D_MODEL, VOCAB, "fp8"),
                                  fp8=True)
            f8[str(b)] = {"us_per_step": round(ms * 1e3, 2),
                          "p50_us": round(pc["p50"] * 1e3, 2),
                          "kernel_us": round(kms * 1e3, 2),
                          "kernel_gbs": round(kb / (kms * 1e-3) / 1e9, 1),
                          "kernel_frac": round(kb / (kms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                          "tokens_per_s": round(b / (ms * 1e-3), 1)}
            log(f"  fp8 B={b}: {f8[str(b)]}")
        result["fp8_weights"] = f8
        del W8, amax

        # MXFP4 weights: the same head in E2M1 with an E8M0 scale per block of 32.
        log("timing the MXFP4-weight fused step")
        W4, S4 = mxfp4_from_bf16(torch, W)
        f4 = {"workload": "W [151936, 4096] MXFP4 (E2M1 + E8M0 per 32), fp32 noise"}
        for b in sorted(set(sweep + [B])):
            Hs, Ts = H[:b].contiguous(), temp[:b].contiguous()
            ms, kms, pc = time_calls(
                torch, fs,
                lambda s: fs.sample_fused_mxfp4(Hs, W4, S4, Ts, seed=1234, offset=4 * 10**6 + s),
                max(20, args.steps // 2), args.warmup)
            kb = mxfp4_alg_bytes(b, D_MODEL, VOCAB, fs.fused_tiles(b, D_MODEL, VOCAB, "mxfp4"))
            f4[str(b)] = {"us_per_step": round(ms * 1e3, 2), "p50_us": round(pc["p50"] * 1e3, 2),
                          "kernel_us": round(kms * 1e3, 2),
                          "kernel_gbs": round(kb / (kms * 1e-3) / 1e9, 1),
                          "kernel_frac": round(kb / (kms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                          "tokens_per_s": round(b / (ms * 1e-3), 1)}
            log(f"  mxfp4 B={b}: {f4[str(b)]}")
        result["mxfp4_weights"] = f4
        del W4, S4

        # Gumbel-top-k (k = 8 draws without replacement per row), fused into the
        # same head, float32 noise.
        log("timing the fused Gumbel-top-k step (k = 8)")
        tk = {"workload": "W [151936, 4096] bf16, k = 8 places per row, fp32 noise"}
        for b in sorted(set(sweep + [B])):
            Hs, Ts = H[:b].contiguous(), temp[:b].contiguous()
            ms, kms, pc = time_calls(
                torch, fs,
                lambda s: fs.sample_fused_topk(Hs, W, Ts, k=8, seed=1234, offset=3 * 10**6 + s),
                max(20, args.steps // 4), args.warmup)
            kb = kernel_alg_bytes(b, D_MODEL, VOCAB, fs.fused_tiles(b, D_MODEL, VOCAB), cand=64)
            tk[str(b)] = {"us_per_step": round(ms * 1e3, 2), "kernel_us": round(kms * 1e3, 2),
                          "kernel_gbs": round(kb / (kms * 1e-3) / 1e9, 1),
                          "kernel_frac": round(kb / (kms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
            log(f"  top-k B={b}: {tk[str(b)]}")
        result["fused_topk"] = tk

        # The standalone sampler over float32 logits: the tail-rate workload's
        # chunk shape (4096 rows x 131072) and a decode-sized batch.
        log("timing the standalone sampler")
        sa = {}
        for (bl, vl, f64) in ((64, 131072, False), (4096, 131072, False), (4096, 131072, True)):
            g = torch.Generator(device=dev).manual_seed(5)
            X = torch.randn(bl, vl, generator=g, dtype=torch.float32, device=dev)
            Tl = torch.full((bl,), 0.8, dtype=torch.float32, device=dev)
            ms, kms, pc = time_calls(
                torch, fs, lambda s: fs.sample_logits(X, Tl, seed=99, offset=s, fp64_noise=f64),
                max(20, args.steps // 4), 5)
            lb = logits_alg_bytes(bl, vl, 16 if f64 else 8)
            key = f"B{bl}_V{vl}_{'fp64' if f64 else 'fp32'}_noise"
            sa[key] = {"us_per_call": round(ms * 1e3, 2), "kernel_us": round(kms * 1e3, 2),
                       "alg_bytes": lb, "kernel_gbs": round(lb / (kms * 1e-3) / 1e9, 1),
                       "kernel_frac": round(lb / (kms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
            log(f"  {key}: {sa[key]}")
            del X
        result["standalone_sampler"] = sa

        # Filtered sampling over float32 logits (temperature -> top-k -> top-p ->
        # min-p -> draw): the settings of the spec-decode-ops card's example
        # (top_k = 50, top_p = 0.95) at its latency vocabulary (V = 128256, B = 1
        # and 8), at the Qwen3-8B vocabulary (B = 64, plus top-p and min-p alone)
        # and at the tail-rate chunk shape; against the eager transformers chain
        # (the card's comparison) on the same tensors.
        log("timing the filtered sampler")
        fl = {"settings": "top_k=50, top_p=0.95 unless named; logits N(0, 3^2), T = 0.8"}
        try:
            from transformers.generation.logits_process import (TemperatureLogitsWarper,
                                                                TopKLogitsWarper, TopPLogitsWarper)
        except Exception:           # the eager baseline needs transformers
            TopKLogitsWarper = None
        for (bl, vl, name, kw) in ((1, 128256, "", dict(top_k=50, top_p=0.95)),
                                   (8, 128256, "", dict(top_k=50, top_p=0.95)),
                                   (64, 151936, "", dict(top_k=50, top_p=0.95)),
                                   (64, 151936, "_top_p_0.95", dict(top_p=0.95)),
                                   (64, 151936, "_min_p_0.05", dict(min_p=0.05)),
                                   (4096, 131072, "", dict(top_k=50, top_p=0.95))):
            g = torch.Generator(device=dev).manual_seed(6)
            X = torch.randn(bl, vl, generator=g, dtype=torch.float32, device=dev) * 3.0
            Tl = torch.full((bl,), 0.8, dtype=torch.float32, device=dev)
            ms, kms, pc = time_calls(
                torch, fs, lambda s: fs.sample_logits_filtered(X, Tl, seed=98, offset=s, **kw),
                max(20, args.steps // 4), 5)
            lb = 4 * bl * vl + 12 * bl
            key = f"B{bl}_V{vl}{name}"
            fl[key] = {"us_per_call": round(ms * 1e3, 2), "kernel_us": round(kms * 1e3, 2),
                       "alg_bytes": lb, "kernel_gbs": round(lb / (kms * 1e-3) / 1e9, 1),
                       "kernel_frac": round(lb / (kms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
            if TopKLogitsWarper is not None and "top_k" in kw and bl <= 64:
                wt = TemperatureLogitsWarper(0.8)
                wk = TopKLogitsWarper(kw["top_k"])
                wp = TopPLogitsWarper(kw["top_p"])

                def eager(s):
                    z = wp(None, wk(None, wt(None, X)))
                    return torch.multinomial(torch.softmax(z, dim=-1), 1)

                fl[key]["eager_transformers_chain_us"] = round(
                    time_region(torch, eager, max(20, args.steps // 4), 5) * 1e3, 2)
                fl[key]["speedup_vs_eager"] = round(
                    fl[key]["eager_transformers_chain_us"] / fl[key]["us_per_call"], 2)
            if bl == 64 and not name:
                # the filter chain's output logits (filter_logits)
                Y = torch.empty_like(X)
                fms, fkms, _ = time_calls(
                    torch, fs, lambda s: fs.filter_logits(X, Tl, out=Y, **kw),
                    max(20, args.steps // 4), 5)
                fl[key]["filter_logits_kernel_us"] = round(fkms * 1e3, 2)
                # the card's whole pipeline: repetition penalty over 256 previous
                # tokens a row, then the filtered draw (two launches)
                prev = torch.randint(0, vl, (bl, 256), generator=g, device=dev)
                pen = torch.full((bl,), 1.3, dtype=torch.float32, device=dev)
                pms, pkms, _ = time_calls(
                    torch, fs, lambda s: fs.sample(X, Tl, repetition_penalty=pen, prev_tokens=prev,
                                                   seed=98, offset=s, **kw),
                    max(20, args.steps // 4), 5)
                fl[key]["pipeline_with_penalty_us"] = round(pms * 1e3, 2)
                # two library calls a pipeline, each timed by its own events
                fl[key]["pipeline_with_penalty_kernels_us"] = round(2 * pkms * 1e3, 2)
                del Y, prev, pen
            log(f"  {key}: {fl[key]}")
            del X
        result["filtered_sampler"] = fl

        # Filtered sampling fused into the LM head (fs_sample_fused_filtered) at
        # the card's settings (top_k 50 + top_p 0.95) on the Qwen3-8B head, and
        # top-p or min-p alone at B = 64 (flat rows send top-p-alone rows through
        # the exact fallback); against the GEMM + fs_sample_logits_filtered.
        log("timing fused filtered sampling")
        ff = {"workload": "W [151936, 4096] bf16, per-row T ~ U[0.5,1.2], fp32 noise"}
        for (bl, name, kw) in ((1, "", dict(top_k=50, top_p=0.95)),
                               (8, "", dict(top_k=50, top_p=0.95)),
                               (64, "", dict(top_k=50, top_p=0.95)),
                               (64, "_top_p_0.95", dict(top_p=0.95)),
                               (64, "_min_p_0.05", dict(min_p=0.05))):
            Hs, Ts = H[:bl].contiguous(), temp[:bl].contiguous()
            ms, kms, pc = time_calls(
                torch, fs, lambda s: fs.sample_fused_filtered(Hs, W, Ts, seed=1234, offset=s, **kw),
                max(20, args.steps // 4), 5)

            def unfused_filtered(s):
                y = torch.matmul(Hs, W.t()).float()
                return fs.sample_logits_filtered(y, Ts, seed=1234, offset=s, **kw)

            unf = time_region(torch, unfused_filtered, max(20, args.steps // 4), 5)
            nTf = fs.fused_tiles(bl, D_MODEL, VOCAB)
            kb = VOCAB * D_MODEL * 2 + bl * D_MODEL * 2 + 2 * 128 * bl * nTf + 16 * bl
            key = f"B{bl}{name}"
            ff[key] = {"us_per_call": round(ms * 1e3, 2), "kernel_us": round(kms * 1e3, 2),
                       "alg_bytes": kb, "kernel_frac": round(kb / (kms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                       "unfused_gemm_filtered_us": round(unf * 1e3, 2),
                       "speedup_vs_unfused": round(unf / ms, 3)}
            log(f"  {key}: {ff[key]}")
        result["fused_filtered"] = ff

        # Speculative-decoding verification over float32 target [B, K+1, V] and
        # draft [B, K, V] logits, K = 4 (the spec-decode-ops card's acceptance
        # length test), at the Qwen3-8B vocabulary: the draft is the target plus
        # N(0, 1) noise and proposes from its own softmax (T = 0.8).  Against an
        # eager PyTorch rejection sampler on the same tensors (softmaxes of every
        # row materialised, the residual of every position formed, multinomial).
        log("timing speculative verification")
        vf = {"settings": "K=4, target N(0, 3^2), draft = target + N(0, 1), T = 0.8"}
        KV = 4
        for bl in (1, 8, 64):
            g = torch.Generator(device=dev).manual_seed(8)
            TG = torch.randn(bl, KV + 1, VOCAB, generator=g, device=dev) * 3.0
            DR = (TG[:, :KV] + torch.randn(bl, KV, VOCAB, generator=g, device=dev)).contiguous()
            Tv = torch.full((bl,), 0.8, dtype=torch.float32, device=dev)
            TOK = torch.multinomial(torch.softmax(DR.reshape(-1, VOCAB) / 0.8, dim=-1), 1,
                                    generator=g).reshape(bl, KV).contiguous()
            ms, kms, pc = time_calls(
                torch, fs, lambda s: fs.verify(TG, DR, TOK, Tv, seed=97, offset=s),
                max(20, args.steps // 4), 5)
            acc, _ = fs.verify(TG, DR, TOK, Tv, seed=97, offset=0)
            n_res = int((acc < KV).sum().item())     # rows whose residual pass ran
            lb = verify_alg_bytes(bl, KV, VOCAB, n_res)
            key = f"B{bl}_K{KV}_V{VOCAB}"
            vf[key] = {"us_per_call": round(ms * 1e3, 2), "kernel_us": round(kms * 1e3, 2),
                       "residual_rows": n_res, "alg_bytes": lb,
                       "kernel_gbs": round(lb / (kms * 1e-3) / 1e9, 1),
                       "kernel_frac": round(lb / (kms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}

            def eager(s):
                pt = torch.softmax(TG / Tv[:, None, None], dim=-1)
                pd = torch.softmax(DR / Tv[:, None, None], dim=-1)
                a = pt[:, :KV].gather(2, TOK[..., None])[..., 0]
                q = pd.gather(2, TOK[..., None])[..., 0]
                ok = torch.rand(bl, KV, device=dev) * q < a
                L = ok.int().cumprod(dim=1).sum(dim=1)
                res = (pt[:, :KV] - pd).clamp_min(0)
                row = res[torch.arange(bl, device=dev), L.clamp(max=KV - 1)]
                r_tok = torch.multinomial(row / row.sum(-1, keepdim=True), 1)[:, 0]
                b_tok = torch.multinomial(pt[:, KV], 1)[:, 0]
                return L, torch.where(L == KV, b_tok, r_tok)

            vf[key]["eager_torch_us"] = round(
                time_region(torch, eager, max(20, args.steps // 4), 5) * 1e3, 2)
            vf[key]["speedup_vs_eager"] = round(vf[key]["eager_torch_us"] / vf[key]["us_per_call"], 2)
            log(f"  {key}: {vf[key]}")
            del TG, DR
        result["verify"] = vf

        # The large-batch end: the Llama-3-shaped head at the compute crossover
        # (H [256, 4096], W [128256, 4096], per-row temperature, fp32 bias with
        # 10% of each row masked), reported against both the MFMA and the HBM peak.
        log("timing the large-batch head (B=256, V=128256, bias + mask)")
        gl = torch.Generator(device=dev).manual_seed(7)
        VL, BL = 128256, 256
        WL = (torch.randn(VL, D_MODEL, generator=gl, device=dev) * 0.02).to(torch.bfloat16)
        HL = torch.randn(BL, D_MODEL, generator=gl, device=dev).to(torch.bfloat16)
        TL = 0.5 + 0.7 * torch.rand(BL, generator=gl, device=dev)
        biasL = torch.randn(BL, VL, generator=gl, device=dev)
        biasL.masked_fill_(torch.rand(BL, VL, generator=gl, device=dev) < 0.1, float("-inf"))
        ms, kms, pc = time_calls(
            torch, fs, lambda s: fs.sample_fused(HL, WL, TL, biasL, seed=77, offset=s),
            max(20, args.steps // 4), 5)
        flops = 2 * BL * VL * D_MODEL
        lb = kernel_alg_bytes(BL, D_MODEL, VL, fs.fused_tiles(BL, D_MODEL, VL), bias=True)

        def unfused_large(s):
            y = torch.matmul(HL, WL.t()).float() + biasL
            return fs.sample_logits(y, TL, seed=77, offset=s)

        unf = time_region(torch, unfused_large, max(20, args.steps // 4), 5)
        result["large_batch"] = {
            "workload": "B=256, D=4096, V=128256, fp32 bias with 10% -inf, fp32 noise",
            "us_per_call": round(ms * 1e3, 2), "kernel_us": round(kms * 1e3, 2),
            "tflops": round(flops / (kms * 1e-3) / 1e12, 1),
            "mfma_frac": round(flops / (kms * 1e-3) / (MFMA_BF16_PEAK_TFLOPS * 1e12), 4),
            "alg_bytes": lb, "hbm_gbs": round(lb / (kms * 1e-3) / 1e9, 1),
            "hbm_frac": round(lb / (kms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "unfused_gemm_bias_sampler_us": round(unf * 1e3, 2),
            "speedup_vs_unfused": round(unf / ms, 3),
        }
        log(f"  {result['large_batch']}")
        if want_cpu:
            # the oracle on 8 of the 256 rows, scaled to the whole step (rows are
            # independent), with the same W, H, temperatures and bias
            rows = torch.arange(0, BL, BL // 8, device=dev)
            cpu_extra["llama_b256_bias_mask"] = cpu_time_subset(
                oracle, HL[rows].cpu(), WL.cpu(), TL[rows].cpu().numpy(),
                biasL[rows].cpu().numpy(), BL, seed=77, fp64=False,
                what=f"B=256 D={D_MODEL} V={VL} bias + mask")
        del WL, HL, biasL

        # The wide head (D = 8192, V = 262144, 4 GiB of bf16 W) with float64 noise,
        # T = 0.7, B = 1, 16, 128; the unfused GEMM + fp64-noise sampler beside each.
        log("timing the wide head (D=8192, V=262144, fp64 noise)")
        gw = torch.Generator(device=dev).manual_seed(9)
        VW, DW = 262144, 8192
        WW = (torch.randn(VW, DW, generator=gw, device=dev) * 0.015).to(torch.bfloat16)
        wide = {"workload": "D=8192, V=262144 bf16 W, T = 0.7, fp64 noise"}
        for bw in (1, 16, 128):
            HW = torch.randn(bw, DW, generator=gw, device=dev).to(torch.bfloat16)
            TW = torch.full((bw,), 0.7, dtype=torch.float32, device=dev)
            ms, kms, pc = time_calls(
                torch, fs, lambda s: fs.sample_fused(HW, WW, TW, seed=5, offset=s, fp64_noise=True),
                max(20, args.steps // 8), 5)
            lb = kernel_alg_bytes(bw, DW, VW, fs.fused_tiles(bw, DW, VW), cand=16)
            flops = 2 * bw * VW * DW

            def unfused_wide(s):
                y = torch.matmul(HW, WW.t())
                return fs.sample_logits(y.float(), TW, seed=5, offset=s, fp64_noise=True)

            unf = time_region(torch, unfused_wide, max(20, args.steps // 8), 5)
            wide[f"B{bw}"] = {"us_per_call": round(ms * 1e3, 2), "kernel_us": round(kms * 1e3, 2),
                              "alg_bytes": lb,
                              "hbm_frac": round(lb / (kms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                              "mfma_frac": round(flops / (kms * 1e-3) /
                                                 (MFMA_BF16_PEAK_TFLOPS * 1e12), 4),
                              "unfused_us": round(unf * 1e3, 2),
                              "speedup_vs_unfused": round(unf / ms, 3)}
            log(f"  B={bw}: {wide[f'B{bw}']}")
            if want_cpu and bw > 1:
                if "WW_h" not in locals():
                    WW_h = WW.cpu()
                rows = torch.arange(0, bw, max(1, bw // 8), device=dev)[:8]
                cpu_extra[f"wide_head_b{bw}_fp64"] = cpu_time_subset(
                    oracle, HW[rows].cpu(), WW_h, TW[rows].cpu().numpy(), None, bw, seed=5,
                    fp64=True, what=f"B={bw} D={DW} V={VW} fp64 noise")
            del HW
        if want_cpu:
            del WW_h
        result["wide_head"] = wide
        del WW

        # Baselines on the same data: (1) unfused: rocBLAS/hipBLASLt GEMM writes bf16
        # logits to HBM, then the standalone sampler; (2) softmax + multinomial.
        log("timing unfused baselines")

        def unfused(s):
            y = torch.matmul(Hb, W.t())
            return fs.sample_logits(y.float(), Tb, seed=1234, offset=s)

        def conventional(s):
            y = torch.matmul(Hb, W.t()).float()
            p = torch.softmax(y / Tb[:, None], dim=-1)
            return torch.multinomial(p, 1)

        def gemm_only(s):
            return torch.matmul(Hb, W.t())

        n_base = max(20, args.steps // 2)
        base = {
            "gemm_plus_fs_sample_logits_us": round(time_region(torch, unfused, n_base, 10) * 1e3, 2),
            "gemm_softmax_multinomial_us": round(time_region(torch, conventional, n_base, 10) * 1e3, 2),
            "gemm_only_us": round(time_region(torch, gemm_only, n_base, 10) * 1e3, 2),
        }
        base["fused_speedup_vs_gemm_plus_sampler"] = round(base["gemm_plus_fs_sample_logits_us"] / us_step, 3)
        base["fused_speedup_vs_softmax_multinomial"] = round(base["gemm_softmax_multinomial_us"] / us_step, 3)
        result["baselines"] = base
        log(f"  {base}")

    if want_cpu:
        threads = oracle.num_threads()
        log(f"CPU oracle: full decode steps on {threads} threads")
        offset = 4242
        got = fs.sample_fused(H[:B].contiguous(), W, temp[:B].contiguous(), seed=1234, offset=offset)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ref, gap, _ = oracle.sample_fused(H_h[:B], W_h, T_h[:B].numpy(), seed=1234, offset=offset)
        cpu_s = time.perf_counter() - t0
        got = got.cpu().numpy()
        decided = gap > 1e-3
        t0 = time.perf_counter()
        oracle.sample_fused(H_h[:1], W_h, T_h[:1].numpy(), seed=1234, offset=offset)
        cpu_b1 = time.perf_counter() - t0
        # the tiny configuration: H [4, 512], W [32768, 512], T = 1
        Ht, Wt = synthetic.hidden(4, 512), synthetic.weight(32768, 512, std=0.02)
        t0 = time.perf_counter()
        oracle.sample_fused(Ht, Wt, np.ones(4, dtype=np.float32), seed=1234, offset=0)
        cpu_tiny = time.perf_counter() - t0
        configs = {
            "qwen_b64": {"us_per_step": round(cpu_s * 1e6, 1), "rows": B, "measured": "full step"},
            "qwen_b1": {"us_per_step": round(cpu_b1 * 1e6, 1), "rows": 1, "measured": "full step"},
            "tiny_b4_d512_v32768": {"us_per_step": round(cpu_tiny * 1e6, 1), "rows": 4,
                                    "measured": "full step"},
        }
        configs.update(cpu_extra)
        result["cpu_baseline"] = {
            "value": round(cpu_s * 1e6, 1),
            "unit": "us/step",
            "cores": threads,
            "kind": "oracle",
            "sample": f"one full decode step: B={B}, D={D_MODEL}, V={VOCAB}, all rows, float64 "
                      "(other configurations under `configs`; the B = 256 and wide heads on 8 "
                      "rows, scaled to the step and marked extrapolated)",
            "configs": configs,
        }
        result["step_parity_vs_oracle"] = {
            "decided_rows": int(decided.sum()),
            "decided_rows_equal": int((got[decided] == ref[decided]).sum()),
            "near_tie_rows": int((~decided).sum()),
        }

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
