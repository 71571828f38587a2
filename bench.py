"""Benchmark of the Qwen3-TTS 12 Hz per-frame generation step on one MI355X.

A step is one whole request of the workload: the prompt prefill (talker
selection 0) followed by the frame loop (per frame: 2-token predictor prefill
+ 14 predictor steps, 15 selections, the embedding-sum feedback, one talker
step and the lookahead selection) until every row stops or reaches the frame
cap. `value` is 16-code frames per second over the timed steps, inputs already
resident in device memory.

Default workload (`value`): the 0.6B-shaped talker + predictor, bf16 weights
(fp32 accumulate), fp16 KV cache, batch 1, greedy, 32-token prompt, 100
frames. The same line reports, under `batches`, one timed request each of the
batch-8 (sampling, prompts 32..256, 200 frames) and batch-64 (sampling,
prompts 128..512, 1024 frames) workloads and of the 1.7B-class shape at
batch 1 and 8 (greedy, 64-token prompts, 250 frames), and the oracle timed on
the host cores on bounded samples.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--batches A,B]

Measurement modes for profiler runs (rocprofv3 wraps the same command):
    --kernel-only      the dominant kernel's timing loop and a 64 MiB copy
    --frame-counters   a prompt prefill and --counter-frames eager frames of a
                       workload, then a 64 MiB copy (byte counters per frame)
    --gemm-kernels     the batched projections at the 0.6B shapes
    --decode-attention the talker's single-token decode attention at batch 1,
                       8 and 64 over 28 layer caches (K/V bytes per launch)
and a summariser of their rocprofv3 CSV output:
    --summarize DIR    per-kernel statistics of a --kernel-trace run, or the
                       counters of a --pmc run, per dispatch or per frame
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

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16 matrix-core peak, vendor figure
FRAMES_PER_AUDIO_SECOND = 12.5

# Counter results of the committed profiles, each valid while the SHA-256
# prefix of the source it depends on is unchanged (else reported as null):
#  * the gate/up projection launch (bench.py --kernel-only): HBM bytes per
#    launch from FETCH_SIZE / WRITE_SIZE scaled by a 64 MiB copy, and its
#    rocprofv3 kernel-trace average duration
#    (profiles/gemv_gate_up_qwen06b_b1_counters.md);
#  * HBM bytes per decode frame of the batch-1 and batch-64 workloads
#    (bench.py --frame-counters; profiles/frame_hbm_bytes_qwen06b.md).
COUNTED = {
    "kernel": {"src_sha256_16": "799ed64ea42fd00d", "bytes": 12726309, "trace_avg_us": 4.712},
    "frame": {"src_sha256_16": "e080c0989fba5a90", "bytes_per_frame": {
        # workload: (HBM bytes per frame, mean context of the counted frames, streamed model there)
        "qwen06b_bf16_b1": (3301200000, 35.5, 3196166144),
        "qwen06b_bf16_b64_sampling": (11098400000, 339.9, 5701422285),
    }},
}
CSRC = os.path.join(ROOT, "codec_lm_autoregressive_amd", "csrc")


def _sha16(text):
    import hashlib
    return hashlib.sha256(text.encode()).hexdigest()[:16]


def dominant_kernel_source():
    """Source text the dominant kernel's counters depend on: the weight-load
    helper and the register GEMV from its comment through its launch-shape
    choice; None when the markers are not found."""
    dev = open(os.path.join(CSRC, "qt_device.h")).read()
    lin = open(os.path.join(CSRC, "qt_linear.hip")).read()
    try:
        a = dev.index("__device__ __forceinline__ u32x4 ld_weight(")
        b = dev.index("}", a)
        c = lin.index("// Register-only projection for a few activation rows")
        d = lin.index("static hipError_t launch_linear_t(", c)
    except ValueError:
        return None
    return dev[a:b + 1] + lin[c:d]


def all_kernel_source():
    """Every kernel and launch source of the library (the frame counters depend on all of them)."""
    names = ("qt_device.h", "qt_internal.h", "qt_linear.hip", "qt_attn.hip", "qt_select.hip", "qt_api.hip")
    return "".join(open(os.path.join(CSRC, n)).read() for n in names)


def counted(kind):
    """The committed counter results of `kind` if their source is unchanged, else None."""
    c = COUNTED[kind]
    if not c["src_sha256_16"]:
        return None
    text = dominant_kernel_source() if kind == "kernel" else all_kernel_source()
    return c if text is not None and _sha16(text) == c["src_sha256_16"] else None


def frame_bytes(dm, B, mean_ctx, wbytes=2, kvbytes=2, unique=False):
    """Algorithmic bytes one frame step must read for B rows.

    Streamed model (default): each forward pass reads its layer weights once:
    the talker once, the predictor 15 times (2-token prefill + 14 steps), one
    predictor head per step and the talker codec head; the talker KV cache is
    read once per step (mean context mean_ctx positions per row). The 14
    single-token steps take their first layer's q/k/v (and the 1.7B-class
    input projection's output) from code-indexed fp32 tables, so they read
    one table row per batch row instead of those weights. Unique model: the
    predictor's layer weights are counted once per frame (the floor if a
    cache holds them across the 15 passes). Gathers of single embedding rows
    are negligible and left out.
    """
    def layer_params(d):
        qkv = (d["n_heads"] + 2 * d["n_kv_heads"]) * d["head_dim"] * d["hidden"]
        o = d["hidden"] * d["n_heads"] * d["head_dim"]
        mlp = 3 * d["hidden"] * d["intermediate"]
        return qkv + o + mlp
    t, p = dm["talker"], dm["predictor"]
    talker = t["layers"] * layer_params(t) + dm["talker_vocab"] * t["hidden"]
    qkv_dim = (p["n_heads"] + 2 * p["n_kv_heads"]) * p["head_dim"]
    passes = 1 if unique else 15
    pred = passes * (p["layers"] * layer_params(p)) + 15 * dm["codebook"] * p["hidden"]
    if not unique:
        pred -= 14 * qkv_dim * p["hidden"]          # steps 1..14: first-layer q/k/v from the tables
    if dm["pred_in_proj"]:
        pred += p["hidden"] * t["hidden"]             # the input projection runs in the 2-token pass only
    table_rows = 14 * B * (qkv_dim + (p["hidden"] if dm["pred_in_proj"] else 0)) * 4
    kv = B * mean_ctx * t["layers"] * 2 * t["n_kv_heads"] * t["head_dim"] * kvbytes
    return (talker + pred) * wbytes + kv + table_rows


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="qwen06b_bf16_b1")
    ap.add_argument("--frames", type=int, default=None, help="override the frame cap of the workload")
    ap.add_argument("--batches", default="qwen06b_bf16_b8_sampling,qwen06b_bf16_b64_sampling,qwen17b_bf16_b1,"
                                         "qwen17b_bf16_b8",
                    help="further workloads reported under 'batches' (one timed request each; '' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-next", action="store_true",
                    help="skip the codec decoder, token-id frontend and continuous-batching measurements")
    ap.add_argument("--cpu-frames", type=int, default=100,
                    help="frames of the oracle's timed sample (row 0 of the workload)")
    ap.add_argument("--kernel-reps", type=int, default=200)
    ap.add_argument("--kernel-only", action="store_true",
                    help="only the dominant-kernel timing loop and a 64 MiB copy (for counter runs)")
    ap.add_argument("--frame-counters", action="store_true",
                    help="only a prefill and --counter-frames eager frames of --workload, then a 64 MiB copy")
    ap.add_argument("--counter-frames", type=int, default=8)
    ap.add_argument("--codec-only", action="store_true",
                    help="only the codec decoder measurement (one JSON line; for kernel traces)")
    ap.add_argument("--gemm-kernels", action="store_true",
                    help="only the batched projections (4096 prefill rows, 64-row decode) at the "
                         "0.6B shapes, timed per launch (for counter runs)")
    ap.add_argument("--decode-attention", action="store_true",
                    help="only the talker's decode attention at batch 1, 8 and 64 (0.6B heads, fp16 cache), "
                         "cycling over 28 layer caches, timed per launch (for kernel traces)")
    ap.add_argument("--summarize", default=None, metavar="DIR",
                    help="summarise the rocprofv3 CSV output under DIR and exit")
    ap.add_argument("--groups", type=int, default=0,
                    help="with --summarize of a kernel trace: average each kernel's dispatches in consecutive "
                         "groups of this many")
    ap.add_argument("--per-frame", action="store_true",
                    help="with --summarize: sum counters per frame (dispatches from the first frame_start_kernel)")
    return ap.parse_args()


class Workload:
    """Seeded inputs of one workload, resident on the device, and its engine."""

    def __init__(self, torch, binding, synth, name, frames=None):
        self.name = name
        self.wl = wl = synth.workload(name)
        self.dm = dm = synth.dims(wl["model"])
        self.frames = frames or wl["frames"]
        self.B = wl["B"]
        H = dm["talker"]["hidden"]
        t0 = time.time()
        self.w = synth.make_weights(dm, seed=0, dtype=wl["dtype"])
        self.lens = synth.prompt_lengths(self.B, *wl["prompt"], seed=2)
        self.prompt_np = synth.make_prompts(self.lens, H, seed=1)
        self.pad_np = synth.make_tts_pad(H, seed=3)
        print(f"[bench] {name}: inputs ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
        self.eng = binding.Engine(dm, self.w, wl["dtype"], max_batch=self.B,
                                  max_positions=max(wl["max_positions"], int(self.lens.max()) + self.frames))
        self.kv = "f16" if wl["dtype"] == "bf16" else "f32"   # the engine's default cache type
        with torch.cuda.stream(self.eng.stream):
            self.prompt = torch.from_numpy(self.prompt_np).cuda()
            self.pad = torch.from_numpy(self.pad_np).cuda()
        torch.cuda.synchronize()

    def request(self, frames=None):
        wl = self.wl
        return self.eng.generate(self.prompt, self.lens, self.pad, wl["talker"], wl["predictor"], 0,
                                 frames or self.frames)

    def run(self, torch, binding, steps, warmup):
        """Whole requests (prefill + frame loop): row-frames per second; then
        the decode-only frame time with HIP events on the engine's stream."""
        for _ in range(warmup):
            self.request()
        torch.cuda.synchronize()
        total_frames = row_frames = 0
        t0 = time.perf_counter()
        for _ in range(steps):
            codes, n, fin = self.request()
            total_frames += int(n.max())
            row_frames += int(n.sum())
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        wl, eng, stream = self.wl, self.eng, self.eng.stream
        torch.cuda.synchronize()
        tp = time.perf_counter()
        eng.prefill(self.prompt, self.lens, self.pad, wl["talker"], wl["predictor"], 0, self.frames)
        prefill_ms = (time.perf_counter() - tp) * 1000   # qt_prefill ends with its stream synchronised
        eng.step_frame()  # the first frame after a prefill runs eagerly; later ones replay the graph
        ttfa_ms = (time.perf_counter() - tp) * 1000      # prompt in HBM -> first 16-code frame on the host
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        nf = 0
        ev0.record(stream)
        try:
            for _ in range(self.frames - 1):
                _, st = eng.step_frame()
                nf += 1
                if np.all(st != 0):
                    break
        except binding.QtError:
            pass
        ev1.record(stream)
        torch.cuda.synchronize()
        frame_ms = ev0.elapsed_time(ev1) / max(nf, 1)
        mean_ctx = float(np.mean(self.lens)) + (self.frames - 1) / 2.0 + 1
        wbytes = 2 if wl["dtype"] == "bf16" else 4
        kvb = 2 if self.kv != "f32" else 4
        fb = frame_bytes(self.dm, self.B, mean_ctx, wbytes, kvb)
        fbu = frame_bytes(self.dm, self.B, mean_ctx, wbytes, kvb, unique=True)
        value = row_frames / dt
        return dict(value=value, dt=dt, steps=steps, total_frames=total_frames, frame_ms=frame_ms, fb=fb, fbu=fbu,
                    ms_per_step=dt * 1000 / steps, prefill_ms=prefill_ms, ttfa_ms=ttfa_ms,
                    prefill_flops=prefill_linear_flops(self.dm, int(np.sum(self.lens))))

    def config(self, total_frames, steps):
        wl, dm = self.wl, self.dm
        return {"workload": self.name, "batch": self.B, "prompt_lens": [int(x) for x in self.lens][:8],
                "frames_cap": self.frames, "frames_per_step": total_frames // max(steps, 1),
                "talker_layers": dm["talker"]["layers"], "predictor_layers": dm["predictor"]["layers"],
                "hidden": dm["talker"]["hidden"], "predictor_hidden": dm["predictor"]["hidden"],
                "kv_cache": self.kv, "sampling": "sampled" if wl["talker"]["do_sample"] else "greedy"}


def prefill_linear_flops(dm, tokens):
    """Useful flops of the prompt prefill's projections: 2 per weight per
    prompt token over the talker's layers (the hi/lo split of the activations
    doubles the matrix-core work; that is not counted)."""
    t = dm["talker"]
    H, d, I = t["hidden"], t["head_dim"], t["intermediate"]
    per_layer = H * (t["n_heads"] + 2 * t["n_kv_heads"]) * d + t["n_heads"] * d * H + 3 * I * H
    return 2.0 * tokens * per_layer * t["layers"]


def prefill_roof(q):
    tf = q["prefill_flops"] / (q["prefill_ms"] * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": round(tf, 1), "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
            "frac": round(tf / MFMA_BF16_PEAK_TFS, 4), "flops": q["prefill_flops"], "ms": round(q["prefill_ms"], 3)}


def roof(q, workload):
    """Frame roofline under both byte models, and the HBM bytes per frame the
    counters measured for this workload (null when not counted or stale)."""
    fb, fbu, frame_ms = q["fb"], q["fbu"], q["frame_ms"]
    gbs = fb / (frame_ms * 1e-3) / 1e9
    gbu = fbu / (frame_ms * 1e-3) / 1e9
    c = counted("frame")
    hbm = c["bytes_per_frame"].get(workload) if c else None
    out = {"bound": "hbm", "bytes_per_frame": int(fb), "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
           "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
           "unique_bytes_per_frame": int(fbu), "unique_achieved": round(gbu, 1),
           "unique_frac": round(gbu / HBM_PEAK_GBS, 4), "counted": None}
    if hbm:
        # counted on the first frames after the prefill (their own mean context)
        out["counted"] = {"hbm_bytes_per_frame": hbm[0], "mean_context": hbm[1],
                          "streamed_model_at_context": hbm[2], "ratio": round(hbm[0] / hbm[2], 3)}
    return out


def main():
    args = parse()
    if args.summarize:
        summarize(args.summarize, args.per_frame, args.groups)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(rows would shard across GPUs with no exchange; see DESIGN.md)", file=sys.stderr)
        sys.exit(2)
    import torch
    from codec_lm_autoregressive_amd import binding, synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.gemm_kernels:
        for line in gemm_kernel_timing(torch, binding, synth):
            print(json.dumps(line), flush=True)
        return
    if args.codec_only:
        print(json.dumps(codec_timing(torch, binding, synth)), flush=True)
        return
    if args.decode_attention:
        for line in decode_attention_timing(torch, binding, synth):
            print(json.dumps(line), flush=True)
        return
    if args.kernel_only:
        wl = synth.workload(args.workload)
        dm = synth.dims(wl["model"])
        w = synth.make_weights(dm, seed=0, dtype=wl["dtype"])
        us, nbytes = kernel_timing(torch, binding, w, dm, wl, wl["B"], args.kernel_reps)
        copy_64mib(torch)
        print(json.dumps({"kernel_avg_us": round(us, 3), "kernel_bytes": nbytes,
                          "achieved_GBs": round(nbytes / (us * 1e-6) / 1e9, 1), "copy_bytes": 64 << 20}))
        return
    if args.frame_counters:
        frame_counter_run(torch, binding, synth, args.workload, args.counter_frames)
        return

    main_wl = Workload(torch, binding, synth, args.workload, args.frames)
    r = main_wl.run(torch, binding, args.steps, args.warmup)
    B, wl, dm, w = main_wl.B, main_wl.wl, main_wl.dm, main_wl.w
    kern_us, kern_bytes = kernel_timing(torch, binding, w, dm, wl, B, args.kernel_reps)
    kern_gbs = kern_bytes / (kern_us * 1e-6) / 1e9
    H, I = dm["talker"]["hidden"], dm["talker"]["intermediate"]
    main_cfg = main_wl.config(r["total_frames"], args.steps)
    main_wl.eng.close()
    main_lens, main_prompt, main_pad = main_wl.lens, main_wl.prompt_np, main_wl.pad_np
    del main_wl
    torch.cuda.empty_cache()

    # the decoder, frontend and serving measurements run before the larger
    # batch workloads, on a device heap that has seen only the main workload
    extra = {}
    if not args.no_next:
        extra["codec"] = codec_timing(torch, binding, synth)
        torch.cuda.empty_cache()
        extra["frontend"] = frontend_timing(torch, binding, synth)
        torch.cuda.empty_cache()
        extra["serving"] = serving_timing(torch, binding, synth)
        torch.cuda.empty_cache()

    batches = []
    for name in [x for x in args.batches.split(",") if x]:
        x = Workload(torch, binding, synth, name)
        # warm-up: a short request captures the frame graph
        x.request(min(x.frames, 4))
        q = x.run(torch, binding, 1, 0)
        batches.append({"workload": name, "batch": x.B, "value": round(q["value"], 3), "unit": "frames/s",
                        "ms_per_request": round(q["ms_per_step"], 3),
                        "decode_ms_per_frame": round(q["frame_ms"], 4),
                        "decode_frames_per_s": round(x.B * 1000.0 / q["frame_ms"], 1),
                        "rtf": round(FRAMES_PER_AUDIO_SECOND * x.B / q["value"], 6) if q["value"] else None,
                        "frame_roofline": roof(q, name),
                        "prefill_tokens": int(np.sum(x.lens)),
                        "ttfa_ms": round(q["ttfa_ms"], 3),
                        "prefill_roofline": prefill_roof(q),
                        "config": x.config(q["total_frames"], 1)})
        x.eng.close()
        del x
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(synth, w, dm, wl, main_lens, main_prompt, main_pad,
                           min(args.cpu_frames, args.frames or wl["frames"]))

    kc = counted("kernel")
    out = {
        "metric": "16-code frames/sec (0.6B-shaped talker + code predictor)",
        "value": round(r["value"], 3),
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 weights, fp32 accumulate" if wl["dtype"] == "bf16" else "f32",
        "data": "synthetic (seeded random weights and prompt embeddings)",
        "config": main_cfg,
        # per-row real-time factor: wall time / audio time (audio = frames / 12.5 Hz)
        "rtf": round(FRAMES_PER_AUDIO_SECOND * B / r["value"], 6) if r["value"] else None,
        "decode_ms_per_frame": round(r["frame_ms"], 4),
        # time to first audio frame: qt_prefill (talker over the prompt, selection 0) + the first frame
        "ttfa_ms": round(r["ttfa_ms"], 3),
        "frame_roofline": roof(r, args.workload),
        "roofline": {"kernel": "gemv_kernel (gate/up SwiGLU projection, N=%d K=%d M=%d)" % (2 * I, H, B),
                     "bound": "hbm", "achieved": round(kern_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(kern_gbs / HBM_PEAK_GBS, 4),
                     "traffic": kc["bytes"] if kc else None,
                     "avg_launch_us": round(kern_us, 3), "bytes_per_launch": int(kern_bytes),
                     # the same launch loop under rocprofv3 --kernel-trace (committed profile)
                     "trace_avg_us": kc["trace_avg_us"] if kc else None,
                     "trace_frac": round(kern_bytes / (kc["trace_avg_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
                     if kc else None},
        "batches": batches,
        **extra,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def copy_64mib(torch):
    """A plain 64 MiB device copy: the calibration kernel of known size for the byte counters."""
    a = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()


def frame_counter_run(torch, binding, synth, name, frames):
    """A prompt prefill and `frames` eager frames of a workload (the frame's
    kernels; teacher-forced codes, which do not change what is read), then a
    64 MiB copy for the counter calibration. The frames are launched one by
    one through qt_debug_step_forced, so a counter run sees every dispatch."""
    x = Workload(torch, binding, synth, name)
    wl = x.wl
    x.eng.prefill(x.prompt, x.lens, x.pad, wl["talker"], wl["predictor"], 0, x.frames)
    B = x.B
    for k in range(frames):
        forced = np.zeros((B, 16), dtype=np.int32)
        forced[:, 0] = (97 * k + 13 * np.arange(B)) % 2048
        forced[:, 1:] = (np.arange(1, 16)[None, :] * 131 + 7 * k + np.arange(B)[:, None]) % 2048
        x.eng.step_forced(forced)
    torch.cuda.synchronize()
    copy_64mib(torch)
    print(json.dumps({"workload": name, "batch": B, "frames": frames, "prompt_lens": [int(v) for v in x.lens][:8],
                      "copy_bytes": 64 << 20}), flush=True)
    x.eng.close()


def _csv_rows(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def summarize(d, per_frame, groups=0):
    """Print a summary of the rocprofv3 CSV output under d: kernel statistics
    (kernel_stats.csv of a --kernel-trace --stats run) and/or counters per
    kernel (counter_collection.csv of a --pmc run), with the 64 MiB copy as
    the calibration of each counter (scale = copy bytes / copy counter value).
    With per_frame, counters are also summed over the dispatches from the
    first frame_start_kernel on (runtime copy kernels excluded) and divided
    by the number of frame_start_kernel dispatches. With groups = N, the
    dispatches of each kernel in a kernel trace (kernel_trace.csv) are also
    split, in start order, into consecutive groups of N, with each group's
    average duration (one group per case of a --decode-attention run)."""
    import glob
    stats = sorted(glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True))
    if groups > 0:
        for path in sorted(glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)):
            by = {}
            for r in sorted(_csv_rows(path), key=lambda r: int(r["Start_Timestamp"])):
                by.setdefault(r["Kernel_Name"], []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
            print(f"kernel trace ({os.path.relpath(path, d)}): groups of {groups} dispatches, average us")
            for n, ds in by.items():
                if len(ds) < groups:
                    continue
                avg = [sum(ds[i:i + groups]) / groups / 1e3 for i in range(0, len(ds) - groups + 1, groups)]
                print(f"`{n[:90]}`: " + ", ".join(f"{a:.2f}" for a in avg))
    ctrs = sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True))
    for path in stats:
        rows = _csv_rows(path)
        total = sum(float(r["TotalDurationNs"]) for r in rows)
        print(f"kernel statistics ({os.path.relpath(path, d)}): total {total / 1e6:.2f} ms")
        print("| kernel | calls | total ms | avg us | min us | max us | % |")
        print("|---|---|---|---|---|---|---|")
        for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
            print(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['TotalDurationNs']) / 1e6:.2f} | "
                  f"{float(r['AverageNs']) / 1e3:.3f} | {float(r['MinNs']) / 1e3:.3f} | {float(r['MaxNs']) / 1e3:.3f} | "
                  f"{float(r['Percentage']):.2f} |")
    for path in ctrs:
        rows = _csv_rows(path)
        by = {}
        order = []
        for r in rows:
            key = (r.get("Dispatch_Id") or r.get("Correlation_Id"), r["Counter_Name"])
            if key not in by:
                order.append(key)
                by[key] = [r["Kernel_Name"], 0.0]
            by[key][1] += float(r["Counter_Value"])
        names = sorted({k[1] for k in order})
        for cn in names:
            disp = [(int(k[0]), by[k][0], by[k][1]) for k in order if k[1] == cn]
            disp.sort()
            copies = [v for _, n, v in disp if n.startswith("__amd_rocclr_copyBuffer")]
            cal = copies[-1] if copies else None
            scale = (64 << 10) / cal if cal else None   # KiB of the 64 MiB copy / counted KiB
            print(f"counter {cn} ({os.path.relpath(path, d)}): {len(disp)} dispatches; "
                  f"calibration copy {cal} -> scale {scale and round(scale, 4)}")
            agg = {}
            for _, n, v in disp:
                a = agg.setdefault(n, [0, 0.0])
                a[0] += 1
                a[1] += v
            print(f"| kernel | dispatches | {cn} KiB / dispatch | scaled MB / dispatch |")
            print("|---|---|---|---|")
            for n, (c, v) in sorted(agg.items(), key=lambda kv: -kv[1][1])[:25]:
                sc = f"{v / c * scale * 1024 / 1e6:.4f}" if scale else "-"
                print(f"| `{n[:90]}` | {c} | {v / c:.1f} | {sc} |")
            if per_frame:
                first = next((i for i, (_, n, _) in enumerate(disp) if "frame_start_kernel" in n), None)
                if first is None:
                    print("no frame_start_kernel dispatch found")
                    continue
                frames = sum(1 for _, n, _ in disp[first:] if "frame_start_kernel" in n)
                tot = sum(v for _, n, v in disp[first:] if not n.startswith("__amd_rocclr"))
                print(f"per frame: {frames} frames, {tot / frames:.1f} KiB counted"
                      + (f" = {tot / frames * scale * 1024 / 1e9:.4f} GB scaled" if scale else ""))


def codec_flops_per_frame(cd):
    """Multiply-adds x 2 of the codec decoder's linear maps and convolutions
    for one frame of codes (attention and elementwise work left out)."""
    D, Hd, dim = cd["hidden"], cd["heads"] * cd["head_dim"], cd["codebook_dim"]
    f = 2 * D * dim                                                    # the two SplitRVQ projections
    f += cd["layers"] * (3 * Hd * D + D * Hd + 2 * D * cd["ffn"])     # transformer
    f += 2 * D * D + 2 * (2 * D * cd["up_ffn"])                       # upsampling stage 1 (2 rows per frame)
    f += 4 * D * D // 2 * 2 + 4 * (2 * D * cd["up_ffn"])              # stage 2 (4 rows per frame)
    ch, rows = cd["voc_channels"], 4
    f += rows * 7 * ch[0] * D                                          # vocoder input convolution
    for b, s in enumerate(cd["strides"]):
        f += rows * s * 2 * ch[b] * ch[b + 1]                          # transposed convolution, 2 taps per output
        rows *= s
        f += len(cd["dilations"]) * rows * (7 * ch[b + 1] ** 2 + ch[b + 1] ** 2)
    f += rows * 7 * ch[-1]
    return 2.0 * f


def codec_timing(torch, binding, synth, frames=300):
    """The codec decoder at its full shape on one 300-frame chunk (24 s of
    audio) with qt_codec_decode_chunked, and the first streamed piece (4
    frames) as the decode part of the time to first audio."""
    cd = synth.codec_dims("12hz")
    w = synth.make_codec_weights(cd, seed=3, dtype="bf16")
    cod = binding.Codec(cd, w, "bf16")
    codes = synth.make_codes(frames, seed=5)
    cod.decode_chunked(codes)
    cod.stream_step(codes[:4], 0)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    reps = 3
    for _ in range(reps):
        cod.decode_chunked(codes)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1000 / reps
    t1 = time.perf_counter()
    cod.stream_step(codes[:4], 0)
    first_ms = (time.perf_counter() - t1) * 1000
    cod.close()
    fl = codec_flops_per_frame(cd) * frames
    tf = fl / (ms * 1e-3) / 1e12
    return {"workload": "codec 12 Hz decoder, 300-frame chunk, bf16 weights", "frames": frames,
            "ms": round(ms, 3), "frames_per_s": round(frames * 1000 / ms, 1),
            "audio_s_per_s": round(frames / FRAMES_PER_AUDIO_SECOND * 1000 / ms, 1),
            "first_piece_ms": round(first_ms, 3),
            "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                         "frac": round(tf / MFMA_BF16_PEAK_TFS, 4), "flops": fl}}


def frontend_timing(torch, binding, synth):
    """qt_embed_ids at the full frontend shape (151936 x 2048 text embedding,
    ResizeMLP 2048 -> 2048 -> 1024) over the batch-64 workload's prompt
    positions (synthetic dual-track ids)."""
    wl = synth.workload("qwen06b_bf16_b64_sampling")
    dm = synth.dims(wl["model"])
    fd = synth.frontend_dims("qwen06b")
    fw = synth.make_frontend_weights(fd, dm["talker"]["hidden"], seed=5, dtype="bf16")
    lens = synth.prompt_lengths(wl["B"], *wl["prompt"], seed=2)
    n = int(np.sum(lens))
    ti, ci = synth.make_prompt_ids(lens, fd["text_vocab"], seed=3)
    small = dict(dm, talker=dict(dm["talker"], layers=1), predictor=dict(dm["predictor"], layers=1))
    eng = binding.Engine(small, synth.make_weights(small, seed=0, dtype="bf16"), "bf16", max_batch=1,
                         max_positions=16)
    eng.attach_frontend(fw, max_rows=n)
    eng.embed_ids(ti, ci)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    reps = 3
    for _ in range(reps):
        eng.embed_ids(ti, ci)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1000 / reps
    eng.close()
    fl = 2.0 * n * (fd["text_hidden"] * fd["mlp_hidden"] + fd["mlp_hidden"] * dm["talker"]["hidden"])
    tf = fl / (ms * 1e-3) / 1e12
    return {"workload": "token-id frontend over the batch-64 prompts", "rows": n, "ms": round(ms, 3),
            "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                         "frac": round(tf / MFMA_BF16_PEAK_TFS, 4), "flops": fl}}


def serving_timing(torch, binding, synth, slots=8, n_req=32):
    """Continuous batching at the 0.6B shape: a queue of requests (prompts
    32..256, sampling, frame caps 40..200) through 8 slots, a finished slot
    refilled by qt_admit before the next frame; against the same requests
    served as static batches of 8 (each batch runs until its longest row
    ends, finished rows fed EOS). Row-frames per second of each."""
    wl = synth.workload("qwen06b_bf16_b8_sampling")
    dm = synth.dims(wl["model"])
    H = dm["talker"]["hidden"]
    w = synth.make_weights(dm, seed=0, dtype="bf16")
    g = np.random.default_rng(13)
    lens = g.integers(32, 257, n_req).astype(np.int32)
    caps = g.integers(40, 201, n_req).astype(np.int32)
    caps[:slots] = caps[0]          # qt_prefill takes one frame cap for the first batch
    prompts = [torch.from_numpy(synth.make_prompts([int(P)], H, seed=100 + i)).cuda() for i, P in enumerate(lens)]
    pad = torch.from_numpy(synth.make_tts_pad(H, seed=3)).cuda()
    eng = binding.Engine(dm, w, "bf16", max_batch=slots, max_positions=512)
    tsamp, psamp = wl["talker"], wl["predictor"]
    # static batches: every row of a batch gets the batch's largest cap (one prefill per batch)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    static_rows = 0
    for b0 in range(0, n_req, slots):
        idx = list(range(b0, min(n_req, b0 + slots)))
        P = torch.cat([prompts[i] for i in idx])
        _, n, _ = eng.generate(P, lens[idx], pad, tsamp, psamp, 0, int(caps[idx].max()))
        static_rows += int(sum(min(int(n[j]), int(caps[i])) for j, i in enumerate(idx)))
    torch.cuda.synchronize()
    static_s = time.perf_counter() - t0
    # continuous batching
    t0 = time.perf_counter()
    first = list(range(slots))
    eng.prefill(torch.cat([prompts[i] for i in first]), lens[first], pad, tsamp, psamp, 0, int(caps[0]))
    holder = list(first)
    got = [0] * n_req
    nxt = slots
    while any(h is not None for h in holder):
        _, st = eng.step_frame()
        for s in range(slots):
            q = holder[s]
            if q is None or st[s] == 3:
                continue
            got[q] += 1
            if st[s] in (1, 2):
                holder[s] = None
                if nxt < n_req:
                    eng.admit(s, prompts[nxt], None, 0, nxt, int(caps[nxt]))
                    holder[s] = nxt
                    nxt += 1
    torch.cuda.synchronize()
    cont_s = time.perf_counter() - t0
    eng.close()
    cont_rows = int(sum(got))
    return {"workload": f"{n_req} requests of the batch-8 shape through {slots} slots (prompts 32..256, caps 40..200)",
            "continuous_row_frames_per_s": round(cont_rows / cont_s, 1), "continuous_s": round(cont_s, 3),
            "static_row_frames_per_s": round(static_rows / static_s, 1), "static_s": round(static_s, 3),
            "row_frames": cont_rows}


def kernel_timing(torch, binding, w, dm, wl, B, reps, copies=40):
    """Dominant kernel: the SwiGLU gate/up projection of one decoder layer,
    launched through the library's projection entry point with the frame's
    shape (N = 2 I rows of K = H, B activation rows), timed with HIP events on
    the stream it runs on. The launches rotate over `copies` distinct weight
    buffers (40 x 12.6 MB at the 0.6B shape, more than the 256 MB Infinity
    Cache) so every launch streams its weights from HBM, as in the frame.
    Returns (average launch microseconds, algorithmic bytes per launch: the
    weight rows once, the activations in and out)."""
    H, I = dm["talker"]["hidden"], dm["talker"]["intermediate"]
    wg = binding.to_device_weight(w["talker_layers"][0]["w_gate"], wl["dtype"])
    wu = binding.to_device_weight(w["talker_layers"][0]["w_up"], wl["dtype"])
    Wgu = torch.stack([wg, wu], dim=1).reshape(2 * I, H).contiguous()
    Ws = Wgu.unsqueeze(0).repeat(copies, 1, 1).contiguous()   # [copies, 2I, H]
    xk = torch.randn(B, H, device="cuda")
    gk = torch.ones(H, device="cuda")
    yk = torch.empty(B, I, device="cuda")
    cur = torch.cuda.current_stream()
    binding.debug_linear(Ws, xk, gk, 1e-6, 2, yk, wdtype=wl["dtype"], reps=copies)
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    k0.record(cur)
    binding.debug_linear(Ws, xk, gk, 1e-6, 2, yk, wdtype=wl["dtype"], reps=reps)
    k1.record(cur)
    torch.cuda.synchronize()
    us = k0.elapsed_time(k1) * 1000 / reps
    wbytes = 2 if wl["dtype"] == "bf16" else 4
    del Ws
    return us, 2 * I * H * wbytes + B * H * 4 + H * 4 + B * I * 4


def gemm_kernel_timing(torch, binding, synth, reps=10):
    """The batched projections of one 0.6B decoder layer through the
    library's projection entry point: 4096 prefill rows (split
    activations + matrix-core GEMM) and 64 decode rows (one-range row GEMM +
    reduce), bf16 weights from a seeded N(0, 0.02) draw. Useful flops count
    2 per weight per row; the hi/lo split doubles the matrix-core work."""
    g = np.random.default_rng(7)
    shapes = [("qkv", 4096, 1024, 0, True), ("o", 1024, 2048, 1, False),
              ("gate/up", 6144, 1024, 2, True), ("down", 1024, 3072, 1, False)]
    out = []
    for M in (4096, 64):
        for name, N, K, epi, norm in shapes:
            W = binding.to_device_weight(synth.bf16_round((g.standard_normal((N, K)) * 0.02).astype(np.float32)), "bf16")
            X = torch.randn(M, K, device="cuda")
            gain = torch.ones(K, device="cuda") if norm else None
            Y = torch.zeros(M, N // 2 if epi == 2 else N, device="cuda")
            binding.debug_linear(W, X, gain, 1e-6, epi, Y, reps=2)
            cur = torch.cuda.current_stream()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(cur)
            binding.debug_linear(W, X, gain, 1e-6, epi, Y, reps=reps)
            e1.record(cur)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1000 / reps
            flops = 2.0 * M * N * K
            out.append({"rows": M, "proj": name, "N": N, "K": K, "us_per_launch": round(us, 2),
                        "useful_TFLOPs": round(flops / (us * 1e-6) / 1e12, 1),
                        "matrix_core_TFLOPs": round(2 * flops / (us * 1e-6) / 1e12, 1),
                        "weight_GBs": round(N * K * 2 / (us * 1e-6) / 1e9, 1)})
    return out


def decode_attention_timing(torch, binding, synth, layers=28, reps=56):
    """The talker's single-token decode attention (16 q / 8 kv heads,
    head_dim 128, fp16 cache) through the library's decode-attention entry
    point, cycling over `layers` separate K/V caches as the layers of a frame
    do (so the 256 MB last-level cache does not hold the keys between
    launches): batch 1 at 41, 131 and 501 keys; batch 8 (8 key ranges, as the
    frame loop runs it) and batch 64 (one range) at the workloads' prompt
    lengths plus 0, 100 / 512 and 199 / 960 decoded frames. Reports the K/V
    bytes each launch reads; the kernel durations come from a trace. The
    entry point synchronises after each launch."""
    nq, nkv, d, max_pos = 16, 8, 128, 1536
    cos_np, sin_np = _rope_tables(max_pos, d, 1.0e6)
    cos, sin = torch.from_numpy(cos_np).cuda(), torch.from_numpy(sin_np).cuda()
    gain = torch.ones(d, device="cuda")
    cases = [("b1", np.array([40]), 1), ("b1", np.array([130]), 1), ("b1", np.array([500]), 1)]
    for name, B, S, extra in (("b8", 8, 8, (0, 100, 199)), ("b64", 64, 1, (0, 512, 960))):
        wl = synth.workload("qwen06b_bf16_b8_sampling" if B == 8 else "qwen06b_bf16_b64_sampling")
        lens = np.asarray(synth.prompt_lengths(B, *wl["prompt"], seed=2), dtype=np.int64)
        for f in extra:
            cases.append((name, lens + f, S))
    out = []
    for name, pos, S in cases:
        B = len(pos)
        g = torch.Generator(device="cuda").manual_seed(11)
        kc = [torch.randn((B, nkv, max_pos, d), generator=g, device="cuda").half() for _ in range(layers)]
        vc = [torch.randn((B, nkv, max_pos, d), generator=g, device="cuda").half() for _ in range(layers)]
        qkv = torch.randn((B, (nq + 2 * nkv) * d), generator=g, device="cuda")
        for i in range(reps):
            binding.debug_decode_attention(qkv, pos, gain, gain, cos, sin, kc[i % layers], vc[i % layers], nq, nkv,
                                           1e-6, "f16", S)
        keys = int(pos.sum()) + B
        out.append({"case": name, "rows": B, "kv_split": S, "mean_keys": round(keys / B, 1),
                    "kv_bytes_per_launch": keys * nkv * d * 2 * 2, "launches": reps})
        del kc, vc
        torch.cuda.empty_cache()
    return out


def _rope_tables(max_pos, d, theta):
    """cos / sin tables [max_pos, d / 2] of the rope angles (float32)."""
    inv = (theta ** (-np.arange(0, d, 2, dtype=np.float64) / d)).astype(np.float32)
    ang = np.arange(max_pos, dtype=np.float32)[:, None] * inv[None, :]
    return np.cos(ang.astype(np.float64)).astype(np.float32), np.sin(ang.astype(np.float64)).astype(np.float32)


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _time_oracle(oracle, w, dm, wl, prompt_rows, pad, n_frames, row=0):
    t0 = time.perf_counter()
    r = oracle.generate(w, dm, prompt_rows, pad, wl["talker"], wl["predictor"], 0, n_frames, rows=[row],
                        record=False)[0]
    return r["n_frames"], time.perf_counter() - t0


def cpu_baseline(synth, w, dm, wl, lens, prompt_np, pad_np, n_frames):
    """The oracle, as it stands, on bounded samples of the workloads: row 0 of
    the batch-1 workload (prefill + n_frames frames) with the BLAS threads the
    host gives it, the same row on 1 thread (prefill + 10 frames), and row 0 of
    the batch-8 and batch-64 workloads (their prefill + 16 / 32 frames)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threadpool_limits = None
        cores = os.cpu_count()
    rows = synth.split_rows(prompt_np, lens)[:1]
    nf, dt = _time_oracle(oracle, w, dm, wl, rows, pad_np, n_frames)
    out = {"value": round(nf / dt, 4), "unit": "frames/s", "cores": int(cores), "kind": "oracle",
           "cpu_model": _cpu_model(),
           "sample": f"row 0: prefill of {int(lens[0])} tokens + {nf} frames "
                     f"(workload: {len(lens)} row(s), {wl['frames']} frames), numpy fp32, {dt:.1f}s"}
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            nf1, dt1 = _time_oracle(oracle, w, dm, wl, rows, pad_np, 10)
        out["one_thread"] = {"value": round(nf1 / dt1, 4), "unit": "frames/s", "cores": 1,
                             "sample": f"row 0: prefill of {int(lens[0])} tokens + {nf1} frames, {dt1:.1f}s"}
    more = []
    for name, frames in (("qwen06b_bf16_b8_sampling", 16), ("qwen06b_bf16_b64_sampling", 32)):
        wl2 = synth.workload(name)
        l2 = synth.prompt_lengths(wl2["B"], *wl2["prompt"], seed=2)
        H = dm["talker"]["hidden"]
        p2 = synth.split_rows(synth.make_prompts(l2[:1], H, seed=1), l2[:1])
        nf2, dt2 = _time_oracle(oracle, w, dm, wl2, p2, pad_np, frames)
        more.append({"workload": name, "value": round(nf2 / dt2, 4), "unit": "frames/s", "cores": int(cores),
                     "sample": f"row 0: prefill of {int(l2[0])} tokens + {nf2} frames "
                               f"(workload: {wl2['B']} rows, {wl2['frames']} frames), {dt2:.1f}s"})
    out["batches"] = more
    return out


if __name__ == "__main__":
    main()
