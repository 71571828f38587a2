"""Benchmark of the Qwen3-TTS 12 Hz per-frame generation step on one MI355X.

A step is one whole request of the workload: the prompt prefill (talker
selection 0) followed by the frame loop (per frame: 2-token predictor prefill
+ 14 predictor steps, 15 selections, the embedding-sum feedback, one talker
step and the lookahead selection) until every row stops or reaches the frame
cap. `value` is 16-code frames per second over the timed steps, inputs already
resident in device memory.

Default workload: the 0.6B-shaped talker + predictor, bf16 weights (fp32
accumulate), bf16 KV cache, batch 1, greedy, 32-token prompt, 100 frames.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
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
FRAMES_PER_AUDIO_SECOND = 12.5

# HBM bytes per launch of the gate/up projection from two rocprofv3 --pmc runs
# (FETCH_SIZE x 1.999, WRITE_SIZE x 1.000, scaled by a 64 MiB copy), valid for
# the kernel source with this SHA-256 prefix only.
COUNTED_TRAFFIC = {"kernel_src_sha256_16": "f808ae5e24cfdc87", "bytes": 12742000}


def counted_traffic():
    import hashlib
    src = os.path.join(ROOT, "codec_lm_autoregressive_amd", "csrc", "qt_kernels.hip")
    h = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    return COUNTED_TRAFFIC["bytes"] if h == COUNTED_TRAFFIC["kernel_src_sha256_16"] else None


def frame_bytes(dm, B, mean_ctx, wbytes=2, kvbytes=2):
    """Algorithmic bytes one frame step must read for B rows.

    Each forward pass reads its layer weights once: the talker once, the
    predictor 15 times (2-token prefill + 14 steps), one predictor head per
    step and the talker codec head; the talker KV cache is read once per step
    (mean context mean_ctx positions per row). Gathers of single embedding
    rows are negligible and left out.
    """
    def layer_params(d):
        qkv = (d["n_heads"] + 2 * d["n_kv_heads"]) * d["head_dim"] * d["hidden"]
        o = d["hidden"] * d["n_heads"] * d["head_dim"]
        mlp = 3 * d["hidden"] * d["intermediate"]
        return qkv + o + mlp
    t, p = dm["talker"], dm["predictor"]
    talker = t["layers"] * layer_params(t) + dm["talker_vocab"] * t["hidden"]
    pred = 15 * (p["layers"] * layer_params(p)) + 15 * dm["codebook"] * p["hidden"]
    if dm["pred_in_proj"]:
        pred += 15 * p["hidden"] * t["hidden"]
    kv = B * mean_ctx * t["layers"] * 2 * t["n_kv_heads"] * t["head_dim"] * kvbytes
    return (talker + pred) * wbytes + kv


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="qwen06b_bf16_b1")
    ap.add_argument("--frames", type=int, default=None, help="override the frame cap of the workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-frames", type=int, default=None,
                    help="frames of the oracle's timed sample (default: the whole workload)")
    ap.add_argument("--kernel-reps", type=int, default=200)
    ap.add_argument("--kernel-only", action="store_true",
                    help="only the dominant-kernel timing loop and a 64 MiB copy (for counter runs)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(rows would shard across GPUs with no exchange; see DESIGN.md)", file=sys.stderr)
        sys.exit(2)
    import torch
    from codec_lm_autoregressive_amd import binding, synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    wl = synth.workload(args.workload)
    dm = synth.dims(wl["model"])
    frames = args.frames or wl["frames"]
    B = wl["B"]
    H = dm["talker"]["hidden"]
    t0 = time.time()
    w = synth.make_weights(dm, seed=0, dtype=wl["dtype"])
    lens = synth.prompt_lengths(B, *wl["prompt"], seed=2)
    prompt_np = synth.make_prompts(lens, H, seed=1)
    pad_np = synth.make_tts_pad(H, seed=3)
    print(f"[bench] inputs ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    if args.kernel_only:
        us, nbytes = kernel_timing(torch, binding, w, dm, wl, B, args.kernel_reps)
        # a plain copy of known size, to scale the byte counters
        a = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"kernel_avg_us": round(us, 3), "kernel_bytes": nbytes,
                          "achieved_GBs": round(nbytes / (us * 1e-6) / 1e9, 1), "copy_bytes": 64 << 20}))
        return
    eng = binding.Engine(dm, w, wl["dtype"], max_batch=B, max_positions=max(wl["max_positions"],
                                                                            int(lens.max()) + frames))
    stream = eng.stream
    with torch.cuda.stream(stream):
        prompt = torch.from_numpy(prompt_np).cuda()
        pad = torch.from_numpy(pad_np).cuda()
    torch.cuda.synchronize()

    def one_request():
        return eng.generate(prompt, lens, pad, wl["talker"], wl["predictor"], 0, frames)


    for _ in range(args.warmup):
        one_request()
    torch.cuda.synchronize()
    total_frames = 0
    row_frames = 0
    t0 = time.perf_counter()
    for _ in range(args.steps):
        codes, n, fin = one_request()
        total_frames += int(n.max())
        row_frames += int(n.sum())
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms_per_step = dt * 1000 / args.steps
    value = row_frames / dt

    # decode-only frame time with HIP events on the engine's stream
    eng.prefill(prompt, lens, pad, wl["talker"], wl["predictor"], 0, frames)
    eng.step_frame()  # first frame of a request runs eagerly when no graph exists yet
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    nf = 0
    ev0.record(stream)
    try:
        for _ in range(frames - 1):
            _, st = eng.step_frame()
            nf += 1
            if np.all(st != 0):
                break
    except binding.QtError:
        pass
    ev1.record(stream)
    torch.cuda.synchronize()
    frame_ms = ev0.elapsed_time(ev1) / max(nf, 1)

    mean_ctx = float(np.mean(lens)) + (frames - 1) / 2.0 + 1
    wbytes = 2 if wl["dtype"] == "bf16" else 4
    kern_us, kern_bytes = kernel_timing(torch, binding, w, dm, wl, B, args.kernel_reps)
    kern_gbs = kern_bytes / (kern_us * 1e-6) / 1e9
    I = dm["talker"]["intermediate"]
    fb = frame_bytes(dm, B, mean_ctx, wbytes, wbytes)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, dm, wl, lens, prompt_np, pad_np, args.cpu_frames or frames)

    out = {
        "metric": "16-code frames/sec (0.6B-shaped talker + code predictor)",
        "value": round(value, 3),
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 weights, fp32 accumulate" if wl["dtype"] == "bf16" else "f32",
        "data": "synthetic (seeded random weights and prompt embeddings)",
        "config": {"workload": args.workload, "batch": B, "prompt_lens": [int(x) for x in lens][:8],
                   "frames_cap": frames, "frames_per_step": total_frames // args.steps,
                   "talker_layers": dm["talker"]["layers"], "predictor_layers": dm["predictor"]["layers"],
                   "hidden": H, "sampling": "sampled" if wl["talker"]["do_sample"] else "greedy"},
        # per-row real-time factor: wall time / audio time (audio = frames / 12.5 Hz)
        "rtf": round(FRAMES_PER_AUDIO_SECOND * B / value, 6) if value else None,
        "decode_ms_per_frame": round(frame_ms, 4),
        "frame_roofline": {"bound": "hbm", "bytes_per_frame": int(fb),
                           "achieved": round(fb / (frame_ms * 1e-3) / 1e9, 1),
                           "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(fb / (frame_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "roofline": {"kernel": "linear_kernel (gate/up SwiGLU projection, N=%d K=%d M=%d)" % (2 * I, H, B),
                     "bound": "hbm", "achieved": round(kern_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(kern_gbs / HBM_PEAK_GBS, 4), "traffic": counted_traffic(),
                     "avg_launch_us": round(kern_us, 3), "bytes_per_launch": int(kern_bytes)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    eng.close()


def kernel_timing(torch, binding, w, dm, wl, B, reps):
    """Dominant kernel: the SwiGLU gate/up projection of one decoder layer,
    launched through the library's projection entry point with the frame's
    shape (N = 2 I rows of K = H, B activation rows), timed with HIP events on
    the stream it runs on. Returns (average launch microseconds, algorithmic
    bytes per launch: the weight rows once, the activations in and out)."""
    H, I = dm["talker"]["hidden"], dm["talker"]["intermediate"]
    wg = binding.to_device_weight(w["talker_layers"][0]["w_gate"], wl["dtype"])
    wu = binding.to_device_weight(w["talker_layers"][0]["w_up"], wl["dtype"])
    Wgu = torch.stack([wg, wu], dim=1).reshape(2 * I, H).contiguous()
    xk = torch.randn(B, H, device="cuda")
    gk = torch.ones(H, device="cuda")
    yk = torch.empty(B, I, device="cuda")
    cur = torch.cuda.current_stream()
    binding.debug_linear(Wgu, xk, gk, 1e-6, 2, yk, wdtype=wl["dtype"], reps=10)
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    k0.record(cur)
    binding.debug_linear(Wgu, xk, gk, 1e-6, 2, yk, wdtype=wl["dtype"], reps=reps)
    k1.record(cur)
    torch.cuda.synchronize()
    us = k0.elapsed_time(k1) * 1000 / reps
    wbytes = 2 if wl["dtype"] == "bf16" else 4
    return us, 2 * I * H * wbytes + B * H * 4 + H * 4 + B * I * 4


def cpu_baseline(w, dm, wl, lens, prompt_np, pad_np, n_frames):
    """The oracle, as it stands, on a bounded sample of the same workload."""
    import oracle
    from codec_lm_autoregressive_amd import synth
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count()
    rows = synth.split_rows(prompt_np, lens)[:1]
    t0 = time.perf_counter()
    r = oracle.generate(w, dm, rows, pad_np, wl["talker"], wl["predictor"], 0, n_frames, record=False)[0]
    dt = time.perf_counter() - t0
    return {"value": round(r["n_frames"] / dt, 4), "unit": "frames/s", "cores": int(cores), "kind": "oracle",
            "sample": f"row 0: prefill of {int(lens[0])} tokens + {r['n_frames']} frames "
                      f"(workload: {len(lens)} row(s), {wl['frames']} frames), numpy fp32, {dt:.1f}s"}


if __name__ == "__main__":
    main()
