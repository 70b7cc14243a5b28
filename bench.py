"""Benchmark of the INT4 decode block step on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--M m]

(a prefill workload name, e.g. 8b_prefill_s2048, times the FP8 prefill of
the QKV projection instead: see prefill_bench)

One step = one decode_block_step (QKV + rho1 + RoPE, KV append through the
Hadamard rotation, split-KV GQA attention + combine + inverse rotation, O +
residual, gate/up + SwiGLU, down + residual) for one batch of decode rows.
Inputs are resident in HBM before timing.  Steps rotate over C independent
copies of the layer (same bytes at different addresses, each with its own
KV cache) so that the 256 MB Infinity Cache cannot serve the weights from
one step to the next; the K timed steps are one captured HIP graph replayed
between two events on the launch stream.

Printed: one JSON line with the time per step, the achieved HBM bandwidth
(algorithmic bytes / time), the roofline entry of the dominant kernel (the
one-launch step kernel itself when M = 1 runs as one launch; otherwise the
gate/up projection, timed live with HIP events over back-to-back launches
of that kernel) and the CPU oracle timed on a bounded sample.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
FP8_PEAK_TFLOPS = 5000.0  # dense fp8 MFMA, MI355X

# HBM traffic of the dominant kernel per launch, from two rocprofv3 --pmc
# runs (FETCH_SIZE, then WRITE_SIZE) scaled by the same counters on a plain
# copy of known size; valid only for the sources it was taken on (sha256
# over the files that build and launch that kernel), else the roofline entry
# reports null.
STEP_M1_SOURCES = ("step.hip", "step.h", "gemv.h", "attn_core.h", "attn.h", "coherent.h", "device_common.h",
                   "proj.h", "i4d_internal.h", "i4d_layout.h", "api_device.hip", "api_host.cpp")
PREFILL_SOURCES = ("prefill.hip", "gemv.h", "attn.h", "coherent.h", "device_common.h", "proj.h", "i4d_internal.h",
                   "i4d_layout.h", "../build.py")
TRAFFIC = {
    "8b_m1_ctx4096": {"kernel": "step_m1_kernel (one-launch decode step)", "sources": STEP_M1_SOURCES,
                      "sha256": "3d63810bae1de70c5c98abcd3cc30dedfffd382c7aa137a3a52809458fc4f664",
                      "fetch_bytes": 118785280, "write_bytes": 779264},
    "8b_prefill_s2048": {"kernel": "prefill_gemm_kernel (FP8 MFMA GEMM + epilogue)", "sources": PREFILL_SOURCES,
                         "sha256": "a2c449ad7e57c9686148c4b487afd42cff405953cbeeff9541df647627809ae8",
                         "fetch_bytes": 213150848, "write_bytes": 10600448},
}


def sources_sha256(names):
    import hashlib
    d = os.path.join(ROOT, "int4_quantized_decode_amd", "csrc")
    h = hashlib.sha256()
    for name in names:
        h.update(name.encode())
        with open(os.path.join(d, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_of(workload, kernel):
    t = TRAFFIC.get(workload)
    if not t or t["kernel"] != kernel or t["sha256"] != sources_sha256(t["sources"]):
        return None
    return t["fetch_bytes"] + t["write_bytes"]


def device_errors(caches):
    """OR of the caches' device error words (I4D_DEVERR_* bits: an invalid
    length or position, or a wait of the one-launch step that timed out).
    A timed region whose steps set any of them measured no valid step."""
    e = 0
    for c in caches:
        e |= c.errors()
    return e


def require_clean(caches, what):
    e = device_errors(caches)
    if e:
        print(f"bench.py: {what}: device error word 0x{e:x} is set (I4D_DEVERR_*); the timed steps are not "
              f"valid and no result is printed", file=sys.stderr)
        sys.exit(3)
    return e


def algorithmic_bytes(shape, lengths, fmt="int4"):
    """Weight codes (INT4: 0.5 B/weight, E4M3: 1 B/weight) + fp16 group
    scales + INT4 KV codes and per-token-per-head fp16 scales read by one
    step."""
    d, F, hd, nq, nkv = shape.d_model, shape.d_ffn, shape.head_dim, shape.n_q_heads, shape.n_kv_heads
    weights = (shape.n_qkv * d + d * nq * hd + 2 * F * d + d * F)
    w_bytes = (weights if fmt == "e4m3" else weights // 2) + (weights // 128) * 2
    kv_bytes = int(np.sum(lengths)) * nkv * 2 * (hd // 2 + 2)
    return w_bytes + kv_bytes, w_bytes, kv_bytes


def gate_up_bytes(shape):
    n = 2 * shape.d_ffn * shape.d_model
    return n // 2 + (n // 128) * 2


TIMELINE_SLOTS = ["entry", "QKV strips stored", "attention units done", "attention outputs seen by O",
                  "O strips stored", "barrier after O passed", "gate/up strips stored",
                  "barrier after gate/up passed", "down strips stored"]


def timeline(args, shape, M, layers, caches, x_in, x_out, ctx, maxL, splits, ws, step, torch, B):
    """Per-stage timestamps of the one-launch step: each workgroup's readings
    of the 100 MHz real-time counter, relative to the first workgroup's
    entry in the same step; medians (and 90th percentiles) over steps and
    workgroups.  Eager launches, so the gaps between steps are not those of
    the timed graph."""
    if args.weights != "int4" or not B.i4d_decode_step_is_one_launch(B.make_shape(shape), M):
        print("bench.py --timeline: the workload does not run as the one-launch step", file=sys.stderr)
        sys.exit(2)
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    per = ncu * B.I4D_STEP_STAMPS
    n = max(args.steps, 1)
    stamps = torch.zeros((n, per), dtype=torch.int64, device="cuda")
    for i in range(args.warmup):
        step(i)
    C = len(layers)
    for i in range(n):
        B.i4d_decode_block_step_timeline(layers[i % C].struct, caches[i % C].struct, x_in, x_out, ctx, M, maxL,
                                         splits, ws.buf, ws.nbytes, stamps[i], per)
    torch.cuda.synchronize()
    require_clean(caches, "timeline steps")
    t_all = stamps.cpu().numpy().reshape(n, ncu, B.I4D_STEP_STAMPS).astype(np.int64)
    t = t_all[:, :, :len(TIMELINE_SLOTS)]
    rel = (t - t[:, :, :1].min(axis=1, keepdims=True)) * 0.01  # 100 MHz ticks -> us
    med = np.median(rel.reshape(-1, len(TIMELINE_SLOTS)), axis=0)
    p90 = np.percentile(rel.reshape(-1, len(TIMELINE_SLOTS)), 90, axis=0)
    if args.timeline_out:
        np.save(args.timeline_out, (t_all - t[:, :, :1].min(axis=1, keepdims=True)) * 0.01)
    span = np.median(rel[:, :, -1].max(axis=1))
    print("%-32s %10s %10s" % ("workgroup event", "median us", "p90 us"))
    for name, a, b in zip(TIMELINE_SLOTS, med, p90):
        print("%-32s %10.2f %10.2f" % (name, a, b))
    print("%-32s %10.2f" % ("last workgroup done (median)", span))
    print(json.dumps({"timeline": {k: round(float(v), 3) for k, v in zip(TIMELINE_SLOTS, med)},
                      "timeline_p90": {k: round(float(v), 3) for k, v in zip(TIMELINE_SLOTS, p90)},
                      "last_done_us": round(float(span), 3), "steps": n, "workgroups": ncu,
                      "workload": args.workload}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="8b_m1_ctx4096")
    ap.add_argument("--M", type=int, default=0, help="override the batch (70B shape sweep)")
    ap.add_argument("--copies", type=int, default=8)
    ap.add_argument("--splits", type=int, default=-1)
    ap.add_argument("--weights", default="int4", choices=["int4", "e4m3"],
                    help="decode-weight format (e4m3: the FP8 decode-weight variant)")
    ap.add_argument("--stage", default="step", choices=["step", "attention"],
                    help="time the whole decode step, or the attention launch alone (i4d_attention on the "
                         "step's query, no append)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-steps", type=int, default=5)
    ap.add_argument("--timeline", action="store_true",
                    help="instead of timing: per-stage timestamps of the one-launch step (M = 1) over --steps "
                         "eager steps (i4d_decode_block_step_timeline), medians over steps and workgroups")
    ap.add_argument("--timeline-out", default="",
                    help="with --timeline: also save every stamp (us from the step's first entry, "
                         "[steps][workgroups][slots]; a slot never stamped reads negative) to this .npy file")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB (the reference "
                         "kernel that scales the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: the library runs on one GPU; --gpus must be 1 (tensor- and sequence-parallel "
              "sharding of the step is not implemented)", file=sys.stderr)
        sys.exit(2)

    import torch

    from int4_quantized_decode_amd import binding as B
    from int4_quantized_decode_amd import device as D
    from int4_quantized_decode_amd import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_mib:
        n = args.copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": 3}), flush=True)
        return
    B.lib()
    if args.workload in synth.PREFILL_WORKLOADS:
        return prefill_bench(args, synth.PREFILL_WORKLOADS[args.workload], torch, B, D, synth)
    wl = synth.WORKLOADS[args.workload]
    if wl.n_layers > 1:
        return full_model(args, wl, torch, B, D, synth)
    shape = wl.shape
    M = args.M or wl.M
    lengths = synth.make_lengths(wl, M)
    maxL = int(lengths.max())
    splits = wl.num_splits if args.splits < 0 else args.splits
    C = args.copies

    t0 = time.time()
    lw = synth.make_layer(shape, wl.seed)
    pre = synth.make_cache_prefill(shape, lengths, wl.seed)
    xb = synth.make_x(shape, M, wl.seed)
    base_layer = D.DeviceLayer(shape, lw, fmt=args.weights)
    base_cache = D.DeviceCache(shape, lengths)
    base_cache.prefill(pre)
    layers = [base_layer] + [base_layer.clone() for _ in range(C - 1)]
    caches = [base_cache]
    for _ in range(C - 1):
        c = D.DeviceCache(shape, lengths)
        for name in ("k_codes", "v_codes", "k_scales", "v_scales"):
            getattr(c, name).copy_(getattr(base_cache, name))
        caches.append(c)
    ws = D.Workspace(shape, M, maxL, splits)
    x_in = D.to_device_u16(xb)
    x_out = torch.empty_like(x_in)
    ctx = torch.from_numpy(lengths).cuda()
    setup_s = time.time() - t0

    stream = torch.cuda.current_stream()

    step_fn = B.i4d_decode_block_step_e4m3 if args.weights == "e4m3" else B.i4d_decode_block_step

    def step(i):
        step_fn(layers[i % C].struct, caches[i % C].struct, x_in, x_out, ctx, M, maxL, splits, ws.buf, ws.nbytes,
                None)

    # eager check that the step runs, then graphs
    step(0)
    torch.cuda.synchronize()
    if args.timeline:
        return timeline(args, shape, M, layers, caches, x_in, x_out, ctx, maxL, splits, ws, step, torch, B)
    if args.stage == "attention":
        # the attention launch alone on the query the step left in the
        # workspace (the caches already hold the step's token: no append)
        cs = B.make_shape(shape)
        q = ws.view("q", torch.float32, M * shape.n_q_heads * shape.head_dim)
        anb = B.i4d_attention_workspace_bytes(cs, M, maxL, max(splits, 0))
        aws = torch.zeros(anb, dtype=torch.uint8, device="cuda")
        a16 = torch.empty((M, shape.n_q_heads * shape.head_dim), dtype=torch.int16, device="cuda")

        def step(i):  # noqa: F811
            B.i4d_attention(caches[i % C].struct, cs, q, ctx, M, maxL, max(splits, 0), aws, anb, None, a16)

    def capture(n, fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                fn(i)
        return g

    g_warm = capture(max(args.warmup, 1), step)
    g_main = capture(args.steps, step)
    g_warm.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    g_main.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_total = e0.elapsed_time(e1)
    require_clean(caches, "timed decode steps")
    ms_step = ms_total / args.steps
    us_step = ms_step * 1e3
    total_b, w_b, kv_b = algorithmic_bytes(shape, lengths, args.weights)
    if args.stage == "attention":
        total_b, w_b = kv_b, 0
    gbps = total_b / (us_step * 1e-6) / 1e9

    one_launch = args.weights == "int4" and B.i4d_decode_step_is_one_launch(B.make_shape(shape), M)
    if args.stage == "attention":
        rf_kernel, rf_bytes, rf_us = "attention launch (split partials and combine)", kv_b, us_step
    elif args.weights == "e4m3":
        # the E4M3 variant's entry is the step as a whole (one launch per
        # stage, no stage-level timing entry point for gate/up)
        rf_kernel, rf_bytes, rf_us = "E4M3 decode step (all stage launches)", total_b, us_step
    elif one_launch:
        # dominant kernel: the one-launch step itself (one kernel per step);
        # its average launch time is the step time measured above
        rf_kernel, rf_bytes, rf_us = "step_m1_kernel (one-launch decode step)", total_b, us_step
    else:
        # dominant kernel: gate/up projection, back-to-back launches over the copies
        a_buf = torch.empty((M, shape.d_ffn), dtype=torch.int16, device="cuda")
        hb = ws.view("h_bf16", torch.int16, M * shape.d_model)
        R = 8 * C

        def gu(i):
            B.i4d_ffn_gate_up(layers[i % C].struct, hb, M, a_buf)

        g_gu = capture(R, gu)
        g_gu.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        g_gu.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        rf_kernel, rf_bytes = "proj gate/up + SwiGLU", gate_up_bytes(shape)
        rf_us = e0.elapsed_time(e1) * 1e3 / R
    rf_gbps = rf_bytes / (rf_us * 1e-6) / 1e9

    result = {
        "metric": ("us per INT4 decode block step (+ achieved HBM GB/s)" if args.stage == "step" else
                   "us per attention launch on the INT4 KV cache (+ achieved HBM GB/s)"),
        "value": round(us_step, 3),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": max(args.warmup, 1),
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3 x bf16 -> f32" if args.weights == "e4m3" else "int4 x bf16/fp16 -> f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "d_model": shape.d_model, "n_q_heads": shape.n_q_heads,
                   "n_kv_heads": shape.n_kv_heads, "head_dim": shape.head_dim, "d_ffn": shape.d_ffn,
                   "M": M, "ctx_total": int(lengths.sum()), "ctx_max": maxL, "num_splits": splits,
                   "layer_copies": C, "one_launch_step": one_launch, "weights": args.weights, "stage": args.stage,
                   "timing": "hip graph of K steps, events on the launch stream"},
        "hbm_GBps": round(gbps, 1),
        "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "bytes_per_step": {"total": total_b, "weights": w_b, "kv": kv_b},
        "roofline": {"kernel": rf_kernel, "bound": "hbm",
                     "achieved": round(rf_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(rf_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": traffic_of(args.workload if not args.M else f"{args.workload}@M{M}", rf_kernel),
                     "avg_launch_us": round(rf_us, 3), "bytes_per_launch": rf_bytes},
        "device_errors": device_errors(caches),
        "setup_s": round(setup_s, 1),
    }

    if not args.no_cpu and args.stage == "step":
        result["cpu_baseline"] = cpu_baseline(shape, lw, lengths, pre, xb, args.cpu_steps, args.workload)
    print(json.dumps(result), flush=True)


def full_model(args, wl, torch, B, D, synth):
    """n_layers stacked blocks (one row, the workload's context per layer and
    its split count) followed by the final RMSNorm, the bf16 LM head and the
    argmax: one decode step of the whole model.  Layer l has its own seed
    (workload seed + l) for its weights and its cached tokens, and its own
    KV cache; one step reads every layer's weights and cache once plus the
    LM head, so nothing stays in the 256 MB Infinity Cache between steps."""
    shape, L, nl = wl.shape, wl.ctx, wl.n_layers
    lengths = np.array([L], np.int32)
    t0 = time.time()
    layers, caches, _ = D.stacked_layers(shape, [wl.seed + l for l in range(nl)], lengths)
    V = synth.LM_VOCAB
    w_lm, g_lm = synth.make_lm_head(shape.d_model, V, synth.LM_HEAD_SEED)
    w16 = torch.from_numpy(B.i4d_pack_lm_head(w_lm, g_lm).view(np.int16)).cuda()
    del w_lm
    ws = D.Workspace(shape, 1, L, wl.num_splits)
    lm_bytes = B.i4d_lm_head_workspace_bytes(V, 1)
    lm_ws = torch.zeros(lm_bytes, dtype=torch.uint8, device="cuda")
    xs = [D.to_device_u16(synth.make_x(shape, 1, wl.seed)), None]
    xs[1] = torch.empty_like(xs[0])
    hs = [torch.empty_like(xs[0]) for _ in range(2)]
    tok = torch.zeros(1, dtype=torch.int32, device="cuda")
    ctx = torch.from_numpy(lengths).cuda()
    setup_s = time.time() - t0

    def step(_):
        cur = xs[0]
        for l in range(nl):
            out = hs[l % 2]
            B.i4d_decode_block_step(layers[l].struct, caches[l].struct, cur, out, ctx, 1, L, wl.num_splits,
                                    ws.buf, ws.nbytes, None)
            cur = out
        B.i4d_lm_head_argmax(w16, V, shape.d_model, cur, 1, shape.rms_eps, None, tok, lm_ws, lm_bytes, None)

    step(0)
    torch.cuda.synchronize()
    require_clean(caches, "eager full-model step")
    K = max(1, min(args.steps, 20))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(K):
            step(i)
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    require_clean(caches, "timed full-model steps")
    ms_step = e0.elapsed_time(e1) / K
    blk_b, w_b, kv_b = algorithmic_bytes(shape, lengths)
    lm_b = V * shape.d_model * 2
    total_b = nl * blk_b + lm_b
    gbps = total_b / (ms_step * 1e-3) / 1e9
    result = {
        "metric": "ms per full-model INT4 decode step (+ achieved HBM GB/s)",
        "value": round(ms_step, 4), "unit": "ms/step", "n_gpus": 1, "steps": K, "warmup": 1,
        "ms_per_step": round(ms_step, 4), "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "int4 x bf16/fp16 -> f32; bf16 LM head", "data": "synthetic",
        "config": {"workload": wl.name, "n_layers": nl, "layer_seeds": [wl.seed, wl.seed + nl - 1],
                   "d_model": shape.d_model, "n_q_heads": shape.n_q_heads,
                   "n_kv_heads": shape.n_kv_heads, "head_dim": shape.head_dim, "d_ffn": shape.d_ffn, "M": 1,
                   "ctx_per_layer": L, "num_splits": wl.num_splits, "vocab": V,
                   "timing": "hip graph of K full steps, events on the launch stream"},
        "hbm_GBps": round(gbps, 1), "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "bytes_per_step": {"total": total_b, "per_layer": blk_b, "lm_head": lm_b},
        "token": int(tok.item()),
        "device_errors": device_errors(caches),
        "pages_context": "the pages report 2.8 ms per full Llama-3.1-8B decode step on one H100 "
                         "(context length not stated), so it is not the same workload",
        "setup_s": round(setup_s, 1),
    }
    print(json.dumps(result), flush=True)


def prefill_bench(args, pw, torch, B, D, synth):
    """The FP8 prefill of the QKV projection on a packed batch: one step =
    i4d_prefill_qkv_e4m3 (prep launch + FP8 GEMM launch with the q / INT4
    cache epilogue) + i4d_fp8_scales_update, inputs resident in HBM, K steps
    in one captured HIP graph between two events.  The roofline entry is the
    GEMM launch alone (i4d_prefill_project replayed over the prepared
    workspace), priced against the dense fp8 MFMA peak with the algorithmic
    2 T N d flops of the projection."""
    shape, T, R = pw.shape, pw.T, len(pw.seqlens)
    t0 = time.time()
    lw = synth.make_layer(shape, pw.seed)
    layer = D.PrefillWeights(shape, lw)
    caps = [s + n for s, n in zip(pw.starts, pw.seqlens)]
    cache = D.DeviceCache(shape, caps)
    xb = synth.make_prefill_x(shape, T, pw.seed)
    x_d = D.to_device_u16(xb)
    cu = torch.from_numpy(synth.prefill_offsets(pw.seqlens)).cuda()
    st = torch.tensor(pw.starts, dtype=torch.int32, device="cuda")
    sx0 = float(np.max(np.abs(synth.bf16_bits_to_f32(xb)))) / 448.0
    scales = torch.tensor([sx0, 1.0, 0.0, 0.0], dtype=torch.float32, device="cuda")
    cs = B.make_shape(shape)
    nbytes = B.i4d_prefill_workspace_bytes(cs, T)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    q8 = torch.empty((T, shape.n_q_heads * shape.head_dim), dtype=torch.uint8, device="cuda")
    setup_s = time.time() - t0
    stream = torch.cuda.current_stream()

    def step(_):
        B.i4d_prefill_qkv_e4m3(layer.struct, cache.struct, x_d, T, cu, st, R, scales, q8, None, None, ws, nbytes)
        B.i4d_fp8_scales_update(scales)

    def project(_):
        B.i4d_prefill_project(layer.struct, cache.struct, T, cu, st, R, scales, q8, None, None, ws, nbytes)

    step(0)  # the delayed scales of this input: the timed steps run with them
    torch.cuda.synchronize()
    require_clean([cache], "prefill warm-up")

    def capture(n, fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                fn(i)
        return g

    def timed(fn, n):
        g_w = capture(max(args.warmup, 1), fn)
        g = capture(n, fn)
        g_w.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n

    us_step = timed(step, args.steps)
    us_gemm = timed(project, args.steps)
    require_clean([cache], "timed prefill steps")
    N = shape.n_qkv
    flops = 2.0 * T * N * shape.d_model
    tflops_gemm = flops / (us_gemm * 1e-6) / 1e12
    result = {
        "metric": "us per FP8 prefill QKV projection step (prep + FP8 GEMM with q / INT4 cache epilogue + "
                  "scale update)",
        "value": round(us_step, 3),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": max(args.warmup, 1),
        "ms_per_step": round(us_step / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3 x e4m3 -> f32",
        "data": "synthetic",
        "config": {"workload": pw.name, "d_model": shape.d_model, "n_q_heads": shape.n_q_heads,
                   "n_kv_heads": shape.n_kv_heads, "head_dim": shape.head_dim, "T": T, "requests": R,
                   "seqlens": list(pw.seqlens), "stage": "prefill",
                   "timing": "hip graph of K steps, events on the launch stream"},
        "tflops_step": round(flops / (us_step * 1e-6) / 1e12, 1),
        "flops_per_step": flops,
        "roofline": {"kernel": "prefill_gemm_kernel (FP8 MFMA GEMM + epilogue)", "bound": "mfma",
                     "achieved": round(tflops_gemm, 1), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops_gemm / FP8_PEAK_TFLOPS, 4),
                     "traffic": traffic_of(pw.name, "prefill_gemm_kernel (FP8 MFMA GEMM + epilogue)"),
                     "avg_launch_us": round(us_gemm, 3), "flops_per_launch": flops},
        "device_errors": device_errors([cache]),
        "pages_context": "the pages time a whole 8B-shape prefill at S = 2048 on one H100 (804.2 us), not this "
                         "projection alone, so there is no like-for-like baseline",
        "setup_s": round(setup_s, 1),
    }
    if not args.no_cpu:
        result["cpu_baseline"] = prefill_cpu_baseline(shape, lw, xb, pw, args.cpu_steps)
    print(json.dumps(result), flush=True)


def prefill_cpu_baseline(shape, lw, xb, pw, n_reps, sample=512):
    """The oracle's prefill_qkv on the first `sample` tokens of the batch
    (one request from position 0; the dense weight computed beforehand),
    median of n_reps, scaled to the batch's T tokens (the projection is
    linear in T)."""
    import oracle as O
    from threadpoolctl import threadpool_info
    blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    model, nproc = host_cpu()
    qkv = O.quantize_weight_e4m3_mx(lw.w_qkv, lw.gamma_attn)
    W = O.dense(qkv)
    n = min(sample, pw.T)
    times = []
    for _ in range(max(1, n_reps)):
        t = time.time()
        O.prefill_qkv(shape, qkv, xb[:n], np.array([0, n], np.int32), [0], np.float32(0.1), np.float32(0.1),
                      W_dense=W)
        times.append(time.time() - t)
    us = float(np.median(times)) * 1e6 * pw.T / n
    return {"value": round(us, 1), "unit": "us/step", "cores": int(blas_threads), "kind": "oracle",
            "sample": f"prefill_qkv on {n} of the {pw.T} tokens of {pw.name} (median of {max(1, n_reps)}; fp64 "
                      f"numpy), scaled by {pw.T}/{n}",
            "host_cpu": model, "nproc": int(nproc)}


def host_cpu():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        nproc = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        nproc = os.cpu_count()
    return model, nproc


def cpu_baseline(shape, lw, lengths, pre, xb, n_steps, workload):
    """The CPU oracle, as it stands, on a bounded sample of the same
    workload: the median of n_steps block steps with numpy's BLAS pool at
    its default size (the threads it used are reported as `cores`), and of
    two steps on one thread for the small single-row workloads."""
    import oracle as O
    from threadpoolctl import threadpool_info, threadpool_limits
    blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    model, nproc = host_cpu()
    ql = O.quantize_layer(lw)

    def timed(n):
        times = []
        for _ in range(n):
            cache = O.build_cache(shape, lengths, pre)
            t = time.time()
            O.decode_block(shape, ql, cache, xb, lengths)
            times.append(time.time() - t)
        return float(np.median(times)) * 1e6

    us = timed(n_steps)
    out = {"value": round(us, 1), "unit": "us/step", "cores": int(blas_threads), "kind": "oracle",
           "sample": f"{n_steps} block steps of {workload} (median; fp64 numpy, weights dequantized each step)",
           "host_cpu": model, "nproc": int(nproc)}
    if len(lengths) == 1 and shape.d_model <= 4096:
        with threadpool_limits(limits=1):
            out["value_1thread"] = round(timed(2), 1)
    return out


if __name__ == "__main__":
    main()
