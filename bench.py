#!/usr/bin/env python3
"""GPT-2 training-step benchmark on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is gpt2_forward (with targets) + gpt2_backward + gpt2_adamw_step over one
synthetic batch (seeded weights and token ids, inputs resident in HBM before the
timed region).  Prints ONE JSON line on stdout: whole-job training tokens/s, the
roofline position of the dominant kernel (timed live with the library's HIP-event
launch profiler) and the CPU oracle's throughput on a bounded sample.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "train tokens/sec (fwd+bwd+AdamW) GPT-2 124M B=8 T=1024; % MFMA peak"
PEAK_TFLOPS = {"bf16": 2500.0, "fp32": 157.3}   # MI355X dense MFMA
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def model_flops_per_step(m, B, T):
    """(6 N + 6 L C (T+1)) B T: dense matmul flops of forward+backward for N
    parameters, plus causal attention counting only unmasked pairs."""
    import synth
    N = synth.num_parameters(m)
    return (6.0 * N + 6.0 * m.num_layers * m.channels * (T + 1)) * B * T


def source_digest():
    """Digest of the library's kernel sources: counter readings taken on other
    sources do not describe the current kernels."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "transformer_lm_fwd_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed FETCH_SIZE / WRITE_SIZE
    counter summary (profiles/traffic_<workload>.json), scaled by the copy-kernel
    calibration; None when there is no reading or the kernel sources changed since."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    out = {"traffic": None}
    if not os.path.exists(path):
        return out
    with open(path) as f:
        t = json.load(f)
    k = t.get("kernels", {}).get(kernel)
    if k is None or t.get("source_digest") != source_digest():
        return out
    out["traffic"] = round(k["fetch_bytes"] + k["write_bytes"])
    out["traffic_fetch"] = round(k["fetch_bytes"])
    out["traffic_write"] = round(k["write_bytes"])
    return out


def cpu_baseline(w, params, x, y, rotary=False, steps=2, threads_alt=8):
    """The float oracle on one whole sequence of the workload: batch row 0, all T
    positions, full forward + backward + AdamW, `steps` steps with one OpenMP thread
    per host core this process may run on, then one step with `threads_alt` threads
    (the thread count of the pages' CPU run).  Tokens/s = T / step time; the step's
    fixed costs (AdamW over every parameter) are spread over T tokens instead of B*T,
    and attention is at the workload's full length."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    o = oracle.Oracle(w.model, 1, w.T, "f32")
    o.set("params", params)
    if rotary:
        o.set_rotary(True)
    xs, ys = x[:1], y[:1]

    def timed(threads, n):
        oracle.set_num_threads(threads)
        used = oracle.num_threads()
        times = []
        for _ in range(n):
            t0 = time.perf_counter()
            o.step(xs, ys, w, len(times) + 1)
            times.append(time.perf_counter() - t0)
        return used, min(times), times

    used, best, times = timed(cores, steps)
    used8, best8, _ = timed(threads_alt, 1)
    o.close()
    oracle.set_num_threads(cores)
    return {"value": round(w.T / best, 2), "unit": "tokens/s", "cores": used, "kind": "oracle",
            "sample": f"float oracle, full step (fwd+bwd+AdamW) on batch row 0 of the {w.name} workload "
                      f"(B=1, T={w.T}), fastest of {steps} steps on {used} threads "
                      f"({', '.join(f'{t:.2f}' for t in times)} s)",
            "at_8_threads": {"value": round(w.T / best8, 2), "unit": "tokens/s", "cores": used8,
                             "step_s": round(best8, 3)}}


def vendor_gemm_bench():
    """The vendor BLAS on the step's product shapes (plain products: no bias, residual or
    GELU epilogue, bf16 out), 5 untimed and 20 timed calls each, HIP events around the 20."""
    import torch
    torch.cuda.set_device(0)
    C, BT, V = 768, 8192, 50257
    # name, M, N, K, form: "xwT" = X[M,K] W[N,K]^T, "dyW" = dY[M,K] W[K,N], "dyTx" = dY[K,M]^T X[K,N]
    shapes = [("qkv forward", BT, 3 * C, C, "xwT"), ("attention projection forward", BT, C, C, "xwT"),
              ("c_fc forward", BT, 4 * C, C, "xwT"), ("c_fc projection forward", BT, C, 4 * C, "xwT"),
              ("lm_head forward", BT, V, C, "xwT"),
              ("c_fc projection dX", BT, 4 * C, C, "dyW"), ("c_fc dX", BT, C, 4 * C, "dyW"),
              ("attention projection dX", BT, C, C, "dyW"), ("qkv dX", BT, C, 3 * C, "dyW"),
              ("lm_head dX", BT, C, V, "dyW"),
              ("c_fc projection dW", C, 4 * C, BT, "dyTx"), ("c_fc dW", 4 * C, C, BT, "dyTx"),
              ("attention projection dW", C, C, BT, "dyTx"), ("qkv dW", 3 * C, C, BT, "dyTx"),
              ("lm_head dW", V, C, BT, "dyTx")]
    g = torch.Generator(device="cuda")
    g.manual_seed(1)
    out = {}
    for name, M, N, K, form in shapes:
        def rnd(r, c):
            return torch.randn(r, c, device="cuda", dtype=torch.bfloat16, generator=g)
        if form == "xwT":
            a, b = rnd(M, K), rnd(N, K)
            f = lambda: torch.matmul(a, b.t())
        elif form == "dyW":
            a, b = rnd(M, K), rnd(K, N)
            f = lambda: torch.matmul(a, b)
        else:
            a, b = rnd(K, M), rnd(K, N)
            f = lambda: torch.matmul(a.t(), b)
        for _ in range(5):
            f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(20):
            f()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / 20
        out[name] = {"M": M, "N": N, "K": K, "us": round(us, 1), "tflops": round(2.0 * M * N * K / us / 1e6, 1)}
        log(f"  {name:30s} {M:6d} x {N:6d} x {K:6d}  {us:8.1f} us  {out[name]['tflops']:7.1f} TFLOP/s")
        del a, b
    print(json.dumps({"vendor_gemm": out, "library": "torch.matmul (bf16)", "unit": "us"}), flush=True)


def vendor_attention_bench():
    """PyTorch's fused attention (scaled_dot_product_attention, causal, bf16, restricted to the
    flash and memory-efficient backends so that no unfused path runs) at the step's attention
    shape, B=8, 12 heads, T=1024, head size 64, on contiguous [B, heads, T, 64] tensors:
    forward alone, then forward + backward, 5 untimed and 20 timed calls each."""
    import torch
    from torch.nn.attention import SDPBackend, sdpa_kernel
    torch.cuda.set_device(0)
    B, NH, T, hs = 8, 12, 1024, 64
    g = torch.Generator(device="cuda")
    g.manual_seed(2)
    q, k, v, do = (torch.randn(B, NH, T, hs, device="cuda", dtype=torch.bfloat16, generator=g) for _ in range(4))
    q.requires_grad_(True)
    k.requires_grad_(True)
    v.requires_grad_(True)
    out = {}
    with sdpa_kernel([SDPBackend.FLASH_ATTENTION, SDPBackend.EFFICIENT_ATTENTION]):
        def fwd():
            with torch.no_grad():
                return torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)

        def fwd_bwd():
            o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)
            torch.autograd.grad(o, (q, k, v), do)  # fresh gradients: no accumulation kernels

        for name, f in (("forward", fwd), ("forward + backward", fwd_bwd)):
            for _ in range(5):
                f()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(20):
                f()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / 20
            pairs = B * NH * T * (T + 1) / 2
            flops = (4 if name == "forward" else 12) * hs * pairs
            out[name] = {"us": round(us, 1), "tflops": round(flops / us / 1e6, 1)}
            log(f"  attention {name:20s} {us:8.1f} us  {out[name]['tflops']:7.1f} TFLOP/s (causal pairs only)")
    print(json.dumps({"vendor_attention": out, "library": "torch scaled_dot_product_attention (bf16, causal)",
                      "shape": {"B": B, "heads": NH, "T": T, "head_size": hs}, "unit": "us"}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gpt2_124m_b8t1024_bf16")
    ap.add_argument("--profile-steps", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernel-table", default=None, help="write the per-kernel profile as JSON here")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy 1 GiB device-to-device 5 times (a kernel of known traffic for the "
                         "FETCH_SIZE / WRITE_SIZE counter calibration) and exit")
    ap.add_argument("--launch-order", default=None,
                    help="write the kernel names of the profiled steps' launches, in launch order, to this JSON file "
                         "(to match a counter trace of the same steps dispatch by dispatch)")
    ap.add_argument("--mfma-probe", action="store_true",
                    help="only measure the matrix cores' sustained rate for three MFMA forms (gpt2_mfma_peak, "
                         "register operands, no memory traffic), five times each, print one JSON line and exit")
    ap.add_argument("--unfused", action="store_true",
                    help="call gpt2_backward and gpt2_adamw_step separately instead of gpt2_backward_adamw")
    ap.add_argument("--decode", action="store_true",
                    help="measure incremental generation instead of training: prefill a prompt, then time "
                         "--steps one-row decode steps per sequence (prints its own JSON line)")
    ap.add_argument("--rotary", action="store_true",
                    help="the training step with the rotary position embedding instead of the learned wpe")
    ap.add_argument("--mxfp8", action="store_true",
                    help="time the forward pass (with the loss) with MX FP8 block and lm_head products beside the "
                         "bf16 forward (prints its own JSON line)")
    ap.add_argument("--io", action="store_true",
                    help="time the host I/O of a run: token-file batches, checkpoint write / read (own JSON line)")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="only time the vendor BLAS (torch.matmul in bf16) on the training step's fifteen product "
                         "shapes, as a point of comparison for this library's GEMM kernels, print one JSON line "
                         "and exit")
    ap.add_argument("--vendor-attention", action="store_true",
                    help="only time PyTorch's fused causal attention (flash / memory-efficient backends, bf16) at "
                         "the step's attention shape, forward and forward + backward, print one JSON line and exit")
    ap.add_argument("--decode-batch", type=int, default=8)
    ap.add_argument("--prompt", type=int, default=512)
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build runs the training step on a single MI355X; "
              "multi-GPU runs are not part of it.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "copies": 5}), flush=True)
        return

    if args.vendor_gemm:
        return vendor_gemm_bench()
    if args.vendor_attention:
        return vendor_attention_bench()

    import synth
    from transformer_lm_fwd_amd import Arena, binding

    if args.mfma_probe:
        torch.cuda.set_device(0)
        kinds = {"bf16_32x32x16": binding.MFMA_BF16_32X32X16, "bf16_16x16x32": binding.MFMA_BF16_16X16X32,
                 "mxfp8_32x32x64": binding.MFMA_MXFP8_32X32X64}
        peaks = {"bf16_32x32x16": 2500.0, "bf16_16x16x32": 2500.0, "mxfp8_32x32x64": 5000.0}
        out = {}
        for name, kind in kinds.items():
            r = [binding.mfma_peak(kind) for _ in range(5)]
            out[name] = {"tflops_runs": [round(v, 1) for v in r], "tflops_best": round(max(r), 1),
                         "published_peak": peaks[name], "frac_of_published": round(max(r) / peaks[name], 4)}
        print(json.dumps({"mfma_probe": out, "unit": "TFLOP/s"}), flush=True)
        return

    if args.decode:
        return decode_bench(args)
    if args.mxfp8:
        return mx_forward_bench(args)
    if args.io:
        return io_bench(args)

    w = synth.WORKLOADS[args.workload]
    m = w.model
    t0 = time.time()
    params = synth.init_params(m)
    x, y = synth.inputs_targets(w)
    log(f"[bench] {w.name}: params generated in {time.time() - t0:.1f} s")
    torch.cuda.set_device(0)
    arena = Arena(m, w.B, w.T, w.dtype)
    arena.load_params(params)
    if args.rotary:
        arena.set_position_encoding(binding.GPT2_POS_ROTARY)
    xi = torch.from_numpy(x).to(torch.int32).cuda()
    yi = torch.from_numpy(y).to(torch.int32).cuda()
    t = 0
    # warm-up (the first call also checks the id range on the host)
    for i in range(max(1, args.warmup)):
        t += 1
        arena.step(xi, yi, w, t, check_ids=(i == 0), fused=not args.unfused)
    torch.cuda.synchronize()
    first_loss = arena.loss()
    log(f"[bench] warm-up done, loss {first_loss:.4f}")

    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        t += 1
        arena.step(xi, yi, w, t, check_ids=False, fused=not args.unfused)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end)
    ms_per_step = ms / args.steps
    loss = arena.loss()
    if not math.isfinite(loss):
        raise SystemExit(f"non-finite loss {loss}")
    tokens = w.B * w.T * args.steps
    value = tokens / (ms / 1e3)
    F = model_flops_per_step(m, w.B, w.T)
    mfma_frac = F / (ms_per_step / 1e3) / (PEAK_TFLOPS[w.dtype] * 1e12)
    log(f"[bench] {args.steps} steps in {ms:.1f} ms: {ms_per_step:.3f} ms/step, {value:,.0f} tokens/s, "
        f"model flops {F / 1e12:.3f} TF/step = {mfma_frac * 100:.1f}% of {w.dtype} MFMA peak, loss {loss:.4f}")

    # per-kernel profile of a few more steps (HIP events around every launch)
    binding.profile(True)
    for _ in range(args.profile_steps):
        t += 1
        arena.step(xi, yi, w, t, check_ids=False, fused=not args.unfused)
    torch.cuda.synchronize()
    binding.profile(False)
    stats = binding.profile_read()
    tot = sum(s["total_ms"] for s in stats)
    stats.sort(key=lambda s: -s["total_ms"])
    log(f"[bench] kernel profile over {args.profile_steps} steps "
        f"({tot / max(1, args.profile_steps):.3f} ms/step in kernels):")
    for s in stats:
        avg = s["total_ms"] / s["launches"]
        tf = s["flops"] / (s["total_ms"] / 1e3) / 1e12 if s["flops"] else 0.0
        gbs = s["bytes"] / (s["total_ms"] / 1e3) / 1e9
        log(f"  {s['name']:<28} {s['launches']:6d} launches {s['total_ms'] / args.profile_steps:9.3f} ms/step "
            f"({100 * s['total_ms'] / tot:5.1f}%) avg {avg * 1e3:9.1f} us  {tf:8.1f} TFLOP/s  {gbs:8.1f} GB/s")
    if args.kernel_table:
        with open(args.kernel_table, "w") as f:
            json.dump({"workload": w.name, "profile_steps": args.profile_steps, "kernels": stats}, f, indent=1)
    if args.launch_order:
        with open(args.launch_order, "w") as f:
            json.dump({"workload": w.name, "profile_steps": args.profile_steps, "launches": binding.profile_order()}, f)
    roof = None
    if stats:
        dom = stats[0]
        avg_s = dom["total_ms"] / dom["launches"] / 1e3
        if dom["flops"] > 0:
            achieved = dom["flops"] / dom["launches"] / avg_s / 1e12
            roof = {"kernel": dom["name"], "bound": "mfma", "achieved": round(achieved, 2),
                    "peak": PEAK_TFLOPS[w.dtype], "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS[w.dtype], 4)}
        else:
            achieved = dom["bytes"] / dom["launches"] / avg_s / 1e9
            roof = {"kernel": dom["name"], "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4)}
        roof["avg_launch_us"] = round(avg_s * 1e6, 2)
        roof["algorithmic_bytes_per_launch"] = round(dom["bytes"] / dom["launches"])
        roof.update(measured_traffic(w.name + ("_rotary" if args.rotary else ""), dom["name"]))

    # the matrix cores' sustained rate on this machine (register operands, no memory traffic)
    probe = {"bf16_32x32x16": round(binding.mfma_peak(binding.MFMA_BF16_32X32X16), 1),
             "bf16_16x16x32": round(binding.mfma_peak(binding.MFMA_BF16_16X16X32), 1),
             "mxfp8_32x32x64": round(binding.mfma_peak(binding.MFMA_MXFP8_32X32X64), 1), "unit": "TFLOP/s"}
    log(f"[bench] MFMA probe: {probe}")
    measured_peak = probe["bf16_32x32x16"] if w.dtype == "bf16" else None
    if roof is not None and roof["bound"] == "mfma" and measured_peak:
        roof["measured_peak"] = measured_peak
        roof["frac_measured_peak"] = round(roof["achieved"] / measured_peak, 4)

    rope = None
    if args.rotary or getattr(m, "block", "gpt2") == "llama":  # the rotary turns and SwiGLU: elementwise, HBM-bound
        rope = {}
        for s in stats:
            if s["name"] in ("rope_fwd", "rope_bwd", "swiglu_fwd", "swiglu_bwd"):
                avg_s = s["total_ms"] / s["launches"] / 1e3
                gbs = s["bytes"] / s["launches"] / avg_s / 1e9
                rope[s["name"]] = {"avg_launch_us": round(avg_s * 1e6, 2), "bytes_per_launch": round(s["bytes"] / s["launches"]),
                                   "achieved_gbs": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                                   "ms_per_step": round(s["total_ms"] / args.profile_steps, 4)}

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline ...")
        cpu = cpu_baseline(w, params, x, y, rotary=args.rotary and getattr(m, "block", "gpt2") == "gpt2")
        log(f"[bench] CPU oracle: {cpu['value']:.1f} tokens/s on {cpu['cores']} threads")

    metric, wname = METRIC, w.name
    if args.rotary:
        metric = METRIC.replace("GPT-2 124M", "GPT-2 124M with rotary positions")
        wname = w.name + "_rotary"
    if getattr(m, "block", "gpt2") == "llama":
        metric = METRIC.replace("GPT-2 124M", "Llama-style 124M (RMSNorm, SwiGLU 2048, rotary)")
    out = {
        "metric": metric, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic (seeded random-init weights, uniform token ids)"
        if w.tokens == "uniform" else "synthetic (seeded random-init weights, Zipf token ids)",
        "config": {"workload": wname, "B": w.B, "T": w.T, "layers": m.num_layers, "heads": m.num_heads,
                   "channels": m.channels, "vocab": m.vocab_size, "tokens": w.tokens},
        "mfma_peak_frac": round(mfma_frac, 4), "model_tflop_per_step": round(F / 1e12, 4),
        "mfma_peak_frac_measured": round(F / (ms_per_step / 1e3) / (measured_peak * 1e12), 4)
        if measured_peak else None, "mfma_probe": probe,
        "loss": round(loss, 5), "roofline": roof, "cpu_baseline": cpu,
    }
    if rope is not None:
        out["elementwise_kernels"] = rope
    print(json.dumps(out), flush=True)


def decode_bytes_per_step(m, batch, ctx):
    """HBM bytes one decode step must move at least: every weight matrix once (bf16:
    the four block products of each layer and the tied lm_head), the cached keys and
    values of every layer ([batch, ctx, 2C] bf16), and the fp32 logits written."""
    C, L, V = m.channels, m.num_layers, m.vocab_size
    weights = 2.0 * (L * 12 * C * C + V * C)
    kv = 2.0 * L * batch * ctx * 2 * C
    return weights + kv + 4.0 * batch * V


def decode_bench(args):
    import numpy as np
    import torch
    import synth
    from transformer_lm_fwd_amd import Arena, Generator, binding

    w = synth.WORKLOADS[args.workload]
    m = w.model
    batch, n, steps = args.decode_batch, args.prompt, args.steps
    name = f"gpt2_124m_decode_b{batch}_ctx{n}" if m == synth.GPT2_124M else f"{w.name}_decode_b{batch}_ctx{n}"
    t0 = time.time()
    params = synth.init_params(m)
    prompt = synth.token_windows(w, B=batch, T=n)[:, :n]
    log(f"[bench] {name}: params generated in {time.time() - t0:.1f} s")
    torch.cuda.set_device(0)
    arena = Arena(m, batch, n, w.dtype)
    arena.load_params(params)
    gen = Generator(arena, batch, min(m.max_seq_len, n + steps + max(1, args.warmup) + 1))
    tok = torch.from_numpy(np.ascontiguousarray(prompt)).to(torch.int32).cuda()
    # the tokens fed to the decode steps: the next ids of the same synthetic stream (the
    # cost of a step does not depend on them; the timed region runs library kernels only)
    feed = synth.token_windows(w, B=batch, T=n + steps + args.warmup + 1)[:, n:]
    feed = [torch.from_numpy(np.ascontiguousarray(feed[:, i])).to(torch.int32).cuda() for i in range(feed.shape[1])]

    # warm-up: a prefill and a few steps, then restart the cache with the same prompt
    gen.prefill(tok)
    for i in range(max(1, args.warmup)):
        gen.decode(feed[i], check_ids=False)
    torch.cuda.synchronize()
    gen.prefill(tok)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        gen.decode(feed[i], check_ids=False)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end)
    ms_per_step = ms / steps
    value = batch * steps / (ms / 1e3)
    ctx_mean = n + (steps + 1) / 2.0  # cached positions read, averaged over the timed steps
    bytes_step = decode_bytes_per_step(m, batch, ctx_mean)
    gbs = bytes_step / (ms_per_step / 1e3) / 1e9
    log(f"[bench] {steps} decode steps in {ms:.2f} ms: {ms_per_step * 1e3:.1f} us/step, {value:,.0f} tokens/s, "
        f"{bytes_step / 1e6:.1f} MB/step at least = {gbs:.0f} GB/s ({100 * gbs / PEAK_HBM_GBS:.1f}% of HBM peak)")

    # per-kernel profile of the same number of steps, after restarting the cache
    gen.prefill(tok)
    torch.cuda.synchronize()
    binding.profile(True)
    pk = max(1, min(args.profile_steps * 8, steps))
    for i in range(pk):
        gen.decode(feed[i], check_ids=False)
    torch.cuda.synchronize()
    binding.profile(False)
    stats = sorted(binding.profile_read(), key=lambda s: -s["total_ms"])
    tot = sum(s["total_ms"] for s in stats)
    log(f"[bench] kernel profile over {pk} decode steps ({tot / pk * 1e3:.1f} us/step in kernels):")
    for s in stats:
        avg = s["total_ms"] / s["launches"]
        gb = s["bytes"] / (s["total_ms"] / 1e3) / 1e9
        log(f"  {s['name']:<20} {s['launches']:6d} launches {s['total_ms'] / pk * 1e3:8.1f} us/step "
            f"({100 * s['total_ms'] / tot:5.1f}%) avg {avg * 1e3:7.2f} us  {gb:8.1f} GB/s")
    if args.kernel_table:
        with open(args.kernel_table, "w") as f:
            json.dump({"workload": name, "profile_steps": pk, "kernels": stats}, f, indent=1)
    dom = stats[0] if stats else None
    roof = {"kernel": "decode step (all kernels)", "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "algorithmic_bytes_per_step": round(bytes_step),
            "traffic": None}
    if dom:
        avg_s = dom["total_ms"] / dom["launches"] / 1e3
        roof["dominant_kernel"] = {"kernel": dom["name"], "avg_launch_us": round(avg_s * 1e6, 2),
                                   "achieved_gbs": round(dom["bytes"] / dom["launches"] / avg_s / 1e9, 1)}

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        T_s = 128
        o = oracle.Oracle(m, 1, T_s, "f32")
        o.set("params", params)
        t1, reps = time.perf_counter(), 0
        while reps < 1 or time.perf_counter() - t1 < 10.0:
            o.forward(prompt[:1, :T_s])  # the oracle's next-token logits: a forward over the prefix
            reps += 1
        el = time.perf_counter() - t1
        cpu = {"value": round(reps / el, 4), "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
               "sample": f"next-token logits of one sequence from a {T_s}-token prefix (a full forward pass, "
                         f"the oracle has no cache), {reps} repetitions"}
        log(f"[bench] CPU oracle: {cpu['value']} tokens/s")

    out = {
        "metric": f"decode tokens/sec (KV cache) GPT-2 124M batch {batch}, context {n}->{n + steps}",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic (seeded random-init weights, uniform token ids for prompt and continuation)",
        "config": {"workload": name, "batch": batch, "prompt": n, "layers": m.num_layers, "heads": m.num_heads,
                   "channels": m.channels, "vocab": m.vocab_size},
        "roofline": roof, "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def io_bench(args):
    """Host I/O around the step for the workload's model: batches of B x (T + 1) ids read
    from an int32 token file (a synthetic stream of 64 batches), and a checkpoint of the
    master weights and both AdamW moments written, read back and loaded into the arena."""
    import tempfile
    import numpy as np
    import torch
    import synth
    from transformer_lm_fwd_amd import Arena, binding

    w = synth.WORKLOADS[args.workload]
    m = w.model
    nb = 64
    ids = synth.token_windows(w, seed=7, B=nb * w.B, T=w.T).reshape(-1)[:nb * w.B * w.T + 1].astype(np.int32)
    tmp = tempfile.mkdtemp(prefix="gpt2_io_")
    tok = os.path.join(tmp, "train.bin")
    ids.tofile(tok)
    steps = max(1, args.steps)
    t0 = time.perf_counter()
    for i in range(steps * 4):
        binding.tokens_batch(tok, w.B, w.T, i % nb)
    el = time.perf_counter() - t0
    batches_s = steps * 4 / el
    tok_bytes = w.B * (w.T + 1) * 4
    log(f"[bench] token batches: {batches_s:,.0f} batches/s = {batches_s * w.B * w.T / 1e6:.1f} M tokens/s "
        f"({batches_s * tok_bytes / 1e9:.2f} GB/s of ids)")

    torch.cuda.set_device(0)
    arena = Arena(m, w.B, w.T, w.dtype)
    arena.load_params(synth.init_params(m))
    torch.cuda.synchronize()
    ck = os.path.join(tmp, "ck.bin")
    nbytes = 3 * 4 * arena.n_params + 64
    t0 = time.perf_counter()
    arena.save_checkpoint(ck, 1)
    t_w = time.perf_counter() - t0
    t0 = time.perf_counter()
    arena.load_checkpoint(ck)
    torch.cuda.synchronize()
    t_r = time.perf_counter() - t0
    log(f"[bench] checkpoint {nbytes / 1e9:.2f} GB: save {t_w:.3f} s ({nbytes / t_w / 1e9:.2f} GB/s incl. device "
        f"copies), load {t_r:.3f} s ({nbytes / t_r / 1e9:.2f} GB/s incl. device copies)")

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        t0, reps = time.perf_counter(), 0
        while reps < 16 or time.perf_counter() - t0 < 2.0:
            oracle.token_batch(ids, w.B, w.T, reps % nb)
            reps += 1
        el2 = time.perf_counter() - t0
        cpu = {"value": round(reps / el2, 1), "unit": "batches/s", "cores": 1, "kind": "oracle",
               "sample": f"oracle.token_batch on the same in-memory stream ({reps} batches of {w.B} x {w.T + 1} ids)"}
        log(f"[bench] oracle batches: {cpu['value']} batches/s")
    for f in (tok, ck):
        os.remove(f)
    os.rmdir(tmp)
    out = {
        "metric": f"token-file batches/sec ({w.B} x {w.T + 1} int32 ids per batch); checkpoint GB/s",
        "value": round(batches_s, 1), "unit": "batches/s", "n_gpus": 1, "steps": steps * 4, "warmup": 0,
        "ms_per_step": round(1e3 / batches_s, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int32", "data": "synthetic (seeded uniform token ids written to a temporary file)",
        "config": {"workload": w.name + "_io", "batch": w.B, "seq_len": w.T, "file_batches": nb,
                   "checkpoint_bytes": nbytes},
        "checkpoint": {"save_s": round(t_w, 4), "load_s": round(t_r, 4), "save_gbs": round(nbytes / t_w / 1e9, 3),
                       "load_gbs": round(nbytes / t_r / 1e9, 3)},
        "roofline": None, "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def mx_forward_bench(args):
    """Forward passes (logits and mean loss, no backward) of the workload with the
    block and lm_head products in MX FP8, timed beside the same passes in bf16."""
    import numpy as np
    import torch
    import synth
    from transformer_lm_fwd_amd import Arena, binding

    w = synth.WORKLOADS[args.workload]
    m = w.model
    t0 = time.time()
    params = synth.init_params(m)
    x, y = synth.inputs_targets(w)
    log(f"[bench] {w.name}: inputs generated in {time.time() - t0:.1f} s")
    torch.cuda.set_device(0)
    arena = Arena(m, w.B, w.T, "bf16")
    arena.load_params(params)
    xt = torch.from_numpy(np.ascontiguousarray(x)).to(torch.int32).cuda()
    yt = torch.from_numpy(np.ascontiguousarray(y)).to(torch.int32).cuda()

    def timed(fmt):
        arena.set_gemm_format(fmt)
        for _ in range(max(1, args.warmup)):
            arena.forward(xt, yt, check_ids=False)
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(args.steps):
            arena.forward(xt, yt, check_ids=False)
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / args.steps, arena.loss()

    ms_bf, loss_bf = timed(binding.GPT2_GEMM_BF16)
    ms_mx, loss_mx = timed(binding.GPT2_GEMM_MXFP8)

    def timed_step(fmt):
        # full training steps (forward with the format's products, the bf16 backward,
        # AdamW fused into it), from the same starting weights for both formats
        arena.load_params(params)
        arena.tensor(binding.T_ADAM_M).zero_()
        arena.tensor(binding.T_ADAM_V).zero_()
        arena.set_gemm_format(fmt)
        t = 0
        for _ in range(max(1, args.warmup)):
            t += 1
            arena.step(xt, yt, w, t, check_ids=False)
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(args.steps):
            t += 1
            arena.step(xt, yt, w, t, check_ids=False)
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / args.steps, arena.loss()

    st_bf, sl_bf = timed_step(binding.GPT2_GEMM_BF16)
    st_mx, sl_mx = timed_step(binding.GPT2_GEMM_MXFP8)
    st_dx, sl_dx = timed_step(binding.GPT2_GEMM_MXFP8_DX)
    arena.set_gemm_format(binding.GPT2_GEMM_MXFP8)
    arena.load_params(params)
    tokens = w.B * w.T
    value = tokens / (ms_mx / 1e3)
    log(f"[bench] forward: bf16 {ms_bf:.3f} ms ({tokens / ms_bf:,.0f}K tok/s, loss {loss_bf:.5f}); "
        f"mxfp8 {ms_mx:.3f} ms ({tokens / ms_mx:,.0f}K tok/s, loss {loss_mx:.5f})")
    log(f"[bench] training step (MX or bf16 forward, bf16 backward, AdamW): bf16 {st_bf:.3f} ms "
        f"({tokens / st_bf:,.0f}K tok/s); mxfp8 forward {st_mx:.3f} ms ({tokens / st_mx:,.0f}K tok/s); "
        f"mxfp8 forward + input gradients {st_dx:.3f} ms ({tokens / st_dx:,.0f}K tok/s)")

    binding.profile(True)
    pk = max(1, args.profile_steps)
    for _ in range(pk):
        arena.forward(xt, yt, check_ids=False)
    torch.cuda.synchronize()
    binding.profile(False)
    stats = sorted(binding.profile_read(), key=lambda s: -s["total_ms"])
    tot = sum(s["total_ms"] for s in stats)
    log(f"[bench] kernel profile over {pk} MX forward passes ({tot / pk:.3f} ms/pass in kernels):")
    for s in stats:
        avg = s["total_ms"] / s["launches"]
        tf = s["flops"] / (s["total_ms"] / 1e3) / 1e12
        log(f"  {s['name']:<44} {s['launches']:5d} launches {s['total_ms'] / pk:7.3f} ms/pass "
            f"({100 * s['total_ms'] / tot:5.1f}%) avg {avg * 1e3:8.2f} us  {tf:7.1f} TFLOP/s")
    if args.kernel_table:
        with open(args.kernel_table, "w") as f:
            json.dump({"workload": w.name + "_mxfp8_forward", "profile_steps": pk, "kernels": stats}, f, indent=1)

    # and of training steps with MX forward and input-gradient products (the backward's
    # weight gradients and the optimizer stay bf16 / fp32)
    arena.load_params(params)
    arena.tensor(binding.T_ADAM_M).zero_()
    arena.tensor(binding.T_ADAM_V).zero_()
    arena.set_gemm_format(binding.GPT2_GEMM_MXFP8_DX)
    arena.step(xt, yt, w, 1, check_ids=False)
    torch.cuda.synchronize()
    binding.profile(True)
    for t in range(2, 2 + pk):
        arena.step(xt, yt, w, t, check_ids=False)
    torch.cuda.synchronize()
    binding.profile(False)
    stats_dx = sorted(binding.profile_read(), key=lambda s: -s["total_ms"])
    tot_dx = sum(s["total_ms"] for s in stats_dx)
    log(f"[bench] kernel profile over {pk} training steps with MX forward and input-gradient products "
        f"({tot_dx / pk:.3f} ms/step in kernels):")
    for s in stats_dx:
        avg = s["total_ms"] / s["launches"]
        tf = s["flops"] / (s["total_ms"] / 1e3) / 1e12
        log(f"  {s['name']:<44} {s['launches']:5d} launches {s['total_ms'] / pk:7.3f} ms/step "
            f"({100 * s['total_ms'] / tot_dx:5.1f}%) avg {avg * 1e3:8.2f} us  {tf:7.1f} TFLOP/s")
    if args.kernel_table:
        with open(args.kernel_table.replace(".json", "_dx_step.json"), "w") as f:
            json.dump({"workload": w.name + "_mxfp8_dx_step", "profile_steps": pk, "kernels": stats_dx}, f, indent=1)
    arena.set_gemm_format(binding.GPT2_GEMM_MXFP8)
    arena.load_params(params)
    dom = next(s for s in stats if s["name"].startswith("gemm_mxfp8"))
    avg_s = dom["total_ms"] / dom["launches"] / 1e3
    ach = dom["flops"] / dom["launches"] / avg_s / 1e12
    roof = {"kernel": dom["name"], "bound": "mfma", "achieved": round(ach, 1), "peak": 5000.0, "unit": "TFLOP/s",
            "frac": round(ach / 5000.0, 4), "traffic": None, "avg_launch_us": round(avg_s * 1e6, 2),
            "flops_per_launch": dom["flops"] / dom["launches"]}

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        T_s = min(256, w.T)
        o = oracle.Oracle(m, 1, T_s, "f32")
        o.set("params", params)
        t1, reps = time.perf_counter(), 0
        while reps < 1 or time.perf_counter() - t1 < 10.0:
            o.forward(x[:1, :T_s], y[:1, :T_s])
            reps += 1
        el = time.perf_counter() - t1
        cpu = {"value": round(reps * T_s / el, 2), "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
               "sample": f"float oracle forward with loss (no quantization) on batch row 0, first {T_s} tokens, "
                         f"{reps} repetitions"}
        log(f"[bench] CPU oracle: {cpu['value']} tokens/s")

    out = {
        "metric": "forward tokens/sec (logits + loss) GPT-2 124M B=8 T=1024, MX FP8 block and lm_head products",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_mx, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "mxfp8", "data": "synthetic (seeded random-init weights, uniform token ids)",
        "config": {"workload": w.name + "_mxfp8_forward", "batch": w.B, "seq_len": w.T, "layers": m.num_layers,
                   "heads": m.num_heads, "channels": m.channels, "vocab": m.vocab_size},
        "bf16_forward": {"ms_per_step": round(ms_bf, 5), "value": round(tokens / (ms_bf / 1e3), 1),
                         "loss": loss_bf},
        "training_step": {"mxfp8_forward": {"ms_per_step": round(st_mx, 5),
                                            "value": round(tokens / (st_mx / 1e3), 1), "loss": sl_mx},
                          "bf16": {"ms_per_step": round(st_bf, 5), "value": round(tokens / (st_bf / 1e3), 1),
                                   "loss": sl_bf},
                          "mxfp8_forward_and_input_gradients": {
                              "ms_per_step": round(st_dx, 5), "value": round(tokens / (st_dx / 1e3), 1),
                              "loss": sl_dx},
                          "unit": "tokens/s", "note": "MX FP8 forward products, bf16 backward, AdamW"},
        "mxfp8_loss": loss_mx,
        "roofline": roof, "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
