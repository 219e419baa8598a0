#!/usr/bin/env python3
"""Benchmark one H3-Omni-Transformer block forward on one MI355X.

Workload (default): the 15 s 16:9 768p packed sequence -- 512 text tokens,
600 audio tokens and a 91 x 24 x 42 video grid (92840 tokens) -- through a
full-width bf16 block (hidden 5376, 56 heads x 128, FFN 14336) with seeded
synthetic activations and random-init weights.  A step is one block forward:
the eight libh3blk calls of the fused block (the output and down
projections carry the gated residual, the gate/up projection SwiGLU) on one
stream, inputs already resident in HBM; --unfused times the eleven-call
form instead.

Prints one JSON line: block tokens/s (`value`, from the median of the timed
steps' durations), attention TFLOP/s and % of the 2.5 PFLOP/s dense bf16
MFMA peak, per-kernel times (mean over the timed steps, as a profiler's
average launch time), the roofline of the dominant kernel (attention) and
the fp64 oracle timed on host cores on a bounded token sample
(`cpu_baseline`, with the BLAS library it ran on).

    python bench.py [--gpus 1] [--steps 10] [--warmup 3] [--config 3] [--unfused]
    python bench.py --copy-calibration 1024     # known-size copy for counter scaling
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "H3 block fwd tokens/s + attention bf16 TFLOPS (% peak), 768p 15s seq"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _code_only(text, hash_comments):
    """text without its comments (C and C++ comments, or '#' comments for
    Python), string and character literals kept as written."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif not hash_comments and text.startswith("//", i):
            i = text.find("\n", i)
            i = n if i < 0 else i
        elif not hash_comments and text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        elif hash_comments and c == "#":
            i = text.find("\n", i)
            i = n if i < 0 else i
        else:
            out.append(c)
            i += 1
    return "\n".join(line.rstrip() for line in "".join(out).splitlines() if line.strip())


def kernel_source_hash():
    """Hash of the kernel sources and of the build script that sets their
    compiler flags (either changes the code the counters were taken on).
    Comments and blank lines are left out, so an edit of the documentation
    alone keeps the counters valid."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "video_audio_diffusion_amd", "csrc")
    files = [os.path.join(csrc, f) for f in sorted(os.listdir(csrc))]
    files.append(os.path.join(ROOT, "video_audio_diffusion_amd", "build.py"))
    for path in files:
        with open(path, encoding="utf-8") as fh:
            code = _code_only(fh.read(), hash_comments=path.endswith(".py"))
        h.update(os.path.basename(path).encode() + code.encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary, if it was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        d = json.load(fh)
    if d.get("source_hash") != kernel_source_hash():
        return None
    k = d.get("kernels", {}).get(kernel)
    return None if k is None else k.get("bytes_per_launch")


def step_bytes(cfg):
    """Algorithmic HBM bytes per launch of the streaming passes."""
    N, D, I, F = cfg.n_tok, cfg.dim, cfg.inner, cfg.ffn
    e = 2 if cfg.dtype == "bf16" else 4
    return {"adaln_attn": 2 * N * D * e, "adaln_ffn": 2 * N * D * e,
            "qknorm_rope": 4 * N * I * e, "swiglu": 3 * N * F * e,
            "gate_attn": 3 * N * D * e, "gate_ffn": 3 * N * D * e}


def step_flops(cfg):
    """Matrix-product flops per launch (a fused epilogue's own arithmetic is
    not counted)."""
    N, D, H, d, I, F = cfg.n_tok, cfg.dim, cfg.heads, cfg.head_dim, cfg.inner, cfg.ffn
    f = {"gemm_qkv": 2 * N * D * 3 * I, "attention": 4 * N * N * H * d, "gemm_o": 2 * N * I * D,
         "gemm_gu": 2 * N * D * 2 * F, "gemm_d": 2 * N * F * D}
    f.update(gemm_qkv_rope=f["gemm_qkv"], gemm_o_gate=f["gemm_o"], gemm_gu_swiglu=f["gemm_gu"],
             gemm_d_gate=f["gemm_d"])
    return f


def cpu_baseline(cfg, host, target_s):
    """The fp64 oracle, as it stands, on a token sample of the same workload.

    Every step but attention is row-wise, and attention's cost per query row
    is one sweep over all keys, so whole-block time is the sum of per-token
    costs: the oracle runs all eleven steps for S sampled tokens (their q, k,
    v included) against a full-length K/V of the same shape (other tokens'
    work, filled untimed), and tokens/s = S / time."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle
    from video_audio_diffusion_amd import inputs

    N, H, d, I, F = cfg.n_tok, cfg.heads, cfg.head_dim, cfg.inner, cfg.ffn
    seg, eps = cfg.segments, cfg.eps
    t = {k: inputs.widen(host[k], cfg.dtype) for k in ("w_qkv", "w_o", "w_gu", "w_d")}
    mod = host["mod"].astype(np.float64)
    gq, gk = host["gamma_q"].astype(np.float64), host["gamma_k"].astype(np.float64)
    blk0 = inputs.widen(inputs.draw_rows(cfg, (1024, 2 * I), 4242), cfg.dtype)
    reps = (N + 1023) // 1024
    K_all = np.tile(blk0[:, :I], (reps, 1))[:N]
    V_all = np.tile(blk0[:, I:], (reps, 1))[:N]
    _, pos = oracle.token_table(seg, N)
    g = np.random.Generator(np.random.PCG64(99))
    perm = g.permutation(N)

    def run(rows):
        rows = np.sort(rows)
        x = inputs.widen(host["x"][rows], cfg.dtype)
        a = oracle.adaln_modulate(x, mod, 0, seg, eps, rows=rows)
        qkv = oracle.linear(a, t["w_qkv"])
        q = oracle.rope3d(oracle.qk_rmsnorm(qkv[:, :I], H, d, gq, eps), pos[rows], H, d, cfg.rope_split,
                          cfg.rope_base)
        oracle.rope3d(oracle.qk_rmsnorm(qkv[:, I:2 * I], H, d, gk, eps), pos[rows], H, d, cfg.rope_split,
                      cfg.rope_base)
        o = oracle.attention(q, K_all, V_all, H, d, cfg.scale, rows=rows)
        x1 = oracle.gate_residual(x, oracle.linear(o, t["w_o"]), mod, 0, seg, rows=rows)
        a2 = oracle.adaln_modulate(x1, mod, 1, seg, eps, rows=rows)
        h = oracle.swiglu(oracle.linear(a2, t["w_gu"]), F)
        return oracle.gate_residual(x1, oracle.linear(h, t["w_d"]), mod, 1, seg, rows=rows)

    t0 = time.perf_counter()
    run(perm[:32])
    per_row = (time.perf_counter() - t0) / 32
    S = int(min(max(target_s / per_row, 32), 4096))
    log(f"cpu baseline: {per_row * 1e3:.1f} ms/token in calibration, timing {S} tokens")
    t0 = time.perf_counter()
    run(perm[32:32 + S])
    el = time.perf_counter() - t0
    pools = [p for p in threadpool_info() if p.get("user_api") == "blas"]
    threads = sum(p.get("num_threads", 0) for p in pools) or 1
    vendor = ", ".join(f"{p.get('internal_api', '?')} {p.get('version', '?')}"
                       + (f" ({p['threading_layer']} threads)" if p.get("threading_layer") else "") for p in pools)
    return {"value": S / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "blas": vendor or "none found", "host_cpus": len(os.sched_getaffinity(0)),
            "sample": f"{S} random tokens of the {N}-token sequence through all eleven fp64 steps "
                      f"(their own q/k/v included) against a full {N}-key K/V; {el:.1f} s wall"}


def device_block_weights(cfg, b):
    """Random-init weights of block b of a stack, drawn on the device (torch's
    generator seeded per block and tensor; 770 MB per full-width block, so
    the host draws of the single-block workloads would take minutes)."""
    import torch

    from video_audio_diffusion_amd import inputs
    from video_audio_diffusion_amd.block import BlockWeights

    D, I, F = cfg.dim, cfg.inner, cfg.ffn
    wdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32

    def rnd(name, shape, std, dtype):
        g = torch.Generator(device="cuda")
        g.manual_seed(inputs.stack_seed(cfg.index, b, name))
        return (torch.randn(shape, generator=g, device="cuda", dtype=torch.float32) * std).to(dtype)

    gain = torch.full((cfg.head_dim,), cfg.gamma, device="cuda", dtype=torch.float32)
    return BlockWeights(rnd("w_qkv", (3 * I, D), cfg.w_std, wdt), rnd("w_o", (D, I), cfg.w_std, wdt),
                        rnd("w_gu", (2 * F, D), cfg.w_std, wdt), rnd("w_d", (D, F), cfg.w_std, wdt),
                        rnd("mod", (inputs.N_MOD_SETS, inputs.N_MOD_CHUNKS, D), 1.0, torch.float32), gain, gain)


def bench_fp8(args):
    """The block's four projections as FP8 GEMMs at one workload: each step
    quantises the activation rows (h3_quantize_fp8) and multiplies them with
    weights quantised once per output channel (h3_gemm_fp8, bf16 out)."""
    import torch

    from video_audio_diffusion_amd import blk, inputs

    cfg = inputs.CONFIGS[args.config]
    N, D, I, F = cfg.n_tok, cfg.dim, cfg.inner, cfg.ffn
    shapes = {"qkv": (D, 3 * I), "o": (I, D), "gu": (D, 2 * F), "d": (F, D)}
    g = torch.Generator(device="cuda")
    g.manual_seed(1000 * cfg.index + 900)
    bufs = {}
    for name, (K, Nout) in shapes.items():
        a = torch.randn(N, K, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
        w = (torch.randn(Nout, K, generator=g, device="cuda", dtype=torch.float32) * cfg.w_std).to(torch.bfloat16)
        qa = torch.empty(N, K, dtype=torch.uint8, device="cuda")
        sa = torch.empty(N, dtype=torch.float32, device="cuda")
        qw = torch.empty(Nout, K, dtype=torch.uint8, device="cuda")
        sw = torch.empty(Nout, dtype=torch.float32, device="cuda")
        blk.h3_quantize_fp8(w, K, Nout, K, qw, K, sw, blk.H3_BF16)
        c = torch.empty(N, Nout, dtype=torch.bfloat16, device="cuda")
        bufs[name] = (a, qa, sa, qw, sw, c, K, Nout)
        del w
    log(f"fp8 projections of {cfg.name}: {N} tokens")

    def one(ev):
        for j, (name, (a, qa, sa, qw, sw, c, K, Nout)) in enumerate(bufs.items()):
            if ev is not None:
                ev[2 * j].record()
            blk.h3_quantize_fp8(a, K, N, K, qa, K, sa, blk.H3_BF16)
            if ev is not None:
                ev[2 * j + 1].record()
            blk.h3_gemm_fp8(qa, K, sa, qw, K, sw, c, Nout, N, Nout, K, blk.H3_BF16)
        if ev is not None:
            ev[-1].record()

    for _ in range(args.warmup):
        one(None)
    torch.cuda.synchronize()
    K_ = args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * len(bufs) + 1)] for _ in range(K_)]
    for i in range(K_):
        one(evs[i])
    torch.cuda.synchronize()
    total = evs[0][0].elapsed_time(evs[-1][-1]) / K_
    kern = {}
    for j, (name, (a, qa, sa, qw, sw, c, K, Nout)) in enumerate(bufs.items()):
        tq = sum(e[2 * j].elapsed_time(e[2 * j + 1]) for e in evs) / K_
        tg = sum(e[2 * j + 1].elapsed_time(e[2 * j + 2]) for e in evs) / K_
        fl = 2.0 * N * Nout * K
        kern["quantize_" + name] = {"ms": round(tq, 4), "gbs": round(N * K * 3 / (tq * 1e-3) / 1e9, 1)}
        kern["gemm_fp8_" + name] = {"ms": round(tg, 4), "tflops": round(fl / (tg * 1e-3) / 1e12, 1),
                                    "frac_peak": round(fl / (tg * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4)}
    flops = sum(2.0 * N * v[7] * v[6] for v in bufs.values())
    result = {"metric": "H3 block projections as FP8 (e4m3) GEMMs, TFLOP/s", "value": round(flops / (total * 1e-3) / 1e12, 1),
              "unit": "TFLOP/s", "n_gpus": 1, "steps": K_, "warmup": args.warmup, "ms_per_step": round(total, 3),
              "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8-e4m3 (bf16 out)",
              "data": "synthetic", "config": {"workload": f"{cfg.name} projections", "tokens": N,
                                               "shapes": {k: [N, v[1], v[0]] for k, v in shapes.items()}},
              "kernels": kern}
    print(json.dumps(result), flush=True)


def bench_fp8_attention(args):
    """Attention of one workload on FP8 operands: each step quantises q, k
    and v (h3_quantize_qkv_fp8) and attends (h3_attention_fp8).  The bf16
    kernel (h3_attention_fwd) on the same q, k, v is timed beside it."""
    import torch

    from video_audio_diffusion_amd import blk, inputs

    cfg = inputs.CONFIGS[args.config]
    N, H, hd = cfg.n_tok, cfg.heads, cfg.head_dim
    if cfg.dtype != "bf16" or hd != 128:
        raise SystemExit("the fp8 attention takes bf16 q, k, v with head_dim 128")
    I = H * hd
    n_pad = -(-N // 64) * 64
    g = torch.Generator(device="cuda")
    g.manual_seed(1000 * cfg.index + 950)
    qkv = torch.empty(N, 3 * I, dtype=torch.bfloat16, device="cuda")
    for c0 in range(0, N, 8192):                      # N(0, 1): q and k as after the per-head RMS norm
        c1 = min(N, c0 + 8192)
        qkv[c0:c1] = torch.randn(c1 - c0, 3 * I, generator=g, device="cuda", dtype=torch.float32)
    q8 = torch.empty(N, I, dtype=torch.uint8, device="cuda")
    k8 = torch.empty(N, I, dtype=torch.uint8, device="cuda")
    vt = torch.empty(I, n_pad, dtype=torch.uint8, device="cuda")
    sq = torch.empty(H, N, dtype=torch.float32, device="cuda")
    sk = torch.empty(H, dtype=torch.float32, device="cuda")
    sv = torch.empty(H, dtype=torch.float32, device="cuda")
    o8 = torch.empty(N, I, dtype=torch.bfloat16, device="cuda")
    o16 = torch.empty(N, I, dtype=torch.bfloat16, device="cuda")
    log(f"fp8 attention of {cfg.name}: {N} tokens x {H} heads")

    def one(ev):
        if ev is not None:
            ev[0].record()
        blk.h3_quantize_qkv_fp8(qkv[:, :I], qkv[:, I:2 * I], qkv[:, 2 * I:], 3 * I, N, H, hd, q8, k8, vt, n_pad,
                                sq, sk, sv, blk.H3_BF16)
        if ev is not None:
            ev[1].record()
        blk.h3_attention_fp8(q8, k8, vt, n_pad, sq, sk, sv, o8, I, N, H, hd, cfg.scale)
        if ev is not None:
            ev[2].record()
        blk.h3_attention_fwd(qkv[:, :I], qkv[:, I:2 * I], qkv[:, 2 * I:], 3 * I, o16, I, N, H, hd, cfg.scale,
                             None, blk.H3_BF16)
        if ev is not None:
            ev[3].record()

    for _ in range(args.warmup):
        one(None)
    torch.cuda.synchronize()
    K_ = args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K_)]
    for i in range(K_):
        one(evs[i])
    torch.cuda.synchronize()
    tq, ta, tb = (sum(e[j].elapsed_time(e[j + 1]) for e in evs) / K_ for j in range(3))
    fl = 4.0 * N * N * hd * H
    qbytes = 3 * N * I * 2 + 3 * N * I + 4 * H * N        # bf16 q, k, v read; codes and q scales written
    kern = {"quantize_qkv_fp8": {"ms": round(tq, 4), "gbs": round(qbytes / (tq * 1e-3) / 1e9, 1)},
            "attention_fp8": {"ms": round(ta, 4), "tflops": round(fl / (ta * 1e-3) / 1e12, 1),
                              "frac_peak": round(fl / (ta * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4)},
            "attention_bf16": {"ms": round(tb, 4), "tflops": round(fl / (tb * 1e-3) / 1e12, 1),
                               "frac_peak": round(fl / (tb * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}}
    total = tq + ta
    result = {"metric": "H3 attention on FP8 (e4m3) operands, quantisation included, TFLOP/s",
              "value": round(fl / (total * 1e-3) / 1e12, 1), "unit": "TFLOP/s", "n_gpus": 1, "steps": K_,
              "warmup": args.warmup, "ms_per_step": round(total, 3), "higher_is_better": True, "scaling": "weak",
              "vs_baseline": None, "dtype": "fp8-e4m3 (fp32 sums, bf16 out)", "data": "synthetic",
              "config": {"workload": f"{cfg.name} attention", "tokens": N, "heads": H, "head_dim": hd},
              "kernels": kern, "speedup_vs_bf16": round(tb / total, 3)}
    print(json.dumps(result), flush=True)


def bench_fp8_stack(args):
    """One sampling step of the 50-block stack with every block on FP8
    operands (H3BlockFP8) and the Euler update; weights drawn on the device
    block by block and quantised as they are made (about 19 GB of e4m3 codes
    stay resident, the bf16 draws do not)."""
    import torch

    from video_audio_diffusion_amd import inputs
    from video_audio_diffusion_amd.block import H3Stack, device_inputs, interleave_gate_up

    scfg = inputs.STACKS[args.config]
    cfg = scfg.block
    log(f"fp8 stack {scfg.name}: {scfg.n_blocks} blocks, {cfg.n_tok} tokens; drawing and quantising weights")
    x = device_inputs(cfg, inputs.make_inputs(cfg, ("x",)))["x"]
    stack = H3Stack(scfg, (interleave_gate_up(device_block_weights(cfg, b), keep_plain=False)
                           for b in range(scfg.n_blocks)), fp8=True)
    torch.cuda.synchronize()
    log(f"weights resident: {torch.cuda.memory_allocated() / 2**30:.1f} GiB allocated")
    n_st = len(stack.block.steps)
    for _ in range(args.warmup):
        stack.forward(x)
    torch.cuda.synchronize()
    K_ = args.steps
    ev = [[[torch.cuda.Event(enable_timing=True) for _ in range(n_st + 1)] for _ in range(scfg.n_blocks)]
          for _ in range(K_)]
    end = [torch.cuda.Event(enable_timing=True) for _ in range(K_)]
    for i in range(K_):
        stack.forward(x, block_events=ev[i])
        end[i].record()
    torch.cuda.synchronize()
    total = ev[0][0][0].elapsed_time(end[-1]) / K_
    per = {st: sum(ev[i][b][j].elapsed_time(ev[i][b][j + 1]) for i in range(K_) for b in range(scfg.n_blocks)) / K_
           for j, st in enumerate(stack.block.steps)}
    result = {"metric": "H3 50-block sampling step, FP8 (e4m3) projections and attention", "unit": "s",
              "value": round(total / 1e3, 4), "n_gpus": 1, "steps": K_, "warmup": args.warmup,
              "ms_per_step": round(total, 2), "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
              "dtype": "fp8-e4m3 (fp32 sums, bf16 activations)", "data": "synthetic",
              "config": {"workload": f"{scfg.name}", "blocks": scfg.n_blocks, "tokens": cfg.n_tok},
              "tokens_per_s": round(cfg.n_tok / (total * 1e-3), 1),
              "kernels_ms_summed_over_blocks": {st: round(ms, 2) for st, ms in per.items()}}
    print(json.dumps(result), flush=True)


def bench_fp8_block(args):
    """The FP8 variant of the block (H3BlockFP8: projections and attention on
    e4m3 operands, quantisation included) at one workload; the fused bf16
    block on the same inputs is timed beside it."""
    import torch

    from video_audio_diffusion_amd import inputs
    from video_audio_diffusion_amd.block import BlockWeights, H3Block, H3BlockFP8, device_inputs, interleave_gate_up

    cfg = inputs.CONFIGS[args.config]
    log(f"fp8 block of {cfg.name}: {cfg.n_tok} tokens; drawing inputs")
    dev = device_inputs(cfg, inputs.make_inputs(cfg))
    w = interleave_gate_up(BlockWeights(dev["w_qkv"], dev["w_o"], dev["w_gu"], dev["w_d"], dev["mod"],
                                        dev["gamma_q"], dev["gamma_k"]))
    blocks = {"fp8": H3BlockFP8(cfg, w), "bf16": H3Block(cfg, w, fused=True)}
    x = dev["x"]
    K_ = args.steps
    times, per = {}, {}
    for name, block in blocks.items():
        for _ in range(args.warmup):
            block.forward(x)
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(block.steps) + 1)] for _ in range(K_)]
        for i in range(K_):
            block.forward(x, events=ev[i])
        torch.cuda.synchronize()
        times[name] = ev[0][0].elapsed_time(ev[-1][-1]) / K_
        per[name] = {st: sum(e[j].elapsed_time(e[j + 1]) for e in ev) / K_ for j, st in enumerate(block.steps)}
        log(f"{name}: {times[name]:.2f} ms per block")
    fl = step_flops(cfg)
    N, D, I, F = cfg.n_tok, cfg.dim, cfg.inner, cfg.ffn
    qbytes = {"quant_a": N * D * 3, "quant_a2": N * D * 3, "quant_o": N * I * 3, "quant_h": N * F * 3,
              "quant_qkv": 3 * N * I * 3}
    sbytes = step_bytes(cfg)
    kern = {}
    for st, ms in per["fp8"].items():
        k = {"ms": round(ms, 4)}
        if st in fl:
            tf = fl[st] / (ms * 1e-3) / 1e12
            k.update(tflops=round(tf, 1), frac_peak=round(tf / PEAK_FP8_TFLOPS, 4))
        elif st in qbytes or st in sbytes:
            gbs = qbytes.get(st, sbytes.get(st, 0)) / (ms * 1e-3) / 1e9
            k.update(gbs=round(gbs, 1), frac_hbm=round(gbs / PEAK_HBM_GBS, 4))
        kern[st] = k
    result = {"metric": "H3 block fwd tokens/s, FP8 (e4m3) projections and attention", "unit": "tokens/s",
              "value": round(cfg.n_tok / (times["fp8"] * 1e-3), 1), "n_gpus": 1, "steps": K_, "warmup": args.warmup,
              "ms_per_step": round(times["fp8"], 3), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
              "dtype": "fp8-e4m3 (fp32 sums, bf16 activations)", "data": "synthetic",
              "config": {"workload": f"{cfg.name} block forward", "tokens": cfg.n_tok},
              "kernels": kern, "bf16_fused_block_ms": round(times["bf16"], 3),
              "speedup_vs_bf16": round(times["bf16"] / times["fp8"], 3)}
    print(json.dumps(result), flush=True)


def shard_config(cfg, P):
    """One GPU's token shard of `cfg` at P GPUs: ceil(N/P) rows at full width,
    laid out as the sequence's first rows (text, audio, whole video frames,
    the rest as a second audio interval)."""
    import dataclasses

    from video_audio_diffusion_amd import inputs

    n = -(-cfg.n_tok // P)
    text, audio = cfg.segments[0], cfg.segments[1]
    video = cfg.segments[-1]
    left = n - text.length - audio.length
    frames = max(0, left // (video.H * video.W))
    rest = left - frames * video.H * video.W
    parts = [("text", text.mod_set, text.length, 1, 1), ("audio", audio.mod_set, audio.length, 1, 1)]
    if frames:
        parts.append(("video", video.mod_set, frames, video.H, video.W))
    if rest:
        parts.append(("audio", audio.mod_set, rest, 1, 1))
    return dataclasses.replace(cfg, name=f"{cfg.name} shard 1/{P}", segments=inputs.pack(parts))


def bench_shard(args):
    """One GPU's share of the block at P GPUs (sequence parallel, one
    all-to-all each way around attention): the row-wise steps of the fused
    block on ceil(N/P) tokens at full width, and attention with 56/P heads
    over all N keys.  The exchange itself is not run (one GPU)."""
    import torch

    from video_audio_diffusion_amd import blk, inputs
    from video_audio_diffusion_amd.block import BlockWeights, H3Block, device_inputs, interleave_gate_up

    cfg = inputs.CONFIGS[args.config]
    P = args.shard
    if cfg.heads % P:
        raise SystemExit(f"{cfg.heads} heads do not split over {P} GPUs")
    scfg = shard_config(cfg, P)
    log(f"one GPU's share at P = {P}: {scfg.n_tok} tokens row-wise, {cfg.heads // P} heads over {cfg.n_tok} keys")
    dev = device_inputs(scfg, inputs.make_inputs(scfg))
    w = interleave_gate_up(BlockWeights(dev["w_qkv"], dev["w_o"], dev["w_gu"], dev["w_d"], dev["mod"],
                                        dev["gamma_q"], dev["gamma_k"]), keep_plain=False)
    block = H3Block(scfg, w, fused=True)
    Hs, d, N = cfg.heads // P, cfg.head_dim, cfg.n_tok
    Is = Hs * d
    g = torch.Generator(device="cuda")
    g.manual_seed(1000 * cfg.index + 960)
    qkv = torch.randn(N, 3 * Is, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    o = torch.empty(N, Is, dtype=torch.bfloat16, device="cuda")

    def attend():
        blk.h3_attention_fwd(qkv[:, :Is], qkv[:, Is:2 * Is], qkv[:, 2 * Is:], 3 * Is, o, Is, N, Hs, d, cfg.scale,
                             None, blk.H3_BF16)

    for _ in range(args.warmup):
        block.forward(dev["x"])
        attend()
    torch.cuda.synchronize()
    K_ = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(block.steps) + 2)] for _ in range(K_)]
    for i in range(K_):
        block.forward(dev["x"], events=ev[i][:-1])
        attend()
        ev[i][-1].record()
    torch.cuda.synchronize()
    steps = {st: sum(e[j].elapsed_time(e[j + 1]) for e in ev) / K_ for j, st in enumerate(block.steps)}
    attn_ms = sum(e[-2].elapsed_time(e[-1]) for e in ev) / K_
    row_ms = sum(ms for st, ms in steps.items() if st != "attention")
    share_ms = row_ms + attn_ms
    fl = 4.0 * N * N * Hs * d
    result = {"metric": f"one GPU's compute share of the block at P = {P} (sequence parallel)", "unit": "ms",
              "value": round(share_ms, 3), "n_gpus": 1, "steps": K_, "warmup": args.warmup,
              "higher_is_better": False, "scaling": "strong", "vs_baseline": None, "dtype": "bf16",
              "data": "synthetic",
              "config": {"workload": f"{cfg.name}, 1/{P} share", "rowwise_tokens": scfg.n_tok,
                         "attention_heads": Hs, "keys": N},
              "rowwise_ms": round(row_ms, 3), "attention_ms": round(attn_ms, 3),
              "attention_tflops": round(fl / (attn_ms * 1e-3) / 1e12, 1),
              "rowwise_steps_ms": {st: round(ms, 4) for st, ms in steps.items() if st != "attention"},
              "note": "the two all-to-alls of q/k/v and o are not run on one GPU"}
    print(json.dumps(result), flush=True)


def bench_adapters(args):
    """The input and output adapters around the backbone at one workload:
    patchify and input projection of every interval into the packed
    sequence, then output projection and unpatchify of the targets."""
    import torch

    from video_audio_diffusion_amd import adapters, inputs
    from video_audio_diffusion_amd.block import device_inputs

    cfg = inputs.CONFIGS[args.config]
    acfg = adapters.AdapterConfig(block=cfg, text_width=64 if cfg.dtype == "f32" else 5120)
    log(f"adapters of {cfg.name}: {cfg.n_tok} tokens; drawing inputs")
    host = inputs.make_adapter_inputs(cfg, acfg.text_width)
    dev = device_inputs(cfg, host)
    w = adapters.AdapterWeights({m: adapters.pad_columns(dev["w_in/" + m], acfg.k_pad(m)) for m in ("text", "video", "audio")},
                                {m: dev["w_out/" + m] for m in ("video", "audio")})
    ad = adapters.H3Adapters(acfg, w)
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    feats = {s.kind: dev["feat/" + s.kind] for s in cfg.segments}
    x = torch.empty(cfg.n_tok, cfg.dim, dtype=tdt, device="cuda")
    shapes = inputs.adapter_shapes(cfg, acfg.text_width)
    lat_out = {k: torch.empty(shapes["feat/" + k], dtype=tdt, device="cuda") for k in adapters.TARGET_KINDS}

    def one(marks):
        mark = (lambda name: marks.append((name, torch.cuda.Event(enable_timing=True)))) if marks is not None else None
        rec = (lambda name: (mark(name), marks[-1][1].record())) if marks is not None else None
        ad.pack(feats, x, mark=rec)
        ad.unpack(x, lat_out, mark=rec)
        if marks is not None:
            rec("end")

    for i in range(args.warmup):
        one(None)
    torch.cuda.synchronize()
    K = args.steps
    runs = [[] for _ in range(K)]
    for i in range(K):
        one(runs[i])
    torch.cuda.synchronize()
    total_ms = runs[0][0][1].elapsed_time(runs[-1][-1][1]) / K
    e = 2 if cfg.dtype == "bf16" else 4
    names = [n for n, _ in runs[0][:-1]]
    per = {n: sum(r[j][1].elapsed_time(r[j + 1][1]) for r in runs) / K for j, n in enumerate(names)}
    kern = {}
    for s in cfg.segments:
        m = inputs.modality(s.kind)
        kp, P = acfg.k_pad(m), acfg.feature_width(m)
        if ("patchify_" + s.kind) in per:
            by = s.length * P * e + s.length * kp * e
            kern["patchify_" + s.kind] = {"ms": round(per["patchify_" + s.kind], 4),
                                          "gbs": round(by / (per["patchify_" + s.kind] * 1e-3) / 1e9, 1)}
        fl = 2 * s.length * cfg.dim * kp
        kern["gemm_in_" + s.kind] = {"ms": round(per["gemm_in_" + s.kind], 4),
                                     "tflops": round(fl / (per["gemm_in_" + s.kind] * 1e-3) / 1e12, 1)}
        if s.kind in adapters.TARGET_KINDS:
            fl = 2 * s.length * cfg.dim * P
            kern["gemm_out_" + s.kind] = {"ms": round(per["gemm_out_" + s.kind], 4),
                                          "tflops": round(fl / (per["gemm_out_" + s.kind] * 1e-3) / 1e12, 1)}
            if ("unpatchify_" + s.kind) in per:
                by = 2 * s.length * P * e
                kern["unpatchify_" + s.kind] = {"ms": round(per["unpatchify_" + s.kind], 4),
                                                "gbs": round(by / (per["unpatchify_" + s.kind] * 1e-3) / 1e9, 1)}
    result = {"metric": "H3 I/O adapters (patchify, input/output projections, unpatchify) tokens/s",
              "value": round(cfg.n_tok / (total_ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": K,
              "warmup": args.warmup, "ms_per_step": round(total_ms, 4), "higher_is_better": True,
              "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
              "config": {"workload": f"{cfg.name} adapters", "tokens": cfg.n_tok, "hidden": cfg.dim,
                         "text_width": acfg.text_width, "video_patch": list(acfg.video_patch),
                         "segments": [f"{s.kind} {s.T}x{s.H}x{s.W}" for s in cfg.segments]},
              "kernels": kern}
    print(json.dumps(result), flush=True)


def copy_calibration(mib, reps):
    """A plain device-to-device copy of `mib` MiB (torch's copy kernel), run
    `reps` times: the known-size transfer that scales rocprofv3's FETCH_SIZE
    and WRITE_SIZE counters to bytes.  Prints one JSON line with the bytes
    moved per launch and the measured copy rate."""
    import torch

    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record()
    for i in range(reps):
        dst.copy_(src)
        ev[i + 1].record()
    torch.cuda.synchronize()
    ms = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(reps))
    med = ms[len(ms) // 2]
    print(json.dumps({"metric": "device-to-device copy (HBM counter calibration)", "bytes_read_per_launch": n,
                      "bytes_written_per_launch": n, "launches": reps + 1, "median_ms": round(med, 4),
                      "gbs_read_plus_write": round(2 * n / (med * 1e-3) / 1e9, 1)}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=3,
                    help="workload index: 1-4 one block; 5 the 50-block stack and one Euler step")
    ap.add_argument("--cpu-seconds", type=float, default=20.0, help="oracle sample budget; 0 skips it")
    ap.add_argument("--unfused", action="store_true", help="time the eleven-call block (no fused epilogues)")
    ap.add_argument("--fp8", action="store_true",
                    help="time the four projections as FP8 (e4m3) GEMMs with row-wise activation quantisation")
    ap.add_argument("--shard", type=int, default=0,
                    help="time one GPU's share of the block at this many GPUs (sequence parallel)")
    ap.add_argument("--fp8-block", action="store_true",
                    help="time the FP8 block (projections and attention on e4m3) beside the fused bf16 block")
    ap.add_argument("--fp8-attn", action="store_true",
                    help="time the attention on FP8 operands (quantise + attend) beside the bf16 kernel")
    ap.add_argument("--io", action="store_true",
                    help="time the input/output adapters (patchify, projections, unpatchify) of the workload")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain MIB-MiB device copy (scale for the HBM traffic counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build runs the block on one GPU only; there is no multi-GPU path "
              "(how it would shard is a design note), so --gpus must be 1", file=sys.stderr)
        sys.exit(2)

    import torch

    from video_audio_diffusion_amd import blk, inputs
    from video_audio_diffusion_amd.block import BlockWeights, H3Block, H3Stack, device_inputs, interleave_gate_up

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, max(args.steps, 1))
        return
    blk.load()
    if args.io:
        bench_adapters(args)
        return
    if args.shard:
        bench_shard(args)
        return
    if args.fp8_block:
        if args.config in inputs.STACKS:
            bench_fp8_stack(args)
        else:
            bench_fp8_block(args)
        return
    if args.fp8_attn:
        bench_fp8_attention(args)
        return
    if args.fp8:
        bench_fp8(args)
        return
    stack = None
    if args.config in inputs.STACKS:
        scfg = inputs.STACKS[args.config]
        cfg = scfg.block
        log(f"workload {scfg.name}: {scfg.n_blocks} blocks, {cfg.n_tok} tokens; drawing weights on device")
        host = inputs.make_inputs(cfg, ("x",))
        dev = device_inputs(cfg, host)
        prep = (lambda w: w) if args.unfused else (lambda w: interleave_gate_up(w, keep_plain=False))
        stack = H3Stack(scfg, [prep(device_block_weights(cfg, b)) for b in range(scfg.n_blocks)],
                        fused=not args.unfused)
        log("weights resident on device")
        n_blk = scfg.n_blocks
    else:
        cfg = inputs.CONFIGS[args.config]
        log(f"workload {cfg.name}: {cfg.n_tok} tokens; drawing inputs")
        host = inputs.make_inputs(cfg)
        dev = device_inputs(cfg, host)
        log("inputs resident on device")
        w = BlockWeights(dev["w_qkv"], dev["w_o"], dev["w_gu"], dev["w_d"], dev["mod"], dev["gamma_q"],
                         dev["gamma_k"])
        if not args.unfused:
            w = interleave_gate_up(w)
        block = H3Block(cfg, w, fused=not args.unfused)
        n_blk = 1
    x = dev["x"]
    steps = (stack.block if stack is not None else block).steps

    def one_step(events):
        """One timed pass: `events` holds len(steps) + 1 events per block and
        one more recorded after the pass."""
        if stack is None:
            block.forward(x, events=events[0])
        else:
            stack.forward(x, block_events=events)
        events[-1][0].record()

    new_events = lambda: [[torch.cuda.Event(enable_timing=True) for _ in range(len(steps) + 1)]
                          for _ in range(n_blk)] + \
        [[torch.cuda.Event(enable_timing=True)]]
    for i in range(args.warmup):
        one_step(new_events())
        torch.cuda.synchronize()
        log(f"warmup {i + 1}/{args.warmup} done")

    K = args.steps
    ev = [new_events() for _ in range(K)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for i in range(K):
        one_step(ev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    total_ms = ev[0][0][0].elapsed_time(ev[K - 1][-1][0])
    step_ms = sorted(ev[i][0][0].elapsed_time(ev[i][-1][0]) for i in range(K))
    ms_step = step_ms[K // 2] if K % 2 else 0.5 * (step_ms[K // 2 - 1] + step_ms[K // 2])
    log(f"timed {K} steps: median {ms_step:.2f} ms/step, mean {total_ms / K:.2f} "
        f"(host wall {wall * 1e3 / K:.2f} ms/step)")

    # per-kernel time of one pass (summed over the blocks of a stack)
    per = {name: sum(ev[i][b][j].elapsed_time(ev[i][b][j + 1]) for i in range(K) for b in range(n_blk)) / K
           for j, name in enumerate(steps)}
    flops = {k: v * n_blk for k, v in step_flops(cfg).items()}
    byts = {k: v * n_blk for k, v in step_bytes(cfg).items()}
    peak_mm = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
    kernels = {}
    for name, ms in per.items():
        k = {"ms": round(ms, 4)}
        if name in flops:
            tf = flops[name] / (ms * 1e-3) / 1e12
            k.update(tflops=round(tf, 1), frac_peak=round(tf / peak_mm, 4))
        else:
            gbs = byts[name] / (ms * 1e-3) / 1e9
            k.update(gbs=round(gbs, 1), frac_hbm=round(gbs / PEAK_HBM_GBS, 4))
        kernels[name] = k
    attn_tf = flops["attention"] / (per["attention"] * 1e-3) / 1e12
    tokens_s = cfg.n_tok / (ms_step * 1e-3)

    result = {
        "metric": METRIC, "value": round(tokens_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": (f"{cfg.name} block forward" if stack is None else
                                f"{inputs.STACKS[args.config].name}: {n_blk} blocks and one Euler step"),
                   "blocks": n_blk, "tokens": cfg.n_tok,
                   "segments": [f"{s.kind} {s.T}x{s.H}x{s.W}" for s in cfg.segments],
                   "hidden": cfg.dim, "heads": cfg.heads, "head_dim": cfg.head_dim, "ffn": cfg.ffn,
                   "rope_split": list(cfg.rope_split), "fused_epilogues": not args.unfused,
                   "global_batch": 1, "seq_len": cfg.n_tok,
                   "parallelism": "none (1 GPU)"},
        "step_ms": {"median": round(ms_step, 3), "mean": round(total_ms / K, 3), "min": round(step_ms[0], 3),
                    "max": round(step_ms[-1], 3), "of_steps": K},
        "attention_tflops": round(attn_tf, 1), "attention_pct_peak": round(100 * attn_tf / peak_mm, 2),
        "kernels": kernels,
        "roofline": {"kernel": "attention", "bound": "mfma", "achieved": round(attn_tf, 1), "peak": peak_mm,
                     "unit": "TFLOP/s", "frac": round(attn_tf / peak_mm, 4),
                     "traffic": measured_traffic("attention"),
                     "algorithmic_per_launch": f"{flops['attention'] / n_blk:.4e} flop (4*N^2*heads*head_dim)"},
        "cpu_baseline": None,
    }
    if args.cpu_seconds > 0 and stack is None:
        log("timing the fp64 oracle on host cores")
        result["cpu_baseline"] = cpu_baseline(cfg, host, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
