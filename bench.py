"""Benchmark of the DFlash drafter hot path on one MI355X.

One step is one drafting iteration of the whole path on the Qwen3-8B-shaped
drafter at a 2048-token context (batch 1, block gamma = 16, 5 layers, bf16
weights, bf16 H_t and KV cache):
  draft forward -> LM-head argmax -> synthetic target tokens (p = 0.8 match)
  -> greedy accept -> append the next 16 target rows (fuse + inject).
The context (fuse + inject of 2048 rows) is ingested once before timing; every
8 iterations the cache length is reset to 2048 (rows below it are never
written), so the timed loop cycles through 8 iteration shapes.

Prints one JSON line.  ``value`` is drafted blocks per second (batch x steps /
time).  ``roofline`` covers the kernel with the most time in a step (per-launch
algorithmic bytes over its launches' HIP-event durations on the library's
stream); ``roofline_lm_head`` the LM head.  ``cpu_baseline`` times the CPU
oracle on a bounded sample (whole iterations).  Further legs: ``sampling``
(the same step decoded at temperature 1 with lossless verification),
``ragged`` (block lengths per sequence), ``blocks`` (anchored blocks, the
training-style mask), ``long_context`` (32768-token context, both cache
types), ``gamma_sweep`` (8-layer drafter, blocks of 8/16/32 at a fixed
cache), ``loops`` (blocks/s of the tiny, long-context, 16-sequence and 8-layer
workloads over their 8-iteration loops with appends) and ``speculative``
(greedy speculative decoding with a 36-layer synthetic Qwen3-8B-shaped target
verifying each block).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "drafted gamma=16 blocks/sec + draft fwd us at 1 GPU; % HBM BW / % MFMA peak"

# HBM bytes per launch of the roofline kernels from two rocprofv3 counter passes
# over this script (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch), each scaled
# by what the same counter reads for the 256 MiB device copy at the end of
# main().  Valid only for the recorded workload and cache and only while the
# GEMM sources hash to ``src``; otherwise the traffic is reported as null.
KERNEL_COUNTERS = {
    # mean KiB per dispatch over the bench's headline run (the summaries under
    # profiles/ give the commands); scales from the copy above
    "short_rk": {"src": "f993241bc7f4c746", "workload": "qwen3_8b_shape_n2048", "cache": "bf16",
                 "fetch_kib": 30380.0, "write_kib": 1536.0, "fetch_scale": 1.9998, "write_scale": 1.0},
    "lm_head": {"src": "f993241bc7f4c746", "workload": "qwen3_8b_shape_n2048", "cache": "bf16",
                "fetch_kib": 608779.2, "write_kib": 52.0, "fetch_scale": 1.9998, "write_scale": 1.0},
}
GEMM_SOURCES = ("csrc/gemm.hip", "csrc/common.h", "csrc/launch.h")


def gemm_sources_hash():
    """Hash of the GEMM sources' code: comments and whitespace are dropped, so
    only a change of the code itself invalidates the recorded counters."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(ROOT, "block_diffusion_drafter_ctx_amd", f), encoding="utf-8") as fh:
            code = fh.read()
        code = re.sub(r"/\*.*?\*/", " ", code, flags=re.S)   # block comments
        code = re.sub(r"//[^\n]*", " ", code)                   # line comments
        h.update(" ".join(code.split()).encode())
    return h.hexdigest()[:16]


def kernel_traffic(which, workload, cache):
    """HBM bytes per launch of a kernel from the recorded rocprofv3 counters
    (null unless they were taken on the current GEMM sources, workload and cache)."""
    c = KERNEL_COUNTERS.get(which)
    if c is None or gemm_sources_hash() != c["src"] or workload != c["workload"] or cache != c["cache"]:
        return None
    return int(round((c["fetch_kib"] * c["fetch_scale"] + c["write_kib"] * c["write_scale"]) * 1024))


# Kernel families of one headline step: (name, per-kernel roles it runs, which of
# them it runs only with an fp32 cache, the key of its recorded counters).  The
# short-weight register-K GEMM takes the Q/K/V, O and down projections and, with
# an fp32 H_t, the 16-row inject.
FAMILIES = (
    ("gemm_rk_kernel<KS, RK_PART, 1, A_F32_SPLIT, 8> (short weights: Q/K/V, O and down projections of every layer, "
     "and the 16-row K/V inject with an fp32 H_t; 8 waves of KS k-steps, KS = 4 (6 for the down projection), 16 "
     "fp32 activation rows as bf16 hi + lo in registers, split-K partials reduced by the next kernel)",
     ("qkv", "o_proj", "down", "inject_append"), ("inject_append",), "short_rk"),
    ("gemm_rk_kernel<8, RK_SWIGLU> (FFN gate/up with SwiGLU in the epilogue)", ("gate_up",), (), None),
    ("attention (split over key ranges + log-sum-exp combine)", ("attention",), (), None),
)


def dominant_roofline(cfg, per_kernel, lm_bytes, lm_us, workload):
    """The roofline entry of the kernel with the most time per step: per-launch
    algorithmic bytes and duration averaged over its launches in a step."""
    import numpy as np  # noqa: F401
    from block_diffusion_drafter_ctx_amd import roofline as RF
    calls = {"qkv": cfg.L, "o_proj": cfg.L, "gate_up": cfg.L, "down": cfg.L, "attention": cfg.L, "inject_append": 1,
             "fuse_append": 1}
    cands = [("gemm_rk_kernel<16, RK_TOP2, 1, A_F32_SPLIT, 8> (LM head with the top-2 epilogue)", lm_bytes, lm_us, 1, "lm_head")]
    for name, roles, f32_only, key in FAMILIES:
        rs = [r for r in roles if r in per_kernel and not (r in f32_only and cfg.cache_dtype != "f32")]
        n = sum(calls[r] for r in rs)
        if n == 0:
            continue
        tb = sum(per_kernel[r]["bytes"] * calls[r] for r in rs)
        tu = sum(per_kernel[r]["us"] * calls[r] for r in rs)
        cands.append((name, tb / n, tu / n, n, key))
    name, b, us, n, key = max(cands, key=lambda c: c[2] * c[3])
    gbs = b / (us * 1e-6) / 1e9
    return {"kernel": name + f"; {n} launch(es) per step, the largest kernel time of a step; HIP events recorded by each "
                             f"launch's own dispatch on the library stream (dflash_profile_events)",
            "bound": "hbm", "achieved": round(gbs, 1), "peak": RF.HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / RF.HBM_PEAK_GBS, 4),
            "traffic": kernel_traffic(key, workload, cfg.cache_dtype) if key else None,
            "bytes_per_launch": int(b), "us_per_launch": round(us, 2), "launches_per_step": n,
            "us_per_step": round(us * n, 1)}


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="qwen3_8b_shape_n2048", help="a workload of dflash_inputs.WORKLOADS")
    ap.add_argument("--fwd-reps", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="run the CPU oracle for about this long (whole iterations)")
    ap.add_argument("--cache", choices=["f32", "bf16"], default="bf16",
                    help="storage type of H_t and the KV cache (bf16: the method's own; f32: for comparison)")
    ap.add_argument("--temperature", type=float, default=1.0, help="temperature of the sampled-decoding leg")
    ap.add_argument("--no-sampling", action="store_true", help="skip the sampled-decoding leg")
    ap.add_argument("--no-ragged", action="store_true", help="skip the per-sequence block-length leg")
    ap.add_argument("--no-blocks", action="store_true", help="skip the anchored-blocks (training-mask) leg")
    ap.add_argument("--no-gamma-sweep", action="store_true", help="skip the block-length sweep on the 8-layer drafter")
    ap.add_argument("--no-long-context", action="store_true", help="skip the 32768-token context leg")
    ap.add_argument("--no-speculative", action="store_true",
                    help="skip the speculative-decoding leg with a 36-layer synthetic target")
    ap.add_argument("--no-loops", action="store_true",
                    help="skip the drafting loops of the tiny, long-context, 16-sequence and 8-layer workloads")
    ap.add_argument("--loops", default="tiny_f32,long_ctx_n32768,batch16_ragged,deep8_b4_n8192",
                    help="comma-separated workloads whose drafting loops to run")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the library runs the drafting "
              "path on one GPU; sharding it over several is not implemented", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from block_diffusion_drafter_ctx_amd import binding as B
    from block_diffusion_drafter_ctx_amd import roofline as RF
    from block_diffusion_drafter_ctx_amd.runtime import DeviceDrafter, upload
    from dflash_inputs import WORKLOADS, Inputs, shrink

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    B.load()
    cfg = shrink(WORKLOADS[args.workload], cache_dtype=args.cache)
    gamma = cfg.gamma
    n = gamma - 1
    Bn = cfg.B
    N = cfg.n_ctx_total
    CYCLE = cfg.iters
    dev = "cuda"
    t0 = time.time()
    inp = Inputs(cfg)
    dr = DeviceDrafter(cfg, inp, dev)
    log(f"weights uploaded in {time.time() - t0:.1f}s ({B.version()}, {torch.cuda.get_device_name(0)})")

    cap = max(cfg.ctx) + CYCLE * cfg.append_rows + max(gamma, cfg.append_rows)
    cap = (cap + 31) // 32 * 32
    cache = dr.cache(Bn, cap)
    dr.ensure_workspace(Bn, gamma, max(N, Bn * cfg.append_rows))
    stream = torch.cuda.current_stream()

    # ---- context ingest, once (timed separately)
    h_ctx = [upload(h, cfg, dev) for h in inp.ctx_states()]
    H_t = dr.context_buffer(N)
    dr.fuse(h_ctx, N, H_t)
    dr.inject(H_t, list(cfg.ctx), cache)     # warm
    torch.cuda.synchronize()
    ctx_reps = 3
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def ingest():
        cache.set_lens([0] * Bn, mirror=False)   # host lengths only: the inject rewrites the mirror
        dr.fuse(h_ctx, N, H_t)
        dr.inject(H_t, list(cfg.ctx), cache)

    ingest()          # queued ahead of the start event: the host's planning of the timed reps overlaps it
    e0.record()
    for _ in range(ctx_reps):
        ingest()
    e1.record()
    torch.cuda.synchronize()
    context_us = e0.elapsed_time(e1) * 1e3 / ctx_reps
    base_lens = cache.len_list()
    del h_ctx

    # ---- per-iteration inputs, resident on the device
    # synthetic verify: target = (draft + shift) mod V with shift = 0 where the
    # position matches (p = 0.8), else r ~ U{1..V-1}; the bonus column is fixed
    app = []
    for it in range(CYCLE):
        st = [upload(h, cfg, dev) for h in inp.append_states(it)]
        m, r, bonus = inp.verify_draws(it, gamma)
        shift = np.where(m, 0, r).astype(np.int32)
        tgt = np.zeros((Bn, gamma), dtype=np.int32)
        tgt[:, n] = bonus
        app.append(dict(states=st, shift=torch.from_numpy(shift).to(dev), target=torch.from_numpy(tgt).to(dev)))
    H_app = dr.context_buffer(Bn * cfg.append_rows)
    tokens = torch.from_numpy(inp.block_tokens(gamma)).to(dev)
    h_final = torch.empty(Bn, gamma, cfg.D, dtype=torch.float32, device=dev)
    draft = torch.empty(Bn, n, dtype=torch.int32, device=dev)
    tau = torch.empty(Bn, dtype=torch.int32, device=dev)
    # with one sequence the next anchor is written straight into block row 0
    nxt = tokens[:, 0] if Bn == 1 else torch.empty(Bn, dtype=torch.int32, device=dev)
    tmp = torch.empty(Bn, n, dtype=torch.int32, device=dev)
    V = cfg.V

    def make_events(n):
        """n (start, stop) event pairs, each created on the device up front (the
        library records them on its stream through the profiling hook)."""
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a, b in pairs:
            a.record(stream)
            b.record(stream)
        torch.cuda.synchronize()
        return pairs

    def hook(role, pairs):
        return B.profile_events(role, [a.cuda_event for a, _ in pairs], [b.cuda_event for _, b in pairs])

    def step(i):
        it = i % CYCLE
        if it == 0:
            cache.set_lens(base_lens, mirror=False)   # host lengths only: the inject rewrites the mirror
        dr.draft(cache, tokens, None, gamma, h_final)
        dr.argmax_accept(B.ARGMAX, h_final, Bn, gamma, draft)
        d = app[it]
        target = d["target"]
        torch.add(draft, d["shift"], out=tmp)
        torch.remainder(tmp, V, out=target[:, :n])
        dr.argmax_accept(B.ACCEPT, None, Bn, gamma, draft, target=target, tau=tau, nxt=nxt)
        if Bn > 1:
            tokens[:, 0].copy_(nxt)
        dr.fuse(d["states"], Bn * cfg.append_rows, H_app)
        dr.inject(H_app, [cfg.append_rows] * Bn, cache)

    for i in range(args.warmup):
        step(i)
    lm_ev = make_events(args.steps)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record(stream)
    hook(B.PROF_LM_HEAD, lm_ev)          # the LM-head kernel of every timed step
    for i in range(args.steps):
        step(args.warmup + i)
    s1.record(stream)
    host_enqueue = time.perf_counter() - t_start   # host time to queue the steps (no wait)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    n_lm = hook(B.PROF_NONE, [])
    assert n_lm == args.steps, (n_lm, args.steps)
    gpu_ms = s0.elapsed_time(s1)
    ms_per_step = max(gpu_ms, wall * 1e3) / args.steps
    blocks_per_s = Bn * args.steps / (ms_per_step * args.steps / 1e3)
    lm_us = float(np.mean([a.elapsed_time(b) for a, b in lm_ev])) * 1e3
    taus = tau.cpu().numpy()

    # ---- every other kernel role over one cycle of steps (outside the timed region)
    # algorithmic bytes count the method's own K/V type (bf16 for a bf16 drafter)
    # whatever the cache holds: an fp32 cache's extra bytes are overhead
    es0 = 2 if cfg.dtype == "bf16" else 4
    cs0 = es0
    M = Bn * gamma
    T_app = Bn * cfg.append_rows
    nqkv = (cfg.Hq + 2 * cfg.Hkv) * cfg.d
    mean_keys = sum(cfg.ctx) / Bn + cfg.append_rows * (CYCLE - 1) / 2 + gamma
    roles = {
        "qkv": (B.PROF_QKV, cfg.L, RF.gemm_bytes(nqkv, cfg.D, M, es0)),
        "o_proj": (B.PROF_O, cfg.L, RF.gemm_bytes(cfg.D, cfg.Hq * cfg.d, M, es0)),
        "gate_up": (B.PROF_GATEUP, cfg.L, RF.gemm_bytes(2 * cfg.F, cfg.D, M, es0)),
        "down": (B.PROF_DOWN, cfg.L, RF.gemm_bytes(cfg.D, cfg.F, M, es0)),
        "attention": (B.PROF_ATTENTION, cfg.L,
                      int(Bn * mean_keys * 2 * cfg.Hkv * cfg.d * cs0 + 2 * M * cfg.Hq * cfg.d * 4)),
        "fuse_append": (B.PROF_FUSE, 1, RF.fuse_bytes(T_app, cfg.D, cfg.n_tgt, es0, cs0)),
        "inject_append": (B.PROF_INJECT, 1, RF.inject_bytes(T_app, cfg.D, cfg.L, cfg.Hkv, cfg.d, es0, cs0)),
    }
    per_kernel = {}
    for name, (role, per_step, nbytes) in roles.items():
        pairs = make_events(per_step * CYCLE)
        hook(role, pairs)
        for i in range(CYCLE):
            step(i)
        torch.cuda.synchronize()
        got = hook(B.PROF_NONE, [])
        us = float(np.mean([a.elapsed_time(b) for a, b in pairs[:got]])) * 1e3
        per_kernel[name] = {"us": round(us, 2), "bytes": int(nbytes), "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
                            "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / RF.HBM_PEAK_GBS, 4)}

    # ---- draft forward us at a fixed cache length (draft forward + LM-head argmax)
    cache.set_lens(base_lens)
    fwd = []
    for rep in range(5 + args.fwd_reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        dr.draft(cache, tokens, None, gamma, h_final)
        dr.argmax_accept(B.ARGMAX, h_final, Bn, gamma, draft)
        b.record(stream)
        if rep >= 5:
            fwd.append((a, b))
    torch.cuda.synchronize()
    draft_fwd_us = float(np.median([a.elapsed_time(b) for a, b in fwd])) * 1e3

    # ---- roofline of the dominant kernel: LM head GEMM + argmax
    es = RF.elem_bytes(cfg.dtype)
    cs = es                                   # the method's K/V bytes (see above)
    lm_bytes = RF.lm_head_bytes(V, cfg.D, Bn * n, es)
    lm_gbs = lm_bytes / (lm_us * 1e-6) / 1e9
    step_bytes = (RF.draft_forward_bytes(cfg.D, cfg.L, cfg.Hq, cfg.Hkv, cfg.d, cfg.F, V, Bn, gamma,
                                         [x + cfg.append_rows * (CYCLE - 1) / 2 for x in cfg.ctx], es, cs)
                  + RF.fuse_bytes(Bn * cfg.append_rows, cfg.D, cfg.n_tgt, es, cs)
                  + RF.inject_bytes(Bn * cfg.append_rows, cfg.D, cfg.L, cfg.Hkv, cfg.d, es, cs))
    fwd_bytes = RF.draft_forward_bytes(cfg.D, cfg.L, cfg.Hq, cfg.Hkv, cfg.d, cfg.F, V, Bn, gamma, list(cfg.ctx),
                                       es, cs)
    ctx_flops = RF.fuse_flops(N, cfg.D, cfg.n_tgt) + RF.inject_flops(N, cfg.D, cfg.L, cfg.Hkv, cfg.d)
    log(f"step {ms_per_step * 1e3:.1f} us, draft fwd {draft_fwd_us:.1f} us, LM head {lm_us:.1f} us "
        f"({lm_gbs:.0f} GB/s), context {context_us:.0f} us, last tau {taus.tolist()}, "
        f"host enqueue {host_enqueue * 1e6 / args.steps:.1f} us per step")

    out = {
        "metric": METRIC,
        "value": round(blocks_per_s, 2),
        "unit": "blocks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "host_enqueue_us_per_step": round(host_enqueue * 1e6 / args.steps, 1),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) target states, N(0,0.02) random-init weights)",
        "config": {
            "workload": (f"{cfg.name}: DFlash drafter, batch {Bn}, context {N}, gamma {gamma} "
                         f"(1 anchor + {n} masks), L={cfg.L}, D={cfg.D}, {cfg.Hq}q/{cfg.Hkv}kv x {cfg.d}, "
                         f"FFN {cfg.F}, V={V}; step = draft forward + LM-head argmax + accept + "
                         f"append {cfg.append_rows} rows (fuse + inject)"),
            "global_batch": Bn, "seq_len": N, "gamma": gamma, "parallelism": "single GPU",
            "weights": cfg.dtype, "cache": cfg.cache_dtype,
        },
        "draft_fwd_us": round(draft_fwd_us, 2),
        "draft_fwd_hbm_frac": round(fwd_bytes / (draft_fwd_us * 1e-6) / 1e9 / RF.HBM_PEAK_GBS, 4),
        "step_hbm_frac": round(step_bytes / (ms_per_step * 1e-3) / 1e9 / RF.HBM_PEAK_GBS, 4),
        "context_us": round(context_us, 1),
        "context_mfma_frac": round(ctx_flops / (context_us * 1e-6) / 1e12 / RF.MFMA_BF16_TFLOPS, 4),
        "per_kernel": per_kernel,
        "roofline": dominant_roofline(cfg, per_kernel, lm_bytes, lm_us, args.workload),
        "roofline_lm_head": {
            "kernel": "gemm_rk_kernel<16, RK_TOP2, 1, A_F32_SPLIT, 8> (LM head: 151936 x 4096 bf16 streamed once "
                      "against the 15 mask rows held in registers of 8 waves as bf16 hi + lo, logits reduced in-kernel to a top-2 per "
                      "workgroup), one launch per step, HIP events recorded by that launch's dispatch on the library "
                      "stream by dflash_profile_events",
            "bound": "hbm", "achieved": round(lm_gbs, 1), "peak": RF.HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(lm_gbs / RF.HBM_PEAK_GBS, 4), "traffic": kernel_traffic("lm_head", args.workload,
                                                                                   cfg.cache_dtype),
            "bytes_per_launch": lm_bytes, "us_per_launch": round(lm_us, 2),
        },
    }

    if not args.no_sampling:
        out["sampling"] = sampled_leg(args, cfg, inp, dr, cache, base_lens, tokens, h_final, draft, tau, nxt, app,
                                      H_app, make_events, hook, ms_per_step)
    if not args.no_ragged and cfg.dtype == "bf16":
        out["ragged"] = ragged_leg(cfg, dr)
    if not args.no_blocks and cfg.dtype == "bf16":
        out["blocks"] = blocks_leg(cfg, dr)
    if not args.no_long_context and cfg.dtype == "bf16":
        out["long_context"] = long_context_leg(cfg, dr)
        other = "bf16" if cfg.cache_dtype == "f32" else "f32"
        out["long_context_" + other + "_cache"] = long_context_leg(shrink(cfg, cache_dtype=other),
                                                                   dr.with_cache_dtype(other))
    if not args.no_gamma_sweep and cfg.dtype == "bf16":
        del dr, cache
        torch.cuda.empty_cache()
        out["gamma_sweep"] = gamma_sweep_leg()
    if not args.no_loops:
        # the other workloads' drafting loops (blocks/s over 8 iterations with appends)
        out["loops"] = {}
        for wl in args.loops.split(","):
            out["loops"][wl] = workload_loop_leg(wl, args.cache)
    if not args.no_speculative:
        out["speculative"] = speculative_leg(args.cache)

    # A plain device copy of a known size: the reference that scales rocprofv3's
    # FETCH_SIZE / WRITE_SIZE counters into bytes (256 MiB read + 256 MiB written).
    src = torch.empty(128 << 20, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst

    if not args.no_cpu_baseline:
        greedy_cpu, sampled_cpu, ragged_cpu, blocks_cpu, long_cpu = cpu_baseline(
            cfg, inp, args.cpu_seconds, None if args.no_sampling else args.temperature, "ragged" in out,
            "blocks" in out, "long_context" in out)
        out["cpu_baseline"] = greedy_cpu
        if sampled_cpu is not None:
            out["sampling"]["cpu_baseline"] = sampled_cpu
        if ragged_cpu is not None:
            out["ragged"]["cpu_baseline"] = ragged_cpu
        if blocks_cpu is not None:
            out["blocks"]["cpu_baseline"] = blocks_cpu
        if long_cpu is not None:
            out["long_context"]["cpu_baseline"] = long_cpu
        if "tiny_f32" in out.get("loops", {}):
            out["loops"]["tiny_f32"]["cpu_baseline"] = cpu_tiny_baseline()
    print(json.dumps(out), flush=True)


def sampled_leg(args, cfg, inp, dr, cache, base_lens, tokens, h_final, draft, tau, nxt, app, H_app, make_events,
                hook, greedy_ms):
    """The drafting step decoded at temperature T: timed like the greedy step,
    then each sampling kernel role over one cycle (outside the timed region)."""
    import numpy as np
    import torch

    from block_diffusion_drafter_ctx_amd import binding as B
    from block_diffusion_drafter_ctx_amd import roofline as RF
    from dflash_inputs import Inputs, shrink

    def Inputs16(c, b):
        return Inputs(shrink(c, B=b))

    T = args.temperature
    gamma, n, Bn, V, CYCLE = cfg.gamma, cfg.gamma - 1, cfg.B, cfg.V, cfg.iters
    dev = "cuda"
    stream = torch.cuda.current_stream()
    ug, ua, ur = inp.sample_uniforms(0, gamma)
    u_draw = torch.from_numpy(ug).to(dev)
    u_acc = torch.from_numpy(ua).to(dev)
    u_emit = torch.from_numpy(ur).to(dev)
    noise = torch.from_numpy(inp.target_noise(0, gamma)).to(dev)
    z = torch.empty(Bn, n, V, dtype=torch.float32, device=dev)
    lse = torch.empty(Bn, n, dtype=torch.float32, device=dev)
    target = torch.empty(Bn, gamma, V, dtype=torch.float32, device=dev)
    target[:, n].copy_(noise[:, n])
    noise_d = noise[:, :n]

    def sstep(i):
        it = i % CYCLE
        if it == 0:
            cache.set_lens(base_lens, mirror=False)   # host lengths only: the inject rewrites the mirror
        dr.draft(cache, tokens, None, gamma, h_final)
        dr.sample_drafts(h_final, Bn, gamma, T, u_draw, draft, z, lse)
        torch.add(z, noise_d, alpha=0.5, out=target[:, :n])       # stands in for the target's verify forward
        dr.sample_accept(Bn, gamma, T, draft, z, target, u_acc, u_emit, tau, nxt, draft_lse=lse)
        if Bn > 1:
            tokens[:, 0].copy_(nxt)
        d = app[it]
        dr.fuse(d["states"], Bn * cfg.append_rows, H_app)
        dr.inject(H_app, [cfg.append_rows] * Bn, cache)

    for i in range(args.warmup):
        sstep(i)
    lm_ev = make_events(args.steps)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record(stream)
    hook(B.PROF_LM_HEAD, lm_ev)
    for i in range(args.steps):
        sstep(args.warmup + i)
    s1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    assert hook(B.PROF_NONE, []) == args.steps
    ms = max(s0.elapsed_time(s1), wall * 1e3) / args.steps
    lm_us = float(np.mean([a.elapsed_time(b) for a, b in lm_ev])) * 1e3

    taus = []
    per = {}
    for name, role, nbytes in (("row_stats", B.PROF_ROW_STATS, RF.row_stats_bytes(Bn * (n + 1), V)),
                               ("verify", B.PROF_VERIFY, None)):
        pairs = make_events(CYCLE)
        hook(role, pairs)
        for i in range(CYCLE):
            sstep(i)
            if role == B.PROF_ROW_STATS:
                torch.cuda.synchronize()
                taus.extend(tau.cpu().tolist())
        torch.cuda.synchronize()
        got = hook(B.PROF_NONE, [])
        us = float(np.mean([a.elapsed_time(b) for a, b in pairs[:got]])) * 1e3
        per[name] = {"us": round(us, 2)}
        if nbytes is not None:
            per[name].update(bytes=int(nbytes), GBps=round(nbytes / (us * 1e-6) / 1e9, 1),
                             hbm_frac=round(nbytes / (us * 1e-6) / 1e9 / RF.HBM_PEAK_GBS, 4))
    # the whole verification call (row statistics + verify kernels), events on the library's stream
    cache.set_lens(base_lens)
    ev = []
    for rep in range(3 + 20):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        dr.sample_accept(Bn, gamma, T, draft, z, target, u_acc, u_emit, tau, nxt, draft_lse=lse)
        b.record(stream)
        if rep >= 3:
            ev.append((a, b))
    torch.cuda.synchronize()
    call_us = float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e3
    vb = RF.verify_bytes(Bn, n, V, lse_given=True)
    # the same call on 16 sequences of seeded synthetic logits (draft logits
    # N(0, 1.28^2), target = draft + N(0, 0.5^2), random drafts): the regime
    # where the verification streams enough bytes to be bandwidth-bound
    B16 = 16
    i16 = Inputs16(cfg, B16)
    z16 = torch.from_numpy(i16.synthetic_logits(0, gamma, 1.28)).to(dev)
    t16 = torch.from_numpy(i16.target_noise(0, gamma)).to(dev)
    t16[:, :n].mul_(0.5).add_(z16)
    d16 = torch.from_numpy(i16.random_ids(0, gamma)).to(dev)
    _, au16, ru16 = (torch.from_numpy(x).to(dev) for x in i16.sample_uniforms(0, gamma))
    lse16 = torch.logsumexp(z16 / T, dim=-1)
    tau16 = torch.empty(B16, dtype=torch.int32, device=dev)
    nxt16 = torch.empty(B16, dtype=torch.int32, device=dev)
    ws16_bytes = B.workspace_size(dr.dims, B16, gamma, 1)
    ws16 = torch.empty(ws16_bytes, dtype=torch.uint8, device=dev)
    ev16 = []
    for rep in range(3 + 20):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        B.sample_accept(dr.dims, B16, gamma, T, d16.data_ptr(), z16.data_ptr(), lse16.data_ptr(), t16.data_ptr(),
                        au16.data_ptr(), ru16.data_ptr(), tau16.data_ptr(), nxt16.data_ptr(), ws16.data_ptr(),
                        ws16_bytes, stream.cuda_stream)
        b.record(stream)
        if rep >= 3:
            ev16.append((a, b))
    torch.cuda.synchronize()
    call16_us = float(np.median([a.elapsed_time(b) for a, b in ev16])) * 1e3
    vb16 = RF.verify_bytes(B16, n, V, lse_given=True)
    del z16, t16, ws16
    lm_bytes = RF.lm_head_sample_bytes(V, cfg.D, Bn * n, RF.elem_bytes(cfg.dtype))
    lm_gbs = lm_bytes / (lm_us * 1e-6) / 1e9
    log(f"sampled step {ms * 1e3:.1f} us (greedy {greedy_ms * 1e3:.1f}), LM head + sampling {lm_us:.1f} us "
        f"({lm_gbs:.0f} GB/s), verify call {call_us:.1f} us, mean tau {np.mean(taus):.2f}")
    return {
        "temperature": T,
        "step": ("draft forward -> LM head with in-epilogue Gumbel-max sampling and log-sum-exp -> synthetic "
                 "target logits (draft logits + N(0, 0.5^2) noise; bonus row N(0, 1)) -> lossless verify -> "
                 f"append {cfg.append_rows} rows"),
        "blocks_per_s": round(Bn / (ms * 1e-3), 2),
        "ms_per_step": round(ms, 4),
        "vs_greedy_step": round(ms / greedy_ms, 4),
        "mean_tau": round(float(np.mean(taus)), 3),
        "lm_head_sample": {"us": round(lm_us, 2), "bytes": int(lm_bytes), "GBps": round(lm_gbs, 1),
                           "hbm_frac": round(lm_gbs / RF.HBM_PEAK_GBS, 4)},
        "row_stats": per["row_stats"],
        "verify_kernels_us": per["verify"]["us"],
        "verify_call": {"us": round(call_us, 2), "bytes": int(vb), "GBps": round(vb / (call_us * 1e-6) / 1e9, 1),
                        "hbm_frac": round(vb / (call_us * 1e-6) / 1e9 / RF.HBM_PEAK_GBS, 4)},
        "verify_call_b16": {"us": round(call16_us, 2), "bytes": int(vb16),
                            "GBps": round(vb16 / (call16_us * 1e-6) / 1e9, 1),
                            "hbm_frac": round(vb16 / (call16_us * 1e-6) / 1e9 / RF.HBM_PEAK_GBS, 4),
                            "mean_tau": round(float(tau16.float().mean().item()), 3)},
    }


RAGGED_GAMMAS = [4, 8, 16, 32] * 4


def ragged_leg(cfg, dr):
    """Blocks with a length per sequence: 16 sequences with the batch16_ragged
    context lengths (U[1024, 4096]) and block lengths 4/8/16/32, drafted in one
    pass (draft forward + LM-head argmax), against the same batch padded to the
    longest block (one uniform pass at gamma = 32)."""
    import numpy as np
    import torch

    from block_diffusion_drafter_ctx_amd import roofline as RF
    from dflash_inputs import BATCH16_RAGGED, DEEP8_B4_N8192

    dev = "cuda"
    ctx = list(BATCH16_RAGGED.ctx)
    gs = RAGGED_GAMMAS
    Bn, gmax, D, V = len(gs), max(gs), cfg.D, cfg.V
    stream = torch.cuda.current_stream()
    # seeded device-side context states (values do not change the timing)
    gen = torch.Generator(device=dev)
    gen.manual_seed(20261202)
    N = sum(ctx)
    cap = (max(ctx) + gmax + 31) // 32 * 32
    cache = dr.cache(Bn, cap)
    dr.ensure_workspace(Bn, gmax, N)
    states = [torch.randn(N, D, generator=gen, device=dev).to(torch.bfloat16) for _ in range(cfg.n_tgt)]
    H_t = dr.context_buffer(N)
    dr.fuse(states, N, H_t)
    dr.inject(H_t, ctx, cache)
    del states, H_t
    M, nd = sum(gs), sum(gs) - Bn
    tok = torch.full((M,), cfg.mask_id, dtype=torch.int32, device=dev)
    off = np.concatenate([[0], np.cumsum(gs)]).astype(int)
    tok[torch.from_numpy(off[:-1]).to(dev)] = torch.arange(Bn, dtype=torch.int32, device=dev)
    hf = torch.empty(M, D, dtype=torch.float32, device=dev)
    dr_ = torch.empty(nd, dtype=torch.int32, device=dev)
    tok_u = torch.full((Bn, gmax), cfg.mask_id, dtype=torch.int32, device=dev)
    tok_u[:, 0] = torch.arange(Bn, dtype=torch.int32, device=dev)
    hf_u = torch.empty(Bn, gmax, D, dtype=torch.float32, device=dev)
    d_u = torch.empty(Bn, gmax - 1, dtype=torch.int32, device=dev)
    from block_diffusion_drafter_ctx_amd import binding as B

    def ragged():
        dr.draft_ragged(cache, tok, None, gs, hf)
        dr.argmax_accept_ragged(B.ARGMAX, hf, gs, dr_)

    def padded():
        dr.draft(cache, tok_u, None, gmax, hf_u)
        dr.argmax_accept(B.ARGMAX, hf_u, Bn, gmax, d_u)

    def timeit(fn, reps=20):
        for _ in range(3):
            fn()
        ev = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            ev.append((a, b))
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e3

    rag_us = timeit(ragged)
    pad_us = timeit(padded)
    es = RF.elem_bytes(cfg.dtype)
    cs = es                                   # the method's K/V bytes
    rb = RF.draft_forward_bytes_ragged(D, cfg.L, cfg.Hq, cfg.Hkv, cfg.d, cfg.F, V, gs, ctx, es, cs)
    log(f"ragged: 16 sequences, blocks {sorted(set(gs))}: {rag_us:.1f} us vs {pad_us:.1f} us padded to {gmax}")
    del cache
    return {
        "workload": (f"16 sequences, contexts U[1024, 4096] (batch16_ragged lengths, sum {N}), block lengths "
                     f"4/8/16/32 ({M} block rows, {nd} drafts), {cfg.L} layers at the bench drafter's shape"),
        "gammas": gs,
        "draft_fwd_us": round(rag_us, 2),
        "padded_to_32_us": round(pad_us, 2),
        "speedup_vs_padded": round(pad_us / rag_us, 3),
        "drafts_per_s": round(nd / (rag_us * 1e-6), 1),
        "bytes": int(rb),
        "GBps": round(rb / (rag_us * 1e-6) / 1e9, 1),
        "hbm_frac": round(rb / (rag_us * 1e-6) / 1e9 / RF.HBM_PEAK_GBS, 4),
    }


LONG_CTX = 32768


def long_context_leg(cfg, dr):
    """The long-context workload (one sequence, a 32768-token context ingested
    untimed from seeded device-side states, gamma 16): draft forward + LM-head
    argmax at a fixed cache (median of 20), and the attention launches alone
    (HIP events the library records around each one on its stream), against
    the context + block K/V each layer reads."""
    import numpy as np
    import torch

    from block_diffusion_drafter_ctx_amd import binding as B
    from block_diffusion_drafter_ctx_amd import roofline as RF

    dev = "cuda"
    g, N = 16, LONG_CTX
    stream = torch.cuda.current_stream()
    cache = dr.cache(1, (N + g + 31) // 32 * 32)
    dr.ensure_workspace(1, g, N)
    gen = torch.Generator(device=dev)
    gen.manual_seed(20261207)
    H_t = dr.context_buffer(N)
    for r0 in range(0, N, 8192):
        states = [torch.randn(8192, cfg.D, generator=gen, device=dev).to(torch.bfloat16) for _ in range(cfg.n_tgt)]
        dr.fuse(states, 8192, H_t[r0:r0 + 8192])
        del states
    dr.inject(H_t, [N], cache)
    del H_t
    tok = torch.full((1, g), cfg.mask_id, dtype=torch.int32, device=dev)
    hf = torch.empty(1, g, cfg.D, dtype=torch.float32, device=dev)
    d = torch.empty(1, g - 1, dtype=torch.int32, device=dev)

    def fwd():
        dr.draft(cache, tok, None, g, hf)
        dr.argmax_accept(B.ARGMAX, hf, 1, g, d)

    for _ in range(3):
        fwd()
    ev = []
    for _ in range(20):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fwd()
        b.record(stream)
        ev.append((a, b))
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(cfg.L * 10)]
    for a, b in pairs:
        a.record(stream)
        b.record(stream)
    torch.cuda.synchronize()
    B.profile_events(B.PROF_ATTENTION, [a.cuda_event for a, _ in pairs], [b.cuda_event for _, b in pairs])
    for _ in range(10):
        dr.draft(cache, tok, None, g, hf)
    torch.cuda.synchronize()
    B.profile_events(B.PROF_ATTENTION, [], [])
    us = float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e3
    att_us = float(np.median([a.elapsed_time(b) for a, b in pairs])) * 1e3
    es = RF.elem_bytes(cfg.dtype)
    cs = es                                   # the method's K/V bytes
    nbytes = RF.draft_forward_bytes(cfg.D, cfg.L, cfg.Hq, cfg.Hkv, cfg.d, cfg.F, cfg.V, 1, g, [N], es, cs)
    att_bytes = (N + g) * 2 * cfg.Hkv * cfg.d * cs
    log(f"long context: {N}-token context, draft fwd + argmax {us:.1f} us, attention {att_us:.1f} us per layer "
        f"({att_bytes / (att_us * 1e-6) / 1e9:.0f} GB/s)")
    del cache
    return {
        "workload": (f"one sequence, {N}-token context (ingested untimed), gamma {g}, {cfg.L} layers at the bench "
                     f"drafter's shape, {cfg.cache_dtype} cache; draft forward + LM-head argmax at a fixed cache"),
        "draft_fwd_us": round(us, 1), "bytes": int(nbytes),
        "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / RF.HBM_PEAK_GBS, 4),
        "attention": {"us_per_layer": round(att_us, 2), "bytes_per_layer": int(att_bytes),
                      "GBps": round(att_bytes / (att_us * 1e-6) / 1e9, 1),
                      "hbm_frac": round(att_bytes / (att_us * 1e-6) / 1e9 / RF.HBM_PEAK_GBS, 4)},
    }


def gamma_sweep_leg():
    """Draft forward + LM-head argmax of the deep8_b4_n8192 workload (8 layers,
    4 sequences with 8192-token contexts) at blocks of 8, 16 and 32 rows, on one
    fixed cache: the drafting cost should stay flat in the block size ([JP]
    "Preliminaries": one pass whatever the block length)."""
    import numpy as np
    import torch

    from block_diffusion_drafter_ctx_amd import binding as B
    from block_diffusion_drafter_ctx_amd import roofline as RF
    from block_diffusion_drafter_ctx_amd.runtime import DeviceDrafter
    from dflash_inputs import BATCH16_RAGGED, DEEP8_B4_N8192

    cfg = DEEP8_B4_N8192
    dev = "cuda"
    gammas = list(cfg.gammas)
    gmax, Bn, N = max(gammas), cfg.B, cfg.ctx[0]
    dr = DeviceDrafter.random_init(cfg, 20261205, dev)
    cache = dr.cache(Bn, (N + gmax + 31) // 32 * 32)
    dr.ensure_workspace(Bn, gmax, cfg.n_ctx_total)
    gen = torch.Generator(device=dev)
    gen.manual_seed(20261206)
    states = [torch.randn(cfg.n_ctx_total, cfg.D, generator=gen, device=dev).to(torch.bfloat16)
              for _ in range(cfg.n_tgt)]
    H_t = dr.context_buffer(cfg.n_ctx_total)
    dr.fuse(states, cfg.n_ctx_total, H_t)
    dr.inject(H_t, list(cfg.ctx), cache)
    del states, H_t
    stream = torch.cuda.current_stream()
    es = RF.elem_bytes(cfg.dtype)
    cs = es                                   # the method's K/V bytes
    res = {}
    for g in gammas:
        tok = torch.full((Bn, g), cfg.mask_id, dtype=torch.int32, device=dev)
        tok[:, 0] = torch.arange(Bn, dtype=torch.int32, device=dev)
        hf = torch.empty(Bn, g, cfg.D, dtype=torch.float32, device=dev)
        d = torch.empty(Bn, g - 1, dtype=torch.int32, device=dev)
        for _ in range(3):
            dr.draft(cache, tok, None, g, hf)
            dr.argmax_accept(B.ARGMAX, hf, Bn, g, d)
        ev = []
        for _ in range(20):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            dr.draft(cache, tok, None, g, hf)
            dr.argmax_accept(B.ARGMAX, hf, Bn, g, d)
            b.record(stream)
            ev.append((a, b))
        torch.cuda.synchronize()
        us = float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e3
        nbytes = RF.draft_forward_bytes(cfg.D, cfg.L, cfg.Hq, cfg.Hkv, cfg.d, cfg.F, cfg.V, Bn, g, list(cfg.ctx),
                                        es, cs)
        res[str(g)] = {"us": round(us, 1), "bytes": int(nbytes),
                       "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / RF.HBM_PEAK_GBS, 4)}
    ratio = res[str(gmax)]["us"] / res[str(min(gammas))]["us"]
    log(f"gamma sweep (8 layers, 4 x 8192): " + ", ".join(f"{g}: {v['us']:.0f} us" for g, v in res.items()) +
        f"; us({gmax}) / us({min(gammas)}) = {ratio:.3f}")
    del dr, cache
    return {"workload": (f"{cfg.name}: {cfg.L} layers, {Bn} sequences x {N}-token contexts, draft forward + "
                         f"LM-head argmax at a fixed cache (seeded device-side random-init weights)"),
            "per_gamma": res, "us_ratio_max_over_min": round(ratio, 3)}


def workload_loop_leg(name, cache_dtype, cycles=3, seed=20261210):
    """The drafting loop of one workload, per block length: ``cycles`` passes
    over its 8 iterations, each one draft forward -> LM-head argmax ->
    synthetic target tokens on the device (the workload's match
    probabilities) -> greedy accept -> append 16 rows per sequence (fuse +
    inject); the cache length returns to the context length at the start of
    every pass.  Blocks/s = sequences x iterations / time, with the algorithmic
    bytes and FLOPs of an iteration (mean over the cycle's cache lengths)
    against the HBM and bf16 MFMA peaks; plus the draft forward + argmax alone
    at the context length (median of 20).  Weights are seeded device-side
    random-init tensors of the workload's shape; context and appended target
    states are device-side N(0, 1)."""
    import numpy as np
    import torch

    from block_diffusion_drafter_ctx_amd import binding as B
    from block_diffusion_drafter_ctx_amd import roofline as RF
    from block_diffusion_drafter_ctx_amd.runtime import DeviceDrafter
    from dflash_inputs import WORKLOADS, shrink

    base = WORKLOADS[name]
    cfg = shrink(base, cache_dtype=cache_dtype if base.dtype == "bf16" else "f32")
    dev = "cuda"
    stream = torch.cuda.current_stream()
    Bn, N, A, I = cfg.B, cfg.n_ctx_total, cfg.append_rows, cfg.iters
    wdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    es = RF.elem_bytes(cfg.dtype)
    dr = DeviceDrafter.random_init(cfg, seed, dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed + 1)
    rng = np.random.default_rng([seed, cfg.cid])
    out = {"workload": (f"{cfg.name}: batch {Bn}, contexts {'U[1024, 4096] (sum %d)' % N if Bn > 1 and len(set(cfg.ctx)) > 1 else cfg.ctx[0]}, "
                        f"{cfg.L} layers, D={cfg.D}, {cfg.Hq}q/{cfg.Hkv}kv x {cfg.d}, FFN {cfg.F}, V={cfg.V}, "
                        f"{cfg.dtype} weights, {cfg.cache_dtype} cache; {I} iterations of draft forward + argmax + "
                        f"accept + {A}-row append per sequence"),
           "per_gamma": {}}
    for g in cfg.gammas:
        n = g - 1
        cap = (max(cfg.ctx) + I * A + g + 31) // 32 * 32
        cache = dr.cache(Bn, cap)
        dr.ensure_workspace(Bn, g, max(min(N, 8192), Bn * A))
        H_t = dr.context_buffer(min(N, 8192))
        rows = 0
        lens0 = [0] * Bn
        # context ingest (untimed) in row blocks of at most 8192, sequence by sequence
        for b, nb in enumerate(cfg.ctx):
            for r0 in range(0, nb, 8192):
                m = min(8192, nb - r0)
                st = [torch.randn(m, cfg.D, generator=gen, device=dev).to(wdt) for _ in range(cfg.n_tgt)]
                dr.fuse(st, m, H_t)
                counts = [0] * Bn
                counts[b] = m
                dr.inject(H_t, counts, cache)
                del st
        base_lens = cache.len_list()
        app = []
        for it in range(I):
            st = [torch.randn(Bn * A, cfg.D, generator=gen, device=dev).to(wdt) for _ in range(cfg.n_tgt)]
            match = rng.random((Bn, n)) < cfg.match_probs(g)[None, :]
            shift = np.where(match, 0, rng.integers(1, cfg.V, (Bn, n))).astype(np.int32)
            tgt = np.zeros((Bn, g), dtype=np.int32)
            tgt[:, n] = rng.integers(0, cfg.V, Bn)
            app.append(dict(states=st, shift=torch.from_numpy(shift).to(dev), target=torch.from_numpy(tgt).to(dev)))
        H_app = dr.context_buffer(Bn * A)
        tokens = torch.full((Bn, g), cfg.mask_id, dtype=torch.int32, device=dev)
        tokens[:, 0] = torch.from_numpy(rng.integers(0, cfg.V - 1, Bn).astype(np.int32)).to(dev)
        h_final = torch.empty(Bn, g, cfg.D, dtype=torch.float32, device=dev)
        draft = torch.empty(Bn, n, dtype=torch.int32, device=dev)
        tau = torch.empty(Bn, dtype=torch.int32, device=dev)
        nxt = torch.empty(Bn, dtype=torch.int32, device=dev)
        tmp = torch.empty(Bn, n, dtype=torch.int32, device=dev)

        def step(i):
            it = i % I
            if it == 0:
                cache.set_lens(base_lens, mirror=False)
            dr.draft(cache, tokens, None, g, h_final)
            dr.argmax_accept(B.ARGMAX, h_final, Bn, g, draft)
            d = app[it]
            torch.add(draft, d["shift"], out=tmp)
            torch.remainder(tmp, cfg.V, out=d["target"][:, :n])
            dr.argmax_accept(B.ACCEPT, None, Bn, g, draft, target=d["target"], tau=tau, nxt=nxt)
            tokens[:, 0].copy_(nxt)
            dr.fuse(d["states"], Bn * A, H_app)
            dr.inject(H_app, [A] * Bn, cache)

        for i in range(I):
            step(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for i in range(cycles * I):
            step(i)
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        us_it = max(e0.elapsed_time(e1) * 1e3, wall * 1e6) / (cycles * I)
        taus = tau.cpu().numpy()
        # the draft forward + argmax alone at the context length
        cache.set_lens(base_lens)
        ev = []
        for rep in range(23):
            a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            dr.draft(cache, tokens, None, g, h_final)
            dr.argmax_accept(B.ARGMAX, h_final, Bn, g, draft)
            b_.record(stream)
            if rep >= 3:
                ev.append((a, b_))
        torch.cuda.synchronize()
        fwd_us = float(np.median([a.elapsed_time(b_) for a, b_ in ev])) * 1e3
        # algorithmic work of one iteration, averaged over the cycle's cache lengths
        nbytes = fl = 0.0
        for it in range(I):
            ctx = [c + A * it for c in cfg.ctx]
            nbytes += (RF.draft_forward_bytes(cfg.D, cfg.L, cfg.Hq, cfg.Hkv, cfg.d, cfg.F, cfg.V, Bn, g, ctx, es, es)
                       + RF.fuse_bytes(Bn * A, cfg.D, cfg.n_tgt, es, es)
                       + RF.inject_bytes(Bn * A, cfg.D, cfg.L, cfg.Hkv, cfg.d, es, es)
                       + RF.accept_bytes(Bn, n)) / I
            fl += (RF.draft_forward_flops(cfg.D, cfg.L, cfg.Hq, cfg.Hkv, cfg.d, cfg.F, cfg.V, Bn, g, ctx)
                   + RF.fuse_flops(Bn * A, cfg.D, cfg.n_tgt) + RF.inject_flops(Bn * A, cfg.D, cfg.L, cfg.Hkv, cfg.d)) / I
        fwd_bytes = RF.draft_forward_bytes(cfg.D, cfg.L, cfg.Hq, cfg.Hkv, cfg.d, cfg.F, cfg.V, Bn, g, list(cfg.ctx),
                                           es, es)
        peak_tf = RF.MFMA_BF16_TFLOPS if cfg.dtype == "bf16" else RF.FP32_VECTOR_TFLOPS
        out["per_gamma"][str(g)] = {
            "blocks_per_s": round(Bn * 1e6 / us_it, 2), "us_per_iteration": round(us_it, 1),
            "bytes_per_iteration": int(nbytes), "gflop_per_iteration": round(fl / 1e9, 2),
            "hbm_frac": round(nbytes / (us_it * 1e-6) / 1e9 / RF.HBM_PEAK_GBS, 4),
            "mfma_frac": round(fl / (us_it * 1e-6) / 1e12 / peak_tf, 4),
            "draft_fwd_us": round(fwd_us, 1),
            "draft_fwd_hbm_frac": round(fwd_bytes / (fwd_us * 1e-6) / 1e9 / RF.HBM_PEAK_GBS, 4),
            "last_tau": taus.tolist()[:16]}
        log(f"loop {cfg.name} gamma {g}: {us_it:.1f} us per iteration ({Bn * 1e6 / us_it:.1f} blocks/s), "
            f"draft fwd {fwd_us:.1f} us")
        del cache, app, H_t, H_app
    if len(cfg.gammas) > 1:
        us = [v["draft_fwd_us"] for v in out["per_gamma"].values()]
        out["draft_fwd_us_ratio_max_over_min"] = round(max(us) / min(us), 3)
    if cfg.dtype != "bf16":
        out["note"] = "fp32 weights: latency-bound (reported, not graded); mfma_frac is against the fp32 vector peak"
    del dr
    torch.cuda.empty_cache()
    return out


def speculative_leg(cache_dtype, steps=24, seed=20261220):
    """Greedy speculative decoding with the target side in the loop, on a
    synthetic Qwen3-8B-shaped target (36 layers of the drafter's layer shape,
    causal attention, seeded device-side random init) and the 5-layer drafter,
    which shares the target's embedding and LM head.  One step: draft forward
    + LM-head argmax -> the target's verify pass over (anchor, drafts) with
    its 5 tapped layers -> greedy accept -> commit (the target keeps tau rows
    of K/V; the drafter fuses and injects the tau rows' tapped states).  The
    host reads tau each step (a serving loop must, to emit the tokens).  Both
    caches start from a 2048-token context (target K/V and drafter context
    states N(0, 1)) and return to it every 8 steps.  Random weights make the
    drafter and target disagree (tau ~ 1), so the figures here are the
    drafting and verify costs of the pages' latency model, (T_draft +
    T_verify) / tau, not an acceptance rate."""
    import numpy as np
    import torch

    from block_diffusion_drafter_ctx_amd import binding as B
    from block_diffusion_drafter_ctx_amd import roofline as RF
    from block_diffusion_drafter_ctx_amd.runtime import DeviceDrafter, tap_layers
    from dflash_inputs import QWEN3_8B_N2048, shrink

    dev = "cuda"
    stream = torch.cuda.current_stream()
    dcfg = shrink(QWEN3_8B_N2048, cache_dtype=cache_dtype)
    tcfg = shrink(QWEN3_8B_N2048, name="qwen3_8b_shaped_target", L=36, cache_dtype=cache_dtype)
    g, n, N = 16, 15, dcfg.ctx[0]
    taps = tap_layers(tcfg.L, tcfg.n_tgt)
    tgt = DeviceDrafter.random_init(tcfg, seed, dev)
    drf = DeviceDrafter.random_init(dcfg, seed + 1, dev)
    drf.embed = tgt.embed
    drf.weights.embed = drf.weights.lm_head = tgt.embed.data_ptr()
    cap = (N + 8 * g + g + 31) // 32 * 32
    tcache, dcache = tgt.cache(1, cap), drf.cache(1, cap)
    tgt.ensure_workspace(1, g, 1)
    drf.ensure_workspace(1, g, N)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed + 2)
    tcache.fill_random(0, N, gen)
    tcache.set_lens([N])
    st = [torch.randn(N, dcfg.D, generator=gen, device=dev).to(torch.bfloat16) for _ in range(dcfg.n_tgt)]
    H = drf.context_buffer(N)
    drf.fuse(st, N, H)
    drf.inject(H, [N], dcache)
    del st, H
    tap_bufs = [torch.empty(g, tcfg.D, dtype=torch.bfloat16, device=dev) for _ in taps]
    block = torch.full((1, g), dcfg.mask_id, dtype=torch.int32, device=dev)
    block[0, 0] = 7
    tokens = torch.full((1, g), dcfg.mask_id, dtype=torch.int32, device=dev)
    hf = torch.empty(1, g, dcfg.D, dtype=torch.float32, device=dev)
    draft = torch.empty(1, n, dtype=torch.int32, device=dev)
    ttok = torch.empty(1, g, dtype=torch.int32, device=dev)
    tau = torch.empty(1, dtype=torch.int32, device=dev)
    nxt = torch.empty(1, dtype=torch.int32, device=dev)
    H_app = drf.context_buffer(g)
    ev = {"draft": [], "verify": []}

    def step(i, timed):
        if i % 8 == 0:
            tcache.set_lens([N], mirror=False)
            dcache.set_lens([N], mirror=False)
        tokens[0, 0] = block[0, 0]
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record(stream)
        drf.draft(dcache, tokens, None, g, hf)
        drf.argmax_accept(B.ARGMAX, hf, 1, g, draft)
        e[1].record(stream)
        block[0, 1:].copy_(draft[0])
        tgt.target_verify(tcache, block, g, taps, tap_bufs, ttok)
        e[2].record(stream)
        drf.argmax_accept(B.ACCEPT, None, 1, g, draft, target=ttok, tau=tau, nxt=nxt)
        t = int(tau.item())                      # the host learns how many tokens were committed
        tcache.set_lens([tcache.len_list()[0] + t], mirror=False)
        drf.fuse([b[:t] for b in tap_bufs], t, H_app)
        drf.inject(H_app, [t], dcache)
        block[0, 0] = nxt[0]
        if timed:
            ev["draft"].append((e[0], e[1]))
            ev["verify"].append((e[1], e[2]))
        return t

    for i in range(8):
        step(i, False)
    torch.cuda.synchronize()
    taus = []
    t0 = time.perf_counter()
    for i in range(steps):
        taus.append(step(i, True))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    d_us = float(np.median([a.elapsed_time(b) for a, b in ev["draft"]])) * 1e3
    v_us = float(np.median([a.elapsed_time(b) for a, b in ev["verify"]])) * 1e3
    step_us = wall / steps * 1e6
    vbytes = (tcfg.L * RF.layer_weight_elems(tcfg.D, tcfg.Hq, tcfg.Hkv, tcfg.d, tcfg.F) + tcfg.D + tcfg.V * tcfg.D) * 2 \
        + tcfg.L * (N + 4 * g) * 2 * tcfg.Hkv * tcfg.d * 2
    log(f"speculative: draft {d_us:.0f} us, verify ({tcfg.L} target layers) {v_us:.0f} us, step {step_us:.0f} us, "
        f"mean tau {np.mean(taus):.2f}")
    del tgt, drf, tcache, dcache
    torch.cuda.empty_cache()
    return {"workload": (f"greedy speculative decoding, batch 1, 2048-token context: the qwen3_8b_shape_n2048 "
                         f"drafter and a synthetic Qwen3-8B-shaped target ({tcfg.L} layers, causal, taps {taps}) "
                         f"sharing the embedding / LM head, random-init weights, {cache_dtype} caches; step = draft "
                         f"forward + argmax + target verify of 16 rows + accept + commit (host reads tau)"),
            "t_draft_us": round(d_us, 1), "t_verify_us": round(v_us, 1), "step_us": round(step_us, 1),
            "verify_over_draft": round(v_us / d_us, 3), "mean_tau": round(float(np.mean(taus)), 3),
            "tokens_per_s": round(float(np.sum(taus)) / wall, 1),
            "verify_bytes": int(vbytes),
            "verify_hbm_frac": round(vbytes / (v_us * 1e-6) / 1e9 / RF.HBM_PEAK_GBS, 4)}


BLOCKS_CTX, BLOCKS_N, BLOCKS_GAMMA = 3072, 64, 16


def blocks_anchors():
    import numpy as np
    rng = np.random.default_rng(20261202)
    return sorted(rng.integers(BLOCKS_CTX // 2, BLOCKS_CTX + 1, BLOCKS_N).tolist())


def blocks_leg(cfg, dr):
    """Many anchored blocks in one pass (the training-style mask): one sequence
    with a 3072-token context (the pages' longest training sequences) and 64
    blocks of 16 rows anchored uniformly in its second half (the response),
    each seeing the context before its anchor and its own rows."""
    import numpy as np
    import torch

    from block_diffusion_drafter_ctx_amd import roofline as RF

    dev = "cuda"
    anchors = blocks_anchors()
    g = BLOCKS_GAMMA
    nb, D = len(anchors), cfg.D
    g32 = (g + 31) // 32 * 32
    cap = (BLOCKS_CTX + 31) // 32 * 32 + nb * g32
    cache = dr.cache(1, cap)
    dr.ensure_workspace(nb, g, BLOCKS_CTX)
    gen = torch.Generator(device=dev)
    gen.manual_seed(20261203)
    states = [torch.randn(BLOCKS_CTX, D, generator=gen, device=dev).to(torch.bfloat16) for _ in range(cfg.n_tgt)]
    H_t = dr.context_buffer(BLOCKS_CTX)
    dr.fuse(states, BLOCKS_CTX, H_t)
    dr.inject(H_t, [BLOCKS_CTX], cache)
    del states, H_t
    tok = torch.full((nb, g), cfg.mask_id, dtype=torch.int32, device=dev)
    tok[:, 0] = torch.arange(nb, dtype=torch.int32, device=dev)
    hf = torch.empty(nb, g, D, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(3):
        dr.draft_blocks(cache, [0] * nb, anchors, g, tok, None, hf)
    ev = []
    for _ in range(20):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        dr.draft_blocks(cache, [0] * nb, anchors, g, tok, None, hf)
        b.record(stream)
        ev.append((a, b))
    torch.cuda.synchronize()
    us = float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e3
    M = nb * g
    flops = 2 * M * cfg.L * (RF.layer_weight_elems(cfg.D, cfg.Hq, cfg.Hkv, cfg.d, cfg.F) - 2 * D) + \
        cfg.L * sum(4 * cfg.Hq * g * (a + g) * cfg.d for a in anchors)
    cs = RF.elem_bytes(cfg.dtype)             # the method's K/V bytes
    nbytes = (cfg.L * RF.layer_weight_elems(cfg.D, cfg.Hq, cfg.Hkv, cfg.d, cfg.F) * RF.elem_bytes(cfg.dtype)
              + cfg.L * sum(a + g for a in anchors) * 2 * cfg.Hkv * cfg.d * cs + M * D * 4 * 2)
    log(f"blocks: {nb} blocks of {g} rows in a {BLOCKS_CTX}-token context: {us:.1f} us")
    del cache
    return {
        "workload": (f"one sequence, {BLOCKS_CTX}-token context, {nb} blocks of {g} rows anchored uniformly in "
                     f"[{BLOCKS_CTX // 2}, {BLOCKS_CTX}] ({M} query rows), {cfg.L} layers at the bench drafter's "
                     f"shape; forward pass only (no LM head)"),
        "anchors": anchors,
        "us": round(us, 1),
        "gflop": round(flops / 1e9, 1),
        "tflops": round(flops / (us * 1e-6) / 1e12, 1),
        "mfma_frac": round(flops / (us * 1e-6) / 1e12 / RF.MFMA_BF16_TFLOPS, 4),
        "bytes": int(nbytes),
        "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / RF.HBM_PEAK_GBS, 4),
        "note": "FLOPs are algorithmic (one product per GEMM); the fp32 activations run as two bf16 products",
    }


def cpu_model():
    """The host CPU's model name (first entry of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_tiny_baseline(seconds=3.0):
    """The oracle on whole drafting iterations of the tiny fp32 workload
    (draft forward + argmax + accept + 16-row append, seeded inputs), on the
    BLAS threads numpy has and on one thread."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import dflash_oracle as O
    from dflash_inputs import TINY_F32, Inputs, build_target_np

    cfg = TINY_F32
    inp = Inputs(cfg)
    f = lambda a: np.asarray(a, dtype=np.float64)  # noqa: E731
    layers = [dict(w_qkv=f(inp.w_qkv(l)), w_o=f(inp.w_o(l)), w_gateup=f(inp.w_gateup(l)), w_down=f(inp.w_down(l)),
                   g_attn=f(inp.g_attn(l)), g_ffn=f(inp.g_ffn(l))) for l in range(cfg.L)]
    E, gf, wc, gc = f(inp.embed()), f(inp.g_final()), inp.w_c(), inp.g_c()
    Ht = O.fuse_context(inp.ctx_states(), wc, gc, cfg.eps, cfg.cache_dtype)
    base = [O.inject_kv(Ht, layers[l]["w_qkv"], cfg.Hq, cfg.Hkv, cfg.d, cfg.cache_dtype) for l in range(cfg.L)]
    appends = [inp.append_states(it) for it in range(cfg.iters)]
    draws = [inp.verify_draws(it, cfg.gamma) for it in range(cfg.iters)]

    def run():
        anchors, done, t0, cache = inp.anchors(), 0, time.perf_counter(), None
        while done < 4096 and (done == 0 or time.perf_counter() - t0 < seconds):
            it = done % cfg.iters
            if it == 0:
                cache = O.OracleCache(cfg.L, 1, cfg.Hkv, cfg.d)
                for l in range(cfg.L):
                    cache.append(l, 0, *base[l])
            hf, _ = O.draft_forward(cfg, layers, gf, cache, cfg.gamma, embed=E, tokens=inp.block_tokens(cfg.gamma, anchors),
                                    storage=cfg.cache_dtype)
            d, _, _ = O.lm_head_argmax(hf, E)
            m, r, bonus = draws[it]
            _, anchors = O.accept(d, build_target_np(d, m, r, bonus, cfg.V))
            Ha = O.fuse_context(appends[it], wc, gc, cfg.eps, cfg.cache_dtype)
            for l in range(cfg.L):
                cache.append(l, 0, *O.inject_kv(Ha, layers[l]["w_qkv"], cfg.Hq, cfg.Hkv, cfg.d, cfg.cache_dtype))
            done += 1
        return done, time.perf_counter() - t0

    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    n_all, t_all = run()
    with threadpool_limits(limits=1):
        n_one, t_one = run()
    log(f"cpu baseline (tiny): {n_all} iterations in {t_all:.1f}s on {threads} threads, {n_one} in {t_one:.1f}s on 1")
    return {"value": round(n_all / t_all, 2), "unit": "blocks/s", "cores": int(threads), "kind": "oracle",
            "us_per_iteration": round(t_all / n_all * 1e6, 1),
            "one_thread": {"value": round(n_one / t_one, 2), "unit": "blocks/s", "cores": 1,
                           "us_per_iteration": round(t_one / n_one * 1e6, 1)},
            "cpu_model": cpu_model(),
            "sample": f"whole drafting iterations of tiny_f32 (draft forward + argmax + accept + 16-row append), "
                      f"float64 numpy oracle, ~{seconds:.0f} s per thread count"}


def cpu_baseline(cfg, inp, seconds, temperature=None, ragged=False, blocks=False, long_ctx=False):
    """The CPU oracle, as it stands, on whole drafting iterations of the same
    workload (draft forward + LM-head argmax + accept + 16-row append), repeated
    for about ``seconds`` with the GPU loop's 8-iteration cache reset; then, when
    ``temperature`` is given, the sampled iteration (draft forward + sampled
    drafts + synthetic target logits + lossless verify + append) for about half
    as long; then, when ``ragged``, one ragged pass over a sample of the ragged
    leg's batch; when ``blocks`` / ``long_ctx``, two of the blocks leg's
    blocks / one block over the long-context leg's 32768-row context (random
    context K/V).  Returns (greedy, sampled, ragged, blocks, long context), None
    for the ones not asked for."""
    import numpy as np
    from oracle import dflash_oracle as O
    from dflash_inputs import build_target_np

    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        cores = os.cpu_count() or 1
    log(f"cpu baseline: oracle context ingest ({cfg.n_ctx_total} rows, untimed)")
    f = lambda a: np.asarray(a, dtype=np.float64)  # noqa: E731
    layers = [dict(w_qkv=f(inp.w_qkv(l)), w_o=f(inp.w_o(l)), w_gateup=f(inp.w_gateup(l)), w_down=f(inp.w_down(l)),
                   g_attn=f(inp.g_attn(l)), g_ffn=f(inp.g_ffn(l))) for l in range(cfg.L)]
    E = f(inp.embed())
    gf = f(inp.g_final())
    wc, gc = inp.w_c(), inp.g_c()
    Ht = O.fuse_context(inp.ctx_states(), wc, gc, cfg.eps, cfg.cache_dtype)
    off = np.concatenate([[0], np.cumsum(cfg.ctx)])
    base = [[O.inject_kv(Ht[off[b]:off[b + 1]], layers[l]["w_qkv"], cfg.Hq, cfg.Hkv, cfg.d, cfg.cache_dtype)
             for b in range(cfg.B)] for l in range(cfg.L)]
    appends = [inp.append_states(it) for it in range(cfg.iters)]
    draws = [inp.verify_draws(it, cfg.gamma) for it in range(cfg.iters)]
    gamma = cfg.gamma
    if temperature is not None:
        from dflash_inputs import build_target_logits_np
        ug, ua, ur = inp.sample_uniforms(0, gamma)
        noise = inp.target_noise(0, gamma)

    def run(sampled, budget):
        anchors = inp.anchors()
        done = 0
        t0 = time.perf_counter()
        cache = None
        while done < 256 and (done == 0 or time.perf_counter() - t0 < budget):
            it = done % cfg.iters
            if it == 0:
                cache = O.OracleCache(cfg.L, cfg.B, cfg.Hkv, cfg.d)
                for l in range(cfg.L):
                    for b in range(cfg.B):
                        cache.append(l, b, *base[l][b])
            tokens = inp.block_tokens(gamma, anchors)
            hf, _ = O.draft_forward(cfg, layers, gf, cache, gamma, embed=E, tokens=tokens, storage=cfg.cache_dtype)
            if sampled:
                d, z, _, _ = O.sample_drafts(hf, E, temperature, ug)
                tgt = build_target_logits_np(z, noise)
                _, anchors, _ = O.sample_accept(d, z, tgt, temperature, ua, ur)
            else:
                d, _, _ = O.lm_head_argmax(hf, E)
                m, r, bonus = draws[it]
                tgt = build_target_np(d, m, r, bonus, cfg.V)
                _, anchors = O.accept(d, tgt)
            Ha = O.fuse_context(appends[it], wc, gc, cfg.eps, cfg.cache_dtype)
            for l in range(cfg.L):
                for b in range(cfg.B):
                    rows = slice(b * cfg.append_rows, (b + 1) * cfg.append_rows)
                    k, v = O.inject_kv(Ha[rows], layers[l]["w_qkv"], cfg.Hq, cfg.Hkv, cfg.d, cfg.cache_dtype)
                    cache.append(l, b, k, v)
            done += 1
        return done, time.perf_counter() - t0

    done, dt = run(False, seconds)
    log(f"cpu baseline: {done} iteration(s) in {dt:.1f}s on {cores} threads")
    greedy = {"value": round(cfg.B * done / dt, 4), "unit": "blocks/s", "cores": int(cores), "kind": "oracle",
              "cpu_model": cpu_model(),
              "sample": f"{done} full drafting iterations of the same workload (draft forward + LM-head argmax "
                        f"+ accept + 16-row append, cache reset every {cfg.iters}), float64 numpy oracle, "
                        f"after an untimed context ingest",
              "seconds": round(dt, 2)}
    sampled = None
    if temperature is not None:
        done, dt = run(True, seconds / 2)
        log(f"cpu baseline (sampled): {done} iteration(s) in {dt:.1f}s")
        sampled = {"value": round(cfg.B * done / dt, 4), "unit": "blocks/s", "cores": int(cores), "kind": "oracle",
                   "sample": f"{done} sampled drafting iterations at T = {temperature} (draft forward + sampled "
                             f"drafts + synthetic target logits + lossless verify + 16-row append), float64 "
                             f"numpy oracle",
                   "seconds": round(dt, 2)}
    blk = None
    if blocks:
        # two of the blocks leg's anchored blocks over seeded random context K/V
        rng = np.random.default_rng(20261203)
        anchors = blocks_anchors()[:2]
        bc = O.OracleCache(cfg.L, 1, cfg.Hkv, cfg.d)
        for l in range(cfg.L):
            bc.append(l, 0, rng.normal(0, 1, (BLOCKS_CTX, cfg.Hkv, cfg.d)), rng.normal(0, 1, (BLOCKS_CTX, cfg.Hkv, cfg.d)))
        toks = np.full((2, BLOCKS_GAMMA), cfg.mask_id)
        toks[:, 0] = [0, 1]
        t0 = time.perf_counter()
        O.draft_forward_blocks(cfg, layers, gf, bc, [(0, a) for a in anchors], BLOCKS_GAMMA, embed=E, tokens=toks,
                               storage=cfg.cache_dtype)
        dt = time.perf_counter() - t0
        log(f"cpu baseline (blocks): 2 blocks in {dt:.1f}s")
        blk = {"value": round(2 / dt, 4), "unit": "blocks/s", "cores": int(cores), "kind": "oracle",
               "sample": f"two anchored blocks (anchors {anchors}) of the blocks leg over random context K/V, "
                         f"float64 numpy oracle", "seconds": round(dt, 2)}
    lng = None
    if long_ctx:
        # one gamma-16 block over a 32768-row context of seeded random K/V
        rng = np.random.default_rng(20261208)
        lc = O.OracleCache(cfg.L, 1, cfg.Hkv, cfg.d)
        for l in range(cfg.L):
            lc.append(l, 0, rng.normal(0, 1, (LONG_CTX, cfg.Hkv, cfg.d)), rng.normal(0, 1, (LONG_CTX, cfg.Hkv, cfg.d)))
        toks = [np.array([0] + [cfg.mask_id] * 15)]
        t0 = time.perf_counter()
        hf, _ = O.draft_forward_ragged(cfg, layers, gf, lc, [16], embed=E, tokens=toks, storage=cfg.cache_dtype)
        O.lm_head_argmax_ragged(hf, E)
        dt = time.perf_counter() - t0
        del lc
        log(f"cpu baseline (long context): 1 block in {dt:.1f}s")
        lng = {"value": round(1 / dt, 4), "unit": "blocks/s", "cores": int(cores), "kind": "oracle",
               "sample": f"one draft forward + LM-head argmax over a {LONG_CTX}-row context of random K/V, float64 "
                         f"numpy oracle", "seconds": round(dt, 2)}
    if not ragged:
        return greedy, sampled, None, blk, lng
    # the first four sequences of the ragged leg (blocks 4, 8, 16, 32) over
    # seeded random context K/V of their batch16_ragged lengths (stand-ins for
    # an untimed ingest), one ragged pass + argmax
    from dflash_inputs import BATCH16_RAGGED, DEEP8_B4_N8192
    rng = np.random.default_rng(20261202)
    gs = RAGGED_GAMMAS[:4]
    ctx = list(BATCH16_RAGGED.ctx[:4])
    rc = O.OracleCache(cfg.L, len(gs), cfg.Hkv, cfg.d)
    for l in range(cfg.L):
        for b, n in enumerate(ctx):
            rc.append(l, b, rng.normal(0, 1, (n, cfg.Hkv, cfg.d)), rng.normal(0, 1, (n, cfg.Hkv, cfg.d)))
    toks = [np.array([b] + [cfg.mask_id] * (g - 1)) for b, g in enumerate(gs)]
    t0 = time.perf_counter()
    hf, _ = O.draft_forward_ragged(cfg, layers, gf, rc, gs, embed=E, tokens=toks, storage=cfg.cache_dtype)
    O.lm_head_argmax_ragged(hf, E)
    dt = time.perf_counter() - t0
    log(f"cpu baseline (ragged): 4 blocks in {dt:.1f}s")
    rag = {"value": round(len(gs) / dt, 4), "unit": "blocks/s", "cores": int(cores), "kind": "oracle",
           "sample": f"one ragged pass + LM-head argmax over 4 sequences (blocks {gs}, contexts {ctx}, random "
                     f"context K/V), float64 numpy oracle",
           "drafts_per_s": round(sum(g - 1 for g in gs) / dt, 3), "seconds": round(dt, 2)}
    return greedy, sampled, rag, blk, lng


if __name__ == "__main__":
    main()
