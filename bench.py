"""Benchmark: one BLOOM-176B TP=4 shard training step's hot path on one MI355X.

A step is one pass over every kernel of the path, on synthetic BLOOM-shaped
data already resident in HBM:

  LayerNorm fwd + bwd          [2048, 14336] bf16
  ALiBi causal softmax fwd+bwd [1, 28, 2048, 2048] bf16 (heads 0..27 of 112)
  bias + GeLU fwd + bwd        [2048, 14336] bf16
  FP32 gradient accumulation   32 micro-batches of a 3.67e9-element bf16 gradient
  BF16Optimizer step           global norm, clip 1.0, AdamW, bf16 parameter copy

Each kernel reads inputs that were last touched a whole step earlier (the
accumulation streams ~1.2 TB per step in between), so no kernel is served by
the 256 MB Infinity Cache from the previous one.  The 32 micro-batch gradients
cycle through GRAD_BUFFERS distinct 7.34 GB buffers (all 32 would need 235 GB).

Prints one JSON line.  `value` is the whole step's algorithmic HBM throughput
(sum of each kernel's algorithmic bytes / step time, GB/s); per-kernel
algorithmic GB/s, the fraction of the 8 TB/s HBM peak and the AdamW step time
are reported beside it, with a roofline entry for the dominant kernel (the
accumulation) and the CPU oracle timed on a bounded sample.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s (% of peak) per fused kernel; AdamW step ms @3.67B shard"
HBM_PEAK_GBS = 8000.0
GRAD_BUFFERS = 8
COUNTERS = os.path.join(ROOT, "profiles", "counters.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------
# Algorithmic bytes of each step row (what the method must read and write).
def bytes_model(sh, n, mb):
    rows, hid = sh["ln"]
    b, h, s = sh["sm"]
    live = b * h * s * (s + 1) // 2          # causal entries read
    full = b * h * s * s                     # entries written
    grows, gcols = sh["gelu"]
    return {
        "layernorm_fwd": rows * hid * 4 + hid * 4 + rows * 8,
        "layernorm_bwd": rows * hid * 6 + hid * 2 + rows * 8 + hid * 4,
        "alibi_softmax_fwd": live * 2 + full * 2,
        "alibi_softmax_bwd": live * 4 + full * 2,
        "bias_gelu_fwd": grows * gcols * 4 + gcols * 2,
        "bias_gelu_bwd": grows * gcols * 6 + gcols * 4,
        "grad_accumulate_first": n * 6,
        "grad_accumulate": n * 10,
        "grad_accumulate_last": n * 10,  # also emits the norm's FP64 partials (1/1024 of a double per element)
        "adamw_step": n * 30,   # update reads acc, master, m, v (16 B), writes master, m, v, bf16 (14 B)
    }


def source_digest(*paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_key):
    """Counter-measured HBM bytes per launch, if the profile matches the current source."""
    if not os.path.exists(COUNTERS):
        return None
    try:
        data = json.load(open(COUNTERS))
        entry = data.get(kernel_key)
        if not entry:
            return None
        if entry.get("source_digest") != source_digest(*entry["sources"]):
            return None
        return entry.get("hbm_bytes_per_launch")
    except Exception:
        return None


# ----------------------------------------------------------------------------
def run_gpu(args):
    import torch

    from bloom_bf16_optimizer_amd import ops
    from synth import device as sdev
    from synth import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    X = W.SHARD
    O = W.OPTIMIZER
    n = O.opt.n if args.n is None else args.n
    mb = O.opt.microbatches
    rows, hid = X.ln.rows, X.ln.hidden
    smb, smh, sms = X.softmax.batch, X.softmax.heads, X.softmax.seq
    grows, gcols = X.gelu.rows, X.gelu.cols
    bf, f32 = torch.bfloat16, torch.float32
    seed = X.seed

    def fill(shape, stream, sigma, offset=0.0, dtype=bf):
        t = torch.empty(shape, dtype=dtype, device=dev)
        sdev.fill_(t, seed, stream, sigma, offset)
        return t

    log(f"bench: allocating the shard workload (n = {n:,}, {GRAD_BUFFERS} gradient buffers)")
    # fused-kernel tensors; every kernel has its own inputs
    ln_x = fill((rows, hid), W.S_LN_X, 1.0)
    ln_g = fill((hid,), W.S_LN_GAMMA, 0.02, 1.0)
    ln_b = fill((hid,), W.S_LN_BETA, 0.02)
    ln_y = torch.empty_like(ln_x)
    ln_mean = torch.empty(rows, dtype=f32, device=dev)
    ln_rstd = torch.empty_like(ln_mean)
    ln_x2 = fill((rows, hid), 50, 1.0)
    ln_dy = fill((rows, hid), W.S_LN_DY, 1.0)
    ln_dx = torch.empty_like(ln_x)
    ln_dg = torch.empty(hid, dtype=bf, device=dev)
    ln_db = torch.empty_like(ln_dg)
    ln_ws = torch.empty(ops.bloom_layernorm_bwd_workspace_size(rows, hid), dtype=torch.uint8, device=dev)
    ln_mean2 = torch.empty_like(ln_mean)
    ln_rstd2 = torch.empty_like(ln_mean)
    ops.bloom_layernorm_fwd(ln_x2, ln_g, ln_b, ln_dx, ln_mean2, ln_rstd2, W.LN_EPS)  # saved stats for the bwd

    scale = X.softmax.scale
    sm_s = fill((smb, smh, sms, sms), W.S_SM_SCORES, 1.0)
    sm_p = torch.empty_like(sm_s)
    sm_s2 = fill((smb, smh, sms, sms), 51, 1.0)
    sm_y = torch.empty_like(sm_s)
    ops.bloom_alibi_softmax_fwd(sm_s2, sm_y, X.softmax.head_offset, X.softmax.total_heads, scale)
    del sm_s2
    sm_dy = fill((smb, smh, sms, sms), W.S_SM_DPROBS, 1.0)
    sm_ds = torch.empty_like(sm_s)

    ge_x = fill((grows, gcols), W.S_GELU_X, 1.0)
    ge_b = fill((gcols,), W.S_GELU_BIAS, 0.02)
    ge_y = torch.empty_like(ge_x)
    ge_x2 = fill((grows, gcols), 52, 1.0)
    ge_dy = fill((grows, gcols), W.S_GELU_DY, 1.0)
    ge_dx = torch.empty_like(ge_x)
    ge_db = torch.empty(gcols, dtype=bf, device=dev)
    ge_ws = torch.empty(ops.bloom_bias_gelu_bwd_workspace_size(grows, gcols), dtype=torch.uint8, device=dev)

    # optimizer shard
    master = fill((n,), W.S_OPT_PARAM, W.PARAM_SIGMA, dtype=f32)
    exp_avg = torch.zeros(n, dtype=f32, device=dev)
    exp_avg_sq = torch.zeros(n, dtype=f32, device=dev)
    acc = torch.empty(n, dtype=f32, device=dev)
    param = torch.empty(n, dtype=bf, device=dev)
    grads = [fill((n,), W.S_OPT_GRAD0 + 1 + k, W.GRAD_SIGMA) for k in range(GRAD_BUFFERS)]
    norm = torch.empty(1, dtype=f32, device=dev)
    opt_ws = torch.empty(ops.bloom_bf16_adamw_workspace_size(n), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    log(f"bench: resident {torch.cuda.memory_allocated() / 2**30:.1f} GiB")

    names = ["layernorm_fwd", "alibi_softmax_fwd", "bias_gelu_fwd", "bias_gelu_bwd", "alibi_softmax_bwd",
             "layernorm_bwd", "grad_accumulate_first", "grad_accumulate", "grad_accumulate_last", "adamw_step"]
    ev = {k: [] for k in names}

    def timed(name, fn, record):
        if record:
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            ev[name].append((a, b))
        else:
            fn()

    def step(t, record):
        timed("layernorm_fwd", lambda: ops.bloom_layernorm_fwd(ln_x, ln_g, ln_b, ln_y, ln_mean, ln_rstd, W.LN_EPS),
              record)
        timed("alibi_softmax_fwd", lambda: ops.bloom_alibi_softmax_fwd(
            sm_s, sm_p, X.softmax.head_offset, X.softmax.total_heads, scale), record)
        timed("bias_gelu_fwd", lambda: ops.bloom_bias_gelu_fwd(ge_x, ge_b, ge_y), record)
        timed("bias_gelu_bwd", lambda: ops.bloom_bias_gelu_bwd(ge_dy, ge_x2, ge_b, ge_dx, ge_db, ge_ws), record)
        timed("alibi_softmax_bwd", lambda: ops.bloom_alibi_softmax_bwd(sm_y, sm_dy, sm_ds, scale), record)
        timed("layernorm_bwd", lambda: ops.bloom_layernorm_bwd(ln_dy, ln_x2, ln_g, ln_mean2, ln_rstd2, ln_dx,
                                                               ln_dg, ln_db, ln_ws), record)
        for k in range(mb):
            g = grads[k % GRAD_BUFFERS]
            if k == mb - 1:   # the last micro-batch also writes the norm's partial sums
                timed("grad_accumulate_last", lambda g=g, k=k: ops.bloom_bf16_grad_accumulate_sumsq(
                    acc, g, k == 0, opt_ws), record)
            else:
                name = "grad_accumulate_first" if k == 0 else "grad_accumulate"
                timed(name, lambda g=g, k=k: ops.bloom_bf16_grad_accumulate(acc, g, k == 0), record)
        hp = ops.adamw_hparams(W.LR, W.BETA1, W.BETA2, W.ADAM_EPS, W.WEIGHT_DECAY, W.MAX_GRAD_NORM, t,
                               sumsq_in_workspace=True)
        timed("adamw_step", lambda: ops.bloom_bf16_adamw_step(master, exp_avg, exp_avg_sq, param, acc, hp, norm,
                                                              opt_ws), record)

    t = 1
    for _ in range(args.warmup):
        step(t, False)
        t += 1
    torch.cuda.synchronize()
    log(f"bench: {args.warmup} warmup steps done; timing {args.steps} steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(t, True)
        t += 1
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    per = {}
    for k in names:
        ts = [a.elapsed_time(b) for a, b in ev[k]]
        per[k] = sum(ts) / len(ts)
    log(f"bench: {ms_step:.2f} ms/step; grad norm {norm.item():.4f}")
    shapes = {"ln": (rows, hid), "sm": (smb, smh, sms), "gelu": (grows, gcols)}
    return ms_step, per, bytes_model(shapes, n, mb), n, mb


# ----------------------------------------------------------------------------
def run_cpu_baseline(min_seconds_per_row: float = 1.5):
    """The oracle as it stands, timed on a bounded sample of each step row.

    Each row's oracle call is repeated until it has run for at least
    `min_seconds_per_row`; returns {row: (bytes per call, seconds per call)}.
    """
    import numpy as np
    from threadpoolctl import threadpool_limits

    import synth
    from synth import workloads as W
    from oracle import alibi as oal, gelu as og, layernorm as oln, optimizer as oopt

    X = W.SHARD
    hid, seq, gcols = X.ln.hidden, X.softmax.seq, X.gelu.cols
    r = {}

    def clock(name, nbytes, fn):
        reps, t0 = 0, time.perf_counter()
        while True:
            fn()
            reps += 1
            el = time.perf_counter() - t0
            if el >= min_seconds_per_row:
                break
        r[name] = (nbytes, el / reps)

    with threadpool_limits(limits=1):
        rows = 64
        x = synth.tensor(2, W.S_LN_X, rows * hid, 1.0, mode=synth.MODE_BF16).reshape(rows, hid)
        g = synth.tensor(2, W.S_LN_GAMMA, hid, 0.02, 1.0, mode=synth.MODE_BF16)
        b = synth.tensor(2, W.S_LN_BETA, hid, 0.02, mode=synth.MODE_BF16)
        dy = synth.tensor(2, W.S_LN_DY, rows * hid, 1.0, mode=synth.MODE_BF16).reshape(rows, hid)
        clock("layernorm_fwd", rows * hid * 4, lambda: oln.layernorm_fwd(x, g, b, W.LN_EPS))
        clock("layernorm_bwd", rows * hid * 6, lambda: oln.layernorm_bwd(dy, x, g, W.LN_EPS))

        srows = np.arange(0, 28 * seq, 28 * seq // 128)  # 128 rows spread over heads and positions
        sc = synth.values(2, W.S_SM_SCORES, srows[:, None] * seq + np.arange(seq)[None, :], 1.0,
                          mode=synth.MODE_BF16)
        i = srows % seq
        live = int((i + 1).sum())
        sl = oal.alibi_slopes_f32(112, 0, 28).astype(np.float64)[(srows // seq) % 28]
        sc32 = float(np.float32(X.softmax.scale))
        yb = oal.round_to_bf16(oal.softmax_fwd_f64(oal.to_f64(sc), i, sl, sc32))
        clock("alibi_softmax_fwd", live * 2 + len(srows) * seq * 2,
              lambda: oal.round_to_bf16(oal.softmax_fwd_f64(oal.to_f64(sc), i, sl, sc32)))
        clock("alibi_softmax_bwd", live * 4 + len(srows) * seq * 2,
              lambda: oal.round_to_bf16(oal.softmax_bwd_f64(oal.to_f64(yb), oal.to_f64(sc), i, sc32)[0]))

        grows = 64
        gx = synth.tensor(2, W.S_GELU_X, grows * gcols, 1.0, mode=synth.MODE_BF16).reshape(grows, gcols)
        gb = synth.tensor(2, W.S_GELU_BIAS, gcols, 0.02, mode=synth.MODE_BF16)
        clock("bias_gelu_fwd", grows * gcols * 4, lambda: og.bias_gelu_fwd(gx, gb))
        clock("bias_gelu_bwd", grows * gcols * 6, lambda: og.bias_gelu_bwd(gx, gx, gb))

        n = 1 << 22
        g1 = synth.tensor(4, 101, n, 1e-3, mode=synth.MODE_BF16)
        g2 = synth.tensor(4, 102, n, 1e-3, mode=synth.MODE_BF16)
        acc = oopt.grad_accumulate(None, g1, True)
        clock("grad_accumulate_first", n * 6, lambda: oopt.grad_accumulate(None, g1, True))
        clock("grad_accumulate", n * 10, lambda: oopt.grad_accumulate(acc, g2, False))
        p = synth.tensor(4, W.S_OPT_PARAM, n, 0.02)
        z = np.zeros(n, dtype=np.float32)
        clock("adamw_step", n * 30, lambda: oopt.bf16_optimizer_step(
            p, z, z, acc, W.LR, W.BETA1, W.BETA2, W.ADAM_EPS, W.WEIGHT_DECAY, W.MAX_GRAD_NORM, 1))
    return r


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--n", type=int, default=None, help="optimizer shard size (default 3.67e9)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the hot path runs on a single MI355X at one GPU's shard shape, "
              "and runs on several GPUs are not supported.", file=sys.stderr)
        sys.exit(2)

    ms_step, per, bts, n, mb = run_gpu(args)
    nfirst, nrest = 1, mb - 2
    step_bytes = (sum(bts[k] for k in ("layernorm_fwd", "layernorm_bwd", "alibi_softmax_fwd",
                                       "alibi_softmax_bwd", "bias_gelu_fwd", "bias_gelu_bwd", "adamw_step",
                                       "grad_accumulate_last"))
                  + nfirst * bts["grad_accumulate_first"] + nrest * bts["grad_accumulate"])
    kernels = {}
    for k, ms in per.items():
        gbs = bts[k] / (ms * 1e-3) / 1e9
        kernels[k] = {"ms": round(ms, 4), "GB/s": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
                      "algorithmic_bytes": bts[k]}
    dom = "grad_accumulate"
    dom_gbs = bts[dom] / (per[dom] * 1e-3) / 1e9
    traffic = measured_traffic(dom)
    result = {
        "metric": METRIC,
        "value": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": {"workload": "bloom176b-tp4-shard-step: layernorm fwd+bwd [2048,14336]; alibi causal softmax "
                               "fwd+bwd [1,28,2048,2048] (heads 0-27 of 112); bias-gelu fwd+bwd [2048,14336]; "
                               f"bf16-optimizer over a {n}-element shard with {mb} fp32-accumulated micro-batch "
                               "gradients, global-norm clip 1.0, adamw, rne bf16 copy",
                   "optimizer_elements": n, "microbatches": mb, "grad_buffers": GRAD_BUFFERS,
                   "storage": "bf16 activations and gradients, fp32 master/moments/accumulator"},
        "adamw_step_ms": round(per["adamw_step"], 3),
        "kernels": kernels,
        "roofline": {"kernel": "grad_accumulate (micro-batches 2-31)", "bound": "hbm",
                     "achieved": round(dom_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dom_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
    }
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle on a bounded sample")
        t0 = time.perf_counter()
        r = run_cpu_baseline()
        cpu_step_s = 0.0
        for k in ("layernorm_fwd", "layernorm_bwd", "alibi_softmax_fwd", "alibi_softmax_bwd", "bias_gelu_fwd",
                  "bias_gelu_bwd", "adamw_step"):
            bb, s = r[k]
            cpu_step_s += bts[k] / (bb / s)
        bb, s = r["grad_accumulate"]
        cpu_step_s += bts["grad_accumulate_last"] / (bb / s)
        bb, s = r["grad_accumulate_first"]
        cpu_step_s += nfirst * bts["grad_accumulate_first"] / (bb / s)
        bb, s = r["grad_accumulate"]
        cpu_step_s += nrest * bts["grad_accumulate"] / (bb / s)
        result["cpu_baseline"] = {
            "value": round(step_bytes / cpu_step_s / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": "NumPy float64 oracle, one thread: 64 LayerNorm rows and 64 bias-GeLU rows of width "
                      "14336, 128 softmax rows of length 2048 spread over the 28 heads, 4.2M optimizer elements "
                      "(one first and one later accumulation, one norm+clip+AdamW+bf16 step, credited with the step's "
                      "30 B/element), each repeated "
                      "for >= 1.5 s; each row's oracle rate is scaled to that row's bytes in the step "
                      f"({time.perf_counter() - t0:.1f} s of CPU time in all)",
            "step_seconds_extrapolated": round(cpu_step_s, 1)}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
