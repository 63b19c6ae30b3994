"""Benchmark: one BLOOM-176B TP=4 shard training step's hot path on one MI355X.

A step is one pass over every kernel of the path, on synthetic BLOOM-shaped
data already resident in HBM:

  LayerNorm fwd + bwd          [2048, 14336] bf16
  ALiBi causal softmax fwd+bwd [1, 28, 2048, 2048] bf16 (heads 0..27 of 112)
  bias + GeLU fwd + bwd        [2048, 14336] bf16
  FP32 gradient accumulation   one pass per pipeline micro-batch: 32 distinct
                               bf16 micro-batch gradients of a 3.67e9-element
                               shard, acc = g_1, then acc += g_k (k = 2..32);
                               the last pass also writes the norm's partial sums
  BF16Optimizer step           global norm, clip 1.0, AdamW, bf16 parameter copy

The micro-batch gradients are what the backward pass of each micro-batch
hands the optimizer; the backward's matrix products are not part of this
path, so each gradient is regenerated on the device from its own generator
stream (micro-batch k = stream 101 + k) into one of two 7.34 GB buffers,
two micro-batches ahead of its accumulation.  Those regenerations are not
timed: `ms_per_step` is the sum of the HIP-event durations of the path's own
launches in a step (six fused kernels, 32 accumulation passes, the AdamW
step), averaged over the timed steps; the wall time per step including the
regenerations is reported beside it.  Every kernel reads inputs that were last
touched at least one 7.34 GB write earlier, so none is served by the 256 MB
Infinity Cache.

Prints one JSON line.  `value` is the step's algorithmic HBM throughput (the
sum of each launch's algorithmic bytes / ms_per_step, GB/s).  Beside it:
per-kernel algorithmic GB/s and fraction of the 8 TB/s peak, the same as a
fraction of a plain streaming copy with the kernel's read/write pattern timed
the same way (`copy_ceilings`), the AdamW step time, a roofline entry for the
dominant kernel (the single-gradient accumulation pass, 30 of the 32 launches
per step), the 16-resident-gradient batched accumulation as a separately
labelled measurement, and the CPU oracle timed on the host's cores.  The fused
kernels (tens of microseconds, where an event pair adds a few) are also timed
after the steps in sweeps of back-to-back launches over rotating cold input
sets; the median of three sweeps is their per-kernel number.
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
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
MAX_ACCUM_BATCH = 16             # the library limit on micro-batches per batched pass
COUNTERS = os.path.join(ROOT, "profiles", "counters.json")
FUSED_STEP = ("layernorm_fwd", "layernorm_bwd", "alibi_softmax_fwd", "alibi_softmax_bwd", "bias_gelu_fwd",
              "bias_gelu_bwd")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------
# Algorithmic bytes of each step row (what the method must read and write).
def bytes_model(sh, n, mb, batch=MAX_ACCUM_BATCH):
    rows, hid = sh["ln"]
    b, h, s = sh["sm"]
    live = b * h * s * (s + 1) // 2          # causal entries read
    full = b * h * s * s                     # entries written
    grows, gcols = sh["gelu"]
    return {
        "layernorm_fwd": rows * hid * 4 + hid * 4 + rows * 8,
        "layernorm_bwd": rows * hid * 6 + hid * 2 + rows * 8 + hid * 4,
        # fused LayerNorm + residual: reads x, r and writes h, y / reads dy, dres, h and writes dh
        "layernorm_residual_fwd": rows * hid * 8 + hid * 4 + rows * 8,
        "layernorm_residual_bwd": rows * hid * 8 + hid * 2 + rows * 8 + hid * 4,
        # fused ALiBi attention forward: q, k, v read, o written (bf16), lse written (fp32)
        "alibi_attention_fwd": b * h * s * sh["head_dim"] * 2 * 4 + b * h * s * 4,
        # ... and its MFMA work: q.k and p.v take 2*D flops each per causal (query, key <= query) pair
        "_attention_flops": 2 * 2 * b * h * (s * (s + 1) // 2) * sh["head_dim"],
        # backward: q, k, v, dout read and dq, dk, dv written (bf16), lse read (fp32)
        "alibi_attention_bwd": b * h * s * sh["head_dim"] * 2 * 7 + b * h * s * 4,
        # ... five products per causal pair: q.k, dout.v, p^T.dout, ds.k, ds^T.q
        "_attention_bwd_flops": 5 * 2 * b * h * (s * (s + 1) // 2) * sh["head_dim"],
        "alibi_softmax_fwd": live * 2 + full * 2,
        "alibi_softmax_bwd": live * 4 + full * 2,
        "bias_gelu_fwd": grows * gcols * 4 + gcols * 2,
        "bias_gelu_bwd": grows * gcols * 6 + gcols * 4,
        "grad_accumulate_first": n * 6,
        "grad_accumulate": n * 10,
        "grad_accumulate_last": n * 10,  # also emits the norm's FP64 partials (1/1024 of a double per element)
        # `batch` resident micro-batch gradients per pass: read them once, read + write acc once
        "grad_accumulate_many_first": n * (2 * batch + 4),
        "grad_accumulate_many": n * (2 * batch + 8),
        "grad_accumulate_many_last": n * (2 * batch + 8),
        "adamw_step": n * 30,   # update reads acc, master, m, v (16 B), writes master, m, v, bf16 (14 B)
    }


def step_bytes(bts, mb):
    """Algorithmic bytes of one step: the six fused kernels, one accumulation
    pass per micro-batch (the first 6 B per element, each later one 10 B) and
    the AdamW step."""
    return (sum(bts[k] for k in FUSED_STEP) + bts["grad_accumulate_first"] + (mb - 2) * bts["grad_accumulate"]
            + bts["grad_accumulate_last"] + bts["adamw_step"])


def long_context_model(ln_rows, hidden, batch, heads, seq, head_dim):
    """Algorithmic bytes (and the attention's FLOP) of the 8192-token extrapolation rows."""
    live = batch * heads * seq * (seq + 1) // 2
    rows = batch * heads * seq
    return {
        # the embedding LayerNorm forward at the extrapolation length
        "layernorm_fwd_8192": ln_rows * hidden * 4 + hidden * 4 + ln_rows * 8,
        # causal softmax forward: the causal half read, the full rows written
        "alibi_softmax_fwd_8192": live * 2 + batch * heads * seq * seq * 2,
        "alibi_attention_fwd_8192": rows * head_dim * 2 * 4 + rows * 4,
        "_attention_flops_8192": 2 * 2 * live * head_dim,
    }


def mini_model():
    """Algorithmic bytes of the mini-BLOOM rows (the same models at the mini shapes)."""
    from synth import workloads as W
    mi = W.MINI
    shapes = {"ln": (mi.ln.rows, mi.ln.hidden), "sm": (mi.softmax.batch, mi.softmax.heads, mi.softmax.seq),
              "gelu": (mi.gelu.rows, mi.gelu.cols), "head_dim": mi.softmax.head_dim}
    m = bytes_model(shapes, mi.opt.n, 32)
    keys = ("layernorm_fwd", "layernorm_bwd", "alibi_softmax_fwd", "alibi_softmax_bwd", "bias_gelu_fwd",
            "bias_gelu_bwd", "adamw_step")
    return {k + "_mini": m[k] for k in keys}


def copy_patterns(sh, n):
    """The plain-copy pattern (inputs, outputs, bytes per stream) each kernel is compared with.

    A kernel's ceiling is a streaming copy that reads and writes what it does:
    LayerNorm and GeLU forward one [rows, H] bf16 stream in and one out, their
    backwards two in and one out; the causal softmax forward reads the causal
    half (one stream of causal entries) and writes full rows (two such
    streams), its backward reads two causal streams; the optimizer passes are
    compared with a flat copy of the FP32 accumulator.
    """
    rows, hid = sh["ln"]
    b, h, s = sh["sm"]
    act = rows * hid * 2
    causal = b * h * s * (s + 1) // 2 * 2
    causal -= causal % 16
    return {
        "1in_1out_act": (1, 1, act),
        "2in_1out_act": (2, 1, act),
        "1in_2out_causal": (1, 2, causal),
        "2in_2out_causal": (2, 2, causal),
        "1in_1out_fp32_shard": (1, 1, n * 4 - (n * 4) % 16),
    }


CEILING_OF = {"layernorm_fwd": "1in_1out_act", "bias_gelu_fwd": "1in_1out_act",
              "layernorm_bwd": "2in_1out_act", "bias_gelu_bwd": "2in_1out_act",
              "alibi_softmax_fwd": "1in_2out_causal", "alibi_softmax_bwd": "2in_2out_causal",
              "grad_accumulate_first": "1in_1out_fp32_shard", "grad_accumulate": "1in_1out_fp32_shard",
              "grad_accumulate_last": "1in_1out_fp32_shard", "adamw_step": "1in_1out_fp32_shard"}


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
# The CPU oracle, timed on the host's cores.
def cpu_share():
    """Cores the oracle may use: the process's CPU affinity, capped by the
    thread allotment OMP_NUM_THREADS states (a job scheduler that shares a
    host between GPUs sets it to the job's CPU share)."""
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:
        aff = os.cpu_count() or 1
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        return min(aff, int(omp))
    return aff


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _cpu_worker(w, nw, barrier, queue, opt_elems):
    """One worker of the oracle pool: its share of every step row, each timed
    between two barriers so that all workers run the row at once."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import synth
    from synth import workloads as W
    from oracle import alibi as oal, gelu as og, layernorm as oln, optimizer as oopt

    out = {}
    try:
        with threadpool_limits(limits=1):
            X, O = W.SHARD, W.OPTIMIZER
            seed = X.seed

            def timed(name, fn, reps=1):
                barrier.wait(timeout=900)
                t0 = time.perf_counter()
                for _ in range(reps):
                    r = fn()
                out[name] = (time.perf_counter() - t0) / reps
                barrier.wait(timeout=900)
                return r

            def rows_of(total):
                lo = total * w // nw
                return lo, total * (w + 1) // nw

            def bf16_rows(stream, lo, hi, width, sigma=1.0):
                idx = np.arange(lo * width, hi * width, dtype=np.uint64)
                return synth.values(seed, stream, idx, sigma, mode=synth.MODE_BF16).reshape(hi - lo, width)

            hid = X.ln.hidden
            g = synth.tensor(seed, W.S_LN_GAMMA, hid, 0.02, 1.0, mode=synth.MODE_BF16)
            b = synth.tensor(seed, W.S_LN_BETA, hid, 0.02, mode=synth.MODE_BF16)
            lo, hi = rows_of(X.ln.rows)
            x = bf16_rows(W.S_LN_X, lo, hi, hid)
            dy = bf16_rows(W.S_LN_DY, lo, hi, hid)
            timed("layernorm_fwd", lambda: oln.layernorm_fwd(x, g, b, W.LN_EPS))
            timed("layernorm_bwd", lambda: oln.layernorm_bwd(dy, x, g, W.LN_EPS))
            del x, dy

            sm = X.softmax
            seq = sm.seq
            lo, hi = rows_of(sm.batch * sm.heads * seq)
            sc = bf16_rows(W.S_SM_SCORES, lo, hi, seq)
            dp = bf16_rows(W.S_SM_DPROBS, lo, hi, seq)
            flat = np.arange(lo, hi, dtype=np.int64)
            slopes = oal.alibi_slopes_f32(sm.total_heads, sm.head_offset, sm.heads).astype(np.float64)
            sc32 = float(np.float32(sm.scale))
            chunk = max(1, (1 << 22) // seq)

            def sm_fwd():
                y = np.empty_like(sc)
                for c in range(0, len(flat), chunk):
                    r = flat[c:c + chunk]
                    y[c:c + len(r)] = oal.round_to_bf16(oal.softmax_fwd_f64(
                        oal.to_f64(sc[c:c + len(r)]), r % seq, slopes[(r // seq) % sm.heads], sc32))
                return y

            def sm_bwd(y):
                ds = np.empty_like(y)
                for c in range(0, len(flat), chunk):
                    r = flat[c:c + chunk]
                    ds[c:c + len(r)] = oal.round_to_bf16(oal.softmax_bwd_f64(
                        oal.to_f64(y[c:c + len(r)]), oal.to_f64(dp[c:c + len(r)]), r % seq, sc32)[0])
                return ds

            y = timed("alibi_softmax_fwd", sm_fwd)
            timed("alibi_softmax_bwd", lambda: sm_bwd(y))
            del sc, dp, y

            gcols = X.gelu.cols
            gb = synth.tensor(seed, W.S_GELU_BIAS, gcols, 0.02, mode=synth.MODE_BF16)
            lo, hi = rows_of(X.gelu.rows)
            gx = bf16_rows(W.S_GELU_X, lo, hi, gcols)
            gdy = bf16_rows(W.S_GELU_DY, lo, hi, gcols)
            timed("bias_gelu_fwd", lambda: og.bias_gelu_fwd(gx, gb))
            timed("bias_gelu_bwd", lambda: og.bias_gelu_bwd(gdy, gx, gb))
            del gx, gdy

            # the optimizer rows on this worker's slice of the shard
            start = w * opt_elems
            g1 = synth.tensor(O.seed, W.S_OPT_GRAD0 + 1, opt_elems, W.GRAD_SIGMA, mode=synth.MODE_BF16, start=start)
            g2 = synth.tensor(O.seed, W.S_OPT_GRAD0 + 2, opt_elems, W.GRAD_SIGMA, mode=synth.MODE_BF16, start=start)
            p = synth.tensor(O.seed, W.S_OPT_PARAM, opt_elems, W.PARAM_SIGMA, start=start)
            z = np.zeros(opt_elems, dtype=np.float32)
            acc = timed("grad_accumulate_first", lambda: oopt.grad_accumulate(None, g1, True), reps=5)
            timed("grad_accumulate", lambda: oopt.grad_accumulate(acc, g2, False), reps=5)
            timed("adamw_step", lambda: oopt.bf16_optimizer_step(
                p, z, z, acc, W.LR, W.BETA1, W.BETA2, W.ADAM_EPS, W.WEIGHT_DECAY, W.MAX_GRAD_NORM, 1), reps=2)
        queue.put((w, out, None))
    except Exception as e:  # reported by the parent; the barrier is broken so the others stop too
        barrier.abort()
        queue.put((w, out, repr(e)))


def run_cpu_baseline(workers, opt_elems):
    """Runs the oracle over the step's rows with `workers` processes.

    Returns {row: wall seconds (the slowest worker, all started together)}.
    The six fused rows cover the whole [2048, 14336] / [1, 28, 2048, 2048]
    shapes; the optimizer rows cover workers * opt_elems elements of the shard.
    Called before the GPU is touched, so the forked workers inherit no GPU state.
    """
    import multiprocessing as mp

    ctx = mp.get_context("fork")
    barrier = ctx.Barrier(workers)
    queue = ctx.Queue()
    procs = [ctx.Process(target=_cpu_worker, args=(w, workers, barrier, queue, opt_elems)) for w in range(workers)]
    for p in procs:
        p.start()
    results, errors = {}, []
    for _ in procs:
        w, out, err = queue.get(timeout=1800)
        if err:
            errors.append(f"worker {w}: {err}")
        for k, v in out.items():
            results[k] = max(results.get(k, 0.0), v)
    for p in procs:
        p.join(timeout=60)
    if errors:
        raise RuntimeError("; ".join(errors))
    return results


# ----------------------------------------------------------------------------
def run_gpu(args):
    import torch

    from bloom_bf16_optimizer_amd import ops
    from synth import device as sdev
    from synth import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy:
        # A plain copy of known size: its FETCH_SIZE / WRITE_SIZE counter values
        # against 1 GiB give the scale for the counter-measured traffic.
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    X = W.SHARD
    O = W.OPTIMIZER
    n = O.opt.n if args.n is None else args.n
    mb = O.opt.microbatches
    assert mb % 2 == 0, "the two gradient buffers alternate by micro-batch parity"
    rows, hid = X.ln.rows, X.ln.hidden
    smb, smh, sms = X.softmax.batch, X.softmax.heads, X.softmax.seq
    grows, gcols = X.gelu.rows, X.gelu.cols
    bf, f32 = torch.bfloat16, torch.float32
    seed = X.seed
    scale = X.softmax.scale

    def fill(shape, stream, sigma, offset=0.0, dtype=bf, s=0, sd=None):
        t = torch.empty(shape, dtype=dtype, device=dev)
        sdev.fill_(t, (seed if sd is None else sd) + 1000 * s, stream, sigma, offset)
        return t

    ln_g = fill((hid,), W.S_LN_GAMMA, 0.02, 1.0)
    ln_b = fill((hid,), W.S_LN_BETA, 0.02)
    ge_b = fill((gcols,), W.S_GELU_BIAS, 0.02)

    # Each fused kernel gets its own input set(s): set 0 runs in the step,
    # sets 0..S-1 rotate in the per-kernel sweep so every launch reads cold data.
    def ln_fwd_set(s):
        x = fill((rows, hid), W.S_LN_X, 1.0, s=s)
        y = torch.empty_like(x)
        m = torch.empty(rows, dtype=f32, device=dev)
        r = torch.empty_like(m)
        return lambda: ops.bloom_layernorm_fwd(x, ln_g, ln_b, y, m, r, W.LN_EPS)

    def ln_bwd_set(s):
        x = fill((rows, hid), 50, 1.0, s=s)
        dy = fill((rows, hid), W.S_LN_DY, 1.0, s=s)
        dx = torch.empty_like(x)
        m = torch.empty(rows, dtype=f32, device=dev)
        r = torch.empty_like(m)
        ops.bloom_layernorm_fwd(x, ln_g, ln_b, dx, m, r, W.LN_EPS)   # saved statistics for the backward
        dg = torch.empty(hid, dtype=bf, device=dev)
        db = torch.empty_like(dg)
        ws = torch.empty(ops.bloom_layernorm_bwd_workspace_size(rows, hid), dtype=torch.uint8, device=dev)
        return lambda: ops.bloom_layernorm_bwd(dy, x, ln_g, m, r, dx, dg, db, ws)

    def sm_fwd_set(s):
        sc = fill((smb, smh, sms, sms), W.S_SM_SCORES, 1.0, s=s)
        p = torch.empty_like(sc)
        return lambda: ops.bloom_alibi_softmax_fwd(sc, p, X.softmax.head_offset, X.softmax.total_heads, scale)

    def sm_bwd_set(s):
        sc = fill((smb, smh, sms, sms), 51, 1.0, s=s)
        y = torch.empty_like(sc)
        ops.bloom_alibi_softmax_fwd(sc, y, X.softmax.head_offset, X.softmax.total_heads, scale)
        del sc
        dy = fill((smb, smh, sms, sms), W.S_SM_DPROBS, 1.0, s=s)
        ds = torch.empty_like(y)
        return lambda: ops.bloom_alibi_softmax_bwd(y, dy, ds, scale)

    def ge_fwd_set(s):
        x = fill((grows, gcols), W.S_GELU_X, 1.0, s=s)
        y = torch.empty_like(x)
        return lambda: ops.bloom_bias_gelu_fwd(x, ge_b, y)

    def ge_bwd_set(s):
        x = fill((grows, gcols), 52, 1.0, s=s)
        dy = fill((grows, gcols), W.S_GELU_DY, 1.0, s=s)
        dx = torch.empty_like(x)
        db = torch.empty(gcols, dtype=bf, device=dev)
        ws = torch.empty(ops.bloom_bias_gelu_bwd_workspace_size(grows, gcols), dtype=torch.uint8, device=dev)
        return lambda: ops.bloom_bias_gelu_bwd(dy, x, ge_b, dx, db, ws)

    def lnr_fwd_set(s):
        x = fill((rows, hid), W.S_LN_X, 1.0, s=s)
        res = fill((rows, hid), W.S_LN_RES, 1.0, s=s)
        h, y = torch.empty_like(x), torch.empty_like(x)
        m = torch.empty(rows, dtype=f32, device=dev)
        r = torch.empty_like(m)
        return lambda: ops.bloom_layernorm_residual_fwd(x, res, ln_g, ln_b, h, y, m, r, W.LN_EPS)

    def lnr_bwd_set(s):
        h = fill((rows, hid), 53, 1.0, s=s)
        dy = fill((rows, hid), W.S_LN_DY, 1.0, s=s)
        dres = fill((rows, hid), W.S_LN_DRES, 1.0, s=s)
        dh = torch.empty_like(h)
        m = torch.empty(rows, dtype=f32, device=dev)
        r = torch.empty_like(m)
        ops.bloom_layernorm_fwd(h, ln_g, ln_b, dh, m, r, W.LN_EPS)   # saved statistics for the backward
        dg = torch.empty(hid, dtype=bf, device=dev)
        db = torch.empty_like(dg)
        ws = torch.empty(ops.bloom_layernorm_bwd_workspace_size(rows, hid), dtype=torch.uint8, device=dev)
        return lambda: ops.bloom_layernorm_residual_bwd(dy, dres, h, ln_g, m, r, dh, dg, db, ws)

    fused = [("layernorm_fwd", ln_fwd_set, 4), ("alibi_softmax_fwd", sm_fwd_set, 2),
             ("bias_gelu_fwd", ge_fwd_set, 4), ("bias_gelu_bwd", ge_bwd_set, 4),
             ("alibi_softmax_bwd", sm_bwd_set, 2), ("layernorm_bwd", ln_bwd_set, 4)]
    step_fused = [(name, make(0)) for name, make, _ in fused]
    # Kernels measured in the sweep only (not rows of the step).
    hd = X.softmax.head_dim

    def att_fwd_set(s):
        q = fill((smb, smh, sms, hd), W.S_ATT_Q, 1.0, s=s)
        k = fill((smb, smh, sms, hd), W.S_ATT_K, 1.0, s=s)
        v = fill((smb, smh, sms, hd), W.S_ATT_V, 1.0, s=s)
        o = torch.empty_like(q)
        lse = torch.empty((smb, smh, sms), dtype=f32, device=dev)
        return lambda: ops.bloom_alibi_attention_fwd(q, k, v, o, lse, X.softmax.head_offset, X.softmax.total_heads,
                                                     scale)

    def att_bwd_set(s):
        q = fill((smb, smh, sms, hd), W.S_ATT_Q, 1.0, s=s)
        k = fill((smb, smh, sms, hd), W.S_ATT_K, 1.0, s=s)
        v = fill((smb, smh, sms, hd), W.S_ATT_V, 1.0, s=s)
        do = fill((smb, smh, sms, hd), W.S_ATT_DO, 1.0, s=s)
        o = torch.empty_like(q)
        lse = torch.empty((smb, smh, sms), dtype=f32, device=dev)
        ops.bloom_alibi_attention_fwd(q, k, v, o, lse, X.softmax.head_offset, X.softmax.total_heads, scale)
        del o
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        ws = torch.empty(ops.bloom_alibi_attention_bwd_workspace_size(smb, smh, sms), dtype=torch.uint8, device=dev)
        return lambda: ops.bloom_alibi_attention_bwd(q, k, v, do, lse, dq, dk, dv, X.softmax.head_offset,
                                                     X.softmax.total_heads, scale, ws)

    L = W.LONG.softmax  # the 8192-token extrapolation shape, 28 heads

    def att_fwd_long_set(s):
        q = fill((L.batch, L.heads, L.seq, L.head_dim), W.S_ATT_Q, 1.0, s=s)
        k = fill((L.batch, L.heads, L.seq, L.head_dim), W.S_ATT_K, 1.0, s=s)
        v = fill((L.batch, L.heads, L.seq, L.head_dim), W.S_ATT_V, 1.0, s=s)
        o = torch.empty_like(q)
        lse = torch.empty((L.batch, L.heads, L.seq), dtype=f32, device=dev)
        return lambda: ops.bloom_alibi_attention_fwd(q, k, v, o, lse, L.head_offset, L.total_heads, L.scale)

    LW = W.LONG  # the 8192-token extrapolation: embedding LayerNorm and causal softmax forward

    def ln_fwd_long_set(s):
        x = fill((LW.ln.rows, LW.ln.hidden), W.S_LN_X, 1.0, s=s)
        y = torch.empty_like(x)
        m = torch.empty(LW.ln.rows, dtype=f32, device=dev)
        r = torch.empty_like(m)
        return lambda: ops.bloom_layernorm_fwd(x, ln_g, ln_b, y, m, r, W.LN_EPS)

    def sm_fwd_long_set(s):
        ls = LW.softmax
        sc = fill((ls.batch, ls.heads, ls.seq, ls.seq), W.S_SM_SCORES, 1.0, s=s)   # 3.76 GB
        p = torch.empty_like(sc)
        return lambda: ops.bloom_alibi_softmax_fwd(sc, p, ls.head_offset, ls.total_heads, ls.scale)

    # The mini-BLOOM layer (hidden 2048, 16 heads, FFN 8192, seq 2048, micro-batch 4): sweep-only rows.
    MI = W.MINI
    mrows, mhid = MI.ln.rows, MI.ln.hidden
    msm = MI.softmax
    mgrows, mgcols = MI.gelu.rows, MI.gelu.cols
    m_g = fill((mhid,), W.S_LN_GAMMA, 0.02, 1.0)
    m_b = fill((mhid,), W.S_LN_BETA, 0.02)
    m_gb = fill((mgcols,), W.S_GELU_BIAS, 0.02)

    def m_ln_fwd_set(s):
        x = fill((mrows, mhid), W.S_LN_X, 1.0, s=s)
        y = torch.empty_like(x)
        m = torch.empty(mrows, dtype=f32, device=dev)
        r = torch.empty_like(m)
        return lambda: ops.bloom_layernorm_fwd(x, m_g, m_b, y, m, r, W.LN_EPS)

    def m_ln_bwd_set(s):
        x = fill((mrows, mhid), 50, 1.0, s=s)
        dy = fill((mrows, mhid), W.S_LN_DY, 1.0, s=s)
        dx = torch.empty_like(x)
        m = torch.empty(mrows, dtype=f32, device=dev)
        r = torch.empty_like(m)
        ops.bloom_layernorm_fwd(x, m_g, m_b, dx, m, r, W.LN_EPS)
        dg, db = torch.empty(mhid, dtype=bf, device=dev), torch.empty(mhid, dtype=bf, device=dev)
        ws = torch.empty(ops.bloom_layernorm_bwd_workspace_size(mrows, mhid), dtype=torch.uint8, device=dev)
        return lambda: ops.bloom_layernorm_bwd(dy, x, m_g, m, r, dx, dg, db, ws)

    def m_sm_fwd_set(s):
        sc = fill((msm.batch, msm.heads, msm.seq, msm.seq), W.S_SM_SCORES, 1.0, s=s)
        p = torch.empty_like(sc)
        return lambda: ops.bloom_alibi_softmax_fwd(sc, p, msm.head_offset, msm.total_heads, msm.scale)

    def m_sm_bwd_set(s):
        sc = fill((msm.batch, msm.heads, msm.seq, msm.seq), 51, 1.0, s=s)
        y = torch.empty_like(sc)
        ops.bloom_alibi_softmax_fwd(sc, y, msm.head_offset, msm.total_heads, msm.scale)
        del sc
        dy = fill((msm.batch, msm.heads, msm.seq, msm.seq), W.S_SM_DPROBS, 1.0, s=s)
        ds = torch.empty_like(y)
        return lambda: ops.bloom_alibi_softmax_bwd(y, dy, ds, msm.scale)

    def m_ge_fwd_set(s):
        x = fill((mgrows, mgcols), W.S_GELU_X, 1.0, s=s)
        y = torch.empty_like(x)
        return lambda: ops.bloom_bias_gelu_fwd(x, m_gb, y)

    def m_ge_bwd_set(s):
        x = fill((mgrows, mgcols), 52, 1.0, s=s)
        dy = fill((mgrows, mgcols), W.S_GELU_DY, 1.0, s=s)
        dx = torch.empty_like(x)
        db = torch.empty(mgcols, dtype=bf, device=dev)
        ws = torch.empty(ops.bloom_bias_gelu_bwd_workspace_size(mgrows, mgcols), dtype=torch.uint8, device=dev)
        return lambda: ops.bloom_bias_gelu_bwd(dy, x, m_gb, dx, db, ws)

    def m_adamw_set(s):
        # the mini model's 1,722,400,768 parameters as slices of the shard's buffers (timed after the
        # steps); one accumulation pass over the slice leaves the norm's partial sums in the workspace
        nm = MI.opt.n
        ws = torch.empty(ops.bloom_bf16_adamw_workspace_size(nm), dtype=torch.uint8, device=dev)
        ops.bloom_bf16_grad_accumulate_sumsq(acc[:nm], grads[0][:nm], True, ws)
        hp = ops.adamw_hparams(W.LR, W.BETA1, W.BETA2, W.ADAM_EPS, W.WEIGHT_DECAY, W.MAX_GRAD_NORM, MI.opt.step,
                               sumsq_in_workspace=True)
        return lambda: ops.bloom_bf16_adamw_step(master[:nm], exp_avg[:nm], exp_avg_sq[:nm], param[:nm], acc[:nm], hp,
                                                 norm, ws)

    sweep_only = [("layernorm_residual_fwd", lnr_fwd_set, 4), ("layernorm_residual_bwd", lnr_bwd_set, 4),
                  ("alibi_attention_fwd", att_fwd_set, 4), ("alibi_attention_fwd_8192", att_fwd_long_set, 2),
                  ("alibi_attention_bwd", att_bwd_set, 4), ("layernorm_fwd_8192", ln_fwd_long_set, 4),
                  ("alibi_softmax_fwd_8192", sm_fwd_long_set, 2),
                  ("layernorm_fwd_mini", m_ln_fwd_set, 4), ("layernorm_bwd_mini", m_ln_bwd_set, 4),
                  ("alibi_softmax_fwd_mini", m_sm_fwd_set, 2), ("alibi_softmax_bwd_mini", m_sm_bwd_set, 2),
                  ("bias_gelu_fwd_mini", m_ge_fwd_set, 4), ("bias_gelu_bwd_mini", m_ge_bwd_set, 4)]
    if n >= MI.opt.n:   # the mini model's update runs on slices of the shard's buffers
        sweep_only.append(("adamw_step_mini", m_adamw_set, 1))

    log(f"bench: allocating the shard workload (n = {n:,}; two gradient buffers)")
    master = fill((n,), W.S_OPT_PARAM, W.PARAM_SIGMA, dtype=f32, sd=O.seed)
    exp_avg = torch.zeros(n, dtype=f32, device=dev)
    exp_avg_sq = torch.zeros(n, dtype=f32, device=dev)
    acc = torch.empty(n, dtype=f32, device=dev)
    param = torch.empty(n, dtype=bf, device=dev)
    grads = [torch.empty(n, dtype=bf, device=dev) for _ in range(2)]
    norm = torch.empty(1, dtype=f32, device=dev)
    opt_ws = torch.empty(ops.bloom_bf16_adamw_workspace_size(n), dtype=torch.uint8, device=dev)

    def make_grad(k):
        # micro-batch k's gradient (what its backward pass would hand over), into buffer k % 2
        sdev.fill_(grads[k % 2], O.seed, W.S_OPT_GRAD0 + 1 + k, W.GRAD_SIGMA)

    make_grad(0)
    make_grad(1)
    torch.cuda.synchronize()
    log(f"bench: resident {torch.cuda.memory_allocated() / 2**30:.1f} GiB")

    path = [name for name, _ in step_fused] + ["grad_accumulate_first", "grad_accumulate", "grad_accumulate_last",
                                               "adamw_step"]
    step_events = []

    def timed(events, name, fn):
        if events is None:
            fn()
            return
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        events.append((name, a, b))

    def step(t, events):
        for name, fn in step_fused:
            timed(events, name, fn)
        for k in range(mb):
            g = grads[k % 2]
            if k == mb - 1:   # the last micro-batch also writes the norm's partial sums
                timed(events, "grad_accumulate_last",
                      lambda g=g: ops.bloom_bf16_grad_accumulate_sumsq(acc, g, False, opt_ws))
            else:
                timed(events, "grad_accumulate_first" if k == 0 else "grad_accumulate",
                      lambda g=g, k=k: ops.bloom_bf16_grad_accumulate(acc, g, k == 0))
            # the buffer is free again: micro-batch k + 2's gradient goes into it (after the last two
            # micro-batches, the next step's first two); not timed
            make_grad((k + 2) % mb)
        hp = ops.adamw_hparams(W.LR, W.BETA1, W.BETA2, W.ADAM_EPS, W.WEIGHT_DECAY, W.MAX_GRAD_NORM, t,
                               sumsq_in_workspace=True)
        timed(events, "adamw_step", lambda: ops.bloom_bf16_adamw_step(master, exp_avg, exp_avg_sq, param, acc, hp,
                                                                      norm, opt_ws))

    t = 1
    for _ in range(args.warmup):
        step(t, None)
        t += 1
    torch.cuda.synchronize()
    log(f"bench: {args.warmup} warmup steps done; timing {args.steps} steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        ev = []
        step(t, ev)
        step_events.append(ev)
        t += 1
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    per_step, samples = [], {k: [] for k in path}
    for ev in step_events:
        tot = 0.0
        for name, a, b in ev:
            ms = a.elapsed_time(b)
            samples[name].append(ms)
            tot += ms
        per_step.append(tot)
    ms_step = sum(per_step) / len(per_step)
    in_step = {k: sum(v) / len(v) for k, v in samples.items() if v}
    launches = {k: len(v) // args.steps for k, v in samples.items()}
    grad_norm = float(norm.item())
    log(f"bench: {ms_step:.2f} ms/step in the path's launches ({wall_ms:.1f} ms wall with the gradient "
        f"regeneration); grad norm {grad_norm:.4f}")

    # Per-kernel sweep of the fused kernels: R back-to-back launches rotating
    # over S cold input sets between one pair of events, so the per-launch
    # event overhead (a few microseconds) is amortised; three such sweeps per
    # kernel, the median reported (and the fastest kept beside it).
    reps, trials = 24, 3

    def sweep_fns(fns):
        sets = len(fns)
        for fn in fns:
            fn()
        torch.cuda.synchronize()
        per_launch = []
        for _ in range(trials):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            for r in range(reps):
                fns[r % sets]()
            b.record()
            b.synchronize()
            per_launch.append(a.elapsed_time(b) / reps)
        per_launch.sort()
        return per_launch[len(per_launch) // 2], per_launch[0]

    sweep, sweep_min = {}, {}
    for name, make, sets in ([] if args.no_sweep else fused + sweep_only):
        if name in dict(step_fused):
            fns = [dict(step_fused)[name]] + [make(s) for s in range(1, sets)]
        else:
            fns = [make(s) for s in range(sets)]
        sweep[name], sweep_min[name] = sweep_fns(fns)
        del fns

    shapes = {"ln": (rows, hid), "sm": (smb, smh, sms), "gelu": (grows, gcols), "head_dim": hd}

    # Copy ceilings: the plain streaming copy with each kernel's read/write
    # pattern, timed the same way (sweeps over 4 rotating cold sets for the
    # activation-sized patterns; three launches over the shard's accumulator).
    ceilings = {}
    if not args.no_sweep:
        for key, (nin, nout, nbytes) in copy_patterns(shapes, n).items():
            if key == "1in_1out_fp32_shard":
                src, dst = acc, exp_avg   # the step's state is no longer needed
                fns = [lambda: sdev.stream_copy([dst], [src])]
                ms, ms_min = sweep_fns(fns)
            else:
                bufs = []
                for s in range(4):
                    ins = [torch.ones(nbytes, dtype=torch.uint8, device=dev) for _ in range(nin)]
                    outs = [torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(nout)]
                    bufs.append((outs, ins))
                fns = [lambda o=o, i=i: sdev.stream_copy(o, i) for o, i in bufs]
                ms, ms_min = sweep_fns(fns)
                del bufs, fns
            moved = (nin + nout) * nbytes
            ceilings[key] = {"inputs": nin, "outputs": nout, "bytes_per_stream": nbytes, "ms": round(ms, 4),
                             "GB/s": round(moved / (ms * 1e-3) / 1e9, 1),
                             "frac_of_peak": round(moved / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}

    # The batched schedule: `K` micro-batch gradients resident at once, added
    # in one pass (bit-identical to K single passes).  It needs K * 7.34 GB of
    # gradients resident, which a pipeline step does not hold; measured and
    # reported beside the step, not as it.
    batched = None
    kb = args.accum_batch
    if kb > 0:
        extra = [torch.empty(n, dtype=bf, device=dev) for _ in range(kb - 2)]
        gbufs = grads + extra
        for k in range(kb):
            sdev.fill_(gbufs[k], O.seed, W.S_OPT_GRAD0 + 1 + k, W.GRAD_SIGMA)
        torch.cuda.synchronize()
        tb = {"first": [], "later": []}
        for _ in range(3):
            for key, first, wsp in (("first", True, None), ("later", False, opt_ws)):
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record()
                ops.bloom_bf16_grad_accumulate_many(acc, gbufs, first, wsp)
                b.record()
                tb[key].append((a, b))
        torch.cuda.synchronize()
        bm = bytes_model(shapes, n, mb, kb)
        ms_first = sum(a.elapsed_time(b) for a, b in tb["first"]) / 3
        ms_later = sum(a.elapsed_time(b) for a, b in tb["later"]) / 3
        passes = mb // kb
        batched = {
            "schedule": f"{kb} micro-batch gradients resident per pass, {passes} passes for {mb} micro-batches "
                        f"(bloom_bf16_grad_accumulate_many); needs {kb * n * 2 / 1e9:.1f} GB of bf16 gradients "
                        f"resident at once, which one pipeline micro-batch at a time does not provide; measured on "
                        f"{kb} distinct gradients (the later pass re-adds the same buffers), not the step's schedule",
            "resident_gradient_bytes": kb * n * 2,
            "first_pass_ms": round(ms_first, 3),
            "first_pass_GB/s": round(bm["grad_accumulate_many_first"] / (ms_first * 1e-3) / 1e9, 1),
            "later_pass_with_norm_partials_ms": round(ms_later, 3),
            "later_pass_GB/s": round(bm["grad_accumulate_many_last"] / (ms_later * 1e-3) / 1e9, 1),
            "accumulation_ms_for_32_microbatches": round(ms_first + (passes - 1) * ms_later, 3),
            "per_microbatch_accumulation_ms_in_step": round(in_step["grad_accumulate_first"] + in_step["grad_accumulate"]
                                                            * (mb - 2) + in_step["grad_accumulate_last"], 3),
        }
        del extra, gbufs

    bts = bytes_model(shapes, n, mb)
    bts.update(long_context_model(W.LONG.ln.rows, W.LONG.ln.hidden, L.batch, L.heads, L.seq, L.head_dim))
    bts.update(mini_model())
    return dict(ms_step=ms_step, wall_ms=wall_ms, in_step=in_step, launches=launches, sweep=sweep,
                sweep_min=sweep_min, ceilings=ceilings, batched=batched, bts=bts, n=n, mb=mb, grad_norm=grad_norm,
                shapes=shapes)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--n", type=int, default=None, help="optimizer shard size (default 3.67e9)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-workers", type=int, default=None,
                    help="oracle worker processes (default: the CPU share, see cpu_share())")
    ap.add_argument("--cpu-opt-elems", type=int, default=1 << 22,
                    help="optimizer elements per oracle worker (the sample of the 3.67e9 shard)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run 3 plain 1 GiB device-to-device copies (counter calibration)")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the per-kernel sweeps and the copy ceilings")
    ap.add_argument("--accum-batch", type=int, default=MAX_ACCUM_BATCH,
                    help="resident gradients per pass in the separately reported batched accumulation (0: skip it)")
    args = ap.parse_args()
    if args.accum_batch != 0 and not (2 <= args.accum_batch <= MAX_ACCUM_BATCH and 32 % (2 * args.accum_batch) == 0):
        print(f"--accum-batch must be 0 or divide the 32 micro-batches into at least two passes of at most "
              f"{MAX_ACCUM_BATCH} (2, 4, 8, 16)", file=sys.stderr)
        sys.exit(2)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the hot path runs on a single MI355X at one GPU's shard shape, "
              "and runs on several GPUs are not supported.", file=sys.stderr)
        sys.exit(2)

    cpu = None
    if not args.no_cpu_baseline:
        workers = args.cpu_workers or cpu_share()
        log(f"bench: timing the CPU oracle with {workers} worker processes")
        t0 = time.perf_counter()
        try:
            cpu = (workers, run_cpu_baseline(workers, args.cpu_opt_elems), time.perf_counter() - t0, None)
        except Exception as e:   # reported in the line; the GPU measurement still runs
            cpu = (workers, None, time.perf_counter() - t0, repr(e))
        log(f"bench: CPU oracle leg took {cpu[2]:.1f} s")

    g = run_gpu(args)
    bts, n, mb, in_step, sweep = g["bts"], g["n"], g["mb"], g["in_step"], g["sweep"]
    per = dict(in_step)
    per.update(sweep)
    total_bytes = step_bytes(bts, mb)
    kernels = {}
    for k, ms in per.items():
        gbs = bts[k] / (ms * 1e-3) / 1e9
        kernels[k] = {"ms": round(ms, 4), "GB/s": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
                      "algorithmic_bytes": bts[k],
                      "timing": "median of 3 sweeps of 24 back-to-back launches on rotating cold inputs"
                      if k in sweep else "events around each launch in the timed steps"}
        if k in g["launches"]:
            kernels[k]["launches_per_step"] = g["launches"][k]
        if k in sweep:
            kernels[k]["min_sweep_ms"] = round(g["sweep_min"][k], 4)
            kernels[k]["in_step_ms"] = round(in_step[k], 4) if k in in_step else None
        ck = CEILING_OF.get(k)
        if ck and ck in g["ceilings"]:
            kernels[k]["frac_of_copy_ceiling"] = round(gbs / g["ceilings"][ck]["GB/s"], 4)
            kernels[k]["copy_ceiling"] = ck
    for att, fk in (("alibi_attention_fwd", "_attention_flops"), ("alibi_attention_fwd_8192", "_attention_flops_8192"),
                    ("alibi_attention_bwd", "_attention_bwd_flops")):
        if att not in kernels:
            continue
        # causal: each D-wide product takes 2*D flops for every (query, key <= query) pair
        flops = bts[fk]
        tf = flops / (per[att] * 1e-3) / 1e12
        kernels[att].update({"flops": flops, "TFLOP/s": round(tf, 1),
                             "frac_of_mfma_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                             "bound": "mfma (bf16 dense, 2500 TFLOP/s)"})
    dom = "grad_accumulate"
    dom_gbs = bts[dom] / (in_step[dom] * 1e-3) / 1e9
    roof = {"kernel": "grad_accumulate_kernel<false, false>: one micro-batch's bf16 gradient added to the fp32 "
                      "accumulator (micro-batches 2-31; 10 B per element)",
            "bound": "hbm", "achieved": round(dom_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(dom_gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(dom),
            "algorithmic_bytes_per_launch": bts[dom], "avg_launch_ms": round(in_step[dom], 4),
            "timing": f"HIP events around each of its {g['launches'][dom]} launches per step, on the launch stream",
            "traffic_source": "profiles/counters.json (FETCH_SIZE and WRITE_SIZE runs of the same command, scaled "
                              "by a plain copy's counters; null when the kernel source has changed since)"}
    if "1in_1out_fp32_shard" in g["ceilings"]:
        roof["frac_of_copy_ceiling"] = round(dom_gbs / g["ceilings"]["1in_1out_fp32_shard"]["GB/s"], 4)
    result = {
        "metric": METRIC,
        "value": round(total_bytes / (g["ms_step"] * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(g["ms_step"], 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": {"workload": "bloom176b-tp4-shard-step: layernorm fwd+bwd [2048,14336]; alibi causal softmax "
                               "fwd+bwd [1,28,2048,2048] (heads 0-27 of 112); bias-gelu fwd+bwd [2048,14336]; "
                               f"bf16-optimizer over a {n}-element shard: {mb} distinct bf16 micro-batch gradients "
                               "accumulated in fp32 one pass per micro-batch, global-norm clip 1.0, adamw, "
                               "rne bf16 copy",
                   "optimizer_elements": n, "microbatches": mb, "accumulation_passes": mb,
                   "storage": "bf16 activations and gradients, fp32 master/moments/accumulator"},
        "step_timing": "ms_per_step = sum of the HIP-event durations of the step's 39 path launches (6 fused "
                       "kernels, 32 accumulation passes, the adamw step), mean over the timed steps; the micro-batch "
                       "gradients are regenerated on the device between the accumulation passes, outside the events",
        "step_bytes": total_bytes,
        "wall_ms_per_step_with_gradient_regeneration": round(g["wall_ms"], 3),
        "grad_norm": round(g["grad_norm"], 4),
        "adamw_step_ms": round(per["adamw_step"], 3),
        "kernels": kernels,
        "copy_ceilings": g["ceilings"],
        "roofline": roof,
    }
    if g["batched"] is not None:
        result["batched_accumulation"] = g["batched"]
    if cpu is not None:
        workers, r, secs, err = cpu
        if err is not None:
            result["cpu_baseline"] = {"value": None, "unit": "GB/s", "cores": workers, "kind": "oracle",
                                      "error": err}
        else:
            sample = workers * args.cpu_opt_elems
            scale = n / sample
            rows = {k: r[k] for k in FUSED_STEP}
            rows["grad_accumulate_first"] = r["grad_accumulate_first"] * scale
            rows["grad_accumulate"] = r["grad_accumulate"] * scale * (mb - 1)
            rows["adamw_step"] = r["adamw_step"] * scale
            cpu_step = sum(rows.values())
            result["cpu_baseline"] = {
                "value": round(total_bytes / cpu_step / 1e9, 3), "unit": "GB/s", "cores": workers, "kind": "oracle",
                "sample": f"NumPy float64 oracle in {workers} processes (one thread each), every row of the step: "
                          "the six fused rows at their full shapes ([2048,14336] LayerNorm and bias-GeLU fwd+bwd, "
                          "[1,28,2048,2048] softmax fwd+bwd), the optimizer rows on "
                          f"{sample:,} of the shard's {n:,} elements (one first and one later accumulation, one "
                          "norm+clip+AdamW+bf16 step, each repeated and averaged) scaled to the shard and to one accumulation per micro-batch; "
                          "value = the step's algorithmic bytes (the same model as the GPU value) / the oracle's "
                          "step time; each row's wall time is its slowest worker's, all workers started together",
                "cpu_model": cpu_model(), "host_logical_cpus": os.cpu_count(),
                "step_seconds": round(cpu_step, 2),
                "row_seconds": {k: round(v, 3) for k, v in rows.items()},
                "leg_wall_seconds": round(secs, 1)}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
