"""Benchmark: one BLOOM-176B TP=4 shard training step's hot path on one MI355X.

A step is one pass over every kernel of the path, on synthetic BLOOM-shaped
data already resident in HBM:

  LayerNorm fwd + bwd          [2048, 14336] bf16
  ALiBi causal softmax fwd+bwd [1, 28, 2048, 2048] bf16 (heads 0..27 of 112)
  bias + GeLU fwd + bwd        [2048, 14336] bf16
  FP32 gradient accumulation   32 micro-batches of a 3.67e9-element bf16 gradient,
                               16 resident micro-batch gradients added per pass
  BF16Optimizer step           global norm, clip 1.0, AdamW, bf16 parameter copy

Each kernel reads inputs that were last touched a whole step earlier (the
accumulation streams ~1.2 TB per step in between), so no kernel is served by
the 256 MB Infinity Cache from the previous one.  The 32 micro-batch gradients
cycle through 16 distinct 7.34 GB buffers (117 GB; all 32 would need 235 GB).
By default each accumulation pass adds `--accum-batch` (16) of them to the FP32
accumulator in micro-batch order: 2 passes of 36 and 40 B per element instead of
32 passes of 10 B, bit-identical; `--accum-batch 8` takes 4 passes (92 B per
element) and `--accum-batch 1` one pass per micro-batch.

Prints one JSON line.  `value` is the whole step's algorithmic HBM throughput
(sum of each kernel's algorithmic bytes / step time, GB/s); per-kernel
algorithmic GB/s, the fraction of the 8 TB/s HBM peak and the AdamW step time
are reported beside it, with a roofline entry for the dominant kernel (the
accumulation) and the CPU oracle timed on a bounded sample.  The optimizer
kernels are timed with events around each launch inside the timed steps; the
fused kernels (tens of microseconds, where an event pair adds a few) are also
timed after the steps in sweeps of back-to-back launches over rotating cold
input sets; the median of three sweeps is their per-kernel number.
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
GRAD_BUFFERS = 16      # resident gradient buffers (at least --accum-batch of them)
MAX_ACCUM_BATCH = 16   # the library limit on micro-batches per pass
COUNTERS = os.path.join(ROOT, "profiles", "counters.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------
# Algorithmic bytes of each step row (what the method must read and write).
def bytes_model(sh, n, mb, batch=GRAD_BUFFERS):
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
    batch = args.accum_batch
    nbuf = max(GRAD_BUFFERS, batch)
    rows, hid = X.ln.rows, X.ln.hidden
    smb, smh, sms = X.softmax.batch, X.softmax.heads, X.softmax.seq
    grows, gcols = X.gelu.rows, X.gelu.cols
    bf, f32 = torch.bfloat16, torch.float32
    seed = X.seed
    scale = X.softmax.scale

    def fill(shape, stream, sigma, offset=0.0, dtype=bf, s=0):
        t = torch.empty(shape, dtype=dtype, device=dev)
        sdev.fill_(t, seed + 1000 * s, stream, sigma, offset)
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
    # Kernels measured in the sweep only (not rows of the step): LayerNorm fused
    # with the residual connection, at the same [2048, 14336] shape.
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

    def acc_one_set(s):
        # one micro-batch per pass (a later micro-batch), over the resident gradient buffers
        return lambda: ops.bloom_bf16_grad_accumulate(acc, grads[s], False)

    sweep_only = [("layernorm_residual_fwd", lnr_fwd_set, 4), ("layernorm_residual_bwd", lnr_bwd_set, 4),
                  ("alibi_attention_fwd", att_fwd_set, 4), ("alibi_attention_fwd_8192", att_fwd_long_set, 2),
                  ("alibi_attention_bwd", att_bwd_set, 4), ("layernorm_fwd_8192", ln_fwd_long_set, 4),
                  ("alibi_softmax_fwd_8192", sm_fwd_long_set, 2),
                  ("layernorm_fwd_mini", m_ln_fwd_set, 4), ("layernorm_bwd_mini", m_ln_bwd_set, 4),
                  ("alibi_softmax_fwd_mini", m_sm_fwd_set, 2), ("alibi_softmax_bwd_mini", m_sm_bwd_set, 2),
                  ("bias_gelu_fwd_mini", m_ge_fwd_set, 4), ("bias_gelu_bwd_mini", m_ge_bwd_set, 4)]
    if n >= MI.opt.n:   # the mini model's update runs on slices of the shard's buffers
        sweep_only.append(("adamw_step_mini", m_adamw_set, 1))
    if batch > 1:
        sweep_only.append(("grad_accumulate", acc_one_set, nbuf))

    log(f"bench: allocating the shard workload (n = {n:,}, {nbuf} gradient buffers)")
    master = fill((n,), W.S_OPT_PARAM, W.PARAM_SIGMA, dtype=f32)
    exp_avg = torch.zeros(n, dtype=f32, device=dev)
    exp_avg_sq = torch.zeros(n, dtype=f32, device=dev)
    acc = torch.empty(n, dtype=f32, device=dev)
    param = torch.empty(n, dtype=bf, device=dev)
    grads = [fill((n,), W.S_OPT_GRAD0 + 1 + k, W.GRAD_SIGMA) for k in range(nbuf)]
    norm = torch.empty(1, dtype=f32, device=dev)
    opt_ws = torch.empty(ops.bloom_bf16_adamw_workspace_size(n), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    log(f"bench: resident {torch.cuda.memory_allocated() / 2**30:.1f} GiB")

    if batch == 1:
        acc_names = ["grad_accumulate_first", "grad_accumulate", "grad_accumulate_last"]
    else:
        acc_names = ["grad_accumulate_many_first", "grad_accumulate_many", "grad_accumulate_many_last"]
    names = [name for name, _ in step_fused] + acc_names + ["adamw_step"]
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
        for name, fn in step_fused:
            timed(name, fn, record)
        if batch == 1:
            for k in range(mb):
                g = grads[k % nbuf]
                if k == mb - 1:   # the last micro-batch also writes the norm's partial sums
                    timed("grad_accumulate_last", lambda g=g, k=k: ops.bloom_bf16_grad_accumulate_sumsq(
                        acc, g, k == 0, opt_ws), record)
                else:
                    name = "grad_accumulate_first" if k == 0 else "grad_accumulate"
                    timed(name, lambda g=g, k=k: ops.bloom_bf16_grad_accumulate(acc, g, k == 0), record)
        else:
            for k0 in range(0, mb, batch):
                group = [grads[(k0 + j) % nbuf] for j in range(batch)]
                last = k0 + batch == mb    # the last pass also writes the norm's partial sums
                name = ("grad_accumulate_many_first" if k0 == 0 else
                        "grad_accumulate_many_last" if last else "grad_accumulate_many")
                timed(name, lambda group=group, k0=k0, last=last: ops.bloom_bf16_grad_accumulate_many(
                    acc, group, k0 == 0, opt_ws if last else None), record)
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
    in_step = {}
    for k in names:
        ts = [a.elapsed_time(b) for a, b in ev[k]]
        if ts:   # with two accumulation passes there is no middle one
            in_step[k] = sum(ts) / len(ts)
    log(f"bench: {ms_step:.2f} ms/step; grad norm {norm.item():.4f}")

    # Per-kernel sweep of the fused kernels: R back-to-back launches rotating
    # over S cold input sets between one pair of events, so the per-launch
    # event overhead (a few microseconds) is amortised; three such sweeps per
    # kernel, the median reported (and the fastest kept beside it).
    sweep = {}
    sweep_min = {}
    reps = 24
    trials = 3
    for name, make, sets in ([] if args.no_sweep else fused + sweep_only):
        if name in dict(step_fused):
            fns = [dict(step_fused)[name]] + [make(s) for s in range(1, sets)]
        else:
            fns = [make(s) for s in range(sets)]
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
        sweep[name] = per_launch[len(per_launch) // 2]
        sweep_min[name] = per_launch[0]
        del fns
    shapes = {"ln": (rows, hid), "sm": (smb, smh, sms), "gelu": (grows, gcols), "head_dim": hd}
    bts = bytes_model(shapes, n, mb, batch)
    bts.update(long_context_model(W.LONG.ln.rows, W.LONG.ln.hidden, L.batch, L.heads, L.seq, L.head_dim))
    bts.update(mini_model())
    return ms_step, in_step, sweep, sweep_min, bts, n, mb


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
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run 3 plain 1 GiB device-to-device copies (counter calibration)")
    ap.add_argument("--no-sweep", action="store_true", help="skip the per-kernel sweep of the fused kernels")
    ap.add_argument("--accum-batch", type=int, default=GRAD_BUFFERS,
                    help="resident micro-batch gradients added per accumulation pass (1 = one pass each)")
    args = ap.parse_args()
    if not (1 <= args.accum_batch <= MAX_ACCUM_BATCH) or (args.accum_batch > 1 and 32 % (2 * args.accum_batch)):
        print(f"--accum-batch must be 1 or divide the 32 micro-batches into at least two passes of at most "
              f"{MAX_ACCUM_BATCH}", file=sys.stderr)
        sys.exit(2)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the hot path runs on a single MI355X at one GPU's shard shape, "
              "and runs on several GPUs are not supported.", file=sys.stderr)
        sys.exit(2)

    ms_step, in_step, sweep, sweep_min, bts, n, mb = run_gpu(args)
    batch = args.accum_batch
    per = dict(in_step)
    per.update(sweep)
    sweep = sweep or {}
    nfirst, nrest = 1, mb - 2
    step_bytes = sum(bts[k] for k in ("layernorm_fwd", "layernorm_bwd", "alibi_softmax_fwd", "alibi_softmax_bwd",
                                      "bias_gelu_fwd", "bias_gelu_bwd", "adamw_step"))
    if batch == 1:
        step_bytes += (bts["grad_accumulate_last"] + nfirst * bts["grad_accumulate_first"]
                       + nrest * bts["grad_accumulate"])
    else:
        step_bytes += (bts["grad_accumulate_many_first"] + bts["grad_accumulate_many_last"]
                       + (mb // batch - 2) * bts["grad_accumulate_many"])
    kernels = {}
    for k, ms in per.items():
        gbs = bts[k] / (ms * 1e-3) / 1e9
        kernels[k] = {"ms": round(ms, 4), "GB/s": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
                      "algorithmic_bytes": bts[k],
                      "timing": "median of 3 sweeps of 24 back-to-back launches on rotating cold inputs"
                      if k in sweep else "events around each launch in the timed steps"}
        if k in sweep:
            kernels[k]["min_sweep_ms"] = round(sweep_min[k], 4)
            kernels[k]["in_step_ms"] = round(in_step[k], 4) if k in in_step else None
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
    if batch == 1:
        dom, dom_label = "grad_accumulate", "grad_accumulate (micro-batches 2-31)"
    elif mb // batch > 2:
        dom = "grad_accumulate_many"
        dom_label = f"grad_accumulate_many ({batch} micro-batches per pass, passes 2-{mb // batch - 1})"
    else:   # two passes: the second, which also writes the norm's partial sums
        dom = "grad_accumulate_many_last"
        dom_label = f"grad_accumulate_many ({batch} micro-batches per pass, pass 2 of 2, with the norm partials)"
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
                   "optimizer_elements": n, "microbatches": mb, "grad_buffers": max(GRAD_BUFFERS, batch),
                   "microbatches_per_accumulation_pass": batch,
                   "storage": "bf16 activations and gradients, fp32 master/moments/accumulator"},
        "adamw_step_ms": round(per["adamw_step"], 3),
        "kernels": kernels,
        "roofline": {"kernel": dom_label, "bound": "hbm",
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
