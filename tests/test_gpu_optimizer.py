"""GPU parity: the BF16Optimizer (grad accumulation, norm + clip, AdamW, bf16 copy)."""

import numpy as np
import pytest
import torch

import synth
from synth import workloads as W
from synth import device as sdev
from oracle import optimizer as oopt
from oracle.bf16 import round_to_bf16, to_f64
from parity_helpers import check_state, gen, host_bf16, require_gpu, sample_rows
from bloom_bf16_optimizer_amd import ops

pytestmark = pytest.mark.gpu

HP = dict(lr=W.LR, beta1=W.BETA1, beta2=W.BETA2, eps=W.ADAM_EPS, weight_decay=W.WEIGHT_DECAY,
          max_grad_norm=W.MAX_GRAD_NORM)


def _hp(step, sumsq_in_workspace=False, **over):
    d = dict(HP)
    d.update(over)
    return ops.adamw_hparams(d["lr"], d["beta1"], d["beta2"], d["eps"], d["weight_decay"], d["max_grad_norm"], step,
                             sumsq_in_workspace)


def _workspace(n):
    return torch.empty(ops.bloom_bf16_adamw_workspace_size(n), dtype=torch.uint8, device="cuda")


def _step_gpu(master, m, v, acc, hp, ws=None):
    n = master.numel()
    param = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    norm = torch.empty(1, dtype=torch.float32, device="cuda")
    if ws is None:
        ws = _workspace(n)
    ops.bloom_bf16_adamw_step(master, m, v, param, acc, hp, norm, ws)
    torch.cuda.synchronize()
    return param, float(norm.item())


def _oracle_step(p, m, v, acc, step, norm=None, **over):
    d = dict(HP)
    d.update(over)
    if norm is None:
        norm = oopt.global_norm(acc)
    c = oopt.clip_coefficient(norm, d["max_grad_norm"])
    out, f64, terms = oopt.adamw_update(p, m, v, acc, c, d["lr"], d["beta1"], d["beta2"], d["eps"],
                                        d["weight_decay"], step, return_f64=True)
    return out, f64, terms, norm


def _compare_step(tag, gpu_master, gpu_m, gpu_v, gpu_param, f64, terms, ref_param):
    check_state(f"{tag} master", gpu_master, f64[0], terms[0])
    check_state(f"{tag} exp_avg", gpu_m, f64[1], terms[1])
    check_state(f"{tag} exp_avg_sq", gpu_v, f64[2], terms[2])
    # the bf16 copy is exactly the RNE of the GPU's own master ...
    assert np.array_equal(gpu_param, round_to_bf16(gpu_master.astype(np.float64))), f"{tag} param RNE"
    # ... and within one bf16 ulp of the RNE of the oracle's master
    a = gpu_param.astype(np.int32)
    b = ref_param.astype(np.int32)
    fin = np.isfinite(to_f64(ref_param))
    assert np.all(np.abs(a[fin] - b[fin]) <= 1), f"{tag} param vs oracle"


def _accumulate_gpu(n, seed, microbatches, start_stream=W.S_OPT_GRAD0 + 1, ws=None):
    """Accumulates the micro-batch gradients; with a workspace the last call is
    the fused accumulate + norm-partials entry point."""
    acc = torch.empty(n, dtype=torch.float32, device="cuda")
    g = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    for k in range(microbatches):
        sdev.fill_(g, seed, start_stream + k, W.GRAD_SIGMA)
        if ws is not None and k == microbatches - 1:
            ops.bloom_bf16_grad_accumulate_sumsq(acc, g, k == 0, ws)
        else:
            ops.bloom_bf16_grad_accumulate(acc, g, first_microbatch=(k == 0))
    torch.cuda.synchronize()
    return acc


def _accumulate_oracle(idx, seed, microbatches, start_stream=W.S_OPT_GRAD0 + 1):
    acc = None
    for k in range(microbatches):
        g = synth.values(seed, start_stream + k, idx, W.GRAD_SIGMA, mode=synth.MODE_BF16)
        acc = oopt.grad_accumulate(acc, g, first=(k == 0))
    return acc


@pytest.mark.parametrize("n,mb,step,zero_moments", [(1_000_000, 1, 1, True), (1_000_003, 3, 5, False),
                                                    (100_003, 32, 1, True), (7, 2, 2, False), (8, 1, 1, True),
                                                    (1, 1, 1, True)])
def test_step_small(n, mb, step, zero_moments):
    """Tiny config (1M elements, one micro-batch, clip right at 1.0), odd sizes,
    32 micro-batches, and nonzero moments at later steps."""
    require_gpu()
    seed = 0
    tp, p = gen((n,), seed, W.S_OPT_PARAM, W.PARAM_SIGMA, dtype=torch.float32)
    if zero_moments:
        tm = torch.zeros(n, dtype=torch.float32, device="cuda")
        tv = torch.zeros(n, dtype=torch.float32, device="cuda")
    else:
        tm = gen((n,), seed, W.S_OPT_M, W.M_SIGMA, dtype=torch.float32)[0]
        tv = gen((n,), seed, W.S_OPT_V, W.V_SIGMA, dtype=torch.float32, absolute=True)[0]
    m, v = tm.cpu().numpy(), tv.cpu().numpy()
    acc_t = _accumulate_gpu(n, seed, mb)
    acc = acc_t.cpu().numpy()
    ref_acc = _accumulate_oracle(np.arange(n, dtype=np.uint64), seed, mb)
    assert np.array_equal(acc.view(np.uint32), ref_acc.view(np.uint32)), "accumulator not bit-exact"
    param, norm = _step_gpu(tp, tm, tv, acc_t, _hp(step))
    (rp, rm, rv, rpb), f64, terms, rnorm = _oracle_step(p, m, v, ref_acc, step)
    assert abs(norm - rnorm) <= 1e-6 * rnorm, (norm, rnorm)
    _compare_step(f"n={n}", tp.cpu().numpy(), tm.cpu().numpy(), tv.cpu().numpy(), host_bf16(param), f64, terms, rpb)


@pytest.mark.parametrize("n,mb", [(1_000_003, 3), (4096, 1), (5, 2), (3_000_000, 32)])
def test_fused_norm_partials_match_standalone(n, mb):
    """The last micro-batch's fused accumulate + norm partials, then the step
    with sumsq_in_workspace = 1, gives the same bits as the unfused path."""
    require_gpu()
    seed = 6
    outs = []
    for fused in (False, True):
        tp = gen((n,), seed, W.S_OPT_PARAM, W.PARAM_SIGMA, dtype=torch.float32)[0]
        tm = gen((n,), seed, W.S_OPT_M, W.M_SIGMA, dtype=torch.float32)[0]
        tv = gen((n,), seed, W.S_OPT_V, W.V_SIGMA, dtype=torch.float32, absolute=True)[0]
        ws = _workspace(n)
        acc = _accumulate_gpu(n, seed, mb, ws=ws if fused else None)
        param, norm = _step_gpu(tp, tm, tv, acc, _hp(4, sumsq_in_workspace=fused), ws=ws)
        outs.append([acc.cpu().numpy(), tp.cpu().numpy(), tm.cpu().numpy(), tv.cpu().numpy(),
                     host_bf16(param), np.array([norm], dtype=np.float32)])
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
    ref = oopt.global_norm(_accumulate_oracle(np.arange(n, dtype=np.uint64), seed, mb))
    assert abs(float(outs[1][5][0]) - ref) <= 1e-6 * ref


@pytest.mark.parametrize("n,mb,batch", [(1_000_003, 11, 4), (4099, 8, 8), (7, 3, 2), (100_000, 32, 8), (1, 1, 1),
                                        (3_000_000, 5, 3), (100_003, 32, 16), (4099, 23, 11), (1_000_001, 16, 16)])
def test_accumulate_many_bit_exact(n, mb, batch):
    """Several micro-batches per pass (groups of `batch`, the last possibly
    shorter): bit-identical to one pass per micro-batch and to the oracle's
    sequential FP32 adds; the last group with the norm partials gives the
    same step as the standalone norm."""
    require_gpu()
    seed = 7
    grads = []
    for k in range(mb):
        g = torch.empty(n, dtype=torch.bfloat16, device="cuda")
        sdev.fill_(g, seed, W.S_OPT_GRAD0 + 1 + k, W.GRAD_SIGMA)
        grads.append(g)
    ws = _workspace(n)
    acc = torch.empty(n, dtype=torch.float32, device="cuda")
    for k0 in range(0, mb, batch):
        group = grads[k0:k0 + batch]
        last = k0 + batch >= mb
        ops.bloom_bf16_grad_accumulate_many(acc, group, k0 == 0, ws if last else None)
    torch.cuda.synchronize()
    got = acc.cpu().numpy()
    ref = _accumulate_oracle(np.arange(n, dtype=np.uint64), seed, mb)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), "accumulator not bit-exact"
    single = _accumulate_gpu(n, seed, mb).cpu().numpy()
    assert np.array_equal(got.view(np.uint32), single.view(np.uint32))
    outs = []
    for fused in (True, False):
        tp = gen((n,), seed, W.S_OPT_PARAM, W.PARAM_SIGMA, dtype=torch.float32)[0]
        tm = torch.zeros(n, dtype=torch.float32, device="cuda")
        tv = torch.zeros(n, dtype=torch.float32, device="cuda")
        param, norm = _step_gpu(tp, tm, tv, acc, _hp(1, sumsq_in_workspace=fused), ws=ws if fused else None)
        outs.append((tp.cpu().numpy(), host_bf16(param), norm))
    assert np.array_equal(outs[0][0].view(np.uint32), outs[1][0].view(np.uint32))
    assert np.array_equal(outs[0][1], outs[1][1]) and outs[0][2] == outs[1][2]


def test_two_steps_and_checkpoint_round_trip():
    """t = 1 then t = 2; a host round trip of the state between steps (the
    checkpoint analogue) continues bit-identically."""
    require_gpu()
    n, seed = 200_001, 4
    tp, p = gen((n,), seed, W.S_OPT_PARAM, W.PARAM_SIGMA, dtype=torch.float32)
    tm = torch.zeros(n, dtype=torch.float32, device="cuda")
    tv = torch.zeros(n, dtype=torch.float32, device="cuda")
    acc1 = _accumulate_gpu(n, seed, 4, start_stream=200)
    acc2 = _accumulate_gpu(n, seed, 4, start_stream=300)
    _step_gpu(tp, tm, tv, acc1, _hp(1))
    saved = [t.cpu().clone() for t in (tp, tm, tv)]
    param_a, norm_a = _step_gpu(tp, tm, tv, acc2, _hp(2))
    after_a = [t.cpu().numpy() for t in (tp, tm, tv)]
    rp, rm, rv = [s.cuda() for s in saved]
    param_b, norm_b = _step_gpu(rp, rm, rv, acc2, _hp(2))
    for x, y in zip(after_a, (rp, rm, rv)):
        assert np.array_equal(x.view(np.uint32), y.cpu().numpy().view(np.uint32))
    assert torch.equal(param_a.view(torch.int16), param_b.view(torch.int16)) and norm_a == norm_b
    # and the two-step result matches the oracle run step by step
    z = np.zeros(n, dtype=np.float32)
    a1 = acc1.cpu().numpy()
    a2 = acc2.cpu().numpy()
    (p1, m1, v1, _), f64_1, terms_1, _ = _oracle_step(p, z, z, a1, 1)
    for got, ref, tm_, nm in zip(saved, f64_1, terms_1, ("master", "exp_avg", "exp_avg_sq")):
        check_state(f"step 1 {nm}", got.numpy(), ref, tm_)
    (p2, m2, v2, pb2), f64, terms, _ = _oracle_step(saved[0].numpy(), saved[1].numpy(), saved[2].numpy(), a2, 2)
    _compare_step("step 2", after_a[0], after_a[1], after_a[2], host_bf16(param_a), f64, terms, pb2)


def test_bf16_copy_rounding_table():
    """lr = 0, weight decay 0, zero gradient: master is unchanged and the bf16
    copy is its round-to-nearest-even (ties, subnormals, overflow, NaN)."""
    require_gpu()
    bits = np.array([0x3F808000, 0x3F818000, 0x3F807FFF, 0x3F808001, 0x7F7FFFFF, 0xFF7FFFFF, 0x00008000,
                     0x00018000, 0x80018000, 0x007FFFFF, 0x3F7FFFFF, 0x7FC00000, 0x7F800001,
                     0x00000001, 0x3F800000, 0xC0490FDB, 0x33333333, 0x4B7FFFFF, 0x0], dtype=np.uint32)
    n = len(bits)
    master = torch.from_numpy(bits.view(np.float32).copy()).cuda()
    z = torch.zeros(n, dtype=torch.float32, device="cuda")
    param, _ = _step_gpu(master, z.clone(), z.clone(), z.clone(), _hp(1, lr=0.0, weight_decay=0.0))
    got = host_bf16(param)
    m = master.cpu().numpy()
    assert np.array_equal(m.view(np.uint32)[~np.isnan(m)], bits[~np.isnan(bits.view(np.float32))])
    want = round_to_bf16(bits.view(np.float32).astype(np.float64))
    assert np.array_equal(got, want), [hex(x) for x in got]


@pytest.mark.parametrize("bad", ["nan", "inf"])
def test_nonfinite_gradient(bad):
    """A NaN norm leaves c = 1 (only the NaN element goes NaN); an infinite norm
    gives c = 0 (finite elements see a zero gradient)."""
    require_gpu()
    n = 4099
    tp, p = gen((n,), 9, W.S_OPT_PARAM, W.PARAM_SIGMA, dtype=torch.float32)
    tm, m = gen((n,), 9, W.S_OPT_M, W.M_SIGMA, dtype=torch.float32)
    tv, v = gen((n,), 9, W.S_OPT_V, W.V_SIGMA, dtype=torch.float32, absolute=True)
    tacc, acc = gen((n,), 9, W.S_OPT_ACC, 1e-2, dtype=torch.float32)
    acc[17] = np.float32(np.nan if bad == "nan" else np.inf)
    tacc.copy_(torch.from_numpy(acc))
    param, norm = _step_gpu(tp, tm, tv, tacc, _hp(3))
    (rp, rm, rv, rpb), f64, terms, rnorm = _oracle_step(p, m, v, acc, 3)
    assert (np.isnan(norm) and np.isnan(rnorm)) or norm == rnorm
    _compare_step(f"{bad} grad", tp.cpu().numpy(), tm.cpu().numpy(), tv.cpu().numpy(), host_bf16(param),
                  f64, terms, rpb)


def test_deterministic_and_no_norm_output():
    require_gpu()
    n = 2_000_000
    outs = []
    for _ in range(2):
        tp = gen((n,), 5, W.S_OPT_PARAM, W.PARAM_SIGMA, dtype=torch.float32)[0]
        tm = gen((n,), 5, W.S_OPT_M, W.M_SIGMA, dtype=torch.float32)[0]
        tv = gen((n,), 5, W.S_OPT_V, W.V_SIGMA, dtype=torch.float32, absolute=True)[0]
        tacc = gen((n,), 5, W.S_OPT_ACC, 0.05, dtype=torch.float32)[0]
        param = torch.empty(n, dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(ops.bloom_bf16_adamw_workspace_size(n), dtype=torch.uint8, device="cuda")
        ops.bloom_bf16_adamw_step(tp, tm, tv, param, tacc, _hp(2), None, ws)
        torch.cuda.synchronize()
        outs.append([t.cpu().numpy().copy() for t in (tp, tm, tv)] + [host_bf16(param)])
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


@pytest.mark.timeout(900)
def test_mini_bloom_optimizer_full_size():
    """1,722,400,768 elements (24 layers + 250880 x 2048 embedding), step 100,
    accumulated gradient drawn directly, nonzero moments."""
    require_gpu()
    wl = W.MINI
    n = wl.opt.n
    tacc = gen((n,), wl.seed, W.S_OPT_ACC, W.GRAD_SIGMA, dtype=torch.float32)[0]
    acc_host = tacc.cpu().numpy()
    rnorm = float(np.sqrt(sum(np.dot(acc_host[i:i + (1 << 26)].astype(np.float64),
                                     acc_host[i:i + (1 << 26)].astype(np.float64))
                              for i in range(0, n, 1 << 26))))
    tp = gen((n,), wl.seed, W.S_OPT_PARAM, W.PARAM_SIGMA, dtype=torch.float32)[0]
    tm = gen((n,), wl.seed, W.S_OPT_M, W.M_SIGMA, dtype=torch.float32)[0]
    tv = gen((n,), wl.seed, W.S_OPT_V, W.V_SIGMA, dtype=torch.float32, absolute=True)[0]
    param, norm = _step_gpu(tp, tm, tv, tacc, _hp(wl.opt.step))
    assert abs(norm - rnorm) <= 1e-6 * rnorm, (norm, rnorm)
    idx = sample_rows(n, 1_000_000, 41, must=list(range(8)) + list(range(n - 8, n)))
    ti = torch.from_numpy(idx).cuda()
    p = synth.values(wl.seed, W.S_OPT_PARAM, idx, W.PARAM_SIGMA)
    m = synth.values(wl.seed, W.S_OPT_M, idx, W.M_SIGMA)
    v = synth.values(wl.seed, W.S_OPT_V, idx, W.V_SIGMA, mode=synth.MODE_ABS_F32)
    (rp, rm, rv, rpb), f64, terms, _ = _oracle_step(p, m, v, acc_host[idx], wl.opt.step, norm=rnorm)
    _compare_step("mini-bloom", tp[ti].cpu().numpy(), tm[ti].cpu().numpy(), tv[ti].cpu().numpy(),
                  host_bf16(param[ti]), f64, terms, rpb)


@pytest.mark.timeout(1200)
def test_shard_optimizer_full_size():
    """3.67e9-element shard: 32 bf16 micro-batch gradients accumulated in FP32,
    global norm and clip, AdamW at t = 1, bf16 copy.  Sampled elements against
    the oracle (accumulator bit-exact), the norm against the float64 norm of
    the accumulator (which the samples pin)."""
    require_gpu()
    wl = W.OPTIMIZER
    n, mb = wl.opt.n, wl.opt.microbatches
    ws = _workspace(n)
    tacc = _accumulate_gpu(n, wl.seed, mb, ws=ws)   # last micro-batch fused with the norm partials
    idx = sample_rows(n, 300_000, 43, must=list(range(8)) + list(range(n - 8, n)) + [2 ** 31 - 1, 2 ** 31, 3 * 2 ** 30])
    ti = torch.from_numpy(idx).cuda()
    acc_s = tacc[ti].cpu().numpy()
    ref_acc = _accumulate_oracle(idx.astype(np.uint64), wl.seed, mb)
    assert np.array_equal(acc_s.view(np.uint32), ref_acc.view(np.uint32)), "accumulator not bit-exact"
    ss = 0.0
    chunk = 1 << 28
    for i in range(0, n, chunk):
        a = tacc[i:i + chunk].cpu().numpy().astype(np.float64)
        ss += float(np.dot(a, a))
    rnorm = float(np.sqrt(ss))
    tp = gen((n,), wl.seed, W.S_OPT_PARAM, W.PARAM_SIGMA, dtype=torch.float32)[0]
    tm = torch.zeros(n, dtype=torch.float32, device="cuda")
    tv = torch.zeros(n, dtype=torch.float32, device="cuda")
    param, norm = _step_gpu(tp, tm, tv, tacc, _hp(1, sumsq_in_workspace=True), ws=ws)
    assert abs(norm - rnorm) <= 1e-6 * rnorm, (norm, rnorm)
    assert norm > 300.0  # clipping active (expected about 342.7)
    p = synth.values(wl.seed, W.S_OPT_PARAM, idx, W.PARAM_SIGMA)
    z = np.zeros(len(idx), dtype=np.float32)
    (rp, rm, rv, rpb), f64, terms, _ = _oracle_step(p, z, z, ref_acc, 1, norm=rnorm)
    _compare_step("shard", tp[ti].cpu().numpy(), tm[ti].cpu().numpy(), tv[ti].cpu().numpy(),
                  host_bf16(param[ti]), f64, terms, rpb)


@pytest.mark.timeout(1200)
def test_shard_accumulate_many_full_size():
    """The batched accumulation at the 3.67e9-element shard: 32 distinct
    micro-batch gradients in two passes of 16 resident gradients (the second
    with the norm partials).  Sampled elements, including indices on both
    sides of 2^31, are bit-exact against the oracle's sequential FP32 adds;
    the fused norm partials give the step the float64 norm of the full
    accumulator within 1e-6."""
    require_gpu()
    wl = W.OPTIMIZER
    n, mb, k = wl.opt.n, wl.opt.microbatches, 16
    ws = _workspace(n)
    acc = torch.empty(n, dtype=torch.float32, device="cuda")
    grads = [torch.empty(n, dtype=torch.bfloat16, device="cuda") for _ in range(k)]
    for p0 in range(0, mb, k):
        for j in range(k):
            sdev.fill_(grads[j], wl.seed, W.S_OPT_GRAD0 + 1 + p0 + j, W.GRAD_SIGMA)
        last = p0 + k == mb
        ops.bloom_bf16_grad_accumulate_many(acc, grads, p0 == 0, ws if last else None)
    torch.cuda.synchronize()
    del grads
    idx = sample_rows(n, 300_000, 47, must=list(range(8)) + list(range(n - 8, n))
                      + [2 ** 31 - 1, 2 ** 31, 2 ** 31 + 1, 3 * 2 ** 30, 3 * 2 ** 30 + 1, 3_600_000_000])
    ti = torch.from_numpy(idx).cuda()
    got = acc[ti].cpu().numpy()
    ref = _accumulate_oracle(idx.astype(np.uint64), wl.seed, mb)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), "accumulator not bit-exact"
    ss = 0.0
    chunk = 1 << 28
    for i in range(0, n, chunk):
        a = acc[i:i + chunk].cpu().numpy().astype(np.float64)
        ss += float(np.dot(a, a))
    rnorm = float(np.sqrt(ss))
    tp = gen((n,), wl.seed, W.S_OPT_PARAM, W.PARAM_SIGMA, dtype=torch.float32)[0]
    tm = torch.zeros(n, dtype=torch.float32, device="cuda")
    tv = torch.zeros(n, dtype=torch.float32, device="cuda")
    _, norm = _step_gpu(tp, tm, tv, acc, _hp(1, sumsq_in_workspace=True), ws=ws)
    assert abs(norm - rnorm) <= 1e-6 * rnorm, (norm, rnorm)
    assert 330.0 < norm < 355.0   # 32 distinct N(0, 1e-3) gradients: about 342.7


@pytest.mark.parametrize("n,segs,fused", [
    (1_000_003, [(0, 600_000, 0.01), (600_000, 300_000, 0.0), (900_000, 100_003, 0.05)], False),
    (1_000_003, [(0, 999_992, 0.01), (999_992, 11, 0.0)], True),
    (24, [(0, 8, 0.0), (8, 8, 0.1), (16, 8, 0.01)], False)])
def test_weight_decay_segments(n, segs, fused):
    """Per-segment weight decay with one global norm and clip, against the
    oracle; one segment spanning everything reproduces the flat step's bits."""
    require_gpu()
    seed, step, mb = 5, 3, 2
    tp, p = gen((n,), seed, W.S_OPT_PARAM, W.PARAM_SIGMA, dtype=torch.float32)
    tm, m = gen((n,), seed, W.S_OPT_M, W.M_SIGMA, dtype=torch.float32)
    tv, v = gen((n,), seed, W.S_OPT_V, W.V_SIGMA, dtype=torch.float32, absolute=True)
    ws = _workspace(n)
    acc_t = _accumulate_gpu(n, seed, mb, ws=ws if fused else None)
    acc = acc_t.cpu().numpy()
    ref_acc = _accumulate_oracle(np.arange(n, dtype=np.uint64), seed, mb)
    assert np.array_equal(acc.view(np.uint32), ref_acc.view(np.uint32))
    # the flat step with one full segment, on copies, for the bit-identity check
    cp, cm, cv = tp.clone(), tm.clone(), tv.clone()
    param = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    norm = torch.empty(1, dtype=torch.float32, device="cuda")
    ops.bloom_bf16_adamw_step_segments(tp, tm, tv, param, acc_t, _hp(step, fused), segs, norm, ws)
    torch.cuda.synchronize()
    rp, rm, rv, rpb, rnorm, c = oopt.bf16_optimizer_step_segments(p, m, v, ref_acc, segs, W.LR, W.BETA1, W.BETA2,
                                                                 W.ADAM_EPS, W.MAX_GRAD_NORM, step)
    assert abs(norm.item() - rnorm) <= 1e-6 * rnorm
    gm, gmm, gv, gpb = tp.cpu().numpy(), tm.cpu().numpy(), tv.cpu().numpy(), host_bf16(param)
    for off, length, wd in segs:
        sl = slice(off, off + length)
        _, f64, terms = oopt.adamw_update(p[sl], m[sl], v[sl], ref_acc[sl], c, W.LR, W.BETA1, W.BETA2, W.ADAM_EPS,
                                          wd, step, return_f64=True)
        _compare_step(f"segment {off}+{length} wd={wd}", gm[sl], gmm[sl], gv[sl], gpb[sl], f64, terms, rpb[sl])
    if not fused:
        # one segment over everything == the flat entry point with that weight decay, bit for bit
        fp, fm, fv = cp.clone(), cm.clone(), cv.clone()
        p2, p3 = torch.empty_like(param), torch.empty_like(param)
        ops.bloom_bf16_adamw_step_segments(cp, cm, cv, p2, acc_t, _hp(step), [(0, n, segs[0][2])], norm, ws)
        ops.bloom_bf16_adamw_step(fp, fm, fv, p3, acc_t, _hp(step, weight_decay=segs[0][2]), norm, ws)
        torch.cuda.synchronize()
        assert torch.equal(cp, fp) and torch.equal(cm, fm) and torch.equal(cv, fv) and torch.equal(p2, p3)
