"""bench.py's contract, on the CPU: the algorithmic byte and FLOP models that
every reported GB/s and TFLOP/s divides by, the argument checks, and the rule
that counter traffic is reported only while the measured kernel source is
unchanged.  Expected values are written out from the shapes by hand."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402  (imports no GPU library at module level)

R, H = 2048, 14336                 # LayerNorm / GeLU rows and width at the 176B TP=4 shard
B, NH, L, D = 1, 28, 2048, 128     # softmax / attention at the shard
N = 3_670_000_000                  # optimizer shard


def _model(batch):
    shapes = {"ln": (R, H), "sm": (B, NH, L), "gelu": (R, H), "head_dim": D}
    return bench.bytes_model(shapes, N, 32, batch)


def test_fused_kernel_bytes():
    m = _model(16)
    # LayerNorm fwd: x read, y written (2 B each), gamma and beta read, mean and rstd written
    assert m["layernorm_fwd"] == R * H * 2 * 2 + H * 2 * 2 + R * 4 * 2
    # LayerNorm bwd: dy, x read, dx written; gamma read, dgamma and dbeta written; mean and rstd read
    assert m["layernorm_bwd"] == R * H * 2 * 3 + H * 2 + H * 2 * 2 + R * 4 * 2
    # softmax: the causal half read (i + 1 entries of row i), the full row written
    causal = B * NH * L * (L + 1) // 2
    assert m["alibi_softmax_fwd"] == causal * 2 + B * NH * L * L * 2
    assert m["alibi_softmax_bwd"] == causal * 2 * 2 + B * NH * L * L * 2
    assert m["bias_gelu_fwd"] == R * H * 2 * 2 + H * 2
    assert m["bias_gelu_bwd"] == R * H * 2 * 3 + H * 2 * 2
    assert m["alibi_softmax_fwd"] == 352_378_880 and m["alibi_softmax_bwd"] == 469_876_736


def test_attention_bytes_and_flops():
    m = _model(16)
    rows = B * NH * L
    pairs = B * NH * L * (L + 1) // 2          # (query, key <= query) pairs
    assert m["alibi_attention_fwd"] == rows * D * 2 * 4 + rows * 4                # q, k, v, o; lse
    assert m["_attention_flops"] == pairs * D * 2 * 2                            # q.k and p.v
    assert m["alibi_attention_bwd"] == rows * D * 2 * 7 + rows * 4                # q, k, v, dO, dq, dk, dv; lse
    assert m["_attention_bwd_flops"] == pairs * D * 2 * 5                        # five products per pair
    assert round(m["_attention_flops"] / 1e9, 2) == 30.08
    assert round(m["_attention_bwd_flops"] / 1e9, 2) == 75.20


@pytest.mark.parametrize("batch", [16, 8, 1])
def test_optimizer_bytes(batch):
    m = _model(batch)
    assert m["adamw_step"] == N * (16 + 14)                    # acc, master, m, v in; master, m, v, bf16 out
    assert m["grad_accumulate_first"] == N * 6
    assert m["grad_accumulate"] == N * 10
    assert m["grad_accumulate_many_first"] == N * (2 * batch + 4)
    assert m["grad_accumulate_many"] == N * (2 * batch + 8)
    if batch == 16:
        assert m["grad_accumulate_many_last"] == 146_800_000_000


def test_step_bytes_one_pass_per_micro_batch():
    """The headline step: six fused kernels, then one accumulation pass per
    micro-batch (6 B per element for the first, 10 B for each of the other 31)
    and the 30 B per element AdamW step."""
    m = _model(16)
    fused = sum(m[k] for k in ("layernorm_fwd", "layernorm_bwd", "alibi_softmax_fwd", "alibi_softmax_bwd",
                               "bias_gelu_fwd", "bias_gelu_bwd"))
    assert bench.step_bytes(m, 32) == fused + N * (6 + 31 * 10 + 30)
    assert round((bench.step_bytes(m, 32) - fused) / 1e12, 3) == 1.270


def test_copy_ceiling_patterns():
    """Each kernel's ceiling copies what it reads and writes."""
    pat = bench.copy_patterns({"ln": (R, H), "sm": (B, NH, L), "gelu": (R, H), "head_dim": D}, N)
    assert pat["1in_1out_act"] == (1, 1, R * H * 2)
    assert pat["2in_1out_act"] == (2, 1, R * H * 2)
    causal = B * NH * L * (L + 1) // 2 * 2
    assert pat["1in_2out_causal"][:2] == (1, 2) and causal - 16 < pat["1in_2out_causal"][2] <= causal
    assert pat["2in_2out_causal"][:2] == (2, 2)
    assert pat["1in_1out_fp32_shard"] == (1, 1, N * 4)
    for k, c in bench.CEILING_OF.items():
        assert c in pat, k


def test_cpu_share_respects_the_thread_allotment(monkeypatch):
    monkeypatch.setenv("OMP_NUM_THREADS", "3")
    assert 1 <= bench.cpu_share() <= 3
    monkeypatch.delenv("OMP_NUM_THREADS")
    assert bench.cpu_share() >= 1


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("batch", ["3", "1", "17", "32", "-1"])
def test_accumulation_batch_must_split_the_32_micro_batches(batch):
    r = _run("--accum-batch", batch)
    assert r.returncode == 2 and "--accum-batch" in r.stderr


def test_counter_traffic_only_for_the_measured_source(tmp_path, monkeypatch):
    src = ["bloom_bf16_optimizer_amd/csrc/optimizer.hip", "bloom_bf16_optimizer_amd/csrc/device_common.h"]
    good = {"grad_accumulate_many_last": {"sources": src, "source_digest": bench.source_digest(*src),
                                          "hbm_bytes_per_launch": 123}}   # any key works the same way
    p = tmp_path / "counters.json"
    p.write_text(json.dumps(good))
    monkeypatch.setattr(bench, "COUNTERS", str(p))
    assert bench.measured_traffic("grad_accumulate_many_last") == 123
    assert bench.measured_traffic("adamw_step") is None
    good["grad_accumulate_many_last"]["source_digest"] = "0" * 16     # source changed since the counters
    p.write_text(json.dumps(good))
    assert bench.measured_traffic("grad_accumulate_many_last") is None


def test_committed_counters_match_the_current_source():
    data = json.load(open(os.path.join(ROOT, "profiles", "counters.json")))
    assert "grad_accumulate" in data       # the roofline kernel of the step
    for key, entry in data.items():
        assert entry["source_digest"] == bench.source_digest(*entry["sources"]), key


def test_long_context_rows():
    m = bench.long_context_model(8192, H, 1, NH, 8192, D)
    assert m["layernorm_fwd_8192"] == 8192 * H * 2 * 2 + H * 2 * 2 + 8192 * 4 * 2
    causal = NH * 8192 * 8193 // 2
    assert m["alibi_softmax_fwd_8192"] == causal * 2 + NH * 8192 * 8192 * 2
    assert m["alibi_attention_fwd_8192"] == NH * 8192 * D * 2 * 4 + NH * 8192 * 4
    assert m["_attention_flops_8192"] == causal * D * 2 * 2
    assert round(m["layernorm_fwd_8192"] / 1e6, 1) == 469.9
    assert round(m["alibi_softmax_fwd_8192"] / 1e9, 2) == 5.64
    assert round(m["_attention_flops_8192"] / 1e9, 2) == 481.10


def test_mini_rows():
    m = bench.mini_model()
    rows, hid, heads, seq, ffn = 4 * 2048, 2048, 16, 2048, 8192
    causal = 4 * heads * seq * (seq + 1) // 2
    assert m["layernorm_fwd_mini"] == rows * hid * 4 + hid * 4 + rows * 8
    assert m["layernorm_bwd_mini"] == rows * hid * 6 + hid * 2 + rows * 8 + hid * 4
    assert m["alibi_softmax_fwd_mini"] == causal * 2 + 4 * heads * seq * seq * 2
    assert m["alibi_softmax_bwd_mini"] == causal * 4 + 4 * heads * seq * seq * 2
    assert m["bias_gelu_fwd_mini"] == rows * ffn * 4 + ffn * 2
    assert m["bias_gelu_bwd_mini"] == rows * ffn * 6 + ffn * 4
    n_mini = 24 * (12 * hid ** 2 + 13 * hid) + 250880 * hid     # 24 layers plus the embedding
    assert n_mini == 1_722_400_768 and m["adamw_step_mini"] == n_mini * 30
