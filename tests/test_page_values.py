"""The workload constants are the numbers the pages print (CPU only)."""

import json
import os

from synth import workloads as W

PAGES = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_values.json")))["values"]


def v(name):
    return PAGES[name]["value"]


def test_optimizer_hyperparameters():
    assert W.LR == v("adamw_lr")
    assert W.WEIGHT_DECAY == v("adamw_weight_decay")
    assert W.MAX_GRAD_NORM == v("clip_grad_global_norm")
    assert W.OPTIMIZER.opt.microbatches == v("gradient_accumulation_steps")


def test_shard_shapes():
    assert W.SHARD.ln.hidden == v("bloom_hidden_size")
    assert W.SHARD.gelu.cols == v("bloom_hidden_size") * 4 // v("tensor_parallel_degree")
    assert W.SHARD.softmax.seq == v("sequence_length")
    assert W.SHARD.ln.rows == v("sequence_length") * v("micro_batch_per_gpu_176b")
    assert W.LONG.softmax.seq == v("alibi_extrapolated_length")
    # the shard of one GPU: 176e9 parameters over TP 4 and PP 12
    per_gpu = v("bloom_parameters") / (v("tensor_parallel_degree") * v("pipeline_parallel_degree"))
    assert abs(W.SHARD_N - per_gpu) / W.SHARD_N < 2e-3


def test_mini_shapes():
    assert W.MINI_HIDDEN == v("mini_hidden_size") == W.MINI.ln.hidden
    assert W.MINI_LAYERS == v("mini_num_layers")
    assert W.VOCAB == v("mini_vocab_size")
    assert W.MINI.softmax.heads == v("mini_num_heads")
    assert W.MINI.ln.rows == v("mini_micro_batch") * v("sequence_length")
    assert W.MINI.gelu.cols == 4 * v("mini_hidden_size")
