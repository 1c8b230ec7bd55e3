"""GPU parity of the streaming matrix-core decode (int8, FP8 and NVFP4 caches
whose G * Tq rows of a kv head fit one 16-row tile: each wave runs its own
blocks, keys and values copied straight into LDS) against the fp64 oracle.

Beyond the shared grid in test_gpu_parity.py: value scales spread over 2^12
(the per-wave value-scale reference is raised and the output rescaled),
all-zero rows (scale 0), partitions shorter than the four waves' blocks,
causal rows with G * Tq <= 16, every head size with fp32 and bf16 queries, and
given partitions above 4096 tokens (the tiled kernel takes those).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import paged_attention_decode_02_amd as pa
from _gpu import cache_bytes_equal, gpu_cache, gpu_decode
from _host import oracle_cache, oracle_decode
from workloads import generate, scaled

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def parity(w, P, tol=2e-2, rel=0.0):
    say("stream: %s B=%d Tq=%d Hq=%d Hkv=%d D=%d kv=%s q=%s max_len=%d P=%d" % (
        w.spec.name, w.spec.B, w.spec.Tq, w.spec.Hq, w.spec.Hkv, w.spec.D, w.spec.cache_dtype, w.spec.q_dtype,
        w.max_seq_len, P))
    host = oracle_cache(w)
    cache = gpu_cache(w)
    assert cache_bytes_equal(cache, host)
    out, lse = gpu_decode(w, cache, P)
    ref, rlse = oracle_decode(w, host)
    o = out.cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64)
    err = np.abs(o - ref)
    bound = tol + rel * np.max(np.abs(ref)) if ref.size else tol
    fin = np.isfinite(rlse)
    lerr = float(np.max(np.abs(l[fin] - rlse[fin]))) if fin.any() else 0.0
    say("  max|out-oracle| = %.3e (bound %.3e), max|lse-oracle| = %.3e" % (float(err.max()) if err.size else 0.0,
                                                                           bound, lerr))
    assert np.all(np.isfinite(o))
    assert np.array_equal(np.isneginf(l), np.isneginf(rlse))
    assert float(err.max()) <= bound
    assert lerr <= 1e-3


TORCH_KV = {"i8": torch.int8, "fp8": torch.float8_e4m3fn, "nvfp4": torch.float4_e2m1fn_x2}


@pytest.mark.parametrize("kv", ["i8", "fp8", "nvfp4"])
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("qdt", ["bf16", "f32"])
def test_head_sizes_and_query_types(kv, D, qdt):
    assert pa.decode_kernel_name(1, 12, 2, TORCH_KV[kv]) == "decode_stream_kernel"
    spec = scaled("int8_250k", B=3, Tq=1, Hq=12, Hkv=2, D=D, seq_lens=(1, 3000), cache_dtype=kv, q_dtype=qdt)
    w = generate(spec, seed=50 + D, seq_lens=[1, 777, 3000])
    for P in (64, 512, 0):
        parity(w, P)


@pytest.mark.parametrize("kv", ["i8", "fp8", "nvfp4"])
@pytest.mark.parametrize("Tq, G", [(2, 8), (4, 4), (16, 1), (3, 5)])
def test_causal_rows_in_one_tile(kv, Tq, G):
    spec = scaled("int8_250k", B=4, Tq=Tq, Hq=2 * G, Hkv=2, D=128, seq_lens=(Tq, 900), cache_dtype=kv)
    w = generate(spec, seed=60 + Tq, seq_lens=[Tq, Tq + 5, 333, 900])
    for P in (16, 128, 0):
        parity(w, P)


@pytest.mark.parametrize("kv", ["i8", "fp8", "nvfp4"])
def test_value_scales_spread_over_many_octaves(kv):
    # value rows scaled per token by 2^u, u uniform in [-6, 6]; a few all-zero
    # key and value rows (scale 0): the waves' value-scale references are
    # raised as larger scales appear, the output rescaled exactly
    spec = scaled("int8_250k", B=2, Tq=1, Hq=6, Hkv=1, D=256, seq_lens=(2500, 4000), cache_dtype=kv)
    w = generate(spec, seed=70)
    rng = np.random.default_rng(71)
    f = np.exp2(rng.uniform(-6, 6, size=w.v_src.shape[0])).astype(np.float32)
    w.v_src = (w.v_src * f[:, None, None]).astype(np.float32)
    zero = rng.choice(w.v_src.shape[0], 50, replace=False)
    w.v_src[zero] = 0.0
    w.k_src[zero[:25]] = 0.0
    # f16 weights times scales: relative error about 2^-11 of the largest value
    for P in (256, 0):
        parity(w, P, tol=2e-2, rel=2e-3)


@pytest.mark.parametrize("kv", ["i8", "nvfp4"])
def test_short_partitions_leave_waves_idle(kv):
    # partitions of 16 and 32 tokens: one or two of the four waves have blocks
    spec = scaled("int8_250k", B=2, Tq=1, Hq=6, Hkv=1, D=128, seq_lens=(5, 200), cache_dtype=kv)
    w = generate(spec, seed=80, seq_lens=[5, 200])
    for P in (16, 32, 48):
        parity(w, P)


def test_given_partition_above_the_streaming_cap():
    # 8192-token partitions: the tiled matrix-core kernel runs them
    spec = scaled("int8_250k", B=1, Tq=1, Hq=6, Hkv=1, D=256, seq_lens=(20000, 20000))
    w = generate(spec, seed=90)
    parity(w, 8192)
    parity(w, 4096)
