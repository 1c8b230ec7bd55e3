"""GPU parity on seeded random shapes: every decode path (vector-ALU, streaming
and tiled matrix-core, fp32) chosen by the library's own rule, against the
fp64 oracle, with random cache and query dtypes, head sizes, group sizes,
query tokens, ragged lengths (some shorter than a block, some a whole number
of blocks) and given or heuristic partition sizes, some with 1% peaked keys;
the shared-prefix call on random batches, prefixes and partition sizes (its
reference is the same plain definition); and the sparse block-selection decode
on random sparse-block sizes, selection sizes and empty sequences (the
selection checked against its validity rule, the output against the oracle on
the GPU's own selection). The configurations are drawn from fixed seeds, so a
failure names a reproducible case."""
from __future__ import annotations

import numpy as np
import pytest

from test_gpu_parity import run_workload
from workloads import generate, scaled

pytestmark = pytest.mark.gpu

N_CASES = 200


def case(i: int) -> dict:
    rng = np.random.default_rng(1000 + i)
    kv = str(rng.choice(["f32", "bf16", "i8", "fp8", "nvfp4"]))
    D = int(rng.choice([64, 128, 256]))
    Hkv = int(rng.choice([1, 2, 3, 4, 8]))
    G = int(rng.choice([1, 2, 3, 4, 5, 6, 7, 8, 12, 16, 20, 24, 32]))
    Tq = int(rng.choice([1, 1, 1, 2, 3, 4, 5, 8, 16]))
    B = int(rng.integers(1, 5))
    hi = int(rng.integers(Tq, 2200))
    lens = [int(x) for x in rng.integers(Tq, hi + 1, size=B)]
    if rng.random() < 0.3:  # a whole number of blocks
        lens[0] = max(Tq, 16 * (lens[0] // 16))
    if rng.random() < 0.3:  # shorter than one block
        lens[-1] = int(rng.integers(Tq, Tq + 16))
    P = int(rng.choice([0, 0, 16, 64, 256, 16 * int(rng.integers(1, 80))]))
    return dict(kv=kv, D=D, Hkv=Hkv, Hq=G * Hkv, Tq=Tq, B=B, lens=lens, P=P,
                q=str(rng.choice(["f32", "bf16"])), src=str(rng.choice(["f32", "bf16"])),
                peaked=bool(rng.random() < 0.2))


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape(i):
    c = case(i)
    spec = scaled("gqa_bf16", name="random%d" % i, B=c["B"], Tq=c["Tq"], Hq=c["Hq"], Hkv=c["Hkv"], D=c["D"],
                  seq_lens=(min(c["lens"]), max(c["lens"])), cache_dtype=c["kv"], q_dtype=c["q"],
                  src_dtype=c["src"], peaked_frac=0.01 if c["peaked"] else 0.0)
    print("random case %d: %s" % (i, c), flush=True)
    w = generate(spec, seed=2000 + i, seq_lens=c["lens"])
    run_workload(w, partition_size=c["P"])


# ------------------------------------------------------------ shared prefix
N_SHARED = 60


def shared_case(i: int) -> dict:
    rng = np.random.default_rng(5000 + i)
    kv = str(rng.choice(["bf16", "i8", "fp8", "nvfp4"]))
    D = int(rng.choice([64, 128, 256]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 3, 4, 6, 8, 12, 16]))
    Tq = int(rng.choice([1, 1, 2, 3, 5, 8, 16]))
    B = int(rng.integers(1, 7))
    prefix = 16 * int(rng.integers(1, 80))
    # every query token after the prefix: prefix + Tq <= L
    lens = [int(x) for x in rng.integers(prefix + Tq, prefix + Tq + int(rng.integers(1, 1500)), size=B)]
    pp = int(rng.choice([0, 0, 16, 64, 16 * int(rng.integers(1, 40))]))
    tp = int(rng.choice([0, 0, 16, 128, 16 * int(rng.integers(1, 40))]))
    return dict(kv=kv, D=D, Hkv=Hkv, Hq=G * Hkv, Tq=Tq, B=B, prefix=prefix, lens=lens, pp=pp, tp=tp,
                q=str(rng.choice(["f32", "bf16"])))


@pytest.mark.parametrize("i", range(N_SHARED))
def test_random_shared_prefix(i):
    from test_gpu_shared_prefix import run_shared

    c = shared_case(i)
    spec = scaled("verify_bf16", name="random_shared%d" % i, B=c["B"], Tq=c["Tq"], Hq=c["Hq"], Hkv=c["Hkv"],
                  D=c["D"], seq_lens=(min(c["lens"]), max(c["lens"])), shared_prefix=c["prefix"],
                  cache_dtype=c["kv"], q_dtype=c["q"], src_dtype="f32")
    print("random shared-prefix case %d: %s" % (i, c), flush=True)
    w = generate(spec, seed=6000 + i, seq_lens=c["lens"])
    run_shared(w, parts=((c["pp"], c["tp"]),))


# ------------------------------------------------------------ sparse selection
N_SPARSE = 60


def sparse_case(i: int) -> dict:
    rng = np.random.default_rng(7000 + i)
    kv = str(rng.choice(["bf16", "i8", "fp8", "nvfp4"]))
    D = int(rng.choice([64, 128, 256]))
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 4, 6, 8, 12]))
    Tq = int(rng.choice([1, 1, 2, 4, 8]))
    B = int(rng.integers(1, 5))
    SB = int(rng.choice([16, 32, 64, 128, 256]))
    lens = [int(x) for x in rng.integers(Tq, 3000, size=B)]
    if rng.random() < 0.2:  # an empty sequence
        lens[0] = 0
    top = int(rng.choice([1, 2, 5, 17, 64, 200]))
    P = int(rng.choice([0, 0, 64, 16 * int(rng.integers(1, 64))]))
    return dict(kv=kv, D=D, Hkv=Hkv, Hq=G * Hkv, Tq=Tq, B=B, SB=SB, lens=lens, top=top, P=P,
                peaked=bool(rng.random() < 0.3))


@pytest.mark.parametrize("i", range(N_SPARSE))
def test_random_sparse(i):
    from test_gpu_sparse import run_sparse

    c = sparse_case(i)
    spec = scaled("gqa_bf16", name="random_sparse%d" % i, B=c["B"], Tq=c["Tq"], Hq=c["Hq"], Hkv=c["Hkv"], D=c["D"],
                  seq_lens=(min(c["lens"]), max(c["lens"])), cache_dtype=c["kv"], src_dtype="f32",
                  peaked_frac=0.01 if c["peaked"] else 0.0)
    print("random sparse case %d: %s" % (i, c), flush=True)
    w = generate(spec, seed=8000 + i, seq_lens=c["lens"])
    run_sparse(w, c["SB"], c["top"], P=c["P"])
