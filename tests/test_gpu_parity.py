"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerances: max|out - oracle| <= 1e-2 for fp32/bf16 caches and <= 2e-2 for
int8 and FP8 caches (fp32 accumulation over 16-bit operands); cache bytes and
block indexing are bit-exact. The oracle runs on the oracle writer's caches,
the GPU on pa_cache_write's caches, after checking the two are identical.
"""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import paged_attention_decode_02_amd as pa
from _gpu import cache_bytes_equal, dev, dev_to_host, gpu_cache, gpu_decode, gpu_inputs, host_to_dev
import oracle
from _host import oracle_cache, oracle_decode
from _refs import nvfp4_split, nvfp4_token_bytes
from workloads import BLOCK_SIZE, SPECS, generate, scaled

pytestmark = pytest.mark.gpu

# fp8: the int8 bound (the oracle dequantises the same codes, so the bound
# covers only the kernel's 16-bit operands and fp32 sums, as for int8)
TOL = {"f32": 1e-2, "bf16": 1e-2, "i8": 2e-2, "fp8": 2e-2, "nvfp4": 2e-2}
LSE_TOL = 1e-3


def say(*a):
    print(*a, flush=True)


def check(w, got, ref, tag=""):
    out, lse = got
    rout, rlse = ref
    o = dev_to_host(out).astype(np.float64) if out.dtype != torch.bfloat16 else \
        dev_to_host(out.float())
    l = dev_to_host(lse).astype(np.float64)
    err = float(np.max(np.abs(o - rout))) if o.size else 0.0
    finite = np.isfinite(rlse)
    lerr = float(np.max(np.abs(l[finite] - rlse[finite]))) if finite.any() else 0.0
    say("%s %s: max|out-oracle| = %.3e  max|lse-oracle| = %.3e" % (w.spec.name, tag, err, lerr))
    assert np.all(np.isfinite(o)), "non-finite output"
    assert np.array_equal(np.isneginf(l), np.isneginf(rlse)), "rows without keys must give lse = -inf"
    assert err <= TOL[w.spec.cache_dtype], err
    assert lerr <= LSE_TOL, lerr
    return err


def run_workload(w, partition_size=0, check_cache=True):
    say("workload %s B=%d Tq=%d Hq=%d Hkv=%d D=%d max_len=%d P=%d" % (
        w.spec.name, w.spec.B, w.spec.Tq, w.spec.Hq, w.spec.Hkv, w.spec.D, w.max_seq_len, partition_size))
    host = oracle_cache(w)
    cache = gpu_cache(w)
    if check_cache:
        assert cache_bytes_equal(cache, host), "pa_cache_write differs from the oracle writer"
    got = gpu_decode(w, cache, partition_size)
    ref = oracle_decode(w, host)
    return check(w, got, ref, "P=%d" % partition_size), cache, host, got


# ------------------------------------------------------------ full workloads
@pytest.mark.parametrize("name", ["tiny_f32", "gqa_bf16", "long64k_bf16", "int8_250k", "verify_bf16", "verify_i8",
                                  "fp8_250k", "verify_fp8", "nvfp4_250k", "verify_nvfp4"])
def test_named_workload_full_size(name):
    w = generate(name)
    run_workload(w, partition_size=SPECS[name].partition_size)
    if SPECS[name].partition_size:
        # also the heuristic's partition size (the benchmark's launch)
        cache = gpu_cache(w)
        ref = oracle_decode(w, oracle_cache(w))
        check(w, gpu_decode(w, cache, 0), ref, "P=heuristic")


# ------------------------------------------------------------ dtype / shape grid
@pytest.mark.parametrize("kv", ["f32", "bf16", "i8", "fp8", "nvfp4"])
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("qdt", ["f32", "bf16"])
def test_dtype_and_head_dim_grid(kv, D, qdt):
    spec = scaled("gqa_bf16", B=3, Tq=1, Hq=12, Hkv=2, D=D, seq_lens=(1, 700), q_dtype=qdt, src_dtype="f32",
                  cache_dtype=kv)
    w = generate(spec, seed=D + len(kv))
    run_workload(w, partition_size=128)


@pytest.mark.parametrize("G", [1, 2, 3, 4, 5, 6, 7, 8, 12, 16, 24])
def test_group_sizes(G):
    spec = scaled("gqa_bf16", B=2, Tq=1, Hq=2 * G, Hkv=2, D=128, seq_lens=(50, 600))
    run_workload(generate(spec, seed=G), partition_size=256)


@pytest.mark.parametrize("P", [16, 64, 256, 512, 2048, 8192])
def test_partition_sizes(P):
    spec = scaled("long64k_bf16", B=2, Tq=1, Hq=12, Hkv=2, D=256, seq_lens=(3000, 6000), peaked_frac=0.01)
    run_workload(generate(spec, seed=1), partition_size=P)


@pytest.mark.parametrize("Hkv", [1, 2, 3, 4, 6, 8])
@pytest.mark.parametrize("P", [16, 0])
@pytest.mark.parametrize("kv", ["bf16", "fp8", "nvfp4"])
def test_kv_heads_per_workgroup(Hkv, P, kv):
    # D=256, 6 heads per group: a workgroup takes 4 (bf16) or 2 (int8, fp8)
    # kv heads, or fewer as Hkv allows, one or more waves each; ragged and
    # empty rows
    spec = scaled("long64k_bf16", B=3, Tq=1, Hq=6 * Hkv, Hkv=Hkv, D=256, seq_lens=(0, 1500), peaked_frac=0.01,
                  cache_dtype=kv)
    w = generate(spec, seed=20 + Hkv, seq_lens=[0, 17, 1500])
    run_workload(w, partition_size=P)


@pytest.mark.parametrize("D", [64, 128, 256])
def test_reduce_splits_columns_of_few_rows(D):
    # more than 160 partitions of only 8 rows: the reduce spreads each row's
    # columns over several workgroups (4 to 16 by D)
    spec = scaled("gqa_bf16", B=2, Tq=1, Hq=4, Hkv=1, D=D, seq_lens=(2600, 3000))
    w = generate(spec, seed=30 + D, seq_lens=[2600, 3000])
    run_workload(w, partition_size=16)


@pytest.mark.parametrize("Tq", [2, 3, 8, 16])
@pytest.mark.parametrize("kv", ["f32", "bf16", "i8", "fp8", "nvfp4"])
def test_query_tokens_causal(Tq, kv):
    spec = scaled("verify_bf16", B=3, Tq=Tq, Hq=8, Hkv=2, D=128, seq_lens=(Tq, 900), shared_prefix=0,
                  cache_dtype=kv)
    run_workload(generate(spec, seed=Tq), partition_size=256)


@pytest.mark.parametrize("Tq", [1, 3])
def test_f32_cache_head_chunks_and_empty_rows(Tq):
    # the fp32-cache kernel with a group of 12 query heads (two head chunks of
    # at most 8), rows with no key and ragged lengths, several partitions
    spec = scaled("gqa_bf16", B=4, Tq=Tq, Hq=24, Hkv=2, D=64, seq_lens=(0, 700), src_dtype="f32",
                  cache_dtype="f32", q_dtype="f32")
    w = generate(spec, seed=40 + Tq, seq_lens=[0, Tq, 37, 700])
    for P in (16, 0):
        run_workload(w, partition_size=P)


def test_empty_and_short_rows():
    spec = scaled("verify_bf16", B=5, Tq=4, Hq=4, Hkv=2, D=64, seq_lens=(0, 40), shared_prefix=0)
    w = generate(spec, seed=3, seq_lens=[0, 1, 3, 4, 37])
    for P in (16, 0):
        run_workload(w, partition_size=P)


def test_bf16_output():
    spec = scaled("gqa_bf16", B=2, Tq=1, Hq=8, Hkv=2, D=128, seq_lens=(100, 900))
    w = generate(spec, seed=4)
    host = oracle_cache(w)
    cache = gpu_cache(w)
    out, lse = gpu_decode(w, cache, 256, out_dtype=torch.bfloat16)
    rout, _ = oracle_decode(w, host)
    o = out.float().cpu().numpy()
    # bf16 output adds at most half a bf16 ulp of |out| to the fp32 error
    assert np.all(np.abs(o - rout) <= 1e-2 + np.abs(rout) * 2.0 ** -8)


# ------------------------------------------------------------ exact indexing
def test_index_probe_exact():
    """V rows encode their logical position; one key per row dominates by a
    logit margin of 128, so every other weight underflows to exactly 0 and the
    output must decode to that key's position exactly."""
    B, Hq, Hkv, D = 24, 4, 2, 64
    rng = np.random.default_rng(5)
    lens = rng.integers(1, 3000, size=B)
    lens[:4] = [1, 16, 17, 2047]
    spec = scaled("gqa_bf16", B=B, Tq=1, Hq=Hq, Hkv=Hkv, D=D, seq_lens=(1, 3000), src_dtype="f32",
                  cache_dtype="bf16", q_dtype="bf16")
    w = generate(spec, seed=5, seq_lens=lens)
    chosen = np.array([int(rng.integers(0, L)) for L in lens])
    chosen[:4] = [0, 15, 16, 2046]
    k = np.zeros_like(w.k_src)
    v = np.zeros_like(w.v_src)
    v[:, :, 0] = (w.row_pos >> 8)[:, None]
    v[:, :, 1] = (w.row_pos & 255)[:, None]
    for b in range(B):
        i = np.nonzero((w.row_seq == b) & (w.row_pos == chosen[b]))[0][0]
        k[i, :, 0] = 1024.0
    w.k_src, w.v_src = k, v
    w.q[:] = 0.0
    w.q[..., 0] = 1.0
    w.q_bits = None
    w.spec = scaled(w.spec, q_dtype="f32")
    w.softmax_scale = 0.125
    cache = gpu_cache(w)
    for P in (16, 128, 0):
        out, _ = gpu_decode(w, cache, P)
        o = out.cpu().numpy()
        pos = o[:, 0, :, 0] * 256 + o[:, 0, :, 1]
        assert np.array_equal(pos, np.repeat(chosen[:, None], Hq, axis=1).astype(np.float32)), P
        assert np.all(o[:, 0, :, 2:] == 0)


def test_single_key_is_exact():
    spec = scaled("gqa_bf16", B=3, Tq=1, Hq=8, Hkv=2, D=256, seq_lens=(1, 1))
    w = generate(spec, seed=6)
    host = oracle_cache(w)
    cache = gpu_cache(w)
    out, _ = gpu_decode(w, cache)
    ref, _ = oracle_decode(w, host)
    assert np.array_equal(out.cpu().numpy().astype(np.float64), ref)


def test_permuted_table_and_reruns_are_bitwise_identical():
    spec = scaled("long64k_bf16", B=2, Tq=1, Hq=12, Hkv=2, D=256, seq_lens=(1000, 3000), peaked_frac=0.01)
    w = generate(spec, seed=7)
    cache = gpu_cache(w)
    a, la = gpu_decode(w, cache, 256)
    b, lb = gpu_decode(w, cache, 256)
    assert torch.equal(a, b) and torch.equal(la, lb)
    perm = torch.from_numpy(np.random.default_rng(8).permutation(w.num_blocks)).to(dev())
    moved = []
    for c in cache:
        if c is None:
            moved.append(None)
            continue
        m = torch.empty_like(c)
        m[perm] = c
        moved.append(m)
    w.block_table = perm.cpu().numpy()[w.block_table].astype(np.int32)
    c2, l2 = gpu_decode(w, tuple(moved), 256)
    assert torch.equal(a, c2) and torch.equal(la, l2)


@pytest.mark.parametrize("kv, Tq, G", [("i8", 1, 6), ("fp8", 1, 6), ("nvfp4", 1, 6), ("bf16", 8, 6), ("i8", 8, 6),
                                       ("fp8", 8, 6), ("nvfp4", 8, 6), ("f32", 1, 4), ("bf16", 1, 4)])
def test_every_kernel_is_deterministic_and_placement_independent(kv, Tq, G):
    # each decode kernel (streaming, tiled, fp32, vector ALU) gives the same
    # bits on reruns and with its blocks moved to other places in the pool
    spec = scaled("verify_bf16", name="determinism_%s_T%d" % (kv, Tq), B=3, Tq=Tq, Hq=2 * G, Hkv=2, D=128,
                  seq_lens=(Tq, 2500), shared_prefix=0, cache_dtype=kv, src_dtype="f32",
                  q_dtype="f32" if kv == "f32" else "bf16", peaked_frac=0.01)
    w = generate(spec, seed=31 + Tq + G, seq_lens=[Tq, 1300, 2500])
    cache = gpu_cache(w)
    a, la = gpu_decode(w, cache, 128)
    for _ in range(3):
        b, lb = gpu_decode(w, cache, 128)
        assert torch.equal(a, b) and torch.equal(la, lb)
    perm = torch.from_numpy(np.random.default_rng(9).permutation(w.num_blocks)).to(dev())
    moved = []
    for c in cache:
        if c is None:
            moved.append(None)
            continue
        m = torch.empty_like(c)
        if c.dtype in (torch.float8_e4m3fn, torch.float4_e2m1fn_x2):  # byte codes: move the bytes
            m.view(torch.uint8)[perm] = c.view(torch.uint8)
        else:
            m[perm] = c
        moved.append(m)
    w.block_table = perm.cpu().numpy()[w.block_table].astype(np.int32)
    c2, l2 = gpu_decode(w, tuple(moved), 128)
    assert torch.equal(a, c2) and torch.equal(la, l2)


def test_splitk_reduce_entry_point_matches_decode():
    """decode_partials + splitk_reduce called separately give decode()'s bits."""
    spec = scaled("gqa_bf16", B=2, Tq=2, Hq=8, Hkv=2, D=128, seq_lens=(500, 1500))
    w = generate(spec, seed=9)
    cache = gpu_cache(w)
    q, table, lens = gpu_inputs(w)
    k, v, ks, vs = cache
    ref, rlse = pa.decode(q, k, v, table, lens, w.max_seq_len, w.softmax_scale, partition_size=256)
    nbytes = pa.workspace_bytes(2, 2, 8, 2, 128, torch.bfloat16, w.max_seq_len, 256)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev())
    out = torch.empty_like(ref)
    lse = torch.empty_like(rlse)
    np_ = pa.decode_partials(q, k, v, table, lens, w.max_seq_len, w.softmax_scale, out, lse, partition_size=256,
                             workspace=ws)
    assert np_ == (w.max_seq_len + 255) // 256
    pa.splitk_reduce(ws, np_, 256, lens, out, lse)
    torch.cuda.synchronize()
    assert torch.equal(out, ref) and torch.equal(lse, rlse)


def test_input_checks_find_planted_violations():
    """pa_decode_check / pa_cache_write_check: clean inputs give (0, -1);
    planted out-of-range block ids, lengths and slots are counted and the
    first one is named. Only the table, lengths and slots are read."""
    spec = scaled("gqa_bf16", B=3, Hq=4, Hkv=2, D=64, seq_lens=(40, 300))
    w = generate(spec, seed=12)
    q, table, lens = gpu_inputs(w)
    nb, mb = w.num_blocks, w.block_table.shape[1]
    st = pa.decode_check(table, lens, w.max_seq_len, nb)
    assert st.cpu().tolist() == [0, -1]
    bad_t = w.block_table.copy()
    used1 = (int(w.seq_lens[1]) + 15) // 16
    bad_t[1, used1 - 1] = nb  # one past the pool, in a used block of sequence 1
    bad_t[2, 0] = -3
    bad_t[0, mb - 1] = 10 ** 6  # past sequence 0's end (if unused): not read, not counted
    bad_l = w.seq_lens.copy()
    bad_l[2] = w.max_seq_len + 1  # longer than max_seq_len (its table row stays in bounds)
    st = pa.decode_check(torch.from_numpy(bad_t).to(dev()), torch.from_numpy(bad_l).to(dev()), w.max_seq_len, nb)
    flagged = [1 * (mb + 1) + used1 - 1, 2 * (mb + 1) + 0, 2 * (mb + 1) + mb]
    if (int(w.seq_lens[0]) + 15) // 16 >= mb:  # sequence 0 uses its last entry
        flagged.append(mb - 1)
    got = st.cpu().tolist()
    assert got == [len(flagged), min(flagged)], (got, flagged)
    slots = torch.from_numpy(w.slot_mapping.copy()).to(dev())
    assert pa.cache_write_check(slots, nb).cpu().tolist() == [0, -1]
    slots[5] = nb * 16
    slots[9] = -1  # skip: valid
    slots[11] = nb * 16 + 100
    assert pa.cache_write_check(slots, nb).cpu().tolist() == [2, 5]


def test_fp8_cache_write_of_hand_derived_rows():
    """The hand-derived E4M3 rows (ties to even, subnormals, saturation, signed
    zero, all-zero row) written by the GPU equal the oracle writer's bits."""
    import json

    with open(os.path.join(os.path.dirname(__file__), "golden", "fp8_e4m3_cases.json")) as f:
        rows = json.load(f)["rows"]
    D = 64
    x = np.zeros((len(rows), 1, D), np.float32)
    for i, c in enumerate(rows):
        x[i, 0, :len(c["x"])] = c["x"]
    N = len(rows)
    hk, hv, hks, hvs = oracle.alloc_cache(1, BLOCK_SIZE, 1, D, "fp8")
    oracle.cache_write(x, x, np.arange(N), hk, hv, hks, hvs)
    k = torch.zeros((1, BLOCK_SIZE, 1, D), dtype=torch.uint8, device=dev()).view(torch.float8_e4m3fn)
    v = k.clone()
    ks = torch.zeros((1, 1, BLOCK_SIZE), dtype=torch.float32, device=dev())
    vs = ks.clone()
    src = torch.from_numpy(x).to(dev())
    pa.cache_write(src, src, torch.arange(N, dtype=torch.int64, device=dev()), k, v, ks, vs)
    torch.cuda.synchronize()
    assert np.array_equal(dev_to_host(k)[0, :N], hk[0, :N])
    assert np.array_equal(dev_to_host(v)[0, :N], hv[0, :N])
    assert np.array_equal(ks.cpu().numpy()[0, 0, :N].view(np.uint32), hks[0, 0, :N].view(np.uint32))
    for i, c in enumerate(rows):
        assert dev_to_host(k)[0, i, 0, :len(c["codes"])].tolist() == c["codes"], c["why"]


def test_nvfp4_cache_write_of_the_hand_derived_row():
    """The hand-derived NVFP4 row (ties to even, saturation, block scales
    rounded to E4M3, zero blocks) written by the GPU to token 5 of a block
    equals the oracle writer's bytes and the hand-derived codes, and leaves
    the other tokens' bytes of the block alone."""
    import json

    with open(os.path.join(os.path.dirname(__file__), "golden", "nvfp4_cases.json")) as f:
        row = json.load(f)["row"]
    D = 128
    x = np.zeros((1, 1, D), np.float32)
    for b, blk in enumerate(row["blocks"]):
        x[0, 0, 16 * b: 16 * b + len(blk["x"])] = blk["x"]
    hk, hv, hks, hvs = oracle.alloc_cache(1, BLOCK_SIZE, 1, D, "nvfp4")
    hk[:] = 0x55
    hv[:] = 0x55
    oracle.cache_write(x, x, np.array([5]), hk, hv, hks, hvs)
    RB = oracle.nvfp4_row_bytes(D)
    k = torch.full((1, BLOCK_SIZE, 1, RB), 0x55, dtype=torch.uint8, device=dev()).view(torch.float4_e2m1fn_x2)
    v = k.clone()
    ks = torch.zeros((1, 1, BLOCK_SIZE), dtype=torch.float32, device=dev())
    vs = ks.clone()
    src = torch.from_numpy(x).to(dev())
    pa.cache_write(src, src, torch.full((1,), 5, dtype=torch.int64, device=dev()), k, v, ks, vs)
    torch.cuda.synchronize()
    assert np.array_equal(dev_to_host(k), hk) and np.array_equal(dev_to_host(v), hv)
    assert ks.cpu().numpy()[0, 0, 5] == hks[0, 0, 5] == np.float32(row["row_scale"])
    codes, scales = nvfp4_split(dev_to_host(k), D)
    for b, blk in enumerate(row["blocks"]):
        assert scales[0, 5, 0, b] == blk["scale_code"], b
        assert codes[0, 5, 0, 16 * b: 16 * b + len(blk["codes"])].tolist() == blk["codes"], b


def _slot_bytes(c: np.ndarray, slots: np.ndarray, spec) -> np.ndarray:
    """The storage of the given slots: [n, Hkv(, last dim)] for rows and
    scales, or for an NVFP4 cache the bytes of each token spread over its block."""
    if c.ndim == 4 and spec.cache_dtype == "nvfp4":
        idx = np.stack([nvfp4_token_bytes(spec.Hkv, spec.D, t) for t in range(BLOCK_SIZE)])
        return c.reshape(c.shape[0], -1)[slots[:, None] // BLOCK_SIZE, idx[slots % BLOCK_SIZE]]
    if c.ndim == 3:  # scales [num_blocks, Hkv, 16]
        return np.swapaxes(c, 1, 2).reshape(-1, spec.Hkv)[slots]
    return c.reshape((-1, spec.Hkv) + c.shape[3:])[slots]


def test_cache_write_skips_negative_slots_and_writes_bits():
    for cache_dtype in ("f32", "bf16", "i8", "fp8", "nvfp4"):
        for src in ("f32", "bf16"):
            spec = scaled("gqa_bf16", B=2, Hq=4, Hkv=2, D=64, seq_lens=(30, 70), src_dtype=src,
                          cache_dtype=cache_dtype)
            w = generate(spec, seed=10)
            w.slot_mapping = w.slot_mapping.copy()
            w.slot_mapping[::7] = -1
            host = oracle_cache(w, poison=False)
            cache = gpu_cache(w)
            # skipped rows' slots stay poisoned on the GPU; compare only written slots
            written = w.slot_mapping[w.slot_mapping >= 0]
            for g, h in zip(cache, host):
                if g is None:
                    continue
                a = _slot_bytes(dev_to_host(g), written, spec)
                hb = _slot_bytes(h, written, spec)
                if a.dtype == np.float32:
                    assert np.array_equal(a.view(np.uint32), hb.view(np.uint32))
                else:
                    assert np.array_equal(a, hb)
            # slots of skipped rows were never written: still poison
            sk_rows = np.arange(w.slot_mapping.size)[::7]
            b_ = w.row_seq[sk_rows]
            p_ = w.row_pos[sk_rows]
            sslots = w.block_table[b_, p_ // BLOCK_SIZE].astype(np.int64) * BLOCK_SIZE + p_ % BLOCK_SIZE
            kc = _slot_bytes(dev_to_host(cache[0]), sslots, spec)
            if kc.dtype in (np.int8, np.uint8):
                assert np.all(kc == 127)
            elif kc.dtype == np.uint16:
                assert np.all(kc == 0x7FC0)
            else:
                assert np.all(np.isnan(kc))


# ------------------------------------------------------------ matrix-core path
# Tq > 1, G >= 16, and int8 / fp8 with G >= 6 run on the MFMA kernel (bf16 / int8 /
# fp8 / nvfp4 caches), including row counts below one 16-row tile.
@pytest.mark.parametrize("kv", ["bf16", "i8", "fp8", "nvfp4"])
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("G, Tq", [(6, 8), (16, 1), (8, 16), (2, 8), (24, 3), (1, 2), (1, 8), (5, 3), (6, 1)])
def test_mfma_rows(kv, D, G, Tq):
    spec = scaled("verify_bf16", B=2, Tq=Tq, Hq=2 * G, Hkv=2, D=D, seq_lens=(Tq, 1300), shared_prefix=0,
                  cache_dtype=kv, src_dtype="bf16")
    w = generate(spec, seed=G * 100 + Tq)
    run_workload(w, partition_size=256)


# the largest group (64 query heads per kv head) and query tile (16 tokens)
# the library takes, alone and together (1024 rows per kv head), on every
# cache type, with ragged lengths and a row shorter than the query tile
@pytest.mark.parametrize("kv", ["f32", "bf16", "i8", "fp8", "nvfp4"])
@pytest.mark.parametrize("G, Tq, D", [(64, 1, 256), (1, 16, 256), (64, 16, 128), (64, 16, 64)])
def test_group_and_query_token_limits(kv, G, Tq, D):
    spec = scaled("verify_bf16", name="limits_%s_G%d_T%d" % (kv, G, Tq), B=2, Tq=Tq, Hq=G, Hkv=1, D=D,
                  seq_lens=(Tq, 400), shared_prefix=0, cache_dtype=kv, src_dtype="f32",
                  q_dtype="f32" if kv == "f32" else "bf16")
    w = generate(spec, seed=G + Tq + D, seq_lens=[Tq, 400])
    run_workload(w, partition_size=0)
    run_workload(w, partition_size=64, check_cache=False)


@pytest.mark.parametrize("qdt", ["f32", "bf16"])
@pytest.mark.parametrize("kv", ["bf16", "i8", "fp8", "nvfp4"])
def test_mfma_query_dtype_and_partitions(qdt, kv):
    spec = scaled("verify_bf16", B=3, Tq=8, Hq=12, Hkv=2, D=128, seq_lens=(8, 3000), shared_prefix=0,
                  cache_dtype=kv, q_dtype=qdt, src_dtype="f32")
    w = generate(spec, seed=11)
    for P in (16, 64, 1024, 0):
        run_workload(w, partition_size=P)


# ------------------------------------------------------------ graph capture
@pytest.mark.parametrize("name", ["gqa_bf16", "verify_i8"])
def test_step_captured_in_a_graph(name):
    """cache_write + decode + reduce recorded in one HIP graph: every replay
    (with other eager work and new query values in between) equals an eager
    run bit for bit. The library allocates and synchronises nothing, so the
    captured step is the whole step."""
    sp0 = SPECS[name]
    spec = scaled(name, seq_lens=(sp0.seq_lens[0] // 8, sp0.seq_lens[1] // 8),
                  shared_prefix=sp0.shared_prefix // 8 // 16 * 16)
    w = generate(spec, seed=12)
    cache = gpu_cache(w)
    k, v, ks, vs = cache
    q, table, lens = gpu_inputs(w)
    rows = w.step_rows()
    new_k = host_to_dev(w.k_src[rows], spec.src_dtype)
    new_v = host_to_dev(w.v_src[rows], spec.src_dtype)
    new_slots = torch.from_numpy(w.slot_mapping[rows]).to(dev())
    P = pa.choose_partition_size(spec.B, spec.Tq, spec.Hq, spec.Hkv, spec.D, k.dtype, w.max_seq_len)
    ws = torch.empty(max(256, pa.workspace_bytes(spec.B, spec.Tq, spec.Hq, spec.Hkv, spec.D, k.dtype,
                                                 w.max_seq_len, P)), dtype=torch.uint8, device=dev())
    out = torch.empty((spec.B, spec.Tq, spec.Hq, spec.D), dtype=torch.float32, device=dev())
    lse = torch.empty((spec.B, spec.Tq, spec.Hq), dtype=torch.float32, device=dev())

    def step():
        pa.cache_write(new_k, new_v, new_slots, k, v, ks, vs)
        pa.decode(q, k, v, table, lens, w.max_seq_len, w.softmax_scale, ks, vs, partition_size=P, out=out,
                  lse=lse, workspace=ws)

    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for i in range(4):
        q.copy_(q.roll(1, dims=2))  # new queries between replays (eager work)
        g.replay()
        torch.cuda.synchronize()
        got_o, got_l = out.clone(), lse.clone()
        step()  # eager
        torch.cuda.synchronize()
        assert torch.equal(got_o, out) and torch.equal(got_l, lse), "replay %d differs from eager" % i
