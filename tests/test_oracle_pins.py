"""Pins of the fp64 oracle against facts fixed outside it (CPU only).

Each test checks the oracle against something it does not share code with:
Decimal brute force, closed forms, dense attention via numpy, torch SDPA,
invariances (block permutation, GQA as repeated MHA, causal rows as a virtual
batch, split = unsplit, shared prefix = private copies, linearity, poison),
hand-derived int8, FP8 (OCP E4M3) and NVFP4 quantiser cases, and torch's
float8_e4m3fn conversions. A dropped term, wrong sign or index, or a
transposed operand in the oracle fails at least one of them.
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from _host import oracle_cache, oracle_decode, poison_host
from _refs import as_f64, brute_decode, dense_decode, nvfp4_split, sdpa_decode
from workloads import BLOCK_SIZE, SPECS, bf16_bits, bf16_bits_to_f32, generate, scaled

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def small(name="gqa_bf16", **kw):
    base = dict(B=2, Tq=1, Hq=4, Hkv=2, D=16, seq_lens=(20, 60))
    base.update(kw)
    return scaled(name, **base)


# ---------------------------------------------------------------- brute force
def test_brute_force_tiny_workload():
    """The tiny fp32 workload at full size against 50-digit Decimal arithmetic."""
    w = generate("tiny_f32")
    cache = oracle_cache(w)
    out, lse = oracle_decode(w, cache)
    bo, bl = brute_decode(w.q_array(), cache[0], cache[1], w.block_table, w.seq_lens, w.softmax_scale)
    assert np.max(np.abs(out - bo)) <= 1e-12
    assert np.max(np.abs(lse - bl)) <= 1e-12


@pytest.mark.parametrize("case", range(6))
def test_brute_force_random_tiny(case):
    rng = np.random.default_rng(100 + case)
    dtype = ["f32", "bf16", "i8"][case % 3]
    Hkv = [1, 2][case % 2]
    G = [1, 3, 2][case % 3]
    Tq = 1 + case % 3
    spec = scaled("gqa_bf16", B=2, Tq=Tq, Hq=Hkv * G, Hkv=Hkv, D=[4, 8][case % 2],
                  seq_lens=(Tq, 40), q_dtype="bf16" if case % 2 else "f32",
                  src_dtype="f32", cache_dtype=dtype)
    lens = rng.integers(Tq, 41, size=2)
    w = generate(spec, seed=case, seq_lens=lens)
    cache = oracle_cache(w)
    out, lse = oracle_decode(w, cache)
    bo, bl = brute_decode(w.q_array(), cache[0], cache[1], w.block_table, w.seq_lens, w.softmax_scale,
                          cache[2], cache[3])
    assert np.max(np.abs(out - bo)) <= 1e-12
    assert np.max(np.abs(lse - bl)) <= 1e-12


# ---------------------------------------------------------------- closed forms
def test_single_key_returns_its_value_row():
    w = generate(small(seq_lens=(1, 1), B=3), seed=1)
    cache = oracle_cache(w)
    out, lse = oracle_decode(w, cache)
    V = as_f64(cache[1])
    K = as_f64(cache[0])
    G = w.spec.G
    for b in range(w.spec.B):
        blk = w.block_table[b, 0]
        for h in range(w.spec.Hq):
            assert np.array_equal(out[b, 0, h], V[blk, 0, h // G])
            s = float(np.float32(w.softmax_scale)) * float(np.dot(w.q[b, 0, h].astype(np.float64), K[blk, 0, h // G]))
            assert abs(lse[b, 0, h] - s) <= 1e-12 * max(1.0, abs(s))


def test_constant_values_return_the_constant():
    w = generate(small(src_dtype="f32", cache_dtype="f32", q_dtype="f32"), seed=2)
    c = np.linspace(-3, 3, w.spec.Hkv * w.spec.D, dtype=np.float32).reshape(w.spec.Hkv, w.spec.D)
    w.v_src[:] = c[None]
    cache = oracle_cache(w)
    out, _ = oracle_decode(w, cache)
    G = w.spec.G
    for h in range(w.spec.Hq):
        assert np.max(np.abs(out[:, :, h] - c[h // G].astype(np.float64))) <= 1e-12


@pytest.mark.parametrize("how", ["zero_query", "zero_scale"])
def test_uniform_weights_give_the_mean(how):
    w = generate(small(Tq=2, src_dtype="f32", cache_dtype="f32", q_dtype="f32"), seed=3)
    if how == "zero_query":
        w.q[:] = 0.0
    else:
        w.softmax_scale = 0.0
    cache = oracle_cache(w)
    out, lse = oracle_decode(w, cache)
    V = as_f64(cache[1])
    G = w.spec.G
    for b in range(w.spec.B):
        L = int(w.seq_lens[b])
        for t in range(w.spec.Tq):
            n = L - w.spec.Tq + t + 1
            rows = [V[w.block_table[b, j // 16], j % 16] for j in range(n)]
            mean = np.mean(np.stack(rows), axis=0)
            for h in range(w.spec.Hq):
                assert np.max(np.abs(out[b, t, h] - mean[h // G])) <= 1e-12
                assert abs(lse[b, t, h] - np.log(n)) <= 1e-12


# ------------------------------------------------------------ library / dense
@pytest.mark.parametrize("dtype", ["f32", "bf16", "i8", "fp8", "nvfp4"])
def test_paged_equals_dense_contiguous(dtype):
    spec = scaled("gqa_bf16", B=3, Tq=2, Hq=8, Hkv=2, D=64 if dtype == "nvfp4" else 32, seq_lens=(2, 200),
                  src_dtype="f32", cache_dtype=dtype, q_dtype="bf16")
    w = generate(spec, seed=4)
    cache = oracle_cache(w)
    out, lse = oracle_decode(w, cache)
    do, dl = dense_decode(w.q_array(), cache[0], cache[1], w.block_table, w.seq_lens, w.softmax_scale,
                          cache[2], cache[3])
    assert np.max(np.abs(out - do)) <= 1e-13
    assert np.max(np.abs(lse - dl)) <= 1e-12


def test_matches_torch_sdpa_fp64_causal():
    spec = scaled("verify_bf16", B=2, Tq=3, Hq=6, Hkv=2, D=16, seq_lens=(3, 90), shared_prefix=0)
    w = generate(spec, seed=5)
    cache = oracle_cache(w)
    out, _ = oracle_decode(w, cache)
    ref = sdpa_decode(w.q_array(), cache[0], cache[1], w.block_table, w.seq_lens, w.softmax_scale)
    assert np.max(np.abs(out - ref)) <= 1e-12


# ------------------------------------------------------------------ invariants
def test_block_permutation_is_bitwise_invariant():
    w = generate(small(B=3, seq_lens=(30, 100)), seed=6)
    k, v, ks, vs = oracle_cache(w)
    out, lse = oracle_decode(w, (k, v, ks, vs))
    perm = np.random.default_rng(7).permutation(w.num_blocks)  # new id of old block i is perm[i]
    k2, v2 = np.empty_like(k), np.empty_like(v)
    k2[perm], v2[perm] = k, v
    w.block_table = perm[w.block_table].astype(np.int32)
    out2, lse2 = oracle_decode(w, (k2, v2, None, None))
    assert np.array_equal(out, out2, equal_nan=True) and np.array_equal(lse, lse2)


def test_gqa_equals_repeated_kv_mha():
    spec = small(Hq=6, Hkv=2, Tq=2, D=8, cache_dtype="i8", src_dtype="f32")
    w = generate(spec, seed=8)
    k, v, ks, vs = oracle_cache(w)
    out, lse = oracle_decode(w, (k, v, ks, vs))
    G = spec.G
    rep = lambda a, axis=2: np.ascontiguousarray(np.repeat(a, G, axis=axis))
    # scales [num_blocks, Hkv, 16]: kv heads on axis 1
    out2, lse2 = oracle.decode(w.q_array(), rep(k), rep(v), w.block_table, w.seq_lens, w.softmax_scale,
                               rep(ks, 1), rep(vs, 1))
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_causal_rows_are_a_virtual_batch():
    spec = scaled("verify_bf16", B=2, Tq=8, Hq=4, Hkv=2, D=16, seq_lens=(8, 70), shared_prefix=0)
    w = generate(spec, seed=9)
    cache = oracle_cache(w)
    out, lse = oracle_decode(w, cache)
    for t in range(8):
        lens_t = (w.seq_lens - 8 + t + 1).astype(np.int32)
        o1, l1 = oracle.decode(w.q_array()[:, t:t + 1], cache[0], cache[1], w.block_table, lens_t,
                               w.softmax_scale)
        assert np.array_equal(out[:, t], o1[:, 0]) and np.array_equal(lse[:, t], l1[:, 0])


@pytest.mark.parametrize("P", [16, 64, 512, 2048, 4096])
def test_split_equals_unsplit(P):
    spec = scaled("long64k_bf16", B=2, Tq=2, Hq=6, Hkv=2, D=32, seq_lens=(900, 3000), peaked_frac=0.01,
                  cache_dtype="bf16")
    w = generate(spec, seed=10)
    cache = oracle_cache(w)
    out, lse = oracle_decode(w, cache)
    o2, l2 = oracle_decode(w, cache, partition_size=P)
    assert np.max(np.abs(out - o2)) <= 1e-13
    assert np.max(np.abs(lse - l2)) <= 1e-12


def test_shared_prefix_equals_private_copies():
    spec = scaled("verify_i8", B=3, Tq=8, Hq=6, Hkv=2, D=16, seq_lens=(80, 200), shared_prefix=64)
    w = generate(spec, seed=11)
    k, v, ks, vs = oracle_cache(w)
    out, lse = oracle_decode(w, (k, v, ks, vs))
    # give every sequence private copies of the prefix blocks
    nshared = 64 // BLOCK_SIZE
    extra = w.spec.B * nshared
    grow = lambda a: np.concatenate([a, np.zeros((extra,) + a.shape[1:], a.dtype)])
    k2, v2, ks2, vs2 = grow(k), grow(v), grow(ks), grow(vs)
    table = w.block_table.copy()
    nxt = w.num_blocks
    for b in range(w.spec.B):
        for j in range(nshared):
            src = table[b, j]
            for a2, a in ((k2, k), (v2, v), (ks2, ks), (vs2, vs)):
                a2[nxt] = a[src]
            table[b, j] = nxt
            nxt += 1
    out2, lse2 = oracle.decode(w.q_array(), k2, v2, table, w.seq_lens, w.softmax_scale, ks2, vs2)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_linear_in_values():
    spec = small(src_dtype="f32", cache_dtype="f32", q_dtype="f32", Tq=2)
    w = generate(spec, seed=12)
    rng = np.random.default_rng(13)
    V1 = (rng.integers(-64, 64, size=w.v_src.shape) / 16).astype(np.float32)
    V2 = (rng.integers(-64, 64, size=w.v_src.shape) / 16).astype(np.float32)
    outs = []
    for V in (V1, V2, 2 * V1 + 0.5 * V2):  # exact in fp32
        w.v_src = V
        outs.append(oracle_decode(w, oracle_cache(w))[0])
    assert np.max(np.abs(outs[2] - (2 * outs[0] + 0.5 * outs[1]))) <= 1e-12


@pytest.mark.parametrize("dtype", ["f32", "bf16", "i8", "fp8", "nvfp4"])
def test_poisoned_slots_are_never_read(dtype):
    spec = small(B=3, Tq=2, seq_lens=(5, 77), cache_dtype=dtype, src_dtype="f32", D=64 if dtype == "nvfp4" else 16)
    w = generate(spec, seed=14)
    clean = oracle_decode(w, oracle_cache(w, poison=False))
    dirty = oracle_decode(w, oracle_cache(w, poison=True))
    assert np.all(np.isfinite(dirty[0]))
    assert np.array_equal(clean[0], dirty[0]) and np.array_equal(clean[1], dirty[1])


def test_rows_without_keys_are_zero_with_minus_inf_lse():
    spec = small(B=3, Tq=4, seq_lens=(0, 6))
    w = generate(spec, seed=15, seq_lens=[0, 2, 6])
    out, lse = oracle_decode(w, oracle_cache(w))
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    # sequence 1 has 2 tokens and 4 query tokens: rows t = 0, 1 see n <= 0 keys
    assert np.all(out[1, :2] == 0) and np.all(np.isneginf(lse[1, :2]))
    assert np.all(np.isfinite(lse[1, 2:])) and np.all(np.isfinite(lse[2]))


# ----------------------------------------------------------------- cache writer
def _write_rows(x: np.ndarray, cache_dtype: str, src_dtype: str = "f32"):
    """Quantise/copy rows x [N, 1, D] into a 1-kv-head cache; return cache and scales."""
    N, _, D = x.shape
    nb = (N + BLOCK_SIZE - 1) // BLOCK_SIZE
    k, v, ks, vs = oracle.alloc_cache(nb, BLOCK_SIZE, 1, D, cache_dtype)
    src = x if src_dtype == "f32" else bf16_bits(x).reshape(x.shape)
    oracle.cache_write(src, src, np.arange(N), k, v, ks, vs)
    k = k.reshape(nb * BLOCK_SIZE, D)[:N]
    if ks is not None:
        ks = ks.reshape(-1)[:N]
    return k, ks


def test_int8_golden_cases():
    with open(os.path.join(GOLDEN, "int8_quantizer_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        x = np.asarray(c["x"], np.float32)[None, None, :]
        codes, scale = _write_rows(x, "i8")
        assert scale[0] == np.float32(c["scale"]), c["why"]
        assert codes[0].tolist() == c["codes"], c["why"]


def test_int8_round_trip_and_error_bound():
    rng = np.random.default_rng(16)
    x = rng.standard_normal((4096, 1, 256), dtype=np.float32)
    x[:64] *= np.float32(1e-30)  # tiny magnitudes
    x[64:128] *= np.float32(1e30)  # huge magnitudes
    codes, s = _write_rows(x, "i8")
    assert codes.min() >= -127 and codes.max() <= 127
    # error bound: |x - code*s| <= s * (1/2 + 2^-18)
    err = np.abs(x[:, 0].astype(np.float64) - codes.astype(np.float64) * s[:, None].astype(np.float64))
    assert np.all(err <= s[:, None].astype(np.float64) * (0.5 + 2.0 ** -18))
    # each row uses the full code range
    assert np.all(np.abs(codes).max(axis=1) == 127)
    # dequantise (fp32 product, and exactly) and quantise again: identical codes and scale
    for deq in (codes.astype(np.float32) * s[:, None], (codes.astype(np.float64) * s[:, None]).astype(np.float32)):
        c2, s2 = _write_rows(deq[:, None, :].astype(np.float32), "i8")
        assert np.array_equal(c2, codes) and np.array_equal(s2, s)


def test_int8_quotient_is_rounded_to_fp32_first():
    """Where the exact quotient x/s lies just off a half-integer but its fp32
    rounding lands on it, the code follows the fp32 quotient (ties to even)."""
    rng = np.random.default_rng(17)
    found = 0
    for _ in range(200000):
        s = np.float32(rng.uniform(0.01, 0.05))
        k = int(rng.integers(-120, 120))
        # the fp32 neighbour of (k + 0.5) * s whose exact quotient is not k + 0.5
        base = np.float32((k + 0.5) * float(s))
        for x in (base, np.nextafter(base, np.float32(np.inf)), np.nextafter(base, np.float32(-np.inf))):
            qf = np.float32(x) / s  # binary32 quotient
            exact = Fraction(float(x)) / Fraction(float(s))
            if float(qf) == k + 0.5 and exact != Fraction(2 * k + 1, 2):
                amax = np.float32(127) * s  # forces the row scale close to s
                row = np.array([x, amax], np.float32)
                if np.float32(row.__abs__().max() / np.float32(127)) != s:
                    continue
                codes, scale = _write_rows(row[None, None, :], "i8")
                assert scale[0] == s
                half_even = k if k % 2 == 0 else k + 1
                assert codes[0, 0] == half_even
                found += 1
        if found >= 5:
            break
    assert found >= 1


# --------------------------------------------------------------- FP8 (E4M3)
def _e4m3_torch_values() -> np.ndarray:
    import torch

    return torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_fp8_golden_values():
    with open(os.path.join(GOLDEN, "fp8_e4m3_cases.json")) as f:
        cases = json.load(f)["values"]
    for c in cases:
        got = oracle.fp8_value(c["code"])
        if c["value"] == "nan":
            assert np.isnan(got), c["why"]
        else:
            want = float(c["value"])
            assert got == want and np.signbit(got) == np.signbit(want), c["why"]


def test_fp8_values_match_torch_e4m3fn():
    ref = _e4m3_torch_values()
    for code in range(256):
        got = oracle.fp8_value(code)
        if np.isnan(ref[code]):
            assert np.isnan(got), code
        else:
            assert got == ref[code] and np.signbit(got) == np.signbit(ref[code]), code


def test_fp8_encoder_matches_torch_saturated_cast():
    """Nearest-even rounding: every finite value, every midpoint and its fp32
    neighbours, random and subnormal-range values, and values past 448 (which
    saturate; torch's cast is applied to the clamped value)."""
    import torch

    vals = _e4m3_torch_values()
    fin = np.unique(vals[np.isfinite(vals)])
    mids = ((fin[:-1] + fin[1:]) / 2).astype(np.float32)
    rng = np.random.default_rng(40)
    y = np.concatenate([
        fin.astype(np.float32), mids, np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(-np.inf)),
        (rng.standard_normal(3000) * 60).astype(np.float32), (rng.random(1000) * 2.0 ** -5).astype(np.float32),
        np.array([448.5, 463.9, 464.0, 465.0, 1e6, -450.0, -1e30, 3.4e38], np.float32)]).astype(np.float32)
    want = torch.from_numpy(np.clip(y, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.fp8_encode(float(v)) for v in y], np.uint8)
    bad = np.nonzero(got != want)[0]
    assert len(bad) == 0, [(float(y[i]), int(got[i]), int(want[i])) for i in bad[:5]]


def test_fp8_round_trip_of_every_finite_code():
    for code in range(256):
        v = oracle.fp8_value(code)
        if not np.isnan(v):
            assert oracle.fp8_encode(np.float32(v)) == code, code


def test_fp8_golden_rows():
    with open(os.path.join(GOLDEN, "fp8_e4m3_cases.json")) as f:
        cases = json.load(f)["rows"]
    for c in cases:
        x = np.asarray(c["x"], np.float32)[None, None, :]
        codes, scale = _write_rows(x, "fp8")
        assert scale[0] == np.float32(c["scale"]), c["why"]
        assert codes[0].tolist() == c["codes"], c["why"]


def test_fp8_quotient_is_rounded_to_fp32_first():
    """Where the exact quotient x/s lies just off the midpoint of two E4M3
    values but its fp32 rounding lands on it, the code is the even neighbour
    (the fp32 quotient, ties to even), not the side the exact quotient is on."""
    vals = _e4m3_torch_values()
    mags = [(c, vals[c]) for c in range(1, 127)]  # ascending finite magnitudes
    rng = np.random.default_rng(42)
    found = 0
    for _ in range(200000):
        s = np.float32(rng.uniform(0.001, 0.05))
        i = int(rng.integers(0, len(mags) - 1))
        (c0, v0), (c1, v1) = mags[i], mags[i + 1]
        m = (v0 + v1) / 2  # exact in binary
        base = np.float32(m * float(s))
        for x in (base, np.nextafter(base, np.float32(np.inf)), np.nextafter(base, np.float32(-np.inf))):
            if float(np.float32(x) / s) != m:
                continue
            exact = Fraction(float(x)) / Fraction(float(s))
            if exact == Fraction(m):
                continue
            even = c0 if c0 % 2 == 0 else c1
            exact_side = c0 if exact < Fraction(m) else c1
            if exact_side == even:
                continue  # both readings agree here
            amax = np.float32(448.0 * float(s))
            if np.float32(amax / np.float32(448)) != s or amax < abs(x):
                continue
            codes, scale = _write_rows(np.array([[[x, amax]]], np.float32), "fp8")
            assert scale[0] == s
            assert codes[0, 0] == even
            found += 1
        if found >= 5:
            break
    assert found >= 1


def test_fp8_quantiser_bound_and_range():
    rng = np.random.default_rng(41)
    x = rng.standard_normal((2048, 1, 256), dtype=np.float32)
    x[:32] *= np.float32(1e-30)
    x[32:64] *= np.float32(1e30)
    codes, s = _write_rows(x, "fp8")
    vals = _e4m3_torch_values()[codes]
    assert np.all(np.isfinite(vals))  # never a NaN code
    # the largest magnitude of every row maps to +-448
    assert np.all(np.abs(vals).max(axis=1) == 448.0)
    # |x/s - value| <= half a step of the E4M3 grid at |x/s| (+ the fp32 quotient's rounding)
    y = x[:, 0].astype(np.float64) / s[:, None].astype(np.float64)
    e = np.maximum(np.floor(np.log2(np.maximum(np.abs(y), 2.0 ** -30))), -6)
    half_step = 2.0 ** (e - 4)
    assert np.all(np.abs(y - vals) <= half_step + np.abs(y) * 2.0 ** -23)


# ------------------------------------------------------------------- NVFP4
def _nvfp4_golden():
    with open(os.path.join(GOLDEN, "nvfp4_cases.json")) as f:
        return json.load(f)


def test_e2m1_golden_values_and_closed_form():
    g = _nvfp4_golden()
    for c in g["e2m1_values"]:
        got = oracle.e2m1_value(c["code"])
        assert got == c["value"] and np.signbit(got) == np.signbit(c["value"]), c
    # closed form: (-1)^s * (e == 0 ? m / 2 : (1 + m / 2) * 2^(e - 1)) for code = s e e m
    for code in range(16):
        s_, e, m = code >> 3, (code >> 1) & 3, code & 1
        want = (m / 2 if e == 0 else (1 + m / 2) * 2.0 ** (e - 1)) * (-1) ** s_
        assert oracle.e2m1_value(code) == want


def test_e2m1_rounding_golden_and_round_trip():
    for c in _nvfp4_golden()["e2m1_rounding"]:
        assert oracle.e2m1_encode(c["y"]) == c["code"], c["why"]
    for code in range(16):
        assert oracle.e2m1_encode(oracle.e2m1_value(code)) == code, code
    # monotone in |y|, saturating, and never further from y than half a step
    ys = np.linspace(0, 8, 4001, dtype=np.float32)
    codes = [oracle.e2m1_encode(float(y)) for y in ys]
    vals = np.array([oracle.e2m1_value(c) for c in codes])
    assert np.all(np.diff(vals) >= 0) and vals.max() == 6.0
    steps = np.array([0.5, 0.5, 0.5, 0.5, 1.0, 1.0, 2.0])  # gaps between consecutive magnitudes
    edges = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6.0])
    inside = ys <= 6
    gap = steps[np.clip(np.searchsorted(edges, ys[inside], side="right") - 1, 0, 6)]
    assert np.all(np.abs(vals[inside] - ys[inside]) <= gap / 2)


def test_nvfp4_golden_row():
    row = _nvfp4_golden()["row"]
    D = 128
    x = np.zeros(D, np.float32)
    for b, blk in enumerate(row["blocks"]):
        x[16 * b: 16 * b + len(blk["x"])] = blk["x"]
    nb = 1
    k, v, ks, vs = oracle.alloc_cache(nb, BLOCK_SIZE, 1, D, "nvfp4")
    k[:] = 0xEE  # bytes of other rows: left as they are
    oracle.cache_write(x[None, None, :], x[None, None, :], np.array([5]), k, v, ks, vs)
    assert ks[0, 0, 5] == np.float32(row["row_scale"])
    all_codes, all_scales = nvfp4_split(k, D)
    codes, scales = all_codes[0, 5, 0], all_scales[0, 5, 0]
    for b, blk in enumerate(row["blocks"]):
        assert scales[b] == blk["scale_code"], (b, scales[b])
        n = len(blk["codes"])
        assert codes[16 * b: 16 * b + n].tolist() == blk["codes"], (b, blk)
        assert np.all(codes[16 * b + n: 16 * b + 16] == 0)
    # token 5 of the block owns D/2 code bytes and D/16 scale bytes, nothing else
    untouched = np.ones(k.size, bool)
    untouched[5 * D // 2: 6 * D // 2] = False
    for kk in range(D // 16):
        untouched[16 * D // 2 + 16 * kk + 4 * (5 % 4) + 5 // 4] = False
    assert np.all(k.reshape(-1)[untouched] == 0xEE)


def test_nvfp4_quantiser_bound():
    rng = np.random.default_rng(43)
    D = 256
    x = rng.standard_normal((512, 1, D), dtype=np.float32)
    x[:16] *= np.float32(1e-20)
    x[16:32, :, :128] *= np.float32(1e4)  # blocks of very different magnitudes in one row
    nb = 512 // BLOCK_SIZE
    k, v, ks, vs = oracle.alloc_cache(nb, BLOCK_SIZE, 1, D, "nvfp4")
    oracle.cache_write(x, x, np.arange(512), k, v, ks, vs)
    all_codes, all_scales = nvfp4_split(k, D)
    codes, scale_codes = all_codes.reshape(512, D), all_scales.reshape(512, D // 16)
    S = ks.reshape(512).astype(np.float64)
    e2 = np.array([oracle.e2m1_value(c) for c in range(16)])
    sb = np.array([oracle.fp8_value(c) for c in range(256)])[scale_codes]
    db = (np.repeat(sb, 16, axis=1) * S[:, None]).astype(np.float32).astype(np.float64)
    y = x[:, 0].astype(np.float64) / np.where(db == 0, 1, db)
    got = e2[codes]
    # |y - value| <= half the E2M1 step at |y| (1/4 below 2, 1/2 below 4, 1 above),
    # or the excess past 6 where a block scale rounded down
    half = np.where(np.abs(y) < 2, 0.25, np.where(np.abs(y) < 4, 0.5, 1.0))
    err = np.abs(y - got)
    ok = (err <= half + np.abs(y) * 2.0 ** -22) | ((np.abs(y) > 6) & (np.abs(got) == 6))
    assert np.all(ok | (db == 0))
    # every row's largest magnitude lands on +-6 in a block scaled by 448 S
    for i in range(512):
        j = int(np.argmax(np.abs(x[i, 0])))
        assert abs(got[i, j]) == 6.0 and sb[i, j // 16] == 448.0


def test_bf16_and_f32_copies():
    rng = np.random.default_rng(18)
    x = rng.standard_normal((40, 1, 64), dtype=np.float32) * np.float32(3.7)
    import torch

    # f32 -> bf16 rounds to nearest even like torch's conversion
    got, _ = _write_rows(x, "bf16")
    want = torch.from_numpy(x[:, 0]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)
    # f32 -> f32 and bf16 -> bf16 copy bits; bf16 -> f32 widens exactly
    got, _ = _write_rows(x, "f32")
    assert np.array_equal(got.view(np.uint32), x[:, 0].view(np.uint32))
    got, _ = _write_rows(x, "bf16", src_dtype="bf16")
    assert np.array_equal(got, bf16_bits(x[:, 0]))
    got, _ = _write_rows(x, "f32", src_dtype="bf16")
    assert np.array_equal(got, bf16_bits_to_f32(bf16_bits(x[:, 0])).reshape(40, 64))


def test_slot_placement_and_skipped_slots():
    rng = np.random.default_rng(19)
    nb, Hkv, D = 6, 2, 8
    N = 20
    x = rng.standard_normal((N, Hkv, D), dtype=np.float32)
    slots = rng.permutation(nb * BLOCK_SIZE)[:N].astype(np.int64)
    slots[[3, 11]] = -1
    k, v, _, _ = oracle.alloc_cache(nb, BLOCK_SIZE, Hkv, D, "f32")
    k[:] = 7.0
    oracle.cache_write(x, -x, slots, k, v)
    flat = k.reshape(nb * BLOCK_SIZE, Hkv, D)
    for i in range(N):
        if slots[i] >= 0:
            assert np.array_equal(flat[slots[i]], x[i])
            assert np.array_equal(v.reshape(-1, Hkv, D)[slots[i]], -x[i])
    untouched = np.setdiff1d(np.arange(nb * BLOCK_SIZE), slots[slots >= 0])
    assert np.all(flat[untouched] == 7.0)


def test_oracle_rejects_bad_arguments():
    w = generate(small(), seed=20)
    k, v, ks, vs = oracle_cache(w)
    with pytest.raises(ValueError):
        oracle.decode(w.q_array(), *oracle.alloc_cache(4, 16, 2, 16, "i8")[:2], w.block_table, w.seq_lens, 0.25)
