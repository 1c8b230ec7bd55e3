"""GPU parity of the sparse block-selection decode against the fp64 oracle.

Mean keys: GPU (fp32 sums in a fixed order) against the oracle's fp64 means,
for every cache type, full builds and the per-step refresh of the blocks
holding the newest tokens. Selection: where floating point decides which
blocks are taken, the GPU's choice is checked for validity against the
oracle's fp64 scores (right count, increasing, the blocks holding the query
tokens kept, and every selected candidate scoring at least the one left out,
within a bound of the fp32 score arithmetic); where the scores are separated
by far more than that bound, the choice must equal the oracle's. Attention:
the GPU output against the oracle's decode over the GPU's own selection,
within the usual tolerances (1e-2 bf16, 2e-2 quantised).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import paged_attention_decode_02_amd as pa
from _gpu import dev, dev_to_host, gpu_cache, gpu_inputs, host_to_dev
from _host import oracle_cache
from _refs import as_f64
from workloads import generate, scaled

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "i8": 2e-2, "fp8": 2e-2, "nvfp4": 2e-2}


def say(*a):
    print(*a, flush=True)


def gpu_mean_keys(w, cache, SB, num_new=None, fill=float("nan")):
    sp = w.spec
    k, v, ks, vs = cache
    q, table, lens = gpu_inputs(w)
    nsb = max(1, oracle.num_sparse_blocks(w.max_seq_len, SB))
    mk = torch.full((sp.B, nsb, sp.Hkv, sp.D), fill, dtype=torch.float32, device=dev())
    pa.sparse_mean_keys(k, table, lens, w.max_seq_len, SB, num_new or max(1, w.max_seq_len), mk, ks)
    torch.cuda.synchronize()
    return mk


def kept_range(L, Tq, SB):
    if L <= 0:
        return 0, 0
    return max(L - Tq, 0) // SB, oracle.num_sparse_blocks(L, SB)


def check_selection(w, sel, host, SB, top, exact=False):
    """Validity of the GPU's selection against the oracle's fp64 scores."""
    sp = w.spec
    k, v, ks, vs = host
    nsb = max(1, oracle.num_sparse_blocks(w.max_seq_len, SB))
    mk = oracle.sparse_mean_keys(k, w.block_table, w.seq_lens, SB, nsb, ks, sp.D)
    S = sel.shape[2]
    osel, ocnt, scores = oracle.sparse_select(w.q_array(), mk, w.seq_lens, w.softmax_scale, SB, top, S)
    q64 = as_f64(w.q_array())
    G = sp.Hq // sp.Hkv
    for b in range(sp.B):
        L = int(w.seq_lens[b])
        kept0, nsb_b = kept_range(L, sp.Tq, SB)
        for g in range(sp.Hkv):
            got = [int(j) for j in sel[b, g] if j >= 0]
            assert len(got) == int(ocnt[b, g]), (b, g, got, ocnt[b, g])
            assert all(x < y for x, y in zip(got, got[1:]))
            assert got[len(got) - (nsb_b - kept0):] == list(range(kept0, nsb_b))
            assert np.all(sel[b, g, len(got):] == -1)
            cand = got[:len(got) - (nsb_b - kept0)]
            if exact:
                assert got == [int(j) for j in osel[b, g, :ocnt[b, g]]], (b, g)
            if 0 < len(cand) < kept0:
                # bound of the fp32 arithmetic behind a GPU score
                qa = np.abs(q64[b, :, g * G:(g + 1) * G]).reshape(-1, sp.D)
                mag = float(np.max(qa @ np.abs(mk[b, :kept0, g]).T)) * w.softmax_scale
                eps = 1e-4 * mag + 1e-6
                s = scores[b, g, :kept0]
                taken = np.zeros(kept0, dtype=bool)
                taken[cand] = True
                assert s[taken].min() >= s[~taken].max() - eps, (b, g, s[taken].min(), s[~taken].max(), eps)


def run_sparse(w, SB, top, P=0, exact=False, check_cache=True):
    sp = w.spec
    say("sparse: %s B=%d Tq=%d Hq=%d Hkv=%d D=%d kv=%s max_len=%d SB=%d top=%d P=%d" % (
        sp.name, sp.B, sp.Tq, sp.Hq, sp.Hkv, sp.D, sp.cache_dtype, w.max_seq_len, SB, top, P))
    host = oracle_cache(w)
    cache = gpu_cache(w)
    k, v, ks, vs = cache
    q, table, lens = gpu_inputs(w)
    mk = gpu_mean_keys(w, cache, SB)
    S = pa.sparse_max_selected(w.max_seq_len, SB, top)
    sel = torch.full((sp.B, sp.Hkv, max(S, 1)), -7, dtype=torch.int32, device=dev())
    out, lse = pa.decode_sparse(q, k, v, table, lens, w.max_seq_len, w.softmax_scale, mk, SB, top, ks, vs,
                                partition_size=P, selected=sel if S > 0 else None)
    torch.cuda.synchronize()
    # the library writes S columns; with S = 0 (every length 0) it gets no buffer at all
    seln = sel.cpu().numpy()[:, :, :S]
    check_selection(w, seln, host, SB, top, exact)
    cnt = (seln >= 0).sum(axis=2).astype(np.int32)
    hk, hv, hks, hvs = host
    ref, rlse = oracle.decode_subset(w.q_array(), hk, hv, w.block_table, w.seq_lens, w.softmax_scale, seln, cnt, SB,
                                     hks, hvs)
    o = dev_to_host(out).astype(np.float64)
    l = dev_to_host(lse).astype(np.float64)
    err = float(np.max(np.abs(o - ref))) if o.size else 0.0
    fin = np.isfinite(rlse)
    lerr = float(np.max(np.abs(l[fin] - rlse[fin]))) if fin.any() else 0.0
    say("  max|out-oracle(selection)| = %.3e  max|lse| = %.3e  selected %d..%d blocks" % (err, lerr, cnt.min(),
                                                                                         cnt.max()))
    assert np.all(np.isfinite(o))
    assert np.array_equal(np.isneginf(l), np.isneginf(rlse))
    assert err <= TOL[sp.cache_dtype]
    assert lerr <= 1e-3
    return out, lse, seln, host


@pytest.mark.parametrize("kv", ["bf16", "i8", "fp8", "nvfp4"])
@pytest.mark.parametrize("SB", [16, 64])
def test_mean_keys_full_and_refresh(kv, SB):
    spec = scaled("gqa_bf16", B=4, Tq=1, Hq=4, Hkv=2, D=128, seq_lens=(0, 1000), cache_dtype=kv, src_dtype="f32")
    w = generate(spec, seed=100 + SB, seq_lens=[0, 5, 70, 1000])
    host = oracle_cache(w)
    cache = gpu_cache(w)
    k, v, ks, vs = host
    nsb = oracle.num_sparse_blocks(w.max_seq_len, SB)
    ref = oracle.sparse_mean_keys(k, w.block_table, w.seq_lens, SB, nsb, ks, w.spec.D)
    scale = float(np.nanmax(np.abs(as_f64(k, ks))))
    mk = gpu_mean_keys(w, cache, SB).cpu().numpy()
    err = np.nanmax(np.abs(mk - ref)) if np.isfinite(ref).any() else 0.0
    say("mean keys %s SB=%d: max err %.3e (scale %.3e)" % (kv, SB, err, scale))
    assert np.array_equal(np.isnan(mk), np.isnan(ref))  # exactly the blocks below each length are written
    assert err <= 2e-5 * scale
    # a decode step's refresh: only the blocks holding each sequence's last 3 tokens
    mk3 = gpu_mean_keys(w, cache, SB, num_new=3).cpu().numpy()
    for b, L in enumerate(w.seq_lens):
        L = int(L)
        fresh = set(range(max(L - 3, 0) // SB, oracle.num_sparse_blocks(L, SB))) if L > 0 else set()
        for j in range(nsb):
            if j in fresh:
                assert np.max(np.abs(mk3[b, j] - ref[b, j])) <= 2e-5 * scale
            else:
                assert np.all(np.isnan(mk3[b, j]))


@pytest.mark.parametrize("kv", ["bf16", "i8", "fp8", "nvfp4"])
@pytest.mark.parametrize("Tq", [1, 4])
@pytest.mark.parametrize("top", [1, 3, 9, 100])
def test_sparse_decode_against_oracle_on_its_selection(kv, Tq, top):
    spec = scaled("gqa_bf16", B=4, Tq=Tq, Hq=12, Hkv=2, D=128, seq_lens=(0, 1700), cache_dtype=kv, src_dtype="f32",
                  peaked_frac=0.01)
    w = generate(spec, seed=110 + Tq + top, seq_lens=[0, Tq, 700, 1700])
    run_sparse(w, 64, top)
    run_sparse(w, 64, top, P=64)


def test_separated_scores_select_exactly():
    # keys of sparse block j (per kv head) all equal a_j e_0, the a_j distinct
    # with gaps far above the fp32 score bound, queries e_0 (plus noise in
    # other dims): the GPU must pick exactly the oracle's blocks
    spec = scaled("gqa_bf16", B=2, Tq=2, Hq=4, Hkv=2, D=64, seq_lens=(1500, 2000), cache_dtype="bf16",
                  src_dtype="f32")
    w = generate(spec, seed=120)
    rng = np.random.default_rng(121)
    SB = 64
    w.k_src[:] = 0.0
    for b in range(2):
        rows = np.nonzero(w.row_seq == b)[0]
        nsb = oracle.num_sparse_blocks(int(w.seq_lens[b]), SB)
        a = rng.permutation(nsb).astype(np.float32) * 0.25 - nsb * 0.1
        for g in range(2):
            w.k_src[rows, g, 0] = a[(w.row_pos[rows] // SB)] * (1 if g == 0 else -1)
    w.q[:] = 0.0
    w.q[..., 0] = 1.0
    w.q_bits = None
    w.spec = scaled(w.spec, q_dtype="f32")
    for top in (2, 5, 13):
        run_sparse(w, SB, top, exact=True)


@pytest.mark.parametrize("kv", ["bf16", "i8"])
def test_all_blocks_selected_is_the_plain_decode(kv):
    spec = scaled("gqa_bf16", B=3, Tq=2, Hq=8, Hkv=2, D=128, seq_lens=(5, 900), cache_dtype=kv, src_dtype="f32")
    w = generate(spec, seed=130, seq_lens=[5, 333, 900])
    out, lse, sel, host = run_sparse(w, 32, 1000)
    hk, hv, hks, hvs = host
    ref, rlse = oracle.decode(w.q_array(), hk, hv, w.block_table, w.seq_lens, w.softmax_scale, hks, hvs)
    assert np.max(np.abs(out.cpu().numpy() - ref)) <= TOL[kv]


@pytest.mark.parametrize("name, SB, top", [("int8_250k", 64, 512), ("long64k_bf16", 64, 128)])
def test_full_size_sparse(name, SB, top):
    w = generate(name)
    run_sparse(w, SB, top)


@pytest.mark.parametrize("SB, lens, top", [(16, [65536, 40000], 300), (4096, [9000, 4097], 2)])
def test_sparse_size_limits(SB, lens, top):
    # 4096 sparse blocks of 16 tokens (the selection's largest candidate set),
    # and sparse blocks of 4096 tokens (the longest the mean-key kernel stages)
    spec = scaled("gqa_bf16", B=2, Tq=2, Hq=2, Hkv=1, D=64, seq_lens=(min(lens), max(lens)), cache_dtype="i8",
                  src_dtype="f32")
    w = generate(spec, seed=140 + SB, seq_lens=lens)
    assert oracle.num_sparse_blocks(w.max_seq_len, SB) <= 4096
    run_sparse(w, SB, top)


@pytest.mark.parametrize("kv", ["bf16", "i8"])
def test_sparse_step_in_a_graph(kv):
    # cache write, mean-key refresh and the sparse decode recorded in one HIP
    # graph; new queries between replays; every replay equals an eager step
    spec = scaled("gqa_bf16", B=3, Tq=2, Hq=12, Hkv=2, D=128, seq_lens=(200, 1500), cache_dtype=kv, src_dtype="f32")
    w = generate(spec, seed=150)
    k, v, ks, vs = gpu_cache(w)
    q, table, lens = gpu_inputs(w)
    rows = w.step_rows()
    new_k = host_to_dev(w.k_src[rows], spec.src_dtype)
    new_v = host_to_dev(w.v_src[rows], spec.src_dtype)
    new_slots = torch.from_numpy(np.ascontiguousarray(w.slot_mapping[rows])).to(dev())
    SB, top = 64, 6
    mk = gpu_mean_keys(w, (k, v, ks, vs), SB)
    S = pa.sparse_max_selected(w.max_seq_len, SB, top)
    ws = torch.empty(pa.sparse_workspace_bytes(spec.B, spec.Tq, spec.Hq, spec.Hkv, spec.D, k.dtype, w.max_seq_len,
                                               SB, top), dtype=torch.uint8, device=dev())
    out = torch.empty((spec.B, spec.Tq, spec.Hq, spec.D), dtype=torch.float32, device=dev())
    lse = torch.empty((spec.B, spec.Tq, spec.Hq), dtype=torch.float32, device=dev())
    sel = torch.empty((spec.B, spec.Hkv, S), dtype=torch.int32, device=dev())

    def step():
        pa.cache_write(new_k, new_v, new_slots, k, v, ks, vs)
        pa.sparse_mean_keys(k, table, lens, w.max_seq_len, SB, spec.Tq, mk, ks)
        pa.decode_sparse(q, k, v, table, lens, w.max_seq_len, w.softmax_scale, mk, SB, top, ks, vs, out=out, lse=lse,
                         selected=sel, workspace=ws)

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
        got = (out.clone(), lse.clone(), sel.clone())
        step()  # eager
        torch.cuda.synchronize()
        assert torch.equal(got[0], out) and torch.equal(got[1], lse) and torch.equal(got[2], sel), i
