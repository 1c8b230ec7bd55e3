"""Pins of the oracle's sparse block-selection decode (CPU only).

The reading (the vllm-sm70 page names per-block sparse-decode mean keys and a
selection over at most 4096 key blocks, not the rule): sparse blocks of SB
tokens; mean key = the plain mean of a block's keys; the blocks holding the
query tokens are always kept; the others score max over the kv head's query
rows of scale * q . mean key; the top ones (ties to the lower index) fill
top_blocks; rows attend to the selected blocks' keys with the plain causal
rule. Each oracle function is pinned here against something other than itself:
numpy means over independently decoded caches, a brute-force sort, the plain
decode (all blocks selected), the plain decode on a compacted block table,
Decimal brute force, and closed forms.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from _host import oracle_cache
from _refs import as_f64, brute_decode, gather
from workloads import BLOCK_SIZE, generate, scaled


def small(kv="bf16", B=3, Tq=1, Hq=6, Hkv=2, D=64, lens=(0, 1, 100, 300), seed=0, src="f32"):
    spec = scaled("gqa_bf16", B=len(lens), Tq=Tq, Hq=Hq, Hkv=Hkv, D=D, seq_lens=(min(lens), max(lens)),
                  cache_dtype=kv, src_dtype=src, q_dtype="bf16")
    return generate(spec, seed=seed, seq_lens=list(lens))


@pytest.mark.parametrize("kv", ["f32", "bf16", "i8", "fp8", "nvfp4"])
@pytest.mark.parametrize("SB", [16, 64])
def test_mean_keys_equal_numpy_means(kv, SB):
    w = small(kv, lens=(0, 1, 17, 100, 300), seed=1)
    k, v, ks, vs = oracle_cache(w)
    nsb = oracle.num_sparse_blocks(300, SB)
    mk = oracle.sparse_mean_keys(k, w.block_table, w.seq_lens, SB, nsb + 2, ks, w.spec.D)
    K = as_f64(k, ks)
    for b, L in enumerate(w.seq_lens):
        L = int(L)
        Kb = gather(K, w.block_table[b], L)  # [L, Hkv, D]
        for j in range(oracle.num_sparse_blocks(L, SB)):
            ref = Kb[j * SB:min(L, (j + 1) * SB)].mean(axis=0)
            assert np.max(np.abs(mk[b, j] - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))
        # entries past the sequence's blocks are left untouched (NaN)
        assert np.all(np.isnan(mk[b, oracle.num_sparse_blocks(L, SB):]))


def brute_select(q64, mk, lens, scale, SB, top, Tq, Hkv):
    """Selection by sorting (score descending, index ascending) in plain Python."""
    B, _, Hq, D = q64.shape
    G = Hq // Hkv
    res = {}
    for b in range(B):
        L = int(lens[b])
        nsb = (L + SB - 1) // SB
        kept0 = max(L - Tq, 0) // SB if L > 0 else 0
        for g in range(Hkv):
            cands = []
            for j in range(kept0):
                s = max(float(np.float32(scale)) * float(np.dot(q64[b, t, g * G + h], mk[b, j, g]))
                        for t in range(Tq) for h in range(G))
                cands.append((-s, j))
            cands.sort()
            want = min(max(top - (nsb - kept0), 0), kept0)
            res[b, g] = sorted([j for _, j in cands[:want]] + list(range(kept0, nsb)))
    return res


@pytest.mark.parametrize("Tq", [1, 3, 8])
@pytest.mark.parametrize("top", [1, 2, 3, 5, 40])
def test_selection_equals_brute_force_sort(Tq, top):
    rng = np.random.default_rng(100 + Tq * 7 + top)
    B, Hq, Hkv, D, SB = 5, 6, 2, 16, 16
    lens = np.array([0, 5, 16, 77, 250], dtype=np.int32)
    q = rng.standard_normal((B, Tq, Hq, D)).astype(np.float32)
    mks = 20
    mk = rng.standard_normal((B, mks, Hkv, D))
    # exact ties: block 4 repeats block 1, block 9 repeats block 3
    mk[:, 4] = mk[:, 1]
    mk[:, 9] = mk[:, 3]
    scale = 0.25
    max_sel = max(top, 2)
    sel, cnt, scores = oracle.sparse_select(q, mk, lens, scale, SB, top, max_sel)
    ref = brute_select(q.astype(np.float64), mk, lens, scale, SB, top, Tq, Hkv)
    for (b, g), blocks in ref.items():
        assert cnt[b, g] == len(blocks)
        assert list(sel[b, g, :cnt[b, g]]) == blocks, (b, g, sel[b, g], blocks)
        assert np.all(sel[b, g, cnt[b, g]:] == -1)
    # candidate scores are the max over the group's rows (numpy einsum)
    G = Hq // Hkv
    for b in range(B):
        kept0 = max(int(lens[b]) - Tq, 0) // SB if lens[b] > 0 else 0
        for g in range(Hkv):
            if kept0:
                s = np.einsum("thd,jd->jth", q[b, :, g * G:(g + 1) * G].astype(np.float64), mk[b, :kept0, g])
                np.testing.assert_allclose(scores[b, g, :kept0], 0.25 * s.reshape(kept0, -1).max(axis=1),
                                           rtol=1e-13)
            assert np.all(np.isnan(scores[b, g, kept0:]))


def test_tied_blocks_go_to_the_lower_index():
    B, Tq, Hq, Hkv, D, SB = 1, 1, 1, 1, 4, 16
    q = np.array([[[[1, 0, 0, 0]]]], dtype=np.float32)
    mk = np.zeros((1, 6, 1, D))
    mk[0, :, 0, 0] = [0.5, 2.0, 1.0, 2.0, 2.0, 0.0]  # blocks 1, 3 and 4 tie; block 5 holds the query
    lens = np.array([90], dtype=np.int32)
    sel, cnt, _ = oracle.sparse_select(q, mk, lens, 1.0, SB, 3, 3)
    assert list(sel[0, 0]) == [1, 3, 5]


def kept_blocks(L, Tq, SB):
    return list(range(max(L - Tq, 0) // SB, (L + SB - 1) // SB))


@pytest.mark.parametrize("L, Tq, expect", [(64 * 3 + 3, 8, [2, 3]), (64 * 3 + 20, 8, [3]), (64, 8, [0]),
                                            (65, 1, [1]), (5, 8, [0])])
def test_blocks_holding_the_query_tokens_are_always_selected(L, Tq, expect):
    # the query tokens' blocks score -inf-like against q but are kept anyway
    SB, D = 64, 8
    q = np.zeros((1, Tq, 1, D), dtype=np.float32)
    q[..., 0] = 1.0
    nsb = (L + SB - 1) // SB
    mk = np.zeros((1, nsb, 1, D))
    mk[0, :, 0, 0] = 1.0
    mk[0, nsb - 2:, 0, 0] = -1e6  # the last blocks are the least similar
    assert kept_blocks(L, Tq, SB) == expect
    sel, cnt, _ = oracle.sparse_select(q, mk, np.array([L], np.int32), 1.0, SB, 1, 2)
    assert list(sel[0, 0, :cnt[0, 0]]) == expect


def test_selection_closed_form_picks_the_aligned_block():
    # keys of sparse block 5 of the sequence all equal 3 e_0 (head 0), every
    # other key is e_1: q = e_0 scores block 5 highest, q = -e_0 lowest
    SB = 16
    w = small("f32", B=1, Hq=2, Hkv=1, D=16, lens=(200,), seed=3)
    w.k_src[:] = 0.0
    w.k_src[:, :, 1] = 1.0
    pos = w.row_pos
    w.k_src[(pos >= 80) & (pos < 96), :, :] = 0.0
    w.k_src[(pos >= 80) & (pos < 96), :, 0] = 3.0
    k, v, ks, vs = oracle_cache(w)
    mk = oracle.sparse_mean_keys(k, w.block_table, w.seq_lens, SB, 13)
    assert np.all(mk[0, 5, 0] == np.eye(16)[0] * 3.0)
    q = np.zeros((1, 1, 2, 16), dtype=np.float32)
    q[..., 0] = 1.0
    sel, cnt, _ = oracle.sparse_select(q, mk, w.seq_lens, 1.0, SB, 2, 2)
    assert list(sel[0, 0]) == [5, 12]  # block 12 holds the query token
    q[..., 0] = -1.0
    sel, cnt, _ = oracle.sparse_select(q, mk, w.seq_lens, 1.0, SB, 12, 12)
    assert 5 not in list(sel[0, 0]) and cnt[0, 0] == 12


@pytest.mark.parametrize("kv", ["bf16", "i8", "nvfp4"])
@pytest.mark.parametrize("Tq", [1, 4])
def test_all_blocks_selected_is_the_plain_decode_bitwise(kv, Tq):
    w = small(kv, Tq=Tq, lens=(0, 3, 100, 300), seed=4)
    cache = oracle_cache(w)
    k, v, ks, vs = cache
    q = w.q_array()
    out, lse, sel, cnt, _ = oracle.decode_sparse(q, k, v, w.block_table, w.seq_lens, w.softmax_scale, 64, 5, ks, vs)
    ref, rlse = oracle.decode(q, k, v, w.block_table, w.seq_lens, w.softmax_scale, ks, vs)
    assert np.array_equal(out, ref) and np.array_equal(lse, rlse)
    for b, L in enumerate(w.seq_lens):
        assert np.all(cnt[b] == oracle.num_sparse_blocks(int(L), 64))


def compacted(w, sel, cnt, g, SB):
    """Per-sequence block table of kv head g listing the cache blocks of its
    selected sparse blocks in order, and the compacted lengths."""
    B = w.spec.B
    per = SB // BLOCK_SIZE
    rows, lens = [], []
    for b in range(B):
        L = int(w.seq_lens[b])
        blocks = []
        n = 0
        for j in sel[b, g, :cnt[b, g]]:
            blocks += list(w.block_table[b, j * per:(j + 1) * per])
            n += min(L, (j + 1) * SB) - j * SB
        rows.append(blocks)
        lens.append(n)
    width = max(1, max(len(r) for r in rows))
    table = np.zeros((B, width), dtype=np.int32)
    for b, r in enumerate(rows):
        table[b, :len(r)] = r
    return table, np.array(lens, dtype=np.int32)


@pytest.mark.parametrize("Tq", [1, 8])
@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_subset_decode_is_the_plain_decode_of_the_compacted_table(Tq, kv):
    # selection with few blocks: the decode over the selected keys equals the
    # plain decode of each kv head on a block table that lists only the
    # selected blocks (all of them full but the last), bit for bit
    SB = 32
    w = small(kv, Tq=Tq, Hq=6, Hkv=2, D=64, lens=(9, 40, 203, 333), seed=5)
    k, v, ks, vs = oracle_cache(w)
    q = w.q_array()
    out, lse, sel, cnt, _ = oracle.decode_sparse(q, k, v, w.block_table, w.seq_lens, w.softmax_scale, SB, 3, ks, vs)
    G = 3
    for g in range(2):
        table, lens = compacted(w, sel, cnt, g, SB)
        sl = slice(g * G, (g + 1) * G)
        qg = np.ascontiguousarray(q[:, :, sl])
        kg, vg = np.ascontiguousarray(k[:, :, g:g + 1]), np.ascontiguousarray(v[:, :, g:g + 1])
        ksg = None if ks is None else np.ascontiguousarray(ks[:, g:g + 1])
        vsg = None if vs is None else np.ascontiguousarray(vs[:, g:g + 1])
        ref, rlse = oracle.decode(qg, kg, vg, table, lens, w.softmax_scale, ksg, vsg)
        assert np.array_equal(out[:, :, sl], ref)
        assert np.array_equal(lse[:, :, sl], rlse)


def test_subset_decode_matches_decimal_brute_force():
    SB = 16
    w = small("bf16", Tq=2, Hq=2, Hkv=1, D=8, lens=(40, 70), seed=6)
    k, v, ks, vs = oracle_cache(w)
    q = w.q_array()
    # an explicit selection: sequence 0 blocks {0, 2} (block 2 holds its
    # query tokens), sequence 1 blocks {1, 4} (block 4 holds its query tokens)
    sel = np.array([[[0, 2]], [[1, 4]]], dtype=np.int32)
    cnt = np.array([[2], [2]], dtype=np.int32)
    out, lse = oracle.decode_subset(q, k, v, w.block_table, w.seq_lens, w.softmax_scale, sel, cnt, SB)
    table, lens = compacted(w, sel, cnt, 0, SB)
    bo, bl = brute_decode(q, k, v, table, lens, w.softmax_scale)
    assert np.max(np.abs(out - bo)) <= 1e-12
    assert np.max(np.abs(lse - bl)) <= 1e-12


def test_sparse_decode_approaches_full_attention_with_more_blocks():
    # not a parity bound (the method is approximate): with peaked keys the
    # error against full attention falls as more blocks are selected and is 0
    # with all of them
    spec = scaled("long64k_bf16", B=2, Tq=1, Hq=4, Hkv=1, D=64, seq_lens=(2000, 2000), peaked_frac=0.01)
    w = generate(spec, seed=7)
    k, v, ks, vs = oracle_cache(w)
    q = w.q_array()
    full, _ = oracle.decode(q, k, v, w.block_table, w.seq_lens, w.softmax_scale)
    errs = []
    for top in (4, 16, 32):
        out, *_ = oracle.decode_sparse(q, k, v, w.block_table, w.seq_lens, w.softmax_scale, 64, top)
        errs.append(float(np.max(np.abs(out - full))))
    assert errs[0] >= errs[1] >= errs[2] == 0.0, errs
