"""GPU parity of the shared-prefix decode (pa_decode_shared_prefix) against the
fp64 oracle.

The shared-prefix decode computes what pa_decode computes: the oracle's plain
definition (every row's softmax over all its visible keys, gathered through
the sequence's block table) is the reference, at the same tolerances as the
plain decode. The batch's sequences share their first prefix_len tokens in the
same physical blocks (the generator's shared_prefix); the library reads them
through prefix_table once for the whole batch, then each sequence's own tail.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import paged_attention_decode_02_amd as pa
from _gpu import cache_bytes_equal, dev, gpu_cache, gpu_decode, gpu_inputs, host_to_dev
from _host import oracle_cache, oracle_decode
from test_gpu_parity import check, say
from workloads import SPECS, generate, scaled

pytestmark = pytest.mark.gpu


def shared_decode(w, cache, prefix_partition=0, tail_partition=0, table=None, out_dtype=torch.float32):
    q, tab, lens = gpu_inputs(w)
    if table is not None:
        tab = table
    k, v, ks, vs = cache
    n_pre = w.spec.shared_prefix // 16
    prefix_table = torch.from_numpy(np.ascontiguousarray(w.block_table[0, :n_pre])).to(dev())
    out, lse = pa.decode_shared_prefix(q, k, v, prefix_table, w.spec.shared_prefix, tab, lens, w.max_seq_len,
                                       w.softmax_scale, ks, vs, prefix_partition=prefix_partition,
                                       tail_partition=tail_partition, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out, lse


def run_shared(w, parts=((0, 0),), check_cache=True):
    sp = w.spec
    say("shared prefix %s B=%d Tq=%d Hq=%d Hkv=%d D=%d kv=%s prefix=%d lens=%d..%d" % (
        sp.name, sp.B, sp.Tq, sp.Hq, sp.Hkv, sp.D, sp.cache_dtype, sp.shared_prefix, w.seq_lens.min(),
        w.seq_lens.max()))
    host = oracle_cache(w)
    cache = gpu_cache(w)
    if check_cache:
        assert cache_bytes_equal(cache, host), "pa_cache_write differs from the oracle writer"
    ref = oracle_decode(w, host)
    for pp, tp in parts:
        check(w, shared_decode(w, cache, pp, tp), ref, "prefix P=%d tail P=%d" % (pp, tp))
    return cache, host, ref


# ------------------------------------------------------------ full size
@pytest.mark.parametrize("name", ["verify_bf16", "verify_i8"])
def test_verify_workload_full_size(name):
    # 4 sequences of 16-32K tokens, 8 query tokens each, 4096 shared tokens
    run_shared(generate(name), parts=((0, 0), (1024, 512)))


def test_prefix_batch_workload_full_size():
    run_shared(generate("prefix32k_bf16"))


# ------------------------------------------------------------ shapes and dtypes
@pytest.mark.parametrize("kv", ["bf16", "i8", "fp8", "nvfp4"])
@pytest.mark.parametrize("Tq", [1, 3, 8])
def test_dtypes_and_query_tokens(kv, Tq):
    spec = scaled("verify_bf16", B=3, Tq=Tq, Hq=12, Hkv=2, D=128, seq_lens=(512 + Tq, 1300), shared_prefix=512,
                  cache_dtype=kv, src_dtype="f32")
    run_shared(generate(spec, seed=40 + Tq), parts=((0, 0), (64, 128)))


@pytest.mark.parametrize("D", [64, 256])
@pytest.mark.parametrize("qdt", ["f32", "bf16"])
def test_head_dims_and_query_dtype(D, qdt):
    spec = scaled("verify_bf16", B=2, Tq=2, Hq=8, Hkv=2, D=D, seq_lens=(300, 900), shared_prefix=256,
                  q_dtype=qdt)
    run_shared(generate(spec, seed=50 + D), parts=((0, 0), (16, 16)))


@pytest.mark.parametrize("B, Tq, G", [(16, 1, 6), (8, 8, 6), (5, 1, 16), (2, 4, 1), (33, 2, 4)])
def test_row_sets_of_many_sequences(B, Tq, G):
    # B * Tq * G rows per kv head in chunks of 64: 96, 384, 80, 8, 264
    spec = scaled("verify_bf16", B=B, Tq=Tq, Hq=2 * G, Hkv=2, D=128, seq_lens=(1024 + Tq, 1600),
                  shared_prefix=1024)
    run_shared(generate(spec, seed=60 + B), parts=((0, 0), (256, 0)))


@pytest.mark.parametrize("pp, tp", [(16, 16), (64, 0), (256, 256), (2048, 4096), (0, 16)])
def test_partition_sizes(pp, tp):
    spec = scaled("verify_bf16", B=3, Tq=8, Hq=24, Hkv=4, D=256, seq_lens=(2048 + 8, 3500), shared_prefix=2048)
    run_shared(generate(spec, seed=7), parts=((pp, tp),))


def test_tails_of_only_the_query_tokens_and_no_prefix():
    # every sequence is the prefix plus its Tq query tokens, or (prefix 0) the
    # plain decode through the same entry point
    spec = scaled("verify_bf16", B=4, Tq=8, Hq=12, Hkv=2, D=128, seq_lens=(776, 776), shared_prefix=768)
    run_shared(generate(spec, seed=8, seq_lens=[776, 776, 777, 800]), parts=((0, 0), (16, 16)))
    spec0 = scaled(spec, shared_prefix=0, seq_lens=(8, 900))
    # (0, 1024): one tail partition and no prefix, so out is written directly
    run_shared(generate(spec0, seed=9, seq_lens=[8, 9, 400, 900]), parts=((0, 0), (0, 16), (0, 1024)))


def test_shared_entries_of_the_block_table_are_not_read():
    # the per-sequence table's prefix entries point at poisoned slack blocks:
    # the prefix must come through prefix_table only
    spec = scaled("verify_bf16", B=3, Tq=4, Hq=8, Hkv=2, D=128, seq_lens=(600, 1000), shared_prefix=512,
                  cache_dtype="i8", src_dtype="f32")
    w = generate(spec, seed=10)
    cache, host, ref = run_shared(w)
    tab = w.block_table.copy()
    tab[:, : 512 // 16] = w.slack_blocks[0]
    check(w, shared_decode(w, cache, 0, 0, table=torch.from_numpy(tab).to(dev())), ref, "poisoned prefix entries")


def test_matches_plain_decode_and_is_deterministic():
    spec = scaled("verify_bf16", B=4, Tq=8, Hq=24, Hkv=4, D=256, seq_lens=(4096 + 8, 6000), shared_prefix=4096)
    w = generate(spec, seed=11)
    cache = gpu_cache(w)
    a, la = shared_decode(w, cache)
    b, lb = shared_decode(w, cache)
    assert torch.equal(a, b) and torch.equal(la, lb)
    c, lc = gpu_decode(w, cache)
    # both within the oracle tolerance of the same exact result
    assert float((a - c).abs().max()) <= 2e-2
    assert float((la - lc).abs().max()) <= 2e-3


def test_bf16_output():
    spec = scaled("verify_bf16", B=2, Tq=4, Hq=8, Hkv=2, D=128, seq_lens=(400, 900), shared_prefix=256)
    w = generate(spec, seed=12)
    host = oracle_cache(w)
    cache = gpu_cache(w)
    out, _ = shared_decode(w, cache, out_dtype=torch.bfloat16)
    rout, _ = oracle_decode(w, host)
    o = out.float().cpu().numpy()
    assert np.all(np.abs(o - rout) <= 1e-2 + np.abs(rout) * 2.0 ** -8)


def test_host_checks():
    spec = scaled("verify_bf16", B=2, Tq=4, Hq=8, Hkv=2, D=128, seq_lens=(400, 900), shared_prefix=256)
    w = generate(spec, seed=13)
    cache = gpu_cache(w)
    q, tab, lens = gpu_inputs(w)
    k, v, ks, vs = cache
    pt = tab[0, :16].contiguous()
    with pytest.raises(pa.PaError) as e:  # not a whole number of blocks
        pa.decode_shared_prefix(q, k, v, pt, 250, tab, lens, w.max_seq_len, w.softmax_scale)
    assert e.value.code == -2
    with pytest.raises(pa.PaError) as e:  # no room for the query tokens
        pa.decode_shared_prefix(q, k, v, tab[0, :52].contiguous(), 832, tab, lens, 834, w.softmax_scale)
    assert e.value.code == -2
    with pytest.raises(ValueError):  # a prefix table shorter than the prefix (caught by the binding)
        pa.decode_shared_prefix(q, k, v, pt, 512, tab, lens, w.max_seq_len, w.softmax_scale)
    with pytest.raises(pa.PaError) as e:  # workspace too small
        pa.decode_shared_prefix(q, k, v, pt, 256, tab, lens, w.max_seq_len, w.softmax_scale,
                                workspace=torch.empty(256, dtype=torch.uint8, device=dev()))
    assert e.value.code == -5


@pytest.mark.parametrize("kv", ["bf16", "i8"])
def test_shared_prefix_step_captured_in_a_graph(kv):
    """cache_write + the shared-prefix decode (three kernels) recorded in one
    HIP graph: every replay, with new query values written eagerly in between,
    equals an eager run bit for bit."""
    spec = scaled("verify_bf16", B=4, Tq=8, Hq=24, Hkv=4, D=256, seq_lens=(2048 + 8, 4000), shared_prefix=2048,
                  cache_dtype=kv, src_dtype="bf16")
    w = generate(spec, seed=14)
    cache = gpu_cache(w)
    k, v, ks, vs = cache
    q, table, lens = gpu_inputs(w)
    rows = w.step_rows()
    new_k = host_to_dev(w.k_src[rows], spec.src_dtype)
    new_v = host_to_dev(w.v_src[rows], spec.src_dtype)
    new_slots = torch.from_numpy(w.slot_mapping[rows]).to(dev())
    prefix_table = torch.from_numpy(np.ascontiguousarray(w.block_table[0, :2048 // 16])).to(dev())
    nbytes = pa.shared_prefix_workspace_bytes(spec.B, spec.Tq, spec.Hq, spec.Hkv, spec.D, k.dtype, w.max_seq_len,
                                              2048)
    ws = torch.empty(max(256, nbytes), dtype=torch.uint8, device=dev())
    out = torch.empty((spec.B, spec.Tq, spec.Hq, spec.D), dtype=torch.float32, device=dev())
    lse = torch.empty((spec.B, spec.Tq, spec.Hq), dtype=torch.float32, device=dev())

    def step():
        pa.cache_write(new_k, new_v, new_slots, k, v, ks, vs)
        pa.decode_shared_prefix(q, k, v, prefix_table, 2048, table, lens, w.max_seq_len, w.softmax_scale, ks, vs,
                                out=out, lse=lse, workspace=ws)

    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for i in range(4):
        q.copy_(q.roll(1, dims=2))
        g.replay()
        torch.cuda.synchronize()
        got_o, got_l = out.clone(), lse.clone()
        step()
        torch.cuda.synchronize()
        assert torch.equal(got_o, out) and torch.equal(got_l, lse), "replay %d differs from eager" % i
