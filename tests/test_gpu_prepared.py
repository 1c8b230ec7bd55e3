"""Prepared calls (checks and argument marshalling done once) launch exactly
the work of the ordinary calls: bitwise equal outputs, also when the tensors'
contents change between calls and when replayed from a HIP graph."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import paged_attention_decode_02_amd as pa
from _gpu import dev, gpu_cache, gpu_inputs, host_to_dev
from workloads import generate, scaled

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kv, P", [("bf16", 0), ("bf16", 64), ("i8", 0), ("fp8", 128), ("nvfp4", 0), ("bf16", 4096)])
def test_prepared_step_equals_the_ordinary_calls(kv, P):
    spec = scaled("gqa_bf16", B=3, Tq=2, Hq=12, Hkv=2, D=128, seq_lens=(100, 1500), cache_dtype=kv,
                  src_dtype="f32")
    w = generate(spec, seed=160)
    k, v, ks, vs = gpu_cache(w)

    def raw(t):  # the bytes of a cache tensor (poisoned slots hold NaN; fp8 / fp4 storage has few torch ops)
        return t.view(torch.uint8)

    k2, v2 = raw(k).clone().view(k.dtype), raw(v).clone().view(v.dtype)
    ks2 = None if ks is None else ks.clone()
    vs2 = None if vs is None else vs.clone()
    q, table, lens = gpu_inputs(w)
    rows = w.step_rows()
    new_k = host_to_dev(w.k_src[rows], spec.src_dtype)
    new_v = host_to_dev(w.v_src[rows], spec.src_dtype)
    slots = torch.from_numpy(np.ascontiguousarray(w.slot_mapping[rows])).to(dev())
    PP = P or pa.choose_partition_size(spec.B, spec.Tq, spec.Hq, spec.Hkv, spec.D, k.dtype, w.max_seq_len)
    nbytes = pa.workspace_bytes(spec.B, spec.Tq, spec.Hq, spec.Hkv, spec.D, k.dtype, w.max_seq_len, PP)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev())
    out = torch.empty((spec.B, spec.Tq, spec.Hq, spec.D), dtype=torch.float32, device=dev())
    lse = torch.empty((spec.B, spec.Tq, spec.Hq), dtype=torch.float32, device=dev())
    cw = pa.prepare_cache_write(new_k, new_v, slots, k2, v2, ks2, vs2)
    dec = pa.prepare_decode(q, k2, v2, table, lens, w.max_seq_len, w.softmax_scale, out, lse, ks2, vs2, P, ws)
    assert dec.num_partitions == (w.max_seq_len + PP - 1) // PP
    for i in range(3):
        q.copy_(q.roll(1, dims=2))  # new contents, same buffers
        cw()
        dec()
        pa.cache_write(new_k, new_v, slots, k, v, ks, vs)
        ref_o, ref_l = pa.decode(q, k, v, table, lens, w.max_seq_len, w.softmax_scale, ks, vs, P)
        torch.cuda.synchronize()
        assert bool(torch.equal(raw(k), raw(k2))) and bool(torch.equal(raw(v), raw(v2))), "caches differ, %d" % i
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), i
    # the same prepared step recorded in a graph
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cw()
        dec()
    torch.cuda.synchronize()
    for i in range(3):
        q.copy_(q.roll(1, dims=2))
        g.replay()
        torch.cuda.synchronize()
        ref_o, ref_l = pa.decode(q, k, v, table, lens, w.max_seq_len, w.softmax_scale, ks, vs, P)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), i


def test_prepared_calls_check_their_tensors_once():
    spec = scaled("gqa_bf16", B=2, Tq=1, Hq=4, Hkv=2, D=64, seq_lens=(50, 300))
    w = generate(spec, seed=161)
    k, v, ks, vs = gpu_cache(w)
    q, table, lens = gpu_inputs(w)
    out = torch.empty((2, 1, 4, 64), dtype=torch.float32, device=dev())
    with pytest.raises(ValueError):
        pa.prepare_decode(q, k, v, table, lens, w.max_seq_len, w.softmax_scale, out[:, :, :2], None)
    with pytest.raises(ValueError):  # partitions need a workspace
        pa.prepare_decode(q, k, v, table, lens, w.max_seq_len, w.softmax_scale, out, None, partition_size=16)
