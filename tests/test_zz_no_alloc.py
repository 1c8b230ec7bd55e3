"""pa_decode_noalloc through the C ABI: the split-K partials live in the
library's own scratch instead of a caller workspace. Two calls in a row (the
second on a smaller input, so the scratch still holds the first call's larger
partials) and one single-partition call must each give exactly the bits of
pa_decode + pa_decode_splitk_reduce with a caller workspace, and stay within
the oracle tolerance."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import paged_attention_decode_02_amd as pa
from _gpu import dev, gpu_cache, gpu_inputs
from _host import oracle_cache, oracle_decode
from workloads import generate, scaled

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "i8": 2e-2}


def noalloc(w, cache, P):
    """Call pa_decode_noalloc directly through ctypes; returns (out, lse)."""
    sp = w.spec
    q, table, lens = gpu_inputs(w)
    k, v, ks, vs = cache
    out = torch.full((sp.B, sp.Tq, sp.Hq, sp.D), float("nan"), dtype=torch.float32, device=dev())
    lse = torch.full((sp.B, sp.Tq, sp.Hq), float("nan"), dtype=torch.float32, device=dev())
    lib = pa.load()
    nb = k.shape[0]
    rc = lib.pa_decode_noalloc(q.data_ptr(), pa.DTYPE_CODE[q.dtype], sp.B, sp.Tq, sp.Hq, sp.Hkv, sp.D, k.data_ptr(),
                               v.data_ptr(), pa.DTYPE_CODE[k.dtype], None if ks is None else ks.data_ptr(),
                               None if vs is None else vs.data_ptr(), nb, 16, table.data_ptr(), table.shape[1],
                               lens.data_ptr(), w.max_seq_len, w.softmax_scale, P, out.data_ptr(), 0, lse.data_ptr(),
                               torch.cuda.current_stream().cuda_stream)
    assert rc == 0, lib.pa_last_error()
    torch.cuda.synchronize()
    return out, lse, q, table, lens


def check_against_decode(w, P):
    print("pa_decode_noalloc: %s B=%d Tq=%d Hq=%d Hkv=%d D=%d max_len=%d P=%d" % (
        w.spec.name, w.spec.B, w.spec.Tq, w.spec.Hq, w.spec.Hkv, w.spec.D, w.max_seq_len, P), flush=True)
    cache = gpu_cache(w)
    out, lse, q, table, lens = noalloc(w, cache, P)
    k, v, ks, vs = cache
    ref, rlse = pa.decode(q, k, v, table, lens, w.max_seq_len, w.softmax_scale, ks, vs, partition_size=P)
    torch.cuda.synchronize()
    assert torch.equal(out, ref), float((out - ref).abs().max())
    assert torch.equal(lse, rlse)
    o, lo = oracle_decode(w, oracle_cache(w))
    err = float(np.max(np.abs(out.cpu().numpy().astype(np.float64) - o)))
    assert err <= TOL[w.spec.cache_dtype], err
    return pa.workspace_bytes(w.spec.B, w.spec.Tq, w.spec.Hq, w.spec.Hkv, w.spec.D, k.dtype, w.max_seq_len, P)


def test_noalloc_matches_decode_on_two_calls_in_a_row():
    # first call: speculative-verify shape with many partitions (int8 KV)
    big = generate(scaled("verify_i8", B=3, Tq=4, Hq=12, Hkv=2, D=128, seq_lens=(300, 3000), shared_prefix=0),
                   seed=11)
    n1 = check_against_decode(big, 256)
    # second call, smaller: fewer rows and partitions than the scratch holds
    small = generate(scaled("gqa_bf16", B=2, Tq=1, Hq=8, Hkv=2, D=64, seq_lens=(40, 900)), seed=12)
    n2 = check_against_decode(small, 0)
    assert 0 < n2 < n1 <= pa.NOALLOC_SCRATCH_BYTES
    # a single partition: out is written by the decode itself
    one = generate(scaled("gqa_bf16", B=2, Tq=1, Hq=8, Hkv=2, D=64, seq_lens=(10, 60)), seed=13)
    assert check_against_decode(one, 64) == 0


def test_noalloc_binding_and_rejection():
    w = generate(scaled("gqa_bf16", B=2, Tq=2, Hq=8, Hkv=2, D=128, seq_lens=(100, 2000)), seed=14)
    cache = gpu_cache(w)
    q, table, lens = gpu_inputs(w)
    k, v, ks, vs = cache
    out = torch.empty((2, 2, 8, 128), dtype=torch.float32, device=dev())
    lse = torch.empty((2, 2, 8), dtype=torch.float32, device=dev())
    pa.decode_noalloc(q, k, v, table, lens, w.max_seq_len, w.softmax_scale, out, lse, partition_size=128)
    ref, rlse = pa.decode(q, k, v, table, lens, w.max_seq_len, w.softmax_scale, partition_size=128)
    torch.cuda.synchronize()
    assert torch.equal(out, ref) and torch.equal(lse, rlse)
    # 40 copies of the batch at 16-token partitions need 78 MiB of partials,
    # beyond the 32 MiB scratch: refused before any launch
    big = torch.empty((2, 2, 8, 128), dtype=torch.float32, device=dev())
    with pytest.raises(pa.PaError) as e:
        pa.decode_noalloc(q.repeat(40, 1, 1, 1), k, v, table.repeat(40, 1), lens.repeat(40), w.max_seq_len,
                          w.softmax_scale, big.repeat(40, 1, 1, 1), None, partition_size=16)
    assert e.value.code == -5
