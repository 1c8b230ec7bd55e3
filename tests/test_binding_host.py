"""The binding's shape and dtype validation (CPU only): the C ABI sees only
pointers, so every size the kernels trust is checked on tensor metadata before
a launch, and a mismatch raises ValueError instead of reading out of bounds."""
from __future__ import annotations

import pytest
import torch

import paged_attention_decode_02_amd as pa


def decode_case(kv=torch.bfloat16, D=128, **over):
    B, Tq, Hq, Hkv, nb = 2, 3, 8, 2, 40
    row = 9 * D // 16 if kv == torch.float4_e2m1fn_x2 else D
    t = dict(
        q=torch.zeros(B, Tq, Hq, D, dtype=torch.bfloat16),
        k_cache=torch.zeros(nb, 16, Hkv, row, dtype=torch.uint8).view(kv) if kv.itemsize == 1 and kv != torch.int8
        else torch.zeros(nb, 16, Hkv, row, dtype=kv),
        block_table=torch.zeros(B, 10, dtype=torch.int32),
        seq_lens=torch.zeros(B, dtype=torch.int32),
        max_seq_len=160,
        out=torch.zeros(B, Tq, Hq, D),
        lse=torch.zeros(B, Tq, Hq),
        k_scale=None, v_scale=None,
    )
    t["v_cache"] = t["k_cache"].clone()
    if kv in pa.QUANTISED:
        t["k_scale"] = torch.zeros(nb, Hkv, 16)
        t["v_scale"] = torch.zeros(nb, Hkv, 16)
    t.update(over)
    return t


def run(t):
    pa.validate_decode_args(t["q"], t["k_cache"], t["v_cache"], t["block_table"], t["seq_lens"], t["max_seq_len"],
                            t["out"], t["lse"], t["k_scale"], t["v_scale"])


@pytest.mark.parametrize("kv", [torch.float32, torch.bfloat16, torch.int8, torch.float8_e4m3fn,
                                torch.float4_e2m1fn_x2])
def test_valid_decode_arguments_pass(kv):
    run(decode_case(kv))


@pytest.mark.parametrize("change", [
    dict(q=torch.zeros(2, 3, 8, 256, dtype=torch.bfloat16)),        # D 256 against D 128 caches
    dict(q=torch.zeros(2, 3, 8, 128, dtype=torch.float16)),         # q dtype
    dict(q=torch.zeros(2, 3, 7, 128, dtype=torch.bfloat16)),        # Hq not a multiple of Hkv
    dict(block_table=torch.zeros(3, 10, dtype=torch.int32)),        # table rows != B
    dict(block_table=torch.zeros(2, 9, dtype=torch.int32)),         # 9 * 16 < max_seq_len
    dict(block_table=torch.zeros(2, 10, dtype=torch.int64)),        # table dtype
    dict(seq_lens=torch.zeros(3, dtype=torch.int32)),               # lengths != B
    dict(seq_lens=torch.zeros(2, dtype=torch.int64)),
    dict(out=torch.zeros(2, 3, 8, 64)),                             # out shape
    dict(out=torch.zeros(2, 3, 8, 128, dtype=torch.float16)),       # out dtype
    dict(lse=torch.zeros(2, 3)),                                    # lse shape
    dict(v_cache=torch.zeros(40, 16, 2, 64, dtype=torch.bfloat16)),  # K and V differ
    dict(k_cache=torch.zeros(40, 8, 2, 128, dtype=torch.bfloat16),
         v_cache=torch.zeros(40, 8, 2, 128, dtype=torch.bfloat16)),  # block size 8
])
def test_bad_decode_arguments_raise(change):
    with pytest.raises(ValueError):
        run(decode_case(**change))


@pytest.mark.parametrize("kv", [torch.int8, torch.float8_e4m3fn, torch.float4_e2m1fn_x2])
def test_quantised_caches_need_matching_scales(kv):
    with pytest.raises(ValueError):
        run(decode_case(kv, k_scale=None))
    with pytest.raises(ValueError):
        run(decode_case(kv, v_scale=torch.zeros(40, 16, 2)))            # token-major scales
    with pytest.raises(ValueError):
        run(decode_case(kv, k_scale=torch.zeros(40, 2, 16, dtype=torch.float64)))


def test_nvfp4_rows_are_checked_against_the_head_size():
    with pytest.raises(ValueError):
        run(decode_case(torch.float4_e2m1fn_x2, q=torch.zeros(2, 3, 8, 256, dtype=torch.bfloat16)))


def test_cache_write_validation():
    k = torch.zeros(5, 2, 128)
    kc = torch.zeros(40, 16, 2, 128, dtype=torch.bfloat16)
    slots = torch.zeros(5, dtype=torch.int64)
    pa.validate_cache_write_args(k, k.clone(), slots, kc, kc.clone())
    with pytest.raises(ValueError):
        pa.validate_cache_write_args(k, k.clone(), slots[:4], kc, kc.clone())            # N mismatch
    with pytest.raises(ValueError):
        pa.validate_cache_write_args(k, k.clone(), slots.int(), kc, kc.clone())          # slot dtype
    with pytest.raises(ValueError):
        pa.validate_cache_write_args(torch.zeros(5, 4, 128), torch.zeros(5, 4, 128), slots, kc, kc.clone())
    with pytest.raises(ValueError):
        pa.validate_cache_write_args(torch.zeros(5, 2, 64), torch.zeros(5, 2, 64), slots, kc, kc.clone())
    kq = torch.zeros(40, 16, 2, 128, dtype=torch.int8)
    with pytest.raises(ValueError):
        pa.validate_cache_write_args(k, k.clone(), slots, kq, kq.clone())               # int8 needs scales
    pa.validate_cache_write_args(k, k.clone(), slots, kq, kq.clone(), torch.zeros(40, 2, 16),
                                 torch.zeros(40, 2, 16))
