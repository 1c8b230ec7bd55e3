"""GPU-side test plumbing: device tensors for a generated workload.

The device caches are first filled with poison, then written by the library's
pa_cache_write, so every slot that holds no source row stays poisoned (NaN for
float caches; code 127 with a NaN scale for int8 and FP8, where 127 is an
E4M3 NaN) exactly as the oracle's
host caches are (tests/_host.py).
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import paged_attention_decode_02_amd as pa
from _host import POISON_CODE
from workloads import BLOCK_SIZE, Workload

TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "i8": torch.int8, "fp8": torch.float8_e4m3fn,
            "nvfp4": torch.float4_e2m1fn_x2}


def dev():
    return torch.device("cuda:0")


def host_to_dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    """Upload a host array (bf16 given as uint16 patterns) as a device tensor."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev())
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def dev_to_host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype in (torch.float8_e4m3fn, torch.float4_e2m1fn_x2):
        return t.view(torch.uint8).numpy()
    return t.numpy()


def poisoned_cache(w: Workload):
    sp = w.spec
    row = oracle.nvfp4_row_bytes(sp.D) if sp.cache_dtype == "nvfp4" else sp.D
    shape = (w.num_blocks, BLOCK_SIZE, sp.Hkv, row)
    dt = TORCH_DT[sp.cache_dtype]
    if sp.cache_dtype in ("i8", "fp8", "nvfp4"):
        k = torch.full(shape, POISON_CODE, dtype=torch.uint8, device=dev()).view(dt)
        ks = torch.full((shape[0], sp.Hkv, BLOCK_SIZE), float("nan"), dtype=torch.float32, device=dev())
        return k, k.clone(), ks, ks.clone()
    if sp.cache_dtype == "bf16":
        k = torch.full(shape, 0x7FC0, dtype=torch.int16, device=dev()).view(torch.bfloat16)
    else:
        k = torch.full(shape, float("nan"), dtype=dt, device=dev())
    return k, k.clone(), None, None


def gpu_cache(w: Workload, chunk: int = 1 << 20):
    """Poisoned caches populated by pa.cache_write (in chunks of source rows)."""
    k, v, ks, vs = poisoned_cache(w)
    N = w.slot_mapping.shape[0]
    for s in range(0, N, chunk):
        e = min(N, s + chunk)
        ksrc = host_to_dev(w.k_src[s:e], w.spec.src_dtype)
        vsrc = host_to_dev(w.v_src[s:e], w.spec.src_dtype)
        slots = torch.from_numpy(w.slot_mapping[s:e]).to(dev())
        pa.cache_write(ksrc, vsrc, slots, k, v, ks, vs)
    torch.cuda.synchronize()
    return k, v, ks, vs


def gpu_inputs(w: Workload):
    q = host_to_dev(w.q_array(), w.spec.q_dtype)
    table = torch.from_numpy(w.block_table).to(dev())
    lens = torch.from_numpy(w.seq_lens).to(dev())
    return q, table, lens


def gpu_decode(w: Workload, cache, partition_size: int = 0, out_dtype=torch.float32, q=None, table=None, lens=None):
    if q is None:
        q, table, lens = gpu_inputs(w)
    k, v, ks, vs = cache
    out, lse = pa.decode(q, k, v, table, lens, w.max_seq_len, w.softmax_scale, ks, vs,
                         partition_size=partition_size, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out, lse


def cache_bytes_equal(gpu_cache_t, host_cache) -> bool:
    for g, h in zip(gpu_cache_t, host_cache):
        if g is None and h is None:
            continue
        a = dev_to_host(g)
        if a.dtype == np.float32:
            if not np.array_equal(a.view(np.uint32), h.view(np.uint32)):
                return False
        elif not np.array_equal(a, h):
            return False
    return True
