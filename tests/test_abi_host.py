"""The C ABI library: it loads, exports every declared symbol, and rejects bad
arguments on the host before touching a device (CPU only, no GPU needed)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import paged_attention_decode_02_amd as pa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pa_decode.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pa.library_path()):
        from paged_attention_decode_02_amd import build

        build.build()
    return pa.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_exports():
    assert set(declared_functions()) == set(pa.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


# dummy, 16-byte aligned, never dereferenced: every call below fails validation first
A = ctypes.c_void_p(0x1000)
NP = ctypes.c_int32(0)


def decode_args(**over):
    args = dict(q=A, q_dtype=1, B=2, Tq=1, Hq=8, Hkv=2, D=128, k_cache=A, v_cache=A, kv_dtype=1, k_scale=None,
                v_scale=None, num_blocks=64, block_size=16, block_table=A, max_blocks=64, seq_lens=A,
                max_seq_len=1000, scale=0.088, partition_size=0, out=A, out_dtype=0, lse=None, workspace=None,
                workspace_bytes=0, num_partitions=ctypes.byref(NP), stream=None)
    args.update(over)
    return list(args.values())


@pytest.mark.parametrize("over, code", [
    (dict(q=None), -1),
    (dict(out=None), -1),
    (dict(num_partitions=None), -1),
    (dict(kv_dtype=2), -1),  # int8 without scales
    (dict(kv_dtype=3), -1),  # fp8 without scales
    (dict(kv_dtype=4), -1),  # nvfp4 without scales
    (dict(q_dtype=2), -3),
    (dict(kv_dtype=7), -3),
    (dict(out_dtype=2), -3),
    (dict(Hq=7), -2),
    (dict(B=-1), -2),
    (dict(Tq=0), -2),
    (dict(Tq=17), -4),
    (dict(D=96), -4),
    (dict(block_size=32), -4),
    (dict(Hq=130, Hkv=2), -4),
    (dict(max_blocks=10), -2),  # 10 * 16 < 1000
    (dict(partition_size=100), -2),
    (dict(q=ctypes.c_void_p(0x1004)), -7),
    (dict(partition_size=256), -5),  # 4 partitions, no workspace
])
def test_decode_rejects_bad_arguments(lib, over, code):
    rc = lib.pa_decode(*decode_args(**over))
    assert rc == code, lib.pa_last_error()
    assert lib.pa_last_error()  # a message is set


def test_workspace_size_and_partition_choice(lib):
    # the long-context workload: 4 sequences x 64 partitions of 1024 tokens =
    # 256 four-wave workgroups (one per CU), each wave one of the 4 kv heads
    P = lib.pa_choose_partition_size(4, 1, 24, 4, 256, 1, 65536)
    assert P == 1024
    need = lib.pa_decode_workspace_bytes(4, 1, 24, 4, 256, 1, 65536, 2048)
    rows = 4 * 24
    assert need == rows * 32 * 256 * 4 + rows * 32 * 4
    # int8 caches with G = 6 run on the streaming matrix-core kernel: one
    # workgroup per CU taking all 4 kv heads (one wave each): 253 partitions
    # of 992 tokens
    assert lib.pa_choose_partition_size(1, 1, 24, 4, 256, 2, 250000) == 992
    # so do fp8 caches (two waves per head); nvfp4 caches with G = 6 stay on the vector ALU: two
    # workgroups per CU, each taking two kv heads: 253 partitions x 2
    assert lib.pa_choose_partition_size(1, 1, 24, 4, 256, 3, 250000) == 992
    assert lib.pa_choose_partition_size(1, 1, 24, 4, 256, 4, 250000) == 992
    # int8 with G = 4 stays on the vector ALU
    assert lib.pa_choose_partition_size(1, 1, 16, 4, 256, 2, 250000) == 992
    assert lib.pa_choose_partition_size(4, 8, 24, 4, 256, 3, 30321) == 960
    # small head chunks (batched GQA, D=128, 4 heads): eight per CU aimed at,
    # and half the usual minimum partition
    assert lib.pa_choose_partition_size(8, 1, 32, 8, 128, 1, 3637) == 128
    # speculative verify on the matrix cores: two per CU
    assert lib.pa_choose_partition_size(4, 8, 24, 4, 256, 1, 30321) == 960
    # the same shape with fp32 caches uses one-wave workgroups, eight per CU
    assert lib.pa_choose_partition_size(4, 1, 24, 4, 256, 0, 65536) == 512
    # one partition covers a short context: no workspace
    assert lib.pa_choose_partition_size(1, 1, 24, 4, 256, 1, 48) == 48
    assert lib.pa_decode_workspace_bytes(1, 1, 24, 4, 256, 1, 48, 0) == 0
    # (vector ALU, two waves per kv head: at least 4 blocks each)
    assert lib.pa_choose_partition_size(1, 1, 16, 4, 256, 2, 200) == 128
    # (streaming kernel: at least 4 blocks per wave; int8 one wave per head,
    # FP8 two)
    assert lib.pa_choose_partition_size(1, 1, 24, 4, 256, 2, 200) == 64
    assert lib.pa_choose_partition_size(1, 1, 24, 4, 256, 3, 200) == 128
    # fp32 caches (one-wave workgroups) split even short contexts into blocks
    assert lib.pa_choose_partition_size(1, 1, 4, 1, 64, 0, 256) == 16
    assert lib.pa_decode_workspace_bytes(1, 1, 4, 1, 64, 0, 256, 0) == 4 * 16 * 64 * 4 + 256
    # partitions are multiples of 16 and never longer than needed
    for L in (1, 17, 300, 5000, 250000):
        P = lib.pa_choose_partition_size(1, 1, 24, 4, 256, 2, L)
        assert P % 16 == 0 and P >= 16
    assert lib.pa_choose_partition_size(1, 1, 7, 2, 64, 0, 100) == -2
    # the workspace test above passes once enough bytes are given (no launch: B == 0)
    rc = lib.pa_decode(*decode_args(B=0, partition_size=256, workspace=A, workspace_bytes=1 << 30))
    assert rc == 0 and NP.value == 4


@pytest.mark.parametrize("over, code", [
    (dict(src_dtype=2), -3),
    (dict(cache_dtype=5), -3),
    (dict(D=48), -4),
    (dict(block_size=8), -4),
    (dict(k_cache=None), -1),
    (dict(cache_dtype=2), -1),
    (dict(cache_dtype=3), -1),  # fp8 without scales
    (dict(cache_dtype=4), -1),  # nvfp4 without scales
    (dict(num_tokens=-1), -2),
    (dict(k_src=ctypes.c_void_p(0x1008)), -7),
])
def test_cache_write_rejects_bad_arguments(lib, over, code):
    args = dict(k_src=A, v_src=A, src_dtype=0, slots=A, num_tokens=5, k_cache=A, v_cache=A, cache_dtype=1,
                k_scale=None, v_scale=None, num_blocks=4, block_size=16, Hkv=2, D=128, stream=None)
    args.update(over)
    rc = lib.pa_cache_write(*args.values())
    assert rc == code, lib.pa_last_error()


def test_cache_write_of_no_tokens_is_a_no_op(lib):
    rc = lib.pa_cache_write(None, None, 0, None, 0, A, A, 1, None, None, 4, 16, 2, 128, None)
    assert rc == 0


def test_reduce_rejects_bad_arguments(lib):
    assert lib.pa_decode_splitk_reduce(None, 4, 512, 1, 1, 8, 128, A, A, 0, None, None) == -1
    assert lib.pa_decode_splitk_reduce(A, 0, 512, 1, 1, 8, 128, A, A, 0, None, None) == -2
    assert lib.pa_decode_splitk_reduce(A, 4, 100, 1, 1, 8, 128, A, A, 0, None, None) == -2
    assert lib.pa_decode_splitk_reduce(A, 4, 512, 1, 1, 8, 100, A, A, 0, None, None) == -4
    odd = ctypes.c_void_p(0x1008)
    assert lib.pa_decode_splitk_reduce(odd, 4, 512, 1, 1, 8, 128, A, A, 0, None, None) == -7
    assert lib.pa_decode_splitk_reduce(A, 4, 512, 1, 1, 8, 128, A, odd, 0, None, None) == -7


def test_checks_reject_bad_arguments(lib):
    assert lib.pa_decode_check(None, 4, A, 2, 64, 16, A, None) == -1
    assert lib.pa_decode_check(A, 4, A, 2, 64, 16, None, None) == -1
    assert lib.pa_decode_check(A, 0, A, 2, 64, 16, A, None) == -2
    assert lib.pa_decode_check(A, 4, A, -1, 64, 16, A, None) == -2
    assert lib.pa_cache_write_check(A, 5, 4, 16, None, None) == -1
    assert lib.pa_cache_write_check(A, -1, 4, 16, A, None) == -2
    assert lib.pa_cache_write_check(A, 5, 0, 16, A, None) == -2


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(pa, "_LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(pa, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        pa.load()


def shared_args(**over):
    args = dict(q=A, q_dtype=1, B=4, Tq=8, Hq=24, Hkv=4, D=256, k_cache=A, v_cache=A, kv_dtype=1, k_scale=None,
                v_scale=None, num_blocks=4096, block_size=16, prefix_table=A, prefix_len=4096, block_table=A,
                max_blocks=1896, seq_lens=A, max_seq_len=30321, scale=0.0625, prefix_partition=0, tail_partition=0,
                out=A, out_dtype=0, lse=None, workspace=None, workspace_bytes=0, stream=None)
    args.update(over)
    return list(args.values())


@pytest.mark.parametrize("over, code", [
    (dict(q=None), -1),
    (dict(prefix_table=None), -1),
    (dict(kv_dtype=0), -4),  # fp32 caches: no matrix-core prefix pass
    (dict(kv_dtype=2), -1),  # int8 without scales
    (dict(prefix_len=4008), -2),  # not whole blocks
    (dict(prefix_len=-16), -2),
    (dict(prefix_len=30320), -2),  # no room for 8 query tokens
    (dict(prefix_partition=100), -2),
    (dict(tail_partition=-16), -2),
    (dict(Tq=17), -4),
    (dict(max_blocks=100), -2),
    (dict(workspace=ctypes.c_void_p(0x1008), workspace_bytes=1 << 30), -7),
    (dict(), -5),  # partials of both passes need a workspace
])
def test_shared_prefix_rejects_bad_arguments(lib, over, code):
    rc = lib.pa_decode_shared_prefix(*shared_args(**over))
    assert rc == code, lib.pa_last_error()
    assert lib.pa_last_error()


def test_shared_prefix_plan_and_workspace(lib):
    # the speculative-verify workload: the prefix pass takes the 4 * 8 * 6 =
    # 192 rows of a kv head in 3 chunks of 64, so 12 workgroups per partition;
    # 512 workgroups would want 43 partitions, 96 tokens each: the minimum of
    # 256 gives 16. The tail pass (26225 tokens at most) is a plain decode:
    # 32 partitions of 832 tokens (4 sequences x 4 kv heads x 32 = 512).
    rows = 4 * 8 * 24
    need = lib.pa_decode_shared_prefix_workspace_bytes(4, 8, 24, 4, 256, 1, 30321, 4096, 0, 0)
    assert need == rows * 48 * 256 * 4 + rows * 48 * 4
    assert lib.pa_choose_partition_size(4, 8, 24, 4, 256, 1, 30321 - 4096) == 832
    # given sizes: 4096 / 1024 + ceil(26225 / 512) = 4 + 52 partitions
    need = lib.pa_decode_shared_prefix_workspace_bytes(4, 8, 24, 4, 256, 1, 30321, 4096, 1024, 512)
    assert need == rows * 56 * 256 * 4 + rows * 56 * 4
    # no prefix and one tail partition: out is written directly, no workspace
    assert lib.pa_decode_shared_prefix_workspace_bytes(1, 1, 24, 4, 256, 1, 48, 0, 0, 0) == 0
    # invalid arguments size nothing
    assert lib.pa_decode_shared_prefix_workspace_bytes(4, 8, 24, 4, 256, 1, 30321, 4008, 0, 0) == 0
    # B == 0 with enough workspace: accepted, nothing launched
    rc = lib.pa_decode_shared_prefix(*shared_args(B=0, workspace=A, workspace_bytes=1 << 30))
    assert rc == 0, lib.pa_last_error()


def test_empty_batch_with_the_heuristic(lib):
    # B = 0 sizes no workgroups: the heuristic must not divide by them
    for kv in (0, 1, 2):
        assert lib.pa_choose_partition_size(0, 1, 24, 4, 256, kv, 65536) > 0
        assert lib.pa_choose_partition_size(0, 8, 24, 4, 256, kv, 65536) > 0
    rc = lib.pa_decode(*decode_args(B=0, partition_size=0, workspace=A, workspace_bytes=1 << 30))
    assert rc == 0, lib.pa_last_error()


def test_decode_rejects_a_misaligned_workspace_before_launching(lib):
    # several partitions: the reduce that must follow reads 16-byte vectors,
    # so the decode refuses the workspace before any launch
    rc = lib.pa_decode(*decode_args(partition_size=256, workspace=ctypes.c_void_p(0x1008),
                                    workspace_bytes=1 << 30))
    assert rc == -7, lib.pa_last_error()
    # one partition needs no workspace, aligned or not (B = 0: nothing launched)
    rc = lib.pa_decode(*decode_args(B=0, partition_size=1008, workspace=ctypes.c_void_p(0x1008),
                                    workspace_bytes=1 << 30))
    assert rc == 0, lib.pa_last_error()


def test_heuristic_follows_the_device_compute_units(lib):
    # no device on this host: the MI355X count, and the plain heuristic equals
    # the injected one at 256 CUs
    assert lib.pa_device_cu_count() == 256
    for args in ((4, 1, 24, 4, 256, 1, 65536), (1, 1, 24, 4, 256, 2, 250000), (4, 8, 24, 4, 256, 1, 30321),
                 (8, 1, 32, 8, 128, 1, 3637)):
        assert lib.pa_choose_partition_size_for_cus(*args, 256) == lib.pa_choose_partition_size(*args)
    # the 64K workload fills one four-wave workgroup per CU: 4 sequences need
    # 64 partitions on 256 CUs, 32 on 128 (a partitioned GPU), 76 on 304
    assert lib.pa_choose_partition_size_for_cus(4, 1, 24, 4, 256, 1, 65536, 256) == 1024
    assert lib.pa_choose_partition_size_for_cus(4, 1, 24, 4, 256, 1, 65536, 128) == 2048
    assert lib.pa_choose_partition_size_for_cus(4, 1, 24, 4, 256, 1, 65536, 304) == 864
    assert lib.pa_choose_partition_size_for_cus(4, 1, 24, 4, 256, 1, 65536, 32) == 8192
    # int8 250K on the streaming kernel (one workgroup of all 4 kv heads per
    # CU, one wave per head): 64 CUs take 64 partitions of ceil(250000 / 64)
    # tokens rounded up to whole blocks; 16 CUs would want 15632, above the
    # 4096-token cap (256 blocks per wave); FP8 (two waves per head) rounds to
    # 32 tokens and is capped at 8192
    assert lib.pa_choose_partition_size_for_cus(1, 1, 24, 4, 256, 2, 250000, 64) == 3920
    assert lib.pa_choose_partition_size_for_cus(1, 1, 24, 4, 256, 2, 250000, 16) == 4096
    assert lib.pa_choose_partition_size_for_cus(1, 1, 24, 4, 256, 3, 250000, 64) == 3936
    assert lib.pa_choose_partition_size_for_cus(1, 1, 24, 4, 256, 3, 250000, 16) == 8192
    assert lib.pa_choose_partition_size_for_cus(4, 1, 24, 4, 256, 1, 65536, 0) == -2


def test_kernel_name_query(lib):
    assert lib.pa_decode_kernel_name(1, 24, 4, 1) == b"decode_wave_kernel"   # bf16, G = 6
    assert lib.pa_decode_kernel_name(1, 24, 4, 2) == b"decode_stream_kernel"  # int8, G = 6: one row tile
    assert lib.pa_decode_kernel_name(1, 24, 4, 3) == b"decode_stream_kernel"  # fp8, G = 6
    assert lib.pa_decode_kernel_name(2, 16, 2, 2) == b"decode_stream_kernel"  # int8, 2 x 8 rows
    assert lib.pa_decode_kernel_name(8, 24, 4, 2) == b"decode_mfma_kernel"    # int8, 48 rows
    assert lib.pa_decode_kernel_name(1, 16, 4, 2) == b"decode_wave_kernel"   # int8, G = 4
    assert lib.pa_decode_kernel_name(8, 24, 4, 1) == b"decode_mfma_kernel"   # Tq > 1
    assert lib.pa_decode_kernel_name(1, 64, 4, 1) == b"decode_mfma_kernel"   # G = 16
    assert lib.pa_decode_kernel_name(1, 24, 4, 4) == b"decode_stream_kernel"  # nvfp4, G = 6
    assert lib.pa_decode_kernel_name(1, 16, 4, 4) == b"decode_wave_kernel"   # nvfp4, G = 4
    assert lib.pa_decode_kernel_name(8, 24, 4, 4) == b"decode_mfma_kernel"   # nvfp4, 48 rows
    assert lib.pa_decode_kernel_name(2, 4, 1, 0) == b"decode_valu_kernel"    # fp32 caches
    assert lib.pa_decode_kernel_name(1, 7, 2, 1) == b""


def test_noalloc_rejects_partials_beyond_its_scratch(lib):
    # 64 x 16 x 64 rows x 64 partitions x 1 KiB of partials: far above the
    # 32 MiB library scratch, refused before any device is touched
    args = decode_args(B=64, Tq=16, Hq=64, Hkv=4, D=256, max_seq_len=65536, max_blocks=4096, partition_size=1024)
    args = args[:23] + [None]  # pa_decode_noalloc: no workspace, size or partition count; then the stream
    rc = lib.pa_decode_noalloc(*args)
    assert rc == -5, lib.pa_last_error()
    assert b"scratch" in lib.pa_last_error()
    assert pa.NOALLOC_SCRATCH_BYTES == 32 << 20
    text = open(HEADER).read()
    assert "#define PA_NOALLOC_SCRATCH_BYTES (32u << 20)" in text


def sparse_args(**over):
    args = dict(q=A, q_dtype=1, B=1, Tq=1, Hq=24, Hkv=4, D=256, k_cache=A, v_cache=A, kv_dtype=2, k_scale=A,
                v_scale=A, num_blocks=16000, block_size=16, block_table=A, max_blocks=15625, seq_lens=A,
                max_seq_len=250000, scale=0.0625, mean_k=A, max_sblocks=3907, sparse_block=64, top_blocks=512,
                partition_size=0, out=A, out_dtype=0, lse=None, selected=None, workspace=None, workspace_bytes=0,
                stream=None)
    args.update(over)
    return list(args.values())


@pytest.mark.parametrize("over, code", [
    (dict(mean_k=None, workspace=A, workspace_bytes=1 << 30), -1),
    (dict(kv_dtype=0, k_scale=None, v_scale=None), -4),          # fp32 caches
    (dict(sparse_block=40), -2),                                  # not whole cache blocks
    (dict(sparse_block=8192), -2),
    (dict(top_blocks=0), -2),
    (dict(max_sblocks=3906, workspace=A, workspace_bytes=1 << 30), -2),
    (dict(sparse_block=16), -4),                                  # 15625 blocks > 4096
    (dict(), -5),                                                 # no workspace
    (dict(workspace=ctypes.c_void_p(0x1008), workspace_bytes=1 << 30), -7),
])
def test_sparse_decode_rejects_bad_arguments(lib, over, code):
    rc = lib.pa_decode_sparse(*sparse_args(**over))
    assert rc == code, lib.pa_last_error()
    assert lib.pa_last_error()


def test_sparse_workspace_plan(lib):
    # int8 250K, 64-token sparse blocks, 512 selected: scores of 3907 blocks
    # for 4 kv heads, compacted tables of 512 * 4 cache blocks, lengths, and
    # the partials over at most 32768 selected keys
    n = lib.pa_decode_sparse_workspace_bytes(1, 1, 24, 4, 256, 2, 250000, 64, 512, 0)
    P = lib.pa_choose_partition_size(1, 1, 24, 4, 256, 2, 32768)
    al = lambda x: (x + 255) // 256 * 256
    # (the per-head tables give one kv head per workgroup, so the heuristic
    # splits finer than pa_choose_partition_size for the same length)
    parts = n - (al(4 * 3907 * 4) + al(4 * 2048 * 4) + al(4 * 4))
    assert parts > 0 and parts % 256 == 0
    rows = 24
    np_ = None
    for Pc in range(16, 32769, 16):
        k = (32768 + Pc - 1) // Pc
        if al(rows * k * 256 * 4) + al(rows * k * 4) == parts:
            np_ = k
            break
    assert np_ is not None and np_ > 1
    # every block selected: at most the 4096 blocks of max_seq_len
    assert lib.pa_decode_sparse_workspace_bytes(1, 1, 24, 4, 256, 2, 1000, 64, 100, 1024) == \
        al(4 * 16 * 4) + al(4 * 64 * 4) + al(4 * 4)
    assert lib.pa_decode_sparse_workspace_bytes(1, 1, 24, 4, 256, 0, 1000, 64, 100, 0) == 0  # fp32: invalid


def test_sparse_mean_keys_rejects_bad_arguments(lib):
    args = dict(k_cache=A, kv_dtype=2, k_scale=A, num_blocks=64, block_size=16, Hkv=2, D=128, block_table=A,
                max_blocks=64, seq_lens=A, B=2, max_seq_len=1000, sparse_block=64, num_new=1, mean_k=A,
                max_sblocks=16, stream=None)

    def call(**over):
        a = dict(args)
        a.update(over)
        return lib.pa_sparse_mean_keys(*a.values())

    assert call(k_scale=None) == -1
    assert call(mean_k=None) == -1
    assert call(max_sblocks=15) == -2
    assert call(num_new=0) == -2
    assert call(sparse_block=24) == -2
    assert call(D=96) == -4
    assert call(B=0) == 0  # nothing to do, nothing launched


def test_prepared_call_marshalling(lib):
    # arguments converted once to the entry point's ctypes types; the
    # trailing stream stays for the call
    import ctypes

    import paged_attention_decode_02_amd as pa

    pa.load()
    out_np = ctypes.c_int32(0)
    fn, args = pa._marshal(pa.load().pa_decode, (0x1000, 1, 2, 1, 8, 2, 128, 0x2000, 0x3000, 1, None, None, 64, 16,
                                                 0x4000, 8, 0x5000, 100, 0.125, 0, 0x6000, 0, None, None, 0,
                                                 ctypes.byref(out_np)))
    assert fn is pa.load().pa_decode and len(args) == len(fn.argtypes) - 1
    assert isinstance(args[0], ctypes.c_void_p) and args[0].value == 0x1000
    assert isinstance(args[2], ctypes.c_int32) and args[2].value == 2
    assert isinstance(args[10], ctypes.c_void_p) and args[10].value is None
    assert isinstance(args[12], ctypes.c_int64) and args[12].value == 64
    assert isinstance(args[18], ctypes.c_float) and args[18].value == 0.125
    assert isinstance(args[24], ctypes.c_size_t)
    assert isinstance(args[25], pa._CARG)


@pytest.mark.parametrize("args, code", [
    ((A, 4096, None, 8), -1),                         # no sink
    ((None, 4096, A, 8), -1),                         # no buffer to read
    ((A, 4100, A, 8), -2),                            # not whole 16-byte chunks
    ((A, 4096, A, 0), -2),                            # no workgroup
    ((A, 4096, A, 65536), -2),
    ((ctypes.c_void_p(0x1008), 4096, A, 8), -7),      # misaligned buffer
])
def test_read_probe_rejects_bad_arguments(lib, args, code):
    rc = lib.pa_read_probe(*args, None)
    assert rc == code, lib.pa_last_error()
    assert lib.pa_last_error()
