"""The seeded input generator: draw order, table validity, sharing, slots (CPU)."""
import numpy as np
import pytest

from workloads import BLOCK_SIZE, SPECS, bf16_bits, bf16_bits_to_f32, generate, kv_bytes_per_token, scaled


def test_seed0_lengths():
    # seed-0 draws of rng.integers(lo, hi + 1, size=B) with numpy's default generator
    assert generate("gqa_bf16").seq_lens.tolist() == [3637, 2981, 2594, 1853, 1969, 1149, 1255, 1074]
    w = generate(scaled("verify_bf16", D=8, Hq=2, Hkv=1))
    assert w.seq_lens.tolist() == [30321, 26820, 24758, 20804]


def test_tiny_pool_and_table():
    w = generate("tiny_f32")
    assert w.num_blocks == 64 and w.block_table.shape == (1, 16)
    assert len(set(w.block_table[0].tolist())) == 16
    assert w.unused_slots().size == 48 * BLOCK_SIZE
    assert w.q.dtype == np.float32 and w.q_bits is None and w.k_src.dtype == np.float32


@pytest.mark.parametrize("name", ["gqa_bf16", "verify_bf16"])
def test_tables_slots_and_sharing(name):
    spec = SPECS[name] if name == "gqa_bf16" else scaled(name, D=8, Hq=2, Hkv=1, seq_lens=(4200, 5000))
    w = generate(spec)
    bs = BLOCK_SIZE
    nblk = (w.seq_lens + bs - 1) // bs
    shared = spec.shared_prefix // bs
    seen = {}
    for b in range(spec.B):
        row = w.block_table[b, : nblk[b]]
        assert row.min() >= 0 and row.max() < w.num_blocks
        for j, blk in enumerate(row.tolist()):
            if j < shared:
                assert blk == w.block_table[0, j]
            else:
                assert blk not in seen, "private blocks must not be shared"
                seen[blk] = b
        # past-the-end entries point at slack blocks
        assert set(w.block_table[b, nblk[b]:].tolist()) <= set(w.slack_blocks.tolist())
    assert len(w.slack_blocks) == 64
    # every source row sits at its sequence's block for its position; slots are distinct
    for i in range(0, w.slot_mapping.shape[0], 97):
        b = w.row_seq[i] if w.row_seq[i] >= 0 else 0
        pos = int(w.row_pos[i])
        assert w.slot_mapping[i] == int(w.block_table[b, pos // bs]) * bs + pos % bs
    assert np.unique(w.slot_mapping).size == w.slot_mapping.size
    assert w.slot_mapping.size == spec.shared_prefix + int((w.seq_lens - spec.shared_prefix).sum())


def test_bf16_sources_and_queries():
    w = generate(scaled("gqa_bf16", B=2, Hq=4, Hkv=2, D=16, seq_lens=(40, 90)))
    assert w.k_src.dtype == np.uint16 and w.q_bits is not None
    assert np.array_equal(bf16_bits(w.q), w.q_bits)  # q holds exactly the bf16 values


def test_peaked_keys_fraction():
    spec = scaled("long64k_bf16", B=2, Hq=2, Hkv=1, D=64, seq_lens=(20000, 20000))
    w = generate(spec)
    k = bf16_bits_to_f32(w.k_src).reshape(w.k_src.shape)
    rms = np.sqrt((k.astype(np.float64) ** 2).mean(axis=(1, 2)))
    assert (rms > 4).sum() == 2 * 200  # round(0.01 * 20000) per sequence, scaled x8


def test_step_rows_are_last_tokens():
    w = generate(scaled("verify_bf16", D=8, Hq=2, Hkv=1, seq_lens=(4200, 5000)))
    rows = w.step_rows()
    assert rows.size == w.spec.B * w.spec.Tq
    for b in range(w.spec.B):
        got = sorted(w.row_pos[rows[w.row_seq[rows] == b]].tolist())
        L = int(w.seq_lens[b])
        assert got == list(range(L - w.spec.Tq, L))


def test_bytes_per_token():
    assert kv_bytes_per_token(SPECS["long64k_bf16"]) == 4096
    assert kv_bytes_per_token(SPECS["int8_250k"]) == 2080
    assert kv_bytes_per_token(SPECS["gqa_bf16"]) == 4096
    assert kv_bytes_per_token(SPECS["tiny_f32"]) == 512
