// Host <-> device parameter blocks and internal launcher declarations.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

struct DecodeParams {
    const void* q;
    int q_bf16;  // 0: fp32 queries, 1: bf16 queries
    int B, Tq, Hq, Hkv, G;
    const void* k_cache;
    const void* v_cache;
    const float* k_scale;
    const float* v_scale;
    const int32_t* block_table;
    int max_blocks;
    const int32_t* seq_lens;
    float qk_scale_log2;  // softmax_scale * log2(e)
    int P;                // partition size in tokens (multiple of 16)
    int NP;               // partitions per row
    int nchunk;           // vector-ALU kernels: head chunks of GT; MFMA kernel: row chunks of 16*NT
    int hpg;              // bf16/int8 vector-ALU kernel: kv heads per workgroup (1, 2 or 4, divides Hkv)
    void* out;
    int out_bf16;
    float* lse;
    float* ws_o;    // [B, Tq, Hq, np_stride, D] when np_stride > 1
    float* ws_lse;  // [B, Tq, Hq, np_stride]
    // Partials of several launches may share one workspace: this launch's
    // partition i is workspace partition part_base + i of np_stride per row.
    // np_stride == 1: one partition covers the row, out/lse are written.
    int np_stride;
    int part_base;
    int fill_empty;  // partitions with no visible key still write lse = -inf
    int kv_begin;    // keys start at this token of every sequence (a multiple of 16)
    // MFMA kernel only: the Tq * G rows of all B sequences form one row set
    // that attends to keys 0 .. prefix_len - 1 of the block list block_table
    int stacked;
    int prefix_len;
    // Per-head block tables: row b * Hkv + g of block_table and seq_lens
    // belongs to kv head g of sequence b (the sparse decode's compacted
    // tables); one kv head per workgroup.
    int head_tables;
};

struct ReduceParams {
    const float* ws_o;
    const float* ws_lse;
    int NP, P, B, Tq, Hq, D;
    int cs;  // column splits: workgroups per row, each taking D / cs output elements
    int all_parts;  // every partition was written (empty ones with lse = -inf): merge all NP
    int Hkv;        // with head_lens: seq_lens[b * Hkv + kv head] is the length of the row's kv head
    int head_lens;
    const int32_t* seq_lens;
    void* out;
    int out_bf16;
    float* lse;
};

// Sparse block-selection decode: mean keys, scores, selection, compacted tables.
struct SparseParams {
    const void* q;
    int q_bf16;
    int B, Tq, Hq, Hkv, D;
    const void* k_cache;
    const float* k_scale;
    const int32_t* block_table;
    int max_blocks;
    const int32_t* seq_lens;
    float softmax_scale;
    int sparse_block;  // tokens per sparse block (a multiple of 16)
    int top_blocks;    // sparse blocks selected per (sequence, kv head), the kept ones included
    int num_new;       // mean keys: refresh the blocks holding each sequence's last num_new tokens
    float* mean_k;     // [B, max_sblocks, Hkv, D]
    int max_sblocks;
    float* scores;     // [B * Hkv, nsb_max] candidate scores
    int nsb_max;       // sparse blocks of the longest sequence
    int max_sel;       // selected blocks per (sequence, kv head) at most
    int32_t* sel_out;  // optional [B, Hkv, max_sel] selected blocks, increasing, -1 after
    int32_t* ctab;     // [B * Hkv, ctab_width] compacted block tables
    int ctab_width;    // max_sel * sparse_block / 16
    int32_t* clen;     // [B * Hkv] compacted lengths
};

struct CacheWriteParams {
    const void* k_src;
    const void* v_src;
    int src_bf16;
    const int64_t* slots;
    int64_t num_tokens;
    void* k_cache;
    void* v_cache;
    float* k_scale;
    float* v_scale;
    int Hkv, D;
};

struct DecodeCheckParams {
    const int32_t* block_table;
    int max_blocks;
    const int32_t* seq_lens;
    int B;
    int max_seq_len;
    int64_t num_blocks;
    int32_t* status;  // [2]: violations, flat index of the first one (-1: none)
};

struct SlotsCheckParams {
    const int64_t* slots;
    int64_t num_tokens;
    int64_t num_slots;  // num_blocks * block_size
    int32_t* status;
};

// Launchers return hipSuccess or the launch error.
hipError_t launch_decode_valu(int kv_type, int D, int GT, const DecodeParams& p, hipStream_t stream);
hipError_t launch_decode_wave(int kv_type, int D, int GT, const DecodeParams& p, hipStream_t stream);
// NT: 16-row tiles per workgroup (1..4); p.nchunk = row chunks of 16*NT rows
hipError_t launch_decode_mfma(int kv_type, int D, int NT, const DecodeParams& p, hipStream_t stream);
// one tile of G * Tq <= 16 rows on the matrix cores, each wave streaming its
// own blocks; p.hpg kv heads per workgroup (1, 2 or 4) of stream_waves waves
// (a head's waves share its blocks); partitions of at most
// kStreamMaxPartition * (waves per head) tokens.
// Waves per workgroup and LDS stages per wave (the block being computed and
// those in flight), one workgroup per CU, measured at 250K tokens: int8, four
// waves (one per SIMD) with three stages each (85.6 us; eight waves with two
// stages: 92.1); FP8, whose key widening is heavier, eight waves with two
// stages (91.0 us; four waves with three: 104.9), the second wave on a SIMD
// hiding the first's latencies; NVFP4 (keys and values widened with their
// block scales) likewise eight waves with two stages (90.9 us; four waves
// with three: 117.3, with two: 128.5). bf16 with D = 256 (16 KB per stage)
// fits four waves with two stages.
constexpr int stream_waves(int kv_type, int D) { return kv_type == 3 || kv_type == 4 ? 8 : 4; }
constexpr int stream_stages(int kv_type, int D) { return kv_type == 2 ? 3 : 2; }
constexpr int kStreamMaxPartition = 4096;
hipError_t launch_decode_stream(int kv_type, int D, const DecodeParams& p, hipStream_t stream);
hipError_t launch_splitk_reduce(const ReduceParams& p, hipStream_t stream);
hipError_t launch_cache_write(int cache_type, const CacheWriteParams& p, hipStream_t stream);
hipError_t launch_decode_check(const DecodeCheckParams& p, hipStream_t stream);
hipError_t launch_slots_check(const SlotsCheckParams& p, hipStream_t stream);

hipError_t launch_sparse_mean(int kv_type, const SparseParams& p, int nref, hipStream_t stream);
// scores of the candidate blocks, then the selection and compacted tables
hipError_t launch_sparse_select(const SparseParams& p, hipStream_t stream);
constexpr int kSparseMaxBlocks = 4096;  // sparse blocks per sequence at most
constexpr int kSparseMaxBlockTokens = 4096;  // tokens per sparse block at most

// Read-bandwidth probe (every 16-byte chunk of buf once, per-workgroup word sums into sink).
hipError_t launch_read_probe(const void* buf, int64_t bytes, uint32_t* sink, int workgroups, hipStream_t stream);

// Valid head-chunk widths of the VALU decode instances.
bool decode_valu_has_gt(int GT);

}  // namespace pa
