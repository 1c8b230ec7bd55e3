/*
 * pa_decode.h — C ABI of the MI355X (gfx950) paged-attention decode library.
 *
 * The operation is PagedAttention decode: each sequence's new query tokens
 * attend to that sequence's keys and values, which sit in fixed-size blocks
 * of a shared pool reached through a per-sequence block table (nvllm page,
 * "About", the PagedAttention citation; 1Cat-vLLM docs index, feature list).
 * The decode is split along the context ("split-K paged decode with an int8
 * KV cache", vllm-sm70 page, "Why", Attention bullet) and the partitions are
 * merged by their log-sum-exp ("split-KV merge", nvllm page,
 * "Acknowledgments", b12x). Several query tokens per sequence (speculative
 * verification, 8 target tokens per step: vllm-sm12x-nvfp4-dflash2 page,
 * "What makes this stack different") are a causal "virtual batch": query
 * token t of Tq sees keys 0 .. L_b - Tq + t.
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers unless marked (host). Every buffer belongs
 *    to the caller; the library never allocates or frees device memory,
 *    never synchronises, never reads device data on the host, and launches
 *    only on `stream` (a hipStream_t; NULL = the null stream). The calls are
 *    therefore safe to record in a HIP graph (the vLLM-fork pages run decode
 *    under full graph capture and keep graph-held buffers at fixed addresses:
 *    nvllm "Roadmap", vllm-sm70 "Changes relative to 1Cat-vLLM").
 *  - Return 0 on success or a negative PA_ERR_* code; nothing is thrown
 *    across the ABI. pa_last_error() gives a message for the calling thread's
 *    last failure. Arguments are checked on the host before any launch, so a
 *    rejected call has no effect. Device-side contracts (valid block ids,
 *    0 <= seq_lens[b] <= max_seq_len, distinct slots) are trusted; breaking
 *    them is undefined behaviour (an out-of-range block id reads out of
 *    bounds). Asynchronous device faults appear at the caller's next sync.
 *  - Layouts are dense row-major with the innermost dimension last:
 *      q        [B, Tq, Hq, D]
 *      caches   [num_blocks, block_size, Hkv, D]   (K and V separately)
 *      scales   [num_blocks, Hkv, block_size]      fp32, int8 / FP8 / NVFP4 caches only;
 *                                                  a kv head's scales of one block are one
 *                                                  64-byte run, read whole by its workgroup
 *                                                  (head-major inside a block, not token-major
 *                                                  [num_blocks, block_size, Hkv]: a token-major
 *                                                  64-byte line holds four tokens of every kv
 *                                                  head and was fetched by every head's
 *                                                  workgroup)
 *      table    [B, max_blocks_per_seq]            int32 physical block ids
 *      out      [B, Tq, Hq, D]
 *      lse      [B, Tq, Hq]                        fp32, natural log
 *    Query head h reads kv head h / (Hq / Hkv).
 *  - Supported: block_size 16; D in {64, 128, 256}; 1 <= Tq <= 16;
 *    Hq % Hkv == 0 and Hq / Hkv <= 64; q in {f32, bf16}; caches in
 *    {f32, bf16, i8, fp8, nvfp4} (the shared-prefix decode: not f32); out
 *    in {f32, bf16}. q, caches and out must be 16-byte aligned; one KV block
 *    (16 * Hkv * row bytes) must be below 2^31 bytes.
 *  - NVFP4 caches are bytes [num_blocks, block_size, Hkv, 9 D / 16] (row
 *    bytes 36, 72, 144 for D = 64, 128, 256), but a block is not stored row
 *    by row: first the code rows of its 16 * Hkv (token, head) pairs, D/2
 *    bytes each in (token, head) order, element 2i in the low nibble of
 *    byte i; then one plane of D bytes per kv head h (at 8 Hkv D + h D in
 *    the block) with that head's E4M3 block scales, the scale of elements
 *    16k .. 16k + 15 of token 4q + r at byte 16k + 4r + q of the plane.
 *    Code rows are 64-byte aligned for D >= 128 and a head's block scales are
 *    one contiguous run, so HBM fetches are never shared between rows.
 */
#ifndef PA_DECODE_H
#define PA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* PA_FP8: OCP FP8 E4M3 codes (sign, 4 exponent bits biased by 7, 3 mantissa
 * bits, no infinities, largest finite 448), the FP8 KV cache of the nvllm
 * page ("Acknowledgments", b12x: FP8 KV dequantised inline). */
/* PA_NVFP4: NVFP4 (the KV format of the vllm-sm12x-nvfp4-dflash2 page,
 * "What makes this stack different"): FP4 E2M1 codes (magnitudes 0, 0.5, 1,
 * 1.5, 2, 3, 4, 6) with an E4M3 scale per 16 elements and an fp32 scale per
 * (token, kv head). */
typedef enum { PA_F32 = 0, PA_BF16 = 1, PA_I8 = 2, PA_FP8 = 3, PA_NVFP4 = 4 } pa_dtype;

enum {
    PA_OK = 0,
    PA_ERR_NULL = -1,        /* a required pointer is NULL */
    PA_ERR_SHAPE = -2,       /* a size is out of range or inconsistent */
    PA_ERR_DTYPE = -3,       /* a dtype or dtype combination is not supported */
    PA_ERR_UNSUPPORTED = -4, /* a valid but unimplemented shape (D, block_size, Tq, group) */
    PA_ERR_WORKSPACE = -5,   /* workspace missing or smaller than pa_decode_workspace_bytes */
    PA_ERR_LAUNCH = -6,      /* the HIP launch itself failed */
    PA_ERR_ALIGN = -7        /* a pointer is not 16-byte aligned */
};

/*
 * pa_cache_write — store new tokens' key/value rows into the paged caches.
 *
 * Defines the cache contents every decode reads (the block pool of
 * PagedAttention; the int8 KV cache of the vllm-sm70 page, "Why"). For each
 * token i < num_tokens with slot = slot_mapping[i] >= 0 and each kv head g,
 * row src[i, g, :] goes to cache row (slot / block_size, slot % block_size,
 * g). A negative slot skips the token: padded rows must not write into other
 * requests' slots (vllm-sm70 page, "Known limitations", fixed defects).
 *   k_src, v_src   [num_tokens, Hkv, D] in src_dtype (f32 or bf16)
 *   slot_mapping   [num_tokens] int64, slot = block * block_size + offset
 *   k_cache, v_cache  caches in cache_dtype; k_scale, v_scale required iff
 *                  cache_dtype is PA_I8, PA_FP8 or PA_NVFP4 (else pass NULL)
 * Conversions: same dtype copies bits; bf16 -> f32 widens exactly;
 * f32 -> bf16 rounds to nearest even; -> i8 is symmetric per (token, kv
 * head): s = fp32(max|x| / 127), code = clamp(rint_even(fp32(x / s)), -127,
 * 127); -> fp8 likewise against 448: s = fp32(max|x| / 448), code = the
 * E4M3 value nearest to fp32(x / s), ties to the even code, saturating at
 * +-448, the sign bit that of the quotient; -> nvfp4: S = fp32(max|x| / 2688)
 * (the row's fp32 scale), per 16-element block u = fp32(fp32(max|x_b| / 6) /
 * S), block scale = the E4M3 code of u (as for fp8), d = fp32(value * S), code
 * = the E2M1 value nearest to fp32(x / d), ties to the even code, saturating
 * at +-6, 0 where d = 0; for all three, an all-zero row gives scale 0 and all
 * codes 0. Bit-exact. Source values must be finite.
 * Slots must lie in [0, num_blocks * block_size) and be distinct within one
 * call. num_tokens == 0 is a no-op.
 */
int pa_cache_write(const void* k_src, const void* v_src, pa_dtype src_dtype, const int64_t* slot_mapping,
                   int64_t num_tokens, void* k_cache, void* v_cache, pa_dtype cache_dtype, float* k_scale,
                   float* v_scale, int64_t num_blocks, int32_t block_size, int32_t Hkv, int32_t D, void* stream);

/*
 * pa_decode — paged attention of B sequences' Tq query tokens.
 *
 * For every b, t, h with n = seq_lens[b] - Tq + t + 1 visible keys:
 *   out[b,t,h,:] = sum_j softmax_j(softmax_scale * q[b,t,h,:] . K_j) V_j,
 *   lse[b,t,h]   = log sum_j exp(softmax_scale * q . K_j),
 * where K_j, V_j are the rows of logical position j of sequence b, read
 * through block_table[b][j / block_size] (int8 and fp8: the code's value
 * times its row's scale; nvfp4: times its block scale too). n <= 0 gives
 * out = 0 and lse = -inf. seq_lens counts the Tq new tokens, whose K/V must
 * already be in the cache (pa_cache_write). Arithmetic is fp32 (16-bit
 * operands: bf16, int8 codes and fp8 values widened exactly; fp32
 * accumulation).
 *   q              [B, Tq, Hq, D] in q_dtype
 *   block_table    [B, max_blocks_per_seq] int32; entries for logical blocks
 *                  < ceil(seq_lens[b] / block_size) must be in [0, num_blocks)
 *   seq_lens       [B] int32, each in [0, max_seq_len]
 *   max_seq_len    (host) an upper bound of seq_lens; it sizes the grid, so
 *                  no device data is read on the host.
 *                  max_blocks_per_seq * block_size >= max_seq_len is required.
 *   partition_size tokens per split-K partition, a multiple of block_size,
 *                  or 0 to let pa_choose_partition_size pick it.
 *   out, lse       outputs; lse may be NULL.
 *   workspace      device scratch of workspace_bytes >= pa_decode_workspace_bytes,
 *                  16-byte aligned (may be NULL when that size is 0;
 *                  PA_ERR_ALIGN otherwise).
 *   num_partitions (host, out) NP = ceil(max_seq_len / P).
 * When *num_partitions == 1 the kernel writes out/lse directly. Otherwise it
 * writes per-partition results to the workspace and leaves out/lse untouched:
 * the caller must then run pa_decode_splitk_reduce on the same stream.
 */
int pa_decode(const void* q, pa_dtype q_dtype, int32_t B, int32_t Tq, int32_t Hq, int32_t Hkv, int32_t D,
              const void* k_cache, const void* v_cache, pa_dtype kv_dtype, const float* k_scale,
              const float* v_scale, int64_t num_blocks, int32_t block_size, const int32_t* block_table,
              int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t max_seq_len, float softmax_scale,
              int32_t partition_size, void* out, pa_dtype out_dtype, float* lse, void* workspace,
              size_t workspace_bytes, int32_t* num_partitions, void* stream);

/*
 * pa_decode_splitk_reduce — merge split-K partials by log-sum-exp.
 *
 * The split-KV merge (nvllm page, "Acknowledgments", b12x): with partial
 * outputs o_i (normalised within partition i) and partial log-sum-exps
 * lse_i, M = max_i lse_i, w_i = exp(lse_i - M),
 *   out = sum_i w_i o_i / sum_i w_i,  lse = M + log sum_i w_i.
 * Partitions with lse_i = -inf weigh 0; a row whose partitions are all -inf
 * gives out = 0, lse = -inf.
 * Workspace layout (fp32, written by pa_decode, also fillable by a caller
 * that merges partials from elsewhere): o [B, Tq, Hq, NP, D] at offset 0,
 * then lse [B, Tq, Hq, NP] at the next 256-byte boundary. Row (b, t, h)
 * reads partitions i < ceil(max(n, 0) / partition_size) with
 * n = seq_lens[b] - Tq + t + 1, which are exactly the ones pa_decode writes.
 * One log-sum-exp per partition stands for the (max, sum) pair a merge could
 * also take (lse_i = m_i + log l_i): the decode forms it once per partition
 * and the merge reads one scalar instead of two.
 * workspace and out must be 16-byte aligned (PA_ERR_ALIGN otherwise).
 */
int pa_decode_splitk_reduce(const void* workspace, int32_t num_partitions, int32_t partition_size, int32_t B,
                            int32_t Tq, int32_t Hq, int32_t D, const int32_t* seq_lens, void* out,
                            pa_dtype out_dtype, float* lse, void* stream);

/*
 * pa_decode_shared_prefix — pa_decode for a batch whose sequences all begin
 * with the same prefix_len tokens stored in the same physical blocks (prefix
 * caching: vllm-sm12x-nvfp4-dflash2 page, "What makes this stack different",
 * capacity-first profile; 1Cat-vLLM docs index, feature list). Computes
 * exactly what pa_decode computes (same out and lse definitions, same
 * tolerances), but reads the shared blocks once per kv head and group of 64
 * query rows for the whole batch instead of once per sequence:
 *  1. prefix pass: the Tq * (Hq / Hkv) query rows of every sequence that use
 *     kv head g form one row set (B * Tq * Hq / Hkv rows) on the matrix
 *     cores, against keys 0 .. prefix_len - 1 read through prefix_table;
 *  2. tail pass: each sequence against its own keys prefix_len ..
 *     seq_lens[b] - 1 through block_table[b][prefix_len / 16 ..], causal mask
 *     as in pa_decode;
 *  3. the log-sum-exp merge of both passes' partials (as in
 *     pa_decode_splitk_reduce) into out and lse.
 * Arguments as for pa_decode, plus:
 *   prefix_table     [prefix_len / 16] int32 physical block ids of the shared
 *                    tokens (a row of block_table may serve); each in
 *                    [0, num_blocks). May be NULL when prefix_len == 0.
 *   prefix_len       (host) shared tokens, a multiple of 16, with
 *                    prefix_len + Tq <= max_seq_len.
 *   prefix_partition, tail_partition  split-K partition sizes of the two
 *                    passes (multiples of 16), 0 = the library's choice.
 *   workspace        >= pa_decode_shared_prefix_workspace_bytes with the same
 *                    arguments; 16-byte aligned; NULL allowed when that is 0.
 * Device contract (trusted, as for pa_decode): every sequence's query tokens
 * lie after the prefix, prefix_len + Tq <= seq_lens[b] <= max_seq_len; the
 * blocks block_table[b][0 .. prefix_len / 16 - 1] are not read. Always
 * writes out (and lse if non-NULL): no separate reduce call. fp32 caches
 * return PA_ERR_UNSUPPORTED.
 */
int pa_decode_shared_prefix(const void* q, pa_dtype q_dtype, int32_t B, int32_t Tq, int32_t Hq, int32_t Hkv,
                            int32_t D, const void* k_cache, const void* v_cache, pa_dtype kv_dtype,
                            const float* k_scale, const float* v_scale, int64_t num_blocks, int32_t block_size,
                            const int32_t* prefix_table, int32_t prefix_len, const int32_t* block_table,
                            int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t max_seq_len,
                            float softmax_scale, int32_t prefix_partition, int32_t tail_partition, void* out,
                            pa_dtype out_dtype, float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace pa_decode_shared_prefix needs for these arguments (0
 * when one partition covers everything, or for invalid arguments). */
size_t pa_decode_shared_prefix_workspace_bytes(int32_t B, int32_t Tq, int32_t Hq, int32_t Hkv, int32_t D,
                                               pa_dtype kv_dtype, int32_t max_seq_len, int32_t prefix_len,
                                               int32_t prefix_partition, int32_t tail_partition);

/* Bytes of workspace pa_decode needs (0 when one partition covers
 * max_seq_len). partition_size 0 means the heuristic's choice, as in
 * pa_decode; the caller must pass the same arguments to both. Hkv and
 * kv_dtype are among them because the heuristic's partition size, and so the
 * partition count, depends on the kernel and grid they select. Returns 0 for
 * invalid arguments (pa_decode then reports the error). */
size_t pa_decode_workspace_bytes(int32_t B, int32_t Tq, int32_t Hq, int32_t Hkv, int32_t D, pa_dtype kv_dtype,
                                 int32_t max_seq_len, int32_t partition_size);

/* The partition size pa_decode uses for partition_size == 0: a multiple of
 * 16 chosen so that the grid (partitions x kv heads x sequences x query
 * groups) fills the GPU's compute units while keeping the split-K workspace
 * small (the stream-K rationale of the nvllm page, "SM120 Stream-K Decode
 * Optimization": split the long dimension when the batch alone cannot fill
 * the machine). The compute units are those of the calling thread's current
 * HIP device (pa_device_cu_count). Returns a negative PA_ERR_* code for
 * invalid arguments. */
int32_t pa_choose_partition_size(int32_t B, int32_t Tq, int32_t Hq, int32_t Hkv, int32_t D, pa_dtype kv_dtype,
                                 int32_t max_seq_len);

/* The same heuristic for a device of num_cus compute units (>= 1): what
 * pa_choose_partition_size returns on such a device. A sizing aid for callers
 * that plan for another device, and the heuristic's host-side test hook. */
int32_t pa_choose_partition_size_for_cus(int32_t B, int32_t Tq, int32_t Hq, int32_t Hkv, int32_t D,
                                         pa_dtype kv_dtype, int32_t max_seq_len, int32_t num_cus);

/* Compute units of the calling thread's current HIP device, as the heuristic
 * uses them (hipDeviceAttributeMultiprocessorCount, read once per device; a
 * partitioned GPU reports its partition's share). With no visible device: 256,
 * the MI355X figure. */
int32_t pa_device_cu_count(void);

/* Name of the decode kernel pa_decode launches for these arguments:
 * "decode_wave_kernel" (vector ALU, one query token, small groups),
 * "decode_stream_kernel" (matrix cores, int8, FP8 and NVFP4 caches whose
 * G * Tq rows of a kv head fit one 16-row tile, from groups of 6 at one query token;
 * each wave streams its own blocks; partitions of at most 4096 tokens, a
 * larger given partition_size takes the next kernel), "decode_mfma_kernel"
 * (matrix cores: Tq > 1, groups of 16+ query heads, int8 and FP8 caches with
 * more rows) or "decode_valu_kernel" (fp32 caches); "" for invalid arguments.
 * The name is the one for the heuristic's partition size. A static string;
 * nothing is launched. */
const char* pa_decode_kernel_name(int32_t Tq, int32_t Hq, int32_t Hkv, pa_dtype kv_dtype);

/*
 * pa_decode_check — debug-time validation of the device data pa_decode
 * trusts (block and slot ids out of range, and padded rows written into other
 * requests' slots, are the defects the vllm-sm70 page reports: "Changes
 * relative to 1Cat-vLLM", "Known limitations").
 * Reads seq_lens[b] for b < B and block_table[b][j] for logical blocks
 * j < min(ceil(seq_lens[b] / 16), max_blocks_per_seq), on `stream`, and
 * writes status[0] = the number of violations (seq_lens[b] outside
 * [0, max_seq_len], or a block id outside [0, num_blocks)) and status[1] =
 * the smallest flat index of one (b * (max_blocks_per_seq + 1) + j for table
 * entry j, b * (max_blocks_per_seq + 1) + max_blocks_per_seq for seq_lens[b]),
 * or -1. status: device int32[2]. Every read stays in bounds whatever the
 * values; nothing else is read or written. Runs as one workgroup: a debug aid,
 * not part of the decode step.
 */
int pa_decode_check(const int32_t* block_table, int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t B,
                    int32_t max_seq_len, int64_t num_blocks, int32_t* status, void* stream);

/*
 * pa_cache_write_check — debug-time validation of slot_mapping for
 * pa_cache_write: status[0] = the number of tokens whose slot is
 * >= num_blocks * block_size, status[1] = the first such token index or -1
 * (negative slots mean "skip" and are valid). Duplicate slots are not
 * detected. status: device int32[2].
 */
int pa_cache_write_check(const int64_t* slot_mapping, int64_t num_tokens, int64_t num_blocks, int32_t block_size,
                         int32_t* status, void* stream);

/*
 * Sparse block-selection decode (vllm-sm70 page: "Changes relative to
 * 1Cat-vLLM", item 8, per-block sparse-decode mean keys refreshed for every
 * request of a decode batch; "Known limitations", a selection over at most
 * 4096 key blocks, a 262,144-token table at 64-token blocks). The pages give
 * no selection rule; the one implemented:
 *  - a sequence's positions form sparse blocks of sparse_block tokens (a
 *    multiple of 16, at most 4096; 64 on the page): block j = positions
 *    sparse_block * j .. sparse_block * (j + 1) - 1 below the length; at most
 *    4096 blocks per sequence (PA_ERR_UNSUPPORTED beyond);
 *  - a block's mean key per kv head is the plain mean of its keys below the
 *    length (quantised caches: dequantised values), in fp32;
 *  - the blocks holding a query token (positions L - Tq .. L - 1) are always
 *    selected; every other block j scores the largest, over the Tq * G query
 *    rows of the kv head, of softmax_scale * q . mean_key[j], and the
 *    top_blocks - (kept blocks) best are selected, ties to the lower index;
 *  - each query row attends with the exact softmax to the keys of its kv
 *    head's selected blocks that the plain causal rule lets it see.
 * With top_blocks >= the block count the result is pa_decode's.
 */

/*
 * pa_sparse_mean_keys — refresh the mean keys of the sparse blocks that hold
 * each sequence's newest num_new tokens (positions seq_lens[b] - num_new ..
 * seq_lens[b] - 1; num_new >= max_seq_len rebuilds every block): call after
 * pa_cache_write of a decode step with num_new = Tq for every request of the
 * batch. mean_k: [B, max_sparse_blocks, Hkv, D] fp32, caller-owned, row b
 * belonging to the sequence in row b of block_table; entries of blocks at or
 * past a sequence's ceil(seq_lens[b] / sparse_block) are not written.
 * Requires max_sparse_blocks >= ceil(max_seq_len / sparse_block). Sums run in
 * fp32 in a fixed order (the same result on every call).
 */
int pa_sparse_mean_keys(const void* k_cache, pa_dtype kv_dtype, const float* k_scale, int64_t num_blocks,
                        int32_t block_size, int32_t Hkv, int32_t D, const int32_t* block_table,
                        int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t B, int32_t max_seq_len,
                        int32_t sparse_block, int32_t num_new, float* mean_k, int32_t max_sparse_blocks,
                        void* stream);

/*
 * pa_decode_sparse — the decode over each (sequence, kv head)'s selected
 * sparse blocks. Arguments as for pa_decode (caches bf16, int8, fp8 or
 * nvfp4; fp32 caches return PA_ERR_UNSUPPORTED), plus:
 *   mean_k, max_sparse_blocks  the mean keys (pa_sparse_mean_keys), current
 *                  for every block below each sequence's length
 *   sparse_block, top_blocks   the selection (top_blocks >= 1)
 *   partition_size split-K partition over the selected keys (0: heuristic)
 *   selected       optional (may be NULL) [B, Hkv, S] int32 output, S =
 *                  min(ceil(max_seq_len / sparse_block), max(top_blocks, 2)):
 *                  the selected blocks in increasing order, -1 after the last
 *   workspace      >= pa_decode_sparse_workspace_bytes with the same
 *                  arguments, 16-byte aligned: scores, the compacted block
 *                  tables (the selected blocks' cache blocks in order, one row
 *                  per (sequence, kv head)) and the split-K partials.
 * Always writes out (and lse if non-NULL). Runs a score kernel, a selection
 * kernel, the decode kernel pa_decode would choose (one kv head per
 * workgroup) over the compacted tables, and the LSE reduce.
 */
int pa_decode_sparse(const void* q, pa_dtype q_dtype, int32_t B, int32_t Tq, int32_t Hq, int32_t Hkv, int32_t D,
                     const void* k_cache, const void* v_cache, pa_dtype kv_dtype, const float* k_scale,
                     const float* v_scale, int64_t num_blocks, int32_t block_size, const int32_t* block_table,
                     int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t max_seq_len, float softmax_scale,
                     const float* mean_k, int32_t max_sparse_blocks, int32_t sparse_block, int32_t top_blocks,
                     int32_t partition_size, void* out, pa_dtype out_dtype, float* lse, int32_t* selected,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace pa_decode_sparse needs for these arguments (0 for
 * invalid arguments). */
size_t pa_decode_sparse_workspace_bytes(int32_t B, int32_t Tq, int32_t Hq, int32_t Hkv, int32_t D, pa_dtype kv_dtype,
                                        int32_t max_seq_len, int32_t sparse_block, int32_t top_blocks,
                                        int32_t partition_size);

/*
 * pa_decode_noalloc — pa_decode followed by pa_decode_splitk_reduce, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the split-K partials
 * go to a scratch array that the library owns, PA_NOALLOC_SCRATCH_BYTES per
 * GPU, held from the library's first use on that GPU until the process ends.
 * Arguments, results and errors as for pa_decode, minus the workspace: out
 * (and lse when non-NULL) are always written, whatever the partition count.
 * Calls whose partials need more than PA_NOALLOC_SCRATCH_BYTES
 * (pa_decode_workspace_bytes with the same arguments) return
 * PA_ERR_WORKSPACE before any launch. No allocation of any kind: no hipMalloc,
 * no hipFree, no allocating library routine. The first call on a device
 * resolves the scratch's device address there (hipGetSymbolAddress); make it
 * outside a graph capture. Every call on one GPU shares that GPU's scratch:
 * calls that overlap in time on one GPU (different streams, or different
 * host threads without ordering) race on it and give wrong results; calls on
 * one stream are ordered and safe. Nothing in the scratch needs to start at
 * zero: each call writes every partial its reduce reads.
 */
#define PA_NOALLOC_SCRATCH_BYTES (32u << 20)
int pa_decode_noalloc(const void* q, pa_dtype q_dtype, int32_t B, int32_t Tq, int32_t Hq, int32_t Hkv, int32_t D,
                      const void* k_cache, const void* v_cache, pa_dtype kv_dtype, const float* k_scale,
                      const float* v_scale, int64_t num_blocks, int32_t block_size, const int32_t* block_table,
                      int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t max_seq_len,
                      float softmax_scale, int32_t partition_size, void* out, pa_dtype out_dtype, float* lse,
                      void* stream);

/* Message for the calling thread's last non-zero return ("" if none). */
/*
 * pa_read_probe — measurement helper, not part of the decode path: the
 * streaming-read ceiling against which a decode's read rate is judged (the
 * decode is a streaming scan of its KV bytes). Reads every byte of buf once
 * with the decode kernels' load (nontemporal 16-byte buffer loads) in
 * `workgroups` workgroups of 256 threads, each taking every workgroups-th
 * 16 KB segment, and writes into sink[i] the 32-bit wrap-around sum of the
 * 32-bit words workgroup i read: the sum over sink[0 .. workgroups - 1] is
 * the sum of every word of buf, a check that each was read exactly once.
 *   buf         device, 16-byte aligned; bytes a multiple of 16 (0: sink zeros)
 *   sink        device, workgroups uint32 (the caller's)
 *   workgroups  1 .. 65535 (the caller sizes the grid to the device: 8 to 64
 *               per CU all read at 6.9-7.1 TB/s on an MI355X)
 * Errors: PA_ERR_NULL (buf with bytes > 0, or sink NULL), PA_ERR_ALIGN,
 * PA_ERR_SHAPE (bytes not a multiple of 16, workgroups out of range),
 * PA_ERR_LAUNCH. Allocates nothing; capture-safe like every entry point.
 */
int pa_read_probe(const void* buf, size_t bytes, uint32_t* sink, int32_t workgroups, void* stream);

const char* pa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_DECODE_H */
