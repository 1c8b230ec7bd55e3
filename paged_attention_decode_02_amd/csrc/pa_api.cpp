// Host side of the C ABI declared in include/pa_decode.h: argument checks,
// the split-K partition heuristic, and dispatch to the gfx950 kernels. No
// device memory is allocated and no device data is read here, so every entry
// point can be recorded in a HIP graph.
#include "../../include/pa_decode.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "pa_internal.hpp"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int ok() {
    g_err.clear();
    return PA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool supported_d(int32_t D) { return D == 64 || D == 128 || D == 256; }

constexpr int kBlock = 16;
constexpr int kMaxTq = 16;
constexpr int kMaxGroup = 64;
constexpr int kDefaultCUs = 256;   // MI355X compute units; used when no HIP device is visible
constexpr int kMaxDevices = 64;
constexpr int kWavesPerCU = 8;     // resident one-wave (fp32-cache) workgroups per CU
constexpr int kMinPartition = 256; // tokens; bounds the split-K partial traffic

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Compute units of the calling thread's current HIP device, read once per
// device (a property query: nothing is enqueued and no device memory is
// read, so the first call may come from inside a graph capture). A
// partitioned GPU exposes fewer CUs per device and gets grids sized for them.
// Without a visible device (sizing on a host with no GPU) the MI355X count.
int device_cus() {
    static std::atomic<int> cached[kMaxDevices];
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();  // leave no error behind for the caller's next check
        return kDefaultCUs;
    }
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
        (void)hipGetLastError();
        n = kDefaultCUs;
    }
    cached[dev].store(n, std::memory_order_relaxed);
    return n;
}

// Head-chunk width of the VALU decode for a query group of G heads, and the
// number of chunks a kv head's group is split into.
void head_chunks(int32_t G, int* GT, int* nchunk) {
    int gt;
    if (G <= 8) {
        gt = G;
        while (!pa::decode_valu_has_gt(gt)) ++gt;  // 3 -> 4, 5 -> 6, 7 -> 8
    } else {
        gt = 8;
    }
    *GT = gt;
    *nchunk = (G + gt - 1) / gt;
}

// Waves per decode workgroup: the fp32-cache kernel uses one, the bf16/int8
// kernel four (they split a partition and merge in LDS).
int waves_per_wg(pa_dtype kv_dtype) { return kv_dtype == PA_F32 ? 1 : 4; }

// The matrix-core kernel takes all G*Tq rows of a kv head at once when they
// fill at least one 16-row MFMA tile (bf16 and int8 caches).
bool kv_supported(pa_dtype t) {
    return t == PA_F32 || t == PA_BF16 || t == PA_I8 || t == PA_FP8 || t == PA_NVFP4;
}

// caches stored as codes with one fp32 scale per (token, kv head)
bool quantised(pa_dtype t) { return t == PA_I8 || t == PA_FP8 || t == PA_NVFP4; }

// storage bytes per (token, kv head): a block is 16 Hkv times this
int64_t row_bytes(pa_dtype t, int32_t D) {
    if (t == PA_NVFP4) return D / 2 + D / 16;
    return (int64_t)D * (t == PA_F32 ? 4 : t == PA_BF16 ? 2 : 1);
}

// The matrix-core kernel reads a kv head's blocks once for all G * Tq rows;
// the vector-ALU kernel once per query token, with work that grows with G.
// Measured (kernel times, 16K-250K tokens, D 128 and 256): with Tq > 1 the
// matrix cores take 0.17-0.86x the time for every group size and cache type;
// with Tq = 1 they win from G = 16 (a full row tile), and for int8 and FP8
// caches already from G = 6 (int8 0.77-0.95x; FP8 at 250K tokens: step 112 ->
// 105 us; the vector-ALU decode is bound by its code widening and dot
// products, the matrix-core one is not). bf16 below 16 rows is a wash (64K:
// decode 0.7% slower, step 1.3% faster through half the partitions; short
// variable-length batches 5% slower) and NVFP4 is faster on the vector ALU
// than on the tiled kernel (250K: decode 92 against 103 us), so both stay
// off it below a full tile (NVFP4 from G = 6 takes the streaming kernel).
bool use_mfma(int32_t Tq, int32_t Hq, int32_t Hkv, pa_dtype kv_dtype) {
    if (kv_dtype == PA_F32) return false;
    const int64_t G = Hq / Hkv;
    return Tq > 1 || G >= 16 || ((kv_dtype == PA_I8 || kv_dtype == PA_FP8) && G >= 6);
}

// The streaming matrix-core kernel (each wave runs its own blocks, keys and
// values copied straight into LDS) takes the quantised caches when all rows
// of a kv head fit one 16-row tile: int8 and FP8 where the matrix cores are
// chosen, NVFP4 from G = 6 or Tq > 1 (250K tokens, G = 6: decode 90.9 us
// against 96.7 on the vector ALU); its partitions hold at most
// kStreamMaxPartition tokens (larger given sizes use the next kernel).
bool stream_kernel(int32_t Tq, int32_t Hq, int32_t Hkv, pa_dtype kv_dtype) {
    if ((int64_t)(Hq / Hkv) * Tq > 16) return false;
    if (kv_dtype == PA_I8 || kv_dtype == PA_FP8) return use_mfma(Tq, Hq, Hkv, kv_dtype);
    if (kv_dtype == PA_NVFP4) return Tq > 1 || Hq / Hkv >= 6;
    return false;
}

// kv heads per workgroup of the streaming kernel, one wave each when 4: the
// workgroup then reads whole token rows of every block (measured at 250K
// int8 tokens: 91.3 -> 84.9 us against one head per workgroup, the heads'
// 256-byte slices of each 1 KB row read by four different workgroups).
// Per-head block tables (sparse decode) take one head per workgroup.
int stream_hpg(int32_t Hkv, bool head_tables) {
    if (head_tables) return 1;
    return Hkv % 4 == 0 ? 4 : Hkv % 2 == 0 ? 2 : 1;
}

// Longest partition the streaming kernel takes (its per-wave table window
// of 256 blocks, the waves of a head sharing a partition's blocks).
int32_t stream_max_partition(pa_dtype kv_dtype, int32_t D, int hpg) {
    return pa::kStreamMaxPartition * (pa::stream_waves((int)kv_dtype, D) / hpg);
}

// Row tiles per workgroup and row chunks of the matrix-core kernel: at most
// four tiles (one per wave) per chunk, the tiles spread evenly over the
// chunks (96 rows: two chunks of three tiles, not four and two).
void row_chunks(int32_t R, int* NT, int* nchunk) {
    const int tiles = R > 16 ? (R + 15) / 16 : 1;  // an empty batch still sizes one tile
    *nchunk = (tiles + 3) / 4;
    *NT = (tiles + *nchunk - 1) / *nchunk;
}

// Workgroups of the decode resident per CU that the partition heuristic aims
// for (measured on the named workloads): the bf16 vector-ALU kernel with
// 512-byte rows streams best with one four-wave workgroup per CU (fewer
// concurrent streams: 2% faster at 64K than two); small head chunks (D * GT
// <= 512, few registers) want eight (more than fit at once: the dispatcher
// backfills CUs whose short partitions finish early), so that short contexts
// still fill the machine; everything else two (the int8 path is bound by its vector ALU work
// and needs the second wave per SIMD).
int wgs_per_cu(pa_dtype kv_dtype, int32_t D, int GT, bool mfma) {
    if (kv_dtype == PA_F32) return kWavesPerCU;  // one-wave workgroups
    if (mfma) return 2;
    if (D * GT <= 512) return 8;
    if (kv_dtype == PA_BF16 && D >= 256) return 1;
    return 2;
}

// kv heads per workgroup of the bf16/int8 vector-ALU decode. Where one
// workgroup per CU streams best (see wgs_per_cu), a workgroup takes as many
// kv heads as divide Hkv up to 4, one wave each: it reads whole token rows of
// every block, and workgroups of different kv heads no longer finish at
// different times (measured: 3.7% faster at 64K). int8 with large head
// chunks takes two kv heads, two waves each (measured at 250K tokens: decode
// 2.5% faster than one head, 4% faster than four, whose partitions get too
// many for the reduce). Elsewhere one kv head, its blocks shared by the four
// waves (short contexts need the finer split).
int heads_per_wg(pa_dtype kv_dtype, int32_t D, int GT, int32_t Hkv) {
    if ((kv_dtype == PA_I8 || kv_dtype == PA_FP8 || kv_dtype == PA_NVFP4) && D * GT > 512) return Hkv % 2 == 0 ? 2 : 1;
    if (wgs_per_cu(kv_dtype, D, GT, false) != 1) return 1;
    return Hkv % 4 == 0 ? 4 : (Hkv % 2 == 0 ? 2 : 1);
}

// Partition length for a context of len tokens when every partition index
// launches per_partition workgroups: enough partitions that the launch fills
// the GPU once at wgs workgroups per CU, each a multiple of gran tokens and at
// least min_p long, and one partition when that covers the context.
int32_t split_len(int64_t len, int64_t per_partition, int wgs, int64_t gran, int64_t min_p, int cus) {
    const int64_t target = (int64_t)cus * wgs;  // workgroups that fill the GPU once
    if (per_partition < 1) per_partition = 1;   // an empty batch (B = 0)
    int64_t want_np = (target + per_partition - 1) / per_partition;
    if (want_np < 1) want_np = 1;
    int64_t P = (len + want_np - 1) / want_np;
    P = (P + gran - 1) / gran * gran;
    if (P < min_p) P = min_p;
    const int64_t whole = (len + kBlock - 1) / kBlock * kBlock;
    if (P >= whole) P = whole;  // one partition covers everything
    return (int32_t)P;
}

// head_tables: every (sequence, kv head) has a block table row of its own
// (the sparse decode's compacted tables), so a workgroup takes one kv head.
int32_t partition_for(int32_t B, int32_t Tq, int32_t Hq, int32_t Hkv, int32_t D, pa_dtype kv_dtype,
                      int32_t max_seq_len, int cus, bool head_tables = false) {
    if (max_seq_len <= kBlock) return kBlock;
    if (stream_kernel(Tq, Hq, Hkv, kv_dtype)) {
        // one workgroup per CU (its LDS stages fill the CU), each partition at
        // least 4 blocks per wave
        const int hpg = stream_hpg(Hkv, head_tables), wph = pa::stream_waves((int)kv_dtype, D) / hpg;
        int32_t P = split_len(max_seq_len, (int64_t)B * (Hkv / hpg), 1, (int64_t)kBlock * wph,
                              (int64_t)4 * kBlock * wph, cus);
        const int32_t cap = stream_max_partition(kv_dtype, D, hpg);
        return P > cap ? cap : P;
    }
    int GT = 0, nchunk, wph = waves_per_wg(kv_dtype);  // waves per kv head
    int64_t per_partition;  // workgroups per partition index
    const bool mfma = use_mfma(Tq, Hq, Hkv, kv_dtype);
    if (mfma) {
        int NT;
        row_chunks((Hq / Hkv) * Tq, &NT, &nchunk);
        per_partition = (int64_t)B * Hkv * nchunk;
    } else {
        head_chunks(Hq / Hkv, &GT, &nchunk);
        const int hpg = (kv_dtype == PA_F32 || head_tables) ? 1 : heads_per_wg(kv_dtype, D, GT, Hkv);
        per_partition = (int64_t)B * Tq * (Hkv / hpg) * nchunk;
        if (kv_dtype != PA_F32) wph = 4 / hpg;
    }
    const int wpw = waves_per_wg(kv_dtype);
    // one block per wave of a kv head at least; four-wave workgroups keep
    // partitions long enough to bound the split-K partials, one-wave
    // (fp32-cache) workgroups split short contexts finely
    const int64_t gran = (int64_t)kBlock * wph;
    int64_t min_p = wpw > 1 ? (int64_t)kMinPartition * wph / 4 : 0;
    // small head chunks on the vector ALU (eight workgroups per CU) split
    // short contexts twice as finely (measured, batched GQA D=128 G=4: 1-4K
    // step 25.3 -> 23.4 us, 8-16K 84.0 -> 72.0 us; the matrix-core decode of
    // short verify batches was 9-10% slower with the finer minimum)
    if (!mfma && D * GT <= 512) min_p /= 2;
    return split_len(max_seq_len, per_partition, wgs_per_cu(kv_dtype, D, GT, mfma), gran, min_p, cus);
}

// Prefix pass of the shared-prefix decode: the matrix-core kernel takes the
// B * Tq * G rows of a kv head as one row set, so a partition index launches
// Hkv * (row chunks) workgroups.
int32_t prefix_partition_for(int32_t B, int32_t Tq, int32_t Hq, int32_t Hkv, int32_t prefix_len, int cus) {
    if (prefix_len <= kBlock) return kBlock;
    int NT, nchunk;
    row_chunks(B * Tq * (Hq / Hkv), &NT, &nchunk);
    return split_len(prefix_len, (int64_t)Hkv * nchunk, 2, (int64_t)kBlock * 4, kMinPartition, cus);
}

int check_dims(int32_t B, int32_t Tq, int32_t Hq, int32_t Hkv, int32_t D) {
    if (B < 0) return fail(PA_ERR_SHAPE, "B=%d must be >= 0", B);
    if (Tq < 1) return fail(PA_ERR_SHAPE, "Tq=%d must be >= 1", Tq);
    if (Tq > kMaxTq) return fail(PA_ERR_UNSUPPORTED, "Tq=%d exceeds %d", Tq, kMaxTq);
    if (Hq < 1 || Hkv < 1) return fail(PA_ERR_SHAPE, "Hq=%d and Hkv=%d must be >= 1", Hq, Hkv);
    if (Hq % Hkv) return fail(PA_ERR_SHAPE, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
    if (Hq / Hkv > kMaxGroup) return fail(PA_ERR_UNSUPPORTED, "group Hq/Hkv=%d exceeds %d", Hq / Hkv, kMaxGroup);
    if (D < 1) return fail(PA_ERR_SHAPE, "D=%d must be >= 1", D);
    if (!supported_d(D)) return fail(PA_ERR_UNSUPPORTED, "D=%d not in {64, 128, 256}", D);
    return PA_OK;
}

// Checks shared by the decode entry points (everything but partitioning and
// the workspace).
int check_decode_args(const void* q, pa_dtype q_dtype, int32_t B, int32_t Tq, int32_t Hq, int32_t Hkv, int32_t D,
                      const void* k_cache, const void* v_cache, pa_dtype kv_dtype, const float* k_scale,
                      const float* v_scale, int64_t num_blocks, int32_t block_size, const int32_t* block_table,
                      int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t max_seq_len, const void* out,
                      pa_dtype out_dtype) {
    int rc = check_dims(B, Tq, Hq, Hkv, D);
    if (rc) return rc;
    if (q_dtype != PA_F32 && q_dtype != PA_BF16) return fail(PA_ERR_DTYPE, "q dtype %d not in {f32, bf16}", (int)q_dtype);
    if (!kv_supported(kv_dtype))
        return fail(PA_ERR_DTYPE, "kv dtype %d not in {f32, bf16, i8, fp8, nvfp4}", (int)kv_dtype);
    if (out_dtype != PA_F32 && out_dtype != PA_BF16)
        return fail(PA_ERR_DTYPE, "out dtype %d not in {f32, bf16}", (int)out_dtype);
    if (block_size < 1) return fail(PA_ERR_SHAPE, "block_size=%d must be >= 1", block_size);
    if (block_size != kBlock) return fail(PA_ERR_UNSUPPORTED, "block_size=%d (only 16)", block_size);
    if (num_blocks < 1) return fail(PA_ERR_SHAPE, "num_blocks=%lld must be >= 1", (long long)num_blocks);
    // kernels address within one KV block with 32-bit offsets
    const int64_t blk_bytes = (int64_t)kBlock * Hkv * row_bytes(kv_dtype, D);
    if (blk_bytes >= ((int64_t)1 << 31))
        return fail(PA_ERR_UNSUPPORTED, "a KV block of %lld bytes (Hkv=%d) exceeds 2^31", (long long)blk_bytes, Hkv);
    if (max_blocks_per_seq < 1) return fail(PA_ERR_SHAPE, "max_blocks_per_seq=%d must be >= 1", max_blocks_per_seq);
    if (max_seq_len < 0) return fail(PA_ERR_SHAPE, "max_seq_len=%d must be >= 0", max_seq_len);
    if ((int64_t)max_blocks_per_seq * block_size < max_seq_len)
        return fail(PA_ERR_SHAPE, "block table too short: %d blocks * %d < max_seq_len %d", max_blocks_per_seq,
                    block_size, max_seq_len);
    if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !out)
        return fail(PA_ERR_NULL, "q, caches, block_table, seq_lens and out must be non-NULL");
    if (quantised(kv_dtype) && (!k_scale || !v_scale))
        return fail(PA_ERR_NULL, "int8/fp8/nvfp4 caches need k_scale and v_scale");
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
        return fail(PA_ERR_ALIGN, "q, caches and out must be 16-byte aligned");
    return PA_OK;
}

// Decode parameters common to every launch of one call (no partitioning,
// no workspace, no offsets).
pa::DecodeParams base_params(const void* q, pa_dtype q_dtype, int32_t B, int32_t Tq, int32_t Hq, int32_t Hkv,
                             const void* k_cache, const void* v_cache, const float* k_scale, const float* v_scale,
                             const int32_t* block_table, int32_t max_blocks_per_seq, const int32_t* seq_lens,
                             float softmax_scale, void* out, pa_dtype out_dtype, float* lse) {
    pa::DecodeParams p{};
    p.q = q;
    p.q_bf16 = q_dtype == PA_BF16;
    p.B = B;
    p.Tq = Tq;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.G = Hq / Hkv;
    p.k_cache = k_cache;
    p.v_cache = v_cache;
    p.k_scale = k_scale;
    p.v_scale = v_scale;
    p.block_table = block_table;
    p.max_blocks = max_blocks_per_seq;
    p.seq_lens = seq_lens;
    p.qk_scale_log2 = softmax_scale * 1.4426950408889634f;
    p.out = out;
    p.out_bf16 = out_dtype == PA_BF16;
    p.lse = lse;
    return p;
}

// Workspace sections: o [rows, np, D], then lse [rows, np], each 256-byte aligned.
void set_workspace(pa::DecodeParams& p, void* workspace, size_t rows, int32_t np, int32_t D) {
    p.ws_o = reinterpret_cast<float*>(workspace);
    p.ws_lse = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + align256(rows * np * D * sizeof(float)));
}

// Kernel choice and launch shape for one decode launch: fp32 caches take the
// plain fp32 kernel; bf16, int8, fp8 and nvfp4 the matrix-core kernel where
// use_mfma says so (always for stacked rows), else the packed-dot kernel.
hipError_t dispatch(pa::DecodeParams p, pa_dtype kv_dtype, int32_t D, hipStream_t stream) {
    // the fp32-cache kernel knows no shared workspace, key offset or stacked rows
    if (kv_dtype == PA_F32 && (p.np_stride != p.NP || p.part_base || p.fill_empty || p.kv_begin || p.stacked))
        return hipErrorInvalidValue;
    const bool mfma = p.stacked || use_mfma(p.Tq, p.Hq, p.Hkv, kv_dtype);
    int GT, nchunk;
    if (mfma)
        row_chunks(p.G * p.Tq * (p.stacked ? p.B : 1), &GT, &nchunk);  // GT = row tiles per workgroup
    else
        head_chunks(p.G, &GT, &nchunk);
    p.nchunk = nchunk;
    p.hpg = (mfma || kv_dtype == PA_F32 || p.head_tables) ? 1 : heads_per_wg(kv_dtype, D, GT, p.Hkv);
    if (!p.stacked && stream_kernel(p.Tq, p.Hq, p.Hkv, kv_dtype)) {
        const int hpg = stream_hpg(p.Hkv, p.head_tables != 0);
        if (p.P <= stream_max_partition(kv_dtype, D, hpg)) {
            p.hpg = hpg;
            return pa::launch_decode_stream((int)kv_dtype, D, p, stream);
        }
    }
    return kv_dtype == PA_F32 ? pa::launch_decode_valu((int)kv_dtype, D, GT, p, stream)
           : mfma             ? pa::launch_decode_mfma((int)kv_dtype, D, GT, p, stream)
                              : pa::launch_decode_wave((int)kv_dtype, D, GT, p, stream);
}

// Partitioning of a shared-prefix decode: the prefix pass's partitions come
// first in each row's workspace, the tail pass's after them.
struct SharedPrefixPlan {
    int32_t p_prefix, np_prefix, p_tail, np_tail, np_total;
    size_t ws_bytes;
};

int plan_shared_prefix(int32_t B, int32_t Tq, int32_t Hq, int32_t Hkv, int32_t D, pa_dtype kv_dtype,
                       int32_t max_seq_len, int32_t prefix_len, int32_t prefix_partition, int32_t tail_partition,
                       SharedPrefixPlan* pl) {
    int rc = check_dims(B, Tq, Hq, Hkv, D);
    if (rc) return rc;
    if (!kv_supported(kv_dtype)) return fail(PA_ERR_DTYPE, "kv dtype %d not supported", (int)kv_dtype);
    if (prefix_len < 0 || prefix_len % kBlock)
        return fail(PA_ERR_SHAPE, "prefix_len=%d must be a non-negative multiple of %d", prefix_len, kBlock);
    if (max_seq_len < (int64_t)prefix_len + Tq)
        return fail(PA_ERR_SHAPE, "max_seq_len=%d leaves no room for %d query tokens after a %d-token prefix",
                    max_seq_len, Tq, prefix_len);
    if (prefix_partition < 0 || prefix_partition % kBlock || tail_partition < 0 || tail_partition % kBlock)
        return fail(PA_ERR_SHAPE, "partition sizes %d, %d must be 0 or positive multiples of %d", prefix_partition,
                    tail_partition, kBlock);
    const int32_t tail_len = max_seq_len - prefix_len;
    const int cus = device_cus();
    pl->p_prefix = prefix_partition ? prefix_partition : prefix_partition_for(B, Tq, Hq, Hkv, prefix_len, cus);
    pl->np_prefix = prefix_len > 0 ? (prefix_len + pl->p_prefix - 1) / pl->p_prefix : 0;
    pl->p_tail = tail_partition ? tail_partition : partition_for(B, Tq, Hq, Hkv, D, kv_dtype, tail_len, cus);
    pl->np_tail = (int32_t)(((int64_t)tail_len + pl->p_tail - 1) / pl->p_tail);
    const int64_t total = (int64_t)pl->np_prefix + pl->np_tail;
    if (total > 0x7FFFFFFF) return fail(PA_ERR_SHAPE, "too many partitions");
    pl->np_total = (int32_t)total;
    const size_t rows = (size_t)B * Tq * Hq;
    pl->ws_bytes = pl->np_total > 1 ? align256(rows * total * D * sizeof(float)) + align256(rows * total * sizeof(float)) : 0;
    return PA_OK;
}

// Sizes of a sparse decode: blocks per sequence, selected blocks, compacted
// table width, partitioning and the workspace sections (scores, compacted
// tables, compacted lengths, split-K partials), each 256-byte aligned.
struct SparsePlan {
    int32_t nsb_max, max_sel, ctab_width, max_len, P, NP;
    size_t off_ctab, off_clen, off_part, ws_bytes;
};

int plan_sparse(int32_t B, int32_t Tq, int32_t Hq, int32_t Hkv, int32_t D, pa_dtype kv_dtype, int32_t max_seq_len,
                int32_t sparse_block, int32_t top_blocks, int32_t partition_size, SparsePlan* pl) {
    int rc = check_dims(B, Tq, Hq, Hkv, D);
    if (rc) return rc;
    if (!kv_supported(kv_dtype)) return fail(PA_ERR_DTYPE, "kv dtype %d not supported", (int)kv_dtype);
    if (kv_dtype == PA_F32) return fail(PA_ERR_UNSUPPORTED, "the sparse decode takes bf16, int8, fp8 or nvfp4 caches");
    if (max_seq_len < 0) return fail(PA_ERR_SHAPE, "max_seq_len=%d must be >= 0", max_seq_len);
    if (sparse_block < kBlock || sparse_block % kBlock || sparse_block > pa::kSparseMaxBlockTokens)
        return fail(PA_ERR_SHAPE, "sparse_block=%d must be a multiple of %d in [16, %d]", sparse_block, kBlock,
                    pa::kSparseMaxBlockTokens);
    if (top_blocks < 1) return fail(PA_ERR_SHAPE, "top_blocks=%d must be >= 1", top_blocks);
    if (partition_size < 0 || partition_size % kBlock)
        return fail(PA_ERR_SHAPE, "partition_size=%d must be 0 or a positive multiple of %d", partition_size, kBlock);
    const int64_t nsb = ((int64_t)max_seq_len + sparse_block - 1) / sparse_block;
    if (nsb > pa::kSparseMaxBlocks)
        return fail(PA_ERR_UNSUPPORTED, "%lld sparse blocks of %d tokens exceed the selection's %d",
                    (long long)nsb, sparse_block, pa::kSparseMaxBlocks);
    pl->nsb_max = (int32_t)nsb;
    pl->max_sel = (int32_t)(nsb < (top_blocks > 2 ? top_blocks : 2) ? nsb : (top_blocks > 2 ? top_blocks : 2));
    pl->ctab_width = pl->max_sel * (sparse_block / kBlock);
    pl->max_len = pl->max_sel * sparse_block;
    if ((int64_t)pl->max_len > 0x7FFFFFFF) return fail(PA_ERR_SHAPE, "selection too long");
    pl->P = partition_size ? partition_size
                           : partition_for(B, Tq, Hq, Hkv, D, kv_dtype, pl->max_len, device_cus(), true);
    pl->NP = pl->max_len > 0 ? (pl->max_len + pl->P - 1) / pl->P : 1;
    const size_t bg = (size_t)B * Hkv, rows = (size_t)B * Tq * Hq;
    pl->off_ctab = align256(bg * (size_t)(pl->nsb_max > 0 ? pl->nsb_max : 1) * sizeof(float));
    pl->off_clen = pl->off_ctab + align256(bg * (size_t)(pl->ctab_width > 0 ? pl->ctab_width : 1) * sizeof(int32_t));
    pl->off_part = pl->off_clen + align256(bg * sizeof(int32_t));
    pl->ws_bytes = pl->off_part;
    if (pl->NP > 1) pl->ws_bytes += align256(rows * pl->NP * D * sizeof(float)) + align256(rows * pl->NP * sizeof(float));
    return PA_OK;
}

}  // namespace

// Library-owned scratch of pa_decode_noalloc (the split-K partials), one copy
// per GPU the library runs on, held until the process ends. In host code the
// name is only a host-side handle: the device address of the copy on the
// current device comes from hipGetSymbolAddress, and only that address is
// passed to kernels.
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace {

// Device address of the current device's scratch copy, resolved once per
// device (on the first pa_decode_noalloc call with that device current).
int scratch_address(void** out) {
    static std::atomic<void*> addr[kMaxDevices];
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return fail(PA_ERR_LAUNCH, "no usable HIP device (%s, device %d)", hipGetErrorString(e), dev);
    }
    void* p = addr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr) {
            (void)hipGetLastError();
            return fail(PA_ERR_LAUNCH, "scratch address on device %d: %s", dev, hipGetErrorString(e));
        }
        addr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return PA_OK;
}

}  // namespace

extern "C" {

const char* pa_last_error(void) { return g_err.c_str(); }

int pa_decode_check(const int32_t* block_table, int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t B,
                    int32_t max_seq_len, int64_t num_blocks, int32_t* status, void* stream) {
    if (!block_table || !seq_lens || !status) return fail(PA_ERR_NULL, "block_table, seq_lens and status must be non-NULL");
    if (B < 0 || max_blocks_per_seq < 1 || max_seq_len < 0 || num_blocks < 1)
        return fail(PA_ERR_SHAPE, "B=%d, max_blocks_per_seq=%d, max_seq_len=%d, num_blocks=%lld out of range", B,
                    max_blocks_per_seq, max_seq_len, (long long)num_blocks);
    pa::DecodeCheckParams p{};
    p.block_table = block_table;
    p.max_blocks = max_blocks_per_seq;
    p.seq_lens = seq_lens;
    p.B = B;
    p.max_seq_len = max_seq_len;
    p.num_blocks = num_blocks;
    p.status = status;
    hipError_t e = pa::launch_decode_check(p, (hipStream_t)stream);
    if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "decode_check launch failed: %s", hipGetErrorString(e));
    return ok();
}

int pa_cache_write_check(const int64_t* slot_mapping, int64_t num_tokens, int64_t num_blocks, int32_t block_size,
                         int32_t* status, void* stream) {
    if (!status || (num_tokens > 0 && !slot_mapping)) return fail(PA_ERR_NULL, "slot_mapping and status must be non-NULL");
    if (num_tokens < 0 || num_blocks < 1 || block_size < 1)
        return fail(PA_ERR_SHAPE, "num_tokens=%lld, num_blocks=%lld, block_size=%d out of range", (long long)num_tokens,
                    (long long)num_blocks, block_size);
    pa::SlotsCheckParams p{};
    p.slots = slot_mapping;
    p.num_tokens = num_tokens;
    p.num_slots = num_blocks * block_size;
    p.status = status;
    hipError_t e = pa::launch_slots_check(p, (hipStream_t)stream);
    if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "cache_write_check launch failed: %s", hipGetErrorString(e));
    return ok();
}

int32_t pa_choose_partition_size_for_cus(int32_t B, int32_t Tq, int32_t Hq, int32_t Hkv, int32_t D,
                                         pa_dtype kv_dtype, int32_t max_seq_len, int32_t num_cus) {
    int rc = check_dims(B, Tq, Hq, Hkv, D);
    if (rc) return rc;
    if (!kv_supported(kv_dtype)) return fail(PA_ERR_DTYPE, "kv dtype %d not supported", (int)kv_dtype);
    if (max_seq_len < 0) return fail(PA_ERR_SHAPE, "max_seq_len=%d must be >= 0", max_seq_len);
    if (num_cus < 1) return fail(PA_ERR_SHAPE, "num_cus=%d must be >= 1", num_cus);
    ok();
    return partition_for(B, Tq, Hq, Hkv, D, kv_dtype, max_seq_len, num_cus);
}

int32_t pa_choose_partition_size(int32_t B, int32_t Tq, int32_t Hq, int32_t Hkv, int32_t D, pa_dtype kv_dtype,
                                 int32_t max_seq_len) {
    return pa_choose_partition_size_for_cus(B, Tq, Hq, Hkv, D, kv_dtype, max_seq_len, device_cus());
}

int32_t pa_device_cu_count(void) { return device_cus(); }

int pa_read_probe(const void* buf, size_t bytes, uint32_t* sink, int32_t workgroups, void* stream) {
    if (!sink || (bytes > 0 && !buf)) return fail(PA_ERR_NULL, "sink (and buf when bytes > 0) must be non-NULL");
    if (bytes % 16) return fail(PA_ERR_SHAPE, "bytes=%zu must be a multiple of 16", bytes);
    if (workgroups < 1 || workgroups > 65535) return fail(PA_ERR_SHAPE, "workgroups=%d not in 1 .. 65535", workgroups);
    if (!aligned16(buf)) return fail(PA_ERR_ALIGN, "buf must be 16-byte aligned");
    hipError_t e = pa::launch_read_probe(buf, (int64_t)bytes, sink, workgroups, (hipStream_t)stream);
    if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "read_probe launch failed: %s", hipGetErrorString(e));
    return ok();
}

const char* pa_decode_kernel_name(int32_t Tq, int32_t Hq, int32_t Hkv, pa_dtype kv_dtype) {
    if (Tq < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || !kv_supported(kv_dtype)) return "";
    if (kv_dtype == PA_F32) return "decode_valu_kernel";
    if (stream_kernel(Tq, Hq, Hkv, kv_dtype)) return "decode_stream_kernel";
    return use_mfma(Tq, Hq, Hkv, kv_dtype) ? "decode_mfma_kernel" : "decode_wave_kernel";
}

size_t pa_decode_workspace_bytes(int32_t B, int32_t Tq, int32_t Hq, int32_t Hkv, int32_t D, pa_dtype kv_dtype,
                                 int32_t max_seq_len, int32_t partition_size) {
    if (check_dims(B, Tq, Hq, Hkv, D) || max_seq_len < 0 || partition_size < 0 || partition_size % kBlock)
        return 0;
    if (!kv_supported(kv_dtype)) return 0;
    const int32_t P =
        partition_size ? partition_size : partition_for(B, Tq, Hq, Hkv, D, kv_dtype, max_seq_len, device_cus());
    const int64_t NP = max_seq_len > 0 ? ((int64_t)max_seq_len + P - 1) / P : 1;
    if (NP <= 1) return 0;
    const size_t rows = (size_t)B * Tq * Hq;
    return align256(rows * NP * D * sizeof(float)) + align256(rows * NP * sizeof(float));
}

int pa_cache_write(const void* k_src, const void* v_src, pa_dtype src_dtype, const int64_t* slot_mapping,
                   int64_t num_tokens, void* k_cache, void* v_cache, pa_dtype cache_dtype, float* k_scale,
                   float* v_scale, int64_t num_blocks, int32_t block_size, int32_t Hkv, int32_t D, void* stream) {
    if (src_dtype != PA_F32 && src_dtype != PA_BF16)
        return fail(PA_ERR_DTYPE, "source dtype %d not in {f32, bf16}", (int)src_dtype);
    if (!kv_supported(cache_dtype))
        return fail(PA_ERR_DTYPE, "cache dtype %d not in {f32, bf16, i8, fp8, nvfp4}", (int)cache_dtype);
    if (num_tokens < 0) return fail(PA_ERR_SHAPE, "num_tokens=%lld must be >= 0", (long long)num_tokens);
    if (num_blocks < 1) return fail(PA_ERR_SHAPE, "num_blocks=%lld must be >= 1", (long long)num_blocks);
    if (block_size < 1 || Hkv < 1 || D < 1)
        return fail(PA_ERR_SHAPE, "block_size=%d, Hkv=%d, D=%d must be >= 1", block_size, Hkv, D);
    if (block_size != kBlock) return fail(PA_ERR_UNSUPPORTED, "block_size=%d (only 16)", block_size);
    if (!supported_d(D)) return fail(PA_ERR_UNSUPPORTED, "D=%d not in {64, 128, 256}", D);
    if (!k_cache || !v_cache) return fail(PA_ERR_NULL, "k_cache/v_cache is NULL");
    if (quantised(cache_dtype) && (!k_scale || !v_scale))
        return fail(PA_ERR_NULL, "int8/fp8/nvfp4 caches need k_scale and v_scale");
    if (num_tokens == 0) return ok();
    if (!k_src || !v_src || !slot_mapping) return fail(PA_ERR_NULL, "k_src/v_src/slot_mapping is NULL");
    if (!aligned16(k_src) || !aligned16(v_src) || !aligned16(k_cache) || !aligned16(v_cache))
        return fail(PA_ERR_ALIGN, "sources and caches must be 16-byte aligned");
    pa::CacheWriteParams p{};
    p.k_src = k_src;
    p.v_src = v_src;
    p.src_bf16 = src_dtype == PA_BF16;
    p.slots = slot_mapping;
    p.num_tokens = num_tokens;
    p.k_cache = k_cache;
    p.v_cache = v_cache;
    p.k_scale = k_scale;
    p.v_scale = v_scale;
    p.Hkv = Hkv;
    p.D = D;
    hipError_t e = pa::launch_cache_write((int)cache_dtype, p, (hipStream_t)stream);
    if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "cache_write launch failed: %s", hipGetErrorString(e));
    return ok();
}

int pa_decode(const void* q, pa_dtype q_dtype, int32_t B, int32_t Tq, int32_t Hq, int32_t Hkv, int32_t D,
              const void* k_cache, const void* v_cache, pa_dtype kv_dtype, const float* k_scale,
              const float* v_scale, int64_t num_blocks, int32_t block_size, const int32_t* block_table,
              int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t max_seq_len, float softmax_scale,
              int32_t partition_size, void* out, pa_dtype out_dtype, float* lse, void* workspace,
              size_t workspace_bytes, int32_t* num_partitions, void* stream) {
    if (!num_partitions) return fail(PA_ERR_NULL, "num_partitions is NULL");
    int rc = check_decode_args(q, q_dtype, B, Tq, Hq, Hkv, D, k_cache, v_cache, kv_dtype, k_scale, v_scale,
                               num_blocks, block_size, block_table, max_blocks_per_seq, seq_lens, max_seq_len,
                               out, out_dtype);
    if (rc) return rc;
    if (partition_size < 0 || partition_size % kBlock)
        return fail(PA_ERR_SHAPE, "partition_size=%d must be 0 or a positive multiple of %d", partition_size, kBlock);

    const int32_t P =
        partition_size ? partition_size : partition_for(B, Tq, Hq, Hkv, D, kv_dtype, max_seq_len, device_cus());
    const int64_t NP64 = max_seq_len > 0 ? ((int64_t)max_seq_len + P - 1) / P : 1;
    if (NP64 > 0x7FFFFFFF) return fail(PA_ERR_SHAPE, "too many partitions");
    const int32_t NP = (int32_t)NP64;
    const size_t need = pa_decode_workspace_bytes(B, Tq, Hq, Hkv, D, kv_dtype, max_seq_len, P);
    if (NP > 1 && (!workspace || workspace_bytes < need))
        return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : 0);
    // the reduce that must follow reads the partials as 16-byte vectors
    if (NP > 1 && !aligned16(workspace)) return fail(PA_ERR_ALIGN, "workspace must be 16-byte aligned");
    *num_partitions = NP;
    if (B == 0) return ok();

    pa::DecodeParams p = base_params(q, q_dtype, B, Tq, Hq, Hkv, k_cache, v_cache, k_scale, v_scale, block_table,
                                     max_blocks_per_seq, seq_lens, softmax_scale, out, out_dtype, lse);
    p.P = P;
    p.NP = NP;
    p.np_stride = NP;
    if (NP > 1) set_workspace(p, workspace, (size_t)B * Tq * Hq, NP, D);
    hipError_t e = dispatch(p, kv_dtype, D, (hipStream_t)stream);
    if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "decode launch failed: %s", hipGetErrorString(e));
    return ok();
}

size_t pa_decode_shared_prefix_workspace_bytes(int32_t B, int32_t Tq, int32_t Hq, int32_t Hkv, int32_t D,
                                               pa_dtype kv_dtype, int32_t max_seq_len, int32_t prefix_len,
                                               int32_t prefix_partition, int32_t tail_partition) {
    SharedPrefixPlan pl;
    if (plan_shared_prefix(B, Tq, Hq, Hkv, D, kv_dtype, max_seq_len, prefix_len, prefix_partition, tail_partition,
                           &pl))
        return 0;
    return pl.ws_bytes;
}

int pa_decode_shared_prefix(const void* q, pa_dtype q_dtype, int32_t B, int32_t Tq, int32_t Hq, int32_t Hkv,
                            int32_t D, const void* k_cache, const void* v_cache, pa_dtype kv_dtype,
                            const float* k_scale, const float* v_scale, int64_t num_blocks, int32_t block_size,
                            const int32_t* prefix_table, int32_t prefix_len, const int32_t* block_table,
                            int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t max_seq_len,
                            float softmax_scale, int32_t prefix_partition, int32_t tail_partition, void* out,
                            pa_dtype out_dtype, float* lse, void* workspace, size_t workspace_bytes, void* stream) {
    int rc = check_decode_args(q, q_dtype, B, Tq, Hq, Hkv, D, k_cache, v_cache, kv_dtype, k_scale, v_scale,
                               num_blocks, block_size, block_table, max_blocks_per_seq, seq_lens, max_seq_len,
                               out, out_dtype);
    if (rc) return rc;
    if (kv_dtype == PA_F32)
        return fail(PA_ERR_UNSUPPORTED, "shared-prefix decode takes bf16, int8, fp8 or nvfp4 caches, not f32");
    SharedPrefixPlan pl;
    rc = plan_shared_prefix(B, Tq, Hq, Hkv, D, kv_dtype, max_seq_len, prefix_len, prefix_partition, tail_partition,
                            &pl);
    if (rc) return rc;
    if (prefix_len > 0 && !prefix_table) return fail(PA_ERR_NULL, "prefix_table is NULL");
    if (pl.np_total > 1 && (!workspace || workspace_bytes < pl.ws_bytes))
        return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", pl.ws_bytes,
                    workspace ? workspace_bytes : 0);
    if (pl.np_total > 1 && !aligned16(workspace)) return fail(PA_ERR_ALIGN, "workspace must be 16-byte aligned");
    if (B == 0) return ok();

    const size_t rows = (size_t)B * Tq * Hq;
    pa::DecodeParams p = base_params(q, q_dtype, B, Tq, Hq, Hkv, k_cache, v_cache, k_scale, v_scale, block_table,
                                     max_blocks_per_seq, seq_lens, softmax_scale, out, out_dtype, lse);
    p.np_stride = pl.np_total;
    p.fill_empty = pl.np_total > 1;
    if (pl.np_total > 1) set_workspace(p, workspace, rows, pl.np_total, D);
    hipError_t e = hipSuccess;
    if (pl.np_prefix > 0) {
        // all rows of a kv head against the shared blocks, partitions 0 .. np_prefix - 1
        pa::DecodeParams pp = p;
        pp.stacked = 1;
        pp.prefix_len = prefix_len;
        pp.block_table = prefix_table;
        pp.max_blocks = prefix_len / kBlock;
        pp.P = pl.p_prefix;
        pp.NP = pl.np_prefix;
        pp.part_base = 0;
        e = dispatch(pp, kv_dtype, D, (hipStream_t)stream);
        if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "shared-prefix pass launch failed: %s", hipGetErrorString(e));
    }
    // each sequence's own keys after the prefix, with the causal mask
    p.kv_begin = prefix_len;
    p.P = pl.p_tail;
    p.NP = pl.np_tail;
    p.part_base = pl.np_prefix;
    e = dispatch(p, kv_dtype, D, (hipStream_t)stream);
    if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "tail pass launch failed: %s", hipGetErrorString(e));
    if (pl.np_total > 1) {
        pa::ReduceParams r{};
        r.ws_o = p.ws_o;
        r.ws_lse = p.ws_lse;
        r.NP = pl.np_total;
        r.P = pl.p_tail;
        r.B = B;
        r.Tq = Tq;
        r.Hq = Hq;
        r.D = D;
        r.seq_lens = seq_lens;
        r.out = out;
        r.out_bf16 = out_dtype == PA_BF16;
        r.lse = lse;
        r.all_parts = 1;
        e = pa::launch_splitk_reduce(r, (hipStream_t)stream);
        if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "reduce launch failed: %s", hipGetErrorString(e));
    }
    return ok();
}

int pa_decode_splitk_reduce(const void* workspace, int32_t num_partitions, int32_t partition_size, int32_t B,
                            int32_t Tq, int32_t Hq, int32_t D, const int32_t* seq_lens, void* out,
                            pa_dtype out_dtype, float* lse, void* stream) {
    if (B < 0 || Tq < 1 || Hq < 1) return fail(PA_ERR_SHAPE, "B=%d, Tq=%d, Hq=%d out of range", B, Tq, Hq);
    if (!supported_d(D)) return fail(PA_ERR_UNSUPPORTED, "D=%d not in {64, 128, 256}", D);
    if (num_partitions < 1) return fail(PA_ERR_SHAPE, "num_partitions=%d must be >= 1", num_partitions);
    if (partition_size < kBlock || partition_size % kBlock)
        return fail(PA_ERR_SHAPE, "partition_size=%d must be a positive multiple of %d", partition_size, kBlock);
    if (out_dtype != PA_F32 && out_dtype != PA_BF16)
        return fail(PA_ERR_DTYPE, "out dtype %d not in {f32, bf16}", (int)out_dtype);
    if (!workspace || !seq_lens || !out) return fail(PA_ERR_NULL, "workspace, seq_lens and out must be non-NULL");
    if (!aligned16(workspace) || !aligned16(out)) return fail(PA_ERR_ALIGN, "workspace and out must be 16-byte aligned");
    if (B == 0) return ok();
    const size_t rows = (size_t)B * Tq * Hq;
    pa::ReduceParams p{};
    p.ws_o = reinterpret_cast<const float*>(workspace);
    p.ws_lse = reinterpret_cast<const float*>(reinterpret_cast<const char*>(workspace) +
                                              align256(rows * num_partitions * D * sizeof(float)));
    p.NP = num_partitions;
    p.P = partition_size;
    p.B = B;
    p.Tq = Tq;
    p.Hq = Hq;
    p.D = D;
    p.seq_lens = seq_lens;
    p.out = out;
    p.out_bf16 = out_dtype == PA_BF16;
    p.lse = lse;
    hipError_t e = pa::launch_splitk_reduce(p, (hipStream_t)stream);
    if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "reduce launch failed: %s", hipGetErrorString(e));
    return ok();
}

int pa_sparse_mean_keys(const void* k_cache, pa_dtype kv_dtype, const float* k_scale, int64_t num_blocks,
                        int32_t block_size, int32_t Hkv, int32_t D, const int32_t* block_table,
                        int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t B, int32_t max_seq_len,
                        int32_t sparse_block, int32_t num_new, float* mean_k, int32_t max_sparse_blocks,
                        void* stream) {
    if (!kv_supported(kv_dtype)) return fail(PA_ERR_DTYPE, "kv dtype %d not supported", (int)kv_dtype);
    if (B < 0 || Hkv < 1 || num_blocks < 1 || max_seq_len < 0 || max_blocks_per_seq < 1)
        return fail(PA_ERR_SHAPE, "B=%d, Hkv=%d, num_blocks=%lld, max_seq_len=%d, max_blocks_per_seq=%d out of range", B,
                    Hkv, (long long)num_blocks, max_seq_len, max_blocks_per_seq);
    if (block_size != kBlock) return fail(PA_ERR_UNSUPPORTED, "block_size=%d (only 16)", block_size);
    if (!supported_d(D)) return fail(PA_ERR_UNSUPPORTED, "D=%d not in {64, 128, 256}", D);
    if ((int64_t)max_blocks_per_seq * kBlock < max_seq_len)
        return fail(PA_ERR_SHAPE, "block table too short: %d blocks for max_seq_len %d", max_blocks_per_seq, max_seq_len);
    if (sparse_block < kBlock || sparse_block % kBlock || sparse_block > pa::kSparseMaxBlockTokens)
        return fail(PA_ERR_SHAPE, "sparse_block=%d must be a multiple of %d in [16, %d]", sparse_block, kBlock,
                    pa::kSparseMaxBlockTokens);
    if (num_new < 1) return fail(PA_ERR_SHAPE, "num_new=%d must be >= 1", num_new);
    const int64_t nsb = ((int64_t)max_seq_len + sparse_block - 1) / sparse_block;
    if (max_sparse_blocks < nsb)
        return fail(PA_ERR_SHAPE, "max_sparse_blocks=%d below the %lld blocks of max_seq_len", max_sparse_blocks,
                    (long long)nsb);
    if (!k_cache || !block_table || !seq_lens || !mean_k)
        return fail(PA_ERR_NULL, "k_cache, block_table, seq_lens and mean_k must be non-NULL");
    if (quantised(kv_dtype) && !k_scale) return fail(PA_ERR_NULL, "int8/fp8/nvfp4 caches need k_scale");
    if (B == 0 || nsb == 0) return ok();
    // the blocks touched by the newest num_new tokens: at most ceil(num_new / SB) + 1
    int64_t nref = ((int64_t)num_new + sparse_block - 1) / sparse_block + 1;
    if (nref > nsb) nref = nsb;
    pa::SparseParams p{};
    p.B = B;
    p.Hkv = Hkv;
    p.D = D;
    p.k_cache = k_cache;
    p.k_scale = k_scale;
    p.block_table = block_table;
    p.max_blocks = max_blocks_per_seq;
    p.seq_lens = seq_lens;
    p.sparse_block = sparse_block;
    p.num_new = num_new;
    p.mean_k = mean_k;
    p.max_sblocks = max_sparse_blocks;
    hipError_t e = pa::launch_sparse_mean((int)kv_dtype, p, (int)nref, (hipStream_t)stream);
    if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "sparse mean-key launch failed: %s", hipGetErrorString(e));
    return ok();
}

size_t pa_decode_sparse_workspace_bytes(int32_t B, int32_t Tq, int32_t Hq, int32_t Hkv, int32_t D, pa_dtype kv_dtype,
                                        int32_t max_seq_len, int32_t sparse_block, int32_t top_blocks,
                                        int32_t partition_size) {
    SparsePlan pl;
    if (plan_sparse(B, Tq, Hq, Hkv, D, kv_dtype, max_seq_len, sparse_block, top_blocks, partition_size, &pl)) return 0;
    return pl.ws_bytes;
}

int pa_decode_sparse(const void* q, pa_dtype q_dtype, int32_t B, int32_t Tq, int32_t Hq, int32_t Hkv, int32_t D,
                     const void* k_cache, const void* v_cache, pa_dtype kv_dtype, const float* k_scale,
                     const float* v_scale, int64_t num_blocks, int32_t block_size, const int32_t* block_table,
                     int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t max_seq_len, float softmax_scale,
                     const float* mean_k, int32_t max_sparse_blocks, int32_t sparse_block, int32_t top_blocks,
                     int32_t partition_size, void* out, pa_dtype out_dtype, float* lse, int32_t* selected,
                     void* workspace, size_t workspace_bytes, void* stream) {
    int rc = check_decode_args(q, q_dtype, B, Tq, Hq, Hkv, D, k_cache, v_cache, kv_dtype, k_scale, v_scale,
                               num_blocks, block_size, block_table, max_blocks_per_seq, seq_lens, max_seq_len,
                               out, out_dtype);
    if (rc) return rc;
    SparsePlan pl;
    rc = plan_sparse(B, Tq, Hq, Hkv, D, kv_dtype, max_seq_len, sparse_block, top_blocks, partition_size, &pl);
    if (rc) return rc;
    if (!mean_k) return fail(PA_ERR_NULL, "mean_k must be non-NULL");
    if (max_sparse_blocks < pl.nsb_max)
        return fail(PA_ERR_SHAPE, "max_sparse_blocks=%d below the %d blocks of max_seq_len", max_sparse_blocks,
                    pl.nsb_max);
    if (!workspace || workspace_bytes < pl.ws_bytes)
        return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", pl.ws_bytes,
                    workspace ? workspace_bytes : 0);
    if (!aligned16(workspace)) return fail(PA_ERR_ALIGN, "workspace must be 16-byte aligned");
    if (B == 0) return ok();
    char* ws = reinterpret_cast<char*>(workspace);
    pa::SparseParams sp{};
    sp.q = q;
    sp.q_bf16 = q_dtype == PA_BF16;
    sp.B = B;
    sp.Tq = Tq;
    sp.Hq = Hq;
    sp.Hkv = Hkv;
    sp.D = D;
    sp.block_table = block_table;
    sp.max_blocks = max_blocks_per_seq;
    sp.seq_lens = seq_lens;
    sp.softmax_scale = softmax_scale;
    sp.sparse_block = sparse_block;
    sp.top_blocks = top_blocks;
    sp.mean_k = const_cast<float*>(mean_k);
    sp.max_sblocks = max_sparse_blocks;
    sp.scores = reinterpret_cast<float*>(ws);
    sp.nsb_max = pl.nsb_max;
    sp.max_sel = pl.max_sel;
    sp.sel_out = selected;
    sp.ctab = reinterpret_cast<int32_t*>(ws + pl.off_ctab);
    sp.ctab_width = pl.ctab_width;
    sp.clen = reinterpret_cast<int32_t*>(ws + pl.off_clen);
    hipError_t e = pa::launch_sparse_select(sp, (hipStream_t)stream);
    if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "sparse selection launch failed: %s", hipGetErrorString(e));
    // the decode over each (sequence, kv head)'s compacted table
    pa::DecodeParams p = base_params(q, q_dtype, B, Tq, Hq, Hkv, k_cache, v_cache, k_scale, v_scale, sp.ctab,
                                     pl.ctab_width, sp.clen, softmax_scale, out, out_dtype, lse);
    p.head_tables = 1;
    p.P = pl.P;
    p.NP = pl.NP;
    p.np_stride = pl.NP;
    if (pl.NP > 1) set_workspace(p, ws + pl.off_part, (size_t)B * Tq * Hq, pl.NP, D);
    e = dispatch(p, kv_dtype, D, (hipStream_t)stream);
    if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "sparse decode launch failed: %s", hipGetErrorString(e));
    if (pl.NP > 1) {
        pa::ReduceParams r{};
        r.ws_o = p.ws_o;
        r.ws_lse = p.ws_lse;
        r.NP = pl.NP;
        r.P = pl.P;
        r.B = B;
        r.Tq = Tq;
        r.Hq = Hq;
        r.D = D;
        r.Hkv = Hkv;
        r.head_lens = 1;
        r.seq_lens = sp.clen;
        r.out = out;
        r.out_bf16 = out_dtype == PA_BF16;
        r.lse = lse;
        e = pa::launch_splitk_reduce(r, (hipStream_t)stream);
        if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "reduce launch failed: %s", hipGetErrorString(e));
    }
    return ok();
}

int pa_decode_noalloc(const void* q, pa_dtype q_dtype, int32_t B, int32_t Tq, int32_t Hq, int32_t Hkv, int32_t D,
                      const void* k_cache, const void* v_cache, pa_dtype kv_dtype, const float* k_scale,
                      const float* v_scale, int64_t num_blocks, int32_t block_size, const int32_t* block_table,
                      int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t max_seq_len,
                      float softmax_scale, int32_t partition_size, void* out, pa_dtype out_dtype, float* lse,
                      void* stream) {
    int rc = check_decode_args(q, q_dtype, B, Tq, Hq, Hkv, D, k_cache, v_cache, kv_dtype, k_scale, v_scale,
                               num_blocks, block_size, block_table, max_blocks_per_seq, seq_lens, max_seq_len,
                               out, out_dtype);
    if (rc) return rc;
    if (partition_size < 0 || partition_size % kBlock)
        return fail(PA_ERR_SHAPE, "partition_size=%d must be 0 or a positive multiple of %d", partition_size, kBlock);
    const int32_t P =
        partition_size ? partition_size : partition_for(B, Tq, Hq, Hkv, D, kv_dtype, max_seq_len, device_cus());
    const size_t need = pa_decode_workspace_bytes(B, Tq, Hq, Hkv, D, kv_dtype, max_seq_len, P);
    if (need > (size_t)PA_NOALLOC_SCRATCH_BYTES)
        return fail(PA_ERR_WORKSPACE,
                    "the split-K partials need %zu bytes, above the %u-byte library scratch of pa_decode_noalloc "
                    "(use pa_decode with a workspace, or a larger partition_size)",
                    need, (unsigned)PA_NOALLOC_SCRATCH_BYTES);
    if (B == 0) return ok();
    void* ws = nullptr;
    rc = scratch_address(&ws);
    if (rc) return rc;
    int32_t np = 0;
    rc = pa_decode(q, q_dtype, B, Tq, Hq, Hkv, D, k_cache, v_cache, kv_dtype, k_scale, v_scale, num_blocks, block_size,
                   block_table, max_blocks_per_seq, seq_lens, max_seq_len, softmax_scale, P, out, out_dtype, lse, ws,
                   need, &np, stream);
    if (rc) return rc;
    if (np > 1) return pa_decode_splitk_reduce(ws, np, P, B, Tq, Hq, D, seq_lens, out, out_dtype, lse, stream);
    return ok();
}

}  // extern "C"
