/*
 * Paged-attention decode oracle: plain, slow, fp64 CPU code.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the independent reference the HIP
 * kernels are checked against. Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load it; the product path never does. It
 * includes no header and shares no code with the GPU library.
 *
 * What it computes, and where the pages say so:
 *  - PagedAttention: each sequence's keys and values live in fixed-size blocks
 *    reached through a per-sequence block table (nvllm page, "About": the
 *    PagedAttention citation; 1Cat-vLLM docs index, feature list: "efficient
 *    management of attention key and value memory with PagedAttention").
 *  - Decode attention verified against an exact-softmax oracle (vllm-sm70
 *    page, "Why", Attention bullet). The softmax here is materialised in full
 *    over all visible keys, in fp64, never computed online.
 *  - Speculative positions as a virtual batch (same bullet): query token t of
 *    Tq new tokens sees keys 0 .. L_b - Tq + t, i.e. it is a one-token decode
 *    of a sequence of length L_b - Tq + t + 1.
 *  - Split-K with a log-sum-exp merge (same bullet, "split-K paged decode";
 *    nvllm page, "Acknowledgments", b12x: "split-KV merge"): decode_split
 *    below follows those steps and must equal the plain definition.
 *  - int8 KV cache (vllm-sm70 page, "Why" and model table: int8 KV cache):
 *    symmetric, one fp32 scale per (token, kv head) = max|x| / 127.
 *  - FP8 KV cache (nvllm page, "Acknowledgments": b12x paged attention with
 *    FP8 KV dequantised inline; vllm-sm12x-nvfp4-dflash2 page, "What makes
 *    this stack different": FP8 KV as the common pairing with NVFP4 weights).
 *  - NVFP4 KV cache (vllm-sm12x-nvfp4-dflash2 page, "What makes this stack
 *    different": target weights, draft weights and the KV cache all NVFP4).
 *
 * Readings where the pages are silent (each also listed with the tests):
 *  - seq_lens counts the Tq new tokens, whose K/V are already in the cache;
 *  - query head h uses kv head h / (Hq / Hkv) (contiguous groups);
 *  - a row with no visible key gives out = 0 and lse = -inf;
 *  - int8: s = fp32(amax / 127); code = clamp(rint_half_even(fp32(x / s)),
 *    -127, 127); amax = 0 gives s = 0 and all codes 0;
 *  - the dequantised key/value is code * scale, formed exactly in fp64;
 *  - FP8 is OCP E4M3 (the vllm-sm70 page names an E4M3 buffer; the pages do
 *    not spell out the encoding, so the public OCP 8-bit floating-point
 *    format is taken): sign, 4 exponent bits with bias 7, 3 mantissa bits,
 *    subnormals at exponent 0, no infinities, S.1111.111 is NaN, largest
 *    finite magnitude 448. Scale as for int8 but against 448:
 *    s = fp32(amax / 448); code = the finite E4M3 value nearest to
 *    y = fp32(x / s), ties to the even code, sign taken from y (so values
 *    beyond 448 saturate); amax = 0 gives s = 0 and all codes 0.
 *  - NVFP4 is taken from NVIDIA's public description of the format (the
 *    pages only name it): FP4 E2M1 elements (sign, 2 exponent bits with bias
 *    1, 1 mantissa bit: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6) in blocks of
 *    16 consecutive elements, each block with an E4M3 scale, and a second
 *    fp32 scale, here one per (token, kv head) as for int8 and FP8. For a row
 *    x: S = fp32(amax / (6 * 448)); per block, u = fp32(fp32(amax_b / 6) / S),
 *    s_b = its E4M3 code (the FP8 rule above), d_b = fp32(value(s_b) * S);
 *    code = the E2M1 value nearest to fp32(x / d_b), ties to the even code,
 *    the sign bit that of the quotient (magnitudes past 6 saturate), or 0
 *    where d_b = 0; amax = 0 gives S = 0 and every code and block scale 0.
 *    Dequantised value: value(code) * value(s_b) * S, exact in fp64.
 *    Storage (this library's own; the pages fix none): a block of 16 tokens
 *    and Hkv heads takes 9 * Hkv * D bytes. First the code rows of its
 *    16 * Hkv (token, head) pairs, D/2 bytes each in (token, head) order,
 *    element 2i in the low nibble of byte i; then one plane of D bytes per
 *    head with that head's block scales: the scale of elements 16k .. 16k + 15
 *    of token t at byte 16k + 4 (t mod 4) + t / 4 of the plane.
 *
 *
 * Sparse block-selection decode (vllm-sm70 page: "Changes relative to
 * 1Cat-vLLM", item 8, sparse-decode mean keys refreshed for every request of a
 * decode batch; "Known limitations", the sparse decode selection supports at
 * most 4096 key blocks, a 262,144-token table at 64-token blocks). The pages
 * name the parts, not the rule; the reading taken here:
 *  - a sequence's positions form sparse blocks of SB tokens (a multiple of
 *    the 16-token cache block; 64 on the page): block j = [SB j, SB j + SB)
 *    below L_b, ceil(L_b / SB) <= 4096 of them;
 *  - the mean key of block j for kv head g is the plain mean of its keys
 *    (dequantised for quantised caches) over the block's tokens below L_b;
 *  - the blocks holding any query token (positions L_b - Tq .. L_b - 1: one or
 *    two blocks, as Tq <= 16 <= SB) are always selected ("kept");
 *  - every other block j (all lie before the kept ones) scores
 *    s_j = max over the query rows (t, h) of kv head g of
 *    softmax_scale * q[b, t, h] . mean_key[b, j, g];
 *  - top_blocks - (kept count) of them with the largest scores are
 *    selected, ties to the lower index (at least the kept blocks are
 *    selected; every block when top_blocks >= ceil(L_b / SB));
 *  - row (b, t, h) attends, with the exact softmax, to the keys of the
 *    selected blocks of its kv head at positions p <= L_b - Tq + t (the same
 *    causal rule as the plain decode).
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fPIC -shared (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F32 = 0, OR_BF16 = 1, OR_I8 = 2, OR_FP8 = 3, OR_NVFP4 = 4 };

/* NVFP4 storage bytes per (token, kv head): D/2 of codes, D/16 of block
 * scales (a block of 16 tokens is 16 * Hkv times this). */
int pa_oracle_nvfp4_row_bytes(int D) { return D / 2 + D / 16; }

/* Byte offsets, in an NVFP4 cache, of row `row`'s codes and of the scale of
 * its elements 16k .. 16k + 15 (row = (block * 16 + t) * Hkv + h). */
static int64_t nvfp4_code_offset(int64_t row, int Hkv, int D) {
    const int64_t per = 16 * (int64_t)Hkv, blk = row / per;
    return blk * 9 * Hkv * (int64_t)D + (row % per) * (D / 2);
}
static int64_t nvfp4_scale_offset(int64_t row, int Hkv, int D, int k) {
    const int64_t per = 16 * (int64_t)Hkv, blk = row / per;
    const int64_t t = (row % per) / Hkv, h = row % Hkv;
    return blk * 9 * Hkv * (int64_t)D + per * (D / 2) + h * D + 16 * k + 4 * (t % 4) + t / 4;
}

static float bits_to_float(uint32_t u) {
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static uint32_t float_to_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return u;
}

/* bfloat16 is the top half of an IEEE binary32: widening is exact. */
static double bf16_to_double(uint16_t b) { return (double)bits_to_float((uint32_t)b << 16); }

/* binary32 -> bfloat16, round to nearest, ties to even (finite inputs; a NaN
 * keeps a quiet-NaN pattern). */
static uint16_t float_to_bf16_rne(float f) {
    uint32_t u = float_to_bits(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

/* OCP E4M3: the value a code stands for (NaN for S.1111.111), exact in fp64. */
double pa_oracle_fp8_value(int code) {
    const int sgn = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
    if (e == 15 && m == 7) return NAN;
    const double mag = e == 0 ? ldexp((double)m, -9) : ldexp(1.0 + (double)m / 8.0, e - 7);
    return sgn ? -mag : mag;
}

/* OCP E4M3 code of a finite binary32 y: among the 127 finite magnitudes the
 * one nearest to |y| (distances exact in fp64), a tie going to the even
 * code; the sign bit is y's. Magnitudes past 448 therefore give 448. The
 * magnitudes of codes 0 .. 126 increase with the code, so the two candidates
 * are found by bisection: the largest code whose value is <= |y| and the
 * next one. */
static void fp8_magnitudes(double mag[127]) {
    for (int c = 0; c < 127; ++c) mag[c] = pa_oracle_fp8_value(c);
}

static int fp8_encode_with(const double mag[127], float y) {
    const double a = fabs((double)y);
    int best;
    if (a >= mag[126]) {
        best = 126;
    } else {
        int lo = 0, hi = 126;  /* mag[lo] <= a < mag[hi] */
        while (hi - lo > 1) {
            const int mid = (lo + hi) / 2;
            if (mag[mid] <= a)
                lo = mid;
            else
                hi = mid;
        }
        const double d0 = a - mag[lo], d1 = mag[hi] - a;
        best = d0 < d1 ? lo : d1 < d0 ? hi : ((lo & 1) == 0 ? lo : hi);
    }
    return (signbit(y) ? 0x80 : 0) | best;
}

int pa_oracle_fp8_encode(float y) {
    double mag[127];
    fp8_magnitudes(mag);
    return fp8_encode_with(mag, y);
}

/* FP4 E2M1: the value a 4-bit code stands for. */
double pa_oracle_e2m1_value(int code) {
    const int sgn = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    const double mag = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return sgn ? -mag : mag;
}

/* E2M1 code of a finite binary32 y: the magnitude (codes 0..7, increasing)
 * nearest to |y|, a tie going to the even code; the sign bit is y's. */
int pa_oracle_e2m1_encode(float y) {
    const double a = fabs((double)y);
    int best = 0;
    double bd = a;
    for (int c = 1; c < 8; ++c) {
        const double d = fabs(pa_oracle_e2m1_value(c) - a);
        if (d < bd || (d == bd && (c & 1) == 0)) {
            best = c;
            bd = d;
        }
    }
    return (signbit(y) ? 8 : 0) | best;
}

/* One element of a query or a source row, as the value it stands for. */
static double elem(const void* base, int dtype, int64_t i) {
    switch (dtype) {
    case OR_F32: return (double)((const float*)base)[i];
    case OR_BF16: return bf16_to_double(((const uint16_t*)base)[i]);
    default: return NAN;
    }
}

/* Index of row `row`'s fp32 scale: scales are [num_blocks, Hkv, bs], a kv
 * head's scales of one block contiguous. */
static int64_t scale_index(int64_t row, int Hkv, int bs) {
    const int64_t blk = row / ((int64_t)bs * Hkv), t = (row / Hkv) % bs, h = row % Hkv;
    return (blk * Hkv + h) * bs + t;
}

/* Element d of cache row `row` (row = (block * bs + offset) * Hkv + g),
 * dequantised: for int8, FP8 and NVFP4 the exact product of the code's value
 * and its scales in fp64. */
static double cache_elem(const void* cache, int dtype, const float* scale, int64_t row, int Hkv, int bs, int D,
                         int d) {
    int64_t i = row * (int64_t)D + d;
    switch (dtype) {
    case OR_F32: return (double)((const float*)cache)[i];
    case OR_BF16: return bf16_to_double(((const uint16_t*)cache)[i]);
    case OR_I8: return (double)((const int8_t*)cache)[i] * (double)scale[scale_index(row, Hkv, bs)];
    case OR_FP8: return pa_oracle_fp8_value(((const uint8_t*)cache)[i]) * (double)scale[scale_index(row, Hkv, bs)];
    case OR_NVFP4: {
        const uint8_t* c = (const uint8_t*)cache;
        const uint8_t pair = c[nvfp4_code_offset(row, Hkv, D) + d / 2];
        const int code = (d & 1) ? pair >> 4 : pair & 15;
        return pa_oracle_e2m1_value(code) * pa_oracle_fp8_value(c[nvfp4_scale_offset(row, Hkv, D, d / 16)]) *
               (double)scale[scale_index(row, Hkv, bs)];
    }
    default: return NAN;
    }
}

/* ---------------------------------------------------------------------------
 * Cache writer. For every source token i with slot_mapping[i] >= 0 and every
 * kv head g, row x = src[i, g, :] goes to cache row (slot / bs, slot % bs, g).
 * f32->f32 and bf16->bf16 copy bits; bf16->f32 widens; f32->bf16 rounds to
 * nearest even; ->int8, ->FP8 and ->NVFP4 quantise symmetrically per
 * (token, kv head).
 * Returns 0, or -1 on an unsupported dtype pair.
 */
int pa_oracle_cache_write(const void* k_src, const void* v_src, int src_dtype, const int64_t* slot_mapping,
                          int64_t num_tokens, void* k_cache, void* v_cache, int cache_dtype, float* k_scale,
                          float* v_scale, int64_t num_blocks, int block_size, int Hkv, int D) {
    if (src_dtype != OR_F32 && src_dtype != OR_BF16) return -1;
    if (cache_dtype != OR_F32 && cache_dtype != OR_BF16 && cache_dtype != OR_I8 && cache_dtype != OR_FP8 &&
        cache_dtype != OR_NVFP4)
        return -1;
    if (cache_dtype == OR_NVFP4 && (D % 16 || block_size != 16)) return -1;
    for (int64_t i = 0; i < num_tokens; ++i)
        if (slot_mapping[i] >= num_blocks * block_size) return -2;
    double fp8_mag[127];
    fp8_magnitudes(fp8_mag);
    for (int which = 0; which < 2; ++which) {
        const void* src = which ? v_src : k_src;
        void* cache = which ? v_cache : k_cache;
        float* scale = which ? v_scale : k_scale;
        /* tokens write distinct slots: independent iterations */
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < num_tokens; ++i) {
            int64_t slot = slot_mapping[i];
            if (slot < 0) continue;
            int64_t blk = slot / block_size, off = slot % block_size;
            for (int g = 0; g < Hkv; ++g) {
                int64_t s0 = (i * Hkv + g) * (int64_t)D;
                int64_t row = (blk * block_size + off) * Hkv + g;
                int64_t srow = (blk * Hkv + g) * block_size + off; /* scales [num_blocks, Hkv, bs] */
                int64_t d0 = row * (int64_t)D;
                if (cache_dtype == OR_I8) {
                    float amax = 0.0f;
                    for (int d = 0; d < D; ++d) {
                        float x = (float)elem(src, src_dtype, s0 + d); /* exact: source is f32 or bf16 */
                        float ax = fabsf(x);
                        if (ax > amax) amax = ax;
                    }
                    float s = amax / 127.0f; /* binary32 division, correctly rounded */
                    scale[srow] = s;
                    for (int d = 0; d < D; ++d) {
                        float x = (float)elem(src, src_dtype, s0 + d);
                        int c = 0;
                        if (amax != 0.0f) {
                            float qf = x / s; /* binary32 quotient first */
                            float r = rintf(qf); /* then nearest integer, ties to even */
                            if (r > 127.0f) r = 127.0f;
                            if (r < -127.0f) r = -127.0f;
                            c = (int)r;
                        }
                        ((int8_t*)cache)[d0 + d] = (int8_t)c;
                    }
                } else if (cache_dtype == OR_FP8) {
                    float amax = 0.0f;
                    for (int d = 0; d < D; ++d) {
                        float ax = fabsf((float)elem(src, src_dtype, s0 + d));
                        if (ax > amax) amax = ax;
                    }
                    float s = amax / 448.0f; /* binary32 division, correctly rounded */
                    scale[srow] = s;
                    for (int d = 0; d < D; ++d) {
                        float x = (float)elem(src, src_dtype, s0 + d);
                        int c = 0;
                        if (amax != 0.0f) c = fp8_encode_with(fp8_mag, x / s); /* binary32 quotient first */
                        ((uint8_t*)cache)[d0 + d] = (uint8_t)c;
                    }
                } else if (cache_dtype == OR_NVFP4) {
                    uint8_t* r = (uint8_t*)cache + nvfp4_code_offset(row, Hkv, D);
                    memset(r, 0, (size_t)(D / 2));
                    for (int k = 0; k < D / 16; ++k) ((uint8_t*)cache)[nvfp4_scale_offset(row, Hkv, D, k)] = 0;
                    float amax = 0.0f;
                    for (int d = 0; d < D; ++d) {
                        float ax = fabsf((float)elem(src, src_dtype, s0 + d));
                        if (ax > amax) amax = ax;
                    }
                    const float S = amax / 2688.0f; /* 6 * 448, binary32 division */
                    scale[srow] = S;
                    if (amax != 0.0f) {
                        for (int b0 = 0; b0 < D; b0 += 16) {
                            float bmax = 0.0f;
                            for (int d = b0; d < b0 + 16; ++d) {
                                float ax = fabsf((float)elem(src, src_dtype, s0 + d));
                                if (ax > bmax) bmax = ax;
                            }
                            const float t = bmax / 6.0f;
                            const int sb = fp8_encode_with(fp8_mag, t / S);
                            ((uint8_t*)cache)[nvfp4_scale_offset(row, Hkv, D, b0 / 16)] = (uint8_t)sb;
                            const float db = (float)fp8_mag[sb & 127] * S; /* binary32 product */
                            for (int d = b0; d < b0 + 16; ++d) {
                                const float x = (float)elem(src, src_dtype, s0 + d);
                                const int c = db != 0.0f ? pa_oracle_e2m1_encode(x / db) : 0;
                                r[d / 2] |= (uint8_t)((d & 1) ? c << 4 : c);
                            }
                        }
                    }
                } else if (cache_dtype == src_dtype) {
                    size_t eb = cache_dtype == OR_F32 ? 4 : 2;
                    memcpy((char*)cache + d0 * eb, (const char*)src + s0 * eb, (size_t)D * eb);
                } else if (cache_dtype == OR_F32) { /* bf16 -> f32 */
                    for (int d = 0; d < D; ++d) ((float*)cache)[d0 + d] = (float)elem(src, src_dtype, s0 + d);
                } else { /* f32 -> bf16 */
                    for (int d = 0; d < D; ++d)
                        ((uint16_t*)cache)[d0 + d] = float_to_bf16_rne(((const float*)src)[s0 + d]);
                }
            }
        }
    }
    return 0;
}

/* Shared argument bundle for the two decode entry points. */
typedef struct {
    const void* q;
    int q_dtype, B, Tq, Hq, Hkv, D;
    const void *k_cache, *v_cache;
    int kv_dtype;
    const float *k_scale, *v_scale;
    int block_size;
    const int32_t* block_table;
    int max_blocks;
    const int32_t* seq_lens;
    float softmax_scale;
} args_t;

/* Logits of query row (b, t, h) against its first n keys, in key order. */
static void row_logits(const args_t* a, int b, int t, int h, int64_t n, double* s) {
    int G = a->Hq / a->Hkv, g = h / G;
    const int64_t qoff = (((int64_t)b * a->Tq + t) * a->Hq + h) * a->D;
    for (int64_t j = 0; j < n; ++j) {
        int64_t blk = a->block_table[(int64_t)b * a->max_blocks + j / a->block_size];
        int64_t row = (blk * a->block_size + j % a->block_size) * a->Hkv + g;
        double dot = 0.0;
        for (int d = 0; d < a->D; ++d)
            dot += elem(a->q, a->q_dtype, qoff + d) * cache_elem(a->k_cache, a->kv_dtype, a->k_scale, row, a->Hkv, a->block_size, a->D, d);
        s[j] = (double)a->softmax_scale * dot;
    }
}

static void value_row_axpy(const args_t* a, int b, int g, int64_t j, double w, double* acc) {
    int64_t blk = a->block_table[(int64_t)b * a->max_blocks + j / a->block_size];
    int64_t row = (blk * a->block_size + j % a->block_size) * a->Hkv + g;
    for (int d = 0; d < a->D; ++d) acc[d] += w * cache_elem(a->v_cache, a->kv_dtype, a->v_scale, row, a->Hkv, a->block_size, a->D, d);
}

/* Number of keys query token t of sequence b sees (causal inside the Tq new
 * tokens, which are the last Tq positions of the sequence). */
static int64_t visible_keys(const args_t* a, int b, int t) {
    return (int64_t)a->seq_lens[b] - a->Tq + t + 1;
}

/* Plain definition: out = softmax(scale * q K^T) V over the visible keys,
 * softmax materialised in full. `rows` selects flat row ids
 * ((b * Tq + t) * Hq + h); NULL means every row. out/lse are indexed by the
 * flat row id. */
static void decode_row_plain(const args_t* a, int64_t r, double* out, double* lse) {
    int h = (int)(r % a->Hq), t = (int)((r / a->Hq) % a->Tq), b = (int)(r / ((int64_t)a->Hq * a->Tq));
    int G = a->Hq / a->Hkv, g = h / G;
    double* o = out + r * a->D;
    int64_t n = visible_keys(a, b, t);
    for (int d = 0; d < a->D; ++d) o[d] = 0.0;
    if (n <= 0) {
        lse[r] = -INFINITY;
        return;
    }
    double* s = (double*)malloc((size_t)n * sizeof(double));
    row_logits(a, b, t, h, n, s);
    double M = -INFINITY;
    for (int64_t j = 0; j < n; ++j)
        if (s[j] > M) M = s[j];
    double Z = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        s[j] = exp(s[j] - M); /* unnormalised weight */
        Z += s[j];
    }
    for (int64_t j = 0; j < n; ++j) value_row_axpy(a, b, g, j, s[j], o);
    for (int d = 0; d < a->D; ++d) o[d] /= Z;
    lse[r] = M + log(Z);
    free(s);
}

/* Split path: keys of a row split into partitions [iP, (i+1)P); each keeps
 * its own max m_i, sum l_i and normalised output o_i; the merge weighs o_i by
 * l_i * exp(m_i - M). Exact in real arithmetic, so it must equal the plain
 * definition up to rounding. */
static void decode_row_split(const args_t* a, int64_t r, int P, double* out, double* lse) {
    int h = (int)(r % a->Hq), t = (int)((r / a->Hq) % a->Tq), b = (int)(r / ((int64_t)a->Hq * a->Tq));
    int G = a->Hq / a->Hkv, g = h / G;
    double* o = out + r * a->D;
    int64_t n = visible_keys(a, b, t);
    for (int d = 0; d < a->D; ++d) o[d] = 0.0;
    if (n <= 0) {
        lse[r] = -INFINITY;
        return;
    }
    int64_t np = (n + P - 1) / P;
    double* s = (double*)malloc((size_t)n * sizeof(double));
    double* m = (double*)malloc((size_t)np * sizeof(double));
    double* l = (double*)malloc((size_t)np * sizeof(double));
    double* op = (double*)calloc((size_t)np * a->D, sizeof(double));
    row_logits(a, b, t, h, n, s);
    for (int64_t i = 0; i < np; ++i) {
        int64_t j0 = i * P, j1 = j0 + P < n ? j0 + P : n;
        m[i] = -INFINITY;
        for (int64_t j = j0; j < j1; ++j)
            if (s[j] > m[i]) m[i] = s[j];
        l[i] = 0.0;
        for (int64_t j = j0; j < j1; ++j) {
            double w = exp(s[j] - m[i]);
            l[i] += w;
            value_row_axpy(a, b, g, j, w, op + i * a->D);
        }
        for (int d = 0; d < a->D; ++d) op[i * a->D + d] /= l[i];
    }
    double M = -INFINITY;
    for (int64_t i = 0; i < np; ++i)
        if (m[i] > M) M = m[i];
    double W = 0.0;
    for (int64_t i = 0; i < np; ++i) {
        double w = l[i] * exp(m[i] - M);
        W += w;
        for (int d = 0; d < a->D; ++d) o[d] += w * op[i * a->D + d];
    }
    for (int d = 0; d < a->D; ++d) o[d] /= W;
    lse[r] = M + log(W);
    free(s);
    free(m);
    free(l);
    free(op);
}

static int check_args(const args_t* a) {
    if (!a->q || !a->k_cache || !a->v_cache || !a->block_table || !a->seq_lens) return -1;
    if (a->B < 0 || a->Tq < 1 || a->Hq < 1 || a->Hkv < 1 || a->D < 1 || a->block_size < 1) return -2;
    if (a->Hq % a->Hkv) return -2;
    if (a->kv_dtype == OR_NVFP4 && (a->D % 16 || a->block_size != 16)) return -2;
    if ((a->kv_dtype == OR_I8 || a->kv_dtype == OR_FP8 || a->kv_dtype == OR_NVFP4) && (!a->k_scale || !a->v_scale))
        return -1;
    return 0;
}

static int run(const args_t* a, const int64_t* rows, int64_t num_rows, int split_P, double* out, double* lse,
               int nthreads) {
    int rc = check_args(a);
    if (rc) return rc;
    int64_t total = (int64_t)a->B * a->Tq * a->Hq;
    int64_t cnt = rows ? num_rows : total;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t k = 0; k < cnt; ++k) {
        int64_t r = rows ? rows[k] : k;
        if (r < 0 || r >= total) continue;
        if (split_P > 0)
            decode_row_split(a, r, split_P, out, lse);
        else
            decode_row_plain(a, r, out, lse);
    }
    return 0;
}

#define ORACLE_ARGS                                                                                            \
    const void *q, int q_dtype, int B, int Tq, int Hq, int Hkv, int D, const void *k_cache, const void *v_cache, \
        int kv_dtype, const float *k_scale, const float *v_scale, int block_size, const int32_t *block_table,    \
        int max_blocks, const int32_t *seq_lens, float softmax_scale
#define ORACLE_PACK                                                                                                \
    args_t a = {q,       q_dtype,  B,          Tq,         Hq,         Hkv,      D, k_cache, v_cache, kv_dtype, \
                k_scale, v_scale,  block_size, block_table, max_blocks, seq_lens, softmax_scale}

/* out: fp64 [B*Tq*Hq, D]; lse: fp64 [B*Tq*Hq]. rows: optional flat row ids. */
int pa_oracle_decode(ORACLE_ARGS, const int64_t* rows, int64_t num_rows, double* out, double* lse, int nthreads) {
    ORACLE_PACK;
    return run(&a, rows, num_rows, 0, out, lse, nthreads);
}

int pa_oracle_decode_split(ORACLE_ARGS, int partition_size, const int64_t* rows, int64_t num_rows, double* out,
                           double* lse, int nthreads) {
    ORACLE_PACK;
    if (partition_size < 1) return -2;
    return run(&a, rows, num_rows, partition_size, out, lse, nthreads);
}

/* ------------------------------------------------------------------------
 * Sparse block-selection decode (the reading in the header).
 * ---------------------------------------------------------------------- */

/* Mean keys: out[((b * max_sblocks + j) * Hkv + g) * D + d] (fp64) for every
 * sparse block j < ceil(L_b / SB) of every sequence; other entries untouched.
 * Returns -2 when a sequence has more than max_sblocks blocks. */
int pa_oracle_sparse_mean_keys(const void* k_cache, int kv_dtype, const float* k_scale, int block_size, int Hkv,
                               int D, const int32_t* block_table, int max_blocks, const int32_t* seq_lens, int B,
                               int sparse_block, int max_sblocks, double* out) {
    if (!k_cache || !block_table || !seq_lens || !out) return -1;
    if (sparse_block < block_size || sparse_block % block_size || B < 0 || Hkv < 1 || D < 1) return -2;
    for (int b = 0; b < B; ++b) {
        const int64_t L = seq_lens[b];
        const int64_t nsb = (L + sparse_block - 1) / sparse_block;
        if (nsb > max_sblocks) return -2;
        for (int64_t j = 0; j < nsb; ++j) {
            const int64_t p0 = j * sparse_block, p1 = p0 + sparse_block < L ? p0 + sparse_block : L;
            for (int g = 0; g < Hkv; ++g) {
                double* m = out + ((b * (int64_t)max_sblocks + j) * Hkv + g) * D;
                for (int d = 0; d < D; ++d) m[d] = 0.0;
                for (int64_t p = p0; p < p1; ++p) {
                    const int64_t blk = block_table[(int64_t)b * max_blocks + p / block_size];
                    const int64_t row = (blk * block_size + p % block_size) * Hkv + g;
                    for (int d = 0; d < D; ++d)
                        m[d] += cache_elem(k_cache, kv_dtype, k_scale, row, Hkv, block_size, D, d);
                }
                for (int d = 0; d < D; ++d) m[d] /= (double)(p1 - p0);
            }
        }
    }
    return 0;
}

/* First sparse block holding a query token of sequence b (the kept blocks
 * run from it to the last block); the number of blocks is ceil(L / SB). */
static int64_t first_kept_block(int64_t L, int Tq, int sparse_block) {
    int64_t first_q = L - Tq;
    if (first_q < 0) first_q = 0;
    return first_q / sparse_block;
}

/* Selection for every (b, g): selected[(b * Hkv + g) * max_sel + i] = the
 * i-th selected sparse block in increasing order, -1 after the last; count
 * [b * Hkv + g] = how many. scores[(b * Hkv + g) * max_sblocks + j] = s_j of
 * every candidate block (NaN for kept blocks and past the end). mean_k:
 * fp64 [B, max_sblocks, Hkv, D]. Returns -2 if max_sel is too small. */
int pa_oracle_sparse_select(const void* q, int q_dtype, int B, int Tq, int Hq, int Hkv, int D, float softmax_scale,
                            const double* mean_k, int max_sblocks, const int32_t* seq_lens, int sparse_block,
                            int top_blocks, int max_sel, int32_t* selected, int32_t* count, double* scores) {
    if (!q || !mean_k || !seq_lens || !selected || !count || !scores) return -1;
    if (Hq % Hkv || top_blocks < 1 || sparse_block < 1) return -2;
    const int G = Hq / Hkv;
    for (int b = 0; b < B; ++b) {
        const int64_t L = seq_lens[b];
        const int64_t nsb = (L + sparse_block - 1) / sparse_block;
        if (nsb > max_sblocks) return -2;
        const int64_t kept0 = L > 0 ? first_kept_block(L, Tq, sparse_block) : 0;
        for (int g = 0; g < Hkv; ++g) {
            double* sc = scores + ((int64_t)b * Hkv + g) * max_sblocks;
            int32_t* sel = selected + ((int64_t)b * Hkv + g) * max_sel;
            for (int64_t j = 0; j < max_sblocks; ++j) sc[j] = NAN;
            for (int i = 0; i < max_sel; ++i) sel[i] = -1;
            /* candidate scores: the largest over the group's query rows */
            for (int64_t j = 0; j < kept0; ++j) {
                const double* m = mean_k + (((int64_t)b * max_sblocks + j) * Hkv + g) * D;
                double best = -INFINITY;
                for (int t = 0; t < Tq; ++t)
                    for (int hh = 0; hh < G; ++hh) {
                        const int64_t qoff = (((int64_t)b * Tq + t) * Hq + g * G + hh) * D;
                        double dot = 0.0;
                        for (int d = 0; d < D; ++d) dot += elem(q, q_dtype, qoff + d) * m[d];
                        const double v = (double)softmax_scale * dot;
                        if (v > best) best = v;
                    }
                sc[j] = best;
            }
            /* take the top candidates one at a time: the largest score, the
             * lower index on a tie */
            int64_t want = (int64_t)top_blocks - (nsb - kept0);
            if (want < 0) want = 0;
            if (want > kept0) want = kept0;
            char* taken = (char*)calloc((size_t)(nsb > 0 ? nsb : 1), 1);
            for (int64_t k = 0; k < want; ++k) {
                int64_t arg = -1;
                for (int64_t j = 0; j < kept0; ++j)
                    if (!taken[j] && (arg < 0 || sc[j] > sc[arg])) arg = j;
                taken[arg] = 1;
            }
            for (int64_t j = kept0; j < nsb; ++j) taken[j] = 1;
            int64_t n = 0;
            for (int64_t j = 0; j < nsb; ++j)
                if (taken[j]) {
                    if (n >= max_sel) {
                        free(taken);
                        return -2;
                    }
                    sel[n++] = (int32_t)j;
                }
            count[(int64_t)b * Hkv + g] = (int32_t)n;
            free(taken);
        }
    }
    return 0;
}

/* Attention of row r over the keys of the listed sparse blocks of its kv head
 * that lie at positions <= L_b - Tq + t, softmax materialised in full, keys
 * taken in increasing position order. */
static void decode_row_subset(const args_t* a, int64_t r, const int32_t* selected, const int32_t* count, int max_sel,
                              int sparse_block, double* out, double* lse) {
    const int h = (int)(r % a->Hq), t = (int)((r / a->Hq) % a->Tq), b = (int)(r / ((int64_t)a->Hq * a->Tq));
    const int G = a->Hq / a->Hkv, g = h / G;
    double* o = out + r * a->D;
    const int64_t n = visible_keys(a, b, t), L = a->seq_lens[b];
    const int32_t* sel = selected + ((int64_t)b * a->Hkv + g) * max_sel;
    const int cnt = count[(int64_t)b * a->Hkv + g];
    for (int d = 0; d < a->D; ++d) o[d] = 0.0;
    /* visible positions of the selected blocks */
    int64_t m = 0;
    int64_t* pos = (int64_t*)malloc(((size_t)cnt * sparse_block + 1) * sizeof(int64_t));
    for (int i = 0; i < cnt; ++i)
        for (int64_t p = (int64_t)sel[i] * sparse_block; p < (int64_t)(sel[i] + 1) * sparse_block; ++p)
            if (p < n && p < L) pos[m++] = p;
    if (m == 0) {
        lse[r] = -INFINITY;
        free(pos);
        return;
    }
    const int64_t qoff = (((int64_t)b * a->Tq + t) * a->Hq + h) * a->D;
    double* s = (double*)malloc((size_t)m * sizeof(double));
    for (int64_t k = 0; k < m; ++k) {
        const int64_t blk = a->block_table[(int64_t)b * a->max_blocks + pos[k] / a->block_size];
        const int64_t row = (blk * a->block_size + pos[k] % a->block_size) * a->Hkv + g;
        double dot = 0.0;
        for (int d = 0; d < a->D; ++d)
            dot += elem(a->q, a->q_dtype, qoff + d) *
                   cache_elem(a->k_cache, a->kv_dtype, a->k_scale, row, a->Hkv, a->block_size, a->D, d);
        s[k] = (double)a->softmax_scale * dot;
    }
    double M = -INFINITY;
    for (int64_t k = 0; k < m; ++k)
        if (s[k] > M) M = s[k];
    double Z = 0.0;
    for (int64_t k = 0; k < m; ++k) {
        s[k] = exp(s[k] - M);
        Z += s[k];
    }
    for (int64_t k = 0; k < m; ++k) value_row_axpy(a, b, g, pos[k], s[k], o);
    for (int d = 0; d < a->D; ++d) o[d] /= Z;
    lse[r] = M + log(Z);
    free(s);
    free(pos);
}

/* Decode over the listed sparse blocks (selected / count as written by
 * pa_oracle_sparse_select, or a selection read back from the GPU). */
int pa_oracle_decode_subset(ORACLE_ARGS, const int32_t* selected, const int32_t* count, int max_sel,
                            int sparse_block, double* out, double* lse, int nthreads) {
    ORACLE_PACK;
    int rc = check_args(&a);
    if (rc) return rc;
    if (!selected || !count) return -1;
    if (sparse_block < 1 || max_sel < 0) return -2;
    const int64_t total = (int64_t)B * Tq * Hq;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < total; ++r) decode_row_subset(&a, r, selected, count, max_sel, sparse_block, out, lse);
    return 0;
}

int pa_oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
