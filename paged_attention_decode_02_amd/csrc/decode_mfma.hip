// Split-K paged decode on the matrix cores (gfx950 MFMA) for query tiles of
// 16 rows or more: speculative verification, where each sequence brings Tq
// new query tokens (8 target tokens per verification step on the
// vllm-sm12x-nvfp4-dflash2 page, "What makes this stack different") and the
// G query heads of a kv head times the Tq tokens form G*Tq rows that share
// every key and value row. The vllm-sm70 page ("Why", Attention bullet) runs
// such speculative positions as a virtual batch of one-token decodes; here
// all rows of a kv head are one MFMA operand, so the KV is read once.
//
// Workgroup = 4 waves for one split-K partition of one kv head g of one
// sequence b and up to 16*NT rows r = t*G + h' (query token t, head g*G + h').
// Row r sees keys 0 .. L_b - Tq + t (causal inside the Tq new tokens).
// Every wave computes the whole score tile of each 16-token block,
//   S^T[token][row] = K[token][:] . Q[row][:]   (v_mfma_f32_16x16x32 bf16 / f16),
// whose result layout (lane l: tokens 4*(l/16)+i of row l%16) is exactly the
// A-operand layout of the PV product, so probabilities go straight from the
// softmax into
//   O[row][d] += P[row][token] V[token][d]      (v_mfma_f32_16x16x16 bf16 / f16)
// where wave w owns output dims [w*D/4, (w+1)*D/4). The V operand needs 4
// consecutive tokens of one dim per lane: lanes load 4 dims of one token and a
// 4x4 transpose inside each lane quad (DPP + byte permutes) regroups them.
// Queries (as MFMA B operands) are staged once per workgroup in LDS.
// int8 caches: codes become f16 (1024 + code + 128) by a byte permute, queries
// are scaled into f16 by a power of two, probabilities times the value scale
// are f16; the code bias is removed once per row (query sums for the scores,
// probability sums for the outputs).
// Softmax: log2 units against a per-row reference raised only when beaten by
// 2^8 (as in the vector-ALU decode).
#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr int kW = 4;  // waves per workgroup
constexpr uint32_t kMagic = 0x64646464u;
constexpr float kCodeBias = 1152.0f;  // 1024 + 128

__device__ __forceinline__ uint32_t f16pair_lo(uint32_t u) { return __builtin_amdgcn_perm(kMagic, u, 0x04010400u); }
__device__ __forceinline__ uint32_t f16pair_hi(uint32_t u) { return __builtin_amdgcn_perm(kMagic, u, 0x04030402u); }

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
}

__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) | ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
}

// 4x4 transpose of 16-bit elements inside a lane quad. Lane i (= lane & 3)
// holds elements (i, 0..3) of a 4x4 tile as two dwords; afterwards lane j
// holds elements (0..3, j).
__device__ __forceinline__ u32x2 quad_transpose16(u32x2 w, int i) {
    const int b1 = (i >> 1) & 1, b0 = i & 1;
    const uint32_t send = b1 ? w.x : w.y;
    const uint32_t recv = dpp_u32<kDppQuadXor2>(send);
    const uint32_t A = b1 ? recv : w.x;
    const uint32_t B = b1 ? w.y : recv;
    const uint32_t pA = dpp_u32<kDppQuadXor1>(A);
    const uint32_t pB = dpp_u32<kDppQuadXor1>(B);
    const uint32_t sel = b0 ? 0x03020706u : 0x05040100u;
    u32x2 r;
    r.x = __builtin_amdgcn_perm(pA, A, sel);
    r.y = __builtin_amdgcn_perm(pB, B, sel);
    return r;
}

// Same for bytes: lane i holds (i, 0..3) in one dword, afterwards lane j holds (0..3, j).
__device__ __forceinline__ uint32_t quad_transpose8(uint32_t w, int i) {
    const int b1 = (i >> 1) & 1, b0 = i & 1;
    const uint32_t recv = dpp_u32<kDppQuadXor2>(w);
    const uint32_t u = __builtin_amdgcn_perm(recv, w, b1 ? 0x03020706u : 0x05040100u);
    const uint32_t pu = dpp_u32<kDppQuadXor1>(u);
    return __builtin_amdgcn_perm(pu, u, b0 ? 0x03070105u : 0x06020400u);
}

}  // namespace

template <int KVT, int D, int NT, int QS>
__global__ __launch_bounds__(64 * kW) void decode_mfma_kernel(DecodeParams p) {
    static_assert(KVT == KV_BF16 || KVT == KV_I8, "bf16 or int8 caches");
    constexpr bool I8 = KVT == KV_I8;
    constexpr int E = Elt<KVT>::bytes;
    constexpr int KS = D / 32;   // k-steps of the score product
    constexpr int DW = D / kW;   // output dims per wave
    constexpr int NDT = DW / 16; // 16-wide output tiles per wave
    constexpr int NQ = QS == 2 ? 2 : 1;  // query parts (hi, lo) for fp32 queries

    // queries as B operands: [part][tile][kstep][lane] of 16 bytes
    __shared__ __align__(16) u32x4 qlds[NQ][NT][KS][64];
    __shared__ float qcorr[NT * 16];           // int8: 1152 * sum_d q'[row]
    __shared__ float redist[kW][NT][16];       // per-wave row values moved to the output layout
    __shared__ float red[kW];

    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int l16 = lane & 15, lg = lane >> 4;

    int wg = blockIdx.x;
    const int part = wg % p.NP;
    wg /= p.NP;
    const int rc = wg % p.nchunk;
    wg /= p.nchunk;
    const int g = wg % p.Hkv;
    const int b = wg / p.Hkv;

    const int G = p.G, Tq = p.Tq, R = G * Tq;
    const int row0 = rc * 16 * NT;
    const int L = p.seq_lens[b];
    // keys visible to the last (largest t) row of this chunk
    const int rlast = min(R, row0 + 16 * NT) - 1;
    const int n_chunk = L - Tq + rlast / G + 1;
    const int start = part * p.P;

    auto row_out = [&](int r) -> int64_t {  // flat (b, t, h) row id of chunk row r
        const int t = r / G, hh = r % G;
        return ((int64_t)b * Tq + t) * p.Hq + g * G + hh;
    };

    if (start >= n_chunk) {
        if (p.NP == 1) {
            for (int r = row0; r <= rlast; ++r) {
                const int64_t rid = row_out(r);
                for (int d = threadIdx.x; d < D; d += 64 * kW) {
                    if (p.out_bf16)
                        reinterpret_cast<uint16_t*>(p.out)[rid * D + d] = 0;
                    else
                        reinterpret_cast<float*>(p.out)[rid * D + d] = 0.0f;
                }
                if (p.lse != nullptr && threadIdx.x == 0) p.lse[rid] = -INFINITY;
            }
        }
        return;
    }
    const int end = min(start + p.P, n_chunk);

    // ----------------------------------------------------- stage the queries
    // entry (tile, ks, l): row row0 + 16 tile + l%16, dims 32 ks + 8 (l/16) .. +7
    float qmax = 0.0f;
    for (int e = threadIdx.x; e < NT * KS * 64; e += 64 * kW) {
        const int l = e & 63, ks = (e >> 6) % KS, tile = (e >> 6) / KS;
        const int r = row0 + 16 * tile + (l & 15);
        const int d0 = 32 * ks + 8 * (l >> 4);
        float x[8];
        if (r < R) {
            const int64_t off = row_out(r) * D + d0;
            if constexpr (QS == 1) {
                Raw<16> raw;
                load_raw<16>(raw, reinterpret_cast<const uint16_t*>(p.q) + off);
#pragma unroll
                for (int k = 0; k < 8; ++k) x[k] = elem_f32<KV_BF16>(raw, k);
            } else {
                Raw<32> raw;
                load_raw<32>(raw, reinterpret_cast<const float*>(p.q) + off);
#pragma unroll
                for (int k = 0; k < 8; ++k) x[k] = elem_f32<KV_F32>(raw, k);
            }
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) x[k] = 0.0f;
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) qmax = fmaxf(qmax, fabsf(x[k]));
        if constexpr (!I8) {
            u32x4 hi, lo;
            hi.x = pack_bf16x2(x[0], x[1]);
            hi.y = pack_bf16x2(x[2], x[3]);
            hi.z = pack_bf16x2(x[4], x[5]);
            hi.w = pack_bf16x2(x[6], x[7]);
            qlds[0][tile][ks][l] = hi;
            if constexpr (QS == 2) {
                const uint32_t hw[4] = {hi.x, hi.y, hi.z, hi.w};
                uint32_t lw[4];
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    lw[k] = pack_bf16x2(x[2 * k] - bf16_to_f32((uint16_t)hw[k]),
                                        x[2 * k + 1] - bf16_to_f32((uint16_t)(hw[k] >> 16)));
                lo.x = lw[0];
                lo.y = lw[1];
                lo.z = lw[2];
                lo.w = lw[3];
                qlds[NQ - 1][tile][ks][l] = lo;
            }
        }
    }
    float qpost = p.qk_scale_log2;
    float qscale = 1.0f;
    if constexpr (I8) {
        // one power of two for the workgroup puts max|q| in [2^14, 2^15)
        qmax = wave_max(qmax);
        if (lane == 0) red[wv] = qmax;
        __syncthreads();
        qmax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        const int e2 = qmax > 0.0f ? 14 - ilogbf(qmax) : 0;
        qscale = ldexpf(1.0f, e2);
        qpost = ldexpf(p.qk_scale_log2, -e2);
        for (int e = threadIdx.x; e < NT * KS * 64; e += 64 * kW) {
            const int l = e & 63, ks = (e >> 6) % KS, tile = (e >> 6) / KS;
            const int r = row0 + 16 * tile + (l & 15);
            const int d0 = 32 * ks + 8 * (l >> 4);
            float x[8];
            if (r < R) {
                const int64_t off = row_out(r) * D + d0;
                if constexpr (QS == 1) {
                    Raw<16> raw;
                    load_raw<16>(raw, reinterpret_cast<const uint16_t*>(p.q) + off);
#pragma unroll
                    for (int k = 0; k < 8; ++k) x[k] = elem_f32<KV_BF16>(raw, k) * qscale;
                } else {
                    Raw<32> raw;
                    load_raw<32>(raw, reinterpret_cast<const float*>(p.q) + off);
#pragma unroll
                    for (int k = 0; k < 8; ++k) x[k] = elem_f32<KV_F32>(raw, k) * qscale;
                }
            } else {
#pragma unroll
                for (int k = 0; k < 8; ++k) x[k] = 0.0f;
            }
            u32x4 hi;
            hi.x = pack_f16x2(x[0], x[1]);
            hi.y = pack_f16x2(x[2], x[3]);
            hi.z = pack_f16x2(x[4], x[5]);
            hi.w = pack_f16x2(x[6], x[7]);
            qlds[0][tile][ks][l] = hi;
            if constexpr (QS == 2) {
                const uint32_t hw[4] = {hi.x, hi.y, hi.z, hi.w};
                uint32_t lw[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const float h0 = (float)__builtin_bit_cast(_Float16, (uint16_t)hw[k]);
                    const float h1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(hw[k] >> 16));
                    lw[k] = pack_f16x2(x[2 * k] - h0, x[2 * k + 1] - h1);
                }
                u32x4 lo;
                lo.x = lw[0];
                lo.y = lw[1];
                lo.z = lw[2];
                lo.w = lw[3];
                qlds[NQ - 1][tile][ks][l] = lo;
            }
        }
    }
    __syncthreads();
    if constexpr (I8) {
        // row sums of the f16 queries (hi + lo) for the code bias
        for (int e = threadIdx.x; e < NT * 16; e += 64 * kW) {
            const int tile = e / 16, rl = e % 16;
            float s = 0.0f;
            for (int ks = 0; ks < KS; ++ks)
                for (int grp = 0; grp < 4; ++grp)
                    for (int part2 = 0; part2 < NQ; ++part2) {
                        const u32x4 v = qlds[part2][tile][ks][grp * 16 + rl];
                        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
                        for (int k = 0; k < 4; ++k)
                            s += (float)__builtin_bit_cast(_Float16, (uint16_t)w4[k]) +
                                 (float)__builtin_bit_cast(_Float16, (uint16_t)(w4[k] >> 16));
                    }
            qcorr[e] = kCodeBias * s;
        }
        __syncthreads();
    }

    // --------------------------------------------------------- per-row state
    // score layout: lane holds row 16*tile + l16 (tokens 4*lg + i of a block)
    int nvis[NT];      // keys visible to the lane's row in each tile
    float mref[NT], lpart[NT], spart[NT], corr[NT];
#pragma unroll
    for (int tile = 0; tile < NT; ++tile) {
        const int r = row0 + 16 * tile + l16;
        nvis[tile] = r < R ? min(end, L - Tq + r / G + 1) : 0;
        mref[tile] = -INFINITY;
        lpart[tile] = 0.0f;
        spart[tile] = 0.0f;
        corr[tile] = I8 ? qcorr[16 * tile + l16] : 0.0f;
    }
    // output layout: lane holds rows 16*tile + 4*lg + i, dim wv*DW + 16*ndt + l16
    f32x4 o[NT][NDT];
#pragma unroll
    for (int tile = 0; tile < NT; ++tile)
#pragma unroll
        for (int nd = 0; nd < NDT; ++nd) o[tile][nd] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    const int32_t* table = p.block_table + (int64_t)b * p.max_blocks;
    const int64_t tok_stride = (int64_t)p.Hkv * D * E;
    const char* kbase = reinterpret_cast<const char*>(p.k_cache) + (int64_t)g * D * E;
    const char* vbase = reinterpret_cast<const char*>(p.v_cache) + (int64_t)g * D * E;
    const int j0 = start / kBlockSize, jend = (end + kBlockSize - 1) / kBlockSize;

    // int8: probabilities times value scales are kept below 2^15 (f16) by 2^vsh
    float vsh = 1.0f, vsh_inv = 1.0f;
    if constexpr (I8) {
        float vmax = 0.0f;
        for (int j = j0 + (threadIdx.x >> 4); j < jend; j += 4 * kW) {
            const int pos = j * kBlockSize + l16;
            if (pos < end) vmax = fmaxf(vmax, p.v_scale[((int64_t)table[j] * kBlockSize + l16) * p.Hkv + g]);
        }
        vmax = wave_max(vmax);
        __syncthreads();
        if (lane == 0) red[wv] = vmax;
        __syncthreads();
        vmax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        const int e2 = vmax > 0.0f ? 6 - ilogbf(vmax) : 0;
        vsh = ldexpf(1.0f, e2);
        vsh_inv = ldexpf(1.0f, -e2);
    }

    constexpr int KB = 8 * E;  // key bytes per lane per k-step
    constexpr int VB = 4 * E;  // value bytes per lane per output tile
    Raw<KB> kr[KS];
    Raw<VB> vr[NDT];
    const int vtok = 4 * lg + (l16 & 3);  // token this lane loads for the V transpose
    const int vdim = wv * DW + 4 * (l16 >> 2);
    auto load_k = [&](int64_t ph) {
        const char* base = kbase + (ph * kBlockSize + l16) * tok_stride + 8 * lg * E;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) load_raw<KB, true>(kr[ks], base + 32 * ks * E);
    };
    auto load_v = [&](int64_t ph) {
        const char* base = vbase + (ph * kBlockSize + vtok) * tok_stride + vdim * E;
#pragma unroll
        for (int nd = 0; nd < NDT; ++nd) load_raw<VB, true>(vr[nd], base + 16 * nd * E);
    };

    int64_t phys = table[j0];
    load_k(phys);
    for (int j = j0; j < jend; ++j) {
        const int pos0 = j * kBlockSize;
        // int8 scales of the lane's four tokens first: a load issued after the
        // prefetches would make its wait drain them (in-order counting)
        float kraw[4], vraw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            kraw[i] = 1.0f;
            vraw[i] = 1.0f;
            if constexpr (I8) {
                kraw[i] = p.k_scale[(phys * kBlockSize + 4 * lg + i) * p.Hkv + g];
                vraw[i] = p.v_scale[(phys * kBlockSize + 4 * lg + i) * p.Hkv + g];
            }
        }
        load_v(phys);
        const int64_t phys_next = j + 1 < jend ? (int64_t)table[j + 1] : phys;

        // ---------------------------------------------------- scores S^T
        f32x4 s[NT];
#pragma unroll
        for (int tile = 0; tile < NT; ++tile) s[tile] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if constexpr (I8) {
                const uint32_t u0 = kr[ks].w[0] ^ 0x80808080u, u1 = kr[ks].w[1] ^ 0x80808080u;
                u32x4 a;
                a.x = f16pair_lo(u0);
                a.y = f16pair_hi(u0);
                a.z = f16pair_lo(u1);
                a.w = f16pair_hi(u1);
                const f16x8 av = __builtin_bit_cast(f16x8, a);
#pragma unroll
                for (int tile = 0; tile < NT; ++tile)
#pragma unroll
                    for (int q2 = 0; q2 < NQ; ++q2)
                        s[tile] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            av, __builtin_bit_cast(f16x8, qlds[q2][tile][ks][lane]), s[tile], 0, 0, 0);
            } else {
                u32x4 a;
                a.x = kr[ks].w[0];
                a.y = kr[ks].w[1];
                a.z = kr[ks].w[2];
                a.w = kr[ks].w[3];
                const bf16x8 av = __builtin_bit_cast(bf16x8, a);
#pragma unroll
                for (int tile = 0; tile < NT; ++tile)
#pragma unroll
                    for (int q2 = 0; q2 < NQ; ++q2)
                        s[tile] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            av, __builtin_bit_cast(bf16x8, qlds[q2][tile][ks][lane]), s[tile], 0, 0, 0);
            }
        }
        // unconditional (the last iteration re-reads its own block): a load under
        // a branch makes the wait counts after the join conservative
        load_k(phys_next);

        // ---------------------------------------------------- softmax
        float ksc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ksc[i] = qpost;
            if constexpr (I8) ksc[i] *= kraw[i];
        }
        bool raise = false;
        float sc[NT][4];
#pragma unroll
        for (int tile = 0; tile < NT; ++tile)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool ok = pos0 + 4 * lg + i < nvis[tile];
                sc[tile][i] = ok ? (s[tile][i] - corr[tile]) * ksc[i] : -INFINITY;
                raise |= sc[tile][i] > mref[tile] + 8.0f;
            }
        if (__builtin_amdgcn_ballot_w64(raise) != 0) {
            // raise the references of the rows to their block maxima; rescale
            float alpha[NT];
#pragma unroll
            for (int tile = 0; tile < NT; ++tile) {
                float bm = fmaxf(fmaxf(sc[tile][0], sc[tile][1]), fmaxf(sc[tile][2], sc[tile][3]));
                bm = fmaxf(bm, __shfl_xor(bm, 16));
                bm = fmaxf(bm, __shfl_xor(bm, 32));
                const float mn = fmaxf(mref[tile], bm);
                const float base = mn == -INFINITY ? 0.0f : mn;
                alpha[tile] = exp2_guarded(mref[tile] - base);
                mref[tile] = mn;
                lpart[tile] *= alpha[tile];
                spart[tile] *= alpha[tile];
                if (lg == 0) redist[wv][tile][l16] = alpha[tile];
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
            for (int tile = 0; tile < NT; ++tile) {
                f32x4 a4;
#pragma unroll
                for (int i = 0; i < 4; ++i) a4[i] = redist[wv][tile][4 * lg + i];
#pragma unroll
                for (int nd = 0; nd < NDT; ++nd) o[tile][nd] *= a4;
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
        float vsc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            vsc[i] = 1.0f;
            if constexpr (I8) {
                const bool ok = pos0 + 4 * lg + i < end;
                vsc[i] = ok ? vraw[i] * vsh : 0.0f;
            }
        }
        uint32_t pa[NT][2];
#pragma unroll
        for (int tile = 0; tile < NT; ++tile) {
            const float base = mref[tile] == -INFINITY ? 0.0f : mref[tile];
            float pr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pr[i] = sc[tile][i] == -INFINITY ? 0.0f : exp2f(sc[tile][i] - base);
                lpart[tile] += pr[i];
            }
            if constexpr (I8) {
                float ph[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    ph[i] = (float)(_Float16)(pr[i] * vsc[i]);
                    spart[tile] += ph[i];
                }
                pa[tile][0] = pack_f16x2(ph[0], ph[1]);
                pa[tile][1] = pack_f16x2(ph[2], ph[3]);
            } else {
                pa[tile][0] = pack_bf16x2(pr[0], pr[1]);
                pa[tile][1] = pack_bf16x2(pr[2], pr[3]);
            }
        }

        // ---------------------------------------------------- PV
        const bool partial = pos0 + kBlockSize > end;  // tokens past the end may hold anything
#pragma unroll
        for (int nd = 0; nd < NDT; ++nd) {
            u32x2 bw;
            if constexpr (I8) {
                const uint32_t tw = quad_transpose8(vr[nd].w[0], l16 & 3) ^ 0x80808080u;
                bw.x = f16pair_lo(tw);
                bw.y = f16pair_hi(tw);
            } else {
                u32x2 w;
                w.x = vr[nd].w[0];
                w.y = vr[nd].w[1];
                bw = quad_transpose16(w, l16 & 3);
                if (partial) {
                    // element k of the operand is token 4*lg + k
                    const int t0 = pos0 + 4 * lg;
                    bw.x = (t0 + 0 < end ? bw.x & 0x0000FFFFu : 0u) | (t0 + 1 < end ? bw.x & 0xFFFF0000u : 0u);
                    bw.y = (t0 + 2 < end ? bw.y & 0x0000FFFFu : 0u) | (t0 + 3 < end ? bw.y & 0xFFFF0000u : 0u);
                }
            }
#pragma unroll
            for (int tile = 0; tile < NT; ++tile) {
                u32x2 av;
                av.x = pa[tile][0];
                av.y = pa[tile][1];
                if constexpr (I8)
                    o[tile][nd] = __builtin_amdgcn_mfma_f32_16x16x16f16(
                        __builtin_bit_cast(f16x4, av), __builtin_bit_cast(f16x4, bw), o[tile][nd], 0, 0, 0);
                else
                    o[tile][nd] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                        __builtin_bit_cast(bf16x4, av), __builtin_bit_cast(bf16x4, bw), o[tile][nd], 0, 0, 0);
            }
        }
        phys = phys_next;
    }

    // ------------------------------------------------------------ epilogue
    // row sums over the four lane groups (score layout)
    float inv[NT], bias[NT];
#pragma unroll
    for (int tile = 0; tile < NT; ++tile) {
        float l = lpart[tile];
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        float sp = spart[tile];
        sp += __shfl_xor(sp, 16);
        sp += __shfl_xor(sp, 32);
        const int r = row0 + 16 * tile + l16;
        inv[tile] = l > 0.0f ? 1.0f / l : 0.0f;
        bias[tile] = kCodeBias * sp;
        if (wv == 0 && lg == 0 && r < R) {
            const float lse2 = l > 0.0f ? (mref[tile] + log2f(l)) * kLn2 : -INFINITY;
            const int64_t rid = row_out(r);
            if (p.NP == 1) {
                if (p.lse != nullptr) p.lse[rid] = lse2;
            } else {
                p.ws_lse[rid * p.NP + part] = lse2;
            }
        }
    }
    // move 1/l (and the int8 bias) to the output layout through LDS
#pragma unroll
    for (int tile = 0; tile < NT; ++tile) {
        float biasrow[4], invrow[4];
        if (lg == 0) redist[wv][tile][l16] = inv[tile];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int i = 0; i < 4; ++i) invrow[i] = redist[wv][tile][4 * lg + i];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if constexpr (I8) {
            if (lg == 0) redist[wv][tile][l16] = bias[tile];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
            for (int i = 0; i < 4; ++i) biasrow[i] = redist[wv][tile][4 * lg + i];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = row0 + 16 * tile + 4 * lg + i;
            if (r >= R) continue;
            const int64_t rid = row_out(r);
#pragma unroll
            for (int nd = 0; nd < NDT; ++nd) {
                float v = o[tile][nd][i];
                if constexpr (I8) v = (v - biasrow[i]) * vsh_inv;
                v *= invrow[i];
                const int d = wv * DW + 16 * nd + l16;
                if (p.NP == 1) {
                    if (p.out_bf16)
                        reinterpret_cast<uint16_t*>(p.out)[rid * D + d] = f32_to_bf16(v);
                    else
                        reinterpret_cast<float*>(p.out)[rid * D + d] = v;
                } else {
                    p.ws_o[(rid * p.NP + part) * D + d] = v;
                }
            }
        }
    }
}

namespace {
template <int KVT, int D, int NT, int QS>
hipError_t launch_one(const DecodeParams& p, hipStream_t s) {
    const int64_t grid = (int64_t)p.NP * p.nchunk * p.Hkv * p.B;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((decode_mfma_kernel<KVT, D, NT, QS>), dim3((unsigned)grid), dim3(64 * kW), 0, s, p);
    return hipGetLastError();
}

template <int KVT, int D, int QS>
hipError_t by_nt(int NT, const DecodeParams& p, hipStream_t s) {
    switch (NT) {
    case 1: return launch_one<KVT, D, 1, QS>(p, s);
    case 2: return launch_one<KVT, D, 2, QS>(p, s);
    case 3: return launch_one<KVT, D, 3, QS>(p, s);
    case 4: return launch_one<KVT, D, 4, QS>(p, s);
    default: return hipErrorInvalidValue;
    }
}

template <int KVT, int QS>
hipError_t by_d(int D, int NT, const DecodeParams& p, hipStream_t s) {
    switch (D) {
    case 64: return by_nt<KVT, 64, QS>(NT, p, s);
    case 128: return by_nt<KVT, 128, QS>(NT, p, s);
    case 256: return by_nt<KVT, 256, QS>(NT, p, s);
    default: return hipErrorInvalidValue;
    }
}
}  // namespace

hipError_t launch_decode_mfma(int kv_type, int D, int NT, const DecodeParams& p, hipStream_t stream) {
    const int qs = p.q_bf16 ? 1 : 2;
    if (kv_type == KV_BF16) return qs == 1 ? by_d<KV_BF16, 1>(D, NT, p, stream) : by_d<KV_BF16, 2>(D, NT, p, stream);
    if (kv_type == KV_I8) return qs == 1 ? by_d<KV_I8, 1>(D, NT, p, stream) : by_d<KV_I8, 2>(D, NT, p, stream);
    return hipErrorInvalidValue;
}

}  // namespace pa
