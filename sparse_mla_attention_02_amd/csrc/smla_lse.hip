// Forward softmax_lse kernel for gfx950 (the input the Softmax-L1Norm
// operation consumes), over the same used entries as the main call: the
// general kernel, for rows the pipelined one (smla_lse_wide.hip) does not
// take (up to 64 heads, or more than 2048 indices).
//
// Built without -amdgpu-mfma-vgpr-form: with one 32-head block per wave it
// measured 9% slower with MFMA results in VGPRs.
#include "smla_device.h"

namespace smla {
namespace {

// ---------------------------------------------------------------------------
// Forward softmax_lse over the same used entries: the input the operation
// consumes (parameter table, softmax_lse: the forward attention pass's
// log-sum-exp, whose formula the article defers to the sparse_flash_mla
// operator; taken here as its plain definition)
//   lse[r, g] = log sum_{t used} exp(scale * q[r,g,:] . K[key(t),:]),
// -inf for a row without a used entry.
//
// Same row walk, gathers and 32-key tiles as the general kernel, with the
// MFMA operands swapped (S = Ksel . Q^T): a lane's accumulator then holds 16
// keys of one head, so the reduction over keys runs inside the lane as an
// online maximum and rescaled sum (base 2); the two half-waves of a head
// meet once at the end of the row.


// One 32-key tile for two blocks of 32 heads (S = K_tile . Q_tile^T, each K
// operand read feeding both MFMAs), with the previous tile's exact online
// log-sum-exp update (the arithmetic of lse_update below, in the same
// order) laid out between the MFMAs. One wave per SIMD issues one
// instruction per 4 cycles and each MFMA keeps the matrix core busy for 32,
// so each gap holds about six instructions: steps 0..15 form the masked
// scaled scores of element s and their running maximum (block 0 in the
// first gap, block 1 in the second), steps 15..16 the new bases, and steps
// 16..31 add each element's exp2 to the rescaled sum. Bit
// 8*(e/4) + e%4 of `used` says whether element e is a used entry.
// `gstep(i)`, called in the second gap of steps 0..15, issues the next
// tile's gather loads one at a time.
template <bool BF16, typename GStep>
__device__ __forceinline__ void kq_tile_exact2(const uint4* __restrict__ src,
                                               const uint4 (*qa)[kChunks / 2], int col, int half,
                                               f32x16_t* acc, const f32x16_t* prev,
                                               uint32_t used, float c, float* m, float* l,
                                               GStep&& gstep) {
    constexpr float kNegInf = -__builtin_inff();
    constexpr int kSteps = kChunks / 2;
    constexpr int kLead = 4;
    acc[0] = f32x16_t{};
    acc[1] = f32x16_t{};
    const uint4* row = src + col * kPitch + half;
    uint4 ring[kLead];
#pragma unroll
    for (int i = 0; i < kLead; ++i) ring[i] = row[2 * i];
    float x0[16], x1[16], mt0 = kNegInf, mt1 = kNegInf, b0 = 0.0f, b1 = 0.0f, s0 = 0.0f,
                          s1 = 0.0f, m0n = kNegInf, m1n = kNegInf;
    bool u = false;
    auto base_of = [&](float mo, float mt, float lo, float& mn, float& b, float& sum) {
        mn = __builtin_fmaxf(mo, mt);
        b = mn == kNegInf ? 0.0f : mn;  // nothing used yet: every term is 0
        sum = lo * __builtin_amdgcn_exp2f(mo - b);
    };
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
        __builtin_amdgcn_sched_barrier(0);
        acc[0] = mfma_32x32x16<BF16>(ring[st % kLead], qa[0][st], acc[0]);
        asm volatile("" ::"a"(acc[0]));
        if (st < 16) {
            const int e = st;
            u = (used >> (8 * (e >> 2) + (e & 3))) & 1u;
            x0[e] = u ? prev[0][e] * c : kNegInf;
            mt0 = __builtin_fmaxf(mt0, x0[e]);
            pin(mt0);
        } else {
            s0 += __builtin_amdgcn_exp2f(x0[st - 16] - b0);
            pin(s0);
        }
        if (st == 16) {
            base_of(m[1], mt1, l[1], m1n, b1, s1);
            pin(s1);
        }
        __builtin_amdgcn_sched_barrier(0);
        acc[1] = mfma_32x32x16<BF16>(ring[st % kLead], qa[1][st], acc[1]);
        asm volatile("" ::"a"(acc[1]));
        if (st + kLead < kSteps) ring[st % kLead] = row[2 * (st + kLead)];
        if (st < 16) gstep(st);
        if (st < 16) {
            const int e = st;
            x1[e] = u ? prev[1][e] * c : kNegInf;
            mt1 = __builtin_fmaxf(mt1, x1[e]);
            pin(mt1);
        }
        if (st == 15) {
            base_of(m[0], mt0, l[0], m0n, b0, s0);
            pin(s0);
        }
        if (st >= 17) {
            s1 += __builtin_amdgcn_exp2f(x1[st - 17] - b1);
            pin(s1);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    s1 += __builtin_amdgcn_exp2f(x1[15] - b1);
    m[0] = m0n;
    l[0] = s0;
    m[1] = m1n;
    l[1] = s1;
}

// Online update of one lane's (m, l) -- base-2 running maximum and sum of
// 2^(x - m) -- with its 16 scores of a tile, x = acc * c. Bit
// 8*(e/4) + e%4 of `used` says whether element e is a used entry.
__device__ __forceinline__ void lse_update(const f32x16_t& acc, uint32_t used, float c,
                                           float& m, float& l) {
    constexpr float kNegInf = -__builtin_inff();
    float x[16];
    float mt = kNegInf;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        x[e] = ((used >> (8 * (e >> 2) + (e & 3))) & 1u) ? acc[e] * c : kNegInf;
        mt = __builtin_fmaxf(mt, x[e]);
    }
    const float mn = __builtin_fmaxf(m, mt);
    const float base = mn == kNegInf ? 0.0f : mn;  // nothing used yet: every term is 0
    float sum = l * __builtin_amdgcn_exp2f(m - base);
#pragma unroll
    for (int e = 0; e < 16; ++e) sum += __builtin_amdgcn_exp2f(x[e] - base);
    m = mn;
    l = sum;
}

// Lazy step of the online log-sum-exp: against the lane's current base b
// (the maximum of an earlier tile, kept while the scores stay within
// kLazyLimit of it), y = x - b for the lane's 16 scores x = acc * c of the
// tile (-inf where unused); returns their maximum and the sum of 2^y. The
// caller adds the sum when the maximum is at most kLazyLimit (every term
// then stays below 2^kLazyLimit), and otherwise redoes the tile exactly
// (lse_update); a lane without a base yet (b = -inf) always does.
constexpr float kLazyLimit = 64.0f;
__device__ __forceinline__ void lse_lazy(const f32x16_t& acc, uint32_t slots, float c, float b,
                                         float& ymax, float& sum) {
    const float nb = -b;
    ymax = -__builtin_inff();
    sum = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const float y =
            select_lanes(used_lanes(slots, e), __builtin_fmaf(acc[e], c, nb), -__builtin_inff());
        ymax = __builtin_fmaxf(ymax, y);
        sum += __builtin_amdgcn_exp2f(y);
    }
}

// One 32-key tile for one block of 32 heads with the previous tile's lazy
// step (lse_lazy, same arithmetic and order) laid out step by step: each
// step holds its MFMA, the operand read four steps ahead, half an element of
// the lazy step (the masked shifted score in even steps, the maximum, the
// exp2 and the sum in odd ones) and `gstep(s)`, at most one gather load.
template <bool BF16, typename GStep>
__device__ __forceinline__ void kq_tile_lazy(const uint4* __restrict__ src, const uint4* qa,
                                             int col, int half, f32x16_t& acc,
                                             const f32x16_t& prev, uint32_t slots, float c,
                                             float b, float& ymax, float& sum, GStep&& gstep) {
    constexpr int kSteps = kChunks / 2;
    constexpr int kLead = 4;
    acc = f32x16_t{};
    const uint4* row = src + col * kPitch + half;
    uint4 ring[kLead];
#pragma unroll
    for (int i = 0; i < kLead; ++i) ring[i] = row[2 * i];
    const float nb = -b;
    float y = 0.0f;
    ymax = -__builtin_inff();
    sum = 0.0f;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
        __builtin_amdgcn_sched_barrier(0);
        acc = mfma_32x32x16<BF16>(ring[s % kLead], qa[s], acc);
        asm volatile("" ::"a"(acc));
        if (s + kLead < kSteps) ring[s % kLead] = row[2 * (s + kLead)];
        const int e = s >> 1;
        if ((s & 1) == 0) {
            y = select_lanes(used_lanes(slots, e), __builtin_fmaf(prev[e], c, nb),
                             -__builtin_inff());
            pin(y);
        } else {
            ymax = __builtin_fmaxf(ymax, y);
            sum += __builtin_amdgcn_exp2f(y);
            pin(sum);
        }
        gstep(s);
    }
    __builtin_amdgcn_sched_barrier(0);
}

// WAVES waves per workgroup, each with NB blocks of 32 heads (1 x 1 for up
// to 32 heads, 2 x 1 for up to 64, 2 x 2 for up to 128). One wave per SIMD
// at two workgroups per CU, so each wave has the whole register file: Q
// takes NB x 128 registers.
template <int NB, int WAVES, bool BF16, bool TND>
__global__ __launch_bounds__(64 * WAVES, 2) void smla_lse_kernel(KernelArgs a) {
    __shared__ uint4 kbuf0[kTile * kPitch];
    __shared__ uint4 kbuf1[kTile * kPitch];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5;
    const int col = lane & 31;
    const uint4* __restrict__ k4 = static_cast<const uint4*>(a.k);
    const uint4* __restrict__ q4 = static_cast<const uint4*>(a.q);
    // lane (col, half) holds head head0 + 32*nb of Q as MFMA B operand of
    // block nb and, in that block's accumulator, keys 8*(e/4) + 4*half + e%4
    // of a tile for that head; heads past G read zeros and are never written
    const int head0 = wave * 32 * NB + col;

    uint4 qa[NB][kChunks / 2];
    auto load_q = [&](int64_t r) {
        const __amdgpu_buffer_rsrc_t rq = rsrc(q4 + r * a.G * kChunks, (uint32_t)a.G * 1024u);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const uint32_t qoff = (uint32_t)(head0 + 32 * nb) * 1024u + (uint32_t)half * 16u;
#pragma unroll
            for (int s = 0; s < kChunks / 2; ++s)
                qa[nb][s] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                          rq, qoff + 32u * s, 0, 2 /* nt */));
        }
    };

    int64_t it = 0;
    int64_t r = row_of(a, 0, blockIdx.x);
    load_q(r < a.R ? r : a.R - 1);

    for (; it * a.num_wg < a.R; ++it) {
        r = row_of(a, it, blockIdx.x);
        if (r >= a.R) continue;
        const int64_t r_next = (it + 1) * a.num_wg < a.R ? row_of(a, it + 1, blockIdx.x) : a.R;
        const RowInfo ri = decode_row<TND>(a, r);
        const int32_t* __restrict__ irow = a.idx + r * a.K;
        const int ntiles = (ri.n + kTile - 1) / kTile;

        const __amdgpu_buffer_rsrc_t ridx = rsrc(irow, a.dense ? 0u : (uint32_t)a.K * 4u);
        auto tile_idx = [&](int tile) -> int32_t {
            const int32_t e = tile * kTile + col;
            const int32_t j = __builtin_amdgcn_raw_buffer_load_b32(ridx, (uint32_t)e * 4u, 0, 0);
            return a.dense ? e : j;
        };
        auto used = [&](int tile, int kk, int32_t j) -> bool {
            return tile * kTile + kk < ri.n && (uint32_t)j < (uint32_t)ri.vis;
        };
        int32_t key_cur = tile_idx(0);
        int32_t key_nxt = tile_idx(1);

        // slot kk of a tile is moved by wave kk % WAVES, one 1 KB row per
        // instruction; unused slots fetch row 0 (never counted)
        const __amdgpu_buffer_rsrc_t krs = k_rsrc(k4, ri.kbase);
        auto gather = [&](uint4* dst, int tile, int32_t idx_reg) {
            const int32_t rows = used(tile, col, idx_reg) ? idx_reg : 0;
#pragma unroll
            for (int i = 0; i < kTile / WAVES; ++i) {
                const int kk = wave + i * WAVES;
                const int32_t j = __builtin_amdgcn_readlane(rows, kk);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, SMLA_LDS(dst + kk * kPitch), 16,
                                                         lane << 4, j << 10, 0, 0);
            }
        };
        if (ntiles > 0) gather(kbuf0, 0, key_cur);

        float m[NB], l[NB];
        f32x16_t acc[NB], acc_prev[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            m[nb] = -__builtin_inff();
            l[nb] = 0.0f;
            acc_prev[nb] = f32x16_t{};
        }
        // (m, l): the lane's base and its sum of 2^(x - m). With one block
        // of heads per wave the lazy step runs between the MFMAs and the
        // check (rarely the exact update) after them; with two, the exact
        // update runs between the MFMAs (measured: the lazy step gains 12%
        // at 64 heads and loses 1% at 128).
        constexpr bool kLazy = NB == 1;
        uint32_t slots_prev = 0;  // tile-1's used slots (wave-uniform)
        float ymax[NB], lsum[NB];
        auto epilogue = [&] {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                if constexpr (kLazy)
                    lse_lazy(acc_prev[nb], slots_prev, a.c_scale, m[nb], ymax[nb], lsum[nb]);
                else
                    lse_update(acc_prev[nb], slots_prev >> (4 * half), a.c_scale, m[nb], l[nb]);
            }
        };
        auto settle = [&] {
            if constexpr (kLazy) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    if (ymax[nb] > kLazyLimit)
                        lse_update(acc_prev[nb], slots_prev >> (4 * half), a.c_scale, m[nb],
                                   l[nb]);
                    else
                        l[nb] += lsum[nb];
                }
            }
        };
        auto body = [&](int tile, const uint4* cur, uint4* nxt) {
            // gathers of this tile landed; every wave is done reading `nxt`
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            const int32_t key_nn = tile_idx(tile + 2);
            // slot kk of the tile is used: bit kk (lanes kk and kk + 32 agree)
            const uint32_t mask =
                (uint32_t)__builtin_amdgcn_ballot_w64(used(tile, col, key_cur));
            // the next tile's rows (row 0 where it has none: the buffer is
            // then not read again, and each slot is always loaded by the same
            // wave, in order) are gathered one per step, 32 / WAVES of them
            const int32_t rows = used(tile + 1, col, key_nxt) ? key_nxt : 0;
            auto gstep = [&](int i) {
                if (i < kTile / WAVES) {
                    const int kk = wave + i * WAVES;
                    const int32_t j = __builtin_amdgcn_readlane(rows, kk);
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, SMLA_LDS(nxt + kk * kPitch), 16,
                                                             lane << 4, j << 10, 0, 0);
                }
            };
            if constexpr (NB == 2) {
                kq_tile_exact2<BF16>(cur, qa, col, half, acc, acc_prev, slots_prev >> (4 * half),
                                     a.c_scale, m, l, gstep);
            } else if constexpr (NB == 1) {
                kq_tile_lazy<BF16>(cur, qa[0], col, half, acc[0], acc_prev[0], slots_prev,
                                   a.c_scale, m[0], ymax[0], lsum[0], gstep);
                settle();
            }
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc_prev[nb] = acc[nb];
            slots_prev = mask;
            key_cur = key_nxt;
            key_nxt = key_nn;
        };
        for (int tile = 0; tile < ntiles; tile += 2) {
            body(tile, kbuf0, kbuf1);
            if (tile + 1 < ntiles) body(tile + 1, kbuf1, kbuf0);
        }
        if (ntiles > 0) {
            epilogue();
            settle();
        }
        // the next row's Q (a clamped row after the last one) is in flight
        // during the combine and store
        load_q(r_next < a.R ? r_next : r);

        // the two half-waves of a head: (m, l) and (m', l') combine into
        // M = max(m, m'), L = l 2^(m-M) + l' 2^(m'-M); lse = ln2 (M + log2 L)
        // (a base is the maximum of the tile that set it, whose term 2^0 is
        // in its sum)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const float m2 = __shfl_xor(m[nb], 32);
            const float l2 = __shfl_xor(l[nb], 32);
            const float mm = __builtin_fmaxf(m[nb], m2);
            const float base = mm == -__builtin_inff() ? 0.0f : mm;
            const float L = l[nb] * __builtin_amdgcn_exp2f(m[nb] - base) +
                            l2 * __builtin_amdgcn_exp2f(m2 - base);
            // a used entry contributes 2^0 = 1 at the maximum, so L >= 1
            // whenever anything is used
            const float v =
                L > 0.0f ? (mm + __builtin_amdgcn_logf(L)) * kLn2 : -__builtin_inff();
            const int h = head0 + 32 * nb;
            if (half == 0 && h < a.G) a.out[r * a.G + h] = v;
        }
        // every wave is done with kbuf0 before the next row gathers into it
        __syncthreads();
    }
    // loads into LDS (the last tile's gathers of row 0) must land before the
    // workgroup's LDS is released
    __builtin_amdgcn_s_waitcnt(0);
}

// head tiles HT (1, 2 or 4 blocks of 32 heads) -> NB blocks per wave x WAVES
template <int HT, bool BF16, bool TND>
hipError_t launch_lse_t(const KernelArgs& a, hipStream_t stream) {
    constexpr int NB = HT == 4 ? 2 : 1;
    constexpr int WAVES = HT / NB;
    hipLaunchKernelGGL((smla_lse_kernel<NB, WAVES, BF16, TND>), dim3(a.num_wg),
                       dim3(64 * WAVES), 0, stream, a);
    return hipGetLastError();
}

template <int HT, bool BF16, bool TND>
hipError_t occupancy_lse_t(int* out) {
    constexpr int NB = HT == 4 ? 2 : 1;
    constexpr int WAVES = HT / NB;
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(
        out, reinterpret_cast<const void*>(&smla_lse_kernel<NB, WAVES, BF16, TND>),
        64 * WAVES, 0);
}

}  // namespace

hipError_t launch_lse(const KernelArgs& a, int ht, bool bf16, bool tnd, hipStream_t stream) {
    switch (lse_variant(a.G, a.dense ? 0 : a.K)) {
        case kLseNarrow: return launch_lse_narrow(a, bf16, tnd, stream);
        case kLseWide: return launch_lse_wide(a, bf16, tnd, stream);
        default: SMLA_DISPATCH(launch_lse_t, a, stream);
    }
}

hipError_t lse_resident_per_cu(int ht, bool bf16, bool tnd, int64_t G, int64_t topk, int* out) {
    switch (lse_variant(G, topk)) {
        case kLseNarrow: return lse_narrow_resident_per_cu(bf16, tnd, out);
        case kLseWide: return lse_wide_resident_per_cu(bf16, tnd, out);
        default: SMLA_DISPATCH(occupancy_lse_t, out);
    }
}

}  // namespace smla
