// General kernel of the sparse Flash-MLA Softmax-L1Norm for gfx950: rows of
// any head count (one wave per 32-head tile) and any number of indices. It
// runs the rows the two pipelined kernels do not take: more than 64 heads
// with more than 2048 indices per row.
//
// The operation ("SparseFlashMlaSoftmaxL1Norm" article, section 三阶段计算公式):
//   stage 1  gather the row's selected rows of K            (sparse_indices)
//   stage 2  P = exp(Mask(Q . Ksel^T * scale) - lse)          (SimpleSoftmax)
//   stage 3  out = sum_g P / G                                (ReduceSum over G)
// written into a zero-filled fp32 row of width S2 (BSND) or T2 (TND).
//
// Work decomposition (one query row = one workgroup at a time):
//  - a workgroup has one wave per 32-head tile (HT = 1, 2 or 4 waves); the
//    persistent grid walks rows in the order the metadata fixes;
//  - each wave keeps its 32 heads x 512 of Q in VGPRs as MFMA A operands
//    (32 x 16 B per lane) for the whole row;
//  - keys are processed in tiles of 32. Tile t+1 is gathered into one of two
//    LDS tiles with direct buffer->LDS loads (one instruction moves one whole
//    1 KB row) while the waves run the 32 v_mfma_f32_32x32x16 of tile t
//    (D = 512) against the other; indices are prefetched two tiles ahead;
//  - the accumulator holds 16 heads x 1 key per lane. The epilogue of tile
//    t-1 (scale and lse folded into one FMA, v_exp_f32 in base 2, sum over
//    the lane's 16 heads) is interleaved with the MFMAs of tile t; half-wave
//    and head-tile partial sums meet in LDS after the next barrier and are
//    added in a fixed order (deterministic, no atomics);
//  - rows of at most kVcap indices collect their values in LDS and are
//    assembled there (zeros + values at their columns) and written once with
//    coalesced stores at the end of the row; longer rows are zero-filled up
//    front and take single stores (indices of a row are distinct).
#include "smla_device.h"

namespace smla {
namespace {

template <bool BF16, bool GATHER, int HT, int LEAD = 4>
__device__ __forceinline__ f32x16_t qk_tile(const uint4* __restrict__ src, const uint4* qa,
                                            int col, int half, const f32x16_t& prev,
                                            const float* l2, float c, float* prev_sum,
                                            uint4* __restrict__ gdst,
                                            __amdgpu_buffer_rsrc_t krs, int32_t rows,
                                            int wave, int lane) {
    constexpr int kSlots = kTile / HT;                 // rows this wave gathers
    constexpr int kGap = kSlots >= 16 ? 1 : 16 / kSlots;  // MFMAs between gathers
    constexpr int kSteps = kChunks / 2;
    // Laid out step by step (one wave per SIMD issues one instruction per 4
    // cycles, and the MFMA keeps the matrix core busy for 32): each step
    // holds its MFMA, the operand read LEAD steps ahead, half an element of
    // the previous tile's epilogue (the fma in even steps, the exp and the
    // add in odd ones) and at most one gather load.
    f32x16_t acc = {};
    const uint4* row = src + col * kPitch + half;
    uint4 ring[LEAD];
#pragma unroll
    for (int i = 0; i < LEAD; ++i) ring[i] = row[2 * i];
    float sum = 0.0f, t = 0.0f;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
        __builtin_amdgcn_sched_barrier(0);
        acc = mfma_32x32x16<BF16>(qa[s], ring[s % LEAD], acc);
        asm volatile("" ::"v"(acc));
        if (s + LEAD < kSteps) ring[s % LEAD] = row[2 * (s + LEAD)];
        if ((s & 1) == 0) {
            t = __builtin_fmaf(prev[s >> 1], c, -l2[s >> 1]);
            pin(t);
        } else {
            sum += __builtin_amdgcn_exp2f(t);
            pin(sum);
        }
        if constexpr (GATHER) {
            if (s % kGap == 0 && s / kGap < kSlots) {
                const int kk = wave + (s / kGap) * HT;
                const int32_t j = __builtin_amdgcn_readlane(rows, kk);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, SMLA_LDS(gdst + kk * kPitch), 16,
                                                         lane << 4, j << 10, 0, 0);
            }
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    *prev_sum = sum;
    return acc;
}

template <int HT, bool BF16, bool TND, bool STAGED>
__global__ __launch_bounds__(64 * HT, 2) void smla_l1norm_kernel(KernelArgs a) {
    constexpr int NT = 64 * HT;
    constexpr int kPerThread = kVcap / NT;  // index re-reads per thread in the row assembly
    // two K tiles (distinct objects, so loads into one never wait on reads of
    // the other); kbuf0 doubles as the row stage at the end of a row
    __shared__ uint4 kbuf0[kTile * kPitch];
    __shared__ uint4 kbuf1[kTile * kPitch];
    __shared__ float red[2][2 * HT][kTile];   // half-wave partial sums, last two tiles
    __shared__ float redl[2 * HT][kTile];     // the same for a row's last tile
    __shared__ float vals[kVcap + 64];        // the row's values by entry; then a sink

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: lives in an SGPR
    const int half = lane >> 5;   // which 8-element k-group of the MFMA operand
    const int col = lane & 31;    // key slot of the MFMA B operand / output column
    const uint4* __restrict__ k4 = static_cast<const uint4*>(a.k);
    const uint4* __restrict__ q4 = static_cast<const uint4*>(a.q);
    constexpr bool staged = STAGED;  // rows assembled in LDS (needs K <= kVcap)
    float* const stage = reinterpret_cast<float*>(kbuf0);

    // this wave's head of lane (m, half) and the heads of its 16 accumulator
    // elements (element e of the 32x32 accumulator is head 8*(e/4) + 4*half + e%4);
    // heads past G read zeros (bounds-checked loads) and get an lse of +inf
    const int head = wave * 32 + col;

    // Raw Q (MFMA A operands: lane (m, half) holds head m, elements 16*s +
    // 8*half .. +8 for k-step s) and lse of row r; loads are only issued here
    uint4 qa[kChunks / 2];
    float lse_raw[16];
    auto load_row_operands = [&](int64_t r) {
        const __amdgpu_buffer_rsrc_t rq = rsrc(q4 + r * a.G * kChunks, (uint32_t)a.G * 1024u);
        const uint32_t qoff = (uint32_t)head * 1024u + (uint32_t)half * 16u;
#pragma unroll
        for (int s = 0; s < kChunks / 2; ++s)
            qa[s] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  rq, qoff + 32u * s, 0, 2 /* nt */));
        const __amdgpu_buffer_rsrc_t rl = rsrc(a.lse + r * a.G, (uint32_t)a.G * 4u);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int h = wave * 32 + 8 * (e >> 2) + 4 * half + (e & 3);
            lse_raw[e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                       rl, (uint32_t)h * 4u, 0, 0));
        }
    };

    int64_t it = 0;
    int64_t r = row_of(a, 0, blockIdx.x);
    load_row_operands(r < a.R ? r : a.R - 1);

    for (; it * a.num_wg < a.R; ++it) {
        r = row_of(a, it, blockIdx.x);
        if (r >= a.R) continue;
        const int64_t r_next = (it + 1) * a.num_wg < a.R ? row_of(a, it + 1, blockIdx.x) : a.R;
        const RowInfo ri = decode_row<TND>(a, r);
        float* __restrict__ orow = a.out + r * a.W;
        const int32_t* __restrict__ irow = a.idx + r * a.K;
        const int ntiles = (ri.n + kTile - 1) / kTile;
        // columns [seg0, seg1) can hold values; everything else is zero
        // (K-wide: the columns are the entries [0, n))
        const int64_t seg0 = ri.col0;
        const int64_t seg1 = ri.col0 + (ntiles > 0 ? (a.kwide ? ri.n : ri.vis) : 0);

        // raw index of slot `col` of a tile (any value; checked where used);
        // dense: the entry itself (the descriptor then has no range, so the
        // load reads nothing)
        const __amdgpu_buffer_rsrc_t ridx = rsrc(irow, a.dense ? 0u : (uint32_t)a.K * 4u);
        auto tile_idx = [&](int tile) -> int32_t {
            const int32_t e = tile * kTile + col;
            const int32_t j = __builtin_amdgcn_raw_buffer_load_b32(ridx, (uint32_t)e * 4u, 0, 0);
            return a.dense ? e : j;
        };
        // is slot kk of a tile, holding raw index j, a used entry?
        auto used = [&](int tile, int kk, int32_t j) -> bool {
            return tile * kTile + kk < ri.n && (uint32_t)j < (uint32_t)ri.vis;
        };
        // key row to gather for slot `col`: its index if used, else row 0
        // (fetched but never read)
        auto gather_row = [&](int tile, int32_t j) -> int32_t {
            return used(tile, col, j) ? j : 0;
        };
        int32_t key_cur = tile_idx(0);
        int32_t key_nxt = tile_idx(1);

        if (staged) {
            zero_span(orow, 0, seg0, tid, NT);
            zero_span(orow, seg1, a.W, tid, NT);
        } else {
            zero_span(orow, 0, a.W, tid, NT);
        }

        float l2[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int h = wave * 32 + 8 * (e >> 2) + 4 * half + (e & 3);
            l2[e] = h < a.G ? lse_raw[e] * kLog2e : __builtin_inff();
        }

        const __amdgpu_buffer_rsrc_t krs = k_rsrc(k4, ri.kbase);
        auto gather = [&](uint4* dst, int tile, int32_t idx_reg) {
            const int32_t rows = gather_row(tile, idx_reg);
#pragma unroll
            for (int i = 0; i < kTile / HT; ++i) {
                const int kk = wave + i * HT;
                const int32_t j = __builtin_amdgcn_readlane(rows, kk);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, SMLA_LDS(dst + kk * kPitch), 16,
                                                         lane << 4, j << 10, 0, 0);
            }
        };
        if (ntiles > 0) gather(kbuf0, 0, key_cur);

        // Head-tile and half-wave partial sums of a tile, added in a fixed
        // order; wave w finishes slots [w*32/HT, (w+1)*32/HT) with its first
        // lanes. `key` is the tile's raw index register. The staged version
        // has no branch: other lanes (and tiles < 0) write to the sink.
        constexpr int kSlotsPerWave = kTile / HT;
        auto reduce_from = [&](const float (*pr)[kTile], int tile, int32_t key) {
            const int slot = (wave * kSlotsPerWave + lane) & (kTile - 1);
            float tot = pr[0][slot];
#pragma unroll
            for (int w = 1; w < 2 * HT; ++w) tot += pr[w][slot];
            const float v = tot * a.inv_g;
            if constexpr (STAGED) {
                const bool mine = lane < kSlotsPerWave && tile >= 0;
                vals[mine ? tile * kTile + slot : kVcap + lane] = v;
            } else {
                const int32_t j = __shfl(key, slot);
                if (lane < kSlotsPerWave && tile >= 0 && used(tile, slot, j))
                    orow[a.kwide ? tile * kTile + slot : ri.col0 + j] = v;
            }
        };
        auto reduce = [&](int tile, int32_t key) { reduce_from(red[tile & 1], tile, key); };

        f32x16_t acc_prev = {};
        int32_t key_p1 = -1, key_p2 = -1;  // raw indices of tiles t-1 and t-2
        // One tile: finish tile-2's head sum, gather tile+1, QK^T of this
        // tile with tile-1's epilogue.
        // A tile with a next tile (GATHER) issues that tile's rows between its
        // MFMAs; the last tile of a row gathers nothing (kbuf0 is the row
        // stage at the end of the row, so no load may land there late).
        auto body = [&](auto GATHER, int tile, const uint4* cur, uint4* nxt) {
            // gathers of this tile landed, partial sums of tile-1 visible
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            reduce(tile - 2, key_p2);
            const int32_t key_nn = tile_idx(tile + 2);
            float sum_prev;
            const f32x16_t acc = qk_tile<BF16, decltype(GATHER)::value != 0, HT>(
                cur, qa, col, half, acc_prev, l2, a.c_scale, &sum_prev, nxt, krs,
                decltype(GATHER)::value ? gather_row(tile + 1, key_nxt) : 0, wave, lane);
            red[(tile - 1) & 1][2 * wave + half][col] = sum_prev;  // tile 0: unused slot
            acc_prev = acc;
            key_p2 = key_p1;
            key_p1 = key_cur;
            key_cur = key_nxt;
            key_nxt = key_nn;
        };
        int tile = 0;
        for (; tile + 2 < ntiles; tile += 2) {
            body(Par<1>{}, tile, kbuf0, kbuf1);
            body(Par<1>{}, tile + 1, kbuf1, kbuf0);
        }
        if (tile + 1 < ntiles) {
            body(Par<1>{}, tile, kbuf0, kbuf1);
            body(Par<0>{}, tile + 1, kbuf1, kbuf0);
        } else if (tile < ntiles) {
            body(Par<0>{}, tile, kbuf0, kbuf1);
        }
        // (the last tile's sums go to their own buffer: a slower wave may
        // still be reading red[(ntiles - 1) & 1] in the last tile's reduce)
        if (ntiles > 0) redl[2 * wave + half][col] = head_sum(acc_prev, l2, a.c_scale);

        // indices for the row assembly, then the next row's Q and lse: all
        // in flight together; waits below cover only the indices
        int32_t jre[kPerThread];
        if (staged) {
#pragma unroll
            for (int i = 0; i < kPerThread; ++i) {
                const int32_t j = __builtin_amdgcn_raw_buffer_load_b32(
                    ridx, (uint32_t)(tid + i * NT) * 4u, 0, 0);
                jre[i] = a.dense ? tid + i * NT : j;
            }
        }
        // unconditional (a clamped row when this is the last one), so the new
        // operands take over the registers of the old ones
        load_row_operands(r_next < a.R ? r_next : r);

        __syncthreads();  // partial sums in LDS (the barrier waits for LDS writes)
        if (ntiles >= 2) reduce(ntiles - 2, key_p2);
        if (ntiles >= 1) reduce_from(redl, ntiles - 1, key_p1);

        if (staged) {
            // assemble columns [seg0, seg1) in LDS and write them once. Stage
            // index of column c is c - c0 + m0, m0 aligning 16-byte groups of
            // the output row with 16-byte groups of the stage.
            for (int64_t c0 = seg0; c0 < seg1; c0 += kStage - 4) {
                const int64_t len = (seg1 - c0 < kStage - 4) ? seg1 - c0 : kStage - 4;
                const int m0 = (int)((r * a.W + c0) & 3);
                __syncthreads();  // vals complete; previous chunk written out
                for (int i = tid; i < (len + m0 + 3) >> 2; i += NT)
                    reinterpret_cast<f32x4_t*>(stage)[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                __syncthreads();
#pragma unroll
                for (int i = 0; i < kPerThread; ++i) {
                    const int t = tid + i * NT;
                    const int32_t j = jre[i];
                    if (t < ri.n && (uint32_t)j < (uint32_t)ri.vis) {
                        const int64_t c = (a.kwide ? t : ri.col0 + j) - c0;
                        if (c >= 0 && c < len) stage[c + m0] = vals[t];
                    }
                }
                __syncthreads();
                // 16-byte groups q cover columns c0 - m0 + 4q .. +3
                const int ngroups = (int)((len + m0 + 3) >> 2);
                for (int qg = tid; qg < ngroups; qg += NT) {
                    const int64_t cb = c0 - m0 + 4 * (int64_t)qg;
                    if (cb >= c0 && cb + 4 <= c0 + len) {
                        const f32x4_t v = reinterpret_cast<const f32x4_t*>(stage)[qg];
                        __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t*>(orow + cb));
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (cb + e >= c0 && cb + e < c0 + len) orow[cb + e] = stage[4 * qg + e];
                    }
                }
            }
            __syncthreads();  // the next row's first gather reuses kbuf0
        }
        // end of row
    }
    // end of kernel
}

template <int HT, bool BF16, bool TND>
hipError_t launch_t(const KernelArgs& a, hipStream_t stream) {
    if (a.K <= kVcap)
        hipLaunchKernelGGL((smla_l1norm_kernel<HT, BF16, TND, true>), dim3(a.num_wg),
                           dim3(64 * HT), 0, stream, a);
    else
        hipLaunchKernelGGL((smla_l1norm_kernel<HT, BF16, TND, false>), dim3(a.num_wg),
                           dim3(64 * HT), 0, stream, a);
    return hipGetLastError();
}

template <int HT, bool BF16, bool TND>
hipError_t occupancy_t(int* out) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(
        out, reinterpret_cast<const void*>(&smla_l1norm_kernel<HT, BF16, TND, true>), 64 * HT,
        0);
}

}  // namespace

hipError_t launch_general(const KernelArgs& a, int ht, bool bf16, bool tnd,
                          hipStream_t stream) {
    SMLA_DISPATCH(launch_t, a, stream);
}

hipError_t general_resident_per_cu(int ht, bool bf16, bool tnd, int* out) {
    SMLA_DISPATCH(occupancy_t, out);
}

}  // namespace smla
