// gfx950 kernels for the sparse Flash-MLA Softmax-L1Norm.
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
//  - the values of a row collect in LDS; at the end of the row the row is
//    assembled in LDS (zeros + values at their columns) and written once
//    with coalesced stores. Columns no index can reach are zero-filled with
//    streaming stores up front. Rows with more than kVcap indices fall back
//    to zero-fill then single stores (indices of a row are distinct).
#include "smla_internal.h"

#include <type_traits>


namespace smla {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;

constexpr int kD = 512;             // head dim (only value supported)
constexpr int kChunks = kD * 2 / 16;  // 16-byte chunks per row of K / head of Q
constexpr int kTile = 32;           // keys per tile (MFMA N)
// LDS pitch of one K row in 16-byte chunks: one spare chunk per row so that
// the 16 lanes of an LDS read phase (16 different rows, same chunk) hit 16
// different bank groups (row * 65 mod 16 = row mod 16)
constexpr int kPitch = kChunks + 1;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kVcap = 2048;         // values of one row kept in LDS for assembly
constexpr int kStage = kTile * kPitch * 4 - 4;  // floats of one K tile usable as row stage

template <bool BF16>
__device__ __forceinline__ f32x16_t mfma_32x32x16(uint4 a, uint4 b, f32x16_t c) {
    if constexpr (BF16) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                        __builtin_bit_cast(bf16x8_t, b),
                                                        c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                       __builtin_bit_cast(f16x8_t, b),
                                                       c, 0, 0, 0);
    }
}

struct RowInfo {
    int64_t kbase;  // first k row of the row's batch / sequence
    int64_t col0;   // first output column of the row's batch / sequence
    int32_t vis;    // keys [0, vis) of the sequence are visible and in range
    int32_t n;      // entries of the index row to look at
};

// Streaming zero stores of row[c0, c1): scalar head/tail, 16-byte body.
__device__ __forceinline__ void zero_span(float* __restrict__ row, int64_t c0, int64_t c1,
                                          int tid, int nt) {
    if (c1 <= c0) return;
    const int64_t head = ((16 - (reinterpret_cast<uintptr_t>(row + c0) & 15)) & 15) >> 2;
    const int64_t h = head < c1 - c0 ? head : c1 - c0;
    if (tid < h) row[c0 + tid] = 0.0f;
    const int64_t b0 = c0 + h;
    const int64_t n4 = (c1 - b0) >> 2;
    f32x4_t* o4 = reinterpret_cast<f32x4_t*>(row + b0);
    const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
    for (int64_t i = tid; i < n4; i += nt) __builtin_nontemporal_store(z, o4 + i);
    const int64_t t0 = b0 + 4 * n4;
    if (tid < c1 - t0) row[t0 + tid] = 0.0f;
}

// Read-only int32 data at a wave-uniform address: the constant address
// space lets the compiler use scalar loads (waited with lgkmcnt, so they do
// not queue behind the vector loads in flight).
typedef const __attribute__((address_space(4))) int32_t* cint_ptr;
__device__ __forceinline__ int32_t uload(const int32_t* p, int64_t i) {
    return ((cint_ptr)p)[i];
}

// Row -> (batch, position) decode, mask limit and entry count.
// Right-down causal with compression ratio r and residual res: the query at
// position i of a sequence with s1 queries and s2 compressed keys is at
// original position i + s2*r + res - s1, and compressed key j (covering
// original positions j*r .. (j+1)*r - 1) is visible iff
// (j+1)*r <= i + 1 + s2*r + res - s1, i.e. iff j < floor((i+1+s2*r+res-s1)/r).
template <bool TND>
__device__ __forceinline__ RowInfo decode_row(const KernelArgs& a, int64_t r) {
    int64_t b, i, s1, s2, kbase, col0;
    if constexpr (TND) {
        // largest b in [0, B) with cu_q[b] <= r
        int lo = 0, hi = a.B - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (uload(a.cu_q, mid) <= r) lo = mid; else hi = mid - 1;
        }
        b = lo;
        const int64_t q0 = uload(a.cu_q, b);
        s1 = (int64_t)uload(a.cu_q, b + 1) - q0;
        i = r - q0;
        kbase = uload(a.cu_k, b);
        s2 = (int64_t)uload(a.cu_k, b + 1) - kbase;
        // never reach past the k tensor or the output row
        if (kbase < 0) kbase = 0;
        if (s2 > a.rows_k - kbase) s2 = a.rows_k - kbase;
        if (s2 > a.W - kbase) s2 = a.W - kbase;
        if (s2 < 0) s2 = 0;
        col0 = kbase;
    } else {
        // rows and k rows number fewer than 2^31 (checked on the host): 32-bit
        // division
        const uint32_t b32 = (uint32_t)r / (uint32_t)a.S1;
        b = b32;
        i = (int64_t)((uint32_t)r - b32 * (uint32_t)a.S1);
        s1 = a.S1;
        s2 = a.S2;
        kbase = (int64_t)(b32 * (uint32_t)a.S2);
        col0 = 0;
    }
    int64_t vis = s2;
    if (a.mask_mode == 3) {
        // floor((d + s2*r) / r) = s2 - ceil(-d / r) with d = i + 1 + res - s1,
        // in 32-bit arithmetic: -d <= s1 - res < 2^32 for any residual >= -2^31
        // with s1 < 2^31 (larger values saturate)
        const int64_t res = a.cmp_res ? (int64_t)uload(a.cmp_res, b) : 0;
        const int64_t d = i + 1 + res - s1;
        if (d < 0) {
            const uint32_t nd = -d > 0xffffffffll ? 0xffffffffu : (uint32_t)(-d);
            const uint32_t rr = (uint32_t)a.cmp_ratio;
            const uint32_t q = nd / rr;
            const int64_t up = (int64_t)q + (nd - q * rr != 0u ? 1 : 0);
            vis = s2 - up;
            if (vis < 0) vis = 0;
        }
    }
    // entries to look at (selectBlockCount): topk_length clamped to [0, K];
    // without it K, or under the causal mask no more than the visible keys
    int32_t n = a.K;
    if (a.topk_len) {
        n = uload(a.topk_len, r);
        n = n < 0 ? 0 : (n > a.K ? a.K : n);
    } else if (a.mask_mode == 3 && vis < n) {
        n = (int32_t)vis;
    }
    if (vis == 0) n = 0;  // nothing visible: no entry can be used
    RowInfo ri;
    ri.kbase = kbase;
    ri.col0 = col0;
    ri.vis = (int32_t)vis;
    ri.n = n;
    return ri;
}

__device__ __forceinline__ int64_t row_of(const KernelArgs& a, int64_t it, int w) {
    const int64_t base = it * a.num_wg;
    return base + ((a.snake && (it & 1)) ? (a.num_wg - 1 - w) : w);
}

#define SMLA_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// Buffer resource over `bytes` bytes at `base` (raw byte addressing; word 3
// is the gfx9-family value for untyped buffer access). Lane offsets at or
// past `bytes` read as zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// Buffer resource over the k rows of one batch / sequence; rows are selected
// with the scalar offset.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t k_rsrc(const uint4* k4, int64_t kbase) {
    return rsrc(k4 + kbase * kChunks, 0x7fffffffu);
}

// One 32-key tile of K is gathered into LDS with direct buffer->LDS loads:
// slot kk (key kk of the tile) is moved by wave kk % HT with one instruction
// (64 lanes x 16 B = the whole 1 KB row, lane l -> chunk l; the row offset
// is a scalar).

// exp(s - lse) = 2^(acc*scale*log2e - lse*log2e), summed over the lane's 16
// heads (padded heads have lse2 = +inf and give 0)
__device__ __forceinline__ float head_sum(const f32x16_t& acc, const float* l2, float c) {
    float sum = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) sum += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[e], c, -l2[e]));
    return sum;
}

// S^T tile (this wave's 32 heads x 32 keys) = Q_tile . K_tile^T over D = 512,
// with the previous tile's head_sum and (GATHER) the gather of the next tile
// scheduled between the MFMAs: this wave's kTile/HT key rows are issued one
// per kGap MFMAs, so the loads stream through the texture unit while the
// matrix core runs instead of arriving in one burst after the barrier.
template <bool BF16, bool GATHER, int HT, int LEAD = 4>
__device__ __forceinline__ f32x16_t qk_tile(const uint4* __restrict__ src, const uint4* qa,
                                            int col, int half, const f32x16_t& prev,
                                            const float* l2, float c, float* prev_sum,
                                            uint4* __restrict__ gdst,
                                            __amdgpu_buffer_rsrc_t krs, int32_t rows,
                                            int wave, int lane) {
    constexpr int kSlots = kTile / HT;                 // rows this wave gathers
    constexpr int kGap = kSlots >= 16 ? 1 : 16 / kSlots;  // MFMAs between gathers
    f32x16_t acc = {};
    const uint4* row = src + col * kPitch + half;
#pragma unroll
    for (int s = 0; s < kChunks / 2; ++s) {
        const uint4 b = row[2 * s];
        acc = mfma_32x32x16<BF16>(qa[s], b, acc);
        if constexpr (GATHER) {
            if (s % kGap == 0 && s / kGap < kSlots) {
                const int kk = wave + (s / kGap) * HT;
                const int32_t j = __builtin_amdgcn_readlane(rows, kk);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, SMLA_LDS(gdst + kk * kPitch), 16,
                                                         lane << 4, j << 10, 0, 0);
            }
        }
    }
    *prev_sum = head_sum(prev, l2, c);
    // kLead operand reads ahead of the MFMAs; between MFMAs one read, two
    // VALU instructions of the previous tile's epilogue, and the gathers
    constexpr int kLead = LEAD;
    __builtin_amdgcn_sched_group_barrier(0x100, kLead, 0);
#pragma unroll
    for (int s = 0; s < kChunks / 2; ++s) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (s < kChunks / 2 - kLead) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
        if (GATHER && s % kGap == 0 && s / kGap < kSlots)
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
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
        const int64_t seg0 = ri.col0;
        const int64_t seg1 = ri.col0 + (ntiles > 0 ? ri.vis : 0);

        // raw index of slot `col` of a tile (any value; checked where used)
        const __amdgpu_buffer_rsrc_t ridx = rsrc(irow, (uint32_t)a.K * 4u);
        auto tile_idx = [&](int tile) -> int32_t {
            return __builtin_amdgcn_raw_buffer_load_b32(ridx, (uint32_t)(tile * kTile + col) * 4u,
                                                        0, 0);
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
        auto reduce = [&](int tile, int32_t key) {
            const int slot = (wave * kSlotsPerWave + lane) & (kTile - 1);
            const int pb = tile & 1;
            float tot = red[pb][0][slot];
#pragma unroll
            for (int w = 1; w < 2 * HT; ++w) tot += red[pb][w][slot];
            const float v = tot * a.inv_g;
            if constexpr (STAGED) {
                const bool mine = lane < kSlotsPerWave && tile >= 0;
                vals[mine ? tile * kTile + slot : kVcap + lane] = v;
            } else {
                const int32_t j = __shfl(key, slot);
                if (lane < kSlotsPerWave && tile >= 0 && used(tile, slot, j))
                    orow[ri.col0 + j] = v;
            }
        };

        f32x16_t acc_prev = {};
        int32_t key_p1 = -1, key_p2 = -1;  // raw indices of tiles t-1 and t-2
        // One tile: finish tile-2's head sum, gather tile+1, QK^T of this
        // tile with tile-1's epilogue.
        auto body = [&](int tile, const uint4* cur, uint4* nxt) {
            // gathers of this tile landed, partial sums of tile-1 visible
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            reduce(tile - 2, key_p2);
            if (tile + 1 < ntiles) gather(nxt, tile + 1, key_nxt);
            const int32_t key_nn = tile_idx(tile + 2);
            float sum_prev;
            const f32x16_t acc = qk_tile<BF16, false, HT>(cur, qa, col, half, acc_prev, l2,
                                                          a.c_scale, &sum_prev, nullptr, krs, 0,
                                                          wave, lane);
            red[(tile - 1) & 1][2 * wave + half][col] = sum_prev;  // tile 0: unused slot
            acc_prev = acc;
            key_p2 = key_p1;
            key_p1 = key_cur;
            key_cur = key_nxt;
            key_nxt = key_nn;
        };
        for (int tile = 0; tile < ntiles; tile += 2) {
            body(tile, kbuf0, kbuf1);
            if (tile + 1 < ntiles) body(tile + 1, kbuf1, kbuf0);
        }
        if (ntiles > 0)
            red[(ntiles - 1) & 1][2 * wave + half][col] = head_sum(acc_prev, l2, a.c_scale);

        // indices for the row assembly, then the next row's Q and lse: all
        // in flight together; waits below cover only the indices
        int32_t jre[kPerThread];
        if (staged) {
#pragma unroll
            for (int i = 0; i < kPerThread; ++i)
                jre[i] = __builtin_amdgcn_raw_buffer_load_b32(ridx, (uint32_t)(tid + i * NT) * 4u,
                                                              0, 0);
        }
        // unconditional (a clamped row when this is the last one), so the new
        // operands take over the registers of the old ones
        load_row_operands(r_next < a.R ? r_next : r);

        __syncthreads();  // partial sums in LDS (the barrier waits for LDS writes)
        if (ntiles >= 2) reduce(ntiles - 2, key_p2);
        if (ntiles >= 1) reduce(ntiles - 1, key_p1);

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
                        const int64_t c = ri.col0 + j - c0;
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

// ---------------------------------------------------------------------------
// Pipelined kernel for rows of 65..128 heads with at most kVcap indices.
//
// One workgroup of 4 waves per CU: one wave per SIMD, so each wave has the
// whole register file (Q of the current and of the next row, a deep operand
// read-ahead) and the workgroup has all of LDS: four K tiles. The gather of
// tile t+3 is spread over the MFMAs of tile t, so three tiles of compute
// cover its latency. A barrier per tile publishes the gathered tile and frees
// the oldest buffer; before it each wave waits only for its own loads of
// that tile (vmcnt = the loads it issued after them), never for later ones.
// The next row's Q is loaded in chunks spread over nine tiles. At the end
// of a row the next row's first three gathers are issued before this row's
// LDS assembly, which uses the fourth buffer as its stage, so the pipeline
// does not drain between rows.
//
// With one wave per SIMD, every instruction of a wave is issued in the time
// of the MFMAs, so the tile body is laid out by hand: each k-step holds one
// MFMA, one operand read, at most two independent VALU instructions of the
// previous tile's epilogue, and every fourth step one gathered key row.
//
// All loads into LDS are inline assembly: the compiler's wait-count
// tracking cannot follow LDS slots reused across loop iterations and would
// otherwise wait for every load in flight before any LDS read. Their
// completion is waited for explicitly, by the barrier that counts them.

// s_waitcnt with vmcnt(N) and lgkmcnt(0), expcnt untouched (immediate: vmcnt
// bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void waitcnt_vm_lgkm0() {
    static_assert(N >= 0 && N <= 63, "vmcnt is six bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (((N >> 4) & 3) << 14));
}
// vmcnt(n) and lgkmcnt(0), then a barrier with no memory fence, so loads
// into LDS still in flight stay in flight.
__device__ __forceinline__ void barrier_after_vmcnt(int n) {
    switch (n) {
        // the counts the pipelined kernel produces; anything else waits for all
        case 2: waitcnt_vm_lgkm0<2>(); break;
        case 5: waitcnt_vm_lgkm0<5>(); break;
        case 10: waitcnt_vm_lgkm0<10>(); break;
        case 13: waitcnt_vm_lgkm0<13>(); break;
        case 18: waitcnt_vm_lgkm0<18>(); break;
        case 21: waitcnt_vm_lgkm0<21>(); break;
        case 63: waitcnt_vm_lgkm0<63>(); break;
        default: waitcnt_vm_lgkm0<0>(); break;
    }
    asm volatile("s_barrier" ::: "memory");
}
// barrier that publishes this wave's LDS writes (loads into LDS excluded)
__device__ __forceinline__ void lds_barrier() {
    waitcnt_vm_lgkm0<63>();
    asm volatile("s_barrier" ::: "memory");
}

// Marks a loaded register as used here, on every path: the compiler then
// waits for its load at this point instead of before a later reuse of the
// register, where the wait would also cover the loads in flight since.
__device__ __forceinline__ void consume(int32_t v) { asm volatile("" ::"v"(v)); }
// Keeps a value's computation at this point of the instruction stream (pure
// arithmetic is otherwise free to move to its first use).
__device__ __forceinline__ void pin(float& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void pin_s(int32_t& v) { asm volatile("" : "+s"(v)); }

// Buffer descriptor as four dwords (base, range in bytes, gfx9 untyped
// format); offsets at or past `bytes` read as zero.
typedef __attribute__((ext_vector_type(4))) int32_t i32x4_t;
__device__ __forceinline__ i32x4_t raw_desc(const void* base, uint32_t bytes) {
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    return i32x4_t{(int32_t)(uint32_t)p, (int32_t)((uint32_t)(p >> 32) & 0xffffu), (int32_t)bytes,
                   0x00020000};
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}
// Lane i moves 16 bytes at byte offset voff + soff of the buffer to LDS
// address m0 + 16 i: with voff = 16 i, one 1 KB key row per instruction.
// soff must not come from a VALU instruction fewer than five wait states
// earlier.
__device__ __forceinline__ void dma_row(i32x4_t desc, uint32_t m0, int32_t soff, uint32_t voff) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen lds"
        :
        : "s"(m0), "v"(voff), "s"(desc), "s"(soff)
        : "memory", "m0");
}
// Lane i moves 4 bytes at byte offset voff + soff to LDS address m0 + 4 i.
__device__ __forceinline__ void dma_dword(i32x4_t desc, uint32_t m0, int32_t soff, uint32_t voff) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "buffer_load_dword %1, %2, %3 offen lds"
        :
        : "s"(m0), "v"(voff), "s"(desc), "s"(soff)
        : "memory", "m0");
}

constexpr int kBufBytes = kTile * kPitch * 16;  // one K tile in LDS
constexpr int kRowBytes = kPitch * 16;          // one key row in LDS

// One tile on the pipelined path. Step s: MFMA s; LDS read of the B operand
// of step s + kLead; epilogue of the previous tile, head e = s/2: FMA at
// step 2e, exp at 2e+1, added to the sum at 2e+2; key row i of this wave's
// share of tile t+3 (GATHER): row offset read at step 4i, load at 4i+2;
// `mid(s)` for the caller's own spread-out work.
template <bool BF16, bool GATHER, typename Mid>
__device__ __forceinline__ f32x16_t qk_tile_seq(const uint4* __restrict__ src, const uint4* qa,
                                                int col, int half, const f32x16_t& prev,
                                                const float* l2, float c, float* prev_sum,
                                                i32x4_t kdesc, uint32_t m0_rows, int32_t rows_off,
                                                uint32_t voff, Mid mid) {
    constexpr int kSteps = kChunks / 2;
    constexpr int kLead = 8;
    const uint4* row = src + col * kPitch + half;
    uint4 b[kSteps];
#pragma unroll
    for (int s = 0; s < kLead; ++s) b[s] = row[2 * s];
    f32x16_t acc = {};
    float sum = 0.0f, t = 0.0f, ex = 0.0f;
    int32_t soff = 0;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
        __builtin_amdgcn_sched_barrier(0);
        acc = mfma_32x32x16<BF16>(qa[s], b[s], acc);
        if (s + kLead < kSteps) b[s + kLead] = row[2 * (s + kLead)];
        if ((s & 1) == 0) {
            if (s >= 2) {
                sum += ex;
                pin(sum);
            }
            t = __builtin_fmaf(prev[s >> 1], c, -l2[s >> 1]);
            pin(t);
        } else {
            ex = __builtin_amdgcn_exp2f(t);
            pin(ex);
        }
        if constexpr (GATHER) {
            if ((s & 3) == 0) {
                soff = __builtin_amdgcn_readlane(rows_off, s >> 2);
                pin_s(soff);
            } else if ((s & 3) == 2) {
                dma_row(kdesc, m0_rows + (uint32_t)((s >> 2) * kRowBytes), soff, voff);
            }
        }
        mid(s);
    }
    __builtin_amdgcn_sched_barrier(0);
    *prev_sum = sum + ex;
    return acc;
}

template <bool BF16, bool TND>
__global__ __launch_bounds__(256, 1) void smla_pipe_kernel(KernelArgs a) {
    constexpr int HT = 4;
    constexpr int NT = 256;
    constexpr int kPerThread = kVcap / NT;
    constexpr int kSlotsPerWave = kTile / HT;
    // mid-row prefetch of the next row: the gather indices of its tiles 0..2
    constexpr int kPrefetchOps = 3;
    // K tiles (tile t in buffer t % 4; the last one doubles as the row stage)
    __shared__ uint4 kbuf[4][kTile * kPitch];
    // index rows: slot t % 4 holds the indices of tile t (lanes 0..31) and of
    // tile t+1 (32..63, unused)
    __shared__ int32_t kring[4][64];
    __shared__ float red[2][2 * HT][kTile];
    __shared__ float vals[kVcap + 64];
    __shared__ float lsebuf[HT][64];       // the next row's lse, heads 32w.. in lsebuf[w]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5;
    const int col = lane & 31;
    // this wave gathers key rows 8w .. 8w+7 of every tile; lane l < 8 holds
    // the index of row 8w + l
    const int my_slot = kSlotsPerWave * wave + (lane & 7);
    const uint4* __restrict__ q4 = static_cast<const uint4*>(a.q);
    const char* __restrict__ kbytes = static_cast<const char*>(a.k);
    float* const stage = reinterpret_cast<float*>(kbuf[3]);
    const uint32_t kbuf_lds = lds_addr(kbuf);
    const uint32_t ring_lds = lds_addr(kring);
    const uint32_t lse_lds = lds_addr(lsebuf);
    const uint32_t voff16 = (uint32_t)lane << 4;
    const uint32_t voff4 = (uint32_t)lane << 2;

    // ---- state of the current row (c*) and of the prefetched next row (n*)
    int64_t it = 0;
    int64_t rc = row_of(a, 0, blockIdx.x);   // num_wg <= R, so rc < R
    RowInfo ric = decode_row<TND>(a, rc);
    uint4 qa[kChunks / 2];
    int32_t nk0, nk1, nk2;                  // next row: index of key row my_slot, tiles 0..2
    int64_t rn = a.R, rln = rc;             // next row, and the row its loads read
    RowInfo rin = ric;

    auto idx_rsrc = [&](int64_t r) { return rsrc(a.idx + r * a.K, (uint32_t)a.K * 4u); };
    auto idx_desc = [&](int64_t r) { return raw_desc(a.idx + r * a.K, (uint32_t)a.K * 4u); };
    auto k_desc = [&](const RowInfo& ri) {
        const int64_t rows = a.rows_k - ri.kbase;
        const int64_t bytes = rows * 1024;
        return raw_desc(kbytes + ri.kbase * 1024,
                        bytes > 0xffffffffll ? 0xffffffffu : (uint32_t)(bytes < 0 ? 0 : bytes));
    };
    // Q and lse of a row pass through LDS: loaded as whole 1 KB head rows
    // (a load of Q straight into the MFMA operand layout would touch 32
    // head rows per instruction, several times slower through the address
    // unit), then read back per lane in the operand layout.
    // Q of row r, heads [h0, h1), into the K buffers (head h -> buffer
    // h / 32, row h % 32); heads past G read as zero
    auto stage_q = [&](int64_t r, int h0, int h1) {
        const i32x4_t qd = raw_desc(q4 + r * a.G * kChunks, (uint32_t)a.G * 1024u);
        for (int h = h0 + wave; h < h1; h += HT)
            dma_row(qd, kbuf_lds + (uint32_t)((h >> 5) * kBufBytes + (h & 31) * kRowBytes),
                    h * 1024, voff16);
    };
    // lse of row r: heads 32w .. 32w+31 into lsebuf[w][0 .. 31]
    auto stage_lse = [&](int64_t r) {
        const i32x4_t ld = raw_desc(a.lse + r * a.G, (uint32_t)a.G * 4u);
        dma_dword(ld, lse_lds + (uint32_t)(wave * 256), wave * 32 * 4, voff4);
    };
    // this wave's Q (MFMA A operands: lane (m, half) holds head 32w + m,
    // elements 16s + 8 half .. +8 for k-step s) and lse (log2 units; padded
    // heads get +inf) from LDS
    float l2[16];
    auto read_q_lse = [&]() {
        const uint4* row = kbuf[wave] + col * kPitch + half;
#pragma unroll
        for (int s = 0; s < kChunks / 2; ++s) qa[s] = row[2 * s];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int hl = 8 * (e >> 2) + 4 * half + (e & 3);
            l2[e] = wave * 32 + hl < a.G ? lsebuf[wave][hl] * kLog2e : __builtin_inff();
        }
    };
    // the next row of this workgroup, decoded, and the gather indices of its
    // tiles 0..2 (kPrefetchOps loads; the decode's scalar loads are waited
    // for here, so that later LDS waits can count)
    auto prefetch_next = [&]() {
        rn = (it + 1) * a.num_wg < a.R ? row_of(a, it + 1, blockIdx.x) : a.R;
        rln = rn < a.R ? rn : rc;  // the last row loads itself again (unused)
        rin = decode_row<TND>(a, rln);
        waitcnt_vm_lgkm0<63>();
        const __amdgpu_buffer_rsrc_t ridx = idx_rsrc(rln);
        nk0 = __builtin_amdgcn_raw_buffer_load_b32(ridx, (uint32_t)(0 * kTile + my_slot) * 4u, 0, 0);
        nk1 = __builtin_amdgcn_raw_buffer_load_b32(ridx, (uint32_t)(1 * kTile + my_slot) * 4u, 0, 0);
        nk2 = __builtin_amdgcn_raw_buffer_load_b32(ridx, (uint32_t)(2 * kTile + my_slot) * 4u, 0, 0);
    };
    auto ntiles_of = [](const RowInfo& ri) { return (ri.n + kTile - 1) / kTile; };
    // byte offset of the key row of slot my_slot of `tile` holding raw index
    // j: j's row if the entry is used, else row 0 (loaded, never read)
    auto row_off = [&](const RowInfo& ri, int tile, int32_t j) -> int32_t {
        return (tile * kTile + my_slot < ri.n && (uint32_t)j < (uint32_t)ri.vis) ? (j << 10) : 0;
    };
    // a row's first three gathers and the index rows of its tiles 3..5
    auto start_row = [&](const RowInfo& ri, int64_t r) {
        const i32x4_t kd = k_desc(ri);
        const int nt = ntiles_of(ri);
        const int32_t o0 = row_off(ri, 0, nk0), o1 = row_off(ri, 1, nk1), o2 = row_off(ri, 2, nk2);
        const uint32_t m0w = kbuf_lds + (uint32_t)(kSlotsPerWave * wave * kRowBytes);
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            if (nt > k) {
                const int32_t o = k == 0 ? o0 : (k == 1 ? o1 : o2);
                int32_t so[kSlotsPerWave];
#pragma unroll
                for (int i = 0; i < kSlotsPerWave; ++i) {
                    so[i] = __builtin_amdgcn_readlane(o, i);
                    pin_s(so[i]);
                }
#pragma unroll
                for (int i = 0; i < kSlotsPerWave; ++i)
                    dma_row(kd, m0w + (uint32_t)(k * kBufBytes + i * kRowBytes), so[i], voff16);
            }
        }
        const i32x4_t id = idx_desc(r);
        dma_dword(id, ring_lds + 3u * 256u, 3 * kTile * 4, voff4);
        dma_dword(id, ring_lds + 0u * 256u, 4 * kTile * 4, voff4);
        dma_dword(id, ring_lds + 1u * 256u, 5 * kTile * 4, voff4);
    };

    // ---- first row: operands, then tiles 0..2 in flight
    {
        stage_q(rc, 0, HT * 32);
        stage_lse(rc);
        barrier_after_vmcnt(0);
        read_q_lse();
        lds_barrier();
        const __amdgpu_buffer_rsrc_t ridx = idx_rsrc(rc);
        nk0 = __builtin_amdgcn_raw_buffer_load_b32(ridx, (uint32_t)(0 * kTile + my_slot) * 4u, 0, 0);
        nk1 = __builtin_amdgcn_raw_buffer_load_b32(ridx, (uint32_t)(1 * kTile + my_slot) * 4u, 0, 0);
        nk2 = __builtin_amdgcn_raw_buffer_load_b32(ridx, (uint32_t)(2 * kTile + my_slot) * 4u, 0, 0);
        start_row(ric, rc);
    }

    for (; it * a.num_wg < a.R && rc < a.R; ++it) {
        const int ntiles = ntiles_of(ric);
        // the tile after whose MFMAs the next row is prefetched
        const int pf = ntiles > 3 ? 2 : ntiles - 1;
        auto extra = [&](int u) -> int { return u == pf ? kPrefetchOps : 0; };
        float* __restrict__ orow = a.out + rc * a.W;
        const __amdgpu_buffer_rsrc_t ridx = idx_rsrc(rc);
        const i32x4_t idesc = idx_desc(rc);
        const i32x4_t kdesc = k_desc(ric);
        const int64_t seg0 = ric.col0;
        const int64_t seg1 = ric.col0 + (ntiles > 0 ? ric.vis : 0);

        if (ntiles == 0) prefetch_next();

        f32x16_t acc_prev = {};
        // One tile: barrier; index row of tile+3 from the ring, of tile+6
        // into it; tile-2's head-tile sums (read now, added over steps
        // 1..7, stored at 8); the gather of tile+3 spread over the MFMAs of
        // this tile; tile-1's epilogue.
        auto body = [&](auto gtag, int tile) {
            constexpr bool kGather = decltype(gtag)::value;
            // Loads issued after the gather of this tile (in tile-3; vector
            // memory returns in order): index row and gather of tiles -2 and
            // -1, and the prefetch if it came after. Tile 0 waits for
            // everything (the previous row's stores and this row's Q
            // included); tiles 1 and 2 were gathered before that wait.
            int later = 63;
            if (tile == 0) {
                later = 0;
            } else if (tile >= 3) {
                later = extra(tile - 3) + 2 + 8 * (tile + 1 < ntiles) + 8 * (tile + 2 < ntiles) +
                        extra(tile - 2) + extra(tile - 1);
                later = later > 63 ? 63 : later;
            }
            barrier_after_vmcnt(later);
            const int32_t key = kring[(tile + 3) & 3][my_slot];
            dma_dword(idesc, ring_lds + (uint32_t)(((tile + 2) & 3) * 256), (tile + 6) * kTile * 4,
                      voff4);
            const int slot = (wave * kSlotsPerWave + lane) & (kTile - 1);
            const int pb = tile & 1;  // parity of tile - 2
            float parts[2 * HT];
#pragma unroll
            for (int w = 0; w < 2 * HT; ++w) parts[w] = red[pb][w][slot];
            const int32_t rows_off = row_off(ric, tile + 3, key);
            const uint32_t m0_rows = kbuf_lds + (uint32_t)(((tile + 3) & 3) * kBufBytes +
                                                           kSlotsPerWave * wave * kRowBytes);
            float tot = 0.0f;
            float sum_prev;
            const f32x16_t acc = qk_tile_seq<BF16, kGather>(
                kbuf[tile & 3], qa, col, half, acc_prev, l2, a.c_scale, &sum_prev, kdesc, m0_rows,
                rows_off, voff16, [&](int s) {
                    if (s == 1) {
                        tot = parts[0] + parts[1];
                        pin(tot);
                    } else if (s >= 2 && s < 2 * HT) {
                        tot += parts[s];
                        pin(tot);
                    } else if (s == 2 * HT) {
                        const bool mine = lane < kSlotsPerWave && tile >= 2;
                        vals[mine ? (tile - 2) * kTile + slot : kVcap + lane] = tot * a.inv_g;
                    }
                });
            red[(tile - 1) & 1][2 * wave + half][col] = sum_prev;  // tile 0: unused slot
            acc_prev = acc;
        };
        using G1 = std::integral_constant<bool, true>;
        using G0 = std::integral_constant<bool, false>;
        for (int tile = 0; tile < ntiles; ++tile) {
            if (tile + 3 < ntiles) body(G1{}, tile); else body(G0{}, tile);
            if (tile == pf) prefetch_next();
        }
        if (ntiles > 0)
            red[(ntiles - 1) & 1][2 * wave + half][col] = head_sum(acc_prev, l2, a.c_scale);

        // indices for this row's assembly
        int32_t jre[kPerThread];
#pragma unroll
        for (int i = 0; i < kPerThread; ++i)
            jre[i] = __builtin_amdgcn_raw_buffer_load_b32(ridx, (uint32_t)(tid + i * NT) * 4u, 0, 0);
        // all MFMAs done and every gather of this row has landed: K buffers
        // are free; partial sums visible
        lds_barrier();
        auto reduce = [&](int tile) {
            const int slot = (wave * kSlotsPerWave + lane) & (kTile - 1);
            const int pb = tile & 1;
            float tot = red[pb][0][slot];
#pragma unroll
            for (int w = 1; w < 2 * HT; ++w) tot += red[pb][w][slot];
            const bool mine = lane < kSlotsPerWave;
            vals[mine ? tile * kTile + slot : kVcap + lane] = tot * a.inv_g;
        };
        if (ntiles >= 2) reduce(ntiles - 2);
        if (ntiles >= 1) reduce(ntiles - 1);

        // the next row's Q (heads 0..95, into K buffers 0..2) and lse land
        // while this row is assembled in buffer 3
        const bool more = rn < a.R;
        if (more) {
            stage_q(rln, 0, 3 * 32);
            stage_lse(rln);
        }

        // assemble columns [seg0, seg1) of this row in LDS and write them once
        // (the next tile 0 barrier frees the stage for the next row's tile 3)
        for (int64_t c0 = seg0; c0 < seg1; c0 += kStage - 4) {
            const int64_t len = (seg1 - c0 < kStage - 4) ? seg1 - c0 : kStage - 4;
            const int m0 = (int)((rc * a.W + c0) & 3);
            lds_barrier();  // values complete; previous chunk written out
            for (int i = tid; i < (len + m0 + 3) >> 2; i += NT)
                reinterpret_cast<f32x4_t*>(stage)[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            lds_barrier();
#pragma unroll
            for (int i = 0; i < kPerThread; ++i) {
                const int t = tid + i * NT;
                const int32_t j = jre[i];
                if (t < ric.n && (uint32_t)j < (uint32_t)ric.vis) {
                    const int64_t c = ric.col0 + j - c0;
                    if (c >= 0 && c < len) stage[c + m0] = vals[t];
                }
            }
            lds_barrier();
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
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) consume(jre[i]);

        // the rest of the next row's Q into buffer 3 once the stage is free;
        // every wave reads its own heads back, then the K buffers take the
        // next row's first three tiles (ring slots: the index rows still in
        // flight into them land before these, in order)
        if (more) {
            lds_barrier();
            stage_q(rln, 3 * 32, HT * 32);
            barrier_after_vmcnt(0);
            read_q_lse();
            lds_barrier();
            start_row(rin, rn);
        }
        consume(nk0);
        consume(nk1);
        consume(nk2);
        zero_span(orow, 0, seg0, tid, NT);
        zero_span(orow, seg1, a.W, tid, NT);

        // the next row becomes current
        rc = rn;
        ric = rin;
    }
}

template <bool BF16, bool TND>
hipError_t launch_pipe_t(const KernelArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL((smla_pipe_kernel<BF16, TND>), dim3(a.num_wg), dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <bool BF16, bool TND>
hipError_t occupancy_pipe_t(int* out) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(
        out, reinterpret_cast<const void*>(&smla_pipe_kernel<BF16, TND>), 256, 0);
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

#define SMLA_DISPATCH(FN, ...)                                                        \
    do {                                                                              \
        if (ht == 1) {                                                                \
            if (bf16) return tnd ? FN<1, true, true>(__VA_ARGS__)                     \
                                 : FN<1, true, false>(__VA_ARGS__);                   \
            return tnd ? FN<1, false, true>(__VA_ARGS__) : FN<1, false, false>(__VA_ARGS__); \
        } else if (ht == 2) {                                                         \
            if (bf16) return tnd ? FN<2, true, true>(__VA_ARGS__)                     \
                                 : FN<2, true, false>(__VA_ARGS__);                   \
            return tnd ? FN<2, false, true>(__VA_ARGS__) : FN<2, false, false>(__VA_ARGS__); \
        } else if (ht == 4) {                                                         \
            if (bf16) return tnd ? FN<4, true, true>(__VA_ARGS__)                     \
                                 : FN<4, true, false>(__VA_ARGS__);                   \
            return tnd ? FN<4, false, true>(__VA_ARGS__) : FN<4, false, false>(__VA_ARGS__); \
        }                                                                             \
        return hipErrorInvalidValue;                                                  \
    } while (0)

bool uses_pipe(int ht, int64_t topk) { return ht == 4 && topk <= kVcap; }

hipError_t launch(const KernelArgs& a, int ht, bool bf16, bool tnd, hipStream_t stream) {
    if (uses_pipe(ht, a.K)) {
        if (bf16) return tnd ? launch_pipe_t<true, true>(a, stream) : launch_pipe_t<true, false>(a, stream);
        return tnd ? launch_pipe_t<false, true>(a, stream) : launch_pipe_t<false, false>(a, stream);
    }
    SMLA_DISPATCH(launch_t, a, stream);
}

hipError_t resident_per_cu(int ht, bool bf16, bool tnd, int64_t topk, int* out) {
    if (uses_pipe(ht, topk)) {
        if (bf16) return tnd ? occupancy_pipe_t<true, true>(out) : occupancy_pipe_t<true, false>(out);
        return tnd ? occupancy_pipe_t<false, true>(out) : occupancy_pipe_t<false, false>(out);
    }
    SMLA_DISPATCH(occupancy_t, out);
}

}  // namespace smla
