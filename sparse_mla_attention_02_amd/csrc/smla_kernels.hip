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
//  - keys are processed in tiles of 32: the workgroup gathers the 32
//    selected 1 KB rows of K into an XOR-swizzled LDS tile (one wave
//    instruction moves one whole row, fully coalesced), then every wave runs
//    32 v_mfma_f32_32x32x16 over D = 512 with its Q tile against the shared
//    K tile;
//  - the accumulator holds 16 heads x 1 key per lane; scale, the lse
//    subtraction and exp are fused as one FMA + v_exp_f32 (base 2), the 16
//    heads are summed in registers, the two half-waves by a cross-lane swap
//    and the head tiles through LDS;
//  - the output row is zero-filled first and the selected columns are then
//    written by single stores (indices of a row are distinct).
#include "smla_internal.h"

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
            int mid = (lo + hi + 1) >> 1;
            if (a.cu_q[mid] <= r) lo = mid; else hi = mid - 1;
        }
        b = lo;
        const int64_t q0 = a.cu_q[b];
        s1 = (int64_t)a.cu_q[b + 1] - q0;
        i = r - q0;
        kbase = a.cu_k[b];
        s2 = (int64_t)a.cu_k[b + 1] - kbase;
        // never reach past the k tensor or the output row
        if (kbase < 0) kbase = 0;
        if (s2 > a.rows_k - kbase) s2 = a.rows_k - kbase;
        if (s2 > a.W - kbase) s2 = a.W - kbase;
        if (s2 < 0) s2 = 0;
        col0 = kbase;
    } else {
        b = r / a.S1;
        i = r - b * a.S1;
        s1 = a.S1;
        s2 = a.S2;
        kbase = b * a.S2;
        col0 = 0;
    }
    int64_t vis = s2;
    if (a.mask_mode == 3) {
        const int64_t res = a.cmp_res ? (int64_t)a.cmp_res[b] : 0;
        const int64_t p1 = i + 1 + s2 * a.cmp_ratio + res - s1;
        vis = p1 > 0 ? p1 / a.cmp_ratio : 0;
        if (vis > s2) vis = s2;
    }
    int32_t n = a.K;
    if (a.topk_len) {
        n = a.topk_len[r];
        n = n < 0 ? 0 : (n > a.K ? a.K : n);
    }
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

// Buffer resource over the k rows of one batch / sequence (raw byte
// addressing; word 3 is the gfx9-family value for untyped buffer access).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t k_rsrc(const uint4* k4, int64_t kbase) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint4*>(k4 + kbase * kChunks),
                                             (short)0, 0x7fffffff, 0x00020000);
}

// Gather one 32-key tile of K into LDS with direct buffer->LDS loads: slot kk
// (key kk of the tile) is moved by wave kk % HT with one instruction (64
// lanes x 16 B = the whole 1 KB row, lane l -> chunk l; the row offset is a
// scalar).
template <int HT>
__device__ __forceinline__ void gather_tile(uint4* __restrict__ dst, __amdgpu_buffer_rsrc_t rs,
                                            int32_t idx_reg, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < kTile / HT; ++i) {
        const int kk = wave + i * HT;
        const int32_t j = __builtin_amdgcn_readlane(idx_reg, kk);
        if (j >= 0)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, SMLA_LDS(dst + kk * kPitch), 16,
                                                     lane << 4, j << 10, 0, 0);
    }
}

// S^T tile (this wave's 32 heads x 32 keys) = Q_tile . K_tile^T over D = 512.
template <bool BF16>
__device__ __forceinline__ f32x16_t qk_tile(const uint4* __restrict__ src, const uint4* qa,
                                            int col, int half) {
    f32x16_t acc = {};
    const uint4* row = src + col * kPitch + half;
#pragma unroll
    for (int s = 0; s < kChunks / 2; ++s) {
        const uint4 b = row[2 * s];
        acc = mfma_32x32x16<BF16>(qa[s], b, acc);
    }
    // keep only kLead operand reads in flight ahead of the MFMAs (bounds the
    // VGPRs the B operands take): kLead reads, then MFMA/read pairs
    constexpr int kLead = 4;
    __builtin_amdgcn_sched_group_barrier(0x100, kLead, 0);
#pragma unroll
    for (int s = 0; s < kChunks / 2 - kLead; ++s) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kLead, 0);
    return acc;
}

template <int HT, bool BF16, bool TND>
__global__ __launch_bounds__(64 * HT, 2) void smla_l1norm_kernel(KernelArgs a) {
    constexpr int NT = 64 * HT;
    // two K tiles (distinct objects, so loads into one never wait on reads of
    // the other) and the per-head-tile partial sums of the last two tiles
    __shared__ uint4 kbuf0[kTile * kPitch];
    __shared__ uint4 kbuf1[kTile * kPitch];
    __shared__ float red[2][HT][kTile];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: lives in an SGPR
    const int half = lane >> 5;   // which 8-element k-group of the MFMA operand
    const int col = lane & 31;    // key slot of the MFMA B operand / output column
    const uint4* __restrict__ k4 = static_cast<const uint4*>(a.k);
    const uint4* __restrict__ q4 = static_cast<const uint4*>(a.q);

    for (int64_t it = 0; it * a.num_wg < a.R; ++it) {
        const int64_t r = row_of(a, it, blockIdx.x);
        if (r >= a.R) continue;
        const RowInfo ri = decode_row<TND>(a, r);
        float* __restrict__ orow = a.out + r * a.W;
        const int32_t* __restrict__ irow = a.idx + r * a.K;
        const int ntiles = (ri.n + kTile - 1) / kTile;

        // key of slot `col` of a tile if that entry is used, else -1
        auto tile_key = [&](int tile) -> int32_t {
            const int t = tile * kTile + col;
            const int32_t j = (tile < ntiles && t < ri.n) ? irow[t] : -1;
            return (uint32_t)j < (uint32_t)ri.vis ? j : -1;
        };
        int32_t key_cur = tile_key(0);
        int32_t key_nxt = tile_key(1);

        // zero-fill the whole output row
        if ((a.W & 3) == 0) {
            f32x4_t* o4 = reinterpret_cast<f32x4_t*>(orow);
            const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
            for (int64_t c = tid; c < (a.W >> 2); c += NT) __builtin_nontemporal_store(z, o4 + c);
        } else {
            for (int64_t c = tid; c < a.W; c += NT) orow[c] = 0.0f;
        }

        // this wave's 32 heads of Q as MFMA A operands: lane (m, half) holds
        // head m, elements 16*s + 8*half .. +8 for k-step s
        const int head = wave * 32 + col;
        uint4 qa[kChunks / 2];
        if (head < a.G) {
            const u32x4_t* qp =
                reinterpret_cast<const u32x4_t*>(q4 + (r * a.G + head) * kChunks);
#pragma unroll
            for (int s = 0; s < kChunks / 2; ++s)
                qa[s] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(qp + 2 * s + half));
        } else {
#pragma unroll
            for (int s = 0; s < kChunks / 2; ++s) qa[s] = make_uint4(0, 0, 0, 0);
        }

        // lse (base 2) of the 16 heads this lane's accumulator holds:
        // element e of the 32x32 accumulator is head 8*(e/4) + 4*half + e%4
        float l2[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int h = wave * 32 + 8 * (e >> 2) + 4 * half + (e & 3);
            l2[e] = h < a.G ? a.lse[r * a.G + h] * kLog2e : __builtin_inff();
        }

        const __amdgpu_buffer_rsrc_t krs = k_rsrc(k4, ri.kbase);
        if (ntiles > 0) gather_tile<HT>(kbuf0, krs, key_cur, wave, lane);

        int32_t key_prev = -1;
        // one tile: finish the previous tile's head sum, start the next
        // tile's gather, then QK^T + exp + head sum of this tile
        auto body = [&](int tile, const uint4* cur, uint4* nxt) {
            // all gathers landed, zero-fill stores and partial sums done
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if constexpr (HT > 1) {
                if (tile > 0 && wave == 0 && lane < kTile) {
                    const int pb = (tile - 1) & 1;
                    float tot = red[pb][0][lane];
#pragma unroll
                    for (int w = 1; w < HT; ++w) tot += red[pb][w][lane];
                    if (key_prev >= 0) orow[ri.col0 + key_prev] = tot * a.inv_g;
                }
            }
            if (tile + 1 < ntiles) gather_tile<HT>(nxt, krs, key_nxt, wave, lane);
            const int32_t key_nn = tile_key(tile + 2);

            const f32x16_t acc = qk_tile<BF16>(cur, qa, col, half);
            // exp(s - lse) = 2^(acc*scale*log2e - lse*log2e), summed over heads
            float sum = 0.0f;
#pragma unroll
            for (int e = 0; e < 16; ++e)
                sum += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[e], a.c_scale, -l2[e]));
            sum += __shfl_xor(sum, 32);
            if constexpr (HT > 1) {
                if (lane < kTile) red[tile & 1][wave][lane] = sum;
            } else {
                if (lane < kTile && key_cur >= 0) orow[ri.col0 + key_cur] = sum * a.inv_g;
            }
            key_prev = key_cur;
            key_cur = key_nxt;
            key_nxt = key_nn;
        };
        for (int tile = 0; tile < ntiles; tile += 2) {
            body(tile, kbuf0, kbuf1);
            if (tile + 1 < ntiles) body(tile + 1, kbuf1, kbuf0);
        }
        // head sum of the last tile; also keeps the next row's first gather
        // from overwriting a tile some wave still reads
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if constexpr (HT > 1) {
            if (ntiles > 0 && wave == 0 && lane < kTile) {
                const int pb = (ntiles - 1) & 1;
                float tot = red[pb][0][lane];
#pragma unroll
                for (int w = 1; w < HT; ++w) tot += red[pb][w][lane];
                if (key_prev >= 0) orow[ri.col0 + key_prev] = tot * a.inv_g;
            }
        }
    }
}

template <int HT, bool BF16, bool TND>
hipError_t launch_t(const KernelArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL((smla_l1norm_kernel<HT, BF16, TND>), dim3(a.num_wg), dim3(64 * HT),
                       0, stream, a);
    return hipGetLastError();
}

template <int HT, bool BF16, bool TND>
hipError_t occupancy_t(int* out) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(
        out, reinterpret_cast<const void*>(&smla_l1norm_kernel<HT, BF16, TND>), 64 * HT, 0);
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

hipError_t launch(const KernelArgs& a, int ht, bool bf16, bool tnd, hipStream_t stream) {
    SMLA_DISPATCH(launch_t, a, stream);
}

hipError_t resident_per_cu(int ht, bool bf16, bool tnd, int* out) {
    SMLA_DISPATCH(occupancy_t, out);
}

}  // namespace smla
