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


// The file is compiled twice: once for the pipelined and general kernels and
// once, with SMLA_LSE_TU defined, for the softmax_lse kernel. The first
// build keeps MFMA results in VGPRs (-amdgpu-mfma-vgpr-form), which the
// pipelined kernel's epilogue relies on; the lse kernel with one 32-head
// block per wave measured 9% slower that way, so it is built with the
// compiler's default.
#ifdef SMLA_LSE_TU
#pragma clang diagnostic ignored "-Wunused-function"
#pragma clang diagnostic ignored "-Wunused-const-variable"
#endif

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
constexpr float kLn2 = 0.6931471805599453f;
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

// Writes row[0, w) from LDS (src[c] holds column c) with 16-byte
// non-temporal stores where the row is 16-byte aligned, single floats for
// the unaligned head and tail.
__device__ __forceinline__ void write_row(float* __restrict__ row, const float* src, int64_t w,
                                          int tid, int nt) {
    const int64_t head = ((16 - (reinterpret_cast<uintptr_t>(row) & 15)) & 15) >> 2;
    const int64_t h = head < w ? head : w;
    if (tid < h) row[tid] = src[tid];
    const int64_t n4 = (w - h) >> 2;
    f32x4_t* o4 = reinterpret_cast<f32x4_t*>(row + h);
    if (h == 0) {
        const f32x4_t* s4 = reinterpret_cast<const f32x4_t*>(src);
        for (int64_t i = tid; i < n4; i += nt) __builtin_nontemporal_store(s4[i], o4 + i);
    } else {
        for (int64_t i = tid; i < n4; i += nt) {
            const float* p = src + h + 4 * i;
            __builtin_nontemporal_store(f32x4_t{p[0], p[1], p[2], p[3]}, o4 + i);
        }
    }
    const int64_t t0 = h + 4 * n4;
    if (tid < w - t0) row[t0 + tid] = src[t0 + tid];
}

// Read-only int32 data at a wave-uniform address: the constant address
// space lets the compiler use scalar loads (waited with lgkmcnt, so they do
// not queue behind the vector loads in flight).
typedef const __attribute__((address_space(4))) int32_t* cint_ptr;
__device__ __forceinline__ int32_t uload(const int32_t* p, int64_t i) {
    return ((cint_ptr)p)[i];
}

// Marks a loaded register as used here, on every path: the compiler then
// waits for its load at this point instead of before a later reuse of the
// register, where the wait would also cover the loads in flight since.
__device__ __forceinline__ void consume(int32_t v) { asm volatile("" ::"v"(v)); }
// Keeps a value's computation at this point of the instruction stream (pure
// arithmetic is otherwise free to move to its first use).
__device__ __forceinline__ void pin(float& v) { asm volatile("" : "+v"(v)); }
// The same for an integer kept in a vector register.
__device__ __forceinline__ void pin_v(int32_t& v) { asm volatile("" : "+v"(v)); }
// The same for a wave-uniform value kept in a scalar register (the
// readfirstlane costs nothing where the compiler already knows the value is
// uniform, and makes it legal where it cannot prove it).
__device__ __forceinline__ void pin_s(int32_t& v) {
    v = __builtin_amdgcn_readfirstlane(v);
    asm volatile("" : "+s"(v));
}

// A compile-time integer (a tile parity, tile & 1, so that the buffer
// addresses of a tile fold into constants; or a flag).
template <int P>
struct Par {
    static constexpr int value = P;
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
            const int mid = (lo + hi + 1) >> 1;
            if (uload(a.cu_q, mid) <= r) lo = mid; else hi = mid - 1;
        }
        b = lo;
        const int64_t q0 = uload(a.cu_q, b);
        s1 = (int64_t)uload(a.cu_q, b + 1) - q0;
        i = r - q0;
        kbase = uload(a.cu_k, b);
        s2 = (int64_t)uload(a.cu_k, b + 1) - kbase;
        // never reach past the k tensor or the output row (K-wide rows hold
        // entries, not key columns)
        if (kbase < 0) kbase = 0;
        if (s2 > a.rows_k - kbase) s2 = a.rows_k - kbase;
        if (!a.kwide && s2 > a.W - kbase) s2 = a.W - kbase;
        if (s2 < 0) s2 = 0;
        col0 = a.kwide ? 0 : kbase;
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
    // seqused_k: keys past the count take no part (the visible keys stay a
    // prefix); seqused_q: a query past the count uses nothing. Both counts
    // are clamped to the sequence's lengths.
    if (a.su_k) {
        const int64_t ku = uload(a.su_k, b);
        if (ku < vis) vis = ku < 0 ? 0 : ku;
    }
    if (a.su_q && i >= (int64_t)uload(a.su_q, b)) vis = 0;
    // entries to look at (selectBlockCount): topk_length clamped to [0, K];
    // without it K, or under the causal mask no more than the visible keys.
    // Dense (no sparse_indices): the row's keys in order, so the visible ones
    // are its leading entries
    int32_t n = a.K;
    if (a.dense) {
        n = vis < a.K ? (int32_t)vis : a.K;
    } else if (a.topk_len) {
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

#ifndef SMLA_LSE_TU
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

#endif  // !SMLA_LSE_TU

#ifdef SMLA_LSE_TU
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

// Lanes of accumulator element e that hold a used entry, as a wave mask:
// lanes 0..31 hold slot k = 8*(e/4) + e%4 of the tile, lanes 32..63 slot
// k + 4, and bit kk of the wave-uniform `slots` says slot kk is used. The
// mask is built by the scalar unit.
__device__ __forceinline__ uint64_t used_lanes(uint32_t slots, int e) {
    const int k = 8 * (e >> 2) + (e & 3);
    const uint64_t lo = ((slots >> k) & 1u) ? 0x00000000ffffffffull : 0ull;
    const uint64_t hi = ((slots >> (k + 4)) & 1u) ? 0xffffffff00000000ull : 0ull;
    return lo | hi;
}

// (lane in m) ? a : b, with the lane mask in a scalar register pair
__device__ __forceinline__ float select_lanes(uint64_t m, float a, float b) {
    float r;
    asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(r) : "v"(b), "v"(a), "s"(m));
    return r;
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

#endif  // SMLA_LSE_TU

#ifndef SMLA_LSE_TU
// ---------------------------------------------------------------------------
// Helpers of the pipelined kernel below.
//
// One wave per SIMD issues every instruction in the time of the MFMAs, so
// its tile body is laid out by hand (scheduling barriers per k-step, empty
// asm statements that keep arithmetic in its step).
//
// All loads into LDS are inline assembly: the compiler's wait-count
// tracking cannot follow LDS buffers reused across loop iterations and would
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
        // the counts in use; anything else waits for all
        case 7: waitcnt_vm_lgkm0<7>(); break;
        default: waitcnt_vm_lgkm0<0>(); break;
    }
    asm volatile("s_barrier" ::: "memory");
}
// barrier that publishes this wave's LDS writes (loads into LDS excluded)
__device__ __forceinline__ void lds_barrier() {
    waitcnt_vm_lgkm0<63>();
    asm volatile("s_barrier" ::: "memory");
}

// Buffer descriptor as four dwords (base, range in bytes, gfx9 untyped
// format); offsets at or past `bytes` read as zero.
typedef __attribute__((ext_vector_type(4))) int32_t i32x4_t;
__device__ __forceinline__ i32x4_t raw_desc(const void* base, uint32_t bytes) {
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    return i32x4_t{(int32_t)(uint32_t)p, (int32_t)((uint32_t)(p >> 32) & 0xffffu), (int32_t)bytes,
                   0x00020000};
}
// A descriptor chosen by a wave-uniform condition, kept in scalar registers
// (the inline-asm loads take it as an "s" operand).
__device__ __forceinline__ i32x4_t uniform_desc(i32x4_t d) {
    return i32x4_t{__builtin_amdgcn_readfirstlane(d[0]), __builtin_amdgcn_readfirstlane(d[1]),
                   __builtin_amdgcn_readfirstlane(d[2]), __builtin_amdgcn_readfirstlane(d[3])};
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
// The loads of one stream in the tile loop go to consecutive LDS rows: the
// first sets M0 and each load then steps it by `step` in place, so the loads
// after the first need neither an M0 write nor its wait state (the compiler
// never writes M0 in the pipelined kernel; these are its only users while a
// stream runs).
__device__ __forceinline__ void dma_row_first(i32x4_t desc, uint32_t m0, int32_t soff,
                                              uint32_t voff, int32_t step) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen lds\n\t"
        "s_add_u32 m0, m0, %4"
        :
        : "s"(m0), "v"(voff), "s"(desc), "s"(soff), "s"(step)
        : "memory", "m0", "scc");
}
__device__ __forceinline__ void dma_row_next(i32x4_t desc, int32_t soff, uint32_t voff,
                                             int32_t step) {
    asm volatile(
        "buffer_load_dwordx4 %0, %1, %2 offen lds\n\t"
        "s_add_u32 m0, m0, %3"
        :
        : "v"(voff), "s"(desc), "s"(soff), "s"(step)
        : "memory", "m0", "scc");
}
// The same with the non-temporal hint, for data read once (Q rows, index
// lists): the key rows, which are gathered again and again, keep their
// place in L2.
__device__ __forceinline__ void dma_row_nt(i32x4_t desc, uint32_t m0, int32_t soff, uint32_t voff) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen nt lds"
        :
        : "s"(m0), "v"(voff), "s"(desc), "s"(soff)
        : "memory", "m0");
}
__device__ __forceinline__ void dma_dword_nt(i32x4_t desc, uint32_t m0, int32_t soff, uint32_t voff) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "buffer_load_dword %1, %2, %3 offen nt lds"
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

constexpr int kRowBytes = kPitch * 16;          // one key row in LDS

// ---------------------------------------------------------------------------
// Wide pipelined kernel for rows of 65..128 heads with at most kVcap indices.
//
// LDS delivers 128 bytes per clock per CU: one 1 KB K-operand read per
// 32-cycle MFMA on each of the four SIMDs already uses all of it, before the
// gathers write into LDS. So each wave here takes 64 heads (two 32-row MFMA
// blocks that share every K operand read) by 32 keys, and the four waves of
// the workgroup cover 128 heads by a 64-key tile: wave w takes heads
// 64 (w & 1) .. +63 and keys 32 (w >> 1) .. +31 of each tile. Two tiles live
// in LDS; the gather of tile t+1 (16 rows per wave, loaded straight into
// LDS) is spread over the first half of the MFMAs of tile t. The row's index
// list sits in LDS, so the tile loop reads no other global memory.
//
// Output: a row is zero-filled (at the end of the previous row) before the
// barrier of its first tile, which waits for every memory operation of the
// wave, so the zeros reach L2 before any wave goes on; each tile's values are
// then stored straight to their columns by the wave that finishes them, two
// tiles later, after the gather loads of that step sequence.
//
// Accumulators alternate between two register sets from tile to tile, so
// the epilogue of tile t reads its scores where the MFMAs of tile t left
// them while the MFMAs of tile t+1 fill the other set.

constexpr int kWideKeys = 64;                      // keys per tile
constexpr int kRowCap = 4096;                      // widest output row assembled in LDS
constexpr int kWideBufBytes = kWideKeys * kRowBytes;

// One 64-key tile t of one wave, 32 steps. Step s issues the two MFMAs of
// k-step s (one shared B operand, from an 8-deep ring of operand registers),
// the LDS read of the operand 8 steps ahead, one element of the previous
// tile's epilogue in three independent pieces (FMA of element s, exp of
// element s-1, sum of element s-2), and the gather loads of this wave's 16
// rows of later tiles: rows 7..15 of tile t+1 at steps 1..9 (from `offa`,
// to LDS address m0a + (r-7) stepa) and rows 0..6 of tile t+2 at steps
// 25..31 (offsets from `offs_b(key_b())`: the key read in step 12, the
// offsets formed in step 20, so that no step waits for an LDS read issued
// just before it; returned in `offb` for the next tile; to m0b + r
// stepb). Each stream has its own buffer descriptor: a stream whose tile
// does not exist loads rows of the next query row's Q into the free buffer
// instead, or (a step of 0) sends its loads to one dummy row. Each row
// offset is read into a scalar register one step before its load.
//
// The workgroup barrier sits after the MFMAs of step kBar = 24: by then every
// wave has read its last operand of tile t (step 31's, read in step 23) and
// waited for its own loads of tile t+1 (the last issued in step 9), so after
// it the operand reads run on into tile t+1 (`nxt`) and the loads of tile
// t+2 may overwrite tile t's buffer. Tile boundaries then need no barrier and
// the MFMA stream does not drain between tiles. `mid(s)` is the caller's
// spread-out work, called at the end of step s.
constexpr int kBarStep = 24;
template <bool BF16, typename Mid1, typename Mid2>
__device__ __forceinline__ void wide_tile(const uint4* __restrict__ cur,
                                          const uint4* __restrict__ nxt, uint4 (&ring)[8],
                                          const uint4* qa0, const uint4* qa1,
                                          const f32x16_t& prev0, const f32x16_t& prev1,
                                          const float* l2, float c, float& pt, float& pex,
                                          float& psum, i32x4_t desc_a, i32x4_t desc_b,
                                          int32_t m0a, int32_t stepa, int32_t offa, int32_t m0b,
                                          int32_t stepb, const int32_t& offb, uint32_t voff,
                                          Mid1 mid1, Mid2 mid2, f32x16_t& acc0,
                                          f32x16_t& acc1) {
    constexpr int kSteps = kChunks / 2;
    constexpr int kLead = 8;
    acc0 = f32x16_t{};
    acc1 = f32x16_t{};
    float sum = 0.0f, t = 0.0f, ex = 0.0f;
    int32_t soa[2] = {0, 0}, sob[2] = {0, 0};
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
        // One wave per SIMD issues one instruction per 4 cycles, and the matrix
        // core takes 32 cycles per MFMA: the step's other instructions are split
        // between the two MFMAs (about six issue slots before each MFMA's
        // successor can start), instead of queueing after the second one.
        __builtin_amdgcn_sched_barrier(0);
        acc0 = mfma_32x32x16<BF16>(qa0[s], ring[s & 7], acc0);
        // keeps the MFMA in its slot (as a pure operation it may otherwise be
        // sunk towards the far uses of the accumulator); the accumulators live
        // in VGPRs, so the epilogue reads the scores without a copy (Q, the A
        // operand, sits in AGPRs, which the matrix core reads at full rate)
        asm volatile("" ::"v"(acc0));
        // first gap: the previous tile's last two elements (step 0), the sum of
        // element s-2, the exp of element s-1, the fma of element s and the
        // scalar offset of the next step's load
        if (s == 0) {
            psum += pex;
            pin(psum);
            pex = __builtin_amdgcn_exp2f(pt);
            pin(pex);
        }
        if (s >= 2) {
            sum += ex;
            pin(sum);
        }
        if (s >= 1) {
            ex = __builtin_amdgcn_exp2f(t);
            pin(ex);
        }
        // (the load of step s+1 takes it: a scalar written by a VALU
        // instruction needs five wait states before a load reads it)
        // the fma of element s (the previous tile's score, read where its
        // MFMAs left it)
        t = __builtin_fmaf(s < 16 ? prev0[s] : prev1[s - 16], c, -l2[s]);
        pin(t);
        if (s <= 8) {
            soa[s & 1] = __builtin_amdgcn_readlane(offa, s + 7);
            pin_s(soa[s & 1]);
        } else if (s >= 24 && s <= 30) {
            sob[s & 1] = __builtin_amdgcn_readlane(offb, s - 24);
            pin_s(sob[s & 1]);
        }
        mid1(s);
        __builtin_amdgcn_sched_barrier(0);
        acc1 = mfma_32x32x16<BF16>(qa1[s], ring[s & 7], acc1);
        asm volatile("" ::"v"(acc1));
        // second gap: the operand read 8 steps ahead and the gather loads
        if (s == 0) {
            psum += pex;  // the previous tile's sum, written out by mid1(1)
            pin(psum);
        }
        if (s == kBarStep) barrier_after_vmcnt(0);
        ring[(s + kLead) & 7] =
            s + kLead < kSteps ? cur[2 * (s + kLead)] : nxt[2 * (s + kLead - kSteps)];
        if (s == 1)  // stream A: row s + 6 of tile t+1
            dma_row_first(desc_a, (uint32_t)m0a, soa[0], voff, stepa);
        else if (s >= 2 && s <= 9)
            dma_row_next(desc_a, soa[(s - 1) & 1], voff, stepa);
        if (s == 25)  // stream B: row s - 25 of tile t+2
            dma_row_first(desc_b, (uint32_t)m0b, sob[0], voff, stepb);
        else if (s >= 26)
            dma_row_next(desc_b, sob[(s - 1) & 1], voff, stepb);
        mid2(s);
    }
    __builtin_amdgcn_sched_barrier(0);
    // this tile's last two elements are finished by the next tile's step 0
    pt = t;
    pex = ex;
    psum = sum;
}


// ROWBUF (output rows of at most kRowCap columns): each row is assembled in
// LDS (zeroed at the row start, values written as they are finished) and
// written out once with 16-byte stores at the row end; the index list is then
// single-buffered to make room. Otherwise rows are zero-filled in memory and
// the values stored straight to their columns.
template <bool BF16, bool TND, bool ROWBUF, bool DENSE>
__global__ __launch_bounds__(256, 1) void smla_wide_kernel(KernelArgs a) {
    constexpr int HT = 4;
    constexpr int NT = 256;
    constexpr int kRowsPerWave = kWideKeys / HT;      // gathered rows per wave and tile
    constexpr int kIdxOps = kVcap / 64 / HT;          // loads of one index list per wave
    __shared__ uint4 kbuf[2][kWideKeys * kPitch];     // tile t in buffer t % 2
    __shared__ int32_t ibuf[ROWBUF ? 1 : 2][kVcap];   // index lists: this row (, next row)
    __shared__ __attribute__((aligned(16))) float rowbuf[ROWBUF ? kRowCap + 64 : 4];  // row, sinks
    __shared__ float red[2][4][kWideKeys];            // partial sums, last two tiles
    __shared__ float redl[4][kWideKeys];              // partial sums of a row's last tile
    __shared__ float lsebuf[HT * 32];                 // the next row's lse
    __shared__ uint4 dummy[64];                       // loads of a tile with nothing to gather

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hg = wave & 1;          // head group: heads 64 hg .. 64 hg + 63
    const int kh = wave >> 1;         // key half: keys 32 kh .. 32 kh + 31 of a tile
    const int half = lane >> 5;
    const int col = lane & 31;
    // this wave gathers rows 16 w .. 16 w + 15 of every tile; lane l < 16
    // holds the index of row 16 w + l
    const int my_slot = kRowsPerWave * wave + (lane & 15);
    const uint4* __restrict__ q4 = static_cast<const uint4*>(a.q);
    const char* __restrict__ kbytes = static_cast<const char*>(a.k);
    const uint32_t kbuf_lds = lds_addr(kbuf);
    const uint32_t ibuf_lds = lds_addr(ibuf);
    const uint32_t lse_lds = lds_addr(lsebuf);
    const uint32_t dummy_lds = lds_addr(dummy);
    const uint32_t voff16 = (uint32_t)lane << 4;
    const uint32_t voff4 = (uint32_t)lane << 2;

    int64_t it = 0;
    int64_t rc = row_of(a, 0, blockIdx.x);   // num_wg <= R, so rc < R
    RowInfo ric = decode_row<TND>(a, rc);
    uint4 qa0[kChunks / 2], qa1[kChunks / 2];
    float l2[32];
    int64_t rn = a.R, rln = rc;             // next row, and the row its loads read
    RowInfo rin = ric;
    int ib = 0;                             // ibuf slot of the current row

    auto k_desc = [&](const RowInfo& ri) {
        const int64_t rows = a.rows_k - ri.kbase;
        const int64_t bytes = rows * 1024;
        return raw_desc(kbytes + ri.kbase * 1024,
                        bytes > 0xffffffffll ? 0xffffffffu : (uint32_t)(bytes < 0 ? 0 : bytes));
    };
    // row r's index list into ibuf[slot] (kIdxOps loads; entries past K read
    // as zero)
    auto load_idx_row = [&](int64_t r, int slot) {
        if (DENSE) return;  // no index list: entry t is key t
        const i32x4_t id = raw_desc(a.idx + r * a.K, (uint32_t)a.K * 4u);
#pragma unroll
        for (int i = 0; i < kIdxOps; ++i) {
            const int c = kIdxOps * wave + i;  // 256-byte piece of the list
            dma_dword_nt(id, ibuf_lds + (uint32_t)(slot * kVcap * 4 + c * 256), c * 256, voff4);
        }
    };
    // Q and lse pass through LDS as whole rows (a load straight into the MFMA
    // operand layout touches 32 head rows per instruction and is several
    // times slower through the address unit). Q of row r, heads [h0, h1),
    // into the K buffers: head h -> buffer h / 64, row h % 64.
    auto stage_q = [&](int64_t r, int h0, int h1) {
        const i32x4_t qd = raw_desc(q4 + r * a.G * kChunks, (uint32_t)a.G * 1024u);
        for (int h = h0 + wave; h < h1; h += HT)
            dma_row_nt(qd, kbuf_lds + (uint32_t)((h >> 6) * kWideBufBytes + (h & 63) * kRowBytes),
                    h * 1024, voff16);
    };
    auto stage_lse = [&](int64_t r) {
        const i32x4_t ld = raw_desc(a.lse + r * a.G, (uint32_t)a.G * 4u);
        if (wave < 2)  // 2 x 64 heads
            dma_dword(ld, lse_lds + (uint32_t)(wave * 256), wave * 256, voff4);
    };
    // this wave's Q (A operands of block j: lane (m, half) holds head
    // 64 hg + 32 j + m, elements 16s + 8 half .. +8 of k-step s) and its lse
    // in log2 units (padded heads +inf), from LDS
    auto read_q_lse = [&]() {
        const uint4* r0 = kbuf[hg] + col * kPitch + half;
        const uint4* r1 = kbuf[hg] + (32 + col) * kPitch + half;
#pragma unroll
        for (int s = 0; s < kChunks / 2; ++s) {
            qa0[s] = r0[2 * s];
            qa1[s] = r1[2 * s];
        }
#pragma unroll
        for (int e = 0; e < 32; ++e) {
            // (the read is unconditional, h < 128 always, and the padding
            // heads take +inf by a select: a conditional read compiles to a
            // branch per element)
            const int h = 64 * hg + 32 * (e >> 4) + 8 * ((e & 15) >> 2) + 4 * half + (e & 3);
            const float v = lsebuf[h];
            l2[e] = h < a.G ? v * kLog2e : __builtin_inff();
        }
    };
    // the next row of this workgroup, decoded (its scalar loads waited for
    // here, so that later LDS waits can count), its output zero-filled and
    // its index list loaded
    auto decode_next = [&]() {
        rn = (it + 1) * a.num_wg < a.R ? row_of(a, it + 1, blockIdx.x) : a.R;
        rln = rn < a.R ? rn : rc;  // the last row loads itself again (unused)
        rin = decode_row<TND>(a, rln);
        waitcnt_vm_lgkm0<63>();
    };
    auto prepare_next = [&]() {
        if (!ROWBUF && rn < a.R) zero_span(a.out + rn * a.W, 0, a.W, tid, NT);
        load_idx_row(rln, ROWBUF ? 0 : ib ^ 1);
    };
    // Q of row r, heads 64 buf + 16 w + i for i in [i0, i1), into rows
    // 16 w + i of K buffer buf (the layout in which the last tiles of a row
    // stage the next row's Q in the buffers they free)
    auto stage_q_rows = [&](int64_t r, int buf, int i0, int i1) {
        const i32x4_t qd = raw_desc(q4 + r * a.G * kChunks, (uint32_t)a.G * 1024u);
        for (int i = i0; i < i1; ++i) {
            // (uniform; said so for the scalar operands of the load)
            const uint32_t m0 = __builtin_amdgcn_readfirstlane(
                kbuf_lds + (uint32_t)(buf * kWideBufBytes + (kRowsPerWave * wave + i) * kRowBytes));
            const int32_t so =
                __builtin_amdgcn_readfirstlane((64 * buf + kRowsPerWave * wave + i) * 1024);
            dma_row_nt(qd, m0, so, voff16);
        }
    };
    auto ntiles_of = [](const RowInfo& ri) { return (ri.n + kWideKeys - 1) / kWideKeys; };
    // byte offset of the key row of slot my_slot of `tile` holding raw index
    // j: j's row if the entry is used, else row 0 (loaded, never read)
    auto row_off = [&](const RowInfo& ri, int tile, int32_t j) -> int32_t {
        // (bitwise: a short-circuit here compiles to a branch)
        return ((tile * kWideKeys + my_slot < ri.n) & ((uint32_t)j < (uint32_t)ri.vis)) ? (j << 10)
                                                                                         : 0;
    };
    // A row's start: tile 0 (16 rows) into buffer 0 and rows 0..6 of tile 1
    // into buffer 1 (to the dummy row when there is no tile 1), 23 loads in
    // all for a row with tiles; returns each lane's row offset in tile 1 for
    // the loads of its rows 7..15 in tile 0.
    auto start_row = [&](const RowInfo& ri, int slot) -> int32_t {
        const int nt = __builtin_amdgcn_readfirstlane(ntiles_of(ri));  // uniform
        if (nt == 0) return 0;
        const i32x4_t kd = k_desc(ri);
        const int32_t* il = ibuf[slot];
        const int32_t o0 = row_off(ri, 0, DENSE ? my_slot : il[my_slot]);
        const int32_t o1 =
            row_off(ri, 1, nt > 1 ? (DENSE ? kWideKeys + my_slot : il[kWideKeys + my_slot]) : 0);
        int32_t so[kRowsPerWave];
#pragma unroll
        for (int i = 0; i < kRowsPerWave; ++i) {
            so[i] = __builtin_amdgcn_readlane(o0, i);
            pin_s(so[i]);
        }
        int32_t m0 = (int32_t)(kbuf_lds + (uint32_t)(kRowsPerWave * wave * kRowBytes));
        pin_s(m0);
#pragma unroll
        for (int i = 0; i < kRowsPerWave; ++i) {
            dma_row(kd, (uint32_t)m0, so[i], voff16);
            m0 += kRowBytes;
            pin_s(m0);
        }
#pragma unroll
        for (int i = 0; i < 7; ++i) {
            so[i] = __builtin_amdgcn_readlane(o1, i);
            pin_s(so[i]);
        }
        const int32_t step1 = nt > 1 ? kRowBytes : 0;
        m0 = __builtin_amdgcn_readfirstlane(
            (int32_t)(nt > 1 ? kbuf_lds + (uint32_t)(kWideBufBytes + kRowsPerWave * wave * kRowBytes)
                             : dummy_lds));
        pin_s(m0);
#pragma unroll
        for (int i = 0; i < 7; ++i) {
            dma_row(kd, (uint32_t)m0, so[i], voff16);
            m0 += step1;
            pin_s(m0);
        }
        return o1;
    };

    // ---- first row: operands, index list and zeroed output, then tile 0 in
    // flight
    load_idx_row(rc, 0);
    stage_q(rc, 0, HT * 32);
    stage_lse(rc);
    if (!ROWBUF) zero_span(a.out + rc * a.W, 0, a.W, tid, NT);
    barrier_after_vmcnt(0);
    read_q_lse();
    lds_barrier();
    int32_t offa = start_row(ric, 0);
    uint4 ring[8];

    for (; it * a.num_wg < a.R && rc < a.R; ++it) {
        // (uniform, but the compiler cannot always see it: say so, so that
        // the LDS addresses derived from it stay in scalar registers)
        const int ntiles = __builtin_amdgcn_readfirstlane(ntiles_of(ric));
        const i32x4_t kdesc = k_desc(ric);
        // the next row, decoded now: the last tiles of this row load its Q
        decode_next();
        const bool more = rn < a.R;
        const i32x4_t qdesc = raw_desc(q4 + rln * a.G * kChunks, (uint32_t)a.G * 1024u);
        // each lane's byte offset in Q of the head that rows 16 w + lane of
        // K buffer buf take when it holds the next row's Q
        auto q_off = [&](int buf) -> int32_t {
            return (64 * buf + kRowsPerWave * wave + (lane & 15)) * 1024;
        };
        const int32_t* __restrict__ irow = ibuf[ib];
        // Finish entry `e` = tile*64 + slot (slot 16 w + lane for lanes < 16):
        // the sum of its four partial sums over G, stored to its column if
        // the entry is used. The store is one buffer store per call whatever
        // the lanes hold (lanes with nothing to store give an offset past
        // the row, which the buffer range check drops).
        const int slot = (kRowsPerWave * wave + lane) & (kWideKeys - 1);
        const int64_t obytes = a.W * 4;
        const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
            a.out + rc * a.W, (short)0, obytes < 0x7ffffff0ll ? (int)obytes : 0x7ffffff0,
            0x00020000);
        auto store_value = [&](int tile, float tot, int32_t j) {
            const int e = tile * kWideKeys + slot;
            const bool used =
                lane < kRowsPerWave && tile >= 0 && e < ric.n && (uint32_t)j < (uint32_t)ric.vis;
            // the entry's column: its key's (col0 + j), or K-wide the entry e
            const int32_t c = a.kwide ? e : (int32_t)(ric.col0 + j);
            if (ROWBUF) {
                // (c < W <= kRowCap; other lanes write their own sink)
                rowbuf[used ? c : kRowCap + lane] = tot * a.inv_g;
            } else {
                // (the builtin's data operand is an integer: pass the bits)
                __builtin_amdgcn_raw_buffer_store_b32(
                    __builtin_bit_cast(uint32_t, tot * a.inv_g), orsrc,
                    used ? (int)((uint32_t)c * 4u) : 0x7ffffff0, 0, 0);
            }
        };

        if (ROWBUF) {  // zeroed before the barrier, so before any value lands
            for (int i = tid; i < (int)((a.W + 3) >> 2); i += NT)
                reinterpret_cast<f32x4_t*>(rowbuf)[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        // tile 0 has landed (tile 1's first rows may still be in flight);
        // the operands of its first 8 steps into the ring
        barrier_after_vmcnt(7);
        {
            const uint4* r0 = kbuf[0] + (32 * kh + col) * kPitch + half;
#pragma unroll
            for (int i = 0; i < 8; ++i) ring[i] = r0[2 * i];
        }
        f32x16_t xa0, xa1, xb0 = {}, xb1 = {};
        // The scalar state of a tile's two load streams: buffer descriptors,
        // LDS destinations and their steps. A stream whose tile does not exist
        // takes the next row's Q (stream A only from tile 1 on: tile 0's
        // offsets come from the row start) or, with no next row, the dummy row.
        struct Ctl {
            int32_t da[4], db[4];
            int32_t m0a, m0b, sa, sb;
        };
        auto ctl_of = [&](auto P, int tile) -> Ctl {
            constexpr int par = decltype(P)::value;  // tile & 1
            const bool has1 = tile + 1 < ntiles, has2 = tile + 2 < ntiles;
            const bool qa = !has1 && more && tile >= 1, qb = !has2 && more;
            const i32x4_t da = uniform_desc(has1 ? kdesc : qdesc);
            const i32x4_t db = uniform_desc(has2 ? kdesc : qdesc);
            Ctl r;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                r.da[i] = da[i];
                r.db[i] = db[i];
            }
            r.m0a = __builtin_amdgcn_readfirstlane((int32_t)(
                has1 || qa ? kbuf_lds + (uint32_t)((1 - par) * kWideBufBytes +
                                                   (kRowsPerWave * wave + 7) * kRowBytes)
                           : dummy_lds));
            r.m0b = __builtin_amdgcn_readfirstlane(
                (int32_t)(has2 || qb ? kbuf_lds + (uint32_t)(par * kWideBufBytes +
                                                             kRowsPerWave * wave * kRowBytes)
                                     : dummy_lds));
            r.sa = has1 || qa ? kRowBytes : 0;
            r.sb = has2 || qb ? kRowBytes : 0;
            return r;
        };
        // the state of a tile with two more tiles after it: both streams
        // gather key rows
        auto ctl_steady = [&](auto P) -> Ctl {
            constexpr int par = decltype(P)::value;
            Ctl r;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                r.da[i] = __builtin_amdgcn_readfirstlane(kdesc[i]);
                r.db[i] = r.da[i];
            }
            r.m0a = __builtin_amdgcn_readfirstlane((int32_t)(
                kbuf_lds + (uint32_t)((1 - par) * kWideBufBytes +
                                      (kRowsPerWave * wave + 7) * kRowBytes)));
            r.m0b = __builtin_amdgcn_readfirstlane((int32_t)(
                kbuf_lds + (uint32_t)(par * kWideBufBytes + kRowsPerWave * wave * kRowBytes)));
            r.sa = kRowBytes;
            r.sb = kRowBytes;
            return r;
        };
        // the previous tile's unfinished epilogue (see wide_tile)
        float pt = 0.0f, pex = 0.0f, psum = 0.0f;
        // Tile `tile` (parity P): `cc` holds its stream state, `oa` the gather
        // offsets of tile+1 (formed by tile-1); tile+2's offsets are formed in
        // step 18 into `ob`. Tile-2's values are stored in steps 25..30: its
        // index is read in step 14 and its destination formed in step 21, its
        // four partial sums (finished in its step 0, written in step 1) read
        // after the barrier.
        auto body = [&](auto P, auto STEADY, int tile, const Ctl& cc, int32_t oa, int32_t& ob,
                        const f32x16_t& prev0, const f32x16_t& prev1, f32x16_t& acc0,
                        f32x16_t& acc1) {
            constexpr int par = decltype(P)::value;
            constexpr bool steady = decltype(STEADY)::value != 0;
            const uint4* cur = kbuf[par] + (32 * kh + col) * kPitch + half;
            const uint4* nxt = kbuf[1 - par] + (32 * kh + col) * kPitch + half;
            int32_t kb = 0, jv = -1, sdst = 0;
            float parts[4], tot = 0.0f;
            wide_tile<BF16>(
                cur, nxt, ring, qa0, qa1, prev0, prev1, l2, a.c_scale, pt, pex, psum,
                i32x4_t{cc.da[0], cc.da[1], cc.da[2], cc.da[3]},
                i32x4_t{cc.db[0], cc.db[1], cc.db[2], cc.db[3]}, cc.m0a, cc.sa, oa, cc.m0b, cc.sb, ob, voff16,
                [&](int s) {  // first gap
                    if (s == 1) {
                        // tile-2's partial sums, finished in step 0 (tiles 0
                        // and 1: an unused slot)
                        red[par][2 * hg + half][32 * kh + col] = psum;
                    } else if (s == kBarStep + 1) {
                        // tile-2's partial sums of every wave, written in step
                        // 1 and visible after the barrier
                        parts[0] = red[par][0][slot];
                        parts[1] = red[par][1][slot];
                    } else if (s == kBarStep + 2) {
                        parts[2] = red[par][2][slot];
                        parts[3] = red[par][3][slot];
                    } else if (s == kBarStep + 3) {
                        tot = parts[0] + parts[1];
                        pin(tot);
                    } else if (s == kBarStep + 4) {
                        tot += parts[2];
                        pin(tot);
                    } else if (s == kBarStep + 5) {
                        tot += parts[3];
                        pin(tot);
                    } else if (s == kBarStep + 6) {
                        const float v = tot * a.inv_g;
                        if (ROWBUF) {
                            // (a column below W <= kRowCap, or this lane's sink)
                            rowbuf[sdst] = v;
                        } else {
                            // (the builtin's data operand is an integer: pass
                            // the bits; an offset past the row is dropped)
                            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v),
                                                                  orsrc, sdst, 0, 0);
                        }
                    }
                },
                [&](int s) {  // second gap (each LDS read is used steps later)
                    // (the tile number is pinned in the step, so that no part
                    // of the step's work is hoisted into an earlier step)
                    int32_t tl = tile;
                    if (s == 12 || s == 14 || s == 18 || s == 21) pin_s(tl);
                    if (s == 12) {
                        kb = DENSE ? (tl + 2) * kWideKeys + my_slot
                                   : irow[((tl + 2) & 31) * kWideKeys + my_slot];
                    } else if (s == 14) {
                        jv = DENSE ? (tl - 2) * kWideKeys + slot
                                   : irow[((tl - 2) & 31) * kWideKeys + slot];
                    } else if (s == 18) {
                        // (a steady tile has tile+2; otherwise stream B takes
                        // the next row's Q, if there is one)
                        const bool has2 = steady || tl + 2 < ntiles;
                        ob = has2 ? row_off(ric, tl + 2, kb) : (more ? q_off(par) : 0);
                        pin_v(ob);  // (computed here, not where it is used)
                    } else if (s == 21) {
                        // entry e = (tile-2)*64 + slot of lanes < 16: its
                        // column (its key's col0 + j, or K-wide e) if used
                        const int e = (tl - 2) * kWideKeys + slot;
                        const bool used = (lane < kRowsPerWave) & (tl >= 2) & (e < ric.n) &
                                          ((uint32_t)jv < (uint32_t)ric.vis);
                        const int32_t cc2 = a.kwide ? e : (int32_t)(ric.col0 + jv);
                        sdst = ROWBUF ? (used ? cc2 : kRowCap + lane)
                                      : (used ? (int32_t)((uint32_t)cc2 * 4u) : 0x7ffffff0);
                        pin_v(sdst);
                    }
                },
                acc0, acc1);
        };
        // Pairs of tiles with two more after them run the steady body (stream
        // state fixed per parity); the last two or three tiles of a row form
        // their state at each tile boundary. Even tiles fill xa from xb, odd
        // tiles xb from xa. (Both loops are unrolled by two, so that each
        // register set keeps its registers across the tiles of a loop.)
        const Ctl cs0 = ctl_steady(Par<0>{}), cs1 = ctl_steady(Par<1>{});
        int32_t offb = 0;
        int tile = 0;
        for (; tile + 3 < ntiles; tile += 2) {
            body(Par<0>{}, Par<1>{}, tile, cs0, offa, offb, xb0, xb1, xa0, xa1);
            body(Par<1>{}, Par<1>{}, tile + 1, cs1, offb, offa, xa0, xa1, xb0, xb1);
        }
        // the next row's index list into L2 (one dword per 128-byte line, 8 KB
        // in one load, into the dummy row), two or three tiles before the row
        // end loads it into LDS; the key rows keep their place in L2
        if (!DENSE && more && wave == 0)
            dma_dword(raw_desc(a.idx + rln * a.K, (uint32_t)a.K * 4u), dummy_lds, 0, voff16 << 3);
        for (; tile < ntiles; tile += 2) {
            const Ctl c0 = ctl_of(Par<0>{}, tile);
            body(Par<0>{}, Par<0>{}, tile, c0, offa, offb, xb0, xb1, xa0, xa1);
            if (tile + 1 >= ntiles) break;
            const Ctl c1 = ctl_of(Par<1>{}, tile + 1);
            body(Par<1>{}, Par<0>{}, tile + 1, c1, offb, offa, xa0, xa1, xb0, xb1);
        }
        // Every wave has passed the last tile's barrier, so no operand read of
        // the last tile's buffer is pending: the rows of the next row's Q that
        // the last tiles did not load (see the streams in the tile loop) and
        // its lse are loaded now, before the row is finished and written out.
        if (more) {
            if (ntiles >= 2) {
                stage_q_rows(rln, (ntiles - 1) & 1, 7, kRowsPerWave);
            } else {
                stage_q_rows(rln, 0, ntiles == 1 ? 7 : 0, kRowsPerWave);
                stage_q_rows(rln, 1, 0, kRowsPerWave);
            }
            stage_lse(rln);
        }
        // tile ntiles-2's epilogue still lacks its last two elements
        if (ntiles >= 2) {
            psum += pex;
            psum += __builtin_amdgcn_exp2f(pt);
            red[ntiles & 1][2 * hg + half][32 * kh + col] = psum;
        }
        const f32x16_t& prev0 = (ntiles & 1) ? xa0 : xb0;
        const f32x16_t& prev1 = (ntiles & 1) ? xa1 : xb1;
        // (the last tile's sums go to their own buffer: other waves may still
        // be reading red[(ntiles - 1) & 1] in the last tile)
        if (ntiles > 0)
            redl[2 * hg + half][32 * kh + col] =
                head_sum(prev0, l2, a.c_scale) + head_sum(prev1, l2 + 16, a.c_scale);

        // all MFMAs done, every operand read done and every gather of this
        // row landed (only loads to the dummy row may be in flight): K
        // buffers are free; partial sums visible
        lds_barrier();
        auto finish = [&](const float (*pr)[kWideKeys], int tile) {
            const float tot = pr[0][slot] + pr[1][slot] + pr[2][slot] + pr[3][slot];
            store_value(tile, tot,
                        DENSE ? tile * kWideKeys + slot : irow[(tile & 31) * kWideKeys + slot]);
        };
        if (ntiles >= 2) finish(red[ntiles & 1], ntiles - 2);
        if (ntiles >= 1) finish(redl, ntiles - 1);
        if (ROWBUF) {
            // every value is in the row buffer and every read of the index
            // list is done: write the row out (16-byte stores where aligned)
            lds_barrier();
            write_row(a.out + rc * a.W, rowbuf, a.W, tid, NT);
        }

        // the next row: index list and zeroed output; once its Q and lse have
        // landed every wave reads its heads back, then buffer 0 takes the next
        // row's first tile
        prepare_next();
        if (more) {
            barrier_after_vmcnt(0);
            read_q_lse();
            lds_barrier();
            offa = start_row(rin, ROWBUF ? 0 : ib ^ 1);
        }

        // the next row becomes current
        rc = rn;
        ric = rin;
        if (!ROWBUF) ib ^= 1;
    }
    // loads into LDS (the last tile's dummy loads) must land before the
    // workgroup's LDS is released
    waitcnt_vm_lgkm0<0>();
}

// ---------------------------------------------------------------------------
// Pipelined kernel for rows of up to 64 heads (NB = 1, 2 or 4 blocks of 16
// heads), any number of indices per row, or the dense case.
//
// v_mfma_f32_16x16x32 with Q as A (16 heads x 32 of D) and K as B (32 of D
// x 16 keys): lane l holds head 16b + (l & 15) of Q and key (l & 15) of K,
// elements 8 (l >> 4) .. +8 of the k-step, and receives the scores of key
// (l & 15) for heads 16b + 4 (l >> 4) + i, i < 4. Wave w takes keys
// 16w .. 16w + 15 of each 64-key tile with all the row's heads, so every
// B operand feeds NB MFMAs, and the sum over heads of a key ends in the
// lanes n, n + 16, n + 32, n + 48: two permlane swaps add it up in registers
// (quad_sum), and the wave stores its 16 values itself.
//
// A wave reads only the key rows it gathers itself, so the tile loop has no
// workgroup barrier: each wave waits for its own loads. Its rows 16w .. +15
// of the two LDS buffers carry one stream of elements, [Q(r0), tiles of r0,
// Q(r1), tiles of r1, ...] over the workgroup's rows that have a used entry:
// element k sits in buffer k & 1. A tile's B operands are read into
// registers during the tile before it, so its buffer is free early: once
// element k has been read (a tile's operands, or a row start's Q), element
// k + 2 is loaded into the same place, and has about two tiles to land. Q
// (up to 64 heads, one buffer) is loaded by the waves together, so a row
// start has two workgroup barriers: Q landed, Q read.
//
// The tile loop is laid out against the issue costs measured for one wave
// per SIMD: a v_mfma_f32_16x16x32 issues every 16.5 cycles and leaves room
// for about two VALU instructions; each further VALU instruction costs 4-5
// cycles; LDS reads and scalar instructions are nearly free; a uniform
// branch costs 17-28 cycles. So the steps hold no branch (tiles whose loads
// are key rows of the row, the steady tiles, are a variant of their own;
// the last tiles plan their loads without branches), and each step's other
// instructions are spread over the gaps after its MFMAs.
//
// Tile t (16 k-steps of NB MFMAs on operands read during tile t-1):
//   step 0        wait for every load but the previous tile's (the rows of
//                 tile t+1 are among them); steps 0..3 read tile t+1's
//                 operands
//   steps 0..9    the previous tile's epilogue (fma, exp2, sum over the lane's
//                 heads), two or one elements per step, pipelined over steps
//   steps 5..6    the row offsets of this tile's load (element k + 2, k =
//                 tile t+1; its indices were loaded two loads earlier)
//   steps 7..14   those offsets into scalar registers, two per step
//   step 7        wait for the operand reads: tile t+1's buffer is free
//   steps 8..15   the indices of tile t+1's stores and of the load two
//                 loads on, then the 16 row loads, two per step
//   steps 10..13  the head sum across lanes, the scale by 1/G, and the
//                 store of tile t-1's values
constexpr int kNarKeys = 64;  // keys per tile, 16 per wave

template <bool BF16>
__device__ __forceinline__ f32x4_t mfma_16x16x32(uint4 a, uint4 b, f32x4_t c) {
    if constexpr (BF16) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                        __builtin_bit_cast(bf16x8_t, b),
                                                        c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                       __builtin_bit_cast(f16x8_t, b),
                                                       c, 0, 0, 0);
    }
}

// Sum of x over the lanes n, n + 16, n + 32, n + 48 (n = lane & 15), the same
// bits in all four: (x_n + x_{n+32}) + (x_{n+16} + x_{n+48}). Each swap
// leaves a lane's value and its partner's in the pair (lower half first).
__device__ __forceinline__ float quad_sum(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const float s = __builtin_bit_cast(float, (uint32_t)a[0]) +
                    __builtin_bit_cast(float, (uint32_t)a[1]);
    const uint32_t v = __builtin_bit_cast(uint32_t, s);
    const auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return __builtin_bit_cast(float, (uint32_t)b[0]) + __builtin_bit_cast(float, (uint32_t)b[1]);
}

// A row's decode in 32 bits (rows, key rows and columns number fewer than
// 2^31, checked on the host): fewer scalar registers than RowInfo.
struct NarRow {
    int32_t kbase;  // first k row of the row's batch / sequence
    int32_t col0;   // first output column of the row's batch / sequence
    int32_t vis;    // keys [0, vis) are visible and in range
    int32_t n;      // entries of the index row to look at
};
__device__ __forceinline__ NarRow nar_row(const RowInfo& r) {
    return NarRow{(int32_t)r.kbase, (int32_t)r.col0, r.vis, r.n};
}

// One element of a wave's load stream: nothing, the key rows of a tile, or a
// row's Q (and its lse).
enum { kElemNone = 0, kElemKeys = 1, kElemQ = 2 };
struct NarElem {
    int32_t kind;  // kElemNone, kElemKeys (tile `tile` of `row`), kElemQ (of `row`)
    int32_t tile;
    int32_t row;
    NarRow ri;
};

// The element d after element j of row r0 (j = 0: the row's Q, j = i + 1:
// its tile i) in the stream over rows r0, r1, r2 (T tiles each; R: none).
// Without branches, and everything by value (a choice between captured
// references would keep the row state in memory).
__device__ __forceinline__ NarElem nar_elem_plus(int j, int d, int32_t R, int32_t r0, int T0,
                                                 NarRow i0, int32_t r1, int T1, NarRow i1,
                                                 int32_t r2, int T2, NarRow i2) {
    const int x0 = j + d;          // offset from r0's Q
    const int x1 = x0 - (T0 + 1);  // from r1's Q
    const int x2 = x1 - (T1 + 1);  // from r2's Q
    const bool in0 = (r0 < R) & (x0 <= T0);
    const bool in1 = !in0 & (r1 < R) & (x1 <= T1);
    const bool in2 = !in0 & !in1 & (r2 < R) & (x2 <= T2);
    const int x = in0 ? x0 : (in1 ? x1 : x2);
    NarElem e;
    e.kind = (in0 | in1 | in2) ? (x == 0 ? kElemQ : kElemKeys) : kElemNone;
    e.tile = x - 1;
    e.row = in0 ? r0 : (in1 ? r1 : (in2 ? r2 : R));
    e.ri.kbase = in0 ? i0.kbase : (in1 ? i1.kbase : i2.kbase);
    e.ri.col0 = in0 ? i0.col0 : (in1 ? i1.col0 : i2.col0);
    e.ri.vis = in0 ? i0.vis : (in1 ? i1.vis : i2.vis);
    e.ri.n = in0 ? i0.n : (in1 ? i1.n : i2.n);
    return e;
}

template <int NB, bool BF16, bool TND, bool DENSE>
__global__ __launch_bounds__(256, 1) void smla_narrow_kernel(KernelArgs a) {
    constexpr int NT = 256;
    constexpr int NE = NB * 4;             // scores per lane and tile
    constexpr int EPS = NE >= 16 ? 2 : 1;  // epilogue elements per step
    constexpr int NG = NE / EPS;           // epilogue groups: fma in step g, exp g+1, sum g+2
    constexpr int kSteps = kChunks / 4;    // 16 k-steps of 32 along D
    static_assert(NG + 2 <= 10, "the epilogue must end by step 9");
    // Loads per tile (index loads: one per wave; the dense case has none):
    // two index loads, 16 rows, one store, one lse load. A row start issues
    // as many after tile 1's rows: that load's lse, the next element's index
    // load, rows and lse, the index-list prefetch.
    constexpr int kIdx = DENSE ? 0 : 1;
    constexpr int kTileLoads = 2 * kIdx + 16 + 1 + 1;
    constexpr int kRowStartTail = 1 + kIdx + 16 + 1 + kIdx;
    static_assert(kRowStartTail == kTileLoads, "one wait count for every tile");
    constexpr int kJsSlot0 = 4;  // index slots 4..7: the stores' indices, by tile
    __shared__ uint4 kbuf[2][kNarKeys * kPitch];
    // per wave: the indices of the next loads' tiles (ring of 4, by load
    // number) and of the tiles whose values are stored next (ring of 4, by
    // tile)
    __shared__ int32_t ixbuf[4][8][64];
    __shared__ float lsebuf[64];
    __shared__ uint4 dummy[64];  // loads with nothing to fetch

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15;
    const int gq = lane >> 4;
    const int my_slot = 16 * wave + n;  // this lane's key slot in a tile
    const uint4* __restrict__ q4 = static_cast<const uint4*>(a.q);
    const char* __restrict__ kbytes = static_cast<const char*>(a.k);
    const uint32_t kbuf_lds = lds_addr(kbuf);
    const uint32_t ix_lds = lds_addr(&ixbuf[wave][0][0]);
    const uint32_t lse_lds = lds_addr(lsebuf);
    const uint32_t dummy_lds = lds_addr(dummy);
    const uint32_t voff16 = (uint32_t)lane << 4;
    const uint32_t voff4 = (uint32_t)lane << 2;
    const int64_t obytes = a.W * 4;
    const int orange = obytes < 0x7ffffff0ll ? (int)obytes : 0x7ffffff0;
    const int32_t R = (int32_t)a.R;

    // ---- the workgroup's rows that have a used entry: current, next, the
    // one after. Every row passed over (and every row found) is zero-filled
    // when it is found, two rows before its values are stored.
    int64_t it_next = 0;
    auto next_row = [&](NarRow& ri, int& T) __attribute__((always_inline)) -> int32_t {
        for (;;) {
            if (it_next * a.num_wg >= a.R) return R;
            const int64_t r = row_of(a, it_next, blockIdx.x);
            ++it_next;
            if (r >= a.R) continue;
            zero_span(a.out + r * a.W, 0, a.W, tid, NT);
            ri = nar_row(decode_row<TND>(a, r));
            T = __builtin_amdgcn_readfirstlane((ri.n + kNarKeys - 1) / kNarKeys);
            if (T > 0) return (int32_t)r;
        }
    };
    NarRow ric, rin, rinn;
    int Tc = 0, Tn = 0, Tnn = 0;
    int32_t rc = next_row(ric, Tc);
    int32_t rn = rc < R ? next_row(rin, Tn) : R;
    int32_t rnn = rn < R ? next_row(rinn, Tnn) : R;
    if (rc >= R) {
        waitcnt_vm_lgkm0<0>();
        return;
    }

    auto elem_plus = [&](int j, int d) __attribute__((always_inline)) -> NarElem {
        return nar_elem_plus(j, d, R, rc, Tc, ric, rn, Tn, rin, rnn, Tnn, rinn);
    };
    auto keys_elem = [&](int tile) __attribute__((always_inline)) -> NarElem {
        NarElem e;
        e.kind = kElemKeys;
        e.tile = tile;
        e.row = rc;
        e.ri = ric;
        return e;
    };
    // The indices of slot my_slot of tile `tile` of row `row` into index slot
    // `slot` of this wave (lane l gets the index of slot 16w + (l & 15)); a
    // load that is not `live` reads zeros. Index loads go to LDS, so the
    // compiler tracks none of them: the waits that cover them are explicit.
    auto idx_dma = [&](int slot, int32_t row, int tile, bool live) __attribute__((always_inline)) {
        if constexpr (!DENSE) {
            const i32x4_t d = uniform_desc(raw_desc(a.idx + (int64_t)(live ? row : 0) * a.K,
                                                    live ? (uint32_t)a.K * 4u : 0u));
            dma_dword(d, (uint32_t)__builtin_amdgcn_readfirstlane(
                             (int32_t)(ix_lds + (uint32_t)slot * 256u)),
                      0, (uint32_t)(tile * kNarKeys + my_slot) * 4u);
        }
    };
    auto idx_read = [&](int slot) __attribute__((always_inline)) -> int32_t {
        return DENSE ? 0 : ixbuf[wave][slot][lane];
    };
    // Row `row`'s index list into L2, one dword per 128-byte line into the
    // dummy row (wave w takes lines 64w .. 64w + 63: lists of up to 8192
    // entries), so that the per-tile index loads hit L2. One load per wave.
    auto idx_prefetch = [&](int32_t row) __attribute__((always_inline)) {
        if constexpr (!DENSE) {
            const bool live = row < R;
            const i32x4_t d = uniform_desc(raw_desc(a.idx + (int64_t)(live ? row : 0) * a.K,
                                                    live ? (uint32_t)a.K * 4u : 0u));
            dma_dword(d, (uint32_t)__builtin_amdgcn_readfirstlane((int32_t)dummy_lds),
                      64 * 128 * wave, voff4 * 32u);
        }
    };
    auto used_of = [&](NarRow ri, int tile, int32_t j) __attribute__((always_inline)) -> bool {
        const int e = tile * kNarKeys + my_slot;
        return (e < ri.n) & ((uint32_t)(DENSE ? e : j) < (uint32_t)ri.vis);
    };
    // byte offset of the row to load into slot my_slot for element e (key
    // rows: the key's row, or row 0 for an unused entry; Q: head 16w + n);
    // selected with masks, so that no path is a branch
    auto elem_off = [&](NarElem e, int32_t jg) __attribute__((always_inline)) -> int32_t {
        const int32_t j = DENSE ? e.tile * kNarKeys + my_slot : jg;
        const int32_t koff = (j << 10) & -(int32_t)used_of(e.ri, e.tile, j);
        const int32_t qoff = (16 * wave + n) * 1024;
        return (koff & -(int32_t)(e.kind == kElemKeys)) | (qoff & -(int32_t)(e.kind == kElemQ));
    };
    struct NarCtl {
        i32x4_t d;
        int32_t m0, step, lm0;
    };
    // buffer descriptor of the key rows of a row (from its first k row)
    auto k_desc32 = [&](int32_t kbase) __attribute__((always_inline)) -> i32x4_t {
        const int64_t bytes = (a.rows_k - kbase) * 1024;
        return raw_desc(kbytes + (int64_t)kbase * 1024,
                        bytes > 0xffffffffll ? 0xffffffffu : (uint32_t)(bytes < 0 ? 0 : bytes));
    };
    // buffer descriptor, first LDS row and row step of element e loaded into
    // buffer `buf` (a wave past the row's head blocks loads no Q rows; loads
    // with nothing to fetch go to the dummy row), and where the lse goes
    auto elem_ctl = [&](NarElem e, int buf) __attribute__((always_inline)) -> NarCtl {
        const bool isq = e.kind == kElemQ;
        const i32x4_t dk = k_desc32(e.kind == kElemKeys ? e.ri.kbase : ric.kbase);
        const i32x4_t dq = raw_desc(q4 + (int64_t)e.row * a.G * kChunks, (uint32_t)a.G * 1024u);
        const bool live = e.kind == kElemKeys || (isq && wave < NB);
        NarCtl c;
        c.d = uniform_desc(isq ? dq : dk);
        c.m0 = __builtin_amdgcn_readfirstlane(
            (int32_t)(live ? kbuf_lds + (uint32_t)(buf * kNarKeys * kRowBytes +
                                                   16 * wave * kRowBytes)
                           : dummy_lds));
        c.step = __builtin_amdgcn_readfirstlane(live ? kRowBytes : 0);
        c.lm0 = __builtin_amdgcn_readfirstlane((int32_t)(isq && wave == 0 ? lse_lds : dummy_lds));
        return c;
    };
    // the lse of a Q element (wave 0; everything else loads into the dummy row)
    auto lse_dma = [&](NarElem e, const NarCtl& c) __attribute__((always_inline)) {
        const bool isq = e.kind == kElemQ;
        dma_dword(uniform_desc(raw_desc(a.lse + (int64_t)(isq ? e.row : 0) * a.G,
                                        isq ? (uint32_t)a.G * 4u : 0u)),
                  (uint32_t)c.lm0, 0, voff4);
    };
    // element e into buffer `buf` at once (row starts); `slot` holds its
    // indices
    auto issue_now = [&](NarElem e, int slot, int buf) __attribute__((always_inline)) {
        const NarCtl c = elem_ctl(e, buf);
        const int32_t ov = elem_off(e, idx_read(slot));
        int32_t so[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            so[i] = __builtin_amdgcn_readlane(ov, i);
            pin_s(so[i]);
        }
        dma_row_first(c.d, (uint32_t)c.m0, so[0], voff16, c.step);
#pragma unroll
        for (int i = 1; i < 16; ++i) dma_row_next(c.d, so[i], voff16, c.step);
        lse_dma(e, c);
    };

    // ---- start: Q of the first row into buffer 0, its tile 0 into buffer 1,
    // the indices of the row start's two loads (load numbers 0 and 1) into
    // their slots
    int qb = 0;        // buffer holding the current row's Q
    int ip = 0;        // load number of the current row's first load
    NarElem pe0, pe1;  // the elements of loads ip and ip + 1
    {
        NarElem eq;
        eq.kind = kElemQ;
        eq.tile = 0;
        eq.row = rc;
        eq.ri = ric;
        const NarElem e0 = elem_plus(0, 1);
        pe0 = elem_plus(0, 2);
        pe1 = elem_plus(0, 3);
        idx_prefetch(rn);
        idx_dma(kJsSlot0 + 3, e0.row, e0.tile, e0.kind == kElemKeys);
        idx_dma(0, pe0.row, pe0.tile, pe0.kind == kElemKeys);
        idx_dma(1, pe1.row, pe1.tile, pe1.kind == kElemKeys);
        issue_now(eq, kJsSlot0 + 3, 0);
        waitcnt_vm_lgkm0<0>();
        issue_now(e0, kJsSlot0 + 3, 1);
    }

    uint4 qa[NB][kSteps];
    float l2[NE];
    uint4 opa[kSteps], opb[kSteps];  // B operands of a tile, read a tile ahead
    f32x4_t xa[NB], xb[NB];

    bool find_rnn = false;
    for (;;) {
        // ---- row start. rnn (found now: its rows are zero-filled before the
        // wait below covers the stores), then Q, lse and tile 0 of row rc
        // have landed (every wave's loads: wait, then barrier); read them,
        // then free both buffers
        if (find_rnn) rnn = rn < R ? next_row(rinn, Tnn) : R;
        find_rnn = false;
        waitcnt_vm_lgkm0<0>();
        asm volatile("s_barrier" ::: "memory");
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int s = 0; s < kSteps; ++s)
                qa[b][s] = kbuf[qb][(16 * b + n) * kPitch + 4 * s + gq];
#pragma unroll
        for (int e = 0; e < NE; ++e) {
            const int h = 16 * (e >> 2) + 4 * gq + (e & 3);
            const float v = lsebuf[h];
            l2[e] = h < a.G ? v * kLog2e : __builtin_inff();
        }
#pragma unroll
        for (int s = 0; s < kSteps; ++s) opa[s] = kbuf[qb ^ 1][my_slot * kPitch + 4 * s + gq];
        waitcnt_vm_lgkm0<0>();
        asm volatile("s_barrier" ::: "memory");
        // load ip (element k + 2, k = this Q) into buffer qb, load ip + 1
        // (element k + 3) into buffer qb ^ 1; each first loads the indices of
        // the load two after it (and load ip the indices of tile 0's stores).
        // Then the index list of the row after next into L2.
        {
            const NarElem e4 = elem_plus(0, 4), e5 = elem_plus(0, 5);
            idx_dma((ip + 2) & 3, e4.row, e4.tile, e4.kind == kElemKeys);
            idx_dma(kJsSlot0, rc, 0, true);
            issue_now(pe0, ip & 3, qb);
            idx_dma((ip + 3) & 3, e5.row, e5.tile, e5.kind == kElemKeys);
            issue_now(pe1, (ip + 1) & 3, qb ^ 1);
            idx_prefetch(rnn);
            pe0 = e4;
            pe1 = e5;
            ip += 2;
        }
        const NarRow ri = ric;
        const int ntiles = Tc;
        const int32_t row = rc;
        const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
            a.out + (int64_t)row * a.W, (short)0, orange, 0x00020000);
        const i32x4_t kdesc = uniform_desc(k_desc32(ri.kbase));  // this row's key rows
        // byte offset of the store of tile `tile`'s value (past the row when
        // the lane has nothing to store)
        auto store_off = [&](int tile, int32_t j) __attribute__((always_inline)) -> int32_t {
            const int e = tile * kNarKeys + my_slot;
            const int32_t jj = DENSE ? e : j;
            const bool st = (gq == 0) & (tile >= 0) & used_of(ri, tile, jj);
            const int32_t c = a.kwide ? e : ri.col0 + jj;
            return st ? (int32_t)((uint32_t)c * 4u) : 0x7ffffff0;
        };

        // One tile: the MFMAs of tile t on `op` (read during the previous
        // tile), the epilogue of tile t-1 (prev) and its stores, the operands
        // of tile t+1 into `nop` (its buffer is free after step 7) and this
        // tile's load (element k + 2, k = tile t+1) into that buffer. Every
        // step's other instructions are spread over the gaps after its MFMAs
        // (sub-slot b follows the MFMA of head block b; with fewer than four
        // blocks the remaining sub-slots follow the last MFMA).
        //   MORE   (compile time) tile t+1 exists: read it, load for it;
        //   STEADY (compile time) this load and the load two on are key rows
        //          of this row (t + 5 < ntiles): no element planning.
        auto tile_body = [&](auto MORE, auto STEADY, int t, const uint4(&op)[kSteps],
                             uint4(&nop)[kSteps], const f32x4_t(&prev)[NB],
                             f32x4_t(&acc)[NB]) __attribute__((always_inline)) {
            constexpr bool more = decltype(MORE)::value != 0;
            constexpr bool steady = decltype(STEADY)::value != 0;
            const int nb = (qb + t) & 1;  // tile t+1's buffer
            const uint4* nsrc = &kbuf[nb][my_slot * kPitch + gq];
            // this load, and the load two on (its indices are loaded now)
            const NarElem E = steady ? keys_elem(t + 3) : pe0;
            const NarElem Enew = steady ? keys_elem(t + 5) : elem_plus(t + 2, 4);
            NarCtl C;
            if constexpr (steady) {
                C.d = kdesc;
                C.m0 = __builtin_amdgcn_readfirstlane((int32_t)(
                    kbuf_lds + (uint32_t)(nb * kNarKeys * kRowBytes + 16 * wave * kRowBytes)));
                C.step = kRowBytes;
                C.lm0 = __builtin_amdgcn_readfirstlane((int32_t)dummy_lds);
            } else {
                C = elem_ctl(E, nb);
            }
            int32_t jg = 0, ov = 0, js = 0, so[4];
            float tt[EPS], ee[EPS], sum = 0.0f, tot = 0.0f, val = 0.0f;
            auto work = [&](int s, int b) __attribute__((always_inline)) {
                if (s == 0 && b == 0) {
                    // the loads of tile t-1 (or, at tile 0, as many of the
                    // row start's) may be in flight; everything older (tile
                    // t+1's rows among them) has landed
                    waitcnt_vm_lgkm0<kTileLoads>();
                    if constexpr (more) jg = idx_read(ip & 3);
                    js = idx_read(kJsSlot0 + ((t - 1) & 3));
                }
                // operands of tile t+1: four reads per step in steps 0..3
                if (s < 4 && more) {
                    if constexpr (NB == 4) {
                        nop[4 * s + b] = nsrc[4 * (4 * s + b)];
                    } else if (b == 3) {
#pragma unroll
                        for (int k = 0; k < 4; ++k) nop[4 * s + k] = nsrc[4 * (4 * s + k)];
                    }
                }
                // epilogue of tile t-1: sum (group s-2), exp2 (s-1), fma (s)
                if ((NB == 4 && b <= 1) || (NB < 4 && b == 3)) {
                    constexpr int kPer = NB == 4 ? 1 : EPS;
#pragma unroll
                    for (int k0 = 0; k0 < kPer; ++k0) {
                        const int k = NB == 4 ? b : k0;
                        if (s >= 2 && s - 2 < NG) {
                            sum += ee[k];
                            pin(sum);
                        }
                        if (s >= 1 && s - 1 < NG) {
                            ee[k] = __builtin_amdgcn_exp2f(tt[k]);
                            pin(ee[k]);
                        }
                    }
                }
                if ((NB == 4 && b >= 2) || (NB < 4 && b == 3)) {
                    constexpr int kPer = NB == 4 ? 1 : EPS;
#pragma unroll
                    for (int k0 = 0; k0 < kPer; ++k0) {
                        const int k = NB == 4 ? b - 2 : k0;
                        if (s < NG) {
                            const int e = s * EPS + k;
                            tt[k] = __builtin_fmaf(prev[e >> 2][e & 3], a.c_scale, -l2[e]);
                            pin(tt[k]);
                        }
                    }
                }
                if (b == (NB == 4 ? 2 : 3)) {
                    if (s == 10) {
                        tot = quad_sum(sum);
                        pin(tot);
                    } else if (s == 11) {
                        val = tot * a.inv_g;
                        pin(val);
                    }
                }
                // the indices of this tile's load and of tile t-1's stores
                // (landed at the wait of step 0) are read in step 0, before
                // the operand reads, and used steps later: an index read used
                // right after it is issued waits for it (and every LDS read
                // in flight) there (not pinned, for the same reason)
                // row offsets of this tile's load in step 6; two scalar
                // offsets per step from step 7 on, one step before their
                // loads
                if (more && b == (NB == 4 ? 1 : 3)) {
                    if (s == 6) {
                        ov = elem_off(E, jg);
                        pin_v(ov);
                    }
                }
                if (more && b == (NB == 4 ? 0 : 3) && s >= 7 && s <= 14) {
#pragma unroll
                    for (int k = 0; k < 2; ++k) {
                        so[((s - 7) & 1) * 2 + k] = __builtin_amdgcn_readlane(ov, 2 * (s - 7) + k);
                        pin_s(so[((s - 7) & 1) * 2 + k]);
                    }
                }
                if (more && b == 3) {
                    if (s == 7) {
                        // the operand reads of tile t+1 (and the index read)
                        // are done: its buffer is free
                        waitcnt_vm_lgkm0<63>();
                    } else if (s == 8) {
                        // this tile's loads, in a fixed order: indices of
                        // tile t+1's stores and of the load two on, the 16
                        // rows (two per step, the store of tile t-1's values
                        // in step 13), the lse of a Q element
                        idx_dma(kJsSlot0 + ((t + 1) & 3), row, t + 1, true);
                        idx_dma((ip + 2) & 3, Enew.row, Enew.tile, Enew.kind == kElemKeys);
                        dma_row_first(C.d, (uint32_t)C.m0, so[0], voff16, C.step);
                        dma_row_next(C.d, so[1], voff16, C.step);
                    } else if (s > 8) {
                        const int g = ((s - 8) & 1) * 2;
                        dma_row_next(C.d, so[g], voff16, C.step);
                        dma_row_next(C.d, so[g + 1], voff16, C.step);
                    }
                }
                if (b == 3 && s == 13)
                    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, val),
                                                          orsrc, store_off(t - 1, js), 0, 0);
                if (more && b == 3 && s == 15) lse_dma(E, C);
            };
#pragma unroll
            for (int s = 0; s < kSteps; ++s) {
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    __builtin_amdgcn_sched_barrier(0);
                    acc[b] = mfma_16x16x32<BF16>(qa[b][s], op[s],
                                                 s == 0 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : acc[b]);
                    asm volatile("" ::"v"(acc[b]));
                    if (b < NB - 1) work(s, b);
                }
#pragma unroll
                for (int b = NB - 1; b < 4; ++b) work(s, b);
            }
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (more) {
                if constexpr (!steady) {
                    pe0 = pe1;
                    pe1 = Enew;
                }
                ++ip;
            }
        };

        // Steady pairs while both loads of each tile are key rows of the row;
        // then the planned loads take over (pe0, pe1: the next two loads)
        int t = 0;
        for (; t + 6 < ntiles; t += 2) {
            tile_body(Par<1>{}, Par<1>{}, t, opa, opb, xb, xa);
            tile_body(Par<1>{}, Par<1>{}, t + 1, opb, opa, xa, xb);
        }
        if (t > 0) {
            // (tile t reads tile t+1, element t + 2 of the row: its load is
            // two elements on)
            pe0 = elem_plus(t + 2, 2);
            pe1 = elem_plus(t + 2, 3);
        }
        for (; t + 2 < ntiles; t += 2) {
            tile_body(Par<1>{}, Par<0>{}, t, opa, opb, xb, xa);
            tile_body(Par<1>{}, Par<0>{}, t + 1, opb, opa, xa, xb);
        }
        if (t + 1 < ntiles) {
            tile_body(Par<1>{}, Par<0>{}, t, opa, opb, xb, xa);
            tile_body(Par<0>{}, Par<0>{}, t + 1, opb, opa, xa, xb);
        } else {
            tile_body(Par<0>{}, Par<0>{}, t, opa, opb, xb, xa);
        }
        // the last tile's epilogue, then its stores once its indices landed
        // (the register set is picked by a branch: a reference chosen at run
        // time would put both sets in memory)
        auto last_value = [&](const f32x4_t(&x)[NB]) __attribute__((always_inline)) -> float {
            float sum = 0.0f;
#pragma unroll
            for (int e = 0; e < NE; ++e)
                sum += __builtin_amdgcn_exp2f(__builtin_fmaf(x[e >> 2][e & 3], a.c_scale, -l2[e]));
            return quad_sum(sum) * a.inv_g;
        };
        const float v = (ntiles & 1) ? last_value(xa) : last_value(xb);
        waitcnt_vm_lgkm0<0>();
        const int32_t js = idx_read(kJsSlot0 + ((ntiles - 1) & 3));
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), orsrc,
                                              store_off(ntiles - 1, js), 0, 0);
        if (rn >= R) break;
        // the next row: its Q is element k + 1 + ntiles
        qb = (qb + 1 + ntiles) & 1;
        rc = rn;
        ric = rin;
        Tc = Tn;
        rn = rnn;
        rin = rinn;
        Tn = Tnn;
        find_rnn = true;
    }
    // loads into LDS (loads with nothing to fetch, to the dummy row) land
    // before the workgroup's LDS is released
    waitcnt_vm_lgkm0<0>();
}

template <int NB, bool BF16, bool TND>
hipError_t launch_narrow_nb(const KernelArgs& a, hipStream_t stream) {
    if (a.dense)
        hipLaunchKernelGGL((smla_narrow_kernel<NB, BF16, TND, true>), dim3(a.num_wg), dim3(256),
                           0, stream, a);
    else
        hipLaunchKernelGGL((smla_narrow_kernel<NB, BF16, TND, false>), dim3(a.num_wg),
                           dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <bool BF16, bool TND>
hipError_t launch_narrow_t(const KernelArgs& a, hipStream_t stream) {
    if (a.G <= 16) return launch_narrow_nb<1, BF16, TND>(a, stream);
    if (a.G <= 32) return launch_narrow_nb<2, BF16, TND>(a, stream);
    return launch_narrow_nb<4, BF16, TND>(a, stream);
}

template <bool BF16, bool TND>
hipError_t occupancy_narrow_t(int* out) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(
        out, reinterpret_cast<const void*>(&smla_narrow_kernel<4, BF16, TND, false>), 256, 0);
}

template <bool BF16, bool TND>
hipError_t launch_wide_t(const KernelArgs& a, hipStream_t stream) {
    // (dense rows, without an index list, are a variant of their own: the
    // choice would otherwise be a branch in every tile)
    const dim3 grid(a.num_wg), block(256);
    if (a.W <= kRowCap) {
        if (a.dense)
            hipLaunchKernelGGL((smla_wide_kernel<BF16, TND, true, true>), grid, block, 0, stream, a);
        else
            hipLaunchKernelGGL((smla_wide_kernel<BF16, TND, true, false>), grid, block, 0, stream, a);
    } else {
        if (a.dense)
            hipLaunchKernelGGL((smla_wide_kernel<BF16, TND, false, true>), grid, block, 0, stream, a);
        else
            hipLaunchKernelGGL((smla_wide_kernel<BF16, TND, false, false>), grid, block, 0, stream, a);
    }
    return hipGetLastError();
}

template <bool BF16, bool TND>
hipError_t occupancy_wide_t(int* out) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(
        out, reinterpret_cast<const void*>(&smla_wide_kernel<BF16, TND, true, false>), 256, 0);
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

#endif  // !SMLA_LSE_TU

#ifdef SMLA_LSE_TU
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

#endif  // SMLA_LSE_TU

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

#ifndef SMLA_LSE_TU
int kernel_variant(int64_t G, int64_t topk) {
    // (the dense case, topk 0, has no index list: no limit on its entries)
    if (G <= 64) return kKernelNarrow;
    return topk <= kVcap ? kKernelWide : kKernelGeneral;
}

hipError_t launch(const KernelArgs& a, int ht, bool bf16, bool tnd, hipStream_t stream) {
    const int v = kernel_variant(a.G, a.dense ? 0 : a.K);
    if (v == kKernelNarrow) {
        if (bf16) return tnd ? launch_narrow_t<true, true>(a, stream) : launch_narrow_t<true, false>(a, stream);
        return tnd ? launch_narrow_t<false, true>(a, stream) : launch_narrow_t<false, false>(a, stream);
    }
    if (v == kKernelWide) {
        if (bf16) return tnd ? launch_wide_t<true, true>(a, stream) : launch_wide_t<true, false>(a, stream);
        return tnd ? launch_wide_t<false, true>(a, stream) : launch_wide_t<false, false>(a, stream);
    }
    SMLA_DISPATCH(launch_t, a, stream);
}

hipError_t resident_per_cu(int ht, bool bf16, bool tnd, int64_t G, int64_t topk, int* out) {
    const int v = kernel_variant(G, topk);
    if (v == kKernelNarrow) {
        if (bf16) return tnd ? occupancy_narrow_t<true, true>(out) : occupancy_narrow_t<true, false>(out);
        return tnd ? occupancy_narrow_t<false, true>(out) : occupancy_narrow_t<false, false>(out);
    }
    if (v == kKernelWide) {
        if (bf16) return tnd ? occupancy_wide_t<true, true>(out) : occupancy_wide_t<true, false>(out);
        return tnd ? occupancy_wide_t<false, true>(out) : occupancy_wide_t<false, false>(out);
    }
    SMLA_DISPATCH(occupancy_t, out);
}

#endif  // !SMLA_LSE_TU

#ifdef SMLA_LSE_TU
hipError_t launch_lse(const KernelArgs& a, int ht, bool bf16, bool tnd, hipStream_t stream) {
    SMLA_DISPATCH(launch_lse_t, a, stream);
}

hipError_t lse_resident_per_cu(int ht, bool bf16, bool tnd, int* out) {
    SMLA_DISPATCH(occupancy_lse_t, out);
}

#endif  // SMLA_LSE_TU

}  // namespace smla
