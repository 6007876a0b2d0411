// Device code shared by the gfx950 kernels of the sparse Flash-MLA
// Softmax-L1Norm: types and constants, the decode of a query row, buffer
// descriptors, the MFMA wrappers, direct loads into LDS and the waits that
// count them.
//
// The operation ("SparseFlashMlaSoftmaxL1Norm" article, section 三阶段计算公式):
//   stage 1  gather the row's selected rows of K            (sparse_indices)
//   stage 2  P = exp(Mask(Q . Ksel^T * scale) - lse)          (SimpleSoftmax)
//   stage 3  out = sum_g P / G                                (ReduceSum over G)
// written into a zero-filled fp32 row of width S2 (BSND) or T2 (TND).
#pragma once

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
// With NT the loads carry the non-temporal hint (rows read once).
template <bool NT = false>
__device__ __forceinline__ void dma_row_first(i32x4_t desc, uint32_t m0, int32_t soff,
                                              uint32_t voff, int32_t step) {
    if constexpr (NT)
        asm volatile(
            "s_mov_b32 m0, %0\n\t"
            "s_nop 0\n\t"
            "buffer_load_dwordx4 %1, %2, %3 offen nt lds\n\t"
            "s_add_u32 m0, m0, %4"
            :
            : "s"(m0), "v"(voff), "s"(desc), "s"(soff), "s"(step)
            : "memory", "m0", "scc");
    else
        asm volatile(
            "s_mov_b32 m0, %0\n\t"
            "s_nop 0\n\t"
            "buffer_load_dwordx4 %1, %2, %3 offen lds\n\t"
            "s_add_u32 m0, m0, %4"
            :
            : "s"(m0), "v"(voff), "s"(desc), "s"(soff), "s"(step)
            : "memory", "m0", "scc");
}
template <bool NT = false>
__device__ __forceinline__ void dma_row_next(i32x4_t desc, int32_t soff, uint32_t voff,
                                             int32_t step) {
    if constexpr (NT)
        asm volatile(
            "buffer_load_dwordx4 %0, %1, %2 offen nt lds\n\t"
            "s_add_u32 m0, m0, %3"
            :
            : "v"(voff), "s"(desc), "s"(soff), "s"(step)
            : "memory", "m0", "scc");
    else
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

constexpr int kRowBytes = kPitch * 16;          // one key row in LDS

}  // namespace

// Dispatch over the head tiles (1, 2 or 4 blocks of 32 heads), the dtype and
// the layout: FN<HT, BF16, TND>(...).
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

// Dispatch over the dtype and the layout: FN<BF16, TND>(...).
#define SMLA_DISPATCH2(FN, ...)                                                       \
    do {                                                                              \
        if (bf16) return tnd ? FN<true, true>(__VA_ARGS__) : FN<true, false>(__VA_ARGS__); \
        return tnd ? FN<false, true>(__VA_ARGS__) : FN<false, false>(__VA_ARGS__);    \
    } while (0)

}  // namespace smla
