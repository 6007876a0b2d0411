// Pipelined kernel of the sparse Flash-MLA Softmax-L1Norm for gfx950: rows of
// up to 64 heads, any number of indices (or dense rows).
//
// The operation ("SparseFlashMlaSoftmaxL1Norm" article, section 三阶段计算公式):
//   stage 1  gather the row's selected rows of K            (sparse_indices)
//   stage 2  P = exp(Mask(Q . Ksel^T * scale) - lse)          (SimpleSoftmax)
//   stage 3  out = sum_g P / G                                (ReduceSum over G)
// written into a zero-filled fp32 row of width S2 (BSND) or T2 (TND).
#include "smla_device.h"

namespace smla {
namespace {

// ---------------------------------------------------------------------------
// Pipelined kernel for rows of up to 64 heads (NB = 1, 2 or 4 blocks of 16
// heads), any number of indices per row, or the dense case.
//
// v_mfma_f32_16x16x32 with Q as A (16 heads x 32 of D) and K as B (32 of D
// x 16 keys): lane l holds head 16b + (l & 15) of Q and key (l & 15) of K,
// 8 elements of D per k-step, and receives the scores of key (l & 15) for
// heads 16b + 4 (l >> 4) + i, i < 4. Any split of D over the k-steps and
// lane groups gives the same dot product as long as Q and K share it: lane
// group g = l >> 4 takes the 16-byte chunk 16 g + s of D in k-step s, so
// that the 16 lanes of a group read 16 consecutive chunks of their rows. (The
// interleaved split, chunk 4 s + g, measured a two-way LDS bank conflict on
// every operand read: 8 cycles per ds_read_b128 against 4; the blocked one
// is conflict-free at the row pitch of 65 chunks.) Wave w takes keys
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
// start has two workgroup barriers: Q landed, Q read. Rows of up to 16
// heads keep Q in a place of its own instead, loaded one row ahead by wave
// 0, and the stream holds key tiles only ([tiles of r0, tiles of r1, ...]):
// a row's last tile reads the next row's tile 0 and loads on. Such a row has
// at least three tiles (the others without a used entry when needed), so
// that the three rows decoded ahead always cover the five elements a tile
// plans ahead.
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

// max(a, b) in one instruction (fmaxf quiets both inputs for its NaN rules
// first; the lse sums here take finite values or -inf, never NaN)
__device__ __forceinline__ float nar_max(float a, float b) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// x of the lane that DPP control CTRL selects within the lane's row of 16
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                         0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
// Maximum and sum of x over each row of 16 lanes, the same bits in all 16:
// lanes pair by xor 1 and xor 2 inside their quad, then with the mirror lane
// in their half row and in their row (each step adds two equal-bit partial
// results of the pair, in either order: the same sum).
__device__ __forceinline__ float row16_max(float x) {
    x = nar_max(x, dpp_f<0xB1>(x));   // quad_perm [1,0,3,2]
    x = nar_max(x, dpp_f<0x4E>(x));   // quad_perm [2,3,0,1]
    x = nar_max(x, dpp_f<0x141>(x));  // row_half_mirror
    return nar_max(x, dpp_f<0x140>(x));  // row_mirror
}
__device__ __forceinline__ float row16_sum(float x) {
    x = x + dpp_f<0xB1>(x);
    x = x + dpp_f<0x4E>(x);
    x = x + dpp_f<0x141>(x);
    return x + dpp_f<0x140>(x);
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

// The element d after element j of row r0 in the stream over rows r0, r1,
// r2 (T tiles each; R: none). Each row's Q comes first (j = 0: the row's Q,
// j = i + 1: its tile i), unless QS (the rows' Q has a place of its own):
// then the stream holds key tiles only (j = i: tile i). Without branches,
// and everything by value (a choice between captured references would keep
// the row state in memory).
template <bool QS>
__device__ __forceinline__ NarElem nar_elem_plus(int j, int d, int32_t R, int32_t r0, int T0,
                                                 NarRow i0, int32_t r1, int T1, NarRow i1,
                                                 int32_t r2, int T2, NarRow i2) {
    constexpr int kQ = QS ? 0 : 1;  // a row's elements besides its tiles
    const int x0 = j + d;           // offset from r0's first element
    const int x1 = x0 - (T0 + kQ);  // from r1's
    const int x2 = x1 - (T1 + kQ);  // from r2's
    const bool in0 = (r0 < R) & (x0 < T0 + kQ);
    const bool in1 = !in0 & (r1 < R) & (x1 < T1 + kQ);
    const bool in2 = !in0 & !in1 & (r2 < R) & (x2 < T2 + kQ);
    const int x = in0 ? x0 : (in1 ? x1 : x2);
    NarElem e;
    e.kind = (in0 | in1 | in2) ? ((!QS && x == 0) ? kElemQ : kElemKeys) : kElemNone;
    e.tile = x - kQ;
    e.row = in0 ? r0 : (in1 ? r1 : (in2 ? r2 : R));
    e.ri.kbase = in0 ? i0.kbase : (in1 ? i1.kbase : i2.kbase);
    e.ri.col0 = in0 ? i0.col0 : (in1 ? i1.col0 : i2.col0);
    e.ri.vis = in0 ? i0.vis : (in1 ? i1.vis : i2.vis);
    e.ri.n = in0 ? i0.n : (in1 ? i1.n : i2.n);
    return e;
}

// The kernel's body, for the main call (LSE false) and for the softmax_lse
// call (LSE true: the same row walk, loads and waits; each lane keeps, per
// score element, the running maximum M and sum L of 2^(x - M) over its keys,
// in log2 units, and the row end combines the lanes and waves of each head
// into lse = ln 2 (M + log2 L); there is no output row, and the value store of
// each tile is kept, to an offset the buffer range drops, so that every tile
// issues the same number of vector memory instructions as the waits count).
template <int NB, bool BF16, bool TND, bool DENSE, bool LSE>
__device__ __forceinline__ void narrow_body(const KernelArgs& a) {
    constexpr int NT = 256;
    constexpr int NE = NB * 4;             // scores per lane and tile
    constexpr int EPS = NE >= 16 ? 2 : 1;  // epilogue elements per step
    constexpr int NG = NE / EPS;           // epilogue groups: fma in step g, exp g+1, sum g+2
    constexpr int kSteps = kChunks / 4;    // 16 k-steps of 32 along D
    static_assert(NG + 2 <= 10, "the epilogue must end by step 9");
    // LSE: below every score, in log2 units (a finite start keeps every
    // rescale factor finite: an unused entry enters as -inf and adds 2^-inf)
    constexpr float kLseFloor = -1.0e30f;
    // Loads per tile (index loads: one per wave; the dense case has none):
    // two index loads, 16 rows, one store, one lse load. A row start issues
    // as many after tile 1's rows: that load's lse, the next element's index
    // load, rows and lse, the index-list prefetch. (QS: a row's tile 1 was
    // loaded by the previous row's tiles, and the waits after a row start
    // need only at least that many operations after each load they cover.)
    constexpr int kIdx = DENSE ? 0 : 1;
    constexpr int kTileLoads = 2 * kIdx + 16 + 1 + 1;
    constexpr int kRowStartTail = 1 + kIdx + 16 + 1 + kIdx;
    static_assert(kRowStartTail == kTileLoads, "one wait count for every tile");
    constexpr int kJsSlot0 = 4;  // index slots 4..7: the stores' indices, by tile
    // value stores of BSND rows with the non-temporal hint (a row's values land
    // a few to a 128-byte line; TND rows land about nine to a line, which the
    // default policy merges in L2 first: measured 3% faster that way)
    constexpr int kStorePolicy = TND ? 0 : 2;
    // Rows of up to 16 heads (QS) keep their Q (16 KB) in a place of its own
    // and the stream holds key tiles only: a row's last tile reads the next
    // row's tile 0 and loads on, and a row start reads only Q and lse. More
    // heads put their Q in one of the two tile buffers (there is no room for
    // a third).
    constexpr bool QS = NB == 1;
    __shared__ uint4 kbuf[2][kNarKeys * kPitch];
    __shared__ uint4 qbuf[QS ? 16 * kPitch : 1];
    // per wave: the indices of the next loads' tiles (ring of 4, by load
    // number) and of the tiles whose values are stored next (ring of 4, by
    // tile)
    __shared__ int32_t ixbuf[4][8][64];
    __shared__ float lsebuf[64];
    __shared__ uint4 dummy[64];  // loads with nothing to fetch
    __shared__ float cmb[LSE ? 4 : 1][64][2];  // LSE: (M, L) per wave and head

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15;
    const int gq = lane >> 4;
    const int my_slot = 16 * wave + n;  // this lane's key slot in a tile
    const uint4* __restrict__ q4 = static_cast<const uint4*>(a.q);
    const char* __restrict__ kbytes = static_cast<const char*>(a.k);
    const uint32_t kbuf_lds = lds_addr(kbuf);
    const uint32_t qbuf_lds = lds_addr(qbuf);
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
            if (!LSE) zero_span(a.out + r * a.W, 0, a.W, tid, NT);
            ri = nar_row(decode_row<TND>(a, r));
            T = __builtin_amdgcn_readfirstlane((ri.n + kNarKeys - 1) / kNarKeys);
            // QS: at least three tiles (the others without a used entry), so
            // that the rows decoded ahead cover the five stream elements a
            // tile plans ahead, a row's last tile included
            if (QS && T > 0 && T < 3) T = 3;
            // LSE: a row without a used entry has lse -inf
            if (LSE && T == 0 && tid < a.G) a.out[r * a.G + tid] = -__builtin_inff();
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
        return nar_elem_plus<QS>(j, d, R, rc, Tc, ric, rn, Tn, rin, rnn, Tnn, rinn);
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
            // (slot < 0: nothing to keep, into the dummy row)
            dma_dword(d, (uint32_t)__builtin_amdgcn_readfirstlane(
                             (int32_t)(slot < 0 ? dummy_lds : ix_lds + (uint32_t)slot * 256u)),
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
        const bool isq = !LSE && e.kind == kElemQ;  // (LSE: no lse input; an empty load)
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
    // QS: row `row`'s Q (its G head rows; rows past G read zeros) and its
    // lse into their places, by wave 0 (the other waves issue nothing here:
    // the waits that follow count only what is older than a tile's loads)
    auto q_load = [&](int32_t row) __attribute__((always_inline)) {
        if constexpr (QS) {
            if (wave == 0) {
                const bool live = row < R;
                const i32x4_t dq =
                    uniform_desc(raw_desc(q4 + (int64_t)(live ? row : 0) * a.G * kChunks,
                                          live ? (uint32_t)a.G * 1024u : 0u));
                const uint32_t m0 =
                    (uint32_t)__builtin_amdgcn_readfirstlane((int32_t)(live ? qbuf_lds : dummy_lds));
                const int32_t step = live ? kRowBytes : 0;
                dma_row_first<true>(dq, m0, 0, voff16, step);
#pragma unroll
                for (int i = 1; i < 16; ++i) dma_row_next<true>(dq, i * 1024, voff16, step);
                const bool lv = !LSE && live;
                dma_dword(uniform_desc(raw_desc(a.lse + (int64_t)(lv ? row : 0) * a.G,
                                                lv ? (uint32_t)a.G * 4u : 0u)),
                          (uint32_t)__builtin_amdgcn_readfirstlane(
                              (int32_t)(lv ? lse_lds : dummy_lds)),
                          0, voff4);
            }
        }
    };

    // ---- start: Q of the first row into buffer 0, its tile 0 into buffer 1,
    // the indices of the row start's two loads (load numbers 0 and 1) into
    // their slots. QS: Q into its place, tiles 0 and 1 into buffers 0 and 1,
    // the indices of the next two loads (tiles 2 and 3, load numbers 0 and
    // 1) into their slots.
    int qb = QS ? 1 : 0;  // tile t of the current row is in buffer (qb + 1 + t) & 1
    int ip = 0;           // load number of the next load
    NarElem pe0, pe1;     // the elements of loads ip and ip + 1
    if constexpr (QS) {
        const NarElem e0 = elem_plus(0, 0), e1 = elem_plus(0, 1);
        pe0 = elem_plus(0, 2);
        pe1 = elem_plus(0, 3);
        idx_prefetch(rn);
        idx_dma(kJsSlot0 + 3, e0.row, e0.tile, e0.kind == kElemKeys);
        idx_dma(kJsSlot0 + 2, e1.row, e1.tile, e1.kind == kElemKeys);
        idx_dma(0, pe0.row, pe0.tile, pe0.kind == kElemKeys);
        idx_dma(1, pe1.row, pe1.tile, pe1.kind == kElemKeys);
        q_load(rc);
        waitcnt_vm_lgkm0<0>();
        issue_now(e0, kJsSlot0 + 3, 0);
        issue_now(e1, kJsSlot0 + 2, 1);
    } else {
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
    float lm[LSE ? NE : 1], ll[LSE ? NE : 1];  // LSE: per element, M and L of the row
    uint4 opa[kSteps], opb[kSteps];  // B operands of a tile, read a tile ahead
    f32x4_t xa[NB], xb[NB];

    bool find_rnn = false;
    bool first = true;      // QS: the workgroup's first row
    bool prev_odd = false;  // QS: the previous row had an odd number of tiles
    for (;;) {
        if constexpr (QS) {
            // ---- row start, QS. rnn (found now: its rows are zero-filled
            // before the next row start's wait covers the stores). Row rc's Q
            // and lse were loaded at the previous row start, followed by at
            // least a tile's loads, so a wait that leaves the last tile's in
            // flight covers them (the first row: everything); the workgroup
            // reads them, and once it has, wave 0 loads the next row's. Tile 0
            // was read by the previous row's last tile into the register set
            // of its parity (the first row: read here, and its tile 2 loaded).
            if (find_rnn) rnn = rn < R ? next_row(rinn, Tnn) : R;
            find_rnn = false;
            if (first)
                waitcnt_vm_lgkm0<0>();
            else
                waitcnt_vm_lgkm0<kTileLoads>();
            asm volatile("s_barrier" ::: "memory");
#pragma unroll
            for (int s = 0; s < kSteps; ++s) qa[0][s] = qbuf[n * kPitch + 16 * gq + s];
#pragma unroll
            for (int e = 0; e < NE; ++e) {
                const int h = 4 * gq + (e & 3);
                if constexpr (LSE) {
                    lm[e] = kLseFloor;
                    ll[e] = 0.0f;
                    l2[e] = 0.0f;
                } else {
                    const float v = lsebuf[h];
                    l2[e] = h < a.G ? v * kLog2e : __builtin_inff();
                }
            }
            if (first) {
#pragma unroll
                for (int s = 0; s < kSteps; ++s)
                    opa[s] = kbuf[(qb + 1) & 1][my_slot * kPitch + 16 * gq + s];
            } else if (prev_odd) {
#pragma unroll
                for (int s = 0; s < kSteps; ++s) opa[s] = opb[s];
            }
            waitcnt_vm_lgkm0<63>();
            asm volatile("s_barrier" ::: "memory");
            if (first) {
                const NarElem e2 = elem_plus(0, 4);
                idx_dma((ip + 2) & 3, e2.row, e2.tile, e2.kind == kElemKeys);
                issue_now(pe0, ip & 3, (qb + 1) & 1);
                pe0 = pe1;
                pe1 = e2;
                ++ip;
            }
            q_load(rn);
            idx_dma(kJsSlot0, rc, 0, true);
            idx_prefetch(rnn);
            first = false;
        } else {
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
                qa[b][s] = kbuf[qb][(16 * b + n) * kPitch + 16 * gq + s];
#pragma unroll
        for (int e = 0; e < NE; ++e) {
            const int h = 16 * (e >> 2) + 4 * gq + (e & 3);
            if constexpr (LSE) {
                lm[e] = kLseFloor;
                ll[e] = 0.0f;
                l2[e] = 0.0f;
            } else {
                const float v = lsebuf[h];
                l2[e] = h < a.G ? v * kLog2e : __builtin_inff();
            }
        }
#pragma unroll
        for (int s = 0; s < kSteps; ++s) opa[s] = kbuf[qb ^ 1][my_slot * kPitch + 16 * gq + s];
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
            const bool st = !LSE & (gq == 0) & (tile >= 0) & used_of(ri, tile, jj);
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
            const uint4* nsrc = &kbuf[nb][my_slot * kPitch + 16 * gq];
            // this load, and the load two on (its indices are loaded now)
            const NarElem E = steady ? keys_elem(t + 3) : pe0;
            const NarElem Enew = steady ? keys_elem(t + 5) : elem_plus(t + (QS ? 1 : 2), 4);
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
            bool uprev = false;             // LSE: tile t-1's key of this lane is used
            // LSE: an element's score, new maximum and rescale factors
            float ly[2], lmn[2], ld1[2], ld2[2];
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
                        nop[4 * s + b] = nsrc[4 * s + b];
                    } else if (b == 3) {
#pragma unroll
                        for (int k = 0; k < 4; ++k) nop[4 * s + k] = nsrc[4 * s + k];
                    }
                }
                // LSE: the lane's key of tile t-1 is used (its index was read
                // in step 0); each element of tile t-1: its scaled score y
                // (-inf if unused), the new maximum, the two rescale factors,
                // the sum. With four head blocks one element per step (steps
                // 1..15, two in step 15), spread over the step's four gaps;
                // with fewer, EPS elements per step from step 2, after the
                // step's last MFMA.
                if constexpr (LSE) {
                    if (s == 1 && b == (NB == 4 ? 0 : 3)) {
                        uprev = (t >= 1) & used_of(ri, t - 1, js);
                    }
                    auto first_half = [&](int e, int k) __attribute__((always_inline)) {
                        ly[k] = uprev ? prev[e >> 2][e & 3] * a.c_scale : -__builtin_inff();
                        lmn[k] = nar_max(lm[e], ly[k]);
                        pin(ly[k]);
                        pin(lmn[k]);
                    };
                    auto second_half = [&](int e, int k) __attribute__((always_inline)) {
                        const float d1 = __builtin_amdgcn_exp2f(lm[e] - lmn[k]);
                        const float d2 = __builtin_amdgcn_exp2f(ly[k] - lmn[k]);
                        ll[e] = __builtin_fmaf(ll[e], d1, d2);
                        lm[e] = lmn[k];
                        pin(ll[e]);
                        pin(lm[e]);
                    };
                    if constexpr (NB == 4) {
                        static_assert(NE == 16, "four head blocks: 16 elements");
#pragma unroll
                        for (int k = 0; k < 2; ++k) {
                            const int e = k == 0 ? s - 1 : 15;
                            if ((k == 0 && s >= 1) || (k == 1 && s == 15)) {
                                if (b == 0) {
                                    first_half(e, k);
                                } else if (b == 1) {
                                    ld1[k] = __builtin_amdgcn_exp2f(lm[e] - lmn[k]);
                                    pin(ld1[k]);
                                } else if (b == 2) {
                                    ld2[k] = __builtin_amdgcn_exp2f(ly[k] - lmn[k]);
                                    pin(ld2[k]);
                                } else {
                                    ll[e] = __builtin_fmaf(ll[e], ld1[k], ld2[k]);
                                    lm[e] = lmn[k];
                                    pin(ll[e]);
                                    pin(lm[e]);
                                }
                            }
                        }
                    } else if (b == 3) {
#pragma unroll
                        for (int k = 0; k < EPS; ++k) {
                            const int e = EPS * (s - 2) + k;
                            if (s >= 2 && e < NE) {
                                first_half(e, k);
                                second_half(e, k);
                            }
                        }
                    }
                }
                // epilogue of tile t-1: sum (group s-2), exp2 (s-1), fma (s)
                if (!LSE && ((NB == 4 && b <= 1) || (NB < 4 && b == 3))) {
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
                if (!LSE && ((NB == 4 && b >= 2) || (NB < 4 && b == 3))) {
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
                if (!LSE && b == (NB == 4 ? 2 : 3)) {
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
                        idx_dma((!QS || t + 1 < ntiles) ? kJsSlot0 + ((t + 1) & 3) : -1, row,
                                t + 1, true);
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
                                                          orsrc, store_off(t - 1, js), 0, kStorePolicy);
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
            pe0 = elem_plus(t + (QS ? 1 : 2), 2);
            pe1 = elem_plus(t + (QS ? 1 : 2), 3);
        }
        for (; t + 2 < ntiles; t += 2) {
            tile_body(Par<1>{}, Par<0>{}, t, opa, opb, xb, xa);
            tile_body(Par<1>{}, Par<0>{}, t + 1, opb, opa, xa, xb);
        }
        // a row's last tile (QS, when a row follows: it reads that row's
        // tile 0 and loads on)
        const bool more_last = QS && rn < R;
        if (t + 1 < ntiles) {
            tile_body(Par<1>{}, Par<0>{}, t, opa, opb, xb, xa);
            if (more_last)
                tile_body(Par<1>{}, Par<0>{}, t + 1, opb, opa, xa, xb);
            else
                tile_body(Par<0>{}, Par<0>{}, t + 1, opb, opa, xa, xb);
        } else {
            if (more_last)
                tile_body(Par<1>{}, Par<0>{}, t, opa, opb, xb, xa);
            else
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
        if constexpr (LSE) {
            // the last tile's scores into M, L; then the 16 lanes of each
            // group (one key each, the same heads) combine in registers, the
            // four waves (their keys) through LDS (wave 0 first), and lanes
            // below G write the row's lse
            // (the last tile's indices are older than its loads; with no
            // loads of its own, wait for everything)
            if (more_last)
                waitcnt_vm_lgkm0<kTileLoads>();
            else
                waitcnt_vm_lgkm0<0>();
            const int32_t js = idx_read(kJsSlot0 + ((ntiles - 1) & 3));
            const bool ul = used_of(ri, ntiles - 1, js);
            auto last_update = [&](const f32x4_t(&x)[NB]) __attribute__((always_inline)) {
#pragma unroll
                for (int e = 0; e < NE; ++e) {
                    const float y = ul ? x[e >> 2][e & 3] * a.c_scale : -__builtin_inff();
                    const float mn = nar_max(lm[e], y);
                    ll[e] = __builtin_fmaf(ll[e], __builtin_amdgcn_exp2f(lm[e] - mn),
                                           __builtin_amdgcn_exp2f(y - mn));
                    lm[e] = mn;
                }
            };
            if (ntiles & 1)
                last_update(xa);
            else
                last_update(xb);
            auto combine = [](float m1, float l1, float m2, float l2v, float& m, float& l) {
                m = nar_max(m1, m2);
                l = l1 * __builtin_amdgcn_exp2f(m1 - m) + l2v * __builtin_amdgcn_exp2f(m2 - m);
            };
#pragma unroll
            for (int e = 0; e < NE; ++e) {
                // the group's maximum, each lane's sum rescaled to it, summed
                const float m = row16_max(lm[e]);
                ll[e] = row16_sum(ll[e] * __builtin_amdgcn_exp2f(lm[e] - m));
                lm[e] = m;
                if (n == 0) {
                    const int h = 16 * (e >> 2) + 4 * gq + (e & 3);
                    cmb[wave][h][0] = lm[e];
                    cmb[wave][h][1] = ll[e];
                }
            }
            lds_barrier();
            if (tid < a.G) {
                float m = cmb[0][tid][0], l = cmb[0][tid][1];
#pragma unroll
                for (int w = 1; w < 4; ++w) combine(m, l, cmb[w][tid][0], cmb[w][tid][1], m, l);
                a.out[(int64_t)row * a.G + tid] =
                    l > 0.0f ? (m + __builtin_amdgcn_logf(l)) * kLn2 : -__builtin_inff();
            }
        } else {
            const float v = (ntiles & 1) ? last_value(xa) : last_value(xb);
            if (more_last)
                waitcnt_vm_lgkm0<kTileLoads>();
            else
                waitcnt_vm_lgkm0<0>();
            const int32_t js = idx_read(kJsSlot0 + ((ntiles - 1) & 3));
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), orsrc,
                                                  store_off(ntiles - 1, js), 0, kStorePolicy);
        }
        if (rn >= R) break;
        // the next row: its Q is element k + 1 + ntiles (QS: its tile 0 is
        // element k + ntiles, k = this row's tile 0)
        qb = (qb + (QS ? 0 : 1) + ntiles) & 1;
        prev_odd = (ntiles & 1) != 0;
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

template <int NB, bool BF16, bool TND, bool DENSE>
__global__ __launch_bounds__(256, 1) void smla_narrow_kernel(KernelArgs a) {
    narrow_body<NB, BF16, TND, DENSE, false>(a);
}

// The softmax_lse call for up to 64 heads on the same pipeline.
template <int NB, bool BF16, bool TND, bool DENSE>
__global__ __launch_bounds__(256, 1) void smla_lse_narrow_kernel(KernelArgs a) {
    narrow_body<NB, BF16, TND, DENSE, true>(a);
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

template <int NB, bool BF16, bool TND>
hipError_t launch_lse_narrow_nb(const KernelArgs& a, hipStream_t stream) {
    if (a.dense)
        hipLaunchKernelGGL((smla_lse_narrow_kernel<NB, BF16, TND, true>), dim3(a.num_wg),
                           dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((smla_lse_narrow_kernel<NB, BF16, TND, false>), dim3(a.num_wg),
                           dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <bool BF16, bool TND>
hipError_t launch_lse_narrow_t(const KernelArgs& a, hipStream_t stream) {
    if (a.G <= 16) return launch_lse_narrow_nb<1, BF16, TND>(a, stream);
    if (a.G <= 32) return launch_lse_narrow_nb<2, BF16, TND>(a, stream);
    return launch_lse_narrow_nb<4, BF16, TND>(a, stream);
}

template <bool BF16, bool TND>
hipError_t occupancy_lse_narrow_t(int* out) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(
        out, reinterpret_cast<const void*>(&smla_lse_narrow_kernel<4, BF16, TND, false>), 256,
        0);
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

}  // namespace

hipError_t launch_narrow(const KernelArgs& a, bool bf16, bool tnd, hipStream_t stream) {
    SMLA_DISPATCH2(launch_narrow_t, a, stream);
}

hipError_t narrow_resident_per_cu(bool bf16, bool tnd, int* out) {
    SMLA_DISPATCH2(occupancy_narrow_t, out);
}

hipError_t launch_lse_narrow(const KernelArgs& a, bool bf16, bool tnd, hipStream_t stream) {
    SMLA_DISPATCH2(launch_lse_narrow_t, a, stream);
}

hipError_t lse_narrow_resident_per_cu(bool bf16, bool tnd, int* out) {
    SMLA_DISPATCH2(occupancy_lse_narrow_t, out);
}

}  // namespace smla
