// Pipelined softmax_lse kernel for gfx950: rows of 65..128 heads with at most
// 2048 indices (or dense rows). It computes the input the Softmax-L1Norm
// operation consumes ("SparseFlashMlaSoftmaxL1Norm" article, parameter
// table, input softmax_lse: the forward attention pass's log-sum-exp, whose
// formula the article defers to the sparse_flash_mla operator; taken here as
// its plain definition over the same used entries as the main call)
//   lse[r, g] = log sum_{t used} exp(scale * q[r,g,:] . K[key(t),:]),
// -inf for a row without a used entry.
//
// Work layout as in the main call's pipelined kernel: one 4-wave workgroup
// per CU walks its rows; wave w takes heads 64 (w & 1) .. +63 (two 32-head
// MFMA blocks) and keys 32 (w >> 1) .. +31 of each 64-key tile; two tiles
// live in LDS and each wave gathers 16 rows of later tiles between its
// MFMAs; one workgroup barrier in the middle of each tile; the next row's Q
// is loaded by the streams of the last tiles into the buffers they free.
//
// The MFMA operands are swapped (S = K_tile . Q^T): K is the A operand,
// read from LDS into an 8-deep ring and shared by the two blocks, Q the B
// operand in registers. Lane (c, h) of block b's accumulator then holds the
// scores of keys 8 (e / 4) + 4 h + e % 4 (e < 16) of the wave's 32 for head
// 64 hg + 32 b + c, so the reduction over keys runs inside the lane: a base
// B and a sum l of 2^(x - B), x the score in log2 units. The two half-waves
// of a head combine in registers at the end of the row, the two key halves
// in LDS.
#include "smla_device.h"

namespace smla {
namespace {

constexpr int kLseKeys = 64;  // keys per tile
static_assert(kVcap == kWideIndexCap, "the index list in LDS holds kVcap entries");
constexpr int kLseBufBytes = kLseKeys * kRowBytes;
constexpr int kLseBar = 24;      // the tile's workgroup barrier, after step 24's MFMAs
constexpr float kLseLazy = 64.0f;  // largest excess over the base summed without rebasing

// max(a, b) in one instruction. The scores here are finite or +-inf, never
// NaN; fmaxf's NaN rules make the compiler quiet both inputs first (three
// instructions in place of one).
__device__ __forceinline__ float max_f32(float a, float b) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// (base, sum) pairs m, l and m2, l2 of one head over disjoint entries,
// combined: M = max(m, m2), L = l 2^(m - M) + l2 2^(m2 - M) (a base of -inf
// has an empty sum)
__device__ __forceinline__ void lse_combine(float m, float l, float m2, float l2, float& M,
                                            float& L) {
    M = max_f32(m, m2);
    const float base = M == -__builtin_inff() ? 0.0f : M;
    L = l * __builtin_amdgcn_exp2f(m - base) + l2 * __builtin_amdgcn_exp2f(m2 - base);
}

// One 64-key tile of one wave, 32 steps, laid out as the main call's
// pipelined tile: step s issues the two MFMAs of k-step s (one shared A
// operand from the ring), the ring read 8 steps ahead, the gather loads of
// this wave's rows of later tiles (rows 7..15 of tile t+1 at steps 1..9,
// rows 0..6 of tile t+2 at steps 25..31) and element s of the previous
// tile's epilogue, y = x - B of element e (elements 0..15 are block 0's,
// 16..31 block 1's), its maximum and the sum of its 2^y. With MASK, y is set
// to -inf for an unused entry: bit 8 (e / 4) + 4 h + e % 4 of `pslots` says
// whether the previous tile's element e of half h is a used entry. The
// masks fill the first gap, so that variant puts y of element s and the
// term of element s - 1 in the first gap, the maximum and 2^y in the
// second. Without MASK (every entry of the previous tile used) the first
// gap holds the whole epilogue: y of element s, the maximum and 2^y of
// element s - 1, the term of element s - 2; the second keeps the operand
// read, the gather load and its wait. The tile's workgroup barrier follows
// step 24's MFMAs (every wave has then read its last operand of this tile
// and has its rows of the next one landed). With NT stream B's loads carry
// the non-temporal hint (as in the main call's kernel: the last tiles of a
// row, where stream B loads the next row's Q).
template <bool BF16, bool MASK, bool NT, typename Mid2>
__device__ __forceinline__ void lse_tile(const uint4* __restrict__ cur,
                                         const uint4* __restrict__ nxt, uint4 (&ring)[8],
                                         const uint4* qa0, const uint4* qa1,
                                         const f32x16_t& prev0, const f32x16_t& prev1,
                                         uint32_t pslots, float c, float b0, float b1,
                                         float& ymax0, float& ymax1, float& sum0, float& sum1,
                                         i32x4_t desc_a, i32x4_t desc_b, int32_t m0a,
                                         int32_t stepa, int32_t offa, int32_t m0b, int32_t stepb,
                                         const int32_t& offb, uint32_t voff, Mid2 mid2,
                                         f32x16_t& acc0, f32x16_t& acc1) {
    constexpr int kSteps = kChunks / 2;
    constexpr int kLead = 8;
    constexpr float kNegInf = -__builtin_inff();
    acc0 = f32x16_t{};
    acc1 = f32x16_t{};
    float nb0 = -b0, nb1 = -b1;
    // (each variant marks its negated bases with its own empty asm, so that
    // the two variants' shifts are not one computation that the compiler
    // could hoist above the branch choosing between them)
    if (MASK)
        asm volatile("; masked" : "+v"(nb0), "+v"(nb1));
    else
        asm volatile("; unmasked" : "+v"(nb0), "+v"(nb1));
    float y = 0.0f, ex = 0.0f;  // y of the latest element, 2^y of the one before
    ymax0 = kNegInf;
    ymax1 = kNegInf;
    sum0 = 0.0f;
    sum1 = 0.0f;
    int32_t soa[2] = {0, 0}, sob[2] = {0, 0};
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
        __builtin_amdgcn_sched_barrier(0);
        acc0 = mfma_32x32x16<BF16>(ring[s & 7], qa0[s], acc0);
        asm volatile("" ::"v"(acc0));
        // first gap: y of element s (masked); the term of element s - 1
        // (with MASK) or s - 2 (without), and without MASK the maximum and
        // 2^y of element s - 1
        const int ls = MASK ? s - 1 : s - 2;  // element whose term is added
        if (ls >= 0 && ls < 16) {
            sum0 += ex;
            pin(sum0);
        } else if (ls >= 16) {
            sum1 += ex;
            pin(sum1);
        }
        if (!MASK && s >= 1) {
            if (s - 1 < 16) {
                ymax0 = max_f32(ymax0, y);
                pin(ymax0);
            } else {
                ymax1 = max_f32(ymax1, y);
                pin(ymax1);
            }
            ex = __builtin_amdgcn_exp2f(y);
            pin(ex);
        }
        {
            const int e = s & 15;
            const float x = s < 16 ? prev0[e] : prev1[e];
            y = __builtin_fmaf(x, c, s < 16 ? nb0 : nb1);
            if (MASK) y = select_lanes(used_lanes(pslots, e), y, kNegInf);
            pin(y);
        }
        if (s <= 8) {
            soa[s & 1] = __builtin_amdgcn_readlane(offa, s + 7);
            pin_s(soa[s & 1]);
        } else if (s >= 24 && s <= 30) {
            sob[s & 1] = __builtin_amdgcn_readlane(offb, s - 24);
            pin_s(sob[s & 1]);
        }
        __builtin_amdgcn_sched_barrier(0);
        acc1 = mfma_32x32x16<BF16>(ring[s & 7], qa1[s], acc1);
        asm volatile("" ::"v"(acc1));
        // second gap: with MASK the element's maximum and term; the operand
        // read 8 steps ahead and the gather loads
        if (MASK) {
            if (s < 16) {
                ymax0 = max_f32(ymax0, y);
                pin(ymax0);
            } else {
                ymax1 = max_f32(ymax1, y);
                pin(ymax1);
            }
            ex = __builtin_amdgcn_exp2f(y);
            pin(ex);
        }
        if (s == kLseBar) barrier_after_vmcnt(0);
        ring[(s + kLead) & 7] =
            s + kLead < kSteps ? cur[2 * (s + kLead)] : nxt[2 * (s + kLead - kSteps)];
        if (s == 1)  // stream A: row s + 6 of tile t+1
            dma_row_first(desc_a, (uint32_t)m0a, soa[0], voff, stepa);
        else if (s >= 2 && s <= 9)
            dma_row_next(desc_a, soa[(s - 1) & 1], voff, stepa);
        if (s == 25)  // stream B: row s - 25 of tile t+2
            dma_row_first<NT>(desc_b, (uint32_t)m0b, sob[0], voff, stepb);
        else if (s >= 26)
            dma_row_next<NT>(desc_b, sob[(s - 1) & 1], voff, stepb);
        mid2(s);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (!MASK) {  // element 30's term, element 31's maximum and term
        sum1 += ex;
        ymax1 = max_f32(ymax1, y);
        ex = __builtin_amdgcn_exp2f(y);
    }
    sum1 += ex;  // element 31's term
}

template <bool BF16, bool TND, bool DENSE>
__global__ __launch_bounds__(256, 1) void smla_lse_wide_kernel(KernelArgs a) {
    constexpr int HT = 4;
    constexpr int kRowsPerWave = kLseKeys / HT;  // gathered rows per wave and tile
    constexpr int kIdxOps = kVcap / 64 / HT;     // loads of one index list per wave
    constexpr float kNegInf = -__builtin_inff();
    __shared__ uint4 kbuf[2][kLseKeys * kPitch];  // tile t in buffer t % 2
    __shared__ int32_t ibuf[2][kVcap];            // index lists: this row, the next row
    __shared__ float cmb[2][HT * 32][2];          // (base, sum) per key half and head
    __shared__ uint4 dummy[64];                   // loads of a tile with nothing to gather

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hg = wave & 1;   // head group: heads 64 hg .. 64 hg + 63
    const int kh = wave >> 1;  // key half: keys 32 kh .. 32 kh + 31 of a tile
    const int half = lane >> 5;
    const int col = lane & 31;
    // this wave gathers rows 16 w .. 16 w + 15 of every tile; lane l < 16
    // holds the index of row 16 w + l
    const int my_slot = kRowsPerWave * wave + (lane & 15);
    const uint4* __restrict__ q4 = static_cast<const uint4*>(a.q);
    const char* __restrict__ kbytes = static_cast<const char*>(a.k);
    const uint32_t kbuf_lds = lds_addr(kbuf);
    const uint32_t ibuf_lds = lds_addr(ibuf);
    const uint32_t dummy_lds = lds_addr(dummy);
    const uint32_t voff16 = (uint32_t)lane << 4;
    const uint32_t voff4 = (uint32_t)lane << 2;

    int64_t it = 0;
    int64_t rc = row_of(a, 0, blockIdx.x);  // num_wg <= R, so rc < R
    RowInfo ric = decode_row<TND>(a, rc);
    uint4 qa0[kChunks / 2], qa1[kChunks / 2];
    int64_t rn = a.R, rln = rc;  // next row, and the row its loads read
    RowInfo rin = ric;
    int ib = 0;  // ibuf slot of the current row

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
    // Q passes through LDS as whole rows: Q of row r, heads [h0, h1), into
    // the K buffers, head h -> buffer h / 64, row h % 64
    auto stage_q = [&](int64_t r, int h0, int h1) {
        const i32x4_t qd = raw_desc(q4 + r * a.G * kChunks, (uint32_t)a.G * 1024u);
        for (int h = h0 + wave; h < h1; h += HT)
            dma_row_nt(qd, kbuf_lds + (uint32_t)((h >> 6) * kLseBufBytes + (h & 63) * kRowBytes),
                       h * 1024, voff16);
    };
    // this wave's Q as B operands of its two blocks: lane (c, h) holds head
    // 64 hg + 32 j + c, elements 16 s + 8 h .. +8 of k-step s
    auto read_q = [&]() {
        const uint4* r0 = kbuf[hg] + col * kPitch + half;
        const uint4* r1 = kbuf[hg] + (32 + col) * kPitch + half;
#pragma unroll
        for (int s = 0; s < kChunks / 2; ++s) {
            qa0[s] = r0[2 * s];
            qa1[s] = r1[2 * s];
        }
    };
    // the next row of this workgroup, decoded (its scalar loads waited for
    // here, so that later LDS waits can count)
    auto decode_next = [&]() {
        rn = (it + 1) * a.num_wg < a.R ? row_of(a, it + 1, blockIdx.x) : a.R;
        rln = rn < a.R ? rn : rc;  // the last row loads itself again (unused)
        rin = decode_row<TND>(a, rln);
        waitcnt_vm_lgkm0<63>();
    };
    // Q of row r, heads 64 buf + 16 w + i for i in [i0, i1), into rows
    // 16 w + i of K buffer buf (the layout in which the last tiles of a row
    // stage the next row's Q in the buffers they free)
    auto stage_q_rows = [&](int64_t r, int buf, int i0, int i1) {
        const i32x4_t qd = raw_desc(q4 + r * a.G * kChunks, (uint32_t)a.G * 1024u);
        for (int i = i0; i < i1; ++i) {
            const uint32_t m0 = __builtin_amdgcn_readfirstlane(
                kbuf_lds + (uint32_t)(buf * kLseBufBytes + (kRowsPerWave * wave + i) * kRowBytes));
            const int32_t so =
                __builtin_amdgcn_readfirstlane((64 * buf + kRowsPerWave * wave + i) * 1024);
            dma_row_nt(qd, m0, so, voff16);
        }
    };
    auto ntiles_of = [](const RowInfo& ri) { return (ri.n + kLseKeys - 1) / kLseKeys; };
    // byte offset of the key row of slot my_slot of `tile` holding raw index
    // j: j's row if the entry is used, else row 0 (loaded, never counted)
    auto row_off = [&](const RowInfo& ri, int tile, int32_t j) -> int32_t {
        return ((tile * kLseKeys + my_slot < ri.n) & ((uint32_t)j < (uint32_t)ri.vis)) ? (j << 10)
                                                                                        : 0;
    };
    // A row's start: tile 0 (16 rows) into buffer 0 and rows 0..6 of tile 1
    // into buffer 1 (to the dummy row when there is no tile 1); returns each
    // lane's row offset in tile 1 for the loads of its rows 7..15 in tile 0.
    auto start_row = [&](const RowInfo& ri, int slot) -> int32_t {
        const int nt = __builtin_amdgcn_readfirstlane(ntiles_of(ri));  // uniform
        if (nt == 0) return 0;
        const i32x4_t kd = uniform_desc(k_desc(ri));
        const int32_t* il = ibuf[slot];
        const int32_t o0 = row_off(ri, 0, DENSE ? my_slot : il[my_slot]);
        const int32_t o1 =
            row_off(ri, 1, nt > 1 ? (DENSE ? kLseKeys + my_slot : il[kLseKeys + my_slot]) : 0);
        int32_t so[kRowsPerWave];
#pragma unroll
        for (int i = 0; i < kRowsPerWave; ++i) {
            so[i] = __builtin_amdgcn_readlane(o0, i);
            pin_s(so[i]);
        }
        int32_t m0 = __builtin_amdgcn_readfirstlane(
            (int32_t)(kbuf_lds + (uint32_t)(kRowsPerWave * wave * kRowBytes)));
        const int32_t step0 = __builtin_amdgcn_readfirstlane(kRowBytes);
        dma_row_first(kd, (uint32_t)m0, so[0], voff16, step0);
#pragma unroll
        for (int i = 1; i < kRowsPerWave; ++i) dma_row_next(kd, so[i], voff16, step0);
#pragma unroll
        for (int i = 0; i < 7; ++i) {
            so[i] = __builtin_amdgcn_readlane(o1, i);
            pin_s(so[i]);
        }
        const int32_t step1 = __builtin_amdgcn_readfirstlane(nt > 1 ? kRowBytes : 0);
        m0 = __builtin_amdgcn_readfirstlane(
            (int32_t)(nt > 1 ? kbuf_lds + (uint32_t)(kLseBufBytes + kRowsPerWave * wave * kRowBytes)
                             : dummy_lds));
        dma_row_first(kd, (uint32_t)m0, so[0], voff16, step1);
#pragma unroll
        for (int i = 1; i < 7; ++i) dma_row_next(kd, so[i], voff16, step1);
        return o1;
    };

    // ---- first row: Q and index list, then tile 0 in flight
    load_idx_row(rc, 0);
    stage_q(rc, 0, HT * 32);
    barrier_after_vmcnt(0);
    read_q();
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

        // tile 0 has landed (tile 1's first rows may still be in flight);
        // the operands of its first 8 steps into the ring
        barrier_after_vmcnt(7);
        {
            const uint4* r0 = kbuf[0] + (32 * kh + col) * kPitch + half;
#pragma unroll
            for (int i = 0; i < 8; ++i) ring[i] = r0[2 * i];
        }
        f32x16_t xa0, xa1, xb0 = {}, xb1 = {};
        // the lane's base and sum per block, and the used entries of the
        // previous tile (none before tile 0). The base starts at 0: scores
        // within kLseLazy of it need no rebase (see `body`)
        float B0 = 0.0f, B1 = 0.0f, l0 = 0.0f, l1 = 0.0f;
        uint32_t pslots = 0;
        // The scalar state of a tile's two load streams (as in the main
        // call's pipelined kernel): buffer descriptors, LDS destinations and
        // steps. A stream whose tile does not exist takes the next row's Q
        // (stream A only from tile 1 on) or, with no next row, the dummy row.
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
                has1 || qa ? kbuf_lds + (uint32_t)((1 - par) * kLseBufBytes +
                                                   (kRowsPerWave * wave + 7) * kRowBytes)
                           : dummy_lds));
            r.m0b = __builtin_amdgcn_readfirstlane(
                (int32_t)(has2 || qb ? kbuf_lds + (uint32_t)(par * kLseBufBytes +
                                                             kRowsPerWave * wave * kRowBytes)
                                     : dummy_lds));
            r.sa = has1 || qa ? kRowBytes : 0;
            r.sb = has2 || qb ? kRowBytes : 0;
            return r;
        };
        auto ctl_steady = [&](auto P) -> Ctl {
            constexpr int par = decltype(P)::value;
            Ctl r;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                r.da[i] = __builtin_amdgcn_readfirstlane(kdesc[i]);
                r.db[i] = r.da[i];
            }
            r.m0a = __builtin_amdgcn_readfirstlane((int32_t)(
                kbuf_lds + (uint32_t)((1 - par) * kLseBufBytes +
                                      (kRowsPerWave * wave + 7) * kRowBytes)));
            r.m0b = __builtin_amdgcn_readfirstlane((int32_t)(
                kbuf_lds + (uint32_t)(par * kLseBufBytes + kRowsPerWave * wave * kRowBytes)));
            r.sa = kRowBytes;
            r.sb = kRowBytes;
            return r;
        };
        // A tile's scores, exactly: the lanes that need it (`redo`) rebase
        // on the larger of the tile's maximum and B + log2 l (at least the
        // maximum of the scores summed so far, since one of their terms is
        // that maximum's: every old term then stays at most 1, and the base
        // within log2 of the count of the true maximum); the others add their
        // lazy sum.
        auto exact = [&](const f32x16_t& x, uint32_t slots, bool redo, float s, float& B,
                         float& l) {
            float mt = kNegInf;
#pragma unroll
            for (int e = 0; e < 16; ++e)
                mt = max_f32(mt, select_lanes(used_lanes(slots, e), x[e] * a.c_scale,
                                                      kNegInf));
            const float Bp = l > 0.0f ? B + __builtin_amdgcn_logf(l) : kNegInf;
            const float Bn = max_f32(Bp, mt);
            const float base = Bn == kNegInf ? 0.0f : Bn;
            // (an empty sum adds nothing whatever its base: B - base may be
            // large there, and 0 * 2^(B - base) would be 0 * inf)
            float sum = l > 0.0f ? l * __builtin_amdgcn_exp2f(B - base) : 0.0f;
#pragma unroll
            for (int e = 0; e < 16; ++e)
                sum += __builtin_amdgcn_exp2f(select_lanes(
                    used_lanes(slots, e), __builtin_fmaf(x[e], a.c_scale, -base), kNegInf));
            l = redo ? sum : l + s;
            B = redo ? Bn : B;
        };
        // Tile `tile` (parity P): `cc` holds its stream state, `oa` the gather
        // offsets of tile+1 (formed by tile-1); tile+2's offsets are formed in
        // step 18 into `ob`. The used entries of this tile's 32 keys per wave
        // are read in step 10 and collected in step 16. After the tile, the
        // previous tile's sums are added, or that tile is redone exactly
        // (rebased on its maximum) where a lane's scores lie more than
        // kLseLazy above its base (terms could overflow), or all of them more
        // than kLseLazy below it while its sum is still below 1 (terms could
        // underflow while nothing near the base has been seen; once the sum
        // is at least 1 such terms are below its rounding).
        auto body = [&](auto P, auto STEADY, auto MK, int tile, const Ctl& cc, int32_t oa,
                        int32_t& ob, const f32x16_t& prev0, const f32x16_t& prev1,
                        f32x16_t& acc0, f32x16_t& acc1) {
            constexpr int par = decltype(P)::value;
            constexpr bool steady = decltype(STEADY)::value != 0;
            constexpr bool mask = decltype(MK)::value != 0;
            const uint4* cur = kbuf[par] + (32 * kh + col) * kPitch + half;
            const uint4* nxt = kbuf[1 - par] + (32 * kh + col) * kPitch + half;
            int32_t kb = 0, jm = 0;
            uint32_t nslots = 0;
            float ym0, ym1, s0, s1;
            lse_tile<BF16, mask, !steady>(
                cur, nxt, ring, qa0, qa1, prev0, prev1, pslots, a.c_scale, B0, B1, ym0, ym1, s0,
                s1, i32x4_t{cc.da[0], cc.da[1], cc.da[2], cc.da[3]},
                i32x4_t{cc.db[0], cc.db[1], cc.db[2], cc.db[3]}, cc.m0a, cc.sa, oa, cc.m0b, cc.sb,
                ob, voff16,
                [&](int s) {  // second gap (each LDS read is used steps later)
                    // (the tile number is pinned in the step, so that no part
                    // of the step's work is hoisted into an earlier step)
                    int32_t tl = tile;
                    if (s == 10 || s == 12 || s == 16 || s == 18) pin_s(tl);
                    if (s == 10) {
                        // this tile's key 32 kh + c, for lanes c and c + 32
                        // (read six steps before its use: waiting for it
                        // also waits for every operand read issued before)
                        jm = DENSE ? tl * kLseKeys + 32 * kh + col
                                   : irow[(tl & 31) * kLseKeys + 32 * kh + col];
                    } else if (s == 12) {
                        kb = DENSE ? (tl + 2) * kLseKeys + my_slot
                                   : irow[((tl + 2) & 31) * kLseKeys + my_slot];
                    } else if (s == 16) {
                        // (two ballots of one comparison each: their masks
                        // are the comparisons' own results)
                        nslots = (uint32_t)(__builtin_amdgcn_ballot_w64(
                                                (tl * kLseKeys + 32 * kh + col) < ric.n) &
                                            __builtin_amdgcn_ballot_w64((uint32_t)jm <
                                                                        (uint32_t)ric.vis));
                    } else if (s == 18) {
                        // (a steady tile has tile+2; otherwise stream B takes
                        // the next row's Q, if there is one)
                        const bool has2 = steady || tl + 2 < ntiles;
                        ob = has2 ? row_off(ric, tl + 2, kb) : (more ? q_off(par) : 0);
                        pin_v(ob);  // (computed here, not where it is used)
                    }
                },
                acc0, acc1);
            auto redo_of = [&](float ym, float l) {
                return (ym > kLseLazy) | ((ym < -kLseLazy) & (ym > kNegInf) & (l < 1.0f));
            };
            const bool r0 = redo_of(ym0, l0), r1 = redo_of(ym1, l1);
            if (__builtin_amdgcn_ballot_w64(r0 | r1) == 0) {
                l0 += s0;
                l1 += s1;
            } else {
                exact(prev0, pslots, r0, s0, B0, l0);
                exact(prev1, pslots, r1, s1, B1, l1);
            }
            pslots = nslots;
        };
        // Pairs of tiles with two more after them run the steady body; the
        // last two or three tiles form their stream state at each boundary.
        // Either drops the masks from its epilogue when the previous tile's
        // entries are all used (every tile of a row but its last, unless the
        // index list holds invalid entries). Even tiles fill xa from xb, odd
        // tiles xb from xa.
        const Ctl cs0 = ctl_steady(Par<0>{}), cs1 = ctl_steady(Par<1>{});
        int32_t offb = 0;
        int tile = 0;
        for (; tile + 3 < ntiles; tile += 2) {
            if (pslots == ~0u)
                body(Par<0>{}, Par<1>{}, Par<0>{}, tile, cs0, offa, offb, xb0, xb1, xa0, xa1);
            else
                body(Par<0>{}, Par<1>{}, Par<1>{}, tile, cs0, offa, offb, xb0, xb1, xa0, xa1);
            if (pslots == ~0u)
                body(Par<1>{}, Par<1>{}, Par<0>{}, tile + 1, cs1, offb, offa, xa0, xa1, xb0, xb1);
            else
                body(Par<1>{}, Par<1>{}, Par<1>{}, tile + 1, cs1, offb, offa, xa0, xa1, xb0, xb1);
        }
        // the next row's index list into L2 (one dword per 128-byte line, 8 KB
        // in one load, into the dummy row) before the row end loads it
        if (!DENSE && more && wave == 0)
            dma_dword(raw_desc(a.idx + rln * a.K, (uint32_t)a.K * 4u), dummy_lds, 0, voff16 << 3);
        for (; tile < ntiles; tile += 2) {
            const Ctl c0 = ctl_of(Par<0>{}, tile);
            if (pslots == ~0u)
                body(Par<0>{}, Par<0>{}, Par<0>{}, tile, c0, offa, offb, xb0, xb1, xa0, xa1);
            else
                body(Par<0>{}, Par<0>{}, Par<1>{}, tile, c0, offa, offb, xb0, xb1, xa0, xa1);
            if (tile + 1 >= ntiles) break;
            const Ctl c1 = ctl_of(Par<1>{}, tile + 1);
            if (pslots == ~0u)
                body(Par<1>{}, Par<0>{}, Par<0>{}, tile + 1, c1, offb, offa, xa0, xa1, xb0, xb1);
            else
                body(Par<1>{}, Par<0>{}, Par<1>{}, tile + 1, c1, offb, offa, xa0, xa1, xb0, xb1);
        }
        // Every wave has passed the last tile's barrier: the rows of the next
        // row's Q that the last tiles did not load go out now.
        if (more) {
            if (ntiles >= 2) {
                stage_q_rows(rln, (ntiles - 1) & 1, 7, kRowsPerWave);
            } else {
                stage_q_rows(rln, 0, ntiles == 1 ? 7 : 0, kRowsPerWave);
                stage_q_rows(rln, 1, 0, kRowsPerWave);
            }
        }
        // the last tile, exactly
        if (ntiles > 0) {
            const f32x16_t& last0 = (ntiles & 1) ? xa0 : xb0;
            const f32x16_t& last1 = (ntiles & 1) ? xa1 : xb1;
            exact(last0, pslots, true, 0.0f, B0, l0);
            exact(last1, pslots, true, 0.0f, B1, l1);
        }
        // the two half-waves of each head (lower half first, the same bits
        // in both), then the two key halves through LDS (key half 0 first);
        // lse = ln 2 (M + log2 L), -inf without a used entry
        {
            float M[2], L[2];
            const float Bs[2] = {B0, B1}, ls[2] = {l0, l1};
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const uint32_t ub = __builtin_bit_cast(uint32_t, Bs[j]);
                const uint32_t ul = __builtin_bit_cast(uint32_t, ls[j]);
                const auto pb = __builtin_amdgcn_permlane32_swap(ub, ub, false, false);
                const auto pl = __builtin_amdgcn_permlane32_swap(ul, ul, false, false);
                lse_combine(__builtin_bit_cast(float, (uint32_t)pb[0]),
                            __builtin_bit_cast(float, (uint32_t)pl[0]),
                            __builtin_bit_cast(float, (uint32_t)pb[1]),
                            __builtin_bit_cast(float, (uint32_t)pl[1]), M[j], L[j]);
                if (half == 0) {
                    cmb[kh][64 * hg + 32 * j + col][0] = M[j];
                    cmb[kh][64 * hg + 32 * j + col][1] = L[j];
                }
            }
            lds_barrier();
            if (kh == 0 && half == 0) {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int h = 64 * hg + 32 * j + col;
                    float Mh, Lh;
                    lse_combine(M[j], L[j], cmb[1][h][0], cmb[1][h][1], Mh, Lh);
                    if (h < a.G)
                        a.out[rc * a.G + h] =
                            Lh > 0.0f ? (Mh + __builtin_amdgcn_logf(Lh)) * kLn2 : kNegInf;
                }
            }
        }

        // the next row: index list; once its Q has landed every wave reads
        // its heads back, then buffer 0 takes the next row's first tile
        if (more) {
            load_idx_row(rln, ib ^ 1);
            barrier_after_vmcnt(0);
            read_q();
            lds_barrier();
            offa = start_row(rin, ib ^ 1);
        }

        // the next row becomes current
        rc = rn;
        ric = rin;
        ib ^= 1;
    }
    // loads into LDS (the last tile's dummy loads) must land before the
    // workgroup's LDS is released
    waitcnt_vm_lgkm0<0>();
}

template <bool BF16, bool TND>
hipError_t launch_lse_wide_t(const KernelArgs& a, hipStream_t stream) {
    if (a.dense)
        hipLaunchKernelGGL((smla_lse_wide_kernel<BF16, TND, true>), dim3(a.num_wg), dim3(256), 0,
                           stream, a);
    else
        hipLaunchKernelGGL((smla_lse_wide_kernel<BF16, TND, false>), dim3(a.num_wg), dim3(256),
                           0, stream, a);
    return hipGetLastError();
}

template <bool BF16, bool TND>
hipError_t occupancy_lse_wide_t(int* out) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(
        out, reinterpret_cast<const void*>(&smla_lse_wide_kernel<BF16, TND, false>), 256, 0);
}

}  // namespace

hipError_t launch_lse_wide(const KernelArgs& a, bool bf16, bool tnd, hipStream_t stream) {
    SMLA_DISPATCH2(launch_lse_wide_t, a, stream);
}

hipError_t lse_wide_resident_per_cu(bool bf16, bool tnd, int* out) {
    SMLA_DISPATCH2(occupancy_lse_wide_t, out);
}

}  // namespace smla
