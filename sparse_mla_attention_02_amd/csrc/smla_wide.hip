// Pipelined kernel of the sparse Flash-MLA Softmax-L1Norm for gfx950: rows of
// 65..128 heads with at most 2048 indices (or dense rows).
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
static_assert(kVcap == kWideIndexCap, "the index list in LDS holds kVcap entries");
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
// offset is read into a scalar register one step before its load. With NT
// (the last two or three tiles of a row) stream B's loads carry the
// non-temporal hint: there they load the next row's Q, read once (in the
// first of three, the last tile's key rows), and Q then does not push the
// key rows, gathered again and again, out of L2.
//
// The workgroup barrier sits after the MFMAs of step kBar = 24: by then every
// wave has read its last operand of tile t (step 31's, read in step 23) and
// waited for its own loads of tile t+1 (the last issued in step 9), so after
// it the operand reads run on into tile t+1 (`nxt`) and the loads of tile
// t+2 may overwrite tile t's buffer. Tile boundaries then need no barrier and
// the MFMA stream does not drain between tiles. `mid(s)` is the caller's
// spread-out work, called at the end of step s.
constexpr int kBarStep = 24;
template <bool BF16, bool NT, typename Mid1, typename Mid2>
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
            dma_row_first<NT>(desc_b, (uint32_t)m0b, sob[0], voff, stepb);
        else if (s >= 26)
            dma_row_next<NT>(desc_b, sob[(s - 1) & 1], voff, stepb);
        mid2(s);
    }
    __builtin_amdgcn_sched_barrier(0);
    // this tile's last two elements are finished by the next tile's step 0
    pt = t;
    pex = ex;
    psum = sum;
}


// Lanes l and l + 32 of a wave hold partial sums of the same key (the two
// halves of the wave's 64 heads): their sum, the same bits in both lanes
// (lower half first), from one cross-lane swap.
__device__ __forceinline__ float half_pair_sum(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __builtin_bit_cast(float, (uint32_t)a[0]) + __builtin_bit_cast(float, (uint32_t)a[1]);
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
    // each key's sums over the heads of one head group (the two half-waves
    // added in registers first): last two tiles, and a row's last tile
    __shared__ float red[2][2][kWideKeys];
    __shared__ float redl[2][kWideKeys];
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
        // the sum of its two head groups' sums, stored to its column if
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
        // partial sums (finished in its step 0, added across the half-waves
        // in step 1, written in step 2) read after the barrier.
        auto body = [&](auto P, auto STEADY, int tile, const Ctl& cc, int32_t oa, int32_t& ob,
                        const f32x16_t& prev0, const f32x16_t& prev1, f32x16_t& acc0,
                        f32x16_t& acc1) {
            constexpr int par = decltype(P)::value;
            constexpr bool steady = decltype(STEADY)::value != 0;
            const uint4* cur = kbuf[par] + (32 * kh + col) * kPitch + half;
            const uint4* nxt = kbuf[1 - par] + (32 * kh + col) * kPitch + half;
            int32_t kb = 0, jv = -1, sdst = 0;
            float parts[2], hs = 0.0f, tot = 0.0f;
            wide_tile<BF16, !steady>(
                cur, nxt, ring, qa0, qa1, prev0, prev1, l2, a.c_scale, pt, pex, psum,
                i32x4_t{cc.da[0], cc.da[1], cc.da[2], cc.da[3]},
                i32x4_t{cc.db[0], cc.db[1], cc.db[2], cc.db[3]}, cc.m0a, cc.sa, oa, cc.m0b, cc.sb, ob, voff16,
                [&](int s) {  // first gap
                    if (s == 2) {
                        // tile-2's sums over this wave's 64 heads, added
                        // across the half-waves in step 1 (tiles 0 and 1: an
                        // unused slot)
                        red[par][hg][32 * kh + col] = hs;
                    } else if (s == kBarStep + 1) {
                        // tile-2's sums of both head groups, written in step
                        // 2 and visible after the barrier
                        parts[0] = red[par][0][slot];
                        parts[1] = red[par][1][slot];
                    } else if (s == kBarStep + 3) {
                        tot = parts[0] + parts[1];
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
                    if (s == 1) {
                        // tile-2's partial sums, finished in step 0: the two
                        // half-waves' halves of the head group, added
                        hs = half_pair_sum(psum);
                        pin(hs);
                    }
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
            red[ntiles & 1][hg][32 * kh + col] = half_pair_sum(psum);
        }
        const f32x16_t& prev0 = (ntiles & 1) ? xa0 : xb0;
        const f32x16_t& prev1 = (ntiles & 1) ? xa1 : xb1;
        // (the last tile's sums go to their own buffer: other waves may still
        // be reading red[(ntiles - 1) & 1] in the last tile)
        if (ntiles > 0)
            redl[hg][32 * kh + col] = half_pair_sum(head_sum(prev0, l2, a.c_scale) +
                                                    head_sum(prev1, l2 + 16, a.c_scale));

        // all MFMAs done, every operand read done and every gather of this
        // row landed (only loads to the dummy row may be in flight): K
        // buffers are free; partial sums visible
        lds_barrier();
        auto finish = [&](const float (*pr)[kWideKeys], int tile) {
            const float tot = pr[0][slot] + pr[1][slot];
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

}  // namespace

hipError_t launch_wide(const KernelArgs& a, bool bf16, bool tnd, hipStream_t stream) {
    SMLA_DISPATCH2(launch_wide_t, a, stream);
}

hipError_t wide_resident_per_cu(bool bf16, bool tnd, int* out) {
    SMLA_DISPATCH2(occupancy_wide_t, out);
}

}  // namespace smla
