// k_gemm.hip -- bf16 MFMA GEMM with a windowed beta-add epilogue.
//
// Second kernel of the large-token path: out[t][c0+j] = bf16(out[t][c0+j] +
// sum_k y[t][k] * W[c0+j][k]) -- the in-place `addmm_` on the narrowed weight
// rows and output columns of [PR50383 Key source snippets,
// `_shard_up_proj_tail`], which folds the shared-expert partial into the
// projection instead of running a separate add.
//
// Layout on gfx950:
//  * Workgroup tile BJ (W rows = output columns) x BT (tokens), WGJ x WGT
//    waves.  Each wave owns BJ/WGJ W rows and the 32-token blocks
//    WGT*mt + wt of the tile, as 32 x 32 tiles of v_mfma_f32_32x32x16_bf16
//    with W as the A operand and the latent as B.
//  * K advances 64 at a time through NS (2 or 4) LDS stages filled straight
//    from L2 by buffer_load_dwordx4 ... lds: while one stage is multiplied
//    the next NS-1 are in flight.  A stage row is 64 bf16 = one whole
//    128-byte line of the operand row, the unit the L2 hands out; half-line
//    slices (32 bf16) measured at half the fill rate.  Buffer resources are
//    clipped per workgroup: rows past the end of W's window or past T read as
//    zero with no branch.
//  * Each direct load writes 1 KB (8 rows) contiguously; the 16-byte chunk a
//    lane fetches is chosen so the rows land XOR-swizzled (key swz8).
//    Fragments of both operands are read from rows perm32(lane % 32) of each
//    32-row block, which with that key keeps every 8- and 16-lane group of a
//    ds_read_b128 on distinct banks (so the latent's token order inside a
//    block is permuted the same way; the epilogue follows it).
//  * Fragments are double-buffered in registers across the four 16-wide K
//    slices of a stage.  One barrier per stage, placed between the two MFMA
//    halves of the last slice: the next stage's first fragments are read right
//    after it while the second half runs.
//  * Epilogue: the `out` tile moves through LDS in two halves of token rows,
//    fetched into stage arrays as soon as the K loop frees them (with two
//    stages: half 0 during the last K stage, half 1 once the MFMAs are done,
//    while every wave forms its sums of half 0 -- the interleaved token
//    blocks give every wave rows in both halves).  Sums are rounded once in
//    place and the tile is written back row by row, so every store covers
//    whole contiguous row segments of `out`.  The residual form (RES) adds
//    the prefix chunks to the rounded rows on the way out and stores the
//    residual the same way ([PR50593 Key source snippets,
//    `forward_attn_residual`]: the layer's post-MLP prefix-sum update).
//  * Ragged edges are masked on store; nothing outside [c0, c0+n) x [0, T) is
//    written.
//  * Tiles are spread so that each of the 8 XCDs receives a contiguous range
//    of the (grouped) tile order, keeping W and latent blocks that are reused
//    by neighbouring tiles in the same XCD's L2.
//  * The largest tiles (256 x 256) run k_gemm_ring, the same GEMM with the
//    operand stream on a ring of five 32 KB slots (half a K stage each), so
//    that 96 KB of operands are in flight instead of 64 KB; its `out` tile
//    moves in quarters through the slots, and a last round that would leave
//    half of the CUs idle runs as 128 x 256 half tiles.
// Each output element's accumulation order depends on L only (K ascending in
// 16-wide MFMA slices), not on c0, n or the tile shape.
#include <type_traits>
#include <utility>

#include "lt_device.h"
#include "lt_gemm.h"
#include "lt_internal.h"
#include "lt_launch.h"

namespace lt {
namespace {

#ifndef LT_RING_OQ
#define LT_RING_OQ 3   // out quarters the 256 x 256 ring fetches into registers (0, 2 or 3)
#endif

// Argument order: everything the tile set-up needs comes first, within the
// 14 argument dwords that are preloaded into scalar registers at wave launch
// (the library is built with kernel-argument preloading); the residual
// pointers, read only by the epilogue, come last.
template <int BJ, int BT, int WGJ, int WGT, int NS, int GROUP_J, bool KTAIL, bool EPI_LDS, bool RES>
__global__ __launch_bounds__(64 * WGJ * WGT) void k_gemm(const u16 *__restrict__ Y, int ntj, int ntt,
                                                         int64_t T, int L, int n,
                                                         const u16 *__restrict__ Wn,
                                                         u16 *__restrict__ outn, int64_t ld_out,
                                                         const u16 *prefn, int64_t ld_pre,
                                                         u16 *resn, int64_t ld_res)
{
    constexpr int NW = WGJ * WGT;               // waves, in a WGJ x WGT grid
    constexpr int NT = 64 * NW;                 // threads
    constexpr int MJ = BJ / WGJ / 32, MT = BT / WGT / 32;   // 32x32 tiles per wave
    constexpr int LR = 8 * NW;                  // stage rows one direct load fills
    constexpr int LA = BJ / LR, LB = BT / LR;   // direct loads per thread per stage
    constexpr int STAGE_A = BJ * ROWB, STAGE = (BJ + BT) * ROWB;
    constexpr int NFR = MJ + MT, NMF = MJ * MT;
    static_assert(MJ >= 1 && MT >= 1 && LA * LR == BJ && LB * LR == BT, "tile shape");
    static_assert(WGT % 2 == 0, "token halves belong to whole rows of waves");
    static_assert(NS >= 2 && NS <= 4, "two to four stages");
    // One __shared__ array per stage, always indexed by a compile-time stage
    // number, so the compiler can tell which array a direct load writes.
    __shared__ __attribute__((aligned(1024))) char st0[STAGE];
    __shared__ __attribute__((aligned(1024))) char st1[STAGE];
    __shared__ __attribute__((aligned(1024))) char st2[NS > 2 ? STAGE : 16];
    __shared__ __attribute__((aligned(1024))) char st3[NS > 3 ? STAGE : 16];
    auto stage = [&](auto S) __attribute__((always_inline)) -> char * {
        if constexpr (decltype(S)::value == 0) return st0;
        else if constexpr (decltype(S)::value == 1) return st1;
        else if constexpr (decltype(S)::value == 2) return st2;
        else return st3;
    };

    // ---- tile coordinates: XCD-contiguous ranges, then GROUP_J-wide groups
    const int G = ntj * ntt;
    const int nb = xcd_contiguous(blockIdx.x, G);
    const int gsize = GROUP_J * ntt;
    const int gid = nb / gsize;
    const int first_j = gid * GROUP_J;
    const int gj = min(ntj - first_j, GROUP_J);
    const int within = nb - gid * gsize;
    const int tj = first_j + within % gj;
    const int tt = within / gj;
    const int j0 = tj * BJ;
    const int64_t t0 = (int64_t)tt * BT;

    const int tid = threadIdx.x;
    const int l = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wj = w / WGT, wt = w % WGT;
    const int nchunk = L >> 3;
    // K stages, padded to a multiple of NS (padded chunks read zeros), so the
    // array of every step is known at compile time.
    const int nk = ((L + NS * BK - 1) / (NS * BK)) * NS;
    const uint32_t row_bytes = (uint32_t)L * 2u;

    // ---- buffer resources clipped to this tile's rows: overhanging rows read 0
    const int rows_a = min(BJ, n - j0);
    const int rows_b = (int)min((int64_t)BT, T - t0);
    const __amdgpu_buffer_rsrc_t ra = lt_rsrc(Wn + (int64_t)j0 * L, (uint32_t)rows_a * row_bytes);
    const __amdgpu_buffer_rsrc_t rb = lt_rsrc(Y + t0 * L, (uint32_t)rows_b * row_bytes);

    // ---- direct loads: lane i of wave w, load q -> stage row LR*q + 8w + i/8,
    // LDS slot i%8, global chunk (slot ^ swz8(row)).
    const int lrow = 8 * w + (l >> 3);
    const int lslot = l & 7;
    uint32_t offa[LA], offb[LB];
    int cha[LA], chb[LB];
#pragma unroll
    for (int q = 0; q < LA; ++q) {
        const int row = LR * q + lrow;
        cha[q] = lslot ^ swz8(row);
        offa[q] = (uint32_t)row * row_bytes + (uint32_t)cha[q] * 16u;
    }
#pragma unroll
    for (int q = 0; q < LB; ++q) {
        const int row = LR * q + lrow;
        chb[q] = lslot ^ swz8(row);
        offb[q] = (uint32_t)row * row_bytes + (uint32_t)chb[q] * 16u;
    }
    auto issue = [&](auto S, int s) __attribute__((always_inline)) {   // K stage s -> array S
        char *sa = stage(S);
        char *sb = sa + STAGE_A;
        const uint32_t kbyte = (uint32_t)s * ROWB;
#pragma unroll
        for (int q = 0; q < LA; ++q) {
            uint32_t vo = offa[q] + kbyte;
            if (KTAIL && s * CPR + cha[q] >= nchunk) vo = OOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void *)(sa + (LR * q + 8 * w) * ROWB),
                                                     16, vo, 0, 0, 0);
        }
#pragma unroll
        for (int q = 0; q < LB; ++q) {
            uint32_t vo = offb[q] + kbyte;
            if (KTAIL && s * CPR + chb[q] >= nchunk) vo = OOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void *)(sb + (LR * q + 8 * w) * ROWB),
                                                     16, vo, 0, 0, 0);
        }
    };

    // ---- fragment reads: lane l reads row perm32(l % 32) of each 32-row
    // block, chunk 2*ks + l/32 of the stage row for K slice ks.
    const int hsel = l >> 5;
    const int arow = wj * (BJ / WGJ) + perm32(l & 31);
    // A wave's token rows are the 32-row blocks WGT*mt + wt of the tile (not
    // one contiguous range), so every wave owns rows in both halves of the
    // out tile and all waves share the work of each epilogue half.
    constexpr int BSTR = 32 * WGT;                       // tile rows between a wave's blocks
    const int brow = 32 * wt + perm32(l & 31);           // token of this lane's D column, block 0
    const int abase = arow * ROWB, bbase = STAGE_A + brow * ROWB;
    const int akey = swz8(arow), bkey = swz8(brow);      // perm32 keeps r % 32 -> same key per block
    auto read_frags = [&](auto S, int ks, bf16x8_t (&fa)[MJ], bf16x8_t (&fb)[MT])
        __attribute__((always_inline)) {
        const char *base = stage(S);
        const int ca = ((2 * ks + hsel) ^ akey) << 4, cb = ((2 * ks + hsel) ^ bkey) << 4;
#pragma unroll
        for (int mj = 0; mj < MJ; ++mj)
            fa[mj] = *reinterpret_cast<const bf16x8_t *>(base + abase + mj * 32 * ROWB + ca);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            fb[mt] = *reinterpret_cast<const bf16x8_t *>(base + bbase + mt * BSTR * ROWB + cb);
    };

    f32x16_t acc[MJ][MT];
#pragma unroll
    for (int mj = 0; mj < MJ; ++mj)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mj][mt] = f32x16_t{};
    // MFMAs [lo, hi) of the MJ x MT grid for one K slice
    auto mfma_range = [&](const bf16x8_t (&fa)[MJ], const bf16x8_t (&fb)[MT], int lo, int hi)
        __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NMF; ++i) {
            if (i >= lo && i < hi) {
                const int mj = i / MT, mt = i % MT;
                acc[mj][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mj], fb[mt], acc[mj][mt],
                                                                      0, 0, 0);
            }
        }
    };

    // ---- the out tile moves through LDS in two halves of BT/2 token rows
    // (row-major, 16-byte chunks XOR-swizzled by row).
    constexpr int CPRE = BJ / 8;               // 16-byte chunks per tile row
    constexpr int RPH = BT / 2;                // tile rows per half
    constexpr int HCH = RPH * CPRE;            // chunks per half
    constexpr int HLD = HCH / NT;              // direct loads per thread per half
    static_assert(!EPI_LDS || HCH % NT == 0, "a half is whole workgroup loads");
    static_assert(RPH * BJ * 2 <= STAGE, "half of the out tile must fit a stage");
    const __amdgpu_buffer_rsrc_t rc = lt_rsrc(
        outn + t0 * ld_out, (uint32_t)(((int64_t)max(rows_b - 1, 0) * ld_out + n) * 2));
    auto load_c_half = [&](char *dst, int h) __attribute__((always_inline)) {
#pragma unroll
        for (int it = 0; it < HLD; ++it) {
            const int idx0 = it * NT + 64 * w;      // wave-uniform
            const int idx = idx0 + l;
            const int r = h * RPH + idx / CPRE;
            const int c = (idx % CPRE) ^ (r & (CPRE - 1));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rc, (lds_void *)(dst + idx0 * 16), 16,
                (uint32_t)(((int64_t)r * ld_out + j0 + 8 * c) * 2), 0, 0, 0);
        }
    };

    // One K stage on array S.  On entry fa/fb[0] hold slice 0's fragments.
    // First the array freed by the previous stage, (S + NS - 1) % NS, receives
    // K stage kb + NS - 1 (ACT < 0), half ACT of the out tile (0, 1), or
    // nothing (2).  Slices alternate between the two fragment buffers; the
    // barrier sits inside the last slice, after waiting until at most WAIT
    // loads of this thread are in flight (the next stage has landed), and is
    // followed by the next stage's slice-0 reads.  The last stage has none.
    bf16x8_t fa[2][MJ], fb[2][MT];
    // scheduling hint: alternate the ND fragment reads with the NM MFMAs
    // just emitted, then the rest of whichever is longer
    auto interleave = [&](auto ND, auto NM) __attribute__((always_inline)) {
        constexpr int nd = decltype(ND)::value, nm = decltype(NM)::value;
        constexpr int np = nd < nm ? nd : nm;
#pragma unroll
        for (int i = 0; i < np; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one DS read
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        }
        if constexpr (nm > np) __builtin_amdgcn_sched_group_barrier(0x008, nm - np, 0);
        if constexpr (nd > np) __builtin_amdgcn_sched_group_barrier(0x100, nd - np, 0);
    };
    auto kstage = [&](auto S, auto ACT, auto WAIT, auto LAST, int kb) __attribute__((always_inline)) {
        constexpr int s = decltype(S)::value;
        constexpr int act = decltype(ACT)::value;
        constexpr bool last = decltype(LAST)::value;
        using SN = I<(s + 1) % NS>;
        using SP = I<(s + NS - 1) % NS>;
        if constexpr (act < 0) issue(SP{}, kb + NS - 1);
        else if constexpr (act < 2 && EPI_LDS) load_c_half(stage(SP{}), act);
        // keep the loads at the top of the stage: left to itself the scheduler
        // sinks them next to the wait at the barrier, serialising them with
        // the MFMAs
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < KSL - 1; ++ks) {
            read_frags(S, ks + 1, fa[(ks + 1) & 1], fb[(ks + 1) & 1]);
            mfma_range(fa[ks & 1], fb[ks & 1], 0, NMF);
            interleave(I<NFR>{}, I<NMF>{});
        }
        constexpr int KL = (KSL - 1) & 1;
        constexpr int HALF = NMF / 2;
        mfma_range(fa[KL], fb[KL], 0, HALF);
        if constexpr (!last) {
            __builtin_amdgcn_s_waitcnt(lt_vm_lgkm0(decltype(WAIT)::value));
            lt_lds_barrier();
            read_frags(SN{}, 0, fa[0], fb[0]);
        }
        mfma_range(fa[KL], fb[KL], HALF, NMF);
        if constexpr (!last) interleave(I<NFR>{}, I<NMF - HALF>{});
    };
    using F = std::false_type;
    using Tr = std::true_type;
    constexpr int LPS = LA + LB;                 // stage loads per thread
    constexpr int HQ = EPI_LDS ? HLD : 0;        // out-half loads per thread

    // ---- prologue: K stages 0 .. NS-2 in flight, wait for stage 0
    issue(I<0>{}, 0);
    if constexpr (NS > 2) issue(I<1>{}, 1);
    if constexpr (NS > 3) issue(I<2>{}, 2);
    __builtin_amdgcn_s_waitcnt(lt_vm_lgkm0((NS - 2) * LPS));
    lt_lds_barrier();
    read_frags(I<0>{}, 0, fa[0], fb[0]);

    constexpr int WM = (NS - 2) * LPS;           // steady state: NS-2 stages stay in flight
    for (int kb = 0; kb < nk - NS; kb += NS) {
        kstage(I<0>{}, I<-1>{}, I<WM>{}, F{}, kb);
        kstage(I<1>{}, I<-1>{}, I<WM>{}, F{}, kb + 1);
        if constexpr (NS > 2) kstage(I<2>{}, I<-1>{}, I<WM>{}, F{}, kb + 2);
        if constexpr (NS > 3) kstage(I<3>{}, I<-1>{}, I<WM>{}, F{}, kb + 3);
    }
    // last trip: the first step issues the last K stage; with three or more
    // stages the next two steps fetch the out-tile halves into arrays 0 and 1,
    // with two the last step fetches half 0 into array 0
    {
        const int kb = nk - NS;
        if constexpr (NS == 2) {
            kstage(I<0>{}, I<-1>{}, I<0>{}, F{}, kb);
            kstage(I<1>{}, I<0>{}, I<0>{}, Tr{}, kb + 1);
        } else if constexpr (NS == 3) {
            kstage(I<0>{}, I<-1>{}, I<LPS>{}, F{}, kb);
            kstage(I<1>{}, I<0>{}, I<HQ>{}, F{}, kb + 1);
            kstage(I<2>{}, I<1>{}, I<0>{}, Tr{}, kb + 2);
        } else {
            kstage(I<0>{}, I<-1>{}, I<2 * LPS>{}, F{}, kb);
            kstage(I<1>{}, I<0>{}, I<LPS + HQ>{}, F{}, kb + 1);
            kstage(I<2>{}, I<1>{}, I<2 * HQ>{}, F{}, kb + 2);
            kstage(I<3>{}, I<2>{}, I<0>{}, Tr{}, kb + 3);
        }
    }

    if constexpr (EPI_LDS) {
        // half 0 goes to st0 and half 1 to st1 (with two stages half 1 is
        // fetched below, once st1 is free; with more it is already in flight)
        // sums in place for the rows of half hh this wave owns
        const bool edge = j0 + BJ > n;            // the window ends inside this tile
        auto sums = [&](char *half, int hh) __attribute__((always_inline)) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                if ((BSTR * mt + 32 * wt) / RPH != hh) continue;   // block in the other half
                const int r = brow + BSTR * mt;           // tile row (token)
                const int rh = r - hh * RPH;              // row within the half
#pragma unroll
                for (int mj = 0; mj < MJ; ++mj) {
#pragma unroll
                    for (int hf = 0; hf < 2; ++hf) {
                        const int c = (wj * (BJ / WGJ) + 32 * mj + 16 * hf + 8 * hsel) >> 3;
                        const f32x16_t &a = acc[mj][mt];
                        u32x4_t *ptr = reinterpret_cast<u32x4_t *>(
                            half + rh * (BJ * 2) + ((c ^ (r & (CPRE - 1))) << 4));
                        u32x4_t ov = *ptr;
                        // The buffer range check is per dword: a chunk that
                        // straddles the window end can come back with its last
                        // valid column zeroed.  Re-read its valid columns.
                        const int jc = j0 + 8 * c;
                        if (edge && jc < n && jc + 8 > n && t0 + r < T) {
                            const u16 *src = outn + (t0 + r) * ld_out + jc;
#pragma unroll
                            for (int e = 0; e < 8; e += 2) {
                                const uint32_t lo = (jc + e < n) ? src[e] : 0u;
                                const uint32_t hi = (jc + e + 1 < n) ? src[e + 1] : 0u;
                                ov[e >> 1] = lo | (hi << 16);
                            }
                        }
                        u32x4_t nv;
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            nv[e] = lt_pack2(lt_bf_lo(ov[e]) + a[8 * hf + 2 * e],
                                             lt_bf_hi(ov[e]) + a[8 * hf + 2 * e + 1]);
                        *ptr = nv;
                    }
                }
            }
        };
        // write back rows [r_lo, r_lo + nrows) of half hh, spread over nwv waves (wave index wi)
        constexpr int LPR = CPRE;                    // lanes per tile row
        constexpr int RPI = 64 / LPR;                // rows per store instruction
        static_assert(CPRE <= 64, "row wider than a wave");
        // residual: prefix and resid tiles, addressed like `out`
        const __amdgpu_buffer_rsrc_t rp = lt_rsrc(
            prefn + t0 * ld_pre, (uint32_t)(((int64_t)max(rows_b - 1, 0) * ld_pre + n) * 2));
        const __amdgpu_buffer_rsrc_t rr = lt_rsrc(
            resn + t0 * ld_res, (uint32_t)(((int64_t)max(rows_b - 1, 0) * ld_res + n) * 2));
        // rows [wi*per, (wi+1)*per) of half hh, per = RPH / NWV, go out in
        // per / RPI store rounds; the residual form adds the prefix chunks of
        // the same rounds, fetched beforehand by load_prefix
        constexpr int IT = RPH / NW / RPI;          // store rounds per wave and half
        auto load_prefix = [&](int hh, int wi, auto NWV, auto &pv) __attribute__((always_inline)) {
            constexpr int per = RPH / decltype(NWV)::value;
            constexpr int ITER = per / RPI;
#pragma unroll
            for (int i = 0; i < ITER; ++i) {
                const int r = hh * RPH + wi * per + i * RPI + l / LPR;
                const int j = j0 + 8 * (l % LPR);
                pv[i] = lt_buf_load16(rp, j + 8 <= n ? (uint32_t)(((int64_t)r * ld_pre + j) * 2)
                                                     : LT_OOB);
            }
        };
        auto write_back = [&](const char *half, int hh, int wi, auto NWV, const auto &pv)
            __attribute__((always_inline)) {
            constexpr int per = RPH / decltype(NWV)::value;
            constexpr int ITER = per / RPI;
#pragma unroll
            for (int i = 0; i < ITER; ++i) {
                const int rh = wi * per + i * RPI + l / LPR;
                const int r = hh * RPH + rh;
                const int c = l % LPR;
                const int64_t t = t0 + r;
                const int j = j0 + 8 * c;
                if (t < T && j < n) {
                    const u32x4_t v = *reinterpret_cast<const u32x4_t *>(
                        half + rh * (BJ * 2) + ((c ^ (r & (CPRE - 1))) << 4));
                    if (j + 8 <= n) {
                        __builtin_amdgcn_raw_buffer_store_b128(
                            v, rc, (uint32_t)(((int64_t)r * ld_out + j) * 2), 0, 0);
                        if constexpr (RES) {
                            u32x4_t rv;
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                rv[e] = lt_pack2(lt_bf_lo(pv[i][e]) + lt_bf_lo(v[e]),
                                                 lt_bf_hi(pv[i][e]) + lt_bf_hi(v[e]));
                            __builtin_amdgcn_raw_buffer_store_b128(
                                rv, rr, (uint32_t)(((int64_t)r * ld_res + j) * 2), 0, 0);
                        }
                    } else {
                        u16 *o = outn + t * ld_out + j;
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            if (j + e < n) {
                                const u16 onew = (u16)((v[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
                                o[e] = onew;
                                if constexpr (RES) {
                                    const float rs = lt_bf_lo((uint32_t)prefn[t * ld_pre + j + e]) +
                                                     lt_bf_lo((uint32_t)onew);
                                    resn[t * ld_res + j + e] = (u16)(lt_pack2(rs, 0.f) & 0xFFFFu);
                                }
                            }
                        }
                    }
                }
            }
        };
        static_assert((RPH / NW) % RPI == 0, "whole store rounds");
        static_assert(2 * IT < 63, "prefix loads fit the vmcnt field");
        // Every wave sums its blocks of half 0, then (half 1 landed) writes
        // half 0 back and sums its blocks of half 1, then writes half 1 back.
        // The residual form's prefix chunks for both halves are in flight
        // from the start; they were issued after half 0's loads, so waiting
        // for half 0 leaves them flying.
        u32x4_t pv0[RES ? IT : 1], pv1[RES ? IT : 1];
        if constexpr (RES) {
            load_prefix(0, w, I<NW>{}, pv0);
            load_prefix(1, w, I<NW>{}, pv1);
        }
        if constexpr (NS == 2) {
            // half 1 is fetched once every wave is past its last reads of st1
            __builtin_amdgcn_s_waitcnt(lt_vm_lgkm0(RES ? 2 * IT : 0));
            lt_lds_barrier();
            load_c_half(st1, 1);
        } else {
            __builtin_amdgcn_s_waitcnt(lt_vm_lgkm0(HLD + (RES ? 2 * IT : 0)));
            lt_lds_barrier();
        }
        sums(st0, 0);
        __builtin_amdgcn_s_waitcnt(lt_vm_lgkm0(0));   // half 1 (and the prefix chunks)
        lt_lds_barrier();
        write_back(st0, 0, w, I<NW>{}, pv0);
        sums(st1, 1);
        __builtin_amdgcn_s_waitcnt(lt_vm_lgkm0(63));  // LDS only: half-0 stores may fly
        lt_lds_barrier();
        write_back(st1, 1, w, I<NW>{}, pv1);
    } else {
        // ---- plain epilogue (unaligned `out`): element-wise read-add-round-write
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int64_t t = t0 + brow + BSTR * mt;
            if (t >= T) continue;
            u16 *orow = outn + t * ld_out;
#pragma unroll
            for (int mj = 0; mj < MJ; ++mj) {
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const int j = j0 + wj * (BJ / WGJ) + 32 * mj + 16 * hf + 8 * hsel;
                    const f32x16_t &a = acc[mj][mt];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        if (j + e < n) {
                            const float v = lt_bf_lo((uint32_t)orow[j + e]) + a[8 * hf + e];
                            const u16 onew = (u16)(lt_pack2(v, 0.f) & 0xFFFFu);
                            orow[j + e] = onew;
                            if constexpr (RES) {
                                const float rs = lt_bf_lo((uint32_t)prefn[t * ld_pre + j + e]) +
                                                 lt_bf_lo((uint32_t)onew);
                                resn[t * ld_res + j + e] = (u16)(lt_pack2(rs, 0.f) & 0xFFFFu);
                            }
                        }
                    }
                }
            }
        }
    }
}

// Tiles of BJ W rows x 256 tokens with the operand stream on a ring of five
// LDS slots.  A K stage is two half-stages of 64 bf16 per row: A (BJ W rows,
// 32 KB at BJ = 256) and B (256 tokens, 32 KB).  Half-stage h (stage h / 2)
// lives in slot h % 5, so while stage k is multiplied out of two slots the
// other three hold stage k + 1 and A of stage k + 2: 96 KB of operands in
// flight per workgroup against the 64 KB of two whole 64 KB stages, in the
// same 160 KB of LDS.  Each stage fetches B of stage k + 1 and A of stage
// k + 2 into the slots stage k - 1 left.  The `out` tile moves through four
// slots in quarters of 64 token rows: quarter 0 is fetched during stage
// nk - 2 (in place of A of stage nk), quarters 1 and 2 during the last stage
// and quarter 3 once it is done.  NKR = nk % 5 fixes, at compile time, the
// slot every stage and quarter uses.  The `out` tile is read and written
// once, so those loads and stores are marked non-temporal (same box,
// alternating runs: T = 8192 about 4-8 % faster).  Same tile order,
// swizzles, K order and epilogue arithmetic as k_gemm, so the results are
// bit-identical to it.
//
// The five slots live at namespace scope so that the full-width (BJ = 256)
// and half-width (BJ = 128) tile bodies of one kernel share them.
constexpr int RING_BT = 256;                  // tokens per ring tile
constexpr int RING_SLOT = RING_BT * ROWB;     // bytes of one slot (a 256-row half-stage)
constexpr int RING_CUS = 256;                 // compute units of the chip
__shared__ __attribute__((aligned(1024))) char ring_sl0[RING_SLOT];
__shared__ __attribute__((aligned(1024))) char ring_sl1[RING_SLOT];
__shared__ __attribute__((aligned(1024))) char ring_sl2[RING_SLOT];
__shared__ __attribute__((aligned(1024))) char ring_sl3[RING_SLOT];
__shared__ __attribute__((aligned(1024))) char ring_sl4[RING_SLOT];

// Full 256 x 256 tiles of a ring launch over G of them.  When the last round
// would leave at least half of the compute units idle (0 < G mod 256 <= 128,
// G > 256), its tiles are handed out as two 128 x 256 halves each, so that
// every CU takes part in that round and each does half the work: the
// workgroups of the halves come last in the grid and start as the CUs finish
// their last full tile.  The halves keep the K order of every output, so the
// results are the same bit for bit.
__host__ __device__ constexpr int ring_full_tiles(int G)
{
    return (G > RING_CUS && G % RING_CUS != 0 && G % RING_CUS <= RING_CUS / 2)
               ? G - G % RING_CUS
               : G;
}

// One BJ x 256 tile (W rows j0.., tokens t0..) of the slot-ring GEMM.
template <int BJ, int WGJ, int WGT, int NKR, bool KTAIL, bool RES, int OQ>
__device__ __forceinline__ void ring_tile(const u16 *__restrict__ Y, int64_t T, int L, int n,
                                          const u16 *__restrict__ Wn, u16 *__restrict__ outn,
                                          int64_t ld_out, const u16 *prefn, int64_t ld_pre,
                                          u16 *resn, int64_t ld_res, int j0, int64_t t0)
{
    constexpr int BT = RING_BT;
    constexpr int NW = WGJ * WGT;
    constexpr int NT = 64 * NW;
    constexpr int MJ = BJ / WGJ / 32, MT = BT / WGT / 32;
    constexpr int LR = 8 * NW;
    constexpr int LA = BJ / LR;                 // direct loads per thread per W half-stage
    constexpr int LB = BT / LR;                 // and per token half-stage
    constexpr int SLOT = RING_SLOT;
    constexpr int NFR = MJ + MT, NMF = MJ * MT;
    static_assert(MJ >= 1 && MT == 4 && LA * LR == BJ && LB * LR == BT && BJ <= BT, "tile shape");
    auto slot = [&](auto S) __attribute__((always_inline)) -> char * {
        constexpr int s = decltype(S)::value;
        if constexpr (s == 0) return ring_sl0;
        else if constexpr (s == 1) return ring_sl1;
        else if constexpr (s == 2) return ring_sl2;
        else if constexpr (s == 3) return ring_sl3;
        else return ring_sl4;
    };

    const int tid = threadIdx.x;
    const int l = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wj = w / WGT, wt = w % WGT;
    const int nchunk = L >> 3;
    const int nk = (L + BK - 1) / BK;           // K stages, no padding (at least 3)
    const uint32_t row_bytes = (uint32_t)L * 2u;

    const int rows_a = min(BJ, n - j0);
    const int rows_b = (int)min((int64_t)BT, T - t0);
    const __amdgpu_buffer_rsrc_t ra = lt_rsrc(Wn + (int64_t)j0 * L, (uint32_t)rows_a * row_bytes);
    const __amdgpu_buffer_rsrc_t rb = lt_rsrc(Y + t0 * L, (uint32_t)rows_b * row_bytes);

    // direct loads as in k_gemm (both operands have row stride L, so the W
    // half-stage uses the first LA of the token half-stage's offsets); the K
    // offset goes in the scalar offset, which keeps the unrolled stages from
    // holding one address register per stage
    const int lrow = 8 * w + (l >> 3);
    const int lslot = l & 7;
    uint32_t off[LB];
    int ch[LB];
#pragma unroll
    for (int q = 0; q < LB; ++q) {
        const int row = LR * q + lrow;
        ch[q] = lslot ^ swz8(row);
        off[q] = (uint32_t)row * row_bytes + (uint32_t)ch[q] * 16u;
    }
    auto issue = [&](const __amdgpu_buffer_rsrc_t &rs, auto S, auto NQ, int s) __attribute__((always_inline)) {
        char *dst = slot(S);
        const uint32_t kbyte = (uint32_t)s * ROWB;
#pragma unroll
        for (int q = 0; q < decltype(NQ)::value; ++q) {
            uint32_t vo = off[q];
            if (KTAIL && s * CPR + ch[q] >= nchunk) vo = OOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(dst + (LR * q + 8 * w) * ROWB),
                                                     16, vo, (int)kbyte, 0, 0);
        }
    };
    auto issueA = [&](auto S, int s) __attribute__((always_inline)) { issue(ra, S, I<LA>{}, s); };
    auto issueB = [&](auto S, int s) __attribute__((always_inline)) { issue(rb, S, I<LB>{}, s); };

    const int hsel = l >> 5;
    const int arow = wj * (BJ / WGJ) + perm32(l & 31);
    constexpr int BSTR = 32 * WGT;
    const int brow = 32 * wt + perm32(l & 31);
    const int abase = arow * ROWB, bbase = brow * ROWB;
    const int akey = swz8(arow), bkey = swz8(brow);
    // slice ks of a row sits at chunk (2 ks + hsel) ^ key = (hsel ^ key) ^ 2 ks,
    // so its byte offset is the slice-0 offset XOR 32 ks (rows are 128-byte
    // aligned).  The per-lane offsets pass through an empty asm at every use,
    // so the compiler recomputes the few address operations instead of
    // keeping one register per slot and slice alive across the loop.
    const int xa0 = abase + ((hsel ^ akey) << 4), xb0 = bbase + ((hsel ^ bkey) << 4);
    auto read_frags = [&](auto SA, auto SB, int ks, bf16x8_t (&fa)[MJ], bf16x8_t (&fb)[MT])
        __attribute__((always_inline)) {
        int xa = xa0, xb = xb0;
        asm volatile("" : "+v"(xa), "+v"(xb));
        const char *ba = slot(SA) + (xa ^ (32 * ks));
        const char *bb = slot(SB) + (xb ^ (32 * ks));
#pragma unroll
        for (int mj = 0; mj < MJ; ++mj)
            fa[mj] = *reinterpret_cast<const bf16x8_t *>(ba + mj * 32 * ROWB);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            fb[mt] = *reinterpret_cast<const bf16x8_t *>(bb + mt * BSTR * ROWB);
    };

    f32x16_t acc[MJ][MT];
#pragma unroll
    for (int mj = 0; mj < MJ; ++mj)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mj][mt] = f32x16_t{};
    auto mfma_range = [&](const bf16x8_t (&fa)[MJ], const bf16x8_t (&fb)[MT], int lo, int hi)
        __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NMF; ++i) {
            if (i >= lo && i < hi) {
                const int mj = i / MT, mt = i % MT;
                acc[mj][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mj], fb[mt], acc[mj][mt],
                                                                      0, 0, 0);
            }
        }
    };

    // out tile in quarters of BT/4 token rows (BJ columns), one slot each
    constexpr int CPRE = BJ / 8;
    constexpr int RPQ = BT / 4;
    constexpr int QCH = RPQ * CPRE;
    constexpr int QLD = QCH / NT;
    static_assert(QCH % NT == 0 && RPQ * BJ * 2 <= SLOT, "quarter fits a slot");
    const __amdgpu_buffer_rsrc_t rc = lt_rsrc(
        outn + t0 * ld_out, (uint32_t)(((int64_t)max(rows_b - 1, 0) * ld_out + n) * 2));
    auto load_c_q = [&](char *dst, int q) __attribute__((always_inline)) {
#pragma unroll
        for (int it = 0; it < QLD; ++it) {
            const int idx0 = it * NT + 64 * w;
            const int idx = idx0 + l;
            const int r = q * RPQ + idx / CPRE;
            const int c = (idx % CPRE) ^ (r & (CPRE - 1));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rc, (lds_void *)(dst + idx0 * 16), 16,
                (uint32_t)(((int64_t)r * ld_out + j0 + 8 * c) * 2), 0, 0, LT_NT);
        }
    };

    // OQ > 0: quarters 1..OQ of the out tile are fetched into registers during
    // the K loop, at stages nk - 8, nk - 6 and nk - 4 (one quarter per stage,
    // QLD 16-byte loads per thread, in the order the direct loads above would
    // write them), and written into their slots with ds_write at the end, so
    // that the epilogue does not wait on them.  Those stages sit in a tail of
    // the loop unrolled at compile time, so each load writes fixed registers.
    static_assert(OQ == 0 || OQ == 2 || OQ == 3, "out quarters in registers");
    u32x4_t oq1[QLD], oq2[QLD], oq3[QLD];
    auto load_c_q_regs = [&](int q, u32x4_t (&rg)[QLD]) __attribute__((always_inline)) {
#pragma unroll
        for (int it = 0; it < QLD; ++it) {
            const int idx = it * NT + 64 * w + l;
            const int r = q * RPQ + idx / CPRE;
            const int c = (idx % CPRE) ^ (r & (CPRE - 1));
            rg[it] = __builtin_bit_cast(
                u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                             rc, (uint32_t)(((int64_t)r * ld_out + j0 + 8 * c) * 2), 0, LT_NT));
        }
    };
    auto store_c_q = [&](char *dst, const u32x4_t (&rg)[QLD]) __attribute__((always_inline)) {
#pragma unroll
        for (int it = 0; it < QLD; ++it)
            *reinterpret_cast<u32x4_t *>(dst + (it * NT + 64 * w + l) * 16) = rg[it];
    };

    bf16x8_t fa[2][MJ], fb[2][MT];
    auto interleave = [&](auto ND, auto NM) __attribute__((always_inline)) {
        constexpr int nd = decltype(ND)::value, nm = decltype(NM)::value;
        constexpr int np = nd < nm ? nd : nm;
#pragma unroll
        for (int i = 0; i < np; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
        if constexpr (nm > np) __builtin_amdgcn_sched_group_barrier(0x008, nm - np, 0);
        if constexpr (nd > np) __builtin_amdgcn_sched_group_barrier(0x100, nd - np, 0);
    };
    // K stage k at ring phase P = k % 5: operand A in slot 2P, B in 2P+1 (mod 5).
    // MODE 0: fetch B of stage k+1 and A of stage k+2 into the slots stage k-1
    // freed; 1 (stage nk-2): B of the last stage and out quarter 0; 2 (last):
    // out quarters 1 and 2.
    auto kst = [&](auto P, auto MODE, int k, auto QN) __attribute__((always_inline)) {
        constexpr int p = decltype(P)::value, mode = decltype(MODE)::value;
        constexpr int qn = decltype(QN)::value;   // out quarter fetched into registers here
        using SA = I<(2 * p) % 5>;
        using SB = I<(2 * p + 1) % 5>;
        using NA = I<(2 * p + 2) % 5>;
        using NB = I<(2 * p + 3) % 5>;
        using FA = I<(2 * p + 4) % 5>;
        static_assert(qn == 0 || (mode == 0 && qn <= OQ), "quarter loads in normal stages");
        if constexpr (mode == 0) {
            issueB(NB{}, k + 1);
            issueA(FA{}, k + 2);
            if constexpr (qn == 1) load_c_q_regs(1, oq1);
            else if constexpr (qn == 2) load_c_q_regs(2, oq2);
            else if constexpr (qn == 3) load_c_q_regs(3, oq3);
        } else if constexpr (mode == 1) {
            issueB(NB{}, k + 1);
            load_c_q(slot(FA{}), 0);
        } else if constexpr (OQ > 0) {
            store_c_q(slot(NB{}), oq1);
            store_c_q(slot(FA{}), oq2);
        } else {
            load_c_q(slot(NB{}), 1);
            load_c_q(slot(FA{}), 2);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < KSL - 1; ++ks) {
            read_frags(SA{}, SB{}, ks + 1, fa[(ks + 1) & 1], fb[(ks + 1) & 1]);
            mfma_range(fa[ks & 1], fb[ks & 1], 0, NMF);
            interleave(I<NFR>{}, I<NMF>{});
        }
        constexpr int KL = (KSL - 1) & 1;
        constexpr int HALF = NMF / 2;
        mfma_range(fa[KL], fb[KL], 0, HALF);
        if constexpr (mode != 2) {
            // the next stage has landed; this stage's later loads stay in flight
            __builtin_amdgcn_s_waitcnt(lt_vm_lgkm0(mode == 0 ? LA + (qn ? QLD : 0) : QLD));
            lt_lds_barrier();
            read_frags(NA{}, NB{}, 0, fa[0], fb[0]);
        }
        mfma_range(fa[KL], fb[KL], HALF, NMF);
        if constexpr (mode != 2) interleave(I<NFR>{}, I<NMF - HALF>{});
    };

    issueA(I<0>{}, 0);
    issueB(I<1>{}, 0);
    issueA(I<2>{}, 1);
    __builtin_amdgcn_s_waitcnt(lt_vm_lgkm0(LA));
    lt_lds_barrier();
    read_frags(I<0>{}, I<1>{}, 0, fa[0], fb[0]);

    constexpr int RN = (NKR + 3) % 5;           // (nk - 2) % 5
    // normal stages unrolled after the loop: the last RN (no out quarters), or
    // the last 10 + RN with the out-quarter loads at nk - 8, nk - 6, nk - 4
    // (the launcher picks OQ > 0 only for nk >= 12 + RN)
    constexpr int TL = OQ > 0 ? 10 + RN : RN;
    using Z = I<0>;
    int k = 0;
    for (; k + 5 <= nk - 2 - TL; k += 5) {
        kst(I<0>{}, Z{}, k, Z{});
        kst(I<1>{}, Z{}, k + 1, Z{});
        kst(I<2>{}, Z{}, k + 2, Z{});
        kst(I<3>{}, Z{}, k + 3, Z{});
        kst(I<4>{}, Z{}, k + 4, Z{});
    }
    // tail stage i (stage k + i) loads out quarter q at i = TL - 8 + 2q
    auto tail = [&](auto IDX) __attribute__((always_inline)) {
        constexpr int i = decltype(IDX)::value;
        constexpr int d = i - (TL - 8);
        constexpr int q = (OQ > 0 && d >= 2 && d % 2 == 0 && d / 2 <= OQ) ? d / 2 : 0;
        kst(I<i % 5>{}, Z{}, k + i, I<q>{});
    };
    [&]<int... Is>(std::integer_sequence<int, Is...>) __attribute__((always_inline)) {
        (tail(I<Is>{}), ...);
    }(std::make_integer_sequence<int, TL>{});
    k += TL;
    kst(I<RN>{}, I<1>{}, k, Z{});
    kst(I<(RN + 1) % 5>{}, I<2>{}, k + 1, Z{});
    constexpr int PL = (RN + 1) % 5;            // phase of the last stage
    using Q0 = I<(2 * PL + 2) % 5>;
    using Q1 = I<(2 * PL + 3) % 5>;
    using Q2 = I<(2 * PL + 4) % 5>;
    using Q3 = I<(2 * PL) % 5>;

    const bool edge = j0 + BJ > n;
    auto sums = [&](char *qb, int qq) __attribute__((always_inline)) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            if ((BSTR * mt + 32 * wt) / RPQ != qq) continue;
            const int r = brow + BSTR * mt;
            const int rh = r - qq * RPQ;
#pragma unroll
            for (int mj = 0; mj < MJ; ++mj) {
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const int c = (wj * (BJ / WGJ) + 32 * mj + 16 * hf + 8 * hsel) >> 3;
                    const f32x16_t &a = acc[mj][mt];
                    u32x4_t *ptr = reinterpret_cast<u32x4_t *>(
                        qb + rh * (BJ * 2) + ((c ^ (r & (CPRE - 1))) << 4));
                    u32x4_t ov = *ptr;
                    const int jc = j0 + 8 * c;
                    if (edge && jc < n && jc + 8 > n && t0 + r < T) {
                        const u16 *src = outn + (t0 + r) * ld_out + jc;
#pragma unroll
                        for (int e = 0; e < 8; e += 2) {
                            const uint32_t lo = (jc + e < n) ? src[e] : 0u;
                            const uint32_t hi = (jc + e + 1 < n) ? src[e + 1] : 0u;
                            ov[e >> 1] = lo | (hi << 16);
                        }
                    }
                    u32x4_t nv;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        nv[e] = lt_pack2(lt_bf_lo(ov[e]) + a[8 * hf + 2 * e],
                                         lt_bf_hi(ov[e]) + a[8 * hf + 2 * e + 1]);
                    *ptr = nv;
                }
            }
        }
    };
    constexpr int LPR = CPRE;
    constexpr int RPI = 64 / LPR;
    constexpr int ITQ = RPQ / NW / RPI;          // store rounds per wave and quarter
    static_assert((RPQ / NW) % RPI == 0, "whole store rounds");
    const __amdgpu_buffer_rsrc_t rp = lt_rsrc(
        prefn + t0 * ld_pre, (uint32_t)(((int64_t)max(rows_b - 1, 0) * ld_pre + n) * 2));
    const __amdgpu_buffer_rsrc_t rr = lt_rsrc(
        resn + t0 * ld_res, (uint32_t)(((int64_t)max(rows_b - 1, 0) * ld_res + n) * 2));
    auto load_prefix = [&](int qq, u32x4_t (&pv)[ITQ]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < ITQ; ++i) {
            const int r = qq * RPQ + w * (RPQ / NW) + i * RPI + l / LPR;
            const int j = j0 + 8 * (l % LPR);
            pv[i] = lt_buf_load16(rp, j + 8 <= n ? (uint32_t)(((int64_t)r * ld_pre + j) * 2)
                                                 : LT_OOB);
        }
    };
    auto write_back = [&](const char *qb, int qq, const u32x4_t (&pv)[ITQ])
        __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < ITQ; ++i) {
            const int rh = w * (RPQ / NW) + i * RPI + l / LPR;
            const int r = qq * RPQ + rh;
            const int c = l % LPR;
            const int64_t t = t0 + r;
            const int j = j0 + 8 * c;
            if (t < T && j < n) {
                const u32x4_t v = *reinterpret_cast<const u32x4_t *>(
                    qb + rh * (BJ * 2) + ((c ^ (r & (CPRE - 1))) << 4));
                if (j + 8 <= n) {
                    __builtin_amdgcn_raw_buffer_store_b128(
                        v, rc, (uint32_t)(((int64_t)r * ld_out + j) * 2), 0, LT_NT);
                    if constexpr (RES) {
                        u32x4_t rv;
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            rv[e] = lt_pack2(lt_bf_lo(pv[i][e]) + lt_bf_lo(v[e]),
                                             lt_bf_hi(pv[i][e]) + lt_bf_hi(v[e]));
                        __builtin_amdgcn_raw_buffer_store_b128(
                            rv, rr, (uint32_t)(((int64_t)r * ld_res + j) * 2), 0, 0);
                    }
                } else {
                    u16 *o = outn + t * ld_out + j;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        if (j + e < n) {
                            const u16 onew = (u16)((v[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
                            o[e] = onew;
                            if constexpr (RES) {
                                const float rs = lt_bf_lo((uint32_t)prefn[t * ld_pre + j + e]) +
                                                 lt_bf_lo((uint32_t)onew);
                                resn[t * ld_res + j + e] = (u16)(lt_pack2(rs, 0.f) & 0xFFFFu);
                            }
                        }
                    }
                }
            }
        }
    };
    // In flight now (in issue order): quarters 0, 1, 2.  Then the prefix
    // chunks of all quarters (residual form), then quarter 3 once every wave
    // is past its last reads of the last stage's slots.  Waits that come after
    // stores count them too (stores retire in order with loads), which is
    // exact only where every row and column of the tile is stored: other
    // tiles wait for everything.
    constexpr int PF = RES ? 4 * ITQ : 0;
    constexpr int SQ = RES ? 2 * ITQ : ITQ;      // stores per wave and quarter
    const bool interior = t0 + BT <= T && j0 + BJ <= n;
    u32x4_t pv0[ITQ], pv1[ITQ], pv2[ITQ], pv3[ITQ];
    if constexpr (RES) {
        load_prefix(0, pv0);
        load_prefix(1, pv1);
        load_prefix(2, pv2);
        load_prefix(3, pv3);
    }
    // quarters loaded from memory after quarter 0: 1 and 2 (OQ == 0), and 3
    // (OQ < 3, issued below)
    constexpr int Q12 = OQ > 0 ? 0 : 2 * QLD;
    constexpr int Q3L = OQ > 2 ? 0 : QLD;
    __builtin_amdgcn_s_waitcnt(lt_vm_lgkm0(Q12 + PF));         // quarter 0
    lt_lds_barrier();
    if constexpr (OQ > 2) store_c_q(slot(Q3{}), oq3);
    else load_c_q(slot(Q3{}), 3);
    sums(slot(Q0{}), 0);
    // quarter 1 (+ prefix 0)
    __builtin_amdgcn_s_waitcnt(lt_vm_lgkm0(RES ? 3 * ITQ + Q3L : (OQ > 0 ? Q3L : 2 * QLD)));
    lt_lds_barrier();
    write_back(slot(Q0{}), 0, pv0);
    sums(slot(Q1{}), 1);
    if (interior) __builtin_amdgcn_s_waitcnt(lt_vm_lgkm0(RES ? 2 * ITQ + Q3L + SQ : Q3L + SQ));
    else __builtin_amdgcn_s_waitcnt(lt_vm_lgkm0(0));         // quarter 2 (+ prefix 1)
    lt_lds_barrier();
    write_back(slot(Q1{}), 1, pv1);
    sums(slot(Q2{}), 2);
    if (interior) __builtin_amdgcn_s_waitcnt(lt_vm_lgkm0(2 * SQ));
    else __builtin_amdgcn_s_waitcnt(lt_vm_lgkm0(0));         // quarter 3 (+ all prefix)
    lt_lds_barrier();
    write_back(slot(Q2{}), 2, pv2);
    sums(slot(Q3{}), 3);
    __builtin_amdgcn_s_waitcnt(lt_vm_lgkm0(63));
    lt_lds_barrier();
    write_back(slot(Q3{}), 3, pv3);
}

// The ring GEMM over ntj x ntt tiles of 256 x 256.  Tile order: groups of
// GROUP_T token panels by every column panel, token panel fastest, so that
// the tiles an XCD runs at one time share few latent panels and the next
// tiles on the XCD reuse them (the latent loads cost about twice the W loads
// per stage otherwise, as the previous order put eight latent panels in
// each XCD's concurrent tiles; T = 8192 125.7 vs 128.6 us, 4 token panels
// 126.6, 2 128.6); each XCD takes a contiguous range of that order.  With a
// split last round (see ring_full_tiles) the halves follow the full tiles in
// the same kind of order, so the two halves of a tile share an XCD wherever
// the XCD ranges of halves have even length (as at T = 8192).
template <int WGJ, int WGT, int GROUP_T, int NKR, bool KTAIL, bool RES, int OQ>
__global__ __launch_bounds__(64 * WGJ * WGT) void k_gemm_ring(const u16 *__restrict__ Y, int ntj, int ntt,
                                                              int64_t T, int L, int n,
                                                              const u16 *__restrict__ Wn,
                                                              u16 *__restrict__ outn, int64_t ld_out,
                                                              const u16 *prefn, int64_t ld_pre,
                                                              u16 *resn, int64_t ld_res)
{
    constexpr int BJ = RING_BT;
    const int G = ntj * ntt;
    const int nfull = ring_full_tiles(G);
    const int b = blockIdx.x;
    int nb, hj = 0;                             // tile in the grouped order, W-row offset
    if (b < nfull) {
        nb = xcd_contiguous(b, nfull);
    } else {
        const int h = xcd_contiguous(b - nfull, 2 * (G - nfull));
        nb = nfull + h / 2;
        hj = (h & 1) ? BJ / 2 : 0;
    }
    const int gsize = GROUP_T * ntj;
    const int gid = nb / gsize;
    const int first_t = gid * GROUP_T;
    const int gt = min(ntt - first_t, GROUP_T);
    const int within = nb - gid * gsize;
    const int tt = first_t + within % gt;
    const int tj = within / gt;
    const int j0 = tj * BJ + hj;
    const int64_t t0 = (int64_t)tt * RING_BT;
    if (b < nfull)
        ring_tile<BJ, WGJ, WGT, NKR, KTAIL, RES, OQ>(Y, T, L, n, Wn, outn, ld_out, prefn, ld_pre,
                                                     resn, ld_res, j0, t0);
    else if (j0 < n)   // the second half of a tile that the window ends in may be empty
        ring_tile<BJ / 2, WGJ, WGT, NKR, KTAIL, RES, OQ>(Y, T, L, n, Wn, outn, ld_out, prefn,
                                                         ld_pre, resn, ld_res, j0, t0);
}

template <int WGJ, int WGT, int GROUP_T>
hipError_t launch_ring(const u16 *y, int64_t T, int L, const u16 *Wn, int n, u16 *outn,
                       int64_t ld_out, const Resid *res, hipStream_t stream)
{
    const int ntj = (n + RING_BT - 1) / RING_BT;
    const int64_t ntt = (T + RING_BT - 1) / RING_BT;
    const int nk = (L + BK - 1) / BK;
    if (nk < 3 || (int64_t)ntj * ntt > (1 << 30)) return hipErrorInvalidValue;
    const int G = (int)(ntj * ntt);
    const int nfull = ring_full_tiles(G);
    const dim3 grid((unsigned)(nfull + 2 * (G - nfull))), block(64 * WGJ * WGT);
    const u16 *pre = res ? res->prefix : nullptr;
    u16 *rsd = res ? res->resid : nullptr;
    const int64_t ldp = res ? res->ld_prefix : 0, ldr = res ? res->ld_resid : 0;
    const bool kt = L % BK != 0;
    // out quarters in registers need an unrolled tail of 10 + (nk - 2) % 5
    // normal stages
    const bool oq = LT_RING_OQ > 0 && nk >= 12 + (nk - 2) % 5;
#define LT_RING(NKR, KT, R, Q)                                                               \
    launch(&k_gemm_ring<WGJ, WGT, GROUP_T, NKR, KT, R, Q>, grid, block, stream, y, ntj,         \
           (int)ntt, T, L, n, Wn, outn, ld_out, pre, ldp, rsd, ldr)
#define LT_RING_Q(NKR, KT, R) (oq ? LT_RING(NKR, KT, R, LT_RING_OQ) : LT_RING(NKR, KT, R, 0))
#define LT_RING_K(NKR)                                                                       \
    (kt ? (res ? LT_RING_Q(NKR, true, true) : LT_RING_Q(NKR, true, false))                  \
        : (res ? LT_RING_Q(NKR, false, true) : LT_RING_Q(NKR, false, false)))
    hipError_t e;
    switch (nk % 5) {
    case 0: e = LT_RING_K(0); break;
    case 1: e = LT_RING_K(1); break;
    case 2: e = LT_RING_K(2); break;
    case 3: e = LT_RING_K(3); break;
    default: e = LT_RING_K(4); break;
    }
#undef LT_RING_K
#undef LT_RING_Q
#undef LT_RING
    return e;
}

template <int BJ, int BT, int WGJ, int WGT, int NS, int GROUP_J>
hipError_t launch_cfg(const u16 *y, int64_t T, int L, const u16 *Wn, int n, u16 *outn,
                      int64_t ld_out, const Resid *res, bool vec16, hipStream_t stream)
{
    const int ntj = (n + BJ - 1) / BJ;
    const int64_t ntt = (T + BT - 1) / BT;
    if ((int64_t)ntj * ntt > 0x7FFFFFFF) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(ntj * ntt)), block(64 * WGJ * WGT);
    // The LDS epilogue moves whole out-tile halves with workgroup-wide 16-byte
    // direct loads and addresses `out` (and the residual buffers) through
    // 32-bit buffer offsets: it needs aligned windows and tile extents below
    // 2 GiB; anything else takes the plain epilogue.
    constexpr bool EPI_OK = ((BT / 2) * (BJ / 8)) % (64 * WGJ * WGT) == 0;
    auto small = [&](int64_t ld) { return (int64_t)BT * ld * 2 < ((int64_t)1 << 31); };
    const bool epi = EPI_OK && vec16 && small(ld_out) &&
                     (!res || (small(res->ld_prefix) && small(res->ld_resid)));
    const u16 *pre = res ? res->prefix : nullptr;
    u16 *rsd = res ? res->resid : nullptr;
    const int64_t ldp = res ? res->ld_prefix : 0, ldr = res ? res->ld_resid : 0;
#define LT_GEMM_LAUNCH(KT, EPI, R)                                                           \
    launch(&k_gemm<BJ, BT, WGJ, WGT, NS, GROUP_J, KT, EPI, R>, grid, block, stream, y, ntj,         \
           (int)ntt, T, L, n, Wn, outn, ld_out, pre, ldp, rsd, ldr)
#define LT_GEMM_LAUNCH_R(KT, EPI)                                                            \
    (res ? LT_GEMM_LAUNCH(KT, EPI, true) : LT_GEMM_LAUNCH(KT, EPI, false))
    const bool kt = L % (NS * BK) != 0;
    if constexpr (EPI_OK) {
        if (epi) return kt ? LT_GEMM_LAUNCH_R(true, true) : LT_GEMM_LAUNCH_R(false, true);
    }
    return kt ? LT_GEMM_LAUNCH_R(true, false) : LT_GEMM_LAUNCH_R(false, false);
#undef LT_GEMM_LAUNCH_R
#undef LT_GEMM_LAUNCH
}

}  // namespace

hipError_t launch_gemm(const uint16_t *y, int64_t T, int L, const uint16_t *Wn, int n,
                       uint16_t *outn, int64_t ld_out, const Resid *res, hipStream_t stream)
{
    auto a16 = [](const void *p, int64_t ld) {
        return (reinterpret_cast<uintptr_t>(p) & 15) == 0 && ld % 8 == 0;
    };
    const bool vec16 = a16(outn, ld_out) && (!res || (a16(res->prefix, res->ld_prefix) &&
                                                      a16(res->resid, res->ld_resid)));
    // Tile shape and stage count by tile count (measured on n = 7168, T = 128
    // .. 8192, random data): the biggest tile that still gives about one tile
    // per CU.  256 x 256 and 128 x 128 tiles run 8 waves (two per SIMD, which
    // hide each other's LDS and barrier waits); up to one tile per CU, four
    // stages in flight hide the L2 latency that two stages leave exposed;
    // beyond that two stages (64 KB of LDS) let two 128 x 128 tiles share a
    // CU, so up to 512 of them run in one round (T = 896: 18.5 vs 22 us).
    // Below a round of 64 x 128 tiles, 64 x 64 tiles put twice as many
    // workgroups on the W stream (T = 128: 6.3 vs 7.7 us).
    auto tiles = [&](int bj, int bt) { return (int64_t)((n + bj - 1) / bj) * ((T + bt - 1) / bt); };
    // the slot ring needs at least three K stages and the LDS epilogue's
    // alignment and 32-bit tile offsets (T = 8192: 130 vs 136 us)
    auto small = [&](int64_t ld) { return (int64_t)256 * ld * 2 < ((int64_t)1 << 31); };
    const bool ring_ok = L > 2 * BK && vec16 && small(ld_out) &&
                         (!res || (small(res->ld_prefix) && small(res->ld_resid)));
    // 256 x 256 tiles from about one round of them, and on the ring also
    // where two-stage 128 x 128 tiles would need a second round of two per
    // CU: one ring round of 140-196 tiles beats two such rounds (n = 7168,
    // T = 1280 / 1536 / 1792: 32.4 / 33.7 / 35.2 vs 39.6 / 41.2 / 43.7 us per
    // call; T = 1152, 504 tiles in one round: 31.6 vs 29.3, so not there)
    if (tiles(256, 256) >= 224 || (ring_ok && tiles(128, 128) > 512)) {
        if (ring_ok) return launch_ring<4, 2, 8>(y, T, L, Wn, n, outn, ld_out, res, stream);
        return launch_cfg<256, 256, 4, 2, 2, 4>(y, T, L, Wn, n, outn, ld_out, res, vec16, stream);
    }
    // about one round of 256 x 128 tiles: the ping-pong kernel (k_gemm_pp.hip;
    // n = 7168, T = 640 .. 1024: 13-20 % faster per call than the shapes below)
    if (!res && vec16 && gemm_pp_rows(T, L, n, ld_out) != 0)
        return launch_gemm_pp(y, T, L, Wn, n, outn, ld_out, stream);
    if (tiles(128, 128) > 256)
        return launch_cfg<128, 128, 4, 2, 2, 4>(y, T, L, Wn, n, outn, ld_out, res, vec16, stream);
    // four-stage 128 x 128 also when 64 x 128 tiles would need a second round
    // (T = 320: 9.9 vs 13.7 us)
    if (tiles(128, 128) >= 224 || tiles(64, 128) > 256)
        return launch_cfg<128, 128, 4, 2, 4, 4>(y, T, L, Wn, n, outn, ld_out, res, vec16, stream);
    if (tiles(64, 128) >= 224)
        return launch_cfg<64, 128, 2, 2, 4, 4>(y, T, L, Wn, n, outn, ld_out, res, vec16, stream);
    // narrow windows at small T (the 896-column shard at T = 256: 56 tiles of
    // 64 x 64): 32 x 64 tiles of two waves put twice as many workgroups on
    // the W stream
    if (tiles(64, 64) < 128)
        return launch_cfg<32, 64, 1, 2, 4, 4>(y, T, L, Wn, n, outn, ld_out, res, vec16, stream);
    return launch_cfg<64, 64, 2, 2, 4, 4>(y, T, L, Wn, n, outn, ld_out, res, vec16, stream);
}

}  // namespace lt
