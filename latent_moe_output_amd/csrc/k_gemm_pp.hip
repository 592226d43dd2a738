// k_gemm_pp.hip -- the large-token GEMM on 256 x 128 tiles with a ping-pong
// wave schedule, for calls that fill about one round of such tiles.
//
// Same operation, operand layout, swizzles, K order and epilogue arithmetic
// as k_gemm.hip (out[t][c0+j] = bf16(out[t][c0+j] + sum_k y[t][k] *
// W[c0+j][k]), the in-place `addmm_` of [PR50383 Key source snippets,
// `_shard_up_proj_tail`]), so its results are the same bits.
//
// Layout on gfx950:
//  * Tile: BJ = 256 (or 128) W rows (output columns) x 128 tokens, 8 waves.
//    Waves 0-3 (group 0) and 4-7 (group 1) each hold one wave per SIMD;
//    wave w owns W rows (BJ / 4) (w % 4).. and the 32-token blocks
//    64 mt + 32 (w / 4), as BJ / 128 x 2 tiles of v_mfma_f32_32x32x16_bf16
//    (W as A, the latent as B).
//  * K advances 64 at a time through three LDS stage arrays of 48 KB (32 KB)
//    filled by direct-to-LDS loads of whole 128-byte lines, XOR-swizzled.
//  * Ping-pong: the two groups run the same sequence one phase apart.  In a
//    memory phase a wave reads all fragments of its stage into registers;
//    in an MFMA phase it issues the stage's 16 (8) MFMAs back to back.  While
//    one group of a SIMD's two waves multiplies, the other reads, so the
//    matrix core of every SIMD has a wave issuing to it in both phases.
//    Each phase ends with a workgroup barrier (both groups pass the same
//    number: group 1 one extra at the start, group 0 one at the end).
//  * The next stages' loads ride in the MFMA phases, one 1 KB direct load
//    after each MFMA: a direct load holds its wave for about 60 clocks while
//    the address unit takes it, which an MFMA (32 clocks of the matrix
//    core per issue) hides.  Stage s + 2 arrives in halves: group 0's in its
//    MFMA phase of stage s, group 1's one phase earlier, so three arrays
//    rotate and every load has two to three phases to land.
//  * Epilogue: the two 64-row quarters of the `out` tile are loaded into the
//    arrays of stages nk - 3 and nk - 2 as soon as both groups have read
//    them, summed with the accumulators in LDS, and written back as whole
//    row segments (the ragged edge element by element).
// Measured against the best of the other tile shapes (same box, interleaved,
// norm off, one partial, n = 7168): T = 640 18.2 -> 15.9 us, 768 20.7 ->
// 16.6, 896 21.8 -> 17.6, 1024 22.8 -> 19.1, bit-identical; at 112 tiles
// (T = 512) or past one round (T = 1280) the other shapes win.
#include <type_traits>

#include "lt_device.h"
#include "lt_gemm.h"
#include "lt_internal.h"
#include "lt_launch.h"

namespace lt {
namespace {

constexpr int PP_BT = 128;                         // tokens per tile
constexpr int PP_MT = 2, PP_BSTR = 64;             // token blocks per wave, their stride
constexpr int PP_GROUP_T = 8;                      // token panels per tile group
constexpr int PP_RPQ = 64;                         // out quarter: 64 token rows

// Tile geometry for BJ W rows (256 or 128) x 128 tokens.
template <int BJ> struct PPGeo {
    static constexpr int STAGE_A = BJ * ROWB, STAGE = (BJ + PP_BT) * ROWB;   // 48 / 32 KB
    static constexpr int NB = (BJ + PP_BT) / 8;    // 1 KB row blocks per stage
    static constexpr int WR = BJ / 4;              // W rows per wave
    static constexpr int MJ = WR / 32;             // 32-row W blocks per wave
    static constexpr int CPRE = BJ / 8;            // 16-byte chunks per out row
    static constexpr int QB = PP_RPQ * BJ * 2;     // out quarter bytes (32 / 16 KB)
    static constexpr int HL = NB / 8;              // 1 KB loads per wave, half a stage
    static constexpr int QL = QB / 4096;           // 1 KB loads per wave, a quarter
    static constexpr int NMF = KSL * MJ * PP_MT;   // MFMAs per wave and stage
    static constexpr int NWB = PP_RPQ * CPRE / 512;   // 16-byte stores per thread, a quarter
    static_assert(HL <= NMF && QL <= NMF, "one load per MFMA at most");
    static_assert(QB <= STAGE, "an out quarter fits a stage array");
};

// BJ: W rows per tile (256 or 128); NKR = nk % 3 fixes which stage array
// every step uses; KTAIL: L % 64 != 0.
template <int BJ, int NKR, bool KTAIL>
__global__ __launch_bounds__(512) void k_gemm_pp(const u16 *__restrict__ Y, int ntj, int ntt,
                                                 int64_t T, int L, int n,
                                                 const u16 *__restrict__ Wn,
                                                 u16 *__restrict__ outn, int64_t ld_out)
{
    using Geo = PPGeo<BJ>;
    constexpr int PP_BJ = BJ, PP_STAGE_A = Geo::STAGE_A, PP_STAGE = Geo::STAGE;
    constexpr int PP_MJ = Geo::MJ, PP_CPRE = Geo::CPRE, PP_HL = Geo::HL, PP_QL = Geo::QL;
    constexpr int PP_NMF = Geo::NMF, PP_WR = Geo::WR, PP_NB = Geo::NB;
    __shared__ __attribute__((aligned(1024))) char st0[PP_STAGE];
    __shared__ __attribute__((aligned(1024))) char st1[PP_STAGE];
    __shared__ __attribute__((aligned(1024))) char st2[PP_STAGE];
    auto stage = [&](auto S) __attribute__((always_inline)) -> char * {
        constexpr int s = decltype(S)::value % 3;
        if constexpr (s == 0) return st0;
        else if constexpr (s == 1) return st1;
        else return st2;
    };

    // ---- tile order: XCD-contiguous ranges of groups of PP_GROUP_T token
    // panels by every column panel, token panel fastest (as the ring GEMM)
    const int G = ntj * ntt;
    const int nb = xcd_contiguous(blockIdx.x, G);
    const int gsize = PP_GROUP_T * ntj;
    const int gid = nb / gsize;
    const int first_t = gid * PP_GROUP_T;
    const int gt = min(ntt - first_t, PP_GROUP_T);
    const int within = nb - gid * gsize;
    const int j0 = (within / gt) * PP_BJ;
    const int64_t t0 = (int64_t)(first_t + within % gt) * PP_BT;

    const int l = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = w >> 2;              // 0: waves 0-3, 1: waves 4-7
    const int wv = w & 3;                // wave within its group = W-row block
    const int nchunk = L >> 3;
    const int nk = (L + BK - 1) / BK;
    const uint32_t row_bytes = (uint32_t)L * 2u;
    const int rows_a = min(PP_BJ, n - j0);
    const int rows_b = (int)min((int64_t)PP_BT, T - t0);
    const __amdgpu_buffer_rsrc_t ra = lt_rsrc(Wn + (int64_t)j0 * L, (uint32_t)rows_a * row_bytes);
    const __amdgpu_buffer_rsrc_t rb = lt_rsrc(Y + t0 * L, (uint32_t)rows_b * row_bytes);

    // One 1 KB direct load: block blk (8 stage rows; the first BJ / 8 blocks
    // are W rows, the rest tokens) of K stage s into dst.  Lane i writes slot i % 8 of row
    // i / 8 with global chunk (slot ^ swz8(row)); rows past the tile's end
    // and chunks past L read zero.
    auto load1 = [&](char *dst, int blk, int s) __attribute__((always_inline)) {
        const int row = 8 * blk + (l >> 3);
        const bool isA = blk < PP_BJ / 8;
        const int r = isA ? row : row - PP_BJ;
        const int ch = (l & 7) ^ swz8(r);
        uint32_t vo = (uint32_t)r * row_bytes + (uint32_t)ch * 16u;
        if (KTAIL && s * CPR + ch >= nchunk) vo = OOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(isA ? ra : rb, (lds_void *)(dst + 8 * blk * ROWB), 16,
                                                 vo, s * ROWB, 0, 0);
    };

    // ---- fragments: lane l reads row perm32(l % 32) of each 32-row block,
    // chunk 2 ks + l / 32 of the stage row for K slice ks (offset XOR 32 ks)
    const int hsel = l >> 5;
    const int arow = PP_WR * wv + perm32(l & 31);
    const int brow = 32 * grp + perm32(l & 31);
    const int xa0 = arow * ROWB + ((hsel ^ swz8(arow)) << 4);
    const int xb0 = PP_STAGE_A + brow * ROWB + ((hsel ^ swz8(brow)) << 4);
    bf16x8_t fa[KSL][PP_MJ], fb[KSL][PP_MT];
    auto read_all = [&](auto S) __attribute__((always_inline)) {
        const char *base = stage(S);
#pragma unroll
        for (int ks = 0; ks < KSL; ++ks) {
#pragma unroll
            for (int mj = 0; mj < PP_MJ; ++mj)
                fa[ks][mj] = *reinterpret_cast<const bf16x8_t *>(base + ((xa0 + mj * 32 * ROWB) ^ (32 * ks)));
#pragma unroll
            for (int mt = 0; mt < PP_MT; ++mt)
                fb[ks][mt] = *reinterpret_cast<const bf16x8_t *>(
                    base + ((xb0 + mt * PP_BSTR * ROWB) ^ (32 * ks)));
        }
    };
    f32x16_t acc[PP_MJ][PP_MT];
#pragma unroll
    for (int mj = 0; mj < PP_MJ; ++mj)
#pragma unroll
        for (int mt = 0; mt < PP_MT; ++mt) acc[mj][mt] = f32x16_t{};

    // ---- out quarter q (token rows 64 q.., BJ columns): 16-byte chunk c of
    // row r at slot c ^ (r % CPRE); loaded by the four waves of group 1
    const __amdgpu_buffer_rsrc_t rc = lt_rsrc(
        outn + t0 * ld_out, (uint32_t)(((int64_t)max(rows_b - 1, 0) * ld_out + n) * 2));
    auto load_q1 = [&](char *dst, int q, int it) __attribute__((always_inline)) {
        const int idx0 = 256 * it + 64 * wv;
        const int r = (idx0 + l) / PP_CPRE, c = ((idx0 + l) % PP_CPRE) ^ (r & (PP_CPRE - 1));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rc, (lds_void *)(dst + idx0 * 16), 16,
            (uint32_t)(((int64_t)(PP_RPQ * q + r) * ld_out + j0 + 8 * c) * 2), 0, 0, LT_NT);
    };

    // MFMA phase: the stage's MFMAs, the first NL of them each followed by
    // one of this phase's loads (LD: 0 none, 1 this group's half of stage
    // sl into SD, 2 out quarter q into SD)
    auto mfma_phase = [&](auto LD, auto SD, int sl, int q) __attribute__((always_inline)) {
        constexpr int ld = decltype(LD)::value;
        constexpr int NL = ld == 1 ? PP_HL : (ld == 2 ? PP_QL : 0);
#pragma unroll
        for (int ks = 0; ks < KSL; ++ks)
#pragma unroll
            for (int mj = 0; mj < PP_MJ; ++mj)
#pragma unroll
                for (int mt = 0; mt < PP_MT; ++mt) {
                    acc[mj][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ks][mj], fb[ks][mt],
                                                                          acc[mj][mt], 0, 0, 0);
                    const int i = (ks * PP_MJ + mj) * PP_MT + mt;
                    if constexpr (ld == 1) {
                        if (i < NL) load1(stage(SD), (PP_NB / 2) * grp + 4 * i + wv, sl);
                    } else if constexpr (ld == 2) {
                        if (i < NL) load_q1(stage(SD), q, i);
                    }
                }
        if constexpr (NL > 0) {
#pragma unroll
            for (int i = 0; i < NL; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // one VMEM load
            }
            __builtin_amdgcn_sched_group_barrier(0x008, PP_NMF - NL, 0);
        }
    };
    auto barrier = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        lt_lds_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };
    // One K stage of one group: memory phase (fragments of the stage in S,
    // then wait until at most WM loads of this wave are in flight), barrier,
    // MFMA phase with its loads, wait for at most WF, barrier.
    auto step = [&](auto S, auto WM, auto LD, auto SD, auto WF, int sl, int q)
        __attribute__((always_inline)) {
        read_all(S);
        __builtin_amdgcn_s_waitcnt(lt_vm_lgkm0(decltype(WM)::value));
        barrier();
        mfma_phase(LD, SD, sl, q);
        __builtin_amdgcn_s_waitcnt(lt_vm_lgkm0(decltype(WF)::value));
        barrier();
    };

    // ---- schedule.  Phase 2s: group 0 reads stage s, group 1 multiplies
    // stage s - 1; phase 2s + 1: group 0 multiplies stage s, group 1 reads
    // it.  Stage s + 2 (array (s + 2) % 3, whose stage s - 1 both groups
    // have read) is loaded by group 0 in phase 2s + 1 and by group 1 in
    // phase 2s; each wave waits for its own half of stage s + 1 before the
    // barrier that opens phase 2s + 2 (group 0 at the end of its MFMA phase,
    // group 1 at the end of its memory phase).
    constexpr int TAIL = 3 + NKR;             // steps after the loop: nk - TAIL = 0 mod 3
    const int nl = nk - TAIL;
    using N = I<0>;                           // LD: no loads
    using H = I<1>;                           // LD: half a K stage
    using Q = I<2>;                           // LD: an out quarter
    using W63 = I<63>;                        // no wait on loads
    using WH = I<PP_HL>;
    using WQ = I<PP_QL>;
    using W0 = I<0>;
    // prologue: stages 0 and 1 by every wave (blocks 8 i + w)
#pragma unroll
    for (int i = 0; i < PP_HL; ++i) load1(stage(I<0>{}), 8 * i + w, 0);
#pragma unroll
    for (int i = 0; i < PP_HL; ++i) load1(stage(I<1>{}), 8 * i + w, 1);
    __builtin_amdgcn_s_waitcnt(lt_vm_lgkm0(0));
    barrier();
    if (grp == 0) {
        for (int s = 0; s < nl; s += 3) {
            step(I<0>{}, W63{}, H{}, I<2>{}, WH{}, s + 2, 0);
            step(I<1>{}, W63{}, H{}, I<0>{}, WH{}, s + 3, 0);
            step(I<2>{}, W63{}, H{}, I<1>{}, WH{}, s + 4, 0);
        }
        // the NKR steps left before nk - 3, then nk - 3 (its load is the
        // last: stage nk - 1), nk - 2 and nk - 1
        if constexpr (NKR >= 1) step(I<0>{}, W63{}, H{}, I<2>{}, WH{}, nl + 2, 0);
        if constexpr (NKR >= 2) step(I<1>{}, W63{}, H{}, I<0>{}, WH{}, nl + 3, 0);
        step(I<NKR>{}, W63{}, H{}, I<NKR + 2>{}, WH{}, nk - 1, 0);
        step(I<NKR + 1>{}, W63{}, N{}, I<0>{}, W0{}, 0, 0);
        step(I<NKR + 2>{}, W63{}, N{}, I<0>{}, W0{}, 0, 0);
        barrier();                            // pairs with group 1's last phase
    } else {
        // group 1's half of stage 2 (its "MFMA phase of stage -1")
#pragma unroll
        for (int i = 0; i < PP_HL; ++i) load1(stage(I<2>{}), PP_NB / 2 + 4 * i + wv, 2);
        barrier();                            // group 1 runs one phase behind
        for (int s = 0; s < nl; s += 3) {
            step(I<0>{}, WH{}, H{}, I<0>{}, W63{}, s + 3, 0);
            step(I<1>{}, WH{}, H{}, I<1>{}, W63{}, s + 4, 0);
            step(I<2>{}, WH{}, H{}, I<2>{}, W63{}, s + 5, 0);
        }
        if constexpr (NKR >= 1) step(I<0>{}, WH{}, H{}, I<0>{}, W63{}, nl + 3, 0);
        if constexpr (NKR >= 2) step(I<1>{}, WH{}, H{}, I<1>{}, W63{}, nl + 4, 0);
        step(I<NKR>{}, WH{}, Q{}, I<NKR>{}, W63{}, 0, 0);            // nk - 3: out quarter 0
        step(I<NKR + 1>{}, WQ{}, Q{}, I<NKR + 1>{}, W63{}, 0, 1);    // nk - 2: out quarter 1
        step(I<NKR + 2>{}, W63{}, N{}, I<0>{}, W63{}, 0, 0);         // nk - 1
    }
    char *q0b = stage(I<NKR>{}), *q1b = stage(I<NKR + 1>{});

    // ---- epilogue: every wave adds its sums of quarter q (acc[.][q]) into
    // the quarter in LDS, rounding once; then the quarters are written back
    // as whole row segments.  Ragged edges: rows past T and columns past n
    // are not written; the chunk that crosses the window's end is read and
    // written element by element.
    const bool edge = j0 + PP_BJ > n;
    const int brow_q = 32 * grp + perm32(l & 31);
    auto sums = [&](char *qb, auto QQ) __attribute__((always_inline)) {
        constexpr int q = decltype(QQ)::value;
        const int64_t t = t0 + PP_RPQ * q + brow_q;
#pragma unroll
        for (int mj = 0; mj < PP_MJ; ++mj)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int c = (PP_WR * wv + 32 * mj + 16 * h + 8 * hsel) >> 3;
                u32x4_t *p = reinterpret_cast<u32x4_t *>(qb + brow_q * (PP_BJ * 2) +
                                                         ((c ^ (brow_q & (PP_CPRE - 1))) << 4));
                u32x4_t ov = *p;
                const int jc = j0 + 8 * c;
                if (edge && jc < n && jc + 8 > n && t < T) {
                    const u16 *src = outn + t * ld_out + jc;
#pragma unroll
                    for (int e = 0; e < 8; e += 2) {
                        const uint32_t lo = (jc + e < n) ? src[e] : 0u;
                        const uint32_t hi = (jc + e + 1 < n) ? src[e + 1] : 0u;
                        ov[e >> 1] = lo | (hi << 16);
                    }
                }
                const f32x16_t &av = acc[mj][q];
                u32x4_t nv;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    nv[e] = lt_pack2(lt_bf_lo(ov[e]) + av[8 * h + 2 * e],
                                     lt_bf_hi(ov[e]) + av[8 * h + 2 * e + 1]);
                *p = nv;
            }
    };
    auto write_back = [&](const char *qb, int q) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < Geo::NWB; ++i) {
            const int idx = 512 * i + (int)threadIdx.x;
            const int r = idx / PP_CPRE, c = idx % PP_CPRE;
            const int64_t t = t0 + PP_RPQ * q + r;
            const int j = j0 + 8 * c;
            if (t < T && j < n) {
                const u32x4_t v = *reinterpret_cast<const u32x4_t *>(qb + r * (PP_BJ * 2) +
                                                                     ((c ^ (r & (PP_CPRE - 1))) << 4));
                if (j + 8 <= n) {
                    __builtin_amdgcn_raw_buffer_store_b128(
                        v, rc, (uint32_t)(((int64_t)(PP_RPQ * q + r) * ld_out + j) * 2), 0, LT_NT);
                } else {
                    u16 *o = outn + t * ld_out + j;
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (j + e < n) o[e] = (u16)((v[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
                }
            }
        }
    };
    __builtin_amdgcn_s_waitcnt(lt_vm_lgkm0(0));       // both quarters (group 1's loads)
    barrier();
    sums(q0b, I<0>{});
    sums(q1b, I<1>{});
    __builtin_amdgcn_s_waitcnt(lt_vm_lgkm0(63));
    barrier();
    write_back(q0b, 0);
    write_back(q1b, 1);
}

}  // namespace

int gemm_pp_rows(int64_t T, int L, int n, int64_t ld_out)
{
    if ((L + BK - 1) / BK < 4 || (int64_t)PP_BT * ld_out * 2 >= ((int64_t)1 << 31)) return 0;
    // 256-row tiles only: on 128-row tiles (which the kernel also takes) it
    // measured slower than the four- and two-stage 128 x 128 kernels wherever
    // it would fill a round (n = 7168, T = 260 .. 512: 3-8 % per call)
    const int64_t tiles = (int64_t)((n + 255) / 256) * ((T + PP_BT - 1) / PP_BT);
    return tiles >= PP_MIN_TILES && tiles <= PP_MAX_TILES ? 256 : 0;
}

template <int BJ>
hipError_t launch_pp_bj(const uint16_t *y, int64_t T, int L, const uint16_t *Wn, int n,
                        uint16_t *outn, int64_t ld_out, hipStream_t stream)
{
    const int ntj = (n + BJ - 1) / BJ;
    const int ntt = (int)((T + PP_BT - 1) / PP_BT);
    const int nk = (L + BK - 1) / BK;
    const bool kt = L % BK != 0;
    const dim3 grid((unsigned)(ntj * ntt)), block(512);
#define LT_PP(NKR, KT)                                                                       \
    launch(&k_gemm_pp<BJ, NKR, KT>, grid, block, stream, y, ntj, ntt, T, L, n, Wn, outn, ld_out)
    switch (nk % 3) {
    case 0: return kt ? LT_PP(0, true) : LT_PP(0, false);
    case 1: return kt ? LT_PP(1, true) : LT_PP(1, false);
    default: return kt ? LT_PP(2, true) : LT_PP(2, false);
    }
#undef LT_PP
}

hipError_t launch_gemm_pp(const uint16_t *y, int64_t T, int L, const uint16_t *Wn, int n,
                          uint16_t *outn, int64_t ld_out, hipStream_t stream)
{
    if (gemm_pp_rows(T, L, n, ld_out) != 256) return hipErrorInvalidValue;
    return launch_pp_bj<256>(y, T, L, Wn, n, outn, ld_out, stream);
}

}  // namespace lt
