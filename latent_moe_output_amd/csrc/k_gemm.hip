// k_gemm.hip -- bf16 MFMA GEMM with a windowed beta-add epilogue.
//
// Second kernel of the large-token path: out[t][c0+j] = bf16(out[t][c0+j] +
// sum_k y[t][k] * W[c0+j][k]) -- the in-place `addmm_` on the narrowed weight
// rows and output columns of [PR50383 Key source snippets,
// `_shard_up_proj_tail`], which folds the shared-expert partial into the
// projection instead of running a separate add.
//
// Layout on gfx950:
//  * Workgroup tile BJ (W rows = output columns) x BT (tokens), 4 waves in a
//    2 x 2 grid, K step 64.  Each wave owns (BJ/2) x (BT/2) as 32 x 32 tiles of
//    v_mfma_f32_32x32x16_bf16 with W as the A operand and the latent as B, so
//    a lane's accumulators run along the output row.
//  * Global -> registers -> LDS, two LDS stages, one barrier per K step; the
//    next step's loads are in flight while the current step multiplies.  A
//    row of a stage is 64 bf16 = eight 16-byte chunks, stored XOR-swizzled so
//    the fragment reads of 8 consecutive lanes hit 8 different chunk slots.
//  * A-operand rows are read through a fixed permutation of the 32 rows of a
//    tile chosen so that each lane ends up holding 16 consecutive output
//    columns (two runs of 8): the epilogue is then 16-byte loads and stores of
//    `out`, and lanes l and l+32 cover 32 contiguous bytes of a row.
//  * Ragged edges (tokens >= T, columns >= n, k >= L) are zero-filled on load
//    and masked on store; nothing outside [c0, c0+n) x [0, T) is written.
//  * Tiles are spread so that each of the 8 XCDs receives a contiguous range
//    of the (grouped) tile order, keeping W and latent blocks that are reused
//    by neighbouring tiles in the same XCD's L2.
// Each output element's accumulation order depends on (L, tile config) only,
// not on c0 or n.
#include "lt_device.h"
#include "lt_internal.h"

namespace lt {
namespace {

constexpr int BK = 64;
constexpr int NUM_XCD = 8;

// Row permutation of a 32-row A tile: MFMA row m reads LDS row perm32(m).
__device__ __forceinline__ int perm32(int m)
{
    const int q = m >> 3, hh = (m >> 2) & 1, alo = m & 3;
    return 16 * (q >> 1) + 8 * hh + 4 * (q & 1) + alo;
}
// Chunk-slot swizzles (8 slots of 16 bytes per 128-byte stage row).
__device__ __forceinline__ int swz_a(int row) { return (row & 3) | ((row >> 1) & 4); }
__device__ __forceinline__ int swz_b(int row) { return row & 7; }

template <int BJ, int BT, int GROUP_J>
__global__ __launch_bounds__(256) void k_gemm(const u16 *__restrict__ Y, int64_t T, int L,
                                              const u16 *__restrict__ Wn, int n,
                                              u16 *__restrict__ outn, int64_t ld_out, int vec16,
                                              int ntj, int ntt)
{
    constexpr int MJ = BJ / 64, MT = BT / 64;   // 32x32 tiles per wave
    constexpr int LA = BJ / 32, LB = BT / 32;   // 16-byte loads per thread per stage
    __shared__ __attribute__((aligned(16))) u16 sA[2][BJ * BK];
    __shared__ __attribute__((aligned(16))) u16 sB[2][BT * BK];

    // ---- tile coordinates: XCD-contiguous ranges, then GROUP_J-wide groups
    const int G = ntj * ntt;
    const int b = blockIdx.x;
    const int xcd = b % NUM_XCD, idx = b / NUM_XCD;
    const int q8 = G / NUM_XCD, r8 = G % NUM_XCD;
    const int nb = (xcd < r8) ? xcd * (q8 + 1) + idx : r8 * (q8 + 1) + (xcd - r8) * q8 + idx;
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
    const int w = tid >> 6, l = tid & 63;
    const int wj = w >> 1, wt = w & 1;
    const int nchunk = L >> 3;
    const int nk = (L + BK - 1) / BK;

    const int lrow = tid >> 3, lch = tid & 7;
    u32x4_t ra[LA], rb[LB];

    auto gload = [&](int kb) {
        const int c = kb * 8 + lch;
        const bool kok = c < nchunk;
#pragma unroll
        for (int q = 0; q < LA; ++q) {
            const int j = j0 + lrow + 32 * q;
            ra[q] = (kok && j < n) ? lt_load16(Wn + (int64_t)j * L + c * 8) : u32x4_t{0, 0, 0, 0};
        }
#pragma unroll
        for (int q = 0; q < LB; ++q) {
            const int64_t t = t0 + lrow + 32 * q;
            rb[q] = (kok && t < T) ? lt_load16(Y + t * L + c * 8) : u32x4_t{0, 0, 0, 0};
        }
    };
    auto lstore = [&](int st) {
#pragma unroll
        for (int q = 0; q < LA; ++q) {
            const int row = lrow + 32 * q;
            *reinterpret_cast<u32x4_t *>(&sA[st][row * BK + ((lch ^ swz_a(row)) << 3)]) = ra[q];
        }
#pragma unroll
        for (int q = 0; q < LB; ++q) {
            const int row = lrow + 32 * q;
            *reinterpret_cast<u32x4_t *>(&sB[st][row * BK + ((lch ^ swz_b(row)) << 3)]) = rb[q];
        }
    };

    f32x16_t acc[MJ][MT];
#pragma unroll
    for (int mj = 0; mj < MJ; ++mj)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mj][mt] = f32x16_t{};

    const int arow0 = wj * (BJ / 2) + perm32(l & 31);
    const int brow0 = wt * (BT / 2) + (l & 31);
    const int hsel = l >> 5;

    gload(0);
    lstore(0);
    __syncthreads();

    for (int kb = 0; kb < nk; ++kb) {
        const int st = kb & 1;
        if (kb + 1 < nk) gload(kb + 1);
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int ch = 2 * ks + hsel;
            bf16x8_t fa[MJ], fb[MT];
#pragma unroll
            for (int mj = 0; mj < MJ; ++mj) {
                const int row = arow0 + 32 * mj;
                fa[mj] = *reinterpret_cast<const bf16x8_t *>(
                    &sA[st][row * BK + ((ch ^ swz_a(row)) << 3)]);
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int row = brow0 + 32 * mt;
                fb[mt] = *reinterpret_cast<const bf16x8_t *>(
                    &sB[st][row * BK + ((ch ^ swz_b(row)) << 3)]);
            }
#pragma unroll
            for (int mj = 0; mj < MJ; ++mj)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    acc[mj][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mj], fb[mt],
                                                                          acc[mj][mt], 0, 0, 0);
        }
        if (kb + 1 < nk) lstore(st ^ 1);
        __syncthreads();
    }

    // ---- epilogue: lane holds columns 16*half + 8*hsel + 0..7 of each tile
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int64_t t = t0 + brow0 + 32 * mt;
        if (t >= T) continue;
        u16 *orow = outn + t * ld_out;
#pragma unroll
        for (int mj = 0; mj < MJ; ++mj) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int j = j0 + wj * (BJ / 2) + 32 * mj + 16 * half + 8 * hsel;
                const f32x16_t &a = acc[mj][mt];
                if (vec16 && j + 8 <= n) {
                    const u32x4_t ov = lt_load16(orow + j);
                    u32x4_t nv;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        nv[e] = lt_pack2(lt_bf_lo(ov[e]) + a[8 * half + 2 * e],
                                         lt_bf_hi(ov[e]) + a[8 * half + 2 * e + 1]);
                    *reinterpret_cast<u32x4_t *>(orow + j) = nv;
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        if (j + e < n) {
                            const float v = lt_bf_lo((uint32_t)orow[j + e]) + a[8 * half + e];
                            orow[j + e] = (u16)(lt_pack2(v, 0.f) & 0xFFFFu);
                        }
                    }
                }
            }
        }
    }
}

template <int BJ, int BT, int GROUP_J>
hipError_t launch_cfg(const u16 *y, int64_t T, int L, const u16 *Wn, int n, u16 *outn,
                      int64_t ld_out, int vec16, hipStream_t stream)
{
    const int ntj = (n + BJ - 1) / BJ;
    const int64_t ntt = (T + BT - 1) / BT;
    if ((int64_t)ntj * ntt > 0x7FFFFFFF) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(ntj * ntt)), block(256);
    hipLaunchKernelGGL((k_gemm<BJ, BT, GROUP_J>), grid, block, 0, stream, y, T, L, Wn, n, outn,
                       ld_out, vec16, ntj, (int)ntt);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const uint16_t *y, int64_t T, int L, const uint16_t *Wn, int n,
                       uint16_t *outn, int64_t ld_out, hipStream_t stream)
{
    const int vec16 = ((reinterpret_cast<uintptr_t>(outn) & 15) == 0) && (ld_out % 8 == 0);
    const int64_t tiles256 = (int64_t)((n + 255) / 256) * ((T + 255) / 256);
    const int64_t tiles128 = (int64_t)((n + 127) / 128) * ((T + 127) / 128);
    if (tiles256 >= 512)
        return launch_cfg<256, 256, 4>(y, T, L, Wn, n, outn, ld_out, vec16, stream);
    if (tiles128 >= 256)
        return launch_cfg<128, 128, 4>(y, T, L, Wn, n, outn, ld_out, vec16, stream);
    return launch_cfg<64, 64, 4>(y, T, L, Wn, n, outn, ld_out, vec16, stream);
}

}  // namespace lt
