// k_norm.hip -- partial sum + bf16 round trip + RMSNorm into a [T][L] latent.
//
// First kernel of the large-token path.  [PR51253 Key source snippets,
// `_check_matches_replicated`]: the routed partials are reduced first and
// RMS-normalised over the latent width second; [PR50593 Implementation,
// item 1]: accumulate in fp32, round to bf16 storage precision, keep the
// variance in fp32.  HBM-bound: every partial is read once and the latent is
// written once.
//
// The latent of a 16-token tile is built by the same tile code (lt_latent.h)
// as the weight-streaming kernel, so both paths give identical latents.  A
// workgroup handles RW = 16 / SUB rows of one tile: with few tiles (small T)
// SUB workgroups share a tile, so that the call still spreads over about 256
// workgroups.  Each token keeps its lane of the tile (token t on lane t % 16)
// and every MFMA output depends on one token only, so rows outside a
// workgroup's range (never loaded, never stored) do not change its bits.
// Rows move between memory and LDS as whole 128-byte lines in the staged
// layout of lt_latent.h: one partial by direct-to-LDS loads; several loaded
// as whole lines into registers, summed there in fp32 in ascending p (the
// order latent_sum uses, so the bits are the same) and rounded once on the
// way into LDS.
#include "lt_internal.h"
#include "lt_latent.h"
#include "lt_launch.h"
#include "lt_store.h"

namespace lt {
namespace {

// `y` may be `part` itself with one partial: every workgroup has copied its
// rows into LDS (and waited for them) before it writes them.
// NTL: the partials are loaded with the non-temporal hint (read once; used
// for calls whose partials total 16 MiB or more, where it measured faster:
// the 4-partial 8191-token shard 36.3 -> 34.9 us per call, T = 8192 with one
// partial 8.8 -> 8.1 us per norm kernel; slower on small calls: the
// 8-partial 256-token shard 9.60 -> 9.95, T = 4096 with one partial 5.4 ->
// 5.6).
template <int NI, int SUB, bool ST, bool NTL>
__global__ __launch_bounds__(64 * KW) void k_sum_rmsnorm(const u16 *part,
                                                         int64_t pstride, int P, int64_t T, int L,
                                                         const u16 *__restrict__ norm_w, float eps,
                                                         float inv_L, u16 *y)
{
    constexpr int RW = 16 / SUB;                // rows of the tile this workgroup owns
    constexpr int SPR = 32 * NI;                // 16-byte slots per staged row
    constexpr int NT = 64 * KW;
    __shared__ float red[1][KW * 16];
    __shared__ __attribute__((aligned(1024))) char lds_t[latent_stage_bytes<1, NI>()];
    __shared__ __attribute__((aligned(1024))) char lds_nw[weight_stage_bytes<NI>()];
    const int64_t t0 = (int64_t)(blockIdx.x / SUB) * 16;
    const int r0 = RW * (int)(blockIdx.x % SUB);
    const int Tv = (int)min((int64_t)16, T - t0);
    const int r1 = min(r0 + RW, Tv);            // rows [r0, r1) of the tile
    if (r0 >= r1) return;                       // whole workgroup: past the last token
    const u16 *tile = part + t0 * L;
    const int tid = threadIdx.x;
    const int l = tid & 63, w = tid >> 6;
    const int nchunk = L >> 3;

    if constexpr (ST) {
        latent_stage<1, NI, NTL ? LT_NT : 0, true>(tile, r1, L, lds_t, r0);
    } else {
        // slot g of rows [r0, r0 + RW): row r0 + g / SPR, chunk g % SPR
        constexpr int CPT = (RW * SPR + NT - 1) / NT;    // slots per thread
        constexpr int BATCH = CPT >= 16 ? 1 : (16 / CPT > 8 ? 8 : 16 / CPT);   // partials per trip
        const uint32_t rbytes = (uint32_t)((r1 - r0) * L) * 2u;
        uint32_t off[CPT];
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int g = tid + NT * j;
            const int rr = g / SPR, c = g % SPR;
            off[j] = (g < RW * SPR && r0 + rr < r1 && c < nchunk) ? (uint32_t)(rr * L + c * 8) * 2u
                                                                  : LT_OOB;
        }
        const u16 *rows = tile + (int64_t)r0 * L;
        float acc[CPT][8];
        // BATCH partials per round trip, partial 0 in the first one; partials
        // past P get an empty resource (nothing is fetched) and are not added
        // (adding their zeros would turn a -0 sum into +0)
        for (int p0 = 0; p0 < P; p0 += BATCH) {
            const int nb = min(BATCH, P - p0);
            u32x4_t x[BATCH][CPT];
#pragma unroll
            for (int b = 0; b < BATCH; ++b) {
                const __amdgpu_buffer_rsrc_t rp =
                    lt_rsrc(rows + (int64_t)(p0 + b) * pstride, b < nb ? rbytes : 0u);
#pragma unroll
                for (int j = 0; j < CPT; ++j)
                    x[b][j] = NTL ? lt_buf_load16_nt(rp, off[j]) : lt_buf_load16(rp, off[j]);
            }
#pragma unroll
            for (int b = 0; b < BATCH; ++b) {
#pragma unroll
                for (int j = 0; j < CPT; ++j) {
                    float f[8];
                    lt_unpack8(x[b][j], f);
                    if (b == 0 && p0 == 0) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) acc[j][e] = f[e];
                    } else if (b < nb) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) acc[j][e] = acc[j][e] + f[e];
                    }
                }
            }
        }
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int g = tid + NT * j;
            const int rr = g / SPR, c = g % SPR;
            const int row = r0 + rr;
            if (g < RW * SPR && row < r1)
                *reinterpret_cast<u32x4_t *>(lds_t + (row * SPR + (c ^ (row & 15))) * 16) =
                    lt_pack8(acc[j]);
        }
    }
    if (norm_w) weight_stage<NI>(norm_w, L, lds_nw);
    __builtin_amdgcn_s_waitcnt(lt_vm_lgkm0(0));
    lt_lds_barrier();

    // the normalised tile goes back into the staged layout (each slot is
    // written by the lane that read it) and is stored from there as whole
    // lines; without the norm the staged rows are the latent already
    if (norm_w) {
        u32x4_t sv[1][NI], wv[NI];
        latent_from_lds<1, NI>(lds_t, sv);
        weight_from_lds<NI>(lds_nw, wv);
        latent_norm<1, NI>(sv, wv, eps, inv_L, red);
        latent_to_lds<1, NI>(lds_t, sv);
        __builtin_amdgcn_s_waitcnt(lt_vm_lgkm0(63));
        lt_lds_barrier();
    }
    // device-scope stores (sc1), whole call back to back: T = 128 11.42 ->
    // 11.30 us, the 8-partial 256-token shard 9.84 -> 9.61, the 4-partial
    // 8191-token shard 36.06 -> 35.71
    const __amdgpu_buffer_rsrc_t ry = lt_rsrc(y + t0 * L, latent_tile_bytes(Tv, L));
#pragma unroll
    for (int k = 0; k < NI; ++k) {
        const int m = KW * k + w;
        const int slot = 64 * m + l;
        const int row = slot / SPR, c = (slot % SPR) ^ (row & 15);
        if (row >= r0 && row < r1 && c < nchunk)
            __builtin_amdgcn_raw_buffer_store_b128(
                *reinterpret_cast<const u32x4_t *>(lds_t + 16 * slot), ry,
                (uint32_t)(row * L + c * 8) * 2u, 0, LT_SC1);
    }
}

template <int NI, int SUB>
hipError_t launch_sub(const u16 *part, int64_t pstride, int P, int64_t T, int L,
                      const u16 *norm_w, float eps, u16 *y, hipStream_t stream)
{
    const dim3 grid((unsigned)((T + 15) / 16 * SUB)), block(64 * KW);
    const bool ntl = (int64_t)P * T * L * 2 >= ((int64_t)16 << 20);
#define LT_SR(ST, NTL)                                                                       \
    launch(&k_sum_rmsnorm<NI, SUB, ST, NTL>, grid, block, stream, part, pstride, P, T, L,      \
           norm_w, eps, 1.0f / (float)L, y)
    if (P == 1) return ntl ? LT_SR(true, true) : LT_SR(true, false);
    return ntl ? LT_SR(false, true) : LT_SR(false, false);
#undef LT_SR
}

// Workgroups per tile: about 256 workgroups in all, at least one row each.
template <int NI>
hipError_t launch_ni(const u16 *part, int64_t pstride, int P, int64_t T, int L,
                     const u16 *norm_w, float eps, u16 *y, hipStream_t stream)
{
    const int64_t tiles = (T + 15) / 16;
    if (tiles >= 256) return launch_sub<NI, 1>(part, pstride, P, T, L, norm_w, eps, y, stream);
    if (tiles >= 128) return launch_sub<NI, 2>(part, pstride, P, T, L, norm_w, eps, y, stream);
    if (tiles >= 64) return launch_sub<NI, 4>(part, pstride, P, T, L, norm_w, eps, y, stream);
    if (tiles >= 32) return launch_sub<NI, 8>(part, pstride, P, T, L, norm_w, eps, y, stream);
    return launch_sub<NI, 16>(part, pstride, P, T, L, norm_w, eps, y, stream);
}

}  // namespace

hipError_t launch_sum_rmsnorm(const uint16_t *part, int64_t pstride, int P, int64_t T, int L,
                              const uint16_t *norm_w, float eps, uint16_t *y,
                              hipStream_t stream)
{
    const int ni = latent_steps(L);
    if (ni <= 1) return launch_ni<1>(part, pstride, P, T, L, norm_w, eps, y, stream);
    if (ni <= 2) return launch_ni<2>(part, pstride, P, T, L, norm_w, eps, y, stream);
    if (ni <= 4) return launch_ni<4>(part, pstride, P, T, L, norm_w, eps, y, stream);
    return launch_ni<8>(part, pstride, P, T, L, norm_w, eps, y, stream);
}

}  // namespace lt
