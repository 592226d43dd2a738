// k_norm.hip -- partial sum + bf16 round trip + RMSNorm into a [T][L] latent.
//
// First kernel of the large-token path.  [PR51253 Key source snippets,
// `_check_matches_replicated`]: the routed partials are reduced first and
// RMS-normalised over the latent width second; [PR50593 Implementation,
// item 1]: accumulate in fp32, round to bf16 storage precision, keep the
// variance in fp32.  HBM-bound: every partial is read once and the latent is
// written once.
//
// One workgroup per 16-token tile, built by the same tile code (lt_latent.h)
// as the weight-streaming kernel, so both paths give identical latents.  The
// tile moves between memory and registers through the staged LDS layout of
// lt_latent.h, so loads and stores cover whole 128-byte lines.
#include "lt_internal.h"
#include "lt_latent.h"
#include "lt_launch.h"

namespace lt {
namespace {

// `y` may be `part` itself with one partial: every workgroup has copied its
// rows into LDS (and waited for them) before it writes them.
template <int NI, bool ST>
__global__ __launch_bounds__(64 * KW) void k_sum_rmsnorm(const u16 *part,
                                                         int64_t pstride, int P, int64_t T, int L,
                                                         const u16 *__restrict__ norm_w, float eps,
                                                         float inv_L, u16 *y)
{
    __shared__ float red[1][KW * 16];
    __shared__ __attribute__((aligned(1024))) char lds_t[latent_stage_bytes<1, NI>()];
    __shared__ __attribute__((aligned(1024))) char lds_nw[ST ? weight_stage_bytes<NI>() : 16];
    const int64_t t0 = (int64_t)blockIdx.x * 16;
    const int Tv = (int)min((int64_t)16, T - t0);
    const u16 *tile = part + t0 * L;

    // one partial: the tile (its rows below Tv) and the norm weight are
    // copied into LDS as whole lines (ST); several: loaded and summed in
    // registers
    u32x4_t sv[1][NI], wv[NI];
    if constexpr (ST) {
        latent_stage<1, NI, 0, true>(tile, Tv, L, lds_t);
        if (norm_w) weight_stage<NI>(norm_w, L, lds_nw);
        __builtin_amdgcn_s_waitcnt(lt_vm_lgkm0(0));
        lt_lds_barrier();
        if (norm_w) {
            latent_from_lds<1, NI>(lds_t, sv);
            weight_from_lds<NI>(lds_nw, wv);
        }
    } else {
        latent_load(tile, Tv, L, sv[0]);
        if (norm_w) latent_load_weight(norm_w, L, wv);
        latent_sum(tile, pstride, P, Tv, L, sv[0]);
    }
    // the normalised tile goes back into the staged layout (each slot is
    // written by the lane that read it) and is stored from there as whole
    // lines; without the norm a staged tile is already there
    if (norm_w) latent_norm<1, NI>(sv, wv, eps, inv_L, red);
    if (!ST || norm_w) {
        latent_to_lds<1, NI>(lds_t, sv);
        __builtin_amdgcn_s_waitcnt(lt_vm_lgkm0(63));
        lt_lds_barrier();
    }
    constexpr int SPR = 32 * NI;
    const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int nchunk = L >> 3;
#pragma unroll
    for (int k = 0; k < NI; ++k) {
        const int m = KW * k + w;
        const int slot = 64 * m + l;
        const int row = slot / SPR, c = (slot % SPR) ^ (row & 15);
        if (row < Tv && c < nchunk)
            *reinterpret_cast<u32x4_t *>(y + (t0 + row) * L + c * 8) =
                *reinterpret_cast<const u32x4_t *>(lds_t + 16 * slot);
    }
}

// s = bf16(sum_p part[p]) elementwise, fp32 accumulation in ascending p (the
// order latent_sum uses, so the result is the same bits): 8 elements per
// thread, all P loads of a thread issued together, whole lines per wave.
__global__ __launch_bounds__(256) void k_sum_partials(const u16 *__restrict__ part, int64_t pstride,
                                                      int P, int64_t count, u16 *__restrict__ s)
{
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
    if (i >= count) return;
    const u16 *src = part + i;
    float acc[8];
    lt_unpack8(*reinterpret_cast<const u32x4_t *>(src), acc);
    constexpr int B = 8;                     // partials in flight per thread
    for (int p = 1; p < P; p += B) {
        u32x4_t x[B];
#pragma unroll
        for (int b = 0; b < B; ++b)
            if (p + b < P) x[b] = *reinterpret_cast<const u32x4_t *>(src + (int64_t)(p + b) * pstride);
#pragma unroll
        for (int b = 0; b < B; ++b) {
            if (p + b >= P) break;
            float f[8];
            lt_unpack8(x[b], f);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = acc[e] + f[e];
        }
    }
    *reinterpret_cast<u32x4_t *>(s + i) = lt_pack8(acc);
}

template <int NI>
hipError_t launch_ni(const u16 *part, int64_t pstride, int P, int64_t T, int L,
                     const u16 *norm_w, float eps, u16 *y, hipStream_t stream)
{
    const dim3 grid((unsigned)((T + 15) / 16)), block(64 * KW);
    if (P == 1)
        return launch(&k_sum_rmsnorm<NI, true>, grid, block, stream, part, pstride, P, T, L, norm_w,
                      eps, 1.0f / (float)L, y);
    return launch(&k_sum_rmsnorm<NI, false>, grid, block, stream, part, pstride, P, T, L, norm_w,
                  eps, 1.0f / (float)L, y);
}

}  // namespace

hipError_t launch_sum_partials(const uint16_t *part, int64_t pstride, int P, int64_t count,
                               uint16_t *s, hipStream_t stream)
{
    const int64_t threads = (count + 7) / 8;
    return launch(&k_sum_partials, dim3((unsigned)((threads + 255) / 256)), dim3(256), stream, part,
                  pstride, P, count, s);
}

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
