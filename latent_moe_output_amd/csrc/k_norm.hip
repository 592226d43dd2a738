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
// as the weight-streaming kernel, so both paths give identical latents; the
// registers are then stored to the packed [T][L] latent.
#include "lt_internal.h"
#include "lt_latent.h"

namespace lt {
namespace {

template <int NI>
__global__ __launch_bounds__(64 * KW) void k_sum_rmsnorm(const u16 *__restrict__ part,
                                                         int64_t pstride, int P, int64_t T, int L,
                                                         const u16 *__restrict__ norm_w, float eps,
                                                         float inv_L, u16 *__restrict__ y)
{
    __shared__ float red[1][KW * 16];
    const int64_t t0 = (int64_t)blockIdx.x * 16;
    const int Tv = (int)min((int64_t)16, T - t0);
    const u16 *tile = part + t0 * L;

    u32x4_t sv[1][NI], wv[NI];
    latent_load(tile, Tv, L, sv[0]);
    if (norm_w) latent_load_weight(norm_w, L, wv);
    latent_sum(tile, pstride, P, Tv, L, sv[0]);
    if (norm_w) latent_norm<1, NI>(sv, wv, eps, inv_L, red);

    const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int t = l & 15, g = l >> 4;
    const int nchunk = L >> 3;
    if (t >= Tv) return;
    u16 *row = y + (t0 + t) * L;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int c = 4 * KW * i + 4 * w + g;
        if (c < nchunk) *reinterpret_cast<u32x4_t *>(row + c * 8) = sv[0][i];
    }
}

template <int NI>
hipError_t launch_ni(const u16 *part, int64_t pstride, int P, int64_t T, int L,
                     const u16 *norm_w, float eps, u16 *y, hipStream_t stream)
{
    const dim3 grid((unsigned)((T + 15) / 16)), block(64 * KW);
    hipLaunchKernelGGL((k_sum_rmsnorm<NI>), grid, block, 0, stream, part, pstride, P, T, L,
                       norm_w, eps, 1.0f / (float)L, y);
    return hipGetLastError();
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
