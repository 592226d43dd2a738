// k_norm.hip -- partial sum + bf16 round trip + RMSNorm into a [T][L] latent.
//
// First kernel of the large-token path.  [PR51253 Key source snippets,
// `_check_matches_replicated`]: the routed partials are reduced first and
// RMS-normalised over the latent width second; [PR50593 Implementation,
// item 1]: accumulate in fp32, round to bf16 storage precision, keep the
// variance in fp32.  HBM-bound: every partial is read once and the latent is
// written once.
//
// Sixteen lanes own one row: lane s reads chunks s, s+16, s+32, ... (so a
// row is read as 256-byte runs) and keeps them in registers between the
// reduction and the scaling.  The sum of squares is combined across the 16
// lanes with xor-1, -2, -4, -8 shuffles, which is the same slot tree the
// weight-streaming kernel uses, so both paths give identical latents.
#include "lt_device.h"
#include "lt_internal.h"

namespace lt {
namespace {

template <int NI>
__global__ __launch_bounds__(256) void k_sum_rmsnorm(const u16 *__restrict__ part,
                                                     int64_t pstride, int P, int64_t T, int L,
                                                     const u16 *__restrict__ norm_w, float eps,
                                                     float inv_L, u16 *__restrict__ y)
{
    const int s = threadIdx.x & 15;
    const int64_t t = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    const bool valid = t < T;
    const int nchunk = L >> 3;
    const u16 *row = part + t * L;

    u32x4_t sv[NI];
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int c = 16 * i + s;
        if (valid && c < nchunk) {
            float v[8];
            sv[i] = lt_sum_chunk(row + c * 8, pstride, P, v);
            acc = lt_ss_chunk(v, acc);
        } else {
            sv[i] = u32x4_t{0, 0, 0, 0};
        }
    }
    if (norm_w) {
        acc = acc + __shfl_xor(acc, 1);
        acc = acc + __shfl_xor(acc, 2);
        acc = acc + __shfl_xor(acc, 4);
        acc = acc + __shfl_xor(acc, 8);
        const float rs = lt_inv_rms(acc, inv_L, eps);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int c = 16 * i + s;
            if (valid && c < nchunk) {
                float v[8];
                lt_unpack8(sv[i], v);
                sv[i] = lt_scale_chunk(v, rs, lt_load16(norm_w + c * 8));
            }
        }
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int c = 16 * i + s;
        if (valid && c < nchunk) *reinterpret_cast<u32x4_t *>(y + t * L + c * 8) = sv[i];
    }
}

template <int NI>
hipError_t launch_ni(const u16 *part, int64_t pstride, int P, int64_t T, int L,
                     const u16 *norm_w, float eps, u16 *y, hipStream_t stream)
{
    const dim3 grid((unsigned)((T + 15) / 16)), block(256);
    hipLaunchKernelGGL((k_sum_rmsnorm<NI>), grid, block, 0, stream, part, pstride, P, T, L,
                       norm_w, eps, 1.0f / (float)L, y);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sum_rmsnorm(const uint16_t *part, int64_t pstride, int P, int64_t T, int L,
                              const uint16_t *norm_w, float eps, uint16_t *y,
                              hipStream_t stream)
{
    const int ni = (L + 127) / 128;
    if (ni <= 1) return launch_ni<1>(part, pstride, P, T, L, norm_w, eps, y, stream);
    if (ni <= 2) return launch_ni<2>(part, pstride, P, T, L, norm_w, eps, y, stream);
    if (ni <= 4) return launch_ni<4>(part, pstride, P, T, L, norm_w, eps, y, stream);
    if (ni <= 8) return launch_ni<8>(part, pstride, P, T, L, norm_w, eps, y, stream);
    return launch_ni<16>(part, pstride, P, T, L, norm_w, eps, y, stream);
}

}  // namespace lt
