// k_skinny.hip -- weight-streaming tail for small token counts (decode).
//
// One launch does the whole tail for up to 64 tokens: partial sum, bf16
// storage round trip, RMSNorm and the windowed projection with its beta-add
// ([PR50383 Key source snippets, `_shard_up_proj_tail`]: reduce, norm,
// narrow, addmm_).  At these token counts the work is bound by reading the
// W window from HBM once, so the kernel is built around that stream:
//
//  * A workgroup owns 16 rows of the W window (16 output columns).  Its four
//    waves split the latent width: chunk c (8 elements) goes to wave
//    (c / 4) % 4, lane group c % 4, step c / 16.  Each lane's W chunks are
//    loaded straight into registers in the A-operand layout of
//    v_mfma_f32_16x16x32_bf16 (row = lane % 16, 8 consecutive k per lane), so
//    W never passes through LDS and each row is read as 64-byte runs.
//  * The partial chunks are loaded first, then the norm weight, then all of
//    the workgroup's W chunks, so the whole W share is in flight while the
//    latent is being normalised.
//  * The latent is built in registers in the B-operand layout (token = lane
//    % 16), with the sum of squares reduced lanes -> waves in the fixed slot
//    tree of lt_device.h.  Tokens ride the MFMA's 16-wide N dimension; the
//    idle columns of a partly filled token tile cost nothing that matters
//    here, the MFMA pipe is far from busy.
//  * The four per-wave partial products are added in LDS in a fixed order
//    and written with one bf16 rounding onto the window.
//
// Every element's accumulation order depends only on (T, L), never on c0 or
// n, so column shards reproduce the full-window result bit for bit.
#include "lt_device.h"
#include "lt_internal.h"

namespace lt {
namespace {

template <int NI, int TT>
__global__ __launch_bounds__(256) void k_skinny(const u16 *__restrict__ part, int64_t pstride,
                                                int P, int T, int L,
                                                const u16 *__restrict__ norm_w, float eps,
                                                float inv_L, const u16 *__restrict__ Wn, int n,
                                                u16 *__restrict__ outn, int64_t ld_out, int vec8)
{
    const int w = threadIdx.x >> 6;
    const int l = threadIdx.x & 63;
    const int r = l & 15;
    const int g = l >> 4;
    const int nchunk = L >> 3;
    const int j0 = blockIdx.x * 16;

    __shared__ float red_ss[4][TT * 16];
    __shared__ f32x4_t red_acc[4][TT][64];

    // 1. issue loads: partial 0, norm weight, W rows
    u32x4_t sv[TT][NI];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        const int t = 16 * tt + r;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int c = 16 * i + 4 * w + g;
            sv[tt][i] = (c < nchunk && t < T) ? lt_load16(part + (int64_t)t * L + c * 8)
                                              : u32x4_t{0, 0, 0, 0};
        }
    }
    u32x4_t wv[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int c = 16 * i + 4 * w + g;
        wv[i] = (norm_w && c < nchunk) ? lt_load16(norm_w + c * 8) : u32x4_t{0, 0, 0, 0};
    }
    u32x4_t wa[NI];
    {
        const int j = j0 + r;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int c = 16 * i + 4 * w + g;
            wa[i] = (c < nchunk && j < n) ? lt_load16(Wn + (int64_t)j * L + c * 8)
                                          : u32x4_t{0, 0, 0, 0};
        }
    }

    // 2. remaining partials, bf16 round trip of the sum, slot sums of squares
    float ss[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        const int t = 16 * tt + r;
        ss[tt] = 0.f;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int c = 16 * i + 4 * w + g;
            if (c < nchunk && t < T) {
                float s[8];
                lt_unpack8(sv[tt][i], s);
                if (P > 1) {
                    const u16 *p0 = part + (int64_t)t * L + c * 8;
                    for (int p = 1; p < P; ++p) {
                        float x[8];
                        lt_unpack8(lt_load16(p0 + (int64_t)p * pstride), x);
#pragma unroll
                        for (int e = 0; e < 8; ++e) s[e] = s[e] + x[e];
                    }
                    sv[tt][i] = lt_pack8(s);
                    lt_unpack8(sv[tt][i], s);
                }
                ss[tt] = lt_ss_chunk(s, ss[tt]);
            }
        }
    }

    // 3. RMSNorm: slots -> lanes (xor 16, xor 32) -> waves, fixed tree
    if (norm_w) {
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
            float v = ss[tt];
            v = v + __shfl_xor(v, 16);
            v = v + __shfl_xor(v, 32);
            if (g == 0) red_ss[w][16 * tt + r] = v;
        }
        __syncthreads();
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
            const int x = 16 * tt + r;
            const float total = (red_ss[0][x] + red_ss[1][x]) + (red_ss[2][x] + red_ss[3][x]);
            const float rs = lt_inv_rms(total, inv_L, eps);
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                float s[8];
                lt_unpack8(sv[tt][i], s);
                sv[tt][i] = lt_scale_chunk(s, rs, wv[i]);
            }
        }
    }

    // 4. projection on the matrix cores: D[j][t] += W[j][k] * y[t][k]
    f32x4_t acc[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) acc[tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, wa[i]);
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
            acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                a, __builtin_bit_cast(bf16x8_t, sv[tt][i]), acc[tt], 0, 0, 0);
    }

    // 5. add the four waves' partial products, then beta-add onto the window
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) red_acc[w][tt][l] = acc[tt];
    __syncthreads();
    for (int tt = w; tt < TT; tt += 4) {
        const f32x4_t a0 = red_acc[0][tt][l], a1 = red_acc[1][tt][l];
        const f32x4_t a2 = red_acc[2][tt][l], a3 = red_acc[3][tt][l];
        const f32x4_t d = (a0 + a1) + (a2 + a3);
        const int t = 16 * tt + r;       // D column = lane % 16
        const int j = j0 + 4 * g;        // D rows 4*(lane/16) + 0..3
        if (t >= T) continue;
        u16 *o = outn + (int64_t)t * ld_out + j;
        if (vec8 && j + 4 <= n) {
            u32x2_t ov = *reinterpret_cast<const u32x2_t *>(o);
            u32x2_t nv;
            nv[0] = lt_pack2(lt_bf_lo(ov[0]) + d[0], lt_bf_hi(ov[0]) + d[1]);
            nv[1] = lt_pack2(lt_bf_lo(ov[1]) + d[2], lt_bf_hi(ov[1]) + d[3]);
            *reinterpret_cast<u32x2_t *>(o) = nv;
        } else {
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                if (j + a < n) {
                    const float v = lt_bf_lo((uint32_t)o[a]) + d[a];
                    o[a] = (u16)(lt_pack2(v, 0.f) & 0xFFFFu);
                }
            }
        }
    }
}

template <int NI, int TT>
hipError_t launch_nt(const u16 *part, int64_t pstride, int P, int T, int L, const u16 *norm_w,
                     float eps, const u16 *Wn, int n, u16 *outn, int64_t ld_out, int vec8,
                     hipStream_t stream)
{
    const dim3 grid((n + 15) / 16), block(256);
    hipLaunchKernelGGL((k_skinny<NI, TT>), grid, block, 0, stream, part, pstride, P, T, L,
                       norm_w, eps, 1.0f / (float)L, Wn, n, outn, ld_out, vec8);
    return hipGetLastError();
}

template <int NI>
hipError_t launch_ni(const u16 *part, int64_t pstride, int P, int T, int L, const u16 *norm_w,
                     float eps, const u16 *Wn, int n, u16 *outn, int64_t ld_out, int vec8,
                     hipStream_t stream)
{
    if (T <= 16)
        return launch_nt<NI, 1>(part, pstride, P, T, L, norm_w, eps, Wn, n, outn, ld_out, vec8,
                                stream);
    if constexpr (NI <= 8) {
        if (T <= 32)
            return launch_nt<NI, 2>(part, pstride, P, T, L, norm_w, eps, Wn, n, outn, ld_out,
                                    vec8, stream);
        return launch_nt<NI, 4>(part, pstride, P, T, L, norm_w, eps, Wn, n, outn, ld_out, vec8,
                                stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

int skinny_tokens_per_launch(int L) { return L > 1024 ? 16 : 64; }

hipError_t launch_skinny(const uint16_t *part, int64_t pstride, int P, int T, int L,
                         const uint16_t *norm_w, float eps, const uint16_t *Wn, int n,
                         uint16_t *outn, int64_t ld_out, hipStream_t stream)
{
    if (T < 1 || T > skinny_tokens_per_launch(L)) return hipErrorInvalidValue;
    const int vec8 = ((reinterpret_cast<uintptr_t>(outn) & 7) == 0) && (ld_out % 4 == 0);
    const int ni = (L + 127) / 128;
    if (ni <= 1) return launch_ni<1>(part, pstride, P, T, L, norm_w, eps, Wn, n, outn, ld_out, vec8, stream);
    if (ni <= 2) return launch_ni<2>(part, pstride, P, T, L, norm_w, eps, Wn, n, outn, ld_out, vec8, stream);
    if (ni <= 4) return launch_ni<4>(part, pstride, P, T, L, norm_w, eps, Wn, n, outn, ld_out, vec8, stream);
    if (ni <= 8) return launch_ni<8>(part, pstride, P, T, L, norm_w, eps, Wn, n, outn, ld_out, vec8, stream);
    return launch_ni<16>(part, pstride, P, T, L, norm_w, eps, Wn, n, outn, ld_out, vec8, stream);
}

}  // namespace lt
