// k_attn_res.hip -- AttnRes state update and output RMSNorm, zero-block path.
//
// [PR50593 Implementation, item 1]: the fused AttnRes kernel adds the delta to
// the prefix sum in fp32, rounds the sum to bf16 storage precision and uses
// that value as the residual source from then on (the prefix is updated in
// place), writes it to the block-residual slot when the layer writes a
// block, and applies the output RMSNorm with its variance in fp32.  With no
// valid blocks the softmax over sources has the prefix as its only source,
// so the aggregated value is the prefix itself and the streaming-softmax
// loop disappears.  The three switches (delta, block write, output norm) are
// template parameters, as the pages' kernel makes them compile-time flags.
//
// The op moves `10*T*H` bytes at most and does no contraction, so it is bound
// by memory latency and bandwidth, not by the matrix cores:
//  * One workgroup of NWV waves per token row.  Lane l of wave v owns the
//    16-byte chunks l + 64*v + 64*NWV*i (i < CH) of the row, so every
//    wave-wide load or store covers 1 KB of contiguous row data and a row of
//    7168 bf16 spreads over 8 waves (two chunks per lane), so one row lands
//    in about one round trip of a few loads per lane (H = 7168, back to back:
//    T = 1 2.6 us against 4.1 with one wave per row, T = 17 3.0 against 4.4,
//    T = 320 7.8 against 8.8; 4 or 16 waves were slower at T = 320).  All
//    of the lane's prefix, delta and norm-weight loads are issued before the
//    first use; chunks past the row end read as zero through the buffer
//    range check and are never stored.
//  * The sum of two bf16 values is exact in fp32 up to one fp32 rounding,
//    and fp32 carries more than twice bf16's precision plus two bits, so
//    bf16(fp32(a + b)) is the correctly rounded bf16 of the exact sum.
//  * Each lane sums the squares of its chunks in fp32 in chunk order; each
//    wave adds its 64 lane totals with an xor butterfly, and the NWV wave
//    totals are added in wave order through LDS (fixed order, no atomics),
//    so every thread of the row holds the same total.
//  * The output is bf16((p' * w) * r): p' * w is exact in fp32 (a product of
//    two bf16 values), then one fp32 rounding of the scaling by r before the
//    bf16 rounding -- the convention of the latent norm in lt_latent.h.
#include "lt_device.h"
#include "lt_internal.h"
#include "lt_launch.h"

namespace lt {
namespace {

template <int CH, int NWV, bool DELTA, bool BLOCK, bool NORM>
__global__ __launch_bounds__(64 * NWV) void k_attn_res(u16 *prefix, const u16 *__restrict__ delta,
                                                       u16 *block, int64_t block_stride,
                                                       const u16 *__restrict__ norm_w,
                                                       u16 *__restrict__ out, int H, float eps,
                                                       float inv_H)
{
    const int64_t t = blockIdx.x;
    const int tid = threadIdx.x;
    const int l = tid & 63;
    [[maybe_unused]] const int v = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nch = H >> 3;
    const uint32_t row_bytes = (uint32_t)H * 2u;
    u16 *prow = prefix + t * H;
    const __amdgpu_buffer_rsrc_t rp = lt_rsrc(prow, row_bytes);
    auto chunk = [&](int i) { return tid + 64 * NWV * i; };   // chunk of the row (l + 64 v + ...)

    u32x4_t pv[CH], dv[CH], wv[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const int c = chunk(i);
        pv[i] = lt_buf_load16(rp, c < nch ? (uint32_t)c * 16u : LT_OOB);
    }
    if constexpr (DELTA) {
        const __amdgpu_buffer_rsrc_t rd = lt_rsrc(delta + t * H, row_bytes);
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = chunk(i);
            dv[i] = lt_buf_load16(rd, c < nch ? (uint32_t)c * 16u : LT_OOB);
        }
    }
    if constexpr (NORM) {
        const __amdgpu_buffer_rsrc_t rw = lt_rsrc(norm_w, row_bytes);
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = chunk(i);
            wv[i] = lt_buf_load16(rw, c < nch ? (uint32_t)c * 16u : LT_OOB);
        }
    }

    // p' = bf16(prefix + delta)
    if constexpr (DELTA) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            u32x4_t x;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                x[e] = lt_pack2(lt_bf_lo(pv[i][e]) + lt_bf_lo(dv[i][e]),
                                lt_bf_hi(pv[i][e]) + lt_bf_hi(dv[i][e]));
            pv[i] = x;
        }
    }

    u16 *brow = BLOCK ? block + t * block_stride : nullptr;
    u16 *orow = out + t * H;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const int c = chunk(i);
        if (c < nch) {
            if constexpr (DELTA) *reinterpret_cast<u32x4_t *>(prow + 8 * c) = pv[i];
            if constexpr (BLOCK) *reinterpret_cast<u32x4_t *>(brow + 8 * c) = pv[i];
            if constexpr (!NORM) *reinterpret_cast<u32x4_t *>(orow + 8 * c) = pv[i];
        }
    }
    if constexpr (NORM) {
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < CH; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float a = lt_bf_lo(pv[i][e]), b = lt_bf_hi(pv[i][e]);
                ss = __builtin_fmaf(a, a, ss);
                ss = __builtin_fmaf(b, b, ss);
            }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) ss = ss + __shfl_xor(ss, m, 64);
        if constexpr (NWV > 1) {
            __shared__ float red[NWV];
            if (l == 0) red[v] = ss;
            __builtin_amdgcn_s_waitcnt(lt_vm_lgkm0(63));   // LDS only: the stores may fly
            lt_lds_barrier();
            ss = red[0];
#pragma unroll
            for (int k = 1; k < NWV; ++k) ss = ss + red[k];
        }
        const float r = lt_inv_rms(ss, inv_H, eps);
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = chunk(i);
            if (c < nch) {
                u32x4_t y;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    y[e] = lt_pack2((lt_bf_lo(pv[i][e]) * lt_bf_lo(wv[i][e])) * r,
                                    (lt_bf_hi(pv[i][e]) * lt_bf_hi(wv[i][e])) * r);
                *reinterpret_cast<u32x4_t *>(orow + 8 * c) = y;
            }
        }
    }
}

template <int CH, int NWV>
hipError_t launch_shape(u16 *prefix, const u16 *delta, int64_t T, int H, u16 *block_slot,
                        int64_t block_stride, const u16 *norm_w, float eps, u16 *out,
                        hipStream_t stream)
{
    const dim3 grid((unsigned)T), block(64 * NWV);
    const float inv_H = 1.0f / (float)H;
#define LT_AR(D, B, N)                                                                           \
    launch(&k_attn_res<CH, NWV, D, B, N>, grid, block, stream, prefix, delta, block_slot,          \
           block_stride, norm_w, out, H, eps, inv_H)
    const int sel = (delta ? 4 : 0) | (block_slot ? 2 : 0) | (norm_w ? 1 : 0);
    switch (sel) {
    case 0: return LT_AR(false, false, false);
    case 1: return LT_AR(false, false, true);
    case 2: return LT_AR(false, true, false);
    case 3: return LT_AR(false, true, true);
    case 4: return LT_AR(true, false, false);
    case 5: return LT_AR(true, false, true);
    case 6: return LT_AR(true, true, false);
    default: return LT_AR(true, true, true);
    }
#undef LT_AR
}

}  // namespace

hipError_t launch_attn_res(uint16_t *prefix, const uint16_t *delta, int64_t T, int H,
                           uint16_t *block_slot, int64_t block_stride, const uint16_t *norm_w,
                           float eps, uint16_t *out, hipStream_t stream)
{
    // waves per row: one per 64 chunks of 16 bytes, up to 8; one chunk per
    // lane up to 512 chunks (H = 4096), two up to 1024 (H = 8192)
    const int nch = H / 8;
    if (nch <= 64) return launch_shape<1, 1>(prefix, delta, T, H, block_slot, block_stride, norm_w, eps, out, stream);
    if (nch <= 128) return launch_shape<1, 2>(prefix, delta, T, H, block_slot, block_stride, norm_w, eps, out, stream);
    if (nch <= 256) return launch_shape<1, 4>(prefix, delta, T, H, block_slot, block_stride, norm_w, eps, out, stream);
    if (nch <= 512) return launch_shape<1, 8>(prefix, delta, T, H, block_slot, block_stride, norm_w, eps, out, stream);
    if (nch <= 1024) return launch_shape<2, 8>(prefix, delta, T, H, block_slot, block_stride, norm_w, eps, out, stream);
    return hipErrorInvalidValue;
}

}  // namespace lt
