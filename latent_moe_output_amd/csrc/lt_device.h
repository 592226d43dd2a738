// lt_device.h -- device-side helpers shared by the tail's HIP kernels.
//
// Holds the vector types, bf16 conversions and the one definition of how a
// latent row is reduced and normalised.  Both the weight-streaming kernel and
// the sum+RMSNorm kernel build their latent from these helpers with the same
// assignment of 8-element chunks to reduction slots, so the two paths produce
// bit-identical latents for the same inputs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t u16;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// One 8-element chunk (16 bytes) of a bf16 row.
#define LT_CHUNK 8
// Chunks of a row are dealt round-robin to 16 reduction slots: chunk c goes to
// slot c % 16 and is that slot's (c / 16)-th term.
#define LT_SLOTS 16

__device__ __forceinline__ float lt_bf_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float lt_bf_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// Two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t lt_pack2(float lo, float hi)
{
    f32x2_t f = {lo, hi};
    bf16x2_t b = __builtin_convertvector(f, bf16x2_t);
    return __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ void lt_unpack8(u32x4_t v, float f[8])
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = lt_bf_lo(v[i]);
        f[2 * i + 1] = lt_bf_hi(v[i]);
    }
}

__device__ __forceinline__ u32x4_t lt_pack8(const float f[8])
{
    u32x4_t v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = lt_pack2(f[2 * i], f[2 * i + 1]);
    return v;
}

__device__ __forceinline__ u32x4_t lt_load16(const u16 *p)
{
    return *reinterpret_cast<const u32x4_t *>(p);
}

// Sum of the P partial chunks starting at `p0` (partial stride `pstride`
// elements), fp32, p ascending; with more than one partial the sum is rounded
// to bf16 (the reduced latent is stored as bf16 before it is normalised).
// Returns the chunk as packed bf16 and its float values in s[8].
__device__ __forceinline__ u32x4_t lt_sum_chunk(const u16 *p0, int64_t pstride, int P,
                                                float s[8])
{
    u32x4_t v = lt_load16(p0);
    if (P == 1) {
        lt_unpack8(v, s);
        return v;
    }
    lt_unpack8(v, s);
    for (int p = 1; p < P; ++p) {
        float x[8];
        lt_unpack8(lt_load16(p0 + (int64_t)p * pstride), x);
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] = s[e] + x[e];
    }
    u32x4_t r = lt_pack8(s);
    lt_unpack8(r, s);
    return r;
}

// Adds the squares of one chunk to a slot's running sum, elements in order.
__device__ __forceinline__ float lt_ss_chunk(const float s[8], float acc)
{
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_fmaf(s[e], s[e], acc);
    return acc;
}

// 1 / sqrt(mean square + eps) from the row's total of squares.
__device__ __forceinline__ float lt_inv_rms(float total, float inv_L, float eps)
{
    return rsqrtf(__builtin_fmaf(total, inv_L, eps));
}

// y = bf16((s * r) * w) for one chunk; w given as packed bf16.
__device__ __forceinline__ u32x4_t lt_scale_chunk(const float s[8], float r, u32x4_t w)
{
    float wf[8], y[8];
    lt_unpack8(w, wf);
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = (s[e] * r) * wf[e];
    return lt_pack8(y);
}

// The 16 slot sums of a row are combined as a balanced binary tree in slot
// order: ((S0+S1)+(S2+S3)) + ((S4+S5)+(S6+S7)) + ...  Both kernels follow it.
