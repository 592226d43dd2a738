// lt_device.h -- device-side helpers shared by the tail's HIP kernels.
//
// Vector types, bf16 conversions, the RMSNorm scaling step and the LDS
// hand-off barrier.  How a latent tile is built lives in lt_latent.h.
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

// Raw buffer resources (stride 0): a load whose byte offset is at or past
// num_records returns zeros, so ragged edges need no branches.
constexpr uint32_t LT_RSRC_W3 = 0x00020000u;   // raw buffer, dword data
constexpr uint32_t LT_OOB = 0x80000000u;       // an offset every resource rejects

__device__ __forceinline__ __amdgpu_buffer_rsrc_t lt_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             LT_RSRC_W3);
}

// 16-byte load at byte offset `off` of a resource (zeros when out of range).
__device__ __forceinline__ u32x4_t lt_buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Cache-policy bit of buffer instructions: non-temporal (streamed data that
// is not read again, e.g. the W window of a decode call).
constexpr int LT_NT = 2;

// The same load, marked non-temporal.
__device__ __forceinline__ u32x4_t lt_buf_load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, LT_NT));
}

// 1 / sqrt(mean square + eps) from the row's total of squares.
__device__ __forceinline__ float lt_inv_rms(float total, float inv_L, float eps)
{
    return rsqrtf(__builtin_fmaf(total, inv_L, eps));
}

// s_waitcnt immediate (gfx9 encoding): wait until at most `n` vector memory
// operations are outstanding and all LDS operations have completed.
constexpr int lt_vm_lgkm0(int n) { return (n & 15) | (7 << 4) | (0 << 8) | ((n >> 4) << 14); }

// Workgroup barrier for LDS hand-offs.  The caller has already waited (with
// s_waitcnt) for exactly the loads and LDS operations the hand-off needs;
// __syncthreads() would add a release fence that drains every outstanding
// global load, including loads meant to stay in flight across the barrier.
// The empty asm statements keep the compiler from moving memory accesses
// across it.
__device__ __forceinline__ void lt_lds_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
