// lt_gemm.h -- pieces shared by the large-token GEMM kernels (k_gemm.hip,
// k_gemm_pp.hip): the K stage geometry, the LDS swizzle and row permutation
// of the operand tiles, and the XCD-contiguous workgroup order.  Every
// kernel that uses them accumulates each output over K in the same order
// (ascending 16-wide slices of v_mfma_f32_32x32x16_bf16), so all tile shapes
// give the same bits.
#pragma once

#include <type_traits>

#include "lt_device.h"

namespace lt {
namespace {

constexpr int BK = 64;                    // K per stage
constexpr int ROWB = BK * 2;              // bytes per stage row (one 128-byte line)
constexpr int CPR = ROWB / 16;            // 16-byte chunks per stage row
constexpr int KSL = BK / 16;              // 16-wide MFMA K slices per stage
constexpr int NUM_XCD = 8;
constexpr uint32_t OOB = LT_OOB;

typedef __attribute__((address_space(3))) void lds_void;

template <int V> using I = std::integral_constant<int, V>;

// Row permutation of a 32-row block: MFMA row m reads LDS row perm32(m).
__device__ __forceinline__ int perm32(int m)
{
    const int q = m >> 3, hh = (m >> 2) & 1, alo = m & 3;
    return 16 * (q >> 1) + 8 * hh + 4 * (q & 1) + alo;
}
// Chunk-slot XOR key (8 slots of 16 bytes per 128-byte stage row).  Over the
// rows perm32(0..31) it is a permutation on every aligned group of 8 lanes and
// on the even and the odd rows of every aligned group of 16 lanes, so
// fragment reads hit distinct banks.
__device__ __forceinline__ int swz8(int r)
{
    return ((r >> 1) & 1) | (((r ^ (r >> 2)) & 1) << 1) | (((r >> 3) & 1) << 2);
}

// Position of workgroup b in an order of G work items that gives each of the
// 8 XCDs (workgroup b runs on XCD b mod 8) one contiguous range.
__device__ __forceinline__ int xcd_contiguous(int b, int G)
{
    const int xcd = b % NUM_XCD, idx = b / NUM_XCD;
    const int q8 = G / NUM_XCD, r8 = G % NUM_XCD;
    return (xcd < r8) ? xcd * (q8 + 1) + idx : r8 * (q8 + 1) + (xcd - r8) * q8 + idx;
}

}  // namespace
}  // namespace lt
