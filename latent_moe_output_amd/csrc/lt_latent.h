// lt_latent.h -- the one definition of how a 16-token tile's latent is built.
//
// Partial sum, bf16 storage round trip and RMSNorm
// ([PR51253 Key source snippets, `_check_matches_replicated`]: reduce the
// routed partials first, then `F.rms_norm` over the latent width with the
// norm weight and eps; [PR50593 Implementation, item 1]: fp32 accumulation,
// bf16 storage round trip, fp32 variance).
//
// A workgroup of KW waves computes the latent of 16 tokens directly in the
// B-operand register layout of v_mfma_f32_16x16x32_bf16: at step i, lane l of
// wave w holds chunk c = 4*KW*i + 4*w + (l >> 4) (latent elements 8c..8c+7)
// of token (l & 15).  Both the weight-streaming kernel (which multiplies the
// registers straight away) and the sum+RMSNorm kernel (which stores them)
// build their latent with these functions and the same KW, so the two paths
// give bit-identical latents.
//
// The sum of squares of each token is taken on the matrix cores: with the
// tile S in both operand slots, v_mfma_f32_16x16x32_bf16 accumulates S * S^T,
// whose diagonal holds each token's sum of squares over the wave's chunks.
// The KW per-wave sums are then added in wave order through LDS.  The norm
// weight is applied on the matrix cores too (one-hot A operands, below), so
// the vector units only multiply by each token's rsqrt and round.
#pragma once

#include "lt_device.h"

namespace lt {

constexpr int KW = 8;   // waves splitting the latent width

// Steps needed for latent width L (chunks of 8, 4*KW chunks per step).
__host__ __device__ constexpr int latent_steps(int L) { return (L + 32 * KW - 1) / (32 * KW); }

// Byte offset of this lane's chunk at step i within a tile of row stride L,
// or LT_OOB past the row end.
__device__ __forceinline__ uint32_t latent_offset(int i, int L)
{
    const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int c = 4 * KW * i + 4 * w + (l >> 4);
    return c < (L >> 3) ? (uint32_t)((l & 15) * L + c * 8) * 2u : LT_OOB;
}

// Bytes of a tile holding Tv valid token rows (none when Tv <= 0).
__device__ __forceinline__ uint32_t latent_tile_bytes(int Tv, int L)
{
    return Tv > 0 ? (uint32_t)(Tv * L) * 2u : 0u;
}

// Loads partial 0 of this lane's chunks of tokens [0, Tv) of the tile whose
// first token row starts at `tile` (row stride L).  Chunks past the row end
// and tokens >= Tv read as zero (buffer range check, no branches).
template <int NI>
__device__ __forceinline__ void latent_load(const u16 *__restrict__ tile, int Tv, int L,
                                            u32x4_t (&sv)[NI])
{
    const __amdgpu_buffer_rsrc_t r = lt_rsrc(tile, latent_tile_bytes(Tv, L));
#pragma unroll
    for (int i = 0; i < NI; ++i) sv[i] = lt_buf_load16(r, latent_offset(i, L));
}

// ---- LDS staging of a partial's tiles.
//
// Loading the B-operand layout straight from memory makes every load
// instruction touch 16 rows at the same 64-byte offset of each row; on this
// chip's vector L1 that pattern moves about a third of what whole contiguous
// lines move (about 21 vs 58 bytes per clock per CU, measured).  So the tile
// is first copied into LDS as whole lines by direct-to-LDS loads, 1 KB of
// contiguous row data per wave instruction, then read back in the operand
// layout.
//
// Staged layout: row r (token 16*tt + t) holds 32*NI slots of 16 bytes at
// lds + r * NI * 512; global chunk c of the row sits in slot c ^ (r & 15).
// The XOR keeps the 16 lanes that read one chunk of 16 rows on distinct LDS
// banks, and keeps every aligned group of 4 lanes of a copy instruction on
// 4 consecutive chunks of one line.  Slots past the row end and rows past
// Tv hold zeros.
template <int TT, int NI>
constexpr int latent_stage_bytes() { return 16 * TT * NI * 512; }

// Issues the copy of tokens [0, min(Tv, 16*TT)) of partial 0 (row stride L)
// into the staged layout: up to TT*NI direct loads per wave, all KW waves
// taking part, with cache policy AUX.  The caller waits for them (vmcnt) and
// runs a workgroup barrier before latent_from_lds.  The A operand of
// v_mfma_f32_16x16x32_bf16 has the same per-lane layout as the B operand
// (row = lane % 16), so W rows can be staged and read back the same way.
// With SKIP, 1 KB blocks that start at or past row Tv are not loaded: those
// rows keep whatever the LDS held.  That is harmless wherever rows >= Tv are
// never stored: every output of an MFMA depends on one row of each operand,
// so stale rows reach only outputs of their own row.
// With SKIP, blocks that hold no row of [rlo, Tv) are not loaded either.
template <int TT, int NI, int AUX = 0, bool SKIP = false>
__device__ __forceinline__ void latent_stage(const u16 *__restrict__ tile, int Tv, int L, char *lds,
                                             int rlo = 0)
{
    static_assert((NI & (NI - 1)) == 0, "slots per row must be a power of two");
    constexpr int SPR = 32 * NI;                  // 16-byte slots per staged row
    const int l = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const __amdgpu_buffer_rsrc_t r = lt_rsrc(tile, latent_tile_bytes(Tv < 16 * TT ? Tv : 16 * TT, L));
#pragma unroll
    for (int k = 0; k < TT * NI; ++k) {
        const int m = KW * k + w;                 // 1 KB block of the staging area
        if (SKIP && (64 * m / SPR >= Tv || (64 * m + 63) / SPR < rlo)) continue;   // wave-uniform
        const int slot = 64 * m + l;
        const int row = slot / SPR, c = (slot % SPR) ^ (row & 15);
        const uint32_t off = c < (L >> 3) ? (uint32_t)(row * L + c * 8) * 2u : LT_OOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            r, (__attribute__((address_space(3))) void *)(lds + 1024 * m), 16, off, 0, 0, AUX);
    }
}

// Reads this lane's chunks of the staged tiles in the B-operand layout (the
// same chunks latent_load would load).
template <int TT, int NI>
__device__ __forceinline__ void latent_from_lds(const char *lds, u32x4_t (&sv)[TT][NI])
{
    constexpr int SPR = 32 * NI;
    const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int t = l & 15, g = l >> 4;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int c = 4 * KW * i + 4 * w + g;
            sv[tt][i] = *reinterpret_cast<const u32x4_t *>(lds + ((16 * tt + t) * SPR + (c ^ t)) * 16);
        }
}

// Writes this lane's chunks back into the staged layout (the inverse of
// latent_from_lds; each slot has exactly one owner lane).
template <int TT, int NI>
__device__ __forceinline__ void latent_to_lds(char *lds, const u32x4_t (&sv)[TT][NI])
{
    constexpr int SPR = 32 * NI;
    const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int t = l & 15, g = l >> 4;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int c = 4 * KW * i + 4 * w + g;
            *reinterpret_cast<u32x4_t *>(lds + ((16 * tt + t) * SPR + (c ^ t)) * 16) = sv[tt][i];
        }
}

// Loads this lane's chunks of the norm weight (zeros past the row end).
template <int NI>
__device__ __forceinline__ void latent_load_weight(const u16 *__restrict__ norm_w, int L,
                                                   u32x4_t (&wv)[NI])
{
    const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int g = l >> 4;
    const __amdgpu_buffer_rsrc_t r = lt_rsrc(norm_w, (uint32_t)L * 2u);
#pragma unroll
    for (int i = 0; i < NI; ++i)
        wv[i] = lt_buf_load16(r, (uint32_t)(4 * KW * i + 4 * w + g) * 16u);
}

// The norm weight staged in LDS: its first 512*NI bytes in natural order
// (zeros past the row end), copied by the first max(1, NI/2) waves with one
// 1 KB direct load each instead of NI loads in every wave.  The caller waits
// (vmcnt) and runs a workgroup barrier before weight_from_lds.
template <int NI>
constexpr int weight_stage_bytes() { return NI >= 2 ? 512 * NI : 1024; }

template <int NI>
__device__ __forceinline__ void weight_stage(const u16 *__restrict__ norm_w, int L, char *lds)
{
    const int l = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (w >= weight_stage_bytes<NI>() / 1024) return;
    const __amdgpu_buffer_rsrc_t r = lt_rsrc(norm_w, (uint32_t)L * 2u);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void *)(lds + 1024 * w), 16,
        (uint32_t)(1024 * w + 16 * l), 0, 0, 0);
}

// This lane's chunks of the staged norm weight (what latent_load_weight loads).
template <int NI>
__device__ __forceinline__ void weight_from_lds(const char *lds, u32x4_t (&wv)[NI])
{
    const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int g = l >> 4;
#pragma unroll
    for (int i = 0; i < NI; ++i)
        wv[i] = *reinterpret_cast<const u32x4_t *>(lds + (4 * KW * i + 4 * w + g) * 16);
}

// Adds partials 1..P-1 (stride pstride elements) in fp32, p ascending, and
// stores the sum as bf16.  Nothing to do for one partial.  Each partial's
// NI chunks are loaded together, so a pass costs one memory round trip.
template <int NI>
__device__ __forceinline__ void latent_sum(const u16 *__restrict__ tile, int64_t pstride, int P,
                                           int Tv, int L, u32x4_t (&sv)[NI])
{
    if (P <= 1) return;
    uint32_t off[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) off[i] = latent_offset(i, L);
    float s[NI][8];
#pragma unroll
    for (int i = 0; i < NI; ++i) lt_unpack8(sv[i], s[i]);
    for (int p = 1; p < P; ++p) {
        const __amdgpu_buffer_rsrc_t r = lt_rsrc(tile + (int64_t)p * pstride, latent_tile_bytes(Tv, L));
        u32x4_t x[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) x[i] = lt_buf_load16(r, off[i]);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            float f[8];
            lt_unpack8(x[i], f);
#pragma unroll
            for (int e = 0; e < 8; ++e) s[i][e] = s[i][e] + f[e];
        }
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) sv[i] = lt_pack8(s[i]);
}

// One-hot A operands that turn v_mfma_f32_16x16x32_bf16 into the norm-weight
// scaling of one 32-wide K step: with A0/A1 in the A slot and a latent tile S
// (B layout) in the B slot, D0[m][t] = w[k] * s[t][k] for k = 8*(m/4) + m%4
// and D1 the same for k + 4.  Every output is one exact bf16 x bf16 product,
// and the output layout (lane: token lane%16, rows 4*(lane/16)..+3) gives each
// lane k = 8g..8g+3 from D0 and 8g+4..8g+7 from D1 (g = lane/16): exactly the
// eight consecutive k its B-layout chunk holds.  Lane (m = lane%16, g) of A0
// keeps element m%4 of its weight chunk when g == m/4, A1 element 4 + m%4.
__device__ __forceinline__ void latent_weight_operands(const u32x4_t w, bf16x8_t &a0, bf16x8_t &a1)
{
    const int l = threadIdx.x & 63;
    const int m = l & 15, g = l >> 4;
    const bool mine = g == (m >> 2);
    const uint32_t keep = (m & 1) ? 0xFFFF0000u : 0x0000FFFFu;
    const int d = (m & 3) >> 1;                 // dword of element m % 4
    u32x4_t v0 = {0u, 0u, 0u, 0u}, v1 = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        v0[k] = (mine && d == k) ? (w[k] & keep) : 0u;
        v1[2 + k] = (mine && d == k) ? (w[2 + k] & keep) : 0u;
    }
    a0 = __builtin_bit_cast(bf16x8_t, v0);
    a1 = __builtin_bit_cast(bf16x8_t, v1);
}

// RMSNorm of TT tiles in place: y = bf16((s * w) * rsqrt(mean(s^2) + eps)),
// with s * w exact (one bf16 x bf16 product, formed on the matrix cores by
// the one-hot operands above) and one fp32 rounding before the bf16 one.
// `red` is LDS scratch of TT * KW * 16 floats.  One workgroup barrier for all
// tiles: every thread of the workgroup must call it.
template <int TT, int NI>
__device__ __forceinline__ void latent_norm(u32x4_t (&sv)[TT][NI], const u32x4_t (&wv)[NI],
                                            float eps, float inv_L, float (*red)[KW * 16])
{
    const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int t = l & 15;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        f32x4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const bf16x8_t s = __builtin_bit_cast(bf16x8_t, sv[tt][i]);
            d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(s, s, d, 0, 0, 0);
        }
        // D[t][t] sits in lane 16*(t/4) + t, element t % 4
        if ((l >> 4) == (t >> 2)) red[tt][w * 16 + t] = d[t & 3];
    }
    bf16x8_t a0[NI], a1[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) latent_weight_operands(wv[i], a0[i], a1[i]);
    __builtin_amdgcn_s_waitcnt(lt_vm_lgkm0(63));   // LDS only: loads may stay in flight
    lt_lds_barrier();
    const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        float total = red[tt][t];
#pragma unroll
        for (int v = 1; v < KW; ++v) total = total + red[tt][v * 16 + t];
        const float rs = lt_inv_rms(total, inv_L, eps);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const bf16x8_t s = __builtin_bit_cast(bf16x8_t, sv[tt][i]);
            const f32x4_t p0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[i], s, zero, 0, 0, 0);
            const f32x4_t p1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[i], s, zero, 0, 0, 0);
            u32x4_t y;
            y[0] = lt_pack2(p0[0] * rs, p0[1] * rs);
            y[1] = lt_pack2(p0[2] * rs, p0[3] * rs);
            y[2] = lt_pack2(p1[0] * rs, p1[1] * rs);
            y[3] = lt_pack2(p1[2] * rs, p1[3] * rs);
            sv[tt][i] = y;
        }
    }
}

}  // namespace lt
