// lt_internal.h -- launchers of the tail's kernels (library-internal).
//
// Every launcher takes device pointers that the C-ABI layer has already
// validated (sizes, alignment, window), so the kernels can rely on:
//   L % 8 == 0, 8 <= L <= LT_MAX_L; rows of partials / latent / W 16-byte
//   aligned; T, n >= 1; outn = out + c0 with row stride ld_out.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lt {

// Optional residual update after the tail: resid[t][j] = bf16(prefix[t][j] +
// out'[t][j]) on the window (pointers already offset by c0, row strides in
// elements).  resid may equal prefix (same stride).
struct Resid {
    const uint16_t *prefix;
    int64_t ld_prefix;
    uint16_t *resid;
    int64_t ld_resid;
};

// Weight-streaming path: fused partial sum + RMSNorm + projection +
// beta-add for tokens [0, T) of `part` (T <= 64; partial stride `pstride`).
hipError_t launch_skinny(const uint16_t *part, int64_t pstride, int P, int T, int L,
                         const uint16_t *norm_w, float eps, const uint16_t *Wn, int n,
                         uint16_t *outn, int64_t ld_out, const Resid *res, hipStream_t stream);

// Largest token count one skinny launch handles for latent width L.
int skinny_tokens_per_launch(int L);

// Partial sum + RMSNorm into a packed [T][L] bf16 latent (y may be part
// itself when P == 1).
hipError_t launch_sum_rmsnorm(const uint16_t *part, int64_t pstride, int P, int64_t T,
                              int L, const uint16_t *norm_w, float eps, uint16_t *y,
                              hipStream_t stream);

// out[t][j] = bf16(out[t][j] + sum_k y[t][k] * Wn[j][k]) for t < T, j < n
// (and the residual update when res is not NULL).
hipError_t launch_gemm(const uint16_t *y, int64_t T, int L, const uint16_t *Wn, int n,
                       uint16_t *outn, int64_t ld_out, const Resid *res, hipStream_t stream);

// The GEMM on 256 x 128 tiles with a ping-pong wave schedule (no residual
// form; `out` 16-byte aligned with ld_out % 8 == 0).  Used where the tile
// count is within [PP_MIN_TILES, PP_MAX_TILES] (about one round of such
// tiles) and there are at least four K stages; gemm_pp_rows() gives the
// tile's W rows (256), or 0 where it is not used.  The window's top, 252
// tiles: T = 1100 / 1152 at n = 7168 (252 tiles) took 27.8 / 28.3 against
// 28.8 / 29.3 us per call on the shapes below; the 896-column shard at
// T = 8191 (256 tiles, the last column tile half full) was no better there.
constexpr int PP_MIN_TILES = 140, PP_MAX_TILES = 252;
int gemm_pp_rows(int64_t T, int L, int n, int64_t ld_out);
hipError_t launch_gemm_pp(const uint16_t *y, int64_t T, int L, const uint16_t *Wn, int n,
                          uint16_t *outn, int64_t ld_out, hipStream_t stream);

// AttnRes zero-block path: per token row t < T of width H (H % 8 == 0,
// H <= 8192, rows 16-byte aligned), p' = bf16(prefix + delta) (delta may be
// NULL), written back to prefix when delta is set and to block_slot +
// t * block_stride when block_slot is set; out = bf16(p' * rsqrt(mean p'^2 +
// eps) * w) when norm_w is set, else p'.
hipError_t launch_attn_res(uint16_t *prefix, const uint16_t *delta, int64_t T, int H,
                           uint16_t *block_slot, int64_t block_stride, const uint16_t *norm_w,
                           float eps, uint16_t *out, hipStream_t stream);

}  // namespace lt
