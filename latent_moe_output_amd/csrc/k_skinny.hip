// k_skinny.hip -- weight-streaming tail for small token counts (decode).
//
// One launch does the whole tail for up to 64 tokens: partial sum, bf16
// storage round trip, RMSNorm and the windowed projection with its beta-add
// ([PR50383 Key source snippets, `_shard_up_proj_tail`]: reduce, norm,
// narrow, addmm_).  At these token counts the work is bound by reading the
// W window from HBM once, so the kernel is built around that stream:
//
//  * A workgroup owns RW rows of the W window (output columns), RW <= 16*JT:
//    the window is cut into about one row block per compute unit, so every CU
//    streams an equal share and the partial tile and norm weight, which every
//    workgroup needs, are fetched as few times as possible.  Its KW waves
//    split the latent width: chunk c (8 elements) belongs to wave
//    (c / 4) % KW, lane group c % 4, step c / (4*KW).  Each lane's W chunks
//    are needed in the A-operand layout of v_mfma_f32_16x16x32_bf16 (row =
//    lane % 16, 8 consecutive k per lane).  While the latent is at most 1024
//    wide (WS) the block's W rows are copied into LDS as whole lines by
//    direct-to-LDS loads, in the staged layout of lt_latent.h, and read back
//    in that layout: a load in the operand layout touches 16 rows at one
//    64-byte offset, which the vector L1 moves at about a third of the rate
//    of whole lines (T = 1: 5.41 vs 5.69 us back to back, bit-identical).
//    For 33..64 tokens with one partial the latent is staged two tiles at a
//    time through one 64 KB area (tiles 2 and 3 are fetched once tiles 0 and
//    1 are in registers, after the W rows), so W fits in LDS beside it; wider
//    latents leave no room and load W straight into registers.
//  * The out values the epilogue will add to are fetched first, then the
//    latent (one partial: copied into LDS as whole lines and read back in the
//    operand layout, see lt_latent.h, only the 1 KB blocks that hold tokens
//    below T, with the norm weight copied once per workgroup; several: loaded
//    and summed in registers before anything else is issued, so the sum's
//    waits never drain the W stream), then all of the workgroup's W chunks:
//    the whole W share is in flight while the latent is normalised, and the
//    read-modify-write of the window adds no memory round trip at the end.
//    Every load instruction issued ahead of W delays the W stream by the
//    time the CU's address unit spends on it; loading only the tokens that
//    exist and the norm weight once took T = 1 from 5.41 to 5.17 us and
//    T = 32 from 7.14 to 6.55.  W is read exactly once per call, so its
//    loads are marked non-temporal (T = 16: 5.83 vs 6.02 us back to back,
//    T = 64: 9.9 vs 10.6).
//  * The latent is built in registers in the B-operand layout (token = lane
//    % 16) by the shared tile code of lt_latent.h; splitting K over KW waves
//    keeps each lane's share of the RMSNorm arithmetic small, and the norm's
//    barrier leaves the W loads in flight.  Tokens ride the MFMA's 16-wide N
//    dimension; the idle columns of a partly filled token tile cost nothing
//    that matters here, the matrix cores are far from busy.
//  * The KW per-wave partial products are added in LDS in wave order and
//    written with one bf16 rounding onto the window, with device-scope
//    stores (lt_store8_dev; back to back T = 1 5.09 -> 4.83 us, T = 16
//    5.43 -> 5.11, T = 64 9.54 -> 8.96: the store is the call's last round
//    trip, and a device-coherent one completes sooner).  The residual form (RES)
//    also writes bf16(prefix + out') with the prefix prefetched alongside
//    `out` ([PR50593 Key source snippets, `forward_attn_residual`]).
//
// Every element's accumulation order depends only on (T, L), never on c0 or
// n, so column shards reproduce the full-window result bit for bit.
#include "lt_internal.h"
#include "lt_latent.h"
#include "lt_launch.h"
#include "lt_store.h"

namespace lt {
namespace {

// Argument order: what the loads ahead of the W stream need (the out
// prefetch, the staged latent, the norm weight, the W rows) fills the 14
// argument dwords that are preloaded into scalar registers at wave launch;
// rw_vec packs the rows per block (bits 0..7) and the 8-byte out flag (bit 8).
template <int NI, int TT, int JT, bool RES, bool ST, bool WS>
__global__ __launch_bounds__(64 * KW) void k_skinny(const u16 *__restrict__ part,
                                                    const u16 *__restrict__ Wn,
                                                    u16 *__restrict__ outn,
                                                    const u16 *__restrict__ norm_w, int64_t ld_out,
                                                    int T, int L, int n, int rw_vec,
                                                    int64_t pstride, int P, float eps, float inv_L,
                                                    const u16 *prefn, int64_t ld_pre, u16 *resn,
                                                    int64_t ld_res)
{
    const int RW = rw_vec & 0xFF, vec8 = rw_vec >> 8;
    static_assert(JT * TT <= KW, "one epilogue fragment per wave");
    const int l = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = l & 15;
    const int g = l >> 4;
    const int nchunk = L >> 3;
    const int j0 = blockIdx.x * RW;
    const int rows = min(RW, n - j0);   // 1..RW rows of this block are in the window

    __shared__ float red_ss[TT][KW * 16];
    // The staged latent tiles (one partial, ST) and, once the latent is in
    // registers, the per-wave partial products share one LDS area.
    // SPLIT: four token tiles with one partial are staged two at a time
    // through one half-size area, so that W fits in LDS next to them
    constexpr bool SPLIT = ST && TT == 4;
    constexpr int TS = SPLIT ? 2 : TT;          // tiles per staging pass
    constexpr int STAGE_BYTES = ST ? latent_stage_bytes<TS, NI>() : 0;
    constexpr int RED_BYTES = KW * JT * TT * 64 * 16;
    __shared__ __attribute__((aligned(1024))) char lds_u[STAGE_BYTES > RED_BYTES ? STAGE_BYTES : RED_BYTES];
    auto red_acc = reinterpret_cast<f32x4_t (*)[JT * TT][64]>(lds_u);
    // W rows staged as whole lines (WS), in the same layout as the latent
    __shared__ __attribute__((aligned(1024))) char lds_w[WS ? latent_stage_bytes<JT, NI>() : 16];
    __shared__ __attribute__((aligned(1024))) char lds_nw[ST ? weight_stage_bytes<NI>() : 16];

    // this wave's epilogue fragment (w < JT*TT): token tile w % TT, row tile w / TT
    const bool has_epi = w < JT * TT;
    const int tte = w % TT, jte = w / TT;
    const int te = 16 * tte + r, jl = 16 * jte + 4 * g;   // token, local row
    const bool out_vec = has_epi && te < T && vec8 && jl + 4 <= rows;

    // 1. the out values the epilogue adds to (first, so that every later wait
    //    counts the same loads in every wave), the latent (one partial: copied
    //    into LDS as whole lines; several: loaded and summed in registers
    //    before anything else is issued, so the sum's waits cover partial
    //    loads only), the norm weight, then all of this block's W rows
    u32x2_t opre = {0u, 0u}, ppre = {0u, 0u};
    if (out_vec) {
        opre = *reinterpret_cast<const u32x2_t *>(outn + (int64_t)te * ld_out + j0 + jl);
        if constexpr (RES) ppre = *reinterpret_cast<const u32x2_t *>(prefn + (int64_t)te * ld_pre + j0 + jl);
    }
    u32x4_t sv[TT][NI], wv[NI];
    if constexpr (ST) {   // token rows past T are never stored: skip them
        latent_stage<TS, NI, 0, true>(part, T, L, lds_u);
        if (norm_w) weight_stage<NI>(norm_w, L, lds_nw);
    } else {
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) latent_load(part + (int64_t)16 * tt * L, T - 16 * tt, L, sv[tt]);
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
            latent_sum(part + (int64_t)16 * tt * L, pstride, P, T - 16 * tt, L, sv[tt]);
        if (norm_w) latent_load_weight(norm_w, L, wv);
    }
    u32x4_t wa[JT][NI];
    if constexpr (WS) {
        latent_stage<JT, NI, LT_NT>(Wn + (int64_t)j0 * L, rows, L, lds_w);
    } else {
        const __amdgpu_buffer_rsrc_t rw = lt_rsrc(Wn + (int64_t)j0 * L, (uint32_t)(rows * L) * 2u);
#pragma unroll
        for (int jt = 0; jt < JT; ++jt)
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int c = 4 * KW * i + 4 * w + g;
                const uint32_t off =
                    c < nchunk ? (uint32_t)((16 * jt + r) * L + c * 8) * 2u : LT_OOB;
                wa[jt][i] = lt_buf_load16_nt(rw, off);
            }
    }
    if constexpr (ST) {
        // the staged tiles and norm weight have landed once at most the W
        // loads issued after them are in flight
        __builtin_amdgcn_s_waitcnt(lt_vm_lgkm0(JT * NI));
        lt_lds_barrier();
        latent_from_lds<TS, NI>(lds_u, *reinterpret_cast<u32x4_t (*)[TS][NI]>(&sv[0]));
        if (norm_w) weight_from_lds<NI>(lds_nw, wv);
        if (SPLIT || !norm_w) {   // the staging area is reused (tiles 2, 3 / the products)
            __builtin_amdgcn_s_waitcnt(lt_vm_lgkm0(63));
            lt_lds_barrier();
        }
        // tiles 2 and 3 follow the W rows; the first two tiles' norm runs
        // while both are in flight
        if constexpr (SPLIT)
            latent_stage<2, NI, 0, true>(part + (int64_t)32 * L, T - 32, L, lds_u);
    }

    // 2. RMSNorm (its barrier waits for LDS only; W stays in flight)
    if constexpr (SPLIT) {
        if (norm_w)
            latent_norm<2, NI>(*reinterpret_cast<u32x4_t (*)[2][NI]>(&sv[0]), wv, eps, inv_L, red_ss);
        __builtin_amdgcn_s_waitcnt(lt_vm_lgkm0(0));   // tiles 2, 3 and the W rows
        lt_lds_barrier();
        latent_from_lds<2, NI>(lds_u, *reinterpret_cast<u32x4_t (*)[2][NI]>(&sv[2]));
        if (norm_w)
            latent_norm<2, NI>(*reinterpret_cast<u32x4_t (*)[2][NI]>(&sv[2]), wv, eps, inv_L, red_ss + 2);
        else {   // the products below reuse the staging area
            __builtin_amdgcn_s_waitcnt(lt_vm_lgkm0(63));
            lt_lds_barrier();
        }
    } else {
        if (norm_w) latent_norm<TT, NI>(sv, wv, eps, inv_L, red_ss);
    }
    if constexpr (WS) {   // every wave's share of the W rows has landed
        if constexpr (!SPLIT) {
            __builtin_amdgcn_s_waitcnt(lt_vm_lgkm0(0));
            lt_lds_barrier();
        }
        latent_from_lds<JT, NI>(lds_w, wa);
    }

    // 3. projection on the matrix cores: D[j][t] += W[j][k] * y[t][k]
    f32x4_t acc[JT][TT];
#pragma unroll
    for (int jt = 0; jt < JT; ++jt)
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) acc[jt][tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) {
            const bf16x8_t a = __builtin_bit_cast(bf16x8_t, wa[jt][i]);
#pragma unroll
            for (int tt = 0; tt < TT; ++tt)
                acc[jt][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    a, __builtin_bit_cast(bf16x8_t, sv[tt][i]), acc[jt][tt], 0, 0, 0);
        }

    // 4. add the KW waves' partial products in wave order, beta-add the window
#pragma unroll
    for (int jt = 0; jt < JT; ++jt)
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) red_acc[w][jt * TT + tt][l] = acc[jt][tt];
    __builtin_amdgcn_s_waitcnt(lt_vm_lgkm0(63));   // LDS only: the out values may still fly
    lt_lds_barrier();
    if (!has_epi || te >= T) return;
    f32x4_t d = red_acc[0][w][l];
#pragma unroll
    for (int v = 1; v < KW; ++v) d = d + red_acc[v][w][l];
    u16 *o = outn + (int64_t)te * ld_out + j0 + jl;   // D column = lane % 16 (token),
    if (out_vec) {                                  // rows 4*(lane/16) + 0..3 (columns)
        u32x2_t nv;
        nv[0] = lt_pack2(lt_bf_lo(opre[0]) + d[0], lt_bf_hi(opre[0]) + d[1]);
        nv[1] = lt_pack2(lt_bf_lo(opre[1]) + d[2], lt_bf_hi(opre[1]) + d[3]);
        lt_store8_dev(o, nv);
        if constexpr (RES) {
            u32x2_t rv;
#pragma unroll
            for (int e = 0; e < 2; ++e)
                rv[e] = lt_pack2(lt_bf_lo(ppre[e]) + lt_bf_lo(nv[e]), lt_bf_hi(ppre[e]) + lt_bf_hi(nv[e]));
            lt_store8_dev(resn + (int64_t)te * ld_res + j0 + jl, rv);
        }
    } else {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            if (jl + a < rows) {
                const float v = lt_bf_lo((uint32_t)o[a]) + d[a];
                const u16 onew = (u16)(lt_pack2(v, 0.f) & 0xFFFFu);
                lt_store2_dev(o + a, onew);
                if constexpr (RES) {
                    const int64_t jj = j0 + jl + a;
                    const float r = lt_bf_lo((uint32_t)prefn[(int64_t)te * ld_pre + jj]) +
                                    lt_bf_lo((uint32_t)onew);
                    lt_store2_dev(resn + (int64_t)te * ld_res + jj, (u16)(lt_pack2(r, 0.f) & 0xFFFFu));
                }
            }
        }
    }
}

// Rows of the window per workgroup: about one block per compute unit, a
// multiple of 4 (the epilogue's column group), at most 32 (two MFMA tiles).
int rows_per_block(int n)
{
    constexpr int CUS = 256;
    const int rw = ((n + CUS - 1) / CUS + 3) / 4 * 4;
    return rw < 4 ? 4 : (rw > 32 ? 32 : rw);
}

template <int NI, int TT, int JT>
hipError_t launch_nt(const u16 *part, int64_t pstride, int P, int T, int L, const u16 *norm_w,
                     float eps, const u16 *Wn, int n, int RW, u16 *outn, int64_t ld_out, int vec8,
                     const Resid *res, hipStream_t stream)
{
    const dim3 grid((n + RW - 1) / RW), block(64 * KW);
    const u16 *pre = res ? res->prefix : nullptr;
    u16 *rsd = res ? res->resid : nullptr;
    const int64_t ldp = res ? res->ld_prefix : 0, ldr = res ? res->ld_resid : 0;
    // W rows through LDS while the staged latent and W fit in it
    constexpr bool WS = NI <= 4;
#define LT_SKINNY_LAUNCH(R, S)                                                                  \
    launch(&k_skinny<NI, TT, JT, R, S, WS>, grid, block, stream, part, Wn, outn, norm_w, ld_out, T,  \
           L, n, RW | (vec8 << 8), pstride, P, eps, 1.0f / (float)L, pre, ldp, rsd, ldr)
    // one partial: the latent tiles are staged through LDS as whole lines
    hipError_t e;
    if (res) e = P == 1 ? LT_SKINNY_LAUNCH(true, true) : LT_SKINNY_LAUNCH(true, false);
    else e = P == 1 ? LT_SKINNY_LAUNCH(false, true) : LT_SKINNY_LAUNCH(false, false);
#undef LT_SKINNY_LAUNCH
    return e;
}

template <int NI, int JT>
hipError_t launch_jt(const u16 *part, int64_t pstride, int P, int T, int L, const u16 *norm_w,
                     float eps, const u16 *Wn, int n, int RW, u16 *outn, int64_t ld_out, int vec8,
                     const Resid *res, hipStream_t stream)
{
    if (T <= 16)
        return launch_nt<NI, 1, JT>(part, pstride, P, T, L, norm_w, eps, Wn, n, RW, outn, ld_out,
                                    vec8, res, stream);
    if (T <= 32)
        return launch_nt<NI, 2, JT>(part, pstride, P, T, L, norm_w, eps, Wn, n, RW, outn, ld_out,
                                    vec8, res, stream);
    if constexpr (NI <= 4)
        return launch_nt<NI, 4, JT>(part, pstride, P, T, L, norm_w, eps, Wn, n, RW, outn, ld_out,
                                    vec8, res, stream);
    return hipErrorInvalidValue;
}

template <int NI>
hipError_t launch_ni(const u16 *part, int64_t pstride, int P, int T, int L, const u16 *norm_w,
                     float eps, const u16 *Wn, int n, u16 *outn, int64_t ld_out, int vec8,
                     const Resid *res, hipStream_t stream)
{
    const int RW = rows_per_block(n);
    if (RW <= 16)
        return launch_jt<NI, 1>(part, pstride, P, T, L, norm_w, eps, Wn, n, RW, outn, ld_out,
                                vec8, res, stream);
    return launch_jt<NI, 2>(part, pstride, P, T, L, norm_w, eps, Wn, n, RW, outn, ld_out, vec8,
                            res, stream);
}

}  // namespace

int skinny_tokens_per_launch(int L) { return latent_steps(L) > 4 ? 32 : 64; }

hipError_t launch_skinny(const uint16_t *part, int64_t pstride, int P, int T, int L,
                         const uint16_t *norm_w, float eps, const uint16_t *Wn, int n,
                         uint16_t *outn, int64_t ld_out, const Resid *res, hipStream_t stream)
{
    if (T < 1 || T > skinny_tokens_per_launch(L)) return hipErrorInvalidValue;
    auto a8 = [](const void *p, int64_t ld) {
        return (reinterpret_cast<uintptr_t>(p) & 7) == 0 && ld % 4 == 0;
    };
    const int vec8 = a8(outn, ld_out) && (!res || (a8(res->prefix, res->ld_prefix) &&
                                                   a8(res->resid, res->ld_resid)));
    const int ni = latent_steps(L);
    if (ni <= 1) return launch_ni<1>(part, pstride, P, T, L, norm_w, eps, Wn, n, outn, ld_out, vec8, res, stream);
    if (ni <= 2) return launch_ni<2>(part, pstride, P, T, L, norm_w, eps, Wn, n, outn, ld_out, vec8, res, stream);
    if (ni <= 4) return launch_ni<4>(part, pstride, P, T, L, norm_w, eps, Wn, n, outn, ld_out, vec8, res, stream);
    return launch_ni<8>(part, pstride, P, T, L, norm_w, eps, Wn, n, outn, ld_out, vec8, res, stream);
}

}  // namespace lt
