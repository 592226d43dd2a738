// k_probe.hip -- measurement probes for the benchmark (libltprobe.so).
//
// Not part of the tail's C ABI.  They measure what any kernel of a given
// launch shape costs on this GPU, so that the weight-streaming kernel's time
// can be set against the floor of a single launch that does nothing but
// stream the same bytes:
//   ltp_stream -- every workgroup copies its contiguous share of `src` into
//                 LDS with 16-byte direct-to-LDS loads (all issued up front,
//                 1 KB per wave instruction, non-temporal like the W stream
//                 of the weight-streaming kernel), waits for them and exits;
//   ltp_empty  -- the same launch shape with an empty body.
// Both return hipLaunchKernel's status.
#include <hip/hip_runtime.h>
#include <stdint.h>

#define LTP_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr int kMaxBlockBytes = 64 * 1024;   // LDS per workgroup

__global__ void k_probe_stream(const char *__restrict__ src, uint32_t block_bytes)
{
    __shared__ __attribute__((aligned(1024))) char lds[kMaxBlockBytes];
    const char *base = src + (size_t)blockIdx.x * block_bytes;
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(base), (short)0, (int)block_bytes,
                                          0x00020000);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l = threadIdx.x & 63;
    const int nw = blockDim.x >> 6;
    for (uint32_t k = (uint32_t)w * 1024u; k < block_bytes; k += (uint32_t)nw * 1024u)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            r, (__attribute__((address_space(3))) void *)(lds + k), 16, (uint32_t)(16 * l), (int)k,
            0, 2);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
}

__global__ void k_probe_empty() {}

}  // namespace

// Streams nwg * block_bytes bytes of src (block_bytes a multiple of 1024, at
// most 64 KiB) with nwg workgroups of nthreads threads (a multiple of 64).
LTP_API int ltp_stream(const void *src, uint32_t block_bytes, uint32_t nwg, uint32_t nthreads,
                       void *stream)
{
    if (!src || block_bytes == 0 || block_bytes % 1024 || block_bytes > (uint32_t)kMaxBlockBytes ||
        nwg == 0 || nthreads == 0 || nthreads % 64 || nthreads > 1024)
        return (int)hipErrorInvalidValue;
    const char *p = static_cast<const char *>(src);
    void *args[] = {&p, &block_bytes};
    return (int)hipLaunchKernel(reinterpret_cast<const void *>(&k_probe_stream), dim3(nwg),
                                dim3(nthreads), args, 0, reinterpret_cast<hipStream_t>(stream));
}

LTP_API int ltp_empty(uint32_t nwg, uint32_t nthreads, void *stream)
{
    if (nwg == 0 || nthreads == 0 || nthreads > 1024) return (int)hipErrorInvalidValue;
    return (int)hipLaunchKernel(reinterpret_cast<const void *>(&k_probe_empty), dim3(nwg),
                                dim3(nthreads), nullptr, 0, reinterpret_cast<hipStream_t>(stream));
}
