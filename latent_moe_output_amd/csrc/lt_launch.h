// lt_launch.h -- kernel launch that reports its own status (library-internal).
//
// hipLaunchKernelGGL returns nothing; its failure is only visible through the
// thread's last-error state, which also holds errors the caller left pending.
// lt_launch calls hipLaunchKernel and returns its status directly, so a
// launcher never has to read (or clear) that state.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <tuple>
#include <utility>

namespace lt {

// Launches kernel `k` on `stream` with `args` converted to its parameter
// types (no dynamic LDS) and returns hipLaunchKernel's status.
template <typename... P, typename... A>
hipError_t launch(void (*k)(P...), dim3 grid, dim3 block, hipStream_t stream, A &&...args)
{
    static_assert(sizeof...(P) == sizeof...(A), "one argument per kernel parameter");
    std::tuple<P...> vals(static_cast<P>(std::forward<A>(args))...);
    void *ptrs[sizeof...(P)];
    std::apply([&ptrs](auto &...v) {
        std::size_t i = 0;
        ((ptrs[i++] = static_cast<void *>(&v)), ...);
    }, vals);
    return hipLaunchKernel(reinterpret_cast<const void *>(k), grid, block, ptrs, 0, stream);
}

}  // namespace lt
