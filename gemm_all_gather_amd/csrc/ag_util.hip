// Small utility kernels of the library.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ag_internal.h"

namespace ag {
namespace {
// Zeroes words [0, n) of p (the tile counters of a heap: 16 words per rank), one thread per word.
__global__ __launch_bounds__(256) void clear_words_kernel(uint32_t* p, uint32_t n)
{
    const uint32_t i = blockIdx.x * 256u + threadIdx.x;
    if (i < n) p[i] = 0u;
}
}  // namespace

hipError_t clear_counters(uint32_t* counters, uint32_t words, hipStream_t stream)
{
    if (counters == nullptr || words == 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(clear_words_kernel, dim3((words + 255u) / 256u), dim3(256), 0, stream, counters, words);
    return hipGetLastError();
}

}  // namespace ag
