// plan.hip -- varlen scheduling plan for the prefill: order the N packed
// sequences by length, longest first (ties by index), into a device table.
//
// The prefill runs one work-group per (sequence, head, value tile) and each
// work-group walks its sequence chunk by chunk, so chunks never straddle a
// cu_seqlens boundary by construction.  What the plan adds is the dispatch
// order: launching the longest sequences first (longest-processing-time
// first) keeps a long sequence from starting last and stretching the whole
// launch.  The plan is computed on the device from cu_seqlens, so the host
// never synchronises to read the lengths.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

// Above this many sequences the quadratic ranking is skipped and the plan is
// the identity order (the kernel's cost stays bounded).
constexpr int kPlanMaxSorted = 16384;

__global__ __launch_bounds__(256)
void plan_order_kernel(const int32_t* __restrict__ cu, int32_t N, int32_t* __restrict__ order)
{
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (N > kPlanMaxSorted) {
        if (i < N) order[i] = i;
        return;
    }
    __shared__ int32_t lens[1024];
    const int32_t li = (i < N) ? cu[i + 1] - cu[i] : 0;
    int rank = 0;
    for (int base = 0; base < N; base += 1024) {
        __syncthreads();
        for (int j = threadIdx.x; j < 1024; j += 256) {
            const int jj = base + j;
            lens[j] = (jj < N) ? cu[jj + 1] - cu[jj] : 0;
        }
        __syncthreads();
        const int cnt = min(1024, N - base);
        if (i < N) {
            for (int j = 0; j < cnt; ++j) {
                const int32_t lj = lens[j];
                rank += (lj > li) || (lj == li && base + j < i);
            }
        }
    }
    if (i < N) order[rank] = i;   // ranks form a permutation of 0..N-1
}

hipError_t launch_plan(const PrefillArgs& a, hipStream_t stream) {
    const unsigned blocks = static_cast<unsigned>((a.N + 255) / 256);
    hipLaunchKernelGGL(plan_order_kernel, dim3(blocks), dim3(256), 0, stream,
                       a.cu_seqlens, a.N, a.order);
    return hipGetLastError();
}

}  // namespace kda
