// seq_order.hip -- launch order of packed sequences: the (sequence, head)
// slices of a packed prefill are independent and each runs as one
// workgroup, so the launch takes as long as its busiest compute unit.
// Handing the longest sequences out first (the longest-processing-time
// rule of list scheduling) lets the hardware dispatcher fill the later gaps
// with short ones.  The order is a counting sort by chunk count, longest
// first, in one workgroup; sequences of equal bucket come out in any order,
// which changes no result (every slice is computed alone).
#include "la_internal.h"

namespace la {
namespace {

constexpr int kOrderThreads = 1024;
constexpr int kOrderBuckets = 4096;

__global__ __launch_bounds__(kOrderThreads) void seq_order_kernel(const int* cu, int B, int T,
                                                                  int chunk, int maxc, int* order) {
    __shared__ int cnt[kOrderBuckets];
    __shared__ int part[kOrderThreads];
    const int tid = threadIdx.x;
    for (int b = tid; b < kOrderBuckets; b += kOrderThreads) cnt[b] = 0;
    __syncthreads();
    // bucket 0 holds the most chunks; offsets clamped as the chunk kernels do
    auto bucket = [&](int n) {
        const int s0 = min(max(cu[n], 0), T);
        const int s1 = min(max(cu[n + 1], s0), T);
        const int c = min((s1 - s0 + chunk - 1) / chunk, maxc);
        return (int)((long long)(maxc - c) * kOrderBuckets / (maxc + 1));
    };
    for (int n = tid; n < B; n += kOrderThreads) atomicAdd(&cnt[bucket(n)], 1);
    __syncthreads();
    // exclusive prefix over the buckets: each thread its PER consecutive
    // buckets, then an inclusive scan of the thread sums
    constexpr int PER = kOrderBuckets / kOrderThreads;
    int loc[PER];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        loc[i] = sum;
        sum += cnt[tid * PER + i];
    }
    part[tid] = sum;
    __syncthreads();
    for (int off = 1; off < kOrderThreads; off *= 2) {
        const int x = tid >= off ? part[tid - off] : 0;
        __syncthreads();
        part[tid] += x;
        __syncthreads();
    }
    const int base = part[tid] - sum;
#pragma unroll
    for (int i = 0; i < PER; ++i) cnt[tid * PER + i] = base + loc[i];
    __syncthreads();
    // every sequence takes the next free place of its bucket
    for (int n = tid; n < B; n += kOrderThreads) order[atomicAdd(&cnt[bucket(n)], 1)] = n;
}

}  // namespace

hipError_t launch_seq_order(const int* cu_seqlens, int B, int T, int chunk, int max_seqlen,
                            int* order, hipStream_t s) {
    const int maxc = (max_seqlen + chunk - 1) / chunk;
    LA_LAUNCH(seq_order_kernel, dim3(1), dim3(kOrderThreads), s, cu_seqlens, B, T, chunk,
                       maxc, order);
    return hipGetLastError();
}

}  // namespace la
