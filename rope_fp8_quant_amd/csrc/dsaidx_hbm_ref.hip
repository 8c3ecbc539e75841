// Reference HBM streams for gfx950: what plain kernels reach with the access
// pattern of the preparation kernel -- 16-byte nontemporal loads and stores by
// every lane, one-shot grid of 256-thread workgroups, four vectors per thread
// with all loads issued before any store.  Three shapes: copy (read and write
// the same byte count), read-only and write-only.  They measure the
// achievable fraction of the HBM peak for a given read/write mix; they are
// not part of the indexer path.
#include "dsaidx_internal.h"

namespace dsaidx {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kVecPerThread = 4;
constexpr int64_t kVecPerBlock = (int64_t)kThreads * kVecPerThread;

__global__ __launch_bounds__(kThreads) void hbm_copy_kernel(const u32x4* src, u32x4* dst,
                                                            int64_t n) {
    const int64_t base = (int64_t)blockIdx.x * kVecPerBlock + threadIdx.x;
    u32x4 v[kVecPerThread];
#pragma unroll
    for (int i = 0; i < kVecPerThread; ++i) {
        const int64_t at = base + (int64_t)i * kThreads;
        if (at < n) v[i] = __builtin_nontemporal_load(src + at);
    }
#pragma unroll
    for (int i = 0; i < kVecPerThread; ++i) {
        const int64_t at = base + (int64_t)i * kThreads;
        if (at < n) __builtin_nontemporal_store(v[i], dst + at);
    }
}

// Reads every vector and folds it into one word per thread; the word is
// stored only when it equals `never` (the caller passes a value the data
// cannot fold to), so the loads cannot be removed and nothing is written.
__global__ __launch_bounds__(kThreads) void hbm_read_kernel(const u32x4* src, u32x4* sink,
                                                            int64_t n, uint32_t never) {
    const int64_t base = (int64_t)blockIdx.x * kVecPerBlock + threadIdx.x;
    uint32_t acc = 0;
#pragma unroll
    for (int i = 0; i < kVecPerThread; ++i) {
        const int64_t at = base + (int64_t)i * kThreads;
        if (at < n) {
            const u32x4 v = __builtin_nontemporal_load(src + at);
            acc ^= v.x ^ v.y ^ v.z ^ v.w;
        }
    }
    if (acc == never) {
        const u32x4 w = {acc, acc, acc, acc};
        sink[0] = w;
    }
}

__global__ __launch_bounds__(kThreads) void hbm_write_kernel(u32x4* dst, int64_t n,
                                                             uint32_t value) {
    const int64_t base = (int64_t)blockIdx.x * kVecPerBlock + threadIdx.x;
    const u32x4 w = {value, value, value, value};
#pragma unroll
    for (int i = 0; i < kVecPerThread; ++i) {
        const int64_t at = base + (int64_t)i * kThreads;
        if (at < n) __builtin_nontemporal_store(w, dst + at);
    }
}

}  // namespace

hipError_t launch_hbm_stream(int mode, const void* src, void* dst, int64_t vectors,
                             uint32_t word, hipStream_t stream) {
    const int64_t blocks = (vectors + kVecPerBlock - 1) / kVecPerBlock;
    const u32x4* s = reinterpret_cast<const u32x4*>(src);
    u32x4* d = reinterpret_cast<u32x4*>(dst);
    if (mode == 0) {
        void* args[] = {&s, &d, &vectors};
        return hipLaunchKernel(reinterpret_cast<const void*>(&hbm_copy_kernel), dim3((unsigned)blocks),
                               dim3(kThreads), args, 0, stream);
    }
    if (mode == 1) {
        void* args[] = {&s, &d, &vectors, &word};
        return hipLaunchKernel(reinterpret_cast<const void*>(&hbm_read_kernel), dim3((unsigned)blocks),
                               dim3(kThreads), args, 0, stream);
    }
    void* args[] = {&d, &vectors, &word};
    return hipLaunchKernel(reinterpret_cast<const void*>(&hbm_write_kernel), dim3((unsigned)blocks),
                           dim3(kThreads), args, 0, stream);
}

}  // namespace dsaidx
