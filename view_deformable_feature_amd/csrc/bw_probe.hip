// Read-bandwidth reference kernel for the benchmark (not part of libdeformagg).
//
// The aggregation kernels read every corner row of every sample through the
// vector memory path (16-byte buffer loads into registers), and most of those
// bytes are served by the vector L1 or the L2, not by HBM.  The benchmark
// compares that delivered rate with what this kernel reaches when it does
// nothing but stream 16-byte loads from a buffer that stays cache-resident:
//   - a buffer of at most 16 KiB stays in each CU's vector L1 (32 KiB);
//   - a buffer of about 2 MiB stays in each XCD's 4 MiB L2 but not in L1.
//
// Each workgroup (256 threads) makes `passes` passes; pass i reads the
// `chunk_vec` 16-byte vectors of chunk (block * 7 + i) mod n_chunks, each
// thread loading vectors tid, tid + 256, ... (one coalesced 4 KiB request per
// wave per step).  The loaded words are XOR-folded into one value per thread,
// stored at the end so the loads cannot be dropped.
//
// Bounds: every index is below n_chunks * chunk_vec, the buffer's vector count
// (checked by the host entry point), and `sink` holds one word per thread.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;

__global__ void __launch_bounds__(kThreads)
read_kernel(const uint4* __restrict__ buf, uint32_t chunk_vec, uint32_t n_chunks, uint32_t passes,
            uint32_t* __restrict__ sink) {
    uint32_t acc = 0;
    for (uint32_t i = 0; i < passes; ++i) {
        const uint32_t chunk = (blockIdx.x * 7u + i) % n_chunks;
        const uint4* p = buf + (size_t)chunk * chunk_vec;
#pragma unroll 8
        for (uint32_t v = threadIdx.x; v < chunk_vec; v += kThreads) {
            const uint4 q = p[v];
            acc ^= q.x ^ q.y ^ q.z ^ q.w;
        }
    }
    sink[(size_t)blockIdx.x * kThreads + threadIdx.x] = acc;
}

}  // namespace

extern "C" __attribute__((visibility("default")))
int bwprobe_read(const void* buf, uint64_t buf_bytes, uint32_t chunk_bytes, uint32_t passes,
                 uint32_t blocks, uint32_t* sink, uint64_t sink_words, void* stream) {
    if (!buf || !sink || chunk_bytes == 0 || chunk_bytes % 16 != 0 || passes == 0 || blocks == 0)
        return 1;
    if ((uintptr_t)buf % 16 != 0 || buf_bytes % chunk_bytes != 0) return 1;
    const uint64_t n_chunks = buf_bytes / chunk_bytes;
    if (n_chunks == 0 || n_chunks > 0xffffffffull) return 1;
    if (sink_words < (uint64_t)blocks * kThreads) return 1;
    hipLaunchKernelGGL(read_kernel, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint4*>(buf), chunk_bytes / 16u, (uint32_t)n_chunks, passes,
                       sink);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
