// Practical HBM ceilings on this GPU, for the traffic mixes of the pooling
// workloads: a kernel that does nothing but stream the same number of bytes
// in the same read/write proportions, with the same kind of stores (16-byte
// streaming stores), timed the way bench.py times the pooling kernels (kernel
// events from hipExtLaunchKernelGGL, an untimed 1 GiB read before every
// launch so no operand is left in the 256 MB last-level cache).
//
// Each launch walks C chunks; chunk c reads the 16-byte units
// [c*R/C, (c+1)*R/C) of one buffer and writes [c*W/C, (c+1)*W/C) of another
// (each bound rounded down to a whole 128-byte line), so reads and writes
// stay in proportion all through the launch, every wavefront's accesses are
// contiguous and no line is written by two chunks.  The written value depends on what
// the thread read, as in the pooling kernels.
//
// Output: one JSON object per case on stdout.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <vector>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 4;                 // units per thread on the larger side

#define CHECK(x)                                                                    \
    do {                                                                            \
        hipError_t e_ = (x);                                                        \
        if (e_ != hipSuccess) {                                                     \
            fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));          \
            return 1;                                                               \
        }                                                                           \
    } while (0)

// Start of chunk c of C over n units, on a 128-byte line (8 units).
__device__ __forceinline__ int64_t chunk_bound(int64_t c, int64_t n, int64_t C) {
    return c >= C ? n : (c * n / C) & ~int64_t(7);
}

// R read units and W write units in C chunks (grid-stride over chunks).
template <bool NT>
__global__ void __launch_bounds__(kThreads)
mix_kernel(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst, int64_t R, int64_t W,
           int64_t C, u32x4 *__restrict__ sink) {
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int64_t c = blockIdx.x; c < C; c += gridDim.x) {
        const int64_t r0 = chunk_bound(c, R, C), r1 = chunk_bound(c + 1, R, C);
        const int64_t w0 = chunk_bound(c, W, C), w1 = chunk_bound(c + 1, W, C);
        for (int64_t r = r0 + threadIdx.x; r < r1; r += kThreads * kUnroll) {
            u32x4 v[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
                v[u] = (r + u * kThreads < r1) ? src[r + u * kThreads] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
        }
        for (int64_t w = w0 + threadIdx.x; w < w1; w += kThreads) {
            u32x4 v = acc;
            v.x ^= (uint32_t)w;
            if (NT)
                __builtin_nontemporal_store(v, dst + w);
            else
                dst[w] = v;
        }
    }
    // keeps the reads live when a case writes nothing
    if (W == 0 && (acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9e3779b9u) sink[threadIdx.x] = acc;
}

__global__ void __launch_bounds__(kThreads)
flush_kernel(const u32x4 *__restrict__ a, int64_t n, u32x4 *__restrict__ sink) {
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * kThreads)
        acc ^= a[i];
    if ((acc.x ^ acc.y) == 0x7f4a7c15u) sink[threadIdx.x] = acc;
}

struct Case {
    const char *name;
    int64_t read_bytes, write_bytes;
    bool nt;
};

}  // namespace

int main() {
    // read/write bytes of the pooling ops (x, y, idx, gy, gx at their storage sizes)
    const Case cases[] = {
        {"read only 1 GiB", int64_t(1) << 30, 0, true},
        {"write only 1 GiB, streaming stores", 0, int64_t(1) << 30, true},
        {"write only 1 GiB, plain stores", 0, int64_t(1) << 30, false},
        {"copy 1 GiB, streaming stores", int64_t(1) << 30, int64_t(1) << 30, true},
        {"fixed_bf16_k2s2.fwd mix", 411041792, 154140672, true},
        {"fixed_f16_k3s2.fwd mix", 205520896, 67184640, true},
        {"fixed_f16_k3s2.bwd mix", 67184640, 205520896, true},
        {"adaptive_f32_large.fwd mix", 536870912, 16056320, true},
        {"adaptive_f32_large.bwd mix", 16056320, 536870912, true},
        {"fixed_bf16_k2s2.bwd mix", 154140672, 411041792, true},
    };
    const int64_t buf_bytes = int64_t(1) << 30;
    u32x4 *src = nullptr, *dst = nullptr, *flush = nullptr, *sink = nullptr;
    CHECK(hipMalloc(&src, buf_bytes));
    CHECK(hipMalloc(&dst, buf_bytes));
    CHECK(hipMalloc(&flush, buf_bytes));
    CHECK(hipMalloc(&sink, kThreads * sizeof(u32x4)));
    CHECK(hipMemset(src, 1, buf_bytes));
    CHECK(hipMemset(dst, 2, buf_bytes));
    CHECK(hipMemset(flush, 3, buf_bytes));
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    hipDeviceProp_t prop;
    CHECK(hipGetDeviceProperties(&prop, 0));
    const int grids[] = {2048, 4096, 8192, 16384};
    const int iters = 20, warm = 3;

    for (const Case &cs : cases) {
        const int64_t R = cs.read_bytes / 16, W = cs.write_bytes / 16;
        if (R * 16 > buf_bytes || W * 16 > buf_bytes) return 2;
        const int64_t big = std::max(R, W);
        const int64_t C = std::max<int64_t>(1, big / (kThreads * kUnroll));
        double best_med = 1e30, best_min = 1e30;
        int best_grid = 0;
        for (int grid : grids) {
            std::vector<float> t;
            for (int it = 0; it < iters + warm; ++it) {
                hipLaunchKernelGGL(flush_kernel, dim3(8192), dim3(kThreads), 0, 0,
                                   (const u32x4 *)flush, buf_bytes / 16, sink);
                CHECK(hipGetLastError());
                if (cs.nt)
                    hipExtLaunchKernelGGL(mix_kernel<true>, dim3(grid), dim3(kThreads), 0, 0, e0, e1,
                                          0, (const u32x4 *)src, dst, R, W, C, sink);
                else
                    hipExtLaunchKernelGGL(mix_kernel<false>, dim3(grid), dim3(kThreads), 0, 0, e0, e1,
                                          0, (const u32x4 *)src, dst, R, W, C, sink);
                CHECK(hipGetLastError());
                CHECK(hipEventSynchronize(e1));
                float ms = 0.f;
                CHECK(hipEventElapsedTime(&ms, e0, e1));
                if (it >= warm) t.push_back(ms * 1e3f);
            }
            std::sort(t.begin(), t.end());
            const double med = t[t.size() / 2];
            if (med < best_med) {
                best_med = med;
                best_min = t[0];
                best_grid = grid;
            }
        }
        const double bytes = double(cs.read_bytes + cs.write_bytes);
        printf("{\"case\": \"%s\", \"read_bytes\": %lld, \"write_bytes\": %lld, \"stores\": \"%s\", "
               "\"grid\": %d, \"us_median\": %.2f, \"us_min\": %.2f, \"GB_s\": %.1f, "
               "\"frac_of_8TBs\": %.4f, \"device\": \"%s\"}\n",
               cs.name, (long long)cs.read_bytes, (long long)cs.write_bytes,
               cs.nt ? "streaming" : "plain", best_grid, best_med, best_min,
               bytes / (best_med * 1e-6) / 1e9, bytes / (best_med * 1e-6) / 8e12, prop.gcnArchName);
        fflush(stdout);
    }
    CHECK(hipFree(src));
    CHECK(hipFree(dst));
    CHECK(hipFree(flush));
    CHECK(hipFree(sink));
    return 0;
}
