// sampler_gpu.hip -- the categorical byte sampler of sampler.c on the GPU, for
// inputs too large to draw on the host in reasonable time (the 80-block
// model). Holds none of the decode method's arithmetic. Output i is the same
// byte sampler.c draws for stream index start + i: the i-th output of
// SplitMix64 seeded with `key` (Steele, Lea and Flood, OOPSLA 2014), mapped to
// the first category whose cumulative threshold exceeds it.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

__device__ __forceinline__ uint64_t sm64(uint64_t key, uint64_t i) {
    uint64_t z = key + (i + 1) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

constexpr int kPer = 16;  // bytes per thread

__global__ void __launch_bounds__(256) k_categorical(uint64_t key, uint64_t start, uint64_t n,
                                                     const uint8_t *__restrict__ cat_sym,
                                                     const uint64_t *__restrict__ cat_thr, int ncat,
                                                     uint8_t *__restrict__ out) {
    __shared__ uint64_t thr[256];
    __shared__ uint8_t sym[256];
    for (int c = threadIdx.x; c < ncat; c += blockDim.x) {
        thr[c] = cat_thr[c];
        sym[c] = cat_sym[c];
    }
    __syncthreads();
    const uint64_t i0 = ((uint64_t)blockIdx.x * blockDim.x + threadIdx.x) * kPer;
    if (i0 >= n) return;
    const int last = ncat - 1;
    uint8_t v[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const uint64_t u = sm64(key, start + i0 + k);
        int c = 0;
        while (c < last && u >= thr[c]) ++c;
        v[k] = sym[c];
    }
    if (i0 + kPer <= n && ((reinterpret_cast<uintptr_t>(out + i0) & 15u) == 0)) {
        uint4 w;
        w.x = v[0] | (v[1] << 8) | (v[2] << 16) | ((uint32_t)v[3] << 24);
        w.y = v[4] | (v[5] << 8) | (v[6] << 16) | ((uint32_t)v[7] << 24);
        w.z = v[8] | (v[9] << 8) | (v[10] << 16) | ((uint32_t)v[11] << 24);
        w.w = v[12] | (v[13] << 8) | (v[14] << 16) | ((uint32_t)v[15] << 24);
        *reinterpret_cast<uint4 *>(out + i0) = w;
    } else {
        for (int k = 0; k < kPer && i0 + k < n; ++k) out[i0 + k] = v[k];
    }
}

}  // namespace

// Draw n bytes for stream indices start .. start+n-1 into device memory
// d_out. d_cat_sym / d_cat_thr: device copies of the categories (most
// probable first) and their cumulative thresholds on the 2^64 grid, ncat in
// 1..256. stream: a hipStream_t (NULL = the null stream). 0 on success.
extern "C" int synth_categorical_gpu(uint64_t key, uint64_t start, uint64_t n, const uint8_t *d_cat_sym,
                                     const uint64_t *d_cat_thr, int ncat, uint8_t *d_out, void *stream) {
    if (ncat < 1 || ncat > 256 || !d_cat_sym || !d_cat_thr || (!d_out && n)) return -1;
    if (n == 0) return 0;
    const uint64_t threads = (n + kPer - 1) / kPer;
    const uint64_t grid = (threads + 255) / 256;
    if (grid > 0x7FFFFFFFull) return -1;
    hipLaunchKernelGGL(k_categorical, dim3((uint32_t)grid), dim3(256), 0, static_cast<hipStream_t>(stream), key,
                       start, n, d_cat_sym, d_cat_thr, ncat, d_out);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}
