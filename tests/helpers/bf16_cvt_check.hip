// Every fp32 bit pattern through gfx950's v_cvt_pk_bf16_f32 (the packing
// the Newton-Schulz B X kernel stores X' with) against the integer
// round-to-nearest-even that the write-back kernels use: prints the number
// of non-NaN inputs where they differ and of NaN inputs that do not give a
// NaN; exits 0 only if both are zero.  Test helper, built by
// tests/helpers/build.py; run by tests/test_gpu_bf16_pack.py.
#include <hip/hip_runtime.h>

#include <cstdio>

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ unsigned rne_bits(unsigned u) {
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__global__ void check(unsigned long long *counts, unsigned *example) {
    const unsigned long long n = 1ull << 32;
    const unsigned long long stride = (unsigned long long)gridDim.x * blockDim.x;
    for (unsigned long long i = (unsigned long long)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += stride) {
        const unsigned u = (unsigned)i;
        const float f = __builtin_bit_cast(float, u);
        const unsigned h =
            __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{f, 0.0f}, bf16x2)) & 0xffffu;
        if ((u & 0x7fffffffu) > 0x7f800000u) {
            if ((h & 0x7f80u) != 0x7f80u || (h & 0x7fu) == 0u) atomicAdd(&counts[1], 1ull);
        } else if (h != rne_bits(u)) {
            atomicAdd(&counts[0], 1ull);
            atomicExch(example, u);
        }
    }
}

int main() {
    unsigned long long *counts = nullptr;
    unsigned *example = nullptr;
    if (hipMalloc(&counts, 2 * sizeof(unsigned long long)) != hipSuccess ||
        hipMalloc(&example, sizeof(unsigned)) != hipSuccess ||
        hipMemset(counts, 0, 2 * sizeof(unsigned long long)) != hipSuccess ||
        hipMemset(example, 0, sizeof(unsigned)) != hipSuccess)
        return 2;
    hipLaunchKernelGGL(check, dim3(4096), dim3(256), 0, 0, counts, example);
    unsigned long long h[2] = {0, 0};
    unsigned ex = 0;
    if (hipGetLastError() != hipSuccess ||
        hipMemcpy(h, counts, sizeof(h), hipMemcpyDeviceToHost) != hipSuccess ||
        hipMemcpy(&ex, example, sizeof(ex), hipMemcpyDeviceToHost) != hipSuccess)
        return 2;
    std::printf("non-NaN differences %llu (e.g. 0x%08x); NaN inputs not giving a NaN %llu\n", h[0],
                ex, h[1]);
    return h[0] == 0 && h[1] == 0 ? 0 : 1;
}
