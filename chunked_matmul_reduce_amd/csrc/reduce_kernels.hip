// The HBM-bound kernels of the block besides the tile kernel (gfx950): the
// reduce+epilogue kernel of the chunked schedules, the W -> W^T transpose, and the fill
// kernel that makes the autotuner's inputs on the device.
#include "device_common.h"
#include "mmar_internal.h"

namespace mmar {

// ------------------------------------------------------------------ reduce + epilogue
// The partials are read once and the output written once: both go through nontemporal
// accesses, streamed past the caches (12 % faster on the GPT-2 MLP block's 1.8 GB than
// plain loads and stores, bit-identical).
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void reduce_epilogue_kernel(ReduceArgs a) {
    const int groups_per_row = a.RN / 4;
    const int total = a.RM * groups_per_row;
    const int64_t plane = static_cast<int64_t>(a.RM) * a.RN;
    for (int q = blockIdx.x * 256 + threadIdx.x; q < total; q += gridDim.x * 256) {
        const int r = q / groups_per_row, c = (q - r * groups_per_row) * 4;
        const float* src = a.ws + static_cast<int64_t>(r) * a.RN + c;
        f32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(src));
        for (int p = 1; p < a.P; ++p) {
            const f32x4_t s =
                __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(src + p * plane));
            t.x = __fadd_rn(t.x, s.x);
            t.y = __fadd_rn(t.y, s.y);
            t.z = __fadd_rn(t.z, s.z);
            t.w = __fadd_rn(t.w, s.w);
        }
        const int64_t e = static_cast<int64_t>(a.rm0 + r) * a.N + (a.rn0 + c);
        const uint2 bb = *reinterpret_cast<const uint2*>(a.bias + a.rn0 + c);
        const uint2 rb = *reinterpret_cast<const uint2*>(a.residual + e);
        const float4 o = epilogue4(make_float4(t.x, t.y, t.z, t.w), bb, rb, e, a.drop);
        __builtin_nontemporal_store(f32x4_t{o.x, o.y, o.z, o.w},
                                    reinterpret_cast<f32x4_t*>(a.out + e));
    }
}

// ------------------------------------------------------------------ W -> W^T
// [K, N] -> [N, K] bf16 through a padded 64 x 64 LDS tile: 16-byte coalesced loads of
// W rows and 16-byte coalesced stores of W^T rows.  K and N are multiples of 8.
__global__ __launch_bounds__(256) void transpose_kernel(const uint16_t* __restrict__ W,
                                                        uint16_t* __restrict__ Wt, int64_t K,
                                                        int64_t N) {
    __shared__ uint16_t tile[64][64 + 2];
    const int64_t k0 = static_cast<int64_t>(blockIdx.y) * 64, n0 = static_cast<int64_t>(blockIdx.x) * 64;
    const int t = threadIdx.x;
#pragma unroll
    for (int r = 0; r < 2; ++r) {   // 64 rows x 8 chunks of 8 elements
        const int idx = t + 256 * r, row = idx / 8, ch = idx % 8;
        const int64_t k = k0 + row, n = n0 + 8 * ch;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (k < K && n < N) v = *reinterpret_cast<const uint4*>(W + k * N + n);
        const uint16_t* e = reinterpret_cast<const uint16_t*>(&v);
#pragma unroll
        for (int i = 0; i < 8; ++i) tile[row][8 * ch + i] = e[i];
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int idx = t + 256 * r, col = idx / 8, ch = idx % 8;
        const int64_t n = n0 + col, k = k0 + 8 * ch;
        if (n < N && k < K) {
            uint16_t e[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) e[i] = tile[8 * ch + i][col];
            *reinterpret_cast<uint4*>(Wt + n * K + k) = *reinterpret_cast<const uint4*>(e);
        }
    }
}

// ------------------------------------------------------------------ fill (tuner inputs)
__global__ __launch_bounds__(256) void fill_bf16_kernel(uint16_t* p, int64_t n, uint32_t salt,
                                                        float amp) {
    for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += gridDim.x * 256ll) {
        uint32_t x = static_cast<uint32_t>(i) * 0x9E3779B1u ^ salt ^ static_cast<uint32_t>(i >> 32);
        x ^= x >> 16;
        x *= 0x7FEB352Du;
        x ^= x >> 15;
        x *= 0x846CA68Bu;
        x ^= x >> 16;
        const float u = __fmul_rn(static_cast<float>(x >> 8), 1.0f / 16777216.0f);  // [0, 1)
        const float v = __fmul_rn(__fsub_rn(__fmul_rn(u, 2.0f), 1.0f), amp);
        p[i] = static_cast<uint16_t>(__float_as_uint(v) >> 16);
    }
}

// ------------------------------------------------------------------ launchers
hipError_t launch_reduce_epilogue(const ReduceArgs& a, int grid, hipStream_t s) {
    hipLaunchKernelGGL(reduce_epilogue_kernel, dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_transpose(const uint16_t* W, uint16_t* Wt, int64_t K, int64_t N, hipStream_t s) {
    hipLaunchKernelGGL(transpose_kernel, dim3(static_cast<unsigned>((N + 63) / 64),
                                             static_cast<unsigned>((K + 63) / 64)),
                       dim3(256), 0, s, W, Wt, K, N);
    return hipGetLastError();
}

hipError_t launch_fill_bf16(uint16_t* p, int64_t n, uint32_t salt, float amp, hipStream_t s) {
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(fill_bf16_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, p,
                       n, salt, amp);
    return hipGetLastError();
}

int reduce_occupancy() {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reduce_epilogue_kernel, 256, 0) !=
        hipSuccess)
        return 0;
    return n;
}

}  // namespace mmar
