// The block computed the unfused way, one kernel per operation, as a framework that
// calls computation and communication as separate library kernels runs it (the
// comparison point of the CoCoNet record, LIT-735, "Key takeaways", first and second
// bullets): the slice GEMMs write every partial to HBM (tile_kernel, partials mode), a
// reduction kernel sums them (the AllReduce), then separate bias-add, dropout (with the
// keep mask written out as bytes) and residual-add kernels.  Each of the four kernels
// here is HBM-bound; beyond the GEMM's partial writes they move 4PMN + 4MN (sum), 8MN
// (bias add), 9MN (dropout and mask) and 10MN (residual add) bytes.
//
// The arithmetic is the fused epilogue's, operation by operation (round to nearest even,
// no fused multiply-add): v = T + bias, y = v * scale, out = residual + y.  A dropped
// element gets y = -0.0, and residual + (-0.0) == residual for every value, so the output
// bits equal the fused path's.
#include "device_common.h"
#include "mmar_internal.h"

namespace mmar {

// T[i] = S_0[i] + S_1[i] + ... + S_{P-1}[i], left to right; T may alias S_0.
__global__ __launch_bounds__(256) void sum_partials_kernel(const float* ws, float* T, int64_t plane,
                                                           int32_t P) {
    const int64_t groups = plane / 4;
    for (int64_t q = blockIdx.x * 256ll + threadIdx.x; q < groups; q += gridDim.x * 256ll) {
        float4 t = reinterpret_cast<const float4*>(ws)[q];
        for (int p = 1; p < P; ++p) {
            const float4 s = reinterpret_cast<const float4*>(ws + p * plane)[q];
            t.x = __fadd_rn(t.x, s.x);
            t.y = __fadd_rn(t.y, s.y);
            t.z = __fadd_rn(t.z, s.z);
            t.w = __fadd_rn(t.w, s.w);
        }
        reinterpret_cast<float4*>(T)[q] = t;
    }
}

// V = T + bias (in place), N a multiple of 4.
__global__ __launch_bounds__(256) void bias_add_kernel(float* T, const uint16_t* bias, int64_t M,
                                                       int64_t N) {
    const int64_t groups = M * N / 4;
    for (int64_t q = blockIdx.x * 256ll + threadIdx.x; q < groups; q += gridDim.x * 256ll) {
        const int64_t n = (4 * q) % N;
        const uint2 b = *reinterpret_cast<const uint2*>(bias + n);
        float4 t = reinterpret_cast<float4*>(T)[q];
        t.x = __fadd_rn(t.x, bf16_lo(b.x));
        t.y = __fadd_rn(t.y, bf16_hi(b.x));
        t.z = __fadd_rn(t.z, bf16_lo(b.y));
        t.w = __fadd_rn(t.w, bf16_hi(b.y));
        reinterpret_cast<float4*>(T)[q] = t;
    }
}

// Dropout in place: mask byte e = keep(e); Y = keep ? V * scale : -0.0.
__global__ __launch_bounds__(256) void dropout_kernel(float* V, uint8_t* mask, int64_t count,
                                                      DropParams d) {
    const int64_t groups = count / 4;
    for (int64_t q = blockIdx.x * 256ll + threadIdx.x; q < groups; q += gridDim.x * 256ll) {
        const uint64_t g = static_cast<uint64_t>(q);   // group of linear elements 4q .. 4q+3
        const uint4 w = philox4x32_10(static_cast<uint32_t>(g), static_cast<uint32_t>(g >> 32),
                                      d.ctr2, d.ctr3, d.key0, d.key1);
        const bool k0 = !d.drop_all && w.x >= d.thr, k1 = !d.drop_all && w.y >= d.thr;
        const bool k2 = !d.drop_all && w.z >= d.thr, k3 = !d.drop_all && w.w >= d.thr;
        float4 v = reinterpret_cast<float4*>(V)[q];
        v.x = k0 ? __fmul_rn(v.x, d.scale) : -0.0f;
        v.y = k1 ? __fmul_rn(v.y, d.scale) : -0.0f;
        v.z = k2 ? __fmul_rn(v.z, d.scale) : -0.0f;
        v.w = k3 ? __fmul_rn(v.w, d.scale) : -0.0f;
        reinterpret_cast<float4*>(V)[q] = v;
        reinterpret_cast<uint32_t*>(mask)[q] = (k0 ? 1u : 0u) | (k1 ? 1u << 8 : 0u) |
                                               (k2 ? 1u << 16 : 0u) | (k3 ? 1u << 24 : 0u);
    }
}

// out = residual + Y.
__global__ __launch_bounds__(256) void residual_add_kernel(const float* Y, const uint16_t* residual,
                                                           float* out, int64_t count) {
    const int64_t groups = count / 4;
    for (int64_t q = blockIdx.x * 256ll + threadIdx.x; q < groups; q += gridDim.x * 256ll) {
        const uint2 r = reinterpret_cast<const uint2*>(residual)[q];
        const float4 y = reinterpret_cast<const float4*>(Y)[q];
        float4 o;
        o.x = __fadd_rn(bf16_lo(r.x), y.x);
        o.y = __fadd_rn(bf16_hi(r.x), y.y);
        o.z = __fadd_rn(bf16_lo(r.y), y.z);
        o.w = __fadd_rn(bf16_hi(r.y), y.w);
        reinterpret_cast<float4*>(out)[q] = o;
    }
}

hipError_t launch_unfused_tail(const float* ws, float* T, const uint16_t* bias,
                               const uint16_t* residual, float* out, uint8_t* mask, int64_t M,
                               int64_t N, int32_t P, const DropParams& d, int grid,
                               hipStream_t s) {
    const int64_t plane = M * N;
    hipLaunchKernelGGL(sum_partials_kernel, dim3(grid), dim3(256), 0, s, ws, T, plane, P);
    hipLaunchKernelGGL(bias_add_kernel, dim3(grid), dim3(256), 0, s, T, bias, M, N);
    hipLaunchKernelGGL(dropout_kernel, dim3(grid), dim3(256), 0, s, T, mask, plane, d);
    hipLaunchKernelGGL(residual_add_kernel, dim3(grid), dim3(256), 0, s,
                       static_cast<const float*>(T), residual, out, plane);
    return hipGetLastError();
}

}  // namespace mmar
