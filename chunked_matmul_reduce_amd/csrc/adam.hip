// The data-parallel side of the CoCoNet record (LIT-735, "Key takeaways", fifth bullet:
// the gradient ReduceScatter, the optimizer and the parameter AllGather fused, against
// DDP's bucketed AllReduce) folded onto one GPU: the P replicas' gradients are summed in
// the fixed order p = 0 .. P-1 and averaged (the reduction), the Adam step updates the
// fp32 parameters and moments in place (the optimizer on each shard), and the bf16 copy
// of the new parameters is written (what the AllGather would hand to the next forward
// pass), all in one pass over HBM.  HBM-bound: 4P + 26 bytes per parameter (P gradient
// reads; parameter, first and second moment read and written; the bf16 copy written).
//
// Per parameter, fp32, round to nearest even, no fused multiply-add:
//   g = (G_0 + G_1 + ... + G_{P-1}) * inv_p
//   m = b1 * m + (1 - b1) * g;   v = b2 * v + (1 - b2) * g * g
//   p = p - lr * ((m * c1) / (sqrt(v * c2) + eps) + wd * p)
// with c1 = 1 / (1 - b1^t), c2 = 1 / (1 - b2^t) computed on the host in fp64.
#include "device_common.h"
#include "mmar_internal.h"

namespace mmar {

__device__ __forceinline__ void adam1(float g, float& p, float& m, float& v, const AdamArgs& a) {
    m = __fadd_rn(__fmul_rn(a.b1, m), __fmul_rn(a.one_minus_b1, g));
    v = __fadd_rn(__fmul_rn(a.b2, v), __fmul_rn(a.one_minus_b2, __fmul_rn(g, g)));
    const float mhat = __fmul_rn(m, a.c1);
    const float den = __fadd_rn(__fsqrt_rn(__fmul_rn(v, a.c2)), a.eps);
    const float upd = __fadd_rn(__fdiv_rn(mhat, den), __fmul_rn(a.wd, p));
    p = __fsub_rn(p, __fmul_rn(a.lr, upd));
}

// One thread per group of four parameters (n is a multiple of 4).
__global__ __launch_bounds__(256) void adam_kernel(AdamArgs a) {
    const int64_t groups = a.n / 4;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
    for (int64_t q = blockIdx.x * 256ll + threadIdx.x; q < groups; q += stride) {
        float4 g = reinterpret_cast<const float4*>(a.grads)[q];
        for (int r = 1; r < a.P; ++r) {
            const float4 s = reinterpret_cast<const float4*>(a.grads + r * a.n)[q];
            g.x = __fadd_rn(g.x, s.x);
            g.y = __fadd_rn(g.y, s.y);
            g.z = __fadd_rn(g.z, s.z);
            g.w = __fadd_rn(g.w, s.w);
        }
        float4 p = reinterpret_cast<float4*>(a.param)[q];
        float4 m = reinterpret_cast<float4*>(a.m)[q];
        float4 v = reinterpret_cast<float4*>(a.v)[q];
        adam1(__fmul_rn(g.x, a.inv_p), p.x, m.x, v.x, a);
        adam1(__fmul_rn(g.y, a.inv_p), p.y, m.y, v.y, a);
        adam1(__fmul_rn(g.z, a.inv_p), p.z, m.z, v.z, a);
        adam1(__fmul_rn(g.w, a.inv_p), p.w, m.w, v.w, a);
        reinterpret_cast<float4*>(a.param)[q] = p;
        reinterpret_cast<float4*>(a.m)[q] = m;
        reinterpret_cast<float4*>(a.v)[q] = v;
        if (a.param_bf16)
            reinterpret_cast<uint2*>(a.param_bf16)[q] = make_uint2(
                bf16_rne(p.x) | (bf16_rne(p.y) << 16), bf16_rne(p.z) | (bf16_rne(p.w) << 16));
    }
}

hipError_t launch_adam(const AdamArgs& a, int grid, hipStream_t s) {
    hipLaunchKernelGGL(adam_kernel, dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace mmar
