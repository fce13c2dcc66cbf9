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

// Every byte is touched once, so all loads and stores are nontemporal (streamed past the
// caches instead of evicting other data into them).
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4_t ld_stream(const float* base, int64_t q) {
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(base) + q);
}
__device__ __forceinline__ void st_stream(float* base, int64_t q, f32x4_t v) {
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t*>(base) + q);
}

// One thread per group of four parameters (n is a multiple of 4); launched with one
// thread per group, the loop only runs again when the grid is capped.
__global__ __launch_bounds__(256) void adam_kernel(AdamArgs a) {
    const int64_t groups = a.n / 4;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
    for (int64_t q = blockIdx.x * 256ll + threadIdx.x; q < groups; q += stride) {
        f32x4_t g = ld_stream(a.grads, q);
        for (int r = 1; r < a.P; ++r) {
            const f32x4_t s = ld_stream(a.grads + r * a.n, q);
            g.x = __fadd_rn(g.x, s.x);
            g.y = __fadd_rn(g.y, s.y);
            g.z = __fadd_rn(g.z, s.z);
            g.w = __fadd_rn(g.w, s.w);
        }
        const f32x4_t p4 = ld_stream(a.param, q), m4 = ld_stream(a.m, q), v4 = ld_stream(a.v, q);
        float p[4], m[4], v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p[i] = p4[i];
            m[i] = m4[i];
            v[i] = v4[i];
            adam1(__fmul_rn(g[i], a.inv_p), p[i], m[i], v[i], a);
        }
        st_stream(a.param, q, f32x4_t{p[0], p[1], p[2], p[3]});
        st_stream(a.m, q, f32x4_t{m[0], m[1], m[2], m[3]});
        st_stream(a.v, q, f32x4_t{v[0], v[1], v[2], v[3]});
        if (a.param_bf16) {
            const u32x2_t h = {bf16_rne(p[0]) | (bf16_rne(p[1]) << 16),
                               bf16_rne(p[2]) | (bf16_rne(p[3]) << 16)};
            __builtin_nontemporal_store(h, reinterpret_cast<u32x2_t*>(a.param_bf16) + q);
        }
    }
}

hipError_t launch_adam(const AdamArgs& a, int grid, hipStream_t s) {
    hipLaunchKernelGGL(adam_kernel, dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace mmar
