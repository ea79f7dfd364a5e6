// combine.hip -- un-permute the expert outputs and add each token's rows
// weighted by its gate weights, for gfx950.
//
// What is computed (Kimi K2 · Add shared output, "Code": moe_infer, last
// lines; Kimi K3 · MoE update, moe_infer): the rows come back to (token,
// slot) order, are cast to the weights' type (float32), multiplied by their
// weight, summed over the slots and cast back to the activation type:
//   y[t, :] = bf16( sum_k w[t, k] * float(out[dest[t*K + k], :]) )
// Here the products are rounded to float32 and summed in ascending k, and
// the result is rounded to bfloat16 (nearest even).
//
// One block per token: each thread owns 8 columns (16 bytes), reads the K
// source rows at dest[] and writes one row.  HBM-bound: K*2d bytes read and
// 2d written per token.
#include "siggate_internal.h"

namespace siggate {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

// float32 -> bfloat16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ unsigned bf16_rne(float f)
{
    const unsigned u = __float_as_uint(f);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a)
{
    const int t = blockIdx.x;
    const int K = a.top_k;
    const long npos = (long)a.T * K;
    int src[MAX_TOPK];
    float w[MAX_TOPK];
#pragma unroll
    for (int k = 0; k < MAX_TOPK; ++k) {
        const int p = k < K ? a.dest[(size_t)t * K + k] : -1;
        src[k] = (p >= 0 && p < npos) ? p : -1;
        w[k] = k < K ? a.weights[(size_t)t * K + k] : 0.0f;
    }
    const int nvec = a.d / 8;
    u32x4 *yrow = (u32x4 *)(a.y + (size_t)t * a.d);
    for (int i = threadIdx.x; i < nvec; i += blockDim.x) {
        float acc[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
#pragma unroll
        for (int k = 0; k < MAX_TOPK; ++k) {
            if (src[k] < 0) continue;
            const u32x4 v = ((const u32x4 *)(a.expert_out + (size_t)src[k] * a.d))[i];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[2 * q] = __fadd_rn(acc[2 * q], __fmul_rn(w[k], bf16_lo(v[q])));
                acc[2 * q + 1] = __fadd_rn(acc[2 * q + 1], __fmul_rn(w[k], bf16_hi(v[q])));
            }
        }
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = bf16_rne(acc[2 * q]) | (bf16_rne(acc[2 * q + 1]) << 16);
        yrow[i] = o;
    }
}

}  // namespace

hipError_t launch_combine(const CombineArgs &a, hipStream_t stream)
{
    if (a.T > 0) hipLaunchKernelGGL(combine_kernel, dim3(a.T), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace siggate
