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
// One block per token: each thread owns 8-column (16-byte) vectors, reads
// the K source rows at dest[] and writes one row.  HBM-bound: K*2d bytes read
// and 2d written per token.
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

// K (top_k) is a template parameter so that every slot's load is issued
// before any is used: the loads of a pass do not wait on each other.  A slot
// whose dest is out of range reads row 0 instead and is masked out of the
// sum (the same arithmetic as skipping it).  Each thread handles two column
// vectors per pass, so 2K loads are in flight.  Every expert row is read
// exactly once, so the loads are non-temporal (they do not displace cached
// data; measured 12% faster than plain loads at T=16384, K=8, d=7168).
template <int K>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a)
{
    const int t = blockIdx.x;
    const long npos = (long)a.T * K;
    const u32x4 *rows[K];
    bool ok[K];
    float w[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int p = a.dest[(size_t)t * K + k];
        ok[k] = p >= 0 && p < npos;
        rows[k] = (const u32x4 *)(a.expert_out + (size_t)(ok[k] ? p : 0) * a.d);
        w[k] = a.weights[(size_t)t * K + k];
    }
    const int nvec = a.d / 8;
    u32x4 *yrow = (u32x4 *)(a.y + (size_t)t * a.d);
    for (int i0 = threadIdx.x; i0 < nvec; i0 += 2 * 256) {
        const int i1 = i0 + 256;
        const int j1 = min(i1, nvec - 1);   // in range; stored only if i1 is
        u32x4 v[2][K];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            v[0][k] = __builtin_nontemporal_load(rows[k] + i0);
            v[1][k] = __builtin_nontemporal_load(rows[k] + j1);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            float acc[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
#pragma unroll
            for (int k = 0; k < K; ++k)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float lo = __fadd_rn(acc[2 * q], __fmul_rn(w[k], bf16_lo(v[h][k][q])));
                    const float hi = __fadd_rn(acc[2 * q + 1], __fmul_rn(w[k], bf16_hi(v[h][k][q])));
                    acc[2 * q] = ok[k] ? lo : acc[2 * q];
                    acc[2 * q + 1] = ok[k] ? hi : acc[2 * q + 1];
                }
            u32x4 o;
#pragma unroll
            for (int q = 0; q < 4; ++q) o[q] = bf16_rne(acc[2 * q]) | (bf16_rne(acc[2 * q + 1]) << 16);
            if (h == 0) yrow[i0] = o;
            else if (i1 < nvec) yrow[i1] = o;
        }
    }
}

}  // namespace

hipError_t launch_combine(const CombineArgs &a, hipStream_t stream)
{
    if (a.T == 0) return hipSuccess;
    const dim3 grid(a.T), block(256);
    switch (a.top_k) {
    case 1: return launch_kernel(combine_kernel<1>, grid, block, stream, a);
    case 2: return launch_kernel(combine_kernel<2>, grid, block, stream, a);
    case 3: return launch_kernel(combine_kernel<3>, grid, block, stream, a);
    case 4: return launch_kernel(combine_kernel<4>, grid, block, stream, a);
    case 5: return launch_kernel(combine_kernel<5>, grid, block, stream, a);
    case 6: return launch_kernel(combine_kernel<6>, grid, block, stream, a);
    case 7: return launch_kernel(combine_kernel<7>, grid, block, stream, a);
    case 8: return launch_kernel(combine_kernel<8>, grid, block, stream, a);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace siggate
