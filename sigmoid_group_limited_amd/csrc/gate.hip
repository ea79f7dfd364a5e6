// gate.hip -- router logits on fp32 MFMA with the fused sigmoid / bias /
// group-limited top-k / renormalise epilogue, for gfx950.
//
// What is computed (DeepSeek-V3.2-Exp · Normalize weights, "Code": Gate
// forward; Kimi K2 · Normalize weights, "Code" and the equation for G_i;
// AI Engineer Exhaustive · DeepSeek-V3 MoE Router, "How it works"):
//   L[t,e] = sum_k float(x[t,k]) * W[e,k]          (float32, no linear bias)
//   s = sigmoid(L);  v = s + bias                   (bias steers choice only)
//   group score = top1 + top2 of v inside each of n_group groups
//   keep topk_group groups, others -> -inf; top_k experts by v
//   w = route_scale * s[winner] / sum(s[winners])
//
// Layout of the work
//   One workgroup (4 waves) owns BM = 32*MB tokens and ALL E experts, so a
//   token's whole score row ends in one workgroup and the selection never
//   writes scores to HBM.  Wave w computes BM x (E/4) of the logits with
//   v_mfma_f32_32x32x2_f32; operands come from LDS, which holds KC = 32
//   k-columns of W [E x KC] and of x [BM x KC] (x upcast from bfloat16 to
//   float32 on the way in, exact), double-buffered: the global loads of step
//   c+1 are in flight while step c feeds the matrix cores.
//   Small batches cut the k range into n_split slices (blockIdx.y); each
//   slice writes float32 partial logits and a second kernel adds the slices
//   in a fixed order (deterministic) and runs the same selection.
#include <math.h>

#include "siggate_internal.h"

namespace siggate {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int NT = 256;         // threads per workgroup (4 waves)
constexpr int KPAD = KC + 4;    // padded LDS row in floats: rows start 4 banks apart

template <int E, int MB>
struct Shape {
    static constexpr int BM = 32 * MB;          // tokens per workgroup
    static constexpr int NB = E / 128;          // 32-expert MFMA blocks per wave
    static constexpr int WCOLS = E / 4;         // experts per wave
    static constexpr int V = E / 64;            // experts per lane in the selection
    static constexpr int LROW = E + 4;          // padded logits row (floats)
    static constexpr int STAGE = 2 * (E + BM) * KPAD;
    static constexpr int EPI = BM * LROW;
    static constexpr int SMEM = STAGE > EPI ? STAGE : EPI;
    static_assert(E % 128 == 0, "E must be a multiple of 128");
};

__device__ __forceinline__ float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

// Monotone map of a float to uint32 (larger float -> larger key; -inf is
// the smallest non-NaN key).
__device__ __forceinline__ uint32_t orderable(float f)
{
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m)
{
    const int lo = __shfl_xor((int)(uint32_t)v, m);
    const int hi = __shfl_xor((int)(uint32_t)(v >> 32), m);
    return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

__device__ __forceinline__ float readlane_f(float v, int lane)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Selection for one token held by one wave: lane l owns experts
// [l*V, l*V + V) and their logits lg[].  Writes weights/indices row t.
template <int V>
__device__ __forceinline__ void select_token(const float (&lg)[V], const float (&bias_r)[V],
                                             const int lane, const GateArgs &a, const int t)
{
    float s[V], v[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
        s[j] = 1.0f / (1.0f + expf(-lg[j]));
        v[j] = s[j] + bias_r[j];
    }

    const int G = a.n_group;
    if (G > 1) {
        // Group score: sum of the two largest v of the group, counting
        // multiplicity.  A group is 64/G consecutive lanes.
        const int lpg = 64 / G;
        float m1 = -INFINITY, m2 = -INFINITY;
#pragma unroll
        for (int j = 0; j < V; ++j) {
            const float x = v[j];
            if (x > m1) {
                m2 = m1;
                m1 = x;
            } else if (x > m2) {
                m2 = x;
            }
        }
        for (int off = 1; off < lpg; off <<= 1) {
            const float o1 = __shfl_xor(m1, off);
            const float o2 = __shfl_xor(m2, off);
            const float hi = fmaxf(m1, o1);
            const float lo = fminf(m1, o1);
            m2 = fmaxf(lo, fmaxf(m2, o2));
            m1 = hi;
        }
        const float gs = m1 + m2;
        const int g = lane / lpg;
        // Rank of this lane's group under (score desc, group index asc).
        int ahead = 0;
        for (int h = 0; h < G; ++h) {
            const float gh = readlane_f(gs, h * lpg);
            ahead += (gh > gs) || (gh == gs && h < g);
        }
        if (ahead >= a.topk_group) {
#pragma unroll
            for (int j = 0; j < V; ++j) v[j] = -INFINITY;
        }
    }

    // Token top-K: K rounds of a wave-wide arg-max under (v desc, id asc).
    const int K = a.top_k;
    int sel_i[MAX_TOPK];
    float sel_s[MAX_TOPK];
#pragma unroll
    for (int k = 0; k < MAX_TOPK; ++k) {
        sel_i[k] = 0x7fffffff;
        sel_s[k] = 0.0f;
        if (k < K) {
            float bv = v[0];
            int bj = 0;
#pragma unroll
            for (int j = 1; j < V; ++j) {
                if (v[j] > bv) {
                    bv = v[j];
                    bj = j;
                }
            }
            uint64_t key = ((uint64_t)orderable(bv) << 32) |
                           (uint32_t)(0xffffffffu - (uint32_t)(lane * V + bj));
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) {
                const uint64_t o = shfl_xor_u64(key, off);
                key = o > key ? o : key;
            }
            const int win = __builtin_amdgcn_readfirstlane((int)(0xffffffffu - (uint32_t)key));
            const int owner = win / V;
            const int wj = win - owner * V;
            float mine = 0.0f;
#pragma unroll
            for (int j = 0; j < V; ++j)
                if (j == wj) mine = s[j];
            sel_s[k] = readlane_f(mine, owner);
            sel_i[k] = win;
            if (lane == owner) {
#pragma unroll
                for (int j = 0; j < V; ++j)
                    if (j == wj) v[j] = -INFINITY;
            }
        }
    }

    // Renormalise over the K winners (unbiased s) and scale.
    float denom = 0.0f;
#pragma unroll
    for (int k = 0; k < MAX_TOPK; ++k)
        if (k < K) denom += sel_s[k];

    int my_i = 0;
    float my_s = 0.0f;
#pragma unroll
    for (int k = 0; k < MAX_TOPK; ++k) {
        if (k < K && lane == k) {
            my_i = sel_i[k];
            my_s = sel_s[k];
        }
    }
    int pos = lane;
    if (a.order == 0) {   // ascending expert id
        pos = 0;
#pragma unroll
        for (int k = 0; k < MAX_TOPK; ++k)
            if (k < K) pos += sel_i[k] < my_i;
    }
    if (lane < K) {
        a.indices[(size_t)t * K + pos] = my_i;
        a.weights[(size_t)t * K + pos] = my_s / denom * a.route_scale;
    }
}

template <int E, int MB, int MODE>
__global__ __launch_bounds__(NT) void gate_gemm_kernel(GateArgs a)
{
    using S = Shape<E, MB>;
    __shared__ __attribute__((aligned(16))) float smem[S::SMEM];
    float *const Ws = smem;                    // [2][E][KPAD]
    float *const Xs = smem + 2 * E * KPAD;     // [2][BM][KPAD]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int t0 = blockIdx.x * S::BM;
    const int d = a.d;
    const int c_begin = blockIdx.y * a.chunks_per_split;
    const int c_end = min(c_begin + a.chunks_per_split, a.chunks_total);

    // ---- global -> register staging: W rows (tid/8) + 32 i, 4 floats at
    // column (tid%8)*4; x row tid/4, 8 bfloat16 at column (tid%4)*8.
    constexpr int WLOADS = E / 32;
    f32x4 wreg[WLOADS];
    u32x4 xreg;
    const int w_row = tid >> 3;
    const int w_col = (tid & 7) * 4;
    const int x_row = tid >> 2;
    const int x_col = (tid & 3) * 8;
    const bool x_thread = x_row < S::BM;
    const bool x_valid = x_thread && (t0 + x_row) < a.T;
    const float *const Wp = a.W + (size_t)w_row * d + w_col;
    const uint16_t *const Xp = a.x + (size_t)(x_valid ? t0 + x_row : 0) * d + x_col;

    auto load_global = [&](int c) {
        const int k0 = c * KC;
        const bool wk = k0 + w_col < d;
#pragma unroll
        for (int i = 0; i < WLOADS; ++i)
            wreg[i] = wk ? *(const f32x4 *)(Wp + (size_t)i * 32 * d + k0) : f32x4{0.f, 0.f, 0.f, 0.f};
        const bool xk = x_valid && k0 + x_col < d;
        xreg = xk ? *(const u32x4 *)(Xp + k0) : u32x4{0u, 0u, 0u, 0u};
    };
    auto store_lds = [&](int buf) {
        float *wb = Ws + buf * E * KPAD;
#pragma unroll
        for (int i = 0; i < WLOADS; ++i)
            *(f32x4 *)(wb + (w_row + 32 * i) * KPAD + w_col) = wreg[i];
        if (x_thread) {
            float *xb = Xs + buf * S::BM * KPAD + x_row * KPAD + x_col;
            const f32x4 lo = {bf16_lo(xreg[0]), bf16_hi(xreg[0]), bf16_lo(xreg[1]), bf16_hi(xreg[1])};
            const f32x4 hi = {bf16_lo(xreg[2]), bf16_hi(xreg[2]), bf16_lo(xreg[3]), bf16_hi(xreg[3])};
            *(f32x4 *)xb = lo;
            *(f32x4 *)(xb + 4) = hi;
        }
    };

    // ---- MFMA main loop.  For a group of 8 k-columns, lane l reads 4
    // consecutive k of row (l%32) at offset 4*(l/32); MFMA j pairs column j
    // (lanes 0-31) with column 4+j (lanes 32-63) for A and B alike.
    f32x16 acc[MB][S::NB];
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int n = 0; n < S::NB; ++n)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[m][n][r] = 0.0f;

    const int f_row = lane & 31;
    const int f_k = (lane >> 5) * 4;
    auto compute = [&](int buf) {
        const float *xb = Xs + buf * S::BM * KPAD;
        const float *wb = Ws + buf * E * KPAD + wave * S::WCOLS * KPAD;
#pragma unroll
        for (int c8 = 0; c8 < KC / 8; ++c8) {
            f32x4 af[MB], bf[S::NB];
#pragma unroll
            for (int m = 0; m < MB; ++m)
                af[m] = *(const f32x4 *)(xb + (m * 32 + f_row) * KPAD + c8 * 8 + f_k);
#pragma unroll
            for (int n = 0; n < S::NB; ++n)
                bf[n] = *(const f32x4 *)(wb + (n * 32 + f_row) * KPAD + c8 * 8 + f_k);
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int m = 0; m < MB; ++m)
#pragma unroll
                    for (int n = 0; n < S::NB; ++n)
                        acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[m][j], bf[n][j],
                                                                         acc[m][n], 0, 0, 0);
        }
    };

    if (c_begin < c_end) {
        load_global(c_begin);
        store_lds(0);
        __syncthreads();
        for (int c = c_begin; c < c_end; ++c) {
            const int buf = (c - c_begin) & 1;
            const bool more = c + 1 < c_end;
            if (more) load_global(c + 1);
            compute(buf);
            if (more) store_lds(buf ^ 1);
            __syncthreads();
        }
    }

    // Accumulator element r of block (m, n) in lane l is token
    // m*32 + 8*(r/4) + 4*(l/32) + r%4 and expert wave*E/4 + n*32 + l%32.
    const int e_base = wave * S::WCOLS + (lane & 31);
    const int r_base = 4 * (lane >> 5);

    if constexpr (MODE == MODE_PARTIAL || MODE == MODE_LOGITS) {
        float *out = MODE == MODE_PARTIAL ? a.partial + (size_t)blockIdx.y * a.T * E : a.logits;
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int n = 0; n < S::NB; ++n)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int t = t0 + m * 32 + 8 * (r >> 2) + r_base + (r & 3);
                    if (t < a.T) out[(size_t)t * E + e_base + n * 32] = acc[m][n][r];
                }
    } else {
        // Scores go to LDS (never to HBM); each wave then selects for BM/4
        // tokens.
        float *const Ls = smem;   // [BM][LROW]
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int n = 0; n < S::NB; ++n)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = m * 32 + 8 * (r >> 2) + r_base + (r & 3);
                    Ls[row * S::LROW + e_base + n * 32] = acc[m][n][r];
                }
        __syncthreads();

        constexpr int V = S::V;
        float bias_r[V];
#pragma unroll
        for (int j = 0; j < V; ++j) bias_r[j] = a.bias[lane * V + j];

        for (int i = 0; i < S::BM / 4; ++i) {
            const int row = wave * (S::BM / 4) + i;
            const int t = t0 + row;
            if (t >= a.T) break;
            float lg[V];
#pragma unroll
            for (int j = 0; j < V; ++j) lg[j] = Ls[row * S::LROW + lane * V + j];
            select_token<V>(lg, bias_r, lane, a, t);
        }
    }
}

// Adds the n_split partial logits of one token (fixed order s = 0, 1, ...)
// and writes the logits or runs the selection.  One wave per token.
template <int E, int MODE>
__global__ __launch_bounds__(NT) void gate_reduce_kernel(GateArgs a)
{
    constexpr int V = E / 64;
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * (NT / 64) + (threadIdx.x >> 6);
    if (t >= a.T) return;
    float lg[V];
#pragma unroll
    for (int j = 0; j < V; ++j) lg[j] = 0.0f;
    for (int s = 0; s < a.n_split; ++s) {
        const float *p = a.partial + ((size_t)s * a.T + t) * E + lane * V;
#pragma unroll
        for (int j = 0; j < V; ++j) lg[j] += p[j];
    }
    if constexpr (MODE == MODE_LOGITS) {
#pragma unroll
        for (int j = 0; j < V; ++j) a.logits[(size_t)t * E + lane * V + j] = lg[j];
    } else {
        float bias_r[V];
#pragma unroll
        for (int j = 0; j < V; ++j) bias_r[j] = a.bias[lane * V + j];
        select_token<V>(lg, bias_r, lane, a, t);
    }
}

template <int E>
hipError_t launch_for_e(const GateArgs &a, const GatePlan &p, GateMode final_mode,
                        hipStream_t stream)
{
    const dim3 block(NT);
    if (p.n_split == 1) {
        const int bm = 32 * p.m_blocks;
        const dim3 grid((a.T + bm - 1) / bm, 1);
        if (p.m_blocks == 2) {
            if (final_mode == MODE_SELECT)
                hipLaunchKernelGGL((gate_gemm_kernel<E, 2, MODE_SELECT>), grid, block, 0, stream, a);
            else
                hipLaunchKernelGGL((gate_gemm_kernel<E, 2, MODE_LOGITS>), grid, block, 0, stream, a);
        } else {
            if (final_mode == MODE_SELECT)
                hipLaunchKernelGGL((gate_gemm_kernel<E, 1, MODE_SELECT>), grid, block, 0, stream, a);
            else
                hipLaunchKernelGGL((gate_gemm_kernel<E, 1, MODE_LOGITS>), grid, block, 0, stream, a);
        }
    } else {
        const dim3 grid((a.T + 31) / 32, p.n_split);
        hipLaunchKernelGGL((gate_gemm_kernel<E, 1, MODE_PARTIAL>), grid, block, 0, stream, a);
        const dim3 rgrid((a.T + 3) / 4);
        if (final_mode == MODE_SELECT)
            hipLaunchKernelGGL((gate_reduce_kernel<E, MODE_SELECT>), rgrid, block, 0, stream, a);
        else
            hipLaunchKernelGGL((gate_reduce_kernel<E, MODE_LOGITS>), rgrid, block, 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace

GatePlan plan_gate(int T, int d, int E)
{
    (void)E;
    GatePlan p{};
    const int chunks = (d + KC - 1) / KC;
    const long tiles64 = ((long)T + 63) / 64;
    const long tiles32 = ((long)T + 31) / 32;
    // 256 compute units: aim for at least one workgroup each.
    if (tiles64 >= 256) {
        p.m_blocks = 2;
        p.n_split = 1;
    } else if (tiles32 >= 256) {
        p.m_blocks = 1;
        p.n_split = 1;
    } else {
        p.m_blocks = 1;
        long s = tiles32 > 0 ? (256 + tiles32 - 1) / tiles32 : 1;
        if (s > 64) s = 64;
        if (s > chunks) s = chunks;
        if (s < 1) s = 1;
        const int cps = (int)((chunks + s - 1) / s);
        p.n_split = (chunks + cps - 1) / cps;
        p.chunks_per_split = cps;
    }
    if (p.n_split == 1) p.chunks_per_split = chunks;
    p.partial_bytes = p.n_split > 1 ? (size_t)p.n_split * (size_t)T * (size_t)E * sizeof(float) : 0;
    return p;
}

hipError_t launch_gate(const GateArgs &a, const GatePlan &p, int E, GateMode final_mode,
                       hipStream_t stream)
{
    switch (E) {
    case 128: return launch_for_e<128>(a, p, final_mode, stream);
    case 256: return launch_for_e<256>(a, p, final_mode, stream);
    case 384: return launch_for_e<384>(a, p, final_mode, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace siggate
