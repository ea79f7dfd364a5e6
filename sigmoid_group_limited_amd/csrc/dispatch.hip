// dispatch.hip -- expert-major dispatch of the (token, slot) pairs, for gfx950.
//
// What is computed (Kimi K2 · Add shared output, "Code": moe_infer, its
// first lines; Kimi K3 · MoE update, moe_infer):
//   tokens_per_expert[e] = #{p : indices_flat[p] == e}
//   perm = expert-major order of the flat pair ids p = t*K + k, stable
//          (ascending p inside an expert; the pages' argsort is unstable and
//          this is one of its valid results)
//   permuted_x[pos] = x[perm[pos] / K]
//
// Four launches (one for small batches, below), none of them with
// order-dependent atomics:
//   count   one block per 256 tokens; each wave ORs a 64-bit lane mask per
//           expert in LDS (bit l = token l of the wave routes there), so the
//           block's count of expert e is the popcount of its 4 masks;
//           written expert-major, counts[e][b].
//   scan    one block per expert: exclusive prefix of counts[e][.] over
//           the token blocks, and the expert's total.
//   scatter each block takes the exclusive prefix of the E totals (the
//           expert offsets), recomputes its masks, and places every pair at
//           offset[e] + prefix[e][b] + (popcount of lower lanes' bits plus
//           earlier waves' counts) -- exactly ascending token order.
//   gather  one block per token: read the row once, write it to its K
//           destinations with non-temporal 16-byte stores.
#include "siggate_internal.h"

namespace siggate {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int BT = DISPATCH_BLOCK_TOKENS;
constexpr int WAVES = BT / 64;
constexpr int SCAN_THREADS = 256;

// Loads the K expert ids of token t into e[] (-1 past K or for t >= T).
__device__ __forceinline__ void load_row(const DispatchArgs &a, int t, int (&e)[MAX_TOPK])
{
#pragma unroll
    for (int k = 0; k < MAX_TOPK; ++k) e[k] = -1;
    if (t >= a.T) return;
    const int32_t *row = a.indices + (size_t)t * a.top_k;
    if (a.top_k == 8) {
        const i32x4 lo = *(const i32x4 *)row;
        const i32x4 hi = *(const i32x4 *)(row + 4);
        e[0] = lo[0]; e[1] = lo[1]; e[2] = lo[2]; e[3] = lo[3];
        e[4] = hi[0]; e[5] = hi[1]; e[6] = hi[2]; e[7] = hi[3];
    } else {
#pragma unroll
        for (int k = 0; k < MAX_TOPK; ++k)
            if (k < a.top_k) e[k] = row[k];
    }
}

// masks[w][e] bit l: token (block, wave w, lane l) has a pair on expert e.
__device__ __forceinline__ void build_masks(const DispatchArgs &a,
                                            unsigned long long (*masks)[MAX_EXPERTS],
                                            const int (&e)[MAX_TOPK], int lane, int wave)
{
    for (int i = threadIdx.x; i < WAVES * MAX_EXPERTS; i += BT) (&masks[0][0])[i] = 0ull;
    __syncthreads();
    const unsigned long long bit = 1ull << lane;
#pragma unroll
    for (int k = 0; k < MAX_TOPK; ++k)
        if ((unsigned)e[k] < (unsigned)a.E) atomicOr(&masks[wave][e[k]], bit);
    __syncthreads();
}

__global__ __launch_bounds__(BT) void dispatch_count_kernel(DispatchArgs a)
{
    __shared__ unsigned long long masks[WAVES][MAX_EXPERTS];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int e[MAX_TOPK];
    load_row(a, blockIdx.x * BT + threadIdx.x, e);
    build_masks(a, masks, e, lane, wave);
    for (int x = threadIdx.x; x < a.E; x += BT) {
        int c = 0;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) c += __popcll(masks[w][x]);
        a.block_counts[(size_t)x * a.n_blocks + blockIdx.x] = c;
    }
}

// Block e: exclusive prefix over token blocks of counts[e][.] (in place
// into block_base[e][.]) and tokens_per_expert[e].
__global__ __launch_bounds__(SCAN_THREADS) void dispatch_scan_kernel(DispatchArgs a)
{
    __shared__ int wave_tot[SCAN_THREADS / 64];
    const int e = blockIdx.x;
    const int NB = a.n_blocks;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int32_t *cnt = a.block_counts + (size_t)e * NB;
    int32_t *base = a.block_base + (size_t)e * NB;
    int carry = 0;
    for (int b0 = 0; b0 < NB; b0 += SCAN_THREADS) {
        const int b = b0 + tid;
        const int c = b < NB ? cnt[b] : 0;
        int inc = c;
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(inc, off);
            if (lane >= off) inc += y;
        }
        if (lane == 63) wave_tot[wave] = inc;
        __syncthreads();
        int before = 0, all = 0;
        for (int w = 0; w < SCAN_THREADS / 64; ++w) {
            before += w < wave ? wave_tot[w] : 0;
            all += wave_tot[w];
        }
        if (b < NB) base[b] = carry + before + inc - c;
        carry += all;
        __syncthreads();
    }
    if (tid == 0) a.tokens_per_expert[e] = carry;
}

__global__ __launch_bounds__(BT) void dispatch_scatter_kernel(DispatchArgs a)
{
    __shared__ unsigned long long masks[WAVES][MAX_EXPERTS];
    __shared__ int offset[MAX_EXPERTS];
    __shared__ int wave_tot[WAVES];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t = blockIdx.x * BT + threadIdx.x;

    // Expert offsets: exclusive prefix of tokens_per_expert over experts.
    for (int e0 = 0; e0 < a.E; e0 += BT) {
        const int x = e0 + threadIdx.x;
        const int c = x < a.E ? a.tokens_per_expert[x] : 0;
        int inc = c;
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(inc, off);
            if (lane >= off) inc += y;
        }
        if (lane == 63) wave_tot[wave] = inc;
        __syncthreads();
        int before = e0 > 0 ? offset[e0 - 1] : 0;   // inclusive total so far
        for (int w = 0; w < wave; ++w) before += wave_tot[w];
        __syncthreads();
        if (x < a.E) offset[x] = before + inc;        // inclusive for now
        __syncthreads();
    }
    for (int x = threadIdx.x; x < a.E; x += BT) {
        const int excl = offset[x] - a.tokens_per_expert[x];
        if (blockIdx.x == 0 && a.offsets) {
            a.offsets[x] = excl;
            if (x == a.E - 1) a.offsets[a.E] = offset[x];
        }
    }
    __syncthreads();
    for (int x = threadIdx.x; x < a.E; x += BT)
        offset[x] -= a.tokens_per_expert[x];   // now exclusive

    int e[MAX_TOPK];
    load_row(a, t, e);
    build_masks(a, masks, e, lane, wave);   // its barriers also publish offset[]
    if (t >= a.T) return;
    const unsigned long long lower = (1ull << lane) - 1ull;
#pragma unroll
    for (int k = 0; k < MAX_TOPK; ++k) {
        if (k >= a.top_k) break;
        const size_t p = (size_t)t * a.top_k + k;
        const int x = e[k];
        if ((unsigned)x >= (unsigned)a.E) {
            a.dest[p] = -1;
            continue;
        }
        int pos = offset[x] + a.block_base[(size_t)x * a.n_blocks + blockIdx.x] +
                  __popcll(masks[wave][x] & lower);
        for (int w = 0; w < wave; ++w) pos += __popcll(masks[w][x]);
        a.perm[pos] = (int)p;
        a.dest[p] = pos;
    }
}

__global__ __launch_bounds__(256) void dispatch_gather_kernel(DispatchArgs a)
{
    const int t = blockIdx.x;
    const long npos = (long)a.T * a.top_k;
    int dst[MAX_TOPK];
#pragma unroll
    for (int k = 0; k < MAX_TOPK; ++k) {
        const int v = k < a.top_k ? a.dest[(size_t)t * a.top_k + k] : -1;
        dst[k] = (v >= 0 && v < npos) ? v : -1;
    }
    const int nvec = a.d / 8;
    const u32x4 *src = (const u32x4 *)(a.x + (size_t)t * a.d);
    for (int i = threadIdx.x; i < nvec; i += blockDim.x) {
        const u32x4 val = src[i];
#pragma unroll
        for (int k = 0; k < MAX_TOPK; ++k)
            if (dst[k] >= 0)
                __builtin_nontemporal_store(val, (u32x4 *)(a.permuted_x + (size_t)dst[k] * a.d) + i);
    }
}

// Small batches (T * top_k <= SMALL_PAIRS): all of the dispatch in one
// launch.  Block b handles token t = b / parts and the part-th slice of its
// row.  Every block recounts all pairs from the (L2-resident) indices --
// per-expert totals and the totals over tokens before t -- and takes the
// exclusive prefix of the totals; pair (t, k) then lands at
// offset[e] + before[e], since a token's experts are distinct and the
// earlier pairs of expert e are exactly those of earlier tokens.  Counts
// come from integer atomics, so the result does not depend on their order.
constexpr int SMALL_PAIRS = 4096;
constexpr int SMALL_NT = 256;
constexpr int SMALL_PF = 4;   // row pieces per thread loaded before the count
constexpr int SMALL_CB = 8;   // index loads per thread issued together in the count

__global__ __launch_bounds__(SMALL_NT) void dispatch_small_kernel(DispatchArgs a, int parts)
{
    __shared__ int cnt[MAX_EXPERTS];
    __shared__ int before[MAX_EXPERTS];
    __shared__ int offset[MAX_EXPERTS];
    __shared__ int wave_tot[SMALL_NT / 64];
    __shared__ int pos_s[MAX_TOPK];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t = blockIdx.x / parts;
    const int part = blockIdx.x - t * parts;
    const int K = a.top_k;
    const int first = t * K;              // pairs of tokens before t
    const int npairs = a.T * K;
    // this block's slice [v0, v1) of row t, in 16-byte pieces; the first
    // SMALL_PF pieces of each thread are loaded now, so that their latency
    // overlaps the count below
    const int nvec = a.d / 8;
    const int per = (nvec + parts - 1) / parts;
    const int v0 = part * per;
    const int v1 = min(nvec, v0 + per);
    const u32x4 *src = (const u32x4 *)(a.x + (size_t)t * a.d);
    u32x4 pf[SMALL_PF] = {};
#pragma unroll
    for (int j = 0; j < SMALL_PF; ++j) {
        const int i = v0 + tid + j * SMALL_NT;
        if (i < v1) pf[j] = src[i];
    }
    for (int x = tid; x < a.E; x += SMALL_NT) cnt[x] = before[x] = 0;
    __syncthreads();
    // SMALL_CB index loads in flight before their atomics
    for (int p0 = 0; p0 < npairs; p0 += SMALL_CB * SMALL_NT) {
        int e[SMALL_CB];
#pragma unroll
        for (int j = 0; j < SMALL_CB; ++j) {
            const int p = p0 + j * SMALL_NT + tid;
            e[j] = p < npairs ? a.indices[p] : -1;
        }
#pragma unroll
        for (int j = 0; j < SMALL_CB; ++j) {
            if ((unsigned)e[j] < (unsigned)a.E) {
                atomicAdd(&cnt[e[j]], 1);
                if (p0 + j * SMALL_NT + tid < first) atomicAdd(&before[e[j]], 1);
            }
        }
    }
    __syncthreads();
    // exclusive prefix of cnt[] over experts, SMALL_NT experts at a time
    int carry = 0;
    for (int e0 = 0; e0 < a.E; e0 += SMALL_NT) {
        const int x = e0 + tid;
        const int c = x < a.E ? cnt[x] : 0;
        int inc = c;
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(inc, off);
            if (lane >= off) inc += y;
        }
        if (lane == 63) wave_tot[wave] = inc;
        __syncthreads();
        int pre = carry, all = 0;
        for (int w = 0; w < SMALL_NT / 64; ++w) {
            pre += w < wave ? wave_tot[w] : 0;
            all += wave_tot[w];
        }
        if (x < a.E) offset[x] = pre + inc - c;
        carry += all;
        __syncthreads();
    }
    if (blockIdx.x == 0) {
        for (int x = tid; x < a.E; x += SMALL_NT) {
            a.tokens_per_expert[x] = cnt[x];
            if (a.offsets) a.offsets[x] = offset[x];
        }
        if (a.offsets && tid == 0) a.offsets[a.E] = carry;
    }
    if (tid < K) {
        const int e = a.indices[first + tid];
        const bool ok = (unsigned)e < (unsigned)a.E;
        const int pos = ok ? offset[e] + before[e] : -1;
        pos_s[tid] = pos;
        if (part == 0) {
            if (ok) a.perm[pos] = first + tid;
            if (a.dest) a.dest[first + tid] = pos;
        }
    }
    __syncthreads();
    int dst[MAX_TOPK];
#pragma unroll
    for (int k = 0; k < MAX_TOPK; ++k) dst[k] = k < K ? pos_s[k] : -1;
#pragma unroll
    for (int j = 0; j < SMALL_PF; ++j) {
        const int i = v0 + tid + j * SMALL_NT;
        if (i < v1) {
#pragma unroll
            for (int k = 0; k < MAX_TOPK; ++k)
                if (dst[k] >= 0)
                    __builtin_nontemporal_store(pf[j], (u32x4 *)(a.permuted_x + (size_t)dst[k] * a.d) + i);
        }
    }
    for (int i = v0 + tid + SMALL_PF * SMALL_NT; i < v1; i += SMALL_NT) {
        const u32x4 val = src[i];
#pragma unroll
        for (int k = 0; k < MAX_TOPK; ++k)
            if (dst[k] >= 0)
                __builtin_nontemporal_store(val, (u32x4 *)(a.permuted_x + (size_t)dst[k] * a.d) + i);
    }
}

// T == 0: every count and offset is zero.
__global__ __launch_bounds__(BT) void dispatch_zero_kernel(DispatchArgs a)
{
    for (int x = threadIdx.x; x <= a.E; x += BT) {
        if (x < a.E) a.tokens_per_expert[x] = 0;
        if (a.offsets) a.offsets[x] = 0;
    }
}

}  // namespace

static size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

size_t dispatch_workspace_bytes(int T, int E, int top_k, bool need_dest)
{
    const size_t nb = ((size_t)T + BT - 1) / BT;
    size_t bytes = 2 * align256(nb * (size_t)E * sizeof(int32_t));
    if (need_dest) bytes += align256((size_t)T * top_k * sizeof(int32_t));
    return bytes;
}

hipError_t launch_dispatch_meta(const DispatchArgs &a, hipStream_t stream)
{
    if (a.n_blocks == 0) return launch_kernel(dispatch_zero_kernel, dim3(1), dim3(BT), stream, a);
    hipError_t e = launch_kernel(dispatch_count_kernel, dim3(a.n_blocks), dim3(BT), stream, a);
    if (e == hipSuccess) e = launch_kernel(dispatch_scan_kernel, dim3(a.E), dim3(SCAN_THREADS), stream, a);
    if (e == hipSuccess) e = launch_kernel(dispatch_scatter_kernel, dim3(a.n_blocks), dim3(BT), stream, a);
    return e;
}

hipError_t launch_dispatch(const DispatchArgs &a, hipStream_t stream)
{
    if (a.n_blocks == 0) return launch_kernel(dispatch_zero_kernel, dim3(1), dim3(BT), stream, a);
    if ((long)a.T * a.top_k <= SMALL_PAIRS) {
        // split each row over enough blocks to reach about 256 of them
        int parts = 1;
        while ((long)a.T * parts * 2 <= 256 && parts * 2 <= a.d / 8) parts *= 2;
        return launch_kernel(dispatch_small_kernel, dim3(a.T * parts), dim3(SMALL_NT), stream, a,
                             parts);
    }
    hipError_t e = launch_dispatch_meta(a, stream);
    if (e == hipSuccess) e = launch_kernel(dispatch_gather_kernel, dim3(a.T), dim3(256), stream, a);
    return e;
}

}  // namespace siggate
