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
// Three launches (one for small batches, below), none of them with
// order-dependent atomics:
//   count   one block per 256 tokens; each wave ORs a 64-bit lane mask per
//           expert in LDS (bit l = token l of the wave routes there), so the
//           block's count of expert e is the popcount of its 4 masks, and a
//           pair's rank among the block's pairs of its expert -- popcount of
//           the lower lanes' bits plus the earlier waves' counts -- is
//           exactly its rank in ascending token order (stable).  Writes the
//           counts block-major, counts[b][e], and the ranks into dest.
//   scan    one block: per expert, the total over token blocks and the
//           exclusive prefix over them; the exclusive prefix of the totals
//           over experts (the expert offsets); base[b][e] = offset[e] +
//           prefix[e][b]; tokens_per_expert and offsets.
//   gather  one block per token: each pair lands at base[b][e] + rank (its
//           block writes dest and perm), then the row is read once and
//           written to its K destinations with non-temporal 16-byte stores.
#include "siggate_internal.h"

namespace siggate {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int BT = DISPATCH_BLOCK_TOKENS;
constexpr int WAVES = BT / 64;

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
    const int t = blockIdx.x * BT + threadIdx.x;
    int e[MAX_TOPK];
    load_row(a, t, e);
    build_masks(a, masks, e, lane, wave);
    int32_t *const cnt = a.block_counts + (size_t)blockIdx.x * a.E;
    for (int x = threadIdx.x; x < a.E; x += BT) {
        int c = 0;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) c += __popcll(masks[w][x]);
        cnt[x] = c;
    }
    // rank of each of this token's pairs among the block's pairs of its
    // expert, in token order; -1 for an id out of range
    if (t >= a.T) return;
    const unsigned long long lower = (1ull << lane) - 1ull;
    int r[MAX_TOPK];
#pragma unroll
    for (int k = 0; k < MAX_TOPK; ++k) {
        const int x = e[k];
        r[k] = -1;
        if (k < a.top_k && (unsigned)x < (unsigned)a.E) {
            r[k] = __popcll(masks[wave][x] & lower);
            for (int w = 0; w < wave; ++w) r[k] += __popcll(masks[w][x]);
        }
    }
    int32_t *const out = a.dest + (size_t)t * a.top_k;
    if (a.top_k == 8) {
        *(i32x4 *)out = i32x4{r[0], r[1], r[2], r[3]};
        *(i32x4 *)(out + 4) = i32x4{r[4], r[5], r[6], r[7]};
    } else {
#pragma unroll
        for (int k = 0; k < MAX_TOPK; ++k)
            if (k < a.top_k) out[k] = r[k];
    }
}

// One block.  Thread (part, e) owns expert e and the part-th run of token
// blocks: it sums their counts (CB loads in flight at a time), the parts'
// sums give the expert's total and each part's starting prefix, a block-wide
// scan of the totals gives the expert offsets, and a second pass over the
// run writes base[b][e] = offset[e] + (counts of e in blocks before b).
// CB is the run length held in registers: 32 or 64, the smallest that holds
// the run (a larger one only adds predicated-off loads: 7.0 against 5.5 us
// at T = 16384, E = 384, whose runs are 32 blocks long).
constexpr int SCAN_NT = 1024;

// parts of the scan: the largest power of two with parts * E <= SCAN_NT
__host__ __device__ inline int scan_parts(int E)
{
    int parts = 1;
    while (parts * 2 * E <= SCAN_NT) parts *= 2;
    return parts;
}

template <int SCAN_CB>
__global__ __launch_bounds__(SCAN_NT) void dispatch_scan_kernel(DispatchArgs a)
{
    __shared__ int part_tot[SCAN_NT];       // [part][e]
    __shared__ int wave_tot[SCAN_NT / 64];
    __shared__ int exp_off[MAX_EXPERTS];
    const int E = a.E, NB = a.n_blocks;
    const int parts = scan_parts(E);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int part = tid / E, e = tid - part * E;
    const bool live = part < parts;
    const int run = (NB + parts - 1) / parts;
    const int b_begin = live ? min(part * run, NB) : NB;
    const int b_end = live ? min(b_begin + run, NB) : NB;
    const int32_t *const cnt = a.block_counts;

    // a run of at most SCAN_CB blocks stays in registers for the second
    // pass; longer runs (T > 16384 * parts) are read again
    const bool one = b_end - b_begin <= SCAN_CB;
    int v[SCAN_CB];
    int sum = 0;
    for (int b0 = b_begin; b0 < b_end; b0 += SCAN_CB) {
#pragma unroll
        for (int u = 0; u < SCAN_CB; ++u) v[u] = b0 + u < b_end ? cnt[(size_t)(b0 + u) * E + e] : 0;
#pragma unroll
        for (int u = 0; u < SCAN_CB; ++u) sum += v[u];
    }
    if (live) part_tot[part * E + e] = sum;
    __syncthreads();
    // expert totals (parts in order) and this part's start inside its expert
    int total = 0, start = 0;
    if (live) {
        for (int q = 0; q < parts; ++q) {
            const int c = part_tot[q * E + e];
            start += q < part ? c : 0;
            total += c;
        }
    }
    // exclusive scan of the totals over experts: the part-0 threads carry
    // experts 0 .. E-1 in thread order
    const int tv = (live && part == 0) ? total : 0;
    int inc = tv;
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(inc, off);
        if (lane >= off) inc += y;
    }
    if (lane == 63) wave_tot[wave] = inc;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += wave_tot[w];
    if (live && part == 0) {
        exp_off[e] = before + inc - tv;
        a.tokens_per_expert[e] = total;
        if (a.offsets) {
            a.offsets[e] = before + inc - tv;
            if (e == E - 1) a.offsets[E] = before + inc;
        }
    }
    __syncthreads();
    if (!live) return;
    int acc = exp_off[e] + start;
    for (int b0 = b_begin; b0 < b_end; b0 += SCAN_CB) {
        if (!one) {
#pragma unroll
            for (int u = 0; u < SCAN_CB; ++u) v[u] = b0 + u < b_end ? cnt[(size_t)(b0 + u) * E + e] : 0;
        }
#pragma unroll
        for (int u = 0; u < SCAN_CB; ++u) {
            if (b0 + u < b_end) a.block_base[(size_t)(b0 + u) * E + e] = acc;
            acc += v[u];
        }
    }
}

// Final position of pair p = t*K + k: base[t / BT][e] + its rank (held in
// dest on entry); -1 for an id out of range.
__device__ __forceinline__ int final_pos(const DispatchArgs &a, int t, int k)
{
    const size_t p = (size_t)t * a.top_k + k;
    const int x = a.indices[p];
    const int r = a.dest[p];
    return ((unsigned)x < (unsigned)a.E && r >= 0)
               ? a.block_base[(size_t)(t / BT) * a.E + x] + r : -1;
}

// Positions without rows (the expert-parallel de-duplication): one thread
// per pair writes dest and perm.
__global__ __launch_bounds__(256) void dispatch_place_kernel(DispatchArgs a)
{
    const long p = (long)blockIdx.x * 256 + threadIdx.x;
    if (p >= (long)a.T * a.top_k) return;
    const int t = (int)(p / a.top_k), k = (int)(p - (long)t * a.top_k);
    const int pos = final_pos(a, t, k);
    if (pos >= 0) a.perm[pos] = (int)p;
    a.dest[p] = pos;
}

// One block per token: the pairs' final positions (written to dest and
// perm by the first top_k threads), then the row, read once, to its K
// destinations.  The first loads of the row are issued before the
// positions are known, so their latency overlaps the index loads.
constexpr int GATHER_NT = 256;
constexpr int GATHER_PF = 2;   // 16-byte pieces per thread loaded up front

__global__ __launch_bounds__(GATHER_NT) void dispatch_gather_kernel(DispatchArgs a)
{
    const int t = blockIdx.x;
    const int nvec = a.d / 8;
    const u32x4 *src = (const u32x4 *)(a.x + (size_t)t * a.d);
    u32x4 pf[GATHER_PF] = {};
#pragma unroll
    for (int j = 0; j < GATHER_PF; ++j) {
        const int i = threadIdx.x + j * GATHER_NT;
        if (i < nvec) pf[j] = src[i];
    }
    int dst[MAX_TOPK];
#pragma unroll
    for (int k = 0; k < MAX_TOPK; ++k) dst[k] = k < a.top_k ? final_pos(a, t, k) : -1;
    // every thread has read its dest entries above before any is rewritten
    __syncthreads();
    if (threadIdx.x < a.top_k) {
        const int k = threadIdx.x;
        const size_t p = (size_t)t * a.top_k + k;
        int pos = -1;
#pragma unroll
        for (int j = 0; j < MAX_TOPK; ++j)
            if (j == k) pos = dst[j];
        if (pos >= 0) a.perm[pos] = (int)p;
        a.dest[p] = pos;
    }
#pragma unroll
    for (int j = 0; j < GATHER_PF; ++j) {
        const int i = threadIdx.x + j * GATHER_NT;
        if (i < nvec) {
#pragma unroll
            for (int k = 0; k < MAX_TOPK; ++k)
                if (dst[k] >= 0)
                    __builtin_nontemporal_store(pf[j], (u32x4 *)(a.permuted_x + (size_t)dst[k] * a.d) + i);
        }
    }
    for (int i = threadIdx.x + GATHER_PF * GATHER_NT; i < nvec; i += GATHER_NT) {
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

// count and scan: the ranks in dest, the base table, tokens_per_expert, offsets
static hipError_t launch_count_scan(const DispatchArgs &a, hipStream_t stream)
{
    hipError_t e = launch_kernel(dispatch_count_kernel, dim3(a.n_blocks), dim3(BT), stream, a);
    if (e != hipSuccess) return e;
    const int parts = scan_parts(a.E);
    const int run = (a.n_blocks + parts - 1) / parts;
    return run <= 32 ? launch_kernel(dispatch_scan_kernel<32>, dim3(1), dim3(SCAN_NT), stream, a)
                     : launch_kernel(dispatch_scan_kernel<64>, dim3(1), dim3(SCAN_NT), stream, a);
}

hipError_t launch_dispatch_meta(const DispatchArgs &a, hipStream_t stream)
{
    if (a.n_blocks == 0) return launch_kernel(dispatch_zero_kernel, dim3(1), dim3(BT), stream, a);
    hipError_t e = launch_count_scan(a, stream);
    const long pairs = (long)a.T * a.top_k;
    if (e == hipSuccess)
        e = launch_kernel(dispatch_place_kernel, dim3((unsigned)((pairs + 255) / 256)), dim3(256), stream, a);
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
    hipError_t e = launch_count_scan(a, stream);
    if (e == hipSuccess) e = launch_kernel(dispatch_gather_kernel, dim3(a.T), dim3(GATHER_NT), stream, a);
    return e;
}

}  // namespace siggate
