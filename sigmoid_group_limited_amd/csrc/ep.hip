// ep.hip -- expert-parallel metadata computed on one GPU, for gfx950.
//
// What is computed (Kimi K2 · Add shared output, "Code": moe_infer, the
// ep_size > 1 branch).  Experts are split into ep_size ranks of
// per = E / ep_size consecutive experts.
//   send splits  rows this GPU sends to each rank: per-rank sums of
//                tokens_per_expert (the pages' tokens_per_ep_rank), and
//                their exclusive prefix; expert-major order is already
//                rank-major, so the splits cut the dispatch buffer directly.
//   regroup      on the receiving side, rows arrive rank after rank and, in a
//                rank, local expert after local expert; each row's label is
//                its local expert and the rows are put in label order,
//                stably (the pages' argsort of gatherd_idxs).  Cell (r, j)
//                of the count matrix is one contiguous run in both orders:
//                it starts at the row-major prefix of the counts on arrival
//                and at the column-major prefix after the regroup.
//   de-duplicated send list
//                a token whose experts sit on one rank several times is sent
//                there once (group-limited routing caps the ranks a token
//                reaches).  The slots are mapped to rank ids with repeats
//                dropped, and the dispatch count / scan / scatter kernels
//                run over ranks; a last pass turns pair ids into token ids
//                and points repeated slots at their first occurrence.
#include "siggate_internal.h"

namespace siggate {
namespace {

constexpr int NT = 256;

__device__ __forceinline__ int block_sum(int v, int *red)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    if (lane == 0) red[wave] = v;
    __syncthreads();
    int tot = 0;
    for (int w = 0; w < NT / 64; ++w) tot += red[w];
    __syncthreads();
    return tot;
}

__global__ __launch_bounds__(NT) void ep_send_splits_kernel(const int32_t *tpe, int E, int ep_size,
                                                            int32_t *counts, int32_t *offsets)
{
    __shared__ int red[NT / 64];
    const int per = E / ep_size;
    int run = 0;
    for (int r = 0; r < ep_size; ++r) {
        int c = 0;
        for (int j = threadIdx.x; j < per; j += NT) c += tpe[r * per + j];
        c = block_sum(c, red);
        if (threadIdx.x == 0) {
            counts[r] = c;
            offsets[r] = run;
        }
        run += c;
    }
    if (threadIdx.x == 0) offsets[ep_size] = run;
}

// Block (r, j): copy the run of cell (r, j) from its arrival position to its
// regrouped position.  Block 0 also writes the local expert totals.
__global__ __launch_bounds__(NT) void ep_regroup_kernel(const int32_t *counts, int ep_size, int per,
                                                        int capacity, int32_t *local_counts,
                                                        int32_t *regroup)
{
    __shared__ int red[NT / 64];
    const int cell = blockIdx.x;
    const int r = cell / per, j = cell - r * per;
    const int n = ep_size * per;
    int in0 = 0, out0 = 0;
    for (int f = threadIdx.x; f < n; f += NT) {
        const int c = counts[f];
        const int fr = f / per, fj = f - fr * per;
        in0 += f < cell ? c : 0;                                     // row-major before
        out0 += (fj < j || (fj == j && fr < r)) ? c : 0;             // column-major before
    }
    in0 = block_sum(in0, red);
    out0 = block_sum(out0, red);
    const int c = counts[cell];
    for (int i = threadIdx.x; i < c; i += NT)
        if (out0 + i < capacity) regroup[out0 + i] = in0 + i;
    if (cell == 0) {
        for (int jj = threadIdx.x; jj < per; jj += NT) {
            int tot = 0;
            for (int rr = 0; rr < ep_size; ++rr) tot += counts[rr * per + jj];
            local_counts[jj] = tot;
        }
    }
}

// Slot -> rank id, -1 when an earlier slot of the token is on the same rank.
__global__ __launch_bounds__(NT) void ep_dedup_map_kernel(EpDedupArgs a)
{
    const int t = blockIdx.x * NT + threadIdx.x;
    if (t >= a.T) return;
    const int32_t *row = a.indices + (size_t)t * a.top_k;
    int rk[MAX_TOPK];
#pragma unroll
    for (int k = 0; k < MAX_TOPK; ++k) {
        rk[k] = -1;
        if (k >= a.top_k) continue;
        const int e = row[k];
        const int r = (e >= 0 && e < a.per * a.ep_size) ? e / a.per : -1;
        bool repeat = false;
#pragma unroll
        for (int k2 = 0; k2 < MAX_TOPK; ++k2)
            if (k2 < k) repeat |= rk[k2] == r;
        rk[k] = r;
        a.rank_ids[(size_t)t * a.top_k + k] = (r >= 0 && !repeat) ? r : -1;
    }
}

__global__ __launch_bounds__(NT) void ep_dedup_finish_kernel(EpDedupArgs a)
{
    const int n = a.T * a.top_k;
    const int total = a.rank_offsets[a.ep_size];
    for (int p = blockIdx.x * NT + threadIdx.x; p < n; p += gridDim.x * NT) {
        if (p < total) a.send_tokens[p] = a.perm[p] / a.top_k;
        int slot = a.dest[p];
        if (slot < 0) {
            // a repeated rank: the slot of its first occurrence in the token
            const int t = p / a.top_k, k = p - t * a.top_k;
            const int32_t *row = a.indices + (size_t)t * a.top_k;
            const int r = row[k] / a.per;
            for (int k2 = 0; k2 < k; ++k2) {
                if (row[k2] / a.per == r) {
                    slot = a.dest[(size_t)t * a.top_k + k2];
                    break;
                }
            }
        }
        a.pair_slot[p] = slot;
    }
}

}  // namespace

hipError_t launch_ep_send_splits(const int32_t *tpe, int E, int ep_size, int32_t *counts,
                                 int32_t *offsets, hipStream_t stream)
{
    return launch_kernel(ep_send_splits_kernel, dim3(1), dim3(NT), stream, tpe, E, ep_size,
                         counts, offsets);
}

hipError_t launch_ep_regroup(const int32_t *counts, int ep_size, int per, int capacity,
                             int32_t *local_counts, int32_t *regroup, hipStream_t stream)
{
    return launch_kernel(ep_regroup_kernel, dim3(ep_size * per), dim3(NT), stream, counts,
                         ep_size, per, capacity, local_counts, regroup);
}

hipError_t launch_ep_dedup_map(const EpDedupArgs &a, hipStream_t stream)
{
    if (a.T == 0) return hipSuccess;
    return launch_kernel(ep_dedup_map_kernel, dim3((a.T + NT - 1) / NT), dim3(NT), stream, a);
}

hipError_t launch_ep_dedup_finish(const EpDedupArgs &a, hipStream_t stream)
{
    const int n = a.T * a.top_k;
    if (n == 0) return hipSuccess;
    const int blocks = (n + NT - 1) / NT < 4096 ? (n + NT - 1) / NT : 4096;
    return launch_kernel(ep_dedup_finish_kernel, dim3(blocks), dim3(NT), stream, a);
}

}  // namespace siggate
