// Internal declarations shared by the HIP translation units of libsiggate.
// Not part of the public ABI (that is include/siggate.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace siggate {

// Launches `kernel` and returns the status of this launch: hipLaunchKernel's
// own result.  The thread's last-error state is neither read nor cleared, so
// an error left there by unrelated earlier calls (the caller's, or another
// library's) is not reported as ours, and stays for its owner to see.
template <typename T> struct arg_of { typedef T type; };
template <typename... P>
inline hipError_t launch_kernel(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t stream,
                                typename arg_of<P>::type... args)
{
    void *argv[] = {(void *)&args..., nullptr};
    return hipLaunchKernel((const void *)kernel, grid, block, argv, 0, stream);
}

// k-elements of x and W staged in LDS per main-loop step
constexpr int KC = 32;
// tokens per dispatch block (4 waves of 64 lanes, one token per lane)
constexpr int DISPATCH_BLOCK_TOKENS = 256;
// largest expert count any kernel instantiates
constexpr int MAX_EXPERTS = 512;
// largest top_k
constexpr int MAX_TOPK = 8;

enum GateMode { MODE_SELECT = 0, MODE_LOGITS = 1, MODE_PARTIAL = 2 };

struct GateArgs {
    const uint16_t *x;      // bfloat16 bits [T, d]
    const float *W;         // [E, d]
    const float *bias;      // [E]
    int T, d;
    int n_group, topk_group, top_k, order;
    int score_func, renorm, mask_zero;
    float route_scale, denom_eps;
    int E;                  // experts: row length of the logits
    int e_stride;           // row length of the partials: E, or E rounded up to
                            // whole 128-expert tiles on the float32 split path
    int chunks_total;       // ceil(d / KC)
    int chunks_per_split;   // KC-chunks of one k-slice
    int n_split;            // k-slices (1 = whole k range in one workgroup)
    int t_tiles, e_tiles;   // token and expert tiles of the split GEMM
    int n_tiles;            // t_tiles * e_tiles * n_split
    int e_fast;             // x3 tiles: expert tile fastest (1) or token tile fastest (0)
    float *weights;         // [T, top_k]      (MODE_SELECT)
    int32_t *indices;       // [T, top_k]      (MODE_SELECT)
    float *logits;          // [T, E]          (MODE_LOGITS)
    float *partial;         // [n_split, T, E] (MODE_PARTIAL, reduce input)
    const uint16_t *w_planes;   // [3, E, d] bfloat16 parts of W (pre-split x3 route)
};

// How the logits GEMM is cut for a given T.
//   fused: one workgroup owns 32*m_blocks tokens x all E experts x the whole
//          k range and runs the selection itself (no partials);
//   split: one workgroup owns 32 tokens x 128 experts x one k-slice (or,
//          wide, 32*m_blocks tokens x all E x one k-slice) and writes float32
//          partial logits [n_split, T, e_stride]; a second kernel adds the
//          slices and runs the selection.
//   x3:    the split layout with the bfloat16 three-way route of
//          logits_x3.hip: x3_bm tokens x 64*x3_nbw experts x one k-slice.
struct GatePlan {
    bool split;
    int x3_bm, x3_nbw;      // x3 tile (0, 0 on the float32 route)
    bool x3_presplit;       // x3: W split once into planes in the workspace
    size_t planes_offset;   // x3 pre-split: byte offset of the planes
    int m_blocks;           // 32-token blocks per workgroup: 1 or 2 (fused, wide split), 1 (split)
    bool wide;              // split path on full-E tiles (32*m_blocks tokens x E, the fused
                            // kernel's tile) instead of 32 x 128
    int n_split;            // k-slices (split path)
    int chunks_per_split;
    int t_tiles, e_tiles;   // split path tiles
    int grid;               // workgroups of the GEMM launch
    int e_stride;           // row length of the partials (GateArgs::e_stride)
    size_t partial_bytes;   // workspace: split partials (+ x3 planes)
};

// Logits routes (siggate_cfg_t.logits_path)
enum LogitsPath { PATH_FP32 = 0, PATH_BF16X3 = 1 };

GatePlan plan_gate(int T, int d, int E, int path);
GatePlan plan_x3(int T, int d, int E);
hipError_t launch_x3_gemm(const GateArgs &a, const GatePlan &p, hipStream_t stream);

// Launchers; return hipSuccess or the launch error.
hipError_t launch_gate(const GateArgs &a, const GatePlan &p, int E, GateMode final_mode,
                       hipStream_t stream);

struct DispatchArgs {
    const uint16_t *x;
    const int32_t *indices;
    int T, d, E, top_k;
    int n_blocks;           // ceil(T / DISPATCH_BLOCK_TOKENS)
    int32_t *block_counts;  // [n_blocks, E]  workspace
    int32_t *block_base;    // [n_blocks, E]  workspace
    int32_t *tokens_per_expert;  // [E]
    int32_t *offsets;       // [E + 1] or nullptr
    int32_t *perm;          // [T * top_k]
    int32_t *dest;          // [T * top_k]
    uint16_t *permuted_x;   // [T * top_k, d]
};

size_t dispatch_workspace_bytes(int T, int E, int top_k, bool need_dest);
hipError_t launch_dispatch(const DispatchArgs &a, hipStream_t stream);
// count, scan and scatter only (no row gather); dest must be set
hipError_t launch_dispatch_meta(const DispatchArgs &a, hipStream_t stream);

struct EpDedupArgs {
    const int32_t *indices;   // [T, top_k]
    int32_t *rank_ids;        // [T, top_k] workspace: rank of the slot, -1 if repeated
    int32_t *perm;            // [T * top_k] workspace (scatter output)
    int32_t *dest;            // [T * top_k] workspace (scatter output)
    const int32_t *rank_offsets;   // [ep_size + 1] (scatter output)
    int32_t *send_tokens;     // [<= T * top_k]
    int32_t *pair_slot;       // [T * top_k]
    int T, top_k, per, ep_size;
};
hipError_t launch_ep_send_splits(const int32_t *tpe, int E, int ep_size, int32_t *counts,
                                 int32_t *offsets, hipStream_t stream);
hipError_t launch_ep_regroup(const int32_t *counts, int ep_size, int per, int capacity,
                             int32_t *local_counts, int32_t *regroup, hipStream_t stream);
hipError_t launch_ep_dedup_map(const EpDedupArgs &a, hipStream_t stream);
hipError_t launch_ep_dedup_finish(const EpDedupArgs &a, hipStream_t stream);

struct CombineArgs {
    const uint16_t *expert_out;   // bfloat16 [T * top_k, d]
    const float *weights;         // [T, top_k]
    const int32_t *dest;          // [T * top_k]
    uint16_t *y;                  // bfloat16 [T, d]
    int T, d, top_k;
};
hipError_t launch_combine(const CombineArgs &a, hipStream_t stream);

}  // namespace siggate
