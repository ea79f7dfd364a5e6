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
//   One workgroup of 8 waves (two per SIMD) owns BM = 32*MB tokens and ALL E
//   experts, so a token's whole score row ends in one workgroup and the
//   selection never writes scores to HBM.  The waves are 4 expert quarters x
//   2 token halves (BM = 64) or x 2 k-halves of every chunk (BM = 32); each
//   computes its share of the logits with v_mfma_f32_32x32x2_f32.  Operands
//   come from LDS, which holds KC = 32 k-columns of W [E x KC] and of x
//   [BM x KC] (x upcast from bfloat16 to float32 on the way in, exact),
//   double-buffered, with two more chunks of global loads in flight.
//   Batches whose fused tiles would leave compute units idle (all small
//   batches, and most mid-size ones, where a partly filled last round of
//   256 workgroups costs a whole round) split the k range instead: a
//   workgroup owns 32 tokens x 128 experts, or the fused tile's 32*MB
//   tokens x all experts, over one slice of k and writes float32 partial
//   logits; a second kernel adds the slices in a fixed order
//   (deterministic) and runs the same selection.  A cost model picks the
//   plan (plan_gate).  Split tiles are ordered so that the token tiles
//   sharing a W slice run on one XCD (one L2), and W crosses from HBM about
//   once.
#include <math.h>

#include "siggate_internal.h"

namespace siggate {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int KPAD = KC + 4;    // padded LDS row in floats: rows start 4 banks apart
constexpr int SPLIT_STAGES = 4; // chunks of global loads in flight in the split GEMM
constexpr int FLUSH_CHUNKS = 16; // chunks per float32 accumulation block

// Workgroup of NW waves: 4 expert quarters x WM token splits x KS k-splits.
// A k-split wave pair shares a tile and processes alternate halves of every
// chunk; their accumulators are added in a fixed order at the end.
template <int E, int MB, int NW>
struct Shape {
    static constexpr int NT = 64 * NW;          // threads per workgroup
    static constexpr int BM = 32 * MB;          // tokens per workgroup
    static constexpr int WM = MB < NW / 4 ? MB : NW / 4;   // token splits
    static constexpr int KS = NW / 4 / WM;      // k-splits (1 or 2)
    static constexpr int MBW = MB / WM;         // 32-token MFMA blocks per wave
    static constexpr int NB = E / 128;          // 32-expert MFMA blocks per wave
    static constexpr int WCOLS = E / 4;         // experts per wave
    static constexpr int V = E / 64;            // experts per lane in the selection
    static constexpr int LROW = E + 4;          // padded logits row (floats)
    static constexpr int STAGE = 2 * (E + BM) * KPAD;
    static constexpr int EPI = BM * LROW;
    static constexpr int SMEM = STAGE > EPI ? STAGE : EPI;
    static_assert(E % 128 == 0, "E must be a multiple of 128");
    static_assert(NW % 4 == 0 && MB % WM == 0 && (KS == 1 || KS == 2), "waves must tile the workgroup");
    static_assert(KC * BM / NT >= 2, "each thread stages at least 2 bfloat16 of x");
    static_assert(KS == 1 || 4 * MBW * NB * 16 * 64 <= SMEM, "k-split reduction fits in LDS");
};

// N packed bfloat16 pairs (one 32-bit word each)
template <int N> struct XVec { typedef unsigned int type __attribute__((ext_vector_type(N))); };
template <> struct XVec<1> { typedef unsigned int type; };

__device__ __forceinline__ float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

// Monotone map of a float to uint32 (larger float -> larger key; -inf is
// the smallest non-NaN key).
__device__ __forceinline__ uint32_t orderable(float f)
{
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float readlane_f(float v, int lane)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Lane exchanges through DPP (register crossbar of the VALU; no LDS round
// trip as with a shuffle).  Each pairs lane i with a partner inside its
// group of 4, 8 or 16 lanes, the groups split into disjoint halves, so
// repeated merges over xor1, xor2, the half-row mirror and the row mirror
// combine 2, 4, 8 and 16 lanes.
enum DppCtrl {
    DPP_XOR1 = 0xB1,          // quad_perm [1,0,3,2]
    DPP_XOR2 = 0x4E,          // quad_perm [2,3,0,1]
    DPP_HALF_MIRROR = 0x141,  // i <-> 7-i inside 8 lanes
    DPP_MIRROR = 0x140,       // i <-> 15-i inside 16 lanes
    DPP_BCAST15 = 0x142,      // lane 15 of a row to the whole next row
    DPP_BCAST31 = 0x143,      // lane 31 to rows 2 and 3
};
template <int CTRL>
__device__ __forceinline__ unsigned dpp_u(unsigned x)
{
    return (unsigned)__builtin_amdgcn_update_dpp((int)x, (int)x, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL,
                                                      0xF, 0xF, false));
}

// Largest and smallest x over the wave's 64 lanes (every lane gets both):
// merges inside rows of 16 lanes, then rows 0+1 into row 1 and 2+3 into
// row 3 (row_bcast:15; rows 0 and 2 keep their value), then rows 0..3 into
// row 3 (row_bcast:31), whose lane 63 holds the result.
__device__ __forceinline__ void wave_max_min(uint32_t &hi, uint32_t &lo)
{
    hi = max(hi, dpp_u<DPP_XOR1>(hi));
    lo = min(lo, dpp_u<DPP_XOR1>(lo));
    hi = max(hi, dpp_u<DPP_XOR2>(hi));
    lo = min(lo, dpp_u<DPP_XOR2>(lo));
    hi = max(hi, dpp_u<DPP_HALF_MIRROR>(hi));
    lo = min(lo, dpp_u<DPP_HALF_MIRROR>(lo));
    hi = max(hi, dpp_u<DPP_MIRROR>(hi));
    lo = min(lo, dpp_u<DPP_MIRROR>(lo));
    hi = max(hi, (unsigned)__builtin_amdgcn_update_dpp((int)hi, (int)hi, DPP_BCAST15, 0xA, 0xF, false));
    lo = min(lo, (unsigned)__builtin_amdgcn_update_dpp((int)lo, (int)lo, DPP_BCAST15, 0xA, 0xF, false));
    hi = max(hi, (unsigned)__builtin_amdgcn_update_dpp((int)hi, (int)hi, DPP_BCAST31, 0xC, 0xF, false));
    lo = min(lo, (unsigned)__builtin_amdgcn_update_dpp((int)lo, (int)lo, DPP_BCAST31, 0xC, 0xF, false));
    hi = (uint32_t)__builtin_amdgcn_readlane((int)hi, 63);
    lo = (uint32_t)__builtin_amdgcn_readlane((int)lo, 63);
}

// The two largest values of a lane set (m1 >= m2, multiplicity counted)
// merged with the partner lane's pair.
__device__ __forceinline__ void merge_top2(float &m1, float &m2, float o1, float o2)
{
    const float hi = fmaxf(m1, o1);
    const float lo = fminf(m1, o1);
    m2 = fmaxf(lo, fmaxf(m2, o2));
    m1 = hi;
}

// Selection for one token held by one wave.  Lane l owns experts
// [l*V, l*V + V) and their logits lg[].  `scratch` is wave-private LDS of at
// least 3 * MAX_TOPK words.  Writes row t of weights and indices.
//
// The K winners are the K largest choice scores under (v desc, id asc).
// Scores map to order-preserving uint32 keys; a threshold is found bit by
// bit from the top (a count of keys >= candidate is one ballot per owned
// expert) until it is the K-th largest key or exactly K keys reach it; then
// every key above it is selected and keys equal to it are taken in
// ascending expert id until K are chosen.
template <int V>
__device__ __forceinline__ void select_token(const float (&lg)[V], const float (&bias_r)[V],
                                             const int lane, const GateArgs &a, const int t,
                                             float *scratch)
{
    float s[V], v[V];
    if (a.score_func == 0) {
#pragma unroll
        for (int j = 0; j < V; ++j) s[j] = 1.0f / (1.0f + expf(-lg[j]));
    } else {
        // softmax over the E logits of the token (wave-wide max and sum; the
        // butterfly gives every lane the same bits)
        float mx = lg[0];
#pragma unroll
        for (int j = 1; j < V; ++j) mx = fmaxf(mx, lg[j]);
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
        float sum = 0.0f;
#pragma unroll
        for (int j = 0; j < V; ++j) {
            s[j] = expf(lg[j] - mx);
            sum += s[j];
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
#pragma unroll
        for (int j = 0; j < V; ++j) s[j] = s[j] / sum;
    }
    // without a bias, bias_r is 0 and v equals s
#pragma unroll
    for (int j = 0; j < V; ++j) v[j] = s[j] + bias_r[j];

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
        // merge over the group's lanes: DPP inside 16 lanes, shuffles
        // across rows (groups of 32 or 64 lanes)
        if (lpg >= 2) merge_top2(m1, m2, dpp_f<DPP_XOR1>(m1), dpp_f<DPP_XOR1>(m2));
        if (lpg >= 4) merge_top2(m1, m2, dpp_f<DPP_XOR2>(m1), dpp_f<DPP_XOR2>(m2));
        if (lpg >= 8) merge_top2(m1, m2, dpp_f<DPP_HALF_MIRROR>(m1), dpp_f<DPP_HALF_MIRROR>(m2));
        if (lpg >= 16) merge_top2(m1, m2, dpp_f<DPP_MIRROR>(m1), dpp_f<DPP_MIRROR>(m2));
        for (int off = 16; off < lpg; off <<= 1) merge_top2(m1, m2, __shfl_xor(m1, off), __shfl_xor(m2, off));
        // with a bias: top-2 sum; without: the group maximum
        const float gs = a.bias ? m1 + m2 : m1;
        const int g = lane / lpg;
        // Rank of this lane's group under (score desc, group index asc).
        int ahead = 0;
        for (int h = 0; h < G; ++h) {
            const float gh = readlane_f(gs, h * lpg);
            ahead += (gh > gs) || (gh == gs && h < g);
        }
        if (ahead >= a.topk_group) {
            const float fill = a.mask_zero ? 0.0f : -INFINITY;
#pragma unroll
            for (int j = 0; j < V; ++j) v[j] = fill;
        }
    }

    const int K = a.top_k;
    uint32_t key[V];
#pragma unroll
    for (int j = 0; j < V; ++j) key[j] = orderable(v[j] + 0.0f);   // -0 -> +0

    // Bracket the K-th largest key X: X <= the wave maximum hi, and, when at
    // least K lanes hold a key above -inf, X >= the K-th largest of those
    // lanes' maxima >= the smallest of them, lo.  X then shares every bit
    // above the first one where its bounds differ, so a search starts there
    // with those bits set.
    uint32_t lm = key[0];
#pragma unroll
    for (int j = 1; j < V; ++j) lm = max(lm, key[j]);
    const uint32_t none = orderable(-INFINITY);
    uint32_t hi = lm, lo = lm > none ? lm : 0xffffffffu;
    wave_max_min(hi, lo);
    uint32_t kth = 0;
    int b_top = 31;
    if (__popcll(__ballot(lm > none)) >= K) {
        // A tighter lower bound first: a key lk that at least K lane
        // maxima reach (the K-th largest lane maximum, or a prefix of it
        // that exactly K reach), by the same bit search over one key per
        // lane -- one compare per bit instead of V.  At least K keys reach
        // lk, so lk <= X.  If exactly K keys reach it -- the usual case: no
        // lane holds two of the winners -- those K are the winners and X
        // is not needed beyond lk.
        uint32_t diff = hi ^ lo;
        int bb = diff ? 31 - __clz(diff) : -1;
        uint32_t lk = bb < 0 ? hi : hi & ~(0xffffffffu >> (31 - bb));
        for (; bb >= 0; --bb) {
            const uint32_t cand = lk | (1u << bb);
            const int c = __popcll(__ballot(lm >= cand));
            if (c >= K) {
                lk = cand;
                if (c == K) break;
            }
        }
        int c0 = 0;
#pragma unroll
        for (int j = 0; j < V; ++j) c0 += __popcll(__ballot(key[j] >= lk));
        if (c0 == K) {
            kth = lk;
            b_top = -1;
        } else {
            diff = hi ^ lk;
            b_top = diff ? 31 - __clz(diff) : -1;
            kth = b_top < 0 ? hi : hi & ~(0xffffffffu >> (31 - b_top));
        }
    }

    // K-th largest key, most significant bit first.  Once exactly K keys
    // are >= the prefix found so far, those K are the winners and the lower
    // bits cannot change the choice: stop there (the counts are ballots, so
    // every lane takes the same branch).  (Two bits per step -- three
    // candidates counted at once -- measured slower: the loop is bound by
    // the issue of its compares and counts, not by their latency.)
    for (int b = b_top; b >= 0; --b) {
        const uint32_t cand = kth | (1u << b);
        int cnt = 0;
#pragma unroll
        for (int j = 0; j < V; ++j) cnt += __popcll(__ballot(key[j] >= cand));
        if (cnt >= K) {
            kth = cand;
            if (cnt == K) break;
        }
    }

    // Keys above kth are in; keys equal to kth fill the rest by ascending id
    // (id = lane*V + j, so lower lanes first, then lower j).
    const uint64_t below = (1ull << lane) - 1ull;
    int above = 0, eq_before = 0;
#pragma unroll
    for (int j = 0; j < V; ++j) {
        above += __popcll(__ballot(key[j] > kth));
        eq_before += __popcll(__ballot(key[j] == kth) & below);
    }
    const int need = K - above;
    bool sel[V];
    int sel_before = 0;
#pragma unroll
    for (int j = 0; j < V; ++j) {
        const bool eq = key[j] == kth;
        sel[j] = key[j] > kth || (eq && eq_before < need);
        eq_before += eq;
    }
#pragma unroll
    for (int j = 0; j < V; ++j) sel_before += __popcll(__ballot(sel[j]) & below);

    // Compact the winners in ascending id into scratch: [0,K) scores s,
    // [K,2K) ids, [2K,3K) keys.
    int p = sel_before;
#pragma unroll
    for (int j = 0; j < V; ++j) {
        if (sel[j]) {
            scratch[p] = s[j];
            scratch[MAX_TOPK + p] = __int_as_float(lane * V + j);
            scratch[2 * MAX_TOPK + p] = __uint_as_float(key[j]);
            ++p;
        }
    }
    __builtin_amdgcn_wave_barrier();

    // Renormalise over the K winners (unbiased s, summed in ascending id
    // order) and scale; lane k < K writes one entry.
    const bool renorm = a.renorm == 0 ? a.score_func == 0 : a.renorm == 1;
    float denom = 0.0f;
    for (int k = 0; k < K; ++k) denom += scratch[k];
    denom += a.denom_eps;
    if (lane < K) {
        const float my_s = scratch[lane];
        const int my_i = __float_as_int(scratch[MAX_TOPK + lane]);
        int pos = lane;
        if (a.order == 1) {   // choice score descending, id ascending on ties
            const uint32_t my_key = __float_as_uint(scratch[2 * MAX_TOPK + lane]);
            pos = 0;
            for (int k = 0; k < K; ++k) {
                const uint32_t kk = __float_as_uint(scratch[2 * MAX_TOPK + k]);
                pos += kk > my_key || (kk == my_key && k < lane);
            }
        }
        a.indices[(size_t)t * K + pos] = my_i;
        a.weights[(size_t)t * K + pos] = renorm ? my_s / denom * a.route_scale
                                                : my_s * a.route_scale;
    }
    __builtin_amdgcn_wave_barrier();
}

// Writes a finished BM x E logits tile: as partial or final logits, or
// through LDS (never HBM) into the selection, BM/NW tokens per wave.  ER is
// the number of real experts: the tile's columns past ER are padding (E
// rounded up to whole 128-expert tiles) and are neither written nor ranked.
template <int E, int MB, int NW, int MODE, int ER>
__device__ __forceinline__ void finish_tile(const GateArgs &a,
                                            f32x16 (&acc)[Shape<E, MB, NW>::MBW][Shape<E, MB, NW>::NB],
                                            float *smem, const int t0, const int e0, const int ks,
                                            const int wave, const int lane, const int wm,
                                            const bool has_acc)
{
    using S = Shape<E, MB, NW>;
    const int wn = wave & 3;
    // Accumulator element r of block (m, n) in lane l is token
    // (wm*MBW + m)*32 + 8*(r/4) + 4*(l/32) + r%4 and expert
    // e0 + wn*E/4 + n*32 + l%32 (E = experts of the tile).
    const int e_base = e0 + wn * S::WCOLS + (lane & 31);
    const int r_base = wm * S::MBW * 32 + 4 * (lane >> 5);

    if constexpr (MODE == MODE_PARTIAL || MODE == MODE_LOGITS) {
        // partial rows are e_stride long (whole tiles); final logits rows E
        const int stride = MODE == MODE_PARTIAL ? a.e_stride : a.E;
        float *out = MODE == MODE_PARTIAL ? a.partial + (size_t)ks * a.T * a.e_stride : a.logits;
#pragma unroll
        for (int m = 0; m < S::MBW; ++m)
#pragma unroll
            for (int n = 0; n < S::NB; ++n)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int t = t0 + m * 32 + 8 * (r >> 2) + r_base + (r & 3);
                    const bool real = MODE == MODE_PARTIAL || ER == E || e_base + n * 32 < ER;
                    if (has_acc && t < a.T && real) out[(size_t)t * stride + e_base + n * 32] = acc[m][n][r];
                }
    } else {
        // Scores go to LDS (never to HBM); each wave then selects for BM/NW
        // tokens.
        float *const Ls = smem;   // [BM][LROW]
        if (has_acc) {
#pragma unroll
            for (int m = 0; m < S::MBW; ++m)
#pragma unroll
                for (int n = 0; n < S::NB; ++n)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int row = m * 32 + 8 * (r >> 2) + r_base + (r & 3);
                        Ls[row * S::LROW + e_base + n * 32] = acc[m][n][r];
                    }
        }
        __syncthreads();

        constexpr int V = ER / 64;
        float bias_r[V];
#pragma unroll
        for (int j = 0; j < V; ++j) bias_r[j] = a.bias ? a.bias[lane * V + j] : 0.0f;

        for (int i = 0; i < S::BM / NW; ++i) {
            const int row = wave * (S::BM / NW) + i;
            const int t = t0 + row;
            if (t >= a.T) break;
            float lg[V];
#pragma unroll
            for (int j = 0; j < V; ++j) lg[j] = Ls[row * S::LROW + lane * V + j];
            // the row is dead once read: it doubles as the wave's scratch
            __builtin_amdgcn_wave_barrier();
            select_token<V>(lg, bias_r, lane, a, t, Ls + row * S::LROW);
        }
    }
}

// BLOCKED: flush the accumulators into the totals every FLUSH_CHUNKS chunks
// (long k ranges); without it only once, at the end (k-slices of at most
// 2 * FLUSH_CHUNKS chunks, whose chains the slicing already keeps short --
// the branch in the unrolled loop measurably slows those short tiles, and
// long split tiles run it with P = 2, where it costs least).
template <int E, int MB, int NW, int MODE, int P, bool BLOCKED, int ER = E>
__global__ __launch_bounds__(64 * NW) void gate_gemm_kernel(GateArgs a)
{
    using S = Shape<E, MB, NW>;
    constexpr int NT = S::NT;
    __shared__ __attribute__((aligned(16))) float smem[S::SMEM];
    float *const Ws = smem;                    // [2][E][KPAD]
    float *const Xs = smem + 2 * E * KPAD;     // [2][BM][KPAD]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wn = wave & 3;                    // expert quarter of this wave
    const int wm = (wave >> 2) % S::WM;         // token split of this wave
    const int wk = (wave >> 2) / S::WM;         // k-split of this wave
    int t0, e0 = 0, ks = 0;
    if constexpr (MODE == MODE_PARTIAL) {
        // Workgroup ids go round-robin over the 8 XCDs; each XCD gets one
        // contiguous run of tile numbers (the grid is a multiple of 8).
        // Tile numbers run token tile fastest, then expert tile, then
        // k-slice, so the token tiles that read one W slice share an L2.
        const int q = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
        if (q >= a.n_tiles) return;   // padding of the grid (whole workgroup)
        const int r = q / a.t_tiles;
        t0 = (q - r * a.t_tiles) * S::BM;
        ks = r / a.e_tiles;
        e0 = (r - ks * a.e_tiles) * E;
    } else {
        t0 = blockIdx.x * S::BM;
    }
    const int d = a.d;
    const int c_begin = ks * a.chunks_per_split;
    const int c_end = min(c_begin + a.chunks_per_split, a.chunks_total);

    // ---- global -> register staging.  Thread tid loads W rows
    // (tid/8) + (NT/8) i, 4 floats at column (tid%8)*4, and x row tid/XT, KC/XT
    // bfloat16 at column (tid%XT)*(KC/XT).  The steady-state loop has no
    // branches: columns past d (last chunk only) read a clamped in-range
    // address, and their x values are zeroed when written to LDS, so the
    // (finite) W values there multiply zero; rows past T read row T-1 and
    // their logits are dropped.
    constexpr int WLOADS = E * 8 / NT;
    constexpr int XT = NT / S::BM;          // threads per x row: 4, 8 or 16
    constexpr int XE = KC / XT;             // bfloat16 per thread: 8, 4 or 2
    typedef typename XVec<XE / 2>::type xvec;
    struct Stage {
        f32x4 w[WLOADS];
        xvec x;
    };
    const int w_row = tid >> 3;
    const int w_col = (tid & 7) * 4;
    const int x_row = tid / XT;
    const int x_col = (tid % XT) * XE;
    const int x_t = min(t0 + x_row, a.T - 1);
    const float *const Wp = a.W + (size_t)(e0 + w_row) * d;
    const uint16_t *const Xp = a.x + (size_t)x_t * d;

    // Expert rows past E -- when E is an odd multiple of 64, the last 64
    // rows of the last tile, which pad it to 128 -- are never read: that row
    // block reads the tile's first rows instead and is stored as zeros, so
    // the padding logits are 0 (and are dropped).
    constexpr bool MAYPAD = MODE == MODE_PARTIAL || ER != E;
    const bool pad_last = MAYPAD && e0 + (NT / 8) * (WLOADS - 1) >= a.E;
    const size_t last_off = pad_last ? 0 : (size_t)(WLOADS - 1) * (NT / 8) * d;
    auto load_global = [&](int c, Stage &st) {
        const int k0 = c * KC;
        const int wc = min(k0 + w_col, d - 4);
        const int xc = min(k0 + x_col, d - XE);
#pragma unroll
        for (int i = 0; i < WLOADS; ++i) {
            const size_t off = MAYPAD && i == WLOADS - 1 ? last_off : (size_t)i * (NT / 8) * d;
            st.w[i] = *(const f32x4 *)(Wp + off + wc);
        }
        st.x = *(const xvec *)(Xp + xc);
    };
    auto store_lds = [&](int c, int buf, const Stage &st) {
        const int k0 = c * KC;
        const bool xk = k0 + x_col < d;
        float *wb = Ws + buf * E * KPAD;
#pragma unroll
        for (int i = 0; i < WLOADS; ++i) {
            const bool zero = MAYPAD && i == WLOADS - 1 && pad_last;
            *(f32x4 *)(wb + (w_row + (NT / 8) * i) * KPAD + w_col) =
                zero ? f32x4{0.0f, 0.0f, 0.0f, 0.0f} : st.w[i];
        }
        float *xb = Xs + buf * S::BM * KPAD + x_row * KPAD + x_col;
        if constexpr (XE >= 4) {
#pragma unroll
            for (int h = 0; h < XE / 4; ++h) {
                const unsigned u0 = xk ? st.x[2 * h] : 0u;
                const unsigned u1 = xk ? st.x[2 * h + 1] : 0u;
                *(f32x4 *)(xb + 4 * h) = f32x4{bf16_lo(u0), bf16_hi(u0), bf16_lo(u1), bf16_hi(u1)};
            }
        } else {
            typedef float f32x2 __attribute__((ext_vector_type(2)));
            const unsigned u0 = xk ? st.x : 0u;
            *(f32x2 *)xb = f32x2{bf16_lo(u0), bf16_hi(u0)};
        }
    };

    // ---- MFMA main loop.  For a group of 8 k-columns, lane l reads 4
    // consecutive k of row (l%32) at offset 4*(l/32); MFMA j pairs column j
    // (lanes 0-31) with column 4+j (lanes 32-63) for A and B alike.
    f32x16 acc[S::MBW][S::NB];
#pragma unroll
    for (int m = 0; m < S::MBW; ++m)
#pragma unroll
        for (int n = 0; n < S::NB; ++n)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[m][n][r] = 0.0f;
    // A wave with a single 32x32 block alternates two accumulators (odd and
    // even k-pairs), so consecutive MFMAs never wait on each other.
    constexpr bool TWO_ACC = S::MBW * S::NB == 1;
    f32x16 acc2;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc2[r] = 0.0f;
    // Blocked summation: every FLUSH_CHUNKS chunks the accumulators are
    // added into float32 totals and restarted from zero, so no rounding
    // chain is longer than FLUSH_CHUNKS chunks (one chain over all of d=7168
    // would be 3584 dependent additions).  Every wave flushes at the same
    // chunks, so equal W rows still give bit-equal logits.  Short k-slices
    // (not BLOCKED) add their accumulators into the totals once, at the end.
    f32x16 tot[S::MBW][S::NB];
#pragma unroll
    for (int m = 0; m < S::MBW; ++m)
#pragma unroll
        for (int n = 0; n < S::NB; ++n)
#pragma unroll
            for (int r = 0; r < 16; ++r) tot[m][n][r] = 0.0f;
    auto flush = [&]() {
#pragma unroll
        for (int m = 0; m < S::MBW; ++m)
#pragma unroll
            for (int n = 0; n < S::NB; ++n)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    tot[m][n][r] += acc[m][n][r];
                    acc[m][n][r] = 0.0f;
                }
        if constexpr (TWO_ACC) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                tot[0][0][r] += acc2[r];
                acc2[r] = 0.0f;
            }
        }
    };

    const int f_row = lane & 31;
    const int f_k = (lane >> 5) * 4;
    // Operand fragments of one 8-column group, and their MFMAs.
    struct Frag {
        f32x4 a[S::MBW];
        f32x4 b[S::NB];
    };
    auto read_frag = [&](int buf, int c8, Frag &f) {
        const float *xb = Xs + buf * S::BM * KPAD + wm * S::MBW * 32 * KPAD;
        const float *wb = Ws + buf * E * KPAD + wn * S::WCOLS * KPAD;
#pragma unroll
        for (int m = 0; m < S::MBW; ++m)
            f.a[m] = *(const f32x4 *)(xb + (m * 32 + f_row) * KPAD + c8 * 8 + f_k);
#pragma unroll
        for (int n = 0; n < S::NB; ++n)
            f.b[n] = *(const f32x4 *)(wb + (n * 32 + f_row) * KPAD + c8 * 8 + f_k);
    };
    auto mma = [&](const Frag &f) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int m = 0; m < S::MBW; ++m)
#pragma unroll
                for (int n = 0; n < S::NB; ++n) {
                    if (TWO_ACC && (j & 1))
                        acc2 = __builtin_amdgcn_mfma_f32_32x32x2f32(f.a[m][j], f.b[n][j], acc2,
                                                                    0, 0, 0);
                    else
                        acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x2f32(f.a[m][j], f.b[n][j],
                                                                         acc[m][n], 0, 0, 0);
                }
    };
    static_assert(KC == 32, "the step below is written for four 8-column groups");

    // Pipeline over KC-column chunks.  While chunk c feeds the matrix cores
    // from one LDS buffer, chunks c+1 .. c+P wait in P register stages.
    // After the first 8-column group of chunk c, chunk c+1 is written to the
    // other LDS buffer and its register stage is refilled with chunk c+1+P,
    // so every global load has P chunks of MFMA work to land in (P = 2 for
    // the long fused tiles and long k-slices; 4 for the short split tiles,
    // whose chunks are a sixth as long).  The one barrier per chunk comes once the last
    // fragments of chunk c are in registers: the MFMAs of that last group
    // then cover the LDS latency of the first fragments of chunk c+1.  Local
    // chunk i uses LDS buffer i%2 and stage (i+1)%P, so the loop is unrolled
    // by lcm(P, 2) to keep both indices static.  Past the last chunk, loads
    // and stores repeat the last chunk (never read) instead of branching.
    if (c_begin < c_end) {
        const int c_last = c_end - 1;
        Stage st[P];
        Frag f, g;
        // this wave's 8-column groups of every chunk: g0 .. g0 + 4/KS - 1
        const int g0 = wk * (4 / S::KS);
        // Issue order inside a step (one wave, KS == 1): one memory
        // operation after each MFMA, so no group waits on its fragments and
        // the LDS stores and global loads hide under matrix work.  Groups
        // 0..2 of the chunk run before the barrier: group 0 alongside the
        // fragment reads of group 1 and the LDS stores of chunk c+1, group 1
        // alongside the global loads of chunk c+1+P and the reads of group
        // 2, group 2 alongside the reads of group 3; group 3 runs after the
        // barrier alongside the reads of the next chunk's group 0.
        constexpr int NMG = 4 * S::MBW * S::NB;               // MFMAs per group
        constexpr int NRG = S::MBW + S::NB;                   // fragment reads per group
        constexpr int NWR = WLOADS + (XE >= 4 ? XE / 4 : 1);  // LDS stores per chunk
        constexpr int NVM = WLOADS + 1;                       // global loads per chunk
        constexpr int SG_MFMA = 0x008, SG_VMEM_READ = 0x020, SG_DS_READ = 0x100,
                      SG_DS_WRITE = 0x200;
        auto interleave_body = [&]() {
#pragma unroll
            for (int i = 0; i < NMG; ++i) {
                __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
                if (i < NRG) __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
                else if (i - NRG < NWR) __builtin_amdgcn_sched_group_barrier(SG_DS_WRITE, 1, 0);
            }
#pragma unroll
            for (int i = 0; i < NMG; ++i) {
                __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
                if (i < NVM) __builtin_amdgcn_sched_group_barrier(SG_VMEM_READ, 1, 0);
                else if (i - NVM < NRG) __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
            }
#pragma unroll
            for (int i = 0; i < NMG; ++i) {
                __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
                if (i < NRG) __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
            }
        };
        // k-split pair (KS == 2): each wave has one group before the barrier;
        // its MFMAs carry the reads of the wave's second group, the LDS
        // stores and the global loads, spread evenly.
        auto interleave_split = [&]() {
            constexpr int OPS = NRG + NWR + NVM;
            constexpr int PER = (OPS + NMG - 1) / NMG;
#pragma unroll
            for (int i = 0; i < NMG; ++i) {
                __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
#pragma unroll
                for (int k = i * PER; k < (i + 1) * PER && k < OPS; ++k) {
                    if (k < NRG) __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
                    else if (k < NRG + NWR) __builtin_amdgcn_sched_group_barrier(SG_DS_WRITE, 1, 0);
                    else __builtin_amdgcn_sched_group_barrier(SG_VMEM_READ, 1, 0);
                }
            }
        };
        auto interleave_tail = [&]() {
#pragma unroll
            for (int i = 0; i < NMG; ++i) {
                __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
                if (i < NRG) __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
            }
        };
        auto step = [&](int c, int buf, Stage &sg) {
            // f holds group g0 of chunk c; sg holds chunk c+1
            read_frag(buf, g0 + 1, g);
            mma(f);
            store_lds(min(c + 1, c_last), buf ^ 1, sg);
            load_global(min(c + 1 + P, c_last), sg);
            if constexpr (S::KS == 1) {
                read_frag(buf, 2, f);
                mma(g);
                read_frag(buf, 3, g);
                mma(f);
                interleave_body();
            } else {
                interleave_split();
            }
            // keep the last group's MFMAs after the barrier (the scheduler
            // would otherwise hoist them and expose the LDS latency below)
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();
            __builtin_amdgcn_sched_barrier(0);
            read_frag(buf ^ 1, g0, f);   // first group of chunk c+1
            mma(g);
            interleave_tail();
        };
        load_global(c_begin, st[0]);
#pragma unroll
        for (int j = 1; j < P; ++j) load_global(min(c_begin + j, c_last), st[j]);
        store_lds(c_begin, 0, st[0]);
        load_global(min(c_begin + P, c_last), st[0]);
        __syncthreads();
        read_frag(0, g0, f);
        constexpr int U = P % 2 ? 2 * P : P;
        static_assert(FLUSH_CHUNKS % U == 0, "flushes fall between unrolled steps");
        int c = c_begin;
        for (; c + U <= c_end; c += U) {
#pragma unroll
            for (int u = 0; u < U; ++u) step(c + u, u & 1, st[(u + 1) % P]);
            if constexpr (BLOCKED) {
                if ((c + U - c_begin) % FLUSH_CHUNKS == 0) flush();
            }
        }
#pragma unroll
        for (int u = 0; u < U - 1; ++u)
            if (c + u < c_end) step(c + u, u & 1, st[(u + 1) % P]);
        __syncthreads();   // every wave is done with the staging buffers
    }

    flush();
#pragma unroll
    for (int m = 0; m < S::MBW; ++m)
#pragma unroll
        for (int n = 0; n < S::NB; ++n) acc[m][n] = tot[m][n];

    if constexpr (S::KS == 2) {
        // k-split pair: the second wave hands its sums to the first, which
        // adds them after its own (fixed order)
        constexpr int REGS = S::MBW * S::NB * 16;
        float *red = smem + wn * REGS * 64 + lane;
        if (wk == 1) {
#pragma unroll
            for (int m = 0; m < S::MBW; ++m)
#pragma unroll
                for (int n = 0; n < S::NB; ++n)
#pragma unroll
                    for (int r = 0; r < 16; ++r) red[((m * S::NB + n) * 16 + r) * 64] = acc[m][n][r];
        }
        __syncthreads();
        if (wk == 0) {
#pragma unroll
            for (int m = 0; m < S::MBW; ++m)
#pragma unroll
                for (int n = 0; n < S::NB; ++n)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[m][n][r] += red[((m * S::NB + n) * 16 + r) * 64];
        }
        __syncthreads();
    }

    finish_tile<E, MB, NW, MODE, ER>(a, acc, smem, t0, e0, ks, wave, lane, wm, wk == 0);
}

// V consecutive floats from p (p 8-byte aligned when V is even, 16-byte
// when V is a multiple of 4; single loads for odd V).
template <int V>
__device__ __forceinline__ void load_row(const float *p, float (&v)[V])
{
    if constexpr (V % 4 == 0) {
#pragma unroll
        for (int h = 0; h < V / 4; ++h) {
            const f32x4 q = *(const f32x4 *)(p + 4 * h);
#pragma unroll
            for (int i = 0; i < 4; ++i) v[4 * h + i] = q[i];
        }
    } else if constexpr (V % 2 == 0) {
        typedef float f32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
        for (int h = 0; h < V / 2; ++h) {
            const f32x2 q = *(const f32x2 *)(p + 2 * h);
            v[2 * h] = q[0];
            v[2 * h + 1] = q[1];
        }
    } else {
#pragma unroll
        for (int h = 0; h < V; ++h) v[h] = p[h];
    }
}

// A token's summed logits: written out, or through the selection (bias_r:
// this lane's bias values, loaded at kernel entry so that their latency
// overlaps the partial loads instead of following the sum).
template <int V, int MODE>
__device__ __forceinline__ void finish_reduce(const GateArgs &a, const float (&lg)[V],
                                              const float (&bias_r)[V], const int lane, const int t,
                                              float *scratch)
{
    constexpr int E = V * 64;
    if constexpr (MODE == MODE_LOGITS) {
#pragma unroll
        for (int j = 0; j < V; ++j) a.logits[(size_t)t * E + lane * V + j] = lg[j];
    } else {
        select_token<V>(lg, bias_r, lane, a, t, scratch);
    }
}

constexpr int ONE_WAVE_SLICES = 24;

// Adds the n_split partial logits of one token in a fixed order -- wave w
// of NWR sums its contiguous run of slices in ascending order, then wave 0
// adds the runs in wave order -- and writes the logits or runs the
// selection.  One workgroup per token; lane l owns experts [l*V, l*V + V).
template <int E, int MODE, int NWR>
__global__ __launch_bounds__(64 * NWR) void gate_reduce_kernel(GateArgs a)
{
    constexpr int V = E / 64;
    constexpr int U = 4;   // slices loaded before they are added
    __shared__ float part[NWR][E];
    __shared__ float scratch[3 * MAX_TOPK];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int t = blockIdx.x;
    const int per = (a.n_split + NWR - 1) / NWR;
    const int s0 = min(wave * per, a.n_split);
    const int s1 = min(s0 + per, a.n_split);
    // partial rows are e_stride floats long (E rounded up to whole tiles)
    const float *const p = a.partial + (size_t)t * a.e_stride + lane * V;
    const size_t slice = (size_t)a.T * a.e_stride;
    float bias_r[V];
#pragma unroll
    for (int j = 0; j < V; ++j) bias_r[j] = MODE == MODE_SELECT && a.bias ? a.bias[lane * V + j] : 0.0f;
    float lg[V];
#pragma unroll
    for (int j = 0; j < V; ++j) lg[j] = 0.0f;
    if constexpr (NWR == 1) {
        if (a.n_split == 1) {   // a single slice: the logits themselves
            load_row<V>(p, lg);
            finish_reduce<V, MODE>(a, lg, bias_r, lane, t, scratch);
            return;
        }
        // one wave, at most ONE_WAVE_SLICES slices: every load is issued
        // before the first add
        float q[ONE_WAVE_SLICES][V];
#pragma unroll
        for (int u = 0; u < ONE_WAVE_SLICES; ++u) {
            if (u < a.n_split) {
                load_row<V>(p + (size_t)u * slice, q[u]);
            } else {
#pragma unroll
                for (int j = 0; j < V; ++j) q[u][j] = 0.0f;
            }
        }
#pragma unroll
        for (int u = 0; u < ONE_WAVE_SLICES; ++u)
            if (u < a.n_split) {
#pragma unroll
                for (int j = 0; j < V; ++j) lg[j] += q[u][j];
            }
        finish_reduce<V, MODE>(a, lg, bias_r, lane, t, scratch);
        return;
    }
    int s = s0;
    for (; s + U <= s1; s += U) {
        float q[U][V];
#pragma unroll
        for (int u = 0; u < U; ++u) load_row<V>(p + (size_t)(s + u) * slice, q[u]);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int j = 0; j < V; ++j) lg[j] += q[u][j];
    }
    for (; s < s1; ++s) {
        float q[V];
        load_row<V>(p + (size_t)s * slice, q);
#pragma unroll
        for (int j = 0; j < V; ++j) lg[j] += q[j];
    }
#pragma unroll
    for (int j = 0; j < V; ++j) part[wave][lane * V + j] = lg[j];
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 1; w < NWR; ++w)
#pragma unroll
        for (int j = 0; j < V; ++j) lg[j] += part[w][lane * V + j];
    finish_reduce<V, MODE>(a, lg, bias_r, lane, t, scratch);
}

// Largest E with 64-token fused tiles: their double-buffered stage of W and x,
// 2*(E + 64)*KPAD floats, exceeds the 160 KB of LDS at E = 512 (162 KB),
// where the fused path uses 32-token tiles only.
constexpr int MAX_E_TILE64 = 384;

// Split GEMM on the fused kernel's full-E tiles (32 or 64 tokens x all
// experts x one k-slice), writing partial logits.
template <int E, int ER>
hipError_t launch_wide(const GateArgs &a, const GatePlan &p, hipStream_t stream)
{
    const dim3 grid(p.grid), block(64 * 8);
    if constexpr (E <= MAX_E_TILE64) {
        if (p.m_blocks == 2)
            return launch_kernel(gate_gemm_kernel<E, 2, 8, MODE_PARTIAL, 2, true, ER>, grid, block, stream, a);
        return launch_kernel(gate_gemm_kernel<E, 1, 8, MODE_PARTIAL, 2, true, ER>, grid, block, stream, a);
    } else {
        return launch_kernel(gate_gemm_kernel<E, 1, 8, MODE_PARTIAL, 1, true, ER>, grid, block, stream, a);
    }
}

// E: the GEMM's expert tile width (whole 128-expert tiles); ER: the real
// expert count (E, or E - 64 when that is an odd multiple of 64).
template <int E, int ER>
hipError_t launch_for_e(const GateArgs &a, const GatePlan &p, GateMode final_mode,
                        hipStream_t stream)
{
    const bool sel = final_mode == MODE_SELECT;
    if (!p.split) {
        // 64 tokens: 8 waves, two per SIMD; 32 tokens: 8 waves, the two of a
        // pair split every chunk's k
        const dim3 grid(p.grid), block(64 * 8);
        if constexpr (E <= MAX_E_TILE64) {
            if (p.m_blocks == 2)
                return sel ? launch_kernel(gate_gemm_kernel<E, 2, 8, MODE_SELECT, 2, true, ER>, grid, block, stream, a)
                           : launch_kernel(gate_gemm_kernel<E, 2, 8, MODE_LOGITS, 2, true, ER>, grid, block, stream, a);
        }
        // one register stage of loads ahead at E = 512, where two would spill
        constexpr int P1 = E > MAX_E_TILE64 ? 1 : 2;
        return sel ? launch_kernel(gate_gemm_kernel<E, 1, 8, MODE_SELECT, P1, true, ER>, grid, block, stream, a)
                   : launch_kernel(gate_gemm_kernel<E, 1, 8, MODE_LOGITS, P1, true, ER>, grid, block, stream, a);
    }
    // split GEMM: 32 tokens x 128 experts, 8 waves (two per SIMD): 4 columns
    // of 32 experts x 2 k-halves of every chunk; or the bfloat16 three-way
    // route, which writes the same partials
    hipError_t e;
    if (p.x3_bm)
        e = launch_x3_gemm(a, p, stream);
    else if (p.wide)   // the fused kernel's full-E tiles, k-sliced
        e = launch_wide<E, ER>(a, p, stream);
    else if (p.chunks_per_split > 2 * FLUSH_CHUNKS)   // long k-slices: blocked, 2 stages
        e = launch_kernel(gate_gemm_kernel<128, 1, 8, MODE_PARTIAL, 2, true>,
                          dim3(p.grid), dim3(64 * 8), stream, a);
    else
        e = launch_kernel(gate_gemm_kernel<128, 1, 8, MODE_PARTIAL, SPLIT_STAGES, false>,
                          dim3(p.grid), dim3(64 * 8), stream, a);
    if (e != hipSuccess) return e;
    // few slices: one wave per token loads them all at once; more: 16 waves
    // per token (8 at E = 512, whose selection needs more than the 128
    // registers a 16-wave workgroup leaves a wave), each loading a
    // contiguous run of them
    const dim3 rgrid(a.T);
    if (p.n_split <= ONE_WAVE_SLICES)
        return sel ? launch_kernel(gate_reduce_kernel<ER, MODE_SELECT, 1>, rgrid, dim3(64), stream, a)
                   : launch_kernel(gate_reduce_kernel<ER, MODE_LOGITS, 1>, rgrid, dim3(64), stream, a);
    constexpr int NWR = ER > MAX_E_TILE64 ? 8 : 16;
    return sel ? launch_kernel(gate_reduce_kernel<ER, MODE_SELECT, NWR>, rgrid, dim3(64 * NWR), stream, a)
               : launch_kernel(gate_reduce_kernel<ER, MODE_LOGITS, NWR>, rgrid, dim3(64 * NWR), stream, a);
}

}  // namespace

// Cost model of the split GEMM, in units of one KC-chunk of a 32-token x
// 128-expert tile on one compute unit (1024 MFMA cycles, about 0.45 us):
// a workgroup costs its chunks + SPLIT_LATENCY, workgroups beyond one per
// compute unit queue behind it, and the partial logits cross HBM twice
// (written, then read by the reduction) at about SPLIT_BYTES_PER_UNIT bytes
// per unit.  (64-token split tiles measured no better overall.)
constexpr double SPLIT_LATENCY = 4.0;
constexpr double SPLIT_BYTES_PER_UNIT = 2.25e6;
constexpr int N_CU = 256;
// Wide and fused tiles, in the same units: a chunk costs WIDE_CHUNK_32
// (32-token tile) or WIDE_CHUNK_64 (64-token tile) per 128 experts, a
// workgroup WIDE_LATENCY, and the partials cross memory at
// WIDE_BYTES_PER_UNIT; a split plan (either tile kind) also pays
// REDUCE_LAUNCH for its reduction kernel, which the fused tiles (whole k,
// selection in the epilogue) do not need.  Fitted, with the 32 x 128 model
// above unchanged, to graph-replayed gate times over forced plans (every
// tile kind and slice count filling 128 to 1024 workgroups, and both fused
// heights; T = 256 ... 24576, E = 64 ... 512): the planner's summed excess
// over the best measured plan is 65 us over 61 configurations, 0.3% of
// their summed time.
constexpr double WIDE_CHUNK_32 = 0.9;
constexpr double WIDE_CHUNK_64 = 1.5;
constexpr double WIDE_LATENCY = 12.0;
constexpr double WIDE_BYTES_PER_UNIT = 5.0e6;
constexpr double REDUCE_LAUNCH = 10.0;
// Largest partial logits a float32 plan may need (so that every batch fits
// the 128 MiB scratch of the no-allocation entry point, and the workspace
// stays modest): plans above it are skipped.
constexpr size_t MAX_PARTIAL_BYTES = (size_t)120 << 20;

GatePlan plan_gate(int T, int d, int E, int path)
{
    if (path == PATH_BF16X3) return plan_x3(T, d, E);
    GatePlan p{};
    // the GEMM's expert tiles are whole 128-expert tiles
    const int EP = (E + 127) / 128 * 128;
    p.e_stride = EP;
    const int chunks = (d + KC - 1) / KC;
    const long tiles32 = ((long)T + 31) / 32;
    const int max_mb = EP <= MAX_E_TILE64 ? 2 : 1;
    p.n_split = 1;
    p.chunks_per_split = chunks;
    p.e_tiles = 1;
    double best = 1e300;
    // Fused tiles: one workgroup per 32- or 64-token tile, all experts,
    // whole k range, selection in the epilogue.  They win once the tiles
    // fill whole rounds of N_CU workgroups; a partly filled last round costs
    // a whole one, which a k-split of the same tiles can avoid.
    for (int mb = 1; mb <= max_mb; ++mb) {
        const long wt = ((long)T + 32 * mb - 1) / (32 * mb);
        const double units = (double)(EP / 128) * (mb == 2 ? WIDE_CHUNK_64 : WIDE_CHUNK_32);
        const double cost = (double)((wt + N_CU - 1) / N_CU) * (chunks * units + WIDE_LATENCY);
        if (cost < best) {
            best = cost;
            p.m_blocks = mb;
            p.t_tiles = (int)wt;
        }
    }
    // Split GEMM on 32-token x 128-expert tiles
    const long tiles = tiles32 * (EP / 128);
    int split_s = 0, split_cps = 0;
    for (int s = 1; s <= chunks; ++s) {
        const int cps = (chunks + s - 1) / s;
        if ((chunks + cps - 1) / cps != s) continue;   // s slices of cps chunks
        if ((size_t)s * T * EP * sizeof(float) > MAX_PARTIAL_BYTES) break;
        const long n = tiles * s;
        const double rounds = (double)((n + N_CU - 1) / N_CU);
        const double cost = rounds * (cps + SPLIT_LATENCY) +
                            2.0 * s * (double)T * EP * sizeof(float) / SPLIT_BYTES_PER_UNIT +
                            REDUCE_LAUNCH;
        if (cost < best) {
            best = cost;
            split_s = s;
            split_cps = cps;
        }
    }
    if (split_s) {
        p.split = true;
        p.m_blocks = 1;
        p.t_tiles = (int)tiles32;
        p.e_tiles = EP / 128;
        p.n_split = split_s;
        p.chunks_per_split = split_cps;
    }
    // Wide tiles: the fused kernel's 32*mb tokens x all EP experts, k-sliced.
    // Each W slice then serves more tokens and each x slice all experts, so a
    // chunk carries more matrix work per LDS stage and barrier.
    for (int mb = 1; mb <= max_mb; ++mb) {
        const long wt = ((long)T + 32 * mb - 1) / (32 * mb);
        const double units = (double)(EP / 128) * (mb == 2 ? WIDE_CHUNK_64 : WIDE_CHUNK_32);
        for (int s = 1; s <= chunks; ++s) {
            const int cps = (chunks + s - 1) / s;
            if ((chunks + cps - 1) / cps != s) continue;
            if ((size_t)s * T * EP * sizeof(float) > MAX_PARTIAL_BYTES) break;
            const long n = wt * s;
            const double rounds = (double)((n + N_CU - 1) / N_CU);
            const double cost = rounds * (cps * units + WIDE_LATENCY) +
                                2.0 * s * (double)T * EP * sizeof(float) / WIDE_BYTES_PER_UNIT +
                                REDUCE_LAUNCH;
            if (cost < best) {
                best = cost;
                p.split = true;
                p.wide = true;
                p.m_blocks = mb;
                p.n_split = s;
                p.chunks_per_split = cps;
                p.t_tiles = (int)wt;
                p.e_tiles = 1;
            }
        }
    }
    if (!p.split) {
        p.grid = p.t_tiles;
        return p;
    }
    const long n = (long)p.t_tiles * p.e_tiles * p.n_split;
    p.grid = (int)((n + 7) / 8 * 8);
    p.partial_bytes = (size_t)p.n_split * (size_t)T * (size_t)EP * sizeof(float);
    return p;
}

hipError_t launch_gate(const GateArgs &a, const GatePlan &p, int E, GateMode final_mode,
                       hipStream_t stream)
{
    switch (E) {
    case 64: return launch_for_e<128, 64>(a, p, final_mode, stream);
    case 128: return launch_for_e<128, 128>(a, p, final_mode, stream);
    case 192: return launch_for_e<256, 192>(a, p, final_mode, stream);
    case 256: return launch_for_e<256, 256>(a, p, final_mode, stream);
    case 320: return launch_for_e<384, 320>(a, p, final_mode, stream);
    case 384: return launch_for_e<384, 384>(a, p, final_mode, stream);
    case 448: return launch_for_e<512, 448>(a, p, final_mode, stream);
    case 512: return launch_for_e<512, 512>(a, p, final_mode, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace siggate
