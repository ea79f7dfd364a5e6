// logits_x3.hip -- router logits x.W^T on the bfloat16 matrix cores of
// gfx950, exact to float32 working precision, for the gate of gate.hip.
//
// What is computed (DeepSeek-V3.2-Exp · Normalize weights, "Code": Gate
// forward; Kimi K2 · Normalize weights, the equation for s_{i,t}): the same
// float32 logits L[t,e] = sum_k x[t,k] * W[e,k] as the float32 GEMM of
// gate.hip, by another route.
//
// The route.  x is bfloat16, so it is exact on the bfloat16 matrix cores.
// Every float32 weight splits exactly into three bfloat16 parts,
//   W = hi + mid + lo,
// hi = W with its low 16 bits cleared (the sign, the exponent and the top 8
// significant bits), mid the same of the remainder W - hi, and lo = W - hi -
// mid, which has at most 8 significant bits left and is itself a bfloat16.
// Each of the three differences is exact (the operands share sign and
// exponent range), so the split loses nothing.  A nonzero part can be as
// small as the last significant bit of W, 2^-23 |W| rounded down to a power
// of two, so every part is a normal number for |W| >= 2^-103; below that a
// part may be subnormal, and exactness then rests on the matrix cores
// keeping subnormal bfloat16 inputs.  The products x*hi, x*mid and x*lo are exact in float32
// (8 x 8 significant bits), and v_mfma_f32_16x16x32_bf16 adds them into
// float32 accumulators, so L carries float32 accumulation error only, as on
// the float32 matrix cores, at 16x their per-instruction rate (3 products
// per term: about 5x the arithmetic rate of the float32 route).
//
// Layout of the work.  A workgroup of 8 waves (two per SIMD: one wave per
// SIMD cannot issue these MFMAs back to back at full rate) owns BM tokens x
// BN = 64*NBW experts x one slice of the k range, and writes float32 partial
// logits [n_split, T, E]; the reduction of gate.hip adds the slices in a
// fixed order and runs the selection.  The waves are 4 expert quarters x 2
// k-halves of every 64-column chunk, so no W element is loaded by two waves:
// each wave loads its W fragments straight into registers (no LDS for W).
// x, shared by the waves, is staged in LDS as bfloat16.  Large batches read
// W as three bfloat16 planes split once per call by x3_split_w_kernel;
// small batches split float32 W in registers.  Tiles are ordered as in the
// split GEMM of gate.hip: token tile fastest, and one contiguous run of
// tiles per XCD, so the tiles that read one W slice share an L2.
#include "siggate_internal.h"

namespace siggate {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Two bfloat16 (the upper halves of two float32 bit patterns whose low
// halves are zero) packed into one word: a in the low half, b in the high.
__device__ __forceinline__ unsigned pack_hi(unsigned a, unsigned b)
{
    return (a >> 16) | (b & 0xffff0000u);
}

// The exact three-way split of 8 float32 weights (two float4) into three
// vectors of 8 bfloat16 (hi, mid, lo), element order preserved.
__device__ __forceinline__ void split3(const f32x4 &w0, const f32x4 &w1, u32x4 &hi, u32x4 &mid,
                                       u32x4 &lo)
{
    unsigned h[8], m[8], l[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float w = i < 4 ? w0[i] : w1[i - 4];
        const unsigned hu = __float_as_uint(w) & 0xffff0000u;
        const float r = w - __uint_as_float(hu);           // exact
        const unsigned mu = __float_as_uint(r) & 0xffff0000u;
        const float lw = r - __uint_as_float(mu);          // exact, a bfloat16
        h[i] = hu;
        m[i] = mu;
        l[i] = __float_as_uint(lw);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        hi[j] = pack_hi(h[2 * j], h[2 * j + 1]);
        mid[j] = pack_hi(m[2 * j], m[2 * j + 1]);
        lo[j] = pack_hi(l[2 * j], l[2 * j + 1]);
    }
}

__device__ __forceinline__ f32x4 mfma_bf16(const u32x4 &a, const u32x4 &b, const f32x4 &c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// The three bfloat16 planes of W (hi, mid, lo) for the pre-split GEMM, in
// MFMA fragment order: fragment (eb, c) of a plane holds experts
// 16*eb .. 16*eb+15 and k-columns 32*c .. 32*c+31 as 64 lanes x 8 bfloat16,
// lane l = expert 16*eb + l%16, k-columns 32*c + 8*(l/16) .. +7 -- the
// operand layout of v_mfma_f32_16x16x32_bf16 -- so that one wave loads a
// fragment as 1 KB of consecutive bytes (whole cache lines).  Plane p,
// fragment (eb, c) starts at element ((p * E/16 + eb) * nc + c) * 512, with
// nc = ceil(d/32); columns past d are zero.  One thread per lane of a
// fragment.
__global__ __launch_bounds__(256) void x3_split_w_kernel(const float *W, uint16_t *planes, int E,
                                                         int d, int nc)
{
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;   // (eb * nc + c) * 64 + lane
    const size_t n_lanes = (size_t)(E / 16) * nc * 64;
    if (i >= n_lanes) return;
    const int lane = (int)(i & 63);
    const size_t frag = i >> 6;
    const int c = (int)(frag % nc);
    const int eb = (int)(frag / nc);
    const int k = 32 * c + 8 * (lane >> 4);
    const float *src = W + (size_t)(16 * eb + (lane & 15)) * d + k;
    const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
    const f32x4 w0 = k < d ? __builtin_nontemporal_load((const f32x4 *)src) : z;
    const f32x4 w1 = k < d ? __builtin_nontemporal_load((const f32x4 *)src + 1) : z;
    u32x4 h, m, l;
    split3(w0, w1, h, m, l);
    u32x4 *const out = (u32x4 *)planes;
    const size_t plane16 = n_lanes;   // 16-byte units per plane
    out[i] = h;
    out[plane16 + i] = m;
    out[2 * plane16 + i] = l;
}

// The GEMM on 8 waves (two per SIMD -- one wave per SIMD cannot issue these
// MFMAs back to back at full rate).  The waves are 4 expert quarters
// (16*NBW experts each) x 2 k-halves: a chunk is 64 k-columns and wave
// (wn, wk) takes its 32-column half wk, so every W fragment is loaded by
// exactly one wave.  x is staged in LDS 64 columns (128 bytes of a row) at a
// time, 8 threads per row (whole cache lines), double-buffered.  Each wave
// holds one chunk of W fragments in registers and refills each with the next
// chunk right after its last MFMA, in the order they are consumed, so every
// load has a whole chunk of MFMA work to land in (small batches, whose
// chunks are short, run a deeper ring instead).  At the end the k-half-1 wave
// of each quarter hands its sums to the k-half-0 wave through LDS, which adds
// them after its own (a fixed order) and writes the partial logits.
// Every X3_FLUSH chunks, and at the end, the two k-half waves of a quarter
// add their accumulators into one float32 total per element in LDS, k-half 0
// first (a fixed order, the same at every flush for every token), and
// restart them from zero; the k-half-0 wave writes the totals.
template <int BM, int NBW>
struct X3Wide {
    static constexpr int MB = BM / 16;               // token blocks per wave
    static constexpr int BN = 64 * NBW;              // experts per workgroup
    static constexpr int XQ = BM * 64 / 8 / 512;     // x pieces per thread per chunk
    static constexpr int STAGE = 2 * BM * 8;         // 16-byte slots: two x buffers
    static constexpr int TOT = 4 * MB * NBW * 64;    // 16-byte slots: float32 totals per quarter
    static constexpr int SLOTS = STAGE + TOT;
    static_assert(XQ >= 1, "every thread stages whole x pieces");
};

// Blocked summation: every X3_FLUSH 64-column chunks the accumulators are
// added into float32 totals in LDS and restarted from zero, so no rounding
// chain spans more than X3_FLUSH chunks (3 MFMAs of 32 exact products each
// per chunk); one chain over a k-half of d = 7168 would be 168 additions.
constexpr int X3_FLUSH = 16;

// 16-byte x pieces of one 128-byte row: 8 per row, permuted by the row so
// that the 16 lanes of a fragment read (rows r..r+15, one piece) cover all
// 64 banks once.
__device__ __forceinline__ int xw_slot(int row, int piece) { return row * 8 + (piece ^ ((row >> 1) & 7)); }

// SPLIT: W fragments are loaded as float32 (row-major W) and split in
// registers (small batches: no extra launch, no planes); otherwise they are
// loaded from the fragment-ordered planes of x3_split_w_kernel.
template <int BM, int NBW, bool SPLIT>
__global__ __launch_bounds__(512) void x3_gemm8_kernel(GateArgs a)
{
    using S = X3Wide<BM, NBW>;
    constexpr int MB = S::MB, XQ = S::XQ;
    __shared__ __attribute__((aligned(16))) u32x4 smem[S::SLOTS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wn = wave & 3;          // expert quarter
    const int wk = wave >> 2;         // k-half of every chunk
    const int q = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
    if (q >= a.n_tiles) return;       // padding of the grid (whole workgroup)
    // Tile numbers run token tile fastest (the token tiles that read one W
    // slice share an XCD's L2: small batches, where W dominates), or expert
    // tile fastest (the expert tiles of one token tile share it, so x, which
    // dominates large batches, crosses from HBM once)
    int t0, e0, ks;
    if (a.e_fast) {
        const int rq = q / a.e_tiles;
        e0 = (q - rq * a.e_tiles) * S::BN;
        ks = rq / a.t_tiles;
        t0 = (rq - ks * a.t_tiles) * BM;
    } else {
        const int rq = q / a.t_tiles;
        t0 = (q - rq * a.t_tiles) * BM;
        ks = rq / a.e_tiles;
        e0 = (rq - ks * a.e_tiles) * S::BN;
    }
    const int d = a.d;
    const int nc = a.chunks_total;                       // 32-column fragments per row
    const int c_begin = ks * a.chunks_per_split;         // in 32-column units
    const int c_end = min(c_begin + a.chunks_per_split, nc);
    const int c_last = c_end - 1;
    const int npairs = (c_end - c_begin + 1) / 2;        // 64-column chunks

    const int f_row = lane & 15;
    const size_t plane16 = (size_t)(a.E / 16) * nc * 64;
    const u32x4 *const planes = (const u32x4 *)a.w_planes;
    // this lane's expert row: e0 + 16(NBW*wn + n) + l%16, k-columns
    // 8*(l/16) .. +7 of a 32-column fragment
    size_t wbase[NBW];
#pragma unroll
    for (int n = 0; n < NBW; ++n) {
        const int eb = e0 / 16 + NBW * wn + n;
        wbase[n] = SPLIT ? (size_t)(16 * eb + f_row) * d : (size_t)eb * nc * 64 + lane;
    }
    // W fragment (plane pl, block n) of 64-column chunk j: 32-column
    // fragment c_begin + 2j + wk (clamped; a fragment past the slice or past
    // d meets zero x)
    auto wfrag = [&](int j, int n, int pl) {
        const int c = min(c_begin + 2 * j + wk, c_last);
        return planes[pl * plane16 + wbase[n] + (size_t)c * 64];
    };
    // the same fragment as 8 float32 (SPLIT), pieces past d clamped
    auto wfrag32 = [&](int j, int n, f32x4 (&w)[2]) {
        const int c = min(c_begin + 2 * j + wk, c_last);
        const float *const p = a.W + wbase[n] + min(c * KC + 8 * (lane >> 4), d - 8);
        w[0] = *(const f32x4 *)p;
        w[1] = *(const f32x4 *)(p + 4);
    };
    // x piece i of this thread: row tid/8 + 64i, k-piece tid%8 of the chunk
    const int kp = tid & 7;
    const uint16_t *xrow[XQ];
    int xsl[XQ];
#pragma unroll
    for (int i = 0; i < XQ; ++i) {
        const int row = (tid >> 3) + 64 * i;
        xrow[i] = a.x + (size_t)min(t0 + row, a.T - 1) * d;
        xsl[i] = xw_slot(row, kp);
    }
    auto load_x = [&](int j, u32x4 (&x)[XQ]) {
        const int k = (c_begin + 2 * j) * KC + 8 * kp;
#pragma unroll
        for (int i = 0; i < XQ; ++i) x[i] = *(const u32x4 *)(xrow[i] + min(k, d - 8));
    };
    // pieces past d or past the slice are stored as zeros (rare: a second
    // store in a uniform branch keeps the common path free of selects)
    auto store_x = [&](int j, int buf, const u32x4 (&x)[XQ]) {
        u32x4 *const xs = smem + buf * BM * 8;
#pragma unroll
        for (int i = 0; i < XQ; ++i) xs[xsl[i]] = x[i];
        if ((c_begin + 2 * j + 2) * KC > d || c_begin + 2 * j + 2 > c_end) {
            const int c = c_begin + 2 * j + (kp >> 2);
            if (c >= c_end || c * KC + 8 * (kp & 3) >= d) {
#pragma unroll
                for (int i = 0; i < XQ; ++i) xs[xsl[i]] = u32x4{0u, 0u, 0u, 0u};
            }
        }
    };

    f32x4 acc[MB][NBW];
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int n = 0; n < NBW; ++n) acc[m][n] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // float32 totals of this quarter's tile in LDS, one 16-byte slot per
    // accumulator and lane, shared by the quarter's two k-half waves
    constexpr int REGS = MB * NBW;
    f32x4 *const tot = (f32x4 *)(smem + S::STAGE) + wn * REGS * 64 + lane;
    bool fresh = true;   // the totals hold nothing yet (the first flush stores)
    auto flush = [&]() {
        if (wk == 0) {
#pragma unroll
            for (int m = 0; m < MB; ++m)
#pragma unroll
                for (int n = 0; n < NBW; ++n) {
                    f32x4 *const p = tot + (m * NBW + n) * 64;
                    *p = fresh ? acc[m][n] : *p + acc[m][n];
                    acc[m][n] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                }
        }
        __syncthreads();
        if (wk == 1) {
#pragma unroll
            for (int m = 0; m < MB; ++m)
#pragma unroll
                for (int n = 0; n < NBW; ++n) {
                    f32x4 *const p = tot + (m * NBW + n) * 64;
                    *p = *p + acc[m][n];
                    acc[m][n] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                }
        }
        __syncthreads();
        fresh = false;
    };
    static_assert(X3_FLUSH % 4 == 0, "flushes fall between unrolled steps");

    constexpr int SG_MFMA = 0x008, SG_VMEM_READ = 0x020, SG_DS_READ = 0x100;
    if (npairs > 0) {
        if constexpr (SPLIT) {
            // Small batches: a step is a few MFMAs, so loads run PW chunks
            // ahead in register rings (W as float32, x as bfloat16) to cover
            // first-touch memory latency.  Chunk j: A fragments from buffer
            // j%2, the split of W slot j%PW (refilled with chunk j+PW), the
            // MFMAs, then chunk j+1's x into the other buffer (its slot
            // refilled with chunk j+1+PW) and the barrier.
            constexpr int PW = BM == 64 ? 4 : 2;
            f32x4 wr[PW][NBW][2];
            u32x4 xr[PW][XQ];
#pragma unroll
            for (int u = 0; u < PW; ++u) {
#pragma unroll
                for (int n = 0; n < NBW; ++n) wfrag32(min(u, npairs - 1), n, wr[u][n]);
                load_x(min(u, npairs - 1), xr[u]);
            }
            store_x(0, 0, xr[0]);
            load_x(min(PW, npairs - 1), xr[0]);
            __syncthreads();
            // One W fragment per wave (NBW = 1): chunk j's MFMAs run on W
            // split one step earlier, and the split of chunk j+1 (ring slot
            // u1, then refilled with chunk j+1+PW) is issued beside them, so
            // its VALU work overlaps the matrix work.  Wider tiles keep the
            // split in front of the MFMAs (two splits in flight would not fit
            // their registers).
            constexpr bool AHEAD = NBW == 1;
            u32x4 bw[NBW][3];
            if constexpr (AHEAD) {
#pragma unroll
                for (int n = 0; n < NBW; ++n) {
                    split3(wr[0][n][0], wr[0][n][1], bw[n][0], bw[n][1], bw[n][2]);
                    wfrag32(min(PW, npairs - 1), n, wr[0][n]);
                }
            }
            auto step = [&](int j, int u) {   // u = j % PW; PW is even, so j%2 = u%2
                const int sb = u & 1;
                const int u1 = (u + 1) % PW;
                const u32x4 *const xs = smem + sb * BM * 8;
                u32x4 af[MB];
#pragma unroll
                for (int m = 0; m < MB; ++m) af[m] = xs[xw_slot(16 * m + f_row, 4 * wk + (lane >> 4))];
                u32x4 bn[NBW][3];
#pragma unroll
                for (int n = 0; n < NBW; ++n) {
                    if constexpr (AHEAD) {
                        split3(wr[u1][n][0], wr[u1][n][1], bn[n][0], bn[n][1], bn[n][2]);
                        wfrag32(min(j + 1 + PW, npairs - 1), n, wr[u1][n]);
                    } else {
                        split3(wr[u][n][0], wr[u][n][1], bw[n][0], bw[n][1], bw[n][2]);
                        wfrag32(min(j + PW, npairs - 1), n, wr[u][n]);
                    }
                }
#pragma unroll
                for (int pl = 0; pl < 3; ++pl)
#pragma unroll
                    for (int n = 0; n < NBW; ++n)
#pragma unroll
                        for (int m = 0; m < MB; ++m) acc[m][n] = mfma_bf16(af[m], bw[n][pl], acc[m][n]);
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (AHEAD) {
#pragma unroll
                    for (int n = 0; n < NBW; ++n)
#pragma unroll
                        for (int pl = 0; pl < 3; ++pl) bw[n][pl] = bn[n][pl];
                }
                store_x(min(j + 1, npairs - 1), sb ^ 1, xr[u1]);
                load_x(min(j + 1 + PW, npairs - 1), xr[u1]);
                __syncthreads();
            };
            int j = 0;
            for (; j + PW <= npairs; j += PW) {
#pragma unroll
                for (int u = 0; u < PW; ++u) step(j + u, u);
                if ((j + PW) % X3_FLUSH == 0) flush();
            }
#pragma unroll
            for (int u = 0; u < PW - 1; ++u)
                if (j + u < npairs) step(j + u, u);
        } else {
            // Large batches: a step is 3*MB*NBW MFMAs per wave, long enough
            // for a one-chunk refill of each W fragment after its last use.
            u32x4 wst[NBW][3];
            u32x4 xst[XQ];
#pragma unroll
            for (int n = 0; n < NBW; ++n)
#pragma unroll
                for (int pl = 0; pl < 3; ++pl) wst[n][pl] = wfrag(0, n, pl);
            load_x(0, xst);
            store_x(0, 0, xst);
            load_x(min(1, npairs - 1), xst);
            __syncthreads();
            // chunk j: A fragments from buffer j%2, MFMAs on the W fragments
            // (each refilled with chunk j+1 after its last use), chunk j+1's
            // x into the other buffer, chunk j+2's x into registers, barrier
            auto step = [&](int j, int sb) {
                const u32x4 *const xs = smem + sb * BM * 8;
                u32x4 af[MB];
#pragma unroll
                for (int m = 0; m < MB; ++m) af[m] = xs[xw_slot(16 * m + f_row, 4 * wk + (lane >> 4))];
                const int jn = min(j + 1, npairs - 1);
#pragma unroll
                for (int pl = 0; pl < 3; ++pl)
#pragma unroll
                    for (int n = 0; n < NBW; ++n) {
                        const u32x4 b = wst[n][pl];
#pragma unroll
                        for (int m = 0; m < MB; ++m) acc[m][n] = mfma_bf16(af[m], b, acc[m][n]);
                        wst[n][pl] = wfrag(jn, n, pl);
                    }
                __builtin_amdgcn_sched_group_barrier(SG_DS_READ, MB, 0);
#pragma unroll
                for (int g = 0; g < 3 * NBW; ++g) {
                    __builtin_amdgcn_sched_group_barrier(SG_MFMA, MB, 0);
                    __builtin_amdgcn_sched_group_barrier(SG_VMEM_READ, 1, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
                store_x(min(j + 1, npairs - 1), sb ^ 1, xst);
                load_x(min(j + 2, npairs - 1), xst);
                __syncthreads();
            };
            int j = 0;
            for (; j + 2 <= npairs; j += 2) {
                step(j, 0);
                step(j + 1, 1);
                if ((j + 2) % X3_FLUSH == 0) flush();
            }
            if (j < npairs) step(j, 0);
        }
    }

    // the last block into the totals (both k-halves, in order), then the
    // k-half-0 wave writes the totals as the tile's partial logits
    flush();
    if (wk == 1) return;
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int n = 0; n < NBW; ++n) acc[m][n] = tot[(m * NBW + n) * 64];
    // accumulator r of block (m, n): token t0 + 16m + 4(l/16) + r, expert
    // e0 + 16(NBW*wn + n) + l%16
    float *const out = a.partial + (size_t)ks * a.T * a.e_stride;
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = t0 + 16 * m + 4 * (lane >> 4) + r;
            if (t < a.T) {
#pragma unroll
                for (int n = 0; n < NBW; ++n)
                    out[(size_t)t * a.e_stride + e0 + 16 * (NBW * wn + n) + f_row] = acc[m][n][r];
            }
        }
}

// Tile shapes: BM tokens x 64*NBW experts.  Large batches (W pre-split
// into planes) choose among all; small batches, which split W in registers,
// among the one-fragment tiles only (a sweep over shapes and slice counts at
// T = 1 ... 1000 found one of them fastest at every T).
struct X3Shape {
    int bm, nbw;
};
constexpr X3Shape X3_SHAPES_PRESPLIT[] = {{128, 3}, {128, 2}, {64, 2}, {64, 1}};
constexpr X3Shape X3_SHAPES_SPLIT[] = {{128, 1}, {64, 1}};

// Cost model, in cycles of one SIMD per 32-column unit of a workgroup's
// k-slice: large batches, 3 * (BM/16) * NBW MFMAs of 16 cycles plus
// X3_CHUNK_OVERHEAD; small batches, X3_SPLIT_CHUNK_FIXED plus
// X3_SPLIT_CHUNK_PER_BLOCK per 16-token block (fitted to graph-replayed gate
// times over tile shapes and slice counts at T = 1 ... 1000, E = 128 ... 512:
// the in-register split and the memory pipeline, not the MFMAs, set the pace
// there).  A workgroup adds X3_LATENCY; workgroups beyond one per compute
// unit queue behind it; the partial logits cross memory twice at
// X3_BYTES_PER_CYCLE.
constexpr double X3_CHUNK_OVERHEAD = 150.0;
constexpr double X3_LATENCY = 3000.0;
constexpr double X3_BYTES_PER_CYCLE = 2400.0;
constexpr double X3_SPLIT_CHUNK_FIXED = 300.0;
constexpr double X3_SPLIT_CHUNK_PER_BLOCK = 20.0;
constexpr int X3_N_CU = 256;
// From this many tokens on, W is split once per call into planes (the split
// kernel reads W once and writes 1.5x its bytes) instead of in registers by
// every token tile.
constexpr int X3_PRESPLIT_MIN_T = 1024;

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

template <int BM, int NBW>
hipError_t launch_shape(const GateArgs &a, const GatePlan &p, hipStream_t stream)
{
    const dim3 grid(p.grid);
    if (p.x3_presplit) return launch_kernel(x3_gemm8_kernel<BM, NBW, false>, grid, dim3(512), stream, a);
    // (the plan never splits a 128 x 192 tile in registers: it would not fit)
    if constexpr (BM == 128 && NBW == 3) return hipErrorInvalidValue;
    else return launch_kernel(x3_gemm8_kernel<BM, NBW, true>, grid, dim3(512), stream, a);
}

}  // namespace

GatePlan plan_x3(int T, int d, int E)
{
    GatePlan p{};
    p.split = true;
    p.e_stride = E;   // the route's tiles cover E exactly (64-expert multiples)
    const int chunks = (d + KC - 1) / KC;
    double best = 1e300;
    const bool presplit = T >= X3_PRESPLIT_MIN_T;
    const X3Shape *const shapes = presplit ? X3_SHAPES_PRESPLIT : X3_SHAPES_SPLIT;
    const int n_shapes = presplit ? (int)(sizeof(X3_SHAPES_PRESPLIT) / sizeof(X3Shape))
                                  : (int)(sizeof(X3_SHAPES_SPLIT) / sizeof(X3Shape));
    for (int i = 0; i < n_shapes; ++i) {
        const X3Shape &sh = shapes[i];
        const int bn = 64 * sh.nbw;
        if (E % bn != 0) continue;
        const long tiles = ((long)T + sh.bm - 1) / sh.bm * (E / bn);
        const double chunk_cost = presplit ? 3.0 * (sh.bm / 16) * sh.nbw * 16.0 + X3_CHUNK_OVERHEAD
                                           : X3_SPLIT_CHUNK_FIXED + X3_SPLIT_CHUNK_PER_BLOCK * (sh.bm / 16) * sh.nbw;
        for (int s = 1; s <= chunks; ++s) {
            const int cps = (chunks + s - 1) / s;
            if ((chunks + cps - 1) / cps != s) continue;   // s slices of cps chunks
            const long n = tiles * s;
            const double rounds = (double)((n + X3_N_CU - 1) / X3_N_CU);
            const double cost = rounds * (cps * chunk_cost + X3_LATENCY) +
                                2.0 * s * (double)T * E * sizeof(float) / X3_BYTES_PER_CYCLE;
            if (cost < best) {
                best = cost;
                p.x3_bm = sh.bm;
                p.x3_nbw = sh.nbw;
                p.n_split = s;
                p.chunks_per_split = cps;
                p.t_tiles = (T + sh.bm - 1) / sh.bm;
                p.e_tiles = E / bn;
            }
        }
    }
    const long n = (long)p.t_tiles * p.e_tiles * p.n_split;
    p.grid = (int)((n + 7) / 8 * 8);
    p.m_blocks = 0;
    p.x3_presplit = presplit;
    const size_t partials = (size_t)p.n_split * (size_t)T * (size_t)E * sizeof(float);
    p.planes_offset = p.x3_presplit ? align256(partials) : 0;
    // planes: 3 x E x (chunks * 32) bfloat16
    p.partial_bytes = p.x3_presplit ? p.planes_offset + (size_t)3 * E * chunks * KC * sizeof(uint16_t)
                                    : partials;
    return p;
}

hipError_t launch_x3_gemm(const GateArgs &args, const GatePlan &p, hipStream_t stream)
{
    GateArgs a = args;
    a.e_fast = p.x3_presplit ? 1 : 0;
    if (p.x3_presplit) {
        uint16_t *planes = (uint16_t *)((char *)a.partial + p.planes_offset);
        const size_t n_lanes = (size_t)(a.E / 16) * a.chunks_total * 64;
        const hipError_t e = launch_kernel(x3_split_w_kernel, dim3((unsigned)((n_lanes + 255) / 256)),
                                           dim3(256), stream, a.W, planes, a.E, a.d, a.chunks_total);
        if (e != hipSuccess) return e;
        a.w_planes = planes;
    }
    if (p.x3_bm == 128 && p.x3_nbw == 3) return launch_shape<128, 3>(a, p, stream);
    if (p.x3_bm == 128 && p.x3_nbw == 2) return launch_shape<128, 2>(a, p, stream);
    if (p.x3_bm == 64 && p.x3_nbw == 2) return launch_shape<64, 2>(a, p, stream);
    if (p.x3_bm == 128 && p.x3_nbw == 1) return launch_shape<128, 1>(a, p, stream);
    if (p.x3_bm == 64 && p.x3_nbw == 1) return launch_shape<64, 1>(a, p, stream);
    return hipErrorInvalidValue;
}

}  // namespace siggate
