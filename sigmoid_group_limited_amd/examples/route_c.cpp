// route_c.cpp -- the C ABI of libsiggate used directly, with no Python and
// no PyTorch: device memory from hipMalloc, one stream, the gate, the
// dispatch and the combine on a synthetic batch, checks of what the results
// must satisfy, and event timing of gate + dispatch.
//
//   route_c [kimi|dsv3] [T] [d] [fp32|x3]   (defaults: kimi 256 7168 fp32)
//
// x3 selects the bfloat16 three-way logits route (cfg.logits_path = 1).
//
// Exit status 0 when every check holds.  One line of JSON on stdout.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "siggate.h"

#define HIP_OK(call)                                                              \
    do {                                                                          \
        hipError_t e_ = (call);                                                   \
        if (e_ != hipSuccess) {                                                   \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));     \
            exit(2);                                                              \
        }                                                                         \
    } while (0)

#define SG_OK(call)                                                               \
    do {                                                                          \
        siggate_status_t s_ = (call);                                             \
        if (s_ != SIGGATE_OK) {                                                   \
            fprintf(stderr, "%s failed: %s\n", #call, siggate_status_str(s_));    \
            exit(3);                                                              \
        }                                                                         \
    } while (0)

static int failures = 0;
#define CHECK(cond, ...)                                                          \
    do {                                                                          \
        if (!(cond) && failures++ < 10) {                                         \
            fprintf(stderr, "check failed: " __VA_ARGS__);                        \
            fputc('\n', stderr);                                                  \
        }                                                                         \
    } while (0)

// splitmix64: a seeded source of uniform doubles in [0, 1)
struct Rng {
    uint64_t s;
    double next()
    {
        uint64_t z = (s += 0x9e3779b97f4a7c15ull);
        z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
        z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
        z ^= z >> 31;
        return (double)(z >> 11) * (1.0 / 9007199254740992.0);
    }
};

static uint16_t to_bf16(float f)   // round to nearest even (finite inputs)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

static float from_bf16(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

template <typename T> static T *dev(size_t n)
{
    void *p = nullptr;
    HIP_OK(hipMalloc(&p, n * sizeof(T) > 0 ? n * sizeof(T) : 16));
    return (T *)p;
}

int main(int argc, char **argv)
{
    const bool dsv3 = argc > 1 && strcmp(argv[1], "dsv3") == 0;
    const int T = argc > 2 ? atoi(argv[2]) : 256;
    const int d = argc > 3 ? atoi(argv[3]) : 7168;
    const bool x3 = argc > 4 && strcmp(argv[4], "x3") == 0;
    siggate_cfg_t cfg;
    memset(&cfg, 0, sizeof cfg);
    cfg.T = T;
    cfg.d = d;
    cfg.E = dsv3 ? 256 : 384;
    cfg.n_group = dsv3 ? 8 : 1;
    cfg.topk_group = dsv3 ? 4 : 1;
    cfg.top_k = 8;
    cfg.route_scale = dsv3 ? 2.5f : 2.827f;
    cfg.logits_path = x3 ? 1 : 0;
    const int E = cfg.E, K = cfg.top_k;
    const size_t n_pairs = (size_t)T * K;

    // synthetic inputs: x uniform with unit variance (bfloat16), W with
    // variance 1/d, bias in [-0.05, 0.05)
    Rng rng{12345};
    std::vector<uint16_t> x((size_t)T * d);
    std::vector<float> W((size_t)E * d), bias(E);
    for (auto &v : x) v = to_bf16((float)((rng.next() * 2.0 - 1.0) * sqrt(3.0)));
    for (auto &v : W) v = (float)((rng.next() * 2.0 - 1.0) * sqrt(3.0 / d));
    for (auto &v : bias) v = (float)((rng.next() * 2.0 - 1.0) * 0.05);

    uint16_t *d_x = dev<uint16_t>(x.size());
    float *d_W = dev<float>(W.size()), *d_b = dev<float>(E);
    float *d_w = dev<float>(n_pairs);
    int32_t *d_i = dev<int32_t>(n_pairs), *d_tpe = dev<int32_t>(E), *d_off = dev<int32_t>(E + 1);
    int32_t *d_perm = dev<int32_t>(n_pairs), *d_dest = dev<int32_t>(n_pairs);
    uint16_t *d_px = dev<uint16_t>(n_pairs * d), *d_y = dev<uint16_t>((size_t)T * d);
    const size_t ws_bytes = siggate_workspace_bytes(&cfg);
    void *d_ws = dev<uint8_t>(ws_bytes);
    HIP_OK(hipMemcpy(d_x, x.data(), x.size() * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_W, W.data(), W.size() * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_b, bias.data(), E * 4, hipMemcpyHostToDevice));
    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));

    SG_OK(siggate_forward(d_x, d_W, d_b, &cfg, d_w, d_i, d_ws, ws_bytes, stream));
    SG_OK(siggate_dispatch(d_x, d_i, &cfg, d_tpe, d_off, d_perm, d_dest, d_px, d_ws, ws_bytes,
                           stream));
    // identity experts: the dispatched rows come straight back
    SG_OK(siggate_combine(d_px, d_w, d_dest, &cfg, d_y, stream));
    HIP_OK(hipStreamSynchronize(stream));

    std::vector<float> w(n_pairs);
    std::vector<int32_t> idx(n_pairs), tpe(E), off(E + 1), perm(n_pairs), dest(n_pairs);
    std::vector<uint16_t> px(n_pairs * d), y((size_t)T * d);
    HIP_OK(hipMemcpy(w.data(), d_w, n_pairs * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(idx.data(), d_i, n_pairs * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(tpe.data(), d_tpe, E * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(off.data(), d_off, (E + 1) * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(perm.data(), d_perm, n_pairs * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(dest.data(), d_dest, n_pairs * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(px.data(), d_px, n_pairs * d * 2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(y.data(), d_y, (size_t)T * d * 2, hipMemcpyDeviceToHost));

    // gate: ids in range, ascending and distinct, at most topk_group groups,
    // weights >= 0 summing to route_scale
    const int S = E / cfg.n_group;
    for (int t = 0; t < T; ++t) {
        double sum = 0.0;
        int groups = 0, last_g = -1;
        for (int k = 0; k < K; ++k) {
            const int e = idx[(size_t)t * K + k];
            CHECK(e >= 0 && e < E, "token %d: id %d out of range", t, e);
            if (k > 0) CHECK(e > idx[(size_t)t * K + k - 1], "token %d: ids not ascending", t);
            if (e / S != last_g) ++groups, last_g = e / S;
            CHECK(w[(size_t)t * K + k] >= 0.0f, "token %d: negative weight", t);
            sum += w[(size_t)t * K + k];
        }
        CHECK(groups <= cfg.topk_group, "token %d: %d groups", t, groups);
        CHECK(fabs(sum - cfg.route_scale) <= 1e-5 * cfg.route_scale, "token %d: weights sum %g", t,
              sum);
    }
    // dispatch: counts, offsets, a stable expert-major permutation, dest its
    // inverse, rows copied bit for bit
    std::vector<int32_t> cnt(E, 0);
    for (size_t p = 0; p < n_pairs; ++p) cnt[idx[p]]++;
    for (int e = 0; e < E; ++e) {
        CHECK(tpe[e] == cnt[e], "expert %d: count %d, expected %d", e, tpe[e], cnt[e]);
        CHECK(off[e + 1] - off[e] == cnt[e], "expert %d: offsets", e);
    }
    CHECK(off[0] == 0 && off[E] == (int32_t)n_pairs, "offset ends");
    std::vector<int32_t> want(n_pairs);
    for (size_t p = 0; p < n_pairs; ++p) want[p] = (int32_t)p;
    std::stable_sort(want.begin(), want.end(), [&](int32_t a, int32_t b) { return idx[a] < idx[b]; });
    for (size_t pos = 0; pos < n_pairs; ++pos) {
        CHECK(perm[pos] == want[pos], "perm[%zu] = %d, expected %d", pos, perm[pos], want[pos]);
        CHECK(dest[perm[pos]] == (int32_t)pos, "dest is not the inverse of perm at %zu", pos);
        const size_t t = (size_t)perm[pos] / K;
        CHECK(memcmp(&px[pos * d], &x[t * d], (size_t)d * 2) == 0, "row %zu differs", pos);
    }
    // combine with identity experts: y = route_scale * x, within the float32
    // sum of K products rounded once to bfloat16
    for (size_t i = 0; i < (size_t)T * d; ++i) {
        const double want_y = (double)cfg.route_scale * from_bf16(x[i]);
        const double got = from_bf16(y[i]);
        CHECK(fabs(got - want_y) <= fabs(want_y) * (1.0 / 128) + 1e-30, "y[%zu] = %g, want %g", i,
              got, want_y);
    }

    // timing: gate + dispatch, 20 calls after 3, HIP events on the stream
    hipEvent_t e0, e1;
    HIP_OK(hipEventCreate(&e0));
    HIP_OK(hipEventCreate(&e1));
    for (int r = 0; r < 23; ++r) {
        if (r == 3) HIP_OK(hipEventRecord(e0, stream));
        SG_OK(siggate_forward(d_x, d_W, d_b, &cfg, d_w, d_i, d_ws, ws_bytes, stream));
        SG_OK(siggate_dispatch(d_x, d_i, &cfg, d_tpe, d_off, d_perm, d_dest, d_px, d_ws, ws_bytes,
                               stream));
    }
    HIP_OK(hipEventRecord(e1, stream));
    HIP_OK(hipEventSynchronize(e1));
    float ms = 0.0f;
    HIP_OK(hipEventElapsedTime(&ms, e0, e1));
    const double us = ms * 1e3 / 20;
    printf("{\"model\": \"%s\", \"T\": %d, \"d\": %d, \"E\": %d, \"logits_path\": %d, "
           "\"checks_failed\": %d, \"gate_dispatch_us\": %.2f, \"tokens_per_s\": %.0f}\n",
           dsv3 ? "dsv3" : "kimi", T, d, E, cfg.logits_path, failures, us, T / (us * 1e-6));
    return failures ? 1 : 0;
}
