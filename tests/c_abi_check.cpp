// c_abi_check.cpp -- drives the step library through its C ABI from plain C++ (no Python,
// no torch): device buffers from hipMalloc, neox_zero1_* calls, state and arrays read back
// and checked against closed forms computed here in double.
//
// Test infrastructure.  Checks:
//   - first step from zero moments: m = (1-b1) g, v = (1-b2) g^2, and
//     w1 = w0 - lr (g / (|g| + eps) + wd w0 [decaying elements]) (Adam with bias
//     correction, Kingma & Ba; decoupled decay, Loshchilov & Hutter); the global norm;
//   - a no-decay element with a zero gradient is left bit for bit unchanged;
//   - the half copy is the stored FP32 master rounded to binary16 (nearest even);
//   - an inf in the gradient skips the step: every array bit for bit unchanged, the
//     dynamic scale halved, the step count unchanged (mixed-precision loss scaling,
//     Micikevicius et al. 2018);
//   - the chunk-table update gives the flat update's bits;
//   - argument errors return NEOX_EINVAL with a message.
// Prints "c_abi_check ok" and exits 0 when every check passes.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "neox_zero1.h"

static int failures = 0;

#define CHECK(cond, ...)                                              \
    do {                                                              \
        if (!(cond)) {                                                \
            std::printf("FAIL %s:%d: ", __FILE__, __LINE__);          \
            std::printf(__VA_ARGS__);                                 \
            std::printf("\n");                                        \
            if (++failures > 20) std::exit(1);                        \
        }                                                             \
    } while (0)

#define HIPCHECK(x)                                                                      \
    do {                                                                                 \
        hipError_t e_ = (x);                                                             \
        if (e_ != hipSuccess) {                                                          \
            std::printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);   \
            std::exit(2);                                                                \
        }                                                                                \
    } while (0)

#define NEOXCHECK(x)                                                                       \
    do {                                                                                   \
        int r_ = (x);                                                                      \
        if (r_ != NEOX_OK) {                                                               \
            std::printf("neox error %d at line %d: %s\n", r_, __LINE__, neox_zero1_last_error()); \
            std::exit(3);                                                                  \
        }                                                                                  \
    } while (0)

static uint16_t f16_bits(float x) {
    _Float16 h = (_Float16)x;   // round to nearest even
    uint16_t b;
    std::memcpy(&b, &h, 2);
    return b;
}

struct Shard {
    size_t n;
    uint16_t *grad, *half;
    float *master, *m, *v;
};

static Shard alloc_shard(size_t n, size_t pad) {
    Shard s{n, nullptr, nullptr, nullptr, nullptr, nullptr};
    uint16_t *g, *h;
    float *w, *m, *v;
    HIPCHECK(hipMalloc(&g, (n + pad) * 2));
    HIPCHECK(hipMalloc(&h, (n + pad) * 2));
    HIPCHECK(hipMalloc(&w, (n + pad) * 4));
    HIPCHECK(hipMalloc(&m, (n + pad) * 4));
    HIPCHECK(hipMalloc(&v, (n + pad) * 4));
    s.grad = g + pad;        // pad = 1 makes every array 2 or 4 bytes past 16-byte alignment
    s.half = h + pad;
    s.master = w + pad;
    s.m = m + pad;
    s.v = v + pad;
    return s;
}

static void free_shard(Shard& s, size_t pad) {
    HIPCHECK(hipFree(s.grad - pad));
    HIPCHECK(hipFree(s.half - pad));
    HIPCHECK(hipFree(s.master - pad));
    HIPCHECK(hipFree(s.m - pad));
    HIPCHECK(hipFree(s.v - pad));
}

struct Host {
    std::vector<uint16_t> half;
    std::vector<float> master, m, v;
};

static Host read_back(const Shard& s) {
    Host h{std::vector<uint16_t>(s.n), std::vector<float>(s.n), std::vector<float>(s.n),
           std::vector<float>(s.n)};
    HIPCHECK(hipMemcpy(h.half.data(), s.half, s.n * 2, hipMemcpyDeviceToHost));
    HIPCHECK(hipMemcpy(h.master.data(), s.master, s.n * 4, hipMemcpyDeviceToHost));
    HIPCHECK(hipMemcpy(h.m.data(), s.m, s.n * 4, hipMemcpyDeviceToHost));
    HIPCHECK(hipMemcpy(h.v.data(), s.v, s.n * 4, hipMemcpyDeviceToHost));
    return h;
}

static bool same_bits(const Host& a, const Host& b) {
    return a.half == b.half && std::memcmp(a.master.data(), b.master.data(), a.master.size() * 4) == 0 &&
           std::memcmp(a.m.data(), b.m.data(), a.m.size() * 4) == 0 &&
           std::memcmp(a.v.data(), b.v.data(), a.v.size() * 4) == 0;
}

// Unscaled gradient and initial weight of element i: small multiples of powers of two,
// exact in every format involved.
static double grad_of(size_t i) { return ((double)(i % 17) - 8.0) / 1024.0; }
static double w0_of(size_t i) { return ((double)(i % 29) - 14.0) / 256.0; }

static void upload(const Shard& s, double scale, long inf_at) {
    std::vector<uint16_t> g(s.n), h(s.n);
    std::vector<float> w(s.n), z(s.n, 0.0f);
    for (size_t i = 0; i < s.n; ++i) {
        g[i] = f16_bits((float)(grad_of(i) * scale));
        w[i] = (float)w0_of(i);
        h[i] = f16_bits(w[i]);
    }
    if (inf_at >= 0) g[inf_at] = 0x7C00;
    HIPCHECK(hipMemcpy(s.grad, g.data(), s.n * 2, hipMemcpyHostToDevice));
    HIPCHECK(hipMemcpy(s.half, h.data(), s.n * 2, hipMemcpyHostToDevice));
    HIPCHECK(hipMemcpy(s.master, w.data(), s.n * 4, hipMemcpyHostToDevice));
    HIPCHECK(hipMemcpy(s.m, z.data(), s.n * 4, hipMemcpyHostToDevice));
    HIPCHECK(hipMemcpy(s.v, z.data(), s.n * 4, hipMemcpyHostToDevice));
}

static void upload_grad(const Shard& s, double scale, long inf_at) {
    std::vector<uint16_t> g(s.n);
    for (size_t i = 0; i < s.n; ++i) g[i] = f16_bits((float)(grad_of(i) * scale));
    if (inf_at >= 0) g[inf_at] = 0x7C00;
    HIPCHECK(hipMemcpy(s.grad, g.data(), s.n * 2, hipMemcpyHostToDevice));
}

int main() {
    const size_t n0 = 3000, n1 = 1099, n = n0 + n1;   // decaying, then non-decaying
    const float lr = 1e-3f;
    neox_zero1_config cfg;
    NEOXCHECK(neox_zero1_default_config(&cfg));
    const double b1 = cfg.beta1, b2 = cfg.beta2, eps = cfg.eps, wd = cfg.weight_decay;
    const double S0 = cfg.init_scale;

    auto segments = [&](const Shard& s) {
        std::vector<neox_segment> segs(2);
        segs[0] = neox_segment{s.grad, s.half, s.master, s.m, s.v, n0, NEOX_SEG_DECAY, 0, 0};
        segs[1] = neox_segment{s.grad + n0, s.half + n0, s.master + n0, s.m + n0, s.v + n0, n1, 0, 1, 0};
        return segs;
    };

    // --- argument errors -------------------------------------------------------------
    CHECK(neox_zero1_step(nullptr, lr, nullptr) == NEOX_EINVAL, "step(NULL) accepted");
    CHECK(std::strlen(neox_zero1_last_error()) > 0, "no error text");
    CHECK(neox_zero1_destroy(nullptr) == NEOX_OK, "destroy(NULL) not a no-op");

    // --- flat shard: step 1 against the closed form -------------------------------------
    Shard a = alloc_shard(n, 0);
    upload(a, S0, -1);
    std::vector<neox_segment> sa = segments(a);
    neox_zero1* ha = nullptr;
    NEOXCHECK(neox_zero1_create(&cfg, sa.data(), sa.size(), nullptr, &ha));
    CHECK(neox_zero1_update_path(ha) == NEOX_PATH_FLAT, "contiguous aligned shard not on the flat path");
    NEOXCHECK(neox_zero1_step(ha, lr, nullptr));
    neox_scaler_state_t st;
    NEOXCHECK(neox_scaler_state(ha, &st));
    double sumsq = 0.0;
    for (size_t i = 0; i < n; ++i) sumsq += grad_of(i) * grad_of(i);   // exact in double
    CHECK(st.step == 1 && st.skipped_total == 0 && st.last_skipped == 0, "step 1 state");
    CHECK(st.loss_scale == (float)S0, "scale changed on a clean step");
    CHECK(std::fabs(st.last_sumsq - sumsq) <= 1e-12 * sumsq, "sumsq %.17g vs %.17g", st.last_sumsq, sumsq);
    CHECK(std::fabs(st.last_grad_norm - std::sqrt(sumsq)) <= 1e-5 * std::sqrt(sumsq), "norm");
    CHECK(st.last_clip_coef == 1.0f, "clip active below the threshold");

    Host h1 = read_back(a);
    for (size_t i = 0; i < n; ++i) {
        const double g = grad_of(i), w0 = w0_of(i);
        const bool decay = i < n0;
        const double m1 = (1.0 - b1) * g, v1 = (1.0 - b2) * g * g;
        const double u = g / (std::fabs(g) + eps) + (decay ? wd * w0 : 0.0);
        const double w1 = w0 - (double)lr * u;
        const double tw = 2e-6 * std::fmax(std::fmax(std::fabs(w1), std::fabs(w0)), (double)lr);
        CHECK(std::fabs(h1.master[i] - w1) <= tw, "master[%zu] %.9g vs %.9g", i, h1.master[i], w1);
        CHECK(std::fabs(h1.m[i] - m1) <= 2e-6 * std::fabs(m1) + 1e-40, "m[%zu] %.9g vs %.9g", i, h1.m[i], m1);
        CHECK(std::fabs(h1.v[i] - v1) <= 2e-6 * std::fabs(v1) + 1e-40, "v[%zu] %.9g vs %.9g", i, h1.v[i], v1);
        CHECK(h1.half[i] == f16_bits(h1.master[i]), "half[%zu] is not RNE(master)", i);
        if (g == 0.0 && !decay)
            CHECK(h1.master[i] == (float)w0 && h1.m[i] == 0.0f && h1.v[i] == 0.0f,
                  "zero-gradient no-decay element %zu moved", i);
    }

    // --- an inf skips the step ------------------------------------------------------------
    upload_grad(a, S0, 123);
    NEOXCHECK(neox_zero1_step(ha, lr, nullptr));
    NEOXCHECK(neox_scaler_state(ha, &st));
    CHECK(st.last_skipped == 1 && st.step == 1 && st.skipped_total == 1, "skip state");
    CHECK(st.loss_scale == (float)(S0 / 2), "scale not halved: %g", (double)st.loss_scale);
    CHECK(std::isinf(st.last_grad_norm), "norm of a skipped step not inf");
    Host h2 = read_back(a);
    CHECK(same_bits(h1, h2), "a skipped step wrote the arrays");

    // --- the next clean step carries the halved scale -------------------------------------
    upload_grad(a, S0 / 2, -1);
    NEOXCHECK(neox_zero1_step(ha, lr, nullptr));
    NEOXCHECK(neox_scaler_state(ha, &st));
    CHECK(st.last_skipped == 0 && st.step == 2 && st.consecutive_overflows == 0, "recovery state");
    CHECK(std::fabs(st.last_sumsq - sumsq) <= 1e-12 * sumsq, "unscaled norm changed with the scale");

    // --- chunk-table update on the same data: same bits -----------------------------------
    Shard b = alloc_shard(n, 0);
    upload(b, S0, -1);
    std::vector<neox_segment> sb = segments(b);
    neox_zero1_config cc = cfg;
    cc.chunked_update = 1;
    neox_zero1* hb = nullptr;
    NEOXCHECK(neox_zero1_create(&cc, sb.data(), sb.size(), nullptr, &hb));
    CHECK(neox_zero1_update_path(hb) == NEOX_PATH_CHUNKED, "chunked_update ignored");
    NEOXCHECK(neox_zero1_step(hb, lr, nullptr));
    NEOXCHECK(neox_scaler_state(hb, &st));
    CHECK(same_bits(h1, read_back(b)), "chunked update differs from the flat one");

    // --- misaligned arrays (scalar heads and tails): same bits again ------------------------
    Shard c = alloc_shard(n, 1);
    upload(c, S0, -1);
    std::vector<neox_segment> sc = segments(c);
    neox_zero1* hc = nullptr;
    NEOXCHECK(neox_zero1_create(&cfg, sc.data(), sc.size(), nullptr, &hc));
    CHECK(neox_zero1_update_path(hc) == NEOX_PATH_CHUNKED, "misaligned shard on the flat path");
    NEOXCHECK(neox_zero1_step(hc, lr, nullptr));
    NEOXCHECK(neox_scaler_state(hc, &st));
    CHECK(same_bits(h1, read_back(c)), "misaligned shard differs from the aligned one");

    NEOXCHECK(neox_zero1_destroy(ha));
    NEOXCHECK(neox_zero1_destroy(hb));
    NEOXCHECK(neox_zero1_destroy(hc));
    free_shard(a, 0);
    free_shard(b, 0);
    free_shard(c, 1);
    if (failures) {
        std::printf("c_abi_check: %d failure(s)\n", failures);
        return 1;
    }
    std::printf("c_abi_check ok\n");
    return 0;
}
