// sanitize_harness.cpp -- host-only checks run under AddressSanitizer and
// UndefinedBehaviorSanitizer (built and run by tests/test_sanitizers.py).
//
// Two pieces of host code are exercised here, each compiled with the
// sanitizers: the C ABI's argument validation (gdn_validate.hpp, the code
// the library runs before any HIP call) and the fp64 oracle
// (oracle/gdn_oracle.c, linked in as C). Pointers handed to the validation
// are never dereferenced by it, so fake addresses stand in for device
// buffers. The oracle runs on small heap buffers sized exactly, so any read
// or write past an end is reported.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "../gated_deltanet_token_amd/csrc/gdn_validate.hpp"

extern "C" int gdn_oracle_chain(const void *q, const void *k, const void *v, int dtype,
                                const void *alpha, const void *beta, int ab_dtype, int64_t T,
                                int64_t stride_qk, int64_t stride_v, int64_t stride_ab, int dk,
                                int dv, double scale, double *S, double *o);

static int g_fail = 0;
#define CHECK(cond)                                                      \
    do {                                                                 \
        if (!(cond)) {                                                   \
            fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond); \
            ++g_fail;                                                    \
        }                                                                \
    } while (0)

using namespace gdn::val;

static const void *P(uintptr_t a) { return reinterpret_cast<const void *>(a); }
static const float *F(uintptr_t a) { return reinterpret_cast<const float *>(a); }

static void validation() {
    // one dense prefill: B=1, T=100, Hk=2, Hv=6, D=128, bf16; buffers 16 GiB apart
    const uintptr_t base = (uintptr_t)1 << 40, gap = (uintptr_t)1 << 34;
    auto at = [&](int i) { return base + (uintptr_t)i * gap; };
    const int64_t tokens = 100;
    CHECK(check_prefill(P(at(0)), P(at(1)), P(at(2)), F(at(3)), F(at(4)), F(at(5)), P(at(6)),
                        F(at(7)), nullptr, 0, nullptr, 0, tokens, 1, 2, 6, 128, 128, GDN_BF16,
                        P(at(8)), 4096) == GDN_OK);
    // in-place state
    CHECK(check_prefill(P(at(0)), P(at(1)), P(at(2)), F(at(3)), F(at(4)), F(at(5)), P(at(6)),
                        F(at(5)), nullptr, 0, nullptr, 0, tokens, 1, 2, 6, 128, 128, GDN_BF16,
                        nullptr, 0) == GDN_OK);
    // out overlapping v
    CHECK(check_prefill(P(at(0)), P(at(1)), P(at(2)), F(at(3)), F(at(4)), nullptr,
                        P(at(2) + 256), F(at(7)), nullptr, 0, nullptr, 0, tokens, 1, 2, 6, 128,
                        128, GDN_BF16, nullptr, 0) == GDN_ERR_ALIAS);
    // misaligned q
    CHECK(check_prefill(P(at(0) + 2), P(at(1)), P(at(2)), F(at(3)), F(at(4)), nullptr, P(at(6)),
                        nullptr, nullptr, 0, nullptr, 0, tokens, 1, 2, 6, 128, 128, GDN_BF16,
                        nullptr, 0) == GDN_ERR_MISALIGNED);
    // NULL input with tokens > 0; none needed with tokens == 0
    CHECK(check_prefill(nullptr, P(at(1)), P(at(2)), F(at(3)), F(at(4)), nullptr, P(at(6)),
                        nullptr, nullptr, 0, nullptr, 0, tokens, 1, 2, 6, 128, 128, GDN_BF16,
                        nullptr, 0) == GDN_ERR_NULL_POINTER);
    CHECK(check_prefill(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, F(at(7)),
                        nullptr, 0, nullptr, 0, 0, 1, 2, 6, 128, 128, GDN_BF16, nullptr,
                        0) == GDN_OK);
    // byte counts that overflow int64
    CHECK(check_prefill(P(at(0)), P(at(1)), P(at(2)), F(at(3)), F(at(4)), nullptr, P(at(6)),
                        nullptr, nullptr, 0, nullptr, 0, INT64_MAX / 2, 1, 2, 6, 128, 128,
                        GDN_BF16, nullptr, 0) == GDN_ERR_BAD_SHAPE);
    CHECK(check_prefill(P(at(0)), P(at(1)), P(at(2)), F(at(3)), F(at(4)), nullptr, P(at(6)),
                        nullptr, nullptr, 0, nullptr, 0, -1, 1, 2, 6, 128, 128, GDN_BF16, nullptr,
                        0) == GDN_ERR_BAD_SHAPE);
    // workspace overlapping the final state; prefix rows overlapping out
    CHECK(check_prefill(P(at(0)), P(at(1)), P(at(2)), F(at(3)), F(at(4)), nullptr, P(at(6)),
                        F(at(7)), nullptr, 0, nullptr, 0, tokens, 1, 2, 6, 128, 128, GDN_BF16,
                        P(at(7) + 1024), 4096) == GDN_ERR_ALIAS);
    CHECK(check_prefill(P(at(0)), P(at(1)), P(at(2)), F(at(3)), F(at(4)), nullptr, P(at(6)),
                        nullptr, F(at(6) + 4096), 1, nullptr, 0, tokens, 1, 2, 6, 128, 128,
                        GDN_BF16, nullptr, 0) == GDN_ERR_ALIAS);
    // head shapes
    CHECK(check_heads(2, 5, 128, 128) == GDN_ERR_BAD_SHAPE);
    CHECK(check_heads(2, 6, 96, 96) == GDN_ERR_UNSUPPORTED);
    CHECK(check_heads(2, 6, 64, 128) == GDN_ERR_UNSUPPORTED);
    CHECK(check_heads(0, 6, 64, 64) == GDN_ERR_BAD_SHAPE);
    CHECK(check_heads(16, 48, 128, 128) == GDN_OK);

    // decode
    CHECK(check_decode(P(at(0)), P(at(1)), P(at(2)), F(at(3)), F(at(4)), F(at(5)), P(at(6)), 256,
                       16, 48, 128, 128, GDN_BF16) == GDN_OK);
    CHECK(check_decode(P(at(0)), P(at(1)), P(at(2)), F(at(3)), F(at(4)), F(at(5)), P(at(5)), 256,
                       16, 48, 128, 128, GDN_BF16) == GDN_ERR_ALIAS);
    CHECK(check_decode(P(at(0)), P(at(1)), P(at(2)), F(at(3)), F(at(4)), F(at(5)), P(at(6)), 0,
                       16, 48, 128, 128, GDN_BF16) == GDN_ERR_BAD_SHAPE);
    CHECK(check_decode(P(at(0)), P(at(1)), P(at(2)), F(at(3)), F(at(4)), F(at(5)), P(at(6)), 256,
                       16, 48, 128, 128, (gdn_dtype_t)7) == GDN_ERR_UNSUPPORTED);

    // K-token decode against a slot pool
    const int32_t *src = reinterpret_cast<const int32_t *>(at(9));
    const int32_t *dst = reinterpret_cast<const int32_t *>(at(10));
    CHECK(check_decode_multi(P(at(0)), P(at(1)), P(at(2)), F(at(3)), F(at(4)), F(at(5)), 512, src,
                             dst, P(at(6)), nullptr, 256, 4, 16, 48, 128, 128,
                             GDN_BF16) == GDN_OK);
    CHECK(check_decode_multi(P(at(0)), P(at(1)), P(at(2)), F(at(3)), F(at(4)), F(at(5)), 512, src,
                             reinterpret_cast<const int32_t *>(at(10) + 2), P(at(6)), nullptr, 256,
                             4, 16, 48, 128, 128, GDN_BF16) == GDN_ERR_MISALIGNED);
    CHECK(check_decode_multi(nullptr, nullptr, nullptr, nullptr, nullptr, F(at(5)), 512, src, dst,
                             nullptr, nullptr, 256, 0, 16, 48, 128, 128, GDN_BF16) == GDN_OK);
    CHECK(check_decode_multi(P(at(0)), P(at(1)), P(at(2)), F(at(3)), F(at(4)), F(at(5)), 0, src,
                             dst, P(at(6)), nullptr, 256, 4, 16, 48, 128, 128,
                             GDN_BF16) == GDN_ERR_BAD_SHAPE);

    // cu_seqlens contents (the GDN_DEBUG check), on exactly sized heap arrays
    {
        std::vector<int32_t> ok = {0, 10, 10, 300};
        CHECK(check_cu_seqlens(ok.data(), 3, 300) == GDN_OK);
        CHECK(check_cu_seqlens(ok.data(), 3, 301) == GDN_ERR_BAD_SHAPE);
        std::vector<int32_t> start = {5, 10, 300};
        CHECK(check_cu_seqlens(start.data(), 2, 300) == GDN_ERR_BAD_SHAPE);
        std::vector<int32_t> dec = {0, 200, 100, 300};
        CHECK(check_cu_seqlens(dec.data(), 3, 300) == GDN_ERR_BAD_SHAPE);
        std::vector<int32_t> one = {0, 0};
        CHECK(check_cu_seqlens(one.data(), 1, 0) == GDN_OK);
        CHECK(check_cu_seqlens(nullptr, 1, 0) == GDN_ERR_NULL_POINTER);
    }
}

// The oracle on exactly sized buffers, checked against two closed forms:
// beta = 0 leaves S_T = (prod alpha) S_0 and o_t = (prod_{s<=t} alpha_s) S_0 q_t;
// one token from a zero state gives o = beta (k . q) v.
static void oracle_runs() {
    const int T = 37, dk = 8, dv = 8;
    std::vector<float> q(T * dk), k(T * dk), v(T * dv), a(T), b(T, 0.f);
    unsigned s = 12345u;
    auto rnd = [&]() {
        s = s * 1664525u + 1013904223u;
        return (double)(s >> 8) / (double)(1u << 24) - 0.5;
    };
    for (auto &x : q) x = (float)rnd();
    for (auto &x : k) x = (float)rnd();
    for (auto &x : v) x = (float)rnd();
    for (auto &x : a) x = (float)(0.9 + 0.1 * rnd());
    std::vector<double> S0(dv * dk), S(dv * dk), o(T * dv);
    for (auto &x : S0) x = rnd();
    S = S0;
    CHECK(gdn_oracle_chain(q.data(), k.data(), v.data(), 0, a.data(), b.data(), 0, T, dk, dv, 1,
                           dk, dv, 1.0, S.data(), o.data()) == 0);
    double prod = 1.0;
    double worst = 0.0;
    for (int t = 0; t < T; ++t) {
        prod *= (double)a[t];
        for (int i = 0; i < dv; ++i) {
            double ref = 0.0;
            for (int j = 0; j < dk; ++j) ref += prod * S0[i * dk + j] * (double)q[t * dk + j];
            worst = fmax(worst, fabs(o[t * dv + i] - ref));
        }
    }
    for (int i = 0; i < dv * dk; ++i) worst = fmax(worst, fabs(S[i] - prod * S0[i]));
    CHECK(worst < 1e-12);

    // one token from zero, bf16 inputs (bit patterns)
    std::vector<uint16_t> qb(dk), kb(dk), vb(dv);
    std::vector<float> a1 = {0.5f}, b1 = {0.75f};
    for (int j = 0; j < dk; ++j) {
        qb[j] = (uint16_t)(0x3F80 + 16 * j);  // 1.0, 1.125, ...
        kb[j] = (uint16_t)(0xBF00 + 8 * j);   // -0.5, ...
    }
    for (int i = 0; i < dv; ++i) vb[i] = (uint16_t)(0x4000 + 4 * i);
    auto bf = [](uint16_t h) {
        uint32_t u = (uint32_t)h << 16;
        float f;
        memcpy(&f, &u, 4);
        return (double)f;
    };
    std::vector<double> S1(dv * dk, 0.0), o1(dv);
    CHECK(gdn_oracle_chain(qb.data(), kb.data(), vb.data(), 1, a1.data(), b1.data(), 0, 1, dk, dv,
                           1, dk, dv, 1.0, S1.data(), o1.data()) == 0);
    double kq = 0.0;
    for (int j = 0; j < dk; ++j) kq += bf(kb[j]) * bf(qb[j]);
    double w1 = 0.0;
    for (int i = 0; i < dv; ++i) w1 = fmax(w1, fabs(o1[i] - 0.75 * kq * bf(vb[i])));
    CHECK(w1 < 1e-12);
    // arguments the oracle refuses
    CHECK(gdn_oracle_chain(q.data(), k.data(), v.data(), 0, a.data(), b.data(), 0, -1, dk, dv, 1,
                           dk, dv, 1.0, S.data(), o.data()) == -1);
    CHECK(gdn_oracle_chain(q.data(), k.data(), v.data(), 5, a.data(), b.data(), 0, T, dk, dv, 1,
                           dk, dv, 1.0, S.data(), o.data()) == -1);
}

int main() {
    validation();
    oracle_runs();
    if (g_fail) {
        fprintf(stderr, "%d check(s) failed\n", g_fail);
        return 1;
    }
    printf("sanitized host checks ok\n");
    return 0;
}
