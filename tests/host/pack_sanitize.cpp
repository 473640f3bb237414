// Host-only driver for the library's offline code (pack.cpp), built with g++ under the address,
// undefined-behaviour and thread sanitizers by tests/test_host_sanitizers.py: ternarise -> pack ->
// unpack round trips and the canonical i2_s repack, for every scale granularity, over many shapes,
// and rejection of invalid input.  The canonical byte rule ([P3] "What i2_s actually is": code =
// t + 1, four codes per byte; byte j of a 128-block holds weights 32g + j, g = 0 in the top bits)
// is restated here, independently of the library.
#include <cstdio>
#include <cstdlib>
#include <cstdint>
#include <random>
#include <vector>
#include "bitnet_w2a8.h"

static int fails = 0;
#define CHECK(c) do { if (!(c)) { std::printf("FAIL %s line %d\n", #c, __LINE__); ++fails; } } while (0)

int main() {
    std::mt19937 rng(7);
    const int grans[3] = {128, 64, 0};
    for (int iter = 0; iter < 60; ++iter) {
        const int64_t N = 16 * (1 + rng() % 40), K = 128 * (1 + rng() % 12);
        const int G = grans[iter % 3];
        std::normal_distribution<float> nd(0.f, 0.02f);
        std::vector<float> w(N * K);
        for (auto &x : w) x = nd(rng);
        if (iter % 7 == 0) for (int64_t k = 0; k < 128; ++k) w[k] = 0.f;  // a zero block
        const size_t ns = bitnet_scale_count_g(N, K, G);
        CHECK(ns > 0);
        std::vector<int8_t> t(N * K), t2(N * K);
        std::vector<float> s(ns), st(ns), s2(ns);
        CHECK(bitnet_ternarize_absmean_g(w.data(), N, K, G, t.data(), s.data()) == BITNET_OK);
        const size_t nb = bitnet_packed_bytes(N, K);
        std::vector<uint8_t> p(nb);
        CHECK(bitnet_pack_i2s_g(t.data(), s.data(), N, K, G, p.data(), st.data()) == BITNET_OK);
        CHECK(bitnet_unpack_i2s_g(p.data(), st.data(), N, K, G, t2.data(), s2.data()) == BITNET_OK);
        CHECK(t == t2);
        CHECK(s == s2);
        // canonical i2_s bytes (code = t + 1; byte j of 128-block b holds weights 32g + j, g in bits 7-2g..6-2g)
        std::vector<uint8_t> canon(N * K / 4, 0);
        for (int64_t n = 0; n < N; ++n)
            for (int64_t b = 0; b < K / 128; ++b)
                for (int g = 0; g < 4; ++g)
                    for (int j = 0; j < 32; ++j) {
                        const int code = t[n * K + b * 128 + 32 * g + j] + 1;
                        canon[(n * K + b * 128) / 4 + j] |= (uint8_t)(code << (6 - 2 * g));
                    }
        if (G == 128) {
            std::vector<uint8_t> p2(nb);
            std::vector<float> st2(ns);
            CHECK(bitnet_repack_i2s_g(canon.data(), s.data(), N, K, G, p2.data(), st2.data()) == BITNET_OK);
            CHECK(p2 == p);
            CHECK(st2 == st);
        }
        // invalid inputs are rejected without touching memory
        t[0] = 2;
        CHECK(bitnet_pack_i2s_g(t.data(), s.data(), N, K, G, p.data(), st.data()) != BITNET_OK);
    }
    CHECK(bitnet_packed_bytes(8, 128) == 0);
    CHECK(bitnet_pack_i2s(nullptr, nullptr, 16, 128, nullptr, nullptr) != BITNET_OK);
    std::printf("%s (%d failures)\n", fails ? "FAILED" : "ok", fails);
    return fails ? 1 : 0;
}
