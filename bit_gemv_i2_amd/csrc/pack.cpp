// Offline host side of the library: absmean ternarisation and the repack of
// ternary weights into the gfx950 tile layout described in bitnet_w2a8.h.
//
// [P3] "BitNet + WebAssembly", "Why WASM": weights are ternary, obtained by
// absmean quantisation.  [P3] "What i2_s actually is": 128-weight blocks, one
// float scale per block, code 0/1/2 <-> -1/0/+1 in the interchange bytes.
// [P2] "GPU kernel breakthroughs": weights are reordered offline so that the
// kernel's loads are contiguous and decoding is a shift and a mask.
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

#include "bitnet_w2a8.h"
#include "layout.h"

using namespace bitnet_layout;

namespace {

// Rows are independent; large matrices are split over a few host threads.
template <typename F>
void parallel_rows(int64_t rows, F &&fn) {
    unsigned hw = std::thread::hardware_concurrency();
    int64_t nthr = hw ? (int64_t)hw : 1;
    if (nthr > 16) nthr = 16;
    if (rows < 64 || nthr <= 1) {
        fn((int64_t)0, rows);
        return;
    }
    if (nthr > rows) nthr = rows;
    std::vector<std::thread> th;
    int64_t per = (rows + nthr - 1) / nthr;
    for (int64_t t = 0; t < nthr; ++t) {
        int64_t r0 = t * per, r1 = std::min(rows, r0 + per);
        if (r0 >= r1) break;
        th.emplace_back([&fn, r0, r1] { fn(r0, r1); });
    }
    for (auto &x : th) x.join();
}

// Tile-layout position of weight (n, k): byte offset and bit shift.
inline void tile_pos(int64_t n, int64_t k, int64_t nblk, int64_t *byte, int *shift) {
    const int64_t T = n / kTileN, j = n % kTileN;
    const int64_t b = k / kBlockK, r = k % kBlockK;
    const int64_t s = r / 64, g = (r % 64) / 16, e = r % 16;  // e = 4*i + p
    const int64_t i = e / 4, p = e % 4;
    const int64_t slot = kTileN * g + j;
    *byte = (T * nblk + b) * kBrickBytes + slot * 8 + s * 4 + p;
    *shift = (int)(2 * i);
}

// t -> 2-bit two's complement code.
inline int tc_code(int t) { return t & 3; }

// Writes rows [n0, n1) of the tile layout from a per-weight getter.
template <typename Get>
void pack_rows(Get get, int64_t n0, int64_t n1, int64_t K, uint8_t *packed) {
    const int64_t nblk = K / kBlockK;
    // Whole tiles only (n0, n1 are multiples of 16): clear their bricks first.
    for (int64_t T = n0 / kTileN; T < n1 / kTileN; ++T)
        std::memset(packed + T * nblk * kBrickBytes, 0, (size_t)(nblk * kBrickBytes));
    for (int64_t n = n0; n < n1; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int64_t byte;
            int shift;
            tile_pos(n, k, nblk, &byte, &shift);
            packed[byte] |= (uint8_t)(tc_code(get(n, k)) << shift);
        }
}

// Scale granularity G (weights per scale): 128, 64, or 0 for one scale per matrix.
bool gran_ok(int G) { return G == 0 || G == 64 || G == 128; }

// Position in the tiled scale buffer of the scale of row n, 128-block b,
// 64-half h: [tile][block][16 rows] for G 128, [tile][block][16 rows][2 halves]
// for G 64 (one 8-byte load gives a row both halves).
inline int64_t tiled_scale_pos(int64_t n, int64_t b, int64_t h, int64_t nblk, int G) {
    const int64_t base = ((n / kTileN) * nblk + b) * kTileN + n % kTileN;
    return G == 64 ? base * 2 + h : base;
}

void tile_scales(const float *scales, int64_t N, int64_t K, int G, float *out) {
    const int64_t nblk = K / kBlockK;
    if (G == 0) {
        out[0] = scales[0];
        return;
    }
    const int64_t per = kBlockK / G;  // scales per row and 128-block
    for (int64_t n = 0; n < N; ++n)
        for (int64_t b = 0; b < nblk; ++b)
            for (int64_t h = 0; h < per; ++h)
                out[tiled_scale_pos(n, b, h, nblk, G)] = scales[(n * nblk + b) * per + h];
}

void untile_scales(const float *tiled, int64_t N, int64_t K, int G, float *out) {
    const int64_t nblk = K / kBlockK;
    if (G == 0) {
        out[0] = tiled[0];
        return;
    }
    const int64_t per = kBlockK / G;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t b = 0; b < nblk; ++b)
            for (int64_t h = 0; h < per; ++h)
                out[(n * nblk + b) * per + h] = tiled[tiled_scale_pos(n, b, h, nblk, G)];
}

int8_t ternary_of(float w, float gamma) {
    if (gamma == 0.0f) return 0;
    volatile float ratio = w / gamma;
    const float r = std::nearbyint((float)ratio);
    return (int8_t)(r > 1.0f ? 1 : (r < -1.0f ? -1 : (int)r));
}

bool shape_ok(int64_t N, int64_t K) {
    return N >= kTileN && K >= kBlockK && N % kTileN == 0 && K % kBlockK == 0 &&
           N <= (int64_t(1) << 30) && K <= (int64_t(1) << 30) && (N * K) < (int64_t(1) << 40);
}

// rows per host work item, a multiple of the tile height
int64_t tiles_of(int64_t N) { return N / kTileN; }

}  // namespace

extern "C" {

bitnet_status_t bitnet_check_shape(int64_t N, int64_t K) {
    return shape_ok(N, K) ? BITNET_OK : BITNET_ERR_UNSUPPORTED_SHAPE;
}

size_t bitnet_packed_bytes(int64_t N, int64_t K) {
    return shape_ok(N, K) ? (size_t)(N * K / 4) : 0;
}

size_t bitnet_scale_count(int64_t N, int64_t K) { return bitnet_scale_count_g(N, K, 128); }

size_t bitnet_scale_count_g(int64_t N, int64_t K, int scale_block) {
    if (!shape_ok(N, K) || !gran_ok(scale_block)) return 0;
    return scale_block == 0 ? 1 : (size_t)(N * K / scale_block);
}

bitnet_status_t bitnet_ternarize_absmean(const float *w, int64_t N, int64_t K, int8_t *ternary,
                                         float *scales) {
    return bitnet_ternarize_absmean_g(w, N, K, 128, ternary, scales);
}

bitnet_status_t bitnet_ternarize_absmean_g(const float *w, int64_t N, int64_t K, int scale_block,
                                           int8_t *ternary, float *scales) {
    if (!w || !ternary || !scales || !gran_ok(scale_block)) return BITNET_ERR_INVALID_ARG;
    if (N < 1 || K < kBlockK || K % kBlockK) return BITNET_ERR_UNSUPPORTED_SHAPE;
    if (scale_block == 0) {  // one gamma: fp64 sum over the matrix in row-major order
        double acc = 0.0;
        for (int64_t e = 0; e < N * K; ++e) acc += std::fabs((double)w[e]);
        const float gamma = (float)(acc / (double)(N * K));
        scales[0] = gamma;
        parallel_rows(N, [&](int64_t n0, int64_t n1) {
            for (int64_t e = n0 * K; e < n1 * K; ++e) ternary[e] = ternary_of(w[e], gamma);
        });
        return BITNET_OK;
    }
    const int64_t G = scale_block, nb = K / G;
    parallel_rows(N, [&](int64_t n0, int64_t n1) {
        for (int64_t n = n0; n < n1; ++n)
            for (int64_t b = 0; b < nb; ++b) {
                const float *src = w + n * K + b * G;
                double acc = 0.0;
                for (int64_t e = 0; e < G; ++e) acc += std::fabs((double)src[e]);
                const float gamma = (float)(acc / (double)G);
                scales[n * nb + b] = gamma;
                for (int64_t e = 0; e < G; ++e) ternary[n * K + b * G + e] = ternary_of(src[e], gamma);
            }
    });
    return BITNET_OK;
}

bitnet_status_t bitnet_pack_i2s(const int8_t *ternary, const float *scales, int64_t N, int64_t K,
                                uint8_t *packed_out, float *scales_out) {
    return bitnet_pack_i2s_g(ternary, scales, N, K, 128, packed_out, scales_out);
}

bitnet_status_t bitnet_pack_i2s_g(const int8_t *ternary, const float *scales, int64_t N, int64_t K,
                                  int scale_block, uint8_t *packed_out, float *scales_out) {
    if (!ternary || !scales || !packed_out || !scales_out || !gran_ok(scale_block)) return BITNET_ERR_INVALID_ARG;
    if (!shape_ok(N, K)) return BITNET_ERR_UNSUPPORTED_SHAPE;
    // validate everything before writing anything
    for (int64_t e = 0; e < N * K; ++e) {
        int8_t t = ternary[e];
        if (t < -1 || t > 1) return BITNET_ERR_INVALID_ARG;
    }
    parallel_rows(tiles_of(N), [&](int64_t t0, int64_t t1) {
        pack_rows([&](int64_t n, int64_t k) { return (int)ternary[n * K + k]; }, t0 * kTileN,
                  t1 * kTileN, K, packed_out);
    });
    tile_scales(scales, N, K, scale_block, scales_out);
    return BITNET_OK;
}

bitnet_status_t bitnet_repack_i2s(const uint8_t *i2s, const float *scales, int64_t N, int64_t K,
                                  uint8_t *packed_out, float *scales_out) {
    return bitnet_repack_i2s_g(i2s, scales, N, K, 128, packed_out, scales_out);
}

bitnet_status_t bitnet_repack_i2s_g(const uint8_t *i2s, const float *scales, int64_t N, int64_t K,
                                    int scale_block, uint8_t *packed_out, float *scales_out) {
    if (!i2s || !scales || !packed_out || !scales_out || !gran_ok(scale_block)) return BITNET_ERR_INVALID_ARG;
    if (!shape_ok(N, K)) return BITNET_ERR_UNSUPPORTED_SHAPE;
    // canonical byte j of block b (cb = 64 for the 64-weight format, else 128)
    // holds weight cb*b + (cb/4)*g + j at bits (7-2g)..(6-2g)
    const int64_t cb = scale_block == 64 ? 64 : 128, gw = cb / 4;
    auto canon = [&](int64_t n, int64_t k) -> int {
        const int64_t b = k / cb, r = k % cb, g = r / gw, j = r % gw;
        const unsigned byte = i2s[n * (K / 4) + b * gw + j];
        return (int)((byte >> (6 - 2 * g)) & 3u) - 1;  // code 3 -> 2 (rejected below)
    };
    for (int64_t e = 0; e < N * K / 4; ++e) {
        const unsigned byte = i2s[e];
        for (int g = 0; g < 4; ++g)
            if (((byte >> (2 * g)) & 3u) == 3u) return BITNET_ERR_INVALID_ARG;
    }
    parallel_rows(tiles_of(N), [&](int64_t t0, int64_t t1) {
        pack_rows(canon, t0 * kTileN, t1 * kTileN, K, packed_out);
    });
    tile_scales(scales, N, K, scale_block, scales_out);
    return BITNET_OK;
}

bitnet_status_t bitnet_unpack_i2s(const uint8_t *packed, const float *scales_tiled, int64_t N, int64_t K,
                                  int8_t *ternary_out, float *scales_out) {
    return bitnet_unpack_i2s_g(packed, scales_tiled, N, K, 128, ternary_out, scales_out);
}

bitnet_status_t bitnet_unpack_i2s_g(const uint8_t *packed, const float *scales_tiled, int64_t N, int64_t K,
                                    int scale_block, int8_t *ternary_out, float *scales_out) {
    if (!packed || !ternary_out || (!scales_tiled) != (!scales_out) || !gran_ok(scale_block))
        return BITNET_ERR_INVALID_ARG;
    if (!shape_ok(N, K)) return BITNET_ERR_UNSUPPORTED_SHAPE;
    const int64_t nblk = K / kBlockK;
    bool bad = false;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int64_t byte;
            int shift;
            tile_pos(n, k, nblk, &byte, &shift);
            const int code = (packed[byte] >> shift) & 3;
            if (code == 2) bad = true;
            ternary_out[n * K + k] = (int8_t)(code == 3 ? -1 : code);
        }
    if (scales_tiled) untile_scales(scales_tiled, N, K, scale_block, scales_out);
    return bad ? BITNET_ERR_INVALID_ARG : BITNET_OK;
}

}  // extern "C"
