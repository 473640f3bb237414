// Table-lookup decode product for one token, an experiment beside the
// matrix-core decode kernel.
//
// Prior art: the CPU lookup-table kernels of [P2] "5x performance leap: BitNet
// vs llama.cpp" ("Architecture foundations", item 1: TL1/TL2 precompute the
// sums a small group of ternary weights can take against the activations, then
// replace the multiply-adds by table lookups) and [P3] "BitNet + WebAssembly"
// (the LUT kernel's table constructor builds a 16-entry table per group).  The
// product computed is the one of bitnet_w2a8_gemv:
//     y[n] = s_a * sum_b S[n][b] * sum_{k in block b} T[n][k] * Q[k]
// with the inner sums exact in int32.
//
// gfx950 form.  The weights stay in the tile layout (include/bitnet_w2a8.h):
// lane l = 16g + j of a wave reads, per 16-row tile and 128-weight block, the
// two words holding row j's weights 64s + 16g + 4i + p (s = word, i = field,
// p = byte).  A nibble of byte p holds two codes: fields 0-1 (weights +p and
// +p+4) or fields 2-3 (+p+8 and +p+12).  For every such pair of activations a
// wave builds a 16-entry int16 table in LDS, entry c1*4 + c0 = t(c0)*Q[ka] +
// t(c1)*Q[kb] with t the 2-bit two's-complement code (0 -> 0, 1 -> +1, 3 ->
// -1; code 2 never occurs and holds 0).  A 16-weight word then costs eight
// table reads instead of a decode and a matrix-core step.
//
// Each wave owns a K-slice of the workgroup's rows (the same split as the
// matrix-core decode), builds the tables of up to three blocks of its slice at
// a time (64 pairs x 16 entries per block) and reuses them for every 16-row
// tile of the workgroup: more tiles per workgroup amortise the table build
// over more weights, fewer leave more workgroups to cover the chip.  Tables
// are wave-private, so the only barrier is the final cross-wave reduction.
// Bank layout: the eight pairs read by one lane group (fixed g) for one word
// form a 128-entry group padded to 144 entries (72 dwords), so the four lane
// groups of one read instruction fall in four disjoint 8-dword bank windows.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "bitnet_w2a8.h"
#include "layout.h"

using namespace bitnet_layout;

namespace {

typedef unsigned v2u_t __attribute__((ext_vector_type(2)));

constexpr int kLutWave = 64;
constexpr int kLutMaxWaves = 8;
constexpr int kLutPair = 16;                        // int16 entries per pair table
constexpr int kLutGroup = 8 * kLutPair + 16;        // 8 pairs of one lane group + pad = 144
constexpr int kLutBlock = 8 * kLutGroup;            // 4 lane groups x 2 words = 1152 entries
constexpr int kLutChunk = 3;  // blocks whose tables a wave holds at once (8 waves: 54 KB of LDS)

__device__ __forceinline__ int code_value(int c, int v) {  // t(c) * v for a 2-bit code
    return c == 1 ? v : (c == 3 ? -v : 0);
}

// Builds the 64 pair tables of one block: lane l owns pair (s, g, h, p) =
// (l >> 5, (l >> 3) & 3, (l >> 2) & 1, l & 3) joining weights
// 64s + 16g + 8h + p and that + 4 of the block.
__device__ __forceinline__ void build_block_tables(int16_t *tab, const int8_t *__restrict__ qb, int l) {
    const int s = l >> 5, g = (l >> 3) & 3, h = (l >> 2) & 1, p = l & 3;
    const int ka = 64 * s + 16 * g + 8 * h + p;
    const int va = qb[ka], vb = qb[ka + 4];
    uint32_t packed[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {  // entries 2e (low half) and 2e+1 (high half)
        const int lo = code_value((2 * e) & 3, va) + code_value((2 * e) >> 2, vb);
        const int hi = code_value((2 * e + 1) & 3, va) + code_value((2 * e + 1) >> 2, vb);
        packed[e] = ((uint32_t)lo & 0xFFFFu) | ((uint32_t)hi << 16);
    }
    uint4 *dst = reinterpret_cast<uint4 *>(tab + (s * 4 + g) * kLutGroup + (h * 4 + p) * kLutPair);
    dst[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    dst[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
}

// Sum of the 16 weights of one word against the activations, by table reads:
// grp points at the lane group's 8 pair tables of that word.
__device__ __forceinline__ int lookup_word(const int16_t *grp, uint32_t w) {
    int sum = 0;
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int h = 0; h < 2; ++h) sum += grp[(h * 4 + p) * kLutPair + ((w >> (8 * p + 4 * h)) & 15u)];
    return sum;
}

// R: 16-row tiles per workgroup.  Workgroup = nw waves; wave w sums blocks
// [w * per, min(nblk, (w + 1) * per)) of each of its tiles.
template <int R>
__global__ __launch_bounds__(kLutWave * kLutMaxWaves) void gemv_lut_kernel(
    const uint8_t *__restrict__ packed, const float *__restrict__ scales, const int8_t *__restrict__ q,
    const float *__restrict__ s_a, float *__restrict__ y, int32_t *__restrict__ acc, int N, int K, int per) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int nblk = K >> 7, ntiles = N >> 4, nw = blockDim.x >> 6;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l = threadIdx.x & 63, g = l >> 4, j = l & 15;
    const int tile0 = blockIdx.x * R;
    int16_t *tab = reinterpret_cast<int16_t *>(smem) + (size_t)w * kLutChunk * kLutBlock;

    const int bw0 = w * per, bw1 = min(nblk, bw0 + per);
    float yacc[R];
    int iacc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        yacc[r] = 0.0f;
        iacc[r] = 0;
    }
    for (int c0 = bw0; c0 < bw1; c0 += kLutChunk) {
        const int nb = min(kLutChunk, bw1 - c0);
        // every brick word and scale of the chunk first (clamped, in bounds), then the tables
        uint2 wv[R][kLutChunk];
        float sc[R][kLutChunk];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int t = min(tile0 + r, ntiles - 1);
#pragma unroll
            for (int i = 0; i < kLutChunk; ++i) {
                const size_t bi = (size_t)t * nblk + c0 + min(i, nb - 1);
                const v2u_t w2 = __builtin_nontemporal_load(reinterpret_cast<const v2u_t *>(packed + bi * kBrickBytes + l * 8));
                wv[r][i] = make_uint2(w2.x, w2.y);
                sc[r][i] = __builtin_nontemporal_load(scales + bi * kTileN + j);
            }
        }
        for (int i = 0; i < nb; ++i) build_block_tables(tab + i * kLutBlock, q + (size_t)(c0 + i) * kBlockK, l);
        // LDS serves one wave's accesses in order; the fence keeps the compiler from
        // moving a table read above the writes of other lanes.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int i = 0; i < kLutChunk; ++i) {
            if (i < nb) {
                const int16_t *blk = tab + i * kLutBlock + g * kLutGroup;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const int a = lookup_word(blk, wv[r][i].x) + lookup_word(blk + 4 * kLutGroup, wv[r][i].y);
                    iacc[r] += a;
                    yacc[r] = fmaf(sc[r][i], (float)a, yacc[r]);
                }
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    // cross-lane-group and cross-wave reduction in a fixed order (deterministic)
    __syncthreads();  // every wave is done with its tables; the region is reused
    float *redf = reinterpret_cast<float *>(smem);
    int *redi = reinterpret_cast<int *>(smem) + nw * R * kLutWave;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        redf[(w * R + r) * kLutWave + l] = yacc[r];
        redi[(w * R + r) * kLutWave + l] = iacc[r];
    }
    __syncthreads();
    const int t = threadIdx.x;
    if (t < 16 * R) {
        const int r = t >> 4, jj = t & 15, tile = tile0 + r;
        if (tile < ntiles) {
            float fs = 0.0f;
            int is = 0;
            for (int ww = 0; ww < nw; ++ww)
#pragma unroll
                for (int gg = 0; gg < 4; ++gg) {
                    fs += redf[(ww * R + r) * kLutWave + 16 * gg + jj];
                    is += redi[(ww * R + r) * kLutWave + 16 * gg + jj];
                }
            const size_t o = (size_t)tile * kTileN + jj;
            y[o] = fs * s_a[0];
            if (acc) acc[o] = is;
        }
    }
}

template <int R>
void lut_launch(const uint8_t *packed, const float *scales, const int8_t *q, const float *s_a, float *y,
                int32_t *acc, int N, int K, hipStream_t stream) {
    const int nblk = K >> 7;
    int nw = nblk < kLutMaxWaves ? nblk : kLutMaxWaves;
    const int per = (nblk + nw - 1) / nw;
    nw = (nblk + per - 1) / per;
    const int ntiles = N >> 4;
    const int grid = (ntiles + R - 1) / R;
    const size_t tables = (size_t)nw * kLutChunk * kLutBlock * sizeof(int16_t);
    const size_t red = (size_t)nw * R * kLutWave * 8;
    const size_t lds = tables > red ? tables : red;
    hipLaunchKernelGGL(gemv_lut_kernel<R>, dim3(grid), dim3(nw * kLutWave), lds, stream, packed, scales, q, s_a, y,
                       acc, N, K, per);
}

bool is_aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

}  // namespace

extern "C" bitnet_status_t bitnet_w2a8_gemv_lut(const uint8_t *packed, const float *scales, const int8_t *q,
                                                const float *s_a, float *y, int32_t *acc, int N, int K,
                                                int tiles_per_group, hipStream_t stream) {
    if (!packed || !scales || !q || !s_a || !y) return BITNET_ERR_INVALID_ARG;
    if (!is_aligned(packed, 16) || !is_aligned(scales, 16) || !is_aligned(s_a, 4) || !is_aligned(y, 4) ||
        (acc && !is_aligned(acc, 4)))
        return BITNET_ERR_INVALID_ARG;
    if (tiles_per_group != 0 && tiles_per_group != 1 && tiles_per_group != 2 && tiles_per_group != 4)
        return BITNET_ERR_INVALID_ARG;
    if (bitnet_check_shape(N, K) != BITNET_OK || K > (1 << 22)) return BITNET_ERR_UNSUPPORTED_SHAPE;
    // default: two tiles per workgroup while that still leaves one workgroup per CU
    // (256 CUs; measured best at 13824 and 20480 rows), else one (2560 rows)
    int R = tiles_per_group;
    if (R == 0) R = (N >> 5) >= 256 ? 2 : 1;
    switch (R) {
        case 1: lut_launch<1>(packed, scales, q, s_a, y, acc, N, K, stream); break;
        case 2: lut_launch<2>(packed, scales, q, s_a, y, acc, N, K, stream); break;
        default: lut_launch<4>(packed, scales, q, s_a, y, acc, N, K, stream); break;
    }
    return hipGetLastError() == hipSuccess ? BITNET_OK : BITNET_ERR_HIP;
}
