// gfx950 (MI355X) kernels of the W2A8 ternary product and their C ABI.
//
// The product ([P2] "5x performance leap: BitNet vs llama.cpp",
// "Architecture foundations", item 2: 2-bit weights x 8-bit activations;
// [P3] "BitNet + WebAssembly", "What i2_s actually is": 128-weight blocks with
// one float scale each, dequantise = lookup then scale):
//     y[m][n] = s_a[m] * sum_b S[n][b] * A[m][n][b],
//     A[m][n][b] = sum_{k in block b} T[n][k] * Q[m][k]   (exact int32)
//
// Matrix-core formulation.  v_mfma_i32_16x16x64_i8 multiplies a 16x64 int8
// tile of activations (16 tokens, padded with zeros) by a 64x16 int8 tile of
// weights (16 rows).  Each lane holds 16 int8 of each operand: lane l = 16g+j
// supplies token j / row j at k = 16g .. 16g+15, and receives the int32
// results for tokens 4g..4g+3 of row j.  The tile layout stores exactly those
// 16 weight codes of one lane in one 32-bit word, so the decode of a K-step is
// one load per lane plus 3 shifts and 4 masks, producing 64*t in every byte
// (two's-complement 2-bit code moved to the byte's top bits).  The block sum is
// then 64*A[m][n][b]; the factor 64 is removed with the token scale (an exact
// power-of-two rescale).  Two K-steps make one 128-weight block, after which
// the int32 tile is drained into fp32 with the block scale.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "bitnet_w2a8.h"
#include "layout.h"

using namespace bitnet_layout;

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kMaxGemvWaves = 16;
constexpr int kGemvMaxM = 16;

inline bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// --------------------------------------------------------------------------
// decode of one tile-layout word: field i of byte p (weight 4i+p) -> byte p of
// lane-word i, as 64*t.  Result words 0..3 hold weights 0..3, 4..7, 8..11,
// 12..15 in byte order: the int8 operand layout of the matrix core.
// --------------------------------------------------------------------------
__device__ __forceinline__ v4i decode16(uint32_t w) {
    v4i r;
    r[0] = (int)((w << 6) & 0xC0C0C0C0u);
    r[1] = (int)((w << 4) & 0xC0C0C0C0u);
    r[2] = (int)((w << 2) & 0xC0C0C0C0u);
    r[3] = (int)(w & 0xC0C0C0C0u);
    return r;
}

__device__ __forceinline__ v4i mfma_i8(v4i a, v4i b, v4i c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// ==========================================================================
// a4: per-token absmax int8 quantisation.  One workgroup of 256 threads per
// token; each thread handles 8 consecutive values per step (16-byte loads for
// bf16, 2x16 for fp32).  Pass 1 finds amax (exact, order-free), pass 2
// quantises (the token is re-read from L2).
// MODE 0: bf16 input; 1: fp32 input; 2: fp32 [M][2H] folded (h = lo + hi).
// ==========================================================================
template <int MODE>
__device__ __forceinline__ void load8(const void *__restrict__ x, int m, int K, int v, float out[8]) {
    if (MODE == 0) {
        const uint4 u = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(x) + (size_t)m * K)[v];
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[2 * i] = __uint_as_float(w[i] << 16);
            out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    } else if (MODE == 1) {
        const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(x) + (size_t)m * K) + 2 * v;
        const float4 a = p[0], b = p[1];
        out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
        out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
    } else {
        const float *row = static_cast<const float *>(x) + (size_t)m * 2 * K;
        const float4 *lo = reinterpret_cast<const float4 *>(row) + 2 * v;
        const float4 *hi = reinterpret_cast<const float4 *>(row + K) + 2 * v;
        const float4 a = lo[0], b = lo[1], c = hi[0], d = hi[1];
        out[0] = __fadd_rn(a.x, c.x); out[1] = __fadd_rn(a.y, c.y);
        out[2] = __fadd_rn(a.z, c.z); out[3] = __fadd_rn(a.w, c.w);
        out[4] = __fadd_rn(b.x, d.x); out[5] = __fadd_rn(b.y, d.y);
        out[6] = __fadd_rn(b.z, d.z); out[7] = __fadd_rn(b.w, d.w);
    }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
    return v;
}

template <int MODE>
__global__ __launch_bounds__(256) void quant_act_kernel(const void *__restrict__ x, int K,
                                                         int8_t *__restrict__ q, float *__restrict__ s_a) {
    __shared__ float part[4];
    const int m = blockIdx.x;
    const int nvec = K >> 3;
    float amax = 0.0f;
    for (int v = threadIdx.x; v < nvec; v += 256) {
        float f[8];
        load8<MODE>(x, m, K, v, f);
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
    }
    amax = wave_max(amax);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
    const float amax_c = fmaxf(amax, 1e-5f);
    const float inv = __fdiv_rn(127.0f, amax_c);
    uint2 *qrow = reinterpret_cast<uint2 *>(q + (size_t)m * K);
    for (int v = threadIdx.x; v < nvec; v += 256) {
        float f[8];
        load8<MODE>(x, m, K, v, f);
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float r = rintf(__fmul_rn(f[i], inv));
            r = fminf(fmaxf(r, -127.0f), 127.0f);
            const uint32_t b = (uint32_t)(uint8_t)(int8_t)(int)r;
            if (i < 4) lo |= b << (8 * i);
            else hi |= b << (8 * (i - 4));
        }
        qrow[v] = make_uint2(lo, hi);
    }
    if (threadIdx.x == 0) s_a[m] = __fdiv_rn(amax_c, 127.0f);
}

// ==========================================================================
// a5: decode product, M <= 16.  One workgroup per 16-row tile, S waves split
// the K blocks (split-K); wave w owns blocks [w*per, w*per + per).  Every lane
// issues all of its weight, scale and activation loads for a chunk of NB
// blocks before the first matrix-core step, so a wave keeps NB x 8 bytes per
// lane of the weight stream in flight.  Partial sums are reduced through LDS
// in wave order (deterministic).
// MW = number of accumulator elements drained per lane (1, 2 or 4): with M <= 4
// only tokens 0..M-1 (lanes 0..15, elements < M) are real.
// ==========================================================================
template <int NB, int MW, bool INT_OUT>
__global__ __launch_bounds__(1024) void gemv_kernel(const uint8_t *__restrict__ packed,
                                                     const float *__restrict__ scales,
                                                     const int8_t *__restrict__ q,
                                                     const float *__restrict__ s_a,
                                                     float *__restrict__ y, int32_t *__restrict__ acc_out,
                                                     int M, int N, int K, int per) {
    __shared__ int red[kMaxGemvWaves][4][kWave];
    const int nblk = K >> 7;
    const int tile = blockIdx.x;
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63, g = l >> 4, j = l & 15;
    const int nw = blockDim.x >> 6;
    const int bw0 = w * per;
    const int bw1 = min(nblk, bw0 + per);
    const bool tok = j < M;

    float yacc[MW];
    int iacc[4];
#pragma unroll
    for (int e = 0; e < MW; ++e) yacc[e] = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) iacc[e] = 0;

    for (int c0 = bw0; c0 < bw1; c0 += NB) {
        const int nb = min(NB, bw1 - c0);
        const uint8_t *wp = packed + ((size_t)tile * nblk + c0) * kBrickBytes + l * 8;
        const float *sp = scales + ((size_t)tile * nblk + c0) * kTileN + j;
        const int8_t *qp = q + (size_t)j * K + (size_t)c0 * kBlockK + g * 16;
        uint2 wv[NB];
        float sc[NB];
        v4i a[NB][2];
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            if (i < nb) {
                wv[i] = *reinterpret_cast<const uint2 *>(wp + i * kBrickBytes);
                if (!INT_OUT) sc[i] = sp[i * kTileN];
            }
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) {
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                a[i][s] = v4i{0, 0, 0, 0};
                if (i < nb && tok) a[i][s] = *reinterpret_cast<const v4i *>(qp + i * kBlockK + s * 64);
            }
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            if (i < nb) {
                v4i c = v4i{0, 0, 0, 0};
                c = mfma_i8(a[i][0], decode16(wv[i].x), c);
                c = mfma_i8(a[i][1], decode16(wv[i].y), c);
                if (INT_OUT) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) iacc[e] += c[e];
                } else {
#pragma unroll
                    for (int e = 0; e < MW; ++e) yacc[e] = fmaf(sc[i], (float)c[e], yacc[e]);
                }
            }
        }
    }

    constexpr int NE = INT_OUT ? 4 : MW;
#pragma unroll
    for (int e = 0; e < NE; ++e) red[w][e][l] = INT_OUT ? iacc[e] : __float_as_int(yacc[e]);
    __syncthreads();
    if (w == 0) {
        const int n = tile * kTileN + j;
#pragma unroll
        for (int e = 0; e < NE; ++e) {
            const int m = 4 * g + e;
            if (INT_OUT) {
                int sum = 0;
                for (int ww = 0; ww < nw; ++ww) sum += red[ww][e][l];
                if (m < M) acc_out[(size_t)m * N + n] = sum >> 6;  // exact: sum is 64 * integer
            } else {
                float sum = 0.0f;
                for (int ww = 0; ww < nw; ++ww) sum += __int_as_float(red[ww][e][l]);
                if (m < M) y[(size_t)m * N + n] = sum * (s_a[m] * 0.015625f);
            }
        }
    }
}

// ==========================================================================
// a6: prefill product, any M.  Workgroup = 4 waves (2 x 2) on a 128-token x
// 128-row output tile; each wave owns 64 tokens x 64 rows = 4 x 4 matrix-core
// tiles.  Per 128-weight block a wave decodes its 4 row-tiles once (8 words
// per lane) and reuses them for its 4 token-tiles (32 matrix-core steps),
// then drains the int32 tiles into fp32 with the block scales.  The next
// block's operands are loaded while the current one computes.
// ==========================================================================
constexpr int kGemmBM = 128, kGemmBN = 128;

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

template <int OUT>  // 0: bf16 y, 1: fp32 y, 2: int32 acc
__global__ __launch_bounds__(256) void gemm_kernel(const uint8_t *__restrict__ packed,
                                                    const float *__restrict__ scales,
                                                    const int8_t *__restrict__ q,
                                                    const float *__restrict__ s_a, void *__restrict__ yout,
                                                    int M, int N, int K) {
    const int nblk = K >> 7;
    const int ntile_n = N >> 4;
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63, g = l >> 4, j = l & 15;
    const int tm0 = blockIdx.y * kGemmBM + (w >> 1) * 64;  // first token of this wave
    const int tt0 = blockIdx.x * (kGemmBN / 16) + (w & 1) * 4;  // first row-tile of this wave

    // per-lane sources
    const int8_t *qp[4];
    bool qok[4];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) {
        const int tokn = tm0 + 16 * ti + j;
        qok[ti] = tokn < M;
        qp[ti] = q + (size_t)(qok[ti] ? tokn : 0) * K + g * 16;
    }
    bool rok[4];
#pragma unroll
    for (int tj = 0; tj < 4; ++tj) rok[tj] = (tt0 + tj) < ntile_n;

    float yacc[4][4][4];
    int iacc[4][4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                yacc[a][b][e] = 0.0f;
                iacc[a][b][e] = 0;
            }

    v4i an[4][2];
    uint2 wn[4];
    float sn[4];
    auto load_block = [&](int b, v4i (&aa)[4][2], uint2 (&ww)[4], float (&ss)[4]) {
#pragma unroll
        for (int ti = 0; ti < 4; ++ti)
#pragma unroll
            for (int s = 0; s < 2; ++s)
                aa[ti][s] = qok[ti] ? *reinterpret_cast<const v4i *>(qp[ti] + (size_t)b * kBlockK + s * 64)
                                    : v4i{0, 0, 0, 0};
#pragma unroll
        for (int tj = 0; tj < 4; ++tj) {
            const size_t brick = (size_t)(rok[tj] ? tt0 + tj : 0) * nblk + b;
            ww[tj] = rok[tj] ? *reinterpret_cast<const uint2 *>(packed + brick * kBrickBytes + l * 8)
                             : make_uint2(0u, 0u);
            ss[tj] = (OUT != 2 && rok[tj]) ? scales[brick * kTileN + j] : 0.0f;
        }
    };
    load_block(0, an, wn, sn);
    for (int b = 0; b < nblk; ++b) {
        v4i ac[4][2];
        uint2 wc[4];
        float sc[4];
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
            ac[ti][0] = an[ti][0];
            ac[ti][1] = an[ti][1];
        }
#pragma unroll
        for (int tj = 0; tj < 4; ++tj) {
            wc[tj] = wn[tj];
            sc[tj] = sn[tj];
        }
        if (b + 1 < nblk) load_block(b + 1, an, wn, sn);
        v4i bw[4][2];
#pragma unroll
        for (int tj = 0; tj < 4; ++tj) {
            bw[tj][0] = decode16(wc[tj].x);
            bw[tj][1] = decode16(wc[tj].y);
        }
#pragma unroll
        for (int ti = 0; ti < 4; ++ti)
#pragma unroll
            for (int tj = 0; tj < 4; ++tj) {
                v4i c = v4i{0, 0, 0, 0};
                c = mfma_i8(ac[ti][0], bw[tj][0], c);
                c = mfma_i8(ac[ti][1], bw[tj][1], c);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (OUT == 2) iacc[ti][tj][e] += c[e];
                    else yacc[ti][tj][e] = fmaf(sc[tj], (float)c[e], yacc[ti][tj][e]);
                }
            }
    }

    // epilogue: lane (g, j), tile (ti, tj), element e -> token tm0+16ti+4g+e, row 16(tt0+tj)+j
#pragma unroll
    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int m = tm0 + 16 * ti + 4 * g + e;
            if (m >= M) continue;
            const float f = (OUT == 2) ? 0.0f : s_a[m] * 0.015625f;
#pragma unroll
            for (int tj = 0; tj < 4; ++tj) {
                if (!rok[tj]) continue;
                const size_t idx = (size_t)m * N + (size_t)(tt0 + tj) * 16 + j;
                if (OUT == 0) static_cast<uint16_t *>(yout)[idx] = f32_to_bf16_rne(yacc[ti][tj][e] * f);
                else if (OUT == 1) static_cast<float *>(yout)[idx] = yacc[ti][tj][e] * f;
                else static_cast<int32_t *>(yout)[idx] = iacc[ti][tj][e] >> 6;
            }
        }
}

// --------------------------------------------------------------------------
// host-side launch helpers
// --------------------------------------------------------------------------
bool shape_ok(int64_t N, int64_t K) { return bitnet_check_shape(N, K) == BITNET_OK; }

bitnet_status_t launched() {
    return hipGetLastError() == hipSuccess ? BITNET_OK : BITNET_ERR_HIP;
}

template <int NB, bool INT_OUT>
void gemv_launch_mw(int mw, dim3 grid, dim3 block, hipStream_t st, const uint8_t *p, const float *s,
                    const int8_t *q, const float *sa, float *y, int32_t *acc, int M, int N, int K, int per) {
    if (INT_OUT || mw == 4)
        hipLaunchKernelGGL((gemv_kernel<NB, 4, INT_OUT>), grid, block, 0, st, p, s, q, sa, y, acc, M, N, K, per);
    else if (mw == 2)
        hipLaunchKernelGGL((gemv_kernel<NB, 2, INT_OUT>), grid, block, 0, st, p, s, q, sa, y, acc, M, N, K, per);
    else
        hipLaunchKernelGGL((gemv_kernel<NB, 1, INT_OUT>), grid, block, 0, st, p, s, q, sa, y, acc, M, N, K, per);
}

template <bool INT_OUT>
void gemv_launch(const uint8_t *p, const float *s, const int8_t *q, const float *sa, float *y, int32_t *acc,
                 int M, int N, int K, hipStream_t st) {
    const int nblk = K / (int)kBlockK;
    // split-K: about 4 blocks per wave, at most 16 waves per workgroup
    int nw = (nblk + 3) / 4;
    if (nw > kMaxGemvWaves) nw = kMaxGemvWaves;
    if (nw < 1) nw = 1;
    const int per = (nblk + nw - 1) / nw;
    nw = (nblk + per - 1) / per;  // no idle wave
    const int nb = per < 8 ? per : 8;
    const int mw = M == 1 ? 1 : (M == 2 ? 2 : 4);
    dim3 grid(N / (int)kTileN), block(kWave * nw);
    switch (nb) {
        case 1: gemv_launch_mw<1, INT_OUT>(mw, grid, block, st, p, s, q, sa, y, acc, M, N, K, per); break;
        case 2: gemv_launch_mw<2, INT_OUT>(mw, grid, block, st, p, s, q, sa, y, acc, M, N, K, per); break;
        case 3: gemv_launch_mw<3, INT_OUT>(mw, grid, block, st, p, s, q, sa, y, acc, M, N, K, per); break;
        case 4: gemv_launch_mw<4, INT_OUT>(mw, grid, block, st, p, s, q, sa, y, acc, M, N, K, per); break;
        case 5: gemv_launch_mw<5, INT_OUT>(mw, grid, block, st, p, s, q, sa, y, acc, M, N, K, per); break;
        case 6: gemv_launch_mw<6, INT_OUT>(mw, grid, block, st, p, s, q, sa, y, acc, M, N, K, per); break;
        case 7: gemv_launch_mw<7, INT_OUT>(mw, grid, block, st, p, s, q, sa, y, acc, M, N, K, per); break;
        default: gemv_launch_mw<8, INT_OUT>(mw, grid, block, st, p, s, q, sa, y, acc, M, N, K, per); break;
    }
}

template <int OUT>
void gemm_launch(const uint8_t *p, const float *s, const int8_t *q, const float *sa, void *y, int M, int N, int K,
                 hipStream_t st) {
    dim3 grid((N + kGemmBN - 1) / kGemmBN, (M + kGemmBM - 1) / kGemmBM), block(256);
    hipLaunchKernelGGL((gemm_kernel<OUT>), grid, block, 0, st, p, s, q, sa, y, M, N, K);
}

bool gemm_grid_ok(int M) { return (M + kGemmBM - 1) / kGemmBM <= 65535; }

}  // namespace

extern "C" {

const char *bitnet_status_str(int status) {
    switch (status) {
        case BITNET_OK: return "ok";
        case BITNET_ERR_INVALID_ARG: return "invalid argument";
        case BITNET_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
        case BITNET_ERR_HIP: return "HIP error";
        default: return "unknown status";
    }
}

bitnet_status_t bitnet_quant_act(const void *x, int xdt, int M, int K, int8_t *q, float *s_a,
                                 hipStream_t stream) {
    if (!x || !q || !s_a || !aligned(x, 16) || !aligned(q, 16) || !aligned(s_a, 4)) return BITNET_ERR_INVALID_ARG;
    if (xdt != BITNET_DT_BF16 && xdt != BITNET_DT_F32) return BITNET_ERR_INVALID_ARG;
    if (M < 1 || M > 65535 * 1024 || K < 16 || K % 16) return BITNET_ERR_UNSUPPORTED_SHAPE;
    if (xdt == BITNET_DT_BF16)
        hipLaunchKernelGGL(quant_act_kernel<0>, dim3(M), dim3(256), 0, stream, x, K, q, s_a);
    else
        hipLaunchKernelGGL(quant_act_kernel<1>, dim3(M), dim3(256), 0, stream, x, K, q, s_a);
    return launched();
}

bitnet_status_t bitnet_quant_act_fold(const float *y, int M, int H, int8_t *q, float *s_a, hipStream_t stream) {
    if (!y || !q || !s_a || !aligned(y, 16) || !aligned(q, 16) || !aligned(s_a, 4)) return BITNET_ERR_INVALID_ARG;
    if (M < 1 || M > 65535 * 1024 || H < 16 || H % 16) return BITNET_ERR_UNSUPPORTED_SHAPE;
    hipLaunchKernelGGL(quant_act_kernel<2>, dim3(M), dim3(256), 0, stream, (const void *)y, H, q, s_a);
    return launched();
}

bitnet_status_t bitnet_w2a8_gemv(const uint8_t *packed, const float *scales, const int8_t *q, const float *s_a,
                                 float *y, int M, int N, int K, hipStream_t stream) {
    if (!packed || !scales || !q || !s_a || !y) return BITNET_ERR_INVALID_ARG;
    if (!aligned(packed, 16) || !aligned(scales, 16) || !aligned(q, 16) || !aligned(s_a, 4) || !aligned(y, 4))
        return BITNET_ERR_INVALID_ARG;
    if (!shape_ok(N, K) || M < 1 || M > kGemvMaxM) return BITNET_ERR_UNSUPPORTED_SHAPE;
    gemv_launch<false>(packed, scales, q, s_a, y, nullptr, M, N, K, stream);
    return launched();
}

bitnet_status_t bitnet_w2a8_gemm(const uint8_t *packed, const float *scales, const int8_t *q, const float *s_a,
                                 void *y, int ydt, int M, int N, int K, hipStream_t stream) {
    if (!packed || !scales || !q || !s_a || !y) return BITNET_ERR_INVALID_ARG;
    if (!aligned(packed, 16) || !aligned(scales, 16) || !aligned(q, 16) || !aligned(s_a, 4) || !aligned(y, 4))
        return BITNET_ERR_INVALID_ARG;
    if (ydt != BITNET_DT_BF16 && ydt != BITNET_DT_F32) return BITNET_ERR_INVALID_ARG;
    if (!shape_ok(N, K) || M < 1 || !gemm_grid_ok(M)) return BITNET_ERR_UNSUPPORTED_SHAPE;
    if (ydt == BITNET_DT_BF16) gemm_launch<0>(packed, scales, q, s_a, y, M, N, K, stream);
    else gemm_launch<1>(packed, scales, q, s_a, y, M, N, K, stream);
    return launched();
}

bitnet_status_t bitnet_w2a8_acc_i32(const uint8_t *packed, const int8_t *q, int32_t *acc, int M, int N, int K,
                                    hipStream_t stream) {
    if (!packed || !q || !acc || !aligned(packed, 16) || !aligned(q, 16) || !aligned(acc, 4))
        return BITNET_ERR_INVALID_ARG;
    if (!shape_ok(N, K) || M < 1 || !gemm_grid_ok(M)) return BITNET_ERR_UNSUPPORTED_SHAPE;
    if (M <= kGemvMaxM) gemv_launch<true>(packed, nullptr, q, nullptr, nullptr, acc, M, N, K, stream);
    else gemm_launch<2>(packed, nullptr, q, nullptr, acc, M, N, K, stream);
    return launched();
}

}  // extern "C"
