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

#include <atomic>
#include <cstdint>

#include "bitnet_w2a8.h"
#include "layout.h"

using namespace bitnet_layout;

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
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
// Activation sources.  XM 0: bf16 [M][K]; 1: fp32 [M][K]; 2: fp32 [M][2K]
// folded, h = lo + hi (one fp32 addition, the junction of a stacked chain).
// load8 reads values 8v .. 8v+7 of token m, widened exactly to fp32.
// ==========================================================================
// Activation modes XM: 0 bf16, 1 fp32, 2 fp32 [2K] folded as lo + hi, 3 fp32 [2K]
// gated as relu(lo)^2 * hi (the two junctions of a stacked decode chain).
// The raw 16-byte words behind 8 values (bf16: one, fp32: two, two-half fp32: four),
// so that loads can be issued early and converted only when their data is needed.
template <int XM>
struct Raw8 {
    uint4 u[XM == 0 ? 1 : (XM == 1 ? 2 : 4)];
};

template <int XM>
__device__ __forceinline__ Raw8<XM> load_raw8(const void *__restrict__ x, int m, int K, int v) {
    Raw8<XM> r;
    if constexpr (XM == 0) {
        r.u[0] = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(x) + (size_t)m * K)[v];
    } else if constexpr (XM == 1) {
        const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const float *>(x) + (size_t)m * K) + 2 * v;
        r.u[0] = p[0];
        r.u[1] = p[1];
    } else {
        const float *row = static_cast<const float *>(x) + (size_t)m * 2 * K;
        const uint4 *lo = reinterpret_cast<const uint4 *>(row) + 2 * v;
        const uint4 *hi = reinterpret_cast<const uint4 *>(row + K) + 2 * v;
        r.u[0] = lo[0];
        r.u[1] = lo[1];
        r.u[2] = hi[0];
        r.u[3] = hi[1];
    }
    return r;
}

__device__ __forceinline__ void words8(const uint4 &a, const uint4 &b, uint32_t w[8]) {
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
}

template <int XM>
__device__ __forceinline__ void cvt8(const Raw8<XM> &r, float out[8]) {
    if constexpr (XM == 0) {
        const uint32_t w[4] = {r.u[0].x, r.u[0].y, r.u[0].z, r.u[0].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[2 * i] = __uint_as_float(w[i] << 16);
            out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    } else {
        uint32_t w[8];
        words8(r.u[0], r.u[1], w);
#pragma unroll
        for (int i = 0; i < 8; ++i) out[i] = __uint_as_float(w[i]);
        if constexpr (XM == 2) {  // linear junction: lo + hi
            uint32_t h[8];
            words8(r.u[2], r.u[3], h);
#pragma unroll
            for (int i = 0; i < 8; ++i) out[i] = __fadd_rn(out[i], __uint_as_float(h[i]));
        } else if constexpr (XM == 3) {  // squared-ReLU gate: (max(lo, 0)^2) * hi, two fp32 roundings
            uint32_t h[8];
            words8(r.u[2], r.u[3], h);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float g = out[i] > 0.0f ? out[i] : 0.0f;
                out[i] = __fmul_rn(__fmul_rn(g, g), __uint_as_float(h[i]));
            }
        }
    }
}

template <int XM>
__device__ __forceinline__ void load8(const void *__restrict__ x, int m, int K, int v, float out[8]) {
    cvt8<XM>(load_raw8<XM>(x, m, K, v), out);
}

__device__ __forceinline__ float max_abs8(const float f[8], float m) {
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(f[i]));
    return m;
}

// q = clamp(rint(x * inv), -127, 127) for 8 values, packed little-endian.
// The clamp never acts, so it is not executed: every x quantised has |x| <= amax_c
// (amax is the exact maximum of the same fp32 values) and inv = 127 / amax_c is
// correctly rounded, so |x * inv| <= 127 (1 + 2^-24)^2 rounds to at most 127 +
// 2^-17 and rint gives at most 127 (8 fewer VALU operations per 8 values, which
// the fused forms execute before requesting their weights: 20480x3200 step
// 6.66 -> 6.39 us).
// Rounding by one fp32 add: for |v| < 2^22, v + 1.5 * 2^23 lies in [2^23, 2^24),
// where the spacing of floats is 1, so the add rounds v to an integer, half to
// even (1.5 * 2^23 is even), and the sum's low mantissa byte is that integer in
// two's complement.  v_perm gathers four such bytes per word.  The product is
// rounded to fp32 first (no contraction into one fused multiply-add, whose single
// rounding would decide ties of the exact product instead).  Checked against
// rint on every fp32 value of magnitude below 127.5; it saves the rint and the
// int conversion (fused 13824x2560 step 4.79 -> 4.73 us, 8 tokens 13.4 -> 12.9).
__device__ __forceinline__ uint2 quantize8(const float f[8], float inv) {
#pragma clang fp contract(off)
    uint32_t u[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float v = f[i] * inv;
        u[i] = __float_as_uint(v + 12582912.0f);
    }
    // perm(hi, lo, sel): selector bytes 0-3 take bytes of lo, 4-7 of hi, 0x0c gives zero
    const uint32_t w0 = __builtin_amdgcn_perm(u[1], u[0], 0x0c0c0400u) | __builtin_amdgcn_perm(u[3], u[2], 0x04000c0cu);
    const uint32_t w1 = __builtin_amdgcn_perm(u[5], u[4], 0x0c0c0400u) | __builtin_amdgcn_perm(u[7], u[6], 0x04000c0cu);
    return make_uint2(w0, w1);
}

// Max over the 64 lanes of a wave of non-negative floats (absolute values), with
// DPP row operations on their bit patterns: for non-negative floats the unsigned
// integer order is the float order, and an integer max needs no NaN
// canonicalisation; with 0 (the identity of the unsigned max) for lanes a
// broadcast does not reach, each step is one max with a DPP operand.  Max is
// idempotent, so mirrored / broadcast partners may repeat: after the row steps
// every lane of a 16-lane row holds the row max, the two broadcasts fold rows
// 0..3 into lane 63, which is then read as a scalar.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ float wave_max(float v) {
    uint32_t u = __float_as_uint(v);
    u = max(u, dpp_u<0xB1>(u));   // quad_perm [1,0,3,2]
    u = max(u, dpp_u<0x4E>(u));   // quad_perm [2,3,0,1]
    u = max(u, dpp_u<0x141>(u));  // row_half_mirror
    u = max(u, dpp_u<0x140>(u));  // row_mirror
    u = max(u, dpp_u<0x142>(u));  // row_bcast:15
    u = max(u, dpp_u<0x143>(u));  // row_bcast:31
    return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)u, 63));
}

// Workgroup barrier that waits only for this wave's LDS traffic: global loads
// issued earlier stay in flight across it (a full __syncthreads() fence would
// also drain them).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ==========================================================================
// a4: per-token absmax int8 quantisation ([P2] "Architecture foundations":
// 8-bit activations).  One 256-thread workgroup per token.  CPT > 0: each
// thread keeps its CPT chunks of 8 values in registers (one read of the
// token); CPT == 0: two passes over the token (any K).
// amax is exact and independent of the reduction order; inv = 127/amax_c is
// a correctly rounded division; the product x*inv is one fp32 multiply.
// ==========================================================================
template <int XM, int CPT>
__global__ __launch_bounds__(256) void quant_act_kernel(const void *__restrict__ x, int K,
                                                         int8_t *__restrict__ q, float *__restrict__ s_a) {
    __shared__ float part[4];
    const int m = blockIdx.x;
    const int nvec = K >> 3;
    constexpr int C = CPT > 0 ? CPT : 1;
    float f[C][8];
    float amax = 0.0f;
    if (CPT > 0) {
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int v = threadIdx.x + 256 * c;
            if (v < nvec) {
                load8<XM>(x, m, K, v, f[c]);
                amax = max_abs8(f[c], amax);
            }
        }
    } else {
        for (int v = threadIdx.x; v < nvec; v += 256) {
            load8<XM>(x, m, K, v, f[0]);
            amax = max_abs8(f[0], amax);
        }
    }
    amax = wave_max(amax);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
    const float amax_c = fmaxf(amax, 1e-5f);
    const float inv = __fdiv_rn(127.0f, amax_c);
    uint2 *qrow = reinterpret_cast<uint2 *>(q + (size_t)m * K);
    if (CPT > 0) {
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int v = threadIdx.x + 256 * c;
            if (v < nvec) qrow[v] = quantize8(f[c], inv);
        }
    } else {
        for (int v = threadIdx.x; v < nvec; v += 256) {
            load8<XM>(x, m, K, v, f[0]);
            qrow[v] = quantize8(f[0], inv);
        }
    }
    if (threadIdx.x == 0) s_a[m] = __fdiv_rn(amax_c, 127.0f);
}

// ==========================================================================
// a5: decode product, M <= 16.  One workgroup per 16-row tile; its nwc
// compute waves split the K blocks (split-K), wave w owning blocks
// [w*per, w*per + per).  Every lane issues all its weight and scale loads for
// a chunk of NB blocks before the first matrix-core step (NB x 8 bytes per
// lane of the weight stream in flight per wave).  Partial sums are reduced
// through LDS in wave order, so results are deterministic.
//
// AM = -1: activations arrive quantised (int8 q, fp32 s_a).
// AM = 0..3 (XM of load8): fused quantisation by QW extra "quant waves"
// (waves nwc .. nwc+QW-1), token-parallel: quant wave qw handles tokens
// qw, qw+QW, ...; it reads the token (pass 1: amax), re-reads it (pass 2:
// quantise, same arithmetic as quant_act_kernel) and writes int8 into an LDS
// copy of q.  The compute waves meanwhile have their weight loads in flight;
// they wait at an LDS-only barrier (vmcnt is not drained), then read their
// matrix-core operands from the LDS copy.  Every workgroup derives bit-
// identical q and s_a, so the result equals quant-then-product.  Workgroup 0
// optionally writes q and s_a out.
// TOK = token capacity (1, 2, 4, 8, 16) of the instantiation, M <= TOK.  Lane
// (g, j) drains elements e < MW = min(TOK, 4) (tokens 4g + e): with M <= 4 only
// tokens 0..M-1 (lanes 0..15, elements < M) carry data.
// ==========================================================================
struct GemvArgs {
    const uint8_t *packed;
    const float *scales;
    const void *act;      // int8 q [M][K] (AM -1) or the unquantised activations
    const float *s_a;     // AM -1 only
    float *y;
    int32_t *acc;
    int8_t *q_out;        // optional (fused modes)
    float *s_a_out;       // optional (fused modes)
    int M, N, K, per, nwc, qw;
};

// LDS of the fused forms: [int8 copy of q, M*K bytes padded | reduction reuse]
// then 16 fp32 dequant factors.
// Row stride of the LDS copy of q: K plus 16 bytes, so that the token rows read
// together by one matrix-core operand load start 4 banks apart (K is a multiple
// of 128 bytes and would put every row on the same banks).
__host__ __device__ inline int lds_qstride(int K) { return K + 16; }

__host__ __device__ inline size_t gemv_fused_region(int M, int K, int nwc) {
    const size_t qbytes = (size_t)M * lds_qstride(K);
    const size_t red = (size_t)nwc * 4 * 64 * sizeof(int);
    return qbytes > red ? qbytes : red;
}

template <int XM>
__device__ void quant_wave(const GemvArgs &args, int8_t *qs, float *sa_lds, int qw, int l) {
    const int M = args.M, K = args.K, nvec = K >> 3;
    for (int m = qw; m < M; m += args.qw) {
        float mx = 0.0f;
        for (int c0 = 0; c0 < nvec; c0 += 4 * kWave) {
            float f[4][8];
#pragma unroll
            for (int u = 0; u < 4; ++u)  // unconditional (clamped) loads: all four in flight together
                load8<XM>(args.act, m, K, min(c0 + u * kWave + l, nvec - 1), f[u]);
#pragma unroll
            for (int u = 0; u < 4; ++u) mx = max_abs8(f[u], mx);  // a clamped repeat cannot change the max
        }
        const float amax_c = fmaxf(wave_max(mx), 1e-5f);
        const float inv = __fdiv_rn(127.0f, amax_c);
        for (int c0 = 0; c0 < nvec; c0 += 4 * kWave) {
            float f[4][8];
#pragma unroll
            for (int u = 0; u < 4; ++u) load8<XM>(args.act, m, K, min(c0 + u * kWave + l, nvec - 1), f[u]);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int c = c0 + u * kWave + l;
                if (c < nvec) {
                    const uint2 qv = quantize8(f[u], inv);
                    *reinterpret_cast<uint2 *>(qs + (size_t)m * lds_qstride(K) + 8 * c) = qv;
                    if (args.q_out && blockIdx.x == 0)
                        *reinterpret_cast<uint2 *>(args.q_out + (size_t)m * K + 8 * c) = qv;
                }
            }
        }
        const float sa = __fdiv_rn(amax_c, 127.0f);
        if (l == 0) {
            sa_lds[m] = sa;
            if (args.s_a_out && blockIdx.x == 0) args.s_a_out[m] = sa;
        }
    }
}

// Kernel forms.
enum GemvForm {
    kDirect = 0,    // int8 q from global memory, one chunk of blocks per wave
    kMulti = 1,     // as kDirect with a loop over chunks (K beyond 12 x 8 blocks)
    kStaged = 2,    // int8 q slice fetched with a few coalesced loads into LDS (when it fits)
    kAllWaves = 3,  // fused quantisation, every compute wave quantises its own K-slice (M <= 4)
    kQuantWaves = 4, // fused quantisation by 4 extra quant waves (4 < M <= 16)
    kAllWavesXF = 5  // as kAllWaves, quantising before the weights are requested
};

template <int AM, int NB, int TOK, bool INT_OUT, int FORM, int SG>
__global__ __launch_bounds__(1024) void gemv_kernel(GemvArgs args) {
    constexpr int MW = TOK < 4 ? TOK : 4;  // accumulator elements drained per lane
    constexpr bool IACC = INT_OUT || SG == 0;  // integer sums over the wave's whole K-slice
    extern __shared__ __align__(16) unsigned char smem[];
    const int M = args.M, N = args.N, K = args.K, per = args.per, nwc = args.nwc;
    const int nblk = K >> 7;
    const int tile = blockIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform (scalar) index
    const int l = threadIdx.x & 63, g = l >> 4, j = l & 15;
    constexpr int NE = INT_OUT ? 4 : MW;
    constexpr bool FUSED = AM >= 0;
    constexpr bool ALLW = FORM == kAllWaves || FORM == kAllWavesXF;  // every wave quantises its slice
    constexpr bool LDSQ = FORM == kStaged || ALLW || FORM == kQuantWaves;  // operands via LDS
    constexpr int XM = AM < 0 ? 0 : AM;
    int *red = reinterpret_cast<int *>(smem);
    int8_t *qs = reinterpret_cast<int8_t *>(smem);
    // LDS forms: after the q region, 16 dequant factors then [4 tokens][12 waves] partial amax
    float *tail = reinterpret_cast<float *>(smem + (LDSQ ? gemv_fused_region(M, K, nwc) : 0));

    if (FORM == kQuantWaves && w >= nwc) {
        quant_wave<XM>(args, qs, tail, w - nwc, l);
        lds_barrier();  // q ready
        lds_barrier();  // operands consumed
        lds_barrier();  // partial sums written
        return;
    }

    const int bw0 = w * per;
    const int bw1 = min(nblk, bw0 + per);
    const int nbw = bw1 - bw0;
    const bool tok = j < M;

    // vmcnt retires loads in issue order: whatever is needed before the
    // weights arrive (activations to quantise or stage) is issued before them.
    // token scale of the output this lane stores (token l/4, see the epilogue)
    const float sa_tok = (!FUSED && !INT_OUT) ? args.s_a[min(l >> 2, M - 1)] : 0.0f;
    const float s_w = (SG == 0 && !INT_OUT) ? args.scales[0] : 0.0f;  // the one weight scale
    // kAllWaves: this wave's K-slice of every token, raw, 8 values per chunk
    constexpr int CR = (NB + 3) / 4;
    Raw8<XM> xr[ALLW ? MW : 1][ALLW ? CR : 1];
    const int nchw = nbw * 16;
    if (ALLW) {
#pragma unroll
        for (int m = 0; m < (ALLW ? MW : 1); ++m)
#pragma unroll
            for (int r = 0; r < (ALLW ? CR : 1); ++r)
                xr[m][r] = load_raw8<XM>(args.act, min(m, M - 1), K, bw0 * 16 + min(l + kWave * r, nchw - 1));
    }
    // kStaged: this wave's K-slice of q for M <= TOK tokens in 16-byte chunks
    constexpr int QR = (TOK * NB + 7) / 8;
    v4i qraw[FORM == kStaged ? QR : 1];  // native vector: a register value, not an aggregate
    const int qper = nbw * 8;  // chunks per token
    if (FORM == kStaged) {
        const int8_t *q = static_cast<const int8_t *>(args.act);
#pragma unroll
        for (int r = 0; r < (FORM == kStaged ? QR : 1); ++r) {
            const int c = min(l + kWave * r, M * qper - 1);
            const int m = c / qper, o = c - m * qper;
            qraw[r] = *reinterpret_cast<const v4i *>(q + (size_t)m * K + (size_t)bw0 * kBlockK + 16 * o);
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    float yacc[MW];
    int iacc[4];
#pragma unroll
    for (int e = 0; e < MW; ++e) yacc[e] = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) iacc[e] = 0;

    const int8_t *qsrc = LDSQ ? qs : static_cast<const int8_t *>(args.act);

    // One chunk of up to NB blocks: all its loads, then its matrix-core steps.
    auto chunk = [&](const int c0) {
        const int nb = min(NB, bw1 - c0);
        const uint8_t *wp = args.packed + ((size_t)tile * nblk + c0) * kBrickBytes + l * 8;
        // scales: SG 128 [tile][block][16 rows]; SG 64 [tile][block][16 rows][2 halves]
        const float *sp = args.scales + (((size_t)tile * nblk + c0) * kTileN + j) * (SG == 64 ? 2 : 1);
        uint2 wv[NB];
        float2 sc[NB];
        // Weights and block scales are read exactly once per launch: non-temporal loads
        // (streaming hint) leave the caches to the activations every workgroup re-reads
        // (13824x2560 product 4.45 -> 4.19 us, 2560x2560 2.98 -> 2.66 us).
        auto load_weights = [&]() {
#pragma unroll
            for (int i = 0; i < NB; ++i) {  // unconditional (clamped) loads, issued back to back
                const int bi = min(i, nb - 1);
                const v2u w2 = __builtin_nontemporal_load(reinterpret_cast<const v2u *>(wp + bi * kBrickBytes));
                wv[i] = make_uint2(w2.x, w2.y);
                if (!INT_OUT && SG == 128) sc[i].x = __builtin_nontemporal_load(sp + bi * kTileN);
                if (!INT_OUT && SG == 64) {
                    const v2f s2 = __builtin_nontemporal_load(reinterpret_cast<const v2f *>(sp + bi * 2 * kTileN));
                    sc[i] = make_float2(s2.x, s2.y);
                }
            }
        };
        if constexpr (ALLW) {
            // each wave quantises its own K-slice of every token; one LDS exchange gives the
            // per-token amax.  No barrier after: each wave reads back only the slice it wrote.
            auto quantise_slices = [&]() {
                float *amax_part = tail + 16;
                float xf[MW][CR][8];
#pragma unroll
                for (int m = 0; m < MW; ++m)
#pragma unroll
                    for (int r = 0; r < CR; ++r) cvt8<XM>(xr[m][r], xf[m][r]);
#pragma unroll
                for (int m = 0; m < MW; ++m) {
                    float mx = 0.0f;
#pragma unroll
                    for (int r = 0; r < CR; ++r)
                        if (l + kWave * r < nchw) mx = max_abs8(xf[m][r], mx);
                    mx = wave_max(mx);
                    if (l == 0) amax_part[m * 12 + w] = mx;
                    if (w == 0 && l >= nwc && l < 12) amax_part[m * 12 + l] = 0.0f;  // slots of no wave
                }
                lds_barrier();
#pragma unroll
                for (int m = 0; m < MW; ++m) {
                    if (m >= M) break;
                    float am = 0.0f;
                    {  // the 12 wave slots of token m in one round trip (non-negative: integer max)
                        const v4i *pv = reinterpret_cast<const v4i *>(amax_part + m * 12);
                        const v4i p0 = pv[0], p1 = pv[1], p2 = pv[2];
                        uint32_t u = 0;
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            u = max(u, max(max((uint32_t)p0[e], (uint32_t)p1[e]), (uint32_t)p2[e]));
                        am = __uint_as_float(u);
                    }
                    const float amax_c = fmaxf(am, 1e-5f);
                    const float inv = __fdiv_rn(127.0f, amax_c);
#pragma unroll
                    for (int r = 0; r < CR; ++r) {
                        const int c = l + kWave * r;
                        if (c < nchw) {
                            const uint2 qv = quantize8(xf[m][r], inv);
                            const size_t off = (size_t)bw0 * kBlockK + 8 * c;
                            *reinterpret_cast<uint2 *>(qs + (size_t)m * lds_qstride(K) + off) = qv;
                            if (args.q_out && blockIdx.x == 0)
                                *reinterpret_cast<uint2 *>(args.q_out + (size_t)m * K + off) = qv;
                        }
                    }
                    if (w == 0 && l == 0) {
                        const float sa = __fdiv_rn(amax_c, 127.0f);
                        tail[m] = sa;
                        if (args.s_a_out && blockIdx.x == 0) args.s_a_out[m] = sa;
                    }
                }
            };
            // The activations were requested before the weights.  When several workgroups
            // share each CU and all fit at once, the weight requests of the whole grid delay
            // that small read and the quantisation lands behind the weight stream; there
            // (kAllWavesXF) the wave quantises first and requests its weights after.
            if constexpr (FORM == kAllWavesXF) {
                quantise_slices();
                __builtin_amdgcn_sched_barrier(0);
                load_weights();
            } else {
                load_weights();
                __builtin_amdgcn_sched_barrier(0);
                quantise_slices();
            }
        } else {
            load_weights();
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (FORM == kStaged) {
#pragma unroll
                for (int r = 0; r < QR; ++r) {
                    const int c = l + kWave * r;
                    if (c < M * qper) {
                        const int m = c / qper, o = c - m * qper;
                        *reinterpret_cast<v4i *>(qs + (size_t)m * lds_qstride(K) + (size_t)bw0 * kBlockK + 16 * o) = qraw[r];
                    }
                }
                // the wave reads back only its own slice: LDS keeps one wave's accesses in order
            } else if constexpr (FORM == kQuantWaves) {
                lds_barrier();  // q ready (written by the quant waves)
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        const int8_t *qp = qsrc + (size_t)j * (LDSQ ? lds_qstride(K) : K) + (size_t)c0 * kBlockK + g * 16;
        v4i a[NB][2];
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
            for (int s = 0; s < 2; ++s) a[i][s] = v4i{0, 0, 0, 0};
        if (tok) {  // only lanes of real tokens fetch operands (padding lanes stay zero)
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const int bi = min(i, nb - 1);
#pragma unroll
                for (int s = 0; s < 2; ++s) a[i][s] = *reinterpret_cast<const v4i *>(qp + bi * kBlockK + s * 64);
            }
        }
        __builtin_amdgcn_sched_barrier(0);  // keep every load above the first matrix-core step
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            if (i < nb) {
                if constexpr (SG == 64 && !INT_OUT) {  // one scale per matrix-core step (64 weights)
                    const v4i c0 = mfma_i8(a[i][0], decode16(wv[i].x), v4i{0, 0, 0, 0});
#pragma unroll
                    for (int e = 0; e < MW; ++e) yacc[e] = fmaf(sc[i].x, (float)c0[e], yacc[e]);
                    const v4i c1 = mfma_i8(a[i][1], decode16(wv[i].y), v4i{0, 0, 0, 0});
#pragma unroll
                    for (int e = 0; e < MW; ++e) yacc[e] = fmaf(sc[i].y, (float)c1[e], yacc[e]);
                } else {
                    v4i c = v4i{0, 0, 0, 0};
                    c = mfma_i8(a[i][0], decode16(wv[i].x), c);
                    c = mfma_i8(a[i][1], decode16(wv[i].y), c);
                    if (IACC) {
#pragma unroll
                        for (int e = 0; e < NE; ++e) iacc[e] += c[e];
                    } else {
#pragma unroll
                        for (int e = 0; e < MW; ++e) yacc[e] = fmaf(sc[i].x, (float)c[e], yacc[e]);
                    }
                }
            }
        }
    };
    // Straight-line for a single chunk; the chunk loop is a separate form,
    // because a loop makes the wait-count pass drain the early loads at its header.
    if constexpr (FORM == kMulti) {
        for (int c0 = bw0; c0 < bw1; c0 += NB) chunk(c0);
    } else {
        chunk(bw0);
    }

    if (LDSQ) lds_barrier();  // the reduction buffer overlaps the LDS copy of q
#pragma unroll
    for (int e = 0; e < NE; ++e) red[(w * 4 + e) * kWave + l] = IACC ? iacc[e] : __float_as_int(yacc[e]);
    if (LDSQ) lds_barrier();
    else __syncthreads();
    // Wave 0 sums the waves' partials (in wave order) and stores.  One token: lanes
    // 0..15 each store row j.  More tokens: lane l takes token mt = l/4 and rows
    // 4(l%4)..4(l%4)+3 of the tile (element mt%4 of lanes 16(mt/4) + r), so each stored
    // token row leaves as 16-byte pieces, one store instruction per workgroup (four
    // 4-byte stores per lane cost ~0.8 us more at 8 tokens; for one token the 16-lane
    // form is ~0.1 us faster).
    if (TOK == 1 && w == 0) {
        if (g == 0) {
            const size_t o = (size_t)tile * kTileN + j;
            if (INT_OUT || SG == 0) {
                int sum = 0;
                for (int ww = 0; ww < nwc; ++ww) sum += red[ww * 4 * kWave + l];
                if (INT_OUT) args.acc[o] = sum >> 6;  // exact: sum is 64 * integer
                else args.y[o] = (float)(sum >> 6) * ((FUSED ? tail[0] : sa_tok) * s_w);
            } else {
                float sum = 0.0f;
                for (int ww = 0; ww < nwc; ++ww) sum += __int_as_float(red[ww * 4 * kWave + l]);
                args.y[o] = sum * ((FUSED ? tail[0] : sa_tok) * 0.015625f);
            }
        }
    } else if (w == 0) {
        const int mt = l >> 2, r4 = (l & 3) * 4;
        const int src = (mt & 3) * kWave + 16 * (mt >> 2) + r4;
        if (mt < M) {
            const size_t o = (size_t)mt * N + (size_t)tile * kTileN + r4;
            if (INT_OUT || SG == 0) {
                int sum[4] = {0, 0, 0, 0};
                for (int ww = 0; ww < nwc; ++ww)
#pragma unroll
                    for (int r = 0; r < 4; ++r) sum[r] += red[ww * 4 * kWave + src + r];
                if (INT_OUT) {  // exact: each sum is 64 * integer
                    *reinterpret_cast<int4 *>(args.acc + o) =
                        make_int4(sum[0] >> 6, sum[1] >> 6, sum[2] >> 6, sum[3] >> 6);
                } else {  // exact integer product, then the two scales
                    const float f = (FUSED ? tail[mt] : sa_tok) * s_w;
                    *reinterpret_cast<float4 *>(args.y + o) =
                        make_float4((float)(sum[0] >> 6) * f, (float)(sum[1] >> 6) * f, (float)(sum[2] >> 6) * f,
                                    (float)(sum[3] >> 6) * f);
                }
            } else {
                float sum[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                for (int ww = 0; ww < nwc; ++ww)
#pragma unroll
                    for (int r = 0; r < 4; ++r) sum[r] += __int_as_float(red[ww * 4 * kWave + src + r]);
                const float f = (FUSED ? tail[mt] : sa_tok) * 0.015625f;
                *reinterpret_cast<float4 *>(args.y + o) = make_float4(sum[0] * f, sum[1] * f, sum[2] * f, sum[3] * f);
            }
        }
    }
}

// ==========================================================================
// a6: prefill product, any M.  A 512-thread workgroup owns a 128-token x
// 64*RT-row output tile (RT = 4 normally; 2 or 1 when few tokens would leave
// the chip short of workgroups); wave (wm, wn) = (w / 4, w % 4) owns 64 tokens
// x 16*RT rows = 4 x RT matrix-core tiles.  Per 128-weight block the workgroup
// stages the block's activations (128 x 128 int8, rows padded to 144 bytes so
// the operand reads are conflict-free), its 4*RT packed bricks and their
// scales in LDS with two or three coalesced 16-byte loads per thread; the
// next block's loads are in flight while the current block computes (double
// buffer, one barrier per block).  Each wave decodes its RT row-tiles once per
// block and reuses them for its 4 token-tiles, then drains the int32 tiles
// into fp32 with the block scales.  Workgroups are
// ordered so that the token tiles sharing a weight tile run on one XCD (one
// L2) when the grid divides evenly over the 8 XCDs.
// ==========================================================================
// Empty asm that takes a value in and out of a VGPR: an ordering point that
// pure arithmetic (matrix-core steps, the fp32 drain) cannot be moved across.
__device__ __forceinline__ void keep(float &x) { asm volatile("" : "+v"(x)); }

constexpr int kGemmBM = 128, kGemmThreads = 512;
constexpr int kAStride = 144;                        // padded LDS row of the activation tile
constexpr int kAStage = kGemmBM * kAStride;          // 18432 bytes
constexpr int kBStage = 16 * 512;                    // 8192 bytes: up to 16 bricks
constexpr int kSStage = 16 * 16 * 4;                 // 1024 bytes: [16 tiles][16 rows] fp32 (x2 for 64-blocks)

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// OUT: 0 bf16 y, 1 fp32 y, 2 int32 acc.  SG: scale granularity, 128 or 64
// weights per scale (scales staged per block: [tile][16 rows] or
// [tile][16 rows][2 halves]) or 0 (one scale: integer sums over all of K,
// scaled once in the epilogue).
// KS (RT <= 2, SG 128 or 0): 64-token tiles, each pipeline stage carrying two
// blocks: LDS rows 0..63 of the activation tile and the first 4*RT brick and
// scale slots hold the even block, rows 64..127 and the next 4*RT slots the odd
// one.  Waves wm = 0 sum the even blocks, wm = 1 the odd ones; the two partial
// sums are added once, through LDS, before the epilogue (a fixed order, so
// results are deterministic).  Half the blocks per workgroup and twice the
// workgroups of the 128-token tiles, at twice the weight decoding.
template <int OUT, int SG, int RT, bool KS = false>
__global__ __launch_bounds__(kGemmThreads) void gemm_kernel(const uint8_t *__restrict__ packed,
                                                             const float *__restrict__ scales,
                                                             const int8_t *__restrict__ q,
                                                             const float *__restrict__ s_a, void *__restrict__ yout,
                                                             int M, int N, int K, int ntm) {
    constexpr bool BLOCKED = OUT != 2 && SG != 0;     // per-block fp32 drain with block scales
    constexpr int SPT = SG == 64 ? 2 : 1;             // scales per row and 128-block
    constexpr int SST = BLOCKED ? kSStage * SPT : 0;  // staged scale bytes per block
    constexpr int STAGE = kAStage + kBStage + SST;
    static_assert(!KS || (RT <= 2 && SG != 64), "two-block stages: up to 2 row tiles, one scale per block");
    __shared__ __align__(16) unsigned char lds[2 * STAGE];
    const int G = gridDim.x;
    int t = blockIdx.x;
    if ((G & 7) == 0) t = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);  // XCD-aware order
    const int tm = t % ntm, tn = t / ntm;
    const int m0 = tm * (KS ? 64 : kGemmBM), T0 = tn * (4 * RT);  // RT row tiles per wave, 4 waves across
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63, g = l >> 4, j = l & 15;
    const int wm = w >> 2, wn = w & 3;
    const int nblk = K >> 7, ntile_n = N >> 4;
    const int nst = KS ? (nblk + 1) >> 1 : nblk;  // pipeline stages (KS: two blocks each)
    constexpr int NSLOT = (KS ? 2 : 1) * 4 * RT;  // brick / scale tile slots per stage

    // staging assignment (global -> registers -> LDS); KS: the second half of the
    // activation rows and of the slots carries the stage's odd block
    int arow[2], acol[2], ahalf[2];
    const int8_t *aptr[2];
    bool aok[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int c = tid + kGemmThreads * r;
        arow[r] = c >> 3;
        acol[r] = (c & 7) * 16;
        ahalf[r] = KS ? arow[r] >> 6 : 0;
        const int tok = m0 + (KS ? arow[r] & 63 : arow[r]);
        aok[r] = tok < M;
        aptr[r] = q + (size_t)(aok[r] ? tok : 0) * K + acol[r];
    }
    const int bslot = min(tid >> 5, NSLOT - 1);  // threads past the stage's bricks repeat the last
    const int bhalf = bslot / (4 * RT);
    const int bT = T0 + bslot % (4 * RT);
    const bool bok = bT < ntile_n;
    const uint8_t *bptr = packed + (size_t)(bok ? bT : 0) * nblk * kBrickBytes + (tid & 31) * 16;
    // scale staging: 64 (SG 128) or 128 (SG 64) threads, one float4 each per block
    constexpr int SCT = 4 * SPT;  // staging threads per tile
    // threads past the 4*RT tiles' scales repeat the last tile's (not stored)
    const int sslot = min(tid / SCT, NSLOT - 1);
    const int shalf = sslot / (4 * RT);
    const int sT = T0 + sslot % (4 * RT);
    const bool sok = BLOCKED && sT < ntile_n;
    const float *sptr = scales + (size_t)(sok ? sT : 0) * nblk * kTileN * SPT + (tid % SCT) * 4;

    // Two register sets of staged data: the loads of block b+2 are issued while
    // block b computes and block b+1's data (issued one iteration earlier) is
    // stored to LDS after it, so each block's load latency is covered by a
    // full iteration plus a barrier.
    struct Staged {  // native vectors: register values, not aggregates
        v4i a[2];
        v4i b;
        v4f s;
    };
    // Unconditional loads from clamped addresses (rows past M or N read row 0 /
    // tile 0, whose products land in outputs that are never stored): branch-free
    // issue lets the wait counters track each block's loads exactly, so the
    // store of block b+1 does not wait for the prefetch of block b+2.
    auto gload = [&](int b, Staged &r) {  // b: pipeline stage
        b = min(b, nst - 1);
        auto blk = [&](int half) { return KS ? min(2 * b + half, nblk - 1) : b; };
#pragma unroll
        for (int i = 0; i < 2; ++i)
            r.a[i] = *reinterpret_cast<const v4i *>(aptr[i] + (size_t)blk(ahalf[i]) * kBlockK);
        r.b = *reinterpret_cast<const v4i *>(bptr + (size_t)blk(bhalf) * kBrickBytes);
        if (BLOCKED) r.s = *reinterpret_cast<const v4f *>(sptr + (size_t)blk(shalf) * kTileN * SPT);
    };
    auto lstore = [&](int st, const Staged &r) {
        unsigned char *base = lds + st * STAGE;
#pragma unroll
        for (int i = 0; i < 2; ++i) *reinterpret_cast<v4i *>(base + arow[i] * kAStride + acol[i]) = r.a[i];
        if (tid < 32 * NSLOT) *reinterpret_cast<v4i *>(base + kAStage + tid * 16) = r.b;
        // LDS scales: [half][16 tiles][16 rows]; global SG 64 order is [tile][row][half]
        if (BLOCKED && tid < NSLOT * SCT) {
            float *sb = reinterpret_cast<float *>(base + kAStage + kBStage);
            if constexpr (SG == 128) {
                *reinterpret_cast<v4f *>(sb + 4 * tid) = r.s;
            } else {  // r.s = rows 2i, 2i+1 of tile tid/8, each (half 0, half 1)
                const int tile = tid >> 3, i = tid & 7;
                *reinterpret_cast<float2 *>(sb + tile * 16 + 2 * i) = make_float2(r.s.x, r.s.z);
                *reinterpret_cast<float2 *>(sb + 256 + tile * 16 + 2 * i) = make_float2(r.s.y, r.s.w);
            }
        }
    };

    float yacc[4][RT][4];
    v4i iacc[4][RT];  // unscaled paths: the matrix core accumulates over all of K
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < RT; ++b) {
            iacc[a][b] = v4i{0, 0, 0, 0};
#pragma unroll
            for (int e = 0; e < 4; ++e) yacc[a][b][e] = 0.0f;
        }

    // Operands of one block: activation fragments of the wave's 4 token tiles and
    // the decoded weights of its RT row tiles (matrix-core A = weights (rows),
    // B = activations (tokens): lane (g, j) receives rows 4g..4g+3 of token j).
    auto operands = [&](int st, v4i (&ao)[4][2], v4i (&bw)[RT][2]) {
        const unsigned char *base = lds + st * STAGE;
#pragma unroll
        for (int ti = 0; ti < 4; ++ti)
#pragma unroll
            for (int s = 0; s < 2; ++s)
                ao[ti][s] = *reinterpret_cast<const v4i *>(base + (64 * wm + 16 * ti + j) * kAStride + 64 * s + 16 * g);
#pragma unroll
        for (int tj = 0; tj < RT; ++tj) {
            const int slot = (KS ? 4 * RT * wm : 0) + RT * wn + tj;
            const uint2 wv = *reinterpret_cast<const uint2 *>(base + kAStage + slot * 512 + l * 8);
            bw[tj][0] = decode16(wv.x);
            bw[tj][1] = decode16(wv.y);
        }
    };
    // scales of rows 4g..4g+3 of the wave's RT row tiles, for half h
    auto load_sc = [&](int st, int h, float (&sc)[RT][4]) {
        const unsigned char *base = lds + st * STAGE;
#pragma unroll
        for (int tj = 0; tj < RT; ++tj) {
            const int slot = (KS ? 4 * RT * wm : 0) + RT * wn + tj;
            const float4 s4 = *reinterpret_cast<const float4 *>(base + kAStage + kBStage + h * 1024 +
                                                                (slot * 16 + 4 * g) * 4);
            sc[tj][0] = s4.x;
            sc[tj][1] = s4.y;
            sc[tj][2] = s4.z;
            sc[tj][3] = s4.w;
        }
    };
    // the 4 x RT tiles' first K-steps are independent and pipeline on the matrix
    // core; the second K-steps then find their accumulators long finished
    auto mma = [&](const v4i (&ao)[4][2], const v4i (&bw)[RT][2], v4i (&c)[4][RT], bool from_zero) {
#pragma unroll
        for (int ti = 0; ti < 4; ++ti)
#pragma unroll
            for (int tj = 0; tj < RT; ++tj)
                c[ti][tj] = mfma_i8(bw[tj][0], ao[ti][0], from_zero ? v4i{0, 0, 0, 0} : c[ti][tj]);
#pragma unroll
        for (int ti = 0; ti < 4; ++ti)
#pragma unroll
            for (int tj = 0; tj < RT; ++tj) c[ti][tj] = mfma_i8(bw[tj][1], ao[ti][1], c[ti][tj]);
    };
    auto drain = [&](const v4i (&c)[4][RT], const float (&sc)[RT][4]) {
#pragma unroll
        for (int ti = 0; ti < 4; ++ti)
#pragma unroll
            for (int tj = 0; tj < RT; ++tj)
#pragma unroll
                for (int e = 0; e < 4; ++e) yacc[ti][tj][e] = fmaf(sc[tj][e], (float)c[ti][tj][e], yacc[ti][tj][e]);
    };

    v4i cl[4][RT];
    float scl[RT][4];

    auto compute = [&](int st) {
        v4i ao[4][2], bw[RT][2];
        if constexpr (SG == 64 && BLOCKED) {
            // one scale per matrix-core step (64 weights): each half's 16 steps are
            // drained with that half's scales, in the registers of the 128 path
            operands(st, ao, bw);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                load_sc(st, h, scl);
#pragma unroll
                for (int ti = 0; ti < 4; ++ti)
#pragma unroll
                    for (int tj = 0; tj < RT; ++tj) cl[ti][tj] = mfma_i8(bw[tj][h], ao[ti][h], v4i{0, 0, 0, 0});
                drain(cl, scl);
                if (h == 0) {  // finish the first half's drain before the second half's steps
#pragma unroll
                    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
                        for (int tj = 0; tj < RT; ++tj)
#pragma unroll
                            for (int e = 0; e < 4; ++e) keep(yacc[ti][tj][e]);
                }
            }
        } else if constexpr (!BLOCKED) {  // integer sums over all of K
            operands(st, ao, bw);
            mma(ao, bw, iacc, false);
        } else {
            operands(st, ao, bw);
            load_sc(st, 0, scl);
            mma(ao, bw, cl, true);
            drain(cl, scl);
        }
    };

    Staged r0, r1;
    gload(0, r0);
    gload(1, r1);
    lstore(0, r0);
    __syncthreads();
    // Block b computes from LDS slot b & 1 while block b+1 (in registers since
    // the previous step) goes to the other slot and block b+2 is fetched into
    // the registers just freed.  Loads past the last block repeat it and their
    // LDS copy goes to a slot nobody reads again.  Both halves of the loop are
    // written out with fixed register sets (no pointer selects between them).
    // Waves whose 64 tokens all lie past M only stage data (few-token launches,
    // which take RT < 4; the 256-row form keeps a branch-free loop).
    // KS: every wave is live; the second half skips an odd block past the last.
    const bool live = KS || RT == 4 || m0 + 64 * wm < M;
    for (int b = 0; b < nst; b += 2) {
        gload(b + 2, r0);
        if (live && (!KS || 2 * b + wm < nblk)) compute(0);
        lstore(1, r1);
        lds_barrier();
        if (b + 1 < nst) {
            gload(b + 3, r1);
            if (live && (!KS || 2 * b + 2 + wm < nblk)) compute(1);
            lstore(0, r0);
            lds_barrier();
        }
    }
    if constexpr (KS) {  // odd-block sums of wave (1, wn) join those of wave (0, wn)
        uint32_t *red = reinterpret_cast<uint32_t *>(lds) + (wn * 64 + l) * 16 * RT;
        if (wm == 1) {
#pragma unroll
            for (int ti = 0; ti < 4; ++ti)
#pragma unroll
                for (int tj = 0; tj < RT; ++tj)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        red[(ti * RT + tj) * 4 + e] = BLOCKED ? __float_as_uint(yacc[ti][tj][e])
                                                              : (uint32_t)iacc[ti][tj][e];
        }
        __syncthreads();
        if (wm == 1) return;
#pragma unroll
        for (int ti = 0; ti < 4; ++ti)
#pragma unroll
            for (int tj = 0; tj < RT; ++tj)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t o = red[(ti * RT + tj) * 4 + e];
                    if (BLOCKED) yacc[ti][tj][e] += __uint_as_float(o);
                    else iacc[ti][tj][e] += (int)o;
                }
    }

    // epilogue: lane (g, j), tile (ti, tj), element e -> token m0+64wm+16ti+j,
    // row 16(T0+RT*wn+tj)+4g+e: four consecutive outputs of one token per store
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) {
        const int m = m0 + (KS ? 0 : 64 * wm) + 16 * ti + j;
        if (m >= M) continue;
        // blocked: y = s_a * sum * 2^-6 (decoded weights are 64 t); SG 0: exact integer
        // sum times s_a * s_w
        const float f = (OUT == 2) ? 0.0f : BLOCKED ? s_a[m] * 0.015625f : s_a[m] * scales[0];
#pragma unroll
        for (int tj = 0; tj < RT; ++tj) {
            const int T = T0 + RT * wn + tj;
            if (T >= ntile_n) continue;
            const size_t idx = (size_t)m * N + (size_t)T * 16 + 4 * g;
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = BLOCKED ? yacc[ti][tj][e] : (float)(iacc[ti][tj][e] >> 6);
            if (OUT == 0) {
                const uint32_t lo = f32_to_bf16_rne(v[0] * f) | ((uint32_t)f32_to_bf16_rne(v[1] * f) << 16);
                const uint32_t hi = f32_to_bf16_rne(v[2] * f) | ((uint32_t)f32_to_bf16_rne(v[3] * f) << 16);
                *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(yout) + idx) = make_uint2(lo, hi);
            } else if (OUT == 1) {
                *reinterpret_cast<float4 *>(static_cast<float *>(yout) + idx) =
                    make_float4(v[0] * f, v[1] * f, v[2] * f, v[3] * f);
            } else {
                *reinterpret_cast<int4 *>(static_cast<int32_t *>(yout) + idx) =
                    make_int4(iacc[ti][tj][0] >> 6, iacc[ti][tj][1] >> 6, iacc[ti][tj][2] >> 6, iacc[ti][tj][3] >> 6);
            }
        }
    }
}

// --------------------------------------------------------------------------
// a6, 256-row form (the prefill shapes): same tiles, operands and arithmetic as
// gemm_kernel<OUT, SG, 4>, so results are bit-identical to it, but the data
// arrives and the work is ordered differently.
//  * Each block's activations (128 x 128 int8), 16 bricks and 256 scales go
//    straight from global memory into one of 4 LDS stages with
//    global_load_lds (no staging registers, no LDS store instructions), three
//    blocks ahead.  The activation tile is unpadded; chunk c of row r sits at
//    position c ^ (r & 7), which keeps the operand reads conflict-free.
//  * A SIMD runs one wave's VALU work in the shadow of that same wave's
//    matrix-core steps (about two VALU operations per step come for free), but
//    VALU work of one wave next to matrix-core work of another wave on the same
//    SIMD runs slower than the two one after the other.  So every wave does the
//    same thing at the same time and interleaves inside its own stream: a block
//    is two halves of 16 steps (row tiles 0-1, then 2-3; K-step 0 of the 8
//    tiles, then K-step 1), and after each step the wave drains half of one
//    finished tile of the other pair into fp32 and decodes one dword of the
//    weights the next half needs.  Half 0 drains the previous block's tiles
//    2-3 and decodes this block's tiles 2-3; half 1 drains this block's tiles
//    0-1 and decodes the next block's tiles 0-1.
//  * bf16 results leave through LDS as whole 512-byte token rows.
// The direct loads are issued from inline asm, so the compiler neither counts
// them nor makes LDS reads wait for them: each wave waits for its own loads of
// a stage (s_waitcnt vmcnt) before the barrier that publishes the stage.
// --------------------------------------------------------------------------
constexpr int kWideStages = 4;
constexpr int kWideAStage = kGemmBM * kBlockK;  // 16384 bytes, unpadded, swizzled
constexpr int kWideRowStride = 528;             // bf16 epilogue: 256 values + 16 bytes per token row

// 16 bytes per lane from global memory into LDS at lds + 16 * lane (the wave's
// 1 KB slice); M0 carries the LDS address and is restored afterwards.
__device__ __forceinline__ void dma16(const void *g, uint32_t lds) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds), "v"(g)
        : "memory");
}

// wait until at most N of this wave's global loads are pending and all its LDS
// reads are done, then meet the workgroup
template <int N>
__device__ __forceinline__ void wait_loads_barrier() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

template <int OUT, int SG>  // SG 128 or 0
__global__ __launch_bounds__(kGemmThreads) void gemm_wide_kernel(const uint8_t *__restrict__ packed,
                                                                  const float *__restrict__ scales,
                                                                  const int8_t *__restrict__ q,
                                                                  const float *__restrict__ s_a,
                                                                  void *__restrict__ yout, int M, int N, int K,
                                                                  int ntm) {
    constexpr bool BLOCKED = OUT != 2 && SG != 0;
    constexpr int S = kWideStages;
    constexpr int STAGE = kWideAStage + kBStage + (BLOCKED ? kSStage : 0);
    __shared__ __align__(16) unsigned char lds[S * STAGE];
    static_assert(kGemmBM * kWideRowStride <= S * STAGE, "epilogue tile fits the stages");
    const uint32_t lds0 = (uint32_t)(uintptr_t)lds;  // LDS byte address (low half of the flat address)
    const int G = gridDim.x;
    int t = blockIdx.x;
    if ((G & 7) == 0) t = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);  // XCD-aware order
    const int tm = t % ntm, tn = t / ntm;
    const int m0 = tm * kGemmBM, T0 = tn * 16;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63, g = l >> 4, j = l & 15;
    const int wm = w >> 2, wn = w & 3;
    const int nblk = K >> 7, ntile_n = N >> 4;

    // Direct-load sources of this lane (block 0; each block adds a fixed step).
    // Activations: wave w fills rows 16w..16w+15 with two 1 KB loads; lane l of
    // load i lands on row 16w + 8i + l/8 at chunk position l%8, which holds
    // logical chunk (l%8) ^ (l/8).  Rows past M repeat row 0 (never stored).
    const int8_t *asrc[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int r = 16 * w + 8 * i + (l >> 3);
        const int tok = m0 + r < M ? m0 + r : 0;
        asrc[i] = q + (size_t)tok * K + (((l & 7) ^ (l >> 3)) * 16);
    }
    // Bricks: wave w fills bricks 2w, 2w+1 (512 B each) with one 1 KB load.
    const int bT = min(T0 + 2 * w + (l >> 5), ntile_n - 1);
    const uint8_t *bsrc = packed + (size_t)bT * nblk * kBrickBytes + (l & 31) * 16;
    // Scales: wave w fills tiles 2w, 2w+1 (64 B each) with lanes 0..7.
    const int sT = min(T0 + 2 * w + (l >> 2), ntile_n - 1);
    const float *ssrc = BLOCKED ? scales + (size_t)sT * nblk * kTileN + (l & 3) * 4 : nullptr;

    auto issue = [&](int b) {  // this wave's loads of block b (clamped) into stage b % S
        const int bb = min(b, nblk - 1);
        const uint32_t st = lds0 + (uint32_t)((b % S) * STAGE);
#pragma unroll
        for (int i = 0; i < 2; ++i) dma16(asrc[i] + (size_t)bb * kBlockK, st + (2 * w + i) * 1024);
        dma16(bsrc + (size_t)bb * kBrickBytes, st + kWideAStage + w * 1024);
        if (BLOCKED && l < 8) dma16(ssrc + (size_t)bb * kTileN, st + kWideAStage + kBStage + w * 128);
    };
    constexpr int kLoadsPerBlock = BLOCKED ? 4 : 3;  // per wave (the scale load with 8 lanes)

    float yacc[4][4][4];
    v4i c[4][4];
    float sc[4][4];  // block scales of rows 4g..4g+3 of the wave's row tiles
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            c[a][b] = v4i{0, 0, 0, 0};
#pragma unroll
            for (int e = 0; e < 4; ++e) yacc[a][b][e] = 0.0f, sc[a][e] = 0.0f;
        }
    v4i ao[4][2], bw[4][2];  // activation operands [token tile][K-step], decoded weights [row tile][K-step]
    uint32_t wr[4][2];        // packed weight words [row tile][K-step]

    auto sbase = [&](int b) { return lds + (b % S) * STAGE; };
    auto read_ao = [&](int b, int s) {
        const unsigned char *base = sbase(b);
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
            const int r = 64 * wm + 16 * ti + j;
            ao[ti][s] = *reinterpret_cast<const v4i *>(base + r * kBlockK + (((4 * s + g) ^ (r & 7)) * 16));
        }
    };
    auto read_wr = [&](int b, int tj0) {  // row tiles tj0, tj0 + 1
        const unsigned char *base = sbase(b);
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            const uint2 v = *reinterpret_cast<const uint2 *>(base + kWideAStage + (4 * wn + tj0 + d) * 512 + l * 8);
            wr[tj0 + d][0] = v.x;
            wr[tj0 + d][1] = v.y;
        }
    };
    auto read_sc = [&](int b, int tj0) {  // row tiles tj0, tj0 + 1
        if constexpr (BLOCKED) {
            const unsigned char *base = sbase(b);
#pragma unroll
            for (int d = 0; d < 2; ++d) {
                const float4 s4 = *reinterpret_cast<const float4 *>(base + kWideAStage + kBStage +
                                                                    ((4 * wn + tj0 + d) * 16 + 4 * g) * 4);
                sc[tj0 + d][0] = s4.x;
                sc[tj0 + d][1] = s4.y;
                sc[tj0 + d][2] = s4.z;
                sc[tj0 + d][3] = s4.w;
            }
        }
    };
    // Half h: 16 steps on row tiles 2h, 2h+1.  After step k: elements 2(k&1), 2(k&1)+1 of
    // tile (k/4, o + (k/2 & 1)) of the other pair o are drained (the order those tiles
    // finished in), and dword k&3 of K-step (k/4 & 1) of row tile dt0 + k/8 is decoded
    // (the shifts of decode16).  Half 1 reloads K-step 0's activations for block bnext
    // once its own K-step-0 steps are done.
    auto half = [&](int h, int dt0, int bnext) {
        const int o = 2 - 2 * h;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int s = k >> 3, ti = (k >> 1) & 3, tj = 2 * h + (k & 1);
            c[ti][tj] = mfma_i8(bw[tj][s], ao[ti][s], (BLOCKED && s == 0) ? v4i{0, 0, 0, 0} : c[ti][tj]);
            if constexpr (BLOCKED) {
                const int dti = k >> 2, dtj = o + ((k >> 1) & 1), e0 = 2 * (k & 1);
#pragma unroll
                for (int e = e0; e < e0 + 2; ++e)
                    yacc[dti][dtj][e] = fmaf(sc[dtj][e], (float)c[dti][dtj][e], yacc[dti][dtj][e]);
            }
            {
                const int dtj = dt0 + (k >> 3), ds = (k >> 2) & 1, p = k & 3;
                bw[dtj][ds][p] = (int)((wr[dtj][ds] << (6 - 2 * p)) & 0xC0C0C0C0u);
            }
            if (h == 1 && k == 7) read_ao(bnext, 0);
            // unscaled: keep the written order (the compiler otherwise hoists K-step 1 steps
            // up to their just-issued operand reads and stalls on them)
            if constexpr (!BLOCKED) __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Prologue: blocks 0..2 in flight, 0 and 1 complete and published.
    issue(0);
    issue(1);
    issue(2);
    wait_loads_barrier<kLoadsPerBlock>();
    read_ao(0, 0);
    read_wr(0, 0);
    read_wr(0, 2);
#pragma unroll
    for (int tj = 0; tj < 2; ++tj) {
        bw[tj][0] = decode16(wr[tj][0]);
        bw[tj][1] = decode16(wr[tj][1]);
    }
    // Block b reads stage b (K-step 1 activations, scales) and stage b+1 (weights and K-step 0
    // activations of the next block).  The barrier at its top publishes block b+1: every wave
    // has finished its own loads of it, only block b+2 may still be pending.  Block b+3 then
    // refills the stage of block b-1, which nobody reads after that barrier.  The first
    // half-0 drains zeros (c and sc start at 0).
    for (int b = 0; b < nblk; ++b) {
        if (b > 0) wait_loads_barrier<kLoadsPerBlock>();
        issue(b + 3);
        read_ao(b, 1);
        read_sc(b, 0);
        half(0, 2, b + 1);
        read_wr(b + 1, 0);
        read_sc(b, 2);
        half(1, 0, b + 1);
        read_wr(b + 1, 2);
    }
    if constexpr (BLOCKED) {  // the last block's tiles 2-3
#pragma unroll
        for (int ti = 0; ti < 4; ++ti)
#pragma unroll
            for (int tj = 2; tj < 4; ++tj)
#pragma unroll
                for (int e = 0; e < 4; ++e) yacc[ti][tj][e] = fmaf(sc[tj][e], (float)c[ti][tj][e], yacc[ti][tj][e]);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the clamped tail loads still in flight

    // epilogue: lane (g, j), tile (ti, tj), element e -> token m0+64wm+16ti+j, row
    // 16(T0+4wn+tj)+4g+e
    if constexpr (OUT == 0) {  // bf16 through LDS: each store instruction writes two whole token rows
        wait_loads_barrier<0>();  // every wave past its last stage read
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
            const int r = 64 * wm + 16 * ti + j;
            const int m = m0 + r;
            const float f = m < M ? (BLOCKED ? s_a[m] * 0.015625f : s_a[m] * scales[0]) : 0.0f;
#pragma unroll
            for (int tj = 0; tj < 4; ++tj) {
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = BLOCKED ? yacc[ti][tj][e] : (float)(c[ti][tj][e] >> 6);
                const uint32_t lo = f32_to_bf16_rne(v[0] * f) | ((uint32_t)f32_to_bf16_rne(v[1] * f) << 16);
                const uint32_t hi = f32_to_bf16_rne(v[2] * f) | ((uint32_t)f32_to_bf16_rne(v[3] * f) << 16);
                *reinterpret_cast<uint2 *>(lds + r * kWideRowStride + ((4 * wn + tj) * 16 + 4 * g) * 2) =
                    make_uint2(lo, hi);
            }
        }
        wait_loads_barrier<0>();
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = 16 * w + 2 * i + (l >> 5);
            const int m = m0 + r;
            const int col = T0 * 16 + (l & 31) * 8;
            if (m < M && col < N)
                *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(yout) + (size_t)m * N + col) =
                    *reinterpret_cast<const uint4 *>(lds + r * kWideRowStride + (l & 31) * 16);
        }
    } else {
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
            const int m = m0 + 64 * wm + 16 * ti + j;
            if (m >= M) continue;
            const float f = (OUT == 2) ? 0.0f : BLOCKED ? s_a[m] * 0.015625f : s_a[m] * scales[0];
#pragma unroll
            for (int tj = 0; tj < 4; ++tj) {
                const int T = T0 + 4 * wn + tj;
                if (T >= ntile_n) continue;
                const size_t idx = (size_t)m * N + (size_t)T * 16 + 4 * g;
                if (OUT == 1) {
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = BLOCKED ? yacc[ti][tj][e] : (float)(c[ti][tj][e] >> 6);
                    *reinterpret_cast<float4 *>(static_cast<float *>(yout) + idx) =
                        make_float4(v[0] * f, v[1] * f, v[2] * f, v[3] * f);
                } else {
                    *reinterpret_cast<int4 *>(static_cast<int32_t *>(yout) + idx) =
                        make_int4(c[ti][tj][0] >> 6, c[ti][tj][1] >> 6, c[ti][tj][2] >> 6, c[ti][tj][3] >> 6);
                }
            }
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

// The all-waves fused form keeps every token's raw activation chunks in registers
// until the weights are in flight: tokens x chunk rounds x 16-byte words per chunk
// must stay within 64 dwords (more spills).
__host__ __device__ constexpr bool allwaves_fits(int xm, int tok, int nb) {
    return tok * ((nb + 3) / 4) * (xm == 0 ? 4 : xm == 1 ? 8 : 16) <= 64;
}

// SG: scale granularity (128 or 64 weights per scale, 0 = one scale for the
// matrix); the fused forms exist for SG 128 only.
template <int AM, int NB, bool INT_OUT, int FORM, int SG>
void gemv_launch_tok(int tok, dim3 grid, dim3 block, size_t lds, hipStream_t st, const GemvArgs &a) {
    if constexpr (FORM == kAllWaves || FORM == kAllWavesXF) {  // M <= 4 and allwaves_fits (checked by the caller)
        if (tok == 1) hipLaunchKernelGGL((gemv_kernel<AM, NB, 1, false, FORM, 128>), grid, block, lds, st, a);
        else if (tok == 2) hipLaunchKernelGGL((gemv_kernel<AM, NB, 2, false, FORM, 128>), grid, block, lds, st, a);
        else if constexpr (allwaves_fits(AM < 0 ? 0 : AM, 4, NB))
            hipLaunchKernelGGL((gemv_kernel<AM, NB, 4, false, FORM, 128>), grid, block, lds, st, a);
    } else if constexpr (FORM == kStaged) {
        if (tok == 1) hipLaunchKernelGGL((gemv_kernel<AM, NB, 1, INT_OUT, FORM, SG>), grid, block, lds, st, a);
        else if (tok == 2) hipLaunchKernelGGL((gemv_kernel<AM, NB, 2, INT_OUT, FORM, SG>), grid, block, lds, st, a);
        else if (tok == 4) hipLaunchKernelGGL((gemv_kernel<AM, NB, 4, INT_OUT, FORM, SG>), grid, block, lds, st, a);
        else if (tok == 8) hipLaunchKernelGGL((gemv_kernel<AM, NB, 8, INT_OUT, FORM, SG>), grid, block, lds, st, a);
        else hipLaunchKernelGGL((gemv_kernel<AM, NB, 16, INT_OUT, FORM, SG>), grid, block, lds, st, a);
    } else if constexpr (FORM == kQuantWaves) {
        hipLaunchKernelGGL((gemv_kernel<AM, NB, 16, false, FORM, 128>), grid, block, lds, st, a);
    } else {  // kDirect, kMulti: token capacity 16
        hipLaunchKernelGGL((gemv_kernel<AM, NB, 16, INT_OUT, FORM, SG>), grid, block, lds, st, a);
    }
}

template <int AM, int NB, bool INT_OUT, int SG>
void gemv_launch_form(int form, int tok, dim3 grid, dim3 block, size_t lds, hipStream_t st, const GemvArgs &a) {
    if constexpr (AM >= 0) {
        if (form == kQuantWaves) {
            gemv_launch_tok<AM, NB, false, kQuantWaves, 128>(tok, grid, block, lds, st, a);
        } else if (form == kAllWavesXF) {
            gemv_launch_tok<AM, NB, false, kAllWavesXF, 128>(tok, grid, block, lds, st, a);
        } else {
            gemv_launch_tok<AM, NB, false, kAllWaves, 128>(tok, grid, block, lds, st, a);
        }
    } else {
        if (form == kStaged) gemv_launch_tok<AM, NB, INT_OUT, kStaged, SG>(tok, grid, block, lds, st, a);
        else if (NB == 8 && form == kMulti) gemv_launch_tok<AM, 8, INT_OUT, kMulti, SG>(tok, grid, block, lds, st, a);
        else gemv_launch_tok<AM, NB, INT_OUT, kDirect, SG>(tok, grid, block, lds, st, a);
    }
}

constexpr size_t kMaxLds = 65536;

#ifndef BITNET_GEMV_BLOCKS_PER_WAVE
#define BITNET_GEMV_BLOCKS_PER_WAVE 4
#endif
#ifndef BITNET_GEMV_MAX_WAVES
#define BITNET_GEMV_MAX_WAVES 12
#endif
// CU count and the waves held at once (CUs x threads per CU / 64) of the
// device that `st` belongs to; zeros if unknown (then no occupancy-based choice
// is made).  Read once per device and cached (the values never change while the
// process runs), so a launch costs no attribute queries.
struct DeviceSlots {
    int64_t cus = 0, waves = 0;
};
constexpr int kSlotCacheDevices = 64;
std::atomic<int64_t> g_slot_cus[kSlotCacheDevices], g_slot_waves[kSlotCacheDevices];
DeviceSlots device_slots(hipStream_t st) {
    DeviceSlots d;
    int dev = 0;
    if (hipStreamGetDevice(st, &dev) != hipSuccess) return d;
    const bool cached = dev >= 0 && dev < kSlotCacheDevices;
    if (cached) {
        d.waves = g_slot_waves[dev].load(std::memory_order_acquire);
        if (d.waves > 0) {
            d.cus = g_slot_cus[dev].load(std::memory_order_relaxed);
            return d;
        }
    }
    int ncu = 0, thr = 0;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        hipDeviceGetAttribute(&thr, hipDeviceAttributeMaxThreadsPerMultiProcessor, dev) == hipSuccess &&
        ncu > 0 && thr >= kWave) {
        d.cus = ncu;
        d.waves = (int64_t)ncu * (thr / kWave);
        if (cached) {
            g_slot_cus[dev].store(d.cus, std::memory_order_relaxed);
            g_slot_waves[dev].store(d.waves, std::memory_order_release);
        }
    }
    return d;
}

// Split-K geometry of the decode product: about 4 blocks per wave, at most 12
// compute waves per workgroup (room for up to 4 quant waves in the fused
// form), no idle wave.  Two occupancy rules refine it (dev = the device's CU
// count and wave slots; zeros skip them):
// - at most one workgroup per CU and at least 8 blocks: a CU's four SIMDs
//   take waves w, w+4, w+8 in turn, so the workgroup lasts as long as its
//   busiest SIMD, ceil(nw/4) * per blocks; the split minimising that is taken
//   (ties keep the base split, else take the fewest waves).  Measured (product
//   / fused step, us): 2560x2560 5x4 -> 4x5 3.12/3.51 -> 2.96/3.34, 8 tokens
//   3.74 -> 3.41; 2560x3200 7x4 -> 4x7 3.27/3.76 -> 3.07/3.59; 2560x6912
//   11x5 -> 8x7 3.76/4.92 -> 3.69/4.40; 4096x2560 3.26/3.62 -> 3.07/3.40;
//   2560x1280 3x4 -> 4x3 fused 2.94 -> 2.86.  Below 8 blocks fixed per-wave
//   costs dominate (2560x384 as 3 waves of 1 block: fused 2.50 -> 2.59);
// - more workgroups than the device holds at once: each wave takes more
//   blocks, up to 8, until all are resident: 20480x3200 runs 5 waves of 5
//   blocks instead of 7 waves of 4 (product 6.17 -> 5.70 us, fused step 7.61
//   -> 6.75 us, 8 tokens 8.58 -> 7.82 us).
// Fused support does not change (per stays <= 8 where the base split has it).
// Every form uses the same geometry and the same summation order, so their fp32
// results are bit-identical.
constexpr int kMaxSplitWaves = BITNET_GEMV_MAX_WAVES;
constexpr int kBlocksPerWave = BITNET_GEMV_BLOCKS_PER_WAVE;
void gemv_split(int K, int N, const DeviceSlots &dev, int *nw_out, int *per_out) {
    const int nblk = K / (int)kBlockK;
    int nw = (nblk + kBlocksPerWave - 1) / kBlocksPerWave;
    if (nw > kMaxSplitWaves) nw = kMaxSplitWaves;
    if (nw < 1) nw = 1;
    int per = (nblk + nw - 1) / nw;
    nw = (nblk + per - 1) / per;
    const int64_t wgs = N / kTileN;
    if (dev.cus > 0 && wgs <= dev.cus && nblk >= 8 && per <= 8) {
        int best = ((nw + 3) / 4) * per;
        for (int p = nblk < 8 ? nblk : 8; p >= 1; --p) {  // ties: the base split, else fewer waves
            const int w = (nblk + p - 1) / p;
            if (w > kMaxSplitWaves) continue;
            const int cost = ((w + 3) / 4) * p;
            if (cost < best) {
                best = cost;
                per = p;
                nw = w;
            }
        }
    }
    while (dev.waves > 0 && per < 8 && per < nblk && wgs * nw > dev.waves) {
        ++per;
        nw = (nblk + per - 1) / per;
    }
    *nw_out = nw;
    *per_out = per;
}

size_t gemv_fused_lds(int M, int K, int nw) { return gemv_fused_region(M, K, nw) + (16 + 48) * sizeof(float); }

// Form of the fused quantise-and-multiply launch for activation mode xm (0 bf16,
// 1 fp32, 2 and 3 two-half fp32): every compute wave quantises its own slice when the
// tokens' raw chunks fit in registers, else four extra quant waves do it.
int gemv_fused_form(int xm, int M, int K, int N, const DeviceSlots &dev) {
    int nw, per;
    gemv_split(K, N, dev, &nw, &per);
    const int tok = M == 1 ? 1 : M == 2 ? 2 : 4;
    return (M <= 4 && allwaves_fits(xm, tok, per < 8 ? per : 8)) ? kAllWaves : kQuantWaves;
}

// Picks the form and launches.  Returns false (nothing launched) if a fused
// form was asked for and does not fit.
template <int AM, bool INT_OUT, int SG = 128>
bool gemv_launch(GemvArgs a, hipStream_t st) {
    const DeviceSlots dev = device_slots(st);
    int nw, per;
    gemv_split(a.K, a.N, dev, &nw, &per);
    a.per = per;
    a.nwc = nw;
    int form;
    size_t lds;
    if (AM >= 0) {
        if (per > 8) return false;
        form = gemv_fused_form(AM, a.M, a.K, a.N, dev);
        a.qw = form == kQuantWaves ? 4 : 0;
        lds = gemv_fused_lds(a.M, a.K, nw);
        if (lds > kMaxLds) return false;
    } else {
        a.qw = 0;
        if (per > 8) {
            form = kMulti;
            lds = (size_t)nw * 4 * kWave * sizeof(int);
        } else if (gemv_fused_lds(a.M, a.K, nw) <= kMaxLds) {
            form = kStaged;
            lds = gemv_fused_lds(a.M, a.K, nw);
        } else {
            form = kDirect;
            lds = (size_t)nw * 4 * kWave * sizeof(int);
        }
    }
    // Fused all-waves form: quantise before requesting the weights (kAllWavesXF) when the
    // grid has more 16-row workgroups than CUs and all of them are resident at once
    // (measured with bf16 activations over 2560..20480 rows x K 2560..4096: 0.1-0.55 us
    // faster there; with at most one workgroup per CU, or more waves than fit, the serial
    // start costs 0.2-0.45 us instead).
    if (form == kAllWaves && dev.cus > 0) {
        const int64_t wgs = a.N / kTileN, waves = wgs * (nw + a.qw);
        if (wgs > dev.cus && waves <= dev.waves) form = kAllWavesXF;
    }
    const int nb = per < 8 ? per : 8;
    const int tok = a.M == 1 ? 1 : a.M == 2 ? 2 : a.M <= 4 ? 4 : a.M <= 8 ? 8 : 16;
    dim3 grid(a.N / (int)kTileN), block(kWave * (nw + a.qw));
    switch (nb) {
        case 1: gemv_launch_form<AM, 1, INT_OUT, SG>(form, tok, grid, block, lds, st, a); break;
        case 2: gemv_launch_form<AM, 2, INT_OUT, SG>(form, tok, grid, block, lds, st, a); break;
        case 3: gemv_launch_form<AM, 3, INT_OUT, SG>(form, tok, grid, block, lds, st, a); break;
        case 4: gemv_launch_form<AM, 4, INT_OUT, SG>(form, tok, grid, block, lds, st, a); break;
        case 5: gemv_launch_form<AM, 5, INT_OUT, SG>(form, tok, grid, block, lds, st, a); break;
        case 6: gemv_launch_form<AM, 6, INT_OUT, SG>(form, tok, grid, block, lds, st, a); break;
        case 7: gemv_launch_form<AM, 7, INT_OUT, SG>(form, tok, grid, block, lds, st, a); break;
        default: gemv_launch_form<AM, 8, INT_OUT, SG>(form, tok, grid, block, lds, st, a); break;
    }
    return true;
}

template <int XM>
void quant_launch(const void *x, int M, int K, int8_t *q, float *s_a, hipStream_t st) {
    const int nvec = K / 8;
    if (nvec <= 256) hipLaunchKernelGGL((quant_act_kernel<XM, 1>), dim3(M), dim3(256), 0, st, x, K, q, s_a);
    else if (nvec <= 512) hipLaunchKernelGGL((quant_act_kernel<XM, 2>), dim3(M), dim3(256), 0, st, x, K, q, s_a);
    else if (nvec <= 1024) hipLaunchKernelGGL((quant_act_kernel<XM, 4>), dim3(M), dim3(256), 0, st, x, K, q, s_a);
    else if (nvec <= 2048) hipLaunchKernelGGL((quant_act_kernel<XM, 8>), dim3(M), dim3(256), 0, st, x, K, q, s_a);
    else hipLaunchKernelGGL((quant_act_kernel<XM, 0>), dim3(M), dim3(256), 0, st, x, K, q, s_a);
}

// Row tiles per wave: 4 (256-row workgroup tiles) unless that leaves the chip
// short of workgroups (few tokens), then 2 or 1 (128 / 64 rows).
int gemm_row_tiles(int M, int N) {
    const int ntm = (M + kGemmBM - 1) / kGemmBM;
    for (int rt = 4; rt > 1; rt >>= 1)
        if ((int64_t)ntm * ((N + 64 * rt - 1) / (64 * rt)) >= 200) return rt;
    return 1;
}

// Launch plan of the prefill product.  With fewer than 256-row tiles, 64-token
// tiles with two blocks per stage (KS) replace the 128-token ones when there
// are at most 128 tokens or the 128-token grid would stay under 200 workgroups
// (measured: 13824x2560 at 16 / 64 / 128 tokens 11.26 / 12.36 / 16.3 -> 9.36 /
// 10.51 / 14.3 us, 2560x2560 at 128 tokens 14.9 -> 9.9 us, 512x2560x6912 35.2 ->
// 31.8 us; at 256 tokens x 13824 rows, 216 workgroups already, 22.5 -> 25.2 us,
// so the 128-token tiles stay there).  Not for 64-weight scales (their staging
// fills the scale slots).
struct GemmPlan {
    int rt, ntm, ntn;
    bool ks;
};
GemmPlan gemm_plan(int M, int N, int SG) {
    GemmPlan g;
    g.rt = gemm_row_tiles(M, N);
    g.ntm = (M + kGemmBM - 1) / kGemmBM;
    g.ntn = (N + 64 * g.rt - 1) / (64 * g.rt);
    g.ks = g.rt < 4 && SG != 64 && (M <= 128 || (int64_t)g.ntm * g.ntn < 200);
    if (g.ks) {
        g.ntm = (M + 63) / 64;
        g.rt = (int64_t)g.ntm * ((N + 127) / 128) >= 200 ? 2 : 1;
        g.ntn = (N + 64 * g.rt - 1) / (64 * g.rt);
    }
    return g;
}

template <int OUT, int SG = 128>
void gemm_launch(const uint8_t *p, const float *s, const int8_t *q, const float *sa, void *y, int M, int N, int K,
                 hipStream_t st) {
    const GemmPlan g = gemm_plan(M, N, SG);
    const int ntm = g.ntm;
    const dim3 grid(g.ntm * g.ntn), block(kGemmThreads);
    if (g.rt == 4) {
        if constexpr (SG != 64)  // direct staging, in-wave interleaving
            hipLaunchKernelGGL((gemm_wide_kernel<OUT, SG>), grid, block, 0, st, p, s, q, sa, y, M, N, K, ntm);
        else
            hipLaunchKernelGGL((gemm_kernel<OUT, SG, 4>), grid, block, 0, st, p, s, q, sa, y, M, N, K, ntm);
    } else if (g.rt == 2) {
        if constexpr (SG != 64)
            if (g.ks) {
                hipLaunchKernelGGL((gemm_kernel<OUT, SG, 2, true>), grid, block, 0, st, p, s, q, sa, y, M, N, K, ntm);
                return;
            }
        hipLaunchKernelGGL((gemm_kernel<OUT, SG, 2>), grid, block, 0, st, p, s, q, sa, y, M, N, K, ntm);
    } else {
        if constexpr (SG != 64)
            if (g.ks) {
                hipLaunchKernelGGL((gemm_kernel<OUT, SG, 1, true>), grid, block, 0, st, p, s, q, sa, y, M, N, K, ntm);
                return;
            }
        hipLaunchKernelGGL((gemm_kernel<OUT, SG, 1>), grid, block, 0, st, p, s, q, sa, y, M, N, K, ntm);
    }
}

// Integer sums over all of K are held as 64 * sum in int32: |64 * 127 * K| < 2^31.
constexpr int kMaxIntK = 262144;

// The launch's work-item count must fit the 32-bit grid size.
bool gemm_grid_ok(int M, int N, int SG) {
    const GemmPlan g = gemm_plan(M, N, SG);
    return (int64_t)g.ntm * g.ntn * kGemmThreads < ((int64_t)1 << 32);
}
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

bitnet_status_t bitnet_gemv_split(int N, int K, int64_t cus, int64_t wave_slots, int *waves,
                                  int *blocks_per_wave) {
    if (!waves || !blocks_per_wave || cus < 0 || wave_slots < 0) return BITNET_ERR_INVALID_ARG;
    if (!shape_ok(N, K)) return BITNET_ERR_UNSUPPORTED_SHAPE;
    DeviceSlots dev;
    dev.cus = cus;
    dev.waves = wave_slots;
    gemv_split(K, N, dev, waves, blocks_per_wave);
    return BITNET_OK;
}

bitnet_status_t bitnet_quant_act(const void *x, int xdt, int M, int K, int8_t *q, float *s_a,
                                 hipStream_t stream) {
    if (!x || !q || !s_a || !aligned(x, 16) || !aligned(q, 16) || !aligned(s_a, 4)) return BITNET_ERR_INVALID_ARG;
    if (xdt != BITNET_DT_BF16 && xdt != BITNET_DT_F32) return BITNET_ERR_INVALID_ARG;
    if (M < 1 || M > 65535 * 1024 || K < 16 || K % 16) return BITNET_ERR_UNSUPPORTED_SHAPE;
    if (xdt == BITNET_DT_BF16) quant_launch<0>(x, M, K, q, s_a, stream);
    else quant_launch<1>(x, M, K, q, s_a, stream);
    return launched();
}

bitnet_status_t bitnet_quant_act_fold(const float *y, int M, int H, int8_t *q, float *s_a, hipStream_t stream) {
    if (!y || !q || !s_a || !aligned(y, 16) || !aligned(q, 16) || !aligned(s_a, 4)) return BITNET_ERR_INVALID_ARG;
    if (M < 1 || M > 65535 * 1024 || H < 16 || H % 16) return BITNET_ERR_UNSUPPORTED_SHAPE;
    quant_launch<2>(y, M, H, q, s_a, stream);
    return launched();
}

bitnet_status_t bitnet_quant_act_relu2_glu(const float *y, int M, int H, int8_t *q, float *s_a,
                                           hipStream_t stream) {
    if (!y || !q || !s_a || !aligned(y, 16) || !aligned(q, 16) || !aligned(s_a, 4)) return BITNET_ERR_INVALID_ARG;
    if (M < 1 || M > 65535 * 1024 || H < 16 || H % 16) return BITNET_ERR_UNSUPPORTED_SHAPE;
    quant_launch<3>(y, M, H, q, s_a, stream);
    return launched();
}

bitnet_status_t bitnet_w2a8_gemv(const uint8_t *packed, const float *scales, const int8_t *q, const float *s_a,
                                 float *y, int M, int N, int K, hipStream_t stream) {
    if (!packed || !scales || !q || !s_a || !y) return BITNET_ERR_INVALID_ARG;
    if (!aligned(packed, 16) || !aligned(scales, 16) || !aligned(q, 16) || !aligned(s_a, 4) || !aligned(y, 16))
        return BITNET_ERR_INVALID_ARG;
    if (!shape_ok(N, K) || M < 1 || M > kGemvMaxM) return BITNET_ERR_UNSUPPORTED_SHAPE;
    GemvArgs a{packed, scales, q, s_a, y, nullptr, nullptr, nullptr, M, N, K, 0, 0, 0};
    gemv_launch<-1, false>(a, stream);
    return launched();
}

bitnet_status_t bitnet_w2a8_gemm(const uint8_t *packed, const float *scales, const int8_t *q, const float *s_a,
                                 void *y, int ydt, int M, int N, int K, hipStream_t stream) {
    if (!packed || !scales || !q || !s_a || !y) return BITNET_ERR_INVALID_ARG;
    if (!aligned(packed, 16) || !aligned(scales, 16) || !aligned(q, 16) || !aligned(s_a, 4) || !aligned(y, 16))
        return BITNET_ERR_INVALID_ARG;
    if (ydt != BITNET_DT_BF16 && ydt != BITNET_DT_F32) return BITNET_ERR_INVALID_ARG;
    if (!shape_ok(N, K) || M < 1 || !gemm_grid_ok(M, N, 128)) return BITNET_ERR_UNSUPPORTED_SHAPE;
    if (ydt == BITNET_DT_BF16) gemm_launch<0>(packed, scales, q, s_a, y, M, N, K, stream);
    else gemm_launch<1>(packed, scales, q, s_a, y, M, N, K, stream);
    return launched();
}

bitnet_status_t bitnet_w2a8_gemv_g(const uint8_t *packed, const float *scales, const int8_t *q, const float *s_a,
                                   float *y, int M, int N, int K, int scale_block, hipStream_t stream) {
    if (scale_block == 128) return bitnet_w2a8_gemv(packed, scales, q, s_a, y, M, N, K, stream);
    if (scale_block != 64 && scale_block != 0) return BITNET_ERR_INVALID_ARG;
    if (!packed || !scales || !q || !s_a || !y) return BITNET_ERR_INVALID_ARG;
    if (!aligned(packed, 16) || !aligned(scales, 16) || !aligned(q, 16) || !aligned(s_a, 4) || !aligned(y, 16))
        return BITNET_ERR_INVALID_ARG;
    if (!shape_ok(N, K) || M < 1 || M > kGemvMaxM) return BITNET_ERR_UNSUPPORTED_SHAPE;
    if (scale_block == 0 && K > kMaxIntK) return BITNET_ERR_UNSUPPORTED_SHAPE;
    GemvArgs a{packed, scales, q, s_a, y, nullptr, nullptr, nullptr, M, N, K, 0, 0, 0};
    if (scale_block == 64) gemv_launch<-1, false, 64>(a, stream);
    else gemv_launch<-1, false, 0>(a, stream);
    return launched();
}

bitnet_status_t bitnet_w2a8_gemm_g(const uint8_t *packed, const float *scales, const int8_t *q, const float *s_a,
                                   void *y, int ydt, int M, int N, int K, int scale_block, hipStream_t stream) {
    if (scale_block == 128) return bitnet_w2a8_gemm(packed, scales, q, s_a, y, ydt, M, N, K, stream);
    if (scale_block != 64 && scale_block != 0) return BITNET_ERR_INVALID_ARG;
    if (!packed || !scales || !q || !s_a || !y) return BITNET_ERR_INVALID_ARG;
    if (!aligned(packed, 16) || !aligned(scales, 16) || !aligned(q, 16) || !aligned(s_a, 4) || !aligned(y, 16))
        return BITNET_ERR_INVALID_ARG;
    if (ydt != BITNET_DT_BF16 && ydt != BITNET_DT_F32) return BITNET_ERR_INVALID_ARG;
    if (!shape_ok(N, K) || M < 1 || !gemm_grid_ok(M, N, scale_block)) return BITNET_ERR_UNSUPPORTED_SHAPE;
    if (scale_block == 0 && K > kMaxIntK) return BITNET_ERR_UNSUPPORTED_SHAPE;
    if (scale_block == 64) {
        if (ydt == BITNET_DT_BF16) gemm_launch<0, 64>(packed, scales, q, s_a, y, M, N, K, stream);
        else gemm_launch<1, 64>(packed, scales, q, s_a, y, M, N, K, stream);
    } else {
        if (ydt == BITNET_DT_BF16) gemm_launch<0, 0>(packed, scales, q, s_a, y, M, N, K, stream);
        else gemm_launch<1, 0>(packed, scales, q, s_a, y, M, N, K, stream);
    }
    return launched();
}

bitnet_status_t bitnet_w2a8_gemv_act(const uint8_t *packed, const float *scales, const void *x, int xdt,
                                     float *y, int8_t *q_out, float *s_a_out, int M, int N, int K,
                                     hipStream_t stream) {
    if (!packed || !scales || !x || !y) return BITNET_ERR_INVALID_ARG;
    if (!aligned(packed, 16) || !aligned(scales, 16) || !aligned(x, 16) || !aligned(y, 16) ||
        !aligned(q_out, 16) || !aligned(s_a_out, 4))
        return BITNET_ERR_INVALID_ARG;
    if (xdt != BITNET_DT_BF16 && xdt != BITNET_DT_F32 && xdt != BITNET_DT_F32_FOLD2 &&
        xdt != BITNET_DT_F32_RELU2_GLU)
        return BITNET_ERR_INVALID_ARG;
    if (!shape_ok(N, K) || M < 1 || M > kGemvMaxM) return BITNET_ERR_UNSUPPORTED_SHAPE;
    int nw, per;
    gemv_split(K, N, device_slots(stream), &nw, &per);
    if (per > 8 || gemv_fused_lds(M, K, nw) > kMaxLds) return BITNET_ERR_UNSUPPORTED_SHAPE;
    GemvArgs a{packed, scales, x, nullptr, y, nullptr, q_out, s_a_out, M, N, K, 0, 0, 0};
    bool ok;
    if (xdt == BITNET_DT_BF16) ok = gemv_launch<0, false>(a, stream);
    else if (xdt == BITNET_DT_F32) ok = gemv_launch<1, false>(a, stream);
    else if (xdt == BITNET_DT_F32_FOLD2) ok = gemv_launch<2, false>(a, stream);
    else ok = gemv_launch<3, false>(a, stream);
    if (!ok) return BITNET_ERR_UNSUPPORTED_SHAPE;
    return launched();
}

bitnet_status_t bitnet_w2a8_acc_i32(const uint8_t *packed, const int8_t *q, int32_t *acc, int M, int N, int K,
                                    hipStream_t stream) {
    if (!packed || !q || !acc || !aligned(packed, 16) || !aligned(q, 16) || !aligned(acc, 16))
        return BITNET_ERR_INVALID_ARG;
    if (!shape_ok(N, K) || M < 1 || !gemm_grid_ok(M, N, 128) || K > kMaxIntK) return BITNET_ERR_UNSUPPORTED_SHAPE;
    if (M <= kGemvMaxM) {
        GemvArgs a{packed, nullptr, q, nullptr, nullptr, acc, nullptr, nullptr, M, N, K, 0, 0, 0};
        gemv_launch<-1, true>(a, stream);
    }
    else gemm_launch<2>(packed, nullptr, q, nullptr, acc, M, N, K, stream);
    return launched();
}

}  // extern "C"

// --------------------------------------------------------------------------
// a7: a chain of products with per-token requantisation between them (the
// decode pass through a stack of BitNet linear layers).  Host-side loop that
// enqueues one fused quantise-and-multiply launch per layer (M <= 2), or a
// quantisation launch and a product launch; intermediate fp32 activations
// ping-pong between two halves of the caller's workspace.
// --------------------------------------------------------------------------
namespace {
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct ChainPlan {
    size_t act_bytes;  // one fp32 activation buffer: M * max N
    size_t q_bytes;    // int8 q: M * max K
    size_t total;
};

bitnet_status_t chain_plan(const bitnet_chain_layer_t *layers, int n, int M, int x_width, ChainPlan *plan) {
    if (!layers || n < 1 || M < 1 || M > kGemvMaxM) return BITNET_ERR_INVALID_ARG;
    int64_t maxN = 0, maxK = 0;
    for (int i = 0; i < n; ++i) {
        const bitnet_chain_layer_t &L = layers[i];
        if (!L.packed || !L.scales || !aligned(L.packed, 16) || !aligned(L.scales, 16)) return BITNET_ERR_INVALID_ARG;
        if (!shape_ok(L.N, L.K)) return BITNET_ERR_UNSUPPORTED_SHAPE;
        const int in = i == 0 ? x_width : layers[i - 1].N;
        if (L.fold_input < BITNET_JUNCTION_NONE || L.fold_input > BITNET_JUNCTION_RELU2_GLU)
            return BITNET_ERR_INVALID_ARG;
        if (L.fold_input ? (in != 2 * L.K) : (in != L.K)) return BITNET_ERR_UNSUPPORTED_SHAPE;
        if (i == 0 && L.fold_input) return BITNET_ERR_UNSUPPORTED_SHAPE;
        maxN = L.N > maxN ? L.N : maxN;
        maxK = L.K > maxK ? L.K : maxK;
    }
    plan->act_bytes = align256((size_t)M * maxN * sizeof(float));
    plan->q_bytes = align256((size_t)M * maxK);
    plan->total = 2 * plan->act_bytes + plan->q_bytes + 256;
    return BITNET_OK;
}
}  // namespace

extern "C" {

size_t bitnet_w2a8_chain_workspace_bytes(const bitnet_chain_layer_t *layers, int n, int M) {
    ChainPlan plan;
    if (!layers || n < 1) return 0;
    return chain_plan(layers, n, M, layers[0].K, &plan) == BITNET_OK ? plan.total : 0;
}

}  // extern "C"

namespace {
// The chain's launches, with the workspace already checked against the plan.
bitnet_status_t chain_run(const bitnet_chain_layer_t *layers, int n, const void *x, int xdt, int M, float *y,
                          unsigned char *ws, const ChainPlan &plan, hipStream_t stream) {
    float *act[2] = {reinterpret_cast<float *>(ws), reinterpret_cast<float *>(ws + plan.act_bytes)};
    int8_t *q = reinterpret_cast<int8_t *>(ws + 2 * plan.act_bytes);
    float *s_a = reinterpret_cast<float *>(ws + 2 * plan.act_bytes + plan.q_bytes);

    const void *in = x;
    int in_dt = xdt;
    const DeviceSlots dev = device_slots(stream);
    for (int i = 0; i < n; ++i) {
        const bitnet_chain_layer_t &L = layers[i];
        float *out = (i == n - 1) ? y : act[i & 1];
        const int dt = L.fold_input == BITNET_JUNCTION_SUM         ? BITNET_DT_F32_FOLD2
                       : L.fold_input == BITNET_JUNCTION_RELU2_GLU ? BITNET_DT_F32_RELU2_GLU
                                                                   : in_dt;
        int nw, per;
        gemv_split(L.K, L.N, dev, &nw, &per);
        // One launch when the cheap fused form applies, else quantise + multiply.  The
        // fused form re-quantises in every workgroup, so its cost grows with the tokens
        // times the waves sharing each SIMD: worth it up to two tokens, and up to four on a
        // plain input while tokens x waves stays within twice the device's wave slots
        // (measured with fp32 input, fused against two launches: 13824x2560 at 3 tokens
        // 6.56 against 7.03 us; 20480x3200 at 3 tokens 11.9 us, two launches about 8.5).
        // Behind a junction the two fp32 halves per token cost more (2560x6912 behind the
        // fold, 3 tokens: 9.35 against 7.26 us), so there it stays at two.
        const int64_t grid_waves = (int64_t)(L.N / kTileN) * nw;
        const bool few = M <= 2 || (M <= 4 && L.fold_input == BITNET_JUNCTION_NONE && dev.waves > 0 &&
                                    M * grid_waves <= 2 * dev.waves);
        const bool fused = few && per <= 8 && gemv_fused_lds(M, L.K, nw) <= kMaxLds &&
                           gemv_fused_form(dt, M, L.K, L.N, dev) == kAllWaves;
        if (fused) {
            GemvArgs a{L.packed, L.scales, in, nullptr, out, nullptr, nullptr, nullptr, M, L.N, L.K, 0, 0, 0};
            bool ok;
            if (dt == BITNET_DT_BF16) ok = gemv_launch<0, false>(a, stream);
            else if (dt == BITNET_DT_F32) ok = gemv_launch<1, false>(a, stream);
            else if (dt == BITNET_DT_F32_FOLD2) ok = gemv_launch<2, false>(a, stream);
            else ok = gemv_launch<3, false>(a, stream);
            if (!ok) return BITNET_ERR_UNSUPPORTED_SHAPE;
        } else {
            if (dt == BITNET_DT_BF16) quant_launch<0>(in, M, L.K, q, s_a, stream);
            else if (dt == BITNET_DT_F32) quant_launch<1>(in, M, L.K, q, s_a, stream);
            else if (dt == BITNET_DT_F32_FOLD2) quant_launch<2>(in, M, L.K, q, s_a, stream);
            else quant_launch<3>(in, M, L.K, q, s_a, stream);
            GemvArgs a{L.packed, L.scales, q, s_a, out, nullptr, nullptr, nullptr, M, L.N, L.K, 0, 0, 0};
            gemv_launch<-1, false>(a, stream);
        }
        if (hipGetLastError() != hipSuccess) return BITNET_ERR_HIP;
        in = out;
        in_dt = BITNET_DT_F32;
    }
    return BITNET_OK;
}

// Argument checks shared by both chain entry points; fills the plan.
bitnet_status_t chain_check(const bitnet_chain_layer_t *layers, int n, const void *x, int xdt, int M, const float *y,
                            ChainPlan *plan) {
    if (!x || !y || !aligned(x, 16) || !aligned(y, 16)) return BITNET_ERR_INVALID_ARG;
    if (xdt != BITNET_DT_BF16 && xdt != BITNET_DT_F32) return BITNET_ERR_INVALID_ARG;
    if (!layers || n < 1) return BITNET_ERR_INVALID_ARG;
    return chain_plan(layers, n, M, layers[0].K, plan);
}

// Workspace of bitnet_w2a8_chain_static: one array per GPU, held until the process ends.
// Host code never uses the array's name as an address (on the host it is only a stand-in
// for the device symbol); it uses the device address hipGetSymbolAddress reports, looked
// up once per device with that device current and kept per device.
constexpr size_t kStaticScratchBytes = (size_t)4 << 20;
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
std::atomic<uintptr_t> g_scratch_ptr[kSlotCacheDevices];

bitnet_status_t static_scratch(hipStream_t stream, unsigned char **out) {
    int dev = 0;
    if (hipStreamGetDevice(stream, &dev) != hipSuccess) return BITNET_ERR_HIP;
    if (dev < 0 || dev >= kSlotCacheDevices) return BITNET_ERR_UNSUPPORTED_SHAPE;
    uintptr_t p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == 0) {
        int cur = 0;
        if (hipGetDevice(&cur) != hipSuccess) return BITNET_ERR_HIP;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return BITNET_ERR_HIP;
        void *addr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
        if (cur != dev && hipSetDevice(cur) != hipSuccess) return BITNET_ERR_HIP;
        if (e != hipSuccess || addr == nullptr) return BITNET_ERR_HIP;
        p = reinterpret_cast<uintptr_t>(addr);
        g_scratch_ptr[dev].store(p, std::memory_order_release);  // the same value on every thread
    }
    *out = reinterpret_cast<unsigned char *>(p);
    return BITNET_OK;
}
}  // namespace

extern "C" {

bitnet_status_t bitnet_w2a8_chain(const bitnet_chain_layer_t *layers, int n, const void *x, int xdt, int M,
                                  float *y, void *workspace, size_t workspace_bytes, hipStream_t stream) {
    ChainPlan plan;
    const bitnet_status_t st = chain_check(layers, n, x, xdt, M, y, &plan);
    if (st != BITNET_OK) return st;
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < plan.total) return BITNET_ERR_INVALID_ARG;
    return chain_run(layers, n, x, xdt, M, y, static_cast<unsigned char *>(workspace), plan, stream);
}

size_t bitnet_w2a8_chain_static_max_bytes(void) { return kStaticScratchBytes; }

bitnet_status_t bitnet_w2a8_chain_static(const bitnet_chain_layer_t *layers, int n, const void *x, int xdt, int M,
                                         float *y, hipStream_t stream) {
    ChainPlan plan;
    bitnet_status_t st = chain_check(layers, n, x, xdt, M, y, &plan);
    if (st != BITNET_OK) return st;
    if (plan.total > kStaticScratchBytes) return BITNET_ERR_UNSUPPORTED_SHAPE;
    unsigned char *ws = nullptr;
    st = static_scratch(stream, &ws);
    if (st != BITNET_OK) return st;
    return chain_run(layers, n, x, xdt, M, y, ws, plan, stream);
}

}  // extern "C"

// --------------------------------------------------------------------------
// a7, persistent form: the whole decode chain in one launch, batch 1.
//
// The chained products ([P2] "Architecture foundations": W2A8 GEMV; [P3] "Why WASM":
// a ternary model's layers) depend on each other only through each layer's full output
// vector, and at batch 1 a layer is a few microseconds of dependent latency against
// well under a microsecond of weight stream.  Here one 16-wave workgroup per CU runs
// every layer in turn; a layer's row tiles are spread over the first `nwg` workgroups
// (1, 2 or 4 tiles each), and:
//  - each layer writes its fp32 output into a buffer of its own that was filled with a
//    NaN pattern (0xFFFFFFFF, never a result of finite inputs) before the launch, with
//    agent-scope stores; the next layer's workgroups read the whole vector with
//    agent-scope loads and read again what still holds the pattern, until nothing does.
//    No fence and no shared counter: a value that is no longer the pattern is final;
//  - every workgroup requests a layer's weights (and block scales) into registers together
//    with the layer's input, so that weights and input arrive in one wait;
//  - every wait is bounded: after `spin_limit` rounds the workgroup writes the layer
//    index + 1 into the status word and leaves, so the kernel always ends;
//  - per tile the arithmetic is that of gemv_kernel's all-waves form: the input is
//    quantised per token exactly as quant_act_kernel does (exact max, correctly rounded
//    127 / amax, one fp32 multiply, half to even), waves split the blocks, each wave
//    sums its blocks' scaled int32 tiles in order and the wave partials are added in
//    wave order.  The split (waves per tile, blocks per wave) is this form's own, so the
//    fp32 order -- and with it the last bits of y -- can differ from the
//    launch-per-layer chain; both are within the product tolerance of the exact value.
// --------------------------------------------------------------------------
namespace {
struct PLayer {
    const uint8_t *packed;
    const float *scales;
    int64_t in_off;   // byte offset of the input in the workspace; -1: the caller's x
    int64_t out_off;  // byte offset of the output in the workspace; -1: the caller's y
    int N, K;
    int xm;           // input: 0 bf16 / 1 fp32 caller x (ready), 4 fp32 layer output,
                      // 5 two-half output folded, 6 two-half output gated
    int tp;           // row tiles per workgroup
    int nw, per;      // waves per tile, blocks per wave
    int nwg;          // workgroups taking part
    int pad;
};
static_assert(sizeof(PLayer) == 64, "PLayer is 64 bytes");

// The layer table is read-only for the whole launch: read through the constant address
// space, its fields arrive by scalar loads, which do not count against the vector-memory
// counter that orders the input and weight requests.
typedef __attribute__((address_space(4))) const PLayer CPLayer;

struct PArgs {
    const PLayer *table;
    int n;
    const void *x;
    float *y;
    unsigned char *ws;
    int64_t ws_bytes;  // the caller's workspace size: every layer buffer must lie inside it
    int *status;
    int spin_limit;
    int withhold;     // test only: the layer whose output is never stored (-1: none)
};

constexpr int kPWaves = 16;
constexpr int kPThreads = kPWaves * kWave;
constexpr int kPMaxK = 16384;        // 16 waves x 8 blocks x 128
constexpr int kPMaxNB = 8;
constexpr uint32_t kPending = 0xFFFFFFFFu;
constexpr int kPCheapPolls = 64;     // single-line polls per round of waiting

// Entry i of the layer table, read field by field through the constant address space.
__device__ __forceinline__ PLayer p_entry(const PLayer *table, int i) {
    CPLayer *t = (CPLayer *)table + i;
    PLayer r;
    r.packed = t->packed;
    r.scales = t->scales;
    r.in_off = t->in_off;
    r.out_off = t->out_off;
    r.N = t->N;
    r.K = t->K;
    r.xm = t->xm;
    r.tp = t->tp;
    r.nw = t->nw;
    r.per = t->per;
    r.nwg = t->nwg;
    r.pad = 0;
    return r;
}

__device__ __forceinline__ void st_agent(float *p, float v) {
    __hip_atomic_store(reinterpret_cast<uint32_t *>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// The weights one wave needs for one layer: up to 8 blocks of its tile, two words and one
// scale each.
struct PWeights {
    v2u w[kPMaxNB];
    float s[kPMaxNB];
};

__device__ __forceinline__ void p_role(const PLayer &L, int wg, int w, bool *active, int *tile, int *b0, int *nb) {
    const int ti = w / L.nw, wv = w - ti * L.nw;
    const int nblk = L.K >> 7;
    *tile = wg * L.tp + ti;
    *b0 = wv * L.per;
    *nb = min(L.per, nblk - *b0);
    *active = wg < L.nwg && ti < L.tp && *tile < (L.N >> 4) && *nb > 0;
}

// Buffer loads: the base address and range sit in a scalar resource, each load takes a
// 32-bit per-lane offset and a wave-uniform one, so a batch of loads costs one vector
// register of addressing; a load past the range returns 0 instead of touching memory.
constexpr int kRsrcWord3 = 0x00020000;  // raw 32-bit dwords, gfx9-family resource format
constexpr int kCpolSc1 = 16;            // cache policy: coherent at device (agent) scope
constexpr int kCpolNt = 2;              // cache policy: non-temporal (streamed once)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t p_rsrc(const void *base, size_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)min(bytes, (size_t)0x7FFFFFF0u),
                                             kRsrcWord3);
}

// Where one wave's weights for one layer start (wave-uniform), computed before any
// request of the layer goes out.
struct PWAddr {
    __amdgpu_buffer_rsrc_t wr, sr;  // the layer's packed weights and block scales
    uint32_t wo, so;                // byte offsets of the wave's first brick / first scale block
    int nb;                         // blocks the wave sums (0 if idle)
};

__device__ __forceinline__ PWAddr p_weight_addr(const PLayer &L, int wg, int w) {
    bool active;
    int tile, b0, nb;
    p_role(L, wg, w, &active, &tile, &b0, &nb);
    const uint32_t base = active ? (uint32_t)(tile * (L.K >> 7) + b0) : 0u;
    PWAddr r;
    const size_t bricks = (size_t)(L.N >> 4) * (L.K >> 7);
    r.wr = p_rsrc(L.packed, bricks * kBrickBytes);
    r.sr = p_rsrc(L.scales, bricks * kTileN * sizeof(float));
    r.wo = base * (uint32_t)kBrickBytes;
    r.so = base * (uint32_t)(kTileN * sizeof(float));
    r.nb = active ? nb : 0;
    return r;
}

// Always 8 weight and 8 scale loads per lane (a fixed count, so that waiting for data
// requested before them never waits for them): blocks past the wave's last read its last
// one again (an idle wave reads the layer's first brick), which the caches hold.
__device__ __forceinline__ void p_load_weights(const PWAddr &ad, int l, PWeights &r) {
    const int last = ad.nb > 0 ? ad.nb - 1 : 0;
    const uint32_t lw = (uint32_t)l * 8u, ls = (uint32_t)(l & 15) * 4u;
#pragma unroll
    for (int i = 0; i < kPMaxNB; ++i) {
        const uint32_t bi = (uint32_t)(i < last ? i : last);
        r.w[i] = __builtin_amdgcn_raw_buffer_load_b64(ad.wr, lw, ad.wo + bi * (uint32_t)kBrickBytes, kCpolNt);
        r.s[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
            ad.sr, ls, ad.so + bi * (uint32_t)(kTileN * sizeof(float)), kCpolNt));
    }
}

// One layer of the persistent chain.  Its weights are requested together with its input
// (a request for the next layer's weights made before waiting here would delay every
// read of the input: a wave's vector-memory requests complete in the order issued).
__device__ __forceinline__ bool p_layer(const PArgs &a, int li, int8_t *qs, float *red, uint32_t *vote,
                                        float *amax_part) {
    const PLayer L = p_entry(a.table, li);
    const int wg = blockIdx.x, t = threadIdx.x, l = t & 63;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    // a table that does not fit the workspace it came with: every workgroup reads the same
    // entry, so all of them stop here (status -(layer + 1)) and none waits on another
    {
        const int64_t in_end = L.in_off + (int64_t)(L.xm >= 5 ? 2 * L.K : L.K) * 4;
        const int64_t out_end = L.out_off + (int64_t)L.N * 4;
        const bool shape_ok = L.K >= (int)kBlockK && (L.K & (kBlockK - 1)) == 0 && L.N >= (int)kTileN &&
                              (L.N & (kTileN - 1)) == 0 && L.K <= (L.xm >= 5 ? kPMaxK / 2 : kPMaxK) &&
                              (L.tp == 1 || L.tp == 2 || L.tp == 4) && L.nw * L.tp == kPWaves && L.per >= 1 &&
                              L.per <= kPMaxNB && L.per * L.nw * (int)kBlockK >= L.K;
        if (!shape_ok || (L.xm >= 4 && (L.in_off < 256 || in_end > a.ws_bytes)) ||
            (L.out_off >= 0 && (L.out_off < 256 || out_end > a.ws_bytes))) {
            if (blockIdx.x == 0 && threadIdx.x == 0)
                __hip_atomic_store(a.status, -(li + 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return false;
        }
    }
    const bool part = wg < L.nwg;
    const int K = L.K;
    const int xm = L.xm;

    // (1) this thread's input: elements t, t + 1024, ... (16 of a plain input, or 8 of each
    //     half of a two-half input), so that every load instruction of a wave reads 256
    //     consecutive bytes.  Requested with agent-scope loads (always 16 of them; those
    //     past the input read 0 without a memory request), then the layer's weights; the words are checked only after
    //     both requests are out, so that check waits for the input alone.
    constexpr int NE = kPMaxK / kPThreads;  // 16 elements per thread at most
    uint32_t u[NE];  // raw words; once complete, the input values' bits (junction applied)
    bool have = true;
    // the input buffer: K values, or 2K for a two-half input (loads past it read 0)
    const __amdgpu_buffer_rsrc_t ir =
        p_rsrc(xm >= 4 ? a.ws + L.in_off : a.ws, (size_t)(xm >= 5 ? 2 * K : K) * sizeof(float));
    const uint32_t to = (uint32_t)t * 4u;
    // The whole offset goes in the per-lane operand: the range check (a load past the
    // buffer returns 0 and makes no memory request) leaves the scalar offset out.
    auto issue = [&]() {
        if (xm >= 5) {
            const uint32_t th = to + (uint32_t)K * 4u;
#pragma unroll
            for (int i = 0; i < NE / 2; ++i) {
                u[i] = __builtin_amdgcn_raw_buffer_load_b32(ir, to + (uint32_t)(i * kPThreads * 4), 0, kCpolSc1);
                u[NE / 2 + i] =
                    __builtin_amdgcn_raw_buffer_load_b32(ir, th + (uint32_t)(i * kPThreads * 4), 0, kCpolSc1);
            }
        } else {
#pragma unroll
            for (int i = 0; i < NE; ++i)
                u[i] = __builtin_amdgcn_raw_buffer_load_b32(ir, to + (uint32_t)(i * kPThreads * 4), 0, kCpolSc1);
        }
    };
    const int nv = (K + kPThreads - 1) / kPThreads;  // element slots in use (wave-uniform)
    // every element this thread holds has arrived: convert (junction applied) in place
    auto check = [&]() {
        bool ok = true;
#pragma unroll
        for (int i = 0; i < NE / 2; ++i) {
            if (i >= nv) break;
            const bool mine = t + i * kPThreads < K;
            if (mine && (u[i] == kPending || (xm >= 5 && u[NE / 2 + i] == kPending))) ok = false;
        }
        if (xm == 4) {
#pragma unroll
            for (int i = NE / 2; i < NE; ++i) {
                if (i >= nv) break;
                if (t + i * kPThreads < K && u[i] == kPending) ok = false;
            }
        }
        have = ok;
        if (!ok || xm == 4) return;
#pragma unroll
        for (int i = 0; i < NE / 2; ++i) {
            if (i >= nv) break;
            const float lo = __uint_as_float(u[i]), hi = __uint_as_float(u[NE / 2 + i]);
            float h;
            if (xm == 5) {
                h = __fadd_rn(lo, hi);
            } else {
                const float r = lo > 0.0f ? lo : 0.0f;
                h = __fmul_rn(__fmul_rn(r, r), hi);
            }
            u[i] = __float_as_uint(h);
        }
    };
    if (!part) return true;
    const PWAddr cad = p_weight_addr(L, wg, w);
    PWeights cur;
    __builtin_amdgcn_sched_barrier(0);
    if (xm >= 4) issue();
    __builtin_amdgcn_sched_barrier(0);
    p_load_weights(cad, l, cur);  // a fixed count: the check of the input waits for the input alone
    __builtin_amdgcn_sched_barrier(0);
    if (xm < 4) {  // the caller's input (first layer): ready, ordinary loads
#pragma unroll
        for (int i = 0; i < NE; ++i) {
            if (i >= nv) break;
            const int k = min(t + i * kPThreads, K - 1);
            u[i] = xm == 0 ? (uint32_t) static_cast<const uint16_t *>(a.x)[k] << 16
                           : static_cast<const uint32_t *>(a.x)[k];
        }
    } else {
        check();
    }

    // (2) until every value of the input has arrived: a double-buffered vote in LDS
    //     behind LDS-only barriers.  A workgroup that produced part of the previous layer
    //     is on time and asks again at once; one that had no work there may be waiting
    //     layers early and first waits cheaply (below).
    const bool on_time = li > 0 && wg < p_entry(a.table, li - 1).nwg;
    int rounds = 0;
    for (int par = 0;; par ^= 1) {
        const uint64_t b = __ballot(!have);
        if (l == 0) vote[par * kPWaves + w] = b != 0;
        lds_barrier();
        uint32_t any = 0;
#pragma unroll
        for (int i = 0; i < kPWaves; ++i) any |= vote[par * kPWaves + i];
        if (!any) break;
        if (++rounds >= a.spin_limit) {
            if (t == 0) __hip_atomic_store(a.status, li + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return false;
        }
        // Not there yet.  A workgroup with no work in the layers before may be waiting
        // several layers early: until the first 64 values have arrived (their producer
        // finishes with the others), only wave 0 asks, one line per poll and at most
        // kPCheapPolls times, while the other waves wait at the barrier.
        if (!on_time && w == 0) {
            for (int c = 0; c < kPCheapPolls; ++c) {
                const uint32_t v0 = __builtin_amdgcn_raw_buffer_load_b32(ir, (uint32_t)l * 4u, 0, kCpolSc1);
                if (__ballot(l < K && v0 == kPending) == 0) break;
            }
        }
        lds_barrier();
        if (!have) {
            issue();
            check();
        }
    }

    // (3) per-token absmax over the whole input, then each element -> int8 in LDS: the
    //     arithmetic of quantize8 (one fp32 multiply, then the add of 1.5 * 2^23 that rounds
    //     half to even; the code is the sum's low byte)
    const int ne = xm >= 5 ? min(nv, NE / 2) : nv;  // element slots holding input values
    float mx = 0.0f;
#pragma unroll
    for (int i = 0; i < NE; ++i) {
        if (i >= ne) break;
        if (t + i * kPThreads < K) mx = fmaxf(mx, fabsf(__uint_as_float(u[i])));
    }
    mx = wave_max(mx);
    if (l == 0) amax_part[w] = mx;
    lds_barrier();
    uint32_t um = 0;
#pragma unroll
    for (int i = 0; i < kPWaves; ++i) um = max(um, __float_as_uint(amax_part[i]));
    const float amax_c = fmaxf(__uint_as_float(um), 1e-5f);
    const float inv = __fdiv_rn(127.0f, amax_c);
    {
#pragma clang fp contract(off)
#pragma unroll
        for (int i = 0; i < NE; ++i) {
            if (i >= ne) break;
            const int k = t + i * kPThreads;
            if (k < K) {
                const float v = __uint_as_float(u[i]) * inv;
                qs[k] = (int8_t)(__float_as_uint(v + 12582912.0f) & 0xFFu);
            }
        }
    }
    const float s_a = __fdiv_rn(amax_c, 127.0f);
    lds_barrier();

    // (4) this wave's blocks of its tile: matrix-core steps on the LDS copy of q (token 0
    //     in lanes 0..15, the other lanes zero) and the decoded weights in `cur`
    bool active;
    int tile, b0, nb;
    p_role(L, wg, w, &active, &tile, &b0, &nb);
    const int g = l >> 4, j = l & 15;
    const int ti = w / L.nw, wv = w - ti * L.nw;
    float yacc = 0.0f;
    if (active) {
#pragma unroll
        for (int i = 0; i < kPMaxNB; ++i) {
            if (i < nb) {
                v4i a0 = v4i{0, 0, 0, 0}, a1 = v4i{0, 0, 0, 0};
                if (j == 0) {
                    const int8_t *qp = qs + (size_t)(b0 + i) * kBlockK + g * 16;
                    a0 = *reinterpret_cast<const v4i *>(qp);
                    a1 = *reinterpret_cast<const v4i *>(qp + 64);
                }
                v4i c = v4i{0, 0, 0, 0};
                c = mfma_i8(a0, decode16(cur.w[i].x), c);
                c = mfma_i8(a1, decode16(cur.w[i].y), c);
                yacc = fmaf(cur.s[i], (float)c[0], yacc);
            }
        }
        red[w * kWave + l] = yacc;
    }
    lds_barrier();

    // (5) wave 0 of each tile adds its waves' partials in wave order and stores the 16 rows
    if (active && wv == 0 && g == 0) {
        const int nblk = K >> 7;
        const int used = (nblk + L.per - 1) / L.per;
        float sum = 0.0f;
        for (int ww = 0; ww < used; ++ww) sum += red[(ti * L.nw + ww) * kWave + j];
        const float yv = sum * (s_a * 0.015625f);
        const int row = tile * (int)kTileN + j;
        if (li != a.withhold) {
            if (L.out_off < 0) a.y[row] = yv;
            else st_agent(reinterpret_cast<float *>(a.ws + L.out_off) + row, yv);
        }
    }
    return true;
}

__global__ __launch_bounds__(kPThreads) void chain_persistent_kernel(PArgs a) {
    __shared__ __align__(16) int8_t qs[kPMaxK];
    __shared__ float red[kPWaves * kWave];
    __shared__ uint32_t vote[2 * kPWaves];
    __shared__ float amax_part[kPWaves];
    for (int li = 0; li < a.n; ++li)
        if (!p_layer(a, li, qs, red, vote, amax_part)) return;
}

// Fills the workspace's layer buffers with the pending pattern and clears the status word.
__global__ void chain_persistent_fill(uint4 *p, size_t n16, int *status) {
    const uint4 v = make_uint4(kPending, kPending, kPending, kPending);
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
        p[i] = v;
    if (blockIdx.x == 0 && threadIdx.x == 0) *status = 0;
}

// Host side: geometry per layer and the workspace layout.
constexpr int kPTableAlign = 256;

bitnet_status_t persist_plan(const bitnet_chain_layer_t *layers, int n, int M, int xdt, int64_t cus, PLayer *out,
                             size_t *ws_bytes, int *grid) {
    if (!layers || n < 1) return BITNET_ERR_INVALID_ARG;
    if (M != 1) return BITNET_ERR_UNSUPPORTED_SHAPE;
    if (xdt != BITNET_DT_BF16 && xdt != BITNET_DT_F32) return BITNET_ERR_INVALID_ARG;
    ChainPlan cp;
    const bitnet_status_t st = chain_plan(layers, n, M, layers[0].K, &cp);
    if (st != BITNET_OK) return st;
    if (cus < 1) return BITNET_ERR_UNSUPPORTED_SHAPE;
    size_t off = kPTableAlign;  // the status word lives in the first 256 bytes
    int g = 0;
    for (int i = 0; i < n; ++i) {
        const bitnet_chain_layer_t &Lc = layers[i];
        PLayer p{};
        p.packed = Lc.packed;
        p.scales = Lc.scales;
        p.N = Lc.N;
        p.K = Lc.K;
        if (Lc.K > kPMaxK || (Lc.fold_input && Lc.K > kPMaxK / 2)) return BITNET_ERR_UNSUPPORTED_SHAPE;
        // weights and scales are read through 32-bit buffer ranges
        if ((size_t)Lc.N * Lc.K / 4 > (size_t)0x7FFFFFF0u) return BITNET_ERR_UNSUPPORTED_SHAPE;
        const int nblk = Lc.K / (int)kBlockK, tiles = Lc.N / (int)kTileN;
        p.tp = 0;
        for (int tp = 4; tp >= 1; tp >>= 1) {
            const int nw = kPWaves / tp, per = (nblk + nw - 1) / nw;
            const int64_t nwg = (tiles + tp - 1) / tp;
            if (per <= kPMaxNB && nwg <= cus) {
                p.tp = tp;
                p.nw = nw;
                p.per = per;
                p.nwg = (int)nwg;
                break;
            }
        }
        if (p.tp == 0) return BITNET_ERR_UNSUPPORTED_SHAPE;
        g = p.nwg > g ? p.nwg : g;
        if (i == 0) {
            p.xm = xdt == BITNET_DT_BF16 ? 0 : 1;
            p.in_off = -1;
        } else {
            p.xm = Lc.fold_input == BITNET_JUNCTION_SUM ? 5 : Lc.fold_input == BITNET_JUNCTION_RELU2_GLU ? 6 : 4;
            p.in_off = out[i - 1].out_off;
        }
        if (i == n - 1) {
            p.out_off = -1;
        } else {
            p.out_off = (int64_t)off;
            off += align256((size_t)Lc.N * sizeof(float));
        }
        out[i] = p;
    }
    *ws_bytes = off;
    *grid = g;
    return BITNET_OK;
}
}  // namespace

extern "C" {

size_t bitnet_w2a8_persist_table_bytes(int n) { return n < 1 ? 0 : (size_t)n * sizeof(PLayer); }

bitnet_status_t bitnet_w2a8_persist_prepare(const bitnet_chain_layer_t *layers, int n, int M, int xdt, int64_t cus,
                                            void *table_host, size_t table_bytes, size_t *workspace_bytes) {
    if (!table_host || !workspace_bytes || n < 1 || table_bytes < (size_t)n * sizeof(PLayer) || cus < 0)
        return BITNET_ERR_INVALID_ARG;
    if (cus == 0) {
        int dev = 0, c = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return BITNET_ERR_HIP;
        cus = c;
    }
    int grid = 0;
    return persist_plan(layers, n, M, xdt, cus, static_cast<PLayer *>(table_host), workspace_bytes, &grid);
}

bitnet_status_t bitnet_w2a8_chain_persistent_ex(const void *table_dev, int n, const void *x, int xdt, int M, float *y,
                                                void *workspace, size_t workspace_bytes, int spin_limit,
                                                int withhold_layer, hipStream_t stream) {
    if (!table_dev || n < 1 || !x || !y || !workspace || !aligned(table_dev, 16) || !aligned(x, 16) ||
        !aligned(y, 16) || !aligned(workspace, 256) || spin_limit < 0)
        return BITNET_ERR_INVALID_ARG;
    if (xdt != BITNET_DT_BF16 && xdt != BITNET_DT_F32) return BITNET_ERR_INVALID_ARG;
    if (M != 1) return BITNET_ERR_UNSUPPORTED_SHAPE;
    const DeviceSlots dev = device_slots(stream);
    if (dev.cus < 1) return BITNET_ERR_HIP;
    if (workspace_bytes < (size_t)kPTableAlign) return BITNET_ERR_INVALID_ARG;
    PArgs a;
    a.table = static_cast<const PLayer *>(table_dev);
    a.n = n;
    a.x = x;
    a.y = y;
    a.ws = static_cast<unsigned char *>(workspace);
    a.ws_bytes = (int64_t)workspace_bytes;
    a.status = reinterpret_cast<int *>(workspace);
    a.spin_limit = spin_limit > 0 ? spin_limit : (1 << 16);  // rounds of up to 64 polls: seconds
    a.withhold = withhold_layer;
    const size_t n16 = (workspace_bytes - kPTableAlign) / 16;
    hipLaunchKernelGGL(chain_persistent_fill, dim3(256), dim3(256), 0, stream,
                       reinterpret_cast<uint4 *>(a.ws + kPTableAlign), n16, a.status);
    // one workgroup per CU: every workgroup is resident at once, so every wait is on a
    // workgroup that is running
    hipLaunchKernelGGL(chain_persistent_kernel, dim3((unsigned)dev.cus), dim3(kPThreads), 0, stream, a);
    return launched();
}

bitnet_status_t bitnet_w2a8_chain_persistent(const void *table_dev, int n, const void *x, int xdt, int M, float *y,
                                             void *workspace, size_t workspace_bytes, hipStream_t stream) {
    return bitnet_w2a8_chain_persistent_ex(table_dev, n, x, xdt, M, y, workspace, workspace_bytes, 0, -1, stream);
}

}  // extern "C"
