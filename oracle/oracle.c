/*
 * CPU oracle for the BitNet b1.58 W2A8 ternary-weight x int8-activation product.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes or
 * calls this file; only the test-suite, the smoke check and the CPU-baseline leg
 * of the benchmark load it.  It shares no code, header, table or helper with the
 * HIP path.  Plain scalar loops, written to be checked by eye against the pages:
 *
 *   [P2] "5x performance leap: BitNet vs llama.cpp, 1-bit LLM inference
 *        architectures" (aicoding.csdn.net) -- section "Architecture
 *        foundations", item 2 (the W2A8 GEMV: 2-bit weights x 8-bit
 *        activations); section "GPU kernel breakthroughs" (A100 shapes).
 *   [P3] "Running 1-bit LLMs in the browser: BitNet + WebAssembly"
 *        (xdnf.cn) -- section "Why WASM" (ternary weights in {-1,0,1} from
 *        absmean quantisation) and section "What i2_s actually is" (the
 *        0/1/2 <-> -1/0/+1 code map, four codes per byte at shift 6-2*group,
 *        128-weight blocks on x86 each carrying one float scale, dequantise =
 *        lookup then scale).
 *
 * Where the pages leave a step open, the reading taken is stated at the
 * function (readings R1..R14 of the design notes).  Floating point is fp64
 * except where the method fixes fp32 (activation quantisation, ternarisation
 * ratio), where it is IEEE fp32 with round-to-nearest-even.
 *
 * Build: gcc -O1 -ffp-contract=off -fno-fast-math -shared -fPIC (see build.py).
 * All functions return 0 on success, a negative value on bad input.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>

#define ORACLE_BLOCK 128 /* [P3] "What i2_s actually is": x86 block of 128 weights */

/* ------------------------------------------------------------------------ */
/* a1. absmean ternarisation, per 128-weight block.                           */
/* [P3] "Why WASM": weights constrained to {-1,0,1} via absmean quantisation;  */
/* [P3] "What i2_s actually is": one float scale per 128-weight block.        */
/* Reading R3: gamma = mean |W| over the block (sum in fp64, in index order,  */
/* divided by 128, rounded once to fp32); T = clamp(rint_fp32(W / gamma),     */
/* -1, 1) with the ratio an IEEE fp32 division; scale = gamma; a block whose  */
/* gamma is 0 gives T = 0 and scale 0.                                         */
/* ------------------------------------------------------------------------ */
int oracle_ternarize_absmean(const float *W, int64_t N, int64_t K, int8_t *T, float *S)
{
    if (N <= 0 || K <= 0 || K % ORACLE_BLOCK) return -1;
    int64_t B = K / ORACLE_BLOCK;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t b = 0; b < B; ++b) {
            const float *w = W + n * K + b * ORACLE_BLOCK;
            double sum = 0.0;
            for (int i = 0; i < ORACLE_BLOCK; ++i) sum += fabs((double)w[i]);
            float gamma = (float)(sum / 128.0);
            S[n * B + b] = gamma;
            for (int i = 0; i < ORACLE_BLOCK; ++i) {
                int8_t t = 0;
                if (gamma != 0.0f) {
                    volatile float ratio = w[i] / gamma; /* fp32 division */
                    float r = rintf(ratio);             /* round half to even */
                    if (r > 1.0f) r = 1.0f;
                    if (r < -1.0f) r = -1.0f;
                    t = (int8_t)r;
                }
                T[n * K + b * ORACLE_BLOCK + i] = t;
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* a2. canonical i2_s pack / unpack.                                          */
/* [P3] "What i2_s actually is": code 1 for zero, 2 for positive, 0 for       */
/* negative; four codes per byte, 2 bits each, code placed at shift           */
/* (6 - 2*group_idx) (the shift operator is lost in the page's text).         */
/* Reading R5: group_idx g in 0..3 names the four 32-wide groups of a         */
/* 128-block, so byte j (0..31) of block b holds weights k = 128b + 32g + j,  */
/* g = 0 in bits 7..6.  Row stride is K/4 bytes (R1: blocks never straddle    */
/* rows).  Code 3 does not occur in valid data.                               */
/* ------------------------------------------------------------------------ */
int oracle_pack_i2s(const int8_t *T, int64_t N, int64_t K, uint8_t *P)
{
    if (N <= 0 || K <= 0 || K % ORACLE_BLOCK) return -1;
    int64_t B = K / ORACLE_BLOCK;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t b = 0; b < B; ++b) {
            for (int j = 0; j < 32; ++j) {
                unsigned byte = 0;
                for (int g = 0; g < 4; ++g) {
                    int t = T[n * K + b * ORACLE_BLOCK + 32 * g + j];
                    unsigned code;
                    if (t == 0) code = 1;
                    else if (t == 1) code = 2;
                    else if (t == -1) code = 0;
                    else return -2;
                    byte |= code << (6 - 2 * g);
                }
                P[n * (K / 4) + b * 32 + j] = (uint8_t)byte;
            }
        }
    }
    return 0;
}

/* Inverse of oracle_pack_i2s: t = code - 1. Returns -2 on code 3. */
int oracle_unpack_i2s(const uint8_t *P, int64_t N, int64_t K, int8_t *T)
{
    if (N <= 0 || K <= 0 || K % ORACLE_BLOCK) return -1;
    int64_t B = K / ORACLE_BLOCK;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t b = 0; b < B; ++b) {
            for (int j = 0; j < 32; ++j) {
                unsigned byte = P[n * (K / 4) + b * 32 + j];
                for (int g = 0; g < 4; ++g) {
                    unsigned code = (byte >> (6 - 2 * g)) & 3u;
                    if (code == 3) return -2;
                    T[n * K + b * ORACLE_BLOCK + 32 * g + j] = (int8_t)((int)code - 1);
                }
            }
        }
    }
    return 0;
}

/* One weight read straight out of canonical i2_s bytes (scalar unpack). */
static int i2s_weight(const uint8_t *P, int64_t K, int64_t n, int64_t k)
{
    int64_t b = k / ORACLE_BLOCK;
    int64_t r = k % ORACLE_BLOCK;
    int64_t g = r / 32, j = r % 32;
    unsigned byte = P[n * (K / 4) + b * 32 + j];
    return (int)((byte >> (6 - 2 * g)) & 3u) - 1;
}

/* ------------------------------------------------------------------------ */
/* a4. per-token absmax int8 activation quantisation.                         */
/* [P2] "Architecture foundations", item 2: activations are 8-bit.  The pages */
/* do not print the quantiser; reading R6: per token, amax = max |x|,         */
/* amax_c = max(amax, 1e-5); inv = 127 / amax_c (fp32, correctly rounded);    */
/* q = clamp(rint(x * inv), -127, 127) with the product in fp32;              */
/* dequantisation factor s_a = amax_c / 127 (fp32).                           */
/* ------------------------------------------------------------------------ */
int oracle_quant_act_f32(const float *x, int64_t M, int64_t K, int8_t *q, float *s_a)
{
    if (M <= 0 || K <= 0) return -1;
    for (int64_t m = 0; m < M; ++m) {
        const float *xr = x + m * K;
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float a = fabsf(xr[k]);
            if (a > amax) amax = a;
        }
        float amax_c = amax > 1e-5f ? amax : 1e-5f;
        volatile float inv = 127.0f / amax_c;
        for (int64_t k = 0; k < K; ++k) {
            volatile float v = xr[k] * inv;
            float r = rintf(v);
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
            q[m * K + k] = (int8_t)r;
        }
        volatile float sa = amax_c / 127.0f;
        s_a[m] = sa;
    }
    return 0;
}

/* bf16 input: each value widened exactly to fp32 (bits << 16), then as above. */
int oracle_quant_act_bf16(const uint16_t *x, int64_t M, int64_t K, int8_t *q, float *s_a, float *scratch)
{
    if (M <= 0 || K <= 0) return -1;
    for (int64_t i = 0; i < M * K; ++i) {
        union { uint32_t u; float f; } cv;
        cv.u = (uint32_t)x[i] << 16;
        scratch[i] = cv.f;
    }
    return oracle_quant_act_f32(scratch, M, K, q, s_a);
}

/* ------------------------------------------------------------------------ */
/* a5/a6. the W2A8 product.                                                   */
/* [P2] "Architecture foundations", item 2 (2-bit weights x 8-bit            */
/* activations); [P3] "What i2_s actually is" (per-block float scale,         */
/* dequantise = lookup then scale, no float matmul).  Reading R2: per block   */
/* an int32 sum A[m,n,b] = sum_k T[n,k] Q[m,k]; the exact integer result is   */
/* acc[m,n] = sum_b A[m,n,b]; the real output is                              */
/* y[m,n] = s_a[m] * sum_b S[n,b] * A[m,n,b], here in fp64.                    */
/* Outputs: acc (int32), y64 (fp64 value), y (y64 rounded once to fp32) and   */
/* mag = s_a[m] * sum_b |S[n,b] * A[m,n,b]| (the size that bounds the         */
/* rounding error of any fp32 evaluation order).  Any pointer may be NULL.    */
/* ------------------------------------------------------------------------ */
int oracle_w2a8(const uint8_t *P, const float *S, const int8_t *Q, const float *s_a,
                int64_t M, int64_t N, int64_t K,
                int32_t *acc, double *y64, float *y, double *mag)
{
    if (M <= 0 || N <= 0 || K <= 0 || K % ORACLE_BLOCK) return -1;
    int64_t B = K / ORACLE_BLOCK;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            int32_t total = 0;
            double sum = 0.0, msum = 0.0;
            for (int64_t b = 0; b < B; ++b) {
                int32_t a = 0;
                for (int64_t i = 0; i < ORACLE_BLOCK; ++i) {
                    int64_t k = b * ORACLE_BLOCK + i;
                    a += i2s_weight(P, K, n, k) * (int32_t)Q[m * K + k];
                }
                total += a;
                double term = (double)S[n * B + b] * (double)a;
                sum += term;
                msum += fabs(term);
            }
            double yv = (double)s_a[m] * sum;
            if (acc) acc[m * N + n] = total;
            if (y64) y64[m * N + n] = yv;
            if (y) y[m * N + n] = (float)yv;
            if (mag) mag[m * N + n] = (double)s_a[m] * msum;
        }
    }
    return 0;
}

/* Exact integer product only, straight from a dense ternary matrix
 * T [N][K] (no packing): acc[m,n] = sum_k T[n,k] Q[m,k]. */
int oracle_acc_dense(const int8_t *T, const int8_t *Q, int64_t M, int64_t N, int64_t K, int32_t *acc)
{
    if (M <= 0 || N <= 0 || K <= 0) return -1;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            int32_t s = 0;
            for (int64_t k = 0; k < K; ++k) s += (int32_t)T[n * K + k] * (int32_t)Q[m * K + k];
            acc[m * N + n] = s;
        }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* bf16 output of the prefill product: round-to-nearest-even of an fp32      */
/* value (reading R8).  Returns the bf16 bit pattern.  NaN is not produced   */
/* by finite inputs and is not handled.                                       */
/* ------------------------------------------------------------------------ */
int oracle_f32_to_bf16(const float *x, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) {
        union { float f; uint32_t u; } cv;
        cv.f = x[i];
        uint32_t u = cv.u;
        uint32_t lsb = (u >> 16) & 1u;
        u += 0x7FFFu + lsb;
        out[i] = (uint16_t)(u >> 16);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* a7. junction of the stacked decode chain (reading R10): the fused          */
/* gate+up output y [M][2H] is folded to h[m][j] = y[m][j] + y[m][H + j]      */
/* (one fp32 addition), then re-quantised per token as in a4.                 */
/* ------------------------------------------------------------------------ */
int oracle_fold_quant(const float *y, int64_t M, int64_t H, int8_t *q, float *s_a, float *scratch)
{
    if (M <= 0 || H <= 0) return -1;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t j = 0; j < H; ++j) {
            volatile float h = y[m * 2 * H + j] + y[m * 2 * H + H + j];
            scratch[m * H + j] = h;
        }
    return oracle_quant_act_f32(scratch, M, H, q, s_a);
}

/* ------------------------------------------------------------------------ */
/* a7 variant: squared-ReLU gated junction.                                   */
/* [P4] "BitRun v0.2 measured", section "Architecture-specific SIMD           */
/* acceleration": the runtime pairs its ternary dot-product kernels with a    */
/* squared-ReLU activation.  Reading: the fused gate+up output y [M][2H]      */
/* carries the gate in its first H columns and the up projection in the      */
/* last H; the next layer's input is h = relu(gate)^2 * up, evaluated in fp32 */
/* as r = max(gate, 0), then (r * r), then that times up (two roundings, no   */
/* fused multiply-add), then re-quantised per token as in a4.                 */
/* ------------------------------------------------------------------------ */
int oracle_glu_quant(const float *y, int64_t M, int64_t H, int8_t *q, float *s_a, float *scratch)
{
    if (M <= 0 || H <= 0) return -1;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t j = 0; j < H; ++j) {
            const float gate = y[m * 2 * H + j];
            const float up = y[m * 2 * H + H + j];
            const float r = gate > 0.0f ? gate : 0.0f;
            volatile float r2 = r * r;
            volatile float h = r2 * up;
            scratch[m * H + j] = h;
        }
    return oracle_quant_act_f32(scratch, M, H, q, s_a);
}

/* ------------------------------------------------------------------------ */
/* Format variants: the scale granularity G.                                  */
/* [P3] "What i2_s actually is": blocks of 128 weights on x86 and of 64 on    */
/* ARM, each block carrying one float scale.  G = 128 is the x86 format of    */
/* the functions above; G = 64 is the ARM block; G = 0 is one scale for the   */
/* whole matrix (the reading in which the scale is applied once, after the    */
/* whole integer sum).  Readings: with G = 64 the canonical bytes of a block  */
/* hold its 64 weights as four 16-wide groups (byte j of block b holds        */
/* k = 64b + 16g + j, g = 0 in bits 7..6), the 128-block rule scaled down;    */
/* with G = 0 the canonical bytes use the 128 layout, gamma is the mean |W|   */
/* over the whole matrix (fp64 sum in row-major index order, divided by N*K,  */
/* rounded once to fp32), and y = s_a * (S * acc) in fp64, rounded once.      */
/* ------------------------------------------------------------------------ */
static int64_t canon_block(int G) { return G == 64 ? 64 : 128; }
static int gran_ok(int G) { return G == 0 || G == 64 || G == 128; }

static int8_t ternary_of(float w, float gamma)
{
    if (gamma == 0.0f) return 0;
    volatile float ratio = w / gamma;
    float r = rintf(ratio);
    if (r > 1.0f) r = 1.0f;
    if (r < -1.0f) r = -1.0f;
    return (int8_t)r;
}

int oracle_ternarize_absmean_g(const float *W, int64_t N, int64_t K, int G, int8_t *T, float *S)
{
    if (!gran_ok(G) || N <= 0 || K <= 0 || K % canon_block(G)) return -1;
    if (G == 0) {
        double sum = 0.0;
        for (int64_t i = 0; i < N * K; ++i) sum += fabs((double)W[i]);
        float gamma = (float)(sum / (double)(N * K));
        S[0] = gamma;
        for (int64_t i = 0; i < N * K; ++i) T[i] = ternary_of(W[i], gamma);
        return 0;
    }
    int64_t B = K / G;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t b = 0; b < B; ++b) {
            const float *w = W + n * K + b * G;
            double sum = 0.0;
            for (int64_t i = 0; i < G; ++i) sum += fabs((double)w[i]);
            float gamma = (float)(sum / (double)G);
            S[n * B + b] = gamma;
            for (int64_t i = 0; i < G; ++i) T[n * K + b * G + i] = ternary_of(w[i], gamma);
        }
    return 0;
}

int oracle_pack_i2s_g(const int8_t *T, int64_t N, int64_t K, int G, uint8_t *P)
{
    if (!gran_ok(G) || N <= 0 || K <= 0 || K % canon_block(G)) return -1;
    const int64_t cb = canon_block(G), gw = cb / 4;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t b = 0; b < K / cb; ++b)
            for (int64_t j = 0; j < gw; ++j) {
                unsigned byte = 0;
                for (int g = 0; g < 4; ++g) {
                    int t = T[n * K + b * cb + gw * g + j];
                    if (t < -1 || t > 1) return -2;
                    byte |= (unsigned)(t + 1) << (6 - 2 * g);
                }
                P[n * (K / 4) + b * gw + j] = (uint8_t)byte;
            }
    return 0;
}

int oracle_unpack_i2s_g(const uint8_t *P, int64_t N, int64_t K, int G, int8_t *T)
{
    if (!gran_ok(G) || N <= 0 || K <= 0 || K % canon_block(G)) return -1;
    const int64_t cb = canon_block(G), gw = cb / 4;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t b = 0; b < K / cb; ++b)
            for (int64_t j = 0; j < gw; ++j) {
                unsigned byte = P[n * (K / 4) + b * gw + j];
                for (int g = 0; g < 4; ++g) {
                    unsigned code = (byte >> (6 - 2 * g)) & 3u;
                    if (code == 3) return -2;
                    T[n * K + b * cb + gw * g + j] = (int8_t)((int)code - 1);
                }
            }
    return 0;
}

static int i2s_weight_g(const uint8_t *P, int64_t K, int G, int64_t n, int64_t k)
{
    const int64_t cb = canon_block(G), gw = cb / 4;
    int64_t b = k / cb, r = k % cb;
    unsigned byte = P[n * (K / 4) + b * gw + r % gw];
    return (int)((byte >> (6 - 2 * (r / gw))) & 3u) - 1;
}

/* The product with scale granularity G; scales S are [N][K/G] row-major, or  */
/* one value when G = 0.  Outputs as oracle_w2a8.                             */
int oracle_w2a8_g(const uint8_t *P, const float *S, const int8_t *Q, const float *s_a,
                  int64_t M, int64_t N, int64_t K, int G,
                  int32_t *acc, double *y64, float *y, double *mag)
{
    if (!gran_ok(G) || M <= 0 || N <= 0 || K <= 0 || K % canon_block(G)) return -1;
    const int64_t blk = G == 0 ? K : G, B = K / blk;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            int32_t total = 0;
            double sum = 0.0, msum = 0.0;
            for (int64_t b = 0; b < B; ++b) {
                int32_t a = 0;
                for (int64_t i = 0; i < blk; ++i) {
                    int64_t k = b * blk + i;
                    a += i2s_weight_g(P, K, G, n, k) * (int32_t)Q[m * K + k];
                }
                total += a;
                double term = (double)(G == 0 ? S[0] : S[n * B + b]) * (double)a;
                sum += term;
                msum += fabs(term);
            }
            double yv = (double)s_a[m] * sum;
            if (acc) acc[m * N + n] = total;
            if (y64) y64[m * N + n] = yv;
            if (y) y[m * N + n] = (float)yv;
            if (mag) mag[m * N + n] = (double)s_a[m] * msum;
        }
    return 0;
}
