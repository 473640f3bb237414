/*
 * bitnet_w2a8.h -- C ABI of the MI355X (gfx950) W2A8 ternary product library.
 *
 * The operation (BitNet b1.58 linear layer, "W2A8"):
 *   weights T[N][K] in {-1,0,+1} with one fp32 scale S[n][b] per 128-weight
 *   block b of a row, activations quantised per token to int8 Q[M][K] with a
 *   dequantisation factor s_a[m], and
 *       y[m][n] = s_a[m] * sum_b S[n][b] * sum_{k in block b} T[n][k] * Q[m][k]
 *   with the inner sums exact in int32.
 * Sources (page, section):
 *   [P2] "5x performance leap: BitNet vs llama.cpp 1-bit LLM inference" --
 *        "Architecture foundations", item 2: a W2A8 GEMV (2-bit weights x
 *        8-bit activations); "GPU kernel breakthroughs": offline weight
 *        reordering for memory access, 8-bit dot products, and an
 *        interleaved 16-codes-per-32-bit-word order that makes decoding cheap.
 *   [P3] "Running 1-bit LLMs in the browser: BitNet + WebAssembly" --
 *        "Why WASM": ternary weights from absmean quantisation;
 *        "What i2_s actually is": code 0/1/2 for -1/0/+1, four codes per byte,
 *        128-weight blocks with one float scale each.
 *   [P4] "BitRun v0.2 measured" -- "Matrix memory bounds and stride safety":
 *        packed rows must have one stride rule shared by reader and kernel;
 *        here bitnet_packed_bytes() is that single authority.
 *
 * Conventions for every entry point
 *   - Return value: bitnet_status_t.  Arguments are validated synchronously,
 *     before any HIP call; an invalid call returns an error and launches
 *     nothing.  Device entry points enqueue work on `stream` and return
 *     without synchronising; a launch failure is reported as BITNET_ERR_HIP.
 *     No C++ exception crosses this interface.
 *   - Ownership: the caller owns every buffer.  The library allocates no
 *     memory and is re-entrant; the only state it keeps between calls is a
 *     cache of each device's CU count and wave slots, read on first use, and
 *     the fixed per-GPU workspace array of bitnet_w2a8_chain_static (whose
 *     device address is looked up on first use).
 *   - "device" pointers are HIP device memory, 16-byte aligned; "host"
 *     pointers are ordinary host memory.  Non-finite inputs are outside the
 *     contract.
 *   - Shapes: K % 128 == 0 (blocks never straddle rows), N % 16 == 0,
 *     N, K >= the block/tile size, and N*K < 2^40.
 *
 * gfx950 tile layout of packed weights ("packed", N*K/4 bytes)
 *   Rows are grouped in tiles of 16 (T = n / 16), K in blocks of 128
 *   (b = k / 128).  Brick (T, b) is 512 bytes at byte offset
 *   (T * (K/128) + b) * 512.  Slot l = 16*g + j (g in 0..3, j in 0..15) of a
 *   brick is 8 bytes at offset 8*l: two little-endian 32-bit words w_s
 *   (s = 0, 1) for row n = 16*T + j and the 16 weights starting at
 *   k0 = 128*b + 64*s + 16*g.  Bits 8p+2i .. 8p+2i+1 of w_s (byte p, field i,
 *   p, i in 0..3) hold weight k0 + 4*i + p as a 2-bit two's-complement code
 *   (0 -> 0, +1 -> 1, -1 -> 3).  This puts the 16 codes one wavefront lane
 *   needs for one int8 matrix-core step in one word, and one shift and one
 *   mask turn field i of all four bytes into four consecutive int8 weights
 *   (times 64) -- the same idea as the interleaved word order of [P2].
 * Tiled scales ("scales_tiled", N*K/128 fp32): the scale of row 16*T + j,
 *   block b sits at index (T * (K/128) + b) * 16 + j.
 * Canonical i2_s bytes (interchange, [P3]; reading of the garbled shift):
 *   row n occupies K/4 bytes; byte j (0..31) of block b holds weights
 *   128b + 32g + j for g = 0..3 at bits (7-2g)..(6-2g), code = t + 1.
 */
#ifndef BITNET_W2A8_H
#define BITNET_W2A8_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    BITNET_OK = 0,
    BITNET_ERR_INVALID_ARG = 1,       /* null / misaligned pointer, bad dtype, non-ternary input */
    BITNET_ERR_UNSUPPORTED_SHAPE = 2, /* shape outside the rules above */
    BITNET_ERR_HIP = 3                /* a HIP launch or runtime call failed */
} bitnet_status_t;

typedef enum {
    BITNET_DT_BF16 = 0,      /* bfloat16 */
    BITNET_DT_F32 = 1,       /* fp32 */
    BITNET_DT_F32_FOLD2 = 2, /* fp32 [M][2K] read as h = x[:, :K] + x[:, K:] (one fp32 add) */
    BITNET_DT_F32_RELU2_GLU = 3 /* fp32 [M][2K] read as h = relu(x[:, :K])^2 * x[:, K:]
                                   (fp32: r = max(x, 0), then r * r, then times the second
                                   half; two roundings, no fused multiply-add) */
} bitnet_dtype_t;

/* Junction between layers of a decode chain (bitnet_chain_layer_t.fold_input). */
typedef enum {
    BITNET_JUNCTION_NONE = 0,     /* input = previous output [M][K] */
    BITNET_JUNCTION_SUM = 1,      /* previous output [M][2K]; input = lo + hi */
    BITNET_JUNCTION_RELU2_GLU = 2 /* previous output [M][2K] = (gate | up); input = relu(gate)^2 * up */
} bitnet_junction_t;

/* Human-readable name of a status code (static string, never NULL). */
const char *bitnet_status_str(int status);

/* Checks (N, K) against the shape rules; BITNET_OK or BITNET_ERR_UNSUPPORTED_SHAPE. */
bitnet_status_t bitnet_check_shape(int64_t N, int64_t K);

/* Bytes of a packed weight buffer, N*K/4 (the only size/stride authority);
 * 0 if the shape is unsupported. */
size_t bitnet_packed_bytes(int64_t N, int64_t K);

/* Number of fp32 block scales, N*K/128; 0 if the shape is unsupported. */
size_t bitnet_scale_count(int64_t N, int64_t K);

/* ---------------------------------------------------------------- offline, host */

/* absmean ternarisation per 128-weight block ([P3] "Why WASM" names absmean;
 * [P3] "What i2_s actually is" gives the 128-block float scale).  For every row
 * n and block b: gamma = (sum of |w| over the block in fp64, in index order) /
 * 128 rounded to fp32; t = clamp(rint(w / gamma), -1, 1) with the ratio an fp32
 * division (round half to even); scale = gamma; gamma == 0 gives t = 0.
 *   w        host, fp32 [N][K] row-major (in)
 *   ternary  host, int8 [N][K] row-major (out), values in {-1,0,1}
 *   scales   host, fp32 [N][K/128] row-major (out) */
bitnet_status_t bitnet_ternarize_absmean(const float *w, int64_t N, int64_t K,
                                         int8_t *ternary, float *scales);

/* Packs a ternary matrix into the gfx950 tile layout (the offline reorder of
 * [P2] "GPU kernel breakthroughs", re-designed for 64-wide wavefronts).
 *   ternary       host, int8 [N][K] row-major, each value in {-1,0,1}
 *                 (anything else -> BITNET_ERR_INVALID_ARG, nothing written)
 *   scales        host, fp32 [N][K/128] row-major block scales
 *   packed_out    host, bitnet_packed_bytes(N,K) bytes, tile layout
 *   scales_out    host, bitnet_scale_count(N,K) fp32, tiled scale order */
bitnet_status_t bitnet_pack_i2s(const int8_t *ternary, const float *scales, int64_t N, int64_t K,
                                uint8_t *packed_out, float *scales_out);

/* Same as bitnet_pack_i2s, reading canonical i2_s bytes (host, uint8
 * [N][K/4], [P3] code map; code 3 -> BITNET_ERR_INVALID_ARG). */
bitnet_status_t bitnet_repack_i2s(const uint8_t *i2s, const float *scales, int64_t N, int64_t K,
                                  uint8_t *packed_out, float *scales_out);

/* Inverse of bitnet_pack_i2s (host): tile layout -> ternary int8 [N][K] and
 * row-major scales [N][K/128].  scales_tiled / scales_out may both be NULL. */
bitnet_status_t bitnet_unpack_i2s(const uint8_t *packed, const float *scales_tiled, int64_t N, int64_t K,
                                  int8_t *ternary_out, float *scales_out);

/* ---------------------------------------------------------------- format variants, host */

/* Scale granularity ([P3] "What i2_s actually is": blocks of 128 weights on x86
 * and of 64 on ARM, one float scale per block): scale_block = 128 (the format of
 * every function without the _g suffix), 64, or 0 for one fp32 scale for the
 * whole matrix (the reading in which the scale multiplies the complete integer
 * sum once).  The packed 2-bit tile layout is the same for all three; only the
 * scales differ.  Tiled scale order: 128: [tile][block][16 rows]; 64: [tile]
 * [128-block][16 rows][2 halves] (half h covers weights 128b + 64h .. +63);
 * 0: the one value.  A scale_block outside {0, 64, 128} gives
 * BITNET_ERR_INVALID_ARG (or 0 from bitnet_scale_count_g). */

/* Number of fp32 scales: N*K/scale_block, 1 for scale_block 0; 0 if the shape
 * or scale_block is unsupported. */
size_t bitnet_scale_count_g(int64_t N, int64_t K, int scale_block);

/* absmean ternarisation at granularity scale_block: per block of 64 or 128
 * weights as bitnet_ternarize_absmean; for 0, gamma = (sum of |w| over the whole
 * matrix in fp64, row-major order) / (N*K) rounded to fp32, scales[0] = gamma.
 *   scales  host, fp32 [N][K/scale_block] row-major, or one value (out) */
bitnet_status_t bitnet_ternarize_absmean_g(const float *w, int64_t N, int64_t K, int scale_block,
                                           int8_t *ternary, float *scales);

/* bitnet_pack_i2s with scales [N][K/scale_block] row-major (one value for 0);
 * scales_out holds bitnet_scale_count_g(N, K, scale_block) fp32. */
bitnet_status_t bitnet_pack_i2s_g(const int8_t *ternary, const float *scales, int64_t N, int64_t K,
                                  int scale_block, uint8_t *packed_out, float *scales_out);

/* bitnet_repack_i2s for canonical bytes of the given format: for scale_block 64
 * byte j of 64-block b holds weights 64b + 16g + j (g = 0 in bits 7..6; the
 * 128-block rule scaled to 64 weights, a reading); for 128 and 0 the 128-block
 * canonical bytes. */
bitnet_status_t bitnet_repack_i2s_g(const uint8_t *i2s, const float *scales, int64_t N, int64_t K,
                                    int scale_block, uint8_t *packed_out, float *scales_out);

/* Inverse of bitnet_pack_i2s_g (host). */
bitnet_status_t bitnet_unpack_i2s_g(const uint8_t *packed, const float *scales_tiled, int64_t N, int64_t K,
                                    int scale_block, int8_t *ternary_out, float *scales_out);

/* ---------------------------------------------------------------- device, async */

/* Per-token absmax int8 quantisation of activations ([P2] "Architecture
 * foundations": 8-bit activations; the quantiser itself is a reading): per
 * token m, amax = max_k |x|, amax_c = max(amax, 1e-5), inv = 127/amax_c (fp32,
 * correctly rounded), q = clamp(rint(x * inv), -127, 127) (fp32 product, half to
 * even), s_a[m] = amax_c / 127.
 *   x    device, [M][K] row-major, dtype xdt (BITNET_DT_BF16 or BITNET_DT_F32)
 *   q    device, int8 [M][K] (out)
 *   s_a  device, fp32 [M] (out)
 * Rules: M >= 1, K >= 1, K % 16 == 0. */
bitnet_status_t bitnet_quant_act(const void *x, int xdt, int M, int K, int8_t *q, float *s_a,
                                 hipStream_t stream);

/* Junction of a stacked decode chain: h[m][j] = y[m][j] + y[m][H + j] (one fp32
 * addition; fused gate+up output folded to the down-projection width), then
 * quantised exactly as bitnet_quant_act does.
 *   y    device, fp32 [M][2H];  q device int8 [M][H];  s_a device fp32 [M].
 * Rules: M >= 1, H % 16 == 0. */
bitnet_status_t bitnet_quant_act_fold(const float *y, int M, int H, int8_t *q, float *s_a,
                                      hipStream_t stream);

/* Squared-ReLU gated junction ([P4] "BitRun v0.2 measured" -- "Architecture-
 * specific SIMD acceleration" pairs the ternary kernels with a squared-ReLU
 * activation; the gated form and the half order are a reading): the fused
 * gate+up output y [M][2H] carries the gate in columns [0, H) and the up
 * projection in [H, 2H); h[m][j] = relu(y[m][j])^2 * y[m][H + j] in fp32 (two
 * roundings), then quantised exactly as bitnet_quant_act does.
 *   y    device, fp32 [M][2H];  q device int8 [M][H];  s_a device fp32 [M].
 * Rules: M >= 1, H % 16 == 0.  Non-finite values are outside the contract. */
bitnet_status_t bitnet_quant_act_relu2_glu(const float *y, int M, int H, int8_t *q, float *s_a,
                                           hipStream_t stream);

/* Decode product, batch 1..16 (the W2A8 GEMV of [P2] "Architecture
 * foundations", item 2), on the gfx950 int8 matrix cores.
 *   packed  device, tile layout, bitnet_packed_bytes(N,K) bytes
 *   scales  device, tiled scales, bitnet_scale_count(N,K) fp32
 *   q       device, int8 [M][K];  s_a device, fp32 [M]
 *   y       device, fp32 [M][N] (out)
 * Rules: 1 <= M <= 16 and the shape rules.  The fp32 epilogue's summation order
 * is unspecified: y agrees with the exact value within 1e-5 of
 * max(|y|, s_a * sum_b |S*A|).  The split of K over waves, and with it the
 * order, depends on the shape and on the device's CU count and wave slots, so
 * on one device the result of a shape is always the same. */
bitnet_status_t bitnet_w2a8_gemv(const uint8_t *packed, const float *scales, const int8_t *q,
                                 const float *s_a, float *y, int M, int N, int K, hipStream_t stream);

/* Split-K geometry of the decode products (bitnet_w2a8_gemv[_g], bitnet_w2a8_gemv_act and
 * the chain) for an N x K weight matrix on a device with `cus` compute units that hold
 * `wave_slots` waves at once (0 and 0: unknown, the base split): the waves per 16-row
 * workgroup and the 128-weight blocks each wave sums.  The geometry fixes the fp32
 * summation order of y.  Host only, makes no HIP call.
 *   waves, blocks_per_wave  host, one int each (out)
 * Rules: the shape rules (else UNSUPPORTED_SHAPE); non-null outputs and cus,
 * wave_slots >= 0 (else INVALID_ARG). */
bitnet_status_t bitnet_gemv_split(int N, int K, int64_t cus, int64_t wave_slots, int *waves,
                                  int *blocks_per_wave);

/* Decode step in one launch: quantise the activations exactly as
 * bitnet_quant_act does (per-token absmax, fp32, half to even) and multiply, as
 * bitnet_w2a8_gemv does.  Each workgroup derives the same int8 values and
 * factors, so y equals bitnet_quant_act followed by bitnet_w2a8_gemv.
 *   x        device, xdt BITNET_DT_BF16 or BITNET_DT_F32: [M][K];
 *            BITNET_DT_F32_FOLD2: fp32 [M][2K], quantised input h = x[:, :K] + x[:, K:]
 *            (the junction of a stacked decode chain, as bitnet_quant_act_fold);
 *            BITNET_DT_F32_RELU2_GLU: fp32 [M][2K], quantised input
 *            h = relu(x[:, :K])^2 * x[:, K:] (as bitnet_quant_act_relu2_glu)
 *   y        device, fp32 [M][N] (out)
 *   q_out    device, int8 [M][K] (out, optional: NULL to skip)
 *   s_a_out  device, fp32 [M] (out, optional: NULL to skip)
 *   packed, scales as bitnet_w2a8_gemv.
 * Rules: 1 <= M <= 16, the shape rules, K <= 12288 and M*(K+16) <= 65280 (the int8
 * copy of the activations lives in LDS); otherwise BITNET_ERR_UNSUPPORTED_SHAPE
 * and the caller uses bitnet_quant_act + bitnet_w2a8_gemv. */
bitnet_status_t bitnet_w2a8_gemv_act(const uint8_t *packed, const float *scales, const void *x, int xdt,
                                     float *y, int8_t *q_out, float *s_a_out, int M, int N, int K,
                                     hipStream_t stream);

/* Prefill product for any M >= 1 on the int8 matrix cores; y is [M][N] in
 * dtype ydt (BITNET_DT_BF16: fp32 value rounded to nearest even; or
 * BITNET_DT_F32).  Arguments otherwise as bitnet_w2a8_gemv. */
bitnet_status_t bitnet_w2a8_gemm(const uint8_t *packed, const float *scales, const int8_t *q,
                                 const float *s_a, void *y, int ydt, int M, int N, int K,
                                 hipStream_t stream);

/* bitnet_w2a8_gemv / bitnet_w2a8_gemm at scale granularity scale_block (tiled
 * scales from bitnet_pack_i2s_g).  For 64: y = s_a * sum over 64-blocks of
 * S * A (fp32, order unspecified, same tolerance as bitnet_w2a8_gemv).  For 0:
 * the exact int32 sum over all of K, converted to fp32 and multiplied by
 * (s_a * S) (two fp32 roundings).  Rules: as the 128 versions; scale_block 0
 * also needs K <= 262144. */
bitnet_status_t bitnet_w2a8_gemv_g(const uint8_t *packed, const float *scales, const int8_t *q,
                                   const float *s_a, float *y, int M, int N, int K, int scale_block,
                                   hipStream_t stream);
bitnet_status_t bitnet_w2a8_gemm_g(const uint8_t *packed, const float *scales, const int8_t *q,
                                   const float *s_a, void *y, int ydt, int M, int N, int K, int scale_block,
                                   hipStream_t stream);

/* One layer of a chain of products (see bitnet_w2a8_chain). */
typedef struct {
    const uint8_t *packed;  /* device, tile layout of an N x K ternary matrix */
    const float *scales;    /* device, tiled block scales */
    int N, K;
    int fold_input;         /* a bitnet_junction_t: 0 the input is the previous output [M][K];
                               1 the previous output is [M][2K] and the input is
                               h = prev[:, :K] + prev[:, K:]; 2 the input is
                               h = relu(prev[:, :K])^2 * prev[:, K:] */
} bitnet_chain_layer_t;

/* Workspace bytes bitnet_w2a8_chain needs for these layers at batch M (0 if the
 * chain is invalid): two fp32 [M][max N] activation buffers, int8 [M][max K] and
 * fp32 [M] for the quantised activations. */
size_t bitnet_w2a8_chain_workspace_bytes(const bitnet_chain_layer_t *layers, int n, int M);

/* Decode pass through a stack of n W2A8 linear layers: layer i quantises its
 * input per token exactly as bitnet_quant_act (or bitnet_quant_act_fold when
 * fold_input 1, bitnet_quant_act_relu2_glu when 2) and multiplies as
 * bitnet_w2a8_gemv; its fp32 output is the next
 * layer's input.  This is the chained decode of a BitNet model's linear layers
 * ([P2] "Architecture foundations": W2A8 products; [P3] "Why WASM": a 2.4B ternary
 * model), with the fused gate+up output brought to the down-projection width
 * by the linear fold or the squared-ReLU gate.  One launch per layer
 * (re-quantisation fused into the product) when M <= 2, or M <= 4 for a layer
 * without a junction in front whose grid is small against the device (M times
 * its waves at most twice the device's wave slots); else two.  Results are the
 * same either way.
 * A fold_input outside 0..2 gives BITNET_ERR_INVALID_ARG.
 *   layers     host array of n descriptors (device pointers inside)
 *   x          device, [M][layers[0].K], xdt BITNET_DT_BF16 or BITNET_DT_F32
 *   y          device, fp32 [M][layers[n-1].N] (out)
 *   workspace  device, >= bitnet_w2a8_chain_workspace_bytes(layers, n, M), 256-byte aligned;
 *              clobbered
 * Rules: 1 <= M <= 16; each layer's shape follows the shape rules; K of layer i
 * equals N of layer i-1 (or half of it when fold_input); layer 0 has fold_input 0.
 * Enqueues everything on `stream` (capturable in a HIP graph); no allocation. */
bitnet_status_t bitnet_w2a8_chain(const bitnet_chain_layer_t *layers, int n, const void *x, int xdt, int M,
                                  float *y, void *workspace, size_t workspace_bytes, hipStream_t stream);

/* bitnet_w2a8_chain for callers that cannot allocate device memory -- code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation: the same launches
 * and results as bitnet_w2a8_chain, with the workspace in a fixed array the library holds
 * on each GPU (bitnet_w2a8_chain_static_max_bytes() = 4 MiB, kept until the process ends)
 * instead of a caller buffer.  Calls no allocating routine.  The first call on a device
 * looks up the array's device address (with that device made current for the lookup and
 * the caller's current device restored).  Every call on one GPU uses the same array, so
 * calls that overlap in time on one GPU (different streams, or host threads) race and
 * give undefined results; calls ordered on one stream are safe.  Nothing in the array
 * needs to start at zero: every intermediate value is written before it is read.
 *   layers, n, x, xdt, M, y   as bitnet_w2a8_chain
 * Rules: as bitnet_w2a8_chain, and bitnet_w2a8_chain_workspace_bytes(layers, n, M) at most
 * bitnet_w2a8_chain_static_max_bytes() (else BITNET_ERR_UNSUPPORTED_SHAPE, no launch). */
size_t bitnet_w2a8_chain_static_max_bytes(void);
bitnet_status_t bitnet_w2a8_chain_static(const bitnet_chain_layer_t *layers, int n, const void *x, int xdt, int M,
                                         float *y, hipStream_t stream);

/* The decode pass of bitnet_w2a8_chain at batch 1 as ONE launch (a persistent form, an
 * experiment beside the launch-per-layer chain): the same operation ([P2] "Architecture
 * foundations": W2A8 products; [P3] "Why WASM": a 2.4B ternary model decoded token by
 * token; the junctions of [P4] "BitRun v0.2 measured"), the same per-layer arithmetic
 * (quantisation exactly as bitnet_quant_act / _fold / _relu2_glu, int32 block sums, one
 * fp32 scale per block), within the fp32 bound of the products called one by one.  One
 * 1024-thread workgroup per compute unit runs every layer; a layer's output goes to the
 * workspace with device-coherent stores and the next layer's workgroups poll it (each
 * value starts as a pending pattern), so no launch separates the layers.  Every wait is
 * bounded: a wait that gives up records its layer in the workspace's status word and its
 * workgroup ends, so the launch always completes.  On this device it is slower than
 * bitnet_w2a8_chain (the exchange between layers costs more than a launch).
 *
 * bitnet_w2a8_persist_table_bytes(n): bytes of the layer table for n layers (0 if n < 1).
 *
 * bitnet_w2a8_persist_prepare: plans the layers into table_host (host memory, at least
 * bitnet_w2a8_persist_table_bytes(n)) and returns the workspace size the launch needs.
 *   layers, n   as bitnet_w2a8_chain (device pointers inside; they must stay valid while
 *               the table is used)
 *   M           1 (else BITNET_ERR_UNSUPPORTED_SHAPE)
 *   xdt         BITNET_DT_BF16 or BITNET_DT_F32, the type of the first layer's input
 *   cus         compute units of the device that will run it; 0 = the current device's
 *   Rules: as bitnet_w2a8_chain, and each K <= 16384 (<= 8192 behind a junction); a layer
 *   must fit in `cus` workgroups (else BITNET_ERR_UNSUPPORTED_SHAPE).
 * The caller copies the table, byte for byte, into device memory (16-byte aligned) and
 * passes that copy to the launches below.
 *
 * bitnet_w2a8_chain_persistent: one pass.
 *   table_dev        device, the prepared table of n layers
 *   x                device, [1][K of layer 0] of xdt (the type given to prepare)
 *   y                device, fp32 [1][N of the last layer] (out)
 *   workspace        device, 256-byte aligned, at least the prepared size; clobbered.
 *                    After the launch: int32 status at offset 0 (0 success; i + 1 when a
 *                    wait for layer i's input gave up; -(i + 1) when layer i of the table
 *                    does not fit the workspace or its shape fields are invalid, found
 *                    before anything of layer i is written), and each intermediate
 *                    layer's fp32 output at its planned offset.
 * Returns BITNET_OK once both launches (a fill of the workspace, then the pass) are
 * enqueued on `stream`; the status word is the pass's own result.  Capturable in a HIP
 * graph; no allocation.  Launches that overlap on one device with work that keeps compute
 * units busy can make the waits give up (status > 0), never hang.
 *
 * bitnet_w2a8_chain_persistent_ex: the same with two test knobs: spin_limit (0 = the
 * default of 65536 poll rounds) bounds every wait; withhold_layer (-1 = none) is a layer
 * whose output is never stored, so that the waits for it give up. */
size_t bitnet_w2a8_persist_table_bytes(int n);
bitnet_status_t bitnet_w2a8_persist_prepare(const bitnet_chain_layer_t *layers, int n, int M, int xdt, int64_t cus,
                                            void *table_host, size_t table_bytes, size_t *workspace_bytes);
bitnet_status_t bitnet_w2a8_chain_persistent(const void *table_dev, int n, const void *x, int xdt, int M, float *y,
                                             void *workspace, size_t workspace_bytes, hipStream_t stream);
bitnet_status_t bitnet_w2a8_chain_persistent_ex(const void *table_dev, int n, const void *x, int xdt, int M, float *y,
                                                void *workspace, size_t workspace_bytes, int spin_limit,
                                                int withhold_layer, hipStream_t stream);

/* Exact integer product acc[m][n] = sum_k T[n][k] * Q[m][k] (int32, device, [M][N]),
 * computed by the same kernels as the two products above (M <= 16: the decode
 * kernel; larger M: the prefill kernel), so that their integer core can be
 * checked bit for bit.  Rules: M >= 1 and the shape rules. */
bitnet_status_t bitnet_w2a8_acc_i32(const uint8_t *packed, const int8_t *q, int32_t *acc,
                                    int M, int N, int K, hipStream_t stream);

/* Decode product for one token by table lookups, an experiment beside
 * bitnet_w2a8_gemv (same operation, same operands).  The lookup-table idea is
 * the CPU prior art of [P2] "5x performance leap: BitNet vs llama.cpp",
 * "Architecture foundations", item 1 (TL1/TL2: precompute the sums a group of
 * ternary weights can take against the activations, then look them up) and of
 * [P3] "BitNet + WebAssembly" (16-entry table per weight group).  Here every
 * pair of activations gets a 16-entry int16 table in LDS, indexed by the pair's
 * two 2-bit codes as they sit in one nibble of the tile layout.
 *   packed  device, tile layout, bitnet_packed_bytes(N,K) bytes
 *   scales  device, tiled scales, bitnet_scale_count(N,K) fp32
 *   q       device, int8 [K] (one token);  s_a device, fp32 [1]
 *   y       device, fp32 [N] (out)
 *   acc     device, int32 [N] (out: the exact sums over k of T[n][k] * Q[k]), or NULL
 *   tiles_per_group  16-row tiles each workgroup covers (1, 2 or 4; 0 = 2 when that
 *           leaves at least 256 workgroups, else 1): more tiles amortise the table
 *           build over more weights, fewer leave more workgroups to fill the chip
 * Rules: the shape rules and K <= 2^22 (else UNSUPPORTED_SHAPE); other
 * tiles_per_group values are INVALID_ARG.  y agrees with the exact value within
 * 1e-5 of max(|y|, s_a * sum_b |S*A|); for a given shape and tiles_per_group the
 * summation order, and so y, is fixed. */
bitnet_status_t bitnet_w2a8_gemv_lut(const uint8_t *packed, const float *scales, const int8_t *q,
                                     const float *s_a, float *y, int32_t *acc, int N, int K,
                                     int tiles_per_group, hipStream_t stream);

/* ---------------------------------------------------------------- measurement helper */

/* Not part of the product path: one pass of 16-byte non-temporal (streaming)
 * loads over `bytes` of device memory, the bandwidth a bare stream attains at
 * that size, against which the benchmark prices the product kernels next to
 * the published HBM peak.  mode 0: every wave writes the wrapping 32-bit sum of the words it
 * read to one sink entry, so the sum of all entries (mod 2^32) is the sum of
 * every 32-bit word of the buffer; mode 1: a wave writes only if its sum equals
 * one fixed value (practically never) -- the floor of a read with no output,
 * since a kernel completes only when its stores are acknowledged.
 *   src   device, 16-byte aligned, bytes % 16 == 0 (else UNSUPPORTED_SHAPE)
 *   sink  device, uint32 [sink_len], sink_len >= bitnet_probe_stream_read_sink_len(bytes)
 *   mode  0 or 1 (else INVALID_ARG) */
size_t bitnet_probe_stream_read_sink_len(size_t bytes);
bitnet_status_t bitnet_probe_stream_read(const void *src, size_t bytes, uint32_t *sink, size_t sink_len, int mode,
                                         hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* BITNET_W2A8_H */
