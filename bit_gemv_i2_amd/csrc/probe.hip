// Measurement helper: one pass of 16-byte non-temporal loads over a device buffer,
// the bandwidth a bare stream attains at a given size on this GPU.  The
// benchmark prices the product kernels against it next to the published HBM
// peak, because at a few MB a single launch cannot reach that peak (launch
// and first-byte latency dominate).  Not part of the product path.
#include <hip/hip_runtime.h>

#include "bitnet_w2a8.h"

namespace {

typedef unsigned v4u __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;
constexpr size_t kProbeMaxBlocks = 65536;

// v + the value DPP control CTRL brings to each lane of the rows in ROWS.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_add(uint32_t v) {
    return v + (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xF, false);
}

// One 16-byte load per thread per round (grid-stride only past 65536
// workgroups): the fastest bare read of a few MB measured on this GPU.  Each
// wave folds its words into one wrapping 32-bit sum with DPP row operations
// (VALU only: quad sums, half-row and row mirrors, then rows 1/3 and 2/3 take
// the previous rows' totals, leaving the wave total in lane 63) and that lane
// writes it to sink[global wave index].
__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const uint4 *__restrict__ src, size_t n16,
                                                                    uint32_t *__restrict__ sink, int mode) {
    const size_t stride = (size_t)gridDim.x * kProbeThreads;
    uint32_t acc = 0;
    for (size_t i = (size_t)blockIdx.x * kProbeThreads + threadIdx.x; i < n16; i += stride) {
        // streaming (non-temporal) 16-byte loads, as the product's weight stream uses
        const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(src + i));
        acc += v.x + v.y + v.z + v.w;
    }
    acc = dpp_add<0xB1, 0xF>(acc);   // quad_perm [1,0,3,2]
    acc = dpp_add<0x4E, 0xF>(acc);   // quad_perm [2,3,0,1]: quad totals
    acc = dpp_add<0x141, 0xF>(acc);  // row_half_mirror: half-row totals
    acc = dpp_add<0x140, 0xF>(acc);  // row_mirror: row totals
    acc = dpp_add<0x142, 0xA>(acc);  // row_bcast:15 into rows 1, 3
    acc = dpp_add<0x143, 0xC>(acc);  // row_bcast:31 into rows 2, 3: lane 63 = wave total
    // mode 0: every wave stores its total; mode 1: only a wave whose total is
    // one fixed value stores (practically none: the timing floor of a read that
    // produces no output, since a kernel ends only when its stores are done)
    if ((threadIdx.x & 63) == 63 && (mode == 0 || acc == 0x9E3779B9u))
        sink[(size_t)blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6)] = acc;
}

size_t probe_blocks(size_t bytes) {
    size_t g = (bytes / 16 + kProbeThreads - 1) / kProbeThreads;
    if (g < 1) g = 1;
    return g > kProbeMaxBlocks ? kProbeMaxBlocks : g;
}

}  // namespace

extern "C" {

size_t bitnet_probe_stream_read_sink_len(size_t bytes) { return probe_blocks(bytes) * (kProbeThreads / 64); }

bitnet_status_t bitnet_probe_stream_read(const void *src, size_t bytes, uint32_t *sink, size_t sink_len, int mode,
                                         hipStream_t stream) {
    if (!src || !sink || (reinterpret_cast<uintptr_t>(src) & 15) || (reinterpret_cast<uintptr_t>(sink) & 3))
        return BITNET_ERR_INVALID_ARG;
    if (mode != 0 && mode != 1) return BITNET_ERR_INVALID_ARG;
    if (bytes < 16 || bytes % 16) return BITNET_ERR_UNSUPPORTED_SHAPE;
    const size_t g = probe_blocks(bytes);
    if (sink_len < g * (kProbeThreads / 64)) return BITNET_ERR_INVALID_ARG;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)g), dim3(kProbeThreads), 0, stream,
                       static_cast<const uint4 *>(src), bytes / 16, sink, mode);
    return hipGetLastError() == hipSuccess ? BITNET_OK : BITNET_ERR_HIP;
}

}  // extern "C"
