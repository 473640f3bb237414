// Library-internal constants of the gfx950 tile layout (the layout itself is
// specified in include/bitnet_w2a8.h).
#pragma once
#include <cstdint>

namespace bitnet_layout {
constexpr int64_t kBlockK = 128;     // weights per scale block (i2_s x86 block)
constexpr int64_t kTileN = 16;       // rows per tile = one int8 matrix-core tile edge
constexpr int64_t kBrickBytes = 512; // 16 rows x 128 weights x 2 bits
}  // namespace bitnet_layout
