// Workspace layout of the decode chain (harp_linear_chain), shared by the
// kernel and the HIP-free argument checks.
#pragma once

#include <stddef.h>

namespace harp {

constexpr int kChainMaxLayers = 48;   // layers per launch (kernel arguments by value, 3 KB)
constexpr int kChainMaxM = 4;
constexpr int kChainFlagCopies = 16;  // copies of each rotation flag (spread polling)

// In uint32 words: [0, 64) control (word 0 the epoch, word 1 a wait that ran
// out, word 2 the final workgroups' arrival count), per-phase rotation flags
// [phase][copy][32], then the data: float32 z [phase][kChainMaxM][dim] for
// phases 0..kChainMaxLayers, and y' after the output side's widest three
// stages as (float32 value, uint32 epoch) pairs [layer][kChainMaxM][dim].
constexpr size_t kChainFlagsOffset = 64;
constexpr size_t kChainDataOffset =
    (kChainFlagsOffset + size_t{kChainMaxLayers + 1} * kChainFlagCopies * 32 + 63) / 64 * 64;

constexpr size_t chain_workspace_bytes(int dim) {
  return (dim != 4096 && dim != 8192)
             ? 0
             : kChainDataOffset * 4 + size_t{kChainMaxLayers + 1 + 2 * kChainMaxLayers} *
                                          kChainMaxM * static_cast<size_t>(dim) * 4;
}

}  // namespace harp
