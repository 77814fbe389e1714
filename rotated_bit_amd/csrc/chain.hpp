// Decode chain (chain.hip): arguments and workspace layout shared by the
// kernel and the host entry point.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "chain_layout.hpp"

namespace harp {

// One layer, pointers only (shapes are uniform over the chain and checked on
// the host): input side (cos, sin) pairs and signs, packed weight, output
// side, and the layer's output y [M][dim].
struct ChainLayer {
  const float2* cs_v;
  const uint32_t* sign_v;
  const uint32_t* qw;
  const uint16_t* sc;
  const uint16_t* zr;
  const float2* cs_u;
  const uint32_t* sign_u;
  void* y;
};

struct ChainArgs {
  int n_layers;
  int M;
  int x_bf16;
  int y_bf16;
  const void* x;
  uint32_t* ws;
  ChainLayer layer[kChainMaxLayers];
};

hipError_t launch_chain(const ChainArgs& a, int dim, int bits, hipStream_t stream);

}  // namespace harp
