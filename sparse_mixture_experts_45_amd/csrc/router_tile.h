// Router score tile width, shared by the route plan and the router launches.
#pragma once
#include "moe.h"

namespace moe {

// Experts per block of the router score kernel: 16, 32 (bf16 layers with up to
// 32 experts) or 64; one tile column of 16 experts per wave group.
inline int router_tile(int E, int dtype) {
  return E <= 16 ? 16 : (E <= 32 && dtype == MOE_BF16 ? 32 : 64);
}

}  // namespace moe
