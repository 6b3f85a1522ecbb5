// Instantiations of the fused kernel for fp32 operands.
#include "coda_fused_impl.h"
#include "coda_plan.h"

namespace coda {
namespace dev {

int launch_tile_f32(const FusedArgs& a, int64_t nwg, bool bkn, int norm, bool akm, bool ext, bool side,
                    hipStream_t s) {
  return launch_variants<kF32Tile.bm, kF32Tile.bn, kF32Tile.wm, kF32Tile.wn, true>(a, nwg, bkn, norm, akm, ext, side,
                                                                                   s);
}

}  // namespace dev
}  // namespace coda
