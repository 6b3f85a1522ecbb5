// Instantiations of the fused kernel for bf16 tile configuration 2.
#include "coda_fused_impl.h"
#include "coda_plan.h"

namespace coda {
namespace dev {

int launch_tile2(const FusedArgs& a, int64_t nwg, bool bkn, int norm, bool akm, bool ext, bool side,
                 hipStream_t s) {
  constexpr TileCfg t = kTileCfgs[1];
  return launch_variants<t.bm, t.bn, t.wm, t.wn, false>(a, nwg, bkn, norm, akm, ext, side, s);
}

}  // namespace dev
}  // namespace coda
