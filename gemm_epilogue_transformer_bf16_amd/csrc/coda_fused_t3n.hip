// Instantiations of the fused kernel for bf16 tile configuration 3 with a
// deferred row norm (RMSNorm / LayerNorm, every gain placement).
#include "coda_fused_impl.h"
#include "coda_plan.h"

namespace coda {
namespace dev {

int launch_tile3_norm(const FusedArgs& a, int64_t nwg, bool bkn, int norm, hipStream_t s) {
  constexpr TileCfg t = kTileCfgs[2];
  return launch_norm_variants<t.bm, t.bn, t.wm, t.wn, false>(a, nwg, bkn, norm, s);
}

}  // namespace dev
}  // namespace coda
