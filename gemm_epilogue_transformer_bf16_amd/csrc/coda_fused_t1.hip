// Instantiations of the fused kernel for bf16 tile configuration 1, without a
// row norm (the norm kernels are in coda_fused_t1n.hip).
#include "coda_fused_impl.h"
#include "coda_plan.h"

namespace coda {
namespace dev {

int launch_tile1(const FusedArgs& a, int64_t nwg, bool bkn, bool akm, bool ext, bool side, hipStream_t s) {
  constexpr TileCfg t = kTileCfgs[0];
  return launch_plain_variants<t.bm, t.bn, t.wm, t.wn, false>(a, nwg, bkn, akm, ext, side, s);
}

}  // namespace dev
}  // namespace coda
