// fsdp_units_adamax.hip -- the unit kernel instantiated for Adamax (fp32 state).
#include "fsdp_units.h"

namespace fsdp {

hipError_t launch_units_adamax(const UnitArgs* units, int n, const UnitLaunch& L) {
    const OptParams& o = L.opt;
    return launch_units_with(units, n, L, OptAdamax{o.clr, o.b1, o.omb1, o.b2, o.eps, o.wd});
}

}  // namespace fsdp
