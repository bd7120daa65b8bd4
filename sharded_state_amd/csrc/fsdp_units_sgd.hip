// fsdp_units_sgd.hip -- the unit kernel instantiated for SGD, without and with momentum (fp32 state).
#include "fsdp_units.h"

namespace fsdp {

hipError_t launch_units_sgd(const UnitArgs* units, int n, const UnitLaunch& L) {
    const OptParams& o = L.opt;
    if (o.kind == kOptSgd) return launch_units_with(units, n, L, OptSgd{o.lr, o.wd});
    return launch_units_with(units, n, L, OptSgdMomentum{o.lr, o.wd, o.mu, o.omd, o.first, o.nesterov});
}

}  // namespace fsdp
