// fsdp_units_adadelta.hip -- the unit kernel instantiated for Adadelta (fp32 state).
#include "fsdp_units.h"

namespace fsdp {

hipError_t launch_units_adadelta(const UnitArgs* units, int n, const UnitLaunch& L) {
    const OptParams& o = L.opt;
    return launch_units_with(units, n, L, OptAdadelta{o.lr, o.rho, o.omr, o.eps, o.wd});
}

}  // namespace fsdp
