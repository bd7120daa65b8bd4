// fsdp_units_adamw.hip -- the unit kernel instantiated for AdamW (fp32 master, m, v or 16-bit parameter, m, v).
#include "fsdp_units.h"

namespace fsdp {

hipError_t launch_units_adamw(const UnitArgs* units, int n, const UnitLaunch& L) {
    return launch_units_with(units, n, L, OptAdamW{L.opt.adam});
}

}  // namespace fsdp
