// fp32 instantiations of the backward.
#include "bwd_dispatch.hpp"

namespace linattn {
hipError_t launch_bwd_f32(const BwdLaunch& p) { return run_bwd_typed<float>(p); }
}  // namespace linattn
