// bf16 instantiations of the backward.
#include "bwd_dispatch.hpp"

namespace linattn {
hipError_t launch_bwd_bf16(const BwdLaunch& p) { return run_bwd_typed<uint16_t>(p); }
}  // namespace linattn
