// bf16 instantiations of the chunked forward.
#include "fwd_dispatch.hpp"

namespace linattn {
hipError_t launch_fwd_bf16(const FwdLaunch& p) { return run_fwd_typed<uint16_t>(p); }
}  // namespace linattn
