// fp32 instantiations of the chunked forward (fp32 MFMA, nothing rounded below fp32).
#include "fwd_dispatch.hpp"

namespace linattn {
hipError_t launch_fwd_f32(const FwdLaunch& p) { return run_fwd_typed<float>(p); }
}  // namespace linattn
