// Instantiations of the decode step.
#include "decode.hpp"
#include "launch.hpp"

namespace linattn {

template <typename E>
static hipError_t run_decode(const void* q, const void* k, const void* v, float* S, float* z, void* o, int BH, int D,
                             int Dv, float eps, const float* g, const float* ga, int normalize, hipStream_t stream) {
    const E* qe = static_cast<const E*>(q);
    const E* ke = static_cast<const E*>(k);
    const E* ve = static_cast<const E*>(v);
    E* oe = static_cast<E*>(o);
    const dim3 grid(BH), block(kThreads);
    if (D == 64 && Dv == 64) hipLaunchKernelGGL((decode_kernel<E, 64, 64>), grid, block, 0, stream, qe, ke, ve, g, ga, S, z, oe, eps, normalize);
    else if (D == 64 && Dv == 128) hipLaunchKernelGGL((decode_kernel<E, 64, 128>), grid, block, 0, stream, qe, ke, ve, g, ga, S, z, oe, eps, normalize);
    else if (D == 128 && Dv == 64) hipLaunchKernelGGL((decode_kernel<E, 128, 64>), grid, block, 0, stream, qe, ke, ve, g, ga, S, z, oe, eps, normalize);
    else if (D == 128 && Dv == 128) hipLaunchKernelGGL((decode_kernel<E, 128, 128>), grid, block, 0, stream, qe, ke, ve, g, ga, S, z, oe, eps, normalize);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_decode(int dtype, const void* q, const void* k, const void* v, float* S, float* z, void* o, int BH,
                         int D, int Dv, float eps, const float* g, const float* ga, int normalize,
                         hipStream_t stream) {
    if (dtype == 1) return run_decode<uint16_t>(q, k, v, S, z, o, BH, D, Dv, eps, g, ga, normalize, stream);
    return run_decode<float>(q, k, v, S, z, o, BH, D, Dv, eps, g, ga, normalize, stream);
}

}  // namespace linattn
