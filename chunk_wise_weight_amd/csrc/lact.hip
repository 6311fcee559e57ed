// LaCT SwiGLU fast-weight kernels (review of "Test-Time Training Done Right",
// LaCT Model Architecture §1, eq. (3)-(4)).
#include "gemm.hpp"
#include "launch.hpp"

namespace ttt {

template <typename T>
size_t lact_workspace_bytes(int, int, int, int, int, int) { return 0; }

template <typename T>
hipError_t launch_lact(const LactArgs&, hipStream_t) { return hipErrorNotSupported; }

template size_t lact_workspace_bytes<float>(int, int, int, int, int, int);
template size_t lact_workspace_bytes<bf16>(int, int, int, int, int, int);
template hipError_t launch_lact<float>(const LactArgs&, hipStream_t);
template hipError_t launch_lact<bf16>(const LactArgs&, hipStream_t);

}  // namespace ttt
