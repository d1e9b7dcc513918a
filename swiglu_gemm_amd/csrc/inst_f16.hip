// fp16 instantiations of the 16-bit MFMA GEMM launchers.
#include "launch16.hpp"
namespace sg {
template hipError_t launch16_dt<DT_F16>(bool, bool, int, int, const Gemm16Params&, int, hipStream_t);
}
