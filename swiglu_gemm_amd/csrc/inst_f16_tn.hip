// f16 TN instantiations of the 16-bit MFMA GEMM launchers.
#include "launch16.hpp"
namespace sg {
template hipError_t launch16_tr<DT_F16, true, false>(int, int, const Gemm16Params&, int, hipStream_t);
}
