// e4m3 TN instantiations of the MFMA GEMM launchers.
#include "launch16.hpp"
namespace sg {
template hipError_t launch16_tr<DT_E4M3, true, false>(int, int, const Gemm16Params&, int, hipStream_t);
}
