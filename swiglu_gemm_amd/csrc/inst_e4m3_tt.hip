// e4m3 TT instantiations of the MFMA GEMM launchers.
#include "launch16.hpp"
namespace sg {
template hipError_t launch16_tr<DT_E4M3, true, true>(int, int, const Gemm16Params&, int, hipStream_t);
}
