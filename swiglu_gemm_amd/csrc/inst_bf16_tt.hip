// bf16 TT instantiations of the 16-bit MFMA GEMM launchers.
#include "launch16.hpp"
namespace sg {
template hipError_t launch16_tr<DT_BF16, true, true>(int, int, const Gemm16Params&, int, hipStream_t);
}
