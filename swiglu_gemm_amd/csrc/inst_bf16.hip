// bf16 instantiations of the 16-bit MFMA GEMM launchers.
#include "launch16.hpp"
namespace sg {
template hipError_t launch16_dt<DT_BF16>(bool, bool, int, int, const Gemm16Params&, int, hipStream_t);
}
