// e4m3 instantiations of the decode-shaped (M <= 32) GEMM launchers.
#include "decode.hpp"
namespace sg {
template hipError_t launch_decode_dt<DT_E4M3>(bool, int, int, const DecodeParams&, bool, hipStream_t);
}
