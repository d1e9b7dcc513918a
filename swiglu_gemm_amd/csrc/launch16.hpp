// launch16.hpp -- launchers for every (configuration, transpose, epilogue) of the
// 16-bit MFMA GEMM kernels.  Instantiated once per dtype (inst_f16.hip,
// inst_bf16.hip) so the two compile in parallel.
#pragma once

#include <hip/hip_runtime.h>

#include "configs16.hpp"
#include "gemm16.hpp"
#include "gemm16_dma.hpp"

namespace sg {

template <typename Kern>
inline hipError_t launch_grid(Kern k, const Gemm16Params& p, int splits, int threads,
                              hipStream_t st) {
    dim3 grid((unsigned)(p.tiles_m * p.tiles_n), (unsigned)splits);
    hipLaunchKernelGGL(k, grid, dim3(threads), 0, st, p);
    return hipGetLastError();
}

template <int DT, bool TA, bool TB, int EPI>
hipError_t launch16_cfg(int cfg, const Gemm16Params& p, int splits, hipStream_t st) {
    switch (cfg) {
#define SG_REG(ID, BM, BN, WM, WN) \
    case ID: return launch_grid(gemm16_kernel<DT, TA, TB, EPI, BM, BN, WM, WN>, p, splits, 64 * WM * WN, st);
#define SG_DMA(ID, BM, BN, BK, S, WM, WN) \
    case ID: return launch_grid(gemm16_dma_kernel<DT, TA, TB, EPI, BM, BN, BK, S, WM, WN>, p, splits, 64 * WM * WN, st);
        SG_REG(0, 256, 256, 2, 2)
        SG_REG(1, 256, 256, 2, 4)
        SG_REG(2, 128, 128, 2, 2)
        SG_DMA(3, 256, 256, 32, 4, 2, 2)
        SG_DMA(4, 256, 256, 32, 4, 2, 4)
        SG_DMA(5, 256, 256, 64, 2, 2, 2)
        SG_DMA(6, 128, 128, 32, 4, 2, 2)
        SG_DMA(7, 128, 128, 64, 3, 2, 2)
#undef SG_REG
#undef SG_DMA
        default: return hipErrorInvalidValue;
    }
}

// epi: EPI_GEMM / EPI_PARTIAL for any transpose pair; EPI_SWIGLU for NN only.
template <int DT>
hipError_t launch16_dt(bool ta, bool tb, int epi, int cfg, const Gemm16Params& p, int splits,
                       hipStream_t st) {
    if (epi == EPI_SWIGLU) return launch16_cfg<DT, false, false, EPI_SWIGLU>(cfg, p, splits, st);
    if (epi == EPI_GEMM) {
        if (!ta && !tb) return launch16_cfg<DT, false, false, EPI_GEMM>(cfg, p, splits, st);
        if (!ta && tb) return launch16_cfg<DT, false, true, EPI_GEMM>(cfg, p, splits, st);
        if (ta && !tb) return launch16_cfg<DT, true, false, EPI_GEMM>(cfg, p, splits, st);
        return launch16_cfg<DT, true, true, EPI_GEMM>(cfg, p, splits, st);
    }
    if (!ta && !tb) return launch16_cfg<DT, false, false, EPI_PARTIAL>(cfg, p, splits, st);
    if (!ta && tb) return launch16_cfg<DT, false, true, EPI_PARTIAL>(cfg, p, splits, st);
    if (ta && !tb) return launch16_cfg<DT, true, false, EPI_PARTIAL>(cfg, p, splits, st);
    return launch16_cfg<DT, true, true, EPI_PARTIAL>(cfg, p, splits, st);
}

}  // namespace sg
