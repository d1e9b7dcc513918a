// launch16.hpp -- launchers for every (configuration, epilogue) of the MFMA GEMM
// kernels (16-bit and e4m3 operands) for one (dtype, transpose pair).  Each pair is instantiated in its
// own translation unit (inst_*.hip) so they compile in parallel.
#pragma once

#include <hip/hip_runtime.h>

#include "configs16.hpp"
#include "gemm16.hpp"
#include "gemm16_dma.hpp"

namespace sg {

template <typename Kern>
inline hipError_t launch_grid(Kern k, const Gemm16Params& p, int splits, int threads,
                              hipStream_t st, bool warm = false) {
    const int tiles = p.tiles_m * p.tiles_n;
    dim3 grid((unsigned)(warm && p.warm_grid > tiles ? p.warm_grid : tiles), (unsigned)splits,
              (unsigned)(p.batch > 1 ? p.batch : 1));
    hipLaunchKernelGGL(k, grid, dim3(threads), 0, st, p);
    return hipGetLastError();
}

// Whether a configuration can run the split-weight SwiGLU (W1 and W2 separate):
// the direct-to-LDS single-group kernel, NN, an even number of fragments per wave
// along N (gate and up halves), and DMA-compatible half tiles of BN/2 columns.
template <int DT, bool TA, bool TB, int DMA, int BM, int BN, int BK, int WM, int WN>
constexpr bool w12_ok() {
    constexpr int ESZ = DT == DT_E4M3 ? 1 : 2;
    return (DMA == 1 || DT == DT_E4M3) && !TA && !TB && (BN / WN / 32) % 2 == 0 &&
           BN % 64 == 0 && dma_tile_ok(true, BM, BK, ESZ, WM * WN) &&
           dma_tile_ok(false, BN / 2, BK, ESZ, WM * WN);
}

template <int DT, bool TA, bool TB, int EPI, int DMA, int BM, int BN, int BK, int S, int WM, int WN>
inline hipError_t launch_one(const Gemm16Params& p, int splits, hipStream_t st) {
    constexpr int ESZ = DT == DT_E4M3 ? 1 : 2;
    if constexpr (EPI == EPI_SWIGLU_SEQ && DMA == 4) {
        // Kernel-1 with producer waves: the loads split over kWsProducers waves
        if constexpr (!TA && !TB && (BN / WN / 32) % 2 == 0 && BN % 64 == 0 &&
                      dma_tile_ok(true, BM, BK, ESZ, kWsProducers) &&
                      dma_tile_ok(false, BN / 2, BK, ESZ, kWsProducers))
            return launch_grid(gemm_ws_kernel<DT, TA, TB, EPI, BM, BN, BK, S, WM, WN>, p, splits,
                               64 * (WM * WN + kWsProducers), st);
        else
            return hipErrorInvalidValue;
    } else if constexpr (EPI == EPI_SWIGLU_W12 || EPI == EPI_SWIGLU_SEQ) {
        if constexpr (w12_ok<DT, TA, TB, DMA, BM, BN, BK, WM, WN>())
            return launch_grid(gemm_dma_kernel<DT, TA, TB, EPI, BM, BN, BK, S, WM, WN>, p, splits,
                               64 * WM * WN, st);
        else
            return hipErrorInvalidValue;
    } else if constexpr (DMA || DT == DT_E4M3) {
        // only this kernel has work for blocks past the tiles (the L2 warm-up), and
        // only with row-major B, one split and one problem (the host checks the same)
        if constexpr (dma_tile_ok(!TA, BM, BK, ESZ, WM * WN) && dma_tile_ok(TB, BN, BK, ESZ, WM * WN))
            return launch_grid(gemm_dma_kernel<DT, TA, TB, EPI, BM, BN, BK, S, WM, WN>, p, splits,
                               64 * WM * WN, st, !TB && splits == 1 && p.batch <= 1);
        else
            return hipErrorInvalidValue;
    } else
        return launch_grid(gemm16_kernel<DT, TA, TB, EPI, BM, BN, WM, WN>, p, splits,
                           64 * WM * WN, st);
}

template <int DT, bool TA, bool TB, int EPI>
hipError_t launch16_cfg(int cfg, const Gemm16Params& p, int splits, hipStream_t st) {
#define SG_CASE(ID, DMA, BM, BN, BK, S, WM, WN) \
    case ID: return launch_one<DT, TA, TB, EPI, DMA, BM, BN, BK, S, WM, WN>(p, splits, st);
    if constexpr (EPI == EPI_SWIGLU_SEQ) {
        if constexpr (DT == DT_E4M3) {
            switch (cfg) {
                SG_CONFIGS_E4M3_SEQ(SG_CASE)
                default: return hipErrorInvalidValue;
            }
        } else {
            switch (cfg) {
                SG_CONFIGS_SEQ(SG_CASE)
                default: return hipErrorInvalidValue;
            }
        }
    } else if constexpr (EPI == EPI_GEMM_EX) {
        if constexpr (DT == DT_E4M3) {
            switch (cfg) {
                SG_CONFIGS_E4M3_EX(SG_CASE)
                default: return hipErrorInvalidValue;
            }
        } else {
            switch (cfg) {
                SG_CONFIGS_EX(SG_CASE)
                default: return hipErrorInvalidValue;
            }
        }
    } else if constexpr (DT == DT_E4M3) {
        switch (cfg) {
            SG_CONFIGS_E4M3(SG_CASE)
            default: return hipErrorInvalidValue;
        }
    } else {
        switch (cfg) {
            SG_CONFIGS(SG_CASE)
            default: break;
        }
        if constexpr (DT == DT_F16 && !TA && !TB && EPI == EPI_GEMM) {
            switch (cfg) {
                SG_CONFIGS_SWEEP(SG_CASE)
                default: break;
            }
        }
        return hipErrorInvalidValue;
    }
#undef SG_CASE
}

// epi: EPI_GEMM / EPI_GEMM_EX / EPI_PARTIAL for any transpose pair; EPI_SWIGLU,
// EPI_SWIGLU_W12 and EPI_SWIGLU_SEQ for NN only.
template <int DT, bool TA, bool TB>
hipError_t launch16_tr(int epi, int cfg, const Gemm16Params& p, int splits, hipStream_t st) {
    if constexpr (!TA && !TB) {
        if (epi == EPI_SWIGLU) return launch16_cfg<DT, TA, TB, EPI_SWIGLU>(cfg, p, splits, st);
        if (epi == EPI_SWIGLU_W12)
            return launch16_cfg<DT, TA, TB, EPI_SWIGLU_W12>(cfg, p, splits, st);
        if (epi == EPI_SWIGLU_SEQ)
            return launch16_cfg<DT, TA, TB, EPI_SWIGLU_SEQ>(cfg, p, splits, st);
    }
    if (epi == EPI_GEMM) return launch16_cfg<DT, TA, TB, EPI_GEMM>(cfg, p, splits, st);
    if (epi == EPI_GEMM_EX) return launch16_cfg<DT, TA, TB, EPI_GEMM_EX>(cfg, p, splits, st);
    if (epi == EPI_PARTIAL) return launch16_cfg<DT, TA, TB, EPI_PARTIAL>(cfg, p, splits, st);
    return hipErrorInvalidValue;
}

}  // namespace sg
