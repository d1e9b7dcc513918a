// configs16.hpp -- the tile configurations of the 16-bit MFMA GEMM kernels.
#pragma once

namespace sg {

struct Cfg16 {
    int dma;            // 1: direct global->LDS ring (gemm16_dma.hpp), 0: register-staged
    int BM, BN, BK, S;  // tile and LDS stages
    int WM, WN;         // waves along M and N
    const char* name;
};

// Index = configuration id (SG_FORCE_CONFIG=<id>[,<splits>] overrides the choice).
constexpr Cfg16 kCfg16[] = {
    {0, 256, 256, 64, 2, 2, 2, "reg 256x256x64 s2 4w"},
    {0, 256, 256, 64, 2, 2, 4, "reg 256x256x64 s2 8w"},
    {0, 128, 128, 64, 2, 2, 2, "reg 128x128x64 s2 4w"},
    {1, 256, 256, 32, 4, 2, 2, "dma 256x256x32 s4 4w"},
    {1, 256, 256, 32, 4, 2, 4, "dma 256x256x32 s4 8w"},
    {1, 256, 256, 64, 2, 2, 2, "dma 256x256x64 s2 4w"},
    {1, 128, 128, 32, 4, 2, 2, "dma 128x128x32 s4 4w"},
    {1, 128, 128, 64, 3, 2, 2, "dma 128x128x64 s3 4w"},
};
constexpr int kNumCfg16 = sizeof(kCfg16) / sizeof(kCfg16[0]);

}  // namespace sg
