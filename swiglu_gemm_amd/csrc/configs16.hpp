// configs16.hpp -- the tile configurations of the 16-bit MFMA GEMM kernels.
#pragma once

namespace sg {

struct Cfg16 {
    int e4m3;           // 1: e4m3 operands (BK in bytes), 0: fp16 / bf16 operands
    int dma;            // 0: register-staged (gemm16.hpp), 1: direct global->LDS ring
                        // (gemm16_dma.hpp), 3: the direct ring for the split-weight
                        // SwiGLU with Gate then Up (EPI_SWIGLU_SEQ only), 4: the same
                        // with the ring driven by separate producer waves
                        // (gemm_ws_kernel); -1: a retired id, kept so that the others
                        // stay stable
    int BM, BN, BK, S;  // tile and LDS stages
    int WM, WN;         // waves along M and N
    const char* name;
};

// Index = configuration id (SG_FORCE_CONFIG=<id>[,<splits>] overrides the choice).
// Every row must also appear in the SG_CONFIGS list below, with the same values.
constexpr Cfg16 kCfg16[] = {
    {0, 0, 256, 256, 64, 2, 2, 2, "reg 256x256x64 s2 2x2w"},
    {0, 0, 256, 256, 64, 2, 2, 4, "reg 256x256x64 s2 2x4w"},
    {0, 0, 128, 128, 64, 2, 2, 2, "reg 128x128x64 s2 2x2w"},
    {0, 1, 256, 256, 32, 4, 2, 2, "dma 256x256x32 s4 2x2w"},
    {0, 1, 256, 256, 32, 4, 2, 4, "dma 256x256x32 s4 2x4w"},
    {0, 1, 256, 256, 64, 2, 2, 2, "dma 256x256x64 s2 2x2w"},
    {0, 1, 128, 128, 32, 4, 2, 2, "dma 128x128x32 s4 2x2w"},
    {0, 1, 128, 128, 64, 3, 2, 2, "dma 128x128x64 s3 2x2w"},
    {0, 1, 256, 256, 64, 2, 2, 4, "dma 256x256x64 s2 2x4w"},
    {0, 1, 256, 256, 32, 4, 4, 2, "dma 256x256x32 s4 4x2w"},
    {0, 1, 256, 256, 64, 2, 4, 2, "dma 256x256x64 s2 4x2w"},
    {0, 1, 128, 256, 64, 2, 2, 2, "dma 128x256x64 s2 2x2w"},
    {0, 1, 256, 128, 64, 2, 2, 2, "dma 256x128x64 s2 2x2w"},
    {0, 1, 128, 128, 64, 2, 2, 4, "dma 128x128x64 s2 2x4w"},
    {1, 1, 256, 256, 128, 2, 4, 2, "e4m3 dma 256x256x128 s2 4x2w"},
    {1, 1, 128, 128, 128, 2, 2, 4, "e4m3 dma 128x128x128 s2 2x4w"},
    {1, 1, 32, 256, 128, 4, 1, 4, "e4m3 dma 32x256x128 s4 1x4w"},
    {1, 1, 32, 128, 128, 4, 1, 4, "e4m3 dma 32x128x128 s4 1x4w"},
    {0, -1, 0, 0, 0, 0, 0, 0, "retired"},
    {0, -1, 0, 0, 0, 0, 0, 0, "retired"},
    {0, -1, 0, 0, 0, 0, 0, 0, "retired"},
    {0, -1, 0, 0, 0, 0, 0, 0, "retired"},
    {0, -1, 0, 0, 0, 0, 0, 0, "retired"},
    {0, -1, 0, 0, 0, 0, 0, 0, "retired"},
    {0, 1, 256, 320, 64, 2, 4, 2, "dma 256x320x64 s2 4x2w"},
    {0, -1, 0, 0, 0, 0, 0, 0, "retired"},
    {0, -1, 0, 0, 0, 0, 0, 0, "retired"},
    {0, 1, 256, 256, 32, 5, 4, 2, "dma 256x256x32 s5 4x2w"},
    {0, 1, 256, 256, 32, 5, 2, 4, "dma 256x256x32 s5 2x4w"},
    {0, -1, 0, 0, 0, 0, 0, 0, "retired"},
    {0, 1, 128, 128, 64, 5, 2, 4, "dma 128x128x64 s5 2x4w"},
    {0, 1, 128, 128, 32, 8, 2, 2, "dma 128x128x32 s8 2x2w"},
    {0, 1, 128, 256, 64, 3, 2, 4, "dma 128x256x64 s3 2x4w"},
    {1, 1, 128, 256, 128, 3, 2, 2, "e4m3 dma 128x256x128 s3 2x2w"},
    // pipeline-depth study only (fp16 NN GEMM; never chosen automatically)
    {0, 1, 256, 256, 32, 2, 4, 2, "sweep dma 256x256x32 s2 4x2w"},
    {0, 1, 256, 256, 32, 3, 4, 2, "sweep dma 256x256x32 s3 4x2w"},
    {0, 1, 128, 128, 64, 3, 2, 4, "sweep dma 128x128x64 s3 2x4w"},
    {0, 1, 128, 128, 64, 4, 2, 4, "sweep dma 128x128x64 s4 2x4w"},
    {0, 1, 128, 128, 32, 2, 2, 2, "sweep dma 128x128x32 s2 2x2w"},
    {0, 1, 128, 128, 32, 3, 2, 2, "sweep dma 128x128x32 s3 2x2w"},
    {0, 1, 256, 256, 32, 5, 2, 2, "sweep dma 256x256x32 s5 2x2w"},
    {0, 1, 256, 256, 32, 3, 2, 2, "sweep dma 256x256x32 s3 2x2w"},
    {0, -1, 0, 0, 0, 0, 0, 0, "retired"},
    // 64-row tiles: twice the work-groups of 128-row tiles for 65..128-row problems
    {0, 1, 64, 256, 64, 3, 1, 4, "dma 64x256x64 s3 1x4w"},
    {0, 1, 64, 128, 64, 4, 1, 4, "dma 64x128x64 s4 1x4w"},
    {1, 1, 128, 256, 128, 3, 2, 4, "e4m3 dma 128x256x128 s3 2x4w"},
    // 192-column tiles: one full round where 256 columns leave CUs idle (N = 3072)
    {0, 1, 256, 192, 64, 2, 4, 2, "dma 256x192x64 s2 4x2w"},
    {1, 1, 128, 192, 128, 4, 4, 2, "e4m3 dma 128x192x128 s4 4x2w"},
    {0, 1, 128, 192, 64, 4, 4, 2, "dma 128x192x64 s4 4x2w"},
    // split-weight SwiGLU, Gate then Up (BN: the fused width, BN/2 outputs)
    {0, 3, 256, 256, 64, 3, 4, 2, "seq 256x256x64 s3 4x2w"},
    {0, 3, 128, 256, 64, 4, 2, 2, "seq 128x256x64 s4 2x2w"},
    {1, 3, 256, 256, 128, 3, 4, 2, "e4m3 seq 256x256x128 s3 4x2w"},
    {1, 3, 128, 256, 128, 4, 2, 2, "e4m3 seq 128x256x128 s4 2x2w"},
    // the same with 4 producer waves beside the 2x2 consumer waves (Kernel-1's
    // producer / consumer split)
    {0, 4, 128, 256, 64, 4, 2, 2, "seq-ws 128x256x64 s4 2x2w+4p"},
    {1, 4, 128, 256, 128, 4, 2, 2, "e4m3 seq-ws 128x256x128 s4 2x2w+4p"},
};
constexpr int kNumCfg16 = sizeof(kCfg16) / sizeof(kCfg16[0]);

// Whether id names a configuration that is still built (in range, not retired).
constexpr bool cfg_live(int id) { return id >= 0 && id < kNumCfg16 && kCfg16[id].dma >= 0; }

constexpr int kFirstCfgE4M3 = 14;
constexpr int kFirstSweepCfg = 34;   // ids 34..41: the fp16 NN pipeline-depth study

// Whether the direct-to-LDS kernel supports an operand tile: k-contiguous rows of
// 64 or 128 bytes; row-contiguous rows of 128..1024 bytes made of an even number
// of 32-byte units (what the bank swizzles cover); a whole number of 1 KiB DMA
// blocks per issuing wave.
constexpr bool dma_tile_ok(bool kc, int rows, int bk, int esz, int nwaves) {
    const int row_bytes = kc ? bk * esz : rows * esz;
    const int bytes = rows * bk * esz;
    const bool rc_ok = row_bytes >= 128 && row_bytes <= 1024 && row_bytes % 64 == 0;
    return (kc ? (row_bytes == 64 || row_bytes == 128) : rc_ok) && bytes % 1024 == 0 &&
           (bytes / 1024) % nwaves == 0;
}

// X(id, dma, BM, BN, BK, S, WM, WN) for every 16-bit row of kCfg16
#define SG_CONFIGS(X)                  \
    X(0, 0, 256, 256, 64, 2, 2, 2)     \
    X(1, 0, 256, 256, 64, 2, 2, 4)     \
    X(2, 0, 128, 128, 64, 2, 2, 2)     \
    X(3, 1, 256, 256, 32, 4, 2, 2)     \
    X(4, 1, 256, 256, 32, 4, 2, 4)     \
    X(5, 1, 256, 256, 64, 2, 2, 2)     \
    X(6, 1, 128, 128, 32, 4, 2, 2)     \
    X(7, 1, 128, 128, 64, 3, 2, 2)     \
    X(8, 1, 256, 256, 64, 2, 2, 4)     \
    X(9, 1, 256, 256, 32, 4, 4, 2)     \
    X(10, 1, 256, 256, 64, 2, 4, 2)    \
    X(11, 1, 128, 256, 64, 2, 2, 2)    \
    X(12, 1, 256, 128, 64, 2, 2, 2)    \
    X(13, 1, 128, 128, 64, 2, 2, 4)     \
    X(24, 1, 256, 320, 64, 2, 4, 2)    \
    X(27, 1, 256, 256, 32, 5, 4, 2)    \
    X(28, 1, 256, 256, 32, 5, 2, 4)    \
    X(30, 1, 128, 128, 64, 5, 2, 4)    \
    X(31, 1, 128, 128, 32, 8, 2, 2)    \
    X(32, 1, 128, 256, 64, 3, 2, 4)    \
    X(43, 1, 64, 256, 64, 3, 1, 4)     \
    X(44, 1, 64, 128, 64, 4, 1, 4)     \
    X(46, 1, 256, 192, 64, 2, 4, 2)    \
    X(48, 1, 128, 192, 64, 4, 4, 2)

// the pipeline-depth study rows, instantiated for fp16 NN EPI_GEMM only
#define SG_CONFIGS_SWEEP(X)            \
    X(34, 1, 256, 256, 32, 2, 4, 2)    \
    X(35, 1, 256, 256, 32, 3, 4, 2)    \
    X(36, 1, 128, 128, 64, 3, 2, 4)    \
    X(37, 1, 128, 128, 64, 4, 2, 4)    \
    X(38, 1, 128, 128, 32, 2, 2, 2)    \
    X(39, 1, 128, 128, 32, 3, 2, 2)    \
    X(40, 1, 256, 256, 32, 5, 2, 2)    \
    X(41, 1, 256, 256, 32, 3, 2, 2)

// the configurations the library chooses by itself, also compiled with the extra
// epilogue steps (EPI_GEMM_EX); any other one maps to the nearest of these (the
// register-staged 256 x 256 tile holds 256 accumulators per lane: no room left)
#define SG_CONFIGS_EX(X)               \
    X(2, 0, 128, 128, 64, 2, 2, 2)     \
    X(6, 1, 128, 128, 32, 4, 2, 2)     \
    X(10, 1, 256, 256, 64, 2, 4, 2)    \
    X(13, 1, 128, 128, 64, 2, 2, 4)    \
    X(24, 1, 256, 320, 64, 2, 4, 2)    \
    X(30, 1, 128, 128, 64, 5, 2, 4)    \
    X(32, 1, 128, 256, 64, 3, 2, 4)    \
    X(46, 1, 256, 192, 64, 2, 4, 2)    \
    X(48, 1, 128, 192, 64, 4, 4, 2)    \
    X(44, 1, 64, 128, 64, 4, 1, 4)

#define SG_CONFIGS_E4M3_EX(X)          \
    X(14, 1, 256, 256, 128, 2, 4, 2)   \
    X(15, 1, 128, 128, 128, 2, 2, 4)   \
    X(16, 1, 32, 256, 128, 4, 1, 4)    \
    X(17, 1, 32, 128, 128, 4, 1, 4)    \
    X(33, 1, 128, 256, 128, 3, 2, 2)   \
    X(45, 1, 128, 256, 128, 3, 2, 4)   \
    X(47, 1, 128, 192, 128, 4, 4, 2)

// the split-weight SwiGLU with Gate then Up (EPI_SWIGLU_SEQ, NN only)
#define SG_CONFIGS_SEQ(X)              \
    X(49, 1, 256, 256, 64, 3, 4, 2)    \
    X(50, 1, 128, 256, 64, 4, 2, 2)    \
    X(53, 4, 128, 256, 64, 4, 2, 2)

#define SG_CONFIGS_E4M3_SEQ(X)         \
    X(51, 1, 256, 256, 128, 3, 4, 2)   \
    X(52, 1, 128, 256, 128, 4, 2, 2)   \
    X(54, 4, 128, 256, 128, 4, 2, 2)

// the same for every e4m3 row (all direct-to-LDS)
#define SG_CONFIGS_E4M3(X)             \
    X(14, 1, 256, 256, 128, 2, 4, 2)   \
    X(15, 1, 128, 128, 128, 2, 2, 4)   \
    X(16, 1, 32, 256, 128, 4, 1, 4)    \
    X(17, 1, 32, 128, 128, 4, 1, 4)    \
    X(33, 1, 128, 256, 128, 3, 2, 2)   \
    X(45, 1, 128, 256, 128, 3, 2, 4)   \
    X(47, 1, 128, 192, 128, 4, 4, 2)

// Every row of the lists above is the kCfg16 row of its id.  The lists' DMA field
// is the kernel family (0 register-staged, 1 direct ring, 4 producer waves); a
// Gate-then-Up row's family 1 is kCfg16's dma 3.
constexpr bool row_is(int id, int e4m3, int fam, int bm, int bn, int bk, int s, int wm, int wn,
                      bool seq) {
    return cfg_live(id) && kCfg16[id].e4m3 == e4m3 &&
           kCfg16[id].dma == (seq && fam == 1 ? 3 : fam) && kCfg16[id].BM == bm &&
           kCfg16[id].BN == bn && kCfg16[id].BK == bk && kCfg16[id].S == s &&
           kCfg16[id].WM == wm && kCfg16[id].WN == wn;
}
#define SG_ROW16(ID, DMA, BM, BN, BK, S, WM, WN) \
    static_assert(row_is(ID, 0, DMA, BM, BN, BK, S, WM, WN, false), "16-bit row " #ID);
#define SG_ROW8(ID, DMA, BM, BN, BK, S, WM, WN) \
    static_assert(row_is(ID, 1, DMA, BM, BN, BK, S, WM, WN, false), "e4m3 row " #ID);
#define SG_ROW16_SEQ(ID, DMA, BM, BN, BK, S, WM, WN) \
    static_assert(row_is(ID, 0, DMA, BM, BN, BK, S, WM, WN, true), "Gate-then-Up row " #ID);
#define SG_ROW8_SEQ(ID, DMA, BM, BN, BK, S, WM, WN) \
    static_assert(row_is(ID, 1, DMA, BM, BN, BK, S, WM, WN, true), "e4m3 Gate-then-Up row " #ID);
SG_CONFIGS(SG_ROW16)
SG_CONFIGS_SWEEP(SG_ROW16)
SG_CONFIGS_EX(SG_ROW16)
SG_CONFIGS_SEQ(SG_ROW16_SEQ)
SG_CONFIGS_E4M3(SG_ROW8)
SG_CONFIGS_E4M3_EX(SG_ROW8)
SG_CONFIGS_E4M3_SEQ(SG_ROW8_SEQ)
#undef SG_ROW16
#undef SG_ROW8
#undef SG_ROW16_SEQ
#undef SG_ROW8_SEQ

}  // namespace sg
