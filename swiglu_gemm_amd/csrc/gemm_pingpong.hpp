// gemm_pingpong.hpp -- 8-wave "ping-pong" MFMA GEMM (gfx950), fp16 / bf16 / e4m3.
//
// Same tiles, LDS layouts, fragments, MFMAs and epilogues as gemm16_dma.hpp; only
// the schedule differs.  Each SIMD hosts two waves, one from each of two groups
// (waves 0-3 and 4-7).  A K tile is processed in two phases per wave:
//   M(t): issue the DMA of a later tile (group 0 only) and read ALL fragments of
//         tile t from LDS into registers;
//   C(t): all MFMAs of tile t on those registers.
// Group 1 runs one phase behind group 0, and every phase ends with a work-group
// barrier, so at any time one wave per SIMD issues MFMAs back to back while the
// other waits on LDS / DMA.  With an S-stage ring, tile t sits in stage t % S;
// group 0 issues the DMA of tile t+S-1 in M(t) (that stage was last read by group
// 1 in M(t-1), one phase earlier) and waits for tile t+1 at the end of C(t).
//
// DMA addressing: a per-operand tile base in SGPRs (advanced by one K tile per
// step) plus a 32-bit per-lane offset, so the 16 DMA streams of group 0 cost one
// VGPR each.
#pragma once

#include "gemm16_dma.hpp"

namespace sg {

// DMA of one operand tile, issued by NWD waves, 32-bit offsets from a uniform base.
template <bool KC, int R, int BK, int ESZ, int NWD>
struct DmaStreamS {
    using T = DmaTile<KC, R, BK, ESZ>;
    static_assert(T::BLOCKS % NWD == 0, "DMA blocks must split evenly over the waves");
    static constexpr int NI = T::BLOCKS / NWD;
    uint32_t off[NI];
    const char* base;   // tile base at the split's first k (wave-uniform)
    int64_t step;       // bytes per K tile

    __device__ __forceinline__ void init(const void* base_, int64_t ld, int r0, int rows, int k0,
                                         int widx, int lane) {
        const char* b0 = reinterpret_cast<const char*>(base_);
        base = KC ? b0 + ((int64_t)r0 * ld + k0) * ESZ : b0 + ((int64_t)k0 * ld + r0) * ESZ;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int b = widx + i * NWD;
            const int chunk = b * 64 + lane;
            const int row = chunk / T::SLOTS;
            const int slot = chunk % T::SLOTS;
            if constexpr (KC) {
                const int c = slot ^ T::swz(row);
                const int r = min(r0 + row, rows - 1) - r0;            // >= 0
                off[i] = (uint32_t)((int64_t)r * ld * ESZ + c * 16);
            } else {
                const int u = (slot >> 1) ^ T::swz(row);
                const int cb = min(r0 * ESZ + u * 32 + (slot & 1) * 16, (rows * ESZ - 1) & ~15) - r0 * ESZ;
                off[i] = (uint32_t)((int64_t)row * ld * ESZ + cb);
            }
        }
        step = KC ? (int64_t)BK * ESZ : (int64_t)BK * ld * ESZ;
    }
    __device__ __forceinline__ void issue(char* stage, int t, int widx) const {
        const char* bt = base + t * step;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int b = widx + i * NWD;
            const uint32_t lds = (uint32_t)(uintptr_t)(
                (__attribute__((address_space(3))) char*)(stage + b * 1024));
            asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                         :: "s"(lds), "v"(off[i]), "s"(bt) : "memory", "m0");
        }
    }
};

template <int DT, bool TA, bool TB, int EPI, int BM, int BN, int BK, int S, int WM, int WN>
__global__ void __launch_bounds__(512, 1) gemm_pp_kernel(const Gemm16Params p_) {
    const Gemm16Params p = batch_item(p_);
    static_assert(WM * WN == 8, "ping-pong runs 8 waves (two per SIMD)");
    constexpr int ESZ = DT == DT_E4M3 ? 1 : 2;
    constexpr int DT_OUT = DT == DT_E4M3 ? DT_BF16 : DT;
    constexpr int KSTEP = ESZ == 2 ? 16 : 64;
    using Frag = typename FragT<ESZ>::type;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    constexpr int KS = BK / KSTEP;
    static_assert(BK % KSTEP == 0, "whole k-steps per tile");
    constexpr bool KCA = !TA, KCB = TB;
    using TA_ = DmaTile<KCA, BM, BK, ESZ>;
    using TB_ = DmaTile<KCB, BN, BK, ESZ>;
    constexpr int STAGE = TA_::BYTES + TB_::BYTES;
    static_assert(S >= 2 && S * STAGE <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(1024))) char smem[S * STAGE];

    const int nblk = p.tiles_m * p.tiles_n;
    const int lid = xcd_remap(blockIdx.x, nblk);
    int tmi, tni;
    tile_coords(lid, p.tiles_m, p.tiles_n, p.group_m, tmi, tni);
    const int m0 = tmi * BM, n0 = tni * BN;
    const int kbeg = blockIdx.y * p.k_per_split;
    const int kend = min(p.K, kbeg + p.k_per_split);
    const int nkt = kend > kbeg ? (kend - kbeg) / BK : 0;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int group = wave >> 2, widx = wave & 3;
    const int wm = wave % WM, wn = wave / WM;

    DmaStreamS<KCA, BM, BK, ESZ, 4> da;
    DmaStreamS<KCB, BN, BK, ESZ, 4> db;
    da.init(p.A, p.lda, m0, p.M, kbeg, widx, lane);
    db.init(p.B, p.ldb, n0, p.N, kbeg, widx, lane);
    constexpr int NL = DmaStreamS<KCA, BM, BK, ESZ, 4>::NI + DmaStreamS<KCB, BN, BK, ESZ, 4>::NI;

    f32x16 acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    // Each K tile runs in NPH phase pairs of KSP k-steps (fragment registers hold
    // KSP k-steps: 16-bit 2 x 16 k, e4m3 1 x 64 k).
    constexpr int KSP = ESZ == 2 ? (KS >= 2 ? 2 : 1) : 1;
    constexpr int NPH = KS / KSP;
    static_assert(KS % KSP == 0, "whole phases per tile");
    Frag fa[KSP][FM], fb[KSP][FN];
    auto issue = [&](int t) {
        char* st = smem + (t % S) * STAGE;
        da.issue(st, t, widx);
        db.issue(st + TA_::BYTES, t, widx);
    };
    auto memory_phase = [&](int t, int ph) {
        if (ph == 0 && group == 0 && t + S - 1 < nkt) issue(t + S - 1);
        const char* st = smem + (t % S) * STAGE;
#pragma unroll
        for (int s = 0; s < KSP; ++s) {
#pragma unroll
            for (int tm = 0; tm < FM; ++tm)
                fa[s][tm] = read_frag<KCA, BM, BK, ESZ>(st, wm * TM + tm * 32, ph * KSP + s, lane);
#pragma unroll
            for (int tn = 0; tn < FN; ++tn)
                fb[s][tn] = read_frag<KCB, BN, BK, ESZ>(st + TA_::BYTES, wn * TN + tn * 32,
                                                        ph * KSP + s, lane);
        }
    };
    auto compute_phase = [&](int t, int ph) {
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int s = 0; s < KSP; ++s)
#pragma unroll
            for (int tn = 0; tn < FN; ++tn)
#pragma unroll
                for (int tm = 0; tm < FM; ++tm)
                    acc[tn][tm] = mfma_op<DT>(fb[s][tn], fa[s][tm], acc[tn][tm]);
        __builtin_amdgcn_s_setprio(0);
        // group 0 owns the DMA: tile t+1 must have landed before its M(t+1)
        if (ph == NPH - 1 && group == 0 && t + 1 < nkt) {
            if (t + S - 1 < nkt) wait_vmcnt<(S - 2) * NL>();
            else wait_vmcnt<0>();
        }
    };
    auto barrier = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };

    if (nkt > 0) {
        if (group == 0) {
#pragma unroll
            for (int i = 0; i < S - 1; ++i)
                if (i < nkt) issue(i);
            if (nkt >= S - 1) wait_vmcnt<(S - 2) * NL>();
            else wait_vmcnt<0>();
        }
        barrier();
        // group 0: M C M C ... ; group 1 runs one phase behind (it passes one extra
        // barrier first, group 0 one extra at the end: equal barrier counts)
        if (group == 1) barrier();
        for (int t = 0; t < nkt; ++t) {
#pragma unroll
            for (int ph = 0; ph < NPH; ++ph) {
                memory_phase(t, ph);
                barrier();
                compute_phase(t, ph);
                barrier();
            }
        }
        if (group == 0) barrier();
    }

    if constexpr (EPI == EPI_SWIGLU) {
        static_assert(BM * (BN + 8) <= S * STAGE, "staged SwiGLU tile fits the LDS ring");
        epilogue_swiglu_lds<DT_OUT, FM, FN, BM, BN, 512, false, DT == DT_E4M3>(
            p, acc, smem, m0, n0, wm * TM, wn * TN, lane);
    } else if constexpr (EPI == EPI_GEMM_EX) {
        static_assert(S * STAGE >= 8 * 32 * 36 * 4, "EX staging fits the LDS ring");
        __syncthreads();
        epilogue_gemm_ex_lds<DT_OUT, FM, FN>(p, acc, smem, m0 + wm * TM, n0 + wn * TN,
                                             threadIdx.x >> 6, lane);
    } else {
        epilogue16<DT_OUT, EPI, FM, FN>(p, acc, m0, n0, BM, BN, m0 + wm * TM, n0 + wn * TN,
                                        lane);
    }
}

}  // namespace sg
