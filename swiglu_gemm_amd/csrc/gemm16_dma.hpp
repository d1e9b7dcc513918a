// gemm16_dma.hpp -- fp16 / bf16 MFMA GEMM with direct global->LDS loads (gfx950).
//
// Same arithmetic and epilogues as gemm16.hpp (acc = op(A)_tile * op(B)_tile in
// fp32 with v_mfma_f32_32x32x16_{f16,bf16}, transposed accumulator D^T), but the
// tiles travel from global memory straight into LDS with global_load_lds_dwordx4
// (16 bytes per lane, no VGPR staging), through a ring of S LDS stages, so loads
// run S-1 tiles ahead of the MFMAs.
//
// LDS layouts, chosen so both operand orientations feed the MFMA directly:
// * k-contiguous operand (A 'N', B 'T'): [R][BK] with 16-byte chunks XOR-swizzled
//   by row; an MFMA fragment (32 rows x 8 k per lane) is one ds_read_b128.
// * row-contiguous operand (A 'T', B 'N', W_fused): [BK][R] as stored in memory,
//   32-byte units XOR-swizzled by k; the fragment is two ds_read_b64_tr_b16
//   (each 16-lane group turns four 32-byte row pieces into 4 k-values per lane).
// The DMA writes 1 KiB per wave instruction in lane order; the swizzle is applied
// by choosing which global 16-byte chunk each lane fetches.
//
// W_fused keeps its interleaved column order here: in the D^T accumulator layout
// fused columns (2n, 2n+1) land in registers (r, r+1) of one lane, so the SwiGLU
// epilogue pairs them in place ("Resumo Técnico: Sobreposição de Ativação em Nível
// de Tile ...", Metodologia / Kernel-2).
//
// Used only when every tile is full (M % BM == N % BN == 0, K-split lengths a
// multiple of BK) and operands are 16-byte aligned with ld % 8 == 0; other
// problems take the register-staged kernel of gemm16.hpp.
#pragma once

#include "epilogue16.hpp"
#include "sg_device.hpp"

namespace sg {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

template <bool KC, int R, int BK>
struct DmaTile {
    static constexpr int ROW_BYTES = KC ? BK * 2 : R * 2;
    static constexpr int BYTES = R * BK * 2;
    static constexpr int SLOTS = ROW_BYTES / 16;         // 16-byte slots per row
    static constexpr int ROWS_PER_KB = 1024 / ROW_BYTES;  // rows per 1 KiB DMA block
    static constexpr int BLOCKS = BYTES / 1024;
    static_assert(ROW_BYTES <= 1024 && 1024 % ROW_BYTES == 0, "row must divide 1 KiB");
    static_assert(KC ? (BK == 32 || BK == 64) : (R >= 128), "unsupported tile");

    // physical 16-byte chunk (KC) or 32-byte unit (row-contiguous) for a row
    static __device__ __forceinline__ int swz(int row) {
        if constexpr (KC) {
            if constexpr (BK == 64) return (row & 7) ^ ((row >> 3) & 1);
            else return (row >> 2) & 3;
        } else {
            return (row & 3) << 1;
        }
    }
};

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// One operand's DMA stream: NI instructions per thread per K tile.
template <bool KC, int R, int BK, int NWAVES>
struct DmaStream {
    using T = DmaTile<KC, R, BK>;
    static_assert(T::BLOCKS % NWAVES == 0, "DMA blocks must split evenly over the waves");
    static constexpr int NI = T::BLOCKS / NWAVES;
    const uint16_t* gp[NI];
    int64_t step;   // elements to advance per K tile

    __device__ __forceinline__ void init(const uint16_t* base, int64_t ld, int r0, int k0,
                                         int wave, int lane) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int b = wave + i * NWAVES;
            const int row = b * T::ROWS_PER_KB + lane / T::SLOTS;
            const int slot = lane % T::SLOTS;
            if constexpr (KC) {
                const int c = slot ^ T::swz(row);
                gp[i] = base + (int64_t)(r0 + row) * ld + (k0 + c * 8);
            } else {
                const int u = (slot >> 1) ^ T::swz(row);
                gp[i] = base + (int64_t)(k0 + row) * ld + (r0 + u * 16 + (slot & 1) * 8);
            }
        }
        step = KC ? (int64_t)BK : (int64_t)BK * ld;
    }
    // Issue the DMA of K tile `t` (relative to the split start) into stage memory.
    // Written as inline asm so the compiler does not model the asynchronous LDS
    // write (it would otherwise drain every outstanding load before each LDS
    // read); completion is enforced by wait_vmcnt + s_barrier in the main loop.
    __device__ __forceinline__ void issue(char* stage, int t, int wave) const {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int b = wave + i * NWAVES;
            const uint32_t lds = (uint32_t)(uintptr_t)(
                (__attribute__((address_space(3))) char*)(stage + b * 1024));
            const uint16_t* g = gp[i] + t * step;
            asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                         :: "s"(lds), "v"(g) : "memory", "m0");
        }
    }
};

// MFMA fragment: 32 rows (rbase + lane%32) x 8 k (16*s + 8*(lane/32) + 0..7).
template <bool KC, int R, int BK>
__device__ __forceinline__ u32x4 read_frag(const char* tile, int rbase, int s, int lane) {
    using T = DmaTile<KC, R, BK>;
    if constexpr (KC) {
        const int row = rbase + (lane & 31);
        const int chunk = 2 * s + (lane >> 5);
        return *reinterpret_cast<const u32x4*>(tile + row * T::ROW_BYTES +
                                               ((chunk ^ T::swz(row)) << 4));
    } else {
        const int g = lane >> 4, L = lane & 15, j = L >> 2, q = L & 3;
        const int r = rbase + 16 * (g & 1) + 4 * q;
        const int k0 = 16 * s + 8 * (g >> 1) + j;
        const int k1 = k0 + 4;
        const char* p0 = tile + k0 * T::ROW_BYTES + (((r >> 4) ^ T::swz(k0)) << 5) + ((r & 15) << 1);
        const char* p1 = tile + k1 * T::ROW_BYTES + (((r >> 4) ^ T::swz(k1)) << 5) + ((r & 15) << 1);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p1));
        const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
        return u32x4{a.x, a.y, b.x, b.y};
    }
}

template <int DT, bool TA, bool TB, int EPI, int BM, int BN, int BK, int S, int WM, int WN>
__global__ void __launch_bounds__(64 * WM * WN, 1) gemm16_dma_kernel(const Gemm16Params p) {
    constexpr int NW = WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    constexpr int KS = BK / 16;
    static_assert(KS % 2 == 0, "k-steps per tile must be even (fragment double buffer)");
    constexpr bool KCA = !TA, KCB = TB;          // k-contiguous operands
    using TA_ = DmaTile<KCA, BM, BK>;
    using TB_ = DmaTile<KCB, BN, BK>;
    constexpr int STAGE = TA_::BYTES + TB_::BYTES;
    static_assert(S * STAGE <= 160 * 1024, "LDS budget");
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
    const int wm = wave % WM, wn = wave / WM;

    DmaStream<KCA, BM, BK, NW> da;
    DmaStream<KCB, BN, BK, NW> db;
    da.init(p.A, p.lda, m0, kbeg, wave, lane);
    db.init(p.B, p.ldb, n0, kbeg, wave, lane);
    constexpr int NL = DmaStream<KCA, BM, BK, NW>::NI + DmaStream<KCB, BN, BK, NW>::NI;

    f32x16 acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    u32x4 fa[2][FM], fb[2][FN];
    auto read_all = [&](const char* st, int s, u32x4 (&af)[FM], u32x4 (&bf)[FN]) {
#pragma unroll
        for (int tm = 0; tm < FM; ++tm) af[tm] = read_frag<KCA, BM, BK>(st, wm * TM + tm * 32, s, lane);
#pragma unroll
        for (int tn = 0; tn < FN; ++tn)
            bf[tn] = read_frag<KCB, BN, BK>(st + TA_::BYTES, wn * TN + tn * 32, s, lane);
    };
    auto mfma_all = [&](const u32x4 (&af)[FM], const u32x4 (&bf)[FN]) {
#pragma unroll
        for (int tn = 0; tn < FN; ++tn)
#pragma unroll
            for (int tm = 0; tm < FM; ++tm) acc[tn][tm] = mfma16<DT>(bf[tn], af[tm], acc[tn][tm]);
    };
    auto issue = [&](int t) {
        char* st = smem + (t % S) * STAGE;
        da.issue(st, t, wave);
        db.issue(st + TA_::BYTES, t, wave);
    };

    if (nkt > 0) {
#pragma unroll
        for (int i = 0; i < S - 1; ++i)
            if (i < nkt) issue(i);
        if (nkt >= S - 1) wait_vmcnt<(S - 2) * NL>();
        else wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        read_all(smem, 0, fa[0], fb[0]);

        constexpr int NMF = FM * FN;
        constexpr int NRD = (KCA ? FM : 2 * FM) + (KCB ? FN : 2 * FN);
        for (int t = 0; t < nkt; ++t) {
            const char* cur = smem + (t % S) * STAGE;
            const bool ahead = t + S - 1 < nkt;
            if (ahead) issue(t + S - 1);
#pragma unroll
            for (int s = 0; s + 1 < KS; ++s) {
                read_all(cur, s + 1, fa[(s + 1) & 1], fb[(s + 1) & 1]);
                mfma_all(fa[s & 1], fb[s & 1]);
                sched_interleave<NMF, NRD, 0, 0>();
                __builtin_amdgcn_sched_barrier(0);
            }
            // tile t+1 must have landed (own DMAs), then everyone's
            if (ahead) wait_vmcnt<(S - 2) * NL>();
            else wait_vmcnt<0>();
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            // last k-step of tile t overlaps the first fragments of tile t+1 (on
            // the last tile this reads a stale stage whose values are never used)
            read_all(smem + ((t + 1) % S) * STAGE, 0, fa[0], fb[0]);
            mfma_all(fa[1], fb[1]);
            sched_interleave<NMF, NRD, 0, 0>();
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    epilogue16<DT, EPI, true, FM, FN>(p, acc, m0, n0, BM, BN, m0 + wm * TM, n0 + wn * TN, lane);
}

}  // namespace sg
