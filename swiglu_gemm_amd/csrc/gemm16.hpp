// gemm16.hpp -- MFMA GEMM main loop for 16-bit operands (fp16 / bf16) on gfx950.
//
// Computes, per output tile, acc = op(A)_tile * op(B)_tile in fp32 with
// v_mfma_f32_32x32x16_{f16,bf16}, then one of three epilogues:
//   EPI_GEMM    C = alpha*acc + beta*C_old (the BLAS update of "GEMM o Coração
//               Matemático" §1), rounded once to the output type;
//   EPI_SWIGLU  Y[m,n] = SiLU(s*acc[m,2n]) * (s*acc[m,2n+1]) over the column-
//               interleaved W_fused ("Resumo Técnico: Sobreposição de Ativação em
//               Nível de Tile ...", Metodologia / Kernel-2 pair epilogue);
//   EPI_PARTIAL fp32 partial sums of one K-split to a workspace (split-K of
//               "为什么 GEMM 是 CUDA 的必修课", 生产级 GEMM 的多级分块 item 5); the
//               reduction applies the real epilogue after all splits are summed.
//
// Design (gfx950, wave64):
// * One work-group computes a BM x BN tile with WM x WN waves; each wave owns a
//   (BM/WM) x (BN/WN) register tile of 32x32 MFMA accumulators.
// * The MFMA computes the transposed tile D^T = op(B)^T op(A)^T: its first
//   operand is 32 rows of the B tile (output columns), its second 32 rows of the
//   A tile.  In the 32x32 accumulator layout each lane then holds four
//   consecutive output COLUMNS per register quad, so stores are 8/16-byte
//   vectors and a gate/up pair can live in the same lane and register index.
// * Both tiles sit in LDS as [row][BK=64] with k contiguous (128 B rows), so every
//   MFMA operand is one 16-byte ds_read per lane.  16-byte chunks are XOR-swizzled
//   by row (chunk ^ f(row)) so the 8/16 lanes of one LDS phase hit distinct banks.
// * Operands whose rows are k-contiguous in memory (A 'N', B 'T') are copied in
//   16-byte chunks.  Operands stored the other way (A 'T', B 'N', and W_fused)
//   are read as 8x8 blocks of 16-byte row pieces and transposed in registers
//   (v_perm) before the 16-byte LDS store, so the LDS layout is the same for all
//   four transpose combinations.  For SwiGLU the same store also de-interleaves
//   W_fused: within each group of 64 fused columns the 32 gate columns go to LDS
//   rows [0,32) and the 32 up columns to rows [32,64).
// * Two LDS stages; the next K tile is prefetched into registers while the
//   current one feeds the MFMAs; one barrier per K tile.
// * Tiles entirely inside M x N with 16-byte-aligned operands take an unguarded
//   path; edge tiles and the K tail zero-fill out-of-range elements so every
//   wave still reaches every barrier, and stores are predicated.
#pragma once

#include <type_traits>

#include "epilogue16.hpp"
#include "sg_device.hpp"

namespace sg {


constexpr int BK16 = 64;

__device__ __forceinline__ int lds_swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int lds_off(int row, int chunk) {
    return row * 128 + ((chunk ^ lds_swz(row)) << 4);
}

// 8 consecutive 16-bit elements starting at p; elements at or beyond `left` and
// whole chunks with !ok read as zero and are never dereferenced.
__device__ __forceinline__ u32x4 load8_guarded(const uint16_t* p, bool ok, int left, bool vec) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (!ok || left <= 0) return v;
    if (vec && left >= 8) return *reinterpret_cast<const u32x4*>(p);
    uint32_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = (e < left) ? (uint32_t)p[e] : 0u;
    v.x = h[0] | (h[1] << 16);
    v.y = h[2] | (h[3] << 16);
    v.z = h[4] | (h[5] << 16);
    v.w = h[6] | (h[7] << 16);
    return v;
}

// Tile rows are k-contiguous in memory: element (r, k) at base[r*ld + k].
template <int R, int NT>
struct LoadDirect {
    static constexpr int CH = R * 8 / NT;
    static_assert((R * 8) % NT == 0, "tile rows must split evenly over the threads");
    static constexpr int NLOAD = CH, NSTORE = CH;   // global loads / LDS stores per thread
    u32x4 v[CH];

    __device__ __forceinline__ void load(const uint16_t* base, int64_t ld, int r0, int rows,
                                         int k0, int kend, bool fast, bool vec) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = threadIdx.x + i * NT;
            const int row = c >> 3, kc = c & 7;
            const uint16_t* p = base + (int64_t)(r0 + row) * ld + (k0 + kc * 8);
            if (fast)
                v[i] = *reinterpret_cast<const u32x4*>(p);
            else
                v[i] = load8_guarded(p, r0 + row < rows, kend - (k0 + kc * 8), vec);
        }
    }
    __device__ __forceinline__ void store(char* lds) const {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = threadIdx.x + i * NT;
            const int row = c >> 3, kc = c & 7;
            *reinterpret_cast<u32x4*>(lds + lds_off(row, kc)) = v[i];
        }
    }
};

// Tile rows are contiguous along the row index in memory: element (r, k) at
// base[k*ld + r].  Each thread moves 8x8 blocks (8 k-rows x 8 r) and transposes
// them in registers.  DEINTERLEAVE maps fused W columns to the gate/up LDS rows.
template <int R, int NT, bool DEINTERLEAVE>
struct LoadTrans {
    static constexpr int NB = R;                  // (BK/8) * (R/8) blocks
    static constexpr int BPT = (NB + NT - 1) / NT;
    static constexpr int NLOAD = BPT * 8, NSTORE = BPT * 8;
    u32x4 v[BPT][8];

    __device__ __forceinline__ void load(const uint16_t* base, int64_t ld, int r0, int rows,
                                         int k0, int kend, bool fast, bool vec) {
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
            const int b = threadIdx.x + i * NT;
            if ((NB % NT) != 0 && b >= NB) continue;
            const int kb = b & 7, rb = b >> 3;
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                const int k = k0 + kb * 8 + kk;
                const uint16_t* p = base + (int64_t)k * ld + (r0 + rb * 8);
                if (fast)
                    v[i][kk] = *reinterpret_cast<const u32x4*>(p);
                else
                    v[i][kk] = load8_guarded(p, k < kend, rows - (r0 + rb * 8), vec);
            }
        }
    }

    static __device__ __forceinline__ uint32_t pick(uint32_t a, uint32_t b, bool hi) {
        return hi ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
    }
    static __device__ __forceinline__ uint32_t lane_word(const u32x4& x, int w) {
        return w == 0 ? x.x : (w == 1 ? x.y : (w == 2 ? x.z : x.w));
    }

    __device__ __forceinline__ void store(char* lds) const {
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
            const int b = threadIdx.x + i * NT;
            if ((NB % NT) != 0 && b >= NB) continue;
            const int kb = b & 7, rb = b >> 3;
#pragma unroll
            for (int rr = 0; rr < 8; ++rr) {
                const bool hi = rr & 1;
                const int w = rr >> 1;
                u32x4 o;
                o.x = pick(lane_word(v[i][0], w), lane_word(v[i][1], w), hi);
                o.y = pick(lane_word(v[i][2], w), lane_word(v[i][3], w), hi);
                o.z = pick(lane_word(v[i][4], w), lane_word(v[i][5], w), hi);
                o.w = pick(lane_word(v[i][6], w), lane_word(v[i][7], w), hi);
                int row = rb * 8 + rr;
                if (DEINTERLEAVE) {
                    const int c = row >> 1, up = row & 1;
                    row = (c >> 5) * 64 + up * 32 + (c & 31);
                }
                *reinterpret_cast<u32x4*>(lds + lds_off(row, kb)) = o;
            }
        }
    }
};

template <int DT, bool TA, bool TB, int EPI, int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(64 * WM * WN, 1) gemm16_kernel(const Gemm16Params p_) {
    const Gemm16Params p = batch_item(p_);
    constexpr int NT = 64 * WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be a multiple of 32");
    static_assert(EPI != EPI_SWIGLU || (TN % 64) == 0, "SwiGLU wave tile pairs 32 gate + 32 up");
    constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128, STAGE = A_BYTES + B_BYTES;
    __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

    const int nblk = p.tiles_m * p.tiles_n;
    const int lid = xcd_remap(blockIdx.x, nblk);
    int tmi, tni;
    tile_coords(lid, p.tiles_m, p.tiles_n, p.group_m, tmi, tni);
    const int m0 = tmi * BM, n0 = tni * BN;
    const int kbeg = blockIdx.y * p.k_per_split;
    const int kend = min(p.K, kbeg + p.k_per_split);
    const int nkt = kend > kbeg ? (kend - kbeg + BK16 - 1) / BK16 : 0;

    const bool full_mn = (m0 + BM <= p.M) && (n0 + BN <= p.N) && p.vec_a && p.vec_b;
    const bool vec_a = p.vec_a, vec_b = p.vec_b;

    using LA = std::conditional_t<TA, LoadTrans<BM, NT, false>, LoadDirect<BM, NT>>;
    using LB = std::conditional_t<TB, LoadDirect<BN, NT>,
                                  LoadTrans<BN, NT, EPI == EPI_SWIGLU>>;
    LA la;
    LB lb;

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wm = wave % WM, wn = wave / WM;

    f32x16 acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    // Software pipeline over K tiles (two LDS stages, fragments double-buffered
    // in registers).  Per tile: k-steps 0..2 each read the fragments of the next
    // k-step while their own MFMAs run; the next tile's global loads are issued
    // with k-step 0 and written to the other LDS stage with k-step 2; after the
    // barrier, the MFMAs of k-step 3 overlap the reads of the next tile's first
    // fragments, so the MFMA pipe stays busy across the barrier.
    if (nkt > 0) {
        const char* const stage0 = smem;
        const int kfull = full_mn ? (kend - kbeg) / BK16 : 0;   // tiles loadable unguarded

        u32x4 fa[2][FM], fb[2][FN];
        auto read_frags = [&](const char* st, int s, u32x4 (&af)[FM], u32x4 (&bf)[FN]) {
            const int chunk = 2 * s + (lane >> 5);
#pragma unroll
            for (int tm = 0; tm < FM; ++tm) {
                const int row = wm * TM + tm * 32 + (lane & 31);
                af[tm] = *reinterpret_cast<const u32x4*>(st + lds_off(row, chunk));
            }
#pragma unroll
            for (int tn = 0; tn < FN; ++tn) {
                const int row = wn * TN + tn * 32 + (lane & 31);
                bf[tn] = *reinterpret_cast<const u32x4*>(st + A_BYTES + lds_off(row, chunk));
            }
        };
        auto mfma_step = [&](const u32x4 (&af)[FM], const u32x4 (&bf)[FN]) {
#pragma unroll
            for (int tn = 0; tn < FN; ++tn)
#pragma unroll
                for (int tm = 0; tm < FM; ++tm)
                    acc[tn][tm] = mfma16<DT>(bf[tn], af[tm], acc[tn][tm]);
        };
        auto load_tile = [&](int t, bool fast) {
            const int k0 = kbeg + t * BK16;
            la.load(p.A, p.lda, m0, p.M, k0, kend, fast, vec_a);
            lb.load(p.B, p.ldb, n0, p.N, k0, kend, fast, vec_b);
        };

        load_tile(0, kfull > 0);
        la.store(smem);
        lb.store(smem + A_BYTES);
        __syncthreads();
        read_frags(stage0, 0, fa[0], fb[0]);

        // FAST: the next tile is loaded without guards (branch-free body)
        constexpr int NMF = FM * FN;           // MFMAs per k-step
        constexpr int NFR = FM + FN;           // fragment reads per k-step
        constexpr int NGL = LA::NLOAD + LB::NLOAD;
        constexpr int NST = LA::NSTORE + LB::NSTORE;
        auto body = [&](int kt, auto fast_tag) {
            constexpr bool FAST = decltype(fast_tag)::value;
            const char* cur = smem + (kt & 1) * STAGE;
            char* nxt = smem + ((kt & 1) ^ 1) * STAGE;
            const bool more = FAST || (kt + 1 < nkt);
            // k-step 0 (+ next tile's global loads)
            if (FAST) load_tile(kt + 1, true);
            else if (more) load_tile(kt + 1, false);
            read_frags(cur, 1, fa[1], fb[1]);
            mfma_step(fa[0], fb[0]);
            if (FAST) sched_interleave<NMF, NFR, NGL, 0>();
            __builtin_amdgcn_sched_barrier(0);
            // k-step 1
            read_frags(cur, 2, fa[0], fb[0]);
            mfma_step(fa[1], fb[1]);
            sched_interleave<NMF, NFR, 0, 0>();
            __builtin_amdgcn_sched_barrier(0);
            // k-step 2 (+ the next tile to the other stage)
            read_frags(cur, 3, fa[1], fb[1]);
            mfma_step(fa[0], fb[0]);
            if (more) {
                la.store(nxt);
                lb.store(nxt + A_BYTES);
            }
            // LDS reads (this stage) first, then the writes (other stage): the
            // compiler cannot prove the two stages disjoint, so keep program order
            if (FAST) {
                sched_interleave<NMF / 2, NFR, 0, 0>();
                sched_interleave<NMF - NMF / 2, 0, 0, NST>();
            }
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();
            // k-step 3 overlapping the next tile's first fragments
            if (more) read_frags(nxt, 0, fa[0], fb[0]);
            mfma_step(fa[1], fb[1]);
            if (FAST) sched_interleave<NMF, NFR, 0, 0>();
            __builtin_amdgcn_sched_barrier(0);
        };
        int kt = 0;
        for (; kt + 1 < kfull; ++kt) body(kt, std::true_type{});
        for (; kt < nkt; ++kt) body(kt, std::false_type{});
    }

    if constexpr (EPI == EPI_GEMM_EX) {
        static_assert(2 * STAGE >= (NT / 64) * 32 * 36 * 4, "EX staging fits the LDS ring");
        __syncthreads();
        epilogue_gemm_ex_lds<DT, FM, FN>(p, acc, smem, m0 + wm * TM, n0 + wn * TN,
                                         threadIdx.x >> 6, lane);
    } else {
        epilogue16<DT, EPI, FM, FN>(p, acc, m0, n0, BM, BN, m0 + wm * TM, n0 + wn * TN, lane);
    }
}

}  // namespace sg
