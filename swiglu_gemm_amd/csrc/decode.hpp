// decode.hpp -- the decode-shaped GEMM: M <= 32 token rows against a weight
// matrix streamed once from HBM ("GEMM o Coração Matemático" §14: one new token
// per sequence turns the projection into a matrix-vector product whose cost is
// reading the weights; §8: such products sit on the bandwidth side of the
// roofline).  Serves the GEMM (B = W as K x N, or W^T as N x K), the fused
// SwiGLU-GEMM on interleaved W_fused and the split-weight form (W1, W2).
//
// Work distribution (stream-K): the weight is cut into units of BK k-rows by BN
// columns; the units, ordered column tile by column tile and k within a tile, are
// dealt out as equal contiguous runs to a persistent grid of one or two work-groups
// per CU, so every CU streams the same number of bytes whatever the shape.  A
// run covers at most two column tiles partially (its first and last) and any
// number fully.  The direct-to-LDS ring of gemm16_dma.hpp runs on across tile
// boundaries; a fully covered tile goes straight through the register epilogue.
//
// Partially covered tiles: each contributor stores its fp32 partial sums to a
// workspace slot of its own, and a second, small kernel (one work-group per
// column tile) adds the partials of every split tile in k order -- a fixed
// order, so results are run-to-run identical -- and applies the epilogue.  The
// kernel boundary is the only synchronisation: on MI355X an in-kernel hand-off
// needs agent-scope release/acquire fences, i.e. a write-back and invalidate of a
// whole XCD L2 per work-group, which cost more than the streaming itself here.
//
// One 32-row MFMA fragment covers the tokens (rows past M read row M-1 and are
// never stored); the 32 x 32 x k MFMA and the LDS fragment reads are those of
// the large-tile kernel.  Requirements: A 'N' (M x K, rows 16-byte aligned), K a
// multiple of BK = 128 bytes of elements, B rows 16-byte aligned.
#pragma once

#include "gemm16_dma.hpp"

namespace sg {

struct DecodeParams {
    const char* A;      // M x K tokens, row-major
    const char* B;      // 'N': K x N weight; 'T': N x K; EPI_SWIGLU_W12: W1 (K x N/2)
    const char* B2;     // EPI_SWIGLU_W12: W2 (same shape and ld as W1)
    void* C;            // EPI_GEMM: C (bf16 for e4m3 operands); SwiGLU: Y
    int64_t lda, ldb, ldc;
    int M, N, K;        // N: fused width (2 x outputs) for both SwiGLU forms
    float alpha, beta;  // SwiGLU: alpha = scale_a * scale_w
    int vec_c;          // C / Y rows take the widest store of the epilogue
    int tiles, nkb;     // column tiles of BN; K tiles of BK
    int units;          // tiles * nkb
    float* part;        // partial sums: [work-groups][2 slots][BN * 32] fp32
    int grid;           // work-groups of the streaming kernel
    EpiEx ex;           // EPI_GEMM_EX: bias / activation / e4m3 output
};


// Register epilogue of one column tile t.  Accumulator layout as in epilogue16.hpp:
// lane l, register r of fragment tn holds row m = l % 32 and tile column
// wave*TN + tn*32 + 8*(r/4) + 4*(l/32) + r%4.
template <int DT_OUT, int EPI, int BN, int NW, int FN>
__device__ __forceinline__ void decode_store(const DecodeParams& p, const f32x16 (&acc)[FN],
                                             int t, int wave, int lane) {
    constexpr int TN = BN / NW;
    const int m = lane & 31;
    if (m >= p.M) return;
    const int lq = (lane >> 5) * 4;
    uint16_t* out = reinterpret_cast<uint16_t*>(p.C) + (int64_t)m * p.ldc;
    const float a = p.alpha;
    if constexpr (EPI == EPI_GEMM_EX) {
        // the EpiEx steps, element by element; C is indexed in its own element size
        // (2 bytes, or 1 for an e4m3 output)
        void* C = reinterpret_cast<char*>(p.C) + (int64_t)m * p.ldc * (p.ex.out_fp8 ? 1 : 2);
#pragma unroll
        for (int tn = 0; tn < FN; ++tn)
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int n = t * BN + wave * TN + tn * 32 + 8 * g + lq + e;
                    if (n < p.N) store_elem<DT_OUT>(C, n, n, a * acc[tn][4 * g + e], p.beta, p.ex);
                }
    } else if constexpr (EPI == EPI_GEMM) {
        const float beta = p.beta;
#pragma unroll
        for (int tn = 0; tn < FN; ++tn)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = t * BN + wave * TN + tn * 32 + 8 * g + lq;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = a * acc[tn][4 * g + e];
                if (p.vec_c && n + 4 <= p.N) {
                    if (beta != 0.0f) {
                        const u32x2 old = *reinterpret_cast<const u32x2*>(out + n);
                        v[0] += beta * to_f32<DT_OUT>((uint16_t)(old.x & 0xffff));
                        v[1] += beta * to_f32<DT_OUT>((uint16_t)(old.x >> 16));
                        v[2] += beta * to_f32<DT_OUT>((uint16_t)(old.y & 0xffff));
                        v[3] += beta * to_f32<DT_OUT>((uint16_t)(old.y >> 16));
                    }
                    u32x2 o;
                    o.x = pack2<DT_OUT>(v[0], v[1]);
                    o.y = pack2<DT_OUT>(v[2], v[3]);
                    *reinterpret_cast<u32x2*>(out + n) = o;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < p.N) {
                            float x = v[e];
                            if (beta != 0.0f) x += beta * to_f32<DT_OUT>(out[n + e]);
                            out[n + e] = from_f32<DT_OUT>(x);
                        }
                }
            }
    } else if constexpr (EPI == EPI_SWIGLU) {
        // interleaved W_fused: fused columns (2j, 2j+1) sit in registers (r, r+1)
        const int nout = p.N >> 1;
#pragma unroll
        for (int tn = 0; tn < FN; ++tn)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int o = (t * BN + wave * TN + tn * 32 + 8 * g + lq) >> 1;
                const float y0 = silu(a * acc[tn][4 * g]) * (a * acc[tn][4 * g + 1]);
                const float y1 = silu(a * acc[tn][4 * g + 2]) * (a * acc[tn][4 * g + 3]);
                if (p.vec_c && o + 2 <= nout) {
                    *reinterpret_cast<uint32_t*>(out + o) = pack2<DT_OUT>(y0, y1);
                } else {
                    if (o < nout) out[o] = from_f32<DT_OUT>(y0);
                    if (o + 1 < nout) out[o + 1] = from_f32<DT_OUT>(y1);
                }
            }
    } else {
        // split weights: fragment tn < FN/2 is gate, tn + FN/2 the up of the same columns
        constexpr int FH = FN / 2;
        const int nout = p.N >> 1;
#pragma unroll
        for (int tn = 0; tn < FH; ++tn)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int o = t * (BN / 2) + wave * (TN / 2) + tn * 32 + 8 * g + lq;
                float y[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    y[e] = silu(a * acc[tn][4 * g + e]) * (a * acc[tn + FH][4 * g + e]);
                if (p.vec_c && o + 4 <= nout) {
                    u32x2 v;
                    v.x = pack2<DT_OUT>(y[0], y[1]);
                    v.y = pack2<DT_OUT>(y[2], y[3]);
                    *reinterpret_cast<u32x2*>(out + o) = v;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (o + e < nout) out[o + e] = from_f32<DT_OUT>(y[e]);
                }
            }
    }
}

// Partial-sum slot: lane-major f32x4, index ((wave*FN + tn)*4 + g)*64 + lane, so
// each store and load instruction is contiguous; rows m >= M are never touched.
template <int BN, int NW, int FN>
__device__ __forceinline__ f32x4* part_slot(const DecodeParams& p, int w, int slot) {
    return reinterpret_cast<f32x4*>(p.part + ((int64_t)w * 2 + slot) * (BN * 32));
}

template <int DT, bool TB, int EPI, int BN, int S, int NW>
__global__ void __launch_bounds__(64 * NW) decode_kernel(const DecodeParams p) {
    constexpr int ESZ = DT == DT_E4M3 ? 1 : 2;
    constexpr int DT_OUT = DT == DT_E4M3 ? DT_BF16 : DT;
    constexpr int BK = 128 / ESZ;                // k-tile: 128 bytes of each row of A
    constexpr int KSTEP = ESZ == 2 ? 16 : 64;
    constexpr int KS = BK / KSTEP;
    constexpr int TN = BN / NW, FN = TN / 32;
    constexpr bool W12 = EPI == EPI_SWIGLU_W12;
    static_assert(TN % 32 == 0 && KS % 2 == 0, "decode tile");
    static_assert(!W12 || (!TB && FN % 2 == 0), "split-weight decode tile");
    constexpr int BNS = W12 ? BN / 2 : BN;       // columns per weight source
    constexpr int NBS = W12 ? 2 : 1;
    using TA_ = DmaTile<true, 32, BK, ESZ>;
    using TB_ = DmaTile<TB, BNS, BK, ESZ>;
    static_assert(TA_::BLOCKS % NW == 0 && TB_::BLOCKS % NW == 0, "DMA blocks per wave");
    constexpr int NIA = TA_::BLOCKS / NW, NIB = TB_::BLOCKS / NW;
    constexpr int NL = NIA + NBS * NIB;          // DMA instructions per thread per unit
    static_assert((S - 2) * NL < 64, "vmcnt range");
    constexpr int STAGE = TA_::BYTES + NBS * TB_::BYTES;
    static_assert(S * STAGE <= 160 * 1024, "LDS budget");
    using Frag = typename FragT<ESZ>::type;
    __shared__ __attribute__((aligned(1024))) char smem[S * STAGE];

    const int G = p.grid;
    const int w = xcd_remap(blockIdx.x, G);      // neighbouring runs share an XCD
    const int ub = sk_start(w, p.units, G), ue = sk_start(w + 1, p.units, G);
    const int n = ue - ub;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;

    // Per-lane DMA addresses without the unit's offsets: A [32][BK] (rows past M
    // read row M-1); B row-contiguous [BK][BNS] (16-byte chunks past the last
    // column read the last chunk) or k-contiguous [BNS][BK] (rows past N read N-1).
    const char* ga[NIA];
#pragma unroll
    for (int i = 0; i < NIA; ++i) {
        const int chunk = (wave + i * NW) * 64 + lane;
        const int row = chunk / TA_::SLOTS, slot = chunk % TA_::SLOTS;
        ga[i] = p.A + (int64_t)min(row, p.M - 1) * p.lda * ESZ + ((slot ^ TA_::swz(row)) << 4);
    }
    const int nb_src = W12 ? p.N / 2 : p.N;      // columns of each weight source
    int64_t boff[NIB];                           // 'N': k-row offset; 'T': chunk offset
    int bcol[NIB];                               // 'N': byte column in tile; 'T': tile row
#pragma unroll
    for (int i = 0; i < NIB; ++i) {
        const int chunk = (wave + i * NW) * 64 + lane;
        const int row = chunk / TB_::SLOTS, slot = chunk % TB_::SLOTS;
        if constexpr (TB) {
            boff[i] = (int64_t)((slot ^ TB_::swz(row)) << 4);
            bcol[i] = row;
        } else {
            boff[i] = (int64_t)row * p.ldb * ESZ;
            bcol[i] = (((slot >> 1) ^ TB_::swz(row)) << 5) + ((slot & 1) << 4);
        }
    }
    auto issue = [&](int i) {                    // DMA of relative unit i
        const int u = ub + i;
        const int t = u / p.nkb, kb = u - t * p.nkb;
        char* st = smem + (i % S) * STAGE;
#pragma unroll
        for (int j = 0; j < NIA; ++j) {
            const uint32_t lds = (uint32_t)(uintptr_t)(
                (__attribute__((address_space(3))) char*)(st + (wave + j * NW) * 1024));
            const char* g = ga[j] + kb * (BK * ESZ);
            asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                         :: "s"(lds), "v"(g) : "memory", "m0");
        }
#pragma unroll
        for (int src = 0; src < NBS; ++src) {
            const char* base = src == 0 ? p.B : p.B2;
            char* sb = st + TA_::BYTES + src * TB_::BYTES;
#pragma unroll
            for (int j = 0; j < NIB; ++j) {
                const uint32_t lds = (uint32_t)(uintptr_t)(
                    (__attribute__((address_space(3))) char*)(sb + (wave + j * NW) * 1024));
                const char* g;
                if constexpr (TB) {
                    const int r = min(t * BNS + bcol[j], nb_src - 1);
                    g = base + (int64_t)r * p.ldb * ESZ + (int64_t)kb * (BK * ESZ) + boff[j];
                } else {
                    const int cb = min(t * (BNS * ESZ) + bcol[j], nb_src * ESZ - 16);
                    g = base + (int64_t)kb * BK * p.ldb * ESZ + boff[j] + cb;
                }
                asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                             :: "s"(lds), "v"(g) : "memory", "m0");
            }
        }
    };

    f32x16 acc[FN];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][e] = 0.0f;
    Frag fa[2], fb[2][FN];
    auto read_all = [&](const char* st, int s, Frag& af, Frag (&bf)[FN]) {
        af = read_frag<true, 32, BK, ESZ>(st, 0, s, lane);
#pragma unroll
        for (int tn = 0; tn < FN; ++tn) {
            if constexpr (W12) {
                constexpr int FH = FN / 2;
                const char* half = st + TA_::BYTES + (tn / FH) * TB_::BYTES;
                bf[tn] = read_frag<false, BNS, BK, ESZ>(half, wave * (TN / 2) + (tn % FH) * 32, s,
                                                       lane);
            } else {
                bf[tn] = read_frag<TB, BN, BK, ESZ>(st + TA_::BYTES, wave * TN + tn * 32, s, lane);
            }
        }
    };
    auto mfma_all = [&](const Frag& af, const Frag (&bf)[FN]) {
#pragma unroll
        for (int tn = 0; tn < FN; ++tn) acc[tn] = mfma_op<DT>(bf[tn], af, acc[tn]);
    };

    {
#pragma unroll
        for (int i = 0; i < S - 1; ++i)
            if (i < n) issue(i);
        if (n >= S - 1) wait_vmcnt<(S - 2) * NL>();
        else wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        read_all(smem, 0, fa[0], fb[0]);

        int t = ub / p.nkb, kb = ub - t * p.nkb;
        int seg_k0 = kb, seg = 0;
        for (int i = 0; i < n; ++i) {
            const char* cur = smem + (i % S) * STAGE;
            const bool ahead = i + S - 1 < n;
            if (ahead) issue(i + S - 1);
#pragma unroll
            for (int s = 0; s + 1 < KS; ++s) {
                read_all(cur, s + 1, fa[(s + 1) & 1], fb[(s + 1) & 1]);
                mfma_all(fa[s & 1], fb[s & 1]);
            }
            if (ahead) wait_vmcnt<(S - 2) * NL>();
            else wait_vmcnt<0>();
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            // the next unit's first fragments (stale and unused after the last unit)
            read_all(smem + ((i + 1) % S) * STAGE, 0, fa[0], fb[0]);
            mfma_all(fa[1], fb[1]);
            __builtin_amdgcn_sched_barrier(0);

            if (kb == p.nkb - 1 || i == n - 1) {     // a segment of tile t ends here
                if (seg_k0 == 0 && kb == p.nkb - 1) {
                    decode_store<DT_OUT, EPI, BN, NW, FN>(p, acc, t, wave, lane);
                } else {
                    const int slot = seg == 0 ? 0 : 1;   // first or last segment of the run
                    if ((lane & 31) < p.M) {
                        f32x4* ps = part_slot<BN, NW, FN>(p, w, slot);
#pragma unroll
                        for (int tn = 0; tn < FN; ++tn)
#pragma unroll
                            for (int g = 0; g < 4; ++g)
                                ps[((wave * FN + tn) * 4 + g) * 64 + lane] =
                                    f32x4{acc[tn][4 * g], acc[tn][4 * g + 1], acc[tn][4 * g + 2],
                                          acc[tn][4 * g + 3]};
                    }
                }
#pragma unroll
                for (int tn = 0; tn < FN; ++tn)
#pragma unroll
                    for (int e = 0; e < 16; ++e) acc[tn][e] = 0.0f;
                ++seg;
                ++t;
                kb = 0;
                seg_k0 = 0;
            } else {
                ++kb;
            }
        }
    }
}

// Finish the split column tiles: work-group tt adds the partials of its
// contributors (the runs that hold its first through last unit) in k order and
// applies the epilogue; a tile that one run covered was stored by that run.
template <int DT, int EPI, int BN, int NW>
__global__ void __launch_bounds__(64 * NW) decode_fixup_kernel(const DecodeParams p) {
    constexpr int DT_OUT = DT == DT_E4M3 ? DT_BF16 : DT;
    constexpr int FN = BN / NW / 32;
    const int tt = blockIdx.x, G = p.grid;
    const int wa = sk_owner(tt * p.nkb, p.units, G);
    const int wz = sk_owner((tt + 1) * p.nkb - 1, p.units, G);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (wa == wz || (lane & 31) >= p.M) return;
    f32x16 acc[FN];
#pragma unroll
    for (int tn = 0; tn < FN; ++tn)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[tn][e] = 0.0f;
    // CH contributors' loads in flight at once, then added in k order
    constexpr int CH = FN == 1 ? 8 : 4;
    for (int c0 = wa; c0 <= wz; c0 += CH) {
        f32x4 v[CH][FN][4];
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const int c = c0 + j;
            if (c > wz) break;
            // slot 0 when run c starts in tile tt, else tile tt is its last segment
            const int cs = sk_start(c, p.units, G) / p.nkb == tt ? 0 : 1;
            const f32x4* ps = part_slot<BN, NW, FN>(p, c, cs);
#pragma unroll
            for (int tn = 0; tn < FN; ++tn)
#pragma unroll
                for (int g = 0; g < 4; ++g) v[j][tn][g] = ps[((wave * FN + tn) * 4 + g) * 64 + lane];
        }
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            if (c0 + j > wz) break;
#pragma unroll
            for (int tn = 0; tn < FN; ++tn)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    acc[tn][4 * g] += v[j][tn][g].x;
                    acc[tn][4 * g + 1] += v[j][tn][g].y;
                    acc[tn][4 * g + 2] += v[j][tn][g].z;
                    acc[tn][4 * g + 3] += v[j][tn][g].w;
                }
        }
    }
    decode_store<DT_OUT, EPI, BN, NW, FN>(p, acc, tt, wave, lane);
}

// Decode configurations: columns per tile, ring depth, waves, work-groups per CU.
struct DecodeCfg {
    int BN, S, NW, occ;
    const char* name;
};
constexpr DecodeCfg kDecodeCfg[] = {
    {128, 6, 4, 1, "decode 128 s6 4w x1"},
    {256, 4, 4, 1, "decode 256 s4 4w x1"},
    {128, 3, 4, 2, "decode 128 s3 4w x2"},
    {128, 7, 4, 1, "decode 128 s7 4w x1"},
    {256, 2, 4, 2, "decode 256 s2 4w x2"},
    {128, 4, 4, 1, "decode 128 s4 4w x1"},
    {128, 2, 4, 2, "decode 128 s2 4w x2"},
};
constexpr int kNumDecodeCfg = sizeof(kDecodeCfg) / sizeof(kDecodeCfg[0]);

#define SG_DECODE_CONFIGS(X) \
    X(0, 128, 6, 4)          \
    X(1, 256, 4, 4)          \
    X(2, 128, 3, 4)          \
    X(3, 128, 7, 4)          \
    X(4, 256, 2, 4)          \
    X(5, 128, 4, 4)          \
    X(6, 128, 2, 4)

#define SG_DECODE_CONFIGS_EX(X) X(5, 128, 4, 4)

// The streaming kernel on p.grid work-groups, then (split: some column tile is
// shared by several runs) the fix-up kernel over the column tiles.
template <int DT, bool TB, int EPI>
hipError_t launch_decode_cfg(int cfg, const DecodeParams& p, bool split, hipStream_t st) {
#define SG_DCASE(ID, BN, S, NW)                                                             \
    case ID:                                                                                \
        if constexpr (EPI != EPI_SWIGLU_W12 || (BN / NW / 32) % 2 == 0) {                  \
            hipLaunchKernelGGL((decode_kernel<DT, TB, EPI, BN, S, NW>), dim3(p.grid),        \
                               dim3(64 * NW), 0, st, p);                                     \
            if (split)                                                                      \
                hipLaunchKernelGGL((decode_fixup_kernel<DT, EPI, BN, NW>), dim3(p.tiles),    \
                                   dim3(64 * NW), 0, st, p);                                 \
            return hipGetLastError();                                                       \
        } else {                                                                            \
            return hipErrorInvalidValue;                                                    \
        }
    if constexpr (EPI == EPI_GEMM_EX) {   // the extra epilogue steps: the default tile only
        switch (cfg) {
            SG_DECODE_CONFIGS_EX(SG_DCASE)
            default: return hipErrorInvalidValue;
        }
    } else {
        switch (cfg) {
            SG_DECODE_CONFIGS(SG_DCASE)
            default: return hipErrorInvalidValue;
        }
    }
#undef SG_DCASE
}

// epi: EPI_GEMM / EPI_GEMM_EX ('N' or 'T' weight), EPI_SWIGLU and EPI_SWIGLU_W12
// ('N' only).
template <int DT>
hipError_t launch_decode_dt(bool tb, int epi, int cfg, const DecodeParams& p, bool split,
                            hipStream_t st) {
    if (epi == EPI_GEMM)
        return tb ? launch_decode_cfg<DT, true, EPI_GEMM>(cfg, p, split, st)
                  : launch_decode_cfg<DT, false, EPI_GEMM>(cfg, p, split, st);
    if (epi == EPI_GEMM_EX)
        return tb ? launch_decode_cfg<DT, true, EPI_GEMM_EX>(cfg, p, split, st)
                  : launch_decode_cfg<DT, false, EPI_GEMM_EX>(cfg, p, split, st);
    if (tb) return hipErrorInvalidValue;
    if (epi == EPI_SWIGLU) return launch_decode_cfg<DT, false, EPI_SWIGLU>(cfg, p, split, st);
    if (epi == EPI_SWIGLU_W12)
        return launch_decode_cfg<DT, false, EPI_SWIGLU_W12>(cfg, p, split, st);
    return hipErrorInvalidValue;
}

}  // namespace sg
