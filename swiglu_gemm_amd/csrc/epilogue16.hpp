// epilogue16.hpp -- register-resident epilogues of the MFMA GEMM kernels.
//
// The kernels accumulate the transposed tile D^T in v_mfma_f32_32x32x* layout:
// accumulator acc[tn][tm], lane l, register r holds the fp32 sum for
//   m = mb + tm*32 + (l & 31),   n = nb + tn*32 + 8*(r/4) + 4*(l/32) + (r%4),
// so every lane owns runs of four consecutive output columns.
//
//   EPI_GEMM     C = alpha*acc + beta*C_old, C_old read only when beta != 0, one
//                round-to-nearest-even conversion ("GEMM o Coração Matemático" §1).
//   EPI_SWIGLU   y = SiLU(s*gate) * (s*up) for each fused column pair (2n, 2n+1)
//                ("Resumo Técnico: Sobreposição de Ativação em Nível de Tile ...",
//                Metodologia / Kernel-2).  epilogue16 serves the register-staged
//                kernel, whose B tile was de-interleaved per 64 fused columns so a
//                pair sits at the same register of tiles 2q, 2q+1.  The direct-to-
//                LDS kernels keep W_fused's interleaved order (a pair sits in
//                registers (r, r+1) of one lane) and use epilogue_swiglu_lds.
//   EPI_PARTIAL  raw fp32 sums of one K split into workspace [split][M][N].
#pragma once

#include <type_traits>

#include "sg_device.hpp"

namespace sg {

// two round-to-nearest-even conversions packed into one word (a in the low half):
// one v_cvt_pk_f16_f32 / v_cvt_pk_bf16_f32
template <int DT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    if constexpr (DT == DT_F16) {
        typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, h2_t));
    } else {
        typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, b2_t));
    }
}

// EPI_GEMM_EX: y = act(alpha*acc + beta*C_old + bias[n]), stored in DT or, for an
// e4m3 output, as the e4m3fn code of y * inv_scale.  This form serves the register-
// staged kernel, and the direct-to-LDS kernel when C is not 16-byte aligned or ldc
// is not a multiple of 8 (else epilogue_gemm_ex_rows_lds).  Each wave stages one 32 x 32
// fp32 fragment at a time in a region of the (by now idle) LDS ring of its own, and
// a rolled loop then finishes four consecutive columns per lane (row-contiguous
// stores).  The accumulator is only ever indexed by constants: with the
// activation code inlined into every register quad instead, the epilogue exceeds
// the unroll limit, the loop stays rolled, and the whole accumulator array --
// main loop included -- is moved to scratch memory.
// f(std::integral_constant<int, I>) for I = B .. E-1, expanded at compile time (the
// index is a constant inside f whether or not the unroller would unroll a loop).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

template <int DT, int FM, int FN>
__device__ __forceinline__ void epilogue_gemm_ex_lds(const Gemm16Params& p, f32x16 (&acc)[FN][FM],
                                                     char* smem, int mb, int nb, int wave,
                                                     int lane) {
    constexpr int LD = 36;                                 // floats per staged row (+4 pad)
    float* frag = reinterpret_cast<float*>(smem) + wave * (32 * LD);
    const EpiEx& ex = p.ex;
    const float alpha = p.alpha, beta = ex.out_fp8 ? 0.0f : p.beta;
    const int lm = lane & 31, lq = (lane >> 5) * 4;
    // a lane finishes columns c4..c4+3 of every fragment (quads q = lane + 64j share
    // q & 7): its bias values are loaded once, before the fragments
    const int c4 = (lane & 7) * 4;
    f32x4 bq[FN];
#pragma unroll
    for (int tn = 0; tn < FN; ++tn)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int n = nb + tn * 32 + c4 + e;
            bq[tn][e] = n < p.N ? ex_bias(ex, n) : 0.0f;
        }
    static_for<0, FM * FN>([&](auto fi) __attribute__((always_inline)) {
        constexpr int tm = decltype(fi)::value / FN, tn = decltype(fi)::value % FN;
        {
            // D^T layout: register quad g of lane l holds row l%32, columns 8g + 4(l/32) + 0..3
            static_for<0, 4>([&](auto gi) __attribute__((always_inline)) {
                constexpr int g = decltype(gi)::value;
                *reinterpret_cast<f32x4*>(frag + lm * LD + 8 * g + lq) =
                    f32x4{acc[tn][tm][4 * g], acc[tn][tm][4 * g + 1], acc[tn][tm][4 * g + 2],
                          acc[tn][tm][4 * g + 3]};
            });
            __builtin_amdgcn_wave_barrier();
            const int n = nb + tn * 32 + c4;
            const int valid = p.N - n < 4 ? p.N - n : 4;
#pragma unroll 2
            for (int j = 0; j < 4; ++j) {   // two independent quads per pass overlap
                const int r = (lane >> 3) + 8 * j;         // quad q = lane + 64j: row q/8
                const int m = mb + tm * 32 + r;
                if (m >= p.M || valid <= 0) continue;
                const int64_t idx = (int64_t)m * p.ldc + n;
                f32x4 v = *reinterpret_cast<const f32x4*>(frag + r * LD + c4);
                const bool vec = p.vec_c && valid == 4;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] *= alpha;
                if (beta != 0.0f) {
                    const uint16_t* c = reinterpret_cast<const uint16_t*>(p.C) + idx;
                    if (vec) {
                        const u32x2 old = *reinterpret_cast<const u32x2*>(c);
                        v[0] = __builtin_fmaf(beta, to_f32<DT>((uint16_t)(old.x & 0xffff)), v[0]);
                        v[1] = __builtin_fmaf(beta, to_f32<DT>((uint16_t)(old.x >> 16)), v[1]);
                        v[2] = __builtin_fmaf(beta, to_f32<DT>((uint16_t)(old.y & 0xffff)), v[2]);
                        v[3] = __builtin_fmaf(beta, to_f32<DT>((uint16_t)(old.y >> 16)), v[3]);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (e < valid) v[e] = __builtin_fmaf(beta, to_f32<DT>(c[e]), v[e]);
                    }
                }
                f32x4 y;
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] = ex_act(ex.act, v[e] + bq[tn][e]);
                if (ex.out_fp8) {
                    uint8_t* c8 = reinterpret_cast<uint8_t*>(p.C) + idx;
                    const float ys[4] = {y[0] * ex.inv_scale, y[1] * ex.inv_scale,
                                         y[2] * ex.inv_scale, y[3] * ex.inv_scale};
                    const uint32_t w = e4m3_code4(ys);
                    if (vec) {
                        *reinterpret_cast<uint32_t*>(c8) = w;
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (e < valid) c8[e] = (uint8_t)(w >> (8 * e));
                    }
                } else {
                    uint16_t* c = reinterpret_cast<uint16_t*>(p.C) + idx;
                    if (vec) {
                        u32x2 o;
                        o.x = pack2<DT>(y[0], y[1]);
                        o.y = pack2<DT>(y[2], y[3]);
                        *reinterpret_cast<u32x2*>(c) = o;
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (e < valid) c[e] = from_f32<DT>(y[e]);
                    }
                }
            }
            __builtin_amdgcn_wave_barrier();
        }
    });
}

template <int DT, int EPI, int FM, int FN>
__device__ __forceinline__ void epilogue16(const Gemm16Params& p, f32x16 (&acc)[FN][FM], int m0,
                                           int n0, int BM, int BN, int mb, int nb, int lane) {
    const int lm = lane & 31, lq = (lane >> 5) * 4;
    const bool inside = (m0 + BM <= p.M) && (n0 + BN <= p.N);

    static_assert(EPI != EPI_GEMM_EX, "EPI_GEMM_EX uses epilogue_gemm_ex_lds");
    if constexpr (EPI == EPI_GEMM) {
        uint16_t* C = reinterpret_cast<uint16_t*>(p.C);
        const bool full_c = inside && p.vec_c;
        const float alpha = p.alpha, beta = p.beta;
#pragma unroll
        for (int tm = 0; tm < FM; ++tm) {
            const int m = mb + tm * 32 + lm;
            if (!full_c && m >= p.M) continue;
#pragma unroll
            for (int tn = 0; tn < FN; ++tn) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int n = nb + tn * 32 + 8 * g + lq;
                    uint16_t* c = C + (int64_t)m * p.ldc + n;
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = alpha * acc[tn][tm][4 * g + e];
                    if (full_c) {
                        if (beta != 0.0f) {
                            const u32x2 old = *reinterpret_cast<const u32x2*>(c);
                            v[0] = __builtin_fmaf(beta, to_f32<DT>((uint16_t)(old.x & 0xffff)), v[0]);
                            v[1] = __builtin_fmaf(beta, to_f32<DT>((uint16_t)(old.x >> 16)), v[1]);
                            v[2] = __builtin_fmaf(beta, to_f32<DT>((uint16_t)(old.y & 0xffff)), v[2]);
                            v[3] = __builtin_fmaf(beta, to_f32<DT>((uint16_t)(old.y >> 16)), v[3]);
                        }
                        u32x2 o;
                        o.x = pack2<DT>(v[0], v[1]);
                        o.y = pack2<DT>(v[2], v[3]);
                        *reinterpret_cast<u32x2*>(c) = o;
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            if (n + e < p.N) {
                                float x = v[e];
                                if (beta != 0.0f) x = __builtin_fmaf(beta, to_f32<DT>(c[e]), x);
                                c[e] = from_f32<DT>(x);
                            }
                        }
                    }
                }
            }
        }
    } else if constexpr (EPI == EPI_SWIGLU) {
        uint16_t* Y = reinterpret_cast<uint16_t*>(p.C);
        const int nout = p.N >> 1;                 // p.N is the fused width
        const bool full_c = inside && p.vec_c;
        const float s = p.alpha;
        {
            const int ob = nb >> 1;                // first output column of this wave
#pragma unroll
            for (int tm = 0; tm < FM; ++tm) {
                const int m = mb + tm * 32 + lm;
                if (!full_c && m >= p.M) continue;
#pragma unroll
                for (int q = 0; q < FN / 2; ++q) {
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int n = ob + q * 32 + 8 * g + lq;
                        uint16_t* y = Y + (int64_t)m * p.ldc + n;
                        float v[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float gate = s * acc[2 * q][tm][4 * g + e];
                            const float up = s * acc[2 * q + 1][tm][4 * g + e];
                            v[e] = silu(gate) * up;
                        }
                        if (full_c) {
                            u32x2 o;
                            o.x = pack2<DT>(v[0], v[1]);
                            o.y = pack2<DT>(v[2], v[3]);
                            *reinterpret_cast<u32x2*>(y) = o;
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                if (n + e < nout) y[e] = from_f32<DT>(v[e]);
                        }
                    }
                }
            }
        }
    } else {  // EPI_PARTIAL
        float* W = reinterpret_cast<float*>(p.C) + (int64_t)blockIdx.y * p.M * p.N;
        const bool full_c = inside && ((p.N & 3) == 0);
#pragma unroll
        for (int tm = 0; tm < FM; ++tm) {
            const int m = mb + tm * 32 + lm;
            if (!full_c && m >= p.M) continue;
#pragma unroll
            for (int tn = 0; tn < FN; ++tn) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int n = nb + tn * 32 + 8 * g + lq;
                    float* w = W + (int64_t)m * p.N + n;
                    if (full_c) {
                        f32x4 o = {acc[tn][tm][4 * g], acc[tn][tm][4 * g + 1],
                                   acc[tn][tm][4 * g + 2], acc[tn][tm][4 * g + 3]};
                        *reinterpret_cast<f32x4*>(w) = o;
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (n + e < p.N) w[e] = acc[tn][tm][4 * g + e];
                    }
                }
            }
        }
    }
}

// Split-K partial sums of a full tile (N a multiple of 4): one 32-row block of every
// wave at a time is staged in LDS as fp32 rows (16 bytes of padding per row), then every
// thread stores whole 16-byte row pieces into this split's [M][N] slab (plain stores:
// the reduction reads them back at once).  rb / cb: first tile row / column of the wave.
template <int FM, int FN, int BM, int BN, int NT>
__device__ __forceinline__ void epilogue_partial_rows_lds(const Gemm16Params& p,
                                                          f32x16 (&acc)[FN][FM], char* smem,
                                                          int m0, int n0, int rb, int cb,
                                                          int lane) {
    constexpr int ROW = 4 * BN + 16;               // bytes per staged row
    constexpr int CPR = BN / 4;                    // 16-byte pieces (4 sums) per row
    constexpr int WMS = BM / (32 * FM);            // wave rows of the tile
    constexpr int PB = WMS * 32 * CPR;             // pieces per 32-row block
    const int lm = lane & 31, lq = (lane >> 5) * 4;
    const int wr = rb / (32 * FM);
    float* W = reinterpret_cast<float*>(p.C) + (int64_t)blockIdx.y * p.M * p.N;
#pragma unroll
    for (int tm = 0; tm < FM; ++tm) {
        __syncthreads();
        char* row = smem + (wr * 32 + lm) * ROW;
#pragma unroll
        for (int tn = 0; tn < FN; ++tn)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                *reinterpret_cast<f32x4*>(row + 4 * (cb + tn * 32 + 8 * g + lq)) =
                    f32x4{acc[tn][tm][4 * g], acc[tn][tm][4 * g + 1], acc[tn][tm][4 * g + 2],
                          acc[tn][tm][4 * g + 3]};
        __syncthreads();
        for (int i = threadIdx.x; i < PB; i += NT) {
            const int rr = i / CPR, c = i - rr * CPR;
            const int r = (rr >> 5) * (32 * FM) + tm * 32 + (rr & 31);
            *reinterpret_cast<f32x4*>(W + (int64_t)(m0 + r) * p.N + n0 + c * 4) =
                *reinterpret_cast<const f32x4*>(smem + rr * ROW + c * 16);
        }
    }
}

// GEMM epilogue (beta = 0, full tile, C 16-byte aligned with ldc a multiple of 8) of the
// direct-to-LDS kernels: one 32-row block of every wave at a time is rounded to the
// output type and staged in LDS as rows of the tile (16 bytes of padding per row), then
// every thread stores whole 16-byte row pieces, consecutive threads covering whole
// lines, as non-temporal stores.  The block buffer is reused: the barrier before each
// block's staging follows the previous block's LDS reads (its global stores may still
// be in flight).  rb: first tile row of the calling wave; cb: its first tile column.
template <int DT, int FM, int FN, int BM, int BN, int NT>
__device__ __forceinline__ void epilogue_gemm_rows_lds(const Gemm16Params& p,
                                                       f32x16 (&acc)[FN][FM], char* smem,
                                                       int m0, int n0, int rb, int cb,
                                                       int lane) {
    constexpr int ROW = 2 * BN + 16;               // bytes per staged row
    constexpr int CPR = BN / 8;                    // 16-byte pieces (8 outputs) per row
    constexpr int WMS = BM / (32 * FM);            // wave rows of the tile
    constexpr int PB = WMS * 32 * CPR;             // pieces per 32-row block
    const int lm = lane & 31, lq = (lane >> 5) * 4;
    const int wr = rb / (32 * FM);                 // the calling wave's row of waves
    const float alpha = p.alpha;
    uint16_t* C = reinterpret_cast<uint16_t*>(p.C);
#pragma unroll
    for (int tm = 0; tm < FM; ++tm) {
        __syncthreads();
        char* row = smem + (wr * 32 + lm) * ROW;
#pragma unroll
        for (int tn = 0; tn < FN; ++tn)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int c = cb + tn * 32 + 8 * g + lq;
                *reinterpret_cast<u32x2*>(row + 2 * c) =
                    u32x2{pack2<DT>(alpha * acc[tn][tm][4 * g], alpha * acc[tn][tm][4 * g + 1]),
                          pack2<DT>(alpha * acc[tn][tm][4 * g + 2],
                                    alpha * acc[tn][tm][4 * g + 3])};
            }
        __syncthreads();
        for (int i = threadIdx.x; i < PB; i += NT) {
            const int rr = i / CPR, c = i - rr * CPR;
            const int r = (rr >> 5) * (32 * FM) + tm * 32 + (rr & 31);
            const u32x4 v = *reinterpret_cast<const u32x4*>(smem + rr * ROW + c * 16);
            __builtin_nontemporal_store(
                v, reinterpret_cast<u32x4*>(C + (int64_t)(m0 + r) * p.ldc + n0 + c * 8));
        }
    }
}

// Wave columns of a tile staged per pass by the fp32 row epilogues below: all WN if
// the fp32 rows of one 32-row block of every wave row fit in LDSB bytes (EXTRA more
// bytes beside them), else the largest power-of-two divisor of WN that fits; 0 if
// not even one wave column fits.
template <int BM, int BN, int FM, int WN, int LDSB, int EXTRA>
constexpr int staged_wave_cols() {
    const int wms = BM / (32 * FM);
    for (int cw = WN; cw >= 1; cw /= 2)
        if (WN % cw == 0 && wms * 32 * (4 * (BN / WN) * cw + 16) + EXTRA <= LDSB) return cw;
    return 0;
}

// The GEMM epilogue with beta != 0 (and with beta = 0 on edge tiles), staged so that
// C_old is read (never at beta = 0) and C written as whole 16-byte row pieces.  For
// one 32-row block (tm) of every wave row and CW wave columns (pass h; CW from
// staged_wave_cols) at a time, the waves of those columns write alpha * acc in fp32
// into LDS rows; all threads then read 8 values of C_old, form alpha * acc + beta *
// C_old in fp32 (one fma) and store the 8 values rounded once.  Pieces past M are
// skipped and the piece that N cuts goes element by element, so edge tiles take this
// path too (C must be 16-byte aligned with ldc a multiple of 8).  Same arithmetic as
// the register epilogue, so the outputs are bit-identical.  Called by every thread
// after the main loop.
template <int DT, int FM, int FN, int BM, int BN, int WN, int NT, int LDSB>
__device__ __forceinline__ void epilogue_gemm_rows_beta_lds(const Gemm16Params& p,
                                                            f32x16 (&acc)[FN][FM], char* smem,
                                                            int m0, int n0, int rb, int wn,
                                                            int lane) {
    constexpr int TN = BN / WN;                    // columns of one wave column
    constexpr int CW = staged_wave_cols<BM, BN, FM, WN, LDSB, 0>();
    static_assert(CW > 0, "one wave column of fp32 rows fits the LDS ring");
    constexpr int TS = CW * TN;                    // columns staged per pass
    constexpr int ROW = 4 * TS + 16;               // bytes per staged row (fp32)
    constexpr int CPR = TS / 8;                    // 16-byte pieces (8 outputs) of C per row
    constexpr int WMS = BM / (32 * FM);            // wave rows of the tile
    constexpr int PB = WMS * 32 * CPR;             // pieces per pass
    static_assert(FN * 32 == TN, "one wave column holds FN fragments");
    const int lm = lane & 31, lq = (lane >> 5) * 4;
    const int wr = rb / (32 * FM);                 // the calling wave's row of waves
    const float alpha = p.alpha, beta = p.beta;
    uint16_t* C = reinterpret_cast<uint16_t*>(p.C);
#pragma unroll
    for (int tm = 0; tm < FM; ++tm) {
#pragma unroll
        for (int h = 0; h < WN / CW; ++h) {
            __syncthreads();
            if (wn / CW == h) {
                char* row = smem + (wr * 32 + lm) * ROW + 4 * (wn % CW) * TN;
#pragma unroll
                for (int tn = 0; tn < FN; ++tn)
#pragma unroll
                    for (int g = 0; g < 4; ++g)
                        *reinterpret_cast<f32x4*>(row + 4 * (tn * 32 + 8 * g + lq)) =
                            f32x4{alpha * acc[tn][tm][4 * g], alpha * acc[tn][tm][4 * g + 1],
                                  alpha * acc[tn][tm][4 * g + 2], alpha * acc[tn][tm][4 * g + 3]};
            }
            __syncthreads();
            for (int i = threadIdx.x; i < PB; i += NT) {
                const int rr = i / CPR, c = i - rr * CPR;
                const int m = m0 + (rr >> 5) * (32 * FM) + tm * 32 + (rr & 31);
                const int n = n0 + h * TS + c * 8;
                if (m >= p.M || n >= p.N) continue;
                const char* src = smem + rr * ROW + c * 32;
                const f32x4 lo = *reinterpret_cast<const f32x4*>(src);
                const f32x4 hi = *reinterpret_cast<const f32x4*>(src + 16);
                const float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
                uint16_t* cp = C + (int64_t)m * p.ldc + n;
                if (n + 8 <= p.N) {
                    uint32_t o[4];
                    if (beta != 0.0f) {
                        const u32x4 old = *reinterpret_cast<const u32x4*>(cp);
                        const uint32_t ow[4] = {old.x, old.y, old.z, old.w};
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            o[j] = pack2<DT>(
                                __builtin_fmaf(beta, to_f32<DT>((uint16_t)(ow[j] & 0xffff)), v[2 * j]),
                                __builtin_fmaf(beta, to_f32<DT>((uint16_t)(ow[j] >> 16)), v[2 * j + 1]));
                    } else {
#pragma unroll
                        for (int j = 0; j < 4; ++j) o[j] = pack2<DT>(v[2 * j], v[2 * j + 1]);
                    }
                    *reinterpret_cast<u32x4*>(cp) = u32x4{o[0], o[1], o[2], o[3]};
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (n + e < p.N)
                            cp[e] = from_f32<DT>(
                                beta != 0.0f ? __builtin_fmaf(beta, to_f32<DT>(cp[e]), v[e]) : v[e]);
                }
            }
        }
    }
}

// EPI_GEMM_EX staged the same way: alpha * acc in fp32, CW wave columns and one
// 32-row block at a time; every thread then finishes 8 consecutive outputs of a row (beta *
// C_old with one fma, bias, activation, one rounding or the e4m3 code of y *
// inv_scale) and stores them as one 16-byte piece (8 bytes of e4m3 codes),
// non-temporally (whole lines).  Rows past M are skipped and the piece that N cuts
// goes element by element, so edge tiles take this path too (C 16-byte aligned,
// ldc a multiple of 8).  The steps never index the accumulator, so the activation
// code is emitted once, in the rolled piece loop.
template <int DT, int FM, int FN, int BM, int BN, int WN, int NT, int LDSB>
__device__ __forceinline__ void epilogue_gemm_ex_rows_lds(const Gemm16Params& p,
                                                          f32x16 (&acc)[FN][FM], char* smem,
                                                          int m0, int n0, int rb, int wn,
                                                          int lane) {
    constexpr int TN = BN / WN;                    // columns of one wave column
    constexpr int CW = staged_wave_cols<BM, BN, FM, WN, LDSB, 4 * BN>();
    static_assert(CW > 0, "one wave column of fp32 rows and the bias fit the LDS ring");
    constexpr int TS = CW * TN;                    // columns staged per pass
    constexpr int ROW = 4 * TS + 16;               // bytes per staged row (fp32)
    constexpr int CPR = TS / 8;                    // pieces of 8 outputs per row
    constexpr int WMS = BM / (32 * FM);            // wave rows of the tile
    constexpr int PB = WMS * 32 * CPR;             // pieces per pass
    static_assert(FN * 32 == TN, "one wave column holds FN fragments");
    const int lm = lane & 31, lq = (lane >> 5) * 4;
    const int wr = rb / (32 * FM);
    const EpiEx& ex = p.ex;
    const float alpha = p.alpha, beta = ex.out_fp8 ? 0.0f : p.beta;
    // the tile's bias values, once, behind the staging rows; written only after every
    // wave is past its last fragment reads of the ring (read after the next barrier)
    float* sbias = reinterpret_cast<float*>(smem + WMS * 32 * ROW);
    __syncthreads();
    for (int j = threadIdx.x; j < BN; j += NT) sbias[j] = n0 + j < p.N ? ex_bias(ex, n0 + j) : 0.0f;
#pragma unroll
    for (int tm = 0; tm < FM; ++tm) {
#pragma unroll
        for (int h = 0; h < WN / CW; ++h) {
            __syncthreads();
            if (wn / CW == h) {
                char* row = smem + (wr * 32 + lm) * ROW + 4 * (wn % CW) * TN;
#pragma unroll
                for (int tn = 0; tn < FN; ++tn)
#pragma unroll
                    for (int g = 0; g < 4; ++g)
                        *reinterpret_cast<f32x4*>(row + 4 * (tn * 32 + 8 * g + lq)) =
                            f32x4{alpha * acc[tn][tm][4 * g], alpha * acc[tn][tm][4 * g + 1],
                                  alpha * acc[tn][tm][4 * g + 2], alpha * acc[tn][tm][4 * g + 3]};
            }
            __syncthreads();
#pragma unroll 2
            for (int i = threadIdx.x; i < PB; i += NT) {
                const int rr = i / CPR, c = i - rr * CPR;
                const int m = m0 + (rr >> 5) * (32 * FM) + tm * 32 + (rr & 31);
                const int n = n0 + h * TS + c * 8;
                if (m >= p.M || n >= p.N) continue;
                const int nv = p.N - n < 8 ? p.N - n : 8;
                const char* src = smem + rr * ROW + c * 32;
                const f32x4 lo = *reinterpret_cast<const f32x4*>(src);
                const f32x4 hi = *reinterpret_cast<const f32x4*>(src + 16);
                float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
                const int64_t idx = (int64_t)m * p.ldc + n;
                if (beta != 0.0f) {
                    const uint16_t* cp = reinterpret_cast<const uint16_t*>(p.C) + idx;
                    if (nv == 8) {
                        const u32x4 old = *reinterpret_cast<const u32x4*>(cp);
                        const uint32_t ow[4] = {old.x, old.y, old.z, old.w};
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            v[2 * j] = __builtin_fmaf(beta, to_f32<DT>((uint16_t)(ow[j] & 0xffff)),
                                                      v[2 * j]);
                            v[2 * j + 1] =
                                __builtin_fmaf(beta, to_f32<DT>((uint16_t)(ow[j] >> 16)), v[2 * j + 1]);
                        }
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            if (e < nv) v[e] = __builtin_fmaf(beta, to_f32<DT>(cp[e]), v[e]);
                    }
                }
                const f32x4 b0 = *reinterpret_cast<const f32x4*>(sbias + h * TS + c * 8);
                const f32x4 b1 = *reinterpret_cast<const f32x4*>(sbias + h * TS + c * 8 + 4);
                const float b[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
                float y[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) y[e] = ex_act(ex.act, v[e] + b[e]);
                if (ex.out_fp8) {
                    const float q0[4] = {y[0] * ex.inv_scale, y[1] * ex.inv_scale,
                                         y[2] * ex.inv_scale, y[3] * ex.inv_scale};
                    const float q1[4] = {y[4] * ex.inv_scale, y[5] * ex.inv_scale,
                                         y[6] * ex.inv_scale, y[7] * ex.inv_scale};
                    const uint32_t w0 = e4m3_code4(q0), w1 = e4m3_code4(q1);
                    uint8_t* c8 = reinterpret_cast<uint8_t*>(p.C) + idx;
                    if (nv == 8) {
                        __builtin_nontemporal_store(u32x2{w0, w1}, reinterpret_cast<u32x2*>(c8));
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            if (e < nv) c8[e] = (uint8_t)((e < 4 ? w0 : w1) >> (8 * (e & 3)));
                    }
                } else {
                    uint16_t* cp = reinterpret_cast<uint16_t*>(p.C) + idx;
                    if (nv == 8) {
                        __builtin_nontemporal_store(
                            u32x4{pack2<DT>(y[0], y[1]), pack2<DT>(y[2], y[3]),
                                  pack2<DT>(y[4], y[5]), pack2<DT>(y[6], y[7])},
                            reinterpret_cast<u32x4*>(cp));
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            if (e < nv) cp[e] = from_f32<DT>(y[e]);
                    }
                }
            }
        }
    }
}

// SwiGLU epilogue of the direct-to-LDS kernels, staged through LDS so that the
// global stores run along rows.  In the MFMA accumulator layout a wave holds 32
// rows x a few columns, so storing from registers touches 32 rows (cache lines)
// per instruction; here each wave first writes its packed output pairs into a
// row-major [BM][BN/2] tile in LDS (rows padded by 8 bytes: 32 rows at one column
// fall on distinct banks), then all threads copy whole 16-byte row pieces out.
// This runs one 32-row block of every wave at a time (block tm: rows wm*TM + tm*32
// + 0..31 of each wave row wm), so the stores of a block drain while the next
// block's SiLU is computed; each block has its own rows of the staged tile, and
// the barrier between blocks orders LDS only.  The 16-byte row pieces are non-temporal stores:
// whole lines that need no write-combining in L2 (measured: bf16 SwiGLU M = 2048 / 8192
// 36.5 -> 35.4 us / 140.3 -> 134.7 us; the same hint on the accumulator-layout stores
// of the GEMM epilogue, 8-byte pieces of 32 rows, made those kernels far slower).
// Called by every thread of the work-group after the main loop (LDS is free once
// every wave passed the barrier at the top).  W12: the tile's B columns were BN/2
// of W1 then BN/2 of W2, so gate and up of one output sit at the same register of
// fragments tn and tn + FN/2, and cb is the wave's first output column in the tile;
// otherwise cb is its first fused column (outputs at half of it).  SCALED: the
// inputs were e4m3 and gate and up are multiplied by s = sA*sW first; 16-bit
// inputs always have s = 1 (the C ABI rejects other scales for them).
// PRE: the gate accumulator already holds SiLU(s*g) (applied during the main loop).
template <bool SCALED, bool PRE = false>
__device__ __forceinline__ float swiglu_pair(float g, float u, float s) {
    if constexpr (PRE) return SCALED ? g * (s * u) : g * u;
    return SCALED ? silu(s * g) * (s * u) : silu(g) * u;
}

// has_acc == false: a wave without accumulators (a producer wave of the wave-
// specialised kernel) takes part in the barriers and the stores but stages nothing.
template <int DT, int FM, int FN, int BM, int BN, int NT, bool W12, bool SCALED, bool PRE = false>
__device__ __forceinline__ void epilogue_swiglu_lds(const Gemm16Params& p,
                                                    f32x16 (&acc)[FN][FM], char* smem, int m0,
                                                    int n0, int rb, int cb, int lane,
                                                    bool has_acc = true) {
    constexpr int ROW = BN + 8;        // bytes per staged row: BN/2 outputs of 2 bytes + pad
    constexpr int CPR = BN / 16;       // 16-byte pieces (8 outputs) per row
    constexpr int WMS = BM / (32 * FM);            // wave rows of the tile
    constexpr int PB = WMS * 32 * CPR;             // pieces per 32-row block
    static_assert(BN % 16 == 0, "whole 16-byte row pieces");
    const int lm = lane & 31, lq = (lane >> 5) * 4;
    const float s = p.alpha;
    uint16_t* Y = reinterpret_cast<uint16_t*>(p.C);
    const int nout = p.N >> 1, o0 = n0 >> 1;
    const bool v16 = (p.epi_flags & EPI_Y16) != 0;
    __syncthreads();
#pragma unroll
    for (int tm = 0; tm < FM; ++tm) {
        char* row = smem + (rb + tm * 32 + lm) * ROW;
        if (!has_acc) {
        } else if constexpr (W12) {
#pragma unroll
            for (int tn = 0; tn < FN / 2; ++tn) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    // outputs c..c+3 (gate in fragment tn, up in tn + FN/2), bytes 2c..
                    const int c = cb + tn * 32 + 8 * g + lq;
                    float y[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        y[e] = swiglu_pair<SCALED, PRE>(acc[tn][tm][4 * g + e],
                                                        acc[tn + FN / 2][tm][4 * g + e], s);
                    *reinterpret_cast<u32x2*>(row + 2 * c) =
                        u32x2{pack2<DT>(y[0], y[1]), pack2<DT>(y[2], y[3])};
                }
            }
        } else {
#pragma unroll
            for (int tn = 0; tn < FN; ++tn) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    // fused columns c..c+3 hold two (gate, up) pairs -> outputs c/2,
                    // c/2+1, at byte offset c of the staged row
                    const int c = cb + tn * 32 + 8 * g + lq;
                    const float y0 = swiglu_pair<SCALED>(acc[tn][tm][4 * g], acc[tn][tm][4 * g + 1], s);
                    const float y1 =
                        swiglu_pair<SCALED>(acc[tn][tm][4 * g + 2], acc[tn][tm][4 * g + 3], s);
                    *reinterpret_cast<uint32_t*>(row + c) = pack2<DT>(y0, y1);
                }
            }
        }
        __syncthreads();
        // piece i of block tm: wave row i / (32 CPR), row (i / CPR) % 32 of its block
        for (int i = threadIdx.x; i < PB; i += NT) {
            const int rr = i / CPR, c = i - rr * CPR;
            const int r = (rr >> 5) * (32 * FM) + tm * 32 + (rr & 31);
            const int m = m0 + r, o = o0 + c * 8;
            if (m >= p.M || o >= nout) continue;
            const char* src = smem + r * ROW + c * 16;
            const u32x2 lo = *reinterpret_cast<const u32x2*>(src);
            const u32x2 hi = *reinterpret_cast<const u32x2*>(src + 8);
            uint16_t* y = Y + (int64_t)m * p.ldc + o;
            if (v16 && o + 8 <= nout) {
                // whole lines from consecutive threads: streamed past the cache
                __builtin_nontemporal_store(u32x4{lo.x, lo.y, hi.x, hi.y},
                                            reinterpret_cast<u32x4*>(y));
            } else {
                const uint32_t w[4] = {lo.x, lo.y, hi.x, hi.y};
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (o + e < nout) y[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
            }
        }
    }
}

}  // namespace sg
