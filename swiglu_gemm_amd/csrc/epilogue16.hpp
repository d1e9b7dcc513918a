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
//                Metodologia / Kernel-2).  PAIR_ADJ: the B tile kept W_fused's
//                interleaved column order, so a pair sits in registers (r, r+1) of
//                one lane.  Otherwise the B tile was de-interleaved per 64 fused
//                columns and a pair sits at the same register of tiles 2q, 2q+1.
//   EPI_PARTIAL  raw fp32 sums of one K split into workspace [split][M][N].
#pragma once

#include "sg_device.hpp"

namespace sg {

template <int DT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    return (uint32_t)from_f32<DT>(a) | ((uint32_t)from_f32<DT>(b) << 16);
}

template <int DT, int EPI, bool PAIR_ADJ, int FM, int FN>
__device__ __forceinline__ void epilogue16(const Gemm16Params& p, f32x16 (&acc)[FN][FM], int m0,
                                           int n0, int BM, int BN, int mb, int nb, int lane) {
    const int lm = lane & 31, lq = (lane >> 5) * 4;
    const bool inside = (m0 + BM <= p.M) && (n0 + BN <= p.N);

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
                            v[0] += beta * to_f32<DT>((uint16_t)(old.x & 0xffff));
                            v[1] += beta * to_f32<DT>((uint16_t)(old.x >> 16));
                            v[2] += beta * to_f32<DT>((uint16_t)(old.y & 0xffff));
                            v[3] += beta * to_f32<DT>((uint16_t)(old.y >> 16));
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
                                if (beta != 0.0f) x += beta * to_f32<DT>(c[e]);
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
        if constexpr (PAIR_ADJ) {
            // fused columns nf..nf+3 in registers 4g..4g+3: pairs (0,1), (2,3)
#pragma unroll
            for (int tm = 0; tm < FM; ++tm) {
                const int m = mb + tm * 32 + lm;
                if (!full_c && m >= p.M) continue;
#pragma unroll
                for (int tn = 0; tn < FN; ++tn) {
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int no = (nb + tn * 32 + 8 * g + lq) >> 1;
                        uint16_t* y = Y + (int64_t)m * nout + no;
                        const float y0 = silu(s * acc[tn][tm][4 * g]) * (s * acc[tn][tm][4 * g + 1]);
                        const float y1 =
                            silu(s * acc[tn][tm][4 * g + 2]) * (s * acc[tn][tm][4 * g + 3]);
                        if (full_c) {
                            *reinterpret_cast<uint32_t*>(y) = pack2<DT>(y0, y1);
                        } else {
                            if (no < nout) y[0] = from_f32<DT>(y0);
                            if (no + 1 < nout) y[1] = from_f32<DT>(y1);
                        }
                    }
                }
            }
        } else {
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
                        uint16_t* y = Y + (int64_t)m * nout + n;
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

}  // namespace sg
