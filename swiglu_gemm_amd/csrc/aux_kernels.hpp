// aux_kernels.hpp -- fp32 GEMM, the beta-only update, split-K reductions and the
// elementwise kernels (W_fused interleave, unfused SiLU(G)*U).
#pragma once

#include "sg_device.hpp"

namespace sg {

// ---------------------------------------------------------------------------
// fp32 GEMM: C = alpha*op(A)*op(B) + beta*C_old ("GEMM o Coração Matemático" §1)
// with v_mfma_f32_32x32x2_f32 (fp32 products, fp32 accumulation).
//
// A (2*WT) x (2*WT) tile per work-group of four waves (2 x 2), each wave a WT x WT
// block of 32x32 accumulators; K in tiles of 16.  Both operand tiles sit in LDS
// as [row][k] (k contiguous, rows padded to 20 floats: the eight 16-byte reads of
// one LDS cycle land on distinct banks), so a lane's operands for four MFMAs are
// one 16-byte read: in a group of 8 k, lane half h supplies k = 4h + s to MFMA
// step s of A and B alike, which sums every k once.  An operand stored k-
// contiguous is copied as 16-byte pieces of a row; one stored row-contiguous is
// read as 16-byte pieces along the row and written to LDS one float per row.
// Two LDS stages: the next K tile is loaded into registers while the current one
// feeds the MFMAs, one barrier per K tile.  Out-of-range elements load as zero
// and never dereference; vector loads only where the operand's base and ld allow
// them and the whole piece is in range.
// ---------------------------------------------------------------------------
struct GemmF32Params {
    const float* A;
    const float* B;
    float* C;
    int64_t lda, ldb, ldc;
    int M, N, K;
    float alpha, beta;
    int tiles_m, tiles_n;
    int group_m;         // tile-rows walked together
    int vec_a, vec_b;    // 16-byte aligned base, ld % 4 == 0 and batch stride % 16 == 0
    int batch;           // strided batch over gridDim.z
    int64_t sA, sB, sC;  // byte distance between consecutive problems
    EpiEx ex;            // bias / activation / e4m3 output (ex.on == 0: none)
};

// Four consecutive floats src[0..3] of which the first `left` exist (zeros past
// them); `vec`: the 16-byte load is allowed when all four exist.
__device__ __forceinline__ f32x4 load4_f32(const float* src, int left, bool vec) {
    f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
    if (left <= 0) return v;
    if (vec && left >= 4) return *reinterpret_cast<const f32x4*>(src);
#pragma unroll
    for (int c = 0; c < 4; ++c)
        if (c < left) v[c] = src[c];
    return v;
}

template <bool TA, bool TB, int WT>
__global__ void __launch_bounds__(256) gemm_f32_kernel(const GemmF32Params p_) {
    GemmF32Params p = p_;
    {
        const int64_t z = blockIdx.z;
        p.A = reinterpret_cast<const float*>(reinterpret_cast<const char*>(p_.A) + z * p_.sA);
        p.B = reinterpret_cast<const float*>(reinterpret_cast<const char*>(p_.B) + z * p_.sB);
        p.C = reinterpret_cast<float*>(reinterpret_cast<char*>(p_.C) + z * p_.sC);
    }
    constexpr int T = 2 * WT, BK = 16, LDR = BK + 4;
    constexpr int NL = T / 64;    // 16-byte pieces per thread and operand per K tile
    constexpr int FM = WT / 32;   // 32x32 accumulators per wave along each dimension
    __shared__ __attribute__((aligned(16))) float As[2][T][LDR];
    __shared__ __attribute__((aligned(16))) float Bs[2][T][LDR];

    const int nblk = p.tiles_m * p.tiles_n;
    const int lid = xcd_remap(blockIdx.x, nblk);
    int tmi, tni;
    tile_coords(lid, p.tiles_m, p.tiles_n, p.group_m, tmi, tni);
    const int m0 = tmi * T, n0 = tni * T;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave & 1, wn = wave >> 1;
    const bool va = p.vec_a != 0, vb = p.vec_b != 0;

    // piece e of a tile: k-contiguous operand: row e/4, k 4*(e%4); row-contiguous
    // operand: k e%16, rows 4*(e/16) .. +3
    auto load = [&](int k0, f32x4 (&ra)[NL], f32x4 (&rb)[NL]) {
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int e = tid + i * 256;
            if (!TA) {
                const int r = e >> 2, k = k0 + ((e & 3) << 2);
                ra[i] = m0 + r < p.M ? load4_f32(p.A + (int64_t)(m0 + r) * p.lda + k, p.K - k, va)
                                     : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            } else {
                const int k = k0 + (e & 15), r = m0 + ((e >> 4) << 2);
                ra[i] = k < p.K ? load4_f32(p.A + (int64_t)k * p.lda + r, p.M - r, va)
                                : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            }
            if (TB) {
                const int r = e >> 2, k = k0 + ((e & 3) << 2);
                rb[i] = n0 + r < p.N ? load4_f32(p.B + (int64_t)(n0 + r) * p.ldb + k, p.K - k, vb)
                                     : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            } else {
                const int k = k0 + (e & 15), r = n0 + ((e >> 4) << 2);
                rb[i] = k < p.K ? load4_f32(p.B + (int64_t)k * p.ldb + r, p.N - r, vb)
                                : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            }
        }
    };
    auto store = [&](int st, const f32x4 (&ra)[NL], const f32x4 (&rb)[NL]) {
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int e = tid + i * 256;
            if (!TA) {
                *reinterpret_cast<f32x4*>(&As[st][e >> 2][(e & 3) << 2]) = ra[i];
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c) As[st][((e >> 4) << 2) + c][e & 15] = ra[i][c];
            }
            if (TB) {
                *reinterpret_cast<f32x4*>(&Bs[st][e >> 2][(e & 3) << 2]) = rb[i];
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c) Bs[st][((e >> 4) << 2) + c][e & 15] = rb[i][c];
            }
        }
    };

    f32x16 acc[FM][FM];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    const int nkt = (p.K + BK - 1) / BK;
    f32x4 ra[NL], rb[NL];
    if (nkt > 0) {
        load(0, ra, rb);
        store(0, ra, rb);
    }
    __syncthreads();
    const int h = lane >> 5, li = lane & 31;
    for (int t = 0; t < nkt; ++t) {
        const int st = t & 1;
        if (t + 1 < nkt) load((t + 1) * BK, ra, rb);
#pragma unroll
        for (int g = 0; g < BK / 8; ++g) {
            f32x4 a[FM], b[FM];
#pragma unroll
            for (int f = 0; f < FM; ++f) {
                a[f] = *reinterpret_cast<const f32x4*>(&As[st][wm * WT + f * 32 + li][8 * g + 4 * h]);
                b[f] = *reinterpret_cast<const f32x4*>(&Bs[st][wn * WT + f * 32 + li][8 * g + 4 * h]);
            }
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FM; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][s], b[j][s],
                                                                          acc[i][j], 0, 0, 0);
        }
        // the other stage was last read before the previous barrier
        if (t + 1 < nkt) store(st ^ 1, ra, rb);
        __syncthreads();
    }
    // D[i][j] of one accumulator: j = lane % 32, i = 8*(r/4) + 4*(lane/32) + r%4
#pragma unroll
    for (int j = 0; j < FM; ++j) {
        const int n = n0 + wn * WT + j * 32 + li;
        if (n >= p.N) continue;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm * WT + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                if (m < p.M)
                    store_elem<DT_F32>(p.C, (int64_t)m * p.ldc + n, n, p.alpha * acc[i][j][r],
                                       p.beta, p.ex);
            }
    }
}

// ---------------------------------------------------------------------------
// C = beta * C_old over M x N (ld ldc); beta == 0 writes zeros without reading.
// The GEMM update when K == 0 or alpha == 0.
// ---------------------------------------------------------------------------
template <int DT>
__global__ void __launch_bounds__(256) scale_kernel(void* C, int64_t ldc, int M, int N, float beta) {
    const int64_t total = (int64_t)M * N;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * 256) {
        const int64_t m = i / N, n = i - m * N;
        if constexpr (DT == DT_F32) {
            float* c = reinterpret_cast<float*>(C) + m * ldc + n;
            *c = beta == 0.0f ? 0.0f : beta * *c;
        } else {
            // bf16 (DT_BF16 and the e4m3 GEMM's bf16 output) or fp16
            constexpr int D = DT == DT_F16 ? DT_F16 : DT_BF16;
            uint16_t* c = reinterpret_cast<uint16_t*>(C) + m * ldc + n;
            *c = from_f32<D>(beta == 0.0f ? 0.0f : beta * to_f32<D>(*c));
        }
    }
}

// The same update with the EpiEx steps: y = act(beta*C_old + bias[n]) (C_old
// read only when beta != 0), stored in DT_OUT or as e4m3 codes.
template <int DT_OUT>
__global__ void __launch_bounds__(256) epilogue_only_kernel(void* C, int64_t ldc, int M, int N,
                                                            float beta, const EpiEx ex) {
    const int64_t total = (int64_t)M * N;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * 256) {
        const int64_t m = i / N, n = i - m * N;
        store_elem<DT_OUT>(C, m * ldc + n, (int)n, 0.0f, beta, ex);
    }
}

// ---------------------------------------------------------------------------
// Split-K reductions: sum the fp32 partials of every split in split order (a
// fixed order, so results are run-to-run identical), then the epilogue.
// ws layout: [splits][M][Nw] fp32, Nw = the GEMM's N (fused width for SwiGLU).
// ---------------------------------------------------------------------------
template <int DT_OUT>
__global__ void __launch_bounds__(256) reduce_gemm_kernel(const float* ws, int splits, int M, int N,
                                                          void* C, int64_t ldc, float alpha,
                                                          float beta, const EpiEx ex) {
    const int64_t total = (int64_t)M * N;
    const int64_t plane = total;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * 256) {
        float s = 0.0f;
        for (int k = 0; k < splits; ++k) s += ws[k * plane + i];
        const int64_t m = i / N, n = i - m * N;
        store_elem<DT_OUT>(C, m * ldc + n, (int)n, alpha * s, beta, ex);
    }
}

// Y[m,n] = SiLU(s*G) * (s*U) with G, U the summed partials of fused columns 2n, 2n+1.
template <int DT_OUT>
__global__ void __launch_bounds__(256) reduce_swiglu_kernel(const float* ws, int splits, int M,
                                                            int Nout, uint16_t* Y, float s) {
    const int64_t total = (int64_t)M * Nout;
    const int64_t plane = (int64_t)M * 2 * Nout;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * 256) {
        const int64_t m = i / Nout, n = i - m * Nout;
        const int64_t base = m * 2 * Nout + 2 * n;
        float g = 0.0f, u = 0.0f;
        for (int k = 0; k < splits; ++k) {
            g += ws[k * plane + base];
            u += ws[k * plane + base + 1];
        }
        Y[i] = from_f32<DT_OUT>(silu(s * g) * (s * u));
    }
}

// ---------------------------------------------------------------------------
// W_fused[k, 2n] = W1[k, n], W_fused[k, 2n+1] = W2[k, n] (bit-exact copy).
// ---------------------------------------------------------------------------
template <typename E>
__global__ void __launch_bounds__(256) interleave_kernel(const E* W1, const E* W2, E* Wf,
                                                         int64_t total) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * 256) {
        Wf[2 * i] = W1[i];
        Wf[2 * i + 1] = W2[i];
    }
}

// Y = SiLU(G) * U elementwise (the separate activation pass of the unfused MLP).
template <int DT>
__global__ void __launch_bounds__(256) silu_mul_kernel(const uint16_t* G, const uint16_t* U,
                                                       uint16_t* Y, int64_t total, int vec) {
    const int64_t nvec = vec ? total / 8 : 0;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nvec;
         i += (int64_t)gridDim.x * 256) {
        const u32x4 g = reinterpret_cast<const u32x4*>(G)[i];
        const u32x4 u = reinterpret_cast<const u32x4*>(U)[i];
        u32x4 y;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float g0 = to_f32<DT>((uint16_t)(g[w] & 0xffff));
            const float g1 = to_f32<DT>((uint16_t)(g[w] >> 16));
            const float u0 = to_f32<DT>((uint16_t)(u[w] & 0xffff));
            const float u1 = to_f32<DT>((uint16_t)(u[w] >> 16));
            y[w] = (uint32_t)from_f32<DT>(silu(g0) * u0) |
                   ((uint32_t)from_f32<DT>(silu(g1) * u1) << 16);
        }
        reinterpret_cast<u32x4*>(Y)[i] = y;
    }
    for (int64_t i = nvec * 8 + (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * 256) {
        Y[i] = from_f32<DT>(silu(to_f32<DT>(G[i])) * to_f32<DT>(U[i]));
    }
}

}  // namespace sg

namespace sg {

// ---------------------------------------------------------------------------
// Re-lays `rows` rows of `cols` bytes (src, row pitch lds, problem z at src + z*sS)
// as rows of ldd bytes (ldd % 16 == 0, dst 16-byte aligned, problem z at dst +
// z*sD), bytes [cols, ldd) of each row zero.  One 16-byte piece of dst per thread
// and step; src is read byte by byte (any alignment).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) pack_rows_kernel(const uint8_t* src, int64_t lds,
                                                        int64_t sS, uint8_t* dst, int64_t ldd,
                                                        int64_t sD, int64_t rows, int64_t cols) {
    src += (int64_t)blockIdx.z * sS;
    dst += (int64_t)blockIdx.z * sD;
    const int64_t per_row = ldd >> 4, total = rows * per_row;
    for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < total;
         q += (int64_t)gridDim.x * 256) {
        const int64_t r = q / per_row, c0 = (q - r * per_row) << 4;
        const uint8_t* s = src + r * lds + c0;
        uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int b = 0; b < 16; ++b)
            if (c0 + b < cols) w[b >> 2] |= (uint32_t)s[b] << (8 * (b & 3));
        *reinterpret_cast<u32x4*>(dst + r * ldd + c0) = u32x4{w[0], w[1], w[2], w[3]};
    }
}

// ---------------------------------------------------------------------------
// Generic e4m3 kernels for problems the direct-to-LDS kernel cannot take even
// with re-laid operands (a tile's rows spanning 2^31 bytes or more, or no room in
// the fixed scratch of sg_gemm_noalloc for the re-laid copies): one thread per
// output, exact e4m3 -> fp32 decode, fp32 accumulation in k order, bf16 output.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float e4m3_to_f32(uint8_t q) {
    const int e = (q >> 3) & 15, f = q & 7;
    float v;
    if (e == 15 && f == 7) v = __builtin_nanf("");
    else if (e == 0) v = ldexpf((float)f, -9);
    else v = ldexpf((float)(8 + f), e - 10);
    return (q & 0x80) ? -v : v;
}

__global__ void __launch_bounds__(256) gemm_e4m3_generic(const uint8_t* A, const uint8_t* B,
                                                         void* C, int64_t lda, int64_t ldb,
                                                         int64_t ldc, int M, int N, int K, int ta,
                                                         int tb, float alpha, float beta,
                                                         const EpiEx ex) {
    const int64_t total = (int64_t)M * N;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * 256) {
        const int m = (int)(i / N), n = (int)(i - (int64_t)m * N);
        float s = 0.0f;
        for (int k = 0; k < K; ++k) {
            const uint8_t a = ta ? A[(int64_t)k * lda + m] : A[(int64_t)m * lda + k];
            const uint8_t b = tb ? B[(int64_t)n * ldb + k] : B[(int64_t)k * ldb + n];
            s += e4m3_to_f32(a) * e4m3_to_f32(b);
        }
        store_elem<DT_BF16>(C, (int64_t)m * ldc + n, n, alpha * s, beta, ex);
    }
}

__global__ void __launch_bounds__(256) swiglu_e4m3_generic(const uint8_t* A, const uint8_t* Wf,
                                                           uint16_t* Y, int M, int N, int K,
                                                           float s) {
    const int64_t total = (int64_t)M * N;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * 256) {
        const int m = (int)(i / N), n = (int)(i - (int64_t)m * N);
        float g = 0.0f, u = 0.0f;
        for (int k = 0; k < K; ++k) {
            const float a = e4m3_to_f32(A[(int64_t)m * K + k]);
            g += a * e4m3_to_f32(Wf[(int64_t)k * 2 * N + 2 * n]);
            u += a * e4m3_to_f32(Wf[(int64_t)k * 2 * N + 2 * n + 1]);
        }
        Y[i] = from_f32<DT_BF16>(silu(s * g) * (s * u));
    }
}

}  // namespace sg
