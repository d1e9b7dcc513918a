// aux_kernels.hpp -- fp32 GEMM, the beta-only update, split-K reductions and the
// elementwise kernels (W_fused interleave, unfused SiLU(G)*U).
#pragma once

#include "sg_device.hpp"

namespace sg {

// ---------------------------------------------------------------------------
// fp32 GEMM: C = alpha*op(A)*op(B) + beta*C_old ("GEMM o Coração Matemático" §1)
// with v_mfma_f32_32x32x2_f32 (fp32 products, fp32 accumulation).  64x64 tile,
// BK = 16, four waves each owning one 32x32 accumulator.  Operands are staged in
// LDS as [k][row] (row contiguous) so each lane's MFMA operand is one float.
// Out-of-range elements are zero-filled; stores are predicated.
// ---------------------------------------------------------------------------
struct GemmF32Params {
    const float* A;
    const float* B;
    float* C;
    int64_t lda, ldb, ldc;
    int M, N, K;
    float alpha, beta;
    int tiles_m, tiles_n;
    int batch;           // strided batch over gridDim.z
    int64_t sA, sB, sC;  // byte distance between consecutive problems
    EpiEx ex;            // bias / activation / e4m3 output (ex.on == 0: none)
};

template <bool TA, bool TB>
__global__ void __launch_bounds__(256) gemm_f32_kernel(const GemmF32Params p_) {
    GemmF32Params p = p_;
    {
        const int64_t z = blockIdx.z;
        p.A = reinterpret_cast<const float*>(reinterpret_cast<const char*>(p_.A) + z * p_.sA);
        p.B = reinterpret_cast<const float*>(reinterpret_cast<const char*>(p_.B) + z * p_.sB);
        p.C = reinterpret_cast<float*>(reinterpret_cast<char*>(p_.C) + z * p_.sC);
    }
    constexpr int T = 64, BK = 16, PAD = 4;
    __shared__ float As[BK][T + PAD];
    __shared__ float Bs[BK][T + PAD];
    const int nblk = p.tiles_m * p.tiles_n;
    const int lid = xcd_remap(blockIdx.x, nblk);
    const int tmi = lid % p.tiles_m, tni = lid / p.tiles_m;
    const int m0 = tmi * T, n0 = tni * T;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave & 1, wn = wave >> 1;
    f32x16 acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.0f;

    for (int k0 = 0; k0 < p.K; k0 += BK) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = tid + i * 256;
            int m, k;
            if (TA) { k = e >> 6; m = e & 63; }   // A stored K x M: m contiguous
            else    { m = e >> 4; k = e & 15; }   // A stored M x K: k contiguous
            float v = 0.0f;
            if (m0 + m < p.M && k0 + k < p.K)
                v = TA ? p.A[(int64_t)(k0 + k) * p.lda + (m0 + m)]
                       : p.A[(int64_t)(m0 + m) * p.lda + (k0 + k)];
            As[k][m] = v;
            int n;
            if (TB) { n = e >> 4; k = e & 15; }   // B stored N x K: k contiguous
            else    { k = e >> 6; n = e & 63; }   // B stored K x N: n contiguous
            float w = 0.0f;
            if (n0 + n < p.N && k0 + k < p.K)
                w = TB ? p.B[(int64_t)(n0 + n) * p.ldb + (k0 + k)]
                       : p.B[(int64_t)(k0 + k) * p.ldb + (n0 + n)];
            Bs[k][n] = w;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < BK; kk += 2) {
            const float a = As[kk + (lane >> 5)][wm * 32 + (lane & 31)];
            const float b = Bs[kk + (lane >> 5)][wn * 32 + (lane & 31)];
            // first operand: rows of A (i = lane%32), second: columns of B
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
        }
        __syncthreads();
    }
    // D[i][j]: j = lane%32, i = 8*(r/4) + 4*(lane/32) + r%4
    const int n = n0 + wn * 32 + (lane & 31);
    if (n >= p.N) return;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (m < p.M) store_elem<DT_F32>(p.C, (int64_t)m * p.ldc + n, n, p.alpha * acc[r], p.beta, p.ex);
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
// Generic e4m3 kernels for shapes the direct-to-LDS kernel does not take (a K
// tail, odd sizes or alignment): one thread per output, exact e4m3 -> fp32
// decode, fp32 accumulation in k order, bf16 output.
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
