// sg_device.hpp -- device-side types and helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sg {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2, DT_E4M3 = 3 };
// EPI_GEMM_EX: EPI_GEMM plus the EpiEx steps (compiled for the configurations the
// library chooses, see SG_CONFIGS_EX / SG_CONFIGS_E4M3_EX).  EPI_SWIGLU_SEQ: the
// split-weight SwiGLU with Gate and Up computed one after the other (SG_CONFIGS_SEQ).
enum : int {
    EPI_GEMM = 0,
    EPI_SWIGLU = 1,
    EPI_PARTIAL = 2,
    EPI_SWIGLU_W12 = 3,
    EPI_GEMM_EX = 4,
    EPI_SWIGLU_SEQ = 5
};

// ---------------------------------------------------------------------------
// 16-bit storage <-> fp32
// ---------------------------------------------------------------------------
template <int DT> __device__ __forceinline__ float to_f32(uint16_t b);
template <> __device__ __forceinline__ float to_f32<DT_F16>(uint16_t b) {
    return (float)__builtin_bit_cast(_Float16, b);
}
template <> __device__ __forceinline__ float to_f32<DT_BF16>(uint16_t b) {
    return __builtin_bit_cast(float, (uint32_t)b << 16);
}
// round-to-nearest-even conversions (v_cvt_f16_f32 / v_cvt_pk_bf16_f32)
template <int DT> __device__ __forceinline__ uint16_t from_f32(float x);
template <> __device__ __forceinline__ uint16_t from_f32<DT_F16>(float x) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);
}
template <> __device__ __forceinline__ uint16_t from_f32<DT_BF16>(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// SiLU(x) = x / (1 + e^-x), evaluated as x * rcp(1 + 2^(-x*log2 e)) with the
// hardware exp2 and reciprocal (about 1 ulp each in fp32, far below the bf16 /
// fp16 output rounding).  e^-x -> +inf for very negative x gives rcp = 0 and
// -0, never NaN; for x >= ~17, 1 + e^-x rounds to 1 and SiLU(x) = x exactly.
__device__ __forceinline__ float silu(float x) {
    const float e = __builtin_amdgcn_exp2f(x * -1.44269504088896341f);
    return x * __builtin_amdgcn_rcpf(1.0f + e);
}

// ---------------------------------------------------------------------------
// Extra epilogue steps of the GEMM ("GEMM o Coração Matemático" §1 and §13.3:
// bias and activations folded into the GEMM's epilogue; "为什么 GEMM 是 CUDA 的必修课",
// optimisation list: bias, activation, scale, quantise before the store).  With
// v = alpha*acc + beta*C_old:  y = act(v + bias[n]);  the stored value is y in
// the output type, or the e4m3fn code of y * (1/out_scale) (per-tensor scale,
// §12.4; the reciprocal rounded to fp32 once, on the host).
// ---------------------------------------------------------------------------
enum : int { ACT_NONE = 0, ACT_RELU = 1, ACT_GELU = 2, ACT_GELU_TANH = 3, ACT_SILU = 4 };

struct EpiEx {
    const void* bias;  // nullptr, or N values (bias_dt), one per column
    int bias_dt;       // DT_F32, DT_F16 or DT_BF16
    int act;           // ACT_*
    int out_fp8;       // 1: C holds e4m3fn codes of y * inv_scale (beta == 0)
    float inv_scale;   // fp32 reciprocal of the output's per-tensor scale
    int on;            // any step present (0: the plain GEMM epilogue)
};

__device__ __forceinline__ float ex_bias(const EpiEx& ex, int n) {
    if (!ex.bias) return 0.0f;
    if (ex.bias_dt == DT_F32) return reinterpret_cast<const float*>(ex.bias)[n];
    const uint16_t b = reinterpret_cast<const uint16_t*>(ex.bias)[n];
    return ex.bias_dt == DT_F16 ? to_f32<DT_F16>(b) : to_f32<DT_BF16>(b);
}

// GELU(x) = x * Phi(x) = x/2 * erfc(-x / sqrt 2), with erfc(u) for u >= 0 from
// Abramowitz & Stegun 7.1.26 (t = 1/(1 + p u), erfc(u) ~ t*(a1 + t*(a2 + ... a5 t))
// * e^(-u^2), absolute error <= 1.5e-7) and erfc(-u) = 2 - erfc(u): no cancellation
// in the negative tail, one reciprocal and one exp2 instead of a library erfc.
// The tanh form: x/2 * (1 + tanh z) = x * sigma(2z) exactly (sigma the logistic
// function), z = sqrt(2/pi) * (x + 0.044715 x^3), evaluated like SiLU.
__device__ __forceinline__ float ex_act(int act, float x) {
    constexpr float kLog2e = 1.44269504088896341f;
    switch (act) {
        case ACT_RELU: return x > 0.0f ? x : 0.0f;
        case ACT_GELU: {
            const float u = x * -0.70710678118654752f;
            const float a = __builtin_fabsf(u);
            const float t = __builtin_amdgcn_rcpf(1.0f + 0.3275911f * a);
            const float poly =
                t * (0.254829592f +
                     t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f + t * 1.061405429f))));
            const float q = poly * __builtin_amdgcn_exp2f(-a * a * kLog2e);
            return 0.5f * x * (u >= 0.0f ? q : 2.0f - q);
        }
        case ACT_GELU_TANH: {
            const float z = 0.79788456080286536f * (x + 0.044715f * x * x * x);
            return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-2.0f * kLog2e * z));
        }
        case ACT_SILU: return silu(x);
        default: return x;
    }
}

// OCP e4m3fn codes of four values (byte e of the result = code of x[e]): round to
// nearest, ties to even, |x| >= 448 (and inf) to +-448, NaN to 0x7F.  gfx950's
// v_cvt_pk_fp8_f32 rounds to e4m3fn to nearest-even (checked against the exact
// code-table search on every midpoint of the grid); the clamp turns its overflow
// into saturation, and NaN, which the clamp would map to -448, is selected back.
__device__ __forceinline__ uint32_t e4m3_code4(const float (&x)[4]) {
    float c[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) c[e] = __builtin_fminf(__builtin_fmaxf(x[e], -448.0f), 448.0f);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], w, true);
    uint32_t u = (uint32_t)w;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (!(x[e] == x[e])) u = (u & ~(0xFFu << (8 * e))) | (0x7Fu << (8 * e));
    return u;
}
__device__ __forceinline__ uint32_t e4m3_code(float x) {
    const float q[4] = {x, 0.0f, 0.0f, 0.0f};
    return e4m3_code4(q) & 0xFFu;
}

// Store one output element: v = alpha * sum; adds beta * C_old (read only when
// beta != 0; never with an e4m3 output), applies the EpiEx steps, rounds once to
// the output type (DT_OUT: DT_F32, DT_F16 or DT_BF16) or quantises to e4m3.
template <int DT_OUT>
__device__ __forceinline__ void store_elem(void* C, int64_t idx, int n, float v, float beta,
                                           const EpiEx& ex) {
    if (ex.out_fp8) {
        const float y = ex_act(ex.act, v + ex_bias(ex, n));
        reinterpret_cast<uint8_t*>(C)[idx] = (uint8_t)e4m3_code(y * ex.inv_scale);
        return;
    }
    if constexpr (DT_OUT == DT_F32) {
        float* c = reinterpret_cast<float*>(C) + idx;
        if (beta != 0.0f) v += beta * *c;
        *c = ex.on ? ex_act(ex.act, v + ex_bias(ex, n)) : v;
    } else {
        uint16_t* c = reinterpret_cast<uint16_t*>(C) + idx;
        if (beta != 0.0f) v += beta * to_f32<DT_OUT>(*c);
        *c = from_f32<DT_OUT>(ex.on ? ex_act(ex.act, v + ex_bias(ex, n)) : v);
    }
}

// Arguments of the 16-bit / 8-bit MFMA GEMM kernels.
struct Gemm16Params {
    const uint16_t* A;   // storage of A (16-bit elements; e4m3 kernels reinterpret)
    const uint16_t* B;   // EPI_SWIGLU_W12: W1
    const uint16_t* B2;  // EPI_SWIGLU_W12: W2 (same shape and ld as W1)
    void* C;            // EPI_GEMM: C (dtype); EPI_SWIGLU(_W12): Y; EPI_PARTIAL: fp32 workspace
    int64_t lda, ldb, ldc;   // SwiGLU: ldc is the row stride of Y (in outputs)
    int M, N, K;        // N is the fused width 2*N_out for SwiGLU (both forms) / partials
    float alpha, beta;  // SwiGLU: alpha = scale_a * scale_w
    int vec_a, vec_b, vec_c;
    int tiles_m, tiles_n, group_m;
    int k_per_split;    // a multiple of 64; gridDim.y splits
    int epi_flags;      // EPI_SWIGLU: EPI_Y16 (Y rows allow 16-byte stores)
    int warm_grid;      // gemm_dma_kernel with row-major B: gridDim.x when larger than
                        // tiles_m*tiles_n; the extra work-groups warm L2 (warm_l2)
    int batch;          // strided batch: gridDim.z problems (0 or 1: one problem)
    int64_t sA, sB, sC; // byte distance between consecutive problems' A, B, C
    EpiEx ex;           // EPI_GEMM_EX: bias / activation / e4m3 output
};

// The problem of work-group blockIdx.z in a strided batch (the identity for z = 0).
__device__ __forceinline__ Gemm16Params batch_item(const Gemm16Params& q) {
    Gemm16Params p = q;
    const int64_t z = blockIdx.z;
    p.A = reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(q.A) + z * q.sA);
    p.B = reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(q.B) + z * q.sB);
    p.C = reinterpret_cast<char*>(q.C) + z * q.sC;
    return p;
}

enum { EPI_Y16 = 1 };

// ---------------------------------------------------------------------------
// XCD-aware block order.  Work-groups are handed to the 8 XCDs round-robin
// (block b runs on XCD b % 8); remap so that consecutive logical tiles share an
// XCD (and so its L2).  Bijective for any count.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
    constexpr int NXCD = 8;
    if (nblocks < NXCD) return bid;
    const int per = nblocks / NXCD, rem = nblocks % NXCD;
    const int xcd = bid % NXCD, idx = bid / NXCD;
    return xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
}

// First unit of work-group w when `units` are dealt to G work-groups.
__device__ __forceinline__ int sk_start(int w, int units, int G) {
    return (int)((int64_t)w * units / G);
}
// The work-group whose run holds unit u: the largest w with sk_start(w) <= u.
__device__ __forceinline__ int sk_owner(int u, int units, int G) {
    return (int)(((int64_t)(u + 1) * G - 1) / units);
}

// Grouped ("super-tile") order: walk GROUP_M tile-rows at a time so the tiles in
// flight share A rows and B columns.
__device__ __forceinline__ void tile_coords(int lid, int tiles_m, int tiles_n, int group_m,
                                            int& tm, int& tn) {
    const int per_group = group_m * tiles_n;
    const int g = lid / per_group;
    const int first_m = g * group_m;
    const int gm = min(tiles_m - first_m, group_m);
    const int r = lid - g * per_group;
    tm = first_m + r % gm;
    tn = r / gm;
}

// ---------------------------------------------------------------------------
// Scheduling hint: spread NR LDS reads, NV global loads and NW LDS writes evenly
// between NM MFMAs of one scheduling region (hint only; never changes results).
template <int NM, int NR, int NV, int NW, int I = 0>
__device__ __forceinline__ void sched_interleave() {
    if constexpr (I < NM) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);               // MFMA
        constexpr int r = (I + 1) * NR / NM - I * NR / NM;
        constexpr int v = (I + 1) * NV / NM - I * NV / NM;
        constexpr int w = (I + 1) * NW / NM - I * NW / NM;
        if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);   // DS read
        if constexpr (v > 0) __builtin_amdgcn_sched_group_barrier(0x020, v, 0);   // VMEM read
        if constexpr (w > 0) __builtin_amdgcn_sched_group_barrier(0x200, w, 0);   // DS write
        sched_interleave<NM, NR, NV, NW, I + 1>();
    }
}

template <int DT>
__device__ __forceinline__ f32x16 mfma16(const u32x4& a, const u32x4& b, const f32x16& c) {
    if constexpr (DT == DT_F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

}  // namespace sg
