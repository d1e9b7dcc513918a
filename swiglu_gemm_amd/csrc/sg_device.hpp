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
enum : int { EPI_GEMM = 0, EPI_SWIGLU = 1, EPI_PARTIAL = 2, EPI_SWIGLU_W12 = 3 };

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

// Arguments of the 16-bit / 8-bit MFMA GEMM kernels.
struct Gemm16Params {
    const uint16_t* A;   // storage of A (16-bit elements; e4m3 kernels reinterpret)
    const uint16_t* B;   // EPI_SWIGLU_W12: W1
    const uint16_t* B2;  // EPI_SWIGLU_W12: W2 (same shape and ld as W1)
    void* C;            // EPI_GEMM: C (dtype); EPI_SWIGLU(_W12): Y; EPI_PARTIAL: fp32 workspace
    int64_t lda, ldb, ldc;
    int M, N, K;        // N is the fused width 2*N_out for SwiGLU (both forms) / partials
    float alpha, beta;  // SwiGLU: alpha = scale_a * scale_w
    int vec_a, vec_b, vec_c;
    int tiles_m, tiles_n, group_m;
    int k_per_split;    // a multiple of 64; gridDim.y splits
    int epi_flags;      // EPI_SWIGLU: EPI_Y16 (Y rows allow 16-byte stores)
    int batch;          // strided batch: gridDim.z problems (0 or 1: one problem)
    int64_t sA, sB, sC; // byte distance between consecutive problems' A, B, C
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
