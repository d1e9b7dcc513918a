// mfma_loop.hip -- diagnostic: sustained MFMA rate on given operand data.
//
// Not part of the GEMM path.  Each wave loads four A and four B operand
// registers once from `src` (whatever data the caller provides: zeros, one
// repeated value, random values) and then issues `iters` rounds of eight
// independent MFMAs on them, so the only work is the matrix core itself.  The
// rate it reaches with random operands is the ceiling a GEMM kernel can reach
// on the same data when the chip holds its power limit by lowering its clock.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// KIND 0: v_mfma_f32_32x32x16_f16, 1: ..._bf16, 2: v_mfma_scale_f32_32x32x64_f8f6f4
// (e4m3 operands, unit block scales); 3, 4: v_mfma_f32_16x16x32_{f16,bf16} (same
// operand registers, sixteen 4-register accumulators so the work per round matches)
template <int KIND>
__global__ void __launch_bounds__(256) mfma_loop(const u32x4* src, int nsrc, int iters,
                                                 float* out) {
    u32x4 a[4], b[4];
    const int base = (int)(threadIdx.x * 8 + blockIdx.x * 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a[i] = src[(base + i) % nsrc];
        b[i] = src[(base + 4 + i) % nsrc];
    }
    f32x16 c[8] = {};
    if constexpr (KIND >= 3) {
        f32x4 d[16] = {};
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const u32x4 x = a[u & 3], y = b[(u >> 2) & 3];
                if constexpr (KIND == 3)
                    d[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, x),
                                                                  __builtin_bit_cast(f16x8, y),
                                                                  d[u], 0, 0, 0);
                else
                    d[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, x),
                                                                   __builtin_bit_cast(bf16x8, y),
                                                                   d[u], 0, 0, 0);
            }
        }
        float s4 = 0.0f;
#pragma unroll
        for (int u = 0; u < 16; ++u) s4 += d[u][threadIdx.x & 3];
        out[blockIdx.x * 256 + threadIdx.x] = s4;
        return;
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const u32x4 x = a[u & 3], y = b[(u >> 1) & 3];
            if constexpr (KIND == 0) {
                c[u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, x),
                                                              __builtin_bit_cast(f16x8, y), c[u],
                                                              0, 0, 0);
            } else if constexpr (KIND == 1) {
                c[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, x),
                                                               __builtin_bit_cast(bf16x8, y),
                                                               c[u], 0, 0, 0);
            } else {
                const u32x4 x2 = a[(u + 1) & 3], y2 = b[(u + 3) & 3];
                const i32x8 xa = {(int)x.x, (int)x.y, (int)x.z, (int)x.w,
                                  (int)x2.x, (int)x2.y, (int)x2.z, (int)x2.w};
                const i32x8 yb = {(int)y.x, (int)y.y, (int)y.z, (int)y.w,
                                  (int)y2.x, (int)y2.y, (int)y2.z, (int)y2.w};
                c[u] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(xa, yb, c[u], 0, 0, 0,
                                                                       0x7F7F7F7F, 0,
                                                                       0x7F7F7F7F);
            }
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int u = 0; u < 8; ++u) s += c[u][threadIdx.x & 15];
    out[blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

// Launches `blocks` work-groups of 4 waves.  src: nsrc 16-byte operand chunks
// (device); out: blocks*256 floats (device).  Returns a hipError_t.  Work:
// blocks*4*iters*8 MFMAs of 2*32*32*16 (kinds 0, 1) or 2*32*32*64 (kind 2) flops;
// kinds 3, 4: blocks*4*iters*16 MFMAs of 2*16*16*32 flops (the same total).
extern "C" int sg_diag_mfma_loop(int kind, int blocks, const void* src, int nsrc, int iters,
                                 void* out, void* stream) {
    if (kind < 0 || kind > 4 || blocks <= 0 || nsrc <= 0 || iters < 0 || !src || !out)
        return (int)hipErrorInvalidValue;
    hipStream_t st = (hipStream_t)stream;
    const u32x4* s = (const u32x4*)src;
    float* o = (float*)out;
    if (kind == 0) hipLaunchKernelGGL(mfma_loop<0>, dim3(blocks), dim3(256), 0, st, s, nsrc, iters, o);
    if (kind == 1) hipLaunchKernelGGL(mfma_loop<1>, dim3(blocks), dim3(256), 0, st, s, nsrc, iters, o);
    if (kind == 2) hipLaunchKernelGGL(mfma_loop<2>, dim3(blocks), dim3(256), 0, st, s, nsrc, iters, o);
    if (kind == 3) hipLaunchKernelGGL(mfma_loop<3>, dim3(blocks), dim3(256), 0, st, s, nsrc, iters, o);
    if (kind == 4) hipLaunchKernelGGL(mfma_loop<4>, dim3(blocks), dim3(256), 0, st, s, nsrc, iters, o);
    return (int)hipGetLastError();
}
