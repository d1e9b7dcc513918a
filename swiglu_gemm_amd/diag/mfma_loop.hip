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

// Streams n16 16-byte chunks of src through the vector memory path (four loads in
// flight per thread per step, grid-stride) and folds them with XOR into one word
// per thread, so the only work is reading: the HBM read ceiling of the board.
__global__ void __launch_bounds__(256) stream_read(const u32x4* src, int64_t n16, uint32_t* out) {
    u32x4 acc = {0u, 0u, 0u, 0u};
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 a = __builtin_nontemporal_load(src + i);
        const u32x4 b = __builtin_nontemporal_load(src + i + stride);
        const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
        const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
        acc ^= a ^ b ^ c ^ d;
    }
    for (; i < n16; i += stride) acc ^= src[i];
    out[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

// Per-CU L2 -> CU throughput on a region small enough to stay in L2: each
// work-group (256 threads, one per CU) reads `region` bytes `iters` times.
// KIND 0: global_load_dwordx4 into registers (DEPTH loads in flight per thread,
// XOR-folded); KIND 1: global_load_lds_dwordx4 into an LDS ring (bursts of DEPTH
// KiB-blocks per wave, the ring 64 KiB), 64-bit lane addresses; KIND 2: the same with
// the compiler builtin; KIND 3: buffer_load_dwordx4 ... lds from a buffer resource
// (compiler builtin); KIND 4: as 1 with a scalar base and 32-bit lane offsets.
template <int KIND, int DEPTH>
__global__ void __launch_bounds__(1024) l2_stream(const char* src, int64_t region, int iters,
                                                  uint32_t* out) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nthr = blockDim.x;
    const int64_t per_pass = (int64_t)nthr * 16;                // bytes per WG instruction round
    const int64_t passes = region / per_pass;
    if constexpr (KIND == 0) {
        u32x4 acc = {0u, 0u, 0u, 0u};
        for (int it = 0; it < iters; ++it) {
            for (int64_t p = 0; p + DEPTH <= passes; p += DEPTH) {
                u32x4 v[DEPTH];
#pragma unroll
                for (int d = 0; d < DEPTH; ++d)
                    v[d] = *reinterpret_cast<const u32x4*>(src + (p + d) * per_pass +
                                                           threadIdx.x * 16);
#pragma unroll
                for (int d = 0; d < DEPTH; ++d) acc ^= v[d];
            }
        }
        out[(int64_t)blockIdx.x * nthr + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
    } else {
        __shared__ __attribute__((aligned(1024))) char ring[65536];
        // bursts of DEPTH loads per wave (unrolled, as a GEMM issues a K tile), then a
        // wait until the previous burst has landed; wave w's block for load d of a
        // burst: ring[((d % 4) * 16 + w) * 1024], 64 lanes x 16 B
        const uint32_t voff = threadIdx.x * 16;
        for (int it = 0; it < iters; ++it) {
            for (int64_t p = 0; p + DEPTH <= passes; p += DEPTH) {
#pragma unroll
                for (int d = 0; d < DEPTH; ++d) {
                    const uint32_t lds = (uint32_t)(uintptr_t)(
                        (__attribute__((address_space(3))) char*)(ring + ((d % 4) * 16 + wave) * 1024));
                    const char* base = src + (p + d) * per_pass;
                    if constexpr (KIND == 1) {
                        const char* g = base + voff;
                        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                                     :: "s"(lds), "v"(g) : "memory", "m0");
                    } else if constexpr (KIND == 4) {
                        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                                     :: "s"(lds), "v"(voff), "s"(base) : "memory", "m0");
                    } else if constexpr (KIND == 2) {
                        __builtin_amdgcn_global_load_lds(
                            (const void*)(base + voff),
                            (__attribute__((address_space(3))) void*)(uintptr_t)lds, 16, 0, 0);
                    } else {
                        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
                            (void*)base, (short)0, (int)per_pass, 0x00020000);
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(
                            r, (__attribute__((address_space(3))) void*)(uintptr_t)lds, 16, voff,
                            0, 0, 0);
                    }
                }
                __builtin_amdgcn_s_waitcnt((DEPTH & 15) | (7 << 4) | (15 << 8) | ((DEPTH >> 4) << 14));
            }
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        out[(int64_t)blockIdx.x * nthr + threadIdx.x] =
            *reinterpret_cast<const uint32_t*>(ring + threadIdx.x * 4);
    }
}

// LDS read throughput: each wave reads its own 16 KiB of a 128 KiB buffer (so at most
// 8 waves), 16 distinct reads per loop trip, addresses rotating with the trip so no
// read can be hoisted.  KIND 0: ds_read_b128 (a wave reads 1 KiB of consecutive
// 16-byte pieces: no bank conflict); KIND 1: the transposing ds_read_b64_tr_b16 (512
// bytes per wave read).
typedef short i16x4_d __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_d lds_i16x4_d;

template <int KIND>
__global__ void __launch_bounds__(512) lds_read(int iters, uint32_t* out) {
    __shared__ __attribute__((aligned(1024))) char buf[131072];
    for (int i = threadIdx.x; i < 131072 / 4; i += blockDim.x)
        reinterpret_cast<uint32_t*>(buf)[i] = (uint32_t)i * 2654435761u;
    __syncthreads();
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int base = (wave & 7) * 16384;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            if constexpr (KIND == 0) {
                const int off = base + (((j + it) & 15) << 10) + lane * 16;
                acc ^= *reinterpret_cast<const u32x4*>(buf + off);
            } else {
                const int off = base + (((j + it) & 15) << 9) + lane * 8;
                const i16x4_d v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_d*)(buf + off));
                acc.x ^= (uint32_t)(uint16_t)v.x | ((uint32_t)(uint16_t)v.y << 16);
                acc.y ^= (uint32_t)(uint16_t)v.z | ((uint32_t)(uint16_t)v.w << 16);
            }
        }
    }
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

}  // namespace

// LDS read throughput probe (see lds_read): kind 0 ds_read_b128, kind 1
// ds_read_b64_tr_b16; `blocks` work-groups of `waves` (1..8) waves, each wave making
// iters*16 reads; out: blocks*64*waves words (device).  Returns a hipError_t.
extern "C" int sg_diag_lds_read(int kind, int blocks, int waves, int iters, void* out,
                                void* stream) {
    if (!out || blocks <= 0 || waves < 1 || waves > 8 || iters < 1 || kind < 0 || kind > 1)
        return (int)hipErrorInvalidValue;
    hipStream_t st = (hipStream_t)stream;
    if (kind == 0)
        hipLaunchKernelGGL(lds_read<0>, dim3(blocks), dim3(64 * waves), 0, st, iters, (uint32_t*)out);
    else
        hipLaunchKernelGGL(lds_read<1>, dim3(blocks), dim3(64 * waves), 0, st, iters, (uint32_t*)out);
    return (int)hipGetLastError();
}

// Per-CU L2 -> CU throughput probe (see l2_stream): kind 0 registers, kinds 1-3 LDS DMA;
// depth in {4, 8, 16}; waves 1..16 per work-group; region (a multiple of waves*1024
// bytes) read iters times by each of `blocks` work-groups; out: blocks*64*waves words.
extern "C" int sg_diag_l2_stream(int kind, int depth, const void* src, int64_t region, int iters,
                                 int blocks, int waves, void* out, void* stream) {
    if (!src || !out || waves < 1 || waves > 16 || region < waves * 1024 ||
        region % (waves * 1024) != 0 || blocks <= 0 || iters < 1)
        return (int)hipErrorInvalidValue;
    hipStream_t st = (hipStream_t)stream;
    const char* s = (const char*)src;
    uint32_t* o = (uint32_t*)out;
#define L2S(K, D) hipLaunchKernelGGL((l2_stream<K, D>), dim3(blocks), dim3(64 * waves), 0, st, s, region, iters, o)
    if (kind == 0 && depth == 4) L2S(0, 4);
    else if (kind == 0 && depth == 8) L2S(0, 8);
    else if (kind == 0 && depth == 16) L2S(0, 16);
    else if (kind == 1 && depth == 4) L2S(1, 4);
    else if (kind == 1 && depth == 8) L2S(1, 8);
    else if (kind == 1 && depth == 16) L2S(1, 16);
    else if (kind == 2 && depth == 4) L2S(2, 4);
    else if (kind == 2 && depth == 8) L2S(2, 8);
    else if (kind == 2 && depth == 16) L2S(2, 16);
    else if (kind == 3 && depth == 4) L2S(3, 4);
    else if (kind == 3 && depth == 8) L2S(3, 8);
    else if (kind == 3 && depth == 16) L2S(3, 16);
    else if (kind == 4 && depth == 4) L2S(4, 4);
    else if (kind == 4 && depth == 8) L2S(4, 8);
    else if (kind == 4 && depth == 16) L2S(4, 16);
    else return (int)hipErrorInvalidValue;
#undef L2S
    return (int)hipGetLastError();
}

// Reads `bytes` (a multiple of 16) from the device buffer src with `blocks`
// work-groups of 256 threads; out: blocks*256 words (device).  Returns a hipError_t.
extern "C" int sg_diag_stream_read(const void* src, int64_t bytes, void* out, int blocks,
                                   void* stream) {
    if (!src || !out || bytes < 0 || bytes % 16 != 0 || blocks <= 0)
        return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(stream_read, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                       (const u32x4*)src, bytes / 16, (uint32_t*)out);
    return (int)hipGetLastError();
}

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
