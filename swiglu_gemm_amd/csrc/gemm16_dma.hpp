// gemm16_dma.hpp -- MFMA GEMM with direct global->LDS loads (gfx950), for 16-bit
// (fp16 / bf16, v_mfma_f32_32x32x16) and 8-bit (OCP e4m3, v_mfma_scale_f32_
// 32x32x64_f8f6f4 with unit block scales) operands; fp32 accumulation; the
// transposed accumulator D^T and the epilogues of epilogue16.hpp.
//
// Tiles travel from global memory straight into LDS with global_load_lds_dwordx4
// (16 bytes per lane, no VGPR staging) through a ring of S LDS stages, so loads
// run S-1 tiles ahead of the MFMAs.
//
// LDS layouts, chosen so both operand orientations feed the MFMA directly:
// * k-contiguous operand (A 'N', B 'T'): [R][BK] with 16-byte chunks XOR-swizzled
//   by row; a fragment (32 rows x one k-step per lane) is one (16-bit) or two
//   (8-bit) ds_read_b128.
// * row-contiguous operand (A 'T', B 'N', W_fused): [BK][R] as stored in memory,
//   32-byte units XOR-swizzled by k; the fragment comes from ds_read_b64_tr_b16
//   (x2) or ds_read_b64_tr_b8 (x4): each 16-lane group turns 4 (8) row pieces into
//   4 (8) k-values per lane.
// The swizzles keep every 16-lane / 32-lane LDS phase on distinct banks.  The DMA
// writes 1 KiB per wave instruction in lane order; the swizzle is applied by
// choosing which global 16-byte chunk each lane fetches.
//
// W_fused keeps its interleaved column order: in the D^T accumulator layout fused
// columns (2n, 2n+1) land in registers (r, r+1) of one lane, so the SwiGLU
// epilogue pairs them in registers ("Resumo Técnico: Sobreposição de Ativação em
// Nível de Tile ...", Metodologia / Kernel-2) and stages the bf16/fp16 outputs
// through the then idle LDS ring for row-contiguous stores.
//
// Edge tiles: a k-contiguous operand's rows past M (N) are clamped to the last
// valid row, and a row-contiguous operand's 16-byte chunks past N (M) to the
// last valid chunk, so every load stays inside the operand; the outputs those
// rows/columns feed are never stored.  K must be a multiple of BK (no K tail),
// operands 16-byte aligned with ld*size % 16 == 0, and for a row-contiguous
// operand its row length*size % 16 == 0; other problems take gemm16.hpp or the
// generic e4m3 kernel.
#pragma once

#include <type_traits>

#include "epilogue16.hpp"
#include "sg_device.hpp"

namespace sg {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));

template <bool KC, int R, int BK, int ESZ>
struct DmaTile {
    static constexpr int ROW_BYTES = KC ? BK * ESZ : R * ESZ;
    static constexpr int BYTES = R * BK * ESZ;
    static constexpr int SLOTS = ROW_BYTES / 16;         // 16-byte slots per row
    static constexpr int BLOCKS = BYTES / 1024;          // 1 KiB DMA blocks
    static constexpr int UNITS = ROW_BYTES / 32;         // row-contiguous: 32-byte units
    static_assert(BYTES % 1024 == 0, "whole 1 KiB DMA blocks");
    static_assert(KC ? (ROW_BYTES == 64 || ROW_BYTES == 128)
                     : (ROW_BYTES >= 128 && ROW_BYTES <= 1024 && ROW_BYTES % 64 == 0),
                  "unsupported tile");

    // Physical 16-byte chunk (KC) or 32-byte unit (row-contiguous) XOR mask for a
    // row.  A row-contiguous fragment read touches one or two units of 4 (16-bit)
    // or 8 (8-bit) consecutive k rows in one LDS phase; unit u of row k sits at
    // 32-byte bank slot (UNITS*k + (u ^ swz(k))) mod 8, and the masks below make
    // those slots distinct for every even UNITS (XOR stays inside the row: UNITS
    // is a multiple of the largest mask + 1 in each case).
    static __device__ __forceinline__ int swz(int row) {
        if constexpr (KC) {
            if constexpr (ROW_BYTES == 128) return (row & 7) ^ ((row >> 3) & 1);
            else return (row >> 2) & 3;
        } else if constexpr (ESZ == 2) {
            if constexpr (UNITS % 8 == 0) return (row & 3) << 1;   // 4 rows x 2 units
            else if constexpr (UNITS % 8 == 4) return row & 2;     // rows alternate halves
            else return 0;                                         // UNITS = 2 mod 4
        } else {
            if constexpr (UNITS % 8 == 0) return row & 7;          // 8 rows x 1 unit
            else if constexpr (UNITS % 8 == 4) return (row >> 1) & 3;
            else return (row >> 2) & 1;                            // UNITS = 2 mod 4
        }
    }
};

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// One operand's DMA stream: NI instructions per thread per K tile.  Each lane's
// chunk is a fixed 32-bit byte offset from a wave-uniform tile base held in SGPRs
// (the global_load_lds "saddr" form), so advancing a K tile costs one scalar add
// and no vector instruction (measured on MI355X: fp16 8192^3 908 -> 865 us, bf16
// 8192 x 4096 x 4096 with B stored N x K 228 -> 217 us against per-lane 64-bit
// addresses; bit-identical).  The host admits a problem only when every offset fits
// in 31 bits (dma_ok in api.hip).
template <bool KC, int R, int BK, int ESZ, int NWAVES>
struct DmaStream {
    using T = DmaTile<KC, R, BK, ESZ>;
    static_assert(T::BLOCKS % NWAVES == 0, "DMA blocks must split evenly over the waves");
    static constexpr int NI = T::BLOCKS / NWAVES;
    uint32_t off[NI];   // byte offset of each lane's chunk from the tile base
    const char* base;   // the tile's base at the stream's first k (wave-uniform)
    int64_t step;       // bytes to advance per K tile

    __device__ __forceinline__ void init(const void* base_, int64_t ld, int r0, int rows, int k0,
                                         int wave, int lane) {
        const char* b0 = reinterpret_cast<const char*>(base_);
        base = KC ? b0 + ((int64_t)r0 * ld + k0) * ESZ : b0 + (int64_t)k0 * ld * ESZ + r0 * ESZ;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int b = wave + i * NWAVES;
            const int chunk = b * 64 + lane;
            const int row = chunk / T::SLOTS;
            const int slot = chunk % T::SLOTS;
            if constexpr (KC) {
                const int c = slot ^ T::swz(row);
                const int r = min(r0 + row, rows - 1) - r0;
                off[i] = (uint32_t)((int64_t)r * ld * ESZ + c * 16);
            } else {
                const int u = (slot >> 1) ^ T::swz(row);
                const int cb = min(r0 * ESZ + u * 32 + (slot & 1) * 16, (rows * ESZ - 1) & ~15);
                off[i] = (uint32_t)((int64_t)row * ld * ESZ + cb - r0 * ESZ);
            }
        }
        step = KC ? (int64_t)BK * ESZ : (int64_t)BK * ld * ESZ;
    }
    // Issue the DMA of K tile `t` (relative to the split start) into stage memory.
    // Written as inline asm so the compiler does not model the asynchronous LDS
    // write (it would otherwise drain every outstanding load before each LDS
    // read); completion is enforced by wait_vmcnt + s_barrier in the main loop.
    // The LDS-DMA reads M0 as its LDS address; a scalar write of M0 needs one wait
    // state before that read on this GPU family (the s_nop the compiler's hazard
    // recognizer would insert, which it cannot do inside an asm statement).
    __device__ __forceinline__ void issue_one(char* stage, int t, int wave, int i) const {
        const char* bt = base + t * step;
        const int b = wave + i * NWAVES;
        const uint32_t lds = (uint32_t)(uintptr_t)(
            (__attribute__((address_space(3))) char*)(stage + b * 1024));
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                     :: "s"(lds), "v"(off[i]), "s"(bt) : "memory", "m0");
    }
    __device__ __forceinline__ void issue(char* stage, int t, int wave) const {
#pragma unroll
        for (int i = 0; i < NI; ++i) issue_one(stage, t, wave, i);
    }
    // A trailing partial K tile (the stream initialised at its first k), of which
    // only the first `kvalid` k belong to the problem: loaded through registers into
    // the LDS positions issue() would fill, zero at k >= kvalid, so fragment reads
    // and MFMAs are those of a full tile.  A chunk that holds the problem's last k
    // is read whole: it is 16-byte aligned and its first byte is in the operand, so
    // it lies in a page that is mapped; the bytes past K are then cleared.  Chunks
    // wholly past K are not read.
    __device__ __forceinline__ void load_tail(char* stage, int kvalid, int wave, int lane) const {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int b = wave + i * NWAVES;
            const int chunk = b * 64 + lane;
            const int row = chunk / T::SLOTS;
            const int slot = chunk % T::SLOTS;
            const char* g = base + off[i];
            u32x4 v = {0u, 0u, 0u, 0u};
            if constexpr (KC) {
                constexpr int EPC = 16 / ESZ;                       // elements per chunk
                const int n = kvalid - (slot ^ T::swz(row)) * EPC;  // of them in the problem
                if (n > 0) {
                    v = *reinterpret_cast<const u32x4*>(g);
                    if (n < EPC) {
#pragma unroll
                        for (int d = 0; d < 4; ++d) {
                            const int nb = n * ESZ - 4 * d;         // valid bytes of dword d
                            v[d] = nb >= 4 ? v[d] : nb <= 0 ? 0u : v[d] & ((1u << (8 * nb)) - 1u);
                        }
                    }
                }
            } else if (row < kvalid) {
                v = *reinterpret_cast<const u32x4*>(g);
            }
            *reinterpret_cast<u32x4*>(stage + b * 1024 + lane * 16) = v;
        }
    }
};

// Per-lane MFMA operand: 16-bit: 8 k-values (u32x4); 8-bit: 32 k-values (u32x8).
template <int ESZ> struct FragT;
template <> struct FragT<2> { typedef u32x4 type; };
template <> struct FragT<1> { typedef u32x8 type; };

// Fragment for k-step s: rows rbase + lane%32; k = KSTEP*s + (KSTEP/2)*(lane/32) +
// 0..KSTEP/2-1, with KSTEP = 16 (16-bit) or 64 (8-bit) elements.
template <bool KC, int R, int BK, int ESZ>
__device__ __forceinline__ typename FragT<ESZ>::type read_frag(const char* tile, int rbase, int s,
                                                               int lane) {
    using T = DmaTile<KC, R, BK, ESZ>;
    if constexpr (KC) {
        const int row = rbase + (lane & 31);
        const char* rp = tile + row * T::ROW_BYTES;
        if constexpr (ESZ == 2) {
            const int chunk = 2 * s + (lane >> 5);
            return *reinterpret_cast<const u32x4*>(rp + ((chunk ^ T::swz(row)) << 4));
        } else {
            const int chunk = 4 * s + 2 * (lane >> 5);
            const u32x4 a = *reinterpret_cast<const u32x4*>(rp + ((chunk ^ T::swz(row)) << 4));
            const u32x4 b = *reinterpret_cast<const u32x4*>(rp + (((chunk + 1) ^ T::swz(row)) << 4));
            return u32x8{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        }
    } else if constexpr (ESZ == 2) {
        const int g = lane >> 4, L = lane & 15, j = L >> 2, q = L & 3;
        const int r = rbase + 16 * (g & 1) + 4 * q;          // element column of this piece
        const int k0 = 16 * s + 8 * (g >> 1) + j;
        const int k1 = k0 + 4;
        const char* p0 = tile + k0 * T::ROW_BYTES + (((r >> 4) ^ T::swz(k0)) << 5) + ((r & 15) << 1);
        const char* p1 = tile + k1 * T::ROW_BYTES + (((r >> 4) ^ T::swz(k1)) << 5) + ((r & 15) << 1);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p1));
        const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
        return u32x4{a.x, a.y, b.x, b.y};
    } else {
        // 16 lanes read an 8 x 16-byte block (lanes 2j, 2j+1 give row j) and lane i
        // receives byte i of each row: 8 consecutive k for column rbase + lane%32
        const int g = lane >> 4, i = lane & 15, j = i >> 1, h = i & 1;
        const int c = rbase + 16 * (g & 1) + 8 * h;          // byte column of this piece
        const int kb = 64 * s + 32 * (g >> 1) + j;
        u32x8 out;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int k = kb + 8 * rr;
            const char* pp = tile + k * T::ROW_BYTES + (((c >> 5) ^ T::swz(k)) << 5) + (c & 31);
            const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(pp));
            out[2 * rr] = (uint32_t)v.x;
            out[2 * rr + 1] = (uint32_t)v.y;
        }
        return out;
    }
}

template <int DT>
__device__ __forceinline__ f32x16 mfma_op(const typename FragT<DT == DT_E4M3 ? 1 : 2>::type& a,
                                          const typename FragT<DT == DT_E4M3 ? 1 : 2>::type& b,
                                          const f32x16& c) {
    if constexpr (DT == DT_E4M3) {
        // format 0 = e4m3 for both operands; E8M0 block scale 0x7F = 2^0
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            __builtin_bit_cast(i32x8, a), __builtin_bit_cast(i32x8, b), c, 0, 0, 0, 0x7F7F7F7F, 0,
            0x7F7F7F7F);
    } else {
        return mfma16<DT>(a, b, c);
    }
}

// Compile-time shape of the direct-to-LDS kernels.  BK is in elements.  Output
// type: DT for 16-bit operands, bf16 for e4m3.
template <int DT, bool TA, bool TB, int EPI, int BM, int BN, int BK, int S, int WM, int WN>
struct DmaShape {
    static constexpr int ESZ = DT == DT_E4M3 ? 1 : 2;
    static constexpr int DT_OUT = DT == DT_E4M3 ? DT_BF16 : DT;
    static constexpr int KSTEP = ESZ == 2 ? 16 : 64;
    static constexpr int NW = WM * WN;
    static constexpr int TM = BM / WM, TN = BN / WN;
    static constexpr int FM = TM / 32, FN = TN / 32;
    static constexpr int KS = BK / KSTEP;
    static_assert(BK % KSTEP == 0 && KS % 2 == 0, "k-steps per tile must be even");
    static constexpr bool KCA = !TA, KCB = TB;          // k-contiguous operands
    // EPI_SWIGLU_W12: the B tile is BN/2 columns of W1 followed by the same BN/2
    // columns of W2; a wave's fragments tn < FN/2 are gate, tn + FN/2 the matching up.
    // EPI_SWIGLU_SEQ: the same output columns and fragment roles, but each stage holds
    // one B tile of BN/2 columns: W1's for the first K/BK tiles, then W2's.
    static constexpr bool W12 = EPI == EPI_SWIGLU_W12;
    static constexpr bool SEQ = EPI == EPI_SWIGLU_SEQ;
    static_assert(!(W12 || SEQ) || (!TA && !TB && FN % 2 == 0 && BN % 64 == 0),
                  "split-weight SwiGLU tile");
    static constexpr int BNS = (W12 || SEQ) ? BN / 2 : BN;   // columns per B source
    static constexpr int NBS = W12 ? 2 : 1;                   // B tiles per stage
    using TA_ = DmaTile<KCA, BM, BK, ESZ>;
    using TB_ = DmaTile<KCB, BNS, BK, ESZ>;
    static constexpr int STAGE = TA_::BYTES + NBS * TB_::BYTES;
    static constexpr int LDS = S * STAGE;
    static_assert(LDS <= 160 * 1024, "LDS budget");
    static constexpr int NL =
        DmaStream<KCA, BM, BK, ESZ, NW>::NI + NBS * DmaStream<KCB, BNS, BK, ESZ, NW>::NI;
    using Frag = typename FragT<ESZ>::type;
    using Acc = f32x16[FN][FM];
};

// acc += op(A) * op(B) over K tiles [kbeg, kbeg + nkt*BK) of the output tile at
// (m0, n0), plus a trailing partial tile of ktail (< BK) k when K is not a multiple
// of BK: the S-stage direct-to-LDS ring feeding the MFMAs.  Every thread of the
// work-group calls it; LDS is free on return only after a barrier (the last k-step
// reads a stage without one).
template <int DT, bool TA, bool TB, int EPI, int BM, int BN, int BK, int S, int WM, int WN>
__device__ __forceinline__ void dma_mainloop(
    const Gemm16Params& p, char* smem, int m0, int n0, int kbeg, int nkt, int ktail,
    typename DmaShape<DT, TA, TB, EPI, BM, BN, BK, S, WM, WN>::Acc& acc, int wave, int lane) {
    using D = DmaShape<DT, TA, TB, EPI, BM, BN, BK, S, WM, WN>;
    constexpr int ESZ = D::ESZ, FM = D::FM, FN = D::FN, KS = D::KS, TM = D::TM, TN = D::TN;
    constexpr bool KCA = D::KCA, KCB = D::KCB, W12 = D::W12;
    constexpr int BNS = D::BNS, NW = D::NW, STAGE = D::STAGE, NL = D::NL;
    using TA_ = typename D::TA_;
    using TB_ = typename D::TB_;
    using Frag = typename D::Frag;
    const int wm = wave % WM, wn = wave / WM;
    // One wave per SIMD: no second wave keeps the matrix core fed while this one
    // issues the next tile's DMA, so the DMA is dealt out between the MFMAs, one
    // slot after each fragment column q of the k-steps before the barrier; with 2
    // stages (tile t+1 must land by the end of tile t) only the first k-step's.
    // Measured on MI355X against the whole DMA at the top of the tile (fp16 8192^3,
    // one run): 256x256x64 2 stages 937 -> 892 us, 256x256x32 4 stages 970 -> 925
    // us, 128x128x64 3 stages 1302 -> 1257 us; the 8-wave tiles keep the burst.
    // Dealing it over the k-step after the barrier as well was no better.
    constexpr bool SPREAD = NW == 4 && !W12;
    // Two-stage rings of 16-bit operands run unrolled by two tiles, so each stage is
    // a compile-time constant; with the stages laid out [A0 A1 | B0 B1] every stage
    // offset is below 64 KiB and folds into the LDS reads' immediate field, and the
    // per-read address adds of a run-time stage go away (NT main loop per two tiles:
    // 60 -> 9 VALU instructions).  Measured on MI355X, alternating builds, bit-
    // identical: fp16 8192^3 NN 873.8 -> 864.7 us, NT 889.1 -> 881.5 us, bf16 NN
    // 836.9 -> 825.9 us, bf16 8192 x 4096 x 4096 NT 216.6 -> 213.2 us.  e4m3
    // fragments are twice as wide: the hoisted addresses there pushed the 256x256
    // tile past 256 registers into scratch (4.6x slower), so 8-bit rings keep the
    // interleaved layout and the rolled loop, and so do waves of more than 8
    // fragments (the 256x320 tile spilled 16-32 bytes).  Other rings: [A0 B0 | A1
    // B1 | ..].
    constexpr bool SPLIT = S == 2 && !W12 && !SPREAD && ESZ == 2 && FM * FN <= 8;
    auto stA = [&](int st) -> char* { return SPLIT ? smem + st * TA_::BYTES : smem + st * STAGE; };
    auto stB = [&](int st) -> char* {
        return SPLIT ? smem + S * TA_::BYTES + st * TB_::BYTES : smem + st * STAGE + TA_::BYTES;
    };

    DmaStream<KCA, BM, BK, ESZ, NW> da;
    DmaStream<KCB, BNS, BK, ESZ, NW> db, db2;
    da.init(p.A, p.lda, m0, p.M, kbeg, wave, lane);
    if constexpr (W12) {
        db.init(p.B, p.ldb, n0 / 2, p.N / 2, kbeg, wave, lane);
        db2.init(p.B2, p.ldb, n0 / 2, p.N / 2, kbeg, wave, lane);
    } else {
        db.init(p.B, p.ldb, n0, p.N, kbeg, wave, lane);
    }

    Frag fa[2][FM], fb[2][FN];
    auto read_all = [&](int sti, int s, Frag (&af)[FM], Frag (&bf)[FN]) __attribute__((always_inline)) {
        const char* sa = stA(sti);
        const char* sb = stB(sti);
#pragma unroll
        for (int tm = 0; tm < FM; ++tm)
            af[tm] = read_frag<KCA, BM, BK, ESZ>(sa, wm * TM + tm * 32, s, lane);
#pragma unroll
        for (int tn = 0; tn < FN; ++tn) {
            if constexpr (W12) {
                constexpr int FH = FN / 2;
                const char* half = sb + (tn / FH) * TB_::BYTES;
                bf[tn] = read_frag<KCB, BNS, BK, ESZ>(half, wn * (TN / 2) + (tn % FH) * 32, s, lane);
            } else {
                bf[tn] = read_frag<KCB, BN, BK, ESZ>(sb, wn * TN + tn * 32, s, lane);
            }
        }
    };
    auto mfma_all = [&](const Frag (&af)[FM], const Frag (&bf)[FN]) __attribute__((always_inline)) {
#pragma unroll
        for (int tn = 0; tn < FN; ++tn)
#pragma unroll
            for (int tm = 0; tm < FM; ++tm) acc[tn][tm] = mfma_op<DT>(bf[tn], af[tm], acc[tn][tm]);
    };
    auto issue = [&](int t) {
        const int sti = t % S;
        da.issue(stA(sti), t, wave);
        db.issue(stB(sti), t, wave);
        if constexpr (W12) db2.issue(stB(sti) + TB_::BYTES, t, wave);
    };

    if (nkt > 0) {
#pragma unroll
        for (int i = 0; i < S - 1; ++i)
            if (i < nkt) issue(i);
        if (nkt >= S - 1) wait_vmcnt<(S - 2) * NL>();
        else wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        read_all(0, 0, fa[0], fb[0]);

        constexpr int NMF = FM * FN;
        constexpr int RD_KC = ESZ == 2 ? 1 : 2, RD_RC = ESZ == 2 ? 2 : 4;
        constexpr int NRD = (KCA ? RD_KC : RD_RC) * FM + (KCB ? RD_KC : RD_RC) * FN;
        constexpr int NIA = DmaStream<KCA, BM, BK, ESZ, NW>::NI;
        constexpr int NSLOT = (S >= 3 ? KS - 1 : 1) * FN;
        // DMA slot j of tile u into stage sti
        auto slot_dma = [&](int sti, int u, int j) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < NL; ++i) {
                if (i * NSLOT / NL != j) continue;
                if (i < NIA) da.issue_one(stA(sti), u, wave, i);
                else db.issue_one(stB(sti), u, wave, i - NIA);
            }
        };
        // fragment column q of k-step s: its MFMAs on fragments (fa, fb)[s & 1], and the
        // reads of k-step s2 of stage st2 into the other fragment set
        auto column = [&](int s, int q, int st2, int s2) __attribute__((always_inline)) {
#pragma unroll
            for (int tm = q % FN; tm < FM; tm += FN)
                fa[s2 & 1][tm] = read_frag<KCA, BM, BK, ESZ>(stA(st2), wm * TM + tm * 32, s2, lane);
            fb[s2 & 1][q] = read_frag<KCB, BN, BK, ESZ>(stB(st2), wn * TN + q * 32, s2, lane);
#pragma unroll
            for (int tm = 0; tm < FM; ++tm)
                acc[q][tm] = mfma_op<DT>(fb[s & 1][q], fa[s & 1][tm], acc[q][tm]);
        };
        // One K tile: its k-steps (with the DMA of tile t+S-1 dealt between the MFMAs
        // for one wave per SIMD, or issued at the top), the wait and barrier for tile
        // t+1, then tile t+1's first fragments under tile t's last MFMAs.  sc, sn:
        // the stages of tiles t and t+1.
        auto tile = [&](int t, int sc, int sn) __attribute__((always_inline)) {
            const bool ahead = t + S - 1 < nkt;
            if constexpr (SPREAD) {
                const int sx = (t + S - 1) % S;
#pragma unroll
                for (int s = 0; s + 1 < KS; ++s) {
#pragma unroll
                    for (int q = 0; q < FN; ++q) {
                        column(s, q, sc, s + 1);
                        if (ahead) slot_dma(sx, t + S - 1, s * FN + q);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            } else {
                if (ahead) issue(t + S - 1);
#pragma unroll
                for (int s = 0; s + 1 < KS; ++s) {
                    read_all(sc, s + 1, fa[(s + 1) & 1], fb[(s + 1) & 1]);
                    mfma_all(fa[s & 1], fb[s & 1]);
                    sched_interleave<NMF, NRD, 0, 0>();
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            // tile t+1 must have landed (own DMAs), then everyone's
            if (ahead) wait_vmcnt<(S - 2) * NL>();
            else wait_vmcnt<0>();
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            // last k-step of tile t overlaps the first fragments of tile t+1 (on
            // the last tile this reads a stale stage whose values are never used)
            read_all(sn, 0, fa[0], fb[0]);
            mfma_all(fa[1], fb[1]);
            sched_interleave<NMF, NRD, 0, 0>();
            __builtin_amdgcn_sched_barrier(0);
        };
        if constexpr (SPLIT) {
            int t = 0;
            for (; t + 1 < nkt; t += 2) {
                tile(t, 0, 1);
                tile(t + 1, 1, 0);
            }
            if (t < nkt) tile(t, 0, 1);
        } else {
            for (int t = 0; t < nkt; ++t) tile(t, t % S, (t + 1) % S);
        }
    }
    if (ktail > 0) {
        // every DMA has landed (the ring's last wait is for all of them); once every
        // wave is past its reads, stage 0 takes the zero-filled tail tile.  The
        // addresses are computed afresh (an opaque lane index keeps the compiler from
        // carrying the main loop's through it).
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int kt = kbeg + nkt * BK;
        __syncthreads();
        {
            DmaStream<KCA, BM, BK, ESZ, NW> ta;
            ta.init(p.A, p.lda, m0, p.M, kt, wave, ln);
            ta.load_tail(stA(0), ktail, wave, ln);
        }
        if constexpr (W12) {
            DmaStream<KCB, BNS, BK, ESZ, NW> tb, tb2;
            tb.init(p.B, p.ldb, n0 / 2, p.N / 2, kt, wave, ln);
            tb.load_tail(stB(0), ktail, wave, ln);
            tb2.init(p.B2, p.ldb, n0 / 2, p.N / 2, kt, wave, ln);
            tb2.load_tail(stB(0) + TB_::BYTES, ktail, wave, ln);
        } else {
            DmaStream<KCB, BNS, BK, ESZ, NW> tb;
            tb.init(p.B, p.ldb, n0, p.N, kt, wave, ln);
            tb.load_tail(stB(0), ktail, wave, ln);
        }
        __syncthreads();
        for (int s = 0; s < KS && s * D::KSTEP < ktail; ++s) {   // k-steps past K add 0
            read_all(0, s, fa[0], fb[0]);
            mfma_all(fa[0], fb[0]);
        }
    }
}

// Split-weight SwiGLU with Gate and Up one after the other ("Resumo Técnico:
// Sobreposição de Ativação em Nível de Tile ...", Metodologia / Kernel-1): the
// work-group's output tile is BM rows x BN/2 columns of Y.  One S-stage ring runs
// over 2*nkt K tiles -- (A, W1) for tiles 0..nkt-1 into the gate accumulators
// (fragments tn < FN/2), then (A, W2) into the up accumulators (tn + FN/2).  The
// ring issues S-1 tiles ahead, so when the last Gate tile is consumed the first Up
// tiles are already in flight: SiLU(s * gate) is evaluated in registers while they
// land (the page's overlap of the Swish with the Up-tile loads), and the epilogue
// multiplies by s * up and stores.  K must be a multiple of BK (the chooser checks).
template <int DT, bool TA, bool TB, int EPI, int BM, int BN, int BK, int S, int WM, int WN>
__device__ __forceinline__ void dma_mainloop_seq(
    const Gemm16Params& p, char* smem, int m0, int n0, int nkt,
    typename DmaShape<DT, TA, TB, EPI, BM, BN, BK, S, WM, WN>::Acc& acc, int wave, int lane) {
    using D = DmaShape<DT, TA, TB, EPI, BM, BN, BK, S, WM, WN>;
    static_assert(D::SEQ, "sequential SwiGLU only");
    constexpr int ESZ = D::ESZ, FM = D::FM, FN = D::FN, KS = D::KS, TM = D::TM, TN = D::TN;
    constexpr int BNS = D::BNS, NW = D::NW, STAGE = D::STAGE, NL = D::NL, FH = FN / 2;
    using TA_ = typename D::TA_;
    using Frag = typename D::Frag;
    const int wm = wave % WM, wn = wave / WM;

    DmaStream<true, BM, BK, ESZ, NW> da;
    DmaStream<false, BNS, BK, ESZ, NW> d1, d2;
    da.init(p.A, p.lda, m0, p.M, 0, wave, lane);
    d1.init(p.B, p.ldb, n0 / 2, p.N / 2, 0, wave, lane);
    d2.init(p.B2, p.ldb, n0 / 2, p.N / 2, 0, wave, lane);
    const int T = 2 * nkt;

    Frag fa[2][FM], fb[2][FH];
    auto read_all = [&](const char* st, int s, Frag (&af)[FM], Frag (&bf)[FH]) {
#pragma unroll
        for (int tm = 0; tm < FM; ++tm)
            af[tm] = read_frag<true, BM, BK, ESZ>(st, wm * TM + tm * 32, s, lane);
#pragma unroll
        for (int tn = 0; tn < FH; ++tn)
            bf[tn] = read_frag<false, BNS, BK, ESZ>(st + TA_::BYTES, wn * (TN / 2) + tn * 32, s,
                                                   lane);
    };
    auto issue = [&](int t) {
        char* st = smem + (t % S) * STAGE;
        if (t < nkt) {
            da.issue(st, t, wave);
            d1.issue(st + TA_::BYTES, t, wave);
        } else {
            da.issue(st, t - nkt, wave);
            d2.issue(st + TA_::BYTES, t - nkt, wave);
        }
    };
    constexpr int NMF = FM * FH;
    constexpr int RD_RC = ESZ == 2 ? 2 : 4, RD_KC = ESZ == 2 ? 1 : 2;
    constexpr int NRD = RD_KC * FM + RD_RC * FH;
    // tiles [t0, t1) into the accumulator fragments OFF .. OFF + FH - 1
    auto phase = [&](auto off, int t0, int t1) __attribute__((always_inline)) {
        constexpr int OFF = decltype(off)::value;
        auto mfma_all = [&](const Frag (&af)[FM], const Frag (&bf)[FH]) {
#pragma unroll
            for (int tn = 0; tn < FH; ++tn)
#pragma unroll
                for (int tm = 0; tm < FM; ++tm)
                    acc[OFF + tn][tm] = mfma_op<DT>(bf[tn], af[tm], acc[OFF + tn][tm]);
        };
        for (int t = t0; t < t1; ++t) {
            const char* cur = smem + (t % S) * STAGE;
            const bool ahead = t + S - 1 < T;
            if (ahead) issue(t + S - 1);
#pragma unroll
            for (int s = 0; s + 1 < KS; ++s) {
                read_all(cur, s + 1, fa[(s + 1) & 1], fb[(s + 1) & 1]);
                mfma_all(fa[s & 1], fb[s & 1]);
                sched_interleave<NMF, NRD, 0, 0>();
                __builtin_amdgcn_sched_barrier(0);
            }
            if (ahead) wait_vmcnt<(S - 2) * NL>();
            else wait_vmcnt<0>();
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            // the next tile's first fragments (on the last tile: a stale stage, unused)
            read_all(smem + ((t + 1) % S) * STAGE, 0, fa[0], fb[0]);
            mfma_all(fa[1], fb[1]);
            sched_interleave<NMF, NRD, 0, 0>();
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    if (nkt <= 0) return;
#pragma unroll
    for (int i = 0; i < S - 1; ++i)
        if (i < T) issue(i);
    if (T >= S - 1) wait_vmcnt<(S - 2) * NL>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    read_all(smem, 0, fa[0], fb[0]);
    phase(std::integral_constant<int, 0>{}, 0, nkt);
    // SiLU(s * gate) while the first Up tiles land
    const float sc = DT == DT_E4M3 ? p.alpha : 1.0f;
#pragma unroll
    for (int tn = 0; tn < FH; ++tn)
#pragma unroll
        for (int tm = 0; tm < FM; ++tm)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[tn][tm][e] = silu(sc * acc[tn][tm][e]);
    __builtin_amdgcn_sched_barrier(0);
    phase(std::integral_constant<int, FH>{}, nkt, T);
}

// Kernel-1 with its loads and its MFMAs in separate wave groups ("Resumo Técnico:
// Sobreposição de Ativação em Nível de Tile ...", Metodologia / Kernel-1: producer
// warps load the tiles, consumer warps compute, SiLU(Gate) overlapping the Up
// loads).  The work-group holds WM x WN consumer waves (the accumulators and MFMAs
// of dma_mainloop_seq) and kWsProducers producer waves that only drive the S-stage
// direct-to-LDS ring: they issue tile t+S-1, wait for their own loads of tile t+1
// and meet the consumers at the one barrier per tile.  Both groups run the same
// loops, so they pass the same barriers; while the consumers evaluate SiLU(s*gate)
// the producers are already issuing the first Up tiles.  Products and K order are
// those of dma_mainloop_seq (bit-identical output).
constexpr int kWsProducers = 4;

template <int DT, bool TA, bool TB, int EPI, int BM, int BN, int BK, int S, int WM, int WN>
__device__ __forceinline__ void ws_mainloop_seq(
    const Gemm16Params& p, char* smem, int m0, int n0, int nkt,
    typename DmaShape<DT, TA, TB, EPI, BM, BN, BK, S, WM, WN>::Acc& acc, int wave, int lane) {
    using D = DmaShape<DT, TA, TB, EPI, BM, BN, BK, S, WM, WN>;
    static_assert(D::SEQ, "sequential SwiGLU only");
    constexpr int ESZ = D::ESZ, FM = D::FM, FN = D::FN, KS = D::KS, TM = D::TM, TN = D::TN;
    constexpr int BNS = D::BNS, NW = D::NW, STAGE = D::STAGE, FH = FN / 2;
    constexpr int NP = kWsProducers;
    using TA_ = typename D::TA_;
    using Frag = typename D::Frag;
    using SA = DmaStream<true, BM, BK, ESZ, NP>;
    using SB = DmaStream<false, BNS, BK, ESZ, NP>;
    constexpr int NLP = SA::NI + SB::NI;           // loads per producer thread and tile
    static_assert((S - 2) * NLP < 64, "vmcnt range");
    const bool producer = wave >= NW;              // wave-uniform
    const int pw = producer ? wave - NW : 0;
    const int wm = wave % WM, wn = (wave / WM) % WN;
    const int T = 2 * nkt;

    SA da;
    SB d1, d2;
    if (producer) {
        da.init(p.A, p.lda, m0, p.M, 0, pw, lane);
        d1.init(p.B, p.ldb, n0 / 2, p.N / 2, 0, pw, lane);
        d2.init(p.B2, p.ldb, n0 / 2, p.N / 2, 0, pw, lane);
    }
    auto issue = [&](int t) {
        char* st = smem + (t % S) * STAGE;
        if (t < nkt) {
            da.issue(st, t, pw);
            d1.issue(st + TA_::BYTES, t, pw);
        } else {
            da.issue(st, t - nkt, pw);
            d2.issue(st + TA_::BYTES, t - nkt, pw);
        }
    };
    if (nkt <= 0) return;
    if (producer) {
        // one barrier after the first tile has landed, then one per tile: the loads of
        // tile t+S-1, then tile t+1 must have landed (the consumers' barrier count)
#pragma unroll
        for (int i = 0; i < S - 1; ++i)
            if (i < T) issue(i);
        if (T >= S - 1) wait_vmcnt<(S - 2) * NLP>();
        else wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();
        for (int t = 0; t < T; ++t) {
            if (t + S - 1 < T) {
                issue(t + S - 1);
                wait_vmcnt<(S - 2) * NLP>();
            } else {
                wait_vmcnt<0>();
            }
            __builtin_amdgcn_s_barrier();
        }
        return;
    }

    Frag fa[2][FM], fb[2][FH];
    auto read_all = [&](const char* st, int s, Frag (&af)[FM], Frag (&bf)[FH]) {
#pragma unroll
        for (int tm = 0; tm < FM; ++tm)
            af[tm] = read_frag<true, BM, BK, ESZ>(st, wm * TM + tm * 32, s, lane);
#pragma unroll
        for (int tn = 0; tn < FH; ++tn)
            bf[tn] = read_frag<false, BNS, BK, ESZ>(st + TA_::BYTES, wn * (TN / 2) + tn * 32, s,
                                                   lane);
    };
    constexpr int NMF = FM * FH;
    constexpr int RD_RC = ESZ == 2 ? 2 : 4, RD_KC = ESZ == 2 ? 1 : 2;
    constexpr int NRD = RD_KC * FM + RD_RC * FH;
    // consumers: tiles [t0, t1) into the accumulator fragments OFF .. OFF + FH - 1,
    // one barrier per tile
    auto phase = [&](auto off, int t0, int t1) __attribute__((always_inline)) {
        constexpr int OFF = decltype(off)::value;
        auto mfma_all = [&](const Frag (&af)[FM], const Frag (&bf)[FH]) {
#pragma unroll
            for (int tn = 0; tn < FH; ++tn)
#pragma unroll
                for (int tm = 0; tm < FM; ++tm)
                    acc[OFF + tn][tm] = mfma_op<DT>(bf[tn], af[tm], acc[OFF + tn][tm]);
        };
        for (int t = t0; t < t1; ++t) {
            const char* cur = smem + (t % S) * STAGE;
#pragma unroll
            for (int s = 0; s + 1 < KS; ++s) {
                read_all(cur, s + 1, fa[(s + 1) & 1], fb[(s + 1) & 1]);
                mfma_all(fa[s & 1], fb[s & 1]);
                sched_interleave<NMF, NRD, 0, 0>();
                __builtin_amdgcn_sched_barrier(0);
            }
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            // the next tile's first fragments (on the last tile: a stale stage, unused)
            read_all(smem + ((t + 1) % S) * STAGE, 0, fa[0], fb[0]);
            mfma_all(fa[1], fb[1]);
            sched_interleave<NMF, NRD, 0, 0>();
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    read_all(smem, 0, fa[0], fb[0]);
    phase(std::integral_constant<int, 0>{}, 0, nkt);
    // SiLU(s * gate) while the producers issue the first Up tiles
    const float sc = DT == DT_E4M3 ? p.alpha : 1.0f;
#pragma unroll
    for (int tn = 0; tn < FH; ++tn)
#pragma unroll
        for (int tm = 0; tm < FM; ++tm)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[tn][tm][e] = silu(sc * acc[tn][tm][e]);
    __builtin_amdgcn_sched_barrier(0);
    phase(std::integral_constant<int, FH>{}, nkt, T);
}

// The epilogue of one finished output tile (every thread of the work-group).
template <int DT, bool TA, bool TB, int EPI, int BM, int BN, int BK, int S, int WM, int WN>
__device__ __forceinline__ void dma_epilogue(
    const Gemm16Params& p, typename DmaShape<DT, TA, TB, EPI, BM, BN, BK, S, WM, WN>::Acc& acc,
    char* smem, int m0, int n0, int wave, int lane) {
    using D = DmaShape<DT, TA, TB, EPI, BM, BN, BK, S, WM, WN>;
    constexpr int DT_OUT = D::DT_OUT, FM = D::FM, FN = D::FN, TM = D::TM, TN = D::TN;
    constexpr bool W12 = D::W12 || D::SEQ;
    const int wm = wave % WM, wn = wave / WM;
    if constexpr (EPI == EPI_SWIGLU || W12) {
        static_assert(BM * (BN + 8) <= D::LDS, "staged SwiGLU tile fits the LDS ring");
        epilogue_swiglu_lds<DT_OUT, FM, FN, BM, BN, 64 * WM * WN, W12, DT == DT_E4M3, D::SEQ>(
            p, acc, smem, m0, n0, wm * TM, W12 ? wn * (TN / 2) : wn * TN, lane);
    } else if constexpr (EPI == EPI_GEMM_EX) {
        static_assert(D::LDS >= D::NW * 32 * 36 * 4, "EX staging fits the LDS ring");
        // finished as whole row pieces from fp32 staging (measured: bf16 2048 x 4864 x
        // 896 + bias + GELU 40-44.5 -> 38-40 us against finishing one 32 x 32 fragment
        // per wave at a time)
        if constexpr (staged_wave_cols<BM, BN, FM, WN, D::LDS, 4 * BN>() > 0) {
            if ((reinterpret_cast<uintptr_t>(p.C) & 15) == 0 && (p.ldc & 7) == 0) {
                epilogue_gemm_ex_rows_lds<DT_OUT, FM, FN, BM, BN, WN, 64 * WM * WN, D::LDS>(
                    p, acc, smem, m0, n0, wm * TM, wn, lane);
                return;
            }
        }
        // C not 16-byte aligned or ldc not a multiple of 8: quads stored from the
        // fragment staging
        __syncthreads();
        epilogue_gemm_ex_lds<DT_OUT, FM, FN>(p, acc, smem, m0 + wm * TM, n0 + wn * TN, wave, lane);
    } else {
        if constexpr (EPI == EPI_PARTIAL && (BM / (32 * FM)) * 32 * (4 * BN + 16) <= D::LDS) {
            // split-K partials of a full tile leave as whole lines (measured: bf16 128 x
            // 4096 x 4096, 4 splits, 20.2-20.6 -> 19.4-19.6 us)
            if (m0 + BM <= p.M && n0 + BN <= p.N && (p.N & 3) == 0) {
                epilogue_partial_rows_lds<FM, FN, BM, BN, 64 * WM * WN>(p, acc, smem, m0, n0,
                                                                        wm * TM, wn * TN, lane);
                return;
            }
        }
        // beta != 0, and edge tiles at beta = 0: C_old read and C written as whole lines
        // (measured: bf16 4097 x 3001 x 2049 at beta = 0.3 94-98 -> 61-68 us, at beta = 0
        // 71-76 -> 57-66 us; bit-identical)
        if constexpr (EPI == EPI_GEMM && staged_wave_cols<BM, BN, FM, WN, D::LDS, 0>() > 0) {
            const bool edge = m0 + BM > p.M || n0 + BN > p.N;
            if ((p.beta != 0.0f || edge) && (reinterpret_cast<uintptr_t>(p.C) & 15) == 0 &&
                (p.ldc & 7) == 0) {
                epilogue_gemm_rows_beta_lds<DT_OUT, FM, FN, BM, BN, WN, 64 * WM * WN, D::LDS>(
                    p, acc, smem, m0, n0, wm * TM, wn, lane);
                return;
            }
        }
        // beta = 0, full tiles: staged row stores where work-groups run in more than one
        // round (measured: fp16 / bf16 8192^3 3-4 % and the e4m3 4096 x 22016 x 4096 GEMM
        // 9 % faster; a single round, 2048 x 9728 x 896, 2.5 % slower); rings too small
        // for a staged 32-row block keep the register epilogue.
        if constexpr (EPI == EPI_GEMM && (BM / (32 * FM)) * 32 * (2 * BN + 16) <= D::LDS) {
            if ((int64_t)gridDim.x * gridDim.y * gridDim.z > 256 && p.beta == 0.0f &&
                m0 + BM <= p.M && n0 + BN <= p.N &&
                (reinterpret_cast<uintptr_t>(p.C) & 15) == 0 && (p.ldc & 7) == 0) {
                epilogue_gemm_rows_lds<DT_OUT, FM, FN, BM, BN, 64 * WM * WN>(
                    p, acc, smem, m0, n0, wm * TM, wn * TN, lane);
                return;
            }
        }
        epilogue16<DT_OUT, EPI, FM, FN>(p, acc, m0, n0, BM, BN, m0 + wm * TM, n0 + wn * TN,
                                        lane);
    }
}

// L2 warm-up for a grid of fewer tiles than CUs (one partial round, short K): the
// work-groups past the tiles (blockIdx.x >= nblk) run this instead of a tile.  Each
// XCD's tiles (xcd_remap: block b runs on XCD b % 8, and the tiles of one XCD are
// consecutive in the grouped order) read one range of B's column tiles; that XCD's
// spare work-groups read the same range of every row of a row-major B, k rows in
// order, one 4-byte load per 64 bytes, so the lines are in that XCD's L2 before its
// tiles' DMA asks for them.  Loads only: the values are folded into a register that
// an empty asm statement consumes, nothing is stored, and no work-group waits for
// another, so the tiles' results do not depend on it (bit-identical either way).
// Measured on MI355X (bf16 SwiGLU, K = 896, fused width 9728, weights cold): M = 128
// 10.6 -> 8.4 us, M = 256 12.8 -> 11.5 us, M = 512 14.9 -> 14.3 us; where an XCD's
// share of B exceeds its 4 MB L2 the lines are evicted before use (e4m3 SwiGLU, K =
// 4096, fused width 22016: 13-29 % slower), so the host launches it only below that.
template <int BN, int ESZ>
__device__ __forceinline__ void warm_l2(const Gemm16Params& p, int nblk) {
    constexpr int NXCD = 8, DEPTH = 8;
    const int bid = blockIdx.x;
    if (nblk < NXCD) return;                       // xcd_remap is the identity there
    const int xcd = bid % NXCD;
    const int per = nblk / NXCD, rem = nblk % NXCD;
    const int tiles_here = per + (xcd < rem ? 1 : 0);
    const int first = xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per;
    const int j = bid / NXCD - tiles_here;                        // this warm-up block
    const int nwarm = (int)((gridDim.x - 1 - xcd) / NXCD) + 1 - tiles_here;   // of nwarm
    if (tiles_here == 0 || j < 0 || nwarm <= 0) return;
    int tm0, tn0, tm1, tn1;
    tile_coords(first, p.tiles_m, p.tiles_n, p.group_m, tm0, tn0);
    tile_coords(first + tiles_here - 1, p.tiles_m, p.tiles_n, p.group_m, tm1, tn1);
    const int per_group = p.group_m * p.tiles_n;
    int lo = min(tn0, tn1), hi = max(tn0, tn1);
    if (first / per_group != (first + tiles_here - 1) / per_group) lo = 0, hi = p.tiles_n - 1;
    // bytes [c0, c1) of each of the K rows: the XCD's column tiles, inside the row
    const int64_t c0 = (int64_t)lo * BN * ESZ;
    const int64_t c1 = min((int64_t)(hi + 1) * BN, (int64_t)p.N) * ESZ;
    if (c1 <= c0) return;
    const int64_t ld = p.ldb * ESZ;
    const char* B = reinterpret_cast<const char*>(p.B);
    const int nseg = (int)((c1 - c0 + 63) / 64);                  // 64-byte pieces per row
    const int64_t items = (int64_t)p.K * nseg;                    // row-major: k ascending
    const int nt = blockDim.x;
    uint32_t fold = 0;
    // chunks of nt pieces dealt round-robin to the nwarm blocks, DEPTH chunks in flight
    for (int64_t base = (int64_t)j * nt; base < items; base += (int64_t)nwarm * nt * DEPTH) {
        uint32_t v[DEPTH];
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            const int64_t w = base + (int64_t)d * nwarm * nt + threadIdx.x;
            v[d] = 0u;
            if (w < items) {
                const int64_t k = w / nseg, sgm = w - k * nseg;
                v[d] = *reinterpret_cast<const uint32_t*>(B + k * ld + c0 + sgm * 64);
            }
        }
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) fold ^= v[d];
    }
    asm volatile("" ::"v"(fold));                  // keeps the loads; nothing is stored
}

template <int DT, bool TA, bool TB, int EPI, int BM, int BN, int BK, int S, int WM, int WN>
__global__ void __launch_bounds__(64 * WM * WN, 1) gemm_dma_kernel(const Gemm16Params p_) {
    using D = DmaShape<DT, TA, TB, EPI, BM, BN, BK, S, WM, WN>;
    const Gemm16Params p = batch_item(p_);
    __shared__ __attribute__((aligned(1024))) char smem[D::LDS];

    const int nblk = p.tiles_m * p.tiles_n;
    if ((int)blockIdx.x >= nblk) {                 // an L2 warm-up block (no tile)
        if constexpr (!TB && !D::SEQ && !D::W12) warm_l2<BN, D::ESZ>(p, nblk);
        return;
    }
    const int lid = xcd_remap(blockIdx.x, nblk);
    int tmi, tni;
    tile_coords(lid, p.tiles_m, p.tiles_n, p.group_m, tmi, tni);
    const int m0 = tmi * BM, n0 = tni * BN;
    const int kbeg = blockIdx.y * p.k_per_split;
    const int kend = min(p.K, kbeg + p.k_per_split);
    const int klen = kend > kbeg ? kend - kbeg : 0;
    const int nkt = klen / BK, ktail = klen - nkt * BK;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;

    typename D::Acc acc;
#pragma unroll
    for (int i = 0; i < D::FN; ++i)
#pragma unroll
        for (int j = 0; j < D::FM; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
    if constexpr (D::SEQ)
        dma_mainloop_seq<DT, TA, TB, EPI, BM, BN, BK, S, WM, WN>(p, smem, m0, n0, nkt, acc, wave,
                                                                 lane);
    else
        dma_mainloop<DT, TA, TB, EPI, BM, BN, BK, S, WM, WN>(p, smem, m0, n0, kbeg, nkt, ktail,
                                                             acc, wave, lane);
    dma_epilogue<DT, TA, TB, EPI, BM, BN, BK, S, WM, WN>(p, acc, smem, m0, n0, wave, lane);
}

// The wave-specialised Kernel-1 (ws_mainloop_seq): WM x WN consumer waves and
// kWsProducers producer waves per work-group; all of them take part in the staged
// epilogue's barriers and stores, the producers with no accumulators to stage.
template <int DT, bool TA, bool TB, int EPI, int BM, int BN, int BK, int S, int WM, int WN>
__global__ void __launch_bounds__(64 * (WM * WN + kWsProducers), 1)
    gemm_ws_kernel(const Gemm16Params p_) {
    using D = DmaShape<DT, TA, TB, EPI, BM, BN, BK, S, WM, WN>;
    static_assert(D::SEQ, "the wave-specialised kernel runs Kernel-1 only");
    const Gemm16Params p = batch_item(p_);
    __shared__ __attribute__((aligned(1024))) char smem[D::LDS];

    const int nblk = p.tiles_m * p.tiles_n;
    const int lid = xcd_remap(blockIdx.x, nblk);
    int tmi, tni;
    tile_coords(lid, p.tiles_m, p.tiles_n, p.group_m, tmi, tni);
    const int m0 = tmi * BM, n0 = tni * BN;
    const int nkt = p.K / BK;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const bool consumer = wave < D::NW;

    typename D::Acc acc;
#pragma unroll
    for (int i = 0; i < D::FN; ++i)
#pragma unroll
        for (int j = 0; j < D::FM; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
    ws_mainloop_seq<DT, TA, TB, EPI, BM, BN, BK, S, WM, WN>(p, smem, m0, n0, nkt, acc, wave, lane);
    static_assert(BM * (BN + 8) <= D::LDS, "staged SwiGLU tile fits the LDS ring");
    const int wm = wave % WM, wn = (wave / WM) % WN;
    epilogue_swiglu_lds<D::DT_OUT, D::FM, D::FN, BM, BN, 64 * (WM * WN + kWsProducers), true,
                        DT == DT_E4M3, true>(p, acc, smem, m0, n0, wm * D::TM, wn * (D::TN / 2),
                                             lane, consumer);
}

}  // namespace sg
