// lf_device.h -- device helpers shared by the gfx950 kernels of the forward
// (lf_fwd_kernels.hip) and of the MFMA backward (lf_bwd_mfma.hip): vector
// types, bf16 packing and splitting, the 32x32x16 bf16 MFMA, transposing LDS
// reads, raw buffer resources and loads into LDS, the score masks and the
// two-halves reductions.  Internal to liblfattn.so.
#ifndef LF_DEVICE_H
#define LF_DEVICE_H

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lfk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

constexpr int KBLK = 32;                  // keys per block (one S^T tile)
constexpr int kNotInClass = -(1 << 30);   // class index of a position outside the tile's residue class

constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kRawBufferWord3 = 0x00020000;   // raw buffer, 32-bit data format, no swizzle
constexpr uint32_t kPastEnd = 0xFFFFFF00u;     // buffer offset past any resource's end (reads zero)
constexpr int kCoherent = 16;                  // buffer cache policy sc1: coherent across the dies' L2s
constexpr float kLn2 = 0.69314718055994531f;

// log2(e) / sqrt(d): scores are taken to base 2 with the 1/sqrt(d) scale
template <int D> struct ScaleLog2;
template <> struct ScaleLog2<32> { static constexpr float v = 0.25503486164919736f; };
template <> struct ScaleLog2<64> { static constexpr float v = 0.18033688011112042f; };
template <> struct ScaleLog2<128> { static constexpr float v = 0.12751743082459868f; };

struct Raw32 { u32x4 a, b; };

// two floats -> two bf16 (round to nearest even) in one dword; one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}
__device__ __forceinline__ float bf_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// split 8 floats into NP bf16 parts (part 0 = RNE(x), part i = RNE of what
// the parts before it leave; every remainder is exact in fp32).  Whole
// vectors are bit-cast: bit-casting single elements of an ext_vector
// miscompiles with this clang (every element reads as element 0).
template <int NP>
__device__ __forceinline__ void split8(const Raw32& r, u32x4* parts) {
    const f32x4 fa = __builtin_bit_cast(f32x4, r.a);
    const f32x4 fb = __builtin_bit_cast(f32x4, r.b);
    float f[8] = {fa[0], fa[1], fa[2], fa[3], fb[0], fb[1], fb[2], fb[3]};
#pragma unroll
    for (int p = 0; p < NP; p++) {
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint32_t hw = pack_bf16(f[2 * i], f[2 * i + 1]);
            w[i] = hw;
            f[2 * i] -= bf_lo(hw);
            f[2 * i + 1] -= bf_hi(hw);
        }
        parts[p] = w;
    }
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ i16x4 ds_tr16(const char* lds_ptr) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(lds_ptr));
}

__device__ __forceinline__ bf16x8 cat_tr(i16x4 a, i16x4 b) {
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// raw buffer over [base, base + bytes): accesses at offsets >= bytes read zero
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRawBufferWord3);
}

// 16 bytes per lane from rsrc at voff + soff into LDS at dst + 16 * lane
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rs, char* dst, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, LDS_PTR(dst), 16, voff, soff, 0, 0);
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Barrier after which every wave's loads into LDS have landed.  A plain
// __syncthreads() waits only for LDS instructions (lgkmcnt), not for
// buffer_load ... lds, which counts on vmcnt: each wave first waits for its
// own (s_waitcnt vmcnt(0): gfx9 encoding, expcnt and lgkmcnt left open).
__device__ __forceinline__ void barrier_lds_loads() {
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
}

// reductions over the two 32-lane halves (lanes l and l^32 hold the two key
// halves of a query): one v_permlane32_swap, no LDS round trip
__device__ __forceinline__ float halves_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                    __builtin_bit_cast(uint32_t, x), false, false);
    const f32x2 f = __builtin_bit_cast(f32x2, r);
    return __builtin_elementwise_maximum(f[0], f[1]);
}
__device__ __forceinline__ float halves_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                    __builtin_bit_cast(uint32_t, x), false, false);
    const f32x2 f = __builtin_bit_cast(f32x2, r);
    return f[0] + f[1];
}

// Masking.  Lane l holds the scores of keys 8*(i>>2) + 4*(l/32) + (i&3) of
// the block in accumulator element i.  Bit t of a block's `bad` word is set
// when key row t is not a real key (past the sequence, class or split end,
// padded, or an unused global slot).

// keep bits of this lane's 16 elements from a 32-bit row word
__device__ __forceinline__ uint32_t lane_bits(uint32_t rows, int lg) {
    const uint32_t sh = rows >> (4 * lg);
    return (sh & 0xfu) | ((sh >> 4) & 0xf0u) | ((sh >> 8) & 0xf00u) | ((sh >> 12) & 0xf000u);
}

// band block: keep kc in [lo, lo + width], where kc is the element's key row
// minus 4*lg and lo = m - r - key0 - 4*lg (the window reaches r keys back
// and width - r forward)
__device__ __forceinline__ void mask_window(f32x16& s, int lo, int width) {
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const int kc = 8 * (i >> 2) + (i & 3);
        s[i] = (uint32_t)(kc - lo) <= (uint32_t)width ? s[i] : kNegInf;
    }
}

// keep the elements whose bit is set in keep16
__device__ __forceinline__ void mask_bits(f32x16& s, uint32_t keep16) {
#pragma unroll
    for (int i = 0; i < 16; i++) s[i] = ((keep16 >> i) & 1u) ? s[i] : kNegInf;
}

// random key block: drop the keys inside this query's window (the band
// counts those): kc in [lo, lo + width] as in mask_window
__device__ __forceinline__ void mask_window_out(f32x16& s, int lo, int width) {
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const int kc = 8 * (i >> 2) + (i & 3);
        s[i] = (uint32_t)(kc - lo) <= (uint32_t)width ? kNegInf : s[i];
    }
}

// global block (32 slots of global positions; gcls: their class indices in
// the tile's class, kNotInClass for the others): drop the slots set in bad
// (unused or padded) and the slots whose class index g has g - m in
// [-r, width - r], pairs the band already counts.  The forward and dq pass
// the window's reach back as r (slot = key, m = query); dk, dv pass the
// reach forward (slot = query, m = key).
__device__ __forceinline__ void mask_global(f32x16& s, uint32_t bad, const int* gcls, int m, int r, int width,
                                            int lg) {
    const uint32_t badl = lane_bits(bad, lg);
#pragma unroll
    for (int q4 = 0; q4 < 4; q4++) {
        const u32x4 g4 = *(const u32x4*)(gcls + 8 * q4 + 4 * lg);
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const int i = 4 * q4 + e;
            const int dk = (int)g4[e] - m;
            const bool ok = ((badl >> i) & 1u) == 0u && (uint32_t)(dk + r) > (uint32_t)width;
            s[i] = ok ? s[i] : kNegInf;
        }
    }
}

}  // namespace lfk

#endif
