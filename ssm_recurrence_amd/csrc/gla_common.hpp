// gla_common.hpp -- device helpers shared by the gfx950 kernels: matrix-core
// fragments, LDS fragment loaders, storage conversions and the chunk prologue
// (document flags and the chunk-local cumulative log gate).
//
// Matrix-core lane layouts (CDNA4, wave64), checked on the hardware:
//   v_mfma_f32_16x16x32_bf16: A lane l holds A[l%16][8*(l/16) + e], e < 8;
//                             B lane l holds B[8*(l/16) + e][l%16];
//   v_mfma_f32_16x16x4_f32  : A lane l holds A[l%16][l/16]; B lane l holds B[l/16][l%16];
//   both accumulate into C lane l = C[4*(l/16) + e][l%16], e < 4 ("C layout").
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gla {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int C = 64;        // tokens per chunk
constexpr int NT = 256;      // threads per workgroup (4 waves)
constexpr int WAVE = 64;

// ------------------------------------------------------------------ conversions
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
// float -> bf16, round to nearest even (the compiler's conversion does RNE)
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// Four consecutive elements (8 bytes of bf16, 16 of fp32) as one LDS access.
template <typename T> struct Vec4;
template <> struct Vec4<bf16> {
    bf16x4 v;
    static __device__ __forceinline__ Vec4 load(const bf16* p) { Vec4 r; r.v = *reinterpret_cast<const bf16x4*>(p); return r; }
    __device__ __forceinline__ void store(bf16* p) const { *reinterpret_cast<bf16x4*>(p) = v; }
    __device__ __forceinline__ float get(int e) const { return (float)v[e]; }
    __device__ __forceinline__ void set(int e, float x) { v[e] = (bf16)x; }
};
template <> struct Vec4<float> {
    f32x4 v;
    static __device__ __forceinline__ Vec4 load(const float* p) { Vec4 r; r.v = *reinterpret_cast<const f32x4*>(p); return r; }
    __device__ __forceinline__ void store(float* p) const { *reinterpret_cast<f32x4*>(p) = v; }
    __device__ __forceinline__ float get(int e) const { return v[e]; }
    __device__ __forceinline__ void set(int e, float x) { v[e] = x; }
};

// ------------------------------------------------------------------ matrix-core traits
template <typename T> struct Mma;
template <> struct Mma<bf16> {
    static constexpr int KPL = 8;     // k values per lane per step
    static constexpr int KSTEP = 32;  // k per instruction
    typedef bf16x8 frag;
    static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ void set(frag& f, int e, float x) { f[e] = (bf16)x; }
    static __device__ __forceinline__ frag zero() { frag f; for (int e = 0; e < 8; ++e) f[e] = (bf16)0.0f; return f; }
};
template <> struct Mma<float> {
    static constexpr int KPL = 1;
    static constexpr int KSTEP = 4;
    typedef float frag;
    static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ void set(frag& f, int, float x) { f = x; }
    static __device__ __forceinline__ frag zero() { return 0.0f; }
};

__device__ __forceinline__ f32x4 zero4() { f32x4 z = {0.f, 0.f, 0.f, 0.f}; return z; }

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
// threadIdx.x and the lane index as values the compiler cannot see through:
// addresses derived from them are formed where they are used, not hoisted out
// of a loop and held in registers across it
__device__ __forceinline__ int opaque_tid() {
    int t = (int)threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
}
__device__ __forceinline__ int opaque_lane() {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

// Block id -> logical id so that consecutive logical ids (the slices of one
// head) land on the same XCD: the hardware deals consecutive block ids round
// robin over the 8 XCDs.
__device__ __forceinline__ int64_t xcd_remap(int64_t x, int64_t nblocks) {
    if (nblocks % 8 != 0) return x;
    return (x % 8) * (nblocks / 8) + x / 8;
}
__device__ __forceinline__ int64_t xcd_logical_block(int64_t nblocks) { return xcd_remap(blockIdx.x, nblocks); }

// Operand fragment from LDS for one matrix-core step ("natural" k order):
// lane (i = l%16, j = l/16) receives X(i0 + i, k0 + j*KPL + e), e < KPL, where
// X(i, k) = base[i*SI + k*SK].  Serves A (i = row m) and B (i = column n).
template <typename T, int SI, int SK>
__device__ __forceinline__ typename Mma<T>::frag frag_ld(const T* base, int i0, int k0, int l = lane_id()) {
    const int i = i0 + (l & 15);
    const int k = k0 + (l >> 4) * Mma<T>::KPL;
    typename Mma<T>::frag f;
    if constexpr (SK == 1 && Mma<T>::KPL == 8) {
        f = *reinterpret_cast<const bf16x8*>(base + i * SI + k);
    } else if constexpr (Mma<T>::KPL == 1) {
        f = base[i * SI + k * SK];
    } else {
#pragma unroll
        for (int e = 0; e < Mma<T>::KPL; ++e) f[e] = base[i * SI + (k + e) * SK];
    }
    return f;
}

// Operand fragment whose k order matches a C-layout accumulator used as the
// other operand ("ctile" order).  bf16: a 32-wide k step takes rows of two
// 16-row C tiles, lane group j holding k = 4j+e (e<4) and 16+4j+(e-4) (e>=4).
// f32: step `sub` (0..3) of a 16-row C tile, lane group j holding k = 4j+sub.
template <typename T, int SI, int SK>
__device__ __forceinline__ typename Mma<T>::frag frag_ld_ctile(const T* base, int i0, int k0,
                                                               int sub) {
    const int l = lane_id();
    const int i = i0 + (l & 15);
    const int j = l >> 4;
    typename Mma<T>::frag f;
    if constexpr (Mma<T>::KPL == 1) {
        f = base[i * SI + (k0 + 4 * j + sub) * SK];
    } else {
        (void)sub;
        if constexpr (SK == 1) {
            bf16x4 lo = *reinterpret_cast<const bf16x4*>(base + i * SI + k0 + 4 * j);
            bf16x4 hi = *reinterpret_cast<const bf16x4*>(base + i * SI + k0 + 16 + 4 * j);
            for (int e = 0; e < 4; ++e) { f[e] = lo[e]; f[4 + e] = hi[e]; }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                f[e] = base[i * SI + (k0 + 4 * j + e) * SK];
                f[4 + e] = base[i * SI + (k0 + 16 + 4 * j + e) * SK];
            }
        }
    }
    return f;
}

// B (or A) fragment built from fp32 C-layout accumulators: tiles lo (k rows
// 0..15 of the step) and hi (16..31) for bf16; tile lo, step `sub` for f32.
template <typename T>
__device__ __forceinline__ typename Mma<T>::frag frag_from_acc(const f32x4& lo, const f32x4& hi,
                                                               int sub) {
    typename Mma<T>::frag f;
    if constexpr (Mma<T>::KPL == 1) {
        (void)hi;
        f = lo[sub];
    } else {
        (void)sub;
        for (int e = 0; e < 4; ++e) { f[e] = (bf16)lo[e]; f[4 + e] = (bf16)hi[e]; }
    }
    return f;
}

// Operand fragment "lane i, k packed" from a natural row-major tile X[k][i]
// (pitch P elements), i.e. a column read, without a transposed copy in LDS.
// bf16 uses the gfx950 transposing LDS read ds_read_b64_tr_b16: within each
// group of 16 lanes, lane i receives element e from source lane 4e + i/4,
// position i%4 (checked on the hardware).  So source lane s of group j points
// at row k(j, s/4) and columns i0 + 4*(s%4); two reads give 8 k values.
// Natural k order: k(j, e) = k0 + 8j + e.  ctile order (matching a C-layout
// accumulator used as the other operand): k0 + 4j + e and k0 + 16 + 4j + e.
// fp32: one element, k = k0 + j (natural) or k0 + 4j + sub (ctile).
typedef short v4i16_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ v4i16_t lds_read_tr16(const bf16* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t*)(p));
}
template <typename T, int P, bool CTILE>
__device__ __forceinline__ typename Mma<T>::frag frag_col(const T* base, int i0, int k0, int sub = 0,
                                                          int l = lane_id()) {
    const int j = l >> 4;
    typename Mma<T>::frag f;
    if constexpr (Mma<T>::KPL == 1) {
        const int k = CTILE ? k0 + 4 * j + sub : k0 + j;
        f = base[k * P + i0 + (l & 15)];
    } else {
        (void)sub;
        const int s = l & 15;
        const int col = i0 + 4 * (s & 3);
        const int r0 = CTILE ? k0 + 4 * j + (s >> 2) : k0 + 8 * j + (s >> 2);
        const int r1 = CTILE ? r0 + 16 : r0 + 4;
        // whole-vector casts: extracting the lanes of the returned short vector
        // one by one is mis-lowered by this compiler (it keeps element 0 only)
        const bf16x4 a = __builtin_bit_cast(bf16x4, lds_read_tr16(base + r0 * P + col));
        const bf16x4 b = __builtin_bit_cast(bf16x4, lds_read_tr16(base + r1 * P + col));
        f = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    return f;
}

// ------------------------------------------------------------------ wave primitives
// Data-parallel moves within rows of 16 lanes (checked on the hardware):
// row_shl:n (0x100 + n) reads lane i + n of the row, 0 past its end;
// row_ror:n (0x120 + n) reads lane (i - n) mod 16 of the row.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
// lane i of each row of 16: sum of lanes i .. 15 of its row
__device__ __forceinline__ float row_suffix16(float y) {
    y += dpp_f<0x101>(y);
    y += dpp_f<0x102>(y);
    y += dpp_f<0x104>(y);
    y += dpp_f<0x108>(y);
    return y;
}
// every lane: sum of its row of 16
__device__ __forceinline__ float row_sum16(float y) {
    y += dpp_f<0x121>(y);
    y += dpp_f<0x122>(y);
    y += dpp_f<0x124>(y);
    y += dpp_f<0x128>(y);
    return y;
}
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// sum_e a[e] * b[e] over a fragment, fp32 accumulation
template <typename F>
__device__ __forceinline__ float frag_dot(const F& a, const F& b, float acc) {
    if constexpr (sizeof(F) == sizeof(float)) {
        return acc + a * b;
    } else {
#pragma unroll
        for (int e = 0; e < 8; e += 2)
            acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{a[e], a[e + 1]}, bf16x2{b[e], b[e + 1]}, acc, false);
        return acc;
    }
}
// Tiles of a 64 x 64 causal score matrix in 16 x 16 blocks: ti = 0 .. 9 are the
// blocks with rt >= st (row-major), 10 and 11 the two zero blocks above the
// diagonal that a 32-wide k step also reads.  Packed as 2-bit fields, so that the
// compiler knows rt and st lie in [0, 3] and keeps the index arithmetic in 32
// bits (a 64-bit multiply-add here reads an undefined high half, and a load in
// flight to that register would then be waited for).
__device__ __forceinline__ int score_tile_rt(int ti) { return (0x8ffa94 >> (2 * ti)) & 3; }
__device__ __forceinline__ int score_tile_st(int ti) { return (0xde4910 >> (2 * ti)) & 3; }

__device__ __forceinline__ float wave_incl_scan(float x) {
    const int l = lane_id();
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        float y = __shfl_up(x, d, 64);
        if (l >= d) x += y;
    }
    return x;
}
__device__ __forceinline__ int wave_incl_scan_i(int x) {
    const int l = lane_id();
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        int y = __shfl_up(x, d, 64);
        if (l >= d) x += y;
    }
    return x;
}

// ------------------------------------------------------------------ chunk prologue
// Per chunk: document index of each position (count of resets up to and
// including it), the first and last reset positions, and validity.
struct ChunkDocs {
    int doc[C];     // inclusive prefix count of resets inside the chunk
    int first_reset;  // C if none
    int last_reset;   // -1 if none
    int nvalid;       // positions < T
};

// Fill `cd` (LDS) for chunk starting at t0 of row b.  Wave 0 does the work;
// caller synchronises afterwards.
__device__ __forceinline__ void chunk_docs(ChunkDocs* cd, const int32_t* seg, int64_t b, int64_t T,
                                           int64_t t0) {
    if (wave_id() != 0) return;
    const int r = lane_id();
    const int64_t t = t0 + r;
    int reset = 0;
    if (seg != nullptr && t < T && t > 0) reset = seg[b * T + t] != seg[b * T + t - 1];
    const int cnt = wave_incl_scan_i(reset);
    cd->doc[r] = cnt;
    // first / last reset via ballot
    const uint64_t m = __ballot(reset);
    if (r == 0) {
        cd->first_reset = m ? __builtin_ctzll(m) : C;
        cd->last_reset = m ? 63 - __builtin_clzll(m) : -1;
        const int64_t nv = T - t0;
        cd->nvalid = nv < C ? (int)nv : C;
    }
}

}  // namespace gla
