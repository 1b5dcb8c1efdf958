// gla_split.hpp -- fp32 operands on the bf16 matrix cores.
//
// Every fp32 operand x is held as two bf16 values, hi = bf16(x) and
// lo = bf16(x - hi), so that x = hi + lo to about 2^-17 relative, and each
// fp32 product a b is taken as lo_a hi_b + hi_a lo_b + hi_a hi_b (three bf16
// matrix-core products into one fp32 accumulator; the dropped lo_a lo_b is
// below 2^-16 of the product).  Three bf16 products cost about a fifth of one
// fp32 matrix-core product on this device.  The FLAT page ("FLAT: Flash Linear
// Attention on TPUs", Pallas Kernels > Backward Kernels, the gate-gradient
// item) splits an fp32 input into two bf16 halves for the same reason, to keep
// fp32 accuracy on a bf16 matrix unit.  A split LDS tile is a hi plane
// followed, PLANE elements later, by a lo plane of the same layout.
#pragma once
#include "gla_common.hpp"
#include "gla_tile.hpp"

namespace gla {

struct SFrag {
    bf16x8 hi, lo;
};

__device__ __forceinline__ f32x4 mma3(const SFrag& a, const SFrag& b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b.hi, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.lo, c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.hi, c, 0, 0, 0);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Two fp32 values split at once: hi = bf16(x) rounded to nearest even, lo =
// bf16(x - hi); each pair packed in one 32-bit word (element 0 in the low half),
// which is what the packed conversion instruction produces.
struct Split2 {
    uint32_t hi, lo;
};
__device__ __forceinline__ Split2 split2(float x0, float x1) {
    const f32x2 x = {x0, x1};
    const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
    const f32x2 r = {x0 - __uint_as_float(h << 16), x1 - __uint_as_float(h & 0xffff0000u)};
    return Split2{h, __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2))};
}

// four consecutive fp32 values to a split tile: 8 bytes to each plane
__device__ __forceinline__ void split4_store(float x0, float x1, float x2, float x3, bf16* hi, bf16* lo) {
    const Split2 a = split2(x0, x1), b = split2(x2, x3);
    *reinterpret_cast<u32x2*>(hi) = u32x2{a.hi, b.hi};
    *reinterpret_cast<u32x2*>(lo) = u32x2{a.lo, b.lo};
}

// eight fp32 values (a: elements 0..3, b: 4..7) as a split operand fragment
__device__ __forceinline__ SFrag split8(const f32x4& a, const f32x4& b) {
    const Split2 s0 = split2(a[0], a[1]), s1 = split2(a[2], a[3]);
    const Split2 s2 = split2(b[0], b[1]), s3 = split2(b[2], b[3]);
    return SFrag{__builtin_bit_cast(bf16x8, u32x4{s0.hi, s1.hi, s2.hi, s3.hi}),
                 __builtin_bit_cast(bf16x8, u32x4{s0.lo, s1.lo, s2.lo, s3.lo})};
}

// operand fragments of a split tile (hi plane at base, lo plane PLANE elements later)
// (l: the lane index, or opaque_lane() inside a loop)
template <int P, int PLANE>
__device__ __forceinline__ SFrag sld(const bf16* base, int i0, int k0, int l = lane_id()) {
    return SFrag{frag_ld<bf16, P, 1>(base, i0, k0, l), frag_ld<bf16, P, 1>(base + PLANE, i0, k0, l)};
}
template <int P, int PLANE>
__device__ __forceinline__ SFrag scol(const bf16* base, int i0, int k0, int l = lane_id()) {
    return SFrag{frag_col<bf16, P, false>(base, i0, k0, 0, l), frag_col<bf16, P, false>(base + PLANE, i0, k0, 0, l)};
}

// eight consecutive fp32 values from global memory as a split fragment; with
// q given, also accumulates their dot product with q's eight values
__device__ __forceinline__ SFrag split_ld8(const float* p, float& dot_with, const float* q) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
    if (q) {
        const f32x4 c = *reinterpret_cast<const f32x4*>(q);
        const f32x4 d = *reinterpret_cast<const f32x4*>(q + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) dot_with += a[e] * c[e] + b[e] * d[e];
    }
    return split8(a, b);
}

// fp32 tile rows from registers to a split LDS tile (8-byte stores per plane)
template <int D, int NTH = NT>
__device__ __forceinline__ void store_rows_split(const TileRegs<float, D, NTH>& t, bf16* dst, int P, int PLANE,
                                                 int tid = (int)threadIdx.x) {
    using TR = TileRegs<float, D, NTH>;
#pragma unroll
    for (int i = 0; i < TR::NVEC; ++i) {
        const int idx = tid + i * NTH;
        if (idx < TR::NV_TOT) {
            const int row = idx / TR::VPR, cv = (idx % TR::VPR) * 4;
            const f32x4 f = __builtin_bit_cast(f32x4, t.get(i));
            split4_store(f[0], f[1], f[2], f[3], dst + row * P + cv, dst + PLANE + row * P + cv);
        }
    }
}

// row fragments in ctile k order (matching a C-layout accumulator operand)
template <int P, int PLANE>
__device__ __forceinline__ SFrag sld_ctile(const bf16* base, int i0, int k0) {
    return SFrag{frag_ld_ctile<bf16, P, 1>(base, i0, k0, 0), frag_ld_ctile<bf16, P, 1>(base + PLANE, i0, k0, 0)};
}

// column fragments in ctile k order (matching a C-layout accumulator operand)
template <int P, int PLANE>
__device__ __forceinline__ SFrag scol_ctile(const bf16* base, int i0, int k0) {
    return SFrag{frag_col<bf16, P, true>(base, i0, k0), frag_col<bf16, P, true>(base + PLANE, i0, k0)};
}

// split operand from two fp32 C-layout accumulator tiles (k rows 0..15 and
// 16..31 of a 32-wide step, ctile order)
__device__ __forceinline__ SFrag split_acc(const f32x4& lo, const f32x4& hi) { return split8(lo, hi); }

// acc += sum over steps i < n of A_i B_i (three-product split form); ld(i, A, B)
// reads step i's operands.  The reads of step i + 1 are issued before step
// i's products (scheduling barriers keep the compiler from merging the two),
// so LDS latency hides behind the matrix cores.  NMAX bounds n at compile time.
template <int NMAX, typename LD>
__device__ __forceinline__ f32x4 mma3_chain(f32x4 acc, int n, LD&& ld) {
    SFrag a0, b0;
    if (n > 0) ld(0, a0, b0);
#pragma unroll
    for (int i = 0; i < NMAX; ++i) {
        if (i < n) {
            SFrag a1, b1;
            if (i + 1 < n) ld(i + 1, a1, b1);
            __builtin_amdgcn_sched_barrier(0);
            acc = mma3(a0, b0, acc);
            __builtin_amdgcn_sched_barrier(0);
            a0 = a1;
            b0 = b1;
        }
    }
    return acc;
}

}  // namespace gla
