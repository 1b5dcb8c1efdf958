// gla_tile.hpp -- register-staged chunk tiles for software-pipelined passes:
// the next chunk's rows are loaded from HBM into registers while the current
// chunk computes, then written to LDS (natural or transposed layout).
#pragma once
#include "gla_common.hpp"

namespace gla {

typedef __attribute__((__vector_size__(16))) int i32x4;

// Row pitch (elements) of [rows][d] tiles in LDS: rows stay 16-byte aligned
// and consecutive rows shift by 16 bytes across the banks.
template <typename T> struct Pitch16 {
    static constexpr int pad = 16 / (int)sizeof(T);
    static constexpr int of(int d) { return d + pad; }
};

template <typename T, int D, int NTH = NT>
struct TileRegs {
    static constexpr int VE = 16 / (int)sizeof(T);   // elements per 16-byte vector
    static constexpr int VPR = D / VE;                // vectors per row
    static constexpr int NV_TOT = C * VPR;            // vectors per tile
    static constexpr int NVEC = (NV_TOT + NTH - 1) / NTH;
    i32x4 r[NVEC];
    uint32_t okm;  // bit i: vector i lies in a row before nvalid (else it reads as zero)

    // rows t0.. of a row-major tensor (row stride rs elements); rows >= nvalid read as
    // zero.  Every lane loads (a row past the end reads row 0 instead) and the
    // zeroing is applied where the registers are used (get): a select on loaded
    // registers here would make the compiler wait for every load in flight.
    // (tid: threadIdx.x, or opaque_tid() in a persistent loop)
    __device__ __forceinline__ void load(const T* src, int64_t rs, int nvalid, int tid = (int)threadIdx.x) {
        okm = 0;
#pragma unroll
        for (int i = 0; i < NVEC; ++i) {
            const int idx = tid + i * NTH;
            const int row = idx / VPR, cv = (idx % VPR) * VE;
            const bool ok = idx < NV_TOT && row < nvalid;
            r[i] = *reinterpret_cast<const i32x4*>(src + (ok ? (int64_t)row * rs + cv : (int64_t)0));
            okm |= (uint32_t)ok << i;
        }
    }
    // vector i as loaded, or zero past the end
    __device__ __forceinline__ i32x4 get(int i) const {
        const i32x4 z = {0, 0, 0, 0};
        return ((okm >> i) & 1u) ? r[i] : z;
    }
    // dst[row][col] with pitch P
    __device__ __forceinline__ void store_rows(T* dst, int P) const {
#pragma unroll
        for (int i = 0; i < NVEC; ++i) {
            const int idx = threadIdx.x + i * NTH;
            if (idx < NV_TOT) {
                const int row = idx / VPR, cv = (idx % VPR) * VE;
                *reinterpret_cast<i32x4*>(dst + row * P + cv) = get(i);
            }
        }
    }
    // multiply every element of row `row` by scale[row]
    __device__ __forceinline__ void scale_rows(const float* scale) {
#pragma unroll
        for (int i = 0; i < NVEC; ++i) {
            const int idx = threadIdx.x + i * NTH;
            if (idx < NV_TOT) {
                const float f = scale[idx / VPR];
                r[i] = get(i);
                okm |= 1u << i;
                T* e = reinterpret_cast<T*>(&r[i]);
#pragma unroll
                for (int k = 0; k < VE; ++k) e[k] = (T)((float)e[k] * f);
            }
        }
    }
    // dst[row][col] with pitch P, as 8-byte stores (rows need only 8-byte alignment)
    __device__ __forceinline__ void store_rows_b64(T* dst, int P) const {
#pragma unroll
        for (int i = 0; i < NVEC; ++i) {
            const int idx = threadIdx.x + i * NTH;
            if (idx < NV_TOT) {
                const int row = idx / VPR, cv = (idx % VPR) * VE;
                typedef __attribute__((__vector_size__(8))) int i32x2;
                const i32x4 x = get(i);
                const i32x2 lo = {x[0], x[1]}, hi = {x[2], x[3]};
                *reinterpret_cast<i32x2*>(dst + row * P + cv) = lo;
                *reinterpret_cast<i32x2*>(dst + row * P + cv + VE / 2) = hi;
            }
        }
    }
    // dst[col][row] with pitch P (transpose)
    __device__ __forceinline__ void store_cols(T* dst, int P) const {
#pragma unroll
        for (int i = 0; i < NVEC; ++i) {
            const int idx = threadIdx.x + i * NTH;
            if (idx < NV_TOT) {
                const int row = idx / VPR, cv = (idx % VPR) * VE;
                const i32x4 x = get(i);
                const T* e = reinterpret_cast<const T*>(&x);
#pragma unroll
                for (int k = 0; k < VE; ++k) dst[(cv + k) * P + row] = e[k];
            }
        }
    }
};

// Per-lane values for one chunk: the scalar gate of row `lane` and the segment
// ids of rows lane - 1 and lane.  They are kept as loaded (raw gate bits,
// unconverted ids) and turned into values only when the chunk is processed
// (g(), reset()): any arithmetic on a loaded value makes the compiler wait for
// every load still in flight, which would make the loads issued ahead with
// this chunk's tiles synchronous.
struct RowRegs {
    uint32_t graw;   // gate bits: bf16 in the low half, or fp32
    int gkind;       // 0: no gate (vector gate, or row past the end), 2: bf16, 4: fp32
    int seg_prev, seg_cur;
    int segok;       // 1 when seg_prev, seg_cur are the ids of rows lane - 1 and lane
    template <typename T>
    __device__ __forceinline__ void load(const T* gcol, int64_t rs_g, const int32_t* seg, int64_t b,
                                         int64_t T_, int64_t t0, int nvalid, bool scalar_gate) {
        const int r = lane_id();
        const int64_t t = t0 + r;
        const bool ok = r < nvalid;
        graw = 0;
        gkind = 0;
        if (scalar_gate) {
            const T x = gcol[(int64_t)(ok ? r : 0) * rs_g];  // an existing row even past the end
            if constexpr (sizeof(T) == 2) graw = (uint32_t)__builtin_bit_cast(uint16_t, x);
            else graw = __builtin_bit_cast(uint32_t, x);
            gkind = ok ? (int)sizeof(T) : 0;
        }
        seg_prev = seg_cur = 0;
        segok = 0;
        if (seg != nullptr && T_ > 1) {
            const int64_t tc = ok && t > 0 ? t : 1;  // an existing pair of rows
            seg_prev = seg[b * T_ + tc - 1];
            seg_cur = seg[b * T_ + tc];
            segok = ok && t > 0;
        }
    }
    // the scalar log gate of row `lane` (0 past the end)
    __device__ __forceinline__ float g() const {
        return gkind == 0 ? 0.f : (gkind == 2 ? __uint_as_float(graw << 16) : __uint_as_float(graw));
    }
    // 1 if row `lane` starts a new document (its id differs from the previous row's)
    __device__ __forceinline__ int reset() const { return segok && seg_cur != seg_prev; }
};

// Document structure of a chunk from the per-row reset flags (wave 0 only).
__device__ __forceinline__ void docs_from_flags(ChunkDocs* cd, int reset, int nvalid) {
    const int r = lane_id();
    const int cnt = wave_incl_scan_i(reset);
    cd->doc[r] = cnt;
    const uint64_t m = __ballot(reset);
    if (r == 0) {
        cd->first_reset = m ? __builtin_ctzll(m) : C;
        cd->last_reset = m ? 63 - __builtin_clzll(m) : -1;
        cd->nvalid = nvalid;
    }
}

// Raw buffer resource over `bytes` bytes from a workgroup-uniform base.  Buffer
// loads and stores take the per-lane part of the address in one register and a
// per-element constant in the instruction (or a scalar register), where global
// accesses at many constant offsets would each hold a 64-bit address.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
__device__ __forceinline__ f32x4 buf_ld4(__amdgpu_buffer_rsrc_t rs, int voff, int soff) {
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    return __builtin_bit_cast(f32x4, (u32x4_t)__builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, 0));
}
__device__ __forceinline__ float buf_ld1(__amdgpu_buffer_rsrc_t rs, int voff, int soff) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, voff, soff, 0));
}

// The 128 x 128 state a workgroup of eight waves holds in accumulators (wave w,
// lane (i, j): S[16 ct + 4 j + e][16 w + i] in S[ct][e]) stored row-major to dst
// ([128][128], element type T, dst uniform over the workgroup).  Buffer stores
// keep the per-lane part of the address in one register and the per-element
// row offset in the instruction, so the 32 stores need no address registers
// of their own (global stores would hold 32 loop-invariant 64-bit addresses).
template <typename T>
__device__ __forceinline__ void store_state_128(T* dst, const f32x4 (&S)[8]) {
    constexpr int B = (int)sizeof(T);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(dst, 0, 128 * 128 * B, 0x00020000);
    // the lane index is read afresh (not hoisted out of a caller's loop, where a
    // precomputed offset would hold a register for the whole loop)
    const int l = opaque_lane();
    const int w = __builtin_amdgcn_readfirstlane(wave_id());
    const int vo = ((4 * (l >> 4)) * 128 + (l & 15)) * B + 16 * B * w;
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int so = (16 * ct + e) * 128 * B;
            if constexpr (B == 4)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(S[ct][e]), rs, vo, so, 0);
            else
                __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (bf16)S[ct][e]), rs, vo, so,
                                                      0);
        }
}

// The state entering piece `piece` of head bh (= b H + h), at the accumulator
// positions of wave w: S[ct][e] = S[16 ct + 4 j4 + e][16 w + i16] of a 128 x 128
// state.  Without a split, h0 (or zero).  With one, the combine's S_in, or (when
// a.entry_from_summaries) the combine's chain S <- D_q S + L_q from h0 over the
// pieces before this one, formed here with the same operations in the same order.
template <typename Args>
__device__ __forceinline__ void load_entry_state_128(const Args& a, int64_t bh, int64_t piece, int w, int j4, int i16,
                                                     f32x4 (&S)[8]) {
    constexpr int DK = 128, DV = 128;
    const int64_t P = a.P;
    const int n = 16 * w + i16;
    if (P > 1 && !a.entry_from_summaries) {
#pragma unroll
        for (int ct = 0; ct < DK / 16; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) S[ct][e] = a.S_in[((bh * P + piece) * DK + 16 * ct + 4 * j4 + e) * DV + n];
        return;
    }
#pragma unroll
    for (int ct = 0; ct < DK / 16; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) S[ct][e] = a.h0 ? a.h0[(bh * DK + 16 * ct + 4 * j4 + e) * DV + n] : 0.f;
    if (P == 1) return;
#pragma unroll 1
    for (int64_t q = 0; q < piece; ++q) {
        const float* L = a.L_out[0] + (bh * P + q) * DK * DV;
        const float* D = a.D_out + (bh * P + q) * DK;
#pragma unroll
        for (int ct = 0; ct < DK / 16; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int c = 16 * ct + 4 * j4 + e;
                S[ct][e] = D[c] * S[ct][e] + L[c * DV + n];
            }
    }
}

// Operands of the triangular matrix of ones L^T (L[r][u] = [u <= r]) for the
// chunk-local prefix below, one per (row tile rt, k step): element e of lane
// (i, j) is [k0 + j*KPL + e <= 16 rt + i].  The same fragment serves as A
// operand of L and as B operand of L^T.  bf16 keeps the six that a 64-row
// chunk needs in registers (built once per workgroup); fp32 builds each on use.
template <typename T> struct TriOnes;
template <> struct TriOnes<bf16> {
    bf16x8 f[6];  // (rt, k0) = (0, 0), (1, 0), (2, 0), (2, 32), (3, 0), (3, 32)
    __device__ __forceinline__ TriOnes() {
        const int l = lane_id(), i = l & 15, j = l >> 4;
#pragma unroll
        for (int q = 0; q < 6; ++q) {
            const int rt = q < 2 ? q : 2 + (q - 2) / 2;
            const int k0 = q < 2 ? 0 : 32 * ((q - 2) % 2);
#pragma unroll
            for (int e = 0; e < 8; ++e) f[q][e] = (bf16)(k0 + 8 * j + e <= 16 * rt + i ? 1.0f : 0.0f);
        }
    }
    __device__ __forceinline__ bf16x8 get(int rt, int k0) const { return f[rt < 2 ? rt : 2 + 2 * (rt - 2) + k0 / 32]; }
};
template <> struct TriOnes<float> {
    __device__ __forceinline__ float get(int rt, int k0) const {
        const int l = lane_id();
        return k0 + (l >> 4) <= 16 * rt + (l & 15) ? 1.0f : 0.0f;
    }
};

// Chunk-local inclusive prefix of the per-channel log gates as one product
// with a triangular matrix of ones (FLAT page, Pallas Kernels > Gated Linear
// Attention: a prefix sum is a linear map, so the matrix unit can compute it):
// beta^T = G^T L^T with L[r][s] = [s <= r]; G is the natural [row][channel]
// tile (pitch PG), read column-wise.  Wave w computes channel tiles CPW*w .. CPW*w + CPW-1 for all four
// row tiles; the result is in C layout with lane (r = 16*rt + l%16) holding
// channels 16*ct + 4*(l/16) + e.
template <typename T, int CPW, int PG>
__device__ __forceinline__ void gate_prefix_mfma(const T* sG, const TriOnes<T>& L, f32x4 (&beta)[CPW][4]) {
    using M = Mma<T>;
    const int w = wave_id();
#pragma unroll
    for (int cc = 0; cc < CPW; ++cc) {
        const int ct = CPW * w + cc;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            f32x4 acc = zero4();
            constexpr int KS = M::KSTEP;
#pragma unroll
            for (int k0 = 0; k0 < ((16 * (rt + 1) + KS - 1) / KS) * KS; k0 += KS)
                acc = M::mma(frag_col<T, PG, false>(sG, 16 * ct, k0), L.get(rt, k0), acc);
            beta[cc][rt] = acc;
        }
    }
}

}  // namespace gla
