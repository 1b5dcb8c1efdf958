// gla_tile.hpp -- register-staged chunk tiles for software-pipelined passes:
// the next chunk's rows are loaded from HBM into registers while the current
// chunk computes, then written to LDS (natural or transposed layout).
#pragma once
#include "gla_common.hpp"

namespace gla {

typedef __attribute__((__vector_size__(16))) int i32x4;

template <typename T, int D>
struct TileRegs {
    static constexpr int VE = 16 / (int)sizeof(T);   // elements per 16-byte vector
    static constexpr int VPR = D / VE;                // vectors per row
    static constexpr int NV_TOT = C * VPR;            // vectors per tile
    static constexpr int NVEC = (NV_TOT + NT - 1) / NT;
    i32x4 r[NVEC];

    // rows t0.. of a row-major tensor (row stride rs elements); rows >= nvalid read as zero
    __device__ __forceinline__ void load(const T* src, int64_t rs, int nvalid) {
#pragma unroll
        for (int i = 0; i < NVEC; ++i) {
            const int idx = threadIdx.x + i * NT;
            const int row = idx / VPR, cv = (idx % VPR) * VE;
            i32x4 z = {0, 0, 0, 0};
            r[i] = z;
            if (idx < NV_TOT && row < nvalid)
                r[i] = *reinterpret_cast<const i32x4*>(src + (int64_t)row * rs + cv);
        }
    }
    // dst[row][col] with pitch P
    __device__ __forceinline__ void store_rows(T* dst, int P) const {
#pragma unroll
        for (int i = 0; i < NVEC; ++i) {
            const int idx = threadIdx.x + i * NT;
            if (idx < NV_TOT) {
                const int row = idx / VPR, cv = (idx % VPR) * VE;
                *reinterpret_cast<i32x4*>(dst + row * P + cv) = r[i];
            }
        }
    }
    // dst[col][row] with pitch P (transpose)
    __device__ __forceinline__ void store_cols(T* dst, int P) const {
#pragma unroll
        for (int i = 0; i < NVEC; ++i) {
            const int idx = threadIdx.x + i * NT;
            if (idx < NV_TOT) {
                const int row = idx / VPR, cv = (idx % VPR) * VE;
                const T* e = reinterpret_cast<const T*>(&r[i]);
#pragma unroll
                for (int k = 0; k < VE; ++k) dst[(cv + k) * P + row] = e[k];
            }
        }
    }
};

// Per-lane values for one chunk that wave 0 needs: the scalar gate of row
// `lane` and the reset flag of row `lane`.
struct RowRegs {
    float g;
    int reset;
    template <typename T>
    __device__ __forceinline__ void load(const T* gcol, int64_t rs_g, const int32_t* seg, int64_t b,
                                         int64_t T_, int64_t t0, int nvalid, bool scalar_gate) {
        const int r = lane_id();
        const int64_t t = t0 + r;
        g = (scalar_gate && r < nvalid) ? to_f32(gcol[(int64_t)r * rs_g]) : 0.f;
        reset = 0;
        if (seg != nullptr && r < nvalid && t > 0) reset = seg[b * T_ + t] != seg[b * T_ + t - 1];
    }
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

// Block id -> logical id so that consecutive logical ids (the slices of one
// head) land on the same XCD: the hardware deals consecutive block ids round
// robin over the 8 XCDs.
__device__ __forceinline__ int64_t xcd_logical_block(int64_t nblocks) {
    const int64_t x = blockIdx.x;
    if (nblocks % 8 != 0) return x;
    return (x % 8) * (nblocks / 8) + x / 8;
}

}  // namespace gla
