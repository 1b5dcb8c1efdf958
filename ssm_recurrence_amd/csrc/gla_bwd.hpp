// gla_bwd.hpp -- device helpers shared by the backward kernels: operand
// fragments read straight from global memory, per-k scaling of fragments, and
// the per-chunk document data (reset structure, scalar-gate prefix factors).
#pragma once
#include "gla_common.hpp"
#include "gla_tile.hpp"

namespace gla {

// rows of a global T tensor as an operand fragment in ctile k order
// (lane i, k = k0 + 4j + e, k0 + 16 + 4j + e; f32: k0 + 4j + sub); zero past nvalid
template <typename T>
__device__ __forceinline__ typename Mma<T>::frag glb_rows_ctile(const T* base, int64_t rs, int i0, int k0,
                                                                int sub, int nvalid) {
    const int l = lane_id();
    const int i = i0 + (l & 15), j = l >> 4;
    typename Mma<T>::frag f = Mma<T>::zero();
    if (i < nvalid) {
        const T* p = base + (int64_t)i * rs;
        if constexpr (Mma<T>::KPL == 1) {
            f = p[k0 + 4 * j + sub];
        } else {
            const bf16x4 lo = *reinterpret_cast<const bf16x4*>(p + k0 + 4 * j);
            const bf16x4 hi = *reinterpret_cast<const bf16x4*>(p + k0 + 16 + 4 * j);
            f = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
    }
    return f;
}

template <typename T>
__device__ __forceinline__ typename Mma<T>::frag glb_rows_nat(const T* base, int64_t rs, int i0, int k0,
                                                              int nvalid) {
    const int l = lane_id();
    const int i = i0 + (l & 15);
    typename Mma<T>::frag f = Mma<T>::zero();
    if (i < nvalid) {
        const T* p = base + (int64_t)i * rs + k0 + (l >> 4) * Mma<T>::KPL;
        if constexpr (Mma<T>::KPL == 1) f = *p;
        else f = *reinterpret_cast<const bf16x8*>(p);
    }
    return f;
}

// scale each k element of a fragment: element e has k = k0 + j*KPL + e
template <typename T, typename F>
__device__ __forceinline__ void frag_scale_k(typename Mma<T>::frag& f, int k0, F&& factor) {
    const int j = lane_id() >> 4;
#pragma unroll
    for (int e = 0; e < Mma<T>::KPL; ++e) {
        float x;
        if constexpr (Mma<T>::KPL == 1) x = to_f32(f); else x = to_f32(f[e]);
        Mma<T>::set(f, e, x * factor(k0 + j * Mma<T>::KPL + e));
    }
}
// same, for a fragment in ctile k order
template <typename T, typename F>
__device__ __forceinline__ void frag_scale_k_ctile(typename Mma<T>::frag& f, int k0, int sub, F&& factor) {
    const int j = lane_id() >> 4;
    if constexpr (Mma<T>::KPL == 1) {
        f = f * factor(k0 + 4 * j + sub);
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int k = e < 4 ? k0 + 4 * j + e : k0 + 16 + 4 * j + (e - 4);
            f[e] = (bf16)((float)f[e] * factor(k));
        }
    }
}

// Chunk-level document data shared by both roles (wave 0 fills it).
struct RevChunk {
    int doc[C];
    float beta[C];   // scalar gate: chunk-local prefix
    float fq[C];     // readout rows: [r in first doc] (* exp(beta_r) for the scalar gate)
    float fu[C];     // update rows:  [s in last doc]  (* exp(Gamma - beta_s) for the scalar gate)
    float decay;     // scalar gate: exp(Gamma), 0 if the chunk has a reset
    int first_reset, last_reset;
};

template <typename T, bool VEC>
__device__ __forceinline__ void rev_chunk_info(RevChunk* ci, const RowRegs& rr) {
    const int r = lane_id();
    const int doc = wave_incl_scan_i(rr.reset);
    const uint64_t msk = __ballot(rr.reset);
    const int first_reset = msk ? __builtin_ctzll(msk) : C;
    const int last_reset = msk ? 63 - __builtin_clzll(msk) : -1;
    ci->doc[r] = doc;
    if (r == 0) {
        ci->first_reset = first_reset;
        ci->last_reset = last_reset;
    }
    if constexpr (!VEC) {
        const float beta = wave_incl_scan(rr.g);
        const float Gam = __shfl(beta, 63, 64);
        ci->beta[r] = beta;
        ci->fq[r] = r < first_reset ? __expf(beta) : 0.f;
        ci->fu[r] = r >= last_reset ? __expf(Gam - beta) : 0.f;
        if (r == 0) ci->decay = msk ? 0.f : __expf(Gam);
    } else {
        ci->fq[r] = r < first_reset ? 1.f : 0.f;
        ci->fu[r] = r >= last_reset ? 1.f : 0.f;
    }
}

}  // namespace gla
