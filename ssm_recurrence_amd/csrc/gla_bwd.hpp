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
    alignas(16) int doc[C];
    alignas(16) float beta[C];   // scalar gate: chunk-local prefix
    alignas(16) float fq[C];     // readout rows: [r in first doc] (* exp(beta_r) for the scalar gate)
    alignas(16) float fu[C];     // update rows:  [s in last doc]  (* exp(Gamma - beta_s) for the scalar gate)
    float decay;     // scalar gate: exp(Gamma), 0 if the chunk has a reset
    int first_reset, last_reset;
};

// Store one 16x16 C-layout tile (rows r = 16rt + 4j + e, column s = 16st + i) of
// an intra-chunk score matrix, causally and document masked (scalar gate: times
// exp(beta_r - beta_s)), transposed: dstT[s][r], four consecutive r per lane in
// one 8-byte store.  `live` false stores zeros (the upper tiles a 32-wide k step reads).
template <typename T, bool VEC, int P>
__device__ __forceinline__ void store_masked_T(T* dstT, const RevChunk& ck, int rt, int st, bool live,
                                               const f32x4& acc) {
    const int l = lane_id(), j = l >> 4, i = l & 15;
    const int r0 = 16 * rt + 4 * j, s = 16 * st + i;
    Vec4<T> out;
    if (live) {
        const int4 dr = *reinterpret_cast<const int4*>(&ck.doc[r0]);
        const int ds = ck.doc[s];
        const int drr[4] = {dr.x, dr.y, dr.z, dr.w};
        float bs = 0.f, br[4] = {0.f, 0.f, 0.f, 0.f};
        if constexpr (!VEC) {
            const float4 b4 = *reinterpret_cast<const float4*>(&ck.beta[r0]);
            br[0] = b4.x; br[1] = b4.y; br[2] = b4.z; br[3] = b4.w;
            bs = ck.beta[s];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float x = 0.f;
            if (s <= r0 + e && drr[e] == ds) {
                x = acc[e];
                if constexpr (!VEC) x *= __expf(br[e] - bs);
            }
            out.set(e, x);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) out.set(e, 0.f);
    }
    out.store(dstT + s * P + r0);
}

// Same, for a tile computed transposed (rows s = 16st + 4j + e, column r = 16rt + i):
// stored in natural orientation dst[r][s], four consecutive s per lane.
template <typename T, bool VEC, int P>
__device__ __forceinline__ void store_masked_N(T* dst, const RevChunk& ck, int rt, int st, bool live,
                                               const f32x4& acc) {
    const int l = lane_id(), j = l >> 4, i = l & 15;
    const int r = 16 * rt + i, s0 = 16 * st + 4 * j;
    Vec4<T> out;
    if (live) {
        const int4 dsv = *reinterpret_cast<const int4*>(&ck.doc[s0]);
        const int dr = ck.doc[r];
        const int dss[4] = {dsv.x, dsv.y, dsv.z, dsv.w};
        float br = 0.f, bs[4] = {0.f, 0.f, 0.f, 0.f};
        if constexpr (!VEC) {
            const float4 b4 = *reinterpret_cast<const float4*>(&ck.beta[s0]);
            bs[0] = b4.x; bs[1] = b4.y; bs[2] = b4.z; bs[3] = b4.w;
            br = ck.beta[r];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float x = 0.f;
            if (s0 + e <= r && dss[e] == dr) {
                x = acc[e];
                if constexpr (!VEC) x *= __expf(br - bs[e]);
            }
            out.set(e, x);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) out.set(e, 0.f);
    }
    out.store(dst + r * P + s0);
}

// Four consecutive values of one row of an output, 16 bytes (fp32) or 8 (bf16).
template <typename T>
__device__ __forceinline__ void store4(T* p, const float (&v)[4]) {
    Vec4<T> x;
#pragma unroll
    for (int e = 0; e < 4; ++e) x.set(e, v[e]);
    x.store(p);
}

// element e of an operand fragment, as float
template <typename T>
__device__ __forceinline__ float frag_get(const typename Mma<T>::frag& f, int e) {
    if constexpr (Mma<T>::KPL == 1) { (void)e; return f; }
    else return (float)f[e];
}

template <typename T, bool VEC>
__device__ __forceinline__ void rev_chunk_info(RevChunk* ci, const RowRegs& rr) {
    const int r = lane_id();
    const int doc = wave_incl_scan_i(rr.reset());
    const uint64_t msk = __ballot(rr.reset());
    const int first_reset = msk ? __builtin_ctzll(msk) : C;
    const int last_reset = msk ? 63 - __builtin_clzll(msk) : -1;
    ci->doc[r] = doc;
    if (r == 0) {
        ci->first_reset = first_reset;
        ci->last_reset = last_reset;
    }
    if constexpr (!VEC) {
        const float beta = wave_incl_scan(rr.g());
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

// Log-gate gradient of a vector-gate chunk for one wave's 16 key channels (lane
// (i, j): rows 16 rt + i, channels c0 + 4 j + e) when documents end inside the
// chunk: a serial suffix sum per channel of the per-row terms x, restarting at
// every document end, with the boundary term bnd added to the chunk's last
// document; 0 at reset tokens, and add[rt][e] added elsewhere.  The sums run in
// the wave's own columns of an fp32 scratch sX[r][c] (pitch PE), so only the
// wave synchronises.  dgo points at row 0, channel 0 of the chunk's dg, rows rs apart.
template <typename T, int PE>
__device__ __forceinline__ void vec_dg_serial(float* sX, float* sBndW, const RevChunk& ck, int c0,
                                              const float (&x)[4][4], const float (&bnd)[4],
                                              const float (&add)[4][4], int nvalid, T* dgo, int64_t rs) {
    const int l = lane_id(), j4 = l >> 4, i16 = l & 15;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
        *reinterpret_cast<f32x4*>(sX + (16 * rt + i16) * PE + c0 + 4 * j4) = f32x4{x[rt][0], x[rt][1], x[rt][2], x[rt][3]};
    if (i16 == 0)
#pragma unroll
        for (int e = 0; e < 4; ++e) sBndW[4 * j4 + e] = bnd[e];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (j4 == 0) {
        const int c = c0 + i16;
        float run = sBndW[i16];
        for (int r = C - 1; r >= 0; --r) {
            float val = 0.f;
            if (r < nvalid) {
                if (r < nvalid - 1 && ck.doc[r + 1] != ck.doc[r]) run = 0.f;
                run += sX[r * PE + c];
                const bool reset = r > 0 ? ck.doc[r] != ck.doc[r - 1] : ck.doc[0] != 0;
                val = reset ? 0.f : run;
            }
            sX[r * PE + c] = val;
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
        const int r = 16 * rt + i16;
        const f32x4 v = *reinterpret_cast<const f32x4*>(sX + r * PE + c0 + 4 * j4);
        const bool reset = r > 0 ? ck.doc[r] != ck.doc[r - 1] : ck.doc[0] != 0;
        float dg[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) dg[e] = v[e] + (reset ? 0.f : add[rt][e]);
        if (r < nvalid) store4<T>(dgo + (int64_t)r * rs + c0 + 4 * j4, dg);
    }
}

}  // namespace gla
