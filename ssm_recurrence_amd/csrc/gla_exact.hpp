// gla_exact.hpp -- the vector gate's intra-chunk decays for chunks whose log
// gates are too strong for the factored form.
//
// Inside a chunk the vector gate's scores are A[r][s] = sum_c q[r][c] k[s][c]
// exp(beta_r[c] - beta_s[c]) (FLAT page, "FLAT: Flash Linear Attention on TPUs",
// Pallas Kernels > Gated Linear Attention: the gate ratios are exponentials of
// differences of chunk-local log-gate prefixes).  The kernels normally factor
// the exponential around one reference row m of the chunk, as
// (q exp(beta_r - m)) (k exp(m - beta_s)), so the scores become one matrix
// product.  Each factor then spans up to 32 rows of log decay: with every
// |g| <= kGateFactored in the chunk the factors stay within exp(+-60), where
// fp32 and bf16 hold them with their full relative precision and their
// products are the exact terms up to rounding.  A chunk with any stronger gate
// (a decay below exp(-1.875) per token on some channel) is computed with the
// helpers below instead: every exp(beta_r - beta_s) is formed directly, which
// for g <= 0 and s <= r never leaves [0, 1], whatever the magnitudes.  The
// carried-state terms use exp(beta_r) and exp(Gamma - beta_s), which are in
// [0, 1] for every g <= 0 in either form.
#pragma once
#include "gla_common.hpp"
#include "gla_tile.hpp"

namespace gla {

constexpr float kGateFactored = 1.875f;  // 32 * 1.875 = 60

// 1 when a gate this thread staged (rows past the end read as 0) exceeds the
// factored form's range in magnitude
template <typename T, int D, int NTH>
__device__ __forceinline__ int gate_regs_strong(const TileRegs<T, D, NTH>& pg) {
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < TileRegs<T, D, NTH>::NVEC; ++i) {
        const i32x4 x = pg.get(i);
        const T* e = reinterpret_cast<const T*>(&x);
#pragma unroll
        for (int k = 0; k < TileRegs<T, D, NTH>::VE; ++k) mx = fmaxf(mx, fabsf(to_f32(e[k])));
    }
    return mx > kGateFactored;
}

// Per-wave flags written before a workgroup barrier and read after it: true in
// every wave when any wave saw a strong gate.
__device__ __forceinline__ void strong_flag_put(int* flags, int mine) {
    const bool any = __ballot(mine) != 0;
    if (lane_id() == 0) flags[wave_id()] = any ? 1 : 0;
}
template <int NW>
__device__ __forceinline__ bool strong_flag_get(const int* flags) {
    int x = 0;
#pragma unroll
    for (int u = 0; u < NW; ++u) x |= flags[u];
    return x != 0;
}

// sum_c q[c] k[c] exp(bq[c] - bk[c]) over n channels (n a multiple of 4), added to acc;
// q and k rows are 8-byte aligned (bf16) or 16-byte aligned (fp32), the prefix rows 16-byte
template <typename T>
__device__ __forceinline__ float exact_dot(const T* q, const T* k, const float* bq, const float* bk,
                                           int n, float acc) {
#pragma unroll 1
    for (int c = 0; c < n; c += 4) {
        const Vec4<T> qv = Vec4<T>::load(q + c), kv = Vec4<T>::load(k + c);
        const float4 b1 = *reinterpret_cast<const float4*>(bq + c);
        const float4 b2 = *reinterpret_cast<const float4*>(bk + c);
        acc += qv.get(0) * kv.get(0) * __expf(b1.x - b2.x);
        acc += qv.get(1) * kv.get(1) * __expf(b1.y - b2.y);
        acc += qv.get(2) * kv.get(2) * __expf(b1.z - b2.z);
        acc += qv.get(3) * kv.get(3) * __expf(b1.w - b2.w);
    }
    return acc;
}

// Intra-chunk scores of one chunk, exactly, for a workgroup of NTH threads:
// A[r][s] (s <= r, one document; else 0) into dst with pitch PD, either
// natural (dst[r][s]) or transposed (dst[s][r]).  Thread t computes row r = t / 8
// (repeated over the rows when NTH < 512), keys 8 (t % 8) .. 8 (t % 8) + 7.
// q, k: [64][DK] tiles (pitches PQ, PK) holding the raw inputs; beta: [64][PBF]
// fp32 chunk-local prefixes of all DK channels; doc: the document index of each row.
template <typename T, int DK, int NTH, int PQ, int PK, int PBF, int PD, bool TRANS>
__device__ __forceinline__ void exact_scores(T* dst, const T* sq, const T* sk, const float* beta,
                                             const int* doc) {
    static_assert(NTH % 8 == 0 && 512 % NTH == 0, "");
    // (loops kept rolled: this path is rare and must not add register pressure)
#pragma unroll 1
    for (int t = threadIdx.x; t < 512; t += NTH) {
        const int r = t >> 3, s0 = 8 * (t & 7);
        const int dr = doc[r];
#pragma unroll 1
        for (int u = 0; u < 8; ++u) {
            const int s = s0 + u;
            float acc = 0.f;
            if (s <= r && doc[s] == dr)
                acc = exact_dot<T>(sq + r * PQ, sk + s * PK, beta + r * PBF, beta + s * PBF, DK, 0.f);
            if constexpr (TRANS) dst[s * PD + r] = from_f32<T>(acc);
            else dst[r * PD + s] = from_f32<T>(acc);
        }
    }
}

// Exact intra-chunk parts of dq and dk for a wave whose lane (i, j) holds rows
// 16 rt + i and the four channels 4 j + e (e < 4) of a 16-channel tile, with the
// chunk-local prefixes of those positions in bp[rt][e]:
//   dq[r][c] = sum_{s <= r} dA[r][s] k[s][c] exp(beta_r[c] - beta_s[c])   (r = 16 rt + i)
//   dk[s][c] = sum_{r >= s} dA[r][s] q[r][c] exp(beta_r[c] - beta_s[c])   (s = 16 st + i)
// (FLAT page, Linear Attention > Backward Recurrence: the gradients of the
// intra-chunk scores, distributed back over the channels with each pair's decay.)
// The pairs with s < r (out) and the pair s = r (diag, whose decay is 1) are
// returned apart: in q dq - k dk the diagonal pairs cancel exactly, so the
// log-gate gradient of a strongly decaying chunk is formed from the others alone.
// dA [r][s] is in LDS with pitch PDA, already 0 for s > r and across documents;
// kc, qc point at the raw k, q tiles (pitch PK) offset to this lane's channels.
// The prefixes of other rows come from the lanes holding them.
template <typename T, int PK, int PDA>
__device__ __forceinline__ void exact_dq(float (&out)[4], float (&diag)[4], int rt, const float (&bp)[4][4],
                                         const T* sdA, const T* kc) {
    const int l = lane_id(), i = l & 15, j = l >> 4;
    const int r = 16 * rt + i;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
        if (st > rt) break;
#pragma unroll 1
        for (int u = 0; u < 16; ++u) {
            const int s = 16 * st + u;
            float bs[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) bs[e] = __shfl(bp[st][e], 16 * j + u, 64);
            if (s <= r) {
                const float a = to_f32(sdA[r * PDA + s]);
                const Vec4<T> kv = Vec4<T>::load(kc + s * PK);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (s < r) out[e] += a * kv.get(e) * __expf(bp[rt][e] - bs[e]);
                    else diag[e] = a * kv.get(e);
                }
            }
        }
    }
}
template <typename T, int PK, int PDA>
__device__ __forceinline__ void exact_dk(float (&out)[4], float (&diag)[4], int st, const float (&bp)[4][4],
                                         const T* sdA, const T* qc) {
    const int l = lane_id(), i = l & 15, j = l >> 4;
    const int s = 16 * st + i;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
        if (rt < st) continue;
#pragma unroll 1
        for (int u = 0; u < 16; ++u) {
            const int r = 16 * rt + u;
            float br[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) br[e] = __shfl(bp[rt][e], 16 * j + u, 64);
            if (r >= s) {
                const float a = to_f32(sdA[r * PDA + s]);
                const Vec4<T> qv = Vec4<T>::load(qc + r * PK);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (r > s) out[e] += a * qv.get(e) * __expf(br[e] - bp[st][e]);
                    else diag[e] = a * qv.get(e);
                }
            }
        }
    }
}

// Exclusive prefix over the 64 rows of a chunk held as z[rt] in lanes 16 rt + i
// of each row of 16 lanes (row r = 16 rt + i): out[rt] = sum of the rows before.
// Formed by adding, never by subtracting from a total.
__device__ __forceinline__ void rows_excl_prefix(const float (&z)[4], float (&out)[4]) {
    float carry = 0.f;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
        // lane i: sum of lanes 0 .. i - 1 of its row (row_shr:n reads lane i - n, 0 before the row)
        float y = dpp_f<0x111>(z[rt]);
        y += dpp_f<0x111>(y);
        y += dpp_f<0x112>(y);
        y += dpp_f<0x114>(y);
        y += dpp_f<0x118>(y);
        out[rt] = carry + y;
        carry += __shfl(y + z[rt], 15, 16);
    }
}

}  // namespace gla
