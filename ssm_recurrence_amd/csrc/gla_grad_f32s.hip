// gla_grad_f32s.hip -- chunk-parallel gradients for fp32 inputs with the scalar
// gate and 128 x 128 heads (gfx950), on the bf16 matrix cores.
//
// fp32 operands are split into bf16 hi/lo pairs and multiplied with three bf16
// matrix-core products (gla_split.hpp).
//
// The mathematics and the two kinds of workgroups are those of gla_grad.hip
// (QK: dq, dk and the log-gate partial sums for 64 key channels; V: dv for 64
// value columns), with every LDS tile stored as a hi plane followed by a lo
// plane; inputs, outputs and all accumulation stay fp32.  A QK workgroup visits
// all heads that share its q/k head and writes the summed dq, dk itself.
#include "gla_bwd.hpp"
#include "gla_common.hpp"
#include "gla_kernels.hpp"
#include "gla_split.hpp"
#include "gla_tile.hpp"

namespace gla {

namespace {

// masked score tile (scalar gate: times exp(beta_r - beta_s)) to a split tile;
// NAT: the tile was computed transposed (rows s, column r) and is stored [r][s];
// otherwise computed [r][s] (rows r, column s) and stored transposed [s][r]
template <bool NAT, int P, int PLANE>
__device__ __forceinline__ void store_masked_split(bf16* dst, const RevChunk& ck, int rt, int st, bool live,
                                                   const f32x4& acc) {
    const int l = lane_id(), j = l >> 4, i = l & 15;
    const int row = NAT ? 16 * rt + i : 16 * st + i;          // stored row (r, or s)
    const int c0 = NAT ? 16 * st + 4 * j : 16 * rt + 4 * j;   // first of four stored columns
    float x[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int r = NAT ? row : c0 + e, s = NAT ? c0 + e : row;
        x[e] = 0.f;
        if (live && s <= r && ck.doc[s] == ck.doc[r]) x[e] = acc[e] * __expf(ck.beta[r] - ck.beta[s]);
    }
    split4_store(x[0], x[1], x[2], x[3], dst + row * P + c0, dst + PLANE + row * P + c0);
}

constexpr int DK = 128, DV = 128, KS = 32;
// row pitches (bf16 elements): 16 mod 64 keeps the 16-byte row reads free of
// LDS bank conflicts on gfx950 (measured); transposed reads are free at these too
constexpr int P64 = 80, PL64 = C * P64;                  // [64][64] split tiles
constexpr int PW = 144, PLW = C * PW;                    // [64][128] split tiles
constexpr int PD = 68, PLD = DK * PD;                    // [128][64] split tile (state-gradient slice)
constexpr int QK_BYTES = 2 * (3 * PL64 + 2 * PLW) * 2;
constexpr int V_BYTES = 2 * (2 * PLW + 2 * PL64 + PLD) * 2;

struct SmallS {
    RevChunk ck;
    float sXs[4][C];
    float sBs[4];
};

// ============================================================== QK role
// Persistent workgroups over (b, q/k head, chunk, 64-channel slice) items: q and
// k are loaded once per item and the G heads that read them are visited in
// turn, each with its own v, dO, gate, state and state gradient; dq and dk are
// summed over those heads in registers (the head-sharing reduction of the FLAT
// page, Pallas Kernels > Gated Linear Attention, done in place of per-head
// buffers), and each head's log-gate partial sums are written for the
// finisher.  The next head's v, dO and gates (or the next item's first head)
// are loaded into registers while the current head computes; a head's state
// and state-gradient rows are requested before its tiles are staged; q and k
// are loaded at the item's start (once per G heads).

// v, dO and gate inputs of one head of a QK item
struct QKHeadRegs {
    TileRegs<float, DV> pv, pdo;
    RowRegs rr;
};

struct QKItem {
    int64_t b, hq, ci;
    int slice;
};
// (item counts fit in 32 bits: the launch bounds B H chunks well below 2^31)
__device__ __forceinline__ QKItem qk_item(const RevArgs& a, int64_t item64) {
    const uint32_t NC = (uint32_t)((a.T + C - 1) / C), Hqk = (uint32_t)a.Hqk;
    const uint32_t item = (uint32_t)item64;
    QKItem it;
    it.slice = (int)(item & 1);
    const uint32_t rest = item >> 1;
    it.ci = rest % NC;
    const uint32_t bq = rest / NC;
    it.b = bq / Hqk;
    it.hq = bq % Hqk;
    return it;
}

__device__ __forceinline__ void qk_load_qk(const RevArgs& a, const QKItem& it, TileRegs<float, 64>& pq,
                                           TileRegs<float, 64>& pk) {
    const int64_t T_ = a.T, t0 = it.ci * C;
    const int nvalid = (T_ - t0) < C ? (int)(T_ - t0) : C;
    const int64_t rs_qk = a.ld_qk;
    const int64_t off = (it.b * T_ + t0) * rs_qk + it.hq * DK + it.slice * 64;
    pq.load((const float*)a.q + off, rs_qk, nvalid);
    pk.load((const float*)a.k + off, rs_qk, nvalid);
}

__device__ __forceinline__ void qk_load_head(const RevArgs& a, const QKItem& it, int64_t gi, QKHeadRegs& R) {
    const int64_t T_ = a.T, t0 = it.ci * C;
    const int nvalid = (T_ - t0) < C ? (int)(T_ - t0) : C;
    const int64_t G = a.H / a.Hqk;
    const int64_t h = it.hq * G + gi;
    const int64_t rs_v = a.ld_v, rs_do = a.H * DV;
    const int w = wave_id();
    R.pv.load((const float*)a.v + (it.b * T_ + t0) * rs_v + h * DV, rs_v, nvalid);
    R.pdo.load((const float*)a.dO + (it.b * T_ + t0) * rs_do + h * DV, rs_do, nvalid);
    if (w == 0) R.rr.load((const float*)a.g + (it.b * T_ + t0) * a.H + h, a.H, a.seg, it.b, T_, t0, nvalid, true);
}

__global__ __launch_bounds__(NT) void k_grad_f32s_qk(const RevArgs a) {
    __shared__ __attribute__((aligned(16))) char lds[QK_BYTES];
    __shared__ SmallS sm;
    bf16* sQ = reinterpret_cast<bf16*>(lds);
    bf16* sK = sQ + 2 * PL64;
    bf16* sdA = sK + 2 * PL64;  // [r][s]
    bf16* sdO = sdA + 2 * PL64;
    bf16* sV = sdO + 2 * PLW;
    RevChunk& ck = sm.ck;

    const int64_t G = a.H / a.Hqk;
    const int w = wave_id(), l = lane_id(), j4 = l >> 4, i16 = l & 15;
    const int64_t T_ = a.T;
    const int64_t NC = (T_ + C - 1) / C;
    const int64_t nitems = a.B * a.Hqk * NC * 2;
    const int64_t stride = gridDim.x;

    QKHeadRegs hr;
    int64_t item = xcd_logical_block(gridDim.x);
    if (item < nitems) qk_load_head(a, qk_item(a, item), 0, hr);
    for (; item < nitems; item += stride) {
        const QKItem it = qk_item(a, item);
        const int64_t b = it.b, hq = it.hq, ci = it.ci;
        const int slice = it.slice;
        const int cw = slice * 64 + 16 * w;
        const int64_t t0 = ci * C;
        const int nvalid = (T_ - t0) < C ? (int)(T_ - t0) : C;

        {
            TileRegs<float, 64> pq, pk;
            qk_load_qk(a, it, pq, pk);
            store_rows_split<64>(pq, sQ, P64, PL64);
            store_rows_split<64>(pk, sK, P64, PL64);
        }
        float dqs[4][4], dks[4][4];  // dq, dk summed over the heads of the group
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int e = 0; e < 4; ++e) dqs[rt][e] = dks[rt][e] = 0.f;

        for (int64_t gi = 0; gi < G; ++gi) {
            const int64_t h = hq * G + gi, bh = b * a.H + h;
            // S0 and dS1 rows cw + i16 (channels of lane group j4), issued first: they are
            // first needed after the score tiles
            f32x4 s0r[2 * DV / KS], dsr[2 * DV / KS];
            {
                const float* S0 = (const float*)a.ws_S + ((bh * (NC + 1) + ci) * DK + cw + i16) * DV + 8 * j4;
                const float* dS1 = (const float*)a.ws_dS + ((bh * NC + ci) * DK + cw + i16) * DV + 8 * j4;
#pragma unroll
                for (int kk = 0; kk < DV / KS; ++kk) {
                    s0r[2 * kk] = *reinterpret_cast<const f32x4*>(S0 + kk * KS);
                    s0r[2 * kk + 1] = *reinterpret_cast<const f32x4*>(S0 + kk * KS + 4);
                    dsr[2 * kk] = *reinterpret_cast<const f32x4*>(dS1 + kk * KS);
                    dsr[2 * kk + 1] = *reinterpret_cast<const f32x4*>(dS1 + kk * KS + 4);
                }
            }
            store_rows_split<DV>(hr.pv, sV, PW, PLW);
            store_rows_split<DV>(hr.pdo, sdO, PW, PLW);
            if (w == 0) rev_chunk_info<float, false>(&ck, hr.rr);
            __syncthreads();
            // the next head's inputs, or the next item's
            if (gi + 1 < G) {
                qk_load_head(a, it, gi + 1, hr);
            } else if (item + stride < nitems) {
                qk_load_head(a, qk_item(a, item + stride), 0, hr);
            }

            // dA^T = v dO^T tiles, masked, stored dA[r][s]
            for (int ti = w; ti < 12; ti += 4) {
                const int rt = score_tile_rt(ti);
                const int st = score_tile_st(ti);
                const f32x4 acc =
                    mma3_chain<DV / KS>(zero4(), ti < 10 ? DV / KS : 0, [&](int i, SFrag& A, SFrag& B) {
                        A = sld<PW, PLW>(sV, 16 * st, i * KS);
                        B = sld<PW, PLW>(sdO, 16 * rt, i * KS);
                    });
                store_masked_split<true, P64, PL64>(sdA, ck, rt, st, ti < 10, acc);
            }
            __syncthreads();

            // S0 and dS1 rows as split A operands (k = n); rowsum(S0 * dS1) in fp32
            float sd = 0.f;
            SFrag s0f[DV / KS], dsf[DV / KS];
#pragma unroll
            for (int kk = 0; kk < DV / KS; ++kk) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sd += s0r[2 * kk][e] * dsr[2 * kk][e] + s0r[2 * kk + 1][e] * dsr[2 * kk + 1][e];
                s0f[kk] = split8(s0r[2 * kk], s0r[2 * kk + 1]);
                dsf[kk] = split8(dsr[2 * kk], dsr[2 * kk + 1]);
            }

            // q, k at this lane's output positions (rows 16rt + i16, channels cw + 4j4 + e),
            // from the split tiles (hi + lo)
            float xr[4];  // per row: sum over this lane's channels of q dq - k dk
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                const int nk = (16 * (rt + 1) + KS - 1) / KS;
                const f32x4 a1 = mma3_chain<C / KS>(zero4(), nk, [&](int i, SFrag& A, SFrag& B) {
                    A = scol<P64, PL64>(sK, 16 * w, i * KS);
                    B = sld<P64, PL64>(sdA, 16 * rt, i * KS);
                });
                const f32x4 a2 = mma3_chain<DV / KS>(zero4(), DV / KS, [&](int i, SFrag& A, SFrag& B) {
                    A = s0f[i];
                    B = sld<PW, PLW>(sdO, 16 * rt, i * KS);
                });
                const int r = 16 * rt + i16;
                const float fq = ck.fq[r];
                const Vec4<bf16> qh = Vec4<bf16>::load(sQ + r * P64 + 16 * w + 4 * j4);
                const Vec4<bf16> ql = Vec4<bf16>::load(sQ + PL64 + r * P64 + 16 * w + 4 * j4);
                xr[rt] = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float dq = a1[e] + fq * a2[e];
                    xr[rt] += (qh.get(e) + ql.get(e)) * dq;
                    dqs[rt][e] += dq;
                }
            }
            float bsum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const int kb = 16 * st / KS;
                const f32x4 a1 = mma3_chain<C / KS>(zero4(), C / KS - kb, [&](int i, SFrag& A, SFrag& B) {
                    A = scol<P64, PL64>(sQ, 16 * w, (kb + i) * KS);
                    B = scol<P64, PL64>(sdA, 16 * st, (kb + i) * KS);
                });
                const f32x4 a2 = mma3_chain<DV / KS>(zero4(), DV / KS, [&](int i, SFrag& A, SFrag& B) {
                    A = dsf[i];
                    B = sld<PW, PLW>(sV, 16 * st, i * KS);
                });
                const int s = 16 * st + i16;
                const float fu = ck.fu[s];
                const Vec4<bf16> kh = Vec4<bf16>::load(sK + s * P64 + 16 * w + 4 * j4);
                const Vec4<bf16> kl = Vec4<bf16>::load(sK + PL64 + s * P64 + 16 * w + 4 * j4);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float inter = fu * a2[e];
                    const float dk = a1[e] + inter;
                    const float kr = kh.get(e) + kl.get(e);
                    xr[st] -= kr * dk;
                    bsum[e] += kr * inter;
                    dks[st][e] += dk;
                }
            }
            sd += __shfl_xor(sd, 16, 64);
            sd += __shfl_xor(sd, 32, 64);
            float bb = 0.f;  // sum over this lane group's four channels of rowsum(S1 * dS1)
#pragma unroll
            for (int e = 0; e < 4; ++e) bb += ck.decay * __shfl(sd, 4 * j4 + e, 64) + row_sum16(bsum[e]);
            // partial sums over this workgroup's channels; a finisher adds the two slices
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                float y = xr[rt];
                y += __shfl_xor(y, 16, 64);
                y += __shfl_xor(y, 32, 64);
                if (j4 == 0) sm.sXs[w][16 * rt + i16] = y;
            }
            bb += __shfl_xor(bb, 16, 64);
            bb += __shfl_xor(bb, 32, 64);
            if (l == 0) sm.sBs[w] = bb;
            __syncthreads();  // also: every wave is done with this head's v, dO and dA
            if (w == 0) {
                const int r = l;
                const float tot = sm.sXs[0][r] + sm.sXs[1][r] + sm.sXs[2][r] + sm.sXs[3][r];
                if (r < nvalid) a.ws_xs[(bh * 2 + slice) * T_ + t0 + r] = tot;
                if (r == 0) a.ws_bnd[(bh * 2 + slice) * NC + ci] = sm.sBs[0] + sm.sBs[1] + sm.sBs[2] + sm.sBs[3];
            }
        }
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            const int r = 16 * rt + i16;
            if (r < nvalid) {
                const int64_t o = (b * T_ + t0 + r) * a.ld_dqk + hq * DK + cw + 4 * j4;
                store4<float>((float*)a.dq + o, dqs[rt]);
                store4<float>((float*)a.dk + o, dks[rt]);
            }
        }
    }
}

// ============================================================== V role
// Persistent workgroups over (b, head, chunk, 64-column slice) items; the next
// item's inputs are loaded into registers while the current item computes.
struct VRegs {
    TileRegs<float, DK> pq, pk;
    TileRegs<float, 64> pdo, pds0, pds1;
    RowRegs rr;
};
struct VItem {
    int64_t b, h, hq, ci;
    int slice;
};
__device__ __forceinline__ VItem v_item(const RevArgs& a, int64_t item64) {
    const uint32_t NC = (uint32_t)((a.T + C - 1) / C), Hqk = (uint32_t)a.Hqk;
    const uint32_t G = (uint32_t)(a.H / a.Hqk);
    const uint32_t item = (uint32_t)item64;
    VItem it;
    it.slice = (int)(item & 1);
    const uint32_t r1 = item >> 1;
    const uint32_t gi = r1 % G, r2 = r1 / G;
    it.ci = r2 % NC;
    const uint32_t bq = r2 / NC;
    it.b = bq / Hqk;
    it.hq = bq % Hqk;
    it.h = it.hq * G + gi;
    return it;
}
__device__ __forceinline__ void v_load(const RevArgs& a, const VItem& it, VRegs& R) {
    const int64_t T_ = a.T, t0 = it.ci * C;
    const int64_t NC = (T_ + C - 1) / C;
    const int nvalid = (T_ - t0) < C ? (int)(T_ - t0) : C;
    const int64_t rs_qk = a.ld_qk, rs_do = a.H * DV;
    const int64_t bh = it.b * a.H + it.h;
    const int n0s = it.slice * 64;
    R.pq.load((const float*)a.q + (it.b * T_ + t0) * rs_qk + it.hq * DK, rs_qk, nvalid);
    R.pk.load((const float*)a.k + (it.b * T_ + t0) * rs_qk + it.hq * DK, rs_qk, nvalid);
    R.pdo.load((const float*)a.dO + (it.b * T_ + t0) * rs_do + it.h * DV + n0s, rs_do, nvalid);
    const float* dS1 = (const float*)a.ws_dS + (bh * NC + it.ci) * DK * DV + n0s;
    R.pds0.load(dS1, DV, 64);
    R.pds1.load(dS1 + (int64_t)64 * DV, DV, 64);
    if (wave_id() == 0)
        R.rr.load((const float*)a.g + (it.b * T_ + t0) * a.H + it.h, a.H, a.seg, it.b, T_, t0, nvalid, true);
}

__global__ __launch_bounds__(NT) void k_grad_f32s_v(const RevArgs a) {
    __shared__ __attribute__((aligned(16))) char lds[V_BYTES];
    __shared__ RevChunk ck;
    bf16* sQ = reinterpret_cast<bf16*>(lds);
    bf16* sK = sQ + 2 * PLW;
    bf16* sdO = sK + 2 * PLW;   // [r][64 columns of the slice]
    bf16* sAT = sdO + 2 * PL64; // [s][r]
    bf16* sdS = sAT + 2 * PL64; // [c][64 columns]

    const int w = wave_id(), j4 = lane_id() >> 4, i16 = lane_id() & 15;
    const int64_t T_ = a.T;
    const int64_t NC = (T_ + C - 1) / C;
    const int64_t nitems = a.B * a.H * NC * 2;
    const int64_t stride = gridDim.x;

    VRegs R;
    int64_t item = xcd_logical_block(gridDim.x);
    if (item < nitems) v_load(a, v_item(a, item), R);
    for (; item < nitems; item += stride) {
        const VItem it = v_item(a, item);
        const int64_t t0 = it.ci * C;
        const int nvalid = (T_ - t0) < C ? (int)(T_ - t0) : C;
        store_rows_split<DK>(R.pq, sQ, PW, PLW);
        store_rows_split<DK>(R.pk, sK, PW, PLW);
        store_rows_split<64>(R.pdo, sdO, P64, PL64);
        store_rows_split<64>(R.pds0, sdS, PD, PLD);
        store_rows_split<64>(R.pds1, sdS + 64 * PD, PD, PLD);
        if (w == 0) rev_chunk_info<float, false>(&ck, R.rr);
        __syncthreads();
        if (item + stride < nitems) v_load(a, v_item(a, item + stride), R);

        // A = q k^T tiles, masked with the scalar decay, stored transposed A^T[s][r]
        for (int ti = w; ti < 12; ti += 4) {
            const int rt = score_tile_rt(ti);
            const int st = score_tile_st(ti);
            const f32x4 acc = mma3_chain<DK / KS>(zero4(), ti < 10 ? DK / KS : 0, [&](int i, SFrag& A, SFrag& B) {
                A = sld<PW, PLW>(sQ, 16 * rt, i * KS);
                B = sld<PW, PLW>(sK, 16 * st, i * KS);
            });
            store_masked_split<false, P64, PL64>(sAT, ck, rt, st, ti < 10, acc);
        }
        __syncthreads();

        // dv^T = dO^T A + [last doc] exp(Gamma - beta_s) dS1^T k^T (rows n, columns s)
        float* dvo = (float*)a.dv + (it.b * T_ + t0) * a.ld_dv + it.h * DV + it.slice * 64 + 16 * w + 4 * j4;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const int kb = 16 * st / KS;
            const f32x4 a1 = mma3_chain<C / KS>(zero4(), C / KS - kb, [&](int i, SFrag& A, SFrag& B) {
                A = scol<P64, PL64>(sdO, 16 * w, (kb + i) * KS);
                B = sld<P64, PL64>(sAT, 16 * st, (kb + i) * KS);
            });
            const f32x4 a2 = mma3_chain<DK / KS>(zero4(), DK / KS, [&](int i, SFrag& A, SFrag& B) {
                A = scol<PD, PLD>(sdS, 16 * w, i * KS);
                B = sld<PW, PLW>(sK, 16 * st, i * KS);
            });
            const int s = 16 * st + i16;
            const float fu = ck.fu[s];
            float dv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) dv[e] = a1[e] + fu * a2[e];
            if (s < nvalid) store4<float>(dvo + (int64_t)s * a.ld_dv, dv);
        }
        __syncthreads();  // LDS is restaged for the next item
    }
}

}  // namespace

hipError_t launch_grad_f32s(const RevArgs& a, hipStream_t st) {
    const int64_t NC = (a.T + C - 1) / C;
    const int64_t nqk = a.B * a.Hqk * NC * 2, nv = a.B * a.H * NC * 2;
    // persistent: one workgroup per compute unit (the LDS allows no more)
    const int64_t workers = 256;
    hipLaunchKernelGGL(k_grad_f32s_qk, dim3((unsigned)(nqk < workers ? nqk : workers)), dim3(NT), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_grad_f32s_v, dim3((unsigned)(nv < workers ? nv : workers)), dim3(NT), 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_dg_scalar(a, 2, false, st);
}

}  // namespace gla
