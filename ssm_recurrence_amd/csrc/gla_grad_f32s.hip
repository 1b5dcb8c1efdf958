// gla_grad_f32s.hip -- chunk-parallel gradients for fp32 inputs with the scalar
// gate and 128 x 128 heads (gfx950), on the bf16 matrix cores.
//
// fp32 operands are split into bf16 hi/lo pairs and multiplied with three bf16
// matrix-core products (gla_split.hpp); inputs, outputs and all accumulation
// stay fp32.  The mathematics is that of gla_grad.hip (dq, dk, dv and the
// log-gate partial sums of one chunk from its inputs, the state entering it
// and the state gradient at its end), done here by one kernel per (b, q/k
// head, chunk) that visits the heads sharing q and k in turn and writes the
// summed dq, dk itself.
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
                                                   const f32x4& acc, int l = lane_id()) {
    const int j = l >> 4, i = l & 15;
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

// One workgroup of MNW waves per (b, q/k head, chunk) item, persistent over
// items.  q and k are staged once per item; the G heads that read them are
// then visited in turn: each head's v, dO, gate, state rows and state-gradient
// rows are requested once (v, dO, gates and the state-gradient rows one head
// ahead), and the workgroup computes that head's dA, A (q k^T with the head's
// decay mask), dv and its share of dq, dk (summed over the heads in registers)
// and of the log-gate partial sums.  Wave w owns the MNCT 16-wide tiles u of
// key channels and of value columns at 16 (MNCT w + u).  Eight waves (two per
// SIMD) measured about 5 % faster than four (one per SIMD, no spills) on the
// fp32 SSD workload, although 17 registers spill at eight.
//
// LDS (bf16 split tiles, hi plane then lo plane): q [64][136], k [64][144],
// v [64][144] (reused for this head's A^T [64][72] once dA and dk's
// inter-chunk term are formed), dO [64][136], dA [64][72] (reused for the
// per-wave x sums once dq, dk are formed): 161,792 bytes, one workgroup per
// compute unit.  The pitches that serve 16-byte row reads (k, v) are 16 mod
// 64 elements; q and dO (mostly transposed reads) are 8 mod 64 to fit.
constexpr int MNW = 8;             // waves per workgroup
constexpr int MNCT = 8 / MNW;      // 16-wide channel (and column) tiles per wave
constexpr int NT8 = 64 * MNW;
constexpr int PQ8 = 136, PK8 = 144, PV8 = 144, PO8 = 136, PA8 = 72;
constexpr int PLQ8 = C * PQ8, PLK8 = C * PK8, PLV8 = C * PV8, PLO8 = C * PO8, PLA8 = C * PA8;
constexpr int M_ELEMS = 2 * (PLQ8 + PLK8 + PLV8 + PLO8 + PLA8);
constexpr int MNQK = (12 + MNW - 1) / MNW;  // score tiles per wave
static_assert(PLA8 <= PLV8, "A^T fits in v's region");
static_assert(MNW * C * sizeof(float) <= 2 * PLA8 * sizeof(bf16), "x sums fit in dA's region");

struct MItem {
    int64_t b, hq, ci;
};
__device__ __forceinline__ MItem m_item(const RevArgs& a, int64_t item64) {
    const uint32_t NC = (uint32_t)((a.T + C - 1) / C), Hqk = (uint32_t)a.Hqk;
    const uint32_t item = (uint32_t)item64;
    MItem it;
    it.ci = item % NC;
    const uint32_t bq = item / NC;
    it.b = bq / Hqk;
    it.hq = bq % Hqk;
    return it;
}

struct MHeadRegs {
    TileRegs<float, DV, NT8> pv, pdo;
    RowRegs rr;
};

// one head's v and gates (part 0), or its dO (part 1); both parts by default
__device__ __forceinline__ void m_load_head(const RevArgs& a, const MItem& it, int64_t gi, MHeadRegs& R,
                                            int part = -1) {
    const int64_t T_ = a.T, t0 = it.ci * C;
    const int nvalid = (T_ - t0) < C ? (int)(T_ - t0) : C;
    const int64_t G = a.H / a.Hqk;
    const int64_t h = it.hq * G + gi;
    const int64_t rs_v = a.ld_v, rs_do = a.H * DV;
    const int tid = opaque_tid();
    if (part != 1) {
        R.pv.load((const float*)a.v + (it.b * T_ + t0) * rs_v + h * DV, rs_v, nvalid, tid);
        if (wave_id() == 0)
            R.rr.load((const float*)a.g + (it.b * T_ + t0) * a.H + h, a.H, a.seg, it.b, T_, t0, nvalid, true);
    }
    if (part != 0) R.pdo.load((const float*)a.dO + (it.b * T_ + t0) * rs_do + h * DV, rs_do, nvalid, tid);
}

// S0 and dS1 rows 16 (MNCT w + u) + i (value columns 32 kk + 8 j ..) of one head
// and chunk (buffer loads over the chunk's 128 x 128 fp32 state and state gradient)
struct MRows {
    f32x4 s0[MNCT][2 * DV / KS], ds[MNCT][2 * DV / KS];
};
// (part 0: the dS1 rows, part 1: the S0 rows)
__device__ __forceinline__ void m_load_rows(const RevArgs& a, const MItem& it, int64_t gi, int w, MRows& R,
                                            int part) {
    const int64_t NC = (a.T + C - 1) / C, G = a.H / a.Hqk;
    const int64_t bh = it.b * a.H + it.hq * G + gi;
    const __amdgpu_buffer_rsrc_t rS0 = buf_rsrc((const float*)a.ws_S + (bh * (NC + 1) + it.ci) * DK * DV, DK * DV * 4);
    const __amdgpu_buffer_rsrc_t rdS1 = buf_rsrc((const float*)a.ws_dS + (bh * NC + it.ci) * DK * DV, DK * DV * 4);
    const int lo = opaque_lane();
#pragma unroll
    for (int u = 0; u < MNCT; ++u) {
        const int vrow = ((16 * (MNCT * w + u) + (lo & 15)) * DV + 8 * (lo >> 4)) * 4;
#pragma unroll
        for (int kk = 0; kk < DV / KS; ++kk) {
            if (part == 1) {
                R.s0[u][2 * kk] = buf_ld4(rS0, vrow, kk * KS * 4);
                R.s0[u][2 * kk + 1] = buf_ld4(rS0, vrow, kk * KS * 4 + 16);
            } else {
                R.ds[u][2 * kk] = buf_ld4(rdS1, vrow, kk * KS * 4);
                R.ds[u][2 * kk + 1] = buf_ld4(rdS1, vrow, kk * KS * 4 + 16);
            }
        }
    }
}
__device__ __forceinline__ void m_load_qk(const RevArgs& a, const MItem& it, TileRegs<float, DK, NT8>& pq,
                                          TileRegs<float, DK, NT8>& pk) {
    const int64_t T_ = a.T, t0 = it.ci * C;
    const int nvalid = (T_ - t0) < C ? (int)(T_ - t0) : C;
    const int64_t off = (it.b * T_ + t0) * a.ld_qk + it.hq * DK;
    const int tid = opaque_tid();
    pq.load((const float*)a.q + off, a.ld_qk, nvalid, tid);
    pk.load((const float*)a.k + off, a.ld_qk, nvalid, tid);
}

__global__ __launch_bounds__(NT8) void k_grad_f32m(const RevArgs a) {
    put_stamp(a.stamp_out, a.stamp_val);  // the states the passes before this one found or stored
    __shared__ __attribute__((aligned(16))) bf16 lds[M_ELEMS];
    __shared__ RevChunk ck;
    __shared__ float sBs[MNW];
    bf16* sQ = lds;
    bf16* sK = sQ + 2 * PLQ8;
    bf16* sV = sK + 2 * PLK8;
    bf16* sAT = sV;  // [s][r], once v is no longer read
    bf16* sdO = sV + 2 * PLV8;
    bf16* sdA = sdO + 2 * PLO8;  // [r][s]
    float* sXs = reinterpret_cast<float*>(sdA);  // [waves][64 rows], once dA is no longer read

    // Lane-dependent values are taken from opaque_lane() at the start of each
    // phase: the compiler would otherwise hoist every lane-derived LDS address
    // out of the loops and hold them all in registers (hundreds of spills).
    const int64_t G = a.H / a.Hqk;
    const int w = __builtin_amdgcn_readfirstlane(wave_id());
    const int64_t T_ = a.T;
    const int64_t NC = (T_ + C - 1) / C;
    const int64_t nitems = a.B * a.Hqk * NC;
    const int64_t stride = gridDim.x;

    // loaded one head ahead: v, dO and gates; dS1 rows
    MHeadRegs hr;
    MRows rows;
    int64_t item = xcd_logical_block(gridDim.x);
    if (item < nitems) {
        const MItem it0 = m_item(a, item);
        m_load_head(a, it0, 0, hr);
        m_load_rows(a, it0, 0, w, rows, 0);
    }
    for (; item < nitems; item += stride) {
        const MItem it = m_item(a, item);
        const int64_t b = it.b, hq = it.hq, ci = it.ci;
        const int64_t t0 = ci * C;
        const int nvalid = (T_ - t0) < C ? (int)(T_ - t0) : C;
        {
            TileRegs<float, DK, NT8> pq, pk;
            m_load_qk(a, it, pq, pk);
            const int tid = opaque_tid();
            store_rows_split<DK, NT8>(pq, sQ, PQ8, PLQ8, tid);
            store_rows_split<DK, NT8>(pk, sK, PK8, PLK8, tid);
        }
        __syncthreads();

        float dqs[MNCT][4][4], dks[MNCT][4][4];  // dq, dk summed over the heads of the group
#pragma unroll
        for (int u = 0; u < MNCT; ++u)
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int e = 0; e < 4; ++e) dqs[u][rt][e] = dks[u][rt][e] = 0.f;

        for (int64_t gi = 0; gi < G; ++gi) {
            const int64_t h = hq * G + gi, bh = b * a.H + h;
            // what the loads issued during this head are for: the next head, else the
            // next item's first head, else (nothing left) this head again.  Loads are
            // unconditional: a load on one path only would keep the registers' previous
            // contents alive across the whole loop.
            int64_t nitem = item, ngi = gi + 1;
            if (ngi >= G) {
                ngi = 0;
                nitem = item + stride;
            }
            if (nitem >= nitems) {
                nitem = item;
                ngi = gi;
            }
            const MItem nx = m_item(a, nitem);
            const __amdgpu_buffer_rsrc_t rdS1 = buf_rsrc((const float*)a.ws_dS + (bh * NC + ci) * DK * DV, DK * DV * 4);
            m_load_rows(a, it, gi, w, rows, 1);  // this head's S0 rows, first needed at the end of dA
            {
                const int tid = opaque_tid();
                store_rows_split<DV, NT8>(hr.pv, sV, PV8, PLV8, tid);
                store_rows_split<DV, NT8>(hr.pdo, sdO, PO8, PLO8, tid);
            }
            if (w == 0) rev_chunk_info<float, false>(&ck, hr.rr);
            __syncthreads();
            // dS1 columns 16 (MNCT w + u) + i (channels 32 kk + 8 j ..) for dv's
            // inter-chunk term, requested soon after the rows (lines still in L2)
            float dtr[MNCT][DK / KS][8];
            {
                const int lo = opaque_lane();
#pragma unroll
                for (int u = 0; u < MNCT; ++u) {
                    const int vcol = ((8 * (lo >> 4)) * DV + 16 * (MNCT * w + u) + (lo & 15)) * 4;
#pragma unroll
                    for (int kk = 0; kk < DK / KS; ++kk)
#pragma unroll
                        for (int e = 0; e < 8; ++e) dtr[u][kk][e] = buf_ld1(rdS1, vcol, (kk * KS + e) * DV * 4);
                }
            }

            // dA^T = v dO^T tiles (computed rows s, column r), masked, stored dA[r][s];
            // dk's inter-chunk term (v dS1^T)[c][s] while v is staged, and each of this
            // lane's channels' rowsum(S0 * dS1) in fp32
            float sd[MNCT];
            f32x4 kin[MNCT][4];
            SFrag s0f[MNCT][DV / KS];
            {
                const int lo = opaque_lane();
#pragma unroll
                for (int m = 0; m < MNQK; ++m) {
                    const int ti = w + MNW * m;
                    if (ti < 10) {
                        const int rt = score_tile_rt(ti), st = score_tile_st(ti);
                        const f32x4 acc = mma3_chain<DV / KS>(zero4(), DV / KS, [&](int i, SFrag& A, SFrag& B) {
                            A = sld<PV8, PLV8>(sV, 16 * st, i * KS, lo);
                            B = sld<PO8, PLO8>(sdO, 16 * rt, i * KS, lo);
                        });
                        store_masked_split<true, PA8, PLA8>(sdA, ck, rt, st, true, acc, lo);
                    } else if (ti < 12) {
                        store_masked_split<true, PA8, PLA8>(sdA, ck, score_tile_rt(ti), score_tile_st(ti), false,
                                                            zero4(), lo);
                    }
                }
#pragma unroll
                for (int u = 0; u < MNCT; ++u) {
                    SFrag dsf[DV / KS];
#pragma unroll
                    for (int kk = 0; kk < DV / KS; ++kk) dsf[kk] = split8(rows.ds[u][2 * kk], rows.ds[u][2 * kk + 1]);
#pragma unroll
                    for (int st = 0; st < 4; ++st)
                        kin[u][st] = mma3_chain<DV / KS>(zero4(), DV / KS, [&](int i, SFrag& A, SFrag& B) {
                            A = dsf[i];
                            B = sld<PV8, PLV8>(sV, 16 * st, i * KS, lo);
                        });
                }
#pragma unroll
                for (int u = 0; u < MNCT; ++u) {
                    sd[u] = 0.f;
#pragma unroll
                    for (int kk = 0; kk < DV / KS; ++kk) {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            sd[u] += rows.s0[u][2 * kk][e] * rows.ds[u][2 * kk][e] +
                                     rows.s0[u][2 * kk + 1][e] * rows.ds[u][2 * kk + 1][e];
                        s0f[u][kk] = split8(rows.s0[u][2 * kk], rows.s0[u][2 * kk + 1]);
                    }
                }
            }
            __syncthreads();  // dA complete; v no longer read

            float xr[4] = {0.f, 0.f, 0.f, 0.f}, bb = 0.f;
            {
                const int lo = opaque_lane(), i16 = lo & 15, j4 = lo >> 4;
                // this head's masked A = q k^T tiles ti = w + MNW m (computed [r][s]:
                // rows r = 16 rt + 4 j + e, column s = 16 st + i), stored transposed
                // A^T[s][r] in v's place (q k^T is formed again per head: held across
                // the heads, its registers would be spilled)
#pragma unroll
                for (int m = 0; m < MNQK; ++m) {
                    const int ti = w + MNW * m;
                    if (ti < 10) {
                        const int rt = score_tile_rt(ti), st = score_tile_st(ti);
                        const f32x4 acc = mma3_chain<DK / KS>(zero4(), DK / KS, [&](int i, SFrag& A, SFrag& B) {
                            A = sld<PQ8, PLQ8>(sQ, 16 * rt, i * KS, lo);
                            B = sld<PK8, PLK8>(sK, 16 * st, i * KS, lo);
                        });
                        store_masked_split<false, PA8, PLA8>(sAT, ck, rt, st, true, acc, lo);
                    } else if (ti < 12) {
                        store_masked_split<false, PA8, PLA8>(sAT, ck, score_tile_rt(ti), score_tile_st(ti), false,
                                                             zero4(), lo);
                    }
                }

                // dq = dA k + fq dO S0^T and dk = dA^T q + fu (v dS1^T) for this wave's
                // channels; x_r = q dq - k dk and the boundary term over them
#pragma unroll
                for (int u = 0; u < MNCT; ++u) {
                    const int cw = 16 * (MNCT * w + u);
                    float bsum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int rt = 0; rt < 4; ++rt) {
                        const int nk = (16 * (rt + 1) + KS - 1) / KS;
                        const f32x4 a1 = mma3_chain<C / KS>(zero4(), nk, [&](int i, SFrag& A, SFrag& B) {
                            A = scol<PK8, PLK8>(sK, cw, i * KS, lo);
                            B = sld<PA8, PLA8>(sdA, 16 * rt, i * KS, lo);
                        });
                        const f32x4 a2 = mma3_chain<DV / KS>(zero4(), DV / KS, [&](int i, SFrag& A, SFrag& B) {
                            A = s0f[u][i];
                            B = sld<PO8, PLO8>(sdO, 16 * rt, i * KS, lo);
                        });
                        const int r = 16 * rt + i16;
                        const float fq = ck.fq[r];
                        const Vec4<bf16> qh = Vec4<bf16>::load(sQ + r * PQ8 + cw + 4 * j4);
                        const Vec4<bf16> ql = Vec4<bf16>::load(sQ + PLQ8 + r * PQ8 + cw + 4 * j4);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float dq = a1[e] + fq * a2[e];
                            xr[rt] += (qh.get(e) + ql.get(e)) * dq;
                            dqs[u][rt][e] += dq;
                        }
                    }
#pragma unroll
                    for (int st = 0; st < 4; ++st) {
                        const int kb = 16 * st / KS;
                        const f32x4 a1 = mma3_chain<C / KS>(zero4(), C / KS - kb, [&](int i, SFrag& A, SFrag& B) {
                            A = scol<PQ8, PLQ8>(sQ, cw, (kb + i) * KS, lo);
                            B = scol<PA8, PLA8>(sdA, 16 * st, (kb + i) * KS, lo);
                        });
                        const int s = 16 * st + i16;
                        const float fu = ck.fu[s];
                        const Vec4<bf16> kh = Vec4<bf16>::load(sK + s * PK8 + cw + 4 * j4);
                        const Vec4<bf16> kl = Vec4<bf16>::load(sK + PLK8 + s * PK8 + cw + 4 * j4);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float inter = fu * kin[u][st][e];
                            const float dk = a1[e] + inter;
                            const float kr = kh.get(e) + kl.get(e);
                            xr[st] -= kr * dk;
                            bsum[e] += kr * inter;
                            dks[u][st][e] += dk;
                        }
                    }
                    float sdu = sd[u];
                    sdu += __shfl_xor(sdu, 16, 64);
                    sdu += __shfl_xor(sdu, 32, 64);
                    // this lane group's four channels of tile u: rowsum(S1 * dS1)
#pragma unroll
                    for (int e = 0; e < 4; ++e) bb += ck.decay * __shfl(sdu, 4 * j4 + e, 64) + row_sum16(bsum[e]);
                }
                bb += __shfl_xor(bb, 16, 64);
                bb += __shfl_xor(bb, 32, 64);
            }
            __syncthreads();  // A^T complete; dA no longer read
            m_load_head(a, nx, ngi, hr);  // the next head's v, dO and gates

            {
                const int lo = opaque_lane(), i16 = lo & 15, j4 = lo >> 4;
                // dv^T = dO^T A + fu dS1^T k^T for this wave's value columns (rows n, columns s)
#pragma unroll
                for (int u = 0; u < MNCT; ++u) {
                    const int cw = 16 * (MNCT * w + u);
                    SFrag dtf[DK / KS];
#pragma unroll
                    for (int kk = 0; kk < DK / KS; ++kk)
                        dtf[kk] = split8(f32x4{dtr[u][kk][0], dtr[u][kk][1], dtr[u][kk][2], dtr[u][kk][3]},
                                         f32x4{dtr[u][kk][4], dtr[u][kk][5], dtr[u][kk][6], dtr[u][kk][7]});
                    float* dvo = (float*)a.dv + (b * T_ + t0) * a.ld_dv + h * DV + cw + 4 * j4;
#pragma unroll
                    for (int st = 0; st < 4; ++st) {
                        const int kb = 16 * st / KS;
                        const f32x4 a1 = mma3_chain<C / KS>(zero4(), C / KS - kb, [&](int i, SFrag& A, SFrag& B) {
                            A = scol<PO8, PLO8>(sdO, cw, (kb + i) * KS, lo);
                            B = sld<PA8, PLA8>(sAT, 16 * st, (kb + i) * KS, lo);
                        });
                        const f32x4 a2 = mma3_chain<DK / KS>(zero4(), DK / KS, [&](int i, SFrag& A, SFrag& B) {
                            A = dtf[i];
                            B = sld<PK8, PLK8>(sK, 16 * st, i * KS, lo);
                        });
                        const int s = 16 * st + i16;
                        const float fu = ck.fu[s];
                        float dv[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) dv[e] = a1[e] + fu * a2[e];
                        if (s < nvalid) store4<float>(dvo + (int64_t)s * a.ld_dv, dv);
                    }
                }
                // the next head's dS1 rows
                m_load_rows(a, nx, ngi, w, rows, 0);
                // per-row x sums of this wave's channels, and its boundary sum
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    float y = xr[rt];
                    y += __shfl_xor(y, 16, 64);
                    y += __shfl_xor(y, 32, 64);
                    if (j4 == 0) sXs[w * C + 16 * rt + i16] = y;
                }
                if (lo == 0) sBs[w] = bb;
            }
            __syncthreads();  // also: every wave is done with this head's A^T, dO and ck
            if (w == 0) {
                // the scalar log-gate gradient of this head's chunk: dg[u] = the sum of x
                // over rows t >= u of u's document, plus the boundary term on the last row
                // (it reaches the rows of the chunk's last document); 0 at reset rows
                const int lo = opaque_lane();
                float tot = 0.f, bt = 0.f;
#pragma unroll
                for (int u = 0; u < MNW; ++u) {
                    tot += sXs[u * C + lo];
                    bt += sBs[u];
                }
                const int doc = ck.doc[lo];
                const int prev = __shfl_up(doc, 1, 64);
                const int reset = doc - (lo > 0 ? prev : 0);  // (doc counts the resets up to row lo)
                float run = (lo < nvalid ? tot : 0.f) + (lo == nvalid - 1 ? bt : 0.f);
#pragma unroll
                for (int d = 1; d < C; d <<= 1) {
                    const float y = __shfl_down(run, d, 64);
                    const int dd = __shfl_down(doc, d, 64);
                    if (lo + d < C && dd == doc) run += y;
                }
                if (lo < nvalid) ((float*)a.dg)[(b * T_ + t0 + lo) * a.H + h] = reset ? 0.f : run;
            }
        }
        {
            const int lo = opaque_lane(), i16 = lo & 15, j4 = lo >> 4;
#pragma unroll
            for (int u = 0; u < MNCT; ++u)
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    const int r = 16 * rt + i16;
                    if (r < nvalid) {
                        const int64_t o = (b * T_ + t0 + r) * a.ld_dqk + hq * DK + 16 * (MNCT * w + u) + 4 * j4;
                        store4<float>((float*)a.dq + o, dqs[u][rt]);
                        store4<float>((float*)a.dk + o, dks[u][rt]);
                    }
                }
        }
    }
}

}  // namespace

hipError_t launch_grad_f32s(const RevArgs& a, hipStream_t st) {
    const int64_t NC = (a.T + C - 1) / C;
    const int64_t n = a.B * a.Hqk * NC;
    // persistent: one workgroup per compute unit (the LDS allows no more)
    const int64_t workers = 256;
    hipLaunchKernelGGL(k_grad_f32m, dim3((unsigned)(n < workers ? n : workers)), dim3(NT8), 0, st, a);
    return hipGetLastError();
}

}  // namespace gla
