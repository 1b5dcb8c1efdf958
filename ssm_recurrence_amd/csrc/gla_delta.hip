// gla_delta.hip -- the gated delta rule (Gated DeltaNet), chunked WY/UT form,
// forward and backward (gfx950).
//
// Recurrence (the published Gated DeltaNet update, in this library's state
// orientation, S d_k x d_v and o = S^T q):
//     S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,   o_t = S_t^T q_t,
// alpha_t = exp(g_t), with the document resets of the gated linear attention.
// The pages name it (FLAT page, "FLAT: Flash Linear Attention on TPUs",
// Conclusion, future work 1; probjax page, "GPU kernels", section Gated
// DeltaNet: a chunked WY/UT form whose backward keeps only chunk-boundary
// states) without writing it out.
//
// Chunked form, per chunk of C = 64 rows with entry state S0, Gamma_t the
// chunk-local cumulative log gate (restarting at each document start, the
// reset row's own gate unused), gamma_t = exp(Gamma_t) for rows the entry
// state reaches (else 0), E_ts = exp(Gamma_t - Gamma_s) within a document:
//     A  = strictly lower part of diag(beta) (K K^T (.) E)
//     T  = (I + A)^-1                      (unit lower triangular)
//     U  = T (beta (.) V),   W = T (beta gamma (.) K)
//     Wv = U - W S0                        (the rows' effective writes)
//     O  = (gamma (.) Q) S0 + ((Q K^T) (.) M) Wv      (M: E with the diagonal)
//     S1 = c S0 + Kt^T Wv,   c = exp(Gamma_last) when the chunk has no reset
//          (else 0), Kt_s = exp(Gamma_last - Gamma_s) k_s on the last document.
// It follows from unrolling the recurrence over the chunk: the write of row t
// is beta_t (v_t - S_{t-1}^T k_t), and S_{t-1} is the decayed S0 plus the
// decayed earlier writes.
//
// Kernels (products on the fp32 matrix cores, operands staged through LDS; the
// Gram matrix K K^T of bf16 inputs on the bf16 matrix cores, exact products):
//   k_delta_prep   per (b, h, chunk): the row prologue, T, U, W, the masked
//                  scores P = (Q K^T) (.) M, gamma (.) Q, Kt, c.
//   k_delta_state  per (b, h, 16 value columns): the chunks in order; o and hT,
//                  or (backward) S0 and Wv of every chunk.
//   k_delta_dstate per (b, h, 16 value columns): the chunks in reverse; the
//                  state gradient at every chunk's end and dWv, then dh0:
//                  dWv = P^T dO + Kt dS1,  dS0 = c dS1 + (gamma (.) Q)^T dO - W^T dWv.
//   k_delta_grad   per (b, h, chunk): dq, dk, dv, dg, dbeta by reverse mode
//                  through the chunk's steps (dA = -T^T dT T^T for the inverse).
#include "gla_common.hpp"
#include "gla_kernels.hpp"

namespace gla {

namespace {

constexpr int DC = 64;     // rows per chunk
constexpr int DTH = 512;   // threads per workgroup (8 waves)
constexpr int NSL = 16;    // value columns per workgroup of the sequential passes
constexpr int LP = 65;     // LDS pitch of 64 x 64 matrices

// C(i, j) = alpha * si[i] * sj[j] * sum_k A(i, k) B(k, j) + beta * C(i, j) for
// i < M, j < N, with A(i, k) = A[i*ai + k*ak], B(k, j) = B[k*bk + j*bj] and
// C(i, j) = C[i*ci + j*cj], for operands in global memory (L2) or LDS (si, sj
// optional): k is taken in tiles of KT; each tile of A (M x KT) and B (KT x N)
// is loaded by the whole workgroup
// with the unit-stride index running across lanes, written to LDS, and the
// next tile's loads are issued before the current tile is used; the products run
// on the fp32 matrix cores.  M, N <= 128 and M N <= 128 x 64: at most four 16 x 16
// output tiles per wave (fewer accumulators and less unrolled code in each of the
// kernel's inlined calls).  `lds` holds MMT_LDS floats.  Contains barriers: every
// thread of the workgroup calls it.
// LDS serves a wave's 32-bit reads in two halves of 32 lanes over 32 banks.  The
// A tile's pitch is 2 mod 32 (a fragment's half reads 16 rows x 2 columns), the
// B tile's 16 mod 32 (16 columns x 2 rows): each half-wave read hits 32 banks.
constexpr int KT = 32, PA = KT + 2, PB = 128 + 16, MMT_LDS = 128 * PA + KT * PB, LDE = 128 * KT / DTH;
template <typename TA, typename TB>
__device__ __forceinline__ void mmt(int M, int N, int K, float alpha, const TA* A, int64_t ai64, int64_t ak64, const TB* B,
                    int64_t bk64, int64_t bj64, float beta, float* C, int64_t ci, int64_t cj, float* lds,
                    const float* sj = nullptr, const float* si = nullptr) {
    // (offsets within one chunk's operands fit in 32 bits)
    const int ai = (int)ai64, ak = (int)ak64, bk = (int)bk64, bj = (int)bj64;
    float* sa = lds;              // [128][PA]: sa[i][kk]
    float* sb = lds + 128 * PA;   // [KT][PB]: sb[kk][j]
    const int tid = threadIdx.x;
    const bool a_i_fast = ai == 1 && ak != 1;  // unit stride along i: lanes run along i
    const bool b_k_fast = bk == 1 && bj != 1;
    // element e of a 128 x KT tile: (row, k) with the unit-stride index fastest
    auto a_ik = [&](int e, int& i, int& kk) {
        if (a_i_fast) { i = e & 127; kk = e >> 7; } else { i = e / KT; kk = e % KT; }  // (e < 128 KT)
    };
    auto b_jk = [&](int e, int& j, int& kb) {
        if (b_k_fast) { j = e / KT; kb = e % KT; } else { j = e & 127; kb = e >> 7; }
    };
    float ra[LDE], rb[LDE];
    auto fetch = [&](int k0) {
#pragma unroll
        for (int r = 0; r < LDE; ++r) {
            const int e = tid + r * DTH;
            int i, kk, j, kb;
            a_ik(e, i, kk);
            b_jk(e, j, kb);
            ra[r] = (i < M && k0 + kk < K) ? to_f32(A[i * ai + (k0 + kk) * ak]) : 0.f;
            rb[r] = (j < N && k0 + kb < K) ? to_f32(B[(k0 + kb) * bk + j * bj]) : 0.f;
        }
    };
    auto stash = [&]() {
#pragma unroll
        for (int r = 0; r < LDE; ++r) {
            const int e = tid + r * DTH;
            int i, kk, j, kb;
            a_ik(e, i, kk);
            b_jk(e, j, kb);
            if (i < M) sa[i * PA + kk] = ra[r];
            if (j < N) sb[kb * PB + j] = rb[r];
        }
    };
    // 16 x 16 output tiles on the fp32 matrix cores (full fp32 products and
    // sums); wave w takes tiles w, w + 8, ...  Rows past M and columns past N of
    // the LDS tiles hold stale values; they only reach outputs that are dropped.
    const int wv = tid >> 6, l = tid & 63;
    const int nti = (M + 15) / 16, ntj = (N + 15) / 16, ntiles = nti * ntj;
    constexpr int TPW = 128 * 64 / 256 / (DTH / 64);  // tiles per wave at most
    f32x4 acc[TPW];
#pragma unroll
    for (int q = 0; q < TPW; ++q) acc[q] = zero4();
    fetch(0);
#pragma unroll 1
    for (int k0 = 0; k0 < K; k0 += KT) {
        __syncthreads();  // the previous tile is no longer read
        stash();
        __syncthreads();
        if (k0 + KT < K) fetch(k0 + KT);
#pragma unroll
        for (int q = 0; q < TPW; ++q) {
            const int t = wv + q * (DTH / 64);
            if (t < ntiles) {
                const int i0 = (t / ntj) * 16, j0 = (t % ntj) * 16;
#pragma unroll
                for (int kk = 0; kk < KT; kk += 4)
                    acc[q] = Mma<float>::mma(frag_ld<float, PA, 1>(sa, i0, kk),
                                             frag_ld<float, 1, PB>(sb, j0, kk), acc[q]);
            }
        }
    }
    // C layout: lane l holds rows 4 (l / 16) + e, column l % 16 of its tile
#pragma unroll
    for (int q = 0; q < TPW; ++q) {
        const int t = wv + q * (DTH / 64);
        if (t < ntiles) {
            const int i0 = (t / ntj) * 16 + 4 * (l >> 4), j = (t % ntj) * 16 + (l & 15);
            float old[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                old[e] = beta != 0.f && i0 + e < M && j < N ? C[(i0 + e) * ci + j * cj] : 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = i0 + e;
                if (i < M && j < N) {
                    const float v = alpha * acc[q][e] * (sj ? sj[j] : 1.f) * (si ? si[i] : 1.f);
                    C[i * ci + j * cj] = beta != 0.f ? v + beta * old[e] : v;
                }
            }
        }
    }
    __syncthreads();  // (lds free for the next call)
}

// st(i, ld(i)) for i < n over the workgroup, EB elements per thread at a time
// with all EB loads issued before the stores (a store through one pointer
// would otherwise keep the next load, through another, from being issued early).
template <int EB = 8, typename L, typename S>
__device__ __forceinline__ void ew(int n, L ld, S st) {
#pragma unroll 1
    for (int base = threadIdx.x; base < n; base += EB * DTH) {
        float v[EB];
#pragma unroll
        for (int u = 0; u < EB; ++u) {
            const int i = base + u * DTH;
            v[u] = i < n ? ld(i) : 0.f;
        }
#pragma unroll
        for (int u = 0; u < EB; ++u) {
            const int i = base + u * DTH;
            if (i < n) st(i, v[u]);
        }
    }
}

// out[t] += sign * sum_d X[t*lx + d] Y[t*ly + d] for t < n (D <= 128): wave w
// takes rows w, w + 8, ...; all of a wave's loads are issued before its sums.
template <typename TX, typename TY>
__device__ __forceinline__ void rowdot(int n, int D, const TX* X, int64_t lx, const TY* Y, int64_t ly, float* out,
                                       float sign) {
    constexpr int NWV = DTH / 64, RPW = DC / NWV;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    float x[RPW][2], y[RPW][2];
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
        const int t = wv + r * NWV;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int d = lane + 64 * h;
            const bool ok = t < n && d < D;
            x[r][h] = ok ? to_f32(X[t * lx + d]) : 0.f;
            y[r][h] = ok ? to_f32(Y[t * ly + d]) : 0.f;
        }
    }
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
        float s = x[r][0] * y[r][0] + x[r][1] * y[r][1];
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m, 64);
        const int t = wv + r * NWV;
        if (lane == 0 && t < n) out[t] += sign * s;
    }
}

// Per-chunk row data in LDS
struct Rows {
    float G[DC];     // Gamma_t (document-local cumulative log gate)
    float gam[DC];   // gamma_t: exp(Gamma_t) where the entry state reaches row t, else 0
    float kts[DC];   // exp(Gamma_last - Gamma_s) on the last document, else 0
    float beta[DC];  // beta_t (0 past the end)
    float bg[DC];    // beta_t gamma_t
    int doc[DC];     // document index within the chunk (resets at or before t)
    int reset[DC];
    float carry;     // c: exp(Gamma_last) when the chunk has no reset, else 0
    int n;           // valid rows
};

// Row prologue (wave 0).  g, beta: [B][T][H]; seg: [B][T] or null.
template <typename T>
__device__ __forceinline__ void prologue(Rows& R, const DeltaArgs& a, int64_t b, int64_t h, int64_t t0) {
    if (threadIdx.x >= 64) return;
    const int t = threadIdx.x;
    const int64_t T_ = a.T;
    const int n = (int)(T_ - t0 < DC ? T_ - t0 : DC);
    const bool valid = t < n;
    const int64_t row = b * T_ + t0 + t;
    const bool rs = valid && t0 + t > 0 && a.seg && a.seg[row] != a.seg[row - 1];
    const float gl = valid && !rs ? to_f32(((const T*)a.g)[row * a.H + h]) : 0.f;
    const float bt = valid ? to_f32(((const T*)a.beta)[row * a.H + h]) : 0.f;
    const uint64_t mask = __ballot(rs);
    const uint64_t upto = t == 63 ? ~0ull : ((2ull << t) - 1);
    const int doc = __popcll(mask & upto);
    // inclusive prefix of the gates, then restarted at the document's first row
    float p = gl;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
        const float o = __shfl_up(p, m, 64);
        if (t >= m) p += o;
    }
    const uint64_t before = mask & upto;
    const int start = before ? 63 - __clzll(before) : 0;
    const float pstart = __shfl(p, start, 64);
    const float G = doc > 0 ? p - pstart : p;  // (the reset row's own gate is 0)
    const int last = n - 1;
    const float Glast = __shfl(G, last > 0 ? last : 0, 64);
    const int doclast = __shfl(doc, last > 0 ? last : 0, 64);
    R.G[t] = G;
    R.doc[t] = valid ? doc : -1;
    R.reset[t] = rs;
    R.beta[t] = bt;
    R.gam[t] = valid && doc == 0 ? __expf(G) : 0.f;
    R.bg[t] = bt * R.gam[t];
    R.kts[t] = valid && doc == doclast ? __expf(Glast - G) : 0.f;
    if (t == 0) {
        R.carry = doclast == 0 ? __expf(Glast) : 0.f;
        R.n = n;
    }
}

__device__ __forceinline__ float decay(const Rows& R, int t, int s) {  // E / M entry, s <= t
    return R.doc[t] >= 0 && R.doc[t] == R.doc[s] ? __expf(R.G[t] - R.G[s]) : 0.f;
}

// K tile in LDS.  bf16: rows 16 bytes apart plus 16 (whole 16-byte fragments
// for the matrix cores, rows spread over the banks); fp32: an odd number of
// dwords apart (a column read across lanes is free of bank conflicts).
template <typename T> constexpr int kpad() { return sizeof(T) == 2 ? 8 : 1; }
template <typename T> __device__ __forceinline__ int kpitch(int D) { return D + kpad<T>(); }

// the chunk's K rows into LDS (rows past n zero)
template <typename T>
__device__ __forceinline__ void load_k(const Rows& R, const T* K, int64_t rs, int D, T* sK) {
    const int KP = kpitch<T>(D), n = R.n;
    ew(DC * D, [&](int i) { const int t = i / D; return t < n ? to_f32(K[t * rs + i % D]) : 0.f; },
       [&](int i, float v) { sK[(i / D) * KP + i % D] = from_f32<T>(v); });
}

// G = K K^T (64 x 64, all rows; rows past n are zero in sK) on the matrix cores:
// 16 tiles of 16 x 16, K fragments read straight from the LDS tile.
template <typename T, int D>
__device__ __forceinline__ void gram_mfma(const T* sK, float* sG) {
    constexpr int KP = D + kpad<T>();
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    for (int t = w; t < 16; t += DTH / 64) {
        const int i0 = (t >> 2) * 16, j0 = (t & 3) * 16;
        f32x4 acc = zero4();
#pragma unroll
        for (int k0 = 0; k0 < D; k0 += Mma<T>::KSTEP)
            acc = Mma<T>::mma(frag_ld<T, KP, 1>(sK, i0, k0), frag_ld<T, KP, 1>(sK, j0, k0), acc);
#pragma unroll
        for (int e = 0; e < 4; ++e) sG[(i0 + 4 * (l >> 4) + e) * LP + j0 + (l & 15)] = acc[e];
    }
}

// GE = (K K^T) (.) E strictly below the diagonal (LDS, pitch LP), and
// T = (I + diag(beta) GE)^-1 by forward substitution (lane j builds column j).
// sK: the chunk's K rows (load_k), complete before the call.
template <typename T, int D>
__device__ __forceinline__ void gram_masked(const Rows& R, const T* sK, float* sGE) {
    gram_mfma<T, D>(sK, sGE);
    __syncthreads();
    for (int i = threadIdx.x; i < DC * DC; i += DTH) {
        const int t = i / DC, s = i % DC;
        sGE[t * LP + s] = s < t ? sGE[t * LP + s] * decay(R, t, s) : 0.f;
    }
    __syncthreads();
}

template <typename T, int D>
__device__ __forceinline__ void wy_inverse(const Rows& R, const T* sK, float* sGE, float* sT) {
    gram_masked<T, D>(R, sK, sGE);
    if (threadIdx.x < DC) {
        // lane j keeps column j of T in registers; row i of GE is read as a
        // broadcast (every lane reads the same address)
        const int j = threadIdx.x;
        float tc[DC];
#pragma unroll
        for (int i = 0; i < DC; ++i) {
            float acc = 0.f;
#pragma unroll
            for (int m = 0; m < i; ++m) acc += sGE[i * LP + m] * tc[m];
            tc[i] = (i == j ? 1.f : 0.f) - R.beta[i] * acc;
        }
#pragma unroll
        for (int i = 0; i < DC; ++i) sT[i * LP + j] = tc[i];
    }
    __syncthreads();
}

// per-chunk workspace blocks (fp32): the forward's factors T .. carry (written
// by the prepare pass only) in ws, the backward's intermediates S0 .. gKb in ws2
struct ChunkWs {
    float *T, *U, *W, *P, *Qg, *Kt, *carry, *S0, *Wv, *dS1, *dWv, *gQ, *gW, *gKb;
};

__device__ __forceinline__ ChunkWs chunk_ws(const DeltaArgs& a, int64_t chunk) {
    const int64_t D = a.dk, Dv = a.dv;
    float* p = a.ws + chunk * a.ws_chunk;
    ChunkWs w;
    w.T = p; p += DC * DC;
    w.U = p; p += DC * Dv;
    w.W = p; p += DC * D;
    w.P = p; p += DC * DC;
    w.Qg = p; p += DC * D;
    w.Kt = p; p += DC * D;
    w.carry = p; p += 4;
    // S0 and Wv: in ws after the factors (states_in_ws), else first in ws2
    // (ws2 is null in the forward)
    float* q = a.ws2 + chunk * a.ws2_chunk;
    float* st = a.states_in_ws ? p : q;
    w.S0 = st;
    w.Wv = st + D * Dv;
    p = a.states_in_ws ? q : q + D * Dv + DC * Dv;
    w.dS1 = p; p += D * Dv;
    w.dWv = p; p += DC * Dv;
    w.gQ = p; p += DC * D;   // (fp32 inputs; bf16 inputs keep dQ in LDS)
    w.gW = p; p += DC * D;
    w.gKb = p; p += DC * D;
    return w;
}

// fp32 matrix-core operand fragment (lane i = l % 16, k = l / 16) from an LDS
// tile of any element type: X(i0 + i, k0 + k), X(i, k) = base[i*SI + k*SK]
template <int SI, int SK, typename TX>
__device__ __forceinline__ float frag_f32(const TX* base, int i0, int k0) {
    const int l = threadIdx.x & 63;
    return to_f32(base[(i0 + (l & 15)) * SI + (k0 + (l >> 4)) * SK]);
}

template <int M, int N, int K, int SIA, int SKA, int SIB, int SKB, int CI, int WB = 0, int NWV = DTH / 64,
          typename TA, typename TB>
__device__ __forceinline__ void mm_lds(float alpha, const TA* A, const TB* B, float beta, float* C) {
    constexpr int NTJ = N / 16, NTILES = (M / 16) * NTJ;
    const int wv = (int)(threadIdx.x >> 6) - WB, l = threadIdx.x & 63;
    if (wv < 0 || wv >= NWV) return;
#pragma unroll
    for (int t0 = 0; t0 < NTILES; t0 += NWV) {
        const int t = t0 + wv;
        if (t < NTILES) {
            const int i0 = (t / NTJ) * 16, j0 = (t % NTJ) * 16;
            f32x4 acc = zero4();
#pragma unroll 8
            for (int k0 = 0; k0 < K; k0 += 4)
                acc = Mma<float>::mma(frag_f32<SIA, SKA>(A, i0, k0), frag_f32<SIB, SKB>(B, j0, k0), acc);
            const int r0 = i0 + 4 * (l >> 4), j = j0 + (l & 15);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float* c = C + (r0 + e) * CI + j;
                *c = beta != 0.f ? alpha * acc[e] + beta * *c : alpha * acc[e];
            }
        }
    }
}

// ---------------------------------------------------------------- prepare
// (d_k = DK, d_v = DV fixed per instance: one kernel's code holds one shape)
template <typename T, int DK, int DV>
__global__ __launch_bounds__(DTH) void k_delta_prep(const DeltaArgs a) {
    __shared__ Rows R;
    __shared__ float sGE[DC * LP], sT[DC * LP];
    __shared__ __attribute__((aligned(16))) T sK[DC * (128 + kpad<T>())];
    __shared__ __attribute__((aligned(16))) T sQ[DC * (128 + kpad<T>())];
    T* sV = sQ;  // (V takes Q's place once gamma Q is written)
    const int64_t NC = (a.T + DC - 1) / DC;
    const int64_t chunk = blockIdx.x, bh = chunk / NC, c = chunk % NC;
    const int64_t b = bh / a.H, h = bh % a.H, t0 = c * DC;
    constexpr int D = DK, Dv = DV;
    const int KP = kpitch<T>(D);
    const int64_t rk = a.H * D, rv = a.H * Dv;
    const T* Q = (const T*)a.q + (b * a.T + t0) * rk + h * D;
    const T* K = (const T*)a.k + (b * a.T + t0) * rk + h * D;
    const T* V = (const T*)a.v + (b * a.T + t0) * rv + h * Dv;
    // the workspace already holds these factors when its stamp is this call's
    if (a.check_stamp && stamp_matches(a.stamp, a.expect)) return;
    prologue<T>(R, a, b, h, t0);
    __syncthreads();
    const int n = R.n;
    load_k<T>(R, K, rk, D, sK);
    load_k<T>(R, Q, rk, D, sQ);  // (the same row loader)
    __syncthreads();
    wy_inverse<T, DK>(R, sK, sGE, sT);
    ChunkWs w = chunk_ws(a, chunk);
    // T (whole 64 x 64), c
    for (int i = threadIdx.x; i < DC * DC; i += DTH) w.T[i] = sT[(i / DC) * LP + i % DC];
    if (threadIdx.x == 0) w.carry[0] = R.carry;
    __syncthreads();
    // P = (Q K^T) (.) M in sGE (reused), then copied whole; rows past n are zero
    // in both tiles
    if constexpr (DK == 128)
        mm_lds<DC, DC, 128, 128 + kpad<T>(), 1, 128 + kpad<T>(), 1, LP>(1.f, sQ, sK, 0.f, sGE);
    else
        mm_lds<DC, DC, 64, 64 + kpad<T>(), 1, 64 + kpad<T>(), 1, LP>(1.f, sQ, sK, 0.f, sGE);
    __syncthreads();
    for (int i = threadIdx.x; i < DC * DC; i += DTH) {
        const int t = i / DC, s = i % DC;
        w.P[i] = s <= t ? sGE[t * LP + s] * decay(R, t, s) : 0.f;
    }
    // gamma (.) Q and Kt, whole 64 rows
    ew(DC * D, [&](int i) { const int t = i / D; return t < n ? R.gam[t] * to_f32(sQ[t * KP + i % D]) : 0.f; },
       [&](int i, float v) { w.Qg[i] = v; });
    ew(DC * D, [&](int i) { const int t = i / D; return t < n ? R.kts[t] * to_f32(sK[t * KP + i % D]) : 0.f; },
       [&](int i, float v) { w.Kt[i] = v; });
    __syncthreads();
    load_k<T>(R, V, rv, Dv, sV);
    // U = T (beta V), W = T (beta gamma K), with beta and beta gamma folded into the
    // columns of T; rows past n are 0 (T is the identity there and beta is 0)
    for (int i = threadIdx.x; i < DC * DC; i += DTH) {
        const int t = i / DC, s = i % DC;
        sGE[t * LP + s] = sT[t * LP + s] * R.bg[s];
        sT[t * LP + s] *= R.beta[s];
    }
    __syncthreads();
    if constexpr (DV == 128)
        mm_lds<DC, 128, DC, LP, 1, 1, 128 + kpad<T>(), 128>(1.f, sT, sV, 0.f, w.U);
    else
        mm_lds<DC, 64, DC, LP, 1, 1, 64 + kpad<T>(), 64>(1.f, sT, sV, 0.f, w.U);
    if constexpr (DK == 128)
        mm_lds<DC, 128, DC, LP, 1, 1, 128 + kpad<T>(), 128>(1.f, sGE, sK, 0.f, w.W);
    else
        mm_lds<DC, 64, DC, LP, 1, 1, 64 + kpad<T>(), 64>(1.f, sGE, sK, 0.f, w.W);
}

// ---------------------------------------------------------------- sequential passes
// The operands a chunk needs are staged through registers: the next chunk's
// values are loaded while the current chunk computes, then written to LDS.
// Registers hold the segments back to back (W [64][D], Kt [64][D], then (QP)
// gamma Q [64][D] and P [64][64], then a [64][16] column slice: U, or dO); each
// register (vector) holds consecutive elements of one segment's row.  In LDS each segment's row pitch is padded for the way the
// products read it (32-bit reads are served in two halves of 32 lanes over 32
// banks): a segment read as 16 rows x 4 columns per fragment (A(i, k) = X[i][k])
// gets pitch = 2 mod 32 dwords, one read as 16 columns x 4 rows (A(i, k) =
// X[k][i]) gets 16 mod 32, so that each half of a fragment read hits 32 distinct
// banks.  REV is the reverse pass, which reads W, gamma Q and P by columns and Kt
// by rows; the forward state pass reads them the other way.
template <int D, bool QP, bool REV> struct SeqLayout {
    static constexpr int RP = D + 2, CP = D + 16;
    static constexpr int PW = REV ? CP : RP, PK = REV ? RP : CP, PQ = REV ? CP : RP;
    static constexpr int PP = REV ? DC + 16 : DC + 2;
    static constexpr int NW = DC * D, NPP = DC * DC, NS = DC * NSL;
    // register (unpadded) offsets
    static constexpr int UKT = NW, UQG = 2 * NW, UP = QP ? 3 * NW : 2 * NW, USL = QP ? UP + NPP : UP;
    // LDS (padded) offsets
    static constexpr int W = 0, KT_ = DC * PW, QG = KT_ + DC * PK;
    static constexpr int P = QP ? QG + DC * PQ : QG;
    static constexpr int SL = QP ? P + DC * PP : P;
    static constexpr int TOTAL = SL + NS;
    static_assert(NW % DTH == 0 && NPP % DTH == 0 && NS % DTH == 0, "segments");
};

// g[(j0 + j) * R + r] = s[r * NSL + j] for an [R][NSL] LDS slice: each wave
// instruction reads 16 rows x 4 columns (half as many bank repeats as 64
// consecutive rows) and writes 64-byte runs
template <int R>
__device__ __forceinline__ void store_transposed(const float* s, float* g, int64_t j0) {
    for (int i = threadIdx.x; i < R * NSL; i += DTH) {
        const int l = i & 63, q = i >> 6;
        const int j = (q & 3) * 4 + (l >> 4), r = (q >> 2) * 16 + (l & 15);
        g[(j0 + j) * R + r] = s[r * NSL + j];
    }
}

// The prefetch registers: the four [64][D] / [64][64] segments as 16-byte
// vectors (each segment is a multiple of 4 x DTH floats and starts 16-byte
// aligned: the workspace is, and every segment size is a multiple of 4 floats),
// then the [64][16] slice one float at a time.
template <int D, bool QP> struct SeqRegs {
    using L = SeqLayout<D, QP, false>;
    static constexpr int NV = L::USL / (4 * DTH), NSS = L::NS / DTH;
    static_assert(L::USL % (4 * DTH) == 0 && L::NW % (4 * DTH) == 0 && L::NPP % (4 * DTH) == 0, "segments");
    f32x4 v[NV];
    float s[NSS];
};

// slice(row, col) gives the [64][16] slice's element (row < 64)
template <int D, bool QP, typename SliceF>
__device__ __forceinline__ void seq_fetch(SeqRegs<D, QP>& pf, const ChunkWs& w, SliceF slice) {
    using L = SeqLayout<D, QP, false>;  // (register offsets only)
#pragma unroll
    for (int u = 0; u < SeqRegs<D, QP>::NV; ++u) {
        const int e = 4 * (u * DTH + (int)threadIdx.x), e0 = 4 * u * DTH;
        const float* src;
        if (e0 < L::UKT) src = w.W + e;
        else if (e0 < L::UQG) src = w.Kt + (e - L::UKT);
        else if (QP && e0 < L::UP) src = w.Qg + (e - L::UQG);
        else src = w.P + (e - L::UP);
        pf.v[u] = *reinterpret_cast<const f32x4*>(src);
    }
#pragma unroll
    for (int u = 0; u < SeqRegs<D, QP>::NSS; ++u) {
        const int e = u * DTH + (int)threadIdx.x;
        pf.s[u] = slice(e / NSL, e % NSL);
    }
}

template <int D, bool QP, bool REV>
__device__ __forceinline__ void seq_stash(const SeqRegs<D, QP>& pf, float* sBuf) {
    using L = SeqLayout<D, QP, REV>;
#pragma unroll
    for (int u = 0; u < SeqRegs<D, QP>::NV; ++u) {
        const int e = 4 * (u * DTH + (int)threadIdx.x), e0 = 4 * u * DTH;
        int a;  // (four consecutive columns of one row)
        if (e0 < L::UKT) a = L::W + (e / D) * L::PW + e % D;
        else if (e0 < L::UQG) a = L::KT_ + ((e - L::UKT) / D) * L::PK + (e - L::UKT) % D;
        else if (QP && e0 < L::UP) a = L::QG + ((e - L::UQG) / D) * L::PQ + (e - L::UQG) % D;
        else a = L::P + ((e - L::UP) / DC) * L::PP + (e - L::UP) % DC;
#pragma unroll
        for (int q = 0; q < 4; ++q) sBuf[a + q] = pf.v[u][q];
    }
#pragma unroll
    for (int u = 0; u < SeqRegs<D, QP>::NSS; ++u) {
        const int e = u * DTH + (int)threadIdx.x;
        sBuf[L::SL + e] = pf.s[u];
    }
}

// C (M x N) = alpha A B + beta C with A and B in LDS (fp32 or bf16, converted
// exactly), on the fp32 matrix cores: A(i, k) = A[i*SIA + k*SKA], B(k, j) =
// B[k*SKB + j*SIB], C(i, j) = C[i*CI + j] (LDS or global); M, N multiples of 16,
// K of 4.  Waves WB .. WB + NWV - 1 take part: wave WB + w computes tiles w,
// w + NWV, ...; the other waves return at once (no barrier inside).  Each output
// element is read (beta) and written by one lane only.
// state pass (chunks in order): o and hT (and, when they live in ws, S0 and Wv of
// every chunk for the backward), or (BWD) S0 and Wv of every chunk; the backward's
// pass exits at once when ws holds them for these inputs
template <typename T, bool BWD, int D>
__global__ __launch_bounds__(DTH) void k_delta_state(const DeltaArgs a) {
    using L = SeqLayout<D, !BWD, false>;
    __shared__ float sBuf[L::TOTAL];
    __shared__ float sS[D * NSL], sWv[DC * NSL], sO[DC * NSL];
    if constexpr (BWD) {
        if (a.check_stamp && a.states_in_ws && stamp_matches(a.stamp, a.expect)) return;
    } else if (a.put_stamp) {
        put_stamp(a.stamp, a.expect);  // what the prepare pass and this one store
    }
    const bool keep = BWD || a.states_in_ws;  // S0 and Wv stored
    const int Dv = (int)a.dv;
    const int nsl = Dv / NSL;
    const int64_t lb = xcd_logical_block(gridDim.x);  // the slices of one head share an XCD's L2
    const int64_t bh = lb / nsl, j0 = (lb % nsl) * NSL;
    const int64_t b = bh / a.H, h = bh % a.H;
    const int64_t NC = (a.T + DC - 1) / DC;
    for (int i = threadIdx.x; i < D * NSL; i += DTH) {
        const int r = i / NSL, j = i % NSL;
        sS[i] = a.h0 ? a.h0[(bh * D + r) * Dv + j0 + j] : 0.f;
    }
    SeqRegs<D, !BWD> pf;
    float carry_next;
    auto fetch = [&](int64_t c) {
        const ChunkWs w = chunk_ws(a, bh * NC + c);
        seq_fetch<D, !BWD>(pf, w, [&](int r, int j) { return w.U[r * Dv + j0 + j]; });
        carry_next = w.carry[0];
    };
    fetch(0);
    int64_t t0_prev = 0;
    int n_prev = 0;
    // o of the previous chunk: sO is complete after the loop's first barrier and
    // rewritten only after its second
    auto store_o = [&]() {
        T* o = (T*)a.o + (b * a.T + t0_prev) * a.H * Dv + h * Dv + j0;
        for (int i = threadIdx.x; i < n_prev * NSL; i += DTH)
            o[(i / NSL) * a.H * Dv + i % NSL] = from_f32<T>(sO[i]);
    };
    for (int64_t c = 0; c < NC; ++c) {
        const ChunkWs w = chunk_ws(a, bh * NC + c);
        const int64_t t0 = c * DC;
        const int n = (int)(a.T - t0 < DC ? a.T - t0 : DC);
        const float carry = carry_next;
        __syncthreads();  // (the previous chunk no longer reads sBuf; sS and sO are complete)
        if (!BWD && c > 0) store_o();
        seq_stash<D, !BWD, false>(pf, sBuf);
        if (keep)
            store_transposed<D>(sS, w.S0, j0);  // S0 transposed: [value column][key row]
        __syncthreads();
        // Wv = U - W S0 on waves 0-3; in the forward, O = (gamma Q) S0 on waves 4-7
        for (int i = threadIdx.x; i < DC * NSL; i += DTH) sWv[i] = sBuf[L::SL + i];
        __syncthreads();
        mm_lds<DC, NSL, D, L::PW, 1, 1, NSL, NSL, 0, 4>(-1.f, sBuf + L::W, sS, 1.f, sWv);
        if (!BWD) mm_lds<DC, NSL, D, L::PQ, 1, 1, NSL, NSL, 4, 4>(1.f, sBuf + L::QG, sS, 0.f, sO);
        __syncthreads();
        if (c + 1 < NC) fetch(c + 1);
        if (keep)
            store_transposed<DC>(sWv, w.Wv, j0);  // Wv transposed: [value column][row]
        if (!BWD)  // O += P Wv on waves 4-7
            mm_lds<DC, NSL, DC, L::PP, 1, 1, NSL, NSL, 4, 4>(1.f, sBuf + L::P, sWv, 1.f, sO);
        // S1 = c S0 + Kt^T Wv (8 tiles; the forward keeps waves 4-7 for O)
        mm_lds<D, NSL, DC, 1, L::PK, 1, NSL, NSL, 0, BWD ? 8 : 4>(1.f, sBuf + L::KT_, sWv, carry, sS);
        t0_prev = t0;
        n_prev = n;
    }
    __syncthreads();
    if (!BWD && NC > 0) store_o();
    if (!BWD && a.hT)
        for (int i = threadIdx.x; i < D * NSL; i += DTH) a.hT[(bh * D + i / NSL) * Dv + j0 + i % NSL] = sS[i];
}

// reverse state-gradient pass (chunks last to first): dS1 and dWv of every
// chunk, then dh0
template <typename T, int D>
__global__ __launch_bounds__(DTH) void k_delta_dstate(const DeltaArgs a) {
    using L = SeqLayout<D, true, true>;
    __shared__ float sBuf[L::TOTAL];
    __shared__ float sdS[D * NSL], sdWv[DC * NSL];
    if (a.put_stamp) put_stamp(a.stamp, a.expect);  // what the passes before this one found or stored
    const int Dv = (int)a.dv;
    const int nsl = Dv / NSL;
    const int64_t lb = xcd_logical_block(gridDim.x);  // the slices of one head share an XCD's L2
    const int64_t bh = lb / nsl, j0 = (lb % nsl) * NSL;
    const int64_t b = bh / a.H, h = bh % a.H;
    const int64_t NC = (a.T + DC - 1) / DC;
    const int64_t rv = a.H * Dv;
    for (int i = threadIdx.x; i < D * NSL; i += DTH) {
        const int r = i / NSL, j = i % NSL;
        sdS[i] = a.dhT ? a.dhT[(bh * D + r) * Dv + j0 + j] : 0.f;
    }
    SeqRegs<D, true> pf;
    float carry_next;
    auto fetch = [&](int64_t c) {
        const ChunkWs w = chunk_ws(a, bh * NC + c);
        const int64_t t0 = c * DC;
        const int n = (int)(a.T - t0 < DC ? a.T - t0 : DC);
        const T* dO = (const T*)a.dO + (b * a.T + t0) * rv + h * Dv + j0;
        seq_fetch<D, true>(pf, w, [&](int r, int j) { return r < n ? to_f32(dO[r * rv + j]) : 0.f; });
        carry_next = w.carry[0];
    };
    fetch(NC - 1);
    for (int64_t c = NC - 1; c >= 0; --c) {
        const ChunkWs w = chunk_ws(a, bh * NC + c);
        const float carry = carry_next;
        __syncthreads();
        seq_stash<D, true, true>(pf, sBuf);
        store_transposed<D>(sdS, w.dS1, j0);  // dS1 transposed: [value column][key row]
        __syncthreads();
        if (c > 0) fetch(c - 1);
        // dWv = P^T dO + Kt dS1 (the dO slice is zero past the end)
        mm_lds<DC, NSL, DC, 1, L::PP, 1, NSL, NSL>(1.f, sBuf + L::P, sBuf + L::SL, 0.f, sdWv);
        mm_lds<DC, NSL, D, L::PK, 1, 1, NSL, NSL>(1.f, sBuf + L::KT_, sdS, 1.f, sdWv);
        __syncthreads();
        store_transposed<DC>(sdWv, w.dWv, j0);  // dWv transposed: [value column][row]
        // dS0 = c dS1 + (gamma Q)^T dO - W^T dWv
        mm_lds<D, NSL, DC, 1, L::PQ, 1, NSL, NSL>(1.f, sBuf + L::QG, sBuf + L::SL, carry, sdS);
        mm_lds<D, NSL, DC, 1, L::PW, 1, NSL, NSL>(-1.f, sBuf + L::W, sdWv, 1.f, sdS);
    }
    __syncthreads();
    if (a.dh0)
        for (int i = threadIdx.x; i < D * NSL; i += DTH) a.dh0[(bh * D + i / NSL) * Dv + j0 + i % NSL] = sdS[i];
}

// ---------------------------------------------------------------- gradients
// (d_k = DK, d_v = DV fixed per instance: one kernel's code holds one shape)
template <typename T, int DK, int DV>
__global__ __launch_bounds__(DTH) void k_delta_grad(const DeltaArgs a) {
    __shared__ Rows R;
    __shared__ __attribute__((aligned(16))) float sXY[2 * DC * LP];
    __shared__ __attribute__((aligned(16))) T sK[DC * (128 + kpad<T>())];  // the chunk's K rows
    float* sX = sXY;
    float* sY = sXY + DC * LP;
    __shared__ float sdG[DC], sdB[DC], sr1[DC], sr2[DC], sdGC;
    __shared__ float smm[MMT_LDS];
    // dK, and for bf16 inputs (whose K tile is half the size) dQ, accumulate in LDS
    // rather than in ws2: T is read from ws where it is used and GE formed again
    // where it is needed, to make the room
    __shared__ __attribute__((aligned(16))) float sGK[DC * DK];
    __shared__ __attribute__((aligned(16))) float sGQ[sizeof(T) == 2 ? DC * DK : 1];
    const int64_t NC = (a.T + DC - 1) / DC;
    const int64_t chunk = blockIdx.x, bh = chunk / NC, c = chunk % NC;
    const int64_t b = bh / a.H, h = bh % a.H, t0 = c * DC;
    // The LDS products are chosen per instance (if constexpr on DK); the staged
    // products and elementwise passes take the sizes as run-time values (held
    // opaque), as constant sizes let the compiler precompute and hold many more
    // addresses across the kernel (it then spills).
    int D = DK, Dv = DV;
    asm volatile("" : "+s"(D), "+s"(Dv));
    const int64_t rk = a.H * D, rv = a.H * Dv;
    const T* Q = (const T*)a.q + (b * a.T + t0) * rk + h * D;
    const T* K = (const T*)a.k + (b * a.T + t0) * rk + h * D;
    const T* V = (const T*)a.v + (b * a.T + t0) * rv + h * Dv;
    const T* dO = (const T*)a.dO + (b * a.T + t0) * rv + h * Dv;
    prologue<T>(R, a, b, h, t0);
    if (threadIdx.x < DC) {
        sdG[threadIdx.x] = 0.f;
        sdB[threadIdx.x] = 0.f;
    }
    if (threadIdx.x == 0) sdGC = 0.f;
    __syncthreads();
    const int n = R.n;
    load_k<T>(R, K, rk, D, sK);
    const ChunkWs w = chunk_ws(a, chunk);
    float* const gK = sGK;
    float* const gQ = sizeof(T) == 2 ? sGQ : w.gQ;
    for (int i = threadIdx.x; i < DC * LP; i += DTH) sX[i] = 0.f;
    __syncthreads();
    // S0, Wv, dS1 and dWv are stored transposed ([value column][row]), so that
    // every product below reads its B operand along rows.

    // (1) output: dQg = dO S0^T; dP = dO Wv^T
    mmt(n, D, Dv, 1.f, dO, rv, 1, w.S0, D, 1, 0.f, gQ, D, 1, smm);
    mmt(n, n, Dv, 1.f, dO, rv, 1, w.Wv, DC, 1, 0.f, sX, LP, 1, smm);
    // (2) state: dKt = Wv dS1^T, in dK's place (dK starts as it, scaled per row)
    mmt(n, D, Dv, 1.f, w.Wv, 1, DC, w.dS1, D, 1, 0.f, gK, D, 1, smm);
    // (3) dW = -dWv S0^T, stored transposed ([key channel][row])
    mmt(DC, D, Dv, -1.f, w.dWv, 1, DC, w.S0, D, 1, 0.f, w.gW, 1, DC, smm);
    __syncthreads();
    // dGamma from gamma Q: rowdot(dQg, Qg); from Kt: -rowdot(dKt, Kt) per row, + sum into dGamma_last
    rowdot(n, D, gQ, D, w.Qg, D, sdG, 1.f);
    if (threadIdx.x < DC) sr1[threadIdx.x] = 0.f;
    __syncthreads();
    rowdot(n, D, gK, D, w.Kt, D, sr1, 1.f);
    // carry term: c <dS1, S0>
    {
        float s = 0.f;
#pragma unroll 1
        for (int base = threadIdx.x; base < D * Dv; base += 8 * DTH) {
            float x[8], y[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = base + u * DTH;
                x[u] = i < D * Dv ? w.dS1[i] : 0.f;
                y[u] = i < D * Dv ? w.S0[i] : 0.f;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) s += x[u] * y[u];
        }
        for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m, 64);
        if ((threadIdx.x & 63) == 0) sr2[threadIdx.x >> 6] = s;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float tot = 0.f;
        for (int t = 0; t < n; ++t) tot += sr1[t];
        float cs = 0.f;
        for (int wv = 0; wv < DTH / 64; ++wv) cs += sr2[wv];
        sdGC = tot + R.carry * cs;
    }
    if (threadIdx.x < DC) sdG[threadIdx.x] -= sr1[threadIdx.x];
    // dP (.) P -> dGamma (rows +, columns -); dP (.) M in sX.  The products
    // dP (.) P go through sY (free here) so that P is read along rows.
    __syncthreads();
    ew(DC * DC, [&](int i) { return sX[(i / DC) * LP + i % DC] * w.P[i]; },
       [&](int i, float v) { sY[(i / DC) * LP + i % DC] = v; });
    __syncthreads();
    if (threadIdx.x < DC) {
        const int t = threadIdx.x;
        float rsum = 0.f, csum = 0.f;
        for (int s = 0; s < DC; ++s) {
            rsum += sY[t * LP + s];
            csum += sY[s * LP + t];
        }
        sr1[t] = rsum;
        sr2[t] = csum;
    }
    __syncthreads();
    if (threadIdx.x < DC) sdG[threadIdx.x] += sr1[threadIdx.x] - sr2[threadIdx.x];
    for (int i = threadIdx.x; i < DC * DC; i += DTH) {
        const int t = i / DC, s = i % DC;
        sX[t * LP + s] = s <= t && t < n ? sX[t * LP + s] * decay(R, t, s) : 0.f;
    }
    // dQ = gamma dQg (in place), then += (dP (.) M) K; dK = (dP (.) M)^T Q + Kt-scale dKt
    __syncthreads();
    ew(DC * D, [&](int i) { return gQ[i] * R.gam[i / D]; }, [&](int i, float v) { gQ[i] = v; });
    ew(DC * D, [&](int i) { return R.kts[i / D] * gK[i]; }, [&](int i, float v) { gK[i] = v; });
    __syncthreads();
    if constexpr (DK == 128)
        mm_lds<DC, 128, DC, LP, 1, 1, 128 + kpad<T>(), 128>(1.f, sX, sK, 1.f, gQ);
    else
        mm_lds<DC, 64, DC, LP, 1, 1, 64 + kpad<T>(), 64>(1.f, sX, sK, 1.f, gQ);
    mmt(n, D, n, 1.f, sX, 1, LP, Q, rk, 1, 1.f, gK, D, 1, smm);
    __syncthreads();
    // (4) dT = dWv (beta V)^T + dW (beta gamma K)^T in sY ([i][j]), formed as
    //     dT^T = diag(beta) V dWv^T + diag(beta gamma) K dW^T
    mmt(n, DC, Dv, 1.f, V, rv, 1, w.dWv, DC, 1, 0.f, sY, 1, LP, smm, nullptr, R.beta);
    mmt(n, DC, D, 1.f, K, rk, 1, w.gW, DC, 1, 1.f, sY, 1, LP, smm, nullptr, R.bg);
    __syncthreads();
    for (int i = threadIdx.x; i < DC * LP; i += DTH)
        if (i % LP >= n && i % LP < DC) sY[i] = 0.f;
    __syncthreads();
    // (5) dA = -T^T dT T^T: sX = dT T^T, then sY = -T^T sX
    mmt(DC, DC, DC, 1.f, sY, LP, 1, w.T, 1, DC, 0.f, sX, LP, 1, smm);
    mmt(DC, DC, DC, -1.f, w.T, 1, DC, sX, LP, 1, 0.f, sY, LP, 1, smm);
    // GE = (K K^T) (.) E strictly below the diagonal, into sX (no longer read)
    gram_masked<T, DK>(R, sK, sX);
    // A = diag(beta) GE (strictly lower, same document): dbeta += sum_s dA GE; dGamma via
    // dA (.) A (rows +, columns -); dG = dA beta E in sX (strictly lower)
    if (threadIdx.x < DC) {
        const int t = threadIdx.x;
        float bsum = 0.f, rsum = 0.f, csum = 0.f;
        for (int s = 0; s < DC; ++s) {
            const float ge_ts = sX[t * LP + s], ge_st = sX[s * LP + t];
            const float da_ts = s < t ? sY[t * LP + s] : 0.f, da_st = t < s ? sY[s * LP + t] : 0.f;
            bsum += da_ts * ge_ts;
            rsum += da_ts * ge_ts;
            csum += da_st * R.beta[s] * ge_st;
        }
        sdB[t] += bsum;
        sr1[t] = R.beta[t] * rsum;
        sr2[t] = csum;
    }
    __syncthreads();
    if (threadIdx.x < DC) sdG[threadIdx.x] += sr1[threadIdx.x] - sr2[threadIdx.x];
    for (int i = threadIdx.x; i < DC * DC; i += DTH) {
        const int t = i / DC, s = i % DC;
        sX[t * LP + s] = s < t && t < n ? sY[t * LP + s] * R.beta[t] * decay(R, t, s) : 0.f;
    }
    __syncthreads();
    // dK += (dG + dG^T) K (one lane reads and writes each element in both calls)
    if constexpr (DK == 128) {
        mm_lds<DC, 128, DC, LP, 1, 1, 128 + kpad<T>(), 128>(1.f, sX, sK, 1.f, gK);
        mm_lds<DC, 128, DC, 1, LP, 1, 128 + kpad<T>(), 128>(1.f, sX, sK, 1.f, gK);
    } else {
        mm_lds<DC, 64, DC, LP, 1, 1, 64 + kpad<T>(), 64>(1.f, sX, sK, 1.f, gK);
        mm_lds<DC, 64, DC, 1, LP, 1, 64 + kpad<T>(), 64>(1.f, sX, sK, 1.f, gK);
    }
    __syncthreads();
    // dVb = T^T dWv (into sX, sY: free from here on), dKb = T^T dW, formed
    // transposed: dVb^T = dWv^T T, dKb^T = dW^T T (T as the prepare pass stored
    // it: this call's, or the forward's when the stamp matched)
    float* const gV = sXY;
    mmt(Dv, n, DC, 1.f, w.dWv, DC, 1, w.T, DC, 1, 0.f, gV, 1, Dv, smm);
    mmt(D, n, DC, 1.f, w.gW, DC, 1, w.T, DC, 1, 0.f, w.gKb, 1, D, smm);
    // (6) dV = beta dVb; dbeta += V . dVb + gamma K . dKb; dK += beta gamma dKb;
    //     dGamma += beta gamma K . dKb
    if (threadIdx.x < DC) sr1[threadIdx.x] = 0.f;
    if (threadIdx.x >= DC && threadIdx.x < 2 * DC) sr2[threadIdx.x - DC] = 0.f;
    __syncthreads();
    rowdot(n, Dv, V, rv, gV, Dv, sr1, 1.f);
    rowdot(n, D, K, rk, w.gKb, D, sr2, 1.f);
    __syncthreads();
    if (threadIdx.x < DC) {
        const int t = threadIdx.x;
        sdB[t] += sr1[t] + R.gam[t] * sr2[t];
        sdG[t] += R.bg[t] * sr2[t];
    }
    ew(DC * D, [&](int i) { return gK[i] + R.bg[i / D] * w.gKb[i]; }, [&](int i, float v) { gK[i] = v; });
    __syncthreads();
    // (7) the gate: dGamma_last goes to the last row; dg_u = sum of dGamma over t >= u
    //     in u's document; 0 at reset rows
    if (threadIdx.x == 0 && n > 0) sdG[n - 1] += sdGC;
    __syncthreads();
    const int64_t row0 = b * a.T + t0;
    if (threadIdx.x < DC) {
        const int u = threadIdx.x;
        if (u < n) {
            float s = 0.f;
            for (int t = u; t < n; ++t)
                if (R.doc[t] == R.doc[u]) s += sdG[t];
            ((T*)a.dg)[(row0 + u) * a.H + h] = from_f32<T>(R.reset[u] ? 0.f : s);
            ((T*)a.dbeta)[(row0 + u) * a.H + h] = from_f32<T>(sdB[u]);
        }
    }
    // outputs
    T* dq = (T*)a.dq + row0 * rk + h * D;
    T* dk = (T*)a.dk_out + row0 * rk + h * D;
    T* dv = (T*)a.dv_out + row0 * rv + h * Dv;
    ew(n * D, [&](int i) { return gQ[i]; }, [&](int i, float v) { dq[(i / D) * rk + i % D] = from_f32<T>(v); });
    ew(n * D, [&](int i) { return gK[i]; }, [&](int i, float v) { dk[(i / D) * rk + i % D] = from_f32<T>(v); });
    ew(n * Dv, [&](int i) { return R.beta[i / Dv] * gV[i]; },
       [&](int i, float v) { dv[(i / Dv) * rv + i % Dv] = from_f32<T>(v); });
}

}  // namespace

// T, P; U; W, Qg, Kt; the carry (4); (states_in_ws) S0, Wv
int64_t delta_fwd_floats_per_chunk(int64_t dk, int64_t dv, bool states_in_ws) {
    return 2 * DC * DC + DC * (dv + 3 * dk) + 4 + (states_in_ws ? dk * dv + DC * dv : 0);
}
// (unless states_in_ws) S0, Wv; dS1, dWv; gQ, gW, gKb
int64_t delta_bwd_floats_per_chunk(int64_t dk, int64_t dv, bool states_in_ws) {
    return 2 * dk * dv + DC * (2 * dv + 3 * dk) - (states_in_ws ? dk * dv + DC * dv : 0);
}


// the per-chunk kernels' instance for the problem's (d_k, d_v)
template <typename T> struct k_delta_prep_ptr {
    template <int DK, int DV> static constexpr auto get() { return &k_delta_prep<T, DK, DV>; }
};
template <typename T> struct k_delta_grad_ptr {
    template <int DK, int DV> static constexpr auto get() { return &k_delta_grad<T, DK, DV>; }
};
template <typename K>
void launch_shape(const DeltaArgs& a, dim3 grid, hipStream_t st) {
    if (a.dk == 128 && a.dv == 128) hipLaunchKernelGGL((K::template get<128, 128>()), grid, dim3(DTH), 0, st, a);
    else if (a.dk == 128) hipLaunchKernelGGL((K::template get<128, 64>()), grid, dim3(DTH), 0, st, a);
    else if (a.dv == 128) hipLaunchKernelGGL((K::template get<64, 128>()), grid, dim3(DTH), 0, st, a);
    else hipLaunchKernelGGL((K::template get<64, 64>()), grid, dim3(DTH), 0, st, a);
}

template <typename T>
hipError_t launch_delta_fwd(const DeltaArgs& a0, hipStream_t st) {
    DeltaArgs a = a0;
    a.check_stamp = 0;
    const int64_t NC = (a.T + DC - 1) / DC;
    launch_shape<k_delta_prep_ptr<T>>(a, dim3((unsigned)(a.B * a.H * NC)), st);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 slices((unsigned)(a.B * a.H * (a.dv / NSL)));
    // the stamp vouches for everything the forward stores in ws: the state pass,
    // the last of the forward's launches, writes it
    a.put_stamp = 1;
    if (a.dk == 128)
        hipLaunchKernelGGL((k_delta_state<T, false, 128>), slices, dim3(DTH), 0, st, a);
    else
        hipLaunchKernelGGL((k_delta_state<T, false, 64>), slices, dim3(DTH), 0, st, a);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_delta_bwd(const DeltaArgs& a0, hipStream_t st) {
    DeltaArgs a = a0;
    a.put_stamp = 0;
    const int64_t NC = (a.T + DC - 1) / DC;
    const dim3 chunks((unsigned)(a.B * a.H * NC)), slices((unsigned)(a.B * a.H * (a.dv / NSL)));
    // the prepare pass (and the state pass, where S0 and Wv live in ws) exits at
    // once when the workspace's stamp shows it holds these inputs' factors already
    // (check_stamp: the caller allows the reuse); both read the stamp as the call
    // found it, and the state-gradient pass then writes the stamp for what ws holds
    launch_shape<k_delta_prep_ptr<T>>(a, chunks, st);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.dk == 128)
        hipLaunchKernelGGL((k_delta_state<T, true, 128>), slices, dim3(DTH), 0, st, a);
    else
        hipLaunchKernelGGL((k_delta_state<T, true, 64>), slices, dim3(DTH), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    DeltaArgs da = a;
    da.put_stamp = 1;
    if (a.dk == 128)
        hipLaunchKernelGGL((k_delta_dstate<T, 128>), slices, dim3(DTH), 0, st, da);
    else
        hipLaunchKernelGGL((k_delta_dstate<T, 64>), slices, dim3(DTH), 0, st, da);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    launch_shape<k_delta_grad_ptr<T>>(a, chunks, st);
    return hipGetLastError();
}

template hipError_t launch_delta_fwd<float>(const DeltaArgs&, hipStream_t);
template hipError_t launch_delta_fwd<bf16>(const DeltaArgs&, hipStream_t);
template hipError_t launch_delta_bwd<float>(const DeltaArgs&, hipStream_t);
template hipError_t launch_delta_bwd<bf16>(const DeltaArgs&, hipStream_t);

}  // namespace gla
