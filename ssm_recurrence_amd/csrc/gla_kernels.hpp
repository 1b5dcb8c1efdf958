// gla_kernels.hpp -- host-visible launch entry points of the gfx950 kernels
// (internal to the library; the public ABI is include/gla.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gla {

// What a workspace's saved intermediates were computed from (the problem, the
// input pointers and the caller's generation value), kept in the workspace's
// first bytes and compared on the device before they are reused.
constexpr int kStampWords = 16;
constexpr int64_t kStampBytes = 256;
struct Stamp {
    uint64_t w[kStampWords];
};
// every thread of the workgroup: the workspace's stamp equals `expect`
// (thread 0 reads it; the answer is shared through LDS with one barrier)
__device__ __forceinline__ bool stamp_matches(const uint64_t* stamp, const Stamp& expect) {
    __shared__ int same;
    if (threadIdx.x == 0) {
        int eq = 1;
#pragma unroll
        for (int i = 0; i < kStampWords; ++i) eq &= stamp[i] == expect.w[i];
        same = eq;
    }
    __syncthreads();
    return __builtin_amdgcn_readfirstlane(same) != 0;
}
// Workgroup 0 writes the stamp `s` to dst (null: nothing).  Launches on one
// stream run in order, so a kernel that stores what a stamp describes, or that
// runs after the kernel that did, may write the stamp itself at its start: no
// later launch reads it before every workgroup of this one has finished.  A
// kernel whose workgroups compare the stamp must not write it (one of them could
// see the new value before another has read the old one).
__device__ __forceinline__ void put_stamp(uint64_t* dst, const Stamp& s) {
    if (dst == nullptr || blockIdx.x != 0 || threadIdx.x >= kStampWords) return;
    uint64_t w = s.w[0];
#pragma unroll
    for (int i = 1; i < kStampWords; ++i)
        if ((int)threadIdx.x == i) w = s.w[i];
    dst[threadIdx.x] = w;
}

struct PassArgs {
    const void *q, *k, *v, *g, *dO;
    const float *h0, *dhT;
    const int32_t* seg;
    void* o;
    float *hT, *dh0;
    float* ws_S;   // state pass output, [B*H][NC+1][DK][DV] in the input dtype
    void* ws_dS;   // state-gradient pass output, [B*H][NC][DK][DV] in the input dtype
    int64_t B, T, H, Hqk;
    // elements between consecutive tokens of q and k, and of v (o, dO are packed)
    int64_t ld_qk, ld_v;
    // exact sequence split: P pieces of PL chunks each (P = 1: no split)
    int64_t P, PL;
    const float* S_in;    // [B*H][P][DK][DV]: state entering each piece (P > 1)
    const float* dS_in;   // [B*H][P][DK][DV]: state gradient at each piece's end (P > 1)
    float* L_out[2];      // piece summaries from zero, [B*H][P][DK][DV]: forward, reverse
    float* D_out;         // decay product of each piece, [B*H][P][DK]
    // forward: also store the state entering every chunk, and the final state, in
    // the input dtype as ws_S's [B*H][NC+1][DK][DV] layout (null: not stored)
    void* save_S;
    // backward: ws_S may hold the forward's states; when the stamp there matches
    // `expect` the passes that would recompute them (ST_STATES, ST_SUM_FWD) exit
    const uint64_t* stamp;
    Stamp expect;
    int32_t check_stamp;
    // the forward kernel, or a backward pass launched after the states were
    // stored: workgroup 0 writes `expect` here (put_stamp; null: nothing)
    uint64_t* stamp_out;
    // split forward, whole-state kernels: each workgroup forms its piece's entry
    // state from h0 and the summaries of the pieces before it (L_out[0], D_out)
    // instead of reading S_in (no combine launch)
    int32_t entry_from_summaries;
    // summaries in one launch: D_out of pieces 1.. comes from ST_SUM_REV (which
    // always runs), of piece 0 from ST_SUM_FWD
    int32_t d_from_rev;
};

struct RevArgs {
    const void *q, *k, *v, *g, *dO;
    const int32_t* seg;
    const void* ws_S;   // [B*H][NC+1][DK][DV] in the input dtype: state entering each chunk, then hT
    const void* ws_dS;  // [B*H][NC][DK][DV] in the input dtype: state gradient at each chunk's end
    const float* dhT;
    void *dq, *dk, *dv, *dg;
    float* dh0;
    float *ws_dq, *ws_dk;  // per-head fp32 [B][T][H][DK] when heads share q/k
    float *ws_xs, *ws_bnd; // scalar gate: per-slice partial sums [B*H][slices][T], [B*H][slices][NC]
    int64_t B, T, H, Hqk;
    // elements between consecutive tokens: q and k, v (inputs); dq and dk, dv
    // (outputs); dO and the per-head fp32 dq, dk are packed
    int64_t ld_qk, ld_v, ld_dqk, ld_dv;
    // the split of the reverse walk (launch_grad8_walk): P pieces of PL chunks
    int64_t P, PL;
    const float* dS_in;    // [B*H][P][DK][DV]: state gradient at each piece's end (P > 1)
    // the reverse walk, launched after the states were stored: workgroup 0 writes
    // stamp_val here (put_stamp; null: nothing)
    uint64_t* stamp_out;
    Stamp stamp_val;
};

struct CombineArgs {
    const float *L_fwd, *L_rev, *D, *h0, *dhT;
    float *S_in, *dS_in;
    int64_t BH, P;
    int DK, DV, which;
    // backward: when the stamp matches, the states entering the chunks are the
    // forward's and the entry states of the pieces are not needed: the forward
    // chain is skipped
    const uint64_t* stamp;
    Stamp expect;
    int32_t check_stamp;
};

// modes of the state pass: per-chunk states or state gradients, per-piece summaries
enum { ST_STATES = 0, ST_SUM_FWD = 1, ST_SUM_REV = 2, ST_DSTATES = 3 };

// wide: blocks of 64 key channels x all value columns (else 64 x 64)
template <typename T, bool VEC, int DK, int DV>
hipError_t launch_states(const PassArgs& a, int mode, bool wide, hipStream_t st);

// ST_STATES and ST_DSTATES (summaries = false) or ST_SUM_FWD and ST_SUM_REV in one launch
template <typename T, bool VEC, int DK, int DV>
hipError_t launch_states_pair(const PassArgs& a, bool summaries, bool wide, hipStream_t st);

// ST_SUM_REV then ST_SUM_FWD (summaries = true) or ST_DSTATES then ST_STATES in
// one launch, the second pass on the last half of the blocks (it may exit at
// once: the forward's stored states found); blocks as launch_states shapes them
template <typename T, bool VEC, int DK, int DV>
hipError_t launch_states_trail(const PassArgs& a, bool summaries, bool wide, hipStream_t st);

hipError_t launch_piece_combine(const CombineArgs& c, hipStream_t st);

// scalar gate: dg from the per-slice partial sums (one wave per chunk)
hipError_t launch_dg_scalar(const RevArgs& a, int nslices, bool bf16_out, hipStream_t st);

// bf16, vector gate, d_k = d_v = 128: one eight-wave workgroup per chunk
hipError_t launch_grad8(const RevArgs& a, hipStream_t st);
// bf16, scalar gate, d_k = d_v = 128: one workgroup per (b, h, piece) walking its
// chunks last to first with the state gradient resident (needs only the per-chunk
// states, not the per-chunk state gradients)
hipError_t launch_grad8_walk(const RevArgs& a, hipStream_t st);

// fp32, scalar gate, d_k = d_v = 128: split-bf16 products (includes the dg finisher)
hipError_t launch_grad_f32s(const RevArgs& a, hipStream_t st);

// chunk-parallel gradients from the per-chunk states and state gradients
template <typename T, bool VEC, int DK, int DV>
hipError_t launch_grad(const RevArgs& a, hipStream_t st);

template <typename T, bool VEC, int DK, int DV, int NV>
hipError_t launch_fwd(const PassArgs& a, hipStream_t st);
// fp32 inputs, scalar gate, d_k = d_v = 128: the forward on the bf16 matrix cores
// (split operands), one 8-wave workgroup per (b, h, piece) holding the whole state
hipError_t launch_fwd_f32h(const PassArgs& a, hipStream_t st);
// bf16 inputs, either gate, d_k = d_v = 128: one 8-wave workgroup per (b, h, piece)
template <bool VEC>
hipError_t launch_fwd_h(const PassArgs& a, hipStream_t st);

// short depthwise causal convolution (K = 4 taps, bias, SiLU), gla_conv.hip
struct ConvArgs {
    const void* x;                 // [B][T][C], input dtype
    const float *w, *bias;         // [K][C], [C] (bias may be null)
    void* y;                       // forward output [B][T][C]
    const void* dy;                // backward: upstream gradient [B][T][C]
    void* dx;                      // backward: [B][T][C]
    float *dw, *db;                // backward: [K][C], [C] (db may be null)
    float* ws;                     // backward: per-workgroup partials [conv_partials][K+1][C]
    int64_t B, T, C;
};
int64_t conv_partials(int64_t B, int64_t T);
template <typename T>
hipError_t launch_conv_fwd(const ConvArgs& a, hipStream_t st);
// the convolution backward and the fixed-order reduction of dW, db (T = 0 included)
template <typename T>
hipError_t launch_conv_bwd(const ConvArgs& a, hipStream_t st);

// output norm and gate (per-head RMSNorm times a swish gate), gla_norm.hip
struct NormArgs {
    const void *o, *z, *dy;  // [rows][D], input dtype (dy: backward)
    const float* gamma;      // [D]
    void* y;                 // forward output [rows][D]
    void *d_o, *dz;          // backward outputs [rows][D]
    float* dgamma;           // backward output [D]
    float* ws;               // backward: per-workgroup dgamma partials [norm_gate_partials][D]
    int64_t rows;
    float eps;
};
template <typename T, int D> int64_t norm_gate_partials(int64_t rows);
template <typename T, int D> hipError_t launch_norm_gate_fwd(const NormArgs& a, hipStream_t st);
// the backward and the fixed-order reduction of dgamma (rows = 0 included)
template <typename T, int D> hipError_t launch_norm_gate_bwd(const NormArgs& a, hipStream_t st);

// the gated delta rule (chunked WY/UT form), gla_delta.hip
struct DeltaArgs {
    const void *q, *k, *v, *g, *beta, *dO;  // [B][T][H][d] (g, beta: [B][T][H]), input dtype
    const float *h0, *dhT;                  // [B][H][dk][dv] or null
    const int32_t* seg;                     // [B][T] or null
    void* o;                                // forward output
    float* hT;                              // forward output or null
    void *dq, *dk_out, *dv_out, *dg, *dbeta;  // backward outputs
    float* dh0;                             // backward output or null
    float* ws;                              // the forward's factors: delta_fwd_floats_per_chunk per (b, h, chunk)
    int64_t ws_chunk;
    float* ws2;                             // backward only: delta_bwd_floats_per_chunk per (b, h, chunk)
    int64_t ws2_chunk;
    uint64_t* stamp;                        // the workspace's stamp words
    Stamp expect;                           // this call's stamp
    int32_t check_stamp;                    // backward: skip the prepare and state passes when stamp == expect
    int32_t put_stamp;                      // this launch's workgroup 0 writes expect to stamp (put_stamp)
    // the states entering the chunks and the effective writes (S0, Wv) live in ws,
    // after each chunk's factors (the forward stores them), not in ws2
    int32_t states_in_ws;
    int64_t B, T, H, dk, dv;
};
constexpr int64_t kDeltaHeaderBytes = kStampBytes;  // the stamp, ahead of the per-chunk factors
int64_t delta_fwd_floats_per_chunk(int64_t dk, int64_t dv, bool states_in_ws);
int64_t delta_bwd_floats_per_chunk(int64_t dk, int64_t dv, bool states_in_ws);
template <typename T> hipError_t launch_delta_fwd(const DeltaArgs& a, hipStream_t st);
template <typename T> hipError_t launch_delta_bwd(const DeltaArgs& a, hipStream_t st);

template <typename T, int DK>
hipError_t launch_group_sum(const float* src, void* dst, int64_t ld_dst, int64_t B, int64_t Tn,
                            int64_t H, int64_t Hqk, hipStream_t st);

}  // namespace gla
