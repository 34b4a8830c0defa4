// Chunk scan with one workgroup per (batch, head) sequence, on gfx950 matrix
// cores (bf16 operands, fp32 accumulation).
//
// The sequence is walked in sub-blocks of 64 tokens and the P x N state stays
// in matrix-core accumulators from the first token to the last.  Per
// sub-block, with Lambda the inclusive prefix sum of dt*A inside it, the block
// decomposition of the "Mamba-2" note (section "taking each path half way")
// and of the "Mamba-2 model walkthrough" (sections 6.1-6.2) gives
//   y_i = exp(Lambda_i) Cm_i . H  +  sum_{j<=i} G[i][j] exp(Lambda_i - Lambda_j) dt_j x_j  +  D x_i
//   H  <- exp(Lambda_63) H  +  sum_j Bm_j (outer) (exp(Lambda_63 - Lambda_j) dt_j x_j)
// with G[i][j] = Cm_i . Bm_j from the gram tiles and H the state entering the
// sub-block.
//
// A workgroup has eight waves, two on each SIMD, in two roles, so that each
// SIMD has a second instruction stream to issue from while one waits on LDS
// or memory:
//   compute waves 0-3  own rows p = 16w..16w+15 of the state.  In step t they
//                      form the whole output of sub-block t (inter-block term,
//                      masked intra-block product with D on the diagonal of
//                      the masked matrix, y into an LDS tile stored as whole
//                      rows in the next step) and advance the state over it;
//                      they also stage x and load dt;
//   prep waves 4-7     build the masked decay matrix of sub-block t+1 from its
//                      gram tiles and the prefix scan of dt*A, and stage its
//                      Bm and Cm.
// One barrier per step; LDS buffers rotate so that nothing written in a step
// is read in the same step by another wave.
#include "tile_ops.h"

namespace ssd {
namespace {

using namespace tile;
constexpr int kThreads = 512;



template <int N>
struct PipeSmem {
    __bf16 X[2][kSub * kP];        // x [j][p] (by t % 2), chunks swizzled (xsw)
    __bf16 Bt[2][kSub * N];        // Bm [j][n] (by t % 2), chunks swizzled (bsw)
    // Cm [i][n] (by t % 2), chunks swizzled (csw).  At N = 256 there is room
    // for one slot only: the compute waves read it in the first part of a
    // step, and the prep waves refill it after a barrier in the middle.
    static constexpr int kCSlots = N == 256 ? 1 : 2;
    __bf16 Ct[kCSlots][ct_bytes<N> / 2];
    __bf16 Mm[2][kSub * kSub];     // masked decay matrix [i][j] (by t % 2), chunks swizzled (msw)
    WaveDecays wd[8];
    // y on its way to global memory as whole 128-byte rows: written by the
    // four compute waves (16 columns each) in one step, stored in the next
    // (by t % 2); chunk c of row r at c ^ ((r >> 1) & 7)
    __bf16 YS[2][kSub * kP];
    // dt of the sub-block of step s (token j at [s % 4][j], 0 past the end):
    // loaded four steps ahead and written two steps ahead by the compute
    // waves, a quarter of the tokens each; read by all eight waves
    float dts[4][kSub];
};



struct Args {
    const __bf16 *x;
    const float *dt, *A;
    const __bf16 *Bm, *Cm;
    const float *D, *init;
    __bf16 *y;
    float *final_state;
    const __bf16 *gram;
    float *seg;              // segment states [nextra][nseg-1][P][N], then their log2 decays [nextra][nseg-1]
    int64_t L, H, G, nsb;    // H: heads of 64 channels (a head of P = 128 is two of them)
    int64_t Hd;              // heads of dt, A and D (the caller's H)
    int hs;                  // heads of 64 channels per caller head (P / 64)
    int nmain;               // sequences run whole, one per workgroup (0: every sequence is cut)
    int nextra;              // further sequences, each cut into nseg segments of seglen sub-blocks;
    int nseg, seglen;        //   segment q of extra sequence e runs on the workgroup whose logical
                             //   index (xcd_chain of its block index) is q*nextra + e
};

// Segment-state buffers in Args::seg.
template <int N>
__device__ __forceinline__ float *seg_state(const Args &a, int e, int q) {
    return a.seg + ((int64_t)e * (a.nseg - 1) + q) * (kP * N);
}
template <int N>
__device__ __forceinline__ float *seg_log2decay(const Args &a, int e, int q) {
    return a.seg + (int64_t)a.nextra * (a.nseg - 1) * (kP * N) + (int64_t)e * (a.nseg - 1) + q;
}



// Packed rows of several independent sequences: the first token of every
// sequence after a row's first carries its dt with the sign bit set, so that
// one load gives both the step and the reset flag.  A reset at token r stops
// everything before r from reaching r and the tokens after it.
__device__ __forceinline__ float dt_mag(float v) { return __builtin_fabsf(v); }
__device__ __forceinline__ uint64_t reset_mask(float v) {
    return __builtin_amdgcn_ballot_w64((__float_as_uint(v) >> 31) != 0u);
}
// bits of tokens 0..k
__device__ __forceinline__ uint64_t upto(int k) { return (2ull << k) - 1ull; }
// last reset at or before token k of a sub-block, -1 if none
__device__ __forceinline__ int last_reset(uint64_t m, int k) {
    const uint64_t r = m & upto(k);
    return r ? 63 - (int)__builtin_clzll(r) : -1;
}

__device__ __forceinline__ int sub_tokens(const Args &a, int sb) {
    const int64_t rem = a.L - (int64_t)sb * kSub;
    return rem < kSub ? (int)rem : kSub;
}

// Global loads of this thread's share of sub-block sb's x (state waves) or Bm
// and Cm (output waves), masked past the end of the sequence.
// Loads of one sub-block given the element offset of its first row in each
// tensor and its number of tokens q (rows past q read as zeros).
template <int N>
__device__ __forceinline__ void load_x_at(BulkX &sl, const Args &a, const LaneOffs<N> &o, int64_t xo, int q) {
    const rsrc_t r = rsrc(a.x + xo, q > 0 ? (int)(((int64_t)(q - 1) * a.H * kP + kP) * 2) : 0);
    const int step = (int)(32 * a.H * kP * 2);
#pragma unroll
    for (int k = 0; k < 2; ++k) sl.x[k] = ld16(r, o.gx + k * step);
}
template <int N>
__device__ __forceinline__ void load_bc_at(BulkBC<N> &sl, const Args &a, const LaneOffs<N> &o, int64_t bo, int q) {
    using O = LaneOffs<N>;
    const int bytes = q > 0 ? (int)(((int64_t)(q - 1) * a.G * N + N) * 2) : 0;
    const rsrc_t rb = rsrc(a.Bm + bo, bytes);
    const rsrc_t rc = rsrc(a.Cm + bo, bytes);
    const int step = (int)((256 / O::CPR) * a.G * N * 2);
#pragma unroll
    for (int k = 0; k < N / 32; ++k) {
        sl.b[k] = ld16(rb, o.gb + k * step);
        sl.c[k] = ld16(rc, o.gb + k * step);
    }
}
// This wave's gram tiles of one sub-block (tiles ow, ow+4, ow+8).
__device__ __forceinline__ void load_g_at(uint2 (&g)[3], const Args &a, int64_t go, int q, int ow, int lane) {
    const rsrc_t rg = rsrc(a.gram + go, q > 0 ? kSub * kSub * 2 : 0);
#pragma unroll
    for (int m = 0; m < 3; ++m) {
        const int k = ow + 4 * m < 10 ? ow + 4 * m : 9;   // waves with two tiles load their last twice
        g[m] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rg, (k * 64 + lane) * 8, 0, 0));
    }
}
// dt of one token of a sub-block (element offset dof of its first row; token
// offset gdq in bytes), 0 past its q tokens.
__device__ __forceinline__ float load_dt_at(const Args &a, int64_t dof, int q, int gdq) {
    const rsrc_t rd = rsrc(a.dt + dof, q > 0 ? (int)(((int64_t)(q - 1) * a.Hd + 1) * 4) : 0);
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rd, gdq, 0, 0));
}

template <int N>
__device__ __forceinline__ void stage_x(PipeSmem<N> &sm, int xbuf, const BulkX &sl, const LaneOffs<N> &o) {
    unsigned char *Xb = reinterpret_cast<unsigned char *>(sm.X[xbuf]);
#pragma unroll
    for (int k = 0; k < 2; ++k) lds_st<uint4>(Xb + o.sx + k * 4096, sl.x[k]);
}
template <int N>
__device__ __forceinline__ void stage_bc(PipeSmem<N> &sm, int par, const BulkBC<N> &sl, const LaneOffs<N> &o) {
    using O = LaneOffs<N>;
    unsigned char *Bb = reinterpret_cast<unsigned char *>(sm.Bt[par]);
    unsigned char *Cb = reinterpret_cast<unsigned char *>(sm.Ct[par % PipeSmem<N>::kCSlots]);
#pragma unroll
    for (int k = 0; k < N / 32; ++k) {
        lds_st<uint4>(Bb + (o.sb ^ sb_flip<N>(k)) + k * (256 / O::CPR) * O::RB, sl.b[k]);
        lds_st<uint4>(Cb + o.sc[k], sl.c[k]);
    }
}
template <int N>
__device__ __forceinline__ void stage_b(PipeSmem<N> &sm, int par, const BulkBC<N> &sl, const LaneOffs<N> &o) {
    using O = LaneOffs<N>;
    unsigned char *Bb = reinterpret_cast<unsigned char *>(sm.Bt[par]);
#pragma unroll
    for (int k = 0; k < N / 32; ++k) lds_st<uint4>(Bb + (o.sb ^ sb_flip<N>(k)) + k * (256 / O::CPR) * O::RB, sl.b[k]);
}
template <int N>
__device__ __forceinline__ void stage_c(PipeSmem<N> &sm, const BulkBC<N> &sl, const LaneOffs<N> &o) {
    unsigned char *Cb = reinterpret_cast<unsigned char *>(sm.Ct[0]);
#pragma unroll
    for (int k = 0; k < N / 32; ++k) lds_st<uint4>(Cb + o.sc[k], sl.c[k]);
}



// Waits for the loads of the state held in H.  Without it the state enters a
// step loop with its loads in flight on that path, and the wait counts the
// compiler derives for the loop (one set for every path in) then make each
// step wait for the latest x loads where it first reads the state.
template <int NT>
__device__ __forceinline__ void settle(f32x4 (&H)[NT]) {
#pragma unroll
    for (int u = 0; u < NT; ++u) asm volatile("" ::"v"(H[u]));
}

template <int N, bool kV>
__global__ __launch_bounds__(kThreads, 1) void pipe_kernel(Args a) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    PipeSmem<N> &sm = *reinterpret_cast<PipeSmem<N> *>(smem_raw);
    using O = LaneOffs<N>;
    constexpr int NT = N / 16;
    constexpr int KS = N / 32;

    // this workgroup's own sequence (steps 0..nown-1; none when nmain is 0) and,
    // after it, segment xq of a further sequence (steps nown..T-1, sub-blocks
    // seg0..seg0+xlen-1)
    const int nsub = (int)((a.L + kSub - 1) / kSub);
    const int nown = a.nmain > 0 ? nsub : 0;
    // logical workgroup index, contiguous within each XCD: the heads of a
    // batch row (own sequences) and the heads of one segment (extra
    // sequences), which share Bm, Cm, dt and the gram tiles, then sit behind
    // one L2 instead of all eight
    const int64_t lid = xcd_chain(blockIdx.x, gridDim.x);
    const int64_t chain = a.nmain > 0 ? lid : lid % a.nextra;
    const int64_t b = __builtin_amdgcn_readfirstlane((int)(chain / a.H));
    const int64_t h = __builtin_amdgcn_readfirstlane((int)(chain % a.H));
    const int64_t g = __builtin_amdgcn_readfirstlane((int)(h / (a.H / a.G)));
    const int64_t dh = h / a.hs;   // the caller's head: dt, A and D
    const float Ah2v = a.A[dh] * kLog2e, Dhv = a.D[dh];
    const bool has_x = lid < (int64_t)a.nextra * a.nseg;
    const int xe = has_x ? (int)(lid % a.nextra) : 0;
    const int xq = has_x ? (int)(lid / a.nextra) : 0;
    const int64_t xchain = has_x ? a.nmain + xe : chain;
    const int64_t bx = __builtin_amdgcn_readfirstlane((int)(xchain / a.H));
    const int64_t hx = __builtin_amdgcn_readfirstlane((int)(xchain % a.H));
    const int64_t gx = __builtin_amdgcn_readfirstlane((int)(hx / (a.H / a.G)));
    const int64_t dhx = hx / a.hs;
    const float Ahx2 = a.A[dhx] * kLog2e, Dhx = a.D[dhx];
    const int seg0 = xq * a.seglen;
    const int xlen = has_x ? (nsub - seg0 < a.seglen ? nsub - seg0 : a.seglen) : 0;
    const int T = nown + xlen;
    // sub-block of step tau, and of the step whose loads are issued at tau
    auto sb_of = [&](int tau) { return tau < nown ? tau : seg0 + (tau - nown); };
    auto q_of = [&](int tau) {
        const int rem = (int)a.L - sb_of(tau) * kSub;
        return rem < kSub ? rem : kSub;
    };
    // element offsets of step tau's first row in x / y, dt, Bm / Cm and the
    // gram tiles: the own sequence's base, or the segment's base shifted so
    // that the step index addresses it directly
    const int64_t SX = kSub * a.H * kP, SD = kSub * a.Hd, SB = kSub * a.G * N, SG = kSub * kSub;
    const int64_t xo0 = (b * a.L * a.H + h) * kP, xo1 = (bx * a.L * a.H + hx) * kP + (int64_t)(seg0 - nown) * SX;
    const int64_t do0 = b * a.L * a.Hd + dh, do1 = bx * a.L * a.Hd + dhx + (int64_t)(seg0 - nown) * SD;
    const int64_t bo0 = (b * a.L * a.G + g) * N, bo1 = (bx * a.L * a.G + gx) * N + (int64_t)(seg0 - nown) * SB;
    const int64_t go0 = (b * a.G + g) * a.nsb * SG, go1 = (bx * a.G + gx) * a.nsb * SG + (int64_t)(seg0 - nown) * SG;
    auto x_at = [&](int tau) { return (tau < nown ? xo0 : xo1) + tau * SX; };
    auto d_at = [&](int tau) { return (tau < nown ? do0 : do1) + tau * SD; };
    auto b_at = [&](int tau) { return (tau < nown ? bo0 : bo1) + tau * SB; };
    auto g_at = [&](int tau) { return (tau < nown ? go0 : go1) + tau * SG; };

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int pq = wave & 3;
    const bool compute_wave = wave < 4;
    const int lane = tid & 63, lrow = lane & 15, lgrp = lane >> 4;
    const LaneOffs<N> o = lane_offsets<N>(tid, pq, a.H, a.G, a.Hd);
    WaveDecays &wd = sm.wd[wave];
    // whole rows of y of step tau from YS[slot] to global memory (compute waves;
    // thread u = tid % 256: rows u/8 and u/8 + 32, chunk u%8)
    const int ysr = ((tid & 255) >> 3) * 128 + ((((tid & 255) & 7) ^ (((tid & 255) >> 4) & 7)) * 16);
    auto store_y = [&](int tau, int slot) __attribute__((always_inline)) {
        const int q = tau >= 0 ? q_of(tau) : 0;
        const rsrc_t ry = rsrc(a.y + x_at(tau), q > 0 ? (int)(((int64_t)(q - 1) * a.H * kP + kP) * 2) : 0);
        const unsigned char *Yr = reinterpret_cast<const unsigned char *>(sm.YS[slot]);
        const int step = (int)(32 * a.H * kP * 2);
#pragma unroll
        for (int k = 0; k < 2; ++k)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, lds_ld<uint4>(Yr + ysr + k * 4096)), ry,
                                                   o.gx + k * step, 0, 0);
    };

    // x and dt of the steps ahead are loaded, staged and published by the
    // compute waves, or at N = 256 (whose compute waves hold twice the state
    // and have no registers to spare) by the prep waves.  Wave pq of that role
    // loads dt of tokens 16pq .. 16pq+15 (four lanes each).  xbulk[s % 2]
    // holds x of step s from its load (issued at the end of step s-3) until
    // it is staged at the end of step s-1; dq[t % 2] holds the dt quarter of
    // step t+2 (loaded in step t-2), written to LDS in step t and replaced by
    // that of t+4.
    constexpr bool kPrepX = PipeSmem<N>::kCSlots == 1;
    const bool x_wave = compute_wave != kPrepX;
    const int dq_tok = 16 * pq + (lane & 15);
    const int gdq = dq_tok * (int)(a.Hd * 4);
    BulkX xbulk[2];
    float dq[2];
    // x of sub-block 0 staged; x of sub-blocks 1 and 2 and the dt quarters of
    // sub-blocks 2 and 3 in flight
    auto xd_prologue = [&]() __attribute__((always_inline)) {
        const int t1 = T > 1 ? 1 : 0, t2 = T > 2 ? 2 : T - 1, t3 = T > 3 ? 3 : T - 1;
        load_x_at<N>(xbulk[0], a, o, x_at(0), q_of(0));
        dq[0] = load_dt_at(a, d_at(t2), q_of(t2), gdq);
        dq[1] = load_dt_at(a, d_at(t3), q_of(t3), gdq);
        stage_x<N>(sm, 0, xbulk[0], o);
        load_x_at<N>(xbulk[1], a, o, x_at(t1), q_of(t1));
        load_x_at<N>(xbulk[0], a, o, x_at(t2), q_of(t2));
    };
    // step t: this wave's dt quarter of step t+2 into LDS, that of t+4 into its register
    auto xd_dt = [&](int t, int par) __attribute__((always_inline)) {
        if (lane < 16) sm.dts[(t + 2) & 3][dq_tok] = dq[par];
        const int td = t + 4 < T ? t + 4 : T - 1;
        dq[par] = load_dt_at(a, d_at(td), q_of(td), gdq);
    };
    // step t: x of step t+1 into LDS, and x of step t+3 into its registers.
    // Unconditional: a conditional stage leaves its loads unwaited on one
    // path, and the loop head then waits for them on every path (the last
    // step stages into a slot nobody reads).
    auto xd_x = [&](int t, int par) __attribute__((always_inline)) {
        stage_x<N>(sm, par ^ 1, xbulk[par ^ 1], o);
        const int tx = t + 3 < T ? t + 3 : T - 1;
        load_x_at<N>(xbulk[par ^ 1], a, o, x_at(tx), q_of(tx));
    };
    if (x_wave) {
        const int t1 = T > 1 ? 1 : 0;
        const float d0 = load_dt_at(a, d_at(0), q_of(0), gdq);
        const float d1 = load_dt_at(a, d_at(t1), q_of(t1), gdq);
        if (lane < 16) {
            sm.dts[0][dq_tok] = d0;
            sm.dts[1][dq_tok] = d1;
        }
    }
    __syncthreads();

    if (compute_wave) {
        // ------------------------------------------------------------------
        // compute waves: rows p = 16pq..16pq+15 of H, held transposed (rows n,
        // columns p): lane holds n = 16t + 4lgrp + 0..3, p = 16pq + lrow.  The
        // outputs of sub-block t: lane holds token i = 16it + lrow,
        // p = 16pq + 4lgrp + 0..3.
        if constexpr (!kPrepX) xd_prologue();
        f32x4 Hacc[NT];
        const int lane_off = (16 * pq + lrow) * N + 4 * lgrp;
        {
            const rsrc_t ri = rsrc(a.init ? (const void *)(a.init + chain * (kP * N)) : (const void *)a.x,
                                   a.init ? kP * N * 4 : 0);
#pragma unroll
            for (int u = 0; u < NT; ++u)
                Hacc[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ri, (lane_off + 16 * u) * 4, 0, 0));
            settle(Hacc);
        }
        __syncthreads();
        // this lane's 8 bytes of the y tile (rows 16it + lrow, columns 16pq + 4lgrp..+3)
        const int ysw = lrow * 128 + (((2 * pq + (lgrp >> 1)) ^ ((lrow >> 1) & 7)) * 16) + (lgrp & 1) * 8;
        // own sequence done: its final state out; the segment's entering state
        // in, from the initial state and the states and log2 decays of the
        // earlier segments (written by the segment-state kernel)
        auto switch_to_segment = [&]() __attribute__((always_inline)) {
            if (a.final_state && nown > 0) {
                float *dst = a.final_state + chain * (kP * N) + lane_off;
#pragma unroll
                for (int u = 0; u < NT; ++u) *reinterpret_cast<f32x4 *>(dst + 16 * u) = Hacc[u];
            }
            {
                const rsrc_t ri = rsrc(a.init ? (const void *)(a.init + xchain * (kP * N)) : (const void *)a.x,
                                       a.init ? kP * N * 4 : 0);
#pragma unroll
                for (int u = 0; u < NT; ++u)
                    Hacc[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                            ri, (lane_off + 16 * u) * 4, 0, 0));
            }
            for (int qq = 0; qq < xq; ++qq) {
                const float gq = ex2(*seg_log2decay<N>(a, xe, qq));
                const float *sq = seg_state<N>(a, xe, qq) + lane_off;
#pragma unroll
                for (int u = 0; u < NT; ++u) Hacc[u] = gq * Hacc[u] + *reinterpret_cast<const f32x4 *>(sq + 16 * u);
            }
            settle(Hacc);
        };
        auto step = [&](int t, int par) __attribute__((always_inline)) {
            const unsigned char *Xb = reinterpret_cast<const unsigned char *>(sm.X[par]);
            const unsigned char *Bb = reinterpret_cast<const unsigned char *>(sm.Bt[par]);
            const unsigned char *Cb = reinterpret_cast<const unsigned char *>(sm.Ct[par % PipeSmem<N>::kCSlots]);
            const unsigned char *Mr = reinterpret_cast<const unsigned char *>(sm.Mm[par]);
            const float Ah2 = t >= nown ? Ahx2 : Ah2v;
            // decays of sub-block t (this wave's own copy)
            const float dtr = sm.dts[t & 3][lane];
            const float dt = kV ? dt_mag(dtr) : dtr;
            const float v = wave_scan(dt * Ah2);
            const float lend = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
            float wv = ex2(lend - v) * dt, rdv = ex2(v), gam = ex2(lend);
            if constexpr (kV) {
                // tokens before the last reset do not reach the end of the
                // sub-block; the entering state reaches only the tokens
                // before the first reset
                const uint64_t rm = reset_mask(dtr);
                if (rm) {
                    if (lane < 63 - (int)__builtin_clzll(rm)) wv = 0.f;
                    if (rm & upto(lane)) rdv = 0.f;
                    gam = 0.f;
                }
            }
            wd.w[lane] = wv;
            wd.rdec[lane] = rdv;
            if constexpr (!kPrepX) xd_dt(t, par);
            // the whole rows of y of step t-1 (written to YS by the four compute waves in step t-1)
            store_y(t - 1, par ^ 1);

            // LDS reads, each a k-step ahead of the products that use them
            auto read_cf = [&](int ks, bf16x8 (&cf)[4]) __attribute__((always_inline)) {
#pragma unroll
                for (int it = 0; it < 4; ++it) {
                    const unsigned char *Ci = Cb + it * (16 * O::RB + ct_pad<N>) + (ks / O::KSO) * 256;
                    const bf16x4 c0 = lds_ld<bf16x4>(Ci + (o.ct[ks % O::KSO][0] ^ csw_tile_bytes<N>(it)));
                    const bf16x4 c1 = lds_ld<bf16x4>(Ci + (o.ct[ks % O::KSO][1] ^ csw_tile_bytes<N>(it)));
                    cf[it] = bf16x8{c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
                }
            };
            // Bm fragments of the update, in groups of four n-tiles (k-step ks, tiles 4v..4v+3)
            auto read_bt = [&](int ks, int v4, bf16x8 (&bt)[4]) __attribute__((always_inline)) {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int nt = 4 * v4 + u;
                    const unsigned char *Bn = Bb + o.bt[nt % O::NTO] + (nt / O::NTO) * 256 + ks * 32 * O::RB;
                    const bf16x4 lo = tr4(Bn);
                    const bf16x4 hi = tr4(Bn + 4 * O::RB);
                    bt[u] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                }
            };
            bf16x8 cf[2][4];
            read_cf(0, cf[0]);
            bf16x8 xf[2];
            auto read_xf = [&]() __attribute__((always_inline)) {
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const bf16x4 lo = tr4(Xb + o.xtr + ks * 4096);
                    const bf16x4 hi = tr4(Xb + o.xtr + ks * 4096 + 512);
                    xf[ks] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                }
            };
            if constexpr (PipeSmem<N>::kCSlots == 2) read_xf();
            const f32x4 rd = {wd.rdec[lrow], wd.rdec[16 + lrow], wd.rdec[32 + lrow], wd.rdec[48 + lrow]};
            __builtin_amdgcn_sched_barrier(0);

            // inter-block term of sub-block t: Y^T[p][i] = exp(Lambda_i) sum_n H[p][n] Cm_i[n]
            f32x4 Y[4];
#pragma unroll
            for (int it = 0; it < 4; ++it) Y[it] = f32x4{0.f, 0.f, 0.f, 0.f};
            // masked-matrix fragments of the intra-block product: read during the
            // last k-step of the inter-block term, or at N = 256 (whose larger
            // state leaves no registers for them there) after it
            bf16x8 mf[4][2];
            auto read_mf = [&]() __attribute__((always_inline)) {
#pragma unroll
                for (int it = 0; it < 4; ++it)
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk)
                        if (!(kk == 1 && it < 2)) mf[it][kk] = lds_ld<bf16x8>(Mr + o.mm[kk] + it * 2048);
            };
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if (ks + 1 < KS)
                    read_cf(ks + 1, cf[(ks + 1) & 1]);
                else if constexpr (PipeSmem<N>::kCSlots == 2)
                    read_mf();
                const bf16x8 ah = to_bf16x8(Hacc[2 * ks], Hacc[2 * ks + 1]);
#pragma unroll
                for (int it = 0; it < 4; ++it) Y[it] = mfma(ah, cf[ks & 1][it], Y[it]);
                __builtin_amdgcn_sched_barrier(0);
            }
            // one Cm slot (N = 256): done with it, the prep waves refill it
            if constexpr (PipeSmem<N>::kCSlots == 1) {
                __syncthreads();
                read_mf();
                read_xf();
            }
            constexpr int NG = NT / 4;   // groups of four n-tiles
            bf16x8 bt[2][4];
            read_bt(0, 0, bt[0]);
            // x scaled by the decay weights: the k-operand of the update
            bf16x8 xw[2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const f32x4 w0 = *reinterpret_cast<const f32x4 *>(&wd.w[32 * ks + 8 * lgrp]);
                const f32x4 w1 = *reinterpret_cast<const f32x4 *>(&wd.w[32 * ks + 8 * lgrp + 4]);
                f32x4 x0, x1;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x0[e] = (float)xf[ks][e] * w0[e];
                    x1[e] = (float)xf[ks][4 + e] * w1[e];
                }
                xw[ks] = to_bf16x8(x0, x1);
            }
            // plus the masked intra-block product (D x_i on the diagonal); y of
            // sub-block t into YS
#pragma unroll
            for (int it = 0; it < 4; ++it) Y[it] *= rd[it];
#pragma unroll
            for (int it = 0; it < 4; ++it)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    if (!(ks == 1 && it < 2)) Y[it] = mfma(xf[ks], mf[it][ks], Y[it]);
            {
                unsigned char *Yw = reinterpret_cast<unsigned char *>(sm.YS[par]);
#pragma unroll
                for (int it = 0; it < 4; ++it)
                    lds_st<uint2>(Yw + ysw + it * 2048, uint2{pack2(Y[it][0], Y[it][1]), pack2(Y[it][2], Y[it][3])});
            }
            __builtin_amdgcn_sched_barrier(0);

            // state update over sub-block t: H <- exp(Lambda_63) H + sum_j Bm_j (outer) (w_j x_j)
#pragma unroll
            for (int u = 0; u < NT; ++u) Hacc[u] *= gam;
#pragma unroll
            for (int r = 0; r < 2 * NG; ++r) {
                const int ks = r / NG, v4 = r % NG;
                if (r + 1 < 2 * NG) read_bt((r + 1) / NG, (r + 1) % NG, bt[(r + 1) & 1]);
#pragma unroll
                for (int u = 0; u < 4; ++u) Hacc[4 * v4 + u] = mfma(bt[r & 1][u], xw[ks], Hacc[4 * v4 + u]);
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (!kPrepX) xd_x(t, par);
            __syncthreads();
        };
        // steps [t0, t1) with the parity of each step known at compile time
        auto run = [&](int t0, int t1) __attribute__((always_inline)) {
            int t = t0;
            if ((t & 1) && t < t1) {
                step(t, 1);
                ++t;
            }
            for (; t + 1 < t1; t += 2) {
                step(t, 0);
                step(t + 1, 1);
            }
            if (t < t1) step(t, 0);
        };
        run(0, nown);
        if (has_x) {
            switch_to_segment();
            run(nown, T);
        }
        __syncthreads();   // matches the prep waves' final barrier
        store_y(T - 1, (T - 1) & 1);
        // final state of the own sequence, or (the segment ran last) of the
        // further sequence after its last segment
        if (a.final_state && (!has_x || xq == a.nseg - 1)) {
            float *dst = a.final_state + (has_x ? xchain : chain) * (kP * N) + lane_off;
#pragma unroll
            for (int u = 0; u < NT; ++u) *reinterpret_cast<f32x4 *>(dst + 16 * u) = Hacc[u];
        }
    } else {
        // ------------------------------------------------------------------
        // prep waves: in step t the masked decay matrix of sub-block t+1 (this
        // wave's tiles, from its gram tiles and a prefix scan of dt*A) and its
        // Bm, Cm into LDS
        BulkBC<N> bulk[2];   // Bm, Cm of step t+1 (staged at the end of step t) and t+2
        // decays and this wave's tiles of the masked matrix of the sub-block
        // of step tau, from sl, into Mm[slot]
        auto build_m = [&](int tau, const uint2 (&gt)[3], int slot) __attribute__((always_inline)) {
            const bool xs = tau >= nown;
            const float Ah2 = xs ? Ahx2 : Ah2v;
            const float Dh = xs ? Dhx : Dhv;
            const float *dtrow = sm.dts[tau & 3];
            const float dself = dtrow[lane];
            uint64_t rm = 0;
            if constexpr (kV) rm = reset_mask(dself);
            wd.lam[lane] = wave_scan((kV ? dt_mag(dself) : dself) * Ah2);
            uint2 mt[3];
#pragma unroll
            for (int m = 0; m < 3; ++m) {
                const int k = pq + 4 * m < 10 ? pq + 4 * m : 9;
                int ti, tj;
                tile_of(k, ti, tj);
                const int i = 16 * ti + lrow, j0 = 16 * tj + 4 * lgrp;
                const float li = wd.lam[i];
                const f32x4 lj = *reinterpret_cast<const f32x4 *>(&wd.lam[j0]);
                const f32x4 dj = *reinterpret_cast<const f32x4 *>(&dtrow[j0]);
                const uint32_t gw[2] = {gt[m].x, gt[m].y};
                // token j reaches token i when j <= i and no reset lies in (j, i]
                const int rho = kV ? last_reset(rm, i) : -1;
                float mv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float gv = (e & 1) ? hi_bf16(gw[e >> 1]) : lo_bf16(gw[e >> 1]);
                    const float d = (j0 + e <= i && j0 + e >= rho) ? li - lj[e] : -__builtin_inff();
                    // the skip term D x_i rides on the diagonal
                    mv[e] = __builtin_fmaf(gv * ex2(d), kV ? dt_mag(dj[e]) : dj[e], j0 + e == i ? Dh : 0.f);
                }
                mt[m] = uint2{pack2(mv[0], mv[1]), pack2(mv[2], mv[3])};
            }
            unsigned char *Mw = reinterpret_cast<unsigned char *>(sm.Mm[slot]);
#pragma unroll
            for (int m = 0; m < 3; ++m) {
                const int k = pq + 4 * m;
                if (k < 10) {
                    int ti, tj;
                    tile_of(k, ti, tj);
                    lds_st<uint2>(Mw + 16 * ti * 128 + (o.mw ^ (32 * tj)), mt[m]);
                }
            }
            if (pq >= 2) {
                // the tiles above the diagonal that the products read: (0,1) and (2,3)
                const int ti = pq == 2 ? 0 : 2;
                uint32_t z = 0;
                asm volatile("" : "+v"(z));
                lds_st<uint2>(Mw + 16 * ti * 128 + (o.mw ^ (32 * (ti + 1))), uint2{z, z});
            }
        };
        // prologue: Bm, Cm of sub-block 0 staged and its masked matrix built;
        // the G tiles of sub-blocks 1 and 2 and Bm, Cm of sub-block 1 in
        // flight, issued in the order a step issues them (G tiles, then Bm,
        // Cm), so that the loop is entered with the loads of its steady state
        uint2 gt[2][3];
        if constexpr (kPrepX) xd_prologue();
        {
            const int t1 = T > 1 ? 1 : 0, t2 = T > 2 ? 2 : T - 1;
            load_g_at(gt[0], a, g_at(0), q_of(0), pq, lane);
            load_g_at(gt[1], a, g_at(t1), q_of(t1), pq, lane);
            load_bc_at<N>(bulk[0], a, o, b_at(0), q_of(0));
            stage_bc<N>(sm, 0, bulk[0], o);
            build_m(0, gt[0], 0);
            load_g_at(gt[0], a, g_at(t2), q_of(t2), pq, lane);
            load_bc_at<N>(bulk[1], a, o, b_at(t1), q_of(t1));
        }
        __syncthreads();
        // Every step issues the same global loads (loads past the last
        // sub-block repeat it), so that the wait counts the compiler derives
        // at the loop head are those of the steady state.
        auto step = [&](int t, int par) __attribute__((always_inline)) {
            if constexpr (kPrepX) {
                // Bm of sub-block t+1 (its slot was last read in step t-1) and
                // the loads of t+2, the dt and x duties; after the compute
                // waves are done with Cm (the middle barrier), Cm of t+1 and
                // the masked matrix of t+1, then the G tiles of t+3 into the
                // slot just used
                stage_b<N>(sm, par ^ 1, bulk[par ^ 1], o);
                {
                    const int tl = t + 2 < T ? t + 2 : T - 1;
                    load_bc_at<N>(bulk[par], a, o, b_at(tl), q_of(tl));
                }
                xd_dt(t, par);
                xd_x(t, par);
                __syncthreads();
                stage_c<N>(sm, bulk[par ^ 1], o);
                build_m(t + 1, gt[par ^ 1], par ^ 1);
                {
                    const int tl = t + 3 < T ? t + 3 : T - 1;
                    load_g_at(gt[par ^ 1], a, g_at(tl), q_of(tl), pq, lane);
                }
                __syncthreads();
                return;
            }
            // sub-block t+1 (its G tiles were loaded in step t-1, its dt is in
            // LDS), then the G tiles of t+3 into the same slot
            build_m(t + 1, gt[par ^ 1], par ^ 1);
            {
                const int tl = t + 3 < T ? t + 3 : T - 1;
                load_g_at(gt[par ^ 1], a, g_at(tl), q_of(tl), pq, lane);
            }
            {
                const int tl = t + 2 < T ? t + 2 : T - 1;
                load_bc_at<N>(bulk[par], a, o, b_at(tl), q_of(tl));
            }
            stage_bc<N>(sm, par ^ 1, bulk[par ^ 1], o);   // unconditional, as stage_x
            __syncthreads();
        };
        int t = 0;
        for (; t + 1 < T; t += 2) {
            step(t, 0);
            step(t + 1, 1);
        }
        if (t < T) step(t, 0);
        __syncthreads();   // matches the compute waves' final barrier
    }
}

// The state that segment q of further sequence e produces from a zero state,
// S = sum over its sub-blocks of the state update, and log2 of its total decay
// (the sum of dt*A over the segment, in base-2 units).  The main kernel
// combines these into each segment's entering state:
// H_{q+1} = 2^(log2 decay_q) H_q + S_q.
//
// A step takes a pair of sub-blocks (a, b) as one 128-token update:
// H <- 2^(l_a + l_b) H + sum_j Bm_j (w_j x_j), w_j = 2^(Lambda_end - Lambda_j) dt_j,
// with Lambda the running sum of dt*A (log2 units) over the pair and l_c the
// total of sub-block c.
//  - Wave 0 alone loads dt (a row of one float per token touches 64 cache
//    lines per sub-block, so it is loaded once per workgroup), three steps
//    ahead, and two steps ahead scans it into the pair's weights and decay,
//    published through a three-slot LDS ring.
//  - The weights are applied to x as it is staged (each x element is
//    multiplied once), so the matrix-core operands come straight from LDS.
//  - The eight waves form two groups, group c taking sub-block c of every
//    pair into a partial state of its own (the two add up to S at the end);
//    in a group, wave (nq, pp) holds n-tiles nq*NT/2 .. +NT/2-1 and p-tiles
//    2pp, 2pp+1, so each fragment read from LDS serves two waves.
// Register slot s % 2 holds the pair of step s from its load (issued in step
// s - 2) until it is staged to LDS slot s % 2 at the end of step s - 1.  A
// pair that runs past the segment's end gets dt = 0 for its missing
// sub-block: weight 0, decay 1.
template <int N, bool kV>
__device__ __forceinline__ void seg_state_block(const Args &a, int blk) {
    __shared__ __align__(16) __bf16 lds_x[2][2][kSub * kP];
    __shared__ __align__(16) __bf16 lds_bt[2][2][kSub * N];
    __shared__ __align__(16) float lds_w[3][2][kSub];
    __shared__ float lds_l[3];
    using O = LaneOffs<N>;
    constexpr int NT = N / 16, NTW = NT / 2;  // n-tiles in all, per wave
    constexpr int KB = N / 64;                // Bm chunks staged per thread and sub-block
    static_assert(sizeof(lds_bt) >= 4 * NTW * 2 * 64 * sizeof(f32x4), "reduction room");
    const int xe = blk % a.nextra, q = blk / a.nextra;
    const int64_t chain = a.nmain + xe;
    const int64_t b = __builtin_amdgcn_readfirstlane((int)(chain / a.H));
    const int64_t h = __builtin_amdgcn_readfirstlane((int)(chain % a.H));
    const int64_t g = __builtin_amdgcn_readfirstlane((int)(h / (a.H / a.G)));
    const int64_t dh = h / a.hs;
    const float Ah2 = a.A[dh] * kLog2e;
    const int s0 = q * a.seglen, len = a.seglen;   // segments before the last are full and inside the sequence
    const int nsteps = (len + 1) / 2;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2, wq = wave & 3, nq = wq & 1, pp = wq >> 1;
    const int lane = tid & 63, lrow = lane & 15, lgrp = lane >> 4;
    const LaneOffs<N> o = lane_offsets<N>(tid, 2 * pp, a.H, a.G, a.Hd);
    const int xtr1 = lane_offsets<N>(tid, 2 * pp + 1, a.H, a.G).xtr;   // second p-tile
    // staging: thread (u = tid % 256, half nh) stages x chunk nh (token
    // u / 8 + 32 nh) and Bm chunks nh*KB .. +KB-1 of u, of each sub-block
    const int nh = tid >> 8;
    const int my_token = ((tid & 255) >> 3) + 32 * nh;

    auto sub_at = [&](int st, int c) __attribute__((always_inline)) {
        const int k = 2 * st + c;
        return k < len ? k : len - 1;
    };
    uint4 xr[2][2], br[2][2][KB];
    auto load = [&](int st, int slot) __attribute__((always_inline)) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int k = sub_at(st, c);
            const int qn = sub_tokens(a, s0 + k);
            const int64_t row0 = b * a.L + (int64_t)(s0 + k) * kSub;
            const rsrc_t rx = rsrc(a.x + (row0 * a.H + h) * kP, (int)(((int64_t)(qn - 1) * a.H * kP + kP) * 2));
            xr[slot][c] = ld16(rx, o.gx + nh * (int)(32 * a.H * kP * 2));
            const rsrc_t rb = rsrc(a.Bm + (row0 * a.G + g) * N, (int)(((int64_t)(qn - 1) * a.G * N + N) * 2));
            const int step = (int)((256 / O::CPR) * a.G * N * 2);
#pragma unroll
            for (int kk = 0; kk < KB; ++kk) br[slot][c][kk] = ld16(rb, o.gb + (nh * KB + kk) * step);
        }
    };
    // wave 0: dt of the pair of step st (lane = token) into register slot `slot`
    float dts[2][2];
    auto load_dt = [&](int st, int slot) __attribute__((always_inline)) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int k = sub_at(st, c);
            const int qn = sub_tokens(a, s0 + k);
            const int64_t row0 = b * a.L + (int64_t)(s0 + k) * kSub;
            const rsrc_t rd = rsrc(a.dt + row0 * a.Hd + dh, (int)(((int64_t)(qn - 1) * a.Hd + 1) * 4));
            dts[slot][c] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rd, o.gd, 0, 0));
        }
    };
    // wave 0: weights and log2 decay of the pair of step st into ring slot st % 3
    auto weights = [&](int st, int slot) __attribute__((always_inline)) {
        const float dra = dts[slot][0];
        const float drb = 2 * st + 1 < len ? dts[slot][1] : 0.f;
        const float dta = kV ? dt_mag(dra) : dra, dtb = kV ? dt_mag(drb) : drb;
        const float va = wave_scan(dta * Ah2), vb = wave_scan(dtb * Ah2);
        const float la = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(va), 63));
        const float lb = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(vb), 63));
        const int r = st % 3;
        float wa = ex2(la + lb - va) * dta, wb = ex2(lb - vb) * dtb, lp = la + lb;
        if constexpr (kV) {
            // a reset in the pair: nothing before it reaches the pair's end,
            // and the pair's decay is zero (log2 -inf)
            const uint64_t ma = reset_mask(dra), mb = reset_mask(drb);
            if (mb) {
                if (lane < 63 - (int)__builtin_clzll(mb)) wb = 0.f;
                wa = 0.f;
                lp = -__builtin_inff();
            }
            if (ma) {
                if (lane < 63 - (int)__builtin_clzll(ma)) wa = 0.f;
                lp = -__builtin_inff();
            }
        }
        lds_w[r][0][lane] = wa;
        lds_w[r][1][lane] = wb;
        if (lane == 0) lds_l[r] = lp;
    };
    // x of the pair of step st (register slot `slot`) times its weights, and
    // Bm, into LDS slot `slot`
    auto stage = [&](int st, int slot) __attribute__((always_inline)) {
        const int r = st % 3;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            unsigned char *Xb = reinterpret_cast<unsigned char *>(lds_x[slot][c]);
            unsigned char *Bb = reinterpret_cast<unsigned char *>(lds_bt[slot][c]);
            const float w = lds_w[r][c][my_token];
            const bf16x8 xv = __builtin_bit_cast(bf16x8, xr[slot][c]);
            f32x4 x0, x1;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x0[e] = (float)xv[e] * w;
                x1[e] = (float)xv[4 + e] * w;
            }
            lds_st<bf16x8>(Xb + o.sx + nh * 4096, to_bf16x8(x0, x1));
#pragma unroll
            for (int kk = 0; kk < KB; ++kk)
                lds_st<uint4>(Bb + o.sb + (nh * KB + kk) * (256 / O::CPR) * O::RB, br[slot][c][kk]);
        }
    };

    // prologue: pairs 0 and 1 loaded, weights of pairs 0 and 1, dt of pair 2
    // in flight, pair 0 staged
    load(0, 0);
    load(nsteps > 1 ? 1 : 0, 1);
    if (wave == 0) {
        load_dt(0, 0);
        load_dt(1, 1);
        weights(0, 0);
        load_dt(2, 0);
        weights(1, 1);
    }
    __syncthreads();
    stage(0, 0);
    __syncthreads();

    f32x4 Hacc[NTW][2];
#pragma unroll
    for (int u = 0; u < NTW; ++u) Hacc[u][0] = Hacc[u][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    float log2dec = 0.f;
    auto step = [&](int st, int par) __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        const float lpair = lds_l[st % 3];
        log2dec += lpair;
        // the pair of step st+2 into the register slot staged at the end of the last step
        load(st + 2 < nsteps ? st + 2 : nsteps - 1, par);
        if (wave == 0) {
            load_dt(st + 3, par ^ 1);   // the slot whose pair (st+1) was scanned in the last step
            weights(st + 2, par);
        }
        const float gam = ex2(lpair);
#pragma unroll
        for (int u = 0; u < NTW; ++u) {
            Hacc[u][0] *= gam;
            Hacc[u][1] *= gam;
        }
        const unsigned char *Xb = reinterpret_cast<const unsigned char *>(lds_x[par][grp]);
        const unsigned char *Bb = reinterpret_cast<const unsigned char *>(lds_bt[par][grp]);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            bf16x8 xw[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int xo = (j ? xtr1 : o.xtr) + ks * 4096;
                const bf16x4 lo = tr4(Xb + xo), hi = tr4(Xb + xo + 512);
                xw[j] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            }
#pragma unroll
            for (int u = 0; u < NTW; ++u) {
                const int bo = nq ? o.bt[NTW + u] : o.bt[u];   // (no run-time index into o)
                const bf16x4 blo = tr4(Bb + bo + ks * 32 * O::RB);
                const bf16x4 bhi = tr4(Bb + bo + ks * 32 * O::RB + 4 * O::RB);
                const bf16x8 bt = bf16x8{blo[0], blo[1], blo[2], blo[3], bhi[0], bhi[1], bhi[2], bhi[3]};
                Hacc[u][0] = mfma(bt, xw[0], Hacc[u][0]);
                Hacc[u][1] = mfma(bt, xw[1], Hacc[u][1]);
            }
        }
        // unconditional (clamped) loads and stages: the same memory operations
        // in every step, so that the wait counts need not cover a shorter path
        stage(st + 1, par ^ 1);
        __syncthreads();
    };
    int st = 0;
    for (; st + 1 < nsteps; st += 2) {
        step(st, 0);
        step(st + 1, 1);
    }
    if (st < nsteps) step(st, 0);
    // S = group 0's partial + group 1's (passed through LDS, free after the last barrier)
    f32x4 *red = reinterpret_cast<f32x4 *>(&lds_bt[0][0][0]) + (wq * NTW * 2) * 64 + lane;
    if (grp == 1) {
#pragma unroll
        for (int u = 0; u < NTW; ++u) {
            red[(2 * u) * 64] = Hacc[u][0];
            red[(2 * u + 1) * 64] = Hacc[u][1];
        }
    }
    __syncthreads();
    if (grp == 0) {
        float *dst = seg_state<N>(a, xe, q) + (32 * pp + lrow) * N + 16 * NTW * nq + 4 * lgrp;
#pragma unroll
        for (int u = 0; u < NTW; ++u)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                *reinterpret_cast<f32x4 *>(dst + 16 * j * N + 16 * u) = Hacc[u][j] + red[(2 * u + j) * 64];
        if (tid == 0) *seg_log2decay<N>(a, xe, q) = log2dec;
    }
}

// The same segment states at N = 256, where the pair layout's LDS (two slots
// of two sub-blocks of Bm) does not fit: one sub-block per step, and the
// eight waves split the state instead of the tokens.  Wave w holds n-tiles
// 4(w & 3) .. +3 and p-tiles 2(w >> 2), +1 (an x fragment serves four waves,
// a Bm fragment two); no partial states to add up at the end.  Wave 0 loads
// dt three steps ahead and scans it two steps ahead into a three-slot LDS
// ring of weights and log2 decays; x is multiplied by its weights as it is
// staged.  Register slot s % 2 holds sub-block s from its load (step s - 2)
// until it is staged to LDS slot s % 2 at the end of step s - 1.
template <int N, bool kV>
__device__ __forceinline__ void seg_state_block_wide(const Args &a, int blk) {
    __shared__ __align__(16) __bf16 lds_x[2][kSub * kP];
    __shared__ __align__(16) __bf16 lds_bt[2][kSub * N];
    __shared__ __align__(16) float lds_w[3][kSub];
    __shared__ float lds_l[3];
    using O = LaneOffs<N>;
    constexpr int NTW = 4;        // n-tiles per wave
    constexpr int KB = N / 64;    // Bm chunks staged per thread
    const int xe = blk % a.nextra, q = blk / a.nextra;
    const int64_t chain = a.nmain + xe;
    const int64_t b = __builtin_amdgcn_readfirstlane((int)(chain / a.H));
    const int64_t h = __builtin_amdgcn_readfirstlane((int)(chain % a.H));
    const int64_t g = __builtin_amdgcn_readfirstlane((int)(h / (a.H / a.G)));
    const int64_t dh = h / a.hs;
    const float Ah2 = a.A[dh] * kLog2e;
    const int s0 = q * a.seglen, len = a.seglen;   // segments before the last are full and inside the sequence

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nq = wave & 3, pp = wave >> 2;
    const int lane = tid & 63, lrow = lane & 15, lgrp = lane >> 4;
    const LaneOffs<N> o = lane_offsets<N>(tid, 2 * pp, a.H, a.G, a.Hd);
    const int xtr1 = lane_offsets<N>(tid, 2 * pp + 1, a.H, a.G).xtr;   // second p-tile
    // staging: thread (u = tid % 256, half nh) stages x chunk nh (token
    // u / 8 + 32 nh) and Bm chunks nh*KB .. +KB-1 of u
    const int nh = tid >> 8;
    const int my_token = ((tid & 255) >> 3) + 32 * nh;

    auto sub_at = [&](int st) __attribute__((always_inline)) { return st < len ? st : len - 1; };
    uint4 xr[2], br[2][KB];
    auto load = [&](int st, int slot) __attribute__((always_inline)) {
        const int k = sub_at(st);
        const int qn = sub_tokens(a, s0 + k);
        const int64_t row0 = b * a.L + (int64_t)(s0 + k) * kSub;
        const rsrc_t rx = rsrc(a.x + (row0 * a.H + h) * kP, (int)(((int64_t)(qn - 1) * a.H * kP + kP) * 2));
        xr[slot] = ld16(rx, o.gx + nh * (int)(32 * a.H * kP * 2));
        const rsrc_t rb = rsrc(a.Bm + (row0 * a.G + g) * N, (int)(((int64_t)(qn - 1) * a.G * N + N) * 2));
        const int step = (int)((256 / O::CPR) * a.G * N * 2);
#pragma unroll
        for (int kk = 0; kk < KB; ++kk) br[slot][kk] = ld16(rb, o.gb + (nh * KB + kk) * step);
    };
    // wave 0: dt of sub-block st (lane = token) into register slot `slot`
    float dts[2];
    auto load_dt = [&](int st, int slot) __attribute__((always_inline)) {
        const int k = sub_at(st);
        const int qn = sub_tokens(a, s0 + k);
        const int64_t row0 = b * a.L + (int64_t)(s0 + k) * kSub;
        const rsrc_t rd = rsrc(a.dt + row0 * a.Hd + dh, (int)(((int64_t)(qn - 1) * a.Hd + 1) * 4));
        dts[slot] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rd, o.gd, 0, 0));
    };
    // wave 0: weights and log2 decay of sub-block st into ring slot st % 3
    auto weights = [&](int st, int slot) __attribute__((always_inline)) {
        const float dr = dts[slot];
        const float d = kV ? dt_mag(dr) : dr;
        const float v = wave_scan(d * Ah2);
        const float l = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
        float w = ex2(l - v) * d, ls = l;
        if constexpr (kV) {
            // a reset: nothing before it reaches the end, and the decay is zero
            const uint64_t m = reset_mask(dr);
            if (m) {
                if (lane < 63 - (int)__builtin_clzll(m)) w = 0.f;
                ls = -__builtin_inff();
            }
        }
        lds_w[st % 3][lane] = w;
        if (lane == 0) lds_l[st % 3] = ls;
    };
    // x of sub-block st (register slot `slot`) times its weights, and Bm,
    // into LDS slot `slot`
    auto stage = [&](int st, int slot) __attribute__((always_inline)) {
        unsigned char *Xb = reinterpret_cast<unsigned char *>(lds_x[slot]);
        unsigned char *Bb = reinterpret_cast<unsigned char *>(lds_bt[slot]);
        const float w = lds_w[st % 3][my_token];
        const bf16x8 xv = __builtin_bit_cast(bf16x8, xr[slot]);
        f32x4 x0, x1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x0[e] = (float)xv[e] * w;
            x1[e] = (float)xv[4 + e] * w;
        }
        lds_st<bf16x8>(Xb + o.sx + nh * 4096, to_bf16x8(x0, x1));
#pragma unroll
        for (int kk = 0; kk < KB; ++kk) {
            const int k = nh * KB + kk;
            lds_st<uint4>(Bb + (o.sb ^ sb_flip<N>(k)) + k * (256 / O::CPR) * O::RB, br[slot][kk]);
        }
    };

    // prologue: sub-blocks 0 and 1 loaded, weights of 0 and 1, dt of 2 in
    // flight, sub-block 0 staged
    load(0, 0);
    load(1, 1);
    if (wave == 0) {
        load_dt(0, 0);
        load_dt(1, 1);
        weights(0, 0);
        load_dt(2, 0);
        weights(1, 1);
    }
    __syncthreads();
    stage(0, 0);
    __syncthreads();

    f32x4 Hacc[NTW][2];
#pragma unroll
    for (int u = 0; u < NTW; ++u) Hacc[u][0] = Hacc[u][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    float log2dec = 0.f;
    auto step = [&](int st, int par) __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        const float lsub = lds_l[st % 3];
        log2dec += lsub;
        // sub-block st+2 into the register slot staged at the end of the last step
        load(st + 2, par);
        if (wave == 0) {
            load_dt(st + 3, par ^ 1);   // the slot whose sub-block (st+1) was scanned in the last step
            weights(st + 2, par);
        }
        const float gam = ex2(lsub);
#pragma unroll
        for (int u = 0; u < NTW; ++u) {
            Hacc[u][0] *= gam;
            Hacc[u][1] *= gam;
        }
        const unsigned char *Xb = reinterpret_cast<const unsigned char *>(lds_x[par]);
        const unsigned char *Bb = reinterpret_cast<const unsigned char *>(lds_bt[par]);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            bf16x8 xw[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int xo = (j ? xtr1 : o.xtr) + ks * 4096;
                const bf16x4 lo = tr4(Xb + xo), hi = tr4(Xb + xo + 512);
                xw[j] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            }
#pragma unroll
            for (int u = 0; u < NTW; ++u) {
                // n-tile 4nq + u: o.bt holds the first eight (no run-time index into o)
                const int bo = ((nq & 1) ? o.bt[4 + u] : o.bt[u]) + (nq >> 1) * 256;
                const bf16x4 blo = tr4(Bb + bo + ks * 32 * O::RB);
                const bf16x4 bhi = tr4(Bb + bo + ks * 32 * O::RB + 4 * O::RB);
                const bf16x8 bt = bf16x8{blo[0], blo[1], blo[2], blo[3], bhi[0], bhi[1], bhi[2], bhi[3]};
                Hacc[u][0] = mfma(bt, xw[0], Hacc[u][0]);
                Hacc[u][1] = mfma(bt, xw[1], Hacc[u][1]);
            }
        }
        // unconditional (clamped) loads and stages: the same memory operations
        // in every step, so that the wait counts need not cover a shorter path
        stage(st + 1, par ^ 1);
        __syncthreads();
    };
    int st = 0;
    for (; st + 1 < len; st += 2) {
        step(st, 0);
        step(st + 1, 1);
    }
    if (st < len) step(st, 0);
    float *dst = seg_state<N>(a, xe, q) + (32 * pp + lrow) * N + 16 * NTW * nq + 4 * lgrp;
#pragma unroll
    for (int u = 0; u < NTW; ++u)
#pragma unroll
        for (int j = 0; j < 2; ++j) *reinterpret_cast<f32x4 *>(dst + 16 * j * N + 16 * u) = Hacc[u][j];
    if (tid == 0) *seg_log2decay<N>(a, xe, q) = log2dec;
}

// The work that must precede pipe_kernel when there are segments, in one
// launch so that the two parts share the device: workgroups below nsegwg
// compute segment states, the others one sub-block's gram tiles each.
template <int N, bool kV>
__global__ __launch_bounds__(512) void prep_kernel(Args a, int nsegwg) {
    if ((int)blockIdx.x < nsegwg) {
        // the segment states of one segment index, which share Bm and dt
        // rows, on as few XCDs as possible (a bijection of 0 .. nsegwg-1)
        const int blk = (int)xcd_chain(blockIdx.x, nsegwg);
        if constexpr (N == 256)
            seg_state_block_wide<N, kV>(a, blk);
        else
            seg_state_block<N, kV>(a, blk);
    } else {
        const int64_t k = (int64_t)blockIdx.x - nsegwg;
        gram_block<N, 8>(a.Bm, a.Cm, const_cast<__bf16 *>(a.gram), a.L, a.G, a.nsb, k % a.nsb, k / a.nsb,
                         threadIdx.x);
    }
}

// Number of compute units of the current device (cached per device).
int device_cus() {
    static std::atomic<int> cached[kMaxDevices] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

template <int N, bool kV>
hipError_t launch(const ScanArgs &sa, const Workspace &ws) {
    const int64_t nsb = (sa.L + kSub - 1) / kSub;
    hipError_t e = hipSuccess;
    // Sequences are spread over the compute units in time segments whose
    // entering states come from the segment states of a first, shorter kernel:
    //  - more sequences than compute units (but fewer than twice as many): one
    //    workgroup per compute unit runs one sequence whole and then one
    //    segment of a remaining sequence;
    //  - at most half as many sequences as compute units: every sequence is
    //    cut into segments, one workgroup per segment;
    //  - otherwise one workgroup per sequence.
    // a head of P = 128 is scanned as two heads of 64 channels (the state
    // rows p < 64 and p >= 64 never mix), sharing dt, A and D
    const int hs = (int)(sa.P / kP);
    const int64_t Hk = sa.H * hs;
    const int64_t chains = sa.B * Hk;
    const int cus = device_cus();
    int nmain = (int)chains, nextra = 0, nseg = 1, seglen = (int)nsb;
    if (cus > 0 && chains > cus && chains < 2 * (int64_t)cus && nsb >= 2) {
        nmain = cus;
        nextra = (int)(chains - cus);
        nseg = cus / nextra;
    } else if (cus > 0 && 2 * chains <= cus && nsb >= 2) {
        nmain = 0;
        nextra = (int)chains;
        nseg = cus / nextra;
    }
    if (nextra > 0) {
        // no more segment states than the workspace holds
        const int64_t cap = (int64_t)(ws.seg_floats / ((size_t)kP * N + 1));
        if ((int64_t)nextra * (nseg - 1) > cap) nseg = (int)(1 + cap / nextra);
        if (nseg > nsb) nseg = (int)nsb;
        if (nseg < 1) nseg = 1;
        seglen = (int)((nsb + nseg - 1) / nseg);
        nseg = (int)((nsb + seglen - 1) / seglen);
    }
    const int nwg = nmain > 0 ? nmain : nextra * nseg;
    const size_t smem = sizeof(PipeSmem<N>);
    auto kern = pipe_kernel<N, kV>;
    static std::atomic<bool> configured[kMaxDevices] = {};
    e = allow_lds((const void *)kern, smem, configured);
    if (e != hipSuccess) return e;
    Args a{(const __bf16 *)sa.x, sa.dt, sa.A, (const __bf16 *)sa.Bm, (const __bf16 *)sa.Cm, sa.D,
           sa.init, (__bf16 *)sa.y, sa.final_state, (const __bf16 *)ws.gram, ws.seg,
           sa.L, Hk, sa.G, nsb, sa.H, hs, nmain, nextra, nseg, seglen};
    if (nextra > 0 && nseg > 1) {
        const int nsegwg = nextra * (nseg - 1);
        prep_kernel<N, kV><<<dim3((unsigned)(nsegwg + nsb * sa.B * sa.G)), 512, 0, sa.stream>>>(a, nsegwg);
    } else {
        e = launch_gram(sa, ws, nsb);
    }
    if (e != hipSuccess) return e;
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    kern<<<dim3((unsigned)nwg), kThreads, smem, sa.stream>>>(a);
    return hipGetLastError();
}

}  // namespace

bool pipe_supported(int64_t H, int64_t P, int64_t G, int64_t N) {
    if (!(N == 64 || N == 128 || N == 256) || !(P == 64 || P == 128)) return false;
    const int64_t lim = (int64_t)1 << 31;
    return (int64_t)kSub * H * P * 2 < lim && (int64_t)kSub * G * N * 2 < lim && (int64_t)kSub * H * 4 < lim;
}

hipError_t launch_pipe_scan(const ScanArgs &a, const Workspace &ws) {
    switch (a.N) {
        case 64: return a.varlen ? launch<64, true>(a, ws) : launch<64, false>(a, ws);
        case 128: return a.varlen ? launch<128, true>(a, ws) : launch<128, false>(a, ws);
        case 256: return a.varlen ? hipErrorInvalidValue : launch<256, false>(a, ws);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace ssd
