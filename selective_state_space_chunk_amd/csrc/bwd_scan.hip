// Backward of the chunk scan on gfx950: the gradients of
//   <dy, y> + <dfinal, final state>
// with respect to x, dt, A, Bm, Cm, D and the initial state, for P = 64 or
// 128, N in {64, 128}, bfloat16 x / Bm / Cm / y.  A head of 128 channels is
// taken as two heads of 64 (the state rows p < 64 and p >= 64 never mix) that
// share dt, A and D; the gradients of those shared inputs are the sums over
// the two halves.
//
// The recurrence is the one of the "Mamba-2" note (section "writing the SSM
// as a matrix", one decay per head as in "reducing A to a number"), cut into
// 64-token sub-blocks as in the block decomposition of the "Mamba-2 model
// walkthrough" (section 6.1).  Only the states are sequential, so the work is
// split into
//   1. state_scans<N> (first half of its workgroups): the state H_c entering
//      every sub-block c;
//   2. state_scans<N> (second half): backwards in time, the adjoint dH'_c of the state
//      leaving every sub-block, dH_c = g_c dH'_c + sum_i exp(Lambda_i) dy_i (x) Cm_i,
//      whose last value is the initial state's gradient;
//   3. chunk_grad<N>: one workgroup per (batch, group, sub-block), all in
//      parallel: from H_c, dH'_c and the sub-block's inputs, for each head of
//      the group dx and ddt of its tokens and its parts of dA, dD; dBm and
//      dCm summed over the group's heads;
//   4. sums of the dA, dD parts over batch rows and sub-blocks.
// The states and adjoints are kept in bfloat16: they enter the products as
// bfloat16 operands.
// Within sub-block c (tokens i, j; Lambda the running sum of dt*A, E_ij =
// exp(Lambda_i - Lambda_j) for j <= i, w_j = exp(Lambda_63 - Lambda_j) dt_j):
//   dx_j  = sum_i M_ij dy_i + w_j dH' Bm_j,      M_ij = (Cm_i.Bm_j) E_ij dt_j + D [i=j]
//   dCm_i = exp(Lambda_i) H^T dy_i + sum_j Q_ij Bm_j,   Q_ij = (dy_i.x_j) E_ij dt_j
//   dBm_j = w_j dH'^T x_j + sum_i Q_ij Cm_i
// and dt enters through Lambda (d/dLambda_i collected per token, then summed
// over i >= k for dt_k) and directly through the factors dt_j.
#include "common.h"
#include "tile_ops.h"

namespace ssd {
namespace {

using namespace tile;

constexpr float kLog2eB = 1.4426950408889634f;

struct BwdArgs {
    const __bf16 *x, *dy, *Bm, *Cm;
    const float *dt, *A, *D, *init, *dfinal;   // init, dfinal nullable
    __bf16 *dx, *dBm, *dCm;
    float *ddt, *dA, *dD, *dinit;              // dinit nullable
    float *Hs;    // [B*H, nsb, P*N] bf16  state entering each sub-block
    float *dHs;   // [B*H, nsb, P*N] bf16  adjoint of the state leaving each sub-block
                  // (both in accumulator order, two tiles per lane and store: the
                  //  16-byte unit ((pq*NT/2 + v)*64 + lane) holds p = 16pq + lane%16,
                  //  n = 32v + 4(lane/16) + 0..3, then n + 16 .. + 19)
    float *dAp;   // [B*Hd, nsb]  each head's part of dA from each sub-block
    float *dDp;   // [B*Hd, nsb]
    int64_t B, L, H, G, nsb;   // H: heads of 64 channels (x, dy, dx, states, init, dfinal, dinit)
    int64_t Hd;                // the caller's heads (dt, ddt, A, D, dA, dD): H / hs
    int hs;                    // heads of 64 channels per caller head (1 or 2)
};

__device__ __forceinline__ float ex2f(float v) { return __builtin_amdgcn_exp2f(v); }
typedef __bf16 bf16x2_dot __attribute__((ext_vector_type(2)));

// 16 bytes of the stored states and adjoints, written non-temporally by the
// state scans and read the same way by the sub-block gradients: each is
// written once and read once by the other kernel, and together they are
// larger than the caches (800 against 809 us per call at the 2.7B shape)
typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void st_nt16(void *p, const uint4 &v) {
    __builtin_nontemporal_store(u32x4_nt{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4_nt *>(p));
}
__device__ __forceinline__ uint4 ld_nt16(const void *p) {
    const u32x4_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt *>(p));
    return uint4{v.x, v.y, v.z, v.w};
}

// Waits for the loads of the state held in H before a step loop (otherwise
// the loop's wait counts, derived for every path into it, make each step wait
// for the latest loads where it first reads the state).
template <int NT>
__device__ __forceinline__ void settle(f32x4 (&H)[NT]) {
#pragma unroll
    for (int u = 0; u < NT; ++u) asm volatile("" ::"v"(H[u]));
}

__device__ __forceinline__ float lane_get(float v, int src) {
    return __int_as_float(__builtin_amdgcn_ds_bpermute(4 * src, __float_as_int(v)));
}
// sum over the 16 lanes of a row with DPP (no LDS round trips): lane pairs,
// then quads, then the two halves of each 8, then the two 8s of the row; every
// lane of the row ends with the sum
template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xf, 0xf, true));
}
__device__ __forceinline__ float row_sum16(float v) {
    v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
    v += dpp<0x141>(v);   // row_half_mirror
    v += dpp<0x140>(v);   // row_mirror
    return v;
}
// sum over the four 16-lane rows of a wave (lanes l, l + 16, l + 32, l + 48),
// the same value in all four, by the row-swapping permutes (no LDS): halves
// first, then adjacent rows
__device__ __forceinline__ float rows_sum4(float v) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
// sum over the wave, the same value in every lane (fixed order: deterministic)
__device__ __forceinline__ float wave_sum(float v) {
    const int r = __float_as_int(row_sum16(v));
    return (__int_as_float(__builtin_amdgcn_readlane(r, 0)) + __int_as_float(__builtin_amdgcn_readlane(r, 16))) +
           (__int_as_float(__builtin_amdgcn_readlane(r, 32)) + __int_as_float(__builtin_amdgcn_readlane(r, 48)));
}

// ---------------------------------------------------------------------------
// 1, 2. The sequential state scans, one workgroup (four waves) per (batch,
// head).  Wave pq holds rows p = 16pq..16pq+15 of the P x N state, transposed
// in the matrix-core accumulators as the forward kernels hold it (lane: n =
// 16u + 4lgrp + 0..3, p = 16pq + lrow).  Step by step it stores the state of
// the step, then applies  S <- g S + sum_t Mt_t (x) (om_t u_t):
//   forward:  u = x,  Mt = Bm, om_t = exp(Lambda_63 - Lambda_t) dt_t, from the
//             initial state, walking c = 0 .. nsb-1 and storing H_c;
//   backward: u = dy, Mt = Cm, om_t = exp(Lambda_t), from dfinal, walking
//             c = nsb-1 .. 0 and storing dH'_c; the last state is dinit.
// with g = exp(Lambda_63) of the sub-block in both.
template <int N, bool kRev>
__device__ __forceinline__ void state_scan_body(const BwdArgs &a, int64_t bh) {
    __shared__ __align__(16) __bf16 lx[kSub * kP];
    __shared__ __align__(16) __bf16 lb[kSub * N];
    using O = LaneOffs<N>;
    constexpr int NT = N / 16, KB = N / 32;
    const int64_t b = bh / a.H, h = bh % a.H, g = h / (a.H / a.G), dh = h / a.hs;
    const float Ah2 = a.A[dh] * kLog2eB;
    const int tid = threadIdx.x;
    const int pq = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, lrow = lane & 15, lgrp = lane >> 4;
    const LaneOffs<N> o = lane_offsets<N>(tid, pq, a.H, a.G, a.Hd);
    const __bf16 *U = kRev ? a.dy : a.x;
    const __bf16 *Mt = kRev ? a.Cm : a.Bm;
    const int nsb = (int)a.nsb;

    // register slot s % 2 holds the inputs of step s from its load (in step
    // s - 2) until they are staged at the start of step s
    uint4 ur[2][2], mr[2][KB];
    float dtv[2];
    auto load = [&](int s, int slot) __attribute__((always_inline)) {
        s = s < nsb ? s : nsb - 1;
        const int c = kRev ? nsb - 1 - s : s;
        const int64_t t0 = (int64_t)c * kSub;
        const int q = a.L - t0 < kSub ? (int)(a.L - t0) : kSub;
        const int64_t row0 = b * a.L + t0;
        const rsrc_t ru = rsrc(U + (row0 * a.H + h) * kP, (int)(((int64_t)(q - 1) * a.H * kP + kP) * 2));
#pragma unroll
        for (int k = 0; k < 2; ++k) ur[slot][k] = ld16(ru, o.gx + k * (int)(32 * a.H * kP * 2));
        const rsrc_t rm = rsrc(Mt + (row0 * a.G + g) * N, (int)(((int64_t)(q - 1) * a.G * N + N) * 2));
        const int step = (int)((256 / O::CPR) * a.G * N * 2);
#pragma unroll
        for (int k = 0; k < KB; ++k) mr[slot][k] = ld16(rm, o.gb + k * step);
        const rsrc_t rd = rsrc(a.dt + row0 * a.Hd + dh, (int)(((int64_t)(q - 1) * a.Hd + 1) * 4));
        dtv[slot] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rd, o.gd, 0, 0));
    };

    const int lane_off = (16 * pq + lrow) * N + 4 * lgrp;
    f32x4 Hacc[NT];
    {
        const float *src = kRev ? a.dfinal : a.init;
#pragma unroll
        for (int u = 0; u < NT; ++u)
            Hacc[u] = src ? *reinterpret_cast<const f32x4 *>(src + bh * (kP * N) + lane_off + 16 * u)
                          : f32x4{0.f, 0.f, 0.f, 0.f};
        settle(Hacc);
    }
    load(0, 0);
    load(1, 1);
    // states go out in accumulator order, two n-tiles per lane: 1 KB of
    // contiguous bytes per store
    __bf16 *sbase = reinterpret_cast<__bf16 *>(kRev ? a.dHs : a.Hs) + bh * a.nsb * (kP * N) +
                    8 * (pq * (NT / 2) * 64 + lane);
    const int row_k0 = tid >> 3;   // staged rows row_k0 and row_k0 + 32 of u
    auto step = [&](int s, int par) __attribute__((always_inline)) {
        const int c = kRev ? nsb - 1 - s : s;
        const float v = wave_scan(dtv[par] * Ah2);
        const float lend = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
        const float om = kRev ? ex2f(v) : ex2f(lend - v) * dtv[par];
        const float gam = ex2f(lend);
#pragma unroll
        for (int v = 0; v < NT / 2; ++v)
            st_nt16(sbase + (int64_t)c * (kP * N) + 8 * 64 * v,
                    uint4{pack2(Hacc[2 * v][0], Hacc[2 * v][1]), pack2(Hacc[2 * v][2], Hacc[2 * v][3]),
                          pack2(Hacc[2 * v + 1][0], Hacc[2 * v + 1][1]), pack2(Hacc[2 * v + 1][2], Hacc[2 * v + 1][3])});
        // u weighted by om, and Mt, into LDS
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const float wgt = lane_get(om, row_k0 + 32 * k);
            const bf16x8 xv = __builtin_bit_cast(bf16x8, ur[par][k]);
            f32x4 x0, x1;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x0[e] = (float)xv[e] * wgt;
                x1[e] = (float)xv[4 + e] * wgt;
            }
            lds_st<bf16x8>(reinterpret_cast<unsigned char *>(lx) + o.sx + k * 4096, to_bf16x8(x0, x1));
        }
#pragma unroll
        for (int k = 0; k < KB; ++k)
            lds_st<uint4>(reinterpret_cast<unsigned char *>(lb) + o.sb + k * (256 / O::CPR) * O::RB, mr[par][k]);
        // step s+2 into the slot just staged (past the end it loads the last one again)
        load(s + 2, par);
        __syncthreads();
#pragma unroll
        for (int u = 0; u < NT; ++u) Hacc[u] *= gam;
        const unsigned char *Xb = reinterpret_cast<const unsigned char *>(lx);
        const unsigned char *Bb = reinterpret_cast<const unsigned char *>(lb);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const bf16x4 lo = tr4(Xb + o.xtr + ks * 4096);
            const bf16x4 hi = tr4(Xb + o.xtr + ks * 4096 + 512);
            const bf16x8 xw = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
            for (int u = 0; u < NT; ++u) {
                const bf16x4 blo = tr4(Bb + o.bt[u] + ks * 32 * O::RB);
                const bf16x4 bhi = tr4(Bb + o.bt[u] + ks * 32 * O::RB + 4 * O::RB);
                Hacc[u] = mfma(bf16x8{blo[0], blo[1], blo[2], blo[3], bhi[0], bhi[1], bhi[2], bhi[3]}, xw, Hacc[u]);
            }
        }
        __syncthreads();
    };
    int s = 0;
    for (; s + 1 < nsb; s += 2) {
        step(s, 0);
        step(s + 1, 1);
    }
    if (s < nsb) step(s, 0);
    if (kRev && a.dinit) {
#pragma unroll
        for (int u = 0; u < NT; ++u) *reinterpret_cast<f32x4 *>(a.dinit + bh * (kP * N) + lane_off + 16 * u) = Hacc[u];
    }
}

// Both scans in one launch: workgroups below B*H take the forward states,
// the others the adjoints, so that the two run side by side.
template <int N>
__global__ __launch_bounds__(256) void state_scans(BwdArgs a) {
    const int64_t bhn = a.B * a.H;
    // logical index, contiguous within each XCD, so that the chains of one
    // batch row, which read the same Bm (or Cm) and dt rows, share an L2
    const int64_t blk = xcd_chain(blockIdx.x, gridDim.x);
    if (blk < bhn)
        state_scan_body<N, false>(a, blk);
    else
        state_scan_body<N, true>(a, blk - bhn);
}

// ---------------------------------------------------------------------------
// 3. Gradients of one sub-block for all heads of a group: one workgroup
// (eight waves) per (batch, group, sub-block), walking the group's heads with
// the next head's inputs loaded during the current one.  Bm, Cm and
// Gm = Cm Bm^T are shared by the heads and formed once; dBm and dCm are summed
// over the heads in the matrix-core accumulators and written once.  Tiles sit
// in LDS row-major with padded rows (S64 = 72, SN = N + 8 bfloat16).  A
// fragment whose 8 k values run along a stored row is one 16-byte read; one
// whose k values run down a column comes from two transposing reads
// (ds_read_b64_tr_b16).  Wave (w, hf), w = 0..3, hf = 0..1, computes rows
// 16w..16w+15 of every 64-row output and half of its column tiles, so that two
// waves share each SIMD and hide each other's latencies; the row sums the
// halves both contribute to meet in LDS.
template <int N>
struct GradSmem {
    static constexpr int S64 = 72, SN = N + 8;
    __bf16 C[64 * SN];       // Cm [i][n]
    __bf16 B[64 * SN];       // Bm [j][n]
    __bf16 X[64 * S64];      // x [j][p]
    __bf16 Y[64 * S64];      // dy [i][p]
    __bf16 H[64 * SN];       // H [p][n]
    __bf16 dH[64 * SN];      // dH' [p][n]
    __bf16 MT[64 * S64];     // M^T [j][i]
    __bf16 QT[64 * S64];     // Q^T [j][i]
    __bf16 DX[64 * S64];     // dx [j][p] of the head, on its way to global memory as whole rows
    // What the dLambda / ddt tail of a head needs, kept for a batch of
    // kBatch consecutive heads so that the eight waves run the batch's tails
    // side by side once it is complete, instead of one wave running each
    // head's tail while the others wait
    static constexpr int kBatch = 8;
    float lam[kBatch][64], dtl[kBatch][64], ww[kBatch][64], ee[64];
    float zcolw[kBatch][4][64], zrcolw[kBatch][4][64];    // column parts per row wave
    float zrow[kBatch][2][64], qv[kBatch][2][64], uv[kBatch][2][64];   // row parts per column half
    float red[kBatch][16];
    // ddt of up to kDdtHeads consecutive heads [token][head], written to
    // global memory together as runs of consecutive heads per token row
    static constexpr int kDdtHeads = 16;
    float ddt[64][kDdtHeads + 1];
};

// The four values a lane's accumulator covers, (r0 + 4 lgrp + r, c0 + lrow) for
// r = 0..3, of a row-major tile: one transposing read instead of four
__device__ __forceinline__ bf16x4 dvals(const __bf16 *base, int r0, int c0, int stride, int lrow, int lgrp) {
    const int a = lrow & 3, qq = lrow >> 2;
    return tr4(reinterpret_cast<const unsigned char *>(base + (r0 + 4 * lgrp + qq) * stride + c0 + 4 * a));
}

// Fragment for the 16x16x32 products, 8 k values from k0 + 8 lgrp:
// row-wise: element (r, k) at base[r * stride + k], r = r0 + lrow;
__device__ __forceinline__ bf16x8 frag_row(const __bf16 *base, int r0, int stride, int k0, int lrow, int lgrp) {
    return *reinterpret_cast<const bf16x8 *>(base + (r0 + lrow) * stride + k0 + 8 * lgrp);
}
// column-wise: element (r, k) at base[k * stride + r], r = r0 + lrow.  Lane
// a + 4qq of each 16-lane group names row k0 + 8 lgrp + qq (and + 4), columns
// r0 + 4a .. + 3; the transposing read gives lane lrow its column.
__device__ __forceinline__ bf16x8 frag_col(const __bf16 *base, int r0, int stride, int k0, int lrow, int lgrp) {
    const int a = lrow & 3, qq = lrow >> 2;
    const unsigned char *p = reinterpret_cast<const unsigned char *>(base + (k0 + 8 * lgrp + qq) * stride + r0 + 4 * a);
    const bf16x4 lo = tr4(p), hi = tr4(p + 4 * stride * 2);
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
__device__ __forceinline__ float red16(float v) { return row_sum16(v); }   // sum over the 16 lanes of a group

template <int N>
__global__ __launch_bounds__(512) void chunk_grad(BwdArgs a) {
    __shared__ __align__(16) GradSmem<N> sm;
    constexpr int S64 = GradSmem<N>::S64, SN = GradSmem<N>::SN;
    constexpr int NT = N / 16, NH = NT / 2, KN = N / 32, CPR = N / 8;
    constexpr int BPASS = 64 * CPR / 512;   // 16-byte chunks of a bf16 [64][N] tile per thread
    const int64_t nsb = a.nsb;
    const int64_t bg = blockIdx.x / nsb;
    const int c = (int)(blockIdx.x % nsb);
    const int64_t b = bg / a.G, g = bg % a.G, hpg = a.H / a.G;
    const int tid = threadIdx.x;
    const int w8 = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int w = w8 & 3, hf = w8 >> 2;   // row block, column half
    const int lane = tid & 63, lrow = lane & 15, lgrp = lane >> 4;
    const int64_t t0 = (int64_t)c * kSub;
    const int q = a.L - t0 < kSub ? (int)(a.L - t0) : kSub;
    const int64_t row0 = b * a.L + t0;

    // ---- Bm, Cm of the sub-block (shared by the heads), and Gm = Cm Bm^T
    {
        const int br = tid / CPR, bc = tid % CPR;
        const int bytes = (int)(((int64_t)(q - 1) * a.G * N + N) * 2);
        const rsrc_t rb = rsrc(a.Bm + (row0 * a.G + g) * N, bytes);
        const rsrc_t rc = rsrc(a.Cm + (row0 * a.G + g) * N, bytes);
#pragma unroll
        for (int k = 0; k < BPASS; ++k) {
            const int r = br + k * (512 / CPR);
            const int off = (int)(((int64_t)r * a.G * N + 8 * bc) * 2);
            *reinterpret_cast<uint4 *>(sm.B + r * SN + 8 * bc) = ld16(rb, off);
            *reinterpret_cast<uint4 *>(sm.C + r * SN + 8 * bc) = ld16(rc, off);
        }
    }
    // this head's inputs: one chunk of x and of dy, dt, and BPASS chunks of H
    // and dH' (bf16, accumulator order)
    const int xr = tid >> 3, xc = tid & 7;
    uint4 xv, yv, hv[BPASS], dv[BPASS];
    float dtv;
    auto load_head = [&](int64_t h) __attribute__((always_inline)) {
        const int bytes = (int)(((int64_t)(q - 1) * a.H * kP + kP) * 2);
        const rsrc_t rx = rsrc(a.x + (row0 * a.H + h) * kP, bytes);
        const rsrc_t ry = rsrc(a.dy + (row0 * a.H + h) * kP, bytes);
        const int off = (int)(((int64_t)xr * a.H * kP + 8 * xc) * 2);
        xv = ld16(rx, off);
        yv = ld16(ry, off);
        const int64_t slot = ((b * a.H + h) * nsb + c) * (kP * N);
        const __bf16 *hs = reinterpret_cast<const __bf16 *>(a.Hs) + slot;
        const __bf16 *ds = reinterpret_cast<const __bf16 *>(a.dHs) + slot;
#pragma unroll
        for (int k = 0; k < BPASS; ++k) {
            hv[k] = ld_nt16(hs + 8 * (k * 512 + tid));
            dv[k] = ld_nt16(ds + 8 * (k * 512 + tid));
        }
        const int64_t dh = h / a.hs;
        const rsrc_t rd = rsrc(a.dt + row0 * a.Hd + dh, (int)(((int64_t)(q - 1) * a.Hd + 1) * 4));
        dtv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rd, lane * (int)(a.Hd * 4), 0, 0));
    };
    load_head(g * hpg);
    __syncthreads();
    f32x4 gm[2];   // Gm tiles (rows 16w.., columns 16jt..) of this wave's column half
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int jt = 2 * hf + e;
        gm[e] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KN; ++kk)
            gm[e] = mfma(frag_row(sm.C, 16 * w, SN, 32 * kk, lrow, lgrp), frag_row(sm.B, 16 * jt, SN, 32 * kk, lrow, lgrp), gm[e]);
    }
    f32x4 dCacc[NH], dBacc[NH];   // column tiles NH hf .. NH hf + NH - 1
#pragma unroll
    for (int e = 0; e < NH; ++e) dCacc[e] = dBacc[e] = f32x4{0.f, 0.f, 0.f, 0.f};

    constexpr int KB = GradSmem<N>::kBatch;
    const int64_t dh0 = g * hpg / a.hs;   // the group's first caller head
    for (int64_t hh = 0; hh < hpg; ++hh) {
        const int64_t h = g * hpg + hh, dh = h / a.hs;
        const int sl = (int)(hh % KB);   // the head's place in its batch
        const float Ah = a.A[dh], Ah2 = Ah * kLog2eB, Dh = a.D[dh];
        // ---- stage this head; decays
        *reinterpret_cast<uint4 *>(sm.X + xr * S64 + 8 * xc) = xv;
        *reinterpret_cast<uint4 *>(sm.Y + xr * S64 + 8 * xc) = yv;
        float hdot = 0.f;
#pragma unroll
        for (int k = 0; k < BPASS; ++k) {
            // one 16-byte unit of the state in accumulator order: unit U =
            // (pq NT/2 + v) 64 + l holds p = 16 pq + l % 16, n = 32 v + 4 (l / 16)
            // .. + 3 and n + 16 .. + 19
            const int U = k * 512 + tid;
            const int l = U % 64, v = (U / 64) % (NT / 2), pq = U / (64 * (NT / 2));
            const int p = 16 * pq + (l & 15), n = 32 * v + 4 * (l >> 4);
            *reinterpret_cast<uint2 *>(sm.H + p * SN + n) = uint2{hv[k].x, hv[k].y};
            *reinterpret_cast<uint2 *>(sm.H + p * SN + n + 16) = uint2{hv[k].z, hv[k].w};
            *reinterpret_cast<uint2 *>(sm.dH + p * SN + n) = uint2{dv[k].x, dv[k].y};
            *reinterpret_cast<uint2 *>(sm.dH + p * SN + n + 16) = uint2{dv[k].z, dv[k].w};
            // <H, dH'> over the unit: four bfloat16 pair dot products into fp32
            const uint32_t hw[4] = {hv[k].x, hv[k].y, hv[k].z, hv[k].w};
            const uint32_t dw[4] = {dv[k].x, dv[k].y, dv[k].z, dv[k].w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
                hdot = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_dot, hw[e]),
                                                       __builtin_bit_cast(bf16x2_dot, dw[e]), hdot, false);
        }
        const float lam = wave_scan(dtv * Ah2);
        const float lend = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lam), 63));
        if (w8 == 0) {
            sm.lam[sl][lane] = lam;
            sm.dtl[sl][lane] = dtv;
            sm.ww[sl][lane] = ex2f(lend - lam) * dtv;
            sm.ee[lane] = ex2f(lam);
        }
        hdot = wave_sum(hdot);
        if (lane == 0) sm.red[sl][w8] = hdot;
        // the next head's inputs (the last head loads itself again)
        load_head(hh + 1 < hpg ? h + 1 : h);
        __syncthreads();

        // ---- S = dy x^T for rows i of this wave, column tiles of its half;
        // M^T, Q^T; sums for d/dLambda and ddt
        float lam_i[4], zr[4] = {0.f, 0.f, 0.f, 0.f}, dd = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) lam_i[r] = sm.lam[sl][16 * w + 4 * lgrp + r];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int jt = 2 * hf + e;
            f32x4 sd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                sd = mfma(frag_row(sm.Y, 16 * w, S64, 32 * kk, lrow, lgrp), frag_row(sm.X, 16 * jt, S64, 32 * kk, lrow, lgrp), sd);
            const int j = 16 * jt + lrow;
            const float lam_j = sm.lam[sl][j], dtj = sm.dtl[sl][j];
            float mv[4], qv[4], zc = 0.f, zrc = 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * w + 4 * lgrp + r;
                const float E = j <= i ? ex2f(lam_i[r] - lam_j) : 0.f;
                mv[r] = gm[e][r] * E * dtj + (i == j ? Dh : 0.f);
                qv[r] = sd[r] * E * dtj;
                const float zrv = sd[r] * gm[e][r] * E;
                zr[r] += zrv * dtj;
                zc += zrv * dtj;
                zrc += zrv;
                if (i == j) dd += sd[r];
            }
            *reinterpret_cast<uint2 *>(sm.MT + j * S64 + 16 * w + 4 * lgrp) = uint2{pack2(mv[0], mv[1]), pack2(mv[2], mv[3])};
            *reinterpret_cast<uint2 *>(sm.QT + j * S64 + 16 * w + 4 * lgrp) = uint2{pack2(qv[0], qv[1]), pack2(qv[2], qv[3])};
            zc = rows_sum4(zc);
            zrc = rows_sum4(zrc);
            if (lgrp == 0) {
                sm.zcolw[sl][w][j] = zc;
                sm.zrcolw[sl][w][j] = zrc;
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float v = red16(zr[r]);
            if (lrow == 0) sm.zrow[sl][hf][16 * w + 4 * lgrp + r] = v;
        }
        dd = wave_sum(dd);
        if (lane == 0) sm.red[sl][8 + w8] = dd;
        __syncthreads();

        // ---- dx = M^T dy + w (Bm dH'^T), rows j, column tiles pt of this
        // half; q_j = x_j . (dH' Bm_j)
        {
            float qs[4] = {0.f, 0.f, 0.f, 0.f}, wj[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) wj[r] = sm.ww[sl][16 * w + 4 * lgrp + r];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int pt = 2 * hf + e;
                f32x4 dxa = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
                    dxa = mfma(frag_row(sm.MT, 16 * w, S64, 32 * kk, lrow, lgrp), frag_col(sm.Y, 16 * pt, S64, 32 * kk, lrow, lgrp), dxa);
#pragma unroll
                for (int kk = 0; kk < KN; ++kk)
                    vv = mfma(frag_row(sm.B, 16 * w, SN, 32 * kk, lrow, lgrp), frag_row(sm.dH, 16 * pt, SN, 32 * kk, lrow, lgrp), vv);
                const int p = 16 * pt + lrow;
                const bf16x4 xj = dvals(sm.X, 16 * w, 16 * pt, S64, lrow, lgrp);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = 16 * w + 4 * lgrp + r;
                    qs[r] += (float)xj[r] * vv[r];
                    sm.DX[j * S64 + p] = (__bf16)(dxa[r] + wj[r] * vv[r]);
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float v = red16(qs[r]);
                if (lrow == 0) sm.qv[sl][hf][16 * w + 4 * lgrp + r] = v;
            }
        }
        // (the phases are kept apart: interleaved, their operands would not fit
        // the registers of two waves per SIMD)
        __builtin_amdgcn_sched_barrier(0);
        // ---- dCm rows i += exp(Lambda_i) dy H + Q Bm; u_i = Cm_i . (exp(Lambda_i) H^T dy_i)
        {
            float us[4] = {0.f, 0.f, 0.f, 0.f}, ei[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) ei[r] = sm.ee[16 * w + 4 * lgrp + r];
#pragma unroll
            for (int e = 0; e < NH; ++e) {
                const int nt = NH * hf + e;
                f32x4 c1 = {0.f, 0.f, 0.f, 0.f}, c2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    c1 = mfma(frag_row(sm.Y, 16 * w, S64, 32 * kk, lrow, lgrp), frag_col(sm.H, 16 * nt, SN, 32 * kk, lrow, lgrp), c1);
                    c2 = mfma(frag_col(sm.QT, 16 * w, S64, 32 * kk, lrow, lgrp), frag_col(sm.B, 16 * nt, SN, 32 * kk, lrow, lgrp), c2);
                }
                const bf16x4 cin = dvals(sm.C, 16 * w, 16 * nt, SN, lrow, lgrp);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float ci = ei[r] * c1[r];
                    us[r] += (float)cin[r] * ci;
                    dCacc[e][r] += ci + c2[r];
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float v = red16(us[r]);
                if (lrow == 0) sm.uv[sl][hf][16 * w + 4 * lgrp + r] = v;
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        // ---- dBm rows j += w_j x dH' + Q^T Cm
        {
            float wj[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) wj[r] = sm.ww[sl][16 * w + 4 * lgrp + r];
#pragma unroll
            for (int e = 0; e < NH; ++e) {
                const int nt = NH * hf + e;
                f32x4 b1 = {0.f, 0.f, 0.f, 0.f}, b2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    b1 = mfma(frag_row(sm.X, 16 * w, S64, 32 * kk, lrow, lgrp), frag_col(sm.dH, 16 * nt, SN, 32 * kk, lrow, lgrp), b1);
                    b2 = mfma(frag_row(sm.QT, 16 * w, S64, 32 * kk, lrow, lgrp), frag_col(sm.C, 16 * nt, SN, 32 * kk, lrow, lgrp), b2);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) dBacc[e][r] += wj[r] * b1[r] + b2[r];
            }
        }
        __syncthreads();

        // ---- dx of the head: 64 rows of 128 bytes, 16 bytes per thread
        if (xr < q)
            *reinterpret_cast<uint4 *>(a.dx + ((row0 + xr) * a.H + h) * kP + 8 * xc) =
                *reinterpret_cast<const uint4 *>(sm.DX + xr * S64 + 8 * xc);
        // ---- once a batch is complete: d/dLambda per token, ddt, and the
        // parts of dA, dD of its heads, one caller head per wave (the two
        // halves of a head of 128 channels are consecutive, in one batch, and
        // their ddt, dA and dD parts are summed: the gradient of an input
        // shared by both halves)
        if (sl == KB - 1 || hh + 1 == hpg) {
            const int64_t hb = hh - sl;   // the batch's first head (in the group)
            const int nb = sl + 1;
            if (w8 * (int)a.hs < nb) {
                const int k = lane;
                float gsum = 0.f, dasum = 0.f, ddsum = 0.f;
                for (int u = 0; u < (int)a.hs; ++u) {
                    const int s = w8 * (int)a.hs + u;
                    const float Au = a.A[(g * hpg + hb + s) / a.hs];
                    const float lendu = sm.lam[s][63];
                    float zc = 0.f, zrc = 0.f;
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        zc += sm.zcolw[s][m][k];
                        zrc += sm.zrcolw[s][m][k];
                    }
                    const float wk = sm.ww[s][k], qk = sm.qv[s][0][k] + sm.qv[s][1][k];
                    float dl = (sm.uv[s][0][k] + sm.uv[s][1][k]) + (sm.zrow[s][0][k] + sm.zrow[s][1][k]) - zc - wk * qk;
                    const float wq = wave_sum(wk * qk);
                    float hd = 0.f, ddp = 0.f;
#pragma unroll
                    for (int m = 0; m < 8; ++m) {
                        hd += sm.red[s][m];
                        ddp += sm.red[s][8 + m];
                    }
                    if (k == 63) dl += ex2f(lendu) * hd + wq;
                    // rs_k = sum over i >= k of dl_i = total - (prefix through k) + dl_k
                    const float pre = wave_scan(dl);
                    const float rs = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pre), 63)) - pre + dl;
                    gsum += Au * rs + zrc + ex2f(lendu - sm.lam[s][k]) * qk;
                    dasum += wave_sum(sm.dtl[s][k] * rs);
                    ddsum += ddp;
                }
                const int64_t dhu = (g * hpg + hb) / a.hs + w8;   // this wave's caller head
                sm.ddt[k][(dhu - dh0) % GradSmem<N>::kDdtHeads] = gsum;
                if (k == 0) {
                    a.dAp[(b * a.Hd + dhu) * nsb + c] = dasum;
                    a.dDp[(b * a.Hd + dhu) * nsb + c] = ddsum;
                }
            }
            __syncthreads();
            // ---- ddt of the last kDdtHeads caller heads (or of the group's last ones)
            constexpr int KD = GradSmem<N>::kDdtHeads;
            static_assert(KD % KB == 0, "a ddt flush ends with a batch");
            const int64_t done = dh - dh0 + 1;   // caller heads of the group finished
            const bool last = hh + 1 == hpg;
            if (done % KD == 0 || last) {
                const int nh = (int)(done % KD == 0 ? KD : done % KD);
                const int64_t base = dh0 + done - nh;
                for (int e = tid; e < 64 * KD; e += 512) {
                    const int k = e / KD, m = e % KD;
                    if (k < q && m < nh) a.ddt[(row0 + k) * a.Hd + base + m] = sm.ddt[k][m];
                }
            }
        }
    }
    // ---- dCm, dBm of the group (all its heads), this wave's column tiles
#pragma unroll
    for (int e = 0; e < NH; ++e) {
        const int n = 16 * (NH * hf + e) + lrow;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * w + 4 * lgrp + r;
            if (i < q) {
                a.dCm[((row0 + i) * a.G + g) * N + n] = (__bf16)dCacc[e][r];
                a.dBm[((row0 + i) * a.G + g) * N + n] = (__bf16)dBacc[e][r];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// 4. dA, dD: sums of the per-(head, sub-block) parts over batch rows and sub-blocks.
__global__ __launch_bounds__(256) void reduce_head(BwdArgs a) {
    // block h: dA[h], dD[h] = sums over batch rows and sub-blocks
    __shared__ float part[2][256];
    const int64_t h = blockIdx.x;
    float sa = 0.f, sd = 0.f;
    for (int64_t k = threadIdx.x; k < a.B * a.nsb; k += blockDim.x) {
        const int64_t b = k / a.nsb, c = k % a.nsb;
        sa += a.dAp[(b * a.Hd + h) * a.nsb + c];
        sd += a.dDp[(b * a.Hd + h) * a.nsb + c];
    }
    part[0][threadIdx.x] = sa;
    part[1][threadIdx.x] = sd;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) {
            part[0][threadIdx.x] += part[0][threadIdx.x + s];
            part[1][threadIdx.x] += part[1][threadIdx.x + s];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        a.dA[h] = part[0][0];
        a.dD[h] = part[1][0];
    }
}

template <int N>
hipError_t launch(const BwdArgs &a, hipStream_t stream) {
    const int64_t bhn = a.B * a.H;
    state_scans<N><<<dim3((unsigned)(2 * bhn)), 256, 0, stream>>>(a);
    chunk_grad<N><<<dim3((unsigned)(a.B * a.G * a.nsb)), 512, 0, stream>>>(a);
    reduce_head<<<dim3((unsigned)a.Hd), 256, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace

bool bwd_supported(int64_t P, int64_t N, int64_t H, int64_t G) {
    if (!(P == 64 || P == 128) || !(N == 64 || N == 128)) return false;
    const int64_t lim = (int64_t)1 << 31;
    return (int64_t)kSub * H * P * 2 < lim && (int64_t)kSub * G * N * 2 < lim && (int64_t)kSub * H * 4 < lim;
}

// Workspace of the backward, in floats: the states and adjoints (bfloat16,
// two per float) of every head of 64 channels, and the per-(head, sub-block)
// parts of dA and dD.
size_t bwd_workspace_floats(int64_t B, int64_t L, int64_t H, int64_t P, int64_t N) {
    const int64_t nsb = (L + kSub - 1) / kSub, Hk = H * (P / kP);
    return (size_t)(B * Hk * nsb * kSub * N + 2 * B * H * nsb);
}

hipError_t launch_scan_bwd(const void *x, const float *dt, const float *A, const void *Bm, const void *Cm,
                           const float *D, const float *init, const void *dy, const float *dfinal, void *dx,
                           float *ddt, float *dA, void *dBm, void *dCm, float *dD, float *dinit, float *ws,
                           int64_t B, int64_t L, int64_t H, int64_t P, int64_t G, int64_t N, hipStream_t stream) {
    const int64_t nsb = (L + kSub - 1) / kSub;
    const int hs = (int)(P / kP);
    const int64_t Hk = H * hs;
    const int64_t big = B * Hk * nsb * kSub * N / 2;   // one bf16 state array, in floats
    BwdArgs a{(const __bf16 *)x, (const __bf16 *)dy, (const __bf16 *)Bm, (const __bf16 *)Cm,
              dt, A, D, init, dfinal,
              (__bf16 *)dx, (__bf16 *)dBm, (__bf16 *)dCm,
              ddt, dA, dD, dinit,
              ws, ws + big, ws + 2 * big, ws + 2 * big + B * H * nsb,
              B, L, Hk, G, nsb, H, hs};
    switch (N) {
        case 64: return launch<64>(a, stream);
        case 128: return launch<128>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace ssd
