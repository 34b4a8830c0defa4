// Backward of the chunk scan on gfx950: the gradients of
//   <dy, y> + <dfinal, final state>
// with respect to x, dt, A, Bm, Cm, D and the initial state, for P = 64,
// N in {64, 128}, bfloat16 x / Bm / Cm / y.
//
// The recurrence is the one of the "Mamba-2" note (section "writing the SSM
// as a matrix", one decay per head as in "reducing A to a number"), cut into
// 64-token sub-blocks as in the block decomposition of the "Mamba-2 model
// walkthrough" (section 6.1).  Only the states are sequential, so the work is
// split into
//   1. state_scan<N, false>: the state H_c entering every sub-block c;
//   2. state_scan<N, true>:  backwards in time, the adjoint dH'_c of the state
//      leaving every sub-block, dH_c = g_c dH'_c + sum_i exp(Lambda_i) dy_i (x) Cm_i,
//      whose last value is the initial state's gradient;
//   3. chunk_grad<N>: one workgroup per (batch, head, sub-block), all in
//      parallel: from H_c, dH'_c and the sub-block's inputs, dx and ddt of its
//      tokens and per-head partials of dBm, dCm, dA, dD;
//   4. sums of the partials over the heads of a group (dBm, dCm) and over the
//      sub-blocks (dA, dD).
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
    float *Hs;    // [B*H, nsb, P, N]  state entering each sub-block
    float *dHs;   // [B*H, nsb, P, N]  adjoint of the state leaving each sub-block
    float *dBp;   // [B*H, nsb*64, N]  this head's part of dBm
    float *dCp;   // [B*H, nsb*64, N]  this head's part of dCm
    float *dAp;   // [B*H, nsb]
    float *dDp;   // [B*H, nsb]
    int64_t B, L, H, G, nsb;
};

__device__ __forceinline__ float ex2f(float v) { return __builtin_amdgcn_exp2f(v); }

__device__ __forceinline__ float shfl_xor(float v, int m) {
    const int lane = __lane_id();
    return __int_as_float(__builtin_amdgcn_ds_bpermute(4 * (lane ^ m), __float_as_int(v)));
}
__device__ __forceinline__ float lane_get(float v, int src) {
    return __int_as_float(__builtin_amdgcn_ds_bpermute(4 * src, __float_as_int(v)));
}
__device__ __forceinline__ float wave_sum(float v) {
    for (int m = 1; m < 64; m <<= 1) v += shfl_xor(v, m);
    return v;
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
__global__ __launch_bounds__(256) void state_scan(BwdArgs a) {
    __shared__ __align__(16) __bf16 lx[kSub * kP];
    __shared__ __align__(16) __bf16 lb[kSub * N];
    using O = LaneOffs<N>;
    constexpr int NT = N / 16, KB = N / 32;
    const int64_t bh = blockIdx.x;
    const int64_t b = bh / a.H, h = bh % a.H, g = h / (a.H / a.G);
    const float Ah2 = a.A[h] * kLog2eB;
    const int tid = threadIdx.x;
    const int pq = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, lrow = lane & 15, lgrp = lane >> 4;
    const LaneOffs<N> o = lane_offsets<N>(tid, pq, a.H, a.G);
    const __bf16 *U = kRev ? a.dy : a.x;
    const __bf16 *Mt = kRev ? a.Cm : a.Bm;
    const int nsb = (int)a.nsb;

    uint4 ur[2], mr[KB];
    float dtv = 0.f;
    auto load = [&](int c) __attribute__((always_inline)) {
        const int64_t t0 = (int64_t)c * kSub;
        const int q = a.L - t0 < kSub ? (int)(a.L - t0) : kSub;
        const int64_t row0 = b * a.L + t0;
        const rsrc_t ru = rsrc(U + (row0 * a.H + h) * kP, (int)(((int64_t)(q - 1) * a.H * kP + kP) * 2));
#pragma unroll
        for (int k = 0; k < 2; ++k) ur[k] = ld16(ru, o.gx + k * (int)(32 * a.H * kP * 2));
        const rsrc_t rm = rsrc(Mt + (row0 * a.G + g) * N, (int)(((int64_t)(q - 1) * a.G * N + N) * 2));
        const int step = (int)((256 / O::CPR) * a.G * N * 2);
#pragma unroll
        for (int k = 0; k < KB; ++k) mr[k] = ld16(rm, o.gb + k * step);
        const rsrc_t rd = rsrc(a.dt + row0 * a.H + h, (int)(((int64_t)(q - 1) * a.H + 1) * 4));
        dtv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rd, o.gd, 0, 0));
    };

    const int lane_off = (16 * pq + lrow) * N + 4 * lgrp;
    f32x4 Hacc[NT];
    {
        const float *src = kRev ? a.dfinal : a.init;
#pragma unroll
        for (int u = 0; u < NT; ++u)
            Hacc[u] = src ? *reinterpret_cast<const f32x4 *>(src + bh * (kP * N) + lane_off + 16 * u)
                          : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    load(kRev ? nsb - 1 : 0);
    float *sbase = (kRev ? a.dHs : a.Hs) + bh * a.nsb * (kP * N) + lane_off;
    const int row_k0 = tid >> 3;   // staged rows row_k0 and row_k0 + 32 of u
    for (int s = 0; s < nsb; ++s) {
        const int c = kRev ? nsb - 1 - s : s;
        const float v = wave_scan(dtv * Ah2);
        const float lend = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
        const float om = kRev ? ex2f(v) : ex2f(lend - v) * dtv;
        const float gam = ex2f(lend);
#pragma unroll
        for (int u = 0; u < NT; ++u) *reinterpret_cast<f32x4 *>(sbase + (int64_t)c * (kP * N) + 16 * u) = Hacc[u];
        // u weighted by om, and Mt, into LDS
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const float wgt = lane_get(om, row_k0 + 32 * k);
            const bf16x8 xv = __builtin_bit_cast(bf16x8, ur[k]);
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
            lds_st<uint4>(reinterpret_cast<unsigned char *>(lb) + o.sb + k * (256 / O::CPR) * O::RB, mr[k]);
        // the next sub-block into registers (past the ends it loads this one again)
        {
            int cn = kRev ? c - 1 : c + 1;
            cn = cn < 0 ? 0 : (cn >= nsb ? nsb - 1 : cn);
            load(cn);
        }
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
    }
    if (kRev && a.dinit) {
#pragma unroll
        for (int u = 0; u < NT; ++u) *reinterpret_cast<f32x4 *>(a.dinit + bh * (kP * N) + lane_off + 16 * u) = Hacc[u];
    }
}

// ---------------------------------------------------------------------------
// 3. Gradients of one sub-block, one workgroup (four waves) per (batch, head,
// sub-block).  Tiles sit in LDS row-major with padded rows (S64 = 72, SN =
// N + 8 bfloat16), so that matrix-core fragments (8 consecutive k values per
// lane) are single 16-byte reads; every product is arranged so that both
// operands are stored k-contiguous, which takes transposed copies of dy, Bm,
// Cm, dH' and H.  Wave w computes rows 16w..16w+15 of every 64-row output.
template <int N>
struct GradSmem {
    static constexpr int S64 = 72, SN = N + 8;
    static constexpr int BIG = (64 * SN > N * S64 ? 64 * SN : N * S64);
    __bf16 s1[BIG];          // Cm [i][n], then Cm^T [n][i]
    __bf16 s2[BIG];          // Bm [j][n], then Bm^T [n][j]
    __bf16 X[64 * S64];      // x [j][p]
    __bf16 Y[64 * S64];      // dy [i][p]
    __bf16 YT[64 * S64];     // dy^T [p][i]
    __bf16 s6[BIG];          // dH' [p][n], then dH'^T [n][p]
    __bf16 HT[N * S64];      // H^T [n][p]
    __bf16 MT[64 * S64];     // M^T [j][i]
    __bf16 Q[64 * S64];      // Q [i][j]
    __bf16 QT[64 * S64];     // Q^T [j][i]
    float lam[64], dtl[64], ww[64], ee[64];
    float zrow[64], zcolw[4][64], zrcolw[4][64], qv[64], uv[64];
    float red[8];
};

__device__ __forceinline__ bf16x8 frag(const __bf16 *base, int row, int stride, int k0, int lgrp) {
    return *reinterpret_cast<const bf16x8 *>(base + row * stride + k0 + 8 * lgrp);
}

template <int N>
__global__ __launch_bounds__(256) void chunk_grad(BwdArgs a) {
    __shared__ __align__(16) GradSmem<N> sm;
    constexpr int S64 = GradSmem<N>::S64, SN = GradSmem<N>::SN;
    constexpr int NT = N / 16, KN = N / 32, CPR = N / 8, KB = N / 32;
    const int64_t nsb = a.nsb;
    const int64_t bh = blockIdx.x / nsb;
    const int c = (int)(blockIdx.x % nsb);
    const int64_t b = bh / a.H, h = bh % a.H, g = h / (a.H / a.G);
    const float Ah = a.A[h], Ah2 = Ah * kLog2eB, Dh = a.D[h];
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, lrow = lane & 15, lgrp = lane >> 4;
    const int64_t t0 = (int64_t)c * kSub;
    const int q = a.L - t0 < kSub ? (int)(a.L - t0) : kSub;
    const int64_t row0 = b * a.L + t0;

    // ---- loads: x, dy (two 16-byte chunks per thread), Bm, Cm (KB each), H and dH' (fp32)
    const int xr = tid >> 3, xc = tid & 7;
    uint4 xv[2], yv[2];
    {
        const int bytes = (int)(((int64_t)(q - 1) * a.H * kP + kP) * 2);
        const rsrc_t rx = rsrc(a.x + (row0 * a.H + h) * kP, bytes);
        const rsrc_t ry = rsrc(a.dy + (row0 * a.H + h) * kP, bytes);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int off = (int)(((int64_t)(xr + 32 * k) * a.H * kP + 8 * xc) * 2);
            xv[k] = ld16(rx, off);
            yv[k] = ld16(ry, off);
        }
    }
    const int br = tid / CPR, bc = tid % CPR;
    uint4 bv[KB], cv[KB];
    {
        const int bytes = (int)(((int64_t)(q - 1) * a.G * N + N) * 2);
        const rsrc_t rb = rsrc(a.Bm + (row0 * a.G + g) * N, bytes);
        const rsrc_t rc = rsrc(a.Cm + (row0 * a.G + g) * N, bytes);
#pragma unroll
        for (int k = 0; k < KB; ++k) {
            const int off = (int)(((int64_t)(br + k * (256 / CPR)) * a.G * N + 8 * bc) * 2);
            bv[k] = ld16(rb, off);
            cv[k] = ld16(rc, off);
        }
    }
    // H and dH': chunk k*256 + tid of the [64][N] fp32 state, 4 floats at (p, 4 n4)
    constexpr int HCH = 64 * N / 4 / 256;   // chunks per thread
    const float *Hsrc = a.Hs + (bh * nsb + c) * (kP * N);
    const float *dHsrc = a.dHs + (bh * nsb + c) * (kP * N);
    f32x4 hv[HCH], dhv[HCH];
#pragma unroll
    for (int k = 0; k < HCH; ++k) {
        const int idx = k * 256 + tid;
        hv[k] = *reinterpret_cast<const f32x4 *>(Hsrc + 4 * idx);
        dhv[k] = *reinterpret_cast<const f32x4 *>(dHsrc + 4 * idx);
    }
    const rsrc_t rd = rsrc(a.dt + row0 * a.H + h, (int)(((int64_t)(q - 1) * a.H + 1) * 4));
    const float dtv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rd, lane * (int)(a.H * 4), 0, 0));

    // ---- decays (each wave its own copy, lane = token); wave 0 publishes them
    const float lam = wave_scan(dtv * Ah2);
    const float lend = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lam), 63));
    if (w == 0) {
        sm.lam[lane] = lam;
        sm.dtl[lane] = dtv;
        sm.ww[lane] = ex2f(lend - lam) * dtv;
        sm.ee[lane] = ex2f(lam);
    }
    // ---- tiles into LDS
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int r = xr + 32 * k;
        *reinterpret_cast<uint4 *>(sm.X + r * S64 + 8 * xc) = xv[k];
        *reinterpret_cast<uint4 *>(sm.Y + r * S64 + 8 * xc) = yv[k];
        const bf16x8 yy = __builtin_bit_cast(bf16x8, yv[k]);
#pragma unroll
        for (int e = 0; e < 8; ++e) sm.YT[(8 * xc + e) * S64 + r] = yy[e];
    }
#pragma unroll
    for (int k = 0; k < KB; ++k) {
        const int r = br + k * (256 / CPR);
        *reinterpret_cast<uint4 *>(sm.s1 + r * SN + 8 * bc) = cv[k];
        *reinterpret_cast<uint4 *>(sm.s2 + r * SN + 8 * bc) = bv[k];
    }
    float hdot = 0.f;
#pragma unroll
    for (int k = 0; k < HCH; ++k) {
        const int idx = k * 256 + tid;
        const int p = idx / (N / 4), n = 4 * (idx % (N / 4));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            sm.HT[(n + e) * S64 + p] = (__bf16)hv[k][e];
            sm.s6[p * SN + n + e] = (__bf16)dhv[k][e];
            hdot += hv[k][e] * dhv[k][e];
        }
    }
    hdot = wave_sum(hdot);
    if (lane == 0) sm.red[w] = hdot;
    __syncthreads();

    // ---- P1: Gm = Cm Bm^T and S = dy x^T for rows i of this wave; the masked
    // matrices M^T, Q, Q^T; row and column sums for d/dLambda and ddt
    float lam_i[4], zr[4] = {0.f, 0.f, 0.f, 0.f}, dd = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) lam_i[r] = sm.lam[16 * w + 4 * lgrp + r];
    for (int jt = 0; jt < 4; ++jt) {
        f32x4 gm = {0.f, 0.f, 0.f, 0.f}, sd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KN; ++kk)
            gm = mfma(frag(sm.s1, 16 * w + lrow, SN, 32 * kk, lgrp), frag(sm.s2, 16 * jt + lrow, SN, 32 * kk, lgrp), gm);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
            sd = mfma(frag(sm.Y, 16 * w + lrow, S64, 32 * kk, lgrp), frag(sm.X, 16 * jt + lrow, S64, 32 * kk, lgrp), sd);
        const int j = 16 * jt + lrow;
        const float lam_j = sm.lam[j], dtj = sm.dtl[j];
        float mv[4], qv[4], zc = 0.f, zrc = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * w + 4 * lgrp + r;
            const float E = j <= i ? ex2f(lam_i[r] - lam_j) : 0.f;
            mv[r] = gm[r] * E * dtj + (i == j ? Dh : 0.f);
            qv[r] = sd[r] * E * dtj;
            const float zrv = sd[r] * gm[r] * E;
            zr[r] += zrv * dtj;
            zc += zrv * dtj;
            zrc += zrv;
            if (i == j) dd += sd[r];
            sm.Q[i * S64 + j] = (__bf16)qv[r];
        }
        *reinterpret_cast<uint2 *>(sm.MT + j * S64 + 16 * w + 4 * lgrp) =
            uint2{pack2(mv[0], mv[1]), pack2(mv[2], mv[3])};
        *reinterpret_cast<uint2 *>(sm.QT + j * S64 + 16 * w + 4 * lgrp) =
            uint2{pack2(qv[0], qv[1]), pack2(qv[2], qv[3])};
        zc += shfl_xor(zc, 16);
        zc += shfl_xor(zc, 32);
        zrc += shfl_xor(zrc, 16);
        zrc += shfl_xor(zrc, 32);
        if (lgrp == 0) {
            sm.zcolw[w][j] = zc;
            sm.zrcolw[w][j] = zrc;
        }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float v = zr[r];
        v += shfl_xor(v, 1);
        v += shfl_xor(v, 2);
        v += shfl_xor(v, 4);
        v += shfl_xor(v, 8);
        if (lrow == 0) sm.zrow[16 * w + 4 * lgrp + r] = v;
    }
    dd = wave_sum(dd);
    if (lane == 0) sm.red[4 + w] = dd;
    __syncthreads();
    // Cm^T over Cm (Cm [i][n] is not read again)
#pragma unroll
    for (int k = 0; k < KB; ++k) {
        const int r = br + k * (256 / CPR);
        const bf16x8 cc = __builtin_bit_cast(bf16x8, cv[k]);
#pragma unroll
        for (int e = 0; e < 8; ++e) sm.s1[(8 * bc + e) * S64 + r] = cc[e];
    }

    // ---- P2: dx = M^T dy + w (Bm dH'^T) for rows j of this wave; q_j = x_j . (dH' Bm_j)
    {
        float qs[4] = {0.f, 0.f, 0.f, 0.f};
        float wj[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) wj[r] = sm.ww[16 * w + 4 * lgrp + r];
        for (int pt = 0; pt < 4; ++pt) {
            f32x4 dxa = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                dxa = mfma(frag(sm.MT, 16 * w + lrow, S64, 32 * kk, lgrp), frag(sm.YT, 16 * pt + lrow, S64, 32 * kk, lgrp), dxa);
#pragma unroll
            for (int kk = 0; kk < KN; ++kk)
                vv = mfma(frag(sm.s2, 16 * w + lrow, SN, 32 * kk, lgrp), frag(sm.s6, 16 * pt + lrow, SN, 32 * kk, lgrp), vv);
            const int p = 16 * pt + lrow;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = 16 * w + 4 * lgrp + r;
                qs[r] += (float)sm.X[j * S64 + p] * vv[r];
                if (j < q) a.dx[((row0 + j) * a.H + h) * kP + p] = (__bf16)(dxa[r] + wj[r] * vv[r]);
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float v = qs[r];
            v += shfl_xor(v, 1);
            v += shfl_xor(v, 2);
            v += shfl_xor(v, 4);
            v += shfl_xor(v, 8);
            if (lrow == 0) sm.qv[16 * w + 4 * lgrp + r] = v;
        }
    }
    __syncthreads();
    // Bm^T over Bm, dH'^T over dH'
#pragma unroll
    for (int k = 0; k < KB; ++k) {
        const int r = br + k * (256 / CPR);
        const bf16x8 bb = __builtin_bit_cast(bf16x8, bv[k]);
#pragma unroll
        for (int e = 0; e < 8; ++e) sm.s2[(8 * bc + e) * S64 + r] = bb[e];
    }
#pragma unroll
    for (int k = 0; k < HCH; ++k) {
        const int idx = k * 256 + tid;
        const int p = idx / (N / 4), n = 4 * (idx % (N / 4));
#pragma unroll
        for (int e = 0; e < 4; ++e) sm.s6[(n + e) * S64 + p] = (__bf16)dhv[k][e];
    }
    __syncthreads();

    // ---- P3: dCm rows i: exp(Lambda_i) dy H + Q Bm; u_i = Cm_i . (exp(Lambda_i) H^T dy_i)
    float* dCrow = a.dCp + (bh * nsb * kSub + (int64_t)c * kSub) * N;
    float* dBrow = a.dBp + (bh * nsb * kSub + (int64_t)c * kSub) * N;
    {
        float us[4] = {0.f, 0.f, 0.f, 0.f};
        float ei[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) ei[r] = sm.ee[16 * w + 4 * lgrp + r];
        for (int nt = 0; nt < NT; ++nt) {
            f32x4 c1 = {0.f, 0.f, 0.f, 0.f}, c2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                c1 = mfma(frag(sm.Y, 16 * w + lrow, S64, 32 * kk, lgrp), frag(sm.HT, 16 * nt + lrow, S64, 32 * kk, lgrp), c1);
                c2 = mfma(frag(sm.Q, 16 * w + lrow, S64, 32 * kk, lgrp), frag(sm.s2, 16 * nt + lrow, S64, 32 * kk, lgrp), c2);
            }
            const int n = 16 * nt + lrow;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * w + 4 * lgrp + r;
                const float ci = ei[r] * c1[r];
                us[r] += (float)sm.s1[n * S64 + i] * ci;
                dCrow[(int64_t)i * N + n] = ci + c2[r];
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float v = us[r];
            v += shfl_xor(v, 1);
            v += shfl_xor(v, 2);
            v += shfl_xor(v, 4);
            v += shfl_xor(v, 8);
            if (lrow == 0) sm.uv[16 * w + 4 * lgrp + r] = v;
        }
    }
    // ---- P4: dBm rows j: w_j x dH' + Q^T Cm
    {
        float wj[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) wj[r] = sm.ww[16 * w + 4 * lgrp + r];
        for (int nt = 0; nt < NT; ++nt) {
            f32x4 b1 = {0.f, 0.f, 0.f, 0.f}, b2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                b1 = mfma(frag(sm.X, 16 * w + lrow, S64, 32 * kk, lgrp), frag(sm.s6, 16 * nt + lrow, S64, 32 * kk, lgrp), b1);
                b2 = mfma(frag(sm.QT, 16 * w + lrow, S64, 32 * kk, lgrp), frag(sm.s1, 16 * nt + lrow, S64, 32 * kk, lgrp), b2);
            }
            const int n = 16 * nt + lrow;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = 16 * w + 4 * lgrp + r;
                dBrow[(int64_t)j * N + n] = wj[r] * b1[r] + b2[r];
            }
        }
    }
    __syncthreads();

    // ---- P5: d/dLambda per token, ddt, and this sub-block's parts of dA, dD (wave 0)
    if (w == 0) {
        const int k = lane;
        const float zc = sm.zcolw[0][k] + sm.zcolw[1][k] + sm.zcolw[2][k] + sm.zcolw[3][k];
        const float zrc = sm.zrcolw[0][k] + sm.zrcolw[1][k] + sm.zrcolw[2][k] + sm.zrcolw[3][k];
        const float wk = sm.ww[k], qk = sm.qv[k];
        float dl = sm.uv[k] + sm.zrow[k] - zc - wk * qk;
        const float wq = wave_sum(wk * qk);
        const float hd = sm.red[0] + sm.red[1] + sm.red[2] + sm.red[3];
        if (k == 63) dl += ex2f(lend) * hd + wq;
        // rs_k = sum over i >= k of dl_i
        const float rev = lane_get(dl, 63 - k);
        const float sc = wave_scan(rev);
        const float rs = lane_get(sc, 63 - k);
        const float dtk = sm.dtl[k];
        const float g_dt = Ah * rs + zrc + ex2f(lend - sm.lam[k]) * qk;
        if (k < q) a.ddt[(row0 + k) * a.H + h] = g_dt;
        const float da = wave_sum(dtk * rs);
        if (k == 0) {
            a.dAp[bh * nsb + c] = da;
            a.dDp[bh * nsb + c] = sm.red[4] + sm.red[5] + sm.red[6] + sm.red[7];
        }
    }
}

// ---------------------------------------------------------------------------
// 4. Sums of the partials.
template <int N>
__global__ __launch_bounds__(256) void reduce_group(BwdArgs a) {
    const int64_t total = a.B * a.L * a.G * N;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int which = blockIdx.y;
    if (idx >= total) return;
    const int n = (int)(idx % N);
    const int64_t r = idx / N;               // (b, t, g)
    const int64_t gg = r % a.G, bt = r / a.G;
    const int64_t t = bt % a.L, b = bt / a.L;
    const int64_t hpg = a.H / a.G;
    const float *src = which ? a.dCp : a.dBp;
    float s = 0.f;
    for (int64_t k = 0; k < hpg; ++k) {
        const int64_t h = gg * hpg + k;
        s += src[((b * a.H + h) * a.nsb * kSub + t) * N + n];
    }
    (which ? a.dCm : a.dBm)[idx] = (__bf16)s;
}

__global__ __launch_bounds__(256) void reduce_head(BwdArgs a) {
    // block h: dA[h], dD[h] = sums over batch rows and sub-blocks
    __shared__ float part[2][256];
    const int64_t h = blockIdx.x;
    float sa = 0.f, sd = 0.f;
    for (int64_t k = threadIdx.x; k < a.B * a.nsb; k += blockDim.x) {
        const int64_t b = k / a.nsb, c = k % a.nsb;
        sa += a.dAp[(b * a.H + h) * a.nsb + c];
        sd += a.dDp[(b * a.H + h) * a.nsb + c];
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
    state_scan<N, false><<<dim3((unsigned)bhn), 256, 0, stream>>>(a);
    state_scan<N, true><<<dim3((unsigned)bhn), 256, 0, stream>>>(a);
    chunk_grad<N><<<dim3((unsigned)(bhn * a.nsb)), 256, 0, stream>>>(a);
    const int64_t total = a.B * a.L * a.G * N;
    reduce_group<N><<<dim3((unsigned)((total + 255) / 256), 2), 256, 0, stream>>>(a);
    reduce_head<<<dim3((unsigned)a.H), 256, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace

bool bwd_supported(int64_t P, int64_t N, int64_t H, int64_t G) {
    if (P != 64 || !(N == 64 || N == 128)) return false;
    const int64_t lim = (int64_t)1 << 31;
    return (int64_t)kSub * H * kP * 2 < lim && (int64_t)kSub * G * N * 2 < lim && (int64_t)kSub * H * 4 < lim;
}

// Workspace of the backward: states, adjoints and partials (floats).
size_t bwd_workspace_floats(int64_t B, int64_t L, int64_t H, int64_t N) {
    const int64_t nsb = (L + kSub - 1) / kSub;
    return (size_t)(4 * B * H * nsb * kSub * N + 2 * B * H * nsb);
}

hipError_t launch_scan_bwd(const void *x, const float *dt, const float *A, const void *Bm, const void *Cm,
                           const float *D, const float *init, const void *dy, const float *dfinal, void *dx,
                           float *ddt, float *dA, void *dBm, void *dCm, float *dD, float *dinit, float *ws,
                           int64_t B, int64_t L, int64_t H, int64_t G, int64_t N, hipStream_t stream) {
    const int64_t nsb = (L + kSub - 1) / kSub;
    const int64_t big = B * H * nsb * kSub * N;
    BwdArgs a{(const __bf16 *)x, (const __bf16 *)dy, (const __bf16 *)Bm, (const __bf16 *)Cm,
              dt, A, D, init, dfinal,
              (__bf16 *)dx, (__bf16 *)dBm, (__bf16 *)dCm,
              ddt, dA, dD, dinit,
              ws, ws + big, ws + 2 * big, ws + 3 * big, ws + 4 * big, ws + 4 * big + B * H * nsb,
              B, L, H, G, nsb};
    switch (N) {
        case 64: return launch<64>(a, stream);
        case 128: return launch<128>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace ssd
