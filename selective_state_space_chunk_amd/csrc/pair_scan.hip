// Chunk scan with one workgroup per pair of adjacent heads of one batch row
// (and one group of Bm / Cm), on gfx950 matrix cores (bf16 operands, fp32
// accumulation).
//
// The arithmetic per 64-token sub-block is that of pipe_scan.hip: with Lambda
// the inclusive prefix sum of dt*A inside the sub-block, the block
// decomposition of the "Mamba-2" note (section "taking each path half way")
// and of the "Mamba-2 model walkthrough" (sections 6.1-6.2) gives
//   y_i = exp(Lambda_i) Cm_i . H  +  sum_{j<=i} G[i][j] exp(Lambda_i - Lambda_j) dt_j x_j  +  D x_i
//   H  <- exp(Lambda_63) H  +  sum_j Bm_j (outer) (exp(Lambda_63 - Lambda_j) dt_j x_j)
// with G[i][j] = Cm_i . Bm_j from the gram kernel and H the state entering
// the sub-block.
//
// Why pairs: the two heads share Bm, Cm and the gram tiles, so one staged copy
// serves both, and each token row of x and y is touched as 256 contiguous
// bytes instead of 128 (streams of single-head rows saturate HBM well below
// its peak on this part).
//
// Eight waves, two on each SIMD: wave w works on head w / 4 and owns rows
// p = 16 (w % 4) .. +15 of its state, which stays in matrix-core accumulators
// from the first token to the last.  In step t a wave
//   - forms the inter-block term of sub-block t from the state entering it,
//     adds the masked intra-block product (the skip term D x_i rides on the
//     diagonal of the masked matrix) and stores its 16 columns of y;
//   - advances its state over sub-block t;
//   - builds its share of the masked decay matrix of sub-block t+1;
//   - stages its share of sub-block t+1: x of its own head, and Bm (waves of
//     the first head) or Cm (waves of the second).
// One barrier per step; x, Bm, Cm and the masked matrices alternate between
// two LDS slots, so nothing written in a step is read in it by another wave.
// Every step issues the same global loads and stores (loads past the last
// sub-block are masked to zeros), and the work past the end is harmless.
#include "tile_ops.h"

namespace ssd {
namespace {

using namespace tile;
constexpr int kThreads = 512;

struct PairArgs {
    const __bf16 *x;
    const float *dt, *A;
    const __bf16 *Bm, *Cm;
    const float *D, *init;
    __bf16 *y;
    float *final_state;
    const __bf16 *gram;
    int64_t L, H, G, nsb;
    int npairs;
};

template <int N>
struct PairSmem {
    __bf16 X[2][2][kSub * kP];     // [slot][head] x [j][p], chunks swizzled (xsw)
    __bf16 Bt[2][kSub * N];        // [slot] Bm [j][n], chunks swizzled (bsw)
    __bf16 Ct[2][kSub * N];        // [slot] Cm [i][n], chunks swizzled (csw)
    __bf16 Mm[2][2][kSub * kSub];  // [slot][head] masked decay matrix [i][j], chunks swizzled (msw)
    WaveDecays wd[2][8];           // [slot][wave] each wave's decays of sub-blocks t and t+1
};

struct PairSmall {                 // one sub-block's dt (lane = token) and this wave's G tiles
    uint2 g[3];
    float dt;
};

// Loads of one sub-block, given the element offset of its first row and its
// number of tokens q (rows past q, and every row when q <= 0, read as zeros).
template <int N>
__device__ __forceinline__ void load_x(BulkX &sl, const __bf16 *x, int64_t H, const LaneOffs<N> &o, int64_t xo, int q) {
    const rsrc_t r = rsrc(x + xo, q > 0 ? (int)(((int64_t)(q - 1) * H * kP + kP) * 2) : 0);
    const int step = (int)(32 * H * kP * 2);
#pragma unroll
    for (int k = 0; k < 2; ++k) sl.x[k] = ld16(r, o.gx + k * step);
}
template <int N>
__device__ __forceinline__ void load_rows(uint4 (&v)[N / 32], const __bf16 *src, int64_t G, const LaneOffs<N> &o,
                                          int64_t bo, int q) {
    using O = LaneOffs<N>;
    const rsrc_t r = rsrc(src + bo, q > 0 ? (int)(((int64_t)(q - 1) * G * N + N) * 2) : 0);
    const int step = (int)((256 / O::CPR) * G * N * 2);
#pragma unroll
    for (int k = 0; k < N / 32; ++k) v[k] = ld16(r, o.gb + k * step);
}
template <int N>
__device__ __forceinline__ void load_small(PairSmall &sl, const PairArgs &a, const LaneOffs<N> &o, int64_t go,
                                           int64_t dof, int q, int pq, int lane) {
    const rsrc_t rg = rsrc(a.gram + go, q > 0 ? kSub * kSub * 2 : 0);
#pragma unroll
    for (int m = 0; m < 3; ++m) {
        const int k = pq + 4 * m < 10 ? pq + 4 * m : 9;   // waves with two tiles load their last twice
        sl.g[m] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rg, (k * 64 + lane) * 8, 0, 0));
    }
    const rsrc_t rd = rsrc(a.dt + dof, q > 0 ? (int)(((int64_t)(q - 1) * a.H + 1) * 4) : 0);
    sl.dt = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rd, o.gd, 0, 0));
}

template <int N>
__global__ __launch_bounds__(kThreads, 1) void pair_kernel(PairArgs a) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    PairSmem<N> &sm = *reinterpret_cast<PairSmem<N> *>(smem_raw);
    using O = LaneOffs<N>;
    constexpr int NT = N / 16;
    constexpr int KS = N / 32;

    const int nsub = (int)((a.L + kSub - 1) / kSub);
    const int64_t pair = xcd_chain(blockIdx.x, a.npairs);
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hd = wave >> 2, pq = wave & 3;
    const int lane = tid & 63, lrow = lane & 15, lgrp = lane >> 4;
    const int64_t hpr = a.H / 2;
    const int64_t b = __builtin_amdgcn_readfirstlane((int)(pair / hpr));
    const int64_t h = __builtin_amdgcn_readfirstlane((int)(2 * (pair % hpr) + hd));
    const int64_t g = __builtin_amdgcn_readfirstlane((int)(h / (a.H / a.G)));   // same for both heads
    const int64_t chain = b * a.H + h;
    const float Ah2 = a.A[h] * kLog2e, Dh = a.D[h];
    const LaneOffs<N> o = lane_offsets<N>(tid, pq, a.H, a.G);

    // element offsets of sub-block tau's first row in x / y, dt, Bm / Cm and the gram tiles
    const int64_t SX = kSub * a.H * kP, SD = kSub * a.H, SB = kSub * a.G * N, SG = kSub * kSub;
    const int64_t xo = (b * a.L * a.H + h) * kP, dof = b * a.L * a.H + h, bo = (b * a.L * a.G + g) * N,
                  go = (b * a.G + g) * a.nsb * SG;
    auto q_of = [&](int tau) {
        const int64_t rem = a.L - (int64_t)tau * kSub;
        return rem < kSub ? (int)rem : kSub;
    };
    // this wave's half of the shared rows: Bm for the first head, Cm for the second
    const __bf16 *rows = hd ? a.Cm : a.Bm;

    BulkX xr[2];                 // x of sub-blocks t+1 (staged at the end of step t) and t+2
    uint4 br[N / 32];            // Bm or Cm rows of sub-block t+1 (loaded at the start of step t)
    PairSmall small[2];          // dt and G tiles of sub-blocks t+1 and t+2

    auto stage = [&](int slot, const BulkX &xs, const uint4 (&bs)[N / 32]) __attribute__((always_inline)) {
        unsigned char *Xb = reinterpret_cast<unsigned char *>(sm.X[slot][hd]);
#pragma unroll
        for (int k = 0; k < 2; ++k) lds_st<uint4>(Xb + o.sx + k * 4096, xs.x[k]);
        if (hd == 0) {
            unsigned char *Bb = reinterpret_cast<unsigned char *>(sm.Bt[slot]);
#pragma unroll
            for (int k = 0; k < N / 32; ++k) lds_st<uint4>(Bb + o.sb + k * (256 / O::CPR) * O::RB, bs[k]);
        } else {
            unsigned char *Cb = reinterpret_cast<unsigned char *>(sm.Ct[slot]);
#pragma unroll
            for (int k = 0; k < N / 32; ++k) lds_st<uint4>(Cb + o.sc[k], bs[k]);
        }
    };
    // decays of a sub-block (dt in lane = token) into this wave's LDS copy in
    // slot `slot`; returns exp(Lambda_63)
    auto decays = [&](float dt, int slot) __attribute__((always_inline)) {
        WaveDecays &wd = sm.wd[slot][wave];
        const float v = wave_scan(dt * Ah2);
        const float lend = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
        wd.lam[lane] = v;
        wd.dt[lane] = dt;
        wd.w[lane] = ex2(lend - v) * dt;
        wd.rdec[lane] = ex2(v);
        return ex2(lend);
    };
    // this wave's tiles of the masked decay matrix of the sub-block whose
    // decays are in slot `slot`, into slot `slot`
    auto build_m = [&](const PairSmall &sl, int slot) __attribute__((always_inline)) {
        const WaveDecays &wd = sm.wd[slot][wave];
        // the lane's row and column group, opaque to the compiler so that the
        // masks below are formed here in each step rather than held in
        // scalar registers across the loop
        int lr = lrow, lg = lgrp;
        asm volatile("" : "+v"(lr), "+v"(lg));
        uint2 mt[3];
#pragma unroll
        for (int m = 0; m < 3; ++m) {
            const int k = pq + 4 * m < 10 ? pq + 4 * m : 9;
            int ti, tj;
            tile_of(k, ti, tj);
            const int i = 16 * ti + lr, j0 = 16 * tj + 4 * lg;
            const float li = wd.lam[i];
            const f32x4 lj = *reinterpret_cast<const f32x4 *>(&wd.lam[j0]);
            const f32x4 dj = *reinterpret_cast<const f32x4 *>(&wd.dt[j0]);
            const uint32_t gw[2] = {sl.g[m].x, sl.g[m].y};
            float mv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float gv = (e & 1) ? hi_bf16(gw[e >> 1]) : lo_bf16(gw[e >> 1]);
                const float d = j0 + e <= i ? li - lj[e] : -__builtin_inff();
                mv[e] = __builtin_fmaf(gv * ex2(d), dj[e], j0 + e == i ? Dh : 0.f);
            }
            mt[m] = uint2{pack2(mv[0], mv[1]), pack2(mv[2], mv[3])};
        }
        unsigned char *Mw = reinterpret_cast<unsigned char *>(sm.Mm[slot][hd]);
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

    // prologue: sub-block 0 staged, its decays and masked matrix built;
    // sub-block 1 in flight
    load_x<N>(xr[0], a.x, a.H, o, xo, q_of(0));
    load_rows<N>(br, rows, a.G, o, bo, q_of(0));
    load_small<N>(small[0], a, o, go, dof, q_of(0), pq, lane);
    load_small<N>(small[1], a, o, go + SG, dof + SD, q_of(1), pq, lane);
    stage(0, xr[0], br);
    load_x<N>(xr[1], a.x, a.H, o, xo + SX, q_of(1));
    if (hd) load_rows<N>(br, rows, a.G, o, bo + SB, q_of(1));
    float gamv[2];   // exp(Lambda_63) of sub-blocks t and t+1, by parity
    gamv[0] = decays(small[0].dt, 0);
    build_m(small[0], 0);
    f32x4 Hacc[NT];
    const int lane_off = (16 * pq + lrow) * N + 4 * lgrp;
    {
        const rsrc_t ri = rsrc(a.init ? (const void *)(a.init + chain * (kP * N)) : (const void *)a.x,
                               a.init ? kP * N * 4 : 0);
#pragma unroll
        for (int u = 0; u < NT; ++u)
            Hacc[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ri, (lane_off + 16 * u) * 4, 0, 0));
    }
    __syncthreads();

    // Step t in two halves.  `body` forms the outputs of sub-block t and
    // advances the state over it; `next` prepares sub-block t+1 (decays, masked
    // matrix, staging).  The waves of the first head run body then next, those
    // of the second head next then body, so that the two waves on a SIMD are in
    // different phases (matrix-core and LDS work against vector work).  The
    // Bm / Cm rows that the second head's waves stage at the start of step t
    // were loaded in step t-1.
    auto body = [&](int t, int par) __attribute__((always_inline)) {
        const WaveDecays &wd = sm.wd[par][wave];
        const float gam = gamv[par];
        const unsigned char *Xb = reinterpret_cast<const unsigned char *>(sm.X[par][hd]);
        const unsigned char *Bb = reinterpret_cast<const unsigned char *>(sm.Bt[par]);
        const unsigned char *Cb = reinterpret_cast<const unsigned char *>(sm.Ct[par]);
        const unsigned char *Mr = reinterpret_cast<const unsigned char *>(sm.Mm[par][hd]);
        // Bm or Cm rows of sub-block t+1; dt, G tiles and x of sub-block t+2 into
        // the slots of sub-block t (staged in the previous step)
        load_rows<N>(br, rows, a.G, o, bo + (t + 1 + hd) * SB, q_of(t + 1 + hd));
        {
            const int tl = t + 2, ql = q_of(tl);
            load_small<N>(small[par], a, o, go + tl * SG, dof + tl * SD, ql, pq, lane);
            load_x<N>(xr[par], a.x, a.H, o, xo + tl * SX, ql);
        }

        // LDS reads are issued one k-step ahead of the products that use them
        // (Cm fragments of the inter-block term, then the masked matrix, then
        // the Bm fragments of the update), so that few fragments are live at once
        auto read_cf = [&](int ks, bf16x8 (&cf)[4]) __attribute__((always_inline)) {
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const bf16x4 c0 = lds_ld<bf16x4>(Cb + it * 16 * O::RB + (o.ct[ks][0] ^ csw_tile_bytes<N>(it)));
                const bf16x4 c1 = lds_ld<bf16x4>(Cb + it * 16 * O::RB + (o.ct[ks][1] ^ csw_tile_bytes<N>(it)));
                cf[it] = bf16x8{c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
            }
        };
        // Bm fragments of the update, in groups of four n-tiles (k-step ks, tiles 4v..4v+3)
        auto read_bt = [&](int ks, int v, bf16x8 (&bt)[4]) __attribute__((always_inline)) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const bf16x4 lo = tr4(Bb + o.bt[4 * v + u] + ks * 32 * O::RB);
                const bf16x4 hi = tr4(Bb + o.bt[4 * v + u] + ks * 32 * O::RB + 4 * O::RB);
                bt[u] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            }
        };
        bf16x8 cf[2][4];
        read_cf(0, cf[0]);
        bf16x8 xf[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const bf16x4 lo = tr4(Xb + o.xtr + ks * 4096);
            const bf16x4 hi = tr4(Xb + o.xtr + ks * 4096 + 512);
            xf[ks] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
        const f32x4 rd = {wd.rdec[lrow], wd.rdec[16 + lrow], wd.rdec[32 + lrow], wd.rdec[48 + lrow]};
        __builtin_amdgcn_sched_barrier(0);

        // inter-block term: Y^T[p][i] = exp(Lambda_i) sum_n H[p][n] Cm_i[n]
        f32x4 Y[4];
#pragma unroll
        for (int it = 0; it < 4; ++it) Y[it] = f32x4{0.f, 0.f, 0.f, 0.f};
        bf16x8 mf[4][2];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + 1 < KS) {
                read_cf(ks + 1, cf[(ks + 1) & 1]);
            } else {
#pragma unroll
                for (int it = 0; it < 4; ++it)
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk)
                        if (!(kk == 1 && it < 2)) mf[it][kk] = lds_ld<bf16x8>(Mr + o.mm[kk] + it * 2048);
            }
            const bf16x8 ah = to_bf16x8(Hacc[2 * ks], Hacc[2 * ks + 1]);
#pragma unroll
            for (int it = 0; it < 4; ++it) Y[it] = mfma(ah, cf[ks & 1][it], Y[it]);
            __builtin_amdgcn_sched_barrier(0);
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
        // plus the masked intra-block product
#pragma unroll
        for (int it = 0; it < 4; ++it) Y[it] *= rd[it];
#pragma unroll
        for (int it = 0; it < 4; ++it)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                if (!(ks == 1 && it < 2)) Y[it] = mfma(xf[ks], mf[it][ks], Y[it]);
        __builtin_amdgcn_sched_barrier(0);
        {
            const int q = q_of(t);
            const rsrc_t ry = rsrc(a.y + xo + t * SX, q > 0 ? (int)(((int64_t)(q - 1) * a.H * kP + kP) * 2) : 0);
            const int ystep = (int)(16 * a.H * kP * 2);
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const uint2 pk = uint2{pack2(Y[it][0], Y[it][1]), pack2(Y[it][2], Y[it][3])};
                __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, pk), ry, o.gy + it * ystep, 0, 0);
            }
        }

        // state update over sub-block t: H <- exp(Lambda_63) H + sum_j Bm_j (outer) (w_j x_j)
#pragma unroll
        for (int u = 0; u < NT; ++u) Hacc[u] *= gam;
#pragma unroll
        for (int r = 0; r < 2 * NG; ++r) {
            const int ks = r / NG, v = r % NG;
            if (r + 1 < 2 * NG) read_bt((r + 1) / NG, (r + 1) % NG, bt[(r + 1) & 1]);
#pragma unroll
            for (int u = 0; u < 4; ++u) Hacc[4 * v + u] = mfma(bt[r & 1][u], xw[ks], Hacc[4 * v + u]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // decays and masked matrix of sub-block t+1; its x, Bm, Cm into LDS
    auto next = [&](int par) __attribute__((always_inline)) {
        gamv[par ^ 1] = decays(small[par ^ 1].dt, par ^ 1);
        build_m(small[par ^ 1], par ^ 1);
        stage(par ^ 1, xr[par ^ 1], br);
    };
    auto step = [&](int t, int par) __attribute__((always_inline)) {
        if (hd) {
            next(par);
            body(t, par);
        } else {
            body(t, par);
            next(par);
        }
        __syncthreads();
    };
    int t = 0;
    for (; t + 1 < nsub; t += 2) {
        step(t, 0);
        step(t + 1, 1);
    }
    if (t < nsub) step(t, 0);

    if (a.final_state) {
        float *dst = a.final_state + chain * (kP * N) + lane_off;
#pragma unroll
        for (int u = 0; u < NT; ++u) *reinterpret_cast<f32x4 *>(dst + 16 * u) = Hacc[u];
    }
}

template <int N>
hipError_t launch(const ScanArgs &sa, const Workspace &ws) {
    const int64_t nsb = (sa.L + kSub - 1) / kSub;
    hipError_t e = launch_gram(sa, ws, nsb);
    if (e != hipSuccess) return e;
    const size_t smem = sizeof(PairSmem<N>);
    auto kern = pair_kernel<N>;
    static bool configured = false;
    if (!configured) {
        e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (e != hipSuccess) return e;
        configured = true;
    }
    PairArgs a{(const __bf16 *)sa.x, sa.dt, sa.A, (const __bf16 *)sa.Bm, (const __bf16 *)sa.Cm, sa.D,
               sa.init, (__bf16 *)sa.y, sa.final_state, (const __bf16 *)ws.gram,
               sa.L, sa.H, sa.G, nsb, (int)(sa.B * sa.H / 2)};
    kern<<<dim3((unsigned)a.npairs), kThreads, smem, sa.stream>>>(a);
    return hipGetLastError();
}

}  // namespace

bool pair_supported(int64_t H, int64_t G, int64_t N) {
    if (!(N == 64 || N == 128)) return false;
    if (H % 2 != 0 || G <= 0 || H % G != 0 || (H / G) % 2 != 0) return false;
    const int64_t lim = (int64_t)1 << 31;
    return (int64_t)kSub * H * kP * 2 < lim && (int64_t)kSub * G * N * 2 < lim && (int64_t)kSub * H * 4 < lim;
}

hipError_t launch_pair_scan(const ScanArgs &a, const Workspace &ws) {
    switch (a.N) {
        case 64: return launch<64>(a, ws);
        case 128: return launch<128>(a, ws);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace ssd
