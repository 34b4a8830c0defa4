// Chunk scan with one workgroup per (batch, head) sequence, on gfx950 matrix
// cores (bf16 operands, fp32 accumulation).
//
// A workgroup walks its sequence in sub-blocks of 64 tokens and carries the
// P x N state in matrix-core accumulators from the first token to the last:
// no state ever leaves the chip between sub-blocks, x is read once and y
// written once.  Per sub-block, with Lambda the inclusive prefix sum of dt*A
// inside the sub-block (Lambda_{-1} = 0), the block decomposition of the
// "Mamba-2" note (section "taking each path half way") and of the "Mamba-2
// model walkthrough" (sections 6.1-6.2) gives
//   y_i = exp(Lambda_i) Cm_i . H  +  sum_{j<=i} G[i][j] exp(Lambda_i - Lambda_j) dt_j x_j  +  D x_i
//   H  <- exp(Lambda_63) H  +  sum_j Bm_j (outer) (exp(Lambda_63 - Lambda_j) dt_j x_j)
// where G[i][j] = Cm_i . Bm_j comes from the gram kernel (shared by every
// head of a group) and H is the state entering the sub-block.
//
// Layout.  Wave w owns rows p = 16w..16w+15 of the state (held transposed,
// rows n, columns p, as in the other matrix-core kernels).  x, Bm and Cm of
// the sub-block are staged in LDS in their global, token-major order (16-byte
// rows written as loaded), with 16-byte chunks permuted per row by an XOR
// swizzle so that both the row writes and the reads below touch distinct
// banks.  The contractions over tokens need operands whose eight k-values are
// eight consecutive tokens of one column; gfx950's transposing LDS read
// (ds_read_b64_tr_b16) delivers them from the token-major tiles directly:
// within each 16-lane group, lane a+4q names row kbase+q, columns 4a..4a+3,
// and lane i receives rows kbase..kbase+3 of column i.
//
// Step.  One sub-block per step, two barriers: compute from LDS (and issue
// the global loads of the sub-block two ahead into a register slot), barrier,
// stage the next sub-block from registers into LDS, barrier.  Every global
// access is an unconditional buffer load or store whose range masks the
// ragged end of the sequence.
#include "common.h"

#include <type_traits>

namespace ssd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kP = 64;
constexpr int kSub = 64;
constexpr int kThreads = 256;
constexpr int kRaw = 0x00020000;   // buffer descriptor word 3: raw 32-bit access
constexpr int TS = kSub + 8;       // row stride (elements) of the masked matrix

struct WaveDecays {          // one wave's copy of a sub-block's decays (no barrier needed)
    float lam[kSub];         // Lambda of the sub-block being prepared
    float dt[kSub];          // its dt (0 past the end)
    float w[2][kSub];        // per step parity: exp(Lambda_63 - Lambda_j) dt_j
    float rdec[2][kSub];     //                  exp(Lambda_i)
    float gam[2][4];         //                  exp(Lambda_63) (element 0)
};

template <int N>
struct ChainSmem {
    __bf16 X[kSub * kP];     // x [j][p], chunks swizzled (xsw)
    __bf16 Bt[kSub * N];     // Bm [j][n], chunks swizzled (bsw)
    __bf16 Ct[kSub * N];     // Cm [i][n], chunks swizzled (csw)
    __bf16 Mm[kSub * TS];    // masked decay matrix [i][j]
    __bf16 Yo[kSub * kP];    // outputs y [i][p] of the step, chunks swizzled (ysw)
    WaveDecays wd[4];        // one per wave
};

// Chunk (16 bytes) swizzles: logical chunk c of row r is stored at c ^ f(r).
// x rows are 128 bytes (8 chunks); Bm and Cm rows are N*2 bytes.
__device__ __forceinline__ int xsw(int r) { return ((r >> 1) & 1) * 2 + ((r >> 3) & 1) * 4; }
__device__ __forceinline__ int ysw(int r) { return (r >> 1) & 7; }
template <int N>
__device__ __forceinline__ int bsw(int r) {
    if constexpr (N == 128) return 2 * (r & 3) + 8 * ((r >> 3) & 1);
    else return xsw(r);
}
template <int N>
__device__ __forceinline__ int csw(int r) {
    if constexpr (N == 128) return r & 15;
    else return (r >> 1) & 7;
}

template <int N>
struct Bulk {                // one sub-block's x, Bm and Cm, per thread (loaded one step ahead)
    uint4 x[2];              // x chunks u = tid + 256k: row u/8, chunk u%8
    uint4 b[N / 32];         // Bm chunks u = tid + 256k: row u/(N/8), chunk u%(N/8)
    uint4 c[N / 32];         // Cm, same mapping
};
struct Small {               // one sub-block's G tiles and dt, per thread (loaded two steps ahead)
    uint2 g[3];              // this wave's causal G tiles (fragment order)
    float dt;                // dt of token tid & 63
};

struct Args {
    const __bf16 *x;
    const float *dt, *A;
    const __bf16 *Bm, *Cm;
    const float *D, *init;
    __bf16 *y;
    float *final_state;
    const __bf16 *gram;
    int64_t L, H, G, nsb;
};

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    const __bf16 a = (__bf16)lo, b = (__bf16)hi;
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ void tile_of(int k, int &it, int &jt) {
    it = k < 1 ? 0 : k < 3 ? 1 : k < 6 ? 2 : 3;
    jt = k - (it * (it + 1)) / 2;
}
// The buffer builtins move raw 32-bit words: values go in and out through bit
// casts.  Only the vector and immediate offsets take part in the range check.
// Every buffer here is uniform across the workgroup (it depends only on the
// sequence and the step); readfirstlane states that, so that the descriptor
// lives in scalar registers instead of being built per lane.
__device__ __forceinline__ rsrc_t rsrc(const void *base, int bytes) {
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
    void *q = reinterpret_cast<void *>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(q, (short)0, __builtin_amdgcn_readfirstlane(bytes), kRaw);
}
__device__ __forceinline__ uint4 ld16(rsrc_t r, int voff) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}
// Transposing LDS read of four 16-bit values (see the file comment).
__device__ __forceinline__ bf16x4 tr4(const unsigned char *p) {
    return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)p));
}
template <class T>
__device__ __forceinline__ T lds_ld(const unsigned char *p) { return *reinterpret_cast<const T *>(p); }
template <class T>
__device__ __forceinline__ void lds_st(unsigned char *p, T v) { *reinterpret_cast<T *>(p) = v; }

// Per-lane byte offsets, fixed for the whole sequence.  Every access in the
// step loop is one of these plus a compile-time or scalar term: with the chunk
// swizzles above, the swizzled chunk of every row a lane touches depends only
// on row bits that its loop indices leave alone.
template <int N>
struct LaneOffs {
    static constexpr int NT = N / 16, KS = N / 32;
    static constexpr int RB = N * 2;          // bytes per Bm / Cm row
    static constexpr int CPR = N / 8;         // 16-byte chunks per Bm / Cm row
    int xtr;          // X, transposing reads:    + ks*4096 (+512 for rows +4)
    int xsk;          // X, skip-term reads:      + it*2048
    int mm;           // Mm, fragment reads:      + it*16*TS*2 + ks*64
    int mw;           // Mm, tile writes:         + (16 ti TS + 16 tj)*2
    int ct[KS][2];    // Ct, pieces n0 and n1:    + it*16*RB
    int bt[NT];       // Bt, transposing reads:   + ks*32*RB (+4*RB for rows +4)
    int sx, sb, sc;   // stage writes:            + k*4096 (x), + k*(256/CPR)*RB (Bm, Cm)
    int gx, gb;       // global loads:            + k*32*H*P*2 (x), + k*(256/CPR)*G*N*2 (Bm, Cm)
    int gd;           // dt loads
};

template <int N>
__device__ __forceinline__ LaneOffs<N> lane_offsets(int tid, int wave, int64_t H, int64_t G) {
    using O = LaneOffs<N>;
    const int lane = tid & 63, lrow = lane & 15, lgrp = lane >> 4, qa = lane & 3, qq = (lane & 15) >> 2;
    O o;
    const int r = 8 * lgrp + qq;                  // row (within a k-step) of the transposing reads
    o.xtr = r * 128 + (((2 * wave + (qa >> 1)) ^ xsw(r)) * 16) + (qa & 1) * 8;
    o.xsk = lrow * 128 + (((2 * wave + (lgrp >> 1)) ^ xsw(lrow)) * 16) + (lgrp & 1) * 8;
    o.mm = lrow * TS * 2 + 16 * lgrp;
    o.mw = lrow * TS * 2 + 8 * lgrp;
#pragma unroll
    for (int ks = 0; ks < O::KS; ++ks)
#pragma unroll
        for (int wh = 0; wh < 2; ++wh) {
            const int n = 32 * ks + 16 * wh + 4 * lgrp;
            o.ct[ks][wh] = lrow * O::RB + (((n >> 3) ^ csw<N>(lrow)) * 16) + (n & 7) * 2;
        }
#pragma unroll
    for (int t = 0; t < O::NT; ++t) {
        const int col = 16 * t + 4 * qa;
        o.bt[t] = r * O::RB + (((col >> 3) ^ bsw<N>(r)) * 16) + (col & 7) * 2;
    }
    {
        const int j = tid >> 3, c = tid & 7;
        o.sx = j * 128 + ((c ^ xsw(j)) * 16);
        o.gx = (int)(((int64_t)j * H * kP + 8 * c) * 2);
    }
    {
        const int j = tid / O::CPR, c = tid % O::CPR;
        o.sb = j * O::RB + ((c ^ bsw<N>(j)) * 16);
        o.sc = j * O::RB + ((c ^ csw<N>(j)) * 16);
        o.gb = (int)(((int64_t)j * G * N + 8 * c) * 2);
    }
    o.gd = (int)((int64_t)lane * H * 4);
    return o;
}

// Tokens of sub-block sb (>= 1) and its first row in the (batch, token) order.
__device__ __forceinline__ int sub_tokens(const Args &a, int sb) {
    const int64_t rem = a.L - (int64_t)sb * kSub;
    return rem < kSub ? (int)rem : kSub;
}

// Global loads of sub-block sb's x, Bm and Cm (masked past the end of the sequence).
template <int N>
__device__ __forceinline__ void load_bulk(Bulk<N> &sl, const Args &a, const LaneOffs<N> &o, int64_t b, int64_t h,
                                          int64_t g, int sb) {
    using O = LaneOffs<N>;
    const int q = sub_tokens(a, sb);
    const int64_t row0 = b * a.L + (int64_t)sb * kSub;
    {
        const rsrc_t r = rsrc(a.x + (row0 * a.H + h) * kP, (int)(((int64_t)(q - 1) * a.H * kP + kP) * 2));
        const int step = (int)(32 * a.H * kP * 2);
#pragma unroll
        for (int k = 0; k < 2; ++k) sl.x[k] = ld16(r, o.gx + k * step);
    }
    const int bytes = (int)(((int64_t)(q - 1) * a.G * N + N) * 2);
    const rsrc_t rb = rsrc(a.Bm + (row0 * a.G + g) * N, bytes);
    const rsrc_t rc = rsrc(a.Cm + (row0 * a.G + g) * N, bytes);
    const int step = (int)((256 / O::CPR) * a.G * N * 2);
#pragma unroll
    for (int k = 0; k < N / 32; ++k) {
        sl.b[k] = ld16(rb, o.gb + k * step);
        sl.c[k] = ld16(rc, o.gb + k * step);
    }
}

// Global loads of sub-block sb's G tiles (this wave's) and dt.
template <int N>
__device__ __forceinline__ void load_small(Small &sl, const Args &a, const LaneOffs<N> &o, int64_t b, int64_t h,
                                           int64_t g, int sb, int wave, int lane) {
    const int q = sub_tokens(a, sb);
    const int64_t row0 = b * a.L + (int64_t)sb * kSub;
    const rsrc_t rg = rsrc(a.gram + ((b * a.G + g) * a.nsb + sb) * (int64_t)(kSub * kSub), kSub * kSub * 2);
#pragma unroll
    for (int m = 0; m < 3; ++m) {
        const int k = wave + 4 * m < 10 ? wave + 4 * m : 9;   // waves with two tiles load their last twice
        sl.g[m] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rg, (k * 64 + lane) * 8, 0, 0));
    }
    const rsrc_t rd = rsrc(a.dt + row0 * a.H + h, (int)(((int64_t)(q - 1) * a.H + 1) * 4));
    sl.dt = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rd, o.gd, 0, 0));
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP: shifts of 1, 2,
// 4 and 8 lanes inside each row of 16 (lanes shifted in from outside the row
// contribute 0), then the last lane of row 0 is added to rows 1 and 3 and the
// last lane of row 1 (by then the total of rows 0-1) to rows 2 and 3.
__device__ __forceinline__ float wave_scan(float v) {
    auto shr = [](float x, auto ctrl) {
        return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), decltype(ctrl)::value, 0xf, 0xf, true));
    };
    v += shr(v, std::integral_constant<int, 0x111>{});   // row_shr:1
    v += shr(v, std::integral_constant<int, 0x112>{});   // row_shr:2
    v += shr(v, std::integral_constant<int, 0x114>{});   // row_shr:4
    v += shr(v, std::integral_constant<int, 0x118>{});   // row_shr:8
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xa, 0xf, false));   // row_bcast:15
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xc, 0xf, false));   // row_bcast:31
    return v;
}

// Per-token decays of one sub-block from its dt, into this wave's own copy
// (lane = token): the scan runs in every wave, so no barrier is needed.
__device__ __forceinline__ void wave_decays(WaveDecays &wd, int par, float dt, float Ah, int lane) {
    const float v = wave_scan(dt * Ah);
    const float lend = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
    wd.lam[lane] = v;
    wd.dt[lane] = dt;
    wd.w[par][lane] = __expf(lend - v) * dt;
    wd.rdec[par][lane] = __expf(v);
    if (lane == 0) wd.gam[par][0] = __expf(lend);
}

// This wave's tiles of the masked decay matrix M[i][j] = G[i][j]
// exp(Lambda_i - Lambda_j) dt_j (j <= i), from its G fragments and the decays
// that wave_decays just wrote, packed to bf16 in registers.
__device__ __forceinline__ void m_tiles(const WaveDecays &wd, const uint2 (&g)[3], uint2 (&mt)[3], int wave,
                                        int lrow, int lgrp) {
#pragma unroll
    for (int m = 0; m < 3; ++m) {
        const int k = wave + 4 * m < 10 ? wave + 4 * m : 9;
        int ti, tj;
        tile_of(k, ti, tj);
        const int i = 16 * ti + lrow, j0 = 16 * tj + 4 * lgrp;
        const float li = wd.lam[i];
        const f32x4 lj = *reinterpret_cast<const f32x4 *>(&wd.lam[j0]);
        const f32x4 dj = *reinterpret_cast<const f32x4 *>(&wd.dt[j0]);
        const uint32_t gw[2] = {g[m].x, g[m].y};
        float mv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float gv = (e & 1) ? hi_bf16(gw[e >> 1]) : lo_bf16(gw[e >> 1]);
            // above the diagonal the exponent is -inf (a select, not a branch)
            const float d = j0 + e <= i ? li - lj[e] : -__builtin_inff();
            mv[e] = gv * __expf(d) * dj[e];
        }
        mt[m] = uint2{pack2(mv[0], mv[1]), pack2(mv[2], mv[3])};
    }
}

// Stage a sub-block into LDS: x, Bm and Cm from registers as loaded (with the
// chunk swizzles), and this wave's tiles of the masked decay matrix.
template <int N>
__device__ __forceinline__ void stage(ChainSmem<N> &sm, const Bulk<N> &sl, const uint2 (&mt)[3],
                                      const LaneOffs<N> &o, int wave) {
    using O = LaneOffs<N>;
    unsigned char *Xb = reinterpret_cast<unsigned char *>(sm.X);
    unsigned char *Bb = reinterpret_cast<unsigned char *>(sm.Bt);
    unsigned char *Cb = reinterpret_cast<unsigned char *>(sm.Ct);
    unsigned char *Mb = reinterpret_cast<unsigned char *>(sm.Mm);
#pragma unroll
    for (int k = 0; k < 2; ++k) lds_st<uint4>(Xb + o.sx + k * 4096, sl.x[k]);
#pragma unroll
    for (int k = 0; k < N / 32; ++k) {
        lds_st<uint4>(Bb + o.sb + k * (256 / O::CPR) * O::RB, sl.b[k]);
        lds_st<uint4>(Cb + o.sc + k * (256 / O::CPR) * O::RB, sl.c[k]);
    }
#pragma unroll
    for (int m = 0; m < 3; ++m) {
        const int k = wave + 4 * m;
        if (k < 10) {
            int ti, tj;
            tile_of(k, ti, tj);
            lds_st<uint2>(Mb + o.mw + (16 * ti * TS + 16 * tj) * 2, mt[m]);
        }
    }
    if (wave >= 2) {
        // the tiles above the diagonal that the products read: (0,1) and (2,3)
        const int ti = wave == 2 ? 0 : 2;
        uint32_t z = 0;
        asm volatile("" : "+v"(z));
        lds_st<uint2>(Mb + o.mw + (16 * ti * TS + 16 * (ti + 1)) * 2, uint2{z, z});
    }
}

constexpr int kXcds = 8;

// Sequence of workgroup `blk` out of `n`: XCD x = blk % 8 runs the workgroups
// blk = x, x+8, x+16, ...; the k-th of them takes sequence start(x) + k, where
// the XCDs' ranges split [0, n) into eight contiguous parts (the first n % 8
// one longer).  A bijection on [0, n).
__device__ __forceinline__ int64_t xcd_chain(int64_t blk, int64_t n) {
    const int64_t x = blk % kXcds, k = blk / kXcds, per = n / kXcds, rem = n % kXcds;
    return x * per + (x < rem ? x : rem) + k;
}

template <int N>
__global__ __launch_bounds__(kThreads, 2) void chain_kernel(Args a) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    ChainSmem<N> &sm = *reinterpret_cast<ChainSmem<N> *>(smem_raw);
    using O = LaneOffs<N>;
    constexpr int NT = N / 16;
    constexpr int KS = N / 32;

    // (batch, head, group) of this workgroup, in scalar registers.  Workgroups
    // are dealt to the eight XCDs round-robin by index; each XCD is given a
    // contiguous range of sequences instead, so that the Bm, Cm, gram tiles and
    // dt lines its heads share stay in that XCD's L2.
    const int64_t chain = xcd_chain(blockIdx.x, gridDim.x);
    const int64_t b = __builtin_amdgcn_readfirstlane((int)(chain / a.H));
    const int64_t h = __builtin_amdgcn_readfirstlane((int)(chain % a.H));
    const int64_t g = __builtin_amdgcn_readfirstlane((int)(h / (a.H / a.G)));
    const int nsub = (int)((a.L + kSub - 1) / kSub);
    const float Ah = a.A[h], Dh = a.D[h];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, lrow = lane & 15, lgrp = lane >> 4;
    const LaneOffs<N> o = lane_offsets<N>(tid, wave, a.H, a.G);
    const unsigned char *Xb = reinterpret_cast<const unsigned char *>(sm.X);
    const unsigned char *Bb = reinterpret_cast<const unsigned char *>(sm.Bt);
    const unsigned char *Cb = reinterpret_cast<const unsigned char *>(sm.Ct);
    const unsigned char *Mb = reinterpret_cast<const unsigned char *>(sm.Mm);
    WaveDecays &wd = sm.wd[wave];

    Bulk<N> bulk;
    Small small[2];
    f32x4 Hacc[NT];
    {
        load_bulk<N>(bulk, a, o, b, h, g, 0);
        load_small<N>(small[0], a, o, b, h, g, 0, wave, lane);
        load_small<N>(small[1], a, o, b, h, g, nsub > 1 ? 1 : 0, wave, lane);
        // entering state: the initial state or zeros
        const rsrc_t ri = rsrc(a.init ? (const void *)(a.init + chain * (kP * N)) : (const void *)a.x,
                               a.init ? kP * N * 4 : 0);
        const int lane_off = (16 * wave + lrow) * N + 4 * lgrp;
#pragma unroll
        for (int t = 0; t < NT; ++t)
            Hacc[t] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ri, (lane_off + 16 * t) * 4, 0, 0));
        uint2 mt[3];
        wave_decays(wd, 0, small[0].dt, Ah, lane);
        m_tiles(wd, small[0].g, mt, wave, lrow, lgrp);
        stage<N>(sm, bulk, mt, o, wave);
        __syncthreads();
    }

    // One step: sub-block s from LDS.  `sm_cur` holds the G tiles and dt of
    // sub-block s+1 (loaded a step ago); `sm_nxt` receives those of s+2, and
    // `bulk` (staged already) receives x, Bm and Cm of s+1.
    auto step = [&](int s, const Small &sm_cur, Small &sm_nxt) {
        const int par = s & 1;

        // ---- loads: G tiles and dt of sub-block s+2
        load_small<N>(sm_nxt, a, o, b, h, g, s + 2 < nsub ? s + 2 : nsub - 1, wave, lane);
        // ---- decays and masked-matrix tiles of sub-block s+1 (in registers until staged)
        uint2 mt[3];
        if (s + 1 < nsub) {
            wave_decays(wd, par ^ 1, sm_cur.dt, Ah, lane);
            m_tiles(wd, sm_cur.g, mt, wave, lrow, lgrp);
        }

        // ---- loads: x, Bm and Cm of sub-block s+1 (issued after the decays,
        // which wait on the dt loaded a step ago)
        load_bulk<N>(bulk, a, o, b, h, g, s + 1 < nsub ? s + 1 : nsub - 1);

        // ---- inter-block part: Y^T[p][i] = exp(Lambda_i) sum_n H[p][n] Cm_i[n]
        f32x4 Y[4];
#pragma unroll
        for (int it = 0; it < 4; ++it) Y[it] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            bf16x8 cf[4];
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const bf16x4 c0 = lds_ld<bf16x4>(Cb + o.ct[ks][0] + it * 16 * O::RB);
                const bf16x4 c1 = lds_ld<bf16x4>(Cb + o.ct[ks][1] + it * 16 * O::RB);
                cf[it] = bf16x8{c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
            }
            bf16x8 ah;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ah[e] = (__bf16)Hacc[2 * ks][e];
                ah[4 + e] = (__bf16)Hacc[2 * ks + 1][e];
            }
#pragma unroll
            for (int it = 0; it < 4; ++it) Y[it] = mfma(ah, cf[it], Y[it]);
        }

        // ---- x fragments (rows p of this wave, eight consecutive tokens per
        // k-group) and the masked-matrix fragments of the intra-block part
        bf16x8 xf[2], mf[4][2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const bf16x4 lo = tr4(Xb + o.xtr + ks * 4096);
            const bf16x4 hi = tr4(Xb + o.xtr + ks * 4096 + 512);
            xf[ks] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
#pragma unroll
        for (int it = 0; it < 4; ++it)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                if (!(ks == 1 && it < 2)) mf[it][ks] = lds_ld<bf16x8>(Mb + o.mm + it * 16 * TS * 2 + ks * 64);
        {
            const f32x4 rd = {wd.rdec[par][lrow], wd.rdec[par][16 + lrow], wd.rdec[par][32 + lrow],
                              wd.rdec[par][48 + lrow]};
#pragma unroll
            for (int it = 0; it < 4; ++it) Y[it] *= rd[it];
        }
        // ---- intra-block part: Y^T[p][i] += sum_j x_j[p] M[i][j] (causal k-steps only)
#pragma unroll
        for (int it = 0; it < 4; ++it)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                if (!(ks == 1 && it < 2)) Y[it] = mfma(xf[ks], mf[it][ks], Y[it]);

        // ---- state update: H <- exp(Lambda_63) H + sum_j Bm_j (outer) (w_j x_j)
        {
            const float gam = wd.gam[par][0];
#pragma unroll
            for (int t = 0; t < NT; ++t) Hacc[t] *= gam;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const f32x4 w0 = *reinterpret_cast<const f32x4 *>(&wd.w[par][32 * ks + 8 * lgrp]);
                const f32x4 w1 = *reinterpret_cast<const f32x4 *>(&wd.w[par][32 * ks + 8 * lgrp + 4]);
                bf16x8 xw;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    xw[e] = (__bf16)((float)xf[ks][e] * w0[e]);
                    xw[4 + e] = (__bf16)((float)xf[ks][4 + e] * w1[e]);
                }
                // Bm fragments in batches of four tiles
#pragma unroll
                for (int t0 = 0; t0 < NT; t0 += 4) {
                    bf16x8 bt[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const bf16x4 lo = tr4(Bb + o.bt[t0 + u] + ks * 32 * O::RB);
                        const bf16x4 hi = tr4(Bb + o.bt[t0 + u] + ks * 32 * O::RB + 4 * O::RB);
                        bt[u] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    }
#pragma unroll
                    for (int u = 0; u < 4; ++u) Hacc[t0 + u] = mfma(bt[u], xw, Hacc[t0 + u]);
                }
            }
        }
        // ---- skip term; the outputs go to LDS (lane holds token i = 16it + lrow,
        // p = 16w + 4lgrp + 0..3) and leave as whole rows after the barrier
        {
            unsigned char *Yb = reinterpret_cast<unsigned char *>(sm.Yo);
            const int p0 = 16 * wave + 4 * lgrp;
            const int yw = lrow * 128 + (((p0 >> 3) ^ ysw(lrow)) * 16) + (p0 & 7) * 2;
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const bf16x4 xs = lds_ld<bf16x4>(Xb + o.xsk + it * 2048);
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = Y[it][e] + Dh * (float)xs[e];
                lds_st<uint2>(Yb + yw + it * 16 * 128, uint2{pack2(v[0], v[1]), pack2(v[2], v[3])});
            }
        }
        __syncthreads();
        // ---- y rows 16w..16w+15 of this step to memory (16 bytes per lane)
        {
            const int64_t t0 = (int64_t)s * kSub;
            const int64_t rem = a.L - t0;
            const int q = rem < kSub ? (int)rem : kSub;
            const rsrc_t ry = rsrc(a.y + ((b * a.L + t0) * a.H + h) * kP, (int)(((int64_t)(q - 1) * a.H * kP + kP) * 2));
            const unsigned char *Yb = reinterpret_cast<const unsigned char *>(sm.Yo);
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int u = lane + 64 * k, row = 16 * wave + (u >> 3), c = u & 7;
                const uint4 v = lds_ld<uint4>(Yb + row * 128 + ((c ^ ysw(row)) * 16));
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), ry,
                                                       (int)(((int64_t)row * a.H * kP + 8 * c) * 2), 0, 0);
            }
        }
        // ---- stage sub-block s+1
        if (s + 1 < nsub) stage<N>(sm, bulk, mt, o, wave);
        __syncthreads();
    };

    int s = 0;
    for (; s + 1 < nsub; s += 2) {
        step(s, small[1], small[0]);
        step(s + 1, small[0], small[1]);
    }
    if (s < nsub) step(s, small[1], small[0]);

    // leaving state
    if (a.final_state) {
        float *dst = a.final_state + chain * (kP * N) + (16 * wave + lrow) * N + 4 * lgrp;
#pragma unroll
        for (int t = 0; t < NT; ++t) *reinterpret_cast<f32x4 *>(dst + 16 * t) = Hacc[t];
    }
}

template <int N>
hipError_t launch(const ScanArgs &sa, const Workspace &ws) {
    const int64_t nsb = (sa.L + kSub - 1) / kSub;
    hipError_t e = launch_gram(sa, ws, nsb);
    if (e != hipSuccess) return e;
    const size_t smem = sizeof(ChainSmem<N>);
    auto kern = chain_kernel<N>;
    static bool configured = false;
    if (!configured) {
        e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (e != hipSuccess) return e;
        configured = true;
    }
    Args a{(const __bf16 *)sa.x, sa.dt, sa.A, (const __bf16 *)sa.Bm, (const __bf16 *)sa.Cm, sa.D,
           sa.init, (__bf16 *)sa.y, sa.final_state, (const __bf16 *)ws.gram, sa.L, sa.H, sa.G, nsb};
    kern<<<dim3((unsigned)(sa.B * sa.H)), kThreads, smem, sa.stream>>>(a);
    return hipGetLastError();
}

}  // namespace

// Shapes the per-sequence kernel takes: P = 64, N in {64, 128}, and one
// sub-block's rows of x, Bm and Cm within the 2^31-byte reach of a buffer
// offset (offsets are taken from each sub-block's first token).
bool chain_supported(int64_t H, int64_t G, int64_t N) {
    if (!(N == 64 || N == 128)) return false;
    const int64_t lim = (int64_t)1 << 31;
    return (int64_t)kSub * H * kP * 2 < lim && (int64_t)kSub * G * N * 2 < lim && (int64_t)kSub * H * 4 < lim;
}

hipError_t launch_chain_scan(const ScanArgs &a, const Workspace &ws) {
    switch (a.N) {
        case 64: return launch<64>(a, ws);
        case 128: return launch<128>(a, ws);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace ssd
