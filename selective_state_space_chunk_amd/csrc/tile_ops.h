// Device helpers of the per-sequence matrix-core scan kernels
// (pipe_scan.hip): vector types, matrix-core and buffer
// intrinsics, the LDS swizzles of the x, Bm, Cm and masked-decay tiles, the
// per-lane offsets of the fragment reads and staging copies, and the wave-wide
// prefix sum of dt*A.
#pragma once
#include "common.h"

#include <type_traits>

namespace ssd {
namespace tile {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kP = 64;
constexpr int kSub = 64;
constexpr int kRaw = 0x00020000;   // buffer descriptor word 3: raw 32-bit access
constexpr int kXcds = 8;

struct WaveDecays {          // one wave's decays of the sub-block it works on
    float lam[kSub];         // Lambda log2(e)
    float dt[kSub];          // dt (0 past the end)
    float w[kSub];           // exp(Lambda_63 - Lambda_j) dt_j
    float rdec[kSub];        // exp(Lambda_i)
};

__device__ __forceinline__ int xsw(int r) { return ((r >> 1) & 1) * 2 + ((r >> 3) & 1) * 4; }
// (rows of 256 or 512 bytes start on the same bank, so N = 256 uses the
// N = 128 patterns, which only permute chunks within each 256-byte half)
template <int N>
__device__ __forceinline__ int bsw(int r) {
    if constexpr (N >= 128) return 2 * (r & 3) + 8 * ((r >> 3) & 1);
    else return xsw(r);
}
// Cm rows: rows 16 apart get different chunk permutations, so that the
// fragment reads of consecutive 16-row tiles never fall on the same banks
// (the compiler would otherwise pair them into one two-address read whose
// halves collide).
// At N = 256 the rows of 16-row tile `it` are shifted by ct_pad * it bytes
// instead (a padded layout): the same bank separation of consecutive tiles,
// but the tile offset of a fragment read becomes an immediate, which saves the
// compute waves 24 address registers.
template <int N>
__device__ __forceinline__ int csw(int r) {
    if constexpr (N == 256) return r & 15;
    else if constexpr (N == 128) return (r & 15) ^ (((r >> 4) & 3) << 2);
    else return ((r >> 1) & 7) ^ (((r >> 4) & 3) << 1);
}
// byte XOR that csw applies to the rows of 16-row tile `it` beyond row-in-tile bits
template <int N>
__device__ __forceinline__ constexpr int csw_tile_bytes(int it) {
    return N == 256 ? 0 : (N == 128 ? 64 : 32) * (it & 3);
}
// bytes by which each 16-row tile of Cm is shifted (N = 256), and the bytes
// of a staged Cm sub-block
template <int N>
constexpr int ct_pad = N == 256 ? 64 : 0;
template <int N>
constexpr int ct_bytes = kSub * N * 2 + 3 * ct_pad<N>;
// Bm staging: chunk k of a thread lies 256/CPR rows below chunk 0; at N = 256
// that is 8 rows, which flips bit 3 of the row and with it bsw's bit 3
// (byte XOR 128) on odd k.  At N <= 128 the rows keep their swizzle.
template <int N>
__device__ __forceinline__ constexpr int sb_flip(int k) { return N == 256 ? 128 * (k & 1) : 0; }
// masked decay matrix rows (128 bytes): chunk c of row r at c ^ msw(r)
__device__ __forceinline__ int msw(int r) { return (r >> 1) & 7; }

// One sub-block's x is loaded and staged by the state waves, its Bm and Cm by
// the output waves (thread u = tid or tid - 256 of its role).
struct BulkX {
    uint4 x[2];              // x chunks u + 256k: row (u + 256k)/8, chunk u%8
};
template <int N>
struct BulkBC {
    uint4 b[N / 32];         // Bm chunks u + 256k: row (u + 256k)/(N/8), chunk u%(N/8)
    uint4 c[N / 32];         // Cm, same mapping
};
struct Small {               // one sub-block's dt (lane = token) and, for output waves, G tiles
    uint2 g[3];
    float dt;
};

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// Two floats to two bfloat16 (round to nearest even) in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}
__device__ __forceinline__ bf16x8 to_bf16x8(f32x4 lo, f32x4 hi) {
    return __builtin_convertvector(f32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]}, bf16x8);
}
// 2^x on the transcendental unit (v_exp_f32).  The decays are kept in base-2
// units (Lambda * log2 e), so exp(Lambda_i - Lambda_j) = exp2(lam_i - lam_j).
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
constexpr float kLog2e = 1.4426950408889634f;
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ void tile_of(int k, int &it, int &jt) {
    it = k < 1 ? 0 : k < 3 ? 1 : k < 6 ? 2 : 3;
    jt = k - (it * (it + 1)) / 2;
}
// Buffer descriptors: only the vector and immediate offsets are range-checked
// (loads outside return 0, stores outside are dropped).  Every buffer here is
// uniform across the workgroup; readfirstlane keeps the descriptor scalar.
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
// Transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group, lane
// a+4q names row kbase+q, columns 4a..4a+3 of a row-major tile, and lane i
// receives rows kbase..kbase+3 of column i.
__device__ __forceinline__ bf16x4 tr4(const unsigned char *p) {
    return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)p));
}
template <class T>
__device__ __forceinline__ T lds_ld(const unsigned char *p) { return *reinterpret_cast<const T *>(p); }
template <class T>
__device__ __forceinline__ void lds_st(unsigned char *p, T v) { *reinterpret_cast<T *>(p) = v; }

__device__ __forceinline__ int64_t xcd_chain(int64_t blk, int64_t n) {
    const int64_t x = blk % kXcds, k = blk / kXcds, per = n / kXcds, rem = n % kXcds;
    return x * per + (x < rem ? x : rem) + k;
}

// Per-lane byte offsets, fixed for the whole sequence (pq = this wave's
// 16-row group of p).
template <int N>
struct LaneOffs {
    static constexpr int NT = N / 16, KS = N / 32;
    static constexpr int RB = N * 2;          // bytes per Bm / Cm row
    static constexpr int CPR = N / 8;         // 16-byte chunks per Bm / Cm row
    // At N = 256 the pieces in the second 256 bytes of a row sit exactly 256
    // bytes after those in the first (the swizzles permute chunks within each
    // half), so only the first half's offsets are kept: KSO k-steps of Cm,
    // NTO n-tiles of Bm; the rest add (index / KSO or NTO) * 256.
    static constexpr int KSO = N == 256 ? KS / 2 : KS, NTO = N == 256 ? NT / 2 : NT;
    int xtr;          // X, transposing reads:    + ks*4096 (+512 for rows +4)
    int mm[2];        // Mm, fragment reads (by ks): + it*2048
    int mw;           // Mm, tile writes:         + 16 ti * 128, chunk bytes ^ 32 tj
    int ct[KSO][2];   // Ct, pieces n0 and n1:    + it*(16*RB + ct_pad), chunk bytes ^ csw_tile_bytes(it)
    int bt[NTO];      // Bt, transposing reads:   + ks*32*RB (+4*RB for rows +4)
    int sx;           // x stage writes (state waves):       + k*4096
    int gx;           // x global loads (state waves):       + k*32*H*P*2
    int sb;           // Bm stage writes (output waves):     ^ sb_flip(k), + k*(256/CPR)*RB
    int sc[N / 32];   // Cm stage writes (output waves), by k
    int gb;           // Bm, Cm global loads (output waves): + k*(256/CPR)*G*N*2
    int gd;           // dt loads
    int gy;           // y stores:                + it*16*H*P*2
};

// H: heads of x and y (64 columns each); Hd: heads of dt (0: H).
template <int N>
__device__ __forceinline__ LaneOffs<N> lane_offsets(int tid, int pq, int64_t H, int64_t G, int64_t Hd = 0) {
    using O = LaneOffs<N>;
    const int lane = tid & 63, lrow = lane & 15, lgrp = lane >> 4, qa = lane & 3, qq = (lane & 15) >> 2;
    O o;
    const int r = 8 * lgrp + qq;                  // row (within a k-step) of the transposing reads
    o.xtr = r * 128 + (((2 * pq + (qa >> 1)) ^ xsw(r)) * 16) + (qa & 1) * 8;
    o.mm[0] = lrow * 128 + ((lgrp ^ msw(lrow)) * 16);
    o.mm[1] = lrow * 128 + (((4 + lgrp) ^ msw(lrow)) * 16);
    o.mw = lrow * 128 + (((lgrp >> 1) ^ msw(lrow)) * 16) + (lgrp & 1) * 8;
#pragma unroll
    for (int ks = 0; ks < O::KSO; ++ks)
#pragma unroll
        for (int wh = 0; wh < 2; ++wh) {
            const int n = 32 * ks + 16 * wh + 4 * lgrp;
            o.ct[ks][wh] = lrow * O::RB + (((n >> 3) ^ csw<N>(lrow)) * 16) + (n & 7) * 2;   // tile 0
        }
#pragma unroll
    for (int t = 0; t < O::NTO; ++t) {
        const int col = 16 * t + 4 * qa;
        o.bt[t] = r * O::RB + (((col >> 3) ^ bsw<N>(r)) * 16) + (col & 7) * 2;
    }
    {
        const int u = tid & 255;
        const int j = u >> 3, c = u & 7;
        o.sx = j * 128 + ((c ^ xsw(j)) * 16);   // row j + 32 has the same swizzle
        o.gx = (int)(((int64_t)j * H * kP + 8 * c) * 2);
        const int jb = u / O::CPR, cb = u % O::CPR;
        o.sb = jb * O::RB + ((cb ^ bsw<N>(jb)) * 16);   // rows jb + 256k/CPR: see sb_flip
#pragma unroll
        for (int k = 0; k < N / 32; ++k) {
            const int jk = jb + k * (256 / O::CPR);
            o.sc[k] = jk * O::RB + (jk >> 4) * ct_pad<N> + ((cb ^ csw<N>(jk)) * 16);
        }
        o.gb = (int)(((int64_t)jb * G * N + 8 * cb) * 2);
    }
    o.gd = (int)((int64_t)lane * (Hd ? Hd : H) * 4);
    o.gy = (int)(((int64_t)lrow * H * kP + 16 * pq + 4 * lgrp) * 2);
    return o;
}

// Gram tiles of one 64-token sub-block and (batch, group): G[i][j] = Cm_i . Bm_j,
// the ten causal 16x16 tiles only (the others are never read), bf16.  Storage
// is in matrix-core fragment order so that a wave reads a tile as one
// contiguous 512-byte run: tile k (0..9, see tile_of) holds, for lane
// l = 16*lgrp + lrow, G[16*it + lrow][16*jt + 4*lgrp + 0..3] at elements
// (64*k + l)*4 .. +3.  Called by the NW waves of a workgroup.
template <int N, int NW = 4>
__device__ __forceinline__ void gram_block(const __bf16 *__restrict__ Bm, const __bf16 *__restrict__ Cm,
                                           __bf16 *__restrict__ gram, int64_t L, int64_t G, int64_t nsb,
                                           int64_t sbg, int64_t bg, int tid) {
    const int wave = tid >> 6, lane = tid & 63;
    const int lrow = lane & 15, lgrp = lane >> 4;
    const int64_t b = bg / G, g = bg % G;
    const int64_t t_base = sbg * kSub;
    __bf16 *out = gram + (bg * nsb + sbg) * (int64_t)(kSub * kSub);
    // a wave's tiles k = wave, wave + NW, ...: every operand loaded first, so
    // that all of them are in flight at once, then the products
    constexpr int MT = (10 + NW - 1) / NW;
    bf16x8 ab[MT][N / 32], bc[MT][N / 32];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int k = wave + m * NW;
        if (k < 10) {
            int it, jt;
            tile_of(k, it, jt);
            const int64_t tj = t_base + 16 * jt + lrow, ti = t_base + 16 * it + lrow;
            const __bf16 *brow = Bm + ((b * L + tj) * G + g) * N;
            const __bf16 *crow = Cm + ((b * L + ti) * G + g) * N;
#pragma unroll
            for (int ks = 0; ks < N / 32; ++ks) {
                const int n0 = 32 * ks + 8 * lgrp;
                ab[m][ks] = bf16x8{};
                bc[m][ks] = bf16x8{};
                if (tj < L) ab[m][ks] = *reinterpret_cast<const bf16x8 *>(brow + n0);
                if (ti < L) bc[m][ks] = *reinterpret_cast<const bf16x8 *>(crow + n0);
            }
        }
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int k = wave + m * NW;
        if (k < 10) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < N / 32; ++ks) acc = mfma(ab[m][ks], bc[m][ks], acc);   // rows j, column i
            uint2 pk;
            pk.x = pack2(acc[0], acc[1]);
            pk.y = pack2(acc[2], acc[3]);
            *reinterpret_cast<uint2 *>(out + (k * 64 + lane) * 4) = pk;
        }
    }
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP row shifts and
// row broadcasts.
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

}  // namespace tile
}  // namespace ssd
