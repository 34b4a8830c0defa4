// Chunk scan on gfx950 matrix cores (bf16 operands, fp32 accumulation).
//
// The sequence is cut into blocks ("chunks") of Q tokens, the block
// decomposition of the "Mamba-2" note (section "taking each path half way")
// and of the "Mamba-2 model walkthrough" (sections 6.1-6.2): the diagonal
// blocks are computed in the quadratic, attention-like form and the rest
// through states passed from block to block.  Inside a block, one workgroup
// (4 waves, one per 16-wide slice of the P = 64 head dimension) walks the
// block in sub-blocks of 64 tokens and applies the same decomposition once
// more, carrying the P x N state in matrix-core accumulators:
//
//   per sub-block, with Lambda the in-block inclusive prefix sum of dt*A,
//   s the first token of the sub-block and e its last:
//     G[i][j]    = Cm_i . Bm_j                 (gram kernel, once per group)
//     M[i][j]    = G[i][j] exp(Lambda_i - Lambda_j) dt_j    for j <= i, else 0
//     y_i        = exp(Lambda_i - Lambda_{s-1}) Cm_i . H  +  sum_j M[i][j] x_j
//                  + D x_i
//     H         <- exp(Lambda_e - Lambda_{s-1}) H
//                  + sum_j exp(Lambda_e - Lambda_j) dt_j x_j (outer) Bm_j
//
// Every contraction is a v_mfma_f32_16x16x32_bf16.  Operand layouts are
// chosen so that no accumulator has to pass through LDS: the state is held
// transposed (rows n, columns p), and a 16x16 accumulator tile gives each
// lane four consecutive rows of one column; two such tiles give the eight
// k-values one lane feeds into the next product, with the other operand read
// from LDS in the same (permuted) k order.  The masked decay matrix M goes
// through LDS because all four waves need all of it.
//
// Memory latency is hidden inside the workgroup: the block's x (the only
// input streamed from HBM per head) is loaded into registers when the
// workgroup starts, and the Bm, Cm and G of the next sub-block are loaded
// into registers while the current one computes (Bm, Cm and G are shared by
// all heads of a group and mostly hit in L2).
//
// Two modes share this code, with the state pass (a short kernel over the
// blocks of every (b, h)) between them:
//   kState   the state each block produces from zero (its "chunk state") and
//            its total decay, written to the workspace;
//   kOutput  the outputs of each block from the state entering it (read from
//            the workspace, where the pass kernel put it).
#include "common.h"
#include "tile_ops.h"

namespace ssd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kP = 64;        // head dimension handled by the matrix-core path
constexpr int kSub = 64;      // tokens per sub-block
constexpr int kThreads = 256;

enum Mode { kState = 0, kOutput = 1 };

template <int N, int Q>
struct Smem {
    static constexpr int RS = N + 8;      // row stride (elements) of Cs: +16 bytes
    static constexpr int TS = kSub + 8;   // row stride of [*][64] tiles
    __bf16 Cs[kSub * RS];                 // Cm of the sub-block, [i][n]
    __bf16 BwT[N * TS];                   // weighted Bm, transposed: [n][j] = w_j Bm_j[n]
    __bf16 xT[kP * TS];                   // x transposed: [p][j]
    __bf16 Mm[kSub * TS];                 // masked decay matrix: [i][j]
    float lam[Q];                         // inclusive prefix of dt*A in the block
    float dts[Q];                         // dt in the block (0 past the end)
    float wsub[Q];                        // exp(lam[e] - lam[j]) dt_j, e = end of j's sub-block
    float rdec[Q];                        // exp(lam[i] - lam[s - 1]), s = start of i's sub-block
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

// causal 16x16 tile k (0..9) of a 64x64 block -> (row tile it, column tile jt), jt <= it
__device__ __forceinline__ void tile_of(int k, int &it, int &jt) {
    it = k < 1 ? 0 : k < 3 ? 1 : k < 6 ? 2 : 3;
    jt = k - (it * (it + 1)) / 2;
}

// Gram kernel: one workgroup per (sub-block, batch * group), one wave per
// causal tile (ten), so that every tile's loads are in flight at once; see
// tile::gram_block.  With four waves taking two or three tiles in turn the
// gram launch of the 130M-layer shape took ~2.4 us more per call.
constexpr int kGramThreads = 640;
template <int N>
__global__ __launch_bounds__(kGramThreads) void gram_kernel(const __bf16 *__restrict__ Bm,
                                                            const __bf16 *__restrict__ Cm,
                                                            __bf16 *__restrict__ gram, int64_t L,
                                                            int64_t G, int64_t nsb) {
    tile::gram_block<N, kGramThreads / 64>(Bm, Cm, gram, L, G, nsb, blockIdx.x, blockIdx.y, threadIdx.x);
}

// ---------------------------------------------------------------------------
// Per-thread registers holding one sub-block's Bm, Cm and G until staged.
// ---------------------------------------------------------------------------
template <int N>
struct SubRegs {
    uint4 b[2 * (N / 64)];   // Bm: N/64 units of (token pair, 8 columns)
    uint4 c[N / 32];         // Cm: row pieces of 8 columns
    uint2 g[3];              // G: this wave's causal tiles, 4 values per lane
};

struct Ctx {
    const __bf16 *x, *Bm, *Cm, *gram;
    int64_t b, h, g, t0, L, H, G, nsb;
    int q;
};

template <int N>
__device__ __forceinline__ void load_sub(SubRegs<N> &r, const Ctx &cx, int s, bool with_b, bool with_cg) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int lrow = lane & 15, lgrp = lane >> 4;
#pragma unroll
    for (int k = 0; k < N / 64 && with_b; ++k) {
        const int u = tid + k * kThreads;
        const int cg = u % (N / 8), tp = u / (N / 8);
        const int j0 = s + 2 * tp;
        const __bf16 *p0 = cx.Bm + (((cx.b * cx.L + cx.t0 + j0) * cx.G + cx.g) * N + 8 * cg);
        r.b[2 * k] = j0 < cx.q ? *reinterpret_cast<const uint4 *>(p0) : uint4{0, 0, 0, 0};
        r.b[2 * k + 1] = j0 + 1 < cx.q ? *reinterpret_cast<const uint4 *>(p0 + cx.G * N) : uint4{0, 0, 0, 0};
    }
    if (with_cg) {
#pragma unroll
        for (int k = 0; k < N / 32; ++k) {
            const int u = tid + k * kThreads;
            const int j = u / (N / 8), cg = u % (N / 8);
            r.c[k] = s + j < cx.q
                         ? *reinterpret_cast<const uint4 *>(cx.Cm + (((cx.b * cx.L + cx.t0 + s + j) * cx.G + cx.g) * N + 8 * cg))
                         : uint4{0, 0, 0, 0};
        }
        const int64_t sbg = (cx.t0 + s) / kSub;
        const __bf16 *gb = cx.gram + ((cx.b * cx.G + cx.g) * cx.nsb + sbg) * (int64_t)(kSub * kSub);
#pragma unroll
        for (int m = 0; m < 3; ++m) {
            const int k = wave + 4 * m;
            if (k < 10) r.g[m] = *reinterpret_cast<const uint2 *>(gb + (k * 64 + lane) * 4);
        }
    }
}

// x of the whole block into registers: per sub-block, tokens 2tp, 2tp+1 and
// columns 8pg..8pg+7 (pg = tid & 7, tp = tid >> 3: eight lanes cover one 128-byte row).
template <int NSB>
__device__ __forceinline__ void load_x(uint4 (&xr)[2 * NSB], const Ctx &cx) {
    const int tid = threadIdx.x, pg = tid & 7, tp = tid >> 3;
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb) {
        const int j0 = sb * kSub + 2 * tp;
        const __bf16 *p0 = cx.x + (((cx.b * cx.L + cx.t0 + j0) * cx.H + cx.h) * kP + 8 * pg);
        xr[2 * sb] = j0 < cx.q ? *reinterpret_cast<const uint4 *>(p0) : uint4{0, 0, 0, 0};
        xr[2 * sb + 1] = j0 + 1 < cx.q ? *reinterpret_cast<const uint4 *>(p0 + cx.H * kP) : uint4{0, 0, 0, 0};
    }
}

// Stage sub-block s: xT always; BwT when WITH_B; Cs and the masked matrix Mm when FULL.
template <int N, int Q, bool WITH_B, bool FULL>
__device__ __forceinline__ void stage(Smem<N, Q> &sm, const SubRegs<N> &r, uint4 x0, uint4 x1, int s) {
    using S = Smem<N, Q>;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int lrow = lane & 15, lgrp = lane >> 4;
    {
        const int pg = tid & 7, tp = tid >> 3, j0 = 2 * tp;
        const uint32_t a0[4] = {x0.x, x0.y, x0.z, x0.w}, a1[4] = {x1.x, x1.y, x1.z, x1.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            *reinterpret_cast<uint32_t *>(&sm.xT[(8 * pg + 2 * k) * S::TS + j0]) = (a0[k] & 0xffffu) | (a1[k] << 16);
            *reinterpret_cast<uint32_t *>(&sm.xT[(8 * pg + 2 * k + 1) * S::TS + j0]) = (a0[k] >> 16) | (a1[k] & 0xffff0000u);
        }
    }
#pragma unroll
    for (int k = 0; k < N / 64 && WITH_B; ++k) {
        const int u = tid + k * kThreads;
        const int cg = u % (N / 8), tp = u / (N / 8), j0 = 2 * tp;
        const float w0 = sm.wsub[s + j0], w1 = sm.wsub[s + j0 + 1];
        const uint4 v0 = r.b[2 * k], v1 = r.b[2 * k + 1];
        const uint32_t a0[4] = {v0.x, v0.y, v0.z, v0.w}, a1[4] = {v1.x, v1.y, v1.z, v1.w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            *reinterpret_cast<uint32_t *>(&sm.BwT[(8 * cg + 2 * m) * S::TS + j0]) =
                pack2(w0 * lo_bf16(a0[m]), w1 * lo_bf16(a1[m]));
            *reinterpret_cast<uint32_t *>(&sm.BwT[(8 * cg + 2 * m + 1) * S::TS + j0]) =
                pack2(w0 * hi_bf16(a0[m]), w1 * hi_bf16(a1[m]));
        }
    }
    if (FULL) {
#pragma unroll
        for (int k = 0; k < N / 32; ++k) {
            const int u = tid + k * kThreads;
            const int j = u / (N / 8), cg = u % (N / 8);
            *reinterpret_cast<uint4 *>(&sm.Cs[j * S::RS + 8 * cg]) = r.c[k];
        }
        // masked decay matrix from this wave's G tiles
#pragma unroll
        for (int m = 0; m < 3; ++m) {
            const int k = wave + 4 * m;
            if (k < 10) {
                int it, jt;
                tile_of(k, it, jt);
                const int i = 16 * it + lrow;
                const float li = sm.lam[s + i];
                const uint32_t gw[2] = {r.g[m].x, r.g[m].y};
                float mv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int j = 16 * jt + 4 * lgrp + e;
                    const float gv = (e & 1) ? hi_bf16(gw[e >> 1]) : lo_bf16(gw[e >> 1]);
                    mv[e] = j <= i ? gv * __expf(li - sm.lam[s + j]) * sm.dts[s + j] : 0.f;
                }
                uint2 pk;
                pk.x = pack2(mv[0], mv[1]);
                pk.y = pack2(mv[2], mv[3]);
                *reinterpret_cast<uint2 *>(&sm.Mm[i * S::TS + 16 * jt + 4 * lgrp]) = pk;
            }
        }
        if (wave >= 2) {
            // tiles above the diagonal that the apply step reads: (0,1), (2,3)
            const int it = wave == 2 ? 0 : 2;
            *reinterpret_cast<uint2 *>(&sm.Mm[(16 * it + lrow) * S::TS + 16 * (it + 1) + 4 * lgrp]) =
                uint2{0u, 0u};
        }
    }
}

// H (transposed state accumulators of this wave) += BwT . xT^T over the sub-block.
template <int N, int Q>
__device__ __forceinline__ void state_update(f32x4 (&Hacc)[N / 16], const Smem<N, Q> &sm,
                                             int wave, int lrow, int lgrp) {
    using S = Smem<N, Q>;
#pragma unroll
    for (int ks = 0; ks < kSub / 32; ++ks) {
        const int j0 = 32 * ks + 8 * lgrp;
        const bf16x8 bx = *reinterpret_cast<const bf16x8 *>(&sm.xT[(16 * wave + lrow) * S::TS + j0]);
#pragma unroll
        for (int t = 0; t < N / 16; ++t) {
            const bf16x8 ba = *reinterpret_cast<const bf16x8 *>(&sm.BwT[(16 * t + lrow) * S::TS + j0]);
            Hacc[t] = mfma(ba, bx, Hacc[t]);
        }
    }
}

template <int N>
__device__ __forceinline__ void scale_state(f32x4 (&Hacc)[N / 16], float f) {
#pragma unroll
    for (int t = 0; t < N / 16; ++t) Hacc[t] *= f;
}

// A state of one (b, h) is [P][N] float32, row-major.  In the accumulator
// layout a lane holds p = 16*wave + lrow, n = 16t + 4*lgrp + 0..3.
template <int N>
__device__ __forceinline__ void load_state(f32x4 (&Hacc)[N / 16], const float *src, int wave,
                                           int lrow, int lgrp) {
    const float *row = src + (int64_t)(16 * wave + lrow) * N + 4 * lgrp;
#pragma unroll
    for (int t = 0; t < N / 16; ++t) Hacc[t] = *reinterpret_cast<const f32x4 *>(row + 16 * t);
}

template <int N>
__device__ __forceinline__ void store_state(const f32x4 (&Hacc)[N / 16], float *dst, int wave,
                                            int lrow, int lgrp) {
    float *row = dst + (int64_t)(16 * wave + lrow) * N + 4 * lgrp;
#pragma unroll
    for (int t = 0; t < N / 16; ++t) *reinterpret_cast<f32x4 *>(row + 16 * t) = Hacc[t];
}

template <int N, int Q, int MODE>
__global__ __launch_bounds__(kThreads, N <= 128 ? 2 : 1) void scan_mfma(
    const __bf16 *__restrict__ x, const float *__restrict__ dt, const float *__restrict__ A,
    const __bf16 *__restrict__ Bm, const __bf16 *__restrict__ Cm, const float *__restrict__ D,
    __bf16 *__restrict__ y, float *states, float *decay, const __bf16 *gram,
    int64_t L, int64_t H, int64_t G) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    using S = Smem<N, Q>;
    S &sm = *reinterpret_cast<S *>(smem_raw);
    constexpr int NT = N / 16;
    constexpr int NSB = Q / kSub;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int lrow = lane & 15, lgrp = lane >> 4;
    const int nc = (int)((L + Q - 1) / Q);
    const int64_t c = blockIdx.x, chain = blockIdx.y;
    Ctx cx;
    cx.x = x; cx.Bm = Bm; cx.Cm = Cm; cx.gram = gram;
    cx.b = chain / H; cx.h = chain % H; cx.g = cx.h / (H / G);
    cx.t0 = c * Q; cx.L = L; cx.H = H; cx.G = G; cx.nsb = (int64_t)nc * (Q / kSub);
    cx.q = (int)((L - cx.t0) < Q ? (L - cx.t0) : Q);
    const int q = cx.q;

    // issue every load the block starts with: dt, the block's x, the first sub-block
    const float dtv = tid < q ? dt[(cx.b * L + cx.t0 + tid) * H + cx.h] : 0.f;
    uint4 xr[2 * NSB];
    load_x<NSB>(xr, cx);
    SubRegs<N> r;
    load_sub<N>(r, cx, 0, true, MODE == kOutput);

    // in-block prefix sums of dt*A (first wave), then per-token weights and decays
    if (tid < Q) sm.dts[tid] = dtv;
    __syncthreads();
    if (wave == 0) {
        const float Ah = A[cx.h];
        float carry = 0.f;
#pragma unroll
        for (int base = 0; base < Q; base += 64) {
            float v = sm.dts[base + lane] * Ah;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float o = __shfl_up(v, off);
                if (lane >= off) v += o;
            }
            v += carry;
            sm.lam[base + lane] = v;
            carry = __shfl(v, 63);
        }
    }
    __syncthreads();
    if (tid < Q) {
        const int s0 = tid & ~(kSub - 1);
        const float lj = sm.lam[tid];
        const float before = s0 == 0 ? 0.f : sm.lam[s0 - 1];
        sm.wsub[tid] = __expf(sm.lam[s0 + kSub - 1] - lj) * sm.dts[tid];
        sm.rdec[tid] = __expf(lj - before);
    }
    __syncthreads();

    f32x4 Hacc[NT];
    const int64_t state_off = ((cx.b * nc + c) * H + cx.h) * (int64_t)(kP * N);

    if (MODE == kState) {
        // the block's own state, from zero
#pragma unroll
        for (int t = 0; t < NT; ++t) Hacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb) {
            const int s = sb * kSub;
            if (s >= q) break;
            stage<N, Q, true, false>(sm, r, xr[2 * sb], xr[2 * sb + 1], s);
            if (sb + 1 < NSB && s + kSub < q) load_sub<N>(r, cx, s + kSub, true, false);
            __syncthreads();
            const float before = s == 0 ? 0.f : sm.lam[s - 1];
            scale_state<N>(Hacc, __expf(sm.lam[s + kSub - 1] - before));
            state_update<N, Q>(Hacc, sm, wave, lrow, lgrp);
            __syncthreads();
        }
        store_state<N>(Hacc, states + state_off, wave, lrow, lgrp);
        if (tid == 0) decay[chain * nc + c] = __expf(sm.lam[Q - 1]);
        return;
    }
    load_state<N>(Hacc, states + state_off, wave, lrow, lgrp);

    // outputs of the block from the entering state
    const float Dh = D[cx.h];
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb) {
        const int s = sb * kSub;
        if (s >= q) break;
        stage<N, Q, true, true>(sm, r, xr[2 * sb], xr[2 * sb + 1], s);
        if (sb + 1 < NSB && s + kSub < q) load_sub<N>(r, cx, s + kSub, true, true);
        __syncthreads();

        // inter-block part: Y^T[p][i] = sum_n H[p][n] Cm_i[n], with H the state
        // entering the sub-block, then the row decay exp(lam_i - lam_{s-1})
        f32x4 Y[4];
#pragma unroll
        for (int it = 0; it < 4; ++it) Y[it] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < N / 32; ++ks) {
            const f32x4 h0 = Hacc[2 * ks], h1 = Hacc[2 * ks + 1];
            bf16x8 ah;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ah[e] = (__bf16)h0[e];
                ah[4 + e] = (__bf16)h1[e];
            }
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const __bf16 *crow = &sm.Cs[(16 * it + lrow) * S::RS + 32 * ks + 4 * lgrp];
                const bf16x4 c0 = *reinterpret_cast<const bf16x4 *>(crow);
                const bf16x4 c1 = *reinterpret_cast<const bf16x4 *>(crow + 16);
                const bf16x8 bc = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
                Y[it] = mfma(ah, bc, Y[it]);
            }
        }
#pragma unroll
        for (int it = 0; it < 4; ++it) Y[it] *= sm.rdec[s + 16 * it + lrow];

        // intra-block part: Y^T[p][i] += sum_j x_j[p] M[i][j] (causal k-steps only)
#pragma unroll
        for (int it = 0; it < 4; ++it) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                if (ks == 1 && it < 2) continue;
                const int j0 = 32 * ks + 8 * lgrp;
                const bf16x8 ax = *reinterpret_cast<const bf16x8 *>(&sm.xT[(16 * wave + lrow) * S::TS + j0]);
                const bf16x8 bm = *reinterpret_cast<const bf16x8 *>(&sm.Mm[(16 * it + lrow) * S::TS + j0]);
                Y[it] = mfma(ax, bm, Y[it]);
            }
        }
        // skip term and store: lane holds p = 16*wave + 4*lgrp + e, token i = 16*it + lrow
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int i = 16 * it + lrow;
            if (s + i < q) {
                const int p0 = 16 * wave + 4 * lgrp;
                float o[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    o[e] = Y[it][e] + Dh * (float)sm.xT[(p0 + e) * S::TS + i];
                uint2 pk;
                pk.x = pack2(o[0], o[1]);
                pk.y = pack2(o[2], o[3]);
                *reinterpret_cast<uint2 *>(y + (((cx.b * L + cx.t0 + s + i) * H + cx.h) * kP + p0)) = pk;
            }
        }
        if (sb + 1 < NSB && s + kSub < q) {
            const float before = s == 0 ? 0.f : sm.lam[s - 1];
            scale_state<N>(Hacc, __expf(sm.lam[s + kSub - 1] - before));
            state_update<N, Q>(Hacc, sm, wave, lrow, lgrp);
        }
        __syncthreads();
    }
}

// The state pass of the staged form: the state entering every block,
// H_{c+1} = decay_c H_c + S_c, written over the block's own state S_c in place,
// and the final state.  Sequential over the blocks, parallel over (b, h) and
// the P*N elements: one thread per four elements (16-byte accesses), the four
// block states of the next group of four blocks loaded before the current four
// are written, so that loads overlap the chain instead of waiting one block at
// a time.
__global__ __launch_bounds__(256) void state_pass_kernel(float4 *__restrict__ states, const float *__restrict__ decay,
                                                         const float4 *init, float4 *final_state, int64_t H,
                                                         int64_t PN4, int nc) {
    const int64_t bh = blockIdx.y;
    const int64_t b = bh / H, h = bh % H;
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= PN4) return;
    float4 s = init ? init[bh * PN4 + e] : float4{0.f, 0.f, 0.f, 0.f};
    const float *dk = decay + bh * nc;
    auto at = [&](int c) { return states + ((b * nc + c) * H + h) * PN4 + e; };
    int c = 0;
    for (; c + 4 <= nc; c += 4) {
        float4 loc[4];
        float dd[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            loc[j] = *at(c + j);
            dd[j] = dk[c + j];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            *at(c + j) = s;                           // state entering block c + j
            s = float4{dd[j] * s.x + loc[j].x, dd[j] * s.y + loc[j].y, dd[j] * s.z + loc[j].z,
                       dd[j] * s.w + loc[j].w};
        }
    }
    for (; c < nc; ++c) {
        const float4 loc = *at(c);
        const float d = dk[c];
        *at(c) = s;
        s = float4{d * s.x + loc.x, d * s.y + loc.y, d * s.z + loc.z, d * s.w + loc.w};
    }
    if (final_state) final_state[bh * PN4 + e] = s;   // the same thread read init[e]: aliasing is safe
}

template <int N, int Q, int MODE>
hipError_t launch_mode(const ScanArgs &a, const Workspace &ws, dim3 grid) {
    const size_t smem = sizeof(Smem<N, Q>);
    auto kern = scan_mfma<N, Q, MODE>;
    static std::atomic<bool> configured[kMaxDevices] = {};
    const hipError_t e = allow_lds((const void *)kern, smem, configured);
    if (e != hipSuccess) return e;
    kern<<<grid, kThreads, smem, a.stream>>>(
        (const __bf16 *)a.x, a.dt, a.A, (const __bf16 *)a.Bm, (const __bf16 *)a.Cm, a.D,
        (__bf16 *)a.y, ws.states, ws.decay, (const __bf16 *)ws.gram, a.L, a.H, a.G);
    return hipGetLastError();
}

template <int N, int Q>
hipError_t run(const ScanArgs &a, const Workspace &ws) {
    const int nc = (int)((a.L + Q - 1) / Q);
    const int64_t nsb = (int64_t)nc * (Q / kSub);
    gram_kernel<N><<<dim3((unsigned)nsb, (unsigned)(a.B * a.G)), kGramThreads, 0, a.stream>>>(
        (const __bf16 *)a.Bm, (const __bf16 *)a.Cm, (__bf16 *)ws.gram, a.L, a.G, nsb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_mode<N, Q, kState>(a, ws, dim3((unsigned)nc, (unsigned)(a.B * a.H)));
    if (e != hipSuccess) return e;
    e = launch_state_pass(ws.states, ws.decay, a.init, a.final_state, a.B, a.H, kP * N, nc, a.stream);
    if (e != hipSuccess) return e;
    return launch_mode<N, Q, kOutput>(a, ws, dim3((unsigned)nc, (unsigned)(a.B * a.H)));
}

template <int N>
hipError_t run_q(const ScanArgs &a, const Workspace &ws) {
    switch (a.Q) {
        case 64: return run<N, 64>(a, ws);
        case 128: return run<N, 128>(a, ws);
        case 256: return run<N, 256>(a, ws);
        default: return hipErrorInvalidValue;
    }
}

hipError_t dispatch(const ScanArgs &a, const Workspace &ws) {
    switch (a.N) {
        case 64: return run_q<64>(a, ws);
        case 128: return run_q<128>(a, ws);
        case 256: return run_q<256>(a, ws);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool mfma_supported(int64_t P, int64_t N, int64_t Q) {
    return P == kP && (N == 64 || N == 128 || N == 256) && (Q == 64 || Q == 128 || Q == 256);
}

size_t gram_bytes(int64_t B, int64_t L, int64_t G, int64_t Q) {
    const int64_t nc = (L + Q - 1) / Q;
    return (size_t)(B * G * nc * Q * kSub) * sizeof(__bf16);
}

hipError_t launch_state_pass(float *states, const float *decay, const float *init, float *final_state,
                             int64_t B, int64_t H, int64_t PN, int nc, hipStream_t stream) {
    const int64_t PN4 = PN / 4;   // P*N is a multiple of 4 (P, N >= 16)
    const dim3 grid((unsigned)((PN4 + 255) / 256), (unsigned)(B * H));
    state_pass_kernel<<<grid, 256, 0, stream>>>(reinterpret_cast<float4 *>(states), decay,
                                                reinterpret_cast<const float4 *>(init),
                                                reinterpret_cast<float4 *>(final_state), H, PN4, nc);
    return hipGetLastError();
}

hipError_t launch_staged_scan(const ScanArgs &a, const Workspace &ws) { return dispatch(a, ws); }

hipError_t launch_gram(const ScanArgs &a, const Workspace &ws, int64_t nsb) {
    switch (a.N) {
        case 64:
            gram_kernel<64><<<dim3((unsigned)nsb, (unsigned)(a.B * a.G)), kGramThreads, 0, a.stream>>>(
                (const __bf16 *)a.Bm, (const __bf16 *)a.Cm, (__bf16 *)ws.gram, a.L, a.G, nsb);
            break;
        case 128:
            gram_kernel<128><<<dim3((unsigned)nsb, (unsigned)(a.B * a.G)), kGramThreads, 0, a.stream>>>(
                (const __bf16 *)a.Bm, (const __bf16 *)a.Cm, (__bf16 *)ws.gram, a.L, a.G, nsb);
            break;
        case 256:
            gram_kernel<256><<<dim3((unsigned)nsb, (unsigned)(a.B * a.G)), kGramThreads, 0, a.stream>>>(
                (const __bf16 *)a.Bm, (const __bf16 *)a.Cm, (__bf16 *)ws.gram, a.L, a.G, nsb);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace ssd
