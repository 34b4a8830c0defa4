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
//     G^T[j][i]  = Bm_j . Cm_i                        (causal 16x16 tiles only)
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
// Three modes share this code:
//   kState   the state each block produces from zero (its "chunk state") and
//            its total decay, written to the workspace;
//   kOutput  the outputs of each block from the state entering it (read from
//            the workspace, where the pass kernel put it);
//   kFused   both in one launch: a block computes its own state, takes the
//            state entering it from its predecessor's workgroup, hands the
//            state leaving it to its successor, then computes its outputs.
//            Workgroups take tickets from a counter in block-major order, so
//            the predecessor of ticket t holds ticket t - (B*H) and has
//            already started: waiting on it always ends.  States are handed
//            over through a two-slot ring per (b, h) and a flag counting the
//            blocks published; both stay in cache.
#include "common.h"

namespace ssd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kP = 64;        // head dimension handled by the matrix-core path
constexpr int kSub = 64;      // tokens per sub-block
constexpr int kThreads = 256;
constexpr unsigned kSpinLimit = 1u << 22;   // hand-off polls before giving up

enum Mode { kState = 0, kOutput = 1, kFused = 2 };

template <int N, int Q>
struct Smem {
    static constexpr int RS = N + 8;      // row stride (elements) of [64][N] tiles: +16 bytes
    static constexpr int TS = kSub + 8;   // row stride of [*][64] tiles
    __bf16 Cs[kSub * RS];                 // Cm of the sub-block, [i][n]
    __bf16 Bs[kSub * RS];                 // Bm of the sub-block, [j][n]
    __bf16 BwT[N * TS];                   // weighted Bm, transposed: [n][j] = w_j Bm_j[n]
    __bf16 xT[kP * TS];                   // x transposed: [p][j]
    __bf16 Mm[kSub * TS];                 // masked decay matrix: [i][j]
    float lam[Q];                         // inclusive prefix of dt*A in the block
    float dts[Q];                         // dt in the block (0 past the end)
    unsigned ticket;
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

struct Dims {
    int64_t L, H, G;
    int nc;
};

// Stage one sub-block into LDS.  Tokens past the valid count q are zeros.
//   xT[p][j]  always;  BwT[n][j] = w_j Bm_j[n] always (w_j = exp(lam_e - lam_j) dt_j);
//   Cs, Bs (row copies) only when FULL.
template <int N, int Q, bool FULL>
__device__ __forceinline__ void stage_sub_block(Smem<N, Q> &sm, const __bf16 *__restrict__ x,
                                                const __bf16 *__restrict__ Bm,
                                                const __bf16 *__restrict__ Cm, const Dims &d,
                                                int64_t b, int64_t h, int64_t g, int64_t t0,
                                                int s, int q) {
    using S = Smem<N, Q>;
    const int tid = threadIdx.x;
    const int e = s + kSub - 1;
    const float lam_e = sm.lam[e];
    // x: thread -> token pair tp (tokens 2tp, 2tp+1 of the sub-block), 8 columns 8pg..8pg+7
    {
        const int tp = tid & 31, pg = tid >> 5;
        const int j0 = 2 * tp;
        uint4 v0 = {0, 0, 0, 0}, v1 = {0, 0, 0, 0};
        if (s + j0 < q)
            v0 = *reinterpret_cast<const uint4 *>(x + ((((int64_t)b * d.L + t0 + s + j0) * d.H + h) * kP + 8 * pg));
        if (s + j0 + 1 < q)
            v1 = *reinterpret_cast<const uint4 *>(x + ((((int64_t)b * d.L + t0 + s + j0 + 1) * d.H + h) * kP + 8 * pg));
        const uint32_t a0[4] = {v0.x, v0.y, v0.z, v0.w}, a1[4] = {v1.x, v1.y, v1.z, v1.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t lo = (a0[k] & 0xffffu) | (a1[k] << 16);          // column 2k
            const uint32_t hi = (a0[k] >> 16) | (a1[k] & 0xffff0000u);      // column 2k+1
            *reinterpret_cast<uint32_t *>(&sm.xT[(8 * pg + 2 * k) * S::TS + j0]) = lo;
            *reinterpret_cast<uint32_t *>(&sm.xT[(8 * pg + 2 * k + 1) * S::TS + j0]) = hi;
        }
    }
    // Bm: units of (token pair, 8 columns); N/8 column groups x 32 pairs
    constexpr int kGroups = N / 8;
    constexpr int kUnits = kGroups * 32;
#pragma unroll
    for (int u = tid; u < kUnits; u += kThreads) {
        const int tp = u & 31, cg = u >> 5;
        const int j0 = 2 * tp;
        uint4 v0 = {0, 0, 0, 0}, v1 = {0, 0, 0, 0};
        if (s + j0 < q)
            v0 = *reinterpret_cast<const uint4 *>(Bm + ((((int64_t)b * d.L + t0 + s + j0) * d.G + g) * N + 8 * cg));
        if (s + j0 + 1 < q)
            v1 = *reinterpret_cast<const uint4 *>(Bm + ((((int64_t)b * d.L + t0 + s + j0 + 1) * d.G + g) * N + 8 * cg));
        if (FULL) {
            *reinterpret_cast<uint4 *>(&sm.Bs[j0 * S::RS + 8 * cg]) = v0;
            *reinterpret_cast<uint4 *>(&sm.Bs[(j0 + 1) * S::RS + 8 * cg]) = v1;
        }
        const float w0 = __expf(lam_e - sm.lam[s + j0]) * sm.dts[s + j0];
        const float w1 = __expf(lam_e - sm.lam[s + j0 + 1]) * sm.dts[s + j0 + 1];
        const uint32_t a0[4] = {v0.x, v0.y, v0.z, v0.w}, a1[4] = {v1.x, v1.y, v1.z, v1.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            *reinterpret_cast<uint32_t *>(&sm.BwT[(8 * cg + 2 * k) * S::TS + j0]) =
                pack2(w0 * lo_bf16(a0[k]), w1 * lo_bf16(a1[k]));
            *reinterpret_cast<uint32_t *>(&sm.BwT[(8 * cg + 2 * k + 1) * S::TS + j0]) =
                pack2(w0 * hi_bf16(a0[k]), w1 * hi_bf16(a1[k]));
        }
    }
    if (FULL) {
        // Cm: plain row copies, 16 bytes per thread per step
        for (int u = tid; u < kSub * kGroups; u += kThreads) {
            const int j = u / kGroups, cg = u % kGroups;
            uint4 v = {0, 0, 0, 0};
            if (s + j < q)
                v = *reinterpret_cast<const uint4 *>(Cm + ((((int64_t)b * d.L + t0 + s + j) * d.G + g) * N + 8 * cg));
            *reinterpret_cast<uint4 *>(&sm.Cs[j * S::RS + 8 * cg]) = v;
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

// Load / store the state of one (b, h) ([P][N] float32, row-major) in the
// accumulator layout: lane holds p = 16*wave + lrow, n = 16t + 4*lgrp + 0..3.
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
__global__ __launch_bounds__(kThreads) void scan_mfma(
    const __bf16 *__restrict__ x, const float *__restrict__ dt, const float *__restrict__ A,
    const __bf16 *__restrict__ Bm, const __bf16 *__restrict__ Cm, const float *__restrict__ D,
    const float *init, __bf16 *__restrict__ y, float *final_state, float *states,
    float *decay, unsigned *flags, unsigned *counters, float *ring, int64_t Bsz, int64_t L,
    int64_t H, int64_t G) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    using S = Smem<N, Q>;
    S &sm = *reinterpret_cast<S *>(smem_raw);
    constexpr int NT = N / 16;
    constexpr int NSB = Q / kSub;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int lrow = lane & 15, lgrp = lane >> 4;
    const int64_t nchains = Bsz * H;
    const int nc = (int)((L + Q - 1) / Q);

    int64_t c, chain;
    if (MODE == kFused) {
        if (tid == 0) sm.ticket = atomicAdd(&counters[0], 1u);
        __syncthreads();
        const int64_t t = sm.ticket;
        if (t >= nchains * nc) {
            // counters were not zero at launch (workspace not zero-filled):
            // record it and do nothing; no index below is ever formed from t
            if (tid == 0) atomicOr(&counters[2], 2u);
            return;
        }
        c = t / nchains;
        chain = t % nchains;
    } else {
        c = blockIdx.x;
        chain = blockIdx.y;
    }
    const int64_t b = chain / H, h = chain % H, g = h / (H / G);
    const int64_t t0 = c * Q;
    const int q = (int)((L - t0) < Q ? (L - t0) : Q);
    const Dims d{L, H, G, nc};

    block_prefix(dt + (b * L + t0) * H + h, H, q, Q, A[h], sm.lam, sm.dts);

    f32x4 Hacc[NT];
    const int64_t state_off = ((b * nc + c) * H + h) * (int64_t)(kP * N);

    if (MODE == kState || MODE == kFused) {
        // the block's own state, from zero
#pragma unroll
        for (int t = 0; t < NT; ++t) Hacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int sb = 0; sb < NSB; ++sb) {
            const int s = sb * kSub;
            if (s >= q) break;
            stage_sub_block<N, Q, false>(sm, x, Bm, Cm, d, b, h, g, t0, s, q);
            __syncthreads();
            const float before = s == 0 ? 0.f : sm.lam[s - 1];
            scale_state<N>(Hacc, __expf(sm.lam[s + kSub - 1] - before));
            state_update<N, Q>(Hacc, sm, wave, lrow, lgrp);
            __syncthreads();
        }
        const float gamma = __expf(sm.lam[Q - 1]);
        if (MODE == kState) {
            store_state<N>(Hacc, states + state_off, wave, lrow, lgrp);
            if (tid == 0) decay[chain * nc + c] = gamma;
            return;
        }
        // take the entering state H_c, publish H_{c+1} = gamma H_c + S_c
        f32x4 Hin[NT];
        if (c == 0) {
            if (init) {
                load_state<N>(Hin, init + chain * (int64_t)(kP * N), wave, lrow, lgrp);
            } else {
#pragma unroll
                for (int t = 0; t < NT; ++t) Hin[t] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        } else {
            if (tid == 0) {
                unsigned spins = 0;
                while (__hip_atomic_load(&flags[chain], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) <
                       (unsigned)c) {
                    __builtin_amdgcn_s_sleep(2);
                    if (++spins > kSpinLimit) {       // never expected: record and go on
                        atomicOr(&counters[2], 1u);
                        break;
                    }
                }
            }
            __syncthreads();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            load_state<N>(Hin, ring + (chain * 2 + (c & 1)) * (int64_t)(kP * N), wave, lrow, lgrp);
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) Hacc[t] = gamma * Hin[t] + Hacc[t];
        if (c + 1 < nc) {
            store_state<N>(Hacc, ring + (chain * 2 + ((c + 1) & 1)) * (int64_t)(kP * N), wave, lrow, lgrp);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            __syncthreads();
            if (tid == 0)
                __hip_atomic_store(&flags[chain], (unsigned)(c + 1), __ATOMIC_RELEASE,
                                   __HIP_MEMORY_SCOPE_AGENT);
        } else {
            if (final_state) store_state<N>(Hacc, final_state + chain * (int64_t)(kP * N), wave, lrow, lgrp);
            if (tid == 0) flags[chain] = 0u;      // last user of this chain's flag
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) Hacc[t] = Hin[t];
    } else {
        load_state<N>(Hacc, states + state_off, wave, lrow, lgrp);
    }

    // outputs of the block from the entering state
    const float Dh = D[h];
    for (int sb = 0; sb < NSB; ++sb) {
        const int s = sb * kSub;
        if (s >= q) break;
        stage_sub_block<N, Q, true>(sm, x, Bm, Cm, d, b, h, g, t0, s, q);
        __syncthreads();
        const float before = s == 0 ? 0.f : sm.lam[s - 1];

        // masked decay matrix: causal 16x16 tiles (it >= jt), 10 of them, round-robin over waves
        for (int k = wave; k < 10; k += 4) {
            const int it = k < 1 ? 0 : k < 3 ? 1 : k < 6 ? 2 : 3;
            const int jt = k - (it * (it + 1)) / 2;
            f32x4 gacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < N / 32; ++ks) {
                const int n0 = 32 * ks + 8 * lgrp;
                const bf16x8 ab = *reinterpret_cast<const bf16x8 *>(&sm.Bs[(16 * jt + lrow) * S::RS + n0]);
                const bf16x8 bc = *reinterpret_cast<const bf16x8 *>(&sm.Cs[(16 * it + lrow) * S::RS + n0]);
                gacc = mfma(ab, bc, gacc);
            }
            const int i = 16 * it + lrow;                 // column of G^T: output token
            const float li = sm.lam[s + i];
            float m[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = 16 * jt + 4 * lgrp + r;     // row of G^T: input token
                m[r] = j <= i ? gacc[r] * __expf(li - sm.lam[s + j]) * sm.dts[s + j] : 0.f;
            }
            uint2 pk;
            pk.x = pack2(m[0], m[1]);
            pk.y = pack2(m[2], m[3]);
            *reinterpret_cast<uint2 *>(&sm.Mm[i * S::TS + 16 * jt + 4 * lgrp]) = pk;
        }
        if (wave >= 2) {
            // zero tiles above the diagonal that the apply step reads: (0,1), (2,3)
            const int it = wave == 2 ? 0 : 2;
            *reinterpret_cast<uint2 *>(&sm.Mm[(16 * it + lrow) * S::TS + 16 * (it + 1) + 4 * lgrp]) =
                uint2{0u, 0u};
        }

        // inter-block part: Y^T[p][i] = sum_n H[p][n] Cm_i[n], then the row decay
        f32x4 Y[4];
#pragma unroll
        for (int it = 0; it < 4; ++it) Y[it] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < N / 32; ++ks) {
            bf16x8 ah;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                ah[r] = (__bf16)Hacc[2 * ks][r];
                ah[4 + r] = (__bf16)Hacc[2 * ks + 1][r];
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
        for (int it = 0; it < 4; ++it) Y[it] *= __expf(sm.lam[s + 16 * it + lrow] - before);
        __syncthreads();   // Mm complete

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
        // skip term and store: lane holds p = 16*wave + 4*lgrp + r, token i = 16*it + lrow
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int i = 16 * it + lrow;
            if (s + i < q) {
                const int p0 = 16 * wave + 4 * lgrp;
                float o[4];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    o[r] = Y[it][r] + Dh * (float)sm.xT[(p0 + r) * S::TS + i];
                uint2 pk;
                pk.x = pack2(o[0], o[1]);
                pk.y = pack2(o[2], o[3]);
                *reinterpret_cast<uint2 *>(y + (((b * L + t0 + s + i) * H + h) * kP + p0)) = pk;
            }
        }
        if (sb + 1 < NSB && s + kSub < q) {
            scale_state<N>(Hacc, __expf(sm.lam[s + kSub - 1] - before));
            state_update<N, Q>(Hacc, sm, wave, lrow, lgrp);
        }
        __syncthreads();
    }

    if (MODE == kFused && tid == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        const unsigned done = atomicAdd(&counters[1], 1u);
        if (done + 1 == (unsigned)(nchains * nc)) {   // last workgroup: reset for the next launch
            counters[0] = 0u;
            counters[1] = 0u;
        }
    }
}

template <int N, int Q, int MODE>
hipError_t launch_mode(const ScanArgs &a, const Workspace &ws, dim3 grid) {
    const size_t smem = sizeof(Smem<N, Q>);
    auto kern = scan_mfma<N, Q, MODE>;
    static bool configured = false;
    if (!configured) {
        const hipError_t e = hipFuncSetAttribute((const void *)kern,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (e != hipSuccess) return e;
        configured = true;
    }
    kern<<<grid, kThreads, smem, a.stream>>>(
        (const __bf16 *)a.x, a.dt, a.A, (const __bf16 *)a.Bm, (const __bf16 *)a.Cm, a.D, a.init,
        (__bf16 *)a.y, a.final_state, ws.states, ws.decay, ws.flags, ws.counters, ws.ring, a.B, a.L,
        a.H, a.G);
    return hipGetLastError();
}

template <int N, int Q>
hipError_t run(const ScanArgs &a, const Workspace &ws, bool fused) {
    const int nc = (int)((a.L + Q - 1) / Q);
    if (fused) return launch_mode<N, Q, kFused>(a, ws, dim3((unsigned)(nc * a.B * a.H)));
    hipError_t e = launch_mode<N, Q, kState>(a, ws, dim3((unsigned)nc, (unsigned)(a.B * a.H)));
    if (e != hipSuccess) return e;
    e = launch_state_pass(ws.states, ws.decay, a.init, a.final_state, a.B, a.H, kP * N, nc, a.stream);
    if (e != hipSuccess) return e;
    return launch_mode<N, Q, kOutput>(a, ws, dim3((unsigned)nc, (unsigned)(a.B * a.H)));
}

template <int N>
hipError_t run_q(const ScanArgs &a, const Workspace &ws, bool fused) {
    switch (a.Q) {
        case 64: return run<N, 64>(a, ws, fused);
        case 128: return run<N, 128>(a, ws, fused);
        case 256: return run<N, 256>(a, ws, fused);
        default: return hipErrorInvalidValue;
    }
}

hipError_t dispatch(const ScanArgs &a, const Workspace &ws, bool fused) {
    switch (a.N) {
        case 64: return run_q<64>(a, ws, fused);
        case 128: return run_q<128>(a, ws, fused);
        case 256: return run_q<256>(a, ws, fused);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool mfma_supported(int64_t P, int64_t N, int64_t Q) {
    return P == kP && (N == 64 || N == 128 || N == 256) && (Q == 64 || Q == 128 || Q == 256);
}

size_t fused_max_chains() { return (size_t)1 << 30; }

hipError_t launch_staged_scan(const ScanArgs &a, const Workspace &ws) { return dispatch(a, ws, false); }

hipError_t launch_fused_scan(const ScanArgs &a, const Workspace &ws) { return dispatch(a, ws, true); }

}  // namespace ssd
