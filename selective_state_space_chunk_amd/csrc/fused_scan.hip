// One-pass chunk scan on gfx950 matrix cores: persistent, software-pipelined.
//
// Work items are (block c, batch b, head h) of Q tokens.  An item computes
//   pass 1: the state its block produces from zero, S_c, sub-block by
//           sub-block (64 tokens), keeping bf16 snapshots of the block-local
//           state at every sub-block boundary;
//   hand-off: takes H_c (the state entering the block) from the item of
//           block c-1 of the same (b, h), hands on H_{c+1} = exp(Lambda_end) H_c + S_c;
//   pass 2: the outputs of every sub-block from H_c and the snapshots
//           (the inter-block term Cm . (exp(Lambda_{s-1}) H_c + T) with its
//           row decay, plus the masked intra-block product, plus D x),
// which is the block decomposition of the "Mamba-2" note (section "taking each
// path half way") and of the "Mamba-2 model walkthrough" (sections 6.1-6.2),
// applied at two levels (blocks of Q, sub-blocks of 64).
//
// Execution.  A fixed grid of workgroups (two per CU) loops over items taken
// from a ticket counter in block-major order.  Each item is 2*Q/64 steps (one
// per sub-block and pass); every step ends in one barrier.  During step s a
// workgroup computes from LDS buffer s%2, stages step s+1 into the other LDS
// buffer from registers, and issues the global loads of step s+3 into the
// register slot it just emptied.  Loads therefore run two to three steps ahead
// of their use, and the next item's x, Bm, Cm, G and dt stream in while the
// current item computes.  Tickets are taken three items ahead.  Waiting on a
// predecessor always ends: the smallest unfinished ticket is always the one a
// workgroup is processing (a ticket held ahead is larger than the one its
// holder works on), and its predecessor, with a smaller ticket, is finished.
#include "common.h"

#include <type_traits>

namespace ssd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kP = 64;
constexpr int kSub = 64;
constexpr int kThreads = 256;
constexpr unsigned kSpinLimit = 1u << 22;
constexpr int TS = kSub + 8;      // row stride of [*][64] bf16 tiles (+16 bytes)

template <int N>
struct StepBuf {                  // one step's staged operands
    static constexpr int RS = N + 8;
    __bf16 xT[kP * TS];           // x transposed [p][j]
    union {
        __bf16 BwT[N * TS];       // pass 1: weighted Bm transposed [n][j]
        struct {
            __bf16 Cs[kSub * RS]; // pass 2: Cm [i][n]
            __bf16 Mm[kSub * TS]; // pass 2: masked decay matrix [i][j]
        } o;
    } u;
};

struct Item {               // one work item, uniform across the workgroup
    int c, chain, b, h, g, t0, q, valid;
};

template <int N, int Q>
struct FSmem {
    StepBuf<N> buf[2];
    float lam[2][Q];              // per item parity: in-block prefix of dt*A
    float dts[2][Q];              // per item parity: dt (0 past the end)
    Item tq[4];                   // decoded ticket queue (item k at tq[k & 3])
};

template <int N>
struct Slot {                     // one step's global data, per thread
    uint4 x[2];                   // tokens 2tp, 2tp+1, columns 8pg..8pg+7
    uint4 m[N / 32];              // pass 1: Bm units; pass 2: Cm pieces
    uint2 g[3];                   // pass 2: this wave's causal G tiles
    float dt;                     // dt of the next item (carrier steps only)
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

struct Args {
    const __bf16 *x;
    const float *dt, *A;
    const __bf16 *Bm, *Cm;
    const float *D, *init;
    __bf16 *y;
    float *final_state;
    unsigned *flags, *counters;
    float *ring;
    const __bf16 *gram;
    int64_t Bsz, L, H, G;
};

template <int Q>
__device__ __forceinline__ Item decode(unsigned t, const Args &a, int64_t nchains, int nc) {
    Item it;
    it.valid = (int64_t)t < nchains * nc;
    const int64_t tt = it.valid ? t : 0;
    it.c = (int)(tt / nchains);
    it.chain = (int)(tt % nchains);
    it.b = (int)(it.chain / a.H);
    it.h = (int)(it.chain % a.H);
    it.g = (int)(it.h / (a.H / a.G));
    it.t0 = it.c * Q;
    it.q = (int)((a.L - it.t0) < Q ? (a.L - it.t0) : Q);
    return it;
}

// An item from the LDS queue, in scalar registers.
__device__ __forceinline__ Item item_at(const Item *q, int64_t k) {
    const Item &e = q[k & 3];
    Item it;
    it.c = __builtin_amdgcn_readfirstlane(e.c);
    it.chain = __builtin_amdgcn_readfirstlane(e.chain);
    it.b = __builtin_amdgcn_readfirstlane(e.b);
    it.h = __builtin_amdgcn_readfirstlane(e.h);
    it.g = __builtin_amdgcn_readfirstlane(e.g);
    it.t0 = __builtin_amdgcn_readfirstlane(e.t0);
    it.q = __builtin_amdgcn_readfirstlane(e.q);
    it.valid = __builtin_amdgcn_readfirstlane(e.valid);
    return it;
}

// Global loads of one step (phase < NSB: pass 1 sub-block; else pass 2).
template <int N, int Q, int PHASE>
__device__ __forceinline__ void load_step(Slot<N> &sl, const Args &a, const Item &it,
                                          const Item &nxt, int64_t nsb, int tid) {
    constexpr int NSB = Q / kSub;
    constexpr bool p1 = PHASE < NSB;
    constexpr bool carry_dt = PHASE == 2 * NSB - 2;
    constexpr int s = (p1 ? PHASE : PHASE - NSB) * kSub;
    const int wave = tid >> 6, lane = tid & 63;
    const int lrow = lane & 15, lgrp = lane >> 4;
    {
        const int pg = tid & 7, tp = tid >> 3, j0 = s + 2 * tp;
        const __bf16 *p0 = a.x + ((((int64_t)it.b * a.L + it.t0 + j0) * a.H + it.h) * kP + 8 * pg);
        sl.x[0] = j0 < it.q ? *reinterpret_cast<const uint4 *>(p0) : uint4{0, 0, 0, 0};
        sl.x[1] = j0 + 1 < it.q ? *reinterpret_cast<const uint4 *>(p0 + a.H * kP) : uint4{0, 0, 0, 0};
    }
    if constexpr (p1) {
#pragma unroll
        for (int k = 0; k < N / 64; ++k) {
            const int u = tid + k * kThreads;
            const int cg = u % (N / 8), tp = u / (N / 8), j0 = s + 2 * tp;
            const __bf16 *p0 = a.Bm + ((((int64_t)it.b * a.L + it.t0 + j0) * a.G + it.g) * N + 8 * cg);
            sl.m[2 * k] = j0 < it.q ? *reinterpret_cast<const uint4 *>(p0) : uint4{0, 0, 0, 0};
            sl.m[2 * k + 1] = j0 + 1 < it.q ? *reinterpret_cast<const uint4 *>(p0 + a.G * N) : uint4{0, 0, 0, 0};
        }
    } else {
#pragma unroll
        for (int k = 0; k < N / 32; ++k) {
            const int u = tid + k * kThreads;
            const int j = u / (N / 8), cg = u % (N / 8);
            sl.m[k] = s + j < it.q
                          ? *reinterpret_cast<const uint4 *>(a.Cm + ((((int64_t)it.b * a.L + it.t0 + s + j) * a.G + it.g) * N + 8 * cg))
                          : uint4{0, 0, 0, 0};
        }
        const int64_t sbg = (it.t0 + s) / kSub;
        const __bf16 *gb = a.gram + (((int64_t)it.b * a.G + it.g) * nsb + sbg) * (int64_t)(kSub * kSub);
#pragma unroll
        for (int m = 0; m < 3; ++m) {
            const int k = wave + 4 * m;
            if (k < 10) {
                sl.g[m] = *reinterpret_cast<const uint2 *>(gb + (k * 64 + lane) * 4);
            }
        }
    }
    if constexpr (carry_dt) sl.dt = (nxt.valid && tid < nxt.q) ? a.dt[((int64_t)nxt.b * a.L + nxt.t0 + tid) * a.H + nxt.h] : 0.f;
}

// Stage one step's operands from registers into an LDS buffer.
template <int N, int Q, int PHASE>
__device__ __forceinline__ void stage_step(StepBuf<N> &bf, const Slot<N> &sl, const float *lam,
                                           const float *dts, int tid) {
    constexpr int NSB = Q / kSub;
    constexpr bool p1 = PHASE < NSB;
    constexpr int s = (p1 ? PHASE : PHASE - NSB) * kSub;
    using B = StepBuf<N>;
    const int wave = tid >> 6, lane = tid & 63;
    const int lrow = lane & 15, lgrp = lane >> 4;
    {
        const int pg = tid & 7, tp = tid >> 3, j0 = 2 * tp;
        const uint4 x0 = sl.x[0], x1 = sl.x[1];
        const uint32_t a0[4] = {x0.x, x0.y, x0.z, x0.w}, a1[4] = {x1.x, x1.y, x1.z, x1.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            *reinterpret_cast<uint32_t *>(&bf.xT[(8 * pg + 2 * k) * TS + j0]) = (a0[k] & 0xffffu) | (a1[k] << 16);
            *reinterpret_cast<uint32_t *>(&bf.xT[(8 * pg + 2 * k + 1) * TS + j0]) = (a0[k] >> 16) | (a1[k] & 0xffff0000u);
        }
    }
    if constexpr (p1) {
        const float lam_e = lam[s + kSub - 1];
#pragma unroll
        for (int k = 0; k < N / 64; ++k) {
            const int u = tid + k * kThreads;
            const int cg = u % (N / 8), tp = u / (N / 8), j0 = 2 * tp;
            const float w0 = __expf(lam_e - lam[s + j0]) * dts[s + j0];
            const float w1 = __expf(lam_e - lam[s + j0 + 1]) * dts[s + j0 + 1];
            const uint4 v0 = sl.m[2 * k], v1 = sl.m[2 * k + 1];
            const uint32_t a0[4] = {v0.x, v0.y, v0.z, v0.w}, a1[4] = {v1.x, v1.y, v1.z, v1.w};
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                *reinterpret_cast<uint32_t *>(&bf.u.BwT[(8 * cg + 2 * m) * TS + j0]) =
                    pack2(w0 * lo_bf16(a0[m]), w1 * lo_bf16(a1[m]));
                *reinterpret_cast<uint32_t *>(&bf.u.BwT[(8 * cg + 2 * m + 1) * TS + j0]) =
                    pack2(w0 * hi_bf16(a0[m]), w1 * hi_bf16(a1[m]));
            }
        }
    } else {
#pragma unroll
        for (int k = 0; k < N / 32; ++k) {
            const int u = tid + k * kThreads;
            const int j = u / (N / 8), cg = u % (N / 8);
            *reinterpret_cast<uint4 *>(&bf.u.o.Cs[j * B::RS + 8 * cg]) = sl.m[k];
        }
#pragma unroll
        for (int m = 0; m < 3; ++m) {
            const int k = wave + 4 * m;
            if (k < 10) {
                int ti, tj;
                tile_of(k, ti, tj);
                const int i = 16 * ti + lrow;
                const float li = lam[s + i];
                const uint32_t gw[2] = {sl.g[m].x, sl.g[m].y};
                float mv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int j = 16 * tj + 4 * lgrp + e;
                    const float gv = (e & 1) ? hi_bf16(gw[e >> 1]) : lo_bf16(gw[e >> 1]);
                    mv[e] = j <= i ? gv * __expf(li - lam[s + j]) * dts[s + j] : 0.f;
                }
                uint2 pk;
                pk.x = pack2(mv[0], mv[1]);
                pk.y = pack2(mv[2], mv[3]);
                *reinterpret_cast<uint2 *>(&bf.u.o.Mm[i * TS + 16 * tj + 4 * lgrp]) = pk;
            }
        }
        if (wave >= 2) {
            const int ti = wave == 2 ? 0 : 2;
            *reinterpret_cast<uint2 *>(&bf.u.o.Mm[(16 * ti + lrow) * TS + 16 * (ti + 1) + 4 * lgrp]) = uint2{0u, 0u};
        }
    }
}

template <int N, int Q>
__global__ __launch_bounds__(kThreads, 2) void scan_fused(Args a) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    using S = FSmem<N, Q>;
    S &sm = *reinterpret_cast<S *>(smem_raw);
    constexpr int NT = N / 16;
    constexpr int NSB = Q / kSub;
    constexpr int STEPS = 2 * NSB;
    constexpr int RAISE = NSB + 1 < STEPS ? NSB + 1 : NSB;   // step of the hand-off flag
    using BF = StepBuf<N>;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int lrow = lane & 15, lgrp = lane >> 4;
    const int64_t nchains = a.Bsz * a.H;
    const int nc = (int)((a.L + Q - 1) / Q);
    const int64_t nsb = (int64_t)nc * NSB;
    const int64_t lane_off = (int64_t)(16 * wave + lrow) * N + 4 * lgrp;   // state layout, floats

    if (tid == 0) {
        for (int k = 0; k < 3; ++k) sm.tq[k] = decode<Q>(atomicAdd(&a.counters[0], 1u), a, nchains, nc);
    }
    __syncthreads();
    Item cur = item_at(sm.tq, 0);
    if (cur.valid) {
        // first item's prefix sums
        const float d0 = tid < cur.q ? a.dt[((int64_t)cur.b * a.L + cur.t0 + tid) * a.H + cur.h] : 0.f;
        if (tid < Q) sm.dts[0][tid] = d0;
        __syncthreads();
        if (wave == 0) {
            const float Ah = a.A[cur.h];
            float carry = 0.f;
#pragma unroll
            for (int base = 0; base < Q; base += 64) {
                float v = sm.dts[0][base + lane] * Ah;
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const float o = __shfl_up(v, off);
                    if (lane >= off) v += o;
                }
                v += carry;
                sm.lam[0][base + lane] = v;
                carry = __shfl(v, 63);
            }
        }
        __syncthreads();

        // prologue: steps 0 and 1 into the slots, stage step 0, step 2 into slot 0.
        // Step t belongs to item t / STEPS and has phase t % STEPS.
        Slot<N> slot[2];
        {
            const Item i0 = item_at(sm.tq, 0);
            const Item i1 = item_at(sm.tq, 1 / STEPS);
            const Item i2 = item_at(sm.tq, 2 / STEPS);
            const Item n0 = item_at(sm.tq, 0 / STEPS + 1);
            const Item n1 = item_at(sm.tq, 1 / STEPS + 1);
            const Item n2 = item_at(sm.tq, 2 / STEPS + 1);
            load_step<N, Q, 0>(slot[0], a, i0, n0, nsb, threadIdx.x);
            if (i1.valid) load_step<N, Q, 1 % STEPS>(slot[1], a, i1, n1, nsb, threadIdx.x);
            stage_step<N, Q, 0>(sm.buf[0], slot[0], sm.lam[0], sm.dts[0], threadIdx.x);
            if constexpr (STEPS == 2) {   // step 0 carries the next item's dt
                if (tid < Q) sm.dts[1][tid] = slot[0].dt;
            }
            if (i2.valid) load_step<N, Q, 2 % STEPS>(slot[0], a, i2, n2, nsb, threadIdx.x);
        }
        __syncthreads();

        f32x4 Hacc[NT];
        uint32_t Ts[NSB > 1 ? NSB - 1 : 1][2 * NT];
        bool raise_pending = false;
        unsigned raise_value = 0;
        int raise_chain = 0;

        // One step of item k at compile-time phase PH.  `sl` is the register
        // slot of steps s+1 (staged now) and s+3 (loaded now).  Returns false
        // when item k is not a valid work item (the queue ran out).
        auto step = [&](auto phc, int64_t k, Slot<N> &sl) -> bool {
            constexpr int ph = decltype(phc)::value;
            // The lane id is made opaque to the optimizer at every step so that
            // addresses derived from it are recomputed here instead of being
            // hoisted out of the loop, where they would hold registers for the
            // whole kernel (and spill).
            int tid = threadIdx.x;
            asm volatile("" : "+v"(tid));
            const int wave = tid >> 6, lane = tid & 63;
            const int lrow = lane & 15, lgrp = lane >> 4;
            const int64_t lane_off = (int64_t)(16 * wave + lrow) * N + 4 * lgrp;
            const int par = (int)(k & 1);
            cur = item_at(sm.tq, k);
            if (!cur.valid) return false;
            if (ph == 0 && tid == 0) sm.tq[(k + 3) & 3] = decode<Q>(atomicAdd(&a.counters[0], 1u), a, nchains, nc);
            const float *lam = sm.lam[par];
            const float *dts = sm.dts[par];
            const BF &bf = sm.buf[ph & 1];

            if constexpr (ph < NSB) {
                // ---- pass 1: block-local state, sub-block ph
                constexpr int sbs = ph * kSub;
                if constexpr (ph == 0) {
#pragma unroll
                    for (int t = 0; t < NT; ++t) Hacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
                const float before = sbs == 0 ? 0.f : lam[sbs > 0 ? sbs - 1 : 0];
                const float gsb = __expf(lam[sbs + kSub - 1] - before);
#pragma unroll
                for (int t = 0; t < NT; ++t) Hacc[t] *= gsb;
#pragma unroll
                for (int ks = 0; ks < kSub / 32; ++ks) {
                    const int j0 = 32 * ks + 8 * lgrp;
                    const bf16x8 bx = *reinterpret_cast<const bf16x8 *>(&bf.xT[(16 * wave + lrow) * TS + j0]);
#pragma unroll
                    for (int t = 0; t < NT; ++t) {
                        const bf16x8 ba = *reinterpret_cast<const bf16x8 *>(&bf.u.BwT[(16 * t + lrow) * TS + j0]);
                        Hacc[t] = mfma(ba, bx, Hacc[t]);
                    }
                }
                if constexpr (ph + 1 < NSB) {
#pragma unroll
                    for (int t = 0; t < NT; ++t) {
                        Ts[ph][2 * t] = pack2(Hacc[t][0], Hacc[t][1]);
                        Ts[ph][2 * t + 1] = pack2(Hacc[t][2], Hacc[t][3]);
                    }
                }
            } else {
                constexpr int sbi = ph - NSB;
                constexpr int sbs = sbi * kSub;
                if constexpr (ph == NSB) {
                    // ---- hand-off: H_c in, H_{c+1} = gamma H_c + S_c out
                    const float gamma = __expf(lam[Q - 1]);
                    f32x4 Hin[NT];
                    if (cur.c == 0) {
                        if (a.init) {
                            const float *src = a.init + (int64_t)cur.chain * (kP * N) + lane_off;
#pragma unroll
                            for (int t = 0; t < NT; ++t) Hin[t] = *reinterpret_cast<const f32x4 *>(src + 16 * t);
                        } else {
#pragma unroll
                            for (int t = 0; t < NT; ++t) Hin[t] = f32x4{0.f, 0.f, 0.f, 0.f};
                        }
                    } else {
                        if (tid == 0) {
                            unsigned spins = 0;
                            while (__hip_atomic_load(&a.flags[cur.chain], __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT) < (unsigned)cur.c) {
                                __builtin_amdgcn_s_sleep(1);
                                if (++spins > kSpinLimit) {
                                    atomicOr(&a.counters[2], 1u);
                                    break;
                                }
                            }
                            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                        }
                        __syncthreads();
                        // device-coherent 16-byte loads (sc1): written by another CU
                        const __amdgpu_buffer_rsrc_t src = __builtin_amdgcn_make_buffer_rsrc(
                            a.ring + ((int64_t)cur.chain * 2 + (cur.c & 1)) * (kP * N), 0, kP * N * 4, 0x00020000);
#pragma unroll
                        for (int t = 0; t < NT; ++t)
                            Hin[t] = __builtin_amdgcn_raw_buffer_load_b128(src, (int)((lane_off + 16 * t) * 4), 0, 16);
                    }
#pragma unroll
                    for (int t = 0; t < NT; ++t) Hacc[t] = gamma * Hin[t] + Hacc[t];
                    if (cur.c + 1 < nc) {
                        const __amdgpu_buffer_rsrc_t dst = __builtin_amdgcn_make_buffer_rsrc(
                            a.ring + ((int64_t)cur.chain * 2 + ((cur.c + 1) & 1)) * (kP * N), 0, kP * N * 4, 0x00020000);
#pragma unroll
                        for (int t = 0; t < NT; ++t)
                            __builtin_amdgcn_raw_buffer_store_b128(Hacc[t], dst, (int)((lane_off + 16 * t) * 4), 0, 16);
                        raise_pending = true;
                        raise_value = (unsigned)(cur.c + 1);
                        raise_chain = cur.chain;
                    } else {
                        if (a.final_state) {
                            float *dst = a.final_state + (int64_t)cur.chain * (kP * N) + lane_off;
#pragma unroll
                            for (int t = 0; t < NT; ++t) *reinterpret_cast<f32x4 *>(dst + 16 * t) = Hacc[t];
                        }
                        if (tid == 0) a.flags[cur.chain] = 0u;   // last user of this chain's flag
                    }
#pragma unroll
                    for (int t = 0; t < NT; ++t) Hacc[t] = Hin[t];
                }
                // ---- pass 2: outputs of sub-block sbi
                const float eb = sbs == 0 ? 1.f : __expf(lam[sbs > 0 ? sbs - 1 : 0]);
                const float before = sbs == 0 ? 0.f : lam[sbs > 0 ? sbs - 1 : 0];
                f32x4 Y[4];
#pragma unroll
                for (int it = 0; it < 4; ++it) Y[it] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < N / 32; ++ks) {
                    f32x4 h0 = Hacc[2 * ks], h1 = Hacc[2 * ks + 1];
                    if constexpr (sbi > 0) {
                        const uint32_t *tw = &Ts[sbi > 0 ? sbi - 1 : 0][4 * ks];
                        h0 = eb * h0 + f32x4{lo_bf16(tw[0]), hi_bf16(tw[0]), lo_bf16(tw[1]), hi_bf16(tw[1])};
                        h1 = eb * h1 + f32x4{lo_bf16(tw[2]), hi_bf16(tw[2]), lo_bf16(tw[3]), hi_bf16(tw[3])};
                    }
                    bf16x8 ah;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        ah[e] = (__bf16)h0[e];
                        ah[4 + e] = (__bf16)h1[e];
                    }
#pragma unroll
                    for (int it = 0; it < 4; ++it) {
                        const __bf16 *crow = &bf.u.o.Cs[(16 * it + lrow) * BF::RS + 32 * ks + 4 * lgrp];
                        const bf16x4 c0 = *reinterpret_cast<const bf16x4 *>(crow);
                        const bf16x4 c1 = *reinterpret_cast<const bf16x4 *>(crow + 16);
                        const bf16x8 bc = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
                        Y[it] = mfma(ah, bc, Y[it]);
                    }
                }
#pragma unroll
                for (int it = 0; it < 4; ++it) Y[it] *= __expf(lam[sbs + 16 * it + lrow] - before);
#pragma unroll
                for (int it = 0; it < 4; ++it) {
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) {
                        if (ks == 1 && it < 2) continue;
                        const int j0 = 32 * ks + 8 * lgrp;
                        const bf16x8 ax = *reinterpret_cast<const bf16x8 *>(&bf.xT[(16 * wave + lrow) * TS + j0]);
                        const bf16x8 bm = *reinterpret_cast<const bf16x8 *>(&bf.u.o.Mm[(16 * it + lrow) * TS + j0]);
                        Y[it] = mfma(ax, bm, Y[it]);
                    }
                }
                // skip term; the sub-block's outputs go through LDS (the mask
                // region, free once every wave is past the apply) so that they
                // leave as whole 128-byte rows
                const float Dh = a.D[cur.h];
                __syncthreads();
                __bf16 *ys = const_cast<__bf16 *>(bf.u.o.Mm);           // [i][p], row stride TS
#pragma unroll
                for (int it = 0; it < 4; ++it) {
                    const int i = 16 * it + lrow;
                    const int p0 = 16 * wave + 4 * lgrp;
                    float o[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[e] = Y[it][e] + Dh * (float)bf.xT[(p0 + e) * TS + i];
                    uint2 pk;
                    pk.x = pack2(o[0], o[1]);
                    pk.y = pack2(o[2], o[3]);
                    *reinterpret_cast<uint2 *>(&ys[i * TS + p0]) = pk;
                }
                __syncthreads();
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    const int u = tid + r * kThreads;                   // 512 pieces of 16 bytes
                    const int i = u >> 3, pc = u & 7;                  // token row, 8-column piece
                    if (sbs + i < cur.q) {
                        const uint4 v = *reinterpret_cast<const uint4 *>(&ys[i * TS + 8 * pc]);
                        *reinterpret_cast<uint4 *>(a.y + ((((int64_t)cur.b * a.L + cur.t0 + sbs + i) * a.H + cur.h) * kP + 8 * pc)) = v;
                    }
                }
            }

            // ---- stage step s+1 (item k1, phase ph1)
            {
                constexpr int ph1 = (ph + 1) % STEPS;
                const int64_t k1 = k + (ph + 1) / STEPS;
                const Item it1 = item_at(sm.tq, k1);
                if (it1.valid) {
                    const int par1 = (int)(k1 & 1);
                    stage_step<N, Q, ph1>(sm.buf[(ph + 1) & 1], sl, sm.lam[par1], sm.dts[par1], tid);
                    if constexpr (ph1 == STEPS - 2) {
                        if (tid < Q) sm.dts[par1 ^ 1][tid] = sl.dt;
                    }
                }
            }
            // ---- prefix sums of the next item (its dt reached LDS one step ago)
            if constexpr (ph == STEPS - 2) {
                if (wave == 0) {
                    const Item nx = item_at(sm.tq, k + 1);
                    if (nx.valid) {
                        const float Ah = a.A[nx.h];
                        float carry = 0.f;
#pragma unroll
                        for (int base = 0; base < Q; base += 64) {
                            float v = sm.dts[par ^ 1][base + lane] * Ah;
#pragma unroll
                            for (int off = 1; off < 64; off <<= 1) {
                                const float o = __shfl_up(v, off);
                                if (lane >= off) v += o;
                            }
                            v += carry;
                            sm.lam[par ^ 1][base + lane] = v;
                            carry = __shfl(v, 63);
                        }
                    }
                }
            }
            constexpr bool raise_step = ph == RAISE;
            const bool raise_now = raise_step && raise_pending;
            if (raise_now) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // hand-off stores done
            // ---- issue the loads of step s+3 (item k3, phase ph3)
            {
                constexpr int ph3 = (ph + 3) % STEPS;
                const int64_t k3 = k + (ph + 3) / STEPS;
                const Item it3 = item_at(sm.tq, k3);
                if (it3.valid) {
                    const Item nxt = item_at(sm.tq, k3 + 1);
                    load_step<N, Q, ph3>(sl, a, it3, nxt, nsb, tid);
                }
            }
            __syncthreads();
            if (raise_now) {
                if (tid == 0)
                    __hip_atomic_store(&a.flags[raise_chain], raise_value, __ATOMIC_RELEASE,
                                       __HIP_MEMORY_SCOPE_AGENT);
                raise_pending = false;
            }
            return true;
        };
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        using I2 = std::integral_constant<int, 2 % STEPS>;
        using I3 = std::integral_constant<int, 3 % STEPS>;
        using I4 = std::integral_constant<int, 4 % STEPS>;
        using I5 = std::integral_constant<int, 5 % STEPS>;
        using I6 = std::integral_constant<int, 6 % STEPS>;
        using I7 = std::integral_constant<int, 7 % STEPS>;
        for (int64_t k = 0;; ++k) {
            if (!step(I0{}, k, slot[1])) break;
            if (!step(I1{}, k, slot[0])) break;
            if constexpr (STEPS > 2) {
                if (!step(I2{}, k, slot[1])) break;
                if (!step(I3{}, k, slot[0])) break;
            }
            if constexpr (STEPS > 4) {
                if (!step(I4{}, k, slot[1])) break;
                if (!step(I5{}, k, slot[0])) break;
                if (!step(I6{}, k, slot[1])) break;
                if (!step(I7{}, k, slot[0])) break;
            }
        }
    }
    // leave: the last workgroup out resets the counters for the next launch
    if (tid == 0) {
        const unsigned out = atomicAdd(&a.counters[1], 1u);
        if (out + 1 == gridDim.x) {
            __hip_atomic_store(&a.counters[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&a.counters[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

int cu_count() {
    static int cus = 0;
    if (cus == 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
    }
    return cus;
}

template <int N, int Q>
hipError_t launch(const ScanArgs &sa, const Workspace &ws) {
    constexpr int NSB = Q / kSub;
    const int nc = (int)((sa.L + Q - 1) / Q);
    const int64_t nsb = (int64_t)nc * NSB;
    hipError_t e = launch_gram(sa, ws, nsb);
    if (e != hipSuccess) return e;
    const size_t smem = sizeof(FSmem<N, Q>);
    auto kern = scan_fused<N, Q>;
    static bool configured = false;
    if (!configured) {
        e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (e != hipSuccess) return e;
        configured = true;
    }
    Args a{(const __bf16 *)sa.x, sa.dt, sa.A, (const __bf16 *)sa.Bm, (const __bf16 *)sa.Cm, sa.D,
           sa.init, (__bf16 *)sa.y, sa.final_state, ws.flags, ws.counters, ws.ring,
           (const __bf16 *)ws.gram, sa.B, sa.L, sa.H, sa.G};
    const int64_t items = (int64_t)nc * sa.B * sa.H;
    const int64_t grid = items < 2 * (int64_t)cu_count() ? items : 2 * (int64_t)cu_count();
    kern<<<dim3((unsigned)grid), kThreads, smem, sa.stream>>>(a);
    return hipGetLastError();
}

}  // namespace

bool fused_supported(int64_t N, int64_t Q) {
    return (N == 64 || N == 128) && (Q == 64 || Q == 128 || Q == 256);
}

hipError_t launch_fused_scan(const ScanArgs &a, const Workspace &ws) {
    switch (a.N * 1000 + a.Q) {
        case 64064: return launch<64, 64>(a, ws);
        case 64128: return launch<64, 128>(a, ws);
        case 64256: return launch<64, 256>(a, ws);
        case 128064: return launch<128, 64>(a, ws);
        case 128128: return launch<128, 128>(a, ws);
        case 128256: return launch<128, 256>(a, ws);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace ssd
