// One-pass chunk scan on gfx950 matrix cores: persistent, software-pipelined.
//
// Work items are (block c, batch b, head h) of Q tokens.  An item computes
//   pass 1: the state its block produces from zero, S_c, sub-block by
//           sub-block (64 tokens), keeping bf16 snapshots T of the
//           block-local state at every sub-block boundary;
//   hand-off: takes H_c (the state entering the block) from the item of
//           block c-1 of the same (b, h) and hands on
//           H_{c+1} = exp(Lambda_end) H_c + S_c;
//   pass 2: the outputs of every sub-block: the inter-block term
//           exp(Lambda_i - Lambda_{s-1}) Cm_i . (exp(Lambda_{s-1}) H_c + T),
//           the masked intra-block product sum_j M[i][j] x_j, and D x_i;
// the block decomposition of the "Mamba-2" note (section "taking each path
// half way") and of the "Mamba-2 model walkthrough" (sections 6.1-6.2),
// applied at two levels (blocks of Q tokens, sub-blocks of 64).
//
// Execution.  A fixed grid of workgroups (two per CU, four waves each) loops
// over items taken from a ticket counter in block-major order.  An item is
// 2*Q/64 steps (one per sub-block and pass) and every step ends in one
// barrier.  During step s a workgroup computes from LDS buffer s%2, stages step
// s+1 into the other LDS buffer from registers, and issues the global loads of
// step s+3 into the register slot it just emptied, so loads run two to three
// steps ahead of their use and the next item's x, Bm, Cm, G, dt, A and D
// stream in while the current item computes.
//
// Every global access in the step loop is an unconditional buffer load or
// store: the buffer's size (per item, in scalar registers) masks the tail of
// the sequence and items past the end of the queue (loads outside return 0,
// stores outside are dropped).  With no conditional memory operations the
// compiler can wait for exactly the loads a step needs instead of for every
// load in flight.
//
// The hand-off wait and the loads of H_c sit at the end of the last pass-1
// step, after that step's staging, where the only loads still in flight are
// the ones the next step stages anyway.  The predecessor's flag is raised one
// step after H_{c+1} is stored.  Tickets are taken four items ahead.  Waiting
// on a predecessor always ends: the smallest unfinished ticket is always the
// one some workgroup is working on (a ticket held ahead is larger than the one
// its holder works on), and its predecessor, with a smaller ticket, is done.
#include "common.h"

#include <type_traits>

namespace ssd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int kP = 64;
constexpr int kSub = 64;
constexpr int kThreads = 256;
constexpr int kAhead = 4;                // tickets taken this many items ahead
constexpr unsigned kSpinLimit = 1u << 22;
constexpr int TS = kSub + 8;             // row stride of [*][64] bf16 tiles (+16 bytes)
constexpr int kRaw = 0x00020000;         // buffer descriptor word 3: raw 32-bit access
constexpr int kCoherent = 16;            // sc1: device-coherent access

template <int N>
struct StepBuf {                         // one step's staged operands
    static constexpr int RS = N + 8;
    __bf16 xT[kP * TS];                  // x transposed [p][j]
    union {
        __bf16 BwT[N * TS];              // pass 1: weighted Bm transposed [n][j]
        struct {
            __bf16 Cs[kSub * RS];        // pass 2: Cm [i][n]
            __bf16 Mm[kSub * TS];        // pass 2: masked decay matrix [i][j]; then y [i][p]
        } o;
    } u;
};

struct Item {                            // one work item, uniform across the workgroup
    int c, chain, b, h, g, t0, q, valid;
};

template <int N, int Q>
struct FSmem {
    StepBuf<N> buf[2];
    float lam[2][Q];                     // per item parity: in-block prefix of dt*A
    float dts[2][Q];                     // per item parity: dt (0 past the end)
    float Ah[2], Dh[2];                  // per item parity: A_h, D_h
    Item tq[2 * kAhead];                 // ticket queue (item k at tq[k % (2*kAhead)])
};

template <int N>
struct Slot {                            // one step's global data, per thread
    uint4 x[2];                          // tokens 2tp, 2tp+1, columns 8pg..8pg+7
    uint4 m[N / 32];                     // pass 1: Bm units; pass 2: Cm pieces
    uint2 g[3];                          // pass 2: this wave's causal G tiles
};

struct Carry {                           // loaded with one step of each item, per thread:
    float dt, Av, Dv;                    // the next item's dt (token tid), A_h and D_h
};

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
__device__ __forceinline__ rsrc_t rsrc(const void *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, kRaw);
}
// (Only the vector and immediate offsets take part in the buffer's range
// check, so every row offset goes into the vector offset.)
// The buffer builtins move raw 32-bit words: every value goes in and out
// through a bit cast (an implicit int <-> float conversion would convert).
__device__ __forceinline__ uint4 ld16(rsrc_t r, int voff) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}
template <int AUX>
__device__ __forceinline__ f32x4 ld16f(rsrc_t r, int voff) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, AUX));
}
__device__ __forceinline__ float ld4f(rsrc_t r, int voff) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0));
}
template <int AUX, class T>
__device__ __forceinline__ void st16(T v, rsrc_t r, int voff) {
    static_assert(sizeof(T) == 16, "16-byte store");
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, voff, 0, AUX);
}

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
    const Item &e = q[k % (2 * kAhead)];
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

// Size in bytes of a buffer over the item's rows 0..q-1 (row stride `stride`
// elements, `width` elements used per row); 0 for an item past the end of the
// queue, so that all its loads read 0 and its stores are dropped.
__device__ __forceinline__ int row_bytes(const Item &it, int64_t stride, int width, int esize) {
    return (it.valid && it.q > 0) ? (int)(((int64_t)(it.q - 1) * stride + width) * esize) : 0;
}

// Global loads of one step (PHASE < NSB: pass 1 sub-block; else pass 2).
template <int N, int Q, int PHASE>
__device__ __forceinline__ void load_step(Slot<N> &sl, Carry &cr, const Args &a, const Item &it,
                                          const Item &nxt, int64_t nsb, int tid) {
    constexpr int NSB = Q / kSub;
    constexpr bool p1 = PHASE < NSB;
    constexpr bool carry = PHASE == 2 * NSB - 2;       // also load the next item's dt, A, D
    constexpr int s = (p1 ? PHASE : PHASE - NSB) * kSub;
    const int wave = tid >> 6, lane = tid & 63;
    const int64_t row0 = (int64_t)it.b * a.L + it.t0;
    {
        const int pg = tid & 7, tp = tid >> 3, j0 = s + 2 * tp;
        const rsrc_t rx = rsrc(a.x + (row0 * a.H + it.h) * kP, row_bytes(it, a.H * kP, kP, 2));
        const int o = (int)(((int64_t)j0 * a.H * kP + 8 * pg) * 2);
        sl.x[0] = ld16(rx, o);
        sl.x[1] = ld16(rx, o + (int)(a.H * kP * 2));
    }
    if constexpr (p1) {
        const rsrc_t rb = rsrc(a.Bm + (row0 * a.G + it.g) * N, row_bytes(it, a.G * N, N, 2));
#pragma unroll
        for (int k = 0; k < N / 64; ++k) {
            const int u = tid + k * kThreads;
            const int cg = u % (N / 8), tp = u / (N / 8), j0 = s + 2 * tp;
            const int o = (int)(((int64_t)j0 * a.G * N + 8 * cg) * 2);
            sl.m[2 * k] = ld16(rb, o);
            sl.m[2 * k + 1] = ld16(rb, o + (int)(a.G * N * 2));
        }
    } else {
        const rsrc_t rc = rsrc(a.Cm + (row0 * a.G + it.g) * N, row_bytes(it, a.G * N, N, 2));
#pragma unroll
        for (int k = 0; k < N / 32; ++k) {
            const int u = tid + k * kThreads;
            const int j = u / (N / 8), cg = u % (N / 8);
            sl.m[k] = ld16(rc, (int)(((int64_t)(s + j) * a.G * N + 8 * cg) * 2));
        }
        // this sub-block's G tiles in fragment order; every wave issues three
        // loads (waves with two tiles load their last one twice)
        const rsrc_t rg = rsrc(a.gram + (((int64_t)it.b * a.G + it.g) * nsb + it.t0 / kSub) * (kSub * kSub),
                               it.valid ? NSB * kSub * kSub * 2 : 0);
#pragma unroll
        for (int m = 0; m < 3; ++m) {
            const int k = wave + 4 * m < 10 ? wave + 4 * m : 9;
            sl.g[m] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(
                rg, ((s / kSub) * kSub * kSub + (k * 64 + lane) * 4) * 2, 0, 0));
        }
    }
    if constexpr (carry) {
        const int64_t nrow0 = (int64_t)nxt.b * a.L + nxt.t0;
        const rsrc_t rd = rsrc(a.dt + nrow0 * a.H + nxt.h, row_bytes(nxt, a.H, 1, 4));
        cr.dt = ld4f(rd, (int)((int64_t)tid * a.H * 4));
        cr.Av = ld4f(rsrc(a.A + nxt.h, nxt.valid ? 4 : 0), 0);
        cr.Dv = ld4f(rsrc(a.D + nxt.h, nxt.valid ? 4 : 0), 0);
    }
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
        // masked decay matrix from this wave's G tiles
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
            // the tiles above the diagonal that the apply reads: (0,1) and (2,3)
            const int ti = wave == 2 ? 0 : 2;
            uint32_t z = 0;
            asm volatile("" : "+v"(z));   // made here, not held in a register across the loop
            *reinterpret_cast<uint2 *>(&bf.u.o.Mm[(16 * ti + lrow) * TS + 16 * (ti + 1) + 4 * lgrp]) = uint2{z, z};
        }
    }
}

// In-block inclusive prefix sums of dt*A (one wave, 64 values per round).
// The lane permutes take their addresses from `lane` (not from the hardware
// lane id) so that they are computed here rather than held across the loop.
template <int Q>
__device__ __forceinline__ void prefix(const float *dts, float *lam, float Ah, int lane) {
    float carry = 0.f;
#pragma unroll
    for (int base = 0; base < Q; base += 64) {
        float v = dts[base + lane] * Ah;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float o = __int_as_float(__builtin_amdgcn_ds_bpermute(((lane - off) & 63) << 2, __float_as_int(v)));
            if (lane >= off) v += o;
        }
        v += carry;
        lam[base + lane] = v;
        carry = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
    }
}

// Vector memory operations each thread issues in the step loop at phase ph:
// the loads of step ph (x, then Bm or Cm, then in pass 2 the G tiles, and on
// the carrier step dt, A and D) and, in pass 2, two stores of y.
template <int N, int Q>
constexpr int loads_of(int ph) {
    return 2 + N / 32 + (ph >= Q / kSub ? 3 : 0) + (ph == 2 * (Q / kSub) - 2 ? 3 : 0);
}

// s_waitcnt immediate (gfx9 encoding) that waits until at most `v` vector
// memory operations are outstanding and does not wait on the other counters.
constexpr int vmcnt_imm(int v) { return (v & 15) | ((v >> 4) << 14) | (7 << 4) | (15 << 8); }

// The hand-off stores are issued at phase NSB; vector memory operations
// complete in issue order, so at the raise point they are complete once no
// more are outstanding than were issued after them: the two y stores of
// phase NSB and, when the flag goes up one step later, the loads issued at
// phase NSB (those of phase NSB+3) and the two y stores of phase NSB+1.
template <int N, int Q>
constexpr int raise_wait_count() {
    constexpr int NSB = Q / kSub, STEPS = 2 * NSB;
    return NSB + 1 < STEPS ? 2 + loads_of<N, Q>((NSB + 3) % STEPS) + 2 : 2;
}

template <int N, int Q>
__global__ __launch_bounds__(kThreads, 2) void scan_fused(Args a) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    using S = FSmem<N, Q>;
    S &sm = *reinterpret_cast<S *>(smem_raw);
    constexpr int NT = N / 16;
    constexpr int NSB = Q / kSub;
    constexpr int STEPS = 2 * NSB;
    constexpr int RAISE = NSB + 1 < STEPS ? NSB + 1 : NSB;   // step that raises the hand-off flag
    constexpr auto raise_wait = [] { return vmcnt_imm(raise_wait_count<N, Q>()); };
    using BF = StepBuf<N>;

    const int64_t nchains = a.Bsz * a.H;
    const int nc = (int)((a.L + Q - 1) / Q);
    const int64_t nsb = (int64_t)nc * NSB;

    if (threadIdx.x == 0) {
        for (int k = 0; k < kAhead; ++k) sm.tq[k] = decode<Q>(atomicAdd(&a.counters[0], 1u), a, nchains, nc);
    }
    __syncthreads();
    Item cur = item_at(sm.tq, 0);
    if (cur.valid) {
        {
            // the first item's dt, A, D and prefix sums
            const int tid = threadIdx.x;
            const float d0 = tid < cur.q ? a.dt[((int64_t)cur.b * a.L + cur.t0 + tid) * a.H + cur.h] : 0.f;
            if (tid < Q) sm.dts[0][tid] = d0;
            if (tid == 0) {
                sm.Ah[0] = a.A[cur.h];
                sm.Dh[0] = a.D[cur.h];
            }
            __syncthreads();
            if (tid < 64) prefix<Q>(sm.dts[0], sm.lam[0], sm.Ah[0], tid);
            __syncthreads();
        }

        // prologue: steps 0 and 1 into the slots, stage step 0, step 2 into slot 0.
        // Step t belongs to item t / STEPS and has phase t % STEPS.
        Slot<N> slot[2];
        Carry carry;
        {
            const int tid = threadIdx.x;
            load_step<N, Q, 0>(slot[0], carry, a, cur, item_at(sm.tq, 1), nsb, tid);
            load_step<N, Q, 1 % STEPS>(slot[1], carry, a, item_at(sm.tq, 1 / STEPS),
                                       item_at(sm.tq, 1 / STEPS + 1), nsb, tid);
            stage_step<N, Q, 0>(sm.buf[0], slot[0], sm.lam[0], sm.dts[0], tid);
            if constexpr (STEPS == 2) {   // step 0 carries the next item's dt, A, D
                if (tid < Q) sm.dts[1][tid] = carry.dt;
                if (tid == 0) {
                    sm.Ah[1] = carry.Av;
                    sm.Dh[1] = carry.Dv;
                }
            }
            load_step<N, Q, 2 % STEPS>(slot[0], carry, a, item_at(sm.tq, 2 / STEPS),
                                       item_at(sm.tq, 2 / STEPS + 1), nsb, tid);
        }
        __syncthreads();

        f32x4 Hacc[NT];                  // pass 1: S_c; pass 2: H_c
        f32x4 Hin[NT];                   // H_c from the last pass-1 step to the hand-off
        uint32_t Ts[NSB > 1 ? NSB - 1 : 1][2 * NT];
        unsigned ticket = 0;

        // One step of item k (`cur`) at compile-time phase PH.  `sl` is the
        // register slot of steps s+1 (staged now) and s+3 (loaded now).
        auto step = [&](auto phc, int64_t k, Slot<N> &sl) {
            constexpr int ph = decltype(phc)::value;
            // The lane id is made opaque to the optimizer at every step so that
            // addresses derived from it are recomputed here instead of being
            // hoisted out of the loop, where they would hold registers for the
            // whole kernel (and spill).
            int tid = threadIdx.x;
            asm volatile("" : "+v"(tid));
            const int wave = tid >> 6, lane = tid & 63;
            const int lrow = lane & 15, lgrp = lane >> 4;
            const int lane_off = (16 * wave + lrow) * N + 4 * lgrp;   // state layout, floats
            const int par = (int)(k & 1);
            if constexpr (ph == 0) {
                if (tid == 0) ticket = atomicAdd(&a.counters[0], 1u);   // item k + kAhead
            }
            const float *lam = sm.lam[par];
            const float *dts = sm.dts[par];
            const BF &bf = sm.buf[ph & 1];
            const int64_t row0 = (int64_t)cur.b * a.L + cur.t0;

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
                    // ---- hand-off out: H_{c+1} = gamma H_c + S_c to the
                    // successor's ring slot (device-coherent: another CU reads
                    // it in this launch), or to the final state (read by later
                    // launches only).  Both branches store the same count.
                    const float gamma = __expf(lam[Q - 1]);
                    if (cur.c + 1 < nc) {
                        const rsrc_t rd = rsrc(a.ring + ((int64_t)cur.chain * 2 + ((cur.c + 1) & 1)) * (kP * N),
                                               kP * N * 4);
#pragma unroll
                        for (int t = 0; t < NT; ++t)
                            st16<kCoherent>(gamma * Hin[t] + Hacc[t], rd, (lane_off + 16 * t) * 4);
                    } else {
                        const rsrc_t rd = rsrc(a.final_state ? a.final_state + (int64_t)cur.chain * (kP * N) : a.ring,
                                               a.final_state ? kP * N * 4 : 0);
#pragma unroll
                        for (int t = 0; t < NT; ++t)
                            st16<0>(gamma * Hin[t] + Hacc[t], rd, (lane_off + 16 * t) * 4);
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
                const float Dh = sm.Dh[par];
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
                const rsrc_t ry = rsrc(a.y + (row0 * a.H + cur.h) * kP, row_bytes(cur, a.H * kP, kP, 2));
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    const int u = tid + r * kThreads;                   // 512 pieces of 16 bytes
                    const int i = u >> 3, pc = u & 7;                  // token row, 8-column piece
                    const uint4 v = *reinterpret_cast<const uint4 *>(&ys[i * TS + 8 * pc]);
                    st16<0>(v, ry, (int)(((int64_t)(sbs + i) * a.H * kP + 8 * pc) * 2));
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
                        // that step's slot carries the next item's dt, A, D
                        if (tid < Q) sm.dts[par1 ^ 1][tid] = carry.dt;
                        if (tid == 0) {
                            sm.Ah[par1 ^ 1] = carry.Av;
                            sm.Dh[par1 ^ 1] = carry.Dv;
                        }
                    }
                }
            }
            // ---- prefix sums of the next item (its dt and A reached LDS one step ago)
            if constexpr (ph == STEPS - 2) {
                if (wave == 0) {
                    const Item nx = item_at(sm.tq, k + 1);
                    if (nx.valid) prefix<Q>(sm.dts[par ^ 1], sm.lam[par ^ 1], sm.Ah[par ^ 1], lane);
                }
            }
            // ---- the ticket taken at phase 0 goes into the queue
            if constexpr (ph == 1 % STEPS) {
                if (tid == 0) sm.tq[(k + kAhead) % (2 * kAhead)] = decode<Q>(ticket, a, nchains, nc);
            }
            // ---- hand-off in: wait for the predecessor's flag, then load H_c
            // (its ring slot, the initial state, or zeros from an empty buffer)
            if constexpr (ph == NSB - 1) {
                if (cur.c > 0) {
                    if (tid == 0) {
                        unsigned spins = 0;
                        while (__hip_atomic_load(&a.flags[cur.chain], __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT) < (unsigned)cur.c) {
                            __builtin_amdgcn_s_sleep(1);
                            if (++spins > kSpinLimit) {   // never expected: record it and go on
                                atomicOr(&a.counters[2], 1u);
                                break;
                            }
                        }
                        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                    }
                    __syncthreads();
                }
                // The ring slot was written in this launch by another CU: a
                // device-coherent load.  The initial state was written before
                // the launch: an ordinary load (a device-coherent one need not
                // see what an earlier kernel left in another L2).  Both
                // branches load the same count.
                if (cur.c > 0) {
                    const rsrc_t rs = rsrc(a.ring + ((int64_t)cur.chain * 2 + (cur.c & 1)) * (kP * N), kP * N * 4);
#pragma unroll
                    for (int t = 0; t < NT; ++t)
                        Hin[t] = ld16f<kCoherent>(rs, (lane_off + 16 * t) * 4);
                } else {
                    const rsrc_t rs = rsrc(a.init ? a.init + (int64_t)cur.chain * (kP * N) : a.ring,
                                           a.init ? kP * N * 4 : 0);
#pragma unroll
                    for (int t = 0; t < NT; ++t)
                        Hin[t] = ld16f<0>(rs, (lane_off + 16 * t) * 4);
                }
            }
            // ---- raise the flag for the successor (the last block clears it
            // for the next launch).  Every wave first sees its stores of
            // H_{c+1} complete; after the barrier one lane publishes with
            // release semantics (L2 write-back, then the flag), before this
            // step's loads are issued so that the release waits only for
            // loads issued a step ago.
            if constexpr (ph == RAISE) {
                __builtin_amdgcn_s_waitcnt(raise_wait());
                __syncthreads();
                if (tid == 0)
                    __hip_atomic_store(&a.flags[cur.chain], cur.c + 1 < nc ? (unsigned)(cur.c + 1) : 0u,
                                       __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
            }
            // ---- issue the loads of step s+3 (item k3, phase ph3)
            {
                constexpr int ph3 = (ph + 3) % STEPS;
                const int64_t k3 = k + (ph + 3) / STEPS;
                load_step<N, Q, ph3>(sl, carry, a, item_at(sm.tq, k3), item_at(sm.tq, k3 + 1), nsb, tid);
            }
            __syncthreads();
        };
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        using I2 = std::integral_constant<int, 2 % STEPS>;
        using I3 = std::integral_constant<int, 3 % STEPS>;
        using I4 = std::integral_constant<int, 4 % STEPS>;
        using I5 = std::integral_constant<int, 5 % STEPS>;
        using I6 = std::integral_constant<int, 6 % STEPS>;
        using I7 = std::integral_constant<int, 7 % STEPS>;
        // every step of an item is valid or none is: one check per item
        for (int64_t k = 0;; ++k) {
            cur = item_at(sm.tq, k);
            if (!cur.valid) break;
            step(I0{}, k, slot[1]);
            step(I1{}, k, slot[0]);
            if constexpr (STEPS > 2) {
                step(I2{}, k, slot[1]);
                step(I3{}, k, slot[0]);
            }
            if constexpr (STEPS > 4) {
                step(I4{}, k, slot[1]);
                step(I5{}, k, slot[0]);
                step(I6{}, k, slot[1]);
                step(I7{}, k, slot[0]);
            }
        }
    }
    // leave: the last workgroup out resets the counters for the next launch
    if (threadIdx.x == 0) {
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

// Shapes the one-pass kernel takes: N and Q it is built for, and a block's rows
// of x, Bm, Cm and dt within the 2^31-byte reach of a buffer offset.
bool fused_supported(int64_t H, int64_t G, int64_t N, int64_t Q) {
    if (!((N == 64 || N == 128) && (Q == 64 || Q == 128 || Q == 256))) return false;
    const int64_t lim = (int64_t)1 << 31;
    return Q * H * kP * 2 < lim && Q * G * N * 2 < lim && Q * H * 4 < lim;
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
