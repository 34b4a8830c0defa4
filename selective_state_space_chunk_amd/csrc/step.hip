// One recurrent decode step (the recurrent path of the "Mamba-2" note,
// four-token section): for each (b, h),
//   alpha = exp(dt A_h);  S <- alpha S + dt x (outer) Bm;  y = S Cm + D x.
//
// The state dominates the traffic: P*N float32 read and written once per
// token, against P + 2N + a few inputs.  The kernel is a coalesced stream over
// the state in small pieces: each workgroup takes R rows of one (b, h) state,
// about 4 KB (R = 1024 / N rows, at most P), each row of N floats as N/4
// float4 lanes, two rows per thread where the piece allows, every load issued
// before any store.  Small pieces spread the stream over many workgroups: a
// plain copy on MI355X runs at 6.6 TB/s in 4 KB pieces against 6.1-6.3 TB/s
// in 16-32 KB ones, and so does this kernel (0.82 of the 8 TB/s peak at
// B 256, H 80, P 64, N 128, against 0.76 with one 32 KB workgroup per state).
// A row's dot product with Cm is reduced across its lanes with shuffles.
// Loads and stores of the state bypass cache allocation (non-temporal):
// nothing re-reads it within the step.
#include "common.h"

namespace ssd {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Rows of one state per workgroup, threads per workgroup and rows per thread.
template <int P, int N>
struct StepShape {
    static constexpr int LPR = N / 4;                           // lanes per state row (4..64)
    static constexpr int R = P < 1024 / N ? P : 1024 / N;       // rows per workgroup (~4 KB)
    static constexpr int ITERS = R * LPR >= 128 ? 2 : 1;        // rows per thread
    static constexpr int NTH = R * LPR / ITERS;                 // threads per workgroup
    static constexpr int S = P / R;                             // workgroups per (b, h)
    static_assert(R * LPR % ITERS == 0 && P % R == 0 && NTH <= 1024, "step shape");
};

template <class T, int P, int N>
__global__ __launch_bounds__((StepShape<P, N>::NTH)) void step_kernel(
    float *__restrict__ state, const T *__restrict__ x, const float *__restrict__ dt,
    const float *__restrict__ A, const T *__restrict__ Bm, const T *__restrict__ Cm,
    const float *__restrict__ D, T *__restrict__ y, int H, int G) {
    using Sh = StepShape<P, N>;
    constexpr int LPR = Sh::LPR, ROWS = Sh::NTH / LPR;            // rows covered per pass
    const int64_t bh = blockIdx.x / Sh::S;
    const int part = (int)(blockIdx.x % Sh::S);
    const int b = (int)(bh / H), h = (int)(bh % H);
    const int g = h / (H / G);
    const int lane = threadIdx.x & (LPR - 1);
    const int row0 = part * Sh::R + (int)threadIdx.x / LPR;

    const float dtv = dt[bh];
    const float alpha = expf(dtv * A[h]);
    const float Dh = D[h];
    float bv[4], cv[4];
    const T *bp = Bm + ((int64_t)b * G + g) * N + lane * 4;
    const T *cp = Cm + ((int64_t)b * G + g) * N + lane * 4;
#pragma unroll
    for (int k = 0; k < 4; ++k) { bv[k] = to_f32(bp[k]); cv[k] = to_f32(cp[k]); }

    f32x4 *sp = reinterpret_cast<f32x4 *>(state + bh * (int64_t)(P * N));
    f32x4 s[Sh::ITERS];
    float xv[Sh::ITERS];
#pragma unroll
    for (int it = 0; it < Sh::ITERS; ++it) {
        const int p = row0 + it * ROWS;
        s[it] = __builtin_nontemporal_load(sp + p * LPR + lane);
        xv[it] = to_f32(x[bh * P + p]);
    }
#pragma unroll
    for (int it = 0; it < Sh::ITERS; ++it) {
        const int p = row0 + it * ROWS;
        const float u = dtv * xv[it];
        f32x4 v = s[it];
        v.x = alpha * v.x + u * bv[0];
        v.y = alpha * v.y + u * bv[1];
        v.z = alpha * v.z + u * bv[2];
        v.w = alpha * v.w + u * bv[3];
        __builtin_nontemporal_store(v, sp + p * LPR + lane);
        float part_ = v.x * cv[0] + v.y * cv[1] + v.z * cv[2] + v.w * cv[3];
#pragma unroll
        for (int off = LPR / 2; off > 0; off >>= 1) part_ += __shfl_xor(part_, off);
        if (lane == 0) y[bh * P + p] = from_f32<T>(part_ + Dh * xv[it]);
    }
}

template <class T, int P>
hipError_t launch_n(float *state, const void *x, const float *dt, const float *A, const void *Bm,
                    const void *Cm, const float *D, void *y, int64_t B, int64_t H, int64_t G,
                    int64_t N, hipStream_t stream) {
#define SSD_STEP_N(NN)                                                                            \
    case NN:                                                                                      \
        step_kernel<T, P, NN><<<dim3((unsigned)(B * H * StepShape<P, NN>::S)), StepShape<P, NN>::NTH, 0, \
                                stream>>>(state, (const T *)x, dt, A, (const T *)Bm, (const T *)Cm, D,   \
                                          (T *)y, (int)H, (int)G);                                \
        break;
    switch (N) {
        SSD_STEP_N(16) SSD_STEP_N(32) SSD_STEP_N(64) SSD_STEP_N(128) SSD_STEP_N(256)
        default: return hipErrorInvalidValue;
    }
#undef SSD_STEP_N
    return hipGetLastError();
}

template <class T>
hipError_t launch_p(float *state, const void *x, const float *dt, const float *A, const void *Bm,
                    const void *Cm, const float *D, void *y, int64_t B, int64_t H, int64_t P,
                    int64_t G, int64_t N, hipStream_t stream) {
    switch (P) {
        case 16: return launch_n<T, 16>(state, x, dt, A, Bm, Cm, D, y, B, H, G, N, stream);
        case 32: return launch_n<T, 32>(state, x, dt, A, Bm, Cm, D, y, B, H, G, N, stream);
        case 64: return launch_n<T, 64>(state, x, dt, A, Bm, Cm, D, y, B, H, G, N, stream);
        case 128: return launch_n<T, 128>(state, x, dt, A, Bm, Cm, D, y, B, H, G, N, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_step(float *state, const void *x, const float *dt, const float *A,
                       const void *Bm, const void *Cm, const float *D, void *y,
                       int64_t B, int64_t H, int64_t P, int64_t G, int64_t N, int bf16,
                       hipStream_t stream) {
    return bf16 ? launch_p<ssd::bf16>(state, x, dt, A, Bm, Cm, D, y, B, H, P, G, N, stream)
                : launch_p<float>(state, x, dt, A, Bm, Cm, D, y, B, H, P, G, N, stream);
}

}  // namespace ssd
