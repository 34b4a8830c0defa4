// Reference chunk scan: float32 vector arithmetic, any supported shape, float32
// or bfloat16 storage.  Three kernels follow the block decomposition of the
// "Mamba-2 model walkthrough" (sections 6.1-6.2):
//
//   ref_block_state  each block's own state, S_c = sum_j w_j x_j (outer) Bm_j,
//                    w_j = exp(Lambda_end - Lambda_j) dt_j, and its total decay
//                    exp(Lambda_end), where Lambda is the in-block prefix sum of
//                    dt*A (the segment sums of the "segsum" helper);
//   ref_state_pass   the state entering every block, H_{c+1} = decay_c H_c + S_c,
//                    written over S_c in place, and the final state;
//   ref_block_output the diagonal block (Cm Bm^T masked by exp(Lambda_i -
//                    Lambda_j), times dt x) plus exp(Lambda_i) Cm_i H_c plus D x.
//
// This path is the float32 mode of the library and the baseline the
// matrix-core paths are checked against; it favours plainness over speed.
#include "common.h"

namespace ssd {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 16;     // tokens per staged tile
constexpr int kMaxQ = 256;
constexpr int kMaxP = 128;
constexpr int kMaxN = 256;

template <class T>
__global__ __launch_bounds__(kThreads) void ref_block_state(
    const T *__restrict__ x, const float *__restrict__ dt, const float *__restrict__ A,
    const T *__restrict__ Bm, float *__restrict__ states, float *__restrict__ decay,
    int64_t L, int64_t H, int64_t P, int64_t G, int64_t N, int64_t Q) {
    const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int nc = gridDim.x;
    const int64_t t0 = (int64_t)c * Q;
    const int q = (int)((L - t0) < Q ? (L - t0) : Q);
    const int g = (int)(h / (H / G));
    __shared__ float lam[kMaxQ], dts[kMaxQ], w[kMaxQ];
    __shared__ float xs[kTile][kMaxP];
    __shared__ float bs[kTile][kMaxN];

    block_prefix(dt + ((int64_t)b * L + t0) * H + h, H, q, q, A[h], lam, dts);
    const float lend = lam[q - 1];
    for (int j = threadIdx.x; j < q; j += kThreads) w[j] = expf(lend - lam[j]) * dts[j];
    __syncthreads();

    const int PN = (int)(P * N);
    float *out = states + (((int64_t)b * nc + c) * H + h) * PN;
    for (int e0 = 0; e0 < PN; e0 += kThreads * 8) {
        float acc[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) acc[r] = 0.f;
        for (int j0 = 0; j0 < q; j0 += kTile) {
            const int tj = (q - j0) < kTile ? (q - j0) : kTile;
            for (int k = threadIdx.x; k < kTile * P; k += kThreads) {
                const int jj = k / (int)P, p = k % (int)P;
                xs[jj][p] = jj < tj ? w[j0 + jj] * to_f32(x[(((int64_t)b * L + t0 + j0 + jj) * H + h) * P + p]) : 0.f;
            }
            for (int k = threadIdx.x; k < kTile * N; k += kThreads) {
                const int jj = k / (int)N, n = k % (int)N;
                bs[jj][n] = jj < tj ? to_f32(Bm[(((int64_t)b * L + t0 + j0 + jj) * G + g) * N + n]) : 0.f;
            }
            __syncthreads();
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const int e = e0 + r * kThreads + (int)threadIdx.x;
                if (e < PN) {
                    const int p = e / (int)N, n = e % (int)N;
                    float s = acc[r];
                    for (int jj = 0; jj < kTile; ++jj) s += xs[jj][p] * bs[jj][n];
                    acc[r] = s;
                }
            }
            __syncthreads();
        }
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int e = e0 + r * kThreads + (int)threadIdx.x;
            if (e < PN) out[e] = acc[r];
        }
    }
    if (threadIdx.x == 0) decay[((int64_t)b * H + h) * nc + c] = expf(lend);
}

__global__ __launch_bounds__(kThreads) void ref_state_pass(
    float *__restrict__ states, const float *__restrict__ decay, const float *init,
    float *final_state, int64_t H, int64_t PN, int nc) {
    const int64_t bh = blockIdx.y;
    const int64_t b = bh / H, h = bh % H;
    const int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (e >= PN) return;
    float s = init ? init[bh * PN + e] : 0.f;
    for (int c = 0; c < nc; ++c) {
        float *p = states + ((b * nc + c) * H + h) * PN + e;
        const float local = *p;
        *p = s;                                   // state entering block c
        s = decay[bh * nc + c] * s + local;
    }
    if (final_state) final_state[bh * PN + e] = s;  // same thread read init[e]: aliasing is safe
}

template <class T>
__global__ __launch_bounds__(kThreads) void ref_block_output(
    const T *__restrict__ x, const float *__restrict__ dt, const float *__restrict__ A,
    const T *__restrict__ Bm, const T *__restrict__ Cm, const float *__restrict__ D,
    const float *__restrict__ states, T *__restrict__ y,
    int64_t L, int64_t H, int64_t P, int64_t G, int64_t N, int64_t Q) {
    const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int nc = gridDim.x;
    const int64_t t0 = (int64_t)c * Q;
    const int q = (int)((L - t0) < Q ? (L - t0) : Q);
    const int g = (int)(h / (H / G));
    __shared__ float lam[kMaxQ], dts[kMaxQ];
    __shared__ float Gm[kTile][kMaxQ];
    __shared__ float cs[kTile][kMaxN];

    block_prefix(dt + ((int64_t)b * L + t0) * H + h, H, q, q, A[h], lam, dts);
    const float Dh = D[h];
    const float *Hc = states + (((int64_t)b * nc + c) * H + h) * P * N;
    const T *xb = x + (((int64_t)b * L + t0) * H + h) * P;     // token j at xb[j*H*P + p]
    const T *bb = Bm + (((int64_t)b * L + t0) * G + g) * N;    // token j at bb[j*G*N + n]
    const T *cb = Cm + (((int64_t)b * L + t0) * G + g) * N;
    T *yb = y + (((int64_t)b * L + t0) * H + h) * P;
    const int64_t xs = H * P, bsd = G * N;

    for (int i0 = 0; i0 < q; i0 += kTile) {
        const int ti = (q - i0) < kTile ? (q - i0) : kTile;
        for (int k = threadIdx.x; k < kTile * N; k += kThreads) {
            const int r = k / (int)N, n = k % (int)N;
            cs[r][n] = r < ti ? to_f32(cb[(int64_t)(i0 + r) * bsd + n]) : 0.f;
        }
        __syncthreads();
        const int jmax = i0 + ti;
        for (int k = threadIdx.x; k < kTile * jmax; k += kThreads) {
            const int r = k / jmax, j = k % jmax, i = i0 + r;
            float v = 0.f;
            if (r < ti && j <= i) {
                float dot = 0.f;
                for (int n = 0; n < N; ++n) dot += cs[r][n] * to_f32(bb[(int64_t)j * bsd + n]);
                v = dot * expf(lam[i] - lam[j]) * dts[j];
            }
            Gm[r][j] = v;
        }
        __syncthreads();
        for (int k = threadIdx.x; k < ti * P; k += kThreads) {
            const int r = k / (int)P, p = k % (int)P, i = i0 + r;
            float acc = 0.f;
            for (int j = 0; j <= i; ++j) acc += Gm[r][j] * to_f32(xb[(int64_t)j * xs + p]);
            float off = 0.f;
            for (int n = 0; n < N; ++n) off += cs[r][n] * Hc[(int64_t)p * N + n];
            const float xi = to_f32(xb[(int64_t)i * xs + p]);
            yb[(int64_t)i * xs + p] = from_f32<T>(acc + expf(lam[i]) * off + Dh * xi);
        }
        __syncthreads();
    }
}

template <class T>
hipError_t launch_typed(const ScanArgs &a, const Workspace &ws) {
    const int nc = (int)((a.L + a.Q - 1) / a.Q);
    const dim3 grid(nc, (unsigned)a.H, (unsigned)a.B);
    ref_block_state<T><<<grid, kThreads, 0, a.stream>>>(
        (const T *)a.x, a.dt, a.A, (const T *)a.Bm, ws.states, ws.decay, a.L, a.H, a.P, a.G, a.N, a.Q);
    const int64_t PN = a.P * a.N;
    const dim3 pgrid((unsigned)((PN + kThreads - 1) / kThreads), (unsigned)(a.B * a.H));
    ref_state_pass<<<pgrid, kThreads, 0, a.stream>>>(ws.states, ws.decay, a.init, a.final_state,
                                                      a.H, PN, nc);
    ref_block_output<T><<<grid, kThreads, 0, a.stream>>>(
        (const T *)a.x, a.dt, a.A, (const T *)a.Bm, (const T *)a.Cm, a.D, ws.states, (T *)a.y,
        a.L, a.H, a.P, a.G, a.N, a.Q);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_reference_scan(const ScanArgs &a, const Workspace &ws) {
    return a.bf16 ? launch_typed<bf16>(a, ws) : launch_typed<float>(a, ws);
}

}  // namespace ssd
