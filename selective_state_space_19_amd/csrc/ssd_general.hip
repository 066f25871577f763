// ssd_general.hip -- Mamba-2 SSD, chunked, for any headdim and d_state up to
// 256, float32 or bfloat16 storage (the sizes the MFMA kernels of ssd.hip do
// not take).
//
// What it computes ("State-Space Model Optimization Patterns" page, section 2
// "State Space Duality" and section 9 "Chunked Computation"): per batch row
// b, head h (group g = h / (H/G)) and head channel p, with a scalar
// transition per head,
//     H[p,n] <- exp(dt_t*A_h) * H[p,n] + dt_t * x_t[p] * B_t[n]
//     y_t[p]  = (sum_n C_t[n] * H[p,n] + D_h * x_t[p]) * silu(z_t[p]),
// chunk by chunk: within a chunk of K tokens the outputs are the masked
// quadratic form plus the carried-in state,
//     y_i = sum_{j<=i} (C_i . B_j) exp(s_i - s_j) dt_j x_j + exp(s_i) C_i . H_in + D x_i,
// s the running sum of dt*A over the chunk, and the state passed to the next
// chunk is exp(s_end) H_in + sum_j exp(s_end - s_j) dt_j x_j B_j^T.
//
// Design: one workgroup (256 threads) per (b, head, 32 head channels) walks
// the sequence in chunks of K = 32 tokens with the fp32 state in LDS.  Per
// chunk it stages dt, x, B and C (as fp32), forms the running sum and the
// 32 x 32 masked score matrix, then the outputs, then the state update.  All
// arithmetic is plain fp32 on the VALU, so float32 inputs keep float32
// accuracy.  The chunk length of the call is a tile size that does not change
// the result beyond rounding; this path always uses 32.  Every exponent
// s_i - s_j (j <= i), s_i and s_end - s_j is <= 0 for A_h <= 0, so no factor
// exceeds 1.
#include "common.h"
#include "kernels.h"

namespace mssm {

namespace {

constexpr int kGK = 32;     // chunk length (tokens)
constexpr int kGP = 32;     // head channels per workgroup
constexpr int kGNMax = 256; // largest d_state

template <typename T>
__device__ __forceinline__ float ldx(const T* p) { return Elem<T>::load1(p); }

// Inclusive prefix sum of v over the 32 lanes of each half-wave (shuffles).
__device__ __forceinline__ float scan32(float v, int lane) {
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) {
        const float u = __shfl_up(v, o, 32);
        if ((lane & 31) >= o) v += u;
    }
    return v;
}

template <typename T>
__global__ __launch_bounds__(256) void ssd_general_kernel(
    const T* __restrict__ X, const T* __restrict__ DT, const float* __restrict__ Ah, const T* __restrict__ Bm,
    const T* __restrict__ Cm, const float* __restrict__ Dh, const T* __restrict__ Z, const float* __restrict__ h0,
    T* __restrict__ Y, float* __restrict__ hT, int L, int H, int P, int N, int G) {
    constexpr int NS = kGNMax + 1;                // row stride of B, C and the state (odd: no bank conflicts)
    __shared__ float sB[kGK][NS];
    __shared__ float sC[kGK][NS];
    __shared__ float sH[kGP][NS];                 // state H[p][n] of this workgroup's head channels
    __shared__ float sX[kGK][kGP + 1];            // x[j][p]
    __shared__ float sXw[kGK][kGP + 1];           // dt_j exp(s_end - s_j) x[j][p]
    __shared__ float sM[kGK][kGK + 1];            // masked scores
    __shared__ float sS[kGK], sDt[kGK];

    const int npt = (P + kGP - 1) / kGP;
    const int pt = blockIdx.x % npt;
    const int bh = blockIdx.x / npt;
    const int h = bh % H;
    const int64_t b = bh / H;
    const int g = h / (H / G);
    const int p0 = pt * kGP;
    const int np = min(kGP, P - p0);
    const int tid = threadIdx.x;
    const float a2 = Ah[h] * kLog2e;
    const float dskip = Dh ? Dh[h] : 0.f;

    const int64_t xrow = (int64_t)H * P;          // elements per token of x, y, z
    const int64_t brow = (int64_t)G * N;          // elements per token of B, C
    const T* xb = X + b * L * xrow + (int64_t)h * P + p0;
    const T* zb = Z ? Z + b * L * xrow + (int64_t)h * P + p0 : nullptr;
    T* yb = Y + b * L * xrow + (int64_t)h * P + p0;
    const T* Bb = Bm + b * L * brow + (int64_t)g * N;
    const T* Cb = Cm + b * L * brow + (int64_t)g * N;
    const T* dtb = DT + b * (int64_t)L * H + h;

    // state from h0 (or zero)
    for (int e = tid; e < kGP * N; e += 256) {
        const int p = e / N, n = e % N;
        sH[p][n] = (h0 && p < np) ? h0[((b * H + h) * (int64_t)P + p0 + p) * N + n] : 0.f;
    }

    for (int t0 = 0; t0 < L; t0 += kGK) {
        const int nt = min(kGK, L - t0);
        __syncthreads();                          // previous chunk done with every buffer
        // ---- stage: dt and the running sum (first half-wave), x, B, C ----
        if (tid < 32) {
            const float dt = tid < nt ? ldx(dtb + (int64_t)(t0 + tid) * H) : 0.f;
            const float s = scan32(dt * a2, tid);
            sDt[tid] = dt;
            sS[tid] = s;
        }
        for (int e = tid; e < kGK * kGP; e += 256) {
            const int j = e / kGP, p = e % kGP;
            sX[j][p] = (j < nt && p < np) ? ldx(xb + (int64_t)(t0 + j) * xrow + p) : 0.f;
        }
        for (int e = tid; e < kGK * N; e += 256) {
            const int j = e / N, n = e % N;
            const bool ok = j < nt;
            sB[j][n] = ok ? ldx(Bb + (int64_t)(t0 + j) * brow + n) : 0.f;
            sC[j][n] = ok ? ldx(Cb + (int64_t)(t0 + j) * brow + n) : 0.f;
        }
        __syncthreads();
        const float send = sS[kGK - 1];           // tokens past the end have dt = 0
        // ---- masked scores M[i][j] = (C_i . B_j) 2^(s_i - s_j) dt_j, j <= i; and the
        //      scaled inputs of the state update ----
        {
            const int i = tid >> 3;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int j = (tid & 7) + 8 * k;
                float acc = 0.f;
                if (j <= i) {
                    for (int n = 0; n < N; ++n) acc = fmaf(sC[i][n], sB[j][n], acc);
                    acc *= fast_exp2(sS[i] - sS[j]) * sDt[j];
                }
                sM[i][j] = acc;
            }
        }
        for (int e = tid; e < kGK * kGP; e += 256) {
            const int j = e / kGP, p = e % kGP;
            sXw[j][p] = sDt[j] * fast_exp2(send - sS[j]) * sX[j][p];
        }
        __syncthreads();
        // ---- outputs: row i, channels p = (tid & 7) + 8k ----
        {
            const int i = tid >> 3;
            const float ei = fast_exp2(sS[i]);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int p = (tid & 7) + 8 * k;
                float yd = 0.f, yo = 0.f;
                for (int j = 0; j <= i; ++j) yd = fmaf(sM[i][j], sX[j][p], yd);
                for (int n = 0; n < N; ++n) yo = fmaf(sC[i][n], sH[p][n], yo);
                float out = fmaf(ei, yo, yd) + dskip * sX[i][p];
                if (i < nt && p < np) {
                    const int64_t o = (int64_t)(t0 + i) * xrow + p;
                    if (zb) out *= silu(ldx(zb + o));
                    Elem<T>::store1(yb + o, out);
                }
            }
        }
        __syncthreads();                          // outputs have read the old state
        // ---- state update: H[p][n] = 2^send H[p][n] + sum_j xw[j][p] B[j][n] ----
        {
            const float ed = fast_exp2(send);
            for (int e = tid; e < kGP * N; e += 256) {
                const int p = e / N, n = e % N;
                float acc = 0.f;
#pragma unroll 8
                for (int j = 0; j < kGK; ++j) acc = fmaf(sXw[j][p], sB[j][n], acc);
                sH[p][n] = fmaf(ed, sH[p][n], acc);
            }
        }
    }
    __syncthreads();
    if (hT) {
        for (int e = tid; e < kGP * N; e += 256) {
            const int p = e / N, n = e % N;
            if (p < np) hT[((b * H + h) * (int64_t)P + p0 + p) * N + n] = sH[p][n];
        }
    }
}

}  // namespace

bool ssd_general_supported(int64_t P, int64_t N) { return P >= 1 && N >= 1 && N <= kGNMax; }

hipError_t launch_ssd_general(const SSDParams& p, bool is_bf16, hipStream_t stream) {
    const int64_t blocks = p.batch * p.H * ((p.P + kGP - 1) / kGP);
    if (is_bf16) {
        hipLaunchKernelGGL(ssd_general_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           static_cast<const uint16_t*>(p.x), static_cast<const uint16_t*>(p.dt), p.A,
                           static_cast<const uint16_t*>(p.Bm), static_cast<const uint16_t*>(p.Cm), p.Dskip,
                           static_cast<const uint16_t*>(p.z), p.h0, static_cast<uint16_t*>(p.y), p.h_final, p.L,
                           p.H, p.P, p.N, p.G);
    } else {
        hipLaunchKernelGGL(ssd_general_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           static_cast<const float*>(p.x), static_cast<const float*>(p.dt), p.A,
                           static_cast<const float*>(p.Bm), static_cast<const float*>(p.Cm), p.Dskip,
                           static_cast<const float*>(p.z), p.h0, static_cast<float*>(p.y), p.h_final, p.L, p.H,
                           p.P, p.N, p.G);
    }
    return hipGetLastError();
}

}  // namespace mssm
