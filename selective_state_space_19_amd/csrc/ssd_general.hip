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
// chunk it stages dt, x, B and C (as fp32; rows of B, C and the state padded
// to whole float4s with zeros), forms the running sum, then three products,
// each thread holding a register tile so that one LDS read feeds several
// FMAs and its accumulators are independent chains:
//   scores  M = C B^T (lower 32 x 32 triangle, 2 x 2 per thread, float4 reads
//           along n), then masked and scaled by the decay and dt;
//   outputs Y = M X + diag(exp(s)) C H^T (2 tokens x 2 channels per thread);
//   state   H = exp(s_end) H + Xw^T B (4 channels x 4 states per thread).
// All arithmetic is plain fp32 on the VALU, so float32 inputs keep float32
// accuracy.  The chunk length of the call is a tile size that does not change
// the result beyond rounding; this path always uses 32.  Every exponent
// s_i - s_j (j <= i), s_i and s_end - s_j is <= 0 for A_h <= 0, so no factor
// exceeds 1.
#include "common.h"
#include "kernels.h"

namespace mssm {

namespace {

constexpr int kGK = 32;          // chunk length (tokens)
constexpr int kGP = 32;          // head channels per workgroup
constexpr int kGNMax = 256;      // largest d_state
constexpr int kRS = kGNMax + 4;  // LDS row stride (floats) of B, C and the state
constexpr int kXS = kGP + 4;     // LDS row stride (floats) of x and the scaled x

template <typename T>
__device__ __forceinline__ float ldx(const T* p) { return Elem<T>::load1(p); }

// Four consecutive elements as floats; `vec` says p is aligned to them.
__device__ __forceinline__ float4 ld4(const float* p, bool vec) {
    if (vec) return *reinterpret_cast<const float4*>(p);
    return make_float4(p[0], p[1], p[2], p[3]);
}
__device__ __forceinline__ float4 ld4(const uint16_t* p, bool vec) {
    if (vec) {
        const uint2 w = *reinterpret_cast<const uint2*>(p);
        return make_float4(bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y));
    }
    return make_float4(Elem<uint16_t>::load1(p), Elem<uint16_t>::load1(p + 1), Elem<uint16_t>::load1(p + 2),
                       Elem<uint16_t>::load1(p + 3));
}

// Inclusive prefix sum of v over the 32 lanes of each half-wave (shuffles).
__device__ __forceinline__ float scan32(float v, int lane) {
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) {
        const float u = __shfl_up(v, o, 32);
        if ((lane & 31) >= o) v += u;
    }
    return v;
}

__device__ __forceinline__ float dot4(float4 a, float4 b, float acc) {
    return fmaf(a.w, b.w, fmaf(a.z, b.z, fmaf(a.y, b.y, fmaf(a.x, b.x, acc))));
}

// VEC: B / C rows are whole aligned float4s (N a multiple of 4, aligned
// arrays); otherwise element loads.
template <typename T, bool VEC>
__global__ __launch_bounds__(256) void ssd_general_kernel(
    const T* __restrict__ X, const T* __restrict__ DT, const float* __restrict__ Ah, const T* __restrict__ Bm,
    const T* __restrict__ Cm, const float* __restrict__ Dh, const T* __restrict__ Z, const float* __restrict__ h0,
    T* __restrict__ Y, float* __restrict__ hT, int L, int H, int P, int N, int G) {
    __shared__ __align__(16) float sB[kGK][kRS];
    __shared__ __align__(16) float sC[kGK][kRS];
    __shared__ __align__(16) float sH[kGP][kRS];      // state H[p][n] of this workgroup's head channels
    __shared__ __align__(16) float sX[kGK][kXS];      // x[j][p]
    __shared__ __align__(16) float sXw[kGK][kXS];     // dt_j exp(s_end - s_j) x[j][p]
    __shared__ float sM[kGK][kGK + 1];                // masked scores
    __shared__ float sS[kGK], sDt[kGK];

    const int npt = (P + kGP - 1) / kGP;
    const int pt = blockIdx.x % npt;
    const int bh = blockIdx.x / npt;
    const int h = bh % H;
    const int64_t b = bh / H;
    const int g = h / (H / G);
    const int p0 = pt * kGP;
    const int np = min(kGP, P - p0);
    const int NP = (N + 3) & ~3;                      // state length in whole float4s
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

    // state from h0 (or zero); columns past N stay zero
    for (int e = tid; e < kGP * NP; e += 256) {
        const int p = e / NP, n = e % NP;
        sH[p][n] = (h0 && p < np && n < N) ? h0[((b * H + h) * (int64_t)P + p0 + p) * N + n] : 0.f;
    }

    // thread tiles: outputs 2 x 2 (tokens i0, i0 + 1; channels c0, c0 + 1), state 4 x 4
    const int i0 = 2 * (tid >> 4);
    const int c0 = 2 * (tid & 15);
    const int sp0 = 4 * (tid & 7);                // state channels sp0 .. sp0 + 3
    const int sn0 = 4 * (tid >> 3);               // state columns sn0 + 128 r .. + 3

    // The next chunk's dt, x, z, B and C are loaded into registers while this
    // one is computed.  Every load is issued unconditionally from a clamped
    // address (a branch around a load would make the compiler wait for all
    // loads in flight at the join) and kept raw; the values out of range are
    // replaced by 0 when they are staged, a chunk later (a select right after
    // the load could be rewritten as a load from a selected address, which
    // would put the zero in scratch memory).
    const int xj = tid >> 3, xp = 4 * (tid & 7);  // x: token xj, channels xp .. xp + 3
    const int bq = tid & 63;                      // B / C: float4 bq of rows (tid >> 6) + 4 m
    float r_dt = 0.f, r_x[4], r_z[2][2];
    float4 r_b[8], r_c[8];
    auto fetch = [&](int t0) {
        r_dt = ldx(dtb + (int64_t)min(t0 + tid, L - 1) * H);
        {
            const T* src = xb + (int64_t)min(t0 + xj, L - 1) * xrow;
#pragma unroll
            for (int k = 0; k < 4; ++k) r_x[k] = ldx(src + min(xp + k, np - 1));
        }
        if (zb) {                                 // the gate of this thread's outputs (a uniform branch)
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int c = 0; c < 2; ++c)
                    r_z[a][c] = ldx(zb + (int64_t)min(t0 + i0 + a, L - 1) * xrow + min(c0 + c, np - 1));
        }
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const int64_t ro = (int64_t)min(t0 + (tid >> 6) + 4 * m, L - 1) * brow;
            if constexpr (VEC) {
                const int64_t o = ro + min(4 * bq, NP - 4);
                r_b[m] = ld4(Bb + o, true);
                r_c[m] = ld4(Cb + o, true);
            } else {
                float eb[4], ec[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int64_t o = ro + min(4 * bq + k, N - 1);
                    eb[k] = ldx(Bb + o);
                    ec[k] = ldx(Cb + o);
                }
                r_b[m] = make_float4(eb[0], eb[1], eb[2], eb[3]);
                r_c[m] = make_float4(ec[0], ec[1], ec[2], ec[3]);
            }
        }
    };

    if (L > 0) fetch(0);
    for (int t0 = 0; t0 < L; t0 += kGK) {
        const int nt = min(kGK, L - t0);
        __syncthreads();                          // previous chunk done with every buffer
        // ---- stage: dt and the running sum (first half-wave), x, B, C ----
        if (tid < 32) {
            const float dt = tid < nt ? r_dt : 0.f;
            const float s = scan32(dt * a2, tid);
            sDt[tid] = dt;
            sS[tid] = s;
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) sX[xj][xp + k] = (xj < nt && xp + k < np) ? r_x[k] : 0.f;
        if (4 * bq < NP) {
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const int j = (tid >> 6) + 4 * m;
                float4 vb = r_b[m], vc = r_c[m];
                if (j >= nt) vb = vc = make_float4(0.f, 0.f, 0.f, 0.f);
                if constexpr (!VEC) {             // columns past N (VEC: N is a multiple of 4)
                    if (4 * bq + 1 > N) vb.x = vc.x = 0.f;
                    if (4 * bq + 2 > N) vb.y = vc.y = 0.f;
                    if (4 * bq + 3 > N) vb.z = vc.z = 0.f;
                    if (4 * bq + 4 > N) vb.w = vc.w = 0.f;
                }
                *reinterpret_cast<float4*>(&sB[j][4 * bq]) = vb;
                *reinterpret_cast<float4*>(&sC[j][4 * bq]) = vc;
            }
        }
        float z_cur[2][2];
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int c = 0; c < 2; ++c) z_cur[a][c] = zb ? r_z[a][c] : 0.f;
        if (t0 + kGK < L) fetch(t0 + kGK);
        __syncthreads();
        const float send = sS[kGK - 1];           // tokens past the end have dt = 0
        // ---- scores M[i][j] = (C_i . B_j) 2^(s_i - s_j) dt_j for j <= i, else 0 ----
        if (tid < 136) {                          // the 2 x 2 blocks on or below the diagonal
            int bi = (int)((sqrtf(8.f * tid + 1.f) - 1.f) * 0.5f);
            if ((bi + 1) * (bi + 2) / 2 <= tid) ++bi;   // guard the float root
            if (bi * (bi + 1) / 2 > tid) --bi;
            const int r0 = 2 * bi, q0 = 2 * (tid - bi * (bi + 1) / 2);
            float s00 = 0.f, s01 = 0.f, s10 = 0.f, s11 = 0.f;
            {
#pragma unroll 4
                for (int n = 0; n < NP; n += 4) {
                    const float4 ca = *reinterpret_cast<const float4*>(&sC[r0][n]);
                    const float4 cb = *reinterpret_cast<const float4*>(&sC[r0 + 1][n]);
                    const float4 ba = *reinterpret_cast<const float4*>(&sB[q0][n]);
                    const float4 bb = *reinterpret_cast<const float4*>(&sB[q0 + 1][n]);
                    s00 = dot4(ca, ba, s00);
                    s01 = dot4(ca, bb, s01);
                    s10 = dot4(cb, ba, s10);
                    s11 = dot4(cb, bb, s11);
                }
            }
            const float sv[2][2] = {{s00, s01}, {s10, s11}};
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    const int i = r0 + a, j = q0 + c;
                    sM[i][j] = j <= i ? sv[a][c] * fast_exp2(sS[i] - sS[j]) * sDt[j] : 0.f;
                }
        }
        {
            // scaled inputs of the state update (M above the diagonal is never
            // read, except inside the diagonal blocks, which are written)
            const int j = tid >> 3, p = 4 * (tid & 7);
            const float w = sDt[j] * fast_exp2(send - sS[j]);
            float4 v = *reinterpret_cast<const float4*>(&sX[j][p]);
            v.x *= w; v.y *= w; v.z *= w; v.w *= w;
            *reinterpret_cast<float4*>(&sXw[j][p]) = v;
        }
        __syncthreads();
        // ---- outputs: tokens i0, i0 + 1; channels c0, c0 + 1 ----
        {
            float yd[2][2] = {{0.f, 0.f}, {0.f, 0.f}}, yo[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
            for (int j = 0; j <= i0 + 1; ++j) {   // M is zero above the diagonal
                const float m0 = sM[i0][j], m1 = sM[i0 + 1][j];
                const float2 xx = *reinterpret_cast<const float2*>(&sX[j][c0]);
                yd[0][0] = fmaf(m0, xx.x, yd[0][0]);
                yd[0][1] = fmaf(m0, xx.y, yd[0][1]);
                yd[1][0] = fmaf(m1, xx.x, yd[1][0]);
                yd[1][1] = fmaf(m1, xx.y, yd[1][1]);
            }
#pragma unroll 4
            for (int n = 0; n < NP; n += 4) {
                const float4 ca = *reinterpret_cast<const float4*>(&sC[i0][n]);
                const float4 cb = *reinterpret_cast<const float4*>(&sC[i0 + 1][n]);
                const float4 ha = *reinterpret_cast<const float4*>(&sH[c0][n]);
                const float4 hb = *reinterpret_cast<const float4*>(&sH[c0 + 1][n]);
                yo[0][0] = dot4(ca, ha, yo[0][0]);
                yo[0][1] = dot4(ca, hb, yo[0][1]);
                yo[1][0] = dot4(cb, ha, yo[1][0]);
                yo[1][1] = dot4(cb, hb, yo[1][1]);
            }
#pragma unroll
            for (int a = 0; a < 2; ++a) {
                const int i = i0 + a;
                const float ei = fast_exp2(sS[i]);
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    const int p = c0 + c;
                    float out = fmaf(ei, yo[a][c], yd[a][c]) + dskip * sX[i][p];
                    if (zb) out *= silu(z_cur[a][c]);
                    if (i < nt && p < np) Elem<T>::store1(yb + (int64_t)(t0 + i) * xrow + p, out);
                }
            }
        }
        __syncthreads();                          // outputs have read the old state
        // ---- state update: H[p][n] = 2^send H[p][n] + sum_j xw[j][p] B[j][n] ----
        {
            const float ed = fast_exp2(send);
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int n = sn0 + 128 * r;
                if (n < NP) {
                    float acc[4][4] = {};
#pragma unroll 4
                    for (int j = 0; j < kGK; ++j) {
                        const float4 xw = *reinterpret_cast<const float4*>(&sXw[j][sp0]);
                        const float4 bv = *reinterpret_cast<const float4*>(&sB[j][n]);
                        const float xa[4] = {xw.x, xw.y, xw.z, xw.w};
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            acc[c][0] = fmaf(xa[c], bv.x, acc[c][0]);
                            acc[c][1] = fmaf(xa[c], bv.y, acc[c][1]);
                            acc[c][2] = fmaf(xa[c], bv.z, acc[c][2]);
                            acc[c][3] = fmaf(xa[c], bv.w, acc[c][3]);
                        }
                    }
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        float4* hp = reinterpret_cast<float4*>(&sH[sp0 + c][n]);
                        float4 hv = *hp;
                        hv.x = fmaf(ed, hv.x, acc[c][0]);
                        hv.y = fmaf(ed, hv.y, acc[c][1]);
                        hv.z = fmaf(ed, hv.z, acc[c][2]);
                        hv.w = fmaf(ed, hv.w, acc[c][3]);
                        *hp = hv;
                    }
                }
            }
        }
    }
    __syncthreads();
    if (hT) {
        for (int e = tid; e < kGP * NP; e += 256) {
            const int p = e / NP, n = e % NP;
            if (p < np && n < N) hT[((b * H + h) * (int64_t)P + p0 + p) * N + n] = sH[p][n];
        }
    }
}

}  // namespace

bool ssd_general_supported(int64_t P, int64_t N) { return P >= 1 && N >= 1 && N <= kGNMax; }

hipError_t launch_ssd_general(const SSDParams& p, bool is_bf16, hipStream_t stream) {
    const int64_t blocks = p.batch * p.H * ((p.P + kGP - 1) / kGP);
    const uintptr_t align = (is_bf16 ? 8 : 16) - 1;
    const bool vec = p.N % 4 == 0 && ((reinterpret_cast<uintptr_t>(p.Bm) | reinterpret_cast<uintptr_t>(p.Cm)) & align) == 0;
    if (is_bf16) {
        auto kern = vec ? ssd_general_kernel<uint16_t, true> : ssd_general_kernel<uint16_t, false>;
        hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), 0, stream,
                           static_cast<const uint16_t*>(p.x), static_cast<const uint16_t*>(p.dt), p.A,
                           static_cast<const uint16_t*>(p.Bm), static_cast<const uint16_t*>(p.Cm), p.Dskip,
                           static_cast<const uint16_t*>(p.z), p.h0, static_cast<uint16_t*>(p.y), p.h_final, p.L,
                           p.H, p.P, p.N, p.G);
    } else {
        auto kern = vec ? ssd_general_kernel<float, true> : ssd_general_kernel<float, false>;
        hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), 0, stream,
                           static_cast<const float*>(p.x), static_cast<const float*>(p.dt), p.A,
                           static_cast<const float*>(p.Bm), static_cast<const float*>(p.Cm), p.Dskip,
                           static_cast<const float*>(p.z), p.h0, static_cast<float*>(p.y), p.h_final, p.L, p.H,
                           p.P, p.N, p.G);
    }
    return hipGetLastError();
}

}  // namespace mssm
