// s6_scan_bwd.hip -- backward of the S6 selective scan for gfx950.
//
// What it computes: the reverse-mode derivative of the scan in s6_scan.hip
// ("State-Space Model Optimization Patterns" page, section 4: the training
// pass recomputes the forward states instead of storing them all; the
// recurrence is that of the "Mamba Architecture Details" page, "Selective
// State Space Mechanism").  For the loss sum(dout * out) + sum(dhT * h_final),
// with g_t = dout_t * silu(z_t), a_t = exp(delta_t A) and the adjoint
// lambda_t = dL/dh_t taken backwards in time:
//     lambda_t = a_{t+1} lambda_{t+1} + g_t C_t      (dhT at the last token)
//     dC_t += g_t h_t,  dB_t += lambda_t delta_t u_t   (summed over channels)
//     du_t = g_t D + sum_n lambda_t delta_t B_t
//     ddelta_t = sum_n lambda_t (A a_t h_{t-1} + u_t B_t)
//     dA += lambda_t delta_t a_t h_{t-1},  dD += g_t u_t
//     dz_t = dout_t y_t silu'(z_t),  dh0 = a_0 lambda_0.
//
// Design (same mapping as the forward kernel): a workgroup of 8 waves owns 64
// channels of one batch row; lane = channel, wave w = states
// [w NS, (w+1) NS); B and C are wave-uniform (scalar operands).
//   1. Forward sweep over the whole sequence in chunks of TC tokens (16, or 8
//      when a lane holds more than 2 states), writing
//      the state at every chunk start to the workspace (one fp32 per
//      channel, state and chunk).
//   2. Backward sweep, last chunk first: stage (delta, delta*u, u, g) of the
//      chunk in LDS; recompute the chunk's TC states from its checkpoint into
//      registers (the per-wave partial outputs go to LDS, from which the row
//      threads form y and dz); then walk the chunk backwards, keeping lambda
//      in registers.  dB and dC are summed over the wave's 64 channels
//      (cross-lane butterfly) and added with one atomic per (state, token);
//      du and ddelta are summed over the waves through LDS by the row threads.
//   dA and dD are accumulated in registers and added with atomics at the end
//   (the entry point zeroes dA, dB, dC, dD first).
#include "common.h"
#include "kernels.h"

namespace mssm {

namespace {

constexpr int kNW = 8;                 // waves per workgroup
constexpr int kSegs = 8;               // row threads per channel

// Tokens per chunk: the chunk's states are held in registers (TC x NS).
template <int NS> struct ChunkLen { static constexpr int value = NS <= 2 ? 16 : 8; };

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

template <typename T, int NS, bool ALIGNED>
__global__ __launch_bounds__(kNW * 64) void s6_scan_bwd_kernel(S6BwdParams p) {
    constexpr int kTC = ChunkLen<NS>::value;
    constexpr int kTPT = kTC / kSegs;      // tokens per row thread
    __shared__ float4 s_tk[kTC][64 + 1];          // (delta, delta*u, u, g) per token and channel
    __shared__ float s_y[kNW][kTC][64 + 1];       // per-wave partial sum_n C h
    __shared__ float2 s_p[kNW][kTC][64 + 1];      // per-wave partial (du, ddelta)

    const T* u_in = static_cast<const T*>(p.u);
    const T* dl_in = static_cast<const T*>(p.delta);
    const T* z_in = static_cast<const T*>(p.z);
    const T* go_in = static_cast<const T*>(p.dout);
    const T* __restrict__ B_in = static_cast<const T*>(p.Bm);
    const T* __restrict__ C_in = static_cast<const T*>(p.Cm);
    const int64_t dim = p.dim;
    const int L = p.L, N = p.N;
    const int nck = (L + kTC - 1) / kTC;

    const int tid = threadIdx.x;
    const int64_t nblk_d = (dim + 63) / 64;
    const int64_t b = blockIdx.x / nblk_d;
    const int64_t d0 = (blockIdx.x % nblk_d) * 64;
    const int nrows = (int)((dim - d0) < 64 ? (dim - d0) : 64);

    // ---- scan mapping: lane = channel cs, wave = state group w ----------------
    const int cs = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool cval = cs < nrows;
    const int64_t ch = b * dim + d0 + (cval ? cs : 0);            // (b, d) of this lane
    float a2[NS], Af[NS], h[NS], lam[NS], dAacc[NS];
    int nst[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int n = w * NS + s;
        nst[s] = n < N ? n : 0;
        const bool ok = cval && n < N;
        Af[s] = ok ? p.A[(d0 + cs) * N + n] : 0.f;
        a2[s] = Af[s] * kLog2e;
        h[s] = (ok && p.h0) ? p.h0[ch * N + n] : 0.f;
        lam[s] = (ok && p.dhT) ? p.dhT[ch * N + n] : 0.f;
        dAacc[s] = 0.f;
    }
    // B / C of this wave's states over one chunk (0 past the end or for a
    // state past N).  ALIGNED (L % 8 == 0) and a whole chunk: one vector load
    // per state row; otherwise element by element.
    float Bf[NS][kTC], Cf[NS][kTC];
    auto load_bc = [&](int t0) {
        const bool vec = ALIGNED && t0 + kTC <= L;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const int n = w * NS + s;
            const T* pb = B_in + (b * N + nst[s]) * (int64_t)L + t0;
            const T* pc = C_in + (b * N + nst[s]) * (int64_t)L + t0;
            if (vec) {
                constexpr int NW4 = kTC * (int)sizeof(T) / 16;        // 16-byte words per chunk row
                uint32_t wb[NW4 * 4], wc[NW4 * 4];
#pragma unroll
                for (int q = 0; q < NW4; ++q) {
                    const uint4 x = reinterpret_cast<const uint4*>(pb)[q];
                    const uint4 y = reinterpret_cast<const uint4*>(pc)[q];
                    wb[4 * q] = x.x; wb[4 * q + 1] = x.y; wb[4 * q + 2] = x.z; wb[4 * q + 3] = x.w;
                    wc[4 * q] = y.x; wc[4 * q + 1] = y.y; wc[4 * q + 2] = y.z; wc[4 * q + 3] = y.w;
                }
#pragma unroll
                for (int k = 0; k < kTC; ++k) {
                    Bf[s][k] = n < N ? Elem<T>::get(wb, k) : 0.f;
                    Cf[s][k] = n < N ? Elem<T>::get(wc, k) : 0.f;
                }
            } else {
#pragma unroll
                for (int k = 0; k < kTC; ++k) {
                    const bool ok = n < N && t0 + k < L;
                    Bf[s][k] = ok ? Elem<T>::load1(pb + (ok ? k : 0)) : 0.f;
                    Cf[s][k] = ok ? Elem<T>::load1(pc + (ok ? k : 0)) : 0.f;
                }
            }
        }
    };
    // checkpoint of state s at the start of chunk ck
    auto ckpt = [&](int ck, int s) -> float* {
        return p.ws + ((b * nck + ck) * (int64_t)N + w * NS + s) * dim + d0 + cs;
    };

    // ---- row mapping: thread -> (row cr, tokens [toff, toff + kTPT)) ----------
    const int cr = tid / kSegs;
    const int seg = tid % kSegs;
    const int toff = seg * kTPT;
    const bool rval = cr < nrows;
    const int64_t rrow = (b * dim + d0 + (rval ? cr : 0)) * (int64_t)L;   // first element of this row
    const float dskip = (rval && p.Dskip) ? p.Dskip[d0 + cr] : 0.f;
    auto ld = [&](const T* base, int t) -> float { return (rval && t < L) ? Elem<T>::load1(base + rrow + t) : 0.f; };

    // ================= 1. forward sweep: chunk-start checkpoints =================
    for (int ck = 0; ck < nck; ++ck) {
        const int t0 = ck * kTC;
#pragma unroll
        for (int j = 0; j < kTPT; ++j) {
            const int t = t0 + toff + j;
            const float dl = ld(dl_in, t), uu = ld(u_in, t);
            s_tk[toff + j][cr] = make_float4(dl, dl * uu, 0.f, 0.f);
        }
        if (cval) {
#pragma unroll
            for (int s = 0; s < NS; ++s)
                if (w * NS + s < N) *ckpt(ck, s) = h[s];
        }
        load_bc(t0);
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kTC; ++k) {
            const float4 q = s_tk[k][cs];
#pragma unroll
            for (int s = 0; s < NS; ++s) h[s] = fmaf(fast_exp2(q.x * a2[s]), h[s], q.y * Bf[s][k]);
        }
        __syncthreads();
    }

    // ================= 2. backward sweep, last chunk first =======================
    float dDacc = 0.f;
    for (int ck = nck - 1; ck >= 0; --ck) {
        const int t0 = ck * kTC;
        // stage (delta, delta*u, u, g) -- the row thread keeps its own tokens
        float uu[kTPT], zz[kTPT], go[kTPT], gg[kTPT];
#pragma unroll
        for (int j = 0; j < kTPT; ++j) {
            const int t = t0 + toff + j;
            const float dl = ld(dl_in, t);
            uu[j] = ld(u_in, t);
            go[j] = ld(go_in, t);
            zz[j] = z_in ? ld(z_in, t) : 0.f;
            gg[j] = z_in ? go[j] * silu(zz[j]) : go[j];
            s_tk[toff + j][cr] = make_float4(dl, dl * uu[j], uu[j], gg[j]);
        }
        float hc[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) hc[s] = (cval && w * NS + s < N) ? *ckpt(ck, s) : 0.f;
        load_bc(t0);
        __syncthreads();

        // recompute the chunk's states; per-wave partial outputs to LDS
        float hs[kTC][NS];
        {
            float hh[NS];
#pragma unroll
            for (int s = 0; s < NS; ++s) hh[s] = hc[s];
#pragma unroll
            for (int k = 0; k < kTC; ++k) {
                const float4 q = s_tk[k][cs];
                float yp = 0.f;
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    hh[s] = fmaf(fast_exp2(q.x * a2[s]), hh[s], q.y * Bf[s][k]);
                    hs[k][s] = hh[s];
                    yp = fmaf(Cf[s][k], hh[s], yp);
                }
                s_y[w][k][cs] = yp;
            }
        }
        __syncthreads();

        // row threads: y, dz, dD
#pragma unroll
        for (int j = 0; j < kTPT; ++j) {
            const int t = t0 + toff + j;
            float y = dskip * uu[j];
#pragma unroll
            for (int q = 0; q < kNW; ++q) y += s_y[q][toff + j][cr];
            if (z_in && rval && t < L) {
                const float e = fast_exp2(-zz[j] * kLog2e);
                const float sg = __builtin_amdgcn_rcpf(1.f + e);
                Elem<T>::store1(static_cast<T*>(p.dz) + rrow + t, go[j] * y * (sg * (1.f + zz[j] * (1.f - sg))));
            }
            dDacc = fmaf(gg[j], uu[j], dDacc);
        }

        // walk the chunk backwards
#pragma unroll
        for (int k = kTC - 1; k >= 0; --k) {
            const float4 q = s_tk[k][cs];
            const int t = t0 + k;
            float dup = 0.f, ddp = 0.f;
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const float bv = Bf[s][k], cv = Cf[s][k];
                const float lt = fmaf(q.w, cv, lam[s]);
                const float hp = k > 0 ? hs[k > 0 ? k - 1 : 0][s] : hc[s];
                const float a = fast_exp2(q.x * a2[s]);
                const float dBp = wave_sum(lt * q.y);
                const float dCp = wave_sum(q.w * hs[k][s]);
                const int n = w * NS + s;
                if (cs == 0 && n < N && t < L) {
                    atomicAdd(p.dB + (b * N + n) * (int64_t)L + t, dBp);
                    atomicAdd(p.dC + (b * N + n) * (int64_t)L + t, dCp);
                }
                dup = fmaf(lt * q.x, bv, dup);
                ddp = fmaf(lt, fmaf(Af[s] * a, hp, q.z * bv), ddp);
                dAacc[s] = fmaf(lt * q.x * a, hp, dAacc[s]);
                lam[s] = a * lt;
            }
            s_p[w][k][cs] = make_float2(dup, ddp);
        }
        __syncthreads();

        // row threads: du, ddelta
#pragma unroll
        for (int j = 0; j < kTPT; ++j) {
            const int t = t0 + toff + j;
            float du = gg[j] * dskip, dd = 0.f;
#pragma unroll
            for (int q = 0; q < kNW; ++q) {
                const float2 v = s_p[q][toff + j][cr];
                du += v.x;
                dd += v.y;
            }
            if (rval && t < L) {
                Elem<T>::store1(static_cast<T*>(p.du) + rrow + t, du);
                Elem<T>::store1(static_cast<T*>(p.ddelta) + rrow + t, dd);
            }
        }
    }

    // ---- ends: dh0, dA, dD -------------------------------------------------------
    if (cval) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const int n = w * NS + s;
            if (n < N) {
                if (p.dh0) p.dh0[ch * N + n] = lam[s];
                atomicAdd(p.dA + (d0 + cs) * N + n, dAacc[s]);
            }
        }
    }
    // dD: the 8 row threads of a channel hold partials over their tokens
#pragma unroll
    for (int m = 1; m < kSegs; m <<= 1) dDacc += __shfl_xor(dDacc, m, 64);
    if (rval && seg == 0 && p.dD) atomicAdd(p.dD + d0 + cr, dDacc);
}

__global__ void zero_kernel(float* a, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) a[i] = 0.f;
}

hipError_t zero(float* a, int64_t n, hipStream_t stream) {
    if (!a || n <= 0) return hipSuccess;
    const int64_t blocks = (n + 255) / 256;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a, n);
    return hipGetLastError();
}

template <typename T, int NS>
hipError_t launch_ns(const S6BwdParams& p, hipStream_t stream) {
    const int64_t blocks = ((p.dim + 63) / 64) * p.batch;
    if (p.L % 8 == 0)
        hipLaunchKernelGGL((s6_scan_bwd_kernel<T, NS, true>), dim3((unsigned)blocks), dim3(kNW * 64), 0, stream, p);
    else
        hipLaunchKernelGGL((s6_scan_bwd_kernel<T, NS, false>), dim3((unsigned)blocks), dim3(kNW * 64), 0, stream, p);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const S6BwdParams& p, hipStream_t stream) {
    if (p.N <= 8) return launch_ns<T, 1>(p, stream);
    if (p.N <= 16) return launch_ns<T, 2>(p, stream);
    if (p.N <= 32) return launch_ns<T, 4>(p, stream);
    return launch_ns<T, 8>(p, stream);
}

}  // namespace

size_t s6_bwd_workspace_bytes(int64_t batch, int64_t dim, int64_t L, int64_t N) {
    const int tc = N <= 16 ? ChunkLen<2>::value : ChunkLen<4>::value;   // NS <= 2 iff N <= 16
    const int64_t nck = (L + tc - 1) / tc;
    return (size_t)(batch * nck * N * dim) * sizeof(float);
}

hipError_t launch_s6_scan_bwd(const S6BwdParams& p, bool is_bf16, hipStream_t stream) {
    hipError_t e;
    if ((e = zero(p.dA, p.dim * p.N, stream)) != hipSuccess) return e;
    if ((e = zero(p.dB, p.batch * p.N * (int64_t)p.L, stream)) != hipSuccess) return e;
    if ((e = zero(p.dC, p.batch * p.N * (int64_t)p.L, stream)) != hipSuccess) return e;
    if ((e = zero(p.dD, p.dD ? p.dim : 0, stream)) != hipSuccess) return e;
    return is_bf16 ? launch_t<uint16_t>(p, stream) : launch_t<float>(p, stream);
}

}  // namespace mssm
