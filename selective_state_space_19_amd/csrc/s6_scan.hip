// s6_scan.hip -- S6 selective scan forward for gfx950.
//
// What it computes (Mamba "Architecture Details" page, "Selective State
// Space Mechanism / How S6 Works"; SSM optimisation catalogue sections 6, 7
// and 3): per batch row b, channel d, state n, with h starting at h0 or 0,
//     h[n] <- exp(delta*A[d,n]) * h[n] + delta*u*B[b,n,t]
//     y     = (sum_n C[b,n,t]*h[n] + D[d]*u) * silu(z)
//
// Design (MI355X-first; the pages' warp/shared-memory notes are prior art):
// - The recurrence is elementwise in n, so the only dependency chain is over
//   time for a fixed (b, d, n).  There are B*D*N such chains (262 144 at the
//   Mamba-1.4B layer shape), enough to fill 256 CUs with one wave per SIMD
//   while every chain runs strictly in time order.  So instead of a
//   parallel-over-time scan (which costs a second pass and a cross-lane
//   combine per element), each lane walks time sequentially for NS states of
//   one channel: per element one exp2, two multiplies and two FMAs -- the
//   minimum the recurrence needs.  The fp32 state lives in registers for the
//   whole sequence and touches HBM only as h0 / h_final.
// - A workgroup (4 waves) owns CW = 64 channels of one batch row; wave g owns
//   the states [g*NS, (g+1)*NS).  The four partial outputs sum_n C*h of a
//   channel are combined through LDS once per token.
// - The sequence is processed in chunks of TC tokens.  Per chunk, all 256
//   threads load the u / delta / z / B / C tiles with 16-byte vector loads,
//   stage delta and delta*u (fp32) and the B / C tile (fp32, state-major) in
//   LDS, and prefetch the next chunk into registers while the waves scan.
//   B and C are shared by every channel, so a wave reads them with
//   uniform-address (broadcast) LDS loads.
// - The epilogue (combine partials, + D*u, * silu(z), convert, store) runs in
//   the same thread -> (channel, token range) mapping as the loads, so u and
//   z come straight from registers.
// - exp(delta*A) is computed as exp2(delta * (A*log2 e)) with A*log2 e
//   precomputed per lane (v_exp_f32).
#include "common.h"
#include "kernels.h"

namespace mssm {

namespace {

constexpr int kThreads = 256;

template <typename T, int CW, int NS, int TC>
__global__ __launch_bounds__(kThreads) void s6_scan_kernel(S6Params p) {
    constexpr int NG = kThreads / CW;              // state groups per workgroup
    constexpr int NP = NG * NS;                    // padded state count (>= N)
    constexpr int TPT = TC / NG;                   // tokens per thread (row mapping)
    constexpr int WPT = TPT * sizeof(T) / 4;       // 32-bit words per thread run
    constexpr int RB = 16 / sizeof(T);             // tokens per B/C load run (16 B)
    constexpr int BC_RUNS = NP * TC / RB;          // upper bound on B/C runs per matrix
    constexpr int BC_PER_THREAD = (BC_RUNS + kThreads - 1) / kThreads;
    static_assert(TPT * sizeof(T) % 16 == 0, "thread runs are whole vectors");

    __shared__ float2 s_dd[TC][CW];                // (delta, delta*u)
    __shared__ float4 s_bc4[2 * TC * NP / 4];      // B then C tiles, [TC][NP] each
    __shared__ float s_y[NG][TC][CW];              // partial outputs per state group
    float* s_B = reinterpret_cast<float*>(s_bc4);
    float* s_C = s_B + TC * NP;

    const int tid = threadIdx.x;
    const int c = tid % CW;                        // channel in block (both mappings)
    const int g = tid / CW;                        // state group / token block
    const int64_t nblk_d = (p.dim + CW - 1) / CW;
    const int64_t b = blockIdx.x / nblk_d;
    const int64_t d = (blockIdx.x % nblk_d) * CW + c;
    const bool dval = d < p.dim;
    const int L = p.L, N = p.N;
    const bool vec = (L % RB) == 0;                // rows are 16-byte aligned

    const int64_t row = (b * p.dim + (dval ? d : 0)) * (int64_t)L;
    const T* __restrict__ u_row = static_cast<const T*>(p.u) + row;
    const T* __restrict__ dl_row = static_cast<const T*>(p.delta) + row;
    const T* __restrict__ z_row = p.z ? static_cast<const T*>(p.z) + row : nullptr;
    T* __restrict__ y_row = static_cast<T*>(p.y) + row;
    const T* __restrict__ Bb = static_cast<const T*>(p.Bm) + b * (int64_t)N * L;
    const T* __restrict__ Cb = static_cast<const T*>(p.Cm) + b * (int64_t)N * L;

    // Padded states (n >= N) keep B = C = 0 for the whole kernel.
    for (int i = tid; i < TC * NP; i += kThreads) {
        if (i % NP >= N) {
            s_B[i] = 0.f;
            s_C[i] = 0.f;
        }
    }

    // Scan-side state: lane owns channel c, states g*NS + s.
    float h[NS], a2[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int n = g * NS + s;
        const bool ok = dval && n < N;
        a2[s] = ok ? p.A[d * N + n] * kLog2e : 0.f;
        h[s] = (ok && p.h0) ? p.h0[(b * p.dim + d) * N + n] : 0.f;
    }
    const float dskip = (dval && p.Dskip) ? p.Dskip[d] : 0.f;

    // Row-mapping registers: this thread's token run of u / delta / z.
    const int toff = g * TPT;
    uint32_t cu[WPT], cdl[WPT], cz[WPT];           // current chunk
    uint32_t nu[WPT], ndl[WPT], nz[WPT];           // next chunk (prefetch)
#pragma unroll
    for (int i = 0; i < WPT; ++i) cz[i] = nz[i] = 0u;
    uint32_t bcw[2][BC_PER_THREAD][4];             // B / C runs of the next chunk

    auto load_chunk = [&](int t0, uint32_t (&wu)[WPT], uint32_t (&wdl)[WPT], uint32_t (&wz)[WPT]) {
        const int valid = dval ? (L - t0 - toff) : 0;
        load_run<T, TPT>(u_row + t0 + toff, valid, vec, wu);
        load_run<T, TPT>(dl_row + t0 + toff, valid, vec, wdl);
        if (z_row) load_run<T, TPT>(z_row + t0 + toff, valid, vec, wz);
#pragma unroll
        for (int k = 0; k < BC_PER_THREAD; ++k) {
            const int r = tid + k * kThreads;
            const int n = r / (TC / RB);
            const int tt = (r % (TC / RB)) * RB;
            const int v = (n < N) ? (L - t0 - tt) : 0;
            const int64_t off = (int64_t)(n < N ? n : 0) * L + t0 + tt;
            load_run<T, RB>(Bb + off, v, vec, bcw[0][k]);
            load_run<T, RB>(Cb + off, v, vec, bcw[1][k]);
        }
    };

    const int nchunks = (L + TC - 1) / TC;
    load_chunk(0, cu, cdl, cz);

    for (int ck = 0; ck < nchunks; ++ck) {
        const int t0 = ck * TC;
        // ---- stage this chunk in LDS -------------------------------------
#pragma unroll
        for (int j = 0; j < TPT; ++j) {
            const float dlt = Elem<T>::get(cdl, j);
            s_dd[toff + j][c] = make_float2(dlt, dlt * Elem<T>::get(cu, j));
        }
#pragma unroll
        for (int k = 0; k < BC_PER_THREAD; ++k) {
            const int r = tid + k * kThreads;
            const int n = r / (TC / RB);
            const int tt = (r % (TC / RB)) * RB;
            if (n < N) {
#pragma unroll
                for (int j = 0; j < RB; ++j) {
                    s_B[(tt + j) * NP + n] = Elem<T>::get(bcw[0][k], j);
                    s_C[(tt + j) * NP + n] = Elem<T>::get(bcw[1][k], j);
                }
            }
        }
        // ---- prefetch the next chunk while this one is scanned -------------
        if (ck + 1 < nchunks) load_chunk(t0 + TC, nu, ndl, nz);
        __syncthreads();

        // ---- sequential scan of TC tokens, NS states per lane ---------------
#pragma unroll 4
        for (int t = 0; t < TC; ++t) {
            const float2 dd = s_dd[t][c];
            float bv[NS], cv[NS];
            const float4* bp = reinterpret_cast<const float4*>(s_B + t * NP + g * NS);
            const float4* cp = reinterpret_cast<const float4*>(s_C + t * NP + g * NS);
            if constexpr (NS % 4 == 0) {
#pragma unroll
                for (int q = 0; q < NS / 4; ++q) {
                    const float4 x = bp[q], w = cp[q];
                    bv[4 * q] = x.x; bv[4 * q + 1] = x.y; bv[4 * q + 2] = x.z; bv[4 * q + 3] = x.w;
                    cv[4 * q] = w.x; cv[4 * q + 1] = w.y; cv[4 * q + 2] = w.z; cv[4 * q + 3] = w.w;
                }
            } else {
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    bv[s] = s_B[t * NP + g * NS + s];
                    cv[s] = s_C[t * NP + g * NS + s];
                }
            }
            float yp = 0.f;
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const float dA = fast_exp2(dd.x * a2[s]);
                h[s] = fmaf(dA, h[s], dd.y * bv[s]);
                yp = fmaf(cv[s], h[s], yp);
            }
            s_y[g][t][c] = yp;
        }
        __syncthreads();

        // ---- epilogue: combine groups, skip term, gate, store ----------------
        {
            float out[TPT];
#pragma unroll
            for (int j = 0; j < TPT; ++j) {
                float acc = 0.f;
#pragma unroll
                for (int q = 0; q < NG; ++q) acc += s_y[q][toff + j][c];
                acc = fmaf(dskip, Elem<T>::get(cu, j), acc);
                if (z_row) acc *= silu(Elem<T>::get(cz, j));
                out[j] = acc;
            }
            if (dval) store_run<T, TPT>(y_row + t0 + toff, L - t0 - toff, vec, out);
        }
        // No barrier here: the epilogue reads only s_y, which the next chunk
        // rewrites after its first barrier; the next staging step writes only
        // s_dd / s_B / s_C, whose last readers finished before the barrier
        // above.
#pragma unroll
        for (int i = 0; i < WPT; ++i) {
            cu[i] = nu[i];
            cdl[i] = ndl[i];
            cz[i] = nz[i];
        }
    }

    if (p.h_final && dval) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const int n = g * NS + s;
            if (n < N) p.h_final[(b * p.dim + d) * N + n] = h[s];
        }
    }
}

template <typename T, int NS>
hipError_t launch_ns(const S6Params& p, hipStream_t stream) {
    constexpr int CW = 64, TC = 64;
    const int64_t blocks = ((p.dim + CW - 1) / CW) * p.batch;
    hipLaunchKernelGGL((s6_scan_kernel<T, CW, NS, TC>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const S6Params& p, hipStream_t stream) {
    if (p.N <= 4) return launch_ns<T, 1>(p, stream);
    if (p.N <= 8) return launch_ns<T, 2>(p, stream);
    if (p.N <= 16) return launch_ns<T, 4>(p, stream);
    if (p.N <= 32) return launch_ns<T, 8>(p, stream);
    return launch_ns<T, 16>(p, stream);
}

__global__ void copy_or_zero_kernel(float* dst, const float* src, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.f;
}

}  // namespace

hipError_t launch_s6_scan(const S6Params& p, bool is_bf16, hipStream_t stream) {
    return is_bf16 ? launch_t<uint16_t>(p, stream) : launch_t<float>(p, stream);
}

hipError_t launch_copy_or_zero(float* dst, const float* src, int64_t n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(copy_or_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, dst, src, n);
    return hipGetLastError();
}

}  // namespace mssm
