// s6_scan.hip -- S6 selective scan forward for gfx950.
//
// What it computes ("Mamba Architecture Details" page, "Selective State
// Space Mechanism / How S6 Works"; "State-Space Model Optimization Patterns" page sections 6, 7
// and 3): per batch row b, channel d, state n, with h starting at h0 or 0,
//     h[n] <- exp(delta*A[d,n]) * h[n] + delta*u*B[b,n,t]
//     y     = (sum_n C[b,n,t]*h[n] + D[d]*u) * silu(z)
//
// Design (MI355X-first; the pages' warp / shared-memory notes are prior art):
// - The recurrence is elementwise in n, so the only dependency chain is over
//   time for a fixed (b, d, n); there are B*D*N such chains (262 144 at the
//   Mamba-1.4B layer shape).  Each lane walks time strictly in order for NS
//   states of one channel: per state element one v_exp_f32, two multiplies
//   and two FMAs -- the least the recurrence needs (a parallel-over-time scan
//   would add a second pass and a cross-lane combine per element).  The fp32
//   state lives in registers for the whole sequence and reaches HBM only as
//   h0 / h_final.
// - A workgroup owns 64 channels of one batch row and has two roles:
//   * 8 scan waves: lanes are channels, wave w owns the states
//     [w*NS, (w+1)*NS).  B and C are shared by all channels, so within a
//     wave they are uniform: they are fetched with scalar loads into SGPRs
//     (bf16 unpacked on the scalar unit) and used as free scalar operands.
//   * 4 row waves: thread = (row, TPT-token segment of the chunk), a row's
//     segments on consecutive lanes, so each load or store instruction moves
//     whole 64-byte row runs.  They stream u, delta, z through a register
//     ring (the loads of the next chunks in flight; in bf16 the two chunks
//     that share each 128-byte line are loaded back to back), stage
//     (delta, delta*u) in LDS for the scan, and run the epilogue: the sum of
//     the 8 per-wave partial outputs sum_n C*h, the D*u term, the silu(z)
//     gate and the y store (streaming cache policy).
//   Time is processed in chunks of TC tokens, the LDS buffers are doubled by
//   chunk parity, and one barrier per chunk hands work between the roles:
//   while the scan waves scan chunk k, the row waves finish chunk k-1 and
//   stage chunk k+1.  Each SIMD holds two scan waves and one row wave, so
//   the row work fills issue slots the scan leaves idle.
// - Inside a chunk the scan runs token groups of 32 bytes of a B / C row,
//   software-pipelined: the next group's scalar B / C loads and LDS
//   (delta, delta*u) loads are issued before the current group is computed
//   and waited for after it (scalar loads complete out of order, so every
//   wait drains them all; a longer group gives each load more cover).
// - exp(delta*A) is computed as exp2(delta * (A*log2 e)) with A*log2 e
//   precomputed per lane.
// - ALIGNED (L a multiple of a group; the common case) addresses rows
//   through range-checked buffer resources: loads past the end read zero and
//   stores there are dropped, so the hot loops have no bounds branches and
//   every load is issued unconditionally.  Other lengths take the same
//   arithmetic with element-wise bounds checks.
#include "common.h"
#include "kernels.h"

namespace mssm {

namespace {

struct alignas(16) Words8 { uint32_t w[8]; };   // bases are 16-byte aligned

// The zero-order-hold input factor (exp(delta*A) - 1) / A, given delta,
// x2 = delta * A * log2(e), e = exp2(x2) and ia = 1/A (0 where A = 0); the
// hold input term is u * B times this.
// - |x2| >= kHoldSwitch2 (|delta*A| >= 1/32): (e - 1) * ia as one fma, so
//   e - 1 is never rounded on its own.  The rounding of e (about 6e-8 near
//   1) moves the factor by at most ~2e-6 relative at the switch, less beyond.
// - below it: delta * (1 + x/2 + x^2/6) for x = delta*A, written in x2; the
//   first dropped term, x^3/24, is under 1.3e-6 relative there.  At A = 0
//   (or delta = 0) this gives exactly delta, the Euler factor.
// Per state element that is one fma, a degree-2 series (two fma and a mul),
// a compare and a select: no division and no second transcendental.
constexpr float kHoldSwitch2 = kLog2e / 32.f;
constexpr float kHold1 = kLn2 / 2.f;              // x/2 in powers of x2
constexpr float kHold2 = kLn2 * kLn2 / 6.f;       // x^2/6 in powers of x2
__device__ __forceinline__ float zoh_factor(float dl, float x2, float e, float ia) {
    const float direct = fmaf(e, ia, -ia);
    const float series = dl * fmaf(x2, fmaf(x2, kHold2, kHold1), 1.f);
    return fabsf(x2) < kHoldSwitch2 ? series : direct;
}

constexpr int kScanWaves = 8;     // waves running the recurrence
constexpr int kRowWaves = 4;      // waves streaming rows: loads, staging, epilogue
// Row-wave register ring (slots of chunk loads).  A chunk's row run is
// TC * sizeof(T) bytes; when that is half a 128-byte line (bf16) the loads
// of two chunks -- the two halves of each line -- are issued back to back,
// so a line is fetched from HBM once rather than once per half when it is
// evicted from L2 between the two uses.  That needs two more slots.
template <typename T, int TC> constexpr int kRing = TC * int(sizeof(T)) < 128 ? 6 : 4;

// Tokens between the saved states the backward pass starts its chunks from
// (its chunk length: 16 with up to 2 states per lane, else 8).
template <int NS> constexpr int kCkptLen = NS <= 2 ? 16 : 8;

template <typename T, int NS, int TC, bool ALIGNED, bool FULLN, bool FUSED, bool ZOH, bool CKPT, bool NOY, int RING>
__global__ __launch_bounds__((kScanWaves + kRowWaves) * 64) void s6_scan_kernel(
    const T* __restrict__ u_in, const T* __restrict__ dl_in, const T* __restrict__ B_in,
    const T* __restrict__ C_in, const T* __restrict__ z_in, const float* __restrict__ A_in,
    const float* __restrict__ D_in, const float* __restrict__ h0_in, T* __restrict__ y_out,
    float* __restrict__ hT_out, int64_t dim, int L, int N, S6FrontEnd fe, float* __restrict__ ck_out) {
    // FUSED: u_in is x before the causal conv and dl_in the step before
    // softplus; the row waves form u = silu(conv(x)) and delta =
    // softplus(raw + bias) while staging.  ZOH: the input term is the
    // zero-order hold (exp(delta*A) - 1) / A * u * B instead of delta * u * B
    // ("State-Space Model Optimization Patterns" page, section 7).  CKPT: the
    // scan waves also store the state at every kCkptLen-th token (before it
    // is applied) for the backward pass, which then need not re-run the
    // recurrence to find its chunk starts ("State-Space Model Optimization
    // Patterns" page, section 4: recompute within chunks from saved states).
    // NOY (with CKPT): the saved states are the only output -- no C, no
    // partial outputs, no z, no epilogue; the backward pass's own call runs
    // this ahead of its chunked sweep.
    // Pointers are separate __restrict__ arguments so the compiler may fetch the
    // wave-uniform B / C words with scalar loads (it must know no store aliases them).
    constexpr int NW = kScanWaves;
    constexpr int SEGS = kRowWaves;                // row threads per row (64 rows x SEGS = the row waves)
    constexpr int TPT = TC / SEGS;                 // tokens per row thread
    constexpr int WPT = TPT * sizeof(T) / 4;       // 32-bit words per thread run
    constexpr int G = 32 / sizeof(T);              // tokens per scan group: 32 bytes of a B / C row
    constexpr int NGRP = TC / G;
    constexpr int BCW = 8;                         // words per B / C row per group
    constexpr int PR = TC / 2;                     // token pairs per chunk
    constexpr int QR = TC / 4;                     // token quads per chunk
    static_assert(TPT % 4 == 0 && (WPT == 2 || WPT == 4 || WPT == 8), "row runs are 8-, 16- or 32-byte vectors");
    static_assert(TC % G == 0 && NGRP % 2 == 0, "whole scan groups per chunk, even count");
    constexpr bool PAIR = TC * int(sizeof(T)) < 128;  // loads of chunk pairs: whole 128-byte lines
    static_assert(RING >= 4 && RING % 2 == 0 && (!PAIR || RING >= 6),
                  "ring: stage, epilogue and reload use distinct slots; pairs need two more");

    // Double-buffered by chunk parity, 16 bytes per (channel, token pair or
    // quad).  The scan waves access one pair / quad per instruction with the
    // 64 channels on consecutive lanes; each quarter-wave of a row wave covers
    // 16 channels of one pair / quad.  Both are free of bank conflicts with
    // the plain layout, and the scan side needs no address arithmetic.
    __shared__ float4 s_dd[2][PR][64];             // (delta_t, (delta*u)_t, delta_t+1, (delta*u)_t+1); ZOH: u for delta*u
    __shared__ float4 s_y[2][NW][QR][64];          // per-scan-wave partial outputs, token quads

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t nblk_d = (dim + 63) / 64;
    // Blocks are dispatched round-robin over the 8 XCDs; number them so that
    // consecutive ids (channel blocks of one batch row, which read the same
    // B and C rows) share an XCD and its L2.
    uint32_t lid = blockIdx.x;
    if ((gridDim.x & 7u) == 0u) lid = (blockIdx.x & 7u) * (gridDim.x >> 3) + (blockIdx.x >> 3);
    const int64_t b = lid / nblk_d;
    const int64_t dblk = lid % nblk_d;
    const int64_t d0 = dblk * 64;
    const int nrows = (int)((dim - d0) < 64 ? (dim - d0) : 64);
    // The scan waves run one iteration per chunk and the row waves one more
    // (the last epilogue); each iteration starts at a barrier.
    const int nit = (L + TC - 1) / TC;

    if (wave < NW) {
        // ================= scan role: lane = channel cs, wave = state group w =================
        const int cs = tid & 63;
        const int w = wave;
        const bool sval_d = cs < nrows;
        const T* brow[NS];
        const T* crow[NS];
        bool sval[NS];
        float h[NS], a2[NS], ia[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const int n = w * NS + s;
            sval[s] = n < N;
            const int64_t off = (b * N + (sval[s] ? n : 0)) * (int64_t)L;
            brow[s] = B_in + off;
            crow[s] = C_in + off;
            const bool ok = sval_d && sval[s];
            const float af = ok ? A_in[(d0 + cs) * N + n] : 0.f;
            a2[s] = af * kLog2e;
            ia[s] = af != 0.f ? 1.f / af : 0.f;       // hold form only
            h[s] = (ok && h0_in) ? h0_in[(b * dim + d0 + cs) * N + n] : 0.f;
        }

        // B / C words of one group, for NS states (scalar registers).  ALIGNED:
        // a group is either inside the sequence or wholly past it; a group past
        // it re-reads the last group (finite data times a zero step: no effect).
        // A state past N gets C = 0, so it adds nothing to y.
        auto load_bc = [&](int t, uint32_t (&bw)[NS][BCW], uint32_t (&cw)[NS][BCW]) {
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                if constexpr (ALIGNED) {
                    const int tc = t < L ? t : L - G;
                    // Raw words (one 32-byte scalar load per row): a state past
                    // N is zeroed where C is used, after the group's wait, so
                    // these loads stay in flight meanwhile.
                    const Words8 x = *reinterpret_cast<const Words8*>(brow[s] + tc);
#pragma unroll
                    for (int i = 0; i < BCW; ++i) bw[s][i] = x.w[i];
                    if constexpr (!NOY) {
                        const Words8 y = *reinterpret_cast<const Words8*>(crow[s] + tc);
#pragma unroll
                        for (int i = 0; i < BCW; ++i) cw[s][i] = y.w[i];
                    }
                } else {
                    const int valid = sval[s] ? L - t : 0;
                    load_run<T, G>(brow[s] + t, valid, false, bw[s]);
                    if constexpr (!NOY) load_run<T, G>(crow[s] + t, valid, false, cw[s]);
                }
            }
        };

        uint32_t bw[2][NS][BCW], cw[2][NS][BCW];
        float4 ddr[2][G / 2];
        // CKPT: this batch row's saved states, [chunk, N, dim] fp32 (the host
        // keeps them under 2 GiB); a lane's own offset, out of range if idle
        const int64_t ck_row = CKPT ? (int64_t)((L + kCkptLen<NS> - 1) / kCkptLen<NS>) * N * dim : 0;
        const rsrc_t rck = make_rsrc(CKPT ? ck_out + b * ck_row : h0_in, (uint32_t)(ck_row * 4));
        const uint32_t ck_lane = sval_d ? (uint32_t)cs * 4u : kOutOfRange;

        // C of state s at token k of the group in buffer `buf`; 0 for a state
        // past N (FULLN: every state of every wave is below N).
        auto cval = [&](int buf, int s, int k) -> float {
            const float c = Elem<T>::get(cw[buf][s], k);
            if constexpr (ALIGNED && !FULLN) return sval[s] ? c : 0.f;
            return c;
        };
        // One group of G tokens in buffer `buf`, all NS states.  The decay
        // factors and input terms of the whole group are formed first (they do
        // not depend on h), so each exp has independent work behind it; then the
        // recurrence runs token by token.
        auto group = [&](int buf, int gi, int par, int tg) {
            float dA[G][NS], bu[G][NS];
#pragma unroll
            for (int k = 0; k < G; k += 2) {
                const float4 q = ddr[buf][k / 2];
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    const float x0 = q.x * a2[s], x1 = q.z * a2[s];
                    dA[k][s] = fast_exp2(x0);
                    dA[k + 1][s] = fast_exp2(x1);
                    if constexpr (ZOH) {
                        // staged (delta, u) pairs: the hold factor times u * B
                        bu[k][s] = zoh_factor(q.x, x0, dA[k][s], ia[s]) * (q.y * Elem<T>::get(bw[buf][s], k));
                        bu[k + 1][s] =
                            zoh_factor(q.z, x1, dA[k + 1][s], ia[s]) * (q.w * Elem<T>::get(bw[buf][s], k + 1));
                    } else {
                        bu[k][s] = q.y * Elem<T>::get(bw[buf][s], k);
                        bu[k + 1][s] = q.w * Elem<T>::get(bw[buf][s], k + 1);
                    }
                }
            }
#pragma unroll
            for (int k = 0; k < G; k += 4) {
                float yv[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    if constexpr (CKPT) {
                        // the state entering token tg + k + kk, if a backward chunk starts
                        // there (a compile-time test: tg is a multiple of G); no branch,
                        // stores past the sequence or for idle lanes are dropped
                        constexpr int CK = kCkptLen<NS>;
                        const int t = tg + k + kk;
                        if ((t % CK) == 0) {
#pragma unroll
                            for (int s = 0; s < NS; ++s) {
                                const uint32_t so = ((uint32_t)((t / CK) * N + w * NS + s) * (uint32_t)dim +
                                                     (uint32_t)d0) * 4u;
                                __builtin_amdgcn_raw_buffer_store_b32(
                                    __float_as_uint(h[s]), rck, off_if(t < L && sval[s], ck_lane), so, 0);
                            }
                        }
                    }
#pragma unroll
                    for (int s = 0; s < NS; ++s) {
                        h[s] = fmaf(dA[k + kk][s], h[s], bu[k + kk][s]);
                        if constexpr (!NOY) yv[kk] = fmaf(cval(buf, s, k + kk), h[s], yv[kk]);
                    }
                }
                if constexpr (!NOY) s_y[par][w][gi * (G / 4) + k / 4][cs] = make_float4(yv[0], yv[1], yv[2], yv[3]);
            }
        };

        // Scalar and LDS loads share one wait counter and scalar loads
        // complete out of order, so any wait on it covers every load in
        // flight.  Hence: issue group gi+1's loads at the start of group gi,
        // compute group gi with no wait inside, and wait once at its end.
        load_bc(0, bw[0], cw[0]);
        for (int ck = 0; ck < nit; ++ck) {
            const int t0 = ck * TC;
            const int par = ck & 1;
            __syncthreads();                       // chunk ck staged; its s_y buffer free
#pragma unroll
            for (int k = 0; k < G / 2; ++k) ddr[0][k] = s_dd[par][k][cs];
            lgkm_wait_all();
#pragma unroll
            for (int gi = 0; gi < NGRP; ++gi) {
                const int cur = gi & 1, nxt = cur ^ 1;
                if (gi + 1 < NGRP) {
                    load_bc(t0 + (gi + 1) * G, bw[nxt], cw[nxt]);
#pragma unroll
                    for (int k = 0; k < G / 2; ++k) {
                        ddr[nxt][k] = s_dd[par][(gi + 1) * (G / 2) + k][cs];
                    }
                } else {
                    load_bc(t0 + TC, bw[nxt], cw[nxt]);
                }
                // The two scan waves of a SIMD (w and w + 4) take turns at the
                // higher issue priority, group by group, so neither falls behind
                // the other and idles at the next barrier.
                if (((gi & 1) ^ (w >> 2)) & 1) __builtin_amdgcn_s_setprio(1);
                else __builtin_amdgcn_s_setprio(0);
                __builtin_amdgcn_sched_barrier(0);
                group(cur, gi, par, t0 + gi * G);
                lgkm_wait_all();
            }
        }
        __syncthreads();                           // last chunk's partials complete

        if (hT_out && sval_d) {
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const int n = w * NS + s;
                if (n < N) hT_out[(b * dim + d0 + cs) * N + n] = h[s];
            }
        }
    } else {
        // ================= row role: thread -> (row cr, tokens [toff, toff + TPT)) =================
        // Row wave v owns rows 16v .. 16v+15; lane l takes row 16v + (l & 15)
        // and segment l >> 4, so one load or store instruction moves 16 rows
        // x TC contiguous tokens.
        static_assert(SEGS * 16 == 64, "a row wave holds 16 rows x SEGS segments");
        const int rt = tid - NW * 64;
        const int cr = 16 * (rt >> 6) + (rt & 15);
        const int seg = (rt >> 4) & (SEGS - 1);
        const int toff = seg * TPT;
        const bool rval = cr < nrows;
        const float dskip = (rval && D_in) ? D_in[d0 + cr] : 0.f;
        // Front end (FUSED): this row's conv taps, right-aligned in a 4-tap
        // window (w4[3] multiplies the current token); the 3 inputs before the
        // current run (`carry`, used by the row's first segment); the biases.
        float w4[4] = {0.f, 0.f, 0.f, 0.f}, carry[3] = {0.f, 0.f, 0.f}, cbias = 0.f, dbias = 0.f;
        if constexpr (FUSED) {
            const int64_t dr = d0 + (rval ? cr : 0);
#pragma unroll
            for (int k = 0; k < 4; ++k) {                      // tap k of the window is conv_w[k - (4 - K)]
                const int i = k - (4 - fe.K);
                w4[k] = i >= 0 ? fe.conv_w[dr * fe.K + i] : 0.f;
            }
            cbias = fe.conv_b ? fe.conv_b[dr] : 0.f;
            dbias = fe.delta_bias ? fe.delta_bias[dr] : 0.f;
            if (fe.conv_init) {
                const T* ci = static_cast<const T*>(fe.conv_init) + (b * dim + dr) * (fe.K - 1);
#pragma unroll
                for (int k = 0; k < 3; ++k) {                  // carry[k] is the input 3 - k tokens back
                    const int i = k - (4 - fe.K);
                    carry[k] = i >= 0 ? Elem<T>::load1(ci + i) : 0.f;
                }
            }
        }
        const int64_t blk0 = (b * dim + d0) * (int64_t)L;        // first element of this block's rows
        const uint32_t blk_bytes = ALIGNED ? (uint32_t)nrows * (uint32_t)L * (uint32_t)sizeof(T) : 0u;
        const rsrc_t rs_u = make_rsrc(u_in + blk0, blk_bytes);
        const rsrc_t rs_dl = make_rsrc(dl_in + blk0, blk_bytes);
        const rsrc_t rs_z = make_rsrc(z_in ? z_in + blk0 : u_in + blk0, z_in ? blk_bytes : 0u);
        const rsrc_t rs_y = make_rsrc(y_out + blk0, blk_bytes);
        auto run_off = [&](int t) -> uint32_t {   // byte offset of this thread's run at token t
            return (uint32_t)t < (uint32_t)L ? ((uint32_t)cr * (uint32_t)L + (uint32_t)t) * (uint32_t)sizeof(T)
                                             : kOutOfRange;
        };
        const int64_t rrow = (int64_t)(rval ? cr : 0) * L;
        const T* u_row = u_in + blk0 + rrow;
        const T* dl_row = dl_in + blk0 + rrow;
        const T* z_row = z_in ? z_in + blk0 + rrow : nullptr;
        T* y_row = y_out + blk0 + rrow;

        uint32_t ru[RING][WPT], rdl[RING][WPT], rz[RING][WPT];
#pragma unroll
        for (int r = 0; r < RING; ++r)
#pragma unroll
            for (int i = 0; i < WPT; ++i) rz[r][i] = 0u;
        auto load_chunk = [&](int ck, uint32_t (&wu)[WPT], uint32_t (&wdl)[WPT], uint32_t (&wz)[WPT]) {
            const int t = ck * TC + toff;
            if constexpr (ALIGNED) {
                // Unconditional: without z, rs_z is empty and the load returns 0.
                const uint32_t off = run_off(t);
                buf_load<WPT>(rs_u, off, wu);
                buf_load<WPT>(rs_dl, off, wdl);
                if constexpr (!NOY) buf_load<WPT>(rs_z, off, wz);
            } else {
                const int valid = rval ? (L - t) : 0;
                load_run<T, TPT>(u_row + t, valid, false, wu);
                load_run<T, TPT>(dl_row + t, valid, false, wdl);
                if (!NOY && z_row) load_run<T, TPT>(z_row + t, valid, false, wz);
            }
        };

        // Stage chunk ck: (delta, delta*u) to LDS; keep u (FUSED: after the
        // conv) for the epilogue.
        auto stage = [&](int ck, const uint32_t (&cu)[WPT], const uint32_t (&cdl)[WPT], float (&uk)[TPT]) {
            const int t0 = ck * TC;
            const int par = ck & 1;
            if constexpr (FUSED) {
                static_assert(TPT >= 3, "a run holds the 3 inputs the next run's conv needs");
                float xr[TPT];
#pragma unroll
                for (int j = 0; j < TPT; ++j) xr[j] = Elem<T>::get(cu, j);
                // the 3 inputs before this run: from the previous segment's lane, or
                // (first segment) the carry from the previous chunk
                const int lane = tid & 63;
                float xp[3];
#pragma unroll
                for (int k = 0; k < 3; ++k) {
                    const float v = __shfl(xr[TPT - 3 + k], lane - 16, 64);
                    xp[k] = seg > 0 ? v : carry[k];
                }
#pragma unroll
                for (int k = 0; k < 3; ++k) carry[k] = __shfl(xr[TPT - 3 + k], (lane & 15) + 16 * (SEGS - 1), 64);
#pragma unroll
                for (int j = 0; j < TPT; ++j) {
                    float a = cbias;
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const int src = j - 3 + k;   // compile-time after unrolling
                        a = fmaf(w4[k], src < 0 ? xp[src + 3] : xr[src < 0 ? 0 : src], a);
                    }
                    uk[j] = silu(a);
                }
#pragma unroll
                for (int j = 0; j < TPT; j += 2) {
                    // computed for every token, then selected: a conditional
                    // call would become a branch per token
                    float s0 = softplus_f(Elem<T>::get(cdl, j) + dbias);
                    float s1 = softplus_f(Elem<T>::get(cdl, j + 1) + dbias);
                    keep_select(s0);
                    keep_select(s1);
                    const float d0v = t0 + toff + j < L ? s0 : 0.f;
                    const float d1v = t0 + toff + j + 1 < L ? s1 : 0.f;
                    s_dd[par][(toff + j) / 2][cr] = make_float4(d0v, d0v * uk[j], d1v, d1v * uk[j + 1]);
                }
            } else {
#pragma unroll
                for (int j = 0; j < TPT; ++j) uk[j] = Elem<T>::get(cu, j);
#pragma unroll
                for (int j = 0; j < TPT; j += 2) {
                    const float e0 = Elem<T>::get(cdl, j), e1 = Elem<T>::get(cdl, j + 1);
                    // ZOH: (delta, u) -- the hold factor replaces delta in the input term
                    s_dd[par][(toff + j) / 2][cr] = ZOH ? make_float4(e0, uk[j], e1, uk[j + 1])
                                                        : make_float4(e0, e0 * uk[j], e1, e1 * uk[j + 1]);
                }
            }
        };

        // Epilogue of chunk ck: combine the scan waves' partials, skip term,
        // gate, store.  Chunk -1 (the first iteration) reads an unused buffer
        // and stores nothing (its offsets are out of range).
        auto epilogue = [&](int ck, const uint32_t (&cz)[WPT], const float (&uk)[TPT]) {
            if constexpr (NOY) return;
            const int t0 = ck * TC;
            const int par = ck & 1;
            float out[TPT];
#pragma unroll
            for (int j = 0; j < TPT; j += 4) {
                const int quad = (toff + j) / 4;
                float4 acc = s_y[par][0][quad][cr];
#pragma unroll
                for (int q = 1; q < NW; ++q) {
                    const float4 v = s_y[par][q][quad][cr];
                    acc.x += v.x;
                    acc.y += v.y;
                    acc.z += v.z;
                    acc.w += v.w;
                }
                const float a4[4] = {acc.x, acc.y, acc.z, acc.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) out[j + i] = fmaf(dskip, uk[j + i], a4[i]);
            }
            if (z_in) {                           // one uniform branch per chunk, not per token
#pragma unroll
                for (int j = 0; j < TPT; ++j) out[j] *= silu(Elem<T>::get(cz, j));
            }
            if constexpr (ALIGNED) {
                uint32_t wy[WPT];
                pack_words<T, TPT>(out, wy);
                buf_store<WPT, kStream>(rs_y, run_off(t0 + toff), wy);
            } else {
                const int t = t0 + toff;
                if (rval && t >= 0) store_run<T, TPT>(y_row + t, L - t, false, out);
            }
        };

        float uk[2][TPT];                          // kept u of the chunks of each parity
#pragma unroll
        for (int j = 0; j < TPT; ++j) uk[0][j] = uk[1][j] = 0.f;
        // Chunk c lives in slot c % RING from its load until its epilogue.
        // Unpaired: iteration ck loads chunk ck+RING-1 into the slot the
        // epilogue of chunk ck-1 has just released.  Paired: even iterations
        // load chunks ck+RING-2 (slot released one iteration earlier) and
        // ck+RING-1 together, each at least RING-3 iterations before staging.
        constexpr int AHEAD = PAIR ? RING - 2 : RING - 1;
#pragma unroll
        for (int r = 0; r < AHEAD; ++r) load_chunk(r, ru[r], rdl[r], rz[r]);
        stage(0, ru[0], rdl[0], uk[0]);
        // Iteration ck: the scan waves scan chunk ck; here the epilogue of
        // chunk ck-1, the staging of chunk ck+1 and the loads ahead.  The
        // last iteration (ck = nit) has only the epilogue to do; its staging
        // and loads are of chunks past the end (zeros, nothing stored).
        for (int ck0 = 0; ck0 <= nit; ck0 += RING) {
#pragma unroll
            for (int r = 0; r < RING; ++r) {
                const int ck = ck0 + r;
                if (ck > nit) break;
                const int sp = (r + RING - 1) % RING, sn = (r + 1) % RING;
                __syncthreads();
                epilogue(ck - 1, rz[sp], uk[(r + 1) & 1]);
                stage(ck + 1, ru[sn], rdl[sn], uk[(r + 1) & 1]);
                if constexpr (PAIR) {
                    if ((r & 1) == 0) {
                        const int s2 = (r + RING - 2) % RING;
                        load_chunk(ck + RING - 2, ru[s2], rdl[s2], rz[s2]);
                        load_chunk(ck + RING - 1, ru[sp], rdl[sp], rz[sp]);
                    }
                } else {
                    load_chunk(ck + RING - 1, ru[sp], rdl[sp], rz[sp]);
                }
            }
        }
    }
}

// The kernel for one mode: ALIGNED, and FULLN for aligned calls.
template <typename T, int NS, int TC, bool FUSED, bool ZOH, bool CKPT, bool NOY>
auto pick_kernel(bool aligned, bool fulln) {
    return aligned ? (fulln ? s6_scan_kernel<T, NS, TC, true, true, FUSED, ZOH, CKPT, NOY, kRing<T, TC>>
                            : s6_scan_kernel<T, NS, TC, true, false, FUSED, ZOH, CKPT, NOY, kRing<T, TC>>)
                   : s6_scan_kernel<T, NS, TC, false, false, FUSED, ZOH, CKPT, NOY, kRing<T, TC>>;
}

// states_only: p.ckpt receives the saved states and nothing else is written.
template <typename T, int NS, int TC>
hipError_t launch_cfg(const S6Params& p, const S6FrontEnd* fe, bool zoh, bool states_only, hipStream_t stream) {
    const int64_t blocks = ((p.dim + 63) / 64) * p.batch;
    // The aligned path addresses a block's rows through 32-bit buffer
    // offsets, and reads B / C in whole 32-byte groups.
    const bool aligned = (p.L % (32 / int(sizeof(T))) == 0) && int64_t(64) * p.L * int64_t(sizeof(T)) < (int64_t(1) << 31);
    const bool fulln = p.N == kScanWaves * NS;
    // The hold form and the saved states are built for the plain scan only
    // (the fused front end is Euler; the backward pass is of the plain scan).
    auto kern = fe ? pick_kernel<T, NS, TC, true, false, false, false>(aligned, fulln)
              : zoh ? pick_kernel<T, NS, TC, false, true, false, false>(aligned, fulln)
              : p.ckpt ? (states_only ? pick_kernel<T, NS, TC, false, false, true, true>(aligned, fulln)
                                      : pick_kernel<T, NS, TC, false, false, true, false>(aligned, fulln))
                       : pick_kernel<T, NS, TC, false, false, false, false>(aligned, fulln);
    const S6FrontEnd none{};
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3((kScanWaves + kRowWaves) * 64), 0, stream,
                       static_cast<const T*>(p.u), static_cast<const T*>(p.delta), static_cast<const T*>(p.Bm),
                       static_cast<const T*>(p.Cm), static_cast<const T*>(p.z), p.A, p.Dskip, p.h0,
                       static_cast<T*>(p.y), p.h_final, p.dim, p.L, p.N, fe ? *fe : none, p.ckpt);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const S6Params& p, const S6FrontEnd* fe, bool zoh, bool states_only, hipStream_t stream) {
    // 8 scan waves per 64 channels; NS = ceil(N / 8) states per lane.
    if (p.N <= 8) return launch_cfg<T, 1, 32>(p, fe, zoh, states_only, stream);
    if (p.N <= 16) return launch_cfg<T, 2, 32>(p, fe, zoh, states_only, stream);
    if (p.N <= 32) return launch_cfg<T, 4, 32>(p, fe, zoh, states_only, stream);
    return launch_cfg<T, 8, 32>(p, fe, zoh, states_only, stream);
}

__global__ void copy_or_zero_kernel(float* dst, const float* src, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.f;
}

}  // namespace

hipError_t launch_s6_scan(const S6Params& p, bool is_bf16, bool zoh, hipStream_t stream) {
    return is_bf16 ? launch_t<uint16_t>(p, nullptr, zoh, false, stream) : launch_t<float>(p, nullptr, zoh, false, stream);
}

hipError_t launch_s6_scan_fused(const S6Params& p, const S6FrontEnd& fe, bool is_bf16, hipStream_t stream) {
    return is_bf16 ? launch_t<uint16_t>(p, &fe, false, false, stream) : launch_t<float>(p, &fe, false, false, stream);
}

hipError_t launch_s6_save_states(const S6Params& p, bool is_bf16, hipStream_t stream) {
    return is_bf16 ? launch_t<uint16_t>(p, nullptr, false, true, stream) : launch_t<float>(p, nullptr, false, true, stream);
}

hipError_t launch_copy_or_zero(float* dst, const float* src, int64_t n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(copy_or_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, dst, src, n);
    return hipGetLastError();
}

}  // namespace mssm
