// ssd.hip -- Mamba-2 SSD (state space duality), chunked forward, gfx950.
//
// What it computes ("State-Space Model Optimization Patterns" page, section 2 "State Space
// Duality" and section 9 "Chunked Computation"; layout from the "Mamba - Selective State
// Space Models" page, "Workflow 3 / Mamba-2"): for batch row b, head h (group g = h / (H/G))
// and head channel p, with a scalar transition per head,
//     H[p,n] <- exp(dt_t*A_h) * H[p,n] + dt_t * x_t[p] * B_t[n]
//     y_t[p]  = (sum_n C_t[n] * H[p,n] + D_h * x_t[p]) * silu(z_t[p])
// computed chunk by chunk (chunk length Q): within a chunk the output is the
// masked quadratic form (L o C B^T)(dt o X) plus the carried-in state,
//     y_i = sum_{j<=i} exp(s_i - s_j) G_ij dt_j x_j + exp(s_i) C_i H_in + D x_i,
// with s the running sum of dt*A over the chunk and G = C B^T; the state
// leaving the chunk is exp(s_end) H_in + sum_j exp(s_end - s_j) dt_j B_j x_j.
//
// Design:
// - ssd_prep_kernel, per (b, chunk, group): G = C B^T on MFMA, only the
//   blocks the causal mask keeps, stored bf16; and B^T (state-major), so the
//   main kernel's contractions over tokens read their A operands contiguously.
//   Both depend on the group only, so they are computed once for all heads.
// - ssd_main_kernel, one workgroup (8 waves: 4 output, 4 state) per (b,
//   head, block of 32 head channels; headdim is a multiple of 32):
//   walks the chunks in order with the fp32 state H (32 x N) held in MFMA
//   accumulators -- the state never round-trips through HBM.  Per chunk:
//   running sum s (wave scan), x staged transposed in LDS (plain, and scaled
//   by dt*beta), then on v_mfma_f32_16x16x32_bf16:
//     Y_off  = C H_in^T                    (rows scaled by exp(s_i))
//     Y_diag = (L o G)(dt o X)             (causal 16 x 32 blocks)
//     H_out  = exp(s_end) H_in + B^T (w o X)
// - The decay mask is never formed for off-diagonal blocks.  For a row block
//   I (rows from i0) and an earlier token block J (ending at jend),
//     exp(s_i - s_j) = exp(s_i - s_i0) * exp(s_i0 - s_jend) * exp(s_jend - s_j),
//   three factors that are each <= 1 (no overflow however long the chunk):
//   the first scales output rows, the last is folded into the staged x, and
//   the middle one is applied to the accumulator per block (Horner form).  The
//   state update uses the same staged x and per-block factors.  Only the
//   diagonal 16 x 32 blocks build the mask element by element.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace mssm {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kPW = 32;    // head channels per workgroup (headdim is a multiple of it)
constexpr float kDiagSpan = 64.f;   // largest decay (log2 units) over a token block for the factored diagonal

__device__ __forceinline__ f32x4_t mfma16(const u32x4_t a, const u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
}
__device__ __forceinline__ u32x4_t lds128(const uint32_t* p) { return *reinterpret_cast<const u32x4_t*>(p); }
// f(integral_constant<int, i>) for i = B .. E - 1, unrolled at compile time.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}
__device__ __forceinline__ u32x4_t gload128(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
// Per-lane offset plus a wave-uniform one (a tile's place in its array).
__device__ __forceinline__ u32x4_t gload128s(rsrc_t r, uint32_t off, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0);
}

// Workspace layout.  G, B^T and a copy of C are stored as MFMA operand
// tiles: a tile is 16 rows x 32 columns of bf16 (1 KB), and the 16 bytes
// lane l = 16 kg + m of a wave needs (row m, columns 8 kg .. 8 kg + 7) sit at
// byte 16 l.  One load instruction then reads 1 KB of consecutive bytes: the
// row-major form had consecutive lanes 256-512 bytes apart, so the vector
// L1 looked up one line per lane -- four times the lookups -- and those
// lookups, not HBM, limited the main kernel.
//   G   : tile (I, J)  = rows 16 I.., columns (tokens j) 32 J..   index I * (Q/32) + J
//   B^T : tile (nb, J) = rows (states) 16 nb.., columns (tokens) 32 J..   index nb * (Q/32) + J
//   C   : tile (I, nk) = rows (tokens) 16 I.., columns (states) 32 nk..   index I * (N/32) + nk
// per (b, chunk, group), in that order: Q*Q, N*Q and Q*N bf16.
constexpr uint32_t kTileBytes = 1024;

// ---------------------------------------------------------------------------
// Prep: the operand tiles of one (b, chunk, group) and one 32-token block rp
// of the chunk: G = C B^T for rows 32 rp .. 32 rp + 31 and the causal column
// blocks J <= rp, B^T for token block rp, and the copy of C for those rows.
// grid = B * nc * G * (Q / 32), 256 threads.  B rows 0 .. 32 rp + 31 are
// staged in LDS with coalesced loads (16-byte pieces XOR-swizzled by row, so
// fragment reads of 16 consecutive rows hit distinct banks without padding:
// two workgroups fit on a CU at N = 128); every tile leaves as one 1 KB
// store per wave.
// ---------------------------------------------------------------------------
template <int Q, int N>
__global__ __launch_bounds__(256) void ssd_prep_kernel(const uint16_t* __restrict__ Bm,
                                                       const uint16_t* __restrict__ Cm,
                                                       uint16_t* __restrict__ Gw, uint16_t* __restrict__ BTw,
                                                       uint16_t* __restrict__ Cw, int L, int G, int nc) {
    constexpr int KB = Q / 32, NKB = N / 32, NB = N / 16;
    constexpr int CPR = N / 8;                   // 16-byte pieces per row
    constexpr int SWZ = (CPR < 16 ? CPR : 16) - 1;
    constexpr int NLD = Q * CPR / 256;           // staging loads per thread
    __shared__ __align__(16) u32x4_t sB[Q][CPR];
    __shared__ __align__(16) uint32_t sT[4][16][20];   // per wave: one 16 x 32 tile (bf16 pairs, padded)
    auto piece = [](int r, int q) { return q ^ (r & SWZ); };

    // Blocks are dispatched round-robin over the 8 XCDs; number them so that
    // the Q/32 blocks of one (b, chunk, group), which read overlapping B
    // rows, share an XCD and its L2.
    uint32_t lid = blockIdx.x;
    if ((gridDim.x & 7u) == 0u) lid = (blockIdx.x & 7u) * (gridDim.x >> 3) + (blockIdx.x >> 3);
    const int rp = lid % KB;
    const int bcg = lid / KB;                    // (b * nc + c) * G + g
    const int g = bcg % G;
    const int c = (bcg / G) % nc;
    const int64_t b = (bcg / G) / nc;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kg = lane >> 4, m = lane & 15;

    const uint32_t rowbytes = (uint32_t)G * N * 2u;
    const rsrc_t rB = make_rsrc(Bm + b * (int64_t)L * G * N, (uint32_t)L * rowbytes);
    const rsrc_t rC = make_rsrc(Cm + b * (int64_t)L * G * N, (uint32_t)L * rowbytes);
    auto tok = [&](int tl, int n, bool ok) -> uint32_t {  // byte offset of (chunk token tl, state n)
        const int t = c * Q + tl;
        return off_if(ok && t < L, (uint32_t)t * rowbytes + ((uint32_t)g * N + n) * 2u);
    };

    // C fragments of rows 32 rp + 16 il + m (rows past the sequence end read as 0)
    u32x4_t ca[2][NKB];
#pragma unroll
    for (int il = 0; il < 2; ++il)
#pragma unroll
        for (int nk = 0; nk < NKB; ++nk) ca[il][nk] = gload128(rC, tok(32 * rp + 16 * il + m, 32 * nk + 8 * kg, true));
    // B rows 0 .. 32 (rp + 1) - 1, every load in flight at once
    {
        const int nB = 32 * (rp + 1) * CPR;
        u32x4_t v[NLD];
#pragma unroll
        for (int k = 0; k < NLD; ++k) {
            const int idx = 256 * k + tid;
            v[k] = gload128(rB, tok(idx / CPR, 8 * (idx % CPR), idx < nB));
        }
#pragma unroll
        for (int k = 0; k < NLD; ++k) {
            const int idx = 256 * k + tid, r = idx / CPR;
            sB[r][piece(r, idx % CPR)] = v[k];
        }
    }
    // the copy of C: tiles (2 rp + il, nk), spread over the waves
    char* Cout = reinterpret_cast<char*>(Cw + (int64_t)bcg * Q * N) + 16u * lane;
#pragma unroll
    for (int il = 0; il < 2; ++il)
#pragma unroll
        for (int nk = 0; nk < NKB; ++nk)
            if ((il * NKB + nk) % 4 == w)
                *reinterpret_cast<u32x4_t*>(Cout + (uint32_t)((2 * rp + il) * NKB + nk) * kTileBytes) = ca[il][nk];
    __syncthreads();

    // ---- G tiles (2 rp + il, J), J = w, w + 4, .. <= rp ----
    char* Gout = reinterpret_cast<char*>(Gw + (int64_t)bcg * Q * Q) + 16u * lane;
    uint16_t* t16 = reinterpret_cast<uint16_t*>(&sT[w][0][0]);
    for (int J = w; J <= rp; J += 4) {
        f32x4_t acc[2][2] = {};
#pragma unroll
        for (int nk = 0; nk < NKB; ++nk)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int r = 32 * J + 16 * u + m;
                const u32x4_t bv = sB[r][piece(r, 4 * nk + kg)];
#pragma unroll
                for (int il = 0; il < 2; ++il) acc[il][u] = mfma16(ca[il][nk], bv, acc[il][u]);
            }
#pragma unroll
        for (int il = 0; il < 2; ++il) {
            // lane holds rows 4 kg + r, column 16 u + m; re-read in operand order
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int r = 0; r < 4; ++r) t16[(4 * kg + r) * 40 + 16 * u + m] = to_bf16(acc[il][u][r]);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            const u32x4_t v = *reinterpret_cast<const u32x4_t*>(&sT[w][m][4 * kg]);
            *reinterpret_cast<u32x4_t*>(Gout + (uint32_t)((2 * rp + il) * KB + J) * kTileBytes) = v;
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
    }

    // ---- B^T tiles (nb, rp): state 16 nb + m, tokens 32 rp + 8 kg .. + 7 ----
    char* BTout = reinterpret_cast<char*>(BTw + (int64_t)bcg * N * Q) + 16u * lane;
#pragma unroll
    for (int nb0 = 0; nb0 < NB; nb0 += 4) {
        const int nb = nb0 + w;
        if (nb < NB) {
            const int n = 16 * nb + m, r0 = 32 * rp + 8 * kg;
            uint32_t wv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                uint32_t h[2];
#pragma unroll
                for (int o = 0; o < 2; ++o) {
                    const int r = r0 + 2 * e + o;
                    const uint16_t* row = reinterpret_cast<const uint16_t*>(&sB[r][0]);
                    h[o] = row[8 * piece(r, n >> 3) + (n & 7)];
                }
                wv[e] = h[0] | (h[1] << 16);
            }
            *reinterpret_cast<uint4*>(BTout + (uint32_t)(nb * KB + rp) * kTileBytes) =
                make_uint4(wv[0], wv[1], wv[2], wv[3]);
        }
    }
}

// Inclusive prefix sum over the 64 lanes of a wave, on DPP moves: within
// each row of 16 lanes by shifts of 1, 2, 4 and 8 lanes, then across rows by
// adding lane 15 of row 0 / 2 to rows 1 / 3 and lane 31 to rows 2 and 3.
// Lanes a move does not reach add 0 (the `old` operand).
__device__ __forceinline__ float wave_incl_scan(float v) {
    auto step = [](float x, auto ctrl, auto rows) {
        return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), decltype(ctrl)::value,
                                                              decltype(rows)::value, 0xf, false));
    };
    using std::integral_constant;
    v = step(v, integral_constant<int, 0x111>{}, integral_constant<int, 0xf>{});   // row_shr:1
    v = step(v, integral_constant<int, 0x112>{}, integral_constant<int, 0xf>{});   // row_shr:2
    v = step(v, integral_constant<int, 0x114>{}, integral_constant<int, 0xf>{});   // row_shr:4
    v = step(v, integral_constant<int, 0x118>{}, integral_constant<int, 0xf>{});   // row_shr:8
    v = step(v, integral_constant<int, 0x142>{}, integral_constant<int, 0xa>{});   // row_bcast:15
    v = step(v, integral_constant<int, 0x143>{}, integral_constant<int, 0xc>{});   // row_bcast:31
    return v;
}

// ---------------------------------------------------------------------------
// Main: one workgroup per (b, head, block of 32 head channels); chunks in order.
// 512 threads in two roles (one wave of each on every SIMD):
//   output waves 0-3: the chunk's outputs from the staged chunk and the
//     carried-in state (Y_diag, Y_off, skip, gate, store);
//   state waves 4-7: the state update for the chunk, then the staging of the
//     next chunk (running sum, x^T and its two scaled copies), so staging is
//     off the output waves' path.  Every LDS buffer a chunk is read from is
//     double-buffered by chunk parity: one barrier per chunk.
// ---------------------------------------------------------------------------
// HASZ: a gate z is given.  Loads for the chunk after the last read zeros
// through zero-size buffer resources (no branches around loads, which would
// make the compiler's wait counting fall back to waiting for everything).
template <int Q, int N, bool HASZ>
__global__ __launch_bounds__(512) void ssd_main_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ DT, const float* __restrict__ Ah,
    const float* __restrict__ Dh, const uint16_t* __restrict__ Z,
    const float* __restrict__ h0, uint16_t* __restrict__ Y, float* __restrict__ hT,
    const uint16_t* __restrict__ Gw, const uint16_t* __restrict__ BTw, const uint16_t* __restrict__ Cw,
    int L, int H, int P, int G, int nc) {
    constexpr int RB = Q / 16;                   // row blocks (16 tokens)
    constexpr int RBW = RB / 4;                  // rounds of row blocks (4 row blocks each)
    constexpr int SRB = RBW > 1 ? 1 : 0;         // rounds the state waves take (the cheapest one)
    constexpr int KB = Q / 32;                   // token blocks (32 tokens, one MFMA K step)
    constexpr int NB = N / 16;                   // state blocks (16 states)
    constexpr int NKB = N / 32;                  // 32-state K steps
    constexpr int NBW = (NB + 3) / 4;            // state blocks per state wave
    constexpr int TPL = Q / 64;                  // tokens per lane when staging
    constexpr int XS = (Q + 8) / 2;              // x^T row stride (bf16 pairs)
    constexpr int HS = (N + 8) / 2;              // Hb row stride (bf16 pairs)
    static_assert(Q % 64 == 0 && N % 32 == 0, "Q multiple of 64, N multiple of 32");

    __shared__ __align__(16) float s_s[2][Q];    // running sum of dt*A*log2(e) within the chunk
    __shared__ __align__(16) float s_dt[2][Q];
    __shared__ __align__(16) uint32_t xT[2][kPW][XS];    // x^T, bf16 pairs along tokens
    __shared__ __align__(16) uint32_t xsT[2][kPW][XS];   // (dt * e^(s_blockend - s) * x)^T
    __shared__ __align__(16) uint32_t xwT[2][kPW][XS];   // (dt * e^(s_chunkend - s) * x)^T
    __shared__ __align__(16) uint32_t Hb[2][kPW][HS];    // carried-in state, bf16 pairs along n
    __shared__ __align__(16) uint32_t ytile[8][16][kPW / 2];  // per wave: one 16 x 32 bf16 output tile
    __shared__ __align__(16) float s_fs[4][Q];                 // per state wave: dt e^(s_blockend - s) by token
    __shared__ __align__(16) float s_fw[4][Q];                 // per state wave: dt e^(s_chunkend - s) by token

    // Blocks are dispatched round-robin over the 8 XCDs; number them so that
    // consecutive ids (the heads of one batch row) share an XCD and its L2,
    // where that row's G, B^T and C tiles are cached.
    uint32_t lid = blockIdx.x;
    if ((gridDim.x & 7u) == 0u) lid = (blockIdx.x & 7u) * (gridDim.x >> 3) + (blockIdx.x >> 3);
    const int npb = P / kPW;                     // channel blocks per head
    const int ph = lid % npb;
    const int bh = lid / npb;
    const int h = bh % H;
    const int64_t b = bh / H;
    const int g = h / (H / G);
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = w & 3;                        // index within the role
    const int kg = lane >> 4, m = lane & 15;

    const float a_h = Ah[h] * kLog2e;

    // Buffers over batch row b (32-bit offsets; the host checks the sizes).
    const uint32_t xrow = (uint32_t)H * P * 2u;                // bytes per token of x / y / z
    const rsrc_t rX = make_rsrc(X + b * (int64_t)L * H * P, (uint32_t)L * xrow);
    const uint32_t chan0 = ((uint32_t)h * P + kPW * ph) * 2u;   // byte offset of this channel block in a token row
    auto send = [&](int pb, int J) { return s_s[pb][32 * J + 31]; };   // s at the end of token block J

    const float dskip = Dh ? Dh[h] : 0.f;
    const rsrc_t rY = make_rsrc(Y + b * (int64_t)L * H * P, (uint32_t)L * xrow);
    const rsrc_t rZ = make_rsrc(Z ? Z + b * (int64_t)L * H * P : X, Z ? (uint32_t)L * xrow : 0u);
    const uint32_t gbytes = (uint32_t)Q * Q * 2u;
    const uint32_t cbytes = (uint32_t)Q * N * 2u;
    const int jhi = wr >> 1;                 // row block I = wr + 4 rb lies in token block 2 rb + jhi

    // G tiles: every row block has its own registers (row block rb needs
    // G tiles J <= 2 rb + 1, at offset rb (rb + 1) in `ga`), and a row
    // block's tiles for the next chunk are requested as soon as its MFMAs
    // have read them, a whole chunk ahead of use.  C tiles and gate values
    // are double-buffered one row block ahead.  Tiles a row block does not
    // need are read at an out-of-range offset (no traffic, value 0), so
    // every load is unconditional.
    constexpr int NGA = RBW * (RBW + 1);
    u32x4_t ga[NGA];
    u32x4_t ca[2][NKB];
    uint32_t zz[2][8];
    auto load_g = [&](int cc, int rb) {
        const int I = wr + 4 * rb;
        const rsrc_t rG = make_rsrc(Gw + (((int64_t)b * nc + (cc < nc ? cc : 0)) * G + g) * Q * Q,
                                    cc < nc ? gbytes : 0u);
        const uint32_t gb = ((uint32_t)I * KB * 64 + lane) * 16u;
        const uint32_t glast = off_if(jhi != 0, gb);
#pragma unroll
        for (int J = 0; J <= 2 * rb + 1; ++J)
            ga[rb * (rb + 1) + J] = gload128s(rG, J <= 2 * rb ? gb : glast, (uint32_t)J * kTileBytes);
    };
    auto load_c = [&](int cc, int rb, int sl) {
        const int I = wr + 4 * rb;
        const rsrc_t rC = make_rsrc(Cw + (((int64_t)b * nc + (cc < nc ? cc : 0)) * G + g) * Q * N,
                                    cc < nc ? cbytes : 0u);
        const uint32_t cb = ((uint32_t)I * NKB * 64 + lane) * 16u;
#pragma unroll
        for (int nk = 0; nk < NKB; ++nk) ca[sl][nk] = gload128s(rC, cb, (uint32_t)nk * kTileBytes);
    };
    auto load_z = [&](int cc, int rb, int sl) {
        if constexpr (HASZ) {
            const int I = wr + 4 * rb;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tr = cc * Q + 16 * I + 4 * kg + r;
                const uint32_t zb = off_if(tr < L, (uint32_t)tr * xrow + chan0 + 2u * m);
#pragma unroll
                for (int pt = 0; pt < 2; ++pt)
                    zz[sl][2 * r + pt] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rZ, zb + 32u * pt, 0, 0);
            }
        }
    };

    // One 16-row block I = wr + 4 rb of chunk c: off-diagonal and diagonal
    // token blocks, C H_in^T, then `mid` (the caller's loads for later row
    // blocks), then combine, skip, gate and store through LDS tile `yt`.
    auto row_block = [&](auto rbc, auto slc, int c, int pb, int yt, auto mid) {
        constexpr int rb = decltype(rbc)::value;
        constexpr int sl = decltype(slc)::value;
        const int I = wr + 4 * rb;
        const int i0 = 16 * I;
        const int Jd = 2 * rb + jhi;     // the token block holding row block I
        const u32x4_t* gt = &ga[rb * (rb + 1)];
        f32x4_t off_[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        f32x4_t dg[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        f32x4_t yo[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        // Every LDS operand is read one step ahead of the MFMAs that
        // use it (the sched_barriers keep the compiler from sinking the
        // reads back next to their use, which would expose each read's
        // latency in turn).
        const float si0 = s_s[pb][i0];
        float se[2 * RBW];
#pragma unroll
        for (int J = 0; J <= 2 * rb; ++J) se[J] = send(pb, J);
        u32x4_t xb[2][2];
#pragma unroll
        for (int pt = 0; pt < 2; ++pt) xb[0][pt] = lds128(&xsT[pb][16 * pt + m][4 * kg]);
        // off-diagonal token blocks J < Jd: each block's product G_IJ xs_J
        // goes to a fresh accumulator and is added scaled by the decay
        // from the end of block J to the first row of block I (<= 1),
        // one block behind, so the adds never wait on an MFMA.
        f32x4_t tq[2][2];
        const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int J = 0; J <= 2 * rb; ++J) {
            if (J < 2 * rb) {
#pragma unroll
                for (int pt = 0; pt < 2; ++pt)
                    xb[(J + 1) & 1][pt] = lds128(&xsT[pb][16 * pt + m][16 * (J + 1) + 4 * kg]);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (J < Jd) {                // J = 2 rb: off-diagonal for jhi = 1 only
#pragma unroll
                for (int pt = 0; pt < 2; ++pt) tq[J & 1][pt] = mfma16(gt[J], xb[J & 1][pt], zero4);
            }
            if (J > 0) {
                const float f = fast_exp2(si0 - se[J - 1]);
#pragma unroll
                for (int pt = 0; pt < 2; ++pt) off_[pt] += f * tq[(J - 1) & 1][pt];
            }
        }
        if (jhi) {
            const float f = fast_exp2(si0 - se[2 * rb]);
#pragma unroll
            for (int pt = 0; pt < 2; ++pt) off_[pt] += f * tq[(2 * rb) & 1][pt];
        }
        // operands of the diagonal block and of C H_in^T
        const int i = i0 + m;
        const float si = s_s[pb][i];
        const int j0 = 32 * Jd + 8 * kg;
        // Diagonal block, usual case: exp(s_i - s_j) = exp(s_i - s_e) exp(s_e - s_j)
        // with s_e the end of token block Jd.  The second factor (with dt) is
        // already in the staged xs, the first scales the accumulator row, and
        // the mask is a select on G.  Both factors stay within 2^+-kDiagSpan
        // when the decay over the block is at most that; otherwise the mask
        // is built element by element.
        const float sbe = send(pb, Jd);
        const bool fast = __builtin_amdgcn_readfirstlane(s_s[pb][32 * Jd] - sbe <= kDiagSpan ? 1 : 0) != 0;
        const float4 d0 = *reinterpret_cast<const float4*>(&s_dt[pb][j0]);
        const float4 d1 = *reinterpret_cast<const float4*>(&s_dt[pb][j0 + 4]);
        const float4 q0 = *reinterpret_cast<const float4*>(&s_s[pb][j0]);
        const float4 q1 = *reinterpret_cast<const float4*>(&s_s[pb][j0 + 4]);
        u32x4_t xd[2], xe[2], hb[2][2];
        uint2 xr[2];                     // x of this lane's output rows (skip term)
#pragma unroll
        for (int pt = 0; pt < 2; ++pt) {
            xd[pt] = lds128(&xT[pb][16 * pt + m][16 * Jd + 4 * kg]);
            xe[pt] = lds128(&xsT[pb][16 * pt + m][16 * Jd + 4 * kg]);
            hb[0][pt] = lds128(&Hb[pb][16 * pt + m][4 * kg]);
            xr[pt] = *reinterpret_cast<const uint2*>(&xT[pb][16 * pt + m][(i0 + 4 * kg) >> 1]);
        }
        const float4 sr = *reinterpret_cast<const float4*>(&s_s[pb][i0 + 4 * kg]);
        __builtin_amdgcn_sched_barrier(0);
        // diagonal token block
        {
            // the two candidate tiles pass through an empty asm, so the
            // choice stays a select: an index into `ga` would put it in scratch
            u32x4_t g0 = gt[2 * rb], g1 = gt[2 * rb + 1];
            asm("" : "+v"(g0), "+v"(g1));
            const u32x4_t gv = jhi ? g1 : g0;
            if (fast) {
                // keep G_ij for j <= i: element e of the lane's 8 is j0 + e
                const int k = i - j0;
                u32x4_t a;
#pragma unroll
                for (int w2 = 0; w2 < 4; ++w2)
                    a[w2] = gv[w2] & (k >= 2 * w2 + 1 ? 0xffffffffu : (k == 2 * w2 ? 0x0000ffffu : 0u));
#pragma unroll
                for (int pt = 0; pt < 2; ++pt) dg[pt] = mfma16(a, xe[pt], dg[pt]);
            } else {
                // element by element: dt and the decay folded into G, plain x
                const float dj[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
                const float sj[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
                uint32_t av[4];
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const uint32_t gw = gv[e / 2];
                    float v0 = __uint_as_float(gw << 16) * dj[e] * fast_exp2(si - sj[e]);
                    float v1 = __uint_as_float(gw & 0xffff0000u) * dj[e + 1] * fast_exp2(si - sj[e + 1]);
                    keep_select(v0);
                    keep_select(v1);
                    av[e / 2] = pack_bf16x2(j0 + e <= i ? v0 : 0.f, j0 + e + 1 <= i ? v1 : 0.f);
                }
                const u32x4_t a = {av[0], av[1], av[2], av[3]};
#pragma unroll
                for (int pt = 0; pt < 2; ++pt) dg[pt] = mfma16(a, xd[pt], dg[pt]);
            }
        }
        // carried-in state: C rows times H_in^T
#pragma unroll
        for (int nk = 0; nk < NKB; ++nk) {
            if (nk + 1 < NKB) {
#pragma unroll
                for (int pt = 0; pt < 2; ++pt)
                    hb[(nk + 1) & 1][pt] = lds128(&Hb[pb][16 * pt + m][16 * (nk + 1) + 4 * kg]);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int pt = 0; pt < 2; ++pt) yo[pt] = mfma16(ca[sl][nk], hb[nk & 1][pt], yo[pt]);
        }
        mid();
        // combine, skip, gate; the tile goes through LDS so that each
        // lane stores 8 consecutive head channels of one token (16 bytes).
        uint16_t* yt16 = reinterpret_cast<uint16_t*>(&ytile[yt][0][0]);
        const float srv[4] = {sr.x, sr.y, sr.z, sr.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float al = fast_exp2(srv[r] - si0);
            const float ei = fast_exp2(srv[r]);
            const float dr = fast ? fast_exp2(srv[r] - sbe) : 1.f;   // the fast diagonal block's row factor
#pragma unroll
            for (int pt = 0; pt < 2; ++pt) {
                const uint32_t xw = (r >> 1) ? xr[pt].y : xr[pt].x;
                const float xv = __uint_as_float((r & 1) ? (xw & 0xffff0000u) : (xw << 16));
                float yv = al * off_[pt][r] + dr * dg[pt][r] + ei * yo[pt][r] + dskip * xv;
                if constexpr (HASZ) yv *= silu(__uint_as_float(zz[sl][2 * r + pt] << 16));
                yt16[(4 * kg + r) * kPW + 16 * pt + m] = to_bf16(yv);
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        {
            const int tr = lane >> 2, cg = lane & 3;          // token row, 8-channel group
            const u32x4_t v = *reinterpret_cast<const u32x4_t*>(&ytile[yt][tr][4 * cg]);
            const int t = c * Q + i0 + tr;
            __builtin_amdgcn_raw_buffer_store_b128(v, rY, off_if(t < L, (uint32_t)t * xrow + chan0 + 16u * cg),
                                                   0, kCached);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    if (w < 4) {
        // ======================= output waves ======================================
        // Row blocks SRB .. RBW - 1 (with more than one per wave the state
        // waves take the first round).  C tiles and gate values alternate
        // between two slots; the next chunk's first row block goes to slot 0
        // once the last row block has read its own.
        constexpr int NRO = RBW - SRB;
#pragma unroll
        for (int rb = SRB; rb < RBW; ++rb) load_g(0, rb);
        load_c(0, SRB, 0);
        load_z(0, SRB, 0);
        __syncthreads();                         // chunk 0 staged, carried-in state written
        for (int c = 0; c < nc; ++c) {
            const int pb = c & 1;
            static_for<SRB, RBW>([&](auto rbc) {
                constexpr int rb = decltype(rbc)::value;
                constexpr int sl = (rb - SRB) & 1;
                if constexpr (rb + 1 < RBW) {
                    load_c(c, rb + 1, sl ^ 1);
                    load_z(c, rb + 1, sl ^ 1);
                }
                row_block(rbc, std::integral_constant<int, sl>{}, c, pb, wr, [&] {
                    load_g(c + 1, rb);           // this row block's G tiles for the next chunk
                    if constexpr (rb + 1 == RBW) {
                        load_c(c + 1, SRB, 0);
                        if constexpr (NRO % 2 == 0) load_z(c + 1, SRB, 0);
                    }
                });
                if constexpr (rb + 1 == RBW && NRO % 2 == 1) load_z(c + 1, SRB, 0);
            });
            __syncthreads();
        }
    } else {
        // ======================= state waves =======================================
        const rsrc_t rDT = make_rsrc(DT + b * (int64_t)L * H, (uint32_t)L * H * 2u);
        const uint32_t btbytes = (uint32_t)N * Q * 2u;

        // State tiles (state block nb = wr + 4 k, head-channel tile pt): lane
        // holds states 16 nb + 4 kg + r (r < 4) of head channel 16 pt + m.
        f32x4_t accH[NBW][2];
#pragma unroll
        for (int k = 0; k < NBW; ++k)
#pragma unroll
            for (int pt = 0; pt < 2; ++pt) {
                const int nb = wr + 4 * k;
                f32x4_t v = {0.f, 0.f, 0.f, 0.f};
                if (h0 && nb < NB) {
                    const int p = kPW * ph + 16 * pt + m;
                    const float4 q = *reinterpret_cast<const float4*>(
                        h0 + (((b * H + h) * P + p) * (int64_t)N + 16 * nb + 4 * kg));
                    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
                }
                accH[k][pt] = v;
            }
        auto write_hb = [&](int pb) {
#pragma unroll
            for (int k = 0; k < NBW; ++k) {
                const int nb = wr + 4 * k;
                if (nb < NB) {
#pragma unroll
                    for (int pt = 0; pt < 2; ++pt) {
                        const f32x4_t v = accH[k][pt];
                        *reinterpret_cast<uint2*>(&Hb[pb][16 * pt + m][(16 * nb + 4 * kg) / 2]) =
                            make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
                    }
                }
            }
        };

        // B^T tiles of this wave's state blocks.  Up to two state blocks are
        // held (slot k % 2): blocks 0 and 1 of a chunk are loaded a chunk
        // ahead, block k + 2 while block k accumulates.
        constexpr int BSL = NBW < 2 ? NBW : 2;
        u32x4_t ba[BSL][KB];
        auto load_bt = [&](int cc, int k) {
            const rsrc_t rBT = make_rsrc(BTw + (((int64_t)b * nc + (cc < nc ? cc : 0)) * G + g) * N * Q,
                                         cc < nc ? btbytes : 0u);
            const int nb = wr + 4 * k;
            const uint32_t base = off_if(nb < NB, ((uint32_t)nb * KB * 64 + lane) * 16u);
#pragma unroll
            for (int J = 0; J < KB; ++J) ba[k % BSL][J] = gload128s(rBT, base, (uint32_t)J * kTileBytes);
        };
        auto load_bt_ahead = [&](int cc) {
#pragma unroll
            for (int k = 0; k < BSL; ++k) load_bt(cc, k);
        };

        // Staging of one chunk.  The running sum: lane l takes the dt of tokens
        // l*TPL .. l*TPL+TPL-1, and every state wave scans the whole chunk
        // itself (no cross-wave step); wave 4 also publishes s and dt for the
        // output waves.  x: 16-token blocks tb = wr + 4 k, read as MFMA A
        // operands (lane (kg, m): token 16 tb + m, head channels 8 kg .. 8 kg + 7
        // of this half, so one load moves 16 tokens x 64 contiguous bytes) and
        // transposed by an MFMA against an identity operand (exact), which
        // leaves 4 consecutive tokens of one head channel in each lane: those
        // go to x^T and its two scaled copies as 8-byte LDS stores.
        constexpr int XU = Q / 64;               // 16-token blocks per state wave
        u32x4_t xv[XU];
        uint32_t dtw[TPL];
        u32x4_t ident[2];                        // B[K][n] = 1 where K = 16 cb + n
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                ident[cb][q] = (8 * kg + 2 * q == 16 * cb + m ? 0x3F80u : 0u) |
                               (8 * kg + 2 * q + 1 == 16 * cb + m ? 0x3F800000u : 0u);
        auto stage_load = [&](int cc) {
#pragma unroll
            for (int i = 0; i < TPL; ++i) {
                const int t = cc * Q + lane * TPL + i;
                dtw[i] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rDT, off_if(t < L, ((uint32_t)t * H + h) * 2u), 0, 0);
            }
#pragma unroll
            for (int k = 0; k < XU; ++k) {
                const int t = cc * Q + 16 * (wr + 4 * k) + m;
                xv[k] = gload128(rX, off_if(t < L, (uint32_t)t * xrow + chan0 + 16u * kg));
            }
        };
        auto stage_store = [&](int pb) -> float {
            float dv[TPL], sv[TPL];
            float run = 0.f;
#pragma unroll
            for (int i = 0; i < TPL; ++i) {
                dv[i] = __uint_as_float(dtw[i] << 16);
                run += dv[i] * a_h;
                sv[i] = run;
            }
            const float tot = wave_incl_scan(run);   // inclusive scan of the lane totals
            const float base = tot - run;
#pragma unroll
            for (int i = 0; i < TPL; ++i) sv[i] += base;
            const float s_be = __shfl(tot, ((lane * TPL) | 31) / TPL, 64);   // end of my 32-token block
            const float s_end = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(tot), 63));  // end of the chunk
            if (wr == 0) {
#pragma unroll
                for (int i = 0; i < TPL; ++i) {
                    s_s[pb][lane * TPL + i] = sv[i];
                    s_dt[pb][lane * TPL + i] = dv[i];
                }
            }
            float fs[TPL], fw[TPL];
#pragma unroll
            for (int i = 0; i < TPL; ++i) {
                fs[i] = dv[i] * fast_exp2(s_be - sv[i]);
                fw[i] = dv[i] * fast_exp2(s_end - sv[i]);
            }
            const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
            // the factors go through this wave's own LDS rows (indexed by
            // token), so each lane reads its 4 consecutive tokens' factors
            // as two 16-byte loads rather than 8 lane shuffles
#pragma unroll
            for (int i = 0; i < TPL; ++i) {
                s_fs[wr][lane * TPL + i] = fs[i];
                s_fw[wr][lane * TPL + i] = fw[i];
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
            for (int k = 0; k < XU; ++k) {
                const int tb = wr + 4 * k;
                // the factors of this lane's tokens 16 tb + 4 kg + r
                const float4 a4 = *reinterpret_cast<const float4*>(&s_fs[wr][16 * tb + 4 * kg]);
                const float4 b4 = *reinterpret_cast<const float4*>(&s_fw[wr][16 * tb + 4 * kg]);
                const float f1[4] = {a4.x, a4.y, a4.z, a4.w};
                const float f2[4] = {b4.x, b4.y, b4.z, b4.w};
                const int wd = 8 * tb + 2 * kg;
#pragma unroll
                for (int cb = 0; cb < 2; ++cb) {
                    const f32x4_t v = mfma16(xv[k], ident[cb], zero4);   // v[r] = x[16 tb + 4 kg + r][16 cb + m]
                    const int row = 16 * cb + m;
                    *reinterpret_cast<uint2*>(&xT[pb][row][wd]) =
                        make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
                    *reinterpret_cast<uint2*>(&xsT[pb][row][wd]) =
                        make_uint2(pack_bf16x2(v[0] * f1[0], v[1] * f1[1]), pack_bf16x2(v[2] * f1[2], v[3] * f1[3]));
                    *reinterpret_cast<uint2*>(&xwT[pb][row][wd]) =
                        make_uint2(pack_bf16x2(v[0] * f2[0], v[1] * f2[1]), pack_bf16x2(v[2] * f2[2], v[3] * f2[3]));
                }
            }
            return s_end;
        };

        stage_load(0);
        load_bt_ahead(0);
        if constexpr (SRB > 0) {                 // the first round of row blocks: I = wr
            load_g(0, 0);
            load_c(0, 0, 0);
            load_z(0, 0, 0);
        }
        write_hb(0);
        float s_end = stage_store(0);
        if (nc > 1) stage_load(1);
        __syncthreads();                         // chunk 0 staged, carried-in state written
        for (int c = 0; c < nc; ++c) {
            const int pb = c & 1;
            // H_out = e^(s_end) H_in + B^T (w o X), w_j = dt_j e^(s_end - s_j) <= 1
            const float dec = fast_exp2(s_end);
            // state blocks in pairs (the held B^T slots); each x tile read
            // from LDS one token block ahead serves both blocks of the pair
#pragma unroll
            for (int k0 = 0; k0 < NBW; k0 += BSL) {
#pragma unroll
                for (int k = k0; k < k0 + BSL; ++k)
#pragma unroll
                    for (int pt = 0; pt < 2; ++pt) accH[k][pt] *= dec;
                u32x4_t xw[2][2];
#pragma unroll
                for (int pt = 0; pt < 2; ++pt) xw[0][pt] = lds128(&xwT[pb][16 * pt + m][4 * kg]);
#pragma unroll
                for (int J = 0; J < KB; ++J) {
                    if (J + 1 < KB) {
#pragma unroll
                        for (int pt = 0; pt < 2; ++pt)
                            xw[(J + 1) & 1][pt] = lds128(&xwT[pb][16 * pt + m][16 * (J + 1) + 4 * kg]);
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int k = k0; k < k0 + BSL; ++k)
                        if (wr + 4 * k < NB) {
#pragma unroll
                            for (int pt = 0; pt < 2; ++pt)
                                accH[k][pt] = mfma16(ba[k % BSL][J], xw[J & 1][pt], accH[k][pt]);
                        }
                }
#pragma unroll
                for (int k = k0; k < k0 + BSL; ++k)
                    if (k + BSL < NBW) load_bt(c, k + BSL);
            }
            // row block I = wr of this chunk, while the MFMAs above drain
            if constexpr (SRB > 0) {
                row_block(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}, c, pb, 4 + wr, [&] {
                    load_g(c + 1, 0);
                    load_c(c + 1, 0, 0);
                });
                load_z(c + 1, 0, 0);
            }
            // the next chunk (past the last one: zeros, results unused)
            load_bt_ahead(c + 1);
            write_hb(pb ^ 1);
            s_end = stage_store(pb ^ 1);
            stage_load(c + 2);
            __syncthreads();
        }
        if (hT) {
#pragma unroll
            for (int k = 0; k < NBW; ++k) {
                const int nb = wr + 4 * k;
                if (nb < NB) {
#pragma unroll
                    for (int pt = 0; pt < 2; ++pt) {
                        const int p = kPW * ph + 16 * pt + m;
                        const f32x4_t v = accH[k][pt];
                        *reinterpret_cast<float4*>(hT + (((b * H + h) * P + p) * (int64_t)N + 16 * nb + 4 * kg)) =
                            make_float4(v[0], v[1], v[2], v[3]);
                    }
                }
            }
        }
    }
}

template <int Q, int N>
hipError_t launch_qn(const SSDParams& p, hipStream_t stream) {
    auto kern = p.z ? ssd_main_kernel<Q, N, true> : ssd_main_kernel<Q, N, false>;
    const int nc = (p.L + Q - 1) / Q;
    uint16_t* Gw = static_cast<uint16_t*>(p.workspace);
    uint16_t* BTw = Gw + (int64_t)p.batch * nc * p.G * Q * Q;
    uint16_t* Cw = BTw + (int64_t)p.batch * nc * p.G * N * Q;
    const int64_t prep_blocks = p.batch * nc * p.G * (Q / 32);
    const int64_t blocks = p.batch * p.H * (p.P / kPW);
    if (prep_blocks > INT32_MAX || blocks > INT32_MAX) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((ssd_prep_kernel<Q, N>), dim3((unsigned)prep_blocks), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(p.Bm), static_cast<const uint16_t*>(p.Cm), Gw, BTw, Cw, p.L, p.G,
                       nc);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(512), 0, stream,
                       static_cast<const uint16_t*>(p.x), static_cast<const uint16_t*>(p.dt), p.A,
                       p.Dskip, static_cast<const uint16_t*>(p.z), p.h0,
                       static_cast<uint16_t*>(p.y), p.h_final, Gw, BTw, Cw, p.L, p.H, p.P, p.G, nc);
    return hipGetLastError();
}

template <int Q>
hipError_t launch_q(const SSDParams& p, hipStream_t stream) {
    switch (p.N) {
        case 32: return launch_qn<Q, 32>(p, stream);
        case 64: return launch_qn<Q, 64>(p, stream);
        case 128: return launch_qn<Q, 128>(p, stream);
        case 256: return launch_qn<Q, 256>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

size_t ssd_fast_workspace_bytes(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G,
                                int64_t Q) {
    (void)H;
    (void)P;
    if (Q <= 0) return 0;
    const int64_t nc = (L + Q - 1) / Q;
    return (size_t)(batch * nc * G * Q * (Q + 2 * N) * 2);     // G, B^T and C tiles
}

bool ssd_fast_supported(int64_t L, int64_t H, int64_t P, int64_t N, int64_t G, int64_t Q) {
    if (P < kPW || P % kPW != 0) return false;
    if (!(N == 32 || N == 64 || N == 128 || N == 256)) return false;
    if (!(Q == 64 || Q == 128 || Q == 256)) return false;
    const int64_t lim = int64_t(1) << 31;
    // 32-bit buffer offsets over one batch row
    return L * H * P * 2 < lim && L * G * N * 2 < lim && L * H * 2 < lim;
}

hipError_t launch_ssd_fast(const SSDParams& p, hipStream_t stream) {
    switch (p.Q) {
        case 64: return launch_q<64>(p, stream);
        case 128: return launch_q<128>(p, stream);
        case 256: return launch_q<256>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace mssm
