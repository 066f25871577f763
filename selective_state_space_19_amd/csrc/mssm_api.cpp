// mssm_api.cpp -- the C ABI of libmssm.so: argument checking, then launch.
//
// Every check happens on the host before anything is enqueued; a failed
// check returns a negative MSSM_ERR_* code and records a message for the
// calling thread (mssm_last_error).  Nothing here allocates or synchronises.
#include "mssm.h"

#include <hip/hip_runtime.h>

#include <climits>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <string>

#include "kernels.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// a*b*c with overflow check against 2^62.
bool prod_ok(int64_t a, int64_t b, int64_t c, int64_t* out) {
    const int64_t lim = int64_t(1) << 62;
    if (a < 0 || b < 0 || c < 0) return false;
    __int128 v = (__int128)a * b * c;
    if (v >= lim) return false;
    if (out) *out = (int64_t)v;
    return true;
}

#define CHECK_PTR(p)                                                           \
    do {                                                                       \
        if (!(p)) return fail(MSSM_ERR_NULL, "%s: %s is NULL", fn, #p);         \
        if (!aligned16(p)) return fail(MSSM_ERR_ALIGN, "%s: %s is not 16-byte aligned", fn, #p); \
    } while (0)
#define CHECK_OPT(p)                                                           \
    do {                                                                       \
        if ((p) && !aligned16(p)) return fail(MSSM_ERR_ALIGN, "%s: %s is not 16-byte aligned", fn, #p); \
    } while (0)

int launched(const char* fn, hipError_t e) {
    if (e != hipSuccess) return fail(MSSM_ERR_LAUNCH, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return MSSM_OK;
}

// Scratch for the entry point that allocates nothing
// (mssm_ssd_chunk_fwd_noalloc): a fixed array in device memory, one copy per
// GPU, held until the process ends.  In host code `scratch` names a host-side
// stand-in, not device memory: kernels get the device address that
// hipGetSymbolAddress returns, looked up once per device (with that device
// current) on the entry point's first call there and kept in g_scratch.
constexpr size_t kScratchBytes = size_t(MSSM_NOALLOC_SCRATCH_BYTES);
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

int scratch_address(const char* fn, void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(MSSM_ERR_LAUNCH, "%s: hipGetDevice failed: %s", fn, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(MSSM_ERR_UNSUPPORTED, "%s: device %d beyond %d", fn, dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(MSSM_ERR_LAUNCH, "%s: hipGetSymbolAddress(scratch) failed: %s", fn, hipGetErrorString(e));
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return MSSM_OK;
}

}  // namespace

extern "C" {

const char* mssm_last_error(void) { return g_err.c_str(); }

int mssm_version(void) { return 100; }

// save: the chunk-start states for mssm_selective_scan_bwd_saved go to the
// start of `workspace` (the backward's own workspace, of its size).
static int scan_fwd(const char* fn, bool zoh, bool save, const void* u, const void* delta, const float* A,
                    const void* Bm, const void* Cm, const float* Dskip, const void* z, const float* h0, void* y,
                    float* h_final, int64_t batch, int64_t d_inner, int64_t seqlen, int64_t d_state,
                    void* workspace, size_t workspace_bytes, mssm_dtype dtype, void* stream) {
    g_err.clear();
    if (dtype != MSSM_F32 && dtype != MSSM_BF16) return fail(MSSM_ERR_DTYPE, "%s: unknown dtype %d", fn, (int)dtype);
    if (batch < 0 || d_inner < 0 || seqlen < 0 || d_state < 0)
        return fail(MSSM_ERR_SHAPE, "%s: negative dimension", fn);
    if (d_state < 1 || d_state > 64) return fail(MSSM_ERR_UNSUPPORTED, "%s: d_state %lld not in [1, 64]", fn, (long long)d_state);
    if (seqlen > MSSM_MAX_SEQLEN)
        return fail(MSSM_ERR_UNSUPPORTED, "%s: seqlen %lld above %lld", fn, (long long)seqlen, MSSM_MAX_SEQLEN);
    if (!prod_ok(batch, d_inner, seqlen, nullptr) || !prod_ok(batch, d_inner, d_state, nullptr))
        return fail(MSSM_ERR_SHAPE, "%s: tensor too large", fn);
    if (batch == 0 || d_inner == 0) return MSSM_OK;
    CHECK_OPT(h0);
    CHECK_OPT(h_final);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (seqlen == 0) {
        if (!h_final) return MSSM_OK;
        return launched(fn, mssm::launch_copy_or_zero(h_final, h0, batch * d_inner * d_state, s));
    }
    CHECK_PTR(u);
    CHECK_PTR(delta);
    CHECK_PTR(A);
    CHECK_PTR(Bm);
    CHECK_PTR(Cm);
    CHECK_PTR(y);
    CHECK_OPT(Dskip);
    CHECK_OPT(z);
    const int64_t blocks = ((d_inner + 63) / 64) * batch;
    if (blocks > INT32_MAX) return fail(MSSM_ERR_UNSUPPORTED, "%s: batch*d_inner too large", fn);
    float* ckpt = nullptr;
    if (save) {
        const size_t need = mssm::s6_bwd_workspace_bytes(batch, d_inner, seqlen, d_state);
        if (!workspace || workspace_bytes < need)
            return fail(MSSM_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need, workspace_bytes);
        CHECK_OPT(workspace);
        if (mssm::s6_bwd_ckpt_floats(1, d_inner, seqlen, d_state) * 4 >= (int64_t(1) << 31))
            return fail(MSSM_ERR_UNSUPPORTED, "%s: saved states of one batch row exceed 2 GiB", fn);
        ckpt = static_cast<float*>(workspace);
    }
    mssm::S6Params p{u, delta, Bm, Cm, z, A, Dskip, h0, y, h_final, batch, d_inner, (int32_t)seqlen, (int32_t)d_state,
                     ckpt};
    return launched(fn, mssm::launch_s6_scan(p, dtype == MSSM_BF16, zoh, s));
}

int mssm_selective_scan_fwd(const void* u, const void* delta, const float* A, const void* Bm,
                            const void* Cm, const float* Dskip, const void* z, const float* h0,
                            void* y, float* h_final, int64_t batch, int64_t d_inner, int64_t seqlen,
                            int64_t d_state, mssm_dtype dtype, void* stream) {
    return scan_fwd("mssm_selective_scan_fwd", false, false, u, delta, A, Bm, Cm, Dskip, z, h0, y, h_final, batch,
                    d_inner, seqlen, d_state, nullptr, 0, dtype, stream);
}

int mssm_selective_scan_fwd_save(const void* u, const void* delta, const float* A, const void* Bm,
                                 const void* Cm, const float* Dskip, const void* z, const float* h0,
                                 void* y, float* h_final, int64_t batch, int64_t d_inner, int64_t seqlen,
                                 int64_t d_state, void* workspace, size_t workspace_bytes, mssm_dtype dtype,
                                 void* stream) {
    return scan_fwd("mssm_selective_scan_fwd_save", false, true, u, delta, A, Bm, Cm, Dskip, z, h0, y, h_final,
                    batch, d_inner, seqlen, d_state, workspace, workspace_bytes, dtype, stream);
}

int mssm_selective_scan_zoh_fwd(const void* u, const void* delta, const float* A, const void* Bm,
                                const void* Cm, const float* Dskip, const void* z, const float* h0,
                                void* y, float* h_final, int64_t batch, int64_t d_inner, int64_t seqlen,
                                int64_t d_state, mssm_dtype dtype, void* stream) {
    return scan_fwd("mssm_selective_scan_zoh_fwd", true, false, u, delta, A, Bm, Cm, Dskip, z, h0, y, h_final,
                    batch, d_inner, seqlen, d_state, nullptr, 0, dtype, stream);
}

int mssm_selective_scan_fused_fwd(const void* x, const float* conv_w, const float* conv_b, const void* conv_init,
                                  const void* delta_raw, const float* delta_bias, const float* A, const void* Bm,
                                  const void* Cm, const float* Dskip, const void* z, const float* h0, void* y,
                                  float* h_final, int64_t batch, int64_t d_inner, int64_t seqlen, int64_t d_state,
                                  int64_t d_conv, mssm_dtype dtype, void* stream) {
    static const char* fn = "mssm_selective_scan_fused_fwd";
    g_err.clear();
    if (dtype != MSSM_F32 && dtype != MSSM_BF16) return fail(MSSM_ERR_DTYPE, "%s: unknown dtype %d", fn, (int)dtype);
    if (batch < 0 || d_inner < 0 || seqlen < 0 || d_state < 0 || d_conv < 0)
        return fail(MSSM_ERR_SHAPE, "%s: negative dimension", fn);
    if (d_state < 1 || d_state > 64) return fail(MSSM_ERR_UNSUPPORTED, "%s: d_state %lld not in [1, 64]", fn, (long long)d_state);
    if (d_conv < 1 || d_conv > 4) return fail(MSSM_ERR_UNSUPPORTED, "%s: d_conv %lld not in [1, 4]", fn, (long long)d_conv);
    if (seqlen > MSSM_MAX_SEQLEN)
        return fail(MSSM_ERR_UNSUPPORTED, "%s: seqlen %lld above %lld", fn, (long long)seqlen, MSSM_MAX_SEQLEN);
    if (!prod_ok(batch, d_inner, seqlen, nullptr) || !prod_ok(batch, d_inner, d_state, nullptr))
        return fail(MSSM_ERR_SHAPE, "%s: tensor too large", fn);
    if (batch == 0 || d_inner == 0) return MSSM_OK;
    CHECK_OPT(h0);
    CHECK_OPT(h_final);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (seqlen == 0) {
        if (!h_final) return MSSM_OK;
        return launched(fn, mssm::launch_copy_or_zero(h_final, h0, batch * d_inner * d_state, s));
    }
    CHECK_PTR(x);
    CHECK_PTR(conv_w);
    CHECK_PTR(delta_raw);
    CHECK_PTR(A);
    CHECK_PTR(Bm);
    CHECK_PTR(Cm);
    CHECK_PTR(y);
    CHECK_OPT(conv_b);
    CHECK_OPT(conv_init);
    CHECK_OPT(delta_bias);
    CHECK_OPT(Dskip);
    CHECK_OPT(z);
    const int64_t blocks = ((d_inner + 63) / 64) * batch;
    if (blocks > INT32_MAX) return fail(MSSM_ERR_UNSUPPORTED, "%s: batch*d_inner too large", fn);
    mssm::S6Params p{x, delta_raw, Bm, Cm, z, A, Dskip, h0, y, h_final, batch, d_inner, (int32_t)seqlen,
                     (int32_t)d_state};
    mssm::S6FrontEnd fe{conv_w, conv_b, conv_init, delta_bias, (int32_t)d_conv};
    return launched(fn, mssm::launch_s6_scan_fused(p, fe, dtype == MSSM_BF16, s));
}

size_t mssm_selective_scan_bwd_workspace_size(int64_t batch, int64_t d_inner, int64_t seqlen, int64_t d_state) {
    if (batch < 0 || d_inner < 0 || seqlen < 0 || d_state < 1 || d_state > 64) return 0;
    if (!prod_ok(batch, d_inner, seqlen, nullptr) || !prod_ok(batch, d_inner, d_state, nullptr)) return 0;
    return mssm::s6_bwd_workspace_bytes(batch, d_inner, seqlen, d_state);
}

// saved: the workspace already holds the chunk-start states written by
// mssm_selective_scan_fwd_save, so the kernel skips its forward sweep.
static int scan_bwd(const char* fn, bool saved, const void* u, const void* delta, const float* A, const void* Bm,
                    const void* Cm, const float* Dskip, const void* z, const float* h0, const void* dout,
                    const float* dh_final, void* du, void* ddelta, float* dA, float* dB, float* dC, float* dD,
                    void* dz, float* dh0, int64_t batch, int64_t d_inner, int64_t seqlen, int64_t d_state,
                    void* workspace, size_t workspace_bytes, mssm_dtype dtype, void* stream) {
    g_err.clear();
    if (dtype != MSSM_F32 && dtype != MSSM_BF16) return fail(MSSM_ERR_DTYPE, "%s: unknown dtype %d", fn, (int)dtype);
    if (batch < 0 || d_inner < 0 || seqlen < 0 || d_state < 0)
        return fail(MSSM_ERR_SHAPE, "%s: negative dimension", fn);
    if (d_state < 1 || d_state > 64) return fail(MSSM_ERR_UNSUPPORTED, "%s: d_state %lld not in [1, 64]", fn, (long long)d_state);
    if (seqlen > MSSM_MAX_SEQLEN)
        return fail(MSSM_ERR_UNSUPPORTED, "%s: seqlen %lld above %lld", fn, (long long)seqlen, MSSM_MAX_SEQLEN);
    if (!prod_ok(batch, d_inner, seqlen, nullptr) || !prod_ok(batch, d_inner, d_state, nullptr))
        return fail(MSSM_ERR_SHAPE, "%s: tensor too large", fn);
    if (batch == 0 || d_inner == 0) return MSSM_OK;
    if (seqlen == 0) {
        // h_final = h0: dh0 = dh_final; no step, so dA = dD = 0.  The
        // per-token tensors are empty and not touched.
        CHECK_PTR(dA);
        CHECK_OPT(dD);
        CHECK_OPT(dh0);
        CHECK_OPT(dh_final);
        hipStream_t s = static_cast<hipStream_t>(stream);
        hipError_t e = mssm::launch_copy_or_zero(dA, nullptr, d_inner * d_state, s);
        if (e == hipSuccess && dD) e = mssm::launch_copy_or_zero(dD, nullptr, d_inner, s);
        if (e == hipSuccess && dh0) e = mssm::launch_copy_or_zero(dh0, dh_final, batch * d_inner * d_state, s);
        return launched(fn, e);
    }
    CHECK_PTR(u);
    CHECK_PTR(delta);
    CHECK_PTR(A);
    CHECK_PTR(Bm);
    CHECK_PTR(Cm);
    CHECK_PTR(dout);
    CHECK_PTR(du);
    CHECK_PTR(ddelta);
    CHECK_PTR(dA);
    CHECK_PTR(dB);
    CHECK_PTR(dC);
    CHECK_OPT(Dskip);
    CHECK_OPT(z);
    CHECK_OPT(h0);
    CHECK_OPT(dh_final);
    CHECK_OPT(dD);
    CHECK_OPT(dz);
    CHECK_OPT(dh0);
    if (z && !dz) return fail(MSSM_ERR_NULL, "%s: dz is NULL while z is given", fn);
    const size_t need = mssm::s6_bwd_workspace_bytes(batch, d_inner, seqlen, d_state);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(MSSM_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need, workspace_bytes);
    CHECK_OPT(workspace);
    const int64_t blocks = ((d_inner + 63) / 64) * batch;
    if (blocks > INT32_MAX) return fail(MSSM_ERR_UNSUPPORTED, "%s: batch*d_inner too large", fn);
    float* ws = static_cast<float*>(workspace);
    hipStream_t s = static_cast<hipStream_t>(stream);
    // Without saved states, the forward scan kernel writes them first (states
    // only: no C, no outputs) when one batch row's states fit its 32-bit
    // offsets; the backward kernel then starts from them, as after
    // mssm_selective_scan_fwd_save.  Otherwise the backward kernel runs its
    // own forward sweep.
    bool from_states = saved;
    if (!saved && mssm::s6_bwd_ckpt_floats(1, d_inner, seqlen, d_state) * 4 < (int64_t(1) << 31)) {
        mssm::S6Params f{u, delta, Bm, Cm, nullptr, A, nullptr, h0, const_cast<void*>(u), nullptr, batch, d_inner,
                         (int32_t)seqlen, (int32_t)d_state, ws};
        const hipError_t e = mssm::launch_s6_save_states(f, dtype == MSSM_BF16, s);
        if (e != hipSuccess) return launched(fn, e);
        from_states = true;
    }
    mssm::S6BwdParams p{u, delta, Bm, Cm, z, dout, A, Dskip, h0, dh_final, du, ddelta, dz, dA, dB, dC, dD, dh0,
                        ws, ws + mssm::s6_bwd_ckpt_floats(batch, d_inner, seqlen, d_state), batch, d_inner,
                        (int32_t)seqlen, (int32_t)d_state, from_states ? 1 : 0};
    return launched(fn, mssm::launch_s6_scan_bwd(p, dtype == MSSM_BF16, s));
}

int mssm_selective_scan_bwd(const void* u, const void* delta, const float* A, const void* Bm, const void* Cm,
                            const float* Dskip, const void* z, const float* h0, const void* dout,
                            const float* dh_final, void* du, void* ddelta, float* dA, float* dB, float* dC,
                            float* dD, void* dz, float* dh0, int64_t batch, int64_t d_inner, int64_t seqlen,
                            int64_t d_state, void* workspace, size_t workspace_bytes, mssm_dtype dtype,
                            void* stream) {
    return scan_bwd("mssm_selective_scan_bwd", false, u, delta, A, Bm, Cm, Dskip, z, h0, dout, dh_final, du, ddelta,
                    dA, dB, dC, dD, dz, dh0, batch, d_inner, seqlen, d_state, workspace, workspace_bytes, dtype,
                    stream);
}

int mssm_selective_scan_bwd_saved(const void* u, const void* delta, const float* A, const void* Bm,
                                  const void* Cm, const float* Dskip, const void* z, const float* h0,
                                  const void* dout, const float* dh_final, void* du, void* ddelta, float* dA,
                                  float* dB, float* dC, float* dD, void* dz, float* dh0, int64_t batch,
                                  int64_t d_inner, int64_t seqlen, int64_t d_state, void* workspace,
                                  size_t workspace_bytes, mssm_dtype dtype, void* stream) {
    return scan_bwd("mssm_selective_scan_bwd_saved", true, u, delta, A, Bm, Cm, Dskip, z, h0, dout, dh_final, du,
                    ddelta, dA, dB, dC, dD, dz, dh0, batch, d_inner, seqlen, d_state, workspace, workspace_bytes,
                    dtype, stream);
}

int mssm_state_update(float* state, const void* u, const void* delta, const float* A, const void* Bm,
                      const void* Cm, const float* Dskip, const void* z, void* y, int64_t batch,
                      int64_t d_inner, int64_t d_state, mssm_dtype dtype, void* stream) {
    static const char* fn = "mssm_state_update";
    g_err.clear();
    if (dtype != MSSM_F32 && dtype != MSSM_BF16) return fail(MSSM_ERR_DTYPE, "%s: unknown dtype %d", fn, (int)dtype);
    if (batch < 0 || d_inner < 0 || d_state < 0) return fail(MSSM_ERR_SHAPE, "%s: negative dimension", fn);
    if (d_state < 1 || d_state > 64) return fail(MSSM_ERR_UNSUPPORTED, "%s: d_state %lld not in [1, 64]", fn, (long long)d_state);
    int64_t nthreads = 0;
    if (!prod_ok(batch, d_inner, d_state, nullptr) || !prod_ok(batch, d_inner, 4, &nthreads))
        return fail(MSSM_ERR_SHAPE, "%s: tensor too large", fn);
    if (batch == 0 || d_inner == 0) return MSSM_OK;
    if ((nthreads + 255) / 256 > INT32_MAX) return fail(MSSM_ERR_UNSUPPORTED, "%s: batch*d_inner too large", fn);
    CHECK_PTR(state);
    CHECK_PTR(u);
    CHECK_PTR(delta);
    CHECK_PTR(A);
    CHECK_PTR(Bm);
    CHECK_PTR(Cm);
    CHECK_PTR(y);
    CHECK_OPT(Dskip);
    CHECK_OPT(z);
    mssm::SUParams p{state, u, delta, Bm, Cm, z, A, Dskip, y, batch, d_inner, (int32_t)d_state};
    return launched(fn, mssm::launch_state_update(p, dtype == MSSM_BF16, static_cast<hipStream_t>(stream)));
}

int mssm_ssd_state_update(float* state, const void* x, const void* dt, const float* A, const void* Bm,
                          const void* Cm, const float* Dskip, const void* z, void* y, int64_t batch,
                          int64_t nheads, int64_t headdim, int64_t d_state, int64_t ngroups, mssm_dtype dtype,
                          void* stream) {
    static const char* fn = "mssm_ssd_state_update";
    g_err.clear();
    if (dtype != MSSM_F32 && dtype != MSSM_BF16) return fail(MSSM_ERR_DTYPE, "%s: unknown dtype %d", fn, (int)dtype);
    if (batch < 0 || nheads < 0 || headdim < 0 || d_state < 0 || ngroups < 0)
        return fail(MSSM_ERR_SHAPE, "%s: negative dimension", fn);
    if (batch == 0 || nheads == 0 || headdim == 0) return MSSM_OK;
    if (ngroups < 1 || nheads % ngroups != 0)
        return fail(MSSM_ERR_SHAPE, "%s: nheads %lld not a multiple of ngroups %lld", fn, (long long)nheads,
                    (long long)ngroups);
    if (!mssm::ssd_state_update_supported(d_state))
        return fail(MSSM_ERR_UNSUPPORTED, "%s: d_state %lld (1 .. 256)", fn, (long long)d_state);
    int64_t rows = 0;
    if (!prod_ok(batch, nheads, headdim, &rows) || !prod_ok(rows, d_state, 1, nullptr) || nheads > INT32_MAX ||
        headdim > INT32_MAX || !prod_ok(batch, ngroups, d_state, nullptr))
        return fail(MSSM_ERR_SHAPE, "%s: tensor too large", fn);
    CHECK_PTR(state);
    CHECK_PTR(x);
    CHECK_PTR(dt);
    CHECK_PTR(A);
    CHECK_PTR(Bm);
    CHECK_PTR(Cm);
    CHECK_PTR(y);
    CHECK_OPT(Dskip);
    CHECK_OPT(z);
    mssm::SSDUParams p{state, x, dt, A, Bm, Cm, Dskip, z, y, batch, (int32_t)nheads, (int32_t)headdim,
                       (int32_t)d_state, (int32_t)ngroups};
    return launched(fn, mssm::launch_ssd_state_update(p, dtype == MSSM_BF16, static_cast<hipStream_t>(stream)));
}

size_t mssm_ssd_workspace_size(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                               int64_t d_state, int64_t ngroups, int64_t chunk) {
    if (batch < 0 || seqlen < 0 || nheads < 1 || headdim < 1 || d_state < 1 || ngroups < 1 || chunk < 1)
        return 0;
    // sizes mssm_ssd_chunk_fwd would reject as too large: 0, not a wrapped product
    int64_t hp = 0, gn = 0;
    if (!prod_ok(nheads, headdim, 1, &hp) || !prod_ok(ngroups, d_state, 1, &gn) ||
        !prod_ok(batch, seqlen, hp, nullptr) || !prod_ok(batch, hp, d_state, nullptr) ||
        !prod_ok(batch, seqlen, gn, nullptr))
        return 0;
    // enough for either kernel: the bf16 MFMA path's where the sizes fit it
    // (its tiles take more than the general kernel's scores), else the
    // general kernel's
    const size_t general = d_state <= 256 ? mssm::ssd_general_workspace_bytes(batch, seqlen, d_state, ngroups) : 0;
    if (!mssm::ssd_fast_supported(seqlen, nheads, headdim, d_state, ngroups, chunk)) return general;
    const size_t fast = mssm::ssd_fast_workspace_bytes(batch, seqlen, nheads, headdim, d_state, ngroups, chunk);
    return fast > general ? fast : general;
}

// scratch: the caller passed no workspace; once the arguments pass, this
// device's static scratch array (workspace_bytes long) is used instead, and a
// size above it is reported as the array's limit.
static int ssd_fwd(const char* fn, const void* x, const void* dt, const float* A, const void* Bm, const void* Cm,
                   const float* Dskip, const void* z, const float* h0, void* y, float* h_final, int64_t batch,
                   int64_t seqlen, int64_t nheads, int64_t headdim, int64_t d_state, int64_t ngroups, int64_t chunk,
                   void* workspace, size_t workspace_bytes, bool scratch, mssm_dtype dtype, void* stream) {
    g_err.clear();
    if (dtype != MSSM_F32 && dtype != MSSM_BF16) return fail(MSSM_ERR_DTYPE, "%s: unknown dtype %d", fn, (int)dtype);
    if (batch < 0 || seqlen < 0 || nheads < 0 || headdim < 0 || d_state < 0 || ngroups < 0 || chunk < 0)
        return fail(MSSM_ERR_SHAPE, "%s: negative dimension", fn);
    if (nheads < 1 || ngroups < 1 || nheads % ngroups != 0)
        return fail(MSSM_ERR_SHAPE, "%s: nheads %lld must be a positive multiple of ngroups %lld", fn,
                    (long long)nheads, (long long)ngroups);
    if (headdim < 1 || !mssm::ssd_general_supported(headdim, d_state))
        return fail(MSSM_ERR_UNSUPPORTED, "%s: headdim %lld / d_state %lld (headdim >= 1, 1 <= d_state <= 256)", fn,
                    (long long)headdim, (long long)d_state);
    if (chunk != 64 && chunk != 128 && chunk != 256)
        return fail(MSSM_ERR_UNSUPPORTED, "%s: chunk %lld (64, 128 or 256)", fn, (long long)chunk);
    if (seqlen > INT32_MAX || nheads > INT32_MAX || headdim > INT32_MAX)
        return fail(MSSM_ERR_UNSUPPORTED, "%s: size too large", fn);
    // bf16 at the sizes the bf16 MFMA kernels take runs there; everything else
    // in the general kernel on the fp32 matrix cores
    const bool fast = dtype == MSSM_BF16 && mssm::ssd_fast_supported(seqlen, nheads, headdim, d_state, ngroups, chunk);
    if (!prod_ok(batch, seqlen, nheads * headdim, nullptr) || !prod_ok(batch, nheads * headdim, d_state, nullptr) ||
        !prod_ok(batch, seqlen, ngroups * d_state, nullptr))
        return fail(MSSM_ERR_SHAPE, "%s: tensor too large", fn);
    if (batch == 0) return MSSM_OK;
    CHECK_OPT(h0);
    CHECK_OPT(h_final);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (seqlen == 0) {
        if (!h_final) return MSSM_OK;
        return launched(fn, mssm::launch_copy_or_zero(h_final, h0, batch * nheads * headdim * d_state, s));
    }
    CHECK_PTR(x);
    CHECK_PTR(dt);
    CHECK_PTR(A);
    CHECK_PTR(Bm);
    CHECK_PTR(Cm);
    CHECK_PTR(y);
    CHECK_OPT(Dskip);
    CHECK_OPT(z);
    const size_t need = fast ? mssm::ssd_fast_workspace_bytes(batch, seqlen, nheads, headdim, d_state, ngroups, chunk)
                             : mssm::ssd_general_workspace_bytes(batch, seqlen, d_state, ngroups);
    if (scratch) {
        if (need > workspace_bytes)
            return fail(MSSM_ERR_WORKSPACE,
                        "%s: these sizes need %zu bytes of scratch, above the %zu bytes of the static scratch "
                        "array (call mssm_ssd_chunk_fwd with a workspace instead)",
                        fn, need, workspace_bytes);
        const int rc = scratch_address(fn, &workspace);
        if (rc != MSSM_OK) return rc;
    }
    if (need > 0) {
        if (!workspace) return fail(MSSM_ERR_WORKSPACE, "%s: workspace is NULL (%zu bytes needed)", fn, need);
        if (!aligned16(workspace)) return fail(MSSM_ERR_ALIGN, "%s: workspace is not 16-byte aligned", fn);
        if (workspace_bytes < need)
            return fail(MSSM_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", fn, workspace_bytes, need);
    }
    mssm::SSDParams p{x, dt, A, Bm, Cm, Dskip, z, h0, y, h_final, workspace, batch, (int32_t)seqlen,
                      (int32_t)nheads, (int32_t)headdim, (int32_t)d_state, (int32_t)ngroups, (int32_t)chunk};
    return launched(fn, fast ? mssm::launch_ssd_fast(p, s) : mssm::launch_ssd_general(p, dtype == MSSM_BF16, s));
}

int mssm_ssd_chunk_fwd(const void* x, const void* dt, const float* A, const void* Bm, const void* Cm,
                       const float* Dskip, const void* z, const float* h0, void* y, float* h_final,
                       int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t d_state,
                       int64_t ngroups, int64_t chunk, void* workspace, size_t workspace_bytes,
                       mssm_dtype dtype, void* stream) {
    return ssd_fwd("mssm_ssd_chunk_fwd", x, dt, A, Bm, Cm, Dskip, z, h0, y, h_final, batch, seqlen, nheads, headdim,
                   d_state, ngroups, chunk, workspace, workspace_bytes, false, dtype, stream);
}

int mssm_ssd_chunk_fwd_noalloc(const void* x, const void* dt, const float* A, const void* Bm, const void* Cm,
                               const float* Dskip, const void* z, const float* h0, void* y, float* h_final,
                               int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t d_state,
                               int64_t ngroups, int64_t chunk, mssm_dtype dtype, void* stream) {
    // the scratch address is looked up after the arguments are checked
    return ssd_fwd("mssm_ssd_chunk_fwd_noalloc", x, dt, A, Bm, Cm, Dskip, z, h0, y, h_final, batch, seqlen, nheads,
                   headdim, d_state, ngroups, chunk, nullptr, kScratchBytes, true, dtype, stream);
}

}  // extern "C"
