// kda_api.cpp - the C ABI of libkda.so: argument validation, routing to the
// kernels, status codes and the thread-local error message.  Every
// host-detectable error is reported before any HIP call is made.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/kda.h"
#include "kda_internal.h"

namespace {

thread_local std::string g_last_error;

kda_status_t fail(kda_status_t st, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

kda_status_t ok()
{
    g_last_error.clear();
    return KDA_OK;
}

bool dim_ok(int32_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }

kda_status_t hip_status(hipError_t e, const char* what)
{
    if (e != hipSuccess) return fail(KDA_EHIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

constexpr uint32_t kKnownFlags = KDA_QK_L2NORM | KDA_CHUNKED | KDA_EJK;

}  // namespace

extern "C" {

int kda_abi_version(void) { return KDA_ABI_VERSION; }

const char* kda_last_error(void) { return g_last_error.c_str(); }

size_t kda_prefill_workspace_bytes(int32_t num_seqs, int32_t B, int32_t T, int32_t H, int32_t dk,
                                   int32_t dv, kda_dtype_t in_dtype, uint32_t flags)
{
    if (B < 0 || T < 0 || H <= 0 || !dim_ok(dk) || !dim_ok(dv)) return 0;
    if (!(flags & KDA_CHUNKED) || (in_dtype != KDA_BF16 && in_dtype != KDA_F32)) return 0;
    const bool packed = num_seqs > 0 && B == 1;
    const int N = packed ? num_seqs : B;
    if (in_dtype == KDA_BF16) {
        kda::PrefillArgs probe{};
        probe.in_bf16 = true;
        probe.ejk = (flags & KDA_EJK) != 0;
        probe.dk = dk;
        probe.dv = dv;
        probe.g = reinterpret_cast<const float*>(1);
        probe.a_log = reinterpret_cast<const float*>(1);
        if (kda::chunked_supported(probe)) return kda::chunked_workspace_bytes(N, T, H, dk, dv, packed);
    }
    if (kda::prefill16_preferred(N, H, dk)) return kda::prefill16_workspace_bytes(N, T, H, dk, packed);
    return 0;
}

// kda_prefill and kda_prefill_noalloc: with noalloc set, the chunked MFMA
// route takes its workspace from the library's fixed scratch array instead of
// workspace / workspace_bytes.
static kda_status_t prefill_impl(const void* q, const void* k, const void* v, kda_dtype_t in_dtype,
                                 const float* g, const float* beta, const float* a_log,
                                 const float* dt_bias, const float* initial_state,
                                 const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T,
                                 int32_t H, int32_t Hkv, int32_t dk, int32_t dv, float scale,
                                 float lower_bound, int32_t chunk_size, uint32_t flags, void* o,
                                 kda_dtype_t out_dtype, float* final_state, void* workspace,
                                 size_t workspace_bytes, void* stream, bool noalloc)
{
    if (flags & ~kKnownFlags) return fail(KDA_EINVAL, "kda_prefill: unknown flag bits 0x%x", flags & ~kKnownFlags);
    const bool ejk = (flags & KDA_EJK) != 0;
    const bool chunked = (flags & KDA_CHUNKED) != 0;
    if (B < 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0)
        return fail(KDA_EINVAL, "kda_prefill: bad sizes B=%d T=%d H=%d dk=%d dv=%d", B, T, H, dk, dv);
    if (in_dtype != KDA_F32 && in_dtype != KDA_BF16) return fail(KDA_EINVAL, "kda_prefill: unknown in_dtype %d", (int)in_dtype);
    if (out_dtype != KDA_F32 && out_dtype != KDA_BF16) return fail(KDA_EINVAL, "kda_prefill: unknown out_dtype %d", (int)out_dtype);
    if (cu_seqlens) {
        if (B != 1) return fail(KDA_EINVAL, "kda_prefill: cu_seqlens requires B == 1 (got %d)", B);
        if (num_seqs < 0) return fail(KDA_EINVAL, "kda_prefill: num_seqs must be >= 0 with cu_seqlens");
    } else if (num_seqs != 0 && num_seqs != B) {
        return fail(KDA_EINVAL, "kda_prefill: num_seqs (%d) must be 0 or B (%d) without cu_seqlens", num_seqs, B);
    }
    if (Hkv == 0) Hkv = H;
    if (Hkv < 0 || H % Hkv != 0)
        return fail(KDA_EINVAL, "kda_prefill: Hkv (%d) must divide H (%d)", Hkv, H);
    const int N = cu_seqlens ? num_seqs : B;
    const bool has_tokens = (cu_seqlens ? (T > 0 && N > 0) : (B > 0 && T > 0));
    if (has_tokens) {
        if (!q || !k || !v || !beta || !o) return fail(KDA_EINVAL, "kda_prefill: q, k, v, beta and o are required");
        if (!ejk && (!g || !a_log)) return fail(KDA_EINVAL, "kda_prefill: KDA mode needs g and a_log");
    }
    if (!ejk && !(std::isfinite(lower_bound) && lower_bound <= 0.f))
        return fail(KDA_EINVAL, "kda_prefill: lower_bound must be finite and <= 0 (got %g)", (double)lower_bound);
    if (!dim_ok(dk) || !dim_ok(dv))
        return fail(KDA_EUNSUPPORTED, "kda_prefill: dk and dv must be in {16, 32, 64, 128} (got %d, %d)", dk, dv);
    if (in_dtype == KDA_F32 && out_dtype == KDA_BF16)
        return fail(KDA_EUNSUPPORTED, "kda_prefill: bf16 output needs bf16 input");
    if (chunked && chunk_size != 64)
        return fail(KDA_EUNSUPPORTED, "kda_prefill: the chunked path implements chunk_size 64 (got %d)", chunk_size);
    if (H > 65535 || N > 65535)
        return fail(KDA_EUNSUPPORTED, "kda_prefill: H and the number of sequences must be <= 65535 (got %d, %d)", H, N);
    if (N == 0) return ok();
    if (!has_tokens && !final_state) return ok();

    kda::PrefillArgs a{};
    a.q = q; a.k = k; a.v = v;
    a.in_bf16 = in_dtype == KDA_BF16;
    a.g = g; a.beta = beta; a.a_log = a_log; a.dt_bias = dt_bias;
    a.init = initial_state;
    a.cu = cu_seqlens;
    a.N = N;
    a.T = T;
    a.H = H; a.dk = dk; a.dv = dv;
    a.Hkv = Hkv;
    a.scale = (scale > 0.f) ? scale : 1.0f / std::sqrt((float)dk);  // NaN also selects the default
    a.lower_bound = lower_bound;
    a.l2norm = (flags & KDA_QK_L2NORM) != 0;
    a.ejk = ejk;
    a.o = o;
    a.out_bf16 = out_dtype == KDA_BF16;
    a.final_state = final_state;
    a.workspace = workspace;
    a.workspace_bytes = workspace_bytes;

    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    // Both chunked kernels move q, k and (KDA) g 16 bytes per lane, and in KDA
    // mode scale by decay factors that stay inside float32's range only for
    // lower_bound >= -5.  A call outside that takes the token-by-token kernel,
    // which computes the same function step by step, on every input dtype.
    auto a16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
    const bool chunk_ok = has_tokens && chunked && (ejk || lower_bound >= -5.0f) &&
                          a16(q) && a16(k) && (ejk || a16(g));
    if (chunk_ok && kda::chunked_supported(a) && a16(v) && a16(o)) {
        // the MFMA kernel also moves v and o 16 bytes per lane
        const size_t need = kda::chunked_workspace_bytes(N, T, H, dk, dv, cu_seqlens != nullptr);
        // a dense batch also runs with less, in segments of whole chunks (the
        // same result bit for bit); packed sequences need the whole records
        const size_t least = cu_seqlens ? need : kda::chunked_min_workspace_bytes(N, H, dk, dv, final_state == nullptr);
        if (noalloc) {
            if (least > (size_t)KDA_NOALLOC_SCRATCH_BYTES)
                return fail(KDA_EUNSUPPORTED, "kda_prefill_noalloc: the call needs %zu bytes of scratch, "
                            "more than the library's fixed %zu", least, (size_t)KDA_NOALLOC_SCRATCH_BYTES);
            const hipError_t e = kda::noalloc_scratch(&a.workspace);
            if (e != hipSuccess) return hip_status(e, "kda_prefill_noalloc: address of the scratch array");
            a.workspace_bytes = KDA_NOALLOC_SCRATCH_BYTES;
        } else if (need > 0 && (!workspace || workspace_bytes < least)) {
            return fail(KDA_EINVAL, "kda_prefill: workspace of %zu bytes required (got %zu; a dense batch "
                        "runs in segments from %zu)", need, workspace_bytes, least);
        }
        return hip_status(kda::launch_chunked(a, st), "kda_prefill (chunked)");
    }
    if (chunk_ok && kda::chunked_f32_supported(a)) {
        // with H dk >= 128 the float32 arithmetic runs as two kernels on
        // 16-token chunks when the workspace (or the fixed scratch) holds their
        // operand blocks; else as the one kernel, which needs none
        if (kda::prefill16_preferred(N, H, dk)) {
            const size_t need = kda::prefill16_workspace_bytes(N, T, H, dk, cu_seqlens != nullptr);
            void* ws = nullptr;
            if (noalloc) {
                if (need <= (size_t)KDA_NOALLOC_SCRATCH_BYTES) {
                    const hipError_t e = kda::noalloc_scratch(&ws);
                    if (e != hipSuccess) return hip_status(e, "kda_prefill_noalloc: address of the scratch array");
                }
            } else if (workspace && workspace_bytes >= need) {
                ws = workspace;
            }
            if (ws) {
                a.workspace = ws;
                a.workspace_bytes = need;
                return hip_status(kda::launch_prefill16(a, st), "kda_prefill (chunked float32, 16-token chunks)");
            }
        }
        return hip_status(kda::launch_chunked_f32(a, st), "kda_prefill (chunked float32)");
    }
    // token-by-token path; with T == 0 it only carries initial_state to final_state
    return hip_status(kda::launch_recurrent(a, st), "kda_prefill (recurrent)");
}

kda_status_t kda_prefill(const void* q, const void* k, const void* v, kda_dtype_t in_dtype,
                         const float* g, const float* beta, const float* a_log,
                         const float* dt_bias, const float* initial_state,
                         const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T,
                         int32_t H, int32_t Hkv, int32_t dk, int32_t dv, float scale, float lower_bound,
                         int32_t chunk_size, uint32_t flags, void* o, kda_dtype_t out_dtype,
                         float* final_state, void* workspace, size_t workspace_bytes,
                         void* stream)
{
    return prefill_impl(q, k, v, in_dtype, g, beta, a_log, dt_bias, initial_state, cu_seqlens, num_seqs,
                        B, T, H, Hkv, dk, dv, scale, lower_bound, chunk_size, flags, o, out_dtype,
                        final_state, workspace, workspace_bytes, stream, false);
}

kda_status_t kda_prefill_noalloc(const void* q, const void* k, const void* v, kda_dtype_t in_dtype,
                                 const float* g, const float* beta, const float* a_log,
                                 const float* dt_bias, const float* initial_state,
                                 const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T,
                                 int32_t H, int32_t Hkv, int32_t dk, int32_t dv, float scale,
                                 float lower_bound, int32_t chunk_size, uint32_t flags, void* o,
                                 kda_dtype_t out_dtype, float* final_state, void* stream)
{
    return prefill_impl(q, k, v, in_dtype, g, beta, a_log, dt_bias, initial_state, cu_seqlens, num_seqs,
                        B, T, H, Hkv, dk, dv, scale, lower_bound, chunk_size, flags, o, out_dtype,
                        final_state, nullptr, 0, stream, true);
}

size_t kda_prefill_backward_workspace_bytes(int32_t num_seqs, int32_t B, int32_t T, int32_t H, int32_t Hkv,
                                            int32_t dk, int32_t dv)
{
    if (B < 0 || T < 0 || H <= 0 || !dim_ok(dk) || !dim_ok(dv)) return 0;
    if (Hkv == 0) Hkv = H;
    if (Hkv < 0 || H % Hkv != 0) return 0;
    const bool packed = num_seqs > 0 && B == 1;
    return kda::backward_workspace_bytes(packed ? num_seqs : B, T, H, Hkv, dk, dv, packed);
}

kda_status_t kda_prefill_backward(const void* q, const void* k, const void* v, kda_dtype_t in_dtype,
                                  const float* g, const float* beta, const float* a_log,
                                  const float* dt_bias, const float* initial_state,
                                  const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T,
                                  int32_t H, int32_t Hkv, int32_t dk, int32_t dv, float scale,
                                  float lower_bound, uint32_t flags, const void* d_o, kda_dtype_t do_dtype,
                                  const float* d_final_state, float* dq, float* dk_out, float* dv_out,
                                  float* dg, float* dbeta, float* da_log, float* ddt_bias,
                                  float* d_initial_state, void* workspace, size_t workspace_bytes,
                                  void* stream)
{
    if (flags & ~kKnownFlags)
        return fail(KDA_EINVAL, "kda_prefill_backward: unknown flag bits 0x%x", flags & ~kKnownFlags);
    const bool ejk = (flags & KDA_EJK) != 0;
    if (B < 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0)
        return fail(KDA_EINVAL, "kda_prefill_backward: bad sizes B=%d T=%d H=%d dk=%d dv=%d", B, T, H, dk, dv);
    if (in_dtype != KDA_F32 && in_dtype != KDA_BF16)
        return fail(KDA_EINVAL, "kda_prefill_backward: unknown in_dtype %d", (int)in_dtype);
    if (do_dtype != KDA_F32 && do_dtype != KDA_BF16)
        return fail(KDA_EINVAL, "kda_prefill_backward: unknown do_dtype %d", (int)do_dtype);
    if (cu_seqlens) {
        if (B != 1) return fail(KDA_EINVAL, "kda_prefill_backward: cu_seqlens requires B == 1 (got %d)", B);
        if (num_seqs < 0) return fail(KDA_EINVAL, "kda_prefill_backward: num_seqs must be >= 0 with cu_seqlens");
    } else if (num_seqs != 0 && num_seqs != B) {
        return fail(KDA_EINVAL, "kda_prefill_backward: num_seqs (%d) must be 0 or B (%d) without cu_seqlens",
                    num_seqs, B);
    }
    if (Hkv == 0) Hkv = H;
    if (Hkv < 0 || H % Hkv != 0)
        return fail(KDA_EINVAL, "kda_prefill_backward: Hkv (%d) must divide H (%d)", Hkv, H);
    const int N = cu_seqlens ? num_seqs : B;
    const bool has_tokens = (cu_seqlens ? (T > 0 && N > 0) : (B > 0 && T > 0));
    if (has_tokens) {
        if (!q || !k || !v || !beta || !d_o || !dq || !dk_out || !dv_out || !dbeta)
            return fail(KDA_EINVAL, "kda_prefill_backward: q, k, v, beta, d_o, dq, dk, dv and dbeta are required");
        if (!ejk && (!g || !a_log || !dg))
            return fail(KDA_EINVAL, "kda_prefill_backward: KDA mode needs g, a_log and dg");
    }
    if (!ejk && !(std::isfinite(lower_bound) && lower_bound <= 0.f))
        return fail(KDA_EINVAL, "kda_prefill_backward: lower_bound must be finite and <= 0 (got %g)",
                    (double)lower_bound);
    if (!dim_ok(dk) || !dim_ok(dv))
        return fail(KDA_EUNSUPPORTED, "kda_prefill_backward: dk and dv must be in {16, 32, 64, 128} (got %d, %d)",
                    dk, dv);
    if (!ejk && lower_bound < -5.0f)
        return fail(KDA_EUNSUPPORTED, "kda_prefill_backward: KDA mode needs lower_bound >= -5 (got %g)",
                    (double)lower_bound);
    if (H > 65535 || N > 65535)
        return fail(KDA_EUNSUPPORTED, "kda_prefill_backward: H and the number of sequences must be <= 65535");
    if ((long long)H * N > (1LL << 26))
        return fail(KDA_EUNSUPPORTED, "kda_prefill_backward: H times the number of sequences must be <= 2^26");
    if (!cu_seqlens && (long long)B * T > 0x7fffffffLL)
        return fail(KDA_EUNSUPPORTED, "kda_prefill_backward: B * T must fit in 31 bits");
    // with no tokens the passes still run: they carry dL/d(final state) to
    // dL/d(initial state) and give zero parameter gradients
    if (N == 0) return ok();
    const size_t need = kda::backward_workspace_bytes(N, T, H, Hkv, dk, dv, cu_seqlens != nullptr);
    if (!workspace || workspace_bytes < need)
        return fail(KDA_EINVAL, "kda_prefill_backward: workspace of %zu bytes required (got %zu)", need,
                    workspace_bytes);
    kda::BackwardArgs a{};
    a.q = q; a.k = k; a.v = v;
    a.in_bf16 = in_dtype == KDA_BF16;
    a.g = g; a.beta = beta; a.a_log = a_log; a.dt_bias = dt_bias;
    a.init = initial_state;
    a.cu = cu_seqlens;
    a.N = N; a.T = T; a.H = H; a.Hkv = Hkv; a.dk = dk; a.dv = dv;
    a.scale = (scale > 0.f) ? scale : 1.0f / std::sqrt((float)dk);
    a.lower_bound = lower_bound;
    a.l2norm = (flags & KDA_QK_L2NORM) != 0;
    a.ejk = ejk;
    a.d_o = d_o;
    a.do_bf16 = do_dtype == KDA_BF16;
    a.d_final_state = d_final_state;
    a.dq = dq; a.dk_out = dk_out; a.dv_out = dv_out; a.dg = dg; a.dbeta = dbeta;
    a.da_log = ejk ? nullptr : da_log;
    a.ddt_bias = ejk ? nullptr : ddt_bias;
    a.d_initial_state = d_initial_state;
    a.workspace = workspace;
    return hip_status(kda::launch_backward(a, reinterpret_cast<hipStream_t>(stream)), "kda_prefill_backward");
}

size_t kda_recurrent_attention_workspace_bytes(int32_t num_seqs, int32_t B, int32_t T, int32_t H, int32_t dk,
                                               int32_t dv)
{
    const bool packed = num_seqs > 0;
    const int N = packed ? num_seqs : B;
    if (N < 0 || T < 0 || H <= 0 || !dim_ok(dk) || !dim_ok(dv) || (packed && B != 1)) return 0;
    return kda::gated_workspace_bytes(N, T, H, dk, packed);
}

kda_status_t kda_recurrent_attention(const void* q, const void* k, const void* v, kda_dtype_t in_dtype,
                                     const float* g, const float* g_gamma, const float* gk, const float* gv,
                                     const float* initial_state, const int32_t* cu_seqlens, int32_t num_seqs,
                                     int32_t B, int32_t T, int32_t H, int32_t Hkv, int32_t dk, int32_t dv,
                                     float scale, int32_t reverse, void* o, kda_dtype_t out_dtype,
                                     float* final_state, void* workspace, size_t workspace_bytes, void* stream)
{
    if (B < 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0)
        return fail(KDA_EINVAL, "kda_recurrent_attention: bad sizes B=%d T=%d H=%d dk=%d dv=%d", B, T, H, dk, dv);
    if (in_dtype != KDA_F32 && in_dtype != KDA_BF16)
        return fail(KDA_EINVAL, "kda_recurrent_attention: unknown in_dtype %d", (int)in_dtype);
    if (out_dtype != KDA_F32 && out_dtype != KDA_BF16)
        return fail(KDA_EINVAL, "kda_recurrent_attention: unknown out_dtype %d", (int)out_dtype);
    if (reverse != 0 && reverse != 1)
        return fail(KDA_EINVAL, "kda_recurrent_attention: reverse must be 0 or 1 (got %d)", reverse);
    if (cu_seqlens) {
        if (B != 1) return fail(KDA_EINVAL, "kda_recurrent_attention: cu_seqlens requires B == 1 (got %d)", B);
        if (num_seqs < 0) return fail(KDA_EINVAL, "kda_recurrent_attention: num_seqs must be >= 0 with cu_seqlens");
    } else if (num_seqs != 0 && num_seqs != B) {
        return fail(KDA_EINVAL, "kda_recurrent_attention: num_seqs (%d) must be 0 or B (%d) without cu_seqlens",
                    num_seqs, B);
    }
    if (Hkv == 0) Hkv = H;
    if (Hkv < 0 || H % Hkv != 0)
        return fail(KDA_EINVAL, "kda_recurrent_attention: Hkv (%d) must divide H (%d)", Hkv, H);
    const int N = cu_seqlens ? num_seqs : B;
    const bool has_tokens = (cu_seqlens ? (T > 0 && N > 0) : (B > 0 && T > 0));
    if (has_tokens && (!q || !k || !v || !o))
        return fail(KDA_EINVAL, "kda_recurrent_attention: q, k, v and o are required");
    if (!dim_ok(dk) || !dim_ok(dv))
        return fail(KDA_EUNSUPPORTED, "kda_recurrent_attention: dk and dv must be in {16, 32, 64, 128} (got %d, %d)",
                    dk, dv);
    if (in_dtype == KDA_F32 && out_dtype == KDA_BF16)
        return fail(KDA_EUNSUPPORTED, "kda_recurrent_attention: bf16 output needs bf16 input");
    if (H > 65535 || N > 65535)
        return fail(KDA_EUNSUPPORTED, "kda_recurrent_attention: H and the number of sequences must be <= 65535");
    if ((long long)H * N > (1LL << 26))
        return fail(KDA_EUNSUPPORTED, "kda_recurrent_attention: H times the number of sequences must be <= 2^26");
    if (!cu_seqlens && (long long)B * T > 0x7fffffffLL)
        return fail(KDA_EUNSUPPORTED, "kda_recurrent_attention: B * T must fit in 31 bits");
    if (N == 0 || (!has_tokens && !final_state)) return ok();
    const size_t need = kda::gated_workspace_bytes(N, T, H, dk, cu_seqlens != nullptr);
    if (!workspace || workspace_bytes < need)
        return fail(KDA_EINVAL, "kda_recurrent_attention: workspace of %zu bytes required (got %zu)", need,
                    workspace_bytes);
    kda::GatedArgs a{};
    a.q = q; a.k = k; a.v = v; a.in_bf16 = in_dtype == KDA_BF16;
    a.g = g; a.g_gamma = g_gamma; a.g_gamma_rows = cu_seqlens ? 1 : B; a.gk = gk; a.gv = gv;
    a.init = initial_state; a.cu = cu_seqlens;
    a.N = N; a.T = T; a.H = H; a.Hkv = Hkv; a.dk = dk; a.dv = dv;
    a.scale = (scale > 0.f) ? scale : 1.0f / std::sqrt((float)dk);
    a.reverse = reverse;
    a.o = o; a.out_bf16 = out_dtype == KDA_BF16; a.final_state = final_state;
    a.workspace = workspace;
    return hip_status(kda::launch_gated(a, reinterpret_cast<hipStream_t>(stream)), "kda_recurrent_attention");
}

kda_status_t kda_decode_step(const float* q, const float* k, const float* g, const float* v,
                             const float* beta, const float* a_log, const float* dt_bias,
                             float scale, float lower_bound, int32_t B, int32_t H, int32_t Hkv,
                             int32_t dk, int32_t dv, uint32_t flags, float* out, float* S, void* stream)
{
    if (flags & ~(KDA_QK_L2NORM | KDA_EJK))
        return fail(KDA_EINVAL, "kda_decode_step: unsupported flag bits 0x%x", flags & ~(KDA_QK_L2NORM | KDA_EJK));
    const bool ejk = (flags & KDA_EJK) != 0;
    if (B < 0 || H <= 0 || dk <= 0 || dv <= 0)
        return fail(KDA_EINVAL, "kda_decode_step: bad sizes B=%d H=%d dk=%d dv=%d", B, H, dk, dv);
    if (Hkv == 0) Hkv = H;
    if (Hkv < 0 || H % Hkv != 0)
        return fail(KDA_EINVAL, "kda_decode_step: Hkv (%d) must divide H (%d)", Hkv, H);
    if (B > 0) {
        if (!q || !k || !v || !beta || !out || !S) return fail(KDA_EINVAL, "kda_decode_step: q, k, v, beta, out and S are required");
        if (!ejk && (!g || !a_log)) return fail(KDA_EINVAL, "kda_decode_step: KDA mode needs g and a_log");
    }
    if (!ejk && !(std::isfinite(lower_bound) && lower_bound <= 0.f))
        return fail(KDA_EINVAL, "kda_decode_step: lower_bound must be finite and <= 0 (got %g)", (double)lower_bound);
    if (!dim_ok(dk) || !dim_ok(dv))
        return fail(KDA_EUNSUPPORTED, "kda_decode_step: dk and dv must be in {16, 32, 64, 128} (got %d, %d)", dk, dv);
    if ((long long)((B + 7) / 8) * 8 * H > 0x7fffffffLL) return fail(KDA_EUNSUPPORTED, "kda_decode_step: B * H too large");
    if (B == 0) return ok();
    kda::DecodeArgs a{};
    a.q = q; a.k = k; a.g = g; a.v = v; a.beta = beta; a.a_log = a_log; a.dt_bias = dt_bias;
    a.scale = (scale > 0.f) ? scale : 1.0f / std::sqrt((float)dk);
    a.lower_bound = lower_bound;
    a.B = B; a.H = H; a.dk = dk; a.dv = dv;
    a.Hkv = Hkv;
    a.l2norm = (flags & KDA_QK_L2NORM) != 0;
    a.ejk = ejk;
    a.out = out;
    a.S = S;
    return hip_status(kda::launch_decode(a, reinterpret_cast<hipStream_t>(stream)), "kda_decode_step");
}

}  // extern "C"
