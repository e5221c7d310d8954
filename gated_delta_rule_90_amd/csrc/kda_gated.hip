// kda_gated.hip - the gated recurrent attention of the ejkernel "recurrent"
// page (recurrent_attention(): query, key, value, the gates g, g_gamma, gk,
// gv, softmax_scale, initial_state, reverse, cu_seqlens), token by token.
//
// The page names the gates (query, key, value and layer level) and their
// shapes but gives no formula.  Reading taken: every gate is a log-space
// factor used as given, and per token, in order (or from the last token to
// the first with reverse):
//     S <- exp(g_gamma[b, h]) * Diag(exp(gk_t)) S Diag(exp(gv_t))
//     S <- S + k_t v_t^T
//     o_t = S^T (scale * exp(g_t) * q_t)
// Absent gates are zero.  There is no delta rule and no normalisation.
//
// Work split: one wave per (sequence, head, tile of C state columns), C = 16
// at dk <= 32 and 8 above.  Lane l holds column l % C of the tile and rows
// [(l / C) * R, +R) of it in registers (R = dk * C / 64, at most 16); the
// output's sum over the 64 / C row groups is a few lane-xor steps.  The
// state columns are independent (the value gate scales a column, the key
// gate a row), so the tiles of a head run in parallel.  The next token's
// inputs are loaded while the current token is computed.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

// state columns per wave at key dimension dk
template <int DK>
constexpr int cols_per_wave() { return DK >= 64 ? 8 : 16; }

struct GatedParams {
    const void* q;
    const void* k;
    const void* v;
    int in_bf16;
    const float* g;
    const float* g_gamma;
    int g_gamma_rows;
    const float* gk;
    const float* gv;
    const float* init;
    const int32_t* cu;
    int N, T, H, Hkv, dv;
    float scale;
    int reverse;
    void* o;
    int out_bf16;
    float* final_state;
};

__device__ __forceinline__ float ldg(const void* p, size_t i, int bf)
{
    if (bf) return __uint_as_float((uint32_t)static_cast<const uint16_t*>(p)[i] << 16);
    return static_cast<const float*>(p)[i];
}

template <int DK>
struct TokenIn {
    static constexpr int RPL = DK * cols_per_wave<DK>() / kWave;
    float q[RPL], k[RPL], g[RPL], gk[RPL];
    float v, gv;
};

template <int DK>
__device__ __forceinline__ void load_token(TokenIn<DK>& x, const GatedParams& p, int t, int h, int hk, int r0,
                                           int col)
{
    constexpr int RPL = TokenIn<DK>::RPL;
    const size_t th = (size_t)t * p.H + h, tkv = (size_t)t * p.Hkv + hk;
#pragma unroll
    for (int m = 0; m < RPL; ++m) {
        x.q[m] = ldg(p.q, th * DK + r0 + m, p.in_bf16);
        x.k[m] = ldg(p.k, tkv * DK + r0 + m, p.in_bf16);
        x.g[m] = p.g ? p.g[th * DK + r0 + m] : 0.f;
        x.gk[m] = p.gk ? p.gk[th * DK + r0 + m] : 0.f;
    }
    x.v = ldg(p.v, tkv * p.dv + col, p.in_bf16);
    x.gv = p.gv ? p.gv[th * p.dv + col] : 0.f;
}

template <int DK>
__global__ __launch_bounds__(kWave) void gated_recurrent_kernel(GatedParams p)
{
    constexpr int GT = cols_per_wave<DK>();
    constexpr int RPL = TokenIn<DK>::RPL;
    const int lane = threadIdx.x;
    const int j = lane % GT, rg = lane / GT;
    const int col = blockIdx.x * GT + j;
    const int h = blockIdx.y, n = blockIdx.z;
    const int hk = h / (p.H / p.Hkv);
    const int r0 = rg * RPL;
    int t0, t1;
    if (p.cu) {
        t0 = min(max(p.cu[n], 0), p.T);
        t1 = min(max(p.cu[n + 1], t0), p.T);
    } else {
        t0 = n * p.T;
        t1 = t0 + p.T;
    }
    const size_t soff = ((size_t)n * p.H + h) * DK;
    float S[RPL];
#pragma unroll
    for (int m = 0; m < RPL; ++m) S[m] = p.init ? p.init[(soff + r0 + m) * p.dv + col] : 0.f;
    const float lg = p.g_gamma ? p.g_gamma[(size_t)min(n, p.g_gamma_rows - 1) * p.H + h] : 0.f;
    const int len = t1 - t0;
    TokenIn<DK> cur, nxt;
    if (len > 0) load_token<DK>(cur, p, p.reverse ? t1 - 1 : t0, h, hk, r0, col);
    for (int m = 0; m < len; ++m) {
        const int t = p.reverse ? t1 - 1 - m : t0 + m;
        if (m + 1 < len) load_token<DK>(nxt, p, p.reverse ? t - 1 : t + 1, h, hk, r0, col);
        const float ec = expf(cur.gv + lg);
        float part = 0.f;
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
            const float f = (p.gk ? expf(cur.gk[r]) : 1.f) * ec;
            S[r] = fmaf(S[r], f, cur.k[r] * cur.v);
            const float qt = p.scale * (p.g ? expf(cur.g[r]) : 1.f) * cur.q[r];
            part = fmaf(S[r], qt, part);
        }
        if (GT == 8) part += __shfl_xor(part, 8);
        part += __shfl_xor(part, 16);
        part += __shfl_xor(part, 32);
        if (rg == 0) {
            const size_t oi = ((size_t)t * p.H + h) * p.dv + col;
            if (p.out_bf16) static_cast<bf16_t*>(p.o)[oi] = from_f32<bf16_t>(part);
            else static_cast<float*>(p.o)[oi] = part;
        }
        cur = nxt;
    }
    if (p.final_state) {
#pragma unroll
        for (int m = 0; m < RPL; ++m) p.final_state[(soff + r0 + m) * p.dv + col] = S[m];
    }
}

template <int DK>
hipError_t launch_dk(const GatedParams& p, hipStream_t st)
{
    const dim3 grid((unsigned)(p.dv / cols_per_wave<DK>()), (unsigned)p.H, (unsigned)p.N);
    hipLaunchKernelGGL(gated_recurrent_kernel<DK>, grid, dim3(kWave), 0, st, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gated(const GatedArgs& a, hipStream_t st)
{
    GatedParams p{};
    p.q = a.q; p.k = a.k; p.v = a.v; p.in_bf16 = a.in_bf16;
    p.g = a.g; p.g_gamma = a.g_gamma; p.g_gamma_rows = a.g_gamma_rows; p.gk = a.gk; p.gv = a.gv;
    p.init = a.init; p.cu = a.cu;
    p.N = a.N; p.T = a.T; p.H = a.H; p.Hkv = a.Hkv; p.dv = a.dv;
    p.scale = a.scale; p.reverse = a.reverse;
    p.o = a.o; p.out_bf16 = a.out_bf16; p.final_state = a.final_state;
    switch (a.dk) {
    case 16: return launch_dk<16>(p, st);
    case 32: return launch_dk<32>(p, st);
    case 64: return launch_dk<64>(p, st);
    default: return launch_dk<128>(p, st);
    }
}

}  // namespace kda
