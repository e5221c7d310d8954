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
// at dk <= 32, 8 at dk = 64 and 4 at dk = 128.  Lane l holds column l % C of
// the tile and rows [(l / C) * R, +R) of it in registers (R = dk * C / 64:
// 4 or 8); the output's sum over the 64 / C row groups is a few lane-xor
// steps.  The state columns are independent (the value gate scales a column,
// the key gate a row), so the tiles of a head run in parallel.  The inputs
// of the next RING tokens are in flight in a register ring while a token is
// computed: the loop is unrolled by the ring depth so the ring stays in
// registers, and loads past the sequence's end re-read its last token, so
// every iteration issues the same loads.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

// state columns per wave at key dimension dk (rows per lane: 4 at dk = 16,
// else 8)
template <int DK>
constexpr int cols_per_wave() { return DK >= 128 ? 4 : (DK >= 64 ? 8 : 16); }
constexpr int RING = 4;   // tokens whose inputs are in flight ahead of use

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

// RPL consecutive elements starting at element i of a float32 or bf16
// array; VEC: in 16-byte (8-byte for 4 bf16) loads, which needs i and the
// array 16-byte aligned (8-byte for bf16 at 4 elements)
template <int RPL, bool VEC>
__device__ __forceinline__ void load_row(float* out, const void* p, size_t i, int bf)
{
    if constexpr (VEC) {
        if (bf) {
            const uint16_t* b = static_cast<const uint16_t*>(p) + i;
            if constexpr (RPL == 8) {
                const uint4 w = *reinterpret_cast<const uint4*>(b);
                const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    out[2 * m] = __uint_as_float(ws[m] << 16);
                    out[2 * m + 1] = __uint_as_float(ws[m] & 0xffff0000u);
                }
            } else {
                const uint2 w = *reinterpret_cast<const uint2*>(b);
                out[0] = __uint_as_float(w.x << 16);
                out[1] = __uint_as_float(w.x & 0xffff0000u);
                out[2] = __uint_as_float(w.y << 16);
                out[3] = __uint_as_float(w.y & 0xffff0000u);
            }
        } else {
            const float4* f = reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
#pragma unroll
            for (int m = 0; m < RPL / 4; ++m) {
                const float4 x = f[m];
                out[4 * m] = x.x; out[4 * m + 1] = x.y; out[4 * m + 2] = x.z; out[4 * m + 3] = x.w;
            }
        }
    } else {
#pragma unroll
        for (int m = 0; m < RPL; ++m) out[m] = ldg(p, i + m, bf);
    }
}

template <int DK, bool VEC>
__device__ __forceinline__ void load_token(TokenIn<DK>& x, const GatedParams& p, int t, int h, int hk, int r0,
                                           int col)
{
    constexpr int RPL = TokenIn<DK>::RPL;
    const size_t th = (size_t)t * p.H + h, tkv = (size_t)t * p.Hkv + hk;
    load_row<RPL, VEC>(x.q, p.q, th * DK + r0, p.in_bf16);
    load_row<RPL, VEC>(x.k, p.k, tkv * DK + r0, p.in_bf16);
    if (p.g) load_row<RPL, VEC>(x.g, p.g, th * DK + r0, 0);
    if (p.gk) load_row<RPL, VEC>(x.gk, p.gk, th * DK + r0, 0);
    x.v = ldg(p.v, tkv * p.dv + col, p.in_bf16);
    x.gv = p.gv ? p.gv[th * p.dv + col] : 0.f;
}

template <int DK, bool VEC>
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
    // token of step m (clamped into the sequence for the ring's look-ahead)
    auto tok = [&](int m) {
        m = min(m, len - 1);
        return p.reverse ? t1 - 1 - m : t0 + m;
    };
    TokenIn<DK> ring[RING];
    if (len > 0) {
#pragma unroll
        for (int u = 0; u < RING; ++u) load_token<DK, VEC>(ring[u], p, tok(u), h, hk, r0, col);
    }
    for (int m0 = 0; m0 < len; m0 += RING) {
#pragma unroll
        for (int u = 0; u < RING; ++u) {
            const int m = m0 + u;
            if (m < len) {
                const TokenIn<DK>& x = ring[u];
                const float ec = expf(x.gv + lg);
                float part = 0.f;
#pragma unroll
                for (int r = 0; r < RPL; ++r) {
                    const float f = (p.gk ? expf(x.gk[r]) : 1.f) * ec;
                    S[r] = fmaf(S[r], f, x.k[r] * x.v);
                    const float qt = p.scale * (p.g ? expf(x.g[r]) : 1.f) * x.q[r];
                    part = fmaf(S[r], qt, part);
                }
                part = xor_sum_from<GT>(part);   // over the lanes of this column
                if (rg == 0) {
                    const size_t oi = ((size_t)tok(m) * p.H + h) * p.dv + col;
                    if (p.out_bf16) static_cast<bf16_t*>(p.o)[oi] = from_f32<bf16_t>(part);
                    else static_cast<float*>(p.o)[oi] = part;
                }
            }
            load_token<DK, VEC>(ring[u], p, tok(m + RING), h, hk, r0, col);
        }
    }
    if (p.final_state) {
#pragma unroll
        for (int m = 0; m < RPL; ++m) p.final_state[(soff + r0 + m) * p.dv + col] = S[m];
    }
}

template <int DK>
hipError_t launch_dk(const GatedParams& p, bool vec, hipStream_t st)
{
    const dim3 grid((unsigned)(p.dv / cols_per_wave<DK>()), (unsigned)p.H, (unsigned)p.N);
    if (vec) hipLaunchKernelGGL((gated_recurrent_kernel<DK, true>), grid, dim3(kWave), 0, st, p);
    else hipLaunchKernelGGL((gated_recurrent_kernel<DK, false>), grid, dim3(kWave), 0, st, p);
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
    // rows move 16 bytes per lane when every row array is 16-byte aligned
    auto a16 = [](const void* x) { return (reinterpret_cast<uintptr_t>(x) & 15u) == 0; };
    const bool vec = a16(a.q) && a16(a.k) && (!a.g || a16(a.g)) && (!a.gk || a16(a.gk));
    switch (a.dk) {
    case 16: return launch_dk<16>(p, vec, st);
    case 32: return launch_dk<32>(p, vec, st);
    case 64: return launch_dk<64>(p, vec, st);
    default: return launch_dk<128>(p, vec, st);
    }
}

}  // namespace kda
