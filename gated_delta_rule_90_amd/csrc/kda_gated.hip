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

// ---------------------------------------------------------------------------
// The chunked form (what kda_recurrent_attention runs): chunks of C = 16
// tokens in processing order.  With a_t = gk_t + g_gamma (key axis) and gv_t
// (value axis), bk_r, bv_r their cumulative sums over the chunk's rows
// r = 0..15 and qt_r = scale e^{g_r} q_r:
//     O_rj  = e^{bv_rj} sum_i qt_ri e^{bk_ri} S0_ij
//             + sum_{s<=r} A_rs e^{bv_rj - bv_sj} v_sj,
//     A_rs  = sum_i qt_ri k_si e^{bk_ri - bk_si}
//     S1_ij = e^{bk_Ci + bv_Cj} S0_ij + sum_s (e^{bk_Ci - bk_si} k_si)(e^{bv_Cj - bv_sj} v_sj)
// (C the chunk's last row), an exact regrouping of the token recurrence.  A
// is the MFMA product (qt e^{bk - bk_0})(k e^{bk_0 - bk})^T when every key
// channel's log-decay over the chunk stays within 120 (log2 units) of its
// first row's, which keeps both factors inside float32's range; the page puts
// no bound on the gates, so a chunk that spans more forms e^{bk_ri - bk_si}
// element by element (a per-chunk, workgroup-uniform choice).  The value-axis
// factors e^{bv_rj - bv_sj} are formed element by element.  For s <= r these
// factors are at most 1 when the gates are at most 0.  The inter-chunk
// read-out and the state update run on 16x16x4 float32 MFMA.  One 256-thread workgroup per (sequence, head, 16
// state columns); the state tile stays in LDS, transposed.  Rows past the
// sequence are neutral (q = k = v = 0, every gate 0).  The next two chunks'
// inputs are in flight in a register ring.
constexpr int GC = 16;    // chunk rows
constexpr int GJ = 16;    // state columns per workgroup
constexpr int GTH = 256;  // threads per workgroup

template <int DK>
struct GatedLds {
    static constexpr int RS = DK + 4;   // row stride of [16][dk] tiles: 16-byte aligned rows
    alignas(16) float QT[GC * RS];   // scale e^{g} q
    alignas(16) float KT[GC * RS];   // k
    alignas(16) float BK[GC * RS];   // gk + g_gamma, then its cumulative sum bk
    alignas(16) float QE[GC * RS];   // qt e^{bk}
    alignas(16) float KC[GC * RS];   // e^{bk_C - bk} k
    alignas(16) float QF[GC * RS];   // qt e^{bk - bk_0}  (A's left factor)
    alignas(16) float KF[GC * RS];   // k e^{bk_0 - bk}   (A's right factor)
    alignas(16) float ST[GJ * RS];   // the state tile, transposed: S[i][j] at ST[j * RS + i]
    float VV[GC][GJ + 1];   // v
    float BV[GC][GJ + 1];   // gv, then its cumulative sum bv
    float VC[GC][GJ + 1];   // e^{bv_C - bv} v
    float AM[GC][GC + 1];   // A (s <= r)
    float OI[GC][GJ + 1];   // the inter-chunk part of O, before its e^{bv} factor
    float EKC[DK];          // e^{bk_C}
    float EVC[GJ];          // e^{bv_C}
    int wide;               // some channel's log-decay spans more than the factor range
};

typedef float gf32x4_t __attribute__((ext_vector_type(4)));

// D += A B on a 16x16x4 float32 MFMA: lane l supplies A[l % 16][l / 16] and
// B[l / 16][l % 16] and holds D[4 (l / 16) + e][l % 16] in element e.
__device__ __forceinline__ gf32x4_t gmfma4(float a, float b, gf32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <int DK, typename Tin, typename Tout>
__global__ __launch_bounds__(GTH) void gated_chunk_kernel(GatedParams p)
{
    using LT = GatedLds<DK>;
    constexpr int RS = LT::RS;
    constexpr int NE = GC * DK / GTH;   // row elements of q, k and the gates per thread
    static_assert(NE >= 1 && NE * GTH == GC * DK && DK + GJ <= GTH, "dk in {16, 32, 64, 128}");
    __shared__ LT L;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int lm = lane & 15, lk = lane >> 4;
    const int r16 = tid >> 4, c16 = tid & 15;
    const int j0 = blockIdx.x * GJ, h = blockIdx.y, n = blockIdx.z;
    const int H = p.H, HKV = p.Hkv, DV = p.dv;
    const int hk = h / (H / HKV);
    int t0, t1;
    if (p.cu) {
        t0 = min(max(p.cu[n], 0), p.T);
        t1 = min(max(p.cu[n + 1], t0), p.T);
    } else {
        t0 = n * p.T;
        t1 = t0 + p.T;
    }
    const int len = t1 - t0;
    const int nch = (len + GC - 1) / GC;
    const size_t soff = ((size_t)n * H + h) * DK;
    for (int e = tid; e < DK * GJ; e += GTH) {
        const int i = e / GJ, j = e % GJ;
        L.ST[j * RS + i] = p.init ? p.init[(soff + i) * DV + j0 + j] : 0.f;
    }
    const float lg = p.g_gamma ? p.g_gamma[(size_t)min(n, p.g_gamma_rows - 1) * H + h] : 0.f;
    const Tin* q = static_cast<const Tin*>(p.q);
    const Tin* k = static_cast<const Tin*>(p.k);
    const Tin* v = static_cast<const Tin*>(p.v);
    // the token of step m of the sequence (m clamped into it: rows past the end
    // read a valid row and are zeroed where used)
    auto tok = [&](int m) -> size_t {
        m = min(m, len - 1);
        return (size_t)(p.reverse ? t1 - 1 - m : t0 + m);
    };
    struct Raw {
        Tin q[NE], k[NE];
        float g[NE], gk[NE];
        Tin v;
        float gv;
    };
    auto load = [&](Raw& R, int c) {
#pragma unroll
        for (int m = 0; m < NE; ++m) {
            const int e = tid + m * GTH;
            const int r = e / DK, i = e % DK;
            const size_t t = tok(c * GC + r);
            R.q[m] = q[(t * H + h) * DK + i];
            R.k[m] = k[(t * HKV + hk) * DK + i];
            R.g[m] = p.g ? p.g[(t * H + h) * DK + i] : 0.f;
            R.gk[m] = p.gk ? p.gk[(t * H + h) * DK + i] : 0.f;
        }
        const size_t t = tok(c * GC + r16);
        R.v = v[(t * HKV + hk) * DV + j0 + c16];
        R.gv = p.gv ? p.gv[(t * H + h) * DV + j0 + c16] : 0.f;
    };
    constexpr int FD = 2;   // chunks in flight ahead
    Raw ring[FD];
    if (nch > 0) {
#pragma unroll
        for (int u = 0; u < FD; ++u) load(ring[u], min(u, nch - 1));
    }
    auto chunk = [&](Raw& R, int c) {
        const int lc = min(GC, len - c * GC);   // rows of this chunk (<= 0: a padding chunk)
        // 1. the inputs to LDS, zero past the rows
#pragma unroll
        for (int m = 0; m < NE; ++m) {
            const int e = tid + m * GTH;
            const int r = e / DK, i = e % DK;
            const bool in = r < lc;
            // the gates in log2 units from here on
            L.QT[r * RS + i] = in ? p.scale * __builtin_amdgcn_exp2f(R.g[m] * kLog2e) * to_f32(R.q[m]) : 0.f;
            L.KT[r * RS + i] = in ? to_f32(R.k[m]) : 0.f;
            L.BK[r * RS + i] = in ? (R.gk[m] + lg) * kLog2e : 0.f;
        }
        {
            const bool in = r16 < lc;
            L.VV[r16][c16] = in ? to_f32(R.v) : 0.f;
            L.BV[r16][c16] = in ? R.gv * kLog2e : 0.f;
        }
        if (tid == 0) L.wide = 0;
        load(R, min(c + FD, nch - 1));   // past the end this reloads the last chunk
        __syncthreads();
        // 2. cumulative log-decays and the decay-scaled tiles: a thread per key
        // channel, a thread per state column
        if (tid < DK) {
            const int i = tid;
            float b[GC];
            float acc = 0.f;
#pragma unroll
            for (int r = 0; r < GC; ++r) {
                acc += L.BK[r * RS + i];
                b[r] = acc;
            }
            L.EKC[i] = __builtin_amdgcn_exp2f(acc);
            // A = (qt 2^{bk - bk_0}) (k 2^{bk_0 - bk})^T when every such factor
            // stays inside float32's range (|bk_r - bk_0| <= 120 in log2 units);
            // else A is formed element by element
            bool wide = false;
#pragma unroll
            for (int r = 0; r < GC; ++r) {
                const float d = b[r] - b[0];
                wide |= !(fabsf(d) <= 120.f);
                const float qt = L.QT[r * RS + i], kt = L.KT[r * RS + i];
                L.QE[r * RS + i] = qt * __builtin_amdgcn_exp2f(b[r]);
                L.KC[r * RS + i] = kt * __builtin_amdgcn_exp2f(acc - b[r]);
                L.QF[r * RS + i] = qt * __builtin_amdgcn_exp2f(d);
                L.KF[r * RS + i] = kt * __builtin_amdgcn_exp2f(-d);
                L.BK[r * RS + i] = b[r];
            }
            if (wide) L.wide = 1;
        } else if (tid < DK + GJ) {
            const int j = tid - DK;
            float b[GC];
            float acc = 0.f;
#pragma unroll
            for (int r = 0; r < GC; ++r) {
                acc += L.BV[r][j];
                b[r] = acc;
            }
            L.EVC[j] = __builtin_amdgcn_exp2f(acc);
#pragma unroll
            for (int r = 0; r < GC; ++r) {
                L.VC[r][j] = L.VV[r][j] * __builtin_amdgcn_exp2f(acc - b[r]);
                L.BV[r][j] = b[r];
            }
        }
        __syncthreads();
        // 3. wave 0: the inter-chunk read-out sum_i QE_ri S0_ij on MFMA (lane
        // group lk supplies channel k0 + 4 lk + u at step u: every channel once);
        // waves 1-3: A_rs for the 136 pairs s <= r, a thread per pair
        if (wave == 0) {
            gf32x4_t acc = gf32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
            for (int k0 = 0; k0 < DK; k0 += 16) {
                const float4 xa = *reinterpret_cast<const float4*>(L.QE + lm * RS + k0 + 4 * lk);
                const float4 xb = *reinterpret_cast<const float4*>(L.ST + lm * RS + k0 + 4 * lk);
                acc = gmfma4(xa.x, xb.x, acc);
                acc = gmfma4(xa.y, xb.y, acc);
                acc = gmfma4(xa.z, xb.z, acc);
                acc = gmfma4(xa.w, xb.w, acc);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) L.OI[4 * lk + e][lm] = acc[e];
        } else if (!L.wide) {
            if (wave == 1) {
                gf32x4_t acc = gf32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
                for (int k0 = 0; k0 < DK; k0 += 16) {
                    const float4 xa = *reinterpret_cast<const float4*>(L.QF + lm * RS + k0 + 4 * lk);
                    const float4 xb = *reinterpret_cast<const float4*>(L.KF + lm * RS + k0 + 4 * lk);
                    acc = gmfma4(xa.x, xb.x, acc);
                    acc = gmfma4(xa.y, xb.y, acc);
                    acc = gmfma4(xa.z, xb.z, acc);
                    acc = gmfma4(xa.w, xb.w, acc);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * lk + e;
                    L.AM[r][lm] = lm <= r ? acc[e] : 0.f;   // the masked pairs may be out of range
                }
            }
        } else {
            const int pr = tid - 64;
            if (pr < GC * (GC + 1) / 2) {
                int r = 0;
                while ((r + 1) * (r + 2) / 2 <= pr) ++r;
                const int s = pr - r * (r + 1) / 2;
                float a = 0.f;
#pragma unroll 4
                for (int i = 0; i < DK; i += 4) {
                    const float4 x = *reinterpret_cast<const float4*>(L.QT + r * RS + i);
                    const float4 y = *reinterpret_cast<const float4*>(L.KT + s * RS + i);
                    const float4 br = *reinterpret_cast<const float4*>(L.BK + r * RS + i);
                    const float4 bs = *reinterpret_cast<const float4*>(L.BK + s * RS + i);
                    a = fmaf(x.x * y.x, __builtin_amdgcn_exp2f(br.x - bs.x), a);
                    a = fmaf(x.y * y.y, __builtin_amdgcn_exp2f(br.y - bs.y), a);
                    a = fmaf(x.z * y.z, __builtin_amdgcn_exp2f(br.z - bs.z), a);
                    a = fmaf(x.w * y.w, __builtin_amdgcn_exp2f(br.w - bs.w), a);
                }
                L.AM[r][s] = a;
            }
        }
        __syncthreads();
        // 4. the outputs: thread (row r16, column c16)
        if (r16 < lc) {
            const int r = r16, j = c16;
            const float bvr = L.BV[r][j];
            float o = __builtin_amdgcn_exp2f(bvr) * L.OI[r][j];
            for (int s = 0; s <= r; ++s)
                o = fmaf(L.AM[r][s] * __builtin_amdgcn_exp2f(bvr - L.BV[s][j]), L.VV[s][j], o);
            const size_t t = tok(c * GC + r);
            static_cast<Tout*>(p.o)[(t * H + h) * DV + j0 + j] = from_f32<Tout>(o);
        }
        // 5. the state update on MFMA: rows [16 tt, +16) of the tile per step,
        // S1 = e^{bk_C + bv_C} S0 + Kc^T Vc (K = the 16 rows)
        for (int tt = wave; tt < DK / 16; tt += 4) {
            const int i0 = 16 * tt;
            gf32x4_t acc;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = i0 + 4 * lk + e;
                acc[e] = L.EKC[i] * L.EVC[lm] * L.ST[lm * RS + i];
            }
#pragma unroll
            for (int s0 = 0; s0 < GC; s0 += 4)
                acc = gmfma4(L.KC[(s0 + lk) * RS + i0 + lm], L.VC[s0 + lk][lm], acc);
#pragma unroll
            for (int e = 0; e < 4; ++e) L.ST[lm * RS + i0 + 4 * lk + e] = acc[e];
        }
        __syncthreads();
    };
    // unrolled by the ring depth so that every ring slot is a fixed set of registers
    for (int cb = 0; cb < nch; cb += FD) {
#pragma unroll
        for (int u = 0; u < FD; ++u)
            if (cb + u < nch) chunk(ring[u], cb + u);
    }
    __syncthreads();
    if (p.final_state) {
        for (int e = tid; e < DK * GJ; e += GTH) {
            const int i = e / GJ, j = e % GJ;
            p.final_state[(soff + i) * DV + j0 + j] = L.ST[j * RS + i];
        }
    }
}

template <int DK, typename Tin, typename Tout>
hipError_t launch_chunk(const GatedParams& p, hipStream_t st)
{
    const dim3 grid((unsigned)(p.dv / GJ), (unsigned)p.H, (unsigned)p.N);
    hipLaunchKernelGGL((gated_chunk_kernel<DK, Tin, Tout>), grid, dim3(GTH), 0, st, p);
    return hipGetLastError();
}

template <int DK>
hipError_t launch_dk(const GatedParams& p, hipStream_t st)
{
    if (!p.in_bf16) return launch_chunk<DK, float, float>(p, st);
    if (p.out_bf16) return launch_chunk<DK, bf16_t, bf16_t>(p, st);
    return launch_chunk<DK, bf16_t, float>(p, st);
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
