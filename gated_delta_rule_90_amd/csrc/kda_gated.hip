// kda_gated.hip - the gated recurrent attention of the ejkernel "recurrent"
// page (recurrent_attention(): query, key, value, the gates g, g_gamma, gk,
// gv, softmax_scale, initial_state, reverse, cu_seqlens).
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
// Chunked form: chunks of C = 16 tokens in processing order.  With
// a_t = gk_t + g_gamma (key axis) and gv_t (value axis), bk_r, bv_r their
// cumulative sums over the chunk's rows r = 0..15 and qt_r = scale e^{g_r} q_r:
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
// read-out and the state update run on 16x16x4 float32 MFMA.  One 256-thread
// workgroup per (sequence, head, 16 state columns); the state tile stays in
// LDS, transposed.  Rows past the sequence are neutral (q = k = v = 0, every
// gate 0).  The next two chunks' inputs are in flight in a register ring.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

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
    const int H = p.H, HKV = p.Hkv, DV = p.dv;
    // Linear workgroup ids are dealt to the 8 XCDs in turn: the column tiles of
    // one (sequence, head), which read the same q, k and gate rows, get ids
    // equal modulo 8, so they run on one XCD and share its L2.  Ids past the
    // last (sequence, head) (the count is padded to a multiple of 8) exit.
    const int ntile = DV / GJ;
    const int xcd = blockIdx.x & 7, qd = blockIdx.x >> 3;
    const int grp = (qd / ntile) * 8 + xcd;
    if (grp >= H * p.N) return;
    const int j0 = (qd % ntile) * GJ, h = grp % H, n = grp / H;
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
    const unsigned groups8 = (unsigned)((p.H * p.N + 7) / 8 * 8);
    if (groups8 == 0) return hipSuccess;
    const dim3 grid(groups8 * (unsigned)(p.dv / GJ));
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
