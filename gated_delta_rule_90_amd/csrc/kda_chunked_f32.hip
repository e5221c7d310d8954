// kda_chunked_f32.hip - chunk-parallel KDA prefill for float32 inputs
// (ejkernel "kernel_delta_attention": chunked mode, "Parallel within chunks").
//
// The chunk algebra is the bf16 MFMA kernel's (an exact regrouping of the
// token recurrence: decay per key channel, residual against the decayed
// state, o = S^T q), evaluated in float32 on the vector ALUs so that the
// result meets the float32 bar.  For a chunk of C tokens with b_r the
// in-chunk cumulative log-decay (per channel, log2 units), beta_r the
// activated beta and S0 the entering state:
//     A_rs = beta_r sum_i kh_ri kh_si 2^{b_ri - b_si}   (s < r)
//     P_rs = sum_i qh_ri kh_si 2^{b_ri - b_si}          (s <= r)
//     T' = (I + A)^-1 diag(beta),  W = T' Kg,  U = T' V - W S0
//     O = Qg S0 + P U,  S = Diag(2^{b_C}) S0 + Kc^T U
// with Kg_s = 2^{b_s} kh_s, Qg_r = 2^{b_r} qh_r, Kc_s = 2^{b_C - b_s} kh_s.
//
// Chunks are C = 16 tokens.  With lower_bound >= -5 a channel's log-decay
// over 16 tokens is at most 16 * 5 * log2(e) < 116 in log2 units, so one
// reference row per chunk keeps every factor inside float32's normal range:
//     L_r = 2^{b_r - b_0} in [2^-116, 1],   R_s = 2^{b_0 - b_s} in [1, 2^116]
// and 2^{b_r - b_s} = L_r R_s for the kept pairs (s <= r) is a product of
// two normal numbers, at most 1.  Kc = 2^{b_C - b_0} R (at most 1 per term)
// and Qg = 2^{b_0} L keep every summand of the state products bounded.
//
// EJK mode (scalar per-head decay d_t, beta used as given, residual against
// the undecayed state): A_rs carries 2^{b_{r-1} - b_s} and Kg_r = 2^{b_{r-1}}
// kh_r (b_{-1} = 0); with d <= 0 (the page's contract) every factor is at most
// 1 and is applied per (r, s) as a scalar.
//
// Work split: one 256-thread workgroup per (sequence, head, 16 state
// columns).  The state tile [dk][16] stays in LDS in float32; the
// column-independent quantities (prologue, A, P, T', W) are recomputed by
// each column tile, which is cheap beside the state products at dk <= 128.
// The next chunk's inputs are loaded into registers while the current chunk
// computes.  Rows past a sequence's end are padded with exact neutral values
// (q = k = v = 0, gamma = 0, beta = 0) and never stored, so a packed batch
// equals each sequence run alone, bit for bit.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int FC = 16;    // tokens per chunk
constexpr int FT = 256;   // threads per workgroup
constexpr int FJ = 16;    // state columns per workgroup
constexpr int F16 = FC + 1;

template <int DK>
struct F32Lds {
    static constexpr int RS = DK + 1;   // row stride of [16][DK] tiles: rows fall in different banks
    float QL[FC * RS];    // qh_r 2^{b_r - b_0} (EJK: qh_r); later W
    float KL[FC * RS];    // kh_r 2^{b_r - b_0} (EJK: kh_r)
    float KR[FC * RS];    // kh_r 2^{b_0 - b_r} (EJK: kh_r)
    float GB[FC * RS];    // raw gates, then b_r (log2 units)
    float SL[DK * F16];   // the state tile S[i][j]
    float VV[FC * F16];   // the value tile V[s][j]
    float AM[FC * F16];   // A (strict lower, beta-scaled)
    float PM[FC * F16];   // P (lower incl. diagonal)
    float TP[FC * F16];   // T' = (I + A)^-1 diag(beta)
    float UM[FC * F16];   // U
    float E0[DK];         // 2^{b_0}
    float NC[DK];         // 2^{b_C - b_0}
    float DC[DK];         // 2^{b_C}
    float NQ[FC], NK[FC], BT[FC];   // query scale / norm, key 1 / norm, activated beta
    float EB[FC], EX[FC], EC[FC];   // EJK: 2^{b_r}, 2^{b_{r-1}}, 2^{b_C - b_r}
    float BR[FC], BX[FC];           // EJK: b_r, b_{r-1}
};

__device__ __forceinline__ void f32_seq_bounds(const int32_t* cu, int n, int T, int& t0, int& t1)
{
    if (cu) {
        t0 = min(max(cu[n], 0), T);
        t1 = min(max(cu[n + 1], t0), T);
    } else {
        t0 = n * T;
        t1 = t0 + T;
    }
}

template <int DK, bool EJK>
__global__ __launch_bounds__(FT) void chunk_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, const float* __restrict__ a_log,
    const float* __restrict__ dt_bias, const float* __restrict__ init, const int32_t* __restrict__ cu,
    int T, int H, int HKV, int DV, float scale, float lower_bound, int l2norm,
    float* __restrict__ o, float* __restrict__ final_state)
{
    constexpr int RS = F32Lds<DK>::RS;
    constexpr int Q4 = FC * DK / 4;            // float4 pieces of a [16][DK] tile
    constexpr int QN = (Q4 + FT - 1) / FT;     // per thread
    constexpr int EPT = FC * DK / FT;          // [16][DK] elements per thread (1..8)
    static_assert(EPT >= 1 && EPT * FT == FC * DK, "dk in {16, 32, 64, 128}");
    __shared__ F32Lds<DK> L;

    const int tid = threadIdx.x;
    const int r16 = tid >> 4;   // row of a 16x16 tile
    const int c16 = tid & 15;   // column of a 16x16 tile
    const int j0 = blockIdx.x * FJ;
    const int h = blockIdx.y;
    const int n = blockIdx.z;
    const int hk = h / (H / HKV);
    int t0, t1;
    f32_seq_bounds(cu, n, T, t0, t1);
    const int nch = (t1 - t0 + FC - 1) / FC;
    const size_t soff = ((size_t)n * H + h) * DK * DV;

    for (int e = tid; e < DK * FJ; e += FT) {
        const int i = e / FJ, j = e % FJ;
        L.SL[i * F16 + j] = init ? init[soff + (size_t)i * DV + j0 + j] : 0.f;
    }
    const float ea = EJK ? 0.f : expf(a_log[h]) * kLog2e;   // exp(a_log) in log2 units
    const float lb2 = lower_bound * kLog2e;
    const float dtb = (!EJK && dt_bias && tid < DK) ? dt_bias[(size_t)tid * H + h] : 0.f;

    // one chunk's inputs in registers: q, k, g as float4 pieces (row e / (DK/4),
    // channels 4 (e % (DK/4)) ..), v at (row r16, column c16), beta and the EJK
    // decay of row tid (tid < 16); rows past the sequence are zero
    float4 rq[QN], rk[QN], rg[QN];
    float rv = 0.f, rb = 0.f, rd = 0.f;
    auto load = [&](int c) {
        const int c0 = t0 + c * FC;
        const int len = min(FC, t1 - c0);
#pragma unroll
        for (int m = 0; m < QN; ++m) {
            const int e = tid + m * FT;
            const int row = e / (DK / 4), c4 = e % (DK / 4);
            const bool in = e < Q4 && row < len;
            const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
            rq[m] = in ? *reinterpret_cast<const float4*>(q + ((size_t)(c0 + row) * H + h) * DK + 4 * c4) : z;
            rk[m] = in ? *reinterpret_cast<const float4*>(k + ((size_t)(c0 + row) * HKV + hk) * DK + 4 * c4) : z;
            if constexpr (!EJK)
                rg[m] = in ? *reinterpret_cast<const float4*>(g + ((size_t)(c0 + row) * H + h) * DK + 4 * c4) : z;
        }
        rv = (r16 < len) ? v[((size_t)(c0 + r16) * HKV + hk) * DV + j0 + c16] : 0.f;
        if (tid < FC) {
            rb = (tid < len) ? beta[(size_t)(c0 + tid) * H + h] : 0.f;
            if constexpr (EJK) rd = (tid < len && g) ? g[(size_t)(c0 + tid) * H + h] : 0.f;
        }
    };
    if (nch > 0) load(0);

    for (int c = 0; c < nch; ++c) {
        const int c0 = t0 + c * FC;
        const int len = min(FC, t1 - c0);
        // ---- raw inputs to LDS, then fetch the next chunk's
#pragma unroll
        for (int m = 0; m < QN; ++m) {
            const int e = tid + m * FT;
            if (e < Q4) {
                const int row = e / (DK / 4), c4 = e % (DK / 4);
                float* pq = L.QL + row * RS + 4 * c4;
                float* pk = L.KL + row * RS + 4 * c4;
                pq[0] = rq[m].x; pq[1] = rq[m].y; pq[2] = rq[m].z; pq[3] = rq[m].w;
                pk[0] = rk[m].x; pk[1] = rk[m].y; pk[2] = rk[m].z; pk[3] = rk[m].w;
                if constexpr (!EJK) {
                    float* pg = L.GB + row * RS + 4 * c4;
                    pg[0] = rg[m].x; pg[1] = rg[m].y; pg[2] = rg[m].z; pg[3] = rg[m].w;
                }
            }
        }
        L.VV[r16 * F16 + c16] = rv;
        if (tid < FC) {
            L.BT[tid] = (tid < len) ? (EJK ? rb : sigmoid_f(rb)) : 0.f;
            if constexpr (EJK) L.BR[tid] = rd * kLog2e;   // the row's log-decay, summed below
        }
        if (c + 1 < nch) load(c + 1);
        lds_barrier();

        // ---- prologue: row norms (16 lanes per row), gates and their in-chunk cumsum
        {
            float sq = 0.f, sk = 0.f;
#pragma unroll
            for (int m = 0; m < DK / 16; ++m) {
                const float x = L.QL[r16 * RS + c16 + 16 * m], y = L.KL[r16 * RS + c16 + 16 * m];
                sq = fmaf(x, x, sq);
                sk = fmaf(y, y, sk);
            }
            sq = group_sum<16>(sq);
            sk = group_sum<16>(sk);
            if (c16 == 0) {
                L.NQ[r16] = l2norm ? scale / sqrtf(sq + kNormEps) : scale;
                L.NK[r16] = l2norm ? 1.0f / sqrtf(sk + kNormEps) : 1.0f;
            }
        }
        if constexpr (!EJK) {
            if (tid < DK) {
                // gamma' = lb * log2(e) * sigmoid(exp(a_log) (g + dt_bias)); padded rows 0
                float b = 0.f;
#pragma unroll
                for (int r = 0; r < FC; ++r) {
                    const float x = L.GB[r * RS + tid];
                    const float gm = (r < len) ? lb2 * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-ea * (x + dtb))) : 0.f;
                    b += gm;
                    L.GB[r * RS + tid] = b;
                }
                const float b0 = L.GB[tid];
                L.E0[tid] = __builtin_amdgcn_exp2f(b0);
                L.NC[tid] = __builtin_amdgcn_exp2f(b - b0);
                L.DC[tid] = __builtin_amdgcn_exp2f(b);
            }
        } else {
            if (tid < FC) {
                // b_r and b_{r-1} of this row, summed in row order (the decays sit in BR)
                float b = 0.f, bx = 0.f;
                for (int s = 0; s <= tid; ++s) {
                    bx = b;
                    b += L.BR[s];
                }
                float bc = 0.f;
                for (int s = 0; s < FC; ++s) bc += L.BR[s];
                // every lane has read BR before any writes it (one wave: LDS in issue order)
                L.BX[tid] = bx;
                L.EB[tid] = __builtin_amdgcn_exp2f(b);
                L.EX[tid] = __builtin_amdgcn_exp2f(bx);
                L.EC[tid] = __builtin_amdgcn_exp2f(bc - b);
                if (tid == FC - 1) L.DC[0] = __builtin_amdgcn_exp2f(bc);
                L.BR[tid] = b;
            }
        }
        lds_barrier();

        // ---- normalised rows with the decay factors
#pragma unroll
        for (int m = 0; m < EPT; ++m) {
            const int e = tid + m * FT;
            const int r = e / DK, i = e % DK;
            const float qh = L.QL[r * RS + i] * L.NQ[r];
            const float kh = L.KL[r * RS + i] * L.NK[r];
            if constexpr (EJK) {
                L.QL[r * RS + i] = qh;
                L.KL[r * RS + i] = kh;
                L.KR[r * RS + i] = kh;
            } else {
                const float d = L.GB[r * RS + i] - L.GB[i];   // b_r - b_0 <= 0
                const float lf = __builtin_amdgcn_exp2f(d), rf = __builtin_amdgcn_exp2f(-d);
                L.QL[r * RS + i] = qh * lf;
                L.KL[r * RS + i] = kh * lf;
                L.KR[r * RS + i] = kh * rf;
            }
        }
        lds_barrier();

        // ---- A and P: thread (r, s) = (r16, c16)
        {
            const int r = r16, s = c16;
            float a0 = 0.f, a1 = 0.f, p0 = 0.f, p1 = 0.f;
#pragma unroll 8
            for (int i = 0; i < DK; i += 2) {
                const float k0 = L.KR[s * RS + i], k1 = L.KR[s * RS + i + 1];
                a0 = fmaf(L.KL[r * RS + i], k0, a0);
                a1 = fmaf(L.KL[r * RS + i + 1], k1, a1);
                p0 = fmaf(L.QL[r * RS + i], k0, p0);
                p1 = fmaf(L.QL[r * RS + i + 1], k1, p1);
            }
            float a = a0 + a1, p = p0 + p1;
            if constexpr (EJK) {
                a *= (s < r) ? __builtin_amdgcn_exp2f(L.BX[r] - L.BR[s]) : 0.f;
                p *= (s <= r) ? __builtin_amdgcn_exp2f(L.BR[r] - L.BR[s]) : 0.f;
            }
            L.AM[r * F16 + s] = (s < r) ? L.BT[r] * a : 0.f;
            L.PM[r * F16 + s] = (s <= r) ? p : 0.f;
        }
        lds_barrier();

        // ---- T' = (I + A)^-1 diag(beta): lane j < 16 solves column j by forward
        // substitution; meanwhile every thread forms its (r, j) entry of Qg S0
        if (tid < FC) {
            const int j = tid;
            float t[FC];
#pragma unroll
            for (int r = 0; r < FC; ++r) t[r] = (r == j) ? 1.f : 0.f;
#pragma unroll
            for (int s = 0; s < FC - 1; ++s) {
                const float ts = t[s];
#pragma unroll
                for (int r = s + 1; r < FC; ++r) t[r] = fmaf(-L.AM[r * F16 + s], ts, t[r]);
            }
            const float bj = L.BT[j];
#pragma unroll
            for (int r = 0; r < FC; ++r) L.TP[r * F16 + j] = t[r] * bj;
        }
        float oq;   // (Qg S0)[r16][c16]
        {
            float o0 = 0.f, o1 = 0.f;
#pragma unroll 8
            for (int i = 0; i < DK; i += 2) {
                if constexpr (EJK) {
                    o0 = fmaf(L.QL[r16 * RS + i], L.SL[i * F16 + c16], o0);
                    o1 = fmaf(L.QL[r16 * RS + i + 1], L.SL[(i + 1) * F16 + c16], o1);
                } else {
                    o0 = fmaf(L.E0[i] * L.QL[r16 * RS + i], L.SL[i * F16 + c16], o0);
                    o1 = fmaf(L.E0[i + 1] * L.QL[r16 * RS + i + 1], L.SL[(i + 1) * F16 + c16], o1);
                }
            }
            oq = o0 + o1;
            if constexpr (EJK) oq *= L.EB[r16];
        }
        lds_barrier();

        // ---- W = T' Kg (into QL's space) and this thread's entry of T' V
#pragma unroll
        for (int m = 0; m < EPT; ++m) {
            const int e = tid + m * FT;
            const int r = e / DK, i = e % DK;
            float w = 0.f;
#pragma unroll
            for (int s = 0; s < FC; ++s) {
                if constexpr (EJK)
                    w = fmaf(L.TP[r * F16 + s], L.EX[s] * L.KL[s * RS + i], w);
                else
                    w = fmaf(L.TP[r * F16 + s], L.KL[s * RS + i], w);
            }
            L.QL[r * RS + i] = EJK ? w : L.E0[i] * w;
        }
        float ut = 0.f;   // (T' V)[r16][c16]
#pragma unroll
        for (int s = 0; s < FC; ++s) ut = fmaf(L.TP[r16 * F16 + s], L.VV[s * F16 + c16], ut);
        lds_barrier();

        // ---- U = T' V - W S0
        {
            float w0 = 0.f, w1 = 0.f;
#pragma unroll 8
            for (int i = 0; i < DK; i += 2) {
                w0 = fmaf(L.QL[r16 * RS + i], L.SL[i * F16 + c16], w0);
                w1 = fmaf(L.QL[r16 * RS + i + 1], L.SL[(i + 1) * F16 + c16], w1);
            }
            L.UM[r16 * F16 + c16] = ut - (w0 + w1);
        }
        lds_barrier();

        // ---- O = Qg S0 + P U (stored for the sequence's rows); S = Diag(2^{b_C}) S0 + Kc^T U
        {
            float ov = oq;
#pragma unroll
            for (int s = 0; s < FC; ++s) ov = fmaf(L.PM[r16 * F16 + s], L.UM[s * F16 + c16], ov);
            if (r16 < len) o[((size_t)(c0 + r16) * H + h) * DV + j0 + c16] = ov;
        }
#pragma unroll
        for (int m = 0; m < DK / 16; ++m) {
            const int i = r16 + 16 * m;
            float acc = 0.f;
            if constexpr (EJK) {
#pragma unroll
                for (int s = 0; s < FC; ++s) acc = fmaf(L.EC[s] * L.KR[s * RS + i], L.UM[s * F16 + c16], acc);
                L.SL[i * F16 + c16] = fmaf(L.DC[0], L.SL[i * F16 + c16], acc);
            } else {
                const float nc = L.NC[i];
#pragma unroll
                for (int s = 0; s < FC; ++s) acc = fmaf(nc * L.KR[s * RS + i], L.UM[s * F16 + c16], acc);
                L.SL[i * F16 + c16] = fmaf(L.DC[i], L.SL[i * F16 + c16], acc);
            }
        }
        lds_barrier();
    }
    if (nch == 0) lds_barrier();   // the initial state tile was written by other threads

    if (final_state) {
        for (int e = tid; e < DK * FJ; e += FT) {
            const int i = e / FJ, j = e % FJ;
            final_state[soff + (size_t)i * DV + j0 + j] = L.SL[i * F16 + j];
        }
    }
}

template <int DK>
hipError_t launch_dk(const PrefillArgs& a, hipStream_t stream)
{
    const dim3 grid((unsigned)(a.dv / FJ), (unsigned)a.H, (unsigned)a.N);
    const float* q = static_cast<const float*>(a.q);
    const float* k = static_cast<const float*>(a.k);
    const float* v = static_cast<const float*>(a.v);
    float* o = static_cast<float*>(a.o);
    if (a.ejk)
        hipLaunchKernelGGL((chunk_f32_kernel<DK, true>), grid, dim3(FT), 0, stream, q, k, v, a.g, a.beta,
                           a.a_log, a.dt_bias, a.init, a.cu, a.T, a.H, a.Hkv, a.dv, a.scale, a.lower_bound,
                           (int)a.l2norm, o, a.final_state);
    else
        hipLaunchKernelGGL((chunk_f32_kernel<DK, false>), grid, dim3(FT), 0, stream, q, k, v, a.g, a.beta,
                           a.a_log, a.dt_bias, a.init, a.cu, a.T, a.H, a.Hkv, a.dv, a.scale, a.lower_bound,
                           (int)a.l2norm, o, a.final_state);
    return hipGetLastError();
}

}  // namespace

bool chunked_f32_supported(const PrefillArgs& a)
{
    const bool dims = (a.dk == 16 || a.dk == 32 || a.dk == 64 || a.dk == 128) && a.dv % FJ == 0 && a.dv > 0;
    // KDA needs the gate inputs and lower_bound >= -5 (the factor range above)
    return !a.in_bf16 && !a.out_bf16 && dims && (a.ejk || (a.g != nullptr && a.a_log != nullptr && a.lower_bound >= -5.0f));
}

hipError_t launch_chunked_f32(const PrefillArgs& a, hipStream_t stream)
{
    switch (a.dk) {
    case 16: return launch_dk<16>(a, stream);
    case 32: return launch_dk<32>(a, stream);
    case 64: return launch_dk<64>(a, stream);
    default: return launch_dk<128>(a, stream);
    }
}

}  // namespace kda
