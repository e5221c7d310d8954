// kda_backward.hip - backward pass (gradients) of the KDA prefill: the
// chunked mode of the ejkernel "kernel_delta_attention" page (section
// "Algorithm modes"), whose chunk parallelism the page offers for training.
//
// The pages give no backward formulas.  The ones below are the adjoint of the
// exact chunk regrouping of the token recurrence that the forward kernels use,
// here with chunks of C = 16 tokens and float32 arithmetic throughout.  With
// b_r = sum_{s<=r} gamma_s (per key channel for KDA, one scalar per token for
// EJK, restarting at the chunk start), b' = b for KDA and b'_r = b_{r-1}
// (b'_0 = 0) for EJK, and S0 the state entering the chunk:
//     GA_rs = sum_i kh_ri kh_si e^{b'_ri - b_si} (s < r),  A = diag(beta) GA
//     GP_rs = sum_i qh_ri kh_si e^{b_ri - b_si}  (s <= r),  P = GP
//     Kg = e^{b'} kh,  Qg = e^{b} qh,  Kc = e^{b_C - b} kh  (b_C: last row)
//     Y = V - Kg S0,  (I + A) U = diag(beta) Y
//     O = Qg S0 + P U,  S1 = Diag(e^{b_C}) S0 + Kc^T U
// Given dO and dS1 = dL/dS1 the adjoint is
//     dU = P^T dO + Kc dS1,  (I + A)^T Z = dU,  dY = diag(beta) Z,  dV = dY
//     dS0 = Qg^T dO + Diag(e^{b_C}) dS1 - Kg^T dY
//     dA = -strict_lower(Z U^T),  dP = lower(dO U^T)
//     dbeta_r = Z_r . Y_r + sum_s dA_rs GA_rs
//     dQg = dO S0^T,  dKg = -dY S0^T,  dKc = U dS1^T
// then through the two Gram products (each row and column role) and the
// decay factors into dqh, dkh and db, db' (db' joins db on the same row for
// KDA, on the row before for EJK), db_C (the carry and Kc) on the last row,
// and dgamma, the reverse cumulative sum of db over the chunk; finally
// through the prologue (L2 norms, gate activation, beta sigmoid).
//
// Barriers wait for LDS only (lds_barrier): no workgroup reads global memory
// that another of its waves wrote, so prefetched loads and stores stay in
// flight across them.
//
// Four kernels (and two small ones):
//   0. bwd_prep: per (chunk, head), every chunk in parallel: the chunk's
//      column-independent operands (normalised, decayed rows Qg, Kg, Kc, the
//      Gram products, the decay factors), formed once for both scans;
//   1. bwd_fwd_scan: per (sequence, head, 16 state columns), the state carried
//      forward over the chunks, storing the state entering every chunk and the
//      chunk's Y and U;
//   2. bwd_rev_scan: per (sequence, head, 16 columns), the state gradient
//      carried backward over the chunks, storing dL/d(state leaving the
//      chunk) and Z for every chunk (and dL/d(initial state) at the end).
//      Both recurrences are independent per state column, so column tiles
//      run in parallel;
//   3. bwd_local: per (chunk, head), all columns, every chunk in parallel:
//      the chunk's own gradients from its two stored states and Y, U, Z.
// A last small kernel sums the parameter gradients over chunks (and the key
// and value gradients over the heads of a group when heads are grouped).
//
// Range: within 16 tokens the KDA log-decay of a channel is at least
// 16 * lower_bound >= -80 (lower_bound >= -5), so e^{+-b} stays inside
// float32's normal range and the Gram products are factorised per channel.
// EJK decays have no lower bound, so the scalar factors e^{b'_r - b_s} are
// formed element by element (masked entries are never exponentiated).
#include <algorithm>
#include <type_traits>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int BC = 16;    // chunk length
constexpr int BT = 256;   // threads per workgroup
constexpr int TV = 16;    // state columns per scan tile (a scan workgroup takes one or two)
constexpr int kCUs = 256; // compute units of an MI355X
constexpr int MAXD = 128;
constexpr int SR = MAXD + 4;   // row stride of [16][<=128] tiles

struct BwdParams {
    const void* q;
    const void* k;
    const void* v;
    int in_bf16;
    const float* g;
    const float* beta;
    const float* a_log;
    const float* dt_bias;
    const float* init;
    const int32_t* cu;
    int N, T, H, Hkv, dv;
    float scale, lb;
    int l2norm;
    const void* d_o;
    int do_bf16;
    const float* dSf;
    float* dq;
    float* dk;        // [Ntok, Hkv, dk], or per query head [Ntok, H, dk] when grouped
    float* dv_out;    // [Ntok, Hkv, dv], or per query head [Ntok, H, dv] when grouped
    float* dg;
    float* dbeta;
    float* dS0;
    const int32_t* off;   // [N + 1] chunk offsets
    const int32_t* poff;  // [N + 1] offsets of the pairs of consecutive chunks
    // the checkpoints, per (pair of chunks, head) in 16-column tiles:
    // [dv / 16][dk][16], so that a scan workgroup's tile is one contiguous 8 KB
    // block (dk 128)
    float* ckS;           // [pairs, H, dv / 16, dk, 16]  state entering a pair's first chunk
    float* ckdS;          // [pairs, H, dv / 16, dk, 16]  dL/d(state leaving a pair's last chunk)
    float* ckYU;          // [slots, H, 2, 16, dv]  Y = V - Kg S0 and U of each chunk
    float* ckZ;           // [slots, H, 16, dv]  Z of each chunk ((I + A)^T Z = dU)
    float* prep;          // [slots, H, PrepLayout<dk>::SIZE]  column-independent chunk operands
    float* part_a;        // [slots, H]          a_log gradient per chunk
    float* part_dt;       // [slots, H, dk]      dt_bias gradient per chunk
    // the forward output (prefill16_scan only)
    void* out;            // [Ntok, H, dv] float32 or bf16
    int out_bf16;
    float* fstate;        // [N, H, dk, dv] or null
};

typedef float bf32x4_t __attribute__((ext_vector_type(4)));

// D += A B on a 16x16x4 float32 MFMA: lane l supplies A[l % 16][l / 16] and
// B[l / 16][l % 16] and holds D[4 (l / 16) + e][l % 16] in element e.
__device__ __forceinline__ bf32x4_t bmfma4(float a, float b, bf32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void seq_bounds(const int32_t* cu, int n, int T, int& t0, int& t1)
{
    if (cu) {
        t0 = min(max(cu[n], 0), T);
        t1 = min(max(cu[n + 1], t0), T);
    } else {
        t0 = n * T;
        t1 = t0 + T;
    }
}

// Chunk offsets: off[n] = sum_{m<n} ceil(len_m / 16), capped at the
// workspace's chunk slots (only ranges that overlap can count more chunks
// than the slots; those sequences then lose their last chunks, and their
// results are unspecified, but every access stays inside the workspace);
// pair offsets poff[n] = sum_{m<n} ceil(chunks_m / 2), capped likewise.
__global__ void bwd_plan_kernel(const int32_t* __restrict__ cu, int N, int T, int slots, int pslots,
                                int32_t* __restrict__ off, int32_t* __restrict__ poff)
{
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    int acc = 0, pacc = 0;
    for (int n = 0; n < N; ++n) {
        int t0, t1;
        seq_bounds(cu, n, T, t0, t1);
        off[n] = acc;
        poff[n] = pacc;
        const int na = min(acc + (t1 - t0 + BC - 1) / BC, slots);
        pacc = min(pacc + (na - acc + 1) / 2, pslots);
        acc = na;
    }
    off[N] = acc;
    poff[N] = pacc;
}

// Chunks of sequence n: its length in chunks, within its slots.
__device__ __forceinline__ int seq_chunks(const int32_t* off, int n, int t0, int t1)
{
    return min((t1 - t0 + BC - 1) / BC, off[n + 1] - off[n]);
}

// The logistic on the hardware exponential and reciprocal (each within about
// an ulp): 1 / (1 + 2^(-x log2 e)).  Rounding x log2 e adds a relative error
// of about |x| 2^-24, under 1e-6 for the |x| < 20 that gate arguments and
// beta logits take; large |x| saturates to 0 or 1.
__device__ __forceinline__ float sigmoid_fast(float x)
{
    return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-x * kLog2e));
}

// ---------------------------------------------------------------------------
// The state-independent part of one chunk, in LDS: normalised rows, decay
// factors, the Gram products GA (strict lower, without beta) and GP (lower).
template <int DK, bool EJK>
struct ChunkLds {
    float qh[BC][SR];
    float kh[BC][SR];
    float eb[BC][SR];    // KDA: e^{b}   (first the gate, then b, then e^b)
    float ein[BC][SR];   // KDA: e^{-b}
    float ecb[BC][SR];   // KDA: e^{b_C - b}
    float ec[MAXD];      // KDA: e^{b_C}
    float beta[BC];
    float nq[BC], nk[BC];   // inverse row norms 1 / sqrt(sum x^2 + eps)
    float sb[BC], seb[BC], sebp[BC], secb[BC];   // EJK: b, e^b, e^{b'}, e^{b_C - b}
    float sec;                                   // EJK: e^{b_C}
    float GA[BC][BC + 1];
    float GP[BC][BC + 1];
    float DA[BC][BC + 1];   // EJK: e^{b'_r - b_s} (s < r)
    float DP[BC][BC + 1];   // EJK: e^{b_r - b_s} (s <= r)

    __device__ float ebr(int r, int i) const { return EJK ? seb[r] : eb[r][i]; }
    __device__ float ebpr(int r, int i) const { return EJK ? sebp[r] : eb[r][i]; }
    __device__ float ecbr(int r, int i) const { return EJK ? secb[r] : ecb[r][i]; }
    __device__ float ecc(int i) const { return EJK ? sec : ec[i]; }
    __device__ float kg(int r, int i) const { return kh[r][i] * ebpr(r, i); }
    __device__ float qg(int r, int i) const { return qh[r][i] * ebr(r, i); }
    __device__ float kc(int r, int i) const { return kh[r][i] * ecbr(r, i); }
};


// Steps 2-4 of a chunk's set-up (step 1, the rows into LDS, is the caller's),
// once the raw rows (qh, kh), the gate activations (KDA: eb, log2 units),
// beta and the EJK gates (sb, log2 units) are in LDS; rows past the chunk's
// end are neutral (q = k = 0, gamma = 0, beta = 0).  The cumulative
// log-decays are formed in log2 units and the factors with exp2; products
// such as Qg * dQg, from which the gradients are built, do not depend on the
// unit.  Begins and ends with a barrier.
template <int DK, bool EJK>
__device__ void setup_rest(ChunkLds<DK, EJK>& L, const BwdParams& p)
{
    const int tid = threadIdx.x;
    constexpr int NE = BC * DK / BT;   // row elements per thread (1 .. 8)
    lds_barrier();
    // 2. row norms: eight lanes per (row, q or k), summed by DPP and swizzle;
    // cumulative log-decays and their factors: a thread per key channel
    {
        const int pr = tid >> 3, part = tid & 7;   // 32 (row, q/k) pairs
        const int r = pr & 15;
        const float* row = pr < 16 ? L.qh[r] : L.kh[r];
        float ss = 0.f;
        for (int i = part; i < DK; i += 8) ss = fmaf(row[i], row[i], ss);
        ss = xor_add<1>(ss);
        ss = xor_add<2>(ss);
        ss = xor_add<4>(ss);
        if (part == 0) (pr < 16 ? L.nq : L.nk)[r] = 1.f / sqrtf(ss + kNormEps);
    }
    if (!EJK) {
        if (tid < DK) {
            const int i = tid;
            float b[BC];
            float acc = 0.f;
#pragma unroll
            for (int r = 0; r < BC; ++r) {
                acc += L.eb[r][i];
                b[r] = acc;
            }
            L.ec[i] = __builtin_amdgcn_exp2f(acc);
#pragma unroll
            for (int r = 0; r < BC; ++r) {
                L.eb[r][i] = __builtin_amdgcn_exp2f(b[r]);
                L.ein[r][i] = __builtin_amdgcn_exp2f(-b[r]);
                L.ecb[r][i] = __builtin_amdgcn_exp2f(acc - b[r]);
            }
        }
    } else if (tid == BT - 1) {
        float acc = 0.f;
        for (int r = 0; r < BC; ++r) {
            acc += L.sb[r];
            L.sb[r] = acc;
        }
    }
    lds_barrier();
    // 3. normalised rows; EJK row factors
#pragma unroll
    for (int m = 0; m < NE; ++m) {
        const int e = tid + m * BT;
        const int r = e / DK, i = e % DK;
        L.qh[r][i] = p.l2norm ? p.scale * L.qh[r][i] * L.nq[r] : p.scale * L.qh[r][i];
        L.kh[r][i] = p.l2norm ? L.kh[r][i] * L.nk[r] : L.kh[r][i];
    }
    if (EJK && tid < BC) {
        const int r = tid;
        const float b = L.sb[r], bp = r > 0 ? L.sb[r - 1] : 0.f, bC = L.sb[BC - 1];
        L.seb[r] = __builtin_amdgcn_exp2f(b);
        L.sebp[r] = __builtin_amdgcn_exp2f(bp);
        L.secb[r] = __builtin_amdgcn_exp2f(bC - b);
        if (r == 0) L.sec = __builtin_amdgcn_exp2f(bC);
    }
    lds_barrier();
    // 4. the Gram products on 16x16x4 float32 MFMA: wave 0 GA (kh e^{b'} against
    // kh e^{-b}), wave 1 GP (qh e^{b} against kh e^{-b}); EJK: the plain dots,
    // scaled by the element factors.  Lane (lm, lk) supplies channel
    // k0 + 4 lk + u of row lm of both operands and holds rows 4 lk + e of
    // column lm.
    {
        const int lane = tid & 63, wave = tid >> 6;
        const int lm = lane & 15, lk = lane >> 4;
        if (wave < 2) {
            const float (*X)[SR] = wave == 0 ? L.kh : L.qh;
            bf32x4_t acc = bf32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
            for (int k0 = 0; k0 < DK; k0 += 16) {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int kk = k0 + 4 * lk + u;
                    const float a = EJK ? X[lm][kk] : X[lm][kk] * L.eb[lm][kk];
                    const float b = EJK ? L.kh[lm][kk] : L.kh[lm][kk] * L.ein[lm][kk];
                    acc = bmfma4(a, b, acc);
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * lk + e, s = lm;
                float x = acc[e];
                if (wave == 0) {
                    if (EJK) {
                        const float bp = r > 0 ? L.sb[r - 1] : 0.f;
                        const float da = s < r ? __builtin_amdgcn_exp2f(bp - L.sb[s]) : 0.f;
                        L.DA[r][s] = da;
                        x *= da;
                    }
                    L.GA[r][s] = s < r ? x : 0.f;
                } else {
                    if (EJK) {
                        const float dp = s <= r ? __builtin_amdgcn_exp2f(L.sb[r] - L.sb[s]) : 0.f;
                        L.DP[r][s] = dp;
                        x *= dp;
                    }
                    L.GP[r][s] = s <= r ? x : 0.f;
                }
            }
        }
    }
    lds_barrier();
}

// ---------------------------------------------------------------------------
// The column-independent operands of one chunk, formed once per (chunk, head)
// by bwd_prep for the two state scans (each of which runs per 16 state
// columns).  In global memory, floats, rows of RS = dk + 4 (the scans copy the
// block to LDS as it is, and rows 16 bytes apart by a multiple of 4 banks
// keep their 16-byte reads conflict-free):
//     QG [16][RS]  Qg (EJK: qh)          KG [16][RS]  Kg (EJK: kh)
//     KC [16][RS]  Kc (KDA)              TI [16][16]  (I + A)^-1, A_rs = beta_r GA_rs (s < r)
//     GP [16][16]  P (s <= r)            EC [dk]      e^{b_C} (KDA)
//     BE [16]      beta                  RF [4][16]   EJK: e^{b}, e^{b'}, e^{b_C - b}, e^{b_C}
// With T = (I + A)^-1 the two triangular systems of a chunk are products:
// U = T diag(beta) Y, and Z = T^T dU.
template <typename Tin>
__device__ __forceinline__ float widen(Tin x)
{
    if constexpr (std::is_same_v<Tin, float>) return x;
    else return __uint_as_float((uint32_t)x << 16);
}

template <int DK>
struct PrepLayout {
    static constexpr int RS = DK + 4;
    // what the forward scan reads comes first (it copies [0, FWD) only)
    static constexpr int KG = 0, KC = BC * RS, TI = 2 * BC * RS, EC = TI + BC * BC, BE = EC + DK, RF = BE + BC;
    static constexpr int FWD = (RF + 4 * BC + 63) / 64 * 64;
    // then Qg and P, which only the reverse scan reads
    static constexpr int QG = FWD, GP = QG + BC * RS;
    static constexpr int SIZE = (GP + BC * BC + 63) / 64 * 64;
};

// The sequence, first row and row count of chunk slot `slot`.
__device__ __forceinline__ void slot_rows(const BwdParams& p, int slot, int& n, int& c0, int& nr)
{
    int lo = 0, hi = p.N - 1;   // the last n with off[n] <= slot
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (p.off[mid] <= slot) lo = mid;
        else hi = mid - 1;
    }
    n = lo;
    int t0, t1;
    seq_bounds(p.cu, n, p.T, t0, t1);
    c0 = t0 + (slot - p.off[n]) * BC;
    nr = min(BC, t1 - c0);
}

// LDS of bwd_prep: the rows as loaded, then the decayed operands in place.
template <int DK, bool EJK>
struct PrepLds {
    static constexpr int RS = DK + 4;
    alignas(16) float QG[BC * RS];   // raw q, then Qg (EJK: qh)
    alignas(16) float KG[BC * RS];   // raw k, then Kg (EJK: kh)
    alignas(16) float KI[BC * RS];   // KDA: gate activations (log2 units), then kh e^{-b}
    float GA[BC][BC + 1];
    float NQ[BC], NK[BC], BE[BC];
    float SB[BC], SBC[BC], SBP[BC];  // EJK: gates (log2), b, b'
};

// One workgroup per (chunk slot, head): the operand block of the chunk (see
// PrepLayout).  Tin: uint16_t (bf16 bits) or float.
template <int DK, bool EJK, typename Tin>
__global__ __launch_bounds__(BT) void bwd_prep(BwdParams p)
{
    using PL = PrepLayout<DK>;
    using LT = PrepLds<DK, EJK>;
    constexpr int RS = LT::RS;
    static_assert(RS == PL::RS, "row strides");
    constexpr int NE = BC * DK / BT;   // row elements per thread
    __shared__ LT L;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int lm = lane & 15, lk = lane >> 4;
    const int slot = blockIdx.x, h = blockIdx.y;
    const int H = p.H, Hkv = p.Hkv;
    const int hk = h / (H / Hkv);
    if (slot >= p.off[p.N]) return;
    int n, c0, nr;
    slot_rows(p, slot, n, c0, nr);
    float* o = p.prep + ((size_t)slot * H + h) * PL::SIZE;
    // 1. the rows to LDS (rows past nr neutral), gate activations in log2 units.
    // Every load is issued before the first is used: through buffer resources
    // over the chunk's rows (rows past nr outside the range, read as zero), so
    // no path differs and one wait covers them all
    {
        const float ea = EJK ? 0.f : expf(p.a_log[h]);
        const float lb2 = p.lb * kLog2e;
        constexpr int SQ = (int)sizeof(Tin);
        const int qs = H * DK, ks = Hkv * DK;   // row strides (elements)
        const char* qsrc = reinterpret_cast<const char*>(static_cast<const Tin*>(p.q) + ((size_t)c0 * H + h) * DK);
        const char* ksrc = reinterpret_cast<const char*>(static_cast<const Tin*>(p.k) + ((size_t)c0 * Hkv + hk) * DK);
        const char* gsrc = EJK ? nullptr : reinterpret_cast<const char*>(p.g + ((size_t)c0 * H + h) * DK);
        // element e = tid + m BT: row e / DK (step m covers rows from m BT / DK
        // on, the lane's row within it is tid / DK), channel e % DK
        const int r0 = tid / DK, i = tid % DK;
        Tin xq[NE], xk[NE];
        float xg[EJK ? 1 : NE];
#pragma unroll
        for (int m = 0; m < NE; ++m) {
            const int rm = m * (BT / DK);
            xq[m] = buf_load<Tin>(rows_rsrc(qsrc, rm, nr, qs * SQ, DK * SQ), (r0 * qs + i) * SQ);
            xk[m] = buf_load<Tin>(rows_rsrc(ksrc, rm, nr, ks * SQ, DK * SQ), (r0 * ks + i) * SQ);
            if constexpr (!EJK) xg[m] = buf_load<float>(rows_rsrc(gsrc, rm, nr, qs * 4, DK * 4), (r0 * qs + i) * 4);
        }
        // dt_bias of the lane's channel (zeros without one); beta and the EJK
        // decay of row tid % BC
        const auto rd = buf_rsrc(EJK ? nullptr : p.dt_bias, (!EJK && p.dt_bias) ? (uint32_t)(DK * H * 4) : 0u);
        const float dtb = buf_load<float>(rd, (uint32_t)((i * H + h) * 4));
        const int rr = tid % BC;
        float bl = buf_load<float>(rows_rsrc(p.beta + (size_t)c0 * H + h, 0, nr, H * 4, 4), rr * H * 4);
        float sg = 0.f;
        if constexpr (EJK)
            sg = buf_load<float>(rows_rsrc(p.g ? p.g + (size_t)c0 * H + h : nullptr, 0, p.g ? nr : 0, H * 4, 4),
                                 rr * H * 4);
#pragma unroll
        for (int m = 0; m < NE; ++m) {
            settle(xq[m]);
            settle(xk[m]);
            if constexpr (!EJK) settle(xg[m]);
        }
        settle(bl);
#pragma unroll
        for (int m = 0; m < NE; ++m) {
            const int r = m * (BT / DK) + r0;
            L.QG[r * RS + i] = widen(xq[m]);
            L.KG[r * RS + i] = widen(xk[m]);
            if constexpr (!EJK) L.KI[r * RS + i] = r < nr ? lb2 * sigmoid_fast(ea * (xg[m] + dtb)) : 0.f;
        }
        if (tid < BC) {
            const bool ok = tid < nr;
            L.BE[tid] = ok ? (EJK ? bl : sigmoid_fast(bl)) : 0.f;
            if (EJK) L.SB[tid] = ok ? sg * kLog2e : 0.f;
        }
    }
    __syncthreads();
    // 2. row scales (eight lanes per row, summed by DPP / swizzle); EJK: the
    // scalar cumulative decays, each of 16 lanes summing in row order; KDA:
    // every thread reads its channel's 16 gates (its rows are rewritten below)
    {
        const int pr = tid >> 3, part = tid & 7;
        const int r = pr & 15;
        const float* row = (pr < 16 ? L.QG : L.KG) + r * RS;
        float ss = 0.f;
#pragma unroll
        for (int m = 0; m < DK / 8; ++m) ss = fmaf(row[part + 8 * m], row[part + 8 * m], ss);
        ss = xor_add<1>(ss);
        ss = xor_add<2>(ss);
        ss = xor_add<4>(ss);
        if (part == 0) {
            const float rn = p.l2norm ? 1.f / sqrtf(ss + kNormEps) : 1.f;
            if (pr < 16) L.NQ[r] = p.scale * rn;
            else L.NK[r] = rn;
        }
    }
    if (EJK && tid >= BT - BC) {
        const int r = tid - (BT - BC);
        float acc = 0.f, b = 0.f, bp = 0.f;
#pragma unroll
        for (int s2 = 0; s2 < BC; ++s2) {
            if (s2 == r) bp = acc;
            acc += L.SB[s2];
            if (s2 == r) b = acc;
        }
        L.SBC[r] = b;
        L.SBP[r] = bp;
        o[PL::RF + r] = __builtin_amdgcn_exp2f(b);
        o[PL::RF + BC + r] = __builtin_amdgcn_exp2f(bp);
        o[PL::RF + 2 * BC + r] = __builtin_amdgcn_exp2f(acc - b);
        o[PL::RF + 3 * BC + r] = __builtin_amdgcn_exp2f(acc);
    }
    constexpr int NPRT = BT / DK, RP = BC / NPRT;   // KDA: parts per channel, rows per part
    float gcol[EJK ? 1 : BC];
    if (!EJK) {
#pragma unroll
        for (int s2 = 0; s2 < BC; ++s2) gcol[s2] = L.KI[s2 * RS + tid % DK];
    }
    __syncthreads();
    // 3. the normalised, decayed rows: in LDS for the Gram products and, for
    // the thread's own rows, to the block
    if constexpr (!EJK) {
        const int i = tid % DK, part = tid / DK;
        float bo[RP];
        float b = 0.f;
#pragma unroll
        for (int s2 = 0; s2 < BC; ++s2) {
            b += gcol[s2];
#pragma unroll
            for (int x = 0; x < RP; ++x)
                if (s2 == part * RP + x) bo[x] = b;
        }
        if (part == 0) o[PL::EC + i] = __builtin_amdgcn_exp2f(b);
#pragma unroll
        for (int x = 0; x < RP; ++x) {
            const int r = part * RP + x;
            const float qn = L.QG[r * RS + i] * L.NQ[r];
            const float kn = L.KG[r * RS + i] * L.NK[r];
            const float f = __builtin_amdgcn_exp2f(bo[x]);
            const float qg = qn * f, kg = kn * f;
            L.QG[r * RS + i] = qg;
            L.KG[r * RS + i] = kg;
            L.KI[r * RS + i] = kn * __builtin_amdgcn_exp2f(-bo[x]);
            o[PL::QG + r * RS + i] = qg;
            o[PL::KG + r * RS + i] = kg;
            o[PL::KC + r * RS + i] = kn * __builtin_amdgcn_exp2f(b - bo[x]);
        }
    } else {
#pragma unroll
        for (int m = 0; m < NE; ++m) {
            const int e = tid + m * BT;
            const int r = e / DK, i = e % DK;
            const float qn = L.QG[r * RS + i] * L.NQ[r];
            const float kn = L.KG[r * RS + i] * L.NK[r];
            L.QG[r * RS + i] = qn;
            L.KG[r * RS + i] = kn;
            o[PL::QG + r * RS + i] = qn;
            o[PL::KG + r * RS + i] = kn;
        }
    }
    if (tid < BC) o[PL::BE + tid] = L.BE[tid];
    __syncthreads();
    // 4. the Gram products on 16x16x4 float32 MFMA: wave 0 GA (Kg against
    // kh e^{-b}), wave 1 P (Qg against kh e^{-b}); EJK: the plain dots scaled
    // by the element factors.  Lane (lm, lk) supplies channel k0 + 4 lk + u of
    // row lm of both operands and holds rows 4 lk + e of column lm.
    if (wave < 2) {
        const float* X = wave == 0 ? L.KG : L.QG;
        const float* Y = EJK ? L.KG : L.KI;
        bf32x4_t acc = bf32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k0 = 0; k0 < DK; k0 += 16) {
            const float4 a4 = *reinterpret_cast<const float4*>(X + lm * RS + k0 + 4 * lk);
            const float4 b4 = *reinterpret_cast<const float4*>(Y + lm * RS + k0 + 4 * lk);
            acc = bmfma4(a4.x, b4.x, acc);
            acc = bmfma4(a4.y, b4.y, acc);
            acc = bmfma4(a4.z, b4.z, acc);
            acc = bmfma4(a4.w, b4.w, acc);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 4 * lk + e, s2 = lm;
            float x = acc[e];
            if (wave == 0) {
                if (EJK) x *= s2 < r ? __builtin_amdgcn_exp2f(L.SBP[r] - L.SBC[s2]) : 0.f;
                L.GA[r][s2] = s2 < r ? x : 0.f;
            } else {
                if (EJK) x *= s2 <= r ? __builtin_amdgcn_exp2f(L.SBC[r] - L.SBC[s2]) : 0.f;
                o[PL::GP + r * BC + s2] = s2 <= r ? x : 0.f;
            }
        }
    }
    __syncthreads();
    if (tid < BC) {
        // column s of (I + A)^-1, A_rt = beta_r GA_rt, by forward substitution
        const int s2 = tid;
        float x[BC];
#pragma unroll
        for (int r = 0; r < BC; ++r) {
            float v = r == s2 ? 1.f : 0.f;
#pragma unroll
            for (int t = 0; t < r; ++t) v = fmaf(-L.BE[r] * L.GA[r][t], x[t], v);
            x[r] = v;
            o[PL::TI + r * BC + s2] = v;
        }
    }
}

// The (16 state columns, head, sequence) unit of a scan workgroup.  Linear
// workgroup ids are dealt to the 8 XCDs in turn, so the column tiles of one
// (head, sequence), which read the same chunk operands, are given ids that
// are equal modulo 8: they run on one XCD and share its L2.  Returns false
// for the padding ids past the last (head, sequence).
__device__ __forceinline__ bool scan_unit(const BwdParams& p, int ng, int& j0, int& h, int& n)
{
    const int ntile = p.dv / (TV * ng);
    const int id = blockIdx.x;
    const int xcd = id & 7, q = id >> 3;
    const int grp = (q / ntile) * 8 + xcd;
    if (grp >= p.H * p.N) return false;
    j0 = (q % ntile) * TV * ng;
    h = grp % p.H;
    n = grp / p.H;
    return true;
}

typedef float f4v __attribute__((ext_vector_type(4)));

// The chunk's operand block, 16 bytes per thread and step, into registers.
// Every thread issues the same loads (an index past the block is clamped to
// its last piece, stored again to the same place), so the count of memory
// operations in flight is the same on every path and the waits for a load
// issued chunks earlier stay exact.
template <int NP, int N4, int NTH>
__device__ __forceinline__ void fetch_block(f4v (&pf)[NP], const float* src)
{
    const f4v* s4 = reinterpret_cast<const f4v*>(src);
#pragma unroll
    for (int m = 0; m < NP; ++m) pf[m] = s4[min((int)threadIdx.x + m * NTH, N4 - 1)];
}

template <int NP, int N4, int NTH>
__device__ __forceinline__ void store_block(float* dst, const f4v (&pf)[NP])
{
#pragma unroll
    for (int m = 0; m < NP; ++m) reinterpret_cast<f4v*>(dst)[min((int)threadIdx.x + m * NTH, N4 - 1)] = pf[m];
}

// An empty use of each register: the compiler waits here for the loads that
// write them.
using kda::settle;
template <int N>
__device__ __forceinline__ void settle(bf32x4_t (&v)[N])
{
#pragma unroll
    for (int x = 0; x < N; ++x) asm volatile("" : "+v"(v[x]));
}

// A buffer resource over [base, base + bytes): the buffer unit drops stores
// at offsets past the end, so a store that only some waves must make is
// issued by all of them, the others given bytes = 0 (no branch, and the same
// count of memory operations on every path).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t store_range(const float* base, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, bytes, 0x00020000);
}

__device__ __forceinline__ void store_at(__amdgpu_buffer_rsrc_t r, int byte_off, float v)
{
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, byte_off, 0, 0);
}

// The local pass's padded columns get an offset past every resource it uses
// (all under 2^31 bytes), so their stores are dropped.
constexpr uint32_t kNoOffset = 0x80000000u;

// The scans' register layout: the dk x 16 state (or state gradient) tile is
// held in the accumulators of 16x16x4 float32 MFMA, 16 rows per tile (tiles
// dealt over the waves); element e of lane (lm, lk) holds row 4 lk + e,
// column lm, which is also what that lane supplies as the B operand at step
// e of a product over those rows.  The 16x16 products U = T diag(beta) Y and
// Z = T^T dU are formed by every wave in the same layout, so each feeds its
// own state update without another exchange.  Per chunk the scan copies the
// chunk's operand block (prefetched into registers while the chunk before
// computed) to one of two LDS buffers; two barriers, waiting for LDS only:
// one after the copy, one after the per-wave partials of the product over
// dk.  A buffer is rewritten two chunks later, after every wave has passed
// the next chunk's first barrier.
template <int DK, int NG>
struct ScanLds {
    alignas(16) float P[2][PrepLayout<DK>::SIZE];
    float X[NG][2][BC][TV + 1];          // V (pass 1) or dO (pass 2) of each group's tile
    float PU[NG][BT / kWave][BC][TV + 1];
};

// Pass 1: the forward state carry per (16 state columns, head, sequence);
// stores the state entering every chunk and the chunk's Y and U:
//     Y = V - Kg S,  U = T diag(beta) Y,  S <- Diag(e^{b_C}) S + Kc^T U
template <int DK, bool EJK, typename Tin, int NG>
__global__ __launch_bounds__(NG * BT) __attribute__((amdgpu_waves_per_eu(2))) void bwd_fwd_scan(BwdParams p)
{
    using PL = PrepLayout<DK>;
    constexpr int RS = PL::RS;
    constexpr int NT = DK / 16, NW = BT / kWave, TPW = (NT + NW - 1) / NW;
    constexpr int N4 = PL::FWD / 4, NP = (N4 + NG * BT - 1) / (NG * BT);   // Qg and P unused here
    __shared__ ScanLds<DK, NG> L;
    // NG groups of four waves, each on its own 16 state columns, share the
    // chunk's operand block in LDS
    // (the group and wave indices are wave-uniform: kept in scalar registers,
    // so that resources built from them need no per-lane loop)
    const int tid = threadIdx.x % BT, grp = __builtin_amdgcn_readfirstlane(threadIdx.x / BT) & (NG - 1);
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6) & (NW - 1);
    // (the masks change no value: they restate the ranges that readfirstlane
    // hides from the compiler, which then folds the per-wave selections)
    static_assert((NG & (NG - 1)) == 0 && (NW & (NW - 1)) == 0, "power-of-two group and wave counts");
    const int lm = lane & 15, lk = lane >> 4;
    int j0, h, n;
    if (!scan_unit(p, NG, j0, h, n)) return;
    j0 += grp * TV;
    const int H = p.H, dv = p.dv;
    const int hk = h / (H / p.Hkv);
    int t0, t1;
    seq_bounds(p.cu, n, p.T, t0, t1);
    // the initial state tile (zeros without one; rows of idle waves' tiles,
    // t >= NT, fall past the range), every load issued before one wait
    bf32x4_t S[TPW];
    {
        const auto ri = buf_rsrc(p.init ? uniform_ptr(p.init + ((size_t)n * H + h) * DK * dv) : nullptr,
                                 p.init ? (uint32_t)(DK * dv * 4) : 0u);
#pragma unroll
        for (int x = 0; x < TPW; ++x) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                S[x][e] = buf_load<float>(ri, (uint32_t)(((16 * (wave + NW * x) + 4 * lk + e) * dv + j0 + lm) * 4));
        }
    }
    // the initial tile is used here, before the loop: else its loads stay
    // pending into the loop body, whose first use would then wait for every
    // load in flight, the next chunk's prefetch included
    settle(S);
    const int nck = seq_chunks(p.off, n, t0, t1);
    const int slot0 = p.off[n];
    // the sequence's pair-checkpoint range, read once and kept wave-uniform (the
    // checkpoint stores through p could alias p.poff, so inside the loop the
    // compiler would reload it after every store, and a divergent-looking range
    // makes every store a per-lane loop)
    const int pair0 = __builtin_amdgcn_readfirstlane(p.poff[n]);
    const int pair1 = __builtin_amdgcn_readfirstlane(p.poff[n + 1]);
    const Tin* vv = static_cast<const Tin*>(p.v);
    // a ring of two register sets: the inputs of chunk c + 2 are loaded while
    // chunk c computes (the loop is unrolled by two, so each set is fixed)
    f4v pfa[NP], pfb[NP];
    Tin pva = 0, pvb = 0;
    const int rr = tid / TV, jj = tid % TV;
    auto fetch = [&](f4v (&pf)[NP], Tin& pv, int c) __attribute__((always_inline)) {
        const int cs = t0 + c * BC;
        fetch_block<NP, N4, NG * BT>(pf, p.prep + ((size_t)(slot0 + c) * H + h) * PL::SIZE);
        pv = vv[((size_t)(cs + (cs + rr < t1 ? rr : 0)) * p.Hkv + hk) * dv + j0 + jj];
    };
    if (nck > 0) {
        fetch(pfa, pva, 0);
        fetch(pfb, pvb, min(1, nck - 1));
        // both sets waited for here: the compiler interleaves their loads, and
        // the count of loads in flight that it assumes at the loop head is the
        // larger of the counts on entry and around the loop, so a wait left
        // pending here would drain the next chunk's prefetch on every chunk
        settle(pfa);
        settle(pfb);
        settle(pva);
        settle(pvb);
    }
    auto chunk = [&](f4v (&pf)[NP], Tin& pv, int c, auto bsel) __attribute__((always_inline)) {
        constexpr int b = decltype(bsel)::value;
            const int c0 = t0 + c * BC;
            const float* P = L.P[b];
            // the prefetched block to LDS first, then the state stores: a later
            // wait for a load then never waits for these stores as well
            store_block<NP, N4, NG * BT>(L.P[b], pf);
            L.X[grp][b][rr][jj] = c0 + rr < t1 ? widen(pv) : 0.f;
            if constexpr (b == 0) {
                // the state entering a pair's first chunk (c even); tiles t >= NT
                // (idle waves at small dk) fall past the range
                // (pairs past the capped count of overlapping ranges store nothing)
                const int pi = pair0 + c / 2;
                const auto rs = store_range(p.ckS + (((size_t)pi * H + h) * (dv / TV) + j0 / TV) * DK * TV,
                                            pi < pair1 ? DK * TV * 4 : 0);
#pragma unroll
                for (int x = 0; x < TPW; ++x) {
                    const int t = wave + NW * x;
#pragma unroll
                    for (int e = 0; e < 4; ++e) store_at(rs, ((16 * t + 4 * lk + e) * TV + lm) * 4, S[x][e]);
                }
            }
            fetch(pf, pv, min(c + 2, nck - 1));   // past the end: the last chunk again
            lds_barrier();
            // Kg S: each wave its tiles' part (A = Kg rows, 16 bytes per lane)
            {
                bf32x4_t acc = bf32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int x = 0; x < TPW; ++x) {
                    const int t = wave + NW * x;
                    if (t < NT) {
                        const float4 a = *reinterpret_cast<const float4*>(P + PL::KG + lm * RS + 16 * t + 4 * lk);
                        acc = bmfma4(a.x, S[x][0], acc);
                        acc = bmfma4(a.y, S[x][1], acc);
                        acc = bmfma4(a.z, S[x][2], acc);
                        acc = bmfma4(a.w, S[x][3], acc);
                    }
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) L.PU[grp][wave][4 * lk + e][lm] = acc[e];
            }
            lds_barrier();
            // Y (rows 4 lk + u of column lm) and U = T diag(beta) Y, in every wave
            bf32x4_t U = bf32x4_t{0.f, 0.f, 0.f, 0.f};
            float y[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int k = 4 * lk + u;
                float ks = (L.PU[grp][0][k][lm] + L.PU[grp][1][k][lm]) + (L.PU[grp][2][k][lm] + L.PU[grp][3][k][lm]);
                if (EJK) ks *= P[PL::RF + BC + k];
                y[u] = L.X[grp][b][k][lm] - ks;
                U = bmfma4(P[PL::TI + lm * BC + k], P[PL::BE + k] * y[u], U);
            }
            {
                // wave 0 stores Y and U (the others' range is empty)
                const auto rs = store_range(p.ckYU + ((size_t)(slot0 + c) * H + h) * 2 * BC * dv,
                                            wave == 0 ? 2 * BC * dv * 4 : 0);
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    store_at(rs, ((4 * lk + u) * dv + j0 + lm) * 4, y[u]);
                    store_at(rs, ((BC + 4 * lk + u) * dv + j0 + lm) * 4, U[u]);
                }
            }
            // S <- Diag(e^{b_C}) S + Kc^T U (EJK: kh^T (e^{b_C - b} U))
            if (EJK) {
#pragma unroll
                for (int u = 0; u < 4; ++u) U[u] *= P[PL::RF + 2 * BC + 4 * lk + u];
            }
#pragma unroll
            for (int x = 0; x < TPW; ++x) {
                const int t = wave + NW * x;
                if (t < NT) {
                    bf32x4_t a = S[x];
#pragma unroll
                    for (int e = 0; e < 4; ++e) a[e] *= EJK ? P[PL::RF + 3 * BC] : P[PL::EC + 16 * t + 4 * lk + e];
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        a = bmfma4(P[(EJK ? PL::KG : PL::KC) + (4 * lk + u) * RS + 16 * t + lm], U[u], a);
                    S[x] = a;
                }
            }
    };
    // both halves of the loop body run on every pass, an odd last chunk after
    // the loop: a half skipped on some path into the loop head would make the
    // compiler assume the shorter count of loads in flight there, and wait for
    // the prefetch on every chunk
    int c = 0;
    for (; c + 1 < nck; c += 2) {
        chunk(pfa, pva, c, std::integral_constant<int, 0>{});
        chunk(pfb, pvb, c + 1, std::integral_constant<int, 1>{});
    }
    if (c < nck) chunk(pfa, pva, c, std::integral_constant<int, 0>{});
}

// The prefill's output on the same 16-token chunks and operand blocks (the
// float32-arithmetic route of calls with a workspace): per (16 state columns, head,
// sequence) and chunk
//     Y = V - Kg S,  U = T diag(beta) Y,  O = Qg S + P U,
//     S <- Diag(e^{b_C}) S + Kc^T U
// (EJK: qh and kh with the scalar row factors, P with its decay factors
// already applied), then the final state.  The products over dk are summed
// over the waves in LDS; every wave then forms U and O in its registers and
// stores one row of O in four.
template <int DK, int NG>
struct OutLds {
    alignas(16) float P[2][PrepLayout<DK>::SIZE];
    float X[NG][2][BC][TV + 1];               // V of each group's tile
    float PU[NG][BT / kWave][BC][TV + 1];     // per-wave partials of Kg S
    float PQ[NG][BT / kWave][BC][TV + 1];     // and of Qg S
};

template <int DK, bool EJK, typename Tin, typename Tout, int NG>
__global__ __launch_bounds__(NG * BT) __attribute__((amdgpu_waves_per_eu(2))) void prefill16_scan(BwdParams p)
{
    using PL = PrepLayout<DK>;
    constexpr int RS = PL::RS;
    constexpr int NT = DK / 16, NW = BT / kWave, TPW = (NT + NW - 1) / NW;
    constexpr int N4 = PL::SIZE / 4, NP = (N4 + NG * BT - 1) / (NG * BT);
    constexpr uint32_t SO = sizeof(Tout);
    __shared__ OutLds<DK, NG> L;
    const int tid = threadIdx.x % BT, grp = __builtin_amdgcn_readfirstlane(threadIdx.x / BT) & (NG - 1);
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6) & (NW - 1);
    // (the masks change no value: they restate the ranges that readfirstlane
    // hides from the compiler, which then folds the per-wave selections)
    static_assert((NG & (NG - 1)) == 0 && (NW & (NW - 1)) == 0, "power-of-two group and wave counts");
    const int lm = lane & 15, lk = lane >> 4;
    int j0, h, n;
    if (!scan_unit(p, NG, j0, h, n)) return;
    j0 += grp * TV;
    const int H = p.H, dv = p.dv;
    const int hk = h / (H / p.Hkv);
    int t0, t1;
    seq_bounds(p.cu, n, p.T, t0, t1);
    t0 = __builtin_amdgcn_readfirstlane(t0);
    t1 = __builtin_amdgcn_readfirstlane(t1);
    // the initial state tile (zeros without one), all loads before one wait
    bf32x4_t S[TPW];
    {
        const auto ri = buf_rsrc(p.init ? uniform_ptr(p.init + ((size_t)n * H + h) * DK * dv) : nullptr,
                                 p.init ? (uint32_t)(DK * dv * 4) : 0u);
#pragma unroll
        for (int x = 0; x < TPW; ++x) {
            const int t = wave + NW * x;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * t + 4 * lk + e;
                // rows of idle waves' tiles (t >= NT) fall past the range
                S[x][e] = buf_load<float>(ri, (uint32_t)((i * dv + j0 + lm) * 4));
            }
        }
        settle(S);
    }
    const int nck = seq_chunks(p.off, n, t0, t1);
    const int slot0 = p.off[n];
    const Tin* vv = static_cast<const Tin*>(p.v);
    // a ring of two register sets: the inputs of chunk c + 2 are loaded while
    // chunk c computes (the loop is unrolled by two, so each set is fixed)
    f4v pfa[NP], pfb[NP];
    Tin pva = 0, pvb = 0;
    const int rr = tid / TV, jj = tid % TV;
    auto fetch = [&](f4v (&pf)[NP], Tin& pv, int c) __attribute__((always_inline)) {
        const int cs = t0 + c * BC;
        fetch_block<NP, N4, NG * BT>(pf, p.prep + ((size_t)(slot0 + c) * H + h) * PL::SIZE);
        pv = vv[((size_t)(cs + (cs + rr < t1 ? rr : 0)) * p.Hkv + hk) * dv + j0 + jj];
    };
    if (nck > 0) {
        fetch(pfa, pva, 0);
        fetch(pfb, pvb, min(1, nck - 1));
        // both sets waited for here: the compiler interleaves their loads, and
        // the count of loads in flight that it assumes at the loop head is the
        // larger of the counts on entry and around the loop, so a wait left
        // pending here would drain the next chunk's prefetch on every chunk
        settle(pfa);
        settle(pfb);
        settle(pva);
        settle(pvb);
    }
    Tout* const ob = static_cast<Tout*>(p.out);
    auto chunk = [&](f4v (&pf)[NP], Tin& pv, int c, auto bsel) __attribute__((always_inline)) {
        constexpr int b = decltype(bsel)::value;
        const int c0 = t0 + c * BC, nr = min(BC, t1 - c0);
        const float* P = L.P[b];
        store_block<NP, N4, NG * BT>(L.P[b], pf);
        L.X[grp][b][rr][jj] = c0 + rr < t1 ? widen(pv) : 0.f;
        fetch(pf, pv, min(c + 2, nck - 1));   // past the end: the last chunk again
        lds_barrier();
        // Kg S and Qg S: each wave its tiles' part (A = the rows, 16 bytes per lane)
        {
            bf32x4_t ak = bf32x4_t{0.f, 0.f, 0.f, 0.f}, aq = ak;
#pragma unroll
            for (int x = 0; x < TPW; ++x) {
                const int t = wave + NW * x;
                if (t < NT) {
                    const float4 a = *reinterpret_cast<const float4*>(P + PL::KG + lm * RS + 16 * t + 4 * lk);
                    const float4 qa = *reinterpret_cast<const float4*>(P + PL::QG + lm * RS + 16 * t + 4 * lk);
                    ak = bmfma4(a.x, S[x][0], ak);
                    aq = bmfma4(qa.x, S[x][0], aq);
                    ak = bmfma4(a.y, S[x][1], ak);
                    aq = bmfma4(qa.y, S[x][1], aq);
                    ak = bmfma4(a.z, S[x][2], ak);
                    aq = bmfma4(qa.z, S[x][2], aq);
                    ak = bmfma4(a.w, S[x][3], ak);
                    aq = bmfma4(qa.w, S[x][3], aq);
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                L.PU[grp][wave][4 * lk + e][lm] = ak[e];
                L.PQ[grp][wave][4 * lk + e][lm] = aq[e];
            }
        }
        lds_barrier();
        // Y (rows 4 lk + u of column lm) and U = T diag(beta) Y, in every wave
        bf32x4_t U = bf32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int k = 4 * lk + u;
            float ks = (L.PU[grp][0][k][lm] + L.PU[grp][1][k][lm]) + (L.PU[grp][2][k][lm] + L.PU[grp][3][k][lm]);
            if (EJK) ks *= P[PL::RF + BC + k];
            const float y = L.X[grp][b][k][lm] - ks;
            U = bmfma4(P[PL::TI + lm * BC + k], P[PL::BE + k] * y, U);
        }
        // O = Qg S + P U (rows 4 lk + e of column lm); U is the B operand as held
        {
            bf32x4_t o;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * lk + e;
                const float qs = (L.PQ[grp][0][r][lm] + L.PQ[grp][1][r][lm]) + (L.PQ[grp][2][r][lm] + L.PQ[grp][3][r][lm]);
                o[e] = EJK ? qs * P[PL::RF + r] : qs;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) o = bmfma4(P[PL::GP + lm * BC + 4 * lk + u], U[u], o);
            // wave w stores rows 4 lk + w; rows past the sequence fall outside
            const float ow = wave == 0 ? o[0] : wave == 1 ? o[1] : wave == 2 ? o[2] : o[3];
            const auto ro = rows_rsrc(ob + ((size_t)c0 * H + h) * dv + j0, 0, nr, (uint32_t)(H * dv) * SO, TV * SO);
            buf_store<Tout>(ro, (uint32_t)(((4 * lk + wave) * H * dv + lm) * SO), from_f32<Tout>(ow));
        }
        // S <- Diag(e^{b_C}) S + Kc^T U (EJK: kh^T (e^{b_C - b} U))
        if (EJK) {
#pragma unroll
            for (int u = 0; u < 4; ++u) U[u] *= P[PL::RF + 2 * BC + 4 * lk + u];
        }
#pragma unroll
        for (int x = 0; x < TPW; ++x) {
            const int t = wave + NW * x;
            if (t < NT) {
                bf32x4_t a = S[x];
#pragma unroll
                for (int e = 0; e < 4; ++e) a[e] *= EJK ? P[PL::RF + 3 * BC] : P[PL::EC + 16 * t + 4 * lk + e];
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    a = bmfma4(P[(EJK ? PL::KG : PL::KC) + (4 * lk + u) * RS + 16 * t + lm], U[u], a);
                S[x] = a;
            }
        }
    };
    // both halves of the loop body run on every pass, an odd last chunk after
    // the loop: a half skipped on some path into the loop head would make the
    // compiler assume the shorter count of loads in flight there, and wait for
    // the prefetch on every chunk
    int c = 0;
    for (; c + 1 < nck; c += 2) {
        chunk(pfa, pva, c, std::integral_constant<int, 0>{});
        chunk(pfb, pvb, c + 1, std::integral_constant<int, 1>{});
    }
    if (c < nck) chunk(pfa, pva, c, std::integral_constant<int, 0>{});
    if (p.fstate) {
        float* fs = p.fstate + ((size_t)n * H + h) * DK * dv;
#pragma unroll
        for (int x = 0; x < TPW; ++x) {
            const int t = wave + NW * x;
            if (t < NT) {
#pragma unroll
                for (int e = 0; e < 4; ++e) fs[(size_t)(16 * t + 4 * lk + e) * dv + j0 + lm] = S[x][e];
            }
        }
    }
}

// Pass 2: the state gradient carried backward per (16 state columns, head,
// sequence); stores dL/d(state leaving) and Z of every chunk, and at the end
// dL/d(initial state).  Per chunk, last to first:
//     dU = Kc dS + P^T dO   (a partial per wave, summed in LDS)
//     Z = T^T dU,  dY = diag(beta) Z
//     dS <- Diag(e^{b_C}) dS + Qg^T dO - Kg^T dY
// (EJK: qh, kh with the scalar row factors applied to dO, dY and dU rows).
template <int DK, bool EJK, typename Tin, int NG>
__global__ __launch_bounds__(NG * BT) __attribute__((amdgpu_waves_per_eu(2))) void bwd_rev_scan(BwdParams p)
{
    using PL = PrepLayout<DK>;
    constexpr int RS = PL::RS;
    constexpr int NT = DK / 16, NW = BT / kWave, TPW = (NT + NW - 1) / NW;
    constexpr int N4 = PL::SIZE / 4, NP = (N4 + NG * BT - 1) / (NG * BT);
    __shared__ ScanLds<DK, NG> L;
    // NG groups of four waves, each on its own 16 state columns, share the
    // chunk's operand block in LDS
    // (the group and wave indices are wave-uniform: kept in scalar registers,
    // so that resources built from them need no per-lane loop)
    const int tid = threadIdx.x % BT, grp = __builtin_amdgcn_readfirstlane(threadIdx.x / BT) & (NG - 1);
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6) & (NW - 1);
    // (the masks change no value: they restate the ranges that readfirstlane
    // hides from the compiler, which then folds the per-wave selections)
    static_assert((NG & (NG - 1)) == 0 && (NW & (NW - 1)) == 0, "power-of-two group and wave counts");
    const int lm = lane & 15, lk = lane >> 4;
    int j0, h, n;
    if (!scan_unit(p, NG, j0, h, n)) return;
    j0 += grp * TV;
    const int H = p.H, dv = p.dv;
    int t0, t1;
    seq_bounds(p.cu, n, p.T, t0, t1);
    bf32x4_t dS[TPW];
    {
        const auto ri = buf_rsrc(p.dSf ? uniform_ptr(p.dSf + ((size_t)n * H + h) * DK * dv) : nullptr,
                                 p.dSf ? (uint32_t)(DK * dv * 4) : 0u);
#pragma unroll
        for (int x = 0; x < TPW; ++x) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                dS[x][e] = buf_load<float>(ri, (uint32_t)(((16 * (wave + NW * x) + 4 * lk + e) * dv + j0 + lm) * 4));
        }
    }
    settle(dS);   // as in the forward scan
    const int nck = seq_chunks(p.off, n, t0, t1);
    const int slot0 = p.off[n];
    // the sequence's pair-checkpoint range, read once and kept wave-uniform (the
    // checkpoint stores through p could alias p.poff, so inside the loop the
    // compiler would reload it after every store, and a divergent-looking range
    // makes every store a per-lane loop)
    const int pair0 = __builtin_amdgcn_readfirstlane(p.poff[n]);
    const int pair1 = __builtin_amdgcn_readfirstlane(p.poff[n + 1]);
    // a ring of two register sets: the inputs of chunk c - 2 are loaded while
    // chunk c computes (the loop is unrolled by two, so each set is fixed);
    // dO as loaded (bf16 or float32 bits), widened where used
    f4v pfa[NP], pfb[NP];
    uint32_t pda = 0, pdb = 0;
    const int rr = tid / TV, jj = tid % TV;
    auto fetch = [&](f4v (&pf)[NP], uint32_t& pd, int c) __attribute__((always_inline)) {
        const int cs = t0 + c * BC;
        fetch_block<NP, N4, NG * BT>(pf, p.prep + ((size_t)(slot0 + c) * H + h) * PL::SIZE);
        const size_t i = ((size_t)(cs + (cs + rr < t1 ? rr : 0)) * H + h) * dv + j0 + jj;
        pd = p.do_bf16 ? (uint32_t)static_cast<const uint16_t*>(p.d_o)[i] : static_cast<const uint32_t*>(p.d_o)[i];
    };
    if (nck > 0) {
        fetch(pfa, pda, nck - 1);
        fetch(pfb, pdb, max(nck - 2, 0));
        // both sets waited for here (as in the forward scan)
        settle(pfa);
        settle(pfb);
        settle(pda);
        settle(pdb);
    }
    auto chunk = [&](f4v (&pf)[NP], uint32_t& pd, int c, auto bsel) __attribute__((always_inline)) {
        constexpr int b = decltype(bsel)::value;
            const int c0 = t0 + c * BC;
            const float* P = L.P[b];
            store_block<NP, N4, NG * BT>(L.P[b], pf);
            L.X[grp][b][rr][jj] = c0 + rr < t1 ? __uint_as_float(p.do_bf16 ? pd << 16 : pd) : 0.f;
            {
                // the state gradient leaving a pair's last chunk (c odd, or the
                // sequence's last); the other chunks' stores get an empty range, as
                // do tiles t >= NT (idle waves at small dk)
                const int pi = pair0 + c / 2;
                const bool keep = ((c & 1) || c == nck - 1) && pi < pair1;
                const auto rs = store_range(p.ckdS + (((size_t)pi * H + h) * (dv / TV) + j0 / TV) * DK * TV,
                                            keep ? DK * TV * 4 : 0);
#pragma unroll
                for (int x = 0; x < TPW; ++x) {
                    const int t = wave + NW * x;
#pragma unroll
                    for (int e = 0; e < 4; ++e) store_at(rs, ((16 * t + 4 * lk + e) * TV + lm) * 4, dS[x][e]);
                }
            }
            fetch(pf, pd, max(c - 2, 0));   // before the start: the first chunk again
            lds_barrier();
            // dU: each wave its tiles' part of Kc dS; wave 1 adds P^T dO
            {
                bf32x4_t acc = bf32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int x = 0; x < TPW; ++x) {
                    const int t = wave + NW * x;
                    if (t < NT) {
                        const float4 a = *reinterpret_cast<const float4*>(P + (EJK ? PL::KG : PL::KC) + lm * RS +
                                                                          16 * t + 4 * lk);
                        acc = bmfma4(a.x, dS[x][0], acc);
                        acc = bmfma4(a.y, dS[x][1], acc);
                        acc = bmfma4(a.z, dS[x][2], acc);
                        acc = bmfma4(a.w, dS[x][3], acc);
                    }
                }
                if (EJK) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[e] *= P[PL::RF + 2 * BC + 4 * lk + e];
                }
                if (wave == 1) {
                    // (P^T dO)[m][j] = sum_s P[s][m] dO[s][j], s = 4 lk + u at step u
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int s2 = 4 * lk + u;
                        acc = bmfma4(P[PL::GP + s2 * BC + lm], L.X[grp][b][s2][lm], acc);
                    }
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) L.PU[grp][wave][4 * lk + e][lm] = acc[e];
            }
            lds_barrier();
            // Z = T^T dU in every wave: at step u the lane supplies T[4 lk + u][lm]
            // and dU[4 lk + u][lm]
            bf32x4_t Z = bf32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int k = 4 * lk + u;
                const float du = (L.PU[grp][0][k][lm] + L.PU[grp][1][k][lm]) + (L.PU[grp][2][k][lm] + L.PU[grp][3][k][lm]);
                Z = bmfma4(P[PL::TI + k * BC + lm], du, Z);
            }
            {
                // wave 0 stores Z (the others' range is empty)
                const auto rs = store_range(p.ckZ + ((size_t)(slot0 + c) * H + h) * BC * dv,
                                            wave == 0 ? BC * dv * 4 : 0);
#pragma unroll
                for (int e = 0; e < 4; ++e) store_at(rs, ((4 * lk + e) * dv + j0 + lm) * 4, Z[e]);
            }
            // dY (EJK: e^{b'} dY), rows 4 lk + e: the B operand of Kg^T dY
            float dy[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int k = 4 * lk + e;
                dy[e] = P[PL::BE + k] * Z[e];
                if (EJK) dy[e] *= P[PL::RF + BC + k];
            }
            // dS <- Diag(e^{b_C}) dS + Qg^T dO - Kg^T dY
#pragma unroll
            for (int x = 0; x < TPW; ++x) {
                const int t = wave + NW * x;
                if (t < NT) {
                    bf32x4_t a = dS[x];
#pragma unroll
                    for (int e = 0; e < 4; ++e) a[e] *= EJK ? P[PL::RF + 3 * BC] : P[PL::EC + 16 * t + 4 * lk + e];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int r = 4 * lk + u;
                        const float d = EJK ? L.X[grp][b][r][lm] * P[PL::RF + r] : L.X[grp][b][r][lm];
                        a = bmfma4(P[PL::QG + r * RS + 16 * t + lm], d, a);
                    }
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        a = bmfma4(-P[PL::KG + (4 * lk + u) * RS + 16 * t + lm], dy[u], a);
                    dS[x] = a;
                }
            }
    };
    int k = 0;   // (loop shape as in the forward scan)
    for (; k + 1 < nck; k += 2) {
        chunk(pfa, pda, nck - 1 - k, std::integral_constant<int, 0>{});
        chunk(pfb, pdb, nck - 2 - k, std::integral_constant<int, 1>{});
    }
    if (k < nck) chunk(pfa, pda, nck - 1 - k, std::integral_constant<int, 0>{});
    if (p.dS0) {
#pragma unroll
        for (int x = 0; x < TPW; ++x) {
            const int t = wave + NW * x;
            if (t < NT) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 16 * t + 4 * lk + e;
                    p.dS0[(((size_t)n * H + h) * DK + i) * dv + j0 + lm] = dS[x][e];
                }
            }
        }
    }
}

// Pass 3: the gradients of the chunks' rows, one workgroup per (pair of
// consecutive chunks of a sequence, head) with all state columns.  The scans
// store the state entering the first chunk of a pair and the state gradient
// leaving its second chunk (checkpoints every 32 tokens); the pair's other two
// are one step of each recurrence away, taken here on MFMA:
//     S entering the second chunk = Diag(e^{b_C}) S0 + Kc^T U   (first chunk's Kc, U)
//     dS leaving the first chunk  = Diag(e^{b_C}) dS1 + Qg^T dO - Kg^T dY   (second chunk's)
// The second chunk is done first (its inputs then still in LDS give the
// backward step), then the first.  A chunk's gradients come from its S0,
// dS1, Y and U (pass 1) and Z (pass 2).  The products run on 16x16x4 float32
// MFMA; from the Gram-role products on, each lane keeps the elements (row
// 4 lk + e, channel 16 t + lm) of its tiles in registers up to their stores,
// so LDS holds the set-up, dO, U, Z and small per-row arrays, and two
// workgroups share a CU.
template <int DK, bool EJK, typename Tin>
__global__ __launch_bounds__(BT) __attribute__((amdgpu_waves_per_eu(2))) void bwd_local(BwdParams p)
{
    constexpr int NT = DK / 16;               // 16-channel tiles
    constexpr int NW = BT / kWave;
    constexpr int TPW = (NT + NW - 1) / NW;   // tiles per wave
    constexpr int NJ = MAXD / 16;
    constexpr int NE = BC * DK / BT;          // q, k elements per thread
    constexpr int NV = BC * MAXD / BT;        // [16][MAXD] elements per thread
    static_assert(BT == 2 * MAXD && NW == 4, "a [16][MAXD] row spans two waves");
    __shared__ ChunkLds<DK, EJK> L;
    __shared__ float dO[BC][SR];
    __shared__ float U[BC][SR];
    __shared__ float Z[BC][SR];
    __shared__ float MA[BC][BC + 1], MP[BC][BC + 1], dA[BC][BC + 1];
    __shared__ float zyw[NW][NV];               // Z.Y partials, row 2 m + (wave >> 1)
    __shared__ float rq[NW][BC], rk[NW][BC];    // row dots of the L2-norm backward, per wave
    __shared__ float ra[NW][BC], rb[NW][BC], rc[NW][BC], rd[NW];   // EJK row sums, per wave
    __shared__ float dbt[BC], dgs[BC];
    __shared__ float red[NW];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int lm = lane & 15, lk = lane >> 4;
    const int slot = blockIdx.x, h = blockIdx.y;
    const int H = p.H, Hkv = p.Hkv, dv = p.dv;
    const int hk = h / (H / Hkv);
    const bool grouped = Hkv != H;
    const int ps = slot;   // the pair slot
    if (ps >= p.poff[p.N]) return;
    // the sequence of this pair: the last n with poff[n] <= ps
    int lo = 0, hi = p.N - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (p.poff[mid] <= ps) lo = mid;
        else hi = mid - 1;
    }
    // the sequence and its ranges in scalar registers, read once: read where
    // used, the chunk offset was a vector load issued after the chunk's inputs
    // and waited for at once, with them
    const int n = __builtin_amdgcn_readfirstlane(lo);
    int t0, t1;
    seq_bounds(p.cu, n, p.T, t0, t1);
    t0 = __builtin_amdgcn_readfirstlane(t0);
    t1 = __builtin_amdgcn_readfirstlane(t1);
    const int offn = __builtin_amdgcn_readfirstlane(p.off[n]);
    const int nck = __builtin_amdgcn_readfirstlane(seq_chunks(p.off, n, t0, t1));
    const int ca = 2 * (ps - __builtin_amdgcn_readfirstlane(p.poff[n]));   // the pair's chunks: ca and, if it exists, ca + 1
    const bool has_b = ca + 1 < nck;
    const int nj = dv / 16;
    const float ea = EJK ? 0.f : expf(p.a_log[h]);
    const float iss = 1.f / (p.scale * p.scale);
    // ---- loads.  S0 and dS1 rows of this wave's channel tiles, 16 bytes per
    // lane per 16 columns (lane (lm, lk): row 16 t + lm, columns 16 jb + 4 lk ..;
    // a 16-column tile's rows are 64 bytes apart)
    float4 s0r[TPW][NJ], d1r[TPW][NJ];
    const float* S0p = p.ckS + ((size_t)ps * H + h) * DK * dv;
    // (16-column tiles past dv fall outside the resource and read as zero)
    auto load_tile = [&](float4 (&dst)[TPW][NJ], const float* src) __attribute__((always_inline)) {
        const auto rs = buf_rsrc(src, nj * DK * TV * 4);
        const int vo = ((16 * wave + lm) * TV + 4 * lk) * 4;
#pragma unroll
        for (int x = 0; x < TPW; ++x) {
#pragma unroll
            for (int jb = 0; jb < NJ; ++jb) {
                const uint32_t __attribute__((ext_vector_type(4))) u =
                    __builtin_amdgcn_raw_buffer_load_b128(rs, vo + ((jb * DK + 16 * NW * x) * TV) * 4, 0, 0);
                dst[x][jb] = make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z),
                                         __uint_as_float(u.w));
            }
        }
    };
    load_tile(s0r, S0p);
    load_tile(d1r, p.ckdS + ((size_t)ps * H + h) * DK * dv);
    // ---- one chunk: its inputs (S0, dS1 in s0r, d1r), its gradients
    auto run_chunk = [&](const int c) __attribute__((always_inline)) {
        const int slot = offn + c;
        const int c0 = t0 + c * BC, nr = min(BC, t1 - c0);
        // the chunk's inputs through buffer resources over its rows: rows past
        // the chunk's end read as zero.  q, k and the gate: element
        // e = tid + m BT, row e / DK, channel e % DK
        const int qs = H * DK, ks = Hkv * DK;   // row strides (elements)
        constexpr int SQ = (int)sizeof(Tin);
        const char* qsrc = reinterpret_cast<const char*>(static_cast<const Tin*>(p.q) + ((size_t)c0 * H + h) * DK);
        const char* ksrc = reinterpret_cast<const char*>(static_cast<const Tin*>(p.k) + ((size_t)c0 * Hkv + hk) * DK);
        const char* gsrc = EJK ? nullptr : reinterpret_cast<const char*>(p.g + ((size_t)c0 * H + h) * DK);
        Tin xq[NE], xk[NE];
        float xg[EJK ? 1 : NE];
        {
            // step m covers rows from m BT / DK on; the lane's row within the
            // step is tid / DK
            const int r0 = tid / DK, i = tid % DK;
#pragma unroll
            for (int m = 0; m < NE; ++m) {
                const int rm = m * (BT / DK);
                xq[m] = buf_load<Tin>(rows_rsrc(qsrc, rm, nr, qs * SQ, DK * SQ), (r0 * qs + i) * SQ);
                xk[m] = buf_load<Tin>(rows_rsrc(ksrc, rm, nr, ks * SQ, DK * SQ), (r0 * ks + i) * SQ);
                if (!EJK) xg[m] = buf_load<float>(rows_rsrc(gsrc, rm, nr, qs * 4, DK * 4), (r0 * qs + i) * 4);
            }
        }
        // dt_bias through a resource that is empty without one: loads on one
        // path only would make the compiler's later waits drain every load in flight
        const auto rdt = buf_rsrc(EJK ? nullptr : p.dt_bias, (!EJK && p.dt_bias) ? (uint32_t)(DK * H * 4) : 0u);
        const float dtb_row = buf_load<float>(rdt, (uint32_t)(((tid % DK) * H + h) * 4));
        // dO (raw bits), U, Z, Y: element e = tid + m BT, row e / MAXD, column
        // e % MAXD (columns past dv are read, then replaced by zero)
        uint32_t xo[NV];
        float xu[NV], xz[NV], xy[NV];
        {
            const int os = H * dv, so = p.do_bf16 ? 2 : 4;
            const auto bo = buf_rsrc(static_cast<const char*>(p.d_o) + ((size_t)c0 * H + h) * dv * so,
                                  ((nr - 1) * os + dv) * so);
            const auto by = buf_rsrc(p.ckYU + ((size_t)slot * H + h) * 2 * BC * dv, 2 * BC * dv * 4);
            const auto bz = buf_rsrc(p.ckZ + ((size_t)slot * H + h) * BC * dv, BC * dv * 4);
            const int r0 = tid / MAXD, j = tid % MAXD;
            const bool ok = j < dv;
            // dO kept as loaded (bf16 bits or float32 bits), widened where used
            if (p.do_bf16) {
#pragma unroll
                for (int m = 0; m < NV; ++m)
                    xo[m] = buf_load<uint16_t>(bo, ((r0 + m * (BT / MAXD)) * os + j) * 2);
            } else {
#pragma unroll
                for (int m = 0; m < NV; ++m)
                    xo[m] = buf_load<uint32_t>(bo, ((r0 + m * (BT / MAXD)) * os + j) * 4);
            }
#pragma unroll
            for (int m = 0; m < NV; ++m) {
                const int r = r0 + m * (BT / MAXD);
                const float y = buf_load<float>(by, (r * dv + j) * 4);
                const float u = buf_load<float>(by, ((BC + r) * dv + j) * 4);
                const float z = buf_load<float>(bz, (r * dv + j) * 4);
                xy[m] = ok ? y : 0.f;
                xu[m] = ok ? u : 0.f;
                xz[m] = ok ? z : 0.f;
            }
        }
        // beta and the EJK decay of row tid % BC (used by lanes tid < BC): rows
        // past the chunk read zero
        const float xb = buf_load<float>(rows_rsrc(p.beta + (size_t)c0 * H + h, 0, nr, H * 4, 4), (tid % BC) * H * 4);
        float xgs = 0.f;
        if constexpr (EJK)
            xgs = buf_load<float>(rows_rsrc(p.g ? p.g + (size_t)c0 * H + h : nullptr, 0, p.g ? nr : 0, H * 4, 4),
                                  (tid % BC) * H * 4);
        // KDA: the gate and dt_bias of the elements this lane owns in the MFMA
        // layout (row 4 lk + e, channel 16 t + lm)
        float gl[TPW][4], dtl[TPW];
#pragma unroll
        for (int x = 0; x < TPW; ++x) {
            const int t = wave + NW * x;
            const bool ok = !EJK && t < NT;
            dtl[x] = buf_load<float>(rdt, (uint32_t)(((16 * t + lm) * H + h) * 4));   // channels past dk: zero
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // rows from e on; the lane's row 4 lk + e is 4 lk past the first
                const float v = EJK ? 0.f : buf_load<float>(rows_rsrc(gsrc, e, nr, qs * 4, DK * 4), (4 * lk * qs + 16 * t + lm) * 4);
                gl[x][e] = ok ? v : 0.f;
            }
        }
        // ---- to LDS: the raw rows, gate activations (log2 units), beta; dO, U, Z
        {
            const float lb2 = p.lb * kLog2e;
#pragma unroll
            for (int m = 0; m < NE; ++m) {
                const int e = tid + m * BT;
                const int r = e / DK, i = e % DK;
                const bool ok = r < nr;
                L.qh[r][i] = ok ? widen(xq[m]) : 0.f;
                L.kh[r][i] = ok ? widen(xk[m]) : 0.f;
                if (!EJK) L.eb[r][i] = ok ? lb2 * sigmoid_fast(ea * (xg[m] + dtb_row)) : 0.f;
            }
            if (tid < BC) {
                const bool ok = tid < nr;
                L.beta[tid] = ok ? (EJK ? xb : sigmoid_fast(xb)) : 0.f;
                if (EJK) L.sb[tid] = ok ? xgs * kLog2e : 0.f;
            }
#pragma unroll
            for (int m = 0; m < NV; ++m) {
                const int e = tid + m * BT;
                const int r = e / MAXD, j = e % MAXD;
                dO[r][j] = j < dv ? __uint_as_float(p.do_bf16 ? xo[m] << 16 : xo[m]) : 0.f;
                U[r][j] = xu[m];
                Z[r][j] = xz[m];
                // Z.Y of row r: a partial per wave (each wave covers half a row)
                const float zy = wave_sum(xz[m] * xy[m]);
                if (lane == 0) zyw[wave][m] = zy;
            }
        }
        setup_rest<DK, EJK>(L, p);
        // (c) over the columns: wave 0 dA = -strict_lower(Z U^T), wave 1 dP =
        // lower(dO U^T); the Gram-product gradients MA = diag(beta) dA, MP = dP
        // (EJK: times the decay factors).  Lane (lm, lk) supplies row lm of both
        // operands at columns 16 jb + 4 lk + u.
        if (wave < 2) {
            const float (*A)[SR] = wave == 1 ? dO : Z;
            bf32x4_t m = bf32x4_t{0.f, 0.f, 0.f, 0.f};
            for (int jb = 0; jb < nj; ++jb) {
                const float4 a = *reinterpret_cast<const float4*>(&A[lm][16 * jb + 4 * lk]);
                const float4 b = *reinterpret_cast<const float4*>(&U[lm][16 * jb + 4 * lk]);
                m = bmfma4(a.x, b.x, m);
                m = bmfma4(a.y, b.y, m);
                m = bmfma4(a.z, b.z, m);
                m = bmfma4(a.w, b.w, m);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * lk + e, s = lm;
                if (wave == 0) {
                    const float da = s < r ? -m[e] : 0.f;
                    dA[r][s] = da;
                    MA[r][s] = EJK ? L.beta[r] * da * L.DA[r][s] : L.beta[r] * da;
                } else {
                    const float b = s <= r ? m[e] : 0.f;
                    MP[r][s] = EJK ? b * L.DP[r][s] : b;
                }
            }
        }
        // (d1) dQg = dO S0^T, dKg = -dY S0^T and dKc = U dS1^T, a 16-channel tile
        // per step: lane (lm, lk) supplies dO[lm][j], dY[lm][j], U[lm][j] and
        // S0[i][j], dS1[i][j] (i = 16 t + lm, j = 16 jb + 4 lk + u at step u) and
        // holds rows 4 lk + e of channel i.  The same S0, dS1 elements give
        // dbc_i = e^{b_C,i} sum_j S0_ij dS1_ij.
        bf32x4_t aq[TPW], ag[TPW], ac[TPW];
        float dbcv[TPW];
#pragma unroll
        for (int x = 0; x < TPW; ++x) {
            const int t = wave + NW * x;
            aq[x] = bf32x4_t{0.f, 0.f, 0.f, 0.f};
            ag[x] = aq[x];
            ac[x] = aq[x];
            dbcv[x] = 0.f;
            if (t < NT) {
                float sdot = 0.f;
                const float nb = -L.beta[lm];
#pragma unroll
                for (int jb = 0; jb < NJ; ++jb) {
                    if (jb < nj) {
                        const float4 s4 = s0r[x][jb], d4 = d1r[x][jb];
                        const float4 o4 = *reinterpret_cast<const float4*>(&dO[lm][16 * jb + 4 * lk]);
                        const float4 z4 = *reinterpret_cast<const float4*>(&Z[lm][16 * jb + 4 * lk]);
                        const float4 u4 = *reinterpret_cast<const float4*>(&U[lm][16 * jb + 4 * lk]);
                        aq[x] = bmfma4(o4.x, s4.x, aq[x]);
                        aq[x] = bmfma4(o4.y, s4.y, aq[x]);
                        aq[x] = bmfma4(o4.z, s4.z, aq[x]);
                        aq[x] = bmfma4(o4.w, s4.w, aq[x]);
                        ag[x] = bmfma4(nb * z4.x, s4.x, ag[x]);
                        ag[x] = bmfma4(nb * z4.y, s4.y, ag[x]);
                        ag[x] = bmfma4(nb * z4.z, s4.z, ag[x]);
                        ag[x] = bmfma4(nb * z4.w, s4.w, ag[x]);
                        ac[x] = bmfma4(u4.x, d4.x, ac[x]);
                        ac[x] = bmfma4(u4.y, d4.y, ac[x]);
                        ac[x] = bmfma4(u4.z, d4.z, ac[x]);
                        ac[x] = bmfma4(u4.w, d4.w, ac[x]);
                        sdot = fmaf(s4.x, d4.x, sdot);
                        sdot = fmaf(s4.y, d4.y, sdot);
                        sdot = fmaf(s4.z, d4.z, sdot);
                        sdot = fmaf(s4.w, d4.w, sdot);
                    }
                }
                // sum over the four lane groups (lanes lm, lm + 16, lm + 32, lm + 48)
                sdot = xor_add<16>(sdot);
                sdot = xor_add<32>(sdot);
                dbcv[x] = L.ecc(16 * t + lm) * sdot;
            }
        }
        lds_barrier();
        if (tid < BC) {
            const int r = tid;
            // rows 2 m + half were covered by waves 2 half and 2 half + 1
            const int m = r >> 1, w0 = 2 * (r & 1);
            float acc = zyw[w0][m] + zyw[w0 + 1][m];
            for (int s = 0; s < r; ++s) acc = fmaf(dA[r][s], L.GA[r][s], acc);
            dbt[r] = acc;
        }
        // (d2) the Gram roles on MFMA, per 16-channel tile: D[r][i] = sum_s M[r][s]
        // X[s][i] with the lane supplying M[lm][s] (or M[s][lm] for M^T) and
        // X[s][16 t + lm] for s = 4 lk + u at step u.  The pair terms whose row and
        // column roles fall on the same b (the diagonal of P, and for EJK the first
        // sub-diagonal of A) are kept apart: they enter dqh and dkh but cancel
        // exactly in dgamma, so they are left out of db.  Then the row gradients
        // dqh, dkh, db, db' and Kc dKc of the lane's elements.
        float dqh[TPW][4], dkh[TPW][4], gb[TPW][4], gp[TPW][4], kd[TPW][4];
#pragma unroll
        for (int x = 0; x < TPW; ++x) {
            const int t = wave + NW * x;
#pragma unroll
            for (int e = 0; e < 4; ++e) dqh[x][e] = dkh[x][e] = gb[x][e] = gp[x][e] = kd[x][e] = 0.f;
            if (t < NT) {
                const int i = 16 * t + lm;
                bf32x4_t R1 = bf32x4_t{0.f, 0.f, 0.f, 0.f}, R2 = R1, R3 = R1, R4 = R1;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int s = 4 * lk + u;
                    float a1 = MA[lm][s], a2 = MA[s][lm];
                    const float a3 = s != lm ? MP[lm][s] : 0.f, a4 = s != lm ? MP[s][lm] : 0.f;
                    if (EJK) {
                        if (s + 1 == lm) a1 = 0.f;
                        if (lm + 1 == s) a2 = 0.f;
                    }
                    const float khs = L.kh[s][i], qhs = L.qh[s][i];
                    float b1, b2, b4;
                    if (EJK) {
                        b1 = khs;
                        b2 = khs;
                        b4 = qhs;
                    } else {
                        const float eb = L.eb[s][i];
                        b1 = khs * L.ein[s][i];
                        b2 = khs * eb;
                        b4 = qhs * eb;
                    }
                    R1 = bmfma4(a1, b1, R1);   // rowA (before the row factor)
                    R2 = bmfma4(a2, b2, R2);   // colA
                    R3 = bmfma4(a3, b1, R3);   // rowP
                    R4 = bmfma4(a4, b4, R4);   // colP
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * lk + e;
                    float rowA = R1[e], colA = R2[e], rowP = R3[e], colP = R4[e], subA = 0.f, subAc = 0.f;
                    if (!EJK) {
                        const float eb = L.eb[r][i], ein = L.ein[r][i];
                        rowA *= eb;
                        rowP *= eb;
                        colA *= ein;
                        colP *= ein;
                    } else {
                        subA = r > 0 ? MA[r][r - 1] * L.kh[r - 1][i] : 0.f;
                        subAc = r + 1 < BC ? MA[r + 1][r] * L.kh[r + 1][i] : 0.f;
                    }
                    const float mpd = MP[r][r];
                    const float qh = L.qh[r][i], kh = L.kh[r][i];
                    const float ebr = L.ebr(r, i), ebpr = L.ebpr(r, i), ecbr = L.ecbr(r, i);
                    const float qg = qh * ebr, kg = kh * ebpr, kc = kh * ecbr;
                    dqh[x][e] = rowP + mpd * kh + ebr * aq[x][e];
                    dkh[x][e] = rowA + subA + colA + subAc + colP + mpd * qh + ebpr * ag[x][e] + ecbr * ac[x][e];
                    const float db = qh * rowP - kh * colA - kh * colP + qg * aq[x][e];
                    const float dbp = kh * rowA + kg * ag[x][e];
                    gb[x][e] = EJK ? db : db + dbp;
                    gp[x][e] = dbp;
                    kd[x][e] = kc * ac[x][e];
                }
            }
        }
        // ---- per-row sums over the channels: a partial per lane over its tiles,
        // summed over the 16 lanes of a row group, one value per wave and row
        {
            float sq[4], sk[4], sa[4], sb2[4], sc[4], sd = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) sq[e] = sk[e] = sa[e] = sb2[e] = sc[e] = 0.f;
#pragma unroll
            for (int x = 0; x < TPW; ++x) {
                const int t = wave + NW * x;
                if (t < NT) {
                    const int i = 16 * t + lm;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 4 * lk + e;
                        sq[e] = fmaf(L.qh[r][i], dqh[x][e], sq[e]);
                        sk[e] = fmaf(L.kh[r][i], dkh[x][e], sk[e]);
                        if (EJK) {
                            sa[e] += gb[x][e];
                            sb2[e] += gp[x][e];
                            sc[e] += kd[x][e];
                        }
                    }
                    if (EJK && lk == 0) sd += dbcv[x];
                }
            }
            auto row16 = [](float v) {
                v = xor_add<1>(v);
                v = xor_add<2>(v);
                v = xor_add<4>(v);
                return xor_add<8>(v);
            };
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float q = row16(sq[e]), k = row16(sk[e]);
                if (lm == 0) {
                    rq[wave][4 * lk + e] = q;
                    rk[wave][4 * lk + e] = k;
                }
                if (EJK) {
                    const float a = row16(sa[e]), b = row16(sb2[e]), c = row16(sc[e]);
                    if (lm == 0) {
                        ra[wave][4 * lk + e] = a;
                        rb[wave][4 * lk + e] = b;
                        rc[wave][4 * lk + e] = c;
                    }
                }
            }
            if (EJK) {
                sd = row16(sd);
                if (lane == 0) rd[wave] = sd;
            }
        }
        lds_barrier();
        // ---- dgamma.  KDA, per element: the reverse cumulative sum of db down the
        // chunk, the carry's e^{b_C} term (dbc, on every row) and the Kc terms of
        // the rows before.  A channel's rows are split over the four lane groups
        // (rows 4 lk .. 4 lk + 3), joined through the group totals.
        // EJK, per row: the same over the per-row sums, in one lane.
        float dgm[TPW][4];
        if (!EJK) {
#pragma unroll
            for (int x = 0; x < TPW; ++x) {
                float G = 0.f, K = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    G += gb[x][e];
                    K += kd[x][e];
                }
                float sufG = 0.f, preK = 0.f;
#pragma unroll
                for (int l = 0; l < 4; ++l) {
                    const float g2 = __shfl(G, lm + 16 * l);
                    const float k2 = __shfl(K, lm + 16 * l);
                    if (l > lk) sufG += g2;
                    if (l < lk) preK += k2;
                }
                float run = dbcv[x] + sufG;
                float pre[4];
                float acc = preK;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    pre[e] = acc;
                    acc += kd[x][e];
                }
#pragma unroll
                for (int e = 3; e >= 0; --e) {
                    run += gb[x][e];
                    dgm[x][e] = run + pre[e];
                }
            }
        } else {
#pragma unroll
            for (int x = 0; x < TPW; ++x)
#pragma unroll
                for (int e = 0; e < 4; ++e) dgm[x][e] = 0.f;
            if (tid == 0) {
                float A[BC], B[BC], C[BC];
                for (int r = 0; r < BC; ++r) {
                    A[r] = (ra[0][r] + ra[1][r]) + (ra[2][r] + ra[3][r]);
                    B[r] = (rb[0][r] + rb[1][r]) + (rb[2][r] + rb[3][r]);
                    C[r] = (rc[0][r] + rc[1][r]) + (rc[2][r] + rc[3][r]);
                }
                float pre[BC];
                float acc = 0.f;
                for (int r = 0; r < BC; ++r) {
                    pre[r] = acc;
                    acc += C[r];
                }
                float run = (rd[0] + rd[1]) + (rd[2] + rd[3]);
                for (int r = BC - 1; r >= 0; --r) {
                    run += A[r] + (r + 1 < BC ? B[r + 1] : 0.f);
                    dgs[r] = run + pre[r];
                }
            }
            lds_barrier();
        }
        // ---- the prologue's backward and the stores, through buffer resources
        // over the chunk's rows (rows past its end are dropped)
        const int hs = grouped ? H : Hkv, hh = grouped ? h : hk;
        const char* dqdst = reinterpret_cast<const char*>(p.dq + ((size_t)c0 * H + h) * DK);
        const char* dkdst = reinterpret_cast<const char*>(p.dk + ((size_t)c0 * hs + hh) * DK);
        const char* dgdst = EJK ? nullptr : reinterpret_cast<const char*>(p.dg + ((size_t)c0 * H + h) * DK);
        float apart = 0.f;
#pragma unroll
        for (int x = 0; x < TPW; ++x) {
            const int t = wave + NW * x;
            float pdt = 0.f;
            if (t < NT) {
                const int i = 16 * t + lm;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * lk + e;
                    // rows from e on; the lane's row r = 4 lk + e is 4 lk past the first
                    const uint32_t vo = (4 * lk * qs + i) * 4, vk = (4 * lk * hs * DK + i) * 4;
                    const float pq = (rq[0][r] + rq[1][r]) + (rq[2][r] + rq[3][r]);
                    const float pk = (rk[0][r] + rk[1][r]) + (rk[2][r] + rk[3][r]);
                    float dq, dk;
                    if (p.l2norm) {
                        const float inq = L.nq[r], ink = L.nk[r];
                        dq = p.scale * inq * (dqh[x][e] - L.qh[r][i] * pq * iss);
                        dk = ink * (dkh[x][e] - L.kh[r][i] * pk);
                    } else {
                        dq = p.scale * dqh[x][e];
                        dk = dkh[x][e];
                    }
                    buf_store(rows_rsrc(dqdst, e, nr, qs * 4, DK * 4), vo, dq);
                    buf_store(rows_rsrc(dkdst, e, nr, hs * DK * 4, DK * 4), vk, dk);
                    if (!EJK) {
                        const float xx = ea * (gl[x][e] + dtl[x]);
                        // sigma'(x) = sigma(x) sigma(-x): no cancellation in
                        // 1 - sigma(x) when the gate saturates; rows past the
                        // chunk add nothing to the parameter partials
                        float dx = dgm[x][e] * p.lb * sigmoid_fast(xx) * sigmoid_fast(-xx);
                        dx = r < nr ? dx : 0.f;
                        buf_store(rows_rsrc(dgdst, e, nr, qs * 4, DK * 4), vo, dx * ea);
                        apart = fmaf(dx, xx, apart);
                        pdt += dx * ea;
                    }
                }
            }
            if (!EJK) {
                // dt_bias partial of channel i: the sum over the four lane groups
                pdt = xor_add<16>(pdt);
                pdt = xor_add<32>(pdt);
                if (t < NT && lk == 0) p.part_dt[((size_t)slot * H + h) * DK + 16 * t + lm] = pdt;
            }
        }
        {
            // dv = beta Z, per step m over rows from 2 m on; columns past dv get an
            // offset past the resource
            const char* dvb = reinterpret_cast<const char*>(p.dv_out + ((size_t)c0 * hs + hh) * dv);
            const int r0 = tid / MAXD, j = tid % MAXD;
            const uint32_t vo = j < dv ? (uint32_t)(r0 * hs * dv + j) * 4 : kNoOffset;
#pragma unroll
            for (int m = 0; m < NV; ++m) {
                const int rm = m * (BT / MAXD);
                buf_store(rows_rsrc(dvb, rm, nr, hs * dv * 4, dv * 4), vo, L.beta[r0 + rm] * xz[m]);
            }
        }
        if (tid < BC && tid < nr) {
            const int r = tid;
            const size_t tok = (size_t)(c0 + r);
            if (EJK) {
                p.dbeta[tok * H + h] = dbt[r];
                if (p.dg) p.dg[tok * H + h] = dgs[r];
            } else {
                p.dbeta[tok * H + h] = dbt[r] * sigmoid_fast(xb) * sigmoid_fast(-xb);
            }
        }
        if (!EJK) {
            apart = wave_sum(apart);
            if (lane == 0) red[wave] = apart;
            lds_barrier();
            if (tid == 0) p.part_a[(size_t)slot * H + h] = (red[0] + red[1]) + (red[2] + red[3]);
        }
    };
    if (has_b) {
        // S entering the second chunk: one forward step through the first
        // (its U from pass 1, its Kc and e^{b_C} from its operand block), in
        // the layout of s0r: D[j][i] = sum_r U[r][j] Kc[r][i] with the lane
        // supplying U[4 lk + u][16 jb + lm] and Kc[4 lk + u][16 t + lm]
        {
            using PL = PrepLayout<DK>;
            const int sa = offn + ca;
            const float* yu = p.ckYU + ((size_t)sa * H + h) * 2 * BC * dv;
            const float* pb = p.prep + ((size_t)sa * H + h) * PL::SIZE;
            for (int e = tid; e < BC * MAXD; e += BT) {
                const int r = e / MAXD, j = e % MAXD;
                U[r][j] = j < dv ? yu[(size_t)(BC + r) * dv + j] : 0.f;
                Z[r][j] = j < DK ? (EJK ? pb[PL::KG + r * PL::RS + j] * pb[PL::RF + 2 * BC + r]
                                        : pb[PL::KC + r * PL::RS + j])
                                 : 0.f;
            }
            if (tid < DK) L.ec[tid] = EJK ? pb[PL::RF + 3 * BC] : pb[PL::EC + tid];
            lds_barrier();
#pragma unroll
            for (int x = 0; x < TPW; ++x) {
                const int t = wave + NW * x;
                if (t < NT) {
                    const float ec = L.ec[16 * t + lm];
#pragma unroll
                    for (int jb = 0; jb < NJ; ++jb) {
                        if (jb < nj) {
                            bf32x4_t a = bf32x4_t{ec * s0r[x][jb].x, ec * s0r[x][jb].y, ec * s0r[x][jb].z,
                                                  ec * s0r[x][jb].w};
#pragma unroll
                            for (int u = 0; u < 4; ++u)
                                a = bmfma4(U[4 * lk + u][16 * jb + lm], Z[4 * lk + u][16 * t + lm], a);
                            s0r[x][jb] = make_float4(a[0], a[1], a[2], a[3]);
                        }
                    }
                }
            }
            lds_barrier();
        }
        run_chunk(ca + 1);
        // dS leaving the first chunk: one backward step through the second,
        // from its set-up, dO and Z still in LDS
#pragma unroll
        for (int x = 0; x < TPW; ++x) {
            const int t = wave + NW * x;
            if (t < NT) {
                const int i = 16 * t + lm;
                const float ec = L.ecc(i);
#pragma unroll
                for (int jb = 0; jb < NJ; ++jb) {
                    if (jb < nj) {
                        bf32x4_t a = bf32x4_t{ec * d1r[x][jb].x, ec * d1r[x][jb].y, ec * d1r[x][jb].z,
                                              ec * d1r[x][jb].w};
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            const int r = 4 * lk + u;
                            a = bmfma4(dO[r][16 * jb + lm], L.qg(r, i), a);
                            a = bmfma4(-L.beta[r] * Z[r][16 * jb + lm], L.kg(r, i), a);
                        }
                        d1r[x][jb] = make_float4(a[0], a[1], a[2], a[3]);
                    }
                }
            }
        }
        load_tile(s0r, S0p);
        lds_barrier();
    }
    run_chunk(ca);

}

// Parameter gradients summed over chunks (fixed order), and key/value
// gradients summed over the heads of a group.
__global__ __launch_bounds__(256) void bwd_param_kernel(const float* __restrict__ part_a,
                                                        const float* __restrict__ part_dt,
                                                        const int32_t* __restrict__ off, int N, int H, int dk,
                                                        float* __restrict__ da_log, float* __restrict__ ddt_bias)
{
    // a workgroup per (32 channels, head): eight lanes per channel take every
    // eighth chunk, then a fixed-order sum (the result does not depend on timing)
    __shared__ float red[8][33];
    __shared__ float ra[256];
    const int slots = off[N];
    const int tid = threadIdx.x, h = blockIdx.y;
    const int i = blockIdx.x * 32 + (tid & 31), grp = tid >> 5;
    float a = 0.f;
    if (ddt_bias && i < dk) {
#pragma unroll 8
        for (int s = grp; s < slots; s += 8) a += part_dt[((size_t)s * H + h) * dk + i];
    }
    red[grp][tid & 31] = a;
    const bool do_a = da_log && blockIdx.x == 0;
    float b = 0.f;
    if (do_a) {
#pragma unroll 4
        for (int s = tid; s < slots; s += 256) b += part_a[(size_t)s * H + h];
    }
    ra[tid] = b;
    lds_barrier();
    if (tid < 32 && ddt_bias && i < dk) {
        float t = 0.f;
#pragma unroll
        for (int g2 = 0; g2 < 8; ++g2) t += red[g2][tid];
        ddt_bias[(size_t)i * H + h] = t;
    }
    if (do_a) {
        for (int w = 128; w > 0; w >>= 1) {
            if (tid < w) ra[tid] += ra[tid + w];
            lds_barrier();
        }
        if (tid == 0) da_log[h] = ra[0];
    }
}

__global__ void bwd_group_sum_kernel(const float* __restrict__ src, size_t ntok, int H, int Hkv, int d,
                                     float* __restrict__ dst)
{
    const size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= ntok * Hkv * d) return;
    const int i = (int)(e % d);
    const size_t th = e / d;
    const int hv = (int)(th % Hkv);
    const size_t t = th / Hkv;
    const int G = H / Hkv;
    float a = 0.f;
    for (int r = 0; r < G; ++r) a += src[(t * H + (size_t)hv * G + r) * d + i];
    dst[e] = a;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

size_t bwd_slots(int N, int T, bool packed)
{
    if (packed) return (size_t)(T / BC) + (size_t)N;
    return (size_t)N * (size_t)((T + BC - 1) / BC);
}

size_t prep_floats(int dk)
{
    switch (dk) {
    case 16: return PrepLayout<16>::SIZE;
    case 32: return PrepLayout<32>::SIZE;
    case 64: return PrepLayout<64>::SIZE;
    default: return PrepLayout<128>::SIZE;
    }
}

template <int DK, bool EJK>
hipError_t launch_dk(const BwdParams& p, size_t slots, hipStream_t st)
{
    const dim3 lgrid((unsigned)slots, (unsigned)p.H);
    hipError_t e = hipSuccess;
    if (slots > 0) {
        if (p.in_bf16) hipLaunchKernelGGL((bwd_prep<DK, EJK, uint16_t>), lgrid, dim3(BT), 0, st, p);
        else hipLaunchKernelGGL((bwd_prep<DK, EJK, float>), lgrid, dim3(BT), 0, st, p);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // scan ids: (head, sequence) groups padded to a multiple of 8, times the
    // column tiles; the scans also run for sequences without rows (the reverse
    // one then passes dL/d(final state) on as dL/d(initial state))
    const unsigned groups8 = (unsigned)((p.H * p.N + 7) / 8 * 8);
    if (groups8 == 0) return hipSuccess;
    // Two 16-column tiles per workgroup (one load of each operand block for
    // both) once that still gives every CU a workgroup; else one, for twice
    // the workgroups
    if (p.dv >= 2 * TV && (size_t)p.H * p.N * (p.dv / (2 * TV)) >= kCUs) {
        const dim3 sgrid(groups8 * (unsigned)(p.dv / (2 * TV)));
        if (p.in_bf16) hipLaunchKernelGGL((bwd_fwd_scan<DK, EJK, uint16_t, 2>), sgrid, dim3(2 * BT), 0, st, p);
        else hipLaunchKernelGGL((bwd_fwd_scan<DK, EJK, float, 2>), sgrid, dim3(2 * BT), 0, st, p);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (p.in_bf16) hipLaunchKernelGGL((bwd_rev_scan<DK, EJK, uint16_t, 2>), sgrid, dim3(2 * BT), 0, st, p);
        else hipLaunchKernelGGL((bwd_rev_scan<DK, EJK, float, 2>), sgrid, dim3(2 * BT), 0, st, p);
    } else {
        const dim3 sgrid(groups8 * (unsigned)(p.dv / TV));
        if (p.in_bf16) hipLaunchKernelGGL((bwd_fwd_scan<DK, EJK, uint16_t, 1>), sgrid, dim3(BT), 0, st, p);
        else hipLaunchKernelGGL((bwd_fwd_scan<DK, EJK, float, 1>), sgrid, dim3(BT), 0, st, p);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (p.in_bf16) hipLaunchKernelGGL((bwd_rev_scan<DK, EJK, uint16_t, 1>), sgrid, dim3(BT), 0, st, p);
        else hipLaunchKernelGGL((bwd_rev_scan<DK, EJK, float, 1>), sgrid, dim3(BT), 0, st, p);
    }
    e = hipGetLastError();
    if (e != hipSuccess || slots == 0) return e;
    const dim3 pgrid((unsigned)((slots + (size_t)p.N + 1) / 2), (unsigned)p.H);
    if (p.in_bf16) hipLaunchKernelGGL((bwd_local<DK, EJK, uint16_t>), pgrid, dim3(BT), 0, st, p);
    else hipLaunchKernelGGL((bwd_local<DK, EJK, float>), pgrid, dim3(BT), 0, st, p);
    return hipGetLastError();
}

template <int DK, bool EJK>
hipError_t launch16_dk(const BwdParams& p, size_t slots, hipStream_t st)
{
    const dim3 lgrid((unsigned)slots, (unsigned)p.H);
    if (slots > 0) {
        if (p.in_bf16) hipLaunchKernelGGL((bwd_prep<DK, EJK, uint16_t>), lgrid, dim3(BT), 0, st, p);
        else hipLaunchKernelGGL((bwd_prep<DK, EJK, float>), lgrid, dim3(BT), 0, st, p);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // every (head, sequence) group runs, those without rows too (they carry
    // the initial state to the final one); tiles as for the backward's scans
    const unsigned groups8 = (unsigned)((p.H * p.N + 7) / 8 * 8);
    if (groups8 == 0) return hipSuccess;
    const bool two = p.dv >= 2 * TV && (size_t)p.H * p.N * (p.dv / (2 * TV)) >= kCUs;
    const dim3 sgrid(groups8 * (unsigned)(p.dv / (two ? 2 * TV : TV)));
    const dim3 blk(two ? 2 * BT : BT);
    if (two) {
        if (!p.in_bf16) hipLaunchKernelGGL((prefill16_scan<DK, EJK, float, float, 2>), sgrid, blk, 0, st, p);
        else if (p.out_bf16) hipLaunchKernelGGL((prefill16_scan<DK, EJK, uint16_t, bf16_t, 2>), sgrid, blk, 0, st, p);
        else hipLaunchKernelGGL((prefill16_scan<DK, EJK, uint16_t, float, 2>), sgrid, blk, 0, st, p);
    } else {
        if (!p.in_bf16) hipLaunchKernelGGL((prefill16_scan<DK, EJK, float, float, 1>), sgrid, blk, 0, st, p);
        else if (p.out_bf16) hipLaunchKernelGGL((prefill16_scan<DK, EJK, uint16_t, bf16_t, 1>), sgrid, blk, 0, st, p);
        else hipLaunchKernelGGL((prefill16_scan<DK, EJK, uint16_t, float, 1>), sgrid, blk, 0, st, p);
    }
    return hipGetLastError();
}

}  // namespace

bool prefill16_preferred(int N, int H, int dk)
{
    // Narrow calls (H dk < 128: fp32 B1 T64 H2 d16 runs in 8.4 us as the one
    // kernel against 12 us as two) stay on the one kernel.  The rule depends on
    // neither the token count nor the packing, so that packed sequences and
    // splits take the route of the sequences run alone.  (Head, sequence)
    // groups as the backward's scans allow.
    return N > 0 && (long long)H * N <= (1LL << 26) && H * dk >= 128;
}

size_t prefill16_workspace_bytes(int N, int T, int H, int dk, bool packed)
{
    if (N <= 0 || T <= 0) return 0;
    const size_t slots = bwd_slots(N, T, packed);
    return 2 * align256((size_t)(N + 1) * 4) + align256(slots * H * prep_floats(dk) * 4);
}

hipError_t launch_prefill16(const PrefillArgs& a, hipStream_t st)
{
    const bool packed = a.cu != nullptr;
    const size_t slots = bwd_slots(a.N, a.T, packed);
    unsigned char* w = static_cast<unsigned char*>(a.workspace);
    BwdParams p{};
    p.q = a.q; p.k = a.k; p.v = a.v; p.in_bf16 = a.in_bf16;
    p.g = a.g; p.beta = a.beta; p.a_log = a.a_log; p.dt_bias = a.dt_bias;
    p.init = a.init; p.cu = a.cu;
    p.N = a.N; p.T = a.T; p.H = a.H; p.Hkv = a.Hkv; p.dv = a.dv;
    p.scale = a.scale; p.lb = a.lower_bound; p.l2norm = a.l2norm;
    p.out = a.o; p.out_bf16 = a.out_bf16; p.fstate = a.final_state;
    const size_t pslots = (slots + (size_t)a.N + 1) / 2;
    int32_t* off = reinterpret_cast<int32_t*>(w);
    w += align256((size_t)(a.N + 1) * 4);
    int32_t* poff = reinterpret_cast<int32_t*>(w);
    w += align256((size_t)(a.N + 1) * 4);
    p.off = off;
    p.poff = poff;
    p.prep = reinterpret_cast<float*>(w);
    hipLaunchKernelGGL(bwd_plan_kernel, dim3(1), dim3(64), 0, st, a.cu, a.N, a.T, (int)slots, (int)pslots, off,
                       poff);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    switch (a.dk * 2 + (a.ejk ? 1 : 0)) {
    case 32: return launch16_dk<16, false>(p, slots, st);
    case 33: return launch16_dk<16, true>(p, slots, st);
    case 64: return launch16_dk<32, false>(p, slots, st);
    case 65: return launch16_dk<32, true>(p, slots, st);
    case 128: return launch16_dk<64, false>(p, slots, st);
    case 129: return launch16_dk<64, true>(p, slots, st);
    case 256: return launch16_dk<128, false>(p, slots, st);
    default: return launch16_dk<128, true>(p, slots, st);
    }
}

size_t backward_workspace_bytes(int N, int T, int H, int Hkv, int dk, int dv, bool packed)
{
    if (N <= 0 || T <= 0) return align256((size_t)(N + 1) * 4);
    const size_t slots = bwd_slots(N, T, packed);
    const size_t ntok = packed ? (size_t)T : (size_t)N * T;
    size_t b = align256((size_t)(N + 1) * 4);
    const size_t pslots = (slots + (size_t)N + 1) / 2;
    b += align256((size_t)(N + 1) * 4);
    b += 2 * align256(pslots * H * dk * dv * 4);
    b += align256(slots * H * 2 * BC * dv * 4) + align256(slots * H * BC * dv * 4);
    b += align256(slots * H * prep_floats(dk) * 4);
    b += align256(slots * H * 4) + align256(slots * H * dk * 4);
    if (Hkv != H) b += align256(ntok * H * dk * 4) + align256(ntok * H * dv * 4);
    return b;
}

hipError_t launch_backward(const BackwardArgs& a, hipStream_t st)
{
    const bool packed = a.cu != nullptr;
    const size_t slots = bwd_slots(a.N, a.T, packed);
    const size_t ntok = packed ? (size_t)a.T : (size_t)a.N * a.T;
    unsigned char* w = static_cast<unsigned char*>(a.workspace);
    BwdParams p{};
    p.q = a.q; p.k = a.k; p.v = a.v; p.in_bf16 = a.in_bf16;
    p.g = a.g; p.beta = a.beta; p.a_log = a.a_log; p.dt_bias = a.dt_bias;
    p.init = a.init; p.cu = a.cu;
    p.N = a.N; p.T = a.T; p.H = a.H; p.Hkv = a.Hkv; p.dv = a.dv;
    p.scale = a.scale; p.lb = a.lower_bound; p.l2norm = a.l2norm;
    p.d_o = a.d_o; p.do_bf16 = a.do_bf16; p.dSf = a.d_final_state;
    p.dq = a.dq; p.dg = a.dg; p.dbeta = a.dbeta; p.dS0 = a.d_initial_state;
    const size_t pslots = (slots + (size_t)a.N + 1) / 2;
    int32_t* off = reinterpret_cast<int32_t*>(w);
    w += align256((size_t)(a.N + 1) * 4);
    int32_t* poff = reinterpret_cast<int32_t*>(w);
    w += align256((size_t)(a.N + 1) * 4);
    p.off = off;
    p.poff = poff;
    p.ckS = reinterpret_cast<float*>(w);
    w += align256(pslots * a.H * a.dk * a.dv * 4);
    p.ckdS = reinterpret_cast<float*>(w);
    w += align256(pslots * a.H * a.dk * a.dv * 4);
    p.ckYU = reinterpret_cast<float*>(w);
    w += align256(slots * a.H * 2 * BC * a.dv * 4);
    p.ckZ = reinterpret_cast<float*>(w);
    w += align256(slots * a.H * BC * a.dv * 4);
    p.prep = reinterpret_cast<float*>(w);
    w += align256(slots * a.H * prep_floats(a.dk) * 4);
    p.part_a = reinterpret_cast<float*>(w);
    w += align256(slots * a.H * 4);
    p.part_dt = reinterpret_cast<float*>(w);
    w += align256(slots * a.H * a.dk * 4);
    const bool grouped = a.Hkv != a.H;
    float* dkq = nullptr;
    float* dvq = nullptr;
    if (grouped) {
        dkq = reinterpret_cast<float*>(w);
        w += align256(ntok * a.H * a.dk * 4);
        dvq = reinterpret_cast<float*>(w);
    }
    p.dk = grouped ? dkq : a.dk_out;
    p.dv_out = grouped ? dvq : a.dv_out;
    hipLaunchKernelGGL(bwd_plan_kernel, dim3(1), dim3(64), 0, st, a.cu, a.N, a.T, (int)slots, (int)pslots, off,
                       poff);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    switch (a.dk * 2 + (a.ejk ? 1 : 0)) {
    case 32: e = launch_dk<16, false>(p, slots, st); break;
    case 33: e = launch_dk<16, true>(p, slots, st); break;
    case 64: e = launch_dk<32, false>(p, slots, st); break;
    case 65: e = launch_dk<32, true>(p, slots, st); break;
    case 128: e = launch_dk<64, false>(p, slots, st); break;
    case 129: e = launch_dk<64, true>(p, slots, st); break;
    case 256: e = launch_dk<128, false>(p, slots, st); break;
    default: e = launch_dk<128, true>(p, slots, st); break;
    }
    if (e != hipSuccess) return e;
    if (!a.ejk && (a.da_log || a.ddt_bias)) {
        hipLaunchKernelGGL(bwd_param_kernel, dim3((unsigned)((a.dk + 31) / 32), (unsigned)a.H), dim3(256), 0, st, p.part_a,
                           p.part_dt, off, a.N, a.H, a.dk, a.da_log, a.ddt_bias);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (grouped && ntok > 0) {
        size_t n = ntok * a.Hkv * a.dk;
        hipLaunchKernelGGL(bwd_group_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, dkq, ntok,
                           a.H, a.Hkv, a.dk, a.dk_out);
        n = ntok * a.Hkv * a.dv;
        hipLaunchKernelGGL(bwd_group_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, dvq, ntok,
                           a.H, a.Hkv, a.dv, a.dv_out);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace kda
