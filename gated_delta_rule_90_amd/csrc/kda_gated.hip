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
// factors are at most 1 when the gates are at most 0.
//
// Two kernels.  gated_prep, one workgroup per (chunk, head), every chunk in
// parallel, forms what does not depend on the value columns: the read-out
// rows qt e^{bk}, the carry rows e^{bk_C - bk} k, A (16 x 16) and e^{bk_C},
// into a per-(chunk, head) block of the caller's workspace.  gated_scan, one
// workgroup per (sequence, head, 16 state columns), walks the chunks in
// order with the dk x 16 state tile in the accumulator registers of 16x16x4
// float32 MFMA: per chunk the inter-chunk read-out (each wave its tiles'
// part, summed in LDS), the intra-chunk term A (e^{bv_0 - bv} v) on MFMA with
// the value-axis factors referenced to the chunk's first row (element by
// element when a column's log-decay over the chunk leaves the factor range),
// and the state update.  The chunk's operand block is copied to one of two
// LDS buffers from registers loaded two chunks ahead; two barriers per chunk,
// for LDS only.  Rows past a sequence's end are neutral (q = k = v = 0, every
// gate 0) and their outputs are dropped by the store's buffer range.
#include <type_traits>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int GC = 16;    // chunk rows
constexpr int GJ = 16;    // state columns per scan tile (a scan workgroup takes one or two)
constexpr int GTH = 256;  // threads per workgroup
constexpr int GNW = GTH / kWave;
constexpr int kGCUs = 256;   // compute units of an MI355X

struct GatedParams {
    const void* q;
    const void* k;
    const void* v;
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
    float* final_state;
    const int32_t* off;   // [N + 1] chunk offsets
    float* prep;          // [slots, H, GPrep<dk>::SIZE]
};

// The column-independent operands of one (chunk, head), floats, rows of
// RS = dk + 4 (copied to LDS as they are; 16-byte rows 4 banks apart):
//     QE [16][RS]  qt e^{bk}             KC [16][RS]  e^{bk_C - bk} k
//     AM [16][16]  A (s <= r, else 0)    EKC [dk]     e^{bk_C}
template <int DK>
struct GPrep {
    static constexpr int RS = DK + 4;
    static constexpr int QE = 0, KC = GC * RS, AM = 2 * GC * RS, EKC = AM + GC * GC;
    static constexpr int SIZE = (EKC + DK + 63) / 64 * 64;
};

size_t gprep_floats(int dk)
{
    switch (dk) {
    case 16: return GPrep<16>::SIZE;
    case 32: return GPrep<32>::SIZE;
    case 64: return GPrep<64>::SIZE;
    default: return GPrep<128>::SIZE;
    }
}

__device__ __forceinline__ void gseq_bounds(const GatedParams& p, int n, int& t0, int& t1)
{
    if (p.cu) {
        t0 = min(max(p.cu[n], 0), p.T);
        t1 = min(max(p.cu[n + 1], t0), p.T);
    } else {
        t0 = n * p.T;
        t1 = t0 + p.T;
    }
}

// Chunk offsets: off[n] = sum_{m<n} ceil(len_m / 16), capped at the slots
// (only overlapping ranges can ask for more; their last chunks are dropped).
__global__ void gated_plan_kernel(GatedParams p, int slots, int32_t* __restrict__ off)
{
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    int acc = 0;
    for (int n = 0; n < p.N; ++n) {
        int t0, t1;
        gseq_bounds(p, n, t0, t1);
        off[n] = acc;
        acc = min(acc + (t1 - t0 + GC - 1) / GC, slots);
    }
    off[p.N] = acc;
}

template <typename T>
__device__ __forceinline__ float widen(T x)
{
    if constexpr (std::is_same_v<T, float>) return x;
    else return __uint_as_float((uint32_t)x << 16);
}

typedef float gf32x4_t __attribute__((ext_vector_type(4)));

// D += A B on a 16x16x4 float32 MFMA: lane l supplies A[l % 16][l / 16] and
// B[l / 16][l % 16] and holds D[4 (l / 16) + e][l % 16] in element e.
__device__ __forceinline__ gf32x4_t gmfma4(float a, float b, gf32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <int DK>
struct GPrepLds {
    static constexpr int RS = DK + 4;
    alignas(16) float QT[GC * RS];   // scale e^{g} q, then (in range) qt 2^{bk - bk_0}, A's left factor
    alignas(16) float KT[GC * RS];   // k, then (in range) k 2^{bk_0 - bk}, A's right factor
    alignas(16) float BK[GC * RS];   // gk + g_gamma (log2 units), then its cumulative sum bk
    int wide;
};

// One workgroup per (chunk slot, head).  Tin: uint16_t (bf16 bits) or float.
template <int DK, typename Tin>
__global__ __launch_bounds__(GTH) void gated_prep(GatedParams p)
{
    using PL = GPrep<DK>;
    constexpr int RS = PL::RS;
    constexpr int NE = GC * DK / GTH;   // row elements per thread
    static_assert(NE >= 1 && NE * GTH == GC * DK, "dk in {16, 32, 64, 128}");
    __shared__ GPrepLds<DK> L;
    const int tid = threadIdx.x;
    const int slot = blockIdx.x, h = blockIdx.y;
    const int H = p.H;
    const int hk = h / (H / p.Hkv);
    if (slot >= p.off[p.N]) return;
    int lo = 0, hi = p.N - 1;   // the last n with off[n] <= slot
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (p.off[mid] <= slot) lo = mid;
        else hi = mid - 1;
    }
    const int n = lo;
    int t0, t1;
    gseq_bounds(p, n, t0, t1);
    const int len = t1 - t0, c = slot - p.off[n];
    const int lc = min(GC, len - c * GC);
    const float lg = p.g_gamma ? p.g_gamma[(size_t)min(n, p.g_gamma_rows - 1) * H + h] : 0.f;
    const Tin* q = static_cast<const Tin*>(p.q);
    const Tin* k = static_cast<const Tin*>(p.k);
    // 1. the rows to LDS, zero past the chunk's rows; the gates in log2 units.
    // The loads go through buffer resources over the chunk's rows in memory
    // (from its lowest row: the first in processing order, or in reverse the
    // last), absent gates through empty ones that read zeros, and are all
    // issued before the first is used, so one wait covers them
    const int base = p.reverse ? t1 - c * GC - lc : t0 + c * GC;
    const int qs = H * DK, ks = p.Hkv * DK;   // row strides (elements)
    constexpr uint32_t SQ = sizeof(Tin);
    const uint32_t qbytes = ((lc - 1) * qs + DK) * 4;   // the chunk's rows of a float32 [T, H, dk] input
    const auto rq = buf_rsrc(uniform_ptr(q + ((size_t)base * H + h) * DK),
                             __builtin_amdgcn_readfirstlane(((lc - 1) * qs + DK) * SQ));
    const auto rk = buf_rsrc(uniform_ptr(k + ((size_t)base * p.Hkv + hk) * DK),
                             __builtin_amdgcn_readfirstlane(((lc - 1) * ks + DK) * SQ));
    const auto rg = buf_rsrc(p.g ? uniform_ptr(p.g + ((size_t)base * H + h) * DK) : nullptr,
                             __builtin_amdgcn_readfirstlane(p.g ? qbytes : 0u));
    const auto rgk = buf_rsrc(p.gk ? uniform_ptr(p.gk + ((size_t)base * H + h) * DK) : nullptr,
                              __builtin_amdgcn_readfirstlane(p.gk ? qbytes : 0u));
    Tin xq[NE], xk[NE];
    float xg[NE], xgk[NE];
#pragma unroll
    for (int m = 0; m < NE; ++m) {
        const int e = tid + m * GTH;
        const int r = e / DK, i = e % DK;
        // the row's place in memory from the chunk's lowest row (row 0 for the
        // padding rows, whose values are replaced below)
        const int mr = r < lc ? (p.reverse ? lc - 1 - r : r) : 0;
        xq[m] = buf_load<Tin>(rq, (mr * qs + i) * SQ);
        xk[m] = buf_load<Tin>(rk, (mr * ks + i) * SQ);
        xg[m] = buf_load<float>(rg, (mr * qs + i) * 4);
        xgk[m] = buf_load<float>(rgk, (mr * qs + i) * 4);
    }
#pragma unroll
    for (int m = 0; m < NE; ++m) {
        settle(xq[m]);
        settle(xk[m]);
        settle(xg[m]);
        settle(xgk[m]);
    }
#pragma unroll
    for (int m = 0; m < NE; ++m) {
        const int e = tid + m * GTH;
        const int r = e / DK, i = e % DK;
        const bool in = r < lc;
        L.QT[r * RS + i] = in ? p.scale * __builtin_amdgcn_exp2f(xg[m] * kLog2e) * widen(xq[m]) : 0.f;
        L.KT[r * RS + i] = in ? widen(xk[m]) : 0.f;
        L.BK[r * RS + i] = in ? (xgk[m] + lg) * kLog2e : 0.f;
    }
    if (tid == 0) L.wide = 0;
    __syncthreads();
    float* o = p.prep + ((size_t)slot * H + h) * PL::SIZE;
    // 2. per key channel: the cumulative log-decay down the rows and the range
    // test; then the read-out and carry rows (to the block) and, when every
    // channel is in range, A's factors in place of the rows.  A =
    // (qt 2^{bk - bk_0}) (k 2^{bk_0 - bk})^T when every such factor stays inside
    // float32's range (|bk_r - bk_0| <= 120 in log2 units); else A is formed
    // element by element from the rows and bk.
    float b[GC];
    float bc = 0.f;
    if (tid < DK) {
        const int i = tid;
        bool wide = false;
#pragma unroll
        for (int r = 0; r < GC; ++r) {
            bc += L.BK[r * RS + i];
            b[r] = bc;
            wide |= !(fabsf(b[r] - b[0]) <= 120.f);
        }
        if (wide) L.wide = 1;
    }
    __syncthreads();
    if (tid < DK) {
        const int i = tid;
        const bool inplace = !L.wide;
        o[PL::EKC + i] = __builtin_amdgcn_exp2f(bc);
#pragma unroll
        for (int r = 0; r < GC; ++r) {
            const float qt = L.QT[r * RS + i], kt = L.KT[r * RS + i];
            o[PL::QE + r * RS + i] = qt * __builtin_amdgcn_exp2f(b[r]);
            o[PL::KC + r * RS + i] = kt * __builtin_amdgcn_exp2f(bc - b[r]);
            if (inplace) {
                const float d = b[r] - b[0];
                L.QT[r * RS + i] = qt * __builtin_amdgcn_exp2f(d);
                L.KT[r * RS + i] = kt * __builtin_amdgcn_exp2f(-d);
            } else {
                L.BK[r * RS + i] = b[r];
            }
        }
    }
    __syncthreads();
    // 3. A: wave 0 on MFMA (lane (lm, lk) supplies channel k0 + 4 lk + u of row
    // lm of both factors at step u), or element by element, a thread per entry
    // (the rows and bk as loaded)
    const int lane = tid & 63, wave = tid >> 6;
    const int lm = lane & 15, lk = lane >> 4;
    if (!L.wide) {
        if (wave == 0) {
            gf32x4_t acc = gf32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
            for (int k0 = 0; k0 < DK; k0 += 16) {
                const float4 xa = *reinterpret_cast<const float4*>(L.QT + lm * RS + k0 + 4 * lk);
                const float4 xb = *reinterpret_cast<const float4*>(L.KT + lm * RS + k0 + 4 * lk);
                acc = gmfma4(xa.x, xb.x, acc);
                acc = gmfma4(xa.y, xb.y, acc);
                acc = gmfma4(xa.z, xb.z, acc);
                acc = gmfma4(xa.w, xb.w, acc);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * lk + e;
                o[PL::AM + r * GC + lm] = lm <= r ? acc[e] : 0.f;   // the masked pairs may be out of range
            }
        }
    } else {
        const int r = tid >> 4, s2 = tid & 15;
        float a = 0.f;
        if (s2 <= r) {
#pragma unroll 4
            for (int i = 0; i < DK; i += 4) {
                const float4 x = *reinterpret_cast<const float4*>(L.QT + r * RS + i);
                const float4 y = *reinterpret_cast<const float4*>(L.KT + s2 * RS + i);
                const float4 br = *reinterpret_cast<const float4*>(L.BK + r * RS + i);
                const float4 bs = *reinterpret_cast<const float4*>(L.BK + s2 * RS + i);
                a = fmaf(x.x * y.x, __builtin_amdgcn_exp2f(br.x - bs.x), a);
                a = fmaf(x.y * y.y, __builtin_amdgcn_exp2f(br.y - bs.y), a);
                a = fmaf(x.z * y.z, __builtin_amdgcn_exp2f(br.z - bs.z), a);
                a = fmaf(x.w * y.w, __builtin_amdgcn_exp2f(br.w - bs.w), a);
            }
        }
        o[PL::AM + tid] = a;
    }
}

typedef float gf4v __attribute__((ext_vector_type(4)));

// The chunk's operand block, 16 bytes per thread and step: every thread
// issues the same loads and stores (an index past the block is clamped to its
// last piece), so the count of memory operations in flight is the same on
// every path and the waits for a load issued chunks earlier stay exact.
template <int NP, int N4, int NTH>
__device__ __forceinline__ void gfetch_block(gf4v (&pf)[NP], const float* src)
{
    const gf4v* s4 = reinterpret_cast<const gf4v*>(src);
#pragma unroll
    for (int m = 0; m < NP; ++m) pf[m] = s4[min((int)threadIdx.x + m * NTH, N4 - 1)];
}

template <int NP, int N4, int NTH>
__device__ __forceinline__ void gstore_block(float* dst, const gf4v (&pf)[NP])
{
#pragma unroll
    for (int m = 0; m < NP; ++m) reinterpret_cast<gf4v*>(dst)[min((int)threadIdx.x + m * NTH, N4 - 1)] = pf[m];
}

// The operand blocks are shared by the NG column groups of a workgroup; the
// rest is per group (cg).
template <int DK, int NG>
struct GScanLds {
    alignas(16) float P[2][GPrep<DK>::SIZE];
    float X[NG][2][GC][GJ + 1];    // v of the tile
    float GV[NG][2][GC][GJ + 1];   // gv of the tile (log2 units)
    float PU[NG][GNW][GC][GJ + 1];
    float VC[NG][GC][GJ + 1];      // e^{bv_C - bv} v
    float VF[NG][GC][GJ + 1];      // e^{bv_0 - bv} v
    float ER[NG][GC][GJ + 1];      // e^{bv}
    float EL[NG][GC][GJ + 1];      // e^{bv - bv_0}
    float EVC[NG][GJ];             // e^{bv_C}
    int vwide[NG];                 // some column's value log-decay leaves the factor range
};

// One workgroup per (NG tiles of 16 state columns, head, sequence): NG groups
// of four waves, one tile each, over one LDS copy of each chunk's operand
// block; ids dealt so that the workgroups of one (sequence, head), which read
// the same blocks, share an XCD (ids equal modulo 8).
template <int DK, typename Tin, typename Tout, int NG>
__global__ __launch_bounds__(NG * GTH) __attribute__((amdgpu_waves_per_eu(2))) void gated_scan(GatedParams p)
{
    using PL = GPrep<DK>;
    constexpr int RS = PL::RS;
    constexpr int NT = DK / 16, TPW = (NT + GNW - 1) / GNW;
    constexpr int N4 = PL::SIZE / 4, NP = (N4 + NG * GTH - 1) / (NG * GTH);
    __shared__ GScanLds<DK, NG> L;
    // (the group and wave indices are wave-uniform: kept in scalar registers,
    // so that resources built from them need no per-lane loop)
    const int tid = threadIdx.x % GTH, cg = __builtin_amdgcn_readfirstlane(threadIdx.x / GTH) & (NG - 1);
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6) & (GNW - 1);
    // (the masks change no value: they restate the ranges that readfirstlane
    // hides from the compiler, which then folds the per-wave selections)
    static_assert((NG & (NG - 1)) == 0 && (GNW & (GNW - 1)) == 0, "power-of-two group and wave counts");
    const int lm = lane & 15, lk = lane >> 4;
    const int H = p.H, DV = p.dv;
    const int ntile = DV / (GJ * NG);
    const int xcd = blockIdx.x & 7, qd = blockIdx.x >> 3;
    const int grp = (qd / ntile) * 8 + xcd;
    if (grp >= H * p.N) return;
    const int j0 = (qd % ntile) * GJ * NG + cg * GJ, h = grp % H, n = grp / H;
    const int hk = h / (H / p.Hkv);
    int t0, t1;
    gseq_bounds(p, n, t0, t1);
    const int len = t1 - t0;
    const int nch = min((len + GC - 1) / GC, p.off[n + 1] - p.off[n]);
    const int slot0 = p.off[n];
    const size_t soff = ((size_t)n * H + h) * DK;
    const bool hv = p.gv != nullptr;
    // the initial state tile (zeros without one; rows of idle waves' tiles,
    // t >= NT, fall past the range), every load issued before one wait
    gf32x4_t S[TPW];
    {
        const auto ri = buf_rsrc(p.init ? uniform_ptr(p.init + soff * DV) : nullptr,
                                 p.init ? (uint32_t)(DK * DV * 4) : 0u);
#pragma unroll
        for (int x = 0; x < TPW; ++x) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                S[x][e] = buf_load<float>(ri, (uint32_t)(((16 * (wave + GNW * x) + 4 * lk + e) * DV + j0 + lm) * 4));
        }
    }
    // the initial tile is used here, before the loop: else its loads stay
    // pending into the loop body, whose first use would wait for every load in
    // flight, the prefetched chunks' included
#pragma unroll
    for (int x = 0; x < TPW; ++x) asm volatile("" : "+v"(S[x]));
    const Tin* vv = static_cast<const Tin*>(p.v);
    const int rr = tid / GJ, jj = tid % GJ;
    auto tok = [&](int m) -> size_t {
        m = min(m, len - 1);
        return (size_t)(p.reverse ? t1 - 1 - m : t0 + m);
    };
    // a ring of two register sets: the inputs of chunk c + 2 are loaded while
    // chunk c computes (the loop is unrolled by two, so each set is fixed)
    gf4v pfa[NP], pfb[NP];
    Tin pva = 0, pvb = 0;
    float pga = 0.f, pgb = 0.f;
    auto fetch = [&](gf4v (&pf)[NP], Tin& pv, float& pg, int c) __attribute__((always_inline)) {
        gfetch_block<NP, N4, NG * GTH>(pf, p.prep + ((size_t)(slot0 + c) * H + h) * PL::SIZE);
        const size_t t = tok(c * GC + rr);
        pv = vv[(t * p.Hkv + hk) * DV + j0 + jj];
        // the value gate through a resource over the chunk's rows in memory
        // (from its lowest row; empty without the gate): a load on one path
        // only would make the compiler's waits count the other path's loads
        const int lc = min(GC, len - c * GC), tb = p.reverse ? t1 - c * GC - lc : t0 + c * GC;
        const float* gb = hv ? p.gv + ((size_t)tb * H + h) * DV + j0 : nullptr;
        const auto rg = buf_rsrc(uniform_ptr(gb), __builtin_amdgcn_readfirstlane(hv ? ((lc - 1) * H * DV + GJ) * 4 : 0));
        const int mr = rr < lc ? (p.reverse ? lc - 1 - rr : rr) : 0;
        pg = buf_load<float>(rg, (uint32_t)((mr * H * DV + jj) * 4));
    };
    if (nch > 0) {
        fetch(pfa, pva, pga, 0);
        fetch(pfb, pvb, pgb, min(1, nch - 1));
        // both sets waited for here: the compiler interleaves their loads, and
        // the count of loads in flight that it assumes at the loop head is the
        // larger of the counts on entry and around the loop, so a wait left
        // pending here would drain the next chunk's prefetch on every chunk
#pragma unroll
        for (int m = 0; m < NP; ++m) {
            asm volatile("" : "+v"(pfa[m]));
            asm volatile("" : "+v"(pfb[m]));
        }
        settle(pva);
        settle(pvb);
        settle(pga);
        settle(pgb);
    }
    auto chunk = [&](gf4v (&pf)[NP], Tin& pv, float& pg, int c, auto bsel) __attribute__((always_inline)) {
        constexpr int b = decltype(bsel)::value;
        const float* P = L.P[b];
        const int lc = min(GC, len - c * GC);
        gstore_block<NP, N4, NG * GTH>(L.P[b], pf);
        L.X[cg][b][rr][jj] = rr < lc ? widen(pv) : 0.f;
        L.GV[cg][b][rr][jj] = rr < lc ? pg * kLog2e : 0.f;
        if (tid == 0) L.vwide[cg] = 0;
        fetch(pf, pv, pg, min(c + 2, nch - 1));   // past the end: the last chunk again
        lds_barrier();
        // the inter-chunk read-out sum_i QE_ri S_ij: each wave its tiles' part
        {
            gf32x4_t acc = gf32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int x = 0; x < TPW; ++x) {
                const int t = wave + GNW * x;
                if (t < NT) {
                    const float4 a = *reinterpret_cast<const float4*>(P + PL::QE + lm * RS + 16 * t + 4 * lk);
                    acc = gmfma4(a.x, S[x][0], acc);
                    acc = gmfma4(a.y, S[x][1], acc);
                    acc = gmfma4(a.z, S[x][2], acc);
                    acc = gmfma4(a.w, S[x][3], acc);
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) L.PU[cg][wave][4 * lk + e][lm] = acc[e];
        }
        // the value-axis factors, a thread per (row rr, column jj): the column's
        // cumulative log-decay to row rr and over the chunk
        if (hv) {
            float bc = 0.f, br = 0.f;
#pragma unroll
            for (int s2 = 0; s2 < GC; ++s2) {
                bc += L.GV[cg][b][s2][jj];
                if (s2 == rr) br = bc;
            }
            const float b0 = L.GV[cg][b][0][jj];
            const float x = L.X[cg][b][rr][jj];
            L.VC[cg][rr][jj] = x * __builtin_amdgcn_exp2f(bc - br);
            L.ER[cg][rr][jj] = __builtin_amdgcn_exp2f(br);
            L.VF[cg][rr][jj] = x * __builtin_amdgcn_exp2f(b0 - br);
            L.EL[cg][rr][jj] = __builtin_amdgcn_exp2f(br - b0);
            if (!(fabsf(br - b0) <= 120.f)) L.vwide[cg] = 1;
            if (rr == GC - 1) L.EVC[cg][jj] = __builtin_amdgcn_exp2f(bc);
        }
        lds_barrier();
        // the outputs: O = e^{bv} (QE S) + e^{bv - bv_0} A (e^{bv_0 - bv} v), the
        // second product on MFMA in every wave (lane (lm, lk) supplies A[lm][4 lk + u]
        // and the scaled v[4 lk + u][lm] at step u; element by element when wide);
        // wave w forms and stores rows 4 lk + w, so every wave issues one store
        {
            gf32x4_t ai = gf32x4_t{0.f, 0.f, 0.f, 0.f};
            const bool ew = hv && L.vwide[cg];
            if (!ew) {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int s2 = 4 * lk + u;
                    ai = gmfma4(P[PL::AM + lm * GC + s2], hv ? L.VF[cg][s2][lm] : L.X[cg][b][s2][lm], ai);
                }
            }
            const int r = 4 * lk + wave;
            const float aiw = wave == 0 ? ai[0] : wave == 1 ? ai[1] : wave == 2 ? ai[2] : ai[3];
            const float oi = (L.PU[cg][0][r][lm] + L.PU[cg][1][r][lm]) + (L.PU[cg][2][r][lm] + L.PU[cg][3][r][lm]);
            float o;
            if (!hv) {
                o = oi + aiw;
            } else if (!ew) {
                o = L.ER[cg][r][lm] * oi + L.EL[cg][r][lm] * aiw;
            } else {
                float bvs[GC];
                float acc = 0.f;
#pragma unroll
                for (int s2 = 0; s2 < GC; ++s2) {
                    acc += L.GV[cg][b][s2][lm];
                    bvs[s2] = acc;
                }
                float br = 0.f;
#pragma unroll
                for (int s2 = 0; s2 < GC; ++s2) br = s2 == r ? bvs[s2] : br;
                o = L.ER[cg][r][lm] * oi;
                for (int s2 = 0; s2 <= r; ++s2)
                    o = fmaf(P[PL::AM + r * GC + s2] * __builtin_amdgcn_exp2f(br - bvs[s2]), L.X[cg][b][s2][lm], o);
            }
            // rows past the chunk fall outside the store's range: forward order
            // from the chunk's first token, reverse order from its last one backwards
            const int tb = p.reverse ? t1 - c * GC - lc : t0 + c * GC;
            const auto rs = buf_rsrc(uniform_ptr(static_cast<Tout*>(p.o) + ((size_t)tb * H + h) * DV + j0),
                                     __builtin_amdgcn_readfirstlane(((lc - 1) * H * DV + GJ) * (int)sizeof(Tout)));
            const int trow = p.reverse ? lc - 1 - r : r;   // negative past the chunk: out of range
            buf_store<Tout>(rs, (uint32_t)((trow * H * DV + lm) * (int)sizeof(Tout)), from_f32<Tout>(o));
        }
        // the state update: S <- e^{bk_C + bv_C} S + Kc^T (e^{bv_C - bv} v)
#pragma unroll
        for (int x = 0; x < TPW; ++x) {
            const int t = wave + GNW * x;
            if (t < NT) {
                gf32x4_t a = S[x];
                const float evc = hv ? L.EVC[cg][lm] : 1.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) a[e] *= P[PL::EKC + 16 * t + 4 * lk + e] * evc;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int s2 = 4 * lk + u;
                    a = gmfma4(P[PL::KC + s2 * RS + 16 * t + lm], hv ? L.VC[cg][s2][lm] : L.X[cg][b][s2][lm], a);
                }
                S[x] = a;
            }
        }
    };
    // both halves of the loop body run on every pass, an odd last chunk after
    // the loop (a half skipped on some path into the loop head would make the
    // compiler assume the shorter count of loads in flight there)
    int c = 0;
    for (; c + 1 < nch; c += 2) {
        chunk(pfa, pva, pga, c, std::integral_constant<int, 0>{});
        chunk(pfb, pvb, pgb, c + 1, std::integral_constant<int, 1>{});
    }
    if (c < nch) chunk(pfa, pva, pga, c, std::integral_constant<int, 0>{});
    if (p.final_state) {
#pragma unroll
        for (int x = 0; x < TPW; ++x) {
            const int t = wave + GNW * x;
            if (t < NT) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 16 * t + 4 * lk + e;
                    p.final_state[(soff + i) * DV + j0 + lm] = S[x][e];
                }
            }
        }
    }
}

size_t galign(size_t x) { return (x + 255) / 256 * 256; }

size_t gslots(int N, int T, bool packed)
{
    if (packed) return (size_t)(T / GC) + (size_t)N;
    return (size_t)N * (size_t)((T + GC - 1) / GC);
}

template <int DK, typename Tin, typename Tout>
hipError_t launch_typed(const GatedParams& p, size_t slots, hipStream_t st)
{
    if (slots > 0) {
        hipLaunchKernelGGL((gated_prep<DK, Tin>), dim3((unsigned)slots, (unsigned)p.H), dim3(GTH), 0, st, p);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const unsigned groups8 = (unsigned)((p.H * p.N + 7) / 8 * 8);
    if (groups8 == 0) return hipSuccess;
    // two column tiles per workgroup (one LDS copy of each block for both)
    // once that still gives every CU a workgroup; else one
    if (p.dv >= 2 * GJ && (size_t)p.H * p.N * (p.dv / (2 * GJ)) >= kGCUs)
        hipLaunchKernelGGL((gated_scan<DK, Tin, Tout, 2>), dim3(groups8 * (unsigned)(p.dv / (2 * GJ))),
                           dim3(2 * GTH), 0, st, p);
    else
        hipLaunchKernelGGL((gated_scan<DK, Tin, Tout, 1>), dim3(groups8 * (unsigned)(p.dv / GJ)), dim3(GTH), 0, st,
                           p);
    return hipGetLastError();
}

template <int DK>
hipError_t launch_dk(const GatedParams& p, size_t slots, bool in_bf16, bool out_bf16, hipStream_t st)
{
    if (!in_bf16) return launch_typed<DK, float, float>(p, slots, st);
    if (out_bf16) return launch_typed<DK, uint16_t, bf16_t>(p, slots, st);
    return launch_typed<DK, uint16_t, float>(p, slots, st);
}

}  // namespace

size_t gated_workspace_bytes(int N, int T, int H, int dk, bool packed)
{
    const size_t slots = (N > 0 && T > 0) ? gslots(N, T, packed) : 0;
    return galign((size_t)(N + 1) * 4) + galign(slots * H * gprep_floats(dk) * 4);
}

hipError_t launch_gated(const GatedArgs& a, hipStream_t st)
{
    const bool packed = a.cu != nullptr;
    const size_t slots = (a.N > 0 && a.T > 0) ? gslots(a.N, a.T, packed) : 0;
    GatedParams p{};
    p.q = a.q; p.k = a.k; p.v = a.v;
    p.g = a.g; p.g_gamma = a.g_gamma; p.g_gamma_rows = a.g_gamma_rows; p.gk = a.gk; p.gv = a.gv;
    p.init = a.init; p.cu = a.cu;
    p.N = a.N; p.T = a.T; p.H = a.H; p.Hkv = a.Hkv; p.dv = a.dv;
    p.scale = a.scale; p.reverse = a.reverse;
    p.o = a.o; p.final_state = a.final_state;
    unsigned char* w = static_cast<unsigned char*>(a.workspace);
    int32_t* off = reinterpret_cast<int32_t*>(w);
    p.off = off;
    p.prep = reinterpret_cast<float*>(w + galign((size_t)(a.N + 1) * 4));
    hipLaunchKernelGGL(gated_plan_kernel, dim3(1), dim3(64), 0, st, p, (int)slots, off);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    switch (a.dk) {
    case 16: return launch_dk<16>(p, slots, a.in_bf16 != 0, a.out_bf16 != 0, st);
    case 32: return launch_dk<32>(p, slots, a.in_bf16 != 0, a.out_bf16 != 0, st);
    case 64: return launch_dk<64>(p, slots, a.in_bf16 != 0, a.out_bf16 != 0, st);
    default: return launch_dk<128>(p, slots, a.in_bf16 != 0, a.out_bf16 != 0, st);
    }
}

}  // namespace kda
