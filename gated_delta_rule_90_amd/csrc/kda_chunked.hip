// kda_chunked.hip - chunk-parallel KDA prefill on gfx950 MFMA: the chunked
// mode of the ejkernel "kernel_delta_attention" page (section "Algorithm
// modes"; run() default chunk_size 64).
//
// The pages give no chunk formulas; the ones below are an exact algebraic
// regrouping of the token recurrence (decay per key channel, residual
// against the decayed state, o = S^T q).  Within a chunk of C = 64 tokens,
// with b_r = sum_{s<=r} gamma_s per channel (restarting at the chunk start),
// beta_r the activated beta and S0 the state entering the chunk:
//     A_rs = beta_r sum_i kh_ri kh_si e^{b_ri - b_si}   (s < r)
//     P_rs = sum_i qh_ri kh_si e^{b_ri - b_si}          (s <= r)
//     T = (I + A)^-1,  T' = T diag(beta)
//     W = T' Kg (Kg_s = e^{b_s} kh_s),   U~ = T' V,   U = U~ - W S0
//     O = Qg S0 + P U (Qg_r = e^{b_r} qh_r)
//     S = Diag(e^{b_C}) S0 + Kc^T U  (Kc_s = e^{b_C - b_s} kh_s)
//
// Two kernels.  chunk_prep runs once per (chunk, head), all in parallel: the
// prologue (L2 norms, gate, beta, per-channel cumulative decay), A and P,
// the triangular inverse and W - everything that does not depend on the
// state.  It writes W, Qg, Kc^T, T', P and e^{b_C} to the workspace as
// bf16 MFMA operands.  chunk_scan then walks the chunks of each (sequence,
// head, 32-column dv tile) in order and does only the state-dependent
// contractions (U~, U, O, the state carry), prefetching the next chunk's
// operands while it computes the current one.  The per-element prologue is
// therefore computed once per chunk instead of once per dv tile.
//
// Overflow-safe per-channel decay: with lower_bound >= -5 the cumulative
// log-decay reaches -320 in a chunk, beyond fp32's exp range, so A and P are
// built on 16-row sub-blocks.  For row block I (first row f_I) and column
// block J (last row e_J):
//     left  L_r  = e^{b_r - b_fI}  in (e^-75, 1]
//     right      = e^{b_fI - b_s} = e^{b_fI - b_eJ} * e^{b_eJ - b_s}   (J < I, both <= 1)
//                = 1 / L_s                                            (J = I, <= e^75)
// so every factor stays inside fp32/bf16 range and every underflow is of a
// value that is itself below 1e-38.  Masks are applied by select.
//
// EJK mode (scalar per-head decay d_t, beta used as given, residual against
// the undecayed state): the residual of row r sees the state decayed up to
// row r-1 only, so A_rs carries e^{b_{r-1} - b_s} and Kg_r = e^{b_{r-1}} kh_r
// (b_{-1} = 0); P, Qg, Kc and the carry are as above with the scalar b.  One
// decay for all channels means A and P are the plain Gram products of the
// normalised rows, scaled element by element: with d <= 0 every factor is at
// most 1, so no factorisation is needed.
//
// Rows of a partial last chunk are padded with exact neutral values
// (q = k = v = 0, gamma = 0, beta = 0) and never stored, so a packed varlen
// batch gives bitwise the same result as each sequence alone.
#include <algorithm>
#include <type_traits>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int C = 64;        // chunk length
constexpr int DK = 128;      // key dimension handled by the MFMA path
constexpr int DV_MULT = 16;  // the MFMA path needs dv to be a multiple of this (one 16-column tile)
constexpr int NTHREADS = 256;

// ---- workspace record of one (chunk, head), bf16 operands in k-slices of 32:
// element (row, k) of a [R][K] operand sits at ((k / 32) * R + row) * 32 + k % 32,
// so the 16x32 MFMA fragment of a wave is 1 KiB of contiguous memory.
constexpr int REC_W = 0;                       // W   [64 r][128 i]
constexpr int REC_QG = REC_W + C * DK * 2;     // Qg  [64 r][128 i]
constexpr int REC_KCT = REC_QG + C * DK * 2;   // Kc^T [128 i][64 s]
constexpr int REC_TP = REC_KCT + DK * C * 2;   // T'  [64 r][64 s]
constexpr int REC_P = REC_TP + C * C * 2;      // P   [64 r][64 s]
constexpr int REC_EC = REC_P + C * C * 2;      // e^{b_C} [128] fp32
constexpr int REC_BYTES = REC_EC + DK * 4;     // 66048
constexpr int OFFSETS_BYTES_ALIGN = 256;

__device__ __forceinline__ int ksl(int R, int row, int k) { return ((k >> 5) * R + row) * 32 + (k & 31); }

// ---- prep-kernel LDS (bytes)
constexpr int SR = DK + 8;   // [64][DK] bf16 tiles (272 B rows)
constexpr int SW = C + 8;    // [*][64] bf16 tiles (144 B rows)
constexpr int SA = C + 4;    // A, fp32 [64][64]
constexpr int ST = C + 4;    // Tcol / Trow bf16 [64][64] (136 B rows, 8 B aligned)
constexpr int SY = 40;       // [32][32] bf16 scratch
constexpr int TILE_R = C * SR * 2;                  // 17408
constexpr int P_QL = 0;                             // QL  -> T' [64][SW] + Y scratch
constexpr int P_KL = P_QL + TILE_R;                 // KL  -> Tcol, Trow
constexpr int P_KRD = P_KL + TILE_R;                // KRd -> A (fp32)
constexpr int P_KGT = P_KRD + TILE_R;               // Kg^T [DK][SW]
constexpr int P_VEC = P_KGT + DK * SW * 2;          // fp32 vectors
constexpr int V_BETA = 0, V_NQ = 64, V_NK = 128, V_BT = 192, V_M = V_BT + 4 * DK, V_C = V_M + 6 * DK;
constexpr int VEC_FLOATS = V_C + 4 * DK;
constexpr int V_B = V_M, V_BX = V_M + C;   // EJK: row cumsums b_r, b_{r-1} (in the pair-vector space)
constexpr int PREP_LDS = P_VEC + VEC_FLOATS * 4;
constexpr int P_TP = P_QL;
constexpr int P_Y = P_QL + C * SW * 2;
constexpr int P_TCOL = P_KL;
constexpr int P_TROW = P_KL + C * ST * 2;
constexpr int P_A = P_KRD;
// staging of an item's inputs at the start of phase 1a (before any of the above
// is written): per wave [16 rows][128] bf16 q, then k, then fp32 gates
constexpr int P_STG_Q = 0;
constexpr int P_STG_K = P_STG_Q + 4 * 16 * DK * 2;
constexpr int P_STG_G = P_STG_K + 4 * 16 * DK * 2;
static_assert(P_STG_G + 4 * 16 * DK * 4 <= P_VEC, "staging below the vectors");
static_assert(PREP_LDS <= 80 * 1024, "two prep workgroups per CU");
static_assert(C * SA * 4 <= TILE_R, "A fits in a tile slot");
static_assert(2 * C * ST * 2 <= TILE_R, "Tcol + Trow fit in a tile slot");
static_assert(C * SW * 2 + 32 * SY * 2 <= TILE_R, "T' + scratch");

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// two floats -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack2(float a, float b)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}
__device__ __forceinline__ float lo_bf(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float hi_bf(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

__device__ __forceinline__ bf16x8_t ld8(const uint16_t* base, int stride, int row, int col)
{
    return *reinterpret_cast<const bf16x8_t*>(base + row * stride + col);
}
__device__ __forceinline__ s16x4_t ld4(const uint16_t* base, int stride, int row, int col)
{
    return *reinterpret_cast<const s16x4_t*>(base + row * stride + col);
}
__device__ __forceinline__ s16x4_t f32_to_s16x4(float4 v)
{
    const uint32_t a = pack2(v.x, v.y), b = pack2(v.z, v.w);
    s16x4_t r;
    r[0] = (short)(a & 0xffff); r[1] = (short)(a >> 16);
    r[2] = (short)(b & 0xffff); r[3] = (short)(b >> 16);
    return r;
}
__device__ __forceinline__ f32x4_t mfma32(bf16x8_t a, bf16x8_t b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma16(s16x4_t a, s16x4_t b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void st4bf(uint16_t* p, float a, float b, float c, float d)
{
    *reinterpret_cast<uint2*>(p) = make_uint2(pack2(a, b), pack2(c, d));
}
__device__ __forceinline__ void st1bf(uint16_t* p, float a)
{
    *p = __builtin_bit_cast(uint16_t, (__bf16)a);
}
__device__ __forceinline__ uint4 pack8(const float* x)
{
    return make_uint4(pack2(x[0], x[1]), pack2(x[2], x[3]), pack2(x[4], x[5]), pack2(x[6], x[7]));
}

// Sum 16 per-row partials over the 64 lanes of a wave.  On return lane l
// holds the total of row (l >> 2).  Each step halves the entries a lane
// carries and sums over a lane partner: the two halves and the row pairs by
// permlane swaps (the swap itself routes entry k to one side and entry
// k + width to the other), then partners whose lane bits 3 and 2 differ by DPP
// mirrors within a row and a half row (lane i <-> 15 - i, 7 - i), and last the
// quad.
__device__ __forceinline__ float rowsum16(float (&a)[16], int lane)
{
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        swap_halves32(a[k], a[k + 8]);
        a[k] += a[k + 8];
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        swap_rows16(a[k], a[k + 4]);
        a[k] += a[k + 4];
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const bool hi = lane & 8;
        const float send = hi ? a[k] : a[k + 2];
        const float keep = hi ? a[k + 2] : a[k];
        a[k] = keep + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, send), 0x140, 0xF, 0xF, true));
    }
    float s;
    {
        const bool hi = lane & 4;
        const float send = hi ? a[0] : a[1];
        const float keep = hi ? a[1] : a[0];
        s = keep + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, send), 0x141, 0xF, 0xF, true));
    }
    return xor_add<1>(xor_add<2>(s));
}

// index of the off-diagonal pair (I, J), I > J, in the pair-vector table
__device__ __forceinline__ int pair_slot(int I, int J) { return I * (I - 1) / 2 + J; }

// Sequence bounds (clamped) of sequence n.  Dense rows: sequences of T rows
// starting ts rows apart (ts = T, except for a segment of longer sequences).
__device__ __forceinline__ void seq_bounds(const int32_t* cu, int n, int T, int ts, int& t0, int& t1)
{
    if (cu) {
        t0 = min(max(cu[n], 0), T);
        t1 = min(max(cu[n + 1], t0), T);
    } else {
        t0 = n * ts;
        t1 = t0 + T;
    }
}

// ------------------------------------------------------------------------
// Plan of a packed batch: chunk offsets off[n] = sum_{m<n} ceil(len_m / 64),
// and order[] = the sequences by decreasing chunk count (ties by index).  The
// scan hands out its workgroups in that order, longest chains first, so the
// longest sequences do not start last (list scheduling by decreasing length).
// Above PLAN_SORT_MAX sequences the order is the identity.
constexpr int PLAN_THREADS = 256;
constexpr int PLAN_SORT_MAX = 2048;

__global__ __launch_bounds__(PLAN_THREADS) void chunk_plan_kernel(const int32_t* __restrict__ cu, int N, int T,
                                                                  int32_t* __restrict__ off,
                                                                  int32_t* __restrict__ order)
{
    __shared__ int nchunks[PLAN_SORT_MAX];
    const int tid = threadIdx.x;
    if (tid == 0) {
        int acc = 0;
        for (int n = 0; n < N; ++n) {
            int t0, t1;
            seq_bounds(cu, n, T, T, t0, t1);
            off[n] = acc;
            acc += (t1 - t0 + C - 1) / C;
        }
        off[N] = acc;
    }
    if (N > PLAN_SORT_MAX) {
        for (int n = tid; n < N; n += PLAN_THREADS) order[n] = n;
        return;
    }
    for (int n = tid; n < N; n += PLAN_THREADS) {
        int t0, t1;
        seq_bounds(cu, n, T, T, t0, t1);
        nchunks[n] = (t1 - t0 + C - 1) / C;
    }
    __syncthreads();
    for (int n = tid; n < N; n += PLAN_THREADS) {
        const int ln = nchunks[n];
        int rank = 0;
        for (int m = 0; m < N; ++m) {
            const int lm = nchunks[m];
            rank += (lm > ln || (lm == ln && m < n)) ? 1 : 0;
        }
        order[rank] = n;
    }
}

// ------------------------------------------------------------------------
// chunk_prep: a persistent grid of two workgroups per CU (by LDS) walks the
// (chunk slot, head) items; each workgroup loads its next item's inputs as
// soon as the current item's prologue has consumed its own, so the loads
// overlap the rest of the item's work.
struct PrepItem {
    int slot, h, c0, len;
    bool valid;
};

// Item = slot * H + head.  Slots past the packed chunk count (and items past
// the end) are not valid.
__device__ __forceinline__ PrepItem prep_item(int item, int nitems, int H, const int32_t* cu, const int32_t* off,
                                              int N, int T, int ts)
{
    PrepItem it{0, 0, 0, 0, false};
    if (item >= nitems) return it;
    it.slot = item / H;
    it.h = item - it.slot * H;
    int n, c;
    if (off) {
        if (it.slot >= off[N]) return it;
        int lo = 0, hi = N - 1;          // largest n with off[n] <= slot
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (off[mid] <= it.slot) lo = mid; else hi = mid - 1;
        }
        n = lo;
        c = it.slot - off[n];
    } else {
        const int ncs = (T + C - 1) / C;
        n = it.slot / ncs;
        c = it.slot - n * ncs;
    }
    int t_begin, t_end;
    seq_bounds(cu, n, T, ts, t_begin, t_end);
    it.c0 = t_begin + c * C;
    it.len = min(C, t_end - it.c0);
    it.valid = true;
    return it;
}

// An item's inputs as loaded, 16 bytes per lane: wide loads keep more bytes in
// flight per outstanding request than one row of two channels per lane would.
struct PrepRaw {
    u32x4_t q[4], k[4];   // rows 16*blk + 4i + (lane >> 4), channels 8*(lane & 15) .. +7 (bf16)
    u32x4_t g[8];         // KDA gates: rows 16*blk + 2i + (lane >> 5), channels 4*(lane & 31) .. +3
    float ge[16];         // EJK: the decay of row 16*blk + m (the same in every lane)
    float beta;           // lanes < 16: beta logit of row 16*blk + lane
};

// q, k and the KDA gates go through a buffer resource per group of rows (the
// group's first row uniform, the lane's row within it in its offset): rows
// past the sequence fall outside and read as zero (they are zeroed on use
// as well).  The beta logits and EJK decays of rows past the sequence read the
// chunk's first row.  EJK: g is [tokens][H] (one decay per token and head;
// NULL = no decay).  PART 0 loads q, k and beta, PART 1 the gates (half of the
// bytes), PART 2 both.
template <bool EJK, int PART = 2>
__device__ __forceinline__ void prep_load(PrepRaw& r, const PrepItem& it, const bf16_t* q, const bf16_t* k,
                                          const float* g, const float* beta, int H, int HKV, int lane, int blk)
{
    const size_t base = ((size_t)it.c0 * H + it.h) * DK;   // channel 0 of the item's first row
    const uint32_t rstride = (uint32_t)H * DK;
    if constexpr (PART != 1) {
        // k: the key/value head of head h, rows HKV heads apart
        const size_t kbase = ((size_t)it.c0 * HKV + it.h / (H / HKV)) * DK;
        const uint32_t kstride = (uint32_t)HKV * DK;
        const uint32_t col = 16 * (lane & 15);   // bytes: 8 bf16 channels per lane
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r0 = 16 * blk + 4 * i;      // rows r0 .. r0 + 3, the lane's is r0 + lane / 16
            r.q[i] = buf_load<u32x4_t>(rows_rsrc(q + base, r0, it.len, 2 * rstride, 2 * DK), (lane >> 4) * 2 * rstride + col);
            r.k[i] = buf_load<u32x4_t>(rows_rsrc(k + kbase, r0, it.len, 2 * kstride, 2 * DK), (lane >> 4) * 2 * kstride + col);
        }
        const int rb = 16 * blk + (lane & 15);
        r.beta = beta[(size_t)(it.c0 + ((rb < it.len) ? rb : 0)) * H + it.h];
    }
    if constexpr (PART != 0) {
        if constexpr (EJK) {
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                const int rr = 16 * blk + m;
                r.ge[m] = g ? g[(size_t)(it.c0 + ((rr < it.len) ? rr : 0)) * H + it.h] : 0.f;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r0 = 16 * blk + 2 * i;      // rows r0, r0 + 1, the lane's is r0 + lane / 32
                r.g[i] = buf_load<u32x4_t>(rows_rsrc(g + base, r0, it.len, 4 * rstride, 4 * DK),
                                           (lane >> 5) * 4 * rstride + 16 * (lane & 31));
            }
        }
    }
}

template <bool EJK>
__global__ __launch_bounds__(NTHREADS, 2) void chunk_prep_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const float* __restrict__ g,
    const float* __restrict__ beta, const float* __restrict__ a_log, const float* __restrict__ dt_bias,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ off, int N, int T, int ts, int H, int HKV, int nslots,
    float scale, float lower_bound, int l2norm, unsigned char* __restrict__ ws)
{
    __shared__ __attribute__((aligned(16))) unsigned char smem[PREP_LDS];
    uint16_t* QL = reinterpret_cast<uint16_t*>(smem + P_QL);
    uint16_t* KL = reinterpret_cast<uint16_t*>(smem + P_KL);
    uint16_t* KRD = reinterpret_cast<uint16_t*>(smem + P_KRD);
    uint16_t* KGT = reinterpret_cast<uint16_t*>(smem + P_KGT);
    float* VEC = reinterpret_cast<float*>(smem + P_VEC);
    uint16_t* TP = reinterpret_cast<uint16_t*>(smem + P_TP);
    uint16_t* YS = reinterpret_cast<uint16_t*>(smem + P_Y);
    uint16_t* TCOL = reinterpret_cast<uint16_t*>(smem + P_TCOL);
    uint16_t* TROW = reinterpret_cast<uint16_t*>(smem + P_TROW);
    float* AB = reinterpret_cast<float*>(smem + P_A);

    const float lb2 = lower_bound * kLog2e;             // gamma in log2 units

    const int nitems = nslots * H;
    int item = blockIdx.x;
    PrepItem it = prep_item(item, nitems, H, cu, off, N, T, ts);
    PrepRaw cur;
    if (it.valid)
        prep_load<EJK>(cur, it, q, k, g, beta, H, HKV, threadIdx.x & 63, __builtin_amdgcn_readfirstlane(threadIdx.x >> 6));
    for (; item < nitems; item += gridDim.x) {
        // Thread indices are re-read opaquely in every iteration, so that the
        // per-lane address arithmetic derived from them is recomputed where it
        // is used instead of being hoisted out of the loop into registers.
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const int lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar address math
        const int l16 = lane & 15;
        const int g4 = lane >> 4;
        const int ch = 2 * lane;          // this lane's key channels in the prologue
        const int blk = wave;             // this wave's 16-row block in the prologue
        const PrepItem me = it;
        if (!me.valid) {   // a slot past the packed chunk count: only move on
            it = prep_item(item + gridDim.x, nitems, H, cu, off, N, T, ts);
            if (it.valid) prep_load<EJK>(cur, it, q, k, g, beta, H, HKV, lane, blk);
            continue;
        }
        const int h = me.h;
        const int len = me.len;
        // the item's record, stored through a buffer resource with 32-bit offsets
        const __amdgpu_buffer_rsrc_t rr = buf_rsrc(ws + ((size_t)me.slot * H + h) * REC_BYTES, REC_BYTES);
        const float ea = EJK ? 0.f : expf(a_log[h]) * kLog2e;   // exp(a_log) folded with log2(e)
        const float dtb0 = (!EJK && dt_bias) ? dt_bias[(size_t)ch * H + h] : 0.f;
        const float dtb1 = (!EJK && dt_bias) ? dt_bias[(size_t)(ch + 1) * H + h] : 0.f;

        // ---------------- phase 1a: partial norms, gate, in-block cumsum (inputs already loaded)
        // The inputs arrive 16 bytes per lane.  This wave's rows go through its
        // own LDS staging region to the prologue's layout, two channels of every
        // row per lane; a wave's LDS operations are performed in order, so no
        // barrier is needed between its writes and its reads.
        uint32_t qin[16], kin[16];
        float2 gin[16];
        {
            uint16_t* stq = reinterpret_cast<uint16_t*>(smem + P_STG_Q) + blk * 16 * DK;
            uint16_t* stk = reinterpret_cast<uint16_t*>(smem + P_STG_K) + blk * 16 * DK;
            float* stg = reinterpret_cast<float*>(smem + P_STG_G) + blk * 16 * DK;
    #pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rl = 4 * i + (lane >> 4);
                *reinterpret_cast<u32x4_t*>(stq + rl * DK + 8 * (lane & 15)) = cur.q[i];
                *reinterpret_cast<u32x4_t*>(stk + rl * DK + 8 * (lane & 15)) = cur.k[i];
            }
            if constexpr (!EJK) {
    #pragma unroll
                for (int i = 0; i < 8; ++i)
                    *reinterpret_cast<u32x4_t*>(stg + (2 * i + (lane >> 5)) * DK + 4 * (lane & 31)) = cur.g[i];
            }
    #pragma unroll
            for (int m = 0; m < 16; ++m) {
                qin[m] = *reinterpret_cast<const uint32_t*>(stq + m * DK + ch);
                kin[m] = *reinterpret_cast<const uint32_t*>(stk + m * DK + ch);
                gin[m] = EJK ? make_float2(cur.ge[m], 0.f) : *reinterpret_cast<const float2*>(stg + m * DK + ch);
            }
        }
        uint32_t qraw[16], kraw[16];
        float cb0[16], cb1[16];
        {
            float sq[16], sk[16];
    #pragma unroll
            for (int m = 0; m < 16; ++m) {
                const bool valid = 16 * blk + m < len;
                qraw[m] = valid ? qin[m] : 0u;
                kraw[m] = valid ? kin[m] : 0u;
                const float q0 = lo_bf(qraw[m]), q1 = hi_bf(qraw[m]);
                const float k0 = lo_bf(kraw[m]), k1 = hi_bf(kraw[m]);
                sq[m] = q0 * q0 + q1 * q1;
                sk[m] = k0 * k0 + k1 * k1;
                if constexpr (EJK) {
                    // the token's log-decay in log2 units, shared by all channels
                    const float gm = valid ? gin[m].x * kLog2e : 0.f;
                    cb0[m] = (m == 0 ? 0.f : cb0[m - 1]) + gm;
                    cb1[m] = cb0[m];
                } else {
                    // gamma' = lb * log2(e) * sigmoid(exp(a_log) * (g + dt_bias))
                    const float e0 = __builtin_amdgcn_exp2f(-ea * (gin[m].x + dtb0));
                    const float e1 = __builtin_amdgcn_exp2f(-ea * (gin[m].y + dtb1));
                    const float gm0 = valid ? lb2 * __builtin_amdgcn_rcpf(1.f + e0) : 0.f;
                    const float gm1 = valid ? lb2 * __builtin_amdgcn_rcpf(1.f + e1) : 0.f;
                    cb0[m] = (m == 0 ? 0.f : cb0[m - 1]) + gm0;
                    cb1[m] = (m == 0 ? 0.f : cb1[m - 1]) + gm1;
                }
            }
            const float rq = rowsum16(sq, lane);
            const float rk = rowsum16(sk, lane);
            if ((lane & 3) == 0) {
                const int r = 16 * blk + (lane >> 2);
                VEC[V_NQ + r] = l2norm ? scale / sqrtf(rq + kNormEps) : scale;
                VEC[V_NK + r] = l2norm ? 1.0f / sqrtf(rk + kNormEps) : 1.0f;
            }
            VEC[V_BT + blk * DK + ch] = cb0[15];
            VEC[V_BT + blk * DK + ch + 1] = cb1[15];
            if (lane < 16) {
                const int r = 16 * blk + lane;
                VEC[V_BETA + r] = (r < len) ? (EJK ? cur.beta : sigmoid_f(cur.beta)) : 0.f;
            }
        }
        // the inputs are in qraw, kraw, cb0, cb1 and VEC now: fetch the next item's,
        // q, k and beta here and the gates after phase 1b, so that a CU's limited
        // outstanding requests drain under this item's compute instead of stalling
        // issue in one place (unconditionally: past the end this reloads the current
        // item, which keeps the loaded registers out of a branch)
        it = prep_item(item + gridDim.x, nitems, H, cu, off, N, T, ts);
        const PrepItem nx = it.valid ? it : me;
        prep_load<EJK, 0>(cur, nx, q, k, g, beta, H, HKV, lane, blk);
        lds_barrier();

        // ---------------- phase 1b: decay factors; QL, KL, KRd and Kg^T in LDS; Qg, Kc^T out
        if constexpr (EJK) {
            // scalar decay: QL, KL hold the normalised rows; the row cumsums b_r and
            // b_{r-1} go to V_B / V_BX for the element-wise scaling of A and P
            float P0 = 0.f, tot = 0.f;
    #pragma unroll
            for (int J = 0; J < 4; ++J) {
                const float t = VEC[V_BT + J * DK];
                if (J < blk) P0 += t;
                tot += t;
            }
            if (blk == 0) {
                const float ec = __builtin_amdgcn_exp2f(tot);
                buf_store(rr, REC_EC + 4 * ch, make_float2(ec, ec));
            }
            float kg0[16], kg1[16], kc0[16], kc1[16];
    #pragma unroll
            for (int m = 0; m < 16; ++m) {
                const int r = 16 * blk + m;
                const float b = P0 + cb0[m];
                const float bx = P0 + (m == 0 ? 0.f : cb0[m - 1]);
                if (lane == 0) {
                    VEC[V_B + r] = b;
                    VEC[V_BX + r] = bx;
                }
                const float nq = VEC[V_NQ + r], nk = VEC[V_NK + r];
                const float qh0 = lo_bf(qraw[m]) * nq, qh1 = hi_bf(qraw[m]) * nq;
                const float kh0 = lo_bf(kraw[m]) * nk, kh1 = hi_bf(kraw[m]) * nk;
                const float eb = __builtin_amdgcn_exp2f(b);
                const float ebx = __builtin_amdgcn_exp2f(bx);
                const float ecb = __builtin_amdgcn_exp2f(tot - b);
                const int at = r * SR + ch;
                *reinterpret_cast<uint32_t*>(QL + at) = pack2(qh0, qh1);
                *reinterpret_cast<uint32_t*>(KL + at) = pack2(kh0, kh1);
                buf_store(rr, REC_QG + 2 * ksl(C, r, ch), pack2(eb * qh0, eb * qh1));
                kg0[m] = ebx * kh0;
                kg1[m] = ebx * kh1;
                kc0[m] = ecb * kh0;
                kc1[m] = ecb * kh1;
            }
            uint16_t* g0p = KGT + ch * SW + 16 * blk;
            uint16_t* g1p = KGT + (ch + 1) * SW + 16 * blk;
            const uint32_t c0o = REC_KCT + 2 * ksl(DK, ch, 16 * blk);
            const uint32_t c1o = REC_KCT + 2 * ksl(DK, ch + 1, 16 * blk);
    #pragma unroll
            for (int h8 = 0; h8 < 2; ++h8) {
                *reinterpret_cast<uint4*>(g0p + 8 * h8) = pack8(kg0 + 8 * h8);
                *reinterpret_cast<uint4*>(g1p + 8 * h8) = pack8(kg1 + 8 * h8);
                buf_store(rr, c0o + 16 * h8, pack8(kc0 + 8 * h8));
                buf_store(rr, c1o + 16 * h8, pack8(kc1 + 8 * h8));
            }
        } else {
            float P0 = 0.f, P1 = 0.f, tot0 = 0.f, tot1 = 0.f;
            float pre0[4], pre1[4];   // b at the end of block J
    #pragma unroll
            for (int J = 0; J < 4; ++J) {
                const float t0 = VEC[V_BT + J * DK + ch], t1 = VEC[V_BT + J * DK + ch + 1];
                if (J < blk) { P0 += t0; P1 += t1; }
                tot0 += t0;
                tot1 += t1;
                pre0[J] = tot0;
                pre1[J] = tot1;
            }
            const float bf0 = P0 + cb0[0], bf1 = P1 + cb1[0];          // b at the first row of the block
            const float E0 = __builtin_amdgcn_exp2f(bf0), E1 = __builtin_amdgcn_exp2f(bf1);
            const float c_0 = __builtin_amdgcn_exp2f(cb0[15] - cb0[0]);  // e^{b_e - b_f} of this block
            const float c_1 = __builtin_amdgcn_exp2f(cb1[15] - cb1[0]);
            const float N0 = __builtin_amdgcn_exp2f(tot0 - pre0[blk]);    // e^{b_C - b_e}
            const float N1 = __builtin_amdgcn_exp2f(tot1 - pre1[blk]);
            // pair vectors e^{b_fI - b_eJ} for rows of this block against earlier blocks J
    #pragma unroll
            for (int J = 0; J < 3; ++J) {
                if (J < blk) {
                    const int ps = pair_slot(blk, J);
                    VEC[V_M + ps * DK + ch] = __builtin_amdgcn_exp2f(bf0 - pre0[J]);
                    VEC[V_M + ps * DK + ch + 1] = __builtin_amdgcn_exp2f(bf1 - pre1[J]);
                }
            }
            if (blk == 0) {
                buf_store(rr, REC_EC + 4 * ch, make_float2(__builtin_amdgcn_exp2f(tot0), __builtin_amdgcn_exp2f(tot1)));
            }
            float kg0[16], kg1[16], kc0[16], kc1[16];
    #pragma unroll
            for (int m = 0; m < 16; ++m) {
                const int r = 16 * blk + m;
                const float nq = VEC[V_NQ + r], nk = VEC[V_NK + r];
                const float qh0 = lo_bf(qraw[m]) * nq, qh1 = hi_bf(qraw[m]) * nq;
                const float kh0 = lo_bf(kraw[m]) * nk, kh1 = hi_bf(kraw[m]) * nk;
                const float L0 = __builtin_amdgcn_exp2f(cb0[m] - cb0[0]);
                const float L1 = __builtin_amdgcn_exp2f(cb1[m] - cb1[0]);
                const float iL0 = __builtin_amdgcn_rcpf(L0), iL1 = __builtin_amdgcn_rcpf(L1);
                const float ql0 = L0 * qh0, ql1 = L1 * qh1;
                const float kl0 = L0 * kh0, kl1 = L1 * kh1;
                const float kd0 = iL0 * kh0, kd1 = iL1 * kh1;
                const int at = r * SR + ch;
                *reinterpret_cast<uint32_t*>(QL + at) = pack2(ql0, ql1);
                *reinterpret_cast<uint32_t*>(KL + at) = pack2(kl0, kl1);
                *reinterpret_cast<uint32_t*>(KRD + at) = pack2(kd0, kd1);
                buf_store(rr, REC_QG + 2 * ksl(C, r, ch), pack2(E0 * ql0, E1 * ql1));
                kg0[m] = E0 * kl0;
                kg1[m] = E1 * kl1;
                kc0[m] = N0 * c_0 * kd0;   // e^{b_C - b_e} e^{b_e - b_f} e^{b_f - b_s} kh_s
                kc1[m] = N1 * c_1 * kd1;
            }
            // 16 consecutive tokens of one channel = 32 contiguous bytes
            uint16_t* g0p = KGT + ch * SW + 16 * blk;
            uint16_t* g1p = KGT + (ch + 1) * SW + 16 * blk;
            const uint32_t c0o = REC_KCT + 2 * ksl(DK, ch, 16 * blk);
            const uint32_t c1o = REC_KCT + 2 * ksl(DK, ch + 1, 16 * blk);
    #pragma unroll
            for (int h8 = 0; h8 < 2; ++h8) {
                *reinterpret_cast<uint4*>(g0p + 8 * h8) = pack8(kg0 + 8 * h8);
                *reinterpret_cast<uint4*>(g1p + 8 * h8) = pack8(kg1 + 8 * h8);
                buf_store(rr, c0o + 16 * h8, pack8(kc0 + 8 * h8));
                buf_store(rr, c1o + 16 * h8, pack8(kc1 + 8 * h8));
            }
            // this block's e^{b_e - b_f}, which turns KRd into e^{b_e - b_s} kh_s for later blocks
            VEC[V_C + blk * DK + ch] = c_0;
            VEC[V_C + blk * DK + ch + 1] = c_1;
        }
        lds_barrier();

        prep_load<EJK, 1>(cur, nx, q, k, g, beta, H, HKV, lane, blk);

        // ---------------- phase 2: A and P on 16x16 block pairs (I >= J)
        f32x4_t accA[3], accP[3];
        int pI[3], pJ[3];
    #pragma unroll
        for (int pp = 0; pp < 3; ++pp) {
            const int pidx = wave + 4 * pp;
            accA[pp] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            accP[pp] = accA[pp];
            int I = 0, J = 0;
            if (pidx < 4) { I = pidx; J = pidx; }
            else if (pidx < 7) { I = pidx - 3; J = I - 1; }
            else if (pidx < 9) { I = pidx - 5; J = I - 2; }
            else { I = 3; J = 0; }
            pI[pp] = I;
            pJ[pp] = J;
            if (pidx >= 10) continue;
    #pragma unroll
            for (int ks = 0; ks < DK / 32; ++ks) {
                const int kc = 32 * ks + 8 * g4;
                const bf16x8_t raw = ld8(EJK ? KL : KRD, SR, 16 * J + l16, kc);
                bf16x8_t x = raw;
                if (!EJK && I != J) {
                    // e^{b_fI - b_eJ} * (e^{b_eJ - b_fJ} * (e^{b_fJ - b_s} kh_s)): the inner product is
                    // <= 1 first, so the outer factor can only underflow what is below 1e-38 anyway
                    const float* mv = VEC + V_M + pair_slot(I, J) * DK + kc;
                    const float* cv = VEC + V_C + J * DK + kc;
                    const float4 m0 = *reinterpret_cast<const float4*>(mv);
                    const float4 m1 = *reinterpret_cast<const float4*>(mv + 4);
                    const float4 q0 = *reinterpret_cast<const float4*>(cv);
                    const float4 q1 = *reinterpret_cast<const float4*>(cv + 4);
                    const float mm[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
                    const float cc[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
                    const uint4 rw = __builtin_bit_cast(uint4, raw);
                    const uint32_t wv[4] = {rw.x, rw.y, rw.z, rw.w};
                    uint4 outw;
                    uint32_t* ow = reinterpret_cast<uint32_t*>(&outw);
    #pragma unroll
                    for (int e = 0; e < 4; ++e)
                        ow[e] = pack2((lo_bf(wv[e]) * cc[2 * e]) * mm[2 * e], (hi_bf(wv[e]) * cc[2 * e + 1]) * mm[2 * e + 1]);
                    x = __builtin_bit_cast(bf16x8_t, outw);
                }
                accA[pp] = mfma32(x, ld8(KL, SR, 16 * I + l16, kc), accA[pp]);
                accP[pp] = mfma32(x, ld8(QL, SR, 16 * I + l16, kc), accP[pp]);
            }
        }
        lds_barrier();
        // A (fp32, beta-scaled, strict lower) to LDS; P (bf16, lower incl. diagonal) out.
        // accumulator element e is (s = 16J + 4*g4 + e, r = 16I + l16)
    #pragma unroll
        for (int pp = 0; pp < 3; ++pp) {
            const int pidx = wave + 4 * pp;
            if (pidx >= 10) continue;
            const int I = pI[pp], J = pJ[pp];
            const int r = 16 * I + l16;
            const float br = VEC[V_BETA + r];
            float a4[4], p4[4];
    #pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int sl = 4 * g4 + e;
                const bool below = (I > J) || (sl < l16);
                const bool belowEq = (I > J) || (sl <= l16);
                if constexpr (EJK) {
                    // e^{b_{r-1} - b_s} and e^{b_r - b_s}: at most 1 where kept
                    const int s = 16 * J + sl;
                    const float fa = __builtin_amdgcn_exp2f(VEC[V_BX + r] - VEC[V_B + s]);
                    const float fp = __builtin_amdgcn_exp2f(VEC[V_B + r] - VEC[V_B + s]);
                    a4[e] = below ? br * (accA[pp][e] * fa) : 0.f;
                    p4[e] = belowEq ? accP[pp][e] * fp : 0.f;
                } else {
                    a4[e] = below ? br * accA[pp][e] : 0.f;
                    p4[e] = belowEq ? accP[pp][e] : 0.f;
                }
            }
            *reinterpret_cast<float4*>(AB + r * SA + 16 * J + 4 * g4) = make_float4(a4[0], a4[1], a4[2], a4[3]);
            buf_store(rr, REC_P + 2 * ksl(C, r, 16 * J + 4 * g4), make_uint2(pack2(p4[0], p4[1]), pack2(p4[2], p4[3])));
        }
        lds_barrier();

        // ---------------- phase 3: T = (I + A)^-1, T' = T diag(beta)
        // level 1: diagonal 16x16 inverses by forward substitution (fp32), lane j = column
        // (wave 0 solves all four blocks, lane = 16 * block + column; waves 1 and 2
        // zero the upper blocks the later stages read)
        if (wave == 1 || wave == 2) {
            const int I = 2 * (wave - 1);
            const int r = 16 * I + (lane >> 2);
            const int s = 16 * I + 16 + 4 * (lane & 3);
            st4bf(TP + r * SW + s, 0.f, 0.f, 0.f, 0.f);
            if (I == 0)
                st4bf(TCOL + (16 + (lane >> 2)) * ST + 4 * (lane & 3), 0.f, 0.f, 0.f, 0.f);
            else
                st4bf(TROW + (32 + (lane >> 2)) * ST + 48 + 4 * (lane & 3), 0.f, 0.f, 0.f, 0.f);
        }
        if (wave == 0) {
            const int I = lane >> 4;
            {
                const int j = l16;
                float t[16];
    #pragma unroll
                for (int r = 0; r < 16; ++r) t[r] = (r == j) ? 1.f : 0.f;
                // column-oriented: once t[s] is final it updates every later row, so the
                // dependent chain is 15 steps long instead of 120 (t[s] = 0 for s < j)
                const float* ablk = AB + (16 * I) * SA + 16 * I;
    #pragma unroll
                for (int s = 0; s < 15; ++s) {
                    const float ts = t[s];
    #pragma unroll
                    for (int r = s + 1; r < 16; ++r) t[r] = fmaf(-ablk[r * SA + s], ts, t[r]);
                }
                const float bj = VEC[V_BETA + 16 * I + j];
                uint16_t* tc = TCOL + (16 * I + j) * ST + 16 * I;
    #pragma unroll
                for (int r = 0; r < 16; r += 4) st4bf(tc + r, t[r], t[r + 1], t[r + 2], t[r + 3]);
    #pragma unroll
                for (int r = 0; r < 16; ++r) {
                    st1bf(TROW + (16 * I + r) * ST + 16 * I + j, t[r]);
                    st1bf(TP + (16 * I + r) * SW + 16 * I + j, t[r] * bj);
                }
            }
        }
        lds_barrier();
        // level 2: T10 = -T11 (A10 T00) on wave 0, T32 = -T33 (A32 T22) on wave 1
        if (wave < 2) {
            const int Ib = 2 * wave + 1, Jb = 2 * wave;
            uint16_t* ys = YS + wave * 16 * SY;
            const float4 af = *reinterpret_cast<const float4*>(AB + (16 * Ib + l16) * SA + 16 * Jb + 4 * g4);
            const f32x4_t y = mfma16(f32_to_s16x4(af), ld4(TCOL, ST, 16 * Jb + l16, 16 * Jb + 4 * g4),
                                     f32x4_t{0.f, 0.f, 0.f, 0.f});
            st4bf(ys + l16 * SY + 4 * g4, y[0], y[1], y[2], y[3]);   // column-major Y
            const f32x4_t tt = mfma16(ld4(TROW, ST, 16 * Ib + l16, 16 * Ib + 4 * g4), ld4(ys, SY, l16, 4 * g4),
                                      f32x4_t{0.f, 0.f, 0.f, 0.f});
            const float bj = VEC[V_BETA + 16 * Jb + l16];
    #pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * Ib + 4 * g4 + e;
                st1bf(TP + r * SW + 16 * Jb + l16, -tt[e] * bj);
                if (wave == 1) st1bf(TROW + r * ST + 16 * Jb + l16, -tt[e]);
            }
            if (wave == 0)
                st4bf(TCOL + (16 * Jb + l16) * ST + 16 * Ib + 4 * g4, -tt[0], -tt[1], -tt[2], -tt[3]);
        }
        lds_barrier();
        // level 3: T[32:64, 0:32] = -T_B (A[32:64, 0:32] T_A), one 16x16 tile per wave
        {
            const int ti = wave >> 1, tj = wave & 1;
            f32x4_t y = f32x4_t{0.f, 0.f, 0.f, 0.f};
    #pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const float4 af = *reinterpret_cast<const float4*>(AB + (32 + 16 * ti + l16) * SA + 16 * kk + 4 * g4);
                y = mfma16(f32_to_s16x4(af), ld4(TCOL, ST, 16 * tj + l16, 16 * kk + 4 * g4), y);
            }
            st4bf(YS + (16 * tj + l16) * SY + 16 * ti + 4 * g4, y[0], y[1], y[2], y[3]);
        }
        lds_barrier();
        {
            const int ti = wave >> 1, tj = wave & 1;
            f32x4_t tt = f32x4_t{0.f, 0.f, 0.f, 0.f};
    #pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                tt = mfma16(ld4(TROW, ST, 32 + 16 * ti + l16, 32 + 16 * kk + 4 * g4),
                            ld4(YS, SY, 16 * tj + l16, 16 * kk + 4 * g4), tt);
            const float bj = VEC[V_BETA + 16 * tj + l16];
    #pragma unroll
            for (int e = 0; e < 4; ++e)
                st1bf(TP + (32 + 16 * ti + 4 * g4 + e) * SW + 16 * tj + l16, -tt[e] * bj);
        }
        lds_barrier();

        // ---------------- phase 4: W = T' Kg (as W^T = Kg^T T'^T); T' out
        {
    #pragma unroll
            for (int ibl = 0; ibl < 2; ++ibl) {
                const int ib = 2 * wave + ibl;
    #pragma unroll
                for (int I = 0; I < 4; ++I) {
                    f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
    #pragma unroll
                    for (int ks = 0; ks < 2; ++ks) {
                        if (ks == 1 && I < 2) continue;
                        acc = mfma32(ld8(KGT, SW, 16 * ib + l16, 32 * ks + 8 * g4),
                                     ld8(TP, SW, 16 * I + l16, 32 * ks + 8 * g4), acc);
                    }
                    // acc[e] = W[r = 16I + l16][i = 16ib + 4*g4 + e]
                    buf_store(rr, REC_W + 2 * ksl(C, 16 * I + l16, 16 * ib + 4 * g4),
                              make_uint2(pack2(acc[0], acc[1]), pack2(acc[2], acc[3])));
                }
            }
            // T' [64][64] -> k-sliced, thread = (row, 16-column block); blocks above the
            // diagonal are written as zeros, except k-slice 1 of rows 0..31, which the
            // scan never reads (it loads zeros for it from past the record's end)
            const int r = tid >> 2;
            const int s0 = 16 * (tid & 3);
            const bool upper = (tid & 3) > (r >> 4);
            if (!(r < 32 && s0 >= 32)) {
    #pragma unroll
                for (int h8 = 0; h8 < 2; ++h8) {
                    uint4 val = *reinterpret_cast<const uint4*>(TP + r * SW + s0 + 8 * h8);
                    if (upper) val = make_uint4(0u, 0u, 0u, 0u);
                    buf_store(rr, REC_TP + 2 * ksl(C, r, s0 + 8 * h8), val);
                    if (upper) buf_store(rr, REC_P + 2 * ksl(C, r, s0 + 8 * h8), val);
                }
            }
        }
        // phase 4 of this item reads KGT and TP, which the next item overwrites
        lds_barrier();
    }
}

// ------------------------------------------------------------------------
// chunk_scan: one workgroup of 4 waves per (sequence, head, tile of 16*NJB state
// columns).  Wave w owns row block I = w (rows [16I, 16I+16) of U and O, state
// rows [32I, 32I+32)) for every 16-column block of the tile, so each operand
// fragment is loaded once per workgroup and reused NJB times.  (Eight waves,
// two per row block, measured slower: each fragment is then fetched twice.)
constexpr int SCAN_WAVES = 4;
constexpr int SCAN_THREADS = 64 * SCAN_WAVES;

template <int NJB>
struct ScanShape {
    static constexpr int DVT = 16 * NJB;
    static constexpr int NJW = NJB * 4 / SCAN_WAVES;                // column blocks per wave
    static constexpr int ST_OFF = 0;                                // S0^T bf16 [DVT][SR]
    static constexpr int UT_OFF = ST_OFF + DVT * SR * 2;            // U^T  bf16 [DVT][SW]
    static constexpr int VT_OFF = UT_OFF + DVT * SW * 2;            // V^T  bf16 [DVT][SW]
    static constexpr int LDS = VT_OFF + DVT * SW * 2;
    static constexpr int VSEG = (C * DVT / 8 + SCAN_THREADS - 1) / SCAN_THREADS;   // 16-byte V pieces per thread
    static_assert(NJW >= 1 && NJW * SCAN_WAVES == 4 * NJB, "column blocks split over the waves");
};

template <int NJB>
struct Frags {
    bf16x8_t tp[2];      // T' rows of this wave's 16-row block, k-slices 0..1
    bf16x8_t w[4];       // W  rows, k-slices 0..3
    bf16x8_t qg[4];      // Qg rows, k-slices 0..3
    bf16x8_t p[2];       // P  rows, k-slices 0..1
    bf16x8_t kc[2][2];   // Kc^T rows [32I + 16ib, +16), k-slices 0..1
    float4 ec[2];        // e^{b_C} for the 4 state rows of each ib
    uint4 v[ScanShape<NJB>::VSEG];   // V tile pieces
};

// The loads of one chunk in three parts, issued at the starts of the three
// phases of the previous chunk so that their drain overlaps its compute:
// part 0 = V tile, T', P, e^{b_C}; part 1 = W, Qg; part 2 = Kc^T.
template <int NJB, int PART>
__device__ __forceinline__ void load_frags(Frags<NJB>& f, const unsigned char* rec, const bf16_t* v, int c0,
                                           int len, int HKV, int hk, int DV, int j0, int I, int lane, int tid)
{
    const int l16 = lane & 15, g4 = lane >> 4;
    const int fo = l16 * 32 + 8 * g4;   // lane offset inside a 16x32 fragment
    const uint16_t* W = reinterpret_cast<const uint16_t*>(rec + REC_W);
    const uint16_t* QG = reinterpret_cast<const uint16_t*>(rec + REC_QG);
    const uint16_t* KCT = reinterpret_cast<const uint16_t*>(rec + REC_KCT);
    const float* EC = reinterpret_cast<const float*>(rec + REC_EC);
    if constexpr (PART == 0) {
        // V tile: row s, 8 columns per piece; rows past the sequence read row 0 and are zeroed on use
        constexpr int DVT = ScanShape<NJB>::DVT;
#pragma unroll
        for (int it = 0; it < ScanShape<NJB>::VSEG; ++it) {
            const int seg = tid + it * SCAN_THREADS;
            const int s = min(seg / (DVT / 8), C - 1);
            const int jj = (seg % (DVT / 8)) * 8;
            const int ss = (s < len) ? s : 0;
            f.v[it] = *reinterpret_cast<const uint4*>(v + ((size_t)(c0 + ss) * HKV + hk) * DV + j0 + jj);
        }
        // T' and P are lower triangular: k-slice 1 (columns 32..63) of the first
        // two row blocks is zero and is not stored.  Those two fragments are
        // loaded from past the end of a buffer resource over the record, which
        // returns zeros without a memory request, so every wave issues the same
        // loads and only rows 32..63 fetch them.
        const __amdgpu_buffer_rsrc_t rr =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(rec), 0, REC_BYTES, 0x00020000);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const bool stored = ks == 0 || I >= 2;
            const int tpo = stored ? REC_TP + 2 * ((ks * C + 16 * I) * 32 + fo) : REC_BYTES;
            const int po = stored ? REC_P + 2 * ((ks * C + 16 * I) * 32 + fo) : REC_BYTES;
            f.tp[ks] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(rr, tpo, 0, 0));
            f.p[ks] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(rr, po, 0, 0));
        }
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
            f.ec[ib] = *reinterpret_cast<const float4*>(EC + 32 * I + 16 * ib + 4 * g4);
    } else if constexpr (PART == 1) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            f.w[ks] = *reinterpret_cast<const bf16x8_t*>(W + (ks * C + 16 * I) * 32 + fo);
            f.qg[ks] = *reinterpret_cast<const bf16x8_t*>(QG + (ks * C + 16 * I) * 32 + fo);
        }
    } else {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int ib = 0; ib < 2; ++ib)
                f.kc[ib][ks] = *reinterpret_cast<const bf16x8_t*>(KCT + (ks * DK + 32 * I + 16 * ib) * 32 + fo);
    }
}

template <int NJB, typename Tout>
__global__ __launch_bounds__(SCAN_THREADS) void chunk_scan_kernel(
    const bf16_t* __restrict__ v, const float* __restrict__ init, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ off, const int32_t* __restrict__ order, int N, int T, int ts, int H, int HKV, int DV,
    int nslots, const unsigned char* __restrict__ ws, Tout* __restrict__ o, float* __restrict__ final_state)
{
    using Sh = ScanShape<NJB>;
    constexpr int DVT = Sh::DVT;
    constexpr int NJW = Sh::NJW;
    __shared__ __attribute__((aligned(16))) unsigned char smem[Sh::LDS];
    uint16_t* STB = reinterpret_cast<uint16_t*>(smem + Sh::ST_OFF);
    uint16_t* UT = reinterpret_cast<uint16_t*>(smem + Sh::UT_OFF);
    uint16_t* VT = reinterpret_cast<uint16_t*>(smem + Sh::VT_OFF);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int I = wave & 3;              // row block
    const int jb0 = (wave >> 2) * NJW;   // first of this wave's column blocks
    const int l16 = lane & 15;
    const int g4 = lane >> 4;

    // XCD-aware placement: the column tiles of one (sequence, head) share an XCD and its L2
    const int ntiles = DV / DVT;
    const int units = N * H;
    const int xcd = blockIdx.x & 7;
    const int w8 = blockIdx.x >> 3;
    const int tile = w8 % ntiles;
    const int urank = (w8 / ntiles) * 8 + xcd;
    if (urank >= units) return;
    const int nrank = urank / H;
    const int h = urank - nrank * H;
    const int n = order ? order[nrank] : nrank;   // packed batches: longest sequences first
    const int unit = n * H + h;
    const int hk = h / (H / HKV);   // the key/value head of head h
    const int j0 = tile * DVT;

    int t_begin, t_end;
    seq_bounds(cu, n, T, ts, t_begin, t_end);
    const int slot0 = off ? off[n] : n * ((T + C - 1) / C);
    // Valid cu_seqlens never need the clamp: a packed batch has at most T / C + N
    // chunks.  Overlapping ranges (a decreasing pair) can count more; their
    // chunks past the workspace's slots are not read (those results are
    // undefined, the memory accesses stay inside the buffers).
    const int nch = max(0, min((t_end - t_begin + C - 1) / C, nslots - slot0));

    // state: rows [32I, 32I+32) x this wave's NJW column blocks
    f32x4_t S[2][NJW];
    const size_t soff = (size_t)unit * DK * DV;
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int jw = 0; jw < NJW; ++jw)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 32 * I + 16 * ib + 4 * g4 + e;
                const int j = j0 + 16 * (jb0 + jw) + l16;
                S[ib][jw][e] = init ? init[soff + (size_t)i * DV + j] : 0.f;
            }
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int jw = 0; jw < NJW; ++jw)
            st4bf(STB + (16 * (jb0 + jw) + l16) * SR + 32 * I + 16 * ib + 4 * g4, S[ib][jw][0], S[ib][jw][1],
                  S[ib][jw][2], S[ib][jw][3]);

    // One chunk: U = T' V - W S0, O = Qg S0 + P U, S = Diag(e^{b_C}) S0 + Kc^T U.
    // Operands are prefetched one chunk ahead into two register sets used in
    // turn (the loop is unrolled by two, so no set is ever copied), in three
    // parts issued at the starts of the current chunk's three phases: a CU's
    // outstanding misses bound how fast a chunk's 64.5 KiB arrive, and spread
    // out, that drain overlaps the compute instead of stalling issue before it.
    // Every prefetch is issued (past the end it reloads the last chunk), so the
    // outstanding-load count is the same on every path and the wait before a
    // chunk's first use only covers that chunk's own loads.
    auto prefetch = [&](auto part, Frags<NJB>& f, int c) {
        const int cc = min(c, nch - 1);
        const int c0 = t_begin + cc * C;
        load_frags<NJB, decltype(part)::value>(f, ws + ((size_t)(slot0 + cc) * H + h) * REC_BYTES, v, c0,
                                               min(C, t_end - c0), HKV, hk, DV, j0, I, lane, tid);
    };
    using Part0 = std::integral_constant<int, 0>;
    using Part1 = std::integral_constant<int, 1>;
    using Part2 = std::integral_constant<int, 2>;
    auto step = [&](const Frags<NJB>& cur, Frags<NJB>& nxt, int c) {
        const int c0 = t_begin + c * C;
        // a step past the last chunk (the padding, or the clamp above) has no rows
        const int len = c < nch ? min(C, t_end - c0) : 0;
        prefetch(Part0{}, nxt, c + 1);
        // V tile, transposed: VT[j][s]
#pragma unroll
        for (int it = 0; it < Sh::VSEG; ++it) {
            const int seg = tid + it * SCAN_THREADS;
            if ((C * DVT / 8) % SCAN_THREADS == 0 || seg < C * DVT / 8) {
                const int s = seg / (DVT / 8);
                const int jj = (seg % (DVT / 8)) * 8;
                const bool in = s < len;
                const uint32_t w4[4] = {in ? cur.v[it].x : 0u, in ? cur.v[it].y : 0u, in ? cur.v[it].z : 0u,
                                        in ? cur.v[it].w : 0u};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    VT[(jj + 2 * e) * SW + s] = (uint16_t)(w4[e] & 0xffff);
                    VT[(jj + 2 * e + 1) * SW + s] = (uint16_t)(w4[e] >> 16);
                }
            }
        }
        lds_barrier();

        prefetch(Part1{}, nxt, c + 1);
        // U = T' V - W S0 and the S0 part of O^T = S0^T Qg^T, per 16-column block
        f32x4_t O[NJW];
#pragma unroll
        for (int jw = 0; jw < NJW; ++jw) {
            const int jb = jb0 + jw;
            bf16x8_t sb[4], vt[2];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) sb[ks] = ld8(STB, SR, 16 * jb + l16, 32 * ks + 8 * g4);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) vt[ks] = ld8(VT, SW, 16 * jb + l16, 32 * ks + 8 * g4);
            const f32x4_t z = f32x4_t{0.f, 0.f, 0.f, 0.f};
            // two partial sums per product halve the dependent MFMA chains
            f32x4_t w0 = mfma32(cur.w[0], sb[0], z), w1 = mfma32(cur.w[1], sb[1], z);
            f32x4_t o0 = mfma32(sb[0], cur.qg[0], z), o1 = mfma32(sb[1], cur.qg[1], z);
            f32x4_t u0 = mfma32(cur.tp[0], vt[0], z), u1 = mfma32(cur.tp[1], vt[1], z);
            w0 = mfma32(cur.w[2], sb[2], w0);
            w1 = mfma32(cur.w[3], sb[3], w1);
            o0 = mfma32(sb[2], cur.qg[2], o0);
            o1 = mfma32(sb[3], cur.qg[3], o1);
            O[jw] = o0 + o1;
            const f32x4_t u = (u0 + u1) - (w0 + w1);   // U[s = 16I + 4*g4 + e][j = 16jb + l16]
            st4bf(UT + (16 * jb + l16) * SW + 16 * I + 4 * g4, u[0], u[1], u[2], u[3]);
        }
        lds_barrier();

        prefetch(Part2{}, nxt, c + 1);
        // O^T += U^T P^T;  S = Diag(e^{b_C}) S0 + Kc^T U
        const int r = 16 * I + l16;
#pragma unroll
        for (int jw = 0; jw < NJW; ++jw) {
            const int jb = jb0 + jw;
            bf16x8_t ut[2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) ut[ks] = ld8(UT, SW, 16 * jb + l16, 32 * ks + 8 * g4);
            const f32x4_t z = f32x4_t{0.f, 0.f, 0.f, 0.f};
            f32x4_t a0 = mfma32(ut[0], cur.p[0], O[jw]);
            f32x4_t d0 = mfma32(cur.kc[0][0], ut[0], z);
            f32x4_t d1 = mfma32(cur.kc[1][0], ut[0], z);
            a0 = mfma32(ut[1], cur.p[1], a0);
            d0 = mfma32(cur.kc[0][1], ut[1], d0);
            d1 = mfma32(cur.kc[1][1], ut[1], d1);
            // a0[e] = O[r = 16I + l16][j = 16jb + 4*g4 + e]
            if (r < len) {
                Tout* op = o + ((size_t)(c0 + r) * H + h) * DV + j0 + 16 * jb + 4 * g4;
                if constexpr (sizeof(Tout) == 2) {
                    *reinterpret_cast<uint2*>(op) = make_uint2(pack2(a0[0], a0[1]), pack2(a0[2], a0[3]));
                } else {
                    *reinterpret_cast<float4*>(op) = make_float4(a0[0], a0[1], a0[2], a0[3]);
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                S[0][jw][e] = (c < nch) ? fmaf(cur.ec[0][e], S[0][jw][e], d0[e]) : S[0][jw][e];
                S[1][jw][e] = (c < nch) ? fmaf(cur.ec[1][e], S[1][jw][e], d1[e]) : S[1][jw][e];
            }
            // S0^T is only read before the previous barrier, so the new state's bf16
            // copy can go in now; the next chunk's first barrier publishes it.
#pragma unroll
            for (int ib = 0; ib < 2; ++ib)
                st4bf(STB + (16 * jb + l16) * SR + 32 * I + 16 * ib + 4 * g4, S[ib][jw][0], S[ib][jw][1],
                      S[ib][jw][2], S[ib][jw][3]);
        }
    };
    if (nch > 0) {
        Frags<NJB> fa, fb;
        // in the loop's issue order, so that its waits count the same way on entry
        prefetch(Part0{}, fa, 0);
        __builtin_amdgcn_sched_barrier(0);
        prefetch(Part1{}, fa, 0);
        __builtin_amdgcn_sched_barrier(0);
        prefetch(Part2{}, fa, 0);
        __builtin_amdgcn_sched_barrier(0);
        // the chunk count is padded to even; a step past the end (len 0) stores
        // nothing and leaves the state as it is
        for (int c = 0; c < nch; c += 2) {
            step(fa, fb, c);
            step(fb, fa, c + 1);
        }
    }

    if (final_state) {
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
            for (int jw = 0; jw < NJW; ++jw)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 32 * I + 16 * ib + 4 * g4 + e;
                    const int j = j0 + 16 * (jb0 + jw) + l16;
                    final_state[soff + (size_t)i * DV + j] = S[ib][jw][e];
                }
    }
}

// workspace: [chunk offsets (N + 1 ints, padded)][records: slots x H x REC_BYTES]
// packed plan: off[N + 1] then order[N], int32
size_t offsets_bytes(int N) { return ((size_t)(2 * N + 1) * 4 + OFFSETS_BYTES_ALIGN - 1) / OFFSETS_BYTES_ALIGN * OFFSETS_BYTES_ALIGN; }

size_t max_slots(int N, int T, bool packed)
{
    if (packed) return (size_t)(T / C) + (size_t)N;   // each sequence adds at most one partial chunk
    return (size_t)N * (size_t)((T + C - 1) / C);
}

// 16-column blocks per scan workgroup.  Every workgroup loads a whole
// record per chunk, and a CU's outstanding misses bound how fast it can, so
// the widest tile that still gives at least one workgroup per CU wins: narrow
// tiles put more chains on the chip, wide tiles load each record fewer times.
int scan_tile_blocks(int N, int H, int dv)
{
    const long units = (long)N * H;
    for (int njb = 4; njb > 1; njb >>= 1)
        if (dv % (16 * njb) == 0 && units * (dv / (16 * njb)) >= 256) return njb;
    return 1;
}

template <typename Tout>
hipError_t launch_typed(const PrefillArgs& a, hipStream_t stream)
{
    const bool packed = a.cu != nullptr;
    const int ts = a.tstride > 0 ? a.tstride : a.T;   // dense: rows between sequence starts
    unsigned char* wsb = static_cast<unsigned char*>(a.workspace);
    int32_t* off = nullptr;
    int32_t* order = nullptr;
    unsigned char* recs = wsb;
    if (packed) {
        off = reinterpret_cast<int32_t*>(wsb);
        recs = wsb + offsets_bytes(a.N);
        order = off + a.N + 1;
        hipLaunchKernelGGL(chunk_plan_kernel, dim3(1), dim3(PLAN_THREADS), 0, stream, a.cu, a.N, a.T, off, order);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const size_t slots = max_slots(a.N, a.T, packed);
    if (slots > 0) {
        // persistent: two workgroups per CU (the LDS limit), at most one per item
        const size_t items = slots * (size_t)a.H;
        const dim3 pgrid((unsigned)std::min<size_t>(items, 2 * 256));
        const bf16_t* qq = static_cast<const bf16_t*>(a.q);
        const bf16_t* kk = static_cast<const bf16_t*>(a.k);
        if (a.ejk)
            hipLaunchKernelGGL(chunk_prep_kernel<true>, pgrid, dim3(NTHREADS), 0, stream, qq, kk, a.g, a.beta,
                               a.a_log, a.dt_bias, a.cu, off, a.N, a.T, ts, a.H, a.Hkv, (int)slots, a.scale,
                               a.lower_bound, (int)a.l2norm, recs);
        else
            hipLaunchKernelGGL(chunk_prep_kernel<false>, pgrid, dim3(NTHREADS), 0, stream, qq, kk, a.g, a.beta,
                               a.a_log, a.dt_bias, a.cu, off, a.N, a.T, ts, a.H, a.Hkv, (int)slots, a.scale,
                               a.lower_bound, (int)a.l2norm, recs);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int units = a.N * a.H;
    const unsigned groups = (unsigned)((units + 7) / 8);
    const int njb = scan_tile_blocks(a.N, a.H, a.dv);
    const unsigned ntiles = (unsigned)(a.dv / (16 * njb));
    const dim3 grid(groups * 8u * ntiles);
    const bf16_t* vv = static_cast<const bf16_t*>(a.v);
    Tout* oo = static_cast<Tout*>(a.o);
    if (njb == 4)
        hipLaunchKernelGGL((chunk_scan_kernel<4, Tout>), grid, dim3(SCAN_THREADS), 0, stream, vv, a.init, a.cu, off,
                           order, a.N, a.T, ts, a.H, a.Hkv, a.dv, (int)slots, recs, oo, a.final_state);
    else if (njb == 2)
        hipLaunchKernelGGL((chunk_scan_kernel<2, Tout>), grid, dim3(SCAN_THREADS), 0, stream, vv, a.init, a.cu, off,
                           order, a.N, a.T, ts, a.H, a.Hkv, a.dv, (int)slots, recs, oo, a.final_state);
    else
        hipLaunchKernelGGL((chunk_scan_kernel<1, Tout>), grid, dim3(SCAN_THREADS), 0, stream, vv, a.init, a.cu, off,
                           order, a.N, a.T, ts, a.H, a.Hkv, a.dv, (int)slots, recs, oo, a.final_state);
    return hipGetLastError();
}

}  // namespace

bool chunked_supported(const PrefillArgs& a)
{
    return a.in_bf16 && a.dk == DK && a.dv % DV_MULT == 0 && (a.ejk || (a.g != nullptr && a.a_log != nullptr));
}

size_t chunked_workspace_bytes(int N, int T, int H, int dk, int dv, bool packed)
{
    if (dk != DK || dv % DV_MULT != 0 || N <= 0 || T <= 0) return 0;
    return (packed ? offsets_bytes(N) : 0) + max_slots(N, T, packed) * (size_t)H * REC_BYTES;
}

size_t chunked_min_workspace_bytes(int N, int H, int dk, int dv, bool carry)
{
    if (dk != DK || dv % DV_MULT != 0 || N <= 0) return 0;
    const size_t st = carry ? ((size_t)N * H * dk * dv * 4 + 255) / 256 * 256 : 0;
    return st + (size_t)N * H * REC_BYTES;
}

hipError_t launch_chunked(const PrefillArgs& a, hipStream_t stream)
{
    auto one = [&](const PrefillArgs& s) {
        return s.out_bf16 ? launch_typed<bf16_t>(s, stream) : launch_typed<float>(s, stream);
    };
    const bool packed = a.cu != nullptr;
    if (packed || a.workspace_bytes >= chunked_workspace_bytes(a.N, a.T, a.H, a.dk, a.dv, packed)) return one(a);
    // Dense rows and a workspace below the whole call's records: segments of
    // whole chunks of every sequence, each segment's final state the next
    // one's initial state (in final_state, or without one in the workspace's
    // first bytes).  Chunks start at the same rows as in one call, and the
    // state passes through in float32, so the result is the same bit for bit.
    const bool carry = a.final_state == nullptr;
    const size_t st = carry ? ((size_t)a.N * a.H * a.dk * a.dv * 4 + 255) / 256 * 256 : 0;
    unsigned char* w = static_cast<unsigned char*>(a.workspace);
    float* state = carry ? reinterpret_cast<float*>(w) : a.final_state;
    const size_t avail = a.workspace_bytes > st ? a.workspace_bytes - st : 0;
    const size_t per_chunk = (size_t)a.N * a.H * REC_BYTES;
    const size_t nchunk = (size_t)(a.T + C - 1) / C;
    const int seg = (int)std::min(avail / per_chunk, nchunk) * C;
    if (seg <= 0) return hipErrorInvalidValue;   // below chunked_min_workspace_bytes (checked by the caller)
    const size_t so = a.out_bf16 ? 2 : 4;
    for (int ta = 0; ta < a.T; ta += seg) {
        PrefillArgs s = a;
        s.T = std::min(seg, a.T - ta);
        s.tstride = a.T;
        const size_t r = (size_t)ta;   // first row of the segment in every sequence
        s.q = static_cast<const unsigned char*>(a.q) + r * a.H * a.dk * 2;
        s.k = static_cast<const unsigned char*>(a.k) + r * a.Hkv * a.dk * 2;
        s.v = static_cast<const unsigned char*>(a.v) + r * a.Hkv * a.dv * 2;
        s.g = a.g ? a.g + r * a.H * (a.ejk ? 1 : a.dk) : nullptr;
        s.beta = a.beta + r * a.H;
        s.o = static_cast<unsigned char*>(a.o) + r * a.H * a.dv * so;
        s.init = ta == 0 ? a.init : state;
        s.final_state = state;
        s.workspace = w + st;
        s.workspace_bytes = avail;
        const hipError_t e = one(s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace kda
