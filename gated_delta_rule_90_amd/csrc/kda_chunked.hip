// kda_chunked.hip - chunk-parallel KDA prefill on gfx950 MFMA (ejkernel
// "kernel_delta_attention": chunked mode, "Parallel within chunks", default
// chunk_size 64).
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
// Every product is a bf16 MFMA (v_mfma_f32_16x16x32_bf16; 16x16x16 for the
// small triangular merges) with fp32 accumulation; S stays fp32 in registers
// and only its bf16 operand copy sits in LDS.
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
// Work split: one workgroup (4 waves) per (sequence, head, 32-column tile of
// dv); chunks run sequentially inside it.  Tiles of one (sequence, head) are
// placed on one XCD so their shared q/k/g reads hit the same L2.
// Rows of a partial last chunk are padded with exact neutral values
// (q = k = v = 0, gamma = 0, beta = 0) and never stored, so a packed varlen
// batch gives bitwise the same result as each sequence alone.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int C = 64;        // chunk length
constexpr int DK = 128;      // key dimension handled by this kernel
constexpr int DVT = 32;      // state columns per workgroup
constexpr int NJB = DVT / 16;
constexpr int NTHREADS = 256;

// LDS row strides, in elements
constexpr int SR = DK + 8;   // [64][DK] bf16 tiles (272 B rows)
constexpr int SW = C + 8;    // [*][64] bf16 tiles (144 B rows)
constexpr int SA = C + 4;    // A, fp32 [64][64]
constexpr int ST = C + 4;    // Tcol / Trow bf16 [64][64] (136 B rows, 8 B aligned)
constexpr int SY = 40;       // [32][32] bf16 scratch

// LDS map (bytes).  Buffers marked "->" are reused once their first tenant is dead.
constexpr int TILE_R = C * SR * 2;                  // 17408
constexpr int OFF_QL = 0;                           // QL  -> T' [64][SW] + Y scratch
constexpr int OFF_KL = OFF_QL + TILE_R;             // KL  -> Tcol, Trow -> W
constexpr int OFF_KRD = OFF_KL + TILE_R;            // KRd -> A (fp32)
constexpr int OFF_KRO = OFF_KRD + TILE_R;           // KRo -> P [64][SW]
constexpr int OFF_QG = OFF_KRO + TILE_R;            // Qg
constexpr int OFF_KGT = OFF_QG + TILE_R;            // Kg^T [DK][SW]
constexpr int OFF_KCT = OFF_KGT + DK * SW * 2;      // Kc^T [DK][SW]
constexpr int OFF_VT = OFF_KCT + DK * SW * 2;       // V^T  [DVT][SW]
constexpr int OFF_UT = OFF_VT + DVT * SW * 2;       // U^T  [DVT][SW]
constexpr int OFF_ST = OFF_UT + DVT * SW * 2;       // S0^T [DVT][SR] (bf16 operand copy)
constexpr int OFF_VEC = OFF_ST + DVT * SR * 2;      // fp32 vectors below
constexpr int V_BETA = 0, V_NQ = 64, V_NK = 128, V_BT = 192, V_M = V_BT + 4 * DK, V_EC = V_M + 6 * DK;
constexpr int VEC_FLOATS = V_EC + DK;
constexpr int LDS_BYTES = OFF_VEC + VEC_FLOATS * 4;
// reuse inside dead tiles
constexpr int OFF_TP = OFF_QL;                      // T' bf16 [64][SW]
constexpr int OFF_Y = OFF_QL + C * SW * 2;          // Y scratch: 2 x [16][SY] (level 2), [32][SY] (level 3)
constexpr int OFF_TCOL = OFF_KL;                    // bf16 [64][ST], column-major copy of T
constexpr int OFF_TROW = OFF_KL + C * ST * 2;       // bf16 [64][ST], row-major copy of T
constexpr int OFF_W = OFF_KL;                       // W bf16 [64][SR]
constexpr int OFF_A = OFF_KRD;                      // fp32 [64][SA]
constexpr int OFF_P = OFF_KRO;                      // bf16 [64][SW]
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
static_assert(C * SA * 4 <= TILE_R, "A fits in a tile slot");
static_assert(2 * C * ST * 2 <= TILE_R, "Tcol + Trow fit in a tile slot");
static_assert(C * SW * 2 + 2 * 16 * SY * 2 <= TILE_R && C * SW * 2 + 32 * SY * 2 <= TILE_R, "T' + scratch");

__device__ __forceinline__ uint32_t pack2(float a, float b)
{
    const uint32_t lo = __builtin_bit_cast(uint16_t, (__bf16)a);
    const uint32_t hi = __builtin_bit_cast(uint16_t, (__bf16)b);
    return lo | (hi << 16);
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

// Sum 16 per-row partials over the 64 lanes of a wave.  On return lane l
// holds the total of row (l >> 2).
__device__ __forceinline__ float rowsum16(float (&a)[16], int lane)
{
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const bool hi = lane & 32;
        const float send = hi ? a[k] : a[k + 8];
        const float keep = hi ? a[k + 8] : a[k];
        a[k] = keep + __shfl_xor(send, 32, kWave);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const bool hi = lane & 16;
        const float send = hi ? a[k] : a[k + 4];
        const float keep = hi ? a[k + 4] : a[k];
        a[k] = keep + __shfl_xor(send, 16, kWave);
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const bool hi = lane & 8;
        const float send = hi ? a[k] : a[k + 2];
        const float keep = hi ? a[k + 2] : a[k];
        a[k] = keep + __shfl_xor(send, 8, kWave);
    }
    {
        const bool hi = lane & 4;
        const float send = hi ? a[0] : a[1];
        const float keep = hi ? a[1] : a[0];
        a[0] = keep + __shfl_xor(send, 4, kWave);
    }
    float s = a[0];
    s += __shfl_xor(s, 2, kWave);
    s += __shfl_xor(s, 1, kWave);
    return s;
}

// index of the off-diagonal pair (I, J), I > J, in the M-vector table
__device__ __forceinline__ int pair_slot(int I, int J) { return I * (I - 1) / 2 + J; }

template <typename Tout>
__global__ __launch_bounds__(NTHREADS) void chunked_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, const float* __restrict__ a_log,
    const float* __restrict__ dt_bias, const float* __restrict__ init,
    const int32_t* __restrict__ cu, int N, int T, int H, int DV, float scale, float lower_bound,
    int l2norm, Tout* __restrict__ o, float* __restrict__ final_state)
{
    __shared__ __attribute__((aligned(16))) unsigned char smem[LDS_BYTES];
    uint16_t* QL = reinterpret_cast<uint16_t*>(smem + OFF_QL);
    uint16_t* KL = reinterpret_cast<uint16_t*>(smem + OFF_KL);
    uint16_t* KRD = reinterpret_cast<uint16_t*>(smem + OFF_KRD);
    uint16_t* KRO = reinterpret_cast<uint16_t*>(smem + OFF_KRO);
    uint16_t* QG = reinterpret_cast<uint16_t*>(smem + OFF_QG);
    uint16_t* KGT = reinterpret_cast<uint16_t*>(smem + OFF_KGT);
    uint16_t* KCT = reinterpret_cast<uint16_t*>(smem + OFF_KCT);
    uint16_t* VT = reinterpret_cast<uint16_t*>(smem + OFF_VT);
    uint16_t* UT = reinterpret_cast<uint16_t*>(smem + OFF_UT);
    uint16_t* STB = reinterpret_cast<uint16_t*>(smem + OFF_ST);
    float* VEC = reinterpret_cast<float*>(smem + OFF_VEC);
    uint16_t* TP = reinterpret_cast<uint16_t*>(smem + OFF_TP);
    uint16_t* YS = reinterpret_cast<uint16_t*>(smem + OFF_Y);
    uint16_t* TCOL = reinterpret_cast<uint16_t*>(smem + OFF_TCOL);
    uint16_t* TROW = reinterpret_cast<uint16_t*>(smem + OFF_TROW);
    uint16_t* WB = reinterpret_cast<uint16_t*>(smem + OFF_W);
    float* AB = reinterpret_cast<float*>(smem + OFF_A);
    uint16_t* PB = reinterpret_cast<uint16_t*>(smem + OFF_P);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l16 = lane & 15;       // MFMA row / column within a 16-tile
    const int g4 = lane >> 4;        // MFMA k-group / output row group

    // XCD-aware placement: the dv tiles of one (sequence, head) share an XCD
    const int ntiles = DV / DVT;
    const int units = N * H;
    const int xcd = blockIdx.x & 7;
    const int w8 = blockIdx.x >> 3;
    const int tile = w8 % ntiles;
    const int unit = (w8 / ntiles) * 8 + xcd;
    if (unit >= units) return;
    const int n = unit / H;
    const int h = unit - n * H;
    const int j0 = tile * DVT;

    int t_begin, t_end;
    if (cu) {
        t_begin = min(max(cu[n], 0), T);
        t_end = min(max(cu[n + 1], t_begin), T);
    } else {
        t_begin = n * T;
        t_end = t_begin + T;
    }

    // per-lane gate constants: this lane owns key channels 2*lane, 2*lane+1 in the prologue
    const int ch = 2 * lane;
    const float ea = expf(a_log[h]) * kLog2e;          // exp(a_log) folded with log2(e)
    const float dtb0 = dt_bias ? dt_bias[(size_t)ch * H + h] : 0.f;
    const float dtb1 = dt_bias ? dt_bias[(size_t)(ch + 1) * H + h] : 0.f;
    const float lb2 = lower_bound * kLog2e;             // gamma in log2 units

    // state: wave w owns rows i in [32w, 32w+32) as 2 x NJB accumulator tiles
    f32x4_t S[2][NJB];
    const size_t soff = (size_t)unit * DK * DV;
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 32 * wave + 16 * ib + 4 * g4 + e;
                const int j = j0 + 16 * jb + l16;
                S[ib][jb][e] = init ? init[soff + (size_t)i * DV + j] : 0.f;
            }
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb)
            st4bf(STB + (16 * jb + l16) * SR + 32 * wave + 16 * ib + 4 * g4, S[ib][jb][0], S[ib][jb][1],
                  S[ib][jb][2], S[ib][jb][3]);

    for (int c0 = t_begin; c0 < t_end; c0 += C) {
        const int len = min(C, t_end - c0);

        // ---------------- phase 1a: loads, partial norms, gate, in-block cumsum
        uint32_t qraw[16], kraw[16];
        float cb0[16], cb1[16], sq[16], sk[16];
        {
            const int blk = wave;
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                const int r = 16 * blk + m;
                uint32_t qq = 0, kk = 0;
                float g0 = 0.f, g1 = 0.f;
                const bool valid = r < len;
                if (valid) {
                    const size_t base = ((size_t)(c0 + r) * H + h) * DK + ch;
                    qq = *reinterpret_cast<const uint32_t*>(q + base);
                    kk = *reinterpret_cast<const uint32_t*>(k + base);
                    const float2 gg = *reinterpret_cast<const float2*>(g + base);
                    g0 = gg.x;
                    g1 = gg.y;
                }
                qraw[m] = qq;
                kraw[m] = kk;
                const float q0 = lo_bf(qq), q1 = hi_bf(qq), k0 = lo_bf(kk), k1 = hi_bf(kk);
                sq[m] = q0 * q0 + q1 * q1;
                sk[m] = k0 * k0 + k1 * k1;
                // gamma' = lb * log2(e) * sigmoid(exp(a_log) * (g + dt_bias))
                const float e0 = __builtin_amdgcn_exp2f(-ea * (g0 + dtb0));
                const float e1 = __builtin_amdgcn_exp2f(-ea * (g1 + dtb1));
                const float gm0 = valid ? lb2 * __builtin_amdgcn_rcpf(1.f + e0) : 0.f;
                const float gm1 = valid ? lb2 * __builtin_amdgcn_rcpf(1.f + e1) : 0.f;
                cb0[m] = (m == 0 ? 0.f : cb0[m - 1]) + gm0;
                cb1[m] = (m == 0 ? 0.f : cb1[m - 1]) + gm1;
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
                VEC[V_BETA + r] = (r < len) ? sigmoid_f(beta[(size_t)(c0 + r) * H + h]) : 0.f;
            }
            // V tile, transposed: VT[j][s]
#pragma unroll
            for (int it = 0; it < (C * DVT / 8) / NTHREADS; ++it) {
                const int seg = tid + it * NTHREADS;
                const int s = seg / (DVT / 8);
                const int jj = (seg % (DVT / 8)) * 8;
                uint4 vv = make_uint4(0, 0, 0, 0);
                if (s < len) vv = *reinterpret_cast<const uint4*>(v + ((size_t)(c0 + s) * H + h) * DV + j0 + jj);
                const uint32_t w4[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    VT[(jj + 2 * e) * SW + s] = (uint16_t)(w4[e] & 0xffff);
                    VT[(jj + 2 * e + 1) * SW + s] = (uint16_t)(w4[e] >> 16);
                }
            }
        }
        __syncthreads();

        // ---------------- phase 1b: decay factors and the seven operand tiles
        {
            const int blk = wave;
            float P0 = 0.f, P1 = 0.f, tot0 = 0.f, tot1 = 0.f;
            float pre0[4], pre1[4];   // prefix (b at the end of block J) for J < 4
#pragma unroll
            for (int J = 0; J < 4; ++J) {
                const float t0 = VEC[V_BT + J * DK + ch], t1 = VEC[V_BT + J * DK + ch + 1];
                if (J < blk) { P0 += t0; P1 += t1; }
                tot0 += t0;
                tot1 += t1;
                pre0[J] = tot0;
                pre1[J] = tot1;
            }
            // b (log2 units) at the first row of this block, and the per-block vectors
            const float bf0 = P0 + cb0[0], bf1 = P1 + cb1[0];
            const float E0 = __builtin_amdgcn_exp2f(bf0), E1 = __builtin_amdgcn_exp2f(bf1);
            const float c_0 = __builtin_amdgcn_exp2f(cb0[15] - cb0[0]);
            const float c_1 = __builtin_amdgcn_exp2f(cb1[15] - cb1[0]);
            const float N0 = __builtin_amdgcn_exp2f(tot0 - pre0[blk]);
            const float N1 = __builtin_amdgcn_exp2f(tot1 - pre1[blk]);
#pragma unroll
            for (int J = 0; J < 3; ++J) {
                if (J < blk) {
                    const int slot = pair_slot(blk, J);
                    VEC[V_M + slot * DK + ch] = __builtin_amdgcn_exp2f(bf0 - pre0[J]);
                    VEC[V_M + slot * DK + ch + 1] = __builtin_amdgcn_exp2f(bf1 - pre1[J]);
                }
            }
            if (blk == 0) {
                VEC[V_EC + ch] = __builtin_amdgcn_exp2f(tot0);
                VEC[V_EC + ch + 1] = __builtin_amdgcn_exp2f(tot1);
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
                const float ko0 = c_0 * kd0, ko1 = c_1 * kd1;
                const int at = r * SR + ch;
                *reinterpret_cast<uint32_t*>(QL + at) = pack2(ql0, ql1);
                *reinterpret_cast<uint32_t*>(KL + at) = pack2(kl0, kl1);
                *reinterpret_cast<uint32_t*>(KRD + at) = pack2(kd0, kd1);
                *reinterpret_cast<uint32_t*>(KRO + at) = pack2(ko0, ko1);
                *reinterpret_cast<uint32_t*>(QG + at) = pack2(E0 * ql0, E1 * ql1);
                kg0[m] = E0 * kl0;
                kg1[m] = E1 * kl1;
                kc0[m] = N0 * ko0;
                kc1[m] = N1 * ko1;
            }
            // transposed tiles: 16 consecutive tokens of one channel = 32 contiguous bytes
            uint16_t* g0p = KGT + ch * SW + 16 * blk;
            uint16_t* g1p = KGT + (ch + 1) * SW + 16 * blk;
            uint16_t* c0p = KCT + ch * SW + 16 * blk;
            uint16_t* c1p = KCT + (ch + 1) * SW + 16 * blk;
#pragma unroll
            for (int h8 = 0; h8 < 2; ++h8) {
                const int m = 8 * h8;
                *reinterpret_cast<uint4*>(g0p + m) = make_uint4(pack2(kg0[m], kg0[m + 1]), pack2(kg0[m + 2], kg0[m + 3]), pack2(kg0[m + 4], kg0[m + 5]), pack2(kg0[m + 6], kg0[m + 7]));
                *reinterpret_cast<uint4*>(g1p + m) = make_uint4(pack2(kg1[m], kg1[m + 1]), pack2(kg1[m + 2], kg1[m + 3]), pack2(kg1[m + 4], kg1[m + 5]), pack2(kg1[m + 6], kg1[m + 7]));
                *reinterpret_cast<uint4*>(c0p + m) = make_uint4(pack2(kc0[m], kc0[m + 1]), pack2(kc0[m + 2], kc0[m + 3]), pack2(kc0[m + 4], kc0[m + 5]), pack2(kc0[m + 6], kc0[m + 7]));
                *reinterpret_cast<uint4*>(c1p + m) = make_uint4(pack2(kc1[m], kc1[m + 1]), pack2(kc1[m + 2], kc1[m + 3]), pack2(kc1[m + 4], kc1[m + 5]), pack2(kc1[m + 6], kc1[m + 7]));
            }
        }
        __syncthreads();

        // ---------------- phase 2: A and P on 16x16 block pairs (I >= J)
        // pair order: diagonal blocks, then distance 1, 2, 3
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
                bf16x8_t x;
                if (I == J) {
                    x = ld8(KRD, SR, 16 * J + l16, kc);
                } else {
                    const bf16x8_t raw = ld8(KRO, SR, 16 * J + l16, kc);
                    const float* mv = VEC + V_M + pair_slot(I, J) * DK + kc;
                    const float4 m0 = *reinterpret_cast<const float4*>(mv);
                    const float4 m1 = *reinterpret_cast<const float4*>(mv + 4);
                    const float mm[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] = (__bf16)((float)raw[e] * mm[e]);
                }
                accA[pp] = mfma32(x, ld8(KL, SR, 16 * I + l16, kc), accA[pp]);
                accP[pp] = mfma32(x, ld8(QL, SR, 16 * I + l16, kc), accP[pp]);
            }
        }
        __syncthreads();
        // store A (fp32, beta-scaled, strict lower) and P (bf16, lower incl. diagonal).
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
                a4[e] = below ? br * accA[pp][e] : 0.f;
                p4[e] = belowEq ? accP[pp][e] : 0.f;
            }
            *reinterpret_cast<float4*>(AB + r * SA + 16 * J + 4 * g4) = make_float4(a4[0], a4[1], a4[2], a4[3]);
            st4bf(PB + r * SW + 16 * J + 4 * g4, p4[0], p4[1], p4[2], p4[3]);
        }
        // P blocks (0,1) and (2,3) are read by the 32-wide k-steps: zero them
        if (wave == 0 || wave == 2) {
            const int r = 16 * wave + (lane >> 2);
            const int s = 16 * wave + 16 + 4 * (lane & 3);
            st4bf(PB + r * SW + s, 0.f, 0.f, 0.f, 0.f);
        }
        __syncthreads();

        // ---------------- phase 3: T = (I + A)^-1, T' = T diag(beta)
        // level 1: diagonal 16x16 inverses by forward substitution (fp32), lane j = column
        {
            const int I = wave;
            // zero the upper blocks other stages read: T'(0,1), T'(2,3), Tcol(T01^T), Trow(T23)
            if (I == 0 || I == 2) {
                const int r = 16 * I + (lane >> 2);
                const int s = 16 * I + 16 + 4 * (lane & 3);
                st4bf(TP + r * SW + s, 0.f, 0.f, 0.f, 0.f);
                if (I == 0) {
                    // Tcol[j][s] for j in [16,32), s in [0,16)
                    st4bf(TCOL + (16 + (lane >> 2)) * ST + 4 * (lane & 3), 0.f, 0.f, 0.f, 0.f);
                } else {
                    // Trow[r][s] for r in [32,48), s in [48,64)
                    st4bf(TROW + (32 + (lane >> 2)) * ST + 48 + 4 * (lane & 3), 0.f, 0.f, 0.f, 0.f);
                }
            }
            if (lane < 16) {
                const int j = lane;
                float t[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) t[r] = (r == j) ? 1.f : 0.f;
                const float* arow = AB + (16 * I) * SA + 16 * I;
#pragma unroll
                for (int r = 1; r < 16; ++r) {
                    float acc = 0.f;
#pragma unroll
                    for (int s = 0; s < r; ++s) acc = fmaf(arow[r * SA + s], t[s], acc);
                    if (r > j) t[r] = -acc;
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
        __syncthreads();
        // level 2: T10 = -T11 (A10 T00) on wave 0, T32 = -T33 (A32 T22) on wave 1
        if (wave < 2) {
            const int Ib = 2 * wave + 1, Jb = 2 * wave;
            uint16_t* ys = YS + wave * 16 * SY;
            const float4 af = *reinterpret_cast<const float4*>(AB + (16 * Ib + l16) * SA + 16 * Jb + 4 * g4);
            f32x4_t y = mfma16(f32_to_s16x4(af), ld4(TCOL, ST, 16 * Jb + l16, 16 * Jb + 4 * g4),
                               f32x4_t{0.f, 0.f, 0.f, 0.f});
            // y[e] = Y[m = 4*g4 + e][n = l16]; stored column-major ys[n][m]
            st4bf(ys + l16 * SY + 4 * g4, y[0], y[1], y[2], y[3]);
            f32x4_t tt = mfma16(ld4(TROW, ST, 16 * Ib + l16, 16 * Ib + 4 * g4), ld4(ys, SY, l16, 4 * g4),
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
        __syncthreads();
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
        __syncthreads();
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
        __syncthreads();

        // ---------------- phase 4: W = T' Kg (as W^T = Kg^T T'^T) and U~ = T' V
        f32x4_t Uacc[NJB];
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
                    st4bf(WB + (16 * I + l16) * SR + 16 * ib + 4 * g4, acc[0], acc[1], acc[2], acc[3]);
                }
            }
            const int I = wave;
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb) {
                f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    if (ks == 1 && I < 2) continue;
                    acc = mfma32(ld8(TP, SW, 16 * I + l16, 32 * ks + 8 * g4),
                                 ld8(VT, SW, 16 * jb + l16, 32 * ks + 8 * g4), acc);
                }
                Uacc[jb] = acc;   // U~[s = 16I + 4*g4 + e][j = 16jb + l16]
            }
        }
        __syncthreads();

        // ---------------- phase 5: U = U~ - W S0, stored as U^T[j][s]
        {
            const int I = wave;
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb) {
                f32x4_t ws = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < DK / 32; ++ks)
                    ws = mfma32(ld8(WB, SR, 16 * I + l16, 32 * ks + 8 * g4),
                                ld8(STB, SR, 16 * jb + l16, 32 * ks + 8 * g4), ws);
                const f32x4_t u = Uacc[jb] - ws;
                st4bf(UT + (16 * jb + l16) * SW + 16 * I + 4 * g4, u[0], u[1], u[2], u[3]);
            }
        }
        __syncthreads();

        // ---------------- phase 6: O^T = S0^T Qg^T + U^T P^T; S = Diag(e^{b_C}) S0 + Kc^T U
        {
            const int I = wave;
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb) {
                f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < DK / 32; ++ks)
                    acc = mfma32(ld8(STB, SR, 16 * jb + l16, 32 * ks + 8 * g4),
                                 ld8(QG, SR, 16 * I + l16, 32 * ks + 8 * g4), acc);
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    if (ks == 1 && I < 2) continue;
                    acc = mfma32(ld8(UT, SW, 16 * jb + l16, 32 * ks + 8 * g4),
                                 ld8(PB, SW, 16 * I + l16, 32 * ks + 8 * g4), acc);
                }
                // acc[e] = O[r = 16I + l16][j = 16jb + 4*g4 + e]
                const int r = 16 * I + l16;
                if (r < len) {
                    Tout* op = o + ((size_t)(c0 + r) * H + h) * DV + j0 + 16 * jb + 4 * g4;
                    if constexpr (sizeof(Tout) == 2) {
                        *reinterpret_cast<uint2*>(op) = make_uint2(pack2(acc[0], acc[1]), pack2(acc[2], acc[3]));
                    } else {
                        *reinterpret_cast<float4*>(op) = make_float4(acc[0], acc[1], acc[2], acc[3]);
                    }
                }
            }
#pragma unroll
            for (int ib = 0; ib < 2; ++ib) {
                const int i0 = 32 * wave + 16 * ib;
                const float4 ec = *reinterpret_cast<const float4*>(VEC + V_EC + i0 + 4 * g4);
#pragma unroll
                for (int jb = 0; jb < NJB; ++jb) {
                    f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks)
                        acc = mfma32(ld8(KCT, SW, i0 + l16, 32 * ks + 8 * g4),
                                     ld8(UT, SW, 16 * jb + l16, 32 * ks + 8 * g4), acc);
                    S[ib][jb][0] = fmaf(ec.x, S[ib][jb][0], acc[0]);
                    S[ib][jb][1] = fmaf(ec.y, S[ib][jb][1], acc[1]);
                    S[ib][jb][2] = fmaf(ec.z, S[ib][jb][2], acc[2]);
                    S[ib][jb][3] = fmaf(ec.w, S[ib][jb][3], acc[3]);
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb)
                st4bf(STB + (16 * jb + l16) * SR + 32 * wave + 16 * ib + 4 * g4, S[ib][jb][0], S[ib][jb][1],
                      S[ib][jb][2], S[ib][jb][3]);
    }

    if (final_state) {
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 32 * wave + 16 * ib + 4 * g4 + e;
                    const int j = j0 + 16 * jb + l16;
                    final_state[soff + (size_t)i * DV + j] = S[ib][jb][e];
                }
    }
}

template <typename Tout>
hipError_t launch_typed(const PrefillArgs& a, hipStream_t stream)
{
    const int ntiles = a.dv / DVT;
    const int units = a.N * a.H;
    const unsigned groups = (unsigned)((units + 7) / 8);
    const dim3 grid(groups * 8u * (unsigned)ntiles);
    hipLaunchKernelGGL((chunked_kernel<Tout>), grid, dim3(NTHREADS), 0, stream,
                       static_cast<const bf16_t*>(a.q), static_cast<const bf16_t*>(a.k),
                       static_cast<const bf16_t*>(a.v), a.g, a.beta, a.a_log, a.dt_bias, a.init,
                       a.cu, a.N, a.T, a.H, a.dv, a.scale, a.lower_bound, (int)a.l2norm,
                       static_cast<Tout*>(a.o), a.final_state);
    return hipGetLastError();
}

}  // namespace

bool chunked_supported(const PrefillArgs& a)
{
    return a.in_bf16 && !a.ejk && a.dk == DK && a.dv % DVT == 0 && a.g != nullptr && a.a_log != nullptr;
}

size_t chunked_workspace_bytes(int, int, int, int, int, bool) { return 0; }

hipError_t launch_chunked(const PrefillArgs& a, hipStream_t stream)
{
    if (a.out_bf16) return launch_typed<bf16_t>(a, stream);
    return launch_typed<float>(a, stream);
}

}  // namespace kda
