// kda_chunked_f32.hip - chunk-parallel KDA prefill in float32 arithmetic: float32
// inputs at any dk, bf16 inputs at dk < 128
// (the chunked mode of the ejkernel "kernel_delta_attention" page, section
// "Algorithm modes").
//
// The chunk algebra is the bf16 MFMA kernel's (an exact regrouping of the
// token recurrence: decay per key channel, residual against the decayed
// state, o = S^T q), evaluated in float32 (float32 MFMA and vector ALU) so
// that the result meets the float32 bar.  For a chunk of C tokens with b_r the
// in-chunk cumulative log-decay (per channel, log2 units), beta_r the
// activated beta and S0 the entering state:
//     A_rs = beta_r sum_i kh_ri kh_si 2^{b_ri - b_si}   (s < r)
//     P_rs = sum_i qh_ri kh_si 2^{b_ri - b_si}          (s <= r)
//     Y = V - Kg S0,  U = (I + A)^-1 diag(beta) Y   (= T' V - W S0 with T' =
//     (I + A)^-1 diag(beta), W = T' Kg: U is solved for directly, no T' or W)
//     O = Qg S0 + P U,  S = Diag(2^{b_C}) S0 + Kc^T U
// with Kg_s = 2^{b_s} kh_s, Qg_r = 2^{b_r} qh_r, Kc_s = 2^{b_C - b_s} kh_s.
//
// A chunk is one 16-row block at dk >= 64 and two at dk <= 32 (where the
// per-chunk latency dominates).  With lower_bound >= -5 a channel's log-decay
// over 16 tokens is at most 16 * 5 * log2(e) < 116 in log2 units, so a
// reference row per block (its first row f) keeps every factor inside
// float32's normal range:
//     L_r = 2^{b_r - b_f} in [2^-116, 1],   R_s = 2^{b_f - b_s} in [1, 2^116]
// and 2^{b_r - b_s} = L_r R_s for the kept pairs (s <= r) is a product of
// two normal numbers, at most 1.  The off-diagonal block of a two-block chunk
// pairs rows referenced to row 16 with block-0 keys referenced to row 16 too
// (2^{b_16 - b_s} <= 1), so both factors are at most 1 and an underflow is of
// a value below 2^-126.  Kc = 2^{b_C - b_16} (R or the row-16-referenced
// keys) and Qg = 2^{b_f} L keep every summand of the state products bounded.
//
// EJK mode (scalar per-head decay d_t, beta used as given, residual against
// the undecayed state): A_rs carries 2^{b_{r-1} - b_s} and Kg_r = 2^{b_{r-1}}
// kh_r (b_{-1} = 0); with d <= 0 (the page's contract) every factor is at most
// 1 and is applied per (r, s) as a scalar.
//
// Work split: one 256-thread workgroup per (sequence, head, 16 state
// columns); the state tile stays in LDS in float32, transposed ([16][dk]).  Per chunk:
//   1. the raw q, k rows go to LDS; gate activations element by element; row
//      norms summed from the load registers;
//   2. the gate cumsum of each channel down the chunk's rows (two-block
//      chunks: 8-row segments on adjacent lanes joined by a prefix);
//   3. every thread scales its elements of q, k by the norms and decay factors;
//   4. the contractions over dk (the blocks of A, of P, Qg S0, Kg S0) run on
//      16x16x4 float32 MFMA, one kind per wave and in parallel, with the row
//      operands read four channels (16 bytes) per lane;
//   5. one wave solves (I + A) U = diag(beta) Y by forward substitution, 16
//      rows at a time (the coupling of the second block on MFMA);
//   6. O and the new state are MFMA products with K = the chunk length.
// The column-independent quantities (prologue, A, P) are recomputed by each
// column tile, which is cheap beside the state products at dk <= 128.  The
// inputs of the next chunks (64 tokens ahead at dk <= 32, 32 above) are
// loaded into a register ring while the current one computes: at small dk a
// chunk takes less than a memory latency.  Rows past a sequence's end are padded with
// exact neutral values (q = k = v = 0, gamma = 0, beta = 0) and never stored,
// so a packed batch equals each sequence run alone, bit for bit.
#include <type_traits>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int FB = 16;    // rows per block (each block has its own decay reference row)
constexpr int FT = 256;   // threads per workgroup
constexpr int FJ = 16;    // state columns per workgroup
constexpr int F16 = FJ + 1;   // row stride of [rows][16] tiles

// A chunk is NB blocks of 16 rows (NB = 1 or 2).
template <int DK, int NB>
struct F32Lds {
    static constexpr int FC = FB * NB;
    static constexpr int FA = FC + 4;    // row stride of A (16-byte aligned rows)
    static constexpr int FP = FC + 4;    // row stride of P (16-byte aligned rows)
    static constexpr int SU = FC + 4;    // row stride of the transposed U tile
    static constexpr int RS = DK + 4;   // row stride of [rows][DK] tiles: 16-byte rows, 16 rows in 16 distinct bank groups
    alignas(16) float QL[FC * RS];    // raw q rows, then qh_r 2^{b_r - b_f} (f: the row's block reference; EJK: qh_r)
    alignas(16) float KL[FC * RS];    // raw k rows, then kh_r 2^{b_r - b_f} (EJK: kh_r)
    alignas(16) float KR[FC * RS];    // kh_r 2^{b_f - b_r} (EJK: kh_r)
    alignas(16) float K1[NB == 2 ? FB * RS : 4];   // block-0 rows referenced to row 16: kh_r 2^{b_16 - b_r} (<= 1)
    alignas(16) float GB[FC * RS];    // gamma', then b_r per channel (log2 units, KDA)
    static constexpr int SRS = DK + 4;   // row stride of the transposed state tile
    alignas(16) float ST[FJ * SRS];   // the state tile, transposed: S[i][j] at ST[j * SRS + i]
    alignas(16) float VT[FJ * SU];   // the value tile, transposed: V[s][j] at VT[j * SU + s]
    alignas(16) float AM[FC * FA];   // A (strict lower, beta-scaled)
    alignas(16) float PM[FC * FP];   // P (lower incl. diagonal)
    alignas(16) float YT[FJ * SU];   // Y = V - Kg S0, then block 1's right-hand side (transposed)
    alignas(16) float UT[FJ * SU];   // U, transposed: U[s][j] at UT[j * SU + s]
    float OM[FC * F16];   // O of the chunk, stored by every thread
    alignas(16) float E0[DK];   // 2^{b_0}
    alignas(16) float E1[DK];   // 2^{b_f} of the last block's reference row f
    float N1[DK];         // 2^{b_C - b_f} of the last block's reference row f
    alignas(16) float DC[DK];   // 2^{b_C}
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

typedef float f32x4_t __attribute__((ext_vector_type(4)));


// Four consecutive input channels as loaded: a float4 (float32 inputs) or
// four bf16 in a uint2 (bf16 inputs), widened when used, so that a prefetched
// load is not waited for where it is issued.
template <typename Tin> struct Piece4;
template <> struct Piece4<float> {
    using type = float4;
    static __device__ __forceinline__ float4 load(__amdgpu_buffer_rsrc_t r, int voff, int soff)
    {
        return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
    }
    static __device__ __forceinline__ float load1(__amdgpu_buffer_rsrc_t r, int voff, int soff)
    {
        return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
    }
    static __device__ __forceinline__ float4 widen(float4 x) { return x; }
};
template <> struct Piece4<bf16_t> {
    using type = uint2;
    static __device__ __forceinline__ uint2 load(__amdgpu_buffer_rsrc_t r, int voff, int soff)
    {
        return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
    }
    static __device__ __forceinline__ bf16_t load1(__amdgpu_buffer_rsrc_t r, int voff, int soff)
    {
        return bf16_t{__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0)};
    }
    static __device__ __forceinline__ float4 widen(uint2 x)
    {
        return make_float4(__uint_as_float(x.x << 16), __uint_as_float(x.x & 0xffff0000u),
                           __uint_as_float(x.y << 16), __uint_as_float(x.y & 0xffff0000u));
    }
};

// D += A B on a 16x16x4 float32 MFMA: lane l supplies A[l % 16][l / 16] and
// B[l / 16][l % 16] and holds D[4 (l / 16) + e][l % 16] in element e.
__device__ __forceinline__ f32x4_t mfma4(float a, float b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Lane K's x in every lane of its quad (DPP quad_perm K, K, K, K).
template <int K>
__device__ __forceinline__ float quad_bcast(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), K * 0x55, 0xF, 0xF, false));
}

// x summed over each aligned group of N lanes (N = 4, 8, 16 or 32), in every
// lane of the group.  The whole wave must be active.
template <int N>
__device__ __forceinline__ float lane_group_sum(float x)
{
    x = xor_add<1>(x);
    x = xor_add<2>(x);
    if constexpr (N >= 8) x = xor_add<4>(x);
    if constexpr (N >= 16) x = xor_add<8>(x);
    if constexpr (N >= 32) x = xor_add<16>(x);
    return x;
}

template <int DK, int NB, bool EJK, typename Tin, typename Tout>
__global__ __launch_bounds__(FT) void chunk_f32_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, const float* __restrict__ a_log,
    const float* __restrict__ dt_bias, const float* __restrict__ init, const int32_t* __restrict__ cu,
    int T, int H, int HKV, int DV, float scale, float lower_bound, int l2norm,
    Tout* __restrict__ o, float* __restrict__ final_state)
{
    using LT = F32Lds<DK, NB>;
    constexpr int RS = LT::RS;
    constexpr int FC = LT::FC, FA = LT::FA, FP = LT::FP;
    constexpr int FL = FB * (NB - 1);   // the last block's reference row
    constexpr int RL = DK / 4;                 // lanes per row in the q, k loads (4 channels each)
    constexpr int Q4 = FC * RL;                // pieces of four channels in a [32][DK] tile
    constexpr int QN = (Q4 + FT - 1) / FT;     // per thread
    static_assert(RL >= 4 && RL <= 32 && FC * DK % FT == 0, "dk in {16, 32, 64, 128}");
    __shared__ LT L;

    const int tid = threadIdx.x;
    const int r16 = tid >> 4;   // row of a 16x16 tile (value loads, output stores)
    const int c16 = tid & 15;   // column of a 16x16 tile
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int lm = lane & 15;   // MFMA: operand row / output column
    const int lk = lane >> 4;   // MFMA: operand k / output row group
    const int ro = 4 * lk;      // MFMA: first output row of this lane
    const int j0 = blockIdx.x * FJ;
    const int h = blockIdx.y;
    const int n = blockIdx.z;
    const int hk = h / (H / HKV);
    int t0, t1;
    f32_seq_bounds(cu, n, T, t0, t1);
    const int nch = (t1 - t0 + FC - 1) / FC;
    const size_t soff = ((size_t)n * H + h) * DK * DV;

    {
        // the initial state tile (zeros without one): every load issued, then stored
        constexpr int SN = DK * FJ / FT;
        static_assert(SN * FT == DK * FJ, "state tile per thread");
        const auto ri = buf_rsrc(init ? uniform_ptr(init + soff) : nullptr, init ? (uint32_t)(DK * DV * 4) : 0u);
        float sv[SN];
#pragma unroll
        for (int m = 0; m < SN; ++m) {
            const int e = tid + m * FT, i = e / FJ, j = e % FJ;
            sv[m] = buf_load<float>(ri, (uint32_t)((i * DV + j0 + j) * 4));
        }
#pragma unroll
        for (int m = 0; m < SN; ++m) {
            const int e = tid + m * FT, i = e / FJ, j = e % FJ;
            L.ST[j * LT::SRS + i] = sv[m];
        }
    }
    // the sequence bounds in scalar registers (the resources built from them
    // would otherwise need a per-lane loop where the compiler keeps them in
    // vector registers)
    t0 = __builtin_amdgcn_readfirstlane(t0);
    t1 = __builtin_amdgcn_readfirstlane(t1);
    const float ea = EJK ? 0.f : expf(a_log[h]) * kLog2e;   // exp(a_log) in log2 units
    const float lb2 = lower_bound * kLog2e;
    // dt_bias of the four channels of this lane's pieces (the piece column
    // tid % RL is the same for every piece of the lane)
    // (loaded on every path, zeros without a bias, and waited for here: a load
    // still in flight on only some paths into the chunk loop makes the compiler
    // wait for all loads at each of its later uses)
    float dtb4[4];
    {
        const auto rd = buf_rsrc(EJK ? nullptr : dt_bias, (!EJK && dt_bias) ? (uint32_t)(DK * H * 4) : 0u);
#pragma unroll
        for (int j = 0; j < 4; ++j) dtb4[j] = buf_load<float>(rd, (uint32_t)(((4 * (tid % RL) + j) * H + h) * 4));
#pragma unroll
        for (int j = 0; j < 4; ++j) settle(dtb4[j]);
    }

    // One chunk's inputs as loaded into registers: q, k and (KDA) g as pieces of
    // four channels (row e / RL, channels 4 (e % RL) ..), v at (rows r16 + 16 hv,
    // column c16), beta and the EJK decay of row tid.  The loads go through
    // buffer resources over the chunk's rows up to the sequence's last (built
    // per chunk in scalar registers); the lane's offset, fixed for the whole
    // sequence, is its place within the chunk, so rows past the sequence fall
    // outside and read zeros, as do all rows of a chunk past the sequence.  The
    // raw values go to LDS unmasked (the gate and beta, which are not zero at
    // zero input, are masked after they are computed), so no load is waited for
    // where it is issued, every path issues the same loads, and the wait before
    // a chunk's first use covers only its own.
    using P4 = Piece4<Tin>;
    using piece_t = typename P4::type;
    struct Raw {
        piece_t q[QN], k[QN];
        float4 g[QN];
        Tin v[NB];
        float b, d;
    };
    constexpr int SI = (int)sizeof(Tin);
    const int nseq = t1 - t0;
    // (the bases are moved to scalar registers: values the compiler carries
    // through the divergent state-initialisation loop above land in vector
    // registers otherwise, and every load would then need a per-lane loop)
    const Tin* qb = uniform_ptr(q + ((size_t)t0 * H + h) * DK);
    const Tin* kb = uniform_ptr(k + ((size_t)t0 * HKV + hk) * DK);
    const float* gb = uniform_ptr((EJK ? (g ? g : beta) : g) + (EJK ? (size_t)t0 * H + h : ((size_t)t0 * H + h) * DK));
    const Tin* vb = uniform_ptr(v + ((size_t)t0 * HKV + hk) * DV + j0);
    const float* bb = uniform_ptr(beta + (size_t)t0 * H + h);
    int vq[QN], vk[QN];
#pragma unroll
    for (int m = 0; m < QN; ++m) {
        const int e = tid + m * FT;
        const int row = e / RL, c4 = e % RL;
        vq[m] = row * H * DK + 4 * c4;     // in elements; q and g share it
        vk[m] = row * HKV * DK + 4 * c4;
    }
    auto load = [&](Raw& R, int c) {
        const int r0 = c * FC;   // the chunk's first row within the sequence
        const auto rq_ = rows_rsrc(qb, r0, nseq, H * DK * SI, DK * SI);
        const auto rk_ = rows_rsrc(kb, r0, nseq, HKV * DK * SI, DK * SI);
        const auto rg_ = EJK ? rows_rsrc(gb, r0, nseq, H * 4, 4) : rows_rsrc(gb, r0, nseq, H * DK * 4, DK * 4);
        const auto rv_ = rows_rsrc(vb, r0, nseq, HKV * DV * SI, FJ * SI);
        const auto rb_ = rows_rsrc(bb, r0, nseq, H * 4, 4);
#pragma unroll
        for (int m = 0; m < QN; ++m) {
            R.q[m] = P4::load(rq_, vq[m] * SI, 0);
            R.k[m] = P4::load(rk_, vk[m] * SI, 0);
            if constexpr (!EJK) R.g[m] = Piece4<float>::load(rg_, vq[m] * 4, 0);
        }
#pragma unroll
        for (int hv = 0; hv < NB; ++hv)
            R.v[hv] = P4::load1(rv_, ((r16 + FB * hv) * HKV * DV + c16) * SI, 0);
        R.b = Piece4<float>::load1(rb_, tid * H * 4, 0);
        if constexpr (EJK) R.d = Piece4<float>::load1(rg_, tid * H * 4, 0);   // NULL decay: zeroed at use
    };
    // chunks loaded ahead: at small dk a chunk computes in less than a memory
    // latency (64 tokens ahead); at large dk 32 tokens cover it
    auto settle_raw = [&](Raw& R) {
#pragma unroll
        for (int m = 0; m < QN; ++m) {
            settle(R.q[m]);
            settle(R.k[m]);
            if constexpr (!EJK) settle(R.g[m]);
        }
#pragma unroll
        for (int hv = 0; hv < NB; ++hv) settle(R.v[hv]);
        settle(R.b);
        if constexpr (EJK) settle(R.d);
    };
    constexpr int FD = (DK <= 32 ? 4 : 2) / NB;
    Raw ring[FD];
    if (nch > 0) {
#pragma unroll
        for (int u = 0; u < FD; ++u) load(ring[u], u);
        // (the first chunks are waited for in full: the compiler's count of the
        // loads in flight at the chunk loop's head is the larger of the counts on
        // entry and around the loop, so waits left pending here would also be
        // paid on every later chunk)
#pragma unroll
        for (int u = 0; u < FD; ++u) settle_raw(ring[u]);
    }

    // Forward substitution of one 16-row block on wave 0: column j on the four
    // lanes of quad j, rows 4p .. 4p + 3 of the block on lane p.  At step s the
    // owner of row s broadcasts u_s within the quad (DPP) and every lane updates
    // its rows; A is zero on and above the diagonal, so rows r <= s keep their
    // value without a mask.  Reads the right-hand side from YT (scaled by beta
    // for block 0), writes U.
    auto solve16 = [&](int rb, bool scale_by_beta) {
        const int jq = lane >> 2, p = lane & 3;
        float u[4], am[4][FB];
        const float4 y4 = *reinterpret_cast<const float4*>(L.YT + jq * LT::SU + rb + 4 * p);
        const float yv[4] = {y4.x, y4.y, y4.z, y4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = rb + 4 * p + e;
            u[e] = (scale_by_beta ? L.BT[r] : 1.f) * yv[e];
#pragma unroll
            for (int s4 = 0; s4 < FB; s4 += 4) {
                const float4 a4 = *reinterpret_cast<const float4*>(L.AM + r * FA + rb + s4);
                am[e][s4] = a4.x; am[e][s4 + 1] = a4.y; am[e][s4 + 2] = a4.z; am[e][s4 + 3] = a4.w;
            }
        }
        auto level = [&](auto sc) {
            constexpr int S = decltype(sc)::value;
            const float us = quad_bcast<S / 4>(u[S % 4]);
#pragma unroll
            for (int e = 0; e < 4; ++e) u[e] = fmaf(-am[e][S], us, u[e]);
        };
        level(std::integral_constant<int, 0>{});  level(std::integral_constant<int, 1>{});
        level(std::integral_constant<int, 2>{});  level(std::integral_constant<int, 3>{});
        level(std::integral_constant<int, 4>{});  level(std::integral_constant<int, 5>{});
        level(std::integral_constant<int, 6>{});  level(std::integral_constant<int, 7>{});
        level(std::integral_constant<int, 8>{});  level(std::integral_constant<int, 9>{});
        level(std::integral_constant<int, 10>{}); level(std::integral_constant<int, 11>{});
        level(std::integral_constant<int, 12>{}); level(std::integral_constant<int, 13>{});
        level(std::integral_constant<int, 14>{});
        *reinterpret_cast<float4*>(L.UT + jq * LT::SU + rb + 4 * p) = make_float4(u[0], u[1], u[2], u[3]);
    };

    auto chunk = [&](Raw& R, int c) {
        const int c0 = t0 + c * FC;
        const int len = min(FC, t1 - c0);   // <= 0 for a padding chunk
        // The chunk's inputs are waited for here, outside any lane-dependent
        // branch, so the wait covers only them: inside such a branch the
        // compiler waits for every load in flight, the prefetched chunks' too.
        settle_raw(R);
        // ---- prologue from the registers: raw q, k rows to LDS, gate activations,
        // row norms (RL lanes per row), beta; then fetch the next chunk
#pragma unroll
        for (int m = 0; m < QN; ++m) {
            const int e = tid + m * FT;
            const int row = e / RL, c4 = e % RL;
            const bool in = e < Q4 && row < len;
            // rows past the sequence were loaded as zeros
            const float4 wq = P4::widen(R.q[m]), wk = P4::widen(R.k[m]);
            if (e < Q4) {
                *reinterpret_cast<float4*>(L.QL + row * RS + 4 * c4) = wq;
                *reinterpret_cast<float4*>(L.KL + row * RS + 4 * c4) = wk;
                if constexpr (!EJK) {
                    // gamma' = lb * log2(e) * sigmoid(exp(a_log) (g + dt_bias)), element by
                    // element here, where every lane holds four; padded rows 0
                    const float xg[4] = {R.g[m].x, R.g[m].y, R.g[m].z, R.g[m].w};
                    float gp[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        gp[j] = in ? lb2 * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-ea * (xg[j] + dtb4[j]))) : 0.f;
                    *reinterpret_cast<float4*>(L.GB + row * RS + 4 * c4) = make_float4(gp[0], gp[1], gp[2], gp[3]);
                }
            }
            float sq = wq.x * wq.x + wq.y * wq.y + wq.z * wq.z + wq.w * wq.w;
            float sk = wk.x * wk.x + wk.y * wk.y + wk.z * wk.z + wk.w * wk.w;
            sq = lane_group_sum<RL>(sq);
            sk = lane_group_sum<RL>(sk);
            if (e < Q4 && c4 == 0) {
                L.NQ[row] = l2norm ? scale * __builtin_amdgcn_rsqf(sq + kNormEps) : scale;
                L.NK[row] = l2norm ? __builtin_amdgcn_rsqf(sk + kNormEps) : 1.0f;
            }
        }
#pragma unroll
        for (int hv = 0; hv < NB; ++hv)
            L.VT[c16 * LT::SU + r16 + FB * hv] = (r16 + FB * hv < len) ? to_f32(R.v[hv]) : 0.f;
        if (tid < FC) {
            // beta = 1 / (1 + 2^{-logit log2(e)}); R.b was loaded by every lane
            L.BT[tid] = (tid < len) ? (EJK ? R.b : __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-kLog2e * R.b))) : 0.f;
            if constexpr (EJK) {
                // b_r and b_{r-1} of row tid, summed in row order; these lanes are one
                // wave, whose LDS operations take effect in issue order
                L.BR[tid] = (tid < len && g) ? R.d * kLog2e : 0.f;
                float b = 0.f, bx = 0.f;
                for (int s = 0; s <= tid; ++s) {
                    bx = b;
                    b += L.BR[s];
                }
                float bc = 0.f;
                for (int s = 0; s < FC; ++s) bc += L.BR[s];
                L.BX[tid] = bx;
                L.EB[tid] = __builtin_amdgcn_exp2f(b);
                L.EX[tid] = __builtin_amdgcn_exp2f(bx);
                L.EC[tid] = __builtin_amdgcn_exp2f(bc - b);
                if (tid == FC - 1) L.DC[0] = __builtin_amdgcn_exp2f(bc);
                L.BR[tid] = b;
            }
        }
        load(R, c + FD);   // a chunk past the sequence loads zeros
        lds_barrier();

        // ---- the gate cumsum of every channel down the chunk's rows.  Two-block
        // chunks: NSEG = 4 adjacent lanes per channel each sum 8 rows, and an
        // exclusive prefix of the segment sums over those lanes (whole waves: dk * 4
        // is a multiple of 64) joins them; one-block chunks: one lane per channel.
        if constexpr (!EJK) {
            constexpr int NSEG = NB == 2 ? 4 : 1;
            constexpr int SEGL = FC / NSEG;   // rows per segment
            static_assert(NSEG == 1 || (DK * NSEG) % 64 == 0, "whole waves of segment lanes");
            if (tid < DK * NSEG) {
                const int i = tid / NSEG, seg = tid % NSEG;
                float gm[SEGL];
#pragma unroll
                for (int k = 0; k < SEGL; ++k) gm[k] = L.GB[(SEGL * seg + k) * RS + i];
                float b = 0.f;
                const int base = lane - seg;   // the lane of this channel's first segment
                if constexpr (NSEG > 1) {
                    float ssum = 0.f;
#pragma unroll
                    for (int k = 0; k < SEGL; ++k) ssum += gm[k];
#pragma unroll
                    for (int s2 = 0; s2 < NSEG - 1; ++s2) {
                        const float o = __shfl(ssum, base + s2);
                        b += (s2 < seg) ? o : 0.f;
                    }
                }
                float bfirst = 0.f;
#pragma unroll
                for (int k = 0; k < SEGL; ++k) {
                    b += gm[k];
                    if (k == 0) bfirst = b;
                    L.GB[(SEGL * seg + k) * RS + i] = b;
                }
                // b_0 and b_FL (first rows of segments 0 and FL / SEGL), b_C (end of the last)
                float b0 = bfirst, bl = bfirst, bc = b;
                if constexpr (NSEG > 1) {
                    b0 = __shfl(bfirst, base);
                    bl = __shfl(bfirst, base + FL / SEGL);
                    bc = __shfl(b, base + NSEG - 1);
                }
                if (seg == 0) {
                    L.E0[i] = __builtin_amdgcn_exp2f(b0);
                    L.E1[i] = __builtin_amdgcn_exp2f(bl);
                    L.N1[i] = __builtin_amdgcn_exp2f(bc - bl);
                    L.DC[i] = __builtin_amdgcn_exp2f(bc);
                }
            }
            lds_barrier();
        }

        // ---- normalised rows with the decay factors of their block: L = 2^{b_r - b_f},
        // R = 1 / L (f = 0 or 16); block-0 keys also referenced to row 16 (K1 <= 1)
        // VW consecutive channels per thread (four, or two where a chunk has fewer
        // than four elements per thread): 16- or 8-byte LDS accesses.
        constexpr int VW = (FC * DK >= 4 * FT) ? 4 : 2;
        typedef float vw_t __attribute__((ext_vector_type(VW)));
        constexpr int DQ = DK / VW;                   // pieces per row
        constexpr int NQD = (FC * DQ + FT - 1) / FT;  // pieces per thread
#pragma unroll
        for (int m = 0; m < NQD; ++m) {
            const int e = tid + m * FT;
            if ((FC * DQ) % FT == 0 || e < FC * DQ) {
                const int r = e / DQ, i = VW * (e % DQ);
                vw_t* pq = reinterpret_cast<vw_t*>(L.QL + r * RS + i);
                vw_t* pk = reinterpret_cast<vw_t*>(L.KL + r * RS + i);
                vw_t* pr = reinterpret_cast<vw_t*>(L.KR + r * RS + i);
                const vw_t qh = *pq * L.NQ[r];
                const vw_t kh = *pk * L.NK[r];
                if constexpr (EJK) {
                    *pq = qh;
                    *pk = kh;
                    *pr = kh;
                } else {
                    const vw_t br = *reinterpret_cast<const vw_t*>(L.GB + r * RS + i);
                    const vw_t d = br - *reinterpret_cast<const vw_t*>(L.GB + (r < FB ? 0 : FB) * RS + i);   // b_r - b_f <= 0
                    vw_t lf, rf;
#pragma unroll
                    for (int j = 0; j < VW; ++j) {
                        lf[j] = __builtin_amdgcn_exp2f(d[j]);
                        rf[j] = __builtin_amdgcn_exp2f(-d[j]);
                    }
                    *pq = qh * lf;
                    *pk = kh * lf;
                    *pr = kh * rf;
                    if constexpr (NB == 2) {
                        if (r < FB) {
                            const vw_t g16 = *reinterpret_cast<const vw_t*>(L.GB + FB * RS + i);
                            vw_t k1;
#pragma unroll
                            for (int j = 0; j < VW; ++j) k1[j] = kh[j] * __builtin_amdgcn_exp2f(g16[j] - br[j]);
                            *reinterpret_cast<vw_t*>(L.K1 + r * RS + i) = k1;
                        }
                    }
                }
            }
        }
        lds_barrier();

        // ---- the products over dk (K = dk in MFMA steps of 4), waves in parallel:
        //   wave 0: the blocks (0,0), (1,1), (1,0) of A,  wave 1: the same of P,
        //   wave 2: Qg S0 for both row blocks (kept in registers for O),
        //   wave 3: Y = V - Kg S0 for both row blocks.
        // Block (1,0) pairs rows referenced to row 16 with block-0 keys referenced to
        // row 16 too, so both factors are at most 1.
        f32x4_t acc0 = f32x4_t{0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
        if (wave <= 1) {
            const float* X = (wave == 0) ? L.KL : L.QL;
            const float* RB = (EJK || NB == 1) ? L.KR : L.K1;   // right operand of block (1,0)
#pragma unroll
            for (int blk = 0; blk < (NB == 2 ? 3 : 1); ++blk) {
                const int I = blk == 0 ? 0 : 1, J = blk == 1 ? 1 : 0;   // (0,0), (1,1), (1,0)
                const float* RR = (blk == 2) ? RB : L.KR;
                f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
                // at step j of a 16-channel block k0, lane group lk supplies channel
                // k0 + 4 lk + j: every channel once, and both operands (rows over the
                // channels) are read four channels at a time
#pragma unroll 4
                for (int k0 = 0; k0 < DK; k0 += 16) {
                    const float4 xa = *reinterpret_cast<const float4*>(X + (FB * I + lm) * RS + k0 + 4 * lk);
                    const float4 xb = *reinterpret_cast<const float4*>(RR + (FB * J + lm) * RS + k0 + 4 * lk);
                    acc = mfma4(xa.x, xb.x, acc);
                    acc = mfma4(xa.y, xb.y, acc);
                    acc = mfma4(xa.z, xb.z, acc);
                    acc = mfma4(xa.w, xb.w, acc);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = FB * I + ro + e, s = FB * J + lm;   // acc[e] = (row r, column s)
                    float x = acc[e];
                    if (wave == 0) {
                        if constexpr (EJK) x *= (s < r) ? __builtin_amdgcn_exp2f(L.BX[r] - L.BR[s]) : 0.f;
                        L.AM[r * FA + s] = (s < r) ? L.BT[r] * x : 0.f;
                    } else {
                        if constexpr (EJK) x *= (s <= r) ? __builtin_amdgcn_exp2f(L.BR[r] - L.BR[s]) : 0.f;
                        L.PM[r * FP + s] = (s <= r) ? x : 0.f;
                    }
                }
            }
        } else {
            // A operand: Qg (wave 2) or Kg (wave 3) = 2^{b_f} X per channel (KDA);
            // the EJK row factor is applied to the result
            const float* X = (wave == 2) ? L.QL : L.KL;
            // channels in the order of the A and P products: k0 + 4 lk + j at step j
#pragma unroll 4
            for (int k0 = 0; k0 < DK; k0 += 16) {
                const int kq = k0 + 4 * lk;
                const float4 x0 = *reinterpret_cast<const float4*>(X + lm * RS + kq);
                const float4 e0 = EJK ? make_float4(1.f, 1.f, 1.f, 1.f) : *reinterpret_cast<const float4*>(L.E0 + kq);
                const float4 s4 = *reinterpret_cast<const float4*>(L.ST + lm * LT::SRS + kq);   // S[kq ..][lm]
                const float sb[4] = {s4.x, s4.y, s4.z, s4.w};
                acc0 = mfma4(e0.x * x0.x, sb[0], acc0);
                acc0 = mfma4(e0.y * x0.y, sb[1], acc0);
                acc0 = mfma4(e0.z * x0.z, sb[2], acc0);
                acc0 = mfma4(e0.w * x0.w, sb[3], acc0);
                if constexpr (NB == 2) {
                    const float4 x1 = *reinterpret_cast<const float4*>(X + (FB + lm) * RS + kq);
                    const float4 e1 = EJK ? make_float4(1.f, 1.f, 1.f, 1.f) : *reinterpret_cast<const float4*>(L.E1 + kq);
                    acc1 = mfma4(e1.x * x1.x, sb[0], acc1);
                    acc1 = mfma4(e1.y * x1.y, sb[1], acc1);
                    acc1 = mfma4(e1.z * x1.z, sb[2], acc1);
                    acc1 = mfma4(e1.w * x1.w, sb[3], acc1);
                }
            }
            if (wave == 2) {
                if constexpr (EJK) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        acc0[e] *= L.EB[ro + e];
                        if constexpr (NB == 2) acc1[e] *= L.EB[FB + ro + e];
                    }
                }
            } else {
                // rows ro .. ro + 3 (and FB + ro ..) of column lm: 16-byte accesses
#pragma unroll
                for (int hb = 0; hb < NB; ++hb) {
                    const f32x4_t a = hb == 0 ? acc0 : acc1;
                    const int r0 = FB * hb + ro;
                    const float4 v4 = *reinterpret_cast<const float4*>(L.VT + lm * LT::SU + r0);
                    float z[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) z[e] = EJK ? L.EX[r0 + e] * a[e] : a[e];
                    *reinterpret_cast<float4*>(L.YT + lm * LT::SU + r0) =
                        make_float4(v4.x - z[0], v4.y - z[1], v4.z - z[2], v4.w - z[3]);
                }
            }
        }
        lds_barrier();

        // ---- U: (I + A) U = diag(beta) Y blockwise on wave 0 (its LDS operations
        // take effect in issue order): block 0, then block 1's right-hand side
        // beta Y_1 - A_10 U_0 on MFMA, then block 1
        if (wave == 0) {
            solve16(0, true);
        }
        if constexpr (NB == 2) {
          if (wave == 0) {
            const float4 y4 = *reinterpret_cast<const float4*>(L.YT + lm * LT::SU + FB + ro);
            f32x4_t y = f32x4_t{L.BT[FB + ro] * y4.x, L.BT[FB + ro + 1] * y4.y, L.BT[FB + ro + 2] * y4.z,
                                L.BT[FB + ro + 3] * y4.w};
            // token s = 4 lk + j at step j (as in the products over dk): A rows and
            // the transposed U read 16 bytes per lane
            {
                const float4 a4 = *reinterpret_cast<const float4*>(L.AM + (FB + lm) * FA + 4 * lk);
                const float4 u4 = *reinterpret_cast<const float4*>(L.UT + lm * LT::SU + 4 * lk);
                y = mfma4(-a4.x, u4.x, y);
                y = mfma4(-a4.y, u4.y, y);
                y = mfma4(-a4.z, u4.z, y);
                y = mfma4(-a4.w, u4.w, y);
            }
            *reinterpret_cast<float4*>(L.YT + lm * LT::SU + FB + ro) = make_float4(y[0], y[1], y[2], y[3]);
            solve16(FB, false);
          }
        }
        lds_barrier();

        // ---- O = Qg S0 + P U (wave 2), S = Diag(2^{b_C}) S0 + Kc^T U (16-row tiles over the waves)
        if (wave == 2) {
            // tokens k0 + 4 lk + j at step j: P rows and the transposed U, 16 bytes per lane
#pragma unroll
            for (int k0 = 0; k0 < FC; k0 += 16) {
                const float4 u4 = *reinterpret_cast<const float4*>(L.UT + lm * LT::SU + k0 + 4 * lk);
                if (k0 < FB) {
                    const float4 p4 = *reinterpret_cast<const float4*>(L.PM + lm * FP + k0 + 4 * lk);
                    acc0 = mfma4(p4.x, u4.x, acc0);
                    acc0 = mfma4(p4.y, u4.y, acc0);
                    acc0 = mfma4(p4.z, u4.z, acc0);
                    acc0 = mfma4(p4.w, u4.w, acc0);
                }
                if constexpr (NB == 2) {
                    const float4 p4 = *reinterpret_cast<const float4*>(L.PM + (FB + lm) * FP + k0 + 4 * lk);
                    acc1 = mfma4(p4.x, u4.x, acc1);
                    acc1 = mfma4(p4.y, u4.y, acc1);
                    acc1 = mfma4(p4.z, u4.z, acc1);
                    acc1 = mfma4(p4.w, u4.w, acc1);
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                L.OM[(ro + e) * F16 + lm] = acc0[e];
                if constexpr (NB == 2) L.OM[(FB + ro + e) * F16 + lm] = acc1[e];
            }
        }
#pragma unroll
        for (int t = wave; t < DK / 16; t += 4) {
            const int ib = 16 * t;
            // S[ib + ro + e][lm], e = 0..3, and their decay factors: 16 bytes each
            const float4 s4 = *reinterpret_cast<const float4*>(L.ST + lm * LT::SRS + ib + ro);
            const float4 dc4 = EJK ? make_float4(L.DC[0], L.DC[0], L.DC[0], L.DC[0])
                                   : *reinterpret_cast<const float4*>(L.DC + ib + ro);
            f32x4_t sc = f32x4_t{dc4.x * s4.x, dc4.y * s4.y, dc4.z * s4.z, dc4.w * s4.w};
            // A operand: Kc^T[ia][s] = 2^{b_C - b_s} kh_s = N1 K1[s] (block 0) or N1 KR[s] (block 1)
            const int ia = ib + lm;
            // token s = k0 + 4 lk + j at step j; the transposed U read 16 bytes per lane
#pragma unroll
            for (int k0 = 0; k0 < FC; k0 += 16) {
                const float4 u4 = *reinterpret_cast<const float4*>(L.UT + lm * LT::SU + k0 + 4 * lk);
                const float uj[4] = {u4.x, u4.y, u4.z, u4.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int s = k0 + 4 * lk + j;
                    float kc;
                    if constexpr (EJK) kc = L.EC[s] * L.KR[s * RS + ia];
                    else kc = L.N1[ia] * ((NB == 2 && k0 < FB) ? L.K1[s * RS + ia] : L.KR[s * RS + ia]);
                    sc = mfma4(kc, uj[j], sc);
                }
            }
            *reinterpret_cast<float4*>(L.ST + lm * LT::SRS + ib + ro) = make_float4(sc[0], sc[1], sc[2], sc[3]);
        }
        lds_barrier();
        // O rows r16 and r16 + 16, column c16, through a buffer resource that ends
        // after the chunk's last row: the buffer unit drops the stores of padded
        // rows, so every lane issues the same stores
        {
            Tout* obase = uniform_ptr(o + ((size_t)c0 * H + h) * DV + j0);
            const int rec = len > 0 ? ((len - 1) * H * DV + FJ) * (int)sizeof(Tout) : 0;
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(obase, 0, rec, 0x00020000);
#pragma unroll
            for (int hv = 0; hv < NB; ++hv) {
                const int r = r16 + FB * hv;
                const int off = (r * H * DV + c16) * (int)sizeof(Tout);
                const Tout val = from_f32<Tout>(L.OM[r * F16 + c16]);
                if constexpr (sizeof(Tout) == 4)
                    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, val), rs, off, 0, 0);
                else
                    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, val), rs, off, 0, 0);
            }
        }
    };
    // Unrolled by the ring depth, so that every ring slot is a fixed set of
    // registers.  The chunk count is padded to a multiple of the depth: a chunk
    // past the end has no rows, so it stores nothing and its state update is
    // exactly S <- 2^0 S.  Every path then issues the same memory operations,
    // and the wait before a chunk's first use counts only that chunk's loads.
    for (int cb = 0; cb < nch; cb += FD) {
#pragma unroll
        for (int u = 0; u < FD; ++u) chunk(ring[u], cb + u);
    }
    if (nch == 0) lds_barrier();   // the initial state tile was written by other threads

    if (final_state) {
        for (int e = tid; e < DK * FJ; e += FT) {
            const int i = e / FJ, j = e % FJ;
            final_state[soff + (size_t)i * DV + j0 + j] = L.ST[j * LT::SRS + i];
        }
    }
}

template <int DK, typename Tin, typename Tout>
hipError_t launch_typed(const PrefillArgs& a, hipStream_t stream)
{
    const dim3 grid((unsigned)(a.dv / FJ), (unsigned)a.H, (unsigned)a.N);
    const Tin* q = static_cast<const Tin*>(a.q);
    const Tin* k = static_cast<const Tin*>(a.k);
    const Tin* v = static_cast<const Tin*>(a.v);
    Tout* o = static_cast<Tout*>(a.o);
    // two 16-row blocks per chunk at small dk, where the per-chunk latency dominates
    constexpr int NB = DK <= 32 ? 2 : 1;
    if (a.ejk)
        hipLaunchKernelGGL((chunk_f32_kernel<DK, NB, true, Tin, Tout>), grid, dim3(FT), 0, stream, q, k, v, a.g,
                           a.beta, a.a_log, a.dt_bias, a.init, a.cu, a.T, a.H, a.Hkv, a.dv, a.scale,
                           a.lower_bound, (int)a.l2norm, o, a.final_state);
    else
        hipLaunchKernelGGL((chunk_f32_kernel<DK, NB, false, Tin, Tout>), grid, dim3(FT), 0, stream, q, k, v, a.g,
                           a.beta, a.a_log, a.dt_bias, a.init, a.cu, a.T, a.H, a.Hkv, a.dv, a.scale,
                           a.lower_bound, (int)a.l2norm, o, a.final_state);
    return hipGetLastError();
}

template <int DK>
hipError_t launch_dk(const PrefillArgs& a, hipStream_t stream)
{
    if (!a.in_bf16) return launch_typed<DK, float, float>(a, stream);
    if (a.out_bf16) return launch_typed<DK, bf16_t, bf16_t>(a, stream);
    return launch_typed<DK, bf16_t, float>(a, stream);
}

}  // namespace

bool chunked_f32_supported(const PrefillArgs& a)
{
    const bool dims = (a.dk == 16 || a.dk == 32 || a.dk == 64 || a.dk == 128) && a.dv % FJ == 0 && a.dv > 0;
    // float32 inputs at any dk; bf16 inputs below dk = 128 (dk = 128 takes the
    // bf16 MFMA kernel).  KDA needs the gate inputs and lower_bound >= -5 (the
    // factor range above).
    // A sequence's rows are addressed with 31-bit byte offsets (T bounds every
    // sequence's length, packed or not).
    const bool spans = (long long)a.T * a.H * (a.dk > a.dv ? a.dk : a.dv) * 4 < (1LL << 31);
    return dims && spans && (!a.in_bf16 || a.dk < 128) &&
           (a.ejk || (a.g != nullptr && a.a_log != nullptr && a.lower_bound >= -5.0f));
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
