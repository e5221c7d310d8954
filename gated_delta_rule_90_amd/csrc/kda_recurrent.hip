// kda_recurrent.hip - token-by-token KDA prefill: the recurrent mode of the
// ejkernel "kernel_delta_attention" page (section "Algorithm modes"; run()
// with use_chunked=False), one step per token.
//
// Grid (column tiles, H, N sequences); one wave per block.  Each state column
// is held in registers by LPC adjacent lanes (16 at dk = 128, 8 at dk = 32
// and 64, 4 at dk = 16), dk / LPC rows each, so the contractions over dk
// (S^T k, S^T q) stay in registers up to a sum over those lanes, and the only
// other cross-lane work per token is the L2 norm of q and k.  Per token: q, k, g become LDS-shared prologue
// vectors (at dk <= 32 for several tokens at once, one token per group of dk
// lanes; else lanes own channels j and j + 64), the squared norms are reduced
// over each token's lanes, the gate and beta activated, then every lane
// advances its column:
//     s <- exp(gamma) * s;  u = s . kh;  s <- s + kh * beta (v_c - u);  o_c = s . qh
// (EJK: u from the undecayed column, s <- e^d s + kh beta (v_c - u)).
// It is evaluated as u = (alpha kh) . s_old and p = (alpha qh) . s_old side by
// side, d = beta (v_c - u), o_c = p + d (kh . qh) and s <- alpha s_old + kh d,
// which is the same column update with a shorter dependent chain per token.
// Packed sequences come from cu_seqlens (ejkernel "recurrent" run()); bounds
// read from device memory are clamped to [0, T].
#include <type_traits>
#include <utility>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

// The per-token gate and norms sit on the kernel's dependent chain: hardware
// exp2, reciprocal and reciprocal square root (about 1 ulp each) instead of the
// correctly rounded library sequences, well inside the fp32 path's 1e-5
// relative bound.
__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }
__device__ __forceinline__ float fast_sigmoid(float x)
{
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x * kLog2e));
}

// Element i of a row of n elements, stored through a buffer resource that
// covers just that row: the buffer unit drops stores with i >= n, so lanes
// past the row need no branch around the store.  The row pointer must be
// uniform across the wave.
template <typename T>
__device__ __forceinline__ void row_store(T* row, int n, int i, T val)
{
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(row, 0, n * (int)sizeof(T), 0x00020000);
    if constexpr (sizeof(T) == 4)
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, val), rs, i * 4, 0, 0);
    else
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, val), rs, i * 2, 0, 0);
}

// f(integral_constant<int, J>) for J = 0 .. N-1, unrolled at compile time.
template <typename F, int... J>
__device__ __forceinline__ void unroll_seq(F&& f, std::integer_sequence<int, J...>)
{
    (f(std::integral_constant<int, J>{}), ...);
}

// Sum over each aligned group of N adjacent lanes (N = 1, 2, 4, 8 or 16), in
// every lane of the group: DPP within quads, then the half-row and row mirrors
// pair quads and half rows whose lanes already agree.
template <int N>
__device__ __forceinline__ float lanes_sum(float x)
{
    if constexpr (N >= 2) x = xor_add<1>(x);
    if constexpr (N >= 4) x = xor_add<2>(x);
    if constexpr (N >= 8)
        x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x141, 0xF, 0xF, true));
    if constexpr (N >= 16)
        x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x140, 0xF, 0xF, true));
    return x;
}

// LPC adjacent lanes share one state column: each holds DK / LPC of its rows,
// and the column's dot products finish with lanes_sum<LPC>.  Fewer rows per
// lane shorten the per-token chain and the registers; the tiles of columns
// run in parallel workgroups, each repeating the (cheap) prologue.
__device__ __forceinline__ float raw_of(float x) { return x; }
__device__ __forceinline__ uint32_t raw_of(bf16_t x) { return x.bits; }
__device__ __forceinline__ float raw_f32(float x) { return x; }
__device__ __forceinline__ float raw_f32(uint32_t b) { return __uint_as_float(b << 16); }

template <int DK, int LPC, typename Tin, typename Tout, bool EJK>
__global__ __launch_bounds__(kWave) void recurrent_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, const float* __restrict__ a_log,
    const float* __restrict__ dt_bias, const float* __restrict__ init,
    const int32_t* __restrict__ cu, int T, int H, int HKV, int DV, float scale, float lower_bound,
    int l2norm, Tout* __restrict__ o, float* __restrict__ final_state)
{
    constexpr int PER_LANE = (DK + kWave - 1) / kWave;  // prologue channels per lane
    // prologue vectors, two sets: token t uses set (t - t0) & 1.  They are padded
    // to whole waves, so every lane writes its slot without a branch (lanes past
    // dk write values that are never read).
    constexpr int DKP = PER_LANE * kWave;
    __shared__ float sh_alpha[2][DKP];   // per-channel decay (KDA)
    __shared__ float sh_k[2][DKP];       // kh
    __shared__ float sh_ak[2][DKP];      // alpha * kh (EJK: kh)
    __shared__ float sh_aq[2][DKP];      // alpha * qh (EJK: qh)

    constexpr int RPL = DK / LPC;        // state rows per lane
    constexpr int CPW = kWave / LPC;     // state columns per workgroup
    static_assert(RPL * LPC == DK && RPL >= 4, "rows per lane");
    const int lane = threadIdx.x;
    const int part = lane % LPC;         // rows part * RPL .. part * RPL + RPL - 1
    const int c = blockIdx.x * CPW + lane / LPC;
    const int h = blockIdx.y;
    const int hk = h / (H / HKV);   // the key/value head of head h
    const int n = blockIdx.z;
    const bool active = c < DV;

    int t0, t1;
    if (cu) {
        t0 = min(max(cu[n], 0), T);
        t1 = min(max(cu[n + 1], t0), T);
    } else {
        t0 = n * T;
        t1 = t0 + T;
    }

    float s[RPL];
    const size_t soff = ((size_t)n * H + h) * DK * DV;
#pragma unroll
    for (int m = 0; m < RPL; ++m) s[m] = (init && active) ? init[soff + (size_t)(part * RPL + m) * DV + c] : 0.f;

    // Tokens are taken in packs of TPP = 64 / dk (dk <= 32; else 1): the
    // prologue of a whole pack runs at once, lane l on token l / dk and channel
    // l % dk (at dk >= 64 one token, lanes on channels l and l + 64), so no
    // lane idles in it.  The prologue vectors of token tk of a pack are
    // entries tk * dk .. tk * dk + dk - 1 of a set.
    constexpr int TPP = (DK <= 32) ? kWave / DK : 1;
    const int ltok = (TPP > 1) ? lane / DK : 0;   // this lane's token in a pack
    const int lch = (TPP > 1) ? lane % DK : lane; // this lane's (first) channel

    const float ea = (EJK || !a_log) ? 0.f : expf(a_log[h]);
    float dtb[PER_LANE];
#pragma unroll
    for (int p = 0; p < PER_LANE; ++p) {
        const int i = lch + p * kWave;
        dtb[p] = (!EJK && dt_bias && i < DK) ? dt_bias[(size_t)i * H + h] : 0.f;
    }

    // Inputs of the pack PD tokens ahead are loaded while the current one is
    // computed (a ring of register sets, the loop unrolled over it so that no
    // set is copied), which hides the global-memory latency that otherwise
    // every token would pay.  Loads past the end reload the last token (in
    // bounds, unused); steps past the end leave the state and the output
    // untouched.  The ring holds the loaded values as they arrive; everything
    // computed from them happens at use, so no instruction waits on a load
    // right after issue.
    // Prefetch distance: with one token taking a few hundred cycles, a global
    // load needs a dozen or more tokens of lead to arrive in time.  PD / TPP
    // ring slots, an even number, so slot j's prologue set is j & 1.
    constexpr int PD = (DK >= 64) ? 8 : 16;
    constexpr int NSLOT = PD / TPP;
    static_assert(NSLOT % 2 == 0, "even ring");
    // bf16 inputs are carried as their bits zero-extended to 32: a 16-bit
    // value carried around the loop gets a zero-extension where the loop
    // starts, which waits for its load there
    using RawT = std::conditional_t<std::is_same<Tin, float>::value, float, uint32_t>;
    struct Raw {
        RawT q[PER_LANE], k[PER_LANE];
        float z[PER_LANE];
        float bt;         // this lane's token's beta
        RawT vc[TPP];     // v of this lane's column for each token of the pack (as loaded)
    };
    const int cc = active ? c : 0;
    const int vz = vector_zero();   // beta and the EJK decay: vector loads, see vector_zero()
    auto load = [&](Raw& r, const int tp) __attribute__((always_inline)) {
        const int tl = min(tp + ltok, t1 - 1);
        const size_t th = (size_t)tl * H + h;
        const size_t tkv = (size_t)tl * HKV + hk;
#pragma unroll
        for (int p = 0; p < PER_LANE; ++p) {
            const int i = lch + p * kWave;
            const int ic = (i < DK) ? i : 0;   // lanes past dk read channel 0 and are zeroed on use
            r.q[p] = raw_of(q[th * DK + ic]);
            r.k[p] = raw_of(k[tkv * DK + ic]);
            if (!EJK) r.z[p] = g[th * DK + ic];
        }
        r.bt = beta[th + vz];
        if (EJK) r.z[0] = g ? g[th + vz] : 0.f;   // EJK: the token's scalar log-decay
#pragma unroll
        for (int tk = 0; tk < TPP; ++tk)
            r.vc[tk] = raw_of(v[((size_t)min(tp + tk, t1 - 1) * HKV + hk) * DV + cc]);
    };
    Raw ring[NSLOT];
    if (t0 < t1) {
#pragma unroll
        for (int j = 0; j < NSLOT; ++j) load(ring[j], t0 + j * TPP);
    }
    // the initial state has to be in registers before the loop: taking it here
    // (after the ring loads are issued) keeps the loop's waits precise instead
    // of a full drain of the prefetch at every token
#pragma unroll
    for (int m = 0; m < RPL; ++m) asm volatile("" ::"v"(s[m]));
    // The prologue of a pack (norms, gate, beta) does not depend on the state,
    // so it runs one pack ahead: step j advances the column over pack j's
    // tokens with its prologue set while it computes the next pack's into the
    // other set, and the compiler interleaves the independent chains.  The
    // workgroup is one wave and the LDS operations of a wave are performed in
    // issue order, so the sets need no barrier between the lanes that write
    // them and the lanes that read them.
    const float fl2 = l2norm ? 1.0f : 0.0f;
    struct Pro {
        float bt, kq, as;   // beta, kh . qh, EJK decay factor e^d (1 for KDA)
    };
    struct ProPack {
        Pro tok[TPP];
    };
    // prologue of the pack in ring slot J, written to set P
    auto prologue = [&](auto J, auto P) __attribute__((always_inline)) {
        constexpr int j = decltype(J)::value, pb = decltype(P)::value;
        Raw& r = ring[j];
        // the slot's loads are waited for here, where they are used: otherwise
        // the compiler may widen them where the loop carries them, right after
        // they are issued
#pragma unroll
        for (int p = 0; p < PER_LANE; ++p) {
            settle(r.q[p]);
            settle(r.k[p]);
            if (!EJK) settle(r.z[p]);
        }
        settle(r.bt);
        if (EJK) settle(r.z[0]);
        float qv[PER_LANE], kv[PER_LANE];
        float sq = 0.f, sk = 0.f, sqk = 0.f;
#pragma unroll
        for (int p = 0; p < PER_LANE; ++p) {
            const bool in = lch + p * kWave < DK;
            qv[p] = in ? raw_f32(r.q[p]) : 0.f;
            kv[p] = in ? raw_f32(r.k[p]) : 0.f;
            sq += qv[p] * qv[p];
            sk += kv[p] * kv[p];
            sqk += qv[p] * kv[p];
        }
        // one token's channels: a row (dk = 16), a half (32) or the wave
        constexpr int NSUM = (DK <= 16) ? 16 : (DK <= 32 ? 32 : 64);
        sq = group_sum<NSUM>(sq);
        sk = group_sum<NSUM>(sk);
        sqk = group_sum<NSUM>(sqk);
        // l2norm blended arithmetically: a branch here would split the block
        // that the compiler interleaves with the column update
        const float nq = scale * fmaf(fl2, __builtin_amdgcn_rsqf(sq + kNormEps) - 1.0f, 1.0f);
        const float nk = fmaf(fl2, __builtin_amdgcn_rsqf(sk + kNormEps) - 1.0f, 1.0f);
#pragma unroll
        for (int p = 0; p < PER_LANE; ++p) {
            const int i = lane + p * kWave;   // = token * dk + channel
            const float qh = qv[p] * nq, kh = kv[p] * nk;
            sh_k[pb][i] = kh;
            if (!EJK) {
                const float a = fast_exp(lower_bound * fast_sigmoid(ea * (r.z[p] + dtb[p])));
                sh_alpha[pb][i] = a;
                sh_ak[pb][i] = a * kh;
                sh_aq[pb][i] = a * qh;
            } else {
                sh_ak[pb][i] = kh;
                sh_aq[pb][i] = qh;
            }
        }
        // the token scalars, from the first lane of each token's group
        const float kql = sqk * nq * nk;
        const float btl = EJK ? r.bt : fast_sigmoid(r.bt);
        const float asl = EJK ? fast_exp(r.z[0]) : 1.0f;
        ProPack pk;
#pragma unroll
        for (int tk = 0; tk < TPP; ++tk) {
            pk.tok[tk].kq = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, kql), tk * DK));
            pk.tok[tk].bt = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, btl), tk * DK));
            pk.tok[tk].as = EJK ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, asl), tk * DK))
                                : 1.0f;
        }
        return pk;
    };
    // column update for token TK of the pack in ring slot J, prologue set P:
    // u = (alpha kh) . s_old and p = (alpha qh) . s_old side by side, in four
    // partial sums each; the output needs no pass over the new column,
    // S_new^T qh = p + d (kh . qh).  (EJK: u, p from the undecayed column,
    // output e^d p + d (kh . qh).)
    auto column = [&](auto J, auto P, auto TK, const Pro& pr, const int t) __attribute__((always_inline)) {
        constexpr int j = decltype(J)::value, pb = decltype(P)::value, tk = decltype(TK)::value;
        constexpr int NP = (RPL >= 4) ? 4 : 1;
        const int base = tk * DK + part * RPL;
        const float* ak = &sh_ak[pb][base];
        const float* aq = &sh_aq[pb][base];
        float up[NP], pp[NP];
#pragma unroll
        for (int e = 0; e < NP; ++e) up[e] = pp[e] = 0.f;
#pragma unroll
        for (int m = 0; m < RPL; ++m) {
            up[m % NP] = fmaf(s[m], ak[m], up[m % NP]);
            pp[m % NP] = fmaf(s[m], aq[m], pp[m % NP]);
        }
        float u = up[0], pq = pp[0];
#pragma unroll
        for (int e = 1; e < NP; ++e) {
            u += up[e];
            pq += pp[e];
        }
        u = lanes_sum<LPC>(u);
        pq = lanes_sum<LPC>(pq);
        settle(ring[j].vc[tk]);
        const float d = pr.bt * (raw_f32(ring[j].vc[tk]) - u);
        // one lane per column stores; the others pass an index past the row
        row_store(o + ((size_t)t * H + h) * DV, DV, part == 0 ? c : DV, from_f32<Tout>(fmaf(d, pr.kq, pr.as * pq)));
        const float* kk = &sh_k[pb][base];
        const float* al = &sh_alpha[pb][base];
#pragma unroll
        for (int m = 0; m < RPL; ++m) s[m] = fmaf(kk[m], d, (EJK ? pr.as : al[m]) * s[m]);
    };
    if (t0 < t1) {
        ProPack pk = prologue(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
        // step j of a block of PD tokens starting at tb; CHECKED: tokens may be past the end
        auto step = [&](auto J, const int tb, auto CHECKED) __attribute__((always_inline)) {
            constexpr int j = decltype(J)::value;
            const int tp = tb + j * TPP;
            unroll_seq(
                [&](auto TK) __attribute__((always_inline)) {
                    const int t = tp + decltype(TK)::value;
                    if (!decltype(CHECKED)::value || t < t1)
                        column(J, std::integral_constant<int, (j & 1)>{}, TK, pk.tok[decltype(TK)::value], t);
                },
                std::make_integer_sequence<int, TPP>{});
            load(ring[j], tp + PD);
            pk = prologue(std::integral_constant<int, (j + 1) % NSLOT>{}, std::integral_constant<int, ((j + 1) & 1)>{});
        };
        int tb = t0;
        for (; tb + PD <= t1; tb += PD)
            unroll_seq([&](auto J) __attribute__((always_inline)) { step(J, tb, std::false_type{}); },
                       std::make_integer_sequence<int, NSLOT>{});
        if (tb < t1)
            unroll_seq([&](auto J) __attribute__((always_inline)) { step(J, tb, std::true_type{}); },
                       std::make_integer_sequence<int, NSLOT>{});
    }

    if (final_state && active) {
#pragma unroll
        for (int m = 0; m < RPL; ++m) final_state[soff + (size_t)(part * RPL + m) * DV + c] = s[m];
    }
}

template <int DK, int LPC, typename Tin, typename Tout>
hipError_t launch_typed(const PrefillArgs& a, hipStream_t stream)
{
    constexpr int CPW = kWave / LPC;
    const dim3 grid((unsigned)((a.dv + CPW - 1) / CPW), (unsigned)a.H, (unsigned)a.N);
    const dim3 block(kWave);
    const Tin* q = static_cast<const Tin*>(a.q);
    const Tin* k = static_cast<const Tin*>(a.k);
    const Tin* v = static_cast<const Tin*>(a.v);
    Tout* o = static_cast<Tout*>(a.o);
    if (a.ejk)
        hipLaunchKernelGGL((recurrent_kernel<DK, LPC, Tin, Tout, true>), grid, block, 0, stream, q, k, v,
                           a.g, a.beta, a.a_log, a.dt_bias, a.init, a.cu, a.T, a.H, a.Hkv, a.dv, a.scale,
                           a.lower_bound, (int)a.l2norm, o, a.final_state);
    else
        hipLaunchKernelGGL((recurrent_kernel<DK, LPC, Tin, Tout, false>), grid, block, 0, stream, q, k, v,
                           a.g, a.beta, a.a_log, a.dt_bias, a.init, a.cu, a.T, a.H, a.Hkv, a.dv, a.scale,
                           a.lower_bound, (int)a.l2norm, o, a.final_state);
    return hipGetLastError();
}

// lanes per column: dk / 4 up to 16 (four or eight rows per lane)
template <int DK, typename Tin, typename Tout>
hipError_t launch_lpc(const PrefillArgs& a, hipStream_t stream)
{
    return launch_typed<DK, (DK >= 128 ? 16 : DK >= 32 ? 8 : 4), Tin, Tout>(a, stream);
}

template <int DK>
hipError_t launch_dk(const PrefillArgs& a, hipStream_t stream)
{
    if (!a.in_bf16) return launch_lpc<DK, float, float>(a, stream);
    if (a.out_bf16) return launch_lpc<DK, bf16_t, bf16_t>(a, stream);
    return launch_lpc<DK, bf16_t, float>(a, stream);
}

}  // namespace

// One object per key dimension (KDA_RECURRENT_DK set by build.py), so the
// instantiations compile in parallel; the dispatch over dk is in kda_api.cpp.
#ifndef KDA_RECURRENT_DK
#error "build kda_recurrent.hip with -DKDA_RECURRENT_DK=16, 32, 64 or 128"
#endif
#define KDA_CAT2(a, b) a##b
#define KDA_CAT(a, b) KDA_CAT2(a, b)
hipError_t KDA_CAT(launch_recurrent_dk, KDA_RECURRENT_DK)(const PrefillArgs& a, hipStream_t stream)
{
    return launch_dk<KDA_RECURRENT_DK>(a, stream);
}

}  // namespace kda
