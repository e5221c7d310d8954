// kda_recurrent.hip - token-by-token KDA prefill (ejkernel use_chunked=False:
// "Recurrent: Pure sequential scan for memory efficiency").
//
// Grid (dv / 64 column tiles, H, N sequences); one wave per block.  Lane j
// owns state column c = 64 * tile + j as dk float32 registers, so the
// contractions over dk (S^T k, S^T q) stay inside the lane and the only
// cross-lane work per token is the L2 norm of q and k.  Per token: load
// q, k, g into LDS-shared prologue vectors (lanes own channels j and j + 64),
// reduce the squared norms over the wave, activate the gate and beta, then
// every lane advances its column:
//     s <- exp(gamma) * s;  u = s . kh;  s <- s + kh * beta (v_c - u);  o_c = s . qh
// (EJK: u from the undecayed column, s <- e^d s + kh beta (v_c - u)).
// Packed sequences come from cu_seqlens (ejkernel "recurrent" run()); bounds
// read from device memory are clamped to [0, T].
#include <type_traits>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

// The per-token gate sits on the kernel's dependent chain: hardware exp2 and
// reciprocal (about 1 ulp each) instead of the correctly rounded library
// sequences, well inside the fp32 path's 1e-5 relative bound.
__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }
__device__ __forceinline__ float fast_sigmoid(float x)
{
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x * kLog2e));
}

template <int DK, typename Tin, typename Tout, bool EJK>
__global__ __launch_bounds__(kWave) void recurrent_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, const float* __restrict__ a_log,
    const float* __restrict__ dt_bias, const float* __restrict__ init,
    const int32_t* __restrict__ cu, int T, int H, int DV, float scale, float lower_bound,
    int l2norm, Tout* __restrict__ o, float* __restrict__ final_state)
{
    constexpr int PER_LANE = (DK + kWave - 1) / kWave;  // prologue channels per lane
    __shared__ float sh_alpha[DK];
    __shared__ float sh_k[DK];
    __shared__ float sh_q[DK];

    const int lane = threadIdx.x;
    const int c = blockIdx.x * kWave + lane;
    const int h = blockIdx.y;
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

    float s[DK];
    const size_t soff = ((size_t)n * H + h) * DK * DV;
#pragma unroll
    for (int i = 0; i < DK; ++i) s[i] = (init && active) ? init[soff + (size_t)i * DV + c] : 0.f;

    const float ea = (EJK || !a_log) ? 0.f : expf(a_log[h]);
    float dtb[PER_LANE];
#pragma unroll
    for (int p = 0; p < PER_LANE; ++p) {
        const int i = lane + p * kWave;
        dtb[p] = (!EJK && dt_bias && i < DK) ? dt_bias[(size_t)i * H + h] : 0.f;
    }

    // Inputs of token t + PD are loaded while token t is computed (a ring of PD
    // register sets, the loop unrolled by PD so that no set is copied), which
    // hides the global-memory latency that otherwise every token would pay.
    // Loads past the end reload the last token (in bounds, unused); steps past
    // the end leave the state and the output untouched.
    // The ring holds the loaded values as they arrive; everything computed from
    // them happens at use, so no instruction waits on a load right after issue.
    constexpr int PD = (DK >= 128) ? 1 : 4;   // dk = 128: the column already takes 128 registers
    struct Raw {
        Tin q[PER_LANE], k[PER_LANE];
        float z[PER_LANE];
        float bt, vc;
    };
    const int cc = active ? c : 0;
    const int vz = vector_zero();   // beta and the EJK decay: vector loads, see vector_zero()
    auto load = [&](Raw& r, int t) {
        t = min(t, t1 - 1);
        const size_t th = (size_t)t * H + h;
#pragma unroll
        for (int p = 0; p < PER_LANE; ++p) {
            const int i = lane + p * kWave;
            const int ic = (i < DK) ? i : 0;   // lanes past dk read channel 0 and are zeroed on use
            r.q[p] = q[th * DK + ic];
            r.k[p] = k[th * DK + ic];
            if (!EJK) r.z[p] = g[th * DK + ic];
        }
        r.bt = beta[th + vz];
        if (EJK) r.z[0] = g ? g[th + vz] : 0.f;   // EJK: the token's scalar log-decay
        r.vc = to_f32(v[th * DV + cc]);
    };
    Raw ring[PD];
    if (t0 < t1) {
#pragma unroll
        for (int j = 0; j < PD; ++j) load(ring[j], t0 + j);
    }
    // the initial state has to be in registers before the loop: taking it here
    // (after the ring loads are issued) keeps the loop's waits precise instead
    // of a full drain of the prefetch at every token
#pragma unroll
    for (int i = 0; i < DK; ++i) asm volatile("" ::"v"(s[i]));
    // one token from ring slot J (a compile-time index, so the ring stays in registers)
    auto token = [&](auto J, const int tb) {
        constexpr int j = decltype(J)::value;
        const int t = tb + j;
        const bool live = t < t1;
        const Raw& r = ring[j];
        float qv[PER_LANE], kv[PER_LANE];
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int p = 0; p < PER_LANE; ++p) {
            const bool in = lane + p * kWave < DK;
            qv[p] = in ? to_f32(r.q[p]) : 0.f;
            kv[p] = in ? to_f32(r.k[p]) : 0.f;
            sq += qv[p] * qv[p];
            sk += kv[p] * kv[p];
        }
        sq = wave_sum(sq);
        sk = wave_sum(sk);
        const float nq = l2norm ? scale / sqrtf(sq + kNormEps) : scale;
        const float nk = l2norm ? 1.0f / sqrtf(sk + kNormEps) : 1.0f;
#pragma unroll
        for (int p = 0; p < PER_LANE; ++p) {
            const int i = lane + p * kWave;
            if (i < DK) {
                sh_q[i] = qv[p] * nq;
                sh_k[i] = kv[p] * nk;
                if (!EJK) sh_alpha[i] = fast_exp(lower_bound * fast_sigmoid(ea * (r.z[p] + dtb[p])));
            }
        }
        float bt, alpha_s = 1.0f;
        if (!EJK) {
            bt = fast_sigmoid(r.bt);
        } else {
            bt = r.bt;
            alpha_s = fast_exp(r.z[0]);
        }
        lds_barrier();

        if (live) {
            // four partial sums per dot product: the per-token dependent chain is
            // what bounds this kernel, not its arithmetic
            constexpr int NP = (DK >= 4) ? 4 : 1;
            float up[NP];
#pragma unroll
            for (int e = 0; e < NP; ++e) up[e] = 0.f;
#pragma unroll
            for (int i = 0; i < DK; ++i) {
                if (!EJK) s[i] *= sh_alpha[i];
                up[i % NP] = fmaf(s[i], sh_k[i], up[i % NP]);
            }
            float u = up[0];
#pragma unroll
            for (int e = 1; e < NP; ++e) u += up[e];
            const float d = bt * (r.vc - u);
            float op[NP];
#pragma unroll
            for (int e = 0; e < NP; ++e) op[e] = 0.f;
#pragma unroll
            for (int i = 0; i < DK; ++i) {
                s[i] = fmaf(sh_k[i], d, EJK ? alpha_s * s[i] : s[i]);
                op[i % NP] = fmaf(s[i], sh_q[i], op[i % NP]);
            }
            float oc = op[0];
#pragma unroll
            for (int e = 1; e < NP; ++e) oc += op[e];
            if (active) o[((size_t)t * H + h) * DV + c] = from_f32<Tout>(oc);
        }
        lds_barrier();   // the next token rewrites the prologue vectors
        load(ring[j], t + PD);
    };
    for (int tb = t0; tb < t1; tb += PD) {
        token(std::integral_constant<int, 0>{}, tb);
        if constexpr (PD > 1) token(std::integral_constant<int, (PD > 1 ? 1 : 0)>{}, tb);
        if constexpr (PD > 2) token(std::integral_constant<int, (PD > 2 ? 2 : 0)>{}, tb);
        if constexpr (PD > 3) token(std::integral_constant<int, (PD > 3 ? 3 : 0)>{}, tb);
    }

    if (final_state && active) {
#pragma unroll
        for (int i = 0; i < DK; ++i) final_state[soff + (size_t)i * DV + c] = s[i];
    }
}

template <int DK, typename Tin, typename Tout>
hipError_t launch_typed(const PrefillArgs& a, hipStream_t stream)
{
    const dim3 grid((unsigned)((a.dv + kWave - 1) / kWave), (unsigned)a.H, (unsigned)a.N);
    const dim3 block(kWave);
    const Tin* q = static_cast<const Tin*>(a.q);
    const Tin* k = static_cast<const Tin*>(a.k);
    const Tin* v = static_cast<const Tin*>(a.v);
    Tout* o = static_cast<Tout*>(a.o);
    if (a.ejk)
        hipLaunchKernelGGL((recurrent_kernel<DK, Tin, Tout, true>), grid, block, 0, stream, q, k, v,
                           a.g, a.beta, a.a_log, a.dt_bias, a.init, a.cu, a.T, a.H, a.dv, a.scale,
                           a.lower_bound, (int)a.l2norm, o, a.final_state);
    else
        hipLaunchKernelGGL((recurrent_kernel<DK, Tin, Tout, false>), grid, block, 0, stream, q, k, v,
                           a.g, a.beta, a.a_log, a.dt_bias, a.init, a.cu, a.T, a.H, a.dv, a.scale,
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

hipError_t launch_recurrent(const PrefillArgs& a, hipStream_t stream)
{
    switch (a.dk) {
    case 16: return launch_dk<16>(a, stream);
    case 32: return launch_dk<32>(a, stream);
    case 64: return launch_dk<64>(a, stream);
    default: return launch_dk<128>(a, stream);
    }
}

}  // namespace kda
