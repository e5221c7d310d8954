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
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

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

    for (int t = t0; t < t1; ++t) {
        const size_t th = (size_t)t * H + h;
        float qv[PER_LANE], kv[PER_LANE], zv[PER_LANE];
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int p = 0; p < PER_LANE; ++p) {
            const int i = lane + p * kWave;
            qv[p] = kv[p] = zv[p] = 0.f;
            if (i < DK) {
                qv[p] = to_f32(q[th * DK + i]);
                kv[p] = to_f32(k[th * DK + i]);
                if (!EJK) zv[p] = g[th * DK + i] + dtb[p];
            }
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
                if (!EJK) sh_alpha[i] = expf(lower_bound * sigmoid_f(ea * zv[p]));
            }
        }
        float bt, alpha_s = 1.0f;
        if (!EJK) {
            bt = sigmoid_f(beta[th]);
        } else {
            bt = beta[th];
            alpha_s = g ? expf(g[th]) : 1.0f;
        }
        const float vc = active ? to_f32(v[th * DV + c]) : 0.f;
        __syncthreads();

        float u = 0.f;
#pragma unroll
        for (int i = 0; i < DK; ++i) {
            if (!EJK) s[i] *= sh_alpha[i];
            u = fmaf(s[i], sh_k[i], u);
        }
        const float d = bt * (vc - u);
        float oc = 0.f;
#pragma unroll
        for (int i = 0; i < DK; ++i) {
            s[i] = fmaf(sh_k[i], d, EJK ? alpha_s * s[i] : s[i]);
            oc = fmaf(s[i], sh_q[i], oc);
        }
        if (active) o[th * DV + c] = from_f32<Tout>(oc);
        __syncthreads();
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
