// kda_decode.hip - single-token KDA step for B requests (kda_tkg semantics).
//
// AWS Neuron "KDA TKG Kernel API Reference" fixes the interface: raw q, k, g
// in [B, dk, num_head], v [B, num_head, dv], beta logits [B, 1, num_head],
// a_log [1, num_head], dt_bias [dk, num_head], state S [B, num_head, dk, dv]
// read and overwritten in place, output [B, num_head, dv].
//
// The step is bound by the state stream: 2 * dk * dv * 4 bytes per
// (request, head) against ~8 flop per state element.  One workgroup owns one
// (request, head) item.  Its 256 threads hold the whole [dk, dv] slice in
// registers as float4 columns: thread (rg, cg) keeps rows rg*RPT .. +RPT-1 of
// columns 4cg .. 4cg+3, so every load and store instruction of a wave covers
// full 512-byte rows.  The prologue's loads are issued just before the state
// loads, so the prologue (L2 norms, gate, beta) runs while the state is in
// flight.  The pass computes
//     S' = Diag(exp gamma) S,  u = S'^T kh,  p = S'^T qh
// in one sweep, reduces u and p over the rows (lane xor within a wave, then
// LDS across waves), and writes
//     delta = beta (v - u),  S_new = S' + kh delta^T,  out = p + delta (kh . qh)
// which equals S_new^T qh without a second pass over the state.
// EJK (ejkernel "The core recurrence"): u and p come from the undecayed S,
// S_new = e^d S + kh delta^T and out = e^d p + delta (kh . qh).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

// The state is streamed: read once and written once per step, and by the next
// step of the same layer it has long left the caches, so its loads and stores
// are non-temporal (no cache allocation).  Measured at B=64, H=32,
// dk=dv=128: 54.2 -> 47.9 us per step.
typedef float f32x4v_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 load_stream(const float* p)
{
    const f32x4v_t x = __builtin_nontemporal_load(reinterpret_cast<const f32x4v_t*>(p));
    return make_float4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ void store_stream(float* p, float4 v)
{
    __builtin_nontemporal_store(f32x4v_t{v.x, v.y, v.z, v.w}, reinterpret_cast<f32x4v_t*>(p));
}

template <int DK, int DV>
struct DecodeShape {
    static constexpr int NCG = DV / 4;                                 // float4 column groups
    static constexpr int THREADS = (NCG * DK < 256) ? NCG * DK : 256;
    static constexpr int NRG = THREADS / NCG;                          // row groups
    static constexpr int RPT = DK / NRG;                               // rows per thread
    static constexpr int NWAVES = (THREADS + kWave - 1) / kWave;
    static_assert(RPT >= 1 && NRG * RPT == DK, "row split");
    static_assert(THREADS >= DK, "prologue needs one thread per key channel");
};

template <int DK, int DV, bool EJK>
__global__ __launch_bounds__((DecodeShape<DK, DV>::THREADS)) void decode_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ g,
    const float* __restrict__ v, const float* __restrict__ beta, const float* __restrict__ a_log,
    const float* __restrict__ dt_bias, float scale, float lower_bound, int B, int H, int HKV, int l2norm,
    float* __restrict__ out, float* __restrict__ S)
{
    using Sh = DecodeShape<DK, DV>;
    constexpr int NCG = Sh::NCG, RPT = Sh::RPT, NWAVES = Sh::NWAVES;

    __shared__ float sh_alpha[DK];
    __shared__ float sh_k[DK];
    __shared__ float sh_q[DK];
    __shared__ float sh_red[NWAVES][3];
    __shared__ float4 sh_uv[NWAVES > 1 ? NWAVES : 1][NCG][2];

    // XCD-aware placement: workgroups are dealt round-robin over the 8 XCDs, and
    // all heads of one request read the same strided q/k/g cache lines, so every
    // head of request b runs on XCD b % 8 and those lines are fetched into one L2.
    const int xcd = blockIdx.x & 7;
    const int idx = blockIdx.x >> 3;
    const int b = 8 * (idx / H) + xcd;
    const int h = idx % H;
    if (b >= B) return;
    const int item = b * H + h;
    const int hk = h / (H / HKV);          // the key/value head of head h
    const int kvitem = b * HKV + hk;
    const int t = threadIdx.x;
    const int cg = t % NCG;
    const int rg = t / NCG;
    const int lane = t % kWave;
    const int wave = t / kWave;
    float* Sp = S + (size_t)item * DK * DV;

    // 1. the prologue's few loads first (thread i < DK owns key channel i), then the
    // state: loads complete in issue order, so the prologue below waits only for
    // its own values and runs while the state streams in
    float qi = 0.f, ki = 0.f, gi = 0.f, di = 0.f;
    // the item's scalars go out with them as vector loads (see vector_zero()):
    // as scalar loads they would be issued late and waited for at an LDS barrier
    const int vz = vector_zero();
    const float braw = beta[item + vz];
    const float araw = EJK ? 0.f : a_log[h + vz];
    const float draw = (EJK && g) ? g[item + vz] : 0.f;
    if (t < DK) {
        const size_t off = ((size_t)b * DK + t) * H + h;
        qi = q[off];
        ki = k[((size_t)b * DK + t) * HKV + hk];
        if (!EJK) {
            gi = g[off];
            di = dt_bias ? dt_bias[(size_t)t * H + h] : 0.f;
        }
    }
    float4 s[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m)
        s[m] = load_stream(Sp + (size_t)(rg * RPT + m) * DV + cg * 4);
    // nothing of the prologue may be scheduled above the state loads: its first
    // use of a loaded value would hold back the rest of the stream
    __builtin_amdgcn_sched_barrier(0);

    // 2. prologue: norms, gate, beta
    const float zi = gi + di;
    {
        const float r0 = wave_sum(qi * qi), r1 = wave_sum(ki * ki), r2 = wave_sum(qi * ki);
        if (lane == 0) {
            sh_red[wave][0] = r0;
            sh_red[wave][1] = r1;
            sh_red[wave][2] = r2;
        }
    }
    lds_barrier();
    float sqq = 0.f, skk = 0.f, sqk = 0.f;
#pragma unroll
    for (int w = 0; w < NWAVES; ++w) {
        sqq += sh_red[w][0];
        skk += sh_red[w][1];
        sqk += sh_red[w][2];
    }
    const float nq = l2norm ? scale / sqrtf(sqq + kNormEps) : scale;
    const float nk = l2norm ? 1.0f / sqrtf(skk + kNormEps) : 1.0f;
    const float kq = sqk * nq * nk;  // kh . qh
    float bt, alpha_s = 1.0f;
    if (!EJK) {
        bt = sigmoid_f(braw);
    } else {
        bt = braw;
        alpha_s = g ? expf(draw) : 1.0f;
    }
    if (t < DK) {
        sh_q[t] = qi * nq;
        sh_k[t] = ki * nk;
        if (!EJK) sh_alpha[t] = expf(lower_bound * sigmoid_f(expf(araw) * zi));
    }
    lds_barrier();

    // 3. one sweep: decay (KDA) and the two column reductions
    float4 u = make_float4(0.f, 0.f, 0.f, 0.f), p = u;
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int r = rg * RPT + m;
        if (!EJK) {
            const float a = sh_alpha[r];
            s[m].x *= a; s[m].y *= a; s[m].z *= a; s[m].w *= a;
        }
        u = fma4(sh_k[r], s[m], u);
        p = fma4(sh_q[r], s[m], p);
    }
    // reduce over row groups: lanes of one wave that share cg, then waves
    if constexpr (NCG < kWave) {
        u.x = xor_sum_from<NCG>(u.x); u.y = xor_sum_from<NCG>(u.y);
        u.z = xor_sum_from<NCG>(u.z); u.w = xor_sum_from<NCG>(u.w);
        p.x = xor_sum_from<NCG>(p.x); p.y = xor_sum_from<NCG>(p.y);
        p.z = xor_sum_from<NCG>(p.z); p.w = xor_sum_from<NCG>(p.w);
    }
    if (NWAVES > 1) {
        if (lane < NCG) {
            sh_uv[wave][cg][0] = u;
            sh_uv[wave][cg][1] = p;
        }
        lds_barrier();
        u = sh_uv[0][cg][0];
        p = sh_uv[0][cg][1];
#pragma unroll
        for (int w = 1; w < NWAVES; ++w) {
            const float4 uw = sh_uv[w][cg][0], pw = sh_uv[w][cg][1];
            u.x += uw.x; u.y += uw.y; u.z += uw.z; u.w += uw.w;
            p.x += pw.x; p.y += pw.y; p.z += pw.z; p.w += pw.w;
        }
    }

    // 4. delta, output, new state (in place)
    const float4 vv = *reinterpret_cast<const float4*>(v + (size_t)kvitem * DV + cg * 4);
    float4 d;
    d.x = bt * (vv.x - u.x); d.y = bt * (vv.y - u.y);
    d.z = bt * (vv.z - u.z); d.w = bt * (vv.w - u.w);
    if (rg == 0) {
        float4 o;
        o.x = fmaf(d.x, kq, alpha_s * p.x); o.y = fmaf(d.y, kq, alpha_s * p.y);
        o.z = fmaf(d.z, kq, alpha_s * p.z); o.w = fmaf(d.w, kq, alpha_s * p.w);
        *reinterpret_cast<float4*>(out + (size_t)item * DV + cg * 4) = o;
    }
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int r = rg * RPT + m;
        const float kr = sh_k[r];
        float4 sn = s[m];
        if (EJK) {
            sn.x *= alpha_s; sn.y *= alpha_s; sn.z *= alpha_s; sn.w *= alpha_s;
        }
        sn = fma4(kr, d, sn);
        store_stream(Sp + (size_t)r * DV + cg * 4, sn);
    }
}

template <int DK, int DV>
hipError_t launch_dk_dv(const DecodeArgs& a, hipStream_t stream)
{
    const dim3 grid((unsigned)(((a.B + 7) / 8) * 8 * a.H));
    const dim3 block(DecodeShape<DK, DV>::THREADS);
    if (a.ejk)
        hipLaunchKernelGGL((decode_kernel<DK, DV, true>), grid, block, 0, stream, a.q, a.k, a.g, a.v,
                           a.beta, a.a_log, a.dt_bias, a.scale, a.lower_bound, a.B, a.H, a.Hkv, (int)a.l2norm,
                           a.out, a.S);
    else
        hipLaunchKernelGGL((decode_kernel<DK, DV, false>), grid, block, 0, stream, a.q, a.k, a.g, a.v,
                           a.beta, a.a_log, a.dt_bias, a.scale, a.lower_bound, a.B, a.H, a.Hkv, (int)a.l2norm,
                           a.out, a.S);
    return hipGetLastError();
}

template <int DK>
hipError_t launch_dk(const DecodeArgs& a, hipStream_t stream)
{
    switch (a.dv) {
    case 16: return launch_dk_dv<DK, 16>(a, stream);
    case 32: return launch_dk_dv<DK, 32>(a, stream);
    case 64: return launch_dk_dv<DK, 64>(a, stream);
    default: return launch_dk_dv<DK, 128>(a, stream);
    }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream)
{
    switch (a.dk) {
    case 16: return launch_dk<16>(a, stream);
    case 32: return launch_dk<32>(a, stream);
    case 64: return launch_dk<64>(a, stream);
    default: return launch_dk<128>(a, stream);
    }
}

}  // namespace kda
