// kda_internal.h - argument blocks passed from the C ABI layer to the kernel
// launchers.  Arguments are already validated when these are filled.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

struct PrefillArgs {
    const void* q;
    const void* k;
    const void* v;
    bool in_bf16;
    const float* g;        // KDA: [Ntok, H, dk]; EJK: [Ntok, H] or null
    const float* beta;     // [Ntok, H]
    const float* a_log;    // [H]
    const float* dt_bias;  // [dk, H] or null
    const float* init;     // [N, H, dk, dv] or null
    const int32_t* cu;     // [N + 1] or null (dense: sequence n = batch row n)
    int N;                 // number of sequences (dense: B)
    int T;                 // dense: tokens per sequence; packed: total tokens
    int H, dk, dv;
    int Hkv;               // key/value heads: head h reads k and v of head h / (H / Hkv)
    float scale;
    float lower_bound;
    bool l2norm;
    bool ejk;
    void* o;               // [Ntok, H, dv]
    bool out_bf16;
    float* final_state;    // [N, H, dk, dv] or null
    void* workspace;
    size_t workspace_bytes;
    int tstride;           // dense: rows between sequence starts (0 = T; set for a segment of longer sequences)
};

struct DecodeArgs {
    const float* q;
    const float* k;
    const float* g;
    const float* v;
    const float* beta;
    const float* a_log;
    const float* dt_bias;
    float scale;
    float lower_bound;
    int B, H, dk, dv;
    int Hkv;               // key/value heads (k [B, dk, Hkv], v [B, Hkv, dv])
    bool l2norm;
    bool ejk;
    float* out;
    float* S;
};

struct BackwardArgs {
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
    int N, T, H, Hkv, dk, dv;
    float scale;
    float lower_bound;
    int l2norm;
    bool ejk;
    const void* d_o;
    int do_bf16;
    const float* d_final_state;
    float* dq;
    float* dk_out;
    float* dv_out;
    float* dg;
    float* dbeta;
    float* da_log;
    float* ddt_bias;
    float* d_initial_state;
    void* workspace;
};

struct GatedArgs {
    const void* q;
    const void* k;
    const void* v;
    int in_bf16;
    const float* g;
    const float* g_gamma;
    int g_gamma_rows;
    const float* gk;
    const float* gv;
    const float* init;
    const int32_t* cu;
    int N, T, H, Hkv, dk, dv;
    float scale;
    int reverse;
    void* o;
    int out_bf16;
    float* final_state;
    void* workspace;   // gated_workspace_bytes(N, T, H, dk, packed) bytes
};

// Each launcher returns the hipError_t of its launch (hipGetLastError).
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
// the recurrent kernel, one object per key dimension
hipError_t launch_recurrent_dk16(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_recurrent_dk32(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_recurrent_dk64(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_recurrent_dk128(const PrefillArgs& a, hipStream_t stream);
inline hipError_t launch_recurrent(const PrefillArgs& a, hipStream_t stream)
{
    switch (a.dk) {
    case 16: return launch_recurrent_dk16(a, stream);
    case 32: return launch_recurrent_dk32(a, stream);
    case 64: return launch_recurrent_dk64(a, stream);
    default: return launch_recurrent_dk128(a, stream);
    }
}
hipError_t launch_chunked(const PrefillArgs& a, hipStream_t stream);
bool chunked_supported(const PrefillArgs& a);
size_t chunked_workspace_bytes(int N, int T, int H, int dk, int dv, bool packed);
// the least workspace with which a dense call still runs (in segments of whole
// chunks of every sequence): one chunk's records per (sequence, head), plus the
// state carried between segments when final_state is not given
size_t chunked_min_workspace_bytes(int N, int H, int dk, int dv, bool carry);
// the float32 chunked kernel (16-token chunks on the vector ALUs)
hipError_t launch_chunked_f32(const PrefillArgs& a, hipStream_t stream);
bool chunked_f32_supported(const PrefillArgs& a);
// the float32-arithmetic route in two kernels on 16-token chunks (the
// backward's operand blocks, then a scan that forms the output), taken over
// from launch_chunked_f32 when H dk >= 128 and the workspace holds the blocks
bool prefill16_preferred(int N, int H, int dk);
size_t prefill16_workspace_bytes(int N, int T, int H, int dk, bool packed);
hipError_t launch_prefill16(const PrefillArgs& a, hipStream_t stream);
// the gated recurrent attention (kda_gated.hip)
hipError_t launch_gated(const GatedArgs& a, hipStream_t stream);
size_t gated_workspace_bytes(int N, int T, int H, int dk, bool packed);
// the prefill backward (kda_backward.hip)
hipError_t launch_backward(const BackwardArgs& a, hipStream_t stream);
size_t backward_workspace_bytes(int N, int T, int H, int Hkv, int dk, int dv, bool packed);
// device address, on the current device, of the fixed scratch array of
// KDA_NOALLOC_SCRATCH_BYTES that kda_prefill_noalloc uses as its workspace
hipError_t noalloc_scratch(void** out);

}  // namespace kda
