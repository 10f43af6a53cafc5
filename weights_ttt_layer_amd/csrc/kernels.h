// kernels.h -- host-side launch interface between the C ABI (ttt_abi.hip) and the
// kernel translation units. Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace ttt {

struct LinearArgs {
    int kind;          // 0 plain, 1 LayerNorm + residual
    int dtype;         // 0 fp32, 1 bf16 token streams
    int B, H, N, d, b;
    const void* Q;
    const void* K;
    const void* V;
    const float* eta;  // [B,H,N] or nullptr
    float eta_const;
    const float* W0;
    const float* gamma;
    const float* beta;
    float eps;
    float* Z;
    float* W_end;
    void* workspace;
    size_t workspace_bytes;
};

struct MlpArgs {
    int dtype;
    int B, H, N, d, hidden, b;
    const void* Q;
    const void* K;
    const void* V;
    const float* eta;
    float eta_const;
    const float* W1;
    const float* W2;
    const float* gamma;
    const float* beta;
    float eps;
    float* Z;
    float* W1_end;
    float* W2_end;
};

// Small-b path: one workgroup per (sequence, head); d = 64 or 128, 1 <= b <= 64.
hipError_t launch_smallb_linear(const LinearArgs& a, hipStream_t stream);
// The generic small-b kernel (midb_linear.hip): d = 64 with 17 <= b <= 64, d = 128
// with 1 <= b <= 64, fp32 or bf16 streams.
hipError_t launch_midb_linear(const LinearArgs& a, hipStream_t stream);
// Plain f with chunks longer than 64 tokens, d = 64 or 128, fp32 or bf16 streams,
// any N: the same kernel in blocks of 64 tokens (no workspace). `outputs` is an
// LC_OUT_* value (below): the dual form's outputs or a block-causal mode.
hipError_t launch_midb_linear_blocks(const LinearArgs& a, int outputs, hipStream_t stream);
// bf16 token streams: the chain-on-one-wave kernel (smallb_chain.hip)
hipError_t launch_smallb_chain(const LinearArgs& a, hipStream_t stream);
// The same kernel on two-term streams: Q, K, V each a bf16 hi plane [B,H,N,d]
// followed directly by its lo plane (the whole layer's projected streams).
hipError_t launch_smallb_chain_terms2(const LinearArgs& a, hipStream_t stream);

// Large-chunk path (plain f, bf16, d = 128, b % 128 == 0). `outputs` selects the
// dual-form outputs (causal inside a chunk) or block-causal ones taken with the
// chunk's starting or ending weights.
enum { LC_OUT_DUAL = 0, LC_OUT_BEFORE = 1, LC_OUT_AFTER = 2 };
size_t large_chunk_workspace_bytes(int B, int H, int N, int d, int b);
hipError_t launch_large_chunk_linear(const LinearArgs& a, int outputs, hipStream_t stream);

// Single-token decode step: one wave per (sequence, head), d = 64.
hipError_t launch_decode_linear(const LinearArgs& a, hipStream_t stream);

// TTT-MLP small-b path: d = 64, hidden = 256, 1 <= b <= 16 (state in registers).
hipError_t launch_smallb_mlp(const MlpArgs& a, hipStream_t stream);
// TTT-MLP for d = 64 with 17 <= b <= 64 and d = 128 with 1 <= b <= 64: state
// and the chunk's intermediates in the caller's workspace (mlp_generic.hip).
size_t mlp_generic_workspace_bytes(int B, int H, int d, int b);
hipError_t launch_mlp_generic(const MlpArgs& a, void* workspace, hipStream_t stream);

// Backward of TTT-Linear (plain / LN), d = 64, 1 <= b <= 16. `f` carries the
// forward's inputs and the workspace (chunk-start states and per-unit partials).
struct BwdArgs {
    LinearArgs f;
    const float* dZ;
    const float* dW_end;   // or nullptr (zero)
    float* dQ;
    float* dK;
    float* dV;
    float* deta;
    float* dW0;
    float* dgamma;
    float* dbeta;
};
size_t bwd_workspace_bytes(int B, int H, int N, int b);
hipError_t launch_bwd_linear(const BwdArgs& a, hipStream_t stream);

// Whole-layer stages around the inner model (head width 64, D % 64 == 0).
struct LayerArgs {
    int B, N, D, H;
    const void* x;     // [B, N, D] bf16
    const void* Wq;    // [H*64, D] bf16
    const void* Wk;
    const void* Wv;
    const void* Wo;    // [D, H*64] bf16
    const float* out_gamma;
    const float* out_beta;
    float eps;
    float* y;          // [B, N, D] fp32
};
// Bytes of one fp32 [B, H, N, 64] workspace array, rounded up to 256.
size_t layer_workspace_region_bytes(int B, int N, int H);
// Q, K (unit rows), V, each as two bf16 planes [B, H, N, 64]: the RNE rounding
// (hi) and the rounding of the remainder (lo), the lo plane right after the hi.
hipError_t launch_layer_qkv(const LayerArgs& a, uint16_t* Q, uint16_t* K, uint16_t* V, hipStream_t stream);
// y = W_O (LayerNorm(Z) * out_gamma + out_beta + Q), per head, Q as the two
// planes above; `aext` is one workspace region that receives the two-term operand.
hipError_t launch_layer_out(const LayerArgs& a, const float* Z, const uint16_t* Q, void* aext, hipStream_t stream);

}  // namespace ttt
