// Internal interface between the C ABI (ssm_api.hip) and the kernel files.
// Not installed; the public interface is include/ssm.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ssm.h"

namespace ssm {

// Tokens between the states the forward stores for the backward (the backward's
// block length).
constexpr int kCkpt = 8;

// Checked, expanded scan dimensions.
struct Shape {
    int64_t S, L, H, P, N, G, R;  // seqs, tokens, heads, head_dim, d_state, groups, state rows
    int a_per_state;
    int K;                        // conv taps (0 = none)
    int chunk;                    // requested chunk (0 = auto)
    int io;                       // SSM_F32 / SSM_BF16
    uint32_t flags;
    int64_t d_inner() const { return H * P; }
    int io_bytes() const { return io == SSM_BF16 ? 2 : 4; }
    int64_t nelem_x() const { return S * L * H * P; }
    int64_t nelem_state() const { return S * H * P * N; }
    int64_t nelem_A() const { return a_per_state ? H * N : H; }
    int64_t nelem_BC() const { return S * L * G * N; }
};

struct FwdArgs {
    Shape sh;
    const float* s;
    const void* x;
    const void* dt;
    const float* A;
    const void* B;
    const void* C;
    const float* D;
    const int32_t* ids;
    const float* conv_w;
    const float* conv_state;
    void* y;               // y block of the packed result
    float* state_out;      // state block of the packed result
    float* conv_state_out;
    uint32_t* err;         // device-error word (workspace)
    char* ws;              // workspace after the error word
    size_t ws_bytes;
    // extras (selective_scan_fwd_ext); all null / S*L for the plain call
    const float* dt_bias;
    const void* z;
    const int32_t* cu;     // [S+1] spans on the packed token axis, or null
    int64_t T;             // tokens on the packed axis (S*L without cu)
    bool has_ext() const { return dt_bias || z || cu; }
};

struct BwdArgs {
    Shape sh;
    const float* s;
    const void* x;
    const void* dt;
    const float* A;
    const void* B;
    const void* C;
    const float* D;
    const int32_t* ids;
    const void* dy;
    const float* dstate;
    const float* conv_w;      // with the fused conv (d_conv > 0), else null
    const float* conv_state;  // nullable: zeros
    float *d_s, *d_x, *d_dt, *d_A, *d_B, *d_C, *d_D;
    float *d_conv_w, *d_conv_state;  // with the fused conv, else null
    uint32_t* err;
    char* ws;
    size_t ws_bytes;
};

struct DecodeArgs {
    Shape sh;              // n_tokens (L) is 1
    float* s;              // state rows, updated in place
    const void* x;
    const void* dt;
    const float* dt_bias;  // nullable
    const float* A;
    const void* B;
    const void* C;
    const float* D;        // nullable
    const void* z;         // nullable
    const int32_t* ids;
    const float* conv_w;   // with K > 0
    float* conv_state;     // with K > 0, updated in place
    void* y;
    uint32_t* err;         // nullable device-error word
};

constexpr size_t kErrBytes = 256;  // the device-error word's slot at the workspace start

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Workspace needed after the error slot.
size_t fwd_workspace_bytes(const Shape& sh);
size_t bwd_workspace_bytes(const Shape& sh);

// Mamba-1 forward for d_state <= 16 with four lanes per channel.
bool quad_supported(const Shape& sh);
size_t quad_workspace_bytes(const Shape& sh);
bool quad_chunked(const Shape& sh);
// relay_k_out: decide the launch without making it and report the relay
// pieces per split job (0: no relay)
int launch_quad_fwd(const FwdArgs& a, hipStream_t stream, int* relay_k_out = nullptr);
// The backward's checkpoint pass: the state entering every kCkpt-token block into ckpt.
// relay_h, relay_flag: room for relay_max_jobs cut jobs of the relay split
// (64 x 16 floats and a flag each, flags zero), or null: no split
int launch_quad_ckpt(const BwdArgs& a, float* ckpt, float* relay_h, int* relay_flag, int relay_max_jobs,
                     hipStream_t stream);

// Mamba-1 forward, d_state 16, time split across the waves of a workgroup
// (for batches with too few channels to fill the GPU otherwise).
bool ts_supported(const Shape& sh, const FwdArgs& a);
int launch_ts_fwd(const FwdArgs& a, hipStream_t stream);

// Mamba-2 form (scalar A per head), bf16 io, no conv: chunked products on MFMA.
bool ssd_supported(const Shape& sh, const FwdArgs& a);
int launch_ssd_fwd(const FwdArgs& a, hipStream_t stream);

// Backward: Mamba-1 form, d_state <= 16, one group, no fused conv.
bool bwd_supported(const Shape& sh);

// Backward of the Mamba-2 form (bf16 io, head_dim 32/64, d_state 64/128, no
// conv): chunked products on MFMA.
bool ssd_bwd_supported(const Shape& sh);
size_t ssd_bwd_workspace_bytes(const Shape& sh);
int launch_ssd_bwd(const BwdArgs& a, hipStream_t stream);

// The forward's kernel family for a call (host-side decision only).
enum class FwdPath { kNone, kTimeSplit, kQuad, kSsd, kRows };
FwdPath fwd_path(const FwdArgs& a);

// Backward for every other shape, and the fused conv: one lane group per
// (sequence, channel) row.
bool rows_bwd_supported(const Shape& sh);
size_t rows_bwd_workspace_bytes(const Shape& sh);
int launch_rows_bwd(const BwdArgs& a, hipStream_t stream);

// Returns SSM_OK, SSM_ERR_UNSUPPORTED, or SSM_ERR_HIP.
int launch_scan_fwd(const FwdArgs& a, hipStream_t stream);
int launch_scan_bwd(const BwdArgs& a, hipStream_t stream);
int launch_conv_fwd(const void* sx, const float* w, void* out, int64_t n_s, int64_t n_t,
                    int64_t d_inner, int d_conv, int io, int apply_silu, hipStream_t stream);
size_t conv_bwd_workspace_bytes(int64_t n_s, int64_t n_t, int64_t d_inner, int d_conv);
int launch_state_update(const DecodeArgs& a, hipStream_t stream);
int launch_conv_bwd(const void* sx, const float* w, const float* dout, float* dgrad, int64_t n_s,
                    int64_t n_t, int64_t d_inner, int d_conv, int io, int apply_silu, void* ws,
                    hipStream_t stream);

// Chunk checkpoints of the Mamba-2 backward, written by the forward's
// recompute (ssd_fwd.hip) and read by ssd_bwd.hip.  The fp32 state [P][N]
// entering a chunk is kept as 16-byte pieces in the order the forward's 8
// waves hold it in their MFMA accumulators: wave w = NS sp + sh owns channels
// 16 sp .. + 15 and state tiles NH sh .. + NH - 1, and lane l16 + 16 g4 of
// its tile j holds channel 16 sp + l16, states 16 (NH sh + j) + 4 g4 .. + 3.
// Each store instruction of the writer then covers 1 KB of whole cache lines
// (a [P][N] row order would give it 64-byte halves of 16 lines).
template <int P, int N>
struct SsdCkptLayout {
    static constexpr int PB = P / 16, NS = 8 / PB, NH = N / NS / 16;
    static __device__ __forceinline__ int piece(int wave, int j, int lane) { return (wave * NH + j) * 64 + lane; }
    // channel p and first state n0 of piece e
    static __device__ __forceinline__ void pn(int e, int& p, int& n0) {
        const int lane = e & 63, wj = e >> 6, j = wj % NH, w = wj / NH;
        p = 16 * (w / NS) + (lane & 15);
        n0 = 16 * (NH * (w % NS) + j) + 4 * (lane >> 4);
    }
};

}  // namespace ssm
