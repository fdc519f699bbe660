// Standalone depthwise causal conv, the ggml ssm_conv operator of the ggmlR
// page ("ggml_ssm_conv matches a depthwise convolution computed in R"):
//   out[s][t][c] = sum_{j<K} sx[s][c][t + j] * w[c][j]     (then SiLU if asked)
// sx is time-fastest and out channel-fastest, so each block stages a
// [64 channels][64 + K - 1 tokens] tile of sx in LDS with loads that are
// contiguous along time, then writes out with stores contiguous along
// channels.  HBM-bound: every input element is read once and every output
// written once (plus the K-1 halo tokens per tile).
#include "device_common.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

constexpr int kTileC = 64;
constexpr int kTileT = 64;
constexpr int kMaxK = 8;

template <typename T>
__global__ __launch_bounds__(256) void conv_fwd_tiled(const T* __restrict__ sx,
                                                      const float* __restrict__ w,
                                                      T* __restrict__ out, int n_t, int d_inner,
                                                      int K, int apply_silu) {
    __shared__ float tile[kTileC][kTileT + kMaxK];  // +K-1 halo, padded against bank conflicts
    const int s = blockIdx.z;
    const int c0 = blockIdx.y * kTileC;
    const int t0 = blockIdx.x * kTileT;
    const int len = n_t + K - 1;
    const int span = kTileT + K - 1;
    const T* src = sx + (int64_t)s * d_inner * len;
    // load: lanes run along time within a channel row
    for (int e = threadIdx.x; e < kTileC * span; e += blockDim.x) {
        const int cc = e / span, tt = e - cc * span;
        const int c = c0 + cc, t = t0 + tt;
        tile[cc][tt] = (c < d_inner && t < len) ? to_f32(src[(int64_t)c * len + t]) : 0.0f;
    }
    __syncthreads();
    // compute: lanes run along channels within a token
    const int cc = threadIdx.x % kTileC;
    const int c = c0 + cc;
    if (c >= d_inner) return;
    float wk[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) wk[j] = j < K ? w[(int64_t)c * K + j] : 0.0f;
    T* dst = out + (int64_t)s * n_t * d_inner + c;
    for (int tt = threadIdx.x / kTileC; tt < kTileT; tt += blockDim.x / kTileC) {
        const int t = t0 + tt;
        if (t >= n_t) break;
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < kMaxK; ++j)
            if (j < K) acc = fmaf(tile[cc][tt + j], wk[j], acc);
        store_io(dst + (int64_t)t * d_inner, apply_silu ? silu(acc) : acc);
    }
}

}  // namespace

int launch_conv_fwd(const void* sx, const float* w, void* out, int64_t n_s, int64_t n_t,
                    int64_t d_inner, int d_conv, int io, int apply_silu, hipStream_t stream) {
    if (n_s == 0 || n_t == 0) return SSM_OK;
    if (d_conv > kMaxK) return SSM_ERR_UNSUPPORTED;
    dim3 grid((unsigned)((n_t + kTileT - 1) / kTileT), (unsigned)((d_inner + kTileC - 1) / kTileC),
              (unsigned)n_s);
    if (io == SSM_F32)
        hipLaunchKernelGGL(conv_fwd_tiled<float>, grid, dim3(256), 0, stream,
                           static_cast<const float*>(sx), w, static_cast<float*>(out), (int)n_t,
                           (int)d_inner, d_conv, apply_silu);
    else
        hipLaunchKernelGGL(conv_fwd_tiled<bf16_t>, grid, dim3(256), 0, stream,
                           static_cast<const bf16_t*>(sx), w, static_cast<bf16_t*>(out), (int)n_t,
                           (int)d_inner, d_conv, apply_silu);
    return hipGetLastError() == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

}  // namespace ssm
