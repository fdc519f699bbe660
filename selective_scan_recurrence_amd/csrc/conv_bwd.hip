// Backward of the standalone depthwise causal conv (the ggmlR extension's
// ssm_conv backward, "ggmlR tests/testthat/test-ssm-rwkv.R", the ssm_conv
// backward block: ggml_ssm_conv_back packs the gradient of sx followed by the
// gradient of the weights).  With z_t = sum_j sx[t+j] w[j] and out_t = z_t,
// or SiLU(z_t):
//   g_t       = dout_t                                   (no SiLU)
//   g_t       = dout_t s(z_t) (1 + z_t (1 - s(z_t)))     (SiLU; s the logistic)
//   d_sx[tau] = sum over j of w[j] g_{tau - j}           (0 <= tau - j < n_t)
//   d_w[j]    = sum over sequences and t of g_t sx[t + j]
//
// One workgroup owns 64 channels of one sequence and 128 positions tau of
// sx.  It stages the gradient rows it needs (tau - K + 1 .. tau, channel-
// fastest in memory) transposed into LDS, and the sx rows around them (time-
// fastest) for the SiLU derivative and the weight gradient; then it writes
// d_sx rows along time and a partial weight gradient over its own 128
// tokens.  A second kernel sums the partials in a fixed order (sequence, then
// tile), so results repeat bitwise.  HBM-bound: sx, dout and d_sx each cross
// HBM once, plus the K-1 halo rows of each tile.
#include "device_common.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

constexpr int kBC = 64;     // channels per workgroup
constexpr int kBT = 128;    // positions of sx per workgroup
constexpr int kMaxK = 8;
constexpr int kGP = kBT + kMaxK + 1;        // LDS pitch of a channel's gradient row (odd)
constexpr int kSP = kBT + 2 * kMaxK + 1;    // LDS pitch of a channel's sx row (odd)

template <typename T>
__global__ __launch_bounds__(256) void conv_bwd_tiled(const T* __restrict__ sx,
                                                      const float* __restrict__ w,
                                                      const float* __restrict__ dout,
                                                      float* __restrict__ d_sx,
                                                      float* __restrict__ dw_part, int n_t,
                                                      int d_inner, int K, int apply_silu, int vec) {
    __shared__ float gl[kBC * kGP];  // [channel][r]: gradient at t = tau0 - (K-1) + r
    __shared__ float sl[kBC * kSP];  // [channel][r]: sx at tau0 - (K-1) + r
    const int tid = threadIdx.x;
    const int s = blockIdx.z, c0 = blockIdx.y * kBC, tau0 = blockIdx.x * kBT;
    const int len = n_t + K - 1;
    const int lo = tau0 - (K - 1);        // first token of the gradient window
    const int g_rows = kBT + K - 1;       // gradient rows t = lo .. tau0 + kBT - 1
    const int s_span = kBT + 2 * (K - 1); // sx positions lo .. tau0 + kBT + K - 2

    // sx rows: lanes along time within a channel (contiguous reads)
    const T* sxs = sx + (int64_t)s * d_inner * len;
    for (int e = tid; e < kBC * s_span; e += 256) {
        const int cc = e / s_span, r = e - cc * s_span;
        const int c = c0 + cc, p = lo + r;
        sl[cc * kSP + r] = (c < d_inner && p >= 0 && p < len) ? to_f32(sxs[(int64_t)c * len + p]) : 0.0f;
    }
    // gradient rows: 16 lanes x 4 channels per token row (contiguous reads),
    // written transposed
    const float* gs = dout + (int64_t)s * n_t * d_inner;
    for (int e = tid; e < g_rows * (kBC / 4); e += 256) {
        const int r = e / (kBC / 4), cq = (e % (kBC / 4)) * 4;
        const int t = lo + r;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (t >= 0 && t < n_t) {
            const float* src = gs + (int64_t)t * d_inner + c0 + cq;
            if (vec && c0 + cq + 3 < d_inner) {  // 16-byte aligned rows
                v = *reinterpret_cast<const float4*>(src);
            } else {
                if (c0 + cq + 3 < d_inner) v.w = src[3];
                if (c0 + cq < d_inner) v.x = src[0];
                if (c0 + cq + 1 < d_inner) v.y = src[1];
                if (c0 + cq + 2 < d_inner) v.z = src[2];
            }
        }
        gl[(cq + 0) * kGP + r] = v.x;
        gl[(cq + 1) * kGP + r] = v.y;
        gl[(cq + 2) * kGP + r] = v.z;
        gl[(cq + 3) * kGP + r] = v.w;
    }
    __syncthreads();

    // the SiLU derivative at the recomputed pre-activation: g *= s(z)(1 + z(1 - s(z)))
    if (apply_silu) {
        for (int e = tid; e < kBC * g_rows; e += 256) {
            const int cc = e / g_rows, r = e - cc * g_rows;
            const int c = c0 + cc;
            if (c >= d_inner) continue;
            float z = 0.0f;
            for (int j = 0; j < K; ++j) z = fmaf(sl[cc * kSP + r + j], w[(int64_t)c * K + j], z);
            const float sg = __builtin_amdgcn_rcpf(1.0f + fast_exp2(-z * kLog2e));
            gl[cc * kGP + r] *= sg * fmaf(z, 1.0f - sg, 1.0f);
        }
        __syncthreads();
    }

    // d_sx rows: lanes along time (two channels per pass of 256 lanes)
    {
        const int tt = tid & (kBT - 1);
        const int tau = tau0 + tt;
        float* dst = d_sx + (int64_t)s * d_inner * len;
        for (int cc = tid >> 7; cc < kBC; cc += 2) {
            const int c = c0 + cc;
            if (c >= d_inner || tau >= len) continue;
            float acc = 0.0f;
            for (int j = 0; j < K; ++j) acc = fmaf(w[(int64_t)c * K + j], gl[cc * kGP + tt + K - 1 - j], acc);
            dst[(int64_t)c * len + tau] = acc;
        }
    }

    // partial weight gradient over this tile's own tokens t = tau0 .. tau0+127
    // (< n_t): lane = channel, four quarters of the tokens, then summed in order
    {
        const int cc = tid & (kBC - 1), part = tid >> 6;
        float acc[kMaxK];
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) acc[j] = 0.0f;
        for (int k = 0; k < kBT / 4; ++k) {
            const int tt = part * (kBT / 4) + k;
            if (tau0 + tt >= n_t) break;
            const float gv = gl[cc * kGP + tt + K - 1];
#pragma unroll
            for (int j = 0; j < kMaxK; ++j)
                if (j < K) acc[j] = fmaf(gv, sl[cc * kSP + tt + K - 1 + j], acc[j]);
        }
        __syncthreads();  // gl is reused for the four partial rows
#pragma unroll
        for (int j = 0; j < kMaxK; ++j)
            if (j < K) gl[(part * kBC + cc) * kMaxK + j] = acc[j];
        __syncthreads();
        if (part == 0 && c0 + cc < d_inner) {
            float* pd = dw_part + (((int64_t)s * gridDim.x + blockIdx.x) * d_inner + c0 + cc) * K;
            for (int j = 0; j < K; ++j) {
                float v = 0.0f;
#pragma unroll
                for (int q = 0; q < 4; ++q) v += gl[(q * kBC + cc) * kMaxK + j];
                pd[j] = v;
            }
        }
    }
}

// d_w[c][j]: the partials of every (sequence, tile) in that order.
__global__ __launch_bounds__(256) void conv_bwd_reduce_w(const float* __restrict__ dw_part,
                                                         float* __restrict__ d_w, int n_parts,
                                                         int d_inner, int K) {
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e >= d_inner * K) return;
    float acc = 0.0f;
    for (int q = 0; q < n_parts; ++q) acc += dw_part[(int64_t)q * d_inner * K + e];
    d_w[e] = acc;
}

}  // namespace

size_t conv_bwd_workspace_bytes(int64_t n_s, int64_t n_t, int64_t d_inner, int d_conv) {
    const int64_t len = n_t + d_conv - 1;
    const int64_t tiles = (len + kBT - 1) / kBT;
    return (size_t)(n_s * tiles * d_inner * d_conv) * sizeof(float);
}

int launch_conv_bwd(const void* sx, const float* w, const float* dout, float* dgrad, int64_t n_s,
                    int64_t n_t, int64_t d_inner, int d_conv, int io, int apply_silu, void* ws,
                    hipStream_t stream) {
    if (d_conv > kMaxK) return SSM_ERR_UNSUPPORTED;
    const int64_t len = n_t + d_conv - 1;
    const int64_t tiles = (len + kBT - 1) / kBT;
    float* d_w = dgrad + n_s * d_inner * len;
    float* part = static_cast<float*>(ws);
    const int vec = (d_inner % 4 == 0) && ((reinterpret_cast<uintptr_t>(dout) & 15) == 0);
    if (n_s > 0 && len > 0) {
        dim3 grid((unsigned)tiles, (unsigned)((d_inner + kBC - 1) / kBC), (unsigned)n_s);
        if (io == SSM_F32)
            hipLaunchKernelGGL(conv_bwd_tiled<float>, grid, dim3(256), 0, stream,
                               static_cast<const float*>(sx), w, dout, dgrad, part, (int)n_t,
                               (int)d_inner, d_conv, apply_silu, vec);
        else
            hipLaunchKernelGGL(conv_bwd_tiled<bf16_t>, grid, dim3(256), 0, stream,
                               static_cast<const bf16_t*>(sx), w, dout, dgrad, part, (int)n_t,
                               (int)d_inner, d_conv, apply_silu, vec);
    }
    const int n_parts = (int)(n_s * tiles);
    hipLaunchKernelGGL(conv_bwd_reduce_w, dim3((unsigned)((d_inner * d_conv + 255) / 256)), dim3(256),
                       0, stream, part, d_w, n_parts, (int)d_inner, d_conv);
    return hipGetLastError() == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

}  // namespace ssm
