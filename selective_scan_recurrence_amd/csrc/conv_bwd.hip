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

#include <type_traits>

namespace ssm {
namespace {

constexpr int kBC = 64;     // channels per workgroup
constexpr int kBT = 128;    // positions of sx per workgroup
constexpr int kMaxK = 8;
constexpr int kGP = kBT + kMaxK + 1;        // LDS pitch of a channel's gradient row (odd)
constexpr int kSP = kBT + 2 * kMaxK + 1;    // LDS pitch of a channel's sx row (odd)

template <typename T, int K>
__global__ __launch_bounds__(256) void conv_bwd_tiled(const T* __restrict__ sx,
                                                      const float* __restrict__ w,
                                                      const float* __restrict__ dout,
                                                      float* __restrict__ d_sx,
                                                      float* __restrict__ dw_part, int n_t,
                                                      int d_inner, int apply_silu, int vec) {
    __shared__ float gl[kBC * kGP];  // [channel][r]: gradient at t = tau0 - (K-1) + r
    __shared__ float sl[kBC * kSP];  // [channel][r]: sx at tau0 - (K-1) + r
    __shared__ float wl[kBC * kMaxK];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int s = blockIdx.z, c0 = blockIdx.y * kBC, tau0 = blockIdx.x * kBT;
    const int len = n_t + K - 1;
    const int lo = tau0 - (K - 1);        // first token of the gradient window
    const int g_rows = kBT + K - 1;       // gradient rows t = lo .. tau0 + kBT - 1
    const int s_span = kBT + 2 * (K - 1); // sx positions lo .. tau0 + kBT + K - 2

    for (int e = tid; e < kBC * kMaxK; e += 256) {
        const int cc = e >> 3, j = e & (kMaxK - 1);
        wl[e] = (c0 + cc < d_inner && j < K) ? w[(int64_t)(c0 + cc) * K + j] : 0.0f;
    }
    // Every load of the tile is issued before the first LDS store, so that
    // their latencies overlap (the trip counts are fixed by kMaxK), and goes
    // through a buffer descriptor whose range ends the row or the tensor:
    // positions outside it read as zero, with no branch around the load.
    constexpr int kSR = (kBT + 2 * (kMaxK - 1) + 63) / 64;  // 64-position passes per sx row
    constexpr int kGR = (kBT + kMaxK - 1 + 15) / 16;        // 16-row passes over the gradient rows
    constexpr int ES = (int)sizeof(T);
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const char* sxs = reinterpret_cast<const char*>(sx) + (int64_t)s * d_inner * len * ES;
    float sv[kBC / 4][kSR];
#pragma unroll
    for (int i = 0; i < kBC / 4; ++i) {
        const int c = c0 + wv + 4 * i;
        const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(sxs) + (int64_t)c * len * ES, 0,
                                                          c < d_inner ? len * ES : 0, 0x00020000);
#pragma unroll
        for (int m = 0; m < kSR; ++m) {
            const int p = lo + lane + 64 * m;  // negative positions wrap past the range
            if constexpr (ES == 2)
                sv[i][m] = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, p * ES, 0, 0) << 16);
            else
                sv[i][m] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, p * ES, 0, 0));
        }
    }
    // gradient rows: 16 lanes x 4 channels per token row, written transposed
    const char* gs = reinterpret_cast<const char*>(dout + (int64_t)s * n_t * d_inner);
    const auto rg = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(gs), 0, n_t * d_inner * 4, 0x00020000);
    const int cq = (tid & 15) * 4;
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    f32x4 gv4[kGR];
#pragma unroll
    for (int i = 0; i < kGR; ++i) {
        const int t = lo + (tid >> 4) + 16 * i;   // rows before 0 wrap past the range
        const int off = (t * d_inner + c0 + cq) * 4;
        if (vec) {
            gv4[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rg, off, 0, 0));
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                gv4[i][k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rg, off + 4 * k, 0, 0));
        }
    }
#pragma unroll
    for (int i = 0; i < kBC / 4; ++i)
#pragma unroll
        for (int m = 0; m < kSR; ++m) {
            const int r = lane + 64 * m;
            if (r < s_span) sl[(wv + 4 * i) * kSP + r] = sv[i][m];
        }
#pragma unroll
    for (int i = 0; i < kGR; ++i) {
        const int r = (tid >> 4) + 16 * i;
        if (r < g_rows) {
            gl[(cq + 0) * kGP + r] = gv4[i][0];
            gl[(cq + 1) * kGP + r] = gv4[i][1];
            gl[(cq + 2) * kGP + r] = gv4[i][2];
            gl[(cq + 3) * kGP + r] = gv4[i][3];
        }
    }
    __syncthreads();

    // lane = channel for the SiLU factor and the weight gradient; each wave
    // takes a quarter of the rows and slides a K-wide window of sx along them
    // (one LDS read per row)
    const int cc = lane;
    float wk[K];
#pragma unroll
    for (int j = 0; j < K; ++j) wk[j] = wl[cc * kMaxK + j];
    const float* slc = sl + cc * kSP;
    float* glc = gl + cc * kGP;

    // the SiLU derivative at the recomputed pre-activation: g *= s(z)(1 + z(1 - s(z))).
    // Rows past the window (up to 4 * RQ) hold no data and are never read back.
    if (apply_silu) {
        constexpr int RQ = (kBT + K - 1 + 3) / 4;
        static_assert(4 * RQ <= kGP && 4 * RQ + K - 1 <= kSP, "rows of the SiLU pass stay in the tiles");
        const int r0 = wv * RQ;
        float win[K];
#pragma unroll
        for (int j = 0; j < K - 1; ++j) win[j + 1] = slc[r0 + j];
#pragma unroll
        for (int k = 0; k < RQ; ++k) {
#pragma unroll
            for (int j = 0; j < K - 1; ++j) win[j] = win[j + 1];
            win[K - 1] = slc[r0 + k + K - 1];
            float z = 0.0f;
#pragma unroll
            for (int j = 0; j < K; ++j) z = fmaf(win[j], wk[j], z);
            const float sg = __builtin_amdgcn_rcpf(1.0f + fast_exp2(-z * kLog2e));
            glc[r0 + k] *= sg * fmaf(z, 1.0f - sg, 1.0f);
        }
        __syncthreads();
    }

    // partial weight gradient over this tile's own tokens t = tau0 .. tau0+127
    // (< n_t): a quarter of the tokens per wave, then summed in order
    {
        constexpr int TQ = kBT / 4;
        float acc[K];
#pragma unroll
        for (int j = 0; j < K; ++j) acc[j] = 0.0f;
        const int t_end = min(kBT, n_t - tau0);
        const int q0 = wv * TQ;
        float win[K];
#pragma unroll
        for (int j = 0; j < K - 1; ++j) win[j + 1] = slc[q0 + K - 1 + j];
#pragma unroll
        for (int k = 0; k < TQ; ++k) {
            const int tt = q0 + k;
#pragma unroll
            for (int j = 0; j < K - 1; ++j) win[j] = win[j + 1];
            win[K - 1] = slc[tt + 2 * (K - 1)];
            const float gv = tt < t_end ? glc[tt + K - 1] : 0.0f;
#pragma unroll
            for (int j = 0; j < K; ++j) acc[j] = fmaf(gv, win[j], acc[j]);
        }
        // the quarter sums go through the sx tile, which is no longer read below
        __syncthreads();
#pragma unroll
        for (int j = 0; j < K; ++j) sl[(wv * kBC + cc) * kMaxK + j] = acc[j];
    }

    // d_sx rows: lanes along time (two channels per pass of 256 lanes); the
    // channel is wave-uniform, so its weights come through scalar loads
    {
        const int tt = tid & (kBT - 1);
        const int tau = tau0 + tt;
        float* dst = d_sx + (int64_t)s * d_inner * len;
        const int half = __builtin_amdgcn_readfirstlane(tid >> 7);
        for (int ch = half; ch < kBC; ch += 2) {
            const int c = c0 + ch;
            if (c >= d_inner) break;
            float acc = 0.0f;
#pragma unroll
            for (int j = 0; j < K; ++j) acc = fmaf(w[(int64_t)c * K + j], gl[ch * kGP + tt + K - 1 - j], acc);
            if (tau < len) dst[(int64_t)c * len + tau] = acc;
        }
    }
    __syncthreads();
    if (wave == 0 && c0 + cc < d_inner) {
        float* pd = dw_part + (((int64_t)s * gridDim.x + blockIdx.x) * d_inner + c0 + cc) * K;
#pragma unroll
        for (int j = 0; j < K; ++j) {
            float v = 0.0f;
#pragma unroll
            for (int q = 0; q < 4; ++q) v += sl[(q * kBC + cc) * kMaxK + j];
            pd[j] = v;
        }
    }
}

// d_w[c][j]: the partials of every (sequence, tile).  Eight lanes share an
// output: lane k sums the partials k, k+8, k+16, ... in order, and the eight
// sums are combined by a fixed tree, so the result repeats bitwise.
__global__ __launch_bounds__(256) void conv_bwd_reduce_w(const float* __restrict__ dw_part,
                                                         float* __restrict__ d_w, int n_parts,
                                                         int d_inner, int K) {
    const int n_out = d_inner * K;
    const int k = threadIdx.x & 7;
    const int e = blockIdx.x * 32 + (threadIdx.x >> 3);
    float acc = 0.0f;
    if (e < n_out)
        for (int q = k; q < n_parts; q += 8) acc += dw_part[(int64_t)q * n_out + e];
    acc += __shfl_xor(acc, 1, 8);
    acc += __shfl_xor(acc, 2, 8);
    acc += __shfl_xor(acc, 4, 8);
    if (k == 0 && e < n_out) d_w[e] = acc;
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
    // 16-byte gradient loads need 16-byte aligned rows; a wave-uniform switch
    const int vec = (d_inner % 4 == 0) && ((reinterpret_cast<uintptr_t>(dout) & 15) == 0);
    if (n_s > 0 && len > 0) {
        dim3 grid((unsigned)tiles, (unsigned)((d_inner + kBC - 1) / kBC), (unsigned)n_s);
        auto go = [&](auto kc) {
            constexpr int KK = decltype(kc)::value;
            if (io == SSM_F32)
                hipLaunchKernelGGL((conv_bwd_tiled<float, KK>), grid, dim3(256), 0, stream,
                                   static_cast<const float*>(sx), w, dout, dgrad, part, (int)n_t,
                                   (int)d_inner, apply_silu, vec);
            else
                hipLaunchKernelGGL((conv_bwd_tiled<bf16_t, KK>), grid, dim3(256), 0, stream,
                                   static_cast<const bf16_t*>(sx), w, dout, dgrad, part, (int)n_t,
                                   (int)d_inner, apply_silu, vec);
        };
        switch (d_conv) {
            case 1: go(std::integral_constant<int, 1>{}); break;
            case 2: go(std::integral_constant<int, 2>{}); break;
            case 3: go(std::integral_constant<int, 3>{}); break;
            case 4: go(std::integral_constant<int, 4>{}); break;
            case 5: go(std::integral_constant<int, 5>{}); break;
            case 6: go(std::integral_constant<int, 6>{}); break;
            case 7: go(std::integral_constant<int, 7>{}); break;
            default: go(std::integral_constant<int, 8>{}); break;
        }
    }
    const int n_parts = (int)(n_s * tiles);
    hipLaunchKernelGGL(conv_bwd_reduce_w, dim3((unsigned)((d_inner * d_conv + 31) / 32)), dim3(256),
                       0, stream, part, d_w, n_parts, (int)d_inner, d_conv);
    return hipGetLastError() == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

}  // namespace ssm
