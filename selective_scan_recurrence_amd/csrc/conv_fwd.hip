// Standalone depthwise causal conv, the ggml ssm_conv operator of the ggmlR
// page ("ggml_ssm_conv matches a depthwise convolution computed in R"):
//   out[s][t][c] = sum_{j<K} sx[s][c][t + j] * w[c][j]     (then SiLU if asked)
// sx is time-fastest and out channel-fastest.  One workgroup (4 waves) owns
// 64 channels of one sequence and 64 output tokens: it reads the 64 + K - 1
// sx positions of each channel along time (one channel per wave
// instruction), stages them in LDS, slides a K-wide window down each
// channel's row (lane = channel), and writes the outputs along channels --
// through LDS as 16-byte row pieces when the rows are aligned for them.
// HBM-bound: every input element crosses HBM once and every output once;
// the K-1 halo positions of a tile are read again by its neighbour in time,
// which the XCD-ordered numbering places on the same XCD at the same time,
// so they come from its L2.
#include "device_common.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

constexpr int kBC = 64;      // channels per workgroup
constexpr int kBT = 64;      // output tokens per workgroup
constexpr int kMaxK = 8;
constexpr int kSP = 79;      // LDS pitch of a channel's f32 sx row (odd: lanes hit distinct banks)
constexpr int kSPh = 82;     // LDS pitch of a bf16 sx row (2 x odd)
constexpr int kOP = 72;      // LDS pitch (in io elements) of a staged output row of 64 channels

template <typename T, int K, bool SILU, bool VEC>
__global__ __launch_bounds__(256) void conv_fwd_tile(const T* __restrict__ sx, const float* __restrict__ w,
                                                     T* __restrict__ out, int n_t, int d_inner) {
    constexpr int H = K - 1;
    constexpr int ES = (int)sizeof(T);
    constexpr int SP = ES == 2 ? kSPh : kSP;
    static_assert(kBT + H <= SP, "a channel's positions fit its LDS row");
    __shared__ T sl[kBC * SP];
    __shared__ __attribute__((aligned(16))) T ol[VEC ? kBT * kOP : 8];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    // XCD-ordered numbering (workgroups are dealt to the 8 XCDs in turn): each
    // XCD runs one contiguous stretch of (sequence, channel block, tile) with
    // time fastest, so neighbouring tiles share their halo in one L2
    const uint32_t n_wg = gridDim.x * gridDim.y * gridDim.z;
    const uint32_t pid = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    const uint32_t per = n_wg / 8, extra = n_wg % 8, xcd = pid % 8;
    const uint32_t lid = xcd * per + min(xcd, extra) + pid / 8;
    const uint32_t tile = lid % gridDim.x, rest = lid / gridDim.x;
    const int s = (int)(rest / gridDim.y), c0 = (int)(rest % gridDim.y) * kBC;
    const int t0 = (int)tile * kBT;
    const int len = n_t + H;

    // loads through a descriptor over the sequence's sx: positions past the
    // row or channels past d_inner are clamped in range and zeroed by a select
    const char* sxs = reinterpret_cast<const char*>(sx) + (int64_t)s * d_inner * len * ES;
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(sxs), 0, d_inner * len * ES, 0x00020000);
    auto ld_sx = [&](int off) -> float {
        if constexpr (ES == 2)
            return to_f32((bf16_t)__builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, 0));
        else
            return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
    };
    // main positions t0 + lane of channels wv + 4i; the H tail positions
    // t0 + 64 + tq of channels tch + 16 i2 (16 lanes per channel)
    const int pm = t0 + lane;
    const int tq = lane & 15, tch = wave + 4 * (lane >> 4);
    const int pt = t0 + kBT + tq;
    float sv[kBC / 4], st[4];
#pragma unroll
    for (int i = 0; i < kBC / 4; ++i) {
        const int c = min(c0 + wv + 4 * i, d_inner - 1);
        sv[i] = ld_sx((c * len + min(pm, len - 1)) * ES);
    }
    if constexpr (H > 0)
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) {
            const int c = min(c0 + tch + 16 * i2, d_inner - 1);
            st[i2] = ld_sx((c * len + min(pt, len - 1)) * ES);
        }
    const int cc = lane;
    const bool cok = c0 + cc < d_inner;
    float wk[K];
#pragma unroll
    for (int j = 0; j < K; ++j) wk[j] = cok ? w[(int64_t)(c0 + cc) * K + j] : 0.0f;
    {
        const bool okm = pm < len;
#pragma unroll
        for (int i = 0; i < kBC / 4; ++i) {
            const bool ok = okm && c0 + wave + 4 * i < d_inner;
            const float v = ok ? sv[i] : 0.0f;
            if constexpr (ES == 2) sl[(wave + 4 * i) * SP + lane] = bf16_rne(v);
            else sl[(wave + 4 * i) * SP + lane] = v;
        }
        if constexpr (H > 0)
            if (tq < H) {
#pragma unroll
                for (int i2 = 0; i2 < 4; ++i2) {
                    const bool ok = pt < len && c0 + tch + 16 * i2 < d_inner;
                    const float v = ok ? st[i2] : 0.0f;
                    if constexpr (ES == 2) sl[(tch + 16 * i2) * SP + kBT + tq] = bf16_rne(v);
                    else sl[(tch + 16 * i2) * SP + kBT + tq] = v;
                }
            }
    }
    __syncthreads();

    // lane = channel: wave w takes output tokens 16w .. 16w + 15 with a sliding window
    const int tb = wave * (kBT / 4);
    const T* row = sl + cc * SP + tb;
    float win[K];
#pragma unroll
    for (int j = 0; j < H; ++j) win[j] = to_f32(row[j]);
    T* dst = out + (int64_t)s * n_t * d_inner;
#pragma unroll
    for (int k = 0; k < kBT / 4; ++k) {
        win[H] = to_f32(row[k + H]);
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < K; ++j) acc = fmaf(wk[j], win[j], acc);
#pragma unroll
        for (int j = 0; j < H; ++j) win[j] = win[j + 1];
        const float o = SILU ? silu(acc) : acc;
        const int t = t0 + tb + k;
        if constexpr (VEC) {
            if constexpr (ES == 2) ol[(tb + k) * kOP + cc] = bf16_rne(o);
            else ol[(tb + k) * kOP + cc] = o;
        } else if (cok && t < n_t) {
            store_io(dst + (int64_t)t * d_inner + c0 + cc, o);
        }
    }
    if constexpr (VEC) {
        // 16-byte pieces of the 64 output rows (d_inner % (16 / ES) == 0 and an
        // aligned out, so a piece never straddles two rows); a descriptor over
        // the sequence's out drops pieces past its last token
        __syncthreads();
        constexpr int PPR = kBC * ES / 16;  // pieces per row
        typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
        const auto ro = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<char*>(dst), 0,
                                                          n_t * d_inner * ES, 0x00020000);
#pragma unroll
        for (int e = tid; e < kBT * PPR; e += 256) {
            const int r = e / PPR, part = e % PPR;
            const int c = c0 + part * (16 / ES);
            const u32x4 v = *reinterpret_cast<const u32x4*>(&ol[r * kOP + part * (16 / ES)]);
            const int t = t0 + r;
            const int off = (t < n_t && c < d_inner) ? (t * d_inner + c) * ES : INT_MIN;
            __builtin_amdgcn_raw_buffer_store_b128(v, ro, off, 0, 2);  // nontemporal: out is not read back here
        }
    }
}

template <typename T, int K>
int launch_k(const void* sx, const float* w, void* out, int64_t n_s, int64_t n_t, int64_t d_inner,
             int apply_silu, hipStream_t stream) {
    const dim3 grid((unsigned)((n_t + kBT - 1) / kBT), (unsigned)((d_inner + kBC - 1) / kBC), (unsigned)n_s);
    constexpr int ES = (int)sizeof(T);
    const bool vec = d_inner % (16 / ES) == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0;
    const T* s = static_cast<const T*>(sx);
    T* o = static_cast<T*>(out);
    if (vec) {
        if (apply_silu) hipLaunchKernelGGL((conv_fwd_tile<T, K, true, true>), grid, dim3(256), 0, stream, s, w, o, (int)n_t, (int)d_inner);
        else hipLaunchKernelGGL((conv_fwd_tile<T, K, false, true>), grid, dim3(256), 0, stream, s, w, o, (int)n_t, (int)d_inner);
    } else {
        if (apply_silu) hipLaunchKernelGGL((conv_fwd_tile<T, K, true, false>), grid, dim3(256), 0, stream, s, w, o, (int)n_t, (int)d_inner);
        else hipLaunchKernelGGL((conv_fwd_tile<T, K, false, false>), grid, dim3(256), 0, stream, s, w, o, (int)n_t, (int)d_inner);
    }
    return hipGetLastError() == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

template <typename T>
int launch_t(const void* sx, const float* w, void* out, int64_t n_s, int64_t n_t, int64_t d_inner, int K,
             int apply_silu, hipStream_t st) {
    switch (K) {
        case 1: return launch_k<T, 1>(sx, w, out, n_s, n_t, d_inner, apply_silu, st);
        case 2: return launch_k<T, 2>(sx, w, out, n_s, n_t, d_inner, apply_silu, st);
        case 3: return launch_k<T, 3>(sx, w, out, n_s, n_t, d_inner, apply_silu, st);
        case 4: return launch_k<T, 4>(sx, w, out, n_s, n_t, d_inner, apply_silu, st);
        case 5: return launch_k<T, 5>(sx, w, out, n_s, n_t, d_inner, apply_silu, st);
        case 6: return launch_k<T, 6>(sx, w, out, n_s, n_t, d_inner, apply_silu, st);
        case 7: return launch_k<T, 7>(sx, w, out, n_s, n_t, d_inner, apply_silu, st);
        case 8: return launch_k<T, 8>(sx, w, out, n_s, n_t, d_inner, apply_silu, st);
        default: return SSM_ERR_UNSUPPORTED;
    }
}

}  // namespace

int launch_conv_fwd(const void* sx, const float* w, void* out, int64_t n_s, int64_t n_t,
                    int64_t d_inner, int d_conv, int io, int apply_silu, hipStream_t stream) {
    if (n_s == 0 || n_t == 0) return SSM_OK;
    if (d_conv > kMaxK) return SSM_ERR_UNSUPPORTED;
    return io == SSM_F32 ? launch_t<float>(sx, w, out, n_s, n_t, d_inner, d_conv, apply_silu, stream)
                         : launch_t<bf16_t>(sx, w, out, n_s, n_t, d_inner, d_conv, apply_silu, stream);
}

}  // namespace ssm
