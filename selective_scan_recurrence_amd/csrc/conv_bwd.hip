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
// One workgroup owns 64 channels of one sequence and 64 positions tau of
// sx.  It stages the gradient rows it needs (tau - K + 1 .. tau, channel-
// fastest in memory) transposed into LDS, and the sx rows around them (time-
// fastest) for the SiLU derivative and the weight gradient; then it writes
// d_sx rows along time and a partial weight gradient over its own 64 tokens.
// A second kernel sums the partials in a fixed order (sequence, then tile),
// so results repeat bitwise.  HBM-bound: sx, dout and d_sx each cross HBM
// once; the K-1 halo rows of a tile are read again by its neighbour in time,
// which runs at the same moment on the same XCD and finds them in L2.
#include "device_common.h"
#include "ssm_internal.h"

#include <type_traits>

namespace ssm {
namespace {

constexpr int kBC = 64;     // channels per workgroup (one per lane)
constexpr int kBT = 64;     // positions of sx per workgroup
constexpr int kMaxK = 8;
constexpr int kGP = 73;     // LDS pitch of a channel's gradient row (odd, >= 4 * ceil((kBT + 7) / 4))
constexpr int kSP = 79;     // LDS pitch of a channel's f32 sx row (odd, >= kBT + 15)
constexpr int kSPh = 82;    // LDS pitch of a channel's bf16 sx row (2 x odd: rows start on distinct banks)

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <typename T>
struct TypeTag {
    using type = T;
};

// SILU: the forward applied SiLU to the conv output.  VEC: gradient rows are
// read 16 bytes at a time (d_inner % 4 == 0 and dout 16-byte aligned).  Both
// are template arguments so that no load sits behind a branch, which keeps
// the compiler's wait counts exact.
template <typename T, int K, bool SILU, bool VEC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void conv_bwd_tile(
    const T* __restrict__ sx, const float* __restrict__ w, const float* __restrict__ dout,
    float* __restrict__ d_sx, float* __restrict__ dw_part, int n_t, int d_inner) {
    // LDS rows of the tile at tau0, per channel:
    //   gl[u] = gradient at t = tau0 - H + u   (u < 4 * RQ)
    //   sl[q] = sx at position tau0 - H + q    (q < kGRows + H)
    // The four waves split the gradient rows u < kBT + H into quarters of RQ;
    // rows past them hold zeros and real sx values, so every value read is
    // finite, and are left out of every sum.
    constexpr int H = K - 1;
    constexpr int ES = (int)sizeof(T);
    constexpr int RQ = (kBT + H + 3) / 4;
    constexpr int kGRows = 4 * RQ;
    constexpr int kTail = kGRows + H - kBT;  // sx positions read past the first 64
    // sx stays in its io type in LDS (bf16 rows take half the space, so five
    // workgroups fit a CU instead of four)
    constexpr int SP = ES == 2 ? kSPh : kSP;
    static_assert(kGRows <= kGP && kTail <= 16 && kGRows + H <= SP, "rows fit the LDS rows");
    static_assert(4 * kBC * kMaxK * 4 <= kBC * SP * ES, "the sx tile holds the d_w partials");
    __shared__ float gl[kBC * kGP];
    __shared__ T sl[kBC * SP];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    // Workgroups are dealt to the 8 XCDs in turn; renumber them so that each
    // XCD runs one contiguous stretch of (sequence, channel block, tile) with
    // time fastest: neighbouring tiles, which share the cache lines at their
    // edges and the halo rows, then meet in the same L2.
    const uint32_t n_wg = gridDim.x * gridDim.y * gridDim.z;
    const uint32_t pid = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    const uint32_t per = n_wg / 8, extra = n_wg % 8, xcd = pid % 8;
    const uint32_t lid = xcd * per + min(xcd, extra) + pid / 8;
    const uint32_t tile = lid % gridDim.x, rest = lid / gridDim.x;
    const int s = (int)(rest / gridDim.y), c0 = (int)(rest % gridDim.y) * kBC;
    const int tau0 = (int)tile * kBT, lo = tau0 - H;
    const int len = n_t + H;

    // Loads go through buffer descriptors over the sequence, so no load sits
    // behind a branch.  Offsets are never negative (the compiler moves
    // constant parts of an offset into the instruction's immediate field,
    // and the range check does not see a register part that wraps below zero
    // come back into range): positions and rows before 0 are clamped, and
    // every value outside the tensor is zeroed by a select.
    const char* sxs = reinterpret_cast<const char*>(sx) + (int64_t)s * d_inner * len * ES;
    const char* gs = reinterpret_cast<const char*>(dout + (int64_t)s * n_t * d_inner);
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(sxs), 0, d_inner * len * ES, 0x00020000);
    const auto rg = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(gs), 0, n_t * d_inner * 4, 0x00020000);
    auto ld_sx = [&](int off) -> T {
        if constexpr (ES == 2)
            return (T)__builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, 0);
        else
            return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
    };

    // sx rows: channel wv + 4i at q = lane, then the positions q = 64 + tq
    // (tq < kTail) with 16 lanes per channel (tch + 16 i2)
    const int tq = lane & 15, tch = wave + 4 * (lane >> 4);
    const int pm = lo + lane, pt = lo + kBT + tq;
    T sv[kBC / 4], st[4];
#pragma unroll
    for (int i = 0; i < kBC / 4; ++i) sv[i] = ld_sx(((c0 + wv + 4 * i) * len + max(pm, 0)) * ES);
    if constexpr (kTail > 0)
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) st[i2] = ld_sx(((c0 + tch + 16 * i2) * len + pt) * ES);
    // gradient rows u = (tid >> 4) + 16 i, 16 lanes x 4 channels each; rows
    // past kGRows are not loaded (an offset past the range moves nothing)
    const int cq = (tid & 15) * 4;
    constexpr int kGR = (kGRows + 15) / 16;
    f32x4 gv4[kGR];
#pragma unroll
    for (int i = 0; i < kGR; ++i) {
        const int u = (tid >> 4) + 16 * i, t = lo + u;
        const int off = (i < kGR - 1 || u < kGRows) ? (max(t, 0) * d_inner + c0 + cq) * 4 : INT_MIN;
        if constexpr (VEC) {
            gv4[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rg, off, 0, 0));
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                gv4[i][k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rg, off < 0 ? off : off + 4 * k, 0, 0));
        }
    }
    // lane = channel for the SiLU factor and the weight gradient
    const int cc = lane;
    float wk[K];
#pragma unroll
    for (int j = 0; j < K; ++j) wk[j] = c0 + cc < d_inner ? w[(int64_t)(c0 + cc) * K + j] : 0.0f;

    // stage, zeroing what lies outside the sequence or the channels; LDS
    // bases come from the per-lane wave index, so that the rows of a wave
    // differ by immediate offsets
    {
        T* slw = sl + wave * SP + lane;
        const bool okm = (unsigned)pm < (unsigned)len;
#pragma unroll
        for (int i = 0; i < kBC / 4; ++i) slw[4 * i * SP] = (okm && c0 + wv + 4 * i < d_inner) ? sv[i] : (T)0;
        T* slt = sl + tch * SP + kBT + tq;
        const bool okt = pt < len;
        if constexpr (kTail > 0)
            if (tq < kTail)
#pragma unroll
                for (int i2 = 0; i2 < 4; ++i2) slt[16 * i2 * SP] = (okt && c0 + tch + 16 * i2 < d_inner) ? st[i2] : (T)0;
        float* glw = gl + cq * kGP + (tid >> 4);
#pragma unroll
        for (int i = 0; i < kGR; ++i) {
            const int u = (tid >> 4) + 16 * i;
            const bool ok = lo + u >= 0;
            if (i < kGR - 1 || u < kGRows) {
#pragma unroll
                for (int k = 0; k < 4; ++k) glw[k * kGP + 16 * i] = ok ? gv4[i][k] : 0.0f;
            }
        }
    }
    __syncthreads();

    // One pass over this wave's quarter of the gradient rows, sliding a
    // K-wide window of sx along them (one LDS read per row): the SiLU
    // derivative at the recomputed pre-activation, g *= s(z)(1 + z(1 - s(z))),
    // and the weight gradient over the tile's own tokens (rows H .. H+63;
    // tokens at or past n_t hold a zero gradient).
    float acc[K];
#pragma unroll
    for (int j = 0; j < K; ++j) acc[j] = 0.0f;
    {
        const T* slc = sl + cc * SP;
        float* glc = gl + cc * kGP;
        const int u0 = wv * RQ;
        float win[K];
#pragma unroll
        for (int j = 0; j < K - 1; ++j) win[j + 1] = to_f32(slc[u0 + j]);
#pragma unroll
        for (int k = 0; k < RQ; ++k) {
            const int u = u0 + k;
#pragma unroll
            for (int j = 0; j < K - 1; ++j) win[j] = win[j + 1];
            win[K - 1] = to_f32(slc[u + K - 1]);
            float g = glc[u];
            if constexpr (SILU) {
                float z = 0.0f;
#pragma unroll
                for (int j = 0; j < K; ++j) z = fmaf(win[j], wk[j], z);
                const float sg = __builtin_amdgcn_rcpf(1.0f + fast_exp2(-z * kLog2e));
                g *= sg * fmaf(z, 1.0f - sg, 1.0f);
                glc[u] = g;
            }
            const float gd = (u >= H && u < H + kBT) ? g : 0.0f;
#pragma unroll
            for (int j = 0; j < K; ++j) acc[j] = fmaf(gd, win[j], acc[j]);
        }
    }
    __syncthreads();

    // d_sx rows: lanes along time, one channel per wave and pass; the
    // channel is wave-uniform, so its weights come through scalar loads.  One
    // descriptor spans the sequence; lanes past the row or the channels take
    // an offset past its range, so the hardware drops their stores.
    {
        const auto rd = __builtin_amdgcn_make_buffer_rsrc(d_sx + (int64_t)s * d_inner * len, 0, d_inner * len * 4, 0x00020000);
        const int tau = tau0 + lane;
        const float* glr = gl + wave * kGP + lane + H;
#pragma unroll
        for (int i = 0; i < kBC / 4; ++i) {
            const int c = c0 + wv + 4 * i, cl = min(c, d_inner - 1);
            float a = 0.0f;
#pragma unroll
            for (int j = 0; j < K; ++j) a = fmaf(w[(int64_t)cl * K + j], glr[4 * i * kGP - j], a);
            const int off = (c < d_inner && tau < len) ? (c * len + tau) * 4 : INT_MIN;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(a), rd, off, 0, 0);
        }
    }

    // d_w partial of the tile: the four waves' sums, added in order (through
    // the sx tile, which is no longer read)
    float* pl = reinterpret_cast<float*>(sl);
#pragma unroll
    for (int j = 0; j < K; ++j) pl[(wv * kBC + cc) * kMaxK + j] = acc[j];
    __syncthreads();
    if (wave == 0 && c0 + cc < d_inner) {
        float* pd = dw_part + (((int64_t)s * gridDim.x + tile) * d_inner + c0 + cc) * K;
#pragma unroll
        for (int j = 0; j < K; ++j) {
            float v = 0.0f;
#pragma unroll
            for (int q = 0; q < 4; ++q) v += pl[(q * kBC + cc) * kMaxK + j];
            pd[j] = v;
        }
    }
}

// d_w[c][j]: the partials of every (sequence, tile).  Lanes run along the
// outputs, so each wave reads 256 contiguous bytes per partial; the 16 waves
// of a workgroup take every 16th partial in order, with 8 loads in flight,
// and their sums are added in a fixed order, so the result repeats bitwise.
constexpr int kRedWaves = 16;
__global__ __launch_bounds__(64 * kRedWaves) void conv_bwd_reduce_w(const float* __restrict__ dw_part,
                                                                    float* __restrict__ d_w, int n_parts,
                                                                    int n_out) {
    __shared__ float red[kRedWaves][64];
    const int l = threadIdx.x & 63, g = threadIdx.x >> 6;
    const int e = blockIdx.x * 64 + l;
    float acc = 0.0f;
    if (e < n_out) {
#pragma unroll 8
        for (int q = g; q < n_parts; q += kRedWaves) acc += dw_part[(int64_t)q * n_out + e];
    }
    red[g][l] = acc;
    __syncthreads();
    if (g == 0 && e < n_out) {
        float v = 0.0f;
#pragma unroll
        for (int k = 0; k < kRedWaves; ++k) v += red[k][l];
        d_w[e] = v;
    }
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
    // the kernel numbers its workgroups in 32 bits
    if (n_s * tiles * ((d_inner + kBC - 1) / kBC) > (int64_t)(UINT32_MAX / 256)) return SSM_ERR_SHAPE;
    float* d_w = dgrad + n_s * d_inner * len;
    float* part = static_cast<float*>(ws);
    // 16-byte gradient loads need 16-byte aligned rows
    const bool vec = (d_inner % 4 == 0) && ((reinterpret_cast<uintptr_t>(dout) & 15) == 0);
    const bool silu = apply_silu != 0;
    if (n_s > 0 && len > 0) {
        dim3 grid((unsigned)tiles, (unsigned)((d_inner + kBC - 1) / kBC), (unsigned)n_s);
        auto go = [&](auto kc) {
            constexpr int KK = decltype(kc)::value;
            auto inst = [&](auto tag, auto sl, auto vc) {
                using TT = typename decltype(tag)::type;
                hipLaunchKernelGGL((conv_bwd_tile<TT, KK, decltype(sl)::value, decltype(vc)::value>), grid,
                                   dim3(256), 0, stream, static_cast<const TT*>(sx), w, dout, dgrad, part,
                                   (int)n_t, (int)d_inner);
            };
            auto by_vec = [&](auto tag, auto sl) {
                if (vec) inst(tag, sl, std::true_type{});
                else inst(tag, sl, std::false_type{});
            };
            auto by_silu = [&](auto tag) {
                if (silu) by_vec(tag, std::true_type{});
                else by_vec(tag, std::false_type{});
            };
            if (io == SSM_F32) by_silu(TypeTag<float>{});
            else by_silu(TypeTag<bf16_t>{});
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
    const int n_out = (int)(d_inner * d_conv);
    hipLaunchKernelGGL(conv_bwd_reduce_w, dim3((unsigned)((n_out + 63) / 64)), dim3(64 * kRedWaves), 0, stream,
                       part, d_w, n_parts, n_out);
    return hipGetLastError() == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

}  // namespace ssm
