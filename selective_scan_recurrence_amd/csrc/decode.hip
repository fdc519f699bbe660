// Single-token decode step over a batch of sequences, states updated in
// place ("mambazip mamba1/model.rs", forward_impl's per-token step: the conv
// window of depthwise_conv_step, SiLU, dt = softplus(dt_raw + dt_bias), the
// state update of selective_scan_state16, the output times SiLU(z); the conv
// taps in ggml's order, the last weight on the newest input).
//
// For sequence i with state row r = ids[i], head h, channel p:
//   u = SiLU(sum_j w[h][j] win[j]) over win = conv_state[r][h][0..K-2], x[i][h]
//       (then conv_state[r][h] keeps the last K-1 entries of win), or x[i][h][p];
//   d = dt[i][h] (+ dt_bias[h]), softplus when asked;
//   s[r][h][p][n] = exp(d A) s[r][h][p][n] + d B[i][g][n] u;
//   y[i][h][p] = (sum_n C[i][g][n] s[r][h][p][n] + D[h] u) * SiLU(z[i][h][p]).
//
// HBM-bound on the state rows (read and written once).  One state row of N
// states is held by N/16 lanes of one wave, 16 fp32 states each, read and
// written as 16-byte pieces; consecutive lanes hold consecutive pieces of
// consecutive rows, so a wave moves one contiguous block of the state.  The
// y partial sums are added across the row's lanes with xor shuffles.
#include "device_common.h"
#include "ssm_internal.h"

#include <type_traits>

namespace ssm {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct DecodeKP {
    float* s;
    const void* x;
    const void* dt;
    const float* dt_bias;
    const float* A;
    const void* B;
    const void* C;
    const float* D;
    const void* z;
    const int32_t* ids;
    const float* conv_w;
    float* conv_state;
    void* y;
    uint32_t* err;
    int64_t n_rows;  // S * H * P
    int H, P, N, G, R, K, a_per_state, softplus;
};

template <typename T>
__device__ __forceinline__ float ld(const void* p, int64_t i) {
    return to_f32(static_cast<const T*>(p)[i]);
}

// The scan input u and the step d of row (i, h, p) whose state row is r; the
// conv state is advanced by the row's lane `writer` only.
template <typename T>
__device__ __forceinline__ void row_inputs(const DecodeKP& k, int64_t i, int h, int p, int r,
                                           bool writer, float& u, float& d) {
    d = ld<T>(k.dt, i * k.H + h) + (k.dt_bias ? k.dt_bias[h] : 0.0f);
    if (k.softplus) d = softplus(d);
    if (k.K) {
        // head_dim is 1 with the conv: the row is channel h
        float* cs = k.conv_state + ((int64_t)r * k.H + h) * (k.K - 1);
        const float* w = k.conv_w + (int64_t)h * k.K;
        const float xin = ld<T>(k.x, i * k.H + h);
        float c = w[k.K - 1] * xin;
        for (int j = 0; j < k.K - 1; ++j) c = fmaf(w[j], cs[j], c);
        // every lane of the row has read the window (same wave, earlier
        // instructions) before the writer shifts it
        if (writer) {
            for (int j = 0; j + 1 < k.K - 1; ++j) cs[j] = cs[j + 1];
            if (k.K > 1) cs[k.K - 2] = xin;
        }
        u = silu(c);
    } else {
        u = ld<T>(k.x, (i * k.H + h) * (int64_t)k.P + p);
    }
}

template <typename T>
__device__ __forceinline__ void store_y(const DecodeKP& k, int64_t e, float v) {
    if (k.z) v *= silu(ld<T>(k.z, e));
    store_io(static_cast<T*>(k.y) + e, v);
}

// N = 16 * LPR: LPR lanes per row, 16 states per lane.
template <typename T, int LPR>
__global__ __launch_bounds__(256) void decode_rows16(DecodeKP k) {
    const int64_t gt = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t row = gt / LPR;
    const int q = (int)(gt % LPR);
    if (row >= k.n_rows) return;  // whole rows leave together (LPR divides 64)
    const int hp = (int)(row % ((int64_t)k.H * k.P));
    const int64_t i = row / ((int64_t)k.H * k.P);
    const int h = hp / k.P, p = hp % k.P;
    const int r = k.ids[i];
    const int64_t e = row;  // y / z / x element of the row
    if (r < 0 || r >= k.R) {
        if (q == 0) {
            store_io(static_cast<T*>(k.y) + e, __builtin_nanf(""));
            if (k.err) atomicOr(k.err, (uint32_t)SSM_DEVERR_IDS);
        }
        return;
    }
    const int g = h / (k.H / k.G);
    float u, d;
    row_inputs<T>(k, i, h, p, r, q == 0, u, d);

    constexpr int NS = 16;
    float* st = k.s + (((int64_t)r * k.H + h) * k.P + p) * k.N + q * NS;
    f32x4 sv[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) sv[m] = reinterpret_cast<const f32x4*>(st)[m];
    float bv[NS], cv[NS], av[NS];
    const int64_t bc = ((int64_t)i * k.G + g) * k.N + q * NS;
    if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const u32x4 b4 = reinterpret_cast<const u32x4*>(static_cast<const T*>(k.B) + bc)[m];
            const u32x4 c4 = reinterpret_cast<const u32x4*>(static_cast<const T*>(k.C) + bc)[m];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                bv[8 * m + 2 * w] = __uint_as_float(b4[w] << 16);
                bv[8 * m + 2 * w + 1] = __uint_as_float(b4[w] & 0xFFFF0000u);
                cv[8 * m + 2 * w] = __uint_as_float(c4[w] << 16);
                cv[8 * m + 2 * w + 1] = __uint_as_float(c4[w] & 0xFFFF0000u);
            }
        }
    } else {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const f32x4 b4 = reinterpret_cast<const f32x4*>(static_cast<const float*>(k.B) + bc)[m];
            const f32x4 c4 = reinterpret_cast<const f32x4*>(static_cast<const float*>(k.C) + bc)[m];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                bv[4 * m + w] = b4[w];
                cv[4 * m + w] = c4[w];
            }
        }
    }
    if (k.a_per_state) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const f32x4 a4 = reinterpret_cast<const f32x4*>(k.A + (int64_t)h * k.N + q * NS)[m];
#pragma unroll
            for (int w = 0; w < 4; ++w) av[4 * m + w] = a4[w];
        }
    } else {
        const float a = k.A[h];
#pragma unroll
        for (int n = 0; n < NS; ++n) av[n] = a;
    }
    const float du = d * u, dl = d * kLog2e;
    float acc = 0.0f;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const int n = 4 * m + w;
            const float hn = fmaf(fast_exp2(dl * av[n]), sv[m][w], du * bv[n]);
            sv[m][w] = hn;
            acc = fmaf(cv[n], hn, acc);
        }
#pragma unroll
    for (int m = 0; m < 4; ++m) reinterpret_cast<f32x4*>(st)[m] = sv[m];
#pragma unroll
    for (int o = 1; o < LPR; o <<= 1) acc += __shfl_xor(acc, o, LPR);
    if (q == 0) store_y<T>(k, e, acc + (k.D ? k.D[h] * u : 0.0f));
}

// Any N: one lane per row, states in a loop.
template <typename T>
__global__ __launch_bounds__(256) void decode_rows_any(DecodeKP k) {
    const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (row >= k.n_rows) return;
    const int hp = (int)(row % ((int64_t)k.H * k.P));
    const int64_t i = row / ((int64_t)k.H * k.P);
    const int h = hp / k.P, p = hp % k.P;
    const int r = k.ids[i];
    if (r < 0 || r >= k.R) {
        store_io(static_cast<T*>(k.y) + row, __builtin_nanf(""));
        if (k.err) atomicOr(k.err, (uint32_t)SSM_DEVERR_IDS);
        return;
    }
    const int g = h / (k.H / k.G);
    float u, d;
    row_inputs<T>(k, i, h, p, r, true, u, d);
    float* st = k.s + (((int64_t)r * k.H + h) * k.P + p) * k.N;
    const int64_t bc = ((int64_t)i * k.G + g) * k.N;
    const float du = d * u, dl = d * kLog2e;
    float acc = 0.0f;
    for (int n = 0; n < k.N; ++n) {
        const float a = k.a_per_state ? k.A[(int64_t)h * k.N + n] : k.A[h];
        const float hn = fmaf(fast_exp2(dl * a), st[n], du * ld<T>(k.B, bc + n));
        st[n] = hn;
        acc = fmaf(ld<T>(k.C, bc + n), hn, acc);
    }
    store_y<T>(k, row, acc + (k.D ? k.D[h] * u : 0.0f));
}

}  // namespace

int launch_state_update(const DecodeArgs& a, hipStream_t stream) {
    const Shape& sh = a.sh;
    DecodeKP k;
    k.s = a.s; k.x = a.x; k.dt = a.dt; k.dt_bias = a.dt_bias; k.A = a.A; k.B = a.B; k.C = a.C;
    k.D = a.D; k.z = a.z; k.ids = a.ids; k.conv_w = a.conv_w; k.conv_state = a.conv_state;
    k.y = a.y; k.err = a.err;
    k.n_rows = sh.S * sh.H * sh.P;
    k.H = (int)sh.H; k.P = (int)sh.P; k.N = (int)sh.N; k.G = (int)sh.G; k.R = (int)sh.R;
    k.K = sh.K; k.a_per_state = sh.a_per_state;
    k.softplus = (sh.flags & SSM_DT_SOFTPLUS) ? 1 : 0;
    if (k.n_rows == 0) return SSM_OK;
    auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
    const bool bf = sh.io == SSM_BF16;
    const int lpr = (sh.N % 16 == 0 && sh.N <= 256) ? (int)(sh.N / 16) : 0;
    const bool fast = lpr && (lpr & (lpr - 1)) == 0 && al16(a.s) && al16(a.B) && al16(a.C) &&
                      (!sh.a_per_state || al16(a.A));
    if (fast) {
        const int64_t threads = k.n_rows * lpr;
        const dim3 grid((unsigned)((threads + 255) / 256));
        auto go = [&](auto lc) {
            constexpr int LPR = decltype(lc)::value;
            if (bf) hipLaunchKernelGGL((decode_rows16<bf16_t, LPR>), grid, dim3(256), 0, stream, k);
            else hipLaunchKernelGGL((decode_rows16<float, LPR>), grid, dim3(256), 0, stream, k);
        };
        switch (lpr) {
            case 1: go(std::integral_constant<int, 1>{}); break;
            case 2: go(std::integral_constant<int, 2>{}); break;
            case 4: go(std::integral_constant<int, 4>{}); break;
            case 8: go(std::integral_constant<int, 8>{}); break;
            default: go(std::integral_constant<int, 16>{}); break;
        }
    } else {
        const dim3 grid((unsigned)((k.n_rows + 255) / 256));
        if (bf) hipLaunchKernelGGL((decode_rows_any<bf16_t>), grid, dim3(256), 0, stream, k);
        else hipLaunchKernelGGL((decode_rows_any<float>), grid, dim3(256), 0, stream, k);
    }
    return hipGetLastError() == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

}  // namespace ssm
