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
// states is held by a group of lanes of one wave, read and written as
// 16-byte pieces that the group's lanes take in turn, so that every wave
// instruction moves whole lines; the state streams past the caches.  The
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

// The scan input u and the step d of row (i, h, p) whose state row is r.
// With the conv, win receives the K-1 conv-state values (oldest first) and
// the new input, kept in registers (fixed trip counts) so that the window is
// written back only after every load of the step has been issued.
constexpr int kMaxWin = 8;
template <typename T>
__device__ __forceinline__ void row_inputs(const DecodeKP& k, int64_t i, int h, int p, int r,
                                           float& u, float& d, float (&win)[kMaxWin]) {
    d = ld<T>(k.dt, i * k.H + h) + (k.dt_bias ? k.dt_bias[h] : 0.0f);
    if (k.softplus) d = softplus(d);
    if (k.K) {
        // head_dim is 1 with the conv: the row is channel h
        const float* cs = k.conv_state + ((int64_t)r * k.H + h) * (k.K - 1);
        const float* w = k.conv_w + (int64_t)h * k.K;
#pragma unroll
        for (int j = 0; j < kMaxWin - 1; ++j) win[j] = j < k.K - 1 ? cs[j] : 0.0f;
        const float xin = ld<T>(k.x, i * k.H + h);
        float c = 0.0f;
#pragma unroll
        for (int j = 0; j < kMaxWin; ++j) {
            if (j == k.K - 1) win[j] = xin;
            if (j < k.K) c = fmaf(w[j], win[j], c);
        }
        u = silu(c);
    } else {
        u = ld<T>(k.x, (i * k.H + h) * (int64_t)k.P + p);
    }
}

// The conv state keeps the last K-1 entries of the window.
__device__ __forceinline__ void shift_window(const DecodeKP& k, int h, int r, const float (&win)[kMaxWin]) {
    float* cs = k.conv_state + ((int64_t)r * k.H + h) * (k.K - 1);
#pragma unroll
    for (int j = 0; j < kMaxWin - 1; ++j)
        if (j < k.K - 1) cs[j] = win[j + 1];
}

template <typename T>
__device__ __forceinline__ void store_y(const DecodeKP& k, int64_t e, float v) {
    if (k.z) v *= silu(ld<T>(k.z, e));
    store_io(static_cast<T*>(k.y) + e, v);
}

// N = SPL * LPR: a row's states lie across LPR lanes, SPL each (4 or 16), as
// 16-byte pieces: lane q of the row holds pieces q, q + LPR, ... (states
// 4q + 4 LPR m + 0..3), so the m-th access of the row's lanes covers
// LPR x 16 contiguous bytes, and with SPL = 4 one access of a wave moves
// 1 KB of contiguous state (a first version with the 16 states of a lane
// contiguous read every line in four accesses of one lane).  Each lane
// takes RPT rows, 64 / LPR rows apart, and issues every load of all of them
// before any arithmetic.  The conv window of a row (Mamba-1 form) is spread
// over the row's lanes too: lane q holds window entries q, q + LPR, ...
// (the newest input last), the taps are summed across the lanes, and each
// lane writes its own entries back one place down.  UNI: every row of a
// lane has one sequence and one group, so B and C are read once.  A row with
// a bad id is read at row 0 (in bounds) and never written.
template <typename T, int SPL, int LPR, int RPT, bool UNI>
__global__ __launch_bounds__(256) void decode_rows(DecodeKP k) {
    constexpr int NQ = SPL / 4;                     // 16-byte state pieces per lane
    constexpr int RW = 64 / LPR;                    // rows per wave instruction
    constexpr int WPL = (kMaxWin + LPR - 1) / LPR;  // window entries per lane
    const int lane = threadIdx.x & 63, q = lane % LPR;
    const int64_t wbase = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * (RPT * RW);
    const int64_t hp_n = (int64_t)k.H * k.P;
    int64_t rowv[RPT], iv[RPT];
    int hv[RPT], pv[RPT], rv[RPT];
    bool live[RPT], okv[RPT];
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
        rowv[j] = wbase + j * RW + lane / LPR;
        live[j] = rowv[j] < k.n_rows;
        const int64_t row = live[j] ? rowv[j] : 0;
        iv[j] = row / hp_n;
        // one sequence per wave: ids[i] through the scalar cache
        if constexpr (UNI) iv[j] = __builtin_amdgcn_readfirstlane((int)iv[j]);
        const int hp = (int)(row - iv[j] * hp_n);
        hv[j] = hp / k.P;
        pv[j] = hp - hv[j] * k.P;
    }
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
        const int r = k.ids[iv[j]];
        okv[j] = live[j] && r >= 0 && r < k.R;
        rv[j] = okv[j] ? r : 0;
    }
    // piece m (4 states) of this lane's part of a row: the row's lanes take
    // consecutive pieces in turn (lane q: pieces q, q + LPR, ...), so each
    // wave instruction reads or writes whole lines of every row it touches
    auto pc = [&](int m) { return 4 * q + 4 * LPR * m; };
    // every load of every row
    f32x4 sv[RPT][NQ];
    float av[RPT][SPL], bv[RPT][SPL], cv[RPT][SPL], u[RPT], d[RPT], wv[RPT][WPL];
    // the lane's pieces of a row of `base` starting at element `off`
    auto load_vals = [&](const void* base, int64_t off, float (&out)[SPL]) {
#pragma unroll
        for (int m = 0; m < NQ; ++m) {
            if constexpr (sizeof(T) == 2) {
                typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
                const u32x2 v = *reinterpret_cast<const u32x2*>(static_cast<const T*>(base) + off + pc(m));
#pragma unroll
                for (int w = 0; w < 2; ++w) {
                    out[4 * m + 2 * w] = __uint_as_float(v[w] << 16);
                    out[4 * m + 2 * w + 1] = __uint_as_float(v[w] & 0xFFFF0000u);
                }
            } else {
                const f32x4 v = *reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + off + pc(m));
#pragma unroll
                for (int w = 0; w < 4; ++w) out[4 * m + w] = v[w];
            }
        }
    };
    auto load_bc = [&](int j) {
        const int64_t bc = (iv[j] * k.G + hv[j] / (k.H / k.G)) * k.N;
        load_vals(k.B, bc, bv[j]);
        load_vals(k.C, bc, cv[j]);
    };
    if constexpr (UNI) load_bc(0);
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
        const int h = hv[j];
        const float* st = k.s + (((int64_t)rv[j] * k.H + h) * k.P + pv[j]) * k.N;
        // the state is read once and written once: streamed past the caches
        // (13% faster on the 256 x 5120 Mamba-1 step)
#pragma unroll
        for (int m = 0; m < NQ; ++m) sv[j][m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(st + pc(m)));
        if constexpr (!UNI) load_bc(j);
        if (k.a_per_state) {
#pragma unroll
            for (int m = 0; m < NQ; ++m) {
                const f32x4 a4 = *reinterpret_cast<const f32x4*>(k.A + (int64_t)h * k.N + pc(m));
#pragma unroll
                for (int w = 0; w < 4; ++w) av[j][4 * m + w] = a4[w];
            }
        } else {
            const float a = k.A[h];
#pragma unroll
            for (int w = 0; w < SPL; ++w) av[j][w] = a;
        }
        d[j] = ld<T>(k.dt, iv[j] * k.H + h) + (k.dt_bias ? k.dt_bias[h] : 0.0f);
        if (k.softplus) d[j] = softplus(d[j]);
        if (k.K) {
            // head_dim 1: the row is channel h; window entry e < K-1 is the
            // conv state, entry K-1 the new input
            const float* cs = k.conv_state + ((int64_t)rv[j] * k.H + h) * (k.K - 1);
            const float xin = ld<T>(k.x, iv[j] * k.H + h);
#pragma unroll
            for (int m = 0; m < WPL; ++m) {
                const int e = q + m * LPR;
                wv[j][m] = e < k.K - 1 ? cs[e] : (e == k.K - 1 ? xin : 0.0f);
            }
        } else {
            u[j] = ld<T>(k.x, (iv[j] * k.H + h) * (int64_t)k.P + pv[j]);
        }
    }
    if constexpr (UNI) {
#pragma unroll
        for (int j = 1; j < RPT; ++j)
#pragma unroll
            for (int w = 0; w < SPL; ++w) {
                bv[j][w] = bv[0][w];
                cv[j][w] = cv[0][w];
            }
    }
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
        const int h = hv[j];
        if (k.K) {
            float c = 0.0f;
#pragma unroll
            for (int m = 0; m < WPL; ++m) {
                const int e = q + m * LPR;
                if (e < k.K) c = fmaf(k.conv_w[(int64_t)h * k.K + e], wv[j][m], c);
            }
#pragma unroll
            for (int o = 1; o < LPR; o <<= 1) c += __shfl_xor(c, o, LPR);
            u[j] = silu(c);
        }
        const float du = d[j] * u[j], dl = d[j] * kLog2e;
        float acc = 0.0f;
#pragma unroll
        for (int m = 0; m < NQ; ++m)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const int n = 4 * m + w;
                const float hn = fmaf(fast_exp2(dl * av[j][n]), sv[j][m][w], du * bv[j][n]);
                sv[j][m][w] = hn;
                acc = fmaf(cv[j][n], hn, acc);
            }
#pragma unroll
        for (int o = 1; o < LPR; o <<= 1) acc += __shfl_xor(acc, o, LPR);
        if (okv[j]) {
            float* st = k.s + (((int64_t)rv[j] * k.H + h) * k.P + pv[j]) * k.N;
#pragma unroll
            for (int m = 0; m < NQ; ++m) __builtin_nontemporal_store(sv[j][m], reinterpret_cast<f32x4*>(st + pc(m)));
            if (k.K) {
                float* cs = k.conv_state + ((int64_t)rv[j] * k.H + h) * (k.K - 1);
#pragma unroll
                for (int m = 0; m < WPL; ++m) {
                    const int e = q + m * LPR;
                    if (e >= 1 && e < k.K) cs[e - 1] = wv[j][m];
                }
            }
        }
        if (q == 0 && live[j]) {
            if (okv[j]) {
                store_y<T>(k, rowv[j], acc + (k.D ? k.D[h] * u[j] : 0.0f));
            } else {
                store_io(static_cast<T*>(k.y) + rowv[j], __builtin_nanf(""));
                if (k.err) atomicOr(k.err, (uint32_t)SSM_DEVERR_IDS);
            }
        }
    }
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
    float u, d, win[kMaxWin];
    row_inputs<T>(k, i, h, p, r, u, d, win);
    if (k.K) shift_window(k, h, r, win);
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
    auto al8 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7) == 0; };
    const bool bf = sh.io == SSM_BF16;
    // 16 states per lane from d_state 64 up (Mamba-2 rows), else 4 per lane
    const int spl = (sh.N >= 64 && sh.N % 16 == 0) ? 16 : 4;
    const int lpr = sh.N % spl == 0 ? (int)(sh.N / spl) : 0;
    const bool bc_al = bf ? (spl == 4 ? al8(a.B) && al8(a.C) : al16(a.B) && al16(a.C))
                          : (al16(a.B) && al16(a.C));
    const bool fast = lpr && lpr <= 64 && (lpr & (lpr - 1)) == 0 && al16(a.s) && bc_al &&
                      (!sh.a_per_state || al16(a.A));
    if (fast) {
        const int rpt = spl == 16 ? 1 : 2;  // rows per lane, as RPT below
        const int64_t rows_per_wave = rpt * (64 / lpr);
        const int64_t rows_per_block = 4 * rows_per_wave;
        const dim3 grid((unsigned)((k.n_rows + rows_per_block - 1) / rows_per_block));
        // one sequence per wave, and one group for a lane's rows
        const bool uni = (sh.H * sh.P) % rows_per_wave == 0 && (sh.G == 1 || sh.P % rows_per_wave == 0);
        auto go = [&](auto sc, auto lc) {
            constexpr int SPL = decltype(sc)::value, LPR = decltype(lc)::value;
            constexpr int RPT = SPL == 16 ? 1 : 2;
            if (bf) {
                if (uni) hipLaunchKernelGGL((decode_rows<bf16_t, SPL, LPR, RPT, true>), grid, dim3(256), 0, stream, k);
                else hipLaunchKernelGGL((decode_rows<bf16_t, SPL, LPR, RPT, false>), grid, dim3(256), 0, stream, k);
            } else {
                if (uni) hipLaunchKernelGGL((decode_rows<float, SPL, LPR, RPT, true>), grid, dim3(256), 0, stream, k);
                else hipLaunchKernelGGL((decode_rows<float, SPL, LPR, RPT, false>), grid, dim3(256), 0, stream, k);
            }
        };
        using I4 = std::integral_constant<int, 4>;
        using I16 = std::integral_constant<int, 16>;
        if (spl == 4) {
            switch (lpr) {
                case 1: go(I4{}, std::integral_constant<int, 1>{}); break;
                case 2: go(I4{}, std::integral_constant<int, 2>{}); break;
                case 4: go(I4{}, std::integral_constant<int, 4>{}); break;
                case 8: go(I4{}, std::integral_constant<int, 8>{}); break;
                case 16: go(I4{}, std::integral_constant<int, 16>{}); break;
                case 32: go(I4{}, std::integral_constant<int, 32>{}); break;
                default: go(I4{}, std::integral_constant<int, 64>{}); break;
            }
        } else {
            switch (lpr) {
                case 4: go(I16{}, std::integral_constant<int, 4>{}); break;
                case 8: go(I16{}, std::integral_constant<int, 8>{}); break;
                default: go(I16{}, std::integral_constant<int, 16>{}); break;
            }
        }
    } else {
        const dim3 grid((unsigned)((k.n_rows + 255) / 256));
        if (bf) hipLaunchKernelGGL((decode_rows_any<bf16_t>), grid, dim3(256), 0, stream, k);
        else hipLaunchKernelGGL((decode_rows_any<float>), grid, dim3(256), 0, stream, k);
    }
    return hipGetLastError() == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

}  // namespace ssm
