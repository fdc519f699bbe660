// Selective-scan forward kernels for gfx950.
//
// Row kernel: one "row" is one (sequence i, channel c = h*head_dim + p).
// LPR lanes share a row; lane j of the row keeps states [16j, 16j+16) of
// that row in fp32 registers and walks the tokens in order, so every lane
// runs the plain recurrence of "mambazip mamba1/model.rs"
// (selective_scan_state16):  h = exp(dt*A) h + (u*dt) B;  y = sum C h + D u.
// The partial sums of y are combined across the row's lanes with shuffles.
// With the fused conv (head_dim 1), the lane also keeps the last d_conv-1
// inputs of its channel and forms u = SiLU(sum_j w[j] x[t-K+1+j]) on the fly
// (tap K-1 on the newest input, as in the ggmlR ssm_conv reference).
// The extras of the decode step of that model page (dt bias before softplus,
// y times SiLU(z)) and variable-length spans of a packed token axis are
// taken here as well.
#include "device_common.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

struct FwdKP {
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
    void* y;
    float* state_out;
    float* conv_state_out;
    uint32_t* err;
    const float* dt_bias;  // [H] or null
    const void* z;         // like x, or null
    const int32_t* cu;     // [S+1] spans, or null
    int64_t T;             // tokens on the packed axis
    int L, H, P, N, G, R, d_inner, heads_per_group;
    int has_D, softplus;
};

constexpr int kNPL = 16;    // states per lane
constexpr int kBlock = 64;  // one wave per block

template <typename T, int LPR, bool PSA, int K, bool G1>
__global__ __launch_bounds__(kBlock) void scan_fwd_rows(FwdKP p) {
    constexpr int kRows = kBlock / LPR;
    const int lr = threadIdx.x / LPR;
    const int j = threadIdx.x % LPR;
    const int c_raw = blockIdx.x * kRows + lr;
    const bool active = c_raw < p.d_inner;
    const int c = active ? c_raw : p.d_inner - 1;  // clamp: inactive lanes read a valid row
    const int i = blockIdx.y;
    const int h = c / p.P;
    const int pp = c - h * p.P;
    const int g = G1 ? 0 : h / p.heads_per_group;
    const int n0 = j * kNPL;

    int r = p.ids[i];
    const SeqSpan sp = seq_span(p.cu, i, p.L, p.T);
    const bool bad_id = (r < 0) | (r >= p.R);
    const bool bad = bad_id | sp.bad;
    if (bad) {
        r = 0;
        if (threadIdx.x == 0 && blockIdx.x == 0)
            atomicOr(p.err, (bad_id ? (uint32_t)SSM_DEVERR_IDS : 0u) | (sp.bad ? (uint32_t)SSM_DEVERR_SEQLENS : 0u));
    }
    const float nan = __builtin_nanf("");
    const float dtb = p.dt_bias ? p.dt_bias[h] : 0.0f;

    float hs[kNPL], a2[kNPL];
    const float* srow = p.s + (((int64_t)r * p.H + h) * p.P + pp) * p.N;
#pragma unroll
    for (int k = 0; k < kNPL; ++k) {
        const int n = n0 + k;
        hs[k] = n < p.N ? (bad ? nan : srow[n]) : 0.0f;
        if constexpr (PSA) a2[k] = n < p.N ? p.A[(int64_t)h * p.N + n] * kLog2e : 0.0f;
    }
    const float a2h = PSA ? 0.0f : p.A[h] * kLog2e;
    const float Dh = p.has_D ? p.D[h] : 0.0f;

    float w[K > 0 ? K : 1], win[K > 1 ? K - 1 : 1];
    if constexpr (K > 0) {
#pragma unroll
        for (int q = 0; q < K; ++q) w[q] = p.conv_w[(int64_t)h * K + q];
#pragma unroll
        for (int q = 0; q < K - 1; ++q)
            win[q] = bad ? nan
                         : (p.conv_state ? p.conv_state[((int64_t)r * p.H + h) * (K - 1) + q] : 0.0f);
    }

    const T* xs = static_cast<const T*>(p.x) + sp.t0 * p.d_inner + c;
    const T* dts = static_cast<const T*>(p.dt) + sp.t0 * p.H + h;
    const T* Bs = static_cast<const T*>(p.B) + (sp.t0 * p.G + g) * p.N + n0;
    const T* Cs = static_cast<const T*>(p.C) + (sp.t0 * p.G + g) * p.N + n0;
    T* ys = static_cast<T*>(p.y) + sp.t0 * p.d_inner + c;
    const T* zs = p.z ? static_cast<const T*>(p.z) + sp.t0 * p.d_inner + c : nullptr;
    const int bc_stride = p.G * p.N;

    for (int t = 0; t < sp.len; ++t) {
        const float xv = to_f32(xs[(int64_t)t * p.d_inner]);
        float dtv = to_f32(dts[(int64_t)t * p.H]) + dtb;
        if (p.softplus) dtv = softplus(dtv);
        float u;
        if constexpr (K > 0) {
            float cacc = w[K - 1] * xv;
#pragma unroll
            for (int q = 0; q < K - 1; ++q) cacc = fmaf(w[q], win[q], cacc);
#pragma unroll
            for (int q = 0; q < K - 2; ++q) win[q] = win[q + 1];
            if constexpr (K > 1) win[K - 2] = xv;
            u = silu(cacc);
        } else {
            u = xv;
        }
        const float dtu = dtv * u;
        const T* Bt = Bs + (int64_t)t * bc_stride;
        const T* Ct = Cs + (int64_t)t * bc_stride;
        float yv = 0.0f;
        const float ah = PSA ? 0.0f : fast_exp2(dtv * a2h);
#pragma unroll
        for (int k = 0; k < kNPL; ++k) {
            if (n0 + k < p.N) {
                const float a = PSA ? fast_exp2(dtv * a2[k]) : ah;
                hs[k] = fmaf(a, hs[k], dtu * to_f32(Bt[k]));
                yv = fmaf(to_f32(Ct[k]), hs[k], yv);
            }
        }
#pragma unroll
        for (int m = LPR / 2; m >= 1; m /= 2) yv += __shfl_xor(yv, m, LPR);
        if (active && j == 0) {
            float yo = fmaf(Dh, u, yv);
            if (zs) yo *= silu(to_f32(zs[(int64_t)t * p.d_inner]));
            store_io(ys + (int64_t)t * p.d_inner, yo);
        }
    }

    if (active) {
        float* so = p.state_out + (((int64_t)i * p.H + h) * p.P + pp) * p.N;
#pragma unroll
        for (int k = 0; k < kNPL; ++k)
            if (n0 + k < p.N) so[n0 + k] = hs[k];
        if constexpr (K > 1) {
            if (p.conv_state_out && j == 0) {
                float* co = p.conv_state_out + ((int64_t)i * p.H + h) * (K - 1);
#pragma unroll
                for (int q = 0; q < K - 1; ++q) co[q] = win[q];
            }
        }
    }
}

template <typename T, int LPR, bool PSA, int K, bool G1>
int launch_rows(const FwdKP& kp, int64_t S, hipStream_t stream) {
    const int rows = kBlock / LPR;
    dim3 grid((unsigned)((kp.d_inner + rows - 1) / rows), (unsigned)S, 1);
    hipLaunchKernelGGL((scan_fwd_rows<T, LPR, PSA, K, G1>), grid, dim3(kBlock), 0, stream, kp);
    return hipGetLastError() == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

template <typename T, int LPR, bool PSA, int K>
int pick_g(const FwdKP& kp, int64_t S, hipStream_t st) {
    return kp.G == 1 ? launch_rows<T, LPR, PSA, K, true>(kp, S, st)
                     : launch_rows<T, LPR, PSA, K, false>(kp, S, st);
}

template <typename T, int LPR, bool PSA>
int pick_k(const FwdKP& kp, int K, int64_t S, hipStream_t st) {
    if constexpr (LPR == 1) {
        switch (K) {
            case 0: return pick_g<T, LPR, PSA, 0>(kp, S, st);
            case 2: return pick_g<T, LPR, PSA, 2>(kp, S, st);
            case 3: return pick_g<T, LPR, PSA, 3>(kp, S, st);
            case 4: return pick_g<T, LPR, PSA, 4>(kp, S, st);
            default: return SSM_ERR_UNSUPPORTED;
        }
    } else {
        return K == 0 ? pick_g<T, LPR, PSA, 0>(kp, S, st) : SSM_ERR_UNSUPPORTED;
    }
}

template <typename T, bool PSA>
int pick_lpr(const FwdKP& kp, int K, int64_t S, hipStream_t st) {
    const int N = kp.N;
    if (N <= 16) return pick_k<T, 1, PSA>(kp, K, S, st);
    if (N <= 32) return pick_k<T, 2, PSA>(kp, K, S, st);
    if (N <= 64) return pick_k<T, 4, PSA>(kp, K, S, st);
    if (N <= 128) return pick_k<T, 8, PSA>(kp, K, S, st);
    if (N <= 256) return pick_k<T, 16, PSA>(kp, K, S, st);
    return SSM_ERR_UNSUPPORTED;
}

}  // namespace

size_t fwd_workspace_bytes(const Shape& sh) {
    return quad_supported(sh) ? quad_workspace_bytes(sh) : 0;
}

FwdPath fwd_path(const FwdArgs& a) {
    const Shape& sh = a.sh;
    if (sh.S == 0 || sh.H * sh.P == 0) return FwdPath::kNone;
    // few (sequence, channel) rows and no explicit chunk: split time inside a workgroup
    if (sh.chunk == 0 && sh.S * ((sh.d_inner() + 63) / 64) * 4 < 2048 && ts_supported(sh, a))
        return FwdPath::kTimeSplit;
    if (quad_supported(sh)) return FwdPath::kQuad;
    if (ssd_supported(sh, a)) return FwdPath::kSsd;
    return FwdPath::kRows;
}

int launch_scan_fwd(const FwdArgs& a, hipStream_t stream) {
    const Shape& sh = a.sh;
    switch (fwd_path(a)) {
        case FwdPath::kNone: return SSM_OK;
        case FwdPath::kTimeSplit: return launch_ts_fwd(a, stream);
        case FwdPath::kQuad: return launch_quad_fwd(a, stream);
        case FwdPath::kSsd: return launch_ssd_fwd(a, stream);
        case FwdPath::kRows: break;
    }
    FwdKP kp;
    kp.s = a.s; kp.x = a.x; kp.dt = a.dt; kp.A = a.A; kp.B = a.B; kp.C = a.C; kp.D = a.D;
    kp.ids = a.ids; kp.conv_w = a.conv_w; kp.conv_state = a.conv_state;
    kp.y = a.y; kp.state_out = a.state_out; kp.conv_state_out = a.conv_state_out; kp.err = a.err;
    kp.dt_bias = a.dt_bias; kp.z = a.z; kp.cu = a.cu; kp.T = a.T;
    kp.L = (int)sh.L; kp.H = (int)sh.H; kp.P = (int)sh.P; kp.N = (int)sh.N; kp.G = (int)sh.G;
    kp.R = (int)sh.R; kp.d_inner = (int)sh.d_inner(); kp.heads_per_group = (int)(sh.H / sh.G);
    kp.has_D = (sh.flags & SSM_HAS_D) ? 1 : 0;
    kp.softplus = (sh.flags & SSM_DT_SOFTPLUS) ? 1 : 0;
    if (sh.io == SSM_F32)
        return sh.a_per_state ? pick_lpr<float, true>(kp, sh.K, sh.S, stream)
                              : pick_lpr<float, false>(kp, sh.K, sh.S, stream);
    return sh.a_per_state ? pick_lpr<bf16_t, true>(kp, sh.K, sh.S, stream)
                          : pick_lpr<bf16_t, false>(kp, sh.K, sh.S, stream);
}

}  // namespace ssm
