// Generic selective-scan backward for gfx950: every shape the forward takes
// (Mamba-1 and Mamba-2 forms, any head_dim, d_state up to 256, several B/C
// groups, f32 or bf16 io, softplus on dt) and the fused causal conv + SiLU.
//
// The adjoint is the one of the specialised kernels (scan_bwd.hip): with
// g = dL/dh_t ("kizzasi-model backprop_ssm.rs", ssm_backward) and the
// per-element terms of "mambazip mamba1/model.rs"
// (accumulate_token_step_gradients):
//     g     += C_t dy_t;            dC_t += dy_t h_t
//     du_t   = D dy_t + dt_t sum_n g_n B_tn;      dB_t += g dt_t u_t
//     ddt_t  = sum_n g_n (h_{t-1,n} a_tn A_n + B_tn u_t)
//     dA    += g h_{t-1} a_t dt_t;   g *= a_t
// With the fused conv, u_t = SiLU(c_t), c_t = sum_j w_j in(t - (K-1) + j),
// where in() is the conv state before token 0 and x after (the ggml ssm_conv
// tap order: the last tap on the newest input), so
//     dc_t = du_t sigma(c_t) (1 + c_t (1 - sigma(c_t)))
//     d in(tau) = sum_j w_j dc_{tau + K-1-j},   dw_j += dc_t in(t - (K-1) + j)
// and d in(tau) for tau < 0 is the gradient of the gathered conv-state row.
//
// Layout.  A "row" is one (sequence i, channel c = h*head_dim + p).  LPR
// lanes share a row and lane j keeps its states 4j..4j+3 in registers.  A
// workgroup (256 lanes) owns 256/LPR consecutive rows of one B/C group.
//  1. bwd_rows_ckpt runs the forward and stores the state entering every
//     8-token block (a checkpoint).
//  2. bwd_rows walks the blocks backwards: it recomputes the block's decays,
//     states and scan inputs from the checkpoint into registers, then runs
//     the adjoint from the block's last token.  The conv adjoint keeps the
//     last K-1 values of dc in registers across blocks.  Each workgroup
//     handles the row blocks w, w+W, ... of its group, so that the sums over
//     channels of dB and dC (across the row's lanes by shuffles, the wave's
//     rows by shuffles, the four waves through LDS) land in W partial slabs
//     per (sequence, group): a bounded workspace, written without atomics.
//  3. Fixed-order reductions: the slabs for dB and dC, the channels of a head
//     for d(dt) (head_dim > 1), sequences for dA, dD and the conv weights,
//     and the rows named by ids for d_s and the conv state.
// Every sum has a fixed order, so results are bitwise repeatable.
#include "device_common.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

constexpr int kT = 256;        // threads per workgroup
constexpr int kSPL = 4;        // states per lane
constexpr int kKb = kCkpt;     // tokens per recompute block (checkpoint spacing)
constexpr int kMaxK = 4;       // conv taps handled here
constexpr size_t kSlabBudget = size_t(256) << 20;  // bytes of dB/dC partial slabs

struct RowsKP {
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
    const void* dy;
    const float* dstate;
    float* ckpt;     // [n_blk][S][d_inner][NP]
    float* d_x;      // [S][L][d_inner]
    float* d_dt;     // head_dim 1: the output [S][L][H]; else partials [S][L][d_inner]
    float* slab;     // [S][G][W][L][2N]: dB then dC of each workgroup's rows
    float* partA;    // [S][d_inner][NP]
    float* partD;    // [S][d_inner]
    float* partS;    // [S][d_inner][NP]: dh_0
    float* partW;    // [S][d_inner][K]
    float* partCS;   // [S][d_inner][K-1]
    uint32_t* err;
    int S, L, H, P, N, G, R, K, d_inner, cpg, NP, W, nrb, n_blk;
    int psa, has_D, softplus;
};

template <typename T>
__device__ __forceinline__ float ldg(const void* base, int64_t idx) {
    return to_f32(static_cast<const T*>(base)[idx]);
}

// Sum over the LPR lanes of a row (every lane of the row gets the total).
template <int LPR>
__device__ __forceinline__ float row_sum(float v) {
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) v += __shfl_xor(v, m);
    return v;
}

// Sum over the rows of a wave, lane by lane within the row (lanes j, j+LPR, ...).
template <int LPR>
__device__ __forceinline__ float wave_rows_sum(float v) {
#pragma unroll
    for (int m = LPR; m < 64; m <<= 1) v += __shfl_xor(v, m);
    return v;
}

// Row of this lane in the workgroup's row block rb of group g.
struct RowOf {
    int c, h;
    bool active;
};
__device__ __forceinline__ RowOf row_of(const RowsKP& p, int g, int rb, int lr, int rwg) {
    const int cg = rb * rwg + lr;  // channel within the group
    RowOf o;
    o.active = cg < p.cpg;
    o.c = g * p.cpg + (o.active ? cg : p.cpg - 1);
    o.h = o.c / p.P;
    return o;
}

// Conv input tau of sequence i, channel c (head_dim 1): conv state before token 0.
template <typename T>
__device__ __forceinline__ float conv_in(const RowsKP& p, int i, int r, int c, int tau, bool bad) {
    if (tau >= 0) return ldg<T>(p.x, ((int64_t)i * p.L + tau) * p.d_inner + c);
    if (bad) return __builtin_nanf("");
    return p.conv_state ? p.conv_state[((int64_t)r * p.H + c) * (p.K - 1) + tau + p.K - 1] : 0.0f;
}

template <typename T>
__device__ __forceinline__ float pre_act(const RowsKP& p, const float (&w)[kMaxK], int i, int r, int c,
                                         int t, bool bad) {
    float acc = 0.0f;
#pragma unroll
    for (int q = 0; q < kMaxK; ++q)
        if (q < p.K) acc = fmaf(w[q], conv_in<T>(p, i, r, c, t - (p.K - 1) + q, bad), acc);
    return acc;
}

template <typename T>
__device__ __forceinline__ float scan_u(const RowsKP& p, const float (&w)[kMaxK], int i, int r, int c,
                                        int t, bool bad, float* pre) {
    if (p.K == 0) return ldg<T>(p.x, ((int64_t)i * p.L + t) * p.d_inner + c);
    const float z = pre_act<T>(p, w, i, r, c, t, bad);
    *pre = z;
    return silu(z);
}

template <typename T, int LPR>
__global__ __launch_bounds__(kT) void bwd_rows_ckpt(RowsKP p) {
    constexpr int RWG = kT / LPR;
    const int lr = threadIdx.x / LPR, j = threadIdx.x % LPR;
    const int g = blockIdx.x / p.nrb, rb = blockIdx.x % p.nrb;
    const int i = blockIdx.y;
    const RowOf ro = row_of(p, g, rb, lr, RWG);
    int r = p.ids[i];
    const bool bad = (r < 0) | (r >= p.R);
    if (bad) {
        r = 0;
        if (threadIdx.x == 0 && blockIdx.x == 0) atomicOr(p.err, (uint32_t)SSM_DEVERR_IDS);
    }
    float hs[kSPL], a2[kSPL];
#pragma unroll
    for (int s = 0; s < kSPL; ++s) {
        const int n = kSPL * j + s;
        const bool on = n < p.N;
        hs[s] = on ? (bad ? __builtin_nanf("") : p.s[((int64_t)r * p.d_inner + ro.c) * p.N + n]) : 0.0f;
        a2[s] = on ? (p.psa ? p.A[(int64_t)ro.h * p.N + n] : p.A[ro.h]) * kLog2e : 0.0f;
    }
    float w[kMaxK] = {0.f, 0.f, 0.f, 0.f};
    for (int q = 0; q < p.K; ++q) w[q] = p.conv_w[(int64_t)ro.c * p.K + q];
    const int grp = g;
    for (int t = 0; t < p.L; ++t) {
        if ((t % kKb) == 0 && ro.active) {
            float* ck = p.ckpt + (((int64_t)(t / kKb) * p.S + i) * p.d_inner + ro.c) * p.NP + kSPL * j;
            *reinterpret_cast<float4*>(ck) = make_float4(hs[0], hs[1], hs[2], hs[3]);
        }
        float d = ldg<T>(p.dt, ((int64_t)i * p.L + t) * p.H + ro.h);
        if (p.softplus) d = softplus(d);
        float pre;
        const float u = scan_u<T>(p, w, i, r, ro.c, t, bad, &pre);
        const float du = d * u;
        const int64_t bc = (((int64_t)i * p.L + t) * p.G + grp) * p.N;
#pragma unroll
        for (int s = 0; s < kSPL; ++s) {
            const int n = kSPL * j + s;
            const float Bn = n < p.N ? ldg<T>(p.B, bc + n) : 0.0f;
            hs[s] = fmaf(fast_exp2(d * a2[s]), hs[s], du * Bn);
        }
    }
}

template <typename T, int LPR>
__global__ __launch_bounds__(kT) void bwd_rows(RowsKP p) {
    constexpr int RWG = kT / LPR;
    constexpr int NP = kSPL * LPR;
    // per token of the block, per wave: the wave's sum of dB (then dC) over its rows
    __shared__ __attribute__((aligned(16))) float red[kKb][4][2][NP];
    const int tid = threadIdx.x;
    const int lr = tid / LPR, j = tid % LPR, wave = tid >> 6;
    const bool row0 = (tid & 63) < LPR;  // lanes of the wave's first row
    const int w_id = blockIdx.x % p.W, g = blockIdx.x / p.W;
    const int i = blockIdx.y;
    int r = p.ids[i];
    const bool bad = (r < 0) | (r >= p.R);
    if (bad) {
        r = 0;
        if (tid == 0 && blockIdx.x == 0) atomicOr(p.err, (uint32_t)SSM_DEVERR_IDS);
    }
    const float nan = __builtin_nanf("");

    for (int rb = w_id; rb < p.nrb; rb += p.W) {
        const RowOf ro = row_of(p, g, rb, lr, RWG);
        const bool first = rb == w_id;
        float a2[kSPL], An[kSPL], gs[kSPL], dA[kSPL];
#pragma unroll
        for (int s = 0; s < kSPL; ++s) {
            const int n = kSPL * j + s;
            const bool on = n < p.N;
            An[s] = on ? (p.psa ? p.A[(int64_t)ro.h * p.N + n] : p.A[ro.h]) : 0.0f;
            a2[s] = An[s] * kLog2e;
            gs[s] = on ? p.dstate[((int64_t)i * p.d_inner + ro.c) * p.N + n] : 0.0f;
            dA[s] = 0.0f;
        }
        const float Dh = p.has_D ? p.D[ro.h] : 0.0f;
        float w[kMaxK] = {0.f, 0.f, 0.f, 0.f};
        for (int q = 0; q < p.K; ++q) w[q] = p.conv_w[(int64_t)ro.c * p.K + q];
        float ring[kMaxK - 1] = {0.f, 0.f, 0.f};  // dc of the K-1 tokens after the current one
        float dw[kMaxK] = {0.f, 0.f, 0.f, 0.f};
        float dD = 0.0f;

        for (int b = p.n_blk - 1; b >= 0; --b) {
            const int t0 = b * kKb;
            const int nk = min(kKb, p.L - t0);
            // recompute the block from its checkpoint
            float a[kKb][kSPL], hh[kKb][kSPL], hprev0[kSPL];
            float dk[kKb], uk[kKb], zk[kKb], rawk[kKb];
            {
                const float4 ck = *reinterpret_cast<const float4*>(
                    p.ckpt + (((int64_t)b * p.S + i) * p.d_inner + ro.c) * p.NP + kSPL * j);
                hprev0[0] = ck.x; hprev0[1] = ck.y; hprev0[2] = ck.z; hprev0[3] = ck.w;
            }
#pragma unroll
            for (int k = 0; k < kKb; ++k) {
                const int t = t0 + k;
                const bool on = k < nk;
                const int tc = on ? t : t0;  // a valid token for the loads
                const float raw = ldg<T>(p.dt, ((int64_t)i * p.L + tc) * p.H + ro.h);
                float d = p.softplus ? softplus(raw) : raw;
                float pre = 0.0f;
                float u = scan_u<T>(p, w, i, r, ro.c, tc, bad, &pre);
                if (!on) { d = 0.0f; u = 0.0f; }
                dk[k] = d; uk[k] = u; zk[k] = pre; rawk[k] = raw;
                const float du = d * u;
                const int64_t bc = (((int64_t)i * p.L + tc) * p.G + g) * p.N;
#pragma unroll
                for (int s = 0; s < kSPL; ++s) {
                    const int n = kSPL * j + s;
                    const float Bn = n < p.N ? ldg<T>(p.B, bc + n) : 0.0f;
                    a[k][s] = fast_exp2(d * a2[s]);
                    hh[k][s] = fmaf(a[k][s], k == 0 ? hprev0[s] : hh[k - 1][s], du * Bn);
                }
            }
            // adjoint over the block, last token first
#pragma unroll
            for (int k = kKb - 1; k >= 0; --k) {
                const int t = t0 + k;
                const bool on = k < nk;
                const int tc = on ? t : t0;
                const float dyk = on ? ldg<T>(p.dy, ((int64_t)i * p.L + tc) * p.d_inner + ro.c) : 0.0f;
                const int64_t bc = (((int64_t)i * p.L + tc) * p.G + g) * p.N;
                float S1 = 0.0f, S2 = 0.0f, dBp[kSPL], dCp[kSPL];
#pragma unroll
                for (int s = 0; s < kSPL; ++s) {
                    const int n = kSPL * j + s;
                    const bool sn = n < p.N && on;
                    const float Bn = sn ? ldg<T>(p.B, bc + n) : 0.0f;
                    const float Cn = sn ? ldg<T>(p.C, bc + n) : 0.0f;
                    gs[s] = fmaf(Cn, dyk, gs[s]);
                    dCp[s] = dyk * hh[k][s];
                    S1 = fmaf(gs[s], Bn, S1);
                    const float ga = gs[s] * a[k][s];
                    const float qv = ga * (k == 0 ? hprev0[s] : hh[k - 1][s]);
                    S2 = fmaf(qv, An[s], S2);
                    dA[s] = fmaf(qv, dk[k], dA[s]);
                    dBp[s] = gs[s] * (dk[k] * uk[k]);
                    gs[s] = ga;
                }
                S1 = row_sum<LPR>(S1);
                S2 = row_sum<LPR>(S2);
                // channel sums of dB and dC over the wave's rows
#pragma unroll
                for (int s = 0; s < kSPL; ++s) {
                    const float vb = ro.active ? dBp[s] : 0.0f, vc = ro.active ? dCp[s] : 0.0f;
                    dBp[s] = wave_rows_sum<LPR>(vb);
                    dCp[s] = wave_rows_sum<LPR>(vc);
                }
                if (row0) {
                    *reinterpret_cast<float4*>(&red[k][wave][0][kSPL * j]) = make_float4(dBp[0], dBp[1], dBp[2], dBp[3]);
                    *reinterpret_cast<float4*>(&red[k][wave][1][kSPL * j]) = make_float4(dCp[0], dCp[1], dCp[2], dCp[3]);
                }
                if (j == 0 && ro.active && on) {
                    const float du_t = fmaf(Dh, dyk, dk[k] * S1);
                    float ddt = fmaf(uk[k], S1, S2);
                    if (p.softplus) ddt *= sigmoid(rawk[k]);
                    if (p.has_D) dD = fmaf(dyk, uk[k], dD);
                    const int64_t tok = (int64_t)i * p.L + t;
                    if (p.P == 1) p.d_dt[tok * p.H + ro.h] = bad ? nan : ddt;
                    else p.d_dt[tok * p.d_inner + ro.c] = bad ? nan : ddt;
                    if (p.K == 0) {
                        p.d_x[tok * p.d_inner + ro.c] = bad ? nan : du_t;
                    } else {
                        const float sg = sigmoid(zk[k]);
                        const float dc = du_t * (sg * fmaf(zk[k], 1.0f - sg, 1.0f));
                        float gin = w[p.K - 1] * dc;
#pragma unroll
                        for (int m = 0; m < kMaxK - 1; ++m)
                            if (m < p.K - 1) gin = fmaf(w[p.K - 2 - m], ring[m], gin);
                        p.d_x[tok * p.d_inner + ro.c] = bad ? nan : gin;
#pragma unroll
                        for (int q = 0; q < kMaxK; ++q)
                            if (q < p.K) dw[q] = fmaf(dc, conv_in<T>(p, i, r, ro.c, t - (p.K - 1) + q, bad), dw[q]);
#pragma unroll
                        for (int m = kMaxK - 2; m >= 1; --m) ring[m] = ring[m - 1];
                        ring[0] = dc;
                    }
                }
            }
            __syncthreads();
            // this block's channel sums into the workgroup's slab, in a fixed order
            const int per_tok = 2 * p.N;
            float* sl = p.slab + ((((int64_t)i * p.G + g) * p.W + w_id) * p.L + t0) * per_tok;
            for (int e = tid; e < nk * per_tok; e += kT) {
                const int k = e / per_tok, rem = e % per_tok;
                const int which = rem / p.N, n = rem % p.N;
                float v = red[k][0][which][n];
                v += red[k][1][which][n];
                v += red[k][2][which][n];
                v += red[k][3][which][n];
                sl[e] = first ? v : sl[e] + v;
            }
            __syncthreads();
        }
        if (ro.active) {
            const int64_t row_i = (int64_t)i * p.d_inner + ro.c;
            *reinterpret_cast<float4*>(p.partS + row_i * p.NP + kSPL * j) = make_float4(gs[0], gs[1], gs[2], gs[3]);
            *reinterpret_cast<float4*>(p.partA + row_i * p.NP + kSPL * j) = make_float4(dA[0], dA[1], dA[2], dA[3]);
            if (j == 0) {
                p.partD[row_i] = dD;
                if (p.K > 0) {
                    for (int q = 0; q < p.K; ++q) p.partW[row_i * p.K + q] = dw[q];
                    // the conv-state inputs tau = m - (K-1): sum_j w_j dc_{m-j} (ring[k] = dc_k now)
                    for (int m = 0; m < p.K - 1; ++m) {
                        float gcs = 0.0f;
                        for (int q = 0; q <= m; ++q) gcs = fmaf(w[q], ring[m - q], gcs);
                        p.partCS[row_i * (p.K - 1) + m] = gcs;
                    }
                }
            }
        }
    }
}

// d_B, d_C: the W slabs of the group in slab order.
__global__ __launch_bounds__(256) void rows_reduce_bc(RowsKP p, float* d_B, float* d_C) {
    const int64_t total = (int64_t)p.S * p.L * p.G * p.N;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += stride) {
        const int n = (int)(e % p.N);
        const int64_t rest = e / p.N;
        const int g = (int)(rest % p.G);
        const int64_t tok = rest / p.G;  // i * L + t
        const int64_t i = tok / p.L, t = tok % p.L;
        float b = 0.0f, c = 0.0f;
        for (int w = 0; w < p.W; ++w) {
            const float* sl = p.slab + (((i * p.G + g) * p.W + w) * p.L + t) * 2 * p.N;
            b += sl[n];
            c += sl[p.N + n];
        }
        d_B[e] = b;
        d_C[e] = c;
    }
}

// d(dt) with head_dim > 1: the head's channels in channel order.
__global__ __launch_bounds__(256) void rows_reduce_dt(RowsKP p, const float* part, float* d_dt) {
    const int64_t total = (int64_t)p.S * p.L * p.H;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += stride) {
        const int64_t tok = e / p.H;
        const int h = (int)(e % p.H);
        const float* src = part + tok * p.d_inner + (int64_t)h * p.P;
        float acc = 0.0f;
        for (int q = 0; q < p.P; ++q) acc += src[q];
        d_dt[e] = acc;
    }
}

// d_A, d_D, d_conv_w: sums over sequences (then channels, then states) in
// that order; d_s and d_conv_state: the rows whose id this is, in sequence
// order (zero when no sequence names the row).
__global__ __launch_bounds__(256) void rows_reduce_params(RowsKP p, float* d_A, float* d_D, float* d_s,
                                                          float* d_cw, float* d_cs) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    const int64_t e0 = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t nA = p.psa ? (int64_t)p.H * p.N : p.H;
    for (int64_t e = e0; e < nA; e += stride) {
        const int h = (int)(p.psa ? e / p.N : e);
        float acc = 0.0f;
        for (int i = 0; i < p.S; ++i)
            for (int q = 0; q < p.P; ++q) {
                const float* src = p.partA + ((int64_t)i * p.d_inner + (int64_t)h * p.P + q) * p.NP;
                if (p.psa) acc += src[e % p.N];
                else for (int n = 0; n < p.N; ++n) acc += src[n];
            }
        d_A[e] = acc;
    }
    if (d_D)
        for (int64_t e = e0; e < p.H; e += stride) {
            float acc = 0.0f;
            for (int i = 0; i < p.S; ++i)
                for (int q = 0; q < p.P; ++q) acc += p.partD[(int64_t)i * p.d_inner + e * p.P + q];
            d_D[e] = acc;
        }
    const int64_t per_row = (int64_t)p.d_inner * p.N;
    for (int64_t f = e0; f < (int64_t)p.R * per_row; f += stride) {
        const int64_t r = f / per_row, rem = f % per_row;
        const int64_t c = rem / p.N;
        const int n = (int)(rem % p.N);
        float acc = 0.0f;
        for (int i = 0; i < p.S; ++i)
            if (p.ids[i] == r) acc += p.partS[((int64_t)i * p.d_inner + c) * p.NP + n];
        d_s[f] = acc;
    }
    if (p.K > 0) {
        for (int64_t e = e0; e < (int64_t)p.H * p.K; e += stride) {
            float acc = 0.0f;
            for (int i = 0; i < p.S; ++i) acc += p.partW[(int64_t)i * p.H * p.K + e];
            d_cw[e] = acc;
        }
        const int64_t per_cs = (int64_t)p.H * (p.K - 1);
        for (int64_t f = e0; f < (int64_t)p.R * per_cs; f += stride) {
            const int64_t r = f / per_cs, rem = f % per_cs;
            float acc = 0.0f;
            for (int i = 0; i < p.S; ++i)
                if (p.ids[i] == r) acc += p.partCS[(int64_t)i * per_cs + rem];
            d_cs[f] = acc;
        }
    }
}

int lpr_of(int64_t N) {
    int lpr = 1;
    while (lpr * kSPL < N) lpr <<= 1;
    return lpr;
}

struct RowsWs {
    float *ckpt, *slab, *ddt, *A, *D, *S, *W, *CS;
    int W_count;
    size_t total;
};

RowsWs rows_carve(const Shape& sh, char* base) {
    const int lpr = lpr_of(sh.N), np = kSPL * lpr, rwg = kT / lpr;
    const int64_t cpg = sh.d_inner() / sh.G;
    const int64_t nrb = (cpg + rwg - 1) / rwg;
    const size_t per_w = (size_t)sh.S * sh.G * sh.L * 2 * sh.N * 4;
    int64_t wc = per_w ? (int64_t)(kSlabBudget / per_w) : nrb;
    if (wc < 1) wc = 1;
    if (wc > nrb) wc = nrb;
    const size_t rows = (size_t)sh.S * sh.d_inner();
    const size_t n_blk = (size_t)((sh.L + kKb - 1) / kKb);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        char* ptr = base ? base + off : nullptr;
        off += align_up(bytes, 256);
        return reinterpret_cast<float*>(ptr);
    };
    RowsWs w;
    w.W_count = (int)wc;
    w.ckpt = take(n_blk * rows * np * 4);
    w.slab = take(per_w * (size_t)wc);
    w.ddt = take(sh.P > 1 ? rows * sh.L * 4 : 0);
    w.A = take(rows * np * 4);
    w.D = take(rows * 4);
    w.S = take(rows * np * 4);
    w.W = take(rows * (size_t)(sh.K > 0 ? sh.K : 0) * 4);
    w.CS = take(rows * (size_t)(sh.K > 1 ? sh.K - 1 : 0) * 4);
    w.total = off;
    return w;
}

template <typename T, int LPR>
void launch_rows_t(const RowsKP& kp, hipStream_t st) {
    if (kp.S > 0 && kp.L > 0)
        hipLaunchKernelGGL((bwd_rows_ckpt<T, LPR>), dim3((unsigned)(kp.nrb * kp.G), (unsigned)kp.S),
                           dim3(kT), 0, st, kp);
    if (kp.S > 0)
        hipLaunchKernelGGL((bwd_rows<T, LPR>), dim3((unsigned)(kp.W * kp.G), (unsigned)kp.S), dim3(kT),
                           0, st, kp);
}

template <typename T>
int pick_lpr(const RowsKP& kp, int lpr, hipStream_t st) {
    switch (lpr) {
        case 1: launch_rows_t<T, 1>(kp, st); return SSM_OK;
        case 2: launch_rows_t<T, 2>(kp, st); return SSM_OK;
        case 4: launch_rows_t<T, 4>(kp, st); return SSM_OK;
        case 8: launch_rows_t<T, 8>(kp, st); return SSM_OK;
        case 16: launch_rows_t<T, 16>(kp, st); return SSM_OK;
        case 32: launch_rows_t<T, 32>(kp, st); return SSM_OK;
        case 64: launch_rows_t<T, 64>(kp, st); return SSM_OK;
        default: return SSM_ERR_UNSUPPORTED;
    }
}

}  // namespace

bool rows_bwd_supported(const Shape& sh) {
    return sh.N <= 256 && (sh.K == 0 || (sh.P == 1 && sh.K >= 2 && sh.K <= kMaxK)) &&
           sh.S <= 65535 && sh.G * ((sh.d_inner() / sh.G + kT - 1) / kT) * kT <= (int64_t(1) << 31);
}

size_t rows_bwd_workspace_bytes(const Shape& sh) { return rows_carve(sh, nullptr).total; }

int launch_rows_bwd(const BwdArgs& a, hipStream_t stream) {
    const Shape& sh = a.sh;
    if (!rows_bwd_supported(sh)) return SSM_ERR_UNSUPPORTED;
    const int lpr = lpr_of(sh.N);
    RowsWs w = rows_carve(sh, a.ws);
    if (w.total > a.ws_bytes) return SSM_ERR_WORKSPACE;
    RowsKP kp = {};
    kp.s = a.s; kp.x = a.x; kp.dt = a.dt; kp.A = a.A; kp.B = a.B; kp.C = a.C;
    kp.D = a.D; kp.ids = a.ids; kp.conv_w = a.conv_w; kp.conv_state = a.conv_state;
    kp.dy = a.dy; kp.dstate = a.dstate;
    kp.ckpt = w.ckpt; kp.d_x = a.d_x; kp.d_dt = sh.P > 1 ? w.ddt : a.d_dt; kp.slab = w.slab;
    kp.partA = w.A; kp.partD = w.D; kp.partS = w.S; kp.partW = w.W; kp.partCS = w.CS;
    kp.err = a.err;
    kp.S = (int)sh.S; kp.L = (int)sh.L; kp.H = (int)sh.H; kp.P = (int)sh.P; kp.N = (int)sh.N;
    kp.G = (int)sh.G; kp.R = (int)sh.R; kp.K = sh.K; kp.d_inner = (int)sh.d_inner();
    kp.cpg = (int)(sh.d_inner() / sh.G); kp.NP = kSPL * lpr;
    kp.W = w.W_count;
    kp.nrb = (kp.cpg + kT / lpr - 1) / (kT / lpr);
    kp.n_blk = (int)((sh.L + kKb - 1) / kKb);
    kp.psa = sh.a_per_state; kp.has_D = (sh.flags & SSM_HAS_D) ? 1 : 0;
    kp.softplus = (sh.flags & SSM_DT_SOFTPLUS) ? 1 : 0;
    if (sh.S > 0) {
        const int rc = sh.io == SSM_BF16 ? pick_lpr<bf16_t>(kp, lpr, stream) : pick_lpr<float>(kp, lpr, stream);
        if (rc) return rc;
    }
    auto blocks = [](int64_t n) {
        const int64_t b = (n + 255) / 256;
        return (unsigned)(b < 1 ? 1 : (b > 16384 ? 16384 : b));
    };
    const int64_t nbc = sh.S * sh.L * sh.G * sh.N;
    if (nbc > 0) hipLaunchKernelGGL(rows_reduce_bc, dim3(blocks(nbc)), dim3(256), 0, stream, kp, a.d_B, a.d_C);
    if (sh.P > 1 && sh.S * sh.L > 0)
        hipLaunchKernelGGL(rows_reduce_dt, dim3(blocks(sh.S * sh.L * sh.H)), dim3(256), 0, stream, kp,
                           (const float*)w.ddt, a.d_dt);
    int64_t par = sh.R * sh.d_inner() * sh.N;
    if (sh.H * sh.N > par) par = sh.H * sh.N;
    hipLaunchKernelGGL(rows_reduce_params, dim3(blocks(par)), dim3(256), 0, stream, kp, a.d_A, a.D ? a.d_D : nullptr,
                       a.d_s, a.d_conv_w, a.d_conv_state);
    return hipGetLastError() == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

}  // namespace ssm
