// Mamba-2 form (one scalar A per head, B/C shared by the heads of a group)
// forward as a chunked "state-space dual" (SSD) computation on MFMA, gfx950.
//
// The recurrence per (sequence i, head h, channel p, state n) is
//     h_t = a_t h_{t-1} + dt_t B_t x_t,   a_t = exp(dt_t A_h),   y_t = C_t . h_t + D_h x_t
// (the ggml ssm_scan operands of the ggmlR page, "make_scan", with the decay
// of "mambazip mamba1/model.rs" made scalar per head).  With l_t = dt_t A_h
// and cum_t = sum of l over the chunk up to and including t, unrolling the
// recurrence over a chunk that starts from state h_in gives, for t in the
// chunk,
//     h_t = exp(cum_t) h_in + sum_{s<=t} exp(cum_t - cum_s) dt_s x_s B_s
//     y_t = sum_{s<=t} (C_t . B_s) exp(cum_t - cum_s) dt_s x_s      (intra-chunk)
//         + exp(cum_t) C_t . h_in                                    (carried state)
//         + D_h x_t
// which are dense products: G = C B^T (Q x Q over the states), M = G o L with
// L[t][s] = exp(cum_t - cum_s) dt_s for s <= t (0 above the diagonal),
// Y = M X + diag(exp(cum)) (C h_in^T), and the state at the chunk end
// h_out = exp(cum_last) h_in + (w o X)^T B with w_s = exp(cum_last - cum_s) dt_s.
// This chunked form is derived here from the recurrence; it reaches the
// sequential result up to rounding.  Every exponent is cum_t - cum_s with
// s <= t, which is <= 0 for A <= 0, so no term overflows.
//
// One workgroup (4 waves) runs one (sequence, head) through its chunks in
// order, keeping the fp32 state [P][N] in MFMA accumulators.  Products run
// on v_mfma_f32_16x16x32_bf16 (bf16 operands, fp32 accumulation); every
// operand tile is read from LDS as one 16-byte load per lane from a
// row-major tile whose k index is contiguous.  The chunk's x, B, C are
// fetched into registers one chunk ahead and written to LDS (natural and
// transposed copies) after the current chunk is done.
#include "device_common.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kQ = 64;       // tokens per chunk
constexpr int kPad = 8;      // bf16 elements of row padding (16 bytes): 2-way LDS bank use
constexpr int kThreads = 256;

struct SsdKP {
    const float* s;
    const bf16_t* x;
    const bf16_t* dt;
    const float* A;
    const bf16_t* B;
    const bf16_t* C;
    const float* D;
    const int32_t* ids;
    bf16_t* y;
    float* state_out;
    uint32_t* err;
    int L, H, G, R, hpg;
    int has_D, softplus;
};

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Operand fragment of a 16 x 32 (rows x k) block of a row-major bf16 tile
// with row stride `stride` elements: lane l reads row r0 + l%16, k0 + 8*(l/16).
__device__ __forceinline__ bf16x8 frag(const bf16_t* tile, int stride, int r0, int k0, int lane) {
    return *reinterpret_cast<const bf16x8*>(tile + (r0 + (lane & 15)) * stride + k0 + 8 * (lane >> 4));
}

__device__ __forceinline__ float bfv(bf16_t v) { return to_f32(v); }

template <int P, int N, bool SOFTPLUS>
__global__ __launch_bounds__(kThreads) void ssd_fwd(SsdKP p) {
    static_assert(P % 16 == 0 && N % 32 == 0 && P <= 64 && N <= 128, "tile shapes");
    constexpr int SN = N + kPad;    // row stride of tiles with k = state
    constexpr int SQ = kQ + kPad;   // row stride of tiles with k = token
    constexpr int PB = P / 16;      // 16-row blocks of channels
    constexpr int NB = N / 16;      // 16-column blocks of states
    __shared__ __attribute__((aligned(16))) bf16_t C_l[kQ * SN];   // [t][n]
    __shared__ __attribute__((aligned(16))) bf16_t B_l[kQ * SN];   // [s][n]
    __shared__ __attribute__((aligned(16))) bf16_t BT_l[N * SQ];   // [n][s]
    __shared__ __attribute__((aligned(16))) bf16_t XT_l[P * SQ];   // [p][s]
    __shared__ __attribute__((aligned(16))) bf16_t XwT_l[P * SQ];  // [p][s] = w_s x_s,p
    __shared__ __attribute__((aligned(16))) bf16_t M_l[kQ * SQ];   // [t][s]
    __shared__ __attribute__((aligned(16))) bf16_t H_l[P * SN];    // [p][n] state, bf16 copy
    __shared__ float dt_l[kQ];
    __shared__ float cum_l[4][kQ], ecum_l[4][kQ], w_l[4][kQ];      // per-wave copies

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hh = (int)(blockIdx.x % (unsigned)p.H), i = (int)(blockIdx.x / (unsigned)p.H);
    const int g = hh / p.hpg;
    const float Ah = p.A[hh];
    const float Dh = p.has_D ? p.D[hh] : 0.0f;
    int r = p.ids[i];
    const bool bad = (r < 0) | (r >= p.R);
    if (bad) {
        r = 0;
        if (tid == 0) atomicOr(p.err, (uint32_t)SSM_DEVERR_IDS);
    }

    // M is zero above the diagonal for every chunk: clear it once
    for (int e = tid; e < kQ * SQ; e += kThreads) M_l[e] = bf16_t(0);

    // the state [P][N]: wave w owns channel block pb = w (if any), all NB state blocks
    f32x4 hacc[NB];
    const bool owns_state = wave < PB;
    const float* s0 = p.s + (((int64_t)r * p.H + hh) * P) * N;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int pp = wave * 16 + 4 * (lane >> 4) + k, n = nb * 16 + (lane & 15);
            hacc[nb][k] = owns_state ? (bad ? __builtin_nanf("") : s0[pp * N + n]) : 0.0f;
        }
    }
    if (owns_state) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int k = 0; k < 4; ++k)
                H_l[(wave * 16 + 4 * (lane >> 4) + k) * SN + nb * 16 + (lane & 15)] = bf16_rne(hacc[nb][k]);
    }

    // staging of one chunk: x [kQ][P], B and C [kQ][N] (bf16), dt [kQ]
    constexpr int XCH = kQ * P / 8, BCH = kQ * N / 8;   // 16-byte chunks
    constexpr int XPER = (XCH + kThreads - 1) / kThreads, BPER = (BCH + kThreads - 1) / kThreads;
    uint4 sx[XPER], sb[BPER], sc[BPER];
    float sdt = 0.0f;
    const int64_t tok_x = (int64_t)p.H * P;         // elements between tokens in x / y
    const int64_t tok_bc = (int64_t)p.G * N;        // elements between tokens in B / C
    const bf16_t* xg = p.x + ((int64_t)i * p.L * p.H + hh) * P;
    const bf16_t* bg = p.B + ((int64_t)i * p.L * p.G + g) * N;
    const bf16_t* cg = p.C + ((int64_t)i * p.L * p.G + g) * N;
    auto load_chunk = [&](int t0) {
#pragma unroll
        for (int k = 0; k < XPER; ++k) {
            const int e = tid + kThreads * k;
            const int t = e / (P / 8), pc = e % (P / 8);
            sx[k] = (e < XCH && t0 + t < p.L)
                        ? *reinterpret_cast<const uint4*>(xg + (int64_t)(t0 + t) * tok_x + pc * 8)
                        : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < BPER; ++k) {
            const int e = tid + kThreads * k;
            const int t = e / (N / 8), nc = e % (N / 8);
            const bool ok = e < BCH && t0 + t < p.L;
            sb[k] = ok ? *reinterpret_cast<const uint4*>(bg + (int64_t)(t0 + t) * tok_bc + nc * 8)
                       : make_uint4(0, 0, 0, 0);
            sc[k] = ok ? *reinterpret_cast<const uint4*>(cg + (int64_t)(t0 + t) * tok_bc + nc * 8)
                       : make_uint4(0, 0, 0, 0);
        }
        if (tid < kQ) {
            float v = (t0 + tid < p.L) ? bfv(p.dt[((int64_t)i * p.L + t0 + tid) * p.H + hh]) : 0.0f;
            if constexpr (SOFTPLUS) v = (t0 + tid < p.L) ? softplus(v) : 0.0f;
            sdt = v;
        }
    };
    auto store_chunk = [&]() {
#pragma unroll
        for (int k = 0; k < XPER; ++k) {
            const int e = tid + kThreads * k;
            if (e < XCH) {
                const int t = e / (P / 8), pc = e % (P / 8);
                const bf16_t* v = reinterpret_cast<const bf16_t*>(&sx[k]);
#pragma unroll
                for (int j = 0; j < 8; ++j) XT_l[(pc * 8 + j) * SQ + t] = v[j];
            }
        }
#pragma unroll
        for (int k = 0; k < BPER; ++k) {
            const int e = tid + kThreads * k;
            if (e < BCH) {
                const int t = e / (N / 8), nc = e % (N / 8);
                *reinterpret_cast<uint4*>(&B_l[t * SN + nc * 8]) = sb[k];
                *reinterpret_cast<uint4*>(&C_l[t * SN + nc * 8]) = sc[k];
                const bf16_t* v = reinterpret_cast<const bf16_t*>(&sb[k]);
#pragma unroll
                for (int j = 0; j < 8; ++j) BT_l[(nc * 8 + j) * SQ + t] = v[j];
            }
        }
        if (tid < kQ) dt_l[tid] = sdt;
    };

    const int n_chunks = (p.L + kQ - 1) / kQ;
    load_chunk(0);
    store_chunk();
    __syncthreads();
    for (int ch = 0; ch < n_chunks; ++ch) {
        const int t0 = ch * kQ;
        if (ch + 1 < n_chunks) load_chunk(t0 + kQ);

        // decays: every wave forms the chunk's cumulative log-decay itself (lane = token)
        float e_last;
        {
            const float lt = dt_l[lane] * Ah;
            float cum = lt;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const float o = __shfl_up(cum, d, 64);
                if (lane >= d) cum += o;
            }
            const float last = __shfl(cum, 63, 64);
            cum_l[wave][lane] = cum;
            ecum_l[wave][lane] = __expf(cum);
            w_l[wave][lane] = __expf(last - cum) * dt_l[lane];
            e_last = __expf(last);
        }
        // the wave reads its own copies back across lanes: LDS serves one wave in order
        __builtin_amdgcn_wave_barrier();
        const float* cumw = cum_l[wave];

        // G = C B^T on the causal 16x16 tiles, then M = G o L into M_l
        for (int tile = wave; tile < 10; tile += 4) {
            // tiles (tb, sb) with sb <= tb, numbered row by row
            const int tb = tile < 1 ? 0 : tile < 3 ? 1 : tile < 6 ? 2 : 3;
            const int sb = tile - (tb * (tb + 1)) / 2;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < N; kk += 32)
                acc = mfma(frag(C_l, SN, tb * 16, kk, lane), frag(B_l, SN, sb * 16, kk, lane), acc);
            const int s = sb * 16 + (lane & 15);
            const float cs = cumw[s], dts = dt_l[s];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int t = tb * 16 + 4 * (lane >> 4) + k;
                const float m = s <= t ? acc[k] * __expf(cumw[t] - cs) * dts : 0.0f;
                M_l[t * SQ + s] = bf16_rne(m);
            }
        }
        // XwT = w o X (transposed), for the state update
        for (int e = tid; e < P * kQ / 8; e += kThreads) {
            const int pp = e / (kQ / 8), sc8 = (e % (kQ / 8)) * 8;
            bf16x8 v = *reinterpret_cast<const bf16x8*>(&XT_l[pp * SQ + sc8]);
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = (__bf16)((float)v[j] * w_l[wave][sc8 + j]);
            *reinterpret_cast<bf16x8*>(&XwT_l[pp * SQ + sc8]) = v;
        }
        __syncthreads();

        // Y = M X + diag(exp(cum)) C H^T + D x: wave w computes channel block pb = w
        if (owns_state) {
            const int pb = wave;
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                f32x4 yd = {0.f, 0.f, 0.f, 0.f}, yo = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < (tb + 1) * 16; kk += 32)
                    yd = mfma(frag(M_l, SQ, tb * 16, kk, lane), frag(XT_l, SQ, pb * 16, kk, lane), yd);
#pragma unroll
                for (int kk = 0; kk < N; kk += 32)
                    yo = mfma(frag(C_l, SN, tb * 16, kk, lane), frag(H_l, SN, pb * 16, kk, lane), yo);
                const int pp = pb * 16 + (lane & 15);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int t = tb * 16 + 4 * (lane >> 4) + k;
                    if (t0 + t < p.L) {
                        const float xv = bfv(XT_l[pp * SQ + t]);
                        const float yv = fmaf(Dh, xv, fmaf(ecum_l[wave][t], yo[k], yd[k]));
                        p.y[((int64_t)i * p.L + t0 + t) * tok_x + (int64_t)hh * P + pp] = bf16_rne(yv);
                    }
                }
            }
            // state: h = exp(cum_last) h + (w o X)^T B
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                f32x4 a = hacc[nb];
#pragma unroll
                for (int k = 0; k < 4; ++k) a[k] *= e_last;
#pragma unroll
                for (int kk = 0; kk < kQ; kk += 32)
                    a = mfma(frag(XwT_l, SQ, pb * 16, kk, lane), frag(BT_l, SQ, nb * 16, kk, lane), a);
                hacc[nb] = a;
            }
        }
        __syncthreads();  // every wave is done with this chunk's tiles and with H_l
        if (owns_state) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    H_l[(wave * 16 + 4 * (lane >> 4) + k) * SN + nb * 16 + (lane & 15)] = bf16_rne(hacc[nb][k]);
        }
        if (ch + 1 < n_chunks) store_chunk();
        __syncthreads();
    }

    if (owns_state) {
        float* so = p.state_out + (((int64_t)i * p.H + hh) * P) * N;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int k = 0; k < 4; ++k)
                so[(wave * 16 + 4 * (lane >> 4) + k) * N + nb * 16 + (lane & 15)] = hacc[nb][k];
    }
}

template <int P, int N>
int launch_ssd_pn(const SsdKP& kp, int S, bool softplus, hipStream_t st) {
    const dim3 grid((unsigned)((int64_t)kp.H * S));
    if (softplus) hipLaunchKernelGGL((ssd_fwd<P, N, true>), grid, dim3(kThreads), 0, st, kp);
    else hipLaunchKernelGGL((ssd_fwd<P, N, false>), grid, dim3(kThreads), 0, st, kp);
    return hipGetLastError() == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

}  // namespace

bool ssd_supported(const Shape& sh, const FwdArgs& a) {
    auto al16 = [](const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) == 0; };
    return !sh.a_per_state && sh.io == SSM_BF16 && sh.K == 0 && (sh.P == 64 || sh.P == 32) &&
           (sh.N == 128 || sh.N == 64) && al16(a.x) && al16(a.B) && al16(a.C) && sh.L > 0 &&
           sh.S * sh.H < (int64_t(1) << 31);
}

int launch_ssd_fwd(const FwdArgs& a, hipStream_t stream) {
    const Shape& sh = a.sh;
    SsdKP kp;
    kp.s = a.s; kp.x = static_cast<const bf16_t*>(a.x); kp.dt = static_cast<const bf16_t*>(a.dt);
    kp.A = a.A; kp.B = static_cast<const bf16_t*>(a.B); kp.C = static_cast<const bf16_t*>(a.C);
    kp.D = a.D; kp.ids = a.ids; kp.y = static_cast<bf16_t*>(a.y); kp.state_out = a.state_out;
    kp.err = a.err;
    kp.L = (int)sh.L; kp.H = (int)sh.H; kp.G = (int)sh.G; kp.R = (int)sh.R;
    kp.hpg = (int)(sh.H / sh.G);
    kp.has_D = (sh.flags & SSM_HAS_D) ? 1 : 0;
    kp.softplus = (sh.flags & SSM_DT_SOFTPLUS) ? 1 : 0;
    const bool sp = kp.softplus != 0;
    const int S = (int)sh.S;
    if (sh.P == 64 && sh.N == 128) return launch_ssd_pn<64, 128>(kp, S, sp, stream);
    if (sh.P == 64 && sh.N == 64) return launch_ssd_pn<64, 64>(kp, S, sp, stream);
    if (sh.P == 32 && sh.N == 128) return launch_ssd_pn<32, 128>(kp, S, sp, stream);
    if (sh.P == 32 && sh.N == 64) return launch_ssd_pn<32, 64>(kp, S, sp, stream);
    return SSM_ERR_UNSUPPORTED;
}

}  // namespace ssm
