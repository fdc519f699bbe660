// Backward of the Mamba-2 form (scalar A per head, B/C shared by the heads of
// a group) on MFMA, gfx950: the chunked products of the forward (ssd_fwd.hip)
// differentiated, chunks taken in reverse.
//
// Per (sequence, head) and chunk of Q tokens, with X [Q][P], the upstream
// dY [Q][P], B, C [Q][N], l_t = dt_t A, cum_t the chunk's inclusive prefix of
// l, h_in [P][N] the state entering the chunk (from the recompute), and G
// [P][N] the gradient with respect to the state leaving the chunk (dstate
// for the last chunk), the chunk's part of the loss is
//     sum_t <dY_t, y_t> + <G, h_out>,
//     y_t   = exp(cum_t) h_in C_t + sum_{s<=t} exp(cum_t - cum_s) dt_s (C_t.B_s) X_s + D X_t,
//     h_out = exp(cum_last) h_in + sum_s w_s X_s B_s^T,   w_s = exp(cum_last - cum_s) dt_s.
// With S = C B^T, R = dY X^T, E[t][s] = exp(cum_t - cum_s) (s <= t, else 0),
// M = E o S dt_s and Lm = E o R dt_s:
//     dX   = M^T dY + diag(w) B G^T + D dY
//     dC   = diag(exp(cum)) dY h_in + Lm B          (summed over the group's heads)
//     dB   = Lm^T C + diag(w) X G                   (summed over the group's heads)
//     dh_in = exp(cum_last) G + dY^T diag(exp(cum)) C   (G of the chunk before)
// and the gradient with respect to cum_t (Z = E o S o R dt_s, u_s = <G, X_s B_s^T>,
// o_t = exp(cum_t) <dY_t, h_in C_t>):
//     dcum_t = sum_s Z[t][s] - sum_s Z[s][t] + o_t - w_t u_t
//              (+ exp(cum_last) <G, h_in> + sum_s w_s u_s at the chunk's last token),
// which reaches dt through cum (A times the suffix sum of dcum) besides the
// explicit dt_s factors (sum_t Z[t][s] / dt_s + exp(cum_last - cum_s) u_s),
// and A through cum_t / A = sum_{tau<=t} dt_tau.  This is the reverse-time
// adjoint of "kizzasi-model backprop_ssm.rs" (ssm_backward) with the
// per-element terms of "mambazip mamba1/model.rs"
// (accumulate_token_step_gradients), gathered chunk-wise; it reaches the
// sequential result up to rounding.
//
// Work split.  One workgroup (8 waves) runs one (sequence, head) through its
// chunks from the last.  G^T [N][P] is held in fp32 MFMA accumulators by the
// waves that own a 16-channel block and half of the states (as the forward
// holds h^T).  G is staged in LDS as a bf16 value plus a bf16 remainder, so
// that the products that read it keep about 16 significant bits of the
// carried gradient, and so are the fp32 checkpoint of h_in (the decay
// gradient multiplies its errors by A), Lm (dB and dC sum it over the
// group's heads, whose terms can cancel) and M (dX sums it over the chunk's
// later tokens; its remainder takes Lm's remainder tile once dB and dC are
// formed, so dX comes after them); with them the chunk's x, dy, B and C
// rows, the next (earlier) chunk's rows being loaded meanwhile.  All products run on v_mfma_f32_16x16x32_bf16: operands
// whose k index runs along a stored row come from 16-byte LDS row reads, the
// others from the transposing read ds_read_b64_tr_b16 (as in the forward).
// dB and dC, which every head of a group adds to, are written per (sequence,
// head) as partial sums and added over the group's heads in head order by a
// second kernel, as are dA, dD (over sequences) and dh_0 (by ids): every
// sum has a fixed order, so results repeat bitwise.
//
// Round split (relay.h).  The workgroup needs most of a compute unit's LDS,
// so one runs per unit, and S*H jobs a little above the unit count take two
// rounds.  Then every job is cut into k pieces of whole chunks, numbered
// piece-major, the later chunks first: a piece starts from the carried
// gradient G and the running dA and dD sums the piece before it (later in
// time) hands on through the workspace, so every value keeps the order of
// the unsplit grid and results are bitwise the same.
#include "device_common.h"
#include "relay.h"
#include "ssm_internal.h"

#include <algorithm>

namespace ssm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int kQ = 64;  // tokens per chunk (as the forward's recompute)

// Offset (floats) of tile (token block tb, state block nb, dB / dC) in one
// head's partial sums of a chunk: each tile is 64 lanes x 16 bytes, lane
// l16 + 16 g4 holding token 16 tb + l16, states 16 nb + 4 g4 .. + 3, so that
// a store instruction writes 1 KB of whole cache lines.
template <int N>
__device__ __forceinline__ int bc_piece(int tb, int nb, int which) {
    return (((tb * (N / 16) + nb) * 2 + which) * 64) * 4;
}
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;

struct SsdBwdKP {
    const bf16_t* x;
    const uint16_t* dt_t;  // [S][H][L] bf16 bits of dt, tokens contiguous (the checkpoint pass writes it)
    const float* A;
    const bf16_t* B;
    const bf16_t* C;
    const float* D;
    const int32_t* ids;
    const bf16_t* dy;
    const float* dstate;
    const float* ckpt;   // [S][H][n_chunks] x the state entering each chunk (SsdCkptLayout)
    float* d_x;
    float* d_dt;
    float* bc_part;      // [S][H][n_chunks] x this head's dB and dC of a chunk (bc_piece)
    float* dA_part;      // [S][H]
    float* dD_part;      // [S][H]
    float* ds_part;      // [S][H][P][N]: dL/dh_0
    int L, H, G, R, hpg, n_chunks;
    int has_D;
    // round split (relay_k == 0: off): block b runs piece b / (S H) of job
    // b % (S H), piece 0 holding the last relay_len chunks
    int relay_k, relay_len;
    int* relay_flag;     // [S H]
    float* relay_buf;    // [S H][kRelayVals][kThreads]: G (16), dD, dA
    uint32_t* err;
};

constexpr int kRelayVals = 18;  // values a piece hands on per thread
constexpr int kMinPieceChunks = 8;  // shortest piece of the round split (chunks)

// Workspace of the round split: the hand-over values and a flag per job
// (none when the sequences are too short to cut).
size_t ssd_relay_bytes(int64_t jobs, int64_t n_chunks) {
    if (n_chunks < 2 * kMinPieceChunks) return 0;
    return align_up((size_t)jobs * kRelayVals * kThreads * 4, 256) + align_up((size_t)jobs * 4, 256);
}

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 ld8(const bf16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ bf16x4 ld4(const bf16_t* p) { return *reinterpret_cast<const bf16x4*>(p); }
__device__ __forceinline__ bf16x8 cat(const bf16x4& lo, const bf16x4& hi) {
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ bf16x4 ldtr(const bf16_t* p) {
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
    return __builtin_bit_cast(bf16x4, v);
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_or_zero(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                 ROW_MASK, 0xF, false));
}
// inclusive prefix sum over the 64 lanes of a wave (DPP row shifts, then the
// row totals through row_bcast15/31)
__device__ __forceinline__ float wave_incl_sum(float v) {
    v += dpp_or_zero<0x111, 0xF>(v);
    v += dpp_or_zero<0x112, 0xF>(v);
    v += dpp_or_zero<0x114, 0xF>(v);
    v += dpp_or_zero<0x118, 0xF>(v);
    v += dpp_or_zero<0x142, 0xA>(v);
    v += dpp_or_zero<0x143, 0xC>(v);
    return v;
}
__device__ __forceinline__ float lane63(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
__device__ __forceinline__ float wave_sum(float v) { return lane63(wave_incl_sum(v)); }
__device__ __forceinline__ u32x2 pack4(float a, float b, float c, float d) {
    return u32x2{uint32_t(bf16_rne(a)) | (uint32_t(bf16_rne(b)) << 16),
                 uint32_t(bf16_rne(c)) | (uint32_t(bf16_rne(d)) << 16)};
}

template <int P, int N, bool SOFTPLUS>
__global__ __launch_bounds__(kThreads) void ssd_bwd(SsdBwdKP p) {
    static_assert((P == 32 || P == 64) && (N == 64 || N == 128), "tile shapes");
    constexpr int PB = P / 16, NB = N / 16;
    // LDS pitches as in the forward: 16-byte row reads conflict-free at 8
    // (mod 16) dwords, transposing reads fast except at multiples of 32 dwords
    constexpr int NP = N + 16;                    // B, C rows
    constexpr int NPH = N + 8;                    // h_in, G rows [p][n]
    constexpr int XP = P == 64 ? P + 8 : P + 16;  // x, dy rows
    constexpr int MP = kQ + 8;                    // M, Lm rows [t][s]
    __shared__ __attribute__((aligned(16))) bf16_t X_l[kQ * XP];
    __shared__ __attribute__((aligned(16))) bf16_t Y_l[kQ * XP];    // dy
    __shared__ __attribute__((aligned(16))) bf16_t B_l[kQ * NP];
    __shared__ __attribute__((aligned(16))) bf16_t C_l[kQ * NP];
    __shared__ __attribute__((aligned(16))) bf16_t H_l[P * NPH];    // h_in as bf16 ...
    __shared__ __attribute__((aligned(16))) bf16_t Hr_l[P * NPH];   // ... and its remainder
    __shared__ __attribute__((aligned(16))) bf16_t G_l[P * NPH];    // G as bf16 ...
    __shared__ __attribute__((aligned(16))) bf16_t Gr_l[P * NPH];   // ... and its remainder, G - G_l in bf16
    __shared__ __attribute__((aligned(16))) bf16_t M_l[kQ * MP];
    __shared__ __attribute__((aligned(16))) bf16_t Lm_l[kQ * MP];
    __shared__ __attribute__((aligned(16))) bf16_t Lmr_l[kQ * MP];  // Lm - Lm_l in bf16
    __shared__ __attribute__((aligned(16))) float dt_l[kQ], cum_l[kQ], ecum_l[kQ], w_l[kQ];
    __shared__ __attribute__((aligned(16))) float zrow_l[4][kQ], zcol_l[4][kQ];  // per tile block
    __shared__ __attribute__((aligned(16))) float yoff_l[2][kQ], u_l[2][kQ];
    __shared__ float gh_l[kWaves], dd_l[kWaves];
    __shared__ float elast_l;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int jobs = p.relay_k ? (int)gridDim.x / p.relay_k : (int)gridDim.x;
    const int job = (int)(blockIdx.x % (unsigned)jobs), piece = p.relay_k ? (int)(blockIdx.x / (unsigned)jobs) : -1;
    const int hh = job % p.H, i = job / p.H;
    const int grp = hh / p.hpg;
    const int L = p.L;
    const float Ah = p.A[hh];
    const float Dh = p.has_D ? p.D[hh] : 0.0f;
    const int r = p.ids[i];
    const bool bad = (r < 0) | (r >= p.R);  // the recompute started from NaN: the gradients follow

    // state-carry role: wave w holds G^T tiles [NH*sh, NH*sh + NH) of channel block sp
    constexpr int NH = NB / 2;
    const bool owns = wave < 2 * PB;
    const int sp = owns ? wave >> 1 : 0, sh = wave & 1;
    const int pw = sp * 16;
    f32x4 gacc[NH];
    float dD_acc = 0.0f, dA_acc = 0.0f;
    // chunks [c_lo, c_hi) of this workgroup, taken from the last
    int c_hi = p.n_chunks, c_lo = 0;
    float* relay = piece >= 0 ? p.relay_buf + (int64_t)job * kRelayVals * kThreads + tid : nullptr;
    if (piece >= 0) {
        c_hi = p.n_chunks - piece * p.relay_len;
        c_lo = max(0, c_hi - p.relay_len);
    }
    if (piece > 0) {  // the later piece's carried gradient and running sums
        relay_wait(p.relay_flag + job, piece, p.err);
        if (piece + 1 == p.relay_k) relay_reset(p.relay_flag + job);
#pragma unroll
        for (int j = 0; j < NH; ++j)
            gacc[j] = f32x4{relay[(4 * j) * kThreads], relay[(4 * j + 1) * kThreads],
                            relay[(4 * j + 2) * kThreads], relay[(4 * j + 3) * kThreads]};
        dD_acc = relay[16 * kThreads];
        dA_acc = relay[17 * kThreads];
    } else {
        const float* g0 = p.dstate + (((int64_t)i * p.H + hh) * P + pw + l16) * N + NH * sh * 16;
#pragma unroll
        for (int j = 0; j < NH; ++j) {
            const float4 v = *reinterpret_cast<const float4*>(g0 + j * 16 + 4 * g4);
            gacc[j] = f32x4{v.x, v.y, v.z, v.w};
        }
    }

    // per-chunk descriptors: rows past the sequence end read as zero / drop stores
    const int64_t xrow = (int64_t)p.H * P * 2, brow = (int64_t)p.G * N * 2;
    const int64_t xrow4 = (int64_t)p.H * P * 4, drow4 = (int64_t)p.H * 4;
    const char* xg = reinterpret_cast<const char*>(p.x) + ((int64_t)i * L * p.H + hh) * P * 2;
    const char* yg = reinterpret_cast<const char*>(p.dy) + ((int64_t)i * L * p.H + hh) * P * 2;
    const char* bg = reinterpret_cast<const char*>(p.B) + ((int64_t)i * L * p.G + grp) * N * 2;
    const char* cg = reinterpret_cast<const char*>(p.C) + ((int64_t)i * L * p.G + grp) * N * 2;
    const char* dg = reinterpret_cast<const char*>(p.dt_t) + ((int64_t)i * p.H + hh) * L * 2;
    char* dxg = reinterpret_cast<char*>(p.d_x) + ((int64_t)i * L * p.H + hh) * P * 4;
    char* ddg = reinterpret_cast<char*>(p.d_dt) + ((int64_t)i * L * p.H + hh) * 4;
    const float* ckg = p.ckpt + ((int64_t)i * p.H + hh) * p.n_chunks * (P * N);
    auto rsrc = [&](const char* base, int t0, int64_t row) {
        // t0 < 0 (before the first chunk) gives an empty range
        const int rows = t0 < 0 ? 0 : L - t0;
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base) + (t0 < 0 ? 0 : (int64_t)t0 * row), 0,
                                                 rows > 0 ? (int)(rows * row) : 0, 0x00020000);
    };

    // staging of a chunk: x, dy, B, C rows and the checkpoint, by 16-byte pieces
    constexpr int XCH = kQ * P / 8, BCH = kQ * N / 8, HCH = P * N / 4;  // HCH: 16-byte pieces of fp32
    constexpr int XPER = (XCH + kThreads - 1) / kThreads, BPER = BCH / kThreads;
    constexpr int HPER = (HCH + kThreads - 1) / kThreads;
    static_assert(BPER >= 1 && BCH % kThreads == 0, "staging covers the chunk");
    u32x4 sx[XPER], sy[XPER], sb[BPER], sc[BPER], sk[HPER];
    uint32_t sdt = 0;
    auto load_chunk = [&](int c) {
        const int t0 = c * kQ;  // c = -1: nothing to load
        const auto rx = rsrc(xg, c < 0 ? -1 : t0, xrow), ry = rsrc(yg, c < 0 ? -1 : t0, xrow);
        const auto rb = rsrc(bg, c < 0 ? -1 : t0, brow), rc = rsrc(cg, c < 0 ? -1 : t0, brow);
        const auto rk = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(ckg) + (c < 0 ? 0 : (int64_t)c * (P * N)), 0, c < 0 ? 0 : P * N * 4, 0x00020000);
#pragma unroll
        for (int k = 0; k < XPER; ++k) {
            const int e = tid + kThreads * k;
            if (e < XCH) {
                const int off = (int)((e / (P / 8)) * xrow) + (e % (P / 8)) * 16;
                sx[k] = __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0);
                sy[k] = __builtin_amdgcn_raw_buffer_load_b128(ry, off, 0, 0);
            }
        }
#pragma unroll
        for (int k = 0; k < BPER; ++k) {
            const int e = tid + kThreads * k;
            const int t = e / (N / 8), part = e % (N / 8);
            sb[k] = __builtin_amdgcn_raw_buffer_load_b128(rb, (int)(t * brow) + part * 16, 0, 0);
            sc[k] = __builtin_amdgcn_raw_buffer_load_b128(rc, (int)(t * brow) + part * 16, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < HPER; ++k)
            if (tid + kThreads * k < HCH) sk[k] = __builtin_amdgcn_raw_buffer_load_b128(rk, (tid + kThreads * k) * 16, 0, 0);
        if (tid < kQ) sdt = __builtin_amdgcn_raw_buffer_load_b16(rsrc(dg, c < 0 ? -1 : t0, 2), tid * 2, 0, 0);
    };
    float dt_raw = 0.0f, sdt_pre = 0.0f;  // wave 0, lane = token
    auto store_chunk = [&](int t0) {
#pragma unroll
        for (int k = 0; k < XPER; ++k) {
            const int e = tid + kThreads * k;
            if (e < XCH) {
                *reinterpret_cast<u32x4*>(&X_l[(e / (P / 8)) * XP + (e % (P / 8)) * 8]) = sx[k];
                *reinterpret_cast<u32x4*>(&Y_l[(e / (P / 8)) * XP + (e % (P / 8)) * 8]) = sy[k];
            }
        }
#pragma unroll
        for (int k = 0; k < BPER; ++k) {
            const int e = tid + kThreads * k;
            const int t = e / (N / 8), part = e % (N / 8);
            *reinterpret_cast<u32x4*>(&B_l[t * NP + part * 8]) = sb[k];
            *reinterpret_cast<u32x4*>(&C_l[t * NP + part * 8]) = sc[k];
        }
#pragma unroll
        for (int k = 0; k < HPER; ++k) {
            const int e = tid + kThreads * k;  // 16-byte piece e (4 states) of the fp32 checkpoint
            if (e < HCH) {
                int pp, n0;
                SsdCkptLayout<P, N>::pn(e, pp, n0);
                float v[4], rem[4];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    v[rr] = __uint_as_float(sk[k][rr]);
                    rem[rr] = v[rr] - to_f32(bf16_rne(v[rr]));
                }
                const int off = pp * NPH + n0;
                *reinterpret_cast<u32x2*>(&H_l[off]) = pack4(v[0], v[1], v[2], v[3]);
                *reinterpret_cast<u32x2*>(&Hr_l[off]) = pack4(rem[0], rem[1], rem[2], rem[3]);
            }
        }
        if (wave == 0) {  // decays of the chunk, lane = token
            dt_raw = to_f32((bf16_t)sdt);
            float d = dt_raw;
            if constexpr (SOFTPLUS) d = softplus(d);
            if (t0 + lane >= L) d = 0.0f;
            const float cum = wave_incl_sum(d * Ah);
            sdt_pre = wave_incl_sum(d);
            const float last = lane63(cum);
            dt_l[lane] = d;
            cum_l[lane] = cum;
            ecum_l[lane] = __expf(cum);
            w_l[lane] = __expf(last - cum) * d;
            if (lane == 0) elast_l = __expf(last);
        }
        if (owns) {  // G of this chunk [p][n], as a bf16 pair (about 16 significant bits)
#pragma unroll
            for (int j = 0; j < NH; ++j) {
                float rem[4];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) rem[rr] = gacc[j][rr] - to_f32(bf16_rne(gacc[j][rr]));
                const int off = (pw + l16) * NPH + (NH * sh + j) * 16 + 4 * g4;
                *reinterpret_cast<u32x2*>(&G_l[off]) = pack4(gacc[j][0], gacc[j][1], gacc[j][2], gacc[j][3]);
                *reinterpret_cast<u32x2*>(&Gr_l[off]) = pack4(rem[0], rem[1], rem[2], rem[3]);
            }
        }
    };

    // operand fetches for v_mfma_f32_16x16x32_bf16 (lane l16 + 16 g4 gives row /
    // column l16 of the 16-wide block and k = k0 + 8 g4 .. + 7; the result's
    // element r of the lane is D[4 g4 + r][l16]):
    //   rowop: the 16-wide block runs down the rows of buf, k along a row;
    //   colop: the block runs along a row of buf, k down the rows (transposing read).
    auto rowop = [&](const bf16_t* buf, int pitch, int r0, int k0) -> bf16x8 {
        return ld8(&buf[(r0 + l16) * pitch + k0 + 8 * g4]);
    };
    auto colop = [&](const bf16_t* buf, int pitch, int c0, int k0) -> bf16x8 {
        const bf16_t* q = &buf[(k0 + 8 * g4 + (l16 >> 2)) * pitch + c0 + 4 * (l16 & 3)];
        return cat(ldtr(q), ldtr(q + 4 * pitch));
    };

    // zero once: M and Lm above the diagonal, and the Z partial sums of the
    // tile blocks above it, are never written
    for (int e = tid; e < kQ * MP / 2; e += kThreads) {
        reinterpret_cast<uint32_t*>(M_l)[e] = 0u;
        reinterpret_cast<uint32_t*>(Lm_l)[e] = 0u;
        reinterpret_cast<uint32_t*>(Lmr_l)[e] = 0u;
    }
    for (int e = tid; e < 4 * kQ; e += kThreads) {
        (&zrow_l[0][0])[e] = 0.0f;
        (&zcol_l[0][0])[e] = 0.0f;
    }

    load_chunk(c_hi - 1);
    for (int ch = c_hi - 1; ch >= c_lo; --ch) {
        const int t0 = ch * kQ;
        __syncthreads();  // every wave is done with the later chunk's tiles and partial sums
        store_chunk(t0);
        __syncthreads();

        // (1) the causal 16x16 tiles of S^T = B C^T and R^T = X dY^T: M, Lm and
        // the sums of Z.  Tile k (row by row: (tb,sb) = (0,0),(1,0),(1,1),...)
        // goes to wave k % 8.  M's remainder waits in registers until (3) is
        // done with Lmr's tile, which then takes it for (2).
        u32x2 mrem[2];
        int mr_off[2];
        const bool mr_two = wave + kWaves < 10;
        {
            const bool two = mr_two;
            int mtb[2], msb[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int k = wave + kWaves * u;
                mtb[u] = k < 1 ? 0 : k < 3 ? 1 : k < 6 ? 2 : 3;
                msb[u] = k - mtb[u] * (mtb[u] + 1) / 2;
                if (!two) { mtb[1] = mtb[0]; msb[1] = msb[0]; }
            }
            f32x4 sacc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
            f32x4 racc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                if (u == 1 && !two) continue;
#pragma unroll
                for (int kk = 0; kk < N / 32; ++kk)
                    sacc[u] = mfma(rowop(B_l, NP, msb[u] * 16, kk * 32), rowop(C_l, NP, mtb[u] * 16, kk * 32), sacc[u]);
#pragma unroll
                for (int kk = 0; kk < P / 32; ++kk)
                    racc[u] = mfma(rowop(X_l, XP, msb[u] * 16, kk * 32), rowop(Y_l, XP, mtb[u] * 16, kk * 32), racc[u]);
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                if (u == 1 && !two) continue;
                // lane: t = 16 mtb + l16, s = 16 msb + 4 g4 + rr
                const int t = mtb[u] * 16 + l16;
                const float ct = cum_l[t];
                float m[4], lm[4], zs = 0.0f, zp[4];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int s = msb[u] * 16 + 4 * g4 + rr;
                    const float e = s <= t ? __expf(fminf(ct - cum_l[s], 0.0f)) : 0.0f;
                    const float ds = dt_l[s];
                    m[rr] = e * ds * sacc[u][rr];
                    lm[rr] = e * ds * racc[u][rr];
                    zp[rr] = e * sacc[u][rr] * racc[u][rr];
                    zs = fmaf(ds, zp[rr], zs);
                }
                *reinterpret_cast<u32x2*>(&M_l[t * MP + msb[u] * 16 + 4 * g4]) = pack4(m[0], m[1], m[2], m[3]);
                *reinterpret_cast<u32x2*>(&Lm_l[t * MP + msb[u] * 16 + 4 * g4]) = pack4(lm[0], lm[1], lm[2], lm[3]);
                float lr[4], mr[4];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    lr[rr] = lm[rr] - to_f32(bf16_rne(lm[rr]));
                    mr[rr] = m[rr] - to_f32(bf16_rne(m[rr]));
                }
                *reinterpret_cast<u32x2*>(&Lmr_l[t * MP + msb[u] * 16 + 4 * g4]) = pack4(lr[0], lr[1], lr[2], lr[3]);
                mrem[u] = pack4(mr[0], mr[1], mr[2], mr[3]);
                mr_off[u] = t * MP + msb[u] * 16 + 4 * g4;
                // row sum of Z for token t over this tile's s (the four lane groups)
                zs += __shfl_xor(zs, 16);
                zs += __shfl_xor(zs, 32);
                if (g4 == 0) zrow_l[msb[u]][t] = zs;
                // column sums of Z' (Z without dt_s) for each s over this tile's t
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    float v = zp[rr];
                    v += __shfl_xor(v, 1);
                    v += __shfl_xor(v, 2);
                    v += __shfl_xor(v, 4);
                    v += __shfl_xor(v, 8);
                    zp[rr] = v;
                }
                if (l16 == 0)
                    *reinterpret_cast<float4*>(&zcol_l[mtb[u]][msb[u] * 16 + 4 * g4]) =
                        make_float4(zp[0], zp[1], zp[2], zp[3]);
            }
        }
        // <G, h_in> over this wave's part of G
        if (owns) {
            float gh = 0.0f;
#pragma unroll
            for (int j = 0; j < NH; ++j)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int off = (pw + l16) * NPH + (NH * sh + j) * 16 + 4 * g4 + rr;
                    const float hv = (float)*reinterpret_cast<const __bf16*>(&H_l[off]) +
                                     (float)*reinterpret_cast<const __bf16*>(&Hr_l[off]);
                    gh = fmaf(gacc[j][rr], hv, gh);
                }
            gh = wave_sum(gh);
            if (lane == 0) gh_l[wave] = gh;
        } else if (lane == 0) {
            gh_l[wave] = 0.0f;
        }
        __syncthreads();

        // (3) dC [t][n] = exp(cum_t) (dY h_in) + Lm B, and dB [s][n] = Lm^T C + w_s (X G),
        // for token block wave % 4 and this wave's half of the states; the
        // dcum terms o_t and u_s on the way.  The products are formed
        // transposed ([n][t]: operands swapped), so that a lane holds four
        // consecutive states n = 16 nb + 4 g4 .. + 3 of one token t = 16 tb + l16
        // and stores them as one 16-byte piece of the token's row.
        {
            constexpr int NPW = NB / 2;
            const int tb = wave & 3, nb0 = (wave >> 2) * NPW, half = wave >> 2;
            const int t = tb * 16 + l16;  // also s for the dB part (the same block)
            float yo = 0.0f, uu = 0.0f;
            // this head's partial sums of the chunk, 16-byte piece of this lane
            // in each (token block, state block, dB / dC) tile (chunks are
            // whole: no store needs a guard)
            float* bcc = p.bc_part + (((int64_t)i * p.H + hh) * p.n_chunks + t0 / kQ) * (kQ * 2 * N) + 4 * lane;
            const float et = ecum_l[t], ws = w_l[t];
            // the dy and x rows of the token block, shared by every state block
            bf16x8 yo8[P / 32], xo[P / 32];
#pragma unroll
            for (int kk = 0; kk < P / 32; ++kk) {
                yo8[kk] = rowop(Y_l, XP, tb * 16, kk * 32);
                xo[kk] = rowop(X_l, XP, tb * 16, kk * 32);
            }
            // not unrolled: the stores of one state block then leave before the
            // next block's products, which keeps the register count under the cap
#pragma unroll 1
            for (int j = 0; j < NPW; ++j) {
                const int nb = nb0 + j, n0 = nb * 16 + 4 * g4;
                f32x4 c1 = {0.f, 0.f, 0.f, 0.f}, c2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < P / 32; ++kk) {
                    c1 = mfma(colop(H_l, NPH, nb * 16, kk * 32), yo8[kk], c1);
                    c1 = mfma(colop(Hr_l, NPH, nb * 16, kk * 32), yo8[kk], c1);
                }
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    if (2 * kk > tb) continue;  // every s of the block is after t
                    c2 = mfma(colop(B_l, NP, nb * 16, kk * 32), rowop(Lm_l, MP, tb * 16, kk * 32), c2);
                    c2 = mfma(colop(B_l, NP, nb * 16, kk * 32), rowop(Lmr_l, MP, tb * 16, kk * 32), c2);
                }
                const bf16x4 cn = ld4(&C_l[t * NP + n0]);
                float dc[4];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const float off = et * c1[rr];
                    yo = fmaf(off, (float)cn[rr], yo);
                    dc[rr] = off + c2[rr];
                }
                *reinterpret_cast<float4*>(bcc + bc_piece<N>(tb, nb, 1)) = make_float4(dc[0], dc[1], dc[2], dc[3]);

                f32x4 b1 = {0.f, 0.f, 0.f, 0.f}, b2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    if (2 * kk + 1 < tb) continue;  // every t of the block is before s
                    b1 = mfma(colop(C_l, NP, nb * 16, kk * 32), colop(Lm_l, MP, tb * 16, kk * 32), b1);
                    b1 = mfma(colop(C_l, NP, nb * 16, kk * 32), colop(Lmr_l, MP, tb * 16, kk * 32), b1);
                }
#pragma unroll
                for (int kk = 0; kk < P / 32; ++kk) {
                    b2 = mfma(colop(G_l, NPH, nb * 16, kk * 32), xo[kk], b2);
                    b2 = mfma(colop(Gr_l, NPH, nb * 16, kk * 32), xo[kk], b2);
                }
                const bf16x4 bn = ld4(&B_l[t * NP + n0]);
                float db[4];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    uu = fmaf(b2[rr], (float)bn[rr], uu);
                    db[rr] = fmaf(ws, b2[rr], b1[rr]);
                }
                *reinterpret_cast<float4*>(bcc + bc_piece<N>(tb, nb, 0)) = make_float4(db[0], db[1], db[2], db[3]);
            }
            // sums over this wave's states: the lane's own, then its four lane groups
            yo += __shfl_xor(yo, 16);
            yo += __shfl_xor(yo, 32);
            uu += __shfl_xor(uu, 16);
            uu += __shfl_xor(uu, 32);
            if (g4 == 0) {
                yoff_l[half][t] = yo;
                u_l[half][t] = uu;
            }
        }

        // the earlier chunk's loads: issued here, they fly through the
        // remainder hand-over, (2) and (4); before (3) their registers would
        // not fit beside its products
        load_chunk(ch - 1);

        // M's remainder into Lmr's tile, once every wave is done with Lm
        __syncthreads();
        *reinterpret_cast<u32x2*>(&Lmr_l[mr_off[0]]) = mrem[0];
        if (mr_two) *reinterpret_cast<u32x2*>(&Lmr_l[mr_off[1]]) = mrem[1];
        __syncthreads();

        // (2) dX^T [p][s] = dY^T M (t >= s) + w_s (G B^T) + D dY, for s-block
        // wave % 4 and this wave's channel blocks
        {
            constexpr int YPW = PB / 2;
            const int sb = wave & 3, pb0 = (wave >> 2) * YPW;
            const int s = sb * 16 + l16;
            const float ws = w_l[s];
            const auto rdx = rsrc(dxg, t0, xrow4);
#pragma unroll
            for (int q = 0; q < YPW; ++q) {
                const int pb = pb0 + q;
                f32x4 a1 = {0.f, 0.f, 0.f, 0.f}, a2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    if (2 * kk + 1 < sb) continue;  // every t of the block is before s
                    a1 = mfma(colop(Y_l, XP, pb * 16, kk * 32), colop(M_l, MP, sb * 16, kk * 32), a1);
                    a1 = mfma(colop(Y_l, XP, pb * 16, kk * 32), colop(Lmr_l, MP, sb * 16, kk * 32), a1);
                }
#pragma unroll
                for (int kk = 0; kk < N / 32; ++kk) {
                    const bf16x8 bo = rowop(B_l, NP, sb * 16, kk * 32);
                    a2 = mfma(rowop(G_l, NPH, pb * 16, kk * 32), bo, a2);
                    a2 = mfma(rowop(Gr_l, NPH, pb * 16, kk * 32), bo, a2);
                }
                // lane: p = 16 pb + 4 g4 + rr, s
                const bf16x4 yv = ld4(&Y_l[s * XP + pb * 16 + 4 * g4]);
                const bf16x4 xv = ld4(&X_l[s * XP + pb * 16 + 4 * g4]);
                float dx[4];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    dx[rr] = fmaf(ws, a2[rr], fmaf(Dh, (float)yv[rr], a1[rr]));
                    if (bad) dx[rr] = __builtin_nanf("");
                    dD_acc = fmaf((float)yv[rr], (float)xv[rr], dD_acc);
                }
                __builtin_amdgcn_raw_buffer_store_b128(
                    u32x4{__float_as_uint(dx[0]), __float_as_uint(dx[1]), __float_as_uint(dx[2]), __float_as_uint(dx[3])},
                    rdx, (int)(s * xrow4) + (pb * 16 + 4 * g4) * 4, 0, 0);
            }
        }


        // (4) the carry: G^T [n][p] = exp(cum_last) G^T + C^T diag(exp(cum)) dY
        if (owns) {
            const float el = elast_l;
            // dy exp(cum) as a bf16 pair, so that the carry keeps about 16 bits
            bf16x8 ye[2], yr[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const bf16x8 yv = colop(Y_l, XP, pw, kk * 32);
                const float4 e0 = *reinterpret_cast<const float4*>(&ecum_l[kk * 32 + 8 * g4]);
                const float4 e1 = *reinterpret_cast<const float4*>(&ecum_l[kk * 32 + 8 * g4 + 4]);
                const float ev[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) {
                    const float v = (float)yv[jj] * ev[jj];
                    ye[kk][jj] = (__bf16)v;
                    yr[kk][jj] = (__bf16)(v - (float)ye[kk][jj]);
                }
            }
#pragma unroll
            for (int j = 0; j < NH; ++j) {
                const int nb = NH * sh + j;
                f32x4 a = gacc[j] * el;
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const bf16x8 co = colop(C_l, NP, nb * 16, kk * 32);
                    a = mfma(co, ye[kk], a);
                    a = mfma(co, yr[kk], a);
                }
                gacc[j] = a;
            }
        }
        __syncthreads();

        // (5) dcum, d(dt) and dA from the partial sums, lane = token
        if (wave == 0) {
            const int t = lane;
            const float zr = zrow_l[0][t] + zrow_l[1][t] + zrow_l[2][t] + zrow_l[3][t];
            const float zc = zcol_l[0][t] + zcol_l[1][t] + zcol_l[2][t] + zcol_l[3][t];
            const float yo = yoff_l[0][t] + yoff_l[1][t];
            const float uu = u_l[0][t] + u_l[1][t];
            const float d = dt_l[t], w = w_l[t];
            float dcum = zr - d * zc + yo - w * uu;
            float gh = 0.0f;
#pragma unroll
            for (int k = 0; k < kWaves; ++k) gh += gh_l[k];
            const float wu = wave_sum(w * uu);
            if (t == kQ - 1) dcum += elast_l * gh + wu;
            // suffix sum over t' >= t
            const float pre = wave_incl_sum(dcum);
            const float suf = lane63(pre) - pre + dcum;
            const float wp = __expf(cum_l[kQ - 1] - cum_l[t]);
            float ddt = fmaf(Ah, suf, fmaf(wp, uu, zc));
            if constexpr (SOFTPLUS) ddt *= sigmoid(dt_raw);
            if (bad) ddt = __builtin_nanf("");
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ddt), rsrc(ddg, t0, drow4), (int)(t * drow4), 0, 0);
            dA_acc += wave_sum(dcum * sdt_pre);
        }
    }

    if (piece >= 0 && piece + 1 < p.relay_k) {  // hand on to the earlier piece
#pragma unroll
        for (int j = 0; j < NH; ++j)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) relay_put(&relay[(4 * j + rr) * kThreads], gacc[j][rr]);
        relay_put(&relay[16 * kThreads], dD_acc);
        relay_put(&relay[17 * kThreads], dA_acc);
        relay_publish_puts(p.relay_flag + job, piece + 1);
        return;
    }
    // dD, dA and dh_0 of this (sequence, head)
    {
        const float v = wave_sum(dD_acc);
        if (lane == 0) dd_l[wave] = v;
        __syncthreads();
        if (tid == 0) {
            float s = 0.0f;
#pragma unroll
            for (int k = 0; k < kWaves; ++k) s += dd_l[k];
            p.dD_part[(int64_t)i * p.H + hh] = s;
            p.dA_part[(int64_t)i * p.H + hh] = dA_acc;
        }
    }
    if (owns) {
        float* dso = p.ds_part + (((int64_t)i * p.H + hh) * P + pw + l16) * N + NH * sh * 16;
#pragma unroll
        for (int j = 0; j < NH; ++j)
            *reinterpret_cast<float4*>(dso + j * 16 + 4 * g4) = make_float4(gacc[j][0], gacc[j][1], gacc[j][2], gacc[j][3]);
    }
}

// d_A[h] and d_D[h]: the per-sequence partials summed in sequence order;
// d_s[row]: the dh_0 of every sequence whose id is row, in sequence order
// (rows no id names are zero; sequences with a bad id add nothing).
__global__ __launch_bounds__(256) void ssd_bwd_reduce(const float* __restrict__ dA_part,
                                                      const float* __restrict__ dD_part,
                                                      const float* __restrict__ ds_part,
                                                      const int32_t* __restrict__ ids, float* d_A, float* d_D,
                                                      float* d_s, int S, int H, int R, int64_t per_row,
                                                      int has_D) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e < H) {
        float a = 0.0f, dd = 0.0f;
        for (int i = 0; i < S; ++i) {
            a += dA_part[(int64_t)i * H + e];
            dd += dD_part[(int64_t)i * H + e];
        }
        d_A[e] = a;
        if (has_D) d_D[e] = dd;
    }
    const int64_t total = (int64_t)R * per_row;
    for (int64_t k = e; k < total; k += (int64_t)gridDim.x * 256) {
        const int row = (int)(k / per_row);
        const int64_t off = k - (int64_t)row * per_row;
        float v = 0.0f;
        for (int i = 0; i < S; ++i)
            if (ids[i] == row) v += ds_part[(int64_t)i * per_row + off];
        d_s[k] = v;
    }
}

// d_B, d_C [S][L][G][N]: the partial sums of the group's heads in head order.
// A thread takes one 16-byte piece of a chunk's partials (as stored: lane
// l16 + 16 g4 of tile (tb, nb, which) holds token 16 tb + l16, states
// 16 nb + 4 g4 .. + 3), so that the reads of a wave are contiguous.  Each
// partial is read once: the loads stream past the caches (C8's reduction
// 270 -> 230 us).
__global__ __launch_bounds__(256) void ssd_bwd_reduce_bc(const float* __restrict__ part, float* d_B,
                                                         float* d_C, int S, int L, int n_chunks, int H, int G,
                                                         int N) {
    const int hpg = H / G, NB = N / 16;
    const int per_chunk = kQ * 2 * N / 4;  // pieces of one head's chunk
    const int64_t total = (int64_t)S * G * n_chunks * per_chunk;
    const int64_t head_stride = (int64_t)n_chunks * per_chunk;
    const f32x4* part4 = reinterpret_cast<const f32x4*>(part);
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
        const int within = (int)(e % per_chunk);
        int64_t r = e / per_chunk;
        const int chunk = (int)(r % n_chunks);
        r /= n_chunks;
        const int g = (int)(r % G);
        const int64_t i = r / G;
        const int lane = within & 63, tile = within >> 6;
        const int which = tile & 1, nb = (tile >> 1) % NB, tb = (tile >> 1) / NB;
        const int t = chunk * kQ + tb * 16 + (lane & 15);
        if (t >= L) continue;  // the padding of the last chunk
        const f32x4* src = part4 + ((i * H + (int64_t)g * hpg) * n_chunks + chunk) * per_chunk + within;
        float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
        for (int h = 0; h < hpg; ++h) {
            const f32x4 v = __builtin_nontemporal_load(src + (int64_t)h * head_stride);
            a0 += v[0];
            a1 += v[1];
            a2 += v[2];
            a3 += v[3];
        }
        float* dst = (which ? d_C : d_B) + ((i * L + t) * G + g) * N + nb * 16 + 4 * (lane >> 4);
        dst[0] = a0;
        dst[1] = a1;
        dst[2] = a2;
        dst[3] = a3;
    }
}

template <int P, int N>
void launch_ssd_bwd_pn(SsdBwdKP kp, int S, bool softplus, hipStream_t st) {
    const int64_t jobs = (int64_t)kp.H * S;
    if (kp.relay_buf) {  // the round split, when it shortens the grid
        const int n_cu = device_cus();
        const int cap = n_cu > 0 ? resident_blocks(softplus ? (const void*)ssd_bwd<P, N, true>
                                                            : (const void*)ssd_bwd<P, N, false>, kThreads)
                                 : 0;
        const RoundSplit rs = cap > 0 ? round_split(jobs, kp.n_chunks, (int64_t)n_cu * cap, kMinPieceChunks)
                                      : RoundSplit{};
        if (rs.k > 1) {
            kp.relay_k = rs.k;
            kp.relay_len = rs.len;
        }
    }
    const dim3 grid((unsigned)(jobs * (kp.relay_k ? kp.relay_k : 1)));
    if (softplus) hipLaunchKernelGGL((ssd_bwd<P, N, true>), grid, dim3(kThreads), 0, st, kp);
    else hipLaunchKernelGGL((ssd_bwd<P, N, false>), grid, dim3(kThreads), 0, st, kp);
}

}  // namespace

bool ssd_bwd_supported(const Shape& sh) {
    const int64_t lim = int64_t(1) << 31;
    return !sh.a_per_state && sh.io == SSM_BF16 && sh.K == 0 && (sh.P == 64 || sh.P == 32) &&
           (sh.N == 128 || sh.N == 64) && sh.L > 0 && sh.S * sh.H < lim &&
           sh.L * sh.H * sh.P * 4 < lim && sh.L * sh.G * sh.N * 2 < lim;
}

size_t ssd_bwd_workspace_bytes(const Shape& sh) {
    const int64_t n_chunks = (sh.L + kQ - 1) / kQ;
    return align_up((size_t)(sh.S * sh.H * n_chunks * sh.P * sh.N) * 4, 256) +
           align_up((size_t)(sh.S * sh.H * sh.P * sh.N) * 4, 256) + 2 * align_up((size_t)(sh.S * sh.H) * 4, 256) +
           align_up((size_t)(sh.S * sh.H * n_chunks * kQ * 2 * sh.N) * 4, 256) +
           align_up((size_t)(sh.S * sh.H * sh.L) * 2, 256) + ssd_relay_bytes(sh.S * sh.H, n_chunks);
}

int launch_ssd_ckpt(const BwdArgs& a, float* ckpt, uint16_t* dt_t, hipStream_t stream);

int launch_ssd_bwd(const BwdArgs& a, hipStream_t stream) {
    const Shape& sh = a.sh;
    auto al16 = [](const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) == 0; };
    if (!al16(a.x) || !al16(a.dy) || !al16(a.B) || !al16(a.C) || !al16(a.dstate) || !al16(a.d_x) ||
        !al16(a.d_s) || !al16(a.s))
        return SSM_ERR_UNSUPPORTED;
    const int64_t n_chunks = (sh.L + kQ - 1) / kQ;
    char* w = a.ws;
    float* ckpt = reinterpret_cast<float*>(w);
    w += align_up((size_t)(sh.S * sh.H * n_chunks * sh.P * sh.N) * 4, 256);
    float* ds_part = reinterpret_cast<float*>(w);
    w += align_up((size_t)(sh.S * sh.H * sh.P * sh.N) * 4, 256);
    float* dA_part = reinterpret_cast<float*>(w);
    w += align_up((size_t)(sh.S * sh.H) * 4, 256);
    float* dD_part = reinterpret_cast<float*>(w);
    w += align_up((size_t)(sh.S * sh.H) * 4, 256);
    float* bc_part = reinterpret_cast<float*>(w);
    w += align_up((size_t)(sh.S * sh.H * n_chunks * kQ * 2 * sh.N) * 4, 256);
    uint16_t* dt_t = reinterpret_cast<uint16_t*>(w);
    w += align_up((size_t)(sh.S * sh.H * sh.L) * 2, 256);
    const size_t relay_bytes = ssd_relay_bytes(sh.S * sh.H, n_chunks);
    float* relay_buf = relay_bytes ? reinterpret_cast<float*>(w) : nullptr;
    int* relay_flag = relay_bytes ? reinterpret_cast<int*>(
                                        w + align_up((size_t)(sh.S * sh.H) * kRelayVals * kThreads * 4, 256))
                                  : nullptr;
    if (ssd_bwd_workspace_bytes(sh) > a.ws_bytes) return SSM_ERR_WORKSPACE;
    int rc = launch_ssd_ckpt(a, ckpt, dt_t, stream);
    if (rc) return rc;
    SsdBwdKP kp;
    kp.x = static_cast<const bf16_t*>(a.x); kp.dt_t = dt_t; kp.A = a.A;
    kp.B = static_cast<const bf16_t*>(a.B); kp.C = static_cast<const bf16_t*>(a.C); kp.D = a.D;
    kp.ids = a.ids; kp.dy = static_cast<const bf16_t*>(a.dy); kp.dstate = a.dstate; kp.ckpt = ckpt;
    kp.d_x = a.d_x; kp.d_dt = a.d_dt; kp.bc_part = bc_part;
    kp.dA_part = dA_part; kp.dD_part = dD_part; kp.ds_part = ds_part;
    kp.L = (int)sh.L; kp.H = (int)sh.H; kp.G = (int)sh.G; kp.R = (int)sh.R;
    kp.hpg = (int)(sh.H / sh.G); kp.n_chunks = (int)n_chunks;
    kp.has_D = a.D ? 1 : 0;
    kp.relay_k = 0; kp.relay_len = 0;
    kp.relay_flag = relay_flag; kp.relay_buf = relay_buf; kp.err = a.err;
    const bool sp = (sh.flags & SSM_DT_SOFTPLUS) != 0;
    const int S = (int)sh.S;
    if (sh.P == 64 && sh.N == 128) launch_ssd_bwd_pn<64, 128>(kp, S, sp, stream);
    else if (sh.P == 64 && sh.N == 64) launch_ssd_bwd_pn<64, 64>(kp, S, sp, stream);
    else if (sh.P == 32 && sh.N == 128) launch_ssd_bwd_pn<32, 128>(kp, S, sp, stream);
    else launch_ssd_bwd_pn<32, 64>(kp, S, sp, stream);
    const int64_t nbc = sh.S * sh.G * n_chunks * (kQ * 2 * sh.N / 4);  // 16-byte pieces of the sums
    hipLaunchKernelGGL(ssd_bwd_reduce_bc, dim3((unsigned)std::min<int64_t>((nbc + 255) / 256, 16384)), dim3(256),
                       0, stream, (const float*)bc_part, a.d_B, a.d_C, (int)sh.S, (int)sh.L, (int)n_chunks,
                       (int)sh.H, (int)sh.G, (int)sh.N);
    const int64_t per_row = sh.H * sh.P * sh.N;
    const int64_t work = std::max<int64_t>(sh.H, sh.R * per_row);
    hipLaunchKernelGGL(ssd_bwd_reduce, dim3((unsigned)std::min<int64_t>((work + 255) / 256, 8192)), dim3(256), 0,
                       stream, dA_part, dD_part, ds_part, a.ids, a.d_A, a.d_D, a.d_s, (int)sh.S, (int)sh.H,
                       (int)sh.R, per_row, a.D ? 1 : 0);
    return hipGetLastError() == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

}  // namespace ssm
