// Selective-scan backward for gfx950: reverse-time adjoint of the Mamba-1
// form with d_state <= 16 and one B/C group (no fused conv); other shapes go
// to the generic kernels of scan_bwd_rows.hip.
//
// Per (sequence i, channel c) the forward step is h_t = a_t h_{t-1} + dt_t B_t u_t,
// a_t = exp(dt_t A_c), y_t = C_t . h_t + D_c u_t.  The adjoint carried from
// the last token to the first is g = dL/dh_t ("kizzasi-model
// backprop_ssm.rs", ssm_backward: dL/dh_t = C^T dy_t + A_bar dL/dh_{t+1}),
// and the per-element terms follow "mambazip mamba1/model.rs"
// (accumulate_token_step_gradients):
//     g      += C_t dy_t                  (now dL/dh_t)
//     dC_t   += dy_t h_t                  (summed over channels)
//     du_t    = D dy_t + dt_t sum_n g_n B_tn
//     ddt_t   = sum_n g_n (h_{t-1,n} a_tn A_n + B_tn u_t)
//     dB_t   += g dt_t u_t                (summed over channels)
//     dA     += g h_{t-1} a_t dt_t        (summed over sequences and tokens)
//     g      *= a_t                       (now dL/dh_{t-1})
// and dD += dy_t u_t, dh_0 = g after the first token, scattered to row ids[i].
//
// Kernel 1 (scan_fwd_quad.hip, quad_ckpt) stores the state entering every
// block of kCkpt (8) tokens.  Kernel 2 (bwd_rev) walks the blocks backwards: it stages
// the block's inputs in LDS, recomputes the block's decays and states from
// the checkpoint into registers, then runs the adjoint over the block.  The
// layout is the forward's quad one: four lanes per channel, four states per
// lane.  Channel sums (dB, dC) are reduced in a fixed order: across the four
// channels of a 16-lane row with DPP shifts, across rows and waves through
// LDS, across channel blocks by kernel 3.  Kernel 3 also sums dA and dD over
// sequences and gathers dh_0 into d_s by ids; every sum has a fixed order,
// so results are bitwise repeatable.
//
// Fused conv (fast path, K = 2..4 taps): x is the conv's input, u = SiLU(c)
// with c = sum_j w_j in(t - (K-1) + j) (in() the gathered conv state before
// token 0).  The checkpoint pass runs the fused forward; bwd_fast recomputes
// c and u per block from the staged x and K-1 history rows, and its owner
// lane turns du into dc = du SiLU'(c), the input gradient
// d in(t) = sum_j w_j dc_{t + K-1-j} (the last K-1 values of dc ride in
// registers from block to block), the weight sums dw_j += dc_t in(t-(K-1)+j)
// and, after the first token, the gradient of the conv-state row.
//
// Relay (fast path): the (sequence, 64-channel block) jobs beyond a whole
// number per compute unit are cut into pieces of whole blocks, run from the
// last piece to the first; each hands on its adjoint g and its running dA and
// dD sums, so every sum keeps the unsplit order (relay.h).
#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "relay.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

constexpr int kThreads = 256;
constexpr int kChan = 64;  // channels per workgroup
constexpr int kBlk = kCkpt;  // tokens per block (checkpoint spacing)

struct BwdKP {
    const float* A;
    const float* D;
    const int32_t* ids;
    const void* x;
    const void* dt;
    const void* B;
    const void* C;
    const void* dy;
    const float* dstate;
    const float* ckpt;   // [n_blk][S][d_inner][16]
    float* d_x;
    float* d_dt;
    float* dbc_part;     // [n_cb][S][L][32]: dB (16) then dC (16)
    float* dA_part;      // [S][d_inner][16]
    float* dD_part;      // [S][d_inner]
    float* ds_part;      // [S][d_inner][16]
    int L, d_inner, N, R, S, n_cb;
    int has_D, softplus;
    // relay (bwd_fast; relay_k == 0: off): blocks [0, relay_full) are whole
    // jobs, then relay_k rounds of relay_rem pieces of relay_len checkpoint
    // blocks, piece 0 being the last in time
    int relay_full, relay_rem, relay_k, relay_len;
    int* relay_flag;     // [relay_rem]
    float* relay_buf;    // [relay_rem][kRelayVals][256]: g (4), dA (4), dD, a dc row, tap sum
    uint32_t* err;       // nullable device-error word
    const float* conv_w;      // [d_inner][K] (bwd_fast with K > 0)
    const float* conv_state;  // [R][d_inner][K-1], nullable: zeros
    float* partW;             // [S][d_inner][K] conv-weight sums per sequence
    float* partCS;            // [S][d_inner][K-1] conv-state gradient per sequence
    int K;
};

constexpr int kRelayVals = 11;  // values a relay piece hands on per lane

constexpr int kRelayMaxJobs = 256;  // cut jobs the workspace has room for

template <int P0, int P1, int P2, int P3>
__device__ __forceinline__ float qperm(float v) {
    constexpr int ctrl = P0 | (P1 << 2) | (P2 << 4) | (P3 << 6);
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), ctrl,
                                                                 0xF, 0xF, true));
}

// Sum over the 4 lanes of each quad (every lane gets the total).
__device__ __forceinline__ float quad_sum(float v) {
    v += qperm<1, 0, 3, 2>(v);
    v += qperm<2, 3, 0, 1>(v);
    return v;
}

// Adds to lane l of each 16-lane row the value of lane l - SHIFT (same row);
// lanes without a source keep their value.
template <int SHIFT>
__device__ __forceinline__ float row_shr_add(float v) {
    constexpr int ctrl = 0x110 + SHIFT;  // DPP row_shr:SHIFT
    const float sh = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, v), ctrl, 0xF, 0xF, true));  // out-of-row sources read 0
    return v + sh;
}

template <typename T>
__device__ __forceinline__ float ldv(const void* base, int64_t idx) {
    return to_f32(static_cast<const T*>(base)[idx]);
}

template <typename T, bool SOFTPLUS>
__global__ __launch_bounds__(kThreads) void bwd_rev(BwdKP p) {
    __shared__ float x_l[kBlk][kChan];
    __shared__ float dt_l[kBlk][kChan];   // dt as given (before softplus)
    __shared__ float dy_l[kBlk][kChan];
    __shared__ __attribute__((aligned(16))) float B_l[kBlk][16];
    __shared__ __attribute__((aligned(16))) float C_l[kBlk][16];
    // [token][wave][row][quad lane][dB 4 | dC 4]: sums over the row's four channels
    __shared__ __attribute__((aligned(16))) float red_l[kBlk][4][4][4][8];

    const int tid = threadIdx.x;
    const int q = tid & 3;
    const int cl = tid >> 2;            // channel within the block
    const int wave = tid >> 6;
    const int row = (tid >> 4) & 3;     // 16-lane row within the wave
    const int lane_in_row = tid & 15;
    const int cb = blockIdx.x, i = blockIdx.y;
    const int c_raw = cb * kChan + cl;
    const bool active = c_raw < p.d_inner;
    const int c = active ? c_raw : p.d_inner - 1;
    const int64_t seq = (int64_t)i * p.L * p.d_inner;
    const int rid = p.ids[i];
    const bool bad = (rid < 0) | (rid >= p.R);  // unknown initial state: d_x, d_dt are NaN

    float a2[4], An[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int n = 4 * q + s;
        An[s] = n < p.N ? p.A[(int64_t)c * p.N + n] : 0.0f;
        a2[s] = An[s] * kLog2e;
    }
    const float Dc = p.has_D ? p.D[c] : 0.0f;
    float g[4], dA_acc[4] = {0.f, 0.f, 0.f, 0.f};
    float dD_acc = 0.0f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int n = 4 * q + s;
        g[s] = n < p.N ? p.dstate[((int64_t)i * p.d_inner + c) * p.N + n] : 0.0f;
    }

    const int n_blk = (p.L + kBlk - 1) / kBlk;
    for (int b = n_blk - 1; b >= 0; --b) {
        const int t0 = b * kBlk;
        const int nk = min(kBlk, p.L - t0);
        // stage the block's inputs (zeros past the end of the sequence)
        for (int e = tid; e < kBlk * kChan; e += kThreads) {
            const int k = e / kChan, ch = e % kChan;
            const int cc = cb * kChan + ch;
            const bool ok = (k < nk) && (cc < p.d_inner);
            const int64_t idx = seq + (int64_t)(t0 + k) * p.d_inner + cc;
            x_l[k][ch] = ok ? ldv<T>(p.x, idx) : 0.0f;
            dt_l[k][ch] = ok ? ldv<T>(p.dt, idx) : 0.0f;
            dy_l[k][ch] = ok ? ldv<T>(p.dy, idx) : 0.0f;
        }
        for (int e = tid; e < kBlk * 16; e += kThreads) {
            const int k = e / 16, n = e % 16;
            const bool ok = (k < nk) && (n < p.N);
            const int64_t idx = ((int64_t)i * p.L + t0 + k) * p.N + n;
            B_l[k][n] = ok ? ldv<T>(p.B, idx) : 0.0f;
            C_l[k][n] = ok ? ldv<T>(p.C, idx) : 0.0f;
        }
        float h0[4];
        {
            const float4 ck = *reinterpret_cast<const float4*>(
                p.ckpt + (((int64_t)b * p.S + i) * p.d_inner + c) * 16 + 4 * q);
            h0[0] = ck.x; h0[1] = ck.y; h0[2] = ck.z; h0[3] = ck.w;
        }
        __syncthreads();

        // recompute the block: decays a[k][s] and states h[k][s] (= h_{t0+k})
        float a[kBlk][4], h[kBlk][4];
#pragma unroll
        for (int k = 0; k < kBlk; ++k) {
            float dk = dt_l[k][cl];
            if constexpr (SOFTPLUS) dk = k < nk ? softplus(dk) : 0.0f;
            const float bk = dk * x_l[k][cl];
            const float4 Bv = *reinterpret_cast<const float4*>(&B_l[k][4 * q]);
            const float Bs[4] = {Bv.x, Bv.y, Bv.z, Bv.w};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                a[k][s] = fast_exp2(dk * a2[s]);
                h[k][s] = fmaf(a[k][s], k == 0 ? h0[s] : h[k - 1][s], bk * Bs[s]);
            }
        }

        // adjoint over the block, last token first
#pragma unroll
        for (int k = kBlk - 1; k >= 0; --k) {
            const float dyk = dy_l[k][cl];
            const float draw = dt_l[k][cl];
            const float dk = SOFTPLUS ? (k < nk ? softplus(draw) : 0.0f) : draw;
            const float uk = x_l[k][cl];
            const float dtuk = dk * uk;
            const float4 Bv = *reinterpret_cast<const float4*>(&B_l[k][4 * q]);
            const float4 Cv = *reinterpret_cast<const float4*>(&C_l[k][4 * q]);
            const float Bs[4] = {Bv.x, Bv.y, Bv.z, Bv.w};
            const float Cs[4] = {Cv.x, Cv.y, Cv.z, Cv.w};
            float S1 = 0.0f, S2 = 0.0f, dBp[4], dCp[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                g[s] = fmaf(Cs[s], dyk, g[s]);
                dCp[s] = dyk * h[k][s];
                S1 = fmaf(g[s], Bs[s], S1);
                const float ga = g[s] * a[k][s];
                const float qv = ga * (k == 0 ? h0[s] : h[k - 1][s]);
                S2 = fmaf(qv, An[s], S2);
                dA_acc[s] = fmaf(qv, dk, dA_acc[s]);
                dBp[s] = g[s] * dtuk;
                g[s] = ga;
            }
            S1 = quad_sum(S1);
            S2 = quad_sum(S2);
            if (q == 0 && active && k < nk) {
                const int64_t idx = seq + (int64_t)(t0 + k) * p.d_inner + c;
                float ddt = fmaf(uk, S1, S2);
                if constexpr (SOFTPLUS) ddt *= sigmoid(draw);
                p.d_x[idx] = bad ? __builtin_nanf("") : fmaf(Dc, dyk, dk * S1);
                p.d_dt[idx] = bad ? __builtin_nanf("") : ddt;
                dD_acc = fmaf(dyk, uk, dD_acc);
            }
            // sum the four channels of this 16-lane row (lanes 4j + q)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                float vb = active ? dBp[s] : 0.0f, vc = active ? dCp[s] : 0.0f;
                vb = row_shr_add<4>(vb);
                vb = row_shr_add<8>(vb);
                vc = row_shr_add<4>(vc);
                vc = row_shr_add<8>(vc);
                dBp[s] = vb;
                dCp[s] = vc;
            }
            if (lane_in_row >= 12) {
                float* dst = &red_l[k][wave][row][q][0];
                *reinterpret_cast<float4*>(dst) = make_float4(dBp[0], dBp[1], dBp[2], dBp[3]);
                *reinterpret_cast<float4*>(dst + 4) = make_float4(dCp[0], dCp[1], dCp[2], dCp[3]);
            }
        }
        __syncthreads();
        // the block's channel sums: kBlk tokens x (16 dB + 16 dC), 16 terms each, fixed order
        for (int e = tid; e < kBlk * 32; e += kThreads) {
            const int k = e / 32, m = e % 32;
            if (k >= nk) continue;
            const int which = m >> 4, n = m & 15, qq = n >> 2, s = n & 3;
            float acc = 0.0f;
#pragma unroll
            for (int w = 0; w < 4; ++w)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc += red_l[k][w][r][qq][which * 4 + s];
            p.dbc_part[(((int64_t)cb * p.S + i) * p.L + t0 + k) * 32 + m] = acc;
        }
        __syncthreads();
    }
    if (active) {
        const int64_t row_i = ((int64_t)i * p.d_inner + c) * 16 + 4 * q;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            p.ds_part[row_i + s] = g[s];
            p.dA_part[row_i + s] = dA_acc[s];
        }
    }
    // dD: lane q == 0 of each quad holds its channel's sum
    if (active && q == 0) p.dD_part[(int64_t)i * p.d_inner + c] = dD_acc;
}

// Fast path for d_state 16, 64 | d_inner and 16-byte aligned tensors.  Same
// arithmetic and reduction order as bwd_rev.
//  - The next block's x, dt, dy, B, C and checkpoint are loaded into
//    registers while the current block runs and written to the other half of
//    a double-buffered LDS tile at its end, already as fp32 (rows past the
//    sequence end as zeros): global-memory latency hides behind a block of
//    work, and no LDS read in the block is followed by an unpack.
//  - d_x and d_dt of the block are gathered in an LDS tile and leave as
//    16-byte row stores once the block is done, after the loads of the tile
//    after next (loads and stores share one completion counter, so the wait
//    for those loads at the end of the next block never waits for these
//    stores).
//  - The products summed across channels (dB, dC) are formed without
//    contraction so that each DPP row step is a single add.
template <typename T, int K, bool SOFTPLUS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void bwd_fast(const BwdKP kp_arg) {
    static_assert(K == 0 || (K >= 2 && K <= 4), "conv taps");
    // lambdas below capture locals only (capturing the kernel argument would
    // force it into scratch memory)
    const BwdKP p = kp_arg;
    constexpr int ES = (int)sizeof(T);
    constexpr int CPR = kChan * ES / 16;        // 16-byte chunks per 64-channel row
    constexpr int CHX = kBlk * CPR;             // chunks per x / dt / dy tile
    constexpr int CPB = 16 * ES / 16;           // chunks per B / C row
    constexpr int CHB = kBlk * CPB;             // chunks per B / C tile
    constexpr int CHK = kChan * 16 * 4 / 16;    // chunks of the checkpoint tile (f32)
    constexpr int VPC = 16 / ES;                // values per chunk
    // x rows: with the conv the lanes of a quad read different rows of one
    // channel, so the row pitch is 8 (mod 32) words to keep them in separate banks
    constexpr int XP = K > 0 ? kChan + 8 : kChan;
    __shared__ __attribute__((aligned(16))) float xs_l[2][kBlk * XP];
    __shared__ __attribute__((aligned(16))) float dts_l[2][kBlk * kChan];
    __shared__ __attribute__((aligned(16))) float dys_l[2][kBlk * kChan];
    // the conv's history: x of tokens t0-3 .. t0-1 (conv state before token 0)
    constexpr int HX = 3;
    __shared__ __attribute__((aligned(16))) float hx_l[2][K > 0 ? HX * XP : 4];
    // u = SiLU(c) and SiLU'(c) of the block's tokens [token][channel]; each
    // wave writes and reads only its own channels
    // (row pitch 4 (mod 16) words: the quad lanes write rows 2q, 2q+1)
    constexpr int UP = kChan + 4;
    __shared__ __attribute__((aligned(16))) float us_l[K > 0 ? kBlk * UP : 4];
    __shared__ __attribute__((aligned(16))) float fs_l[K > 0 ? kBlk * UP : 4];
    // dc = du SiLU'(c) of the block's tokens, double-buffered: the block after
    // (in time) keeps its first rows for the d_x of this block's last tokens
    __shared__ __attribute__((aligned(16))) float dc_l[2][K > 0 ? kBlk * kChan : 4];
    __shared__ __attribute__((aligned(16))) float wl[K > 0 ? kChan * 4 : 4];  // conv taps [tap][channel]
    __shared__ __attribute__((aligned(16))) float Bs_l[2][kBlk * 16];
    __shared__ __attribute__((aligned(16))) float Cs_l[2][kBlk * 16];
    // the checkpoint is read into registers right after the barrier that
    // publishes it, so one buffer is enough (the next one is written after
    // the following barrier)
    __shared__ __attribute__((aligned(16))) float ck_l[kChan * 16];
    // [token][wave][row][quad lane][dB 4 | dC 4]: sums over the row's four channels
    __shared__ __attribute__((aligned(16))) float red_l[kBlk][4][4][4][8];
    // d_x and d_dt of the block, [token][channel]
    __shared__ __attribute__((aligned(16))) float gx_l[kBlk * kChan];
    __shared__ __attribute__((aligned(16))) float gdt_l[kBlk * kChan];
    // where quad lanes 2 and 3 put their copies of the per-channel terms (K == 0)
    __shared__ __attribute__((aligned(16))) float spare_l[K == 0 ? kBlk * kChan : 4];

    const int tid = threadIdx.x;
    const int q = tid & 3;
    const int cl = tid >> 2;            // channel within the block
    const int wave = tid >> 6;
    const int row = (tid >> 4) & 3;     // 16-lane row within the wave
    const int lane_in_row = tid & 15;
    int cb = blockIdx.x, i = blockIdx.y;
    const int n_blk = (p.L + kBlk - 1) / kBlk;
    int b_lo = 0, b_hi = n_blk;  // checkpoint blocks [b_lo, b_hi) of this workgroup
    RelayBlock rb{0, -1, 0};
    if (p.relay_k) {  // 1-D grid
        rb = relay_block(blockIdx.x, p.relay_full, p.relay_rem);
        cb = rb.job % p.n_cb;
        i = rb.job / p.n_cb;
        if (rb.piece >= 0) {
            // the adjoint runs backwards in time: piece 0 takes the last blocks
            __builtin_amdgcn_s_setprio(2);  // a piece chain goes first (relay.h)
            b_hi = n_blk - rb.piece * p.relay_len;
            b_lo = max(0, b_hi - p.relay_len);
        }
    }
    const int c = cb * kChan + cl;
    const int L = p.L, d_inner = p.d_inner;
    const int64_t seq = (int64_t)i * L * d_inner;
    const int rid = p.ids[i];
    const bool bad = (rid < 0) | (rid >= p.R);  // unknown initial state: d_x, d_dt are NaN

    float a2[4], An[4];
    {
        const float4 Av = *reinterpret_cast<const float4*>(p.A + (int64_t)c * 16 + 4 * q);
        An[0] = Av.x; An[1] = Av.y; An[2] = Av.z; An[3] = Av.w;
#pragma unroll
        for (int s = 0; s < 4; ++s) a2[s] = An[s] * kLog2e;
    }
    const float Dc = p.has_D ? p.D[c] : 0.0f;
    float g[4], dA_acc[4] = {0.f, 0.f, 0.f, 0.f};
    float dD_acc = 0.0f;
    // conv: quad lane q's running weight sum for tap q; the dc rows that the
    // first block in time after this workgroup's range hands in (lanes q < 3)
    float dwq = 0.0f, dc_in = 0.0f;
    if constexpr (K > 0) wl[q * kChan + cl] = q < K ? p.conv_w[(int64_t)c * K + q] : 0.0f;
    float* relay = rb.piece >= 0 ? p.relay_buf + (int64_t)rb.cut * kRelayVals * kThreads + tid : nullptr;
    if (rb.piece > 0) {  // the later piece's adjoint and running sums
        relay_wait(p.relay_flag + rb.cut, rb.piece, p.err);
        if (rb.piece + 1 == p.relay_k) relay_reset(p.relay_flag + rb.cut);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            g[s] = relay[s * kThreads];
            dA_acc[s] = relay[(4 + s) * kThreads];
        }
        dD_acc = relay[8 * kThreads];
        if constexpr (K > 0) {
            dc_in = relay[9 * kThreads];
            dwq = relay[10 * kThreads];
        }
    } else {
        const float4 gv = *reinterpret_cast<const float4*>(p.dstate + ((int64_t)i * d_inner + c) * 16 + 4 * q);
        g[0] = gv.x; g[1] = gv.y; g[2] = gv.z; g[3] = gv.w;
    }

    // staging: the chunks of x, dt, dy (rows of this block's 64 channels), B,
    // C (rows of 16 states) and the checkpoint (64 channels x 16 states)
    const char* xg = static_cast<const char*>(p.x) + (seq + (int64_t)cb * kChan) * ES;
    const char* dg = static_cast<const char*>(p.dt) + (seq + (int64_t)cb * kChan) * ES;
    const char* yg = static_cast<const char*>(p.dy) + (seq + (int64_t)cb * kChan) * ES;
    const char* bg = static_cast<const char*>(p.B) + (int64_t)i * L * 16 * ES;
    const char* cg = static_cast<const char*>(p.C) + (int64_t)i * L * 16 * ES;
    const int64_t xrow = (int64_t)d_inner * ES;
    const float* ckpt = p.ckpt;
    const int S = p.S;
    float* d_x = p.d_x + seq + (int64_t)cb * kChan;
    float* d_dt = p.d_dt + seq + (int64_t)cb * kChan;
    // Slots: each thread stages at most NS 16-byte chunks per tile, every slot
    // drawn from arrays split at wave or 16-lane boundaries (so the choice of
    // array is a select, not a lookup).  fp32: x (threads 0-127) or dt
    // (128-255); dy (0-127) or B (128-159) or C (160-191); checkpoint.  bf16:
    // x (wave 0) or dt (wave 1) or dy (wave 2) or B (192-207) or C (208-223);
    // checkpoint.
    // With the conv, 3 history rows of x (array 6): bf16 threads 224-247 of
    // slot 0, fp32 threads 192-239 of slot 1.
    constexpr int NS = ES == 4 ? 3 : 2;
    constexpr int CHH = HX * CPR;               // chunks of the history rows
    static_assert(kBlk == 8 && CHK == kThreads &&
                  (ES == 2 ? CHX == 64 && CHB == 16 && 224 + CHH <= kThreads
                           : CHX == 128 && CHB == 32 && 192 + CHH <= kThreads), "slot layout");
    uint4 stg[NS];
    // where slot k of this thread comes from: array id (0 x, 1 dt, 2 dy, 3 B, 4 C, 5 ckpt, 6 history) and chunk
    auto slot = [&](int k, int& arr, int& w) __attribute__((always_inline)) {
        if constexpr (ES == 4) {
            if (k == 0) { arr = tid < 128 ? 0 : 1; w = tid & 127; }
            else if (k == 1) {
                arr = tid < 128 ? 2 : tid < 160 ? 3 : tid < 192 ? 4 : 6;
                w = tid < 128 ? tid : tid < 192 ? (tid - 128) & 31 : tid - 192;
            } else { arr = 5; w = tid; }
        } else {
            if (k == 0) {
                arr = tid < 192 ? (tid >> 6) : tid < 208 ? 3 : tid < 224 ? 4 : 6;
                w = tid < 192 ? (tid & 63) : tid < 224 ? (tid & 15) : tid - 224;
            } else { arr = 5; w = tid; }
        }
    };
    auto slot_used = [&](int k) __attribute__((always_inline)) {
        if constexpr (ES == 2) return !(k == 0 && tid >= (K > 0 ? 224 + CHH : 224));
        else return !(k == 1 && tid >= (K > 0 ? 192 + CHH : 192));
    };
    auto load_tile = [&](int b) __attribute__((always_inline)) {
        const int bb = b < 0 ? 0 : b;
        const int t0 = bb * kBlk;
        const char* ckb = reinterpret_cast<const char*>(ckpt + (((int64_t)bb * S + i) * d_inner + cb * kChan) * 16);
#pragma unroll
        for (int k = 0; k < NS; ++k) {
            if (!slot_used(k)) continue;
            int arr, w;
            slot(k, arr, w);
            const char* src;
            if (arr < 3) {
                const int t = min(t0 + w / CPR, L - 1);
                const char* base = arr == 0 ? xg : (arr == 1 ? dg : yg);
                src = base + (int64_t)t * xrow + (w % CPR) * 16;
            } else if (arr < 5) {
                const int t = min(t0 + w / CPB, L - 1);
                src = (arr == 3 ? bg : cg) + (int64_t)t * 16 * ES + (w % CPB) * 16;
            } else if (arr == 5) {
                src = ckb + w * 16;
            } else {  // history row: tokens before 0 come from the conv state instead
                const int t = min(max(t0 - HX + w / CPR, 0), L - 1);
                src = xg + (int64_t)t * xrow + (w % CPR) * 16;
            }
            stg[k] = *reinterpret_cast<const uint4*>(src);
        }
    };
    // a staged chunk of io values into an fp32 tile (zeros for rows past the end)
    auto put = [&](float* dst, const uint4& v, bool ok) __attribute__((always_inline)) {
        if constexpr (ES == 2) {
            const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
            float f[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                f[2 * e] = ok ? __uint_as_float(wv[e] << 16) : 0.0f;
                f[2 * e + 1] = ok ? __uint_as_float(wv[e] & 0xffff0000u) : 0.0f;
            }
            *reinterpret_cast<float4*>(dst) = make_float4(f[0], f[1], f[2], f[3]);
            *reinterpret_cast<float4*>(dst + 4) = make_float4(f[4], f[5], f[6], f[7]);
        } else {
            *reinterpret_cast<uint4*>(dst) = ok ? v : make_uint4(0, 0, 0, 0);
        }
    };
    auto store_tile = [&](int buf, int b) __attribute__((always_inline)) {
        const int t0 = b * kBlk;
#pragma unroll
        for (int k = 0; k < NS; ++k) {
            if (!slot_used(k)) continue;
            int arr, w;
            slot(k, arr, w);
            if (arr < 3) {
                float* tile = arr == 0 ? xs_l[buf] + (w / CPR) * (XP - kChan) : (arr == 1 ? dts_l[buf] : dys_l[buf]);
                put(tile + w * VPC, stg[k], t0 + w / CPR < L);
            } else if (arr < 5) {
                put((arr == 3 ? Bs_l[buf] : Cs_l[buf]) + w * VPC, stg[k], t0 + w / CPB < L);
            } else if (arr == 5) {
                *reinterpret_cast<uint4*>(ck_l + w * 4) = stg[k];
            } else if constexpr (K > 0) {
                if (t0 - HX + w / CPR >= 0) put(hx_l[buf] + (w / CPR) * XP + (w % CPR) * VPC, stg[k], true);
            }
        }
        if constexpr (K > 0) {
            if (t0 < HX && tid < HX * kChan) {  // the first block: history from the gathered conv state
                const int hr = tid / kChan, ch = tid % kChan, tau = t0 - HX + hr;
                if (tau < 0) {
                    float v = 0.0f;
                    if (tau >= -(K - 1))
                        v = bad ? __builtin_nanf("")
                                : (p.conv_state ? p.conv_state[((int64_t)rid * d_inner + cb * kChan + ch) * (K - 1) +
                                                               tau + K - 1]
                                                : 0.0f);
                    hx_l[buf][hr * XP + ch] = v;
                }
            }
        }
    };
    auto rowv = [&](const float* tile, int k) __attribute__((always_inline)) { return tile[k * kChan + cl]; };
    auto quad4 = [&](const float* tile, int k, float (&v)[4]) __attribute__((always_inline)) {
        const float4 w = *reinterpret_cast<const float4*>(tile + k * 16 + 4 * q);
        v[0] = w.x; v[1] = w.y; v[2] = w.z; v[3] = w.w;
    };

    load_tile(b_hi - 1);
    store_tile((b_hi - 1) & 1, b_hi - 1);
    load_tile(b_hi - 2);
    if constexpr (K > 0)  // dc of the tokens after the range: zero past the end, else handed in
        if (q < K - 1) dc_l[b_hi & 1][q * kChan + cl] = dc_in;
    __syncthreads();
    for (int b = b_hi - 1; b >= b_lo; --b) {
        const int t0 = b * kBlk, buf = b & 1;
        const int nk = min(kBlk, L - t0);
        const float* xs = xs_l[buf];
        const float* dts = dts_l[buf];
        const float* dys = dys_l[buf];
        const float* Bt = Bs_l[buf];
        const float* Ct = Cs_l[buf];
        float h0[4];
        {
            const float4 ck = *reinterpret_cast<const float4*>(&ck_l[cl * 16 + 4 * q]);
            h0[0] = ck.x; h0[1] = ck.y; h0[2] = ck.z; h0[3] = ck.w;
        }
        auto dt_of = [&](int k) __attribute__((always_inline)) {
            float dk = rowv(dts, k);
            if constexpr (SOFTPLUS) dk = k < nk ? softplus(dk) : 0.0f;
            return dk;
        };
        // input row kk of the block for this lane's channel (kk < 0: history)
        auto xin = [&](int kk) __attribute__((always_inline)) {
            return kk >= 0 ? xs[kk * XP + cl] : hx_l[buf][(HX + kk) * XP + cl];
        };
        if constexpr (K > 0) {
            // quad lane q forms c = sum_j w_j in(t-(K-1)+j) (the forward's order,
            // oldest input first), u = SiLU(c) and SiLU'(c) of tokens 2q, 2q+1;
            // LDS operations of a wave complete in order, so its lanes read
            // them back below without a barrier
            float win[K + 1];
#pragma unroll
            for (int j = 0; j <= K; ++j) win[j] = xin(2 * q - (K - 1) + j);
            const float w[4] = {wl[cl], wl[kChan + cl], wl[2 * kChan + cl], wl[3 * kChan + cl]};
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                float cv = w[0] * win[e];
#pragma unroll
                for (int j = 1; j < K; ++j) cv = fmaf(w[j], win[e + j], cv);
                const float sg = __builtin_amdgcn_rcpf(1.0f + fast_exp2(-cv * kLog2e));
                us_l[(2 * q + e) * UP + cl] = cv * sg;
                fs_l[(2 * q + e) * UP + cl] = sg * fmaf(cv, 1.0f - sg, 1.0f);
            }
            __builtin_amdgcn_wave_barrier();
        }
        auto u_of = [&](int k) __attribute__((always_inline)) {
            if constexpr (K > 0) return us_l[k * UP + cl];
            else return rowv(xs, k);
        };
        // recompute the block: decays a[k][s] and states h[k][s] (= h_{t0+k});
        // with the conv (more live values) the adjoint forms the decays again
        // instead of holding them
        constexpr bool KEEP_A = K == 0;
        float a[KEEP_A ? kBlk : 1][4], h[kBlk][4];
#pragma unroll
        for (int k = 0; k < kBlk; ++k) {
            const float dk = dt_of(k), bk = dk * u_of(k);
            float Bq[4];
            quad4(Bt, k, Bq);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const float ak = fast_exp2(dk * a2[s]);
                if constexpr (KEEP_A) a[k][s] = ak;
                h[k][s] = fmaf(ak, k == 0 ? h0[s] : h[k - 1][s], bk * Bq[s]);
            }
        }
        // adjoint over the block, last token first
        float* const own_row = (q == 0 ? gx_l : q == 1 ? gdt_l : spare_l) + cl;  // K == 0
#pragma unroll
        for (int k = kBlk - 1; k >= 0; --k) {
            // no contraction here: a product summed across lanes would otherwise be
            // fused into the DPP add and formed twice
#pragma clang fp contract(off)
            const float dyk = rowv(dys, k);
            const float draw = rowv(dts, k);
            const float dk = SOFTPLUS ? (k < nk ? softplus(draw) : 0.0f) : draw;
            const float uk = u_of(k);
            const float dtuk = dk * uk;
            float Bq[4], Cq[4];
            quad4(Bt, k, Bq);
            quad4(Ct, k, Cq);
            float S1 = 0.0f, S2 = 0.0f, dBp[4], dCp[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                g[s] = fmaf(Cq[s], dyk, g[s]);
                dCp[s] = dyk * h[k][s];
                S1 = fmaf(g[s], Bq[s], S1);
                const float ga = g[s] * (KEEP_A ? a[KEEP_A ? k : 0][s] : fast_exp2(dk * a2[s]));
                const float qv = ga * (k == 0 ? h0[s] : h[k - 1][s]);
                S2 = fmaf(qv, An[s], S2);
                dA_acc[s] = fmaf(qv, dk, dA_acc[s]);
                dBp[s] = g[s] * dtuk;
                g[s] = ga;
            }
            S1 = quad_sum(S1);
            S2 = quad_sum(S2);
            if constexpr (K == 0) {
                // every lane of the quad forms its channel's terms (no branch):
                // lane 0 stores du, lane 1 ddt, lanes 2 and 3 a copy of lane
                // 0's value to a spare row
                float ddt = fmaf(uk, S1, S2);
                if constexpr (SOFTPLUS) ddt *= sigmoid(draw);
                const float du = fmaf(Dc, dyk, dk * S1);
                own_row[k * kChan] = q == 1 ? ddt : du;
                if (k < nk) dD_acc = fmaf(dyk, uk, dD_acc);
            } else if (q == 0) {  // (the conv variants have no registers to spare)
                float ddt = fmaf(uk, S1, S2);
                if constexpr (SOFTPLUS) ddt *= sigmoid(draw);
                const float du = fmaf(Dc, dyk, dk * S1);
                dc_l[buf][k * kChan + cl] = du * fs_l[k * UP + cl];  // through SiLU
                gdt_l[k * kChan + cl] = ddt;
                if (k < nk) dD_acc = fmaf(dyk, uk, dD_acc);
            }
            // sum the four channels of this 16-lane row (lanes 4j + q); the empty asm
            // keeps the last add ahead of the branch below, where it stays fused
            // with its DPP move
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                dBp[s] = row_shr_add<8>(row_shr_add<4>(dBp[s]));
                dCp[s] = row_shr_add<8>(row_shr_add<4>(dCp[s]));
                asm volatile("" : "+v"(dBp[s]), "+v"(dCp[s]));
            }
            if (lane_in_row >= 12) {
                float* dst = &red_l[k][wave][row][q][0];
                *reinterpret_cast<float4*>(dst) = make_float4(dBp[0], dBp[1], dBp[2], dBp[3]);
                *reinterpret_cast<float4*>(dst + 4) = make_float4(dCp[0], dCp[1], dCp[2], dCp[3]);
            }
        }
        __syncthreads();
        // the block's channel sums: kBlk tokens x (16 dB + 16 dC), 16 terms each, fixed order
        constexpr int NBC = kBlk * 32 / kThreads;  // channel sums per thread
        float bc[NBC];
#pragma unroll
        for (int u = 0; u < NBC; ++u) {
            const int e = tid + kThreads * u;
            const int k = e / 32, m = e % 32;
            const int which = m >> 4, n = m & 15, qq = n >> 2, s = n & 3;
            float acc = 0.0f;
#pragma unroll
            for (int w = 0; w < 4; ++w)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc += red_l[k][w][r][qq][which * 4 + s];
            bc[u] = acc;
        }
        // the block's d_x / d_dt rows: thread -> token tid / 16, channels 4 (tid % 16) + 0..3
        constexpr int NGX = kBlk * kChan / 4;  // 16-byte pieces of the d_x tile
        const int tg = tid < NGX ? tid : 0;
        float4 gxv;
        if constexpr (K > 0) {
            // through the conv: d in(t) = sum_m w_{K-1-m} dc_{t+m}, rows past the
            // block from the later one's buffer
            const int k = tg >> 4, ch = 4 * (tg & 15);
            float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
            for (int m = 0; m < K; ++m) {
                const int rr = k + m;
                const float4 d = *reinterpret_cast<const float4*>(
                    rr < kBlk ? &dc_l[buf][rr * kChan + ch] : &dc_l[buf ^ 1][(rr - kBlk) * kChan + ch]);
                const float dv[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] = fmaf(wl[(K - 1 - m) * kChan + ch + e], dv[e], acc[e]);
            }
            gxv = make_float4(acc[0], acc[1], acc[2], acc[3]);
            // tap q's weight sum: dc_t in(t - (K-1) + q), tokens in reverse order
            if (q < K) {
#pragma unroll 1
                for (int kk = kBlk - 1; kk >= 0; --kk)
                    dwq = fmaf(dc_l[buf][kk * kChan + cl], xin(kk - (K - 1) + q), dwq);
            }
        } else {
            gxv = *reinterpret_cast<const float4*>(&gx_l[tg * 4]);
        }
        float4 gdv = *reinterpret_cast<const float4*>(&gdt_l[tg * 4]);
        // next block's tiles into the other buffer; fetch the one after
        if (b > b_lo) store_tile(buf ^ 1, b - 1);
        load_tile(b - 2);
#pragma unroll
        for (int u = 0; u < NBC; ++u) {
            const int e = tid + kThreads * u;
            const int k = e / 32, m = e % 32;
            if (k < nk) p.dbc_part[(((int64_t)cb * p.S + i) * L + t0 + k) * 32 + m] = bc[u];
        }
        {
            const int k = tid >> 4;
            if (bad) {
                const float nan = __builtin_nanf("");
                gxv = make_float4(nan, nan, nan, nan);
                gdv = gxv;
            }
            if (tid < NGX && k < nk) {
                const int64_t off = (int64_t)(t0 + k) * d_inner + 4 * (tid & 15);
                *reinterpret_cast<float4*>(d_x + off) = gxv;
                *reinterpret_cast<float4*>(d_dt + off) = gdv;
            }
        }
        __syncthreads();
    }
    if (rb.piece >= 0 && rb.piece + 1 < p.relay_k) {  // hand on to the earlier piece
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            relay_put(&relay[s * kThreads], g[s]);
            relay_put(&relay[(4 + s) * kThreads], dA_acc[s]);
        }
        relay_put(&relay[8 * kThreads], dD_acc);
        if constexpr (K > 0) {
            // the first rows of dc of this range, for the d_x of the range before
            relay_put(&relay[9 * kThreads], q < K - 1 ? dc_l[b_lo & 1][q * kChan + cl] : 0.0f);
            relay_put(&relay[10 * kThreads], dwq);
        }
        relay_publish_puts(p.relay_flag + rb.cut, rb.piece + 1);
        return;
    }
    {
        const int64_t row_i = ((int64_t)i * d_inner + c) * 16 + 4 * q;
        *reinterpret_cast<float4*>(p.ds_part + row_i) = make_float4(g[0], g[1], g[2], g[3]);
        *reinterpret_cast<float4*>(p.dA_part + row_i) = make_float4(dA_acc[0], dA_acc[1], dA_acc[2], dA_acc[3]);
    }
    // dD and the conv-state gradient: lane q == 0 of each quad holds its
    // channel's; the weight sum of tap q: quad lane q
    const int64_t rowc = (int64_t)i * d_inner + c;
    if constexpr (K > 0)
        if (q < K) p.partW[rowc * K + q] = dwq;
    if (q == 0) {
        p.dD_part[rowc] = dD_acc;
        if constexpr (K > 0) {
            // the conv-state inputs tau = m - (K-1): sum_j w_j dc_{m-j} (dc of
            // tokens 0 .. K-2, block 0's buffer)
#pragma unroll
            for (int m = 0; m < K - 1; ++m) {
                float gcs = 0.0f;
#pragma unroll
                for (int j = 0; j <= m; ++j) gcs = fmaf(wl[j * kChan + cl], dc_l[0][(m - j) * kChan + cl], gcs);
                p.partCS[rowc * (K - 1) + m] = gcs;
            }
        }
    }
}

// d_B, d_C: sum of the channel-block partials in block order.
__global__ __launch_bounds__(256) void bwd_reduce_bc(BwdKP p, float* d_B, float* d_C) {
    // a thread sums one 16-byte piece (4 states of dB or of dC) of a token
    // over the channel blocks, in block order; the partials are read once
    using v4 = float __attribute__((ext_vector_type(4)));
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t tokens = (int64_t)p.S * p.L;
    if (e >= tokens * 8) return;
    const int64_t tok = e >> 3;
    const int m0 = 4 * (int)(e & 7), n0 = m0 & 15;
    if (n0 >= p.N) return;
    const v4* src = reinterpret_cast<const v4*>(p.dbc_part + tok * 32 + m0);
    const int64_t cb_stride = tokens * 8;  // 16-byte pieces between channel blocks
    v4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    int cb = 0;
    for (; cb + 8 <= p.n_cb; cb += 8) {
        v4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(src + (cb + u) * cb_stride);
#pragma unroll
        for (int u = 0; u < 8; ++u) acc += v[u];
    }
    for (; cb < p.n_cb; ++cb) acc += __builtin_nontemporal_load(src + cb * cb_stride);
    float* dst = (m0 < 16 ? d_B : d_C) + tok * p.N;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        if (n0 + j < p.N) dst[n0 + j] = acc[j];
}

// d_A, d_D: sums over sequences in sequence order; d_s: dh_0 of every
// sequence whose id is this row, in sequence order (zero if none).
// ds_src rows have stride ds_stride floats (16 for the partials, d_state for
// dstate itself when there are no tokens).
__global__ __launch_bounds__(256) void bwd_reduce_params(BwdKP p, const float* ds_src, int ds_stride,
                                                         float* d_A, float* d_D, float* d_s, float* d_cw,
                                                         float* d_cs) {
    const int64_t per_row = (int64_t)p.d_inner * p.N;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < per_row; e += stride) {
        const int64_t c = e / p.N;
        const int n = (int)(e % p.N);
        float acc = 0.0f;
        if (p.dA_part)
            for (int i = 0; i < p.S; ++i) acc += p.dA_part[((int64_t)i * p.d_inner + c) * 16 + n];
        d_A[e] = acc;
        if (d_D && n == 0) {
            float dd = 0.0f;
            if (p.dD_part)
                for (int i = 0; i < p.S; ++i) dd += p.dD_part[(int64_t)i * p.d_inner + c];
            d_D[c] = dd;
        }
    }
    const int64_t ds_total = (int64_t)p.R * per_row;
    for (int64_t f = (int64_t)blockIdx.x * 256 + threadIdx.x; f < ds_total; f += stride) {
        const int64_t r = f / per_row, rem = f % per_row;
        const int64_t c = rem / p.N;
        const int n = (int)(rem % p.N);
        float acc = 0.0f;
        for (int i = 0; i < p.S; ++i)
            if (p.ids[i] == r) acc += ds_src[((int64_t)i * p.d_inner + c) * ds_stride + n];
        d_s[f] = acc;
    }
    if (p.K > 0 && d_cw && d_cs) {  // d_conv_w over sequences; d_conv_state rows by ids, in sequence order
        for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < (int64_t)p.d_inner * p.K; e += stride) {
            float acc = 0.0f;
            for (int i = 0; i < p.S; ++i) acc += p.partW[(int64_t)i * p.d_inner * p.K + e];
            d_cw[e] = acc;
        }
        const int64_t per_cs = (int64_t)p.d_inner * (p.K - 1);
        for (int64_t f = (int64_t)blockIdx.x * 256 + threadIdx.x; f < (int64_t)p.R * per_cs; f += stride) {
            const int64_t r = f / per_cs, rem = f % per_cs;
            float acc = 0.0f;
            for (int i = 0; i < p.S; ++i)
                if (p.ids[i] == r) acc += p.partCS[(int64_t)i * per_cs + rem];
            d_cs[f] = acc;
        }
    }
}

size_t blocks_of(const Shape& sh) { return (size_t)((sh.L + kBlk - 1) / kBlk); }

struct BwdWs {
    float *ckpt, *dbc, *dA, *dD, *ds, *partW, *partCS;
    char* relay;   // the relay of bwd_fast
    size_t relay_bytes;
    size_t total;
};

size_t relay_room(const Shape& sh) {
    const int64_t jobs = sh.S * ((sh.d_inner() + kChan - 1) / kChan);
    return (size_t)(jobs < kRelayMaxJobs ? jobs : kRelayMaxJobs);
}

BwdWs carve(const Shape& sh, char* base) {
    const size_t rows = (size_t)sh.S * sh.d_inner();
    const size_t n_cb = (size_t)((sh.d_inner() + kChan - 1) / kChan);
    size_t off = 0;
    BwdWs w;
    auto take = [&](size_t bytes) { char* ptr = base ? base + off : nullptr; off += align_up(bytes, 256); return reinterpret_cast<float*>(ptr); };
    w.ckpt = take(blocks_of(sh) * rows * 16 * 4);
    w.dbc = take(n_cb * (size_t)sh.S * sh.L * 32 * 4);
    w.dA = take(rows * 16 * 4);
    w.dD = take(rows * 4);
    w.ds = take(rows * 16 * 4);
    w.partW = sh.K > 0 ? take(rows * sh.K * 4) : nullptr;
    w.partCS = sh.K > 0 ? take(rows * (sh.K - 1) * 4) : nullptr;
    const size_t room = relay_room(sh);
    w.relay_bytes = align_up(room * kRelayVals * kThreads * 4, 256) + align_up(room * 4, 256);
    w.relay = reinterpret_cast<char*>(take(w.relay_bytes));
    w.total = off;
    return w;
}

}  // namespace

bool bwd_supported(const Shape& sh) {
    return sh.a_per_state && sh.P == 1 && sh.N <= 16 && sh.G == 1 && sh.K == 0;
}

// The fused conv on the fast path: the shape side of its conditions (the
// tensors' alignment decides between it and the generic kernels).
bool bwd_conv_fast_shape(const Shape& sh) {
    return sh.a_per_state && sh.P == 1 && sh.N == 16 && sh.G == 1 && sh.K >= 2 && sh.K <= 4 &&
           sh.d_inner() % kChan == 0;
}

size_t bwd_workspace_bytes(const Shape& sh) {
    if (ssd_bwd_supported(sh)) return ssd_bwd_workspace_bytes(sh);
    if (bwd_supported(sh)) return (sh.S == 0 || sh.L == 0) ? 0 : carve(sh, nullptr).total;
    const size_t rows = rows_bwd_supported(sh) ? rows_bwd_workspace_bytes(sh) : 0;
    if (bwd_conv_fast_shape(sh) && sh.S > 0 && sh.L > 0) {
        const size_t fast = carve(sh, nullptr).total;
        return fast > rows ? fast : rows;
    }
    return rows;
}

template <typename T, int K, bool SOFTPLUS>
int launch_fast(BwdKP kp, const BwdWs& w, const Shape& sh, hipStream_t stream) {
    auto fn = bwd_fast<T, K, SOFTPLUS>;
    const int64_t jobs = (int64_t)kp.n_cb * kp.S;
    const int n_cu = device_cus();
    const int cap = n_cu > 0 ? resident_blocks((const void*)fn, kThreads) : 0;
    const RelaySplit rs = relay_split(jobs, blocks_of(sh), 1, cap, n_cu, (int)relay_room(sh));
    if (rs.k) {
        char* r = w.relay;
        kp.relay_buf = reinterpret_cast<float*>(r);
        kp.relay_flag = reinterpret_cast<int*>(r + align_up(relay_room(sh) * kRelayVals * kThreads * 4, 256));
        kp.relay_full = rs.full;
        kp.relay_rem = rs.rem;
        kp.relay_k = rs.k;
        kp.relay_len = rs.len;
        hipLaunchKernelGGL(fn, dim3((unsigned)(rs.full + rs.rem * rs.k)), dim3(kThreads), 0, stream, kp);
    } else {
        hipLaunchKernelGGL(fn, dim3((unsigned)kp.n_cb, (unsigned)kp.S), dim3(kThreads), 0, stream, kp);
    }
    return hipGetLastError() == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

template <int K>
int launch_fast_k(const BwdKP& kp, const BwdWs& w, const Shape& sh, bool bf, hipStream_t stream) {
    if (bf) return kp.softplus ? launch_fast<bf16_t, K, true>(kp, w, sh, stream)
                               : launch_fast<bf16_t, K, false>(kp, w, sh, stream);
    return kp.softplus ? launch_fast<float, K, true>(kp, w, sh, stream)
                       : launch_fast<float, K, false>(kp, w, sh, stream);
}

int launch_scan_bwd(const BwdArgs& a, hipStream_t stream) {
    const Shape& sh = a.sh;
    if (ssd_bwd_supported(sh)) return launch_ssd_bwd(a, stream);
    auto al16 = [](const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) == 0; };
    const bool fast_io = sh.N == 16 && sh.d_inner() % kChan == 0 && al16(a.x) && al16(a.dt) &&
                         al16(a.dy) && al16(a.B) && al16(a.C) && al16(a.A) && al16(a.dstate) &&
                         al16(a.d_x) && al16(a.d_dt);
    const bool conv_fast = bwd_conv_fast_shape(sh) && fast_io && sh.S > 0 && sh.L > 0;
    if (!bwd_supported(sh) && !conv_fast) return launch_rows_bwd(a, stream);
    const int64_t per_row = sh.d_inner() * sh.N;
    BwdKP kp = {};
    kp.A = a.A; kp.D = a.D; kp.ids = a.ids; kp.x = a.x; kp.dt = a.dt; kp.B = a.B; kp.C = a.C;
    kp.dy = a.dy; kp.dstate = a.dstate; kp.d_x = a.d_x; kp.d_dt = a.d_dt; kp.err = a.err;
    kp.conv_w = a.conv_w; kp.conv_state = a.conv_state; kp.K = (int)sh.K;
    kp.L = (int)sh.L; kp.d_inner = (int)sh.d_inner(); kp.N = (int)sh.N; kp.R = (int)sh.R;
    kp.S = (int)sh.S; kp.n_cb = (int)((sh.d_inner() + kChan - 1) / kChan);
    kp.has_D = (sh.flags & SSM_HAS_D) ? 1 : 0;
    kp.softplus = (sh.flags & SSM_DT_SOFTPLUS) ? 1 : 0;
    const int64_t par = sh.R * per_row > per_row ? sh.R * per_row : per_row;
    const unsigned par_blocks = (unsigned)((par + 255) / 256 > 65535 ? 65535 : (par + 255) / 256);
    if (sh.S == 0 || sh.L == 0) {
        // no tokens: dh_0 is dstate itself; dA and dD are zero (no partials)
        kp.dA_part = nullptr;
        kp.dD_part = nullptr;
        hipLaunchKernelGGL(bwd_reduce_params, dim3(par_blocks), dim3(256), 0, stream, kp,
                           a.dstate, (int)sh.N, a.d_A, a.d_D, a.d_s, nullptr, nullptr);
        return hipGetLastError() == hipSuccess ? SSM_OK : SSM_ERR_HIP;
    }
    BwdWs w = carve(sh, a.ws);
    if (w.total > a.ws_bytes) return SSM_ERR_WORKSPACE;
    kp.ckpt = w.ckpt; kp.dbc_part = w.dbc; kp.dA_part = w.dA; kp.dD_part = w.dD; kp.ds_part = w.ds;
    kp.partW = w.partW; kp.partCS = w.partCS;
    // the checkpoint pass may split its uneven grid too, in the relay room of
    // bwd_fast (used one after the other; every finished pass leaves the flags at zero)
    const size_t room = relay_room(sh);
    int rc = launch_quad_ckpt(a, w.ckpt, reinterpret_cast<float*>(w.relay),
                              reinterpret_cast<int*>(w.relay + align_up(room * kRelayVals * kThreads * 4, 256)),
                              (int)room, stream);
    if (rc) return rc;
    const dim3 grid((unsigned)kp.n_cb, (unsigned)sh.S);
    const bool bf = sh.io == SSM_BF16;
    if (fast_io) {
        switch (sh.K) {
            case 0: rc = launch_fast_k<0>(kp, w, sh, bf, stream); break;
            case 2: rc = launch_fast_k<2>(kp, w, sh, bf, stream); break;
            case 3: rc = launch_fast_k<3>(kp, w, sh, bf, stream); break;
            case 4: rc = launch_fast_k<4>(kp, w, sh, bf, stream); break;
            default: rc = SSM_ERR_UNSUPPORTED;
        }
        if (rc) return rc;
    } else if (bf) {
        if (kp.softplus) hipLaunchKernelGGL((bwd_rev<bf16_t, true>), grid, dim3(kThreads), 0, stream, kp);
        else hipLaunchKernelGGL((bwd_rev<bf16_t, false>), grid, dim3(kThreads), 0, stream, kp);
    } else {
        if (kp.softplus) hipLaunchKernelGGL((bwd_rev<float, true>), grid, dim3(kThreads), 0, stream, kp);
        else hipLaunchKernelGGL((bwd_rev<float, false>), grid, dim3(kThreads), 0, stream, kp);
    }
    const int64_t tok8 = sh.S * sh.L * 8;  // 16-byte pieces of the sums
    hipLaunchKernelGGL(bwd_reduce_bc, dim3((unsigned)((tok8 + 255) / 256)), dim3(256), 0, stream, kp,
                       a.d_B, a.d_C);
    const int64_t cpar = sh.R * sh.d_inner() * (sh.K > 0 ? sh.K - 1 : 0);
    const unsigned red_blocks = cpar > par ? (unsigned)std::min<int64_t>((cpar + 255) / 256, 65535) : par_blocks;
    hipLaunchKernelGGL(bwd_reduce_params, dim3(red_blocks), dim3(256), 0, stream, kp,
                       (const float*)w.ds, 16, a.d_A, a.d_D, a.d_s, a.d_conv_w, a.d_conv_state);
    return hipGetLastError() == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

}  // namespace ssm
