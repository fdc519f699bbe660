// Mamba-1 forward for d_state <= 16 ("quad" layout), gfx950.
//
// Per (sequence i, channel c) the scan is the recurrence of "mambazip
// mamba1/model.rs" (selective_scan_state16): h_n = exp(dt*A_cn) h_n + (u*dt) B_n,
// y = sum_n C_n h_n + D_c u, with u = SiLU(causal conv of x) when the conv is
// fused (ggmlR ssm_conv reference: tap K-1 on the newest input).
//
// Layout.  Four lanes ("a quad") share one channel; quad lane q keeps states
// 4q..4q+3 in fp32 registers.  Tokens go in groups of four and quad lane q
// "owns" token t0+q of each group: it alone loads x and dt for that token,
// forms the conv, SiLU, dt*u and D*u, and finally stores y.  The other lanes
// read the owner's dt and dt*u through DPP quad permutes, which the
// compiler folds into the multiplies that use them.  Each lane forms the
// partial sum of C.h over its four states for each of the four tokens; a
// reduce-scatter across the quad leaves each owner the full y of its token.
// B and C rows are shared by every channel of a sequence, so each workgroup
// (64 channels) stages them in LDS as fp32 once per 64-token tile.
//
// Time chunks.  With few (sequence, channel) rows the tokens are split into
// chunks run by separate workgroups: kernel 1 scans chunks 0..n-2 from a zero
// state (chunk 0 from the true initial state) keeping only the end state and
// the chunk's dt sum; kernel 2 runs the carry h_in(c+1) = exp(A*sum dt(c))
// h_in(c) + end(c), the associative combine of the chunk operators
// (a, b) o (a', b') = (a a', a' b + b') ("kizzasi-model backprop_ssm.rs",
// associative scan); kernel 3 re-scans every chunk from its carried-in state
// and writes y and the final state.
//
// Relay (aligned case, no chunks, equal lengths): the (sequence, 64-channel
// block) jobs beyond a whole number per compute unit are cut into time
// pieces that hand on their fp32 state (relay.h).
//
// Extras (selective_scan_fwd_ext).  The dt bias is added where dt is read,
// before softplus; the gate y * SiLU(z) is applied where y is written (in the
// tiled variant on the 16-byte rows that leave LDS, with z read along the
// same rows).  With spans on a packed token axis every workgroup takes its
// sequence's first token and length; a chunk past the end of its sequence
// is empty, which the carry treats as the identity.
#include "device_common.h"
#include "relay.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

constexpr int kWaves = 4;                  // waves per workgroup
constexpr int kThreads = 64 * kWaves;      // 256
constexpr int kChanPerBlock = kThreads / 4;  // 64 channels
constexpr int kTile = 64;                  // tokens of B/C staged per LDS tile

struct QuadKP {
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
    float* agg;      // [n_chunks-1][S][d_inner][16] chunk end states (kernel 1)
    float* dtsum;    // [n_chunks-1][S][d_inner]     chunk dt sums    (kernel 1)
    float* hin;      // [n_chunks][S][d_inner][16]   carried-in states (kernel 2)
    const float* dt_bias;  // [d_inner] or null
    const void* z;         // like x, or null
    const int32_t* cu;     // [S+1] spans, or null
    int64_t T;             // tokens on the packed axis
    int L, d_inner, N, R, S;
    int chunk_len;   // multiple of 4
    int n_chunks;
    int has_D, softplus;
    int tiled;       // 1: aligned case, use quad_tiled
    // relay (quad_out only; relay_k == 0: off): blocks [0, relay_full) are
    // full jobs, then relay_k rounds of relay_rem pieces of chunk_len tokens
    int relay_full, relay_rem, relay_k;
    int* relay_flag;     // [relay_rem]  pieces of the job allowed to start
    float* relay_h;      // [relay_rem][64][16] state handed to the next piece
    int relay_max_jobs;  // cut jobs relay_h and relay_flag have room for (quad_ckpt)
};

template <typename T>
__device__ __forceinline__ float ld(const T* p) { return to_f32(*p); }

// The scan over tokens [t_begin, t_end) of one chunk.  MODE 0: end state
// only (kernel 1); MODE 1: y, and the final state if this is the last chunk;
// MODE 2: the state entering every kCkpt-token block, for the backward pass.
template <typename T, int K, int MODE>
__device__ __forceinline__ void quad_chunk(const QuadKP& p, int i, int64_t tok0, int c_raw, int q,
                                           int t_begin, int t_end, float (&h)[4],
                                           const float (&a2)[4], float& dt_acc, bool active,
                                           bool bad) {
    __shared__ __attribute__((aligned(16))) float B_l[2][kTile][16];
    __shared__ __attribute__((aligned(16))) float C_l[2][kTile][16];
    const int c = active ? c_raw : p.d_inner - 1;
    const int64_t seq_x = tok0 * p.d_inner;
    const T* xs = static_cast<const T*>(p.x) + seq_x + c;
    const T* dts = static_cast<const T*>(p.dt) + seq_x + c;
    T* ys = static_cast<T*>(p.y) + seq_x + c;
    const T* zs = p.z ? static_cast<const T*>(p.z) + seq_x + c : nullptr;
    const T* Bg = static_cast<const T*>(p.B) + tok0 * p.N;
    const T* Cg = static_cast<const T*>(p.C) + tok0 * p.N;
    const float Dc = p.has_D ? p.D[c] : 0.0f;
    const float dtb = p.dt_bias ? p.dt_bias[c] : 0.0f;

    float w[4] = {0.f, 0.f, 0.f, 0.f};
    float xp = 0.0f;  // the owner's input one group back (token t_begin - 4 + q)
    if constexpr (K > 0) {
#pragma unroll
        for (int j = 0; j < K; ++j) w[j] = p.conv_w[(int64_t)c * K + j];
        const int tp = t_begin - 4 + q;
        if (tp >= 0) {
            xp = ld(xs + (int64_t)tp * p.d_inner);
        } else if (tp >= -(K - 1)) {
            const int r = bad ? 0 : p.ids[i];
            xp = bad ? __builtin_nanf("")
                     : (p.conv_state ? p.conv_state[((int64_t)r * p.d_inner + c) * (K - 1) +
                                                    (tp + K - 1)]
                                     : 0.0f);
        }
    }

    const int tid = threadIdx.x;
    const int n_groups = (t_end - t_begin + 3) / 4;
    // stage B/C tile 0
    auto stage = [&](int buf, int tile_t0) {
        for (int e = tid; e < kTile * 16; e += kThreads) {
            const int tt = e >> 4, n = e & 15;
            const int t = tile_t0 + tt;
            const bool ok = (t < t_end) && (n < p.N);
            B_l[buf][tt][n] = ok ? ld(Bg + (int64_t)t * p.N + n) : 0.0f;
            C_l[buf][tt][n] = ok ? ld(Cg + (int64_t)t * p.N + n) : 0.0f;
        }
    };
    stage(0, t_begin);
    __syncthreads();

    // prefetch the first group's owned token
    int t_own = t_begin + q;
    float x_nx = 0.f, dt_nx = 0.f;
    if (t_own < t_end) {
        x_nx = ld(xs + (int64_t)t_own * p.d_inner);
        dt_nx = ld(dts + (int64_t)t_own * p.d_inner);
    }

    for (int g = 0; g < n_groups; ++g) {
        const int t0 = t_begin + 4 * g;
        const int tt0 = (4 * g) & (kTile - 1);
        const int buf = ((4 * g) / kTile) & 1;
        if constexpr (MODE == 2) {  // state entering each kCkpt-token block
            if (((t0 - t_begin) & (kCkpt - 1)) == 0 && active) {
                float* ck = p.agg + ((((int64_t)(t0 / kCkpt) * p.S + i) * p.d_inner + c) * 16 + 4 * q);
                *reinterpret_cast<float4*>(ck) = make_float4(h[0], h[1], h[2], h[3]);
            }
        }
        if (tt0 == 0 && t0 + kTile < t_end) stage(buf ^ 1, t0 + kTile);  // next tile
        const bool own_ok = (t0 + q) < t_end;
        float xc = x_nx, dtv = dt_nx;
        // prefetch the next group
        const int t_next = t0 + 4 + q;
        if (t_next < t_end) {
            x_nx = ld(xs + (int64_t)t_next * p.d_inner);
            dt_nx = ld(dts + (int64_t)t_next * p.d_inner);
        }
        dtv += dtb;
        if (p.softplus) dtv = softplus(dtv);
        float u;
        if constexpr (K > 0) {
            float cv = w[K - 1] * xc;
            if constexpr (K >= 2) cv = fmaf(w[K - 2], quad_rot<1>(q <= 2 ? xc : xp), cv);
            if constexpr (K >= 3) cv = fmaf(w[K - 3], quad_rot<2>(q <= 1 ? xc : xp), cv);
            if constexpr (K >= 4) cv = fmaf(w[K - 4], quad_rot<3>(q <= 0 ? xc : xp), cv);
            u = silu(cv);
            xp = xc;
        } else {
            u = xc;
        }
        if (!own_ok) { dtv = 0.0f; u = 0.0f; }  // padding token: identity step
        const float dtu = dtv * u;

        float yp[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            float dk, bk;
            if (k == 0) { dk = quad_bcast<0>(dtv); bk = quad_bcast<0>(dtu); }
            if (k == 1) { dk = quad_bcast<1>(dtv); bk = quad_bcast<1>(dtu); }
            if (k == 2) { dk = quad_bcast<2>(dtv); bk = quad_bcast<2>(dtu); }
            if (k == 3) { dk = quad_bcast<3>(dtv); bk = quad_bcast<3>(dtu); }
            if constexpr (MODE == 0) dt_acc += dk;  // sum over every token of the chunk
            const float4 Bv = *reinterpret_cast<const float4*>(&B_l[buf][tt0 + k][4 * q]);
            const float Bs[4] = {Bv.x, Bv.y, Bv.z, Bv.w};
            float acc = 0.0f;
            if constexpr (MODE == 1) {
                const float4 Cv = *reinterpret_cast<const float4*>(&C_l[buf][tt0 + k][4 * q]);
                const float Cs[4] = {Cv.x, Cv.y, Cv.z, Cv.w};
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const float a = fast_exp2(dk * a2[s]);
                    h[s] = fmaf(a, h[s], bk * Bs[s]);
                    acc = fmaf(Cs[s], h[s], acc);
                }
            } else {
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const float a = fast_exp2(dk * a2[s]);
                    h[s] = fmaf(a, h[s], bk * Bs[s]);
                }
            }
            yp[k] = acc;
        }
        if constexpr (MODE == 1) {
            // reduce-scatter: quad lane q ends with sum over the quad of yp[q]
            const bool hi2 = (q & 2) != 0;
            const float keep0 = hi2 ? yp[2] : yp[0], send0 = hi2 ? yp[0] : yp[2];
            const float keep1 = hi2 ? yp[3] : yp[1], send1 = hi2 ? yp[1] : yp[3];
            const float r0 = keep0 + quad_xor2(send0);
            const float r1 = keep1 + quad_xor2(send1);
            const bool hi1 = (q & 1) != 0;
            const float keep = hi1 ? r1 : r0, send = hi1 ? r0 : r1;
            const float yv = keep + quad_xor1(send);
            if (active && own_ok) {
                float yo = fmaf(Dc, u, yv);
                if (zs) yo *= silu(ld(zs + (int64_t)(t0 + q) * p.d_inner));
                store_io(ys + (int64_t)(t0 + q) * p.d_inner, yo);
            }
        }
        if (tt0 == kTile - 4) __syncthreads();  // next tile staged; this one fully read
    }
}

// Tiled variant of quad_chunk for the aligned case (d_inner a multiple of 64,
// d_state 16, 16-byte aligned tensors).  The workgroup moves whole
// [tile x 64 channels] blocks of x, dt and y and [tile x 16] blocks of B and
// C between HBM and LDS with 16-byte loads and stores that run along
// contiguous token rows; the loads for tile j+1 are issued into registers
// before tile j is computed, so their latency overlaps the compute, and
// written to LDS after it.  Owner lanes read x and dt of their token from
// LDS and write y there; B and C are converted to fp32 once per tile.
template <typename T>
struct TileCfg;
template <>
struct TileCfg<bf16_t> { static constexpr int TT = 64; };
template <>
struct TileCfg<float> { static constexpr int TT = 32; };

template <typename T, int K, int MODE, bool SOFTPLUS, bool GATE = false>
__device__ __forceinline__ void quad_tiled(const QuadKP& p, int i, int64_t tok0, int cb, int q, int cl,
                                           int t_begin, int t_end, float (&h)[4],
                                           const float (&a2)[4], float& dt_acc, bool bad) {
    constexpr int TT = TileCfg<T>::TT;
    constexpr int ES = (int)sizeof(T);
    constexpr int ROWB = 64 * ES;    // one token row of the block's 64 channels
    constexpr int CPR = ROWB / 16;   // 16-byte chunks per row
    constexpr int XS = ROWB + 32;    // padded LDS row stride: owners read 4 rows x 16 channels
    constexpr int CPT = 16 * ES / 16;  // 16-byte chunks per B/C token row (16 states)
    static_assert(TT * CPR == 2 * kThreads, "two x (and dt) chunks per thread per tile");
    static_assert(TT * CPT == kThreads / 2, "one B or C chunk per thread per tile");
    // x is staged as fp32 behind HX history rows (the conv's inputs before the
    // tile), so that an owner lane reads its K taps straight from LDS; a row
    // pitch of 8 (mod 32) words keeps the owners' 4 rows x 16 channels apart
    constexpr int HX = 3;
    constexpr int XPF = 64 + 8;
    __shared__ __attribute__((aligned(16))) float xf_l[(HX + TT) * XPF];
    __shared__ __attribute__((aligned(16))) char dt_l[TT * XS];
    // y tile in the io type; with the gate the owner multiplies its fp32 y by
    // SiLU(z) before the one rounding
    __shared__ __attribute__((aligned(16))) char y_l[MODE == 1 ? TT * XS : 16];
    __shared__ __attribute__((aligned(16))) float B_l[TT][16];
    __shared__ __attribute__((aligned(16))) float C_l[TT][16];
    // y reduce-scatter within each wave: lane (cl, q) leaves its four partial
    // sums (one per token of the group) at [cl][q][0..3] and reads those of
    // its own token, [cl][0..3][q]; a pitch of 20 words per channel keeps the
    // reads to two lanes per bank
    constexpr int YRP = 20;
    __shared__ __attribute__((aligned(16))) float yr_l[MODE == 1 ? kThreads / 4 * YRP : 4];

    const int tid = threadIdx.x;
    const int c = cb * 64 + cl;
    const int64_t row_stride = (int64_t)p.d_inner * ES;  // bytes between token rows
    const char* xg = static_cast<const char*>(p.x) + (tok0 * p.d_inner + cb * 64) * ES;
    const char* dg = static_cast<const char*>(p.dt) + (tok0 * p.d_inner + cb * 64) * ES;
    char* yg = static_cast<char*>(p.y) + (tok0 * p.d_inner + cb * 64) * ES;
    const char* zg = GATE ? static_cast<const char*>(p.z) + (tok0 * p.d_inner + cb * 64) * ES : nullptr;
    // B for waves 0-1, C for waves 2-3 (readfirstlane: wave-uniform, so its
    // buffer descriptor stays in scalar registers)
    const int c_half = __builtin_amdgcn_readfirstlane(tid >> 7);
    const char* bcg = static_cast<const char*>(c_half ? p.C : p.B) + tok0 * 16 * ES;
    const float Dc = p.has_D ? p.D[c] : 0.0f;
    const float dtb = p.dt_bias ? p.dt_bias[c] : 0.0f;

    float w[4] = {0.f, 0.f, 0.f, 0.f};
    if constexpr (K > 0) {
#pragma unroll
        for (int j = 0; j < K; ++j) w[j] = p.conv_w[(int64_t)c * K + j];
        // history rows of the first tile: the inputs t_begin-3 .. t_begin-1 of
        // the block's 64 channels (tokens before 0 from the gathered conv state)
        if (tid < HX * 64) {
            const int hrow = tid >> 6, hch = tid & 63;
            const int tp = t_begin - HX + hrow;
            float v = 0.0f;
            if (tp >= 0) {
                v = to_f32(*reinterpret_cast<const T*>(xg + (int64_t)tp * row_stride + hch * ES));
            } else if (tp >= -(K - 1)) {
                const int r = bad ? 0 : p.ids[i];
                v = bad ? __builtin_nanf("")
                        : (p.conv_state ? p.conv_state[((int64_t)r * p.d_inner + cb * 64 + hch) * (K - 1) +
                                                       (tp + K - 1)]
                                        : 0.0f);
            }
            xf_l[hrow * XPF + hch] = v;
        }
    }

    // Tile traffic goes through buffer descriptors based at the tile's first
    // row and ending at t_end: rows past the end read as zero and stores past
    // it are dropped, so no branch stands around a load or a store and the
    // per-lane offsets stay the same on every tile.
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    auto rsrc = [&](const char* base, int tb, int64_t row_bytes) {
        const int rows = min(t_end - tb, TT);
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base) + (int64_t)tb * row_bytes, 0,
                                                 rows > 0 ? (int)(rows * row_bytes) : 0, 0x00020000);
    };
    int xoff[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int e = tid + kThreads * r;
        xoff[r] = (int)((e / CPR) * row_stride) + (e % CPR) * 16;
    }
    const int bcoff = ((tid & (kThreads / 2 - 1)) / CPT) * 16 * ES + ((tid & (kThreads / 2 - 1)) % CPT) * 16;
    u32x4 sx[2], sdt[2], sbc, sz[GATE ? 2 : 1];
    auto load_tile = [&](int tb) {
        const auto rx = rsrc(xg, tb, row_stride), rd = rsrc(dg, tb, row_stride);
        const auto rb = rsrc(bcg, tb, 16 * ES);
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            sx[r] = __builtin_amdgcn_raw_buffer_load_b128(rx, xoff[r], 0, 0);
            sdt[r] = __builtin_amdgcn_raw_buffer_load_b128(rd, xoff[r], 0, 0);
        }
        sbc = __builtin_amdgcn_raw_buffer_load_b128(rb, bcoff, 0, 0);
        if constexpr (GATE && MODE == 1) {
            const auto rz = rsrc(zg, tb, row_stride);
#pragma unroll
            for (int r = 0; r < 2; ++r) sz[r] = __builtin_amdgcn_raw_buffer_load_b128(rz, xoff[r], 0, 0);
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int e = tid + kThreads * r;
            const int row = e / CPR, col = e % CPR;
            float* xd = xf_l + (HX + row) * XPF + col * (16 / ES);
            if constexpr (ES == 2) {
                float f[8];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    f[2 * k] = __uint_as_float(sx[r][k] << 16);
                    f[2 * k + 1] = __uint_as_float(sx[r][k] & 0xffff0000u);
                }
                *reinterpret_cast<float4*>(xd) = make_float4(f[0], f[1], f[2], f[3]);
                *reinterpret_cast<float4*>(xd + 4) = make_float4(f[4], f[5], f[6], f[7]);
            } else {
                *reinterpret_cast<u32x4*>(xd) = sx[r];
            }
            *reinterpret_cast<u32x4*>(dt_l + row * XS + col * 16) = sdt[r];
            // the gate's z goes where this tile's y will go: the owner of
            // (token, channel) reads its z there and writes its y in its place
            // (this thread stored the previous tile's y from these same
            // pieces just before)
            if constexpr (GATE && MODE == 1) *reinterpret_cast<u32x4*>(y_l + row * XS + col * 16) = sz[r];
        }
        const int e = tid & (kThreads / 2 - 1);
        const int tok = e / CPT, part = e % CPT;
        float* dst = (tid >> 7) ? &C_l[tok][0] : &B_l[tok][0];
        if constexpr (ES == 2) {
            const uint32_t wv[4] = {sbc.x, sbc.y, sbc.z, sbc.w};
            float f[8];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                f[2 * k] = __uint_as_float(wv[k] << 16);
                f[2 * k + 1] = __uint_as_float(wv[k] & 0xffff0000u);
            }
            *reinterpret_cast<float4*>(dst + part * 8) = make_float4(f[0], f[1], f[2], f[3]);
            *reinterpret_cast<float4*>(dst + part * 8 + 4) = make_float4(f[4], f[5], f[6], f[7]);
        } else {
            *reinterpret_cast<u32x4*>(dst + part * 4) = sbc;
        }
    };

    // One group of four tokens; FULL: every token of the group is < t_end.
    auto group = [&](int g, bool full_tile, int tb) {
        const int tt = 4 * g + q;  // owned row of this tile
        if constexpr (MODE == 2) {  // state entering each kCkpt-token block
            if (((tb + 4 * g - t_begin) & (kCkpt - 1)) == 0) {
                float* ck = p.agg + ((((int64_t)((tb + 4 * g) / kCkpt) * p.S + i) * p.d_inner + c) * 16 + 4 * q);
                *reinterpret_cast<float4*>(ck) = make_float4(h[0], h[1], h[2], h[3]);
            }
        }
        const bool own_ok = full_tile || (tb + tt < t_end);
        float dtv = to_f32(*reinterpret_cast<const T*>(dt_l + tt * XS + cl * ES)) + dtb;
        if constexpr (SOFTPLUS) dtv = softplus(dtv);
        float u;
        if constexpr (K > 0) {
            // the taps' inputs, tokens tt-K+1 .. tt (the first ones in the history rows)
            const float* xr = xf_l + (HX + tt - (K - 1)) * XPF + cl;
            float cv = w[0] * xr[0];
#pragma unroll
            for (int j = 1; j < K; ++j) cv = fmaf(w[j], xr[j * XPF], cv);
            u = silu(cv);
        } else {
            u = xf_l[(HX + tt) * XPF + cl];
        }
        if (!own_ok) { dtv = 0.0f; u = 0.0f; }
        const float dtu = dtv * u;
        // all decays and input terms of the group first (independent of h)
        float dec[4][4], inp[4][4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            float dk, bk;
            if (k == 0) { dk = quad_bcast<0>(dtv); bk = quad_bcast<0>(dtu); }
            if (k == 1) { dk = quad_bcast<1>(dtv); bk = quad_bcast<1>(dtu); }
            if (k == 2) { dk = quad_bcast<2>(dtv); bk = quad_bcast<2>(dtu); }
            if (k == 3) { dk = quad_bcast<3>(dtv); bk = quad_bcast<3>(dtu); }
            if constexpr (MODE == 0) dt_acc += dk;
            const float4 Bv = *reinterpret_cast<const float4*>(&B_l[4 * g + k][4 * q]);
            dec[k][0] = fast_exp2(dk * a2[0]);
            dec[k][1] = fast_exp2(dk * a2[1]);
            dec[k][2] = fast_exp2(dk * a2[2]);
            dec[k][3] = fast_exp2(dk * a2[3]);
            inp[k][0] = bk * Bv.x;
            inp[k][1] = bk * Bv.y;
            inp[k][2] = bk * Bv.z;
            inp[k][3] = bk * Bv.w;
        }
        float yp[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
#pragma unroll
            for (int s = 0; s < 4; ++s) h[s] = fmaf(dec[k][s], h[s], inp[k][s]);
            if constexpr (MODE == 1) {
                const float4 Cv = *reinterpret_cast<const float4*>(&C_l[4 * g + k][4 * q]);
                yp[k] = fmaf(Cv.w, h[3], fmaf(Cv.z, h[2], fmaf(Cv.y, h[1], Cv.x * h[0])));
            }
        }
        if constexpr (MODE == 1) {
            // LDS operations of one wave complete in order, so the quad's
            // partials are in place for the reads that follow; the wave
            // barrier keeps the compiler from reordering them
            float* yr = yr_l + cl * YRP;
            *reinterpret_cast<float4*>(yr + 4 * q) = make_float4(yp[0], yp[1], yp[2], yp[3]);
            __builtin_amdgcn_wave_barrier();
            const float ysum = (yr[q] + yr[4 + q]) + (yr[8 + q] + yr[12 + q]);
            __builtin_amdgcn_wave_barrier();
            float yv = fmaf(Dc, u, ysum);
            if constexpr (GATE) {  // y * SiLU(z), rounded once; z was staged in y's place
                const float zv = to_f32(*reinterpret_cast<const T*>(y_l + tt * XS + cl * ES));
                yv *= silu(zv);
            }
            if constexpr (ES == 2)
                *reinterpret_cast<bf16_t*>(y_l + tt * XS + cl * ES) = bf16_rne(yv);
            else
                *reinterpret_cast<float*>(y_l + tt * XS + cl * ES) = yv;
        }
    };

    const int n_tiles = (t_end - t_begin + TT - 1) / TT;
    load_tile(t_begin);
    store_tile();
    __syncthreads();
    for (int tile = 0; tile < n_tiles; ++tile) {
        const int tb = t_begin + tile * TT;
        const bool more = tile + 1 < n_tiles;
        load_tile(tb + TT);  // past the end: zero rows, never staged
        if (tb + TT <= t_end) {
#pragma unroll 2
            for (int g = 0; g < TT / 4; ++g) group(g, true, tb);
        } else {
            const int n_g = (t_end - tb + 3) / 4;
            for (int g = 0; g < n_g; ++g) group(g, false, tb);
        }
        // this tile's last HX inputs become the next tile's history rows: read
        // them now, write them once every wave is past this tile
        float hx = 0.0f;
        if constexpr (K > 0)
            if (tid < HX * 64) hx = xf_l[(TT + (tid >> 6)) * XPF + (tid & 63)];
        __syncthreads();  // tile fully read (and y tile fully written)
        if constexpr (MODE == 1) {
            const auto ry = rsrc(yg, tb, row_stride);
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int e = tid + kThreads * r;
                const int row = e / CPR, col = e % CPR;
                const u32x4 yv = *reinterpret_cast<const u32x4*>(y_l + row * XS + col * 16);
                __builtin_amdgcn_raw_buffer_store_b128(yv, ry, xoff[r], 0, 0);
            }
        }
        if (more) {
            store_tile();
            if constexpr (K > 0)
                if (tid < HX * 64) xf_l[(tid >> 6) * XPF + (tid & 63)] = hx;
        }
        __syncthreads();
    }
}

template <typename T, int K, bool TILED, bool SOFTPLUS>
__global__ __launch_bounds__(kThreads) void quad_agg(QuadKP p) {
    const int q = threadIdx.x & 3;
    const int c_raw = blockIdx.x * kChanPerBlock + (threadIdx.x >> 2);
    const bool active = c_raw < p.d_inner;
    const int c = active ? c_raw : p.d_inner - 1;
    const int i = blockIdx.y;
    const int chunk = blockIdx.z;  // 0 .. n_chunks-2
    int r = p.ids[i];
    const SeqSpan sp = seq_span(p.cu, i, p.L, p.T);
    const bool bad = (r < 0) | (r >= p.R) | sp.bad;
    float h[4], a2[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int n = 4 * q + s;
        a2[s] = n < p.N ? p.A[(int64_t)c * p.N + n] * kLog2e : 0.0f;
        h[s] = 0.0f;
        if (chunk == 0 && n < p.N)
            h[s] = bad ? __builtin_nanf("") : p.s[((int64_t)r * p.d_inner + c) * p.N + n];
    }
    float dt_acc = 0.0f;
    const int t_begin = chunk * p.chunk_len;
    const int t_end = min(sp.len, t_begin + p.chunk_len);
    if (t_begin < t_end) {  // workgroup-uniform: a chunk past the sequence's end is empty
        if constexpr (TILED)
            quad_tiled<T, K, 0, SOFTPLUS>(p, i, sp.t0, blockIdx.x, q, threadIdx.x >> 2, t_begin, t_end, h, a2, dt_acc, bad);
        else
            quad_chunk<T, K, 0>(p, i, sp.t0, c_raw, q, t_begin, t_end, h, a2, dt_acc, active, bad);
    }
    if (active) {
        const int64_t row = ((int64_t)chunk * p.S + i) * p.d_inner + c;
#pragma unroll
        for (int s = 0; s < 4; ++s) p.agg[row * 16 + 4 * q + s] = h[s];
        if (q == 0) p.dtsum[row] = dt_acc;
    }
}

// One thread per (sequence, channel, state): fold the chunk end states.
__global__ __launch_bounds__(256) void quad_carry(QuadKP p) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t rows = (int64_t)p.S * p.d_inner;
    if (e >= rows * 16) return;
    const int64_t row = e >> 4;
    const int n = (int)(e & 15);
    const int c = (int)(row % p.d_inner);
    const float a2 = n < p.N ? p.A[(int64_t)c * p.N + n] * kLog2e : 0.0f;
    const float* __restrict__ agg = p.agg;
    const float* __restrict__ dts = p.dtsum;
    float* __restrict__ hin = p.hin;
    float h = agg[row * 16 + n];  // chunk 0's end state (from the true initial state)
#pragma unroll 4
    for (int ch = 1; ch < p.n_chunks; ++ch) {
        hin[((int64_t)ch * rows + row) * 16 + n] = h;
        if (ch + 1 < p.n_chunks) {
            const int64_t src = (int64_t)ch * rows + row;
            h = fmaf(fast_exp2(a2 * dts[src]), h, agg[src * 16 + n]);
        }
    }
}

template <typename T, int K, bool TILED, bool SOFTPLUS, bool GATE>
__global__ __launch_bounds__(kThreads) void quad_out(QuadKP p) {
    const int q = threadIdx.x & 3;
    int cbk = blockIdx.x, i = blockIdx.y, chunk = blockIdx.z;
    int piece = -1, sj = 0;  // relay: piece of cut job sj, or -1 for a whole job
    if (TILED && p.relay_k) {  // 1-D grid
        const int cblocks = p.d_inner / kChanPerBlock;
        const RelayBlock rb = relay_block(blockIdx.x, p.relay_full, p.relay_rem);
        piece = rb.piece;
        sj = rb.cut;
        cbk = rb.job % cblocks;
        i = rb.job / cblocks;
        chunk = 0;
    }
    // the pieces of a split job run one after another, so their waves go
    // first at the instruction arbiter; the full jobs beside them take the
    // issue slots the pieces leave
    if (piece >= 0) __builtin_amdgcn_s_setprio(2);
    const int c_raw = cbk * kChanPerBlock + (threadIdx.x >> 2);
    const bool active = c_raw < p.d_inner;
    const int c = active ? c_raw : p.d_inner - 1;
    int r = p.ids[i];
    const SeqSpan sp = seq_span(p.cu, i, p.L, p.T);
    if (p.cu && piece < 0 && p.n_chunks == 1) {
        // packed sequences of mixed lengths: a workgroup whose sequence is
        // longer than the mean (T / S) is on the critical path, so its waves
        // go first at the instruction arbiter of the compute unit it shares
        // with shorter ones (length over the mean in eighths: from 10 / 8 up
        // priority 3, from 9 / 8 2, from 7 / 8 1)
        const int64_t e8 = (8 * (int64_t)sp.len * p.S) / (p.T > 0 ? p.T : 1);
        if (e8 >= 10) __builtin_amdgcn_s_setprio(3);
        else if (e8 >= 9) __builtin_amdgcn_s_setprio(2);
        else if (e8 >= 7) __builtin_amdgcn_s_setprio(1);
    }
    const bool bad_id = (r < 0) | (r >= p.R);
    const bool bad = bad_id | sp.bad;
    if (bad) {
        r = 0;
        if (threadIdx.x == 0 && chunk == 0)
            atomicOr(p.err, (bad_id ? (uint32_t)SSM_DEVERR_IDS : 0u) | (sp.bad ? (uint32_t)SSM_DEVERR_SEQLENS : 0u));
    }
    float h[4], a2[4];
    const int64_t rows = (int64_t)p.S * p.d_inner;
    float* relay_h = piece >= 0 ? p.relay_h + ((int64_t)sj * kChanPerBlock + (threadIdx.x >> 2)) * 16 + 4 * q
                                : nullptr;
    if (piece > 0) {  // the previous piece's end state
        relay_wait(p.relay_flag + sj, piece, p.err);
        if (piece + 1 == p.relay_k) relay_reset(p.relay_flag + sj);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int n = 4 * q + s;
        a2[s] = n < p.N ? p.A[(int64_t)c * p.N + n] * kLog2e : 0.0f;
        if (piece > 0)
            h[s] = relay_h[s];
        else if (chunk == 0)
            h[s] = n < p.N ? (bad ? __builtin_nanf("") : p.s[((int64_t)r * p.d_inner + c) * p.N + n])
                           : 0.0f;
        else
            h[s] = p.hin[((int64_t)chunk * rows + (int64_t)i * p.d_inner + c) * 16 + n];
    }
    float dt_acc = 0.0f;
    const int t_begin = (piece > 0 ? piece : chunk) * p.chunk_len;
    const int t_end = min(sp.len, piece < 0 && p.relay_k ? sp.len : t_begin + p.chunk_len);
    if (t_begin < t_end) {  // workgroup-uniform
        if constexpr (TILED)
            quad_tiled<T, K, 1, SOFTPLUS, GATE>(p, i, sp.t0, cbk, q, threadIdx.x >> 2, t_begin, t_end, h, a2,
                                                dt_acc, bad);
        else
            quad_chunk<T, K, 1>(p, i, sp.t0, c_raw, q, t_begin, t_end, h, a2, dt_acc, active, bad);
    }
    if (piece >= 0 && piece + 1 < p.relay_k) {
#pragma unroll
        for (int s = 0; s < 4; ++s) relay_put(&relay_h[s], h[s]);  // hand the state on
        relay_publish_puts(p.relay_flag + sj, piece + 1);
        return;
    }
    if (active && chunk == p.n_chunks - 1) {
        float* so = p.state_out + ((int64_t)i * p.d_inner + c) * p.N;
#pragma unroll
        for (int s = 0; s < 4; ++s)
            if (4 * q + s < p.N) so[4 * q + s] = h[s];
        if constexpr (K > 1) {
            if (p.conv_state_out && q == 0) {
                const T* xs = static_cast<const T*>(p.x) + sp.t0 * p.d_inner + c;
                float* co = p.conv_state_out + ((int64_t)i * p.d_inner + c) * (K - 1);
#pragma unroll
                for (int j = 0; j < K - 1; ++j) {
                    const int tau = sp.len - (K - 1) + j;
                    float v;
                    if (tau >= 0) v = ld(xs + (int64_t)tau * p.d_inner);
                    else if (bad) v = __builtin_nanf("");
                    else v = p.conv_state ? p.conv_state[((int64_t)r * p.d_inner + c) * (K - 1) + tau + K - 1] : 0.0f;
                    co[j] = v;
                }
            }
        }
    }
}

// Forward scan that stores the state entering every kCkpt-token block to
// p.agg ([n_blocks][S][d_inner][16]); the backward pass recomputes each block
// from it.
template <typename T, int K, bool TILED, bool SOFTPLUS>
__global__ __launch_bounds__(kThreads) void quad_ckpt(QuadKP p) {
    static_assert(TILED || K == 0, "the fused conv runs on the tiled variant");
    const int q = threadIdx.x & 3;
    int cbk = blockIdx.x, i = blockIdx.y;
    int piece = -1, sj = 0;  // relay: piece of cut job sj, or -1 for a whole job
    if (TILED && p.relay_k) {  // 1-D grid, as quad_out's
        const int cblocks = p.d_inner / kChanPerBlock;
        const RelayBlock rb = relay_block(blockIdx.x, p.relay_full, p.relay_rem);
        piece = rb.piece;
        sj = rb.cut;
        cbk = rb.job % cblocks;
        i = rb.job / cblocks;
    }
    if (piece >= 0) __builtin_amdgcn_s_setprio(2);  // a piece chain goes first (relay.h)
    const int c_raw = cbk * kChanPerBlock + (threadIdx.x >> 2);
    const bool active = c_raw < p.d_inner;
    const int c = active ? c_raw : p.d_inner - 1;
    const int r = p.ids[i];
    const bool bad = (r < 0) | (r >= p.R);
    if (bad && threadIdx.x == 0 && cbk == 0 && piece <= 0) atomicOr(p.err, (uint32_t)SSM_DEVERR_IDS);
    float h[4], a2[4];
    float* relay_h = piece >= 0 ? p.relay_h + ((int64_t)sj * kChanPerBlock + (threadIdx.x >> 2)) * 16 + 4 * q
                                : nullptr;
    if (piece > 0) {  // the previous piece's end state
        relay_wait(p.relay_flag + sj, piece, p.err);
        if (piece + 1 == p.relay_k) relay_reset(p.relay_flag + sj);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int n = 4 * q + s;
        a2[s] = n < p.N ? p.A[(int64_t)c * p.N + n] * kLog2e : 0.0f;
        if (piece > 0)
            h[s] = relay_h[s];
        else
            h[s] = n < p.N ? (bad ? __builtin_nanf("") : p.s[((int64_t)r * p.d_inner + c) * p.N + n]) : 0.0f;
    }
    float dt_acc = 0.0f;
    const int t_begin = piece > 0 ? piece * p.chunk_len : 0;
    const int t_end = piece >= 0 ? min(p.L, t_begin + p.chunk_len) : p.L;
    if constexpr (TILED)
        quad_tiled<T, K, 2, SOFTPLUS>(p, i, (int64_t)i * p.L, cbk, q, threadIdx.x >> 2, t_begin, t_end, h, a2,
                                      dt_acc, bad);
    else
        quad_chunk<T, 0, 2>(p, i, (int64_t)i * p.L, c_raw, q, 0, p.L, h, a2, dt_acc, active, bad);
    if (piece >= 0 && piece + 1 < p.relay_k) {
#pragma unroll
        for (int s = 0; s < 4; ++s) relay_put(&relay_h[s], h[s]);  // hand the state on
        relay_publish_puts(p.relay_flag + sj, piece + 1);
    }
}

constexpr int kRelayMaxJobs = 1024;  // cut jobs the workspace has room for

size_t relay_bytes(int64_t jobs) {
    return align_up((size_t)jobs * kChanPerBlock * 16 * 4, 256) + align_up((size_t)jobs * 4, 256);
}

// dry: decide only (no launch); returns the relay pieces per split job.
template <typename T, int K, bool TILED, bool SOFTPLUS, bool GATE = false>
int launch_quad_t(QuadKP kp, hipStream_t st, int* relay_k_out) {
    const dim3 block(kThreads);
    const unsigned cblocks = (unsigned)((kp.d_inner + kChanPerBlock - 1) / kChanPerBlock);
    // (not for packed sequences: the split assumes jobs of equal length; those
    // raise the wave priority of the longer sequences instead)
    if (TILED && kp.relay_h && !kp.cu) {
        const int n_cu = device_cus();
        const int cap = n_cu > 0 ? resident_blocks((const void*)quad_out<T, K, TILED, SOFTPLUS, GATE>, kThreads) : 0;
        const RelaySplit rs = relay_split((int64_t)kp.S * cblocks, kp.L, TileCfg<T>::TT, cap, n_cu, kRelayMaxJobs);
        if (rs.k) {
            kp.relay_full = rs.full;
            kp.relay_rem = rs.rem;
            kp.relay_k = rs.k;
            kp.chunk_len = rs.len;
        }
    }
    if (relay_k_out) {
        *relay_k_out = kp.relay_k;
        return SSM_OK;
    }
    if (kp.relay_k) {
        const unsigned n_blocks = (unsigned)(kp.relay_full + kp.relay_rem * kp.relay_k);
        hipLaunchKernelGGL((quad_out<T, K, TILED, SOFTPLUS, GATE>), dim3(n_blocks), block, 0, st, kp);
        return hipGetLastError() == hipSuccess ? SSM_OK : SSM_ERR_HIP;
    }
    if (kp.n_chunks > 1) {
        hipLaunchKernelGGL((quad_agg<T, K, TILED, SOFTPLUS>), dim3(cblocks, kp.S, kp.n_chunks - 1), block, 0,
                           st, kp);
        const int64_t threads = (int64_t)kp.S * kp.d_inner * 16;
        hipLaunchKernelGGL(quad_carry, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, kp);
    }
    hipLaunchKernelGGL((quad_out<T, K, TILED, SOFTPLUS, GATE>), dim3(cblocks, kp.S, kp.n_chunks), block, 0, st, kp);
    return hipGetLastError() == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

template <typename T, int K>
int launch_quad(const QuadKP& kp, hipStream_t st, int* relay_k_out) {
    if (kp.tiled) {
        if (kp.z)
            return kp.softplus ? launch_quad_t<T, K, true, true, true>(kp, st, relay_k_out)
                               : launch_quad_t<T, K, true, false, true>(kp, st, relay_k_out);
        return kp.softplus ? launch_quad_t<T, K, true, true>(kp, st, relay_k_out)
                           : launch_quad_t<T, K, true, false>(kp, st, relay_k_out);
    }
    return launch_quad_t<T, K, false, false>(kp, st, relay_k_out);
}

// Chunk length (tokens, multiple of 4) so that the grid has about
// target_waves waves; 0 means no split.
int pick_chunk(const Shape& sh) {
    if (sh.chunk > 0) return (sh.chunk + 3) / 4 * 4;
    const int64_t waves = sh.S * ((sh.d_inner() + kChanPerBlock - 1) / kChanPerBlock) * kWaves;
    const int64_t target = 4096;  // about 4 waves per SIMD on 1024 SIMDs
    if (waves >= target / 2 || sh.L <= 256) return 0;
    int64_t n = (target + waves - 1) / waves;
    int64_t len = (sh.L + n - 1) / n;
    len = (len + 3) / 4 * 4;
    if (len < 64) len = 64;
    return (int)len;
}

}  // namespace

bool quad_supported(const Shape& sh) {
    return sh.a_per_state && sh.P == 1 && sh.N <= 16 && sh.G == 1 && (sh.K == 0 || sh.K == 2 ||
                                                                      sh.K == 3 || sh.K == 4);
}

bool quad_chunked(const Shape& sh) {
    const int len = pick_chunk(sh);
    return len > 0 && len < sh.L;
}

size_t quad_workspace_bytes(const Shape& sh) {
    if (!quad_chunked(sh)) {
        // room for the relay of an aligned, unchunked grid
        const int64_t jobs = sh.S * (sh.d_inner() / kChanPerBlock);
        if (sh.N != 16 || sh.d_inner() % kChanPerBlock != 0 || jobs == 0 || sh.L < 2) return 0;
        return relay_bytes(jobs < kRelayMaxJobs ? jobs : kRelayMaxJobs);
    }
    const int len = pick_chunk(sh);
    const int64_t n = (sh.L + len - 1) / len;
    const int64_t rows = sh.S * sh.d_inner();
    return (size_t)((n - 1) * rows * 16 + (n - 1) * rows + n * rows * 16) * 4 + 3 * 256;
}

namespace {
template <int K>
void launch_ckpt_k(QuadKP kp, dim3 grid, bool bf, hipStream_t stream) {
    if (kp.relay_h) {  // the relay split of an uneven grid (as the forward's)
        const int n_cu = device_cus();
        const void* fn = bf ? (kp.softplus ? (const void*)quad_ckpt<bf16_t, K, true, true>
                                           : (const void*)quad_ckpt<bf16_t, K, true, false>)
                            : (kp.softplus ? (const void*)quad_ckpt<float, K, true, true>
                                           : (const void*)quad_ckpt<float, K, true, false>);
        const int cap = n_cu > 0 ? resident_blocks(fn, kThreads) : 0;
        const int cblocks = kp.d_inner / kChanPerBlock;
        const RelaySplit rs = relay_split((int64_t)kp.S * cblocks, kp.L, bf ? TileCfg<bf16_t>::TT : TileCfg<float>::TT,
                                          cap, n_cu, kp.relay_max_jobs);
        if (rs.k) {
            kp.relay_full = rs.full;
            kp.relay_rem = rs.rem;
            kp.relay_k = rs.k;
            kp.chunk_len = rs.len;
            grid = dim3((unsigned)(rs.full + rs.rem * rs.k));
        }
    }
    if (bf) {
        if (kp.softplus) hipLaunchKernelGGL((quad_ckpt<bf16_t, K, true, true>), grid, dim3(kThreads), 0, stream, kp);
        else hipLaunchKernelGGL((quad_ckpt<bf16_t, K, true, false>), grid, dim3(kThreads), 0, stream, kp);
    } else {
        if (kp.softplus) hipLaunchKernelGGL((quad_ckpt<float, K, true, true>), grid, dim3(kThreads), 0, stream, kp);
        else hipLaunchKernelGGL((quad_ckpt<float, K, true, false>), grid, dim3(kThreads), 0, stream, kp);
    }
}
}  // namespace

int launch_quad_ckpt(const BwdArgs& a, float* ckpt, float* relay_h, int* relay_flag, int relay_max_jobs,
                     hipStream_t stream) {
    const Shape& sh = a.sh;
    QuadKP kp = {};
    kp.T = sh.S * sh.L;
    kp.s = a.s; kp.x = a.x; kp.dt = a.dt; kp.A = a.A; kp.B = a.B; kp.C = a.C; kp.D = nullptr;
    kp.ids = a.ids; kp.err = a.err; kp.agg = ckpt;
    kp.conv_w = a.conv_w; kp.conv_state = a.conv_state;  // the fused conv (sh.K > 0)
    kp.L = (int)sh.L; kp.d_inner = (int)sh.d_inner(); kp.N = (int)sh.N; kp.R = (int)sh.R;
    kp.S = (int)sh.S;
    kp.has_D = 0;
    kp.softplus = (sh.flags & SSM_DT_SOFTPLUS) ? 1 : 0;
    auto al16 = [](const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) == 0; };
    // the tiled path also stages y; the checkpoint pass writes none, so only inputs matter
    kp.tiled = (sh.N == 16 && sh.d_inner() % 64 == 0 && al16(a.x) && al16(a.dt) && al16(a.B) &&
                al16(a.C) && sh.d_inner() * 4 * 64 < (int64_t(1) << 31)) ? 1 : 0;
    kp.chunk_len = (int)sh.L;
    kp.n_chunks = 1;
    if (kp.tiled) {  // (the tiled path covers whole 64-channel blocks)
        kp.relay_h = relay_h;
        kp.relay_flag = relay_flag;
        kp.relay_max_jobs = relay_max_jobs;
    }
    const dim3 grid((unsigned)((kp.d_inner + kChanPerBlock - 1) / kChanPerBlock), (unsigned)sh.S);
    const bool bf = sh.io == SSM_BF16;
    if (sh.K > 0 && !kp.tiled) return SSM_ERR_UNSUPPORTED;  // the fused conv runs tiled only
    if (kp.tiled) {
        switch (sh.K) {
            case 0: launch_ckpt_k<0>(kp, grid, bf, stream); break;
            case 2: launch_ckpt_k<2>(kp, grid, bf, stream); break;
            case 3: launch_ckpt_k<3>(kp, grid, bf, stream); break;
            case 4: launch_ckpt_k<4>(kp, grid, bf, stream); break;
            default: return SSM_ERR_UNSUPPORTED;
        }
    } else {
        if (bf) hipLaunchKernelGGL((quad_ckpt<bf16_t, 0, false, false>), grid, dim3(kThreads), 0, stream, kp);
        else hipLaunchKernelGGL((quad_ckpt<float, 0, false, false>), grid, dim3(kThreads), 0, stream, kp);
    }
    return hipGetLastError() == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

int launch_quad_fwd(const FwdArgs& a, hipStream_t stream, int* relay_k_out) {
    const Shape& sh = a.sh;
    QuadKP kp;
    kp.s = a.s; kp.x = a.x; kp.dt = a.dt; kp.A = a.A; kp.B = a.B; kp.C = a.C; kp.D = a.D;
    kp.ids = a.ids; kp.conv_w = a.conv_w; kp.conv_state = a.conv_state; kp.y = a.y;
    kp.state_out = a.state_out; kp.conv_state_out = a.conv_state_out; kp.err = a.err;
    kp.dt_bias = a.dt_bias; kp.z = a.z; kp.cu = a.cu; kp.T = a.T;
    kp.L = (int)sh.L; kp.d_inner = (int)sh.d_inner(); kp.N = (int)sh.N; kp.R = (int)sh.R;
    kp.S = (int)sh.S;
    kp.has_D = (sh.flags & SSM_HAS_D) ? 1 : 0;
    kp.softplus = (sh.flags & SSM_DT_SOFTPLUS) ? 1 : 0;
    const int es = sh.io_bytes();
    auto al16 = [](const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) == 0; };
    // one tile's rows of x/dt/y must fit the 31-bit sizes of a buffer descriptor
    kp.tiled = (sh.N == 16 && sh.d_inner() % 64 == 0 && al16(a.x) && al16(a.dt) && al16(a.B) &&
                al16(a.C) && al16(a.y) && al16(a.z) &&
                sh.d_inner() * 4 * 64 < (int64_t(1) << 31)) ? 1 : 0;
    const int tile = es == 2 ? 64 : 32;
    int len = pick_chunk(sh);
    if (len == 0 || len >= sh.L) len = (int)((sh.L + 3) / 4 * 4);
    if (len == 0) len = 4;
    if (kp.tiled) len = (len + tile - 1) / tile * tile;
    kp.chunk_len = len;
    kp.n_chunks = (int)((sh.L + len - 1) / len);
    if (kp.n_chunks < 1) kp.n_chunks = 1;
    kp.agg = kp.dtsum = kp.hin = nullptr;
    kp.relay_full = kp.relay_rem = kp.relay_k = 0;
    kp.relay_flag = nullptr;
    kp.relay_h = nullptr;
    if (kp.n_chunks == 1 && kp.tiled && !a.cu && sh.L >= 2) {
        const int64_t jobs = sh.S * (sh.d_inner() / kChanPerBlock);
        const int64_t room = jobs < kRelayMaxJobs ? jobs : kRelayMaxJobs;
        if (a.ws && a.ws_bytes >= relay_bytes(room)) {
            kp.relay_h = reinterpret_cast<float*>(a.ws);
            kp.relay_flag = reinterpret_cast<int*>(a.ws + align_up((size_t)room * kChanPerBlock * 16 * 4, 256));
        }
    }
    if (kp.n_chunks > 1) {
        const int64_t rows = sh.S * sh.d_inner();
        char* w = a.ws;
        kp.agg = reinterpret_cast<float*>(w);
        w += align_up((size_t)(kp.n_chunks - 1) * rows * 16 * 4, 256);
        kp.dtsum = reinterpret_cast<float*>(w);
        w += align_up((size_t)(kp.n_chunks - 1) * rows * 4, 256);
        kp.hin = reinterpret_cast<float*>(w);
        if ((size_t)(w - a.ws) + (size_t)kp.n_chunks * rows * 16 * 4 > a.ws_bytes)
            return SSM_ERR_WORKSPACE;
    }
    const bool bf = sh.io == SSM_BF16;
    switch (sh.K) {
        case 0: return bf ? launch_quad<bf16_t, 0>(kp, stream, relay_k_out) : launch_quad<float, 0>(kp, stream, relay_k_out);
        case 2: return bf ? launch_quad<bf16_t, 2>(kp, stream, relay_k_out) : launch_quad<float, 2>(kp, stream, relay_k_out);
        case 3: return bf ? launch_quad<bf16_t, 3>(kp, stream, relay_k_out) : launch_quad<float, 3>(kp, stream, relay_k_out);
        case 4: return bf ? launch_quad<bf16_t, 4>(kp, stream, relay_k_out) : launch_quad<float, 4>(kp, stream, relay_k_out);
        default: return SSM_ERR_UNSUPPORTED;
    }
}

}  // namespace ssm
