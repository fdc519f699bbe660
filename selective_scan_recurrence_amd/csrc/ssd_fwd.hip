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
// which are dense products: G = C B^T over the states, M = G o L with
// L[t][s] = exp(cum_t - cum_s) dt_s for s <= t (0 above the diagonal), and
// the state at the chunk end h_out = exp(cum_last) h_in + (w o X)^T B with
// w_s = exp(cum_last - cum_s) dt_s.  This chunked form is derived here from
// the recurrence; it reaches the sequential result up to rounding.  Every
// exponent is cum_t - cum_s with s <= t, which is <= 0 for A <= 0.
//
// Work split.  One workgroup (8 waves) runs one (sequence, head) through its
// 64-token chunks in order.  With NS = 8 / (P/16) waves per 16-channel block,
// wave w = (channel block w / NS, part w % NS) keeps the states
// [part*N/NS, (part+1)*N/NS) of its channel block (h^T, fp32) in MFMA
// accumulators and produces the y of its channel block for the token blocks
// [part*4/NS, (part+1)*4/NS) of every chunk.  All products run on
// v_mfma_f32_16x16x32_bf16 (bf16 operands, fp32 accumulation), computed
// transposed:
//     G^T[s][t]   = B C^T          (A: B rows, B: C rows; natural LDS rows)
//     M           = G o L          (the 10 causal tiles, spread over the waves,
//                                   written to LDS as bf16 rows [t][s])
//     Yd^T[p][t]  = X^T M^T        (A: x columns, B: M rows)
//     Yo^T[p][t]  = h C^T          (A: the wave's own fp32 state, taken from
//                                   its accumulators as a bf16 pair hi + lo,
//                                   B: C rows; summed over its state part)
//     h^T[n][p]  += B^T (w o X)    (A: B columns, B: x columns scaled by w)
// The carried-state product needs every state of a channel, so each wave
// forms it over its own part of the states for all 64 tokens and hands the
// partial sums of the other waves' token blocks to them through LDS.  The
// state enters that product as hi + lo, about 16 significant bits, so y's
// error does not grow with the size of the state.  Within a 32-wide k block
// the MFMA pairs A and B by the k slot a lane supplies, so the slots may map
// to any state as long as both operands use the same map: lane 16g + i holds
// states 16j + 4g + r (r = 0..3) of accumulator tile j, and reads C at the
// same states.
// Operands whose k index is the token (x and B columns) are read from the
// natural row-major tiles with gfx950's transposing LDS read
// (ds_read_b64_tr_b16): within each 16-lane group, lane i receives element
// i%4 of the 8-byte blocks addressed by lanes 4k + i/4 (k = 0..3), so lanes
// 4k+q addressing row s_k, columns 4q..4q+3 of a 16-column block give lane i
// the column i of rows s_0..s_3.
// Three barriers per chunk: chunk staged; M and the partial carried-state
// sums written; chunk consumed.
//
#include "device_common.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int kQ = 64;        // tokens per chunk
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;

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
    float* ckpt;   // CKPT: [S][H][n_chunks] x the state entering each chunk (SsdCkptLayout)
    const uint16_t* dt_t;  // CKPT: dt's bf16 bits as [S][H][L], tokens contiguous (read in place of dt)
    uint32_t* err;
    const float* dt_bias;  // [H] or null
    const bf16_t* z;       // like x (GATE), or null
    const int32_t* cu;     // [S+1] spans on the packed token axis, or null
    int64_t T;             // tokens on the packed axis
    int L, H, G, R, hpg;
    int has_D;
};

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 ld8(const bf16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ bf16x4 ld4(const bf16_t* p) { return *reinterpret_cast<const bf16x4*>(p); }
__device__ __forceinline__ bf16x8 cat(const bf16x4& lo, const bf16x4& hi) {
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ bf16x8 to_bf16x8(const f32x4& lo, const f32x4& hi) {
    bf16x8 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        r[j] = (__bf16)lo[j];
        r[4 + j] = (__bf16)hi[j];
    }
    return r;
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_or_zero(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                 ROW_MASK, 0xF, false));
}
// Inclusive prefix sum over the 64 lanes of a wave with DPP: shifts of 1, 2,
// 4, 8 within each 16-lane row, then the row totals through row_bcast15/31.
__device__ __forceinline__ float wave_incl_sum(float v) {
    v += dpp_or_zero<0x111, 0xF>(v);  // row_shr:1
    v += dpp_or_zero<0x112, 0xF>(v);  // row_shr:2
    v += dpp_or_zero<0x114, 0xF>(v);  // row_shr:4
    v += dpp_or_zero<0x118, 0xF>(v);  // row_shr:8
    v += dpp_or_zero<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
    v += dpp_or_zero<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
    return v;
}

// B and C rows sit in LDS with their states in a permuted order: state
// n = 32b + 16h + 4g + r at position 32b + 8g + 4h + r.  Products over the
// states (C B^T) pair the same positions and do not see the order; the
// carried-state product reads the states 4g..4g+3 of a lane's two
// accumulator tiles (16 apart) as one 16-byte run.
__device__ __forceinline__ int spos(int n) {
    return (n & ~31) | ((n & 12) << 1) | ((n & 16) >> 2) | (n & 3);
}

// transposing LDS read of this lane's 8-byte block (see the layout above)
__device__ __forceinline__ bf16x4 ldtr(const bf16_t* p) {
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(p));
    return __builtin_bit_cast(bf16x4, v);
}

// CKPT: the backward's recompute: no y, no final state; the fp32 state
// entering every chunk is stored for the reverse pass.
template <int P, int N, bool SOFTPLUS, bool CKPT, bool GATE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void ssd_fwd(SsdKP p) {
    static_assert((P == 32 || P == 64) && (N == 64 || N == 128), "tile shapes");
    constexpr int PB = P / 16;      // 16-channel blocks
    constexpr int NB = N / 16;      // state blocks
    // LDS row pitches, from measured gfx950 throughput of each access pattern
    // (row r read by lane 16g + r):
    //   16-byte row reads run conflict-free at pitches of 8 (mod 16) dwords,
    //   and at 1.7x the time otherwise;
    //   transposing 8-byte reads (4 rows per 16-lane group) are fast at
    //   most pitches except multiples of 32 dwords;
    //   8-byte row writes are fastest at 2 (mod 4) dwords and 2x slower at
    //   8 (mod 16).
    // B and C are read as 16-byte rows on the hot loop (N + 16: 40 or 72
    // dwords); x is read transposed and written once (P + 8 = 36 dwords for
    // P = 64).
    constexpr int NP = N + 16;      // bf16 pitch of B/C rows (state axis)
    constexpr int XP = P == 64 ? P + 8 : P + 16;  // bf16 pitch of x rows
    constexpr int NS = 8 / PB;      // waves per channel block (state parts)
    constexpr int NW = N / NS;      // states per wave
    constexpr int NH = NW / 16;     // accumulator tiles per wave
    constexpr int NKB = (NW + 31) / 32;  // 32-state k blocks of the carried-state product
    constexpr int TBW = 4 / NS;     // 16-token blocks of y per wave
    static_assert(NS * PB == kWaves && NH >= 1 && TBW >= 1, "wave roles");
    __shared__ __attribute__((aligned(16))) bf16_t C_l[kQ * NP];   // [t][n]
    __shared__ __attribute__((aligned(16))) bf16_t B_l[kQ * NP];   // [s][n]
    __shared__ __attribute__((aligned(16))) bf16_t X_l[kQ * XP];   // [s][p]
    // partial carried-state sums for the other parts' token blocks:
    // [channel block][receiving part][sender slot][block][lane] x 4 floats
    __shared__ __attribute__((aligned(16))) f32x4 Yx_l[PB * NS * (NS > 1 ? NS - 1 : 1) * TBW * 64];
    constexpr int MP = kQ + 8;      // bf16 pitch of M rows
    __shared__ __attribute__((aligned(16))) bf16_t M_l[kQ * MP];   // [t][s], causal (zero above the diagonal)
    __shared__ __attribute__((aligned(16))) float dt_l[kQ];
    __shared__ __attribute__((aligned(16))) float cum_l[kQ];
    __shared__ __attribute__((aligned(16))) float ecum_l[kQ];
    __shared__ __attribute__((aligned(16))) float w_l[kQ];
    __shared__ float elast_l;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int hh = (int)(blockIdx.x % (unsigned)p.H), i = (int)(blockIdx.x / (unsigned)p.H);
    const int grp = hh / p.hpg;
    // this sequence's tokens: [t0, t0 + L) of the token axis
    const SeqSpan span = seq_span(p.cu, i, p.L, p.T);
    const int L = span.len;
    const float Ah = p.A[hh];
    const float Dh = p.has_D ? p.D[hh] : 0.0f;
    const float dtb = p.dt_bias ? p.dt_bias[hh] : 0.0f;
    int r = p.ids[i];
    const bool bad_id = (r < 0) | (r >= p.R);
    const bool bad = bad_id | span.bad;
    if (bad) {
        r = 0;
        if (tid == 0)
            atomicOr(p.err, (bad_id ? (uint32_t)SSM_DEVERR_IDS : 0u) | (span.bad ? (uint32_t)SSM_DEVERR_SEQLENS : 0u));
    }
    // wave w: channel block sp, state part sh (tiles [NH*sh, NH*sh + NH) of
    // 16 states), y token blocks [TBW*sh, TBW*sh + TBW)
    const int sp = wave / NS, sh = wave % NS;
    const int pw = sp * 16;  // first channel of the block
    static_assert(NB == NS * NH, "state parts cover the states");

    // state h^T[n][p]: tile j holds rows n = 16(NH*sh + j) + 4g + r, column p = pw + l16
    f32x4 hacc[NH];
    {
        const float* s0 = p.s + (((int64_t)r * p.H + hh) * P + pw + l16) * N + NH * sh * 16;
#pragma unroll
        for (int j = 0; j < NH; ++j) {
            const float4 v = *reinterpret_cast<const float4*>(s0 + j * 16 + 4 * g4);
            hacc[j] = f32x4{v.x, v.y, v.z, v.w};
            if (bad) hacc[j] = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
        }
    }

    // chunk-based descriptors: rows past the sequence end read as zero / drop stores
    const int64_t xrow = (int64_t)p.H * P * 2;   // bytes between tokens of x / y
    const int64_t brow = (int64_t)p.G * N * 2;   // bytes between tokens of B / C
    const int64_t drow = CKPT ? 2 : (int64_t)p.H * 2;  // bytes between tokens of dt
    const int64_t tok0 = span.t0;
    const char* xg = reinterpret_cast<const char*>(p.x) + (tok0 * p.H + hh) * P * 2;
    const char* bg = reinterpret_cast<const char*>(p.B) + (tok0 * p.G + grp) * N * 2;
    const char* cg = reinterpret_cast<const char*>(p.C) + (tok0 * p.G + grp) * N * 2;
    const char* dg = CKPT ? reinterpret_cast<const char*>(p.dt_t) + ((int64_t)i * p.H + hh) * p.L * 2
                          : reinterpret_cast<const char*>(p.dt) + (tok0 * p.H + hh) * 2;
    char* yg = reinterpret_cast<char*>(p.y) + (tok0 * p.H + hh) * P * 2;
    const char* zg = reinterpret_cast<const char*>(p.z) + (tok0 * p.H + hh) * P * 2;  // GATE only
    auto rsrc = [&](const char* base, int t0, int64_t row) {
        const int rows = L - t0;
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base) + (int64_t)t0 * row, 0,
                                                 rows > 0 ? (int)(rows * row) : 0, 0x00020000);
    };

    const int n_chunks = (L + kQ - 1) / kQ;
    // staging: x, B, C rows by 16-byte chunks
    constexpr int XCH = kQ * P / 8, BCH = kQ * N / 8;     // chunks per chunk-tile
    constexpr int XPER = (XCH + kThreads - 1) / kThreads, BPER = BCH / kThreads;
    static_assert(BPER >= 1 && BCH % kThreads == 0, "staging covers the chunk");
    u32x4 sx[XPER], sb[BPER], sc[BPER];
    uint32_t sdt = 0;
    auto load_chunk = [&](int t0) {
        const auto rx = rsrc(xg, t0, xrow), rb = rsrc(bg, t0, brow), rc = rsrc(cg, t0, brow);
#pragma unroll
        for (int k = 0; k < XPER; ++k) {
            const int e = tid + kThreads * k;
            if (e < XCH)
                sx[k] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)((e / (P / 8)) * xrow) + (e % (P / 8)) * 16, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < BPER; ++k) {
            const int e = tid + kThreads * k;
            const int t = e / (N / 8), part = e % (N / 8);
            sb[k] = __builtin_amdgcn_raw_buffer_load_b128(rb, (int)(t * brow) + part * 16, 0, 0);
            if constexpr (!CKPT) sc[k] = __builtin_amdgcn_raw_buffer_load_b128(rc, (int)(t * brow) + part * 16, 0, 0);
        }
        if (tid < kQ) sdt = __builtin_amdgcn_raw_buffer_load_b16(rsrc(dg, t0, drow), (int)(tid * drow), 0, 0);
    };
    auto store_chunk = [&](int t0) {
#pragma unroll
        for (int k = 0; k < XPER; ++k) {
            const int e = tid + kThreads * k;
            if (e < XCH) *reinterpret_cast<u32x4*>(&X_l[(e / (P / 8)) * XP + (e % (P / 8)) * 8]) = sx[k];
        }
#pragma unroll
        for (int k = 0; k < BPER; ++k) {
            const int e = tid + kThreads * k;
            const int t = e / (N / 8), part = e % (N / 8);
            // states 8*part .. +7 go to their places in the permuted order (spos)
            const int pos = 32 * (part >> 2) + 16 * (part & 1) + 4 * ((part >> 1) & 1);
            *reinterpret_cast<u32x2*>(&B_l[t * NP + pos]) = u32x2{sb[k].x, sb[k].y};
            *reinterpret_cast<u32x2*>(&B_l[t * NP + pos + 8]) = u32x2{sb[k].z, sb[k].w};
            if constexpr (!CKPT) {
                *reinterpret_cast<u32x2*>(&C_l[t * NP + pos]) = u32x2{sc[k].x, sc[k].y};
                *reinterpret_cast<u32x2*>(&C_l[t * NP + pos + 8]) = u32x2{sc[k].z, sc[k].w};
            }
        }
        if (wave == 0) {  // decays of the chunk, lane = token
            float d = to_f32((bf16_t)sdt) + dtb;
            if constexpr (SOFTPLUS) d = softplus(d);
            if (t0 + lane >= L) d = 0.0f;
            const float cum = wave_incl_sum(d * Ah);
            const float last = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, cum), 63));
            dt_l[lane] = d;
            cum_l[lane] = cum;
            ecum_l[lane] = __expf(cum);
            w_l[lane] = __expf(last - cum) * d;
            if (lane == 0) elast_l = __expf(last);
        }
        if constexpr (CKPT) {  // the fp32 state entering this chunk, in the checkpoint piece order
            static_assert(SsdCkptLayout<P, N>::NH == NH && SsdCkptLayout<P, N>::NS == NS, "checkpoint layout");
            float* ck = p.ckpt + (((int64_t)i * p.H + hh) * n_chunks + t0 / kQ) * (P * N);
#pragma unroll
            for (int j = 0; j < NH; ++j)
                *reinterpret_cast<f32x4*>(ck + 4 * SsdCkptLayout<P, N>::piece(wave, j, lane)) = hacc[j];
        }
    };

    // y stores: lane (t = 16tb + l16, channels pw + 4g .. +3), one 8-byte store per token block
    auto yoff = [&](int tb) { return (int)((tb * 16 + l16) * xrow) + (pw + 4 * g4) * 2; };

    // M's tiles above the diagonal are never written: zero the whole tile once
    for (int e = tid; e < kQ * MP / 2; e += kThreads) reinterpret_cast<uint32_t*>(M_l)[e] = 0u;

    load_chunk(0);
    bf16x8 xcol[2];  // x columns p = pw + l16, rows s = 32kk + 8g + j
    for (int ch = 0; ch < n_chunks; ++ch) {
        const int t0 = ch * kQ;
        __syncthreads();  // every wave is done with the previous chunk's tiles
        store_chunk(t0);
        __syncthreads();
        load_chunk(t0 + kQ);  // next chunk (past the end: reads zero, never used)

        if constexpr (!CKPT) {
        // M = G o L on the 10 causal 16x16 tiles, to LDS as bf16.  Tile k (row by
        // row: (tb,sb) = (0,0),(1,0),(1,1),(2,0),...) goes to wave k % 8: every
        // wave has tile k = w, waves 0 and 1 also tile w + 8; their G products
        // run interleaved.
        {
            const bool two = wave + kWaves < 10;
            int mtb[2], msb[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int k = wave + kWaves * u;
                mtb[u] = k < 1 ? 0 : k < 3 ? 1 : k < 6 ? 2 : 3;
                msb[u] = k - mtb[u] * (mtb[u] + 1) / 2;
                if (!two) { mtb[1] = mtb[0]; msb[1] = msb[0]; }
            }
            f32x4 gacc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int kk = 0; kk < N / 32; ++kk) {
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    if (u == 1 && !two) continue;
                    gacc[u] = mfma(ld8(&B_l[(msb[u] * 16 + l16) * NP + kk * 32 + 8 * g4]),
                                   ld8(&C_l[(mtb[u] * 16 + l16) * NP + kk * 32 + 8 * g4]), gacc[u]);
                }
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                if (u == 1 && !two) continue;
                // G^T tile: column t, rows s = 16msb + 4g + r; exponents clamped to <= 0
                // (above the diagonal the product is replaced by 0 anyway)
                const int mt_t = mtb[u] * 16 + l16;
                const float ct = cum_l[mt_t];
                const float4 cs = *reinterpret_cast<const float4*>(&cum_l[msb[u] * 16 + 4 * g4]);
                const float4 ds = *reinterpret_cast<const float4*>(&dt_l[msb[u] * 16 + 4 * g4]);
                const float csv[4] = {cs.x, cs.y, cs.z, cs.w}, dsv[4] = {ds.x, ds.y, ds.z, ds.w};
                float m[4];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int sidx = msb[u] * 16 + 4 * g4 + rr;
                    const float v = gacc[u][rr] * __expf(fminf(ct - csv[rr], 0.0f)) * dsv[rr];
                    m[rr] = sidx <= mt_t ? v : 0.0f;
                }
                const uint32_t lo = uint32_t(bf16_rne(m[0])) | (uint32_t(bf16_rne(m[1])) << 16);
                const uint32_t hi = uint32_t(bf16_rne(m[2])) | (uint32_t(bf16_rne(m[3])) << 16);
                *reinterpret_cast<u32x2*>(&M_l[mt_t * MP + msb[u] * 16 + 4 * g4]) = u32x2{lo, hi};
            }
        }
        // the gate's z of this chunk as whole-line 16-byte pieces (x's
        // staging pattern), issued once the M tiles are done (fewer live
        // registers there); they go to LDS in C's place once every wave is
        // done with C (below)
        u32x4 sz[GATE ? XPER : 1];
        if constexpr (GATE && !CKPT) {
            const auto rz = rsrc(zg, t0, xrow);
#pragma unroll
            for (int k = 0; k < XPER; ++k) {
                const int e = tid + kThreads * k;
                if (e < XCH)
                    sz[k] = __builtin_amdgcn_raw_buffer_load_b128(rz, (int)((e / (P / 8)) * xrow) + (e % (P / 8)) * 16, 0, 0);
            }
        }
        // carried-state product over this wave's state part, for all four token
        // blocks: A = the state as bf16 hi + lo from the accumulators, B = C at
        // the same states (see the header); the other parts' blocks go to LDS
        f32x4 yo[4];
        {
            bf16x8 ahi[NKB], alo[NKB];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int j = 2 * kb + (e >> 2);
                    const float v = j < NH ? hacc[j][e & 3] : 0.0f;
                    const __bf16 hi = (__bf16)v;
                    ahi[kb][e] = hi;
                    alo[kb][e] = (__bf16)(v - (float)hi);
                }
            }
#pragma unroll
            for (int tbk = 0; tbk < 4; ++tbk) {
                yo[tbk] = f32x4{0.f, 0.f, 0.f, 0.f};
                // C at this lane's states: with the permuted order, states
                // 32kb + 4g + r and 32kb + 16 + 4g + r of the part sit side by side
                const bf16_t* crow = &C_l[(tbk * 16 + l16) * NP + spos(NW * sh + 4 * g4)];
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    const bf16x8 cop = 2 * kb + 1 < NH ? ld8(crow + 32 * kb)
                                                       : cat(ld4(crow + 32 * kb), bf16x4{0, 0, 0, 0});
                    yo[tbk] = mfma(ahi[kb], cop, yo[tbk]);
                    yo[tbk] = mfma(alo[kb], cop, yo[tbk]);
                }
            }
        }
        if constexpr (NS > 1) {
#pragma unroll
            for (int tbk = 0; tbk < 4; ++tbk) {
                const int dst = tbk / TBW;
                if (dst == sh) continue;
                const int slot = (sh - dst - 1 + NS) % NS;  // 0 .. NS-2
                Yx_l[(((sp * NS + dst) * (NS - 1) + slot) * TBW + tbk % TBW) * 64 + lane] = yo[tbk];
            }
        }
        __syncthreads();
        // the gate's z tile [t][p] (pitch XP) in C's place, which no wave reads
        // again before the next chunk is staged
        bf16_t* const Z_l = C_l;
        if constexpr (GATE) {
#pragma unroll
            for (int k = 0; k < XPER; ++k) {
                const int e = tid + kThreads * k;
                if (e < XCH) *reinterpret_cast<u32x4*>(&Z_l[(e / (P / 8)) * XP + (e % (P / 8)) * 8]) = sz[k];
            }
            __syncthreads();
        }

        const auto ry = rsrc(yg, t0, xrow);
        // Yd^T = X^T M^T over s for the wave's token blocks (x columns of its
        // channel block, shared by the blocks and by the state update below)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const bf16_t* xr = &X_l[(kk * 32 + 8 * g4 + (l16 >> 2)) * XP + pw + 4 * (l16 & 3)];
            xcol[kk] = cat(ldtr(xr), ldtr(xr + 4 * XP));
        }
#pragma unroll
        for (int q = 0; q < TBW; ++q) {
            const int tb = TBW * sh + q;
            const int t = tb * 16 + l16;
            f32x4 yd = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                if (2 * kk > tb) continue;
                yd = mfma(xcol[kk], ld8(&M_l[t * MP + kk * 32 + 8 * g4]), yd);
            }
            f32x4 yot = yo[0];  // yo[tb], selected with constant indices
#pragma unroll
            for (int k = 1; k < 4; ++k)
                if (k == tb) yot = yo[k];
            if constexpr (NS > 1) {
#pragma unroll
                for (int slot = 0; slot < NS - 1; ++slot)
                    yot += Yx_l[(((sp * NS + sh) * (NS - 1) + slot) * TBW + q) * 64 + lane];
            }
            const float et = ecum_l[t];
            // y[t][p] for p = pw + 4g + r: y = yd + exp(cum_t) yo + D x
            uint32_t packed[2];
            const bf16x4 xv = ld4(&X_l[t * XP + pw + 4 * g4]);
            bf16x4 zq;
            if constexpr (GATE) zq = ld4(&Z_l[t * XP + pw + 4 * g4]);
#pragma unroll
            for (int rr = 0; rr < 4; rr += 2) {
                float y0 = fmaf(Dh, (float)xv[rr], fmaf(et, yot[rr], yd[rr]));
                float y1 = fmaf(Dh, (float)xv[rr + 1], fmaf(et, yot[rr + 1], yd[rr + 1]));
                if constexpr (GATE) {  // y * SiLU(z), rounded once
                    y0 *= silu((float)zq[rr]);
                    y1 *= silu((float)zq[rr + 1]);
                }
                packed[rr / 2] = uint32_t(bf16_rne(y0)) | (uint32_t(bf16_rne(y1)) << 16);
            }
            __builtin_amdgcn_raw_buffer_store_b64(u32x2{packed[0], packed[1]}, ry, yoff(tb), 0, 0);
        }

        }  // !CKPT

        // state of this wave's block: h^T = exp(cum_last) h^T + B^T (w o X)
        {
            const float e_last = elast_l;
            bf16x8 xw[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                if constexpr (CKPT) {  // (the output pass has them already)
                    const bf16_t* xr = &X_l[(kk * 32 + 8 * g4 + (l16 >> 2)) * XP + pw + 4 * (l16 & 3)];
                    xcol[kk] = cat(ldtr(xr), ldtr(xr + 4 * XP));
                }
                const bf16x8 xv = xcol[kk];
                const float4 w0 = *reinterpret_cast<const float4*>(&w_l[kk * 32 + 8 * g4]);
                const float4 w1 = *reinterpret_cast<const float4*>(&w_l[kk * 32 + 8 * g4 + 4]);
                const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
                for (int j = 0; j < 8; ++j) xw[kk][j] = (__bf16)((float)xv[j] * wv[j]);
            }
#pragma unroll
            for (int j = 0; j < NH; ++j) {
                const int nb = NH * sh + j;
                f32x4 a = hacc[j] * e_last;
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    // B column n = 16nb + l16, rows s = 32kk + 8g + j (4 consecutive
                    // states stay consecutive in the permuted order)
                    const bf16_t* br = &B_l[(kk * 32 + 8 * g4 + (l16 >> 2)) * NP + spos(nb * 16 + 4 * (l16 & 3))];
                    a = mfma(cat(ldtr(br), ldtr(br + 4 * NP)), xw[kk], a);
                }
                hacc[j] = a;
            }
        }
    }

    if (!CKPT) {
        float* so = p.state_out + (((int64_t)i * p.H + hh) * P + pw + l16) * N + NH * sh * 16;
#pragma unroll
        for (int j = 0; j < NH; ++j)
            *reinterpret_cast<float4*>(so + j * 16 + 4 * g4) =
                make_float4(hacc[j][0], hacc[j][1], hacc[j][2], hacc[j][3]);
    }
}

template <int P, int N, bool CKPT = false>
int launch_ssd_pn(const SsdKP& kp, int S, bool softplus, hipStream_t st) {
    const dim3 grid((unsigned)((int64_t)kp.H * S));
    if (kp.z && !CKPT) {
        if (softplus) hipLaunchKernelGGL((ssd_fwd<P, N, true, CKPT, true>), grid, dim3(kThreads), 0, st, kp);
        else hipLaunchKernelGGL((ssd_fwd<P, N, false, CKPT, true>), grid, dim3(kThreads), 0, st, kp);
    } else {
        if (softplus) hipLaunchKernelGGL((ssd_fwd<P, N, true, CKPT, false>), grid, dim3(kThreads), 0, st, kp);
        else hipLaunchKernelGGL((ssd_fwd<P, N, false, CKPT, false>), grid, dim3(kThreads), 0, st, kp);
    }
    return hipGetLastError() == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

}  // namespace

bool ssd_supported(const Shape& sh, const FwdArgs& a) {
    auto al16 = [](const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) == 0; };
    // per-sequence byte extents must fit the 31-bit offsets of the buffer descriptors
    const int64_t lim = int64_t(1) << 31;
    return !sh.a_per_state && sh.io == SSM_BF16 && sh.K == 0 && (sh.P == 64 || sh.P == 32) &&
           (sh.N == 128 || sh.N == 64) && al16(a.x) && al16(a.B) && al16(a.C) && al16(a.s) &&
           al16(a.state_out) && (reinterpret_cast<uintptr_t>(a.y) & 7) == 0 &&
           (reinterpret_cast<uintptr_t>(a.z) & 7) == 0 && sh.L > 0 &&
           sh.S * sh.H < lim && sh.L * sh.H * sh.P * 2 < lim && sh.L * sh.G * sh.N * 2 < lim;
}

int launch_ssd_fwd(const FwdArgs& a, hipStream_t stream) {
    const Shape& sh = a.sh;
    SsdKP kp;
    kp.s = a.s; kp.x = static_cast<const bf16_t*>(a.x); kp.dt = static_cast<const bf16_t*>(a.dt);
    kp.A = a.A; kp.B = static_cast<const bf16_t*>(a.B); kp.C = static_cast<const bf16_t*>(a.C);
    kp.D = a.D; kp.ids = a.ids; kp.y = static_cast<bf16_t*>(a.y); kp.state_out = a.state_out;
    kp.ckpt = nullptr; kp.dt_t = nullptr;
    kp.err = a.err;
    kp.dt_bias = a.dt_bias; kp.z = static_cast<const bf16_t*>(a.z); kp.cu = a.cu; kp.T = a.T;
    kp.L = (int)sh.L; kp.H = (int)sh.H; kp.G = (int)sh.G; kp.R = (int)sh.R;
    kp.hpg = (int)(sh.H / sh.G);
    kp.has_D = (sh.flags & SSM_HAS_D) ? 1 : 0;
    const bool sp = (sh.flags & SSM_DT_SOFTPLUS) != 0;
    const int S = (int)sh.S;
    if (sh.P == 64 && sh.N == 128) return launch_ssd_pn<64, 128>(kp, S, sp, stream);
    if (sh.P == 64 && sh.N == 64) return launch_ssd_pn<64, 64>(kp, S, sp, stream);
    if (sh.P == 32 && sh.N == 128) return launch_ssd_pn<32, 128>(kp, S, sp, stream);
    if (sh.P == 32 && sh.N == 64) return launch_ssd_pn<32, 64>(kp, S, sp, stream);
    return SSM_ERR_UNSUPPORTED;
}

// dt [S][L][H] -> dt_t [S][H][L] through an LDS tile of 64 tokens x up to
// 128 heads, so that a chunk's 64 decays of one head are 128 contiguous bytes
// (a column of the token-major dt touches 64 cache lines).  With H <= 128 a
// tile is one contiguous range of dt: every load of a wave reads 128 bytes.
constexpr int kDtTok = 64, kDtHeads = 128;
__global__ __launch_bounds__(256) void ssd_dt_transpose(const uint16_t* __restrict__ dt, uint16_t* __restrict__ dt_t,
                                                        int L, int H) {
    __shared__ uint16_t tile[kDtHeads * (kDtTok + 1)];  // [head][token], rows padded
    const int tiles = (L + kDtTok - 1) / kDtTok;  // blockIdx.x = sequence x token tile, blockIdx.y = head tile
    const int64_t s = blockIdx.x / (unsigned)tiles;
    const int t0 = (int)(blockIdx.x % (unsigned)tiles) * kDtTok, h0 = blockIdx.y * kDtHeads;
    const int ht = min(kDtHeads, H - h0), nt = min(kDtTok, L - t0);
    // every load first (offsets past the tile read zero), then the LDS writes
    const int lim = ((nt - 1) * H + ht) * 2;
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(dt) + (s * L + t0) * H + h0, 0, lim,
                                                      0x00020000);
    constexpr int PER = kDtHeads * kDtTok / 256;
    uint32_t v[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int e = threadIdx.x + 256 * k, t = e / ht, h = e - t * ht;
        v[k] = __builtin_amdgcn_raw_buffer_load_b16(rs, t < nt ? (t * H + h) * 2 : lim, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int e = threadIdx.x + 256 * k, t = e / ht, h = e - t * ht;
        if (t < nt) tile[h * (kDtTok + 1) + t] = (uint16_t)v[k];
    }
    __syncthreads();
    const int c = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int k = 0; k < kDtHeads / 4; ++k) {
        const int h = w + 4 * k;
        if (h < ht && c < nt) dt_t[(s * H + h0 + h) * L + t0 + c] = tile[h * (kDtTok + 1) + c];
    }
}

// The backward's recompute: dt transposed into dt_t [S][H][L] (the backward
// reads it too), then the chunk-entry states of every (sequence, head) into
// ckpt [S][H][n_chunks], each state in the SsdCkptLayout piece order.
int launch_ssd_ckpt(const BwdArgs& a, float* ckpt, uint16_t* dt_t, hipStream_t stream) {
    const Shape& sh = a.sh;
    hipLaunchKernelGGL(ssd_dt_transpose, dim3((unsigned)(sh.S * ((sh.L + kDtTok - 1) / kDtTok)),
                                              (unsigned)((sh.H + kDtHeads - 1) / kDtHeads)),
                       dim3(256), 0, stream, static_cast<const uint16_t*>(a.dt), dt_t, (int)sh.L, (int)sh.H);
    SsdKP kp;
    kp.dt_t = dt_t;
    kp.s = a.s; kp.x = static_cast<const bf16_t*>(a.x); kp.dt = static_cast<const bf16_t*>(a.dt);
    kp.A = a.A; kp.B = static_cast<const bf16_t*>(a.B); kp.C = static_cast<const bf16_t*>(a.C);
    kp.D = a.D; kp.ids = a.ids; kp.y = nullptr; kp.state_out = nullptr; kp.ckpt = ckpt;
    kp.err = a.err;
    kp.dt_bias = nullptr; kp.z = nullptr; kp.cu = nullptr; kp.T = sh.S * sh.L;
    kp.L = (int)sh.L; kp.H = (int)sh.H; kp.G = (int)sh.G; kp.R = (int)sh.R;
    kp.hpg = (int)(sh.H / sh.G);
    kp.has_D = (sh.flags & SSM_HAS_D) ? 1 : 0;
    const bool sp = (sh.flags & SSM_DT_SOFTPLUS) != 0;
    const int S = (int)sh.S;
    if (sh.P == 64 && sh.N == 128) return launch_ssd_pn<64, 128, true>(kp, S, sp, stream);
    if (sh.P == 64 && sh.N == 64) return launch_ssd_pn<64, 64, true>(kp, S, sp, stream);
    if (sh.P == 32 && sh.N == 128) return launch_ssd_pn<32, 128, true>(kp, S, sp, stream);
    if (sh.P == 32 && sh.N == 64) return launch_ssd_pn<32, 64, true>(kp, S, sp, stream);
    return SSM_ERR_UNSUPPORTED;
}

}  // namespace ssm
