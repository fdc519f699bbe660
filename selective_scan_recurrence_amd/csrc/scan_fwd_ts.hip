// Mamba-1 forward for d_state 16 with the time axis split across the waves
// of a workgroup ("time-split quad" layout), gfx950.
//
// Per (sequence i, channel c) the scan is the recurrence of "mambazip
// mamba1/model.rs" (selective_scan_state16): h_n = exp(dt*A_cn) h_n + (u*dt) B_n,
// y = sum_n C_n h_n + D_c u, with u = SiLU(causal conv of x) when the conv is
// fused (ggmlR ssm_conv reference: tap K-1 on the newest input).
//
// A workgroup of J waves owns 16 channels of one sequence and walks the
// sequence in tiles of M*J tokens; wave w takes tokens Mw..Mw+M-1 of each
// tile.  Within a wave four lanes share a channel and each keeps four of the
// 16 states (the quad layout of scan_fwd_quad.hip).  Per tile:
//   1. sweep 1: in each group of four tokens, quad lane q forms the conv,
//      SiLU and dt transform of token q once; the four lanes then form the
//      decays a_t = exp(dt_t A) and input terms b_t = dt_t u_t B_t of all
//      four tokens (dt and dt*u reach them through DPP broadcasts), keep all
//      of them in registers, and scan them from a zero state.  The result is
//      the sub-chunk operator (prod a, local end state): the pair of the
//      associative combine (a, b) o (a', b') = (a a', a' b + b')
//      ("kizzasi-model backprop_ssm.rs", associative scan), with
//      prod a = exp(A sum dt);
//   2. the J operators go through LDS; each wave folds the ones before it
//      onto the state entering the tile, giving its carried-in state;
//   3. sweep 2: each wave replays its tokens from the carried-in state with
//      the decays held in registers (no exp is recomputed) and forms
//      y = C.h + D u with a reduce-scatter across the quad; the last wave's
//      end state enters the next tile.  The next tile's x, dt, B, C, loaded
//      into registers at the end of the previous tile, are then written to
//      the other LDS buffer, the loads of the tile after next are issued, and
//      only then is y stored (stores and loads share one completion counter,
//      so waiting for the loads must not wait for y).
// Two barriers per tile.  Token rows of 16 channels are 64 B (fp32) or 32 B
// (bf16); the workgroup order is remapped so that neighbouring channel blocks
// of one sequence are dispatched to the same XCD and share its L2 lines.
//
// The extras of selective_scan_fwd_ext ride along: the dt bias is added where
// the owner lane reads dt (before the softplus), the owner lane's z values are
// loaded at the start of each tile and scale y by SiLU(z) before its one
// rounding, and with packed sequences each workgroup takes its own span of
// the token axis (its tile count follows the span's length).
#include "device_common.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

// 16 waves of 8 tokens (128-token tiles, 125 VGPRs: four waves per SIMD)
// measured 2.5% faster on 8 x 2048 x 512 than 8 waves of 16 (207 VGPRs, two
// per SIMD); 8 waves of 8 (64-token tiles) was slower than either.
constexpr int kSub = 8;   // tokens per wave per tile
constexpr int kCh = 16;   // channels per workgroup
constexpr int kHalo = 3;  // conv history rows kept ahead of the tile (d_conv <= 4)
constexpr int kJ = 16;    // waves per workgroup

struct TsKP {
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
    // extras of selective_scan_fwd_ext (null: none)
    const float* dt_bias;  // [d_inner], added to dt before the softplus
    const void* z;         // gate, laid out as x: y is multiplied by SiLU(z)
    const int32_t* cu;     // [S+1] spans on the packed token axis
    int64_t T;             // tokens on the packed axis
    int L, d_inner, R, S, ncb;
    int has_D;
    int xcd_swizzle;  // 1: workgroup count is a multiple of 8
};

template <typename T>
__device__ __forceinline__ void unpack_store(float* dst, const uint4& v);
template <>
__device__ __forceinline__ void unpack_store<float>(float* dst, const uint4& v) {
    *reinterpret_cast<uint4*>(dst) = v;
}
template <>
__device__ __forceinline__ void unpack_store<bf16_t>(float* dst, const uint4& v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float f[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        f[2 * k] = __uint_as_float(w[k] << 16);
        f[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
    *reinterpret_cast<float4*>(dst) = make_float4(f[0], f[1], f[2], f[3]);
    *reinterpret_cast<float4*>(dst + 4) = make_float4(f[4], f[5], f[6], f[7]);
}

template <typename T, int K, bool SOFTPLUS, bool GATE, int J, int M>
__global__ __launch_bounds__(64 * J) void ts_fwd(TsKP p) {
    constexpr int NT = 64 * J;
    constexpr int TT = M * J;               // tokens per tile
    constexpr int ES = (int)sizeof(T);
    constexpr int CPR = kCh * ES / 16;      // 16-byte chunks per row of 16 values
    constexpr int VPC = 16 / ES;            // values per chunk
    constexpr int CH_ARR = TT * CPR;        // chunks per array per tile
    constexpr int XR = TT + kHalo;          // x rows per buffer (history rows first)
    static_assert(M % 4 == 0, "sub-chunks are whole groups of four tokens");

    // two tile buffers: tile t+1 is written while tile t is still being read
    __shared__ __attribute__((aligned(16))) float xs_l[2][XR * kCh];
    __shared__ __attribute__((aligned(16))) float dt_l[2][TT * kCh];
    __shared__ __attribute__((aligned(16))) float B_l[2][TT * 16];
    __shared__ __attribute__((aligned(16))) float C_l[2][TT * 16];
    __shared__ __attribute__((aligned(16))) float agg_l[J][2][kCh * 16];  // (prod a, local end)
    __shared__ __attribute__((aligned(16))) float hT_l[2][kCh * 16];      // state entering the tile

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int cl = lane >> 2, q = lane & 3;
    int b = blockIdx.x;
    if (p.xcd_swizzle) {
        const int per = (int)(gridDim.x >> 3);
        b = (b & 7) * per + (b >> 3);
    }
    const int i = b / p.ncb, c0 = (b % p.ncb) * kCh;
    const int c = c0 + cl;
    const int d_inner = p.d_inner;
    // this sequence's tokens: [t0, t0 + L) of the token axis (an invalid span
    // scans nothing and ends in a NaN state)
    const SeqSpan span = seq_span(p.cu, i, p.L, p.T);
    const int L = span.len;

    int r = p.ids[i];
    const bool bad_id = (r < 0) | (r >= p.R);
    const bool bad = bad_id | span.bad;
    if (bad) {
        r = 0;
        if (tid == 0)
            atomicOr(p.err, (bad_id ? (uint32_t)SSM_DEVERR_IDS : 0u) | (span.bad ? (uint32_t)SSM_DEVERR_SEQLENS : 0u));
    }

    float a2[4];
    {
        const float4 Av = *reinterpret_cast<const float4*>(p.A + (int64_t)c * 16 + 4 * q);
        a2[0] = Av.x * kLog2e; a2[1] = Av.y * kLog2e; a2[2] = Av.z * kLog2e; a2[3] = Av.w * kLog2e;
    }
    if (wave == 0) {
        float4 hv = *reinterpret_cast<const float4*>(p.s + ((int64_t)r * d_inner + c) * 16 + 4 * q);
        if (bad) hv = make_float4(__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""));
        *reinterpret_cast<float4*>(&hT_l[0][cl * 16 + 4 * q]) = hv;
    }
    const float Dc = p.has_D ? p.D[c] : 0.0f;
    const float dtb = p.dt_bias ? p.dt_bias[c] : 0.0f;
    float w[4] = {0.f, 0.f, 0.f, 0.f};
    if constexpr (K > 0) {
#pragma unroll
        for (int j = 0; j < K; ++j) w[j] = p.conv_w[(int64_t)c * K + j];
    }
    // conv history entering the sequence: the K-1 entries of the gathered conv state
    if constexpr (K > 1) {
        if (tid < kHalo * kCh) {
            const int row = tid / kCh, cc = tid % kCh;
            const int jj = row - kHalo + (K - 1);  // index into the conv state, or < 0
            float v = 0.0f;
            if (jj >= 0) {
                if (bad) v = __builtin_nanf("");
                else if (p.conv_state) v = p.conv_state[((int64_t)r * d_inner + c0 + cc) * (K - 1) + jj];
            }
            xs_l[0][row * kCh + cc] = v;
        }
    }

    // All tile traffic goes through buffer descriptors whose base is the
    // tile's first row and whose size ends at the sequence's last token:
    // the per-lane offsets stay the same on every tile (no address register
    // is rewritten while a store from it may be in flight), rows past the
    // end read as zero and stores past it are dropped by the hardware.
    const int64_t tok0 = span.t0;
    const char* xg = static_cast<const char*>(p.x) + (tok0 * d_inner + c0) * ES;
    const char* dg = static_cast<const char*>(p.dt) + (tok0 * d_inner + c0) * ES;
    const char* bg = static_cast<const char*>(p.B) + tok0 * 16 * ES;
    const char* cg = static_cast<const char*>(p.C) + tok0 * 16 * ES;
    char* yg = static_cast<char*>(p.y) + (tok0 * d_inner + c0) * ES;
    const char* zg = GATE ? static_cast<const char*>(p.z) + (tok0 * d_inner + c0) * ES : nullptr;
    const int xrow = d_inner * ES;  // bytes between token rows of x, dt, y (bounded on the host)
    // a descriptor spans at most the TT rows of one tile (the loads and y
    // stores through it never reach further), so its size stays below 2^31
    // however long the sequence is
    auto rsrc = [&](const char* base, int tb, int row_bytes) {
        const int rows = min(L - tb, TT);
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base) + (int64_t)tb * row_bytes, 0,
                                                 rows > 0 ? rows * row_bytes : 0, 0x00020000);
    };

    // Staging of one tile: x, dt, B, C are four arrays of TT rows x 16 values
    // (CH_ARR 16-byte chunks each).  With CH_ARR >= NT every thread loads
    // each array; with fewer, the threads split into NG groups of CH_ARR and
    // group j loads arrays j, j + NG, ...
    constexpr int NG = CH_ARR < NT ? NT / CH_ARR : 1;
    static_assert(NG == 1 ? CH_ARR % NT == 0 : (NG * CH_ARR == NT && 4 % NG == 0),
                  "whole chunks per thread");
    constexpr int KA = NG == 1 ? CH_ARR / NT : 1;  // chunks per array per thread
    constexpr int NA = 4 / NG;                     // arrays per thread
    // wave-uniform (CH_ARR is a multiple of 64); readfirstlane tells the compiler
    // so, which keeps the buffer descriptors in scalar registers
    const int grp = NG == 1 ? 0 : __builtin_amdgcn_readfirstlane(tid / CH_ARR);
    const int te = NG == 1 ? tid : tid % CH_ARR;
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    u32x4 stg[NA][KA];
    auto arr_of = [&](int a) { return grp + NG * a; };
    auto load_tile = [&](int tb) {
#pragma unroll
        for (int a = 0; a < NA; ++a) {
            const int arr = arr_of(a);
            const int rb = arr < 2 ? xrow : 16 * ES;
            const auto rs = rsrc(arr == 0 ? xg : arr == 1 ? dg : arr == 2 ? bg : cg, tb, rb);
#pragma unroll
            for (int k = 0; k < KA; ++k) {
                const int e = te + NT * k;
                const int row = e / CPR, part = e % CPR;
                stg[a][k] = __builtin_amdgcn_raw_buffer_load_b128(rs, row * rb + part * 16, 0, 0);
            }
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int a = 0; a < NA; ++a) {
            const int arr = arr_of(a);
            float* dstb = arr == 0 ? xs_l[buf] + kHalo * kCh : arr == 1 ? dt_l[buf] : arr == 2 ? B_l[buf] : C_l[buf];
#pragma unroll
            for (int k = 0; k < KA; ++k) {
                const int e = te + NT * k;
                const int row = e / CPR, part = e % CPR;
                const uint4 v = make_uint4(stg[a][k].x, stg[a][k].y, stg[a][k].z, stg[a][k].w);
                unpack_store<T>(dstb + row * 16 + part * VPC, v);
            }
        }
    };
    // byte offset of this lane's y element for group g, within a tile
    auto y_off = [&](int g) { return (wave * M + 4 * g + q) * xrow + cl * ES; };

    const int n_tiles = (L + TT - 1) / TT;
    uint32_t ykeep[M / 4] = {};  // data registers of the y stores in flight
    // unconditional even with no tokens: every row is then past the end and
    // reads as zero (no branch around the loads keeps the compiler's wait
    // bookkeeping exact across the tile loop)
    load_tile(0);
    store_tile(0);
    load_tile(TT);
    __syncthreads();
    for (int tile = 0; tile < n_tiles; ++tile) {
        const int tb = tile * TT, buf = tile & 1;
        const float* xs = xs_l[buf];
        const float* dts = dt_l[buf];
        const float* Bs_l = B_l[buf];
        const float* Cs_l = C_l[buf];
        // the gate's z at this lane's y positions, needed only at the y stores
        uint32_t zv[GATE ? M / 4 : 1];
        if constexpr (GATE) {
            const auto rz = rsrc(zg, tb, xrow);
#pragma unroll
            for (int g = 0; g < M / 4; ++g) {
                if constexpr (ES == 2)
                    zv[g] = __builtin_amdgcn_raw_buffer_load_b16(rz, y_off(g), 0, 0);
                else
                    zv[g] = __builtin_amdgcn_raw_buffer_load_b32(rz, y_off(g), 0, 0);
            }
        }

        // sweep 1: lane q owns token 4g+q of each group: conv + SiLU, dt; the
        // quad's four lanes then form decays and input terms of all four tokens
        const int tw = wave * M;
        float dec[M][4], inp[M][4], hl[4] = {0.f, 0.f, 0.f, 0.f};
        float u_own[M / 4];
        float sdt = 0.0f;
#pragma unroll
        for (int g = 0; g < M / 4; ++g) {
            const int row = tw + 4 * g + q;
            float u;
            if constexpr (K > 0) {
                float cv = 0.0f;
#pragma unroll
                for (int j = 0; j < K; ++j) cv = fmaf(w[j], xs[(kHalo + row - (K - 1) + j) * kCh + cl], cv);
                u = silu(cv);
            } else {
                u = xs[(kHalo + row) * kCh + cl];
            }
            float d = dts[row * kCh + cl] + dtb;
            if constexpr (SOFTPLUS) d = softplus(d);
            if (tb + row >= L) { d = 0.0f; u = 0.0f; }
            u_own[g] = u;
            sdt += d;
            const float du = d * u;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                float dk, bk;
                if (kk == 0) { dk = quad_bcast<0>(d); bk = quad_bcast<0>(du); }
                if (kk == 1) { dk = quad_bcast<1>(d); bk = quad_bcast<1>(du); }
                if (kk == 2) { dk = quad_bcast<2>(d); bk = quad_bcast<2>(du); }
                if (kk == 3) { dk = quad_bcast<3>(d); bk = quad_bcast<3>(du); }
                const int k = 4 * g + kk;
                const float4 Bv = *reinterpret_cast<const float4*>(&Bs_l[(tw + k) * 16 + 4 * q]);
                const float Bq[4] = {Bv.x, Bv.y, Bv.z, Bv.w};
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    dec[k][s] = fast_exp2(dk * a2[s]);
                    inp[k][s] = bk * Bq[s];
                    hl[s] = fmaf(dec[k][s], hl[s], inp[k][s]);
                }
            }
        }
        sdt += quad_xor1(sdt);
        sdt += quad_xor2(sdt);
        *reinterpret_cast<float4*>(&agg_l[wave][0][cl * 16 + 4 * q]) =
            make_float4(fast_exp2(a2[0] * sdt), fast_exp2(a2[1] * sdt), fast_exp2(a2[2] * sdt),
                        fast_exp2(a2[3] * sdt));
        *reinterpret_cast<float4*>(&agg_l[wave][1][cl * 16 + 4 * q]) = make_float4(hl[0], hl[1], hl[2], hl[3]);
        __syncthreads();

        // carried-in state of this wave's sub-chunk: fold the operators before it
        float h[4];
        {
            const float4 hv = *reinterpret_cast<const float4*>(&hT_l[buf][cl * 16 + 4 * q]);
            h[0] = hv.x; h[1] = hv.y; h[2] = hv.z; h[3] = hv.w;
        }
        for (int j = 0; j < wave; ++j) {
            const float4 Pv = *reinterpret_cast<const float4*>(&agg_l[j][0][cl * 16 + 4 * q]);
            const float4 Hv = *reinterpret_cast<const float4*>(&agg_l[j][1][cl * 16 + 4 * q]);
            h[0] = fmaf(Pv.x, h[0], Hv.x);
            h[1] = fmaf(Pv.y, h[1], Hv.y);
            h[2] = fmaf(Pv.z, h[2], Hv.z);
            h[3] = fmaf(Pv.w, h[3], Hv.w);
        }
        // sweep 2: replay from the carried-in state; y for token 4g+q lands on lane q
        float y_own[M / 4];
#pragma unroll
        for (int g = 0; g < M / 4; ++g) {
            float yp[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int k = 4 * g + kk;
#pragma unroll
                for (int s = 0; s < 4; ++s) h[s] = fmaf(dec[k][s], h[s], inp[k][s]);
                const float4 Cv = *reinterpret_cast<const float4*>(&Cs_l[(tw + k) * 16 + 4 * q]);
                yp[kk] = fmaf(Cv.w, h[3], fmaf(Cv.z, h[2], fmaf(Cv.y, h[1], Cv.x * h[0])));
            }
            const bool hi2 = (q & 2) != 0;
            const float keep0 = hi2 ? yp[2] : yp[0], send0 = hi2 ? yp[0] : yp[2];
            const float keep1 = hi2 ? yp[3] : yp[1], send1 = hi2 ? yp[1] : yp[3];
            const float r0 = keep0 + quad_xor2(send0);
            const float r1 = keep1 + quad_xor2(send1);
            const bool hi1 = (q & 1) != 0;
            const float keep = hi1 ? r1 : r0, send = hi1 ? r0 : r1;
            y_own[g] = fmaf(Dc, u_own[g], keep + quad_xor1(send));
        }
        // the next tile's buffer: its rows, and the last three x rows of this tile as history
        store_tile(buf ^ 1);
        if constexpr (K > 1) {
            if (tid < kHalo * kCh) xs_l[buf ^ 1][tid] = xs[TT * kCh + tid];
        }
        // the tile after next is fetched now and lands during the next tile;
        // it is fetched on every tile (the last ones included: rows past the
        // end read as zero) so that no branch stands between loads and use
        load_tile(tb + 2 * TT);
        // y goes out after the loads, so that waiting for them never waits
        // for this tile's stores; tokens past the end fall outside the
        // descriptor and are dropped
        {
            const auto ry = rsrc(yg, tb, xrow);
#pragma unroll
            for (int g = 0; g < M / 4; ++g) {
                // the previous tile's store data stay reserved up to here; the
                // new data go to the same registers
                float yv = y_own[g];
                if constexpr (GATE) {  // y * SiLU(z), rounded once
                    const float zf = ES == 2 ? __uint_as_float(zv[g] << 16) : __uint_as_float(zv[g]);
                    yv *= silu(zf);
                }
                uint32_t v = ES == 2 ? (uint32_t)bf16_rne(yv) : __float_as_uint(yv);
                asm volatile("v_mov_b32 %0, %1" : "+v"(ykeep[g]) : "v"(v));
                if constexpr (ES == 2)
                    __builtin_amdgcn_raw_buffer_store_b16((unsigned short)ykeep[g], ry, y_off(g), 0, 0);
                else
                    __builtin_amdgcn_raw_buffer_store_b32(ykeep[g], ry, y_off(g), 0, 0);
            }
        }
        // the last sub-chunk's end state enters the next tile
        if (wave == J - 1)
            *reinterpret_cast<float4*>(&hT_l[buf ^ 1][cl * 16 + 4 * q]) = make_float4(h[0], h[1], h[2], h[3]);
        __syncthreads();
    }

    if (wave == 0) {
        *reinterpret_cast<float4*>(p.state_out + ((int64_t)i * d_inner + c) * 16 + 4 * q) =
            *reinterpret_cast<const float4*>(&hT_l[n_tiles & 1][cl * 16 + 4 * q]);
    }
    if constexpr (K > 1) {
        if (p.conv_state_out && tid < kCh * (K - 1)) {
            const int cc = tid % kCh, j = tid / kCh;
            const int tau = L - (K - 1) + j;
            float v;
            if (tau >= 0) v = to_f32(*reinterpret_cast<const T*>(xg + (int64_t)tau * xrow + cc * ES));
            else if (bad) v = __builtin_nanf("");
            else v = p.conv_state ? p.conv_state[((int64_t)r * d_inner + c0 + cc) * (K - 1) + tau + K - 1]
                                  : 0.0f;
            p.conv_state_out[((int64_t)i * d_inner + c0 + cc) * (K - 1) + j] = v;
        }
    }
}

template <typename T, int K>
int launch_ts_k(const TsKP& kp, bool softplus, hipStream_t st) {
    const dim3 grid((unsigned)(kp.S * kp.ncb)), block(64 * kJ);
    if (kp.z) {
        if (softplus) hipLaunchKernelGGL((ts_fwd<T, K, true, true, kJ, kSub>), grid, block, 0, st, kp);
        else hipLaunchKernelGGL((ts_fwd<T, K, false, true, kJ, kSub>), grid, block, 0, st, kp);
    } else {
        if (softplus) hipLaunchKernelGGL((ts_fwd<T, K, true, false, kJ, kSub>), grid, block, 0, st, kp);
        else hipLaunchKernelGGL((ts_fwd<T, K, false, false, kJ, kSub>), grid, block, 0, st, kp);
    }
    return hipGetLastError() == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

}  // namespace

bool ts_supported(const Shape& sh, const FwdArgs& a) {
    auto al16 = [](const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) == 0; };
    return sh.a_per_state && sh.P == 1 && sh.N == 16 && sh.G == 1 &&
           (sh.K == 0 || sh.K == 2 || sh.K == 3 || sh.K == 4) && sh.d_inner() % kCh == 0 &&
           al16(a.x) && al16(a.dt) && al16(a.B) && al16(a.C) && al16(a.y) && al16(a.A) &&
           al16(a.s) && al16(a.state_out) && al16(a.z) && sh.S * (sh.d_inner() / kCh) < (int64_t(1) << 31) &&
           // one tile's rows of x/dt/y (kJ * kSub tokens plus the descriptor's
           // reach) must fit the 31-bit byte sizes and offsets of a descriptor
           sh.d_inner() * sh.io_bytes() * (kJ * kSub + kHalo + 1) < (int64_t(1) << 31);
}

int launch_ts_fwd(const FwdArgs& a, hipStream_t stream) {
    const Shape& sh = a.sh;
    TsKP kp;
    kp.s = a.s; kp.x = a.x; kp.dt = a.dt; kp.A = a.A; kp.B = a.B; kp.C = a.C; kp.D = a.D;
    kp.ids = a.ids; kp.conv_w = a.conv_w; kp.conv_state = a.conv_state; kp.y = a.y;
    kp.state_out = a.state_out; kp.conv_state_out = a.conv_state_out; kp.err = a.err;
    kp.dt_bias = a.dt_bias; kp.z = a.z; kp.cu = a.cu; kp.T = a.T;
    kp.L = (int)sh.L; kp.d_inner = (int)sh.d_inner(); kp.R = (int)sh.R; kp.S = (int)sh.S;
    kp.ncb = (int)(sh.d_inner() / kCh);
    kp.has_D = (sh.flags & SSM_HAS_D) ? 1 : 0;
    const int64_t nwg = sh.S * kp.ncb;
    kp.xcd_swizzle = (nwg % 8 == 0) ? 1 : 0;
    const bool sp = (sh.flags & SSM_DT_SOFTPLUS) != 0;
    const bool bf = sh.io == SSM_BF16;
    switch (sh.K) {
        case 0: return bf ? launch_ts_k<bf16_t, 0>(kp, sp, stream) : launch_ts_k<float, 0>(kp, sp, stream);
        case 2: return bf ? launch_ts_k<bf16_t, 2>(kp, sp, stream) : launch_ts_k<float, 2>(kp, sp, stream);
        case 3: return bf ? launch_ts_k<bf16_t, 3>(kp, sp, stream) : launch_ts_k<float, 3>(kp, sp, stream);
        case 4: return bf ? launch_ts_k<bf16_t, 4>(kp, sp, stream) : launch_ts_k<float, 4>(kp, sp, stream);
        default: return SSM_ERR_UNSUPPORTED;
    }
}

}  // namespace ssm
