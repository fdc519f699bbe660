// The C ABI of libssm.so (declared in include/ssm.h): argument checks on the
// host, packed-buffer arithmetic, and dispatch to the kernel launchers.
// Nothing here reads device memory or allocates.
#include <limits.h>
#include <string.h>

#include <mutex>

#include "ssm_internal.h"

namespace ssm {
namespace {

bool mul_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_mul_overflow(a, b, out); }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }  // NULL passes

// Validates a descriptor and expands it.  Every size the kernels index with
// 32-bit arithmetic is bounded here.
int check_desc(const ssm_scan_desc* d, Shape* out) {
    if (!d) return SSM_ERR_NULL;
    if (d->reserved != 0) return SSM_ERR_SHAPE;
    if (d->io_dtype != SSM_F32 && d->io_dtype != SSM_BF16) return SSM_ERR_DTYPE;
    if (d->n_seqs < 0 || d->n_tokens < 0 || d->n_head < 1 || d->head_dim < 1 || d->d_state < 1 ||
        d->d_state > 256 || d->n_group < 1 || d->n_state_rows < 1 || d->chunk < 0)
        return SSM_ERR_SHAPE;
    if (d->n_head % d->n_group) return SSM_ERR_SHAPE;
    if (d->a_per_state != 0 && d->a_per_state != 1) return SSM_ERR_SHAPE;
    if (d->d_conv < 0 || d->d_conv > 8) return SSM_ERR_SHAPE;
    if (d->d_conv > 0 && d->head_dim != 1) return SSM_ERR_SHAPE;
    if (d->flags & ~(uint32_t)(SSM_HAS_D | SSM_DT_SOFTPLUS)) return SSM_ERR_SHAPE;
    Shape s;
    s.S = d->n_seqs; s.L = d->n_tokens; s.H = d->n_head; s.P = d->head_dim; s.N = d->d_state;
    s.G = d->n_group; s.R = d->n_state_rows; s.a_per_state = d->a_per_state; s.K = d->d_conv;
    s.chunk = d->chunk; s.io = d->io_dtype; s.flags = d->flags;
    int64_t din, per_seq, t1, t2, t3;
    // per-sequence element counts must fit in int32 (kernels index within a
    // sequence with 32-bit offsets); totals must fit in int64 bytes.
    if (!mul_ok(s.H, s.P, &din) || din > INT_MAX) return SSM_ERR_SHAPE;
    if (!mul_ok(s.L, din, &per_seq) || per_seq > INT_MAX) return SSM_ERR_SHAPE;
    if (!mul_ok(s.L, s.G * s.N, &t1) || t1 > INT_MAX) return SSM_ERR_SHAPE;
    if (!mul_ok(per_seq, s.S, &t2) || !mul_ok(t2, 4, &t3)) return SSM_ERR_SHAPE;
    if (!mul_ok(din * s.N, s.R > s.S ? s.R : s.S, &t2) || !mul_ok(t2, 4, &t3)) return SSM_ERR_SHAPE;
    if (!mul_ok(t1, s.S, &t2) || !mul_ok(t2, 4, &t3)) return SSM_ERR_SHAPE;
    if (s.R > INT_MAX) return SSM_ERR_SHAPE;
    *out = s;
    return SSM_OK;
}

size_t out_bytes(const Shape& s) {
    return (size_t)s.nelem_x() * s.io_bytes() + (size_t)s.nelem_state() * 4;
}

size_t state_offset(const Shape& s) { return (size_t)s.nelem_x() * s.io_bytes(); }

// Blocks of the packed gradient: d_s, d_x, d_dt, d_A, d_B, d_C, d_D, then
// with the fused conv d_conv_w and d_conv_state.
void dgrad_layout9(const Shape& s, size_t off[9], size_t* total) {
    size_t o = 0;
    const int64_t K = s.K;
    const int64_t sizes[9] = {s.R * s.H * s.P * s.N, s.nelem_x(), s.S * s.L * s.H, s.nelem_A(),
                              s.nelem_BC(), s.nelem_BC(), (s.flags & SSM_HAS_D) ? s.H : 0,
                              K > 0 ? s.H * K : 0, K > 1 ? s.R * s.H * (K - 1) : 0};
    for (int k = 0; k < 9; ++k) {
        off[k] = o;
        o += (size_t)sizes[k] * 4;
    }
    *total = o;
}

void dgrad_layout(const Shape& s, size_t off[7]) {
    size_t o9[9], total;
    dgrad_layout9(s, o9, &total);
    memcpy(off, o9, 7 * sizeof(size_t));
}

size_t dgrad_total(const Shape& s) {
    size_t off[9], total;
    dgrad_layout9(s, off, &total);
    return total;
}

size_t workspace_bytes(const Shape& s, int backward) {
    size_t body = backward ? bwd_workspace_bytes(s) : fwd_workspace_bytes(s);
    return kErrBytes + align_up(body, 256);
}

}  // namespace
}  // namespace ssm

using namespace ssm;

extern "C" {

const char* ssm_status_str(int status) {
    switch (status) {
        case SSM_OK: return "ok";
        case SSM_ERR_NULL: return "a required pointer is NULL";
        case SSM_ERR_SHAPE: return "a dimension is out of range or inconsistent";
        case SSM_ERR_DTYPE: return "unknown io dtype";
        case SSM_ERR_UNSUPPORTED: return "no kernel for this combination";
        case SSM_ERR_WORKSPACE: return "workspace missing or too small";
        case SSM_ERR_ALIGN: return "misaligned pointer";
        case SSM_ERR_HIP: return "HIP launch error";
        default: return "unknown status";
    }
}

int ssm_version(void) { return 100; }

size_t ssm_scan_out_bytes(const ssm_scan_desc* desc) {
    Shape s;
    return check_desc(desc, &s) == SSM_OK ? out_bytes(s) : 0;
}

size_t ssm_scan_state_offset_bytes(const ssm_scan_desc* desc) {
    Shape s;
    return check_desc(desc, &s) == SSM_OK ? state_offset(s) : 0;
}

size_t ssm_scan_dgrad_layout(const ssm_scan_desc* desc, size_t offsets[7]) {
    Shape s;
    if (check_desc(desc, &s) != SSM_OK) return 0;
    size_t off[7];
    dgrad_layout(s, off);
    if (offsets) memcpy(offsets, off, sizeof off);
    return dgrad_total(s);
}

size_t ssm_scan_workspace_bytes(const ssm_scan_desc* desc, int backward) {
    Shape s;
    return check_desc(desc, &s) == SSM_OK ? workspace_bytes(s, backward) : 0;
}

int ssm_conv_fwd(const void* sx, const float* w, void* out, int64_t n_s, int64_t n_t,
                 int64_t d_inner, int32_t d_conv, int32_t io_dtype, int32_t apply_silu,
                 ssm_stream_t stream) {
    if (io_dtype != SSM_F32 && io_dtype != SSM_BF16) return SSM_ERR_DTYPE;
    if (n_s < 0 || n_t < 0 || d_inner < 1 || d_conv < 1 || d_conv > 8) return SSM_ERR_SHAPE;
    if (n_s > 65535) return SSM_ERR_SHAPE;
    int64_t len = d_conv - 1 + n_t, t1, t2;
    if (!mul_ok(len, d_inner, &t1) || t1 > INT_MAX || !mul_ok(t1, n_s, &t2)) return SSM_ERR_SHAPE;
    // per-sequence byte extents, with a margin of one channel block and one
    // tile, must fit the 31-bit offsets of the kernel's buffer descriptors
    if (!mul_ok(len + 128, d_inner + 64, &t1) || t1 > (INT_MAX >> 2)) return SSM_ERR_SHAPE;
    if (!sx || !w || !out) return SSM_ERR_NULL;
    const size_t es = io_dtype == SSM_BF16 ? 2 : 4;
    if (!aligned(sx, es) || !aligned(out, es) || !aligned(w, 4)) return SSM_ERR_ALIGN;
    return launch_conv_fwd(sx, w, out, n_s, n_t, d_inner, d_conv, io_dtype, apply_silu,
                           static_cast<hipStream_t>(stream));
}

size_t ssm_conv_bwd_workspace_bytes(int64_t n_s, int64_t n_t, int64_t d_inner, int32_t d_conv) {
    if (n_s < 0 || n_t < 0 || d_inner < 1 || d_conv < 1 || d_conv > 8 || n_s > 65535) return 0;
    int64_t len = d_conv - 1 + n_t, t1, t2;
    if (!mul_ok(len, d_inner, &t1) || t1 > INT_MAX || !mul_ok(t1, n_s, &t2)) return 0;
    return conv_bwd_workspace_bytes(n_s, n_t, d_inner, d_conv);
}

int ssm_conv_bwd(const void* sx, const float* w, const float* dout, float* dgrad, int64_t n_s,
                 int64_t n_t, int64_t d_inner, int32_t d_conv, int32_t io_dtype, int32_t apply_silu,
                 void* workspace, size_t workspace_bytes_, ssm_stream_t stream) {
    if (io_dtype != SSM_F32 && io_dtype != SSM_BF16) return SSM_ERR_DTYPE;
    if (n_s < 0 || n_t < 0 || d_inner < 1 || d_conv < 1 || d_conv > 8) return SSM_ERR_SHAPE;
    if (n_s > 65535) return SSM_ERR_SHAPE;
    int64_t len = d_conv - 1 + n_t, t1, t2;
    if (!mul_ok(len, d_inner, &t1) || t1 > INT_MAX || !mul_ok(t1, n_s, &t2)) return SSM_ERR_SHAPE;
    // per-sequence byte extents, with a margin of one channel block and one
    // tile and its staged rows, must fit the 31-bit offsets of the kernel's buffer descriptors
    if (!mul_ok(len + 128, d_inner + 64, &t1) || t1 > (INT_MAX >> 2)) return SSM_ERR_SHAPE;
    // sx and dout may be NULL only when they have no elements
    if (!w || !dgrad || (!sx && n_s * len > 0) || (!dout && n_s * n_t > 0)) return SSM_ERR_NULL;
    const size_t need = conv_bwd_workspace_bytes(n_s, n_t, d_inner, d_conv);
    if (need && !workspace) return SSM_ERR_NULL;
    if (workspace_bytes_ < need) return SSM_ERR_WORKSPACE;
    const size_t es = io_dtype == SSM_BF16 ? 2 : 4;
    if (!aligned(sx, es) || !aligned(w, 4) || !aligned(dout, 4) || !aligned(dgrad, 4) ||
        (need && !aligned(workspace, 4)))
        return SSM_ERR_ALIGN;
    return launch_conv_bwd(sx, w, dout, dgrad, n_s, n_t, d_inner, d_conv, io_dtype, apply_silu,
                           workspace, static_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace ssm {
namespace {

// Checks the extras against the descriptor and gives the packed token count.
int check_ext(const Shape& sh, const ssm_scan_ext* ext, int64_t* T) {
    *T = sh.S * sh.L;
    if (!ext) return SSM_OK;
    if (!ext->cu_seqlens) return ext->total_tokens == 0 ? SSM_OK : SSM_ERR_SHAPE;
    int64_t t1, t2;
    if (ext->total_tokens < 0 || !mul_ok(ext->total_tokens, sh.d_inner(), &t1) ||
        !mul_ok(t1, 4, &t2) || !mul_ok(ext->total_tokens, sh.G * sh.N * 4, &t2))
        return SSM_ERR_SHAPE;
    *T = ext->total_tokens;
    return SSM_OK;
}

int fwd_impl(const ssm_scan_desc* desc, const ssm_scan_ext* ext, const float* s, const void* x,
             const void* dt, const float* A, const void* B, const void* C, const float* D,
             const int32_t* ids, const float* conv_w, const float* conv_state, void* out,
             float* conv_state_out, void* workspace, size_t workspace_bytes_, hipStream_t stream,
             uint32_t* err_word = nullptr) {
    Shape sh;
    int rc = check_desc(desc, &sh);
    if (rc) return rc;
    if (sh.S > 65535) return SSM_ERR_SHAPE;  // grid y
    int64_t T;
    if ((rc = check_ext(sh, ext, &T))) return rc;
    const int32_t* cu = ext ? ext->cu_seqlens : nullptr;
    const void* z = ext ? ext->z : nullptr;
    // a pointer may be NULL only when its tensor has no elements
    const bool has_x = T * sh.d_inner() > 0, has_bc = T * sh.G * sh.N > 0, has_seq = sh.S > 0;
    if (!s || !A || !workspace || (has_x && (!x || !dt)) || (has_bc && (!B || !C)) ||
        (has_seq && (!ids || !out)))
        return SSM_ERR_NULL;
    if ((sh.flags & SSM_HAS_D) && !D) return SSM_ERR_NULL;
    if (sh.K > 0 && !conv_w) return SSM_ERR_NULL;
    if (workspace_bytes_ < workspace_bytes(sh, 0)) return SSM_ERR_WORKSPACE;
    const size_t es = sh.io_bytes();
    if (!aligned(x, es) || !aligned(dt, es) || !aligned(B, es) || !aligned(C, es) ||
        !aligned(out, es) || !aligned(s, 4) || !aligned(A, 4) || !aligned(ids, 4) ||
        (D && !aligned(D, 4)) || (conv_w && !aligned(conv_w, 4)) ||
        (conv_state && !aligned(conv_state, 4)) || (conv_state_out && !aligned(conv_state_out, 4)) ||
        !aligned(workspace, 256) || !aligned(z, es) || (ext && !aligned(ext->dt_bias, 4)) ||
        !aligned(cu, 4) || !aligned(err_word, 4))
        return SSM_ERR_ALIGN;
    char* state_block = static_cast<char*>(out) + (size_t)(T * sh.d_inner()) * es;
    if (!aligned(state_block, 4)) return SSM_ERR_ALIGN;
    FwdArgs a;
    a.sh = sh; a.s = s; a.x = x; a.dt = dt; a.A = A; a.B = B; a.C = C;
    a.D = (sh.flags & SSM_HAS_D) ? D : nullptr;
    a.ids = ids; a.conv_w = sh.K ? conv_w : nullptr; a.conv_state = sh.K ? conv_state : nullptr;
    a.y = out; a.state_out = reinterpret_cast<float*>(state_block);
    a.conv_state_out = sh.K ? conv_state_out : nullptr;
    a.err = err_word ? err_word : static_cast<uint32_t*>(workspace);
    a.ws = static_cast<char*>(workspace) + kErrBytes;
    a.ws_bytes = workspace_bytes_ - kErrBytes;
    a.dt_bias = ext ? ext->dt_bias : nullptr;
    a.z = z;
    a.cu = cu;
    a.T = T;
    return launch_scan_fwd(a, stream);
}

// Device scratch of selective_scan_fwd_static: a file-scope array each GPU
// holds for the life of the process.  Host code never passes the array's
// name to a kernel (on the host it is only a stand-in for the symbol): the
// device address comes from hipGetSymbolAddress, looked up once per device
// with that device current, and is kept in static_scratch_ptr.
constexpr size_t kStaticScratchBytes = size_t(32) << 20;
static __device__ __attribute__((aligned(256))) char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex static_scratch_mu;
void* static_scratch_ptr[kMaxDevices] = {};

int static_scratch(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SSM_ERR_HIP;
    std::lock_guard<std::mutex> lock(static_scratch_mu);
    if (!static_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return SSM_ERR_HIP;
        static_scratch_ptr[dev] = ptr;
    }
    *out = static_scratch_ptr[dev];
    return SSM_OK;
}

}  // namespace
}  // namespace ssm

extern "C" {

int selective_scan_fwd_static(const ssm_scan_desc* desc, const float* s, const void* x,
                              const void* dt, const float* A, const void* B, const void* C,
                              const float* D, const int32_t* ids, const float* conv_w,
                              const float* conv_state, void* out, float* conv_state_out,
                              uint32_t* err, ssm_stream_t stream) {
    Shape sh;
    int rc = check_desc(desc, &sh);
    if (rc) return rc;
    // the call's workspace must fit the static scratch; checked before any HIP call
    const size_t need = workspace_bytes(sh, 0);
    if (need > kStaticScratchBytes) return SSM_ERR_WORKSPACE;
    void* ws = nullptr;
    if ((rc = static_scratch(&ws))) return rc;
    // without a caller's error word, the bits go to the scratch's own word (never read)
    return fwd_impl(desc, nullptr, s, x, dt, A, B, C, D, ids, conv_w, conv_state, out,
                    conv_state_out, ws, kStaticScratchBytes, static_cast<hipStream_t>(stream), err);
}

int selective_scan_fwd(const ssm_scan_desc* desc, const float* s, const void* x, const void* dt,
                       const float* A, const void* B, const void* C, const float* D,
                       const int32_t* ids, const float* conv_w, const float* conv_state,
                       void* out, float* conv_state_out, void* workspace, size_t workspace_bytes_,
                       ssm_stream_t stream) {
    return fwd_impl(desc, nullptr, s, x, dt, A, B, C, D, ids, conv_w, conv_state, out,
                    conv_state_out, workspace, workspace_bytes_, static_cast<hipStream_t>(stream));
}

size_t ssm_scan_ext_out_bytes(const ssm_scan_desc* desc, const ssm_scan_ext* ext,
                              size_t* state_offset_) {
    Shape sh;
    int64_t T;
    if (check_desc(desc, &sh) != SSM_OK || check_ext(sh, ext, &T) != SSM_OK) return 0;
    const size_t off = (size_t)(T * sh.d_inner()) * sh.io_bytes();
    if (state_offset_) *state_offset_ = off;
    return off + (size_t)sh.nelem_state() * 4;
}

const char* ssm_scan_fwd_plan(const ssm_scan_desc* desc, const ssm_scan_ext* ext) {
    Shape sh;
    int64_t T;
    if (check_desc(desc, &sh) != SSM_OK || check_ext(sh, ext, &T) != SSM_OK) return nullptr;
    // every tensor taken as present and 256-byte aligned
    static char dummy[256] __attribute__((aligned(256)));
    void* pp = dummy;
    FwdArgs a = {};
    a.sh = sh;
    a.s = a.A = a.D = a.conv_w = a.conv_state = static_cast<const float*>(pp);
    a.x = a.dt = a.B = a.C = pp;
    a.ids = static_cast<const int32_t*>(pp);
    a.y = pp;
    a.state_out = a.conv_state_out = static_cast<float*>(pp);
    a.T = T;
    if (ext) {
        a.dt_bias = ext->dt_bias ? static_cast<const float*>(pp) : nullptr;
        a.z = ext->z ? pp : nullptr;
        a.cu = ext->cu_seqlens ? static_cast<const int32_t*>(pp) : nullptr;
    }
    switch (fwd_path(a)) {
        case FwdPath::kNone: return "none";
        case FwdPath::kTimeSplit: return "time_split";
        case FwdPath::kQuad: {
            if (quad_chunked(sh)) return "quad_chunked";
            // the relay split depends on the current device (compute units,
            // resident blocks) and needs the workspace the shape asks for
            static char ws_probe[256] __attribute__((aligned(256)));
            a.ws = ws_probe;
            a.ws_bytes = fwd_workspace_bytes(sh);
            int relay_k = 0;
            launch_quad_fwd(a, nullptr, &relay_k);
            return relay_k > 0 ? "quad_relay" : "quad";
        }
        case FwdPath::kSsd: return "ssd";
        case FwdPath::kRows: return "rows";
    }
    return nullptr;
}

int selective_scan_fwd_ext(const ssm_scan_desc* desc, const ssm_scan_ext* ext, const float* s,
                           const void* x, const void* dt, const float* A, const void* B,
                           const void* C, const float* D, const int32_t* ids,
                           const float* conv_w, const float* conv_state, void* out,
                           float* conv_state_out, void* workspace, size_t workspace_bytes_,
                           ssm_stream_t stream) {
    return fwd_impl(desc, ext, s, x, dt, A, B, C, D, ids, conv_w, conv_state, out,
                    conv_state_out, workspace, workspace_bytes_, static_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace ssm {
namespace {

int bwd_impl(const ssm_scan_desc* desc, const float* s, const void* x, const void* dt,
             const float* A, const void* B, const void* C, const float* D, const int32_t* ids,
             const float* conv_w, const float* conv_state, bool with_conv, const void* dout,
             float* dgrad, void* workspace, size_t workspace_bytes_, hipStream_t stream) {
    Shape sh;
    int rc = check_desc(desc, &sh);
    if (rc) return rc;
    if (sh.K != 0 && !with_conv) return SSM_ERR_UNSUPPORTED;
    if (sh.K > 0 && !conv_w) return SSM_ERR_NULL;
    if (sh.S > 65535) return SSM_ERR_SHAPE;
    const bool has_x = sh.nelem_x() > 0, has_bc = sh.nelem_BC() > 0, has_seq = sh.S > 0;
    if (!s || !A || !dgrad || !workspace || (has_x && (!x || !dt)) || (has_bc && (!B || !C)) ||
        (has_seq && (!ids || !dout)))
        return SSM_ERR_NULL;
    if ((sh.flags & SSM_HAS_D) && !D) return SSM_ERR_NULL;
    if (workspace_bytes_ < workspace_bytes(sh, 1)) return SSM_ERR_WORKSPACE;
    const size_t es = sh.io_bytes();
    if (!aligned(x, es) || !aligned(dt, es) || !aligned(B, es) || !aligned(C, es) ||
        !aligned(dout, es) || !aligned(s, 4) || !aligned(A, 4) || !aligned(ids, 4) ||
        (D && !aligned(D, 4)) || !aligned(dgrad, 4) || !aligned(workspace, 256) ||
        !aligned(conv_w, 4) || !aligned(conv_state, 4))
        return SSM_ERR_ALIGN;
    const char* dstate = static_cast<const char*>(dout) + state_offset(sh);
    if (!aligned(dstate, 4)) return SSM_ERR_ALIGN;
    size_t off[9], total;
    dgrad_layout9(sh, off, &total);
    BwdArgs a;
    a.sh = sh; a.s = s; a.x = x; a.dt = dt; a.A = A; a.B = B; a.C = C;
    a.D = (sh.flags & SSM_HAS_D) ? D : nullptr;
    a.ids = ids; a.dy = dout; a.dstate = reinterpret_cast<const float*>(dstate);
    char* g = reinterpret_cast<char*>(dgrad);
    a.d_s = reinterpret_cast<float*>(g + off[0]);
    a.d_x = reinterpret_cast<float*>(g + off[1]);
    a.d_dt = reinterpret_cast<float*>(g + off[2]);
    a.d_A = reinterpret_cast<float*>(g + off[3]);
    a.d_B = reinterpret_cast<float*>(g + off[4]);
    a.d_C = reinterpret_cast<float*>(g + off[5]);
    a.d_D = (sh.flags & SSM_HAS_D) ? reinterpret_cast<float*>(g + off[6]) : nullptr;
    a.conv_w = sh.K ? conv_w : nullptr;
    a.conv_state = sh.K ? conv_state : nullptr;
    a.d_conv_w = sh.K ? reinterpret_cast<float*>(g + off[7]) : nullptr;
    a.d_conv_state = sh.K ? reinterpret_cast<float*>(g + off[8]) : nullptr;
    a.err = static_cast<uint32_t*>(workspace);
    a.ws = static_cast<char*>(workspace) + kErrBytes;
    a.ws_bytes = workspace_bytes_ - kErrBytes;
    return launch_scan_bwd(a, stream);
}

}  // namespace
}  // namespace ssm

extern "C" {

int selective_scan_bwd(const ssm_scan_desc* desc, const float* s, const void* x, const void* dt,
                       const float* A, const void* B, const void* C, const float* D,
                       const int32_t* ids, const void* dout, float* dgrad, void* workspace,
                       size_t workspace_bytes_, ssm_stream_t stream) {
    return bwd_impl(desc, s, x, dt, A, B, C, D, ids, nullptr, nullptr, false, dout, dgrad,
                    workspace, workspace_bytes_, static_cast<hipStream_t>(stream));
}

int selective_scan_bwd_conv(const ssm_scan_desc* desc, const float* s, const void* x,
                            const void* dt, const float* A, const void* B, const void* C,
                            const float* D, const int32_t* ids, const float* conv_w,
                            const float* conv_state, const void* dout, float* dgrad,
                            void* workspace, size_t workspace_bytes_, ssm_stream_t stream) {
    return bwd_impl(desc, s, x, dt, A, B, C, D, ids, conv_w, conv_state, true, dout, dgrad,
                    workspace, workspace_bytes_, static_cast<hipStream_t>(stream));
}

int selective_state_update(const ssm_scan_desc* desc, float* s, const void* x, const void* dt,
                           const float* dt_bias, const float* A, const void* B, const void* C,
                           const float* D, const void* z, const int32_t* ids,
                           const float* conv_w, float* conv_state, void* y, uint32_t* err,
                           ssm_stream_t stream) {
    Shape sh;
    int rc = check_desc(desc, &sh);
    if (rc) return rc;
    if (sh.L != 1) return SSM_ERR_SHAPE;
    int64_t rows;
    if (!mul_ok(sh.S, sh.d_inner(), &rows) || rows > (int64_t)INT_MAX * 16) return SSM_ERR_SHAPE;
    const bool has_seq = sh.S > 0;
    if (!s || !A || (has_seq && (!x || !dt || !B || !C || !ids || !y))) return SSM_ERR_NULL;
    if ((sh.flags & SSM_HAS_D) && !D) return SSM_ERR_NULL;
    if (sh.K > 0 && (!conv_w || !conv_state)) return SSM_ERR_NULL;
    const size_t es = sh.io_bytes();
    if (!aligned(x, es) || !aligned(dt, es) || !aligned(B, es) || !aligned(C, es) ||
        !aligned(z, es) || !aligned(y, es) || !aligned(s, 4) || !aligned(A, 4) ||
        !aligned(ids, 4) || !aligned(D, 4) || !aligned(dt_bias, 4) || !aligned(conv_w, 4) ||
        !aligned(conv_state, 4) || !aligned(err, 4))
        return SSM_ERR_ALIGN;
    DecodeArgs a;
    a.sh = sh; a.s = s; a.x = x; a.dt = dt; a.dt_bias = dt_bias; a.A = A; a.B = B; a.C = C;
    a.D = (sh.flags & SSM_HAS_D) ? D : nullptr;
    a.z = z; a.ids = ids;
    a.conv_w = sh.K ? conv_w : nullptr;
    a.conv_state = sh.K ? conv_state : nullptr;
    a.y = y; a.err = err;
    return launch_state_update(a, static_cast<hipStream_t>(stream));
}

int ssm_get_device_error(const void* workspace, ssm_stream_t stream, uint32_t* bits) {
    if (!workspace || !bits) return SSM_ERR_NULL;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (hipMemcpyAsync(bits, workspace, sizeof(uint32_t), hipMemcpyDeviceToHost, st) != hipSuccess)
        return SSM_ERR_HIP;
    return hipStreamSynchronize(st) == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

}  // extern "C"
