// C ABI of the library: host-side validation, workspace carving and launches.
// Declarations and the contract of every entry point are in include/gdn.h.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include "../../include/gdn.h"
#include "gdn_common.h"

namespace {

constexpr size_t kWorkspaceBytes = 256;   // status word, padded to one cache line

bool aligned16(const void *p) { return p == nullptr || ((uintptr_t)p & 15u) == 0; }

void debug(const char *msg)
{
    static const int on = [] {
        const char *e = getenv("GDN_DEBUG");
        return e && e[0] == '1';
    }();
    if (on) fprintf(stderr, "gdn: %s\n", msg);
}

int32_t check_desc(const gdn_desc *d, bool replay)
{
    if (!d) return GDN_ERR_NULL;
    if (d->n_seqs < 0 || d->h_qk <= 0 || d->h_v <= 0 || d->d_k <= 0 || d->d_v <= 0 ||
        d->total_tokens < 0 || d->total_out_tokens < 0) {
        debug("negative or zero size in descriptor");
        return GDN_ERR_SHAPE;
    }
    if (d->h_v % d->h_qk != 0) {
        debug("h_v must be a multiple of h_qk");
        return GDN_ERR_SHAPE;
    }
    if (!replay && d->total_out_tokens != d->total_tokens) {
        debug("prefill writes one output row per token: total_out_tokens must equal total_tokens");
        return GDN_ERR_SHAPE;
    }
    if (replay && d->total_out_tokens > d->total_tokens) {
        debug("replay outputs cannot exceed the packed tokens");
        return GDN_ERR_SHAPE;
    }
    if (d->total_tokens > 0x7fffffffLL) {
        debug("more than 2^31-1 packed tokens");
        return GDN_ERR_SHAPE;
    }
    if ((d->qkv_dtype != GDN_F32 && d->qkv_dtype != GDN_BF16) ||
        (d->o_dtype != GDN_F32 && d->o_dtype != GDN_BF16)) {
        debug("unknown dtype code");
        return GDN_ERR_DTYPE;
    }
    if (d->o_dtype != d->qkv_dtype && d->o_dtype != GDN_F32) {
        debug("o_dtype must equal qkv_dtype or be fp32");
        return GDN_ERR_DTYPE;
    }
    const bool d_ok = (d->d_k == 64 || d->d_k == 128) && (d->d_v == 64 || d->d_v == 128);
    if (!d_ok) {
        debug("unsupported head dims: d_k and d_v must be 64 or 128");
        return GDN_ERR_UNSUPPORTED;
    }
    // one chunk (64 tokens) of any packed tensor is addressed with 32-bit byte offsets
    const int64_t row_bytes = (int64_t)(d->h_v > d->h_qk ? d->h_v : d->h_qk) * 128 * 4;
    if (row_bytes * 64 >= 0x7fffffffLL) {
        debug("too many heads: a 64-token chunk must span less than 2 GiB");
        return GDN_ERR_SHAPE;
    }
    return GDN_OK;
}

int32_t run(const gdn_desc *d, const void *q, const void *k, const void *v, const float *g,
            const float *beta, const int32_t *cu, const int32_t *r, const float *S0, float *S_out,
            void *o_out, int32_t *cu_out, void *ws, size_t ws_bytes, void *stream)
{
    const bool replay = r != nullptr;
    int32_t st = check_desc(d, replay);
    if (st != GDN_OK) return st;
    if (!cu || !S_out || !ws) return GDN_ERR_NULL;
    const bool any_tokens = d->total_tokens > 0;
    if (any_tokens && (!q || !k || !v || !g || !beta)) return GDN_ERR_NULL;
    if (o_out && d->total_out_tokens > 0 && !any_tokens) return GDN_ERR_SHAPE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) || !aligned16(beta) ||
        !aligned16(S0) || !aligned16(S_out) || !aligned16(o_out) || !aligned16(ws) ||
        ((uintptr_t)cu & 3u) || ((uintptr_t)r & 3u) || ((uintptr_t)cu_out & 3u)) {
        debug("pointer alignment: 16 bytes required (4 for integer arrays)");
        return GDN_ERR_ALIGN;
    }
    if (ws_bytes < kWorkspaceBytes) return GDN_ERR_WORKSPACE;
    if (d->n_seqs == 0) return GDN_OK;

    gdn::ChunkArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
    a.cu = cu; a.r = r; a.S0 = replay ? nullptr : S0;
    a.S_out = S_out; a.o_out = o_out; a.cu_out = cu_out;
    a.status = reinterpret_cast<int32_t *>(ws);
    a.total_tokens = d->total_tokens;
    a.total_out = d->total_out_tokens;
    a.n_seqs = d->n_seqs; a.h_qk = d->h_qk; a.h_v = d->h_v;
    a.o_f32 = (d->o_dtype == GDN_F32 && d->qkv_dtype == GDN_BF16) ? 1 : 0;
    a.scale = d->scale;
    const hipError_t e = gdn::launch_chunk_ws(a, d->qkv_dtype == GDN_BF16, d->d_k, d->d_v,
                                              o_out != nullptr, reinterpret_cast<hipStream_t>(stream));
    if (e == hipErrorNotSupported) return GDN_ERR_UNSUPPORTED;
    return e == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

// Segment-parallel replay: segments per window and the workspace plan after the status
// word -- virtual cu_seqlens, virtual r, the map launch's states (S_local and M of every
// segment), every segment's true start state.
// The default: enough segments that the map launch and the output launch each fill about
// half the chip (128 / (n_seqs h_v)), but at least ~6 chunks per segment, estimated from the
// mean replay length total_out_tokens / n_seqs when it is given (measured: shorter segments
// cost more in the extra launches and the combine than they save).
int32_t seg_count(const gdn_desc *d, int32_t n_segments)
{
    if (n_segments > 0) return n_segments;
    const int64_t heads = (int64_t)d->n_seqs * d->h_v;
    int64_t p = heads > 0 ? 128 / heads : 1;
    if (d->total_out_tokens > 0 && d->n_seqs > 0) {
        const int64_t chunks = (d->total_out_tokens / d->n_seqs + 63) / 64;
        if (chunks / 6 < p) p = chunks / 6;
    }
    return (int32_t)(p < 1 ? 1 : p > 16 ? 16 : p);
}
struct SegPlan {
    size_t vcu, vr, lm, ss, bytes;
};
SegPlan seg_plan(const gdn_desc *d, int32_t P)
{
    auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
    const size_t nv = (size_t)d->n_seqs * (size_t)P;
    const size_t st = nv * (size_t)d->h_v * (size_t)d->d_k * (size_t)d->d_k * sizeof(float);
    SegPlan s;
    s.vcu = kWorkspaceBytes;
    s.vr = s.vcu + up((nv + 1) * sizeof(int32_t));
    s.lm = s.vr + up(nv * sizeof(int32_t));
    s.ss = s.lm + 2 * st;
    s.bytes = nv > 0 ? s.ss + st : kWorkspaceBytes;
    return s;
}

// per-(sequence, v-head) lengths of gdn_adaptive_replay_len, after the status word
size_t adaptive_scratch_bytes(const gdn_desc *d)
{
    if (!d || d->n_seqs <= 0 || d->h_v <= 0) return 0;
    const size_t b = (size_t)d->n_seqs * (size_t)d->h_v * sizeof(int32_t);
    return (b + 255) & ~(size_t)255;
}

}  // namespace

extern "C" {

int32_t gdn_abi_version(void) { return GDN_ABI_VERSION; }

const char *gdn_status_str(int32_t s)
{
    switch (s) {
    case GDN_OK: return "ok";
    case GDN_ERR_NULL: return "required pointer is NULL";
    case GDN_ERR_SHAPE: return "invalid or inconsistent sizes";
    case GDN_ERR_DTYPE: return "unknown or unsupported dtype combination";
    case GDN_ERR_UNSUPPORTED: return "head dims / dtype combination not supported by the library";
    case GDN_ERR_ALIGN: return "pointer not 16-byte aligned";
    case GDN_ERR_WORKSPACE: return "workspace missing or too small";
    case GDN_ERR_LAUNCH: return "kernel launch failed";
    case GDN_ERR_DEVICE_INPUT: return "device-side cu_seqlens / r invalid";
    case GDN_ERR_HIP: return "HIP runtime call failed";
    case GDN_ERR_DEVICE_WAIT: return "a bounded in-kernel wait expired (results invalid)";
    case GDN_ERR_SCRATCH: return "request larger than the library's static device scratch";
    default: return "unknown status";
    }
}

int32_t gdn_replay_len(int32_t L, double rho)
{
    if (L <= 0 || !(rho > 0.0)) return 0;
    const double x = rho * (double)L;
    double c = ceil(x - 1e-9 * (x > 1.0 ? x : 1.0));
    if (c < 0.0) c = 0.0;
    if (c > (double)L) c = (double)L;
    return (int32_t)c;
}

size_t gdn_workspace_bytes(const gdn_desc *desc)
{
    return kWorkspaceBytes + adaptive_scratch_bytes(desc);
}

int32_t gdn_replay(const gdn_desc *d, const void *q, const void *k, const void *v, const float *g,
                   const float *beta, const int32_t *cu_seqlens, const int32_t *r, float *S_out,
                   void *o_out, int32_t *cu_out, void *ws, size_t ws_bytes, void *stream)
{
    if (!r) return GDN_ERR_NULL;
    return run(d, q, k, v, g, beta, cu_seqlens, r, nullptr, S_out, o_out, cu_out, ws, ws_bytes,
               stream);
}

int32_t gdn_prefill(const gdn_desc *d, const void *q, const void *k, const void *v, const float *g,
                    const float *beta, const int32_t *cu_seqlens, const float *S0, float *S_out,
                    void *o_out, void *ws, size_t ws_bytes, void *stream)
{
    return run(d, q, k, v, g, beta, cu_seqlens, nullptr, S0, S_out, o_out, nullptr, ws, ws_bytes,
               stream);
}

size_t gdn_segmented_workspace_bytes(const gdn_desc *d, int32_t n_segments)
{
    if (check_desc(d, true) != GDN_OK || n_segments < 0 || n_segments > 64 || d->d_k != d->d_v) return 0;
    return seg_plan(d, seg_count(d, n_segments)).bytes;
}

int32_t gdn_replay_segmented(const gdn_desc *d, const void *q, const void *k, const void *v,
                             const float *g, const float *beta, const int32_t *cu, const int32_t *r,
                             float *S_out, void *o_out, int32_t *cu_out, int32_t n_segments, void *ws,
                             size_t ws_bytes, void *stream)
{
    int32_t st = check_desc(d, true);
    if (st != GDN_OK) return st;
    if (n_segments < 0 || n_segments > 64) {
        debug("n_segments must be in [0, 64]");
        return GDN_ERR_SHAPE;
    }
    if (d->d_k != d->d_v) {
        debug("segmented replay needs square states (d_k == d_v)");
        return GDN_ERR_UNSUPPORTED;
    }
    if (!cu || !r || !S_out || !ws) return GDN_ERR_NULL;
    const bool any_tokens = d->total_tokens > 0;
    if (any_tokens && (!q || !k || !v || !g || !beta)) return GDN_ERR_NULL;
    if (o_out && d->total_out_tokens > 0 && !any_tokens) return GDN_ERR_SHAPE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) || !aligned16(beta) ||
        !aligned16(S_out) || !aligned16(o_out) || !aligned16(ws) || ((uintptr_t)cu & 3u) ||
        ((uintptr_t)r & 3u) || ((uintptr_t)cu_out & 3u)) {
        debug("pointer alignment: 16 bytes required (4 for integer arrays)");
        return GDN_ERR_ALIGN;
    }
    const int32_t P = seg_count(d, n_segments);
    if ((int64_t)d->n_seqs * P > 0x7ffffffeLL) return GDN_ERR_SHAPE;
    const SegPlan plan = seg_plan(d, P);
    if (ws_bytes < plan.bytes) return GDN_ERR_WORKSPACE;
    if (d->n_seqs == 0) return GDN_OK;
    if (P == 1)   // one segment is the plain replay (bit for bit): run it directly
        return run(d, q, k, v, g, beta, cu, r, nullptr, S_out, o_out, cu_out, ws, ws_bytes, stream);

    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    char *w = reinterpret_cast<char *>(ws);
    int32_t *status = reinterpret_cast<int32_t *>(w);
    int32_t *vcu = reinterpret_cast<int32_t *>(w + plan.vcu);
    int32_t *vr = reinterpret_cast<int32_t *>(w + plan.vr);
    float *lm = reinterpret_cast<float *>(w + plan.lm);
    float *ss = reinterpret_cast<float *>(w + plan.ss);
    const int32_t nv = d->n_seqs * P;
    const bool bf16 = d->qkv_dtype == GDN_BF16;

    hipError_t e = gdn::launch_seg_setup(cu, r, d->n_seqs, P, d->total_tokens, vcu, vr, cu_out, status, s);
    if (e != hipSuccess) return GDN_ERR_LAUNCH;

    gdn::ChunkArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
    a.cu = vcu; a.r = vr; a.S0 = nullptr;
    a.S_out = lm; a.o_out = nullptr; a.cu_out = nullptr;
    a.status = status;
    a.total_tokens = d->total_tokens;
    a.total_out = d->total_out_tokens;
    a.n_seqs = nv; a.h_qk = d->h_qk; a.h_v = d->h_v;
    a.o_f32 = (d->o_dtype == GDN_F32 && bf16) ? 1 : 0;
    a.scale = d->scale;
    a.mpart = 1;   // every segment's S_local and transition map M in one launch
    e = gdn::launch_chunk_ws(a, bf16, d->d_k, d->d_v, false, s);
    if (e == hipErrorNotSupported) return GDN_ERR_UNSUPPORTED;
    if (e != hipSuccess) return GDN_ERR_LAUNCH;

    const size_t half = (size_t)nv * (size_t)d->h_v * (size_t)d->d_k * (size_t)d->d_k;
    e = gdn::launch_seg_combine(lm, lm + half, ss, S_out, d->n_seqs, d->h_v, d->d_k, P, bf16, s);
    if (e != hipSuccess) return GDN_ERR_LAUNCH;

    if (o_out) {   // every segment again from its true start, for the outputs
        a.mpart = 0;
        a.S0 = ss;
        a.S_out = lm;   // (scratch: the final state came from the combine)
        a.o_out = o_out;
        e = gdn::launch_chunk_ws(a, bf16, d->d_k, d->d_v, true, s);
        if (e != hipSuccess) return GDN_ERR_LAUNCH;
    }
    return GDN_OK;
}

int32_t gdn_state_relerr(const float *S_a, const float *S_ref, int64_t n_states, int32_t d_k,
                         int32_t d_v, float *relerr_out, int32_t *nonfinite_out, void *stream)
{
    if (n_states < 0 || d_k <= 0 || d_v <= 0) return GDN_ERR_SHAPE;
    if ((int64_t)d_k * d_v % 4 != 0 || (int64_t)d_k * d_v > 0x7fffffffLL) return GDN_ERR_UNSUPPORTED;
    if (n_states == 0) return GDN_OK;
    if (!S_a || !S_ref || !relerr_out) return GDN_ERR_NULL;
    if (!aligned16(S_a) || !aligned16(S_ref) || ((uintptr_t)relerr_out & 3u) ||
        ((uintptr_t)nonfinite_out & 3u))
        return GDN_ERR_ALIGN;
    const hipError_t e = gdn::launch_relerr(S_a, S_ref, n_states, d_k * d_v, relerr_out,
                                            nonfinite_out, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

int32_t gdn_adaptive_replay_len(const gdn_desc *d, const float *g, const int32_t *cu_seqlens,
                                double eps, int32_t r_min, int32_t r_max, int32_t *r_out,
                                void *ws, size_t ws_bytes, void *stream)
{
    if (!d) return GDN_ERR_NULL;
    if (d->n_seqs < 0 || d->h_v <= 0 || d->total_tokens < 0 || d->total_tokens > 0x7fffffffLL ||
        r_min < 0 || r_max < r_min || !(eps > 0.0)) {
        debug("adaptive replay length: bad sizes, clamp range or eps");
        return GDN_ERR_SHAPE;
    }
    if (!cu_seqlens || !r_out || !ws || (d->total_tokens > 0 && !g)) return GDN_ERR_NULL;
    if (!aligned16(g) || !aligned16(ws) || ((uintptr_t)cu_seqlens & 3u) || ((uintptr_t)r_out & 3u))
        return GDN_ERR_ALIGN;
    if (ws_bytes < kWorkspaceBytes + adaptive_scratch_bytes(d)) return GDN_ERR_WORKSPACE;
    if (d->n_seqs == 0) return GDN_OK;
    // threshold on the window's summed log-gates, in units of 2^-32 nats
    int64_t thr = 0;
    if (eps < 1.0) thr = (int64_t)floor(log(eps) * 4294967296.0);   // >= -745 * 2^32
    int32_t *scratch = reinterpret_cast<int32_t *>(reinterpret_cast<char *>(ws) + kWorkspaceBytes);
    const hipError_t e = gdn::launch_adaptive(g, cu_seqlens, d->n_seqs, d->h_v, d->total_tokens,
                                              thr, r_min, r_max, scratch, r_out,
                                              reinterpret_cast<int32_t *>(ws),
                                              reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

int32_t gdn_adaptive_replay_len_static(const gdn_desc *d, const float *g, const int32_t *cu_seqlens,
                                       double eps, int32_t r_min, int32_t r_max, int32_t *r_out,
                                       void *stream)
{
    if (!d) return GDN_ERR_NULL;
    if (d->n_seqs < 0 || d->h_v <= 0 || d->total_tokens < 0 || d->total_tokens > 0x7fffffffLL ||
        r_min < 0 || r_max < r_min || !(eps > 0.0)) {
        debug("adaptive replay length: bad sizes, clamp range or eps");
        return GDN_ERR_SHAPE;
    }
    if ((int64_t)d->n_seqs * d->h_v > gdn::kStaticHeads) {
        debug("allocation-free adaptive replay length: n_seqs * h_v exceeds the static scratch (65536)");
        return GDN_ERR_SCRATCH;
    }
    if (!cu_seqlens || !r_out || (d->total_tokens > 0 && !g)) return GDN_ERR_NULL;
    if (!aligned16(g) || ((uintptr_t)cu_seqlens & 3u) || ((uintptr_t)r_out & 3u)) return GDN_ERR_ALIGN;
    if (d->n_seqs == 0) return GDN_OK;
    int64_t thr = 0;
    if (eps < 1.0) thr = (int64_t)floor(log(eps) * 4294967296.0);
    const hipError_t e = gdn::launch_adaptive_static(g, cu_seqlens, d->n_seqs, d->h_v, d->total_tokens,
                                                     thr, r_min, r_max, r_out,
                                                     reinterpret_cast<hipStream_t>(stream));
    if (e == hipErrorInvalidSymbol) return GDN_ERR_HIP;
    return e == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

int32_t gdn_device_status(const void *ws, void *stream, int32_t *status_host)
{
    if (!ws || !status_host) return GDN_ERR_NULL;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (hipStreamSynchronize(s) != hipSuccess) return GDN_ERR_HIP;
    int32_t v = 0;
    if (hipMemcpy(&v, ws, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) return GDN_ERR_HIP;
    // the kernels only OR bits into the word: reading it starts a new accumulation
    if (v != 0 && (hipMemsetAsync(const_cast<void *>(ws), 0, sizeof(v), s) != hipSuccess ||
                   hipStreamSynchronize(s) != hipSuccess))
        return GDN_ERR_HIP;
    *status_host = (v & gdn::kStatusBitInput) ? GDN_ERR_DEVICE_INPUT
                 : (v & gdn::kStatusBitWait)  ? GDN_ERR_DEVICE_WAIT
                                              : GDN_OK;
    return GDN_OK;
}

}  // extern "C"
