/*
 * gdn.h -- C ABI of the Gated DeltaNet state-rebuild library for MI355X (gfx950).
 *
 * What the library computes.  Hybrid LLMs interleave full-attention layers with
 * Gated DeltaNet linear-attention layers whose recurrent state cannot be rolled
 * back to an arbitrary prefix boundary.  Tail-Replay (arXiv 2608.30310, abstract;
 * gist.science technical summary, "Mecanismos Principais") rebuilds each
 * linear-attention layer's state at a matched-prefix boundary by replaying only the
 * most recent r tokens of the prefix, starting from a zero state, through the
 * Gated DeltaNet recurrence.  Full prefill of the whole prefix is the baseline it
 * is compared with (same pages, "Resultados").  Per (sequence, v-head):
 *
 *     S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,
 *     o_t = scale * S_t^T q_t,        alpha_t = exp(g_t),  g_t <= 0,
 *
 * with S a d_k x d_v matrix.  g = -inf is legal and means alpha = 0.
 *
 * Layouts (row-major, contiguous, packed varlen in "THD" order):
 *     q, k       [T, h_qk, d_k]      in qkv_dtype
 *     v          [T, h_v,  d_v]      in qkv_dtype
 *     g, beta    [T, h_v]            fp32
 *     cu_seqlens [n_seqs + 1]        int32, sequence n owns tokens [cu[n], cu[n+1])
 *     r          [n_seqs]            int32 replay lengths, 0 <= r[n] <= cu[n+1]-cu[n]
 *     S0, S_out  [n_seqs, h_v, d_k, d_v]  fp32
 *     o_out      [T_out, h_v, d_v]   in o_dtype; rows packed per sequence in order
 * v-head h reads q/k head floor(h * h_qk / h_v) (grouped value heads).
 *
 * Pointers are device pointers unless marked (host).  Every call is asynchronous
 * on `stream` (a hipStream_t; NULL = the null stream) except gdn_device_status.
 *
 * Ownership: the caller owns every buffer, including the workspace.  The compute
 * calls never allocate, free or synchronise; they print nothing unless the
 * environment variable GDN_DEBUG is 1 (then a host-side rejection says why on
 * stderr).  Their only global state is a per-device cache of the occupancy query
 * (written once, atomically); calls are re-entrant given distinct workspaces.
 *
 * Errors: problems checkable on the host (null required pointer, bad dims,
 * h_v % h_qk != 0, unsupported d, misaligned pointer, small workspace) return a
 * non-zero gdn_status before anything is enqueued.  A failed launch returns
 * GDN_ERR_LAUNCH.  The device-resident cu_seqlens / r are validated by the kernel
 * itself: on a bad value it sets a bit in the workspace's status word, skips the
 * offending sequences and leaves their outputs unspecified.  The kernels only ever
 * set bits in that word (atomically), never clear it: gdn_device_status reports
 * what the calls since the previous gdn_device_status on that workspace (or since
 * it was zero-filled) recorded, and clears it.  A new workspace must therefore be
 * zero-filled once before its first use.  Non-finite q/k/v/beta or g > 0 are not
 * checked; the result is then undefined and gdn_state_relerr's non-finite count
 * exposes it.
 *
 * Arithmetic: the state is fp32 throughout.  fp32 inputs use fp32 matrix products.
 * bf16 inputs use matrix products with fp16 operands and fp32 accumulation: q and k
 * enter exactly (bf16 values of magnitude in [2^-14, 65504], which L2-normalised q and
 * k are; smaller entries round to fp16 subnormals), the intermediate state and pseudo-
 * values are rounded to fp16 once per product (relative error <= 2^-11).  Their range
 * is checked nowhere: state entries, and v-sized intermediates, must stay below ~10^3
 * in magnitude (the state is scaled by at most 64 internally); beyond that the fp16
 * operands overflow and the outputs turn non-finite (again exposed by the non-finite
 * count).  Gated DeltaNet states with unit keys, beta in [0, 1] and O(1) values stay
 * orders of magnitude inside this.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 3

typedef enum {
    GDN_OK = 0,
    GDN_ERR_NULL = 1,          /* a required pointer is NULL */
    GDN_ERR_SHAPE = 2,         /* negative / inconsistent sizes, h_v % h_qk != 0 */
    GDN_ERR_DTYPE = 3,         /* unknown dtype code */
    GDN_ERR_UNSUPPORTED = 4,   /* valid but not built: d_k or d_v outside {64, 128} */
    GDN_ERR_ALIGN = 5,         /* a pointer is not 16-byte aligned */
    GDN_ERR_WORKSPACE = 6,     /* workspace missing or smaller than gdn_workspace_bytes() */
    GDN_ERR_LAUNCH = 7,        /* the HIP launch failed */
    GDN_ERR_DEVICE_INPUT = 8,  /* device-side cu_seqlens / r invalid (from gdn_device_status) */
    GDN_ERR_HIP = 9,           /* a HIP runtime call failed (gdn_device_status only) */
    GDN_ERR_DEVICE_WAIT = 10,  /* a bounded wait inside a workgroup expired: results invalid
                                  (from gdn_device_status; not expected on working hardware) */
    GDN_ERR_SCRATCH = 11       /* request larger than the static device scratch of an
                                  allocation-free entry point */
} gdn_status;

typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

typedef struct {
    int32_t n_seqs;            /* packed sequences (a stack of independent layers may be packed as sequences) */
    int32_t h_qk, h_v;         /* q/k heads and v heads, h_v % h_qk == 0 */
    int32_t d_k, d_v;          /* head dims, each 64 or 128 */
    int32_t qkv_dtype;         /* gdn_dtype of q, k, v */
    int32_t o_dtype;           /* gdn_dtype of o: qkv_dtype, or GDN_F32 */
    float scale;               /* o_t = scale * S_t^T q_t */
    int64_t total_tokens;      /* T == cu_seqlens[n_seqs] (host copy) */
    int64_t total_out_tokens;  /* rows of o_out: sum r[n] (replay) or T (prefill); a replay
                                  without o_out only needs total_out_tokens <= total_tokens */
} gdn_desc;

/* ABI version of the loaded library (GDN_ABI_VERSION). */
int32_t gdn_abi_version(void);

/* Static description of a status code. */
const char *gdn_status_str(int32_t status);

/* (host) Replay length for a matched prefix of L tokens under budget fraction rho:
 * clamp(ceil(rho * L), 0, L) -- the pages replay the last 5-10 % of the matched
 * prefix (Tail-Replay abstract; technical summary, "Resultados"). */
int32_t gdn_replay_len(int32_t L, double rho);

/* (host) Workspace bytes a call with this descriptor needs: 256 (the status word), plus
 * n_seqs * h_v * 4 rounded up to 256 for gdn_adaptive_replay_len.  Zero-fill a new
 * workspace once before its first use (the status word accumulates bits). */
size_t gdn_workspace_bytes(const gdn_desc *desc);

/* Tail replay: for every sequence n and v-head h, run the recurrence from S = 0 over
 * the last r[n] tokens [cu[n+1]-r[n], cu[n+1]) and write the state after the last
 * token to S_out (the state at the prefix boundary; technical summary,
 * "Reconstrucao de Estado Independente").  o_out (nullable) receives o_t for the
 * replayed tokens, packed per sequence; cu_out (nullable, [n_seqs+1]) receives the
 * output row offsets.  r[n] = 0 gives S = 0 (the pages' Zero-Only baseline) and no
 * o rows; r[n] = L_n gives exactly gdn_prefill with S0 = NULL. */
int32_t gdn_replay(const gdn_desc *desc, const void *q, const void *k, const void *v,
                   const float *g, const float *beta, const int32_t *cu_seqlens,
                   const int32_t *r, float *S_out, void *o_out, int32_t *cu_out,
                   void *workspace, size_t workspace_bytes, void *stream);

/* Full prefill: the recurrence over every whole sequence from S0 (NULL = zero
 * state).  This is the baseline Tail-Replay is measured against: processing the
 * whole matched prefix again (fugumt.com page, English abstract; gist.science
 * technical summary, "Resultados", where replay is compared with full prefill for
 * quality and time to first token).  o_out (nullable) has one row per token, in token
 * order.  With S0 set to a rebuilt state it continues a prefix into its unmatched
 * suffix, the step that produces the first token after a cache hit (same section). */
int32_t gdn_prefill(const gdn_desc *desc, const void *q, const void *k, const void *v,
                    const float *g, const float *beta, const int32_t *cu_seqlens,
                    const float *S0, float *S_out, void *o_out,
                    void *workspace, size_t workspace_bytes, void *stream);

/* Error report: relerr[s] = ||S_a[s] - S_ref[s]||_F / ||S_ref[s]||_F (||S_a[s]||_F when
 * the reference is zero), fp64 accumulation; nonfinite[s] (nullable) counts the
 * non-finite entries of S_a[s].  States are d_k x d_v fp32 blocks.  It measures how
 * far a replayed state is from the full-prefill state at the same boundary: the pages'
 * claim is that a short recent tail approximates that state because the gated updates
 * attenuate older inputs (fugumt.com page, English abstract), and that zeroing the state
 * instead ("Zero-Only", relative error 1 here) degrades quality (technical summary,
 * "Resultados"). */
int32_t gdn_state_relerr(const float *S_a, const float *S_ref, int64_t n_states, int32_t d_k,
                         int32_t d_v, float *relerr_out, int32_t *nonfinite_out, void *stream);

/* Adaptive replay length.  The replayed state differs from the full-prefill state by
 * the older state carried through the window's per-token maps alpha_t (I - beta_t k_t
 * k_t^T), whose product has norm at most prod alpha_t for unit keys and beta in
 * [0, 1]; the gated updates attenuate distant tokens (Tail-Replay, arXiv 2608.30310,
 * abstract; technical summary, "Mecanismos Principais"), while the pages fix r as a
 * 5-10 % budget ("Resultados").  This picks r per sequence from the gates instead:
 *
 *     r_h[n] = the smallest r in [0, min(L_n, r_max)] with sum over the last r tokens
 *              of g[t, h] <= ln(eps)   (i.e. prod alpha <= eps), or min(L_n, r_max);
 *     r_out[n] = clamp(max_h r_h[n], min(r_min, L_n), min(r_max, L_n)),
 *
 * so ||S_full - S_replay||_F <= eps ||S_before||_F in every head whenever r_out[n] is
 * below the cap.  The comparison is exact: each g is rounded to a multiple of 2^-32
 * nats (g >= 0 or NaN counts as 0; g <= -2^20, including -inf, as -2^20) and summed in
 * integers against floor(ln(eps) * 2^32); eps >= 1 gives r_h = 0.
 * desc: n_seqs, h_v and total_tokens are read (the other fields are ignored).
 * g [T, h_v] fp32 and cu_seqlens [n_seqs+1] are device arrays; r_out [n_seqs] (device,
 * int32) can be passed straight to gdn_replay.  The workspace must hold
 * gdn_workspace_bytes(desc) bytes; its status word reports GDN_ERR_DEVICE_INPUT for a
 * bad cu_seqlens (those sequences get r_out = 0).  Host errors: eps <= 0 or NaN,
 * r_min < 0 or r_max < r_min -> GDN_ERR_SHAPE. */
int32_t gdn_adaptive_replay_len(const gdn_desc *desc, const float *g, const int32_t *cu_seqlens,
                                double eps, int32_t r_min, int32_t r_max, int32_t *r_out,
                                void *workspace, size_t workspace_bytes, void *stream);

/* Allocation-free gdn_adaptive_replay_len, for callers that cannot allocate device
 * memory or take a workspace (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments and result as
 * gdn_adaptive_replay_len minus the workspace: its per-head lengths live in the
 * library's own static device scratch, 65536 int32 per GPU (plus a 256-byte status
 * block), held until the process ends; it calls no allocator.  Limit: n_seqs * h_v <=
 * 65536, else GDN_ERR_SCRATCH before anything is enqueued.  All calls on one GPU share
 * that scratch: calls that overlap on one GPU (concurrent streams, threads) race and give
 * undefined r_out; calls ordered on one stream are fine.  A bad device cu_seqlens shows
 * as r_out[n] = 0 for the sequences concerned (there is no status word to read).
 * GDN_ERR_HIP if the scratch's device address cannot be looked up. */
int32_t gdn_adaptive_replay_len_static(const gdn_desc *desc, const float *g,
                                       const int32_t *cu_seqlens, double eps, int32_t r_min,
                                       int32_t r_max, int32_t *r_out, void *stream);

/* Segment-parallel tail replay: gdn_replay's result (up to rounding) in less time when
 * few (sequence, v-head) chains are long, e.g. one layer of one sequence.  The recurrence
 * is affine in the state, so over any stretch of tokens S_end = M S_start + S_local, with
 * S_local the state the stretch builds from zero and M the product of its per-token maps
 * alpha_t (I - beta_t k_t k_t^T) (technical summary, "Mecanismos Principais", for the
 * recurrence; the pages replay one window per layer from a zero state).  Each window is
 * cut into P chunk-aligned segments of ceil(ceil(r/64)/P) chunks (trailing ones may be
 * empty); one launch forms every segment's S_local and M together, a combine chains
 * S_start(p+1) = M_p S_start(p) + S_local(p) from S_start(0) = 0 with fp32 sums (bf16
 * inputs: each fp32 operand as fp16 hi + lo halves, three products, about fp32 accuracy
 * inside the fp16 range the bf16 path already requires) and writes the final state to
 * S_out, and, when o_out is given, a second launch re-runs each segment
 * from its true start for the outputs (layouts as gdn_replay; cu_out likewise).
 * n_segments: P in [1, 64], or 0 for the library's choice, clamp(min(128 / (n_seqs h_v),
 * chunks / 6), 1, 16) with chunks = ceil(total_out_tokens / n_seqs / 64) when
 * total_out_tokens > 0 (segments shorter than ~6 chunks cost more than they save); P = 1
 * runs gdn_replay itself.  Requires d_k == d_v (else GDN_ERR_UNSUPPORTED); n_segments
 * outside [0, 64] -> GDN_ERR_SHAPE.  The
 * workspace must hold gdn_segmented_workspace_bytes(desc, n_segments) bytes (its first
 * 256 are the status word, as for every call); it also carries the segments' states,
 * 3 n_seqs P h_v d_k^2 floats.  Errors in the device cu_seqlens / r are reported through
 * the status word as for gdn_replay.  Compared with gdn_replay: S and o agree to the
 * rounding of the products (fp16 operands for bf16 inputs), not bit for bit. */
size_t gdn_segmented_workspace_bytes(const gdn_desc *desc, int32_t n_segments);
int32_t gdn_replay_segmented(const gdn_desc *desc, const void *q, const void *k, const void *v,
                             const float *g, const float *beta, const int32_t *cu_seqlens,
                             const int32_t *r, float *S_out, void *o_out, int32_t *cu_out,
                             int32_t n_segments, void *workspace, size_t workspace_bytes,
                             void *stream);

/* (host, synchronising) Wait for `stream`, read the status word of `workspace` and
 * clear it.  *status_host: GDN_OK, GDN_ERR_DEVICE_INPUT (a call since the previous
 * read found a bad cu_seqlens / r) or GDN_ERR_DEVICE_WAIT.  Returns GDN_ERR_HIP if the
 * wait, the copy or the clear failed. */
int32_t gdn_device_status(const void *workspace, void *stream, int32_t *status_host);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
