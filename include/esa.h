/*
 * esa.h - C ABI of libesa.so: the gated linear recurrence of Entangled State Attention (ESA)
 * on AMD Instinct MI355X (gfx950).
 *
 * The operation (page "entangled-state-attention 0.1.0", section "Core idea"; page
 * "Entangled State Attention v2.1", introduction; page "Entangled State Attention",
 * section "[ ARCHITECTURE ]"):
 *
 *   s_t = sigma(a_t)                                     gate from the gate logit a_t
 *   direct:      E_t = s_t * E_{t-1} + v_t               (A = sigma(a), B = V)
 *   controlled:  E_t = s_t * E_{t-1} + (1 - s_t) * v_t   (g = sigma(a), B = (1 - g) V)
 *   y_t = q_t * E_t / sqrt(mean_h(E_t^2) + 1e-6)         readout, per head over Dh channels
 *
 * elementwise for every (batch b, head h, channel d) lane and causal over t.  The pages
 * leave "Norm" undefined; this library reads it as per-head RMSNorm with eps = 1e-6 inside
 * the square root and no gain.  The projections x W_A, x W_V, x W_Q and the output
 * projection W_O are outside the library: it takes the gate logits, values and queries.
 *
 * Layout.  Sequence tensors are contiguous [B, T, H, Dh] with Dh fastest, in the storage
 * dtype.  States are contiguous [B, H, Dh] and always fp32.  Arithmetic is fp32, with fp64
 * accumulation for fp32 storage (states, gradients and the scans' compositions; gates,
 * readout and the cross-tile words stay fp32); outputs in a 16- or 8-bit dtype are rounded
 * to nearest even.  An 8-bit
 * output beyond its format's range becomes what the format's conversion gives: NaN for E4M3
 * (magnitude at least 464), infinity for E5M2 (at least 61440).
 *
 * Ownership and execution.  The caller owns every buffer (device memory).  The library
 * never allocates or frees; each call validates its arguments on the host, enqueues its
 * kernels on `stream` (a hipStream_t; NULL is the default stream) and returns.  Two calls
 * also wait for the stream: esa_workspace_status (to read the header) and the first call of
 * esa_scan_fwd_noalloc on a device (which clears its static scratch once).  Errors that occur while the kernels run surface at the caller's next
 * synchronisation.  The library is reentrant; its only global state is a process-wide
 * counter that tags each scan launch's look-back words.  Calls that share one workspace
 * must not run concurrently (use one workspace per stream).
 *
 * Graphs.  Every call may be recorded into a HIP graph by stream capture.  A scan launch
 * recorded into a graph takes its look-back tag from word 0 of the workspace, which a
 * one-thread kernel recorded just before it advances, so each replay is correct with no host
 * work; no call records a memset.  Replays of graphs that share a workspace must not run
 * concurrently with each other or with eager calls on that workspace.
 *
 * Errors.  Every entry point returns an esa_status.  All argument checks run before any
 * HIP call, so an invalid call changes nothing on the device:
 *   ESA_ERR_INVALID_ARG  null required pointer, negative size, bad enum, pointer not
 *                        16-byte aligned, element count overflowing int64, or an output
 *                        that overlaps an input
 *   ESA_ERR_UNSUPPORTED  Dh not in {16, 32, 64, 128}, or a problem whose tile count
 *                        exceeds 2^31 - 1
 *   ESA_ERR_WORKSPACE    workspace NULL or smaller than esa_scan_workspace_bytes()
 *   ESA_ERR_HIP          a kernel launch was rejected by the HIP runtime
 *   ESA_ERR_SCRATCH_LIMIT  (esa_scan_fwd_noalloc only) the problem needs more look-back
 *                        scratch than ESA_NOALLOC_SCRATCH_BYTES
 *   ESA_ERR_TIMEOUT      (esa_workspace_status only) a scan on the workspace had a
 *                        cross-tile wait time out since the workspace was last initialised
 */
#ifndef ESA_H
#define ESA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 1: fp32 / fp16 / bf16 storage.  2: adds the fp8 storage dtypes ESA_F8E4M3, ESA_F8E5M2,
 * the sequence-segment calls and the ESA_DETERMINISTIC mode flag.  3: adds the
 * ESA_TEST_FORCE_TIMEOUT mode flag.  4: adds esa_scan_fwd_noalloc and
 * ESA_ERR_SCRATCH_LIMIT.  5: adds esa_workspace_status, ESA_ERR_TIMEOUT and the
 * ESA_LOOKBACK_STATS mode flag; a timed-out wait no longer makes later launches give up. */
#define ESA_ABI_VERSION 5

/* Checkpoint granularity: the forward can store the fp32 state at every 64th step. */
#define ESA_CKPT_CHUNK 64

typedef enum {
    ESA_OK = 0,
    ESA_ERR_INVALID_ARG = 1,
    ESA_ERR_UNSUPPORTED = 2,
    ESA_ERR_WORKSPACE = 3,
    ESA_ERR_HIP = 4,
    ESA_ERR_SCRATCH_LIMIT = 5,
    ESA_ERR_TIMEOUT = 6
} esa_status;

/* Storage dtype of the sequence tensors (precision modes of page "Entangled State
 * Attention v2.1", section "3. Precision": fp16 default, bf16, fp32, and fp8, which that
 * section calls experimental).  The fp8 dtypes are the OCP 8-bit formats: E4M3 (no
 * infinities, largest finite 448) and E5M2 (largest finite 57344).  One dtype serves every
 * sequence tensor of a call; arithmetic and states stay fp32 whatever the storage. */
typedef enum {
    ESA_F32 = 0,
    ESA_F16 = 1,
    ESA_BF16 = 2,
    ESA_F8E4M3 = 3,
    ESA_F8E5M2 = 4
} esa_dtype;

/* Recurrence form (page "entangled-state-attention 0.1.0", "Direct vs controlled mode"). */
typedef enum { ESA_DIRECT = 0, ESA_CONTROLLED = 1 } esa_mode;

/* Flag OR-ed into the mode argument of the scan calls: bitwise reproducible results.
 * Without it a tile may combine whatever earlier tiles have published, so the last bits can
 * differ from run to run (always within the parity bar).  With it every chain of tiles is cut
 * into blocks of K tiles (a power of two up to 16, picked from the sizes and the storage type
 * alone): the last tile of each block publishes its inclusive value and the others only their
 * aggregates, so every carry is one fixed fp32 expression of the inputs.  A problem's results
 * are then the same bits on every run; problems of other sizes may differ in the last bits.
 * Measured cost: +0-20 % against the default look-back, from one chain of tiles (B*H*Dh = 64
 * lanes) to many (the 64K-context workload, where K = 1).  esa_state_step accepts and
 * ignores it. */
#define ESA_DETERMINISTIC 0x100

/* Test control OR-ed into the mode argument of esa_scan_fwd and esa_scan_bwd, never set in
 * normal use: a separate instance of the kernels runs in which the first tile of every chain
 * (first in the scan's direction) withholds its published values and the cross-tile wait
 * gives up after a few thousand polls, so every wait on a withheld value times out.  The
 * call returns normally: the workspace records the timeout (see esa_workspace_status), and
 * every output that depends on a withheld value is NaN.  It exercises the failure path of
 * the bounded wait from the host.  Only fp16 storage with Dh = 64 has that instance
 * (ESA_ERR_UNSUPPORTED otherwise); the other calls reject the flag (ESA_ERR_INVALID_ARG). */
#define ESA_TEST_FORCE_TIMEOUT 0x200

/* Diagnostic flag OR-ed into the mode argument of esa_scan_fwd and esa_scan_bwd: a separate
 * instance of the kernels runs that counts what the cross-tile look-back did, into the
 * workspace header (read them with esa_workspace_status).  Results are those of the
 * default look-back; the counting costs one set of atomics per workgroup.  fp16 and fp8 E4M3
 * storage with Dh = 64 only (ESA_ERR_UNSUPPORTED otherwise); not combinable with
 * ESA_DETERMINISTIC or ESA_TEST_FORCE_TIMEOUT, and rejected by the other calls
 * (ESA_ERR_INVALID_ARG). */
#define ESA_LOOKBACK_STATS 0x400

/* ABI version of the loaded library (ESA_ABI_VERSION at build time). */
int esa_abi_version(void);

/* Static, human-readable text for a status code; never NULL. */
const char *esa_status_string(int status);

/* Bytes of device workspace that esa_scan_fwd / esa_scan_bwd need for this problem.  One
 * workspace sized for the largest problem serves every smaller one.  Returns 0 for
 * invalid or unsupported sizes.  A workspace must be zero-filled once before its first use
 * (hipMemset, torch.zeros, or esa_workspace_init); every call that completes leaves it
 * ready for the next call. */
size_t esa_scan_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t Dh, int dtype);

/* Bytes of the forward's checkpoint: fp32 [B, ceil(T / 64), H, Dh], the state E_t at
 * t = 64 k + 63 for each chunk k (the last chunk holds E_{T-1}).  Returns 0 on bad sizes. */
size_t esa_scan_ckpt_bytes(int64_t B, int64_t T, int64_t H, int64_t Dh);

/* Zero-fills `bytes` of workspace on `stream` (a fill kernel, safe inside graph capture).
 * This also clears the workspace's timeout record and look-back counters (see
 * esa_workspace_status). */
int esa_workspace_init(void *workspace, size_t bytes, void *stream);

/* The state a workspace's header records, read on the host: waits for `stream`, then copies
 * the header (a few hundred bytes; nothing is allocated).  Not callable while `stream` is
 * being recorded into a graph (ESA_ERR_INVALID_ARG).
 *   workspace  a scan workspace, or NULL for this device's no-allocation scratch (all zeros
 *              before the first esa_scan_fwd_noalloc on the device)
 *   info       uint32_t[6], out:
 *     info[0]  0, or the tag of the last scan launch whose cross-tile wait timed out (about
 *              a second of polling; never in a correct run, but forced by
 *              ESA_TEST_FORCE_TIMEOUT).  That launch's outputs that depend on the missing
 *              value are NaN; later launches are unaffected.  Cleared only by
 *              esa_workspace_init.
 *     info[1..5]  look-back counters of ESA_LOOKBACK_STATS launches since the last
 *              esa_workspace_init, over the lanes of every tile but a chain's first: lanes
 *              that found their neighbouring tile's inclusive value published; lanes that
 *              walked back over earlier tiles' aggregates; tiles folded by those walks; the
 *              longest walk (tiles read, the inclusive one included); unproductive polls.
 * Returns ESA_ERR_TIMEOUT when info[0] is non-zero, ESA_OK otherwise. */
int esa_workspace_status(const void *workspace, uint32_t *info, void *stream);

/* Forward scan with fused gate and readout: prefill and training forward (page "Entangled
 * State Attention", "[ ARCHITECTURE ]": associative composition over the sequence, then a
 * compact final state; "[ QUICK START ]": esa.prefill returns the output and the state).
 *   B, T, H, Dh   sizes; T = 0 is allowed: only final_state is written, and the sequence
 *                 pointers may then be NULL
 *   dtype, mode   esa_dtype, esa_mode
 *   gate_logit    [B,T,H,Dh] dtype, in: a_t
 *   value         [B,T,H,Dh] dtype, in: v_t
 *   query         [B,T,H,Dh] dtype, in: q_t
 *   init_state    [B,H,Dh] fp32, in, or NULL for E_{-1} = 0
 *   y             [B,T,H,Dh] dtype, out: y_t
 *   final_state   [B,H,Dh] fp32, out (E_{T-1}), or NULL; may equal init_state (in place)
 *   ckpt          esa_scan_ckpt_bytes() fp32, out (for esa_scan_bwd), or NULL
 *   workspace     device buffer of workspace_bytes >= esa_scan_workspace_bytes()
 *   stream        hipStream_t or NULL */
int esa_scan_fwd(int64_t B, int64_t T, int64_t H, int64_t Dh, int dtype, int mode,
                 const void *gate_logit, const void *value, const void *query,
                 const float *init_state, void *y, float *final_state, float *ckpt,
                 void *workspace, size_t workspace_bytes, void *stream);

/* ---- The forward without a workspace, for callers that cannot allocate ----
 *
 * For code that may not call hipMalloc (work recorded into a HIP graph, tight serving
 * loops, harnesses that forbid allocation): esa_scan_fwd with the same arguments, minus the
 * workspace.  Its look-back words live in a static device array of ESA_NOALLOC_SCRATCH_BYTES
 * that every device the library runs on holds until the process ends; the call allocates
 * nothing.  The problem needs 256 + 2 * ceil(T / TT) * B * H * Dh * 8 bytes of it, TT being
 * the forward's tile length in steps: 256 (16-bit storage, Dh <= 64; 128 for the fp16,
 * Dh = 64 sizes that the forward's measured tile table gives 256-thread workgroups), 128
 * (16-bit with Dh = 128, 8-bit, fp32 with Dh <= 64) or 64 (fp32 with Dh = 128);
 * esa_scan_workspace_bytes() of the same problem is an upper bound.  Larger
 * problems get ESA_ERR_SCRATCH_LIMIT before anything is launched.  Example: B = 256,
 * T = 8192, H = 8, Dh = 64 in fp16 needs 64 MiB + 256 bytes and is refused; T = 4096 fits.
 *
 * The first call on a device looks up that device's copy of the array and clears it once
 * (a fill kernel on `stream`; outside graph capture that first call then waits for the
 * stream).  Every later call on the device reuses the array as it was left.  All calls on one
 * device share the one array: calls that overlap in time on one device race (run them on
 * one stream, or one after another); replays of graphs that recorded this call count as
 * calls.  ESA_DETERMINISTIC is accepted; ESA_TEST_FORCE_TIMEOUT is refused
 * (ESA_ERR_INVALID_ARG).  Arguments, results and the other errors are those of
 * esa_scan_fwd. */
#define ESA_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)
int esa_scan_fwd_noalloc(int64_t B, int64_t T, int64_t H, int64_t Dh, int dtype, int mode,
                         const void *gate_logit, const void *value, const void *query,
                         const float *init_state, void *y, float *final_state, float *ckpt,
                         void *stream);

/* Backward of esa_scan_fwd: the chain rule through readout, recurrence and gate, run as a
 * reverse-time scan dE_t = gE_t + s_{t+1} dE_{t+1} (no page states it; it is derived from
 * the forward of page "entangled-state-attention 0.1.0", "Core idea").
 *   gate_logit, value, query, init_state   the forward's inputs (init_state may be NULL)
 *   dy             [B,T,H,Dh] dtype, in: gradient of y
 *   d_final_state  [B,H,Dh] fp32, in: gradient of final_state, or NULL for zero
 *   ckpt           the forward's checkpoint, or NULL (the library then recomputes it into
 *                  the workspace with one extra pass that reads a and v)
 *   d_gate_logit, d_value, d_query  [B,T,H,Dh] dtype, out
 *   d_init_state   [B,H,Dh] fp32, out, or NULL
 * T = 0 is allowed: d_init_state receives d_final_state (or zeros), and the sequence
 * pointers may then be NULL. */
int esa_scan_bwd(int64_t B, int64_t T, int64_t H, int64_t Dh, int dtype, int mode,
                 const void *gate_logit, const void *value, const void *query,
                 const float *init_state, const void *dy, const float *d_final_state,
                 const float *ckpt, void *d_gate_logit, void *d_value, void *d_query,
                 float *d_init_state, void *workspace, size_t workspace_bytes, void *stream);

/* One-token recurrent update with readout, for generation (page "Entangled State
 * Attention", "[ ARCHITECTURE ]" one-token update and "[ QUICK START ]" esa.decode_step;
 * page "Entangled State Attention v2.1", section 5, lightning_step):
 *   gate_logit, value, query   [B,H,Dh] dtype, in: this token's a, v, q
 *   state                      [B,H,Dh] fp32, in/out, updated in place
 *   y                          [B,H,Dh] dtype, out
 * Needs no workspace. */
int esa_state_step(int64_t B, int64_t H, int64_t Dh, int dtype, int mode,
                   const void *gate_logit, const void *value, const void *query, float *state,
                   void *y, void *stream);

/* ---- Sequence segments: the scan over T split into consecutive segments ----
 *
 * The recurrence composes associatively (page "Entangled State Attention", "[ ARCHITECTURE ]"),
 * so a sequence cut into segments 0..n-1 (one per device, say) is scanned in two passes:
 *   1. each segment's aggregate over its own steps from a zero state: the state it produces,
 *      E_seg, and the product of its gates, P_seg (esa_scan_segment_fwd, reads a and v only);
 *   2. the aggregates of all segments composed in order (esa_segment_compose), giving the
 *      state entering each segment; each segment then runs esa_scan_fwd with that state as
 *      init_state.
 * The backward mirrors it: each segment's gradient reaching its start with no gradient
 * arriving at its end (esa_scan_segment_bwd), the composition from the last segment
 * (esa_segment_compose, reverse = 1, with the same P_seg), then esa_scan_bwd per segment
 * with that gradient as d_final_state.  Results equal the unsegmented scan up to fp32
 * rounding order. */

/* Segment aggregate (pass 1).  Over this call's T steps from a zero state:
 *   seg_state      [B,H,Dh] fp32, out: E_{T-1}
 *   seg_gate_prod  [B,H,Dh] fp32, out: the product over t of A_t = sigma(a_t)
 * T = 0 gives the identity (zeros and ones).  Sizes, dtypes, modes, alignment, workspace and
 * errors as esa_scan_fwd. */
int esa_scan_segment_fwd(int64_t B, int64_t T, int64_t H, int64_t Dh, int dtype, int mode,
                         const void *gate_logit, const void *value, float *seg_state,
                         float *seg_gate_prod, void *workspace, size_t workspace_bytes,
                         void *stream);

/* Backward segment aggregate: the gradient reaching the segment's initial state when no
 * gradient arrives at its final state (d_final_state = 0), i.e. esa_scan_bwd's d_init_state
 * without writing the sequence gradients.
 *   gate_logit, value, query, init_state, dy, ckpt   as esa_scan_bwd (init_state is the
 *                  state entering the segment; ckpt from its esa_scan_fwd, or NULL)
 *   seg_d_init     [B,H,Dh] fp32, out */
int esa_scan_segment_bwd(int64_t B, int64_t T, int64_t H, int64_t Dh, int dtype, int mode,
                         const void *gate_logit, const void *value, const void *query,
                         const float *init_state, const void *dy, const float *ckpt,
                         float *seg_d_init, void *workspace, size_t workspace_bytes,
                         void *stream);

/* Composition of segment aggregates (pass 2), per lane, c <- P_k c + X_k segment by segment:
 *   nseg, nLanes   segments and lanes (nLanes = B*H*Dh)
 *   reverse        0: segments 0..n-1 in order; 1: from segment n-1 down to 0
 *   seg_gate_prod  [nseg, nLanes] fp32, in: P_k of each segment
 *   seg_agg        [nseg, nLanes] fp32, in: X_k = seg_state (forward) or seg_d_init (reverse)
 *   boundary       [nLanes] fp32, in: init_state (forward) or d_final_state (reverse) of the
 *                  whole sequence, or NULL for zeros
 *   carry          [nseg, nLanes] fp32, out: the value entering segment k from its earlier
 *                  side: its init_state (forward) or its d_final_state (reverse)
 *   total          [nLanes] fp32, out, or NULL: the value after the last segment: the final
 *                  state (forward) or d_init_state of the whole sequence (reverse)
 * Pointers need 4-byte alignment; outputs may not overlap inputs or each other. */
int esa_segment_compose(int64_t nseg, int64_t nLanes, int reverse, const float *seg_gate_prod,
                        const float *seg_agg, const float *boundary, float *carry, float *total,
                        void *stream);

#ifdef __cplusplus
}
#endif

#endif /* ESA_H */
