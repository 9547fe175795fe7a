/*
 * sgdn.h - C ABI of libsgdn.so: chunkwise Gated DeltaNet (GDN) core prefill,
 * dense and SparseGDN, on AMD Instinct MI355X (gfx950).
 *
 * The operations follow the web page "SparseGDN: Chunk Sparse in Linear
 * Attention" (reading notes of arXiv 2610.41420v1); citations give the
 * paper section and equation as that page prints them.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every array argument is a DEVICE pointer to memory owned by the caller
 *   (the library never allocates or frees device memory and never
 *   synchronises the stream).  Problem / parameter structs are HOST pointers.
 * - Arrays are dense, row-major, without padding, in the shapes given below.
 *   B = batch, T = tokens, Nq = query/key heads, Nv = value heads,
 *   d = d_k, dv = d_v, C = ceil(T / 64) chunks, G = ceil(C / 2) groups,
 *   NP = Nv / 2 head pairs.
 * - Value head h reads query/key head h / (Nv / Nq).  Supported: d = dv = 128,
 *   Nv = 2 * Nq (value heads 2p and 2p+1 share query/key head p; Sec. 2.1).
 * - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *   ordered after prior work on it.  The library keeps no state between
 *   calls (no streams, events or buffers of its own): calls are reentrant,
 *   except that two calls must not share a workspace, a stats array or the
 *   auxiliary events of sgdn_sparse_params concurrently.
 * - sgdn_prefill_sparse can run part of its work on a second,
 *   caller-owned stream (sgdn_sparse_params.aux_stream, forked from and
 *   joined back to `stream` with the caller's two events): later work on
 *   `stream` still sees every output.  Without it, every kernel runs on
 *   `stream`.  Both forms can be captured in a HIP graph.
 * - Errors: a negative sgdn_status is returned BEFORE anything is enqueued
 *   when an argument is invalid; SGDN_EHIP reports a failed launch.
 *   Data-dependent conditions are reported through sgdn_stats (below),
 *   including inputs outside the operator's domain.
 * - Domain (Sec. 2.1): the decay must satisfy a <= 0 (a is the log2
 *   retention; a > 0 is outside the operator's domain), every input must be
 *   finite, and q and k are expected to be L2-normalised rows (the
 *   operator's convention; the kernels do not normalise them, and their
 *   fp16 operand copies below rely on |q_i|, |k_i| <= 1).  Violations are
 *   not refused up front (that would need a pass over the inputs); the
 *   kernels flag them in sgdn_stats.nonfinite_input / nonfinite_output.
 * - Precision with bf16 inputs: the matrix products run on the fp16 / bf16
 *   matrix cores with fp32 accumulation, and the stage-to-stage
 *   intermediates (U, U', the staged coefficients Cb, the key tiles, the
 *   compact state snapshots, and the state slices fed to the products) are
 *   stored as fp16: 11-bit significands, so each rounding adds about 2^-12
 *   relative error; measured end to end, max |o - o_ref| / rms(o_ref) is
 *   2e-3 to 6e-3 at the workload's decays (fp32 inputs: every intermediate
 *   is fp32, about 1e-5).  fp16 holds magnitudes up to 65504: an
 *   intermediate beyond that (for example |v| in the thousands with beta
 *   near 1, or a state that large) becomes infinite, which surfaces as a
 *   non-finite o or s_final and sets nonfinite_output.  The state and its
 *   accumulation are always fp32.  A bf16 o adds its own rounding (up to
 *   2^-8 of each element), an fp16 o up to 2^-11 of each element (and holds
 *   magnitudes up to 65504: a larger output element is stored as infinite
 *   and sets nonfinite_output).
 * - T need not be a multiple of 64: the last chunk is padded with tokens
 *   that have a = 0, beta = 0, q = k = v = 0; their outputs are not written.
 * - Packed variable-length batches: with sgdn_problem.cu_seqlens set, the B
 *   sequences are packed along one token axis (below, "[B, T" then reads
 *   "[N_tok"): sequence b is tokens cu_seqlens[b] .. cu_seqlens[b+1] - 1 of
 *   q, k, v, a, beta, z and o, and seqlen is an upper bound on every length
 *   (longer sequences are cut to seqlen tokens).  Each sequence is computed
 *   exactly as if it were passed alone: its own chunks (padded at its own
 *   end), its own s0 / s_final row, and in the sparse path its own valid
 *   chunks for the selector (Sec. 2.4 ranks, anchors and counts the valid
 *   chunks of a sequence).  Empty sequences are allowed (s_final = s0).
 *   Per-chunk workspace arrays and debug outputs keep the stride
 *   C = ceil(seqlen / 64) per sequence.
 */
#ifndef SGDN_H
#define SGDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SGDN_OK = 0,
  SGDN_EINVAL = -1,        /* null pointer, bad shape, bad parameter            */
  SGDN_EUNSUPPORTED = -2,  /* valid but not supported (d != 128, Nv != 2 Nq ...) */
  SGDN_EWORKSPACE = -3,    /* ws_bytes smaller than sgdn_workspace_bytes()       */
  SGDN_EHIP = -4           /* a HIP launch failed                                */
} sgdn_status;

/* SGDN_F16 (IEEE binary16) is accepted for o_dtype only. */
typedef enum { SGDN_F32 = 0, SGDN_BF16 = 1, SGDN_F16 = 2 } sgdn_dtype;
typedef enum { SGDN_SOLVE_EXACT = 0, SGDN_SOLVE_BLOCKADJ = 1 } sgdn_solve;

/* Problem shape.  dtype applies to q, k, v, beta and z; o_dtype to o (a, s0
 * and s_final are always fp32).  solve selects the local Delta solve
 * (Sec. 2.3): SGDN_SOLVE_EXACT = M^{-1}, SGDN_SOLVE_BLOCKADJ = the 7-block
 * form of Eqs. (7)-(8).  Precision: see the conventions above. */
typedef struct {
  int32_t batch, seqlen, n_qk, n_v, d_k, d_v;
  int32_t dtype;    /* sgdn_dtype of q, k, v, beta, z */
  int32_t solve;    /* sgdn_solve */
  int32_t o_dtype;  /* sgdn_dtype of o: SGDN_F32, SGDN_BF16 or SGDN_F16 */
  /* DEVICE [batch + 1] int32 token offsets of packed sequences (non-
   * decreasing, cu_seqlens[0] = 0, cu_seqlens[batch] < 2^31 - seqlen), or
   * NULL for the dense [B, T] layout.  Read by the kernels, not the host. */
  const int32_t* cu_seqlens;
} sgdn_problem;

/* Selector parameters (Sec. 2.4).  keep_budget in (0, 1]: 0.29 gives the
 * page's tier rates (0.08, 0.30, 0.95); other budgets rescale them
 * (b <= 0.29: rho * b / 0.29; b > 0.29: 1 - (1 - rho)(1 - b) / 0.71);
 * 1.0 keeps every event.  tail: rows of the score of Eq. (9), 16 by default;
 * 8, 32 and 64 are the window ablations of Fig. 10.  r_window = 16 chunks for
 * r_h of Eq. (11) (the only supported value).  norm_weight: DEVICE [dv] fp32
 * RMSNorm scale used in the gate energy, or NULL for ones.
 * Selector ablations of Sec. 3.5 (0 = the method as defined):
 *   fixed_tiers = 1      3 High / 4 Medium / 9 Low head pairs in every layer
 *                        (Table 5) instead of the counts of Eqs. (13)-(14);
 *                        pairs are still assigned by x_H, then x_M.
 *   unit_visibility = 1  G_h = 1 for every head (gate energy not used).
 *   rank_key             DEVICE [B, NP, C] fp32 keys, or NULL: the kept
 *                        non-anchor chunks of a pair are those with the
 *                        largest keys (ties: lower chunk) instead of the
 *                        largest q_c; tiers and keep counts stay adaptive
 *                        (random keys = random selection at matched budget). */
typedef struct {
  float keep_budget;
  /* Tier rates (rho_L, rho_M, rho_H) of Eq. (13) overriding the ones derived
   * from keep_budget (which is then not used), or all three 0 for the derived
   * rates.  Each is taken in basis points, floor(rho * 10000 + 0.5), must lie
   * in (0, 1] and must not decrease from Low to High; otherwise SGDN_EINVAL.
   * k_l = clip(round(rho_l C), 2, C) with halves rounded up, as for the
   * derived rates. */
  float tier_rate[3];
  int32_t tail;
  int32_t r_window;
  const float* norm_weight;
  int32_t fixed_tiers;
  int32_t unit_visibility;
  const float* rank_key;
  int32_t ablate;   /* SGDN_ABLATE_* bits, 0 for the method as defined */
  /* Optional second stream: a hipStream_t of the caller's (default priority)
   * and two hipEvent_t of the caller's (created with hipEventDisableTiming is
   * enough), used to fork the H scan and O of CSR rows 4-15 of every sequence
   * onto aux_stream beside those of rows 0-3 on `stream` and to join them
   * back (not for sequences of at most 64 chunks, where the fork and join
   * cost more than the overlap gains, nor with several sequences whose tiers
   * all keep the same count: there every chain is equally long and the fork
   * cannot gain).  NULL aux_stream: one stream (same outputs).  The events
   * must not be used by another call at the same time. */
  void* aux_stream;
  void* aux_events[2];
} sgdn_sparse_params;

/* Kernel-pipeline ablations (Sec. 3.6, Table 6): reference paths that undo
 * one mechanism each, for measuring what it buys; outputs agree with the
 * default path within rounding.
 *   SGDN_ABLATE_DEFERRED_W      W of every chunk is formed in the intra stage
 *                               and read by chunk in the H scan (the packed-W
 *                               path), instead of W of the kept events after
 *                               selection (Eq. (15); with bf16 inputs the H
 *                               scan then forms W S as Cb (K S) and W is
 *                               never stored).  Not with cu_seqlens.
 *   SGDN_ABLATE_COMPACT_STATES  the entry state of every output group is
 *                               written out densely (decayed from the compact
 *                               snapshots) and O reads it, instead of O
 *                               reading the compact snapshots with the gap
 *                               factor (Eq. (21)).
 *   SGDN_ABLATE_CSR             the H scan steps through every chunk of each
 *                               head pair, forming the products of the
 *                               chunks outside the mask and dropping them,
 *                               instead of walking the CSR event list
 *                               (Eq. (16)); W of every chunk as with
 *                               SGDN_ABLATE_DEFERRED_W.  Not with cu_seqlens.
 *   SGDN_ABLATE_MAPPED_O        O runs one chunk per workgroup instead of
 *                               one two-chunk group (Eqs. (22)-(24)): both
 *                               workgroups of a group restore its entry
 *                               state, and the second also forms the cross
 *                               term A_{c+1,c} U'_c from the first chunk's
 *                               K and U'.  Same outputs; combined with
 *                               COMPACT_STATES it isolates the O mapping.
 *   SGDN_ABLATE_TIER_SCHEDULE   the CSR rows are laid out in head-pair order
 *                               instead of by tier (High first), and each
 *                               stage is one launch on `stream` (the
 *                               second-stream schedule relies on the High
 *                               tier in the first rows).  Same outputs. */
enum {
  SGDN_ABLATE_DEFERRED_W = 1,
  SGDN_ABLATE_COMPACT_STATES = 2,
  SGDN_ABLATE_CSR = 4,
  SGDN_ABLATE_MAPPED_O = 8,
  SGDN_ABLATE_TIER_SCHEDULE = 16
};

/* Per-sequence statistics written on the device (every field is written by
 * each call that is given the array).  The dense path reports every chunk of
 * every head pair as an event: E = NP C_b (C_b the sequence's chunks),
 * E_max = NP C, n_tier and k zero, n_snapshots = Nv (G_b - 1) group-entry
 * states.
 * nonfinite_input: bits of the inputs in which the kernels met a value
 *   outside the operator's domain (Sec. 2.1): SGDN_NF_Q, _K, _V, _A (a
 *   non-finite or a > 0), _BETA, _Z (the gate samples the selector reads),
 *   _S0.  0 for a clean call.
 * nonfinite_output: SGDN_NF_O if o holds a non-finite value, SGDN_NF_SFINAL
 *   if s_final does (with finite inputs: an fp16 intermediate overflowed). */
typedef struct {
  int32_t E;            /* kept events (row_ptr[NP])                          */
  int32_t E_max;        /* capacity 16 * k_H                                  */
  int32_t n_tier[3];    /* head pairs per tier: [0] Low, [1] Medium, [2] High */
  int32_t k[3];         /* events per pair in each tier: k_L, k_M, k_H        */
  int32_t n_snapshots;  /* compact state snapshots written by the H scan      */
  int32_t nonfinite_input;
  int32_t nonfinite_output;
} sgdn_stats;

enum {
  SGDN_NF_Q = 1, SGDN_NF_K = 2, SGDN_NF_V = 4, SGDN_NF_A = 8, SGDN_NF_BETA = 16,
  SGDN_NF_Z = 32, SGDN_NF_S0 = 64,          /* nonfinite_input bits  */
  SGDN_NF_O = 1, SGDN_NF_SFINAL = 2         /* nonfinite_output bits */
};

/* Optional DEVICE outputs of intermediate stages (tests and diagnostics).
 * Any member may be NULL; pass NULL for the whole struct in production. */
typedef struct {
  float* g;        /* [B, Nv, C, 64]   in-chunk inclusive log2 decay          */
  float* gamma;    /* [B, Nv, C]       chunk log2 retention                   */
  double* prefix;  /* [B, Nv, C + 1]   P of Eqs. (19)-(20)                    */
  float* score;    /* [B, Nv, C]       tail score of Eq. (9) (sparse)         */
  float* eta;      /* [B, Nv]          gate energy of Eq. (11) (sparse)       */
  float* U;        /* [B, Nv, C, 64, dv] U before the state correction (fp32) */
  uint8_t* mask;   /* [B, NP, C]       event mask (sparse)                    */
  uint8_t* tier;   /* [B, NP]          0 Low, 1 Medium, 2 High (sparse)       */
  /* Stage timing: caller-created hipEvent_t handles, recorded on the stream
   * at the stage boundaries SGDN_EV_*; events[i] is used when i < n_events.
   * Stages a call does not run leave adjacent events at the same point. */
  void** events;
  int32_t n_events;
} sgdn_debug;

/* Stage boundaries recorded into sgdn_debug.events. */
enum {
  SGDN_EV_START = 0,     /* before the first kernel                       */
  SGDN_EV_INTRA = 1,     /* after the intra-chunk kernel                  */
  SGDN_EV_PREFIX = 2,    /* after the log-decay prefix (sparse); dense:
                            after the event records                       */
  SGDN_EV_GATE = 3,      /* after the gate energy (sparse)                */
  SGDN_EV_SELECT = 4,    /* after selector + CSR layout (sparse)          */
  SGDN_EV_DEFERRED = 5,  /* after deferred W and the event records        */
  SGDN_EV_HSCAN = 6,     /* after the H-scan kernel alone                 */
  SGDN_EV_O = 7,         /* after the O kernel                            */
  SGDN_EV_COUNT = 8
};

/* Bytes of device workspace a call with this problem needs (256-byte
 * aligned sub-buffers).  sparse = 0 sizes sgdn_prefill_dense, 1 sizes
 * sgdn_prefill_sparse and sgdn_select.  Returns 0 for an invalid problem. */
size_t sgdn_workspace_bytes(const sgdn_problem* prob, int sparse,
                            const sgdn_sparse_params* params);

/* Event capacity of the selector (Sec. 2.4.3, Eq. (13); Sec. 2.5: the CSR
 * column array holds at most E_max = 16 k_H events per sequence, and the
 * device-side E never exceeds it).  Writes k = (k_L, k_M, k_H) for C =
 * ceil(seqlen / 64) chunks at params->keep_budget or params->tier_rate
 * (host memory, may be NULL)
 * and *e_max = 16 k_H, the per-sequence length of sgdn_select's col array.
 * Packed sequences with fewer chunks select fewer events.  Returns a negative
 * status for an invalid problem or parameters (nothing written). */
int sgdn_event_capacity(const sgdn_problem* prob, const sgdn_sparse_params* params,
                        int32_t* k, int32_t* e_max);

/* Dense GDN-core prefill, Sec. 2.1, Eqs. (1)-(4), with the local system of
 * Sec. 2.3, Eqs. (5)-(6) solved exactly or by the 7-block form.
 *   q, k    [B, T, Nq, d]   dtype
 *   v       [B, T, Nv, dv]  dtype
 *   a       [B, T, Nv]      fp32 log2 retention per token (<= 0)
 *   beta    [B, T, Nv]      dtype
 *   s0      [B, Nv, d, dv]  fp32 initial state, or NULL for zero
 *   o       [B, T, Nv, dv]  o_dtype, output before norm / gate / projection
 *   s_final [B, Nv, d, dv]  fp32 final state, or NULL
 *   stats   [B] device statistics (see sgdn_stats), or NULL
 *   ws      device workspace of at least sgdn_workspace_bytes(prob, 0, NULL)
 *   debug   optional stage outputs (may be NULL) */
int sgdn_prefill_dense(const sgdn_problem* prob, const void* q, const void* k,
                       const void* v, const float* a, const void* beta,
                       const float* s0, void* o, float* s_final, sgdn_stats* stats,
                       void* ws, size_t ws_bytes, void* stream, sgdn_debug* debug);

/* Dynamic event selection and CSR event layout, Sec. 2.4, Eqs. (10)-(14),
 * Sec. 2.5, Eq. (16), from the fp32 selection statistics of one batch.
 * Requires Nv = 32 (the tier table is written for 16 head pairs) and
 * C <= 8192.  Decisions are evaluated in binary64 in a fixed order (see the
 * selector source), so identical inputs give identical integers.
 *   score      [B, Nv, C]  fp32 tail scores (Eq. (9))
 *   gamma      [B, Nv, C]  fp32 chunk log2 retentions
 *   eta        [B, Nv]     fp32 gate energies (Eq. (11))
 *   mask       [B, NP, C]  out: 1 = event kept
 *   tier       [B, NP]     out: 0 Low, 1 Medium, 2 High
 *   row_pair   [B, NP]     out: head pair of each CSR row (High, Medium, Low;
 *                          ascending pair index within a tier)
 *   row_ptr    [B, NP + 1] out: row offsets into col
 *   col        [B, 16 k_H] out: kept chunk indices, ascending within a row
 *   pred       [B, NP, G]  out: last kept event before chunk 2r, or -1
 *   group_slot [B, NP, G]  out: snapshot slot of pred (slots number the
 *                          distinct predecessor events in CSR order), or -1
 *   stats      [B]         out (may be NULL) */
int sgdn_select(const sgdn_problem* prob, const float* score, const float* gamma,
                const float* eta, const sgdn_sparse_params* params, uint8_t* mask,
                uint8_t* tier, int32_t* row_pair, int32_t* row_ptr, int32_t* col,
                int32_t* pred, int32_t* group_slot, sgdn_stats* stats, void* ws,
                size_t ws_bytes, void* stream);

/* sgdn_select without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, results and statistics
 * as sgdn_select; the selector's scratch (rank tables, tier counts, event
 * slots) lives in a static device array of SGDN_NOALLOC_SCRATCH_BYTES that
 * every device the library runs on holds until the process ends, located on
 * the first call on a device (which must be the current device).  It calls
 * no allocation routine.  Limit: the selector's 64 B C + 32 B + 64 B k_H
 * bytes (plus 64 B C with rank_key), each rounded up to 256, must fit; about
 * B * C <= 22,000 sequence-chunks in every case (one sequence of 1.4M
 * tokens, or 8 sequences of 131,072), SGDN_EWORKSPACE beyond it (nothing
 * enqueued).  Calls that overlap on one device share the
 * scratch and race: serialise them (one stream, or events). */
#define SGDN_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)
int sgdn_select_noalloc(const sgdn_problem* prob, const float* score, const float* gamma,
                        const float* eta, const sgdn_sparse_params* params, uint8_t* mask,
                        uint8_t* tier, int32_t* row_pair, int32_t* row_ptr, int32_t* col,
                        int32_t* pred, int32_t* group_slot, sgdn_stats* stats, void* stream);

/* SparseGDN prefill, Secs. 2.2-2.7, Eqs. (5)-(25): local solve with fused
 * tail score, gate energy, selector, deferred W over CSR events (with bf16
 * inputs formed inside the H scan as W S = Cb (K S)),
 * event-sparse state propagation with compact snapshots, and two-chunk
 * mapped output.  Requires Nv = 32.  Arguments as sgdn_prefill_dense, plus
 *   z             [B, T, Nv, dv] dtype output gate (pre-activation)
 *   mask_override [B, NP, C] uint8 event mask to use instead of the
 *                 selector, or NULL (z may then be NULL)
 *   stats         [B] device statistics, or NULL */
int sgdn_prefill_sparse(const sgdn_problem* prob, const void* q, const void* k,
                        const void* v, const float* a, const void* beta,
                        const void* z, const sgdn_sparse_params* params,
                        const uint8_t* mask_override, const float* s0, void* o,
                        float* s_final, sgdn_stats* stats, void* ws,
                        size_t ws_bytes, void* stream, sgdn_debug* debug);

/* Single-token decode step: the gated delta rule applied to one new token of
 * each sequence, continuing from the final state a prefill returned (Sec. 2.6
 * hands S_{C,h} to autoregressive decoding; the step is the per-token form of
 * Sec. 2.1).  For value head h, with alpha = 2^a and query/key head
 * h / (Nv / Nq):
 *     S' = alpha S + k u^T,  u = beta (v - alpha S^T k),  o = S'^T q / sqrt(d)
 * prob: batch = B sequences, seqlen must be 1, Nv a multiple of Nq,
 * d = dv = 128, cu_seqlens NULL; dtype applies to q, k, v, beta, o_dtype to
 * o; solve is ignored.
 *   q, k   [B, Nq, d]       dtype
 *   v      [B, Nv, dv]      dtype
 *   a      [B, Nv]          fp32 log2 retention (<= 0)
 *   beta   [B, Nv]          dtype
 *   s_in   [B, Nv, d, dv]   fp32 state before the token
 *   s_out  [B, Nv, d, dv]   fp32 state after the token; may be s_in itself
 *                           (updated in place), must not overlap it otherwise
 *   o      [B, Nv, dv]      o_dtype output of the token
 * s_in and s_out must be 16-byte aligned.  Needs no workspace.  SGDN_EINVAL
 * for a null pointer, seqlen != 1, cu_seqlens set, a misaligned state or
 * partially overlapping states. */
int sgdn_decode_step(const sgdn_problem* prob, const void* q, const void* k,
                     const void* v, const float* a, const void* beta,
                     const float* s_in, float* s_out, void* o, void* stream);

/* Static description of a status code. */
const char* sgdn_status_string(int status);

/* Diagnostic: the selector's decisions are bit-reproducible only if the
 * device's binary64 division and square root round correctly (Sec. 2.4,
 * Eqs. (10)-(14) are evaluated with them).  This runs the selector's own
 * compiled forms of both operations: quot[i] = x[i] / y[i] and
 * root[i] = sqrt(x[i]) for i < n, so that callers can compare them with a
 * correctly rounded host.  All arrays DEVICE [n]; n >= 0.  SGDN_EINVAL for
 * a null pointer with n > 0. */
int sgdn_fp64_selftest(const double* x, const double* y, double* quot, double* root,
                       int64_t n, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SGDN_H */
