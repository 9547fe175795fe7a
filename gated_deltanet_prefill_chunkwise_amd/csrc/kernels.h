// Launch interfaces of the gfx950 kernels (internal to libsgdn.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sgdn {

// Element type of the output o (the values of the boundary's sgdn_dtype).
constexpr int OUT_F32 = 0, OUT_BF16 = 1, OUT_F16 = 2;

// Workspace tensors (all per batch b, head-major).  I is the intermediate
// element type: fp16 for bf16 inputs, fp32 for fp32 inputs.
//   g      [B][Nv][C][64]      fp32  in-chunk inclusive log2 decay
//   fac    [B][Nv][C][64]      fp32  2^(gamma - g_t), the K^T X row factors
//   gamma  [B][Nv][C]          fp32  chunk retention g[63]
//   P      [B][Nv][C+1]        fp64  prefix of gamma
//   U      [B][Nv][C][dv][64]  I     U (then U' in place), dv-major tiles
//   W      [B][Nv][C][8192]    I     dense W tiles, fragment-major (below)
//   Cb     [B][Nv][C][64][64]  I     staged C diag(beta 2^g), row-major
//   KT     [B][Nq][C][8192]    I     key tiles, fragment-major (below)
//   snap   [..][dv][dk]        I     compact state snapshots (transposed)
//   s0T    [B][Nv][dv][dk]     I     initial state, transposed
//   Wpk    [B][Emax][2][8192]  I     deferred W of kept events, fragment-major
//   rec    dense [B][Nv][C], sparse [B][Emax][2]: int4 event records
//          {F_in, 2^gamma F_in (fp32 bits), snapshot index or -1, chunk}
//
// Fragment-major tiles: 16 blocks of 512 elements, block = one 64-lane MFMA
// operand fragment (lane l = 16 g + n holds 8 consecutive elements), so a wave
// reads one block as one contiguous 1 KB (bf16) request.  Both tiles use the
// permuted reduction order  r(g, e) = 4g + e (e < 4),  16 + 4g + e - 4 (e >= 4)
// within each 32-wide step, the order in which two stacked accumulator tiles
// hold their rows (so results feed the next product from registers):
//   W  block 4q + i  (dk step q, token tile i):  W[16i + n][32q + r(g, e)]
//   KT block 2mt + ks (dk tile mt, token step ks): K[32ks + r(g, e)][16mt + n]

struct IntraArgs {
  const void* k; const void* v; const float* a; const void* beta;
  int B, T, Nq, Nv, C, solve;
  const int32_t* cu;        // packed sequence offsets [B+1] or null
  // packed sequences: entry i = b C + c of the i-th valid chunk, the number
  // of valid chunks at index B C (written by the chunk-table kernel)
  const int32_t* chunks;
  float* g; float* gamma; float* fac;
  void* U; void* W; void* Cb; void* KT;
  float* score_part;        // sparse: [B][Nv][C][8] sums of squares of U per 8-row block
  int32_t* stats;           // [B][STATS_INTS] nonfinite_input bits K, V, A, BETA are ORed in
};

// Tail score of Eq. (9) over the last `tail` rows (8, 16, 32 or 64) from the
// 8-row parts: score = sqrt(sum of the parts of the window, in row order).
struct ScoreArgs { const float* part; float* score; long long n; int tail; };

struct PrefixArgs {
  const float* gamma; double* P; int B, Nv, C;
  const int32_t* cu; int T;   // packed sequences: gamma is read for valid chunks only
};

// Valid chunks of packed sequences, in (sequence, chunk) order.
//   table [B*C + 1 + B + 1]: entries b C + c, the count at index B C, then
//   the per-sequence offsets into the entries
struct ChunkTableArgs { const int32_t* cu; int32_t* table; int B, T, C; };

// Chain scan over the events of one value head, one dv slice of 16 columns
// per workgroup.  Dense: every chunk is an event, W from the intra kernel.
// Sparse: events from the CSR rows, W packed per event.
struct HScanArgs {
  const void* KT; const void* W; void* U;
  const void* k;            // key rows [tokens][Nq][dk] (Cb operand: K^T blocks formed in the kernel)
  const float* fac; const int32_t* rec; const double* P;
  const float* s0;          // [B][Nv][dk][dv] or null
  float* s_final;           // [B][Nv][dk][dv] or null
  void* snap;               // snapshots
  int B, Nq, Nv, C;
  int sparse;
  const int32_t* cu; int T;  // packed sequences: a dense chain stops at its valid chunks
  int w_by_chunk;           // sparse: W [B][Nv][C][8192] per chunk (deferred-W ablation)
  // rows row_lo .. row_lo + nrows - 1 of every sequence (CSR rows, sparse;
  // head pairs, dense); pair groups start at XCD xcd_shift, or (spread) each
  // pair group's 16 workgroups are dealt over all 8 XCDs, 2 per XCD
  int row_lo, nrows, xcd_shift, spread;
  // sparse metadata (per batch)
  const int32_t* row_pair;  // [B][NP]
  const int32_t* row_ptr;   // [B][NP+1]
  const int32_t* col;       // [B][Emax]
  const int32_t* event_slot;// [B][Emax]
  int Emax;
  int snap_cap;             // snapshot slots per batch (sparse)
  // sparse, fp16 intermediates: staged Cb [B][Nv][C][6][512] (fragment-major
  // blocks); W S is formed as Cb (K S) from it and the K^T tile
  const void* Cb;
  int blockadj;             // Cb block (3,0) is zero (block-adjacent solve)
  int32_t* stats;           // [B][STATS_INTS]: NF_SFINAL of nonfinite_output
};

struct OChunkArgs {
  const void* q; const void* k; const void* U; const void* snap; const void* s0T;
  const float* g; const float* gamma; const double* P;
  void* o; int o_type;   // OUT_* element type of o
  int B, T, Nq, Nv, C, G;
  const int32_t* cu;          // packed sequence offsets [B+1] or null
  int sparse;
  const int32_t* pred;        // [B][NP][G]
  const int32_t* group_slot;  // [B][NP][G]
  int snap_cap;
  // compact-states ablation: dense group-entry states [B][Nv][G][dv][dk]
  // (already decayed), read instead of the compact snapshots; or null
  const void* entry;
  const int32_t* row_pair;    // sparse: [B][NP] head pair of each CSR row
  int row_lo, nrows;          // rows covered by this launch
  int per_chunk;              // mapped-O ablation: one chunk per workgroup
  int32_t* stats;             // [B][STATS_INTS]: NF_Q of nonfinite_input, NF_O of nonfinite_output
};

// Compact-states ablation: every group's entry state S_2r written out densely
// from the compact snapshots (or s0), decayed by 2^(P_2r - P_e+1).
struct ExpandArgs {
  const void* snap; const void* s0T; const double* P;
  const int32_t* pred; const int32_t* group_slot;
  void* entry;
  int B, Nv, C, G, snap_cap, T;
  const int32_t* cu;
  const int32_t* row_pair;   // [B][NP] head pair of each CSR row
  int row_lo, nrows;         // CSR rows covered by this launch
};

// Per-event records of the H scan: the gap factor F_in that carries the state
// from the previous event of the row to this one, the step factor
// 2^gamma F_in, the snapshot index and the chunk.
struct EvRecArgs {
  const float* gamma; const double* P;
  const int32_t* row_pair; const int32_t* row_ptr; const int32_t* col; const int32_t* event_slot;
  int32_t* rec;
  int B, Nv, C, Emax, sparse;
  int row_lo, row_hi;   // sparse: CSR rows row_lo .. row_hi - 1
};

// Snapshot field of a null event in a record: the H scan forms its products
// and drops them (the CSR-off control of the sparse path).
constexpr int NULL_EVENT = -2;

// CSR-off control: every chunk of a CSR row is an event of the H scan, the
// chunks outside the mask null events.  Writes the all-chunk event lists
// (row_ptr_all [B][NP+1], col_all [B][NP*C]) and records [B][NP*C][2].
struct EvAllArgs {
  const float* gamma; const double* P; const uint8_t* mask;
  const int32_t* row_pair; const int32_t* row_ptr; const int32_t* event_slot;
  int32_t* rec; int32_t* col_all; int32_t* row_ptr_all;
  int B, Nv, C, Emax;
};

struct S0PrepArgs { const float* s0; void* s0T; int B, Nv; int32_t* stats; };

// Statistics words at the start of a call: the nonfinite fields cleared
// (sparse: the selector's layout kernel writes the others); dense: every
// field, with each chunk of each pair an event and Nv (G_b - 1) group-entry
// states.
struct StatsInitArgs { int32_t* stats; int B, Nv, C, T; const int32_t* cu; int dense; };

// The samples of a head are split over GATE_SPLIT workgroups, each writing
// its sum of squares to eta_part [B][Nv][GATE_SPLIT]; the selector adds
// the parts in order and divides by the sample count.
constexpr int GATE_SPLIT = 8;
struct GateArgs {
  const void* z; const float* w; float* eta_part; int B, T, Nv, C;
  const int32_t* cu;        // packed sequence offsets [B+1] or null
  int32_t* stats;           // NF_Z of nonfinite_input (the sampled gates)
};

// Bytes of the per-(sequence, head pair) record the selector passes between
// its kernels.
constexpr int PAIRREC_BYTES = 32;

struct SelectArgs {
  const float* score; const float* gamma; const float* eta;
  // (prefill) eta from the gate kernel's parts, written to eta_out
  const float* eta_part; float* eta_out;
  int B, C, keep_bp;
  int rate_bp[3];   // caller's tier rates in basis points, or {0, 0, 0}
  // packed sequence offsets [B+1] or null: sequence b has ceil(len_b / 64)
  // valid chunks (arrays keep the stride C); T bounds every length
  const int32_t* cu; int T;
  // ablations: 3 High / 4 Medium / 9 Low pairs; G_h = 1; caller rank keys
  // [B][16][C] that choose the kept chunks (the tiers still follow Eq. (10))
  int fixed_tiers, unit_visibility;
  int pair_order;       // tier-schedule ablation: CSR rows in head-pair order
  const float* rank_key;
  int32_t* rank_alt;    // [B][16][C]   workspace: ranks by rank_key
  int32_t* rank;        // [B][16][C]   workspace
  void* pair_rec;       // [B][16] pair records of PAIRREC_BYTES (gains, referenced events)
  uint8_t* mask; uint8_t* tier;
  int32_t* row_pair; int32_t* row_ptr; int32_t* col; int32_t* pred;
  int32_t* group_slot; int32_t* event_slot;
  int Emax, G;
  void* stats;          // sgdn_stats* or null
  int nf_clear;         // also zero the nonfinite fields (sgdn_select)
  const uint8_t* mask_in;  // override mask [B][16][C] or null
  // (prefill) the H scan's event records [B][Emax][2] int4 written by the
  // decide kernel with the layout, from the prefix P [B][Nv][C+1]; or null
  const double* P; int32_t* rec;
};

// (fp32 intermediates only: with fp16 the H scan forms W S = Cb (K S) from
// the staged Cb and the key rows, and the kept events need only records)
struct DeferredWArgs {
  const void* k;        // keys [tokens][Nq][dk] (the input)
  const void* Cb;
  void* Wpk;            // [B][Emax][2][64 * 128] W per kept event and head
  void* KTpk;           // [B][Emax][128 * 64] K^T blocks per kept event
  const int32_t* row_pair; const int32_t* row_ptr; const int32_t* col;
  int B, Nv, Nq, C, Emax, solve;
  const int32_t* cu; int T;   // packed sequences
  int row_lo, row_hi;   // the events of CSR rows row_lo .. row_hi - 1
};

// Single-token decode step (decode.hip).  q, k [B][Nq][128], v [B][Nv][128],
// a [B][Nv] fp32, beta [B][Nv], s_in / s_out [B][Nv][128][128] fp32.
struct DecodeArgs {
  const void* q; const void* k; const void* v; const float* a; const void* beta;
  const float* s_in; float* s_out; void* o;
  int B, Nq, Nv, o_type;   // OUT_* element type of o
};

hipError_t launch_intra(const IntraArgs& a, int bf16, hipStream_t s);
hipError_t launch_prefix(const PrefixArgs& a, hipStream_t s);
hipError_t launch_score(const ScoreArgs& a, hipStream_t s);
hipError_t launch_expand(const ExpandArgs& a, int bf16, hipStream_t s);
hipError_t launch_chunk_table(const ChunkTableArgs& a, hipStream_t s);
hipError_t launch_hscan(const HScanArgs& a, int bf16, hipStream_t s);
hipError_t launch_ochunk(const OChunkArgs& a, int bf16, hipStream_t s);
hipError_t launch_evrec(const EvRecArgs& a, hipStream_t s);
hipError_t launch_evrec_all(const EvAllArgs& a, hipStream_t s);
hipError_t launch_s0prep(const S0PrepArgs& a, int bf16, hipStream_t s);
hipError_t launch_gate(const GateArgs& a, int bf16, hipStream_t s);
// gate energies (ga non-null), prefix and tail scores in one launch (sparse path)
hipError_t launch_prep(const PrefixArgs& pa, const GateArgs* ga, const ScoreArgs& sc, int bf16,
                       hipStream_t s);
// deferred W + sparse event records of rows ea.row_lo .. ea.row_hi - 1 in one
// launch (da and ea cover the same rows)
hipError_t launch_events(const DeferredWArgs& da, const EvRecArgs& ea, hipStream_t s);   // fp32
hipError_t launch_select_full(const SelectArgs& a, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, int bf16, hipStream_t s);
hipError_t launch_stats_init(const StatsInitArgs& a, hipStream_t s);
hipError_t launch_fp64_selftest(const double* x, const double* y, double* q, double* r, long long n,
                                hipStream_t s);
hipError_t launch_debug_u(const void* Ut, float* U, int B, int Nv, int C, int bf16, hipStream_t s);

}  // namespace sgdn
