// C ABI of libsgdn.so (declared in include/sgdn.h): argument validation,
// workspace carve-up and the launch sequence of the dense and sparse
// GDN-core prefill.  Nothing here allocates device memory or synchronises.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "../../include/sgdn.h"
#include "common.h"
#include "kernels.h"

namespace {

using namespace sgdn;

constexpr int NP_SPARSE = 16;
static_assert(OUT_F32 == SGDN_F32 && OUT_BF16 == SGDN_BF16 && OUT_F16 == SGDN_F16,
              "output element codes");

struct Plan {
  int B, T, Nq, Nv, C, G, esz, isz, bf16, solve;
  const int32_t* cu;   // packed sequence offsets or null
  int kL, kM, kH;
  int ablate;      // SGDN_ABLATE_* bits (sparse)
  int Emax;        // event capacity per sequence inside prefill_sparse
  int snap_cap;    // snapshot slots per sequence (sparse) or per head (dense)
  size_t off[32];
  size_t total;
};

enum Buf { B_G, B_GAMMA, B_P, B_U, B_W, B_CB, B_KT, B_SNAP, B_S0T, B_SCORE, B_ETA, B_RANK,
           B_PREC, B_MASK, B_TIER, B_ROWPAIR, B_ROWPTR, B_COL, B_PRED, B_GSLOT, B_ESLOT,
           B_WPK, B_STATS, B_FAC, B_REC, B_CHUNKS, B_SPART, B_RANK2, B_ENTRY, B_COLALL,
           B_RPALL, B_ETAP, B_COUNT };

static_assert(B_COUNT <= (int)(sizeof(Plan::off) / sizeof(size_t)), "workspace table too small");

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// k = clip(round(rho C), 2, C) in exact integer arithmetic, round half up.
// rbp: the caller's tier rates in basis points, or rbp[0] = 0 for the rates
// derived from the budget bp.
void tier_counts(int C, int bp, const int rbp[3], int k[3]) {
  static const int pct[3] = {8, 30, 95};
  for (int i = 0; i < 3; ++i) {
    if (C == 1) { k[i] = 1; continue; }
    long long num, den;
    if (rbp[0] > 0) {
      num = (long long)rbp[i] * C;
      den = 10000;
    } else if (bp <= 2900) {
      num = (long long)pct[i] * bp * C;
      den = 290000;
    } else {
      num = (long long)C * (710000LL - (long long)(100 - pct[i]) * (10000 - bp));
      den = 710000;
    }
    long long kk = (2 * num + den) / (2 * den);
    if (kk < 2) kk = 2;
    if (kk > C) kk = C;
    k[i] = (int)kk;
  }
}

int budget_bp(float b) { return (int)floor((double)b * 10000.0 + 0.5); }

// The caller's tier rates in basis points (floor(rho 10000 + 0.5)), or
// {0, 0, 0} when all three are zero (rates derived from the keep budget).
// Returns SGDN_EINVAL for a rate outside (0, 1], a non-finite rate, or rates
// that decrease from Low to Medium to High.
int rates_bp(const sgdn_sparse_params* sp, int r[3]) {
  r[0] = r[1] = r[2] = 0;
  if (sp->tier_rate[0] == 0.f && sp->tier_rate[1] == 0.f && sp->tier_rate[2] == 0.f) return SGDN_OK;
  for (int i = 0; i < 3; ++i) {
    const float x = sp->tier_rate[i];
    if (!(x > 0.f) || !(x <= 1.f)) return SGDN_EINVAL;
    r[i] = budget_bp(x);
    if (r[i] < 1 || r[i] > 10000) return SGDN_EINVAL;
  }
  if (r[0] > r[1] || r[1] > r[2]) return SGDN_EINVAL;
  return SGDN_OK;
}

int check_problem(const sgdn_problem* pr) {
  if (pr == nullptr) return SGDN_EINVAL;
  if (pr->batch < 1 || pr->seqlen < 1 || pr->n_qk < 1 || pr->n_v < 1) return SGDN_EINVAL;
  if (pr->dtype != SGDN_F32 && pr->dtype != SGDN_BF16) return SGDN_EINVAL;
  if (pr->solve != SGDN_SOLVE_EXACT && pr->solve != SGDN_SOLVE_BLOCKADJ) return SGDN_EINVAL;
  if (pr->o_dtype != SGDN_F32 && pr->o_dtype != SGDN_BF16 && pr->o_dtype != SGDN_F16)
    return SGDN_EINVAL;
  if (pr->d_k != 128 || pr->d_v != 128) return SGDN_EUNSUPPORTED;
  if (pr->n_v != 2 * pr->n_qk) return SGDN_EUNSUPPORTED;
  // grid dimensions and 32-bit in-kernel offsets
  if ((long long)pr->batch * pr->seqlen > (1LL << 31) / 4 / pr->n_v) return SGDN_EUNSUPPORTED;
  return SGDN_OK;
}

int check_params(const sgdn_problem* pr, const sgdn_sparse_params* sp) {
  if (sp == nullptr) return SGDN_EINVAL;
  const int bp = budget_bp(sp->keep_budget);
  if (!(sp->keep_budget > 0.f) || bp < 1 || bp > 10000) return SGDN_EINVAL;
  int rbp[3];
  if (rates_bp(sp, rbp) != SGDN_OK) return SGDN_EINVAL;
  if (sp->tail != 8 && sp->tail != 16 && sp->tail != 32 && sp->tail != 64) return SGDN_EUNSUPPORTED;
  if (sp->r_window != 16) return SGDN_EUNSUPPORTED;
  if (sp->aux_stream != nullptr && (sp->aux_events[0] == nullptr || sp->aux_events[1] == nullptr ||
                                    sp->aux_events[0] == sp->aux_events[1]))
    return SGDN_EINVAL;
  if ((sp->fixed_tiers != 0 && sp->fixed_tiers != 1) ||
      (sp->unit_visibility != 0 && sp->unit_visibility != 1))
    return SGDN_EINVAL;
  constexpr int ALL = SGDN_ABLATE_DEFERRED_W | SGDN_ABLATE_COMPACT_STATES | SGDN_ABLATE_CSR |
                      SGDN_ABLATE_MAPPED_O | SGDN_ABLATE_TIER_SCHEDULE;
  if (sp->ablate & ~ALL) return SGDN_EINVAL;
  if ((sp->ablate & (SGDN_ABLATE_DEFERRED_W | SGDN_ABLATE_CSR)) && pr->cu_seqlens != nullptr)
    return SGDN_EUNSUPPORTED;
  if (pr->n_v != 2 * NP_SPARSE) return SGDN_EUNSUPPORTED;
  const int C = (pr->seqlen + 63) / 64;
  if (C > 8192) return SGDN_EUNSUPPORTED;
  return SGDN_OK;
}

void make_plan(const sgdn_problem* pr, int sparse, const sgdn_sparse_params* sp, Plan& p) {
  p.B = pr->batch; p.T = pr->seqlen; p.Nq = pr->n_qk; p.Nv = pr->n_v; p.cu = pr->cu_seqlens;
  p.C = (p.T + 63) / 64; p.G = (p.C + 1) / 2;
  p.bf16 = pr->dtype == SGDN_BF16; p.esz = p.bf16 ? 2 : 4; p.solve = pr->solve;
  p.isz = p.bf16 ? 2 : 4;   // intermediates: fp16 for bf16 inputs, fp32 for fp32 inputs
  int k[3] = {p.C, p.C, p.C};
  if (sparse) {
    int rbp[3];
    rates_bp(sp, rbp);
    tier_counts(p.C, budget_bp(sp->keep_budget), rbp, k);
  }
  p.ablate = sparse ? sp->ablate : 0;
  p.kL = k[0]; p.kM = k[1]; p.kH = k[2];
  const int NP = p.Nv / 2;
  p.Emax = NP * p.C;
  p.snap_cap = sparse ? NP * (p.G > 1 ? p.G - 1 : 1) : (p.G > 1 ? p.G - 1 : 1);
  const size_t B = p.B, Nv = p.Nv, C = p.C, G = p.G, I = p.isz;
  size_t sz[B_COUNT];
  memset(sz, 0, sizeof(sz));
  sz[B_G] = B * Nv * C * L * 4;
  sz[B_GAMMA] = B * Nv * C * 4;
  sz[B_FAC] = B * Nv * C * L * 4;
  sz[B_REC] = B * Nv * C * 16;   // sparse: B * Emax * 2 records, Emax <= NP * C
  sz[B_P] = B * Nv * (C + 1) * 8;
  sz[B_U] = B * Nv * C * L * DV * I;
  // K^T blocks for the W-operand H scan (fp32 inputs; the sparse controls
  // with W of every chunk): per chunk (dense, and those controls) or per
  // kept event (sparse: at most E_max = NP C per sequence).  The Cb-operand
  // H scan forms them from the key rows.
  const bool wall_plan = sparse && (p.ablate & (SGDN_ABLATE_DEFERRED_W | SGDN_ABLATE_CSR)) != 0;
  if (I == 4 || wall_plan)
    sz[B_KT] = B * (size_t)std::max(p.Nq * p.C, sparse ? p.Emax : 0) * DK * L * I;
  sz[B_S0T] = B * Nv * DV * DK * I;
  if (p.cu != nullptr) sz[B_CHUNKS] = (B * C + 1 + B + 1) * 4;   // valid-chunk table
  if (!sparse) {
    // fp16: Cb blocks for the Cb-operand H scan; fp32: W
    if (I == 2) sz[B_CB] = B * Nv * C * CB_BLOCKS * 512 * I;
    else sz[B_W] = B * Nv * C * L * DK * I;
    sz[B_SNAP] = B * Nv * (size_t)p.snap_cap * DV * DK * I;
  } else {
    const bool wall = (p.ablate & (SGDN_ABLATE_DEFERRED_W | SGDN_ABLATE_CSR)) != 0;
    if (wall) sz[B_W] = B * Nv * C * L * DK * I;   // W of every chunk
    else sz[B_CB] = B * Nv * C * (I == 2 ? CB_BLOCKS * 512 : L * L) * I;
    if (p.ablate & SGDN_ABLATE_CSR) {                 // all-chunk event lists
      sz[B_COLALL] = B * NP * C * 4;
      sz[B_RPALL] = B * (NP + 1) * 4;
    }
    if (p.ablate & SGDN_ABLATE_COMPACT_STATES) sz[B_ENTRY] = B * Nv * G * DV * DK * I;
    sz[B_SNAP] = B * (size_t)p.snap_cap * 2 * DV * DK * I;
    sz[B_SCORE] = B * Nv * C * 4;
    sz[B_SPART] = B * Nv * C * 8 * 4;
    if (sp->rank_key != nullptr) sz[B_RANK2] = B * NP * C * 4;
    sz[B_ETA] = B * Nv * 4;
    sz[B_ETAP] = B * Nv * GATE_SPLIT * 4;
    sz[B_RANK] = B * NP * C * 4;
    sz[B_PREC] = B * NP * PAIRREC_BYTES;
    sz[B_MASK] = B * NP * C;
    sz[B_TIER] = B * NP;
    sz[B_ROWPAIR] = B * NP * 4;
    sz[B_ROWPTR] = B * (NP + 1) * 4;
    sz[B_COL] = B * (size_t)p.Emax * 4;
    sz[B_PRED] = B * NP * G * 4;
    sz[B_GSLOT] = B * NP * G * 4;
    sz[B_ESLOT] = B * (size_t)p.Emax * 4;
    if (!wall && I == 4) sz[B_WPK] = B * (size_t)p.Emax * 2 * L * DK * I;   // fp32: W per event
  }
  sz[B_STATS] = B * STATS_INTS * 4;   // used when the caller passes no stats array
  size_t o = 0;
  for (int i = 0; i < B_COUNT; ++i) {
    p.off[i] = o;
    o += align256(sz[i]);
  }
  p.total = o;
}

template <typename T> T* at(void* ws, const Plan& p, Buf b) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + p.off[b]);
}

void mark(sgdn_debug* dbg, int i, hipStream_t s) {
  if (dbg != nullptr && dbg->events != nullptr && i < dbg->n_events && dbg->events[i] != nullptr)
    (void)hipEventRecord(static_cast<hipEvent_t>(dbg->events[i]), s);
}

void mark_range(sgdn_debug* dbg, int lo, int hi, hipStream_t s) {
  for (int i = lo; i <= hi; ++i) mark(dbg, i, s);
}

#define SGDN_TRY(expr)                        \
  do {                                        \
    if ((expr) != hipSuccess) return SGDN_EHIP; \
  } while (0)

IntraArgs intra_args(const Plan& pl, void* ws, const void* k, const void* v, const float* a,
                     const void* beta, int sparse) {
  IntraArgs ia{};
  ia.k = k; ia.v = v; ia.a = a; ia.beta = beta;
  ia.B = pl.B; ia.T = pl.T; ia.Nq = pl.Nq; ia.Nv = pl.Nv; ia.C = pl.C; ia.solve = pl.solve;
  ia.cu = pl.cu;
  ia.chunks = pl.cu ? at<int32_t>(ws, pl, B_CHUNKS) : nullptr;
  ia.g = at<float>(ws, pl, B_G);
  ia.gamma = at<float>(ws, pl, B_GAMMA);
  ia.fac = at<float>(ws, pl, B_FAC);
  ia.U = at<void>(ws, pl, B_U);
  const bool wall = sparse && (pl.ablate & (SGDN_ABLATE_DEFERRED_W | SGDN_ABLATE_CSR));
  // sparse: staged Cb (W of every chunk for the W controls); dense: W, or
  // with fp16 intermediates Cb for the Cb-operand H scan
  const bool cb = sparse ? !wall : pl.bf16 != 0;
  ia.W = cb ? nullptr : at<void>(ws, pl, B_W);
  ia.Cb = cb ? at<void>(ws, pl, B_CB) : nullptr;
  ia.KT = at<void>(ws, pl, B_KT);
  ia.score_part = sparse ? at<float>(ws, pl, B_SPART) : nullptr;
  return ia;
}

// The statistics words of a call: the caller's array or the workspace's.
int32_t* stats_words(const Plan& pl, void* ws, sgdn_stats* st) {
  return st != nullptr ? reinterpret_cast<int32_t*>(st) : at<int32_t>(ws, pl, B_STATS);
}
static_assert(sizeof(sgdn_stats) == STATS_INTS * sizeof(int32_t), "stats layout");

// CSR rows 0-3 hold every High-tier pair (at most 4) of a sequence.
constexpr int SPLIT_ROWS = 4;

// Packed sequences: the table of valid chunks the intra kernel walks.
int chunk_table(const Plan& pl, void* ws, hipStream_t s) {
  if (pl.cu == nullptr) return SGDN_OK;
  ChunkTableArgs ca{pl.cu, at<int32_t>(ws, pl, B_CHUNKS), pl.B, pl.T, pl.C};
  SGDN_TRY(launch_chunk_table(ca, s));
  return SGDN_OK;
}

int debug_copies(const Plan& pl, void* ws, sgdn_debug* dbg, hipStream_t st, int with_prefix) {
  if (dbg == nullptr) return SGDN_OK;
  const size_t nhc = (size_t)pl.B * pl.Nv * pl.C;
  if (dbg->g) SGDN_TRY(hipMemcpyAsync(dbg->g, at<void>(ws, pl, B_G), nhc * L * 4, hipMemcpyDeviceToDevice, st));
  if (dbg->gamma) SGDN_TRY(hipMemcpyAsync(dbg->gamma, at<void>(ws, pl, B_GAMMA), nhc * 4, hipMemcpyDeviceToDevice, st));
  if (dbg->prefix) {
    if (!with_prefix) {
      PrefixArgs pa{at<float>(ws, pl, B_GAMMA), at<double>(ws, pl, B_P), pl.B, pl.Nv, pl.C,
                    pl.cu, pl.T};
      SGDN_TRY(launch_prefix(pa, st));
    }
    SGDN_TRY(hipMemcpyAsync(dbg->prefix, at<void>(ws, pl, B_P), (size_t)pl.B * pl.Nv * (pl.C + 1) * 8,
                            hipMemcpyDeviceToDevice, st));
  }
  if (dbg->U)
    SGDN_TRY(launch_debug_u(at<void>(ws, pl, B_U), static_cast<float*>(dbg->U), pl.B, pl.Nv, pl.C, pl.bf16, st));
  return SGDN_OK;
}

// Selector scratch: rank tables (q-ranks; caller-key ranks), pair records,
// snapshot slot of every event.
struct SelectScratch { int32_t *rank, *rank_alt; void* pair_rec; int32_t* event_slot; };

int check_select(const sgdn_problem* prob, const float* score, const float* gamma, const float* eta,
                 const sgdn_sparse_params* params, const uint8_t* mask, const uint8_t* tier,
                 const int32_t* row_pair, const int32_t* row_ptr, const int32_t* col,
                 const int32_t* pred, const int32_t* group_slot) {
  int st = check_problem(prob);
  if (st != SGDN_OK) return st;
  if ((st = check_params(prob, params)) != SGDN_OK) return st;
  if (!score || !gamma || !eta || !mask || !tier || !row_pair || !row_ptr || !col || !pred ||
      !group_slot)
    return SGDN_EINVAL;
  return SGDN_OK;
}

int launch_select_call(const Plan& pl, const float* score, const float* gamma, const float* eta,
                       const sgdn_sparse_params* params, uint8_t* mask, uint8_t* tier,
                       int32_t* row_pair, int32_t* row_ptr, int32_t* col, int32_t* pred,
                       int32_t* group_slot, sgdn_stats* stats, const SelectScratch& sc,
                       hipStream_t s) {
  SelectArgs sa{};
  sa.score = score; sa.gamma = gamma; sa.eta = eta;
  sa.B = pl.B; sa.C = pl.C; sa.keep_bp = budget_bp(params->keep_budget);
  rates_bp(params, sa.rate_bp);
  sa.cu = pl.cu; sa.T = pl.T;
  sa.fixed_tiers = params->fixed_tiers; sa.unit_visibility = params->unit_visibility;
  sa.rank_key = params->rank_key;
  sa.rank_alt = sc.rank_alt;
  sa.rank = sc.rank; sa.pair_rec = sc.pair_rec;
  sa.mask = mask; sa.tier = tier; sa.row_pair = row_pair; sa.row_ptr = row_ptr; sa.col = col;
  sa.pred = pred; sa.group_slot = group_slot; sa.event_slot = sc.event_slot;
  sa.Emax = NP_SPARSE * pl.kH; sa.G = pl.G;
  sa.stats = stats; sa.nf_clear = 1; sa.mask_in = nullptr;
  SGDN_TRY(launch_select_full(sa, s));
  return SGDN_OK;
}

// ---- scratch of sgdn_select_noalloc --------------------------------------
// A file-scope device array instead of a caller workspace.  Each device
// the library runs on holds its own copy until the process ends; its address
// on a device comes from hipGetSymbolAddress, taken once per device (on the
// first call there, with that device current) and kept.  The array's name
// itself is a host-side stand-in and is never passed to a kernel or a copy.
// Every call on a device shares that device's copy: calls that overlap on
// one device race.  Nothing in it needs to start at zero (every entry the
// selector reads is written by the same call first).
__device__ __align__(256) static unsigned char scratch[SGDN_NOALLOC_SCRATCH_BYTES];
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[MAX_DEVICES] = {};

int noalloc_scratch(char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return SGDN_EHIP;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return SGDN_EHIP;
    g_scratch_ptr[dev] = static_cast<char*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return SGDN_OK;
}

// Offsets of the four selector arrays inside the scratch (256-byte aligned);
// returns the bytes used.
size_t noalloc_layout(const Plan& pl, bool with_key, size_t off[4]) {
  const size_t ranks = align256((size_t)pl.B * NP_SPARSE * pl.C * 4);
  off[0] = 0;
  off[1] = ranks;
  off[2] = off[1] + (with_key ? ranks : 0);
  off[3] = off[2] + align256((size_t)pl.B * NP_SPARSE * PAIRREC_BYTES);
  return off[3] + align256((size_t)pl.B * NP_SPARSE * pl.kH * 4);
}

}  // namespace

extern "C" {

const char* sgdn_status_string(int status) {
  switch (status) {
    case SGDN_OK: return "ok";
    case SGDN_EINVAL: return "invalid argument";
    case SGDN_EUNSUPPORTED: return "unsupported problem";
    case SGDN_EWORKSPACE: return "workspace too small";
    case SGDN_EHIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

size_t sgdn_workspace_bytes(const sgdn_problem* prob, int sparse, const sgdn_sparse_params* params) {
  if (check_problem(prob) != SGDN_OK) return 0;
  if (sparse && check_params(prob, params) != SGDN_OK) return 0;
  Plan pl;
  make_plan(prob, sparse, params, pl);
  return pl.total;
}

int sgdn_event_capacity(const sgdn_problem* prob, const sgdn_sparse_params* params, int32_t* k,
                        int32_t* e_max) {
  int st = check_problem(prob);
  if (st != SGDN_OK) return st;
  if ((st = check_params(prob, params)) != SGDN_OK) return st;
  if (e_max == nullptr) return SGDN_EINVAL;
  Plan pl;
  make_plan(prob, 1, params, pl);
  if (k != nullptr) {
    k[0] = pl.kL; k[1] = pl.kM; k[2] = pl.kH;
  }
  *e_max = NP_SPARSE * pl.kH;
  return SGDN_OK;
}

int sgdn_fp64_selftest(const double* x, const double* y, double* quot, double* root, int64_t n,
                       void* stream) {
  if (n < 0) return SGDN_EINVAL;
  if (n > 0 && (!x || !y || !quot || !root)) return SGDN_EINVAL;
  SGDN_TRY(launch_fp64_selftest(x, y, quot, root, (long long)n, static_cast<hipStream_t>(stream)));
  return SGDN_OK;
}

int sgdn_prefill_dense(const sgdn_problem* prob, const void* q, const void* k, const void* v,
                       const float* a, const void* beta, const float* s0, void* o,
                       float* s_final, sgdn_stats* stats, void* ws, size_t ws_bytes, void* stream,
                       sgdn_debug* dbg) {
  int st = check_problem(prob);
  if (st != SGDN_OK) return st;
  if (!q || !k || !v || !a || !beta || !o || !ws) return SGDN_EINVAL;
  Plan pl;
  make_plan(prob, 0, nullptr, pl);
  if (ws_bytes < pl.total) return SGDN_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* stw = stats_words(pl, ws, stats);

  mark(dbg, SGDN_EV_START, s);
  SGDN_TRY(launch_stats_init(StatsInitArgs{stw, pl.B, pl.Nv, pl.C, pl.T, pl.cu, 1}, s));
  if ((st = chunk_table(pl, ws, s)) != SGDN_OK) return st;
  IntraArgs ia = intra_args(pl, ws, k, v, a, beta, 0);
  ia.stats = stw;
  SGDN_TRY(launch_intra(ia, pl.bf16, s));
  mark(dbg, SGDN_EV_INTRA, s);
  if ((st = debug_copies(pl, ws, dbg, s, 0)) != SGDN_OK) return st;
  if (s0 != nullptr) {
    S0PrepArgs sa{s0, at<void>(ws, pl, B_S0T), pl.B, pl.Nv, stw};
    SGDN_TRY(launch_s0prep(sa, pl.bf16, s));
  }
  EvRecArgs ea{};
  ea.gamma = at<float>(ws, pl, B_GAMMA); ea.rec = at<int32_t>(ws, pl, B_REC);
  ea.B = pl.B; ea.Nv = pl.Nv; ea.C = pl.C; ea.sparse = 0;
  SGDN_TRY(launch_evrec(ea, s));
  mark_range(dbg, SGDN_EV_PREFIX, SGDN_EV_DEFERRED, s);
  HScanArgs ha{};
  ha.KT = at<void>(ws, pl, B_KT); ha.W = at<void>(ws, pl, B_W); ha.U = at<void>(ws, pl, B_U);
  ha.k = k;
  ha.fac = at<float>(ws, pl, B_FAC); ha.rec = ea.rec; ha.P = nullptr;
  ha.s0 = s0; ha.s_final = s_final; ha.snap = at<void>(ws, pl, B_SNAP);
  ha.B = pl.B; ha.Nq = pl.Nq; ha.Nv = pl.Nv; ha.C = pl.C; ha.sparse = 0;
  ha.cu = pl.cu; ha.T = pl.T;
  ha.Cb = at<void>(ws, pl, B_CB); ha.blockadj = pl.solve == SGDN_SOLVE_BLOCKADJ;
  ha.row_lo = 0; ha.nrows = pl.Nv / 2; ha.xcd_shift = 0;
  ha.stats = stw;
  SGDN_TRY(launch_hscan(ha, pl.bf16, s));
  mark(dbg, SGDN_EV_HSCAN, s);
  OChunkArgs oa{};
  oa.stats = stw;
  oa.q = q; oa.k = k; oa.U = at<void>(ws, pl, B_U); oa.snap = at<void>(ws, pl, B_SNAP);
  oa.s0T = s0 ? at<void>(ws, pl, B_S0T) : nullptr;
  oa.o_type = prob->o_dtype;
  oa.g = at<float>(ws, pl, B_G); oa.gamma = at<float>(ws, pl, B_GAMMA); oa.P = nullptr;
  oa.o = o; oa.B = pl.B; oa.T = pl.T; oa.Nq = pl.Nq; oa.Nv = pl.Nv; oa.C = pl.C; oa.G = pl.G;
  oa.cu = pl.cu;
  oa.row_lo = 0; oa.nrows = pl.Nv / 2;
  oa.sparse = 0;
  SGDN_TRY(launch_ochunk(oa, pl.bf16, s));
  mark(dbg, SGDN_EV_O, s);
  return SGDN_OK;
}

int sgdn_decode_step(const sgdn_problem* prob, const void* q, const void* k, const void* v,
                     const float* a, const void* beta, const float* s_in, float* s_out, void* o,
                     void* stream) {
  if (prob == nullptr) return SGDN_EINVAL;
  const sgdn_problem& pr = *prob;
  if (pr.batch < 1 || pr.seqlen != 1 || pr.n_qk < 1 || pr.n_v < 1) return SGDN_EINVAL;
  if (pr.cu_seqlens != nullptr) return SGDN_EINVAL;
  if (pr.dtype != SGDN_F32 && pr.dtype != SGDN_BF16) return SGDN_EINVAL;
  if (pr.o_dtype != SGDN_F32 && pr.o_dtype != SGDN_BF16 && pr.o_dtype != SGDN_F16)
    return SGDN_EINVAL;
  if (pr.d_k != 128 || pr.d_v != 128 || pr.n_v % pr.n_qk != 0) return SGDN_EUNSUPPORTED;
  if ((long long)pr.batch * pr.n_v > (1LL << 29)) return SGDN_EUNSUPPORTED;
  if (!q || !k || !v || !a || !beta || !s_in || !s_out || !o) return SGDN_EINVAL;
  const size_t sbytes = (size_t)pr.batch * pr.n_v * DK * DV * sizeof(float);
  const char* i0 = reinterpret_cast<const char*>(s_in);
  const char* o0 = reinterpret_cast<const char*>(s_out);
  if (i0 != o0 && i0 < o0 + sbytes && o0 < i0 + sbytes) return SGDN_EINVAL;
  if (((uintptr_t)s_in | (uintptr_t)s_out) & 15) return SGDN_EINVAL;   // 16-byte vector access
  DecodeArgs da{q, k, v, a, beta, s_in, s_out, o, pr.batch, pr.n_qk, pr.n_v, pr.o_dtype};
  SGDN_TRY(launch_decode(da, pr.dtype == SGDN_BF16, static_cast<hipStream_t>(stream)));
  return SGDN_OK;
}

int sgdn_select(const sgdn_problem* prob, const float* score, const float* gamma, const float* eta,
                const sgdn_sparse_params* params, uint8_t* mask, uint8_t* tier, int32_t* row_pair,
                int32_t* row_ptr, int32_t* col, int32_t* pred, int32_t* group_slot,
                sgdn_stats* stats, void* ws, size_t ws_bytes, void* stream) {
  int st = check_select(prob, score, gamma, eta, params, mask, tier, row_pair, row_ptr, col, pred,
                        group_slot);
  if (st != SGDN_OK) return st;
  if (!ws) return SGDN_EINVAL;
  Plan pl;
  make_plan(prob, 1, params, pl);
  if (ws_bytes < pl.total) return SGDN_EWORKSPACE;
  SelectScratch sc{at<int32_t>(ws, pl, B_RANK), params->rank_key ? at<int32_t>(ws, pl, B_RANK2) : nullptr,
                   at<void>(ws, pl, B_PREC), at<int32_t>(ws, pl, B_ESLOT)};
  return launch_select_call(pl, score, gamma, eta, params, mask, tier, row_pair, row_ptr, col, pred,
                            group_slot, stats, sc, static_cast<hipStream_t>(stream));
}

int sgdn_select_noalloc(const sgdn_problem* prob, const float* score, const float* gamma,
                        const float* eta, const sgdn_sparse_params* params, uint8_t* mask,
                        uint8_t* tier, int32_t* row_pair, int32_t* row_ptr, int32_t* col,
                        int32_t* pred, int32_t* group_slot, sgdn_stats* stats, void* stream) {
  int st = check_select(prob, score, gamma, eta, params, mask, tier, row_pair, row_ptr, col, pred,
                        group_slot);
  if (st != SGDN_OK) return st;
  Plan pl;
  make_plan(prob, 1, params, pl);
  size_t off[4];
  if (noalloc_layout(pl, params->rank_key != nullptr, off) > SGDN_NOALLOC_SCRATCH_BYTES)
    return SGDN_EWORKSPACE;
  char* base = nullptr;
  if ((st = noalloc_scratch(&base)) != SGDN_OK) return st;
  SelectScratch sc{reinterpret_cast<int32_t*>(base + off[0]),
                   params->rank_key ? reinterpret_cast<int32_t*>(base + off[1]) : nullptr,
                   static_cast<void*>(base + off[2]), reinterpret_cast<int32_t*>(base + off[3])};
  return launch_select_call(pl, score, gamma, eta, params, mask, tier, row_pair, row_ptr, col, pred,
                            group_slot, stats, sc, static_cast<hipStream_t>(stream));
}

int sgdn_prefill_sparse(const sgdn_problem* prob, const void* q, const void* k, const void* v,
                        const float* a, const void* beta, const void* z,
                        const sgdn_sparse_params* params, const uint8_t* mask_override,
                        const float* s0, void* o, float* s_final, sgdn_stats* stats, void* ws,
                        size_t ws_bytes, void* stream, sgdn_debug* dbg) {
  int st = check_problem(prob);
  if (st != SGDN_OK) return st;
  if ((st = check_params(prob, params)) != SGDN_OK) return st;
  if (!q || !k || !v || !a || !beta || !o || !ws) return SGDN_EINVAL;
  if (z == nullptr && mask_override == nullptr) return SGDN_EINVAL;
  Plan pl;
  make_plan(prob, 1, params, pl);
  if (ws_bytes < pl.total) return SGDN_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int NP = pl.Nv / 2;
  int32_t* stw = stats_words(pl, ws, stats);

  // intra: local solve, U, staged Cb, tail score, gamma
  mark(dbg, SGDN_EV_START, s);
  SGDN_TRY(launch_stats_init(StatsInitArgs{stw, pl.B, pl.Nv, pl.C, pl.T, pl.cu, 0}, s));
  if ((st = chunk_table(pl, ws, s)) != SGDN_OK) return st;
  IntraArgs ia = intra_args(pl, ws, k, v, a, beta, 1);
  ia.stats = stw;
  SGDN_TRY(launch_intra(ia, pl.bf16, s));
  mark(dbg, SGDN_EV_INTRA, s);
  // tail scores, prefix and (with the selector) gate energies in one launch
  ScoreArgs sca{at<float>(ws, pl, B_SPART), at<float>(ws, pl, B_SCORE),
                (long long)pl.B * pl.Nv * pl.C, params->tail};
  PrefixArgs pa{at<float>(ws, pl, B_GAMMA), at<double>(ws, pl, B_P), pl.B, pl.Nv, pl.C,
                pl.cu, pl.T};
  GateArgs ga{z, params->norm_weight, at<float>(ws, pl, B_ETAP), pl.B, pl.T, pl.Nv, pl.C, pl.cu, stw};
  SGDN_TRY(launch_prep(pa, mask_override == nullptr ? &ga : nullptr, sca, pl.bf16, s));
  mark(dbg, SGDN_EV_PREFIX, s);
  if ((st = debug_copies(pl, ws, dbg, s, 1)) != SGDN_OK) return st;
  mark(dbg, SGDN_EV_GATE, s);

  // selector and event layout
  const int Emax = mask_override ? NP * pl.C : NP * pl.kH;
  SelectArgs sa{};
  sa.score = at<float>(ws, pl, B_SCORE); sa.gamma = at<float>(ws, pl, B_GAMMA);
  sa.eta = at<float>(ws, pl, B_ETA);
  sa.eta_part = at<float>(ws, pl, B_ETAP); sa.eta_out = at<float>(ws, pl, B_ETA);
  sa.B = pl.B; sa.C = pl.C; sa.keep_bp = budget_bp(params->keep_budget);
  rates_bp(params, sa.rate_bp);
  sa.cu = pl.cu; sa.T = pl.T;
  sa.fixed_tiers = params->fixed_tiers; sa.unit_visibility = params->unit_visibility;
  sa.pair_order = (pl.ablate & SGDN_ABLATE_TIER_SCHEDULE) != 0;
  sa.rank_key = params->rank_key;
  sa.rank_alt = params->rank_key ? at<int32_t>(ws, pl, B_RANK2) : nullptr;
  sa.rank = at<int32_t>(ws, pl, B_RANK); sa.pair_rec = at<void>(ws, pl, B_PREC);
  sa.mask = at<uint8_t>(ws, pl, B_MASK); sa.tier = at<uint8_t>(ws, pl, B_TIER);
  sa.row_pair = at<int32_t>(ws, pl, B_ROWPAIR); sa.row_ptr = at<int32_t>(ws, pl, B_ROWPTR);
  sa.col = at<int32_t>(ws, pl, B_COL); sa.pred = at<int32_t>(ws, pl, B_PRED);
  sa.group_slot = at<int32_t>(ws, pl, B_GSLOT); sa.event_slot = at<int32_t>(ws, pl, B_ESLOT);
  sa.Emax = Emax; sa.G = pl.G;
  sa.stats = stw; sa.nf_clear = 0;
  sa.mask_in = mask_override;
  // the selector's decide kernel also writes the event records (one launch
  // fewer) on the default path with fp16 intermediates
  const bool wall = (pl.ablate & (SGDN_ABLATE_DEFERRED_W | SGDN_ABLATE_CSR)) != 0;
  const bool csr_off = (pl.ablate & SGDN_ABLATE_CSR) != 0;
  const bool rec_in_select = pl.bf16 && !wall && mask_override == nullptr;
  sa.P = at<double>(ws, pl, B_P);
  sa.rec = rec_in_select ? at<int32_t>(ws, pl, B_REC) : nullptr;
  SGDN_TRY(launch_select_full(sa, s));
  mark(dbg, SGDN_EV_SELECT, s);
  if (dbg != nullptr) {
    if (dbg->score) SGDN_TRY(hipMemcpyAsync(dbg->score, sa.score, (size_t)pl.B * pl.Nv * pl.C * 4, hipMemcpyDeviceToDevice, s));
    if (dbg->eta && !mask_override) SGDN_TRY(hipMemcpyAsync(dbg->eta, sa.eta, (size_t)pl.B * pl.Nv * 4, hipMemcpyDeviceToDevice, s));
    if (dbg->mask) SGDN_TRY(hipMemcpyAsync(dbg->mask, sa.mask, (size_t)pl.B * NP * pl.C, hipMemcpyDeviceToDevice, s));
    if (dbg->tier) SGDN_TRY(hipMemcpyAsync(dbg->tier, sa.tier, (size_t)pl.B * NP, hipMemcpyDeviceToDevice, s));
  }

  // deferred W of the kept events (the deferred-W ablation has W of every
  // chunk from the intra stage instead) and event records
  DeferredWArgs da{};
  da.k = k; da.Cb = at<void>(ws, pl, B_CB); da.Wpk = pl.bf16 ? nullptr : at<void>(ws, pl, B_WPK);
  da.KTpk = at<void>(ws, pl, B_KT); da.cu = pl.cu; da.T = pl.T;
  da.row_pair = sa.row_pair; da.row_ptr = sa.row_ptr; da.col = sa.col;
  da.B = pl.B; da.Nv = pl.Nv; da.Nq = pl.Nq; da.C = pl.C; da.Emax = Emax; da.solve = pl.solve;
  EvRecArgs ea{};
  ea.gamma = at<float>(ws, pl, B_GAMMA); ea.P = at<double>(ws, pl, B_P);
  ea.row_pair = sa.row_pair; ea.row_ptr = sa.row_ptr; ea.col = sa.col; ea.event_slot = sa.event_slot;
  ea.rec = at<int32_t>(ws, pl, B_REC);
  ea.B = pl.B; ea.Nv = pl.Nv; ea.C = pl.C; ea.Emax = Emax; ea.sparse = 1;
  EvAllArgs xa_all{ea.gamma, ea.P, sa.mask, sa.row_pair, sa.row_ptr, sa.event_slot, ea.rec,
                    at<int32_t>(ws, pl, B_COLALL), at<int32_t>(ws, pl, B_RPALL),
                    pl.B, pl.Nv, pl.C, Emax};
  auto events = [&](int lo, int hi, hipStream_t q) -> hipError_t {
    if (csr_off) return launch_evrec_all(xa_all, q);   // every chunk an event
    ea.row_lo = lo; ea.row_hi = hi;
    // fp16 intermediates: the H scan forms W S = Cb (K S) with K^T taken
    // from the key rows, so the kept events need only their records (on the
    // default path written by the selector already)
    if (rec_in_select) return hipSuccess;
    if (wall || pl.bf16) return launch_evrec(ea, q);
    da.row_lo = lo; da.row_hi = hi;
    return launch_events(da, ea, q);                   // fp32: deferred W and the records
  };
  if (s0 != nullptr) {
    S0PrepArgs s0a{s0, at<void>(ws, pl, B_S0T), pl.B, pl.Nv, stw};
    SGDN_TRY(launch_s0prep(s0a, pl.bf16, s));
  }
  HScanArgs ha{};
  ha.KT = at<void>(ws, pl, B_KT); ha.W = at<void>(ws, pl, wall ? B_W : B_WPK); ha.U = at<void>(ws, pl, B_U);
  ha.k = k;
  ha.w_by_chunk = wall;
  ha.Cb = at<void>(ws, pl, B_CB); ha.blockadj = pl.solve == SGDN_SOLVE_BLOCKADJ;
  ha.fac = at<float>(ws, pl, B_FAC); ha.rec = ea.rec; ha.P = at<double>(ws, pl, B_P);
  ha.s0 = s0; ha.s_final = s_final; ha.snap = at<void>(ws, pl, B_SNAP);
  ha.B = pl.B; ha.Nq = pl.Nq; ha.Nv = pl.Nv; ha.C = pl.C; ha.sparse = 1;
  ha.cu = pl.cu; ha.T = pl.T;   // (sequence offsets of the key rows)
  ha.row_pair = sa.row_pair; ha.row_ptr = sa.row_ptr; ha.col = sa.col; ha.event_slot = sa.event_slot;
  ha.Emax = Emax; ha.snap_cap = pl.snap_cap;
  ha.stats = stw;
  if (csr_off) {
    ha.row_ptr = xa_all.row_ptr_all; ha.col = xa_all.col_all; ha.Emax = NP * pl.C;
  }
  OChunkArgs oa{};
  oa.q = q; oa.k = k; oa.U = at<void>(ws, pl, B_U); oa.snap = at<void>(ws, pl, B_SNAP);
  oa.s0T = s0 ? at<void>(ws, pl, B_S0T) : nullptr;
  oa.o_type = prob->o_dtype;
  oa.g = at<float>(ws, pl, B_G); oa.gamma = at<float>(ws, pl, B_GAMMA); oa.P = at<double>(ws, pl, B_P);
  oa.o = o; oa.B = pl.B; oa.T = pl.T; oa.Nq = pl.Nq; oa.Nv = pl.Nv; oa.C = pl.C; oa.G = pl.G;
  oa.cu = pl.cu; oa.row_pair = sa.row_pair;
  oa.sparse = 1; oa.pred = sa.pred; oa.group_slot = sa.group_slot; oa.snap_cap = pl.snap_cap;
  oa.stats = stw;

  SGDN_TRY(events(0, NP, s));
  mark(dbg, SGDN_EV_DEFERRED, s);

  // compact-states ablation: dense group-entry states for O, per row range
  const bool dense_entry = (pl.ablate & SGDN_ABLATE_COMPACT_STATES) != 0;
  ExpandArgs xa{at<void>(ws, pl, B_SNAP), s0 ? at<void>(ws, pl, B_S0T) : nullptr,
                at<double>(ws, pl, B_P), sa.pred, sa.group_slot,
                dense_entry ? at<void>(ws, pl, B_ENTRY) : nullptr,
                pl.B, pl.Nv, pl.C, pl.G, pl.snap_cap, pl.T, pl.cu, sa.row_pair, 0, NP};
  oa.entry = xa.entry;
  oa.per_chunk = (pl.ablate & SGDN_ABLATE_MAPPED_O) != 0;
  auto expand = [&](int lo, int n, hipStream_t q) -> hipError_t {
    if (!dense_entry) return hipSuccess;
    xa.row_lo = lo; xa.nrows = n;
    return launch_expand(xa, pl.bf16, q);
  };

  // (With several sequences and every tier keeping the same count, all
  // chains are equally long: nothing overlaps, and the O launch of rows 0-3
  // would cut into the second round of H-scan workgroups; one launch each.
  // Sequences of at most 64 chunks take one launch each as well: there the
  // stages are short and the fork and join cost more than the overlap
  // gains, 2.61 vs 2.29 ms per 24 layers of 2048 tokens, even at 4096, and
  // 5.24 vs 5.77 ms at 8192.)
  const bool fork_rows = pl.C > 64 && (pl.B == 1 || pl.kL != pl.kH);
  if (!(pl.ablate & SGDN_ABLATE_TIER_SCHEDULE) && params->aux_stream != nullptr && fork_rows) {
    // CSR rows 0-3 of a sequence hold every High-tier pair (at most 4), whose
    // chains are the longest and bound the H scan.  The H scan and O of rows
    // 4-15 of every sequence run on the caller's second stream beside those
    // of rows 0-3, so O of the shorter chains overlaps the long ones (with
    // many sequences the H scan's total work rather than its longest chains
    // sets its time, and the gain shrinks: -5% at 2 x 32K tokens, -1% at 4
    // and 8).  Both H-scan launches spread
    // each pair group over two XCDs (one head on each): rows 4-15 put 24
    // workgroups and rows 0-3 put 8 on every XCD, whatever XCD each launch's
    // round-robin dispatch starts at, so every chain finds a CU at once.
    // (Splitting deferred W and the event records the same way, or moving
    // the gate energy beside the intra kernel, measured no faster: the GPU
    // is busy in those phases.)
    hipStream_t aux = static_cast<hipStream_t>(params->aux_stream);
    hipEvent_t fork = static_cast<hipEvent_t>(params->aux_events[0]);
    hipEvent_t join = static_cast<hipEvent_t>(params->aux_events[1]);
    SGDN_TRY(hipEventRecord(fork, s));
    SGDN_TRY(hipStreamWaitEvent(aux, fork, 0));
    ha.row_lo = SPLIT_ROWS; ha.nrows = NP - SPLIT_ROWS; ha.xcd_shift = SPLIT_ROWS; ha.spread = pl.bf16;
    SGDN_TRY(launch_hscan(ha, pl.bf16, aux));
    SGDN_TRY(expand(SPLIT_ROWS, NP - SPLIT_ROWS, aux));
    oa.row_lo = SPLIT_ROWS; oa.nrows = NP - SPLIT_ROWS;
    SGDN_TRY(launch_ochunk(oa, pl.bf16, aux));
    SGDN_TRY(hipEventRecord(join, aux));
    // The High-tier chains of rows 0-3 keep CUs busy long after the other
    // rows' H scan; spread over two XCDs per pair they leave three quarters
    // of those XCDs' CUs free, so the O launch beside them (whose workgroups
    // are dealt to the XCDs in equal shares) is not held up by an XCD that
    // has only half of its CUs.
    ha.row_lo = 0; ha.nrows = SPLIT_ROWS; ha.xcd_shift = 0; ha.spread = pl.bf16;
    SGDN_TRY(launch_hscan(ha, pl.bf16, s));
    ha.spread = 0;
    SGDN_TRY(expand(0, SPLIT_ROWS, s));
    mark(dbg, SGDN_EV_HSCAN, s);
    oa.row_lo = 0; oa.nrows = SPLIT_ROWS;
    SGDN_TRY(launch_ochunk(oa, pl.bf16, s));
    SGDN_TRY(hipStreamWaitEvent(s, join, 0));
    mark(dbg, SGDN_EV_O, s);
    return SGDN_OK;
  }

  ha.row_lo = 0; ha.nrows = NP; ha.xcd_shift = 0;
  SGDN_TRY(launch_hscan(ha, pl.bf16, s));
  SGDN_TRY(expand(0, NP, s));
  mark(dbg, SGDN_EV_HSCAN, s);
  oa.row_lo = 0; oa.nrows = NP;
  SGDN_TRY(launch_ochunk(oa, pl.bf16, s));
  mark(dbg, SGDN_EV_O, s);
  return SGDN_OK;
}

}  // extern "C"
