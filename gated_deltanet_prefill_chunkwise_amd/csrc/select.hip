// Dynamic event selector and CSR event layout (SparseGDN reading notes,
// Sec. 2.4, Eqs. (10)-(14); Sec. 2.5, Eq. (16)).
//
// Every floating-point value that decides an integer (rank, tier count, tier,
// mask) is evaluated in IEEE binary64 with these fixed rules, so identical
// fp32 statistics always give identical decisions:
//  * only correctly rounded +, -, *, /, sqrt; FMA contraction is off in this
//    file (pragma below and -ffp-contract=off);
//  * a sum over a sequence x[0..n) is taken as 64 interleaved running sums
//    (lane l adds x[l], x[l+64], ... in order, starting from 0), then
//    combined pairwise: for w = 32, 16, ..., 1, lane l < w adds lane l + w;
//  * 2^x: x clamped to [-2000, 1000], n = rint(x), f = x - n,
//    y = f * ln2 (binary64 nearest), Taylor sum_{i<=14} y^i / i! by Horner
//    from i = 14 down, then ldexp(., n);
//  * r^n for integer n: binary powering from the least significant bit;
//  * orderings (rank keys, pair gains) treat NaN as -infinity, so that they
//    stay total orders (a rank is a permutation, each tier gets its count)
//    even when non-finite inputs reach the statistics.
#pragma clang fp contract(off)

#include "common.h"
#include "kernels.h"

namespace sgdn {

namespace {

constexpr int NP = 16;   // head pairs (the tier table is written for 16)
constexpr int NV = 32;

constexpr double kLn2 = 0.6931471805599453;
// 1 / i! for i = 0..14, each rounded once from the exact quotient
constexpr double kInvFact[15] = {
    1.0 / 1.0, 1.0 / 1.0, 1.0 / 2.0, 1.0 / 6.0, 1.0 / 24.0, 1.0 / 120.0,
    1.0 / 720.0, 1.0 / 5040.0, 1.0 / 40320.0, 1.0 / 362880.0,
    1.0 / 3628800.0, 1.0 / 39916800.0, 1.0 / 479001600.0,
    1.0 / 6227020800.0, 1.0 / 87178291200.0};

__device__ double wave_sum(double p) {
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) {
    const double o = __shfl_down(p, w, 64);
    p = p + o;
  }
  return __shfl(p, 0, 64);
}

__device__ double exp2_fixed(double x) {
  x = fmax(-2000.0, fmin(1000.0, x));
  const double n = rint(x);
  const double f = x - n;
  const double y = f * kLn2;
  double pp = kInvFact[14];
#pragma unroll
  for (int i = 13; i >= 0; --i) pp = pp * y + kInvFact[i];
  return ldexp(pp, (int)n);
}

__device__ __forceinline__ double ord_key(double x) { return x != x ? -__builtin_inf() : x; }

// Orders one wave's LDS writes before its later LDS reads by other lanes.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ double powi_fixed(double r, int n) {
  double res = 1.0, base = r;
  while (n) {
    if (n & 1) res = res * base;
    base = base * base;
    n >>= 1;
  }
  return res;
}

// Valid chunks of sequence b (Sec. 2.4 counts, ranks and anchors them per
// sequence); arrays keep the stride p.C.
__device__ int valid_chunks(const SelectArgs& p, int b) {
  return p.cu == nullptr ? p.C : chunks_of(seq_span(p.cu, b, p.T).len);
}

// k = clip(round(rho C), 2, C) (Sec. 2.4.3) in exact integer arithmetic with
// halves rounded up.  With the caller's rates (rbp[0] > 0, basis points) rho
// is those; otherwise rho = (0.08, 0.30, 0.95) at a budget of 2900 bp, scaled
// linearly below it and towards 1 above it.  k = 1 when C = 1 and 0 for an
// empty sequence.
__device__ void tier_counts(int C, int bp, const int rbp[3], int k[3]) {
  const int pct[3] = {8, 30, 95};
#pragma unroll
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

// L_h = sum_{j=1}^{C-2} r^j in closed form (Eq. (11)).
__device__ double lifetime(double r, int C) {
  const int n = C - 2;
  if (n <= 0) return 0.0;
  if (r == 1.0) return (double)n;
  return r * (1.0 - powi_fixed(r, n)) / (1.0 - r);
}

// Eq. (10): per-head norms of the tail scores, the within-pair rank key q and
// the rank of every non-anchor chunk (q descending, chunk index ascending).
// Workgroup (blk, pp, b) ranks chunks 128 blk .. 128 blk + 127 of pair pp:
// eight threads per chunk count disjoint eighths of the other chunks.  Every
// workgroup stages the pair's scores in LDS and forms the norms and keys
// itself, with the same operations.  KEY: rank by the caller's keys instead
// (the random-selection ablation), into rank_alt.
// Dynamic LDS: C doubles (keys) + 2 C floats (scores).
constexpr int RANK_CHUNKS = 128;
constexpr int MAX_C = 8192;
template <bool KEY>
__global__ __launch_bounds__(1024) void select_rank_kernel(SelectArgs p) {
  extern __shared__ double sq[];
  __shared__ double snorm[2];
  const int blk = blockIdx.x, pp = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int CS = p.C, C = valid_chunks(p, b);
  if (KEY) {
    const float* key = p.rank_key + ((size_t)b * NP + pp) * CS;
    for (int c = tid; c < C; c += 1024) sq[c] = ord_key((double)key[c]);
  } else {
    float* ss = reinterpret_cast<float*>(sq + CS);   // [2][CS] staged scores
    const float* s0 = p.score + ((size_t)b * NV + 2 * pp) * CS;
    const float* s1 = s0 + CS;
    {
      // every load of a thread is issued before the first store
      constexpr int U = MAX_C / 1024;
      float x0[U], x1[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = tid + 1024 * u;
        x0[u] = c < C ? s0[c] : 0.f;
        x1[u] = c < C ? s1[c] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = tid + 1024 * u;
        if (c < C) { ss[c] = x0[u]; ss[CS + c] = x1[u]; }
      }
    }
    __syncthreads();
    if (w < 2) {
      const float* s = ss + w * CS;
      double acc = 0.0;
      for (int c = lane; c < C; c += 64) {
        const double x = (double)s[c];
        acc = acc + x * x;
      }
      const double tot = wave_sum(acc);
      if (lane == 0) snorm[w] = sqrt(tot);
    }
    __syncthreads();
    const double n0 = snorm[0], n1 = snorm[1];
    for (int c = tid; c < C; c += 1024) {
      const double t0 = n0 > 0.0 ? (double)ss[c] / n0 : 0.0;
      const double t1 = n1 > 0.0 ? (double)ss[CS + c] / n1 : 0.0;
      sq[c] = ord_key(0.5 * (t0 + t1));
    }
  }
  __syncthreads();
  int32_t* rk = (KEY ? p.rank_alt : p.rank) + ((size_t)b * NP + pp) * CS;
  const int c = RANK_CHUNKS * blk + (tid >> 3), part = tid & 7;
  int r = 0;
  if (c >= 1 && c <= C - 2) {
    // candidates c2 = 1 + part + 8 j (j < J, c2 <= C - 2): one before c
    // outranks it when q2 >= qc (ties go to the lower chunk), one after it
    // when q2 > qc; c2 = c counts neither way
    const double qc = sq[c];
    const double* qb = sq + 1 + part;
    const int J = C - 3 - part >= 0 ? (C - 3 - part) / 8 + 1 : 0;
    const int js = min(c - 1 - part > 0 ? (c - 1 - part + 7) / 8 : 0, J);
    int j = 0;
    for (; j + 8 <= js; j += 8) {
      double v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = qb[8 * (j + u)];
#pragma unroll
      for (int u = 0; u < 8; ++u) r += v[u] >= qc ? 1 : 0;
    }
    for (; j < js; ++j) r += qb[8 * j] >= qc ? 1 : 0;
    for (; j + 8 <= J; j += 8) {
      double v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = qb[8 * (j + u)];
#pragma unroll
      for (int u = 0; u < 8; ++u) r += v[u] > qc ? 1 : 0;
    }
    for (; j < J; ++j) r += qb[8 * j] > qc ? 1 : 0;
  }
  // the eight partial counts of a chunk sit in eight adjacent lanes
  r += __shfl_xor(r, 1, 64);
  r += __shfl_xor(r, 2, 64);
  r += __shfl_xor(r, 4, 64);
  if (part == 0 && c < C) rk[c] = (c >= 1 && c <= C - 2) ? r : -1;
}

// B(x, k) = k (n-k) / n (mean x[:k] - mean x[k:])^2 (Eq. (14)) over the
// sorted values vals[0..n) (n <= 16) for the candidate counts k0 .. k0 +
// ncand - 1 (ncand <= 4) at once; B = 0 for k <= 0 or k >= n.  Candidate s
// takes lanes 16 s .. 16 s + 15, which form its two sums as the 64-lane
// interleaved sums of the selector's rules: with at most 16 values the
// 64-lane tree's first two levels only add +0 (and no partial sum here is
// -0), so its 16-lane part gives the same results.  Returns the first count
// with the largest B (ties: the earlier one).
__device__ int best_split(const double* vals, int n, int k0, int ncand, int lane) {
  const int sg = lane >> 4, j = lane & 15;
  const int k = sg < ncand ? k0 + sg : -1;
  const bool valid = k > 0 && k < n;
  double a = (valid && j < k) ? vals[j] : 0.0;
  double c = (valid && j < n - k) ? vals[k + j] : 0.0;
#pragma unroll
  for (int w = 8; w >= 1; w >>= 1) {
    const double oa = __shfl_down(a, w, 16);
    const double oc = __shfl_down(c, w, 16);
    a = a + oa;
    c = c + oc;
  }
  double v = 0.0;
  if (valid) {
    const double m1 = a / k;
    const double m2 = c / (n - k);
    const double f = (double)(k * (n - k)) / n;
    const double dm = m1 - m2;
    v = f * (dm * dm);
  }
  int best_i = 0;
  double best = 0.0;
  for (int i = 0; i < ncand; ++i) {
    const double vi = __shfl(v, 16 * i, 64);
    if (i == 0 || vi > best) { best = vi; best_i = i; }
  }
  return k0 + best_i;
}

// Per (sequence, head pair) record handed from select_pair_kernel to
// select_decide_kernel: the upgrade gains of Eq. (12) and the number of
// referenced events (group predecessors) the pair would have in each tier.
struct PairRec {
  double glm, gmh;
  int32_t nref[3];
  int32_t pad;
};
static_assert(sizeof(PairRec) == PAIRREC_BYTES, "pair record size");

// Kept chunks of one pair as 64-bit words (bit l of word i: chunk 64 i + l)
// for keep count k, from its ranks (anchors always kept); lane = bit.
__device__ __forceinline__ unsigned long long kept_word(const int32_t* rank, int i, int lane, int C,
                                                        int k) {
  const int c = 64 * i + lane;
  bool z = false;
  if (c < C) {
    const int r = rank[c];
    z = c == 0 || c == C - 1 || (r >= 0 && r < k - 2);
  }
  return __ballot(z);
}

// Referenced events of word i: kept chunk e is the predecessor of some group
// r (2 r <= 2 (G - 1)) iff an even number lies in [e + 1, min(next kept,
// 2 (G - 1))]; nextfirst is the first kept chunk after word i (C + 1 if none).
__device__ __forceinline__ unsigned long long ref_word(unsigned long long bal, int i, int lane,
                                                       int nextfirst, int G) {
  const int c = 64 * i + lane;
  const unsigned long long above = lane == 63 ? 0ull : (bal >> (lane + 1));
  const int nxt = above ? c + 1 + (int)__builtin_ctzll(above) : nextfirst;
  const int lo = c + 1, lo_e = lo + (lo & 1), hi = min(nxt, 2 * (G - 1));
  return __ballot(((bal >> lane) & 1ull) && lo_e <= hi);
}

// Eqs. (11)-(12) for one head pair, and its referenced-event counts:
// workgroup (pp, b) stages the pair's ranks and scores, forms the kept words
// of the pair for each of the three keep counts (all but waves 0-4), finds
// the first kept chunk after every word (waves 5-7, one keep count each),
// then in parallel: waves 0-1 the band sums of head 0 and 1 (the ranks of
// Eq. (10) between k_L - 2 and k_M - 2, and between k_M - 2 and k_H - 2; each
// sum one wave's lane-interleaved sum), waves 2-3 their lifetimes (Eq. (11)),
// wave 4 the visibilities (and, in pair 0, eta from the gate kernel's parts),
// the others the referenced events with each keep count.  Dynamic LDS: 2 C
// ints (ranks, keep ranks) and 2 C floats (scores).
__global__ __launch_bounds__(1024) void select_pair_kernel(SelectArgs p) {
  extern __shared__ int32_t s_rank[];
  constexpr int NWMAX = MAX_C / 64;
  __shared__ double s_sum[4], s_L[2], s_G[2];
  __shared__ int s_nref[3];
  __shared__ unsigned long long s_kw[3][NWMAX];
  __shared__ int s_nf[3][NWMAX];
  const int pp = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const int CS = p.C, C = valid_chunks(p, b), G = (C + 1) / 2, NW = (C + 63) / 64;
  const bool key = p.rank_key != nullptr;
  int32_t* s_keep = key ? s_rank + CS : s_rank;
  float* s_sc = reinterpret_cast<float*>(s_rank + 2 * CS);
  int kk[3];
  tier_counts(C, p.keep_bp, p.rate_bp, kk);
  const int kL = kk[0], kM = kk[1], kH = kk[2];
  const int h0 = 2 * pp;
  constexpr int FIRST_REF_WAVE = 5;
  {
    const int32_t* rk = p.rank + ((size_t)b * NP + pp) * CS;
    const int32_t* ra = key ? p.rank_alt + ((size_t)b * NP + pp) * CS : nullptr;
    const float* sc = p.score + ((size_t)b * NV + h0) * CS;
    constexpr int U = MAX_C / 1024;
    int r0[U], r1[U];
    float x0[U], x1[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = tid + 1024 * u;
      r0[u] = c < C ? rk[c] : -1;
      r1[u] = (key && c < C) ? ra[c] : -1;
      x0[u] = c < C ? sc[c] : 0.f;
      x1[u] = c < C ? sc[CS + c] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = tid + 1024 * u;
      if (c < C) {
        s_rank[c] = r0[u];
        if (key) s_keep[c] = r1[u];
        s_sc[c] = x0[u];
        s_sc[CS + c] = x1[u];
      }
    }
    if (tid < 3) s_nref[tid] = 0;
  }
  __syncthreads();
  // kept words for the three keep counts (word t NW + i over the ref waves)
  for (int q = wv - FIRST_REF_WAVE; q >= 0 && q < 3 * NW; q += 16 - FIRST_REF_WAVE) {
    const int t = q / NW, i = q - t * NW;
    const unsigned long long bal = kept_word(s_keep, i, lane, C, kk[t]);
    if (lane == 0) s_kw[t][i] = bal;
  }
  __syncthreads();
  if (wv >= FIRST_REF_WAVE && wv < FIRST_REF_WAVE + 3) {
    // first kept chunk after each word (C + 1 if none): lane l holds words
    // 2 l and 2 l + 1, suffix minimum over the lanes
    const int t = wv - FIRST_REF_WAVE;
    int f2[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int i = 2 * lane + h;
      const unsigned long long bal = i < NW ? s_kw[t][i] : 0ull;
      f2[h] = bal ? 64 * i + (int)__builtin_ctzll(bal) : C + 1;
    }
    int suf = min(f2[0], f2[1]);
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int f = __shfl_down(suf, d, 64);
      if (lane + d < 64) suf = min(suf, f);
    }
    int after = __shfl_down(suf, 1, 64);
    if (lane == 63) after = C + 1;
    if (2 * lane < NW) s_nf[t][2 * lane] = min(f2[1], after);
    if (2 * lane + 1 < NW) s_nf[t][2 * lane + 1] = after;
  }
  __syncthreads();
  if (wv < 2) {
    // band sums of head wv: each lane sums its chunks in ascending order;
    // eight chunks' operands are read before their additions
    const int hh = wv;
    double alm = 0.0, amh = 0.0;
    for (int c0 = lane; c0 < C; c0 += 64 * 8) {
      int rr[8];
      float xs[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int c = c0 + 64 * u;
        rr[u] = c < C ? s_rank[c] : -1;
        xs[u] = c < C ? s_sc[hh * CS + c] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (c0 + 64 * u < C) {
          const int r = rr[u];
          const bool inm = r >= kL - 2 && r < kM - 2, inh = r >= kM - 2 && r < kH - 2;
          const double x = (double)xs[u];
          alm = alm + (inm ? x : 0.0);
          amh = amh + (inh ? x : 0.0);
        }
    }
    const double tl = wave_sum(alm), th = wave_sum(amh);
    if (lane == 0) { s_sum[hh] = tl; s_sum[2 + hh] = th; }
  } else if (wv < 4) {
    const int hh = wv - 2;
    const int lo = C > 16 ? C - 16 : 0, nwin = C - lo;
    const float* gm = p.gamma + ((size_t)b * NV + h0 + hh) * CS;
    const double xw = lane < nwin ? exp2_fixed((double)gm[lo + lane]) : 0.0;
    const double tot = wave_sum(xw);
    if (lane == 0) s_L[hh] = lifetime(tot / nwin, C);
  } else if (wv == 4) {
    // eta of head `lane`: given, or the mean from the gate kernel's parts
    float eh = 0.f;
    if (lane < NV) {
      if (p.eta_part != nullptr) {
        const float* ep = p.eta_part + ((size_t)b * NV + lane) * GATE_SPLIT;
        float t = 0.f;
        for (int i = 0; i < GATE_SPLIT; ++i) t += ep[i];
        eh = C > 0 ? t / (float)(4 * C) : 0.f;
        if (pp == 0) p.eta_out[(size_t)b * NV + lane] = eh;
      } else {
        eh = p.eta[(size_t)b * NV + lane];
      }
    }
    const double etab = wave_sum(lane < NV ? (double)eh : 0.0) / NV;
    if (lane == h0 || lane == h0 + 1)
      s_G[lane - h0] = (etab > 0.0 && !p.unit_visibility) ? sqrt((double)eh / etab) : 1.0;
  } else {
    int cnt[3] = {0, 0, 0};
    for (int q = wv - FIRST_REF_WAVE; q < 3 * NW; q += 16 - FIRST_REF_WAVE) {
      const int t = q / NW, i = q - t * NW;
      const int n = __popcll(ref_word(s_kw[t][i], i, lane, s_nf[t][i], G));
      cnt[0] += t == 0 ? n : 0;
      cnt[1] += t == 1 ? n : 0;
      cnt[2] += t == 2 ? n : 0;
    }
    if (lane == 0)
      for (int t = 0; t < 3; ++t)
        if (cnt[t]) atomicAdd(&s_nref[t], cnt[t]);
  }
  __syncthreads();
  if (tid == 0) {
    PairRec* rec = reinterpret_cast<PairRec*>(p.pair_rec) + (size_t)b * NP + pp;
    PairRec q;
    q.glm = (s_L[0] * s_G[0]) * s_sum[0] + (s_L[1] * s_G[1]) * s_sum[1];
    q.gmh = (s_L[0] * s_G[0]) * s_sum[2] + (s_L[1] * s_G[1]) * s_sum[3];
    q.nref[0] = s_nref[0]; q.nref[1] = s_nref[1]; q.nref[2] = s_nref[2];
    q.pad = 0;
    *rec = q;
  }
}

// Eqs. (13)-(14) and Eq. (16): every workgroup (pp, b) takes the sequence's
// tier decision from the pair records (the same operations in every
// workgroup, so the same tiers), orders the CSR rows (High, Medium, Low;
// ascending pair within a tier) and numbers the compact snapshots over the
// rows; then its 16 waves lay out pair pp: mask, kept chunks ascending at
// the row's offset, the snapshot slot of every event and the predecessor of
// every output group.  Workgroup 0 writes the sequence's tiers, rows and
// statistics.  Dynamic LDS: C ints (keep ranks).
__global__ __launch_bounds__(1024) void select_decide_kernel(SelectArgs p) {
  extern __shared__ int32_t s_keep[];
  constexpr int NWMAX = MAX_C / 64;
  __shared__ double sxm[NP], sxh[NP], svals[NP];
  __shared__ int sorder[NP], shigh[NP], s_tier[NP], s_rowof[NP], s_rowpair[NP];
  __shared__ int s_rowptr[NP + 1], s_refbase[NP + 1], s_nref[NP][3];
  __shared__ unsigned long long s_kept[NWMAX], s_refd[NWMAX];
  __shared__ int s_run[NWMAX], s_rrun[NWMAX], s_next[NWMAX], s_last[NWMAX];
  const int pp = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const int CS = p.C, GS = p.G, C = valid_chunks(p, b), G = (C + 1) / 2;
  const int NW = (C + 63) / 64, NWS = (CS + 63) / 64;
  int kk[3];
  tier_counts(C, p.keep_bp, p.rate_bp, kk);
  const PairRec* recs = reinterpret_cast<const PairRec*>(p.pair_rec) + (size_t)b * NP;
  // waves 1-15 stage this pair's keep ranks while wave 0 decides the tiers
  // (its steps are ordered by wave-level syncs; one workgroup barrier
  // follows)
  if (wv != 0) {
    const int32_t* src = (p.rank_key != nullptr ? p.rank_alt : p.rank) + ((size_t)b * NP + pp) * CS;
    for (int c = tid - 64; c < C; c += 1024 - 64) s_keep[c] = src[c];
  } else {
    // wave 0: the tier decision (Eqs. (13)-(14)); the records are read once
    {
      double glm = 0.0, gmh = 0.0;
      if (lane < NP) {
        const PairRec r = recs[lane];
        glm = r.glm;
        gmh = r.gmh;
        s_nref[lane][0] = r.nref[0]; s_nref[lane][1] = r.nref[1]; s_nref[lane][2] = r.nref[2];
      }
      const double mum = wave_sum(glm) / NP;
      const double muh = wave_sum(gmh) / NP;
      if (lane < NP) {
        sxm[lane] = ord_key(mum > 0.0 ? glm / mum : 0.0);
        sxh[lane] = ord_key(muh > 0.0 ? gmh / muh : 0.0);
      }
    }
    wave_sync();
    // High count: pairs sorted by x_H descending (ties: lower pair first)
    if (lane < NP) {
      int pos = 0;
      for (int q = 0; q < NP; ++q)
        pos += (sxh[q] > sxh[lane] || (sxh[q] == sxh[lane] && q < lane)) ? 1 : 0;
      sorder[pos] = lane;
    }
    wave_sync();
    if (lane < NP) svals[lane] = sxh[sorder[lane]];
    wave_sync();
    int nH = 3;               // the fixed 9 Low / 4 Medium / 3 High split
    if (!p.fixed_tiers) nH = best_split(svals, NP, 1, 4, lane);
    if (lane < NP) shigh[lane] = 0;
    wave_sync();
    if (lane < nH) shigh[sorder[lane]] = 1;
    wave_sync();
    // Medium count among the remaining pairs, sorted by x_M descending
    const int nrest = NP - nH;
    if (lane < NP && !shigh[lane]) {
      int pos = 0;
      for (int q = 0; q < NP; ++q)
        if (!shigh[q]) pos += (sxm[q] > sxm[lane] || (sxm[q] == sxm[lane] && q < lane)) ? 1 : 0;
      sorder[pos] = lane;
    }
    wave_sync();
    if (lane < nrest) svals[lane] = sxm[sorder[lane]];
    wave_sync();
    // Medium candidates for the High count (Sec. 2.4.3 table): 11-13, 7-9,
    // 3-5, or 0 with four High pairs
    const int m0 = nH == 1 ? 11 : nH == 2 ? 7 : nH == 3 ? 3 : 0;
    const int nm = nH <= 3 ? 3 : 1;
    const int nM = p.fixed_tiers ? 4 : best_split(svals, nrest, m0, nm, lane);
    if (lane < NP) {
      int t = 2;
      if (!shigh[lane]) {
        int pos = 0;   // position among the remaining pairs
        for (int q = 0; q < nrest; ++q) pos += (sorder[q] == lane) ? q : 0;
        t = pos < nM ? 1 : 0;
      }
      s_tier[lane] = t;
    }
    wave_sync();
    // rows: High first, ascending pair within a tier (head-pair order with
    // pair_order); each row holds the k of its tier events
    if (lane < NP) {
      int row = lane;
      if (!p.pair_order) {
        const int t = s_tier[lane];
        row = 0;
        for (int q = 0; q < NP; ++q)
          row += (s_tier[q] > t || (s_tier[q] == t && q < lane)) ? 1 : 0;
      }
      s_rowof[lane] = row;
      s_rowpair[row] = lane;
    }
    wave_sync();
    {
      // row offsets: exclusive scans of the events and referenced events per row
      int e = 0, f = 0;
      if (lane < NP) {
        const int q = s_rowpair[lane], tq = s_tier[q];
        e = kk[tq];
        f = s_nref[q][tq];
      }
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int ue = __shfl_up(e, d, 64), uf = __shfl_up(f, d, 64);
        if (lane >= d) { e += ue; f += uf; }
      }
      // lane r now holds the inclusive sums of rows 0 .. r
      if (lane < NP) { s_rowptr[lane + 1] = e; s_refbase[lane + 1] = f; }
      if (lane == 0) { s_rowptr[0] = 0; s_refbase[0] = 0; }
    }
    wave_sync();
    if (pp == 0) {
      if (lane < NP) {
        p.tier[b * NP + lane] = (uint8_t)s_tier[lane];
        p.row_pair[b * NP + lane] = s_rowpair[lane];
      }
      if (lane <= NP) p.row_ptr[b * (NP + 1) + lane] = s_rowptr[lane];
      if (lane == 0 && p.stats != nullptr) {
        int32_t* st = static_cast<int32_t*>(p.stats) + (size_t)b * STATS_INTS;
        if (p.nf_clear) st[ST_NF_IN] = st[ST_NF_OUT] = 0;
        int nt[3] = {0, 0, 0};
        for (int q = 0; q < NP; ++q) nt[s_tier[q]]++;
        st[0] = s_rowptr[NP];
        st[1] = p.Emax;
        st[2] = nt[0]; st[3] = nt[1]; st[4] = nt[2];
        st[5] = kk[0]; st[6] = kk[1]; st[7] = kk[2];
        st[8] = s_refbase[NP];
      }
    }
  }
  __syncthreads();
  const int k = kk[s_tier[pp]];
  const int row = s_rowof[pp], base = s_rowptr[row], rbase = s_refbase[row];
  // kept words (wave w: words w, w + 16, ...)
  for (int i = wv; i < NW; i += 16) {
    const unsigned long long bal = kept_word(s_keep, i, lane, C, k);
    if (lane == 0) s_kept[i] = bal;
  }
  __syncthreads();
  if (wv == 0) {
    // per word: kept events before it, the first kept chunk after it and the
    // last kept chunk before it (lane l: words 2 l and 2 l + 1)
    int cnt2[2], first2[2], last2[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int i = 2 * lane + h;
      const unsigned long long bal = i < NW ? s_kept[i] : 0ull;
      cnt2[h] = __popcll(bal);
      first2[h] = bal ? 64 * i + (int)__builtin_ctzll(bal) : C + 1;
      last2[h] = bal ? 64 * i + 63 - (int)__builtin_clzll(bal) : -1;
    }
    // inclusive scans over lanes of the lane totals
    int incl = cnt2[0] + cnt2[1];
    int lastin = max(last2[0], last2[1]);
    int firstin = min(first2[0], first2[1]);
    int firstsuf = firstin;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int a = __shfl_up(incl, d, 64), m = __shfl_up(lastin, d, 64);
      const int f = __shfl_down(firstsuf, d, 64);
      if (lane >= d) { incl += a; lastin = max(lastin, m); }
      if (lane + d < 64) firstsuf = min(firstsuf, f);
    }
    const int excl = incl - cnt2[0] - cnt2[1];
    int lastex = __shfl_up(lastin, 1, 64);
    if (lane == 0) lastex = -1;
    int firstafter = __shfl_down(firstsuf, 1, 64);
    if (lane == 63) firstafter = C + 1;
    if (2 * lane < NW) {
      s_run[2 * lane] = excl;
      s_last[2 * lane] = lastex;
      s_next[2 * lane] = min(first2[1], firstafter);
    }
    if (2 * lane + 1 < NW) {
      s_run[2 * lane + 1] = excl + cnt2[0];
      s_last[2 * lane + 1] = max(lastex, last2[0]);
      s_next[2 * lane + 1] = firstafter;
    }
  }
  __syncthreads();
  for (int i = wv; i < NW; i += 16) {
    const unsigned long long rb = ref_word(s_kept[i], i, lane, s_next[i], G);
    if (lane == 0) s_refd[i] = rb;
  }
  __syncthreads();
  if (wv == 0) {
    int c2[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) c2[h] = 2 * lane + h < NW ? __popcll(s_refd[2 * lane + h]) : 0;
    int incl = c2[0] + c2[1];
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int a = __shfl_up(incl, d, 64);
      if (lane >= d) incl += a;
    }
    const int excl = incl - c2[0] - c2[1];
    if (2 * lane < NW) s_rrun[2 * lane] = excl;
    if (2 * lane + 1 < NW) s_rrun[2 * lane + 1] = excl + c2[0];
  }
  __syncthreads();
  // outputs of pair pp: words w, w + 16, ... (and the mask bytes and groups
  // of every word of the stride C, past the sequence's end too)
  const unsigned long long below = (1ull << lane) - 1ull;
  uint8_t* mask = p.mask + ((size_t)b * NP + pp) * CS;
  int32_t* col = p.col + (size_t)b * p.Emax;
  int32_t* eslot = p.event_slot + (size_t)b * p.Emax;
  for (int i = wv; i < NWS; i += 16) {
    const int c = 64 * i + lane;
    const unsigned long long bal = i < NW ? s_kept[i] : 0ull;
    const unsigned long long rb = i < NW ? s_refd[i] : 0ull;
    const bool kept = (bal >> lane) & 1ull;
    if (c < CS) mask[c] = kept ? 1 : 0;
    if (kept) {
      const int e = base + s_run[i] + __popcll(bal & below);
      const int slot = ((rb >> lane) & 1ull) ? rbase + s_rrun[i] + __popcll(rb & below) : -1;
      col[e] = c;
      eslot[e] = slot;
      if (p.rec != nullptr) {
        // the event records of the H scan (Sec. 2.1 Eq. (2), Sec. 2.6
        // Eq. (21)), as the record kernel forms them: F_in = 2^(P_c -
        // P_{e'+1}) from the previous kept chunk e' of the row (1 for the
        // first), 2^gamma F_in, the snapshot slot and the chunk
        const unsigned long long m = bal & below;
        const int prev = m ? 64 * i + 63 - (int)__builtin_clzll(m) : s_last[i];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const size_t bh = (size_t)b * NV + 2 * pp + hh;
          const double* P = p.P + bh * (CS + 1);
          const float fin = prev >= 0 ? exp2f((float)(P[c] - P[prev + 1])) : 1.f;
          int4 r;
          r.x = __float_as_int(fin);
          r.y = __float_as_int(exp2f(p.gamma[bh * CS + c]) * fin);
          r.z = slot;
          r.w = c;
          reinterpret_cast<int4*>(p.rec)[((size_t)b * p.Emax + e) * 2 + hh] = r;
        }
      }
    }
    if ((c & 1) == 0 && c < CS) {
      // group c / 2: the last kept chunk before c and its snapshot slot
      int pc = -1, ps = -1;
      if (c < C) {
        const unsigned long long m = bal & below;
        pc = m ? 64 * i + 63 - (int)__builtin_clzll(m) : s_last[i];
        if (pc >= 0) {
          const int j = pc >> 6, el = pc & 63;
          ps = rbase + s_rrun[j] + __popcll(s_refd[j] & ((1ull << el) - 1ull));
        }
      }
      const size_t o = ((size_t)b * NP + pp) * GS + (c >> 1);
      p.pred[o] = pc;
      p.group_slot[o] = ps;
    }
  }
}

// Eq. (16) for a caller's mask (mask_in): event mask, CSR rows (every pair a
// Low row, in pair order), kept chunks ascending, predecessor of every output
// group and compact-snapshot slots numbered over the referenced events in CSR
// order.  One block of 16 waves per sequence; wave w works on pair w or row w.
__global__ __launch_bounds__(1024) void mask_layout_kernel(SelectArgs p) {
  // Wave w handles head pair w.  Each pair's kept chunks are held as 64-bit
  // words (bit l of word i: chunk 64 i + l), and so are its referenced events,
  // so the CSR columns, the snapshot slots and the group predecessors follow
  // from bit counts without reading back what this kernel writes.
  constexpr int NWMAX = 128;   // 64-chunk words per pair (C <= 8192)
  __shared__ int s_cnt[NP], s_rowpair[NP], s_rowof[NP], s_rowptr[NP + 1];
  __shared__ int s_ref[NP], s_refbase[NP + 1];
  __shared__ unsigned long long s_kept[NP][NWMAX], s_refd[NP][NWMAX];
  const int b = blockIdx.x, tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  // CS, GS: strides of the per-chunk and per-group arrays; C, G: this
  // sequence's valid chunks and groups.  Chunks past C are not kept (their
  // mask bytes are written as 0) and groups past G have no predecessor.
  const int CS = p.C, GS = p.G, NW = (CS + 63) / 64;
  const int C = valid_chunks(p, b), G = (C + 1) / 2;
  int kk[3];
  tier_counts(C, p.keep_bp, p.rate_bp, kk);
  const unsigned long long below = (1ull << lane) - 1ull;
  uint8_t* mask = p.mask + (size_t)b * NP * CS;
  const int pp = w;
  {
    // mask of pair w (the loads of a batch of words are issued together)
    int cnt = 0;
    for (int i0 = 0; i0 < NW; i0 += 16) {
      int val[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int c = 64 * (i0 + u) + lane;
        const size_t idx = (size_t)b * NP * CS + (size_t)pp * CS + c;
        val[u] = 0;
        if (i0 + u < NW && c < C) val[u] = p.mask_in[idx];
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int i = i0 + u;
        if (i < NW) {
          const int c = 64 * i + lane;
          const int z = (c < C && val[u]) ? 1 : 0;
          if (c < CS) mask[(size_t)pp * CS + c] = (uint8_t)z;
          const unsigned long long bal = __ballot(z);
          if (lane == 0) s_kept[pp][i] = bal;
          cnt += z;
        }
      }
    }
    for (int off = 32; off >= 1; off >>= 1) cnt += __shfl_xor(cnt, off, 64);
    if (lane == 0) s_cnt[pp] = cnt;
  }
  __syncthreads();
  if (tid == 0) {
    // CSR rows in head-pair order
    s_rowptr[0] = 0;
    for (int q = 0; q < NP; ++q) {
      s_rowpair[q] = q;
      s_rowof[q] = q;
      s_rowptr[q + 1] = s_rowptr[q] + s_cnt[q];
    }
  }
  __syncthreads();
  if (tid < NP) p.row_pair[b * NP + tid] = s_rowpair[tid];
  if (tid <= NP) p.row_ptr[b * (NP + 1) + tid] = s_rowptr[tid];
  int32_t* col = p.col + (size_t)b * p.Emax;
  const int row = s_rowof[pp], base = s_rowptr[row];
  {
    // kept chunks of pair w, ascending, at its row's offset
    int run = 0;
    for (int i = 0; i < NW; ++i) {
      const unsigned long long bal = s_kept[pp][i];
      if ((bal >> lane) & 1ull) col[base + run + __popcll(bal & below)] = 64 * i + lane;
      run += __popcll(bal);
    }
  }
  {
    // referenced events: e is the predecessor of some group r (2r <= 2(G-1))
    // iff there is an even number in [e+1, min(next kept, 2(G-1))]; the
    // next kept chunk is found from the words, walking backwards
    int nextfirst = C + 1, refcnt = 0;
    for (int i = NW - 1; i >= 0; --i) {
      const unsigned long long bal = s_kept[pp][i];
      const int c = 64 * i + lane;
      const unsigned long long above = lane == 63 ? 0ull : (bal >> (lane + 1));
      const int nxt = above ? c + 1 + (int)__builtin_ctzll(above) : nextfirst;
      const int lo = c + 1, lo_e = lo + (lo & 1), hi = min(nxt, 2 * (G - 1));
      const bool ref = ((bal >> lane) & 1ull) && lo_e <= hi;
      const unsigned long long rb = __ballot(ref);
      if (lane == 0) s_refd[pp][i] = rb;
      refcnt += __popcll(rb);
      if (bal) nextfirst = 64 * i + (int)__builtin_ctzll(bal);
    }
    if (lane == 0) s_ref[row] = refcnt;
  }
  __syncthreads();
  if (tid == 0) {
    s_refbase[0] = 0;
    for (int r = 0; r < NP; ++r) s_refbase[r + 1] = s_refbase[r] + s_ref[r];
  }
  __syncthreads();
  int32_t* eslot = p.event_slot + (size_t)b * p.Emax;
  {
    // snapshot slot of each event (rank among the referenced ones, rows in
    // CSR order) and, per group r, the last kept chunk before 2r with its slot
    const int rbase = s_refbase[row];
    int run = 0, rrun = 0, lastc = -1, lasts = -1;
    for (int i = 0; i < NW; ++i) {
      const unsigned long long bal = s_kept[pp][i], rb = s_refd[pp][i];
      const int c = 64 * i + lane;
      if ((bal >> lane) & 1ull)
        eslot[base + run + __popcll(bal & below)] = ((rb >> lane) & 1ull) ? rbase + rrun + __popcll(rb & below) : -1;
      if ((c & 1) == 0 && c < CS) {
        const unsigned long long m = bal & below;
        int pc = lastc, ps = lasts;
        if (m) {
          const int el = 63 - (int)__builtin_clzll(m);
          pc = 64 * i + el;
          ps = rbase + rrun + __popcll(rb & ((1ull << el) - 1ull));
        }
        if (c >= C) pc = -1;   // group past the sequence's end
        const size_t o = ((size_t)b * NP + pp) * GS + (c >> 1);
        p.pred[o] = pc;
        p.group_slot[o] = pc >= 0 ? ps : -1;
      }
      if (bal) {
        const int el = 63 - (int)__builtin_clzll(bal);
        lastc = 64 * i + el;
        lasts = rbase + rrun + __popcll(rb & ((1ull << el) - 1ull));
      }
      run += __popcll(bal);
      rrun += __popcll(rb);
    }
  }
  if (tid == 0 && p.stats != nullptr) {
    int32_t* st = static_cast<int32_t*>(p.stats) + (size_t)b * STATS_INTS;
    if (p.nf_clear) st[ST_NF_IN] = st[ST_NF_OUT] = 0;
    st[0] = s_rowptr[NP];
    st[1] = p.Emax;
    st[2] = NP; st[3] = 0; st[4] = 0;   // every pair a Low row
    st[5] = kk[0]; st[6] = kk[1]; st[7] = kk[2];
    st[8] = s_refbase[NP];
  }
}

// Diagnostic: this file's binary64 division and square root (the forms the
// selector's decisions are computed with), element by element.
__global__ __launch_bounds__(256) void fp64_selftest_kernel(const double* x, const double* y, double* q,
                                                            double* r, long long n) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256) {
    const double a = x[i];
    q[i] = a / y[i];
    r[i] = sqrt(a);
  }
}

}  // namespace

hipError_t launch_fp64_selftest(const double* x, const double* y, double* q, double* r, long long n,
                                hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const long long blocks = (n + 255) / 256;
  hipLaunchKernelGGL(fp64_selftest_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0,
                     s, x, y, q, r, n);
  return hipGetLastError();
}

hipError_t launch_select_full(const SelectArgs& a, hipStream_t s) {
  if (a.mask_in != nullptr) {
    hipLaunchKernelGGL(mask_layout_kernel, dim3(a.B), dim3(1024), 0, s, a);
    return hipGetLastError();
  }
  const int nblk = (a.C + RANK_CHUNKS - 1) / RANK_CHUNKS;
  const size_t rank_lds = (size_t)a.C * (sizeof(double) + 2 * sizeof(float));
  hipLaunchKernelGGL(select_rank_kernel<false>, dim3(nblk, NP, a.B), dim3(1024), rank_lds, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.rank_key != nullptr) {
    hipLaunchKernelGGL(select_rank_kernel<true>, dim3(nblk, NP, a.B), dim3(1024), rank_lds, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(select_pair_kernel, dim3(NP, a.B), dim3(1024), (size_t)a.C * 16, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(select_decide_kernel, dim3(NP, a.B), dim3(1024), (size_t)a.C * 4, s, a);
  return hipGetLastError();
}

}  // namespace sgdn
