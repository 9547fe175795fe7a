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
//  * r^n for integer n: binary powering from the least significant bit.
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

__device__ double powi_fixed(double r, int n) {
  double res = 1.0, base = r;
  while (n) {
    if (n & 1) res = res * base;
    base = base * base;
    n >>= 1;
  }
  return res;
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
// workgroup forms the norms and keys itself, with the same operations.
constexpr int RANK_CHUNKS = 128;
__global__ __launch_bounds__(1024) void select_rank_kernel(SelectArgs p) {
  extern __shared__ double sq[];
  __shared__ double snorm[2];
  const int blk = blockIdx.x, pp = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int C = p.C;
  const float* s0 = p.score + ((size_t)b * NV + 2 * pp) * C;
  const float* s1 = s0 + C;
  if (w < 2) {
    const float* s = w ? s1 : s0;
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
    const double t0 = n0 > 0.0 ? (double)s0[c] / n0 : 0.0;
    const double t1 = n1 > 0.0 ? (double)s1[c] / n1 : 0.0;
    sq[c] = 0.5 * (t0 + t1);
  }
  __syncthreads();
  int32_t* rk = p.rank + ((size_t)b * NP + pp) * C;
  const int c = RANK_CHUNKS * blk + (tid >> 3), part = tid & 7;
  int r = 0;
  const bool inner = c >= 1 && c <= C - 2;
  if (inner) {
    const double qc = sq[c];
    for (int c2 = 1 + part; c2 <= C - 2; c2 += 8) {
      const double q2 = sq[c2];
      r += (q2 > qc || (q2 == qc && c2 < c)) ? 1 : 0;
    }
  }
  // the eight partial counts of a chunk sit in eight adjacent lanes
  r += __shfl_xor(r, 1, 64);
  r += __shfl_xor(r, 2, 64);
  r += __shfl_xor(r, 4, 64);
  if (part == 0 && c < C) rk[c] = inner ? r : -1;
}

// B(x, k) = k (n-k) / n (mean x[:k] - mean x[k:])^2 over the wave-held sorted
// values vals[0..n) (Eq. (14)).
__device__ double split_score(const double* vals, int n, int k, int lane) {
  if (k <= 0 || k >= n) return 0.0;
  const double a = wave_sum(lane < k ? vals[lane] : 0.0);
  const double c = wave_sum(lane < n - k ? vals[k + lane] : 0.0);
  const double m1 = a / k;
  const double m2 = c / (n - k);
  const double f = (double)(k * (n - k)) / n;
  const double dm = m1 - m2;
  return f * (dm * dm);
}

// Eqs. (11)-(14): lifetime, visibility, upgrade gains, dynamic tier counts.
// Wave w forms the per-head sums of the two heads of pair w (each sum is one
// wave's lane-interleaved sum, as everywhere in this file); wave 0 then takes
// the decisions.
__global__ __launch_bounds__(1024) void select_tier_kernel(SelectArgs p, int kL, int kM, int kH) {
  __shared__ double sL[NV], sGv[NV], slm[NV], smh[NV];
  __shared__ double sxm[NP], sxh[NP], svals[NP];
  __shared__ int sorder[NP], shigh[NP];
  const int b = blockIdx.x, tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, C = p.C;
  const float* sc = p.score + (size_t)b * NV * C;
  const float* gm = p.gamma + (size_t)b * NV * C;
  const float* et = p.eta + (size_t)b * NV;
  const int32_t* rk = p.rank + (size_t)b * NP * C;

  const int lo = C > 16 ? C - 16 : 0, nwin = C - lo;
  for (int h = 2 * wv; h < 2 * wv + 2; ++h) {
    const double x = lane < nwin ? exp2_fixed((double)gm[h * C + lo + lane]) : 0.0;
    const double tot = wave_sum(x);
    if (lane == 0) sL[h] = lifetime(tot / nwin, C);
    const int pp = h >> 1;
    double alm = 0.0, amh = 0.0;
    for (int c = lane; c < C; c += 64) {
      const int r = rk[pp * C + c];
      const double xs = (double)sc[h * C + c];
      alm = alm + ((r >= kL - 2 && r < kM - 2) ? xs : 0.0);
      amh = amh + ((r >= kM - 2 && r < kH - 2) ? xs : 0.0);
    }
    const double tl = wave_sum(alm), th = wave_sum(amh);
    if (lane == 0) { slm[h] = tl; smh[h] = th; }
  }
  __syncthreads();
  if (wv != 0) return;
  const double etab = wave_sum(lane < NV ? (double)et[lane] : 0.0) / NV;
  if (lane < NV) sGv[lane] = etab > 0.0 ? sqrt((double)et[lane] / etab) : 1.0;
  __syncthreads();
  double glm = 0.0, gmh = 0.0;
  if (lane < NP) {
    const int h0 = 2 * lane, h1 = h0 + 1;
    glm = (sL[h0] * sGv[h0]) * slm[h0] + (sL[h1] * sGv[h1]) * slm[h1];
    gmh = (sL[h0] * sGv[h0]) * smh[h0] + (sL[h1] * sGv[h1]) * smh[h1];
  }
  const double mum = wave_sum(glm) / NP;
  const double muh = wave_sum(gmh) / NP;
  if (lane < NP) {
    sxm[lane] = mum > 0.0 ? glm / mum : 0.0;
    sxh[lane] = muh > 0.0 ? gmh / muh : 0.0;
  }
  __syncthreads();

  // High count: pairs sorted by x_H descending (ties: lower pair first)
  if (lane < NP) {
    int pos = 0;
    for (int q = 0; q < NP; ++q)
      pos += (sxh[q] > sxh[lane] || (sxh[q] == sxh[lane] && q < lane)) ? 1 : 0;
    sorder[pos] = lane;
  }
  __syncthreads();
  if (lane < NP) svals[lane] = sxh[sorder[lane]];
  __syncthreads();
  int nH = 1;
  {
    double best = 0.0;
    for (int k = 1; k <= 4; ++k) {
      const double v = split_score(svals, NP, k, lane);
      if (k == 1 || v > best) { best = v; nH = k; }
    }
  }
  if (lane < NP) shigh[lane] = 0;
  __syncthreads();
  if (lane < nH) shigh[sorder[lane]] = 1;
  __syncthreads();

  // Medium count among the remaining pairs, sorted by x_M descending
  const int nrest = NP - nH;
  if (lane < NP && !shigh[lane]) {
    int pos = 0;
    for (int q = 0; q < NP; ++q)
      if (!shigh[q]) pos += (sxm[q] > sxm[lane] || (sxm[q] == sxm[lane] && q < lane)) ? 1 : 0;
    sorder[pos] = lane;
  }
  __syncthreads();
  if (lane < nrest) svals[lane] = sxm[sorder[lane]];
  __syncthreads();
  int cand[3], ncand;
  if (nH == 1) { cand[0] = 11; cand[1] = 12; cand[2] = 13; ncand = 3; }
  else if (nH == 2) { cand[0] = 7; cand[1] = 8; cand[2] = 9; ncand = 3; }
  else if (nH == 3) { cand[0] = 3; cand[1] = 4; cand[2] = 5; ncand = 3; }
  else { cand[0] = 0; ncand = 1; }
  int nM = cand[0];
  {
    double best = 0.0;
    for (int i = 0; i < ncand; ++i) {
      const double v = split_score(svals, nrest, cand[i], lane);
      if (i == 0 || v > best) { best = v; nM = cand[i]; }
    }
  }
  if (lane < NP) {
    int t = 0;
    if (shigh[lane]) t = 2;
    else {
      // position among the remaining pairs
      int pos = 0;
      for (int q = 0; q < nrest; ++q) pos += (sorder[q] == lane) ? q : 0;
      t = pos < nM ? 1 : 0;
    }
    p.tier[b * NP + lane] = (uint8_t)t;
  }
  if (lane == 0) {
    int32_t* ti = p.tierinfo + b * 8;
    ti[0] = kL; ti[1] = kM; ti[2] = kH; ti[3] = nH; ti[4] = nM;
  }
}

// Eq. (16): event mask, CSR rows (High, Medium, Low; ascending pair within a
// tier), kept chunks ascending, predecessor of every output group and
// compact-snapshot slots numbered over the referenced events in CSR order.
// One block of 16 waves per sequence; wave w works on pair w or row w.
__global__ __launch_bounds__(1024) void layout_kernel(SelectArgs p, int kL, int kM, int kH) {
  __shared__ int s_tier[NP], s_cnt[NP], s_rowpair[NP], s_rowof[NP], s_rowptr[NP + 1];
  __shared__ int s_ref[NP], s_refbase[NP + 1];
  const int b = blockIdx.x, tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int C = p.C, G = p.G;
  uint8_t* mask = p.mask + (size_t)b * NP * C;
  const bool ovr = p.mask_in != nullptr;
  if (tid < NP) s_tier[tid] = ovr ? 0 : p.tier[b * NP + tid];
  __syncthreads();
  {
    const int pp = w;
    const int t = s_tier[pp];
    const int k = t == 2 ? kH : (t == 1 ? kM : kL);
    int cnt = 0;
    for (int c = lane; c < C; c += 64) {
      const size_t idx = (size_t)pp * C + c;
      uint8_t z;
      if (ovr) {
        z = p.mask_in[(size_t)b * NP * C + idx] ? 1 : 0;
      } else {
        const int r = p.rank[(size_t)b * NP * C + idx];
        z = (c == 0 || c == C - 1 || (r >= 0 && r < k - 2)) ? 1 : 0;
      }
      mask[idx] = z;
      cnt += z;
    }
    for (int off = 32; off >= 1; off >>= 1) cnt += __shfl_xor(cnt, off, 64);
    if (lane == 0) s_cnt[pp] = cnt;
  }
  __syncthreads();
  if (tid == 0) {
    int r = 0;
    s_rowptr[0] = 0;
    for (int t = 2; t >= 0; --t)
      for (int pp = 0; pp < NP; ++pp)
        if (s_tier[pp] == t) {
          s_rowpair[r] = pp;
          s_rowof[pp] = r;
          s_rowptr[r + 1] = s_rowptr[r] + s_cnt[pp];
          ++r;
        }
  }
  __syncthreads();
  if (tid < NP) p.row_pair[b * NP + tid] = s_rowpair[tid];
  if (tid <= NP) p.row_ptr[b * (NP + 1) + tid] = s_rowptr[tid];
  int32_t* col = p.col + (size_t)b * p.Emax;
  {
    // kept chunks of pair w, ascending, at its row's offset
    const int pp = w, base = s_rowptr[s_rowof[pp]];
    int run = 0;
    for (int c0 = 0; c0 < C; c0 += 64) {
      const int c = c0 + lane;
      const bool z = c < C && mask[(size_t)pp * C + c];
      const unsigned long long bal = __ballot(z);
      const int before = __popcll(bal & ((1ull << lane) - 1ull));
      if (z) col[base + run + before] = c;
      run += __popcll(bal);
    }
  }
  __syncthreads();
  // referenced events: e is the predecessor of some group r (2r <= 2(G-1))
  // iff there is an even number in [e+1, min(next kept, 2(G-1))]
  auto referenced = [&](int i, int end) {
    const int c = col[i];
    const int nxt = (i + 1 < end) ? col[i + 1] : C + 1;
    const int lo = c + 1, lo_e = lo + (lo & 1);
    const int hi = min(nxt, 2 * (G - 1));
    return lo_e <= hi;
  };
  {
    const int beg = s_rowptr[w], end = s_rowptr[w + 1];
    int cnt = 0;
    for (int i = beg + lane; i < end; i += 64) cnt += referenced(i, end) ? 1 : 0;
    for (int off = 32; off >= 1; off >>= 1) cnt += __shfl_xor(cnt, off, 64);
    if (lane == 0) s_ref[w] = cnt;
  }
  __syncthreads();
  if (tid == 0) {
    s_refbase[0] = 0;
    for (int r = 0; r < NP; ++r) s_refbase[r + 1] = s_refbase[r] + s_ref[r];
  }
  __syncthreads();
  int32_t* eslot = p.event_slot + (size_t)b * p.Emax;
  {
    const int beg = s_rowptr[w], end = s_rowptr[w + 1];
    int run = s_refbase[w];
    for (int i0 = beg; i0 < end; i0 += 64) {
      const int i = i0 + lane;
      const bool ref = i < end && referenced(i, end);
      const unsigned long long bal = __ballot(ref);
      const int before = __popcll(bal & ((1ull << lane) - 1ull));
      if (i < end) eslot[i] = ref ? run + before : -1;
      run += __popcll(bal);
    }
  }
  __syncthreads();
  {
    // predecessor of each group r of pair w: the last kept chunk < 2r, i.e.
    // CSR entry beg + (number of kept chunks before 2r) - 1
    const int pp = w, row = s_rowof[pp];
    const int beg = s_rowptr[row];
    int run = 0;   // kept chunks before c0
    for (int c0 = 0; c0 < C; c0 += 64) {
      const int c = c0 + lane;
      const bool z = c < C && mask[(size_t)pp * C + c];
      const unsigned long long bal = __ballot(z);
      const int before = run + __popcll(bal & ((1ull << lane) - 1ull));
      if ((c & 1) == 0 && c < C && (c >> 1) < G) {
        const int r = c >> 1, i = beg + before - 1;
        const size_t o = ((size_t)b * NP + pp) * G + r;
        p.pred[o] = before > 0 ? col[i] : -1;
        p.group_slot[o] = before > 0 ? eslot[i] : -1;
      }
      run += __popcll(bal);
    }
  }
  if (tid == 0 && p.stats != nullptr) {
    int32_t* st = static_cast<int32_t*>(p.stats) + b * 9;
    int nt[3] = {0, 0, 0};
    for (int pp = 0; pp < NP; ++pp) nt[s_tier[pp]]++;
    st[0] = s_rowptr[NP];
    st[1] = p.Emax;
    st[2] = nt[0]; st[3] = nt[1]; st[4] = nt[2];
    st[5] = kL; st[6] = kM; st[7] = kH;
    st[8] = s_refbase[NP];
  }
}

}  // namespace

hipError_t launch_select_full(const SelectArgs& a, int kL, int kM, int kH, hipStream_t s) {
  if (a.mask_in == nullptr) {
    const int nblk = (a.C + RANK_CHUNKS - 1) / RANK_CHUNKS;
    hipLaunchKernelGGL(select_rank_kernel, dim3(nblk, NP, a.B), dim3(1024), (size_t)a.C * sizeof(double), s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(select_tier_kernel, dim3(a.B), dim3(1024), 0, s, a, kL, kM, kH);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(layout_kernel, dim3(a.B), dim3(1024), 0, s, a, kL, kM, kH);
  return hipGetLastError();
}

}  // namespace sgdn
