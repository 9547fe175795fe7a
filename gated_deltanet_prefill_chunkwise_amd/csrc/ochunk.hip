// O kernel: outputs of one two-chunk group (2r, 2r+1) of one value head.
//
// SparseGDN reading notes, Sec. 2.7, Eqs. (22)-(24):
//   O_c   = d^-1/2 [2^g_c * (Q_c S) + A_cc U'_c]
//   O_c+1 = d^-1/2 [2^(g_c+1 + gamma_c) * (Q_c+1 S) + A_c+1,c U'_c + A_c+1,c+1 U'_c+1]
// with the group entry state S = S_2r restored from the compact snapshot of
// the last kept event e before 2r by the factor 2^(P_2r - P_e+1) (Eq. (21)),
// or from the initial state, or zero.  With every event kept this equals the
// per-chunk form of Eqs. (3)-(4) (Eq. (25)).
//
// Writing G[t] for the log decay accumulated from the group start to token t
// (g_c in the first chunk, gamma_c + g_c+1 in the second), all three local
// blocks are A^T[s][t] = <q_t, k_s> 2^(G[t] - G[s]) for s <= t over the
// group's 128 tokens, and the inter-chunk factor is 2^G[t].
//
// Computed transposed, O^T = S^T Q^T + U'^T A^T:
//   phase 1: wave i computes the A^T blocks of source tile i (K rows from
//            global, Q rows from LDS), applies the decay and stores them in
//            LDS (B operand layout [t][s]);
//   phase 2: wave w owns dv rows 16w..16w+15 of O^T for all 128 tokens, so
//            each row of the state and of U' is read exactly once.
// All products run in the intermediate type I of the state snapshots and U'
// (fp16 for bf16 inputs: q and k are unit-norm rows, so their conversion is
// exact; fp32 for fp32 inputs).
#include "common.h"
#include "kernels.h"

namespace sgdn {

namespace {

constexpr int QSTR = DK + 8;      // Q rows [t][dk]
constexpr int ASTR = 2 * L + 8;   // A^T rows [t][s], s over the group's 128 tokens
constexpr int OSTR = DV + 4;      // O staging rows [t][dv] (fp32)

// Two workgroups per CU (four waves per SIMD: at most 128 registers per lane)
// so one group's loads
// overlap the other's products.
//
// ONE (the mapped-O ablation): one chunk per workgroup.  Block 2r + half
// computes the 64 output rows of chunk 2r + half of group r: half 0 with
// the sources of the first chunk, half 1 with all 128 sources (the cross
// term A_{c+1,c} U'_c included); both restore the group entry state, so the
// outputs are those of the two-chunk form.
template <typename E, typename OT, bool ONE>
__global__ __launch_bounds__(512, 4) void ochunk_kernel(OChunkArgs p) {
  constexpr int NT = ONE ? 4 : 8;   // 16-token tiles computed
  using I = inter_t<E>;
  // Q and A^T during the products; afterwards the same bytes hold the
  // group's O rows, so that each store writes whole rows (a wave's own O^T
  // tile covers only 16 of a row's 128 values)
  constexpr int QA_MIN = (int)sizeof(I) * NT * 16 * (QSTR + ASTR), O_MIN = NT * 16 * OSTR * 4;
  constexpr int QA_BYTES = QA_MIN > O_MIN ? QA_MIN : O_MIN;
  __shared__ __align__(32) char sQA[QA_BYTES];
  I* sQ = reinterpret_cast<I*>(sQA);
  I* sA = sQ + NT * 16 * QSTR;
  float* sO = reinterpret_cast<float*>(sQA);
  __shared__ float sG[2 * L];

  const int T = p.T, Nq = p.Nq, Nv = p.Nv, C = p.C, G = p.G;
  // Block -> (group r, row, batch b; head hh of the pair).  The two heads of
  // a pair read the same Q and K rows: they are dispatched one after the
  // other onto the same XCD (workgroups are dealt to the 8 XCDs
  // round-robin), so the second read hits that XCD's L2.  A launch covers
  // rows row_lo .. row_lo + nrows - 1: head pairs (dense) or CSR rows, whose
  // pair is row_pair (sparse).
  const int id = blockIdx.x, NP = Nv / 2;
  int unit, hh;
  if ((gridDim.x & 15) == 0) {
    const int local = id >> 3;
    hh = local & 1;
    unit = (local >> 1) * 8 + (id & 7);
  } else {
    hh = id & 1;
    unit = id >> 1;
  }
  const int nr = p.nrows, NU = ONE ? 2 * G : G;   // blocks per row of a sequence
  const int row = p.row_lo + unit % nr, rb = (unit / nr) % NU, b = unit / (nr * NU);
  const int r = ONE ? rb >> 1 : rb, half = ONE ? rb & 1 : 0;
  const int pr = p.sparse ? ((const cint32*)p.row_pair)[__builtin_amdgcn_readfirstlane(b * NP + row)] : row;
  const int h = 2 * pr + hh;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int n16 = lane & 15, g4 = lane >> 4;
  const int c0 = 2 * r, j0 = 4 * half;   // j0: first token tile computed
  // a group (chunk, with ONE) past the end of its (shorter, packed) sequence
  // has no outputs; the whole workgroup leaves before any load or barrier
  const SeqSpan sp = seq_span(p.cu, b, T);
  if ((c0 + half) * L >= sp.len) return;
  const bool has1 = c0 + 1 < chunks_of(sp.len);
  // the sources include the second chunk (not for the first half with ONE)
  const bool need1 = has1 && (!ONE || half == 1);
  // Every group is computed as two chunks (straight-line code); a group
  // without a second chunk reads zeros for its Q, K, U' and decays there,
  // so those products vanish, and its rows are not stored.
  const size_t bh = (size_t)b * Nv + h;

  // ---- group entry state: source and log2 factor
  const I* Ssrc = nullptr;
  float lf = 0.f;
  if (p.entry != nullptr) {
    Ssrc = static_cast<const I*>(p.entry) + (bh * G + r) * DV * DK;
  } else if (p.sparse) {
    const size_t pg = ((size_t)b * (Nv / 2) + pr) * G + r;
    const int slot = p.group_slot[pg];
    const double* P = p.P + bh * (C + 1);
    if (slot >= 0) {
      const int e = p.pred[pg];
      Ssrc = static_cast<const I*>(p.snap) + (((size_t)b * p.snap_cap + slot) * 2 + hh) * DV * DK;
      lf = (float)(P[c0] - P[e + 1]);
    } else if (p.s0T != nullptr) {
      Ssrc = static_cast<const I*>(p.s0T) + bh * DV * DK;
      lf = (float)P[c0];
    }
  } else {
    if (r > 0)
      Ssrc = static_cast<const I*>(p.snap) + (bh * (G - 1) + r - 1) * DV * DK;
    else if (p.s0T != nullptr)
      Ssrc = static_cast<const I*>(p.s0T) + bh * DV * DK;
  }

  // ---- global loads of both phases are issued up front so that their
  //      latencies overlap; the Q rows to stage go first, because loads
  //      retire in order
  const E* Qin = static_cast<const E*>(p.q);
  const E* Kin = static_cast<const E*>(p.k);
  frag_t<E> qst[NT / 2];
#pragma unroll
  for (int it = 0; it < NT / 2; ++it) {
    const int q = tid + 512 * it;
    const int rr = q >> 4, c8 = (q & 15) * 8;
    const int t = c0 * L + 16 * j0 + rr;
    qst[it] = (t < sp.len) ? ld8(Qin + ((size_t)(sp.tok0 + t) * Nq + pr) * DK + c8) : zero_frag<E>();
  }
  frag_t<E> kf[4];
  {
    const int ts = c0 * L + 16 * w + n16;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      kf[ks] = (ts < sp.len && (!ONE || w < 4 || need1)) ? ld8(Kin + ((size_t)(sp.tok0 + ts) * Nq + pr) * DK + 32 * ks + 8 * g4)
                        : zero_frag<E>();
  }
  const int dvr = 16 * w + n16;
  const I* Up = static_cast<const I*>(p.U);
  frag_t<I> sfr[4], ufr[4];
  // a dense group snapshot is read by one group only; a sparse compact
  // snapshot serves every group up to the next kept event, so it stays cached
  const bool dense_snap = !p.sparse && p.entry == nullptr && r > 0;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    sfr[ks] = Ssrc == nullptr ? zero_frag<I>()
              : dense_snap ? ld8nt(Ssrc + s_elem(dvr, 32 * ks + 8 * g4)) : ld8(Ssrc + s_elem(dvr, 32 * ks + 8 * g4));

  // ---- stage Q rows of the group and G (a non-finite q is flagged)
  uint32_t nfq = 0;
#pragma unroll
  for (int it = 0; it < NT / 2; ++it) {
    const int q = tid + 512 * it;
    const int rr = q >> 4, c8 = (q & 15) * 8;
    nfq |= nonfinite8(qst[it]);
    *reinterpret_cast<frag_t<I>*>(&sQ[rr * QSTR + c8]) = cvt8<I, E>(qst[it]);
  }
  flag_or(p.stats, b, ST_NF_IN, nfq ? NF_Q : 0);
  if (tid < 128) {
    const int cc = tid >> 6;
    float gv = 0.f;
    if (cc == 0) {
      gv = p.g[(bh * C + c0) * L + lane];
    } else if (need1) {
      gv = p.gamma[bh * C + c0] + p.g[(bh * C + c0 + 1) * L + lane];
    }
    sG[tid] = gv;
  }
  __syncthreads();

  // ---- phase 1: A^T blocks of source tile w (s in 16w..16w+15)
  if (!ONE || half == 1 || w < 4) {
    frag_t<I> kfi[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) kfi[ks] = cvt8<I, E>(kf[ks]);
    float gs[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) gs[j] = sG[16 * w + 4 * g4 + j];
    // the block just above the diagonal (source tile w, token tile w - 1) is
    // read by the 32-wide k-steps of phase 2; the causal mask makes it zero
    for (int jt = max(w - 1, j0); jt < j0 + NT; ++jt) {
      f32x4 at = zero4();
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        at = mma(kfi[ks], ld8(&sQ[(16 * (jt - j0) + n16) * QSTR + 32 * ks + 8 * g4]), at);
      const int t = 16 * jt + n16;
      const float gt = sG[t];
      f32x4 a4;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int s = 16 * w + 4 * g4 + j;
        const float v = (s <= t) ? at[j] * exp2f(gt - gs[j]) : 0.f;
        a4[j] = v;
      }
      st4<I>(&sA[(t - 16 * j0) * ASTR + 16 * w + 4 * g4], a4);
    }
  }
  // U' rows for phase 2 (requested here, not with the other loads, so that
  // they are not live across phase 1; their latency overlaps S^T Q^T)
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    ufr[ks] = ((ks >> 1) == 0 || need1) ? ld8nt(Up + (bh * C + c0 + (ks >> 1)) * DV * L + u_elem(dvr, 32 * (ks & 1) + 8 * g4))
                                   : zero_frag<I>();
  __syncthreads();

  // ---- phase 2: dv rows 16w..16w+15 of O^T for every token tile
  f32x4 acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = zero4();
  if (Ssrc != nullptr) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const frag_t<I> qf = ld8(&sQ[(16 * j + n16) * QSTR + 32 * ks + 8 * g4]);
        acc[j] = mma(sfr[ks], qf, acc[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const float fac = exp2f(sG[16 * (j0 + j) + n16] + lf);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) acc[j][jj] *= fac;
    }
  }
  // local terms: U'^T A^T, source 32-blocks ks (chunk c0 + ks / 2)
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      if (ks <= ((j0 + j) >> 1)) {
        const frag_t<I> af = ld8(&sA[(16 * j + n16) * ASTR + 32 * ks + 8 * g4]);
        acc[j] = mma(ufr[ks], af, acc[j]);
      }
    }
  }

  const float scale = 0.08838834764831845f;   // 128^-1/2
  __syncthreads();   // Q and A^T are no longer read
  // (rows past the end of a sequence hold zeros, so the check covers only
  // what is stored; a finite value beyond the range of o's type counts too)
  bool nfo = false;
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    f32x4 v = acc[j];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      v[jj] *= scale;
      nfo |= !__builtin_isfinite(to_f(from_f<OT>(v[jj])));   // as stored (range of o's type)
    }
    *reinterpret_cast<f32x4*>(&sO[(16 * j + n16) * OSTR + 16 * w + 4 * g4]) = v;
  }
  flag_or(p.stats, b, ST_NF_OUT, nfo ? NF_O : 0);
  __syncthreads();
  // rows of 128 values: 32 consecutive lanes write one token's row
  OT* O = static_cast<OT*>(p.o);
#pragma unroll
  for (int it = 0; it < NT; ++it) {
    const int q = tid + 512 * it;
    const int t = q >> 5, c4 = (q & 31) * 4;
    const int tok = c0 * L + 16 * j0 + t;
    if (tok < sp.len)
      st4o_nt<OT>(O + ((size_t)(sp.tok0 + tok) * Nv + h) * DV + c4, *reinterpret_cast<const f32x4*>(&sO[t * OSTR + c4]));
  }
}

template <typename E, bool ONE>
void launch_e(const OChunkArgs& a, dim3 grid, hipStream_t s) {
  if (a.o_type == OUT_BF16)
    hipLaunchKernelGGL((ochunk_kernel<E, sgdn::bf16, ONE>), grid, dim3(512), 0, s, a);
  else if (a.o_type == OUT_F16)
    hipLaunchKernelGGL((ochunk_kernel<E, sgdn::fp16, ONE>), grid, dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL((ochunk_kernel<E, float, ONE>), grid, dim3(512), 0, s, a);
}

template <bool ONE>
void launch_one(const OChunkArgs& a, int bf16, dim3 grid, hipStream_t s) {
  if (bf16)
    launch_e<sgdn::bf16, ONE>(a, grid, s);
  else
    launch_e<float, ONE>(a, grid, s);
}

}  // namespace

hipError_t launch_ochunk(const OChunkArgs& a, int bf16, hipStream_t s) {
  dim3 grid(a.G * (a.per_chunk ? 2 : 1) * 2 * a.nrows * a.B);
  if (a.per_chunk)
    launch_one<true>(a, bf16, grid, s);
  else
    launch_one<false>(a, bf16, grid, s);
  return hipGetLastError();
}

}  // namespace sgdn
