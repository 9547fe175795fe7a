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
//            LDS as bf16 hi + lo halves (B operand layout [t][s]);
//   phase 2: wave w owns dv rows 16w..16w+15 of O^T for all 128 tokens, so
//            each row of the fp32 state and of U' is read exactly once.
// fp32-valued operands (state, U', A) enter the bf16 matrix cores as hi + lo
// halves (products: S x Q two terms, U' x A three terms).
#include "common.h"
#include "kernels.h"

namespace sgdn {

namespace {

constexpr int QSTR = DK + 8;      // Q rows [t][dk]
constexpr int ASTR = 2 * L + 8;   // A^T rows [t][s], s over the group's 128 tokens

template <typename E, typename OT>
__global__ __launch_bounds__(512) void ochunk_kernel(OChunkArgs p) {
  constexpr bool kSplit = sizeof(E) == 2;
  __shared__ __align__(32) E sQ[2 * L * QSTR];
  __shared__ __align__(32) E sAh[2 * L * ASTR];
  __shared__ __align__(32) E sAl[kSplit ? 2 * L * ASTR : 8];
  __shared__ float sG[2 * L];

  const int r = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int n16 = lane & 15, g4 = lane >> 4;
  const int T = p.T, Nq = p.Nq, Nv = p.Nv, C = p.C, G = p.G;
  const int pr = h >> 1, hh = h & 1;
  const int c0 = 2 * r;
  const bool has1 = c0 + 1 < C;
  const int ntile = has1 ? 8 : 4;           // 16-token tiles in this group
  const size_t bh = (size_t)b * Nv + h;

  // ---- group entry state: source and log2 factor
  const float* Ssrc = nullptr;
  float lf = 0.f;
  if (p.sparse) {
    const size_t pg = ((size_t)b * (Nv / 2) + pr) * G + r;
    const int slot = p.group_slot[pg];
    const double* P = p.P + bh * (C + 1);
    if (slot >= 0) {
      const int e = p.pred[pg];
      Ssrc = p.snap + (((size_t)b * p.snap_cap + slot) * 2 + hh) * DV * DK;
      lf = (float)(P[c0] - P[e + 1]);
    } else if (p.s0T != nullptr) {
      Ssrc = p.s0T + bh * DV * DK;
      lf = (float)P[c0];
    }
  } else {
    if (r > 0)
      Ssrc = p.snap + (bh * (G - 1) + r - 1) * DV * DK;
    else if (p.s0T != nullptr)
      Ssrc = p.s0T + bh * DV * DK;
  }

  // ---- global loads of both phases are issued up front so that their
  //      latencies overlap (one workgroup holds the CU's LDS); the Q rows to
  //      stage go first, because loads retire in order
  const E* Qin = static_cast<const E*>(p.q);
  const E* Kin = static_cast<const E*>(p.k);
  frag_t<E> qst[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int q = tid + 512 * it;
    const int rr = q >> 4, c8 = (q & 15) * 8;
    const int t = c0 * L + rr;
    qst[it] = (rr < ntile * 16 && t < T) ? ld8(Qin + ((size_t)(b * T + t) * Nq + pr) * DK + c8)
                                         : zero_frag<E>();
  }
  frag_t<E> kf[4];
  {
    const int ts = c0 * L + 16 * w + n16;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      kf[ks] = (w < ntile && ts < T) ? ld8(Kin + ((size_t)(b * T + ts) * Nq + pr) * DK + 32 * ks + 8 * g4)
                                     : zero_frag<E>();
  }
  const int dvr = 16 * w + n16;
  f32x8 sfr[4], ufr[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    sfr[ks] = Ssrc != nullptr ? ld8f(Ssrc + (size_t)dvr * DK + 32 * ks + 8 * g4) : f32x8{};
    ufr[ks] = (2 * ks < ntile) ? ld8f(p.U + ((bh * C + c0 + (ks >> 1)) * DV + dvr) * L + 32 * (ks & 1) + 8 * g4)
                               : f32x8{};
  }

  // ---- stage Q rows of the group and G
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int q = tid + 512 * it;
    const int rr = q >> 4, c8 = (q & 15) * 8;
    *reinterpret_cast<frag_t<E>*>(&sQ[rr * QSTR + c8]) = qst[it];
  }
  if (tid < 128) {
    const int cc = tid >> 6;
    float gv = 0.f;
    if (cc == 0) {
      gv = p.g[(bh * C + c0) * L + lane];
    } else if (has1) {
      gv = p.gamma[bh * C + c0] + p.g[(bh * C + c0 + 1) * L + lane];
    }
    sG[tid] = gv;
  }
  __syncthreads();

  // ---- phase 1: A^T blocks of source tile w (s in 16w..16w+15)
  if (w < ntile) {
    float gs[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) gs[j] = sG[16 * w + 4 * g4 + j];
    // the block just above the diagonal (source tile w, token tile w - 1) is
    // read by the 32-wide k-steps of phase 2; the causal mask makes it zero
    for (int jt = (w > 0 ? w - 1 : 0); jt < ntile; ++jt) {
      f32x4 at = zero4();
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        at = mma(kf[ks], ld8(&sQ[(16 * jt + n16) * QSTR + 32 * ks + 8 * g4]), at);
      const int t = 16 * jt + n16;
      const float gt = sG[t];
      f32x4 hi4, lo4;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int s = 16 * w + 4 * g4 + j;
        const float v = (s <= t) ? at[j] * exp2f(gt - gs[j]) : 0.f;
        hi4[j] = v;
      }
      if constexpr (kSplit) {
        half_t<E> hh4, ll4;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          hh4[j] = (bf16)hi4[j];
          ll4[j] = (bf16)(hi4[j] - (float)hh4[j]);
        }
        *reinterpret_cast<half_t<E>*>(&sAh[t * ASTR + 16 * w + 4 * g4]) = hh4;
        *reinterpret_cast<half_t<E>*>(&sAl[t * ASTR + 16 * w + 4 * g4]) = ll4;
      } else {
        st4<E>(&sAh[t * ASTR + 16 * w + 4 * g4], hi4);
      }
    }
  }
  __syncthreads();

  // ---- phase 2: dv rows 16w..16w+15 of O^T for every token tile
  f32x4 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = zero4();
  if (Ssrc != nullptr) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const f32x8 sf = sfr[ks];
      frag_t<E> sh, sl;
      if constexpr (kSplit) split8(sf, sh, sl); else sh = sf;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j < ntile) {
          const frag_t<E> qf = ld8(&sQ[(16 * j + n16) * QSTR + 32 * ks + 8 * g4]);
          acc[j] = mma(sh, qf, acc[j]);
          if constexpr (kSplit) acc[j] = mma(sl, qf, acc[j]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float fac = exp2f(sG[16 * j + n16] + lf);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) acc[j][jj] *= fac;
    }
  }
  // local terms: U'^T A^T, source 32-blocks ks (chunk c0 + ks / 2)
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    if (2 * ks >= ntile) break;
    const f32x8 uf = ufr[ks];
    frag_t<E> uh, ul;
    if constexpr (kSplit) split8(uf, uh, ul); else uh = uf;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < ntile && ks <= (j >> 1)) {
        const frag_t<E> ah = ld8(&sAh[(16 * j + n16) * ASTR + 32 * ks + 8 * g4]);
        acc[j] = mma(uh, ah, acc[j]);
        if constexpr (kSplit) {
          const frag_t<E> al = ld8(&sAl[(16 * j + n16) * ASTR + 32 * ks + 8 * g4]);
          acc[j] = mma(ul, ah, acc[j]);
          acc[j] = mma(uh, al, acc[j]);
        }
      }
    }
  }

  const float scale = 0.08838834764831845f;   // 128^-1/2
  OT* O = static_cast<OT*>(p.o);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int tok = c0 * L + 16 * j + n16;
    if (j < ntile && tok < T) {
      f32x4 v = acc[j];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) v[jj] *= scale;
      st4o<OT>(O + ((size_t)(b * T + tok) * Nv + h) * DV + 16 * w + 4 * g4, v);
    }
  }
}

}  // namespace

hipError_t launch_ochunk(const OChunkArgs& a, int bf16, hipStream_t s) {
  dim3 grid(a.G, a.Nv, a.B);
  if (bf16) {
    if (a.o_bf16)
      hipLaunchKernelGGL((ochunk_kernel<sgdn::bf16, sgdn::bf16>), grid, dim3(512), 0, s, a);
    else
      hipLaunchKernelGGL((ochunk_kernel<sgdn::bf16, float>), grid, dim3(512), 0, s, a);
  } else {
    if (a.o_bf16)
      hipLaunchKernelGGL((ochunk_kernel<float, sgdn::bf16>), grid, dim3(512), 0, s, a);
    else
      hipLaunchKernelGGL((ochunk_kernel<float, float>), grid, dim3(512), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace sgdn
