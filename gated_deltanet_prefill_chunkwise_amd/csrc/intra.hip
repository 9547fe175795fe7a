// Intra-chunk kernel: decay prefix, gated Gram matrix, local Delta solve
// (exact or block-adjacent), U = C diag(beta) V, W = C diag(beta 2^g) K (dense)
// or the staged coefficients C diag(beta 2^g) (sparse), the Tail-16 score, and
// transposed key tiles for the later stages.
//
// SparseGDN reading notes: Sec. 2.1 (g, gamma), Sec. 2.3 Eqs. (5)-(8) (local
// system, block-adjacent inverse, weighted coefficients), Sec. 2.4 Eq. (9)
// (tail score from the fp32 U while it is on chip).
//
// One workgroup (4 waves) per (chunk, head pair, batch): the pair shares its
// key tile and Gram matrix; the two value heads are solved one after the other.
#include "common.h"
#include "kernels.h"

namespace sgdn {

namespace {

constexpr int PAD = 8;
constexpr int KRS = DK + PAD;  // row stride of the row-major key tile
constexpr int TS = L + PAD;    // row stride of token-minor tiles (K^T, V^T, C)

// 16x16 blocks of the 64x64 lower triangle that the Gram matrix must fill.
__constant__ int kGramExact[10][2] = {{0, 0}, {1, 1}, {2, 2}, {3, 3}, {1, 0},
                                      {2, 1}, {3, 2}, {2, 0}, {3, 1}, {3, 0}};

template <typename E>
__global__ __launch_bounds__(256) void intra_kernel(IntraArgs p) {
  constexpr int KV_ELEMS = (L * KRS > DV * TS) ? L * KRS : DV * TS;
  __shared__ __align__(32) E sKV[KV_ELEMS];   // key tile row-major, later V^T
  __shared__ __align__(32) E sKT[DK * TS];    // key tile transposed [dk][t]
  __shared__ __align__(32) E sCC[L * TS];     // weighted coefficients [t][s]
  constexpr bool kSplit = sizeof(E) == 2;     // bf16: coefficients as hi + lo
  __shared__ __align__(32) E sCL[kSplit ? L * TS : 8];
  __shared__ float sG[L][L + 1];              // Gram <k_t, k_s>
  __shared__ float sM[L][L + 1];              // strictly lower part of M
  __shared__ float sC[L][L + 1];              // C ~ M^{-1}
  __shared__ float sY[3][16][17];
  __shared__ float sg[2][L], sb[2][L];

  const int c = blockIdx.x, pq = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int n16 = lane & 15, g4 = lane >> 4;
  const int T = p.T, Nq = p.Nq, Nv = p.Nv, C = p.C;
  const int t0 = c * L;
  const bool blockadj = p.solve == 1;
  const E* K = static_cast<const E*>(p.k);
  const E* V = static_cast<const E*>(p.v);
  const E* BETA = static_cast<const E*>(p.beta);

  // ---- key tile: row-major and transposed copies; a and beta of both heads
  for (int q = tid; q < L * 16; q += 256) {
    const int r = q >> 4, c8 = (q & 15) * 8, t = t0 + r;
    frag_t<E> val = zero_frag<E>();
    if (t < T) val = ld8(K + ((size_t)(b * T + t) * Nq + pq) * DK + c8);
    *reinterpret_cast<frag_t<E>*>(&sKV[r * KRS + c8]) = val;
#pragma unroll
    for (int j = 0; j < 8; ++j) sKT[(c8 + j) * TS + r] = val[j];
  }
  // ---- V tiles of both heads are fetched after the key tile (registers; loads retire in
  //      order) so their latency overlaps the Gram matrix and the solve
  frag_t<E> vpre[2][4];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int q = tid + 256 * it;
      const int r = q >> 4, c8 = (q & 15) * 8, t = t0 + r;
      vpre[hh][it] = t < T ? ld8(V + ((size_t)(b * T + t) * Nv + 2 * pq + hh) * DV + c8) : zero_frag<E>();
    }

  if (tid < 128) {
    const int hh = tid >> 6, t = t0 + lane, h = 2 * pq + hh;
    float av = 0.f, bv = 0.f;
    if (t < T) {
      av = p.a[(size_t)(b * T + t) * Nv + h];
      bv = to_f(BETA[(size_t)(b * T + t) * Nv + h]);
    }
    // inclusive prefix over the chunk (g, Sec. 2.1)
    float x = av;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(x, off, 64);
      if (lane >= off) x += y;
    }
    sg[hh][lane] = x;
    sb[hh][lane] = bv;
    const size_t hc = (size_t)(b * Nv + h) * C + c;
    p.g[hc * L + lane] = x;
    if (lane == 63) p.gamma[hc] = x;
  }
  __syncthreads();

  // ---- Gram matrix of the pair's keys (fp32 accumulation of bf16 products)
  {
    const int ntiles = blockadj ? 7 : 10;
    for (int ti = w; ti < ntiles; ti += 4) {
      const int bi = kGramExact[ti][0], bj = kGramExact[ti][1];
      f32x4 acc = zero4();
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const frag_t<E> fa = ld8(&sKV[(16 * bi + n16) * KRS + 32 * ks + 8 * g4]);
        const frag_t<E> fb = ld8(&sKV[(16 * bj + n16) * KRS + 32 * ks + 8 * g4]);
        acc = mma(fa, fb, acc);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) sG[16 * bi + 4 * g4 + j][16 * bj + n16] = acc[j];
    }
  }
  // transposed key tile for the H and deferred-W stages
  {
    E* kt = static_cast<E*>(p.KT) + ((size_t)(b * Nq + pq) * C + c) * DK * L;
    for (int q = tid; q < DK * 8; q += 256) {
      const int r = q >> 3, c8 = (q & 7) * 8;
      *reinterpret_cast<frag_t<E>*>(kt + r * L + c8) = ld8(&sKT[r * TS + c8]);
    }
  }
  __syncthreads();

  for (int hh = 0; hh < 2; ++hh) {
    const int h = 2 * pq + hh;
    const size_t hc = (size_t)(b * Nv + h) * C + c;
    // ---- M: beta_t <k_t,k_s> 2^(g_t - g_s) for s < t (Eq. (5)); C cleared
    for (int idx = tid; idx < L * L; idx += 256) {
      const int t = idx >> 6, s = idx & 63;
      const int bt = t >> 4, bs = s >> 4;
      float m = 0.f;
      if (s < t && (!blockadj || bt - bs <= 1))
        m = sb[hh][t] * sG[t][s] * exp2f(sg[hh][t] - sg[hh][s]);
      sM[t][s] = m;
      sC[t][s] = 0.f;
    }
    __syncthreads();
    // ---- diagonal blocks: C_ii = M_ii^{-1} by forward substitution, one
    //      column per thread (Eq. (8))
    if (tid < 64) {
      const int blk = tid >> 4, j = tid & 15, o = 16 * blk;
      float x[16];
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        float sum = (t == j) ? 1.f : 0.f;
#pragma unroll
        for (int s = 0; s < t; ++s) sum -= sM[o + t][o + s] * x[s];
        x[t] = sum;
      }
#pragma unroll
      for (int t = 0; t < 16; ++t) sC[o + t][o + j] = x[t];
    }
    __syncthreads();
    // ---- off-diagonal blocks, by distance d = i - j:
    //      C_ij = -C_ii sum_{k=j}^{i-1} M_ik C_kj.  Block-adjacent keeps d = 1
    //      only (C_i,i-1 = -C_ii M_i,i-1 C_i-1,i-1, Eq. (8)); exact adds d = 2, 3.
    const int dmax = blockadj ? 1 : 3;
    for (int d = 1; d <= dmax; ++d) {
      const int nb = 4 - d;
      const int r = tid >> 4, cc = tid & 15;
      for (int m = 0; m < nb; ++m) {
        const int i = d + m, j = i - d;
        float y = 0.f;
        for (int kb = j; kb < i; ++kb) {
#pragma unroll
          for (int u = 0; u < 16; ++u) y += sM[16 * i + r][16 * kb + u] * sC[16 * kb + u][16 * j + cc];
        }
        sY[m][r][cc] = y;
      }
      __syncthreads();
      for (int m = 0; m < nb; ++m) {
        const int i = d + m, j = i - d;
        float x = 0.f;
#pragma unroll
        for (int u = 0; u < 16; ++u) x -= sC[16 * i + r][16 * i + u] * sY[m][u][cc];
        sC[16 * i + r][16 * j + cc] = x;
      }
      __syncthreads();
    }

    // ---- U = C diag(beta) V  (Ct = C diag(beta)), and the tail score.
    //      Ct is applied as hi + lo halves so U keeps fp32 accuracy.
    for (int idx = tid; idx < L * L; idx += 256) {
      const int t = idx >> 6, s = idx & 63;
      const float ct = sC[t][s] * sb[hh][s];
      const E hi = from_f<E>(ct);
      sCC[t * TS + s] = hi;
      if constexpr (kSplit) sCL[t * TS + s] = from_f<E>(ct - to_f(hi));
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int q = tid + 256 * it;
      const int r = q >> 4, c8 = (q & 15) * 8;
      const frag_t<E> val = vpre[hh][it];
#pragma unroll
      for (int j = 0; j < 8; ++j) sKV[(c8 + j) * TS + r] = val[j];
    }
    __syncthreads();
    {
      // k-steps over s with non-zero coefficients for token tile w
      const int ks_lo = (blockadj && w == 3) ? 1 : 0;
      const int ks_hi = (w >= 2) ? 1 : 0;
      f32x4 acc[8];
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) acc[nt] = zero4();
      for (int ks = ks_lo; ks <= ks_hi; ++ks) {
        const frag_t<E> fa = ld8(&sCC[(16 * w + n16) * TS + 32 * ks + 8 * g4]);
        frag_t<E> fl;
        if constexpr (kSplit) fl = ld8(&sCL[(16 * w + n16) * TS + 32 * ks + 8 * g4]);
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
          const frag_t<E> fb = ld8(&sKV[(16 * nt + n16) * TS + 32 * ks + 8 * g4]);
          acc[nt] = mma(fa, fb, acc[nt]);
          if constexpr (kSplit) acc[nt] = mma(fl, fb, acc[nt]);
        }
      }
      float* U = p.U + hc * DV * L;
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) st4f(U + (16 * nt + n16) * L + 16 * w + 4 * g4, acc[nt]);
      if (p.score != nullptr && w == 3) {
        // Eq. (9): Frobenius norm of U rows 48..63, from the fp32 accumulators
        float ss = 0.f;
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
#pragma unroll
          for (int j = 0; j < 4; ++j) ss += acc[nt][j] * acc[nt][j];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
        if (lane == 0) p.score[hc] = sqrtf(ss);
      }
    }
    __syncthreads();

    // ---- Cb = C diag(beta 2^g): W (dense) or staged for deferred W (sparse)
    for (int idx = tid; idx < L * L; idx += 256) {
      const int t = idx >> 6, s = idx & 63;
      sCC[t * TS + s] = from_f<E>(sC[t][s] * sb[hh][s] * exp2f(sg[hh][s]));
    }
    __syncthreads();
    if (p.W != nullptr) {
      // W^T = K^T Cb^T: rows dk, columns t (so W is stored token-major)
      const int ks_lo = (blockadj && w == 3) ? 1 : 0;
      const int ks_hi = (w >= 2) ? 1 : 0;
      f32x4 acc[8];
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) acc[mt] = zero4();
      for (int ks = ks_lo; ks <= ks_hi; ++ks) {
        const frag_t<E> fb = ld8(&sCC[(16 * w + n16) * TS + 32 * ks + 8 * g4]);
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
          const frag_t<E> fa = ld8(&sKT[(16 * mt + n16) * TS + 32 * ks + 8 * g4]);
          acc[mt] = mma(fa, fb, acc[mt]);
        }
      }
      E* W = static_cast<E*>(p.W) + hc * L * DK;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) st4(W + (16 * w + n16) * DK + 16 * mt + 4 * g4, acc[mt]);
    }
    if (p.Cb != nullptr) {
      E* cb = static_cast<E*>(p.Cb) + hc * L * L;
      for (int q = tid; q < L * 8; q += 256) {
        const int r = q >> 3, c8 = (q & 7) * 8;
        *reinterpret_cast<frag_t<E>*>(cb + r * L + c8) = ld8(&sCC[r * TS + c8]);
      }
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_intra(const IntraArgs& a, int bf16, hipStream_t s) {
  dim3 grid(a.C, a.Nq, a.B);
  if (bf16)
    hipLaunchKernelGGL(intra_kernel<sgdn::bf16>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(intra_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace sgdn
