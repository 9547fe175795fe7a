// H scan: the sequential state recurrence over the events of one value head.
//
// SparseGDN reading notes: Sec. 2.1 Eqs. (1)-(2) (U' = U - W S,
// S <- 2^gamma S + K^T (U' * 2^(gamma - g))), Sec. 2.6 Eqs. (17)-(21)
// (skipped events only decay; consecutive kept events e < c are joined by the
// gap factor 2^(P_c - P_{e+1}); U' overwrites U in place; only snapshots that
// later output groups reference are stored; the final state is returned).
//
// Value columns of S evolve independently (both equations act column-wise),
// so one workgroup owns one 16-column slice of one head's 128x128 state and
// walks that head's events in time.  Four waves split each step:
//   W S    : wave w computes token rows 16w..16w+15 of U' (A = W from global,
//            B = S from LDS, 4 k-steps over d)
//   K^T X  : wave w updates state rows 32w..32w+31 (A = K^T tile from global,
//            B = X = U' * 2^(gamma - g) from LDS, 2 k-steps over tokens)
// The fp32 state stays in registers; a bf16 (or fp32) copy in LDS is the
// operand of the next step's W S (a single bf16 rounding there costs < 0.3% of
// the output RMS).  U, U' and X are fp32; X enters K^T X as bf16 hi + lo
// halves, and snapshots are stored in fp32, because single bf16 roundings of
// these move the outputs by 1-4% of their RMS.
#include "common.h"
#include "kernels.h"

namespace sgdn {

namespace {

constexpr int PAD = 8;
constexpr int SSTR = DK + PAD;  // LDS state copy [16 dv][dk]
constexpr int XSTR = L + PAD;   // LDS X [16 dv][64 tokens]

template <typename E>
__global__ __launch_bounds__(256) void hscan_kernel(HScanArgs p) {
  __shared__ __align__(32) E sS[16 * SSTR];
  __shared__ __align__(32) float sX[16 * XSTR];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int n16 = lane & 15, g4 = lane >> 4;
  const int Nv = p.Nv, C = p.C, B = p.B;
  const int NP = Nv / 2;
  const int G = (C + 1) / 2;

  // Block -> (row, batch, head-in-pair, slice).  The 16 workgroups of one
  // head pair (2 heads x 8 slices) share K^T and W tiles, so they are placed
  // on one XCD (workgroups are dealt to the 8 XCDs round-robin); rows are
  // dispatched in order, so the longest (High-tier) chains start first.
  const int id = blockIdx.x, nblk = gridDim.x;
  int pg, local;
  if ((nblk & 127) == 0) {
    pg = (id >> 7) * 8 + (id & 7);
    local = (id >> 3) & 15;
  } else {
    pg = id >> 4;
    local = id & 15;
  }
  const int row = pg / B, b = pg % B;
  const int hh = local >> 3, slice = local & 7;
  const int pr = p.sparse ? p.row_pair[b * NP + row] : row;
  const int h = 2 * pr + hh;
  const int dv0 = 16 * slice;

  int i0, i1;
  if (p.sparse) {
    i0 = p.row_ptr[b * (NP + 1) + row];
    i1 = p.row_ptr[b * (NP + 1) + row + 1];
  } else {
    i0 = 0;
    i1 = C;
  }
  const int32_t* colb = p.sparse ? p.col + (size_t)b * p.Emax : nullptr;
  auto chunk_of = [&](int i) { return p.sparse ? colb[i] : i; };
  const size_t bh = (size_t)b * Nv + h;
  const double* P = p.P ? p.P + bh * (C + 1) : nullptr;

  // ---- initial state: s0 decayed over the chunks before the first event
  f32x4 S[2];
  {
    const int cf = (i0 < i1) ? chunk_of(i0) : C;
    const float f0 = (P != nullptr) ? exp2f((float)P[cf]) : 1.f;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int dk = 32 * w + 16 * tt + 4 * g4 + j;
        S[tt][j] = p.s0 ? f0 * p.s0[(bh * DK + dk) * DV + dv0 + n16] : 0.f;
      }
      st4(&sS[n16 * SSTR + 32 * w + 16 * tt + 4 * g4], S[tt]);
    }
  }
  __syncthreads();

  const E* Wbase = static_cast<const E*>(p.W);
  const E* KTbase = static_cast<const E*>(p.KT);
  float* Ubase = p.U;
  float* snap = p.snap;

  for (int i = i0; i < i1; ++i) {
    const int c = chunk_of(i);
    const size_t hc = bh * C + c;
    // ---- operands of this event
    const E* Wt = p.sparse ? Wbase + (((size_t)b * p.Emax + i) * 2 + hh) * L * DK
                           : Wbase + hc * L * DK;
    const E* KTt = KTbase + (((size_t)b * p.Nq + pr) * C + c) * DK * L;
    float* Ut = Ubase + hc * DV * L + (dv0 + n16) * L + 16 * w + 4 * g4;
    frag_t<E> wf[4], kf[2][2];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) wf[ks] = ld8(Wt + (16 * w + n16) * DK + 32 * ks + 8 * g4);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) kf[tt][ks] = ld8(KTt + (32 * w + 16 * tt + n16) * L + 32 * ks + 8 * g4);
    const f32x4 u = *reinterpret_cast<const f32x4*>(Ut);
    const f32x4 gv = *reinterpret_cast<const f32x4*>(p.g + hc * L + 16 * w + 4 * g4);
    const float gam = p.gamma[hc];

    // ---- U' = U - W S   (Eq. (1))
    f32x4 acc = zero4();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) acc = mma(wf[ks], ld8(&sS[n16 * SSTR + 32 * ks + 8 * g4]), acc);
    f32x4 up, x;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      up[j] = u[j] - acc[j];
      x[j] = up[j] * exp2f(gam - gv[j]);
    }
    st4f(Ut, up);
    st4f(&sX[n16 * XSTR + 16 * w + 4 * g4], x);
    __syncthreads();

    // ---- S <- 2^gamma S + K^T (U' * 2^(gamma - g))   (Eq. (2))
    const float dec = exp2f(gam);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      f32x4 d = zero4();
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) d = mma_split_b(kf[tt][ks], ld8f(&sX[n16 * XSTR + 32 * ks + 8 * g4]), d);
#pragma unroll
      for (int j = 0; j < 4; ++j) S[tt][j] = dec * S[tt][j] + d[j];
    }

    // ---- compact snapshot of S_{c+1} if an output group starts from it
    float* sp = nullptr;
    if (p.sparse) {
      const int es = p.event_slot[(size_t)b * p.Emax + i];
      if (es >= 0) sp = snap + (((size_t)b * p.snap_cap + es) * 2 + hh) * DV * DK;
    } else if ((c & 1) && c + 1 < C) {
      sp = snap + (bh * (G - 1) + (c + 1) / 2 - 1) * DV * DK;
    }
    if (sp != nullptr) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) st4f(sp + (dv0 + n16) * DK + 32 * w + 16 * tt + 4 * g4, S[tt]);
    }

    // ---- gap to the next event (Eq. (21)): S_next = 2^(P_next - P_{c+1}) S
    const int cn = (i + 1 < i1) ? chunk_of(i + 1) : C;
    if (P != nullptr && cn != c + 1) {
      const float f = exp2f((float)(P[cn] - P[c + 1]));
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int j = 0; j < 4; ++j) S[tt][j] *= f;
    }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) st4(&sS[n16 * SSTR + 32 * w + 16 * tt + 4 * g4], S[tt]);
    __syncthreads();
  }

  if (p.s_final != nullptr) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int dk = 32 * w + 16 * tt + 4 * g4 + j;
        p.s_final[(bh * DK + dk) * DV + dv0 + n16] = S[tt][j];
      }
  }
}

}  // namespace

hipError_t launch_hscan(const HScanArgs& a, int bf16, hipStream_t s) {
  const int nblk = a.B * (a.Nv / 2) * 16;
  if (bf16)
    hipLaunchKernelGGL(hscan_kernel<sgdn::bf16>, dim3(nblk), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(hscan_kernel<float>, dim3(nblk), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace sgdn
