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

constexpr int EVT = 256;         // sparse: events per LDS metadata tile

template <typename E, bool SPARSE>
__global__ __launch_bounds__(256) void hscan_kernel(HScanArgs p) {
  __shared__ __align__(32) E sS[16 * SSTR];
  __shared__ __align__(32) float sX[16 * XSTR];
  // sparse event metadata of the current tile: chunk, snapshot slot, gap factor
  __shared__ int sEvC[SPARSE ? EVT + 1 : 1];
  __shared__ int sEvSlot[SPARSE ? EVT : 1];
  __shared__ float sEvF[SPARSE ? EVT : 1];

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
  const int pr = SPARSE ? p.row_pair[b * NP + row] : row;
  const int h = 2 * pr + hh;
  const int dv0 = 16 * slice;

  int i0 = 0, i1 = C;
  if constexpr (SPARSE) {
    i0 = p.row_ptr[b * (NP + 1) + row];
    i1 = p.row_ptr[b * (NP + 1) + row + 1];
  }
  const int32_t* colb = SPARSE ? p.col + (size_t)b * p.Emax : nullptr;
  const int32_t* slotb = SPARSE ? p.event_slot + (size_t)b * p.Emax : nullptr;
  const size_t bh = (size_t)b * Nv + h;
  const double* P = SPARSE ? p.P + bh * (C + 1) : nullptr;

  // Stage the metadata of events [t0, t0 + EVT): chunk index, snapshot slot
  // and the gap factor 2^(P_next - P_{c+1}) that carries S_{c+1} to the next
  // event (Eq. (21)); the last event carries it to the end of the sequence.
  auto stage_meta = [&](int t0) {
    if constexpr (SPARSE) {
      for (int e = tid; e <= EVT; e += 256) {
        const int i = t0 + e;
        if (i < i1) {
          const int c = colb[i];
          sEvC[e] = c;
          if (e < EVT) {
            sEvSlot[e] = slotb[i];
            const int cn = (i + 1 < i1) ? colb[i + 1] : C;
            sEvF[e] = exp2f((float)(P[cn] - P[c + 1]));
          }
        }
      }
      __syncthreads();
    }
  };
  auto chunk_at = [&](int i, int t0) { return SPARSE ? sEvC[i - t0] : i; };

  // ---- initial state: s0 decayed over the chunks before the first event
  f32x4 S[2];
  {
    float f0 = 1.f;
    if constexpr (SPARSE) f0 = exp2f((float)P[(i0 < i1) ? colb[i0] : C]);
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
  int t0 = i0;
  stage_meta(t0);
  __syncthreads();

  const E* Wbase = static_cast<const E*>(p.W);
  const E* KTbase = static_cast<const E*>(p.KT);
  float* Ubase = p.U;
  float* snap = p.snap;

  // Operands of one event, loaded one event ahead so that the global-memory
  // latency of event i+1 overlaps the matrix work of event i.
  struct Ops {
    frag_t<E> wf[4], kf[2][2];
    f32x4 u, gv;
    float gam;
    int c;
  };
  auto load = [&](int i, int c, Ops& o) {
    const size_t hc = bh * C + c;
    const E* Wt = SPARSE ? Wbase + (((size_t)b * p.Emax + i) * 2 + hh) * L * DK
                         : Wbase + hc * L * DK;
    const E* KTt = KTbase + (((size_t)b * p.Nq + pr) * C + c) * DK * L;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) o.wf[ks] = ld8(Wt + (16 * w + n16) * DK + 32 * ks + 8 * g4);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) o.kf[tt][ks] = ld8(KTt + (32 * w + 16 * tt + n16) * L + 32 * ks + 8 * g4);
    o.u = *reinterpret_cast<const f32x4*>(Ubase + hc * DV * L + (dv0 + n16) * L + 16 * w + 4 * g4);
    o.gv = *reinterpret_cast<const f32x4*>(p.g + hc * L + 16 * w + 4 * g4);
    o.gam = p.gamma[hc];
    o.c = c;
  };

  // One event step; `cur` holds this event's operands, `nxt` receives the
  // next event's.  The loop alternates two buffers (no register copies, so
  // the wait for `nxt` lands at its first use one step later).
  auto step = [&](int i, Ops& cur, Ops& nxt) {
    if constexpr (SPARSE) {
      // event i opens the next metadata tile; the barrier that ended the
      // previous step guarantees nobody still reads the old tile
      if (i - t0 == EVT) {
        t0 += EVT;
        stage_meta(t0);
      }
    }
    const bool more = i + 1 < i1;
    const int c = cur.c;
    const size_t hc = bh * C + c;
    float* Ut = Ubase + hc * DV * L + (dv0 + n16) * L + 16 * w + 4 * g4;

    // ---- U' = U - W S   (Eq. (1))
    f32x4 acc = zero4();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) acc = mma(cur.wf[ks], ld8(&sS[n16 * SSTR + 32 * ks + 8 * g4]), acc);
    // next event's operands are requested only after this event's are in use,
    // so waiting for `cur` never waits for `nxt` (loads retire in order).  The
    // request is unconditional (the last event re-reads its own operands): a
    // branch here would make the wait counts merge to a full drain.
    // sEvC holds EVT + 1 entries, so i + 1 - t0 <= EVT is always staged.
    {
      const int in = more ? i + 1 : i;
      load(in, chunk_at(in, t0), nxt);
    }
    f32x4 up, x;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      up[j] = cur.u[j] - acc[j];
      x[j] = up[j] * exp2f(cur.gam - cur.gv[j]);
    }
    st4f(Ut, up);
    st4f(&sX[n16 * XSTR + 16 * w + 4 * g4], x);
    lds_barrier();

    // ---- S <- 2^gamma S + K^T (U' * 2^(gamma - g))   (Eq. (2))
    const float dec = exp2f(cur.gam);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      f32x4 d = zero4();
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) d = mma_split_b(cur.kf[tt][ks], ld8f(&sX[n16 * XSTR + 32 * ks + 8 * g4]), d);
#pragma unroll
      for (int j = 0; j < 4; ++j) S[tt][j] = dec * S[tt][j] + d[j];
    }

    // ---- compact snapshot of S_{c+1} if an output group starts from it
    float* sp = nullptr;
    if constexpr (SPARSE) {
      const int es = sEvSlot[i - t0];
      if (es >= 0) sp = snap + (((size_t)b * p.snap_cap + es) * 2 + hh) * DV * DK;
    } else {
      if ((c & 1) && c + 1 < C) sp = snap + (bh * (G - 1) + (c + 1) / 2 - 1) * DV * DK;
    }
    if (sp != nullptr) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) st4f(sp + (dv0 + n16) * DK + 32 * w + 16 * tt + 4 * g4, S[tt]);
    }

    // ---- gap to the next event (Eq. (21)): S_next = 2^(P_next - P_{c+1}) S
    if constexpr (SPARSE) {
      const float f = sEvF[i - t0];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int j = 0; j < 4; ++j) S[tt][j] *= f;
    }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) st4(&sS[n16 * SSTR + 32 * w + 16 * tt + 4 * g4], S[tt]);
    lds_barrier();
  };

  Ops bufA, bufB;
  if (i0 < i1) load(i0, chunk_at(i0, t0), bufA);
  for (int i = i0; i < i1; i += 2) {
    step(i, bufA, bufB);
    if (i + 1 < i1) step(i + 1, bufB, bufA);
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
  if (bf16) {
    if (a.sparse)
      hipLaunchKernelGGL((hscan_kernel<sgdn::bf16, true>), dim3(nblk), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((hscan_kernel<sgdn::bf16, false>), dim3(nblk), dim3(256), 0, s, a);
  } else {
    if (a.sparse)
      hipLaunchKernelGGL((hscan_kernel<float, true>), dim3(nblk), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((hscan_kernel<float, false>), dim3(nblk), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace sgdn
