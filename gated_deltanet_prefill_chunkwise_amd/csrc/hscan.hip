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
//   W S    : wave w computes token rows 16w..16w+15 of U' (A = W blocks,
//            B = S from its LDS copy, 4 k-steps over d)
//   K^T X  : wave w updates state rows 32w..32w+31 (A = K^T blocks, B = X from
//            LDS, 2 k-steps over tokens)
// W and K^T are fragment-major in memory (one contiguous 1 KB read per
// operand fragment) in a permuted reduction order; the LDS operands S and X
// are read in the same order.  The operands of an event do not depend on the
// state, so they are requested DEPTH events ahead into a ring of registers.
// The fp32 state stays in registers.  Operands and stored intermediates use
// the intermediate type I (fp16 for bf16 inputs, fp32 for fp32 inputs): the
// LDS copy of S for the next W S, X for K^T X, U, U' and the snapshots.
#include "common.h"
#include "kernels.h"

namespace sgdn {

namespace {

constexpr int PAD = 8;
constexpr int SSTR = DK + PAD;  // LDS state copy [16 dv][dk]
constexpr int XSTR = L + PAD;   // LDS X [16 dv][64 tokens]
constexpr int EVT = 240;        // events per LDS metadata tile

// 2^x for x <= 0 on the hardware exponential (results below 2^-126 flush to
// zero, far below the fp32 terms they are added to).
__device__ __forceinline__ float exp2_neg(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename E, bool SPARSE>
__global__ __launch_bounds__(256, 1) void hscan_kernel(HScanArgs p) {
  // events whose operands are in flight: 10 loads per event and wave, so the
  // ring plus the stores stays below the 63 vector-memory operations a wave
  // can count (fp32 intermediates are twice as large: a shorter ring)
  constexpr int DEPTH = sizeof(E) == 2 ? 4 : 2;
  static_assert(EVT % DEPTH == 0, "buffer ring must align with the tiles");
  using I = inter_t<E>;
  __shared__ __align__(16) I sS[16 * SSTR];
  __shared__ __align__(16) I sX[16 * XSTR];
  // event metadata of the current tile: chunk retention gamma; sparse also
  // chunk, snapshot slot and gap factor (chunk indices also for the DEPTH
  // events past the tile)
  __shared__ float sEvGam[EVT];
  __shared__ int sEvC[SPARSE ? EVT + DEPTH : 1];
  __shared__ int sEvSlot[SPARSE ? EVT : 1];
  __shared__ float sEvF[SPARSE ? EVT : 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
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

  // Stage the metadata of events [t0, t0 + EVT): gamma, and (sparse) chunk
  // index, snapshot slot and the gap factor 2^(P_next - P_{c+1}) that carries
  // S_{c+1} to the next event (Eq. (21)); the last event carries it to the end
  // of the sequence.  Chunk indices are staged DEPTH events further for the
  // operand requests.  Read from LDS, the per-event scalars stay out of the
  // vector-memory wait counts.
  auto stage_meta = [&](int t0) __attribute__((always_inline)) {
    for (int e = tid; e < EVT + DEPTH; e += 256) {
      const int i = t0 + e;
      if (i < i1) {
        const int c = SPARSE ? colb[i] : i;
        if (SPARSE) sEvC[e] = c;
        if (e < EVT) {
          sEvGam[e] = p.gamma[bh * C + c];
          if (SPARSE) {
            sEvSlot[e] = slotb[i];
            const int cn = (i + 1 < i1) ? colb[i + 1] : C;
            sEvF[e] = exp2f((float)(P[cn] - P[c + 1]));
          }
        }
      }
    }
    __syncthreads();
  };
  int t0 = i0;
  auto chunk_at = [&](int i) __attribute__((always_inline)) { return SPARSE ? sEvC[i - t0] : i; };

  // ---- initial state rows 32w + 16tt + 4g + j of column dv0 + n: s0 decayed
  //      over the chunks before the first event
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
      st4<I>(&sS[n16 * SSTR + 32 * w + 16 * tt + 4 * g4], S[tt]);
    }
    // the initial state is complete before any operand request, so the loop
    // never waits on these loads
    __builtin_amdgcn_s_waitcnt(0);
  }
  stage_meta(t0);

  const I* Wbase = static_cast<const I*>(p.W);
  const I* KTbase = static_cast<const I*>(p.KT);
  I* Ubase = static_cast<I*>(p.U);
  I* snap = static_cast<I*>(p.snap);

  // Operands of one event for this wave.
  struct Ops {
    frag_t<I> wf[4];      // W blocks (dk step q, token tile w)
    frag_t<I> kf[2][2];   // K^T blocks (dk tile 2w + tt, token step ks)
    half_t<I> u;          // U of tokens 16w + 4g .. 16w + 4g + 3
    f32x4 gv;             // g of the same tokens
    int c;
  };
  auto load = [&](int i, int c, Ops& o) __attribute__((always_inline)) {
    const size_t hc = bh * C + c;
    const I* Wt = SPARSE ? Wbase + (((size_t)b * p.Emax + i) * 2 + hh) * L * DK
                         : Wbase + hc * L * DK;
    const I* KTt = KTbase + (((size_t)b * p.Nq + pr) * C + c) * DK * L;
#pragma unroll
    for (int q = 0; q < 4; ++q) o.wf[q] = ld8(Wt + wblk(q, w) + 8 * lane);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) o.kf[tt][ks] = ld8(KTt + kblk(2 * w + tt, ks) + 8 * lane);
    o.u = *reinterpret_cast<const half_t<I>*>(Ubase + hc * DV * L + (dv0 + n16) * L + 16 * w + 4 * g4);
    o.gv = *reinterpret_cast<const f32x4*>(p.g + hc * L + 16 * w + 4 * g4);
    o.c = c;
  };
  // Request event i's operands (past the last event: the last event again,
  // unconditionally, so that no branch merges the wait counts into a drain).
  // sEvC holds EVT + DEPTH entries, so i - t0 < EVT + DEPTH is always staged.
  auto request = [&](int i, Ops& o) __attribute__((always_inline)) {
    const int in = i < i1 ? i : i1 - 1;
    load(in, chunk_at(in), o);
  };

  // One event step on the operands in `cur`; ends by requesting event
  // i + DEPTH into the same buffer.
  auto step = [&](int i, Ops& cur) __attribute__((always_inline)) {
    const int c = cur.c;
    const size_t hc = bh * C + c;
    const float gam = sEvGam[i - t0];

    // ---- U' = U - W S   (Eq. (1)); S read in the blocks' permuted order
    f32x4 acc = zero4();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const I* sr = &sS[n16 * SSTR + 32 * q + 4 * g4];
      acc = mma(cur.wf[q], ld44(sr, sr + 16), acc);
    }
    f32x4 up, x;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      up[j] = to_f(cur.u[j]) - acc[j];
      x[j] = up[j] * exp2_neg(gam - cur.gv[j]);
    }
    st4<I>(Ubase + hc * DV * L + (dv0 + n16) * L + 16 * w + 4 * g4, up);
    st4<I>(&sX[n16 * XSTR + 16 * w + 4 * g4], x);
    lds_barrier();

    // ---- S <- 2^gamma S + K^T (U' * 2^(gamma - g))   (Eq. (2)); X read in
    //      the K^T blocks' permuted token order
    const float dec = exp2_neg(gam);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      f32x4 d = S[tt] * dec;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const I* xr = &sX[n16 * XSTR + 32 * ks + 4 * g4];
        d = mma(cur.kf[tt][ks], ld44(xr, xr + 16), d);
      }
      S[tt] = d;
    }
    // the request reuses cur's registers: keep it after their last use, so the
    // buffers stay in place (a copy of an in-flight register forces a drain)
    __builtin_amdgcn_sched_barrier(0);
    request(i + DEPTH, cur);

    // ---- compact snapshot of S_{c+1} if an output group starts from it
    I* sp = nullptr;
    if constexpr (SPARSE) {
      const int es = sEvSlot[i - t0];
      if (es >= 0) sp = snap + (((size_t)b * p.snap_cap + es) * 2 + hh) * DV * DK;
    } else {
      if ((c & 1) && c + 1 < C) sp = snap + (bh * (G - 1) + (c + 1) / 2 - 1) * DV * DK;
    }
    if (sp != nullptr) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) st4<I>(sp + (dv0 + n16) * DK + 32 * w + 16 * tt + 4 * g4, S[tt]);
    }

    // ---- gap to the next event (Eq. (21)): S_next = 2^(P_next - P_{c+1}) S
    if constexpr (SPARSE) {
      const float f = sEvF[i - t0];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) S[tt] *= f;
    }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) st4<I>(&sS[n16 * SSTR + 32 * w + 16 * tt + 4 * g4], S[tt]);
    lds_barrier();
  };

  Ops buf[DEPTH];
  if (i0 < i1) {
#pragma unroll
    for (int k = 0; k < DEPTH; ++k) request(i0 + k, buf[k]);
  }
  // One metadata tile of EVT events per outer pass (EVT is a multiple of
  // DEPTH, so event i0 + k + n DEPTH always sits in buffer k).  The next tile
  // is staged at the end of a pass (the barrier that ends every step
  // guarantees nobody still reads the old one).  Only the last tile can end in
  // a partial group, so the way back to the event loop never follows
  // remainder steps (whose requests would look like the newest loads to the
  // wait-count analysis).
  auto run = [&](int ts, int te, bool last) __attribute__((always_inline)) {
    // whole groups of DEPTH events: straight-line steps, no guards
    int i = ts;
    for (; i + DEPTH <= te; i += DEPTH) {
#pragma unroll
      for (int k = 0; k < DEPTH; ++k) step(i + k, buf[k]);
    }
    if (last) {
      // the remaining 0 .. DEPTH-1 events; only the last tile has any
#pragma unroll
      for (int k = 0; k < DEPTH - 1; ++k)
        if (i + k < te) step(i + k, buf[k]);
    }
  };
  // (one call site: a second copy of the event loop would get its own
  // register assignment and copies of in-flight buffers)
  for (int ts = i0; ts < i1;) {
    const int te = (i1 - ts < EVT) ? i1 : ts + EVT;
    const bool last = te >= i1;
    run(ts, te, last);
    if (last) break;
    t0 = ts = te;
    stage_meta(t0);
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

template <typename E, bool SPARSE>
hipError_t launch_one(const HScanArgs& a, hipStream_t s) {
  const int nblk = a.B * (a.Nv / 2) * 16;
  hipLaunchKernelGGL((hscan_kernel<E, SPARSE>), dim3(nblk), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_hscan(const HScanArgs& a, int bf16, hipStream_t s) {
  if (bf16) return a.sparse ? launch_one<sgdn::bf16, true>(a, s) : launch_one<sgdn::bf16, false>(a, s);
  return a.sparse ? launch_one<float, true>(a, s) : launch_one<float, false>(a, s);
}

}  // namespace sgdn
