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
// walks that head's events in time.  Its compute wave holds the slice (eight
// 16x16 fp32 tiles over the key rows) in registers, so both products feed
// each other without leaving the wave:
//   W S    : A = W blocks, B = the state tiles stacked in pairs (permuted
//            reduction order, converted to the intermediate type)
//   K^T X  : A = K^T blocks, B = the U' tiles stacked in pairs, scaled
// The other waves keep the compute wave's instruction stream free of global
// memory operations, which would queue behind the operand requests of the
// CU:
//   two loader waves stream each event's operands (W, K^T, the U slice, the
//     per-token factors 2^(gamma - g) and a 16-byte event record) straight
//     from global memory into a ring of LDS slots with the direct
//     global-to-LDS loads of gfx950, DEPTH events ahead (with the Cb
//     operand three: one for the direct loads of Cb, U, the factors and the
//     record, and two that form the K^T blocks from the chunk's bf16 key
//     rows in their registers, so that no K^T copy is written to memory);
//   a storer wave copies U' and the snapshots, which the compute wave leaves
//     in a two-entry LDS staging ring, to global memory one event later.
// One workgroup barrier per event hands a filled slot to the compute wave and
// an emptied one back to the loaders.
//
// Two operand forms (template CBP): the W operand above (dense path, fp32
// inputs, and the sparse controls with W of every chunk), and for the sparse
// path with fp16 intermediates the Cb operand, where W = Cb K is never formed
// (W S = Cb (K S)) and the state rows are split over two compute waves; see
// the comment at the kernel.
//
// The gap factor that carries S to the next event is kept out of the state
// registers: with S_true = F_in * S, the step forms U' = U - F_in (W S) and
// S <- (2^gamma F_in) S + K^T X, so S is the true state after every update
// (the snapshot) and one scaling per event remains.
#include "common.h"
#include "kernels.h"

#include <type_traits>

namespace sgdn {

namespace {

typedef __attribute__((address_space(1))) void gvoid;
typedef __attribute__((address_space(3))) void lvoid;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int NLD = 2;          // loader waves (W operand)
// waves: compute (one; two with the Cb operand), loaders (two; three with
// the Cb operand: two for the key rows, one for the direct loads), storer
constexpr int NWAVE = 2 + NLD;
constexpr int NWAVE_CB = 6;

// One ring slot per event: W blocks (or, CBP, the six Cb blocks of the head),
// K^T blocks, the U slice [16 dv][64 t] (rearranged for conflict-free reads),
// 64 factors 2^(gamma - g_t), and the event record {F_in, 2^gamma F_in,
// snapshot index, chunk} (repeated).
// Staging entry: U' (same arrangement as U), the snapshot [16 dv][128 dk] in
// 16-byte units (8 keys of one value row), and {chunk, snapshot index}.
template <typename I, bool PFON, bool CBP> struct Ring {
  static constexpr int FB = 512 * (int)sizeof(I);   // one fragment block
  static constexpr int NWB = CBP ? CB_BLOCKS : 16;   // blocks of W (of Cb)
  static constexpr int W_OFF = 0;
  static constexpr int K_OFF = NWB * FB;
  // (CBP: the K^T blocks of key tile mt start 16 mt bytes later, see kblk_r)
  static constexpr int U_OFF = (NWB + 16) * FB + (CBP ? 128 : 0);
  static constexpr int U_BYTES = 16 * L * (int)sizeof(I);
  static constexpr int F_OFF = U_OFF + U_BYTES;
  static constexpr int R_OFF = F_OFF + 256;
  static constexpr int BYTES = R_OFF + 256;
  // events requested ahead (CBP: the compute waves also read the slot of the
  // next event, so one more is in the ring)
  static constexpr int DEPTH = CBP ? 4 : (sizeof(I) == 2 ? 3 : 1);
  static constexpr int NS = DEPTH + 1;
  // copy units of one event: 1 KB pieces (16 bytes per lane), then the
  // factors and the record (4 bytes per lane)
  static constexpr int NWA = NWB * FB / 1024;       // pieces of W (of Cb)
  // pieces of K^T copied by direct loads (CBP: none; the loader waves form
  // the K^T blocks from the key rows themselves)
  static constexpr int NW = CBP ? 0 : 16 * FB / 1024;
  static constexpr int NUS = U_BYTES / 1024;         // pieces of the U slice
  static constexpr int NX4 = NWA + NW + NUS;
  // L2 prefetch (fp16 operands): one scattered 4-byte request per event that
  // touches this workgroup's share of the W (Cb) and K^T lines its XCD will
  // copy, and its own U and factor lines, PF_AHEAD events before they are
  // copied (its data lands in a scratch row).  The workgroups of a pair on
  // one XCD request each line once between them, so the copies of the others
  // hit in L2.
  static constexpr bool PF = PFON;
  static constexpr int PF_AHEAD = 6;
  static constexpr int NU = NX4 + 2 + (PF ? 1 : 0);
  // units per loader wave (CBP: loader 2 issues all of them, loaders 0 and 1
  // form the K^T blocks)
  static constexpr int PER = (NU + NLD - 1) / NLD;
  // staging (the fp32 ring leaves no room: there the compute wave stores)
  static constexpr bool STAGE = sizeof(I) == 2;
  static constexpr int SN_BYTES = 16 * DK * (int)sizeof(I);
  static constexpr int ST_SN = U_BYTES;
  static constexpr int ST_HDR = ST_SN + SN_BYTES;
  static constexpr int ST_BYTES = STAGE ? ST_HDR + 16 : 16;
};

// Element offset of K^T block (mt, ks) in a ring slot of the Cb-operand
// scan: the fragment-major block of kblk, shifted by 16 mt bytes, so that
// the loader's stores of one unit per lane into the eight key tiles fall into
// different LDS banks (the blocks are otherwise a multiple of the bank
// period apart); reads within one block are unchanged.
__device__ __forceinline__ int kblk_r(int mt, int ks) { return kblk(mt, ks) + 8 * mt; }

template <int N> __device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}

// Barrier of the loader waves: they write LDS through the direct loads,
// whose completion they have waited for, and (Cb operand) through their own
// stores of the K^T blocks, waited for here; no fence (which could also wait
// for the requests still in flight) is needed.
__device__ __forceinline__ void loader_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Barrier of the storer wave: its LDS reads are complete (so the compute wave
// may refill the entry), while its global stores stay in flight (nothing in
// this kernel reads them; a fence would wait for them and hold the compute
// wave up).
__device__ __forceinline__ void storer_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Two transposed LDS reads (ds_read_b64_tr_b16) forming one 8-element MFMA
// operand: in each 16-lane group lane m supplies the address of 4 contiguous
// elements (row m / 4, columns 4 (m % 4) .. + 3 of a 4 x 16 block) and lane n
// receives column n, rows 0 .. 3.
__device__ __forceinline__ fp16x8 ld_tr_pair(const fp16* p0, const fp16* p1) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p1));
  return __builtin_bit_cast(fp16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// direct global-to-LDS loads: lane l's 16 (4) bytes land at lds + 16 l (4 l)
__device__ __forceinline__ void dma16(const void* src, void* lds) {
  __builtin_amdgcn_global_load_lds((gvoid*)src, (lvoid*)lds, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* src, void* lds) {
  __builtin_amdgcn_global_load_lds((gvoid*)src, (lvoid*)lds, 4, 0, 0);
}

// Byte offset of lane (n, g)'s 4 values of token tile i in a U slice
// [16 dv][64 t] as the ring holds it.  fp16: row n is 8 consecutive 16-byte
// units (8 tokens each), token unit u at position u ^ (n >> 1) of the row, so
// that the 16 rows a wave reads at once fall into distinct LDS banks while
// every 1 KiB copy moves 8 whole rows, i.e. whole 128-byte lines of the
// slice in global memory; fp32: unit 64 i + 16 g + n holds tokens
// 16 i + 4 g .. + 3 of row n.
template <typename I> __device__ __forceinline__ int u_off(int i, int n, int g) {
  if constexpr (sizeof(I) == 2) return (8 * n + ((2 * i + (g >> 1)) ^ (n >> 1))) * 16 + 8 * (g & 1);
  else return (64 * i + 16 * g + n) * 16;
}
// Element offset (from the slice's first row, u_elem(dv0, 0), in global
// memory) of the 16-byte unit P of that arrangement: each 1 KiB copy moves
// whole lines (fp16: 8 rows of all four token tiles; fp32: one token tile).
template <typename I> __device__ __forceinline__ int u_unit(int P) {
  if constexpr (sizeof(I) == 2) return u_elem(P >> 3, 8 * ((P & 7) ^ (P >> 4)));
  else return u_elem(P & 15, 16 * (P >> 6) + 4 * ((P >> 4) & 3));
}
// Staged snapshot slice [16 dv][128 dk]: row n is 16 consecutive 16-byte
// units (8 keys each), key unit c at position c ^ n of the row (the writers'
// 16 rows fall into distinct LDS banks; each 1 KiB copy moves 4 whole rows).
__device__ __forceinline__ int sn_unit(int c, int n) { return 16 * n + (c ^ n); }

// (two waves per SIMD for the register budget: at most 256 registers per
// lane, so the products accumulate in ordinary vector registers; the LDS ring
// keeps one workgroup per CU)
// CBP (sparse, fp16 intermediates): the ring holds the head's Cb blocks
// instead of W, and the compute wave forms W S = Cb (K S): Y = K S from the
// K^T blocks read transposed (gfx950's ds_read_b64_tr_b16: four consecutive
// tokens of one key are 8 contiguous bytes of a K^T block), then Cb Y from Y
// converted to the intermediate type.  The operand stream per event drops
// from 34 KiB (W, K^T, U) to 24 KiB (Cb, K^T, U).
//
// CBP also splits the compute over two waves (on two SIMDs): compute wave cw
// owns key rows 64 cw .. 64 cw + 63 of the slice's state.  Each forms its
// half of the next event's Y = K S from that event's slot at the end of the
// current step and leaves it in LDS; after the event barrier both add the
// two halves (in the same order) and form Cb Y, U' and X identically; each
// then updates its own state rows with K^T X.  The loaders keep two events
// complete at every barrier (the current and the next).
// BA (Cb operand only): the block-adjacent solve, whose Cb has no block (3,0).
template <typename E, bool SPARSE, bool CBP, bool BA>
__global__ __launch_bounds__(64 * (CBP ? NWAVE_CB : NWAVE), 2) void hscan_kernel(HScanArgs p) {
  using I = inter_t<E>;
  static_assert(!CBP || sizeof(I) == 2, "Cb operand: fp16 intermediates only");
  // (the sparse Cb-operand scan issues no L2 prefetch: its High-tier chains
  // run on a quarter of the CUs, their loads hit in L2 without one, and the
  // scattered request only adds to the per-CU memory pipeline that bounds
  // the step; measured 2% faster without.  The dense scan keeps it.)
  using R = Ring<I, sizeof(I) == 2 && !(CBP && SPARSE), CBP>;
  constexpr int D = R::DEPTH, NS = R::NS;
  // copy unit of the Cb block (3,0) (zero with the block-adjacent solve)
  constexpr int CB_SKIP = 4;
  static_assert(!CBP || cb_block(3, 0) == CB_SKIP, "Cb block (3,0)");
  constexpr int NCW = CBP ? 2 : 1;         // compute waves 0 .. NCW - 1
  constexpr int NL = CBP ? 3 : NLD;        // loader waves
  constexpr int WST = NCW + NL;            // storer wave (loaders in between)
  static_assert(WST + 1 == (CBP ? NWAVE_CB : NWAVE), "wave roles");
  static_assert(!CBP || D >= 2, "two events complete at each barrier");
  __shared__ __align__(16) char ring[NS * R::BYTES];
  __shared__ __align__(16) char stage[2 * R::ST_BYTES];
  __shared__ __align__(16) char pf_sink[256];
  // CBP: halves of the next event's Y, [parity][compute wave][token tile][lane]
  __shared__ __align__(16) f32x4 ych[CBP ? 2 * 2 * 4 * 64 : 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15, g4 = lane >> 4;
  const int Nv = p.Nv, C = p.C, B = p.B;
  const int NP = Nv / 2;
  const int G = (C + 1) / 2;

  // Block -> (row, batch, head-in-pair, slice).  The 16 workgroups of one
  // head pair (2 heads x 8 slices) share K^T tiles and each head's 8 share W,
  // so they are placed on one XCD (workgroups are dealt to the 8 XCDs
  // round-robin, starting at an XCD that varies between launches; XCD k
  // below counts from it): a window of 128 workgroups holds 8 pair groups,
  // group k on XCD (k + xcd_shift) mod 8.  Spread: group k of a window (k < 4) has its
  // head 0 on XCD k and its head 1 on XCD k + 4 (group k + 4 likewise), so a
  // long chain takes a quarter of two XCDs rather than half of one, and the
  // launches beside it find the XCDs more evenly free.  A launch covers rows
  // row_lo .. row_lo + nrows - 1 of every sequence; its grid is padded to
  // whole windows and the padding leaves at once.  Rows are dispatched in
  // order, so the longest (High-tier) chains start first.
  const int id = blockIdx.x, nr = p.nrows;
  const int xc = id & 7, jx = (id >> 3) & 15;   // XCD (counted as above) and slot on it
  const int pg = (id >> 7) * 8 + (p.spread ? (xc & 3) + 4 * (jx >> 3) : ((xc - p.xcd_shift) & 7));
  if (pg >= B * nr) return;
  const int local = p.spread ? (xc >> 2) * 8 + (jx & 7) : jx;
  // Packed sequences (dense): sequence-major, so the pair groups dispatched
  // together belong to one sequence and their chains are equally long (they
  // start and finish together and keep sharing the pair's lines in L2).
  const bool seq_major = !SPARSE && p.cu != nullptr;
  const int row = p.row_lo + (seq_major ? pg % nr : pg / B), b = seq_major ? pg / nr : pg % B;
  const int hh = local >> 3, slice = local & 7;
  const int pr = SPARSE ? p.row_pair[b * NP + row] : row;
  const int h = 2 * pr + hh;
  const int dv0 = 16 * slice;

  // dense: every chunk is an event (a packed sequence's valid chunks only)
  int i0 = 0, i1 = p.cu == nullptr ? C : chunks_of(seq_span(p.cu, b, p.T).len);
  if constexpr (SPARSE) {
    i0 = p.row_ptr[b * (NP + 1) + row];
    i1 = p.row_ptr[b * (NP + 1) + row + 1];
  }
  const int32_t* colb = SPARSE ? p.col + (size_t)b * p.Emax : nullptr;
  const size_t bh = (size_t)b * Nv + h;
  I* Ubase = static_cast<I*>(p.U);
  I* snap = static_cast<I*>(p.snap);
  const int snap_cap = SPARSE ? p.snap_cap : G - 1;
  auto snap_at = [&](int si) __attribute__((always_inline)) {
    return SPARSE ? snap + (((size_t)b * p.snap_cap + si) * 2 + hh) * DV * DK
                  : snap + (bh * (G - 1) + si) * DV * DK;
  };

  if (w == WST) {
    // ======================= storer wave =======================
    // copy staging entry e (U' and the snapshot of one event) to global memory
    auto copy_out = [&](int e) __attribute__((always_inline)) {
      const char* st = stage + e * R::ST_BYTES;
      const int2 hd = *reinterpret_cast<const int2*>(st + R::ST_HDR);
      // (clamped like the compute wave's record fields: no staging content
      // can address memory outside U and the snapshots)
      const int c = min(max(__builtin_amdgcn_readfirstlane(hd.x), 0), C - 1);
      const int sn = __builtin_amdgcn_readfirstlane(hd.y);
      const int si = (sn >= 0 && sn < snap_cap) ? sn : -1;
      I* Ug = Ubase + (bh * C + c) * DV * L + u_elem(dv0, 0);
      if (sn != NULL_EVENT) {   // a null event keeps U
#pragma unroll
        for (int r = 0; r < R::U_BYTES / 1024; ++r) {
          const int P = 64 * r + lane;
          stv(Ug + u_unit<I>(P), ldv(st + P * 16));
        }
      }
      if (si >= 0) {
        I* sp = snap_at(si);
#pragma unroll
        for (int r = 0; r < R::SN_BYTES / 1024; ++r) {
          const int P = 64 * r + lane;   // unit of row n = P >> 4 (see sn_unit)
          stv(sp + s_elem(dv0 + (P >> 4), 8 * ((P & 15) ^ (P >> 4))), ldv(st + R::ST_SN + P * 16));
        }
      }
    };
    for (int j = i0; j < i1; ++j) {
      storer_barrier();   // the compute wave has left event j - 1 in staging
      if (R::STAGE && j > i0) copy_out((j - 1 - i0) & 1);
    }
    storer_barrier();     // the compute wave is done
    if (R::STAGE && i1 > i0) copy_out((i1 - 1 - i0) & 1);
    return;
  }

  if (w >= NCW) {
    // ======================= loader waves =======================
    const int k = w - NCW;
    // event chunks are read through the scalar cache (constant address space:
    // the event list is not written during the kernel), so their waits never
    // mix with the counted direct loads
    const cint32* colc = (const cint32*)(colb);
    auto col_at = [&](int e) __attribute__((always_inline)) {
      return SPARSE ? colc[__builtin_amdgcn_readfirstlane(e)] : e;
    };
    const I* Wbase = static_cast<const I*>(p.W);
    // W and K^T packed per kept event (deferred W), or per chunk (dense, and
    // the deferred-W ablation of the sparse path)
    const bool w_ev = SPARSE && !p.w_by_chunk;
    const I* KTbase = static_cast<const I*>(p.KT);
    const I* Cbase = static_cast<const I*>(p.Cb);
    // Cb operand: the key rows (input type E) of the event's chunk
    const E* Kin = static_cast<const E*>(p.k);
    const SeqSpan ksp = seq_span(p.cu, b, p.T);
    // L2 prefetch of event e (clamped to the row): lanes 0-15 the 16 W lines
    // of this slice's share of the head's tile (CBP: lanes 0-5 the 6 of the
    // head's 48 Cb lines, 6-15 repeat lane 0), 16-31 this workgroup's share of
    // the pair's 128 K^T lines (16 when spread; 8 with the pair on one XCD,
    // lanes 24-31 repeating 16-23), 32-47 the 16 lines of its U slice, 48-49
    // the factors, the rest repeat lane 0
    auto prefetch = [&](int e) __attribute__((always_inline)) {
      e = e < i1 ? e : i1 - 1;
      const int c = col_at(e);
      const size_t hc = bh * C + c;
      const char* Wt = reinterpret_cast<const char*>(
          w_ev ? Wbase + (((size_t)b * p.Emax + e) * 2 + hh) * L * DK : Wbase + hc * L * DK);
      const char* Kt = reinterpret_cast<const char*>(
          w_ev ? KTbase + ((size_t)b * p.Emax + e) * DK * L : KTbase + (((size_t)b * p.Nq + pr) * C + c) * DK * L);
      const char* Ut = reinterpret_cast<const char*>(Ubase + hc * DV * L + u_elem(dv0, 0));
      const char* Ct = reinterpret_cast<const char*>(Cbase + hc * (CB_BLOCKS * 512));
      const char* src = CBP ? Ct + slice * 6 * 128 : Wt + slice * 16 * 128;
      if (lane < 16) {
        if (!CBP) src = Wt + (slice * 16 + lane) * 128;
        else if (lane < 6) src = Ct + (slice * 6 + lane) * 128;
      } else if (lane < 32) {
        const int kl = p.spread ? slice * 16 + lane - 16 : (hh * 8 + slice) * 8 + ((lane - 16) & 7);
        if constexpr (CBP) {
          // line kl of the chunk's 64 key rows (two 128-byte lines per row)
          const int tc = min(c * L + (kl >> 1), ksp.len - 1);
          src = reinterpret_cast<const char*>(Kin + ((size_t)(ksp.tok0 + tc) * p.Nq + pr) * DK) + (kl & 1) * 128;
        } else {
          src = Kt + kl * 128;
        }
      } else if (lane < 48) {
        // the slice's 512 bytes of each token tile: four lines per tile
        src = Ut + ((lane - 32) >> 2) * (DV * 16 * (int)sizeof(I)) + ((lane - 32) & 3) * 128;
      } else if (lane < 50) src = reinterpret_cast<const char*>(p.fac + hc * L) + (lane - 48) * 128;
      dma4(src, pf_sink);
    };
    // copy units [u0, u1) of event j (chunk c) into slot s
    auto issue = [&](int j, int c, int s, int u0, int u1) __attribute__((always_inline)) {
      const size_t hc = bh * C + c;
      const char* Wt = reinterpret_cast<const char*>(
          w_ev ? Wbase + (((size_t)b * p.Emax + j) * 2 + hh) * L * DK : Wbase + hc * L * DK);
      const char* Kt = reinterpret_cast<const char*>(
          w_ev ? KTbase + ((size_t)b * p.Emax + j) * DK * L : KTbase + (((size_t)b * p.Nq + pr) * C + c) * DK * L);
      const I* Ut = Ubase + hc * DV * L + u_elem(dv0, 0);
      const int32_t* rec = SPARSE ? p.rec + (((size_t)b * p.Emax + j) * 2 + hh) * 4 : p.rec + hc * 4;
      char* sl = ring + s * R::BYTES;
#pragma unroll
      for (int u = u0; u < u1; ++u) {
        if (CBP && BA && u == CB_SKIP) {
          // the block-adjacent Cb has no block (3,0): nothing to copy
        } else if (u < R::NWA) {
          if constexpr (CBP)
            dma16(reinterpret_cast<const char*>(Cbase + hc * (CB_BLOCKS * 512)) + u * 1024 + lane * 16,
                  sl + R::W_OFF + u * 1024);
          else
            dma16(Wt + u * 1024 + lane * 16, sl + R::W_OFF + u * 1024);
        } else if (u < R::NWA + R::NW) {
          dma16(Kt + (u - R::NWA) * 1024 + lane * 16, sl + R::K_OFF + (u - R::NWA) * 1024);
        } else if (u < R::NX4) {
          const int r = u - R::NWA - R::NW;
          dma16(Ut + u_unit<I>(64 * r + lane), sl + R::U_OFF + r * 1024);
        } else if (u == R::NX4) {
          dma4(p.fac + hc * L + lane, sl + R::F_OFF);
        } else if (u == R::NX4 + 1) {
          dma4(rec + (lane & 3), sl + R::R_OFF);
        } else {
          prefetch(j + R::PF_AHEAD);
        }
      }
    };
    // Cb operand: the K^T blocks of an event come from the chunk's key rows
    // through the registers of loader waves 0 and 1 (token steps 0 and 1),
    // which issue no direct loads (their LDS stores then never wait for
    // direct loads still in flight); loader wave 2 issues every direct load.
    // Lane (n, g) of key wave ks loads keys 8 n .. 8 n + 7 of the eight
    // tokens 32 ks + 4 g + r (r < 4) and 32 ks + 16 + 4 g + r - 4 (r >= 4),
    // i.e. one 16-byte unit of eight tokens for each of its eight keys in the
    // permuted reduction order of the blocks.  Rows past the end of the
    // sequence repeat its last token (finite: they meet only exact zeros, the
    // rows of X and the columns of Cb there, so the products are those of
    // zero rows).  The requests of event j + 4 go out two steps before their
    // conversion (bf16 -> fp32 -> fp16, rounded to nearest even) and stores.
    static_assert(!CBP || std::is_same<E, sgdn::bf16>::value, "key rows are bf16");
    const int kws = w - NCW;   // token step of a key wave
    auto ktok = [&](int r) __attribute__((always_inline)) {
      return 32 * kws + 4 * g4 + (r & 3) + 16 * (r >> 2);
    };
    auto kload = [&](int c, u32x4 (&kr)[8]) __attribute__((always_inline)) {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int tc = min(c * L + ktok(r), ksp.len - 1);
        kr[r] = *reinterpret_cast<const u32x4*>(Kin + ((size_t)(ksp.tok0 + tc) * p.Nq + pr) * DK + 8 * n16);
      }
    };
    auto kstore = [&](int s, u32x4 (&kv)[8]) __attribute__((always_inline)) {
      // (the key registers pass through an empty asm here, so that their
      // conversion is not scheduled ahead of the barrier and of the requests
      // before this point, whose overlap with the wait it would undo)
#pragma unroll
      for (int r = 0; r < 8; ++r) asm volatile("" : "+v"(kv[r]) :: "memory");
      I* Ks = reinterpret_cast<I*>(ring + s * R::BYTES + R::K_OFF);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        // key 8 n + e of each token: bf16 bits in the low half of word e / 2
        // for even e, the high half for odd e
        frag_t<I> u;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const uint32_t x = kv[r][e >> 1];
          u[r] = from_f<I>(__uint_as_float((e & 1) ? (x & 0xffff0000u) : (x << 16)));
        }
        const int key = 8 * n16 + e;
        *reinterpret_cast<frag_t<I>*>(Ks + kblk_r(key >> 4, kws) + 8 * kswz((key & 15) + 16 * g4)) = u;
      }
    };
    auto run_keys = [&]() __attribute__((always_inline)) {
      static_assert(!CBP || (D == 4 && NS == 5), "key path: events j + 2 .. j + 4 in flight");
      // Every step issues the same requests (events past the row's end are
      // clamped to its last event; their stores land in ring slots no event
      // uses), so the wait counts are exact and no branch skips a request.
      const int jlast = i1 - 1;
      auto ev = [&](int e) __attribute__((always_inline)) { return e < jlast ? e : jlast; };
      // three register sets: event i0 + m in set m mod 3
      u32x4 k0[8], k1[8], k2[8];
      int s2 = 2;   // slot of event j + 2
      // (the chunk of event j + 4 is read a step early, so that its latency
      // is not paid between barrier and request)
      int c4 = 0;
      // step j: requests of event j + 4's keys (into kl), then event j + 2
      // (its keys, requested two steps earlier into kc_) converted and stored
      auto step = [&](int j, u32x4 (&kl)[8], u32x4 (&kc_)[8]) __attribute__((always_inline)) {
        loader_barrier();   // event j handed over; this wave's stores of j + 1 done
        kload(c4, kl);
        c4 = col_at(ev(j + 5));
        wait_vm<16>();      // the keys of j + 2 (those of j + 3 and j + 4 in flight)
        kstore(s2, kc_);
        s2 = (s2 + 1 == NS) ? 0 : s2 + 1;
      };
      if (i0 < i1) {
        kload(col_at(i0), k0);
        kload(col_at(ev(i0 + 1)), k1);
        wait_vm<0>();
        kstore(0, k0);   // events i0 and i0 + 1 before the first barrier
        kstore(1, k1);
        kload(col_at(ev(i0 + 2)), k2);
        kload(col_at(ev(i0 + 3)), k0);
        c4 = col_at(ev(i0 + 4));
        int j = i0;
        for (; j + 2 < i1; j += 3) {
          step(j, k1, k2);
          step(j + 1, k2, k0);
          step(j + 2, k0, k1);
        }
        if (j < i1) step(j, k1, k2);
        if (j + 1 < i1) step(j + 1, k2, k0);
        wait_vm<0>();   // no request outlives the loop
      }
      loader_barrier();
    };
    // per-loader unit ranges are compile-time constants, so every loop above
    // unrolls into straight-line requests
    auto run = [&](auto u0c, auto u1c) __attribute__((always_inline)) {
      constexpr int U0 = decltype(u0c)::value, U1 = decltype(u1c)::value;
      // requests per event (the block-adjacent Cb operand skips one unit)
      constexpr int CNT = U1 - U0 - ((CBP && BA && U0 <= CB_SKIP && CB_SKIP < U1) ? 1 : 0);
      if (i0 < i1) {
        const int npro = (i1 - i0 < D) ? i1 - i0 : D;
#pragma unroll
        for (int e = 0; e < D; ++e)
          if (e < npro) issue(i0 + e, col_at(i0 + e), e, U0, U1);
        if (npro == D) wait_vm<CNT * (D - (CBP ? 2 : 1))>();   // first (two) events complete
        else wait_vm<0>();
      }
      // sparse: the chunk of the next request is read one event early, so
      // that its load latency is not paid between barrier and request
      const int jlast = i1 > i0 ? i1 - 1 : i0;
      int cnext = col_at(min(i0 + D, jlast));
      int s = D;   // slot of event j + D
      for (int j = i0; j < i1; ++j) {
        loader_barrier();   // event j handed over; slot of j - 1 emptied
        if (j + D < i1) {
          const int c = cnext;
          cnext = col_at(min(j + D + 1, jlast));
          issue(j + D, c, s, U0, U1);
          wait_vm<CNT * (D - (CBP ? 2 : 1))>();   // event j + 1 (CBP: and j + 2) complete
        } else {
          wait_vm<0>();
        }
        s = (s + 1 == NS) ? 0 : s + 1;
      }
      loader_barrier();
    };
    static_assert(NL == (CBP ? 3 : 2), "one branch per loader wave");
    using I0 = std::integral_constant<int, 0>;
    using IN = std::integral_constant<int, R::NU>;
    if constexpr (CBP) {
      if (k < 2) run_keys();
      else run(I0{}, IN{});
    } else {
      constexpr int P1 = R::PER < R::NU ? R::PER : R::NU;
      if (k == 0) run(I0{}, std::integral_constant<int, P1>{});
      else run(std::integral_constant<int, P1>{}, IN{});
    }
    return;
  }

  if constexpr (CBP) {
    // =================== compute waves (Cb operand) ===================
    const int cw = w;
    // the compute waves' chain is one of the step's two limits (the other
    // is the CU's memory pipeline, shared by the key, direct-load and storer
    // waves): they win issue arbitration against the direct-load and storer
    // waves that share their SIMDs (the six waves of a workgroup are dealt
    // to the four SIMDs in order)
    __builtin_amdgcn_s_setprio(3);
    const double* P = SPARSE ? p.P + bh * (C + 1) : nullptr;
    // initial state (all rows: the first event's Y is formed from it in
    // full by both waves), s0 decayed over the chunks before the first event
    f32x4 S[8];
    {
      const float f0 = SPARSE ? exp2f((float)P[(i0 < i1) ? colb[i0] : C]) : 1.f;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int dk = 16 * mt + 4 * g4 + j;
          S[mt][j] = p.s0 ? f0 * p.s0[(bh * DK + dk) * DV + dv0 + n16] : 0.f;
        }
    }
    // own rows: tiles 4 cw .. 4 cw + 3 (key steps 2 cw, 2 cw + 1), read
    // again rather than picked from S (a runtime pick would index S)
    f32x4 So[4];
    {
      const float f0 = SPARSE ? exp2f((float)P[(i0 < i1) ? colb[i0] : C]) : 1.f;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int dk = 16 * (4 * cw + t) + 4 * g4 + j;
          So[t][j] = p.s0 ? f0 * p.s0[(bh * DK + dk) * DV + dv0 + n16] : 0.f;
        }
    }
    frag_t<I> Sfo[2];
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) Sfo[qq] = pack44<I>(So[2 * qq], So[2 * qq + 1]);

    // A fragment of K over key step q (keys 32 q + 4 g + e, 32 q + 16 + 4 g +
    // e) for token tile i: lane m of group g points at key 32 q + 4 g + m / 4
    // (+ 16), tokens 16 i + 4 (m % 4) .. + 3: 8 contiguous bytes of the K^T
    // block (key tile, token step i / 2), unit kswz(key % 16 + 16 (m % 4))
    const int koff = 8 * kswz(4 * g4 + (n16 >> 2) + 16 * (n16 & 3));
    auto kfrag = [&](const I* Kb, int q, int i) __attribute__((always_inline)) {
      const int o = koff + 4 * (i & 1);
      return ld_tr_pair(Kb + kblk_r(2 * q, i >> 1) + o, Kb + kblk_r(2 * q + 1, i >> 1) + o);
    };
    const int kl = kswz(lane);

    // Operands of one event, read from its slot one step ahead: the event
    // after the current one is complete at every barrier, so each part of its
    // operands (Cb blocks; record, U slice and factors; this wave's K^T
    // blocks) is requested as soon as the current step has consumed the same
    // part, and their latency overlaps the step's remaining products instead
    // of the wait for LDS completion at the barrier.  (For the row's last
    // event the read slot is stale and the values unused.)
    struct Ops {
      int4 rc;
      frag_t<I> cb[CB_BLOCKS];
      half_t<I> u[4];
      f32x4 fc[4];
      frag_t<I> kt[4][2];
    };
    auto load_cb = [&](int slot, Ops& o) __attribute__((always_inline)) {
      const I* Cs = reinterpret_cast<const I*>(ring + slot * R::BYTES + R::W_OFF);
#pragma unroll
      for (int b = 0; b < CB_BLOCKS; ++b) o.cb[b] = ld8(Cs + b * 512 + 8 * lane);
    };
    auto load_uf = [&](int slot, Ops& o) __attribute__((always_inline)) {
      const char* sl = ring + slot * R::BYTES;
      o.rc = *reinterpret_cast<const int4*>(sl + R::R_OFF);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o.u[i] = *reinterpret_cast<const half_t<I>*>(sl + R::U_OFF + u_off<I>(i, n16, g4));
        o.fc[i] = *reinterpret_cast<const f32x4*>(sl + R::F_OFF + (16 * i + 4 * g4) * 4);
      }
    };
    auto load_kt = [&](int slot, Ops& o) __attribute__((always_inline)) {
      const I* Ks = reinterpret_cast<const I*>(ring + slot * R::BYTES + R::K_OFF);
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) o.kt[t][ks] = ld8(Ks + kblk_r(4 * cw + t, ks) + 8 * kl);
    };

    f32x4 y[4], ym[4];
    Ops op;
    int s = 0;
    int last_c = -1;   // chunk of the last event that updated the state
    if (i0 < i1) {
      lds_barrier();   // events i0 and i0 + 1 are in the ring
      const I* Ks = reinterpret_cast<const I*>(ring + R::K_OFF);
      frag_t<I> Sf[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) Sf[q] = pack44<I>(S[2 * q], S[2 * q + 1]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        y[i] = zero4();
#pragma unroll
        for (int q = 0; q < 4; ++q) y[i] = mma(kfrag(Ks, q, i), Sf[q], y[i]);
      }
      load_cb(0, op);
      load_uf(0, op);
      load_kt(0, op);
    }
    for (int j = i0; j < i1; ++j) {
      if (j > i0) {
        lds_barrier();   // event j + 1 in the ring; halves of Y(j) in LDS
        const f32x4* yo = ych + ((j & 1) * 2 + (1 - cw)) * 4 * 64;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x4 o = yo[i * 64 + lane];
          y[i] = cw == 0 ? ym[i] + o : o + ym[i];   // both: half 0 + half 1
        }
      }
      char* st = stage + ((j - i0) & 1) * R::ST_BYTES;
      const float fin = __int_as_float(__builtin_amdgcn_readfirstlane(op.rc.x));
      const float decf = __int_as_float(__builtin_amdgcn_readfirstlane(op.rc.y));
      // (chunk and snapshot index are clamped to their ranges, so that no
      // record content can address memory outside U and the snapshots)
      const int sn = __builtin_amdgcn_readfirstlane(op.rc.z);
      const int snapi = (sn >= 0 && sn < snap_cap) ? sn : -1;
      const int c = min(max(__builtin_amdgcn_readfirstlane(op.rc.w), 0), C - 1);
      last_c = c;
      // the next event's K fragments of this wave's key steps, requested now
      // (its slot is complete at this barrier) so that their latency overlaps
      // this step.  The step below has no branches, so the loads of all its
      // operands can be issued ahead of their products.
      const int s1 = (s + 1 == NS) ? 0 : s + 1;
      frag_t<I> kn[2][4];
      {
        const I* Kn = reinterpret_cast<const I*>(ring + s1 * R::BYTES + R::K_OFF);
#pragma unroll
        for (int qq = 0; qq < 2; ++qq)
#pragma unroll
          for (int i = 0; i < 4; ++i) kn[qq][i] = kfrag(Kn, 2 * cw + qq, i);
      }

      // ---- W S = Cb Y over source steps 0 (tokens 0-31) and 1 (32-63)
      const frag_t<I> Y0 = pack44<I>(y[0], y[1]), Y1 = pack44<I>(y[2], y[3]);
      auto cbf = [&](int i, int ks) __attribute__((always_inline)) { return op.cb[cb_block(i, ks)]; };
      const f32x4 a0 = mma(cbf(0, 0), Y0, zero4());
      const f32x4 a1 = mma(cbf(1, 0), Y0, zero4());
      const f32x4 a2 = mma(cbf(2, 1), Y1, mma(cbf(2, 0), Y0, zero4()));
      // (the block-adjacent solve stores no block (3,0))
      f32x4 a3 = mma(cbf(3, 1), Y1, zero4());
      if constexpr (!BA) a3 = mma(cbf(3, 0), Y0, a3);
      Ops nx;
      load_cb(s1, nx);

      // ---- U' = U - F_in W S (Eq. (1)); X = U' 2^(gamma - g); both waves
      //      form the same U' values, compute wave cw stages token tiles
      //      2 cw and 2 cw + 1 of it
      auto ux = [&](int i, const f32x4& ai) __attribute__((always_inline)) {
        f32x4 up, x;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          up[jj] = to_f(op.u[i][jj]) - fin * ai[jj];
          x[jj] = up[jj] * op.fc[i][jj];
        }
        if ((i >> 1) == cw) st4<I>(reinterpret_cast<I*>(st + u_off<I>(i, n16, g4)), up);
        return x;
      };
      const frag_t<I> X0 = pack44<I>(ux(0, a0), ux(1, a1));
      const frag_t<I> X1 = pack44<I>(ux(2, a2), ux(3, a3));
      load_uf(s1, nx);
      // ---- own rows: S <- 2^gamma F_in S + K^T X (Eq. (2))
#pragma unroll
      for (int t = 0; t < 4; ++t) So[t] = mma(op.kt[t][0], X0, So[t] * decf);
#pragma unroll
      for (int t = 0; t < 4; ++t) So[t] = mma(op.kt[t][1], X1, So[t]);
      load_kt(s1, nx);
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) Sfo[qq] = pack44<I>(So[2 * qq], So[2 * qq + 1]);

      // ---- compact snapshot of S_{c+1}, own key rows (key steps 2 cw + qq);
      //      staged only where a later output group references it
      if (snapi >= 0) {
#pragma unroll
        for (int qq = 0; qq < 2; ++qq)
#pragma unroll
          for (int hi = 0; hi < 2; ++hi) {
            const int c8 = 4 * (2 * cw + qq) + 2 * hi + (g4 >> 1);
            const half_t<I> v = hi ? __builtin_shufflevector(Sfo[qq], Sfo[qq], 4, 5, 6, 7)
                                   : __builtin_shufflevector(Sfo[qq], Sfo[qq], 0, 1, 2, 3);
            *reinterpret_cast<half_t<I>*>(st + R::ST_SN + sn_unit(c8, n16) * 16 + 8 * (g4 & 1)) = v;
          }
      }
      if (lane == 0) *reinterpret_cast<int2*>(st + R::ST_HDR) = make_int2(c, snapi);

      // ---- own half of the next event's Y
      f32x4* yw = ych + (((j + 1) & 1) * 2 + cw) * 4 * 64;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ym[i] = mma(kn[1][i], Sfo[1], mma(kn[0][i], Sfo[0], zero4()));
        yw[i * 64 + lane] = ym[i];
      }
      op = nx;
      s = s1;
    }
    lds_barrier();   // the last staging entry is complete

    if (p.s_final != nullptr) {
      // gap from the last event to the end of the sequence
      const float fl = (SPARSE && i1 > i0) ? exp2f((float)(P[C] - P[last_c + 1])) : 1.f;
      bool nfs = false;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int dk = 16 * (4 * cw + t) + 4 * g4 + j;
          const float x = fl * So[t][j];
          nfs |= !__builtin_isfinite(x);
          p.s_final[(bh * DK + dk) * DV + dv0 + n16] = x;
        }
      flag_or(p.stats, b, ST_NF_OUT, nfs ? NF_SFINAL : 0);
    }
    return;
  }

  // ======================= compute wave =======================
  const double* P = SPARSE ? p.P + bh * (C + 1) : nullptr;

  // initial state rows 16 mt + 4 g + j of column dv0 + n: s0 decayed over the
  // chunks before the first event
  f32x4 S[8];
  {
    float f0 = 1.f;
    if constexpr (SPARSE) f0 = exp2f((float)P[(i0 < i1) ? colb[i0] : C]);
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int dk = 16 * mt + 4 * g4 + j;
        S[mt][j] = p.s0 ? f0 * p.s0[(bh * DK + dk) * DV + dv0 + n16] : 0.f;
      }
  }
  frag_t<I> Sf[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) Sf[q] = pack44<I>(S[2 * q], S[2 * q + 1]);

  int s = 0;
  int last_c = -1;   // chunk of the last event that updated the state
  for (int j = i0; j < i1; ++j) {
    lds_barrier();   // the slot of event j is filled; staging entry free
    const char* sl = ring + s * R::BYTES;
    char* st = stage + ((j - i0) & 1) * R::ST_BYTES;
    const int4 rc = *reinterpret_cast<const int4*>(sl + R::R_OFF);
    const float fin = __int_as_float(__builtin_amdgcn_readfirstlane(rc.x));
    const float decf = __int_as_float(__builtin_amdgcn_readfirstlane(rc.y));
    // (chunk and snapshot index are clamped to their ranges, so that no
    // record content can address memory outside U and the snapshots)
    const int sn = __builtin_amdgcn_readfirstlane(rc.z);
    const int snapi = (sn >= 0 && sn < snap_cap) ? sn : -1;
    const int c = min(max(__builtin_amdgcn_readfirstlane(rc.w), 0), C - 1);
    // a null event (the CSR-off control) computes the products but leaves the
    // state and U as they are: X = 0, decay 1
    const bool null_ev = sn == NULL_EVENT;
    const float xsc = null_ev ? 0.f : 1.f;
    if (!null_ev) last_c = c;
    const I* Ws = reinterpret_cast<const I*>(sl + R::W_OFF);
    const I* Ks = reinterpret_cast<const I*>(sl + R::K_OFF);

    // ---- U' = U - F_in W S   (Eq. (1)) and
    //      S <- 2^gamma F_in S + K^T (U' 2^(gamma - g))   (Eq. (2)),
    // in token halves so that each half's vector work overlaps the products
    // of the next: W S of tiles 2-3 runs beside U' and X of tiles 0-1, K^T X
    // over tokens 0-31 beside U' and X of tiles 2-3
    auto ws_pair = [&](int i, f32x4& a0, f32x4& a1) __attribute__((always_inline)) {
      a0 = zero4();
      a1 = zero4();
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        a0 = mma(ld8(Ws + wblk(q, i) + 8 * lane), Sf[q], a0);
        a1 = mma(ld8(Ws + wblk(q, i + 1) + 8 * lane), Sf[q], a1);
      }
    };
    auto ux = [&](int i, const f32x4& a) __attribute__((always_inline)) {
      const half_t<I> u = *reinterpret_cast<const half_t<I>*>(sl + R::U_OFF + u_off<I>(i, n16, g4));
      const f32x4 fc = *reinterpret_cast<const f32x4*>(sl + R::F_OFF + (16 * i + 4 * g4) * 4);
      f32x4 up, x;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        up[jj] = to_f(u[jj]) - fin * a[jj];
        x[jj] = up[jj] * (fc[jj] * xsc);
      }
      if constexpr (R::STAGE)
        st4<I>(reinterpret_cast<I*>(st + u_off<I>(i, n16, g4)), up);
      else if (!null_ev)
        st4<I>(Ubase + (bh * C + c) * DV * L + u_elem(dv0 + n16, 16 * i + 4 * g4), up);
      return x;
    };
    f32x4 a0, a1, a2, a3;
    ws_pair(0, a0, a1);
    ws_pair(2, a2, a3);
    const frag_t<I> X0 = pack44<I>(ux(0, a0), ux(1, a1));
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) S[mt] = mma(ld8(Ks + kblk(mt, 0) + 8 * lane), X0, S[mt] * decf);
    const frag_t<I> X1 = pack44<I>(ux(2, a2), ux(3, a3));
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) S[mt] = mma(ld8(Ks + kblk(mt, 1) + 8 * lane), X1, S[mt]);
#pragma unroll
    for (int q = 0; q < 4; ++q) Sf[q] = pack44<I>(S[2 * q], S[2 * q + 1]);

    // ---- compact snapshot of S_{c+1} if an output group starts from it:
    //      lane (n, g) holds keys 32 q + 4 g .. + 3 and 32 q + 16 + 4 g .. + 3
    if constexpr (R::STAGE) {
      if (snapi >= 0) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int hi = 0; hi < 2; ++hi) {
            const int c8 = 4 * q + 2 * hi + (g4 >> 1);
            const half_t<I> v = hi ? __builtin_shufflevector(Sf[q], Sf[q], 4, 5, 6, 7)
                                   : __builtin_shufflevector(Sf[q], Sf[q], 0, 1, 2, 3);
            *reinterpret_cast<half_t<I>*>(st + R::ST_SN + sn_unit(c8, n16) * 16 + 8 * (g4 & 1)) = v;
          }
      }
      if (lane == 0) *reinterpret_cast<int2*>(st + R::ST_HDR) = make_int2(c, null_ev ? NULL_EVENT : snapi);
    } else if (snapi >= 0) {
      I* sp = snap_at(snapi);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        *reinterpret_cast<half_t<I>*>(sp + s_elem(dv0 + n16, 32 * q + 4 * g4)) = __builtin_shufflevector(Sf[q], Sf[q], 0, 1, 2, 3);
        *reinterpret_cast<half_t<I>*>(sp + s_elem(dv0 + n16, 32 * q + 16 + 4 * g4)) = __builtin_shufflevector(Sf[q], Sf[q], 4, 5, 6, 7);
      }
    }
    s = (s + 1 == NS) ? 0 : s + 1;
  }
  lds_barrier();   // the last staging entry is complete

  if (p.s_final != nullptr) {
    // gap from the last event to the end of the sequence
    float fl = 1.f;
    if constexpr (SPARSE)
      if (i1 > i0) fl = exp2f((float)(P[C] - P[last_c + 1]));
    bool nfs = false;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int dk = 16 * mt + 4 * g4 + j;
        const float x = fl * S[mt][j];
        nfs |= !__builtin_isfinite(x);
        p.s_final[(bh * DK + dk) * DV + dv0 + n16] = x;
      }
    flag_or(p.stats, b, ST_NF_OUT, nfs ? NF_SFINAL : 0);
  }
}

template <typename E, bool SPARSE, bool CBP, bool BA = false>
hipError_t launch_one(const HScanArgs& a, hipStream_t s) {
  const int nblk = 128 * ((a.B * a.nrows + 7) / 8);
  hipLaunchKernelGGL((hscan_kernel<E, SPARSE, CBP, BA>), dim3(nblk), dim3(64 * (CBP ? NWAVE_CB : NWAVE)), 0, s, a);
  return hipGetLastError();
}

template <bool SPARSE>
hipError_t launch_cb(const HScanArgs& a, hipStream_t s) {
  return a.blockadj ? launch_one<sgdn::bf16, SPARSE, true, true>(a, s)
                    : launch_one<sgdn::bf16, SPARSE, true, false>(a, s);
}

}  // namespace

hipError_t launch_hscan(const HScanArgs& a, int bf16, hipStream_t s) {
  if (bf16) {
    if (!a.sparse) return launch_cb<false>(a, s);
    // W of every chunk (the deferred-W and CSR-off controls) or W S from Cb
    return a.w_by_chunk ? launch_one<sgdn::bf16, true, false>(a, s) : launch_cb<true>(a, s);
  }
  return a.sparse ? launch_one<float, true, false>(a, s) : launch_one<float, false, false>(a, s);
}

}  // namespace sgdn
