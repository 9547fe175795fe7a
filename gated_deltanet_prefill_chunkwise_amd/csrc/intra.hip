// Intra-chunk kernel: decay prefix, gated Gram matrix, local Delta solve
// (exact or block-adjacent), U = C diag(beta) V, W = C diag(beta 2^g) K (dense)
// or the staged coefficients C diag(beta 2^g) (sparse), the parts of the tail
// score, and transposed key tiles for the later stages.
//
// SparseGDN reading notes: Sec. 2.1 (g, gamma), Sec. 2.3 Eqs. (5)-(8) (local
// system, block-adjacent inverse, weighted coefficients), Sec. 2.4 Eq. (9)
// (sums of squares of U over 8-row blocks, from the fp32 U while it is on
// chip, for the tail score of any window).
//
// Persistent kernel: each workgroup (4 waves) walks over (chunk, head pair,
// batch) items and loads the next item's keys, values and gates into registers
// while it works on the current one.  The pair shares its key tile and Gram
// matrix; the two value heads are solved one after the other.
//
// Solve of the unit lower triangular 64x64 system (I + M) C = I in 16x16
// blocks: each wave inverts one diagonal block by forward substitution, then
// the off-diagonal blocks follow from fp32 matrix-core products (block
// adjacent: C_i,i-1 = -C_ii M_i,i-1 C_i-1,i-1 only; exact: the same for the
// two 32x32 halves, then the lower-left 32x32 block -C_hi M_hl C_lo).
//
// Key and value tiles stay row-major (token x feature) in LDS; products that
// contract over tokens read them with the gfx950 transposing LDS load.
#include "common.h"
#include "kernels.h"

namespace sgdn {

namespace {

constexpr int KS = DK + 8;      // row stride (elements) of the key / value tiles
constexpr int TP = 20;          // column stride (floats) of a stored 16x16 fp32 tile
constexpr int TILE = 16 * TP;   // floats per stored tile
constexpr int NT = 11;          // 10 lower-triangle blocks + one all-zero block
constexpr int ZT = 10;

// Slot of block (i, j) of the 4x4 block grid: the lower triangle, zero above
// it, and (block-adjacent solve) zero below the first sub-diagonal.
__device__ __forceinline__ int slot(int i, int j, bool ba) {
  if (j > i || (ba && i - j > 1)) return ZT;
  return i * (i + 1) / 2 + j;
}

// Gram block ti: the diagonal (0..3), the first sub-diagonal (4..6), then
// (2,0), (3,1), (3,0).
__device__ __forceinline__ void gram_block(int ti, int& bi, int& bj) {
  if (ti < 4) { bi = ti; bj = ti; }
  else if (ti < 7) { bi = ti - 3; bj = ti - 4; }
  else if (ti < 9) { bi = ti - 5; bj = ti - 7; }
  else { bi = 3; bj = 0; }
}

// Stored tiles are column-major: element (r, c) at c * TP + r.
// D += A B for two stored 16x16 fp32 tiles (v_mfma_f32_16x16x4_f32: lane l
// gives A[l%16][k] and B[k][l%16] with k = l/16 of the 4-wide step).
__device__ __forceinline__ f32x4 tile_mma(const float* A, const float* B, f32x4 d, int lane) {
  const int n = lane & 15, q = lane >> 4;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const int k = 4 * kb + q;
    d = __builtin_amdgcn_mfma_f32_16x16x4f32(A[k * TP + n], B[n * TP + k], d, 0, 0, 0);
  }
  return d;
}
// Store a D tile (lane holds rows 4q..4q+3 of column n).
__device__ __forceinline__ void tile_st(float* T, f32x4 d, int lane) {
  *reinterpret_cast<f32x4*>(T + (lane & 15) * TP + 4 * (lane >> 4)) = d;
}

// Fragment of a row-major tile read along its rows: lane (n, g) receives
// base[(8g + e) * ld + n], e = 0..7, i.e. the B fragment of a product that
// contracts over the tile's rows (or the A fragment of the transposed tile).
__device__ __forceinline__ bf16x8 ld_tr8(const bf16* base, int ld, int lane) {
  // ds_read_b64_tr_b16: in each 16-lane group, lane m points at 4 elements
  // (row m/4, columns 4(m%4)..+3) of a 4x16 block; lane n then holds column
  // n, rows 0..3.  Two such reads give rows 8g..8g+3 and 8g+4..8g+7.
  const int m = lane & 15, g = lane >> 4;
  const bf16* p0 = base + (8 * g + (m >> 2)) * ld + 4 * (m & 3);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0 + 4 * ld));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}
__device__ __forceinline__ f32x8 ld_tr8(const float* base, int ld, int lane) {
  const int n = lane & 15, g = lane >> 4;
  f32x8 f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = base[(8 * g + e) * ld + n];
  return f;
}

// Coefficient fragments of one k-step: C~ = C diag(beta) (hi + lo halves for
// bf16 operands) and Cb = C diag(beta 2^g), as an MFMA operand (cb) and in the
// stored intermediate type (cbi).
template <typename E> struct CoefFrag { frag_t<E> hi, lo, cb; frag_t<inter_t<E>> cbi; };

template <typename E>
__device__ __forceinline__ CoefFrag<E> coef_frag(const float* sCt, const float* sb, const float* sbe,
                                                 int w, int ks, bool ba, int lane) {
  const int n = lane & 15, g = lane >> 4;
  const int jt = 2 * ks + (g >> 1), co = 8 * (g & 1), s0 = 16 * jt + co;
  const float* T = sCt + slot(w, jt, ba) * TILE + co * TP + n;
  const f32x8 b8 = ld8f(sb + s0), be8 = ld8f(sbe + s0);
  CoefFrag<E> f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float c = T[e * TP];
    const float ct = c * b8[e];
    const E h = from_f<E>(ct);
    f.hi[e] = h;
    f.lo[e] = from_f<E>(ct - to_f(h));
    const float cbv = c * be8[e];
    f.cb[e] = from_f<E>(cbv);
    f.cbi[e] = from_f<inter_t<E>>(cbv);
  }
  return f;
}

// MODE 0: dense (W); 1: sparse (staged Cb and the tail-score parts; W is
// deferred to the kept events); 2: the deferred-W ablation (W of every chunk
// and the tail-score parts).  VARLEN: packed sequences (offsets in p.cu); the
// dense-layout instances have no offset reads at all.
template <typename E, bool BA, int MODE, bool VARLEN>
__global__ __launch_bounds__(256, 2) void intra_kernel(IntraArgs p) {
  using I = inter_t<E>;
  __shared__ __align__(16) E sK[L * KS];      // key tile, row-major [t][dk]
  __shared__ __align__(16) E sV[L * KS];      // value tile of the current head [t][dv]
  __shared__ __align__(16) float sMt[NT * TILE];
  __shared__ __align__(16) float sCt[NT * TILE];
  __shared__ __align__(16) float sYt[4 * TILE];
  __shared__ __align__(32) float sg[2][L], sb[2][L], sbe[2][L];

  // thread index; made opaque again at every item (see the loop head)
  int tid = threadIdx.x;
  const int w_uniform = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int T = p.T, Nq = p.Nq, Nv = p.Nv, C = p.C;
  const int32_t* const cu = VARLEN ? p.cu : nullptr;
  // items are (chunk, head pair); packed sequences enumerate their valid
  // chunks from the chunk table, the dense layout every (b, c)
  const int n_items = VARLEN ? ((const cint32*)p.chunks)[(size_t)p.B * C] * Nq : p.B * C * Nq;
  // item -> (sequence b, chunk c, head pair pq) and the sequence's tokens
  struct Item { int b, c, pq, tok0, len; };
  auto locate = [&](int item) __attribute__((always_inline)) {
    Item x;
    x.pq = item % Nq;
    if constexpr (VARLEN) {
      const int v = ((const cint32*)p.chunks)[__builtin_amdgcn_readfirstlane(item / Nq)];
      x.b = v / C;
      x.c = v - x.b * C;
    } else {
      x.c = (item / Nq) % C;
      x.b = item / (Nq * C);
    }
    const SeqSpan sp = seq_span(cu, x.b, T);
    x.tok0 = sp.tok0;
    x.len = sp.len;
    return x;
  };
  const E* K = static_cast<const E*>(p.k);
  const E* V = static_cast<const E*>(p.v);
  const E* BETA = static_cast<const E*>(p.beta);
  constexpr int NGRAM = BA ? 7 : 10;

  for (int q = tid; q < TILE; q += 256) sCt[ZT * TILE + q] = 0.f;

  // ---- operand registers of the item being staged (loaded one item ahead)
  frag_t<E> kreg[4], v0reg[4], v1reg[4];
  float areg = 0.f, breg = 0.f;
  // Rows past the end of the item's sequence read its last token and are
  // zeroed when staged (a = beta = 0 there, so they neither decay nor write
  // the state).  A chunk wholly past the end of a shorter packed sequence
  // loads nothing (its rows may lie past the end of the arrays).
  auto load_kv = [&](const Item& x, frag_t<E>* kr, frag_t<E>* vr, int hh, bool with_k) {
    if (!VARLEN || x.c * L < x.len) {   // always true for the dense layout
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int q = tid + 256 * it, r = q >> 4, c8 = (q & 15) * 8;
        const size_t tok = (size_t)(x.tok0 + min(x.c * L + r, x.len - 1));
        if (with_k) kr[it] = ld8(K + (tok * Nq + x.pq) * DK + c8);
        vr[it] = ld8(V + (tok * Nv + 2 * x.pq + hh) * DV + c8);
      }
    } else {
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        if (with_k) kr[it] = zero_frag<E>();
        vr[it] = zero_frag<E>();
      }
    }
  };
  auto load_ab = [&](const Item& x) {
    areg = 0.f;
    breg = 0.f;
    if (!VARLEN || x.c * L < x.len) {
      const int hh = (tid >> 6) & 1, t = min(x.c * L + (tid & 63), x.len - 1);
      const size_t idx = (size_t)(x.tok0 + t) * Nv + 2 * x.pq + hh;
      areg = p.a[idx];
      breg = to_f(BETA[idx]);
    }
  };
  // rows past the sequence end are zero
  auto mask_rows = [&](const Item& x, frag_t<E>* r) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int row = (tid + 256 * it) >> 4;
      if (x.c * L + row >= x.len) r[it] = zero_frag<E>();
    }
  };

  int item = blockIdx.x;
  if (item < n_items) {
    const Item x = locate(item);
    load_kv(x, kreg, v0reg, 0, true);
    load_ab(x);
    load_kv(x, kreg, v1reg, 1, false);
  }
  // The first item's operands are complete before the loop: otherwise the
  // wait counts at the loop head, merged over this path (few requests after
  // the gate loads) and the loop's back edge, would make every item wait for
  // the previous item's stores before it reads its prefetched gates.
  __builtin_amdgcn_s_waitcnt(0);

  for (; item < n_items; item += gridDim.x) {
    // wave and thread index as opaque values per item, so that the addresses
    // derived from them are formed where they are used instead of being kept
    // in registers across the whole loop
    int w = w_uniform;
    asm volatile("" : "+s"(w), "+v"(tid));
    const int lane = tid & 63, n16 = lane & 15, g4 = lane >> 4;
    const Item cur = locate(item);
    const Item nxt = locate(min(item + (int)gridDim.x, n_items - 1));
    const int b = cur.b, c = cur.c, pq = cur.pq, len = cur.len;
    lds_barrier();  // the previous item's readers of sK, sV, sg are done

    // ---- stage keys and the first head's values; decay prefix of both heads.
    //      Inputs outside the operator's domain (non-finite k, v, beta; a
    //      non-finite or positive) are flagged for the sequence's statistics.
    mask_rows(cur, kreg);
    mask_rows(cur, v0reg);
    int nfbits = 0;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int q = tid + 256 * it, r = q >> 4, c8 = (q & 15) * 8;
      if (nonfinite8(kreg[it])) nfbits |= NF_K;
      if (nonfinite8(v0reg[it])) nfbits |= NF_V;
      *reinterpret_cast<frag_t<E>*>(&sK[r * KS + c8]) = kreg[it];
      *reinterpret_cast<frag_t<E>*>(&sV[r * KS + c8]) = v0reg[it];
    }
    if (tid < 128) {
      const int hh = tid >> 6, h = 2 * pq + hh;
      const bool live = c * L + lane < len;
      if (live && (nonfinite1(areg) || areg > 0.f)) nfbits |= NF_A;
      if (live && nonfinite1(breg)) nfbits |= NF_BETA;
      float x = live ? areg : 0.f;
      const float bv = live ? breg : 0.f;
      // inclusive prefix over the chunk (g, Sec. 2.1)
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
      }
      sg[hh][lane] = x;
      sb[hh][lane] = bv;
      sbe[hh][lane] = bv * exp2f(x);
      const size_t hc = (size_t)(b * Nv + h) * C + c;
      p.g[hc * L + lane] = x;
      if (lane == 63) p.gamma[hc] = x;
      // row factors 2^(gamma - g_t) of the H scan's K^T X
      p.fac[hc * L + lane] = exp2f(__shfl(x, 63, 64) - x);
    }
    flag_or(p.stats, b, ST_NF_IN, nfbits);
    lds_barrier();
    // next item's keys, first-head values and gates (registers are free now)
    load_kv(nxt, kreg, v0reg, 0, true);
    load_ab(nxt);

    // ---- fragment-major key tile (K^T operand blocks) for the W-operand H
    //      scan (fp32 inputs, and the sparse controls with W of every
    //      chunk); the Cb-operand H scan forms them from the key rows itself
    if constexpr (MODE == 2 || (MODE == 0 && sizeof(E) == 4)) {
      I* kt = static_cast<I*>(p.KT) + ((size_t)(b * Nq + pq) * C + c) * DK * L;
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int mt = 2 * w + mi;
          const frag_t<E> f = ld_tr44(&sK[32 * ks * KS + 16 * mt], KS, lane);
          *reinterpret_cast<frag_t<I>*>(kt + kblk(mt, ks) + 8 * lane) = cvt8<I, E>(f);
        }
    }

#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int h = 2 * pq + hh;
      const size_t hc = (size_t)(b * Nv + h) * C + c;
      // ---- M = beta_t <k_t, k_s> 2^(g_t - g_s), s < t (Eq. (5)), stored
      //      blockwise; the Gram blocks of the pair's keys are recomputed per
      //      head (cheaper than keeping them in registers)
#pragma unroll
      for (int r = 0; r < 3; ++r) {
        const int ti = w + 4 * r;
        if (ti < NGRAM) {
          int bi, bj;
          gram_block(ti, bi, bj);
          f32x4 gram = zero4();
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            const frag_t<E> fa = ld8(&sK[(16 * bi + n16) * KS + 32 * ks + 8 * g4]);
            const frag_t<E> fb = ld8(&sK[(16 * bj + n16) * KS + 32 * ks + 8 * g4]);
            gram = mma(fa, fb, gram);
          }
          const int s = 16 * bj + n16;
          const float gs = sg[hh][s];
          f32x4 m;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int t = 16 * bi + 4 * g4 + j;
            const float v = sb[hh][t] * gram[j] * exp2f(sg[hh][t] - gs);
            m[j] = (s < t) ? v : 0.f;
          }
          tile_st(sMt + slot(bi, bj, false) * TILE, m, lane);
        }
      }
      lds_barrier();
      if (hh == 1) {
        // the first head's products are done: second head's values in, and
        // the next item's second-head values requested
        mask_rows(cur, v1reg);
        uint32_t nfv = 0;
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const int q = tid + 256 * it, r = q >> 4, c8 = (q & 15) * 8;
          nfv |= nonfinite8(v1reg[it]);
          *reinterpret_cast<frag_t<E>*>(&sV[r * KS + c8]) = v1reg[it];
        }
        flag_or(p.stats, b, ST_NF_IN, nfv ? NF_V : 0);
        load_kv(nxt, kreg, v1reg, 1, false);
      }
      // ---- diagonal blocks: C_ii = (I + M_ii)^{-1}, wave w takes block w,
      //      lane j column j, forward substitution (Eq. (8))
      {
        const float* Mw = sMt + slot(w, w, false) * TILE;
        const int j = n16;
        float x[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) x[t] = (t == j) ? 1.f : 0.f;
#pragma unroll
        for (int s = 0; s < 15; ++s) {
          const float* col = Mw + s * TP;  // M[.][s]
#pragma unroll
          for (int t = s + 1; t < 16; ++t) x[t] -= col[t] * x[s];
        }
        if (lane < 16) {
          float* Cw = sCt + slot(w, w, false) * TILE + j * TP;
#pragma unroll
          for (int t = 0; t < 16; t += 4) *reinterpret_cast<f32x4*>(Cw + t) = f32x4{x[t], x[t + 1], x[t + 2], x[t + 3]};
        }
      }
      lds_barrier();
      // ---- first sub-diagonal: C_i,i-1 = -C_ii M_i,i-1 C_i-1,i-1
      //      (block-adjacent: i = 1, 2, 3; exact: i = 1, 3, the 32x32 halves)
      {
        const int i = BA ? w + 1 : 2 * w + 1;
        if (BA ? (w < 3) : (w < 2)) {
          const f32x4 y = tile_mma(sMt + slot(i, i - 1, false) * TILE,
                                   sCt + slot(i - 1, i - 1, false) * TILE, zero4(), lane);
          tile_st(sYt + w * TILE, y, lane);
          const f32x4 z = tile_mma(sCt + slot(i, i, false) * TILE, sYt + w * TILE, zero4(), lane);
          tile_st(sCt + slot(i, i - 1, false) * TILE, -z, lane);
        }
      }
      lds_barrier();
      if constexpr (!BA) {
        // ---- lower-left 32x32 block: Y = M_hl C_lo, then -C_hi Y
        {
          const float* Mt_ = sMt;
          const float* Ct_ = sCt;
          f32x4 y = zero4();
          if (w == 0) {         // Y20 = M20 C00 + M21 C10
            y = tile_mma(Mt_ + slot(2, 0, false) * TILE, Ct_ + slot(0, 0, false) * TILE, y, lane);
            y = tile_mma(Mt_ + slot(2, 1, false) * TILE, Ct_ + slot(1, 0, false) * TILE, y, lane);
          } else if (w == 1) {  // Y30 = M30 C00 + M31 C10
            y = tile_mma(Mt_ + slot(3, 0, false) * TILE, Ct_ + slot(0, 0, false) * TILE, y, lane);
            y = tile_mma(Mt_ + slot(3, 1, false) * TILE, Ct_ + slot(1, 0, false) * TILE, y, lane);
          } else if (w == 2) {  // Y21 = M21 C11
            y = tile_mma(Mt_ + slot(2, 1, false) * TILE, Ct_ + slot(1, 1, false) * TILE, y, lane);
          } else {              // Y31 = M31 C11
            y = tile_mma(Mt_ + slot(3, 1, false) * TILE, Ct_ + slot(1, 1, false) * TILE, y, lane);
          }
          tile_st(sYt + w * TILE, y, lane);
        }
        lds_barrier();
        {
          // Y tiles: 0 = Y20, 1 = Y30, 2 = Y21, 3 = Y31
          f32x4 z = zero4();
          int dst;
          if (w == 0) {         // C20 = -C22 Y20
            z = tile_mma(sCt + slot(2, 2, false) * TILE, sYt + 0 * TILE, z, lane);
            dst = slot(2, 0, false);
          } else if (w == 1) {  // C30 = -(C32 Y20 + C33 Y30)
            z = tile_mma(sCt + slot(3, 2, false) * TILE, sYt + 0 * TILE, z, lane);
            z = tile_mma(sCt + slot(3, 3, false) * TILE, sYt + 1 * TILE, z, lane);
            dst = slot(3, 0, false);
          } else if (w == 2) {  // C21 = -C22 Y21
            z = tile_mma(sCt + slot(2, 2, false) * TILE, sYt + 2 * TILE, z, lane);
            dst = slot(2, 1, false);
          } else {              // C31 = -(C32 Y21 + C33 Y31)
            z = tile_mma(sCt + slot(3, 2, false) * TILE, sYt + 2 * TILE, z, lane);
            z = tile_mma(sCt + slot(3, 3, false) * TILE, sYt + 3 * TILE, z, lane);
            dst = slot(3, 1, false);
          }
          tile_st(sCt + dst * TILE, -z, lane);
        }
        lds_barrier();
      }

      // ---- U = C diag(beta) V for token tile w (Eq. (6)), the tail score,
      //      and Cb = C diag(beta 2^g) (Eq. (7)): W^T = K^T Cb^T (dense) or
      //      Cb itself (sparse, for the deferred W of kept events)
      const int ks_lo = (BA && w == 3) ? 1 : 0;
      const int ks_hi = (w >= 2) ? 1 : 0;
      CoefFrag<E> cf[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if (ks >= ks_lo && ks <= ks_hi) {
          cf[ks] = coef_frag<E>(sCt, sb[hh], sbe[hh], w, ks, BA, lane);
        } else {
          cf[ks].hi = cf[ks].lo = cf[ks].cb = zero_frag<E>();
          cf[ks].cbi = zero_frag<I>();
        }
      }
      {
        // two halves of 64 value columns each, to bound the live fragments
        I* U = static_cast<I*>(p.U) + hc * DV * L;
        float ss = 0.f;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          f32x4 acc[4];
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) acc[nt] = zero4();
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            if (ks >= ks_lo && ks <= ks_hi) {
#pragma unroll
              for (int nt = 0; nt < 4; ++nt) {
                const frag_t<E> fb = ld_tr8(&sV[32 * ks * KS + 16 * (4 * half + nt)], KS, lane);
                acc[nt] = mma(cf[ks].hi, fb, acc[nt]);
                if constexpr (sizeof(E) == 2) acc[nt] = mma(cf[ks].lo, fb, acc[nt]);
              }
            }
          }
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) {
            st4<I>(U + u_elem(16 * (4 * half + nt) + n16, 16 * w + 4 * g4), acc[nt]);
#pragma unroll
            for (int j = 0; j < 4; ++j) ss += acc[nt][j] * acc[nt][j];
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (MODE != 0) {
          // Eq. (9) in parts: sums of squares of U over 8-row blocks, from the
          // fp32 accumulators (lanes 0-31 hold rows 16w..16w+7, lanes 32-63
          // rows 16w+8..16w+15); the tail score sums the blocks of its window
#pragma unroll
          for (int off = 1; off < 32; off <<= 1) ss += __shfl_xor(ss, off, 64);
          if ((lane & 31) == 0) p.score_part[hc * 8 + 2 * w + (lane >> 5)] = ss;
        }
      }
      // keep the U and W products apart (their accumulators would otherwise
      // be live at the same time)
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (MODE != 2 && sizeof(I) == 2) {
        // fragment-major blocks for the H scan (W S = Cb (K S)): lane
        // (n, g) holds sources 8g .. 8g+7, which are positions 4 (g >> 1) ..
        // + 3 of lanes n + 16 (2 (g & 1)) and n + 16 (2 (g & 1) + 1) there
        I* cb = static_cast<I*>(p.Cb) + hc * CB_BLOCKS * 512;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          if (ks >= ks_lo && ks <= ks_hi) {
            I* blk = cb + cb_block(w, ks) * 512 + 4 * (g4 >> 1);
            const int l0 = n16 + 32 * (g4 & 1);
            *reinterpret_cast<half_t<I>*>(blk + 8 * l0) = __builtin_shufflevector(cf[ks].cbi, cf[ks].cbi, 0, 1, 2, 3);
            *reinterpret_cast<half_t<I>*>(blk + 8 * (l0 + 16)) = __builtin_shufflevector(cf[ks].cbi, cf[ks].cbi, 4, 5, 6, 7);
          }
      } else if constexpr (MODE == 1) {
        // only the 32-column blocks the deferred-W stage reads (the others
        // are zero by the causal or block-adjacent structure)
        I* cb = static_cast<I*>(p.Cb) + hc * L * L;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          if (ks >= ks_lo && ks <= ks_hi)
            *reinterpret_cast<frag_t<I>*>(cb + (16 * w + n16) * L + 32 * ks + 8 * g4) = cf[ks].cbi;
      } else {
        // W^T = K^T Cb^T: rows dk, columns t
        I* W = static_cast<I*>(p.W) + hc * L * DK;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          f32x4 acc[4];
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) acc[mt] = zero4();
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            if (ks >= ks_lo && ks <= ks_hi) {
#pragma unroll
              for (int mt = 0; mt < 4; ++mt) {
                const frag_t<E> fa = ld_tr8(&sK[32 * ks * KS + 16 * (4 * half + mt)], KS, lane);
                acc[mt] = mma(fa, cf[ks].cb, acc[mt]);
              }
            }
          }
          // two stacked W^T tiles form one fragment-major W block
#pragma unroll
          for (int qq = 0; qq < 2; ++qq)
            *reinterpret_cast<frag_t<I>*>(W + wblk(2 * half + qq, w) + 8 * lane) =
                pack44<I>(acc[2 * qq], acc[2 * qq + 1]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  }
}

template <typename E, bool BA, int MODE, bool VARLEN>
hipError_t launch_one(const IntraArgs& a, hipStream_t s) {
  const auto fn = intra_kernel<E, BA, MODE, VARLEN>;
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 256, 0);
  if (e != hipSuccess) return e;
  const long long items = (long long)a.B * a.C * a.Nq;
  const long long slots = (long long)cus * (per_cu > 0 ? per_cu : 1);
  const int grid = (int)(items < slots ? items : slots);
  hipLaunchKernelGGL(fn, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

template <typename E, bool BA, int MODE>
hipError_t launch_vl(const IntraArgs& a, hipStream_t s) {
  return a.cu != nullptr ? launch_one<E, BA, MODE, true>(a, s) : launch_one<E, BA, MODE, false>(a, s);
}

template <typename E, bool BA>
hipError_t launch_mode(const IntraArgs& a, hipStream_t s) {
  if (a.score_part == nullptr) return launch_vl<E, BA, 0>(a, s);
  if (a.Cb != nullptr) return launch_vl<E, BA, 1>(a, s);
  // deferred-W ablation: dense layout only
  return a.cu == nullptr ? launch_one<E, BA, 2, false>(a, s) : hipErrorInvalidValue;
}

hipError_t launch_intra(const IntraArgs& a, int bf16, hipStream_t s) {
  const bool ba = a.solve == 1;
  if (bf16) return ba ? launch_mode<sgdn::bf16, true>(a, s) : launch_mode<sgdn::bf16, false>(a, s);
  return ba ? launch_mode<float, true>(a, s) : launch_mode<float, false>(a, s);
}

}  // namespace sgdn
