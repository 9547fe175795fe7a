// Small kernels of the pipeline: log-decay prefix, initial-state transpose,
// gate energy, deferred W of kept events, debug copy of U.
#include "common.h"
#include "kernels.h"

namespace sgdn {

namespace {

// P_0 = 0, P_{c+1} = P_c + gamma_c in fp64 (SparseGDN reading notes,
// Sec. 2.6, Eqs. (19)-(20)).  One wave per (batch, head): each lane sums a
// contiguous run of chunks, then an exclusive wave scan joins the runs.
// Chunks past the end of a shorter packed sequence retain everything
// (gamma = 0 there; their gamma entries are not read).
__device__ __forceinline__ void prefix_body(const PrefixArgs& p, int bh, int lane) {
  const int C = p.C;
  const int Cv = p.cu == nullptr ? C : chunks_of(seq_span(p.cu, bh / p.Nv, p.T).len);
  const float* gm = p.gamma + (size_t)bh * C;
  double* P = p.P + (size_t)bh * (C + 1);
  const int per = (C + 63) / 64;
  const int lo = lane * per, hi = min(C, lo + per);
  auto gam = [&](int c) { return c < Cv ? (double)gm[c] : 0.0; };
  // the run's loads are issued eight at a time; sums keep chunk order
  double run = 0.0;
  for (int c0 = lo; c0 < hi; c0 += 8) {
    double x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = c0 + u < hi ? gam(c0 + u) : 0.0;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (c0 + u < hi) run += x[u];
  }
  double incl = run;
  for (int off = 1; off < 64; off <<= 1) {
    const double y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  double acc = incl - run;
  if (lane == 0) P[0] = 0.0;
  for (int c0 = lo; c0 < hi; c0 += 8) {
    double x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = c0 + u < hi ? gam(c0 + u) : 0.0;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (c0 + u < hi) {
        acc += x[u];
        P[c0 + u + 1] = acc;
      }
  }
}

__global__ __launch_bounds__(64) void prefix_kernel(PrefixArgs p) {
  prefix_body(p, blockIdx.x, threadIdx.x);
}

// Table of the valid chunks of packed sequences (one workgroup): per-thread
// runs of sequences are counted, scanned in LDS, their offsets stored, and
// the entries b C + c then written by all threads, each finding its
// sequence by binary search over the offsets.
__global__ __launch_bounds__(1024) void chunk_table_kernel(ChunkTableArgs p) {
  __shared__ int part[1024];
  const int tid = threadIdx.x, B = p.B;
  const size_t BC = (size_t)B * p.C;
  int32_t* off = p.table + BC + 1;   // [B + 1]
  auto nchunks = [&](int b) {
    const int n = min(max(p.cu[b + 1] - p.cu[b], 0), p.T);
    return chunks_of(n);
  };
  const int per = (B + 1023) / 1024;
  const int lo = min(tid * per, B), hi = min(lo + per, B);
  int sum = 0;
  for (int b = lo; b < hi; ++b) sum += nchunks(b);
  part[tid] = sum;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {
    const int v = tid >= d ? part[tid - d] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int base = part[tid] - sum;
  for (int b = lo; b < hi; ++b) {
    off[b] = base;
    base += nchunks(b);
  }
  const int total = part[1023];
  if (tid == 0) {
    off[B] = total;
    p.table[BC] = total;
  }
  __syncthreads();
  for (int i = tid; i < total; i += 1024) {
    int l = 0, r = B - 1;            // last b with off[b] <= i
    while (l < r) {
      const int m = (l + r + 1) >> 1;
      if (off[m] <= i) l = m; else r = m - 1;
    }
    p.table[i] = l * p.C + (i - off[l]);
  }
}

// s_{c,h} = ||U_{c,h}[64 - tail : 64]||_F (SparseGDN reading notes, Sec. 2.4,
// Eq. (9); Tail-8/32/64 are the window ablations of Fig. 10).
__device__ __forceinline__ void score_body(const ScoreArgs& p, long long i) {
  if (i >= p.n) return;
  const float* q = p.part + i * 8;
  float s = 0.f;
  for (int k = 8 - p.tail / 8; k < 8; ++k) s += q[k];
  p.score[i] = sqrtf(s);
}

__global__ __launch_bounds__(256) void score_kernel(ScoreArgs p) {
  score_body(p, (long long)blockIdx.x * 256 + threadIdx.x);
}

// Compact-states ablation (SparseGDN reading notes, Sec. 3.6, Table 6): the
// entry state of every output group r, S_2r = 2^(P_2r - P_e+1) S_e+1 from the
// snapshot of its predecessor event e (Sec. 2.6, Eq. (21)), or 2^P_2r s0, or
// zero, written densely.  One workgroup per (group, head of a pair in CSR
// rows row_lo .. row_lo + nrows - 1); groups past a packed sequence's end
// are skipped (nothing reads them).
template <typename I>
__global__ __launch_bounds__(256) void expand_kernel(ExpandArgs p) {
  const int r = blockIdx.x, y = blockIdx.y, NP = p.Nv / 2;
  const int hh = y & 1, row = p.row_lo + (y >> 1) % p.nrows, b = (y >> 1) / p.nrows;
  const int pr = p.row_pair[b * NP + row], h = 2 * pr + hh, bh = b * p.Nv + h;
  if (p.cu != nullptr && 2 * r * L >= seq_span(p.cu, b, p.T).len) return;
  const size_t pg = ((size_t)b * (p.Nv / 2) + pr) * p.G + r;
  const int slot = p.group_slot[pg];
  const double* P = p.P + (size_t)bh * (p.C + 1);
  const I* src = nullptr;
  float f = 0.f;
  if (slot >= 0) {
    src = static_cast<const I*>(p.snap) + (((size_t)b * p.snap_cap + slot) * 2 + hh) * DV * DK;
    f = exp2f((float)(P[2 * r] - P[p.pred[pg] + 1]));
  } else if (p.s0T != nullptr) {
    src = static_cast<const I*>(p.s0T) + (size_t)bh * DV * DK;
    f = exp2f((float)P[2 * r]);
  }
  I* dst = static_cast<I*>(p.entry) + ((size_t)bh * p.G + r) * DV * DK;
  for (int i = threadIdx.x * 8; i < DV * DK; i += 256 * 8) {
    frag_t<I> y;
    if (src != nullptr) {
      const frag_t<I> x = *reinterpret_cast<const frag_t<I>*>(src + i);
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = from_f<I>(f * to_f(x[j]));
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = from_f<I>(0.f);
    }
    *reinterpret_cast<frag_t<I>*>(dst + i) = y;
  }
}

// s0 [dk][dv] -> transposed [dv][dk] in the snapshot element type and
// layout (s_elem), the "virtual snapshot" that output groups without a
// predecessor read.
template <typename I>
__global__ __launch_bounds__(256) void s0prep_kernel(S0PrepArgs p) {
  const size_t bh = blockIdx.x;
  const float* s = p.s0 + bh * DK * DV;
  I* o = static_cast<I*>(p.s0T) + bh * DV * DK;
  uint32_t bad = 0;
  for (int q = threadIdx.x; q < DK * DV; q += 256) {
    const int dv = q >> 7, dk = q & 127;
    const float x = s[dk * DV + dv];
    bad |= nonfinite1(x);
    o[s_elem(dv, dk)] = from_f<I>(x);
  }
  flag_or(p.stats, (int)(bh / p.Nv), ST_NF_IN, bad ? NF_S0 : 0);
}

// Statistics at the start of a prefill call (one thread per sequence).
__global__ __launch_bounds__(256) void stats_init_kernel(StatsInitArgs p) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= p.B) return;
  int32_t* st = p.stats + (size_t)b * STATS_INTS;
  if (p.dense) {
    const int NP = p.Nv / 2;
    const int Cb = p.cu == nullptr ? p.C : chunks_of(seq_span(p.cu, b, p.T).len);
    const int Gb = (Cb + 1) / 2;
    st[0] = NP * Cb;
    st[1] = NP * p.C;
    for (int i = 2; i < 8; ++i) st[i] = 0;
    st[8] = p.Nv * (Gb > 1 ? Gb - 1 : 0);
  }
  st[ST_NF_IN] = 0;
  st[ST_NF_OUT] = 0;
}

// eta_h = mean over the 4C samples of (w_v SiLU(z[64c + 8 + 16a, h, v]))^2,
// v = 73 (4c + a) mod 128 (SparseGDN reading notes, Sec. 2.4, Eq. (11)), C the
// sequence's own (valid) chunks; 0 for an empty sequence.  Workgroup
// (h, b, z) sums the squares of the samples in batches z, z + GATE_SPLIT, ...
// of 1024 (one sample per thread and batch): spread over many CUs, the
// scattered sample reads are not held up by one CU's outstanding misses.
constexpr int GATE_THREADS = 1024;
template <typename E>
__device__ __forceinline__ void gate_body(const GateArgs& p, int h, int b, int zb, int tid) {
  const E* z = static_cast<const E*>(p.z);
  const SeqSpan sp = seq_span(p.cu, b, p.T);
  const int ns = 4 * chunks_of(sp.len);
  float acc = 0.f;
  uint32_t bad = 0;
  for (int j = zb * GATE_THREADS + tid; j < ns; j += GATE_SPLIT * GATE_THREADS) {
    const int c = j >> 2, a = j & 3;
    const int pos = c * L + 8 + 16 * a;
    const int v = (73 * j) & (DV - 1);
    if (pos < sp.len) {
      const float x = to_f(z[((size_t)(sp.tok0 + pos) * p.Nv + h) * DV + v]);
      bad |= nonfinite1(x);
      const float s = (p.w ? p.w[v] : 1.f) * (x / (1.f + __expf(-x)));
      acc += s * s;
    }
  }
  flag_or(p.stats, b, ST_NF_IN, bad ? NF_Z : 0);
  constexpr int NWV = GATE_THREADS / 64;
  __shared__ float red[NWV];
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if ((tid & 63) == 0) red[tid >> 6] = acc;
  __syncthreads();
  if (tid == 0) {
    float t = 0.f;
    for (int i = 0; i < NWV; ++i) t += red[i];
    p.eta_part[((size_t)b * p.Nv + h) * GATE_SPLIT + zb] = t;
  }
}

template <typename E>
__global__ __launch_bounds__(GATE_THREADS) void gate_kernel(GateArgs p) {
  gate_body<E>(p, blockIdx.x, blockIdx.y, blockIdx.z, threadIdx.x);
}

// The gate energies, the prefix and the tail scores in one launch (each reads
// only the inputs and what the intra kernel left; two dependent launches
// fewer): workgroups 0 .. ng - 1 are gate_kernel's (h, b, z) in that order,
// the next np one prefix wave each (batch-major heads; the other waves leave:
// a head's strided loads and stores want a CU's address unit of their own,
// as in prefix_kernel), the rest 1024 scores each.
template <typename E>
__global__ __launch_bounds__(GATE_THREADS) void prep_kernel(PrefixArgs pa, GateArgs ga, ScoreArgs sc,
                                                            int ng, int np) {
  const int id = blockIdx.x, tid = threadIdx.x;
  if (id < ng) {
    gate_body<E>(ga, id % ga.Nv, (id / ga.Nv) % ga.B, id / (ga.Nv * ga.B), tid);
  } else if (id < ng + np) {
    if (tid < 64) prefix_body(pa, id - ng, tid);
  } else {
    score_body(sc, (long long)(id - ng - np) * GATE_THREADS + tid);
  }
}

// Deferred W of kept events only (SparseGDN reading notes, Sec. 2.5,
// Eq. (15)), fp32 intermediates.  The event's key rows are staged in LDS
// (zero past the end of the sequence) and turned into the fragment-major K^T
// blocks the W-operand H scan reads, and W = Cb K is formed as W^T = K^T Cb^T
// and stored as fragment-major W tiles, both per event (both heads of the
// pair): only kept chunks get them.  (With fp16 intermediates the H scan
// forms W S = Cb (K S) from the staged Cb and the key rows itself, and the
// kept events need only their records.)
// Each workgroup walks events blockIdx.x, blockIdx.x + gridDim.x, ... of the
// CSR rows row_lo .. row_hi - 1 (the count is on the device; the grid is
// sized by the host and does not depend on it).
constexpr int DW_KS = DK + 8;   // row stride (elements) of the staged key rows
constexpr int DW_BLOCKS = 2048; // workgroups per sequence

template <typename E>
__device__ __forceinline__ void deferred_w_body(const DeferredWArgs& p, int bx, int nbx, int b) {
  using I = inter_t<E>;
  __shared__ __align__(16) E sK[L * DW_KS];
  __shared__ int s_ptr[17];
  const int NP = p.Nv / 2;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int n16 = lane & 15, g4 = lane >> 4;
  if (tid <= NP) s_ptr[tid] = p.row_ptr[b * (NP + 1) + tid];
  __syncthreads();
  const bool blockadj = p.solve == 1;
  const SeqSpan sp = seq_span(p.cu, b, p.T);
  const E* K = static_cast<const E*>(p.k);
  int row = p.row_lo;
  for (int i = s_ptr[p.row_lo] + bx; i < s_ptr[p.row_hi]; i += nbx) {
    while (row + 1 < p.row_hi && s_ptr[row + 1] <= i) ++row;
    const int pr = p.row_pair[b * NP + row];
    const int c = p.col[(size_t)b * p.Emax + i];
    {
      // key rows c*64 .. c*64+63 in 16-byte pieces
      constexpr int PV = 16 / (int)sizeof(E), PR = DK / PV;
#pragma unroll
      for (int it = 0; it < L * PR / 256; ++it) {
        const int q = tid + 256 * it;
        const int t = q / PR, e0 = (q % PR) * PV, tok = c * L + t;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (tok < sp.len) v = *reinterpret_cast<const uint4*>(K + ((size_t)(sp.tok0 + tok) * p.Nq + pr) * DK + e0);
        *reinterpret_cast<uint4*>(&sK[t * DW_KS + e0]) = v;
      }
    }
    __syncthreads();
    // K^T blocks of the event: wave w forms key tiles 2w and 2w+1
    I* KT = static_cast<I*>(p.KTpk) + ((size_t)b * p.Emax + i) * DK * L;
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int mt = 2 * w + mi;
        *reinterpret_cast<frag_t<I>*>(KT + kblk(mt, ks) + 8 * lane) =
            cvt8<I, E>(ld_tr44(&sK[32 * ks * DW_KS + 16 * mt], DW_KS, lane));
      }
    if (p.Wpk != nullptr) {
      const int ks_lo = (blockadj && w == 3) ? 1 : 0;
      const int ks_hi = (w >= 2) ? 1 : 0;
      for (int hh = 0; hh < 2; ++hh) {
        const int h = 2 * pr + hh;
        const I* Cb = static_cast<const I*>(p.Cb) + (((size_t)b * p.Nv + h) * p.C + c) * L * L;
        // W^T = K^T Cb^T (rows dk, columns t).  K^T blocks are fragment-major in
        // the permuted token order, so Cb is read in the same order.
        f32x4 acc[8];
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) acc[mt] = zero4();
        for (int ks = ks_lo; ks <= ks_hi; ++ks) {
          const I* cr = Cb + (16 * w + n16) * L + 32 * ks + 4 * g4;
          const frag_t<I> fb = ld44(cr, cr + 16);
#pragma unroll
          for (int mt = 0; mt < 8; ++mt)
            acc[mt] = mma(cvt8<I, E>(ld_tr44(&sK[32 * ks * DW_KS + 16 * mt], DW_KS, lane)), fb, acc[mt]);
        }
        // two stacked W^T tiles form one fragment-major W block
        I* W = static_cast<I*>(p.Wpk) + (((size_t)b * p.Emax + i) * 2 + hh) * L * DK;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<frag_t<I>*>(W + wblk(q, w) + 8 * lane) = pack44<I>(acc[2 * q], acc[2 * q + 1]);
      }
    }
    __syncthreads();   // the next event rewrites sK
  }
}

// Event records of the H scan (SparseGDN reading notes, Sec. 2.1 Eq. (2) and
// Sec. 2.6 Eq. (21)).  Dense: every chunk is an event, F_in = 1, and the state
// after odd chunk c (c + 1 < C) is the snapshot (c + 1) / 2 - 1 of the group
// that starts at chunk c + 1.  Sparse: one record per kept event and head of
// the pair; F_in = 2^(P_c - P_{e+1}) joins the previous kept event e of the
// row (1 for the first event, whose gap the initial state already carries).
__global__ __launch_bounds__(256) void evrec_dense_kernel(EvRecArgs p) {
  const size_t n = (size_t)p.B * p.Nv * p.C;
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int c = (int)(i % p.C);
  int4 r;
  r.x = __float_as_int(1.f);
  r.y = __float_as_int(exp2f(p.gamma[i]));
  r.z = ((c & 1) && c + 1 < p.C) ? (c + 1) / 2 - 1 : -1;
  r.w = c;
  reinterpret_cast<int4*>(p.rec)[i] = r;
}

__device__ __forceinline__ void evrec_sparse_body(const EvRecArgs& p, int row, int b, int tid, int nthr) {
  const int NP = p.Nv / 2;
  const int beg = p.row_ptr[b * (NP + 1) + row], end = p.row_ptr[b * (NP + 1) + row + 1];
  const int pr = p.row_pair[b * NP + row];
  const int32_t* col = p.col + (size_t)b * p.Emax;
  for (int i = beg + tid; i < end; i += nthr) {
    const int c = col[i];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const size_t bh = (size_t)b * p.Nv + 2 * pr + hh;
      const double* P = p.P + bh * (p.C + 1);
      const float fin = (i > beg) ? exp2f((float)(P[c] - P[col[i - 1] + 1])) : 1.f;
      int4 r;
      r.x = __float_as_int(fin);
      r.y = __float_as_int(exp2f(p.gamma[bh * p.C + c]) * fin);
      r.z = p.event_slot[(size_t)b * p.Emax + i];
      r.w = c;
      reinterpret_cast<int4*>(p.rec)[((size_t)b * p.Emax + i) * 2 + hh] = r;
    }
  }
}

__global__ __launch_bounds__(1024) void evrec_sparse_kernel(EvRecArgs p) {
  evrec_sparse_body(p, p.row_lo + (int)blockIdx.x, blockIdx.y, threadIdx.x, 1024);
}

// Deferred W and the event records of the same rows in one launch (both read
// only the CSR layout and the prefix; one dependent launch fewer):
// workgroups 0 .. nd - 1 walk the kept events (deferred_w_body), the rest
// write the records of one row each.
template <typename E>
__global__ __launch_bounds__(256) void events_kernel(DeferredWArgs da, EvRecArgs ea, int nd) {
  if ((int)blockIdx.x < nd)
    deferred_w_body<E>(da, blockIdx.x, nd, blockIdx.y);
  else
    evrec_sparse_body(ea, ea.row_lo + (int)blockIdx.x - nd, blockIdx.y, threadIdx.x, 256);
}

// CSR-off control (SparseGDN reading notes, Sec. 3.6, Table 6): the H scan
// steps through every chunk of a row with the same mask and decay arithmetic.
// A kept chunk's record is the CSR one (gap factor from the previous kept
// chunk, or from the start of the sequence, whose decay the event-list scan
// then carries instead of the initial state); a chunk outside the mask is a
// null event.  One workgroup per (row, sequence); chunks in tiles of 1024
// with block scans for the kept count and the last kept chunk.
__global__ __launch_bounds__(1024) void evrec_all_kernel(EvAllArgs p) {
  __shared__ int s_cnt[1024], s_last[1024];
  const int row = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int NP = p.Nv / 2, C = p.C;
  const int pr = p.row_pair[b * NP + row];
  const int beg = p.row_ptr[b * (NP + 1) + row];
  const uint8_t* m = p.mask + ((size_t)b * NP + pr) * C;
  const size_t ebase = ((size_t)b * NP + row) * C;   // event index of chunk 0 of this row
  if (tid == 0) {
    p.row_ptr_all[b * (NP + 1) + row] = row * C;
    if (row == NP - 1) p.row_ptr_all[b * (NP + 1) + NP] = NP * C;
  }
  int carry_cnt = 0, carry_last = -1;
  for (int c0 = 0; c0 < C; c0 += 1024) {
    const int c = c0 + tid;
    const int kept = (c < C && m[c]) ? 1 : 0;
    s_cnt[tid] = kept;
    s_last[tid] = kept ? c : -1;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {
      const int a = tid >= d ? s_cnt[tid - d] : 0;
      const int l = tid >= d ? s_last[tid - d] : -1;
      __syncthreads();
      s_cnt[tid] += a;
      s_last[tid] = max(s_last[tid], l);
      __syncthreads();
    }
    const int cnt = carry_cnt + s_cnt[tid];                      // kept in [0, c]
    const int prev = max(carry_last, tid > 0 ? s_last[tid - 1] : -1);   // last kept before c
    if (c < C) {
      const size_t j = ebase + c;
      p.col_all[j] = c;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const size_t bh = (size_t)b * p.Nv + 2 * pr + hh;
        int4 r;
        if (kept) {
          const double* P = p.P + bh * (C + 1);
          const float fin = exp2f((float)(P[c] - P[prev + 1]));
          r.x = __float_as_int(fin);
          r.y = __float_as_int(exp2f(p.gamma[bh * C + c]) * fin);
          r.z = p.event_slot[(size_t)b * p.Emax + beg + cnt - 1];
        } else {
          r.x = __float_as_int(1.f);
          r.y = __float_as_int(1.f);
          r.z = NULL_EVENT;
        }
        r.w = c;
        reinterpret_cast<int4*>(p.rec)[j * 2 + hh] = r;
      }
    }
    const int tile_cnt = s_cnt[1023], tile_last = s_last[1023];
    __syncthreads();
    carry_cnt += tile_cnt;
    carry_last = max(carry_last, tile_last);
  }
}

// U tiles (intermediate type, token-tile-major, see u_elem) -> token-major
// fp32 [t][dv] copy for the debug output.
template <typename I>
__global__ __launch_bounds__(256) void debug_u_kernel(const void* Ut_, float* U) {
  const I* Ut = static_cast<const I*>(Ut_);
  const size_t tile = blockIdx.x;
  for (int q = threadIdx.x; q < L * DV; q += 256) {
    const int t = q >> 7, dv = q & 127;
    U[tile * L * DV + q] = to_f(Ut[tile * DV * L + u_elem(dv, t)]);
  }
}

}  // namespace

hipError_t launch_stats_init(const StatsInitArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(stats_init_kernel, dim3((a.B + 255) / 256), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_prefix(const PrefixArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(prefix_kernel, dim3(a.B * a.Nv), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_expand(const ExpandArgs& a, int bf16, hipStream_t s) {
  const dim3 grid(a.G, a.B * a.nrows * 2);
  if (bf16)
    hipLaunchKernelGGL(expand_kernel<fp16>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(expand_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_score(const ScoreArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(score_kernel, dim3((unsigned)((a.n + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_chunk_table(const ChunkTableArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(1024), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_evrec(const EvRecArgs& a, hipStream_t s) {
  if (a.sparse) {
    hipLaunchKernelGGL(evrec_sparse_kernel, dim3(a.row_hi - a.row_lo, a.B), dim3(1024), 0, s, a);
  } else {
    const size_t n = (size_t)a.B * a.Nv * a.C;
    hipLaunchKernelGGL(evrec_dense_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_evrec_all(const EvAllArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(evrec_all_kernel, dim3(a.Nv / 2, a.B), dim3(1024), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_s0prep(const S0PrepArgs& a, int bf16, hipStream_t s) {
  if (bf16)
    hipLaunchKernelGGL(s0prep_kernel<fp16>, dim3(a.B * a.Nv), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(s0prep_kernel<float>, dim3(a.B * a.Nv), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gate(const GateArgs& a, int bf16, hipStream_t s) {
  if (bf16)
    hipLaunchKernelGGL(gate_kernel<sgdn::bf16>, dim3(a.Nv, a.B, GATE_SPLIT), dim3(GATE_THREADS), 0, s, a);
  else
    hipLaunchKernelGGL(gate_kernel<float>, dim3(a.Nv, a.B, GATE_SPLIT), dim3(GATE_THREADS), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_prep(const PrefixArgs& pa, const GateArgs* ga, const ScoreArgs& sc, int bf16,
                       hipStream_t s) {
  const int ng = ga != nullptr ? ga->Nv * ga->B * GATE_SPLIT : 0;
  const int np = pa.B * pa.Nv;
  const int ns = (int)((sc.n + GATE_THREADS - 1) / GATE_THREADS);
  const GateArgs g = ga != nullptr ? *ga : GateArgs{};
  const dim3 grid(ng + np + ns);
  if (bf16)
    hipLaunchKernelGGL(prep_kernel<sgdn::bf16>, grid, dim3(GATE_THREADS), 0, s, pa, g, sc, ng, np);
  else
    hipLaunchKernelGGL(prep_kernel<float>, grid, dim3(GATE_THREADS), 0, s, pa, g, sc, ng, np);
  return hipGetLastError();
}

hipError_t launch_events(const DeferredWArgs& da, const EvRecArgs& ea, hipStream_t s) {
  const int nd = da.Emax < DW_BLOCKS ? da.Emax : DW_BLOCKS;
  const dim3 grid(nd + (ea.row_hi - ea.row_lo), da.B);
  hipLaunchKernelGGL(events_kernel<float>, grid, dim3(256), 0, s, da, ea, nd);
  return hipGetLastError();
}

hipError_t launch_debug_u(const void* Ut, float* U, int B, int Nv, int C, int bf16, hipStream_t s) {
  if (bf16)
    hipLaunchKernelGGL(debug_u_kernel<fp16>, dim3(B * Nv * C), dim3(256), 0, s, Ut, U);
  else
    hipLaunchKernelGGL(debug_u_kernel<float>, dim3(B * Nv * C), dim3(256), 0, s, Ut, U);
  return hipGetLastError();
}

}  // namespace sgdn
