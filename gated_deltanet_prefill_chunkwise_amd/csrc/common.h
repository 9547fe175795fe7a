// Shared device helpers for the gfx950 kernels: element types, MFMA
// fragments and their loads/stores.
//
// Matrix-core convention (v_mfma_f32_16x16x32_bf16, 64-lane wavefront):
//   lane l, n = l % 16, g = l / 16
//   A fragment (16 x 32, row-major M x K): row n,    k = 8g .. 8g+7
//   B fragment (32 x 16, K x N):           column n, k = 8g .. 8g+7
//   C/D tile   (16 x 16):                  column n, rows 4g .. 4g+3
// The fp32 path keeps the same 8-values-per-lane fragments and issues eight
// v_mfma_f32_16x16x4_f32: product i takes value i of every lane, i.e. the
// k-slots {i, 8+i, 16+i, 24+i}; together the eight cover all 32 slots once.
//
// "Permuted" fragments: two D tiles stacked along the reduction index (rows
// r0..r0+15 and r0+16..r0+31) already hold, per lane, the 8 values
// {r0+4g..r0+4g+3, r0+16+4g..r0+16+4g+3}.  Used as a B (or A) fragment, slot
// 8g+j stands for row r0+4g+j (j<4) or r0+16+4g+j-4 (j>=4); the other operand
// is then loaded with the same order (two 4-element runs), so a product's
// result feeds the next product without leaving the registers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sgdn {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 fp16;
typedef fp16 fp16x8 __attribute__((ext_vector_type(8)));
typedef fp16 fp16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

constexpr int L = 64;      // chunk length
constexpr int DK = 128;    // key dimension
constexpr int DV = 128;    // value dimension
// U (overwritten in place by U') of one (chunk, head) in global memory: four
// 16-token tiles, each [128 dv][16 t], so that one 16x16 tile of U a wave
// writes, and 16 value rows of one token tile, are 512 contiguous bytes
// (whole lines) in the intermediate type.
__host__ __device__ constexpr int u_elem(int dv, int t) { return (t >> 4) * (DV * 16) + dv * 16 + (t & 15); }
// A state snapshot S^T [dv][dk] (group entry states, the prepared s0) in
// global memory: four 32-key tiles, each [128 dv][32 dk], so that the
// 16-row fragment loads of O and the 4-row copies of the H scan's storer are
// whole 128-byte lines.
__host__ __device__ constexpr int s_elem(int dv, int dk) { return (dk >> 5) * (DV * 32) + dv * 32 + (dk & 31); }

template <typename E> struct FragOf;
template <> struct FragOf<bf16> { using T = bf16x8; using H = bf16x4; };
template <> struct FragOf<fp16> { using T = fp16x8; using H = fp16x4; };
template <> struct FragOf<float> { using T = f32x8; using H = f32x4; };
template <typename E> using frag_t = typename FragOf<E>::T;
template <typename E> using half_t = typename FragOf<E>::H;

// Element type of the stage-to-stage intermediates (U, U', W, K^T, Cb,
// snapshots and the in-LDS state / X operands): fp16 when the inputs are
// bf16 (11-bit significands, so the stored intermediates add about an eighth
// of a bf16 rounding), fp32 when the inputs are fp32.
template <typename E> struct InterOf;
template <> struct InterOf<bf16> { using T = fp16; };
template <> struct InterOf<float> { using T = float; };
template <typename E> using inter_t = typename InterOf<E>::T;

__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f(fp16 x) { return (float)x; }
__device__ __forceinline__ float to_f(float x) { return x; }
template <typename E> __device__ __forceinline__ E from_f(float x);
template <> __device__ __forceinline__ bf16 from_f<bf16>(float x) { return (bf16)x; }
template <> __device__ __forceinline__ fp16 from_f<fp16>(float x) { return (fp16)x; }
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }

// Convert a fragment between element types (elementwise, round to nearest).
template <typename D, typename S> __device__ __forceinline__ frag_t<D> cvt8(const frag_t<S>& x) {
  frag_t<D> y;
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = from_f<D>(to_f(x[i]));
  return y;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ f32x4 mma(const bf16x8& a, const bf16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(const fp16x8& a, const fp16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(const f32x8& a, const f32x8& b, f32x4 c) {
#pragma unroll
  for (int i = 0; i < 8; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], c, 0, 0, 0);
  return c;
}

// 8 consecutive elements (16 B for bf16, 32 B for fp32; aligned).
template <typename E> __device__ __forceinline__ frag_t<E> ld8(const E* p) {
  return *reinterpret_cast<const frag_t<E>*>(p);
}
// 4 consecutive elements from p0 followed by 4 from p1 (permuted fragment).
template <typename E> __device__ __forceinline__ frag_t<E> ld44(const E* p0, const E* p1) {
  half_t<E> lo = *reinterpret_cast<const half_t<E>*>(p0);
  half_t<E> hi = *reinterpret_cast<const half_t<E>*>(p1);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
// 4 consecutive elements as fp32.
template <typename E> __device__ __forceinline__ f32x4 ld4f(const E* p) {
  half_t<E> h = *reinterpret_cast<const half_t<E>*>(p);
  return f32x4{to_f(h[0]), to_f(h[1]), to_f(h[2]), to_f(h[3])};
}
template <typename E> __device__ __forceinline__ void st4(E* p, f32x4 v) {
  half_t<E> h;
  h[0] = from_f<E>(v[0]); h[1] = from_f<E>(v[1]);
  h[2] = from_f<E>(v[2]); h[3] = from_f<E>(v[3]);
  *reinterpret_cast<half_t<E>*>(p) = h;
}
// Two stacked D tiles -> one permuted fragment.
template <typename E> __device__ __forceinline__ frag_t<E> pack44(f32x4 a, f32x4 b) {
  frag_t<E> f;
  f[0] = from_f<E>(a[0]); f[1] = from_f<E>(a[1]); f[2] = from_f<E>(a[2]); f[3] = from_f<E>(a[3]);
  f[4] = from_f<E>(b[0]); f[5] = from_f<E>(b[1]); f[6] = from_f<E>(b[2]); f[7] = from_f<E>(b[3]);
  return f;
}
// Staged Cb of the sparse path with fp16 intermediates: per (chunk, head) six
// fragment-major blocks of 512 elements, block cb_block(i, ks) the MFMA A
// operand of token tile i over source tokens 32 ks .. 32 ks + 31 (lane
// (n, g): row 16 i + n, sources in the permuted order 4g + e, 16 + 4g + e - 4).
// Blocks (0,1) and (1,1) are zero by causality and not stored; (3,0) is zero
// with the block-adjacent solve and not written then.
constexpr int CB_BLOCKS = 6;
// Position of lane l's 16-byte unit inside a K^T block of the sparse path
// with fp16 intermediates: unit n + 16 g is stored at 16 g + (n ^ 4 g), so
// that the transposed reads of four consecutive tokens of one key by lanes
// with different g fall into different LDS banks (a permutation: the plain
// per-lane reads stay conflict-free).
__device__ __forceinline__ int kswz(int l) { return (l & 48) | ((l & 15) ^ ((l >> 2) & 12)); }
__host__ __device__ constexpr int cb_block(int i, int ks) { return i < 2 ? i : 2 * i - 2 + ks; }

// Fragment of a row-major LDS tile read along its rows, in the permuted
// reduction order of the fragment-major tiles: lane (n, g) receives rows
// 4g .. 4g+3 and 16+4g .. 16+4g+3 of column n (the A fragment of the
// transposed tile).  bf16: ds_read_b64_tr_b16, where in each 16-lane group
// lane m points at 4 elements (row m/4, columns 4(m%4)..+3) of a 4x16 block
// and lane n then holds column n, rows 0..3.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
__device__ __forceinline__ bf16x8 ld_tr44(const bf16* base, int ld, int lane) {
  const int m = lane & 15, g = lane >> 4;
  const bf16* p0 = base + (4 * g + (m >> 2)) * ld + 4 * (m & 3);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0 + 16 * ld));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}
__device__ __forceinline__ f32x8 ld_tr44(const float* base, int ld, int lane) {
  const int n = lane & 15, g = lane >> 4;
  f32x8 f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = base[((e < 4) ? 4 * g + e : 16 + 4 * g + e - 4) * ld + n];
  return f;
}

template <typename E> __device__ __forceinline__ frag_t<E> zero_frag() {
  frag_t<E> f;
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = from_f<E>(0.f);
  return f;
}

// fp32 -> bf16 hi/lo split: x ~= hi + lo with |x - hi - lo| <= 2^-16 |x|.
// Products with an fp32 operand use both halves (two or three MFMAs), so the
// fp32-grade intermediates keep fp32 accuracy on the bf16 matrix cores.
__device__ __forceinline__ void split8(const f32x8& x, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    hi[i] = (bf16)x[i];
    lo[i] = (bf16)(x[i] - (float)hi[i]);
  }
}
__device__ __forceinline__ f32x8 ld8f(const float* p) { return *reinterpret_cast<const f32x8*>(p); }
__device__ __forceinline__ f32x8 cat44(f32x4 a, f32x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ void st4f(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }

// Accumulate a (fp32 values) x b into acc: one product for fp32 operands, two
// (hi, lo) for bf16 operands.
__device__ __forceinline__ f32x4 mma_split_a(const f32x8& a, const bf16x8& b, f32x4 acc) {
  bf16x8 hi, lo;
  split8(a, hi, lo);
  acc = mma(hi, b, acc);
  return mma(lo, b, acc);
}
__device__ __forceinline__ f32x4 mma_split_a(const f32x8& a, const f32x8& b, f32x4 acc) {
  return mma(a, b, acc);
}
__device__ __forceinline__ f32x4 mma_split_b(const bf16x8& a, const f32x8& b, f32x4 acc) {
  bf16x8 hi, lo;
  split8(b, hi, lo);
  acc = mma(a, hi, acc);
  return mma(a, lo, acc);
}
__device__ __forceinline__ f32x4 mma_split_b(const f32x8& a, const f32x8& b, f32x4 acc) {
  return mma(a, b, acc);
}

// Fragment-major chunk tiles (W, KT): 16 blocks of 512 elements, one MFMA
// operand fragment per block, lane-major; see the workspace notes.
constexpr int FRAG = 512;
__device__ __forceinline__ int wblk(int q, int i) { return (q * 4 + i) * FRAG; }
__device__ __forceinline__ int kblk(int mt, int ks) { return (mt * 2 + ks) * FRAG; }

// Output element type (o may be fp32, bf16 or fp16 independently of the
// inputs; the narrow types round to nearest even).
template <typename O> __device__ __forceinline__ void st4o(O* p, f32x4 v);
template <> __device__ __forceinline__ void st4o<float>(float* p, f32x4 v) { st4f(p, v); }
template <> __device__ __forceinline__ void st4o<bf16>(bf16* p, f32x4 v) { st4<bf16>(p, v); }
template <> __device__ __forceinline__ void st4o<fp16>(fp16* p, f32x4 v) { st4<fp16>(p, v); }

// Streaming variants for data that is read or written exactly once (the
// output rows; U' and the state snapshots read by O): non-temporal, so that
// they do not displace lines other workgroups still read from L2.
template <typename E> __device__ __forceinline__ frag_t<E> ld8nt(const E* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const frag_t<E>*>(p));
}
template <typename O> __device__ __forceinline__ void st4o_nt(O* p, f32x4 v) {
  half_t<O> h;
  h[0] = from_f<O>(v[0]); h[1] = from_f<O>(v[1]);
  h[2] = from_f<O>(v[2]); h[3] = from_f<O>(v[3]);
  __builtin_nontemporal_store(h, reinterpret_cast<half_t<O>*>(p));
}
template <> __device__ __forceinline__ void st4o_nt<float>(float* p, f32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
}

// 16-byte vector copy helpers (global <-> LDS staging).
struct alignas(16) V16 { uint32_t w[4]; };
__device__ __forceinline__ V16 ldv(const void* p) { return *reinterpret_cast<const V16*>(p); }
__device__ __forceinline__ void stv(void* p, const V16& v) { *reinterpret_cast<V16*>(p) = v; }
__device__ __forceinline__ V16 zv() { V16 v; v.w[0] = v.w[1] = v.w[2] = v.w[3] = 0u; return v; }

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Workgroup barrier that orders LDS only.  __syncthreads() also releases
// global memory, which on gfx9 waits for every outstanding vector-memory
// operation (loads included), draining software-prefetched loads; kernels
// whose global writes are not read back by other waves in the same launch use
// this instead.
// The explicit wait for this wave's outstanding LDS operations does not rely
// on the fence's lowering, which can omit it for a barrier at a loop header.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt, expcnt unconstrained
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Tokens of sequence b.  Packed variable-length batches give offsets cu
// [B + 1] (sequence b is tokens cu[b] .. cu[b+1] - 1, its length clamped to
// [0, T]); without them sequence b is tokens b T .. b T + T - 1.  The offsets
// are read through the scalar cache (they are written before the launch), so
// reading them adds no wait on the vector memory counter.
typedef const __attribute__((address_space(4))) int32_t cint32;   // scalar-cache reads

struct SeqSpan { int tok0, len; };
__device__ __forceinline__ SeqSpan seq_span(const int32_t* cu, int b, int T) {
  if (cu == nullptr) return SeqSpan{b * T, T};
  const int bb = __builtin_amdgcn_readfirstlane(b);
  const cint32* c = (const cint32*)cu;
  const int s = c[bb], e = c[bb + 1];
  return SeqSpan{s, min(max(e - s, 0), T)};
}
__device__ __forceinline__ int chunks_of(int len) { return (len + L - 1) / L; }

// sgdn_stats as int32 words per sequence: E, E_max, n_tier[3], k[3],
// n_snapshots, nonfinite_input, nonfinite_output.
constexpr int STATS_INTS = 11;
constexpr int ST_NF_IN = 9, ST_NF_OUT = 10;
// nonfinite_input / nonfinite_output bits (the SGDN_NF_* values)
constexpr int NF_Q = 1, NF_K = 2, NF_V = 4, NF_A = 8, NF_BETA = 16, NF_Z = 32, NF_S0 = 64;
constexpr int NF_O = 1, NF_SFINAL = 2;

// Nonzero iff an element of the fragment is infinite or NaN.  bf16: an
// exponent field of all ones; with x = w & 0x7F807F80 per 32-bit word, adding
// 0x00800080 sets bit 15 (31) exactly for such a half (no carry crosses
// halves), so two integer operations test two elements.
__device__ __forceinline__ uint32_t nonfinite8(const bf16x8& f) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 u = __builtin_bit_cast(u32x4, f);
  const uint32_t m = 0x7F807F80u, o = 0x00800080u;
  return (((u[0] & m) + o) | ((u[1] & m) + o) | ((u[2] & m) + o) | ((u[3] & m) + o)) & 0x80008000u;
}
__device__ __forceinline__ uint32_t nonfinite8(const f32x8& f) {
  bool bad = false;
#pragma unroll
  for (int i = 0; i < 8; ++i) bad |= !__builtin_isfinite(f[i]);
  return bad ? 1u : 0u;
}
__device__ __forceinline__ uint32_t nonfinite1(float x) { return __builtin_isfinite(x) ? 0u : 1u; }

// OR `bits` into word `field` of sequence b's statistics (vector atomics;
// the wave-uniform test keeps the clean path to one ballot).
__device__ __forceinline__ void flag_or(int32_t* stats, int b, int field, int bits) {
  if (stats == nullptr) return;
  if (__ballot(bits != 0) == 0ull) return;
  if (bits != 0) atomicOr(stats + (size_t)b * STATS_INTS + field, bits);
}


}  // namespace sgdn
