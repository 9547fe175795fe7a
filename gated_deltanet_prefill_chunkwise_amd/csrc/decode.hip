// Single-token decode step of the gated delta rule: the recurrence that
// continues from the final state a prefill returns (SparseGDN reading notes,
// Sec. 2.6, which hands S_{C,h} to autoregressive decoding; the step itself is
// the per-token form of Sec. 2.1).  For value head h of sequence b, with
// alpha = 2^a and the key/query of head h / (Nv / Nq):
//   S'  = alpha S + k u^T,   u = beta (v - alpha S^T k)
//   o   = S'^T q / sqrt(d)  = (alpha S^T q + (k . q) u) / sqrt(d)
// Both reductions over the key index read the old state, so S is read once
// and written once.
//
// The state columns are independent, so a head's 128 x 128 fp32 state is
// split into two 64-column blocks, one workgroup each: 128 rows x 256 bytes
// in and out.  Thread t holds columns 4 (t % 16) .. +3 of the block for rows
// t / 16 + 16 i (i < 8) in registers; the two column sums and k . q reduce
// over the 16 row groups (lane shuffles inside a wave, then LDS across the
// four waves) and every thread updates its own 32 values (it writes only what
// it read, so s_out may alias s_in).  The bound is HBM: per head 64 KiB of
// state read and 64 KiB written.  The state is streamed with non-temporal
// loads and stores (it is touched once per step), which brings the kernel to
// the rate of a plain copy with the same access pattern.
#include "common.h"
#include "kernels.h"

namespace sgdn {

namespace {

constexpr int NCB = 2;          // column blocks per head
constexpr int CB = DV / NCB;    // 64 columns per block
constexpr int TPR = CB / 4;     // 16 threads per row, 4 columns each
constexpr int RG = 256 / TPR;   // 16 row groups
constexpr int NR = DK / RG;     // 8 rows per thread
constexpr int NVAL = 2 * 4 + 1; // per thread: 4 S^T k, 4 S^T q, k . q

__device__ __forceinline__ f32x4 ld4(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
}
__device__ __forceinline__ void st4(float* p, f32x4 x) {
  __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(p));
}

template <typename E, typename O>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs p) {
  __shared__ float red[4][TPR][NVAL];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cb = blockIdx.x % NCB;
  const int bh = blockIdx.x / NCB;          // b * Nv + h
  const int b = bh / p.Nv, h = bh - b * p.Nv;
  const int hq = h / (p.Nv / p.Nq);
  const int cg = tid % TPR, rg = tid / TPR;
  const int col = cb * CB + cg * 4;

  const float* sin = p.s_in + (size_t)bh * DK * DV + col;
  f32x4 s[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) s[i] = ld4(sin + (size_t)(rg + RG * i) * DV);

  const E* kp = static_cast<const E*>(p.k) + ((size_t)b * p.Nq + hq) * DK;
  const E* qp = static_cast<const E*>(p.q) + ((size_t)b * p.Nq + hq) * DK;
  float kr[NR], qr[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    kr[i] = to_f(kp[rg + RG * i]);
    qr[i] = to_f(qp[rg + RG * i]);
  }
  const E* vp = static_cast<const E*>(p.v) + (size_t)bh * DV + col;
  float vv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) vv[j] = to_f(vp[j]);
  const float alpha = exp2f(p.a[bh]);
  const float beta = to_f(static_cast<const E*>(p.beta)[bh]);

  float acc[NVAL];
#pragma unroll
  for (int j = 0; j < NVAL; ++j) acc[j] = 0.f;
#pragma unroll
  for (int i = 0; i < NR; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[j] += kr[i] * s[i][j];
      acc[4 + j] += qr[i] * s[i][j];
    }
    acc[8] += kr[i] * qr[i];
  }
  // sum over the four row groups of the wave (lane bits 4..5)
#pragma unroll
  for (int off = TPR; off < 64; off <<= 1) {
#pragma unroll
    for (int j = 0; j < NVAL; ++j) acc[j] += __shfl_xor(acc[j], off, 64);
  }
  if (lane < TPR) {
#pragma unroll
    for (int j = 0; j < NVAL; ++j) red[wave][lane][j] = acc[j];
  }
  __syncthreads();
  float tot[NVAL];
#pragma unroll
  for (int j = 0; j < NVAL; ++j)
    tot[j] = (red[0][cg][j] + red[1][cg][j]) + (red[2][cg][j] + red[3][cg][j]);

  float u[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) u[j] = beta * (vv[j] - alpha * tot[j]);

  float* sout = p.s_out + (size_t)bh * DK * DV + col;
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    f32x4 y;
#pragma unroll
    for (int j = 0; j < 4; ++j) y[j] = alpha * s[i][j] + kr[i] * u[j];
    st4(sout + (size_t)(rg + RG * i) * DV, y);
  }
  if (rg == 0) {
    const float scale = 0.08838834764831845f;   // 1 / sqrt(128)
    O* op = static_cast<O*>(p.o) + (size_t)bh * DV + col;
#pragma unroll
    for (int j = 0; j < 4; ++j) op[j] = from_f<O>((alpha * tot[4 + j] + tot[8] * u[j]) * scale);
  }
}

template <typename E>
hipError_t launch_decode_e(const DecodeArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((size_t)a.B * a.Nv * NCB));
  if (a.o_type == OUT_BF16)
    hipLaunchKernelGGL((decode_kernel<E, bf16>), grid, dim3(256), 0, s, a);
  else if (a.o_type == OUT_F16)
    hipLaunchKernelGGL((decode_kernel<E, fp16>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((decode_kernel<E, float>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int in_bf16, hipStream_t s) {
  return in_bf16 ? launch_decode_e<bf16>(a, s) : launch_decode_e<float>(a, s);
}

}  // namespace sgdn
