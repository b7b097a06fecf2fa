// Query absorption and value up-projection on the vector ALUs (fp32 FMAs).
//
//   absorb:   q_abs[n][h][c] = sum_{k < d_nope} W[h][k][c] * q[n][h][k];
//             q_abs[n][h][d_latent + i] = q[n][h][d_nope + i]
//   out_proj: out[n][h][v]   = sum_c W[h][d_nope + v][c] * o[n][h][c]
//
// Workgroup = one head x 16 tokens, so each weight element read from memory
// serves 16 tokens.  grid = (ceil(N / 16), H).
#include "device_common.h"
#include "internal.h"

namespace mla {
namespace {

constexpr int kTokBlk = 16;
constexpr int kThreads = 256;
constexpr int kMaxDim = 512;

__device__ __forceinline__ float load_val(const void* p, int64_t i, bool f32) {
  return f32 ? static_cast<const float*>(p)[i]
             : bf16_bits_to_f32(static_cast<const uint16_t*>(p)[i]);
}

__device__ __forceinline__ void store_val(void* p, int64_t i, float v, bool f32) {
  if (f32) static_cast<float*>(p)[i] = v;
  else static_cast<uint16_t*>(p)[i] = (uint16_t)f32_to_bf16_bits(v);
}

template <bool kQF32, bool kWF32, bool kOF32>
__global__ __launch_bounds__(kThreads) void absorb_simt_kernel(ProjArgs a) {
  __shared__ float sq[kTokBlk][kMaxDim + 1];
  const int n0 = blockIdx.x * kTokBlk, h = blockIdx.y;
  const int nt = min(kTokBlk, a.N - n0);
  const int qw = a.dn + a.dr, ow = a.dc + a.dr;
  for (int idx = threadIdx.x; idx < kTokBlk * a.dn; idx += kThreads) {
    const int i = idx / a.dn, k = idx % a.dn;
    sq[i][k] = i < nt ? load_val(a.in, ((int64_t)(n0 + i) * a.H + h) * qw + k, kQF32) : 0.f;
  }
  __syncthreads();
  const int64_t wbase = (int64_t)h * (a.dn + a.dv) * a.dc;
  for (int c = threadIdx.x; c < a.dc; c += kThreads) {
    float acc[kTokBlk];
#pragma unroll
    for (int i = 0; i < kTokBlk; ++i) acc[i] = 0.f;
    for (int k = 0; k < a.dn; ++k) {
      const float w = load_val(a.w, wbase + (int64_t)k * a.dc + c, kWF32);
#pragma unroll
      for (int i = 0; i < kTokBlk; ++i) acc[i] = fmaf(sq[i][k], w, acc[i]);
    }
    for (int i = 0; i < nt; ++i) store_val(a.out, ((int64_t)(n0 + i) * a.H + h) * ow + c, acc[i], kOF32);
  }
  for (int idx = threadIdx.x; idx < nt * a.dr; idx += kThreads) {
    const int i = idx / a.dr, k = idx % a.dr;
    const int64_t row = (int64_t)(n0 + i) * a.H + h;
    store_val(a.out, row * ow + a.dc + k, load_val(a.in, row * qw + a.dn + k, kQF32), kOF32);
  }
}

constexpr int kCChunk = 32;

template <bool kWF32>
__global__ __launch_bounds__(kThreads) void out_proj_simt_kernel(ProjArgs a) {
  __shared__ float so[kTokBlk][kMaxDim + 1];
  __shared__ float sw[kCChunk][kMaxDim + 1];
  const int n0 = blockIdx.x * kTokBlk, h = blockIdx.y;
  const int nt = min(kTokBlk, a.N - n0);
  const float* o = static_cast<const float*>(a.in);
  for (int idx = threadIdx.x; idx < kTokBlk * a.dc; idx += kThreads) {
    const int i = idx / a.dc, c = idx % a.dc;
    so[i][c] = i < nt ? o[((int64_t)(n0 + i) * a.H + h) * a.dc + c] : 0.f;
  }
  const int64_t wbase = ((int64_t)h * (a.dn + a.dv) + a.dn) * a.dc;
  float acc[2][kTokBlk];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < kTokBlk; ++i) acc[j][i] = 0.f;
  for (int c0 = 0; c0 < a.dc; c0 += kCChunk) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < a.dv * kCChunk; idx += kThreads) {
      const int v = idx / kCChunk, c = idx % kCChunk;
      sw[c][v] = load_val(a.w, wbase + (int64_t)v * a.dc + c0 + c, kWF32);
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int v = threadIdx.x + j * kThreads;
      if (v < a.dv) {
        for (int c = 0; c < kCChunk; ++c) {
          const float w = sw[c][v];
#pragma unroll
          for (int i = 0; i < kTokBlk; ++i) acc[j][i] = fmaf(so[i][c0 + c], w, acc[j][i]);
        }
      }
    }
  }
  float* out = static_cast<float*>(a.out);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int v = threadIdx.x + j * kThreads;
    if (v < a.dv)
      for (int i = 0; i < nt; ++i) out[((int64_t)(n0 + i) * a.H + h) * a.dv + v] = acc[j][i];
  }
}

}  // namespace

hipError_t launch_absorb_q(const ProjArgs& a, hipStream_t s) {
  if (a.N == 0) return hipSuccess;
  if (absorb_mfma_supported(a)) return launch_absorb_mfma(a, s);
  const dim3 grid((a.N + kTokBlk - 1) / kTokBlk, a.H);
  const int key = (a.in_f32 ? 4 : 0) | (a.w_f32 ? 2 : 0) | (a.out_f32 ? 1 : 0);
  switch (key) {
    case 0: absorb_simt_kernel<false, false, false><<<grid, kThreads, 0, s>>>(a); break;
    case 1: absorb_simt_kernel<false, false, true><<<grid, kThreads, 0, s>>>(a); break;
    case 2: absorb_simt_kernel<false, true, false><<<grid, kThreads, 0, s>>>(a); break;
    case 3: absorb_simt_kernel<false, true, true><<<grid, kThreads, 0, s>>>(a); break;
    case 4: absorb_simt_kernel<true, false, false><<<grid, kThreads, 0, s>>>(a); break;
    case 5: absorb_simt_kernel<true, false, true><<<grid, kThreads, 0, s>>>(a); break;
    case 6: absorb_simt_kernel<true, true, false><<<grid, kThreads, 0, s>>>(a); break;
    default: absorb_simt_kernel<true, true, true><<<grid, kThreads, 0, s>>>(a); break;
  }
  return hipGetLastError();
}

hipError_t launch_out_proj(const ProjArgs& a, hipStream_t s) {
  if (a.N == 0) return hipSuccess;
  if (out_proj_mfma_supported(a)) return launch_out_proj_mfma(a, s);
  const dim3 grid((a.N + kTokBlk - 1) / kTokBlk, a.H);
  if (a.w_f32) out_proj_simt_kernel<true><<<grid, kThreads, 0, s>>>(a);
  else out_proj_simt_kernel<false><<<grid, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mla
