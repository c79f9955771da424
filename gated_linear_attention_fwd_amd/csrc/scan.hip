// scan.hip -- inter-frame decayed state scan.
//
// S_f = gamma_f * S_{f-1} + U_f and z_f = gamma_f * z_{f-1} + u_f, S_{-1} = S_in
// (or 0): the frame-wise decayed running state of the gated linear attention
// (decay gates: "SANA-WM" analysis page, method components; additive update of
// a fixed D x D state carried block to block: SANA-Video ICLR 2026 oral talk,
// block KV cache passage). Bidirectional mode is the same scan with one frame
// and no decay.
//
// One thread owns one of the d*d + d state elements of one slab and walks the
// frames in order. The chain of FMAs is serial, the loads are not: a batch of
// FB frames is loaded first (summing each frame's parts in a fixed order), then
// folded in, so FB loads per thread are in flight at once.
#include "common.hpp"
#include "plan.hpp"

namespace gla {
namespace {

constexpr int kScanThreads = 256;
constexpr int kFrameBatch = 16;

__global__ __launch_bounds__(kScanThreads) void scan_kernel(
    float *__restrict__ ws, const float *__restrict__ gamma, const float *S_in,
    const float *z_in, float *S_out, float *z_out, int F, int P, int d, int64_t blocks_per_slab,
    int store_frames) {
  const int64_t dd = (int64_t)d * d;
  const int64_t E = dd + d;
  const int64_t bh = blockIdx.x / blocks_per_slab;
  const int64_t e = (blockIdx.x % blocks_per_slab) * kScanThreads + threadIdx.x;
  if (e >= E) return;

  float s = 0.f;
  if (S_in) s = (e < dd) ? S_in[bh * dd + e] : z_in[bh * d + (e - dd)];

  const int64_t frame_stride = (int64_t)P * E;
  float *base = ws + bh * (int64_t)F * frame_stride + e;
  const float *gm_slab = gamma ? gamma + bh * F : nullptr;

  for (int f0 = 0; f0 < F; f0 += kFrameBatch) {
    float acc[kFrameBatch];
    float gm[kFrameBatch];
#pragma unroll
    for (int j = 0; j < kFrameBatch; ++j) {
      const int f = f0 + j;
      acc[j] = 0.f;
      gm[j] = 1.f;
      if (f < F) {
        const float *src = base + (int64_t)f * frame_stride;
        float a = src[0];
        for (int p = 1; p < P; ++p) a += src[(int64_t)p * E];
        acc[j] = a;
        if (gm_slab) gm[j] = gm_slab[f];
      }
    }
#pragma unroll
    for (int j = 0; j < kFrameBatch; ++j) {
      const int f = f0 + j;
      if (f < F) {
        s = fmaf(gm[j], s, acc[j]);
        if (store_frames) base[(int64_t)f * frame_stride] = s;
      }
    }
  }

  if (S_out) {
    if (e < dd)
      S_out[bh * dd + e] = s;
    else
      z_out[bh * d + (e - dd)] = s;
  }
}

}  // namespace

hipError_t launch_scan(const Plan &p, const ScanArgs &a, hipStream_t stream) {
  const int64_t E = p.state_elems();
  const int64_t blocks_per_slab = (E + kScanThreads - 1) / kScanThreads;
  const int64_t grid = p.BH * blocks_per_slab;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(scan_kernel, dim3((unsigned)grid), dim3(kScanThreads), 0, stream, a.ws,
                     a.gamma, a.S_in, a.z_in, a.S_out, a.z_out, p.F, p.P, p.d, blocks_per_slab,
                     a.store_frames);
  return hipGetLastError();
}

}  // namespace gla
