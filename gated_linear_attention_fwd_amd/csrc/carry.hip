// carry.hip -- the carry chain of the decayed state scan across frame groups.
//
// The running state of the frame-causal gated linear attention obeys
// S_f = gamma_f * S_{f-1} + U_f (and z likewise), S_{-1} = S_in or 0: the
// frame-wise decay of the "SANA-WM" analysis page (method components) applied
// to the fixed D x D state that the SANA-Video ICLR 2026 oral talk carries
// additively from block to block (block KV cache passage). The kv kernel has
// already folded each group of G consecutive frames into its local sums
// S_loc; what remains is the chain over groups:
//
//   carry_0 = S_in (or 0)
//   carry_{g+1} = S_loc_{last frame of g} + (prod_{m in g} gamma_m) * carry_g
//
// and S_out = carry_{NG}. With one frame per group (G = 1) no carries are
// kept: the walk is the plain scan S_f = gamma_f S_{f-1} + U_f (the frame's
// parts summed in a fixed order), and S_f is written where the readout will
// read it: in place over the frame's slot (part 0), or into a caller's record
// of the per-frame states. Bidirectional mode is that walk with one frame and
// no decay.
//
// One thread owns one of the d*d + d state elements of one slab. The chain of
// FMAs is serial, the loads are not: a batch of groups is loaded first, then
// folded in, so many loads per thread are in flight at once.
#include "common.hpp"
#include "plan.hpp"

namespace gla {
namespace {

constexpr int kCarryThreads = 256;
constexpr int kGroupBatch = 16;
constexpr int kMaxGroupFrames = 8;  // the plan's most frames per group

// Sum of a frame's P parts (P > 4), left to right as in the unrolled case:
// loads go out eight at a time so that they overlap, the additions keep their
// order (bidirectional 720p/5s: 61 parts per slab).
__device__ __forceinline__ float sum_parts(const float *src, int P, int64_t E) {
  constexpr int kBatch = 8;
  float a = src[0];
  for (int p0 = 1; p0 < P; p0 += kBatch) {
    float x[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) x[j] = src[(int64_t)min(p0 + j, P - 1) * E];
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      if (p0 + j < P) a += x[j];
  }
  return a;
}

// kP > 0: frames of kP parts, their loads unrolled so that a batch's loads
// are all in flight at once; kP == 0: more parts, summed by sum_parts, for
// the groups that exist only (a frame of many parts is typically the one
// frame of a bidirectional call, where reloading it for every slot of the
// batch cost 16 times its reads).
template <int kP>
__global__ __launch_bounds__(kCarryThreads) void carry_kernel(
    float *ws, const float *__restrict__ gamma, const float *S_in,
    const float *z_in, float *S_out, float *z_out, int F, int P, int G, int NG, int d,
    int64_t blocks_per_slab, int64_t carry_offset, int keep_frames, float *frames,
    int64_t frames_stride) {
  const int64_t dd = (int64_t)d * d;
  const int64_t E = dd + d;
  const int64_t bh = blockIdx.x / blocks_per_slab;
  const int tid = threadIdx.x;
  const int64_t e_own = (blockIdx.x % blocks_per_slab) * kCarryThreads + tid;
  // threads past the state walk its last element too (the workgroup meets at
  // barriers) and store nothing
  const bool valid = e_own < E;
  const int64_t e = valid ? e_own : E - 1;

  float s = 0.f;
  if (S_in) s = (e < dd) ? S_in[bh * dd + e] : z_in[bh * d + (e - dd)];

  const int64_t frame_stride = (int64_t)P * E;
  float *slots = ws + bh * (int64_t)F * frame_stride + e;
  float *carry = ws + carry_offset + bh * (int64_t)NG * E + e;
  // G == 1: S_f of frame f (may be the slots themselves: ws is not restrict)
  float *dst = frames + bh * (int64_t)F * frames_stride + e;
  const float *gm_slab = gamma ? gamma + bh * F : nullptr;
  // The decays go through vector loads (an opaque zero in the index), all of
  // a batch at once. A group's decay is the product of its frames' decays:
  // one thread per group of the batch forms it (its loads issued together,
  // frames past the group reloading the last one and counting as 1, so the
  // product keeps its order) and shares it through LDS. Loaded and multiplied
  // one frame at a time, each scalar load was a memory round trip on the
  // critical path (720p/60s, 8-frame groups: 23 us per call).
  int vzero = 0;
  asm volatile("" : "+v"(vzero));
  __shared__ float gdec[2][kGroupBatch];

  for (int g0 = 0, bi = 0; g0 < NG; g0 += kGroupBatch, bi ^= 1) {
    float x[kGroupBatch];
    float w[kGroupBatch];
#pragma unroll
    for (int j = 0; j < kGroupBatch; ++j) {
      // groups past the end load the last group again (no branch around the
      // loads) and are dropped
      const int grp = g0 + j;
      const bool ok = grp < NG;
      const int gc = ok ? grp : NG - 1;
      const int last = min(F, (gc + 1) * G) - 1;
      const float *src = slots + (int64_t)last * frame_stride;
      float a = 0.f;
      if constexpr (kP > 0) {
        a = src[0];
#pragma unroll
        for (int p = 1; p < kP; ++p) a += src[(int64_t)p * E];
      } else {
        if (ok) a = sum_parts(src, P, E);
      }
      x[j] = ok ? a : 0.f;
      w[j] = 1.f;
      if (gm_slab && G == 1) w[j] = ok ? gm_slab[gc + vzero] : 1.f;
    }
    if (gm_slab && G > 1) {
      if (tid < kGroupBatch) {
        const int gc = min(g0 + tid, NG - 1);
        const int f0 = gc * G;
        const int last = min(F, f0 + G) - 1;
        float wj = 1.f;
        if (G <= kMaxGroupFrames) {
          float gv[kMaxGroupFrames];
#pragma unroll
          for (int m = 0; m < kMaxGroupFrames; ++m) gv[m] = gm_slab[min(f0 + m, last) + vzero];
#pragma unroll
          for (int m = 0; m < kMaxGroupFrames; ++m) wj *= f0 + m <= last ? gv[m] : 1.f;
        } else {
          for (int m = f0; m <= last; ++m) wj *= gm_slab[m + vzero];
        }
        gdec[bi][tid] = wj;
      }
      // one barrier per batch: the buffer written here was last read before
      // the previous batch's barrier
      __syncthreads();
#pragma unroll
      for (int j = 0; j < kGroupBatch; ++j) w[j] = g0 + j < NG ? gdec[bi][j] : 1.f;
    }
#pragma unroll
    for (int j = 0; j < kGroupBatch; ++j) {
      const int grp = g0 + j;
      if (grp < NG) {
        if (valid && keep_frames && G > 1) carry[(int64_t)grp * E] = s;
        s = fmaf(w[j], s, x[j]);
        if (valid && keep_frames && G == 1) dst[(int64_t)grp * frames_stride] = s;
      }
    }
  }

  if (S_out && valid) {
    if (e < dd)
      S_out[bh * dd + e] = s;
    else
      z_out[bh * d + (e - dd)] = s;
  }
}

}  // namespace

hipError_t launch_carry(const Plan &p, const CarryArgs &a, hipStream_t stream) {
  const int64_t E = p.state_elems();
  const int64_t blocks_per_slab = (E + kCarryThreads - 1) / kCarryThreads;
  const int64_t grid = p.BH * blocks_per_slab;
  if (grid == 0) return hipSuccess;
#define GLA_CARRY_LAUNCH(KP)                                                                  \
  hipLaunchKernelGGL(carry_kernel<KP>, dim3((unsigned)grid), dim3(kCarryThreads), 0, stream,   \
                     a.ws, a.gamma, a.S_in, a.z_in, a.S_out, a.z_out, p.F, p.P, p.G, p.NG, p.d, \
                     blocks_per_slab, p.carry_offset(), a.keep_frames, a.frames.base,         \
                     a.frames.stride)
  switch (p.P) {
    case 1: GLA_CARRY_LAUNCH(1); break;
    case 2: GLA_CARRY_LAUNCH(2); break;
    case 3: GLA_CARRY_LAUNCH(3); break;
    case 4: GLA_CARRY_LAUNCH(4); break;
    default: GLA_CARRY_LAUNCH(0); break;
  }
#undef GLA_CARRY_LAUNCH
  return hipGetLastError();
}

}  // namespace gla
