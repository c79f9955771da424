// valu.hip -- fp32 vector-ALU kernels for the KV sums and the readout.
//
// These serve the float32 dtype and any (dtype, d) pair without a matrix-core
// kernel, and act as an independent cross-check of the MFMA kernels (no
// transposed LDS tiles, no operand packing). Same contract as the MFMA path:
//   kv:      U = sum_{t in part} phi(k_t) v_t^T, u = sum phi(k_t)
//   readout: o_t = sigmoid(g_t) * (phi(q_t)^T S_f) / (phi(q_t)^T z_f + eps)
#include "common.hpp"
#include "plan.hpp"

namespace gla {
namespace {

constexpr int kThreads = 256;
constexpr int kKvTile = 32;  // tokens staged in LDS per step

// One workgroup per (slab, group of frames, part). Thread layout: key feature
// i = tid % D, value columns j = tid / D + (256 / D) * c for c < D*D/256. Each
// token adds phi(k[i]) * v[j] to the thread's entries; u[i] is kept by threads
// with tid < D. Entering each frame after the group's first, the running sums
// are scaled by that frame's gamma; after each frame they are written to the
// frame's slot (S_loc_f, z_loc_f).
template <typename TIn, int D, bool kRope>
__global__ __launch_bounds__(kThreads) void kv_valu_kernel(View kview, View vview, int H,
                                                           const float *__restrict__ gamma,
                                                           float *__restrict__ ws, int F,
                                                           int64_t T, int P, int G,
                                                           int64_t part_len, RopeK rope) {
  static_assert(D * D >= kThreads && (D * D) % kThreads == 0, "D must be 16..128");
  constexpr int EPT = D * D / kThreads;
  constexpr int JS = kThreads / D;
  __shared__ float sk[kKvTile][D];                  // phi(k), turned with kRope
  __shared__ float sv[kKvTile][D];
  __shared__ float su[kRope ? kKvTile : 1][D];      // kRope: phi(k) unturned (for z)

  const int tid = threadIdx.x;
  const int NG = (F + G - 1) / G;
  const int64_t wg = blockIdx.x;
  const int p = (int)(wg % P);
  const int grp = (int)((wg / P) % NG);
  const int64_t bh = wg / ((int64_t)P * NG);
  const int64_t t0 = min((int64_t)p * part_len, T);
  const int64_t t1 = min(t0 + part_len, T);
  const int f_begin = grp * G;
  const int f_end = min(F, f_begin + G);
  const TIn *kslab = static_cast<const TIn *>(kview.data) + kview.slab(bh, H);
  const TIn *vslab = static_cast<const TIn *>(vview.data) + vview.slab(bh, H);

  const int i = tid % D;
  const int jc = tid / D;
  float acc[EPT];
#pragma unroll
  for (int c = 0; c < EPT; ++c) acc[c] = 0.f;
  float uacc = 0.f;

  for (int f = f_begin; f < f_end; ++f) {
    if (f > f_begin) {
      const float gm = gamma ? gamma[bh * F + f] : 1.f;
#pragma unroll
      for (int c = 0; c < EPT; ++c) acc[c] *= gm;
      uacc *= gm;
    }
    const TIn *kb = kslab + (int64_t)f * T * kview.sn;
    const TIn *vb = vslab + (int64_t)f * T * vview.sn;
    for (int64_t c0 = t0; c0 < t1; c0 += kKvTile) {
      const int n = (int)min((int64_t)kKvTile, t1 - c0);
      __syncthreads();
      for (int e = tid; e < kKvTile * D; e += kThreads) {
        const int tt = e / D, ii = e % D;
        float kk = 0.f, vv = 0.f;
        if (tt < n) {
          kk = relu(Elem<TIn>::load(kb, (c0 + tt) * kview.sn + ii));
          vv = Elem<TIn>::load(vb, (c0 + tt) * vview.sn + ii);
        }
        sk[tt][ii] = kk;
        sv[tt][ii] = vv;
      }
      if constexpr (kRope) {
        __syncthreads();
        // turn each pair of phi(k) by its token's full rotation; keep the
        // unturned copy for z
        for (int e = tid; e < kKvTile * (D / 2); e += kThreads) {
          const int tt = e / (D / 2), pp = e % (D / 2);
          const float a = sk[tt][2 * pp], b = sk[tt][2 * pp + 1];
          su[tt][2 * pp] = a;
          su[tt][2 * pp + 1] = b;
          const float2 ab = rotate_pair(a, b, token_rope_cs(rope, f, (int)(c0 + tt), pp));
          sk[tt][2 * pp] = ab.x;
          sk[tt][2 * pp + 1] = ab.y;
        }
      }
      __syncthreads();
      for (int tt = 0; tt < n; ++tt) {
        const float kk = sk[tt][i];
        uacc += kRope ? su[tt][i] : kk;
#pragma unroll
        for (int c = 0; c < EPT; ++c) acc[c] = fmaf(kk, sv[tt][jc + JS * c], acc[c]);
      }
    }
    float *out = ws + ((bh * F + f) * (int64_t)P + p) * ((int64_t)D * D + D);
#pragma unroll
    for (int c = 0; c < EPT; ++c) out[i * D + jc + JS * c] = acc[c];
    if (jc == 0) out[D * D + i] = uacc;
  }
}

// One workgroup per (slab, frame, split). Thread layout: 4 value columns
// j = 4 * (tid % (D/4)) .. +3 of token tid / (D/4) of the current tile. phi(q)
// of the tile is staged in LDS; S_f comes from LDS (D <= 64) or global memory.
template <typename TIn, int D, bool kRope>
__global__ __launch_bounds__(kThreads) void readout_valu_kernel(
    View qview, View gview, View oview, int H, const float *__restrict__ gamma,
    const float *__restrict__ ws, const float *__restrict__ st, int64_t sstride, int F, int64_t T,
    int G, int64_t carry_offset, int R, int64_t read_len, float eps, int state_frame, RopeK rope) {
  constexpr int CG = D / 4;             // column groups
  constexpr int TT = kThreads / CG;     // tokens per tile
  constexpr bool kSInLds = (D <= 64);
  __shared__ float sS[kSInLds ? D * D : 1];
  __shared__ float sz[D];
  __shared__ float sq[TT][D];                  // phi(q), turned with kRope (numerator)
  __shared__ float sqd[kRope ? TT : 1][D];     // kRope: phi(q) unturned (normaliser)

  const int tid = threadIdx.x;
  const int64_t wg = blockIdx.x;
  const int r = (int)(wg % R);
  const int f = (int)((wg / R) % F);
  const int64_t bh = wg / ((int64_t)R * F);
  const int64_t t0 = min((int64_t)r * read_len, T);
  const int64_t t1 = min(t0 + read_len, T);
  if (t0 >= t1) return;

  // S_fs = S_loc_fs + w * carry of the group (fs: the frame's own state, or
  // the one all frames share)
  const int fs = state_frame >= 0 ? state_frame : f;
  constexpr int64_t E = (int64_t)D * D + D;
  const int NG = (F + G - 1) / G;
  const float *Sg = st + (bh * F + fs) * sstride;
  // G == 1: the carry kernel has written S_f itself (no carries kept)
  const float *Cg = G > 1 ? ws + carry_offset + (bh * NG + fs / G) * E : Sg;
  const float w = G > 1 ? carry_weight(gamma ? gamma + bh * F : nullptr, fs, G) : 0.f;
  if (kSInLds)
    for (int e = tid; e < D * D; e += kThreads) sS[e] = fmaf(w, Cg[e], Sg[e]);
  for (int e = tid; e < D; e += kThreads) sz[e] = fmaf(w, Cg[D * D + e], Sg[D * D + e]);

  const int64_t trow0 = (int64_t)f * T;
  const TIn *qs = static_cast<const TIn *>(qview.data) + qview.slab(bh, H);
  const TIn *gs = static_cast<const TIn *>(gview.data) + gview.slab(bh, H);
  TIn *os = const_cast<TIn *>(static_cast<const TIn *>(oview.data)) + oview.slab(bh, H);
  const int cg = tid % CG;
  const int tl = tid / CG;

  for (int64_t c0 = t0; c0 < t1; c0 += TT) {
    const int n = (int)min((int64_t)TT, t1 - c0);
    __syncthreads();
    for (int e = tid; e < TT * D; e += kThreads) {
      const int tt = e / D, ii = e % D;
      sq[tt][ii] =
          (tt < n) ? relu(Elem<TIn>::load(qs, (trow0 + c0 + tt) * qview.sn + ii)) : 0.f;
    }
    if constexpr (kRope) {
      __syncthreads();
      for (int e = tid; e < TT * (D / 2); e += kThreads) {
        const int tt = e / (D / 2), pp = e % (D / 2);
        const float a = sq[tt][2 * pp], b = sq[tt][2 * pp + 1];
        sqd[tt][2 * pp] = a;
        sqd[tt][2 * pp + 1] = b;
        const float2 ab = rotate_pair(a, b, token_rope_cs(rope, f, (int)(c0 + tt), pp));
        sq[tt][2 * pp] = ab.x;
        sq[tt][2 * pp + 1] = ab.y;
      }
    }
    __syncthreads();
    if (tl < n) {
      float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
      float den = 0.f;
      for (int ii = 0; ii < D; ++ii) {
        const float qi = sq[tl][ii];
        den = fmaf(kRope ? sqd[tl][ii] : qi, sz[ii], den);
        float4 s4;
        if (kSInLds) {
          s4 = *reinterpret_cast<const float4 *>(sS + ii * D + 4 * cg);
        } else {
          const float4 a4 = *reinterpret_cast<const float4 *>(Sg + ii * D + 4 * cg);
          const float4 c4 = *reinterpret_cast<const float4 *>(Cg + ii * D + 4 * cg);
          s4 = make_float4(fmaf(w, c4.x, a4.x), fmaf(w, c4.y, a4.y), fmaf(w, c4.z, a4.z),
                           fmaf(w, c4.w, a4.w));
        }
        num.x = fmaf(qi, s4.x, num.x);
        num.y = fmaf(qi, s4.y, num.y);
        num.z = fmaf(qi, s4.z, num.z);
        num.w = fmaf(qi, s4.w, num.w);
      }
      const float inv = 1.f / (den + eps);
      const int64_t row = trow0 + c0 + tl;
      const float4 gg = Elem<TIn>::load4(gs, row * gview.sn + 4 * cg);
      float4 out;
      out.x = sigmoid(gg.x) * (num.x * inv);
      out.y = sigmoid(gg.y) * (num.y * inv);
      out.z = sigmoid(gg.z) * (num.z * inv);
      out.w = sigmoid(gg.w) * (num.w * inv);
      Elem<TIn>::store4(os, row * oview.sn + 4 * cg, out);
    }
  }
}

template <typename TIn, int D>
void kv_valu_launch(const Plan &p, const KvArgs &a, int64_t grid, hipStream_t s) {
  if (a.rope.on)
    hipLaunchKernelGGL((kv_valu_kernel<TIn, D, true>), dim3((unsigned)grid), dim3(kThreads), 0,
                       s, a.k, a.v, a.H, a.gamma, a.ws, p.F, p.T, p.P, p.G, p.part_len, a.rope);
  else
    hipLaunchKernelGGL((kv_valu_kernel<TIn, D, false>), dim3((unsigned)grid), dim3(kThreads), 0,
                       s, a.k, a.v, a.H, a.gamma, a.ws, p.F, p.T, p.P, p.G, p.part_len, a.rope);
}

template <typename TIn>
hipError_t kv_valu_dispatch(const Plan &p, const KvArgs &a, hipStream_t s) {
  const int64_t grid = p.BH * p.NG * p.P;
  switch (p.d) {
    case 16: kv_valu_launch<TIn, 16>(p, a, grid, s); break;
    case 32: kv_valu_launch<TIn, 32>(p, a, grid, s); break;
    case 64: kv_valu_launch<TIn, 64>(p, a, grid, s); break;
    case 128: kv_valu_launch<TIn, 128>(p, a, grid, s); break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename TIn, int D>
void readout_valu_launch(const Plan &p, const ReadoutArgs &a, int64_t grid, hipStream_t s) {
  if (a.rope.on)
    hipLaunchKernelGGL((readout_valu_kernel<TIn, D, true>), dim3((unsigned)grid),
                       dim3(kThreads), 0, s, a.q, a.g, a.o, a.H, a.gamma, a.ws, a.states.base,
                       a.states.stride, p.F, p.T, p.G, p.carry_offset(), p.R, p.read_len, a.eps,
                       a.state_frame, a.rope);
  else
    hipLaunchKernelGGL((readout_valu_kernel<TIn, D, false>), dim3((unsigned)grid),
                       dim3(kThreads), 0, s, a.q, a.g, a.o, a.H, a.gamma, a.ws, a.states.base,
                       a.states.stride, p.F, p.T, p.G, p.carry_offset(), p.R, p.read_len, a.eps,
                       a.state_frame, a.rope);
}

template <typename TIn>
hipError_t readout_valu_dispatch(const Plan &p, const ReadoutArgs &a, hipStream_t s) {
  const int64_t grid = p.BH * p.F * p.R;
  switch (p.d) {
    case 16: readout_valu_launch<TIn, 16>(p, a, grid, s); break;
    case 32: readout_valu_launch<TIn, 32>(p, a, grid, s); break;
    case 64: readout_valu_launch<TIn, 64>(p, a, grid, s); break;
    case 128: readout_valu_launch<TIn, 128>(p, a, grid, s); break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kv_valu(const Plan &p, int dtype, const KvArgs &a, hipStream_t s) {
  if (p.BH * p.NG * p.P == 0) return hipSuccess;
  return dtype == 0 ? kv_valu_dispatch<float>(p, a, s) : kv_valu_dispatch<bf16_t>(p, a, s);
}

hipError_t launch_readout_valu(const Plan &p, int dtype, const ReadoutArgs &a, hipStream_t s) {
  if (p.BH * p.F * p.R == 0 || p.T == 0) return hipSuccess;
  return dtype == 0 ? readout_valu_dispatch<float>(p, a, s)
                    : readout_valu_dispatch<bf16_t>(p, a, s);
}

}  // namespace gla
