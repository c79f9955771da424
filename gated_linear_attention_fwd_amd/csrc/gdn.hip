// gdn.hip -- frame-wise Gated DeltaNet: vector-ALU kernels and the scan.
//
// The SANA-WM analysis page (method components) names the mixer -- decay gates
// plus a delta-rule correction of the recurrent state, keys scaled by
// 1/sqrt(D S) -- without its equations. Reading taken: one block delta-rule
// update per frame, every token measuring its error against the same decayed
// prior (S = tokens per frame, c = key_scale):
//   P_f = gamma_f S_{f-1},  e_t = v_t - P_f^T (c k_t),  S_f = P_f + sum_t beta_t (c k_t) e_t^T
//   o_t = S_f^T q_t  for every token of frame f.
// With the frame's sums U_f = sum_t beta_t k_t v_t^T and A_f = sum_t beta_t k_t k_t^T
// (both d x d) this is the matrix recurrence
//   S_f = gamma_f (S_{f-1} - c^2 A_f S_{f-1}) + c U_f
// whose columns evolve independently -- which is how the scan is split.
//
// Workspace: one slot of 2 d^2 floats per (slab, frame, part): U, then A.
// After the scan, part 0's U area of frame f holds S_f.
#include "common.hpp"
#include "plan.hpp"

namespace gla {
namespace {

constexpr int kThreads = 256;
constexpr int kKvTile = 32;

// One workgroup per (slab, frame, part). Thread layout as the kv kernel's:
// key feature i = tid % D, value (or key) columns j = tid / D + (256 / D) c.
template <typename TIn, int D>
__global__ __launch_bounds__(kThreads) void gdn_kv_valu_kernel(View kv, View vv, int H,
                                                               const float *__restrict__ beta,
                                                               float *__restrict__ ws, int F,
                                                               int64_t T, int P,
                                                               int64_t part_len) {
  constexpr int EPT = D * D / kThreads;
  constexpr int JS = kThreads / D;
  __shared__ float sk[kKvTile][D];
  __shared__ float sv[kKvTile][D];
  __shared__ float sb[kKvTile];

  const int tid = threadIdx.x;
  const int64_t wg = blockIdx.x;
  const int p = (int)(wg % P);
  const int f = (int)((wg / P) % F);
  const int64_t bh = wg / ((int64_t)P * F);
  const int64_t N = (int64_t)F * T;
  const int64_t t0 = min((int64_t)p * part_len, T);
  const int64_t t1 = min(t0 + part_len, T);
  const TIn *ks = static_cast<const TIn *>(kv.data) + kv.slab(bh, H) + (int64_t)f * T * kv.sn;
  const TIn *vs = static_cast<const TIn *>(vv.data) + vv.slab(bh, H) + (int64_t)f * T * vv.sn;
  const float *bs = beta + bh * N + (int64_t)f * T;

  const int i = tid % D, jc = tid / D;
  float u[EPT], a[EPT];
#pragma unroll
  for (int c = 0; c < EPT; ++c) u[c] = a[c] = 0.f;
  for (int64_t c0 = t0; c0 < t1; c0 += kKvTile) {
    const int n = (int)min((int64_t)kKvTile, t1 - c0);
    __syncthreads();
    for (int e = tid; e < kKvTile * D; e += kThreads) {
      const int tt = e / D, ii = e % D;
      const bool ok = tt < n;
      sk[tt][ii] = ok ? Elem<TIn>::load(ks, (c0 + tt) * kv.sn + ii) : 0.f;
      sv[tt][ii] = ok ? Elem<TIn>::load(vs, (c0 + tt) * vv.sn + ii) : 0.f;
    }
    if (tid < kKvTile) sb[tid] = tid < n ? bs[c0 + tid] : 0.f;
    __syncthreads();
    for (int tt = 0; tt < n; ++tt) {
      const float kb = sb[tt] * sk[tt][i];
#pragma unroll
      for (int c = 0; c < EPT; ++c) {
        u[c] = fmaf(kb, sv[tt][jc + JS * c], u[c]);
        a[c] = fmaf(kb, sk[tt][jc + JS * c], a[c]);
      }
    }
  }
  float *out = ws + ((bh * F + f) * (int64_t)P + p) * (2 * (int64_t)D * D);
#pragma unroll
  for (int c = 0; c < EPT; ++c) {
    out[i * D + jc + JS * c] = u[c];
    out[D * D + i * D + jc + JS * c] = a[c];
  }
}

// One workgroup per (slab, block of CB columns of S), frames in order:
//   S[:, cols] <- gamma_f (S[:, cols] - c^2 A_f S[:, cols]) + c U_f[:, cols]
// A_f (summed over parts) goes through LDS; the next frame's A_f and U_f are
// loaded while the current one is applied (d <= 64).
template <int D>
struct ScanCfg {
  static constexpr int CB = 8;                  // columns per workgroup
  static constexpr int NEL = D * CB;            // state elements per workgroup
  static constexpr int EPT = NEL >= kThreads ? NEL / kThreads : 1;
  static constexpr int APT = D * D / kThreads;  // A elements loaded per thread
  static constexpr bool kPrefetch = D <= 64;
};

template <int D>
__global__ __launch_bounds__(kThreads) void gdn_scan_kernel(
    float *__restrict__ ws, const float *__restrict__ gamma, const float *S_in, float *S_out,
    int F, int P, float key_scale) {
  using C = ScanCfg<D>;
  __shared__ float sA[D * D];
  __shared__ float sS[D * C::CB];
  constexpr int64_t SLOT = 2 * (int64_t)D * D;
  constexpr int NCB = D / C::CB;
  const int tid = threadIdx.x;
  const int64_t bh = blockIdx.x / NCB;
  const int j0 = (int)(blockIdx.x % NCB) * C::CB;
  const float c1 = key_scale, c2 = key_scale * key_scale;
  // this thread's elements (i, j0 + jj) of the column block
  int ei[C::EPT], ej[C::EPT];
  bool ev[C::EPT];
#pragma unroll
  for (int x = 0; x < C::EPT; ++x) {
    const int e = tid + kThreads * x;
    ev[x] = e < C::NEL;
    ei[x] = (e % C::NEL) / C::CB;
    ej[x] = (e % C::NEL) % C::CB;
  }
  float s[C::EPT];
#pragma unroll
  for (int x = 0; x < C::EPT; ++x)
    s[x] = (S_in && ev[x]) ? S_in[bh * D * D + ei[x] * D + j0 + ej[x]] : 0.f;

  float *slab = ws + bh * (int64_t)F * P * SLOT;
  auto load_frame = [&](int f, float *areg, float *ureg) {
    const float *src = slab + (int64_t)f * P * SLOT;
#pragma unroll
    for (int x = 0; x < C::APT; ++x) {
      float acc = 0.f;
      for (int p = 0; p < P; ++p) acc += src[p * SLOT + D * D + tid + kThreads * x];
      areg[x] = acc;
    }
#pragma unroll
    for (int x = 0; x < C::EPT; ++x) {
      float acc = 0.f;
      if (ev[x])
        for (int p = 0; p < P; ++p) acc += src[p * SLOT + ei[x] * D + j0 + ej[x]];
      ureg[x] = acc;
    }
  };
  float areg[C::APT], ureg[C::EPT];
  if (F > 0) load_frame(0, areg, ureg);
  for (int f = 0; f < F; ++f) {
    __syncthreads();  // the previous frame's sA / sS reads are done
#pragma unroll
    for (int x = 0; x < C::APT; ++x) sA[tid + kThreads * x] = areg[x];
#pragma unroll
    for (int x = 0; x < C::EPT; ++x)
      if (ev[x]) sS[ei[x] * C::CB + ej[x]] = s[x];
    float u[C::EPT];
#pragma unroll
    for (int x = 0; x < C::EPT; ++x) u[x] = ureg[x];
    __syncthreads();
    if (C::kPrefetch && f + 1 < F) load_frame(f + 1, areg, ureg);
    const float gm = gamma[bh * F + f];
#pragma unroll
    for (int x = 0; x < C::EPT; ++x) {
      if (!ev[x]) continue;
      float as = 0.f;
      for (int m = 0; m < D; ++m) as = fmaf(sA[ei[x] * D + m], sS[m * C::CB + ej[x]], as);
      s[x] = fmaf(gm, fmaf(-c2, as, s[x]), c1 * u[x]);
      slab[(int64_t)f * P * SLOT + ei[x] * D + j0 + ej[x]] = s[x];  // S_f, in part 0's U area
    }
    if (!C::kPrefetch && f + 1 < F) {
      __syncthreads();  // the frame's sA reads are done before it is overwritten
      load_frame(f + 1, areg, ureg);
    }
  }
  if (S_out) {
#pragma unroll
    for (int x = 0; x < C::EPT; ++x)
      if (ev[x]) S_out[bh * D * D + ei[x] * D + j0 + ej[x]] = s[x];
  }
}

// One workgroup per (slab, frame, split): o_t = S_f^T q_t. Thread (cg, tl):
// value columns 4cg .. 4cg+3 of token tl of the tile; S_f in LDS (d <= 64).
template <typename TIn, int D>
__global__ __launch_bounds__(kThreads) void gdn_readout_valu_kernel(
    View qv, View ov, int H, const float *__restrict__ ws, int F, int64_t T, int P, int R,
    int64_t read_len) {
  constexpr int CG = D / 4;
  constexpr int TT = kThreads / CG;
  constexpr bool kSInLds = (D <= 64);
  __shared__ float sS[kSInLds ? D * D : 1];
  __shared__ float sq[TT][D];
  const int tid = threadIdx.x;
  const int64_t wg = blockIdx.x;
  const int r = (int)(wg % R);
  const int f = (int)((wg / R) % F);
  const int64_t bh = wg / ((int64_t)R * F);
  const int64_t t0 = min((int64_t)r * read_len, T);
  const int64_t t1 = min(t0 + read_len, T);
  if (t0 >= t1) return;
  const float *Sg = ws + ((bh * F + f) * (int64_t)P) * (2 * (int64_t)D * D);
  if (kSInLds)
    for (int e = tid; e < D * D; e += kThreads) sS[e] = Sg[e];
  const TIn *qs = static_cast<const TIn *>(qv.data) + qv.slab(bh, H);
  TIn *os = const_cast<TIn *>(static_cast<const TIn *>(ov.data)) + ov.slab(bh, H);
  const int64_t trow0 = (int64_t)f * T;
  const int cg = tid % CG, tl = tid / CG;
  for (int64_t c0 = t0; c0 < t1; c0 += TT) {
    const int n = (int)min((int64_t)TT, t1 - c0);
    __syncthreads();
    for (int e = tid; e < TT * D; e += kThreads) {
      const int tt = e / D, ii = e % D;
      sq[tt][ii] = (tt < n) ? Elem<TIn>::load(qs, (trow0 + c0 + tt) * qv.sn + ii) : 0.f;
    }
    __syncthreads();
    if (tl < n) {
      float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int ii = 0; ii < D; ++ii) {
        const float qi = sq[tl][ii];
        const float4 s4 = *reinterpret_cast<const float4 *>((kSInLds ? sS : Sg) + ii * D + 4 * cg);
        num.x = fmaf(qi, s4.x, num.x);
        num.y = fmaf(qi, s4.y, num.y);
        num.z = fmaf(qi, s4.z, num.z);
        num.w = fmaf(qi, s4.w, num.w);
      }
      Elem<TIn>::store4(os, (trow0 + c0 + tl) * ov.sn + 4 * cg, num);
    }
  }
}

template <typename TIn>
hipError_t gdn_kv_valu_dispatch(const Plan &p, const GdnKvArgs &a, hipStream_t s) {
  const int64_t grid = p.BH * p.F * p.P;
#define GLA_GK_CASE(DD)                                                                       \
  case DD:                                                                                    \
    hipLaunchKernelGGL((gdn_kv_valu_kernel<TIn, DD>), dim3((unsigned)grid), dim3(kThreads), 0, \
                       s, a.k, a.v, a.H, a.beta, a.ws, p.F, p.T, p.P, p.part_len);            \
    break;
  switch (p.d) {
    GLA_GK_CASE(16)
    GLA_GK_CASE(32)
    GLA_GK_CASE(64)
    GLA_GK_CASE(128)
    default:
      return hipErrorInvalidValue;
  }
#undef GLA_GK_CASE
  return hipGetLastError();
}

template <typename TIn>
hipError_t gdn_readout_valu_dispatch(const Plan &p, const GdnReadoutArgs &a, hipStream_t s) {
  const int64_t grid = p.BH * p.F * p.R;
#define GLA_GR_CASE(DD)                                                                    \
  case DD:                                                                                 \
    hipLaunchKernelGGL((gdn_readout_valu_kernel<TIn, DD>), dim3((unsigned)grid),           \
                       dim3(kThreads), 0, s, a.q, a.o, a.H, a.ws, p.F, p.T, p.P, p.R,       \
                       p.read_len);                                                        \
    break;
  switch (p.d) {
    GLA_GR_CASE(16)
    GLA_GR_CASE(32)
    GLA_GR_CASE(64)
    GLA_GR_CASE(128)
    default:
      return hipErrorInvalidValue;
  }
#undef GLA_GR_CASE
  return hipGetLastError();
}

template <int D>
void gdn_scan_launch(const Plan &p, const GdnScanArgs &a, hipStream_t s) {
  const int64_t grid = p.BH * (D / ScanCfg<D>::CB);
  hipLaunchKernelGGL((gdn_scan_kernel<D>), dim3((unsigned)grid), dim3(kThreads), 0, s, a.ws,
                     a.gamma, a.S_in, a.S_out, p.F, p.P, a.key_scale);
}

}  // namespace

hipError_t launch_gdn_kv_valu(const Plan &p, int dtype, const GdnKvArgs &a, hipStream_t s) {
  if (p.BH * p.F * p.P == 0) return hipSuccess;
  return dtype == 0 ? gdn_kv_valu_dispatch<float>(p, a, s)
                    : gdn_kv_valu_dispatch<bf16_t>(p, a, s);
}

hipError_t launch_gdn_readout_valu(const Plan &p, int dtype, const GdnReadoutArgs &a,
                                   hipStream_t s) {
  if (p.BH * p.F * p.R == 0 || p.T == 0) return hipSuccess;
  return dtype == 0 ? gdn_readout_valu_dispatch<float>(p, a, s)
                    : gdn_readout_valu_dispatch<bf16_t>(p, a, s);
}

hipError_t launch_gdn_scan_valu(const Plan &p, const GdnScanArgs &a, hipStream_t s) {
  if (p.BH == 0) return hipSuccess;
  switch (p.d) {
    case 16: gdn_scan_launch<16>(p, a, s); break;
    case 32: gdn_scan_launch<32>(p, a, s); break;
    case 64: gdn_scan_launch<64>(p, a, s); break;
    case 128: gdn_scan_launch<128>(p, a, s); break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace gla
