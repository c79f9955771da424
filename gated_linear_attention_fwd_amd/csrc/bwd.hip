// bwd.hip -- backward pass of the gated linear attention: vector-ALU kernels,
// the reverse scan of the state adjoints and the dgamma reduction.
//
// The gradients are the chain rule through the forward definition (taken in
// reverse order of its steps). Per slab, with h_t = num_t / (den_t + eps) and
// o_t = sigmoid(g_t) (.) h_t:
//   dg_t   = dO_t (.) h_t (.) sigmoid'(g_t)
//   dnum_t = dO_t (.) sigmoid(g_t) / (den_t + eps)
//   dden_t = -((dO_t (.) sigmoid(g_t)) . h_t) / (den_t + eps)
//   dq_t   = [q_t > 0] (.) (S_f dnum_t + dden_t z_f)                t in frame f
//   Sh_f   = sum_{t in f} phi(q_t) dnum_t^T + gamma_{f+1} Sh_{f+1},  Sh_{F-1} adds dS_out
//   zh_f   = sum_{t in f} dden_t phi(q_t) + gamma_{f+1} zh_{f+1},    zh_{F-1} adds dz_out
//   dk_t   = [k_t > 0] (.) (Sh_f v_t + zh_f),   dv_t = Sh_f^T phi(k_t)
//   dgamma_f = <Sh_f, S_{f-1}> + <zh_f, z_{f-1}>,   dS_in = gamma_0 Sh_0
// (S_f, z_f: the forward states, recomputed by the forward kv and carry
// kernels before these run, or read from the forward's record of them.)
#include "common.hpp"
#include "mfma_util.hpp"
#include "plan.hpp"

namespace gla {
namespace {

constexpr int kThreads = 256;

// One workgroup per (slab, frame, split). Token tiles of TT tokens: thread
// (cg, tl) owns value columns j = 4cg .. 4cg+3 of token tl for num, dg and
// dnum, and key features i = 4cg .. 4cg+3 for dq. The split's sums
// G = sum phi(q) dnum^T use the kv layout (thread: key feature i, value
// columns jc + JS c) and gz = sum dden phi(q) the threads with jc == 0.
// kRope: num and G take the turned phi(q), den, gz and the ReLU mask the
// unturned one, and S_f dnum turns back (R^T) before dden z_f is added; a
// thread's four key features are two whole pairs.
template <typename TIn, int D, bool kRope>
__global__ __launch_bounds__(kThreads) void bwd_q_valu_kernel(
    View qv, View gv, View dov, View dqv, View dgv, int H, const float *__restrict__ st,
    int64_t sstride, float *__restrict__ gs, int F, int64_t T, int R, int64_t read_len,
    float eps, int state_frame, RopeK rope) {
  constexpr int CG = D / 4;
  constexpr int TT = kThreads / CG;
  constexpr bool kSInLds = (D <= 64);
  constexpr int EPT = D * D / kThreads;
  constexpr int JS = kThreads / D;
  constexpr int64_t E = (int64_t)D * D + D;
  __shared__ float sS[kSInLds ? D * D : 1];
  __shared__ float sz[D];
  // token rows padded by CG floats: the two token rows a half-wave reads sit
  // 16 banks apart, so row reads that differ by column group do not collide
  constexpr int PITCH = D + CG;
  __shared__ float sq[TT][PITCH];   // phi(q), turned with kRope
  __shared__ float sqd[kRope ? TT : 1][PITCH];  // kRope: phi(q) unturned
  __shared__ float sdn[TT][PITCH];  // dnum
  // kRope: the pairs' frequencies, and the tile's turns from the staging (used
  // again to turn S_f dnum back)
  __shared__ double sfreq[kRope ? D / 2 : 1];
  __shared__ float2 scs[kRope ? TT : 1][kRope ? D / 2 : 1];
  __shared__ float sred[TT][CG];
  __shared__ float sdd[TT];     // dden

  const int tid = threadIdx.x;
  const int64_t wg = blockIdx.x;
  const int r = (int)(wg % R);
  const int f = (int)((wg / R) % F);
  const int64_t bh = wg / ((int64_t)R * F);
  const int64_t t0 = min((int64_t)r * read_len, T);
  const int64_t t1 = min(t0 + read_len, T);

  const float *Sg = st + (bh * F + (state_frame >= 0 ? state_frame : f)) * sstride;  // S_f
  if constexpr (kRope)
    for (int pp = tid; pp < D / 2; pp += kThreads) sfreq[pp] = pair_freq(rope, pp);
  if (kSInLds)
    for (int e = tid; e < D * D; e += kThreads) sS[e] = Sg[e];
  for (int e = tid; e < D; e += kThreads) sz[e] = Sg[D * D + e];

  const TIn *qs = static_cast<const TIn *>(qv.data) + qv.slab(bh, H);
  const TIn *gsl = static_cast<const TIn *>(gv.data) + gv.slab(bh, H);
  const TIn *dos = static_cast<const TIn *>(dov.data) + dov.slab(bh, H);
  TIn *dqs = const_cast<TIn *>(static_cast<const TIn *>(dqv.data)) + dqv.slab(bh, H);
  TIn *dgs = const_cast<TIn *>(static_cast<const TIn *>(dgv.data)) + dgv.slab(bh, H);
  const int64_t trow0 = (int64_t)f * T;
  const int cg = tid % CG, tl = tid / CG;
  const int ig = tid % D, jc = tid / D;
  float Gacc[EPT];
#pragma unroll
  for (int c = 0; c < EPT; ++c) Gacc[c] = 0.f;
  float gzacc = 0.f;

  for (int64_t c0 = t0; c0 < t1; c0 += TT) {
    const int n = (int)min((int64_t)TT, t1 - c0);
    __syncthreads();
    if constexpr (kRope) {
      for (int e = tid; e < TT * (D / 2); e += kThreads) {
        const int tt = e / (D / 2), pp = e % (D / 2);
        float a = 0.f, b = 0.f;
        if (tt < n) {
          const int64_t off = (trow0 + c0 + tt) * qv.sn + 2 * pp;
          a = relu(Elem<TIn>::load(qs, off));
          b = relu(Elem<TIn>::load(qs, off + 1));
        }
        sqd[tt][2 * pp] = a;
        sqd[tt][2 * pp + 1] = b;
        const float2 cs = token_rope_cs_freq(rope, f, (int)(c0 + tt), pp, sfreq[pp]);
        scs[tt][pp] = cs;
        const float2 ab = rotate_pair(a, b, cs);
        sq[tt][2 * pp] = ab.x;
        sq[tt][2 * pp + 1] = ab.y;
      }
    } else {
      for (int e = tid; e < TT * D; e += kThreads) {
        const int tt = e / D, ii = e % D;
        sq[tt][ii] =
            (tt < n) ? relu(Elem<TIn>::load(qs, (trow0 + c0 + tt) * qv.sn + ii)) : 0.f;
      }
    }
    __syncthreads();
    const int64_t row = trow0 + c0 + tl;
    float inv = 0.f;
    if (tl < n) {
      float num[4] = {0.f, 0.f, 0.f, 0.f};
      float den = 0.f;
      for (int ii = 0; ii < D; ++ii) {
        const float qi = sq[tl][ii];
        den = fmaf(kRope ? sqd[tl][ii] : qi, sz[ii], den);
        const float *Srow = kSInLds ? sS + ii * D : Sg + ii * D;
#pragma unroll
        for (int c = 0; c < 4; ++c) num[c] = fmaf(qi, Srow[4 * cg + c], num[c]);
      }
      inv = 1.f / (den + eps);
      const float4 gg = Elem<TIn>::load4(gsl, row * gv.sn + 4 * cg);
      const float4 dd = Elem<TIn>::load4(dos, row * dov.sn + 4 * cg);
      const float ga[4] = {gg.x, gg.y, gg.z, gg.w}, da[4] = {dd.x, dd.y, dd.z, dd.w};
      float dgo[4], part = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float sg = sigmoid(ga[c]);
        const float hh = num[c] * inv;
        const float dh = da[c] * sg;
        dgo[c] = da[c] * hh * sg * (1.f - sg);
        part = fmaf(dh, hh, part);
        sdn[tl][4 * cg + c] = dh * inv;
      }
      Elem<TIn>::store4(dgs, row * dgv.sn + 4 * cg, make_float4(dgo[0], dgo[1], dgo[2], dgo[3]));
      sred[tl][cg] = part;
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) sdn[tl][4 * cg + c] = 0.f;
      sred[tl][cg] = 0.f;
    }
    __syncthreads();
    if (tl < n) {
      float tot = 0.f;
      for (int c = 0; c < CG; ++c) tot += sred[tl][c];
      const float dden = -tot * inv;
      if (cg == 0) sdd[tl] = dden;
      float dqo[4];
      if constexpr (kRope) {
        float u[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float *Srow = kSInLds ? sS + (4 * cg + c) * D : Sg + (4 * cg + c) * D;
          float acc = 0.f;
          // each column group starts its sweep at its own column: the rows
          // 4cg + c of S (D floats apart) then fall in distinct banks
          for (int jj = 0; jj < D; ++jj) {
            const int j = (jj + cg) & (D - 1);
            acc = fmaf(Srow[j], sdn[tl][j], acc);
          }
          u[c] = acc;
        }
#pragma unroll
        for (int hp = 0; hp < 2; ++hp) {
          const float2 cs = scs[tl][2 * cg + hp];
          const float2 back = rotate_pair(u[2 * hp], u[2 * hp + 1], make_float2(cs.x, -cs.y));
          u[2 * hp] = back.x;
          u[2 * hp + 1] = back.y;
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int i = 4 * cg + c;
          dqo[c] = sqd[tl][i] > 0.f ? fmaf(dden, sz[i], u[c]) : 0.f;
        }
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int i = 4 * cg + c;
          const float *Srow = kSInLds ? sS + i * D : Sg + i * D;
          float acc = dden * sz[i];
          // each column group starts its sweep at its own column: the rows
          // 4cg + c of S (D floats apart) then fall in distinct banks
          for (int jj = 0; jj < D; ++jj) {
            const int j = (jj + cg) & (D - 1);
            acc = fmaf(Srow[j], sdn[tl][j], acc);
          }
          dqo[c] = sq[tl][i] > 0.f ? acc : 0.f;
        }
      }
      Elem<TIn>::store4(dqs, row * dqv.sn + 4 * cg, make_float4(dqo[0], dqo[1], dqo[2], dqo[3]));
    } else if (cg == 0) {
      sdd[tl] = 0.f;
    }
    __syncthreads();
    for (int tt = 0; tt < n; ++tt) {
      const float qi = sq[tt][ig];
#pragma unroll
      for (int c = 0; c < EPT; ++c) Gacc[c] = fmaf(qi, sdn[tt][jc + JS * c], Gacc[c]);
      gzacc = fmaf(sdd[tt], kRope ? sqd[tt][ig] : qi, gzacc);
    }
  }
  float *out = gs + ((bh * F + f) * (int64_t)R + r) * E;
#pragma unroll
  for (int c = 0; c < EPT; ++c) out[ig * D + jc + JS * c] = Gacc[c];
  if (jc == 0) out[D * D + ig] = gzacc;
}

// One workgroup per (slab, frame, part). Thread (cg, tl): dk for key features
// i = 4cg .. 4cg+3 and dv for value features j = 4cg .. 4cg+3 of token tl.
// kRope: dv takes the turned phi(k), the mask the unturned one, and Sh_f v
// turns back (R^T) before zh_f is added.
template <typename TIn, int D, bool kRope>
__global__ __launch_bounds__(kThreads) void bwd_k_valu_kernel(
    View kv, View vv, View dkv, View dvv, int H, const float *__restrict__ gs, int F, int64_t T,
    int P, int R, int64_t part_len, int adj_frame, RopeK rope) {
  constexpr int CG = D / 4;
  constexpr int TT = kThreads / CG;
  constexpr bool kSInLds = (D <= 64);
  constexpr int64_t E = (int64_t)D * D + D;
  __shared__ float sSh[kSInLds ? D * D : 1];
  __shared__ float szh[D];
  constexpr int PITCH = D + CG;  // padded token rows, as in bwd_q_valu_kernel
  __shared__ float sk[TT][PITCH];  // phi(k), turned with kRope
  __shared__ float skd[kRope ? TT : 1][PITCH];  // kRope: phi(k) unturned
  __shared__ float sv[TT][PITCH];
  __shared__ double sfreq[kRope ? D / 2 : 1];  // kRope: as in bwd_q_valu_kernel
  __shared__ float2 scs[kRope ? TT : 1][kRope ? D / 2 : 1];

  const int tid = threadIdx.x;
  const int64_t wg = blockIdx.x;
  const int p = (int)(wg % P);
  const int f = (int)((wg / P) % F);
  const int64_t bh = wg / ((int64_t)P * F);
  const int64_t t0 = min((int64_t)p * part_len, T);
  const int64_t t1 = min(t0 + part_len, T);
  if (t0 >= t1) return;

  const float *Sh = gs + ((bh * F + (adj_frame >= 0 ? adj_frame : f)) * (int64_t)R) * E;  // adjoint of S_f
  if constexpr (kRope)
    for (int pp = tid; pp < D / 2; pp += kThreads) sfreq[pp] = pair_freq(rope, pp);
  if (kSInLds)
    for (int e = tid; e < D * D; e += kThreads) sSh[e] = Sh[e];
  for (int e = tid; e < D; e += kThreads) szh[e] = Sh[D * D + e];

  const TIn *ks = static_cast<const TIn *>(kv.data) + kv.slab(bh, H);
  const TIn *vs = static_cast<const TIn *>(vv.data) + vv.slab(bh, H);
  TIn *dks = const_cast<TIn *>(static_cast<const TIn *>(dkv.data)) + dkv.slab(bh, H);
  TIn *dvs = const_cast<TIn *>(static_cast<const TIn *>(dvv.data)) + dvv.slab(bh, H);
  const int64_t trow0 = (int64_t)f * T;
  const int cg = tid % CG, tl = tid / CG;

  for (int64_t c0 = t0; c0 < t1; c0 += TT) {
    const int n = (int)min((int64_t)TT, t1 - c0);
    __syncthreads();
    if constexpr (kRope) {
      for (int e = tid; e < TT * (D / 2); e += kThreads) {
        const int tt = e / (D / 2), pp = e % (D / 2);
        float a = 0.f, b = 0.f, va = 0.f, vb = 0.f;
        if (tt < n) {
          const int64_t rr = trow0 + c0 + tt;
          a = relu(Elem<TIn>::load(ks, rr * kv.sn + 2 * pp));
          b = relu(Elem<TIn>::load(ks, rr * kv.sn + 2 * pp + 1));
          va = Elem<TIn>::load(vs, rr * vv.sn + 2 * pp);
          vb = Elem<TIn>::load(vs, rr * vv.sn + 2 * pp + 1);
        }
        skd[tt][2 * pp] = a;
        skd[tt][2 * pp + 1] = b;
        const float2 cs = token_rope_cs_freq(rope, f, (int)(c0 + tt), pp, sfreq[pp]);
        scs[tt][pp] = cs;
        const float2 ab = rotate_pair(a, b, cs);
        sk[tt][2 * pp] = ab.x;
        sk[tt][2 * pp + 1] = ab.y;
        sv[tt][2 * pp] = va;
        sv[tt][2 * pp + 1] = vb;
      }
    } else {
      for (int e = tid; e < TT * D; e += kThreads) {
        const int tt = e / D, ii = e % D;
        const bool ok = tt < n;
        const int64_t rr = trow0 + c0 + tt;
        sk[tt][ii] = ok ? relu(Elem<TIn>::load(ks, rr * kv.sn + ii)) : 0.f;
        sv[tt][ii] = ok ? Elem<TIn>::load(vs, rr * vv.sn + ii) : 0.f;
      }
    }
    __syncthreads();
    if (tl < n) {
      const int64_t row = trow0 + c0 + tl;
      float dko[4], dvo[4] = {0.f, 0.f, 0.f, 0.f};
      if constexpr (kRope) {
        float u[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float *Srow = kSInLds ? sSh + (4 * cg + c) * D : Sh + (4 * cg + c) * D;
          float acc = 0.f;
          for (int jj = 0; jj < D; ++jj) {  // staggered start, as in bwd_q_valu_kernel
            const int j = (jj + cg) & (D - 1);
            acc = fmaf(Srow[j], sv[tl][j], acc);
          }
          u[c] = acc;
        }
#pragma unroll
        for (int hp = 0; hp < 2; ++hp) {
          const float2 cs = scs[tl][2 * cg + hp];
          const float2 back = rotate_pair(u[2 * hp], u[2 * hp + 1], make_float2(cs.x, -cs.y));
          u[2 * hp] = back.x;
          u[2 * hp + 1] = back.y;
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int i = 4 * cg + c;
          dko[c] = skd[tl][i] > 0.f ? u[c] + szh[i] : 0.f;
        }
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int i = 4 * cg + c;
          const float *Srow = kSInLds ? sSh + i * D : Sh + i * D;
          float acc = szh[i];
          for (int jj = 0; jj < D; ++jj) {  // staggered start, as in bwd_q_valu_kernel
            const int j = (jj + cg) & (D - 1);
            acc = fmaf(Srow[j], sv[tl][j], acc);
          }
          dko[c] = sk[tl][i] > 0.f ? acc : 0.f;
        }
      }
      for (int i = 0; i < D; ++i) {
        const float ki = sk[tl][i];
        const float *Srow = kSInLds ? sSh + i * D : Sh + i * D;
#pragma unroll
        for (int c = 0; c < 4; ++c) dvo[c] = fmaf(Srow[4 * cg + c], ki, dvo[c]);
      }
      Elem<TIn>::store4(dks, row * dkv.sn + 4 * cg, make_float4(dko[0], dko[1], dko[2], dko[3]));
      Elem<TIn>::store4(dvs, row * dvv.sn + 4 * cg, make_float4(dvo[0], dvo[1], dvo[2], dvo[3]));
    }
  }
}

// One thread per (slab, state element), frames walked last to first, in
// batches of 8 frames: a batch's loads are issued while the previous batch is
// folded into the serial chain. Per frame, the block sums Sh_f[e] * S_{f-1}[e]
// over its elements (waves by DPP moves, then LDS) into dgp[(slab, frame)][block].
// At 720p/60s: 160 us with one batch in flight and shuffle sums, 94 us now.
constexpr int kScanThreads = 256;
constexpr int kScanBatch = 8;

// Sum over the 64 lanes of a wave, complete in lane 63, by DPP moves (vector
// ALU only: no LDS round trip per step). Quads, then half-rows and rows by
// mirroring, then rows 1 and 3 take the last lane of the row below, and row 3
// that of row 1.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp_move(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, kRowMask, 0xF, false));
}

__device__ __forceinline__ float wave_sum_lane63(float v) {
  v += dpp_move<0xB1, 0xF>(v);   // quad_perm [1, 0, 3, 2]
  v += dpp_move<0x4E, 0xF>(v);   // quad_perm [2, 3, 0, 1]
  v += dpp_move<0x141, 0xF>(v);  // row_half_mirror
  v += dpp_move<0x140, 0xF>(v);  // row_mirror
  v += dpp_move<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_move<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

__global__ __launch_bounds__(kScanThreads) void rev_scan_kernel(
    const float *__restrict__ st, int64_t sstride, float *__restrict__ gs,
    const float *__restrict__ gamma, const float *S_in, const float *z_in, const float *dS_out,
    const float *dz_out, float *dS_in, float *dz_in, float *__restrict__ dgp, int F, int R, int d,
    int NB) {
  const int64_t dd = (int64_t)d * d;
  const int64_t E = dd + d;
  const int64_t bh = blockIdx.x / NB;
  const int blk = blockIdx.x % NB;
  const int tid = threadIdx.x;
  const int64_t e = (int64_t)blk * kScanThreads + tid;
  const bool valid = e < E;
  const bool is_S = e < dd;
  __shared__ float red[kScanBatch][kScanThreads / 64];

  float a = 0.f;  // incoming adjoint: gamma_{f+1} Sh_{f+1}
  if (valid) {
    if (is_S && dS_out) a = dS_out[bh * dd + e];
    if (!is_S && dz_out) a = dz_out[bh * d + (e - dd)];
  }
  struct Batch {
    float x[kScanBatch], prev[kScanBatch], gm[kScanBatch];
  };
  // gamma through vector loads (an opaque zero in the index): a scalar load
  // would be waited for by the next barrier's lgkmcnt(0)
  int vzero = 0;
  asm volatile("" : "+v"(vzero));
  // loads of frames fb, fb - 1, ..., fb - kScanBatch + 1
  auto load = [&](int fb, Batch &b) {
#pragma unroll
    for (int j = 0; j < kScanBatch; ++j) {
      const int f = fb - j;
      b.x[j] = 0.f;
      b.prev[j] = 0.f;
      b.gm[j] = 1.f;
      if (f >= 0 && valid) {
        const float *src = gs + ((bh * F + f) * (int64_t)R) * E + e;
        float s = src[0];
        for (int r = 1; r < R; ++r) s += src[(int64_t)r * E];
        b.x[j] = s;
        if (dgp) {
          if (f > 0)
            b.prev[j] = st[(bh * F + f - 1) * sstride + e];
          else if (is_S && S_in)
            b.prev[j] = S_in[bh * dd + e];
          else if (!is_S && z_in)
            b.prev[j] = z_in[bh * d + (e - dd)];
        }
        if (gamma) b.gm[j] = gamma[bh * F + f + vzero];
      }
    }
  };
  auto process = [&](int fb, const Batch &b) {
#pragma unroll
    for (int j = 0; j < kScanBatch; ++j) {
      const int f = fb - j;
      if (f < 0) break;
      const float sh = b.x[j] + a;
      if (valid) gs[((bh * F + f) * (int64_t)R) * E + e] = sh;
      if (dgp) {
        float pr = valid ? sh * b.prev[j] : 0.f;
        pr = wave_sum_lane63(pr);
        if ((tid & 63) == 63) red[j][tid >> 6] = pr;
      }
      a = b.gm[j] * sh;
    }
    if (dgp) {
      // LDS-only barriers: the next batch's global loads stay in flight
      sync_lds();
      if (tid < kScanBatch && fb - tid >= 0) {
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < kScanThreads / 64; ++w) sum += red[tid][w];
        dgp[(bh * F + (fb - tid)) * (int64_t)NB + blk] = sum;
      }
      sync_lds();
    }
  };
  // the next batch's loads are in flight while this one is folded in (two
  // register sets used in turn: a copy would wait for the loads)
  Batch b0, b1;
  int fb = F - 1;
  if (fb >= 0) load(fb, b0);
  while (fb >= 0) {
    if (fb - kScanBatch >= 0) load(fb - kScanBatch, b1);
    process(fb, b0);
    fb -= kScanBatch;
    if (fb < 0) break;
    if (fb - kScanBatch >= 0) load(fb - kScanBatch, b0);
    process(fb, b1);
    fb -= kScanBatch;
  }
  if (valid) {
    if (is_S && dS_in) dS_in[bh * dd + e] = a;
    if (!is_S && dz_in) dz_in[bh * d + (e - dd)] = a;
  }
}

__global__ __launch_bounds__(256) void dgamma_kernel(const float *__restrict__ dgp,
                                                     float *__restrict__ dgamma, int64_t n,
                                                     int NB) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s = 0.f;
  for (int b = 0; b < NB; ++b) s += dgp[i * NB + b];
  dgamma[i] = s;
}

template <typename TIn>
hipError_t bwd_q_valu_dispatch(const BwdPlan &bp, const BwdQArgs &a, hipStream_t s) {
  const Plan &p = bp.f;
  const int64_t grid = p.BH * p.F * p.R;
  float *gs = a.gs;
#define GLA_BQ_CASE(DD)                                                                         \
  case DD:                                                                                      \
    if (a.rope.on)                                                                              \
      hipLaunchKernelGGL((bwd_q_valu_kernel<TIn, DD, true>), dim3((unsigned)grid),              \
                         dim3(kThreads), 0, s, a.q, a.g, a.dO, a.dq, a.dg, a.H, a.st.base,       \
                         a.st.stride, gs, p.F, p.T, p.R, p.read_len, a.eps, a.state_frame,       \
                         a.rope);                                                               \
    else                                                                                        \
      hipLaunchKernelGGL((bwd_q_valu_kernel<TIn, DD, false>), dim3((unsigned)grid),             \
                         dim3(kThreads), 0, s, a.q, a.g, a.dO, a.dq, a.dg, a.H, a.st.base,       \
                         a.st.stride, gs, p.F, p.T, p.R, p.read_len, a.eps, a.state_frame,       \
                         a.rope);                                                               \
    break;
  switch (p.d) {
    GLA_BQ_CASE(16)
    GLA_BQ_CASE(32)
    GLA_BQ_CASE(64)
    GLA_BQ_CASE(128)
    default:
      return hipErrorInvalidValue;
  }
#undef GLA_BQ_CASE
  return hipGetLastError();
}

template <typename TIn>
hipError_t bwd_k_valu_dispatch(const BwdPlan &bp, const BwdKArgs &a, hipStream_t s) {
  const Plan &p = bp.f;
  const int64_t grid = p.BH * p.F * p.P;
#define GLA_BK_CASE(DD)                                                                         \
  case DD:                                                                                      \
    if (a.rope.on)                                                                              \
      hipLaunchKernelGGL((bwd_k_valu_kernel<TIn, DD, true>), dim3((unsigned)grid),              \
                         dim3(kThreads), 0, s, a.k, a.v, a.dk, a.dv, a.H, a.gs, p.F, p.T, p.P,   \
                         p.R, p.part_len, a.adj_frame, a.rope);                                 \
    else                                                                                        \
      hipLaunchKernelGGL((bwd_k_valu_kernel<TIn, DD, false>), dim3((unsigned)grid),             \
                         dim3(kThreads), 0, s, a.k, a.v, a.dk, a.dv, a.H, a.gs, p.F, p.T, p.P,   \
                         p.R, p.part_len, a.adj_frame, a.rope);                                 \
    break;
  switch (p.d) {
    GLA_BK_CASE(16)
    GLA_BK_CASE(32)
    GLA_BK_CASE(64)
    GLA_BK_CASE(128)
    default:
      return hipErrorInvalidValue;
  }
#undef GLA_BK_CASE
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_q_valu(const BwdPlan &p, int dtype, const BwdQArgs &a, hipStream_t s) {
  if (p.f.BH * p.f.F * p.f.R == 0) return hipSuccess;
  return dtype == 0 ? bwd_q_valu_dispatch<float>(p, a, s) : bwd_q_valu_dispatch<bf16_t>(p, a, s);
}

hipError_t launch_bwd_k_valu(const BwdPlan &p, int dtype, const BwdKArgs &a, hipStream_t s) {
  if (p.f.BH * p.f.F * p.f.P == 0 || p.f.T == 0) return hipSuccess;
  return dtype == 0 ? bwd_k_valu_dispatch<float>(p, a, s) : bwd_k_valu_dispatch<bf16_t>(p, a, s);
}

hipError_t launch_rev_scan(const BwdPlan &p, const RevScanArgs &a, hipStream_t s) {
  const int64_t grid = p.f.BH * p.NB;
  if (grid == 0) return hipSuccess;  // F == 0 still runs: dS_in = dS_out
  hipLaunchKernelGGL(rev_scan_kernel, dim3((unsigned)grid), dim3(kScanThreads), 0, s, a.st.base,
                     a.st.stride, a.gs, a.gamma, a.S_in, a.z_in, a.dS_out, a.dz_out, a.dS_in,
                     a.dz_in, a.dgp, p.f.F, p.f.R, p.f.d, p.NB);
  return hipGetLastError();
}

hipError_t launch_dgamma(const BwdPlan &p, const float *dgp, float *dgamma, hipStream_t s) {
  const int64_t n = p.f.BH * p.f.F;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(dgamma_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, dgp,
                     dgamma, n, p.NB);
  return hipGetLastError();
}

}  // namespace gla
