// gdn_mfma.hip -- bf16 matrix-core (MFMA) kernels of the frame-wise Gated
// DeltaNet for gfx950: the frame sums and the readout.
//
//   kv:      U_f = (beta K)^T V and A_f = (beta K)^T K over a part of frame f
//            (d x C times C x d, tokens as the contraction)
//   scan:    S_f = gamma_f (S_{f-1} - c^2 A_f S_{f-1}) + c U_f, the product
//            A_f S_{f-1} on the matrix cores, the state in registers
//   readout: o^T = S_f^T Q^T (d x d times d x C)
//
// beta * k is an fp32 product; it enters the MFMA as hi + lo with both parts
// bf16 (hi = bf16(x), lo = bf16(x - hi)), so the sums keep ~16 significant
// bits of beta k against the exact bf16 v and k. The fp32 state S_f enters the
// readout split the same way. Accumulation is fp32 throughout.
//
// (MFMA operand layouts and the transposed LDS reads: mfma_util.hpp.)
#include "common.hpp"
#include "mfma_util.hpp"
#include "plan.hpp"

namespace gla {
namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------------------
// Frame sums U_f, A_f
// ---------------------------------------------------------------------------
template <int D>
struct GkCfg {
  static constexpr int CH = 64;             // tokens per LDS chunk (4 k-steps of 16)
  static constexpr int PITCH = 2 * D + 32;  // bytes per LDS row
  static constexpr int MB = D / 32;         // 32 x 32 blocks per side of U and A
  // D = 32: each wave runs one k-step of every chunk and the four partial sums
  // meet in LDS at the end. D >= 64: the blocks are split 2 x 2 over the waves,
  // every wave runs every k-step and owns its blocks of U and A outright.
  static constexpr bool kSplitTokens = (D == 32);
  static constexpr int TM = kSplitTokens ? MB : MB / 2;
  static constexpr int ROW_CHUNKS = D / 8;                // 16-byte pieces per row
  static constexpr int CPT = CH * ROW_CHUNKS / kThreads;  // pieces per thread per array
  static constexpr int ROWS_PER_PASS = kThreads / ROW_CHUNKS;
  static constexpr int TILE_BYTES = CH * PITCH;
  // tiles: beta k (hi), beta k (lo), k, v
  static constexpr int RED_BYTES = kSplitTokens ? 4 * 2 * 1024 * 4 : 0;  // 4 waves x (U, A)
  static constexpr int SMEM = 4 * TILE_BYTES > RED_BYTES ? 4 * TILE_BYTES : RED_BYTES;
};

// One workgroup per (slab, frame, part); the slot of (slab, frame, part)
// receives U (d x d, row = key feature) and then A.
template <int D>
__global__ __launch_bounds__(kThreads) void gdn_kv_mfma_kernel(View kview, View vview, int H,
                                                               const float *__restrict__ beta,
                                                               float *__restrict__ ws, int F,
                                                               int64_t T, int P,
                                                               int64_t part_len) {
  using C = GkCfg<D>;
  __shared__ __attribute__((aligned(16))) char smem[C::SMEM];
  lds_char *const sbase = (lds_char *)smem;
  lds_char *const tbh = sbase;
  lds_char *const tbl = sbase + C::TILE_BYTES;
  lds_char *const tk = sbase + 2 * C::TILE_BYTES;
  lds_char *const tv = sbase + 3 * C::TILE_BYTES;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t wg = blockIdx.x;
  const int p = (int)(wg % P);
  const int f = (int)((wg / P) % F);
  const int64_t bh = wg / ((int64_t)P * F);
  const int64_t N = (int64_t)F * T;
  const int64_t t0 = min((int64_t)p * part_len, T);
  const int64_t t1 = min(t0 + part_len, T);
  const int L = (int)(t1 - t0);
  const int ncf = (L + C::CH - 1) / C::CH;
  const int64_t row0 = (int64_t)f * T + t0;

  // row strides in 16-byte pieces (host-checked multiples of 8 elements)
  const int64_t snk = kview.sn / 8, snv = vview.sn / 8;
  const int c = tid % C::ROW_CHUNKS;
  const int r0 = tid / C::ROW_CHUNKS;
  const uint4 *kp = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(kview.data) +
                                                    kview.slab(bh, H) + row0 * kview.sn) +
                    (int64_t)r0 * snk + c;
  const uint4 *vp = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(vview.data) +
                                                    vview.slab(bh, H) + row0 * vview.sn) +
                    (int64_t)r0 * snv + c;
  const float *bp = beta + bh * N + row0 + r0;
  const int64_t k_pass = C::ROWS_PER_PASS * snk, v_pass = C::ROWS_PER_PASS * snv;

  uint4 rk[C::CPT], rv[C::CPT];
  float rb[C::CPT];
  int lcc = 0;
  auto load = [&]() {
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int row = lcc * C::CH + r0 + i * C::ROWS_PER_PASS;
      if (row < L) {
        rk[i] = ld_stream16<true>(kp + i * k_pass);
        rv[i] = ld_stream16<true>(vp + i * v_pass);
        rb[i] = bp[i * C::ROWS_PER_PASS];
      } else {
        rk[i] = rv[i] = make_uint4(0, 0, 0, 0);
        rb[i] = 0.f;
      }
    }
    ++lcc;
    kp += C::CH * snk;
    vp += C::CH * snv;
    bp += C::CH;
  };

  f32x16 au[C::TM][C::TM], aa[C::TM][C::TM];
#pragma unroll
  for (int a = 0; a < C::TM; ++a)
#pragma unroll
    for (int b = 0; b < C::TM; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) au[a][b][r] = aa[a][b][r] = 0.f;

  // lane geometry of the transposed fragment reads
  const int h = lane >> 5;
  const int j = lane & 15;
  const int frag_row = 8 * h + (j >> 2);
  const int frag_col = 16 * ((lane >> 4) & 1) + 4 * (j & 3);
  const int wm = C::kSplitTokens ? 0 : (wave >> 1);
  const int wn = C::kSplitTokens ? 0 : (wave & 1);

  if (ncf > 0) load();
  for (int cc = 0; cc < ncf; ++cc) {
    sync_lds();  // the previous chunk's fragment reads are done
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int off = (r0 + i * C::ROWS_PER_PASS) * C::PITCH + c * 16;
      const uint32_t kw[4] = {rk[i].x, rk[i].y, rk[i].z, rk[i].w};
      uint32_t hv[4], lv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) split2(rb[i] * lo_bf16(kw[e]), rb[i] * hi_bf16(kw[e]), hv[e], lv[e]);
      *reinterpret_cast<uint4 *>(smem + off) = make_uint4(hv[0], hv[1], hv[2], hv[3]);
      *reinterpret_cast<uint4 *>(smem + C::TILE_BYTES + off) = make_uint4(lv[0], lv[1], lv[2], lv[3]);
      *reinterpret_cast<uint4 *>(smem + 2 * C::TILE_BYTES + off) = rk[i];
      *reinterpret_cast<uint4 *>(smem + 3 * C::TILE_BYTES + off) = rv[i];
    }
    sync_lds();
    if (cc + 1 < ncf) load();

    constexpr int KS_PER_WAVE = C::kSplitTokens ? 1 : 4;
#pragma unroll
    for (int kk = 0; kk < KS_PER_WAVE; ++kk) {
      const int ks = C::kSplitTokens ? wave : kk;
      const int rr = ks * 16 + frag_row;
      bf16x8 fh[C::TM], fl[C::TM], fv[C::TM], fk[C::TM];
#pragma unroll
      for (int a = 0; a < C::TM; ++a) {
        const int ca = 32 * (wm * C::TM + a) + frag_col;
        const int cb = 32 * (wn * C::TM + a) + frag_col;
        fh[a] = tr_fragment(tbh, rr, ca, C::PITCH);
        fl[a] = tr_fragment(tbl, rr, ca, C::PITCH);
        fv[a] = tr_fragment(tv, rr, cb, C::PITCH);
        fk[a] = tr_fragment(tk, rr, cb, C::PITCH);
      }
#pragma unroll
      for (int a = 0; a < C::TM; ++a)
#pragma unroll
        for (int b = 0; b < C::TM; ++b) {
          au[a][b] = mfma_32x32x16(fh[a], fv[b], au[a][b]);
          au[a][b] = mfma_32x32x16(fl[a], fv[b], au[a][b]);
          aa[a][b] = mfma_32x32x16(fh[a], fk[b], aa[a][b]);
          aa[a][b] = mfma_32x32x16(fl[a], fk[b], aa[a][b]);
        }
    }
  }

  float *out = ws + ((bh * F + f) * (int64_t)P + p) * (2 * (int64_t)D * D);
  if constexpr (C::kSplitTokens) {
    // the four waves' partial sums of the single block pair, through LDS
    float *red = (float *)smem;  // [wave][U | A][r][lane], aliases the tiles
    sync_lds();
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      red[wave * 2048 + r * 64 + lane] = au[0][0][r];
      red[wave * 2048 + 1024 + r * 64 + lane] = aa[0][0][r];
    }
    sync_lds();
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const int idx = tid + kThreads * x;  // (U | A, r, lane)
      const int which = idx >> 10, rl = idx & 1023;
      const float sum = red[idx] + red[2048 + idx] + red[4096 + idx] + red[6144 + idx];
      const int r = rl >> 6, ln = rl & 63;
      const int m = 8 * (r >> 2) + 4 * (ln >> 5) + (r & 3);
      out[which * D * D + m * D + (ln & 31)] = sum;
    }
  } else {
#pragma unroll
    for (int a = 0; a < C::TM; ++a)
#pragma unroll
      for (int b = 0; b < C::TM; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = 8 * (r >> 2) + 4 * h + (r & 3);
          const int idx = (32 * (wm * C::TM + a) + m) * D + 32 * (wn * C::TM + b) + (lane & 31);
          out[idx] = au[a][b][r];
          out[D * D + idx] = aa[a][b][r];
        }
  }
}

// ---------------------------------------------------------------------------
// Readout o = S_f^T q
// ---------------------------------------------------------------------------
template <int D>
struct GrCfg {
  static constexpr int MB = D / 32;         // 32-feature output blocks
  static constexpr int TG = 4 / MB;         // token groups of 32 across the waves
  static constexpr int BLK = 32 * TG;       // tokens per iteration
  static constexpr int KS = D / 16;         // k-steps over the input features
  static constexpr int PITCH = 2 * D + 16;  // bytes per LDS row of q and of o
  static constexpr int ROW_CHUNKS = D / 8;
  static constexpr int CPT = BLK * ROW_CHUNKS / kThreads;
  static constexpr int ROWS_PER_PASS = kThreads / ROW_CHUNKS;
};

// One workgroup per (slab, frame, split). q rows are staged in LDS (16-byte
// loads covering whole rows), read there as B fragments; o is gathered in LDS
// from the accumulator layout and written back as whole rows.
template <int D>
__global__ __launch_bounds__(kThreads) void gdn_readout_mfma_kernel(
    View qview, View oview, int H, const float *__restrict__ ws, int F, int64_t T, int P, int R,
    int64_t read_len) {
  using C = GrCfg<D>;
  __shared__ __attribute__((aligned(16))) char qtile[C::BLK * C::PITCH];
  __shared__ __attribute__((aligned(16))) char otile[C::BLK * C::PITCH];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;
  const int mb = wave % C::MB;
  const int tg = wave / C::MB;
  const int64_t wg = blockIdx.x;
  const int r = (int)(wg % R);
  const int f = (int)((wg / R) % F);
  const int64_t bh = wg / ((int64_t)R * F);
  const int64_t t0 = min((int64_t)r * read_len, T);
  const int64_t t1 = min(t0 + read_len, T);
  const int L = (int)(t1 - t0);
  if (L <= 0) return;
  const int64_t trow0 = (int64_t)f * T + t0;

  bf16x8 ahi[C::KS], alo[C::KS];
  frag_transposed<D>(ws + ((bh * F + f) * (int64_t)P) * (2 * (int64_t)D * D), mb, lane, ahi, alo);

  const int c = tid % C::ROW_CHUNKS;
  const int r0 = tid / C::ROW_CHUNKS;
  const int64_t snq = qview.sn / 8, sno = oview.sn / 8;
  const uint4 *qp = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(qview.data) +
                                                    qview.slab(bh, H) + trow0 * qview.sn) +
                    (int64_t)r0 * snq + c;
  uint4 *op = reinterpret_cast<uint4 *>(const_cast<uint16_t *>(
                  static_cast<const uint16_t *>(oview.data) + oview.slab(bh, H) +
                  trow0 * oview.sn)) +
              (int64_t)r0 * sno + c;
  uint4 rq[C::CPT];
  // Rows past the split load (and later store) its last row again: each o row
  // depends on its own q row alone, and a row stored twice gets the same
  // value. Without branches the compiler can count these loads and stores,
  // and waits for the loads alone (the counter covers both).
  auto load = [&](int blk) {
    const int last = L - 1 - blk * C::BLK;  // the block's last row, >= 0
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int64_t row = min(r0 + i * C::ROWS_PER_PASS, last) - r0;
      rq[i] = ld_stream16<true>(qp + row * snq);
    }
    qp += C::BLK * snq;
  };

  const int tl = 32 * tg + (lane & 31);
  const int nblk = (L + C::BLK - 1) / C::BLK;
  load(0);
  wait_vmem_all();  // no load outstanding into the loop: its waits count its own
  for (int blk = 0; blk < nblk; ++blk) {
    sync_lds();  // the previous block's q fragments and o rows have been read
#pragma unroll
    for (int i = 0; i < C::CPT; ++i)
      *reinterpret_cast<uint4 *>(qtile + (r0 + i * C::ROWS_PER_PASS) * C::PITCH + c * 16) = rq[i];
    sync_lds();
    if (blk + 1 < nblk) load(blk + 1);

    f32x16 acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const bf16x8 bf = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const uint4 *>(qtile + tl * C::PITCH + (16 * ks + 8 * h) * 2));
      acc = mfma_32x32x16(ahi[ks], bf, acc);
      acc = mfma_32x32x16(alo[ks], bf, acc);
    }
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      uint2 ow;
      ow.x = pack_bf16x2(acc[4 * rg + 0], acc[4 * rg + 1]);
      ow.y = pack_bf16x2(acc[4 * rg + 2], acc[4 * rg + 3]);
      *reinterpret_cast<uint2 *>(otile + tl * C::PITCH + (32 * mb + 8 * rg + 4 * h) * 2) = ow;
    }
    sync_lds();
    {
      const int last = L - 1 - blk * C::BLK;
#pragma unroll
      for (int i = 0; i < C::CPT; ++i) {
        const int row = min(r0 + i * C::ROWS_PER_PASS, last);
        st_stream16(op + (int64_t)(row - r0) * sno,
                    *reinterpret_cast<const uint4 *>(otile + row * C::PITCH + c * 16));
      }
    }
    op += C::BLK * sno;
  }
}

// ---------------------------------------------------------------------------
// Scan S_f = gamma_f (S_{f-1} - c^2 A_f S_{f-1}) + c U_f
//
// The per-frame product A_f S_{f-1} (d x d times d x d) runs on the 16x16x32
// MFMA with both factors split into bf16 hi + lo parts (hi*hi + hi*lo + lo*hi:
// the dropped lo*lo term is below 2^-16 of the product); the update itself is
// fp32. Each wave owns 16 columns of S for all d rows and keeps them in
// registers in the accumulator layout: for row block ib, lane l (g = l / 16)
// holds S[16 ib + 4g + r][j0 + l % 16], r = 0..3. Relabelling the contraction
// index, the B operand of k-step ks (state rows 32 ks .. 32 ks + 31) is made
// of the lane's own values: slot e < 4 is row 32 ks + 4g + e and slot e >= 4
// row 32 ks + 16 + 4g + (e - 4). A_f is staged per frame in LDS as bf16 hi and
// lo planes whose 32-column blocks are permuted into that same order, so the
// eight values of a lane's A operand are one 16-byte read.
// ---------------------------------------------------------------------------
template <int D>
struct GsCfg {
  static constexpr int NW = D >= 64 ? 4 : D / 16;     // waves per workgroup
  static constexpr int THREADS = 64 * NW;
  static constexpr int NWG = D / (16 * NW);           // workgroups per slab
  static constexpr int RB = D / 16;                   // 16-row blocks of the state
  static constexpr int KS = D / 32;                   // k-steps of 32 rows
  static constexpr int PITCH = 2 * D + 16;            // bytes per LDS row of a plane
  static constexpr int APT = D * D / (4 * THREADS);   // float4 pieces of A_f per thread
  // frames loaded ahead (at d = 128 a second buffer would not fit beside the
  // state in registers)
#ifdef GLA_SCAN_AHEAD
  static constexpr int AHEAD = D == 128 ? 1 : GLA_SCAN_AHEAD;
#else
  static constexpr int AHEAD = D == 128 ? 1 : 2;
#endif
};

// LDS position (in elements) of column col of a plane row
__device__ __forceinline__ int scan_perm(int col) {
  const int c32 = col & 31;
  return (col & ~31) + 8 * ((c32 & 15) >> 2) + 4 * (c32 >> 4) + (c32 & 3);
}

// The scan runs in one of four modes, each a sequence of steps
//   X <- g0 X + g1 (A X) + g2 U     (A d x d; X, U d x ncols)
// with X kept in registers as above:
//   kWhole:    one pass over the F frames of a slab: A = A_f, U = U_f,
//              (g0, g1, g2) = (gamma_f, -gamma_f c^2, c); S_f stored after each step.
//   kTransfer: per chunk of frames, from [0 | I] on d x 2d columns: the chunk's
//              local end state (left d columns) and its transfer matrix
//              M = prod_f gamma_f (I - c^2 A_f) (right d columns, U = 0).
//   kChain:    per slab, over the chunks in order: A = M_c, U = L_c (the local
//              end state), (g0, g1, g2) = (0, 1, 1); X before each step is the
//              chunk's start state.
//   kApply:    per chunk, kWhole's steps from the chunk's start state.
// The chunked form cuts the chain of dependent steps from F to about
// 2 Fc + F / Fc; the products are the same matrix-core steps.
enum ScanMode { kWhole = 0, kTransfer = 1, kChain = 2, kApply = 3 };

template <int D, int kMode>
struct ScanJob {
  static constexpr int AHEAD = kMode == kWhole ? GsCfg<D>::AHEAD : 1;
  static constexpr int COLS = kMode == kTransfer ? 2 * D : D;
  // At d <= 64 the transfer's d x 2d columns go to twice the waves rather
  // than to twice the workgroups: every workgroup stages each frame's A from
  // HBM, so one workgroup per chunk reads it once (720p/60s: 379 -> 253 MB).
  // At d = 128, 8 waves of 128 rows would spill; it keeps two workgroups.
#ifndef GLA_SCAN_WIDE_TRANSFER
#define GLA_SCAN_WIDE_TRANSFER 1
#endif
  static constexpr int NW = (kMode == kTransfer && GLA_SCAN_WIDE_TRANSFER && D <= 64)
                                ? 2 * GsCfg<D>::NW
                                : GsCfg<D>::NW;
  static constexpr int THREADS = 64 * NW;
  static constexpr int APT = D * D / (4 * THREADS);  // float4 pieces of A_f per thread
  static constexpr int NWG = COLS / (16 * NW);       // workgroups per item
};

template <int D, int kMode>
__global__ __launch_bounds__((ScanJob<D, kMode>::THREADS)) void gdn_scan_mfma_kernel(
    float *__restrict__ ws, const float *__restrict__ gamma, const float *S_in, float *S_out,
    int F, int P, float key_scale, int Fc, int nc, float *__restrict__ tws,
    float *__restrict__ sws) {
  using C = GsCfg<D>;
  using J = ScanJob<D, kMode>;
  __shared__ __attribute__((aligned(16))) char planes[2 * D * C::PITCH];  // hi, then lo
  constexpr int64_t SLOT = 2 * (int64_t)D * D;
  constexpr int64_t DD = (int64_t)D * D;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4, n = lane & 15;
  const int cb = (int)(blockIdx.x % J::NWG);
  const int64_t item = blockIdx.x / J::NWG;
  const bool per_chunk = kMode == kTransfer || kMode == kApply;
  const int64_t bh = per_chunk ? item / nc : item;
  const int chunk = per_chunk ? (int)(item % nc) : 0;
  const int f0 = per_chunk ? chunk * Fc : 0;
  const int nsteps = kMode == kChain ? nc : (per_chunk ? min(Fc, F - f0) : F);
  const int cx = 16 * (cb * J::NW + wave) + n;  // the lane's column of X (< COLS)
  const bool right = kMode == kTransfer && cx >= D;  // a column of the transfer matrix
  const int col = cx % D;                            // its column within a d x d matrix
  const float c1 = key_scale, c2 = key_scale * key_scale;
  float *slab = ws + bh * (int64_t)F * P * SLOT;  // part 0 of each frame holds the whole sums
  float *tw = tws + bh * (int64_t)nc * 2 * DD;    // per chunk: L_c, then M_c
  float *sw = sws + bh * (int64_t)nc * DD;        // per chunk: its start state

  f32x4 s[C::RB];
#pragma unroll
  for (int ib = 0; ib < C::RB; ++ib)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * ib + 4 * g + r;
      float x = 0.f;
      if constexpr (kMode == kWhole || kMode == kChain) {
        if (S_in) x = S_in[bh * DD + row * D + col];
      } else if constexpr (kMode == kTransfer) {
        x = right && row == col ? 1.f : 0.f;
      } else {
        x = sw[(int64_t)chunk * DD + row * D + col];
      }
      s[ib][r] = x;
    }

  // a step's A (this thread's pieces), U (the lane's values) and gamma
  struct Frame {
    float4 a[J::APT];
    f32x4 u[C::RB];
    float g;
  };
  // gamma_f goes through a vector load (an address the compiler cannot prove
  // uniform): a scalar load would be waited for by the next LDS barrier
  // (lgkmcnt(0)), a few instructions after its issue
  int vzero = 0;
  asm volatile("" : "+v"(vzero));
  auto load_step = [&](int t, Frame &b) {
    const float *amat, *umat;
    if constexpr (kMode == kChain) {
      umat = tw + (int64_t)t * 2 * DD;
      amat = umat + DD;
    } else {
      umat = slab + (int64_t)(f0 + t) * P * SLOT;
      amat = umat + DD;
    }
#pragma unroll
    for (int it = 0; it < J::APT; ++it) {
      const int x = tid + J::THREADS * it;
      b.a[it] = *reinterpret_cast<const float4 *>(amat + (x / (D / 4)) * D + 4 * (x % (D / 4)));
    }
#pragma unroll
    for (int ib = 0; ib < C::RB; ++ib)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        b.u[ib][r] = right ? 0.f : umat[(16 * ib + 4 * g + r) * D + col];
    if constexpr (kMode != kChain) b.g = gamma[bh * F + f0 + t + vzero];
  };

  // step t from the loaded buffer b, which then receives step t_next
  auto step = [&](int t, Frame &b, int t_next) {
    sync_lds();  // the previous step's A reads are done
#pragma unroll
    for (int it = 0; it < J::APT; ++it) {
      const int x = tid + J::THREADS * it;
      const int off = (x / (D / 4)) * C::PITCH + 2 * scan_perm(4 * (x % (D / 4)));
      uint32_t h0, l0, h1, l1;
      split2(b.a[it].x, b.a[it].y, h0, l0);
      split2(b.a[it].z, b.a[it].w, h1, l1);
      *reinterpret_cast<uint2 *>(planes + off) = make_uint2(h0, h1);
      *reinterpret_cast<uint2 *>(planes + D * C::PITCH + off) = make_uint2(l0, l1);
    }
    f32x4 u[C::RB];
#pragma unroll
    for (int ib = 0; ib < C::RB; ++ib) u[ib] = b.u[ib];
    const float gm = kMode == kChain ? 0.f : b.g;
    sync_lds();
    if (t_next < nsteps) load_step(t_next, b);
    if constexpr (kMode == kChain) {
      // the chunk's start state, before its step
#pragma unroll
      for (int ib = 0; ib < C::RB; ++ib)
#pragma unroll
        for (int r = 0; r < 4; ++r) sw[(int64_t)t * DD + (16 * ib + 4 * g + r) * D + col] = s[ib][r];
    }

    f32x4 acc[C::RB];
#pragma unroll
    for (int ib = 0; ib < C::RB; ++ib) acc[ib] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      uint32_t bh4[4], bl4[4];
      split2(s[2 * ks][0], s[2 * ks][1], bh4[0], bl4[0]);
      split2(s[2 * ks][2], s[2 * ks][3], bh4[1], bl4[1]);
      split2(s[2 * ks + 1][0], s[2 * ks + 1][1], bh4[2], bl4[2]);
      split2(s[2 * ks + 1][2], s[2 * ks + 1][3], bh4[3], bl4[3]);
      const bf16x8 bhi = __builtin_bit_cast(bf16x8, make_uint4(bh4[0], bh4[1], bh4[2], bh4[3]));
      const bf16x8 blo = __builtin_bit_cast(bf16x8, make_uint4(bl4[0], bl4[1], bl4[2], bl4[3]));
      bf16x8 ahi[C::RB], alo[C::RB];
#pragma unroll
      for (int ib = 0; ib < C::RB; ++ib) {
        const int off = (16 * ib + n) * C::PITCH + (32 * ks + 8 * g) * 2;
        ahi[ib] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(planes + off));
        alo[ib] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const uint4 *>(planes + D * C::PITCH + off));
      }
#pragma unroll
      for (int ib = 0; ib < C::RB; ++ib) acc[ib] = mfma_16x16x32(ahi[ib], bhi, acc[ib]);
#pragma unroll
      for (int ib = 0; ib < C::RB; ++ib) acc[ib] = mfma_16x16x32(ahi[ib], blo, acc[ib]);
#pragma unroll
      for (int ib = 0; ib < C::RB; ++ib) acc[ib] = mfma_16x16x32(alo[ib], bhi, acc[ib]);
    }
    float *dst = slab + (int64_t)(f0 + t) * P * SLOT;  // S_f, over part 0's U
#pragma unroll
    for (int ib = 0; ib < C::RB; ++ib)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (kMode == kChain) {
          s[ib][r] = acc[ib][r] + u[ib][r];
        } else {
          s[ib][r] = fmaf(gm, fmaf(-c2, acc[ib][r], s[ib][r]), c1 * u[ib][r]);
          if constexpr (kMode != kTransfer) dst[(16 * ib + 4 * g + r) * D + col] = s[ib][r];
        }
      }
  };

  // AHEAD steps in flight: step t + AHEAD is requested as step t is staged
  Frame buf[J::AHEAD];
#pragma unroll
  for (int i = 0; i < J::AHEAD; ++i)
    if (i < nsteps) load_step(i, buf[i]);
  for (int t = 0; t < nsteps; t += J::AHEAD) {
#pragma unroll
    for (int i = 0; i < J::AHEAD; ++i)
      if (t + i < nsteps) step(t + i, buf[i], t + i + J::AHEAD);
  }
  float *fin = nullptr;  // where the final state goes
  if constexpr (kMode == kWhole) fin = S_out ? S_out + bh * DD : nullptr;
  if constexpr (kMode == kApply) fin = (S_out && chunk == nc - 1) ? S_out + bh * DD : nullptr;
  if constexpr (kMode == kTransfer) fin = tw + ((int64_t)chunk * 2 + (right ? 1 : 0)) * DD;
  if (fin) {
#pragma unroll
    for (int ib = 0; ib < C::RB; ++ib)
#pragma unroll
      for (int r = 0; r < 4; ++r) fin[(16 * ib + 4 * g + r) * D + col] = s[ib][r];
  }
}

// Sums the P parts of every (slab, frame) slot into part 0, one float4 per
// thread, the parts added in order.
__global__ __launch_bounds__(kThreads) void gdn_sum_parts_kernel(float *__restrict__ ws,
                                                                 int64_t slots, int P, int E4) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= slots * E4) return;
  const int64_t slot = i / E4, e = i - slot * E4;
  float4 *w = reinterpret_cast<float4 *>(ws) + slot * P * E4 + e;
  float4 a = w[0];
  for (int p = 1; p < P; ++p) {
    const float4 b = w[p * (int64_t)E4];
    a.x += b.x;
    a.y += b.y;
    a.z += b.z;
    a.w += b.w;
  }
  w[0] = a;
}

template <int D, int kMode>
void gdn_scan_run(const Plan &p, const GdnScanArgs &a, int64_t items, hipStream_t s) {
  float *tws = a.ws + p.scan_tws, *sws = a.ws + p.scan_sws;
  hipLaunchKernelGGL((gdn_scan_mfma_kernel<D, kMode>),
                     dim3((unsigned)(items * ScanJob<D, kMode>::NWG)),
                     dim3(ScanJob<D, kMode>::THREADS), 0, s,
                     a.ws, a.gamma, a.S_in, a.S_out, p.F, p.P, a.key_scale, p.scan_fc, p.scan_nc,
                     tws, sws);
}

template <int D>
void gdn_scan_launch(const Plan &p, const GdnScanArgs &a, hipStream_t s) {
  if (p.P > 1) {
    const int64_t slots = p.BH * p.F, E4 = (int64_t)D * D / 2;
    hipLaunchKernelGGL(gdn_sum_parts_kernel, dim3((unsigned)((slots * E4 + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, s, a.ws, slots, p.P, (int)E4);
  }
  if (p.scan_nc > 1) {  // chunks of frames: transfer, chain, apply
    gdn_scan_run<D, kTransfer>(p, a, p.BH * p.scan_nc, s);
    gdn_scan_run<D, kChain>(p, a, p.BH, s);
    gdn_scan_run<D, kApply>(p, a, p.BH * p.scan_nc, s);
  } else {
    gdn_scan_run<D, kWhole>(p, a, p.BH, s);
  }
}

template <int D>
void gdn_kv_launch(const Plan &p, const GdnKvArgs &a, hipStream_t s) {
  hipLaunchKernelGGL((gdn_kv_mfma_kernel<D>), dim3((unsigned)(p.BH * p.F * p.P)), dim3(kThreads),
                     0, s, a.k, a.v, a.H, a.beta, a.ws, p.F, p.T, p.P, p.part_len);
}

template <int D>
void gdn_readout_launch(const Plan &p, const GdnReadoutArgs &a, hipStream_t s) {
  hipLaunchKernelGGL((gdn_readout_mfma_kernel<D>), dim3((unsigned)(p.BH * p.F * p.R)),
                     dim3(kThreads), 0, s, a.q, a.o, a.H, a.ws, p.F, p.T, p.P, p.R, p.read_len);
}

}  // namespace

hipError_t launch_gdn_kv_mfma(const Plan &p, const GdnKvArgs &a, hipStream_t s) {
  if (p.BH * p.F * p.P == 0) return hipSuccess;
  switch (p.d) {
    case 32: gdn_kv_launch<32>(p, a, s); break;
    case 64: gdn_kv_launch<64>(p, a, s); break;
    case 128: gdn_kv_launch<128>(p, a, s); break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gdn_scan_mfma(const Plan &p, const GdnScanArgs &a, hipStream_t s) {
  if (p.BH == 0) return hipSuccess;
  switch (p.d) {
    case 32: gdn_scan_launch<32>(p, a, s); break;
    case 64: gdn_scan_launch<64>(p, a, s); break;
    case 128: gdn_scan_launch<128>(p, a, s); break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gdn_readout_mfma(const Plan &p, const GdnReadoutArgs &a, hipStream_t s) {
  if (p.BH * p.F * p.R == 0 || p.T == 0) return hipSuccess;
  switch (p.d) {
    case 32: gdn_readout_launch<32>(p, a, s); break;
    case 64: gdn_readout_launch<64>(p, a, s); break;
    case 128: gdn_readout_launch<128>(p, a, s); break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace gla
