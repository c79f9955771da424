// bwd_mfma.hip -- bf16 matrix-core (MFMA) kernels of the backward pass (gfx950).
//
// Key side, per (slab, frame, part), with Sh_f, zh_f the adjoints of the
// frame's state (fp32, split into bf16 hi + lo as the forward readout does
// with S_f):
//   dv^T = Sh_f^T phi(K)^T                    (d x d times d x C)
//   dk^T = [K > 0]^T (.) (Sh_f V^T + zh_f)    (d x d times d x C)
// Query side, per (slab, frame, split):
//   num^T = S_f^T phi(Q)^T, den = phi(Q) z_f       (the forward readout again)
//   dg = dO (.) h (.) sigmoid'(g), dnum = dO (.) sigmoid(g) / (den + eps),
//   dden = -((dO (.) sigmoid(g)) . h) / (den + eps)     with h = num / (den + eps)
//   dq^T = [Q > 0]^T (.) (S_f dnum^T + z_f dden^T)
//   G += phi(Q)^T dnum, gz += phi(Q)^T dden     (the split's share of Sh_f, zh_f)
// dnum is fp32; it enters the matrix cores as a bf16 hi + lo pair.
#include "common.hpp"
#include "mfma_util.hpp"
#include "plan.hpp"
#include "rope_tab.hpp"

namespace gla {
namespace {

// ---------------------------------------------------------------------------
// Key side: one workgroup of 8 waves per (slab, frame, part). The 2 MB
// (role, feature block) pairs -- role dv (A = Sh^T) or dk (A = Sh) -- are
// spread over the waves, WPP = 8 / (2 MB) waves per pair, each wave taking 32
// of the block's BLK = 32 WPP tokens: a wave holds one set of A fragments.
// k and v rows are staged in LDS (phi(k) and v, the B operands); the outputs
// go back through LDS as whole rows.
// kRope (3D rotary positions): dv = Sh^T R phi(k) takes the turned phi(k) as
// bf16 hi + lo B operands (hi x hi, lo x hi, hi x lo), and dk's rows (a lane
// holds both features of a pair) turn back by R^T before zh is added; phi(k)
// unturned stays staged for the ReLU mask. The turns come from an LDS table
// filled for the workgroup's frame.
// ---------------------------------------------------------------------------
constexpr int kBwThreads = 512;

template <int D>
struct BkCfg {
  static constexpr int MB = D / 32;
  static constexpr int WPP = 8 / (2 * MB);     // waves per (role, block) pair
  static constexpr int BLK = 32 * WPP;         // tokens per iteration
  static constexpr int KS = D / 16;
  static constexpr int PITCH = 2 * D + 16;
  static constexpr int ROW_CHUNKS = D / 8;
  static constexpr int CPT = BLK * ROW_CHUNKS / kBwThreads;  // 16-byte pieces per thread
  static constexpr int ROWS_PER_PASS = kBwThreads / ROW_CHUNKS;
};

// Waves per SIMD bwd_k is held to: 4 (128 registers) at d = 128 without
// rotary positions, so that two of its 8-wave workgroups share a CU (136
// registers left it one)
template <int D, bool kRope>
constexpr int kBkWaves = (D == 128 && !kRope) ? 4 : 1;

template <int D, bool kRope>
__global__ __launch_bounds__(kBwThreads)
__attribute__((amdgpu_waves_per_eu(kBkWaves<D, kRope>))) void bwd_k_mfma_kernel(
    View kview, View vview, View dkview, View dvview, int H, const float *__restrict__ gs, int F,
    int64_t T, int P, int R, int64_t part_len, int adj_frame, RopeK rope) {
  using C = BkCfg<D>;
  static_assert(C::CPT >= 1, "tile too small for the workgroup");
  constexpr int kTurnBytes = kRope ? C::BLK * C::PITCH : 16;
  __shared__ __attribute__((aligned(16))) char ktile[C::BLK * C::PITCH];
  __shared__ __attribute__((aligned(16))) char vtile[C::BLK * C::PITCH];
  __shared__ __attribute__((aligned(16))) char dktile[C::BLK * C::PITCH];
  __shared__ __attribute__((aligned(16))) char dvtile[C::BLK * C::PITCH];
  __shared__ __attribute__((aligned(16))) char khtile[kTurnBytes];  // kRope: turned phi(k), hi
  __shared__ __attribute__((aligned(16))) char kltile[kTurnBytes];  // kRope: turned phi(k), lo
  __shared__ float szh[D];
  extern __shared__ float2 rope_tab[];  // kRope: RopeK::entries() turns, one frame

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;
  const int pair = wave / C::WPP;
  const int tg = wave % C::WPP;
  const bool role_dk = pair >= C::MB;
  const int mb = pair % C::MB;
  const int64_t wg = blockIdx.x;
  const int p = (int)(wg % P);
  const int f = (int)((wg / P) % F);
  const int64_t bh = wg / ((int64_t)P * F);
  const int64_t t0 = min((int64_t)p * part_len, T);
  const int64_t t1 = min(t0 + part_len, T);
  const int L = (int)(t1 - t0);
  if (L <= 0) return;

  constexpr int64_t E = (int64_t)D * D + D;
  const float *Sh = gs + ((bh * F + (adj_frame >= 0 ? adj_frame : f)) * (int64_t)R) * E;
  if (tid < D) szh[tid] = Sh[D * D + tid];
  if constexpr (kRope) fill_rope_table(rope_tab, rope, f);  // read after the loop's first barrier
  bf16x8 ahi[C::KS], alo[C::KS];
  if (role_dk)
    frag_direct<D>(Sh, mb, lane, ahi, alo);
  else
    frag_transposed<D>(Sh, mb, lane, ahi, alo);

  const int c = tid % C::ROW_CHUNKS;
  const int r0 = tid / C::ROW_CHUNKS;
  [[maybe_unused]] const PieceRope prope(rope, c);
  const int64_t trow0 = (int64_t)f * T + t0;
  const int64_t snk = kview.sn / 8, snv = vview.sn / 8, sdk = dkview.sn / 8, sdv = dvview.sn / 8;
  const uint4 *kp = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(kview.data) +
                                                    kview.slab(bh, H) + trow0 * kview.sn) +
                    (int64_t)r0 * snk + c;
  const uint4 *vp = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(vview.data) +
                                                    vview.slab(bh, H) + trow0 * vview.sn) +
                    (int64_t)r0 * snv + c;
  uint4 *dkp = reinterpret_cast<uint4 *>(const_cast<uint16_t *>(
                   static_cast<const uint16_t *>(dkview.data) + dkview.slab(bh, H) +
                   trow0 * dkview.sn)) +
               (int64_t)r0 * sdk + c;
  uint4 *dvp = reinterpret_cast<uint4 *>(const_cast<uint16_t *>(
                   static_cast<const uint16_t *>(dvview.data) + dvview.slab(bh, H) +
                   trow0 * dvview.sn)) +
               (int64_t)r0 * sdv + c;
  uint4 rk[C::CPT], rv[C::CPT];
  // Rows past the part load (and later store) its last row again: every
  // output row depends on its own token alone, and a row stored twice gets the
  // same value. Without branches the compiler can count these loads and
  // stores, and waits for the loads alone (the counter covers both).
  auto load = [&](int blk) {
    const int last = L - 1 - blk * C::BLK;  // the block's last row, >= 0
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int64_t row = min(r0 + i * C::ROWS_PER_PASS, last) - r0;
      rk[i] = ld_stream16<true>(kp + row * snk);
      rv[i] = ld_stream16<true>(vp + row * snv);
    }
    kp += C::BLK * snk;
    vp += C::BLK * snv;
  };

  const int tl = 32 * tg + (lane & 31);
  // role dv multiplies phi(k) rows (turned with kRope), role dk multiplies v rows
  const char *btile = role_dk ? vtile : (kRope ? khtile : ktile);
  char *otile = role_dk ? dktile : dvtile;
  const int nblk = (L + C::BLK - 1) / C::BLK;
  load(0);
  wait_vmem_all();  // no load outstanding into the loop: its waits count its own
  for (int blk = 0; blk < nblk; ++blk) {
    sync_lds();  // the previous block's output rows have been read
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int row = r0 + i * C::ROWS_PER_PASS;
      const uint4 kk = relu8(rk[i]);
      *reinterpret_cast<uint4 *>(ktile + row * C::PITCH + c * 16) = kk;
      *reinterpret_cast<uint4 *>(vtile + row * C::PITCH + c * 16) = rv[i];
      if constexpr (kRope) {
        // the token whose row was loaded (rows past the part repeat the last)
        const int l = (int)t0 + blk * C::BLK + min(row, L - 1 - blk * C::BLK);
        uint4 hi, lo;
        prope.turn_whole(kk, l, rope, rope_tab, hi, lo);
        *reinterpret_cast<uint4 *>(khtile + row * C::PITCH + c * 16) = hi;
        *reinterpret_cast<uint4 *>(kltile + row * C::PITCH + c * 16) = lo;
      }
    }
    sync_lds();
    if (blk + 1 < nblk) load(blk + 1);

    f32x16 acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const bf16x8 b = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const uint4 *>(btile + tl * C::PITCH + (16 * ks + 8 * h) * 2));
      acc = mfma_32x32x16(ahi[ks], b, acc);
      acc = mfma_32x32x16(alo[ks], b, acc);
      if constexpr (kRope) {
        if (!role_dk) {  // the low parts of the turned keys
          const bf16x8 bl = __builtin_bit_cast(
              bf16x8,
              *reinterpret_cast<const uint4 *>(kltile + tl * C::PITCH + (16 * ks + 8 * h) * 2));
          acc = mfma_32x32x16(ahi[ks], bl, acc);
        }
      }
    }
    [[maybe_unused]] int ty = 0, tx = 0;  // kRope: the position of token tl
    if constexpr (kRope) {
      const int l = (int)t0 + blk * C::BLK + min(tl, L - 1 - blk * C::BLK);
      grid_pos(l, rope.grid_w, rope.inv_gw, ty, tx);
    }
    // C layout: element 4rg + e is feature 32mb + 8rg + 4h + e of token tl
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int fo = 32 * mb + 8 * rg + 4 * h;
      const int off = tl * C::PITCH + fo * 2;
      float o4[4] = {acc[4 * rg], acc[4 * rg + 1], acc[4 * rg + 2], acc[4 * rg + 3]};
      if (role_dk) {
        if constexpr (kRope) {  // Sh v turns back: features fo .. fo+3 are pairs fo/2, fo/2+1
#pragma unroll
          for (int hp = 0; hp < 2; ++hp) {
            const float2 cs = pair_turn(rope, rope_tab, ty, tx, (fo >> 1) + hp);
            const float2 back = rotate_pair(o4[2 * hp], o4[2 * hp + 1], make_float2(cs.x, -cs.y));
            o4[2 * hp] = back.x;
            o4[2 * hp + 1] = back.y;
          }
        }
        const uint2 kk = *reinterpret_cast<const uint2 *>(ktile + off);  // phi(k) > 0 <=> k > 0
        const float k4[4] = {lo_bf16(kk.x), hi_bf16(kk.x), lo_bf16(kk.y), hi_bf16(kk.y)};
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = k4[e] > 0.f ? o4[e] + szh[fo + e] : 0.f;
      }
      *reinterpret_cast<uint2 *>(otile + off) =
          make_uint2(pack_bf16x2(o4[0], o4[1]), pack_bf16x2(o4[2], o4[3]));
    }
    sync_lds();
    {
      const int last = L - 1 - blk * C::BLK;
#pragma unroll
      for (int i = 0; i < C::CPT; ++i) {
        const int row = min(r0 + i * C::ROWS_PER_PASS, last);
        st_stream16(dkp + (int64_t)(row - r0) * sdk,
                    *reinterpret_cast<const uint4 *>(dktile + row * C::PITCH + c * 16));
        st_stream16(dvp + (int64_t)(row - r0) * sdv,
                    *reinterpret_cast<const uint4 *>(dvtile + row * C::PITCH + c * 16));
      }
    }
    dkp += C::BLK * sdk;
    dvp += C::BLK * sdv;
  }
}

// ---------------------------------------------------------------------------
// Query side: one workgroup of 8 waves per (slab, frame, split). Per block of
// BLK tokens:
//   1. all threads: phi(q) rows -> LDS; den = phi(q) . z_f; from the g and dO
//      rows in registers dh = dO (.) sigmoid(g) (an fp32 tile), 1 - sigmoid(g)
//      (an fp16 tile) and dnum = dh / (den + eps) (it needs den, not num;
//      bf16 hi + lo tiles);
//   2. at once: waves 0-3 ("N") num^T = S^T phi(Q)^T (hi + lo of S), then in
//      the C layout dg = dh (.) h (.) (1 - sigmoid(g)) (written over the fp16
//      tile) and the per-token sums of dh . h;
//      waves 4-7 ("Q") S dnum^T (hi + lo of both, less lo x lo);
//   3. waves 4-7: dq = [q > 0] (.) (S dnum^T + dden z) -> LDS (over the dh
//      tile); waves 0-3:
//      G += phi(Q)^T dnum (transposed LDS reads, as in kv); every thread adds
//      dden phi(q) of its staged rows to gz;
//   4. dq and dg rows -> global memory.
// Wave w of a role takes feature block mb = w % MB and tokens 32 (w / MB)..
// After the last block, G (reduced over the waves that split its k-steps) and
// gz (reduced over the threads of a column piece) go to the split's gslot.
// kRope (3D rotary positions): num and G take the turned phi(q), staged as
// bf16 hi + lo tiles (three MFMAs per step instead of two); den, gz and the
// ReLU mask the unturned one; S dnum^T's rows (a lane holds both features of
// a pair) turn back by R^T before dden z is added.
// ---------------------------------------------------------------------------
#define GLA_BQ_GROUP_BARRIER() __builtin_amdgcn_sched_barrier(0)
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

template <int D>
struct BqCfg {
  static constexpr int MB = D / 32;
  static constexpr int TG = 4 / MB;            // token groups of 32 per role
  static constexpr int BLK = 32 * TG;
  static constexpr int KS = D / 16;            // k-steps over features
  static constexpr int KT = BLK / 16;          // k-steps over the block's tokens
  static constexpr int PITCH = 2 * D + 16;
  static constexpr int ROW_CHUNKS = D / 8;
  static constexpr int CPT = BLK * ROW_CHUNKS / kBwThreads;
  static constexpr int ROWS_PER_PASS = kBwThreads / ROW_CHUNKS;
  static constexpr int GB = MB * MB;           // 32 x 32 blocks of G
  static constexpr int GPW = GB >= 4 ? GB / 4 : 1;   // G blocks per N wave
  static constexpr int KSPLIT = GB >= 4 ? 1 : 4 / GB;  // N waves sharing a G block
  // d <= 64: G accumulates in LDS (fp32, one image per k-step split), which
  // keeps its registers free between blocks; d = 128 keeps 4 blocks in registers
  static constexpr bool kGInLds = D <= 64;
  // image rows padded by 4 floats: the 32 lanes of a half-wave update 32
  // consecutive rows n at one column, which an unpadded D-float stride would
  // put on the same 4 banks
  static constexpr int GLP = D + 4;
  static constexpr int GL_FLOATS = kGInLds ? KSPLIT * D * GLP : 1;
};

// Waves per SIMD bwd_q is held to: 4 (128 registers) at d <= 64 without
// rotary positions, which keeps two workgroups per CU
template <int D, bool kRope>
constexpr int kBqWaves = (D <= 64 && !kRope) ? 4 : 1;

template <int D, bool kRope>
__global__ __launch_bounds__(kBwThreads)
__attribute__((amdgpu_waves_per_eu(kBqWaves<D, kRope>))) void bwd_q_mfma_kernel(
    View qview, View gview, View doview, View dqview, View dgview, int H,
    const float *__restrict__ st, int64_t sstride, float *__restrict__ gs, int F, int64_t T,
    int R, int64_t read_len, float eps, int state_frame, RopeK rope) {
  using C = BqCfg<D>;
  static_assert(C::CPT >= 1, "tile too small for the workgroup");
  // six row tiles in one array (eight with kRope); after the last block it
  // holds the G reduction
  constexpr int TILE = C::BLK * C::PITCH;
  static_assert(6 * TILE >= 4 * 16 * 64 * 4, "LDS too small for the G reduction");
  __shared__ __attribute__((aligned(16))) char smem[(kRope ? 8 : 6) * TILE];
  [[maybe_unused]] char *const qhi = smem + 6 * TILE;  // kRope: turned phi(q), hi
  [[maybe_unused]] char *const qlo = smem + 7 * TILE;  // kRope: turned phi(q), lo
  extern __shared__ float2 rope_tab[];                 // kRope: turns of one frame
  // The dg epilogue takes dh = dO (.) sigmoid(g) in fp32 and 1 - sigmoid(g)
  // as fp16, both formed once when the block is staged (dO and g themselves
  // are read there only); dq then goes over the dh tile, which its last
  // reader is done with.
  constexpr int HPITCH = 4 * D + 16;  // bytes per fp32 row of the dh tile
  static_assert(C::BLK * HPITCH <= 2 * TILE, "dh tile larger than two tiles");
  char *const qtile = smem;              // phi(q)
  char *const gtile = smem + TILE;       // 1 - sigmoid(g) (fp16), then dg
  char *const dnhi = smem + 2 * TILE;    // dnum, hi
  char *const dnlo = smem + 3 * TILE;    // dnum, lo
  char *const htile = smem + 4 * TILE;   // dh (fp32)
  char *const dqtile = htile;            // dq
  __shared__ float szf[D];
  __shared__ __attribute__((aligned(16))) float gl[C::GL_FLOATS];  // G^T images [n][m]
  __shared__ float inv_s[C::BLK];
  __shared__ float ddp[C::MB][C::BLK];  // per feature block: sum of dh . h

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;
  const bool role_q = wave >= 4;
  const int rw = wave & 3;            // wave index within its role
  const int mb = rw % C::MB;
  const int tg = rw / C::MB;
  const int64_t wg = blockIdx.x;
  const int r = (int)(wg % R);
  const int f = (int)((wg / R) % F);
  const int64_t bh = wg / ((int64_t)R * F);
  const int64_t t0 = min((int64_t)r * read_len, T);
  const int64_t t1 = min(t0 + read_len, T);
  const int L = (int)max(t1 - t0, (int64_t)0);

  constexpr int64_t E = (int64_t)D * D + D;
  const float *Sg = st + (bh * F + (state_frame >= 0 ? state_frame : f)) * sstride;  // S_f
  if (tid < D) szf[tid] = Sg[D * D + tid];
  if constexpr (kRope) fill_rope_table(rope_tab, rope, f);  // read after the loop's first barrier
  bf16x8 ahi[C::KS], alo[C::KS];
  if (role_q)
    frag_direct<D>(Sg, mb, lane, ahi, alo);
  else
    frag_transposed<D>(Sg, mb, lane, ahi, alo);

  // G accumulators of an N wave: blocks gb = rw * GPW + u (GPW > 1), or the
  // single block of its KSPLIT group taking k-steps ks % KSPLIT == rw % KSPLIT
  constexpr int NACC = C::kGInLds ? 1 : C::GPW;
  f32x16 gacc[NACC];
#pragma unroll
  for (int u = 0; u < NACC; ++u)
#pragma unroll
    for (int e = 0; e < 16; ++e) gacc[u][e] = 0.f;
  if constexpr (C::kGInLds)
    for (int e = tid; e < C::GL_FLOATS; e += kBwThreads) gl[e] = 0.f;
  const int grp16 = (lane >> 4) & 1;
  const int jj = lane & 15;
  const int frag_row = 8 * h + (jj >> 2);
  const int frag_col = 16 * grp16 + 4 * (jj & 3);

  const int c = tid % C::ROW_CHUNKS;
  const int r0 = tid / C::ROW_CHUNKS;
  [[maybe_unused]] const PieceRope prope(rope, c);
  // the turned phi(q) tiles: B operands of num, A operands of G
  const char *const qnum = kRope ? qhi : qtile;
  float gz8[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) gz8[e] = 0.f;
  // d <= 64 re-reads z and its staged phi(q) pieces from LDS (registers are
  // what limits its occupancy); d = 128 keeps them (its occupancy is set by the
  // fragments either way)
  constexpr bool kKeep = !C::kGInLds;
  float zk[kKeep ? 8 : 1];
  uint4 qkeep[kKeep ? C::CPT : 1];
  if constexpr (kKeep) {
#pragma unroll
    for (int e = 0; e < 8; ++e) zk[e] = Sg[D * D + 8 * c + e];
  }

  const int64_t trow0 = (int64_t)f * T + t0;
  const int64_t snq = qview.sn / 8, sng = gview.sn / 8, sno = doview.sn / 8;
  const int64_t sdq = dqview.sn / 8, sdg = dgview.sn / 8;
  const uint4 *qp = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(qview.data) +
                                                    qview.slab(bh, H) + trow0 * qview.sn) +
                    (int64_t)r0 * snq + c;
  const uint4 *gp = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(gview.data) +
                                                    gview.slab(bh, H) + trow0 * gview.sn) +
                    (int64_t)r0 * sng + c;
  const uint4 *op = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(doview.data) +
                                                    doview.slab(bh, H) + trow0 * doview.sn) +
                    (int64_t)r0 * sno + c;
  uint4 *dqp = reinterpret_cast<uint4 *>(const_cast<uint16_t *>(
                   static_cast<const uint16_t *>(dqview.data) + dqview.slab(bh, H) +
                   trow0 * dqview.sn)) +
               (int64_t)r0 * sdq + c;
  uint4 *dgp = reinterpret_cast<uint4 *>(const_cast<uint16_t *>(
                   static_cast<const uint16_t *>(dgview.data) + dgview.slab(bh, H) +
                   trow0 * dgview.sn)) +
               (int64_t)r0 * sdg + c;
  uint4 rq[C::CPT], rg[C::CPT], ro[C::CPT];
  // Rows past the split load (and later store) its last row again: their
  // 1 / (den + eps) is set to 0 below, which zeroes dnum and dden and with
  // them their share of G and gz, and a row stored twice gets the same value.
  // Without branches the compiler can count these loads and stores, and waits
  // for the loads alone (the counter covers both).
  auto load = [&](int blk) {
    const int last = L - 1 - blk * C::BLK;  // the block's last row, >= 0
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int64_t pass = min(r0 + i * C::ROWS_PER_PASS, last) - r0;
      rq[i] = ld_stream16<true>(qp + pass * snq);
      rg[i] = ld_stream16<true>(gp + pass * sng);
      ro[i] = ld_stream16<true>(op + pass * sno);
    }
    qp += C::BLK * snq;
    gp += C::BLK * sng;
    op += C::BLK * sno;
  };

  const int tl = 32 * tg + (lane & 31);
  const int nblk = (L + C::BLK - 1) / C::BLK;
  if (nblk > 0) load(0);
  wait_vmem_all();  // no load outstanding into the loop: its waits count its own
  for (int blk = 0; blk < nblk; ++blk) {
    sync_lds();  // the previous block's tiles are consumed
    // staging, all threads: phi(q), g and dO rows; den; and dnum, which needs
    // only den: dnum = dO (.) sigmoid(g) / (den + eps)
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int row = r0 + i * C::ROWS_PER_PASS;
      const uint4 w = relu8(rq[i]);
      *reinterpret_cast<uint4 *>(qtile + row * C::PITCH + c * 16) = w;
      if constexpr (kRope) {
        // the token whose row was loaded (rows past the split repeat the last)
        const int l = (int)t0 + blk * C::BLK + min(row, L - 1 - blk * C::BLK);
        uint4 th, tlo;
        prope.turn_whole(w, l, rope, rope_tab, th, tlo);
        *reinterpret_cast<uint4 *>(qhi + row * C::PITCH + c * 16) = th;
        *reinterpret_cast<uint4 *>(qlo + row * C::PITCH + c * 16) = tlo;
      }
      float zc[8];
      if constexpr (kKeep) {
        qkeep[i] = w;
#pragma unroll
        for (int e = 0; e < 8; ++e) zc[e] = zk[e];
      } else {
        const float4 za = *reinterpret_cast<const float4 *>(szf + 8 * c);
        const float4 zb = *reinterpret_cast<const float4 *>(szf + 8 * c + 4);
        zc[0] = za.x; zc[1] = za.y; zc[2] = za.z; zc[3] = za.w;
        zc[4] = zb.x; zc[5] = zb.y; zc[6] = zb.z; zc[7] = zb.w;
      }
      float dp = lo_bf16(w.x) * zc[0];
      dp = fmaf(hi_bf16(w.x), zc[1], dp);
      dp = fmaf(lo_bf16(w.y), zc[2], dp);
      dp = fmaf(hi_bf16(w.y), zc[3], dp);
      dp = fmaf(lo_bf16(w.z), zc[4], dp);
      dp = fmaf(hi_bf16(w.z), zc[5], dp);
      dp = fmaf(lo_bf16(w.w), zc[6], dp);
      dp = fmaf(hi_bf16(w.w), zc[7], dp);
      dp = group_sum<C::ROW_CHUNKS>(dp);  // over the row's pieces
      // rows past the split: 0, so that they add nothing (even with eps = 0)
      const float inv = blk * C::BLK + row < L ? __builtin_amdgcn_rcpf(dp + eps) : 0.f;
      if (c == 0) inv_s[row] = inv;
      const uint32_t gw[4] = {rg[i].x, rg[i].y, rg[i].z, rg[i].w};
      const uint32_t ow[4] = {ro[i].x, ro[i].y, ro[i].z, ro[i].w};
      uint32_t hw[4], lw[4], omw[4];
      float dh8[8];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const float s0 = fast_sigmoid(lo_bf16(gw[e2])), s1 = fast_sigmoid(hi_bf16(gw[e2]));
        dh8[2 * e2] = lo_bf16(ow[e2]) * s0;
        dh8[2 * e2 + 1] = hi_bf16(ow[e2]) * s1;
        split2(dh8[2 * e2] * inv, dh8[2 * e2 + 1] * inv, hw[e2], lw[e2]);
        const f16x2_t om = __builtin_convertvector(f32x2{1.f - s0, 1.f - s1}, f16x2_t);  // nearest
        omw[e2] = __builtin_bit_cast(uint32_t, om);
      }
      *reinterpret_cast<uint4 *>(gtile + row * C::PITCH + c * 16) = make_uint4(omw[0], omw[1], omw[2], omw[3]);
      *reinterpret_cast<float4 *>(htile + row * HPITCH + c * 32) = make_float4(dh8[0], dh8[1], dh8[2], dh8[3]);
      *reinterpret_cast<float4 *>(htile + row * HPITCH + c * 32 + 16) = make_float4(dh8[4], dh8[5], dh8[6], dh8[7]);
      *reinterpret_cast<uint4 *>(dnhi + row * C::PITCH + c * 16) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      *reinterpret_cast<uint4 *>(dnlo + row * C::PITCH + c * 16) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    }
    sync_lds();
    if (blk + 1 < nblk) load(blk + 1);

    f32x16 acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;
    if (!role_q) {
      // num^T for features 32mb.., tokens 32tg..; then dg and the sums dh . h
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const int boff = tl * C::PITCH + (16 * ks + 8 * h) * 2;
        const bf16x8 b = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(qnum + boff));
        acc = mfma_32x32x16(ahi[ks], b, acc);
        acc = mfma_32x32x16(alo[ks], b, acc);
        if constexpr (kRope) {
          const bf16x8 bl = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(qlo + boff));
          acc = mfma_32x32x16(ahi[ks], bl, acc);
        }
      }
      const float inv = inv_s[tl];
      float part = 0.f;
      // Unrolled (a loop would index the accumulator at run time, which takes
      // indexed register moves); a scheduling barrier after each row group
      // keeps only one group's temporaries live, so the kernel stays within
      // the 128 registers of 4 waves per SIMD.
#pragma unroll
      for (int rgp = 0; rgp < 4; ++rgp) {
        GLA_BQ_GROUP_BARRIER();
        const int off = tl * C::PITCH + (32 * mb + 8 * rgp + 4 * h) * 2;
        const uint2 gv = *reinterpret_cast<const uint2 *>(gtile + off);
        const float4 hv = *reinterpret_cast<const float4 *>(htile + tl * HPITCH + (32 * mb + 8 * rgp + 4 * h) * 4);
        const f16x2_t om01 = __builtin_bit_cast(f16x2_t, gv.x), om23 = __builtin_bit_cast(f16x2_t, gv.y);
        const float om4[4] = {(float)om01[0], (float)om01[1], (float)om23[0], (float)om23[1]};
        const float dh4[4] = {hv.x, hv.y, hv.z, hv.w};
        float dg4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float hh = acc[4 * rgp + e] * inv;
          dg4[e] = dh4[e] * hh * om4[e];
          part = fmaf(dh4[e], hh, part);
        }
        *reinterpret_cast<uint2 *>(gtile + off) =
            make_uint2(pack_bf16x2(dg4[0], dg4[1]), pack_bf16x2(dg4[2], dg4[3]));
      }
      part += __shfl_xor(part, 32);  // the other half of the block's features, same token
      if (h == 0) ddp[mb][tl] = part;
    } else {
      // dphi(q)^T without dden z: S dnum^T for features 32mb.., tokens 32tg..
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const int off = tl * C::PITCH + (16 * ks + 8 * h) * 2;
        const bf16x8 bh_ = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(dnhi + off));
        const bf16x8 bl_ = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(dnlo + off));
        acc = mfma_32x32x16(ahi[ks], bh_, acc);
        acc = mfma_32x32x16(alo[ks], bh_, acc);
        acc = mfma_32x32x16(ahi[ks], bl_, acc);
      }
    }
    sync_lds();  // the sums dh . h of every feature block are in ddp

    if (role_q) {
      float dsum = 0.f;
#pragma unroll
      for (int m = 0; m < C::MB; ++m) dsum += ddp[m][tl];
      const float dden = -dsum * inv_s[tl];
      [[maybe_unused]] int ty = 0, tx = 0;  // kRope: the position of token tl
      if constexpr (kRope) {
        const int l = (int)t0 + blk * C::BLK + min(tl, L - 1 - blk * C::BLK);
        grid_pos(l, rope.grid_w, rope.inv_gw, ty, tx);
      }
#pragma unroll
      for (int rgp = 0; rgp < 4; ++rgp) {  // unrolled as above
        GLA_BQ_GROUP_BARRIER();
        const int fo = 32 * mb + 8 * rgp + 4 * h;
        const int off = tl * C::PITCH + fo * 2;
        const uint2 qv = *reinterpret_cast<const uint2 *>(qtile + off);
        const float q4[4] = {lo_bf16(qv.x), hi_bf16(qv.x), lo_bf16(qv.y), hi_bf16(qv.y)};
        float a4[4] = {acc[4 * rgp], acc[4 * rgp + 1], acc[4 * rgp + 2], acc[4 * rgp + 3]};
        if constexpr (kRope) {  // features fo .. fo+3 are pairs fo/2, fo/2 + 1: turn back
#pragma unroll
          for (int hp = 0; hp < 2; ++hp) {
            const float2 cs = pair_turn(rope, rope_tab, ty, tx, (fo >> 1) + hp);
            const float2 back = rotate_pair(a4[2 * hp], a4[2 * hp + 1], make_float2(cs.x, -cs.y));
            a4[2 * hp] = back.x;
            a4[2 * hp + 1] = back.y;
          }
        }
        float d4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) d4[e] = q4[e] > 0.f ? fmaf(dden, szf[fo + e], a4[e]) : 0.f;
        *reinterpret_cast<uint2 *>(dqtile + off) =
            make_uint2(pack_bf16x2(d4[0], d4[1]), pack_bf16x2(d4[2], d4[3]));
      }
    }
    if (!role_q) {
      // G += phi(Q)^T dnum over the block's tokens (waves 0-3, their accumulators free)
#pragma unroll
      for (int u = 0; u < C::GPW; ++u) {
        const int gb = C::KSPLIT > 1 ? 0 : rw * C::GPW + u;
        const int bi = gb / C::MB, bj = gb % C::MB;
        f32x16 blk_acc;
        if constexpr (C::kGInLds) {
#pragma unroll
          for (int e = 0; e < 16; ++e) blk_acc[e] = 0.f;
        } else {
          blk_acc = gacc[u];
        }
#pragma unroll
        for (int kt = 0; kt < C::KT; ++kt) {
          if (C::KSPLIT > 1 && kt % C::KSPLIT != rw % C::KSPLIT) continue;
          const bf16x8 fa = tr_fragment((const lds_char *)qnum, kt * 16 + frag_row,
                                        32 * bi + frag_col, C::PITCH);
          const bf16x8 fh = tr_fragment((const lds_char *)dnhi, kt * 16 + frag_row,
                                        32 * bj + frag_col, C::PITCH);
          const bf16x8 fl = tr_fragment((const lds_char *)dnlo, kt * 16 + frag_row,
                                        32 * bj + frag_col, C::PITCH);
          blk_acc = mfma_32x32x16(fa, fh, blk_acc);
          blk_acc = mfma_32x32x16(fa, fl, blk_acc);
          if constexpr (kRope) {  // the low parts of the turned queries
            const bf16x8 fal = tr_fragment((const lds_char *)qlo, kt * 16 + frag_row,
                                           32 * bi + frag_col, C::PITCH);
            blk_acc = mfma_32x32x16(fal, fh, blk_acc);
          }
        }
        if constexpr (C::kGInLds) {
          // add into this wave's image (rows m = 8(e/4) + 4h + e%4 of column n)
          float *img = gl + (C::KSPLIT > 1 ? rw % C::KSPLIT : 0) * D * C::GLP;
          const int n = 32 * bj + (lane & 31);
#pragma unroll
          for (int e4 = 0; e4 < 4; ++e4) {
            float4 *cell = reinterpret_cast<float4 *>(img + n * C::GLP + 32 * bi + 8 * e4 + 4 * h);
            float4 v = *cell;
            v.x += blk_acc[4 * e4];
            v.y += blk_acc[4 * e4 + 1];
            v.z += blk_acc[4 * e4 + 2];
            v.w += blk_acc[4 * e4 + 3];
            *cell = v;
          }
        } else {
          gacc[u] = blk_acc;
        }
      }
    }
    // gz += dden phi(q) over this thread's staged rows
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int row = r0 + i * C::ROWS_PER_PASS;
      float dsum = 0.f;
#pragma unroll
      for (int m = 0; m < C::MB; ++m) dsum += ddp[m][row];
      const float dden = -dsum * inv_s[row];
      uint4 w;
      if constexpr (kKeep)
        w = qkeep[i];
      else
        w = *reinterpret_cast<const uint4 *>(qtile + row * C::PITCH + c * 16);
      gz8[0] = fmaf(dden, lo_bf16(w.x), gz8[0]);
      gz8[1] = fmaf(dden, hi_bf16(w.x), gz8[1]);
      gz8[2] = fmaf(dden, lo_bf16(w.y), gz8[2]);
      gz8[3] = fmaf(dden, hi_bf16(w.y), gz8[3]);
      gz8[4] = fmaf(dden, lo_bf16(w.z), gz8[4]);
      gz8[5] = fmaf(dden, hi_bf16(w.z), gz8[5]);
      gz8[6] = fmaf(dden, lo_bf16(w.w), gz8[6]);
      gz8[7] = fmaf(dden, hi_bf16(w.w), gz8[7]);
    }
    sync_lds();
    {
      const int last = L - 1 - blk * C::BLK;
#pragma unroll
      for (int i = 0; i < C::CPT; ++i) {
        const int row = min(r0 + i * C::ROWS_PER_PASS, last);
        const int64_t pass = row - r0;
        st_stream16(dqp + pass * sdq, *reinterpret_cast<const uint4 *>(dqtile + row * C::PITCH + c * 16));
        st_stream16(dgp + pass * sdg, *reinterpret_cast<const uint4 *>(gtile + row * C::PITCH + c * 16));
      }
    }
    dqp += C::BLK * sdq;
    dgp += C::BLK * sdg;
  }

  // ---- the split's G and gz -> its gslot (the tiles are free now) ----
  float *out = gs + ((bh * F + f) * (int64_t)R + r) * E;
  sync_lds();
  if constexpr (C::kGInLds) {
    // sum the images, transpose back: out[m * D + n] = sum_img gl[img][n][m]
    for (int e = tid; e < D * D; e += kBwThreads) {
      const int m = e / D, n = e % D;
      float sum = 0.f;
#pragma unroll
      for (int im = 0; im < C::KSPLIT; ++im) sum += gl[(im * D + n) * C::GLP + m];
      out[e] = sum;
    }
  }
  float *red = reinterpret_cast<float *>(smem);  // [wave][16][64] partial G blocks
  if (!C::kGInLds && C::KSPLIT > 1) {
    if (!role_q) {
#pragma unroll
      for (int e = 0; e < 16; ++e) red[(rw * 16 + e) * 64 + lane] = gacc[0][e];
    }
    sync_lds();
    if (!role_q && rw == 0) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float sum = 0.f;
        for (int w2 = 0; w2 < C::KSPLIT; ++w2) sum += red[(w2 * 16 + e) * 64 + lane];
        gacc[0][e] = sum;
      }
    }
  }
  if (!C::kGInLds && !role_q && (C::KSPLIT == 1 || rw == 0)) {
#pragma unroll
    for (int u = 0; u < C::GPW; ++u) {
      const int gb = C::KSPLIT > 1 ? 0 : rw * C::GPW + u;
      const int bi = gb / C::MB, bj = gb % C::MB;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = 8 * (e >> 2) + 4 * h + (e & 3);
        out[(32 * bi + m) * D + 32 * bj + (lane & 31)] = gacc[u][e];
      }
    }
  }
  // gz: sum over the lanes of a column piece, then over the waves
#pragma unroll
  for (int e = 0; e < 8; ++e)
#pragma unroll
    for (int off = C::ROW_CHUNKS; off < 64; off <<= 1) gz8[e] += __shfl_xor(gz8[e], off);
  sync_lds();
  float *gzr = reinterpret_cast<float *>(smem + 5 * TILE);  // [wave][D], clear of red
  if (lane < C::ROW_CHUNKS) {
#pragma unroll
    for (int e = 0; e < 8; ++e) gzr[wave * D + 8 * lane + e] = gz8[e];
  }
  sync_lds();
  if (tid < D) {
    float sum = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < kBwThreads / 64; ++w2) sum += gzr[w2 * D + tid];
    out[D * D + tid] = sum;
  }
}

template <int D>
void bwd_q_launch(const BwdPlan &bp, const BwdQArgs &a, hipStream_t s) {
  const Plan &p = bp.f;
  const dim3 grid((unsigned)(p.BH * p.F * p.R));
  if (a.rope.on) {
    RopeK r = a.rope;
    r.frames = 1;  // a workgroup covers one frame
    hipLaunchKernelGGL((bwd_q_mfma_kernel<D, true>), grid, dim3(kBwThreads),
                       (unsigned)(r.entries() * sizeof(float2)), s, a.q, a.g, a.dO, a.dq, a.dg,
                       a.H, a.st.base, a.st.stride, a.gs, p.F, p.T, p.R, p.read_len, a.eps,
                       a.state_frame, r);
  } else {
    hipLaunchKernelGGL((bwd_q_mfma_kernel<D, false>), grid, dim3(kBwThreads), 0, s, a.q, a.g,
                       a.dO, a.dq, a.dg, a.H, a.st.base, a.st.stride, a.gs, p.F, p.T, p.R,
                       p.read_len, a.eps, a.state_frame, a.rope);
  }
}

template <int D>
void bwd_k_launch(const BwdPlan &bp, const BwdKArgs &a, hipStream_t s) {
  const Plan &p = bp.f;
  const dim3 grid((unsigned)(p.BH * p.F * p.P));
  if (a.rope.on) {
    RopeK r = a.rope;
    r.frames = 1;  // a workgroup covers one frame
    hipLaunchKernelGGL((bwd_k_mfma_kernel<D, true>), grid, dim3(kBwThreads),
                       (unsigned)(r.entries() * sizeof(float2)), s, a.k, a.v, a.dk, a.dv, a.H,
                       a.gs, p.F, p.T, p.P, p.R, p.part_len, a.adj_frame, r);
  } else {
    hipLaunchKernelGGL((bwd_k_mfma_kernel<D, false>), grid, dim3(kBwThreads), 0, s, a.k, a.v,
                       a.dk, a.dv, a.H, a.gs, p.F, p.T, p.P, p.R, p.part_len, a.adj_frame,
                       a.rope);
  }
}

}  // namespace

hipError_t launch_bwd_q_mfma(const BwdPlan &p, const BwdQArgs &a, hipStream_t s) {
  if (p.f.BH * p.f.F * p.f.R == 0) return hipSuccess;
  switch (p.f.d) {
    case 32: bwd_q_launch<32>(p, a, s); break;
    case 64: bwd_q_launch<64>(p, a, s); break;
    case 128: bwd_q_launch<128>(p, a, s); break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_bwd_k_mfma(const BwdPlan &p, const BwdKArgs &a, hipStream_t s) {
  if (p.f.BH * p.f.F * p.f.P == 0 || p.f.T == 0) return hipSuccess;
  switch (p.f.d) {
    case 32: bwd_k_launch<32>(p, a, s); break;
    case 64: bwd_k_launch<64>(p, a, s); break;
    case 128: bwd_k_launch<128>(p, a, s); break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace gla
