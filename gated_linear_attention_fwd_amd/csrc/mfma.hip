// mfma.hip -- bf16 matrix-core (MFMA) kernels for gfx950: KV sums and readout.
//
// Both contractions of the gated linear attention run on
// v_mfma_f32_32x32x16_bf16 (fp32 accumulation; bf16 x bf16 products are exact
// in fp32):
//
//   kv:      U = phi(K)^T V over a token range (d x C times C x d), u = phi(K)^T 1
//   readout: o^T = S_f^T phi(Q)^T (d x d times d x C), den = phi(Q) z_f, then
//            o = sigmoid(g) * num / (den + eps), rounded to bf16
//
// The state is fp32; for the readout it is split as S = S_hi + S_lo with both
// parts bf16 (S_lo = bf16(S - S_hi)), so the product keeps ~16 bits of S.
//
// (MFMA operand layouts: mfma_util.hpp.)
//
// KV: the contraction runs over tokens, the slow axis of the [N][d] layout, so
// both operands are read transposed out of row-major LDS tiles with
// ds_read_b64_tr_b16 (gfx950): within each group of 16 lanes, lane j supplies
// the address of 4 consecutive bf16 in row j/4 (columns 4(j%4)..) of a 4 x 16
// block and receives column j of that block (rows 0..3).
#include "common.hpp"
#include "mfma_util.hpp"
#include "plan.hpp"
#include "rope_tab.hpp"

namespace gla {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxGroup = 8;  // most frames per kv workgroup (the plan's limit)

// Waves per SIMD the compiler must allow. The rotary variants at d <= 64 would
// otherwise take 3 (accumulators in AGPRs on top of ~120 VGPRs); with all
// registers in one file they fit 4, without spills. 1: no constraint.
template <int D, bool kRope>
constexpr int kMinWaves = (kRope && D <= 64) ? 4 : 1;

// q, k, v and g are read exactly once and o is written once: nontemporal
// loads and stores keep that stream from displacing lines the next kernel
// reuses (measured on the 720p/60s shape: kv -10%, readout -7%). Every such
// access is a 16-byte-per-lane instruction covering whole rows.
#ifndef GLA_KV_NT_LOADS
#define GLA_KV_NT_LOADS 1
#endif
#ifndef GLA_RO_NT_LOADS
#define GLA_RO_NT_LOADS 1
#endif
#ifndef GLA_RO_NT_STORES
#define GLA_RO_NT_STORES 1
#endif
#ifndef GLA_RO_XCD_REMAP
#define GLA_RO_XCD_REMAP 1
#endif

// ---------------------------------------------------------------------------
// KV sums
// ---------------------------------------------------------------------------
template <int D>
struct KvCfg {
  static constexpr int CH = 64;             // tokens per LDS chunk (4 k-steps of 16)
  static constexpr int PITCH = 2 * D + 32;  // bytes per LDS row
  static constexpr int MB = D / 32;         // 32 x 32 blocks per side of U
  // D = 32: every wave owns the single block and one k-step of each chunk
  // (partials summed across waves per frame). D >= 64: the MB x MB blocks are
  // split 2 x 2 over the waves and each wave runs every k-step, so a wave owns
  // its blocks outright and no cross-wave sum is needed.
  static constexpr bool kSplitTokens = (D == 32);
  static constexpr int TM = kSplitTokens ? MB : MB / 2;
  // running decayed state kept across the frames of a group, in registers of
  // its own (d <= 64); at d = 128 those would be 64 more registers per lane,
  // so there the accumulators themselves carry it: after a frame's slot is
  // written they are scaled by the next frame's decay (kInPlace; the file is
  // built with MFMA accumulators in VGPRs, where that scaling is plain vector
  // work: 165 VGPRs, 3 waves per SIMD)
  static constexpr bool kGroups = (D <= 64);
  static constexpr bool kInPlace = (D == 128);
  static constexpr int ROW_CHUNKS = D / 8;                 // 16-byte pieces per row
  static constexpr int CPT = CH * ROW_CHUNKS / kThreads;   // pieces per thread per array
  static constexpr int ROWS_PER_PASS = kThreads / ROW_CHUNKS;
  static constexpr int TILE_BYTES = CH * PITCH;
  static constexpr int RED_BYTES = kSplitTokens ? 4 * 1024 * 4 : 0;  // 4 waves x 32x32 fp32
  static constexpr int U_RED_BYTES = 4 * D * 4;                       // 4 waves x D fp32
  static constexpr int SMEM = (2 * TILE_BYTES > RED_BYTES ? 2 * TILE_BYTES : RED_BYTES);
  // with rotary positions a third tile holds the low bf16 parts of turned phi(k)
  static constexpr int SMEM_ROPE = (3 * TILE_BYTES > RED_BYTES ? 3 * TILE_BYTES : RED_BYTES);
};

// One workgroup per (slab, group of G frames, part). Per frame the MFMA
// accumulators collect that frame's U_f; a per-thread running state then
// becomes S_loc_f = gamma_f * S_loc_{f-1} + U_f and is written to the frame's
// slot (z likewise). d = 128 keeps no running state (it would cost 64 more
// registers per lane) and runs one frame per workgroup. Chunks are numbered
// across the group's frames so that the next chunk's loads (possibly the next
// frame's) overlap the MFMAs and the write-out of the current one.
template <int D, bool kRope>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(kMinWaves<D, kRope>))) void kv_mfma_kernel(View kview, View vview, int H,
                                                           const float *__restrict__ gamma,
                                                           float *__restrict__ ws, int F,
                                                           int64_t T, int P, int G,
                                                           int64_t part_len, RopeK rope) {
  using C = KvCfg<D>;
  constexpr int kSmem = kRope ? C::SMEM_ROPE : C::SMEM;
  __shared__ __attribute__((aligned(16))) char smem[kSmem + C::U_RED_BYTES];
  extern __shared__ float2 rope_tab[];  // kRope: RopeK::entries() (cos, sin) pairs
  // the running state's elements per thread (d = 128 keeps none: 1 unused)
  constexpr int kSt = !C::kGroups ? 1 : (C::kSplitTokens ? C::TM * C::TM * 4 : C::TM * C::TM * 16);
  // an even frame's state and z, parked here until the next frame's slot is
  // written with it (thread-private layout [element][thread]); not with
  // rotary positions, whose turn table and third tile leave no room for it
  // (and whose registers it would push to 3 waves per SIMD)
  constexpr bool kStash = C::kGroups && !kRope;
  __shared__ float stash[kStash ? (kSt + 1) * kThreads : 1];
  lds_char *const sbase = (lds_char *)smem;
  lds_char *const tk = sbase;
  lds_char *const tv = sbase + C::TILE_BYTES;
  lds_char *const tk_lo = sbase + 2 * C::TILE_BYTES;  // kRope only

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int NG = (F + G - 1) / G;
  const int64_t wg = blockIdx.x;
  const int p = (int)(wg % P);
  const int grp = (int)((wg / P) % NG);
  const int64_t bh = wg / ((int64_t)P * NG);
  const int64_t N = (int64_t)F * T;
  const int64_t t0 = min((int64_t)p * part_len, T);
  const int64_t t1 = min(t0 + part_len, T);
  const int L = (int)(t1 - t0);
  const int f_begin = grp * G;
  // in-place groups at d = 128 without rotary positions only (the frame's
  // turn applies to U_f, not to the running sum; the plan keeps G = 1 there)
  constexpr bool kInPlace = C::kInPlace && !kRope;
  constexpr bool kAnyGroups = C::kGroups || kInPlace;
  const int nf = kAnyGroups ? min(F, f_begin + G) - f_begin : 1;
  const int ncf = (L + C::CH - 1) / C::CH;  // chunks per frame
  const int total = nf * ncf;
  (void)N;
  // row strides in 16-byte pieces (host-checked multiples of 8 elements)
  const int64_t snk = kview.sn / 8, snv = vview.sn / 8;
  const uint4 *kb = reinterpret_cast<const uint4 *>(
      static_cast<const uint16_t *>(kview.data) + kview.slab(bh, H) +
      ((int64_t)f_begin * T + t0) * kview.sn);
  const uint4 *vb = reinterpret_cast<const uint4 *>(
      static_cast<const uint16_t *>(vview.data) + vview.slab(bh, H) +
      ((int64_t)f_begin * T + t0) * vview.sn);

  // this thread's 16-byte pieces: fixed column piece c, rows r0 + i * ROWS_PER_PASS
  const int c = tid % C::ROW_CHUNKS;
  const int r0 = tid / C::ROW_CHUNKS;
  [[maybe_unused]] const PieceRope prope(rope, c);
  uint4 rk[C::CPT], rv[C::CPT];
  // Chunks are loaded in order (frame by frame): the addresses of this
  // thread's pieces advance by additions only.
  const uint4 *kp = kb + (int64_t)r0 * snk + c, *vp = vb + (int64_t)r0 * snv + c;
  const int64_t k_pass = C::ROWS_PER_PASS * snk, v_pass = C::ROWS_PER_PASS * snv;
  // from a frame's last chunk to the next frame's first: T - (ncf - 1) * CH rows
  const int64_t jump_rows = T - (int64_t)(ncf > 0 ? ncf - 1 : 0) * C::CH;
  int lcc = 0;  // chunk index within its frame of the next load
  auto load = [&]() {
    const int base = lcc * C::CH;
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int row = base + r0 + i * C::ROWS_PER_PASS;
      if (row < L) {
        rk[i] = ld_stream16<GLA_KV_NT_LOADS>(kp + i * k_pass);
        rv[i] = ld_stream16<GLA_KV_NT_LOADS>(vp + i * v_pass);
      } else {
        rk[i] = make_uint4(0, 0, 0, 0);
        rv[i] = make_uint4(0, 0, 0, 0);
      }
    }
    if (++lcc == ncf) {  // on to the next frame's first chunk
      lcc = 0;
      kp += jump_rows * snk;
      vp += jump_rows * snv;
    } else {
      kp += C::CH * snk;
      vp += C::CH * snv;
    }
  };

  float uacc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) uacc[e] = 0.f;
  f32x16 acc[C::TM][C::TM];
#pragma unroll
  for (int a = 0; a < C::TM; ++a)
#pragma unroll
    for (int b = 0; b < C::TM; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  // lane geometry of the transposed fragment reads
  const int h = lane >> 5;
  const int grp16 = (lane >> 4) & 1;
  const int j = lane & 15;
  const int frag_row = 8 * h + (j >> 2);
  const int frag_col = 16 * grp16 + 4 * (j & 3);
  const int wm = C::kSplitTokens ? 0 : (wave >> 1);
  const int wn = C::kSplitTokens ? 0 : (wave & 1);
  float *red = (float *)smem;                 // [wave][r][lane], aliases the tiles
  float *ured = (float *)(smem + kSmem);      // [wave][D]

  // running state of the group: accumulator layout (d = 64) or the layout of
  // the cross-wave sum (d = 32)
  float st[kSt];
  float zst = 0.f;
#pragma unroll
  for (int e = 0; e < kSt; ++e) st[e] = 0.f;

  // the group's decays, loaded once up front (a load per frame would stall
  // every frame's write-out for a full memory latency); branch-free, frames
  // past the group reloading its last one, so that all go out at once (with
  // a test per load each was a memory round trip of its own)
  constexpr int kNg = kAnyGroups ? kMaxGroup : 1;
  float gms[kNg];
  if (gamma) {
    const float *gsl = gamma + bh * F + f_begin;
#pragma unroll
    for (int e = 0; e < kNg; ++e) gms[e] = gsl[min(e, nf - 1)];
  } else {
#pragma unroll
    for (int e = 0; e < kNg; ++e) gms[e] = 1.f;
  }
#pragma unroll
  for (int e = 0; e < kNg; ++e) gms[e] = (e > 0 && e < nf) ? gms[e] : 0.f;

  if constexpr (kRope) {
    fill_rope_table(rope_tab, rope, f_begin);
    sync_lds();
  }
  // U_f's rows (key features) turn with the frame: rows 2p and 2p+1 of a C
  // block sit in one lane (elements r and r+1, r even)
  auto turn_rows = [&](int fi) {
    if constexpr (kRope) {
#pragma unroll
      for (int a = 0; a < C::TM; ++a) {
        const int rb = C::kSplitTokens ? a : wm * C::TM + a;
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const int pr = 16 * rb + 4 * (r >> 2) + 2 * h + ((r & 3) >> 1);
          const float2 cs = rope_tab[pr < rope.Pt ? rope.t_base() + fi * rope.Pt + pr : 0];
#pragma unroll
          for (int b = 0; b < C::TM; ++b) {
            const float2 ab = rotate_pair(acc[a][b][r], acc[a][b][r + 1], cs);
            acc[a][b][r] = ab.x;
            acc[a][b][r + 1] = ab.y;
          }
        }
      }
    }
  };

  // After a frame's last chunk, frame_close() folds U_f into the running state
  // (registers; z through an LDS sum), and the slot is written later:
  //  - vmcnt counts loads and stores alike, and with a store outstanding the
  //    wait for a load takes the store's completion with it. Stores are
  //    therefore issued right after a chunk's loads have been waited for, one
  //    chunk after the frame closed, so that they meet no outstanding prefetch.
  //  - Each such write-out still costs the workgroup a store round trip before
  //    its next load is consumed. An even frame's state therefore waits in LDS
  //    and goes out together with the next frame's: half the write-outs
  //    (720p/60s: kv 0.361 -> 0.351 ms; with all of a workgroup's states
  //    written at its end, kv is 0.338 ms, but that needs LDS for G states).
  auto frame_close = [&](int fi) {
    turn_rows(fi);
    float gm = 0.f;
#pragma unroll
    for (int e = 1; e < (kAnyGroups ? kMaxGroup : 1); ++e) gm = (fi == e) ? gms[e] : gm;
    if constexpr (C::kSplitTokens) {
#pragma unroll
      for (int a = 0; a < C::TM; ++a)
#pragma unroll
        for (int b = 0; b < C::TM; ++b) {
          sync_lds();
#pragma unroll
          for (int r = 0; r < 16; ++r) red[wave * 1024 + r * 64 + lane] = acc[a][b][r];
          sync_lds();
#pragma unroll
          for (int e4 = 0; e4 < 4; ++e4) {
            const int idx = tid + kThreads * e4;
            const float sum = red[idx] + red[1024 + idx] + red[2048 + idx] + red[3072 + idx];
            float &sv = st[(a * C::TM + b) * 4 + e4];
            sv = fmaf(gm, sv, sum);  // kSplitTokens implies kGroups
          }
        }
    } else if constexpr (C::kGroups) {
#pragma unroll
      for (int a = 0; a < C::TM; ++a)
#pragma unroll
        for (int b = 0; b < C::TM; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float &run = st[(a * C::TM + b) * 16 + r];
            run = fmaf(gm, run, acc[a][b][r]);
          }
    }
    // z: sum the thread's 8 features over lanes with the same column piece, then waves
    float us[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      us[e] = uacc[e];
#pragma unroll
      for (int off = C::ROW_CHUNKS; off < 64; off <<= 1) us[e] += __shfl_xor(us[e], off);
    }
    sync_lds();  // previous frame's ured reads (and the red rounds) are done
    if (lane < C::ROW_CHUNKS) {
#pragma unroll
      for (int e = 0; e < 8; ++e) ured[wave * D + lane * 8 + e] = us[e];
    }
    sync_lds();
    if (tid < D)
      zst = fmaf(gm, zst, ured[tid] + ured[D + tid] + ured[2 * D + tid] + ured[3 * D + tid]);
  };

  // Writes frame fi's slot. src(e, tid) is element e of the running state in
  // st's layout, z(tid) the normaliser sum (d = 128: the accumulators).
  auto write_slot = [&](int fi, auto src, auto z) {
    float *out = ws + ((bh * F + f_begin + fi) * (int64_t)P + p) * ((int64_t)D * D + D);
    // Recompute the offsets from an opaque copy of the thread id: hoisted out
    // of the loop they would stay live in registers.
    int tidv = tid;
    asm volatile("" : "+v"(tidv));
    const int lanev = tidv & 63;
    if constexpr (C::kSplitTokens) {
#pragma unroll
      for (int a = 0; a < C::TM; ++a)
#pragma unroll
        for (int b = 0; b < C::TM; ++b)
#pragma unroll
          for (int e4 = 0; e4 < 4; ++e4) {
            const int idx = tidv + kThreads * e4;
            const int r = idx >> 6, ln = idx & 63;
            const int m = 8 * (r >> 2) + 4 * (ln >> 5) + (r & 3);
            out[(32 * a + m) * D + 32 * b + (ln & 31)] = src((a * C::TM + b) * 4 + e4, tidv);
          }
    } else {
#pragma unroll
      for (int a = 0; a < C::TM; ++a)
#pragma unroll
        for (int b = 0; b < C::TM; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float sv = C::kGroups ? src((a * C::TM + b) * 16 + r, tidv) : acc[a][b][r];
            const int m = 8 * (r >> 2) + 4 * (lanev >> 5) + (r & 3);
            out[(32 * (wm * C::TM + a) + m) * D + 32 * (wn * C::TM + b) + (lanev & 31)] = sv;
          }
    }
    if (tidv < D) out[D * D + tidv] = z(tidv);
  };
  auto store_state = [&](int fi) {
    write_slot(fi, [&](int e, int) { return st[e]; }, [&](int) { return zst; });
  };
  auto store_stash = [&](int fi) {
    write_slot(fi, [&](int e, int t) { return stash[e * kThreads + t]; },
               [&](int t) { return stash[kSt * kThreads + t]; });
  };

  int pending = -1;  // frame whose slot is still to be written
  int stashed = -1;  // frame whose state waits in the stash
  if (total > 0) load();
  for (int fi = 0; fi < nf; ++fi) {
    if (fi > 0) {
      if constexpr (!kInPlace) {
#pragma unroll
        for (int a = 0; a < C::TM; ++a)
#pragma unroll
          for (int b = 0; b < C::TM; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) uacc[e] = 0.f;
    }
    for (int cc = 0; cc < ncf; ++cc) {
      const int ch = fi * ncf + cc;
      sync_lds();
#pragma unroll
      for (int i = 0; i < C::CPT; ++i) {
        const int row = r0 + i * C::ROWS_PER_PASS;
        const uint4 kk = relu8(rk[i]);
        if constexpr (kRope) {
          // z takes phi(k) unturned; S the spatially turned one (rows past the
          // part are zeros: any in-frame position does)
          const int l = (int)min(t0 + cc * C::CH + row, T - 1);
          uint4 khi, klo;
          prope.turn(kk, l, rope, rope_tab, khi, klo);
          *reinterpret_cast<uint4 *>(smem + row * C::PITCH + c * 16) = khi;
          *reinterpret_cast<uint4 *>(smem + 2 * C::TILE_BYTES + row * C::PITCH + c * 16) = klo;
        } else {
          *reinterpret_cast<uint4 *>(smem + row * C::PITCH + c * 16) = kk;
        }
        *reinterpret_cast<uint4 *>(smem + C::TILE_BYTES + row * C::PITCH + c * 16) = rv[i];
        uacc[0] += lo_bf16(kk.x);
        uacc[1] += hi_bf16(kk.x);
        uacc[2] += lo_bf16(kk.y);
        uacc[3] += hi_bf16(kk.y);
        uacc[4] += lo_bf16(kk.z);
        uacc[5] += hi_bf16(kk.z);
        uacc[6] += lo_bf16(kk.w);
        uacc[7] += hi_bf16(kk.w);
      }
      sync_lds();
      if (pending >= 0) {
        if (stashed >= 0) {
          store_stash(stashed);
          stashed = -1;
        }
        store_state(pending);
        pending = -1;
      }
      if constexpr (kInPlace) {
        if (cc == 0 && fi > 0) {  // the previous frame's slot is written: decay the running sum
          float gm = 0.f;
#pragma unroll
          for (int e = 1; e < kMaxGroup; ++e) gm = (fi == e) ? gms[e] : gm;
#pragma unroll
          for (int a = 0; a < C::TM; ++a)
#pragma unroll
            for (int b = 0; b < C::TM; ++b)
#pragma unroll
              for (int r = 0; r < 16; ++r) acc[a][b][r] *= gm;
        }
      }
      if (ch + 1 < total) load();

      constexpr int KS_PER_WAVE = C::kSplitTokens ? 1 : 4;
#pragma unroll
      for (int kk = 0; kk < KS_PER_WAVE; ++kk) {
        const int ks = C::kSplitTokens ? wave : kk;
        bf16x8 fa[C::TM], fb[C::TM];
#pragma unroll
        for (int a = 0; a < C::TM; ++a) {
          fa[a] = tr_fragment(tk, ks * 16 + frag_row, 32 * (wm * C::TM + a) + frag_col, C::PITCH);
          fb[a] = tr_fragment(tv, ks * 16 + frag_row, 32 * (wn * C::TM + a) + frag_col, C::PITCH);
        }
#pragma unroll
        for (int a = 0; a < C::TM; ++a)
#pragma unroll
          for (int b = 0; b < C::TM; ++b) acc[a][b] = mfma_32x32x16(fa[a], fb[b], acc[a][b]);
        if constexpr (kRope) {
          // low parts of the turned keys
#pragma unroll
          for (int a = 0; a < C::TM; ++a) {
            const bf16x8 fl =
                tr_fragment(tk_lo, ks * 16 + frag_row, 32 * (wm * C::TM + a) + frag_col, C::PITCH);
#pragma unroll
            for (int b = 0; b < C::TM; ++b) acc[a][b] = mfma_32x32x16(fl, fb[b], acc[a][b]);
          }
        }
      }
    }
    frame_close(fi);
    if (kStash && (fi & 1) == 0 && fi + 1 < nf && ncf > 0 && pending < 0) {
#pragma unroll
      for (int e = 0; e < kSt; ++e) stash[e * kThreads + tid] = st[e];
      stash[kSt * kThreads + tid] = zst;
      stashed = fi;
    } else if (pending >= 0 || ncf == 0) {  // no chunk follows to carry the store
      if (stashed >= 0) {
        store_stash(stashed);
        stashed = -1;
      }
      store_state(fi);
    } else {
      pending = fi;
    }
  }
  if (stashed >= 0) store_stash(stashed);
  if (pending >= 0) store_state(pending);
}

// ---------------------------------------------------------------------------
// Readout
// ---------------------------------------------------------------------------
template <int D>
struct RoCfg {
  static constexpr int MB = D / 32;            // 32-feature output blocks
  static constexpr int TG = 4 / MB;            // token groups of 32 across the waves
  static constexpr int BLK = 32 * TG;          // tokens per iteration
  static constexpr int KS = D / 16;            // k-steps over the input features
  static constexpr int PITCH = 2 * D + 16;     // bytes per LDS row of phi(q)
  static constexpr int ROW_CHUNKS = D / 8;
  static constexpr int CPT = BLK * ROW_CHUNKS / kThreads;  // 16-byte pieces per thread
  static constexpr int ROWS_PER_PASS = kThreads / ROW_CHUNKS;
};

// One workgroup per (slab, frame, split). q, g and o move through LDS so that
// every global access is a 16-byte-per-lane load or store covering whole rows;
// the MFMA operand reads (phi(q), B layout) and the epilogue's C-layout
// gather of g / scatter of o happen in LDS. Per block of tokens:
//   1. phi(q) and g rows -> LDS; den = phi(q) . z_f computed on the way
//   2. acc = S_f^T phi(q)^T over the input features (hi and lo parts of S_f)
//   3. o = sigmoid(g) * acc / (den + eps) -> bf16, written over g in LDS
//   4. o rows -> global memory
template <int D, bool kRope>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(kMinWaves<D, kRope>))) void readout_kernel(
    View qview, View gview, View oview, int H, const float *__restrict__ gamma,
    const float *__restrict__ ws, const float *__restrict__ st, int64_t sstride, int F, int64_t T,
    int G, int64_t carry_offset, int R, int64_t read_len, float eps, int state_frame, RopeK rope, int heads_fastest) {
  using C = RoCfg<D>;
  constexpr int GP = 2 * D + 16;  // bytes per LDS row of g / o
  __shared__ __attribute__((aligned(16))) char qtile[C::BLK * C::PITCH];
  __shared__ __attribute__((aligned(16))) char qtile_lo[kRope ? C::BLK * C::PITCH : 16];
  __shared__ __attribute__((aligned(16))) char gtile[C::BLK * GP];
  __shared__ float den_s[C::BLK];
  extern __shared__ float2 rope_tab[];  // kRope: RopeK::entries() (cos, sin) pairs

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;
  const int mb = wave % C::MB;
  const int tg = wave / C::MB;
  // work item order (after the XCD renumbering): (slab slowest, frame, split
  // fastest), or with heads_fastest (frame slowest, split, slab fastest) -- for
  // layouts whose heads sit side by side within a token: concurrent workgroups
  // then read neighbouring lines (720p/60s, fused [B,N,3,H,d] q: readout -6%;
  // the same order for kv measured neutral at d = 64 and slower at d = 128)
  const int wg = (int)(GLA_RO_XCD_REMAP ? xcd_contiguous(blockIdx.x, gridDim.x) : blockIdx.x);
  int r, f, bhi;
  if (heads_fastest) {
    const int nbh = (int)gridDim.x / (R * F);
    bhi = wg % nbh;
    r = (wg / nbh) % R;
    f = wg / (nbh * R);
  } else {
    r = wg % R;
    f = (wg / R) % F;
    bhi = wg / (R * F);
  }
  const int64_t bh = bhi;
  const int64_t t0 = min((int64_t)r * read_len, T);
  const int64_t t1 = min(t0 + read_len, T);
  const int L = (int)(t1 - t0);
  if (L <= 0) return;
  const int64_t trow0 = (int64_t)f * T + t0;  // first token row of the slab

  // S_fs = S_loc_fs + w * carry of the group, as bf16 hi/lo A fragments (fs is
  // the frame's own state, or the one all frames share)
  const int fs = state_frame >= 0 ? state_frame : f;
  constexpr int64_t E = (int64_t)D * D + D;
  const int NG = (F + G - 1) / G;
  const float *Sg = st + (bh * F + fs) * sstride;
  // G == 1: the carry kernel has written S_f itself (no carries kept)
  const bool has_carry = G > 1;
  const float *Cg = ws + carry_offset + (bh * NG + fs / G) * E;
  const float w = carry_weight(gamma ? gamma + bh * F : nullptr, fs, G);
  if constexpr (kRope) {
    fill_rope_table(rope_tab, rope, f);
    sync_lds();
  }
  const int c = tid % C::ROW_CHUNKS;
  const int r0 = tid / C::ROW_CHUNKS;
  // row strides in 16-byte pieces (host-checked multiples of 8 elements)
  const int64_t snq = qview.sn / 8, sng = gview.sn / 8, sno = oview.sn / 8;
  const uint4 *qb = reinterpret_cast<const uint4 *>(
      static_cast<const uint16_t *>(qview.data) + qview.slab(bh, H) + trow0 * qview.sn);
  const uint4 *gb = reinterpret_cast<const uint4 *>(
      static_cast<const uint16_t *>(gview.data) + gview.slab(bh, H) + trow0 * gview.sn);
  uint4 *ob = reinterpret_cast<uint4 *>(const_cast<uint16_t *>(
      static_cast<const uint16_t *>(oview.data) + oview.slab(bh, H) + trow0 * oview.sn));
  [[maybe_unused]] const PieceRope prope(rope, c);
  // this thread's piece of its first row in the block; blocks are visited in
  // order, so the addresses advance by additions only
  const uint4 *qp = qb + (int64_t)r0 * snq + c;
  const uint4 *gp = gb + (int64_t)r0 * sng + c;
  uint4 rq[C::CPT], rgv[C::CPT];
  // Rows past the split load (and later store) its last row again: each o row
  // depends on its own q and g rows alone, and a row stored twice gets the
  // same value. Without branches the compiler can count these loads and
  // stores and waits at the next block's staging for its loads alone, not for
  // the stores too (the counter covers both): 720p/60s readout -0.5%, d = 128
  // streaming -2%.
  auto load = [&](int blk) {
    const int last = L - 1 - blk * C::BLK;  // the block's last row, >= 0
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int64_t row = min(r0 + i * C::ROWS_PER_PASS, last) - r0;
      rq[i] = ld_stream16<GLA_RO_NT_LOADS>(qp + row * snq);
      rgv[i] = ld_stream16<GLA_RO_NT_LOADS>(gp + row * sng);
    }
    qp += C::BLK * snq;
    gp += C::BLK * sng;
  };
  // the first block's q and g go out before the state: their latency
  // overlaps the state's
  load(0);
  bf16x8 ahi[C::KS], alo[C::KS];
  // The fragments are built in one straight run per case (the carry test is
  // outside the k-step loop, and the normaliser's likewise below), so that the
  // compiler issues every k-step's loads before it waits: with the test
  // inside, each k-step and each of the eight normaliser loads was a memory
  // round trip of its own, 13 (d = 64) to 17 (d = 128) of them before the
  // first token (720p/5s readout 52 -> 50 us).
  {
    const int jcol = 32 * mb + (lane & 31);
    auto build = [&](auto state_at) {
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        float sv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) sv[e] = state_at((16 * ks + 8 * h + e) * D + jcol);
        if constexpr (kRope) {
          // rows i = 16ks + 8h + e of S turned by R_t(f)^T: pair (i, i+1) for even e
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const int pr = 8 * ks + 4 * h + e / 2;
            const float2 cs = rope_tab[pr < rope.Pt ? rope.t_base() + pr : 0];
            const float2 ab = rotate_pair(sv[e], sv[e + 1], make_float2(cs.x, -cs.y));
            sv[e] = ab.x;
            sv[e + 1] = ab.y;
          }
        }
        // S = hi + lo, both bf16
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) split2(sv[2 * e], sv[2 * e + 1], hw[e], lw[e]);
        ahi[ks] = __builtin_bit_cast(bf16x8, make_uint4(hw[0], hw[1], hw[2], hw[3]));
        alo[ks] = __builtin_bit_cast(bf16x8, make_uint4(lw[0], lw[1], lw[2], lw[3]));
      }
    };
    if (has_carry)
      build([&](int idx) { return fmaf(w, Cg[idx], Sg[idx]); });
    else
      build([&](int idx) { return Sg[idx]; });
  }
  float zc[8];
  if (has_carry) {
#pragma unroll
    for (int e = 0; e < 8; ++e) zc[e] = fmaf(w, Cg[D * D + 8 * c + e], Sg[D * D + 8 * c + e]);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) zc[e] = Sg[D * D + 8 * c + e];
  }

  uint4 *op = ob + (int64_t)r0 * sno + c;

  const int tl = 32 * tg + (lane & 31);
  const int nblk = (L + C::BLK - 1) / C::BLK;
  wait_vmem_all();  // no load outstanding into the loop: its waits count its own
  for (int blk = 0; blk < nblk; ++blk) {
    sync_lds();  // the previous block's o rows have been read out of gtile
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int row = r0 + i * C::ROWS_PER_PASS;
      const uint4 w = relu8(rq[i]);
      if constexpr (kRope) {
        // the numerator takes phi(q) spatially turned, the normaliser unturned
        const int l = (int)min(t0 + blk * C::BLK + row, T - 1);
        uint4 qhi, qlo;
        prope.turn(w, l, rope, rope_tab, qhi, qlo);
        *reinterpret_cast<uint4 *>(qtile + row * C::PITCH + c * 16) = qhi;
        *reinterpret_cast<uint4 *>(qtile_lo + row * C::PITCH + c * 16) = qlo;
      } else {
        *reinterpret_cast<uint4 *>(qtile + row * C::PITCH + c * 16) = w;
      }
      *reinterpret_cast<uint4 *>(gtile + row * GP + c * 16) = rgv[i];
      float dp = lo_bf16(w.x) * zc[0];
      dp = fmaf(hi_bf16(w.x), zc[1], dp);
      dp = fmaf(lo_bf16(w.y), zc[2], dp);
      dp = fmaf(hi_bf16(w.y), zc[3], dp);
      dp = fmaf(lo_bf16(w.z), zc[4], dp);
      dp = fmaf(hi_bf16(w.z), zc[5], dp);
      dp = fmaf(lo_bf16(w.w), zc[6], dp);
      dp = fmaf(hi_bf16(w.w), zc[7], dp);
      dp = group_sum<C::ROW_CHUNKS>(dp);  // over the row's pieces
      if (c == 0) den_s[row] = dp;
    }
    sync_lds();
    if (blk + 1 < nblk) load(blk + 1);

    f32x16 acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const uint4 bw =
          *reinterpret_cast<const uint4 *>(qtile + tl * C::PITCH + (16 * ks + 8 * h) * 2);
      const bf16x8 bf = __builtin_bit_cast(bf16x8, bw);
      acc = mfma_32x32x16(ahi[ks], bf, acc);
      acc = mfma_32x32x16(alo[ks], bf, acc);
      if constexpr (kRope) {
        // low parts of the turned queries (times S_hi; S_lo x q_lo is below fp32 rounding)
        const uint4 bl =
            *reinterpret_cast<const uint4 *>(qtile_lo + tl * C::PITCH + (16 * ks + 8 * h) * 2);
        acc = mfma_32x32x16(ahi[ks], __builtin_bit_cast(bf16x8, bl), acc);
      }
    }
    const float inv = __builtin_amdgcn_rcpf(den_s[tl] + eps);
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      uint2 *cell = reinterpret_cast<uint2 *>(gtile + tl * GP + (32 * mb + 8 * rg + 4 * h) * 2);
      const uint2 gv = *cell;
      const float o0 = fast_sigmoid(lo_bf16(gv.x)) * (acc[4 * rg + 0] * inv);
      const float o1 = fast_sigmoid(hi_bf16(gv.x)) * (acc[4 * rg + 1] * inv);
      const float o2 = fast_sigmoid(lo_bf16(gv.y)) * (acc[4 * rg + 2] * inv);
      const float o3 = fast_sigmoid(hi_bf16(gv.y)) * (acc[4 * rg + 3] * inv);
      *cell = make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
    }
    sync_lds();
    {
      const int last = L - 1 - blk * C::BLK;
#pragma unroll
      for (int i = 0; i < C::CPT; ++i) {
        const int row = min(r0 + i * C::ROWS_PER_PASS, last);
        const uint4 ov = *reinterpret_cast<const uint4 *>(gtile + row * GP + c * 16);
        uint4 *dst = op + (int64_t)(row - r0) * sno;
        if constexpr (GLA_RO_NT_STORES != 0) {
          const u32x4 x = {ov.x, ov.y, ov.z, ov.w};
          __builtin_nontemporal_store(x, reinterpret_cast<u32x4 *>(dst));
        } else {
          *dst = ov;
        }
      }
    }
    op += C::BLK * sno;
  }
}

template <int D, bool kRope>
void kv_launch(const Plan &p, const KvArgs &a, RopeK rope, int64_t grid, hipStream_t s) {
  const size_t lds = kRope ? (size_t)rope.entries() * sizeof(float2) : 0;
  hipLaunchKernelGGL((kv_mfma_kernel<D, kRope>), dim3((unsigned)grid), dim3(kThreads), lds, s,
                     a.k, a.v, a.H, a.gamma, a.ws, p.F, p.T, p.P, p.G, p.part_len, rope);
}

template <int D, bool kRope>
void readout_launch(const Plan &p, const ReadoutArgs &a, RopeK rope, int64_t grid,
                    hipStream_t s) {
  const size_t lds = kRope ? (size_t)rope.entries() * sizeof(float2) : 0;
  hipLaunchKernelGGL((readout_kernel<D, kRope>), dim3((unsigned)grid), dim3(kThreads), lds, s,
                     a.q, a.g, a.o, a.H, a.gamma, a.ws, a.states.base, a.states.stride, p.F,
                     p.T, p.G, p.carry_offset(), p.R, p.read_len, a.eps, a.state_frame, rope,
                     a.heads_fastest);
}

}  // namespace

bool mfma_supports(int d) { return d == 32 || d == 64 || d == 128; }

hipError_t launch_kv_mfma(const Plan &p, const KvArgs &a, hipStream_t s) {
  const int64_t grid = p.BH * p.NG * p.P;
  if (grid == 0) return hipSuccess;
  RopeK rope = a.rope;
  rope.frames = p.G;  // temporal table rows: the group's frames
  const bool r = rope.on != 0;
  switch (p.d) {
    case 32: r ? kv_launch<32, true>(p, a, rope, grid, s) : kv_launch<32, false>(p, a, rope, grid, s); break;
    case 64: r ? kv_launch<64, true>(p, a, rope, grid, s) : kv_launch<64, false>(p, a, rope, grid, s); break;
    case 128: r ? kv_launch<128, true>(p, a, rope, grid, s) : kv_launch<128, false>(p, a, rope, grid, s); break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_readout_mfma(const Plan &p, const ReadoutArgs &a, hipStream_t s) {
  const int64_t grid = p.BH * p.F * p.R;
  if (grid == 0 || p.T == 0) return hipSuccess;
  RopeK rope = a.rope;
  rope.frames = 1;  // a readout workgroup covers one frame
  const bool r = rope.on != 0;
  switch (p.d) {
    case 32: r ? readout_launch<32, true>(p, a, rope, grid, s) : readout_launch<32, false>(p, a, rope, grid, s); break;
    case 64: r ? readout_launch<64, true>(p, a, rope, grid, s) : readout_launch<64, false>(p, a, rope, grid, s); break;
    case 128: r ? readout_launch<128, true>(p, a, rope, grid, s) : readout_launch<128, false>(p, a, rope, grid, s); break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace gla
