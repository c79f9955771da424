// anchor.hip -- the gated softmax anchor: softmax attention over whole frames
// with sink frames and a local temporal window, gated like the linear layers.
//
//   o_t = sigmoid(g_t) (.) sum_{s in V(t)} softmax_s(scale q_t . k_s) v_s
//
// Keys are F frames of T tokens; queries are the tokens of the last Fq key
// frames. V(t) is every key (full mode), or the key frames i <= f with
// i < n_sink or i > f - window, f the query's key frame (frame-causal): at
// most two contiguous key ranges, the sink frames and the window.
//
// Work items: one per (slab, query segment, tile of queries). A segment is
// the whole query range in full mode and one frame in frame-causal mode, so
// every query of a tile sees the same key ranges and no per-element mask is
// needed except at the end of a range.
//
// Matrix-core kernel (bf16, d = 32, 64, 128), online softmax in fp32:
// 128 queries per workgroup, 32 per wave; blocks of 64 keys move through LDS
// (double-buffered, one barrier per block). The scores are formed transposed,
// S^T = K Q^T on the 32x32x16 MFMA (row = key, column = query), so each lane
// owns one query and 16 keys of each 32-key half: the running max needs one
// exchange between the two lane halves per block, the running sum none until
// the end. The probabilities' accumulator layout is the B operand of
// O^T = V^T P^T as it stands, with the contraction index relabelled: slot e of
// lane half h is key 16kk + 4h + e (e < 4) or 16kk + 8 + 4h + (e - 4); V^T is
// read from LDS with ds_read_b64_tr_b16 in that same key order.
//
// P V runs on the fp16 matrix cores: V is converted from bf16 to fp16 as it is
// staged (exact for magnitudes in [2^-14, 65504]) and the probabilities are
// packed to fp16 (11 significant bits against bf16's 8; worst slab-relative
// error on the shape sweep 5.2e-3 against 1.4e-2 with bf16 probabilities).
// A workgroup also takes the largest |v| of the keys it staged. If that lies
// outside [2^-6, 65504] (values fp16 cannot hold, or a V so small that fp16's
// subnormals would cost it precision) it writes a marker instead of its
// output, and a second launch recomputes exactly those tiles with bf16 P V,
// the probabilities split into bf16 hi + lo pairs (about 16 significant
// bits, 3.9e-3 on the sweep); every other workgroup of that launch reads one
// element and exits.
//
// Vector-ALU kernel (fp32 inputs, other d, or forced): one query per thread,
// blocks of 32 keys through LDS.
#include <type_traits>

#include "common.hpp"
#include "mfma_util.hpp"
#include "plan.hpp"

namespace gla {
namespace {

// The key ranges [a0, a1) and [b0, b1) (in tokens) seen by segment seg.
struct KeyRanges {
  int64_t a0, a1, b0, b1;
};

// a wave-uniform 64-bit value, read into scalar registers
__device__ __forceinline__ int64_t uniform64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ KeyRanges anchor_ranges(const AnchorArgs &a, int seg) {
  const int64_t T = a.T;
  KeyRanges r{0, (int64_t)a.F * T, 0, 0};
  if (!a.causal) return r;
  const int f = a.F - a.Fq + seg;  // the segment's key frame
  const int64_t hi = (int64_t)(f + 1) * T;
  const int64_t sink_end = (int64_t)min(a.n_sink, f + 1) * T;
  const int64_t win_lo = a.window > 0 ? (int64_t)max(0, f - a.window + 1) * T : 0;
  if (win_lo <= sink_end) {
    r.a1 = hi;  // the sinks run into the window: one range
  } else {
    r.a1 = sink_end;
    r.b0 = win_lo;
    r.b1 = hi;
  }
  return r;
}

// ---------------------------------------------------------------------------
// Matrix-core kernel
// ---------------------------------------------------------------------------
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// two floats -> packed fp16, rounded toward zero (v_cvt_pkrtz_f16_f32)
__device__ __forceinline__ uint32_t pack_f16x2_rtz(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}

// eight bf16 -> eight fp16, with the running maximum of their magnitudes
__device__ __forceinline__ uint4 bf16x8_to_f16x8(uint4 v, float &vmax) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = lo_bf16(w[i]), hi = hi_bf16(w[i]);
    vmax = fmaxf(vmax, fmaxf(fabsf(lo), fabsf(hi)));
    w[i] = pack_f16x2_rtz(lo, hi);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

__device__ __forceinline__ f32x16 mfma_32x32x16_f16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// bf16 bits of a quiet NaN with payload 1: written by a workgroup of the fp16
// pass at its tile's first output element when the tile is to be recomputed
// (arithmetic never produces this payload: a NaN result is the canonical 0x7FC0)
constexpr uint16_t kRedoMark = 0x7FC1;
// |v| range in which fp16 P V is taken
constexpr float kF16VMin = 0x1p-6f, kF16VMax = 65504.f;
template <int D>
struct AmCfg {
  static constexpr int BM = 128;               // queries per workgroup (32 per wave)
  static constexpr int BN = 64;                // keys per block
  // LDS row pitches (64 banks of 4 bytes): K rows are read whole, 16 bytes a
  // lane on 16 consecutive rows per pass (a pitch of 4 mod 8 dwords keeps them
  // apart); V goes through transposed reads of 4 consecutive rows x 64 bytes
  // per pass (a pitch of 16 or 48 mod 64 dwords). Both measured conflict-free
  // with the LDS bank-conflict counter.
  static constexpr int KPITCH = 2 * D + 16;
  static constexpr int VPITCH = 2 * D + (D == 32 ? 0 : 64);
  static constexpr int PITCH = KPITCH;         // the epilogue's g / o rows
  static constexpr int KS = D / 16;            // k-steps of the scores
  static constexpr int JB = D / 32;            // 32-feature blocks of the output
  static constexpr int ROW_CHUNKS = D / 8;     // 16-byte pieces per row
  static constexpr int RPP = 256 / ROW_CHUNKS; // rows per staging pass
  static constexpr int CPT = BN / RPP;         // pieces per thread per tensor and block
  static constexpr int KTILE = BN * KPITCH;
  static constexpr int BUF = KTILE + BN * VPITCH;  // one K and one V tile
  static constexpr int SMEM = 2 * BUF;             // double-buffered
  static constexpr int GPT = BM / RPP;         // g / o pieces per thread in the epilogue
  static_assert(BM * PITCH <= SMEM, "the epilogue tile reuses the K/V buffers");
};

// Waves per SIMD the compiler must allow.
//  - fp16 P V: d = 64 fits 3 waves (168 VGPRs, 16 bytes spilled; 720p/60s
//    window of 4: 12.6 ms at 2 waves -> 11.6 ms), d = 128 takes 256 VGPRs
//    (2 waves).
//  - bf16 hi + lo P V (the recomputed tiles): d = 64 takes 222 VGPRs (2 waves;
//    forcing 3 spills and measured slower) and d = 128 would take 260 (1
//    wave): held to 2, it spills 16 bytes and runs 20% faster than at 1.
template <int D, bool kF16>
constexpr int kAnchorWaves = D == 64 ? (kF16 ? 3 : 2) : D == 128 ? 2 : 1;

// One tile of queries, work item wg = (slab, segment, tile), with the
// workgroup's LDS. kF16: P V in fp16 (a tile whose V is out of range is marked
// instead of computed); otherwise P V in bf16 with hi + lo probabilities.
template <int D, bool kF16>
__device__ __forceinline__ void anchor_tile(const AnchorArgs &a, int tiles_per_seg,
                                            int64_t seg_len, int64_t wg, char *smem) {
  using C = AmCfg<D>;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;
  const int n = lane & 31;
  const int nseg = a.causal ? a.Fq : 1;
  // The work item is uniform, but 64-bit divisions leave it in vector
  // registers: read it into scalars, so that the key ranges and the block
  // addresses derived from it are scalar work (vector-ALU time is what bounds
  // this kernel)
  const int tile = __builtin_amdgcn_readfirstlane((int)(wg % tiles_per_seg));
  const int seg = __builtin_amdgcn_readfirstlane((int)((wg / tiles_per_seg) % nseg));
  const int bh = __builtin_amdgcn_readfirstlane((int)(wg / ((int64_t)tiles_per_seg * nseg)));
  const int64_t Nq = (int64_t)a.Fq * a.T, Nk = (int64_t)a.F * a.T;
  const int64_t q0 = (int64_t)seg * seg_len + (int64_t)tile * C::BM;  // first query row
  const int nq = (int)min((int64_t)C::BM, seg_len - (int64_t)tile * C::BM);
  uint16_t *os = static_cast<uint16_t *>(a.o) + bh * Nq * D;
  KeyRanges kr = anchor_ranges(a, seg);
  kr = KeyRanges{uniform64(kr.a0), uniform64(kr.a1), uniform64(kr.b0), uniform64(kr.b1)};
  const int nb_a = __builtin_amdgcn_readfirstlane((int)((kr.a1 - kr.a0 + C::BN - 1) / C::BN));
  const int nb = __builtin_amdgcn_readfirstlane(nb_a + (int)((kr.b1 - kr.b0 + C::BN - 1) / C::BN));

  const uint16_t *qs = static_cast<const uint16_t *>(a.q) + bh * Nq * D;
  const uint16_t *ks = static_cast<const uint16_t *>(a.k) + bh * Nk * D;
  const uint16_t *vs = static_cast<const uint16_t *>(a.v) + bh * Nk * D;

  // this lane's query (column n of the wave's 32) as B fragments, k = feature
  const int qrow = 32 * wave + n;
  bf16x8 qf[C::KS];
#pragma unroll
  for (int kk = 0; kk < C::KS; ++kk) {
    uint4 w = make_uint4(0, 0, 0, 0);
    if (qrow < nq) w = *reinterpret_cast<const uint4 *>(qs + (q0 + qrow) * D + 16 * kk + 8 * h);
    qf[kk] = __builtin_bit_cast(bf16x8, w);
  }

  // staging: this thread's 16-byte pieces of a block (rows r0 + i * RPP, piece c)
  const int c = tid % C::ROW_CHUNKS;
  const int r0 = tid / C::ROW_CHUNKS;
  uint4 rk[C::CPT], rv[C::CPT];
  int nv_next = 0;  // valid keys of the block in the registers
  auto load_block = [&](int b) {
    const int64_t start = b < nb_a ? kr.a0 + (int64_t)b * C::BN : kr.b0 + (int64_t)(b - nb_a) * C::BN;
    const int64_t end = b < nb_a ? kr.a1 : kr.b1;
    const int nv = (int)min((int64_t)C::BN, end - start);
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      // rows past the range load its last key again (in bounds, finite): the
      // softmax gives them probability 0, so neither K nor V of them counts,
      // and the loads need no branch or zero fill
      // a scalar block base plus a 32-bit offset within the block
      const int row = min(r0 + i * C::RPP, nv - 1);
      const uint32_t off = (uint32_t)(row * D + 8 * c);
      rk[i] = ld_stream16<false>(reinterpret_cast<const uint4 *>(ks + start * D + off));
      rv[i] = ld_stream16<false>(reinterpret_cast<const uint4 *>(vs + start * D + off));
    }
    nv_next = nv;
  };
  float vmax = 0.f;  // largest |v| staged by this thread (fp16 pass)
  auto store_block = [&](int buf) {
    char *kt = smem + buf * C::BUF;
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int row = r0 + i * C::RPP;
      *reinterpret_cast<uint4 *>(kt + row * C::KPITCH + 16 * c) = rk[i];
      *reinterpret_cast<uint4 *>(kt + C::KTILE + row * C::VPITCH + 16 * c) =
          kF16 ? bf16x8_to_f16x8(rv[i], vmax) : rv[i];
    }
  };

  // running state of the lane's query: max (log2 domain), partial sum over
  // this half's keys, output O^T in the accumulator layout (feature rows)
  const float cl2 = a.scale * 1.44269504088896340736f;  // scale * log2(e)
  float m_run = -1e30f, l_run = 0.f;
  f32x16 o[C::JB];
#pragma unroll
  for (int jb = 0; jb < C::JB; ++jb)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[jb][r] = 0.f;

  const int j16 = lane & 15;
  const int grp16 = (lane >> 4) & 1;
  if (nb > 0) {
    load_block(0);
    store_block(0);
  }
  int nv = nv_next;
  sync_lds();
  // the query fragments and the first block have landed (otherwise the wait
  // for them sits inside the loop and takes the next block's prefetch with it:
  // 720p/60s window of 4 11.39 -> 11.2 ms; every key at 720p/5s 3.57 -> 3.50)
  wait_vmem_all();
  for (int b = 0; b < nb; ++b) {
    const int buf = b & 1;
    if (b + 1 < nb) load_block(b + 1);
    const lds_char *vt = (const lds_char *)(smem + buf * C::BUF + C::KTILE);

    // scores S^T: two 32-key blocks x the wave's 32 queries
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < C::KS; ++kk) {
        const bf16x8 kf = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const uint4 *>(smem + buf * C::BUF + (32 * kb + n) * C::KPITCH +
                                                     (16 * kk + 8 * h) * 2));
        s[kb] = mfma_32x32x16(kf, qf[kk], s[kb]);
      }
    }
    // online softmax over the block (keys past nv are not there; only the
    // last block of a range is partial)
    // probabilities as packed pairs, per 32-key block: fp16 (fp16 pass), or
    // p = hi + lo with both bf16 (bf16 pass: one more MFMA per P V step)
    uint32_t pw[2][8];
    [[maybe_unused]] uint32_t pl[kF16 ? 1 : 2][8];
    // the last block of a range: keys past nv get a score whose probability
    // is 0 (one softmax path for every block: with a second, masked copy the
    // two paths held the output accumulators in different registers and
    // copied them at the join)
    if (nv < C::BN) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
          s[kb][r] = key < nv ? s[kb][r] : -1e30f;
        }
    }
    {
      float mx = -1e30f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx *= cl2;
      // Lazy rescaling: the reference m_run moves (and O, l are rescaled)
      // only when some query's maximum exceeds it by more than 8 (a factor
      // 256): the probabilities stay below 2^8 and O, l keep one reference,
      // so the result is unchanged. The test takes each lane half's own
      // maximum (if neither half's passes, the query's cannot), so the
      // exchange between the halves (an LDS round trip) is needed only in the
      // rare branch, which the whole wave takes together.
      if (__builtin_amdgcn_read_exec() & __ballot(mx > m_run + 8.f)) {
        const float m_new = fmaxf(m_run, fmaxf(mx, __shfl_xor(mx, 32)));
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int jb = 0; jb < C::JB; ++jb)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[jb][r] *= alpha;
      }
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb][r], cl2, -m_run));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kb][r + 1], cl2, -m_run));
          if constexpr (kF16) {
            // the normaliser sums the fp16 probabilities P V takes (one
            // v_dot2_f32_f16 a pair instead of two additions)
            pw[kb][r >> 1] = pack_f16x2_rtz(p0, p1);
            psum = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pw[kb][r >> 1]),
                                          f16x2{(_Float16)1.f, (_Float16)1.f}, psum, false);
          } else {
            psum += p0 + p1;
            split2(p0, p1, pw[kb][r >> 1], pl[kb][r >> 1]);
          }
        }
      l_run += psum;
    }

    // O^T += V^T P^T over the block's 4 k-steps of 16 keys
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int kb = kk >> 1, g0 = 2 * (kk & 1);  // accumulator row groups g0, g0 + 1
      const uint4 pu = make_uint4(pw[kb][2 * g0], pw[kb][2 * g0 + 1], pw[kb][2 * g0 + 2], pw[kb][2 * g0 + 3]);
      const int rowA = 16 * kk + 4 * h + (j16 >> 2);
#pragma unroll
      for (int jb = 0; jb < C::JB; ++jb) {
        const int col = 32 * jb + 16 * grp16 + 4 * (j16 & 3);
        const i16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4 *)(vt + rowA * C::VPITCH + col * 2));
        const i16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4 *)(vt + (rowA + 8) * C::VPITCH + col * 2));
        const i16x8 x = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        if constexpr (kF16) {
          o[jb] = mfma_32x32x16_f16(__builtin_bit_cast(f16x8, x), __builtin_bit_cast(f16x8, pu), o[jb]);
        } else {
          const uint4 lu = make_uint4(pl[kb][2 * g0], pl[kb][2 * g0 + 1], pl[kb][2 * g0 + 2],
                                      pl[kb][2 * g0 + 3]);
          o[jb] = mfma_32x32x16(__builtin_bit_cast(bf16x8, x), __builtin_bit_cast(bf16x8, pu), o[jb]);
          o[jb] = mfma_32x32x16(__builtin_bit_cast(bf16x8, x), __builtin_bit_cast(bf16x8, lu), o[jb]);
        }
      }
    }
    if (b + 1 < nb) {
      store_block(buf ^ 1);
      nv = nv_next;
    }
    sync_lds();
  }

  if constexpr (kF16) {
    // the workgroup's largest staged |v| (the K/V buffers are free after the
    // loop's last barrier): out of the fp16 range, mark the tile for the bf16
    // pass and write nothing else
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) vmax = fmaxf(vmax, __shfl_xor(vmax, off));
    float *wmax = reinterpret_cast<float *>(smem);
    if (lane == 0) wmax[wave] = vmax;
    sync_lds();
    vmax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    sync_lds();  // wmax is read before the epilogue reuses the LDS
    if (nb > 0 && !(vmax >= kF16VMin && vmax <= kF16VMax)) {
      if (tid == 0) os[q0 * D] = kRedoMark;
      return;
    }
  }
  // epilogue: o = sigmoid(g) * O / l, through LDS so that g is read and o is
  // written as whole rows (the K/V buffers are free after the last barrier)
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = nb > 0 ? __builtin_amdgcn_rcpf(l_tot) : 0.f;
  const uint16_t *gs = static_cast<const uint16_t *>(a.g) + bh * Nq * D;
#pragma unroll
  for (int i = 0; i < C::GPT; ++i) {
    const int row = r0 + i * C::RPP;
    uint4 w = make_uint4(0, 0, 0, 0);
    if (row < nq) w = ld_stream16<true>(reinterpret_cast<const uint4 *>(gs + (q0 + row) * D + 8 * c));
    *reinterpret_cast<uint4 *>(smem + row * C::PITCH + 16 * c) = w;
  }
  sync_lds();
#pragma unroll
  for (int jb = 0; jb < C::JB; ++jb)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      uint2 *cell = reinterpret_cast<uint2 *>(smem + qrow * C::PITCH + (32 * jb + 8 * rg + 4 * h) * 2);
      const uint2 gv = *cell;
      uint2 ow;
      ow.x = pack_bf16x2(fast_sigmoid(lo_bf16(gv.x)) * (o[jb][4 * rg + 0] * inv),
                         fast_sigmoid(hi_bf16(gv.x)) * (o[jb][4 * rg + 1] * inv));
      ow.y = pack_bf16x2(fast_sigmoid(lo_bf16(gv.y)) * (o[jb][4 * rg + 2] * inv),
                         fast_sigmoid(hi_bf16(gv.y)) * (o[jb][4 * rg + 3] * inv));
      *cell = ow;
    }
  sync_lds();
#pragma unroll
  for (int i = 0; i < C::GPT; ++i) {
    const int row = r0 + i * C::RPP;
    if (row < nq)
      st_stream16(reinterpret_cast<uint4 *>(os + (q0 + row) * D + 8 * c),
                  *reinterpret_cast<const uint4 *>(smem + row * C::PITCH + 16 * c));
  }
}

// A redo workgroup checks this many tiles' marks and computes the marked ones
// in turn: on ordinary inputs the launch is 8 times fewer workgroups that each
// make 8 loads (one per tile: 125 us at 720p/60s), and with every tile marked
// it still has thousands of workgroups.
constexpr int kRedoBatch = 8;

// kF16: the fp16 pass, one tile per workgroup. Otherwise the bf16 hi + lo pass
// over the tiles the fp16 pass marked, kRedoBatch tiles per workgroup.
template <int D, bool kF16>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kAnchorWaves<D, kF16>))) void
anchor_mfma_kernel(AnchorArgs a, int tiles_per_seg, int64_t seg_len) {
  using C = AmCfg<D>;
  __shared__ __attribute__((aligned(16))) char smem[C::SMEM];
  if constexpr (kF16) {
    anchor_tile<D, true>(a, tiles_per_seg, seg_len, xcd_contiguous(blockIdx.x, gridDim.x), smem);
  } else {
    const int nseg = a.causal ? a.Fq : 1;
    const int64_t total = a.BH * nseg * (int64_t)tiles_per_seg;
    const int64_t Nq = (int64_t)a.Fq * a.T;
    // the marks first, all loads in flight together (a tile's first output
    // element, read as the aligned word that holds it: D is even)
    uint32_t mark[kRedoBatch];
#pragma unroll
    for (int i = 0; i < kRedoBatch; ++i) {
      const int64_t wg = min((int64_t)blockIdx.x * kRedoBatch + i, total - 1);
      const int tile = (int)(wg % tiles_per_seg);
      const int seg = (int)((wg / tiles_per_seg) % nseg);
      const int64_t bh = wg / ((int64_t)tiles_per_seg * nseg);
      const int64_t q0 = (int64_t)seg * seg_len + (int64_t)tile * C::BM;
      const uint32_t *m = reinterpret_cast<const uint32_t *>(static_cast<const uint16_t *>(a.o) +
                                                             (bh * Nq + q0) * D);
      mark[i] = __builtin_nontemporal_load(m);
    }
#pragma unroll 1
    for (int i = 0; i < kRedoBatch; ++i) {
      const int64_t wg = (int64_t)blockIdx.x * kRedoBatch + i;
      if (wg >= total || (mark[i] & 0xFFFFu) != kRedoMark) continue;
      anchor_tile<D, false>(a, tiles_per_seg, seg_len, wg, smem);
      sync_lds();  // the next marked tile reuses the LDS
    }
  }
}

// ---------------------------------------------------------------------------
// Vector-ALU kernel: one query per thread, 64 per workgroup
// ---------------------------------------------------------------------------
constexpr int kValuQ = 64;
constexpr int kValuKeys = 32;

template <typename TIn, int D>
__global__ __launch_bounds__(kValuQ) void anchor_valu_kernel(AnchorArgs a, int tiles_per_seg,
                                                             int64_t seg_len) {
  __shared__ float sk[kValuKeys][D];
  __shared__ float sv[kValuKeys][D];
  const int tid = threadIdx.x;
  const int nseg = a.causal ? a.Fq : 1;
  const int64_t wg = blockIdx.x;
  const int tile = (int)(wg % tiles_per_seg);
  const int seg = (int)((wg / tiles_per_seg) % nseg);
  const int64_t bh = wg / ((int64_t)tiles_per_seg * nseg);
  const int64_t Nq = (int64_t)a.Fq * a.T, Nk = (int64_t)a.F * a.T;
  const int64_t q0 = (int64_t)seg * seg_len + (int64_t)tile * kValuQ;
  const int nq = (int)min((int64_t)kValuQ, seg_len - (int64_t)tile * kValuQ);
  const bool active = tid < nq;
  const KeyRanges kr = anchor_ranges(a, seg);
  const TIn *qs = static_cast<const TIn *>(a.q) + bh * Nq * D;
  const TIn *ks = static_cast<const TIn *>(a.k) + bh * Nk * D;
  const TIn *vs = static_cast<const TIn *>(a.v) + bh * Nk * D;
  float q[D], acc[D];
#pragma unroll
  for (int x = 0; x < D; ++x) {
    q[x] = active ? Elem<TIn>::load(qs, (q0 + tid) * D + x) * a.scale : 0.f;
    acc[x] = 0.f;
  }
  float m_run = -1e30f, l_run = 0.f;
  for (int part = 0; part < 2; ++part) {
    const int64_t lo = part ? kr.b0 : kr.a0, hi = part ? kr.b1 : kr.a1;
    for (int64_t s0 = lo; s0 < hi; s0 += kValuKeys) {
      const int nk = (int)min((int64_t)kValuKeys, hi - s0);
      __syncthreads();
      for (int e = tid; e < kValuKeys * D; e += kValuQ) {
        const int r = e / D, x = e % D;
        sk[r][x] = r < nk ? Elem<TIn>::load(ks, (s0 + r) * D + x) : 0.f;
        sv[r][x] = r < nk ? Elem<TIn>::load(vs, (s0 + r) * D + x) : 0.f;
      }
      __syncthreads();
      // one key at a time: rescale by the change of the running max
      for (int r = 0; r < nk; ++r) {
        float dot = 0.f;
#pragma unroll
        for (int x = 0; x < D; ++x) dot = fmaf(q[x], sk[r][x], dot);
        const float m_new = fmaxf(m_run, dot);
        const float alpha = __expf(m_run - m_new), p = __expf(dot - m_new);
        m_run = m_new;
        l_run = fmaf(l_run, alpha, p);
#pragma unroll
        for (int x = 0; x < D; ++x) acc[x] = fmaf(p, sv[r][x], acc[x] * alpha);
      }
    }
  }
  if (!active) return;
  const TIn *gs = static_cast<const TIn *>(a.g) + bh * Nq * D;
  TIn *os = static_cast<TIn *>(a.o) + bh * Nq * D;
  const float inv = 1.f / l_run;
#pragma unroll
  for (int x = 0; x < D; ++x) {
    const int64_t i = (q0 + tid) * D + x;
    const float gt = Elem<TIn>::load(gs, i);
    Elem<TIn>::store(os, i, acc[x] * inv / (1.f + expf(-gt)));
  }
}

template <int D>
void anchor_mfma_launch(const AnchorArgs &a, int64_t seg_len, bool f16, hipStream_t s) {
  const int nseg = a.causal ? a.Fq : 1;
  const int tiles = (int)((seg_len + AmCfg<D>::BM - 1) / AmCfg<D>::BM);
  const int64_t items = a.BH * nseg * tiles;
  if (f16)
    hipLaunchKernelGGL((anchor_mfma_kernel<D, true>), dim3((unsigned)items), dim3(256), 0, s, a,
                       tiles, seg_len);
  else
    hipLaunchKernelGGL((anchor_mfma_kernel<D, false>),
                       dim3((unsigned)((items + kRedoBatch - 1) / kRedoBatch)), dim3(256), 0, s, a,
                       tiles, seg_len);
}

template <typename TIn, int D>
void anchor_valu_launch(const AnchorArgs &a, int64_t seg_len, hipStream_t s) {
  const int nseg = a.causal ? a.Fq : 1;
  const int tiles = (int)((seg_len + kValuQ - 1) / kValuQ);
  hipLaunchKernelGGL((anchor_valu_kernel<TIn, D>), dim3((unsigned)(a.BH * nseg * tiles)),
                     dim3(kValuQ), 0, s, a, tiles, seg_len);
}

template <typename TIn>
hipError_t anchor_valu_dispatch(const AnchorArgs &a, int64_t seg_len, hipStream_t s) {
  switch (a.d) {
    case 16: anchor_valu_launch<TIn, 16>(a, seg_len, s); break;
    case 32: anchor_valu_launch<TIn, 32>(a, seg_len, s); break;
    case 64: anchor_valu_launch<TIn, 64>(a, seg_len, s); break;
    case 128: anchor_valu_launch<TIn, 128>(a, seg_len, s); break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int64_t anchor_tiles(const AnchorArgs &a, Path path) {
  const int64_t seg_len = a.causal ? a.T : (int64_t)a.Fq * a.T;
  const int64_t per = path == Path::kMfma ? AmCfg<64>::BM : kValuQ;
  return a.BH * (a.causal ? a.Fq : 1) * ((seg_len + per - 1) / per);
}

namespace {
hipError_t anchor_mfma_dispatch(const AnchorArgs &a, int64_t seg_len, bool f16, hipStream_t s) {
  switch (a.d) {
    case 32: anchor_mfma_launch<32>(a, seg_len, f16, s); break;
    case 64: anchor_mfma_launch<64>(a, seg_len, f16, s); break;
    case 128: anchor_mfma_launch<128>(a, seg_len, f16, s); break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_anchor(const AnchorArgs &a, int dtype, Path path, hipStream_t s) {
  const int64_t seg_len = a.causal ? a.T : (int64_t)a.Fq * a.T;
  if (a.BH == 0 || seg_len == 0 || a.Fq == 0) return hipSuccess;
  if (path == Path::kMfma) return anchor_mfma_dispatch(a, seg_len, true, s);
  return dtype == 0 ? anchor_valu_dispatch<float>(a, seg_len, s)
                    : anchor_valu_dispatch<bf16_t>(a, seg_len, s);
}

hipError_t launch_anchor_redo(const AnchorArgs &a, Path path, hipStream_t s) {
  const int64_t seg_len = a.causal ? a.T : (int64_t)a.Fq * a.T;
  if (a.BH == 0 || seg_len == 0 || a.Fq == 0 || path != Path::kMfma) return hipSuccess;
  return anchor_mfma_dispatch(a, seg_len, false, s);
}

}  // namespace gla
