// rope_tab.hpp -- the LDS table of 3D rotary turns and the per-piece turn of
// the matrix-core kernels (forward kv and readout, backward bwd_k).
#pragma once

#include "common.hpp"
#include "mfma_util.hpp"
#include "plan.hpp"

namespace gla {

// ---------------------------------------------------------------------------
// 3D rotary positions
//
// Temporal and spatial sections turn disjoint feature pairs, so the rotation
// of a token factors as R = R_t(frame) R_s(y, x), and R_t is shared by every
// token of a frame. The kernels therefore turn each token by R_s only, and
// apply R_t once per frame to a d x d operand: kv turns the rows of the
// frame's sum U_f (U = sum R_t R_s phi(k) v^T = R_t sum R_s phi(k) v^T), the
// readout turns the rows of S_f by R_t^T ((R_t R_s phi(q))^T S = (R_s phi(q))^T
// R_t^T S). The (cos, sin) values come from an LDS table (RopeK::entries()),
// filled once per workgroup.
// ---------------------------------------------------------------------------
__device__ inline void fill_rope_table(float2 *tab, const RopeK &r, int f0) {
  const int n = r.entries();
  for (int e = threadIdx.x; e < n; e += blockDim.x) {
    float2 cs = make_float2(1.f, 0.f);
    if (e >= r.t_base()) {
      const int i = e - r.t_base(), fi = i / r.Pt;
      cs = rope_cs((double)r.frame_offset + f0 + fi, i - fi * r.Pt, r.Pt, r.log_theta);
    } else if (e >= r.x_base()) {
      const int i = e - r.x_base(), x = i / r.Pw;
      cs = rope_cs((double)x, i - x * r.Pw, r.Pw, r.log_theta);
    } else if (e >= r.y_base()) {
      const int i = e - r.y_base(), y = i / r.Ph;
      cs = rope_cs((double)y, i - y * r.Ph, r.Ph, r.log_theta);
    }
    tab[e] = cs;
  }
}

// The whole turn of feature pair pp of a token at (y, x) in the table's one
// frame (filled with frames = 1: entry t_base() + pp is that frame's turn).
__device__ __forceinline__ float2 pair_turn(const RopeK &r, const float2 *tab, int y, int x,
                                            int pp) {
  if (pp < r.Pt) return tab[r.t_base() + pp];
  if (pp < r.Pt + r.Ph) return tab[r.y_base() + y * r.Ph + pp - r.Pt];
  return tab[r.x_base() + x * r.Pw + pp - r.Pt - r.Ph];
}

// The spatial turn of one 16-byte piece (8 bf16 = feature pairs 4c .. 4c+3) of
// the token at in-frame index l. is_t / is_h mark which of the four pairs are
// temporal (not turned here) or in the height section.
struct PieceRope {
  bool is_t[4], is_h[4];
  int c4;
  __device__ PieceRope(const RopeK &r, int c) : c4(4 * c) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      is_t[e] = c4 + e < r.Pt;
      is_h[e] = c4 + e < r.Pt + r.Ph;
    }
  }
  // The turned features as hi + lo, both bf16 (hi = bf16(x), lo = bf16(x - hi):
  // together 16 significant bits, like the state's split in the readout).
  __device__ __forceinline__ void turn(uint4 w, int l, const RopeK &r, const float2 *tab,
                                       uint4 &hi, uint4 &lo) const {
    int y, x;
    grid_pos(l, r.grid_w, r.inv_gw, y, x);
    // entry of pair 4c + e: by + e in the height section, bx + e in the width one
    const int by = r.y_base() + y * r.Ph - r.Pt + c4;
    const int bx = r.x_base() + x * r.Pw - r.Pt - r.Ph + c4;
    const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
    uint32_t hv[4], lv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = is_t[e] ? -e : (is_h[e] ? by : bx);
      const float2 cs = tab[idx + e];
      const float2 ab = rotate_pair(lo_bf16(wv[e]), hi_bf16(wv[e]), cs);
      hv[e] = pack_bf16x2(ab.x, ab.y);
      lv[e] = pack_bf16x2(ab.x - lo_bf16(hv[e]), ab.y - hi_bf16(hv[e]));
    }
    hi = make_uint4(hv[0], hv[1], hv[2], hv[3]);
    lo = make_uint4(lv[0], lv[1], lv[2], lv[3]);
  }
  // The whole turn (temporal pairs too, from a table filled for one frame),
  // as hi + lo: for kernels whose operands are not summed over a frame first.
  __device__ __forceinline__ void turn_whole(uint4 w, int l, const RopeK &r, const float2 *tab,
                                             uint4 &hi, uint4 &lo) const {
    int y, x;
    grid_pos(l, r.grid_w, r.inv_gw, y, x);
    const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
    uint32_t hv[4], lv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float2 ab = rotate_pair(lo_bf16(wv[e]), hi_bf16(wv[e]), pair_turn(r, tab, y, x, c4 + e));
      hv[e] = pack_bf16x2(ab.x, ab.y);
      lv[e] = pack_bf16x2(ab.x - lo_bf16(hv[e]), ab.y - hi_bf16(hv[e]));
    }
    hi = make_uint4(hv[0], hv[1], hv[2], hv[3]);
    lo = make_uint4(lv[0], lv[1], lv[2], lv[3]);
  }
};

}  // namespace gla
