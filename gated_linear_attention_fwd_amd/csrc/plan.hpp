// plan.hpp -- how one call is cut into workgroups, and the kernel launchers.
//
// Every (batch, head) slab is independent. Within a slab the tokens form F
// frames of T tokens (bidirectional mode: one frame of all N tokens). The
// forward pass runs as three launches on the caller's stream:
//
//   1. kv      one workgroup per (slab, group of G consecutive frames, part).
//              It keeps the decayed running sum of its frames in its
//              accumulators, S_loc_f = gamma_f S_loc_{f-1} + U_f (S_loc = U
//              at the group's first frame), with U_f = sum phi(k) v^T over the
//              part's tokens, and writes S_loc_f and z_loc_f (fp32) into the
//              workspace slot of every (slab, frame, part);
//   2. carry   one thread per (slab, state element): walks the groups in order,
//              carry_0 = S_in (or 0), carry_{g+1} = S_loc_{last of g} +
//              (prod of gamma over g) carry_g, and stores carry_g per group;
//              with one frame per group (G = 1) it is the plain scan, summing
//              the frame's parts and leaving S_f in place in the slot;
//   3. readout one workgroup per (slab, frame, split): S_f = S_loc_f +
//              (prod_{m=first of group}^{f} gamma_m) carry_g (G > 1) or the
//              slot itself (G = 1), then phi(q) S_f, phi(q) z_f, the
//              normalise-and-gate epilogue and the store of o.
//
// Groups cut the workspace traffic of the scan (only one state per group is
// chained) and parts give small problems enough workgroups; the partition
// depends on the sizes alone, so results are bitwise reproducible.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gla {

struct Plan {
  int64_t BH = 0;        // B * H slabs
  int F = 0;             // frames per slab (1 in bidirectional mode)
  int64_t T = 0;         // tokens per frame
  int d = 0;             // head dimension
  int P = 1;             // kv parts per frame
  int64_t part_len = 0;  // tokens per kv part (a multiple of 32)
  int R = 1;             // readout splits per frame
  int64_t read_len = 0;  // tokens per readout split (a multiple of 32)
  int G = 1;             // frames per kv group (G > 1 only with P == 1)
  int NG = 0;            // groups per slab, ceil(F / G)
  // Gated DeltaNet scan in chunks of frames (scan_nc > 1): scan_fc frames per
  // chunk; float offsets of the per-chunk local states and transfer matrices
  // (BH * nc * 2 d^2) and of the chunk start states (BH * nc * d^2)
  int scan_fc = 0, scan_nc = 0;
  int64_t scan_tws = 0, scan_sws = 0;
  size_t ws_bytes = 0;   // workspace bytes, 256-byte rounded:
                         //   slots  BH * F * P  states of d*d + d floats
                         //   carry  BH * NG     states of d*d + d floats (G > 1 only)

  int64_t state_elems() const { return (int64_t)d * d + d; }
  int64_t carry_offset() const { return BH * F * (int64_t)P * state_elems(); }  // floats
  int64_t slot_stride() const { return (int64_t)P * state_elems(); }  // floats per frame
};

// Where the per-frame states S_f, z_f (d*d + d floats each) are read or
// written: frame f of slab bh at base + (bh * F + f) * stride. The workspace
// slots (part 0 of each frame, stride P (d*d + d)), or a caller's state record
// ([B][H][F][d*d + d], stride d*d + d).
struct FrameStates {
  float *base;
  int64_t stride;
};

// Cut sizes into a plan. Returns false if the sizes overflow the indexing.
bool make_plan(int64_t BH, int F, int64_t T, int d, Plan *plan);
// One frame per kv group (no carries): the carry then writes S_f of every
// frame. The workspace shrinks to the slots.
void single_frame_groups(Plan *plan);
// The forward readout's splits: a frame also cut into pieces of a few hundred
// tokens (the backward keeps make_plan's).
void forward_readout_splits(Plan *plan);

// Which kernel family runs a (dtype, d) pair; the choice is a pure function of
// them so that parity tests know what they exercise.
enum class Path { kValu = 0, kMfma = 1 };
Path select_path(int dtype, int d);

// A strided [B][H][N][d] tensor: element (b, h, n, c) sits at
// data + b * sb + h * sh + n * sn + c (element units; the feature stride is 1).
// Slab bh = b * H + h.
struct View {
  const void *data;
  int64_t sb, sh, sn;
  // bh < 2^31 (the grid limits keep it far below): 32-bit division
  __host__ __device__ int64_t slab(int64_t bh, int H) const {
    const int b = (int)bh / H;
    return b * sb + ((int)bh - b * H) * sh;
  }
};

__host__ __device__ inline View contiguous_view(const void *p, int H, int64_t N, int d) {
  return View{p, (int64_t)H * N * d, N * d, (int64_t)d};
}

// 3D rotary positions (host-validated). Token l of frame f sits at
// (t, y, x) = (frame_offset + f, l / grid_w, l % grid_w); feature pairs
// (2p, 2p+1) form three consecutive sections of Pt, Ph and Pw pairs that turn
// with t, y and x, pair j of an m-pair section by pos * theta^(-j/m).
struct RopeK {
  int on = 0;
  int grid_h = 1, grid_w = 1;
  int frame_offset = 0;
  int Pt = 0, Ph = 0, Pw = 0;
  double inv_gw = 1.0;      // 1 / grid_w, for the position decode
  double log_theta = 0.0;   // ln(theta)
  int frames = 1;           // temporal rows in a workgroup's table (frames per kv group)
  // LDS table of (cos, sin): [0] identity, then [grid_h][Ph], [grid_w][Pw],
  // [frames][Pt]
  __host__ __device__ int y_base() const { return 1; }
  __host__ __device__ int x_base() const { return 1 + grid_h * Ph; }
  __host__ __device__ int t_base() const { return 1 + grid_h * Ph + grid_w * Pw; }
  __host__ __device__ int entries() const { return t_base() + frames * Pt; }
};

struct KvArgs {
  View k;
  View v;
  int H;
  const float *gamma;  // NULL: no decay
  float *ws;
  RopeK rope;
};

struct CarryArgs {
  float *ws;
  const float *gamma;  // NULL: no decay (bidirectional)
  const float *S_in;   // NULL: zero carried state
  const float *z_in;
  float *S_out;        // NULL: not written
  float *z_out;
  int keep_frames;     // 1: leave what the readout needs (carries, summed parts)
  FrameStates frames;  // G == 1 with keep_frames: where S_f goes (the slots: in place)
};

struct ReadoutArgs {
  View q;
  View g;
  View o;  // written
  int H;
  const float *gamma;  // NULL: no decay
  const float *ws;     // carries (G > 1)
  FrameStates states;  // S_loc_f (G > 1) or S_f (G == 1)
  float eps;
  int state_frame;     // -1: every frame reads its own state; else all read this one
  RopeK rope;
  int heads_fastest;   // 1: work items ordered with the slab fastest (matrix-core kernels)
};

// Decay weight of a frame's carry-in: prod_{m = first frame of f's group}^{f} gamma_m.
__device__ __forceinline__ float carry_weight(const float *gamma_slab, int f, int G) {
  float w = 1.f;
  if (gamma_slab)
    for (int m = (f / G) * G; m <= f; ++m) w *= gamma_slab[m];
  return w;
}

// ---------------------------------------------------------------------------
// Backward pass. Launches on the caller's stream:
//   1. kv + carry of the forward (one frame per group: after the carry, slot
//      (f, part 0) holds S_f itself), unless the caller hands over the record
//      of every frame's state that the forward wrote;
//   2. bwd_q    one workgroup per (slab, frame, split): recomputes num, den,
//               writes dg and dq, and the split's sums G = sum phi(q) dnum^T,
//               gz = sum dden phi(q) into its "gslot";
//   3. rev_scan one thread per (slab, state element): Sh_f = sum of the frame's
//               gslots + gamma_{f+1} Sh_{f+1} (from dS_out), stored in place in
//               gslot (f, 0); per-block partial sums of Sh_f . S_{f-1} for
//               dgamma; dS_in = gamma_0 Sh_0;
//   4. bwd_k    one workgroup per (slab, frame, part): dk = [k > 0] (Sh_f v + zh_f),
//               dv = Sh_f^T phi(k);
//      with rotary positions the numerator side takes turned features (S_f and
//      Sh_f hold turned keys and queries) and its adjoints turn back before the
//      normaliser's terms are added; bidirectional with positions runs on the
//      frames with no decay, every frame reading the last frame's S and frame
//      0's adjoint (the sums over all frames);
//   5. dgamma   one thread per (slab, frame): the partial sums in fixed order.
// ---------------------------------------------------------------------------
struct BwdPlan {
  Plan f;                    // forward recompute (G == 1), its slots first in the workspace
                             // (none when the caller gives the states)
  int64_t gslot_offset = 0;  // floats: BH * F * R states of d*d + d
  int64_t dgp_offset = 0;    // floats: BH * F * NB partial sums of dgamma
  int NB = 0;                // reverse-scan blocks per slab, ceil((d*d + d) / 256)
  size_t ws_bytes = 0;
};

// with_slots false: the forward's states come from the caller (no recompute).
bool make_bwd_plan(int64_t BH, int F, int64_t T, int d, BwdPlan *plan, bool with_slots = true);

struct BwdQArgs {
  View q, g, dO, dq, dg;  // dq, dg written
  int H;
  FrameStates st;         // the forward's S_f
  float *gs;              // gslots
  float eps;
  RopeK rope;             // on: turned queries (both kernels)
  int state_frame;        // >= 0: every frame reads that frame's S (bidirectional with positions)
};

struct RevScanArgs {
  FrameStates st;         // the forward's S_f
  float *gs;              // gslots: in the frame's sums, out the adjoints in (f, 0)
  const float *gamma;     // NULL: no decay (bidirectional)
  const float *S_in, *z_in;      // NULL: zero
  const float *dS_out, *dz_out;  // NULL: zero
  float *dS_in, *dz_in;          // NULL: not written
  float *dgp;             // partial sums of dgamma; NULL: not computed
};

struct BwdKArgs {
  View k, v, dk, dv;      // dk, dv written
  int H;
  const float *gs;        // adjoints Sh_f, zh_f in gslot (f, 0)
  RopeK rope;             // on: turned keys (both kernels)
  int adj_frame;          // >= 0: every frame reads that frame's adjoint (bidirectional with positions)
};

hipError_t launch_bwd_q(const BwdPlan &p, int dtype, Path path, const BwdQArgs &a, hipStream_t s);
hipError_t launch_rev_scan(const BwdPlan &p, const RevScanArgs &a, hipStream_t s);
hipError_t launch_bwd_k(const BwdPlan &p, int dtype, Path path, const BwdKArgs &a, hipStream_t s);
hipError_t launch_dgamma(const BwdPlan &p, const float *dgp, float *dgamma, hipStream_t s);

// ---------------------------------------------------------------------------
// Frame-wise Gated DeltaNet: gdn_kv (per slab, frame, part: U = sum beta k v^T,
// A = sum beta k k^T into a slot of 2 d^2 floats), gdn_scan (per slab and
// block of state columns: S_f = gamma_f (S_{f-1} - c^2 A_f S_{f-1}) + c U_f,
// left in part 0's U area), gdn_readout (o = S_f^T q). One frame per group.
// ---------------------------------------------------------------------------
struct GdnKvArgs {
  View k, v;
  int H;
  const float *beta;  // [B][H][N]
  float *ws;
};

struct GdnScanArgs {
  float *ws;
  const float *gamma;  // [B][H][F]
  const float *S_in;   // NULL: zero
  float *S_out;        // NULL: not written
  float key_scale;
};

struct GdnReadoutArgs {
  View q, o;  // o written
  int H;
  const float *ws;
};

bool make_gdn_plan(int64_t BH, int F, int64_t T, int d, Plan *plan);
hipError_t launch_gdn_kv(const Plan &p, int dtype, Path path, const GdnKvArgs &a, hipStream_t s);
hipError_t launch_gdn_scan(const Plan &p, Path path, const GdnScanArgs &a, hipStream_t s);
hipError_t launch_gdn_readout(const Plan &p, int dtype, Path path, const GdnReadoutArgs &a,
                              hipStream_t s);

// ---------------------------------------------------------------------------
// Gated softmax anchor (no workspace): k, v [BH][F*T][d]; q, g, o [BH][Fq*T][d],
// the tokens of the last Fq key frames. causal = 0: every key visible; 1: key
// frames i <= f with i < n_sink or i > f - window (window <= 0: unlimited).
// ---------------------------------------------------------------------------
struct AnchorArgs {
  const void *q, *k, *v, *g;
  void *o;
  int64_t BH;
  int Fq, F, T, d;
  int causal, n_sink, window;
  float scale;
};

int64_t anchor_tiles(const AnchorArgs &a, Path path);  // workgroups of one launch
hipError_t launch_anchor(const AnchorArgs &a, int dtype, Path path, hipStream_t s);
// Matrix-core path: recomputes the tiles launch_anchor marked (probabilities
// as bf16 hi + lo); launches nothing on the vector-ALU path.
hipError_t launch_anchor_redo(const AnchorArgs &a, Path path, hipStream_t s);

hipError_t launch_kv(const Plan &p, int dtype, Path path, const KvArgs &a, hipStream_t s);
hipError_t launch_carry(const Plan &p, const CarryArgs &a, hipStream_t s);
hipError_t launch_readout(const Plan &p, int dtype, Path path, const ReadoutArgs &a,
                          hipStream_t s);

}  // namespace gla
