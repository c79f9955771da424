// plan.hpp -- how one call is cut into workgroups, and the kernel launchers.
//
// Every (batch, head) slab is independent. Within a slab the tokens form F
// frames of T tokens (bidirectional mode: one frame of all N tokens). The
// forward pass runs as three launches on the caller's stream:
//
//   1. kv      one workgroup per (slab, frame, part): the part's sums
//              U = sum phi(k) v^T (d x d) and u = sum phi(k) (d), fp32, into
//              the workspace slot of that (slab, frame, part);
//   2. scan    one thread per (slab, state element): sums the parts of each
//              frame in a fixed order and runs S_f = gamma_f S_{f-1} + U_f
//              over the frames, leaving S_f in the frame's part-0 slot;
//   3. readout one workgroup per (slab, frame, split): phi(q) S_f, phi(q) z_f,
//              the normalise-and-gate epilogue, the store of o.
//
// Parts and splits exist only to give small problems enough workgroups; the
// partition depends on the sizes alone, so results are bitwise reproducible.
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
  size_t ws_bytes = 0;   // workspace: BH * F * P * (d*d + d) floats, 256-byte rounded

  int64_t state_elems() const { return (int64_t)d * d + d; }
};

// Cut sizes into a plan. Returns false if the sizes overflow the indexing.
bool make_plan(int64_t BH, int F, int64_t T, int d, Plan *plan);

// Which kernel family runs a (dtype, d) pair; the choice is a pure function of
// them so that parity tests know what they exercise.
enum class Path { kValu = 0, kMfma = 1 };
Path select_path(int dtype, int d);

struct KvArgs {
  const void *k;
  const void *v;
  float *ws;
};

struct ScanArgs {
  float *ws;
  const float *gamma;  // NULL: no decay (bidirectional)
  const float *S_in;   // NULL: zero carried state
  const float *z_in;
  float *S_out;        // NULL: not written
  float *z_out;
  int store_frames;    // 1: keep S_f of every frame for the readout
};

struct ReadoutArgs {
  const void *q;
  const void *g;
  void *o;
  const float *ws;
  float eps;
};

hipError_t launch_kv(const Plan &p, int dtype, Path path, const KvArgs &a, hipStream_t s);
hipError_t launch_scan(const Plan &p, const ScanArgs &a, hipStream_t s);
hipError_t launch_readout(const Plan &p, int dtype, Path path, const ReadoutArgs &a,
                          hipStream_t s);

}  // namespace gla
