// abi_stubs.cpp -- host stand-ins for the kernel launchers and the few HIP
// runtime calls of gla_api.cpp, for a host-only build of the C ABI under
// AddressSanitizer and UndefinedBehaviorSanitizer.
//
// Each launcher, instead of enqueueing a kernel, touches the first and last
// byte of every element range its kernel would read or write, computed from
// the plan and the arguments it was handed. The test driver passes host
// buffers of exactly the sizes the header documents (and workspaces of exactly
// the size the *_workspace queries return), so a plan or a view whose reach
// exceeds its buffer shows up as a heap-buffer-overflow report. Every launch
// is logged by kernel name, and a launcher can be told to fail, so the driver
// can check which launches a call made and how a launch error is reported.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "../../gated_linear_attention_fwd_amd/csrc/plan.hpp"
#include "../../include/gla.h"
#include "abi_stubs.hpp"

namespace stubs {

std::vector<std::string> g_log;
std::string g_fail_next;  // a kernel name: its next launch returns an error

namespace {

volatile unsigned char g_sink;

void touch(const void *base, int64_t elem, size_t es) {
  const unsigned char *p = static_cast<const unsigned char *>(base) + elem * (int64_t)es;
  g_sink = p[0];
  g_sink = p[es - 1];
}

// Corners of a [BH][N][d] view: first and last slab, token and feature.
void touch_view(const gla::View &v, int64_t BH, int H, int64_t N, int d, size_t es) {
  if (BH == 0 || N == 0) return;
  if (!v.data) {
    std::fprintf(stderr, "stub: a view with rows has a NULL base\n");
    std::abort();
  }
  for (int64_t bh : {int64_t(0), BH - 1})
    for (int64_t n : {int64_t(0), N - 1})
      for (int c : {0, d - 1}) touch(v.data, v.slab(bh, H) + n * v.sn + c, es);
}

void touch_range(const void *p, int64_t n, size_t es) {
  if (!p || n <= 0) return;
  touch(p, 0, es);
  touch(p, n - 1, es);
}

hipError_t record(const char *name) {
  g_log.emplace_back(name);
  if (g_fail_next == name) {
    g_fail_next.clear();
    return hipErrorInvalidConfiguration;
  }
  return hipSuccess;
}

size_t elem(int dtype) { return dtype == 0 ? 4 : 2; }

// Frame f of slab bh in a per-frame state record, last element.
void touch_frame(const gla::FrameStates &fs, int64_t bh, int F, int f, int64_t E) {
  touch(fs.base, (bh * F + f) * fs.stride + E - 1, 4);
  touch(fs.base, (bh * F + f) * fs.stride, 4);
}

void kv(const gla::Plan &p, size_t es, const gla::KvArgs &a) {
  const int64_t N = (int64_t)p.F * p.T;
  touch_view(a.k, p.BH, a.H, N, p.d, es);
  touch_view(a.v, p.BH, a.H, N, p.d, es);
  touch_range(a.gamma, p.BH * p.F, 4);
  touch_range(a.ws, p.BH * p.F * p.P * p.state_elems(), 4);
}

void readout(const gla::Plan &p, size_t es, const gla::ReadoutArgs &a) {
  const int64_t N = (int64_t)p.F * p.T, E = p.state_elems();
  touch_view(a.q, p.BH, a.H, N, p.d, es);
  touch_view(a.g, p.BH, a.H, N, p.d, es);
  touch_view(a.o, p.BH, a.H, N, p.d, es);
  touch_range(a.gamma, p.BH * p.F, 4);
  if (p.BH > 0 && p.F > 0) {
    const int f = a.state_frame >= 0 ? a.state_frame : p.F - 1;
    touch_frame(a.states, p.BH - 1, p.F, f, E);
    touch_frame(a.states, 0, p.F, 0, E);
    if (p.G > 1) touch_range(a.ws + p.carry_offset(), p.BH * p.NG * E, 4);
  }
}

void bwd_q(const gla::BwdPlan &bp, size_t es, const gla::BwdQArgs &a) {
  const gla::Plan &p = bp.f;
  const int64_t N = (int64_t)p.F * p.T, E = p.state_elems();
  for (const gla::View *v : {&a.q, &a.g, &a.dO, &a.dq, &a.dg}) touch_view(*v, p.BH, a.H, N, p.d, es);
  if (p.BH > 0 && p.F > 0) {
    const int f = a.state_frame >= 0 ? a.state_frame : p.F - 1;
    touch_frame(a.st, p.BH - 1, p.F, f, E);
  }
  touch_range(a.gs, p.BH * p.F * p.R * E, 4);
}

void bwd_k(const gla::BwdPlan &bp, size_t es, const gla::BwdKArgs &a) {
  const gla::Plan &p = bp.f;
  const int64_t N = (int64_t)p.F * p.T, E = p.state_elems();
  for (const gla::View *v : {&a.k, &a.v, &a.dk, &a.dv}) touch_view(*v, p.BH, a.H, N, p.d, es);
  if (p.BH > 0 && p.F > 0) {
    const int f = a.adj_frame >= 0 ? a.adj_frame : p.F - 1;
    touch(a.gs, (((p.BH - 1) * p.F + f) * p.R) * E + E - 1, 4);
  }
}

void gdn_kv(const gla::Plan &p, size_t es, const gla::GdnKvArgs &a) {
  const int64_t N = (int64_t)p.F * p.T;
  touch_view(a.k, p.BH, a.H, N, p.d, es);
  touch_view(a.v, p.BH, a.H, N, p.d, es);
  touch_range(a.beta, p.BH * N, 4);
  touch_range(a.ws, p.BH * p.F * p.P * 2 * (int64_t)p.d * p.d, 4);
}

void gdn_readout(const gla::Plan &p, size_t es, const gla::GdnReadoutArgs &a) {
  const int64_t N = (int64_t)p.F * p.T;
  touch_view(a.q, p.BH, a.H, N, p.d, es);
  touch_view(a.o, p.BH, a.H, N, p.d, es);
  touch_range(a.ws, p.BH * p.F * p.P * 2 * (int64_t)p.d * p.d, 4);
}

}  // namespace
}  // namespace stubs

namespace gla {

// The same rule as the matrix-core launcher's: the path choice depends on it.
bool mfma_supports(int d) { return d == 32 || d == 64 || d == 128; }

hipError_t launch_kv_valu(const Plan &p, int dtype, const KvArgs &a, hipStream_t) {
  stubs::kv(p, stubs::elem(dtype), a);
  return stubs::record("kv");
}
hipError_t launch_kv_mfma(const Plan &p, const KvArgs &a, hipStream_t) {
  stubs::kv(p, 2, a);
  return stubs::record("kv");
}

hipError_t launch_carry(const Plan &p, const CarryArgs &a, hipStream_t) {
  const int64_t E = p.state_elems(), dd = (int64_t)p.d * p.d;
  stubs::touch_range(a.ws, p.BH * p.F * p.P * E, 4);
  stubs::touch_range(a.gamma, p.BH * p.F, 4);
  stubs::touch_range(a.S_in, p.BH * dd, 4);
  stubs::touch_range(a.z_in, p.BH * p.d, 4);
  stubs::touch_range(a.S_out, p.BH * dd, 4);
  stubs::touch_range(a.z_out, p.BH * p.d, 4);
  if (a.keep_frames && p.BH > 0 && p.F > 0) {
    if (p.G > 1) stubs::touch_range(a.ws + p.carry_offset(), p.BH * p.NG * E, 4);
    else stubs::touch_frame(a.frames, p.BH - 1, p.F, p.F - 1, E);
  }
  return stubs::record("carry");
}

hipError_t launch_readout_valu(const Plan &p, int dtype, const ReadoutArgs &a, hipStream_t) {
  stubs::readout(p, stubs::elem(dtype), a);
  return stubs::record("readout");
}
hipError_t launch_readout_mfma(const Plan &p, const ReadoutArgs &a, hipStream_t) {
  stubs::readout(p, 2, a);
  return stubs::record("readout");
}

hipError_t launch_bwd_q_valu(const BwdPlan &p, int dtype, const BwdQArgs &a, hipStream_t) {
  stubs::bwd_q(p, stubs::elem(dtype), a);
  return stubs::record("bwd_q");
}
hipError_t launch_bwd_q_mfma(const BwdPlan &p, const BwdQArgs &a, hipStream_t) {
  stubs::bwd_q(p, 2, a);
  return stubs::record("bwd_q");
}
hipError_t launch_bwd_k_valu(const BwdPlan &p, int dtype, const BwdKArgs &a, hipStream_t) {
  stubs::bwd_k(p, stubs::elem(dtype), a);
  return stubs::record("bwd_k");
}
hipError_t launch_bwd_k_mfma(const BwdPlan &p, const BwdKArgs &a, hipStream_t) {
  stubs::bwd_k(p, 2, a);
  return stubs::record("bwd_k");
}

hipError_t launch_rev_scan(const BwdPlan &bp, const RevScanArgs &a, hipStream_t) {
  const Plan &p = bp.f;
  const int64_t E = p.state_elems(), dd = (int64_t)p.d * p.d;
  if (p.BH > 0 && p.F > 0) stubs::touch_frame(a.st, p.BH - 1, p.F, p.F - 1, E);
  stubs::touch_range(a.gs, p.BH * p.F * p.R * E, 4);
  stubs::touch_range(a.gamma, p.BH * p.F, 4);
  for (const float *x : {a.S_in, a.dS_out, static_cast<const float *>(a.dS_in)})
    stubs::touch_range(x, p.BH * dd, 4);
  for (const float *x : {a.z_in, a.dz_out, static_cast<const float *>(a.dz_in)})
    stubs::touch_range(x, p.BH * p.d, 4);
  stubs::touch_range(a.dgp, p.BH * p.F * bp.NB, 4);
  return stubs::record("rev_scan");
}

hipError_t launch_dgamma(const BwdPlan &bp, const float *dgp, float *dgamma, hipStream_t) {
  stubs::touch_range(dgp, bp.f.BH * bp.f.F * bp.NB, 4);
  stubs::touch_range(dgamma, bp.f.BH * bp.f.F, 4);
  return stubs::record("dgamma");
}

hipError_t launch_gdn_kv_valu(const Plan &p, int dtype, const GdnKvArgs &a, hipStream_t) {
  stubs::gdn_kv(p, stubs::elem(dtype), a);
  return stubs::record("gdn_kv");
}
hipError_t launch_gdn_kv_mfma(const Plan &p, const GdnKvArgs &a, hipStream_t) {
  stubs::gdn_kv(p, 2, a);
  return stubs::record("gdn_kv");
}

static hipError_t gdn_scan(const Plan &p, const GdnScanArgs &a) {
  const int64_t dd = (int64_t)p.d * p.d;
  stubs::touch_range(a.ws, p.BH * p.F * p.P * 2 * dd, 4);
  if (p.scan_nc > 1) {
    stubs::touch_range(a.ws + p.scan_tws, p.BH * p.scan_nc * 2 * dd, 4);
    stubs::touch_range(a.ws + p.scan_sws, p.BH * p.scan_nc * dd, 4);
  }
  stubs::touch_range(a.gamma, p.BH * p.F, 4);
  stubs::touch_range(a.S_in, p.BH * dd, 4);
  stubs::touch_range(a.S_out, p.BH * dd, 4);
  return stubs::record("gdn_scan");
}
hipError_t launch_gdn_scan_valu(const Plan &p, const GdnScanArgs &a, hipStream_t) {
  return gdn_scan(p, a);
}
hipError_t launch_gdn_scan_mfma(const Plan &p, const GdnScanArgs &a, hipStream_t) {
  return gdn_scan(p, a);
}
hipError_t launch_gdn_readout_valu(const Plan &p, int dtype, const GdnReadoutArgs &a,
                                   hipStream_t) {
  stubs::gdn_readout(p, stubs::elem(dtype), a);
  return stubs::record("gdn_readout");
}
hipError_t launch_gdn_readout_mfma(const Plan &p, const GdnReadoutArgs &a, hipStream_t) {
  stubs::gdn_readout(p, 2, a);
  return stubs::record("gdn_readout");
}

// Workgroups per launch: queries per workgroup as in the anchor launchers (128 on
// the matrix-core path, 64 on the vector path), one launch per query frame
// segment in causal mode.
int64_t anchor_tiles(const AnchorArgs &a, Path path) {
  const int64_t seg = a.causal ? a.T : (int64_t)a.Fq * a.T;
  const int64_t per = path == Path::kMfma ? 128 : 64;
  return a.BH * (a.causal ? a.Fq : 1) * ((seg + per - 1) / per);
}

hipError_t launch_anchor_redo(const AnchorArgs &a, Path, hipStream_t) {
  const int64_t nq = a.BH * a.Fq * a.T * a.d;
  stubs::touch_range(a.o, nq, 2);  // reads the tile marks
  return stubs::record("anchor_redo");
}

hipError_t launch_anchor(const AnchorArgs &a, int dtype, Path, hipStream_t) {
  const size_t es = stubs::elem(dtype);
  const int64_t nq = a.BH * a.Fq * a.T * a.d, nk = a.BH * a.F * a.T * a.d;
  stubs::touch_range(a.q, nq, es);
  stubs::touch_range(a.g, nq, es);
  stubs::touch_range(a.o, nq, es);
  stubs::touch_range(a.k, nk, es);
  stubs::touch_range(a.v, nk, es);
  return stubs::record("anchor");
}

// The scratch array of the allocation-free entry point: a host buffer of the
// declared size, aligned as the device array.
void *noalloc_scratch(hipError_t *err) {
  static void *buf = nullptr;
  if (!buf && posix_memalign(&buf, 256, GLA_NOALLOC_SCRATCH_BYTES) != 0) buf = nullptr;
  *err = buf ? hipSuccess : hipErrorOutOfMemory;
  return buf;
}

int probe_kinds() { return 9; }

hipError_t launch_probe(int kind, const void *a, const void *b, void *out, size_t bytes,
                        hipStream_t) {
  const bool reads = kind != 2 && kind != 3, writes = kind >= 2, two = kind >= 6;
  if (reads) stubs::touch_range(a, (int64_t)bytes, 1);
  if (two) stubs::touch_range(b, (int64_t)bytes, 1);
  if (writes) stubs::touch_range(out, (int64_t)bytes, 1);
  return stubs::record("probe");
}

}  // namespace gla

// ---- HIP runtime calls made by the event timing of gla_profile_begin/end ----
struct ihipEvent_t {
  int recorded;
};

extern "C" {

hipError_t hipEventCreate(hipEvent_t *e) {
  *e = reinterpret_cast<hipEvent_t>(new ihipEvent_t{0});
  return hipSuccess;
}
hipError_t hipEventDestroy(hipEvent_t e) {
  delete reinterpret_cast<ihipEvent_t *>(e);
  return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t e, hipStream_t) {
  reinterpret_cast<ihipEvent_t *>(e)->recorded = 1;
  return hipSuccess;
}
hipError_t hipEventSynchronize(hipEvent_t e) {
  return reinterpret_cast<ihipEvent_t *>(e)->recorded ? hipSuccess : hipErrorInvalidHandle;
}
hipError_t hipEventElapsedTime(float *ms, hipEvent_t a, hipEvent_t b) {
  if (!reinterpret_cast<ihipEvent_t *>(a)->recorded || !reinterpret_cast<ihipEvent_t *>(b)->recorded)
    return hipErrorInvalidHandle;
  *ms = 0.25f;
  return hipSuccess;
}
const char *hipGetErrorString(hipError_t e) {
  return e == hipSuccess ? "no error" : "stub launch error";
}

}  // extern "C"
