// gla_api.cpp -- the exported C ABI: validation, planning and launches.
//
// Entry points and their contract are declared and documented in include/gla.h.
// Everything here runs on the host; nothing is enqueued unless every argument
// passed validation.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/gla.h"
#include "plan.hpp"

#define GLA_EXPORT extern "C" __attribute__((visibility("default")))

namespace gla {

hipError_t launch_kv_valu(const Plan &p, int dtype, const KvArgs &a, hipStream_t s);
hipError_t launch_readout_valu(const Plan &p, int dtype, const ReadoutArgs &a, hipStream_t s);
hipError_t launch_kv_mfma(const Plan &p, const KvArgs &a, hipStream_t s);
hipError_t launch_readout_mfma(const Plan &p, const ReadoutArgs &a, hipStream_t s);
hipError_t launch_bwd_q_valu(const BwdPlan &p, int dtype, const BwdQArgs &a, hipStream_t s);
hipError_t launch_bwd_k_valu(const BwdPlan &p, int dtype, const BwdKArgs &a, hipStream_t s);
hipError_t launch_bwd_k_mfma(const BwdPlan &p, const BwdKArgs &a, hipStream_t s);
hipError_t launch_bwd_q_mfma(const BwdPlan &p, const BwdQArgs &a, hipStream_t s);
hipError_t launch_gdn_kv_valu(const Plan &p, int dtype, const GdnKvArgs &a, hipStream_t s);
hipError_t launch_gdn_kv_mfma(const Plan &p, const GdnKvArgs &a, hipStream_t s);
hipError_t launch_gdn_scan_valu(const Plan &p, const GdnScanArgs &a, hipStream_t s);
hipError_t launch_gdn_scan_mfma(const Plan &p, const GdnScanArgs &a, hipStream_t s);
hipError_t launch_gdn_readout_mfma(const Plan &p, const GdnReadoutArgs &a, hipStream_t s);
hipError_t launch_gdn_readout_valu(const Plan &p, int dtype, const GdnReadoutArgs &a,
                                   hipStream_t s);
bool mfma_supports(int d);
void *noalloc_scratch(hipError_t *err);  // noalloc.hip
hipError_t launch_probe(int kind, const void *a, const void *b, void *out, size_t bytes,
                        hipStream_t s);  // probe.hip
int probe_kinds();

namespace {

constexpr int64_t kTargetWorkgroups = 2048;  // enough to fill 256 CUs several times
constexpr int64_t kMinPartTokens = 128;
constexpr int64_t kMinSplitTokens = 64;
constexpr int64_t kTokenAlign = 32;
// Forward readout: a frame is also cut into splits of about this many tokens.
// A readout workgroup's state prologue is then amortised over a few hundred
// tokens while the grid holds many workgroups per resident slot, which cuts
// the last round's tail (720p/60s, d = 64: 1 -> 3 splits, readout 0.513 ->
// 0.484 ms, call 0.887 -> 0.857 ms; the d = 128 stream at B = 2, H = 40:
// 0.357 -> 0.319 ms per block; 2 and 4 splits measured slower than 3 on
// both). A split changes no token's arithmetic. The backward keeps the plan's
// splits: each of its splits writes a partial sum of the state adjoint. Calls
// with rotary positions keep them too (see run()).
constexpr int64_t kSplitTargetTokens = 320;
constexpr int64_t kMaxGroupFrames = 8;  // the kv kernels hold up to 8 decays
// d = 128: frame pairs from 2 x 768 frames (1.5 rounds of resident kv workgroups)
constexpr int64_t kPairFramesMinUnits = 1536;
// kv workgroups resident at once on 256 CUs (4 per CU at d <= 64): grouping
// frames down to about this many workgroups removes the tail of a second wave.
constexpr int64_t kResidentKvWorkgroups = 1024;
constexpr int kChunkedScanMinFrames = 64;  // Gated DeltaNet: scan in chunks from here on
constexpr int kScanChunkFrames = 32;  // transfer and apply stay memory-bound (16..32 measured)

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

thread_local char g_last_error[512] = "";

gla_status fail(gla_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return s;
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Range {
  const void *p;
  size_t n;
  const char *name;
};

bool overlap(const Range &a, const Range &b) {
  if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.n && b0 < a0 + a.n;
}

// Path override for testing: GLA_PATH=valu forces the vector-ALU kernels.
int path_override() {
  const char *e = getenv("GLA_PATH");
  if (!e) return -1;
  if (!strcmp(e, "valu")) return 0;
  if (!strcmp(e, "mfma")) return 1;
  return -1;
}

gla_status check_dims(int B, int H, int d, int dt) {
  if (B < 0 || H < 0) return fail(GLA_ERR_SHAPE, "B=%d and H=%d must be >= 0", B, H);
  if (d != 16 && d != 32 && d != 64 && d != 128)
    return fail(GLA_ERR_UNSUPPORTED, "head dimension d=%d not in {16, 32, 64, 128}", d);
  if (dt != GLA_F32 && dt != GLA_BF16) return fail(GLA_ERR_UNSUPPORTED, "dtype %d unknown", dt);
  return GLA_OK;
}

gla_status check_eps(float eps) {
  if (!std::isfinite(eps) || eps < 0.f)
    return fail(GLA_ERR_VALUE, "eps=%g must be finite and >= 0", (double)eps);
  return GLA_OK;
}

gla_status check_tensor_align(const void *p, const char *name) {
  if (p && !aligned(p, 16)) return fail(GLA_ERR_ALIGN, "%s is not 16-byte aligned", name);
  return GLA_OK;
}

gla_status check_ws(const Plan &p, void *ws, size_t ws_bytes) {
  if (p.ws_bytes == 0) return GLA_OK;
  if (!ws) return fail(GLA_ERR_WORKSPACE, "workspace is NULL but %zu bytes are needed", p.ws_bytes);
  if (ws_bytes < p.ws_bytes)
    return fail(GLA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, p.ws_bytes);
  if (!aligned(ws, 256)) return fail(GLA_ERR_ALIGN, "workspace is not 256-byte aligned");
  return GLA_OK;
}

gla_status check_no_overlap(const Range *outs, int nout, const Range *all, int nall) {
  for (int i = 0; i < nout; ++i)
    for (int j = 0; j < nall; ++j) {
      if (outs[i].p == all[j].p && !strcmp(outs[i].name, all[j].name)) continue;  // itself
      if (overlap(outs[i], all[j]))
        return fail(GLA_ERR_ALIAS, "%s overlaps %s", outs[i].name, all[j].name);
    }
  return GLA_OK;
}

gla_status launched(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(GLA_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return GLA_OK;
}

// ---- optional event timing of every launch (gla_profile_begin/end) ----
enum Kind {
  kKindKv = 0,
  kKindCarry = 1,
  kKindReadout = 2,
  kKindBwdQ = 3,
  kKindRevScan = 4,
  kKindBwdK = 5,
  kKindDgamma = 6,
  kKindGdnKv = 7,
  kKindGdnScan = 8,
  kKindGdnReadout = 9,
  kKindAnchor = 10,
  kKindAnchorRedo = 11,
  kNumKinds = 12
};
const char *const kKindNames[kNumKinds] = {"kv",     "carry",  "readout",  "bwd_q",
                                           "rev_scan", "bwd_k", "dgamma", "gdn_kv",
                                           "gdn_scan", "gdn_readout", "anchor",
                                           "anchor_redo"};

struct Profiler {
  std::mutex mu;
  bool on = false;
  int cap = 0;
  int used = 0;
  std::vector<hipEvent_t> ev;  // start/stop pairs
  std::vector<int> kind;
};
Profiler g_prof;

// ---- optional launch log: GLA_LOG=1 prints each call's plan (how the work is
// cut into workgroups) and each launch, in order, on stderr ----
bool log_on() {
  static const bool on = [] {
    const char *e = getenv("GLA_LOG");
    return e != nullptr && atoi(e) != 0;
  }();
  return on;
}

const char *path_name(Path path) { return path == Path::kMfma ? "mfma" : "valu"; }

// A plan's geometry: kv workgroups BH * NG * P (G frames each, P parts of a
// frame), carry workgroups BH * ceil((d*d + d) / 256), readout workgroups
// BH * F * R (R splits of a frame).
void log_plan(const char *call, const Plan &p, Path path) {
  if (!log_on()) return;
  fprintf(stderr,
          "gla: %s path=%s BH=%lld F=%d T=%lld d=%d P=%d part_len=%lld G=%d NG=%d R=%d "
          "read_len=%lld kv_wgs=%lld carry_wgs=%lld readout_wgs=%lld ws_bytes=%zu\n",
          call, path_name(path), (long long)p.BH, p.F, (long long)p.T, p.d, p.P,
          (long long)p.part_len, p.G, p.NG, p.R, (long long)p.read_len,
          (long long)(p.BH * p.NG * p.P), (long long)(p.BH * ((p.state_elems() + 255) / 256)),
          (long long)(p.BH * p.F * p.R), p.ws_bytes);
}

template <class Fn>
hipError_t timed(Kind k, hipStream_t s, Fn &&fn) {
  if (log_on()) fprintf(stderr, "gla: launch %s\n", kKindNames[k]);
  int slot = -1;
  {
    std::lock_guard<std::mutex> lock(g_prof.mu);
    if (g_prof.on && g_prof.used < g_prof.cap) {
      slot = g_prof.used++;
      g_prof.kind[slot] = k;
    }
  }
  if (slot >= 0) (void)hipEventRecord(g_prof.ev[2 * slot], s);
  const hipError_t e = fn();
  if (slot >= 0) (void)hipEventRecord(g_prof.ev[2 * slot + 1], s);
  return e;
}

#define GLA_TRY(expr)                     \
  do {                                    \
    gla_status _st = (expr);              \
    if (_st != GLA_OK) return _st;        \
  } while (0)

constexpr int kMaxRopeEntries = 3072;  // LDS table of 24 KiB: with the kernels' own LDS (up to 57 KiB) it leaves two workgroups per CU

// A [B][H][N][d] tensor argument: validated view plus its address span.
gla_status check_view(const gla_tensor *t, const char *name, int64_t B, int64_t H, int64_t N,
                      int d, size_t es, bool output, View *view, Range *span) {
  *view = View{nullptr, 0, 0, 0};
  *span = Range{nullptr, 0, name};
  if (!t || !t->data) return GLA_OK;
  if (t->stride_b < 0 || t->stride_h < 0 || t->stride_n < 0)
    return fail(GLA_ERR_SHAPE, "%s has a negative stride", name);
  const int64_t q = (int64_t)(16 / es);  // elements per 16 bytes
  if (!aligned(t->data, 16)) return fail(GLA_ERR_ALIGN, "%s is not 16-byte aligned", name);
  if (t->stride_b % q || t->stride_h % q || t->stride_n % q)
    return fail(GLA_ERR_ALIGN, "%s strides must be multiples of 16 bytes (%lld elements)", name,
                (long long)q);
  *view = View{t->data, t->stride_b, t->stride_h, t->stride_n};
  if (B == 0 || H == 0 || N == 0) return GLA_OK;
  // last element + 1, in elements (each term checked against overflow)
  const __int128 ext = (__int128)(B - 1) * t->stride_b + (__int128)(H - 1) * t->stride_h +
                       (__int128)(N - 1) * t->stride_n + d;
  if (ext * (__int128)es > ((__int128)1 << 62))
    return fail(GLA_ERR_SHAPE, "%s spans more than 2^62 bytes", name);
  *span = Range{t->data, (size_t)(ext * (__int128)es), name};
  if (output) {
    // distinct (b, h, n) must be distinct rows: with the axes of size > 1 in
    // increasing stride order, each stride must clear what the smaller ones span
    int64_t st[3] = {t->stride_n, t->stride_h, t->stride_b}, sz[3] = {N, H, B};
    for (int a = 0; a < 3; ++a)
      for (int b = a + 1; b < 3; ++b)
        if (st[b] < st[a]) {
          std::swap(st[a], st[b]);
          std::swap(sz[a], sz[b]);
        }
    __int128 extent = d;
    for (int a = 0; a < 3; ++a) {
      if (sz[a] <= 1) continue;
      if ((__int128)st[a] < extent)
        return fail(GLA_ERR_ALIAS, "%s rows overlap one another (strides %lld, %lld, %lld)",
                    name, (long long)t->stride_b, (long long)t->stride_h,
                    (long long)t->stride_n);
      extent += (__int128)st[a] * (sz[a] - 1);
    }
  }
  return GLA_OK;
}

gla_status make_rope(const gla_rope3d *r, int F, int64_t T, int d, RopeK *out) {
  *out = RopeK{};
  if (!r) return GLA_OK;
  if (r->grid_h < 1 || r->grid_w < 1 || (int64_t)r->grid_h * r->grid_w != T)
    return fail(GLA_ERR_SHAPE, "rope grid %d x %d must be >= 1 and hold the T=%lld tokens of a frame",
                r->grid_h, r->grid_w, (long long)T);
  if (r->dim_t < 0 || r->dim_h < 0 || r->dim_w < 0 || (r->dim_t | r->dim_h | r->dim_w) & 1 ||
      (int64_t)r->dim_t + r->dim_h + r->dim_w != d)
    return fail(GLA_ERR_SHAPE, "rope sections (%d, %d, %d) must be even, >= 0 and sum to d=%d",
                r->dim_t, r->dim_h, r->dim_w, d);
  if (!std::isfinite(r->theta) || !(r->theta > 0.0))
    return fail(GLA_ERR_VALUE, "rope theta=%g must be finite and > 0", r->theta);
  if (r->frame_offset <= -(1 << 30) || r->frame_offset >= (1 << 30) || F >= (1 << 30))
    return fail(GLA_ERR_VALUE, "rope frame_offset=%d and F=%d must be below 2^30 in magnitude",
                r->frame_offset, F);
  // the table offsets (RopeK::x_base, t_base, entries) are int: bound the
  // entry count in 64 bits first
  const int64_t entries = 1 + (int64_t)r->grid_h * (r->dim_h / 2) +
                          (int64_t)r->grid_w * (r->dim_w / 2) + kMaxGroupFrames * (r->dim_t / 2);
  if (entries > INT32_MAX)
    return fail(GLA_ERR_SHAPE, "rope grid %d x %d gives a turn table of %lld entries (over 2^31)",
                r->grid_h, r->grid_w, (long long)entries);
  RopeK k;
  k.on = 1;
  k.grid_h = r->grid_h;
  k.grid_w = r->grid_w;
  k.frame_offset = r->frame_offset;
  k.Pt = r->dim_t / 2;
  k.Ph = r->dim_h / 2;
  k.Pw = r->dim_w / 2;
  k.inv_gw = 1.0 / r->grid_w;
  k.log_theta = std::log(r->theta);
  k.frames = (int)kMaxGroupFrames;
  *out = k;
  return GLA_OK;
}

// Work order of the matrix-core kernels for a view: slab fastest when heads sit
// closer together than tokens. GLA_HEADS_FASTEST=0/1 overrides (measurement).
int heads_fastest(const View &v) {
  if (const char *e = getenv("GLA_HEADS_FASTEST")) return atoi(e) != 0;
  return v.sh < v.sn ? 1 : 0;
}

enum class Mode { kBidir, kFrameCausal, kStateCarry };

// The body of every entry point. Bidirectional calls take F frames of T tokens
// (N = F * T); without rotary positions the frames do not matter and the
// sequence runs as one frame of N tokens, with them it runs on the frame
// structure with no decay and every frame reading the last frame's state.
gla_status run(Mode mode, const gla_tensor *q, const gla_tensor *k, const gla_tensor *v,
               const gla_tensor *g, const float *gamma, const float *S_in, const float *z_in,
               const gla_tensor *o, float *S_out, float *z_out, int B, int H, int F, int64_t T,
               int d, gla_dtype dt, float eps, const gla_rope3d *rope, float *states, void *ws,
               size_t ws_bytes, void *stream) {
  const bool outputs = mode != Mode::kStateCarry;
  const bool bidir = mode == Mode::kBidir;
  GLA_TRY(check_dims(B, H, d, dt));
  if (F < 0 || T < 0) return fail(GLA_ERR_SHAPE, "F=%d and T=%lld must be >= 0", F, (long long)T);
  if (outputs) GLA_TRY(check_eps(eps));
  if ((S_in == nullptr) != (z_in == nullptr))
    return fail(GLA_ERR_NULL, "S_in and z_in must both be given or both be NULL");
  if ((S_out == nullptr) != (z_out == nullptr))
    return fail(GLA_ERR_NULL, "S_out and z_out must both be given or both be NULL");
  if (!outputs && !S_out) return fail(GLA_ERR_NULL, "S_out and z_out are required");
  if (T > 0 && F > INT64_MAX / T) return fail(GLA_ERR_SHAPE, "F * T overflows");

  const int64_t BH = (int64_t)B * H;
  const int64_t N = (int64_t)F * T;
  const size_t es = dt == GLA_F32 ? 4 : 2;
  View vq, vk, vv, vg, vo;
  Range rq, rk, rv, rg, ro;
  GLA_TRY(check_view(k, "k", B, H, N, d, es, false, &vk, &rk));
  GLA_TRY(check_view(v, "v", B, H, N, d, es, false, &vv, &rv));
  if (outputs) {
    GLA_TRY(check_view(q, "q", B, H, N, d, es, false, &vq, &rq));
    GLA_TRY(check_view(g, "g", B, H, N, d, es, false, &vg, &rg));
    GLA_TRY(check_view(o, "o", B, H, N, d, es, true, &vo, &ro));
  } else {
    vq = vg = vo = View{nullptr, 0, 0, 0};
    rq = Range{nullptr, 0, "q"};
    rg = Range{nullptr, 0, "g"};
    ro = Range{nullptr, 0, "o"};
  }
  const bool have_tokens = BH > 0 && N > 0;
  if (have_tokens) {
    if (!vk.data || !vv.data) return fail(GLA_ERR_NULL, "k and v are required");
    if (outputs && (!vq.data || !vg.data || !vo.data))
      return fail(GLA_ERR_NULL, "q, g and o are required");
  }
  if (!bidir && BH > 0 && F > 0 && !gamma) return fail(GLA_ERR_NULL, "gamma is required when F > 0");
  GLA_TRY(check_tensor_align(S_in, "S_in"));
  GLA_TRY(check_tensor_align(z_in, "z_in"));
  GLA_TRY(check_tensor_align(S_out, "S_out"));
  GLA_TRY(check_tensor_align(z_out, "z_out"));
  if (gamma && !aligned(gamma, 4)) return fail(GLA_ERR_ALIGN, "gamma is not 4-byte aligned");
  GLA_TRY(check_tensor_align(states, "states"));
  RopeK rk_;
  GLA_TRY(make_rope(rope, F, T, d, &rk_));

  // bidirectional without positions: one frame of all N tokens
  const bool flat = bidir && !rk_.on;
  Plan p;
  if (!make_plan(BH, flat ? (N > 0 ? 1 : 0) : F, flat ? N : T, d, &p))
    return fail(GLA_ERR_SHAPE, "sizes overflow the indexing");
  // a record of every frame's state: the scan runs frame by frame and writes
  // S_f there, where the readout then reads it
  if (states) single_frame_groups(&p);
  // d = 128 carries a group's running sum in the accumulators, which the
  // frame's rotary turn must not touch: one frame per group there
  if (rk_.on && d == 128 && p.G > 1) single_frame_groups(&p);
  // (not with rotary positions: each split builds the turn table and the
  // turned state fragments again; 720p/60s readout 0.568 -> 0.590 ms at 3)
  if (!rk_.on) forward_readout_splits(&p);
  if (BH == 0 || (bidir && N == 0)) return GLA_OK;
  GLA_TRY(check_ws(p, ws, ws_bytes));
  const Path path = select_path(dt, d);
  log_plan(bidir ? "forward (bidirectional)" : states ? "forward (frame-causal, state record)"
                                                     : "forward (frame-causal)",
           p, path);
  if (rk_.on && path == Path::kMfma && rk_.entries() > kMaxRopeEntries)
    return fail(GLA_ERR_UNSUPPORTED,
                "rope table of %d entries exceeds %d (1 + grid_h*dim_h/2 + grid_w*dim_w/2 + "
                "8*dim_t/2)",
                rk_.entries(), kMaxRopeEntries);

  const size_t sbytes = (size_t)(BH * d * d) * 4, zbytes = (size_t)(BH * d) * 4;
  const Range all[] = {rq, rk, rv, rg,
                       {gamma, bidir ? 0 : (size_t)(BH * F) * 4, "gamma"},
                       {S_in, sbytes, "S_in"},   {z_in, zbytes, "z_in"},
                       ro,
                       {S_out, sbytes, "S_out"}, {z_out, zbytes, "z_out"},
                       {ws, p.ws_bytes, "workspace"},
                       {states, (size_t)(BH * F * p.state_elems()) * 4, "states"}};
  // S_out may be S_in exactly (and z_out z_in): compare them without the inputs.
  const Range outs_o[] = {ro, all[10], all[11]};
  GLA_TRY(check_no_overlap(outs_o, 3, all, 12));
  const Range outs_s[] = {{S_out, sbytes, "S_out"}, {z_out, zbytes, "z_out"}};
  const Range others[] = {all[0], all[1], all[2], all[3], all[4],
                          all[7], all[8], all[9], all[10], all[11]};
  GLA_TRY(check_no_overlap(outs_s, 2, others, 10));
  if (S_out && S_in && S_out != S_in && overlap(outs_s[0], all[5]))
    return fail(GLA_ERR_ALIAS, "S_out partially overlaps S_in");
  if (z_out && z_in && z_out != z_in && overlap(outs_s[1], all[6]))
    return fail(GLA_ERR_ALIAS, "z_out partially overlaps z_in");
  if (S_out && overlap(outs_s[0], all[6])) return fail(GLA_ERR_ALIAS, "S_out overlaps z_in");
  if (z_out && overlap(outs_s[1], all[5])) return fail(GLA_ERR_ALIAS, "z_out overlaps S_in");

  hipStream_t s = static_cast<hipStream_t>(stream);
  float *wsf = static_cast<float *>(ws);
  const float *gm = bidir ? nullptr : gamma;
  // Heads side by side within a token (head stride below the token stride, as
  // in [B][N][H][d] or a fused projection): the readout orders its work with
  // the slab fastest so that concurrent workgroups read neighbouring lines.
  const int ro_heads = heads_fastest(vq);
  if (p.F > 0)
    GLA_TRY(launched(timed(kKindKv, s,
                           [&] {
                             return launch_kv(p, dt, path, KvArgs{vk, vv, H, gm, wsf, rk_}, s);
                           }),
                     "kv"));
  const FrameStates fs = states ? FrameStates{states, p.state_elems()}
                                : FrameStates{wsf, p.slot_stride()};
  const CarryArgs sa{wsf,   gm,    bidir ? nullptr : S_in, bidir ? nullptr : z_in,
                     S_out, z_out, (outputs || states) ? 1 : 0, fs};
  GLA_TRY(launched(timed(kKindCarry, s, [&] { return launch_carry(p, sa, s); }), "carry"));
  if (outputs && have_tokens) {
    const ReadoutArgs ra{vq,  vg, vo, H, gm, wsf, fs, eps, (bidir && !flat) ? p.F - 1 : -1,
                         rk_, ro_heads};
    GLA_TRY(launched(timed(kKindReadout, s, [&] { return launch_readout(p, dt, path, ra, s); }),
                     "readout"));
  }
  return GLA_OK;
}

// Strides of a dense [B][H][N][d] tensor. They are formed before the sizes are
// validated: a stride beyond 64 bits saturates, and the span check of the
// view then refuses the sizes.
gla_tensor contiguous(const void *p, int H, int64_t N, int d) {
  const auto sat = [](__int128 x) {
    return x > INT64_MAX ? INT64_MAX : x < INT64_MIN ? INT64_MIN : (int64_t)x;
  };
  return gla_tensor{const_cast<void *>(p), sat((__int128)H * N * d), sat((__int128)N * d),
                    (int64_t)d};
}

// The body of the two backward entry points (contiguous [B][H][N][d] tensors).
gla_status run_bwd(bool bidir, const gla_tensor *q, const gla_tensor *k, const gla_tensor *v,
                   const gla_tensor *g, const float *gamma, const float *S_in, const float *z_in,
                   const gla_tensor *dO, const float *dS_out, const float *dz_out,
                   const gla_tensor *dq, const gla_tensor *dk, const gla_tensor *dv,
                   const gla_tensor *dg, float *dgamma, float *dS_in, float *dz_in,
                   bool want_states, const float *states, int B, int H, int F, int64_t T, int d,
                   gla_dtype dt, float eps, const gla_rope3d *rope, void *ws, size_t ws_bytes,
                   void *stream) {
  GLA_TRY(check_dims(B, H, d, dt));
  if (F < 0 || T < 0) return fail(GLA_ERR_SHAPE, "F=%d and T=%lld must be >= 0", F, (long long)T);
  GLA_TRY(check_eps(eps));
  if ((S_in == nullptr) != (z_in == nullptr))
    return fail(GLA_ERR_NULL, "S_in and z_in must both be given or both be NULL");
  if ((dS_out == nullptr) != (dz_out == nullptr))
    return fail(GLA_ERR_NULL, "dS_out and dz_out must both be given or both be NULL");
  if ((dS_in == nullptr) != (dz_in == nullptr))
    return fail(GLA_ERR_NULL, "dS_in and dz_in must both be given or both be NULL");
  if (T > 0 && F > INT64_MAX / T) return fail(GLA_ERR_SHAPE, "F * T overflows");
  const int64_t BH = (int64_t)B * H;
  const int64_t N = (int64_t)F * T;
  const bool have_tokens = BH > 0 && N > 0;
  const size_t es = dt == GLA_F32 ? 4 : 2;
  // token tensors: any [B][H][N][d] view with unit feature stride (outputs
  // may not overlap themselves); each view's span enters the overlap checks
  View vq, vk, vv, vg, vdo, vdq, vdk, vdv, vdg;
  Range rq, rk, rv, rg, rdo, rdq, rdk, rdv, rdg;
  GLA_TRY(check_view(q, "q", B, H, N, d, es, false, &vq, &rq));
  GLA_TRY(check_view(k, "k", B, H, N, d, es, false, &vk, &rk));
  GLA_TRY(check_view(v, "v", B, H, N, d, es, false, &vv, &rv));
  GLA_TRY(check_view(g, "g", B, H, N, d, es, false, &vg, &rg));
  GLA_TRY(check_view(dO, "dO", B, H, N, d, es, false, &vdo, &rdo));
  GLA_TRY(check_view(dq, "dq", B, H, N, d, es, true, &vdq, &rdq));
  GLA_TRY(check_view(dk, "dk", B, H, N, d, es, true, &vdk, &rdk));
  GLA_TRY(check_view(dv, "dv", B, H, N, d, es, true, &vdv, &rdv));
  GLA_TRY(check_view(dg, "dg", B, H, N, d, es, true, &vdg, &rdg));
  if (have_tokens && (!vq.data || !vk.data || !vv.data || !vg.data || !vdo.data))
    return fail(GLA_ERR_NULL, "q, k, v, g and dO are required");
  if (have_tokens && (!vdq.data || !vdk.data || !vdv.data || !vdg.data))
    return fail(GLA_ERR_NULL, "dq, dk, dv and dg are required");
  if (!bidir && BH > 0 && F > 0 && !gamma) return fail(GLA_ERR_NULL, "gamma is required when F > 0");
  const float *st[] = {S_in, z_in, dS_out, dz_out, dS_in, dz_in};
  const char *snames[] = {"S_in", "z_in", "dS_out", "dz_out", "dS_in", "dz_in"};
  for (int i = 0; i < 6; ++i) GLA_TRY(check_tensor_align(st[i], snames[i]));
  if (gamma && !aligned(gamma, 4)) return fail(GLA_ERR_ALIGN, "gamma is not 4-byte aligned");
  if (dgamma && !aligned(dgamma, 4)) return fail(GLA_ERR_ALIGN, "dgamma is not 4-byte aligned");
  GLA_TRY(check_tensor_align(states, "states"));
  if (want_states && BH > 0 && F > 0 && !states) return fail(GLA_ERR_NULL, "states is required");
  RopeK rk_;
  GLA_TRY(make_rope(rope, F, T, d, &rk_));

  // bidirectional without positions: one frame of all N tokens; with them the
  // frames place the positions (no decay; every frame reads the sums over all)
  const bool flat = bidir && !rk_.on;
  BwdPlan bp;
  if (!make_bwd_plan(BH, flat ? (N > 0 ? 1 : 0) : F, flat ? N : T, d, &bp, !want_states))
    return fail(GLA_ERR_SHAPE, "sizes overflow the indexing");
  if (BH == 0 || (bidir && N == 0)) return GLA_OK;
  if (bp.ws_bytes) {
    if (!ws) return fail(GLA_ERR_WORKSPACE, "workspace is NULL but %zu bytes are needed", bp.ws_bytes);
    if (ws_bytes < bp.ws_bytes)
      return fail(GLA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, bp.ws_bytes);
    if (!aligned(ws, 256)) return fail(GLA_ERR_ALIGN, "workspace is not 256-byte aligned");
  }
  const size_t sbytes = (size_t)(BH * d * d) * 4, zbytes = (size_t)(BH * d) * 4;
  const bool causal = !bidir;
  const Range all[] = {rq,
                       rk,
                       rv,
                       rg,
                       rdo,
                       {gamma, causal ? (size_t)(BH * F) * 4 : 0, "gamma"},
                       {S_in, causal ? sbytes : 0, "S_in"},
                       {z_in, causal ? zbytes : 0, "z_in"},
                       {dS_out, causal ? sbytes : 0, "dS_out"},
                       {dz_out, causal ? zbytes : 0, "dz_out"},
                       rdq,
                       rdk,
                       rdv,
                       rdg,
                       {dgamma, causal ? (size_t)(BH * F) * 4 : 0, "dgamma"},
                       {dS_in, causal ? sbytes : 0, "dS_in"},
                       {dz_in, causal ? zbytes : 0, "dz_in"},
                       {ws, bp.ws_bytes, "workspace"},
                       {states, causal ? (size_t)(BH * F * bp.f.state_elems()) * 4 : 0, "states"}};
  GLA_TRY(check_no_overlap(all + 10, 8, all, 19));

  hipStream_t s = static_cast<hipStream_t>(stream);
  const Path path = select_path(dt, d);
  log_plan(bidir ? "backward (bidirectional)" : states ? "backward (frame-causal, state record)"
                                                      : "backward (frame-causal)",
           bp.f, path);
  if (rk_.on && path == Path::kMfma && rk_.entries() > kMaxRopeEntries)
    return fail(GLA_ERR_UNSUPPORTED,
                "rope table of %d entries exceeds %d (1 + grid_h*dim_h/2 + grid_w*dim_w/2 + "
                "8*dim_t/2)",
                rk_.entries(), kMaxRopeEntries);
  float *wsf = static_cast<float *>(ws);
  float *gsf = wsf + bp.gslot_offset;
  const Plan &p = bp.f;
  const float *gm = causal ? gamma : nullptr;
  // the forward's S_f: recomputed into the workspace slots, or the caller's record
  const FrameStates fst = want_states
                              ? FrameStates{const_cast<float *>(states), p.state_elems()}
                              : FrameStates{wsf, p.slot_stride()};
  if (p.F > 0) {
    if (!want_states) {
      GLA_TRY(launched(timed(kKindKv, s,
                             [&] {
                               return launch_kv(p, dt, path, KvArgs{vk, vv, H, gm, wsf, rk_}, s);
                             }),
                       "kv"));
      const CarryArgs ca{wsf, gm, causal ? S_in : nullptr, causal ? z_in : nullptr,
                         nullptr, nullptr, 1, fst};
      GLA_TRY(launched(timed(kKindCarry, s, [&] { return launch_carry(p, ca, s); }), "carry"));
    }
    const BwdQArgs qa{vq, vg, vdo, vdq, vdg, H, fst, gsf, eps, rk_, (bidir && !flat) ? p.F - 1 : -1};
    GLA_TRY(launched(timed(kKindBwdQ, s, [&] { return launch_bwd_q(bp, dt, path, qa, s); }),
                     "bwd_q"));
  }
  float *dgp = (causal && dgamma && p.F > 0) ? wsf + bp.dgp_offset : nullptr;
  const RevScanArgs ra{fst,
                       gsf,
                       gm,
                       causal ? S_in : nullptr,
                       causal ? z_in : nullptr,
                       causal ? dS_out : nullptr,
                       causal ? dz_out : nullptr,
                       causal ? dS_in : nullptr,
                       causal ? dz_in : nullptr,
                       dgp};
  GLA_TRY(launched(timed(kKindRevScan, s, [&] { return launch_rev_scan(bp, ra, s); }),
                   "rev_scan"));
  if (have_tokens) {
    const BwdKArgs ka{vk, vv, vdk, vdv, H, gsf, rk_, (bidir && !flat) ? 0 : -1};
    GLA_TRY(launched(timed(kKindBwdK, s, [&] { return launch_bwd_k(bp, dt, path, ka, s); }),
                     "bwd_k"));
  }
  if (dgp)
    GLA_TRY(launched(timed(kKindDgamma, s, [&] { return launch_dgamma(bp, dgp, dgamma, s); }),
                     "dgamma"));
  return GLA_OK;
}

// The body of gla_gdn_framecausal (contiguous [B][H][N][d] tensors).
gla_status run_gdn(const void *q, const void *k, const void *v, const float *beta,
                   const float *gamma, const float *S_in, void *o, float *S_out, int B, int H,
                   int F, int T, int d, gla_dtype dt, float key_scale, void *ws,
                   size_t ws_bytes, void *stream) {
  GLA_TRY(check_dims(B, H, d, dt));
  if (F < 0 || T < 0) return fail(GLA_ERR_SHAPE, "F=%d and T=%d must be >= 0", F, T);
  if (!std::isfinite(key_scale) || !(key_scale > 0.f))
    return fail(GLA_ERR_VALUE, "key_scale=%g must be finite and > 0", (double)key_scale);
  if ((q == nullptr) != (o == nullptr))
    return fail(GLA_ERR_NULL, "q and o must both be given (outputs) or both be NULL (state only)");
  if (!o && !S_out) return fail(GLA_ERR_NULL, "nothing to compute: o and S_out are both NULL");
  const int64_t BH = (int64_t)B * H;
  const int64_t N = (int64_t)F * T;
  const bool have_tokens = BH > 0 && N > 0;
  if (have_tokens && (!k || !v || !beta)) return fail(GLA_ERR_NULL, "k, v and beta are required");
  if (BH > 0 && F > 0 && !gamma) return fail(GLA_ERR_NULL, "gamma is required when F > 0");
  const void *tens[] = {q, k, v, o};
  const char *tn[] = {"q", "k", "v", "o"};
  for (int i = 0; i < 4; ++i) GLA_TRY(check_tensor_align(tens[i], tn[i]));
  GLA_TRY(check_tensor_align(S_in, "S_in"));
  GLA_TRY(check_tensor_align(S_out, "S_out"));
  if (beta && !aligned(beta, 4)) return fail(GLA_ERR_ALIGN, "beta is not 4-byte aligned");
  if (gamma && !aligned(gamma, 4)) return fail(GLA_ERR_ALIGN, "gamma is not 4-byte aligned");
  Plan p;
  if (!make_gdn_plan(BH, F, T, d, &p)) return fail(GLA_ERR_SHAPE, "sizes overflow the indexing");
  if (BH == 0) return GLA_OK;
  GLA_TRY(check_ws(p, ws, ws_bytes));
  const size_t es = dt == GLA_F32 ? 4 : 2;
  const size_t tb = (size_t)(BH * N * d) * es;
  const size_t sbytes = (size_t)(BH * d * d) * 4;
  const Range all[] = {{q, tb, "q"},
                       {k, tb, "k"},
                       {v, tb, "v"},
                       {beta, (size_t)(BH * N) * 4, "beta"},
                       {gamma, (size_t)(BH * F) * 4, "gamma"},
                       {S_in, sbytes, "S_in"},
                       {o, tb, "o"},
                       {S_out, sbytes, "S_out"},
                       {ws, p.ws_bytes, "workspace"}};
  const Range outs[] = {all[6], all[7], all[8]};
  // S_out may be S_in (in-place carry): compare it without S_in
  for (int i = 0; i < 3; ++i)
    for (int j = 0; j < 9; ++j) {
      if (!strcmp(outs[i].name, all[j].name)) continue;
      if (i == 1 && j == 5 && S_out == S_in) continue;
      if (overlap(outs[i], all[j]))
        return fail(GLA_ERR_ALIAS, "%s overlaps %s", outs[i].name, all[j].name);
    }

  hipStream_t s = static_cast<hipStream_t>(stream);
  const Path path = select_path(dt, d);
  if (log_on())
    fprintf(stderr,
            "gla: gated deltanet path=%s BH=%lld F=%d T=%lld d=%d P=%d part_len=%lld "
            "scan_frames_per_chunk=%d scan_chunks=%d gdn_kv_wgs=%lld ws_bytes=%zu\n",
            path_name(path), (long long)p.BH, p.F, (long long)p.T, p.d, p.P,
            (long long)p.part_len, p.scan_fc, p.scan_nc, (long long)(p.BH * p.F * p.P),
            p.ws_bytes);
  float *wsf = static_cast<float *>(ws);
  // (T == 0 still launches it: every frame's sums are then written as zeros)
  if (p.F > 0)
    GLA_TRY(launched(timed(kKindGdnKv, s,
                           [&] {
                             return launch_gdn_kv(p, dt, path,
                                                  GdnKvArgs{contiguous_view(k, H, N, d),
                                                            contiguous_view(v, H, N, d), H, beta,
                                                            wsf},
                                                  s);
                           }),
                     "gdn_kv"));
  GLA_TRY(launched(timed(kKindGdnScan, s,
                         [&] {
                           return launch_gdn_scan(
                               p, path, GdnScanArgs{wsf, gamma, S_in, S_out, key_scale}, s);
                         }),
                   "gdn_scan"));
  if (o && have_tokens)
    GLA_TRY(launched(timed(kKindGdnReadout, s,
                           [&] {
                             return launch_gdn_readout(
                                 p, dt, path,
                                 GdnReadoutArgs{contiguous_view(q, H, N, d),
                                                contiguous_view(o, H, N, d), H, wsf},
                                 s);
                           }),
                     "gdn_readout"));
  return GLA_OK;
}

// The body of gla_softmax_anchor (contiguous tensors; no workspace).
gla_status run_anchor(const void *q, const void *k, const void *v, const void *g, void *o, int B,
                      int H, int Fq, int F, int T, int d, gla_dtype dt, int causal, int n_sink,
                      int window, float scale, void *stream) {
  GLA_TRY(check_dims(B, H, d, dt));
  if (F < 0 || Fq < 0 || T < 0 || Fq > F)
    return fail(GLA_ERR_SHAPE, "need 0 <= Fq <= F and T >= 0 (Fq=%d F=%d T=%d)", Fq, F, T);
  if (causal != 0 && causal != 1) return fail(GLA_ERR_VALUE, "causal=%d must be 0 or 1", causal);
  if (n_sink < 0) return fail(GLA_ERR_VALUE, "n_sink=%d must be >= 0", n_sink);
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(GLA_ERR_VALUE, "scale=%g must be finite and > 0", (double)scale);
  const int64_t BH = (int64_t)B * H;
  const int64_t Nq = (int64_t)Fq * T, Nk = (int64_t)F * T;
  if (BH == 0 || Nq == 0) return GLA_OK;
  if (!q || !k || !v || !g || !o) return fail(GLA_ERR_NULL, "q, k, v, g and o are required");
  const void *tens[] = {q, k, v, g, o};
  const char *tn[] = {"q", "k", "v", "g", "o"};
  for (int i = 0; i < 5; ++i) GLA_TRY(check_tensor_align(tens[i], tn[i]));
  if (Nk > (int64_t(1) << 62) / BH / d) return fail(GLA_ERR_SHAPE, "sizes overflow the indexing");
  const size_t es = dt == GLA_F32 ? 4 : 2;
  const size_t qb = (size_t)(BH * Nq * d) * es, kb = (size_t)(BH * Nk * d) * es;
  const Range ins[] = {{q, qb, "q"}, {k, kb, "k"}, {v, kb, "v"}, {g, qb, "g"}};
  const Range out{o, qb, "o"};
  for (const Range &r : ins)
    if (overlap(out, r)) return fail(GLA_ERR_ALIAS, "o overlaps %s", r.name);
  const Path path = select_path(dt, d);
  const AnchorArgs a{q, k, v, g, o, BH, Fq, F, T, d, causal, n_sink, window, scale};
  if (anchor_tiles(a, path) >= (int64_t(1) << 31))
    return fail(GLA_ERR_SHAPE, "sizes overflow the grid");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (log_on())
    fprintf(stderr,
            "gla: softmax anchor path=%s BH=%lld Fq=%d F=%d T=%d d=%d causal=%d n_sink=%d "
            "window=%d tiles=%lld\n",
            path_name(path), (long long)BH, Fq, F, T, d, causal, n_sink, window,
            (long long)anchor_tiles(a, path));
  GLA_TRY(launched(timed(kKindAnchor, s, [&] { return launch_anchor(a, dt, path, s); }),
                   "anchor"));
  GLA_TRY(launched(timed(kKindAnchorRedo, s, [&] { return launch_anchor_redo(a, path, s); }),
                   "anchor_redo"));
  return GLA_OK;
}

}  // namespace

bool make_gdn_plan(int64_t BH, int F, int64_t T, int d, Plan *plan) {
  Plan p;
  if (!make_plan(BH, F, T, d, &p)) return false;
  p.G = 1;
  p.NG = F;
  int64_t floats = BH * F * (int64_t)p.P * 2 * d * d;
  // long sequences scan in chunks of frames (matrix-core path): the chain of
  // dependent steps drops from F to about 2 Fc + F / Fc
  int fc = kScanChunkFrames;
  if (const char *e = getenv("GLA_SCAN_CHUNK"))  // testing knob
    if (atoi(e) >= 1) fc = atoi(e);
  if (F >= kChunkedScanMinFrames && fc < F) {
    p.scan_fc = fc;
    p.scan_nc = (int)ceil_div(F, p.scan_fc);
    p.scan_tws = floats;
    p.scan_sws = floats + BH * p.scan_nc * 2 * (int64_t)d * d;
    floats = p.scan_sws + BH * p.scan_nc * (int64_t)d * d;
  }
  p.ws_bytes = (size_t)round_up(floats * 4, 256);
  *plan = p;
  return true;
}

hipError_t launch_gdn_kv(const Plan &p, int dtype, Path path, const GdnKvArgs &a,
                         hipStream_t s) {
  if (path == Path::kMfma) return launch_gdn_kv_mfma(p, a, s);
  return launch_gdn_kv_valu(p, dtype, a, s);
}

hipError_t launch_gdn_scan(const Plan &p, Path path, const GdnScanArgs &a, hipStream_t s) {
  if (path == Path::kMfma) return launch_gdn_scan_mfma(p, a, s);
  return launch_gdn_scan_valu(p, a, s);
}

hipError_t launch_gdn_readout(const Plan &p, int dtype, Path path, const GdnReadoutArgs &a,
                              hipStream_t s) {
  if (path == Path::kMfma) return launch_gdn_readout_mfma(p, a, s);
  return launch_gdn_readout_valu(p, dtype, a, s);
}

bool make_plan(int64_t BH, int F, int64_t T, int d, Plan *plan) {
  Plan p;
  p.BH = BH;
  p.F = F;
  p.T = T;
  p.d = d;
  if (BH < 0 || F < 0 || T < 0) return false;
  // indexing limits, checked by division before any product is formed: 1-D
  // grids of 256-thread workgroups (slab x frame units, the carry's slab x
  // element blocks), 64-bit element offsets
  const int64_t max_grid = (int64_t(1) << 31) / 256;
  const int64_t E = p.state_elems();
  if (d < 1 || BH > (max_grid - 1) / ceil_div(E, 256)) return false;
  if (F > 0 && BH > (max_grid - 1) / F) return false;
  if (T > (int64_t(1) << 62) / d) return false;
  const int64_t units = BH * F;
  if (T > 0 && units > (int64_t(1) << 62) / T / d) return false;
  if (units > 0 && T > 0) {
    // kv parts fill at most one round of resident kv workgroups: the carry
    // then sums fewer parts and each part streams more tokens (720p/5s:
    // frame-causal 0.110 -> 0.102 ms, bidirectional 0.102 -> 0.093 ms against
    // cutting to 2048), and a second, mostly empty round costs more than the
    // idle slots of a partial first one (720p/5s frame-causal, 672 frames:
    // 2 parts -> 1, kv 0.0386 -> 0.0348 ms). Readout splits aim at 2048
    // workgroups.
    int64_t P = 1, R = 1;
    if (units < kResidentKvWorkgroups)
      P = std::min(std::max<int64_t>(1, kResidentKvWorkgroups / units),
                   std::max<int64_t>(1, ceil_div(T, kMinPartTokens)));
    if (units < kTargetWorkgroups)
      R = std::min(ceil_div(kTargetWorkgroups, units),
                   std::max<int64_t>(1, ceil_div(T, kMinSplitTokens)));
    p.part_len = round_up(ceil_div(T, P), kTokenAlign);
    p.P = (int)ceil_div(T, p.part_len);
    p.read_len = round_up(ceil_div(T, R), kTokenAlign);
    p.R = (int)ceil_div(T, p.read_len);
    // Enough frames for a full grid: group consecutive frames in one kv
    // workgroup. d <= 64 keeps the running sum in registers of its own and
    // groups up to 8 frames once the grid is twice the target. d = 128 keeps
    // it in the accumulators and pairs frames while the pairs still fill 1.5
    // rounds of its 768 resident workgroups: a mid-workgroup write-out of its
    // 64 KB states costs more, so larger groups lost more in kv than the carry
    // saved (the 720p/60s stream at B = 2, H = 40, per 30-frame block: G = 2
    // carry 0.058 -> 0.038 ms, kv 0.229 -> 0.232, call 4.79 -> 4.72 ms for 8
    // blocks; G = 3, 4, 8: 4.91, 4.82, 5.05 ms). Rotary positions keep G = 1
    // at d = 128 (run() below).
    const bool can_group = p.P == 1 && (d <= 64 || d == 128);
    if (can_group && d <= 64 && units >= 2 * kTargetWorkgroups)
      p.G = (int)std::min<int64_t>(kMaxGroupFrames, ceil_div(units, kResidentKvWorkgroups));
    if (can_group && d == 128 && units >= kPairFramesMinUnits) p.G = 2;
    if (const char *e = getenv("GLA_FRAMES_PER_GROUP"))
      if (can_group && atoi(e) >= 1)
        p.G = (int)std::min<int64_t>({(int64_t)atoi(e), (int64_t)std::max(F, 1), kMaxGroupFrames});
  } else {
    p.P = p.R = 1;
    p.part_len = p.read_len = round_up(T, kTokenAlign);
  }
  if (units > 0 && (units * std::max(p.P, p.R) >= max_grid)) return false;
  p.NG = (int)ceil_div(F, p.G);
  // carries are kept only for groups of several frames (G == 1 scans in place)
  p.ws_bytes = (size_t)round_up((units * p.P + (p.G > 1 ? BH * p.NG : 0)) * E * 4, 256);
  *plan = p;
  return true;
}

void single_frame_groups(Plan *plan) {
  Plan &p = *plan;
  p.G = 1;
  p.NG = p.F;
  p.ws_bytes = (size_t)round_up(p.BH * p.F * (int64_t)p.P * p.state_elems() * 4, 256);
}

void forward_readout_splits(Plan *plan) {
  Plan &p = *plan;
  const int64_t units = p.BH * p.F;
  if (units == 0 || p.T == 0) return;
  const int64_t max_grid = (int64_t(1) << 31) / 256;
  const int64_t want = std::min(ceil_div(p.T, kSplitTargetTokens), (max_grid - 1) / units);
  if (want <= p.R) return;
  p.read_len = round_up(ceil_div(p.T, want), kTokenAlign);
  p.R = (int)ceil_div(p.T, p.read_len);
}

bool make_bwd_plan(int64_t BH, int F, int64_t T, int d, BwdPlan *plan, bool with_slots) {
  BwdPlan b;
  if (!make_plan(BH, F, T, d, &b.f)) return false;
  Plan &p = b.f;
  single_frame_groups(&p);  // the carry leaves S_f in place in its slot
  const int64_t E = p.state_elems();
  const int64_t slots = with_slots ? BH * F * (int64_t)p.P * E : 0;
  p.ws_bytes = (size_t)slots * 4;
  b.NB = (int)ceil_div(E, 256);
  b.gslot_offset = slots;
  b.dgp_offset = slots + BH * F * (int64_t)p.R * E;
  b.ws_bytes = (size_t)round_up((b.dgp_offset + BH * F * b.NB) * 4, 256);
  *plan = b;
  return true;
}

hipError_t launch_bwd_q(const BwdPlan &p, int dtype, Path path, const BwdQArgs &a,
                        hipStream_t s) {
  if (path == Path::kMfma) return launch_bwd_q_mfma(p, a, s);
  return launch_bwd_q_valu(p, dtype, a, s);
}

hipError_t launch_bwd_k(const BwdPlan &p, int dtype, Path path, const BwdKArgs &a,
                        hipStream_t s) {
  if (path == Path::kMfma) return launch_bwd_k_mfma(p, a, s);
  return launch_bwd_k_valu(p, dtype, a, s);
}

Path select_path(int dtype, int d) {
  const int ov = path_override();
  const bool mfma_ok = dtype == GLA_BF16 && mfma_supports(d);
  if (ov == 0) return Path::kValu;
  return mfma_ok ? Path::kMfma : Path::kValu;
}

hipError_t launch_kv(const Plan &p, int dtype, Path path, const KvArgs &a, hipStream_t s) {
  if (path == Path::kMfma) return launch_kv_mfma(p, a, s);
  return launch_kv_valu(p, dtype, a, s);
}

hipError_t launch_readout(const Plan &p, int dtype, Path path, const ReadoutArgs &a,
                          hipStream_t s) {
  if (path == Path::kMfma) return launch_readout_mfma(p, a, s);
  return launch_readout_valu(p, dtype, a, s);
}

}  // namespace gla

using namespace gla;

GLA_EXPORT size_t gla_fwd_bidir_workspace(int B, int H, int64_t N, int d) {
  Plan p;
  if (B < 0 || H < 0 || N < 0 || d <= 0) return 0;
  if (!make_plan((int64_t)B * H, N > 0 ? 1 : 0, N, d, &p)) return 0;
  return p.ws_bytes;
}

GLA_EXPORT size_t gla_fwd_framecausal_workspace(int B, int H, int F, int T, int d) {
  Plan p;
  if (B < 0 || H < 0 || F < 0 || T < 0 || d <= 0) return 0;
  if (!make_plan((int64_t)B * H, F, T, d, &p)) return 0;
  return p.ws_bytes;
}

GLA_EXPORT size_t gla_state_carry_workspace(int B, int H, int F, int T, int d) {
  return gla_fwd_framecausal_workspace(B, H, F, T, d);
}

GLA_EXPORT size_t gla_fwd_bidir_ex_workspace(int B, int H, int F, int T, int d,
                                              const gla_rope3d *rope) {
  if (B < 0 || H < 0 || F < 0 || T < 0 || d <= 0) return 0;
  if (rope) return gla_fwd_framecausal_workspace(B, H, F, T, d);
  return gla_fwd_bidir_workspace(B, H, (int64_t)F * T, d);
}

GLA_EXPORT gla_status gla_fwd_bidir(const void *q, const void *k, const void *v, const void *g,
                                    void *o, int B, int H, int64_t N, int d, gla_dtype dt,
                                    float eps, void *ws, size_t ws_bytes, void *stream) {
  if (N < 0) return fail(GLA_ERR_SHAPE, "N=%lld must be >= 0", (long long)N);
  const gla_tensor tq = contiguous(q, H, N, d), tk = contiguous(k, H, N, d),
                   tv = contiguous(v, H, N, d), tg = contiguous(g, H, N, d),
                   to = contiguous(o, H, N, d);
  return run(Mode::kBidir, &tq, &tk, &tv, &tg, nullptr, nullptr, nullptr, &to, nullptr, nullptr,
             B, H, N > 0 ? 1 : 0, N, d, dt, eps, nullptr, nullptr, ws, ws_bytes, stream);
}

GLA_EXPORT gla_status gla_fwd_bidir_ex(const gla_tensor *q, const gla_tensor *k,
                                       const gla_tensor *v, const gla_tensor *g,
                                       const gla_tensor *o, int B, int H, int F, int T, int d,
                                       gla_dtype dt, float eps, const gla_rope3d *rope, void *ws,
                                       size_t ws_bytes, void *stream) {
  return run(Mode::kBidir, q, k, v, g, nullptr, nullptr, nullptr, o, nullptr, nullptr, B, H, F,
             T, d, dt, eps, rope, nullptr, ws, ws_bytes, stream);
}

GLA_EXPORT gla_status gla_fwd_framecausal(const void *q, const void *k, const void *v,
                                          const void *g, const float *gamma, const float *S_in,
                                          const float *z_in, void *o, float *S_out, float *z_out,
                                          int B, int H, int F, int T, int d, gla_dtype dt,
                                          float eps, void *ws, size_t ws_bytes, void *stream) {
  const int64_t N = (int64_t)std::max(F, 0) * std::max(T, 0);
  const gla_tensor tq = contiguous(q, H, N, d), tk = contiguous(k, H, N, d),
                   tv = contiguous(v, H, N, d), tg = contiguous(g, H, N, d),
                   to = contiguous(o, H, N, d);
  return run(Mode::kFrameCausal, &tq, &tk, &tv, &tg, gamma, S_in, z_in, &to, S_out, z_out, B, H,
             F, T, d, dt, eps, nullptr, nullptr, ws, ws_bytes, stream);
}

GLA_EXPORT gla_status gla_fwd_framecausal_noalloc(const void *q, const void *k, const void *v,
                                                  const void *g, const float *gamma,
                                                  const float *S_in, const float *z_in, void *o,
                                                  float *S_out, float *z_out, int B, int H, int F,
                                                  int T, int d, gla_dtype dt, float eps,
                                                  void *stream) {
  // the size check needs no GPU: refuse before the scratch lookup
  Plan p;
  if (B >= 0 && H >= 0 && F >= 0 && T >= 0 && make_plan((int64_t)B * H, F, T, d, &p) &&
      p.ws_bytes > GLA_NOALLOC_SCRATCH_BYTES)
    return fail(GLA_ERR_WORKSPACE,
                "these sizes need %zu bytes of workspace; the static scratch of the no-alloc "
                "call holds %zu (GLA_NOALLOC_SCRATCH_BYTES): use gla_fwd_framecausal with a "
                "workspace",
                p.ws_bytes, (size_t)GLA_NOALLOC_SCRATCH_BYTES);
  hipError_t e = hipSuccess;
  void *ws = noalloc_scratch(&e);
  if (!ws)
    return fail(GLA_ERR_HIP, "device address of the static scratch: %s", hipGetErrorString(e));
  return gla_fwd_framecausal(q, k, v, g, gamma, S_in, z_in, o, S_out, z_out, B, H, F, T, d, dt,
                             eps, ws, GLA_NOALLOC_SCRATCH_BYTES, stream);
}

GLA_EXPORT gla_status gla_fwd_framecausal_ex(const gla_tensor *q, const gla_tensor *k,
                                             const gla_tensor *v, const gla_tensor *g,
                                             const float *gamma, const float *S_in,
                                             const float *z_in, const gla_tensor *o,
                                             float *S_out, float *z_out, int B, int H, int F,
                                             int T, int d, gla_dtype dt, float eps,
                                             const gla_rope3d *rope, void *ws, size_t ws_bytes,
                                             void *stream) {
  return run(Mode::kFrameCausal, q, k, v, g, gamma, S_in, z_in, o, S_out, z_out, B, H, F, T, d,
             dt, eps, rope, nullptr, ws, ws_bytes, stream);
}

GLA_EXPORT gla_status gla_state_carry(const void *k, const void *v, const float *gamma,
                                      const float *S_in, const float *z_in, float *S_out,
                                      float *z_out, int B, int H, int F, int T, int d,
                                      gla_dtype dt, void *ws, size_t ws_bytes, void *stream) {
  const int64_t N = (int64_t)std::max(F, 0) * std::max(T, 0);
  const gla_tensor tk = contiguous(k, H, N, d), tv = contiguous(v, H, N, d);
  return run(Mode::kStateCarry, nullptr, &tk, &tv, nullptr, gamma, S_in, z_in, nullptr, S_out,
             z_out, B, H, F, T, d, dt, 0.f, nullptr, nullptr, ws, ws_bytes, stream);
}

GLA_EXPORT gla_status gla_state_carry_ex(const gla_tensor *k, const gla_tensor *v,
                                         const float *gamma, const float *S_in,
                                         const float *z_in, float *S_out, float *z_out, int B,
                                         int H, int F, int T, int d, gla_dtype dt,
                                         const gla_rope3d *rope, void *ws, size_t ws_bytes,
                                         void *stream) {
  return run(Mode::kStateCarry, nullptr, k, v, nullptr, gamma, S_in, z_in, nullptr, S_out, z_out,
             B, H, F, T, d, dt, 0.f, rope, nullptr, ws, ws_bytes, stream);
}

GLA_EXPORT size_t gla_bwd_framecausal_workspace(int B, int H, int F, int T, int d) {
  BwdPlan p;
  if (B < 0 || H < 0 || F < 0 || T < 0 || d <= 0) return 0;
  if (!make_bwd_plan((int64_t)B * H, F, T, d, &p)) return 0;
  return p.ws_bytes;
}

GLA_EXPORT size_t gla_bwd_bidir_workspace(int B, int H, int64_t N, int d) {
  BwdPlan p;
  if (B < 0 || H < 0 || N < 0 || d <= 0) return 0;
  if (!make_bwd_plan((int64_t)B * H, N > 0 ? 1 : 0, N, d, &p)) return 0;
  return p.ws_bytes;
}

GLA_EXPORT gla_status gla_bwd_framecausal(const void *q, const void *k, const void *v,
                                          const void *g, const float *gamma, const float *S_in,
                                          const float *z_in, const void *dO, const float *dS_out,
                                          const float *dz_out, void *dq, void *dk, void *dv,
                                          void *dg, float *dgamma, float *dS_in, float *dz_in,
                                          int B, int H, int F, int T, int d, gla_dtype dt,
                                          float eps, void *ws, size_t ws_bytes, void *stream) {
  const int64_t N = (int64_t)std::max(F, 0) * std::max(T, 0);
  const gla_tensor t[9] = {contiguous(q, H, N, d),  contiguous(k, H, N, d),  contiguous(v, H, N, d),
                           contiguous(g, H, N, d),  contiguous(dO, H, N, d), contiguous(dq, H, N, d),
                           contiguous(dk, H, N, d), contiguous(dv, H, N, d), contiguous(dg, H, N, d)};
  return run_bwd(false, &t[0], &t[1], &t[2], &t[3], gamma, S_in, z_in, &t[4], dS_out, dz_out,
                 &t[5], &t[6], &t[7], &t[8], dgamma, dS_in, dz_in, false, nullptr, B, H, F, T, d,
                 dt, eps, nullptr, ws, ws_bytes, stream);
}

GLA_EXPORT gla_status gla_bwd_bidir(const void *q, const void *k, const void *v, const void *g,
                                    const void *dO, void *dq, void *dk, void *dv, void *dg, int B,
                                    int H, int64_t N, int d, gla_dtype dt, float eps, void *ws,
                                    size_t ws_bytes, void *stream) {
  if (N < 0) return fail(GLA_ERR_SHAPE, "N=%lld must be >= 0", (long long)N);
  const gla_tensor t[9] = {contiguous(q, H, N, d),  contiguous(k, H, N, d),  contiguous(v, H, N, d),
                           contiguous(g, H, N, d),  contiguous(dO, H, N, d), contiguous(dq, H, N, d),
                           contiguous(dk, H, N, d), contiguous(dv, H, N, d), contiguous(dg, H, N, d)};
  return run_bwd(true, &t[0], &t[1], &t[2], &t[3], nullptr, nullptr, nullptr, &t[4], nullptr,
                 nullptr, &t[5], &t[6], &t[7], &t[8], nullptr, nullptr, nullptr, false, nullptr, B,
                 H, N > 0 ? 1 : 0, N, d, dt, eps, nullptr, ws, ws_bytes, stream);
}

GLA_EXPORT gla_status gla_fwd_framecausal_states(const void *q, const void *k, const void *v,
                                                 const void *g, const float *gamma,
                                                 const float *S_in, const float *z_in, void *o,
                                                 float *S_out, float *z_out, float *states, int B,
                                                 int H, int F, int T, int d, gla_dtype dt,
                                                 float eps, void *ws, size_t ws_bytes,
                                                 void *stream) {
  if ((int64_t)B * H > 0 && F > 0 && !states) return fail(GLA_ERR_NULL, "states is required");
  const int64_t N = (int64_t)std::max(F, 0) * std::max(T, 0);
  const gla_tensor tq = contiguous(q, H, N, d), tk = contiguous(k, H, N, d),
                   tv = contiguous(v, H, N, d), tg = contiguous(g, H, N, d),
                   to = contiguous(o, H, N, d);
  return run(Mode::kFrameCausal, &tq, &tk, &tv, &tg, gamma, S_in, z_in, &to, S_out, z_out, B, H,
             F, T, d, dt, eps, nullptr, F > 0 ? states : nullptr, ws, ws_bytes, stream);
}

GLA_EXPORT size_t gla_bwd_framecausal_states_workspace(int B, int H, int F, int T, int d) {
  BwdPlan p;
  if (B < 0 || H < 0 || F < 0 || T < 0 || d <= 0) return 0;
  if (!make_bwd_plan((int64_t)B * H, F, T, d, &p, false)) return 0;
  return p.ws_bytes;
}

GLA_EXPORT gla_status gla_bwd_framecausal_states(
    const void *q, const void *k, const void *v, const void *g, const float *gamma,
    const float *S_in, const float *z_in, const float *states, const void *dO,
    const float *dS_out, const float *dz_out, void *dq, void *dk, void *dv, void *dg,
    float *dgamma, float *dS_in, float *dz_in, int B, int H, int F, int T, int d, gla_dtype dt,
    float eps, void *ws, size_t ws_bytes, void *stream) {
  const int64_t N = (int64_t)std::max(F, 0) * std::max(T, 0);
  const gla_tensor t[9] = {contiguous(q, H, N, d),  contiguous(k, H, N, d),  contiguous(v, H, N, d),
                           contiguous(g, H, N, d),  contiguous(dO, H, N, d), contiguous(dq, H, N, d),
                           contiguous(dk, H, N, d), contiguous(dv, H, N, d), contiguous(dg, H, N, d)};
  return run_bwd(false, &t[0], &t[1], &t[2], &t[3], gamma, S_in, z_in, &t[4], dS_out, dz_out,
                 &t[5], &t[6], &t[7], &t[8], dgamma, dS_in, dz_in, true, states, B, H, F, T, d, dt,
                 eps, nullptr, ws, ws_bytes, stream);
}

GLA_EXPORT gla_status gla_fwd_framecausal_states_ex(
    const gla_tensor *q, const gla_tensor *k, const gla_tensor *v, const gla_tensor *g,
    const float *gamma, const float *S_in, const float *z_in, const gla_tensor *o, float *S_out,
    float *z_out, float *states, int B, int H, int F, int T, int d, gla_dtype dt, float eps,
    const gla_rope3d *rope, void *ws, size_t ws_bytes, void *stream) {
  if ((int64_t)B * H > 0 && F > 0 && !states) return fail(GLA_ERR_NULL, "states is required");
  return run(Mode::kFrameCausal, q, k, v, g, gamma, S_in, z_in, o, S_out, z_out, B, H, F, T, d,
             dt, eps, rope, F > 0 ? states : nullptr, ws, ws_bytes, stream);
}

GLA_EXPORT gla_status gla_bwd_framecausal_ex(
    const gla_tensor *q, const gla_tensor *k, const gla_tensor *v, const gla_tensor *g,
    const float *gamma, const float *S_in, const float *z_in, const float *states,
    const gla_tensor *dO, const float *dS_out, const float *dz_out, const gla_tensor *dq,
    const gla_tensor *dk, const gla_tensor *dv, const gla_tensor *dg, float *dgamma,
    float *dS_in, float *dz_in, int B, int H, int F, int T, int d, gla_dtype dt, float eps,
    const gla_rope3d *rope, void *ws, size_t ws_bytes, void *stream) {
  return run_bwd(false, q, k, v, g, gamma, S_in, z_in, dO, dS_out, dz_out, dq, dk, dv, dg, dgamma,
                 dS_in, dz_in, states != nullptr, states, B, H, F, T, d, dt, eps, rope, ws,
                 ws_bytes, stream);
}

GLA_EXPORT size_t gla_bwd_bidir_ex_workspace(int B, int H, int F, int T, int d,
                                             const gla_rope3d *rope) {
  if (!rope) return gla_bwd_bidir_workspace(B, H, (int64_t)std::max(F, 0) * std::max(T, 0), d);
  BwdPlan p;
  if (B < 0 || H < 0 || F < 0 || T < 0 || d <= 0) return 0;
  if (!make_bwd_plan((int64_t)B * H, F, T, d, &p)) return 0;
  return p.ws_bytes;
}

GLA_EXPORT gla_status gla_bwd_bidir_ex(const gla_tensor *q, const gla_tensor *k,
                                       const gla_tensor *v, const gla_tensor *g,
                                       const gla_tensor *dO, const gla_tensor *dq,
                                       const gla_tensor *dk, const gla_tensor *dv,
                                       const gla_tensor *dg, int B, int H, int F, int T, int d,
                                       gla_dtype dt, float eps, const gla_rope3d *rope, void *ws,
                                       size_t ws_bytes, void *stream) {
  if (F < 0 || T < 0) return fail(GLA_ERR_SHAPE, "F=%d and T=%d must be >= 0", F, T);
  if (rope)
    return run_bwd(true, q, k, v, g, nullptr, nullptr, nullptr, dO, nullptr, nullptr, dq, dk, dv,
                   dg, nullptr, nullptr, nullptr, false, nullptr, B, H, F, T, d, dt, eps, rope,
                   ws, ws_bytes, stream);
  const int64_t N = (int64_t)F * T;
  return run_bwd(true, q, k, v, g, nullptr, nullptr, nullptr, dO, nullptr, nullptr, dq, dk, dv,
                 dg, nullptr, nullptr, nullptr, false, nullptr, B, H, N > 0 ? 1 : 0, N, d, dt,
                 eps, nullptr, ws, ws_bytes, stream);
}

GLA_EXPORT size_t gla_gdn_framecausal_workspace(int B, int H, int F, int T, int d) {
  Plan p;
  if (B < 0 || H < 0 || F < 0 || T < 0 || d <= 0) return 0;
  if (!make_gdn_plan((int64_t)B * H, F, T, d, &p)) return 0;
  return p.ws_bytes;
}

GLA_EXPORT gla_status gla_gdn_framecausal(const void *q, const void *k, const void *v,
                                          const float *beta, const float *gamma,
                                          const float *S_in, void *o, float *S_out, int B, int H,
                                          int F, int T, int d, gla_dtype dt, float key_scale,
                                          void *ws, size_t ws_bytes, void *stream) {
  return run_gdn(q, k, v, beta, gamma, S_in, o, S_out, B, H, F, T, d, dt, key_scale, ws,
                 ws_bytes, stream);
}

GLA_EXPORT gla_status gla_softmax_anchor(const void *q, const void *k, const void *v,
                                         const void *g, void *o, int B, int H, int Fq, int F,
                                         int T, int d, gla_dtype dt, int causal, int n_sink,
                                         int window, float scale, void *stream) {
  return run_anchor(q, k, v, g, o, B, H, Fq, F, T, d, dt, causal, n_sink, window, scale, stream);
}

GLA_EXPORT const char *gla_status_string(gla_status s) {
  switch (s) {
    case GLA_OK: return "ok";
    case GLA_ERR_NULL: return "required pointer is NULL";
    case GLA_ERR_SHAPE: return "invalid or inconsistent sizes";
    case GLA_ERR_UNSUPPORTED: return "unsupported head dimension or dtype";
    case GLA_ERR_ALIGN: return "misaligned pointer";
    case GLA_ERR_WORKSPACE: return "workspace missing or too small";
    case GLA_ERR_VALUE: return "invalid scalar argument";
    case GLA_ERR_HIP: return "HIP runtime error";
    case GLA_ERR_ALIAS: return "output overlaps another argument";
    default: break;
  }
  return "unknown status";
}

GLA_EXPORT const char *gla_last_error(void) { return g_last_error; }

GLA_EXPORT int gla_version(void) { return 10600; }

GLA_EXPORT gla_status gla_stream_probe(int kind, const void *a, const void *b, void *out,
                                      size_t bytes, void *stream) {
  if (kind < 0 || kind >= probe_kinds())
    return fail(GLA_ERR_VALUE, "probe kind %d not in 0..%d", kind, probe_kinds() - 1);
  constexpr size_t kRange = size_t(256) << 10;
  if (bytes == 0 || bytes % kRange)
    return fail(GLA_ERR_SHAPE, "probe size %zu must be a positive multiple of 256 KiB", bytes);
  const bool reads_a = kind != 2 && kind != 3, reads_b = kind >= 6;
  if (!out || (reads_a && !a) || (reads_b && !b))
    return fail(GLA_ERR_NULL, "probe kind %d needs out%s%s", kind, reads_a ? ", a" : "",
                reads_b ? ", b" : "");
  if (!aligned(out, 16) || (a && !aligned(a, 16)) || (b && !aligned(b, 16)))
    return fail(GLA_ERR_ALIGN, "probe buffers must be 16-byte aligned");
  const Range ro{out, bytes, "out"};
  const Range ra{reads_a ? a : nullptr, bytes, "a"}, rb{reads_b ? b : nullptr, bytes, "b"};
  if (overlap(ro, ra) || overlap(ro, rb)) return fail(GLA_ERR_ALIAS, "probe out overlaps a or b");
  return launched(launch_probe(kind, a, b, out, bytes, static_cast<hipStream_t>(stream)),
                  "probe");
}

GLA_EXPORT gla_status gla_profile_begin(int max_launches) {
  if (max_launches < 1 || max_launches > 65536)
    return fail(GLA_ERR_VALUE, "max_launches=%d must be in 1..65536", max_launches);
  std::lock_guard<std::mutex> lock(g_prof.mu);
  if (g_prof.on) return fail(GLA_ERR_VALUE, "a profiling session is already open");
  g_prof.ev.assign(2 * (size_t)max_launches, nullptr);
  g_prof.kind.assign((size_t)max_launches, 0);
  for (auto &e : g_prof.ev) {
    if (hipEventCreate(&e) != hipSuccess) {
      for (auto &x : g_prof.ev)
        if (x) (void)hipEventDestroy(x);
      g_prof.ev.clear();
      return fail(GLA_ERR_HIP, "hipEventCreate failed");
    }
  }
  g_prof.cap = max_launches;
  g_prof.used = 0;
  g_prof.on = true;
  return GLA_OK;
}

GLA_EXPORT gla_status gla_profile_end(gla_kernel_time *out, int max_out, int *n_out) {
  std::lock_guard<std::mutex> lock(g_prof.mu);
  if (!g_prof.on) return fail(GLA_ERR_VALUE, "no profiling session is open");
  double total[kNumKinds] = {};
  int count[kNumKinds] = {};
  gla_status st = GLA_OK;
  for (int i = 0; i < g_prof.used; ++i) {
    float ms = 0.f;
    if (hipEventSynchronize(g_prof.ev[2 * i + 1]) != hipSuccess ||
        hipEventElapsedTime(&ms, g_prof.ev[2 * i], g_prof.ev[2 * i + 1]) != hipSuccess) {
      st = fail(GLA_ERR_HIP, "reading profiling events failed");
      break;
    }
    total[g_prof.kind[i]] += ms;
    count[g_prof.kind[i]] += 1;
  }
  for (auto &e : g_prof.ev) (void)hipEventDestroy(e);
  g_prof.ev.clear();
  g_prof.on = false;
  int n = 0;
  for (int k = 0; k < kNumKinds; ++k) {
    if (count[k] == 0) continue;
    if (out && n < max_out) {
      snprintf(out[n].name, sizeof out[n].name, "%s", kKindNames[k]);
      out[n].launches = count[k];
      out[n].total_ms = total[k];
    }
    ++n;
  }
  if (n_out) *n_out = n;
  return st;
}
