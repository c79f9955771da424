// abi_driver.cpp -- drives every entry point of the C ABI, built for the host
// with the launchers replaced by abi_stubs.cpp, under AddressSanitizer and
// UndefinedBehaviorSanitizer (the test that builds it aborts on the first
// report).
//
// Valid calls get host buffers of exactly the documented sizes (workspaces of
// exactly what the *_workspace query returns), so every range a launcher's
// plan reaches is checked against the buffer it lands in; the expected
// launches are checked by name. Invalid calls must return the documented
// status and launch nothing. Size queries and calls with sizes that overflow
// must be refused without undefined arithmetic.
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/gla.h"
#include "abi_stubs.hpp"

namespace {

int g_failures = 0;
int g_checks = 0;

#define CHECK(cond, ...)                                              \
  do {                                                                \
    ++g_checks;                                                       \
    if (!(cond)) {                                                    \
      ++g_failures;                                                   \
      std::fprintf(stderr, "FAIL %s:%d: %s -- ", __FILE__, __LINE__, #cond); \
      std::fprintf(stderr, __VA_ARGS__);                              \
      std::fprintf(stderr, " [last error: %s]\n", gla_last_error()); \
    }                                                                 \
  } while (0)

// A host buffer of exactly n bytes, 256-byte aligned (a distinct, inaccessible
// address for n == 0: empty tensors still get a pointer).
struct Buf {
  void *p = nullptr;
  explicit Buf(size_t n) {
    if (posix_memalign(&p, 256, n) != 0 || !p) {
      std::fprintf(stderr, "out of host memory for %zu bytes\n", n);
      std::exit(2);
    }
    if (n) std::memset(p, 0, n < 4096 ? n : 4096);
  }
  ~Buf() { std::free(p); }
  Buf(const Buf &) = delete;
  Buf &operator=(const Buf &) = delete;
  float *f() const { return static_cast<float *>(p); }
  char *c() const { return static_cast<char *>(p); }
};

size_t es_of(gla_dtype dt) { return dt == GLA_F32 ? 4 : 2; }

std::string launches() {
  std::string s;
  for (const auto &n : stubs::g_log) s += (s.empty() ? "" : ",") + n;
  return s;
}

void reset() { stubs::g_log.clear(); }

// All the buffers of one frame-causal call, sized from the header's layout.
struct FcBufs {
  int B, H, F, T, d;
  gla_dtype dt;
  int64_t BH, N;
  Buf q, k, v, g, o, gamma, S_in, z_in, S_out, z_out, states;
  FcBufs(int B_, int H_, int F_, int T_, int d_, gla_dtype dt_)
      : B(B_), H(H_), F(F_), T(T_), d(d_), dt(dt_), BH((int64_t)B_ * H_),
        N((int64_t)F_ * T_),
        q(BH * N * d * es_of(dt)), k(BH * N * d * es_of(dt)), v(BH * N * d * es_of(dt)),
        g(BH * N * d * es_of(dt)), o(BH * N * d * es_of(dt)), gamma(BH * F * 4),
        S_in(BH * d * d * 4), z_in(BH * d * 4), S_out(BH * d * d * 4), z_out(BH * d * 4),
        states(BH * F * ((int64_t)d * d + d) * 4) {}
};

// ---------------------------------------------------------------- forward
void forward_calls() {
  struct Shape { int B, H, F, T, d; gla_dtype dt; };
  const Shape shapes[] = {
      {1, 2, 5, 77, 64, GLA_BF16},   {2, 1, 37, 32, 32, GLA_BF16}, {1, 3, 4, 100, 16, GLA_F32},
      {1, 1, 9, 33, 128, GLA_BF16},  {1, 2, 3, 50, 64, GLA_F32},   {2, 2, 1, 1, 32, GLA_BF16},
      {1, 32, 241, 920, 64, GLA_BF16},  // 720p / 60 s latents: large buffers, corners touched
      {1, 1, 3, 0, 64, GLA_BF16},    {1, 1, 0, 10, 64, GLA_BF16},  {0, 4, 5, 77, 64, GLA_BF16},
  };
  for (const Shape &s : shapes) {
    FcBufs b(s.B, s.H, s.F, s.T, s.d, s.dt);
    const size_t wsb = gla_fwd_framecausal_workspace(s.B, s.H, s.F, s.T, s.d);
    Buf ws(wsb);
    // carried state in and out (in place), then without any state
    reset();
    gla_status st = gla_fwd_framecausal(b.q.p, b.k.p, b.v.p, b.g.p, b.gamma.f(), b.S_in.f(),
                                        b.z_in.f(), b.o.p, b.S_in.f(), b.z_in.f(), s.B, s.H, s.F,
                                        s.T, s.d, s.dt, 1e-6f, ws.p, wsb, nullptr);
    CHECK(st == GLA_OK, "framecausal B%d H%d F%d T%d d%d: status %d", s.B, s.H, s.F, s.T, s.d, st);
    if (b.BH > 0 && s.F > 0 && s.T > 0)
      CHECK(launches() == "kv,carry,readout", "framecausal launches %s", launches().c_str());
    reset();
    st = gla_fwd_framecausal(b.q.p, b.k.p, b.v.p, b.g.p, b.gamma.f(), nullptr, nullptr, b.o.p,
                             b.S_out.f(), b.z_out.f(), s.B, s.H, s.F, s.T, s.d, s.dt, 0.f, ws.p,
                             wsb, nullptr);
    CHECK(st == GLA_OK, "framecausal without S_in: status %d", st);

    // the record of every frame's state
    const size_t wss = wsb;
    reset();
    st = gla_fwd_framecausal_states(b.q.p, b.k.p, b.v.p, b.g.p, b.gamma.f(), b.S_in.f(),
                                    b.z_in.f(), b.o.p, b.S_out.f(), b.z_out.f(), b.states.f(),
                                    s.B, s.H, s.F, s.T, s.d, s.dt, 1e-6f, ws.p, wss, nullptr);
    CHECK(st == GLA_OK, "states: status %d", st);

    // block-cache commit
    reset();
    st = gla_state_carry(b.k.p, b.v.p, b.gamma.f(), b.S_in.f(), b.z_in.f(), b.S_out.f(),
                         b.z_out.f(), s.B, s.H, s.F, s.T, s.d, s.dt,
                         ws.p, gla_state_carry_workspace(s.B, s.H, s.F, s.T, s.d), nullptr);
    CHECK(st == GLA_OK, "state carry: status %d", st);
    if (b.BH > 0 && s.F > 0)
      CHECK(launches() == "kv,carry", "state carry launches %s", launches().c_str());

    // the same tokens as one bidirectional sequence
    const size_t wbb = gla_fwd_bidir_workspace(s.B, s.H, b.N, s.d);
    Buf wb(wbb);
    reset();
    st = gla_fwd_bidir(b.q.p, b.k.p, b.v.p, b.g.p, b.o.p, s.B, s.H, b.N, s.d, s.dt, 1e-6f, wb.p,
                       wbb, nullptr);
    CHECK(st == GLA_OK, "bidir N=%lld: status %d", (long long)b.N, st);
    if (b.BH > 0 && b.N > 0)
      CHECK(launches() == "kv,carry,readout", "bidir launches %s", launches().c_str());
  }
}

// Heads between tokens and features ([B][N][H][d]) with 3D rotary positions.
void strided_calls() {
  const int B = 2, H = 3, F = 4, T = 6 * 10, d = 64;
  const gla_dtype dt = GLA_BF16;
  const int64_t N = (int64_t)F * T;
  const size_t bytes = (size_t)B * N * H * d * 2;
  Buf q(bytes), k(bytes), v(bytes), g(bytes), o(bytes), dO(bytes), dq(bytes), dk(bytes),
      dv(bytes), dg(bytes);
  const int64_t sb = N * H * d, sh = d, sn = (int64_t)H * d;
  auto view = [&](const Buf &x) { return gla_tensor{x.p, sb, sh, sn}; };
  const gla_tensor tq = view(q), tk = view(k), tv = view(v), tg = view(g), to = view(o),
                   tdO = view(dO), tdq = view(dq), tdk = view(dk), tdv = view(dv), tdg = view(dg);
  const gla_rope3d rope{6, 10, 3, 16, 24, 24, 10000.0};
  Buf gamma((size_t)B * H * F * 4), S((size_t)B * H * d * d * 4), z((size_t)B * H * d * 4),
      dS((size_t)B * H * d * d * 4), dz((size_t)B * H * d * 4), dgamma((size_t)B * H * F * 4),
      states((size_t)B * H * F * ((int64_t)d * d + d) * 4);

  for (const gla_rope3d *r : {(const gla_rope3d *)nullptr, &rope}) {
    size_t n = gla_fwd_bidir_ex_workspace(B, H, F, T, d, r);
    Buf w1(n);
    reset();
    gla_status st = gla_fwd_bidir_ex(&tq, &tk, &tv, &tg, &to, B, H, F, T, d, dt, 1e-6f, r, w1.p,
                                     n, nullptr);
    CHECK(st == GLA_OK, "bidir_ex rope=%d: status %d", r != nullptr, st);

    n = gla_fwd_framecausal_workspace(B, H, F, T, d);
    Buf w2(n);
    st = gla_fwd_framecausal_ex(&tq, &tk, &tv, &tg, gamma.f(), S.f(), z.f(), &to, S.f(), z.f(), B,
                                H, F, T, d, dt, 1e-6f, r, w2.p, n, nullptr);
    CHECK(st == GLA_OK, "framecausal_ex rope=%d: status %d", r != nullptr, st);
    st = gla_state_carry_ex(&tk, &tv, gamma.f(), nullptr, nullptr, S.f(), z.f(), B, H, F, T, d,
                            dt, r, w2.p, n, nullptr);
    CHECK(st == GLA_OK, "state_carry_ex rope=%d: status %d", r != nullptr, st);
    st = gla_fwd_framecausal_states_ex(&tq, &tk, &tv, &tg, gamma.f(), nullptr, nullptr, &to,
                                       nullptr, nullptr, states.f(), B, H, F, T, d, dt, 1e-6f, r,
                                       w2.p, n, nullptr);
    CHECK(st == GLA_OK, "states_ex rope=%d: status %d", r != nullptr, st);

    n = gla_bwd_framecausal_states_workspace(B, H, F, T, d);
    Buf w3(n);
    reset();
    st = gla_bwd_framecausal_ex(&tq, &tk, &tv, &tg, gamma.f(), S.f(), z.f(), states.f(), &tdO,
                                dS.f(), dz.f(), &tdq, &tdk, &tdv, &tdg, dgamma.f(), nullptr,
                                nullptr, B, H, F, T, d, dt, 1e-6f, r, w3.p, n, nullptr);
    CHECK(st == GLA_OK, "bwd_framecausal_ex rope=%d: status %d", r != nullptr, st);
    CHECK(launches().find("bwd_q") != std::string::npos, "bwd launches %s", launches().c_str());

    n = gla_bwd_bidir_ex_workspace(B, H, F, T, d, r);
    Buf w4(n);
    st = gla_bwd_bidir_ex(&tq, &tk, &tv, &tg, &tdO, &tdq, &tdk, &tdv, &tdg, B, H, F, T, d, dt,
                          1e-6f, r, w4.p, n, nullptr);
    CHECK(st == GLA_OK, "bwd_bidir_ex rope=%d: status %d", r != nullptr, st);
  }
}

// ---------------------------------------------------------------- backward
void backward_calls() {
  struct Shape { int B, H, F, T, d; gla_dtype dt; };
  const Shape shapes[] = {{1, 2, 5, 77, 64, GLA_BF16}, {2, 1, 3, 40, 16, GLA_F32},
                          {1, 1, 2, 130, 128, GLA_BF16}, {1, 4, 1, 1, 32, GLA_BF16},
                          {1, 32, 241, 920, 64, GLA_BF16}};
  for (const Shape &s : shapes) {
    FcBufs b(s.B, s.H, s.F, s.T, s.d, s.dt);
    const size_t tb = b.BH * b.N * s.d * es_of(s.dt);
    Buf dO(tb), dq(tb), dk(tb), dv(tb), dg(tb), dS_out(b.BH * s.d * s.d * 4),
        dz_out(b.BH * s.d * 4), dgamma(b.BH * s.F * 4), dS_in(b.BH * s.d * s.d * 4),
        dz_in(b.BH * s.d * 4);
    size_t n = gla_bwd_framecausal_workspace(s.B, s.H, s.F, s.T, s.d);
    Buf w(n);
    reset();
    gla_status st = gla_bwd_framecausal(
        b.q.p, b.k.p, b.v.p, b.g.p, b.gamma.f(), b.S_in.f(), b.z_in.f(), dO.p, dS_out.f(),
        dz_out.f(), dq.p, dk.p, dv.p, dg.p, dgamma.f(), dS_in.f(), dz_in.f(), s.B, s.H, s.F, s.T,
        s.d, s.dt, 1e-6f, w.p, n, nullptr);
    CHECK(st == GLA_OK, "bwd_framecausal B%d H%d F%d T%d d%d: status %d", s.B, s.H, s.F, s.T,
          s.d, st);
    CHECK(launches() == "kv,carry,bwd_q,rev_scan,bwd_k,dgamma", "bwd launches %s",
          launches().c_str());
    st = gla_bwd_framecausal(b.q.p, b.k.p, b.v.p, b.g.p, b.gamma.f(), nullptr, nullptr, dO.p,
                             nullptr, nullptr, dq.p, dk.p, dv.p, dg.p, nullptr, nullptr, nullptr,
                             s.B, s.H, s.F, s.T, s.d, s.dt, 1e-6f, w.p, n, nullptr);
    CHECK(st == GLA_OK, "bwd_framecausal without states or dgamma: status %d", st);

    n = gla_bwd_framecausal_states_workspace(s.B, s.H, s.F, s.T, s.d);
    Buf w2(n);
    reset();
    st = gla_bwd_framecausal_states(b.q.p, b.k.p, b.v.p, b.g.p, b.gamma.f(), b.S_in.f(),
                                    b.z_in.f(), b.states.f(), dO.p, dS_out.f(), dz_out.f(), dq.p,
                                    dk.p, dv.p, dg.p, dgamma.f(), dS_in.f(), dz_in.f(), s.B, s.H,
                                    s.F, s.T, s.d, s.dt, 1e-6f, w2.p, n, nullptr);
    CHECK(st == GLA_OK, "bwd_framecausal_states: status %d", st);
    CHECK(launches().find("kv") == std::string::npos, "saved states recomputed: %s",
          launches().c_str());

    n = gla_bwd_bidir_workspace(s.B, s.H, b.N, s.d);
    Buf w3(n);
    st = gla_bwd_bidir(b.q.p, b.k.p, b.v.p, b.g.p, dO.p, dq.p, dk.p, dv.p, dg.p, s.B, s.H, b.N,
                       s.d, s.dt, 1e-6f, w3.p, n, nullptr);
    CHECK(st == GLA_OK, "bwd_bidir: status %d", st);
  }
}

// ------------------------------------------------- Gated DeltaNet, anchor
void other_calls() {
  for (int F : {3, 70}) {
    const int B = 1, H = 2, T = 40, d = 64;
    const int64_t BH = B * H, N = (int64_t)F * T;
    Buf q(BH * N * d * 2), k(BH * N * d * 2), v(BH * N * d * 2), o(BH * N * d * 2),
        beta(BH * N * 4), gamma(BH * F * 4), S(BH * d * d * 4);
    const size_t n = gla_gdn_framecausal_workspace(B, H, F, T, d);
    Buf w(n);
    reset();
    gla_status st = gla_gdn_framecausal(q.p, k.p, v.p, beta.f(), gamma.f(), S.f(), o.p, S.f(), B,
                                        H, F, T, d, GLA_BF16, 0.02f, w.p, n, nullptr);
    CHECK(st == GLA_OK, "gdn F=%d: status %d", F, st);
    CHECK(launches() == "gdn_kv,gdn_scan,gdn_readout", "gdn launches %s", launches().c_str());
  }
  for (int causal : {0, 1})
    for (gla_dtype dt : {GLA_BF16, GLA_F32}) {
      const int B = 1, H = 2, Fq = 2, F = 5, T = 90, d = 64;
      const size_t es = es_of(dt);
      Buf q((size_t)B * H * Fq * T * d * es), g((size_t)B * H * Fq * T * d * es),
          o((size_t)B * H * Fq * T * d * es), k((size_t)B * H * F * T * d * es),
          v((size_t)B * H * F * T * d * es);
      reset();
      const gla_status st = gla_softmax_anchor(q.p, k.p, v.p, g.p, o.p, B, H, Fq, F, T, d, dt,
                                               causal, 1, 2, 0.125f, nullptr);
      CHECK(st == GLA_OK, "anchor causal=%d dt=%d: status %d", causal, dt, st);
      CHECK(launches() == "anchor,anchor_redo", "anchor launches %s", launches().c_str());
    }
}

// ------------------------------------------------------ allocation-free call
void noalloc_calls() {
  FcBufs b(1, 4, 6, 300, 64, GLA_BF16);
  reset();
  gla_status st = gla_fwd_framecausal_noalloc(b.q.p, b.k.p, b.v.p, b.g.p, b.gamma.f(), nullptr,
                                              nullptr, b.o.p, b.S_out.f(), b.z_out.f(), 1, 4, 6,
                                              300, 64, GLA_BF16, 1e-6f, nullptr);
  CHECK(st == GLA_OK, "noalloc: status %d", st);
  CHECK(launches() == "kv,carry,readout", "noalloc launches %s", launches().c_str());
  // far more workspace than the static scratch holds: refused, nothing launched
  reset();
  st = gla_fwd_framecausal_noalloc(b.q.p, b.k.p, b.v.p, b.g.p, b.gamma.f(), nullptr, nullptr,
                                   b.o.p, nullptr, nullptr, 64, 64, 1000, 920, 128, GLA_BF16,
                                   1e-6f, nullptr);
  CHECK(st == GLA_ERR_WORKSPACE, "noalloc beyond the scratch: status %d", st);
  CHECK(stubs::g_log.empty(), "noalloc beyond the scratch launched %s", launches().c_str());
}

// --------------------------------------------------- probes and timing
void probe_and_profile_calls() {
  const size_t n = 256 << 10;
  Buf a(n), b(n), out(n);
  for (int kind = 0; kind < 9; ++kind) {
    reset();
    CHECK(gla_stream_probe(kind, a.p, b.p, out.p, n, nullptr) == GLA_OK, "probe kind %d", kind);
    CHECK(launches() == "probe", "probe launches %s", launches().c_str());
  }
  reset();
  CHECK(gla_stream_probe(9, a.p, b.p, out.p, n, nullptr) != GLA_OK, "probe kind 9 accepted");
  CHECK(gla_stream_probe(8, a.p, nullptr, out.p, n, nullptr) != GLA_OK, "kv-mix probe without b");
  CHECK(gla_stream_probe(0, a.p, b.p, out.p, n + 16, nullptr) != GLA_OK, "odd size accepted");
  CHECK(gla_stream_probe(4, a.p, b.p, a.p, n, nullptr) != GLA_OK, "aliased copy accepted");
  CHECK(stubs::g_log.empty(), "refused probes launched %s", launches().c_str());

  FcBufs fb(1, 2, 4, 64, 64, GLA_BF16);
  const size_t wsb = gla_fwd_framecausal_workspace(1, 2, 4, 64, 64);
  Buf ws(wsb);
  CHECK(gla_profile_begin(2) == GLA_OK, "profile_begin");
  for (int rep = 0; rep < 2; ++rep)  // 6 launches, 2 timed
    CHECK(gla_fwd_framecausal(fb.q.p, fb.k.p, fb.v.p, fb.g.p, fb.gamma.f(), nullptr, nullptr,
                              fb.o.p, nullptr, nullptr, 1, 2, 4, 64, 64, GLA_BF16, 1e-6f, ws.p,
                              wsb, nullptr) == GLA_OK,
          "timed call");
  gla_kernel_time kt[16];
  int nk = -1;
  CHECK(gla_profile_end(kt, 16, &nk) == GLA_OK, "profile_end");
  int launches_seen = 0;
  for (int i = 0; i < nk; ++i) {
    CHECK(std::memchr(kt[i].name, 0, sizeof kt[i].name) != nullptr, "unterminated name");
    launches_seen += kt[i].launches;
  }
  CHECK(nk > 0 && launches_seen == 2, "profile: %d kinds, %d launches", nk, launches_seen);
  CHECK(gla_profile_end(kt, 16, &nk) != GLA_OK, "a second profile_end succeeded");
}

// ------------------------------------------------------ refused arguments
void refused_calls() {
  const int B = 1, H = 2, F = 3, T = 64, d = 64;
  FcBufs b(B, H, F, T, d, GLA_BF16);
  const size_t wsb = gla_fwd_framecausal_workspace(B, H, F, T, d);
  Buf ws(wsb);
  struct Case {
    const char *what;
    gla_status want;
    const void *q, *k;
    const float *gamma, *S_in, *z_in;
    void *o;
    float *S_out, *z_out;
    int F, T, d, dt;
    float eps;
    void *ws;
    size_t ws_bytes;
  };
  void *mis = b.q.c() + 2;
  const float nan = std::nanf("");
  const Case cases[] = {
      {"valid", GLA_OK, b.q.p, b.k.p, b.gamma.f(), nullptr, nullptr, b.o.p, nullptr, nullptr, F, T, d, 1, 1e-6f, ws.p, wsb},
      {"k NULL", GLA_ERR_NULL, b.q.p, nullptr, b.gamma.f(), nullptr, nullptr, b.o.p, nullptr, nullptr, F, T, d, 1, 1e-6f, ws.p, wsb},
      {"S_in without z_in", GLA_ERR_NULL, b.q.p, b.k.p, b.gamma.f(), b.S_in.f(), nullptr, b.o.p, nullptr, nullptr, F, T, d, 1, 1e-6f, ws.p, wsb},
      {"gamma NULL", GLA_ERR_NULL, b.q.p, b.k.p, nullptr, nullptr, nullptr, b.o.p, nullptr, nullptr, F, T, d, 1, 1e-6f, ws.p, wsb},
      {"F < 0", GLA_ERR_SHAPE, b.q.p, b.k.p, b.gamma.f(), nullptr, nullptr, b.o.p, nullptr, nullptr, -1, T, d, 1, 1e-6f, ws.p, wsb},
      {"T < 0", GLA_ERR_SHAPE, b.q.p, b.k.p, b.gamma.f(), nullptr, nullptr, b.o.p, nullptr, nullptr, F, -5, d, 1, 1e-6f, ws.p, wsb},
      {"d = 48", GLA_ERR_UNSUPPORTED, b.q.p, b.k.p, b.gamma.f(), nullptr, nullptr, b.o.p, nullptr, nullptr, F, T, 48, 1, 1e-6f, ws.p, wsb},
      {"dtype 7", GLA_ERR_UNSUPPORTED, b.q.p, b.k.p, b.gamma.f(), nullptr, nullptr, b.o.p, nullptr, nullptr, F, T, d, 7, 1e-6f, ws.p, wsb},
      {"q misaligned", GLA_ERR_ALIGN, mis, b.k.p, b.gamma.f(), nullptr, nullptr, b.o.p, nullptr, nullptr, F, T, d, 1, 1e-6f, ws.p, wsb},
      {"workspace short", GLA_ERR_WORKSPACE, b.q.p, b.k.p, b.gamma.f(), nullptr, nullptr, b.o.p, nullptr, nullptr, F, T, d, 1, 1e-6f, ws.p, wsb - 1},
      {"workspace NULL", GLA_ERR_WORKSPACE, b.q.p, b.k.p, b.gamma.f(), nullptr, nullptr, b.o.p, nullptr, nullptr, F, T, d, 1, 1e-6f, nullptr, wsb},
      {"eps NaN", GLA_ERR_VALUE, b.q.p, b.k.p, b.gamma.f(), nullptr, nullptr, b.o.p, nullptr, nullptr, F, T, d, 1, nan, ws.p, wsb},
      {"eps < 0", GLA_ERR_VALUE, b.q.p, b.k.p, b.gamma.f(), nullptr, nullptr, b.o.p, nullptr, nullptr, F, T, d, 1, -1.f, ws.p, wsb},
      {"o is q", GLA_ERR_ALIAS, b.q.p, b.k.p, b.gamma.f(), nullptr, nullptr, b.q.p, nullptr, nullptr, F, T, d, 1, 1e-6f, ws.p, wsb},
      {"o in workspace", GLA_ERR_ALIAS, b.q.p, b.k.p, b.gamma.f(), nullptr, nullptr, ws.p, nullptr, nullptr, F, T, d, 1, 1e-6f, ws.p, wsb},
      {"S_out over z_in", GLA_ERR_ALIAS, b.q.p, b.k.p, b.gamma.f(), b.S_in.f(), b.S_in.f() + 4, b.o.p, b.S_in.f(), b.z_in.f(), F, T, d, 1, 1e-6f, ws.p, wsb},
  };
  for (const Case &c : cases) {
    reset();
    const gla_status st = gla_fwd_framecausal(c.q, c.k, b.v.p, b.g.p, c.gamma, c.S_in, c.z_in, c.o,
                                              c.S_out, c.z_out, B, H, c.F, c.T, c.d,
                                              (gla_dtype)c.dt, c.eps, c.ws, c.ws_bytes, nullptr);
    CHECK(st == c.want, "%s: status %d, want %d", c.what, st, c.want);
    if (c.want != GLA_OK)
      CHECK(stubs::g_log.empty() && gla_last_error()[0], "%s: launched %s", c.what,
            launches().c_str());
  }

  // strided views: negative stride, output rows that overlap, odd strides
  gla_tensor tq{b.q.p, (int64_t)H * F * T * d, (int64_t)F * T * d, d}, tk = tq, tv = tq, tg = tq;
  tk.data = b.k.p;
  tv.data = b.v.p;
  tg.data = b.g.p;
  gla_tensor to = tq;
  to.data = b.o.p;
  struct ViewCase { const char *what; gla_tensor o; gla_status want; };
  const ViewCase vc[] = {
      {"negative stride", {b.o.p, -(int64_t)H * F * T * d, (int64_t)F * T * d, d}, GLA_ERR_SHAPE},
      {"rows overlap", {b.o.p, (int64_t)H * F * T * d, (int64_t)F * T * d, d / 2}, GLA_ERR_ALIAS},
      {"odd stride", {b.o.p, (int64_t)H * F * T * d, (int64_t)F * T * d, d + 1}, GLA_ERR_ALIGN},
      {"span over 2^62", {b.o.p, (int64_t)1 << 61, 8, d}, GLA_ERR_SHAPE},
  };
  for (const ViewCase &c : vc) {
    reset();
    const gla_status st = gla_fwd_framecausal_ex(&tq, &tk, &tv, &tg, b.gamma.f(), nullptr, nullptr,
                                                 &c.o, nullptr, nullptr, c.what[0] == 's' ? 2 : B,
                                                 H, F, T, d, GLA_BF16, 1e-6f, nullptr, ws.p, wsb,
                                                 nullptr);
    CHECK(st == c.want, "%s: status %d, want %d", c.what, st, c.want);
    CHECK(stubs::g_log.empty(), "%s launched %s", c.what, launches().c_str());
  }

  // rotary positions that do not fit
  struct RopeCase { const char *what; gla_rope3d r; gla_status want; };
  const RopeCase rc[] = {
      {"grid not T", {7, 9, 0, 16, 24, 24, 1e4}, GLA_ERR_SHAPE},
      {"odd section", {8, 8, 0, 15, 25, 24, 1e4}, GLA_ERR_SHAPE},
      {"sections not d", {8, 8, 0, 16, 16, 16, 1e4}, GLA_ERR_SHAPE},
      {"theta 0", {8, 8, 0, 16, 24, 24, 0.0}, GLA_ERR_VALUE},
      {"theta inf", {8, 8, 0, 16, 24, 24, INFINITY}, GLA_ERR_VALUE},
      {"offset 2^30", {8, 8, 1 << 30, 16, 24, 24, 1e4}, GLA_ERR_VALUE},
  };
  for (const RopeCase &c : rc) {
    reset();
    const gla_status st = gla_fwd_framecausal_ex(&tq, &tk, &tv, &tg, b.gamma.f(), nullptr, nullptr,
                                                 &to, nullptr, nullptr, B, H, F, T, d, GLA_BF16,
                                                 1e-6f, &c.r, ws.p, wsb, nullptr);
    CHECK(st == c.want, "rope %s: status %d, want %d", c.what, st, c.want);
    CHECK(stubs::g_log.empty(), "rope %s launched %s", c.what, launches().c_str());
  }

  // a launch that fails is reported with its kernel's name, and stops the call
  reset();
  stubs::g_fail_next = "readout";
  gla_status st = gla_fwd_framecausal(b.q.p, b.k.p, b.v.p, b.g.p, b.gamma.f(), nullptr, nullptr,
                                      b.o.p, nullptr, nullptr, B, H, F, T, d, GLA_BF16, 1e-6f,
                                      ws.p, wsb, nullptr);
  CHECK(st == GLA_ERR_HIP && std::strstr(gla_last_error(), "readout"),
        "failed launch: status %d", st);
  stubs::g_fail_next = "kv";
  reset();
  st = gla_fwd_framecausal(b.q.p, b.k.p, b.v.p, b.g.p, b.gamma.f(), nullptr, nullptr, b.o.p,
                           nullptr, nullptr, B, H, F, T, d, GLA_BF16, 1e-6f, ws.p, wsb, nullptr);
  CHECK(st == GLA_ERR_HIP && launches() == "kv", "failed kv launch: status %d, launches %s", st,
        launches().c_str());
  stubs::g_fail_next.clear();

  for (int s = -1; s <= 9; ++s) CHECK(gla_status_string((gla_status)s) != nullptr, "status %d", s);
}

// ----------------------------------------------- sizes at the extremes
// Every size query over a grid of extreme sizes, and the entry points with
// sizes whose tensors would span more than 2^62 bytes: refused (never
// launched), with no overflowing arithmetic on the way.
void extreme_sizes() {
  const int64_t vals[] = {0, 1, 2, 31, 33, 920, 65535, 1 << 20, INT_MAX - 1, INT_MAX};
  const int ds[] = {16, 32, 64, 128, 0, -64, 48, INT_MAX};
  const gla_rope3d rope{1, 1, 0, 0, 0, 64, 1e4};
  size_t sink = 0;
  for (int64_t B : vals)
    for (int64_t H : vals)
      for (int64_t F : vals)
        for (int64_t T : vals)
          for (int d : ds) {
            const int b = (int)B, h = (int)H, f = (int)F, t = (int)T;
            sink ^= gla_fwd_framecausal_workspace(b, h, f, t, d);
            sink ^= gla_state_carry_workspace(b, h, f, t, d);
            sink ^= gla_bwd_framecausal_workspace(b, h, f, t, d);
            sink ^= gla_bwd_framecausal_states_workspace(b, h, f, t, d);
            sink ^= gla_gdn_framecausal_workspace(b, h, f, t, d);
            sink ^= gla_fwd_bidir_ex_workspace(b, h, f, t, d, nullptr);
            sink ^= gla_fwd_bidir_ex_workspace(b, h, f, t, d, &rope);
            sink ^= gla_bwd_bidir_ex_workspace(b, h, f, t, d, nullptr);
            sink ^= gla_bwd_bidir_ex_workspace(b, h, f, t, d, &rope);
            sink ^= gla_fwd_bidir_workspace(b, h, F * T, d);
            sink ^= gla_bwd_bidir_workspace(b, h, F * T, d);
          }
  for (int64_t N : {INT64_MAX, INT64_MAX / 2, (int64_t)1 << 62, (int64_t)1 << 40}) {
    sink ^= gla_fwd_bidir_workspace(INT_MAX, INT_MAX, N, 128);
    sink ^= gla_bwd_bidir_workspace(INT_MAX, INT_MAX, N, 128);
  }
  std::printf("size queries folded to %zx\n", sink);

  // tensors spanning more than 2^62 bytes: refused before anything is touched
  // (the pointers stand for device memory and are never dereferenced on a
  // refusal)
  void *fake = reinterpret_cast<void *>(uintptr_t(1) << 20);
  float *ff = static_cast<float *>(fake);
  Buf ws(1 << 12);
  struct Big { int B, H, F, T; };
  const Big big[] = {{INT_MAX, INT_MAX, INT_MAX, INT_MAX}, {INT_MAX, INT_MAX, 1, INT_MAX},
                     {1, INT_MAX, INT_MAX, INT_MAX}, {INT_MAX, 1, INT_MAX, 2}};
  for (const Big &s : big) {
    reset();
    gla_status st = gla_fwd_framecausal(fake, fake, fake, fake, ff, nullptr, nullptr, fake,
                                        nullptr, nullptr, s.B, s.H, s.F, s.T, 128, GLA_F32, 1e-6f,
                                        ws.p, 1 << 12, nullptr);
    CHECK(st != GLA_OK && stubs::g_log.empty(), "framecausal B%d H%d F%d T%d: status %d", s.B,
          s.H, s.F, s.T, st);
    st = gla_bwd_framecausal(fake, fake, fake, fake, ff, nullptr, nullptr, fake, nullptr, nullptr,
                             fake, fake, fake, fake, nullptr, nullptr, nullptr, s.B, s.H, s.F,
                             s.T, 128, GLA_F32, 1e-6f, ws.p, 1 << 12, nullptr);
    CHECK(st != GLA_OK && stubs::g_log.empty(), "bwd_framecausal B%d H%d F%d T%d: status %d",
          s.B, s.H, s.F, s.T, st);
    st = gla_gdn_framecausal(fake, fake, fake, ff, ff, nullptr, fake, nullptr, s.B, s.H, s.F, s.T,
                             128, GLA_F32, 0.01f, ws.p, 1 << 12, nullptr);
    CHECK(st != GLA_OK && stubs::g_log.empty(), "gdn B%d H%d F%d T%d: status %d", s.B, s.H, s.F,
          s.T, st);
    st = gla_softmax_anchor(fake, fake, fake, fake, fake, s.B, s.H, s.F, s.F, s.T, 128, GLA_F32,
                            1, 1, 4, 0.1f, nullptr);
    CHECK(st != GLA_OK && stubs::g_log.empty(), "anchor B%d H%d F%d T%d: status %d", s.B, s.H,
          s.F, s.T, st);
  }
  for (int64_t N : {INT64_MAX, INT64_MAX / 2, (int64_t)1 << 62}) {
    reset();
    gla_status st = gla_fwd_bidir(fake, fake, fake, fake, fake, 4, 8, N, 128, GLA_F32, 1e-6f,
                                  ws.p, 1 << 12, nullptr);
    CHECK(st != GLA_OK && stubs::g_log.empty(), "bidir N=%lld: status %d", (long long)N, st);
    st = gla_bwd_bidir(fake, fake, fake, fake, fake, fake, fake, fake, fake, 4, 8, N, 128,
                       GLA_F32, 1e-6f, ws.p, 1 << 12, nullptr);
    CHECK(st != GLA_OK && stubs::g_log.empty(), "bwd_bidir N=%lld: status %d", (long long)N, st);
  }
}

}  // namespace

int main() {
  forward_calls();
  strided_calls();
  backward_calls();
  other_calls();
  noalloc_calls();
  probe_and_profile_calls();
  refused_calls();
  extreme_sizes();
  std::printf("%d checks, %d failures\n", g_checks, g_failures);
  return g_failures ? 1 : 0;
}
