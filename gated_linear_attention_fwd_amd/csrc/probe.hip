// probe.hip -- streaming HBM bandwidth probes for measurement tools.
//
// Plain kernels that move a buffer through HBM in the access patterns the
// mixer's kernels use: 16-byte loads and stores per lane covering whole
// 1 KiB runs per wave, plain or nontemporal. Timed with events, they give the
// practical ceilings the mixer's kernels are held against: a read-only
// stream (kv reads k and v), a write-only stream, a copy, and two reads plus
// one write (the readout reads q and g and writes o).
//
// Each thread takes kUnroll 16-byte pieces per iteration (the loads of one
// iteration are in flight together). Two layouts, the faster of each
// measured on the 1 GiB buffers of the ceiling measurement: the write-only
// probes give every workgroup a contiguous 256 KiB range; the others stride
// over the buffer with a grid of 8192 workgroups, so that the workgroups in
// flight sweep one region of memory together (nontemporal read 6.6 -> 6.9,
// two reads and one write 5.7 -> 6.1 TB/s against contiguous ranges).
// Read-only probes fold what they load into one word per thread and store it
// only if it equals a value no input of the measurement produces, so the
// loads cannot be dropped.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "mfma_util.hpp"

namespace gla {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kUnroll = 4;
constexpr int64_t kRangePieces = int64_t(kProbeThreads) * kUnroll * 16;  // 256 KiB per workgroup
constexpr int64_t kStrideGrid = 8192;  // workgroups of the striding layout

enum ProbeKind {
  kRead = 0,
  kReadNt = 1,
  kWrite = 2,
  kWriteNt = 3,
  kCopy = 4,
  kCopyNt = 5,
  kRead2Write1 = 6,
  kRead2Write1Nt = 7,
  kRead2WriteEighth = 8,
  kNumProbeKinds = 9
};

template <bool kNt>
__device__ __forceinline__ void st16(uint4 *p, uint4 v) {
  if constexpr (kNt) {
    st_stream16(p, v);
  } else {
    *p = v;
  }
}

// n: 16-byte pieces. a, b read; out written (as the kind needs).
template <int kKind>
__global__ __launch_bounds__(kProbeThreads) void probe_kernel(const uint4 *__restrict__ a,
                                                             const uint4 *__restrict__ b,
                                                             uint4 *__restrict__ out, int64_t n,
                                                             uint32_t *__restrict__ sink) {
  constexpr bool kNt = (kKind & 1) != 0 || kKind == kRead2WriteEighth;
  constexpr bool kTwo = kKind == kRead2Write1 || kKind == kRead2Write1Nt || kKind == kRead2WriteEighth;
  constexpr bool kRanges = kKind == kWrite || kKind == kWriteNt;
  // ranges: [r0, r1) of this workgroup; striding: the whole buffer
  const int64_t r0 = kRanges ? (int64_t)blockIdx.x * kRangePieces : 0;
  const int64_t r1 = kRanges ? min(r0 + kRangePieces, n) : n;
  const int64_t first = kRanges ? r0 : (int64_t)blockIdx.x * kProbeThreads * kUnroll;
  const int64_t step = kProbeThreads * kUnroll * (kRanges ? 1 : (int64_t)gridDim.x);
  uint32_t fold = 0;
  int64_t it = blockIdx.x;  // kRead2WriteEighth: this iteration writes when it % 8 == 7
  for (int64_t base = first + threadIdx.x; base < r1; base += step, ++it) {
    uint4 x[kUnroll], y[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = min(base + (int64_t)u * kProbeThreads, r1 - 1);
      if constexpr (kKind != kWrite && kKind != kWriteNt) x[u] = ld_stream16<kNt>(a + i);
      if constexpr (kTwo) y[u] = ld_stream16<kNt>(b + i);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + (int64_t)u * kProbeThreads;
      if constexpr (kKind == kRead || kKind == kReadNt) {
        fold ^= x[u].x ^ x[u].y ^ x[u].z ^ x[u].w;
      } else if constexpr (kKind == kRead2WriteEighth) {
        // every workgroup writes on one iteration in eight, a different one for
        // neighbouring workgroups (with the grid a multiple of 8, exactly an
        // eighth of each iteration's pieces)
        if ((it & 7) == 7 && i < r1)
          out[i] = make_uint4(x[u].x ^ y[u].x, x[u].y ^ y[u].y, x[u].z ^ y[u].z, x[u].w ^ y[u].w);
      } else if (i < r1) {
        if constexpr (kKind == kWrite || kKind == kWriteNt) {
          const uint32_t w = (uint32_t)i;
          st16<kNt>(out + i, make_uint4(w, w, w, w));
        } else if constexpr (kKind == kCopy || kKind == kCopyNt) {
          st16<kNt>(out + i, x[u]);
        } else {
          st16<kNt>(out + i, make_uint4(x[u].x ^ y[u].x, x[u].y ^ y[u].y, x[u].z ^ y[u].z,
                                        x[u].w ^ y[u].w));
        }
      }
    }
  }
  if constexpr (kKind == kRead || kKind == kReadNt) {
    if (fold == 0x9E3779B9u) sink[blockIdx.x * kProbeThreads + threadIdx.x] = fold;
  }
}

}  // namespace

// kind: ProbeKind; bytes a multiple of 256 KiB (checked by the caller).
hipError_t launch_probe(int kind, const void *a, const void *b, void *out, size_t bytes,
                        hipStream_t s) {
  const int64_t n = (int64_t)(bytes / 16);
  const bool ranges = kind == kWrite || kind == kWriteNt;
  // striding: at most kStrideGrid workgroups, each iteration of the grid
  // covering kStrideGrid * 16 KiB (the caller's size is a multiple of 256 KiB,
  // so a grid of n / (256 KiB) workgroups divides it exactly when smaller)
  const int64_t ranges_grid = (n + kRangePieces - 1) / kRangePieces;
  int64_t grid = ranges_grid;
  if (!ranges) {
    grid = kStrideGrid;
    while (grid > 1 && n % (grid * kProbeThreads * kUnroll)) grid /= 2;
  }
  if (n == 0) return hipSuccess;
  const uint4 *pa = static_cast<const uint4 *>(a), *pb = static_cast<const uint4 *>(b);
  uint4 *po = static_cast<uint4 *>(out);
  uint32_t *sink = static_cast<uint32_t *>(out);
#define GLA_PROBE(K)                                                                         \
  case K:                                                                                    \
    hipLaunchKernelGGL(probe_kernel<K>, dim3((unsigned)grid), dim3(kProbeThreads), 0, s, pa, \
                       pb, po, n, sink);                                                     \
    break;
  switch (kind) {
    GLA_PROBE(kRead)
    GLA_PROBE(kReadNt)
    GLA_PROBE(kWrite)
    GLA_PROBE(kWriteNt)
    GLA_PROBE(kCopy)
    GLA_PROBE(kCopyNt)
    GLA_PROBE(kRead2Write1)
    GLA_PROBE(kRead2Write1Nt)
    GLA_PROBE(kRead2WriteEighth)
    default:
      return hipErrorInvalidValue;
  }
#undef GLA_PROBE
  return hipGetLastError();
}

int probe_kinds() { return kNumProbeKinds; }

}  // namespace gla
