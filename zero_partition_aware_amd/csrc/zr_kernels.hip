// HIP kernels and their C-ABI entry points for CDNA4 (gfx950).
//
// Every kernel here is an HBM-bound stream: no data is reused, so there is no
// LDS staging and no MFMA.  Work is cut into tiles of kTileElems elements of
// one "segment" (a merged slice of the plan, a param's piece of an IPG
// window, a ring chunk); a workgroup walks tiles with a grid-stride loop and
// finds each tile's segment by a binary search over per-segment tile offsets.
// Inside a tile, each lane handles groups of VE consecutive elements, VE being
// one 16-byte load of the input type (8 bf16 or 4 fp32), so that every load
// instruction of a wavefront covers 1 KiB of contiguous memory.  A group is
// taken on the vector path when it lies wholly inside the segment and every
// stream it touches is 16-byte aligned there; the alignment phase is derived
// per segment from the actual addresses, so any element-aligned pointers
// work, and groups at ragged segment edges fall back to element-wise code.
//
// Arithmetic follows the method's definition exactly: each replica's value is
// divided by D first, the quotients are summed in rank order 0..R-1 starting
// from the rank-0 quotient, every operation is a separate fp32 operation
// (this file is compiled with -ffp-contract=off; subnormals are kept).  When D
// is a power of two, x * (1/D) is the same correctly rounded number as x / D,
// so the multiply is used; otherwise a true IEEE division.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <set>
#include <string>
#include <tuple>
#include <vector>

#include "zr_internal.h"

using zr::fail;

namespace {

constexpr int kThreads = 256;
constexpr int64_t kTileElems = 4096;
constexpr int kIpgMaxSegs = 48;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------ device helpers

template <typename T>
__device__ __forceinline__ T ld_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const T*>(p));
}
template <typename T>
__device__ __forceinline__ void st_stream(void* p, T v) {
  __builtin_nontemporal_store(v, reinterpret_cast<T*>(p));
}

__device__ __forceinline__ bool aligned(uint64_t addr, uint64_t bytes) {
  return (addr & (bytes - 1)) == 0;
}

// Input element types: bf16 as its 16-bit pattern, or fp32.
template <typename InT> struct In;
template <> struct In<uint16_t> {
  static constexpr int VE = 8;  // elements per 16-byte load
  __device__ static __forceinline__ float widen(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
  }
  __device__ static __forceinline__ void unpack(u32x4 w, float* x) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};
template <> struct In<float> {
  static constexpr int VE = 4;
  __device__ static __forceinline__ float widen(float v) { return v; }
  __device__ static __forceinline__ void unpack(u32x4 w, float* x) {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(w[i]);
  }
};

// fp32 -> bf16, round to nearest even; NaN becomes a quiet NaN with its sign
// and top payload bits.
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  uint32_t b = __float_as_uint(x);
  if ((b & 0x7fffffffu) > 0x7f800000u) return (b >> 16) | 0x40u;
  b += 0x7fffu + ((b >> 16) & 1u);
  return b >> 16;
}

struct AdamConsts {
  float b1, c1, b2, c2, bc1, bc2, lr, eps;  // c = 1 - b, bc = 1 - b^t
};

// One Adam step on one element, each operation a separate fp32 operation.
__device__ __forceinline__ void adam_elem(const AdamConsts& k, float g,
                                          float& th, float& m, float& v) {
  const float m1 = k.b1 * m + k.c1 * g;
  const float gg = g * g;
  const float v1 = k.b2 * v + k.c2 * gg;
  const float mh = m1 / k.bc1;
  const float vh = v1 / k.bc2;
  const float denom = __builtin_sqrtf(vh) + k.eps;
  const float upd = (k.lr * mh) / denom;
  th = th - upd;
  m = m1;
  v = v1;
}

// ------------------------------------------------------ reduce (+ Adam) ---

struct Seg {
  int64_t flat;   // first element in the source's index space
  int64_t part;   // first element in the destination partition
  int64_t numel;
  int64_t tile0;  // first tile of this segment (segs[nseg].tile0 = total)
  int32_t dst;    // destination partition
  int32_t pad;    // 1: padding -- gradient 0, no replica is read
};

struct RedArgs {
  uint64_t in[ZR_MAX_WORLD];   // replica r's flat element f: in[r] + f*sizeof
  uint64_t out[ZR_MAX_WORLD];  // reduce mode: partition d's element j: out[d] + 4j
  const Seg* segs;
  int64_t total_tiles;
  int32_t nseg;
  int32_t R;
  float divisor;
  float inv_divisor;
  // fused mode: the one destination partition's buffers
  float* master;
  float* m;
  float* v;
  uint16_t* pbf16;
  float* gout;
  AdamConsts ac;
};

template <bool kDiv>
__device__ __forceinline__ float predivide(const RedArgs& a, float x) {
  if constexpr (kDiv) return x / a.divisor;
  else return x * a.inv_divisor;
}

// Reduced gradient of VE consecutive flat elements starting at f (vector path).
template <typename InT, int R, bool kDiv>
__device__ __forceinline__ void reduce_vec(const RedArgs& a, int rr, int64_t f,
                                           float* acc) {
  constexpr int VE = In<InT>::VE;
  const uint64_t off = static_cast<uint64_t>(f) * sizeof(InT);
  if constexpr (R > 0) {
    u32x4 w[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
      w[r] = ld_stream<u32x4>(reinterpret_cast<const void*>(a.in[r] + off));
    float x[VE];
    In<InT>::unpack(w[0], x);
#pragma unroll
    for (int e = 0; e < VE; ++e) acc[e] = (R == 1) ? x[e] : predivide<kDiv>(a, x[e]);
#pragma unroll
    for (int r = 1; r < R; ++r) {
      In<InT>::unpack(w[r], x);
#pragma unroll
      for (int e = 0; e < VE; ++e) acc[e] = acc[e] + predivide<kDiv>(a, x[e]);
    }
  } else {
    float x[VE];
    In<InT>::unpack(ld_stream<u32x4>(reinterpret_cast<const void*>(a.in[0] + off)), x);
#pragma unroll
    for (int e = 0; e < VE; ++e) acc[e] = (rr == 1) ? x[e] : predivide<kDiv>(a, x[e]);
    for (int r = 1; r < rr; ++r) {
      In<InT>::unpack(ld_stream<u32x4>(reinterpret_cast<const void*>(a.in[r] + off)), x);
#pragma unroll
      for (int e = 0; e < VE; ++e) acc[e] = acc[e] + predivide<kDiv>(a, x[e]);
    }
  }
}

// Reduced gradient of one flat element (edge path).
template <typename InT, int R, bool kDiv>
__device__ __forceinline__ float reduce_one(const RedArgs& a, int rr, int64_t f) {
  const int n = R > 0 ? R : rr;
  const uint64_t off = static_cast<uint64_t>(f) * sizeof(InT);
  float acc = In<InT>::widen(*reinterpret_cast<const InT*>(a.in[0] + off));
  if (n > 1) acc = predivide<kDiv>(a, acc);
  for (int r = 1; r < n; ++r) {
    const float x = In<InT>::widen(*reinterpret_cast<const InT*>(a.in[r] + off));
    acc = acc + predivide<kDiv>(a, x);
  }
  return acc;
}

template <typename InT, int R, bool kDiv, bool kFused>
__global__ __launch_bounds__(kThreads) void reduce_kernel(const RedArgs a) {
  constexpr int VE = In<InT>::VE;
  constexpr int U = static_cast<int>(kTileElems / (kThreads * VE));
  const int rr = R > 0 ? R : a.R;

  for (int64_t t = blockIdx.x; t < a.total_tiles; t += gridDim.x) {
    int lo = 0, hi = a.nseg - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.segs[mid].tile0 <= t) lo = mid; else hi = mid - 1;
    }
    const Seg sg = a.segs[lo];
    const int64_t lt = t - sg.tile0;

    // First offset j (0 <= j < VE) at which every stream is 16-byte aligned.
    int j0 = -1;
    for (int j = 0; j < VE && j0 < 0; ++j) {
      bool ok = true;
      if (!sg.pad)
        for (int r = 0; r < rr; ++r)
          ok = ok && aligned(a.in[r] + static_cast<uint64_t>(sg.flat + j) * sizeof(InT), 16);
      const uint64_t p4 = static_cast<uint64_t>(sg.part + j) * 4;
      if constexpr (kFused) {
        ok = ok && aligned(reinterpret_cast<uint64_t>(a.master) + p4, 16) &&
             aligned(reinterpret_cast<uint64_t>(a.m) + p4, 16) &&
             aligned(reinterpret_cast<uint64_t>(a.v) + p4, 16);
        if (a.pbf16)
          ok = ok && aligned(reinterpret_cast<uint64_t>(a.pbf16) + p4 / 2, VE * 2);
        if (a.gout) ok = ok && aligned(reinterpret_cast<uint64_t>(a.gout) + p4, 16);
      } else {
        ok = ok && aligned(a.out[sg.dst] + p4, 16);
      }
      if (ok) j0 = j;
    }
    const bool vec = j0 >= 0;
    const int64_t rel0 = (j0 > 0 ? j0 - VE : 0) + lt * kTileElems;

#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t rel = rel0 + static_cast<int64_t>(u * kThreads + threadIdx.x) * VE;
      if (rel >= sg.numel || rel + VE <= 0) continue;
      if (vec && rel >= 0 && rel + VE <= sg.numel) {
        float g[VE];
        if (sg.pad) {
#pragma unroll
          for (int e = 0; e < VE; ++e) g[e] = 0.0f;
        } else {
          reduce_vec<InT, R, kDiv>(a, rr, sg.flat + rel, g);
        }
        const int64_t j = sg.part + rel;
        if constexpr (!kFused) {
          float* o = reinterpret_cast<float*>(a.out[sg.dst]) + j;
#pragma unroll
          for (int q = 0; q < VE / 4; ++q)
            st_stream<f32x4>(o + 4 * q, f32x4{g[4 * q], g[4 * q + 1], g[4 * q + 2], g[4 * q + 3]});
        } else {
          float th[VE], mm[VE], vv[VE];
#pragma unroll
          for (int q = 0; q < VE / 4; ++q) {
            const f32x4 a0 = ld_stream<f32x4>(a.master + j + 4 * q);
            const f32x4 a1 = ld_stream<f32x4>(a.m + j + 4 * q);
            const f32x4 a2 = ld_stream<f32x4>(a.v + j + 4 * q);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              th[4 * q + i] = a0[i];
              mm[4 * q + i] = a1[i];
              vv[4 * q + i] = a2[i];
            }
          }
#pragma unroll
          for (int e = 0; e < VE; ++e) adam_elem(a.ac, g[e], th[e], mm[e], vv[e]);
#pragma unroll
          for (int q = 0; q < VE / 4; ++q) {
            st_stream<f32x4>(a.master + j + 4 * q, f32x4{th[4 * q], th[4 * q + 1], th[4 * q + 2], th[4 * q + 3]});
            st_stream<f32x4>(a.m + j + 4 * q, f32x4{mm[4 * q], mm[4 * q + 1], mm[4 * q + 2], mm[4 * q + 3]});
            st_stream<f32x4>(a.v + j + 4 * q, f32x4{vv[4 * q], vv[4 * q + 1], vv[4 * q + 2], vv[4 * q + 3]});
            if (a.gout)
              st_stream<f32x4>(a.gout + j + 4 * q, f32x4{g[4 * q], g[4 * q + 1], g[4 * q + 2], g[4 * q + 3]});
          }
          if (a.pbf16) {
            uint32_t h[VE];
#pragma unroll
            for (int e = 0; e < VE; ++e) h[e] = bf16_rne(th[e]);
            if constexpr (VE == 8) {
              st_stream<u32x4>(a.pbf16 + j, u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16),
                                                  h[4] | (h[5] << 16), h[6] | (h[7] << 16)});
            } else {
              st_stream<u32x2>(a.pbf16 + j, u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)});
            }
          }
        }
      } else {
        const int64_t e0 = rel < 0 ? 0 : rel;
        const int64_t e1 = rel + VE < sg.numel ? rel + VE : sg.numel;
        for (int64_t e = e0; e < e1; ++e) {
          const float g = sg.pad ? 0.0f : reduce_one<InT, R, kDiv>(a, rr, sg.flat + e);
          const int64_t j = sg.part + e;
          if constexpr (!kFused) {
            reinterpret_cast<float*>(a.out[sg.dst])[j] = g;
          } else {
            float th = a.master[j], mm = a.m[j], vv = a.v[j];
            adam_elem(a.ac, g, th, mm, vv);
            a.master[j] = th;
            a.m[j] = mm;
            a.v[j] = vv;
            if (a.gout) a.gout[j] = g;
            if (a.pbf16) a.pbf16[j] = static_cast<uint16_t>(bf16_rne(th));
          }
        }
      }
    }
  }
}

// ------------------------------------------------------- standalone Adam ---

struct AdamArgs {
  const float* grad;
  float* master;
  float* m;
  float* v;
  uint16_t* pbf16;
  int64_t n;
  AdamConsts ac;
};

// Contiguous partition; kVec: every pointer 16-byte aligned (bf16 8-byte).
template <bool kVec>
__global__ __launch_bounds__(kThreads) void adam_kernel(const AdamArgs a) {
  constexpr int64_t VE = 4;
  const int64_t ntiles = (a.n + kTileElems - 1) / kTileElems;
  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
#pragma unroll
    for (int u = 0; u < static_cast<int>(kTileElems / (kThreads * VE)); ++u) {
      const int64_t j = t * kTileElems + (u * kThreads + threadIdx.x) * VE;
      if (j >= a.n) continue;
      if (kVec && j + VE <= a.n) {
        const f32x4 g = ld_stream<f32x4>(a.grad + j);
        f32x4 th = ld_stream<f32x4>(a.master + j);
        f32x4 mm = ld_stream<f32x4>(a.m + j);
        f32x4 vv = ld_stream<f32x4>(a.v + j);
        float t4[4], m4[4], v4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          t4[e] = th[e];
          m4[e] = mm[e];
          v4[e] = vv[e];
          adam_elem(a.ac, g[e], t4[e], m4[e], v4[e]);
        }
        st_stream<f32x4>(a.master + j, f32x4{t4[0], t4[1], t4[2], t4[3]});
        st_stream<f32x4>(a.m + j, f32x4{m4[0], m4[1], m4[2], m4[3]});
        st_stream<f32x4>(a.v + j, f32x4{v4[0], v4[1], v4[2], v4[3]});
        if (a.pbf16)
          st_stream<u32x2>(a.pbf16 + j, u32x2{bf16_rne(t4[0]) | (bf16_rne(t4[1]) << 16),
                                              bf16_rne(t4[2]) | (bf16_rne(t4[3]) << 16)});
      } else {
        const int64_t e1 = j + VE < a.n ? j + VE : a.n;
        for (int64_t e = j; e < e1; ++e) {
          float th = a.master[e], mm = a.m[e], vv = a.v[e];
          adam_elem(a.ac, a.grad[e], th, mm, vv);
          a.master[e] = th;
          a.m[e] = mm;
          a.v[e] = vv;
          if (a.pbf16) a.pbf16[e] = static_cast<uint16_t>(bf16_rne(th));
        }
      }
    }
  }
}

// ----------------------------------------------------------------- IPG ---

struct IpgSeg {
  uint64_t src;   // address of the segment's first gradient element
  int64_t dst;    // first element index in the main_grad window
  int64_t numel;
  int64_t tile0;
};

struct IpgArgs {
  IpgSeg seg[kIpgMaxSegs];
  int64_t total_tiles;
  float* main_grad;
  int32_t nseg;
};

template <typename InT>
__global__ __launch_bounds__(kThreads) void ipg_kernel(const IpgArgs a) {
  constexpr int VE = In<InT>::VE;
  constexpr int U = static_cast<int>(kTileElems / (kThreads * VE));
  for (int64_t t = blockIdx.x; t < a.total_tiles; t += gridDim.x) {
    int s = 0;
    while (s + 1 < a.nseg && a.seg[s + 1].tile0 <= t) ++s;
    const IpgSeg sg = a.seg[s];
    const int64_t lt = t - sg.tile0;
    const uint64_t mg = reinterpret_cast<uint64_t>(a.main_grad);
    int j0 = -1;
    for (int j = 0; j < VE && j0 < 0; ++j)
      if (aligned(sg.src + j * sizeof(InT), 16) &&
          aligned(mg + static_cast<uint64_t>(sg.dst + j) * 4, 16))
        j0 = j;
    const bool vec = j0 >= 0;
    const int64_t rel0 = (j0 > 0 ? j0 - VE : 0) + lt * kTileElems;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t rel = rel0 + static_cast<int64_t>(u * kThreads + threadIdx.x) * VE;
      if (rel >= sg.numel || rel + VE <= 0) continue;
      if (vec && rel >= 0 && rel + VE <= sg.numel) {
        float x[VE];
        In<InT>::unpack(ld_stream<u32x4>(reinterpret_cast<const void*>(sg.src + rel * sizeof(InT))), x);
        float* o = a.main_grad + sg.dst + rel;
#pragma unroll
        for (int q = 0; q < VE / 4; ++q) {
          const f32x4 cur = ld_stream<f32x4>(o + 4 * q);
          st_stream<f32x4>(o + 4 * q, f32x4{cur[0] + x[4 * q], cur[1] + x[4 * q + 1],
                                            cur[2] + x[4 * q + 2], cur[3] + x[4 * q + 3]});
        }
      } else {
        const int64_t e0 = rel < 0 ? 0 : rel;
        const int64_t e1 = rel + VE < sg.numel ? rel + VE : sg.numel;
        for (int64_t e = e0; e < e1; ++e) {
          const float x = In<InT>::widen(*reinterpret_cast<const InT*>(sg.src + e * sizeof(InT)));
          a.main_grad[sg.dst + e] = a.main_grad[sg.dst + e] + x;
        }
      }
    }
  }
}

// --------------------------------------------------------------- copy ---

struct CopyArgs {
  const float* src;  // bucket-layout source
  float* dst;        // partition
  const Seg* segs;   // flat = bucket offset, part = partition offset
  int64_t total_tiles;
  int32_t nseg;
};

__global__ __launch_bounds__(kThreads) void copy_kernel(const CopyArgs a) {
  constexpr int VE = 4;
  constexpr int U = static_cast<int>(kTileElems / (kThreads * VE));
  for (int64_t t = blockIdx.x; t < a.total_tiles; t += gridDim.x) {
    int lo = 0, hi = a.nseg - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.segs[mid].tile0 <= t) lo = mid; else hi = mid - 1;
    }
    const Seg sg = a.segs[lo];
    const int64_t lt = t - sg.tile0;
    const float* s = a.src + sg.flat;
    float* d = a.dst + sg.part;
    int j0 = -1;
    for (int j = 0; j < VE && j0 < 0; ++j)
      if (aligned(reinterpret_cast<uint64_t>(s + j), 16) &&
          aligned(reinterpret_cast<uint64_t>(d + j), 16))
        j0 = j;
    const bool vec = j0 >= 0;
    const int64_t rel0 = (j0 > 0 ? j0 - VE : 0) + lt * kTileElems;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t rel = rel0 + static_cast<int64_t>(u * kThreads + threadIdx.x) * VE;
      if (rel >= sg.numel || rel + VE <= 0) continue;
      if (vec && rel >= 0 && rel + VE <= sg.numel) {
        st_stream<f32x4>(d + rel, ld_stream<f32x4>(s + rel));
      } else {
        const int64_t e0 = rel < 0 ? 0 : rel;
        const int64_t e1 = rel + VE < sg.numel ? rel + VE : sg.numel;
        for (int64_t e = e0; e < e1; ++e) d[e] = s[e];
      }
    }
  }
}

// --------------------------------------------------------------- ring ---

struct RingArgs {
  uint64_t buf[ZR_MAX_WORLD];
  int64_t chunk;
  int64_t tiles_per_rank;
  int32_t n;
  int32_t step;
};

__global__ __launch_bounds__(kThreads) void ring_kernel(const RingArgs a) {
  constexpr int VE = 4;
  constexpr int U = static_cast<int>(kTileElems / (kThreads * VE));
  const int64_t total = a.tiles_per_rank * a.n;
  for (int64_t t = blockIdx.x; t < total; t += gridDim.x) {
    const int k = static_cast<int>(t / a.tiles_per_rank);
    const int64_t lt = t - static_cast<int64_t>(k) * a.tiles_per_rank;
    int c = (k - a.step - 2) % a.n;
    if (c < 0) c += a.n;
    const int prev = (k == 0) ? a.n - 1 : k - 1;
    float* d = reinterpret_cast<float*>(a.buf[k]) + static_cast<int64_t>(c) * a.chunk;
    const float* s = reinterpret_cast<const float*>(a.buf[prev]) + static_cast<int64_t>(c) * a.chunk;
    int j0 = -1;
    for (int j = 0; j < VE && j0 < 0; ++j)
      if (aligned(reinterpret_cast<uint64_t>(s + j), 16) &&
          aligned(reinterpret_cast<uint64_t>(d + j), 16))
        j0 = j;
    const bool vec = j0 >= 0;
    const int64_t rel0 = (j0 > 0 ? j0 - VE : 0) + lt * kTileElems;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t rel = rel0 + static_cast<int64_t>(u * kThreads + threadIdx.x) * VE;
      if (rel >= a.chunk || rel + VE <= 0) continue;
      if (vec && rel >= 0 && rel + VE <= a.chunk) {
        const f32x4 x = ld_stream<f32x4>(s + rel);
        const f32x4 y = ld_stream<f32x4>(d + rel);
        st_stream<f32x4>(d + rel, f32x4{y[0] + x[0], y[1] + x[1], y[2] + x[2], y[3] + x[3]});
      } else {
        const int64_t e0 = rel < 0 ? 0 : rel;
        const int64_t e1 = rel + VE < a.chunk ? rel + VE : a.chunk;
        for (int64_t e = e0; e < e1; ++e) d[e] = d[e] + s[e];
      }
    }
  }
}

// ================================================================= host ===

int64_t tiles_for(int64_t numel) {
  // +7: a segment whose start is not group-aligned spans one extra group.
  return (numel + 7 + kTileElems - 1) / kTileElems;
}

// Launch tables derived from a plan: the host segment list (pure host data,
// used for validation) and its device copy, both built on first use.
struct HostTable {
  std::vector<Seg> segs;  // nseg entries + a sentinel holding the total tiles
};
struct DevTable {
  Seg* dev = nullptr;
  int device = 0;
};
enum TableKind { kReduceTable = 0, kCopyTable = 1 };
using HostKey = std::tuple<int, int32_t, int64_t, int32_t>;      // kind, group, bucket, dst
using DevKey = std::tuple<int, int, int32_t, int64_t, int32_t>;  // device + HostKey

struct DevCache {
  std::mutex mu;
  std::map<HostKey, HostTable> host;
  std::map<DevKey, DevTable> dev;
};

void release_cache(void* p) {
  DevCache* c = static_cast<DevCache*>(p);
  int cur = 0;
  const bool have = hipGetDevice(&cur) == hipSuccess;
  for (auto& kv : c->dev)
    if (kv.second.dev) {
      (void)hipSetDevice(kv.second.device);
      (void)hipFree(kv.second.dev);
    }
  if (have) (void)hipSetDevice(cur);
  delete c;
}

std::mutex g_cache_init_mu;

DevCache* cache_of(const zr_plan* plan) {
  zr_plan* p = const_cast<zr_plan*>(plan);  // the cache is not plan state
  std::lock_guard<std::mutex> lk(g_cache_init_mu);
  if (!p->dev) {
    p->dev = new DevCache();
    p->dev_release = release_cache;
  }
  return static_cast<DevCache*>(p->dev);
}

int g_cu_count[64] = {0};

zr_status device_info(int* dev, int* cus) {
  hipError_t e = hipGetDevice(dev);
  if (e != hipSuccess) return fail(ZR_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (*dev < 0 || *dev >= 64) return fail(ZR_ERR_UNSUPPORTED, "device index above 63");
  if (g_cu_count[*dev] == 0) {
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, *dev);
    if (e != hipSuccess) return fail(ZR_ERR_HIP, std::string("hipDeviceGetAttribute: ") + hipGetErrorString(e));
    g_cu_count[*dev] = n > 0 ? n : 1;
  }
  *cus = g_cu_count[*dev];
  return ZR_OK;
}

unsigned grid_for(int64_t tiles, int cus) {
  const int64_t cap = static_cast<int64_t>(cus) * 8;
  return static_cast<unsigned>(std::max<int64_t>(1, std::min(tiles, cap)));
}

// Segments of `group`, `bucket` (-1 all), `dst` (-1 all) in bucket order, plus
// the padding of the selected partitions when the call covers the last bucket
// (reduce tables only); each gets its tile offset.
std::vector<Seg> build_segments(const zr_plan* plan, int kind, int32_t group,
                                int64_t bucket, int32_t dst) {
  std::vector<Seg> out;
  const int64_t a = bucket < 0 ? 0 : plan->bucket_first[bucket];
  const int64_t b = bucket < 0 ? static_cast<int64_t>(plan->slices.size())
                               : plan->bucket_first[bucket + 1];
  for (int64_t i = a; i < b; ++i) {
    const zr_slice& s = plan->slices[i];
    if (s.group != group || (dst >= 0 && s.dst != dst)) continue;
    Seg g{};
    g.flat = kind == kCopyTable ? s.bucket_offset : s.flat_offset;
    g.part = s.part_offset;
    g.numel = s.numel;
    g.dst = s.dst;
    g.pad = 0;
    out.push_back(g);
  }
  if (kind == kReduceTable && (bucket < 0 || bucket == plan->num_buckets - 1)) {
    const zr::GroupInfo& gi = plan->groups[group];
    for (int32_t k = 0; k < gi.world; ++k) {
      if (dst >= 0 && k != dst) continue;
      const int64_t start = std::max(gi.total, k * gi.part);
      const int64_t end = (k + 1) * gi.part;
      if (start >= end) continue;
      Seg g{};
      g.flat = start;
      g.part = start - k * gi.part;
      g.numel = end - start;
      g.dst = k;
      g.pad = 1;
      out.push_back(g);
    }
  }
  int64_t tiles = 0;
  for (auto& g : out) {
    g.tile0 = tiles;
    tiles += tiles_for(g.numel);
  }
  Seg sentinel{};
  sentinel.tile0 = tiles;
  out.push_back(sentinel);
  return out;
}

// Host segment list for a call (no HIP call is made).
zr_status get_host_table(const zr_plan* plan, int kind, int32_t group, int64_t bucket,
                         int32_t dst, const std::vector<Seg>** out) {
  DevCache* c = cache_of(plan);
  std::lock_guard<std::mutex> lk(c->mu);
  const HostKey key{kind, group, bucket, dst};
  auto it = c->host.find(key);
  if (it == c->host.end()) {
    HostTable t;
    try {
      t.segs = build_segments(plan, kind, group, bucket, dst);
    } catch (const std::bad_alloc&) {
      return fail(ZR_ERR_OOM, "out of host memory building a launch table");
    }
    it = c->host.emplace(key, std::move(t)).first;
  }
  *out = &it->second.segs;  // std::map nodes are stable
  return ZR_OK;
}

// Device copy of the same list on `device` (synchronous upload on first use).
zr_status get_dev_table(const zr_plan* plan, int kind, int32_t group, int64_t bucket,
                        int32_t dst, int device, const std::vector<Seg>& host,
                        const Seg** out) {
  DevCache* c = cache_of(plan);
  std::lock_guard<std::mutex> lk(c->mu);
  const DevKey key{device, kind, group, bucket, dst};
  auto it = c->dev.find(key);
  if (it != c->dev.end()) {
    *out = it->second.dev;
    return ZR_OK;
  }
  DevTable t;
  t.device = device;
  const size_t bytes = host.size() * sizeof(Seg);
  hipError_t e = hipMalloc(&t.dev, bytes);
  if (e != hipSuccess) return fail(ZR_ERR_OOM, std::string("hipMalloc: ") + hipGetErrorString(e));
  e = hipMemcpy(t.dev, host.data(), bytes, hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    (void)hipFree(t.dev);
    return fail(ZR_ERR_HIP, std::string("hipMemcpy: ") + hipGetErrorString(e));
  }
  c->dev.emplace(key, t);
  *out = t.dev;
  return ZR_OK;
}

zr_status check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(ZR_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return ZR_OK;
}

size_t dtype_size(zr_dtype d) { return d == ZR_BF16 ? 2 : 4; }
bool valid_dtype(zr_dtype d) { return d == ZR_BF16 || d == ZR_FP32; }
bool elem_aligned(const void* p, size_t s) { return (reinterpret_cast<uintptr_t>(p) % s) == 0; }
bool pow2(int32_t d) { return d > 0 && (d & (d - 1)) == 0; }

zr_status adam_consts(const zr_adam* h, AdamConsts* k) {
  if (!h) return fail(ZR_ERR_INVALID, "adam hyper-parameters are null");
  if (h->step < 1) return fail(ZR_ERR_INVALID, "adam step must be >= 1");
  if (!(h->beta1 >= 0.0 && h->beta1 < 1.0) || !(h->beta2 >= 0.0 && h->beta2 < 1.0))
    return fail(ZR_ERR_INVALID, "adam betas must lie in [0, 1)");
  if (!(h->eps >= 0.0) || !(h->lr == h->lr))
    return fail(ZR_ERR_INVALID, "adam eps must be >= 0 and lr a number");
  const double t = static_cast<double>(h->step);
  k->b1 = static_cast<float>(h->beta1);
  k->c1 = static_cast<float>(1.0 - h->beta1);
  k->b2 = static_cast<float>(h->beta2);
  k->c2 = static_cast<float>(1.0 - h->beta2);
  k->bc1 = static_cast<float>(1.0 - std::pow(h->beta1, t));
  k->bc2 = static_cast<float>(1.0 - std::pow(h->beta2, t));
  k->lr = static_cast<float>(h->lr);
  k->eps = static_cast<float>(h->eps);
  if (!(k->bc1 > 0.0f) || !(k->bc2 > 0.0f))
    return fail(ZR_ERR_INVALID, "adam bias correction rounds to 0");
  return ZR_OK;
}

template <typename InT, bool kFused>
zr_status launch_reduce_t(const RedArgs& a, int R, bool div, unsigned grid, hipStream_t st) {
#define ZR_LAUNCH(RR, DD) reduce_kernel<InT, RR, DD, kFused><<<grid, kThreads, 0, st>>>(a)
  if (div) {
    switch (R) {
      case 2: ZR_LAUNCH(2, true); break;
      case 3: ZR_LAUNCH(3, true); break;
      case 4: ZR_LAUNCH(4, true); break;
      case 6: ZR_LAUNCH(6, true); break;
      case 8: ZR_LAUNCH(8, true); break;
      default: ZR_LAUNCH(0, true); break;
    }
  } else {
    switch (R) {
      case 1: ZR_LAUNCH(1, false); break;
      case 2: ZR_LAUNCH(2, false); break;
      case 4: ZR_LAUNCH(4, false); break;
      case 8: ZR_LAUNCH(8, false); break;
      case 16: ZR_LAUNCH(16, false); break;
      default: ZR_LAUNCH(0, false); break;
    }
  }
#undef ZR_LAUNCH
  return check_launch(kFused ? "reduce_scatter_adam launch" : "reduce_scatter launch");
}

// Shared validation + launch of the reduce kernel in either mode.
zr_status run_reduce(const zr_plan* plan, int32_t group, int64_t bucket, int32_t dst,
                     const zr_replica* reps, zr_dtype dt, float* const* part_out,
                     const zr_adam* h, float* master, float* m, float* v,
                     uint16_t* pbf16, float* gout, bool fused, hipStream_t stream) {
  zr::clear_error();
  if (!plan) return fail(ZR_ERR_INVALID, "plan is null");
  if (group < 0 || group >= static_cast<int32_t>(plan->groups.size()))
    return fail(ZR_ERR_INVALID, "group index out of range");
  if (bucket < -1 || bucket >= plan->num_buckets)
    return fail(ZR_ERR_INVALID, "bucket index out of range");
  const zr::GroupInfo& gi = plan->groups[group];
  if (dst < -1 || dst >= gi.world) return fail(ZR_ERR_INVALID, "dst out of range");
  if (fused && dst < 0) return fail(ZR_ERR_INVALID, "the fused step needs one dst");
  if (!reps) return fail(ZR_ERR_INVALID, "replicas are null");
  if (!valid_dtype(dt)) return fail(ZR_ERR_INVALID, "unsupported gradient dtype");
  const size_t s = dtype_size(dt);
  for (int r = 0; r < gi.world; ++r) {
    if (!reps[r].ptr) return fail(ZR_ERR_INVALID, "replica " + std::to_string(r) + " is null");
    if (!elem_aligned(reps[r].ptr, s))
      return fail(ZR_ERR_INVALID, "replica " + std::to_string(r) + " is not element-aligned");
    if (reps[r].flat_base < 0 || reps[r].len < 0)
      return fail(ZR_ERR_INVALID, "replica window has a negative base or length");
  }
  RedArgs a;
  std::memset(&a, 0, sizeof(a));
  AdamConsts ac{};
  if (fused) {
    zr_status st = adam_consts(h, &ac);
    if (st != ZR_OK) return st;
    if (!master || !m || !v) return fail(ZR_ERR_INVALID, "master, m and v are required");
    if (!elem_aligned(master, 4) || !elem_aligned(m, 4) || !elem_aligned(v, 4) ||
        (gout && !elem_aligned(gout, 4)) || (pbf16 && !elem_aligned(pbf16, 2)))
      return fail(ZR_ERR_INVALID, "partition buffers are not element-aligned");
    a.master = master;
    a.m = m;
    a.v = v;
    a.pbf16 = pbf16;
    a.gout = gout;
    a.ac = ac;
  } else {
    if (!part_out) return fail(ZR_ERR_INVALID, "part_out is null");
    const int nout = dst < 0 ? gi.world : 1;
    for (int i = 0; i < nout; ++i) {
      if (!part_out[i]) return fail(ZR_ERR_INVALID, "a partition output is null");
      if (!elem_aligned(part_out[i], 4))
        return fail(ZR_ERR_INVALID, "a partition output is not element-aligned");
      a.out[dst < 0 ? i : dst] = reinterpret_cast<uint64_t>(part_out[i]);
    }
  }
  const std::vector<Seg>* hs = nullptr;
  zr_status st = get_host_table(plan, kReduceTable, group, bucket, dst, &hs);
  if (st != ZR_OK) return st;
  const int nseg = static_cast<int>(hs->size()) - 1;
  // Every replica window must cover every slice this call reads.
  for (int i = 0; i < nseg; ++i) {
    const Seg& g = (*hs)[i];
    if (g.pad) continue;
    for (int r = 0; r < gi.world; ++r)
      if (g.flat < reps[r].flat_base || g.flat + g.numel > reps[r].flat_base + reps[r].len)
        return fail(ZR_ERR_INVALID, "replica " + std::to_string(r) +
                                        " window does not cover flat elements [" +
                                        std::to_string(g.flat) + ", " +
                                        std::to_string(g.flat + g.numel) + ")");
  }
  if (nseg == 0) return ZR_OK;
  int device = 0, cus = 1;
  st = device_info(&device, &cus);
  if (st != ZR_OK) return st;
  st = get_dev_table(plan, kReduceTable, group, bucket, dst, device, *hs, &a.segs);
  if (st != ZR_OK) return st;
  for (int r = 0; r < gi.world; ++r)
    a.in[r] = reinterpret_cast<uint64_t>(reps[r].ptr) -
              static_cast<uint64_t>(reps[r].flat_base) * s;
  a.nseg = nseg;
  a.total_tiles = (*hs)[nseg].tile0;
  a.R = gi.world;
  a.divisor = static_cast<float>(gi.divisor);
  a.inv_divisor = 1.0f / static_cast<float>(gi.divisor);
  const bool div = !pow2(gi.divisor);
  const unsigned grid = grid_for(a.total_tiles, cus);
  if (dt == ZR_BF16)
    return fused ? launch_reduce_t<uint16_t, true>(a, gi.world, div, grid, stream)
                 : launch_reduce_t<uint16_t, false>(a, gi.world, div, grid, stream);
  return fused ? launch_reduce_t<float, true>(a, gi.world, div, grid, stream)
               : launch_reduce_t<float, false>(a, gi.world, div, grid, stream);
}

}  // namespace

// =============================================================== C ABI ===

extern "C" zr_status zr_reduce_scatter_local(const zr_plan* plan, int32_t group,
                                             int64_t bucket, int32_t dst,
                                             const zr_replica* reps, zr_dtype grad_dtype,
                                             float* const* part_out, hipStream_t stream) {
  try {
    return run_reduce(plan, group, bucket, dst, reps, grad_dtype, part_out, nullptr,
                      nullptr, nullptr, nullptr, nullptr, nullptr, false, stream);
  } catch (...) {
    return fail(ZR_ERR_OOM, "unexpected host error");
  }
}

extern "C" zr_status zr_reduce_scatter_adam(const zr_plan* plan, int32_t group,
                                            int64_t bucket, int32_t dst,
                                            const zr_replica* reps, zr_dtype grad_dtype,
                                            const zr_adam* h, float* master, float* m,
                                            float* v, uint16_t* param_bf16,
                                            float* grad_out, hipStream_t stream) {
  try {
    return run_reduce(plan, group, bucket, dst, reps, grad_dtype, nullptr, h, master, m,
                      v, param_bf16, grad_out, true, stream);
  } catch (...) {
    return fail(ZR_ERR_OOM, "unexpected host error");
  }
}

extern "C" zr_status zr_adam_partition(const zr_adam* h, const float* grad, float* master,
                                       float* m, float* v, uint16_t* param_bf16,
                                       int64_t n, hipStream_t stream) {
  zr::clear_error();
  AdamArgs a{};
  zr_status st = adam_consts(h, &a.ac);
  if (st != ZR_OK) return st;
  if (n < 0) return fail(ZR_ERR_INVALID, "n must be >= 0");
  if (n == 0) return ZR_OK;
  if (!grad || !master || !m || !v) return fail(ZR_ERR_INVALID, "null buffer");
  if (!elem_aligned(grad, 4) || !elem_aligned(master, 4) || !elem_aligned(m, 4) ||
      !elem_aligned(v, 4) || (param_bf16 && !elem_aligned(param_bf16, 2)))
    return fail(ZR_ERR_INVALID, "buffers are not element-aligned");
  int device = 0, cus = 1;
  st = device_info(&device, &cus);
  if (st != ZR_OK) return st;
  a.grad = grad;
  a.master = master;
  a.m = m;
  a.v = v;
  a.pbf16 = param_bf16;
  a.n = n;
  const bool vec = elem_aligned(grad, 16) && elem_aligned(master, 16) &&
                   elem_aligned(m, 16) && elem_aligned(v, 16) &&
                   (!param_bf16 || elem_aligned(param_bf16, 8));
  const unsigned grid = grid_for((n + kTileElems - 1) / kTileElems, cus);
  if (vec) adam_kernel<true><<<grid, kThreads, 0, stream>>>(a);
  else adam_kernel<false><<<grid, kThreads, 0, stream>>>(a);
  return check_launch("adam_partition launch");
}

extern "C" zr_status zr_ipg_accumulate(const zr_plan* plan, const int64_t* param_ids,
                                       const void* const* grads, int64_t n,
                                       zr_dtype grad_dtype, float* main_grad,
                                       int64_t window_base, int64_t window_len,
                                       hipStream_t stream) {
  zr::clear_error();
  try {
    if (!plan) return fail(ZR_ERR_INVALID, "plan is null");
    if (n < 0) return fail(ZR_ERR_INVALID, "n must be >= 0");
    if (n > 0 && (!param_ids || !grads)) return fail(ZR_ERR_INVALID, "null param list");
    if (!valid_dtype(grad_dtype)) return fail(ZR_ERR_INVALID, "unsupported gradient dtype");
    if (window_base < 0 || window_len < 0)
      return fail(ZR_ERR_INVALID, "window base and length must be >= 0");
    if (window_len > 0 && (!main_grad || !elem_aligned(main_grad, 4)))
      return fail(ZR_ERR_INVALID, "main_grad is null or not element-aligned");
    const size_t s = dtype_size(grad_dtype);
    const int64_t np = static_cast<int64_t>(plan->params.size());
    std::set<int64_t> seen;
    int32_t group = -1;
    std::vector<IpgSeg> segs;
    for (int64_t i = 0; i < n; ++i) {
      const int64_t p = param_ids[i];
      if (p < 0 || p >= np) return fail(ZR_ERR_INVALID, "param id out of range");
      if (!seen.insert(p).second) return fail(ZR_ERR_INVALID, "param listed twice in one call");
      const zr::ParamInfo& pi = plan->params[p];
      if (group < 0) group = pi.group;
      if (pi.group != group) return fail(ZR_ERR_INVALID, "params of one call must share a group");
      if (!grads[i] || !elem_aligned(grads[i], s))
        return fail(ZR_ERR_INVALID, "gradient pointer is null or not element-aligned");
      const int64_t lo = std::max(pi.offset, window_base);
      const int64_t hi = std::min(pi.offset + pi.numel, window_base + window_len);
      if (lo >= hi) continue;
      IpgSeg g{};
      g.src = reinterpret_cast<uint64_t>(grads[i]) + static_cast<uint64_t>(lo - pi.offset) * s;
      g.dst = lo - window_base;
      g.numel = hi - lo;
      segs.push_back(g);
    }
    if (group >= 0 && window_base + window_len > plan->groups[group].padded)
      return fail(ZR_ERR_INVALID, "window runs past the group's padded flat space");
    if (segs.empty()) return ZR_OK;
    int device = 0, cus = 1;
    zr_status st = device_info(&device, &cus);
    if (st != ZR_OK) return st;
    for (size_t b = 0; b < segs.size(); b += kIpgMaxSegs) {
      IpgArgs a;
      std::memset(&a, 0, sizeof(a));
      const size_t e = std::min(segs.size(), b + kIpgMaxSegs);
      int64_t tiles = 0;
      for (size_t i = b; i < e; ++i) {
        a.seg[i - b] = segs[i];
        a.seg[i - b].tile0 = tiles;
        tiles += tiles_for(segs[i].numel);
      }
      a.nseg = static_cast<int32_t>(e - b);
      a.total_tiles = tiles;
      a.main_grad = main_grad;
      const unsigned grid = grid_for(tiles, cus);
      if (grad_dtype == ZR_BF16) ipg_kernel<uint16_t><<<grid, kThreads, 0, stream>>>(a);
      else ipg_kernel<float><<<grid, kThreads, 0, stream>>>(a);
      st = check_launch("ipg_accumulate launch");
      if (st != ZR_OK) return st;
    }
    return ZR_OK;
  } catch (...) {
    return fail(ZR_ERR_OOM, "unexpected host error");
  }
}

extern "C" zr_status zr_copy_grads_in_partition(const zr_plan* plan, int32_t group,
                                                int64_t bucket, int32_t dst,
                                                const float* bucket_layout_src,
                                                float* part_out, hipStream_t stream) {
  zr::clear_error();
  try {
    if (!plan) return fail(ZR_ERR_INVALID, "plan is null");
    if (group < 0 || group >= static_cast<int32_t>(plan->groups.size()))
      return fail(ZR_ERR_INVALID, "group index out of range");
    if (bucket < 0 || bucket >= plan->num_buckets)
      return fail(ZR_ERR_INVALID, "bucket index out of range (one bucket per call)");
    if (dst < 0 || dst >= plan->groups[group].world)
      return fail(ZR_ERR_INVALID, "dst out of range");
    if (!bucket_layout_src || !part_out || !elem_aligned(bucket_layout_src, 4) ||
        !elem_aligned(part_out, 4))
      return fail(ZR_ERR_INVALID, "buffers are null or not element-aligned");
    const std::vector<Seg>* hs = nullptr;
    zr_status st = get_host_table(plan, kCopyTable, group, bucket, dst, &hs);
    if (st != ZR_OK) return st;
    const int nseg = static_cast<int>(hs->size()) - 1;
    if (nseg == 0) return ZR_OK;
    int device = 0, cus = 1;
    st = device_info(&device, &cus);
    if (st != ZR_OK) return st;
    CopyArgs a{};
    st = get_dev_table(plan, kCopyTable, group, bucket, dst, device, *hs, &a.segs);
    if (st != ZR_OK) return st;
    a.src = bucket_layout_src;
    a.dst = part_out;
    a.nseg = nseg;
    a.total_tiles = (*hs)[nseg].tile0;
    copy_kernel<<<grid_for(a.total_tiles, cus), kThreads, 0, stream>>>(a);
    return check_launch("copy_grads_in_partition launch");
  } catch (...) {
    return fail(ZR_ERR_OOM, "unexpected host error");
  }
}

extern "C" zr_status zr_ring_rs_step(float* const* rank_bufs, int32_t n_ranks,
                                     int64_t chunk_numel, int32_t step,
                                     hipStream_t stream) {
  zr::clear_error();
  if (n_ranks < 2 || n_ranks > ZR_MAX_WORLD)
    return fail(ZR_ERR_INVALID, "n_ranks must lie in [2, ZR_MAX_WORLD]");
  if (step < 0 || step > n_ranks - 2) return fail(ZR_ERR_INVALID, "step out of range");
  if (chunk_numel < 0) return fail(ZR_ERR_INVALID, "chunk_numel must be >= 0");
  if (!rank_bufs) return fail(ZR_ERR_INVALID, "rank_bufs is null");
  const uint64_t bytes = static_cast<uint64_t>(chunk_numel) * n_ranks * 4;
  for (int k = 0; k < n_ranks; ++k) {
    if (!rank_bufs[k] || !elem_aligned(rank_bufs[k], 4))
      return fail(ZR_ERR_INVALID, "a rank buffer is null or not element-aligned");
    for (int j = 0; j < k; ++j) {
      const uint64_t a0 = reinterpret_cast<uint64_t>(rank_bufs[k]);
      const uint64_t b0 = reinterpret_cast<uint64_t>(rank_bufs[j]);
      if (bytes > 0 && a0 < b0 + bytes && b0 < a0 + bytes)
        return fail(ZR_ERR_INVALID, "rank buffers overlap");
    }
  }
  if (chunk_numel == 0) return ZR_OK;
  int device = 0, cus = 1;
  zr_status st = device_info(&device, &cus);
  if (st != ZR_OK) return st;
  RingArgs a;
  std::memset(&a, 0, sizeof(a));
  for (int k = 0; k < n_ranks; ++k) a.buf[k] = reinterpret_cast<uint64_t>(rank_bufs[k]);
  a.chunk = chunk_numel;
  a.tiles_per_rank = tiles_for(chunk_numel);
  a.n = n_ranks;
  a.step = step;
  ring_kernel<<<grid_for(a.tiles_per_rank * n_ranks, cus), kThreads, 0, stream>>>(a);
  return check_launch("ring_rs_step launch");
}
