// HIP kernels and their C-ABI entry points for CDNA4 (gfx950).
//
// Every kernel here is an HBM-bound stream: no data is reused, so there is no
// LDS staging and no MFMA (the reduce launches only reserve LDS, to hold a CU
// to a measured number of their workgroups: reduce_wgs_per_cu).  Work is cut
// into tiles of one "segment" (a merged
// slice of the plan, a param's piece of an IPG window, a ring chunk): the
// reduce kernels take 256 elements per one-wave workgroup (512 per two waves
// for the bf16 fused step), Adam 512 per 128 lanes -- one 4-element slot per
// lane -- and the lighter IPG, copy, ring reduce-scatter and all-gather
// kernels 1024 per 128 lanes (two slots per lane).  By default every
// workgroup takes exactly one tile, so the hardware dispatcher hands tiles
// out in address order and the set of DRAM pages being touched at any moment
// stays compact.  A workgroup finds its tile's segment by a binary search
// over per-segment tile offsets, read through the scalar cache.
// Reduce-kernel tiles start where replica 0's tiles sit on whole 128-byte
// lines, when the other streams allow it.
//
// Inside a tile each lane owns "slots" of four consecutive elements, and the
// 64 lanes of a wavefront own 64 consecutive slots, so every load or store
// instruction of one stream covers one contiguous range (1 KiB of fp32, 512 B
// of bf16): stores fill whole cache lines and never leave partially written
// lines behind.  All loads of a tile's slots are issued before any arithmetic.
// A slot takes the vector path when it lies wholly inside its segment and
// every stream is aligned there (16 B for fp32, 8 B for bf16); the alignment
// phase is derived per segment from the actual addresses, so any
// element-aligned pointers work, and slots at ragged segment edges fall back
// to element-wise code.  Loads and stores carry the non-temporal hint: every
// byte is touched once.  (With stores that fill only part of a line per
// instruction the same hint costs half the bandwidth, so the whole-line store
// layout above is what makes it pay.)
//
// Long selections are cut into several launches of at most ZR_LAUNCH_BYTES
// of traffic each.  Within one launch the eight XCDs take every eighth tile in
// dispatch order but run at different speeds (measured: the odd XCDs 2-7%
// slower than the even ones; the reduce kernels weight their shares for it,
// skew_tile below), so in a long launch they drift apart -- by 140k tiles, 290 MB of
// every stream, late in a 10 ms launch -- the addresses in flight spread over
// a widening window, and the launch ends on the slowest XCD.  A kernel
// boundary brings them back together.  Measured on the fused fp32 8-replica
// step over a 1.0e9-element share: 5.88 TB/s as one launch, 6.06 TB/s in
// launches of 2 GiB (interleaved in one process).  Every kernel therefore
// takes a tile range [tile_base, tile_end) in its arguments.
//
// Arithmetic follows the method's definition exactly: each replica's value is
// divided by D first, the quotients are summed in rank order 0..R-1 starting
// from the rank-0 quotient, every operation is a separate fp32 operation
// (this file is compiled with -ffp-contract=off; subnormals are kept).  When D
// is a power of two, x * (1/D) is the same correctly rounded number as x / D,
// so the multiply is used; otherwise a true IEEE division.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <set>
#include <string>
#include <type_traits>
#include <tuple>
#include <utility>
#include <vector>

#include "zr_internal.h"

using zr::fail;

// The no-allocation entry point's staging buffer: its launch tables (at most
// kScratchBytes, i.e. 6,552 segments) are written here by a staging kernel on
// the caller's stream, then read by the reduce kernel.  Each GPU holds its own
// copy for the life of the process.  Host code never uses this name as a
// device address (on the host it is a stand-in, not the array): it uses the
// per-device address from hipGetSymbolAddress (scratch_for below).
constexpr size_t kScratchBytes = 256 * 1024;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

// Launch-shape constants (compile-time; the defaults are the tuned values).
// The reduce kernels (reduce-scatter, fused reduce + Adam) give each lane one
// 4-element slot: 256 elements on one wave for fp32 replicas and for the
// bf16 reduce-scatter, 512 on two waves for the bf16 fused step
// (red_threads below).  The other kernels use workgroups of ZR_THREADS lanes.
#ifndef ZR_RED_THREADS_F32
#define ZR_RED_THREADS_F32 64
#endif
#ifndef ZR_RED_THREADS_BF16
#define ZR_RED_THREADS_BF16 128
#endif
#ifndef ZR_RED_THREADS_BF16_UNFUSED
#define ZR_RED_THREADS_BF16_UNFUSED 64
#endif
#ifndef ZR_THREADS
#define ZR_THREADS 128
#endif
// Workgroups per CU when a grid-stride loop is wanted; 0 = one tile per WG.
#ifndef ZR_GRID_PER_CU
#define ZR_GRID_PER_CU 0
#endif
// Non-temporal hints on the single-touch streams (measured: +7% on the fused
// step once every store instruction writes whole cache lines).
#ifndef ZR_NT_LOADS
#define ZR_NT_LOADS 1
#endif
#ifndef ZR_NT_STORES
#define ZR_NT_STORES 1
#endif
// Workgroups per CU that an uncapped reduce launch may hold at once (the
// launch reserves LDS it does not use so that no more fit: reduce_lds_bytes
// below).  Fewer streams in flight than the register limit allows measured
// faster for the shapes the table lists; every other shape, and grid-capped
// calls, keep the register-limited occupancy.  0 turns the table off.
#ifndef ZR_RED_WGS_CAP
#define ZR_RED_WGS_CAP 1
#endif
// Launch of kernel __VA_ARGS__ over `grid` workgroups of `block` lanes on
// `stream` with the argument block `args`, reserving `lds` bytes of dynamic
// LDS per workgroup (a CPU build of this file for bounds checking
// substitutes its own).
#ifndef ZR_KERNEL_LAUNCH_LDS
#define ZR_KERNEL_LAUNCH_LDS(grid, block, lds, stream, args, ...) \
  __VA_ARGS__<<<(grid), (block), (lds), (stream)>>>(args)
#endif
#define ZR_KERNEL_LAUNCH(grid, block, stream, args, ...) \
  ZR_KERNEL_LAUNCH_LDS(grid, block, 0, stream, args, __VA_ARGS__)
constexpr int kThreads = ZR_THREADS;
constexpr int VE = 4;  // elements per lane slot
// Cache-line size the reduce kernels align replica tiles to, and the largest
// tile shift that alignment can need (a bf16 line minus one element).
constexpr int64_t kLineBytes = 128;
constexpr int64_t kMaxLineShift = kLineBytes / 2 - 1;
// Lanes of a reduce-kernel workgroup and elements of its tile, by replica
// element type and kernel.  A/B-measured, calls interleaved in one process:
// fp32 fused on a 1.0e9-element share 6.15 TB/s with 256-element one-wave
// tiles against 6.03 with 512-element two-wave tiles, on the 5.4e8-element
// MoE expert share 6.13 against 6.00; bf16 fused on a 15.5M-element share
// 5.94 against 6.00, the bf16 reduce-scatter on the same share 6.04 against
// 5.96.
template <typename InT, bool kFused>
__host__ __device__ constexpr int red_threads() {
  return sizeof(InT) == 4 ? ZR_RED_THREADS_F32
                          : (kFused ? ZR_RED_THREADS_BF16 : ZR_RED_THREADS_BF16_UNFUSED);
}
template <typename InT, bool kFused>
__host__ __device__ constexpr int64_t red_tile() {
  return int64_t(red_threads<InT, kFused>()) * VE;
}
constexpr int kIpgMaxSegs = 48;
// Slots per lane in the IPG kernel (its tiles are kIpgSlots lane slots of
// every thread).
#ifndef ZR_IPG_SLOTS
#define ZR_IPG_SLOTS 2
#endif
constexpr int kIpgSlots = ZR_IPG_SLOTS;
constexpr int64_t kIpgTileElems = int64_t(kIpgSlots) * kThreads * VE;
// Slots per lane of the standalone Adam, segmented copy and ring-step kernels,
// and the all-gather's tile size in units of 512 fp32 elements.  Each
// of these kernels covers kXSlots * kThreads * VE elements per tile.  Values
// from A/B measurement: two slots pay for the light streams (copy +10%, ring
// reduce-scatter step +2%, all-gather +2.5%, IPG +2.6%); Adam (-4%) and the
// ring all-gather step (-1%) keep one.
#ifndef ZR_ADAM_SLOTS
#define ZR_ADAM_SLOTS 1
#endif
#ifndef ZR_COPY_SLOTS
#define ZR_COPY_SLOTS 2
#endif
#ifndef ZR_RING_SLOTS
#define ZR_RING_SLOTS 2
#endif
#ifndef ZR_RING_AG_SLOTS
#define ZR_RING_AG_SLOTS 1
#endif
#ifndef ZR_GATHER_SLOTS
#define ZR_GATHER_SLOTS 2
#endif
constexpr int kAdamSlots = ZR_ADAM_SLOTS;
constexpr int64_t kAdamTileElems = int64_t(kAdamSlots) * kThreads * VE;
constexpr int kCopySlots = ZR_COPY_SLOTS;
constexpr int64_t kCopyTileElems = int64_t(kCopySlots) * kThreads * VE;
constexpr int kRingSlots = ZR_RING_SLOTS;
constexpr int64_t kRingTileElems = int64_t(kRingSlots) * kThreads * VE;
constexpr int kRingAgSlots = ZR_RING_AG_SLOTS;
constexpr int64_t kRingAgTileElems = int64_t(kRingAgSlots) * kThreads * VE;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// Alignment a vector access may assume.  The kernels' dword-aligned variants
// (reduce, IPG, Adam, copy, ring steps, all-gather) access two- and
// four-dword vectors at merely dword-aligned addresses, which global loads
// and stores of this part accept.  Each variant is a separate instantiation
// that the host launches only when some segment has no phase at which every
// stream is slot-aligned, so the common instantiations carry none of its
// code.  The alignment travels as a template value (kDW), not as an aligned()
// typedef: template arguments are canonical types, so a typedef's reduced
// alignment would be lost inside the access helpers.
constexpr int kDW = 4;

// ------------------------------------------------------------ device helpers

// Every buffer the library touches is device (global) memory.  Addressing it
// through global-address-space pointers lets the compiler use global_load /
// global_store with a uniform 64-bit base and a 32-bit lane offset instead of
// flat instructions with a 64-bit address per lane.
#ifndef ZR_GLOBAL
#define ZR_GLOBAL __attribute__((address_space(1)))
#endif
template <typename T>
__device__ __forceinline__ const ZR_GLOBAL T* gptr(const void* p) {
  return (const ZR_GLOBAL T*)(p);
}
template <typename T>
__device__ __forceinline__ ZR_GLOBAL T* gptr(void* p) {
  return (ZR_GLOBAL T*)(p);
}

// A access (load or store) of T that may assume A-byte alignment (A = 0: T's
// natural alignment).
template <typename T, int A = 0>
__device__ __forceinline__ T ld_global(const ZR_GLOBAL T* p) {
  typedef T __attribute__((aligned(A ? A : alignof(T)))) TA;
  const ZR_GLOBAL TA* q = reinterpret_cast<const ZR_GLOBAL TA*>(p);
#if ZR_NT_LOADS
  return __builtin_nontemporal_load(q);
#else
  return *q;
#endif
}
template <typename T, int A = 0>
__device__ __forceinline__ void st_global(ZR_GLOBAL T* p, T v) {
  typedef T __attribute__((aligned(A ? A : alignof(T)))) TA;
  ZR_GLOBAL TA* q = reinterpret_cast<ZR_GLOBAL TA*>(p);
#if ZR_NT_STORES
  __builtin_nontemporal_store(v, q);
#else
  *q = v;
#endif
}
template <typename T, int A = 0>
__device__ __forceinline__ T ld_stream(const void* p) {
  return ld_global<T, A>(gptr<T>(p));
}
template <typename T, int A = 0>
__device__ __forceinline__ void st_stream(void* p, T v) {
  st_global<T, A>(gptr<T>(p), v);
}

// Slot loads/stores relative to a per-tile stream base (uniform across the
// workgroup) at a per-lane byte offset.
template <typename V, int A = 0>
__device__ __forceinline__ V ld_tile(uint64_t base, uint32_t off) {
  const ZR_GLOBAL char* b = gptr<char>(reinterpret_cast<const void*>(base)) + off;
  return ld_global<V, A>(reinterpret_cast<const ZR_GLOBAL V*>(b));
}
template <typename V, int A = 0>
__device__ __forceinline__ void st_tile(uint64_t base, uint32_t off, V v) {
  ZR_GLOBAL char* b = gptr<char>(reinterpret_cast<void*>(base)) + off;
  st_global<V, A>(reinterpret_cast<ZR_GLOBAL V*>(b), v);
}

// Four bf16 values that start 2 bytes into a dword (an odd element offset):
// read the dwords that hold them (bytes -2 .. +10 of the slot, so one value
// either side) and shift each pair down by 16 bits.  The caller keeps those
// two extra values inside the segment.
__device__ __forceinline__ u32x2 ld_bf16_odd(uint64_t base, uint32_t off) {
  const u32x2 lo = ld_tile<u32x2, kDW>(base - 2, off);
  const uint32_t hi = ld_tile<uint32_t>(base - 2, off + 8);
  return u32x2{__builtin_amdgcn_alignbit(lo[1], lo[0], 16),
                __builtin_amdgcn_alignbit(hi, lo[1], 16)};
}

// The same for a 16-byte slot of eight bf16 values (the all-gather's slot).
__device__ __forceinline__ u32x4 ld_bf16x8_odd(uint64_t base, uint32_t off) {
  const u32x4 lo = ld_tile<u32x4, kDW>(base - 2, off);
  const uint32_t hi = ld_tile<uint32_t>(base - 2, off + 16);
  return u32x4{__builtin_amdgcn_alignbit(lo[1], lo[0], 16),
                __builtin_amdgcn_alignbit(lo[2], lo[1], 16),
                __builtin_amdgcn_alignbit(lo[3], lo[2], 16),
                __builtin_amdgcn_alignbit(hi, lo[3], 16)};
}

__host__ __device__ __forceinline__ bool aligned(uint64_t addr, uint64_t bytes) {
  return (addr & (bytes - 1)) == 0;
}

// Input element types: bf16 as its 16-bit pattern, or fp32.  Vec holds one
// slot (four elements).
template <typename InT> struct In;
template <> struct In<uint16_t> {
  using Vec = u32x2;
  __device__ static __forceinline__ float widen(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
  }
  template <typename V>
  __device__ static __forceinline__ void unpack(V w, float* x) {
    x[0] = __uint_as_float(w[0] << 16);
    x[1] = __uint_as_float(w[0] & 0xffff0000u);
    x[2] = __uint_as_float(w[1] << 16);
    x[3] = __uint_as_float(w[1] & 0xffff0000u);
  }
};
template <> struct In<float> {
  using Vec = u32x4;
  __device__ static __forceinline__ float widen(float v) { return v; }
  template <typename V>
  __device__ static __forceinline__ void unpack(V w, float* x) {
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

// Adam on one slot held in registers; writes master, m, v and the optional
// bf16 param / reduced-gradient copies of that slot.  Each destination is a
// per-tile stream base plus the slot's byte offset (o4 for fp32 streams, o2
// for the bf16 param); a zero base means "not written".
template <int A = 0>
__device__ __forceinline__ void adam_slot(const AdamConsts& k, const float* g,
                                          f32x4 th, f32x4 mm, f32x4 vv,
                                          uint64_t master, uint64_t m, uint64_t v,
                                          uint64_t pbf16, uint64_t gout,
                                          uint32_t o4, uint32_t o2) {
  float t[4], a[4], b[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    t[e] = th[e];
    a[e] = mm[e];
    b[e] = vv[e];
    adam_elem(k, g[e], t[e], a[e], b[e]);
  }
  st_tile<f32x4, A>(master, o4, f32x4{t[0], t[1], t[2], t[3]});
  st_tile<f32x4, A>(m, o4, f32x4{a[0], a[1], a[2], a[3]});
  st_tile<f32x4, A>(v, o4, f32x4{b[0], b[1], b[2], b[3]});
  if (gout) st_tile<f32x4, A>(gout, o4, f32x4{g[0], g[1], g[2], g[3]});
  if (pbf16)
    st_tile<u32x2, A>(pbf16, o2, u32x2{bf16_rne(t[0]) | (bf16_rne(t[1]) << 16),
                                    bf16_rne(t[2]) | (bf16_rne(t[3]) << 16)});
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

// XCD-weighted tile order.  The dispatcher deals a launch's workgroups to
// the 8 XCDs in turn (workgroup b runs on XCD b % 8), and each XCD then works
// through its share at its own pace; measured on MI355X with a probe that
// records each workgroup's XCD and start time, the odd XCDs stream 2-7%
// slower than the even ones on the fused step's access pattern, so with
// equal shares the even XCDs idle at the end of every launch while the odd
// ones finish.  In every round of ZR_XCD_SKEW x 8 workgroups the last
// round's odd-slot workgroups take no tile, which gives the odd XCDs
// (K-1)/K of the even XCDs' tiles while every XCD still walks the tiles in
// address order.  0 = equal shares.  A/B-measured, calls interleaved in one
// process on two machines, K = 32 against equal shares: 8 fp32 replicas on
// the 1.0e9-element share +0.3-0.7%, 8 bf16 replicas fused on the
// 15.5M-element share +0.75-1.0%, the 8-replica bf16 reduce-scatter
// +1.9-2.4%.  With the workgroups-per-CU table in place, 2 replicas gain
// too (two machines): the fp32 MoE expert share fused +2.7-3.9%, its
// reduce-scatter +7.1-7.5%, and the same share's range calls as buckets
// complete +1.9-2.0% (reduce-scatter) and +2.1% (fused).  (Before that
// table, equal shares had measured 1.3% faster for the fused 2-replica
// call.)  Selections of at least ZR_XCD_SKEW_MIN_WORLD replicas take the
// weighted order.
#ifndef ZR_XCD_SKEW
#define ZR_XCD_SKEW 32
#endif
#ifndef ZR_XCD_SKEW_MIN_WORLD
#define ZR_XCD_SKEW_MIN_WORLD 2
#endif
constexpr int kXcdSkew = ZR_XCD_SKEW;
// Tile offset (within the launch) of workgroup b, or -1 for no tile.
__host__ __device__ inline int64_t skew_tile(uint32_t b) {
  constexpr uint32_t per = 8u * (kXcdSkew > 0 ? kXcdSkew : 1), tiles_per = per - 4;
  const uint32_t sr = b / per, rem = b % per, q = rem >> 3, x = rem & 7;
  const int64_t base = static_cast<int64_t>(sr) * tiles_per;
  if (q + 1 < static_cast<uint32_t>(kXcdSkew)) return base + q * 8 + x;
  if (x & 1) return -1;
  return base + (kXcdSkew - 1) * 8 + (x >> 1);
}
// Workgroups a launch of n tiles needs in that order: up to and including
// the one that holds tile n - 1 (so n <= 8 (K - 1) tiles take n workgroups).
inline int64_t skew_grid(int64_t n) {
  constexpr int64_t K = kXcdSkew > 0 ? kXcdSkew : 1, per = 8 * K, tiles_per = per - 4;
  if (n <= 1) return 1;
  const int64_t full = (n - 1) / tiles_per, r = (n - 1) % tiles_per;
  return full * per + (r < (K - 1) * 8 ? r : (K - 1) * 8 + 2 * (r - (K - 1) * 8)) + 1;
}

struct RedArgs {
  uint64_t in[ZR_MAX_WORLD];   // replica r's flat element f: in[r] + f*sizeof
  uint64_t out[ZR_MAX_WORLD];  // reduce mode: partition d's element j: out[d] + 4j
  const Seg* segs;
  int64_t tile_base;  // this launch's tiles: [tile_base, tile_end)
  int64_t tile_end;
  int32_t nseg;
  int32_t R;
  float divisor;
  float inv_divisor;
  int32_t skew;  // 1: one tile per workgroup in the XCD-weighted order (skew_tile)
  // fused mode: the state buffers.  Partition d's element j sits at index
  // d*state_stride + j (state_stride 0: the buffers hold one partition).
  int64_t state_stride;
  float* master;
  float* m;
  float* v;
  uint16_t* pbf16;
  float* gout;
  AdamConsts ac;
};

// Segment tables of the no-allocation entry point are staged in a
// file-scope device array (`scratch`, below) instead of memory the library
// allocates.  A staging launch copies up to kStageSegs segments from its
// kernel arguments into the array, one segment per lane.
constexpr int kStageSegs = 64;
struct StageArgs {
  Seg seg[kStageSegs];
  Seg* out;  // scratch address of the first segment this launch writes
  int32_t n;
};
__global__ __launch_bounds__(kStageSegs) void stage_segs_kernel(const StageArgs a) {
  const int i = static_cast<int>(threadIdx.x);
  if (i < a.n) a.out[i] = a.seg[i];
}

template <bool kDiv>
__device__ __forceinline__ float predivide(const RedArgs& a, float x) {
  if constexpr (kDiv) return x / a.divisor;
  else return x * a.inv_divisor;
}

// Rank-ordered pre-divided sum of one slot from its loaded replica vectors.
template <typename InT, int R, bool kDiv, typename V>
__device__ __forceinline__ void reduce_slot(const RedArgs& a, const V* w, float* acc) {
  float x[4];
  In<InT>::unpack(w[0], x);
#pragma unroll
  for (int e = 0; e < 4; ++e) acc[e] = (R == 1) ? x[e] : predivide<kDiv>(a, x[e]);
#pragma unroll
  for (int r = 1; r < R; ++r) {
    In<InT>::unpack(w[r], x);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = acc[e] + predivide<kDiv>(a, x[e]);
  }
}

// Same for a run-time replica count (loads issued inside the rank loop).
// kOdd: replicas whose bit is set in odd_mask are read with ld_bf16_odd.
template <typename InT, bool kDiv, typename Vec, bool kOdd = false, int A = 0>
__device__ __forceinline__ void reduce_slot_rt(const RedArgs& a, int rr, int64_t f,
                                               float* acc, uint64_t odd_mask = 0) {
  const uint64_t off = static_cast<uint64_t>(f) * sizeof(InT);
  auto load = [&](int r) -> Vec {
    if constexpr (kOdd) {
      if ((odd_mask >> r) & 1u) return ld_bf16_odd(a.in[r] + off, 0);
    }
    return ld_stream<Vec, A>(reinterpret_cast<const void*>(a.in[r] + off));
  };
  float x[4];
  In<InT>::unpack(load(0), x);
#pragma unroll
  for (int e = 0; e < 4; ++e) acc[e] = (rr == 1) ? x[e] : predivide<kDiv>(a, x[e]);
  for (int r = 1; r < rr; ++r) {
    In<InT>::unpack(load(r), x);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = acc[e] + predivide<kDiv>(a, x[e]);
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

// Segment tables in device memory are read-only while a kernel runs and
// every lane of a workgroup reads the same entry, so the kernels read them
// through the constant address space: scalar loads through the scalar data
// cache, instead of vector loads that each wait out a full memory round trip
// under the streams' load (a workgroup makes log2(segments) + 1 dependent
// table reads before its first stream load).  The tables are written before
// the launch (host copy or a staging kernel's vector stores); caches are
// invalidated at kernel start.
#ifndef ZR_CONST
#define ZR_CONST __attribute__((address_space(4)))
#endif
__device__ __forceinline__ const ZR_CONST Seg* cseg(const Seg* p) {
  return (const ZR_CONST Seg*)(p);
}

// A value every lane of the wave holds, moved to a scalar register.
// Broadcasting the segment fields tells the compiler they are uniform, so
// stream bases stay in scalar registers and the slot accesses take a scalar
// base plus a 32-bit lane offset.
__device__ __forceinline__ int64_t uniform64(int64_t x) {
  const uint64_t u = static_cast<uint64_t>(x);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}
__device__ __forceinline__ int32_t uniform32(int32_t x) {
  return static_cast<int32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x)));
}
__device__ __forceinline__ Seg load_seg(const Seg* p) {
  const ZR_CONST Seg* c = cseg(p);
  return Seg{uniform64(c->flat), uniform64(c->part), uniform64(c->numel),
             uniform64(c->tile0), uniform32(c->dst), uniform32(c->pad)};
}

// Tile -> segment for a segment array passed in the kernel arguments
// (ascending first-tile indices, segs[0].tile0 == 0): a binary search, so a
// workgroup waits on at most log2(nseg) dependent scalar loads before its
// first stream load.
template <typename S>
__device__ __forceinline__ int find_arg_seg(const S* segs, int nseg, int64_t t) {
  int lo = 0, hi = nseg - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (segs[mid].tile0 <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Tile -> segment by binary search over the segments' first-tile indices.
__device__ __forceinline__ int find_seg(const Seg* segs, int nseg, int64_t t) {
  const ZR_CONST Seg* cs = cseg(segs);
  int lo = 0, hi = nseg - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (uniform64(cs[mid].tile0) <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Optional occupancy target for the reduce kernels (waves per SIMD, 0 = the
// compiler's choice).
#ifndef ZR_WAVES_PER_EU
#define ZR_WAVES_PER_EU 0
#endif
#if ZR_WAVES_PER_EU > 0
#define ZR_OCCUPANCY __attribute__((amdgpu_waves_per_eu(ZR_WAVES_PER_EU, 8)))
#else
#define ZR_OCCUPANCY
#endif

// kDword: also accept tile phases at which every stream is only
// dword-aligned (vector types with 4-byte alignment).  The host launches that
// variant only for selections with a segment at which no phase is
// slot-aligned, so the common instantiations carry none of its code.
template <typename InT, int R, bool kDiv, bool kFused, bool kDword>
__global__ __launch_bounds__((red_threads<InT, kFused>())) ZR_OCCUPANCY void reduce_kernel(
    const RedArgs a) {
  using Vec = typename In<InT>::Vec;
  constexpr int A = kDword ? kDW : 0;  // alignment the slot accesses may assume
  constexpr bool kOddBf16 = kDword && std::is_same_v<InT, uint16_t>;
  constexpr int kRL = R > 0 ? R : 1;  // replica vectors held per slot
  constexpr int kTH = red_threads<InT, kFused>();
  constexpr int64_t kTile = red_tile<InT, kFused>();
  const int rr = R > 0 ? R : a.R;

  int64_t t = a.tile_base + blockIdx.x, tstep = gridDim.x;
  if constexpr (kXcdSkew > 0) {
    if (a.skew) {
      const int64_t j = skew_tile(blockIdx.x);
      t = j < 0 ? a.tile_end : a.tile_base + j;
      tstep = a.tile_end;  // one tile per workgroup
    }
  }
  for (; t < a.tile_end; t += tstep) {
    const Seg sg = load_seg(a.segs + find_seg(a.segs, a.nseg, t));
    const int64_t lt = t - sg.tile0;
    // First element of the segment in the output or state buffers.
    const int64_t spart =
        kFused ? sg.part + static_cast<int64_t>(sg.dst) * a.state_stride : sg.part;

    // Every stream is slot-aligned at segment offset j (VE elements of 4 or
    // 2 bytes land on one 16- or 8-byte access).
    auto slot_aligned = [&](int64_t j) {
      bool ok = true;
      if (!sg.pad)
        for (int r = 0; r < rr; ++r)
          ok = ok && aligned(a.in[r] + static_cast<uint64_t>(sg.flat + j) * sizeof(InT),
                             VE * sizeof(InT));
      const uint64_t p4 = static_cast<uint64_t>(spart + j) * 4;
      if constexpr (kFused) {
        ok = ok && aligned(reinterpret_cast<uint64_t>(a.master) + p4, 16) &&
             aligned(reinterpret_cast<uint64_t>(a.m) + p4, 16) &&
             aligned(reinterpret_cast<uint64_t>(a.v) + p4, 16);
        if (a.pbf16)
          ok = ok && aligned(reinterpret_cast<uint64_t>(a.pbf16) +
                                 static_cast<uint64_t>(spart + j) * 2, 8);
        if (a.gout) ok = ok && aligned(reinterpret_cast<uint64_t>(a.gout) + p4, 16);
      } else {
        ok = ok && aligned(a.out[sg.dst] + p4, 16);
      }
      return ok;
    };
    // Tile phase.  Tiles start at segment offsets congruent to ph modulo
    // `period` elements, shifted down by `shift` so the first tile begins at
    // or before offset 0.  Preferred: the phase that puts replica 0's tiles
    // on whole 128-byte lines (the replicas are most of the bytes read; a
    // tile boundary inside a line makes two workgroups fetch that line).
    // Otherwise the first phase below VE at which every stream is
    // slot-aligned; if there is none the segment goes element by element.
    int64_t ph = -1, period = VE;
    // kOddBf16 variant only: replicas read with ld_bf16_odd (bit r = replica r).
    uint64_t odd_mask = 0;
    if (!sg.pad) {
      constexpr int64_t kLineElems = kLineBytes / sizeof(InT);
      const uint64_t b0 = (a.in[0] + static_cast<uint64_t>(sg.flat) * sizeof(InT)) % kLineBytes;
      const int64_t cand = static_cast<int64_t>((kLineBytes - b0) % kLineBytes / sizeof(InT));
      if (cand < sg.numel && slot_aligned(cand)) {
        ph = cand;
        period = kLineElems;
      }
    }
    for (int64_t j = 0; j < VE && ph < 0; ++j)
      if (slot_aligned(j)) ph = j;
    if constexpr (kDword) {
      // Every stream dword-aligned at j; with stores16 the fp32 state and
      // output streams also 16-byte aligned (whole-line stores), preferred.
      auto dword_aligned = [&](int64_t j, bool stores16, bool reps = true) {
        const uint64_t st_al = stores16 ? 16 : 4;
        bool ok = true;
        if (!sg.pad && reps)
          for (int r = 0; r < rr; ++r)
            ok = ok && aligned(a.in[r] + static_cast<uint64_t>(sg.flat + j) * sizeof(InT), 4);
        const uint64_t p4 = static_cast<uint64_t>(spart + j) * 4;
        if constexpr (kFused) {
          ok = ok && aligned(reinterpret_cast<uint64_t>(a.master) + p4, st_al) &&
               aligned(reinterpret_cast<uint64_t>(a.m) + p4, st_al) &&
               aligned(reinterpret_cast<uint64_t>(a.v) + p4, st_al);
          if (a.pbf16)
            ok = ok && aligned(reinterpret_cast<uint64_t>(a.pbf16) +
                                   static_cast<uint64_t>(spart + j) * 2, 4);
          if (a.gout) ok = ok && aligned(reinterpret_cast<uint64_t>(a.gout) + p4, st_al);
        } else {
          ok = ok && aligned(a.out[sg.dst] + p4, st_al);
        }
        return ok;
      };
      // Preference: whole-line (16-byte-aligned) fp32 stores first, then
      // plain replica reads.  bf16 replicas an odd number of elements off
      // the other streams are read with ld_bf16_odd (kOddBf16 variants).
      for (int64_t j = 0; j < VE && ph < 0; ++j)
        if (dword_aligned(j, true)) ph = j;
      if constexpr (kOddBf16)
        for (int64_t j = 0; j < VE && ph < 0; ++j)
          if (dword_aligned(j, true, false)) ph = j;
      for (int64_t j = 0; j < VE && ph < 0; ++j)
        if (dword_aligned(j, false)) ph = j;
      if constexpr (kOddBf16) {
        for (int64_t j = 0; j < VE && ph < 0; ++j)
          if (dword_aligned(j, false, false)) ph = j;
        if (ph >= 0 && !sg.pad)
          for (int r = 0; r < rr; ++r)
            if ((a.in[r] + static_cast<uint64_t>(sg.flat + ph) * sizeof(InT)) & 2)
              odd_mask |= uint64_t(1) << r;
      }
    }
    const bool vec = ph >= 0;
    const int64_t shift = vec ? (period - ph) % period : 0;
    const int64_t rel0 = lt * kTile - shift;

    // Per-tile stream bases: element rel0 of the segment in every stream.
    // spart + rel0 (and sg.flat + rel0) can be negative for a segment's
    // first tile; the byte offsets are formed by multiplying the signed
    // element offset, so they wrap modulo 2^64 and every lane's address
    // (base + its non-negative slot offset) comes out exact.  Never derive
    // one from another by division.
    const uint64_t in_off = static_cast<uint64_t>(sg.flat + rel0) * sizeof(InT);
    const uint64_t p4 = static_cast<uint64_t>(spart + rel0) * 4;
    const uint64_t p2 = static_cast<uint64_t>(spart + rel0) * 2;
    uint64_t b_master = 0, b_m = 0, b_v = 0, b_pb = 0, b_go = 0, b_out = 0;
    if constexpr (kFused) {
      b_master = reinterpret_cast<uint64_t>(a.master) + p4;
      b_m = reinterpret_cast<uint64_t>(a.m) + p4;
      b_v = reinterpret_cast<uint64_t>(a.v) + p4;
      b_pb = a.pbf16 ? reinterpret_cast<uint64_t>(a.pbf16) + p2 : 0;
      b_go = a.gout ? reinterpret_cast<uint64_t>(a.gout) + p4 : 0;
    } else {
      b_out = a.out[sg.dst] + p4;
    }

    // Issue every load of the tile's slots first.
    constexpr int kSlots = 1;
    Vec w[kSlots][kRL];
    f32x4 s0[kSlots], s1[kSlots], s2[kSlots];
    bool full[kSlots];
#pragma unroll
    for (int u = 0; u < kSlots; ++u) {
      const int slot = u * kTH + static_cast<int>(threadIdx.x);
      const int64_t rel = rel0 + static_cast<int64_t>(slot) * VE;
      if constexpr (kOddBf16) {
        // ld_bf16_odd reads one value either side of the slot.
        const int64_t lo = odd_mask ? 1 : 0;
        full[u] = vec && rel >= lo && rel + VE + lo <= sg.numel;
      } else {
        full[u] = vec && rel >= 0 && rel + VE <= sg.numel;
      }
      if (full[u]) {
        if constexpr (R > 0) {
          if (!sg.pad) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
              if constexpr (kOddBf16) {
                if ((odd_mask >> r) & 1u)
                  w[u][r] = ld_bf16_odd(a.in[r] + in_off, slot * VE * sizeof(InT));
                else
                  w[u][r] = ld_tile<Vec, A>(a.in[r] + in_off, slot * VE * sizeof(InT));
              } else {
                w[u][r] = ld_tile<Vec, A>(a.in[r] + in_off, slot * VE * sizeof(InT));
              }
            }
          }
        }
        if constexpr (kFused) {
          s0[u] = ld_tile<f32x4, A>(b_master, slot * 16);
          s1[u] = ld_tile<f32x4, A>(b_m, slot * 16);
          s2[u] = ld_tile<f32x4, A>(b_v, slot * 16);
        }
      }
    }

#pragma unroll
    for (int u = 0; u < kSlots; ++u) {
      const int slot = u * kTH + static_cast<int>(threadIdx.x);
      const int64_t rel = rel0 + static_cast<int64_t>(slot) * VE;
      if (full[u]) {
        float g[4];
        if (sg.pad) {
#pragma unroll
          for (int e = 0; e < 4; ++e) g[e] = 0.0f;
        } else if constexpr (R > 0) {
          reduce_slot<InT, R, kDiv>(a, w[u], g);
        } else {
          reduce_slot_rt<InT, kDiv, Vec, kOddBf16, A>(a, rr, sg.flat + rel, g, odd_mask);
        }
        if constexpr (!kFused) {
          st_tile<f32x4, A>(b_out, slot * 16, f32x4{g[0], g[1], g[2], g[3]});
        } else {
          adam_slot<A>(a.ac, g, s0[u], s1[u], s2[u], b_master, b_m, b_v, b_pb, b_go,
                    slot * 16, slot * 8);
        }
      } else if (rel < sg.numel && rel + VE > 0) {
        const int64_t e0 = rel < 0 ? 0 : rel;
        const int64_t e1 = rel + VE < sg.numel ? rel + VE : sg.numel;
        for (int64_t e = e0; e < e1; ++e) {
          const float g = sg.pad ? 0.0f : reduce_one<InT, R, kDiv>(a, rr, sg.flat + e);
          const int64_t j = spart + e;
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
  int64_t tile_base;  // this launch's tiles: [tile_base, tile_end)
  int64_t tile_end;
  AdamConsts ac;
};

// Contiguous partition; kVec: every pointer 16-byte aligned (bf16 8-byte),
// or with kDword only dword-aligned (vector types with 4-byte alignment; the
// host launches that variant when the pointers are not all slot-aligned).
template <bool kVec, bool kDword>
__global__ __launch_bounds__(kThreads) void adam_kernel(const AdamArgs a) {
  constexpr int A = kDword ? kDW : 0;  // alignment the slot accesses may assume
  for (int64_t t = a.tile_base + blockIdx.x; t < a.tile_end; t += gridDim.x) {
    const uint64_t t4 = static_cast<uint64_t>(t) * kAdamTileElems * 4;
    const uint64_t b_g = reinterpret_cast<uint64_t>(a.grad) + t4;
    const uint64_t b_master = reinterpret_cast<uint64_t>(a.master) + t4;
    const uint64_t b_m = reinterpret_cast<uint64_t>(a.m) + t4;
    const uint64_t b_v = reinterpret_cast<uint64_t>(a.v) + t4;
    const uint64_t b_pb = a.pbf16 ? reinterpret_cast<uint64_t>(a.pbf16) + t4 / 2 : 0;
    f32x4 g[kAdamSlots], th[kAdamSlots], mm[kAdamSlots], vv[kAdamSlots];
    bool full[kAdamSlots];
#pragma unroll
    for (int u = 0; u < kAdamSlots; ++u) {
      const int slot = u * kThreads + static_cast<int>(threadIdx.x);
      const int64_t j = t * kAdamTileElems + static_cast<int64_t>(slot) * VE;
      full[u] = kVec && j + VE <= a.n;
      if (full[u]) {
        g[u] = ld_tile<f32x4, A>(b_g, slot * 16);
        th[u] = ld_tile<f32x4, A>(b_master, slot * 16);
        mm[u] = ld_tile<f32x4, A>(b_m, slot * 16);
        vv[u] = ld_tile<f32x4, A>(b_v, slot * 16);
      }
    }
#pragma unroll
    for (int u = 0; u < kAdamSlots; ++u) {
      const int slot = u * kThreads + static_cast<int>(threadIdx.x);
      const int64_t j = t * kAdamTileElems + static_cast<int64_t>(slot) * VE;
      if (full[u]) {
        const float gg[4] = {g[u][0], g[u][1], g[u][2], g[u][3]};
        adam_slot<A>(a.ac, gg, th[u], mm[u], vv[u], b_master, b_m, b_v, b_pb, 0,
                          slot * 16, slot * 8);
      } else if (j < a.n) {
        const int64_t e1 = j + VE < a.n ? j + VE : a.n;
        for (int64_t e = j; e < e1; ++e) {
          float t1 = a.master[e], m1 = a.m[e], v1 = a.v[e];
          adam_elem(a.ac, a.grad[e], t1, m1, v1);
          a.master[e] = t1;
          a.m[e] = m1;
          a.v[e] = v1;
          if (a.pbf16) a.pbf16[e] = static_cast<uint16_t>(bf16_rne(t1));
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
  int64_t tile_base;  // this launch's tiles: [tile_base, tile_end)
  int64_t tile_end;
  float* main_grad;
  int32_t nseg;
};

// kDword: when no phase leaves both streams slot-aligned, take the phase
// that puts main_grad on 16 bytes (there always is one) and read the
// gradient dword-aligned -- or, for bf16 an odd number of elements off, with
// ld_bf16_odd.  The host launches that variant only for calls that need it.
// kFirst: the step's first micro-batch into a window the step would have
// zeroed: main_grad is not read, and each element becomes fl(+0 + widen(g)),
// the bits the add into a zeroed buffer gives (-0 becomes +0).
template <typename InT, bool kDword, bool kFirst>
__global__ __launch_bounds__(kThreads) void ipg_kernel(const IpgArgs a) {
  using Vec = typename In<InT>::Vec;
  constexpr int A = kDword ? kDW : 0;  // alignment the gradient reads may assume
  for (int64_t t = a.tile_base + blockIdx.x; t < a.tile_end; t += gridDim.x) {
    const IpgSeg sg = a.seg[find_arg_seg(a.seg, a.nseg, t)];
    const int64_t lt = t - sg.tile0;
    const uint64_t mg = reinterpret_cast<uint64_t>(a.main_grad);
    int j0 = -1;
    for (int j = 0; j < VE && j0 < 0; ++j)
      if (aligned(sg.src + j * sizeof(InT), VE * sizeof(InT)) &&
          aligned(mg + static_cast<uint64_t>(sg.dst + j) * 4, 16))
        j0 = j;
    bool odd = false;  // kDword only: bf16 gradient read with ld_bf16_odd
    if constexpr (kDword) {
      for (int j = 0; j < VE && j0 < 0; ++j)
        if (aligned(mg + static_cast<uint64_t>(sg.dst + j) * 4, 16)) j0 = j;
      if constexpr (std::is_same_v<InT, uint16_t>)
        odd = j0 >= 0 && ((sg.src + static_cast<uint64_t>(j0) * sizeof(InT)) & 2);
    }
    const bool vec = j0 >= 0;
    const int64_t rel0 = (j0 > 0 ? j0 - VE : 0) + lt * kIpgTileElems;
    Vec x[kIpgSlots];
    f32x4 cur[kIpgSlots];
    bool full[kIpgSlots];
#pragma unroll
    for (int u = 0; u < kIpgSlots; ++u) {
      const int64_t rel = rel0 + static_cast<int64_t>(u * kThreads + threadIdx.x) * VE;
      if constexpr (kDword) {
        // ld_bf16_odd reads one value either side of the slot.
        const int64_t lo = odd ? 1 : 0;
        full[u] = vec && rel >= lo && rel + VE + lo <= sg.numel;
      } else {
        full[u] = vec && rel >= 0 && rel + VE <= sg.numel;
      }
      if (full[u]) {
        if constexpr (kDword && std::is_same_v<InT, uint16_t>) {
          if (odd)
            x[u] = ld_bf16_odd(sg.src + rel * sizeof(InT), 0);
          else
            x[u] = ld_stream<Vec, A>(reinterpret_cast<const void*>(sg.src + rel * sizeof(InT)));
        } else {
          x[u] = ld_stream<Vec, A>(reinterpret_cast<const void*>(sg.src + rel * sizeof(InT)));
        }
        if constexpr (kFirst)
          cur[u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        else
          cur[u] = ld_stream<f32x4>(a.main_grad + sg.dst + rel);
      }
    }
#pragma unroll
    for (int u = 0; u < kIpgSlots; ++u) {
      const int64_t rel = rel0 + static_cast<int64_t>(u * kThreads + threadIdx.x) * VE;
      if (full[u]) {
        float g[4];
        In<InT>::unpack(x[u], g);
        st_stream<f32x4>(a.main_grad + sg.dst + rel,
                         f32x4{cur[u][0] + g[0], cur[u][1] + g[1], cur[u][2] + g[2],
                               cur[u][3] + g[3]});
      } else if (rel < sg.numel && rel + VE > 0) {
        const int64_t e0 = rel < 0 ? 0 : rel;
        const int64_t e1 = rel + VE < sg.numel ? rel + VE : sg.numel;
        for (int64_t e = e0; e < e1; ++e) {
          const float v = In<InT>::widen(*reinterpret_cast<const InT*>(sg.src + e * sizeof(InT)));
          const float c = kFirst ? 0.0f : a.main_grad[sg.dst + e];
          a.main_grad[sg.dst + e] = c + v;
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
  int64_t tile_base;  // this launch's tiles: [tile_base, tile_end)
  int64_t tile_end;
  int32_t nseg;
};

// kDword: when no phase leaves source and destination both 16-byte aligned,
// take the destination's (whole-line stores) and read the source merely
// dword-aligned; the host launches that variant only for calls that need it.
template <bool kDword>
__global__ __launch_bounds__(kThreads) void copy_kernel(const CopyArgs a) {
  constexpr int A = kDword ? kDW : 0;  // alignment the source reads may assume
  for (int64_t t = a.tile_base + blockIdx.x; t < a.tile_end; t += gridDim.x) {
    const Seg sg = load_seg(a.segs + find_seg(a.segs, a.nseg, t));
    const int64_t lt = t - sg.tile0;
    const float* s = a.src + sg.flat;
    float* d = a.dst + sg.part;
    int j0 = -1;
    for (int j = 0; j < VE && j0 < 0; ++j)
      if (aligned(reinterpret_cast<uint64_t>(s + j), 16) &&
          aligned(reinterpret_cast<uint64_t>(d + j), 16))
        j0 = j;
    if constexpr (kDword)
      for (int j = 0; j < VE && j0 < 0; ++j)
        if (aligned(reinterpret_cast<uint64_t>(d + j), 16)) j0 = j;
    const bool vec = j0 >= 0;
    const int64_t rel0 = (j0 > 0 ? j0 - VE : 0) + lt * kCopyTileElems;
    f32x4 x[kCopySlots];
    bool full[kCopySlots];
#pragma unroll
    for (int u = 0; u < kCopySlots; ++u) {
      const int64_t rel = rel0 + static_cast<int64_t>(u * kThreads + threadIdx.x) * VE;
      full[u] = vec && rel >= 0 && rel + VE <= sg.numel;
      if (full[u]) x[u] = ld_stream<f32x4, A>(s + rel);
    }
#pragma unroll
    for (int u = 0; u < kCopySlots; ++u) {
      const int64_t rel = rel0 + static_cast<int64_t>(u * kThreads + threadIdx.x) * VE;
      if (full[u]) {
        st_stream<f32x4>(d + rel, x[u]);
      } else if (rel < sg.numel && rel + VE > 0) {
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
  int64_t tile_base;  // this launch's tiles: [tile_base, tile_end) of
  int64_t tile_end;   // tiles_per_rank * n
  int32_t n;
  int32_t step;
};

template <bool kDword>
__global__ __launch_bounds__(kThreads) void ring_kernel(const RingArgs a) {
  constexpr int A = kDword ? kDW : 0;  // alignment the source reads may assume
  for (int64_t t = a.tile_base + blockIdx.x; t < a.tile_end; t += gridDim.x) {
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
    if constexpr (kDword)   // the destination's phase; the source dword-aligned
      for (int j = 0; j < VE && j0 < 0; ++j)
        if (aligned(reinterpret_cast<uint64_t>(d + j), 16)) j0 = j;
    const bool vec = j0 >= 0;
    const int64_t rel0 = (j0 > 0 ? j0 - VE : 0) + lt * kRingTileElems;
    f32x4 x[kRingSlots];
    f32x4 y[kRingSlots];
    bool full[kRingSlots];
#pragma unroll
    for (int u = 0; u < kRingSlots; ++u) {
      const int64_t rel = rel0 + static_cast<int64_t>(u * kThreads + threadIdx.x) * VE;
      full[u] = vec && rel >= 0 && rel + VE <= a.chunk;
      if (full[u]) {
        x[u] = ld_stream<f32x4, A>(s + rel);
        y[u] = ld_stream<f32x4>(d + rel);
      }
    }
#pragma unroll
    for (int u = 0; u < kRingSlots; ++u) {
      const int64_t rel = rel0 + static_cast<int64_t>(u * kThreads + threadIdx.x) * VE;
      if (full[u]) {
        st_stream<f32x4>(d + rel, f32x4{y[u][0] + x[u][0], y[u][1] + x[u][1],
                                        y[u][2] + x[u][2], y[u][3] + x[u][3]});
      } else if (rel < a.chunk && rel + VE > 0) {
        const int64_t e0 = rel < 0 ? 0 : rel;
        const int64_t e1 = rel + VE < a.chunk ? rel + VE : a.chunk;
        for (int64_t e = e0; e < e1; ++e) d[e] = d[e] + s[e];
      }
    }
  }
}


// ------------------------------------------------------------- gather ---

constexpr int kXMaxSegs = ZR_MAX_WORLD;

struct XSeg {
  uint64_t src;   // address of the segment's first source element
  uint64_t dst;   // address of its first destination element
  int64_t numel;
  int64_t tile0;
};

struct XArgs {
  XSeg seg[kXMaxSegs];
  int64_t tile_base;  // this launch's tiles: [tile_base, tile_end)
  int64_t tile_end;
  int32_t nseg;
};

// Segmented copy driven by a table in the kernel arguments; T is uint16_t
// (bf16 patterns) or float.  Used by the parameter all-gather.  There is no
// fp32 stream to match, so a slot is one 16-byte vector of either type
// (8 bf16 or 4 fp32) and a tile holds kGatherTileBytes.
constexpr int64_t kGatherTileBytes = int64_t(kThreads) * VE * 4 * ZR_GATHER_SLOTS;
template <typename T>
__host__ __device__ constexpr int64_t gather_tile_elems() {
  return kGatherTileBytes / static_cast<int64_t>(sizeof(T));
}

// kDword: when no phase leaves a partition and the output both 16-byte
// aligned, take the output's (whole-line stores) and read the partition
// merely dword-aligned, or for bf16 an odd number of elements off with
// ld_bf16x8_odd; the host launches that variant only when needed.
template <typename T, bool kDword>
__global__ __launch_bounds__(kThreads) void gather_kernel(const XArgs a) {
  constexpr int A = kDword ? kDW : 0;  // alignment the partition reads may assume
  constexpr int ES = sizeof(T);
  constexpr int GV = 16 / ES;                          // elements per slot
  constexpr int64_t TE = gather_tile_elems<T>();       // elements per tile
  constexpr int GS = static_cast<int>(TE / (kThreads * GV));
  static_assert(GS >= 1 && TE == int64_t(GS) * kThreads * GV, "gather tile shape");
  for (int64_t t = a.tile_base + blockIdx.x; t < a.tile_end; t += gridDim.x) {
    const XSeg sg = a.seg[find_arg_seg(a.seg, a.nseg, t)];
    const int64_t lt = t - sg.tile0;
    int j0 = -1;
    for (int j = 0; j < GV && j0 < 0; ++j)
      if (aligned(sg.src + j * ES, 16) && aligned(sg.dst + j * ES, 16)) j0 = j;
    bool odd = false;  // kDword bf16 only: partition read with ld_bf16x8_odd
    if constexpr (kDword) {
      for (int j = 0; j < GV && j0 < 0; ++j)
        if (aligned(sg.src + j * ES, 4) && aligned(sg.dst + j * ES, 16)) j0 = j;
      if constexpr (ES == 2) {
        for (int j = 0; j < GV && j0 < 0; ++j)
          if (aligned(sg.dst + j * ES, 16)) j0 = j;
        odd = j0 >= 0 && ((sg.src + static_cast<uint64_t>(j0) * ES) & 2);
      }
    }
    const bool vec = j0 >= 0;
    const int64_t rel0 = (j0 > 0 ? j0 - GV : 0) + lt * TE;
    const uint64_t bs = sg.src + rel0 * ES, bd = sg.dst + rel0 * ES;
    u32x4 x[GS];
    bool full[GS];
#pragma unroll
    for (int u = 0; u < GS; ++u) {
      const int slot = u * kThreads + static_cast<int>(threadIdx.x);
      const int64_t rel = rel0 + static_cast<int64_t>(slot) * GV;
      if constexpr (kDword && ES == 2) {
        // ld_bf16x8_odd reads one value either side of the slot.
        const int64_t lo = odd ? 1 : 0;
        full[u] = vec && rel >= lo && rel + GV + lo <= sg.numel;
        if (full[u]) x[u] = odd ? ld_bf16x8_odd(bs, slot * 16) : ld_tile<u32x4, A>(bs, slot * 16);
      } else {
        full[u] = vec && rel >= 0 && rel + GV <= sg.numel;
        if (full[u]) x[u] = ld_tile<u32x4, A>(bs, slot * 16);
      }
    }
#pragma unroll
    for (int u = 0; u < GS; ++u) {
      const int slot = u * kThreads + static_cast<int>(threadIdx.x);
      const int64_t rel = rel0 + static_cast<int64_t>(slot) * GV;
      if (full[u]) {
        st_tile<u32x4>(bd, slot * 16, x[u]);
      } else if (rel < sg.numel && rel + GV > 0) {
        const int64_t e0 = rel < 0 ? 0 : rel;
        const int64_t e1 = rel + GV < sg.numel ? rel + GV : sg.numel;
        for (int64_t e = e0; e < e1; ++e)
          reinterpret_cast<T*>(sg.dst)[e] = reinterpret_cast<const T*>(sg.src)[e];
      }
    }
  }
}

// Ring all-gather step: rank k copies chunk (k - step - 1) mod n from rank
// k-1's buffer into its own.
template <bool kDword>
__global__ __launch_bounds__(kThreads) void ring_ag_kernel(const RingArgs a) {
  constexpr int A = kDword ? kDW : 0;  // alignment the source reads may assume
  for (int64_t t = a.tile_base + blockIdx.x; t < a.tile_end; t += gridDim.x) {
    const int k = static_cast<int>(t / a.tiles_per_rank);
    const int64_t lt = t - static_cast<int64_t>(k) * a.tiles_per_rank;
    int c = (k - a.step - 1) % a.n;
    if (c < 0) c += a.n;
    const int prev = (k == 0) ? a.n - 1 : k - 1;
    float* d = reinterpret_cast<float*>(a.buf[k]) + static_cast<int64_t>(c) * a.chunk;
    const float* s = reinterpret_cast<const float*>(a.buf[prev]) + static_cast<int64_t>(c) * a.chunk;
    int j0 = -1;
    for (int j = 0; j < VE && j0 < 0; ++j)
      if (aligned(reinterpret_cast<uint64_t>(s + j), 16) &&
          aligned(reinterpret_cast<uint64_t>(d + j), 16))
        j0 = j;
    if constexpr (kDword)   // the destination's phase; the source dword-aligned
      for (int j = 0; j < VE && j0 < 0; ++j)
        if (aligned(reinterpret_cast<uint64_t>(d + j), 16)) j0 = j;
    const bool vec = j0 >= 0;
    const int64_t rel0 = (j0 > 0 ? j0 - VE : 0) + lt * kRingAgTileElems;
    f32x4 x[kRingAgSlots];
    bool full[kRingAgSlots];
#pragma unroll
    for (int u = 0; u < kRingAgSlots; ++u) {
      const int64_t rel = rel0 + static_cast<int64_t>(u * kThreads + threadIdx.x) * VE;
      full[u] = vec && rel >= 0 && rel + VE <= a.chunk;
      if (full[u]) x[u] = ld_stream<f32x4, A>(s + rel);
    }
#pragma unroll
    for (int u = 0; u < kRingAgSlots; ++u) {
      const int64_t rel = rel0 + static_cast<int64_t>(u * kThreads + threadIdx.x) * VE;
      if (full[u]) {
        st_stream<f32x4>(d + rel, x[u]);
      } else if (rel < a.chunk && rel + VE > 0) {
        const int64_t e0 = rel < 0 ? 0 : rel;
        const int64_t e1 = rel + VE < a.chunk ? rel + VE : a.chunk;
        for (int64_t e = e0; e < e1; ++e) d[e] = s[e];
      }
    }
  }
}

// ================================================================= host ===

// Tiles of `tile` elements covering a segment of numel elements; + VE - 1: a
// segment whose start is not slot-aligned spans one more slot.
int64_t tiles_for(int64_t numel, int64_t tile) {
  return (numel + VE - 1 + tile - 1) / tile;
}
// Reduce-kernel segments may start their tiles up to kMaxLineShift elements
// early (line-aligned replica tiles); the count covers the largest shift.
int64_t reduce_tiles_for(int64_t numel, int64_t tile) {
  return (numel + kMaxLineShift + tile - 1) / tile;
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
// kind, group, first bucket, end bucket (exclusive), dst, tile elements
using HostKey = std::tuple<int, int32_t, int64_t, int64_t, int32_t, int64_t>;
using DevKey = std::tuple<int, int, int32_t, int64_t, int64_t, int32_t, int64_t>;  // device + HostKey

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

std::atomic<int> g_cu_count[64];  // per device, 0 until first queried

zr_status device_info(int* dev, int* cus) {
  hipError_t e = hipGetDevice(dev);
  if (e != hipSuccess) return fail(ZR_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (*dev < 0 || *dev >= 64) return fail(ZR_ERR_UNSUPPORTED, "device index above 63");
  int n = g_cu_count[*dev].load(std::memory_order_relaxed);
  if (n == 0) {
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, *dev);
    if (e != hipSuccess) return fail(ZR_ERR_HIP, std::string("hipDeviceGetAttribute: ") + hipGetErrorString(e));
    n = n > 0 ? n : 1;
    g_cu_count[*dev].store(n, std::memory_order_relaxed);
  }
  *cus = n;
  return ZR_OK;
}

std::atomic<int> g_lds_per_cu[64];  // per device, 0 until first queried

// Workgroups per CU for an uncapped reduce launch of R replicas (0 = as many
// as the registers allow), by replica type and kernel.  Each value is the
// best of an interleaved in-process sweep of the cap (launches alternating,
// 12 rounds, one session per line), listed with what no cap gives and with
// its neighbours, in TB/s:
//   fp32 fused, R = 8 (Llama-3-8B share): 8 -> 6.45; none 6.22, 10 6.42,
//     9 6.42, 7 6.29
//   bf16 fused, R = 8 (GPT-2 share, two-wave workgroups): 6 -> 6.11; none
//     6.07, 8 6.08, 7 6.10, 5 6.05
//   bf16 reduce-scatter, R = 8 (GPT-2, every partition): 20 -> 6.54; none
//     6.31, 24 6.39, 22 6.43, 18 6.55
//   fp32 reduce-scatter, R = 8 (MoE dense share): 12 -> 6.40; none 6.20,
//     14 6.27, 13 6.32, 11 6.14
//   fp32 fused, R = 2 (MoE expert share): 18 -> 6.24; none 6.11, 20 6.23,
//     17 6.25, 16 6.25; its range calls as buckets complete 18 -> 6.15
//     against 6.05; rechecked once 2 replicas took the XCD-weighted order:
//     18 -> 6.42, none 6.31, 20 6.42, 16 6.42
//   fp32 fused, R = 4 (one 125M-element share): 14 -> 6.38 and 6.42 (two
//     machines); none 6.20 and 6.22, 16 6.31 and 6.35, 13 6.43, 12 6.37 and
//     6.38, 11 6.13, 10 5.97
//   bf16 fused, R = 4 (one 62.5M-element share): 7 -> 6.34 and 6.38; none
//     6.06 and 6.04, 9 6.26, 8 6.33 and 6.34, 6 6.37 and 6.38, 5 6.29
//   fp32 fused, R = 16 (one 31.25M-element share): 6 -> 6.24 and 6.27; none
//     6.06 and 6.06, 9 6.14, 8 6.18, 7 6.22, 5 6.17 and 6.19, 4 5.60
//   fp32 reduce-scatter, R = 16 (same share): 7 -> 6.65; none 6.25 and
//     6.24, 9 6.49, 8 6.54 and 6.59, 6 6.59 and 6.62, 5 6.10
//   (At an eighth of those shares the four gain 0.8-1.9%; at a 32nd, where
//   launches are a few microseconds, they are within +-1% of none.)
// The fp32 reduce-scatter at R = 2 takes none: in equal XCD shares 28 per CU
// gave +7% on the whole MoE expert share but -4.5% on the same share's range
// calls as buckets complete; in the weighted order 28 gave -1.3% on the
// whole share and 24 -9%.  The reduce-scatter at R = 4 (fp32 +0.6%, bf16
// none) and the bf16 fused step at R = 16 (+0.7-1.0%) take none either;
// other replica counts were not measured and take no cap.
int reduce_wgs_per_cu(bool bf16, bool fused, int R) {
  if (!ZR_RED_WGS_CAP) return 0;
  if (R == 8) return fused ? (bf16 ? 6 : 8) : (bf16 ? 20 : 12);
  if (R == 4 && fused) return bf16 ? 7 : 14;
  if (R == 16 && !bf16) return fused ? 6 : 7;
  if (R == 2 && !bf16 && fused) return 18;
  return 0;
}

// Whether an uncapped reduce launch over `world` replicas hands its tiles out
// in the XCD-weighted order (skew_tile) rather than in equal shares.
bool xcd_weighted(int world) {
  return kXcdSkew > 0 && ZR_GRID_PER_CU == 0 && world >= ZR_XCD_SKEW_MIN_WORLD;
}

// Dynamic LDS a reduce launch reserves per workgroup: 0, or for an uncapped
// launch with a table entry k enough that at most k workgroups fit in a CU's
// LDS L.  The value 2L / (2k + 1) sits mid-way in the range
// (L / (k + 1), L / k] that admits exactly k, so rounding to the allocation
// granularity cannot tip it.
zr_status reduce_lds_bytes(int dev, bool fused, bool bf16, int world, bool capped,
                           unsigned* lds) {
  *lds = 0;
  const int k = reduce_wgs_per_cu(bf16, fused, world);
  if (capped || k <= 0) return ZR_OK;
  int n = g_lds_per_cu[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    const hipError_t e =
        hipDeviceGetAttribute(&n, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev);
    if (e != hipSuccess) return fail(ZR_ERR_HIP, std::string("hipDeviceGetAttribute: ") + hipGetErrorString(e));
    n = n > 0 ? n : -1;
    g_lds_per_cu[dev].store(n, std::memory_order_relaxed);
  }
  if (n > 0) *lds = static_cast<unsigned>(2 * static_cast<int64_t>(n) / (2 * k + 1));
  return ZR_OK;
}

// One workgroup per tile (ZR_GRID_PER_CU == 0), else a capped grid-stride
// grid.  Kernels loop over tiles either way, so any grid size is correct.
unsigned grid_for(int64_t tiles, int cus) {
  const int64_t cap = ZR_GRID_PER_CU > 0 ? static_cast<int64_t>(cus) * ZR_GRID_PER_CU
                                         : int64_t(1) << 30;
  return static_cast<unsigned>(std::max<int64_t>(1, std::min(tiles, cap)));
}

// Traffic one launch should carry at most (the file comment says why long
// launches are cut).  A/B-measured, launches interleaved in one process: on
// the 1.0e9-element fp32 8-replica fused share 1 GiB 6.02, 2 GiB 6.06, 4 GiB
// 6.05, uncut 5.88 TB/s; on the 5.4e8-element 2-replica MoE expert share
// 5.99 / 6.08 / 6.11 / 6.10 TB/s.
#ifndef ZR_LAUNCH_BYTES
#define ZR_LAUNCH_BYTES (int64_t(2) << 30)
#endif

// Number of equal launches that cover `total` tiles of `tile_bytes` bytes of
// algorithmic traffic each, every launch carrying at most ~ZR_LAUNCH_BYTES.
int64_t launches_for(int64_t total, int64_t tile_bytes) {
  const int64_t per = std::max<int64_t>(1, int64_t(ZR_LAUNCH_BYTES) / std::max<int64_t>(1, tile_bytes));
  return std::max<int64_t>(1, (total + per - 1) / per);
}
// Tiles [first, end) of launch i of n over `total` tiles.
int64_t launch_first(int64_t total, int64_t n, int64_t i) { return total * i / n; }

// Segments of `group` in buckets [first, last), `dst` (-1 all) in bucket order,
// plus the padding of the selected partitions when the range covers the last
// bucket
// (reduce tables only); each gets its tile offset.
std::vector<Seg> build_segments(const zr_plan* plan, int kind, int32_t group,
                                int64_t first, int64_t last, int32_t dst, int64_t tile) {
  std::vector<Seg> out;
  const int64_t a = plan->bucket_first[first];
  const int64_t b = plan->bucket_first[last];
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
  if (kind == kReduceTable && first < last && last == plan->num_buckets) {
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
    tiles += kind == kReduceTable ? reduce_tiles_for(g.numel, tile) : tiles_for(g.numel, tile);
  }
  Seg sentinel{};
  sentinel.tile0 = tiles;
  out.push_back(sentinel);
  return out;
}

// Host segment list for a call (no HIP call is made).
zr_status get_host_table(const zr_plan* plan, int kind, int32_t group, int64_t first,
                         int64_t last, int32_t dst, int64_t tile, const std::vector<Seg>** out) {
  DevCache* c = cache_of(plan);
  std::lock_guard<std::mutex> lk(c->mu);
  const HostKey key{kind, group, first, last, dst, tile};
  auto it = c->host.find(key);
  if (it == c->host.end()) {
    HostTable t;
    try {
      t.segs = build_segments(plan, kind, group, first, last, dst, tile);
    } catch (const std::bad_alloc&) {
      return fail(ZR_ERR_OOM, "out of host memory building a launch table");
    }
    it = c->host.emplace(key, std::move(t)).first;
  }
  *out = &it->second.segs;  // std::map nodes are stable
  return ZR_OK;
}

// Device copy of the same list on `device` (synchronous upload on first use).
zr_status get_dev_table(const zr_plan* plan, int kind, int32_t group, int64_t first,
                        int64_t last, int32_t dst, int64_t tile, int device,
                        const std::vector<Seg>& host,
                        const Seg** out) {
  DevCache* c = cache_of(plan);
  std::lock_guard<std::mutex> lk(c->mu);
  const DevKey key{device, kind, group, first, last, dst, tile};
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
zr_status launch_reduce_t(const RedArgs& a, int R, bool div, bool dword, unsigned grid,
                          unsigned lds, hipStream_t st) {
#define ZR_LAUNCH(RR, DD)                                                          \
  do {                                                                             \
    constexpr int kTH = red_threads<InT, kFused>();                                \
    if (dword)                                                                     \
      ZR_KERNEL_LAUNCH_LDS(grid, kTH, lds, st, a,                                  \
                           reduce_kernel<InT, RR, DD, kFused, true>);              \
    else                                                                           \
      ZR_KERNEL_LAUNCH_LDS(grid, kTH, lds, st, a,                                  \
                           reduce_kernel<InT, RR, DD, kFused, false>);             \
  } while (0)
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

// Largest segment table (sentinel excluded) the no-allocation call stages.
constexpr int64_t kScratchSegs = static_cast<int64_t>(kScratchBytes / sizeof(Seg)) - 1;
static_assert(sizeof(Seg) == 40 && kScratchSegs == 6552, "scratch capacity stated in the header");

// Device address of `scratch` on the current device: looked up once per
// device (with that device current) and kept.
std::mutex g_scratch_mu;
void* g_scratch_ptr[64];

zr_status scratch_for(int device, Seg** out) {
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(ZR_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_ptr[device] = ptr;
  }
  *out = static_cast<Seg*>(g_scratch_ptr[device]);
  return ZR_OK;
}

// Writes segs[0, n) into the scratch table on `stream` (vector stores from a
// staging kernel; nothing allocated).
zr_status stage_segments(const Seg* segs, int64_t n, Seg* table, hipStream_t stream) {
  for (int64_t b = 0; b < n; b += kStageSegs) {
    StageArgs sa;
    std::memset(&sa, 0, sizeof(sa));
    sa.n = static_cast<int32_t>(std::min<int64_t>(kStageSegs, n - b));
    for (int i = 0; i < sa.n; ++i) sa.seg[i] = segs[b + i];
    sa.out = table + b;
    ZR_KERNEL_LAUNCH(1, kStageSegs, stream, sa, stage_segs_kernel);
    const zr_status st = check_launch("segment staging launch");
    if (st != ZR_OK) return st;
  }
  return ZR_OK;
}

// Shared validation + launch of the reduce kernel in either mode; max_wgs > 0
// caps the grid (0: one workgroup per tile).  noalloc: the segment table is
// staged in `scratch` instead of the plan's device table.
// Tile shape of a reduce call's kernels, by replica element type and kernel.
int64_t reduce_tile(zr_dtype dt, bool fused) {
  return dt != ZR_BF16 ? red_tile<float, true>()
         : fused       ? red_tile<uint16_t, true>()
                       : red_tile<uint16_t, false>();
}
// Bytes one tile of a reduce call moves (the replicas, plus the partition
// output or the Adam state), which sets how many launches a selection is cut
// into.
int64_t reduce_tile_bytes(int64_t tile, int world, size_t s, bool fused, bool gout) {
  return tile * (static_cast<int64_t>(world) * static_cast<int64_t>(s) +
                 (fused ? 26 + (gout ? 4 : 0) : 4));
}

zr_status run_reduce(const zr_plan* plan, int32_t group, int64_t first, int64_t last,
                     int32_t dst,
                     const zr_replica* reps, zr_dtype dt, float* const* part_out,
                     const zr_adam* h, float* master, float* m, float* v,
                     uint16_t* pbf16, float* gout, bool fused, int64_t max_wgs,
                     hipStream_t stream, bool noalloc = false) {
  zr::clear_error();
  if (!plan) return fail(ZR_ERR_INVALID, "plan is null");
  if (group < 0 || group >= static_cast<int32_t>(plan->groups.size()))
    return fail(ZR_ERR_INVALID, "group index out of range");
  if (first < 0 || last > plan->num_buckets || first > last)
    return fail(ZR_ERR_INVALID, "bucket index out of range");
  const zr::GroupInfo& gi = plan->groups[group];
  if (dst < -1 || dst >= gi.world) return fail(ZR_ERR_INVALID, "dst out of range");
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
    a.state_stride = dst < 0 ? gi.part : 0;
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
  const int64_t tile = reduce_tile(dt, fused);
  zr_status st = get_host_table(plan, kReduceTable, group, first, last, dst, tile, &hs);
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
  if (noalloc && nseg > kScratchSegs)
    return fail(ZR_ERR_INVALID, "the selection has " + std::to_string(nseg) +
                                    " segments; the no-allocation call stages at most " +
                                    std::to_string(kScratchSegs));
  if (nseg == 0) return ZR_OK;
  int device = 0, cus = 1;
  st = device_info(&device, &cus);
  if (st != ZR_OK) return st;
  for (int r = 0; r < gi.world; ++r)
    a.in[r] = reinterpret_cast<uint64_t>(reps[r].ptr) -
              static_cast<uint64_t>(reps[r].flat_base) * s;
  a.nseg = nseg;
  const int64_t total = (*hs)[nseg].tile0;
  a.R = gi.world;
  a.divisor = static_cast<float>(gi.divisor);
  a.inv_divisor = 1.0f / static_cast<float>(gi.divisor);
  const bool div = !pow2(gi.divisor);
  // Does some segment have no tile phase at which every stream is
  // slot-aligned (the kernel's first two choices)?  Then launch the variant
  // that also accepts dword-aligned phases.
  auto slot_phase_exists = [&](const Seg& g) {
    const int64_t spart = fused ? g.part + static_cast<int64_t>(g.dst) * a.state_stride : g.part;
    for (int64_t j = 0; j < VE; ++j) {
      bool ok = true;
      if (!g.pad)
        for (int r = 0; r < gi.world && ok; ++r)
          ok = aligned(a.in[r] + static_cast<uint64_t>(g.flat + j) * s, VE * s);
      const uint64_t p4 = static_cast<uint64_t>(spart + j) * 4;
      if (fused) {
        ok = ok && aligned(reinterpret_cast<uint64_t>(a.master) + p4, 16) &&
             aligned(reinterpret_cast<uint64_t>(a.m) + p4, 16) &&
             aligned(reinterpret_cast<uint64_t>(a.v) + p4, 16) &&
             (!a.pbf16 || aligned(reinterpret_cast<uint64_t>(a.pbf16) +
                                      static_cast<uint64_t>(spart + j) * 2, 8)) &&
             (!a.gout || aligned(reinterpret_cast<uint64_t>(a.gout) + p4, 16));
      } else {
        ok = ok && aligned(a.out[g.dst] + p4, 16);
      }
      if (ok) return true;
    }
    return false;
  };
  bool dword = false;
  for (int i = 0; i < nseg && !dword; ++i) dword = !slot_phase_exists((*hs)[i]);
  const int64_t nl = launches_for(total, reduce_tile_bytes(tile, gi.world, s, fused, gout));
  // Queried before anything is enqueued (the staging launch included).
  unsigned lds = 0;
  st = reduce_lds_bytes(device, fused, dt == ZR_BF16, gi.world, max_wgs > 0, &lds);
  if (st != ZR_OK) return st;
  if (noalloc) {
    Seg* table = nullptr;
    st = scratch_for(device, &table);
    if (st != ZR_OK) return st;
    st = stage_segments(hs->data(), nseg + 1, table, stream);
    if (st != ZR_OK) return st;
    a.segs = table;
  } else {
    st = get_dev_table(plan, kReduceTable, group, first, last, dst, tile, device, *hs, &a.segs);
    if (st != ZR_OK) return st;
  }
  for (int64_t i = 0; i < nl; ++i) {
    a.tile_base = launch_first(total, nl, i);
    a.tile_end = launch_first(total, nl, i + 1);
    // A capped grid walks the tiles in steps of its size (the kernel's
    // grid-stride loop), so the launch holds at most max_wgs workgroup slots.
    const int64_t n = a.tile_end - a.tile_base;
    // Uncapped launches of one tile per workgroup over enough replicas take
    // the XCD-weighted order.
    a.skew = max_wgs <= 0 && xcd_weighted(gi.world);
    const unsigned grid = max_wgs > 0
        ? static_cast<unsigned>(std::min<int64_t>(grid_for(n, cus), max_wgs))
        : a.skew ? static_cast<unsigned>(skew_grid(n))
                 : grid_for(n, cus);
    if (dt == ZR_BF16)
      st = fused ? launch_reduce_t<uint16_t, true>(a, gi.world, div, dword, grid, lds, stream)
                 : launch_reduce_t<uint16_t, false>(a, gi.world, div, dword, grid, lds, stream);
    else
      st = fused ? launch_reduce_t<float, true>(a, gi.world, div, dword, grid, lds, stream)
                 : launch_reduce_t<float, false>(a, gi.world, div, dword, grid, lds, stream);
    if (st != ZR_OK) return st;
  }
  return ZR_OK;
}

}  // namespace

// =============================================================== C ABI ===

namespace {
// A call's bucket argument (-1 = every bucket) as a range [first, last);
// out-of-range values give an empty-checked range that run_reduce rejects.
std::pair<int64_t, int64_t> bucket_range(const zr_plan* plan, int64_t bucket) {
  if (!plan) return {0, 0};
  if (bucket == -1) return {0, plan->num_buckets};
  if (bucket < -1 || bucket >= plan->num_buckets) return {1, 0};   // invalid
  return {bucket, bucket + 1};
}
// [first, first + count) as a range, or an invalid one.
std::pair<int64_t, int64_t> count_range(const zr_plan* plan, int64_t first, int64_t count) {
  if (!plan || first < 0 || count < 0 || first > plan->num_buckets ||
      count > plan->num_buckets - first)
    return {1, 0};   // invalid
  return {first, first + count};
}
}  // namespace

extern "C" zr_status zr_plan_reduce_launches(const zr_plan* plan, int32_t group,
                                             int64_t bucket_first, int64_t bucket_count,
                                             int32_t dst, zr_dtype grad_dtype, int32_t fused,
                                             int32_t with_grad_out, int64_t* tiles,
                                             int64_t* launches) {
  zr::clear_error();
  try {
    if (!plan) return fail(ZR_ERR_INVALID, "plan is null");
    if (group < 0 || group >= static_cast<int32_t>(plan->groups.size()))
      return fail(ZR_ERR_INVALID, "group index out of range");
    const auto fl = count_range(plan, bucket_first, bucket_count);
    if (fl.first > fl.second) return fail(ZR_ERR_INVALID, "bucket range out of range");
    const zr::GroupInfo& gi = plan->groups[group];
    if (dst < -1 || dst >= gi.world) return fail(ZR_ERR_INVALID, "dst out of range");
    if (!valid_dtype(grad_dtype)) return fail(ZR_ERR_INVALID, "unsupported gradient dtype");
    if (!tiles && !launches) return fail(ZR_ERR_INVALID, "no output pointer");
    const int64_t tile = reduce_tile(grad_dtype, fused != 0);
    const std::vector<Seg>* hs = nullptr;
    const zr_status st = get_host_table(plan, kReduceTable, group, fl.first, fl.second, dst,
                                        tile, &hs);
    if (st != ZR_OK) return st;
    const int64_t nseg = static_cast<int64_t>(hs->size()) - 1;
    const int64_t total = nseg > 0 ? (*hs)[nseg].tile0 : 0;
    if (tiles) *tiles = total;
    if (launches)
      *launches = nseg > 0 ? launches_for(total, reduce_tile_bytes(tile, gi.world,
                                                                   dtype_size(grad_dtype),
                                                                   fused != 0,
                                                                   with_grad_out != 0))
                           : 0;
    return ZR_OK;
  } catch (...) {
    return fail(ZR_ERR_OOM, "unexpected host error");
  }
}

extern "C" zr_status zr_reduce_launch_occupancy(zr_dtype grad_dtype, int32_t fused,
                                                int32_t world, int32_t* wgs_per_cu,
                                                int32_t* weighted) {
  zr::clear_error();
  if (!valid_dtype(grad_dtype)) return fail(ZR_ERR_INVALID, "unsupported gradient dtype");
  if (world < 1) return fail(ZR_ERR_INVALID, "world must be at least 1");
  if (!wgs_per_cu && !weighted) return fail(ZR_ERR_INVALID, "no output pointer");
  if (wgs_per_cu) *wgs_per_cu = reduce_wgs_per_cu(grad_dtype == ZR_BF16, fused != 0, world);
  if (weighted) *weighted = xcd_weighted(world) ? 1 : 0;
  return ZR_OK;
}

extern "C" zr_status zr_reduce_scatter_local(const zr_plan* plan, int32_t group,
                                             int64_t bucket, int32_t dst,
                                             const zr_replica* reps, zr_dtype grad_dtype,
                                             float* const* part_out, hipStream_t stream) {
  try {
    const auto r = bucket_range(plan, bucket);
    return run_reduce(plan, group, r.first, r.second, dst, reps, grad_dtype, part_out,
                      nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, false, 0, stream);
  } catch (...) {
    return fail(ZR_ERR_OOM, "unexpected host error");
  }
}

extern "C" zr_status zr_reduce_scatter_local_range(const zr_plan* plan, int32_t group,
                                                   int64_t bucket_first, int64_t bucket_count,
                                                   int32_t dst, const zr_replica* reps,
                                                   zr_dtype grad_dtype, float* const* part_out,
                                                   hipStream_t stream) {
  try {
    const auto r = count_range(plan, bucket_first, bucket_count);
    return run_reduce(plan, group, r.first, r.second, dst, reps, grad_dtype, part_out,
                      nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, false, 0, stream);
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
    const auto r = bucket_range(plan, bucket);
    return run_reduce(plan, group, r.first, r.second, dst, reps, grad_dtype, nullptr, h,
                      master, m, v, param_bf16, grad_out, true, 0, stream);
  } catch (...) {
    return fail(ZR_ERR_OOM, "unexpected host error");
  }
}

extern "C" zr_status zr_reduce_scatter_adam_range(const zr_plan* plan, int32_t group,
                                                  int64_t bucket_first, int64_t bucket_count,
                                                  int32_t dst, const zr_replica* reps,
                                                  zr_dtype grad_dtype, const zr_adam* h,
                                                  float* master, float* m, float* v,
                                                  uint16_t* param_bf16, float* grad_out,
                                                  hipStream_t stream) {
  try {
    const auto r = count_range(plan, bucket_first, bucket_count);
    return run_reduce(plan, group, r.first, r.second, dst, reps, grad_dtype, nullptr, h,
                      master, m, v, param_bf16, grad_out, true, 0, stream);
  } catch (...) {
    return fail(ZR_ERR_OOM, "unexpected host error");
  }
}

extern "C" zr_status zr_reduce_scatter_adam_capped(const zr_plan* plan, int32_t group,
                                                   int64_t bucket, int32_t dst,
                                                   const zr_replica* reps,
                                                   zr_dtype grad_dtype, const zr_adam* h,
                                                   float* master, float* m, float* v,
                                                   uint16_t* param_bf16, float* grad_out,
                                                   int32_t max_workgroups,
                                                   hipStream_t stream) {
  try {
    if (max_workgroups < 1) {
      zr::clear_error();
      return fail(ZR_ERR_INVALID, "max_workgroups must be >= 1");
    }
    const auto r = bucket_range(plan, bucket);
    return run_reduce(plan, group, r.first, r.second, dst, reps, grad_dtype, nullptr, h,
                      master, m, v, param_bf16, grad_out, true, max_workgroups, stream);
  } catch (...) {
    return fail(ZR_ERR_OOM, "unexpected host error");
  }
}

extern "C" zr_status zr_reduce_scatter_adam_noalloc(const zr_plan* plan, int32_t group,
                                                    int64_t bucket, int32_t dst,
                                                    const zr_replica* reps,
                                                    zr_dtype grad_dtype, const zr_adam* h,
                                                    float* master, float* m, float* v,
                                                    uint16_t* param_bf16, float* grad_out,
                                                    hipStream_t stream) {
  try {
    const auto r = bucket_range(plan, bucket);
    return run_reduce(plan, group, r.first, r.second, dst, reps, grad_dtype, nullptr, h,
                      master, m, v, param_bf16, grad_out, true, 0, stream, true);
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
  // fp32 pointers are always dword-aligned; the bf16 output must be too
  // for its 8-byte stores (an even element offset).
  const bool dword = !param_bf16 || elem_aligned(param_bf16, 4);
  const int64_t total = (n + kAdamTileElems - 1) / kAdamTileElems;
  const int64_t nl = launches_for(total, kAdamTileElems * 30);
  for (int64_t i = 0; i < nl; ++i) {
    a.tile_base = launch_first(total, nl, i);
    a.tile_end = launch_first(total, nl, i + 1);
    const unsigned grid = grid_for(a.tile_end - a.tile_base, cus);
    if (vec) ZR_KERNEL_LAUNCH(grid, kThreads, stream, a, adam_kernel<true, false>);
    else if (dword) ZR_KERNEL_LAUNCH(grid, kThreads, stream, a, adam_kernel<true, true>);
    else ZR_KERNEL_LAUNCH(grid, kThreads, stream, a, adam_kernel<false, false>);
    st = check_launch("adam_partition launch");
    if (st != ZR_OK) return st;
  }
  return ZR_OK;
}

namespace {
template <bool kFirst>
void launch_ipg(const IpgArgs& a, zr_dtype grad_dtype, bool dword, unsigned grid,
                hipStream_t stream) {
  if (grad_dtype == ZR_BF16) {
    if (dword) ZR_KERNEL_LAUNCH(grid, kThreads, stream, a, ipg_kernel<uint16_t, true, kFirst>);
    else ZR_KERNEL_LAUNCH(grid, kThreads, stream, a, ipg_kernel<uint16_t, false, kFirst>);
  } else {
    if (dword) ZR_KERNEL_LAUNCH(grid, kThreads, stream, a, ipg_kernel<float, true, kFirst>);
    else ZR_KERNEL_LAUNCH(grid, kThreads, stream, a, ipg_kernel<float, false, kFirst>);
  }
}

// Validation and launches of both IPG entry points; `first`: main_grad is
// taken as zero and not read.
zr_status run_ipg(const zr_plan* plan, const int64_t* param_ids, const void* const* grads,
                  int64_t n, zr_dtype grad_dtype, float* main_grad, int64_t window_base,
                  int64_t window_len, bool first, hipStream_t stream) {
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
        tiles += tiles_for(segs[i].numel, kIpgTileElems);
      }
      a.nseg = static_cast<int32_t>(e - b);
      a.main_grad = main_grad;
      // The dword-aligned variant is needed when some segment has no phase
      // at which the gradient and main_grad are both slot-aligned.
      bool dword = false;
      const uint64_t mgp = reinterpret_cast<uint64_t>(main_grad);
      for (int i = 0; i < a.nseg && !dword; ++i) {
        bool any = false;
        for (int64_t j = 0; j < VE && !any; ++j)
          any = aligned(a.seg[i].src + static_cast<uint64_t>(j) * s, VE * s) &&
                aligned(mgp + static_cast<uint64_t>(a.seg[i].dst + j) * 4, 16);
        dword = !any;
      }
      // Bytes per tile: the gradient read, main_grad written (and read).
      const int64_t nl =
          launches_for(tiles, kIpgTileElems * static_cast<int64_t>(s + (first ? 4 : 8)));
      for (int64_t i = 0; i < nl; ++i) {
        a.tile_base = launch_first(tiles, nl, i);
        a.tile_end = launch_first(tiles, nl, i + 1);
        const unsigned grid = grid_for(a.tile_end - a.tile_base, cus);
        if (first)
          launch_ipg<true>(a, grad_dtype, dword, grid, stream);
        else
          launch_ipg<false>(a, grad_dtype, dword, grid, stream);
        st = check_launch("ipg_accumulate launch");
        if (st != ZR_OK) return st;
      }
    }
    return ZR_OK;
  } catch (...) {
    return fail(ZR_ERR_OOM, "unexpected host error");
  }
}
}  // namespace

extern "C" zr_status zr_ipg_accumulate(const zr_plan* plan, const int64_t* param_ids,
                                       const void* const* grads, int64_t n,
                                       zr_dtype grad_dtype, float* main_grad,
                                       int64_t window_base, int64_t window_len,
                                       hipStream_t stream) {
  return run_ipg(plan, param_ids, grads, n, grad_dtype, main_grad, window_base, window_len,
                 false, stream);
}

extern "C" zr_status zr_ipg_accumulate_first(const zr_plan* plan, const int64_t* param_ids,
                                             const void* const* grads, int64_t n,
                                             zr_dtype grad_dtype, float* main_grad,
                                             int64_t window_base, int64_t window_len,
                                             hipStream_t stream) {
  return run_ipg(plan, param_ids, grads, n, grad_dtype, main_grad, window_base, window_len,
                 true, stream);
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
    zr_status st = get_host_table(plan, kCopyTable, group, bucket, bucket + 1, dst, kCopyTileElems, &hs);
    if (st != ZR_OK) return st;
    const int nseg = static_cast<int>(hs->size()) - 1;
    if (nseg == 0) return ZR_OK;
    int device = 0, cus = 1;
    st = device_info(&device, &cus);
    if (st != ZR_OK) return st;
    CopyArgs a{};
    st = get_dev_table(plan, kCopyTable, group, bucket, bucket + 1, dst, kCopyTileElems, device, *hs,
                       &a.segs);
    if (st != ZR_OK) return st;
    a.src = bucket_layout_src;
    a.dst = part_out;
    a.nseg = nseg;
    const int64_t total = (*hs)[nseg].tile0;
    // The dword-aligned variant is needed when some segment has no phase at
    // which source and destination are both 16-byte aligned.
    bool dword = false;
    for (int i = 0; i < nseg && !dword; ++i) {
      const uint64_t sa = reinterpret_cast<uint64_t>(bucket_layout_src + (*hs)[i].flat);
      const uint64_t da = reinterpret_cast<uint64_t>(part_out + (*hs)[i].part);
      bool any = false;
      for (uint64_t j = 0; j < VE && !any; ++j) any = aligned(sa + 4 * j, 16) && aligned(da + 4 * j, 16);
      dword = !any;
    }
    const int64_t nl = launches_for(total, kCopyTileElems * 8);
    for (int64_t i = 0; i < nl; ++i) {
      a.tile_base = launch_first(total, nl, i);
      a.tile_end = launch_first(total, nl, i + 1);
      const unsigned grid = grid_for(a.tile_end - a.tile_base, cus);
      if (dword) ZR_KERNEL_LAUNCH(grid, kThreads, stream, a, copy_kernel<true>);
      else ZR_KERNEL_LAUNCH(grid, kThreads, stream, a, copy_kernel<false>);
      st = check_launch("copy_grads_in_partition launch");
      if (st != ZR_OK) return st;
    }
    return ZR_OK;
  } catch (...) {
    return fail(ZR_ERR_OOM, "unexpected host error");
  }
}


extern "C" zr_status zr_all_gather_params(const zr_plan* plan, int32_t group,
                                          const void* const* parts, zr_dtype dtype,
                                          void* out, int64_t out_base, int64_t out_len,
                                          hipStream_t stream) {
  zr::clear_error();
  try {
    if (!plan) return fail(ZR_ERR_INVALID, "plan is null");
    if (group < 0 || group >= static_cast<int32_t>(plan->groups.size()))
      return fail(ZR_ERR_INVALID, "group index out of range");
    if (!valid_dtype(dtype)) return fail(ZR_ERR_INVALID, "unsupported element dtype");
    if (out_base < 0 || out_len < 0)
      return fail(ZR_ERR_INVALID, "window base and length must be >= 0");
    const zr::GroupInfo& gi = plan->groups[group];
    if (out_base + out_len > gi.total)
      return fail(ZR_ERR_INVALID, "window runs past the group's real elements");
    if (out_len == 0) return ZR_OK;
    const size_t es = dtype_size(dtype);
    if (!parts) return fail(ZR_ERR_INVALID, "parts is null");
    if (!out || !elem_aligned(out, es)) return fail(ZR_ERR_INVALID, "out is null or misaligned");
    XArgs a;
    std::memset(&a, 0, sizeof(a));
    int64_t tiles = 0;
    int n = 0;
    for (int32_t k = 0; k < gi.world; ++k) {
      const int64_t lo = std::max(out_base, k * gi.part);
      const int64_t hi = std::min(out_base + out_len, (k + 1) * gi.part);
      if (lo >= hi) continue;
      if (!parts[k] || !elem_aligned(parts[k], es))
        return fail(ZR_ERR_INVALID, "partition " + std::to_string(k) + " is null or misaligned");
      XSeg& g = a.seg[n++];
      g.src = reinterpret_cast<uint64_t>(parts[k]) + static_cast<uint64_t>(lo - k * gi.part) * es;
      g.dst = reinterpret_cast<uint64_t>(out) + static_cast<uint64_t>(lo - out_base) * es;
      g.numel = hi - lo;
      g.tile0 = tiles;
      // + one slot: a segment whose start is not slot-aligned spans one more.
      const int64_t te = es == 2 ? gather_tile_elems<uint16_t>() : gather_tile_elems<float>();
      tiles += (g.numel + 16 / static_cast<int64_t>(es) - 1 + te - 1) / te;
    }
    a.nseg = n;
    int device = 0, cus = 1;
    zr_status st = device_info(&device, &cus);
    if (st != ZR_OK) return st;
    // The dword-aligned variant is needed when some partition has no phase
    // at which it and the output are both 16-byte aligned.
    bool dword = false;
    for (int i = 0; i < n && !dword; ++i) {
      bool any = false;
      for (int64_t j = 0; j < 16 / static_cast<int64_t>(es) && !any; ++j)
        any = aligned(a.seg[i].src + j * es, 16) && aligned(a.seg[i].dst + j * es, 16);
      dword = !any;
    }
    const int64_t nl = launches_for(tiles, kGatherTileBytes * 2);
    for (int64_t i = 0; i < nl; ++i) {
      a.tile_base = launch_first(tiles, nl, i);
      a.tile_end = launch_first(tiles, nl, i + 1);
      const unsigned grid = grid_for(a.tile_end - a.tile_base, cus);
      if (dtype == ZR_BF16) {
        if (dword) ZR_KERNEL_LAUNCH(grid, kThreads, stream, a, gather_kernel<uint16_t, true>);
        else ZR_KERNEL_LAUNCH(grid, kThreads, stream, a, gather_kernel<uint16_t, false>);
      } else {
        if (dword) ZR_KERNEL_LAUNCH(grid, kThreads, stream, a, gather_kernel<float, true>);
        else ZR_KERNEL_LAUNCH(grid, kThreads, stream, a, gather_kernel<float, false>);
      }
      st = check_launch("all_gather_params launch");
      if (st != ZR_OK) return st;
    }
    return ZR_OK;
  } catch (...) {
    return fail(ZR_ERR_OOM, "unexpected host error");
  }
}

// Shared validation of the ring steps.
namespace {
// Does some rank's chunk of this step have no phase at which its source (the
// previous rank's buffer) and destination are both 16-byte aligned?  The chunk
// index of rank k is (k - step - lag) mod n (lag 2 for the reduce-scatter
// steps, 1 for the all-gather steps).
bool ring_needs_dword(const RingArgs& a, int lag) {
  for (int k = 0; k < a.n; ++k) {
    int c = (k - a.step - lag) % a.n;
    if (c < 0) c += a.n;
    const int prev = k == 0 ? a.n - 1 : k - 1;
    const uint64_t off = static_cast<uint64_t>(c) * static_cast<uint64_t>(a.chunk) * 4;
    if ((a.buf[k] + off - (a.buf[prev] + off)) % 16 != 0) return true;
  }
  return false;
}

zr_status ring_args(float* const* rank_bufs, int32_t n_ranks, int64_t chunk_numel,
                    int32_t step, int64_t tile, RingArgs* a) {
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
  std::memset(a, 0, sizeof(*a));
  for (int k = 0; k < n_ranks; ++k) a->buf[k] = reinterpret_cast<uint64_t>(rank_bufs[k]);
  a->chunk = chunk_numel;
  a->tiles_per_rank = tiles_for(chunk_numel, tile);
  a->n = n_ranks;
  a->step = step;
  return ZR_OK;
}
}  // namespace

extern "C" zr_status zr_ring_ag_step(float* const* rank_bufs, int32_t n_ranks,
                                     int64_t chunk_numel, int32_t step,
                                     hipStream_t stream) {
  zr::clear_error();
  RingArgs a;
  zr_status st = ring_args(rank_bufs, n_ranks, chunk_numel, step, kRingAgTileElems, &a);
  if (st != ZR_OK || chunk_numel == 0) return st;
  int device = 0, cus = 1;
  st = device_info(&device, &cus);
  if (st != ZR_OK) return st;
  const bool dword = ring_needs_dword(a, 1);
  const int64_t total = a.tiles_per_rank * n_ranks;
  const int64_t nl = launches_for(total, kRingAgTileElems * 8);
  for (int64_t i = 0; i < nl; ++i) {
    a.tile_base = launch_first(total, nl, i);
    a.tile_end = launch_first(total, nl, i + 1);
    const unsigned grid = grid_for(a.tile_end - a.tile_base, cus);
    if (dword) ZR_KERNEL_LAUNCH(grid, kThreads, stream, a, ring_ag_kernel<true>);
    else ZR_KERNEL_LAUNCH(grid, kThreads, stream, a, ring_ag_kernel<false>);
    st = check_launch("ring_ag_step launch");
    if (st != ZR_OK) return st;
  }
  return ZR_OK;
}

extern "C" zr_status zr_ring_rs_step(float* const* rank_bufs, int32_t n_ranks,
                                     int64_t chunk_numel, int32_t step,
                                     hipStream_t stream) {
  zr::clear_error();
  RingArgs a;
  zr_status st = ring_args(rank_bufs, n_ranks, chunk_numel, step, kRingTileElems, &a);
  if (st != ZR_OK || chunk_numel == 0) return st;
  int device = 0, cus = 1;
  st = device_info(&device, &cus);
  if (st != ZR_OK) return st;
  const bool dword = ring_needs_dword(a, 2);
  const int64_t total = a.tiles_per_rank * n_ranks;
  const int64_t nl = launches_for(total, kRingTileElems * 12);
  for (int64_t i = 0; i < nl; ++i) {
    a.tile_base = launch_first(total, nl, i);
    a.tile_end = launch_first(total, nl, i + 1);
    const unsigned grid = grid_for(a.tile_end - a.tile_base, cus);
    if (dword) ZR_KERNEL_LAUNCH(grid, kThreads, stream, a, ring_kernel<true>);
    else ZR_KERNEL_LAUNCH(grid, kThreads, stream, a, ring_kernel<false>);
    st = check_launch("ring_rs_step launch");
    if (st != ZR_OK) return st;
  }
  return ZR_OK;
}
