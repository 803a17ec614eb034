// CPU build of the library's HIP sources, for bounds checking under
// AddressSanitizer and UndefinedBehaviorSanitizer.
//
// Every kernel of the library is a per-lane stream: no LDS, no barriers, and
// the only cross-lane operation (readfirstlane) is applied to values every
// lane of the wave already holds.  Running the lanes of each workgroup one
// after another therefore makes exactly the memory accesses a GPU launch
// makes, and the sanitizers see every one of them.  This header stands in for
// <hip/hip_runtime.h> when the sources are compiled for the host (it comes
// first on the include path); tests/native/emu/emu_runtime.cpp provides the
// few runtime calls the library makes.
#pragma once

#include <hip/hip_runtime_api.h>   // the runtime's types and declarations

#include <cstddef>
#include <cstdint>
#include <cstring>

#define __global__
#define __launch_bounds__(...)
#define __align__(n) __attribute__((aligned(n)))
#define HIP_SYMBOL(x) x
#define ZR_GLOBAL
#define ZR_CONST

struct zr_emu_dim {
  unsigned x = 0, y = 0, z = 0;
};
extern thread_local zr_emu_dim zr_emu_block, zr_emu_thread, zr_emu_grid;
#define blockIdx zr_emu_block
#define threadIdx zr_emu_thread
#define gridDim zr_emu_grid

inline float __uint_as_float(uint32_t u) {
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}
inline uint32_t __float_as_uint(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return u;
}
#define __builtin_amdgcn_readfirstlane(x) (x)
inline uint32_t zr_emu_alignbit(uint32_t hi, uint32_t lo, uint32_t s) {
  return static_cast<uint32_t>(((static_cast<uint64_t>(hi) << 32) | lo) >> (s & 31));
}
#define __builtin_amdgcn_alignbit(hi, lo, s) zr_emu_alignbit((hi), (lo), (s))

// Every vector access of a kernel goes through the non-temporal load/store
// builtins; here each one is checked against the registered buffers (the
// driver's exact-size buffers and the library's own device allocations)
// before it is made.
// The access copies bytes (no alignment assumed): the kernels' dword-aligned
// variants make two- and four-dword accesses at merely dword-aligned
// addresses, which the GPU's global loads and stores accept (the alignment a
// kernel may assume is a template value there, and a deduced template type
// here would carry the vector's natural alignment instead).
void zr_emu_check(const void* p, size_t bytes, bool store);
template <typename T>
inline T zr_emu_nt_load(const T* p) {
  zr_emu_check(p, sizeof(T), false);
  T v;
  std::memcpy(static_cast<void*>(&v), static_cast<const void*>(p), sizeof(T));
  return v;
}
template <typename T>
inline void zr_emu_nt_store(T v, T* p) {
  zr_emu_check(p, sizeof(T), true);
  std::memcpy(static_cast<void*>(p), static_cast<const void*>(&v), sizeof(T));
}
#define __builtin_nontemporal_load(p) zr_emu_nt_load(p)
#define __builtin_nontemporal_store(v, p) zr_emu_nt_store((v), (p))

// Kernel launch: every lane of every workgroup, in order.  Each launch is
// counted per kernel instantiation (zr_emu_count names the kernel from its
// address) for the coverage report.
extern long long zr_emu_launches;
extern unsigned zr_emu_lds_max;  // most dynamic LDS a launch reserved since reset
void zr_emu_count(void* kernel);
template <auto K, typename Args>
inline void zr_emu_launch(unsigned grid, unsigned block, const Args& args) {
  zr_emu_count(reinterpret_cast<void*>(K));
  zr_emu_grid.x = grid;
  for (unsigned b = 0; b < grid; ++b) {
    zr_emu_block.x = b;
    for (unsigned t = 0; t < block; ++t) {
      zr_emu_thread.x = t;
      K(args);
    }
  }
  ++zr_emu_launches;
}
#define ZR_KERNEL_LAUNCH_LDS(grid, block, lds, stream, args, ...) \
  (zr_emu_lds_max = zr_emu_lds_max > unsigned(lds) ? zr_emu_lds_max : unsigned(lds), \
   zr_emu_launch<&__VA_ARGS__>((grid), (block), (args)))
