// The HIP runtime calls the library makes, for its CPU build: "device"
// memory is host memory, registered for the access checks of the kernels'
// vector loads and stores (tests/native/emu/hip/hip_runtime.h).

#include <hip/hip_runtime.h>
#include <sanitizer/common_interface_defs.h>

#include <cstdio>
#include <cstdlib>
#include <map>
#include <mutex>
#include <string>

namespace {
std::mutex g_mu;
std::map<uintptr_t, size_t>& regions() {
  static std::map<uintptr_t, size_t> r;
  return r;
}
}  // namespace

thread_local zr_emu_dim zr_emu_block, zr_emu_thread, zr_emu_grid;
long long zr_emu_launches = 0;
unsigned zr_emu_lds_max = 0;

// Launches per kernel instantiation, named by the sanitizer runtime's
// symbolizer from the kernel's address (this build always runs under it).
std::map<std::string, long long>& zr_emu_coverage() {
  static std::map<std::string, long long> c;
  return c;
}
void zr_emu_count(void* kernel) {
  static std::map<void*, std::string> names;
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = names.find(kernel);
  if (it == names.end()) {
    char buf[1024] = {0};
    // the symbolizer takes a return address (it looks one byte back)
    __sanitizer_symbolize_pc(static_cast<char*>(kernel) + 1, "%f", buf, sizeof(buf));
    // "void (anonymous namespace)::name<args>(params)" -> "name<args>"
    std::string n(buf);
    const std::string anon = "(anonymous namespace)::";
    const size_t at = n.find(anon);
    if (at != std::string::npos) n = n.substr(at + anon.size());
    size_t end = n.find('(');
    const size_t lt = n.find('<');
    if (lt != std::string::npos && lt < end) {
      int depth = 0;
      for (size_t i = lt; i < n.size(); ++i) {
        if (n[i] == '<') ++depth;
        if (n[i] == '>' && --depth == 0) { end = i + 1; break; }
      }
    }
    if (end != std::string::npos) n = n.substr(0, end);
    it = names.emplace(kernel, n).first;
  }
  ++zr_emu_coverage()[it->second];
}

void zr_emu_register(const void* p, size_t bytes) {
  std::lock_guard<std::mutex> lk(g_mu);
  regions()[reinterpret_cast<uintptr_t>(p)] = bytes;
}
void zr_emu_unregister(const void* p) {
  std::lock_guard<std::mutex> lk(g_mu);
  regions().erase(reinterpret_cast<uintptr_t>(p));
}
void zr_emu_check(const void* p, size_t bytes, bool store) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = regions().upper_bound(a);
  if (it != regions().begin()) {
    --it;
    if (a >= it->first && a + bytes <= it->first + it->second) return;
  }
  std::fprintf(stderr,
               "out-of-bounds %s of %zu bytes at %p (block %u, lane %u of a %u-workgroup "
               "launch)\n",
               store ? "store" : "load", bytes, p, zr_emu_block.x, zr_emu_thread.x,
               zr_emu_grid.x);
  std::abort();
}

extern "C" {
hipError_t hipGetDevice(int* d) {
  *d = 0;
  return hipSuccess;
}
hipError_t hipSetDevice(int) { return hipSuccess; }
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t attr, int) {
  *v = attr == hipDeviceAttributeMultiprocessorCount          ? 256
       : attr == hipDeviceAttributeMaxSharedMemoryPerMultiprocessor ? 160 * 1024
                                                                    : 0;
  return hipSuccess;
}
hipError_t hipGetLastError(void) { return hipSuccess; }
const char* hipGetErrorString(hipError_t) { return "emulated runtime"; }
hipError_t hipMalloc(void** p, size_t n) {
  *p = std::malloc(n ? n : 1);
  if (!*p) return hipErrorOutOfMemory;
  zr_emu_register(*p, n);
  return hipSuccess;
}
hipError_t hipFree(void* p) {
  zr_emu_unregister(p);
  std::free(p);
  return hipSuccess;
}
hipError_t hipMemcpy(void* d, const void* s, size_t n, hipMemcpyKind) {
  std::memcpy(d, s, n);
  return hipSuccess;
}
hipError_t hipGetSymbolAddress(void** d, const void* symbol) {
  *d = const_cast<void*>(symbol);
  return hipSuccess;
}
}
