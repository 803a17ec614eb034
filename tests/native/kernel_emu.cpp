// Bounds and value check of every kernel of the library, run on the CPU.
//
// Built together with the library's own sources (zr_kernels.hip compiled as
// C++ with tests/native/emu on the include path, zr_plan.cpp) under
// AddressSanitizer + UndefinedBehaviorSanitizer, with tiny launch caps so
// that small cases take the multi-launch path.  Random plans, selections (every bucket, one bucket, a bucket
// range; every destination or one), element types, windows and pointer
// offsets of 0-3 elements drive every entry point.  Each buffer ends exactly
// at the end of its allocation (an overrun is an ASan error to the byte);
// its guard prefix is poisoned where ASan's 8-byte granules allow and filled
// with a sentinel checked after every call; every vector access is checked
// against the buffer's exact range (tests/native/emu/hip/hip_runtime.h).
// Outputs are compared bit for bit with a plain loop over the plan's
// slices, and elements outside the selection must keep their sentinel.
//
// usage: kernel_emu <cases> [first seed]

#include <sanitizer/asan_interface.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "zr.h"

#include <map>

void zr_emu_register(const void* p, size_t bytes);
void zr_emu_unregister(const void* p);
extern long long zr_emu_launches;
extern unsigned zr_emu_lds_max;
std::map<std::string, long long>& zr_emu_coverage();

namespace {

int g_failures = 0;
#define CHECK(cond, ...)                                               \
  do {                                                                 \
    if (!(cond)) {                                                     \
      std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__);        \
      std::fprintf(stderr, __VA_ARGS__);                               \
      std::fprintf(stderr, "\n");                                      \
      ++g_failures;                                                    \
      if (g_failures > 20) std::abort();                               \
    }                                                                  \
  } while (0)

// Workgroups per CU an uncapped reduce launch is held to (0 = no cap), as
// the library states it: at 8 replicas fp32 fused 8, bf16 fused 6, bf16
// reduce-scatter 20, fp32 reduce-scatter 12; at 4 replicas fp32 fused 14,
// bf16 fused 7; at 16 replicas fp32 fused 6, fp32 reduce-scatter 7; at 2
// replicas fp32 fused 18; no other shape.
int want_wgs_per_cu(bool bf16, bool fused, int R) {
  if (R == 8) return fused ? (bf16 ? 6 : 8) : (bf16 ? 20 : 12);
  if (R == 4 && fused) return bf16 ? 7 : 14;
  if (R == 16 && !bf16) return fused ? 6 : 7;
  if (R == 2 && !bf16 && fused) return 18;
  return 0;
}

// A call that launched the reduce kernel reserved 2L / (2k + 1) bytes of LDS
// per workgroup for L = 160 KiB (the emulated device's LDS per CU) when k > 0,
// and nothing otherwise; no launch of the call reserved more.
void check_lds(int seed, int nd, int64_t span, const std::vector<std::vector<char>>& written, int k) {
  bool launched = false;
  for (int d = 0; d < nd && !launched; ++d)
    for (int64_t j = 0; j < span && !launched; ++j) launched = written[d][j] != 0;
  const unsigned want = launched && k > 0 ? unsigned(2 * 160 * 1024 / (2 * k + 1)) : 0u;
  CHECK(zr_emu_lds_max == want, "seed %d: LDS reserved %u, want %u", seed, zr_emu_lds_max, want);
}

struct Rng {
  uint64_t s;
  explicit Rng(uint64_t seed) : s(seed * 0x9E3779B97F4A7C15ull + 1) {}
  uint64_t next() {
    uint64_t z = (s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
  int64_t uni(int64_t lo, int64_t hi) { return lo + static_cast<int64_t>(next() % uint64_t(hi - lo + 1)); }
  double u01() { return (next() >> 11) * (1.0 / 9007199254740992.0); }
  float normal(float sigma) {
    const double u1 = u01() + 1e-300, u2 = u01();
    return static_cast<float>(std::sqrt(-2 * std::log(u1)) * std::cos(6.283185307179586 * u2) * sigma);
  }
  template <typename T>
  const T& pick(const std::vector<T>& v) { return v[next() % v.size()]; }
};

float bits_f(uint32_t u) { float f; std::memcpy(&f, &u, 4); return f; }
uint32_t f_bits(float f) { uint32_t u; std::memcpy(&u, &f, 4); return u; }
uint16_t bf16_of(float x) {            // round to nearest even (test data only)
  uint32_t b = f_bits(x);
  if ((b & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((b >> 16) | 0x40u);
  b += 0x7fffu + ((b >> 16) & 1u);
  return static_cast<uint16_t>(b >> 16);
}

constexpr size_t kGuard = 64;          // guard bytes before every buffer
constexpr unsigned char kSentinel = 0xA5;

// n elements of es bytes, starting off elements (plus the guard) into a fresh
// allocation that ends exactly where the buffer ends.
struct Buf {
  unsigned char* block = nullptr;
  unsigned char* p = nullptr;
  size_t bytes = 0, pre = 0;
  Buf(size_t n, size_t es, int off) {
    bytes = n * es;
    pre = kGuard + static_cast<size_t>(off) * es;
    block = static_cast<unsigned char*>(std::malloc(pre + bytes + (bytes ? 0 : 1)));
    std::memset(block, kSentinel, pre);
    p = block + pre;
    ASAN_POISON_MEMORY_REGION(block, pre & ~size_t(7));
    zr_emu_register(p, bytes);
  }
  ~Buf() {
    ASAN_UNPOISON_MEMORY_REGION(block, pre);
    zr_emu_unregister(p);
    std::free(block);
  }
  Buf(const Buf&) = delete;
  Buf& operator=(const Buf&) = delete;
  bool guard_intact() const {
    for (size_t i = pre & ~size_t(7); i < pre; ++i)
      if (block[i] != kSentinel) return false;
    return true;
  }
  float* f() { return reinterpret_cast<float*>(p); }
  uint16_t* h() { return reinterpret_cast<uint16_t*>(p); }
};

// Element offsets of a case's buffers: half the cases put every buffer on its
// natural alignment (the kernels' common instantiations), a quarter shift
// every buffer by one common offset (streams still share a 4-element slot
// phase, bf16 and fp32 alike), a quarter shift each independently (the
// dword-aligned variants and the shifted bf16 reads).
struct Offsets {
  int mode, common;
  explicit Offsets(Rng& r) : mode(static_cast<int>(r.uni(0, 3))), common(static_cast<int>(r.uni(1, 3))) {}
  int operator()(Rng& r) const { return mode <= 1 ? 0 : mode == 2 ? common : static_cast<int>(r.uni(0, 3)); }
};

// ------------------------------------------------------------ references

struct AdamK { float b1, c1, b2, c2, bc1, bc2, lr, eps; };
AdamK adam_k(const zr_adam& h) {
  const double t = static_cast<double>(h.step);
  return AdamK{static_cast<float>(h.beta1), static_cast<float>(1.0 - h.beta1),
               static_cast<float>(h.beta2), static_cast<float>(1.0 - h.beta2),
               static_cast<float>(1.0 - std::pow(h.beta1, t)),
               static_cast<float>(1.0 - std::pow(h.beta2, t)),
               static_cast<float>(h.lr), static_cast<float>(h.eps)};
}
void adam_ref(const AdamK& k, float g, float& th, float& m, float& v) {
  const float m1 = k.b1 * m + k.c1 * g;
  const float gg = g * g;
  const float v1 = k.b2 * v + k.c2 * gg;
  const float mh = m1 / k.bc1;
  const float vh = v1 / k.bc2;
  const float den = std::sqrt(vh) + k.eps;
  th = th - (k.lr * mh) / den;
  m = m1;
  v = v1;
}

struct Plan {
  zr_plan* h = nullptr;
  std::vector<int64_t> numels;
  std::vector<int32_t> pg;
  std::vector<zr_group> groups;
  int64_t B = 0, nb = 0;
  ~Plan() { zr_plan_free(h); }
};

bool make_plan(Rng& r, Plan& pl, int max_elems) {
  const int ng = static_cast<int>(r.uni(1, 2));
  for (int g = 0; g < ng; ++g) {
    const int R = static_cast<int>(r.pick(std::vector<int64_t>{1, 2, 3, 4, 5, 6, 8, 8, 16, 17}));
    std::vector<int> sps;
    for (int d = 1; d <= 4; ++d) if (R % d == 0) sps.push_back(d);
    pl.groups.push_back(zr_group{R, sps[r.next() % sps.size()]});
  }
  const int n = static_cast<int>(r.uni(1, 9));
  for (int i = 0; i < n; ++i) {
    const int64_t kind = r.uni(0, 3);
    pl.numels.push_back(kind == 0 ? r.uni(1, 5) : kind == 1 ? r.uni(6, 700) : r.uni(701, max_elems));
    pl.pg.push_back(static_cast<int32_t>(r.uni(0, ng - 1)));
  }
  pl.B = r.pick(std::vector<int64_t>{1, 7, 100, 1000, 4096, 5000, int64_t(1) << 40});
  const int64_t align = r.pick(std::vector<int64_t>{1, 1, 2, 4, 8});
  std::vector<zr_param> ps;
  for (int i = 0; i < n; ++i) ps.push_back(zr_param{pl.numels[i], pl.pg[i]});
  if (zr_plan_buckets(ps.data(), n, pl.groups.data(), ng, pl.B, 0, align, &pl.h) != ZR_OK) {
    std::fprintf(stderr, "plan failed: %s\n", zr_last_error());
    return false;
  }
  zr_plan_num_buckets(pl.h, &pl.nb);
  return true;
}

struct GI { int64_t T, L, P; float D; int R; };
GI ginfo(const Plan& pl, int g) {
  GI gi{};
  zr_plan_group_info(pl.h, g, &gi.T, &gi.L, &gi.P, &gi.D);
  gi.R = pl.groups[g].world;
  return gi;
}

// ------------------------------------------------------------ reduce cases

void reduce_case(Rng& r, int seed) {
  const Offsets off(r);
  Plan pl;
  if (!make_plan(r, pl, 9000)) { ++g_failures; return; }
  const int g = static_cast<int>(r.uni(0, static_cast<int64_t>(pl.groups.size()) - 1));
  const GI gi = ginfo(pl, g);
  if (gi.T == 0) return;
  const bool bf16 = r.uni(0, 1) == 1;
  const size_t es = bf16 ? 2 : 4;
  const int dst = r.uni(0, 2) == 0 ? -1 : static_cast<int>(r.uni(0, gi.R - 1));
  // selection: every bucket, one bucket, or a range
  int64_t first = 0, last = pl.nb;
  const int mode = static_cast<int>(r.uni(0, 2));
  if (mode == 1) { first = r.uni(0, pl.nb - 1); last = first + 1; }
  if (mode == 2) { first = r.uni(0, pl.nb - 1); last = r.uni(first, pl.nb); }
  const bool fused = r.uni(0, 1) == 1;
  const bool noalloc = fused && r.uni(0, 3) == 0 && mode != 2;
  // the grid-capped fused call (a grid-stride walk of the tiles)
  const int32_t cap = fused && !noalloc && mode != 2 && r.uni(0, 4) == 0
                          ? static_cast<int32_t>(r.uni(1, 40)) : 0;
  // replicas: the whole flat space, or (one destination) its window
  const bool window = dst >= 0 && r.uni(0, 1) == 1;
  const int64_t base = window ? std::min<int64_t>(dst * gi.P, gi.T) : 0;
  const int64_t len = window ? std::max<int64_t>(0, std::min<int64_t>(gi.P, gi.T - dst * gi.P)) : gi.T;
  std::vector<Buf*> reps;
  std::vector<zr_replica> zreps;
  for (int q = 0; q < gi.R; ++q) {
    Buf* b = new Buf(static_cast<size_t>(std::max<int64_t>(len, 1)), es, off(r));
    for (int64_t i = 0; i < len; ++i) {
      const float x = r.normal(1.0f);
      if (bf16) b->h()[i] = bf16_of(x); else b->f()[i] = x;
    }
    reps.push_back(b);
    zreps.push_back(zr_replica{b->p, base, len});
  }
  auto xval = [&](int q, int64_t f) -> float {
    const int64_t i = f - base;
    return bf16 ? bits_f(static_cast<uint32_t>(reps[q]->h()[i]) << 16) : reps[q]->f()[i];
  };
  // which partition elements the call writes, and their reduced gradient
  const int nd = dst < 0 ? gi.R : 1;
  const int64_t span = gi.P;
  std::vector<std::vector<float>> want(nd, std::vector<float>(span, 0.0f));
  std::vector<std::vector<char>> written(nd, std::vector<char>(span, 0));
  const zr_slice* sl = nullptr;
  int64_t nsl = 0;
  zr_plan_slices(pl.h, -1, &sl, &nsl);
  for (int64_t i = 0; i < nsl; ++i) {
    const zr_slice& s = sl[i];
    if (s.group != g || s.bucket < first || s.bucket >= last || (dst >= 0 && s.dst != dst)) continue;
    const int d = dst < 0 ? s.dst : 0;
    for (int64_t j = 0; j < s.numel; ++j) {
      float acc = xval(0, s.flat_offset + j);
      if (gi.R > 1) acc = acc / gi.D;
      for (int q = 1; q < gi.R; ++q) acc = acc + xval(q, s.flat_offset + j) / gi.D;
      CHECK(!written[d][s.part_offset + j], "seed %d: element covered by two slices", seed);
      want[d][s.part_offset + j] = acc;
      written[d][s.part_offset + j] = 1;
    }
  }
  if (first < last && last == pl.nb)           // padding of the selected partitions
    for (int d = 0; d < nd; ++d) {
      const int k = dst < 0 ? d : dst;
      for (int64_t j = std::max<int64_t>(0, gi.T - k * gi.P); j < gi.P; ++j) {
        want[d][j] = 0.0f;
        written[d][j] = 1;
      }
    }
  const uint32_t kUntouched = 0x7fc0dead;     // a NaN no kernel writes
  zr_status st;
  std::vector<Buf*> outs;
  if (!fused) {
    std::vector<float*> po;
    for (int d = 0; d < nd; ++d) {
      Buf* b = new Buf(static_cast<size_t>(span), 4, off(r));
      for (int64_t j = 0; j < span; ++j) std::memcpy(b->f() + j, &kUntouched, 4);
      outs.push_back(b);
      po.push_back(b->f());
    }
    const zr_dtype dt = bf16 ? ZR_BF16 : ZR_FP32;
    zr_emu_lds_max = 0;
    st = mode == 2 ? zr_reduce_scatter_local_range(pl.h, g, first, last - first, dst, zreps.data(), dt, po.data(), nullptr)
                   : zr_reduce_scatter_local(pl.h, g, mode == 0 ? -1 : first, dst, zreps.data(), dt, po.data(), nullptr);
    CHECK(st == ZR_OK, "seed %d: reduce failed: %s", seed, zr_last_error());
    check_lds(seed, nd, span, written, want_wgs_per_cu(bf16, false, gi.R));
    for (int d = 0; d < nd; ++d) {
      for (int64_t j = 0; j < span; ++j) {
        const uint32_t got = f_bits(outs[d]->f()[j]);
        if (written[d][j])
          CHECK(got == f_bits(want[d][j]), "seed %d: reduced [%d][%lld] %08x want %08x", seed, d,
                (long long)j, got, f_bits(want[d][j]));
        else
          CHECK(got == kUntouched, "seed %d: element [%d][%lld] outside the selection written", seed, d,
                (long long)j);
      }
      CHECK(outs[d]->guard_intact(), "seed %d: store before a partition output", seed);
    }
  } else {
    const int64_t n = dst < 0 ? gi.L : gi.P;
    Buf th(static_cast<size_t>(n), 4, off(r));
    Buf m(static_cast<size_t>(n), 4, off(r));
    Buf v(static_cast<size_t>(n), 4, off(r));
    const bool with_pb = r.uni(0, 3) != 0, with_go = r.uni(0, 1) == 1;
    Buf pb(static_cast<size_t>(n), 2, off(r));
    Buf go(static_cast<size_t>(n), 4, off(r));
    std::vector<float> th0(n), m0(n), v0(n);
    for (int64_t j = 0; j < n; ++j) {
      th0[j] = r.normal(0.02f); m0[j] = r.normal(1e-3f); v0[j] = std::fabs(r.normal(1e-6f));
      th.f()[j] = th0[j]; m.f()[j] = m0[j]; v.f()[j] = v0[j];
      pb.h()[j] = 0x7fc1;
      std::memcpy(go.f() + j, &kUntouched, 4);
    }
    const zr_adam h{1e-3, 0.9, 0.999, 1e-8, r.uni(1, 5)};
    const zr_dtype dt = bf16 ? ZR_BF16 : ZR_FP32;
    uint16_t* pbp = with_pb ? pb.h() : nullptr;
    float* gop = with_go ? go.f() : nullptr;
    zr_emu_lds_max = 0;
    if (mode == 2)
      st = zr_reduce_scatter_adam_range(pl.h, g, first, last - first, dst, zreps.data(), dt, &h,
                                        th.f(), m.f(), v.f(), pbp, gop, nullptr);
    else if (noalloc)
      st = zr_reduce_scatter_adam_noalloc(pl.h, g, mode == 0 ? -1 : first, dst, zreps.data(), dt, &h,
                                          th.f(), m.f(), v.f(), pbp, gop, nullptr);
    else if (cap > 0)
      st = zr_reduce_scatter_adam_capped(pl.h, g, mode == 0 ? -1 : first, dst, zreps.data(), dt, &h,
                                         th.f(), m.f(), v.f(), pbp, gop, cap, nullptr);
    else
      st = zr_reduce_scatter_adam(pl.h, g, mode == 0 ? -1 : first, dst, zreps.data(), dt, &h,
                                  th.f(), m.f(), v.f(), pbp, gop, nullptr);
    // the no-allocation call refuses selections beyond its staging array
    // (6,552 segments: the merged slices plus one padding segment per
    // selected partition that has padding), leaving every output untouched
    int64_t nseg = 0;
    for (int64_t i = 0; i < nsl; ++i)
      nseg += sl[i].group == g && sl[i].bucket >= first && sl[i].bucket < last &&
              (dst < 0 || sl[i].dst == dst);
    if (first < last && last == pl.nb)
      for (int d = 0; d < nd; ++d) nseg += (dst < 0 ? d : dst) * gi.P + gi.P > gi.T;
    if (noalloc && nseg > 6552) {
      CHECK(st == ZR_ERR_INVALID, "seed %d: oversized no-allocation call accepted", seed);
      for (int64_t e = 0; e < n; ++e)
        CHECK(f_bits(th.f()[e]) == f_bits(th0[e]) && pb.h()[e] == 0x7fc1 &&
                  f_bits(go.f()[e]) == kUntouched,
              "seed %d: refused call touched element %lld", seed, (long long)e);
      for (Buf* b : reps) delete b;
      return;
    }
    CHECK(st == ZR_OK, "seed %d: fused failed: %s", seed, zr_last_error());
    check_lds(seed, nd, span, written, cap <= 0 ? want_wgs_per_cu(bf16, true, gi.R) : 0);
    const AdamK k = adam_k(h);
    for (int d = 0; d < nd; ++d)
      for (int64_t j = 0; j < span; ++j) {
        const int64_t e = d * span + j;        // state index (dst = -1: partition d at d*P)
        float t1 = th0[e], m1 = m0[e], v1 = v0[e];
        if (written[d][j]) adam_ref(k, want[d][j], t1, m1, v1);
        CHECK(f_bits(th.f()[e]) == f_bits(t1) && f_bits(m.f()[e]) == f_bits(m1) &&
                  f_bits(v.f()[e]) == f_bits(v1),
              "seed %d: Adam state [%d][%lld] differs", seed, d, (long long)j);
        if (with_pb)
          CHECK(pb.h()[e] == (written[d][j] ? bf16_of(t1) : 0x7fc1), "seed %d: bf16 param [%lld]", seed,
                (long long)e);
        if (with_go) {
          const uint32_t got = f_bits(go.f()[e]);
          CHECK(got == (written[d][j] ? f_bits(want[d][j]) : kUntouched), "seed %d: grad_out [%lld]", seed,
                (long long)e);
        }
      }
    CHECK(th.guard_intact() && m.guard_intact() && v.guard_intact() && pb.guard_intact() &&
              go.guard_intact(),
          "seed %d: store before a state buffer", seed);
  }
  for (Buf* b : reps) { CHECK(b->guard_intact(), "seed %d: store before a replica", seed); delete b; }
  for (Buf* b : outs) delete b;
}

// --------------------------------------------------------------- IPG case

void ipg_case(Rng& r, int seed) {
  const Offsets off(r);
  Plan pl;
  if (!make_plan(r, pl, 9000)) { ++g_failures; return; }
  const int g = static_cast<int>(r.uni(0, static_cast<int64_t>(pl.groups.size()) - 1));
  const GI gi = ginfo(pl, g);
  std::vector<int64_t> ids;
  for (size_t p = 0; p < pl.numels.size(); ++p)
    if (pl.pg[p] == g && r.uni(0, 3) != 0) ids.push_back(static_cast<int64_t>(p));
  if (ids.empty() || gi.L == 0) return;
  const bool bf16 = r.uni(0, 1) == 1;
  // the step's first micro-batch: main_grad taken as +0 and not read
  const bool first = r.uni(0, 2) == 0;
  const int64_t wb = r.uni(0, gi.L - 1), wl = r.uni(0, gi.L - wb);
  Buf mg(static_cast<size_t>(std::max<int64_t>(wl, 1)), 4, off(r));
  std::vector<float> want(wl);
  for (int64_t i = 0; i < wl; ++i) { want[i] = r.normal(1.0f); mg.f()[i] = want[i]; }
  std::vector<char> touched(static_cast<size_t>(wl), 0);
  std::vector<Buf*> gs;
  std::vector<const void*> ptrs;
  for (int64_t p : ids) {
    Buf* b = new Buf(static_cast<size_t>(pl.numels[p]), bf16 ? 2 : 4, off(r));
    int64_t off = 0;
    zr_plan_param_offset(pl.h, p, &off);
    for (int64_t i = 0; i < pl.numels[p]; ++i) {
      const float x = r.normal(1.0f);
      float w = x;
      if (bf16) { b->h()[i] = bf16_of(x); w = bits_f(static_cast<uint32_t>(b->h()[i]) << 16); }
      else b->f()[i] = x;
      const int64_t f = off + i;
      if (f >= wb && f < wb + wl) {
        // +0 + w, not w: a -0 gradient gives +0 into a zeroed buffer
        if (first && !touched[f - wb]) want[f - wb] = 0.0f;
        touched[f - wb] = 1;
        want[f - wb] = want[f - wb] + w;
      }
    }
    gs.push_back(b);
    ptrs.push_back(b->p);
  }
  const zr_status st =
      (first ? zr_ipg_accumulate_first : zr_ipg_accumulate)(
          pl.h, ids.data(), ptrs.data(), static_cast<int64_t>(ids.size()),
          bf16 ? ZR_BF16 : ZR_FP32, mg.f(), wb, wl, nullptr);
  CHECK(st == ZR_OK, "seed %d: ipg failed: %s", seed, zr_last_error());
  for (int64_t i = 0; i < wl; ++i)
    CHECK(f_bits(mg.f()[i]) == f_bits(want[i]), "seed %d: main_grad [%lld]", seed, (long long)i);
  CHECK(mg.guard_intact(), "seed %d: store before main_grad", seed);
  for (Buf* b : gs) delete b;
}

// -------------------------------------------------------------- copy case

void copy_case(Rng& r, int seed) {
  const Offsets off(r);
  Plan pl;
  if (!make_plan(r, pl, 9000)) { ++g_failures; return; }
  const int g = static_cast<int>(r.uni(0, static_cast<int64_t>(pl.groups.size()) - 1));
  const GI gi = ginfo(pl, g);
  const int64_t b = r.uni(0, pl.nb - 1);
  const int dst = static_cast<int>(r.uni(0, gi.R - 1));
  const zr_slice* sl = nullptr;
  int64_t nsl = 0;
  zr_plan_slices(pl.h, b, &sl, &nsl);
  int64_t need = 0;
  for (int64_t i = 0; i < nsl; ++i) need = std::max(need, sl[i].bucket_offset + sl[i].numel);
  Buf src(static_cast<size_t>(std::max<int64_t>(need, 1)), 4, off(r));
  for (int64_t i = 0; i < need; ++i) src.f()[i] = r.normal(1.0f);
  Buf out(static_cast<size_t>(std::max<int64_t>(gi.P, 1)), 4, off(r));
  const uint32_t kUntouched = 0x7fc0beef;
  for (int64_t j = 0; j < gi.P; ++j) std::memcpy(out.f() + j, &kUntouched, 4);
  std::vector<uint32_t> want(gi.P, kUntouched);
  for (int64_t i = 0; i < nsl; ++i)
    if (sl[i].group == g && sl[i].dst == dst)
      for (int64_t j = 0; j < sl[i].numel; ++j) want[sl[i].part_offset + j] = f_bits(src.f()[sl[i].bucket_offset + j]);
  const zr_status st = zr_copy_grads_in_partition(pl.h, g, b, dst, src.f(), out.f(), nullptr);
  CHECK(st == ZR_OK, "seed %d: copy failed: %s", seed, zr_last_error());
  for (int64_t j = 0; j < gi.P; ++j) CHECK(f_bits(out.f()[j]) == want[j], "seed %d: copy [%lld]", seed, (long long)j);
  CHECK(out.guard_intact(), "seed %d: store before the copy output", seed);
}

// -------------------------------------------------------- all-gather case

void gather_case(Rng& r, int seed) {
  const Offsets off(r);
  Plan pl;
  if (!make_plan(r, pl, 9000)) { ++g_failures; return; }
  const int g = static_cast<int>(r.uni(0, static_cast<int64_t>(pl.groups.size()) - 1));
  const GI gi = ginfo(pl, g);
  if (gi.T == 0) return;
  const bool bf16 = r.uni(0, 1) == 1;
  const size_t es = bf16 ? 2 : 4;
  std::vector<Buf*> parts;
  std::vector<const void*> pp;
  for (int k = 0; k < gi.R; ++k) {
    Buf* b = new Buf(static_cast<size_t>(std::max<int64_t>(gi.P, 1)), es, off(r));
    for (int64_t j = 0; j < gi.P; ++j) {
      if (bf16) b->h()[j] = static_cast<uint16_t>(r.next()); else b->f()[j] = r.normal(1.0f);
    }
    parts.push_back(b);
    pp.push_back(b->p);
  }
  const int64_t ob = r.uni(0, gi.T - 1), ol = r.uni(0, gi.T - ob);
  Buf out(static_cast<size_t>(std::max<int64_t>(ol, 1)), es, off(r));
  const zr_status st = zr_all_gather_params(pl.h, g, pp.data(), bf16 ? ZR_BF16 : ZR_FP32, out.p, ob, ol, nullptr);
  CHECK(st == ZR_OK, "seed %d: all-gather failed: %s", seed, zr_last_error());
  for (int64_t i = 0; i < ol; ++i) {
    const int64_t f = ob + i, k = f / gi.P, j = f % gi.P;
    if (bf16) CHECK(out.h()[i] == parts[k]->h()[j], "seed %d: gather [%lld]", seed, (long long)i);
    else CHECK(f_bits(out.f()[i]) == f_bits(parts[k]->f()[j]), "seed %d: gather [%lld]", seed, (long long)i);
  }
  CHECK(out.guard_intact(), "seed %d: store before the gather output", seed);
  for (Buf* b : parts) delete b;
}

// ------------------------------------------------------------- ring cases

void ring_case(Rng& r, int seed) {
  const Offsets off(r);
  const int n = static_cast<int>(r.uni(2, 8));
  const int64_t C = r.uni(0, 3000);
  const int step = static_cast<int>(r.uni(0, n - 2));
  const bool ag = r.uni(0, 1) == 1;
  std::vector<Buf*> bufs;
  std::vector<float*> bp;
  std::vector<std::vector<float>> before(n);
  for (int k = 0; k < n; ++k) {
    Buf* b = new Buf(static_cast<size_t>(std::max<int64_t>(n * C, 1)), 4, off(r));
    for (int64_t i = 0; i < n * C; ++i) b->f()[i] = r.normal(1.0f);
    before[k].assign(b->f(), b->f() + n * C);
    bufs.push_back(b);
    bp.push_back(b->f());
  }
  const zr_status st = ag ? zr_ring_ag_step(bp.data(), n, C, step, nullptr)
                          : zr_ring_rs_step(bp.data(), n, C, step, nullptr);
  CHECK(st == ZR_OK, "seed %d: ring failed: %s", seed, zr_last_error());
  for (int k = 0; k < n; ++k) {
    const int lag = ag ? 1 : 2;
    const int c = (((k - step - lag) % n) + n) % n;
    const int prev = k == 0 ? n - 1 : k - 1;
    for (int64_t i = 0; i < n * C; ++i) {
      float want = before[k][i];
      if (i / std::max<int64_t>(C, 1) == c && C > 0)
        want = ag ? before[prev][i] : before[k][i] + before[prev][i];
      CHECK(f_bits(bufs[k]->f()[i]) == f_bits(want), "seed %d: ring rank %d [%lld]", seed, k, (long long)i);
    }
    CHECK(bufs[k]->guard_intact(), "seed %d: store before a rank buffer", seed);
  }
  for (Buf* b : bufs) delete b;
}

// ------------------------------------------------------------- Adam case

void adam_case(Rng& r, int seed) {
  const Offsets off(r);
  const int64_t n = r.pick(std::vector<int64_t>{0, 1, 3, 511, 512, 513, r.uni(1, 20000)});
  Buf g(static_cast<size_t>(std::max<int64_t>(n, 1)), 4, off(r));
  Buf th(static_cast<size_t>(std::max<int64_t>(n, 1)), 4, off(r));
  Buf m(static_cast<size_t>(std::max<int64_t>(n, 1)), 4, off(r));
  Buf v(static_cast<size_t>(std::max<int64_t>(n, 1)), 4, off(r));
  Buf pb(static_cast<size_t>(std::max<int64_t>(n, 1)), 2, off(r));
  std::vector<float> t1(n), m1(n), v1(n);
  for (int64_t i = 0; i < n; ++i) {
    g.f()[i] = r.normal(1e-3f);
    t1[i] = th.f()[i] = r.normal(0.02f);
    m1[i] = m.f()[i] = r.normal(1e-4f);
    v1[i] = v.f()[i] = std::fabs(r.normal(1e-8f));
  }
  const zr_adam h{1e-3, 0.9, 0.999, 1e-8, r.uni(1, 9)};
  const bool with_pb = r.uni(0, 1) == 1;
  const zr_status st = zr_adam_partition(&h, g.f(), th.f(), m.f(), v.f(), with_pb ? pb.h() : nullptr, n, nullptr);
  CHECK(st == ZR_OK, "seed %d: adam failed: %s", seed, zr_last_error());
  const AdamK k = adam_k(h);
  for (int64_t i = 0; i < n; ++i) {
    adam_ref(k, g.f()[i], t1[i], m1[i], v1[i]);
    CHECK(f_bits(th.f()[i]) == f_bits(t1[i]) && f_bits(m.f()[i]) == f_bits(m1[i]) &&
              f_bits(v.f()[i]) == f_bits(v1[i]),
          "seed %d: Adam [%lld]", seed, (long long)i);
    if (with_pb) CHECK(pb.h()[i] == bf16_of(t1[i]), "seed %d: Adam bf16 [%lld]", seed, (long long)i);
  }
  CHECK(th.guard_intact() && m.guard_intact() && v.guard_intact() && pb.guard_intact(),
        "seed %d: store before an Adam buffer", seed);
}

}  // namespace

int main(int argc, char** argv) {
  const int cases = argc > 1 ? std::atoi(argv[1]) : 200;
  const int first = argc > 2 ? std::atoi(argv[2]) : 0;
  for (int c = first; c < first + cases; ++c) {
    Rng r(static_cast<uint64_t>(c));
    switch (c % 8) {
      case 0: case 1: case 2: reduce_case(r, c); break;
      case 3: ipg_case(r, c); break;
      case 4: copy_case(r, c); break;
      case 5: gather_case(r, c); break;
      case 6: ring_case(r, c); break;
      case 7: adam_case(r, c); break;
    }
  }
  if (g_failures) {
    std::printf("kernel emulation: %d failures\n", g_failures);
    return 1;
  }
  std::printf("kernel emulation ok: %d cases, %lld launches\n", cases, zr_emu_launches);
  for (const auto& kv : zr_emu_coverage()) std::printf("launches %lld %s\n", kv.second, kv.first.c_str());
  return 0;
}
