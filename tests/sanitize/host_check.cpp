// Host-side check of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).
//
// Built by tests/test_host_sanitize.py with g++ together with csrc/gdr_api.cpp and stub definitions of
// the kernel launchers and of the few HIP runtime calls the host code makes. Valid calls therefore run
// the whole host path (validation, workspace carving, segment planning, launch order, timing) and the
// stubs check what the launchers receive: every pointer into the workspace must lie inside it. Invalid
// calls must fail before any launch. Exit status 0 and the line "host_check OK" mean every case passed.
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "gdr.h"
#include "gdr_internal.h"

// ------------------------------------------------------------------ stubs
static std::vector<std::string> g_launches;
static uintptr_t g_ws_lo = 0, g_ws_hi = 0;   // the workspace of the call under test

static void fail_here(const char* what) {
  std::fprintf(stderr, "host_check FAILED: %s\n", what);
  std::exit(1);
}
static void in_ws(const void* p, size_t bytes, const char* what) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  if (!p || a < g_ws_lo || a + bytes > g_ws_hi) fail_here(what);
}

namespace gdr {
hipError_t launch_prep(const PrepParams& p, int, int, hipStream_t) {
  g_launches.push_back("prep");
  in_ws(p.ws, 1, "prep records");
  if (p.chunk_list) in_ws(p.chunk_list, 4, "chunk list");
  return hipSuccess;
}
static void check_scan(const ScanParams& p) {
  if (p.row_order) {   // the rows longest first: only without segments, after the chunk list
    if (p.P != 1) fail_here("row order with segments");
    in_ws(p.row_order, size_t(p.B) * 4, "row order");
  }
  if (p.P > 1) {
    in_ws(p.seg, size_t(p.B) * p.Hv * p.P * kSlotFloats * 4, "segment slots");
    in_ws(p.status, 4, "status word");
    in_ws(p.plan, size_t(p.B) * p.Hv * p.P * sizeof(PlanEntry), "plan entries");
    in_ws(p.cert, size_t(p.B) * p.Hv * p.P * kCertFloats * 4, "certificate parts");
  }
}
hipError_t launch_transition(const ScanParams& p, hipStream_t) { g_launches.push_back("transition"); check_scan(p); return hipSuccess; }
hipError_t launch_combine(const ScanParams& p, hipStream_t) { g_launches.push_back("combine"); check_scan(p); return hipSuccess; }
hipError_t launch_scan(const ScanParams& p, int, hipStream_t) { g_launches.push_back("scan"); check_scan(p); return hipSuccess; }
hipError_t launch_finalize(const ScanParams& p, hipStream_t) { g_launches.push_back("finalize"); check_scan(p); return hipSuccess; }
hipError_t launch_decode(const DecodeParams&, int, int, hipStream_t) { g_launches.push_back("decode"); return hipSuccess; }
hipError_t launch_gates(const GatesParams&, int, hipStream_t) { g_launches.push_back("gates"); return hipSuccess; }
hipError_t launch_conv_silu(const ConvParams&, int, hipStream_t) { g_launches.push_back("conv"); return hipSuccess; }
hipError_t launch_gated_rmsnorm(const NormParams&, int, hipStream_t) { g_launches.push_back("norm"); return hipSuccess; }
static unsigned char g_fake_scratch_tag;
hipError_t noalloc_scratch(void** out) {
  *out = reinterpret_cast<void*>(uintptr_t(1) << 44);   // a fake, 256-byte aligned device address
  (void)g_fake_scratch_tag;
  return hipSuccess;
}
}  // namespace gdr

static int g_events = 0;
extern "C" {
hipError_t hipEventCreate(hipEvent_t* e) { *e = reinterpret_cast<hipEvent_t>(uintptr_t(0x1000 + 16 * ++g_events)); return hipSuccess; }
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
hipError_t hipEventSynchronize(hipEvent_t) { return hipSuccess; }
hipError_t hipEventElapsedTime(float* ms, hipEvent_t, hipEvent_t) { *ms = 0.5f; return hipSuccess; }
const char* hipGetErrorString(hipError_t) { return "stub"; }
}

// ------------------------------------------------------------------ cases
static int g_cases = 0;
static void expect(bool ok, const char* what) {
  ++g_cases;
  if (!ok) {
    std::fprintf(stderr, "case failed: %s (last error: %s)\n", what, gdr_last_error());
    std::exit(1);
  }
}

struct Fake {   // fake device addresses, far apart, 256-byte aligned
  uintptr_t next = uintptr_t(1) << 32;
  void* take(size_t bytes) {
    void* p = reinterpret_cast<void*>(next);
    next += (bytes + 4095) / 4096 * 4096 + 4096;
    return p;
  }
};

struct Call {
  gdr_desc d{};
  void *q, *k, *v, *g, *beta, *len, *s0, *s0_row, *o, *sf, *ws;
  size_t ws_bytes;
  Call(int B, int L, int Hk, int Hv, bool bf16, bool lengths, bool with_s0) {
    Fake f;
    d = gdr_desc{B, L, Hk, Hv, 128, 128, with_s0 ? B : 0, bf16 ? GDR_BF16 : GDR_F32, GDR_F32};
    const size_t e = bf16 ? 2 : 4, BL = size_t(B) * L;
    q = f.take(BL * Hk * 128 * e);
    k = f.take(BL * Hk * 128 * e);
    v = f.take(BL * Hv * 128 * e);
    g = f.take(BL * Hv * 4);
    beta = f.take(BL * Hv * 4);
    len = lengths ? f.take(size_t(B) * 4) : nullptr;
    s0 = with_s0 ? f.take(size_t(B) * Hv * 128 * 128 * 4) : nullptr;
    s0_row = nullptr;
    o = f.take(BL * Hv * 128 * e);
    sf = f.take(size_t(B) * Hv * 128 * 128 * 4);
    ws_bytes = gdr_prefill_workspace_size(&d);
    ws = f.take(ws_bytes);
  }
  gdr_status check() const {
    return gdr_prefill_check(&d, q, k, v, static_cast<float*>(g), beta, static_cast<int32_t*>(len),
                             static_cast<float*>(s0), static_cast<int32_t*>(s0_row), o, static_cast<float*>(sf), ws,
                             ws_bytes);
  }
  gdr_status run() {
    g_launches.clear();
    g_ws_lo = reinterpret_cast<uintptr_t>(ws);
    g_ws_hi = g_ws_lo + ws_bytes;
    return gdr_prefill(&d, q, k, v, static_cast<float*>(g), beta, static_cast<int32_t*>(len), static_cast<float*>(s0),
                       static_cast<int32_t*>(s0_row), o, static_cast<float*>(sf), ws, ws_bytes, nullptr);
  }
};

static std::string order() {
  std::string s;
  for (const auto& l : g_launches) s += (s.empty() ? "" : ",") + l;
  return s;
}

int main() {
  // valid calls: the whole host path, launches in order, workspace pointers inside the workspace
  {
    Call c(1, 16384, 16, 32, true, false, false);   // the long prefill: 8 segments
    expect(c.check() == GDR_OK, "long prefill valid");
    expect(c.run() == GDR_OK && order() == "prep,transition,combine,scan,finalize", "long prefill launch order");
    expect(gdr_prefill_status_offset(&c.d) != size_t(-1) && gdr_prefill_status_offset(&c.d) < c.ws_bytes, "status offset");
  }
  {
    Call c(64, 1024, 16, 32, true, true, true);   // forks: one segment, chunk list
    expect(c.run() == GDR_OK && order() == "prep,scan", "forks launch order");
    expect(gdr_prefill_status_offset(&c.d) == size_t(-1), "no status without segments");
  }
  {
    Call c(2, 300, 2, 4, false, true, true);   // float32
    expect(c.run() == GDR_OK && order() == "prep,scan", "float32 launch order");
  }
  {
    Call c(1, 200, 1, 2, true, true, true);   // short bf16 with segments, in-place state
    c.sf = c.s0;
    expect(c.run() == GDR_OK && order() == "prep,transition,combine,scan,finalize", "in place with segments");
  }
  // timing: events recorded around each launch and read back
  {
    Call c(1, 4096, 4, 8, true, false, false);
    gdr_timing_enable(1);
    expect(c.run() == GDR_OK, "timed call");
    double ms[GDR_KERNEL_COUNT];
    int64_t n[GDR_KERNEL_COUNT];
    expect(gdr_timing_read(ms, n, GDR_KERNEL_COUNT) == GDR_OK && n[GDR_KERNEL_PREP] == 1 && n[GDR_KERNEL_SCAN] == 1,
           "timing read");
    gdr_timing_enable(0);
  }
  // invalid calls: rejected before any launch
  {
    Call c(2, 130, 2, 4, true, true, true);
    auto rejected = [&](const char* what) {
      g_launches.clear();
      const gdr_status st = c.run();
      expect(st != GDR_OK && g_launches.empty() && std::strlen(gdr_last_error()) > 0, what);
    };
    void* keep = c.q;
    c.q = nullptr; rejected("null q"); c.q = keep;
    c.q = static_cast<char*>(keep) + 8; rejected("misaligned q"); c.q = keep;
    keep = c.o; c.o = c.v; rejected("o overlaps v"); c.o = keep;
    const size_t wb = c.ws_bytes; c.ws_bytes = wb - 1; rejected("small workspace"); c.ws_bytes = wb;
    c.d.Dk = 64; rejected("Dk 64"); c.d.Dk = 128;
    c.d.Hk = 3; rejected("Hv % Hk"); c.d.Hk = 2;
    c.d.qkv_dtype = 7; rejected("bad dtype"); c.d.qkv_dtype = GDR_BF16;
    c.s0_row = c.len; c.sf = c.s0; rejected("s_final aliases s0 with s0_row"); c.s0_row = nullptr;
  }
  expect(gdr_prefill_workspace_size(nullptr) == size_t(-1), "null desc");
  // the entry that allocates nothing: oversized shapes rejected, small ones run on the fixed array
  {
    Call c(4, 16384, 16, 32, true, false, false);
    g_launches.clear();
    expect(gdr_prefill_noalloc(&c.d, c.q, c.k, c.v, static_cast<float*>(c.g), c.beta, nullptr, nullptr, nullptr, c.o,
                               static_cast<float*>(c.sf), nullptr) == GDR_EUNSUPPORTED && g_launches.empty(),
           "noalloc oversized");
    Call s(1, 2048, 4, 8, true, false, false);
    g_launches.clear();
    g_ws_lo = uintptr_t(1) << 44;
    g_ws_hi = g_ws_lo + (size_t(128) << 20);
    expect(gdr_prefill_noalloc(&s.d, s.q, s.k, s.v, static_cast<float*>(s.g), s.beta, nullptr, nullptr, nullptr, s.o,
                               static_cast<float*>(s.sf), nullptr) == GDR_OK &&
               order() == "prep,transition,combine,scan,finalize",
           "noalloc small");
  }
  // decode and the layer steps: valid and invalid
  {
    Call c(64, 1, 16, 32, true, false, true);
    g_launches.clear();
    expect(gdr_decode(&c.d, c.q, c.k, c.v, static_cast<float*>(c.g), c.beta, nullptr, static_cast<float*>(c.s0), nullptr,
                      c.o, static_cast<float*>(c.s0), nullptr) == GDR_OK && order() == "decode",
           "decode in place");
    g_launches.clear();
    expect(gdr_decode(&c.d, nullptr, c.k, c.v, static_cast<float*>(c.g), c.beta, nullptr, nullptr, nullptr, c.o, nullptr,
                      nullptr) != GDR_OK && g_launches.empty(),
           "decode null q");
  }
  {
    Fake f;
    void* b = f.take(4096); void* a = f.take(4096); void* Al = f.take(64); void* dt = f.take(64);
    void* be = f.take(4096); void* gg = f.take(8192);
    g_launches.clear();
    expect(gdr_gates(1, 64, 16, GDR_F32, b, a, static_cast<float*>(Al), static_cast<float*>(dt), nullptr, be,
                     static_cast<float*>(gg), nullptr) == GDR_OK && order() == "gates", "gates");
    expect(gdr_gates(1, 64, 16, GDR_F32, b, a, static_cast<float*>(Al), static_cast<float*>(dt), nullptr, b,
                     static_cast<float*>(gg), nullptr) == GDR_EINVAL, "gates overlap");
    const size_t Cm = (2 * 1 + 2) * 128;
    void* mixed = f.take(64 * Cm * 2); void* w = f.take(Cm * 4 * 4);
    void* qq = f.take(64 * 128 * 2); void* kk = f.take(64 * 128 * 2); void* vv = f.take(64 * 256 * 2);
    void* tail = f.take(3 * Cm * 2);
    g_launches.clear();
    expect(gdr_conv_silu(1, 64, 1, 2, 4, GDR_BF16, mixed, tail, static_cast<float*>(w), nullptr, qq, kk, vv, tail,
                         nullptr) == GDR_OK && order() == "conv", "conv in-place tail");
    expect(gdr_conv_silu(1, 64, 1, 2, 9, GDR_BF16, mixed, tail, static_cast<float*>(w), nullptr, qq, kk, vv, tail,
                         nullptr) == GDR_EUNSUPPORTED, "conv K 9");
    void* x = f.take(1024 * 256); void* z = f.take(1024 * 256); void* nw = f.take(512);
    g_launches.clear();
    expect(gdr_gated_rmsnorm(1024, GDR_BF16, x, z, static_cast<float*>(nw), 1e-6f, x, nullptr) == GDR_OK &&
               order() == "norm", "norm in place");
    expect(gdr_gated_rmsnorm(1024, GDR_BF16, x, z, static_cast<float*>(nw), -1.f, x, nullptr) == GDR_EINVAL, "norm eps");
  }
  expect(gdr_set_truncation(0) == GDR_OK && gdr_set_truncation(1) == GDR_OK, "truncation switch");
  expect(std::strcmp(gdr_kernel_name(GDR_KERNEL_FINALIZE), "gdr_finalize") == 0 && gdr_kernel_name(99)[0] == 0, "names");
  std::printf("host_check OK: %d cases\n", g_cases);
  return 0;
}
