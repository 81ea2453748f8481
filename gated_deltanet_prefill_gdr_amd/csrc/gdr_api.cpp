// C ABI of the chunked gated delta rule prefill (declared in include/gdr.h).
//
// Host side only: argument validation (no GPU call before every host-checkable argument has
// passed), workspace sizing, the kernel launches on the caller's stream, and optional
// per-kernel HIP-event timing for benchmarks.
#include "gdr.h"

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <climits>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "gdr_internal.h"

namespace {

thread_local std::string g_last_error;

gdr_status fail(gdr_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

size_t dtype_size(int dt) { return dt == GDR_BF16 ? 2 : 4; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Range {
  const char* name;
  uintptr_t lo, hi;   // [lo, hi)
};

Range range(const char* name, const void* p, size_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{name, lo, p ? lo + bytes : lo};
}

bool overlap(const Range& a, const Range& b) {
  return a.lo != a.hi && b.lo != b.hi && a.lo < b.hi && b.lo < a.hi;
}

int num_chunks(int L) { return (L + gdr::kChunk - 1) / gdr::kChunk; }

gdr_status check_desc(const gdr_desc* d) {
  if (!d) return fail(GDR_EINVAL, "desc is NULL");
  if (d->B < 0 || d->L < 0) return fail(GDR_EINVAL, "B (%d) and L (%d) must be >= 0", d->B, d->L);
  if (d->Hk <= 0 || d->Hv <= 0) return fail(GDR_EINVAL, "Hk (%d) and Hv (%d) must be > 0", d->Hk, d->Hv);
  if (d->Hv % d->Hk) return fail(GDR_EINVAL, "Hv (%d) must be a multiple of Hk (%d)", d->Hv, d->Hk);
  if (d->qkv_dtype != GDR_F32 && d->qkv_dtype != GDR_BF16)
    return fail(GDR_EINVAL, "qkv_dtype %d is not a gdr_dtype", d->qkv_dtype);
  if (d->beta_dtype != GDR_F32 && d->beta_dtype != d->qkv_dtype)
    return fail(GDR_EINVAL, "beta_dtype must be GDR_F32 or qkv_dtype");
  if (d->Dk != gdr::kHeadDim || d->Dv != gdr::kHeadDim)
    return fail(GDR_EUNSUPPORTED, "Dk = %d, Dv = %d: only Dk = Dv = 128 is built", d->Dk, d->Dv);
  if (d->Hv > 65535 || d->Hk > 65535 || d->B > 65535 || int64_t(d->B) * d->Hv * (gdr::kHeadDim / 16) > INT32_MAX ||
      int64_t(d->B) * d->Hv * num_chunks(d->L) > INT32_MAX)
    return fail(GDR_EUNSUPPORTED, "B, Hk, Hv <= 65535, B*Hv*8 < 2^31 and B*Hv*ceil(L/64) < 2^31 are required (grid limits)");
  if ((int64_t(d->L) + 2 * gdr::kChunk) * std::max(d->Hk, d->Hv) * gdr::kHeadDim * 4 >= (int64_t(1) << 32))
    return fail(GDR_EUNSUPPORTED, "(L + 128) * max(Hk, Hv) * 128 * 4 bytes must stay below 4 GiB per batch row");
  return GDR_OK;
}

gdr_status check_all(const gdr_desc* d, const void* q, const void* k, const void* v, const float* g,
                     const void* beta, const int32_t* lengths, const float* s0, const int32_t* s0_row,
                     const void* o, const float* s_final, const void* ws, size_t ws_bytes, bool need_ws = true,
                     const gdr_fusion* fu = nullptr) {
  gdr_status st = check_desc(d);
  if (st != GDR_OK) return st;
  const size_t B = d->B, L = d->L, Hk = d->Hk, Hv = d->Hv, Dd = gdr::kHeadDim;
  const size_t esz = dtype_size(d->qkv_dtype), bsz = dtype_size(d->beta_dtype);
  const bool any_tokens = B * L > 0;
  const bool fused_gates = fu && (fu->b_raw || fu->a_raw || fu->A_log || fu->dt_bias);
  const bool fused_norm = fu && (fu->z || fu->norm_w);
  if (fused_gates) {
    if (!fu->b_raw || !fu->a_raw || !fu->A_log || !fu->dt_bias)
      return fail(GDR_EINVAL, "fusion: b_raw, a_raw, A_log and dt_bias go together");
    if (g || beta) return fail(GDR_EINVAL, "fusion: g and beta must be NULL when the gate prologue is fused");
    if (!aligned(fu->b_raw, bsz) || !aligned(fu->a_raw, bsz) || !aligned(fu->A_log, 4) || !aligned(fu->dt_bias, 4))
      return fail(GDR_EINVAL, "fusion: b_raw, a_raw, A_log and dt_bias must be element-aligned");
  }
  if (fused_norm) {
    if (!fu->z || !fu->norm_w) return fail(GDR_EINVAL, "fusion: z and norm_w go together");
    if (!aligned(fu->z, 16) || !aligned(fu->norm_w, 16)) return fail(GDR_EINVAL, "fusion: z and norm_w must be 16-byte aligned");
    if (!(fu->norm_eps >= 0.f) || fu->norm_eps > 1e30f) return fail(GDR_EINVAL, "fusion: norm_eps must be finite and >= 0");
  }
  if (any_tokens) {
    if (!q || !k || !v || !o || (!fused_gates && (!g || !beta)))
      return fail(GDR_EINVAL, "q, k, v, g, beta and o must be non-NULL");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
      return fail(GDR_EINVAL, "q, k, v and o must be 16-byte aligned");
    if (!fused_gates && (!aligned(g, 4) || !aligned(beta, bsz))) return fail(GDR_EINVAL, "g and beta must be element-aligned");
  }
  if (s0_row && !s0) return fail(GDR_EINVAL, "s0_row given without s0");
  if (s0) {
    if (d->n_s0 < 1) return fail(GDR_EINVAL, "n_s0 must be >= 1 when s0 is given");
    if (!s0_row && size_t(d->n_s0) < B) return fail(GDR_EINVAL, "n_s0 (%d) < B (%d) with identity s0_row", d->n_s0, d->B);
    if (!aligned(s0, 16)) return fail(GDR_EINVAL, "s0 must be 16-byte aligned");
  }
  if (s_final && !aligned(s_final, 16)) return fail(GDR_EINVAL, "s_final must be 16-byte aligned");
  if (lengths && !aligned(lengths, 4)) return fail(GDR_EINVAL, "lengths must be 4-byte aligned");
  if (s0_row && !aligned(s0_row, 4)) return fail(GDR_EINVAL, "s0_row must be 4-byte aligned");
  if (s_final && s0 && reinterpret_cast<const void*>(s_final) == reinterpret_cast<const void*>(s0) && s0_row)
    return fail(GDR_EINVAL, "s_final may alias s0 only when s0_row is NULL");

  const size_t need = need_ws ? gdr_prefill_workspace_size(d) : 0;
  if (need > 0) {
    if (!ws) return fail(GDR_EWORKSPACE, "workspace is NULL, %zu bytes needed", need);
    if (ws_bytes < need) return fail(GDR_EWORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, need);
    if (!aligned(ws, 256)) return fail(GDR_EINVAL, "workspace must be 256-byte aligned");
  }

  const size_t state_bytes = Hv * Dd * Dd * sizeof(float);
  const Range inputs[] = {
      range("q", q, B * L * Hk * Dd * esz),   range("k", k, B * L * Hk * Dd * esz),
      range("v", v, B * L * Hv * Dd * esz),   range("g", g, g ? B * L * Hv * sizeof(float) : 0),
      range("beta", beta, beta ? B * L * Hv * bsz : 0),  range("lengths", lengths, lengths ? B * 4 : 0),
      range("s0", s0, s0 ? size_t(d->n_s0) * state_bytes : 0), range("s0_row", s0_row, s0_row ? B * 4 : 0),
      range("b_raw", fused_gates ? fu->b_raw : nullptr, B * L * Hv * bsz),
      range("a_raw", fused_gates ? fu->a_raw : nullptr, B * L * Hv * bsz),
      range("A_log", fused_gates ? fu->A_log : nullptr, Hv * 4),
      range("dt_bias", fused_gates ? fu->dt_bias : nullptr, Hv * 4),
      range("z", fused_norm ? fu->z : nullptr, B * L * Hv * Dd * esz),
      range("norm_w", fused_norm ? fu->norm_w : nullptr, Dd * 4),
  };
  const Range outs[] = {
      range("o", o, B * L * Hv * Dd * esz),
      range("s_final", s_final, s_final ? B * state_bytes : 0),
      range("workspace", ws, need),
  };
  for (const Range& out : outs) {
    for (const Range& in : inputs) {
      if (!overlap(out, in)) continue;
      if (std::strcmp(out.name, "s_final") == 0 && std::strcmp(in.name, "s0") == 0 && out.lo == in.lo) continue;
      return fail(GDR_EINVAL, "%s overlaps %s", out.name, in.name);
    }
  }
  for (size_t i = 0; i < 3; ++i)
    for (size_t j = i + 1; j < 3; ++j)
      if (overlap(outs[i], outs[j])) return fail(GDR_EINVAL, "%s overlaps %s", outs[i].name, outs[j].name);
  return GDR_OK;
}

// ---------------------------------------------------------------- timing
struct TimingRecord {
  int kernel;
  hipEvent_t start, stop;
};
bool g_timing = false;
bool g_truncation = true;
std::vector<TimingRecord> g_records;
std::vector<hipEvent_t> g_event_pool;

hipEvent_t take_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Launch through `launch` (returns hipError_t), bracketed by timing events when timing is on.
// Set while gdr_prefill_noalloc runs on this thread: no timing events (creating one may allocate).
thread_local bool t_no_alloc = false;

template <typename F>
hipError_t timed(int kernel, hipStream_t s, F&& launch) {
  TimingRecord rec{kernel, nullptr, nullptr};
  if (g_timing && !t_no_alloc) {
    rec.start = take_event();
    rec.stop = take_event();
    if (rec.start) (void)hipEventRecord(rec.start, s);
  }
  hipError_t e = launch();
  if (g_timing && !t_no_alloc && rec.start && rec.stop) {
    (void)hipEventRecord(rec.stop, s);
    g_records.push_back(rec);
  }
  return e;
}

const char* const kKernelNames[GDR_KERNEL_COUNT] = {"gdr_prep",   "gdr_scan",  "gdr_transition", "gdr_combine",
                                                    "gdr_decode", "gdr_gates", "gdr_conv_silu",  "gdr_gated_rmsnorm",
                                                    "gdr_finalize"};

bool bad_dtype(int dt) { return dt != GDR_F32 && dt != GDR_BF16; }

gdr_status check_overlaps(const Range* ins, size_t n_in, const Range* outs, size_t n_out,
                          const char* inplace_out = nullptr, const char* inplace_in = nullptr) {
  for (size_t o = 0; o < n_out; ++o) {
    for (size_t i = 0; i < n_in; ++i) {
      if (!overlap(outs[o], ins[i])) continue;
      if (inplace_out && std::strcmp(outs[o].name, inplace_out) == 0 && std::strcmp(ins[i].name, inplace_in) == 0 &&
          outs[o].lo == ins[i].lo)
        continue;
      return fail(GDR_EINVAL, "%s overlaps %s", outs[o].name, ins[i].name);
    }
    for (size_t j = o + 1; j < n_out; ++j)
      if (overlap(outs[o], outs[j])) return fail(GDR_EINVAL, "%s overlaps %s", outs[o].name, outs[j].name);
  }
  return GDR_OK;
}

}  // namespace

extern "C" {

size_t gdr_prefill_workspace_size(const gdr_desc* d) {
  if (check_desc(d) != GDR_OK) return size_t(-1);
  if (size_t(d->B) * d->L == 0) return 0;
  return gdr::workspace_bytes(d->B, d->Hv, num_chunks(d->L), dtype_size(d->qkv_dtype));
}

gdr_status gdr_prefill_check(const gdr_desc* d, const void* q, const void* k, const void* v, const float* g,
                             const void* beta, const int32_t* lengths, const float* s0, const int32_t* s0_row,
                             const void* o, const float* s_final, const void* ws, size_t ws_bytes) {
  return check_all(d, q, k, v, g, beta, lengths, s0, s0_row, o, s_final, ws, ws_bytes);
}

gdr_status gdr_prefill(const gdr_desc* d, const void* q, const void* k, const void* v, const float* g,
                       const void* beta, const int32_t* lengths, const float* s0, const int32_t* s0_row, void* o,
                       float* s_final, void* ws, size_t ws_bytes, void* stream) {
  return gdr_prefill_ex(d, q, k, v, g, beta, lengths, s0, s0_row, nullptr, o, s_final, ws, ws_bytes, stream);
}

gdr_status gdr_prefill_ex(const gdr_desc* d, const void* q, const void* k, const void* v, const float* g,
                          const void* beta, const int32_t* lengths, const float* s0, const int32_t* s0_row,
                          const gdr_fusion* fu, void* o, float* s_final, void* ws, size_t ws_bytes, void* stream) {
  gdr_status st = check_all(d, q, k, v, g, beta, lengths, s0, s0_row, o, s_final, ws, ws_bytes, true, fu);
  if (st != GDR_OK) return st;
  const bool fused_gates = fu && fu->b_raw;
  const bool fused_norm = fu && fu->z;
  if (d->B == 0) return GDR_OK;
  if (d->L == 0 && !s_final) return GDR_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int NC = num_chunks(d->L);
  const int bf16 = d->qkv_dtype == GDR_BF16;

  if (NC > 0) {
    gdr::PrepParams pp{q, k, g, beta, lengths, ws, d->B, d->L, d->Hk, d->Hv, NC};
    if (bf16 && lengths)
      pp.chunk_list = reinterpret_cast<int32_t*>(static_cast<char*>(ws) +
                                                 gdr::records_bytes(d->B, d->Hv, NC, dtype_size(d->qkv_dtype)) +
                                                 gdr::seg_bytes(d->B, d->Hv, NC, dtype_size(d->qkv_dtype)));
    if (fused_gates) {
      pp.b_raw = fu->b_raw;
      pp.a_raw = fu->a_raw;
      pp.A_log = fu->A_log;
      pp.dt_bias = fu->dt_bias;
    }
    hipError_t e = timed(GDR_KERNEL_PREP, s, [&] { return gdr::launch_prep(pp, bf16, d->beta_dtype == GDR_BF16, s); });
    if (e != hipSuccess) return fail(GDR_EHIP, "prep launch: %s", hipGetErrorString(e));
  }
  const gdr::SegPlan plan = gdr::seg_plan(d->B, d->Hv, NC, bf16);
  float* seg = plan.P > 1 ? reinterpret_cast<float*>(static_cast<char*>(ws) +
                                                     gdr::records_bytes(d->B, d->Hv, NC, dtype_size(d->qkv_dtype)))
                          : nullptr;
  gdr::ScanParams sp{q, k, v, lengths, s0, s0_row, o, s_final, NC > 0 ? ws : nullptr, seg,
                     d->B, d->L, d->Hk, d->Hv, NC, s0 ? d->n_s0 : 0, plan.P, plan.Ls};
  if (plan.P > 1) {   // truncated segment starts: plan, certificate parts and status in the workspace
    const size_t esz = dtype_size(d->qkv_dtype);
    char* tr = static_cast<char*>(ws) + gdr::trunc_offset(d->B, d->Hv, NC, esz);
    const size_t n = size_t(d->B) * d->Hv * plan.P;
    sp.status = reinterpret_cast<int32_t*>(tr);
    sp.plan = reinterpret_cast<gdr::PlanEntry*>(tr + gdr::kTruncHeader);
    sp.cert = reinterpret_cast<float*>(tr + gdr::kTruncHeader + n * sizeof(gdr::PlanEntry));
    sp.trunc = g_truncation ? 1 : 0;
  }
  if (bf16 && lengths && plan.P == 1 && NC > 0)   // rows longest first (written with the chunk list)
    sp.row_order = reinterpret_cast<const int32_t*>(static_cast<char*>(ws) +
                                                    gdr::records_bytes(d->B, d->Hv, NC, dtype_size(d->qkv_dtype)) +
                                                    gdr::seg_bytes(d->B, d->Hv, NC, dtype_size(d->qkv_dtype))) +
                   1 + size_t(d->B) * NC;
  if (fused_norm && bf16) {   // applied in the output pass's registers
    sp.z = fu->z;
    sp.norm_w = fu->norm_w;
    sp.eps = fu->norm_eps;
  }
  if (plan.P > 1) {
    hipError_t e = timed(GDR_KERNEL_TRANSITION, s, [&] { return gdr::launch_transition(sp, s); });
    if (e != hipSuccess) return fail(GDR_EHIP, "transition launch: %s", hipGetErrorString(e));
    e = timed(GDR_KERNEL_COMBINE, s, [&] { return gdr::launch_combine(sp, s); });
    if (e != hipSuccess) return fail(GDR_EHIP, "combine launch: %s", hipGetErrorString(e));
  }
  hipError_t e = timed(GDR_KERNEL_SCAN, s, [&] { return gdr::launch_scan(sp, bf16, s); });
  if (e != hipSuccess) return fail(GDR_EHIP, "scan launch: %s", hipGetErrorString(e));
  if (plan.P > 1) {
    e = timed(GDR_KERNEL_FINALIZE, s, [&] { return gdr::launch_finalize(sp, s); });
    if (e != hipSuccess) return fail(GDR_EHIP, "finalize launch: %s", hipGetErrorString(e));
  }
  if (fused_norm && !bf16 && d->L > 0) {   // float32: normalise o in place
    gdr::NormParams np{o, fu->z, fu->norm_w, fu->norm_eps, o, int64_t(d->B) * d->L * d->Hv};
    e = timed(GDR_KERNEL_NORM, s, [&] { return gdr::launch_gated_rmsnorm(np, 0, s); });
    if (e != hipSuccess) return fail(GDR_EHIP, "norm launch: %s", hipGetErrorString(e));
  }
  return GDR_OK;
}

gdr_status gdr_prefill_noalloc(const gdr_desc* d, const void* q, const void* k, const void* v, const float* g,
                               const void* beta, const int32_t* lengths, const float* s0, const int32_t* s0_row,
                               void* o, float* s_final, void* stream) {
  const gdr_status st = check_desc(d);
  if (st != GDR_OK) return st;
  const size_t need = gdr_prefill_workspace_size(d);
  if (need > gdr::kNoAllocScratchBytes)
    return fail(GDR_EUNSUPPORTED, "gdr_prefill_noalloc: this shape needs %zu bytes of workspace; the device-resident "
                "workspace holds at most %zu bytes (use gdr_prefill with a workspace of its own)",
                need, gdr::kNoAllocScratchBytes);
  // host-checkable errors first, as for every entry point (the workspace is checked below, once known)
  gdr_status chk = check_all(d, q, k, v, g, beta, lengths, s0, s0_row, o, s_final, nullptr, 0, /*need_ws=*/false);
  if (chk != GDR_OK) return chk;
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t e = gdr::noalloc_scratch(&ws);
    if (e != hipSuccess) return fail(GDR_EHIP, "gdr_prefill_noalloc: device workspace lookup: %s", hipGetErrorString(e));
  }
  t_no_alloc = true;
  const gdr_status r = gdr_prefill_ex(d, q, k, v, g, beta, lengths, s0, s0_row, nullptr, o, s_final, ws,
                                      need > 0 ? gdr::kNoAllocScratchBytes : 0, stream);
  t_no_alloc = false;
  return r;
}

gdr_status gdr_decode(const gdr_desc* d, const void* q, const void* k, const void* v, const float* g,
                      const void* beta, const int32_t* lengths, const float* s0, const int32_t* s0_row, void* o,
                      float* s_final, void* stream) {
  return gdr_decode_ex(d, q, k, v, g, beta, lengths, s0, s0_row, nullptr, o, s_final, stream);
}

gdr_status gdr_decode_ex(const gdr_desc* d, const void* q, const void* k, const void* v, const float* g,
                         const void* beta, const int32_t* lengths, const float* s0, const int32_t* s0_row,
                         const gdr_fusion* fu, void* o, float* s_final, void* stream) {
  // same validation as gdr_prefill_ex, with no workspace
  gdr_status st = check_desc(d);
  if (st != GDR_OK) return st;
  st = check_all(d, q, k, v, g, beta, lengths, s0, s0_row, o, s_final, nullptr, 0, /*need_ws=*/false, fu);
  if (st != GDR_OK) return st;
  if (d->B == 0) return GDR_OK;
  if (d->L == 0 && !s_final) return GDR_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  gdr::DecodeParams dp{q, k, v, g, beta, lengths, s0, s0_row, o, s_final, d->B, d->L, d->Hk, d->Hv, s0 ? d->n_s0 : 0};
  if (fu && fu->b_raw) {
    dp.b_raw = fu->b_raw;
    dp.a_raw = fu->a_raw;
    dp.A_log = fu->A_log;
    dp.dt_bias = fu->dt_bias;
  }
  if (fu && fu->z) {
    dp.z = fu->z;
    dp.norm_w = fu->norm_w;
    dp.eps = fu->norm_eps;
  }
  hipError_t e = timed(GDR_KERNEL_DECODE, s, [&] {
    return gdr::launch_decode(dp, d->qkv_dtype == GDR_BF16, d->beta_dtype == GDR_BF16, s);
  });
  if (e != hipSuccess) return fail(GDR_EHIP, "decode launch: %s", hipGetErrorString(e));
  return GDR_OK;
}

gdr_status gdr_gates(int32_t B, int32_t L, int32_t Hv, gdr_dtype ab_dtype, const void* b, const void* a,
                     const float* A_log, const float* dt_bias, const int32_t* lengths, void* beta, float* g,
                     void* stream) {
  if (B < 0 || L < 0 || Hv <= 0) return fail(GDR_EINVAL, "gates: B (%d), L (%d) >= 0 and Hv (%d) > 0 required", B, L, Hv);
  if (bad_dtype(ab_dtype)) return fail(GDR_EINVAL, "gates: ab_dtype %d is not a gdr_dtype", ab_dtype);
  const size_t n = size_t(B) * L * Hv, esz = dtype_size(ab_dtype);
  if (n == 0) return GDR_OK;
  if (!b || !a || !A_log || !dt_bias || !beta || !g) return fail(GDR_EINVAL, "gates: b, a, A_log, dt_bias, beta and g must be non-NULL");
  if (!aligned(b, esz) || !aligned(a, esz) || !aligned(beta, esz) || !aligned(g, 4) || !aligned(A_log, 4) ||
      !aligned(dt_bias, 4) || (lengths && !aligned(lengths, 4)))
    return fail(GDR_EINVAL, "gates: pointers must be element-aligned");
  const Range ins[] = {range("b", b, n * esz), range("a", a, n * esz), range("A_log", A_log, Hv * 4u),
                       range("dt_bias", dt_bias, Hv * 4u), range("lengths", lengths, lengths ? B * 4u : 0)};
  const Range outs[] = {range("beta", beta, n * esz), range("g", g, n * 4)};
  gdr_status st = check_overlaps(ins, 5, outs, 2);
  if (st != GDR_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  gdr::GatesParams p{b, a, A_log, dt_bias, lengths, beta, g, B, L, Hv};
  hipError_t e = timed(GDR_KERNEL_GATES, s, [&] { return gdr::launch_gates(p, ab_dtype == GDR_BF16, s); });
  if (e != hipSuccess) return fail(GDR_EHIP, "gates launch: %s", hipGetErrorString(e));
  return GDR_OK;
}

gdr_status gdr_conv_silu(int32_t B, int32_t L, int32_t Hk, int32_t Hv, int32_t K, gdr_dtype dtype, const void* mixed,
                         const void* tail, const float* w, const int32_t* lengths, void* q, void* k, void* v,
                         void* new_tail, void* stream) {
  if (B < 0 || L < 0 || Hk <= 0 || Hv <= 0)
    return fail(GDR_EINVAL, "conv_silu: B (%d), L (%d) >= 0 and Hk (%d), Hv (%d) > 0 required", B, L, Hk, Hv);
  if (K < 1 || K > gdr::kMaxConvTaps) return fail(GDR_EUNSUPPORTED, "conv_silu: K = %d, 1 <= K <= %d is built", K, gdr::kMaxConvTaps);
  if (bad_dtype(dtype)) return fail(GDR_EINVAL, "conv_silu: dtype %d is not a gdr_dtype", dtype);
  const size_t Dd = gdr::kHeadDim, esz = dtype_size(dtype);
  const size_t Cm = (2 * size_t(Hk) + Hv) * Dd;
  if (B > 65535 || (int64_t(L) + 63) / 64 > 65535 || Cm > (size_t(1) << 24))
    return fail(GDR_EUNSUPPORTED, "conv_silu: B <= 65535, ceil(L/64) <= 65535 and (2 Hk + Hv) 128 <= 2^24 required (grid limits)");
  if ((int64_t(L) + 64) * int64_t(Cm) * int64_t(esz) >= (int64_t(1) << 32))
    return fail(GDR_EUNSUPPORTED, "conv_silu: (L + 64) * (2 Hk + Hv) * 128 elements must stay below 4 GiB per batch row");
  const size_t K1 = size_t(K) - 1;
  const bool work = size_t(B) * L > 0 || (new_tail && B > 0 && K1 > 0);
  if (!work) return GDR_OK;
  if (!w) return fail(GDR_EINVAL, "conv_silu: w must be non-NULL");
  if (size_t(B) * L > 0 && (!mixed || !q || !k || !v)) return fail(GDR_EINVAL, "conv_silu: mixed, q, k and v must be non-NULL");
  if (!aligned(mixed, 16) || !aligned(tail, 16) || !aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) ||
      !aligned(new_tail, 16) || !aligned(w, 4) || (lengths && !aligned(lengths, 4)))
    return fail(GDR_EINVAL, "conv_silu: mixed, tail, q, k, v and new_tail must be 16-byte aligned");
  const size_t tok = size_t(B) * L;
  const Range ins[] = {range("mixed", mixed, tok * Cm * esz), range("tail", tail, tail ? B * K1 * Cm * esz : 0),
                       range("w", w, Cm * K * 4), range("lengths", lengths, lengths ? B * 4u : 0)};
  const Range outs[] = {range("q", q, tok * Hk * Dd * esz), range("k", k, tok * Hk * Dd * esz),
                        range("v", v, tok * Hv * Dd * esz), range("new_tail", new_tail, new_tail ? B * K1 * Cm * esz : 0)};
  gdr_status st = check_overlaps(ins, 4, outs, 4, "new_tail", "tail");
  if (st != GDR_OK) return st;
  if (B == 0) return GDR_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  gdr::ConvParams p{mixed, tail, w, lengths, q, k, v, new_tail, B, L, Hk, Hv, K};
  // L = 0 with a tail to carry: one tile still runs (its stores fall past L and are dropped)
  hipError_t e = timed(GDR_KERNEL_CONV, s, [&] { return gdr::launch_conv_silu(p, dtype == GDR_BF16, s); });
  if (e != hipSuccess) return fail(GDR_EHIP, "conv_silu launch: %s", hipGetErrorString(e));
  return GDR_OK;
}

gdr_status gdr_gated_rmsnorm(int64_t rows, gdr_dtype dtype, const void* x, const void* z, const float* w, float eps,
                             void* out, void* stream) {
  if (rows < 0) return fail(GDR_EINVAL, "gated_rmsnorm: rows (%lld) must be >= 0", (long long)rows);
  if (bad_dtype(dtype)) return fail(GDR_EINVAL, "gated_rmsnorm: dtype %d is not a gdr_dtype", dtype);
  if (!(eps >= 0.f) || eps > 1e30f) return fail(GDR_EINVAL, "gated_rmsnorm: eps must be finite and >= 0");
  if (rows > (int64_t(1) << 35)) return fail(GDR_EUNSUPPORTED, "gated_rmsnorm: rows must stay below 2^35");
  if (rows == 0) return GDR_OK;
  if (!x || !z || !w || !out) return fail(GDR_EINVAL, "gated_rmsnorm: x, z, w and out must be non-NULL");
  if (!aligned(x, 16) || !aligned(z, 16) || !aligned(out, 16) || !aligned(w, 4))
    return fail(GDR_EINVAL, "gated_rmsnorm: x, z and out must be 16-byte aligned");
  const size_t bytes = size_t(rows) * gdr::kHeadDim * dtype_size(dtype);
  const Range ins[] = {range("x", x, bytes), range("z", z, bytes), range("w", w, gdr::kHeadDim * 4)};
  const Range outs[] = {range("out", out, bytes)};
  gdr_status st = check_overlaps(ins, 3, outs, 1, "out", "x");
  if (st != GDR_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  gdr::NormParams p{x, z, w, eps, out, rows};
  hipError_t e = timed(GDR_KERNEL_NORM, s, [&] { return gdr::launch_gated_rmsnorm(p, dtype == GDR_BF16, s); });
  if (e != hipSuccess) return fail(GDR_EHIP, "gated_rmsnorm launch: %s", hipGetErrorString(e));
  return GDR_OK;
}

const char* gdr_last_error(void) { return g_last_error.c_str(); }

gdr_status gdr_set_truncation(int on) {
  g_truncation = on != 0;
  return GDR_OK;
}

size_t gdr_prefill_status_offset(const gdr_desc* d) {
  if (check_desc(d) != GDR_OK) return size_t(-1);
  const int NC = num_chunks(d->L);
  const size_t esz = dtype_size(d->qkv_dtype);
  if (size_t(d->B) * d->L == 0 || gdr::trunc_bytes(d->B, d->Hv, NC, esz) == 0) return size_t(-1);
  return gdr::trunc_offset(d->B, d->Hv, NC, esz);
}

gdr_status gdr_timing_enable(int on) {
  g_timing = on != 0;
  return GDR_OK;
}

gdr_status gdr_timing_read(double* total_ms, int64_t* launches, int n_kernels) {
  if (n_kernels < 0 || (n_kernels > 0 && (!total_ms || !launches)))
    return fail(GDR_EINVAL, "timing_read: bad output arrays");
  for (int i = 0; i < n_kernels; ++i) {
    total_ms[i] = 0.0;
    launches[i] = 0;
  }
  gdr_status st = GDR_OK;
  for (const TimingRecord& r : g_records) {
    float ms = 0.f;
    if (hipEventSynchronize(r.stop) != hipSuccess || hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess)
      st = fail(GDR_EHIP, "timing_read: event query failed");
    if (r.kernel < n_kernels) {
      total_ms[r.kernel] += ms;
      launches[r.kernel] += 1;
    }
    g_event_pool.push_back(r.start);
    g_event_pool.push_back(r.stop);
  }
  g_records.clear();
  return st;
}

const char* gdr_kernel_name(int kernel_id) {
  if (kernel_id < 0 || kernel_id >= GDR_KERNEL_COUNT) return "";
  return kKernelNames[kernel_id];
}

}  // extern "C"
