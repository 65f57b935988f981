// C ABI of libkvq: argument validation, cache layout, split planning and
// kernel launches. Every check happens before anything is enqueued.
#include <string.h>

#include <algorithm>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "kvq_internal.h"
#include "kvq_testing.h"

namespace {

constexpr size_t kAlign = 256;
constexpr size_t kScratchBytes = kvq::kAmaxBlocks * sizeof(unsigned);
constexpr int kMaxDecodeLen = 128 * 1024 * kvq::kTile;  // 128 splits x 1024 tiles
// Default split-planner targets (workgroups per decode launch), from same-box
// sweeps on the 8B-shape FP8 and Qwen3-shape FP4 steps (GQA) and the
// DeepSeek-R1-shape step (MLA: one workgroup per CU).
constexpr int kGqaTargetWgs = 512;
constexpr int kMlaTargetWgs = 256;
constexpr int kMaxTargetWgs = 1 << 20;
// Descriptor limits: they keep every per-page index of the kernels (int
// arithmetic over num_kv_heads x page_size x head_dim) inside 32 bits.
constexpr int kMaxPageSize = 1 << 16;
constexpr int kMaxKvHeads = 1 << 12;
// A launch covers at most 2^32 work-items (the dispatch's 32-bit grid size).
constexpr int64_t kMaxLaunchItems = (int64_t(1) << 32) - 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool is_fp8(int dt) { return dt == KVQ_FP8_E4M3 || dt == KVQ_FP8_E5M2; }

// KVQ_OK, or the reason this descriptor cannot be used.
int check_desc(const kvq_cache_desc* d) {
  if (!d) return KVQ_ERR_ARG;
  if (d->dtype < KVQ_FP8_E4M3 || d->dtype > KVQ_NVFP4) return KVQ_ERR_ARG;
  if (d->kind != KVQ_GQA && d->kind != KVQ_MLA) return KVQ_ERR_ARG;
  if (d->num_kv_heads < 1 || d->head_dim < 16 || d->v_dim < 1 || d->page_size < 1 || d->num_pages < 1)
    return KVQ_ERR_ARG;
  if (d->page_size % kvq::kTile) return KVQ_ERR_ARG;
  if (d->page_size > kMaxPageSize || d->num_kv_heads > kMaxKvHeads) return KVQ_ERR_UNSUPPORTED;
  if (d->head_dim % 16) return KVQ_ERR_ARG;
  if (d->scale_mode < KVQ_SCALE_TENSOR || d->scale_mode > KVQ_SCALE_KIVI) return KVQ_ERR_ARG;
  if (d->scale_mode != KVQ_SCALE_TENSOR && !(d->kind == KVQ_GQA && is_fp8(d->dtype))) return KVQ_ERR_UNSUPPORTED;
  if (d->kind == KVQ_GQA) {
    if (d->v_dim != d->head_dim) return KVQ_ERR_ARG;
    if (is_fp8(d->dtype)) return (d->head_dim == 64 || d->head_dim == 128) ? KVQ_OK : KVQ_ERR_UNSUPPORTED;
    if (d->dtype == KVQ_FP4_MX16) return d->head_dim == 128 ? KVQ_OK : KVQ_ERR_UNSUPPORTED;
    return KVQ_ERR_UNSUPPORTED;
  }
  if (d->num_kv_heads != 1 || d->v_dim > d->head_dim || d->v_dim % 16) return KVQ_ERR_ARG;
  if (d->dtype != KVQ_NVFP4) return KVQ_ERR_UNSUPPORTED;
  return (d->head_dim == 576 && d->v_dim == 512) ? KVQ_OK : KVQ_ERR_UNSUPPORTED;
}

// Scale buffers: FP4 block scales for K and V (bytes per row = D/16), or for
// KIVI caches only the V buffer of one fp32 per token (scale_block = 4*P).
void compute_layout(const kvq_cache_desc* d, kvq_layout* L, int64_t* code_block, int64_t* scale_block) {
  const bool kivi = d->scale_mode == KVQ_SCALE_KIVI;
  const int64_t row_code = is_fp8(d->dtype) ? d->head_dim : d->head_dim / 2;
  const int64_t row_scale = kivi ? 4 : (is_fp8(d->dtype) ? 0 : d->head_dim / 16);
  *code_block = row_code * d->page_size;
  *scale_block = row_scale * d->page_size;
  const size_t per_code = (size_t)d->num_pages * d->num_kv_heads * (size_t)*code_block;
  const size_t per_scale = (size_t)d->num_pages * d->num_kv_heads * (size_t)*scale_block;
  const size_t per_k_scale = kivi ? 0 : per_scale;
  // KIVI channel calibration keeps one running max per (kv head, channel)
  const size_t scratch = std::max(kScratchBytes, (size_t)d->num_kv_heads * d->head_dim * sizeof(unsigned));
  const bool has_v = d->kind == KVQ_GQA;
  memset(L, 0, sizeof(*L));
  size_t off = 0;
  L->k_codes_offset = off;
  L->k_codes_bytes = per_code;
  off = align_up(off + per_code);
  L->v_codes_offset = off;
  L->v_codes_bytes = has_v ? per_code : 0;
  off = align_up(off + L->v_codes_bytes);
  L->k_scales_offset = off;
  L->k_scales_bytes = per_k_scale;
  off = align_up(off + per_k_scale);
  L->v_scales_offset = off;
  L->v_scales_bytes = has_v ? per_scale : 0;
  off = align_up(off + L->v_scales_bytes);
  L->scratch_offset = off;
  L->scratch_bytes = scratch;
  off = align_up(off + scratch);
  L->total_bytes = off;
}

struct SplitPlan {
  int tiles_per_split;
  int num_splits;
};

// Context split: enough workgroups to fill 256 CUs several times over, each
// split an even number of 16-token tiles (waves consume tile pairs), at most
// 1024 tiles per split and 128 splits per sequence (so max_len <= 2M tokens).
// `target` = workgroups to aim at, 0 = the default.
SplitPlan plan_gqa(int batch, int hkv, int max_len, int target_wgs) {
  const int ntiles = (max_len + kvq::kTile - 1) / kvq::kTile;
  const int64_t units = (int64_t)batch * hkv;
  const int64_t target = target_wgs > 0 ? target_wgs : kGqaTargetWgs;
  int64_t tps = units > 0 ? (ntiles * units + target - 1) / target : ntiles;
  if (tps < 16) tps = 16;  // 2 tile pairs per wave at least
  tps = (tps + 1) & ~(int64_t)1;
  if (tps > 1024) tps = 1024;  // the kernel stages one split's page ids in LDS
  int64_t ns = ntiles > 0 ? (ntiles + tps - 1) / tps : 1;
  if (ns > 128) {
    ns = 128;
    tps = (ntiles + ns - 1) / ns;
    tps = (tps + 1) & ~(int64_t)1;
    ns = (ntiles + tps - 1) / tps;
  }
  if (ns < 1) ns = 1;
  return {(int)tps, (int)ns};
}

// MLA: one workgroup (4 waves, all query heads) per (sequence, split) and one
// per CU, so the default target is one round of 256 workgroups; each split
// is an even number of 16-token tiles (whole 32-token steps) whose pages fit
// the LDS page-id stage.
SplitPlan plan_mla(int batch, int max_len, int page_size, int target_wgs) {
  const int ntiles = (max_len + kvq::kTile - 1) / kvq::kTile;
  const int tpp = page_size / kvq::kTile;
  const int64_t units = batch;
  const int64_t target = target_wgs > 0 ? target_wgs : kMlaTargetWgs;
  const int64_t cap = ((int64_t)(kvq::kMlaMaxSplitPages - 1) * tpp) & ~(int64_t)1;
  int64_t tps = units > 0 ? (ntiles * units + target - 1) / target : ntiles;
  if (tps < 2) tps = 2;
  tps = (tps + 1) & ~(int64_t)1;  // whole 32-token steps
  if (tps > cap) tps = cap;
  int64_t ns = ntiles > 0 ? (ntiles + tps - 1) / tps : 1;
  if (ns > 128) {
    ns = 128;
    tps = (ntiles + ns - 1) / ns;
    tps = (tps + 1) & ~(int64_t)1;
    ns = (ntiles + tps - 1) / tps;
  }
  if (ns < 1) ns = 1;
  return {(int)tps, (int)ns};
}

// Pages one MLA split touches at most (splits start at multiples of the split size).
int64_t mla_split_pages(const SplitPlan& p, int page_size) {
  const int64_t tpp = page_size / kvq::kTile, tps = p.tiles_per_split;
  return tps % tpp == 0 ? tps / tpp : (tps - 1) / tpp + 2;
}

// Workspace: [partial outputs fp32 B*Hq*S*Dv] [partial LSEs fp32 B*Hq*S].
struct WsLayout {
  size_t o, lse, total;
};
WsLayout workspace_for(const SplitPlan& p, int batch, int hq, int dv) {
  WsLayout w = {0, 0, 0};
  if (p.num_splits <= 1) return w;
  const size_t parts = (size_t)batch * hq * p.num_splits;
  w.o = 0;
  w.lse = align_up(parts * dv * sizeof(float));
  w.total = w.lse + align_up(parts * sizeof(float));
  return w;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// ------------------------------------------------------------ instrumentation
struct ProfRecord {
  int family;  // 0 store, 1 decode, 2 merge, 3 amax, 4 dequant_prev, 5 extend
  hipEvent_t start, stop;
};
const char* const kFamilies[] = {"store", "decode", "merge", "amax", "dequant_prev", "extend"};
constexpr int kNumFamilies = 6;
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRecord> g_prof;
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

void clear_records_locked() {
  for (auto& r : g_prof) {
    (void)hipEventSynchronize(r.stop);
    g_event_pool.push_back(r.start);
    g_event_pool.push_back(r.stop);
  }
  g_prof.clear();
}

// Brackets one launch with events when instrumentation is on.
struct Timed {
  int family;
  hipStream_t stream;
  hipEvent_t start = nullptr, stop = nullptr;
  Timed(int f, hipStream_t s) : family(f), stream(s) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (!g_prof_on) return;
    start = take_event();
    stop = take_event();
    if (start && stop) (void)hipEventRecord(start, stream);
  }
  ~Timed() {
    if (!start || !stop) return;
    (void)hipEventRecord(stop, stream);
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof.push_back({family, start, stop});
  }
};

}  // namespace

extern "C" {

int kvq_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  clear_records_locked();
  g_prof_on = on != 0;
  return KVQ_OK;
}

int kvq_profile_read(const char* kernel, double* total_ms, int64_t* launches) {
  if (!kernel || !total_ms || !launches) return KVQ_ERR_ARG;
  int fam = -1;
  for (int i = 0; i < kNumFamilies; ++i)
    if (std::string(kernel) == kFamilies[i]) fam = i;
  if (fam < 0) return KVQ_ERR_ARG;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  double tot = 0.0;
  int64_t n = 0;
  int status = KVQ_OK;
  std::vector<ProfRecord> keep;
  for (auto& r : g_prof) {
    if (r.family != fam) {
      keep.push_back(r);
      continue;
    }
    float ms = 0.f;
    if (hipEventSynchronize(r.stop) != hipSuccess || hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess)
      status = KVQ_ERR_HIP;
    tot += ms;
    ++n;
    g_event_pool.push_back(r.start);
    g_event_pool.push_back(r.stop);
  }
  g_prof.swap(keep);
  *total_ms = tot;
  *launches = n;
  return status;
}

const char* kvq_status_string(int status) {
  switch (status) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_ARG: return "invalid argument";
    case KVQ_ERR_UNSUPPORTED: return "unsupported format or shape";
    case KVQ_ERR_SIZE: return "buffer too small";
    case KVQ_ERR_HIP: return "HIP launch error";
    case KVQ_ERR_WORKSPACE: return "decode needs more workspace than the library's static workspace holds";
    default: return "unknown status";
  }
}

int kvq_bytes_per_token(const kvq_cache_desc* d, double* bytes_out) {
  if (!bytes_out) return KVQ_ERR_ARG;
  const int st = check_desc(d);
  if (st == KVQ_ERR_ARG) return st;
  const double bits = is_fp8(d->dtype) ? 8.0 : 4.0 + 8.0 / 16.0;
  const double rows = d->kind == KVQ_GQA ? 2.0 * d->num_kv_heads : 1.0;
  *bytes_out = rows * d->head_dim * bits / 8.0;
  if (d->scale_mode == KVQ_SCALE_KIVI) *bytes_out += 4.0 * d->num_kv_heads;  // one fp32 V scale per token-head
  return KVQ_OK;
}

int kvq_alloc_pages(const kvq_cache_desc* d, void* dev_mem, size_t dev_bytes, size_t* bytes_needed,
                    kvq_cache** out) {
  const int st = check_desc(d);
  if (st != KVQ_OK) return st;
  kvq_layout L;
  int64_t cb, sb;
  compute_layout(d, &L, &cb, &sb);
  if (bytes_needed) *bytes_needed = L.total_bytes;
  if (!dev_mem) return bytes_needed ? KVQ_OK : KVQ_ERR_ARG;
  if (!out) return KVQ_ERR_ARG;
  if (reinterpret_cast<uintptr_t>(dev_mem) % kAlign) return KVQ_ERR_ARG;
  if (dev_bytes < L.total_bytes) return KVQ_ERR_SIZE;
  kvq_cache* c = new (std::nothrow) kvq_cache;
  if (!c) return KVQ_ERR_ARG;
  c->desc = *d;
  c->layout = L;
  c->base = static_cast<uint8_t*>(dev_mem);
  c->code_block_bytes = cb;
  c->scale_block_bytes = sb;
  c->split_target = 0;
  *out = c;
  return KVQ_OK;
}

int kvq_cache_layout(const kvq_cache* c, kvq_layout* out) {
  if (!c || !out) return KVQ_ERR_ARG;
  *out = c->layout;
  return KVQ_OK;
}

void kvq_free_handle(kvq_cache* c) { delete c; }

int kvq_testing_set_split_target(kvq_cache* c, int32_t target_wgs) {
  if (!c || target_wgs < 0 || target_wgs > kMaxTargetWgs) return KVQ_ERR_ARG;
  c->split_target = target_wgs;
  return KVQ_OK;
}

int kvq_compute_scale(const kvq_cache* c, const void* x0, int64_t n0, const void* x1, int64_t n1, float* scale_out,
                      void* stream) {
  if (!c || !scale_out || n0 < 0 || n1 < 0) return KVQ_ERR_ARG;
  if ((n0 > 0 && !x0) || (n1 > 0 && !x1)) return KVQ_ERR_ARG;
  float div;
  switch (c->desc.dtype) {
    case KVQ_FP8_E4M3: div = 448.0f; break;
    case KVQ_FP8_E5M2: div = 57344.0f; break;
    case KVQ_NVFP4: div = 6.0f * 448.0f; break;
    default: return KVQ_ERR_UNSUPPORTED;
  }
  unsigned* scratch = reinterpret_cast<unsigned*>(c->base + c->layout.scratch_offset);
  if (c->desc.scale_mode != KVQ_SCALE_TENSOR) {
    const int64_t row = (int64_t)c->desc.num_kv_heads * c->desc.head_dim;
    if (n0 % row || n1 % row) return KVQ_ERR_ARG;
    if ((n0 && !aligned16(x0)) || (n1 && !aligned16(x1))) return KVQ_ERR_ARG;
    Timed timer(3, static_cast<hipStream_t>(stream));
    if (c->desc.scale_mode == KVQ_SCALE_KIVI) {
      const hipError_t e = kvq_launch_amax_channels(static_cast<const uint16_t*>(x0), n0 / row,
                                                    static_cast<const uint16_t*>(x1), n1 / row, (int)row, scratch,
                                                    div, scale_out, static_cast<hipStream_t>(stream));
      return e == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
    }
    const hipError_t e = kvq_launch_amax_heads(static_cast<const uint16_t*>(x0), n0 / row,
                                               static_cast<const uint16_t*>(x1), n1 / row, c->desc.num_kv_heads,
                                               c->desc.head_dim, scratch, div, scale_out,
                                               static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
  }
  Timed timer(3, static_cast<hipStream_t>(stream));
  const hipError_t e = kvq_launch_amax(static_cast<const uint16_t*>(x0), n0, static_cast<const uint16_t*>(x1), n1,
                                       scratch, div, scale_out, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

int kvq_store(const kvq_cache* c, const void* k, const void* v, const int64_t* slots, int32_t n, const float* k_scale,
              const float* v_scale, void* stream) {
  if (!c || n < 0) return KVQ_ERR_ARG;
  if (n == 0) return KVQ_OK;
  if (!k || !slots || !aligned16(k)) return KVQ_ERR_ARG;
  if (c->desc.kind == KVQ_GQA) {
    if (!v || !aligned16(v)) return KVQ_ERR_ARG;
    if (c->desc.scale_mode == KVQ_SCALE_KIVI && (!k_scale || !aligned16(k_scale))) return KVQ_ERR_ARG;
  } else {
    if (v) return KVQ_ERR_ARG;
    if (!k_scale) return KVQ_ERR_ARG;  // NVFP4 needs its global scale
  }
  // one thread per 16 elements of every stored row
  const int64_t rows = c->desc.kind == KVQ_GQA ? c->desc.num_kv_heads : 1;
  if ((int64_t)n * rows * (c->desc.head_dim / 16) > kMaxLaunchItems) return KVQ_ERR_UNSUPPORTED;
  Timed timer(0, static_cast<hipStream_t>(stream));
  const hipError_t e = kvq_launch_store(c, static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), slots, n,
                                        k_scale, v_scale, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

size_t kvq_decode_workspace_bytes(const kvq_cache* c, int32_t batch, int32_t hq, int32_t max_len) {
  if (!c || batch < 0 || hq < 1 || max_len < 0) return 0;
  if (c->desc.kind == KVQ_GQA)
    return workspace_for(plan_gqa(batch, c->desc.num_kv_heads, max_len, c->split_target), batch, hq,
                         c->desc.v_dim).total;
  if (hq > 128) return 0;
  return workspace_for(plan_mla(batch, max_len, c->desc.page_size, c->split_target), batch, hq, c->desc.v_dim).total;
}

namespace {

// kvq_decode_noalloc: the library's static workspace in place of a caller
// buffer, once every argument has been checked (the size limit first, then
// the device address of this stream's device).
int bind_static_workspace(size_t need, hipStream_t s, void** ws, size_t* ws_bytes) {
  if (need > kvq::kStaticWorkspaceBytes) return KVQ_ERR_WORKSPACE;
  *ws = nullptr;
  *ws_bytes = 0;
  if (need == 0) return KVQ_OK;
  if (kvq_static_workspace(s, ws) != hipSuccess) return KVQ_ERR_HIP;
  *ws_bytes = kvq::kStaticWorkspaceBytes;
  return KVQ_OK;
}

// kvq_decode, optionally appending the token at position seq_lens[b] - 1 of
// every sequence first (k_new / v_new non-null: kvq_decode_append)
// (q8: FP8-domain attention, kvq_decode_fp8q / kvq_decode_append_fp8q)
int decode_impl(const kvq_cache* c, const void* k_new, const void* v_new, const void* q, int32_t batch, int32_t hq,
                const int32_t* page_table, int32_t page_table_stride, const int32_t* seq_lens, int32_t max_len,
                float sm_scale, const float* k_scale, const float* v_scale, float* out, float* lse, void* ws,
                size_t ws_bytes, void* stream, bool q8 = false, const float* q_scale = nullptr,
                bool static_ws = false) {
  if (!c || batch < 0 || hq < 1 || max_len < 0) return KVQ_ERR_ARG;
  if (q8) {
    // FP8 GQA caches with tensor or head scales, and the NVFP4 MLA latent
    const kvq_cache_desc& d = c->desc;
    const bool gqa = d.kind == KVQ_GQA && is_fp8(d.dtype) && d.scale_mode != KVQ_SCALE_KIVI;
    if (!gqa && !(d.kind == KVQ_MLA && d.dtype == KVQ_NVFP4)) return KVQ_ERR_UNSUPPORTED;
    if (q_scale && reinterpret_cast<uintptr_t>(q_scale) % 4) return KVQ_ERR_ARG;
  }
  if (batch == 0) return KVQ_OK;
  if (!q || !page_table || !seq_lens || !out || !aligned16(q)) return KVQ_ERR_ARG;
  const kvq_cache_desc& d = c->desc;
  if (k_new) {
    if (!aligned16(k_new)) return KVQ_ERR_ARG;
    if (d.kind == KVQ_GQA ? (!v_new || !aligned16(v_new)) : v_new != nullptr) return KVQ_ERR_ARG;
  }
  // the length cap first: it keeps the page count below in range
  if (max_len > kMaxDecodeLen) return KVQ_ERR_UNSUPPORTED;
  const int P = d.page_size;
  if (page_table_stride < ((int64_t)max_len + P - 1) / P || page_table_stride < 1) return KVQ_ERR_ARG;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (d.kind == KVQ_GQA) {
    if (hq % d.num_kv_heads) return KVQ_ERR_ARG;
    const int G = hq / d.num_kv_heads;
    if (G > 16) return KVQ_ERR_UNSUPPORTED;
    if (d.scale_mode == KVQ_SCALE_KIVI && (!k_scale || !aligned16(k_scale))) return KVQ_ERR_ARG;
    const SplitPlan plan = plan_gqa(batch, d.num_kv_heads, max_len, c->split_target);
    const WsLayout wl = workspace_for(plan, batch, hq, d.v_dim);
    const size_t need = wl.total;
    if (static_ws) {
      const int st = bind_static_workspace(need, s, &ws, &ws_bytes);
      if (st != KVQ_OK) return st;
    }
    if (need && (!ws || ws_bytes < need || reinterpret_cast<uintptr_t>(ws) % kAlign)) return KVQ_ERR_SIZE;
    GqaDecodeArgs a;
    memset(&a, 0, sizeof(a));
    a.k_codes = c->base + c->layout.k_codes_offset;
    a.v_codes = c->base + c->layout.v_codes_offset;
    a.k_scales = c->base + c->layout.k_scales_offset;
    a.v_scales = c->base + c->layout.v_scales_offset;
    a.code_block_bytes = c->code_block_bytes;
    a.scale_block_bytes = c->scale_block_bytes;
    a.num_pages = d.num_pages;
    a.q = static_cast<const uint16_t*>(q);
    a.page_table = page_table;
    a.page_table_stride = page_table_stride;
    a.seq_lens = seq_lens;
    const bool fp8 = is_fp8(d.dtype);
    a.k_scale = fp8 ? k_scale : nullptr;
    a.v_scale = fp8 ? v_scale : nullptr;
    a.scale_mode = d.scale_mode;
    if (d.scale_mode == KVQ_SCALE_KIVI) a.v_scale = nullptr;  // V scales come from the cache
    a.sm_scale_log2 = sm_scale * 1.4426950408889634f;
    a.batch = batch;
    a.hq = hq;
    a.hkv = d.num_kv_heads;
    a.group = G;
    a.page_size = P;
    a.max_len = max_len;
    a.tiles_per_split = plan.tiles_per_split;
    a.num_splits = plan.num_splits;
    uint8_t* wsb = static_cast<uint8_t*>(ws);
    a.ws_o = need ? reinterpret_cast<float*>(wsb + wl.o) : nullptr;
    a.ws_lse = need ? reinterpret_cast<float*>(wsb + wl.lse) : nullptr;
    a.out = out;
    a.lse = lse;
    a.new_k = static_cast<const uint16_t*>(k_new);
    a.new_v = static_cast<const uint16_t*>(v_new);
    a.q8 = q8 ? 1 : 0;
    a.q_scale = q_scale;
    hipError_t e;
    {
      Timed timer(1, s);
      e = kvq_launch_decode_gqa(c, a, s);
    }
    if (e != hipSuccess) return KVQ_ERR_HIP;
    if (plan.num_splits > 1) {
      Timed timer(2, s);
      CombineArgs cb;
      cb.ws_o = a.ws_o;
      cb.ws_lse = a.ws_lse;
      cb.seq_lens = seq_lens;
      cb.out = out;
      cb.lse = lse;
      cb.batch = batch;
      cb.hq = hq;
      cb.dv = d.v_dim;
      cb.num_splits = plan.num_splits;
      cb.tokens_per_split = plan.tiles_per_split * kvq::kTile;
      cb.max_len = max_len;
      e = kvq_launch_combine(cb, s);
      if (e != hipSuccess) return KVQ_ERR_HIP;
    }
    return KVQ_OK;
  }
  // MLA
  if (hq < 1 || hq > 128) return KVQ_ERR_UNSUPPORTED;
  if (!k_scale) return KVQ_ERR_ARG;  // the NVFP4 global scale
  const SplitPlan plan = plan_mla(batch, max_len, c->desc.page_size, c->split_target);
  // pages one split touches, whatever its alignment to page boundaries
  if (mla_split_pages(plan, P) > kvq::kMlaMaxSplitPages) return KVQ_ERR_UNSUPPORTED;
  const WsLayout wl = workspace_for(plan, batch, hq, d.v_dim);
  const size_t need = wl.total;
  if (static_ws) {
    const int st = bind_static_workspace(need, s, &ws, &ws_bytes);
    if (st != KVQ_OK) return st;
  }
  if (need && (!ws || ws_bytes < need || reinterpret_cast<uintptr_t>(ws) % kAlign)) return KVQ_ERR_SIZE;
  MlaDecodeArgs a;
  memset(&a, 0, sizeof(a));
  a.codes = c->base + c->layout.k_codes_offset;
  a.scales = c->base + c->layout.k_scales_offset;
  a.num_pages = d.num_pages;
  a.q = static_cast<const uint16_t*>(q);
  a.page_table = page_table;
  a.page_table_stride = page_table_stride;
  a.seq_lens = seq_lens;
  a.g_scale = k_scale;
  a.sm_scale_log2 = sm_scale * 1.4426950408889634f;
  a.batch = batch;
  a.hq = hq;
  a.page_size = P;
  a.max_len = max_len;
  a.tiles_per_split = plan.tiles_per_split;
  a.num_splits = plan.num_splits;
  uint8_t* wsb = static_cast<uint8_t*>(ws);
  a.ws_o = need ? reinterpret_cast<float*>(wsb + wl.o) : nullptr;
  a.ws_lse = need ? reinterpret_cast<float*>(wsb + wl.lse) : nullptr;
  a.out = out;
  a.lse = lse;
  a.new_k = static_cast<const uint16_t*>(k_new);
  a.q8 = q8 ? 1 : 0;
  a.q_scale = q_scale;
  hipError_t e;
  {
    Timed timer(1, s);
    e = kvq_launch_decode_mla(c, a, s);
  }
  if (e != hipSuccess) return KVQ_ERR_HIP;
  if (plan.num_splits > 1) {
    Timed timer(2, s);
    CombineArgs cb;
    cb.ws_o = a.ws_o;
    cb.ws_lse = a.ws_lse;
    cb.seq_lens = seq_lens;
    cb.out = out;
    cb.lse = lse;
    cb.batch = batch;
    cb.hq = hq;
    cb.dv = d.v_dim;
    cb.num_splits = plan.num_splits;
    cb.tokens_per_split = plan.tiles_per_split * kvq::kTile;
    cb.max_len = max_len;
    e = kvq_launch_combine(cb, s);
    if (e != hipSuccess) return KVQ_ERR_HIP;
  }
  return KVQ_OK;
}

}  // namespace

int kvq_decode(const kvq_cache* c, const void* q, int32_t batch, int32_t hq, const int32_t* page_table,
               int32_t page_table_stride, const int32_t* seq_lens, int32_t max_len, float sm_scale,
               const float* k_scale, const float* v_scale, float* out, float* lse, void* ws, size_t ws_bytes,
               void* stream) {
  return decode_impl(c, nullptr, nullptr, q, batch, hq, page_table, page_table_stride, seq_lens, max_len, sm_scale,
                     k_scale, v_scale, out, lse, ws, ws_bytes, stream);
}

int kvq_decode_noalloc(const kvq_cache* c, const void* q, int32_t batch, int32_t hq, const int32_t* page_table,
                       int32_t page_table_stride, const int32_t* seq_lens, int32_t max_len, float sm_scale,
                       const float* k_scale, const float* v_scale, float* out, float* lse, void* stream) {
  return decode_impl(c, nullptr, nullptr, q, batch, hq, page_table, page_table_stride, seq_lens, max_len, sm_scale,
                     k_scale, v_scale, out, lse, nullptr, 0, stream, false, nullptr, true);
}

int kvq_decode_append(const kvq_cache* c, const void* k_new, const void* v_new, const void* q, int32_t batch,
                      int32_t hq, const int32_t* page_table, int32_t page_table_stride, const int32_t* seq_lens,
                      int32_t max_len, float sm_scale, const float* k_scale, const float* v_scale, float* out,
                      float* lse, void* ws, size_t ws_bytes, void* stream) {
  if (!k_new) return KVQ_ERR_ARG;
  return decode_impl(c, k_new, v_new, q, batch, hq, page_table, page_table_stride, seq_lens, max_len, sm_scale,
                     k_scale, v_scale, out, lse, ws, ws_bytes, stream);
}

int kvq_decode_fp8q(const kvq_cache* c, const void* q, int32_t batch, int32_t hq, const int32_t* page_table,
                    int32_t page_table_stride, const int32_t* seq_lens, int32_t max_len, float sm_scale,
                    const float* q_scale, const float* k_scale, const float* v_scale, float* out, float* lse,
                    void* ws, size_t ws_bytes, void* stream) {
  return decode_impl(c, nullptr, nullptr, q, batch, hq, page_table, page_table_stride, seq_lens, max_len, sm_scale,
                     k_scale, v_scale, out, lse, ws, ws_bytes, stream, true, q_scale);
}

int kvq_decode_append_fp8q(const kvq_cache* c, const void* k_new, const void* v_new, const void* q, int32_t batch,
                           int32_t hq, const int32_t* page_table, int32_t page_table_stride, const int32_t* seq_lens,
                           int32_t max_len, float sm_scale, const float* q_scale, const float* k_scale,
                           const float* v_scale, float* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  if (!k_new) return KVQ_ERR_ARG;
  return decode_impl(c, k_new, v_new, q, batch, hq, page_table, page_table_stride, seq_lens, max_len, sm_scale,
                     k_scale, v_scale, out, lse, ws, ws_bytes, stream, true, q_scale);
}

int kvq_compute_q_scale(const kvq_cache* c, const void* q, int64_t n_tokens, int32_t num_q_heads, float* q_scale_out,
                        void* stream) {
  if (!c || !q_scale_out || n_tokens < 0 || num_q_heads < 1) return KVQ_ERR_ARG;
  const kvq_cache_desc& d = c->desc;
  const bool gqa = d.kind == KVQ_GQA && is_fp8(d.dtype) && d.scale_mode != KVQ_SCALE_KIVI;
  if (!gqa && !(d.kind == KVQ_MLA && d.dtype == KVQ_NVFP4)) return KVQ_ERR_UNSUPPORTED;
  if (num_q_heads % d.num_kv_heads) return KVQ_ERR_ARG;
  if (n_tokens > 0 && (!q || !aligned16(q))) return KVQ_ERR_ARG;
  if (d.scale_mode == KVQ_SCALE_HEAD && num_q_heads > kvq::kAmaxBlocks) return KVQ_ERR_UNSUPPORTED;
  unsigned* scratch = reinterpret_cast<unsigned*>(c->base + c->layout.scratch_offset);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  Timed timer(3, s);
  hipError_t e;
  if (d.scale_mode == KVQ_SCALE_HEAD)
    e = kvq_launch_amax_heads(static_cast<const uint16_t*>(q), n_tokens, nullptr, 0, num_q_heads, d.head_dim,
                              scratch, 448.0f, q_scale_out, s);
  else
    e = kvq_launch_amax(static_cast<const uint16_t*>(q), n_tokens * num_q_heads * d.head_dim, nullptr, 0, scratch,
                        448.0f, q_scale_out, s);
  return e == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

int kvq_dequantize_prev_kv(const kvq_cache* c, const int32_t* pages, int32_t n_pages, const float* g_scale,
                           const float* k_scale_out, const float* v_scale_out, void* dq_k, void* dq_v, void* stream) {
  if (!c || n_pages < 0) return KVQ_ERR_ARG;
  const kvq_cache_desc& d = c->desc;
  if (d.dtype != KVQ_FP4_MX16 && d.dtype != KVQ_NVFP4) return KVQ_ERR_UNSUPPORTED;
  if (d.kind == KVQ_GQA) {
    if (n_pages > 0 && (!dq_v || !aligned16(dq_v))) return KVQ_ERR_ARG;
  } else {
    if (dq_v || v_scale_out || !g_scale) return KVQ_ERR_ARG;
  }
  if (n_pages == 0) return KVQ_OK;
  if (!pages || !dq_k || !aligned16(dq_k)) return KVQ_ERR_ARG;
  const int64_t threads = (int64_t)n_pages * d.num_kv_heads * d.page_size * (d.head_dim / 16);
  if ((threads + 255) / 256 > INT32_MAX) return KVQ_ERR_UNSUPPORTED;
  Timed timer(4, static_cast<hipStream_t>(stream));
  const hipError_t e = kvq_launch_dequant_prev(c, pages, n_pages, g_scale, k_scale_out, v_scale_out,
                                               static_cast<uint8_t*>(dq_k), static_cast<uint8_t*>(dq_v),
                                               static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

int kvq_extend_attention(const void* q, const void* k_new, const void* v_new, const int32_t* cu_q, int32_t total_q,
                         const int32_t* prefix_len, const void* dq_k, const void* dq_v, const int32_t* page_off,
                         int32_t n_pages, const float* s_k, const float* s_v, int32_t batch, int32_t num_q_heads,
                         int32_t num_kv_heads, int32_t head_dim, int32_t page_size, int32_t max_chunk,
                         float sm_scale, float* out, float* lse, void* stream) {
  if (batch < 0 || total_q < 0 || n_pages < 0 || max_chunk < 0 || page_size < 1) return KVQ_ERR_ARG;
  if (num_kv_heads < 1 || num_q_heads < 1 || num_q_heads % num_kv_heads) return KVQ_ERR_ARG;
  if (head_dim != 128) return KVQ_ERR_UNSUPPORTED;
  const int G = num_q_heads / num_kv_heads;
  if (G > 16 || (G & (G - 1))) return KVQ_ERR_UNSUPPORTED;  // 256 query rows per workgroup = 256/G tokens
  if (batch == 0 || total_q == 0 || max_chunk == 0) return KVQ_OK;
  if (!q || !k_new || !v_new || !cu_q || !prefix_len || !page_off || !out) return KVQ_ERR_ARG;
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(out)) return KVQ_ERR_ARG;
  if (n_pages > 0 && (!dq_k || !dq_v || !aligned16(dq_k) || !aligned16(dq_v))) return KVQ_ERR_ARG;
  const int TT = kvq::kExtendRows / G;
  const int64_t q_tiles = ((int64_t)max_chunk + TT - 1) / TT;
  const int64_t n_work = (int64_t)batch * num_kv_heads * q_tiles;
  if (n_work > INT32_MAX - 8) return KVQ_ERR_UNSUPPORTED;
  ExtendArgs a;
  memset(&a, 0, sizeof(a));
  a.q = static_cast<const uint16_t*>(q);
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.cu_q = cu_q;
  a.prefix_len = prefix_len;
  a.page_off = page_off;
  a.dq_k = static_cast<const uint8_t*>(dq_k);
  a.dq_v = static_cast<const uint8_t*>(dq_v);
  a.s_k = s_k;
  a.s_v = s_v;
  a.out = out;
  a.lse = lse;
  a.total_q = total_q;
  a.n_pages = n_pages;
  a.batch = batch;
  a.hq = num_q_heads;
  a.hkv = num_kv_heads;
  a.group = G;
  a.page_size = page_size;
  a.max_chunk = max_chunk;
  a.q_tiles = (int)q_tiles;
  a.n_work = (int)n_work;
  a.sm_scale = sm_scale;
  Timed timer(5, static_cast<hipStream_t>(stream));
  const hipError_t e = kvq_launch_extend(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

}  // extern "C"
