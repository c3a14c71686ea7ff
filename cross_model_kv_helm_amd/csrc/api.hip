// api.hip — the C ABI (include/helm_kv.h): host-side validation, workspace
// layout, the device/arch gate, and kernel dispatch.  Every check runs
// before anything is enqueued, so a refused call writes nothing and the
// caller can fall back to a normal prefill ("Helm Intelligent Routing",
// section "What happens when a transfer cannot be used").
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <vector>

#include "../../include/helm_kv.h"
#include "internal.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  std::va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return status;
}

void clear_error() { g_err[0] = '\0'; }

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Multiplies non-negative factors; returns false on int64 overflow.
bool mul_ok(int64_t& acc, int64_t f) {
  if (f < 0) return false;
  if (f != 0 && acc > INT64_MAX / f) return false;
  acc *= f;
  return true;
}

bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  if (!a || !b || na <= 0 || nb <= 0) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

// Fields common to both shapes.
struct Common {
  int32_t L_s, L_t, H, D, k, dtype;
  double theta_src, theta_tgt;
};

int check_common(const Common& c) {
  if (c.L_s < 1 || c.L_t < 1 || c.H < 1)
    return fail(HELM_E_INVALID_ARG, "layer and head counts must be >= 1 (L_s=%d L_t=%d H=%d)",
                c.L_s, c.L_t, c.H);
  if (c.dtype != HELM_BF16 && c.dtype != HELM_F32)
    return fail(HELM_E_DTYPE, "unknown dtype code %d (HELM_BF16=0, HELM_F32=1)", c.dtype);
  if (c.D <= 0 || (c.D & 1))
    return fail(HELM_E_PAIR_SHAPE, "head_dim must be positive and even for rotate-half RoPE (D=%d)", c.D);
  if (c.D != 64 && c.D != 128)
    return fail(HELM_E_PAIR_SHAPE, "head_dim %d is not supported (64 or 128)", c.D);
  if (c.k < 1 || c.k > c.L_s)
    return fail(HELM_E_INVALID_ARG, "k=%d must lie in 1..L_s (L_s=%d)", c.k, c.L_s);
  if (c.k > 64) return fail(HELM_E_INVALID_ARG, "k=%d exceeds the supported maximum of 64", c.k);
  if ((int64_t)c.L_t * c.H > 65535)
    return fail(HELM_E_INVALID_ARG, "L_t*H=%lld exceeds 65535", (long long)c.L_t * c.H);
  if (!(c.theta_src > 0.0) || !std::isfinite(c.theta_src) || !(c.theta_tgt > 0.0) ||
      !std::isfinite(c.theta_tgt))
    return fail(HELM_E_INVALID_ARG, "RoPE bases must be finite and > 0 (src=%g tgt=%g)", c.theta_src,
                c.theta_tgt);
  return HELM_OK;
}

Common common_of(const helm_shape_t* s) {
  return {s->n_src_layers, s->n_tgt_layers, s->n_kv_heads, s->head_dim, s->k, s->dtype,
          s->rope_theta_src, s->rope_theta_tgt};
}
Common common_of(const helm_paged_shape_t* s) {
  return {s->n_src_layers, s->n_tgt_layers, s->n_kv_heads, s->head_dim, s->k, s->dtype,
          s->rope_theta_src, s->rope_theta_tgt};
}

size_t elem_bytes(int32_t dtype) { return dtype == HELM_BF16 ? 2 : 4; }

// Workspace: [rope_src: ceil(N/16)*16*D/2 float2][rope_tgt: same]{[src_row: N int32][dst_row: N int32]}
struct Workspace {
  size_t rope_bytes = 0, rows_bytes = 0, total = 0;
};

bool workspace_layout(int64_t n_tok, int32_t D, bool paged, Workspace& w) {
  // the tables' entries, (n_tok rounded up to a block) * D/2, must not
  // overflow before their byte count is checked
  const int64_t per_block = (int64_t)helm::kRopeBlock * (D / 2) * (int64_t)sizeof(float2);
  if (n_tok < 0 || n_tok / helm::kRopeBlock + 1 > INT64_MAX / per_block) return false;
  int64_t rb = helm::rope_table_entries(n_tok, D / 2);
  if (!mul_ok(rb, (int64_t)sizeof(float2))) return false;
  w.rope_bytes = align_up((size_t)rb);
  w.rows_bytes = paged ? align_up((size_t)n_tok * sizeof(int32_t)) : 0;
  w.total = 2 * w.rope_bytes + 2 * w.rows_bytes;
  if (w.total == 0) w.total = kAlign;   // never ask for a zero-byte buffer
  return true;
}

// ---- device gate -------------------------------------------------------
constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_state[kMaxDevices];   // 0 unknown, 1 ok, 2 wrong arch

int device_gate(int device) {
  int count = 0;
  hipError_t e = hipGetDeviceCount(&count);
  if (e != hipSuccess || count <= 0) {
    (void)hipGetLastError();
    return fail(HELM_E_NO_DEVICE, "no GPU is visible (%s)", e == hipSuccess ? "count 0" : hipGetErrorString(e));
  }
  if (device < 0) {
    e = hipGetDevice(&device);
    if (e != hipSuccess) return fail(HELM_E_NO_DEVICE, "hipGetDevice failed: %s", hipGetErrorString(e));
  }
  if (device >= count) return fail(HELM_E_NO_DEVICE, "device %d does not exist (%d visible)", device, count);
  const int slot = device < kMaxDevices ? device : -1;
  int st = slot >= 0 ? g_dev_state[slot].load(std::memory_order_relaxed) : 0;
  if (st == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, device);
    if (e != hipSuccess) return fail(HELM_E_NO_DEVICE, "hipGetDeviceProperties failed: %s", hipGetErrorString(e));
    st = helm_arch_supported(prop.gcnArchName) ? 1 : 2;
    if (st == 2) {
      if (slot >= 0) g_dev_state[slot].store(st, std::memory_order_relaxed);
      return fail(HELM_E_ARCH, "device %d is %s; this library runs on gfx950 (MI355X) only", device,
                  prop.gcnArchName);
    }
    if (slot >= 0) g_dev_state[slot].store(st, std::memory_order_relaxed);
  }
  if (st == 2) return fail(HELM_E_ARCH, "device %d is not a gfx950 part", device);
  return HELM_OK;
}

int launch_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return HELM_OK;
  return fail(HELM_E_LAUNCH, "%s: %s", what, hipGetErrorString(e));
}

int run_transfer(helm::XferArgs& a, int32_t dtype, const int32_t* src_pos, const int32_t* tgt_pos,
                 double th_s, double th_t, hipStream_t stream, int stages = HELM_STAGE_ALL) {
  int rc = HELM_OK;
  if (stages & HELM_STAGE_TABLES)
    rc = launch_status(helm::launch_rope_tables(src_pos, tgt_pos, a.n_tok, a.D, th_s, th_t,
                                                const_cast<float2*>(a.rope_src),
                                                const_cast<float2*>(a.rope_tgt), stream),
                       "RoPE table kernel launch");
  if (rc != HELM_OK || !(stages & HELM_STAGE_MAP)) return rc;
  if (dtype == HELM_BF16 && helm::mfma_supports(a))
    rc = launch_status(helm::launch_transfer_mfma(a, stream), "matrix-core transfer kernel launch");
  else
    rc = launch_status(helm::launch_transfer_generic(a, dtype == HELM_BF16 ? helm::Dtype::BF16 : helm::Dtype::F32,
                                                     stream),
                       "transfer kernel launch");
  return rc;
}


// ---- ridge fit ---------------------------------------------------------
struct RidgeWorkspace {
  size_t gram, cross, sums, M, total;   // byte offsets of each part (sums: the sums, then the shifts), total size
};

int check_ridge_shape(const helm_ridge_shape_t* s) {
  if (!s) return fail(HELM_E_INVALID_ARG, "shape is NULL");
  if (s->dtype != HELM_BF16 && s->dtype != HELM_F32)
    return fail(HELM_E_DTYPE, "unknown dtype code %d (HELM_BF16=0, HELM_F32=1)", s->dtype);
  if (s->dtype != HELM_BF16) return fail(HELM_E_DTYPE, "the ridge fit takes bf16 observations only");
  if (s->out_features != 128)
    return fail(HELM_E_PAIR_SHAPE, "the ridge fit takes out_features = 128 (got %d)", s->out_features);
  if (s->in_features < 128 || s->in_features > 1024 || s->in_features % 128)
    return fail(HELM_E_PAIR_SHAPE, "in_features must be a multiple of 128 in [128, 1024] (got %d)",
                s->in_features);
  if (s->n_groups < 1 || s->n_obs < 1)
    return fail(HELM_E_INVALID_ARG, "n_groups = %lld and n_obs = %lld must be >= 1", (long long)s->n_groups,
                (long long)s->n_obs);
  if (s->n_obs > 0xffffff00LL / (2LL * s->in_features))
    return fail(HELM_E_INVALID_ARG, "one group's observations exceed 4 GB (n_obs = %lld)", (long long)s->n_obs);
  if (!(s->lambda >= 0.0) || std::isinf(s->lambda))
    return fail(HELM_E_INVALID_ARG, "lambda must be finite and >= 0");
  if (s->n_groups > 0x7fffffffLL / helm::ridge_tiles_per_group(s->in_features))
    return fail(HELM_E_INVALID_ARG, "too many groups (%lld)", (long long)s->n_groups);
  return HELM_OK;
}

bool ridge_workspace_layout(const helm_ridge_shape_t* s, RidgeWorkspace& w) {
  const int64_t G = s->n_groups, IN = s->in_features, D = s->out_features;
  int64_t g = G, c = G, u = G, m = G;
  if (!mul_ok(g, IN * IN * 4) || !mul_ok(c, IN * D * 4) || !mul_ok(u, (IN + D) * 8) || !mul_ok(m, IN * (IN + D) * 8))
    return false;
  w.gram = 0;
  w.cross = align_up((size_t)g);
  w.sums = w.cross + align_up((size_t)c);
  w.M = w.sums + align_up((size_t)u);
  w.total = w.M + align_up((size_t)m);
  return true;
}
}  // namespace

extern "C" {

int helm_abi_version(void) { return HELM_ABI_VERSION; }

const char* helm_last_error(void) { return g_err; }

const char* helm_status_string(int status) {
  switch (status) {
    case HELM_OK: return "HELM_OK";
    case HELM_E_INVALID_ARG: return "HELM_E_INVALID_ARG";
    case HELM_E_PAIR_SHAPE: return "HELM_E_PAIR_SHAPE";
    case HELM_E_LAYER_SEL: return "HELM_E_LAYER_SEL";
    case HELM_E_NO_DEVICE: return "HELM_E_NO_DEVICE";
    case HELM_E_DTYPE: return "HELM_E_DTYPE";
    case HELM_E_ARCH: return "HELM_E_ARCH";
    case HELM_E_WORKSPACE: return "HELM_E_WORKSPACE";
    case HELM_E_ALIAS: return "HELM_E_ALIAS";
    case HELM_E_PAGED_TABLE: return "HELM_E_PAGED_TABLE";
    case HELM_E_LAUNCH: return "HELM_E_LAUNCH";
    default: return "unknown";
  }
}

int helm_arch_supported(const char* name) {
  if (!name) return 0;
  // "gfx950" optionally followed by target features (":sramecc+:xnack-").
  return std::strncmp(name, "gfx950", 6) == 0 && (name[6] == '\0' || name[6] == ':') ? 1 : 0;
}

int helm_device_check(int device) {
  clear_error();
  return device_gate(device);
}

size_t helm_kv_workspace_bytes(const helm_shape_t* s) {
  clear_error();
  if (!s) { fail(HELM_E_INVALID_ARG, "shape is NULL"); return 0; }
  if (check_common(common_of(s)) != HELM_OK) return 0;
  if (s->n_tokens < 0) { fail(HELM_E_INVALID_ARG, "n_tokens < 0"); return 0; }
  Workspace w;
  if (!workspace_layout(s->n_tokens, s->head_dim, false, w)) { fail(HELM_E_INVALID_ARG, "size overflow"); return 0; }
  return w.total;
}

size_t helm_kv_paged_workspace_bytes(const helm_paged_shape_t* s) {
  clear_error();
  if (!s) { fail(HELM_E_INVALID_ARG, "shape is NULL"); return 0; }
  if (check_common(common_of(s)) != HELM_OK) return 0;
  if (s->n_tokens_total < 0) { fail(HELM_E_INVALID_ARG, "n_tokens_total < 0"); return 0; }
  Workspace w;
  if (!workspace_layout(s->n_tokens_total, s->head_dim, true, w)) { fail(HELM_E_INVALID_ARG, "size overflow"); return 0; }
  return w.total;
}

int helm_mapper_check(const helm_shape_t* s, const int32_t* sel) {
  clear_error();
  if (!s || !sel) return fail(HELM_E_INVALID_ARG, "shape or layer_sel_host is NULL");
  int rc = check_common(common_of(s));
  if (rc != HELM_OK) return rc;
  for (int64_t l = 0; l < s->n_tgt_layers; ++l)
    for (int64_t j = 0; j < s->k; ++j) {
      const int32_t v = sel[l * s->k + j];
      if (v < 0 || v >= s->n_src_layers)
        return fail(HELM_E_LAYER_SEL, "layer_sel[%lld][%lld] = %d lies outside [0, %d)", (long long)l,
                    (long long)j, v, s->n_src_layers);
    }
  return HELM_OK;
}

int helm_paged_check(const helm_paged_shape_t* s, const int32_t* sbt, const int32_t* tbt,
                     const int32_t* cu) {
  clear_error();
  if (!s || !sbt || !tbt || !cu) return fail(HELM_E_INVALID_ARG, "a NULL argument");
  int rc = check_common(common_of(s));
  if (rc != HELM_OK) return rc;
  if (s->block_size < 1 || s->n_requests < 1 || s->max_blocks_src < 1 || s->max_blocks_tgt < 1 ||
      s->n_src_blocks < 1 || s->n_tgt_blocks < 1)
    return fail(HELM_E_INVALID_ARG, "paged sizes must be >= 1");
  if (cu[0] != 0) return fail(HELM_E_PAGED_TABLE, "cu_seqlens[0] = %d, expected 0", cu[0]);
  const int32_t B = s->block_size;
  std::vector<uint8_t> used((size_t)s->n_tgt_blocks, 0);
  for (int32_t r = 0; r < s->n_requests; ++r) {
    const int64_t len = (int64_t)cu[r + 1] - cu[r];
    if (len < 0) return fail(HELM_E_PAGED_TABLE, "cu_seqlens decreases at request %d", r);
    const int64_t pages = (len + B - 1) / B;
    if (pages > s->max_blocks_src || pages > s->max_blocks_tgt)
      return fail(HELM_E_PAGED_TABLE, "request %d needs %lld pages; tables hold %d / %d", r,
                  (long long)pages, s->max_blocks_src, s->max_blocks_tgt);
    for (int64_t p = 0; p < pages; ++p) {
      const int32_t a = sbt[(int64_t)r * s->max_blocks_src + p];
      const int32_t b = tbt[(int64_t)r * s->max_blocks_tgt + p];
      if (a < 0 || a >= s->n_src_blocks)
        return fail(HELM_E_PAGED_TABLE, "src_block_table[%d][%lld] = %d lies outside [0, %d)", r,
                    (long long)p, a, s->n_src_blocks);
      if (b < 0 || b >= s->n_tgt_blocks)
        return fail(HELM_E_PAGED_TABLE, "tgt_block_table[%d][%lld] = %d lies outside [0, %d)", r,
                    (long long)p, b, s->n_tgt_blocks);
      if (used[(size_t)b])
        return fail(HELM_E_PAGED_TABLE, "target block %d is used twice (request %d, page %lld)", b, r,
                    (long long)p);
      used[(size_t)b] = 1;
    }
  }
  if ((int64_t)cu[s->n_requests] != s->n_tokens_total)
    return fail(HELM_E_PAGED_TABLE, "cu_seqlens[R] = %d but n_tokens_total = %lld", cu[s->n_requests],
                (long long)s->n_tokens_total);
  return HELM_OK;
}

}  // extern "C"

namespace {
// Every check of the contiguous transfer, then its kernel arguments.  With
// need_workspace false (the path query) the workspace fields are not read
// and the tables' addresses stand for any 256-byte aligned workspace.
int contiguous_args(const void* src_k, const void* src_v, const int32_t* src_pos, const int32_t* tgt_pos,
                    const int32_t* layer_sel, const void* W_k, const float* b_k, const void* W_v, const float* b_v,
                    void* out_k, void* out_v, const helm_shape_t* s, bool need_workspace, helm::XferArgs& a) {
  if (!s) return fail(HELM_E_INVALID_ARG, "shape is NULL");
  int rc = check_common(common_of(s));
  if (rc != HELM_OK) return rc;
  if (s->n_tokens < 0) return fail(HELM_E_INVALID_ARG, "n_tokens = %lld < 0", (long long)s->n_tokens);
  if (s->n_tokens > 0x7fffffffLL) return fail(HELM_E_INVALID_ARG, "n_tokens exceeds 2^31-1");
  if (s->n_tokens == 0) return HELM_OK;   // nothing to map; no pointer or device is touched
  if (!src_k || !src_v || !src_pos || !tgt_pos || !layer_sel || !W_k || !b_k || !W_v || !b_v || !out_k ||
      !out_v)
    return fail(HELM_E_INVALID_ARG, "a tensor pointer is NULL");

  const int64_t es = (int64_t)elem_bytes(s->dtype);
  int64_t src_b = s->n_src_layers, out_b = s->n_tgt_layers, w_b = s->n_tgt_layers, b_b = s->n_tgt_layers;
  if (!mul_ok(src_b, s->n_kv_heads) || !mul_ok(src_b, s->n_tokens) || !mul_ok(src_b, s->head_dim) ||
      !mul_ok(src_b, es) || !mul_ok(out_b, s->n_kv_heads) || !mul_ok(out_b, s->n_tokens) ||
      !mul_ok(out_b, s->head_dim) || !mul_ok(out_b, es) || !mul_ok(w_b, s->n_kv_heads) ||
      !mul_ok(w_b, (int64_t)s->k * s->head_dim) || !mul_ok(w_b, s->head_dim) || !mul_ok(w_b, es) ||
      !mul_ok(b_b, s->n_kv_heads) || !mul_ok(b_b, (int64_t)s->head_dim * 4))
    return fail(HELM_E_INVALID_ARG, "tensor sizes overflow int64");

  const int64_t pos_b = s->n_tokens * 4, sel_b = (int64_t)s->n_tgt_layers * s->k * 4;
  const struct { const void* p; int64_t n; const char* name; } ins[] = {
      {src_k, src_b, "src_k"}, {src_v, src_b, "src_v"}, {src_pos, pos_b, "src_pos"},
      {tgt_pos, pos_b, "tgt_pos"}, {layer_sel, sel_b, "layer_sel"}, {W_k, w_b, "W_k"},
      {b_k, b_b, "b_k"}, {W_v, w_b, "W_v"}, {b_v, b_b, "b_v"}};
  for (const auto& in : ins) {
    if (overlaps(out_k, out_b, in.p, in.n)) return fail(HELM_E_ALIAS, "out_k overlaps %s", in.name);
    if (overlaps(out_v, out_b, in.p, in.n)) return fail(HELM_E_ALIAS, "out_v overlaps %s", in.name);
  }
  if (overlaps(out_k, out_b, out_v, out_b)) return fail(HELM_E_ALIAS, "out_k overlaps out_v");

  Workspace w;
  if (!workspace_layout(s->n_tokens, s->head_dim, false, w)) return fail(HELM_E_INVALID_ARG, "size overflow");
  char* ws = (char*)(uintptr_t)kAlign;   // stands for any aligned workspace (path query)
  if (need_workspace) {
    if (!s->workspace || s->workspace_bytes < w.total)
      return fail(HELM_E_WORKSPACE, "workspace of %zu bytes at %p; %zu bytes needed", s->workspace_bytes,
                  s->workspace, w.total);
    if ((uintptr_t)s->workspace % kAlign)
      return fail(HELM_E_WORKSPACE, "workspace %p is not %zu-byte aligned", s->workspace, kAlign);
    for (const auto& in : ins)
      if (overlaps(s->workspace, (int64_t)w.total, in.p, in.n))
        return fail(HELM_E_ALIAS, "workspace overlaps %s", in.name);
    if (overlaps(s->workspace, (int64_t)w.total, out_k, out_b) ||
        overlaps(s->workspace, (int64_t)w.total, out_v, out_b))
      return fail(HELM_E_ALIAS, "workspace overlaps an output");
    ws = (char*)s->workspace;
  }

  rc = device_gate(-1);
  if (rc != HELM_OK) return rc;

  a = helm::XferArgs{};
  a.src_k = src_k; a.src_v = src_v; a.layer_sel = layer_sel;
  a.W_k = W_k; a.b_k = b_k; a.W_v = W_v; a.b_v = b_v; a.out_k = out_k; a.out_v = out_v;
  a.rope_src = (const float2*)ws;
  a.rope_tgt = (const float2*)(ws + w.rope_bytes);
  a.src_row = nullptr; a.dst_row = nullptr;
  a.n_tok = s->n_tokens;
  a.L_s = s->n_src_layers; a.L_t = s->n_tgt_layers; a.H = s->n_kv_heads; a.D = s->head_dim; a.k = s->k;
  a.src_tok = s->head_dim; a.src_head = s->n_tokens * s->head_dim; a.src_layer = a.src_head * s->n_kv_heads;
  a.dst_tok = a.src_tok; a.dst_head = a.src_head; a.dst_layer = a.src_layer;
  a.src_rows = a.dst_rows = s->n_tokens;
  return HELM_OK;
}
}  // namespace

extern "C" {

int helm_kv_transfer_stage(int stages, const void* src_k, const void* src_v, const int32_t* src_pos,
                           const int32_t* tgt_pos, const int32_t* layer_sel, const void* W_k,
                           const float* b_k, const void* W_v, const float* b_v, void* out_k, void* out_v,
                           const helm_shape_t* s) {
  clear_error();
  if (stages < HELM_STAGE_TABLES || stages > HELM_STAGE_ALL)
    return fail(HELM_E_INVALID_ARG, "stages = %d; expected 1 (tables), 2 (map) or 3 (both)", stages);
  helm::XferArgs a;
  const int rc = contiguous_args(src_k, src_v, src_pos, tgt_pos, layer_sel, W_k, b_k, W_v, b_v, out_k, out_v, s,
                                 true, a);
  if (rc != HELM_OK || s->n_tokens == 0) return rc;
  return run_transfer(a, s->dtype, src_pos, tgt_pos, s->rope_theta_src, s->rope_theta_tgt,
                      (hipStream_t)s->stream, stages);
}

}  // extern "C"

namespace {
// ---- allocation-free variant --------------------------------------------
// The transfer's one scratch buffer is its pair of RoPE (cos, sin) tables.
// For callers that cannot allocate, they live in this file-scope device
// array: one copy per GPU the library runs on, held until the process ends.
// 64 MiB holds the tables of 65,536 tokens at head_dim 128 (131,072 at 64).
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of `scratch` on each device, looked up once per device with
// that device current (host code never passes the array's own name: on the
// host it only stands for the symbol, not a device address).
std::atomic<uintptr_t> g_scratch_addr[kMaxDevices];

int scratch_of_current_device(char** out) {
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(HELM_E_NO_DEVICE, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(HELM_E_INVALID_ARG, "device %d is beyond the %d devices the static scratch is kept for", dev,
                kMaxDevices);
  uintptr_t p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p == 0) {
    void* addr = nullptr;
    const hipError_t r = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (r != hipSuccess || addr == nullptr)
      return fail(HELM_E_LAUNCH, "hipGetSymbolAddress of the static scratch failed: %s", hipGetErrorString(r));
    p = (uintptr_t)addr;
    g_scratch_addr[dev].store(p, std::memory_order_release);
  }
  *out = (char*)p;
  return HELM_OK;
}
}  // namespace

extern "C" {

size_t helm_kv_noalloc_max_bytes(void) { return kScratchBytes; }

int helm_kv_transfer_noalloc(const void* src_k, const void* src_v, const int32_t* src_pos, const int32_t* tgt_pos,
                             const int32_t* layer_sel, const void* W_k, const float* b_k, const void* W_v,
                             const float* b_v, void* out_k, void* out_v, const helm_shape_t* s) {
  clear_error();
  helm::XferArgs a;
  int rc = contiguous_args(src_k, src_v, src_pos, tgt_pos, layer_sel, W_k, b_k, W_v, b_v, out_k, out_v, s, false,
                           a);
  if (rc != HELM_OK || s->n_tokens == 0) return rc;
  Workspace w;
  if (!workspace_layout(s->n_tokens, s->head_dim, false, w)) return fail(HELM_E_INVALID_ARG, "size overflow");
  if (w.total > kScratchBytes)
    return fail(HELM_E_WORKSPACE,
                "n_tokens = %lld needs %zu bytes of tables; the static scratch holds %zu (up to %lld tokens at "
                "head_dim %d)",
                (long long)s->n_tokens, w.total, kScratchBytes,
                (long long)(kScratchBytes / (2 * (size_t)s->head_dim / 2 * sizeof(float2))), s->head_dim);
  char* ws = nullptr;
  rc = scratch_of_current_device(&ws);
  if (rc != HELM_OK) return rc;
  a.rope_src = (const float2*)ws;
  a.rope_tgt = (const float2*)(ws + w.rope_bytes);
  return run_transfer(a, s->dtype, src_pos, tgt_pos, s->rope_theta_src, s->rope_theta_tgt, (hipStream_t)s->stream,
                      HELM_STAGE_ALL);
}

int helm_kv_transfer_path(const void* src_k, const void* src_v, const int32_t* src_pos, const int32_t* tgt_pos,
                          const int32_t* layer_sel, const void* W_k, const float* b_k, const void* W_v,
                          const float* b_v, void* out_k, void* out_v, const helm_shape_t* s, int* path_out) {
  clear_error();
  if (!path_out) return fail(HELM_E_INVALID_ARG, "path_out is NULL");
  helm::XferArgs a;
  const int rc = contiguous_args(src_k, src_v, src_pos, tgt_pos, layer_sel, W_k, b_k, W_v, b_v, out_k, out_v, s,
                                 false, a);
  if (rc != HELM_OK) return rc;
  if (s->n_tokens == 0) {
    *path_out = s->dtype == HELM_BF16 && s->head_dim == 128 && s->k <= 4 ? HELM_PATH_MATRIX : HELM_PATH_PORTABLE;
    return HELM_OK;
  }
  *path_out = s->dtype == HELM_BF16 && helm::mfma_supports(a) ? HELM_PATH_MATRIX : HELM_PATH_PORTABLE;
  return HELM_OK;
}

int helm_kv_transfer(const void* src_k, const void* src_v, const int32_t* src_pos,
                     const int32_t* tgt_pos, const int32_t* layer_sel, const void* W_k,
                     const float* b_k, const void* W_v, const float* b_v, void* out_k, void* out_v,
                     const helm_shape_t* s) {
  return helm_kv_transfer_stage(HELM_STAGE_ALL, src_k, src_v, src_pos, tgt_pos, layer_sel, W_k, b_k, W_v, b_v,
                                out_k, out_v, s);
}

int helm_kv_transfer_paged(const void* src_k_pool, const void* src_v_pool, const int32_t* src_bt,
                           const int32_t* tgt_bt, const int32_t* cu, const int32_t* src_pos,
                           const int32_t* tgt_pos, const int32_t* layer_sel, const void* W_k,
                           const float* b_k, const void* W_v, const float* b_v, void* tgt_k_pool,
                           void* tgt_v_pool, const helm_paged_shape_t* s) {
  clear_error();
  if (!s) return fail(HELM_E_INVALID_ARG, "shape is NULL");
  int rc = check_common(common_of(s));
  if (rc != HELM_OK) return rc;
  if (s->block_size < 1 || s->n_requests < 1 || s->max_blocks_src < 1 || s->max_blocks_tgt < 1 ||
      s->n_src_blocks < 1 || s->n_tgt_blocks < 1)
    return fail(HELM_E_INVALID_ARG, "paged sizes must be >= 1");
  if (s->n_tokens_total < 0 || s->n_tokens_total > 0x7fffffffLL)
    return fail(HELM_E_INVALID_ARG, "n_tokens_total = %lld outside [0, 2^31)", (long long)s->n_tokens_total);
  if (s->n_tokens_total == 0) return HELM_OK;   // nothing to map; no pointer or device is touched
  if ((int64_t)s->n_src_blocks * s->block_size > 0x7fffffffLL ||
      (int64_t)s->n_tgt_blocks * s->block_size > 0x7fffffffLL)
    return fail(HELM_E_INVALID_ARG, "pool slot counts must stay below 2^31");
  if (!src_k_pool || !src_v_pool || !src_bt || !tgt_bt || !cu || !src_pos || !tgt_pos || !layer_sel || !W_k ||
      !b_k || !W_v || !b_v || !tgt_k_pool || !tgt_v_pool)
    return fail(HELM_E_INVALID_ARG, "a tensor pointer is NULL");

  const int64_t es = (int64_t)elem_bytes(s->dtype);
  int64_t src_b = s->n_src_layers, out_b = s->n_tgt_layers, w_b = s->n_tgt_layers, b_b = s->n_tgt_layers;
  if (!mul_ok(src_b, s->n_src_blocks) || !mul_ok(src_b, s->block_size) || !mul_ok(src_b, s->n_kv_heads) ||
      !mul_ok(src_b, s->head_dim) || !mul_ok(src_b, es) || !mul_ok(out_b, s->n_tgt_blocks) ||
      !mul_ok(out_b, s->block_size) || !mul_ok(out_b, s->n_kv_heads) || !mul_ok(out_b, s->head_dim) ||
      !mul_ok(out_b, es) || !mul_ok(w_b, s->n_kv_heads) || !mul_ok(w_b, (int64_t)s->k * s->head_dim) ||
      !mul_ok(w_b, s->head_dim) || !mul_ok(w_b, es) || !mul_ok(b_b, s->n_kv_heads) ||
      !mul_ok(b_b, (int64_t)s->head_dim * 4))
    return fail(HELM_E_INVALID_ARG, "tensor sizes overflow int64");
  const int64_t pos_b = s->n_tokens_total * 4, sel_b = (int64_t)s->n_tgt_layers * s->k * 4;
  const int64_t sbt_b = (int64_t)s->n_requests * s->max_blocks_src * 4;
  const int64_t tbt_b = (int64_t)s->n_requests * s->max_blocks_tgt * 4;
  const struct { const void* p; int64_t n; const char* name; } ins[] = {
      {src_k_pool, src_b, "src_k_pool"}, {src_v_pool, src_b, "src_v_pool"}, {src_bt, sbt_b, "src_block_table"},
      {tgt_bt, tbt_b, "tgt_block_table"}, {cu, (int64_t)(s->n_requests + 1) * 4, "cu_seqlens"},
      {src_pos, pos_b, "src_pos"}, {tgt_pos, pos_b, "tgt_pos"}, {layer_sel, sel_b, "layer_sel"},
      {W_k, w_b, "W_k"}, {b_k, b_b, "b_k"}, {W_v, w_b, "W_v"}, {b_v, b_b, "b_v"}};
  for (const auto& in : ins) {
    if (overlaps(tgt_k_pool, out_b, in.p, in.n)) return fail(HELM_E_ALIAS, "tgt_k_pool overlaps %s", in.name);
    if (overlaps(tgt_v_pool, out_b, in.p, in.n)) return fail(HELM_E_ALIAS, "tgt_v_pool overlaps %s", in.name);
  }
  if (overlaps(tgt_k_pool, out_b, tgt_v_pool, out_b)) return fail(HELM_E_ALIAS, "tgt_k_pool overlaps tgt_v_pool");

  Workspace w;
  if (!workspace_layout(s->n_tokens_total, s->head_dim, true, w)) return fail(HELM_E_INVALID_ARG, "size overflow");
  if (!s->workspace || s->workspace_bytes < w.total)
    return fail(HELM_E_WORKSPACE, "workspace of %zu bytes at %p; %zu bytes needed", s->workspace_bytes,
                s->workspace, w.total);
  if ((uintptr_t)s->workspace % kAlign)
    return fail(HELM_E_WORKSPACE, "workspace %p is not %zu-byte aligned", s->workspace, kAlign);
  for (const auto& in : ins)
    if (overlaps(s->workspace, (int64_t)w.total, in.p, in.n))
      return fail(HELM_E_ALIAS, "workspace overlaps %s", in.name);
  if (overlaps(s->workspace, (int64_t)w.total, tgt_k_pool, out_b) ||
      overlaps(s->workspace, (int64_t)w.total, tgt_v_pool, out_b))
    return fail(HELM_E_ALIAS, "workspace overlaps an output pool");

  rc = device_gate(-1);
  if (rc != HELM_OK) return rc;
  if (s->n_tokens_total == 0) return HELM_OK;

  char* ws = (char*)s->workspace;
  helm::XferArgs a{};
  a.src_k = src_k_pool; a.src_v = src_v_pool; a.layer_sel = layer_sel;
  a.W_k = W_k; a.b_k = b_k; a.W_v = W_v; a.b_v = b_v; a.out_k = tgt_k_pool; a.out_v = tgt_v_pool;
  a.rope_src = (const float2*)ws;
  a.rope_tgt = (const float2*)(ws + w.rope_bytes);
  int32_t* src_row = (int32_t*)(ws + 2 * w.rope_bytes);
  int32_t* dst_row = (int32_t*)(ws + 2 * w.rope_bytes + w.rows_bytes);
  a.src_row = src_row; a.dst_row = dst_row;
  a.n_tok = s->n_tokens_total;
  a.L_s = s->n_src_layers; a.L_t = s->n_tgt_layers; a.H = s->n_kv_heads; a.D = s->head_dim; a.k = s->k;
  a.src_tok = (int64_t)s->n_kv_heads * s->head_dim; a.src_head = s->head_dim;
  a.src_layer = (int64_t)s->n_src_blocks * s->block_size * a.src_tok;
  a.dst_tok = a.src_tok; a.dst_head = a.src_head;
  a.dst_layer = (int64_t)s->n_tgt_blocks * s->block_size * a.dst_tok;
  a.src_rows = (int64_t)s->n_src_blocks * s->block_size;
  a.dst_rows = (int64_t)s->n_tgt_blocks * s->block_size;

  const hipStream_t stream = (hipStream_t)s->stream;
  rc = launch_status(helm::launch_paged_rows(cu, s->n_requests, src_bt, s->max_blocks_src, s->n_src_blocks,
                                             tgt_bt, s->max_blocks_tgt, s->n_tgt_blocks, s->block_size,
                                             s->n_tokens_total, src_row, dst_row, stream),
                     "paged slot kernel launch");
  if (rc != HELM_OK) return rc;
  return run_transfer(a, s->dtype, src_pos, tgt_pos, s->rope_theta_src, s->rope_theta_tgt, stream);
}

// Wide-input map workspace: [rope_src][rope_tgt] (K1 tables) [U: L_s*H*T*D bf16]
// [WT_k: L_t*H*D*IN bf16][WT_v: same].
struct WideWorkspace {
  size_t rope_bytes = 0, u_bytes = 0, wt_bytes = 0, total = 0;
};

static bool wide_workspace_layout(const helm_shape_t* s, WideWorkspace& w) {
  Workspace base;
  if (!workspace_layout(s->n_tokens, s->head_dim, false, base)) return false;
  int64_t u = s->n_src_layers, wt = s->n_tgt_layers;
  const int64_t IN = helm::wide_in_features(s->k, s->n_kv_heads, s->head_dim);
  if (!mul_ok(u, s->n_kv_heads) || !mul_ok(u, s->n_tokens) || !mul_ok(u, s->head_dim) || !mul_ok(u, 2) ||
      !mul_ok(wt, s->n_kv_heads) || !mul_ok(wt, s->head_dim) || !mul_ok(wt, IN) || !mul_ok(wt, 2))
    return false;
  w.rope_bytes = base.rope_bytes;
  w.u_bytes = align_up((size_t)u);
  w.wt_bytes = align_up((size_t)wt);
  w.total = 2 * w.rope_bytes + w.u_bytes + 2 * w.wt_bytes;
  if (w.total == 0) w.total = kAlign;
  return true;
}

static int check_wide_shape(const helm_shape_t* s) {
  if (!s) return fail(HELM_E_INVALID_ARG, "shape is NULL");
  int rc = check_common(common_of(s));
  if (rc != HELM_OK) return rc;
  if (s->dtype != HELM_BF16) return fail(HELM_E_DTYPE, "the wide-input map runs on bf16 caches and maps only");
  if (s->head_dim != 128) return fail(HELM_E_PAIR_SHAPE, "the wide-input map needs head_dim 128 (got %d)", s->head_dim);
  if (s->n_tokens < 0) return fail(HELM_E_INVALID_ARG, "n_tokens = %lld < 0", (long long)s->n_tokens);
  if (s->n_tokens > 0x7fffffffLL) return fail(HELM_E_INVALID_ARG, "n_tokens exceeds 2^31-1");
  return HELM_OK;
}

size_t helm_kv_wide_workspace_bytes(const helm_shape_t* s) {
  clear_error();
  if (check_wide_shape(s) != HELM_OK) return 0;
  WideWorkspace w;
  if (!wide_workspace_layout(s, w)) { fail(HELM_E_INVALID_ARG, "size overflow"); return 0; }
  return w.total;
}

int helm_kv_transfer_wide_stage(int stages, const void* src_k, const void* src_v, const int32_t* src_pos,
                                const int32_t* tgt_pos, const int32_t* layer_sel, const void* W_k, const float* b_k,
                                const void* W_v, const float* b_v, void* out_k, void* out_v,
                                const helm_shape_t* s) {
  clear_error();
  if (stages < 1 || stages > HELM_STAGE_ALL) return fail(HELM_E_INVALID_ARG, "stages = %d is not 1, 2 or 3", stages);
  int rc = check_wide_shape(s);
  if (rc != HELM_OK) return rc;
  if (s->n_tokens == 0) return HELM_OK;   // nothing to map; no pointer or device is touched
  if (!src_k || !src_v || !src_pos || !tgt_pos || !layer_sel || !W_k || !b_k || !W_v || !b_v || !out_k ||
      !out_v)
    return fail(HELM_E_INVALID_ARG, "a tensor pointer is NULL");
  const int64_t IN = helm::wide_in_features(s->k, s->n_kv_heads, s->head_dim);
  int64_t src_b = s->n_src_layers, out_b = s->n_tgt_layers, w_b = s->n_tgt_layers, b_b = s->n_tgt_layers;
  if (!mul_ok(src_b, s->n_kv_heads) || !mul_ok(src_b, s->n_tokens) || !mul_ok(src_b, s->head_dim * 2) ||
      !mul_ok(out_b, s->n_kv_heads) || !mul_ok(out_b, s->n_tokens) || !mul_ok(out_b, s->head_dim * 2) ||
      !mul_ok(w_b, s->n_kv_heads) || !mul_ok(w_b, IN) || !mul_ok(w_b, s->head_dim * 2) ||
      !mul_ok(b_b, s->n_kv_heads) || !mul_ok(b_b, (int64_t)s->head_dim * 4))
    return fail(HELM_E_INVALID_ARG, "tensor sizes overflow int64");
  const int64_t pos_b = s->n_tokens * 4, sel_b = (int64_t)s->n_tgt_layers * s->k * 4;
  const struct { const void* p; int64_t n; const char* name; } ins[] = {
      {src_k, src_b, "src_k"}, {src_v, src_b, "src_v"}, {src_pos, pos_b, "src_pos"},
      {tgt_pos, pos_b, "tgt_pos"}, {layer_sel, sel_b, "layer_sel"}, {W_k, w_b, "W_k"},
      {b_k, b_b, "b_k"}, {W_v, w_b, "W_v"}, {b_v, b_b, "b_v"}};
  for (const auto& in : ins) {
    if (overlaps(out_k, out_b, in.p, in.n)) return fail(HELM_E_ALIAS, "out_k overlaps %s", in.name);
    if (overlaps(out_v, out_b, in.p, in.n)) return fail(HELM_E_ALIAS, "out_v overlaps %s", in.name);
  }
  if (overlaps(out_k, out_b, out_v, out_b)) return fail(HELM_E_ALIAS, "out_k overlaps out_v");
  WideWorkspace w;
  if (!wide_workspace_layout(s, w)) return fail(HELM_E_INVALID_ARG, "size overflow");
  if (!s->workspace || s->workspace_bytes < w.total)
    return fail(HELM_E_WORKSPACE, "workspace of %zu bytes at %p; %zu bytes needed", s->workspace_bytes,
                s->workspace, w.total);
  if ((uintptr_t)s->workspace % kAlign)
    return fail(HELM_E_WORKSPACE, "workspace %p is not %zu-byte aligned", s->workspace, kAlign);
  for (const auto& in : ins)
    if (overlaps(s->workspace, (int64_t)w.total, in.p, in.n))
      return fail(HELM_E_ALIAS, "workspace overlaps %s", in.name);
  if (overlaps(s->workspace, (int64_t)w.total, out_k, out_b) || overlaps(s->workspace, (int64_t)w.total, out_v, out_b))
    return fail(HELM_E_ALIAS, "workspace overlaps an output");

  char* ws = (char*)s->workspace;
  helm::WideXfer x{};
  x.src_k = src_k; x.src_v = src_v; x.layer_sel = layer_sel;
  x.W_k = W_k; x.b_k = b_k; x.W_v = W_v; x.b_v = b_v; x.out_k = out_k; x.out_v = out_v;
  x.rope_src = (const float2*)ws;
  x.rope_tgt = (const float2*)(ws + w.rope_bytes);
  x.U = (uint16_t*)(ws + 2 * w.rope_bytes);
  x.WT_k = (uint16_t*)(ws + 2 * w.rope_bytes + w.u_bytes);
  x.WT_v = (uint16_t*)(ws + 2 * w.rope_bytes + w.u_bytes + w.wt_bytes);
  x.L_s = s->n_src_layers; x.L_t = s->n_tgt_layers; x.H = s->n_kv_heads; x.D = s->head_dim; x.k = s->k;
  x.T = (int32_t)s->n_tokens;
  if ((uintptr_t)out_k % 16 || (uintptr_t)out_v % 16)
    return fail(HELM_E_INVALID_ARG, "the wide-input map stores 16-byte pieces: out_k %p and out_v %p must be 16-byte aligned",
                out_k, out_v);
  if (!helm::wide_supports(x))
    return fail(HELM_E_INVALID_ARG, "the wide-input map needs 16-byte aligned caches and a cache slab below 4 GB");
  rc = device_gate(-1);
  if (rc != HELM_OK) return rc;
  const hipStream_t stream = (hipStream_t)s->stream;
  if (stages & HELM_STAGE_TABLES) {
    rc = launch_status(helm::launch_rope_tables(src_pos, tgt_pos, s->n_tokens, s->head_dim, s->rope_theta_src,
                                                s->rope_theta_tgt, const_cast<float2*>(x.rope_src),
                                                const_cast<float2*>(x.rope_tgt), stream),
                       "RoPE table kernel launch");
    if (rc != HELM_OK) return rc;
  }
  return launch_status(helm::launch_wide(x, stages & HELM_STAGE_TABLES, stages & HELM_STAGE_MAP, stream),
                       "wide-input map launch");
}

int helm_kv_transfer_wide(const void* src_k, const void* src_v, const int32_t* src_pos, const int32_t* tgt_pos,
                          const int32_t* layer_sel, const void* W_k, const float* b_k, const void* W_v,
                          const float* b_v, void* out_k, void* out_v, const helm_shape_t* s) {
  return helm_kv_transfer_wide_stage(HELM_STAGE_ALL, src_k, src_v, src_pos, tgt_pos, layer_sel, W_k, b_k, W_v, b_v,
                                     out_k, out_v, s);
}

int helm_kv_cosine(const void* k_mapped, const void* v_mapped, const void* k_ref, const void* v_ref,
                   float* cos_out, const helm_shape_t* s) {
  clear_error();
  if (!s) return fail(HELM_E_INVALID_ARG, "shape is NULL");
  int rc = check_common(common_of(s));
  if (rc != HELM_OK) return rc;
  if (s->n_tokens < 0) return fail(HELM_E_INVALID_ARG, "n_tokens = %lld < 0", (long long)s->n_tokens);
  if (s->n_tokens > 0x7fffffffLL) return fail(HELM_E_INVALID_ARG, "n_tokens exceeds 2^31-1");
  if (!cos_out) return fail(HELM_E_INVALID_ARG, "cos_out is NULL");
  if (s->n_tokens > 0 && (!k_mapped || !v_mapped || !k_ref || !v_ref))
    return fail(HELM_E_INVALID_ARG, "a cache pointer is NULL");
  const int64_t es = (int64_t)elem_bytes(s->dtype);
  int64_t slab = s->n_tokens, cache_b = s->n_tgt_layers;
  if (!mul_ok(slab, s->head_dim) || !mul_ok(cache_b, s->n_kv_heads) || !mul_ok(cache_b, slab) ||
      !mul_ok(cache_b, es))
    return fail(HELM_E_INVALID_ARG, "cache sizes overflow int64");
  const int64_t n_slabs = (int64_t)s->n_tgt_layers * s->n_kv_heads;
  const int64_t out_b = 2 * n_slabs * (int64_t)sizeof(float);
  const struct { const void* p; const char* name; } ins[] = {
      {k_mapped, "k_mapped"}, {v_mapped, "v_mapped"}, {k_ref, "k_ref"}, {v_ref, "v_ref"}};
  for (const auto& in : ins)
    if (overlaps(cos_out, out_b, in.p, cache_b)) return fail(HELM_E_ALIAS, "cos_out overlaps %s", in.name);
  rc = device_gate(-1);
  if (rc != HELM_OK) return rc;
  return launch_status(helm::launch_kv_cosine(k_mapped, v_mapped, k_ref, v_ref, n_slabs, slab,
                                              s->dtype == HELM_BF16 ? helm::Dtype::BF16 : helm::Dtype::F32,
                                              cos_out, (hipStream_t)s->stream),
                       "KV-cosine kernel launch");
}

size_t helm_ridge_workspace_bytes(const helm_ridge_shape_t* s) {
  clear_error();
  if (check_ridge_shape(s) != HELM_OK) return 0;
  RidgeWorkspace w;
  if (!ridge_workspace_layout(s, w)) { fail(HELM_E_INVALID_ARG, "size overflow"); return 0; }
  return w.total;
}

int helm_ridge_fit_stage(int stages, const void* X, const void* Y, float* W, float* b,
                         const helm_ridge_shape_t* s) {
  clear_error();
  if (stages < 1 || stages > HELM_STAGE_ALL) return fail(HELM_E_INVALID_ARG, "stages = %d is not 1, 2 or 3", stages);
  int rc = check_ridge_shape(s);
  if (rc != HELM_OK) return rc;
  if (!X || !Y || !W || !b) return fail(HELM_E_INVALID_ARG, "a tensor pointer is NULL");
  if ((uintptr_t)X % 16 || (uintptr_t)Y % 16) return fail(HELM_E_INVALID_ARG, "X and Y must be 16-byte aligned");
  const int64_t G = s->n_groups, N = s->n_obs, IN = s->in_features, D = s->out_features;
  int64_t x_b = G, y_b = G, w_b = G, b_b = G;
  if (!mul_ok(x_b, N) || !mul_ok(x_b, IN * 2) || !mul_ok(y_b, N) || !mul_ok(y_b, D * 2) || !mul_ok(w_b, IN * D * 4) ||
      !mul_ok(b_b, D * 4))
    return fail(HELM_E_INVALID_ARG, "tensor sizes overflow int64");
  RidgeWorkspace w;
  if (!ridge_workspace_layout(s, w)) return fail(HELM_E_INVALID_ARG, "size overflow");
  if (!s->workspace || s->workspace_bytes < w.total)
    return fail(HELM_E_WORKSPACE, "workspace of %zu bytes at %p; %zu bytes needed", s->workspace_bytes,
                s->workspace, w.total);
  if ((uintptr_t)s->workspace % kAlign)
    return fail(HELM_E_WORKSPACE, "workspace %p is not %zu-byte aligned", s->workspace, kAlign);
  const struct { const void* p; int64_t n; const char* name; } outs[] = {
      {W, w_b, "W"}, {b, b_b, "b"}, {s->workspace, (int64_t)w.total, "the workspace"}};
  const struct { const void* p; int64_t n; const char* name; } ins[] = {{X, x_b, "X"}, {Y, y_b, "Y"}};
  for (int i = 0; i < 3; ++i) {
    for (const auto& in : ins)
      if (overlaps(outs[i].p, outs[i].n, in.p, in.n)) return fail(HELM_E_ALIAS, "%s overlaps %s", outs[i].name, in.name);
    for (int j = i + 1; j < 3; ++j)
      if (overlaps(outs[i].p, outs[i].n, outs[j].p, outs[j].n))
        return fail(HELM_E_ALIAS, "%s overlaps %s", outs[i].name, outs[j].name);
  }
  char* ws = (char*)s->workspace;
  helm::RidgeFit f{};
  f.X = X;
  f.Y = Y;
  f.gram = (float*)(ws + w.gram);
  f.cross = (float*)(ws + w.cross);
  f.sums = (float*)(ws + w.sums);
  f.shift = f.sums + s->n_groups * (int64_t)(s->in_features + s->out_features);
  f.M = (double*)(ws + w.M);
  f.W = W;
  f.b = b;
  f.G = G;
  f.N = N;
  f.IN = (int32_t)IN;
  f.D = (int32_t)D;
  f.lambda = s->lambda;
  if (!helm::ridge_supports(f)) return fail(HELM_E_INVALID_ARG, "shape outside the ridge kernels' limits");
  rc = device_gate(-1);
  if (rc != HELM_OK) return rc;
  return launch_status(helm::launch_ridge(f, stages & HELM_STAGE_TABLES, stages & HELM_STAGE_MAP,
                                          (hipStream_t)s->stream),
                       "ridge fit launch");
}

int helm_ridge_fit(const void* X, const void* Y, float* W, float* b, const helm_ridge_shape_t* s) {
  return helm_ridge_fit_stage(HELM_STAGE_ALL, X, Y, W, b, s);
}

}  // extern "C"
