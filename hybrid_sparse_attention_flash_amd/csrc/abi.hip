// C ABI of libhys: argument validation, launch configuration and dispatch.
// Every check runs on the host before any GPU work; failures return a status
// and leave a thread-local message (see include/hys.h for the contract).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <string>

#include "../../include/hys.h"
#include "bwd.h"
#include "kernels.h"

namespace {

thread_local std::string g_last_error;

hys_status fail(hys_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

hys_status ok() {
  g_last_error.clear();
  return HYS_OK;
}

hys_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(HYS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t elem_size(int32_t dt) { return dt == HYS_F32 ? 4 : (dt == HYS_BF16 ? 2 : 1); }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// ---------------------------------------------------------------------------
// Launch-arithmetic checks of the debug build (compiled with -DHYS_DEBUG).
// Before each launch the derived configuration (work decomposition, grid,
// score and workspace layout, 32-bit offsets the kernels form) is re-derived
// from the shapes and compared; a violation returns HYS_ERR_INTERNAL naming
// the broken invariant.  In the normal build the checks compile to nothing.
#ifdef HYS_DEBUG
#define HYS_DCHECK(cond)                                                                                   \
  do {                                                                                                     \
    if (!(cond)) return fail(HYS_ERR_INTERNAL, "launch check failed: %s (line %d)", #cond, __LINE__);     \
  } while (0)
#else
#define HYS_DCHECK(cond) \
  do {                   \
  } while (0)
#endif


// Shape/stride sanity of one [B, T, H, D] tensor.
hys_status check_tensor(const hys_tensor4& t, const char* name, bool allow_fp8) {
  if (!t.ptr) return fail(HYS_ERR_INVALID_ARG, "%s: null pointer", name);
  if (t.dtype != HYS_F32 && t.dtype != HYS_BF16 && t.dtype != HYS_FP8_E4M3)
    return fail(HYS_ERR_INVALID_ARG, "%s: unknown dtype %d", name, (int)t.dtype);
  if (t.dtype == HYS_FP8_E4M3 && !allow_fp8) return fail(HYS_ERR_UNSUPPORTED, "%s: fp8 not accepted here", name);
  for (int i = 0; i < 4; ++i) {
    if (t.shape[i] < 0) return fail(HYS_ERR_INVALID_ARG, "%s: negative shape[%d]", name, i);
    if (t.stride[i] < 0) return fail(HYS_ERR_INVALID_ARG, "%s: negative stride[%d]", name, i);
  }
  if (t.shape[0] < 1 || t.shape[2] < 1) return fail(HYS_ERR_INVALID_ARG, "%s: batch and heads must be >= 1", name);
  if (t.shape[3] != 64 && t.shape[3] != 128)
    return fail(HYS_ERR_UNSUPPORTED, "%s: head dim %lld not in {64, 128}", name, (long long)t.shape[3]);
  if (t.stride[3] != 1) return fail(HYS_ERR_INVALID_ARG, "%s: head-dim stride must be 1", name);
  if (t.stride[1] >= (1ll << 24) || t.stride[2] >= (1ll << 24))
    return fail(HYS_ERR_UNSUPPORTED, "%s: token/head strides must be below 2^24 elements", name);
  if (t.shape[1] >= (1ll << 30)) return fail(HYS_ERR_UNSUPPORTED, "%s: more than 2^30 tokens", name);
  const size_t es = elem_size(t.dtype);
  if (!aligned16(t.ptr)) return fail(HYS_ERR_INVALID_ARG, "%s: pointer not 16-byte aligned", name);
  for (int i = 0; i < 3; ++i)
    if (((size_t)t.stride[i] * es) % 16 != 0 && t.shape[i] > 1)
      return fail(HYS_ERR_INVALID_ARG, "%s: stride[%d] not a multiple of 16 bytes", name, i);
  return HYS_OK;
}

hys::ElemType et(int32_t dt) {
  return dt == HYS_F32 ? hys::ET_F32 : (dt == HYS_BF16 ? hys::ET_BF16 : hys::ET_FP8);
}

// q [B,Lq,Hq,D], k/v [B,Lk,Hkv,D] consistency and type rule.  q_off >= 0: a
// prefill call whose query rows sit at positions q_off .. q_off + Lq - 1 of
// the keys (q_off + Lq <= Lk); q_off < 0: no length relation (decode).
hys_status check_qkv(const hys_tensor4& q, const hys_tensor4& k, const hys_tensor4& v, int64_t q_off) {
  hys_status s;
  if ((s = check_tensor(q, "q", false)) != HYS_OK) return s;
  if ((s = check_tensor(k, "k", true)) != HYS_OK) return s;
  if ((s = check_tensor(v, "v", true)) != HYS_OK) return s;
  if (k.dtype != v.dtype) return fail(HYS_ERR_INVALID_ARG, "k and v dtypes differ");
  if (q.dtype == HYS_F32 && k.dtype != HYS_F32) return fail(HYS_ERR_UNSUPPORTED, "fp32 q needs fp32 k/v");
  if (q.dtype == HYS_BF16 && k.dtype == HYS_F32) return fail(HYS_ERR_UNSUPPORTED, "bf16 q needs bf16 or fp8 k/v");
  if (k.shape[0] != q.shape[0] || v.shape[0] != q.shape[0]) return fail(HYS_ERR_INVALID_ARG, "batch sizes differ");
  if (k.shape[3] != q.shape[3] || v.shape[3] != q.shape[3]) return fail(HYS_ERR_INVALID_ARG, "head dims differ");
  if (k.shape[2] != v.shape[2]) return fail(HYS_ERR_INVALID_ARG, "k and v head counts differ");
  if (k.shape[1] != v.shape[1]) return fail(HYS_ERR_INVALID_ARG, "k and v lengths differ");
  if (q.shape[2] % k.shape[2] != 0)
    return fail(HYS_ERR_INVALID_ARG, "query heads (%lld) not a multiple of KV heads (%lld)", (long long)q.shape[2],
                (long long)k.shape[2]);
  if (q_off >= 0 && q_off + q.shape[1] > k.shape[1])
    return fail(HYS_ERR_INVALID_ARG, "q_offset (%lld) + query length (%lld) exceeds the key length (%lld)",
                (long long)q_off, (long long)q.shape[1], (long long)k.shape[1]);
  return HYS_OK;
}

hys_status check_out(const hys_tensor4& o, const hys_tensor4& q, const char* name) {
  hys_status s;
  if ((s = check_tensor(o, name, false)) != HYS_OK) return s;
  for (int i = 0; i < 4; ++i)
    if (o.shape[i] != q.shape[i]) return fail(HYS_ERR_INVALID_ARG, "%s: shape differs from q", name);
  return HYS_OK;
}

hys::AttnArgs base_args(const hys_attn_params* p, const hys_tensor4& q, const hys_tensor4& k, const hys_tensor4& v,
                        const hys_tensor4& o, float* lse) {
  hys::AttnArgs a{};
  a.q = q.ptr; a.q_sb = q.stride[0]; a.q_st = q.stride[1]; a.q_sh = q.stride[2];
  a.k = k.ptr; a.k_sb = k.stride[0]; a.k_st = k.stride[1]; a.k_sh = k.stride[2];
  a.v = v.ptr; a.v_sb = v.stride[0]; a.v_st = v.stride[1]; a.v_sh = v.stride[2];
  a.o = o.ptr; a.o_sb = o.stride[0]; a.o_st = o.stride[1]; a.o_sh = o.stride[2];
  a.o_f32 = o.dtype == HYS_F32 ? 1 : 0;
  a.lse = lse;
  a.B = (int)q.shape[0]; a.Lq = (int)q.shape[1]; a.Lk = (int)k.shape[1];
  a.q_off = (int)p->q_offset;
  a.Hq = (int)q.shape[2]; a.Hkv = (int)k.shape[2]; a.G = a.Hq / a.Hkv;
  a.logit_scale = p->softmax_scale * p->k_scale;
  a.scale_log2 = a.logit_scale * 1.4426950408889634f;
  a.v_scale = p->v_scale;
  return a;
}

hys_status check_params(const hys_attn_params* p) {
  if (!p) return fail(HYS_ERR_INVALID_ARG, "null params");
  if (p->causal != 1)
    return fail(HYS_ERR_UNSUPPORTED, "causal must be 1: every layer of the hybrid block attends causally");
  if (p->q_offset < 0 || p->q_offset >= (1ll << 30))
    return fail(HYS_ERR_INVALID_ARG, "q_offset must be in [0, 2^30)");
  if (!std::isfinite(p->softmax_scale) || !(p->softmax_scale > 0.f))
    return fail(HYS_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  if (!std::isfinite(p->k_scale) || !(p->k_scale > 0.f) || !std::isfinite(p->v_scale) || !(p->v_scale > 0.f))
    return fail(HYS_ERR_INVALID_ARG, "k_scale and v_scale must be finite and > 0");
  return HYS_OK;
}

// Launch the top-k kernels; arguments already validated, ws holds topk_workspace_bytes.
hys_status topk_launch(const float* scores, int64_t rows, int64_t cols, int64_t row_stride, int32_t k, int32_t* idx,
                       int32_t* count, void* ws, hipStream_t st, bool hist_zeroed = false) {
  if (rows == 0) return ok();
  if (k == 0 || cols == 0) {
    hipError_t e = hipSuccess;
    if (k > 0) e = hys::launch_fill_i32(idx, -1, rows * (int64_t)k, st);
    if (e == hipSuccess && count) e = hys::launch_fill_i32(count, 0, rows, st);
    return hip_status(e, "empty top-k fill");
  }
  hys::TopkArgs a{};
  a.scores = scores; a.rows = rows; a.cols = cols; a.row_stride = row_stride; a.k = k;
  a.idx = idx; a.count = count;
  if (cols > hys::topk_chunk_cols()) {
    a.ws = ws;
    a.hist_zeroed = hist_zeroed;
    HYS_DCHECK(ws != nullptr && ((uintptr_t)ws & 3) == 0 && hys::topk_workspace_bytes(rows, cols, k) > 0);
  }
  return hip_status(hys::launch_topk(a, st), "top-k launch");
}

// Largest top-k grid: 1024-thread workgroups, grid x threads below 2^32.
constexpr int64_t kMaxGrid = (int64_t)1 << 22;

// every prefill attention launch (engine modes and the sparse-layer kernel)
hys_status check_attn_launch(const hys::AttnArgs& a, int mode, int grid) {
  const bool tile_mode = mode == hys::M_FULL_TILE || mode == hys::M_SPARSE_TOKEN;
  const bool blocksel = mode == hys::M_SPARSE_BLOCK || mode == hys::M_SPARSE_SWA;
  (void)tile_mode; (void)blocksel; (void)a; (void)grid;
  HYS_DCHECK(grid >= 1 && grid == a.grid_used);
  HYS_DCHECK(a.B >= 1 && a.Lq >= 1 && a.q_off >= 0 && (int64_t)a.q_off + a.Lq <= a.Lk && a.Lk < (1 << 30));
  HYS_DCHECK(a.Hkv >= 1 && a.G >= 1 && a.Hq == a.G * a.Hkv);
  HYS_DCHECK(a.BQ >= 1 && a.ntq == (a.Lq + a.BQ - 1) / a.BQ);
  HYS_DCHECK(a.HC >= 1 && (int64_t)a.nhc * a.HC >= a.G && (int64_t)(a.nhc - 1) * a.HC < a.G);
  HYS_DCHECK(a.BQ * a.HC <= ((mode == hys::M_FULL || mode == hys::M_FULL_BLOCK) ? hys::kFullLayerRows : 128));
  if (tile_mode) {
    HYS_DCHECK(a.BQ == 64);
    HYS_DCHECK((int64_t)grid == ((int64_t)a.B * a.ntq + 7) / 8 * 8 * a.Hkv * a.nhc);
  } else {
    HYS_DCHECK(a.nhc == 1 && a.HC == a.G);
    HYS_DCHECK((int64_t)grid == (int64_t)a.B * a.ntq * a.Hkv);
  }
  // the kernels address 64 key rows of an operand with 32-bit offsets
  HYS_DCHECK(a.k_st >= 0 && a.v_st >= 0 && 64 * a.k_st < (1ll << 31) && 64 * a.v_st < (1ll << 31));
  if (mode == hys::M_FULL_BLOCK)
    HYS_DCHECK(a.scores && a.nblk == (a.Lk + 63) / 64 && a.sc_sr >= a.nblk && a.sc_sb >= (int64_t)a.Lq * a.sc_sr);
  if (mode == hys::M_FULL_TILE) HYS_DCHECK(a.scores && a.sc_sr == a.Lk && a.sc_sb == (int64_t)a.ntq * a.Lk);
  if (blocksel) {
    HYS_DCHECK(a.nblk == (a.Lk + 63) / 64 && a.nblk <= 16384);
    HYS_DCHECK(a.BQ <= 64 && a.topk >= 0 && a.topk <= 64 && a.BQ * a.topk <= 512 && a.idx_sr >= a.topk);
  }
  // token mode: the selected-token list and the window flags of one query tile fit their LDS arrays
  if (mode == hys::M_SPARSE_TOKEN) HYS_DCHECK(a.topk >= 0 && a.topk <= 2048 && a.window >= 0 && a.window + a.BQ - 1 <= 2048);
  if (mode == hys::M_SWA_GATE || mode == hys::M_SPARSE_SWA) HYS_DCHECK(a.window >= 1);
  if (mode == hys::M_SPARSE_SWA) HYS_DCHECK(a.kw && a.vw && a.gate_w);
  return HYS_OK;
}

// a workspace carved into consecutive parts: [p, p + bytes) inside [ws, ws + total)
bool inside(const void* p, size_t bytes, const void* ws, size_t total) {
  const char* c = (const char*)p;
  const char* w = (const char*)ws;
  return c >= w && (size_t)(c - w) <= total && bytes <= total - (size_t)(c - w);
}


}  // namespace

// Scratch of hys_decode_step_noalloc: a file-scope device array, one copy per
// GPU, alive until the process ends.  Host code never uses its name as an
// address (on the host the name is only a stand-in); the device address of
// each GPU's copy comes from hipGetSymbolAddress, taken once per device with
// that device current, and is the only pointer passed to kernels.
static __device__ __align__(256) unsigned char scratch[HYS_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of the current device's scratch array (set up on the first
// call on that device).
hys_status noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(HYS_ERR_UNSUPPORTED, "device ordinal %d above %d", dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!ptr) return fail(HYS_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return HYS_OK;
}

}  // namespace

extern "C" {

const char* hys_last_error(void) { return g_last_error.c_str(); }

const char* hys_status_string(hys_status s) {
  switch (s) {
    case HYS_OK: return "HYS_OK";
    case HYS_ERR_INVALID_ARG: return "HYS_ERR_INVALID_ARG";
    case HYS_ERR_UNSUPPORTED: return "HYS_ERR_UNSUPPORTED";
    case HYS_ERR_WORKSPACE: return "HYS_ERR_WORKSPACE";
    case HYS_ERR_HIP: return "HYS_ERR_HIP";
    case HYS_ERR_INTERNAL: return "HYS_ERR_INTERNAL";
  }
  return "HYS_ERR_UNKNOWN";
}

int hys_abi_version(void) { return HYS_ABI_VERSION; }

// ---------------------------------------------------------------------------
hys_status hys_full_attn_fwd(const hys_attn_params* p, hys_tensor4 q, hys_tensor4 k, hys_tensor4 v, hys_tensor4 o,
                             float* lse, const hys_score_params* sp, float* scores, void* ws, size_t* ws_bytes,
                             void* stream) {
  try {
    hys_status s;
    if ((s = check_params(p)) != HYS_OK) return s;
    if ((s = check_qkv(q, k, v, p->q_offset)) != HYS_OK) return s;
    if ((s = check_out(o, q, "o")) != HYS_OK) return s;
    if (!ws_bytes) return fail(HYS_ERR_INVALID_ARG, "ws_bytes must not be null");
    const int mode_in = sp ? sp->mode : HYS_SCORE_NONE;
    if (mode_in != HYS_SCORE_NONE && mode_in != HYS_SCORE_BLOCK && mode_in != HYS_SCORE_TILE_TOKEN &&
        mode_in != HYS_SCORE_BLOCK_GROUP)
      return fail(HYS_ERR_INVALID_ARG, "unknown score mode %d", mode_in);
    if (mode_in != HYS_SCORE_NONE) {
      if (sp->size != 64) return fail(HYS_ERR_UNSUPPORTED, "score size must be 64 (got %d)", sp->size);
      if (!scores) return fail(HYS_ERR_INVALID_ARG, "scores must not be null when a score mode is set");
    }
    const int64_t B = q.shape[0], L = q.shape[1], Lk = k.shape[1], Hq = q.shape[2], Hkv = k.shape[2], D = q.shape[3];
    const int64_t G = Hq / Hkv;
    if (G > 256 && mode_in != HYS_SCORE_TILE_TOKEN)
      return fail(HYS_ERR_UNSUPPORTED, "more than 256 query heads per KV head");
    const int64_t nblk = (Lk + 63) / 64;
    size_t need = 0;
    if (mode_in == HYS_SCORE_BLOCK && Hkv > 1) need = (size_t)(Hkv * B * L * nblk) * sizeof(float);
    if (!ws) { *ws_bytes = need; return ok(); }
    if (*ws_bytes < need) return fail(HYS_ERR_WORKSPACE, "workspace %zu < required %zu bytes", *ws_bytes, need);
    if (need > 0 && !aligned16(ws)) return fail(HYS_ERR_INVALID_ARG, "workspace not 16-byte aligned");
    if (L == 0) return ok();

    hys::AttnArgs a = base_args(p, q, k, v, o, lse);
    hipStream_t st = (hipStream_t)stream;
    int mode, grid;
    bool use_fl = false;
    a.nb = 1;
    const int rows = 128;                        // rows per workgroup
    if (mode_in == HYS_SCORE_TILE_TOKEN) {
      mode = hys::M_FULL_TILE;
      a.BQ = 64;
      a.HC = (int)(G < rows / 64 ? G : rows / 64);
      a.nhc = (int)((G + a.HC - 1) / a.HC);
      a.ntq = (int)((L + 63) / 64);
      a.scores = scores; a.sc_sb = (int64_t)a.ntq * Lk; a.sc_sr = Lk; a.sc_sg = 0;
      // one workgroup per (query tile, head chunk), tiles padded to the 8 XCDs
      const int64_t wgs = ((B * a.ntq + 7) / 8) * 8 * Hkv * a.nhc;
      if (wgs > 0x7fffffff) return fail(HYS_ERR_UNSUPPORTED, "too many query tiles x head chunks (%lld)", (long long)wgs);
      grid = (int)wgs;
    } else {
      mode = (mode_in == HYS_SCORE_BLOCK || mode_in == HYS_SCORE_BLOCK_GROUP) ? hys::M_FULL_BLOCK : hys::M_FULL;
      if (G > rows) return fail(HYS_ERR_UNSUPPORTED, "more than %d query heads per KV head", rows);
      a.HC = (int)G;
      a.nhc = 1;
      // the bf16 full-layer kernel takes 256 rows per workgroup, the engine 128
      a.BQ = (int)(hys::kFullLayerRows / G);
      a.ntq = (int)((L + a.BQ - 1) / a.BQ);
      use_fl = et(q.dtype) == hys::ET_BF16 && et(k.dtype) == hys::ET_BF16 &&
               hys::full_layer_supported((int)D, a, mode == hys::M_FULL_BLOCK);
      if (!use_fl) {
        a.BQ = (int)(rows / G);
        a.ntq = (int)((L + a.BQ - 1) / a.BQ);
      }
      if (mode == hys::M_FULL_BLOCK) {
        a.nblk = (int)nblk;
        a.sc_sb = L * nblk; a.sc_sr = nblk;
        if (mode_in == HYS_SCORE_BLOCK_GROUP) { a.scores = scores; a.sc_sg = B * L * nblk; }   // one matrix per group
        else if (Hkv > 1) { a.scores = (float*)ws; a.sc_sg = B * L * nblk; }
        else { a.scores = scores; a.sc_sg = 0; }
      }
      grid = (int)(B * a.ntq * Hkv);
    }
    a.grid_used = grid;
    if ((s = check_attn_launch(a, mode, grid)) != HYS_OK) return s;
    hipError_t e;
    if (mode == hys::M_FULL_TILE) {
      e = hys::launch_tile_scores(a.scores, (int)B, a.ntq, a.BQ, (int)L, (int)Lk, a.q_off, a.sc_sb, a.sc_sr, 0, st);
      if (e != hipSuccess) return hip_status(e, "score clear launch");
    }
    if (use_fl)
      e = hys::launch_full_layer((int)D, a, mode == hys::M_FULL_BLOCK, grid, st);
    else
      e = hys::launch_attn(mode, et(q.dtype), et(k.dtype), (int)D, a, grid, st);
    if (e != hipSuccess) return hip_status(e, "full attention launch");
    if (mode == hys::M_FULL_TILE) {
      e = hys::launch_tile_scores(a.scores, (int)B, a.ntq, a.BQ, (int)L, (int)Lk, a.q_off, a.sc_sb, a.sc_sr, 1, st);
      if (e != hipSuccess) return hip_status(e, "score decode launch");
    }
    if (mode == hys::M_FULL_BLOCK && mode_in == HYS_SCORE_BLOCK && Hkv > 1) {
      e = hys::launch_reduce_max((const float*)ws, (int)Hkv, B * L * nblk, scores, B * L * nblk, st);
      if (e != hipSuccess) return hip_status(e, "score reduction launch");
    }
    return ok();
  } catch (...) {
    return fail(HYS_ERR_INTERNAL, "internal error");
  }
}

// ---------------------------------------------------------------------------
hys_status hys_select_topk(const float* scores, int64_t rows, int64_t cols, int64_t row_stride, int32_t k,
                           int32_t* idx, int32_t* count, void* ws, size_t* ws_bytes, void* stream) {
  try {
    if (!ws_bytes) return fail(HYS_ERR_INVALID_ARG, "ws_bytes must not be null");
    if (rows < 0 || cols < 0) return fail(HYS_ERR_INVALID_ARG, "negative rows/cols");
    if (k < 0) return fail(HYS_ERR_INVALID_ARG, "k must be >= 0");
    if (k > 4096) return fail(HYS_ERR_UNSUPPORTED, "k > 4096");
    if (cols >= (1ll << 31)) return fail(HYS_ERR_UNSUPPORTED, "cols >= 2^31");
    if (rows > 0 && row_stride < cols) return fail(HYS_ERR_INVALID_ARG, "row_stride < cols");
    if (rows > (1ll << 31) - 1) return fail(HYS_ERR_UNSUPPORTED, "rows >= 2^31");
    if (hys::topk_max_workgroups(rows, cols, k) > kMaxGrid)
      return fail(HYS_ERR_UNSUPPORTED, "rows x column chunks of the top-k launch above %lld workgroups",
                  (long long)kMaxGrid);
    const size_t need = hys::topk_workspace_bytes(rows, cols, k);
    if (!ws) { *ws_bytes = need; return ok(); }
    if (*ws_bytes < need) return fail(HYS_ERR_WORKSPACE, "workspace %zu < required %zu bytes", *ws_bytes, need);
    if (rows > 0 && k > 0 && (!idx || (cols > 0 && !scores))) return fail(HYS_ERR_INVALID_ARG, "null scores or idx");
    if (rows > 0 && k == 0 && count == nullptr) return ok();
    return topk_launch(scores, rows, cols, row_stride, k, idx, count, ws, (hipStream_t)stream);
  } catch (...) {
    return fail(HYS_ERR_INTERNAL, "internal error");
  }
}

// Row sets of the block-selection modes (granularity 64, per-query selection):
// BQ queries x G heads per workgroup, BQ * k <= 4 * rows so the union of the
// row set's selected blocks fits the per-workgroup list.
hys_status setup_block_selection(hys::AttnArgs& a, const hys_sparse_params* sp, int64_t G, int64_t L, int64_t Lk,
                                 int64_t B, int64_t Hkv, int& grid) {
  if (sp->q_tile != 1) return fail(HYS_ERR_UNSUPPORTED, "granularity 64 needs q_tile 1");
  if (sp->forced_window != 0) return fail(HYS_ERR_UNSUPPORTED, "granularity 64 has no forced window");
  if (sp->k > 64) return fail(HYS_ERR_UNSUPPORTED, "granularity 64 needs k <= 64");
  if (G > 256) return fail(HYS_ERR_UNSUPPORTED, "more than 256 query heads per KV head");
  const int64_t nblk = (Lk + 63) / 64;
  if (nblk > 16384) return fail(HYS_ERR_UNSUPPORTED, "more than 16384 key blocks");
  a.nb = 1;
  const int rows = 128;
  if (G > rows) return fail(HYS_ERR_UNSUPPORTED, "more than %d query heads per KV head", rows);
  a.HC = (int)G;
  int bq = (int)(rows / G);
  if (bq > 64) bq = 64;
  if (sp->k > 0 && bq > 4 * rows / sp->k) bq = 4 * rows / sp->k;
  if (bq < 1) bq = 1;
  a.BQ = bq; a.nhc = 1; a.nblk = (int)nblk;
  a.ntq = (int)((L + a.BQ - 1) / a.BQ);
  grid = (int)(B * a.ntq * Hkv);
  return HYS_OK;
}

// ---------------------------------------------------------------------------
hys_status hys_select_topk_blocks(const float* scores, int64_t rows, int64_t cols, int64_t row_stride, int32_t block,
                                  int32_t k_blocks, int32_t* idx, void* ws, size_t* ws_bytes, void* stream) {
  try {
    if (!ws_bytes) return fail(HYS_ERR_INVALID_ARG, "ws_bytes must not be null");
    if (rows < 0 || cols < 1) return fail(HYS_ERR_INVALID_ARG, "rows must be >= 0 and cols >= 1");
    if (row_stride < cols) return fail(HYS_ERR_INVALID_ARG, "row_stride < cols");
    if (block != 64) return fail(HYS_ERR_UNSUPPORTED, "block must be 64");
    if (k_blocks < 1 || k_blocks > 32) return fail(HYS_ERR_UNSUPPORTED, "k_blocks must be in [1, 32]");
    if (cols >= (1ll << 31)) return fail(HYS_ERR_UNSUPPORTED, "cols must be below 2^31");
    const int64_t nblk = (cols + 63) / 64;
    if (hys::topk_max_workgroups(rows, nblk, k_blocks) > kMaxGrid)
      return fail(HYS_ERR_UNSUPPORTED, "too many rows x block chunks for the top-k launch");
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t mb = (size_t)(rows * nblk) * sizeof(float), ib = (size_t)(rows * k_blocks) * sizeof(int32_t);
    const size_t tk = hys::topk_workspace_bytes(rows, nblk, k_blocks);
    const size_t need = up(mb) + up(ib) + up(tk);
    if (!ws) { *ws_bytes = need; return ok(); }
    if (*ws_bytes < need) return fail(HYS_ERR_WORKSPACE, "workspace %zu < required %zu bytes", *ws_bytes, need);
    if (!aligned16(ws)) return fail(HYS_ERR_INVALID_ARG, "workspace not 16-byte aligned");
    if (rows == 0) return ok();
    if (!scores || !idx) return fail(HYS_ERR_INVALID_ARG, "null scores or idx");
    char* w = (char*)ws;
    float* M = (float*)w;
    int32_t* blk = (int32_t*)(w + up(mb));
    void* tkws = w + up(mb) + up(ib);
    hipStream_t st = (hipStream_t)stream;
    hipError_t e = hys::launch_block_max_rows(scores, rows, cols, row_stride, (int)nblk, M, st);
    if (e != hipSuccess) return hip_status(e, "block maxima launch");
    hys_status ts = topk_launch(M, rows, nblk, nblk, k_blocks, blk, nullptr, tkws, st);
    if (ts != HYS_OK) return ts;
    return hip_status(hys::launch_expand_blocks(blk, rows, k_blocks, cols, idx, st), "block expansion launch");
  } catch (...) {
    return fail(HYS_ERR_INTERNAL, "internal error");
  }
}

// ---------------------------------------------------------------------------
hys_status hys_sparse_attn_fwd(const hys_attn_params* p, hys_tensor4 q, hys_tensor4 k, hys_tensor4 v,
                               const hys_sparse_params* sp, const int32_t* idx, hys_tensor4 o, float* lse, void* ws,
                               size_t* ws_bytes, void* stream) {
  (void)ws;
  try {
    hys_status s;
    if ((s = check_params(p)) != HYS_OK) return s;
    if ((s = check_qkv(q, k, v, p->q_offset)) != HYS_OK) return s;
    if ((s = check_out(o, q, "o")) != HYS_OK) return s;
    if (!sp) return fail(HYS_ERR_INVALID_ARG, "null sparse params");
    if (ws_bytes && !ws) { *ws_bytes = 0; return ok(); }
    if (sp->k < 0) return fail(HYS_ERR_INVALID_ARG, "k must be >= 0");
    if (sp->k > 0 && !idx) return fail(HYS_ERR_INVALID_ARG, "null idx");
    if (sp->idx_row_stride < sp->k || sp->idx_batch_stride < 0 || sp->idx_group_stride < 0)
      return fail(HYS_ERR_INVALID_ARG, "idx strides too small");
    if (sp->idx_group_stride != 0 && sp->granularity != 64)
      return fail(HYS_ERR_UNSUPPORTED, "per-KV-group index sets need granularity 64");
    const int64_t B = q.shape[0], L = q.shape[1], Hq = q.shape[2], Hkv = k.shape[2], D = q.shape[3];
    const int64_t G = Hq / Hkv;
    hys::AttnArgs a = base_args(p, q, k, v, o, lse);
    a.idx = idx; a.idx_sb = sp->idx_batch_stride; a.idx_sr = sp->idx_row_stride; a.topk = sp->k;
    a.idx_sg = sp->idx_group_stride;
    int mode, grid;
    if (sp->granularity == 64) {
      hys_status bs = setup_block_selection(a, sp, G, L, k.shape[1], B, Hkv, grid);
      if (bs != HYS_OK) return bs;
      mode = hys::M_SPARSE_BLOCK;
    } else if (sp->granularity == 1) {
      if (sp->q_tile != 64) return fail(HYS_ERR_UNSUPPORTED, "granularity 1 needs q_tile 64");
      if (sp->k > 2048) return fail(HYS_ERR_UNSUPPORTED, "granularity 1 needs k <= 2048");
      if (sp->forced_window < 0 || sp->forced_window > 1984)
        return fail(HYS_ERR_UNSUPPORTED, "forced_window must be in [0, 1984]");
      mode = hys::M_SPARSE_TOKEN;
      a.nb = 1;
      const int hcmax = 2;                       // 64 queries x hcmax heads = the workgroup's rows
      a.BQ = 64;
      a.HC = (int)(G < hcmax ? G : hcmax);
      a.nhc = (int)((G + a.HC - 1) / a.HC);
      a.ntq = (int)((L + 63) / 64);
      a.window = sp->forced_window;
      const int64_t tiles = B * a.ntq;
      grid = (int)(((tiles + 7) / 8) * 8 * (Hkv * a.nhc));
    } else {
      return fail(HYS_ERR_UNSUPPORTED, "granularity must be 64 or 1");
    }
    if (L == 0) return ok();
    a.grid_used = grid;
    if ((s = check_attn_launch(a, mode, grid)) != HYS_OK) return s;
    return hip_status(hys::launch_attn(mode, et(q.dtype), et(k.dtype), (int)D, a, grid, (hipStream_t)stream),
                      "sparse attention launch");
  } catch (...) {
    return fail(HYS_ERR_INTERNAL, "internal error");
  }
}

// ---------------------------------------------------------------------------
hys_status hys_swa_gate_fwd(const hys_attn_params* p, hys_tensor4 q, hys_tensor4 k_win, hys_tensor4 v_win,
                            int32_t window, hys_tensor4 o_sparse, const float* lse_sparse, const float* gate_w,
                            const float* gate_b, hys_tensor4 o, void* stream) {
  try {
    hys_status s;
    if ((s = check_params(p)) != HYS_OK) return s;
    if ((s = check_qkv(q, k_win, v_win, p->q_offset)) != HYS_OK) return s;
    if (k_win.dtype != q.dtype && !(q.dtype == HYS_BF16 && k_win.dtype == HYS_FP8_E4M3))
      return fail(HYS_ERR_UNSUPPORTED, "window K/V must have q's dtype or be fp8 with bf16 q");
    if ((s = check_out(o, q, "o")) != HYS_OK) return s;
    if ((s = check_out(o_sparse, q, "o_sparse")) != HYS_OK) return s;
    if (o_sparse.dtype != HYS_F32) return fail(HYS_ERR_UNSUPPORTED, "o_sparse must be fp32");
    if (!lse_sparse || !gate_w) return fail(HYS_ERR_INVALID_ARG, "null lse_sparse or gate_w");
    if (window < 1) return fail(HYS_ERR_INVALID_ARG, "window must be >= 1");
    const int64_t B = q.shape[0], L = q.shape[1], Hq = q.shape[2], Hkv = k_win.shape[2], D = q.shape[3];
    const int64_t G = Hq / Hkv;
    if (L == 0) return ok();
    hys::AttnArgs a = base_args(p, q, k_win, v_win, o, nullptr);
    a.window = window;
    a.nb = 1;
    if (G > 128) return fail(HYS_ERR_UNSUPPORTED, "more than 128 query heads per KV head");
    a.HC = (int)G; a.BQ = (int)(128 / G); a.nhc = 1;
    a.ntq = (int)((L + a.BQ - 1) / a.BQ);
    a.o_sp = (const float*)o_sparse.ptr;
    a.osp_sb = o_sparse.stride[0]; a.osp_st = o_sparse.stride[1]; a.osp_sh = o_sparse.stride[2];
    a.lse_sp = lse_sparse; a.gate_w = gate_w; a.gate_b = gate_b;
    const int grid = (int)(B * a.ntq * Hkv);
    a.grid_used = grid;
    if ((s = check_attn_launch(a, hys::M_SWA_GATE, grid)) != HYS_OK) return s;
    return hip_status(hys::launch_attn(hys::M_SWA_GATE, et(q.dtype), et(k_win.dtype), (int)D, a, grid,
                                       (hipStream_t)stream),
                      "window+gate launch");
  } catch (...) {
    return fail(HYS_ERR_INTERNAL, "internal error");
  }
}

// ---------------------------------------------------------------------------
hys_status hys_sparse_layer_fwd(const hys_attn_params* p, hys_tensor4 q, hys_tensor4 k, hys_tensor4 v,
                                const hys_sparse_params* sp, const int32_t* idx, hys_tensor4 k_win,
                                hys_tensor4 v_win, int32_t window, const float* gate_w, const float* gate_b,
                                hys_tensor4 o, void* stream) {
  try {
    hys_status s;
    if ((s = check_params(p)) != HYS_OK) return s;
    if (p->k_scale != 1.f || p->v_scale != 1.f)
      return fail(HYS_ERR_UNSUPPORTED, "k_scale and v_scale must be 1 (K/V of q's type)");
    if ((s = check_qkv(q, k, v, p->q_offset)) != HYS_OK) return s;
    if (k.dtype != q.dtype) return fail(HYS_ERR_UNSUPPORTED, "k/v must have q's dtype");
    if ((s = check_qkv(q, k_win, v_win, p->q_offset)) != HYS_OK) return s;
    if (k_win.dtype != q.dtype) return fail(HYS_ERR_UNSUPPORTED, "window K/V must have q's dtype");
    for (int i = 0; i < 4; ++i) {
      if (k_win.shape[i] != k.shape[i] || v_win.shape[i] != v.shape[i])
        return fail(HYS_ERR_INVALID_ARG, "window K/V shapes differ from k/v");
      if (k_win.stride[i] != k.stride[i] || v_win.stride[i] != v.stride[i])
        return fail(HYS_ERR_UNSUPPORTED, "window K/V strides must equal those of k/v");
    }
    if ((s = check_out(o, q, "o")) != HYS_OK) return s;
    if (!sp) return fail(HYS_ERR_INVALID_ARG, "null sparse params");
    if (sp->granularity != 64) return fail(HYS_ERR_UNSUPPORTED, "granularity must be 64");
    if (sp->k < 0) return fail(HYS_ERR_INVALID_ARG, "k must be >= 0");
    if (sp->k > 0 && !idx) return fail(HYS_ERR_INVALID_ARG, "null idx");
    if (sp->idx_row_stride < sp->k || sp->idx_batch_stride < 0 || sp->idx_group_stride < 0)
      return fail(HYS_ERR_INVALID_ARG, "idx strides too small");
    if (!gate_w) return fail(HYS_ERR_INVALID_ARG, "null gate_w");
    if (window < 1) return fail(HYS_ERR_INVALID_ARG, "window must be >= 1");
    const int64_t B = q.shape[0], L = q.shape[1], Hq = q.shape[2], Hkv = k.shape[2], D = q.shape[3];
    const int64_t G = Hq / Hkv;
    hys::AttnArgs a = base_args(p, q, k, v, o, nullptr);
    a.idx = idx; a.idx_sb = sp->idx_batch_stride; a.idx_sr = sp->idx_row_stride; a.topk = sp->k;
    a.idx_sg = sp->idx_group_stride;
    a.kw = k_win.ptr; a.vw = v_win.ptr; a.window = window;
    a.gate_w = gate_w; a.gate_b = gate_b;
    int grid = 0;
    if ((s = setup_block_selection(a, sp, G, L, k.shape[1], B, Hkv, grid)) != HYS_OK) return s;
    if (L == 0) return ok();
    a.grid_used = grid;
    if ((s = check_attn_launch(a, hys::M_SPARSE_SWA, grid)) != HYS_OK) return s;
    // bf16 inputs: the dedicated kernel (LDS-direct tile loads); fp32 and fp8: the engine
    if (q.dtype == HYS_BF16 && k.dtype == HYS_BF16)
      return hip_status(hys::launch_sparse_layer((int)D, a, grid, (hipStream_t)stream), "sparse layer launch");
    return hip_status(hys::launch_attn(hys::M_SPARSE_SWA, et(q.dtype), et(k.dtype), (int)D, a, grid,
                                       (hipStream_t)stream),
                      "sparse layer launch");
  } catch (...) {
    return fail(HYS_ERR_INTERNAL, "internal error");
  }
}

// ---------------------------------------------------------------------------
// The HySparse2 decode step; hys_decode_step passes the caller's workspace,
// hys_decode_step_noalloc the library's fixed scratch array.  With ws == NULL
// it validates and returns the workspace size without any HIP call.
static hys_status decode_step_impl(const hys_decode_params* p, hys_tensor4 q_full, hys_tensor4 k_cache,
                                   hys_tensor4 v_cache, const int64_t* cache_len, hys_tensor4 o_full,
                                   float* token_scores, int32_t* idx, int32_t n_sparse, const hys_tensor4* q_sparse,
                                   const hys_tensor4* o_sparse, void* ws, size_t* ws_bytes, void* stream) {
  try {
    if (!p) return fail(HYS_ERR_INVALID_ARG, "null params");
    if (!ws_bytes) return fail(HYS_ERR_INVALID_ARG, "ws_bytes must not be null");
    hys_attn_params ap{p->softmax_scale, p->k_scale, p->v_scale, 1, 0};
    hys_status s;
    if ((s = check_params(&ap)) != HYS_OK) return s;
    if ((s = check_qkv(q_full, k_cache, v_cache, -1)) != HYS_OK) return s;
    if (q_full.dtype != HYS_BF16) return fail(HYS_ERR_UNSUPPORTED, "decode queries must be bf16");
    const int64_t B = q_full.shape[0], Hq = q_full.shape[2], D = q_full.shape[3], Nmax = k_cache.shape[1];
    if (q_full.shape[1] != 1) return fail(HYS_ERR_INVALID_ARG, "decode takes one query token per sequence");
    if (k_cache.shape[2] != 1) return fail(HYS_ERR_UNSUPPORTED, "decode needs an MQA cache (one KV head)");
    if (Hq > 64) return fail(HYS_ERR_UNSUPPORTED, "decode supports at most 64 query heads");
    if (B > hys::kMaxDecodeBatch) return fail(HYS_ERR_UNSUPPORTED, "decode batch > %d", hys::kMaxDecodeBatch);
    if (n_sparse < 0 || n_sparse > hys::kMaxDecodeLayers)
      return fail(HYS_ERR_UNSUPPORTED, "n_sparse must be in [0, %d]", hys::kMaxDecodeLayers);
    if (p->topk < 1 || p->topk > 2048) return fail(HYS_ERR_UNSUPPORTED, "topk must be in [1, 2048]");
    if (p->window < 0) return fail(HYS_ERR_INVALID_ARG, "window must be >= 0");
    if (Nmax < 1) return fail(HYS_ERR_INVALID_ARG, "empty cache");
    if (hys::topk_max_workgroups(B, Nmax, p->topk) > kMaxGrid)
      return fail(HYS_ERR_UNSUPPORTED, "cache too long for the top-k launch");
    if ((s = check_out(o_full, q_full, "o_full")) != HYS_OK) return s;
    if (!cache_len || !token_scores || !idx) return fail(HYS_ERR_INVALID_ARG, "null cache_len, token_scores or idx");
    if (n_sparse > 0 && (!q_sparse || !o_sparse)) return fail(HYS_ERR_INVALID_ARG, "null q_sparse or o_sparse");
    for (int64_t b = 0; b < B; ++b)
      if (cache_len[b] < 1 || cache_len[b] > Nmax)
        return fail(HYS_ERR_INVALID_ARG, "cache_len[%lld] = %lld outside [1, %lld]", (long long)b,
                    (long long)cache_len[b], (long long)Nmax);
    for (int l = 0; l < n_sparse; ++l) {
      if ((s = check_out(q_sparse[l], q_full, "q_sparse")) != HYS_OK) return s;
      if (q_sparse[l].dtype != HYS_BF16) return fail(HYS_ERR_UNSUPPORTED, "q_sparse must be bf16");
      if (q_sparse[l].stride[0] != q_sparse[0].stride[0] || q_sparse[l].stride[2] != q_sparse[0].stride[2])
        return fail(HYS_ERR_UNSUPPORTED, "all q_sparse must share strides");
      if ((s = check_out(o_sparse[l], q_full, "o_sparse")) != HYS_OK) return s;
      if (o_sparse[l].dtype != o_sparse[0].dtype || o_sparse[l].stride[0] != o_sparse[0].stride[0] ||
          o_sparse[l].stride[2] != o_sparse[0].stride[2])
        return fail(HYS_ERR_UNSUPPORTED, "all o_sparse must share dtype and strides");
    }
    // split-K: two workgroups (two compute waves and one staging wave each)
    // per CU, at least 8 key tiles each
    const int64_t ntiles = (Nmax + 63) / 64;
    int nsplit = (int)(512 / B);
    if (nsplit < 1) nsplit = 1;
    if ((int64_t)nsplit * 8 > ntiles) nsplit = (int)((ntiles + 7) / 8);
    const int nsplit_sp = 8;
    const size_t part_full = (size_t)(B * nsplit * Hq) * (size_t)(D + 2) * sizeof(float);
    const size_t part_sp = (size_t)((int64_t)n_sparse * B * nsplit_sp * Hq) * (size_t)(D + 2) * sizeof(float);
    const size_t tk = hys::topk_workspace_bytes(B, Nmax, p->topk);
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t need = up(part_full) + up(part_sp) + up(tk);
    if (!ws) { *ws_bytes = need; return ok(); }
    if (*ws_bytes < need) return fail(HYS_ERR_WORKSPACE, "workspace %zu < required %zu bytes", *ws_bytes, need);
    if (!aligned16(ws)) return fail(HYS_ERR_INVALID_ARG, "workspace not 16-byte aligned");
    char* w = (char*)ws;
    float* pf_o = (float*)w;
    float* pf_ml = pf_o + (size_t)(B * nsplit * Hq) * D;
    w += up(part_full);
    float* ps_o = (float*)w;
    float* ps_ml = ps_o + (size_t)((int64_t)n_sparse * B * nsplit_sp * Hq) * D;
    w += up(part_sp);
    void* tkws = w;
    HYS_DCHECK(nsplit >= 1 && nsplit <= ntiles && (int64_t)nsplit * B <= 512 + B);
    HYS_DCHECK(inside(pf_ml, (size_t)(B * nsplit * Hq) * 2 * sizeof(float), ws, up(part_full)));
    HYS_DCHECK(inside(ps_ml, (size_t)((int64_t)n_sparse * B * nsplit_sp * Hq) * 2 * sizeof(float), ws,
                      up(part_full) + up(part_sp)));
    HYS_DCHECK(inside(tkws, tk, ws, need));

    hipStream_t st = (hipStream_t)stream;
    const float logit_scale = p->softmax_scale * p->k_scale;
    hys::DecArgs d{};
    d.k = k_cache.ptr; d.k_sb = k_cache.stride[0]; d.k_st = k_cache.stride[1];
    d.v = v_cache.ptr; d.v_sb = v_cache.stride[0]; d.v_st = v_cache.stride[1];
    for (int64_t b = 0; b < B; ++b) d.lens[b] = (int)cache_len[b];
    d.B = (int)B; d.Hq = (int)Hq; d.Nmax = (int)Nmax;
    {
      int dev = 0, ncu = 0;
      if (hipGetDevice(&dev) != hipSuccess ||
          hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu < 1)
        return fail(HYS_ERR_HIP, "device query failed");
      d.ncu = ncu;
    }
    d.scale_log2 = logit_scale * 1.4426950408889634f; d.logit_scale = logit_scale;
    // the split launch also clears the top-k's row histograms (one launch fewer)
    const int64_t tk_zero = hys::topk_zero_ints(B, Nmax);
    HYS_DCHECK(tk_zero * (int64_t)sizeof(int32_t) <= (int64_t)tk);
    d.zero = tk_zero > 0 ? (int32_t*)tkws : nullptr;
    d.zero_n = tk_zero;
    // 1. full layer, split over the cache
    d.q[0] = q_full.ptr; d.q_sb = q_full.stride[0]; d.q_sh = q_full.stride[2];
    d.nsplit = nsplit; d.nlayer = 1;
    d.scores = token_scores; d.sc_sb = Nmax;
    d.part_o = pf_o; d.part_ml = pf_ml;
    hipError_t e = hys::launch_decode(0, et(k_cache.dtype), (int)D, d, st);
    if (e != hipSuccess) return hip_status(e, "decode split launch");
    hys::MergeArgs m{};
    m.B = (int)B; m.Hq = (int)Hq; m.logit_scale = logit_scale; m.v_scale = p->v_scale;
    m.scale_log2 = d.scale_log2;
    m.part_o = pf_o; m.part_ml = pf_ml; m.nsplit = nsplit; m.nlayer = 1;
    m.o[0] = o_full.ptr; m.o_sb = o_full.stride[0]; m.o_sh = o_full.stride[2]; m.o_f32 = o_full.dtype == HYS_F32;
    // 2. selection over the token scores (the full layer's merge waits for the
    // sparse layers' and runs in the same launch)
    hys_status ts = topk_launch(token_scores, B, Nmax, Nmax, p->topk, idx, nullptr, tkws, st, d.zero != nullptr);
    if (ts != HYS_OK) return ts;
    if (n_sparse == 0) return hip_status(hys::launch_decode_merge((int)D, m, st), "decode merge launch");
    // 3. all sparse layers in one launch
    if (n_sparse > 0) {
      for (int l = 0; l < n_sparse; ++l) d.q[l] = q_sparse[l].ptr;
      d.q_sb = q_sparse[0].stride[0]; d.q_sh = q_sparse[0].stride[2];
      d.nsplit = nsplit_sp; d.nlayer = n_sparse;
      d.scores = nullptr; d.zero = nullptr; d.zero_n = 0;
      d.idx = idx; d.idx_sb = p->topk; d.topk = p->topk; d.window = p->window;
      d.part_o = ps_o; d.part_ml = ps_ml;
      e = hys::launch_decode(1, et(k_cache.dtype), (int)D, d, st);
      if (e != hipSuccess) return hip_status(e, "decode sparse launch");
      hys::MergeArgs ms = m;
      ms.part_o = ps_o; ms.part_ml = ps_ml; ms.nsplit = nsplit_sp; ms.nlayer = n_sparse;
      for (int l = 0; l < n_sparse; ++l) { ms.o[l] = o_sparse[l].ptr; ms.lse[l] = nullptr; }
      ms.o_sb = o_sparse[0].stride[0]; ms.o_sh = o_sparse[0].stride[2]; ms.o_f32 = o_sparse[0].dtype == HYS_F32;
      e = hys::launch_decode_merge2((int)D, m, ms, st);
      if (e != hipSuccess) return hip_status(e, "decode merge launch");
    }
    return ok();
  } catch (...) {
    return fail(HYS_ERR_INTERNAL, "internal error");
  }
}

hys_status hys_decode_step(const hys_decode_params* p, hys_tensor4 q_full, hys_tensor4 k_cache, hys_tensor4 v_cache,
                           const int64_t* cache_len, hys_tensor4 o_full, float* token_scores, int32_t* idx,
                           int32_t n_sparse, const hys_tensor4* q_sparse, const hys_tensor4* o_sparse, void* ws,
                           size_t* ws_bytes, void* stream) {
  return decode_step_impl(p, q_full, k_cache, v_cache, cache_len, o_full, token_scores, idx, n_sparse, q_sparse,
                          o_sparse, ws, ws_bytes, stream);
}

hys_status hys_decode_step_noalloc(const hys_decode_params* p, hys_tensor4 q_full, hys_tensor4 k_cache,
                                   hys_tensor4 v_cache, const int64_t* cache_len, hys_tensor4 o_full,
                                   float* token_scores, int32_t* idx, int32_t n_sparse, const hys_tensor4* q_sparse,
                                   const hys_tensor4* o_sparse, void* stream) {
  try {
    // validation and the workspace size first: no HIP call yet
    size_t need = 0;
    hys_status s = decode_step_impl(p, q_full, k_cache, v_cache, cache_len, o_full, token_scores, idx, n_sparse,
                                    q_sparse, o_sparse, nullptr, &need, nullptr);
    if (s != HYS_OK) return s;
    if (need > HYS_NOALLOC_SCRATCH_BYTES)
      return fail(HYS_ERR_WORKSPACE, "this decode step needs %zu bytes of scratch; the fixed scratch holds %zu",
                  need, (size_t)HYS_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    if ((s = noalloc_scratch(&ws)) != HYS_OK) return s;
    size_t have = HYS_NOALLOC_SCRATCH_BYTES;
    return decode_step_impl(p, q_full, k_cache, v_cache, cache_len, o_full, token_scores, idx, n_sparse, q_sparse,
                            o_sparse, ws, &have, stream);
  } catch (...) {
    return fail(HYS_ERR_INTERNAL, "internal error");
  }
}

// ---------------------------------------------------------------------------
hys_status hys_kv_bridge_fwd(const hys_bridge_params* p, hys_tensor4 h, const void* w_k, const void* w_v,
                             hys_tensor4 k_cache, hys_tensor4 v_cache, float* amax, void* stream) {
  try {
    if (!p) return fail(HYS_ERR_INVALID_ARG, "null params");
    if (!std::isfinite(p->k_scale) || !(p->k_scale > 0.f) || !std::isfinite(p->v_scale) || !(p->v_scale > 0.f))
      return fail(HYS_ERR_INVALID_ARG, "k_scale and v_scale must be finite and > 0");
    const float inv_k = 1.0f / p->k_scale, inv_v = 1.0f / p->v_scale;
    if (!std::isfinite(inv_k) || !std::isfinite(inv_v))
      return fail(HYS_ERR_INVALID_ARG, "k_scale and v_scale must have finite reciprocals");
    // with no tokens nothing is read or written: null tensor pointers are
    // accepted (an empty torch tensor has none) and stand in as an aligned
    // placeholder for the checks below
    if (h.shape[1] == 0) {
      void* const placeholder = (void*)(uintptr_t)256;
      if (!h.ptr) h.ptr = placeholder;
      if (!k_cache.ptr) k_cache.ptr = placeholder;
      if (!v_cache.ptr) v_cache.ptr = placeholder;
    }
    // h [B, L, 1, d_model] bf16
    if (!h.ptr) return fail(HYS_ERR_INVALID_ARG, "h: null pointer");
    if (h.dtype != HYS_BF16) return fail(HYS_ERR_UNSUPPORTED, "h must be bf16");
    for (int i = 0; i < 4; ++i)
      if (h.shape[i] < 0 || h.stride[i] < 0) return fail(HYS_ERR_INVALID_ARG, "h: negative shape or stride");
    if (h.shape[0] < 1 || h.shape[2] != 1) return fail(HYS_ERR_INVALID_ARG, "h must be [B >= 1, L, 1, d_model]");
    const int64_t B = h.shape[0], L = h.shape[1], dm = h.shape[3];
    if (dm < 64 || dm > 32768 || dm % 64 != 0)
      return fail(HYS_ERR_UNSUPPORTED, "d_model %lld not a multiple of 64 in [64, 32768]", (long long)dm);
    if (h.stride[3] != 1) return fail(HYS_ERR_INVALID_ARG, "h: d_model stride must be 1");
    if (!aligned16(h.ptr)) return fail(HYS_ERR_INVALID_ARG, "h: pointer not 16-byte aligned");
    if ((h.stride[0] % 8 != 0 && B > 1) || (h.stride[1] % 8 != 0 && L > 1))
      return fail(HYS_ERR_INVALID_ARG, "h: token and batch strides must be multiples of 8 elements");
    if (L >= (1ll << 30)) return fail(HYS_ERR_UNSUPPORTED, "more than 2^30 tokens");
    if (B * L >= (1ll << 31) - 256) return fail(HYS_ERR_UNSUPPORTED, "B*L too large");
    // caches [B, L, Hkv, D] fp8, one shape and one set of strides
    hys_status s;
    if ((s = check_tensor(k_cache, "k_cache", true)) != HYS_OK) return s;
    if ((s = check_tensor(v_cache, "v_cache", true)) != HYS_OK) return s;
    if (k_cache.dtype != HYS_FP8_E4M3 || v_cache.dtype != HYS_FP8_E4M3)
      return fail(HYS_ERR_UNSUPPORTED, "k_cache and v_cache must be fp8 e4m3");
    for (int i = 0; i < 4; ++i)
      if (k_cache.shape[i] != v_cache.shape[i]) return fail(HYS_ERR_INVALID_ARG, "k_cache and v_cache shapes differ");
    for (int i = 0; i < 4; ++i)
      if (k_cache.stride[i] != v_cache.stride[i])
        return fail(HYS_ERR_UNSUPPORTED, "k_cache and v_cache strides must be equal");
    if (k_cache.shape[0] != B || k_cache.shape[1] != L)
      return fail(HYS_ERR_INVALID_ARG, "cache [B, L] differs from h");
    const int64_t Hkv = k_cache.shape[2], D = k_cache.shape[3];
    if ((Hkv * D) % 128 != 0) return fail(HYS_ERR_UNSUPPORTED, "Hkv*D must be a multiple of 128");
    if (Hkv * D > 65536) return fail(HYS_ERR_UNSUPPORTED, "Hkv*D above 65536");
    if (!w_k || !w_v) return fail(HYS_ERR_INVALID_ARG, "null w_k or w_v");
    if (!aligned16(w_k) || !aligned16(w_v)) return fail(HYS_ERR_INVALID_ARG, "w_k, w_v not 16-byte aligned");
    if (amax && ((uintptr_t)amax & 3u)) return fail(HYS_ERR_INVALID_ARG, "amax not 4-byte aligned");

    hipStream_t st = (hipStream_t)stream;
    if (amax) {
      hipError_t e = hys::launch_fill_i32((int32_t*)amax, 0, 2, st);
      if (e != hipSuccess) return hip_status(e, "amax clear");
    }
    hys::BridgeArgs a{};
    a.h = h.ptr; a.h_sb = h.stride[0]; a.h_st = h.stride[1];
    a.w_k = w_k; a.w_v = w_v;
    a.k_out = k_cache.ptr; a.v_out = v_cache.ptr;
    a.o_sb = k_cache.stride[0]; a.o_st = k_cache.stride[1]; a.o_sh = k_cache.stride[2];
    a.amax = amax; a.inv_k = inv_k; a.inv_v = inv_v;
    a.B = (int)B; a.L = (int)L; a.d_model = (int)dm; a.Hkv = (int)Hkv; a.D = (int)D;
    return hip_status(hys::launch_kv_bridge(a, st), "kv bridge launch");
  } catch (...) {
    return fail(HYS_ERR_INTERNAL, "internal error");
  }
}

// ---------------------------------------------------------------------------
hys_status hys_hysparse_decode_step(const hys_hs_decode_params* p, hys_tensor4 q_full, hys_tensor4 k_cache,
                                    hys_tensor4 v_cache, const int64_t* cache_len, hys_tensor4 o_full,
                                    float* block_scores, int32_t* idx, int32_t n_sparse, const hys_tensor4* q_sparse,
                                    const hys_tensor4* k_win_new, const hys_tensor4* v_win_new,
                                    const hys_tensor4* k_ring, const hys_tensor4* v_ring, const float* const* gate_w,
                                    const hys_tensor4* o_sparse, void* ws, size_t* ws_bytes, void* stream) {
  try {
    if (!p) return fail(HYS_ERR_INVALID_ARG, "null params");
    if (!ws_bytes) return fail(HYS_ERR_INVALID_ARG, "ws_bytes must not be null");
    hys_attn_params ap{p->softmax_scale, 1.f, 1.f, 1, 0};
    hys_status s;
    if ((s = check_params(&ap)) != HYS_OK) return s;
    if ((s = check_qkv(q_full, k_cache, v_cache, -1)) != HYS_OK) return s;
    if (q_full.dtype != HYS_BF16 || k_cache.dtype != HYS_BF16)
      return fail(HYS_ERR_UNSUPPORTED, "HySparse decode takes bf16 queries and a bf16 cache");
    const int64_t B = q_full.shape[0], Hq = q_full.shape[2], D = q_full.shape[3], Nmax = k_cache.shape[1];
    const int64_t Hkv = k_cache.shape[2], G = Hq / Hkv;
    if (q_full.shape[1] != 1) return fail(HYS_ERR_INVALID_ARG, "decode takes one query token per sequence");
    if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16)
      return fail(HYS_ERR_UNSUPPORTED, "query heads per KV head must be 1, 2, 4, 8 or 16");
    if (B > hys::kMaxDecodeBatch) return fail(HYS_ERR_UNSUPPORTED, "decode batch > %d", hys::kMaxDecodeBatch);
    if (n_sparse < 0 || n_sparse > hys::kMaxDecodeLayers)
      return fail(HYS_ERR_UNSUPPORTED, "n_sparse must be in [0, %d]", hys::kMaxDecodeLayers);
    if (p->block != 64) return fail(HYS_ERR_UNSUPPORTED, "block must be 64");
    if (p->topk < 1 || p->topk > 64) return fail(HYS_ERR_UNSUPPORTED, "topk must be in [1, 64]");
    if (Nmax < 1) return fail(HYS_ERR_INVALID_ARG, "empty cache");
    const int64_t nblk = (Nmax + 63) / 64;
    if (hys::topk_max_workgroups(B, nblk, p->topk) > kMaxGrid)
      return fail(HYS_ERR_UNSUPPORTED, "cache too long for the top-k launch");
    if ((s = check_out(o_full, q_full, "o_full")) != HYS_OK) return s;
    if (!cache_len || !block_scores || !idx) return fail(HYS_ERR_INVALID_ARG, "null cache_len, block_scores or idx");
    for (int64_t b = 0; b < B; ++b)
      if (cache_len[b] < 1 || cache_len[b] > Nmax)
        return fail(HYS_ERR_INVALID_ARG, "cache_len[%lld] = %lld outside [1, %lld]", (long long)b,
                    (long long)cache_len[b], (long long)Nmax);
    int64_t W = 0;
    if (n_sparse > 0) {
      if (!q_sparse || !o_sparse || !k_win_new || !v_win_new || !k_ring || !v_ring || !gate_w)
        return fail(HYS_ERR_INVALID_ARG, "null per-layer array");
      W = k_ring[0].shape[1];
      if (W < 1) return fail(HYS_ERR_INVALID_ARG, "ring window must have at least one slot");
      for (int l = 0; l < n_sparse; ++l) {
        if ((s = check_out(q_sparse[l], q_full, "q_sparse")) != HYS_OK) return s;
        if (q_sparse[l].dtype != HYS_BF16) return fail(HYS_ERR_UNSUPPORTED, "q_sparse must be bf16");
        if (q_sparse[l].stride[0] != q_sparse[0].stride[0] || q_sparse[l].stride[2] != q_sparse[0].stride[2])
          return fail(HYS_ERR_UNSUPPORTED, "all q_sparse must share strides");
        if ((s = check_out(o_sparse[l], q_full, "o_sparse")) != HYS_OK) return s;
        if (o_sparse[l].dtype != o_sparse[0].dtype || o_sparse[l].stride[0] != o_sparse[0].stride[0] ||
            o_sparse[l].stride[2] != o_sparse[0].stride[2])
          return fail(HYS_ERR_UNSUPPORTED, "all o_sparse must share dtype and strides");
        const hys_tensor4* nw[4] = {&k_win_new[l], &v_win_new[l], &k_ring[l], &v_ring[l]};
        const char* nm[4] = {"k_win_new", "v_win_new", "k_ring", "v_ring"};
        for (int i = 0; i < 4; ++i) {
          if ((s = check_tensor(*nw[i], nm[i], false)) != HYS_OK) return s;
          if (nw[i]->dtype != HYS_BF16) return fail(HYS_ERR_UNSUPPORTED, "%s must be bf16", nm[i]);
          const int64_t want[4] = {B, i < 2 ? 1 : W, Hkv, D};
          for (int d = 0; d < 4; ++d)
            if (nw[i]->shape[d] != want[d]) return fail(HYS_ERR_INVALID_ARG, "%s: shape mismatch", nm[i]);
        }
        for (int d = 0; d < 3; ++d) {
          if (v_win_new[l].stride[d] != k_win_new[0].stride[d] || k_win_new[l].stride[d] != k_win_new[0].stride[d])
            return fail(HYS_ERR_UNSUPPORTED, "all new-token window tensors must share strides");
          if (v_ring[l].stride[d] != k_ring[0].stride[d] || k_ring[l].stride[d] != k_ring[0].stride[d])
            return fail(HYS_ERR_UNSUPPORTED, "all ring tensors must share strides");
        }
        if (!gate_w[l]) return fail(HYS_ERR_INVALID_ARG, "null gate_w");
      }
    }
    // the full layer runs once per KV head on the split-K kernel (G heads each)
    const int64_t ntiles = (Nmax + 63) / 64;
    int nsplit = (int)(512 / B);
    if (nsplit < 1) nsplit = 1;
    if ((int64_t)nsplit * 8 > ntiles) nsplit = (int)((ntiles + 7) / 8);
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t ts_bytes = (size_t)(Hkv * B * Nmax) * sizeof(float);
    const size_t tk = hys::topk_workspace_bytes(B, nblk, p->topk);
    const int hs_split = hys::hs_decode_splits(p->topk);
    const size_t sp_bytes = (size_t)n_sparse * B * Hq * hs_split * (size_t)(D + 2) * sizeof(float);
    // every KV head's split partials in one layout, [(g*B + b)*nsplit + s][G][D] then
    // [..][G][2], so one merge launch serves up to kMaxDecodeLayers heads
    const size_t po_floats = (size_t)(Hkv * B * nsplit * G) * D, pml_floats = (size_t)(Hkv * B * nsplit * G) * 2;
    const size_t need = up(ts_bytes) + up((po_floats + pml_floats) * sizeof(float)) + up(tk) + up(sp_bytes);
    if (!ws) { *ws_bytes = need; return ok(); }
    if (*ws_bytes < need) return fail(HYS_ERR_WORKSPACE, "workspace %zu < required %zu bytes", *ws_bytes, need);
    if (!aligned16(ws)) return fail(HYS_ERR_INVALID_ARG, "workspace not 16-byte aligned");
    char* w = (char*)ws;
    float* ts = (float*)w;
    w += up(ts_bytes);
    float* po_all = (float*)w;
    float* pml_all = po_all + po_floats;
    w += up((po_floats + pml_floats) * sizeof(float));
    void* tkws = w;
    w += up(tk);
    float* sp_part = (float*)w;
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu < 1)
      return fail(HYS_ERR_HIP, "device query failed");

    hipStream_t st = (hipStream_t)stream;
    const float logit_scale = p->softmax_scale;
    const size_t oes = o_full.dtype == HYS_F32 ? 4 : 2;
    // the KV heads as the "layers" of one split launch (up to kMaxDecodeLayers at a time)
    for (int64_t g0 = 0; g0 < Hkv; g0 += hys::kMaxDecodeLayers) {
      const int nl = (int)std::min<int64_t>(hys::kMaxDecodeLayers, Hkv - g0);
      hys::DecArgs d{};
      for (int l = 0; l < nl; ++l) d.q[l] = (const uint16_t*)q_full.ptr + (g0 + l) * G * q_full.stride[2];
      d.q_sb = q_full.stride[0]; d.q_sh = q_full.stride[2];
      d.k = (const uint16_t*)k_cache.ptr + g0 * k_cache.stride[2]; d.k_sb = k_cache.stride[0]; d.k_st = k_cache.stride[1];
      d.v = (const uint16_t*)v_cache.ptr + g0 * v_cache.stride[2]; d.v_sb = v_cache.stride[0]; d.v_st = v_cache.stride[1];
      d.k_sl = k_cache.stride[2]; d.v_sl = v_cache.stride[2]; d.sc_sl = B * Nmax;
      for (int64_t b = 0; b < B; ++b) d.lens[b] = (int)cache_len[b];
      d.B = (int)B; d.Hq = (int)G; d.Nmax = (int)Nmax; d.ncu = ncu;
      d.scale_log2 = logit_scale * 1.4426950408889634f; d.logit_scale = logit_scale;
      d.nsplit = nsplit; d.nlayer = nl;
      d.scores = ts + (size_t)g0 * B * Nmax; d.sc_sb = Nmax;
      d.part_o = po_all + (size_t)(g0 * B * nsplit * G) * D;
      d.part_ml = pml_all + (size_t)(g0 * B * nsplit * G) * 2;
      HYS_DCHECK((int64_t)nl * B * nsplit < ((int64_t)1 << 31));
      hipError_t e = hys::launch_decode(0, hys::ET_BF16, (int)D, d, st);
      if (e != hipSuccess) return hip_status(e, "decode split launch");
    }
    // the KV heads' merges, as the "layers" of one merge launch (up to kMaxDecodeLayers at a time)
    for (int64_t g0 = 0; g0 < Hkv; g0 += hys::kMaxDecodeLayers) {
      const int nl = (int)std::min<int64_t>(hys::kMaxDecodeLayers, Hkv - g0);
      hys::MergeArgs m{};
      m.B = (int)B; m.Hq = (int)G; m.logit_scale = logit_scale; m.v_scale = 1.f;
      m.scale_log2 = logit_scale * 1.4426950408889634f;
      m.part_o = po_all + (size_t)(g0 * B * nsplit * G) * D;
      m.part_ml = pml_all + (size_t)(g0 * B * nsplit * G) * 2;
      m.nsplit = nsplit; m.nlayer = nl;
      for (int l = 0; l < nl; ++l) m.o[l] = (char*)o_full.ptr + (size_t)((g0 + l) * G * o_full.stride[2]) * oes;
      m.o_sb = o_full.stride[0]; m.o_sh = o_full.stride[2]; m.o_f32 = o_full.dtype == HYS_F32;
      hipError_t e = hys::launch_decode_merge((int)D, m, st);
      if (e != hipSuccess) return hip_status(e, "decode merge launch");
    }
    hipError_t e = hys::launch_hs_block_max(ts, (int)Hkv, B * Nmax, (int)B, (int)Nmax, (int)nblk, block_scores, st);
    if (e != hipSuccess) return hip_status(e, "block score launch");
    hys_status ts_status = topk_launch(block_scores, B, nblk, nblk, p->topk, idx, nullptr, tkws, st);
    if (ts_status != HYS_OK) return ts_status;
    if (n_sparse > 0) {
      hys::HsDecArgs h{};
      h.k = (const uint16_t*)k_cache.ptr; h.k_sb = k_cache.stride[0]; h.k_st = k_cache.stride[1]; h.k_sh = k_cache.stride[2];
      h.v = (const uint16_t*)v_cache.ptr; h.v_sb = v_cache.stride[0]; h.v_st = v_cache.stride[1]; h.v_sh = v_cache.stride[2];
      for (int64_t b = 0; b < B; ++b) h.lens[b] = (int)cache_len[b];
      h.B = (int)B; h.Hkv = (int)Hkv; h.G = (int)G; h.nlayer = n_sparse; h.topk = p->topk; h.W = (int)W;
      h.nsplit = hs_split; h.part = sp_part;
      h.scale_log2 = logit_scale * 1.4426950408889634f;
      h.idx = idx; h.idx_sb = p->topk;
      h.q_sb = q_sparse[0].stride[0]; h.q_sh = q_sparse[0].stride[2];
      h.n_sb = k_win_new[0].stride[0]; h.n_sh = k_win_new[0].stride[2];
      h.r_sb = k_ring[0].stride[0]; h.r_st = k_ring[0].stride[1]; h.r_sh = k_ring[0].stride[2];
      h.o_sb = o_sparse[0].stride[0]; h.o_sh = o_sparse[0].stride[2]; h.o_f32 = o_sparse[0].dtype == HYS_F32;
      for (int l = 0; l < n_sparse; ++l) {
        h.q[l] = (const uint16_t*)q_sparse[l].ptr;
        h.knew[l] = (const uint16_t*)k_win_new[l].ptr; h.vnew[l] = (const uint16_t*)v_win_new[l].ptr;
        h.kring[l] = (uint16_t*)k_ring[l].ptr; h.vring[l] = (uint16_t*)v_ring[l].ptr;
        h.gate_w[l] = gate_w[l];
        h.o[l] = o_sparse[l].ptr;
      }
      e = hys::launch_hs_decode_sparse((int)D, h, st);
      if (e != hipSuccess) return hip_status(e, "sparse layer launch");
    }
    return ok();
  } catch (...) {
    return fail(HYS_ERR_INTERNAL, "internal error");
  }
}


// ---------------------------------------------------------------------------
// backward pass
// ---------------------------------------------------------------------------
hys_status hys_window_attn_fwd(const hys_attn_params* p, hys_tensor4 q, hys_tensor4 k_win, hys_tensor4 v_win,
                               int32_t window, hys_tensor4 o, float* lse, void* stream) {
  try {
    hys_status s;
    if ((s = check_params(p)) != HYS_OK) return s;
    if ((s = check_qkv(q, k_win, v_win, p->q_offset)) != HYS_OK) return s;
    if (k_win.dtype != q.dtype && !(q.dtype == HYS_BF16 && k_win.dtype == HYS_FP8_E4M3))
      return fail(HYS_ERR_UNSUPPORTED, "window K/V must have q's dtype or be fp8 with bf16 q");
    if ((s = check_out(o, q, "o")) != HYS_OK) return s;
    if (window < 1) return fail(HYS_ERR_INVALID_ARG, "window must be >= 1");
    const int64_t B = q.shape[0], L = q.shape[1], Hq = q.shape[2], Hkv = k_win.shape[2], D = q.shape[3];
    const int64_t G = Hq / Hkv;
    if (L == 0) return ok();
    hys::AttnArgs a = base_args(p, q, k_win, v_win, o, lse);
    a.window = window;
    a.nb = 1;
    if (G > 128) return fail(HYS_ERR_UNSUPPORTED, "more than 128 query heads per KV head");
    a.HC = (int)G; a.BQ = (int)(128 / G); a.nhc = 1;
    a.ntq = (int)((L + a.BQ - 1) / a.BQ);
    a.gate_w = nullptr;                       // no gate: the window branch alone, with its LSE
    const int grid = (int)(B * a.ntq * Hkv);
    a.grid_used = grid;
    if ((s = check_attn_launch(a, hys::M_SWA_GATE, grid)) != HYS_OK) return s;
    return hip_status(hys::launch_attn(hys::M_SWA_GATE, et(q.dtype), et(k_win.dtype), (int)D, a, grid,
                                       (hipStream_t)stream),
                      "window launch");
  } catch (...) {
    return fail(HYS_ERR_INTERNAL, "internal error");
  }
}

}  // extern "C"

namespace {

hys_status check_grad(const hys_tensor4& g, const hys_tensor4& like, const char* name) {
  hys_status s;
  if ((s = check_tensor(g, name, false)) != HYS_OK) return s;
  if (g.dtype != HYS_F32) return fail(HYS_ERR_UNSUPPORTED, "%s must be fp32", name);
  for (int i = 0; i < 4; ++i)
    if (g.shape[i] != like.shape[i]) return fail(HYS_ERR_INVALID_ARG, "%s: shape differs from its input", name);
  return HYS_OK;
}

bool same_strides(const hys_tensor4& x, const hys_tensor4& y) {
  for (int i = 0; i < 3; ++i)
    if (x.stride[i] != y.stride[i] && x.shape[i] > 1) return false;
  return true;
}

// q, k, v bf16 self-attention inputs of a backward call, k and v sharing strides
hys_status check_bwd_inputs(const hys_attn_params* p, const hys_tensor4& q, const hys_tensor4& k,
                            const hys_tensor4& v, const char* what) {
  hys_status s;
  if ((s = check_params(p)) != HYS_OK) return s;
  if (p->k_scale != 1.f || p->v_scale != 1.f) return fail(HYS_ERR_UNSUPPORTED, "k_scale and v_scale must be 1");
  if (p->q_offset != 0) return fail(HYS_ERR_UNSUPPORTED, "%s: the backward pass takes whole sequences (q_offset 0)", what);
  if ((s = check_qkv(q, k, v, 0)) != HYS_OK) return s;
  if (q.shape[1] != k.shape[1])
    return fail(HYS_ERR_UNSUPPORTED, "%s: the backward pass needs equal query and key lengths", what);
  if (q.dtype != HYS_BF16 || k.dtype != HYS_BF16)
    return fail(HYS_ERR_UNSUPPORTED, "%s: the backward pass takes bf16 q, k, v", what);
  if (!same_strides(k, v)) return fail(HYS_ERR_UNSUPPORTED, "%s: k and v must share strides", what);
  return HYS_OK;
}

hys::BwdArgs bwd_args(const hys_attn_params* p, const hys_tensor4& q, const hys_tensor4& k, const hys_tensor4& v,
                      const hys_tensor4& dq, const hys_tensor4& dk, float* dv) {
  hys::BwdArgs a{};
  a.q = (const uint16_t*)q.ptr; a.q_sb = q.stride[0]; a.q_st = q.stride[1]; a.q_sh = q.stride[2];
  a.k = (const uint16_t*)k.ptr; a.v = (const uint16_t*)v.ptr;
  a.k_sb = k.stride[0]; a.k_st = k.stride[1]; a.k_sh = k.stride[2];
  a.dq = (float*)dq.ptr; a.dq_sb = dq.stride[0]; a.dq_st = dq.stride[1]; a.dq_sh = dq.stride[2];
  a.dk = (float*)dk.ptr; a.dv = dv; a.dk_sb = dk.stride[0]; a.dk_st = dk.stride[1]; a.dk_sh = dk.stride[2];
  a.B = (int)q.shape[0]; a.L = (int)q.shape[1]; a.Lk = (int)k.shape[1];
  a.Hq = (int)q.shape[2]; a.Hkv = (int)k.shape[2]; a.G = a.Hq / a.Hkv;
  a.scale = p->softmax_scale;
  a.scale_log2 = p->softmax_scale * 1.4426950408889634f;
  a.ng = 1;
  return a;
}

size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

extern "C" {

hys_status hys_full_attn_bwd(const hys_attn_params* p, hys_tensor4 q, hys_tensor4 k, hys_tensor4 v, hys_tensor4 o,
                             const float* lse, hys_tensor4 d_o, hys_tensor4 dq, hys_tensor4 dk, hys_tensor4 dv,
                             int32_t accumulate_kv, void* ws, size_t* ws_bytes, void* stream) {
  try {
    hys_status s;
    if (!ws_bytes) return fail(HYS_ERR_INVALID_ARG, "ws_bytes must not be null");
    if ((s = check_bwd_inputs(p, q, k, v, "full layer")) != HYS_OK) return s;
    if ((s = check_out(o, q, "o")) != HYS_OK) return s;
    if ((s = check_out(d_o, q, "d_o")) != HYS_OK) return s;
    if (d_o.dtype != HYS_BF16) return fail(HYS_ERR_UNSUPPORTED, "d_o must be bf16");
    if ((s = check_grad(dq, q, "dq")) != HYS_OK) return s;
    if ((s = check_grad(dk, k, "dk")) != HYS_OK) return s;
    if ((s = check_grad(dv, v, "dv")) != HYS_OK) return s;
    if (!same_strides(dk, dv)) return fail(HYS_ERR_UNSUPPORTED, "dk and dv must share strides");
    if (!lse) return fail(HYS_ERR_INVALID_ARG, "null lse");
    if (accumulate_kv != 0 && accumulate_kv != 1) return fail(HYS_ERR_INVALID_ARG, "accumulate_kv must be 0 or 1");
    const int64_t B = q.shape[0], L = q.shape[1], Hq = q.shape[2], Hkv = k.shape[2], D = q.shape[3];
    int srb = 1;
    const int nsplit = hys::bwd_dkdv_plan(hys::BW_CAUSAL, (int)L, 0, &srb);
    const size_t n_dd = up256((size_t)(B * Hq * L) * sizeof(float));
    const size_t need = n_dd + hys::bwd_dkdv_ws_bytes(nsplit, (int)B, (int)L, (int)Hkv, (int)D);
    if (!ws) { *ws_bytes = need; return ok(); }
    if (*ws_bytes < need) return fail(HYS_ERR_WORKSPACE, "workspace %zu < required %zu bytes", *ws_bytes, need);
    if (!aligned16(ws)) return fail(HYS_ERR_INVALID_ARG, "workspace not 16-byte aligned");
    if (L == 0) return ok();
    hipStream_t st = (hipStream_t)stream;
    float* Dd = (float*)ws;
    hys::BwdPrepArgs pa{};
    pa.dO = d_o.ptr; pa.do_sb = d_o.stride[0]; pa.do_st = d_o.stride[1]; pa.do_sh = d_o.stride[2]; pa.do_f32 = 0;
    pa.o = o.ptr; pa.o_sb = o.stride[0]; pa.o_st = o.stride[1]; pa.o_sh = o.stride[2];
    pa.o_f32 = o.dtype == HYS_F32;
    pa.Dd = Dd; pa.B = (int)B; pa.L = (int)L; pa.Hq = (int)Hq; pa.D = (int)D;
    hipError_t e = hys::launch_bwd_prep_full(pa, st);
    if (e != hipSuccess) return hip_status(e, "backward preparation launch");
    hys::BwdArgs a = bwd_args(p, q, k, v, dq, dk, (float*)dv.ptr);
    a.dO = (const uint16_t*)d_o.ptr; a.do_sb = d_o.stride[0]; a.do_st = d_o.stride[1]; a.do_sh = d_o.stride[2];
    a.lse = lse; a.Dd = Dd;
    a.acc_q = 0; a.acc_kv = accumulate_kv;
    a.nsplit = nsplit; a.split_rb = srb;
    hys::bwd_dkdv_bind_ws(a, (char*)ws + n_dd, (int)D);
    if ((e = hys::launch_bwd_dq(hys::BW_CAUSAL, (int)D, a, st)) != hipSuccess) return hip_status(e, "dq launch");
    return hip_status(hys::launch_bwd_dkdv(hys::BW_CAUSAL, (int)D, a, st), "dk/dv launch");
  } catch (...) {
    return fail(HYS_ERR_INTERNAL, "internal error");
  }
}

hys_status hys_sparse_layer_bwd(const hys_attn_params* p, hys_tensor4 q, hys_tensor4 k, hys_tensor4 v,
                                const hys_sparse_params* sp, const int32_t* idx, hys_tensor4 k_win, hys_tensor4 v_win,
                                int32_t window, const float* gate_w, const float* gate_b, hys_tensor4 o_sparse,
                                const float* lse_sparse, hys_tensor4 o_win, const float* lse_win, hys_tensor4 d_o,
                                hys_tensor4 dq, hys_tensor4 dk, hys_tensor4 dv, int32_t accumulate_kv,
                                hys_tensor4 dk_win, hys_tensor4 dv_win, float* dgate_w, float* dgate_b, void* ws,
                                size_t* ws_bytes, void* stream) {
  try {
    hys_status s;
    if (!ws_bytes) return fail(HYS_ERR_INVALID_ARG, "ws_bytes must not be null");
    if ((s = check_bwd_inputs(p, q, k, v, "shared K/V")) != HYS_OK) return s;
    if ((s = check_bwd_inputs(p, q, k_win, v_win, "window K/V")) != HYS_OK) return s;
    for (int i = 0; i < 4; ++i)
      if (k_win.shape[i] != k.shape[i]) return fail(HYS_ERR_INVALID_ARG, "window K/V shapes differ from k/v");
    if ((s = check_out(o_sparse, q, "o_sparse")) != HYS_OK) return s;
    if ((s = check_out(o_win, q, "o_win")) != HYS_OK) return s;
    if ((s = check_out(d_o, q, "d_o")) != HYS_OK) return s;
    if ((s = check_grad(dq, q, "dq")) != HYS_OK) return s;
    if ((s = check_grad(dk, k, "dk")) != HYS_OK) return s;
    if ((s = check_grad(dv, v, "dv")) != HYS_OK) return s;
    if ((s = check_grad(dk_win, k_win, "dk_win")) != HYS_OK) return s;
    if ((s = check_grad(dv_win, v_win, "dv_win")) != HYS_OK) return s;
    if (!same_strides(dk, dv) || !same_strides(dk_win, dv_win))
      return fail(HYS_ERR_UNSUPPORTED, "dk and dv (dk_win and dv_win) must share strides");
    if (!lse_sparse || !lse_win || !gate_w || !dgate_w)
      return fail(HYS_ERR_INVALID_ARG, "null lse_sparse, lse_win, gate_w or dgate_w");
    if (window < 1) return fail(HYS_ERR_INVALID_ARG, "window must be >= 1");
    if (accumulate_kv != 0 && accumulate_kv != 1) return fail(HYS_ERR_INVALID_ARG, "accumulate_kv must be 0 or 1");
    if (!sp) return fail(HYS_ERR_INVALID_ARG, "null sparse params");
    if (sp->granularity != 64 || sp->q_tile != 1 || sp->forced_window != 0)
      return fail(HYS_ERR_UNSUPPORTED, "granularity 64, q_tile 1 and no forced window");
    if (sp->k < 0 || sp->k > 64) return fail(HYS_ERR_UNSUPPORTED, "k must be in [0, 64]");
    if (sp->k > 0 && !idx) return fail(HYS_ERR_INVALID_ARG, "null idx");
    if (sp->idx_row_stride < sp->k || sp->idx_batch_stride < 0 || sp->idx_group_stride < 0)
      return fail(HYS_ERR_INVALID_ARG, "idx strides too small");
    const int64_t B = q.shape[0], L = q.shape[1], Hq = q.shape[2], Hkv = k.shape[2], D = q.shape[3];
    const int64_t nblk = (L + 63) / 64;
    if (nblk > 16384) return fail(HYS_ERR_UNSUPPORTED, "more than 16384 key blocks");
    const int64_t nwords = (nblk + 31) / 32;
    const int64_t ng = sp->idx_group_stride > 0 ? Hkv : 1;
    const size_t n_do = (size_t)(B * L * Hq * D) * 2, n_row = (size_t)(B * Hq * L) * 4;
    const size_t n_rb = (size_t)(ng * B * L * nwords) * 4;
    const size_t n_rl = (size_t)(ng * B * nblk * L) * 4, n_rc = (size_t)(ng * B * nblk) * 4;
    const size_t n_tb16 = (size_t)(ng * B * ((L + 15) / 16) * nwords) * 4;
    const size_t n_gp = hys::bwd_gate_partial_floats((int)Hq, (int)D) * 4;
    int srb = 1, wsrb = 1;
    const int nsplit = hys::bwd_dkdv_plan(hys::BW_BLOCK, (int)L, 0, &srb);
    hys::bwd_dkdv_plan(hys::BW_WINDOW, (int)L, window, &wsrb);
    const size_t n_kv = hys::bwd_dkdv_ws_bytes(nsplit, (int)B, (int)L, (int)Hkv, (int)D);
    const size_t need = 2 * up256(n_do) + 3 * up256(n_row) + up256(n_rb) + up256(n_rl) + up256(n_rc) +
                        up256(n_tb16) + up256(n_gp) + n_kv;
    if (!ws) { *ws_bytes = need; return ok(); }
    if (*ws_bytes < need) return fail(HYS_ERR_WORKSPACE, "workspace %zu < required %zu bytes", *ws_bytes, need);
    if (!aligned16(ws)) return fail(HYS_ERR_INVALID_ARG, "workspace not 16-byte aligned");
    if (L == 0) return ok();
    char* w = (char*)ws;
    uint16_t* do_sp = (uint16_t*)w; w += up256(n_do);
    uint16_t* do_w = (uint16_t*)w; w += up256(n_do);
    float* Dd_sp = (float*)w; w += up256(n_row);
    float* Dd_w = (float*)w; w += up256(n_row);
    float* dz = (float*)w; w += up256(n_row);
    uint32_t* rowbits = (uint32_t*)w; w += up256(n_rb);
    int32_t* rowlist = (int32_t*)w; w += up256(n_rl);
    int32_t* rowcnt = (int32_t*)w; w += up256(n_rc);
    uint32_t* tilebits16 = (uint32_t*)w; w += up256(n_tb16);
    float* gpart = (float*)w; w += up256(n_gp);
    void* kvws = w;
    hipStream_t st = (hipStream_t)stream;
    hipError_t e;

    hys::BwdGateArgs ga{};
    ga.q = (const uint16_t*)q.ptr; ga.q_sb = q.stride[0]; ga.q_st = q.stride[1]; ga.q_sh = q.stride[2];
    ga.dO = d_o.ptr; ga.do_sb = d_o.stride[0]; ga.do_st = d_o.stride[1]; ga.do_sh = d_o.stride[2];
    ga.do_f32 = d_o.dtype == HYS_F32;
    ga.osp = o_sparse.ptr; ga.osp_sb = o_sparse.stride[0]; ga.osp_st = o_sparse.stride[1];
    ga.osp_sh = o_sparse.stride[2]; ga.osp_f32 = o_sparse.dtype == HYS_F32;
    ga.ow = o_win.ptr; ga.ow_sb = o_win.stride[0]; ga.ow_st = o_win.stride[1]; ga.ow_sh = o_win.stride[2];
    ga.ow_f32 = o_win.dtype == HYS_F32;
    ga.lse_sp = lse_sparse; ga.gate_w = gate_w; ga.gate_b = gate_b;
    ga.do_sp = do_sp; ga.do_w = do_w; ga.Dd_sp = Dd_sp; ga.Dd_w = Dd_w; ga.dz = dz;
    ga.dq = (float*)dq.ptr; ga.dq_sb = dq.stride[0]; ga.dq_st = dq.stride[1]; ga.dq_sh = dq.stride[2];
    ga.B = (int)B; ga.L = (int)L; ga.Hq = (int)Hq; ga.D = (int)D;
    if ((e = hys::launch_bwd_prep_gate(ga, st)) != hipSuccess) return hip_status(e, "gate preparation launch");
    if ((e = hys::launch_bwd_gate_grad(dz, (const uint16_t*)q.ptr, q.stride[0], q.stride[1], q.stride[2], (int)B,
                                       (int)L, (int)Hq, (int)D, gpart, dgate_w, dgate_b, st)) != hipSuccess)
      return hip_status(e, "gate gradient launch");
    if ((e = hys::launch_bwd_selbits(idx, sp->idx_group_stride, sp->idx_batch_stride, sp->idx_row_stride, sp->k,
                                     (int)ng, (int)B, (int)L, (int)nblk, (int)nwords, rowbits, tilebits16, rowlist,
                                     rowcnt, st)) !=
        hipSuccess)
      return hip_status(e, "selection bitmap launch");

    // block-sparse branch over the shared K/V
    const int64_t do_st = Hq * D, do_sb = L * Hq * D;
    hys::BwdArgs a = bwd_args(p, q, k, v, dq, dk, (float*)dv.ptr);
    a.dO = do_sp; a.do_sb = do_sb; a.do_st = do_st; a.do_sh = D;
    a.lse = lse_sparse; a.Dd = Dd_sp;
    a.rowbits = rowbits; a.rowlist = rowlist; a.rowcnt = rowcnt; a.tilebits16 = tilebits16;
    a.nwords = (int)nwords; a.ng = (int)ng;
    HYS_DCHECK(a.Lk == (int)L && (int64_t)srb * 32 * nsplit >= L);
    a.acc_q = 1; a.acc_kv = accumulate_kv;
    a.nsplit = nsplit; a.split_rb = srb;
    hys::bwd_dkdv_bind_ws(a, kvws, (int)D);
    if ((e = hys::launch_bwd_dq(hys::BW_BLOCK, (int)D, a, st)) != hipSuccess) return hip_status(e, "sparse dq launch");
    if ((e = hys::launch_bwd_dkdv(hys::BW_BLOCK, (int)D, a, st)) != hipSuccess)
      return hip_status(e, "sparse dk/dv launch");
    // window branch over the layer's own K/V
    hys::BwdArgs wa = bwd_args(p, q, k_win, v_win, dq, dk_win, (float*)dv_win.ptr);
    wa.dO = do_w; wa.do_sb = do_sb; wa.do_st = do_st; wa.do_sh = D;
    wa.lse = lse_win; wa.Dd = Dd_w; wa.window = window;
    wa.acc_q = 1; wa.acc_kv = 0;
    wa.nsplit = 1; wa.split_rb = wsrb;
    if ((e = hys::launch_bwd_dq(hys::BW_WINDOW, (int)D, wa, st)) != hipSuccess) return hip_status(e, "window dq launch");
    return hip_status(hys::launch_bwd_dkdv(hys::BW_WINDOW, (int)D, wa, st), "window dk/dv launch");
  } catch (...) {
    return fail(HYS_ERR_INTERNAL, "internal error");
  }
}

}  // extern "C"
