// C-ABI of the attention library: argument validation, status codes, the decode
// split chooser, workspace handling and dispatch to the gfx950 kernels.  Every
// argument is checked before any HIP call; nothing throws across the interface.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "attn.h"

#include "attn_launch.h"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = 0;
  return ATTN_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool head_dim_ok(int d) { return d == 32 || d == 64 || d == 96 || d == 128 || d == 256; }

int check_common(int B, int H, int rows, int d, int dtype, float scale, const char* rows_name) {
  if (B < 1 || H < 1 || rows < 1)
    return fail(ATTN_ERR_INVALID_ARG, "B=%d, H=%d and %s=%d must all be >= 1", B, H, rows_name, rows);
  if (dtype != ATTN_F16 && dtype != ATTN_BF16) return fail(ATTN_ERR_INVALID_ARG, "dtype %d is not ATTN_F16/ATTN_BF16", dtype);
  if (!head_dim_ok(d))
    return fail(ATTN_ERR_UNSUPPORTED, "head dimension d=%d has no kernel (32, 64, 96, 128 or 256)", d);
  if (!std::isfinite(scale)) return fail(ATTN_ERR_INVALID_ARG, "scale must be finite");
  // Element offsets are formed in 64 bits, but per-head row counts and grid sizes stay in int.
  const long long elems = (long long)B * H * rows;
  if (elems > (1LL << 40) / d) return fail(ATTN_ERR_INVALID_ARG, "tensor too large");
  return ATTN_OK;
}

// The decode kernels carry the batch and the head (or head group) in the launch grid's
// second and third dimensions, whose limit is 65535.
constexpr int kDecodeGridMax = 65535;
int check_decode_grid(int B, int H) {
  if (B > kDecodeGridMax || H > kDecodeGridMax)
    return fail(ATTN_ERR_INVALID_ARG, "decode takes B and H up to %d (B=%d, H=%d)", kDecodeGridMax, B, H);
  return ATTN_OK;
}

int check_heads(int H, int Hkv) {
  if (Hkv < 1 || Hkv > H || H % Hkv != 0)
    return fail(ATTN_ERR_INVALID_ARG, "Hkv=%d must divide the query head count H=%d", Hkv, H);
  return ATTN_OK;
}

int check_ptr(const void* p, const char* name) {
  if (!p) return fail(ATTN_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(p)) return fail(ATTN_ERR_ALIGNMENT, "%s is not 16-byte aligned", name);
  return ATTN_OK;
}

// Compute units of the current device, queried once per device.
int device_cus(int* cus) {
  static std::mutex mu;
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(ATTN_ERR_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= 64) return fail(ATTN_ERR_HIP, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lk(mu);
  if (!cached[dev]) {
    int n = 0;
    hipError_t e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess || n <= 0) return fail(ATTN_ERR_HIP, "compute-unit count query failed: %s", hipGetErrorString(e));
    cached[dev] = n;
  }
  *cus = cached[dev];
  return ATTN_OK;
}

}  // namespace

extern "C" {

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID_ARG: return "invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case ATTN_ERR_ALIGNMENT: return "pointer not 16-byte aligned";
    case ATTN_ERR_WORKSPACE: return "workspace too small";
    case ATTN_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* attn_last_error(void) { return g_err; }

#ifndef ATTN_SOURCE_HASH
#define ATTN_SOURCE_HASH "unknown"
#endif
const char* attn_build_id(void) { return ATTN_SOURCE_HASH; }

static int prefill_impl(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H, int Hkv,
                        int N, int d, int dtype, int causal, float scale, void* stream) {
  int st;
  if ((st = check_common(B, H, N, d, dtype, scale, "N")) != ATTN_OK) return st;
  if ((st = check_heads(H, Hkv)) != ATTN_OK) return st;
  if (causal != 0 && causal != 1) return fail(ATTN_ERR_INVALID_ARG, "causal must be 0 or 1, got %d", causal);
  if ((st = check_ptr(q, "q")) || (st = check_ptr(k, "k")) || (st = check_ptr(v, "v")) || (st = check_ptr(out, "out")))
    return st;
  if (out == q || out == k || out == v) return fail(ATTN_ERR_INVALID_ARG, "out must not alias an input");
  if (lse) {
    if (((uintptr_t)lse & 3u) != 0) return fail(ATTN_ERR_ALIGNMENT, "lse is not 4-byte aligned");
    if ((void*)lse == q || (void*)lse == k || (void*)lse == v || (void*)lse == out)
      return fail(ATTN_ERR_INVALID_ARG, "lse must not alias another tensor");
  }
  int cus = 0;
  if ((st = device_cus(&cus)) != ATTN_OK) return st;
  hipError_t e =
      attn::launch_prefill(q, k, v, out, lse, B, H, Hkv, N, d, dtype, causal, scale, cus, (hipStream_t)stream);
  if (e != hipSuccess) return fail(ATTN_ERR_HIP, "prefill launch failed: %s", hipGetErrorString(e));
  return ok();
}

int attn_prefill(const void* q, const void* k, const void* v, void* out, int B, int H, int N, int d, int dtype,
                 int causal, float scale, void* stream) {
  return prefill_impl(q, k, v, out, nullptr, B, H, H, N, d, dtype, causal, scale, stream);
}

int attn_prefill_gqa(const void* q, const void* k, const void* v, void* out, int B, int Hq, int Hkv, int N, int d,
                     int dtype, int causal, float scale, void* stream) {
  return prefill_impl(q, k, v, out, nullptr, B, Hq, Hkv, N, d, dtype, causal, scale, stream);
}

int attn_prefill_ex(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq, int Hkv, int N,
                    int d, int dtype, int causal, float scale, void* stream) {
  return prefill_impl(q, k, v, out, lse, B, Hq, Hkv, N, d, dtype, causal, scale, stream);
}

int attn_prefill_plan(int B, int H, int N, int d, int causal, int num_cus, int* waves_per_workgroup,
                      int* rows_per_wave, int* lds_stages, int* key_groups) {
  if (B < 1 || H < 1 || N < 1 || num_cus < 1) return fail(ATTN_ERR_INVALID_ARG, "B, H, N and num_cus must be >= 1");
  if (!head_dim_ok(d))
    return fail(ATTN_ERR_UNSUPPORTED, "head dimension d=%d has no kernel (32, 64, 96, 128 or 256)", d);
  if (causal != 0 && causal != 1) return fail(ATTN_ERR_INVALID_ARG, "causal must be 0 or 1, got %d", causal);
  if (!waves_per_workgroup || !rows_per_wave || !lds_stages || !key_groups)
    return fail(ATTN_ERR_INVALID_ARG, "the plan outputs must be non-NULL host pointers");
  const attn::PrefillForm f = attn::prefill_form(B, H, N, d, causal, num_cus);
  *waves_per_workgroup = f.nw;
  *rows_per_wave = 32 * f.qb;
  *lds_stages = f.st;
  *key_groups = f.kg;
  return ok();
}

// The split for `pairs` wave columns (one wave per column and split) aiming at
// `target` waves in all.
static void choose_split_core(long long pairs, int max_len, long long target, int* chunk, int* n_split) {
  const long long T = ATTN_DECODE_ROW_GRANULE;
  // Smallest chunk: ATTN_DECODE_MIN_CHUNK rows, or the whole (granule-rounded) cache
  // when it is shorter.
  const long long rounded_len = (max_len + T - 1) / T * T;
  const long long cmin = rounded_len < ATTN_DECODE_MIN_CHUNK ? rounded_len : ATTN_DECODE_MIN_CHUNK;
  const long long max_splits = (max_len + cmin - 1) / cmin;
  long long ns = (target + pairs - 1) / pairs;
  if (ns < 1) ns = 1;
  if (ns > max_splits) ns = max_splits;
  long long c = (max_len + ns - 1) / ns;
  c = (c + T - 1) / T * T;
  if (c < cmin) c = cmin;
  // Rounding the chunk up to the granule can drop the split count below the target;
  // shrink it one granule at a time until the target is met again.
  while (c - T >= cmin && pairs * ((max_len + c - 1) / c) < target) c -= T;
  *chunk = (int)c;
  *n_split = (int)((max_len + c - 1) / c);
}

int attn_decode_choose_split(int B, int H, int max_len, int d, int num_cus, int* chunk, int* n_split) {
  if (B < 1 || H < 1 || max_len < 1 || num_cus < 1)
    return fail(ATTN_ERR_INVALID_ARG, "B, H, max_len and num_cus must be >= 1");
  if (!head_dim_ok(d))
    return fail(ATTN_ERR_UNSUPPORTED, "head dimension d=%d has no kernel (32, 64, 96, 128 or 256)", d);
  if (!chunk || !n_split) return fail(ATTN_ERR_INVALID_ARG, "chunk and n_split must be non-NULL host pointers");
  choose_split_core((long long)B * H, max_len, (long long)ATTN_DECODE_WGS_PER_CU * num_cus, chunk, n_split);
  return ok();
}

size_t attn_backward_workspace_bytes(int B, int Hq, int N) {
  if (B < 1 || Hq < 1 || N < 1) return 0;
  return 2 * (size_t)B * Hq * N * sizeof(float);
}

int attn_backward(const void* q, const void* k, const void* v, const void* out, const void* dout, const float* lse,
                  void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int N, int d, int dtype, int causal,
                  float scale, void* workspace, size_t ws_bytes, void* stream) {
  int st;
  if ((st = check_common(B, Hq, N, d, dtype, scale, "N")) != ATTN_OK) return st;
  if ((st = check_heads(Hq, Hkv)) != ATTN_OK) return st;
  if (causal != 0 && causal != 1) return fail(ATTN_ERR_INVALID_ARG, "causal must be 0 or 1, got %d", causal);
  if ((st = check_ptr(q, "q")) || (st = check_ptr(k, "k")) || (st = check_ptr(v, "v")) ||
      (st = check_ptr(out, "out")) || (st = check_ptr(dout, "dout")) || (st = check_ptr(dq, "dq")) ||
      (st = check_ptr(dk, "dk")) || (st = check_ptr(dv, "dv")))
    return st;
  if (!lse) return fail(ATTN_ERR_INVALID_ARG, "lse is NULL");
  if (((uintptr_t)lse & 3u) != 0) return fail(ATTN_ERR_ALIGNMENT, "lse is not 4-byte aligned");
  const void* ins[] = {q, k, v, out, dout, lse};
  const void* outs[] = {dq, dk, dv};
  for (const void* o : outs)
    for (const void* i : ins)
      if (o == i) return fail(ATTN_ERR_INVALID_ARG, "a gradient output aliases an input");
  if (dq == dk || dq == dv || dk == dv) return fail(ATTN_ERR_INVALID_ARG, "gradient outputs must be distinct");
  if (workspace && !aligned16(workspace)) return fail(ATTN_ERR_ALIGNMENT, "workspace is not 16-byte aligned");
  if (!workspace && ws_bytes != 0) return fail(ATTN_ERR_INVALID_ARG, "workspace is NULL but ws_bytes > 0");
  const size_t need = attn_backward_workspace_bytes(B, Hq, N);
  if (workspace && ws_bytes < need)
    return fail(ATTN_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", ws_bytes, need);
  int cus = 0;
  if ((st = device_cus(&cus)) != ATTN_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  void* ws = workspace;
  bool own = false;
  if (!workspace) {
    hipError_t e = hipMallocAsync(&ws, need, s);
    if (e != hipSuccess) return fail(ATTN_ERR_HIP, "workspace allocation of %zu bytes failed: %s", need, hipGetErrorString(e));
    own = true;
  }
  hipError_t e = attn::launch_backward(q, k, v, out, dout, lse, (float*)ws, dq, dk, dv, B, Hq, Hkv, N, d, dtype, causal,
                                       scale, cus, s);
  if (own) {
    hipError_t e2 = hipFreeAsync(ws, s);
    if (e == hipSuccess) e = e2;
  }
  if (e != hipSuccess) return fail(ATTN_ERR_HIP, "backward launch failed: %s", hipGetErrorString(e));
  return ok();
}

int attn_decode_gqa_choose_split(int B, int Hq, int Hkv, int max_len, int d, int num_cus, int* chunk, int* n_split) {
  if (Hq < 1 || Hkv < 1 || Hkv > Hq || Hq % Hkv != 0)
    return fail(ATTN_ERR_INVALID_ARG, "Hkv=%d must divide the query head count Hq=%d", Hkv, Hq);
  if (B < 1 || max_len < 1 || num_cus < 1) return fail(ATTN_ERR_INVALID_ARG, "B, max_len and num_cus must be >= 1");
  if (!head_dim_ok(d))
    return fail(ATTN_ERR_UNSUPPORTED, "head dimension d=%d has no kernel (32, 64, 96, 128 or 256)", d);
  if (!chunk || !n_split) return fail(ATTN_ERR_INVALID_ARG, "chunk and n_split must be non-NULL host pointers");
  // One wave serves decode_heads_per_wave query heads: that many fewer waves per split.
  const long long cols = (long long)B * (Hq / attn::decode_heads_per_wave(Hq, Hkv));
  // The matrix-core form holds LDS tiles, so fewer of its waves fit on a CU: aim at
  // one resident round of them rather than at the vector form's target.
  const int per_cu = attn::decode_uses_mfma(Hq, Hkv) ? attn::decode_mfma_waves_per_cu(d) : ATTN_DECODE_WGS_PER_CU;
  choose_split_core(cols, max_len, (long long)per_cu * num_cus, chunk, n_split);
  return ok();
}

size_t attn_decode_workspace_bytes(int B, int H, int n_split, int d) {
  if (B < 1 || H < 1 || n_split < 1 || d < 1) return 0;
  return (size_t)B * H * n_split * (size_t)(d + 2) * sizeof(float);
}

static int decode_impl(const void* q, const void* k_cache, const void* v_cache, const int32_t* seq_lens, void* out,
                       int B, int H, int Hkv, int max_len, int d, int dtype, float scale, int chunk, void* workspace,
                       size_t ws_bytes, void* stream, bool caller_ws, bool use_scratch = false,
                       int passes = attn::kDecodeSplitPass | attn::kDecodeMergePass) {
  int st;
  if ((st = check_common(B, H, max_len, d, dtype, scale, "max_len")) != ATTN_OK) return st;
  if ((st = check_decode_grid(B, H)) != ATTN_OK) return st;
  if ((st = check_heads(H, Hkv)) != ATTN_OK) return st;
  if ((st = check_ptr(q, "q")) || (st = check_ptr(k_cache, "k_cache")) || (st = check_ptr(v_cache, "v_cache")))
    return st;
  // The split pass alone writes no output.
  if ((passes & attn::kDecodeMergePass) && (st = check_ptr(out, "out"))) return st;
  if (!seq_lens) return fail(ATTN_ERR_INVALID_ARG, "seq_lens is NULL");
  if (((uintptr_t)seq_lens & 3u) != 0) return fail(ATTN_ERR_ALIGNMENT, "seq_lens is not 4-byte aligned");
  if (out == q || out == k_cache || out == v_cache) return fail(ATTN_ERR_INVALID_ARG, "out must not alias an input");
  const int T = ATTN_DECODE_ROW_GRANULE;
  const int cap = (max_len + T - 1) / T * T;
  if (chunk != 0 && (chunk < T || chunk % T != 0 || chunk > cap))
    return fail(ATTN_ERR_INVALID_ARG, "chunk=%d must be 0 or a multiple of %d in [%d, %d]", chunk, T, T, cap);
  if (caller_ws && workspace && !aligned16(workspace)) return fail(ATTN_ERR_ALIGNMENT, "workspace is not 16-byte aligned");
  if (caller_ws && !workspace && ws_bytes != 0) return fail(ATTN_ERR_INVALID_ARG, "workspace is NULL but ws_bytes > 0");

  int n_split = 0;
  if (use_scratch && chunk != 0 &&
      attn_decode_workspace_bytes(B, H, (max_len + chunk - 1) / chunk, d) > (size_t)ATTN_DECODE_SCRATCH_BYTES)
    return fail(ATTN_ERR_WORKSPACE, "the partials of chunk=%d (%zu bytes) exceed the %d-byte decode scratch", chunk,
                attn_decode_workspace_bytes(B, H, (max_len + chunk - 1) / chunk, d), ATTN_DECODE_SCRATCH_BYTES);
  if (use_scratch && attn_decode_workspace_bytes(B, H, 1, d) > (size_t)ATTN_DECODE_SCRATCH_BYTES)
    return fail(ATTN_ERR_WORKSPACE, "B*H=%lld partials of d=%d exceed the %d-byte decode scratch even with one split",
                (long long)B * H, d, ATTN_DECODE_SCRATCH_BYTES);
  if (chunk == 0) {
    int cus = 0;
    if ((st = device_cus(&cus)) != ATTN_OK) return st;
    if ((st = attn_decode_gqa_choose_split(B, H, Hkv, max_len, d, cus, &chunk, &n_split)) != ATTN_OK) return st;
    // The scratch form takes the smallest legal chunk at or above the automatic one
    // whose partials fit the scratch (one split always fits, checked above).
    while (use_scratch && attn_decode_workspace_bytes(B, H, n_split, d) > (size_t)ATTN_DECODE_SCRATCH_BYTES) {
      chunk += ATTN_DECODE_ROW_GRANULE;
      n_split = (max_len + chunk - 1) / chunk;
    }
  } else {
    n_split = (max_len + chunk - 1) / chunk;
  }
  const size_t need = attn_decode_workspace_bytes(B, H, n_split, d);
  hipStream_t s = (hipStream_t)stream;
  void* ws = workspace;
  bool own = false;
  if (use_scratch) {
    float* sp = nullptr;
    hipError_t e = attn::decode_scratch(&sp);
    if (e != hipSuccess) return fail(ATTN_ERR_HIP, "decode scratch lookup failed: %s", hipGetErrorString(e));
    ws = sp;
  } else if (!caller_ws || (workspace == nullptr && ws_bytes == 0)) {
    hipError_t e = hipMallocAsync(&ws, need, s);
    if (e != hipSuccess) return fail(ATTN_ERR_HIP, "workspace allocation of %zu bytes failed: %s", need, hipGetErrorString(e));
    own = true;
  } else if (ws_bytes < need) {
    return fail(ATTN_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", ws_bytes, need);
  }
  hipError_t e = attn::launch_decode(q, k_cache, v_cache, seq_lens, out, B, H, Hkv, max_len, d, dtype, scale, chunk,
                                     n_split, (float*)ws, s, passes);
  if (own) {
    hipError_t e2 = hipFreeAsync(ws, s);
    if (e == hipSuccess) e = e2;
  }
  if (e != hipSuccess) return fail(ATTN_ERR_HIP, "decode launch failed: %s", hipGetErrorString(e));
  return ok();
}

int attn_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* seq_lens, void* out, int B,
                int H, int max_len, int d, int dtype, float scale, void* stream) {
  return decode_impl(q, k_cache, v_cache, seq_lens, out, B, H, H, max_len, d, dtype, scale, 0, nullptr, 0, stream, false);
}

int attn_decode_ex(const void* q, const void* k_cache, const void* v_cache, const int32_t* seq_lens, void* out, int B,
                   int H, int max_len, int d, int dtype, float scale, int chunk, void* workspace, size_t ws_bytes,
                   void* stream) {
  return decode_impl(q, k_cache, v_cache, seq_lens, out, B, H, H, max_len, d, dtype, scale, chunk, workspace, ws_bytes,
                     stream, true);
}

int attn_decode_gqa(const void* q, const void* k_cache, const void* v_cache, const int32_t* seq_lens, void* out, int B,
                    int Hq, int Hkv, int max_len, int d, int dtype, float scale, int chunk, void* workspace,
                    size_t ws_bytes, void* stream) {
  return decode_impl(q, k_cache, v_cache, seq_lens, out, B, Hq, Hkv, max_len, d, dtype, scale, chunk, workspace,
                     ws_bytes, stream, true);
}

int attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, const int32_t* seq_lens, void* out,
                        int B, int Hq, int Hkv, int max_len, int d, int dtype, float scale, int chunk, void* stream) {
  return decode_impl(q, k_cache, v_cache, seq_lens, out, B, Hq, Hkv, max_len, d, dtype, scale, chunk, nullptr, 0,
                     stream, false, true);
}

int attn_decode_split(const void* q, const void* k_cache, const void* v_cache, const int32_t* seq_lens, int B, int Hq,
                      int Hkv, int max_len, int d, int dtype, float scale, int chunk, void* workspace, size_t ws_bytes,
                      void* stream) {
  if (chunk == 0) return fail(ATTN_ERR_INVALID_ARG, "the split pass needs an explicit chunk");
  if (!workspace) return fail(ATTN_ERR_INVALID_ARG, "the split pass needs a workspace");
  return decode_impl(q, k_cache, v_cache, seq_lens, nullptr, B, Hq, Hkv, max_len, d, dtype, scale, chunk, workspace,
                     ws_bytes, stream, true, false, attn::kDecodeSplitPass);
}

int attn_decode_merge(const void* workspace, size_t ws_bytes, void* out, int B, int Hq, int max_len, int d, int dtype,
                      int chunk, void* stream) {
  int st;
  if ((st = check_common(B, Hq, max_len, d, dtype, 1.f, "max_len")) != ATTN_OK) return st;
  if ((st = check_decode_grid(B, Hq)) != ATTN_OK) return st;
  if ((st = check_ptr(out, "out")) || (st = check_ptr(workspace, "workspace"))) return st;
  if (out == workspace) return fail(ATTN_ERR_INVALID_ARG, "out must not alias the workspace");
  const int T = ATTN_DECODE_ROW_GRANULE;
  const int cap = (max_len + T - 1) / T * T;
  if (chunk < T || chunk % T != 0 || chunk > cap)
    return fail(ATTN_ERR_INVALID_ARG, "chunk=%d must be a multiple of %d in [%d, %d]", chunk, T, T, cap);
  const int n_split = (max_len + chunk - 1) / chunk;
  const size_t need = attn_decode_workspace_bytes(B, Hq, n_split, d);
  if (ws_bytes < need) return fail(ATTN_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", ws_bytes, need);
  hipError_t e = attn::launch_decode(nullptr, nullptr, nullptr, nullptr, out, B, Hq, Hq, max_len, d, dtype, 1.f, chunk,
                                     n_split, (float*)workspace, (hipStream_t)stream, attn::kDecodeMergePass);
  if (e != hipSuccess) return fail(ATTN_ERR_HIP, "decode merge launch failed: %s", hipGetErrorString(e));
  return ok();
}

int attn_measure_read(const void* buf, size_t bytes, int waves, void* sink, size_t sink_bytes, void* stream) {
  if (!buf || !sink) return fail(ATTN_ERR_INVALID_ARG, "buf and sink must be non-NULL");
  if (!aligned16(buf)) return fail(ATTN_ERR_ALIGNMENT, "buf is not 16-byte aligned");
  if (((uintptr_t)sink & 3u) != 0) return fail(ATTN_ERR_ALIGNMENT, "sink is not 4-byte aligned");
  if (bytes < 16 || bytes % 16 != 0) return fail(ATTN_ERR_INVALID_ARG, "bytes=%zu must be a positive multiple of 16", bytes);
  if (waves < 1 || (size_t)waves > bytes / 16) return fail(ATTN_ERR_INVALID_ARG, "waves=%d must lie in [1, bytes/16]", waves);
  if (sink_bytes < (size_t)waves * 256)
    return fail(ATTN_ERR_WORKSPACE, "sink of %zu bytes is smaller than the %zu needed", sink_bytes, (size_t)waves * 256);
  hipError_t e = attn::launch_measure_read(buf, bytes, waves, (uint32_t*)sink, (hipStream_t)stream);
  if (e != hipSuccess) return fail(ATTN_ERR_HIP, "read launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
