// Decode: one query row per (batch, head) over a ragged KV cache, split-K.
//
// Page 3 of the pages ("Kernel design"): a single query row against thousands of
// cached rows has almost no parallelism of its own, so the cache is cut into chunks
// (split-K), each chunk produces a partial (m, l, acc), and a small second kernel
// merges the partials exactly, without atomics.  The chunk size is chosen at launch
// (host side) so that even a batch of one fills every compute unit.
//
// The split kernel is a streaming read of K and V rows: arithmetic intensity is about
// one flop per byte, so it is bound by HBM, not by the matrix cores, and runs on the
// vector ALUs.  A row of the cache (d 16-bit values) is read by d/8 lanes with one
// 16-byte load each, so one wave-wide load covers consecutive rows in one contiguous
// kilobyte.  Four row-groups per lane are loaded before any is used to keep enough
// bytes in flight.  Scores are kept in the base-2 domain (c = scale*log2(e)).
//
// Partial layout in the workspace, for pair = b*H + h and split s:
//   acc[(pair*n_split + s)*d + 0 .. d-1]  sum_t 2^(c s_t - m) v_t       (fp32)
//   ml [(pair*n_split + s)*2 + 0, 1]      m = max_t c s_t, l = sum_t 2^(c s_t - m)
// where acc is the first B*H*n_split*d floats and ml follows it.
#include "attn_device.h"

namespace attn {

namespace decode_cfg {
constexpr int kThreads = 256;
constexpr int kUnroll = 4;
constexpr int kGranule = 32;  // legal chunks are multiples of this many rows
}  // namespace decode_cfg

struct DecodeParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* seq_lens;
  uint16_t* o;
  float* ws_acc;
  float* ws_ml;
  int B, H, max_len, chunk, n_split;
  float c;  // scale * log2(e), any sign
};

__device__ __forceinline__ int clamp_len(int L, int max_len) { return L < 0 ? 0 : (L > max_len ? max_len : L); }

template <int DT, int D>
__global__ __launch_bounds__(decode_cfg::kThreads) void decode_split_kernel(DecodeParams p) {
  using namespace decode_cfg;
  constexpr int LPR = D / 8;             // lanes per cache row
  constexpr int RPW = 64 / LPR;          // rows per wave per load
  constexpr int NW = kThreads / 64;      // waves
  constexpr int RSTEP = NW * RPW;        // rows per workgroup per load
  constexpr int RITER = RSTEP * kUnroll;  // rows per loop iteration
  constexpr int NG = NW * RPW;           // independent row groups per workgroup

  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int L = clamp_len(p.seq_lens[b], p.max_len);
  const int r0 = s * p.chunk;
  if (r0 >= L) return;  // empty chunk: the merge pass never reads it
  const int r1 = min(L, r0 + p.chunk);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int seg = lane % LPR;       // which 8 elements of d
  const int rsub = lane / LPR;      // row within the wave's load
  const int grp = wave * RPW + rsub;  // row group id (0 .. NG-1)
  const size_t pair = (size_t)b * p.H + h;
  const uint16_t* kg = p.k + pair * p.max_len * D + seg * 8;
  const uint16_t* vg = p.v + pair * p.max_len * D + seg * 8;

  float qv[8];
  {
    const u32x4 t = *(const u32x4*)(p.q + pair * D + seg * 8);
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      qv[2 * x] = to_f32<DT>(t[x] & 0xffffu) * p.c;
      qv[2 * x + 1] = to_f32<DT>(t[x] >> 16) * p.c;
    }
  }

  float m = -INFINITY, l = 0.f, acc[8];
#pragma unroll
  for (int x = 0; x < 8; ++x) acc[x] = 0.f;

  for (int base = r0; base < r1; base += RITER) {
    u32x4 kr[kUnroll], vr[kUnroll];
    int rows[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      rows[u] = base + u * RSTEP + grp;
      kr[u] = (u32x4){0, 0, 0, 0};
      vr[u] = (u32x4){0, 0, 0, 0};
      if (rows[u] < r1) {
        kr[u] = *(const u32x4*)(kg + (size_t)rows[u] * D);
        vr[u] = *(const u32x4*)(vg + (size_t)rows[u] * D);
      }
    }
    float sc[kUnroll];
    float mx = m;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      float part = 0.f;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        part = __builtin_fmaf(qv[2 * x], to_f32<DT>(kr[u][x] & 0xffffu), part);
        part = __builtin_fmaf(qv[2 * x + 1], to_f32<DT>(kr[u][x] >> 16), part);
      }
      // Sum the LPR lanes of this row (aligned groups of LPR consecutive lanes).
#pragma unroll
      for (int off = 1; off < LPR; off <<= 1) part += __shfl_xor(part, off);
      sc[u] = rows[u] < r1 ? part : -INFINITY;
      mx = fmaxf(mx, sc[u]);
    }
    if (mx == -INFINITY) continue;  // nothing valid for this group in this iteration
    const float alpha = fast_exp2(m - mx);  // m = -inf gives 0
    m = mx;
    l *= alpha;
#pragma unroll
    for (int x = 0; x < 8; ++x) acc[x] *= alpha;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const float pu = fast_exp2(sc[u] - m);  // -inf gives 0
      l += pu;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        acc[2 * x] = __builtin_fmaf(pu, to_f32<DT>(vr[u][x] & 0xffffu), acc[2 * x]);
        acc[2 * x + 1] = __builtin_fmaf(pu, to_f32<DT>(vr[u][x] >> 16), acc[2 * x + 1]);
      }
    }
  }

  // Merge the NG row groups of this workgroup through LDS.
  __shared__ float sm_m[NG], sm_l[NG], sm_w[NG];
  __shared__ float sm_acc[NG][D + 1];
  if (seg == 0) {
    sm_m[grp] = m;
    sm_l[grp] = l;
  }
#pragma unroll
  for (int x = 0; x < 8; ++x) sm_acc[grp][seg * 8 + x] = acc[x];
  __syncthreads();
  __shared__ float sm_M;
  if (tid == 0) {
    float M = -INFINITY;
    for (int g = 0; g < NG; ++g) M = fmaxf(M, sm_m[g]);
    sm_M = M;
  }
  __syncthreads();
  const float M = sm_M;
  if (tid < NG) sm_w[tid] = (sm_m[tid] == -INFINITY) ? 0.f : fast_exp2(sm_m[tid] - M);
  __syncthreads();
  const size_t pidx = pair * p.n_split + s;
  if (tid < D) {
    float a = 0.f;
    for (int g = 0; g < NG; ++g) a = __builtin_fmaf(sm_w[g], sm_acc[g][tid], a);
    p.ws_acc[pidx * D + tid] = a;
  }
  if (tid == 0) {
    float lt = 0.f;
    for (int g = 0; g < NG; ++g) lt = __builtin_fmaf(sm_w[g], sm_l[g], lt);
    p.ws_ml[pidx * 2 + 0] = M;
    p.ws_ml[pidx * 2 + 1] = lt;
  }
}

// Exact merge: O = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s over the non-empty
// splits s < ceil(L / chunk); a length of 0 writes zeros.
template <int DT, int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(DecodeParams p) {
  const int h = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const size_t pair = (size_t)b * p.H + h;
  const int L = clamp_len(p.seq_lens[b], p.max_len);
  const int nv = (L + p.chunk - 1) / p.chunk;
  const float* ml = p.ws_ml + pair * p.n_split * 2;
  const float* ac = p.ws_acc + pair * p.n_split * D;
  float M = -INFINITY;
  for (int s = 0; s < nv; ++s) M = fmaxf(M, ml[2 * s]);
  float num = 0.f, den = 0.f;
  for (int s = 0; s < nv; ++s) {
    const float w = fast_exp2(ml[2 * s] - M);
    den = __builtin_fmaf(w, ml[2 * s + 1], den);
    num = __builtin_fmaf(w, ac[(size_t)s * D + t], num);
  }
  const float o = nv > 0 ? num / den : 0.f;
  // Pair up neighbouring lanes so each even lane stores one dword.
  const float o_next = __shfl_down(o, 1);
  if ((t & 1) == 0) *(uint32_t*)(p.o + pair * D + t) = pack2<DT>(o, o_next);
}

template <int DT, int D>
static hipError_t launch_decode_t(const DecodeParams& p, hipStream_t st) {
  hipLaunchKernelGGL((decode_split_kernel<DT, D>), dim3(p.n_split, p.H, p.B), dim3(decode_cfg::kThreads), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<DT, D>), dim3(p.H, p.B), dim3(D), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_decode(const void* q, const void* k, const void* v, const int32_t* seq_lens, void* o, int B, int H,
                         int max_len, int d, int dt, float scale, int chunk, int n_split, float* ws, hipStream_t st) {
  DecodeParams p;
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.seq_lens = seq_lens;
  p.o = (uint16_t*)o;
  p.ws_acc = ws;
  p.ws_ml = ws + (size_t)B * H * n_split * d;
  p.B = B;
  p.H = H;
  p.max_len = max_len;
  p.chunk = chunk;
  p.n_split = n_split;
  p.c = scale * kLog2e;
  if (dt == DT_F16 && d == 64) return launch_decode_t<DT_F16, 64>(p, st);
  if (dt == DT_F16 && d == 128) return launch_decode_t<DT_F16, 128>(p, st);
  if (dt == DT_BF16 && d == 64) return launch_decode_t<DT_BF16, 64>(p, st);
  if (dt == DT_BF16 && d == 128) return launch_decode_t<DT_BF16, 128>(p, st);
  return hipErrorInvalidValue;
}

}  // namespace attn
