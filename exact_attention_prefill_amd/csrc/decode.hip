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
// vector ALUs.  One wave owns one chunk.  A cache row (d 16-bit values) is read by d/8
// lanes with one 16-byte load each (d = 96: a group of 16 lanes, of which 12 load), so
// one wave-wide load covers consecutive rows of one contiguous stretch; two iterations
// of four such loads of K and of V are in flight per lane.  The wave's row groups are combined with cross-lane exchanges,
// so the kernel needs neither LDS nor barriers and many chunk-waves share a CU.
// Scores are kept in the base-2 domain (c = scale*log2(e)).
//
// Partial layout in the workspace, for pair = b*H + h and split s:
//   acc[(pair*n_split + s)*d + 0 .. d-1]  sum_t 2^(c s_t - m) v_t       (fp32)
//   ml [(pair*n_split + s)*2 + 0, 1]      m = max_t c s_t, l = sum_t 2^(c s_t - m)
// where acc is the first B*H*n_split*d floats and ml follows it.  A chunk at or past
// the sequence's length writes only (m, l) = (-inf, 0); its acc is never read.
#include "attn_device.h"

namespace attn {

namespace decode_cfg {
constexpr int kUnroll = 4;          // row loads of K (and of V) per lane per buffer (two buffers)
constexpr int kMergeThreads = 256;  // merge workgroup: 4 split groups x 64
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
  int Hkv, g;  // K/V heads and query heads per K/V head (H = Hkv * g)
  float c;     // scale * log2(e), any sign
};

__device__ __forceinline__ int clamp_len(int L, int max_len) { return L < 0 ? 0 : (L > max_len ? max_len : L); }

// Dot product of two packed pairs of 16-bit values, accumulated in fp32.
template <int DT>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc);
template <>
__device__ __forceinline__ float dot2<DT_BF16>(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), acc, false);
}
template <>
__device__ __forceinline__ float dot2<DT_F16>(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), acc, false);
}

// Combine two online-softmax states (m, l, acc[8]) exactly: the larger m wins and the
// other side is scaled by 2^(m_other - m).  m = -inf means empty.
__device__ __forceinline__ void combine(float& m, float& l, float (&acc)[8], float m2, float l2, const float (&acc2)[8]) {
  const float mn = fmaxf(m, m2);
  const float a = (m == -INFINITY) ? 0.f : fast_exp2(m - mn);
  const float b = (m2 == -INFINITY) ? 0.f : fast_exp2(m2 - mn);
  m = mn;
  l = l * a + l2 * b;
#pragma unroll
  for (int x = 0; x < 8; ++x) acc[x] = acc[x] * a + acc2[x] * b;
}

// One wave per (split, group of G query heads, batch).  The G heads share one K/V
// head (grouped heads: G divides the group size g), so the wave streams that head's
// cache rows once and keeps G online-softmax states; for each head the arithmetic
// is exactly that of a single-head wave.  Scores: q . k from packed 16-bit pairs
// (v_dot2, fp32 accumulation), summed over the row's lanes, then times scale*log2(e).
// V rows are widened to fp32 once and shared by the G heads.
template <int DT, int D, int G>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(G == 1 ? 4 : 2))) void decode_split_kernel(
    DecodeParams p) {
  using namespace decode_cfg;
  constexpr int CH = D / 8;                  // 16-byte chunks of a row
  constexpr int LPR = CH == 12 ? 16 : CH;    // lanes per cache row (a power of two)
  constexpr int RPW = 64 / LPR;              // rows per wave-wide load
  constexpr int RITER = RPW * kUnroll;

  const int s = blockIdx.x, b = blockIdx.z;
  const int h0 = blockIdx.y * G;  // first query head of this wave
  const int kvh = h0 / p.g;       // the K/V head all G of them read
  const int L = clamp_len(p.seq_lens[b], p.max_len);
  const int r0 = s * p.chunk;
  const int lane = threadIdx.x;
  const size_t pair0 = (size_t)b * p.H + h0;  // (b, h0) as a query-head pair index
  if (r0 >= L) {  // empty chunk: mark it so the merge needs no lengths
    if (lane < G) *(float2*)(p.ws_ml + ((pair0 + lane) * p.n_split + s) * 2) = make_float2(-INFINITY, 0.f);
    return;
  }
  const int r1 = min(L, r0 + p.chunk);

  const int seg = lane % LPR;   // which 8 elements of d
  const int rsub = lane / LPR;  // row within one wave-wide load
  const bool seg_ok = seg < CH; // lanes past the row's data (d = 96) load zeros and store nothing
  const size_t kvpair = (size_t)b * p.Hkv + kvh;
  const uint16_t* kg = p.k + kvpair * p.max_len * D + seg * 8;
  const uint16_t* vg = p.v + kvpair * p.max_len * D + seg * 8;

  u32x4 qp[G];  // this lane's 8 elements of each head's query row, packed as stored
#pragma unroll
  for (int j = 0; j < G; ++j) qp[j] = seg_ok ? *(const u32x4*)(p.q + (pair0 + j) * D + seg * 8) : (u32x4){0, 0, 0, 0};

  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.f;
#pragma unroll
    for (int x = 0; x < 8; ++x) acc[j][x] = 0.f;
  }

  // Rows of one iteration: base + u*RPW + rsub.  The loads of iteration i+1 are
  // issued before iteration i is reduced, so a wave keeps two iterations in flight.
  auto load = [&](int base, u32x4 (&kr)[kUnroll], u32x4 (&vr)[kUnroll]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int row = base + u * RPW + rsub;
      kr[u] = (u32x4){0, 0, 0, 0};
      vr[u] = (u32x4){0, 0, 0, 0};
      if (row < r1 && seg_ok) {
        kr[u] = *(const u32x4*)(kg + (size_t)row * D);
        vr[u] = *(const u32x4*)(vg + (size_t)row * D);
      }
    }
  };
  auto reduce = [&](int base, const u32x4 (&kr)[kUnroll], const u32x4 (&vr)[kUnroll]) __attribute__((always_inline)) {
    // V elements widened to fp32: once for all G heads, or at their single use (G = 1).
    auto vx = [&](int u, int x) __attribute__((always_inline)) {
      return to_f32<DT>((x & 1) ? (vr[u][x >> 1] >> 16) : (vr[u][x >> 1] & 0xffffu));
    };
    float vf[kUnroll][8];
    if constexpr (G > 1) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
#pragma unroll
        for (int x = 0; x < 8; ++x) vf[u][x] = vx(u, x);
    }
#pragma unroll
    for (int j = 0; j < G; ++j) {
      float sc[kUnroll];
      float mx = m[j];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        float part = 0.f;
#pragma unroll
        for (int x = 0; x < 4; ++x) part = dot2<DT>(qp[j][x], kr[u][x], part);
        // Sum the LPR lanes of this row (aligned groups of LPR consecutive lanes).
#pragma unroll
        for (int off = 1; off < LPR; off <<= 1) part += __shfl_xor(part, off);
        sc[u] = base + u * RPW + rsub < r1 ? part * p.c : -INFINITY;
        mx = fmaxf(mx, sc[u]);
      }
      if (mx != -INFINITY) {  // this row group has valid rows in this iteration
        const float alpha = fast_exp2(m[j] - mx);  // m = -inf gives 0
        m[j] = mx;
        l[j] *= alpha;
#pragma unroll
        for (int x = 0; x < 8; ++x) acc[j][x] *= alpha;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          const float pu = fast_exp2(sc[u] - m[j]);  // -inf gives 0
          l[j] += pu;
#pragma unroll
          for (int x = 0; x < 8; ++x) acc[j][x] = __builtin_fmaf(pu, G > 1 ? vf[u][x] : vx(u, x), acc[j][x]);
        }
      }
    }
  };
  u32x4 ka[kUnroll], va[kUnroll], kb[kUnroll], vb[kUnroll];
  load(r0, ka, va);
  for (int base = r0; base < r1; base += 2 * RITER) {
    if (base + RITER < r1) load(base + RITER, kb, vb);
    reduce(base, ka, va);
    if (base + RITER >= r1) break;
    if (base + 2 * RITER < r1) load(base + 2 * RITER, ka, va);
    reduce(base + RITER, kb, vb);
  }

  // Combine the RPW row groups of the wave (lanes rsub*LPR + seg) pairwise, per head.
#pragma unroll
  for (int j = 0; j < G; ++j) {
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
      float acc2[8];
#pragma unroll
      for (int x = 0; x < 8; ++x) acc2[x] = __shfl_xor(acc[j][x], off);
      const float m2 = __shfl_xor(m[j], off), l2 = __shfl_xor(l[j], off);
      combine(m[j], l[j], acc[j], m2, l2, acc2);
    }
  }
  if (rsub == 0 && seg_ok) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const size_t pidx = (pair0 + j) * p.n_split + s;
      float* out = p.ws_acc + pidx * D + seg * 8;
      *(f32x4*)out = (f32x4){acc[j][0], acc[j][1], acc[j][2], acc[j][3]};
      *(f32x4*)(out + 4) = (f32x4){acc[j][4], acc[j][5], acc[j][6], acc[j][7]};
      if (seg == 0) *(float2*)(p.ws_ml + pidx * 2) = make_float2(m[j], l[j]);
    }
  }
}

// Exact merge: O = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s over the non-empty
// splits (empty ones carry m = -inf); a length of 0 writes zeros.  Four groups of 64
// threads take every fourth split, eight splits per round, each round's loads issued
// together (one memory latency per round rather than per split).  The groups' sums
// meet in LDS in a fixed order, so the result is deterministic.
template <int DT, int D>
__global__ __launch_bounds__(decode_cfg::kMergeThreads) void decode_merge_kernel(DecodeParams p) {
  using namespace decode_cfg;
  constexpr int NG = kMergeThreads / 64;
  constexpr int DPT = (D + 63) / 64;  // d elements per thread (the last pass may be partial)
  constexpr int NBAT = 8;      // splits per group per round
  __shared__ float sm_M[NG];
  __shared__ float sm_den[NG];
  __shared__ float sm_num[NG][D];
  const int h = blockIdx.x, b = blockIdx.y;
  const int t = threadIdx.x, g = t >> 6, lane = t & 63;
  const size_t pair = (size_t)b * p.H + h;
  const int nv = p.n_split;  // empty chunks carry m = -inf and weigh nothing
  const float* ml = p.ws_ml + pair * p.n_split * 2;
  const float* ac = p.ws_acc + pair * p.n_split * D;
  // Running state of this group: max, denominator and numerator relative to it.
  float M = -INFINITY, den = 0.f, num[DPT];
#pragma unroll
  for (int x = 0; x < DPT; ++x) num[x] = 0.f;
  for (int s0 = g; s0 < nv; s0 += NG * NBAT) {
    float2 mlv[NBAT];
    float av[NBAT][DPT];
    // All of the round's loads go out together.  The acc of an empty chunk was never
    // written and may hold any bits: it is loaded but discarded by a select below.
#pragma unroll
    for (int i = 0; i < NBAT; ++i) {
      const int s = s0 + i * NG;
      mlv[i] = make_float2(-INFINITY, 0.f);
#pragma unroll
      for (int x = 0; x < DPT; ++x) av[i][x] = 0.f;
      if (s < nv) {
        mlv[i] = *(const float2*)(ml + 2 * s);
#pragma unroll
        for (int x = 0; x < DPT; ++x)
          if (x * 64 + lane < D) av[i][x] = ac[(size_t)s * D + x * 64 + lane];
      }
    }
    float Mb = M;
#pragma unroll
    for (int i = 0; i < NBAT; ++i) Mb = fmaxf(Mb, mlv[i].x);
    const float sc = (M == -INFINITY) ? 0.f : fast_exp2(M - Mb);
    den *= sc;
#pragma unroll
    for (int x = 0; x < DPT; ++x) num[x] *= sc;
#pragma unroll
    for (int i = 0; i < NBAT; ++i) {
      const bool live = mlv[i].x != -INFINITY;
      const float w = live ? fast_exp2(mlv[i].x - Mb) : 0.f;
      den = live ? __builtin_fmaf(w, mlv[i].y, den) : den;
#pragma unroll
      for (int x = 0; x < DPT; ++x) num[x] = live ? __builtin_fmaf(w, av[i][x], num[x]) : num[x];
    }
    M = Mb;
  }
  if (lane == 0) sm_M[g] = M;
  __syncthreads();
  float Mall = sm_M[0];
#pragma unroll
  for (int i = 1; i < NG; ++i) Mall = fmaxf(Mall, sm_M[i]);
  const float sc = (M == -INFINITY) ? 0.f : fast_exp2(M - Mall);
  if (lane == 0) sm_den[g] = den * sc;
#pragma unroll
  for (int x = 0; x < DPT; ++x)
    if (x * 64 + lane < D) sm_num[g][x * 64 + lane] = num[x] * sc;
  __syncthreads();
  if (g == 0) {
    float dn = 0.f;
#pragma unroll
    for (int i = 0; i < NG; ++i) dn += sm_den[i];
#pragma unroll
    for (int x = 0; x < DPT; ++x) {
      const int d = x * 64 + lane;
      float nm = 0.f;
#pragma unroll
      for (int i = 0; i < NG; ++i) nm += d < D ? sm_num[i][d] : 0.f;
      const float o = dn > 0.f ? nm / dn : 0.f;  // a length of 0 leaves every chunk empty
      // Pair up neighbouring lanes so each even lane stores one dword.
      const float o_next = __shfl_down(o, 1);
      if ((lane & 1) == 0 && d < D) *(uint32_t*)(p.o + pair * D + d) = pack2<DT>(o, o_next);
    }
  }
}

template <int DT, int D, int G>
static hipError_t launch_decode_t(const DecodeParams& p, hipStream_t st) {
  hipLaunchKernelGGL((decode_split_kernel<DT, D, G>), dim3(p.n_split, p.H / G, p.B), dim3(64), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<DT, D>), dim3(p.H, p.B), dim3(decode_cfg::kMergeThreads), 0, st, p);
  return hipGetLastError();
}

template <int DT, int D>
static hipError_t launch_decode_g(const DecodeParams& p, int G, hipStream_t st) {
  switch (G) {
    case 1: return launch_decode_t<DT, D, 1>(p, st);
    case 2: return launch_decode_t<DT, D, 2>(p, st);
    case 3: return launch_decode_t<DT, D, 3>(p, st);
    case 4: return launch_decode_t<DT, D, 4>(p, st);
    case 5: return launch_decode_t<DT, D, 5>(p, st);
    case 6: return launch_decode_t<DT, D, 6>(p, st);
    case 7: return launch_decode_t<DT, D, 7>(p, st);
    case 8: return launch_decode_t<DT, D, 8>(p, st);
    default: return hipErrorInvalidValue;
  }
}

int decode_heads_per_wave(int H, int Hkv) {
  const int g = H / Hkv;
  for (int G = 8; G > 1; --G)
    if (g % G == 0) return G;
  return 1;
}

hipError_t launch_decode(const void* q, const void* k, const void* v, const int32_t* seq_lens, void* o, int B, int H,
                         int Hkv, int max_len, int d, int dt, float scale, int chunk, int n_split, float* ws,
                         hipStream_t st) {
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
  p.Hkv = Hkv;
  p.g = H / Hkv;
  p.max_len = max_len;
  p.chunk = chunk;
  p.n_split = n_split;
  p.c = scale * kLog2e;
  const int G = decode_heads_per_wave(H, Hkv);
#define ATTN_DEC(D_)                                                          \
  if (dt == DT_F16 && d == D_) return launch_decode_g<DT_F16, D_>(p, G, st); \
  if (dt == DT_BF16 && d == D_) return launch_decode_g<DT_BF16, D_>(p, G, st);
  ATTN_DEC(64)
  ATTN_DEC(128)
  ATTN_DEC(32)
  ATTN_DEC(96)
  ATTN_DEC(256)
#undef ATTN_DEC
  return hipErrorInvalidValue;
}

}  // namespace attn
