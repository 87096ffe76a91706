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
#include <mutex>

#include "attn.h"
#include "attn_device.h"
#include "attn_launch.h"

namespace attn {

namespace decode_cfg {
constexpr int kUnroll = 4;          // row loads of K (and of V) per lane per buffer (two buffers)
constexpr int kMergeBatch = 8;      // splits per merge group per round of loads
constexpr int kMfmaMinGroup = 3;    // smallest group of query heads decoded on the matrix cores
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

// Split handled by this workgroup of an (n_split, ny, B) grid.  Workgroups are
// dealt to the 8 XCDs round-robin by linear id, so with a split count that is a
// multiple of 8 split s of every column would land on XCD s mod 8; the sequences'
// non-empty splits are prefixes, which would load the low XCDs more.  Skewing the
// split by the column index starts each column on another XCD.
__device__ __forceinline__ int skewed_split(int n_split, int ny) {
  return (int)(((unsigned)group_x() + group_y() + (unsigned)group_z() * ny) % (unsigned)n_split);
}

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

  const int b = group_z();
  const int s = skewed_split(p.n_split, p.H / G);
  const int h0 = group_y() * G;  // first query head of this wave
  const int kvh = h0 / p.g;       // the K/V head all G of them read
  const int L = clamp_len(p.seq_lens[b], p.max_len);
  const int r0 = s * p.chunk;
  const int lane = thread_x();
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
      if (row < r1 && seg_ok) {  // read once: non-temporal, so the stream does not displace other lines
        kr[u] = __builtin_nontemporal_load((const u32x4*)(kg + (size_t)row * D));
        vr[u] = __builtin_nontemporal_load((const u32x4*)(vg + (size_t)row * D));
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

// lds_dma16 with the non-temporal policy: cache rows are read once, so their lines
// need not stay in the caches.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16_nt(const u32x4& rsrc, uint32_t voff, uint32_t lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %0, 0 offen nt lds"
      :
      : "s"(rsrc), "v"(voff), "s"(lds_addr)
      : "memory", "m0");
}
#pragma clang diagnostic pop

// Grouped heads on the matrix cores.  One wave per (split, K/V head, batch) scores
// all g query heads of the group at once: they are the columns of one 32-wide MFMA
// tile (g <= 32; columns past g hold zeros), exactly as a block of query rows is in
// the prefill.  The chunk's K and V rows stream through LDS in 32-row tiles
// (LDS-direct loads, two stages, the prefill's swizzles):
//   S^T = K Q^T (one query head per lane column, 16 keys per lane),
//   per head: m, l and the rescale of O as in the online softmax,
//   O^T += V^T P^T with V^T from LDS transpose reads and P rounded to 16 bits.
// The partials (m, l, acc) have the split kernel's layout, per query head.  Per byte
// of cache read this takes a few VALU instructions however many heads the group has,
// where the VALU form spends them once per head.
template <int DT, int D>
__global__ __launch_bounds__(64) void decode_split_mfma_kernel(DecodeParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int RBG = 2 * D;                 // bytes per cache row in memory
  constexpr int RB = lds_row_bytes<D>();     // bytes per row in LDS
  constexpr int CH = D / 8;                  // 16-byte chunks of a row that hold data
  constexpr bool W256 = RB % 256 == 0;
  constexpr int KS = D / 16, DB = D / 32;
  constexpr int UK = 32;                     // keys per tile (one MFMA block)
  constexpr int TILE = UK * RB;
  constexpr int NLD = TILE / 1024;           // 1 KiB LDS-direct loads per tile and operand
  __shared__ __attribute__((aligned(1024))) char kbuf0[TILE];
  __shared__ __attribute__((aligned(1024))) char kbuf1[TILE];
  __shared__ __attribute__((aligned(1024))) char vbuf0[TILE];
  __shared__ __attribute__((aligned(1024))) char vbuf1[TILE];

  const int kvh = group_y(), b = group_z();
  const int s = skewed_split(p.n_split, p.Hkv);
  const int lane = thread_x(), l32 = lane & 31, half = lane >> 5;
  const int g = p.g;
  // Uniform values the buffer descriptors are built from are pinned to SGPRs.
  const int L = __builtin_amdgcn_readfirstlane(clamp_len(p.seq_lens[b], p.max_len));
  const int r0 = s * p.chunk;
  const size_t pair0 = (size_t)b * p.H + (size_t)kvh * g;  // the group's first query head
  if (r0 >= L) {  // empty chunk: mark it so the merge needs no lengths
    if (lane < g) *(float2*)(p.ws_ml + ((pair0 + lane) * p.n_split + s) * 2) = make_float2(-INFINITY, 0.f);
    return;
  }
  const int r1 = min(L, r0 + p.chunk);
  const int nu = (r1 - r0 + UK - 1) / UK;
  const size_t kvpair = (size_t)b * p.Hkv + kvh;
  const char* kbase = (const char*)(p.k + kvpair * p.max_len * D);
  const char* vbase = (const char*)(p.v + kvpair * p.max_len * D);
  const bool col_ok = l32 < g;

  // Q^T as the B operand: lane holds q[head l32][16ks + 8half + 0..7].
  u32x4 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    qf[ks] = col_ok ? *(const u32x4*)(p.q + (pair0 + l32) * D + 16 * ks + 8 * half) : (u32x4){0, 0, 0, 0};

  auto kkey = [](int row) __attribute__((always_inline)) { return W256 ? (row & 15) : ((row >> 1) & 7); };
  auto vkey = [](int row) __attribute__((always_inline)) { return W256 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2); };
  auto src_chunk = [](int c) __attribute__((always_inline)) { return c >= CH ? c - CH : c; };
  uint32_t ldk_off[NLD], ldv_off[NLD];
#pragma unroll
  for (int r = 0; r < NLD; ++r) {
    const int ci = r * 64 + lane;
    const int row = ci / (RB / 16), sl = ci % (RB / 16);
    ldk_off[r] = row * RBG + (src_chunk(sl ^ kkey(row)) << 4);
    ldv_off[r] = row * RBG + (src_chunk(sl ^ vkey(row)) << 4);
  }
  uint32_t k_off[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) k_off[ks] = l32 * RB + (((2 * ks + half) ^ kkey(l32)) << 4);
  uint32_t v_off[DB];
  {
    const int r = lane & 15, gg = (lane >> 4) & 1;
    const int rowlo = 4 * half + (r >> 2);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int chunk = 4 * db + 2 * gg + ((r & 3) >> 1);
      v_off[db] = rowlo * RB + ((chunk ^ vkey(rowlo)) << 4) + 8 * (r & 1);
    }
  }

  if ((r1 - r0) % UK != 0) {
    // The last tile is partial and its missing rows are never written: start from
    // zeros so no uninitialised LDS bits reach the MFMA (masked p is exactly 0).
    for (int i = lane; i < TILE / 16; i += 64) {
      ((u32x4*)kbuf0)[i] = (u32x4){0, 0, 0, 0};
      ((u32x4*)kbuf1)[i] = (u32x4){0, 0, 0, 0};
      ((u32x4*)vbuf0)[i] = (u32x4){0, 0, 0, 0};
      ((u32x4*)vbuf1)[i] = (u32x4){0, 0, 0, 0};
    }
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  }

  auto load_tile = [&](int u, char* kb, char* vb) __attribute__((always_inline)) {
    const int row0 = r0 + u * UK;
    const int left = r1 - row0;
    const uint32_t nrec = (uint32_t)(left < UK ? left : UK) * RBG;
    u32x4 rk = buffer_rsrc(kbase + (size_t)row0 * RBG, nrec);
    u32x4 rv = buffer_rsrc(vbase + (size_t)row0 * RBG, nrec);
#pragma unroll
    for (int w = 0; w < 4; ++w) {  // uniform: keep the descriptors in SGPRs
      rk[w] = __builtin_amdgcn_readfirstlane(rk[w]);
      rv[w] = __builtin_amdgcn_readfirstlane(rv[w]);
    }
    const uint32_t lk = __builtin_amdgcn_readfirstlane(lds_addr_of(kb));
    const uint32_t lv = __builtin_amdgcn_readfirstlane(lds_addr_of(vb));
#pragma unroll
    for (int i = 0; i < NLD; ++i) lds_dma16_nt(rk, ldk_off[i], lk + i * 1024);
#pragma unroll
    for (int i = 0; i < NLD; ++i) lds_dma16_nt(rv, ldv_off[i], lv + i * 1024);
  };

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = (f32x16){};
  float m_run = -INFINITY, l_run = 0.f;

  // Unit u from the tile in (kb, vb); `next` says whether the following tile's loads
  // were issued after this one's (then they may stay in flight).
  auto unit = [&](int u, const char* kb, const char* vb, bool next) __attribute__((always_inline)) {
    if (next) __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * NLD));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    f32x16 st = {};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) st = mfma32x32x16<DT>(lds_read_b128((const uint16_t*)kb, k_off[ks]), qf[ks], st);
    const int key0 = r0 + u * UK + 4 * half;
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = key0 + 8 * (i >> 2) + (i & 3);
      st[i] = key < r1 ? st[i] * p.c : -INFINITY;
      mx = fmaxf(mx, st[i]);
    }
    // Key r0 + 32u is in range, so every column's max is finite.
    const float m_new = fmaxf(m_run, xhalf_max(mx));
    const float alpha = fast_exp2(m_run - m_new);  // m_run = -inf gives 0
    m_run = m_new;
    u32x4 pf[2];
    float lu = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const uint32_t t = pack2<DT>(fast_exp2(st[2 * w] - m_new), fast_exp2(st[2 * w + 1] - m_new));
      pf[w >> 2][w & 3] = t;
      lu = add_pair<DT>(t, lu);  // l sums the rounded weights that enter the MFMA
    }
    l_run = l_run * alpha + lu;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
#pragma unroll
    for (int si = 0; si < 2; ++si)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint32_t off = v_off[db] + 16 * si * RB;
        const u32x2 lo = lds_read_tr((const uint16_t*)vb, off);
        const u32x2 hi = lds_read_tr((const uint16_t*)vb, off + 8 * RB);
        oacc[db] = mfma32x32x16<DT>((u32x4){lo[0], lo[1], hi[0], hi[1]}, pf[si], oacc[db]);
      }
    // Every read of this tile has returned before the buffers take another tile.
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  };

  load_tile(0, kbuf0, vbuf0);
  if (nu > 1) load_tile(1, kbuf1, vbuf1);
  for (int u = 0; u < nu; u += 2) {
    unit(u, kbuf0, vbuf0, u + 1 < nu);
    if (u + 2 < nu) load_tile(u + 2, kbuf0, vbuf0);
    if (u + 1 < nu) {
      unit(u + 1, kbuf1, vbuf1, u + 2 < nu);
      if (u + 3 < nu) load_tile(u + 3, kbuf1, vbuf1);
    }
  }

  // Column l32 is query head pair0 + l32; its keys are split over the two lane
  // halves, its d rows too: acc row 32db + 8(i/4) + 4half + i%4.
  const float l_tot = xhalf_sum(l_run);
  if (col_ok) {
    const size_t pidx = (pair0 + l32) * p.n_split + s;
    float* out = p.ws_acc + pidx * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a)
        *(f32x4*)(out + 32 * db + 8 * a + 4 * half) =
            (f32x4){oacc[db][4 * a], oacc[db][4 * a + 1], oacc[db][4 * a + 2], oacc[db][4 * a + 3]};
    if (half == 0) *(float2*)(p.ws_ml + pidx * 2) = make_float2(m_run, l_tot);
  }
#endif
}

// Exact merge: O = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s over the non-empty
// splits (empty ones carry m = -inf); a length of 0 writes zeros.  NG groups of 64
// threads take every NG-th split, eight splits per round, each round's loads issued
// together (one memory latency per round rather than per split): four groups cover up
// to 32 splits in one round, eight groups up to 64.  The groups' sums meet in LDS in a
// fixed order, so the result is deterministic.
template <int DT, int D, int NG>
__global__ __launch_bounds__(64 * NG) void decode_merge_kernel(DecodeParams p) {
  using namespace decode_cfg;
  constexpr int DPT = (D + 63) / 64;  // d elements per thread (the last pass may be partial)
  constexpr int NBAT = kMergeBatch;   // splits per group per round
  __shared__ float sm_M[NG];
  __shared__ float sm_den[NG];
  __shared__ float sm_num[NG][D];
  const int h = group_x(), b = group_y();
  const int t = thread_x(), g = t >> 6, lane = t & 63;
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

// The merge: eight groups of 64 threads when the splits exceed what four groups load in
// one round (32), four otherwise.  Measured at B = 1 (64 splits): 12.4 -> 12.0 us for
// the call; at 22 splits four groups and eight measure the same.
template <int DT, int D>
static hipError_t launch_merge(const DecodeParams& p, hipStream_t st) {
  if (p.n_split > 4 * decode_cfg::kMergeBatch)
    hipLaunchKernelGGL((decode_merge_kernel<DT, D, 8>), dim3(p.H, p.B), dim3(512), 0, st, p);
  else
    hipLaunchKernelGGL((decode_merge_kernel<DT, D, 4>), dim3(p.H, p.B), dim3(256), 0, st, p);
  return hipGetLastError();
}

// `passes`: kDecodeSplitPass and/or kDecodeMergePass.
template <int DT, int D, int G>
static hipError_t launch_decode_t(const DecodeParams& p, int passes, hipStream_t st) {
  if (passes & kDecodeSplitPass) {
    hipLaunchKernelGGL((decode_split_kernel<DT, D, G>), dim3(p.n_split, p.H / G, p.B), dim3(64), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return (passes & kDecodeMergePass) ? launch_merge<DT, D>(p, st) : hipSuccess;
}

bool decode_uses_mfma(int H, int Hkv);

template <int DT, int D>
static hipError_t launch_decode_mfma(const DecodeParams& p, int passes, hipStream_t st) {
  if (passes & kDecodeSplitPass) {
    hipLaunchKernelGGL((decode_split_mfma_kernel<DT, D>), dim3(p.n_split, p.Hkv, p.B), dim3(64), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return (passes & kDecodeMergePass) ? launch_merge<DT, D>(p, st) : hipSuccess;
}

template <int DT, int D>
static hipError_t launch_decode_g(const DecodeParams& p, int G, int passes, hipStream_t st) {
  if (decode_uses_mfma(p.H, p.Hkv)) return launch_decode_mfma<DT, D>(p, passes, st);
  switch (G) {
    case 1: return launch_decode_t<DT, D, 1>(p, passes, st);
    case 2: return launch_decode_t<DT, D, 2>(p, passes, st);
    case 3: return launch_decode_t<DT, D, 3>(p, passes, st);
    case 4: return launch_decode_t<DT, D, 4>(p, passes, st);
    case 5: return launch_decode_t<DT, D, 5>(p, passes, st);
    case 6: return launch_decode_t<DT, D, 6>(p, passes, st);
    case 7: return launch_decode_t<DT, D, 7>(p, passes, st);
    case 8: return launch_decode_t<DT, D, 8>(p, passes, st);
    default: return hipErrorInvalidValue;
  }
}

bool decode_uses_mfma(int H, int Hkv) {
  // Groups of 3..32 query heads: one matrix-core wave serves the whole group (pairs
  // of heads measured faster on the vector ALUs).
  const int g = H / Hkv;
  return g >= decode_cfg::kMfmaMinGroup && g <= 32;
}

// Resident waves per CU of the matrix-core split kernel: its two K and two V tiles of
// 32 rows take the CU's LDS first (registers allow at least as many).
int decode_mfma_waves_per_cu(int d) {
  const int pitch = d == 32 ? 128 : d == 96 ? 256 : 2 * d;
  return ATTN_DECODE_MFMA_LDS_BYTES / (4 * 32 * pitch);
}

int decode_heads_per_wave(int H, int Hkv) {
  const int g = H / Hkv;
  if (decode_uses_mfma(H, Hkv)) return g;
  for (int G = 8; G > 1; --G)
    if (g % G == 0) return G;
  return 1;
}

hipError_t launch_decode(const void* q, const void* k, const void* v, const int32_t* seq_lens, void* o, int B, int H,
                         int Hkv, int max_len, int d, int dt, float scale, int chunk, int n_split, float* ws,
                         hipStream_t st, int passes) {
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
  if (dt == DT_F16 && d == D_) return launch_decode_g<DT_F16, D_>(p, G, passes, st); \
  if (dt == DT_BF16 && d == D_) return launch_decode_g<DT_BF16, D_>(p, G, passes, st);
  ATTN_DEC(64)
  ATTN_DEC(128)
  ATTN_DEC(32)
  ATTN_DEC(96)
  ATTN_DEC(256)
#undef ATTN_DEC
  return hipErrorInvalidValue;
}

// Partials of the allocation-free decode entry point: a fixed device array that the
// code object carries, so a call needs no allocation.  Each device that loads the
// library holds its own copy until the process ends.  Host code must never pass the
// array's name to a kernel (on the host it is a stand-in, not a device address): the
// device address comes from hipGetSymbolAddress, looked up once per device below.
static __device__ __align__(256) char scratch[ATTN_DECODE_SCRATCH_BYTES];

hipError_t decode_scratch(float** ptr) {
  static std::mutex mu;
  static void* addr[64] = {nullptr};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));  // with `dev` current
    if (e != hipSuccess) return e;
    if (!a) return hipErrorInvalidSymbol;
    addr[dev] = a;
  }
  *ptr = (float*)addr[dev];
  return hipSuccess;
}

}  // namespace attn
