// Backward pass of exact attention for gfx950 (CDNA4): dQ, dK, dV of the loss
// sum(dO * O) for O = softmax(scale Q K^T [causal]) V, the step page 3 lists as
// future work ("Future work").  The softmax is not stored: every kernel recomputes
// P = exp(scale q.k - lse) from the row log-sum-exp the forward wrote
// (attn_prefill_ex), so P is the forward's exact normalised probability.
//
//   delta_i = sum_d dO_id O_id                     (pre-pass, one value per row,
//                                                   beside lse_i log2(e))
//   dS      = P * (dO V^T - delta)                 (elementwise, rows x keys)
//   dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO
//
// Two matrix-core kernels, no atomics, every output written once:
//   * dQ: a workgroup owns a block of query rows and streams K/V tiles (the forward's
//     layout: S^T = K Q^T puts one query row per lane column); dP^T = V dO^T, and
//     dQ^T += K^T dS^T reads K^T with LDS transpose loads.
//   * dK, dV: a workgroup owns a block of keys and streams Q/dO tiles with S = Q K^T,
//     so one key per lane column; dV^T += dO^T P and dK^T += Q^T dS read dO^T and
//     Q^T with transpose loads.  With grouped heads it loops over the group's query
//     heads, so a K/V head's gradient sums theirs.
// Tiles staged through LDS are read both as row operands (ds_read_b128) and through
// transpose loads, so their 16-byte chunks carry a key that is conflict-free for both
// (verified with the LDS bank-conflict counter): rows of 256 bytes (d = 128, and
// d = 96 padded): ((r&3)<<2) | ((r>>2)&3); rows of 128 bytes (d = 64, and d = 32
// padded): (((r>>1)&1)<<2) | ((r>>2)&3).  Tiles read only as row operands keep the
// forward's K key.  P and dS enter the matrix cores rounded to the input type (RNE),
// as P does in the forward.
#include <type_traits>

#include "attn_device.h"
#include "attn_launch.h"

namespace attn {

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;  // [B][H][N] natural log
  float* delta;      // [B][H][N] rowsum(dO * O), written by the pre-pass
  float* lse2;       // [B][H][N] lse * log2(e), written by the pre-pass
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  int B, H, Hkv, g, N;
  int nblk;     // blocks per head along the kernel's own dimension
  float c;      // scale * log2(e), signed
  float scale;  // the softmax scale
};

namespace bwd_cfg {
constexpr int BN = 64;  // rows of a streamed tile (keys for dQ, query rows for dK/dV)
constexpr int NW = 4;   // waves per dK/dV workgroup, 32 keys each
}  // namespace bwd_cfg

// Chunk keys of a tile row r (16-byte chunks XOR key), by LDS row pitch: rows of a
// multiple of 256 bytes (d = 96, 128, 256; the bank pattern repeats every 256 bytes, and
// keys below 16 keep a chunk within its 256-byte half) or of 128 bytes (d = 32, 64;
// lds_row_bytes pads 32 and 96).
template <int D>
__device__ __forceinline__ int dual_key(int r) {
  return lds_row_bytes<D>() % 256 == 0 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}
template <int D>
__device__ __forceinline__ int row_key(int r) {
  return lds_row_bytes<D>() % 256 == 0 ? (r & 15) : ((r >> 1) & 7);
}

// Row operand read (A operand of a 32x32x16 MFMA): lane l gets 16 bytes of tile row
// (32h + l%32), logical chunk 2ks + l/32.
template <int D, bool DUAL>
__device__ __forceinline__ u32x4 row_read(const char* buf, int h, int ks, int lane) {
  constexpr int RB = lds_row_bytes<D>();
  const int row = 32 * h + (lane & 31);
  const int key = DUAL ? dual_key<D>(row & 15) : row_key<D>(row & 15);
  return lds_read_b128((const uint16_t*)buf, row * RB + (((2 * ks + (lane >> 5)) ^ key) << 4));
}

// Transposed operand (A operand of (d x rows) = X^T P): for the unit in half h of
// the tile, 16 rows starting at 32h + 16s, d block db; lane l gets d = 32db + l%32
// at four rows from each of two transpose loads, in the order the packed P / dS
// operand (from a 32x32 accumulator) lists its rows.
template <int D>
__device__ __forceinline__ u32x4 tr_read(const char* buf, int h, int s, int db, int lane) {
  constexpr int RB = lds_row_bytes<D>();
  const int r = lane & 15, gg = (lane >> 4) & 1, half = lane >> 5;
  const int rowlo = 4 * half + (r >> 2);
  const int chunk = 4 * db + 2 * gg + ((r & 3) >> 1);
  const int row = 32 * h + 16 * s + rowlo;  // row & 15 == rowlo; the second load reads rows + 8
  const uint32_t off_lo = row * RB + ((chunk ^ dual_key<D>(rowlo)) << 4) + 8 * (r & 1);
  const uint32_t off_hi = (row + 8) * RB + ((chunk ^ dual_key<D>(rowlo + 8)) << 4) + 8 * (r & 1);
  const u32x2 lo = lds_read_tr((const uint16_t*)buf, off_lo);
  const u32x2 hi = lds_read_tr((const uint16_t*)buf, off_hi);
  return (u32x4){lo[0], lo[1], hi[0], hi[1]};
}

// The same reads from per-lane bases, for kernels short of registers.  The physical
// chunk (2ks + half) ^ key equals 2ks ^ (half ^ key), and a row's chunk field lies in
// bits below its row offset, so operand (h, ks) of row_read sits at
// (row_base ^ (ks << 5)) + 32h RB: one XOR per read from one register.  Likewise the
// transposed chunk (4db + c) ^ key equals 4db ^ (c ^ key), so tr_read's two loads sit
// at (tr_base ^ (db << 6)) + (32h + 16s) RB, from one base per load.
template <int D, bool DUAL>
__device__ __forceinline__ uint32_t row_base(int lane) {
  constexpr int RB = lds_row_bytes<D>();
  const int row = lane & 31;
  const int key = DUAL ? dual_key<D>(row & 15) : row_key<D>(row & 15);
  return (uint32_t)(row * RB + (((lane >> 5) ^ key) << 4));
}
template <int D>
__device__ __forceinline__ u32x4 row_read_at(const char* buf, uint32_t base, int h, int ks) {
  constexpr int RB = lds_row_bytes<D>();
  return lds_read_b128((const uint16_t*)buf, (base ^ (uint32_t)(ks << 5)) + 32 * h * RB);
}
template <int D>
__device__ __forceinline__ uint32_t tr_base(int lane, int hi) {
  constexpr int RB = lds_row_bytes<D>();
  const int r = lane & 15, gg = (lane >> 4) & 1, half = lane >> 5;
  const int rowlo = 4 * half + (r >> 2) + 8 * hi;
  const int c = 2 * gg + ((r & 3) >> 1);
  return (uint32_t)(rowlo * RB + ((c ^ dual_key<D>(rowlo)) << 4) + 8 * (r & 1));
}
template <int D>
__device__ __forceinline__ u32x4 tr_read_at(const char* buf, uint32_t lo_base, uint32_t hi_base, int h, int s,
                                            int db) {
  constexpr int RB = lds_row_bytes<D>();
  const uint32_t x = (uint32_t)(db << 6), o = (32 * h + 16 * s) * RB;
  const u32x2 lo = lds_read_tr((const uint16_t*)buf, (lo_base ^ x) + o);
  const u32x2 hi = lds_read_tr((const uint16_t*)buf, (hi_base ^ x) + o);
  return (u32x4){lo[0], lo[1], hi[0], hi[1]};
}

// Stage one BN-row tile of a [rows][D] tensor into LDS: this wave's share of 1 KiB
// LDS-direct loads; physical slot sl of row r receives logical chunk sl ^ key(r).
// Padded rows (d = 32, 96) have slots past the data, which take a copy of a chunk of
// the same row and are never read.
template <int D, bool DUAL, int NW = bwd_cfg::NW, int BN = bwd_cfg::BN>
__device__ __forceinline__ void stage_tile(const uint16_t* src, int row0, int rows_total, char* dst, int wave,
                                           int lane) {
  constexpr int RBG = 2 * D;                // bytes per row in memory
  constexpr int RB = lds_row_bytes<D>();    // bytes per row in LDS
  constexpr int CH = D / 8;
  constexpr int TILE = BN * RB;
  constexpr int NLD = TILE / 1024 / NW;
  static_assert(NLD >= 1, "tile too small for the load pattern");
  const int left = rows_total - row0;
  const uint32_t nrec = (uint32_t)(left < BN ? left : BN) * RBG;
  const u32x4 rs = buffer_rsrc((const char*)src + (size_t)row0 * RBG, nrec);
  const uint32_t l0 = __builtin_amdgcn_readfirstlane(lds_addr_of(dst) + wave * NLD * 1024);
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int ci = (wave * NLD + i) * 64 + lane;
    const int row = ci / (RB / 16), sl = ci % (RB / 16);
    const int key = DUAL ? dual_key<D>(row & 15) : row_key<D>(row & 15);
    const int c = sl ^ key;
    lds_dma16(rs, row * RBG + ((c >= CH ? c - CH : c) << 4), l0 + i * 1024);
  }
}

template <int DT>
__device__ __forceinline__ void pack_unit(const f32x16& x, u32x4 (&pf)[2]) {
#pragma unroll
  for (int w = 0; w < 8; ++w) pf[w >> 2][w & 3] = pack2<DT>(x[2 * w], x[2 * w + 1]);
}

// ---------------------------------------------------------------------------------
// delta = rowsum(dO * O), D/8 lanes per row; beside it lse * log2(e), the row's
// log-sum-exp in the base-2 domain the gradient kernels exponentiate in.
template <int DT, int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(BwdParams p) {
  constexpr int CH = D / 8;                  // 16-byte chunks of a row
  constexpr int LPR = CH == 12 ? 16 : CH;    // lanes per row (a power of two)
  constexpr int RPB = 256 / LPR;
  const long long total = (long long)p.B * p.H * p.N;
  const long long row = (long long)group_x() * RPB + thread_x() / LPR;
  const int seg = thread_x() % LPR;
  float acc = 0.f;
  if (row < total && seg < CH) {
    const u32x4 a = *(const u32x4*)(p.o + row * D + seg * 8);
    const u32x4 b = *(const u32x4*)(p.dout + row * D + seg * 8);
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      acc = __builtin_fmaf(to_f32<DT>(a[x] & 0xffffu), to_f32<DT>(b[x] & 0xffffu), acc);
      acc = __builtin_fmaf(to_f32<DT>(a[x] >> 16), to_f32<DT>(b[x] >> 16), acc);
    }
  }
#pragma unroll
  for (int off = 1; off < LPR; off <<= 1) acc += __shfl_xor(acc, off);
  if (row < total && seg == 0) {
    p.delta[row] = acc;
    p.lse2[row] = p.lse[row] * kLog2e;
  }
}

// ---------------------------------------------------------------------------------
// dQ: workgroup = 128 query rows of one (b, h); tiles of 64 keys.
// d = 256: Q, dO operands and the dQ accumulators alone take 256 registers, so one
// wave per SIMD.
template <int DT, int D, bool CAUSAL, int NW>
__global__ __launch_bounds__(64 * NW, D > 128 ? 1 : 8 / NW) void bwd_dq_kernel(BwdParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int BN = bwd_cfg::BN;
  constexpr int RB = lds_row_bytes<D>(), KS = D / 16, DB = D / 32, BM = 32 * NW;
  constexpr int TILE = BN * RB;
  __shared__ __attribute__((aligned(1024))) char kbuf0[TILE];
  __shared__ __attribute__((aligned(1024))) char kbuf1[TILE];
  __shared__ __attribute__((aligned(1024))) char vbuf0[TILE];
  __shared__ __attribute__((aligned(1024))) char vbuf1[TILE];

  const int tid = thread_x();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, half = lane >> 5;
  const int G = p.nblk * p.B * p.H, bid = group_x();  // the grid: query blocks x heads x batch
  const int xcd = bid & 7, slot = bid >> 3, per = G >> 3, rem = G & 7;
  const int work = xcd * per + min(xcd, rem) + slot;
  const int bh = __builtin_amdgcn_readfirstlane(work / p.nblk);
  int qb = __builtin_amdgcn_readfirstlane(work - bh * p.nblk);
  if (CAUSAL) qb = p.nblk - 1 - qb;
  const int kvbh = __builtin_amdgcn_readfirstlane(bh / p.g);
  const int N = p.N;
  const int q0 = qb * BM, qw0 = q0 + 32 * wave, qrow = qw0 + l32;
  const bool row_ok = qrow < N;
  const uint16_t* kg = p.k + (size_t)kvbh * N * D;
  const uint16_t* vg = p.v + (size_t)kvbh * N * D;

  u32x4 qf[KS], df[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qf[ks] = (u32x4){0, 0, 0, 0};
    df[ks] = (u32x4){0, 0, 0, 0};
    if (row_ok) {
      const size_t off = ((size_t)bh * N + qrow) * D + 16 * ks + 8 * half;
      qf[ks] = *(const u32x4*)(p.q + off);
      df[ks] = *(const u32x4*)(p.dout + off);
    }
  }
  const float lse2 = row_ok ? p.lse2[(size_t)bh * N + qrow] : 0.f;
  const float dl = row_ok ? p.delta[(size_t)bh * N + qrow] : 0.f;

  f32x16 dqa[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dqa[db] = (f32x16){};

  const int kv_end = CAUSAL ? min(N, q0 + BM) : N;
  const int nt = (kv_end + BN - 1) / BN;
  const int nu = (kv_end + 31) / 32;
  const int nu_w = qw0 >= N ? 0 : (CAUSAL ? min(nu, (qw0 + 31) / 32 + 1) : nu);

  if (N % BN != 0) {  // rows past N are never loaded: start from zeros
    for (int i = tid; i < TILE / 16; i += 64 * NW) {
      ((u32x4*)kbuf0)[i] = (u32x4){0, 0, 0, 0};
      ((u32x4*)kbuf1)[i] = (u32x4){0, 0, 0, 0};
      ((u32x4*)vbuf0)[i] = (u32x4){0, 0, 0, 0};
      ((u32x4*)vbuf1)[i] = (u32x4){0, 0, 0, 0};
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  stage_tile<D, true, NW>(kg, 0, N, kbuf0, wave, lane);
  stage_tile<D, false, NW>(vg, 0, N, vbuf0, wave, lane);
  if (nt > 1) {
    stage_tile<D, true, NW>(kg, BN, N, kbuf1, wave, lane);
    stage_tile<D, false, NW>(vg, BN, N, vbuf1, wave, lane);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // Keys visible to this lane's row: below N and (causal) at most the row.
  const int key_end = CAUSAL ? min(N, qrow + 1) : N;
  const uint32_t kbase = row_base<D, true>(lane), vbase = row_base<D, false>(lane);
  const uint32_t tlo = tr_base<D>(lane, 0), thi = tr_base<D>(lane, 1);
  auto unit = [&](int u, const char* kb, const char* vb, int h) __attribute__((always_inline)) {
    f32x16 st = {}, dpt = {};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      st = mfma32x32x16<DT>(row_read_at<D>(kb, kbase, h, ks), qf[ks], st);
      dpt = mfma32x32x16<DT>(row_read_at<D>(vb, vbase, h, ks), df[ks], dpt);
    }
    f32x16 ds;
    // Entry i holds key 32u + 4half + 8(i/4) + i%4: visible iff its offset 8(i/4) + i%4
    // (a constant) is below lim.
#pragma unroll
    for (int i = 0; i < 16; ++i) ds[i] = fast_exp2(__builtin_fmaf(st[i], p.c, -lse2)) * (dpt[i] - dl);
    // Only the sequence's last unit and (causal) the wave's diagonal unit hold entries a
    // row cannot see: there, those entries are replaced by 0 (a select, so whatever the
    // arithmetic gave them is dropped); every other unit skips the per-entry test.
    const bool need = (32 * u + 32 > N) || (CAUSAL && 32 * u + 31 > qw0);
    if (__builtin_expect(need, 0)) {
      const int lim = key_end - 32 * u - 4 * half;
#pragma unroll
      for (int i = 0; i < 16; ++i) ds[i] = 8 * (i >> 2) + (i & 3) < lim ? ds[i] : 0.f;
    }
    u32x4 dsf[2];
    pack_unit<DT>(ds, dsf);
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int db = 0; db < DB; ++db) dqa[db] = mfma32x32x16<DT>(tr_read_at<D>(kb, tlo, thi, h, s, db), dsf[s], dqa[db]);
  };

  // Tile t from (kb, vb); the loop is unrolled over the two buffer pairs so that every
  // LDS read addresses a compile-time buffer (its base folds into the offset).
  auto tile = [&](int t, char* kb, char* vb) __attribute__((always_inline)) {
    if (2 * t < nu_w) unit(2 * t, kb, vb, 0);
    if (2 * t + 1 < nu_w) unit(2 * t + 1, kb, vb, 1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t + 2 < nt) {
      stage_tile<D, true, NW>(kg, (t + 2) * BN, N, kb, wave, lane);
      stage_tile<D, false, NW>(vg, (t + 2) * BN, N, vb, wave, lane);
    }
  };
  for (int t = 0; t < nt; t += 2) {
    tile(t, kbuf0, vbuf0);
    if (t + 1 < nt) tile(t + 1, kbuf1, vbuf1);
  }

  if (row_ok) {
    uint16_t* og = p.dq + ((size_t)bh * N + qrow) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        u32x2 w;
        w[0] = pack2<DT>(dqa[db][4 * a + 0] * p.scale, dqa[db][4 * a + 1] * p.scale);
        w[1] = pack2<DT>(dqa[db][4 * a + 2] * p.scale, dqa[db][4 * a + 3] * p.scale);
        *(u32x2*)(og + 32 * db + 8 * a + 4 * half) = w;
      }
  }
#endif
}

// ---------------------------------------------------------------------------------
// dK, dV: workgroup = 128 keys of one (b, kv head); tiles of 64 query rows of each
// query head of the group, a unit being one 32-row half of a tile.  One wave per
// SIMD (the two gradient accumulators and the wave's K and V operands need about 300
// registers), so the wave overlaps its own work with a three-stage pipeline over
// units, as the forward does:
//   matrix cores: S_{v+2} = Q K^T and dP_{v+2} = dO V^T  interleaved with
//                 dV^T += dO_v^T P_v and dK^T += Q_v^T dS_v;
//   VALU:         P_{v+1} = 2^(c S - lse log2 e), dS_{v+1} = P (dP - delta), rounded.
// Unit v reads tile v/2, so each pipeline step reads two tiles: three LDS tile sets
// rotate, and the loads of a tile are issued two pipeline steps before it is read.
template <int DT, int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(BwdParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
  using namespace bwd_cfg;
  constexpr int RB = lds_row_bytes<D>(), KS = D / 16, DB = D / 32, BK = 32 * NW;
  constexpr int TILE = BN * RB;
  constexpr int NS = 3;       // tile sets in LDS
  constexpr int M = 2 * KS;   // issue slots per pipeline step: one S/dP and one dV/dK MFMA each
  constexpr int PF = 2;       // operand prefetch distance in slots
  constexpr int R = PF + 1;   // operand ring size
  __shared__ __attribute__((aligned(1024))) char qbuf[NS][TILE];
  __shared__ __attribute__((aligned(1024))) char dbuf[NS][TILE];
  __shared__ __attribute__((aligned(256))) float lsebuf[NS][BN];
  __shared__ __attribute__((aligned(256))) float dlbuf[NS][BN];

  const int tid = thread_x();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, half = lane >> 5;
  const int G = p.nblk * p.B * p.Hkv, bid = group_x();  // the grid: key blocks x K/V heads x batch
  const int xcd = bid & 7, slot = bid >> 3, per = G >> 3, rem = G & 7;
  const int work = xcd * per + min(xcd, rem) + slot;
  const int kvbh = __builtin_amdgcn_readfirstlane(work / p.nblk);
  const int kblk = __builtin_amdgcn_readfirstlane(work - kvbh * p.nblk);
  const int b = __builtin_amdgcn_readfirstlane(kvbh / p.Hkv);
  const int kvh = kvbh - b * p.Hkv;
  const int N = p.N;
  const int k0 = kblk * BK, kw0 = k0 + 32 * wave, key = kw0 + l32;
  const bool key_ok = key < N;

  u32x4 kf[KS], vf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    kf[ks] = (u32x4){0, 0, 0, 0};
    vf[ks] = (u32x4){0, 0, 0, 0};
    if (key_ok) {
      const size_t off = ((size_t)kvbh * N + key) * D + 16 * ks + 8 * half;
      kf[ks] = *(const u32x4*)(p.k + off);
      vf[ks] = *(const u32x4*)(p.v + off);
    }
  }
  f32x16 dka[DB], dva[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dka[db] = (f32x16){};
    dva[db] = (f32x16){};
  }

  // Query rows that see any of this block's keys: all of them, or (causal) rows from
  // the block's first key on, in whole 64-row tiles.
  const int r_start = CAUSAL ? (k0 / BN) * BN : 0;
  const int nt = k0 >= N ? 0 : (N - r_start + BN - 1) / BN;
  const int steps = p.g * nt;  // tiles, over the group's query heads in turn

  if (N % BN != 0) {  // rows past N are never loaded: every set starts from zeros
    for (int i = tid; i < NS * TILE / 16; i += 64 * NW) {
      ((u32x4*)&qbuf[0][0])[i] = (u32x4){0, 0, 0, 0};
      ((u32x4*)&dbuf[0][0])[i] = (u32x4){0, 0, 0, 0};
    }
    for (int i = tid; i < NS * BN; i += 64 * NW) {
      (&lsebuf[0][0])[i] = 0.f;
      (&dlbuf[0][0])[i] = 0.f;
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // Tile n of the flattened (query head, row tile) order into set n % NS.
  auto stage = [&](int n) __attribute__((always_inline)) {
    const int jh = n / nt, j = n - jh * nt, set = n % NS;
    const int bh = b * p.H + kvh * p.g + jh;
    const int row0 = r_start + j * BN;
    stage_tile<D, true>(p.q + (size_t)bh * N * D, row0, N, qbuf[set], wave, lane);
    stage_tile<D, true>(p.dout + (size_t)bh * N * D, row0, N, dbuf[set], wave, lane);
    if (wave == 0) {
      const int left = N - row0;
      // Rows past N take lse = +inf, so their P (and dS) is exactly 0 without a test;
      // the loads below write only rows < left.
      if (lane >= left) lsebuf[set][lane] = INFINITY;
      const uint32_t nrec = (uint32_t)(left < BN ? left : BN) * 4;
      const u32x4 rl = buffer_rsrc(p.lse2 + (size_t)bh * N + row0, nrec);
      const u32x4 rd = buffer_rsrc(p.delta + (size_t)bh * N + row0, nrec);
      lds_dma4(rl, 4 * lane, __builtin_amdgcn_readfirstlane(lds_addr_of(&lsebuf[set][0])));
      lds_dma4(rd, 4 * lane, __builtin_amdgcn_readfirstlane(lds_addr_of(&dlbuf[set][0])));
    }
  };
  auto row0_of = [&](int n) __attribute__((always_inline)) { return r_start + (n % nt) * BN; };

  // Softmax gradient of one unit, element by element.  Accumulator entry i of lane l
  // is (row 8(i/4) + 4(l/32) + i%4 of the unit, key l%32).  Rows past N carry lse =
  // +inf (see stage), and under the causal mask rows before the key get x = -inf, so
  // P = 0 and dS = 0 exactly.
  struct GradIn {
    const float* lse;
    const float* dl;
    int lo;  // causal: entries whose row offset 8(i/4) + i%4 is below lo precede the key
  };
  auto grad_in = [&](int n, int hb) __attribute__((always_inline)) {
    const int set = n % NS;
    GradIn g;
    g.lse = &lsebuf[set][32 * hb];
    g.dl = &dlbuf[set][32 * hb];
    g.lo = key - (row0_of(n) + 32 * hb + 4 * half);
    return g;
  };
  auto grad_rows = [&](const GradIn& g, int a, f32x4& l4, f32x4& d4) __attribute__((always_inline)) {
    l4 = *(const f32x4*)(g.lse + 8 * a + 4 * half);
    d4 = *(const f32x4*)(g.dl + 8 * a + 4 * half);
  };
  auto grad_elem = [&](const GradIn& g, const f32x16& s, const f32x16& dp, const f32x4& l4, const f32x4& d4,
                       int i, float& pm, float& ds) __attribute__((always_inline)) {
    const int e = i & 3;
    float x = __builtin_fmaf(s[i], p.c, -l4[e]);
    if (CAUSAL) x = 8 * (i >> 2) + e >= g.lo ? x : -INFINITY;
    pm = fast_exp2(x);
    ds = pm * (dp[i] - d4[e]);
  };
  // The whole unit at once (the pipeline prologue).
  auto grad_unit = [&](const GradIn& g, const f32x16& s, const f32x16& dp, u32x4 (&pf)[2], u32x4 (&dsf)[2])
      __attribute__((always_inline)) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      f32x4 l4, d4;
      grad_rows(g, a, l4, d4);
#pragma unroll
      for (int e = 0; e < 4; e += 2) {
        float p0, d0, p1, d1;
        grad_elem(g, s, dp, l4, d4, 4 * a + e, p0, d0);
        grad_elem(g, s, dp, l4, d4, 4 * a + e + 1, p1, d1);
        const int w = 2 * a + e / 2;
        pf[w >> 2][w & 3] = pack2<DT>(p0, p1);
        dsf[w >> 2][w & 3] = pack2<DT>(d0, d1);
      }
    }
  };

  // Operands: S/dP MFMA i reads row operand i (Q for even i, dO for odd, chunk i/2);
  // dV/dK MFMA i reads transposed operand i (dO for even i, Q for odd; si = i/(2DB),
  // db = (i/2) % DB).  Both are read PF slots ahead into rings that span the two
  // pipeline steps of a tile (operand j of step h sits at (hM + j) mod R).
  auto a_read = [&](const char* qb, const char* dbb, int h, int i) __attribute__((always_inline)) {
    return row_read<D, true>((i & 1) ? dbb : qb, h, i >> 1, lane);
  };
  auto c_read = [&](const char* qb, const char* dbb, int h, int i) __attribute__((always_inline)) {
    return tr_read<D>((i & 1) ? qb : dbb, h, (i >> 1) / DB, (i >> 1) % DB, lane);
  };

  f32x16 sacc[2], dpacc[2];  // S, dP of the units in flight (by unit parity)
  u32x4 pk[2][2], dsk[2][2]; // packed P, dS of the units in flight (by unit parity)

  // One pipeline step (unit v = 2n + h of tile n, tile n in set SC): A = S/dP of unit
  // v + 2 (tile n + 1, half h), B = P/dS of unit v + 1 (tile n + h, half 1 - h), C =
  // dV/dK of unit v (tile n, half h).  The set indices are compile-time so that every
  // LDS read folds its set into the instruction's offset.  In the last tile, A and B
  // work on a set that holds no tile of this workgroup's range: their results are
  // never consumed.
  auto step = [&](auto h_c, auto sc_c, int n, u32x4 (&ar)[R], u32x4 (&cr)[R]) __attribute__((always_inline)) {
    constexpr int h = decltype(h_c)::value;
    constexpr int SC = decltype(sc_c)::value, SA = (SC + 1) % NS, SB = h == 0 ? SC : SA;
    const char* qc = qbuf[SC];
    const char* dc = dbuf[SC];
    const char* qa = qbuf[SA];
    const char* da = dbuf[SA];
    GradIn gi;
    gi.lse = &lsebuf[SB][32 * (1 - h)];
    gi.dl = &dlbuf[SB][32 * (1 - h)];
    gi.lo = key - (row0_of(n + h) + 32 * (1 - h) + 4 * half);
    f32x16& sn = sacc[h];
    f32x16& dpn = dpacc[h];
    const f32x16& sb = sacc[1 - h];
    const f32x16& dpb = dpacc[1 - h];
    f32x4 l4[2], d4[2];  // row groups a and a + 1 (by parity of a)
    grad_rows(gi, 0, l4[0], d4[0]);
    grad_rows(gi, 1, l4[1], d4[1]);
    float pp = 0.f, dpp = 0.f;  // the even element of a pair, waiting for its partner
    float pe = 0.f, de = 0.f;
#pragma unroll
    for (int i = 0; i < M; ++i) {
      const int j = h * M + i;
      if (i + PF < M) ar[(j + PF) % R] = a_read(qa, da, h, i + PF);
      else if (h == 0) ar[(j + PF) % R] = a_read(qa, da, 1, i + PF - M);
      const int ks = i >> 1;
      if (i & 1) dpn = mfma32x32x16<DT>(ar[j % R], vf[ks], ks == 0 ? (f32x16){} : dpn);
      else sn = mfma32x32x16<DT>(ar[j % R], kf[ks], ks == 0 ? (f32x16){} : sn);
      if (i + PF < M) cr[(j + PF) % R] = c_read(qc, dc, h, i + PF);
      else if (h == 0) cr[(j + PF) % R] = c_read(qc, dc, 1, i + PF - M);
      const int si = (i >> 1) / DB, db = (i >> 1) % DB;
      if (i & 1) dka[db] = mfma32x32x16<DT>(cr[j % R], dsk[h][si], dka[db]);
      else dva[db] = mfma32x32x16<DT>(cr[j % R], pk[h][si], dva[db]);
      // Slot i takes the unit's elements 16i/M .. 16(i+1)/M - 1 (one at d = 128).
#pragma unroll
      for (int e = 16 * i / M; e < 16 * (i + 1) / M; ++e) {
        grad_elem(gi, sb, dpb, l4[(e >> 2) & 1], d4[(e >> 2) & 1], e, pe, de);
        if (e & 1) {
          const int w = e >> 1;
          pk[1 - h][w >> 2][w & 3] = pack2<DT>(pp, pe);
          dsk[1 - h][w >> 2][w & 3] = pack2<DT>(dpp, de);
        } else {
          pp = pe;
          dpp = de;
        }
        if ((e & 3) == 3 && e < 8) grad_rows(gi, (e >> 2) + 2, l4[(e >> 2) & 1], d4[(e >> 2) & 1]);
      }
      // Anchor the slot's VALU results in the slot (IR-level code motion ignores
      // sched_barrier and would gather the softmax gradient after the MFMAs).
      asm volatile("" ::"v"(pp), "v"(dpp), "v"(pe), "v"(de));
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Tile n (in set SC): its two pipeline steps, then the barrier that frees set SC
  // for tile n + 3.
  auto tile = [&](auto sc_c, int n) __attribute__((always_inline)) {
    constexpr int SC = decltype(sc_c)::value, SA = (SC + 1) % NS;
    u32x4 ar[R], cr[R];
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      ar[i] = a_read(qbuf[SA], dbuf[SA], 0, i);
      cr[i] = c_read(qbuf[SC], dbuf[SC], 0, i);
    }
    step(std::integral_constant<int, 0>(), sc_c, n, ar, cr);
    step(std::integral_constant<int, 1>(), sc_c, n, ar, cr);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (n + 3 < steps) stage(n + 3);
  };

  if (steps > 0) {
    // Prologue: tiles 0 and 1 in; S/dP of units 0 and 1; P/dS of unit 0; tile 2 in flight.
    stage(0);
    if (steps > 1) stage(1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (steps > 2) stage(2);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      f32x16 s = {}, dp = {};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s = mfma32x32x16<DT>(row_read<D, true>(qbuf[0], hh, ks, lane), kf[ks], s);
        dp = mfma32x32x16<DT>(row_read<D, true>(dbuf[0], hh, ks, lane), vf[ks], dp);
      }
      sacc[hh] = s;
      dpacc[hh] = dp;
    }
    grad_unit(grad_in(0, 0), sacc[0], dpacc[0], pk[0], dsk[0]);
    for (int n = 0; n < steps; n += NS) {
      tile(std::integral_constant<int, 0>(), n);
      if (n + 1 < steps) tile(std::integral_constant<int, 1>(), n + 1);
      if (n + 2 < steps) tile(std::integral_constant<int, 2>(), n + 2);
    }
  }

  if (key_ok) {
    const size_t off = ((size_t)kvbh * N + key) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        u32x2 wk, wv;
        wk[0] = pack2<DT>(dka[db][4 * a + 0] * p.scale, dka[db][4 * a + 1] * p.scale);
        wk[1] = pack2<DT>(dka[db][4 * a + 2] * p.scale, dka[db][4 * a + 3] * p.scale);
        wv[0] = pack2<DT>(dva[db][4 * a + 0], dva[db][4 * a + 1]);
        wv[1] = pack2<DT>(dva[db][4 * a + 2], dva[db][4 * a + 3]);
        *(u32x2*)(p.dk + off + 32 * db + 8 * a + 4 * half) = wk;
        *(u32x2*)(p.dv + off + 32 * db + 8 * a + 4 * half) = wv;
      }
  }
#endif
}

// ---------------------------------------------------------------------------------
// dK, dV at d = 256.  The pipelined kernel above would need three sets of 32 KiB Q and
// dO tiles (192 KiB of LDS) and both full accumulators beside the K and V operands
// (over 512 registers).  Here a workgroup of four waves owns 128 keys of one (b, kv
// head), each wave 32 keys whose K and V rows it keeps as MFMA B operands, and streams
// 32-row Q and dO tiles (double-buffered, 64 KiB) of every query head of the group.
// The gradients are accumulated in two passes over the halves of d: each pass
// recomputes S = Q K^T and dP = dO V^T over the full d, forms P and dS as the pipelined
// kernel does, and adds dV^T += dO^T P and dK^T += Q^T dS for its 128 columns.
template <int DT, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_d256_kernel(BwdParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int D = 256, NW = 4, BT = 32;  // waves, rows per streamed tile
  constexpr int RB = lds_row_bytes<D>(), KS = D / 16, DBH = D / 64;  // d blocks per half
  constexpr int TILE = BT * RB;
  constexpr int BK = 32 * NW;
  __shared__ __attribute__((aligned(1024))) char qbuf[2][TILE];
  __shared__ __attribute__((aligned(1024))) char dbuf[2][TILE];
  __shared__ __attribute__((aligned(256))) float lsebuf[2][BT];
  __shared__ __attribute__((aligned(256))) float dlbuf[2][BT];

  const int tid = thread_x();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, half = lane >> 5;
  const int G = p.nblk * p.B * p.Hkv, bid = group_x();  // the grid: key blocks x K/V heads x batch
  const int xcd = bid & 7, slot = bid >> 3, per = G >> 3, rem = G & 7;
  const int work = xcd * per + min(xcd, rem) + slot;
  const int kvbh = __builtin_amdgcn_readfirstlane(work / p.nblk);
  const int kblk = __builtin_amdgcn_readfirstlane(work - kvbh * p.nblk);
  const int b = __builtin_amdgcn_readfirstlane(kvbh / p.Hkv);
  const int kvh = kvbh - b * p.Hkv;
  const int N = p.N;
  const int k0 = kblk * BK, kw0 = k0 + 32 * wave, key = kw0 + l32;
  const bool key_ok = key < N;

  u32x4 kf[KS], vf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    kf[ks] = (u32x4){0, 0, 0, 0};
    vf[ks] = (u32x4){0, 0, 0, 0};
    if (key_ok) {
      const size_t off = ((size_t)kvbh * N + key) * D + 16 * ks + 8 * half;
      kf[ks] = *(const u32x4*)(p.k + off);
      vf[ks] = *(const u32x4*)(p.v + off);
    }
  }

  // Query rows that see any of this block's keys: all of them, or (causal) rows from
  // the block's first key on, in whole 32-row tiles.
  const int r_start = CAUSAL ? (k0 / BT) * BT : 0;
  const int nt = k0 >= N ? 0 : (N - r_start + BT - 1) / BT;
  const int steps = p.g * nt;  // tiles, over the group's query heads in turn

  if (N % BT != 0) {  // rows past N are never loaded: both sets start from zeros
    for (int i = tid; i < 2 * TILE / 16; i += 64 * NW) {
      ((u32x4*)&qbuf[0][0])[i] = (u32x4){0, 0, 0, 0};
      ((u32x4*)&dbuf[0][0])[i] = (u32x4){0, 0, 0, 0};
    }
    for (int i = tid; i < 2 * BT; i += 64 * NW) {
      (&lsebuf[0][0])[i] = 0.f;
      (&dlbuf[0][0])[i] = 0.f;
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // Tile n of the flattened (query head, row tile) order into set n % 2.
  auto stage = [&](int n) __attribute__((always_inline)) {
    const int jh = n / nt, j = n - jh * nt, set = n & 1;
    const int bh = b * p.H + kvh * p.g + jh;
    const int row0 = r_start + j * BT;
    stage_tile<D, true, NW, BT>(p.q + (size_t)bh * N * D, row0, N, qbuf[set], wave, lane);
    stage_tile<D, true, NW, BT>(p.dout + (size_t)bh * N * D, row0, N, dbuf[set], wave, lane);
    if (wave == 0 && lane < BT) {
      const int left = N - row0;
      // Rows past N take lse = +inf, so their P (and dS) is exactly 0 without a test.
      if (lane >= left) lsebuf[set][lane] = INFINITY;
      const uint32_t nrec = (uint32_t)(left < BT ? left : BT) * 4;
      const u32x4 rl = buffer_rsrc(p.lse2 + (size_t)bh * N + row0, nrec);
      const u32x4 rd = buffer_rsrc(p.delta + (size_t)bh * N + row0, nrec);
      lds_dma4(rl, 4 * lane, __builtin_amdgcn_readfirstlane(lds_addr_of(&lsebuf[set][0])));
      lds_dma4(rd, 4 * lane, __builtin_amdgcn_readfirstlane(lds_addr_of(&dlbuf[set][0])));
    }
  };

  for (int pass = 0; pass < 2; ++pass) {
    f32x16 dka[DBH], dva[DBH];
#pragma unroll
    for (int db = 0; db < DBH; ++db) {
      dka[db] = (f32x16){};
      dva[db] = (f32x16){};
    }
    if (steps > 0) {
      stage(0);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
    for (int n = 0; n < steps; ++n) {
      const int set = n & 1;
      if (n + 1 < steps) stage(n + 1);  // into the other set, read two tiles ago
      const char* qb = qbuf[set];
      const char* dbb = dbuf[set];
      // S and dP of the tile: entry i of lane l is (row 8(i/4) + 4(l/32) + i%4, key l%32).
      f32x16 st = {}, dp = {};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        st = mfma32x32x16<DT>(row_read<D, true>(qb, 0, ks, lane), kf[ks], st);
        dp = mfma32x32x16<DT>(row_read<D, true>(dbb, 0, ks, lane), vf[ks], dp);
      }
      const int row0 = r_start + (n % nt) * BT;
      const int lo = key - (row0 + 4 * half);  // causal: entries with row offset below lo precede the key
      u32x4 pf[2], dsf[2];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const f32x4 l4 = *(const f32x4*)(&lsebuf[set][8 * a + 4 * half]);
        const f32x4 d4 = *(const f32x4*)(&dlbuf[set][8 * a + 4 * half]);
        float pv[4], dv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float x = __builtin_fmaf(st[4 * a + e], p.c, -l4[e]);
          if (CAUSAL) x = 8 * a + e >= lo ? x : -INFINITY;
          pv[e] = fast_exp2(x);
          dv[e] = pv[e] * (dp[4 * a + e] - d4[e]);
        }
        pf[a >> 1][2 * (a & 1)] = pack2<DT>(pv[0], pv[1]);
        pf[a >> 1][2 * (a & 1) + 1] = pack2<DT>(pv[2], pv[3]);
        dsf[a >> 1][2 * (a & 1)] = pack2<DT>(dv[0], dv[1]);
        dsf[a >> 1][2 * (a & 1) + 1] = pack2<DT>(dv[2], dv[3]);
      }
      // dV^T += dO^T P and dK^T += Q^T dS over this pass's d blocks.
#pragma unroll
      for (int si = 0; si < 2; ++si)
#pragma unroll
        for (int db = 0; db < DBH; ++db) {
          dva[db] = mfma32x32x16<DT>(tr_read<D>(dbb, 0, si, DBH * pass + db, lane), pf[si], dva[db]);
          dka[db] = mfma32x32x16<DT>(tr_read<D>(qb, 0, si, DBH * pass + db, lane), dsf[si], dka[db]);
        }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();  // tile n + 1 is in; set n & 1 is free for tile n + 2
    }
    if (key_ok) {
      const size_t off = ((size_t)kvbh * N + key) * D + 32 * DBH * pass;
#pragma unroll
      for (int db = 0; db < DBH; ++db)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          u32x2 wk, wv;
          wk[0] = pack2<DT>(dka[db][4 * a + 0] * p.scale, dka[db][4 * a + 1] * p.scale);
          wk[1] = pack2<DT>(dka[db][4 * a + 2] * p.scale, dka[db][4 * a + 3] * p.scale);
          wv[0] = pack2<DT>(dva[db][4 * a + 0], dva[db][4 * a + 1]);
          wv[1] = pack2<DT>(dva[db][4 * a + 2], dva[db][4 * a + 3]);
          *(u32x2*)(p.dk + off + 32 * db + 8 * a + 4 * half) = wk;
          *(u32x2*)(p.dv + off + 32 * db + 8 * a + 4 * half) = wv;
        }
    }
  }
#endif
}

// dQ with NWQ waves of 32 query rows per workgroup.
template <int DT, int D, bool CAUSAL, int NWQ>
static hipError_t launch_dq(BwdParams p, hipStream_t s) {
  p.nblk = (p.N + 32 * NWQ - 1) / (32 * NWQ);
  hipLaunchKernelGGL((bwd_dq_kernel<DT, D, CAUSAL, NWQ>), dim3((unsigned)((long long)p.nblk * p.B * p.H)),
                     dim3(64 * NWQ), 0, s, p);
  return hipGetLastError();
}

template <int DT, int D, bool CAUSAL>
static hipError_t launch_bwd_t(BwdParams p, int num_cus, hipStream_t s) {
  constexpr int LPR = D / 8 == 12 ? 16 : D / 8, RPB = 256 / LPR;  // as bwd_delta_kernel
  const long long rows = (long long)p.B * p.H * p.N;
  hipLaunchKernelGGL((bwd_delta_kernel<DT, D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // Eight-wave dQ workgroups (256 rows, one per CU) stage each K/V tile for twice the
  // rows; as in the prefill they pay (about 2% at 16K tokens) once the grid gives every
  // CU four of them, and smaller grids keep four waves.  So do short workgroups on any
  // grid (full N <= 2048, causal N <= 4096), where two four-wave workgroups per CU
  // overlap one's prologue and epilogue with the other's tiles: +2-5% for causal
  // N = 2048..4096, +0.5-2.6% for full N = 1024..2048 (whole backward pass).  As in the
  // prefill, full grids take eight waves from two blocks per CU (+0.4-2.1% at two to
  // three per CU), causal grids from four.
  const long long blocks8 = (long long)p.B * p.H * ((p.N + 255) / 256);
  const bool short_wgs = CAUSAL ? p.N <= 4096 : p.N <= 2048;
  // d = 256 runs one wave per SIMD: four-wave workgroups only.
  if constexpr (D > 128)
    e = launch_dq<DT, D, CAUSAL, 4>(p, s);
  else
    e = blocks8 >= (CAUSAL ? 4LL : 2LL) * num_cus && !short_wgs ? launch_dq<DT, D, CAUSAL, 8>(p, s)
                                                                  : launch_dq<DT, D, CAUSAL, 4>(p, s);
  if (e != hipSuccess) return e;
  const int blk = 32 * bwd_cfg::NW;
  p.nblk = (p.N + blk - 1) / blk;
  if constexpr (D > 128)
    hipLaunchKernelGGL((bwd_dkdv_d256_kernel<DT, CAUSAL>), dim3((unsigned)((long long)p.nblk * p.B * p.Hkv)),
                       dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((bwd_dkdv_kernel<DT, D, CAUSAL>), dim3((unsigned)((long long)p.nblk * p.B * p.Hkv)),
                       dim3(64 * bwd_cfg::NW), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_backward(const void* q, const void* k, const void* v, const void* o, const void* dout,
                           const float* lse, float* ws, void* dq, void* dk, void* dv, int B, int H, int Hkv, int N,
                           int d, int dt, int causal, float scale, int num_cus, hipStream_t s) {
  BwdParams p;
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.o = (const uint16_t*)o;
  p.dout = (const uint16_t*)dout;
  p.lse = lse;
  p.delta = ws;
  p.lse2 = ws + (size_t)B * H * N;
  p.dq = (uint16_t*)dq;
  p.dk = (uint16_t*)dk;
  p.dv = (uint16_t*)dv;
  p.B = B;
  p.H = H;
  p.Hkv = Hkv;
  p.g = H / Hkv;
  p.N = N;
  p.nblk = 0;
  p.c = scale * kLog2e;
  p.scale = scale;
#define ATTN_BW(DT_, D_, C_) \
  if (dt == DT_ && d == D_ && causal == C_) return launch_bwd_t<DT_, D_, C_>(p, num_cus, s);
#define ATTN_BW_D(D_)         \
  ATTN_BW(DT_F16, D_, false)  \
  ATTN_BW(DT_F16, D_, true)   \
  ATTN_BW(DT_BF16, D_, false) \
  ATTN_BW(DT_BF16, D_, true)
  ATTN_BW_D(64)
  ATTN_BW_D(128)
  ATTN_BW_D(32)
  ATTN_BW_D(96)
  ATTN_BW_D(256)
#undef ATTN_BW_D
#undef ATTN_BW
  return hipErrorInvalidValue;
}

}  // namespace attn
