// Prefill: fused exact attention forward for gfx950 (CDNA4).
//
// Computes O = softmax(scale * Q K^T [causal]) V for [B][H][N][d] fp16/bf16 tensors,
// the prompt-phase operation of the flash-attention-cuda README (page 3, "What can it
// do" and "Kernel design"): K/V tiles are staged through on-chip memory, scores live
// only in registers, a running row max m and row sum l in fp32 rescale the output
// when the max moves (online softmax), and tiles wholly above the diagonal are skipped
// by the loop bound.  Both contractions run on the matrix cores
// (v_mfma_f32_32x32x16_{bf16,f16}, fp32 accumulation), the step page 3 lists as
// missing from its own kernel ("Limitations", "Future work").
//
// Work decomposition: one workgroup of 4 or 8 waves per (128- or 256-query block,
// head, batch); each wave owns 32 query rows.  Scores are computed transposed, S^T = K Q^T, so that
// in the MFMA result layout every lane holds 16 scores of ONE query row per 32-key
// block: row max and row sum are in-lane reductions plus one exchange with the lane
// 32 apart (v_permlane32_swap), and the output rescale is a per-lane scalar.  After
// rounding to 16 bits, the S^T accumulator registers are directly the B operand of
// the second contraction O^T = V^T P^T.
//
// Staging: K and V tiles go from HBM/L2 straight into LDS with buffer loads that
// write LDS (no registers, no VALU), 16 bytes per lane, in row-major order with the
// 16-byte chunks of each row XOR-swizzled by a per-row key so the MFMA operand reads
// are free of bank conflicts.  V^T operands are read with the LDS transpose load
// (ds_read_b64_tr_b16), which gathers four keys of one d column per lane.  Rows past
// the end of the sequence fall outside the buffer's range and are not loaded.
// Two LDS stages: tile j+1 is in flight while tile j is computed.
//
// Softmax runs in the base-2 domain: with c = scale*log2(e), p = 2^(c*s - m) where m
// is a reference for the row max of c*s.  P is computed with the current m without
// waiting for the new scores' max; m is raised (and P redone, l and O rescaled) only
// when a row's max exceeds it by more than 2^8, which a cheap guard on the sum of the
// new p detects (p <= sum <= 4096 otherwise: harmless in fp32 accumulators and in
// fp16/bf16 P).  The final O = acc / l is unaffected, since acc and l always share
// the same m.
#include <type_traits>

#include "attn_device.h"
#include "attn_launch.h"

namespace attn {

namespace prefill_cfg {
[[maybe_unused]] constexpr int BN = 64;               // keys per tile
[[maybe_unused]] constexpr float kLazyLog2 = 8.f;     // raise m only when a score exceeds it by > 2^8
[[maybe_unused]] constexpr float kSumGuard = 4096.f;  // a unit's per-lane sum of p above this prompts a check
[[maybe_unused]] constexpr float kMaxFloor = 1e30f;   // -m of a key-group row that has seen no visible key
}  // namespace prefill_cfg

struct PrefillParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  int B, H, N;
  int g;          // query heads per K/V head (grouped heads; 1 for multi-head)
  int nqblk;      // ceil(N / BM), BM = 32 * waves per workgroup
  float c;        // |scale| * log2(e) (> 0); log2(e) when scale == 0
  uint32_t qxor;  // 0x80008000 flips Q's sign (scale < 0), else 0
  uint32_t qand;  // 0 zeroes Q (scale == 0), else 0xffffffff
  float* lse;     // optional [B][H][N] row log-sum-exp (natural log), or null
};

// Two waves per SIMD need <= 256 registers a wave: QB = 1 up to d = 128, and QB = 2
// at d = 64 (246 registers).
template <int D, int QB>
constexpr int prefill_waves_per_simd() {
  return ((QB == 1 && D <= 128) || (QB == 2 && D == 64)) ? 2 : 1;
}

// NW waves per workgroup, each owning QB blocks of 32 query rows.  S4: four LDS stages
// per operand and one barrier per two tiles (loads two tiles ahead) instead of two
// stages and a barrier per tile.  QB = 1: two waves
// share each SIMD (<= 256 registers) up to d = 128; d = 256 runs one wave per SIMD.
// QB = 2: the two row blocks share every K and V operand read, halving LDS traffic
// per MFMA and giving each wave two independent softmax chains.  At d = 64 a wave of
// two blocks still fits two per SIMD; at d = 128 it needs ~350 registers, one wave
// per SIMD with the MFMA accumulators in AGPRs.
// The four-stage forms at d = 96 and 128 hold one workgroup per CU by their LDS; the
// bound of two waves per SIMD still caps their registers at 256 as measured, and the
// compiler's report that it cannot reach that occupancy is expected there.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Wpass-failed"
// KG > 1: key groups.  The NW waves form NW/KG row waves times KG key groups; the KG
// waves of one row block sweep interleaved tiles (group g takes tiles g, g + KG, ...),
// so a workgroup covers 32*QB*NW/KG query rows with KG times the waves on each, and the
// groups' (m, l, acc) states meet in LDS at the end and are merged exactly (the decode
// merge's rule, in a fixed order).  Staging then moves KG consecutive tiles per step.
template <int DT, int D, bool CAUSAL, int NW, int QB, int ST, int KG>
__global__ __launch_bounds__(64 * NW, (prefill_waves_per_simd<D, QB>())) void prefill_kernel(PrefillParams p) {
#if defined(__HIP_DEVICE_COMPILE__)  // the body uses gfx950-only types; the host pass needs only the stub
  using namespace prefill_cfg;
  constexpr int kWaves = NW;
  constexpr int kThreads = 64 * NW;
  constexpr int QW = 32 * QB;                      // query rows per wave
  constexpr int RW = NW / KG;                      // row waves (blocks of QW query rows)
  constexpr int BM = QW * RW;                      // query rows per workgroup
  constexpr int RBG = D * 2;                       // bytes per K/V row in memory
  constexpr int RB = lds_row_bytes<D>();           // bytes per K/V row in LDS
  constexpr int CH = D / 8;                        // 16-byte chunks of a row that hold data
  constexpr bool W256 = RB % 256 == 0;             // swizzle family (rows of 256 or 512 bytes)
  constexpr int KS = D / 16;                       // MFMA k-steps over the head dimension
  constexpr int DB = D / 32;                       // 32-wide output blocks along d
  constexpr int TILE_BYTES = BN * RB;              // one K (or V) tile
  constexpr int STEP_BYTES = KG * TILE_BYTES;      // staged per step: KG consecutive tiles
  constexpr int BNS = BN * KG;                     // keys per step
  constexpr int NLD = STEP_BYTES / 1024 / kWaves;  // 1 KiB LDS-direct loads per wave per step
  constexpr bool S4 = ST == 4;  // four stages, one barrier per two tiles
  static_assert(ST == 2 || ST == 4, "two or four K/V stages");
  static_assert(KG == 1 || (ST == 2 && NW == 8), "key groups run on eight-wave, two-stage workgroups");
  static_assert(NLD >= 1, "tile too small for the load pattern");
  // Two K and two V tile buffers, each its own array so the compiler can tell the
  // in-flight LDS-direct loads into one from the operand reads of another.
  __shared__ __attribute__((aligned(1024))) char kbuf0[STEP_BYTES];
  __shared__ __attribute__((aligned(1024))) char kbuf1[STEP_BYTES];
  __shared__ __attribute__((aligned(1024))) char vbuf0[STEP_BYTES];
  __shared__ __attribute__((aligned(1024))) char vbuf1[STEP_BYTES];
  constexpr int XB = S4 ? TILE_BYTES : 16;  // the third and fourth stages (four stages only)
  __shared__ __attribute__((aligned(1024))) char kbuf2[XB];
  __shared__ __attribute__((aligned(1024))) char kbuf3[XB];
  __shared__ __attribute__((aligned(1024))) char vbuf2[XB];
  __shared__ __attribute__((aligned(1024))) char vbuf3[XB];

  const int tid = thread_x();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in an SGPR
  const int lane = tid & 63;
  const int kgrp = __builtin_amdgcn_readfirstlane(wave / RW);  // key group (0 when KG == 1)
  const int rwave = wave - kgrp * RW;                          // row wave
  const int l32 = lane & 31;
  const int half = lane >> 5;

  // XCD-aware mapping: consecutive workgroup ids are dealt round-robin to the 8 XCDs;
  // give each XCD a contiguous run of work so the q-blocks sharing one head's K/V
  // (and hence its L2) run on the same XCD.
  const int G = p.nqblk * p.H * p.B;  // the grid (one workgroup per q-block, head and batch)
  const int bid = group_x();
  const int xcd = bid & 7, slot = bid >> 3;
  const int per = G >> 3, rem = G & 7;
  // Integer division is expanded on the VALU; pin the (uniform) results to SGPRs so
  // the buffer descriptors built from them stay scalar.
  int bh, qb;
  if (CAUSAL && rem == 0 && per % p.nqblk == 0) {
    // Causal, each XCD holding k whole heads: its q-blocks go out longest first across
    // all k heads (slot s takes head s mod k, the (s div k)-th longest block), so the
    // XCD's CUs finish together for any k.  Longest first within each head in turn
    // leaves an odd k unbalanced when a head has about as many blocks as the XCD has
    // CUs (one head's blocks pair up only with the next head's): measured 1131 -> 925
    // us at d = 64, H = 24, N = 16384; other causal grids +0-15%.
    const int k = __builtin_amdgcn_readfirstlane(per / p.nqblk);
    const int r = __builtin_amdgcn_readfirstlane(slot / k);
    bh = __builtin_amdgcn_readfirstlane(xcd * k + (slot - r * k));
    qb = p.nqblk - 1 - r;
  } else {
    const int work = xcd * per + min(xcd, rem) + slot;
    bh = __builtin_amdgcn_readfirstlane(work / p.nqblk);
    qb = __builtin_amdgcn_readfirstlane(work - bh * p.nqblk);
    if (CAUSAL) qb = p.nqblk - 1 - qb;  // longest rows first
  }
  bh = __builtin_amdgcn_readfirstlane(bh);
  qb = __builtin_amdgcn_readfirstlane(qb);
  const int N = p.N;
  const int q0 = qb * BM;
  const int qw0 = q0 + QW * rwave;
  int qrow[QB];
#pragma unroll
  for (int cb = 0; cb < QB; ++cb) qrow[cb] = qw0 + 32 * cb + l32;

  const size_t head_off = (size_t)bh * N * D;
  // Query head h of batch b reads K/V head h / g; with H = Hkv * g that pair index is
  // (b*H + h) / g = b*Hkv + h/g.
  const int kvbh = __builtin_amdgcn_readfirstlane(bh / p.g);
  const size_t kv_off = (size_t)kvbh * N * D;
  const uint16_t* __restrict__ qg = p.q + head_off;
  const char* kbase = (const char*)(p.k + kv_off);
  const char* vbase = (const char*)(p.v + kv_off);

  // Q as the B operand of S^T = K Q^T: lane holds Q[qrow][16ks + 8*half + 0..7].
  u32x4 qf[QB][KS];
#pragma unroll
  for (int cb = 0; cb < QB; ++cb)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 t = {0, 0, 0, 0};
      if (qrow[cb] < N) t = *(const u32x4*)(qg + (size_t)qrow[cb] * D + 16 * ks + 8 * half);
      qf[cb][ks] = (t ^ p.qxor) & p.qand;
    }

  // Tile layout in LDS: row-major rows of RB bytes whose 16-byte chunks are permuted
  // by XOR with a per-row key so that both operand reads are free of bank conflicts
  // (64 banks of 4 bytes; a wave's read is served 256 bytes per cycle, in halves of 32
  // lanes for the transpose reads).  K reads (one chunk of each of 32 consecutive
  // rows; 16 rows per pass): key row & 15 (rows of 256 or 512 B, a multiple of the
  // bank width) or (row>>1) & 7 (rows of 128 B).  V^T transpose reads (per 32-lane
  // half: 4 rows x 4 consecutive chunks): the four rows must land on four disjoint
  // 64-byte bank groups, key 4*(row & 3) (rows of 256 or 512 B) or 4*((row>>1) & 1)
  // (rows of 128 B, odd rows already offset by 128 B).  The keys stay below the
  // row's chunk count, so a swizzled chunk stays in its row.
  auto kkey = [](int row) __attribute__((always_inline)) { return W256 ? (row & 15) : ((row >> 1) & 7); };
  auto vkey = [](int row) __attribute__((always_inline)) { return W256 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2); };
  // LDS-direct load r of this wave fills LDS chunk ci = (wave*NLD + r)*64 + lane, i.e.
  // row ci / (RB/16) and physical slot ci % (RB/16), which holds logical chunk
  // slot ^ key(row): fetch that chunk from memory.  Padded rows (d = 32, 96) have
  // logical chunks past the data; those slots are never read and take a copy of a
  // chunk of the same row.
  auto src_chunk = [](int c) __attribute__((always_inline)) { return c >= CH ? c - CH : c; };
  uint32_t ldk_off[NLD], ldv_off[NLD];
#pragma unroll
  for (int r = 0; r < NLD; ++r) {
    const int ci = (wave * NLD + r) * 64 + lane;
    const int row = ci / (RB / 16), sl = ci % (RB / 16);
    ldk_off[r] = row * RBG + (src_chunk(sl ^ kkey(row)) << 4);
    ldv_off[r] = row * RBG + (src_chunk(sl ^ vkey(row)) << 4);
  }
  // K operand (A of S^T): row 32kb + l32 (key(row) does not depend on kb), logical
  // chunk 2ks + half.
  uint32_t k_off[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) k_off[ks] = kgrp * TILE_BYTES + l32 * RB + (((2 * ks + half) ^ kkey(l32)) << 4);
  // V^T operand via transpose loads: in each 16-lane group, source lane r points at
  // 4 consecutive d of key row (base + r/4), d0 = 32db + 16*((lane>>4)&1) + 4*(r&3);
  // base is a multiple of 8, so key(row) = key(row & 7).
  uint32_t v_off[DB];
  {
    const int r = lane & 15, gg = (lane >> 4) & 1;
    const int rowlo = 4 * half + (r >> 2);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int chunk = 4 * db + 2 * gg + ((r & 3) >> 1);
      v_off[db] = kgrp * TILE_BYTES + rowlo * RB + ((chunk ^ vkey(rowlo)) << 4) + 8 * (r & 1);
    }
  }

  f32x16 oacc[QB][DB];
  float m_run[QB];  // reference max of c*s for this lane's query row
  float neg_m[QB];  // -m_run, kept beside it (m_run is finite once unit 0 is seen)
  float l_run[QB];  // this lane's half of the row sum, relative to m_run
#pragma unroll
  for (int cb = 0; cb < QB; ++cb) {
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[cb][db] = (f32x16){};
    m_run[cb] = -INFINITY;
    neg_m[cb] = 0.f;
    l_run[cb] = 0.f;
  }

  const int kv_end = CAUSAL ? min(N, q0 + BM) : N;
  const int nt = (kv_end + BNS - 1) / BNS;  // steps (KG 64-key tiles each) this workgroup stages
  const int nu = (kv_end + 31) / 32;        // 32-key units in those tiles
  // Units this wave computes: a prefix of its own units (causal waves stop at their
  // diagonal).  With key groups a wave's units are the two halves of its tiles
  // kgrp, kgrp + KG, ...: count those of them up to the last unit the rows need.
  int nu_w;
  if constexpr (KG == 1) {
    nu_w = qw0 >= N ? 0 : (CAUSAL ? min(nu, (qw0 + QW - 1) / 32 + 1) : nu);
  } else {
    const int ulim = (CAUSAL ? min(nu, (qw0 + QW - 1) / 32 + 1) : nu) - 1;  // last unit needed
    const int nfull = (ulim + 1) / 2;  // tiles whose two units are both needed
    const int mine = nfull > kgrp ? (nfull - kgrp - 1) / KG + 1 : 0;
    const bool half_tile = (ulim % 2 == 0) && ((ulim / 2) % KG == kgrp);
    nu_w = qw0 >= N ? 0 : 2 * mine + (half_tile ? 1 : 0);
  }
  // First key of this wave's unit u.
  auto unit_key0 = [&](int u) __attribute__((always_inline)) {
    return KG == 1 ? 32 * u : BN * ((u >> 1) * KG + kgrp) + 32 * (u & 1);
  };

  if (N % BNS != 0) {
    // The last tile is partial and its missing rows are never written: start from
    // zeros so no uninitialised LDS bits can reach the MFMA (masked p is exactly 0).
    for (int i = tid; i < STEP_BYTES / 16; i += kThreads) {
      ((u32x4*)kbuf0)[i] = (u32x4){0, 0, 0, 0};
      ((u32x4*)kbuf1)[i] = (u32x4){0, 0, 0, 0};
      ((u32x4*)vbuf0)[i] = (u32x4){0, 0, 0, 0};
      ((u32x4*)vbuf1)[i] = (u32x4){0, 0, 0, 0};
      if constexpr (S4) {
        ((u32x4*)kbuf2)[i] = (u32x4){0, 0, 0, 0};
        ((u32x4*)kbuf3)[i] = (u32x4){0, 0, 0, 0};
        ((u32x4*)vbuf2)[i] = (u32x4){0, 0, 0, 0};
        ((u32x4*)vbuf3)[i] = (u32x4){0, 0, 0, 0};
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  auto load_tile = [&](const char* src_base, const uint32_t (&offs)[NLD], int t, char* dst) __attribute__((always_inline)) {
    const int k0 = t * BNS;
    const int rows_left = N - k0;
    const uint32_t nrec = (uint32_t)(rows_left < BNS ? rows_left : BNS) * RBG;
    // Buffer descriptor: base address, stride 0, nrec bytes in range (rows past the
    // end read nothing), raw dword format.
    const u32x4 r = buffer_rsrc(src_base + (size_t)k0 * RBG, nrec);
    const uint32_t l0 = __builtin_amdgcn_readfirstlane(lds_addr_of(dst) + wave * NLD * 1024);
#pragma unroll
    for (int i = 0; i < NLD; ++i) lds_dma16(r, offs[i], l0 + i * 1024);
  };
  auto load_k = [&](int t, char* dst) __attribute__((always_inline)) { load_tile(kbase, ldk_off, t, dst); };
  auto load_v = [&](int t, char* dst) __attribute__((always_inline)) { load_tile(vbase, ldv_off, t, dst); };

  // ---- per-unit pieces (a unit is 32 keys: one half of a staged 64-key tile) ----
  // Operand of score MFMA ks for the unit in half h of a K tile.
  auto kread = [&](const char* kb_, int h, int ks) __attribute__((always_inline)) {
    return lds_read_b128((const uint16_t*)kb_, k_off[ks] + 32 * h * RB);
  };
  // V^T operand of P*V MFMA (s, db) for the unit in half h of a V tile.
  auto vread = [&](const char* vb_, int h, int s, int db) __attribute__((always_inline)) {
    const uint32_t off = v_off[db] + (32 * h + 16 * s) * RB;
    const u32x2 lo = lds_read_tr((const uint16_t*)vb_, off);
    const u32x2 hi = lds_read_tr((const uint16_t*)vb_, off + 8 * RB);
    return (u32x4){lo[0], lo[1], hi[0], hi[1]};
  };
  // Keys past the end, and (causal) keys after the query row, score -inf.
  auto mask_unit = [&](f32x16& sc, int u, int cb) __attribute__((always_inline)) {
    const int k0 = unit_key0(u);
    const bool need = (k0 + 32 > N) || (CAUSAL && k0 + 31 > qw0 + 32 * cb);
    if (__builtin_expect(need, 0)) {  // rare: tail and diagonal units only
      const int lim = CAUSAL ? min(qrow[cb], N - 1) : N - 1;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = k0 + 8 * (i >> 2) + 4 * half + (i & 3);
        if (key > lim) sc[i] = -INFINITY;
      }
    }
  };
  // Row max of a unit (in-lane over 16 scores, then across the two lane halves).
  auto unit_max = [&](const f32x16& sc) __attribute__((always_inline)) {
    float mx = fmaxf(sc[0], sc[1]);
#pragma unroll
    for (int i = 2; i < 16; i += 2) mx = fmaxf(mx, fmaxf(sc[i], sc[i + 1]));
    return xhalf_max(mx);
  };
  // P dword w (of 8) of a unit, in three steps that the schedule spreads over
  // consecutive issue slots: x = c s - m (two FMAs), e = 2^x, then round to 16 bits,
  // pack and add into the unit's row sum.  The sum runs as two chains (even and odd
  // dwords), added at the end of the unit: half the dependent latency before the guard.
  auto p_arg = [&](const f32x16& sc, float nm, int w, float (&x)[2]) __attribute__((always_inline)) {
    x[0] = __builtin_fmaf(sc[2 * w], p.c, nm);
    x[1] = __builtin_fmaf(sc[2 * w + 1], p.c, nm);
  };
  auto p_exp = [&](float (&x)[2]) __attribute__((always_inline)) {
    x[0] = fast_exp2(x[0]);
    x[1] = fast_exp2(x[1]);
  };
  auto p_pack = [&](const float (&e)[2], u32x4 (&pf)[2], float (&l2)[2], int w) __attribute__((always_inline)) {
    const uint32_t t = pack2<DT>(e[0], e[1]);
    pf[w >> 2][w & 3] = t;
    l2[w & 1] = add_pair<DT>(t, l2[w & 1]);
  };
  // All of a unit's P with the given -m (the slow path and the prologue).
  auto p_all = [&](const f32x16& sc, u32x4 (&pf)[2], float& l_unit, float nm) __attribute__((always_inline)) {
    float l2[2] = {0.f, 0.f};
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      float x[2];
      p_arg(sc, nm, w, x);
      p_exp(x);
      p_pack(x, pf, l2, w);
    }
    l_unit = l2[0] + l2[1];
  };

  // One pipeline iteration u of this wave, a three-stage pipeline over units:
  //   matrix cores: S_{u+2} = K_{u+2} Q^T  interleaved with  O += V_u^T P_u;
  //   VALU:         P_{u+1} = 2^(c S_{u+1} - m).
  // P_{u+1} is computed optimistically with the current m.  Every p of a lane is at
  // most the lane's sum of the unit, so a sum within kSumGuard means no p left the
  // safe range and m may stay; otherwise the real row max decides: a row whose own
  // guard fired (in either half of its keys) and whose max exceeds m by more than 2^8
  // raises m, P_{u+1} is recomputed and l and O rescaled (O after this iteration's
  // MFMAs into it).  Every other row of the wave keeps m with alpha = 1 exactly and
  // recomputes the same P, so a row's result depends on its own scores alone, never on
  // which rows share its wave.  The softmax is spread over all the
  // iteration's MFMAs, about three VALU instructions (one exponential) per MFMA, with
  // each dependent step in a later slot than its input.
  // scur = S_{u+1} (scored last iteration), snext receives S_{u+2}; pcur = P_u,
  // pnext receives P_{u+1}.  kb_ holds K of unit u+2 and vb_ V of unit u, each in half h.
  // Near the end of a wave's range S_{u+2} may score keys it never uses: such a unit
  // is fully masked when it is consumed, so m and l do not move and P is zero.
  // Eight issue slots per iteration (one per dword of P).  Score MFMA a goes to slot
  // 8a / KS and P*V MFMA b to slot 8b / NP plus an offset that puts it between two
  // score slots when there are fewer than eight: d = 128 issues one of each per slot,
  // d = 64 alternates, d = 256 issues two of each per slot.
  // Each K or V operand read feeds the MFMAs of all QB row blocks.
  // Operands are read PF MFMAs ahead into a ring of PF + 1 registers that spans the
  // tile: operand a of the tile's unit h sits in slot (h*KS + a) mod (PF + 1) (K) or
  // (h*NP + a) mod (PF + 1) (V), so the first unit of a tile already reads the second
  // unit's leading operands (same buffers, no barrier between them) and only the
  // first unit after a barrier starts with reads of its own.
  constexpr int NP = 2 * DB;  // P*V MFMAs per unit and row block
  constexpr int PF = 2;       // operand prefetch distance (MFMAs of the same kind)
  constexpr int R = PF + 1;   // operand ring size
  constexpr int P_OFF = NP >= 8 ? 0 : (4 / NP > 1 ? 4 / NP : 1);
  auto s_slot = [](int a) __attribute__((always_inline)) { return 8 * a / KS; };
  auto p_slot = [](int b) __attribute__((always_inline)) { return 8 * b / NP + P_OFF; };
  auto iterate = [&](int u, f32x16 (&scur)[QB], f32x16 (&snext)[QB], const u32x4 (&pcur)[QB][2],
                     u32x4 (&pnext)[QB][2], const char* kb_, const char* vb_, int h, u32x4 (&kf)[R],
                     u32x4 (&vf)[R]) __attribute__((always_inline)) {
    const int kg = h * KS, vg = h * NP;  // ring positions of this unit's operand 0
    float l_unit[QB];
    float l2[QB][2];
    float xa[QB][2], xb[QB][2];  // P arguments / exponentials in flight, two dwords apart
#pragma unroll
    for (int cb = 0; cb < QB; ++cb) {
      mask_unit(scur[cb], u + 1, cb);  // a unit past this wave's keys masks entirely: p = 0
      l2[cb][0] = 0.f;
      l2[cb][1] = 0.f;
    }
#pragma unroll
    for (int cb = 0; cb < QB; ++cb) p_arg(scur[cb], neg_m[cb], 0, xa[cb]);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int a = 0; a < KS; ++a) {
        if (s_slot(a) != i) continue;
        if (a + PF < KS) kf[(kg + a + PF) % R] = kread(kb_, h, a + PF);
        else if (h == 0) kf[(kg + a + PF) % R] = kread(kb_, 1, a + PF - KS);
#pragma unroll
        for (int cb = 0; cb < QB; ++cb)  // the first MFMA of a chain takes a literal zero addend
          snext[cb] = mfma32x32x16<DT>(kf[(kg + a) % R], qf[cb][a], a == 0 ? (f32x16){} : snext[cb]);
      }
#pragma unroll
      for (int b = 0; b < NP; ++b) {
        if (p_slot(b) != i) continue;
        if (b + PF < NP) vf[(vg + b + PF) % R] = vread(vb_, h, (b + PF) / DB, (b + PF) % DB);
        else if (h == 0) vf[(vg + b + PF) % R] = vread(vb_, 1, (b + PF - NP) / DB, (b + PF - NP) % DB);
#pragma unroll
        for (int cb = 0; cb < QB; ++cb)
          oacc[cb][b % DB] = mfma32x32x16<DT>(vf[(vg + b) % R], pcur[cb][b / DB], oacc[cb][b % DB]);
      }
      // slot i: exponentials of dword i, pack of dword i-1, arguments of dword i+1
#pragma unroll
      for (int cb = 0; cb < QB; ++cb) {
        float (&cur_x)[2] = (i & 1) ? xb[cb] : xa[cb];
        float (&oth_x)[2] = (i & 1) ? xa[cb] : xb[cb];
        p_exp(cur_x);
        if (i >= 1) p_pack(oth_x, pnext[cb], l2[cb], i - 1);
        if (i + 1 < 8) p_arg(scur[cb], neg_m[cb], i + 1, oth_x);
        // Anchor this slot's VALU results in the slot: IR-level code motion ignores
        // sched_barrier and would otherwise gather the softmax after the MFMAs.
        asm volatile("" ::"v"(cur_x[0]), "v"(cur_x[1]), "v"(oth_x[0]), "v"(oth_x[1]), "v"(l2[cb][0]), "v"(l2[cb][1]));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    bool over = false;
#pragma unroll
    for (int cb = 0; cb < QB; ++cb) {
      p_pack((7 & 1) ? xb[cb] : xa[cb], pnext[cb], l2[cb], 7);
      l_unit[cb] = l2[cb][0] + l2[cb][1];
      over = over || (l_unit[cb] > kSumGuard);
    }
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(over) != 0, 0)) {  // rare: laid out off the hot path
#pragma unroll
      for (int cb = 0; cb < QB; ++cb) {
        const bool row_over = xhalf_max(l_unit[cb]) > kSumGuard;  // this row's own guard
        const float cand = unit_max(scur[cb]) * p.c;
        const bool raise = row_over && cand > m_run[cb] + kLazyLog2;
        const float alpha = raise ? fast_exp2(m_run[cb] - cand) : 1.f;
        m_run[cb] = raise ? cand : m_run[cb];
        neg_m[cb] = -m_run[cb];
        p_all(scur[cb], pnext[cb], l_unit[cb], neg_m[cb]);
        l_run[cb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[cb][db] *= alpha;
      }
    }
#pragma unroll
    for (int cb = 0; cb < QB; ++cb) l_run[cb] += l_unit[cb];
  };

  // Prologue: K_0, V_0, K_1 in; S_0 and S_1; P_0; then V_1 and K_2 in flight.
  f32x16 sx[QB], sy[QB];
  u32x4 pa[QB][2], pb[QB][2];
  load_k(0, kbuf0);
  load_v(0, vbuf0);
  if (nt > 1) load_k(1, kbuf1);
  if constexpr (S4) {  // tiles 0 and 1 are read before the first barrier of the loop
    if (nt > 1) load_v(1, vbuf1);
    if (nt > 2) load_k(2, kbuf2);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (nu_w > 0) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 k0f = kread(kbuf0, 0, ks), k1f = kread(kbuf0, 1, ks);
#pragma unroll
      for (int cb = 0; cb < QB; ++cb) {
        sx[cb] = mfma32x32x16<DT>(k0f, qf[cb][ks], ks == 0 ? (f32x16){} : sx[cb]);
        sy[cb] = mfma32x32x16<DT>(k1f, qf[cb][ks], ks == 0 ? (f32x16){} : sy[cb]);
      }
    }
#pragma unroll
    for (int cb = 0; cb < QB; ++cb) {
      mask_unit(sx[cb], 0, cb);
      // Key 0 is visible to every row, so group 0's first max is finite.  The first tile
      // of a later key group may hold no key a row can see: such a row starts from a
      // finite floor instead of -inf, its p are 0 until a visible key arrives, whose p
      // (2^(c s + kMaxFloor), an overflow) trips the sum guard and raises m to the
      // row's real max with alpha = 0 (l and O are still 0 then).
      m_run[cb] = unit_max(sx[cb]) * p.c;
      if constexpr (KG > 1) m_run[cb] = fmaxf(m_run[cb], -kMaxFloor);
      neg_m[cb] = -m_run[cb];
      p_all(sx[cb], pa[cb], l_run[cb], neg_m[cb]);
    }
  }
  __syncthreads();
  if constexpr (S4) {  // in flight during tiles 0 and 1: V_2, V_3, K_3, K_4
    if (nt > 2) load_v(2, vbuf2);
    if (nt > 3) load_v(3, vbuf3);
    if (nt > 3) load_k(3, kbuf3);
    if (nt > 4) load_k(4, kbuf0);
  } else {
    if (nt > 1) load_v(1, vbuf1);
    if (nt > 2) load_k(2, kbuf0);
  }

  // Tile t: units 2t, 2t+1 use V_t (vbuf[t&1]) and score units 2t+2, 2t+3 from
  // K_{t+1} (kbuf[(t+1)&1]).  After the tile, V_{t+2} and K_{t+3} take the buffers
  // just read.  Every wave passes the same nt barriers; a wave computes units
  // u < nu_w only.  Scores of units past nu_w (or of tiles never staged) are
  // computed but only ever consumed fully masked.
  auto sync_and_load = [&](int t, char* kb_next, char* vb_cur) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t + 2 < nt) load_v(t + 2, vb_cur);
    if (t + 3 < nt) load_k(t + 3, kb_next);
  };
  auto tile = [&](int t, char* kb_next, char* vb_cur) __attribute__((always_inline)) {
    u32x4 kf[R], vf[R];
#pragma unroll
    for (int a = 0; a < PF; ++a) {
      kf[a] = kread(kb_next, 0, a);
      vf[a] = vread(vb_cur, 0, a / DB, a % DB);
    }
    if (2 * t < nu_w) iterate(2 * t, sy, sx, pa, pb, kb_next, vb_cur, 0, kf, vf);
    if (2 * t + 1 < nu_w) iterate(2 * t + 1, sx, sy, pb, pa, kb_next, vb_cur, 1, kf, vf);
    sync_and_load(t, kb_next, vb_cur);
  };
  if constexpr (S4) {
    // Tile t reads V_t from vbuf[t % 4] and K_{t+1} from kbuf[(t+1) % 4].  A barrier
    // after every odd tile t frees the two V and two K buffers just read, which take
    // V_{t+3}, V_{t+4}, K_{t+4}, K_{t+5}: the tiles of the pair after next.  Scores of
    // units past the wave's range may read a buffer no tile was staged into; such units
    // are fully masked when consumed, as in the two-stage form.
    auto tile4 = [&](int t, char* kb_next, char* vb_cur) __attribute__((always_inline)) {
      u32x4 kf[R], vf[R];
#pragma unroll
      for (int a = 0; a < PF; ++a) {
        kf[a] = kread(kb_next, 0, a);
        vf[a] = vread(vb_cur, 0, a / DB, a % DB);
      }
      if (2 * t < nu_w) iterate(2 * t, sy, sx, pa, pb, kb_next, vb_cur, 0, kf, vf);
      if (2 * t + 1 < nu_w) iterate(2 * t + 1, sx, sy, pb, pa, kb_next, vb_cur, 1, kf, vf);
    };
    auto sync4 = [&](int to, char* v_a, char* v_b, char* k_a, char* k_b) __attribute__((always_inline)) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (to + 3 < nt) load_v(to + 3, v_a);
      if (to + 4 < nt) load_v(to + 4, v_b);
      if (to + 4 < nt) load_k(to + 4, k_a);
      if (to + 5 < nt) load_k(to + 5, k_b);
    };
    for (int t = 0; t < nt; t += 4) {
      tile4(t, kbuf1, vbuf0);
      if (t + 1 < nt) tile4(t + 1, kbuf2, vbuf1);
      if (t + 2 < nt) sync4(t + 1, vbuf0, vbuf1, kbuf1, kbuf2);
      if (t + 2 < nt) tile4(t + 2, kbuf3, vbuf2);
      if (t + 3 < nt) tile4(t + 3, kbuf0, vbuf3);
      if (t + 4 < nt) sync4(t + 3, vbuf2, vbuf3, kbuf3, kbuf0);
    }
  } else {
    for (int t = 0; t < nt; t += 2) {
      tile(t, kbuf1, vbuf0);
      if (t + 1 < nt) tile(t + 1, kbuf0, vbuf1);
    }
  }

  if constexpr (KG > 1) {
    // Key groups 1..KG-1 hand their states to group 0 of the same row block through the
    // staging buffers, which every wave has finished reading; group 0 merges them in
    // group order: M = max m, each state scaled by 2^(m_g - M) (a floor m gives 0).
    // Both lanes of a row hold the same m, so the per-lane halves of l merge alike.
    constexpr int RS = 64 * 4 * (QB * DB * 16 + 2 * QB);  // bytes of one wave's state
    constexpr int PER = STEP_BYTES / RS;                   // states per staging buffer
    static_assert(4 * PER >= (KG - 1) * RW, "the key groups' states do not fit the staging buffers");
    auto region = [&](int g) __attribute__((always_inline)) {
      const int r = (g - 1) * RW + rwave;
      const int a = r / PER, o = (r - a * PER) * RS;
      char* base = a == 0 ? kbuf0 : (a == 1 ? kbuf1 : (a == 2 ? vbuf0 : vbuf1));
      return base + o;
    };
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (kgrp > 0) {
      char* st = region(kgrp);
#pragma unroll
      for (int cb = 0; cb < QB; ++cb) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int a = 0; a < 4; ++a)
            *(f32x4*)(st + (((cb * DB + db) * 4 + a) * 64 + lane) * 16) =
                (f32x4){oacc[cb][db][4 * a], oacc[cb][db][4 * a + 1], oacc[cb][db][4 * a + 2], oacc[cb][db][4 * a + 3]};
        *(float2*)(st + QB * DB * 16 * 64 * 4 + (cb * 64 + lane) * 8) = make_float2(m_run[cb], l_run[cb]);
      }
    }
    __syncthreads();
    if (kgrp == 0) {
#pragma unroll
      for (int g = 1; g < KG; ++g) {
        const char* st = region(g);
#pragma unroll
        for (int cb = 0; cb < QB; ++cb) {
          const float2 ml = *(const float2*)(st + QB * DB * 16 * 64 * 4 + (cb * 64 + lane) * 8);
          const float M = fmaxf(m_run[cb], ml.x);
          const float a0 = fast_exp2(m_run[cb] - M), a1 = fast_exp2(ml.x - M);
          m_run[cb] = M;
          l_run[cb] = l_run[cb] * a0 + ml.y * a1;
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
              const f32x4 o = *(const f32x4*)(st + (((cb * DB + db) * 4 + a) * 64 + lane) * 16);
#pragma unroll
              for (int e = 0; e < 4; ++e) oacc[cb][db][4 * a + e] = oacc[cb][db][4 * a + e] * a0 + o[e] * a1;
            }
        }
      }
    }
    if (kgrp != 0) return;
  }

  // Epilogue: O = acc / l.  Lane holds d = 32db + 8a + 4*half + b for a, b in 0..3.
  // The row's scaled scores satisfy sum_j exp(scale s_j) = 2^m l for the reference m
  // the row settled on, whatever it is, so its log-sum-exp is (m + log2 l) ln 2.
#pragma unroll
  for (int cb = 0; cb < QB; ++cb) {
    const float l_tot = xhalf_sum(l_run[cb]);
    const float inv = 1.f / l_tot;
    if (p.lse && half == 0 && qrow[cb] < N)
      p.lse[(size_t)bh * N + qrow[cb]] = (m_run[cb] + __builtin_amdgcn_logf(l_tot)) * kLn2;
    if (qrow[cb] < N) {
      uint16_t* og = p.o + head_off + (size_t)qrow[cb] * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          u32x2 t;
          t[0] = pack2<DT>(oacc[cb][db][4 * a + 0] * inv, oacc[cb][db][4 * a + 1] * inv);
          t[1] = pack2<DT>(oacc[cb][db][4 * a + 2] * inv, oacc[cb][db][4 * a + 3] * inv);
          *(u32x2*)(og + 32 * db + 8 * a + 4 * half) = t;
        }
    }
  }
#endif
}
#pragma clang diagnostic pop

template <int DT, int D, bool CAUSAL, int NW, int QB, int ST = 2, int KG = 1>
static hipError_t launch_prefill_t(PrefillParams p, hipStream_t s) {
  constexpr int BM = 32 * QB * NW / KG;
  p.nqblk = (p.N + BM - 1) / BM;
  const long long grid = (long long)p.nqblk * p.H * p.B;
  hipLaunchKernelGGL((prefill_kernel<DT, D, CAUSAL, NW, QB, ST, KG>), dim3((unsigned)grid), dim3(64 * NW), 0, s, p);
  return hipGetLastError();
}

// Longest sequence whose workgroups count as short: these keep the four-wave form on
// any grid.  Measured per head size (see prefill_form).
static int short_workgroup_limit(int d, bool causal) {
  if (causal) return d == 64 ? 12288 : (d == 96 ? 6144 : 8192);
  return d == 64 ? 4096 : 2048;
}

// The workgroup form a launch takes, from the grid alone (host-side rule).
// Waves of 32 query rows, two per SIMD.  Eight waves per workgroup (256 query rows,
// one workgroup per CU) stage each K/V tile once for twice the rows of the
// four-wave form (128 rows, two workgroups per CU), halving L2-to-LDS traffic per
// MFMA; it pays (+2-3% at d = 128, 16K tokens) when the grid still gives every CU
// at least two (full) or four (causal) such workgroups, and small grids keep the
// finer four-wave blocks.
// The 64-row form (QB = 2) halves LDS operand reads per MFMA.  At d = 128 it runs
// one wave per SIMD and measured 5-8% slower, so it is not selected there; at d = 64
// it keeps two waves per SIMD and measured 9-10% faster (3-4% causal) on the
// eight-wave grids, which then take 512-row workgroups.  d = 32 measured 5-6% slower
// with it and keeps one block per wave.
// Short workgroups stay on the four-wave form whatever the grid (full: N <= 2048,
// d = 64 N <= 4096; causal: N <= 8192, d = 96 N <= 6144, d = 64 N <= 12288): the
// two workgroups a CU holds overlap one's prologue and epilogue with the other's
// tiles, and the causal diagonal's spread between waves is halved.  Measured: causal
// N = 1024..8192 +1-21% at d = 128, +5-11% at d = 32, +13-41% at d = 64 (N up to
// 12288) against two blocks per wave; full N = 512..2048 +1-11%, d = 64 at 4096 +2%.
// Longer sequences lose on it: 1-2% at d = 128, d = 96 2.6% at causal N = 8192, d = 64
// 5-6.5% at full N >= 8192 and 6% at causal N = 16384.
// d = 256 needs one SIMD per wave (its Q operands and O accumulators alone take
// 192 registers) and 128 KiB of LDS per four-wave workgroup: four waves, one
// workgroup per CU.
// Small grids (at most one 128-row block per CU, causal at most two) leave CUs idle or
// run one wave per SIMD; they take eight-wave workgroups whose waves split the keys
// (KG key groups), so every SIMD holds two waves and a block's tiles are shared out:
// 128-row blocks of two groups, or, at d <= 64 (whose four tiles per stage fit the
// LDS), 64-row blocks of four groups when those fit one round on the CUs, or for causal
// grids of long sequences (N >= 2048: the long diagonal blocks hold a quarter of their
// tiles each; the short ones of a second round fill in behind them).  Measured against
// the four-wave forms (graph replays, us): B=1 H=12 d=64 N=512 / 1024 / 2048 full 9.9 /
// 15.8 / 27.3 -> 7.8 / 10.3 / 22.4, causal 9.7 / 15.7 / 27.5 -> 8.2 / 10.7 / 21.4;
// causal N=4096 67.2 -> 47.8, d=128 H=16 N=1024 / 2048 / 4096 causal 23.5 / 41.7 / 87.9
// -> 20.7 / 33.3 / 75.6; causal B=4 N=512 9.97 -> 10.23 and B=4 N=1024 17.5 -> 17.8
// (four groups there, whose 64-row blocks take two short rounds, measured 13.1).
PrefillForm prefill_form(int B, int H, int N, int d, int causal, int num_cus) {
  if (d > 128) return {4, 1, 2, 1};
  const long long blocks4 = (long long)B * H * ((N + 127) / 128);
  if (blocks4 <= (causal ? 2LL : 1LL) * num_cus) {
    if (d <= 64 && (2 * blocks4 <= num_cus || (causal && N >= 2048 && blocks4 <= num_cus))) return {8, 1, 2, 4};
    return {8, 1, 2, 2};
  }
  // Full grids take the eight-wave forms from two 256-row blocks per CU (+3-5% at
  // two to three per CU, d = 64 +13%); causal grids, whose workgroups vary in length,
  // from four (at three per CU they measured 3% slower on it).
  const long long blocks8 = (long long)B * H * ((N + 255) / 256);
  const bool short_wgs = N <= short_workgroup_limit(d, causal != 0);
  // Four LDS stages there cost no occupancy (one eight-wave workgroup per CU either
  // way) but pay only on the full d = 64 grids: +1.4-1.9% at B*H*N = 0.26M..0.79M
  // rows; d = 128 lost 3%, causal d = 64 4%, d = 96 up to 1%, d = 32 measured flat.
  if (blocks8 >= (causal ? 4LL : 2LL) * num_cus && !short_wgs) {
    if (d == 64) return {8, 2, causal ? 2 : 4, 1};
    return {8, 1, 2, 1};
  }
  // d = 32 and 64 on the four-wave form (64 KiB of LDS for four stages, so two
  // workgroups still share a CU): four stages for grids of at most two 128-row blocks
  // per CU, and at d = 64 for causal grids, where the loads issued two tiles ahead
  // pay; other grids keep two stages.  Measured: the GPT-2-like prompts (B = 1,
  // H = 12, N = 1024..4096) +2.5-7% at d = 64 and +5-7% at d = 32; causal d = 64
  // +1-7%; full B = 4, N = 4096 d = 64 -1.6 to -2.8%; causal d = 32 on large grids
  // -6 to -8%.
  // d = 96 and 128 need 96 and 128 KiB for four stages, one workgroup per CU: they
  // take them on grids of at most one 128-row block per CU, which run one workgroup
  // per CU anyway (+2-8% at B = 1, H = 4..16, N = 2048..8192, full and causal), and
  // causal grids of at most two (+8-13% at B = 1, H = 12..16, N = 4096).  Full grids
  // of two blocks per CU lost 23-36% on it (two rounds of workgroups), causal grids
  // of three to eight 14-40%.
  if (d <= 64) {
    if (blocks4 <= 2LL * num_cus || (d == 64 && causal)) return {4, 1, 4, 1};
  } else {
    if (blocks4 <= (causal ? 2LL : 1LL) * num_cus) return {4, 1, 4, 1};
  }
  return {4, 1, 2, 1};
}

template <int DT, int D, bool CAUSAL>
static hipError_t launch_prefill_w(const PrefillParams& p, int num_cus, hipStream_t s) {
  const PrefillForm f = prefill_form(p.B, p.H, p.N, D, CAUSAL, num_cus);
  if constexpr (D > 128) {
    return launch_prefill_t<DT, D, CAUSAL, 4, 1>(p, s);
  } else {
    if constexpr (D <= 64) {
      if (f.kg == 4) return launch_prefill_t<DT, D, CAUSAL, 8, 1, 2, 4>(p, s);
    }
    if (f.kg == 2) return launch_prefill_t<DT, D, CAUSAL, 8, 1, 2, 2>(p, s);
    if (f.nw == 8) {
      if constexpr (D == 64) return launch_prefill_t<DT, D, CAUSAL, 8, 2, CAUSAL ? 2 : 4>(p, s);
      else return launch_prefill_t<DT, D, CAUSAL, 8, 1>(p, s);
    }
    if (f.st == 4) return launch_prefill_t<DT, D, CAUSAL, 4, 1, 4>(p, s);
    return launch_prefill_t<DT, D, CAUSAL, 4, 1>(p, s);
  }
}

hipError_t launch_prefill(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv, int N,
                          int d, int dt, int causal, float scale, int num_cus, hipStream_t s) {
  PrefillParams p;
  p.lse = lse;
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.o = (uint16_t*)o;
  p.B = B;
  p.H = H;
  p.N = N;
  p.g = H / Hkv;
  p.nqblk = 0;
  // Scores use c = |scale| log2(e) > 0 so the running max is a max of c*s; a negative
  // scale is carried by flipping Q's sign bits, a zero scale by a zero Q (all scores 0).
  const float as = scale < 0 ? -scale : scale;
  p.c = (scale == 0.f) ? kLog2e : as * kLog2e;
  p.qxor = scale < 0 ? 0x80008000u : 0u;
  p.qand = scale == 0.f ? 0u : 0xffffffffu;
#define ATTN_PF(DT_, D_, C_) \
  if (dt == DT_ && d == D_ && causal == C_) return launch_prefill_w<DT_, D_, C_>(p, num_cus, s);
#define ATTN_PF_D(D_)         \
  ATTN_PF(DT_F16, D_, false)  \
  ATTN_PF(DT_F16, D_, true)   \
  ATTN_PF(DT_BF16, D_, false) \
  ATTN_PF(DT_BF16, D_, true)
  ATTN_PF_D(64)
  ATTN_PF_D(128)
  ATTN_PF_D(32)
  ATTN_PF_D(96)
  ATTN_PF_D(256)
#undef ATTN_PF_D
#undef ATTN_PF
  return hipErrorInvalidValue;
}

}  // namespace attn
