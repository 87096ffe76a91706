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
// Work decomposition: one workgroup of 4 waves per (128-query block, head, batch);
// each wave owns 32 query rows.  Scores are computed transposed, S^T = K Q^T, so that
// in the MFMA result layout every lane holds 16 scores of ONE query row per 32-key
// block: row max and row sum are in-lane reductions plus one exchange with the lane
// 32 apart (v_permlane32_swap), and the output rescale is a per-lane scalar.  After
// rounding to 16 bits, the S^T accumulator registers are directly the B operand of
// the second contraction O^T = V^T P^T.
//
// Staging: K and V tiles go from HBM/L2 straight into LDS with buffer loads that
// write LDS (no registers, no VALU), 16 bytes per lane, in row-major order with the
// 16-byte chunks of each row XOR-swizzled by (row mod 8) so the MFMA operand reads
// are free of bank conflicts.  V^T operands are read with the LDS transpose load
// (ds_read_b64_tr_b16), which gathers four keys of one d column per lane.  Rows past
// the end of the sequence fall outside the buffer's range and are not loaded.
// Two LDS stages: tile j+1 is in flight while tile j is computed.
//
// Softmax runs in the base-2 domain: with c = scale*log2(e), p = 2^(c*s - m) where m
// tracks the row max of c*s.  m is only raised when a new score exceeds it by more
// than 2^8 (so p <= 256, harmless in fp32 accumulators and in fp16/bf16 P); most
// tiles then skip the rescale of l and the output registers entirely.  The final
// O = acc / l is unaffected, since acc and l always share the same m.
#include <type_traits>

#include "attn_device.h"

namespace attn {

namespace prefill_cfg {
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int BM = 32 * kWaves;  // query rows per workgroup
constexpr int BN = 64;           // keys per tile
constexpr float kLazyLog2 = 8.f;  // raise m only when a score exceeds it by > 2^8
}  // namespace prefill_cfg

struct PrefillParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  int B, H, N;
  int nqblk;      // ceil(N / BM)
  float c;        // |scale| * log2(e) (> 0); log2(e) when scale == 0
  uint32_t qxor;  // 0x80008000 flips Q's sign (scale < 0), else 0
  uint32_t qand;  // 0 zeroes Q (scale == 0), else 0xffffffff
};

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ u32x2 lds_read_tr(const uint16_t* lds_base, uint32_t byte_off) {
  const s16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)((__attribute__((address_space(3))) char*)lds_base + byte_off));
  return __builtin_bit_cast(u32x2, t);
}

__device__ __forceinline__ u32x4 lds_read_b128(const uint16_t* lds_base, uint32_t byte_off) {
  return *(const u32x4*)((const char*)lds_base + byte_off);
}

// max(x, x of the lane 32 apart) and the sum likewise, from one v_permlane32_swap:
// it returns (x with its upper half replaced by the partner's lower half, and the
// partner half's view), so the two results hold {x, partner} in some order.
__device__ __forceinline__ float xhalf_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Row sum of packed 16-bit P pairs: sum += lo + hi (v_dot2 with (1, 1)).
template <int DT>
__device__ __forceinline__ float add_pair(uint32_t pair, float acc);
template <>
__device__ __forceinline__ float add_pair<DT_BF16>(uint32_t pair, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), __builtin_bit_cast(bf16x2, 0x3f803f80u),
                                         acc, false);
}
template <>
__device__ __forceinline__ float add_pair<DT_F16>(uint32_t pair, float acc) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pair), __builtin_bit_cast(f16x2, 0x3c003c00u), acc, false);
}

template <int DT, int D, bool CAUSAL>
__global__ __launch_bounds__(prefill_cfg::kThreads, 2) void prefill_kernel(PrefillParams p) {
#if defined(__HIP_DEVICE_COMPILE__)  // the body uses gfx950-only types; the host pass needs only the stub
  using namespace prefill_cfg;
  constexpr int RB = D * 2;                  // bytes per K/V row
  constexpr int KS = D / 16;                 // MFMA k-steps over the head dimension
  constexpr int DB = D / 32;                 // 32-wide output blocks along d
  constexpr int TILE_BYTES = BN * RB;        // one K (or V) tile
  constexpr int NLD = TILE_BYTES / 1024 / kWaves;  // 1 KiB LDS-direct loads per wave per tile
  constexpr int STAGE_BYTES = 2 * TILE_BYTES;      // K tile then V tile
  static_assert(NLD >= 1, "tile too small for the load pattern");
  // One array per stage, so the compiler can tell the in-flight LDS-direct loads of
  // one stage from the operand reads of the other and not wait on them.
  __shared__ __attribute__((aligned(1024))) uint16_t lds0[STAGE_BYTES / 2];
  __shared__ __attribute__((aligned(1024))) uint16_t lds1[STAGE_BYTES / 2];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int half = lane >> 5;

  // XCD-aware mapping: consecutive workgroup ids are dealt round-robin to the 8 XCDs;
  // give each XCD a contiguous run of work so the q-blocks sharing one head's K/V
  // (and hence its L2) run on the same XCD.
  const int G = gridDim.x;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, slot = bid >> 3;
  const int per = G >> 3, rem = G & 7;
  const int work = xcd * per + min(xcd, rem) + slot;
  const int bh = work / p.nqblk;
  int qb = work - bh * p.nqblk;
  if (CAUSAL) qb = p.nqblk - 1 - qb;  // longest rows first
  const int N = p.N;
  const int q0 = qb * BM;
  const int qw0 = q0 + 32 * wave;
  const int qrow = qw0 + l32;

  const size_t head_off = (size_t)bh * N * D;
  const uint16_t* __restrict__ qg = p.q + head_off;
  const char* kbase = (const char*)(p.k + head_off);
  const char* vbase = (const char*)(p.v + head_off);

  // Q as the B operand of S^T = K Q^T: lane holds Q[qrow][16ks + 8*half + 0..7].
  u32x4 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 t = {0, 0, 0, 0};
    if (qrow < N) t = *(const u32x4*)(qg + (size_t)qrow * D + 16 * ks + 8 * half);
    qf[ks] = (t ^ p.qxor) & p.qand;
  }

  // Per-lane byte offsets of the LDS-direct loads: load r of this wave fills LDS
  // chunk ci = (wave*NLD + r)*64 + lane, i.e. row ci / (RB/16), physical slot
  // ci % (RB/16), which holds logical 16-byte chunk slot ^ (row & 7).
  uint32_t ld_off[NLD];
#pragma unroll
  for (int r = 0; r < NLD; ++r) {
    const int ci = (wave * NLD + r) * 64 + lane;
    const int row = ci / (RB / 16), sl = ci % (RB / 16);
    ld_off[r] = row * RB + ((sl ^ (row & 7)) << 4);
  }
  // K operand (A of S^T): row 32kb + l32, logical chunk 2ks + half.
  uint32_t k_off[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) k_off[ks] = l32 * RB + ((((2 * ks + half) ^ (l32 & 7))) << 4);
  // V^T operand via transpose loads: in each 16-lane group, source lane r points at
  // 4 consecutive d of key row (base + r/4), d0 = 32db + 16*((lane>>4)&1) + 4*(r&3).
  uint32_t v_off[DB];
  {
    const int r = lane & 15, gg = (lane >> 4) & 1;
    const int rowlo = 4 * half + (r >> 2);  // row within an 8-row group, = row & 7
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int chunk = 4 * db + 2 * gg + ((r & 3) >> 1);
      v_off[db] = rowlo * RB + ((chunk ^ rowlo) << 4) + 8 * (r & 1);
    }
  }

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = (f32x16){};
  float m_run = -INFINITY;  // reference max of c*s for this lane's query row
  float l_run = 0.f;        // this lane's half of the row sum, relative to m_run

  const int kv_end = CAUSAL ? min(N, q0 + BM) : N;
  const int ntiles = (kv_end + BN - 1) / BN;

  if (N % BN != 0) {
    // The last tile is partial and its missing rows are never written: start from
    // zeros so no uninitialised LDS bits can reach the MFMA (masked p is exactly 0).
    for (int i = tid; i < STAGE_BYTES / 16; i += kThreads) {
      ((u32x4*)lds0)[i] = (u32x4){0, 0, 0, 0};
      ((u32x4*)lds1)[i] = (u32x4){0, 0, 0, 0};
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  auto issue_loads = [&](int k0, auto stage_c) {
    constexpr int stage = decltype(stage_c)::value;
    const int rows_left = N - k0;
    const uint32_t nrec = (uint32_t)(rows_left < BN ? rows_left : BN) * RB;
    const __amdgpu_buffer_rsrc_t kr =
        __builtin_amdgcn_make_buffer_rsrc((void*)(kbase + (size_t)k0 * RB), 0, nrec, 0x00020000);
    const __amdgpu_buffer_rsrc_t vr =
        __builtin_amdgcn_make_buffer_rsrc((void*)(vbase + (size_t)k0 * RB), 0, nrec, 0x00020000);
    char* st = (char*)(stage == 0 ? lds0 : lds1);
#pragma unroll
    for (int r = 0; r < NLD; ++r) {
      char* dst = st + (wave * NLD + r) * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void*)dst, 16, ld_off[r], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void*)(dst + TILE_BYTES), 16, ld_off[r], 0, 0, 0);
    }
  };

  const float c = p.c;
  auto compute = [&](int k0, auto stage_c) {
    constexpr int stage = decltype(stage_c)::value;
    const bool active = (qw0 < N) && (!CAUSAL || k0 <= qw0 + 31);
    if (!active) return;
    const uint16_t* ks_ = stage == 0 ? lds0 : lds1;
    const uint16_t* vs_ = ks_ + TILE_BYTES / 2;

    // S^T (keys x queries) for two 32-key blocks.
    f32x16 sacc[2] = {(f32x16){}, (f32x16){}};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u32x4 kf = lds_read_b128(ks_, k_off[ks] + 32 * kb * RB);
        sacc[kb] = mfma32x32x16<DT>(kf, qf[ks], sacc[kb]);
      }
    }

    // Mask keys past the end, and (causal) keys after the query row.
    const bool need_mask = (k0 + BN > N) || (CAUSAL && k0 + BN - 1 > qw0);
    if (need_mask) {
      const int lim = CAUSAL ? min(qrow, N - 1) : N - 1;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = k0 + 32 * kb + 8 * (i >> 2) + 4 * half + (i & 3);
          if (key > lim) sacc[kb][i] = -INFINITY;
        }
    }

    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; i += 2) mx = fmaxf(mx, fmaxf(sacc[kb][i], sacc[kb][i + 1]));
    mx = xhalf_max(mx);
    const float cand = mx * c;
    const bool raise = cand > m_run + kLazyLog2;
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {
      // Only rows that need it move their m (alpha = 1 exactly elsewhere), so every
      // row's arithmetic depends on its own scores alone.
      const float alpha = raise ? fast_exp2(m_run - cand) : 1.f;  // m_run = -inf gives 0
      m_run = raise ? cand : m_run;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
    }
    const float neg_m = (m_run == -INFINITY) ? 0.f : -m_run;

    u32x4 pf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        u32x4 t;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const float e0 = fast_exp2(__builtin_fmaf(sacc[kb][8 * s + 2 * x], c, neg_m));
          const float e1 = fast_exp2(__builtin_fmaf(sacc[kb][8 * s + 2 * x + 1], c, neg_m));
          t[x] = pack2<DT>(e0, e1);
          l_run = add_pair<DT>(t[x], l_run);
        }
        pf[kb][s] = t;
      }
    }

    // O^T (d x queries) += V^T P^T.
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const uint32_t rowoff = (32 * kb + 16 * s) * RB;
          const u32x2 lo = lds_read_tr(vs_, v_off[db] + rowoff);
          const u32x2 hi = lds_read_tr(vs_, v_off[db] + rowoff + 8 * RB);
          const u32x4 vf = {lo[0], lo[1], hi[0], hi[1]};
          oacc[db] = mfma32x32x16<DT>(vf, pf[kb][s], oacc[db]);
        }
      }
    }
  };

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  issue_loads(0, S0{});
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int j = 0; j < ntiles; j += 2) {
    if (j + 1 < ntiles) issue_loads((j + 1) * BN, S1{});
    compute(j * BN, S0{});
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (j + 1 >= ntiles) break;
    if (j + 2 < ntiles) issue_loads((j + 2) * BN, S0{});
    compute((j + 1) * BN, S1{});
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // Epilogue: O = acc / l.  Lane holds d = 32db + 8a + 4*half + b for a, b in 0..3.
  const float l_tot = xhalf_sum(l_run);
  const float inv = 1.f / l_tot;
  if (qrow < N) {
    uint16_t* og = p.o + head_off + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        u32x2 t;
        t[0] = pack2<DT>(oacc[db][4 * a + 0] * inv, oacc[db][4 * a + 1] * inv);
        t[1] = pack2<DT>(oacc[db][4 * a + 2] * inv, oacc[db][4 * a + 3] * inv);
        *(u32x2*)(og + 32 * db + 8 * a + 4 * half) = t;
      }
  }
#endif
}

template <int DT, int D, bool CAUSAL>
static hipError_t launch_prefill_t(const PrefillParams& p, hipStream_t s) {
  const long long grid = (long long)p.nqblk * p.H * p.B;
  hipLaunchKernelGGL((prefill_kernel<DT, D, CAUSAL>), dim3((unsigned)grid), dim3(prefill_cfg::kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_prefill(const void* q, const void* k, const void* v, void* o, int B, int H, int N, int d, int dt,
                          int causal, float scale, hipStream_t s) {
  PrefillParams p;
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.o = (uint16_t*)o;
  p.B = B;
  p.H = H;
  p.N = N;
  p.nqblk = (N + prefill_cfg::BM - 1) / prefill_cfg::BM;
  // Scores use c = |scale| log2(e) > 0 so the running max is a max of c*s; a negative
  // scale is carried by flipping Q's sign bits, a zero scale by a zero Q (all scores 0).
  const float as = scale < 0 ? -scale : scale;
  p.c = (scale == 0.f) ? kLog2e : as * kLog2e;
  p.qxor = scale < 0 ? 0x80008000u : 0u;
  p.qand = scale == 0.f ? 0u : 0xffffffffu;
#define ATTN_PF(DT_, D_, C_) \
  if (dt == DT_ && d == D_ && causal == C_) return launch_prefill_t<DT_, D_, C_>(p, s);
  ATTN_PF(DT_F16, 64, false)
  ATTN_PF(DT_F16, 64, true)
  ATTN_PF(DT_F16, 128, false)
  ATTN_PF(DT_F16, 128, true)
  ATTN_PF(DT_BF16, 64, false)
  ATTN_PF(DT_BF16, 64, true)
  ATTN_PF(DT_BF16, 128, false)
  ATTN_PF(DT_BF16, 128, true)
#undef ATTN_PF
  return hipErrorInvalidValue;
}

}  // namespace attn
