// Prefill: fused exact attention forward for gfx950 (CDNA4).
//
// Computes O = softmax(scale * Q K^T [causal]) V for [B][H][N][d] fp16/bf16 tensors,
// the prompt-phase operation of the flash-attention-cuda README (page 3, "What can it
// do" and "Kernel design"): K/V tiles are staged through on-chip memory, scores live
// only in registers, a running row max m and row sum l in fp32 rescale the output
// whenever the max moves (online softmax), and tiles wholly above the diagonal are
// skipped by the loop bound.  Both contractions run on the matrix cores
// (v_mfma_f32_32x32x16_{bf16,f16}, fp32 accumulation), the step page 3 lists as
// missing from its own kernel ("Limitations", "Future work").
//
// Work decomposition: one workgroup of 4 waves per (128-query block, head, batch).
// Each wave owns 32 query rows.  The scores are computed transposed, S^T = K Q^T, so
// that in the MFMA result layout every lane holds 16 scores of ONE query row: the
// row max and row sum are in-lane reductions plus one exchange with the lane 32
// apart, and the output rescale is a per-lane scalar.  The fp32 accumulator
// registers of S^T are, after rounding to 16 bits, directly the B operand of the
// second contraction O^T = V^T P^T.  That operand order needs V with the key index
// along each lane's eight elements; V tiles are therefore written to LDS transposed
// (d-major), with the key order permuted so each lane's eight keys are contiguous.
//
// Softmax runs in the base-2 domain: with c = scale*log2(e), p = 2^(c*s - m) where m
// is the running max of c*s, which is the hardware exponential (v_exp_f32).
#include "attn_device.h"

namespace attn {

namespace prefill_cfg {
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int BM = 32 * kWaves;  // query rows per workgroup
constexpr int BN = 64;           // keys per tile
constexpr int VP = BN + 8;       // LDS pitch (elements) of one transposed V row
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

// Position of key kk (0..63) of a tile inside a transposed V row: keys read together
// by one lane for one MFMA step become 8 contiguous elements.  For the S^T result
// layout, lane half h holds keys {8a + 4h + b} (a, b in 0..3) of each 32-key block.
__device__ __forceinline__ int vt_pos(int kk) {
  const int kb = kk >> 5, r = kk & 31;
  const int a = r >> 3, h = (r >> 2) & 1, b = r & 3;
  return 32 * kb + 16 * h + 4 * a + b;
}

template <int DT, int D, bool CAUSAL>
__global__ __launch_bounds__(prefill_cfg::kThreads, 2) void prefill_kernel(PrefillParams p) {
  using namespace prefill_cfg;
  constexpr int KP = D + 8;            // LDS pitch (elements) of one K row
  constexpr int KS = D / 16;           // MFMA k-steps over the head dimension
  constexpr int DB = D / 32;           // 32-wide output blocks along d
  constexpr int KCH = BN * D / 8 / kThreads;  // 16-byte K chunks per thread per tile
  constexpr int VUNITS = (BN / 4) * (D / 8);  // 4-key x 8-d transpose units per tile
  constexpr int K_ELEMS = BN * KP;
  constexpr int V_ELEMS = D * VP;
  constexpr int STAGE = K_ELEMS + V_ELEMS;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * STAGE];

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
  const uint16_t* __restrict__ kg = p.k + head_off;
  const uint16_t* __restrict__ vg = p.v + head_off;

  // Q as the B operand of S^T = K Q^T: lane holds Q[qrow][16ks + 8*half + 0..7].
  u32x4 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 t = {0, 0, 0, 0};
    if (qrow < N) t = *(const u32x4*)(qg + (size_t)qrow * D + 16 * ks + 8 * half);
    t = (t ^ p.qxor) & p.qand;
    qf[ks] = t;
  }

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = (f32x16){};
  float m_run = -INFINITY;  // running max of c*s for this lane's query row
  float l_run = 0.f;        // this lane's half of the running row sum

  const int kv_end = CAUSAL ? min(N, q0 + BM) : N;
  const int ntiles = (kv_end + BN - 1) / BN;

  // ---- global -> register staging of one K/V tile ----
  u32x4 kreg[KCH];
  u32x4 vreg[4];
  const int vc = tid & 15;   // 4-key group of the V unit
  const int vdc = tid >> 4;  // 8-wide d chunk of the V unit
  const bool vunit = tid < VUNITS;

  auto load_tile = [&](int k0) {
#pragma unroll
    for (int r = 0; r < KCH; ++r) {
      const int ci = tid + r * kThreads;
      const int row = ci / (D / 8), col = (ci % (D / 8)) * 8;
      u32x4 t = {0, 0, 0, 0};
      if (k0 + row < N) t = *(const u32x4*)(kg + (size_t)(k0 + row) * D + col);
      kreg[r] = t;
    }
    if (vunit) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int row = k0 + 4 * vc + b;
        u32x4 t = {0, 0, 0, 0};
        if (row < N) t = *(const u32x4*)(vg + (size_t)row * D + 8 * vdc);
        vreg[b] = t;
      }
    }
  };

  auto store_tile = [&](int stage) {
    uint16_t* ks_ = lds + stage * STAGE;
    uint16_t* vs_ = ks_ + K_ELEMS;
#pragma unroll
    for (int r = 0; r < KCH; ++r) {
      const int ci = tid + r * kThreads;
      const int row = ci / (D / 8), col = (ci % (D / 8)) * 8;
      *(u32x4*)(ks_ + row * KP + col) = kreg[r];
    }
    if (vunit) {
      // Transpose 4 keys x 8 d into 8 rows (one per d) of 4 consecutive keys.
      const int pos = vt_pos(4 * vc);
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const uint32_t w0 = vreg[0][x], w1 = vreg[1][x], w2 = vreg[2][x], w3 = vreg[3][x];
        u32x2 lo, hi;
        lo[0] = (w0 & 0xffffu) | (w1 << 16);
        lo[1] = (w2 & 0xffffu) | (w3 << 16);
        hi[0] = (w0 >> 16) | (w1 & 0xffff0000u);
        hi[1] = (w2 >> 16) | (w3 & 0xffff0000u);
        *(u32x2*)(vs_ + (8 * vdc + 2 * x) * VP + pos) = lo;
        *(u32x2*)(vs_ + (8 * vdc + 2 * x + 1) * VP + pos) = hi;
      }
    }
  };

  load_tile(0);
  store_tile(0);
  __syncthreads();

  const float c = p.c;
  for (int j = 0; j < ntiles; ++j) {
    const int k0 = j * BN;
    if (j + 1 < ntiles) load_tile(k0 + BN);

    const bool active = (qw0 < N) && (!CAUSAL || k0 <= qw0 + 31);
    if (active) {
      const uint16_t* ks_ = lds + (j & 1) * STAGE;
      const uint16_t* vs_ = ks_ + K_ELEMS;

      // S^T (keys x queries) for two 32-key blocks.
      f32x16 sacc[2] = {(f32x16){}, (f32x16){}};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const u32x4 kf = *(const u32x4*)(ks_ + (32 * kb + l32) * KP + 16 * ks + 8 * half);
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
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx * c);
      const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run - m_new);
      m_run = m_new;
      const float neg_m = (m_new == -INFINITY) ? 0.f : -m_new;

      u32x4 pf[2][2];
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          float e[8];
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) {
            e[jj] = fast_exp2(__builtin_fmaf(sacc[kb][8 * s + jj], c, neg_m));
            psum += e[jj];
          }
          u32x4 t;
#pragma unroll
          for (int x = 0; x < 4; ++x) t[x] = pack2<DT>(e[2 * x], e[2 * x + 1]);
          pf[kb][s] = t;
        }
      }
      l_run = l_run * alpha + psum;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;

      // O^T (d x queries) += V^T P^T.
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            const u32x4 vf = *(const u32x4*)(vs_ + (32 * db + l32) * VP + 32 * kb + 16 * half + 8 * s);
            oacc[db] = mfma32x32x16<DT>(vf, pf[kb][s], oacc[db]);
          }
        }
      }
    }

    if (j + 1 < ntiles) store_tile((j + 1) & 1);
    __syncthreads();
  }

  // Epilogue: O = acc / l.  Lane holds d = 32db + 8a + 4*half + b for a, b in 0..3.
  const float l_tot = l_run + __shfl_xor(l_run, 32);
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
