// Host-side launchers of the attention kernels and the prefill launch rule, shared by
// the C interface (attn_api.hip) and the kernel files.  Internal: not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// The workgroup form a prefill launch takes: waves per workgroup, 32-row query blocks
// per wave, K/V tiles staged in LDS per operand (2, or 4 with one barrier per two
// tiles), and the key groups that split each row block's keys between waves.
struct PrefillForm {
  int nw;
  int qb;
  int st;
  int kg;
};

// The rule launch_prefill applies (host only; no HIP call).
PrefillForm prefill_form(int B, int H, int N, int d, int causal, int num_cus);

hipError_t launch_prefill(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv, int N,
                          int d, int dt, int causal, float scale, int num_cus, hipStream_t s);
// The two passes of the decode: the split pass writes the (m, l, acc) partials to ws,
// the merge pass combines them into o.
constexpr int kDecodeSplitPass = 1;
constexpr int kDecodeMergePass = 2;
hipError_t launch_decode(const void* q, const void* k, const void* v, const int32_t* seq_lens, void* o, int B, int H,
                         int Hkv, int max_len, int d, int dt, float scale, int chunk, int n_split, float* ws,
                         hipStream_t st, int passes = kDecodeSplitPass | kDecodeMergePass);
// A plain streaming read for measurement (attn_measure_read).
hipError_t launch_measure_read(const void* buf, size_t bytes, int waves, uint32_t* sink, hipStream_t st);
// Device address of this device's decode scratch array (ATTN_DECODE_SCRATCH_BYTES),
// looked up on the first call per device.
hipError_t decode_scratch(float** ptr);
int decode_heads_per_wave(int H, int Hkv);
bool decode_uses_mfma(int H, int Hkv);
int decode_mfma_waves_per_cu(int d);
hipError_t launch_backward(const void* q, const void* k, const void* v, const void* o, const void* dout,
                           const float* lse, float* ws, void* dq, void* dk, void* dv, int B, int H, int Hkv, int N,
                           int d, int dt, int causal, float scale, int num_cus, hipStream_t s);

}  // namespace attn
