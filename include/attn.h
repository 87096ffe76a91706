/*
 * attn.h - C interface of the MI355X (gfx950) exact attention forward library.
 *
 * The operation is exact softmax attention, O = softmax(scale * Q K^T [causal mask]) V,
 * as defined on the flash-attention-cuda README (page 3, "What is Attention?" and
 * "The Problem"), computed tile by tile with an online softmax so that the N x N
 * score table never reaches device memory (page 3, "What is Flash Attention?" and
 * "Kernel design"; page 2, "Technical details").
 *
 * Two paths, matching the two calls of page 3's "Installation" usage block:
 *   attn_prefill - the prompt phase: batched, multi-head, causal or full attention;
 *   attn_decode  - the generation phase: one new query row per (batch, head) over a
 *                  KV cache whose current length differs per sequence, computed as a
 *                  split-K pass that writes partial (m, l, acc) per chunk, then an
 *                  exact merge pass with no atomics (page 3, "Kernel design").
 * Page 3's "Future work" items built on the same kernels: grouped K/V heads
 * (attn_prefill_gqa, attn_decode_gqa), the row log-sum-exp (attn_prefill_ex), the
 * backward pass (attn_backward) and head dimensions 32, 96 and 256 beside 64 and 128.
 *
 * Conventions shared by every entry point
 *   - Tensors are dense, row-major (batch, heads, rows, d) with d fastest, no strides.
 *     All tensors of one call share one element type (attn_dtype); the output has the
 *     input's type, rounded from fp32 to nearest-even.
 *   - Pointers are DEVICE pointers (except where a parameter says host) owned by the
 *     caller; they must be non-null and 16-byte aligned (seq_lens and lse: 4-byte).
 *     The library keeps no allocation and no state between calls other than a
 *     thread-local error text, a per-device compute-unit count and the per-device
 *     scratch array of attn_decode_noalloc (part of the code object, not allocated).
 *   - `stream` is a hipStream_t (NULL selects the default stream).  Calls enqueue
 *     work on it and return without waiting; kernel faults surface on later
 *     synchronisation, launch failures are reported as ATTN_ERR_HIP.
 *   - Every argument is validated before any HIP call; an invalid call returns a
 *     negative status, enqueues nothing and sets attn_last_error().
 *   - scale may be any finite float (the pages pass 1/8 for d = 64).
 */
#ifndef ATTN_H_
#define ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { ATTN_F16 = 0, ATTN_BF16 = 1 } attn_dtype;

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = -1, /* a size, flag, pointer or scale outside its domain   */
  ATTN_ERR_UNSUPPORTED = -2, /* a head dimension or dtype this build has no kernel for */
  ATTN_ERR_ALIGNMENT = -3,   /* a pointer not 16-byte aligned                          */
  ATTN_ERR_WORKSPACE = -4,   /* caller workspace too small                             */
  ATTN_ERR_HIP = -5          /* the HIP runtime refused a launch or an allocation      */
} attn_status;

/* Prefill (page 3, "What can it do": prompt phase; "Installation": prefill(q, k, v,
 * causal, scale)).
 *   q, k, v : [B][H][N][d] inputs;  out : [B][H][N][d] output, must not alias an input.
 *   B, H, N >= 1;  d in {32, 64, 96, 128, 256} (page 3, "Future work": head sizes
 *   beyond its 64);  dtype ATTN_F16 or ATTN_BF16;  causal in {0, 1}
 *   (1: key j is visible to query row i iff j <= i).
 * Allocates nothing.  Returns ATTN_OK or a negative attn_status. */
int attn_prefill(const void* q, const void* k, const void* v, void* out, int B, int H, int N, int d,
                 int dtype, int causal, float scale, void* stream);

/* Host-only: the workgroup form attn_prefill / attn_prefill_gqa / attn_prefill_ex take
 * for this shape on a device with num_cus compute units (page 3, "Kernel design": the
 * work is cut into independent (query block, head, batch) pieces sized so that the
 * device stays full; "Challenges and debugging": a launch of too few blocks starves
 * the GPU).  Writes to HOST pointers:
 *   waves_per_workgroup : 4 or 8 waves of 64 lanes;
 *   rows_per_wave       : query rows each wave owns (32 or 64);
 *   lds_stages          : K/V tiles held in on-chip memory per operand (2 or 4);
 *   key_groups          : 1, or 2 or 4 when the waves of each row block split its keys
 *                         (small grids); a workgroup covers
 *                         waves_per_workgroup * rows_per_wave / key_groups query rows.
 * Forms with one key group compute each row with the same arithmetic (bit-identical
 * rows); key groups sum a row's keys in another order, within the same tolerance.
 * Validation as for attn_prefill (Hkv does not affect the form).  No HIP call. */
int attn_prefill_plan(int B, int H, int N, int d, int causal, int num_cus, int* waves_per_workgroup,
                      int* rows_per_wave, int* lds_stages, int* key_groups);

/* Decode (page 3, "What can it do": generation phase; "Installation": decode(q,
 * k_cache, v_cache, seq_lens, scale)).
 *   q        : [B][H][1][d] one query row per sequence and head;
 *   k_cache, v_cache : [B][H][max_len][d];
 *   seq_lens : DEVICE int32 [B], 4-byte aligned; sequence b attends to cache rows
 *              0 .. seq_lens[b]-1
 *              (the current token's own row included, so decoding token t with
 *              seq_lens = t + 1 equals causal prefill row t).  Valid lengths are
 *              1 .. max_len; the kernels clamp other values into [0, max_len] for
 *              memory safety and write zeros for a length of 0.
 *   out      : [B][H][1][d].
 *   B and H at most 65535 (the launch grid carries them in dimensions of that limit;
 *   larger values return ATTN_ERR_INVALID_ARG), here and in every decode entry point.
 * The chunk size is chosen at launch (attn_decode_choose_split with this device's
 * compute-unit count).  The partials live in a workspace taken with hipMallocAsync and
 * released with hipFreeAsync on `stream` (stream ordered, no synchronisation). */
int attn_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* seq_lens,
                void* out, int B, int H, int max_len, int d, int dtype, float scale, void* stream);

/* Decode with a caller-chosen chunk and caller-owned workspace.
 *   chunk     : cache rows per split; 0 selects the automatic choice, otherwise it must
 *               be a multiple of ATTN_DECODE_ROW_GRANULE in [granule, roundup(max_len,
 *               granule)] (every such chunk gives the same result up to fp32 rounding).
 *   workspace : DEVICE buffer of at least attn_decode_workspace_bytes(B, H, n_split, d)
 *               bytes (n_split = ceil(max_len / chunk)), 16-byte aligned; its contents on
 *               entry do not matter.  May be NULL only when ws_bytes is 0, which asks the
 *               call to behave like attn_decode (stream-ordered allocation).
 * Returns ATTN_ERR_WORKSPACE if ws_bytes is too small. */
int attn_decode_ex(const void* q, const void* k_cache, const void* v_cache, const int32_t* seq_lens,
                   void* out, int B, int H, int max_len, int d, int dtype, float scale, int chunk,
                   void* workspace, size_t ws_bytes, void* stream);

/* Rows of the decode split kernel's work granule: legal chunk sizes are multiples of it. */
#define ATTN_DECODE_ROW_GRANULE 32

/* Split chunks (one wave each) per compute unit that the automatic decode split aims for. */
#define ATTN_DECODE_WGS_PER_CU 8

/* LDS per compute unit that sizes the matrix-core decode split (160 KiB on gfx950). */
#define ATTN_DECODE_MFMA_LDS_BYTES 163840

/* Smallest chunk the automatic decode split picks (a multiple of the granule): below it
 * a wave's fixed work (query load, cross-lane combine, partial store) outweighs the
 * parallelism it adds.  Explicit chunks in attn_decode_ex may still be one granule. */
#define ATTN_DECODE_MIN_CHUNK 64

/* Host-only: the automatic decode split (page 3, "Kernel design": the chunk size is
 * chosen at launch so that even batch size 1 fills the GPU).  Each chunk is one
 * wave; aims at ATTN_DECODE_WGS_PER_CU chunks per compute unit over the B*H
 * (sequence, head) pairs, without going below ATTN_DECODE_MIN_CHUNK rows (or the
 * whole cache when it is shorter).  Writes the chunk (rows, a multiple of the granule) and the number of
 * splits to the HOST pointers chunk and n_split.  No HIP call. */
int attn_decode_choose_split(int B, int H, int max_len, int d, int num_cus, int* chunk, int* n_split);

/* Grouped K/V heads (grouped-query and multi-query attention; page 3, "Future work",
 * where the pages serve it by repeating K/V heads on the host).  Q and the output
 * keep Hq heads; K and V (or the caches) carry Hkv heads, Hkv dividing Hq, and query
 * head h reads K/V head h / (Hq / Hkv): each K/V head serves a consecutive group of
 * query heads, as repeating it in place would.  Hkv == Hq is ordinary multi-head
 * attention and gives the same results as attn_prefill / attn_decode_ex; Hkv == 1
 * is multi-query attention.  Everything else (layout, dtype, validation, ownership,
 * asynchrony) is as for the multi-head entry points; a Hkv that does not divide Hq
 * returns ATTN_ERR_INVALID_ARG.
 *
 * attn_prefill_gqa: q, out [B][Hq][N][d]; k, v [B][Hkv][N][d].  Allocates nothing. */
int attn_prefill_gqa(const void* q, const void* k, const void* v, void* out, int B, int Hq, int Hkv, int N, int d,
                     int dtype, int causal, float scale, void* stream);

/* attn_prefill_ex: attn_prefill_gqa that can also write each row's log-sum-exp
 * (page 3, "Future work", lists it with the backward pass, which needs it):
 *   lse : DEVICE float [B][Hq][N], 4-byte aligned, or NULL for none;
 *         lse[b][h][i] = log( sum over the keys j visible to row i of
 *                             exp(scale * q[b][h][i] . k[b][h / (Hq/Hkv)][j]) ), natural log,
 *         so that out[b][h][i] = sum_j exp(scale q_i . k_j - lse[b][h][i]) v_j.
 * Allocates nothing.  With lse NULL it is attn_prefill_gqa. */
int attn_prefill_ex(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq, int Hkv, int N,
                    int d, int dtype, int causal, float scale, void* stream);

/* attn_decode_gqa: q, out [B][Hq][1][d]; k_cache, v_cache [B][Hkv][max_len][d].
 * chunk / workspace / ws_bytes as for attn_decode_ex (chunk 0: automatic, from
 * attn_decode_gqa_choose_split; workspace NULL with ws_bytes 0: stream-ordered
 * allocation).  The workspace holds partials per query head:
 * attn_decode_workspace_bytes(B, Hq, n_split, d).  Groups of 3 to 32 query heads per
 * K/V head are scored together on the matrix cores, one split wave per K/V head, so the
 * cache is read once per group; otherwise each split wave reads its K/V rows once for
 * up to 8 query heads of one group. */
int attn_decode_gqa(const void* q, const void* k_cache, const void* v_cache, const int32_t* seq_lens, void* out,
                    int B, int Hq, int Hkv, int max_len, int d, int dtype, float scale, int chunk, void* workspace,
                    size_t ws_bytes, void* stream);

/* The two passes of attn_decode_gqa as separate calls (page 3, "Kernel design": the
 * split-K pass writes a partial (m, l, acc) per chunk, a second pass merges them exactly,
 * without atomics).  attn_decode_split followed by attn_decode_merge on the same stream,
 * with the same chunk and workspace, gives exactly attn_decode_gqa's output; callers use
 * the pair to time the passes apart or to run other work between them.
 *   attn_decode_split: arguments as attn_decode_gqa without `out`; chunk must be given
 *   (a legal chunk, not 0) and workspace must hold attn_decode_workspace_bytes(B, Hq,
 *   ceil(max_len / chunk), d) bytes; it is left holding the partials.
 *   attn_decode_merge: reads those partials (workspace, ws_bytes, B, Hq, max_len, d,
 *   dtype and chunk as given to the split) and writes out [B][Hq][1][d]. */
int attn_decode_split(const void* q, const void* k_cache, const void* v_cache, const int32_t* seq_lens, int B, int Hq,
                      int Hkv, int max_len, int d, int dtype, float scale, int chunk, void* workspace, size_t ws_bytes,
                      void* stream);
int attn_decode_merge(const void* workspace, size_t ws_bytes, void* out, int B, int Hq, int max_len, int d, int dtype,
                      int chunk, void* stream);

/* Measurement only, not part of the attention computation: a plain streaming read of
 * `bytes` (a positive multiple of 16) from DEVICE buffer buf (16-byte aligned) by `waves`
 * single-wave workgroups, wave w reading the w-th contiguous 1/waves of the buffer with
 * 16-byte non-temporal loads, as the decode's split waves read their chunks.  It states
 * the memory-read floor the decode is measured against.  sink: DEVICE buffer of at least
 * waves * 256 bytes that the kernel may write (in practice it writes nothing).
 * Asynchronous on `stream`; allocates nothing. */
int attn_measure_read(const void* buf, size_t bytes, int waves, void* sink, size_t sink_bytes, void* stream);

/* Host-only: the automatic split of attn_decode_gqa (writes HOST *chunk, *n_split).
 * The rule of attn_decode_choose_split over the split waves' columns:
 *   - groups of 3 to 32 query heads (matrix cores): B*Hkv columns, aiming at
 *     ATTN_DECODE_MFMA_LDS_BYTES / (4 * 32 * pitch) waves per compute unit, the number
 *     whose LDS tiles fit on one (pitch: 128 bytes for d = 32 and 64, 256 for d = 96
 *     and 128, 512 for d = 256: 10, 5 and 2 waves);
 *   - otherwise: B*Hq/G columns for G query heads per wave, aiming at
 *     ATTN_DECODE_WGS_PER_CU waves per compute unit.
 * With Hkv == Hq it equals attn_decode_choose_split.  No HIP call. */
int attn_decode_gqa_choose_split(int B, int Hq, int Hkv, int max_len, int d, int num_cus, int* chunk, int* n_split);

/* Bytes of the device scratch array that holds attn_decode_noalloc's partials (16 MiB
 * on every device the library runs on, held until the process ends). */
#define ATTN_DECODE_SCRATCH_BYTES 16777216

/* attn_decode_noalloc: attn_decode_gqa with no workspace and no allocation of any kind,
 * for callers that cannot allocate device memory: code being captured into a HIP
 * graph, tight serving loops, and hosts that forbid allocation during a step.  The
 * (m, l, acc) partials live in a fixed device array of ATTN_DECODE_SCRATCH_BYTES
 * that the library carries, one per device.
 *   Arguments, layout, validation and results as attn_decode_gqa (Hkv == Hq for
 *   multi-head decode); chunk 0 selects the automatic chunk, raised to the smallest
 *   legal chunk whose partials, attn_decode_workspace_bytes(B, Hq, n_split, d), fit the
 *   scratch.  Given the same chunk, the output equals attn_decode_gqa's bit for bit.
 *   Returns ATTN_ERR_WORKSPACE when an explicit chunk's partials exceed the scratch,
 *   or when B*Hq*(d + 2)*4 bytes (one split per head) already does.
 * Every call on a device shares that device's one array: calls that overlap in time
 * on one device (other streams, other threads) race and must be serialised by the
 * caller.  Each call overwrites every partial it reads, so nothing needs clearing. */
int attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, const int32_t* seq_lens, void* out,
                        int B, int Hq, int Hkv, int max_len, int d, int dtype, float scale, int chunk, void* stream);

/* Backward pass (page 3, "Future work"): gradients of the loss sum(dout * out) for
 * out = attn_prefill_ex(q, k, v, causal, scale), given that call's out and lse.
 *   q, out, dout, dq : [B][Hq][N][d];  k, v, dk, dv : [B][Hkv][N][d] (Hkv divides Hq);
 *   lse : DEVICE float [B][Hq][N] from attn_prefill_ex (4-byte aligned);
 *   dq = scale dS K, dk = scale dS^T Q, dv = P^T dout with P the softmax and
 *   dS = P * (dout v^T - rowsum(dout * out)); with grouped heads dk and dv sum over the
 *   query heads that read each K/V head.  Outputs are written whole (no accumulation
 *   into their previous contents) and must not alias an input or each other.
 *   workspace : DEVICE buffer of at least attn_backward_workspace_bytes(B, Hq, N) bytes
 *   (16-byte aligned; contents on entry do not matter), or NULL with ws_bytes 0 for a
 *   stream-ordered allocation.
 * Same dtype, layout, validation and asynchrony rules as attn_prefill (d in {32, 64,
 * 96, 128, 256}).  Deterministic:
 * no atomics, every output element written by one wave. */
int attn_backward(const void* q, const void* k, const void* v, const void* out, const void* dout, const float* lse,
                  void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int N, int d, int dtype, int causal,
                  float scale, void* workspace, size_t ws_bytes, void* stream);

/* Host-only: workspace bytes of attn_backward (two fp32 per query row: rowsum(dout *
 * out) and lse * log2(e), written by its pre-pass). */
size_t attn_backward_workspace_bytes(int B, int Hq, int N);

/* Host-only: bytes of decode workspace for B*H*n_split partials of (m, l, acc[d]) fp32. */
size_t attn_decode_workspace_bytes(int B, int H, int n_split, int d);

/* Host-only: a static description of a status code. */
const char* attn_status_string(int status);

/* Host-only: thread-local detail for the last non-OK return on this thread ("" if none). */
const char* attn_last_error(void);

/* Host-only: identifier of the sources this library was built from (the first 16 hex
 * digits of a sha256 over its kernel, interface and header files, fixed at compile
 * time; "unknown" for a build that did not set it).  Lets a caller check that the
 * library it loaded matches the sources it expects. */
const char* attn_build_id(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H_ */
