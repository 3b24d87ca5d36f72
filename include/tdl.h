/*
 * tdl.h -- C ABI of an MI355X (gfx950) implementation of one Qwen-style
 * grouped-query-attention decoder layer: RMSNorm -> Q/K/V projection (+bias)
 * -> (optional per-head Q/K RMSNorm) -> RoPE -> causal GQA attention ->
 * output projection + residual -> RMSNorm -> SwiGLU MLP + residual.
 *
 * Sources of the operations (pages the design follows):
 *  [QWEN] "从零实现 C++ LLM 推理引擎：加载 Qwen2.5-7B 并跑通单层 Forward Pass":
 *         architecture overview (the op sequence of one layer), section 2
 *         (RMSNorm, RoPE over Q and K heads in one kernel), section 3 (GQA,
 *         28 Q heads over 4 KV heads), section 4 (row-major Y = X W^T with W
 *         stored [out, in]), section 5 (owning handles free their memory).
 *  [TFF]  "十年 C++ 后端 GAP 六个月 ... LLM-TFFInfer推理框架项目解析": section
 *         3.6.4 (paged KV cache: LIFO free list, allocate fails when empty,
 *         page table, get_location(t) = (table[t / page], t % page)),
 *         section 3.7.2 (flash attention: tiled K/V, online softmax), the
 *         layer hyper-parameter set of its graph context (section 3.5).
 *  [HET]  devpress article on a C++-native heterogeneous inference engine:
 *         section 2.3 / 4.3 (paged attention, 16-token blocks, a kernel that
 *         walks the block table), section 2.6 (int8 asymmetric per-channel
 *         formula), section 2.2 (prefill and decode mixed in one step,
 *         chunked prefill), the C-ABI as its cross-language surface.
 *
 * Conventions for every call:
 *  - Every function returns tdl_status; nothing throws across the ABI.  On an
 *    error, tdl_last_error() (thread-local) holds a message.
 *  - All host-side argument checks happen before anything is enqueued, so a
 *    call that fails leaves no partial work behind.
 *  - "device pointer" = memory on the current HIP device (e.g. a torch CUDA
 *    tensor's data_ptr()); "host pointer" = ordinary host memory.  The
 *    library never dereferences a device pointer on the host.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = default stream) and
 *    is asynchronous: inputs must stay valid and outputs untouched until the
 *    stream reaches that point.  No call synchronises the stream, except
 *    layer_create / kv_cache_alloc at set-up.
 *  - Activation arrays (x, y of the layer calls) must be 16-byte aligned
 *    (the kernels move them in 16-byte chunks); a misaligned one is
 *    TDL_E_INVALID.  torch allocations are 256-byte aligned.
 *  - bf16 means IEEE bfloat16 (16-bit, 8-bit exponent); every fp32 -> bf16
 *    conversion rounds to nearest, ties to even.
 *  - A layer handle and a KV handle each serve one host thread at a time.
 */
#ifndef TDL_H
#define TDL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TDL_OK = 0,
  TDL_E_INVALID = 1,      /* bad argument (null pointer, size out of range, ...) */
  TDL_E_UNSUPPORTED = 2,  /* valid request this build does not implement        */
  TDL_E_CAPACITY = 3,     /* a size limit fixed at create time, or no free blocks */
  TDL_E_NOMEM = 4,        /* device allocation failed                            */
  TDL_E_HIP = 5           /* a HIP runtime call or kernel launch failed          */
} tdl_status;

typedef enum {
  TDL_BF16 = 0,
  TDL_F32 = 1,
  TDL_Q8_0 = 2,    /* 32 int8 codes + one fp16 scale per block along K          */
  TDL_U8_ASYM = 3, /* uint8 codes + per-channel fp32 scale and int32 zero point */
  TDL_U4_ASYM = 4, /* uint4 codes, two per byte, + the same per-channel parameters */
  TDL_I8_ROW = 5,  /* weight-only int8: codes + per-output-row fp32 scale and int8 zero point */
  TDL_A8W8 = 6     /* int8 weights + per-output-row fp32 scale, int8 activations ([HET] 4.5) */
} tdl_dtype;

typedef void* tdl_stream; /* hipStream_t */
typedef struct tdl_layer tdl_layer;
typedef struct tdl_kv_cache tdl_kv_cache;
typedef struct tdl_stack tdl_stack;

/* Layer hyper-parameters ([TFF] 3.5 graph context: heads, kv heads, head
 * size, rope base, rms eps; [QWEN] "运行结果" config line). */
typedef struct {
  int32_t hidden;         /* H                                              */
  int32_t n_q_heads;      /* Hq                                             */
  int32_t n_kv_heads;     /* Hkv; Hq % Hkv == 0, Hq / Hkv <= 16             */
  int32_t head_dim;       /* D: 64 or 128                                   */
  int32_t intermediate;   /* I of the SwiGLU MLP                            */
  float rms_eps;
  float rope_theta;       /* RoPE base; half-split pairs (i, i + D/2)       */
  int32_t qkv_bias;       /* 1: Q/K/V projections have a bias               */
  int32_t qk_norm;        /* 1: per-head RMSNorm on q and k before RoPE     */
  int32_t weight_dtype;   /* TDL_F32, TDL_BF16, TDL_Q8_0, TDL_I8_ROW or TDL_A8W8 */
  int32_t max_tokens;     /* most rows (new tokens) in one call             */
  int32_t max_seqs;       /* most sequences in one call                     */
  int32_t max_position;   /* positions 0 .. max_position-1 can be rotated   */
  int32_t rope_fused;     /* 1: prefill rows' queries are normalised (Qwen3
                             Q-norm), given their bias and rotated by the
                             prefill attention kernel as it loads them from
                             the QKV projection ([TFF] 3.7.2 item 4, RoPE
                             applied while Q is loaded); the RoPE kernel then
                             handles only their K and V.  0: the RoPE kernel
                             writes every row's rotated q.  Same results
                             either way up to the rounding of q.             */
} tdl_layer_config;

/* Weights, device pointers in PyTorch Linear layout ([out, in], row-major).
 * Matrices wq [Hq*D, H], wk/wv [Hkv*D, H], wo [H, Hq*D], wg/wu [I, H],
 * wd [H, I] hold weight_dtype elements: float32, bf16, or for Q8_0 the int8
 * codes, with the fp16 scales in w*_scale [out, in/32].  TDL_I8_ROW
 * (weight-only per-channel int8, [HET] 4.4): int8 codes, w*_scale float32
 * [out] and w*_zp int8 [out], W[n][k] = (code[n][k] - zp[n]) * scale[n];
 * decode-sized calls (<= 128 rows) stream the codes, larger ones use fp16 /
 * bf16 copies expanded at create time (when max_tokens > 128).  TDL_A8W8
 * (int8 activations x int8 weights, [HET] 4.5): int8 codes and w*_scale
 * float32 [out] (symmetric, W[n][k] = code[n][k] * scale[n]); every
 * projection quantises its input rows to int8 with a float32 scale per row
 * (s = max|x| / 127 of the row as the layer holds it: xn, o, hn in fp16, the
 * SwiGLU product in bf16; codes round-half-even(x / s), clipped to +-127),
 * multiplies on the int8 matrix units with int32 sums and dequantises with
 * both scales in fp32 before the usual bias / residual / SiLU-gate.
 * Needs every input dimension a multiple of 16.  Biases bq/bk/bv
 * (if qkv_bias) and gains ln1/ln2 [H], q_norm/k_norm [D] (if qk_norm) are
 * float32.  Unused pointers may be NULL.  layer_create copies (and repacks)
 * everything into library-owned memory; the caller may free its copies once
 * layer_create has returned. */
typedef struct {
  const void *ln1, *wq, *bq, *wk, *bk, *wv, *bv, *wo, *ln2, *wg, *wu, *wd, *q_norm, *k_norm;
  const void *wq_scale, *wk_scale, *wv_scale, *wo_scale, *wg_scale, *wu_scale, *wd_scale;
  const void *wq_zp, *wk_zp, *wv_zp, *wo_zp, *wg_zp, *wu_zp, *wd_zp;  /* TDL_I8_ROW only */
} tdl_layer_weights;

/* Paged KV cache ([TFF] 3.6.4 KVConfig; [HET] 4.3 BlockManager). */
typedef struct {
  int32_t n_blocks;       /* physical blocks in the pool                    */
  int32_t block_size;     /* tokens per block; must be 16                   */
  int32_t n_kv_heads;
  int32_t head_dim;       /* 64 or 128                                      */
  int32_t kv_dtype;       /* TDL_BF16, TDL_U8_ASYM or TDL_U4_ASYM ([HET] 2.4) */
  uint64_t free_list_seed;/* 0: blocks handed out 0,1,2,...; otherwise the
                             free list is a seeded random permutation       */
  int32_t block_scales;   /* 0: per-channel parameters only.  1 (u8 / u4):
                             per-block x per-channel ([HET] 2.4 scales per
                             channel and per block; 4.3 dequantises block b
                             with its own scales[b]): block b's KV head g
                             multiplies the per-channel scales of K and of V
                             by 2^e, e in [0, 7] the smallest exponent for
                             which none of the values that the call writing
                             the block's first slot puts there clamps; later
                             calls appending to the block keep it.  A block
                             whose first slot was never written by a call
                             uses what its exponent bytes hold (0 in a
                             library-allocated cache).                      */
} tdl_kv_config;

/* Where a cache's bytes live.  Element (block b, kv head g, token slot s,
 * channel d) of K is at k_pool[b*k_strides[0] + g*k_strides[1] +
 * s*k_strides[2] + d*k_strides[3]] (strides in elements; same for V).  K is
 * stored [block][head][slot][d]; V is stored [block][head][d][slot] so that
 * the 16 tokens of one channel are contiguous.  For TDL_U8_ASYM and
 * TDL_U4_ASYM the four parameter arrays hold [n_kv_heads * head_dim]
 * entries; otherwise NULL.
 * TDL_U4_ASYM (elem_bytes 0): two 4-bit codes per byte, low nibble first,
 * and the strides count bytes.  K row (block b, head g, slot s) is D/2
 * bytes; its byte 4j + i (i < 4) holds channels 8j + i and 8j + 4 + i.  V
 * is [block][head][D/2 channel pairs][16 slots] bytes: byte (c, s) holds
 * channels 2c and 2c + 1 of slot s.  Every byte belongs to one token. */
typedef struct {
  void* k_pool;
  void* v_pool;
  int64_t k_strides[4];
  int64_t v_strides[4];
  int32_t elem_bytes;
  float* k_scale;
  int32_t* k_zero_point;
  float* v_scale;
  int32_t* v_zero_point;
  int8_t* block_exp;      /* block_scales: [n_blocks][n_kv_heads][2] exponents
                             (K, V); otherwise NULL */
} tdl_kv_view;

/* A batch of sequences for layer_step ([HET] 2.2, 4.2: prefill chunks and
 * decode tokens mixed in one step).  Sequence i owns rows q_start[i] ..
 * q_start[i]+q_len[i]-1 of x and y; its new tokens take positions
 * ctx_len[i] .. ctx_len[i]+q_len[i]-1; its first ctx_len[i] tokens are in the
 * cache already.  Sequences 0 .. n_prefill_seqs-1 may have any q_len >= 1;
 * sequences n_prefill_seqs .. n_seqs-1 must have q_len == 1 (decode).
 * q_start/q_len/ctx_len/block_tables are device int32 arrays (block_tables
 * [n_seqs, max_blocks]); the host bounds size the launch grids and must hold:
 * n_rows == sum q_len, max_q_len >= every prefill q_len, max_ctx_len >=
 * every ctx_len + q_len. */
typedef struct {
  int32_t n_seqs;
  int32_t n_prefill_seqs;
  int32_t n_rows;
  int32_t max_q_len;
  int32_t max_ctx_len;
  int32_t max_blocks;
  const int32_t* q_start;
  const int32_t* q_len;
  const int32_t* ctx_len;
  const int32_t* block_tables;
} tdl_batch;

/* Device pointers to a layer's intermediate buffers, valid after a call has
 * completed on its stream, for stage-by-stage checks.  Row r of each holds
 * the call's row r.  xn [rows, H] fp16 (RMSNorm-1 output); qkv [rows,
 * (Hq+2Hkv)*D] float32 (projections + bias, before RoPE; not written when a
 * decode-sized projection is split over K: the RoPE kernel then sums the
 * split partial products itself); q [rows, Hq, D]
 * float32 (after Q-norm and RoPE; with rope_fused, written for decode rows
 * only); o [rows, Hq*D] fp16 (attention output);
 * h [rows, H] float32 (first residual); hn [rows, H] fp16 (RMSNorm-2
 * output); a [rows, I] bf16 (silu(gate) * up).
 * The projections take fp16 operands where their input is bounded (xn, o,
 * hn: weights converted to fp16 at layer_create, which refuses weights
 * beyond +-65504) and bf16 for the down projection (a is unbounded).
 * Ranges: xn and hn are fp16, |x * g / rms(x)| <= sqrt(H) * max|g|, so they
 * saturate (at +-65504, finite) only for a norm gain above 65504/sqrt(H).
 * Prefill attention computes on fp16 copies of K and V (exactly the values
 * the cache holds while they lie in the fp16 range) and writes o in fp16:
 * |K| and |V| above 65504 saturate there, finite but not the bf16 value.
 * Decode attention reads a bf16 cache as bf16 (hi + lo pairs of q and P)
 * and u8 / u4 codes within their calibrated range, with no such limit. */
typedef struct {
  const void *xn, *qkv, *q, *o, *h, *hn, *a;
} tdl_workspace_view;

/* ---------------------------------------------------------------- layer */

/* Validates the configuration, allocates the library-owned weight copies and
 * workspace (sized by max_tokens / max_seqs), converts f32 weights to bf16
 * and interleaves gate/up rows for the fused SiLU-gate epilogue.  A Q8_0
 * layer keeps only its codes (repacked into 1 KB tiles of 16 rows x 64
 * inputs where N % 16 == 0 and K % 64 == 0) and fp16 block scales, about
 * 1.06 bytes per weight: every call multiplies exact fp16/bf16 copies of the
 * codes on the matrix units and scales each 32-input block's product by its
 * scale in fp32.
 * Synchronises `stream` before returning.  *out is NULL on failure.
 * TDL_E_UNSUPPORTED when min(max_seqs, max_tokens) > 2048 (decode sequences
 * in one call) or max_position > 131072. */
tdl_status layer_create(const tdl_layer_config* cfg, const tdl_layer_weights* w,
                        tdl_stream stream, tdl_layer** out);

/* Frees everything the handle owns.  Work still queued on a stream that uses
 * the handle must have finished.  NULL is accepted. */
tdl_status layer_destroy(tdl_layer* layer);

/* Prompt prefill of one sequence ([QWEN] architecture overview): x, y are
 * [n_tokens, H] bf16 device arrays (y must not overlap x); the new tokens
 * take positions start_pos .. start_pos+n_tokens-1.  With kv != NULL their
 * K/V are written into the cache through block_table (device int32, at least
 * ceil((start_pos+n_tokens)/16) valid entries) and attention also reads
 * the start_pos tokens already cached (chunked prefill).  With kv == NULL,
 * start_pos must be 0 and K/V live only for the call.
 * 1 <= n_tokens <= max_tokens; start_pos + n_tokens <= max_position. */
tdl_status layer_prefill(tdl_layer* layer, tdl_stream stream, const void* x, void* y,
                         int32_t n_tokens, int32_t start_pos, tdl_kv_cache* kv,
                         const int32_t* block_table);

/* One decode step of `batch` sequences, one new token each ([HET] 4.3;
 * [TFF] 3.6.4 append_token): x, y [batch, H] bf16.  ctx_lens (device int32
 * [batch]) counts the tokens already cached; the new token's K/V goes to
 * position ctx_lens[b] first, then attention covers ctx_lens[b]+1 keys read
 * through block_tables (device int32 [batch, max_blocks]).  max_ctx_len is a
 * host bound >= every ctx_lens[b]+1 and <= max_blocks*16 (it sizes the grid).
 * The device arrays are trusted; TDL_DEBUG=1 in the environment copies them
 * back and checks them (and synchronises) before enqueuing. */
tdl_status layer_decode_paged(tdl_layer* layer, tdl_stream stream, const void* x, void* y,
                              int32_t batch, const int32_t* ctx_lens,
                              const int32_t* block_tables, int32_t max_blocks,
                              int32_t max_ctx_len, tdl_kv_cache* kv);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops, harnesses that forbid hipMalloc): layer_decode_paged
 * with the same arguments, kernels and results, whose split-K partial slices
 * and decode partition results live in a static 32 MiB array the library
 * holds on each GPU it runs on (until the process ends) instead of the
 * layer's workspace.  Calls no hipMalloc, hipFree, event or synchronising
 * function; records no stage timing; skips the TDL_DEBUG table check.  A
 * step whose partial results exceed 32 MiB is TDL_E_CAPACITY (for example a
 * Qwen3-8B-shaped layer at batch 128 over 8192-token contexts; a
 * Qwen2.5-7B-shaped one at batch 64 needs about 10 MB).  Every call on a GPU
 * shares that GPU's array (each call writes what it reads first): calls that
 * overlap on one GPU, on any streams, race. */
tdl_status layer_decode_paged_noalloc(tdl_layer* layer, tdl_stream stream, const void* x, void* y,
                                      int32_t batch, const int32_t* ctx_lens,
                                      const int32_t* block_tables, int32_t max_blocks,
                                      int32_t max_ctx_len, tdl_kv_cache* kv);

/* A mixed step over a tdl_batch: all rows go through the projections and the
 * MLP together; prefill sequences use the flash prefill attention kernel and
 * decode sequences the paged decode kernel.  x, y [n_rows, H] bf16. */
tdl_status layer_step(tdl_layer* layer, tdl_stream stream, const tdl_batch* batch,
                      const void* x, void* y, tdl_kv_cache* kv);

/* Pointers to the intermediate buffers (see tdl_workspace_view). */
tdl_status layer_workspace_view(const tdl_layer* layer, tdl_workspace_view* out);

/* Per-stage timing.  While enabled, every call records a pair of hipEvents
 * around each of its kernels on the call's stream (a few microseconds per
 * call; timing-only events, created without the system-scope fence, so that
 * recording one does not write back and invalidate the caches between
 * stages).  layer_profile_read synchronises those events, adds their elapsed
 * times to the totals and returns the totals since the last enable. */
enum {
  TDL_STAGE_RMSNORM1 = 0,  /* x -> xn                         */
  TDL_STAGE_QKV = 1,       /* xn W_qkv^T + b                   */
  TDL_STAGE_ROPE_KV = 2,   /* q/k norm, RoPE, KV slot write     */
  TDL_STAGE_ATTN_PREFILL = 3,
  TDL_STAGE_ATTN_DECODE = 4,
  TDL_STAGE_O_PROJ = 5,    /* h = x + o W_o^T                  */
  TDL_STAGE_RMSNORM2 = 6,  /* h -> hn                          */
  TDL_STAGE_GATE_UP = 7,   /* a = silu(hn W_g^T) * (hn W_u^T)  */
  TDL_STAGE_DOWN = 8,      /* y = h + a W_d^T                  */
  TDL_N_STAGES = 9
};
typedef struct {
  double ms[TDL_N_STAGES];        /* summed kernel time per stage          */
  int64_t launches[TDL_N_STAGES]; /* kernel launches counted per stage     */
} tdl_profile;

tdl_status layer_profile_enable(tdl_layer* layer, int enable);
tdl_status layer_profile_read(tdl_layer* layer, tdl_profile* out);

/* ---------------------------------------------------------------- stack */

/* A stack of layers applied in order, as one decode step of a whole model
 * ([TFF] 3.6.1: the runtime's decode loop runs every layer per generated
 * token; 3.6.2: a captured graph replays such a step).  The layers stay
 * caller-owned and must outlive the stack; they must share `hidden`.  The
 * stack owns two bf16 activation buffers of min(max_seqs, max_tokens) rows
 * (over its layers) x hidden, allocated here.  *out is NULL on failure. */
tdl_status stack_create(tdl_layer* const* layers, int32_t n_layers, tdl_stack** out);

/* Frees the activation buffers (not the layers).  Work still queued on a
 * stream that uses the stack must have finished.  NULL is accepted. */
tdl_status stack_destroy(tdl_stack* stack);

/* One decode step through every layer: layer 0 reads x, layer i>0 reads
 * layer i-1's output, the last layer writes y (x, y [batch, hidden] bf16;
 * y must not alias x).  kvs[i] (n_layers handles) is layer i's cache; all
 * caches use the same block_tables and ctx_lens (the same sequences), with
 * the arguments of layer_decode_paged.  Every layer's arguments are checked
 * before the first layer is enqueued; a failure there enqueues nothing.  No
 * allocation and, unless TDL_DEBUG=1, no synchronisation: a graph capture
 * records the whole step. */
tdl_status stack_decode_paged(tdl_stack* stack, tdl_stream stream, const void* x, void* y,
                              int32_t batch, const int32_t* ctx_lens,
                              const int32_t* block_tables, int32_t max_blocks,
                              int32_t max_ctx_len, tdl_kv_cache* const* kvs);

/* ------------------------------------------------------------- KV cache */

/* Bytes of device memory a cache with this configuration needs (pools plus,
 * for TDL_U8_ASYM / TDL_U4_ASYM, the per-channel parameters).  0 for an
 * invalid config. */
size_t kv_cache_bytes(const tdl_kv_config* cfg);

/* Creates a cache handle.  dev_mem == NULL: the library allocates
 * kv_cache_bytes(cfg) device bytes (zeroed) and frees them in kv_cache_free;
 * otherwise dev_mem (caller-owned, >= kv_cache_bytes, 256-byte aligned) is
 * used as is and never touched by the host.  The host-side free list
 * ([TFF] 3.6.4 PageManager) always lives in the handle. */
tdl_status kv_cache_alloc(const tdl_kv_config* cfg, void* dev_mem, tdl_kv_cache** out);

/* Frees the handle (and the device memory if the library allocated it).
 * NULL is accepted. */
tdl_status kv_cache_free(tdl_kv_cache* kv);

tdl_status kv_cache_view(const tdl_kv_cache* kv, tdl_kv_view* out);

/* Block tables on the host ([TFF] 3.6.4 append_token / allocate; [HET] 4.3
 * acquire).  table (host int32 [n_seqs, max_blocks]) is read and updated:
 * for sequence i, entries 0 .. ceil(n_tokens[i]/16)-1 that are < 0 receive a
 * block popped from the free list; entries already >= 0 are kept; entries
 * from ceil(n_tokens[i]/16) on are left alone.  All or nothing: if the free
 * list is too short (TDL_E_CAPACITY) or any n_tokens[i] needs more than
 * max_blocks blocks (TDL_E_INVALID), nothing changes. */
tdl_status kv_block_table(tdl_kv_cache* kv, int32_t n_seqs, const int32_t* n_tokens,
                          int32_t max_blocks, int32_t* table);

/* Block holders ([HET] 4.3: each physical block carries a ref_count).  A
 * block handed out by kv_block_table has one holder; kv_block_share adds
 * one per listed entry, kv_block_release drops one per listed entry, and a
 * block whose last holder lets go returns to the free list.  Sequences that
 * share a block read it; only a block with one holder may be written (the
 * kernels cannot check this: the caller appends only to blocks it holds
 * alone).  A listed block that is out of range or free, or (release) listed
 * more often than it has holders, fails the whole call with TDL_E_INVALID
 * and nothing changes. */
tdl_status kv_block_release(tdl_kv_cache* kv, const int32_t* blocks, int32_t n);
tdl_status kv_block_share(tdl_kv_cache* kv, const int32_t* blocks, int32_t n);

/* Holders of a block (0: free); -1 for a NULL handle or a block out of range. */
int32_t kv_block_refs(const tdl_kv_cache* kv, int32_t block);

/* Number of blocks on the free list. */
int32_t kv_free_blocks(const tdl_kv_cache* kv);

/* Prefix index ([HET] 4.7 prefix cache: block-aligned longest common prefix,
 * matched blocks serve as the initial KV of a prefill at start_pos =
 * 16 * matched).  Host-side map from a caller-chosen 64-bit key to a full
 * block.  The key of a sequence's block i must identify every token of
 * blocks 0..i (for example a hash chain over the token ids), because a
 * block's K/V depend on all earlier tokens.
 *
 * kv_prefix_publish: block i (allocated, full, never written again) is
 * indexed under keys[i]; the index becomes one of its holders.  A key that
 * is already indexed keeps its block (the first publisher wins; the
 * caller's block is left as it is).  A block indexed under another key, an
 * entry that pairs a key or block of an earlier entry differently, or a
 * free or out-of-range block fails the call (TDL_E_INVALID, no change).
 *
 * kv_prefix_match: walks keys[0..n-1] and stops at the first key not in the
 * index; blocks[0 .. *n_matched-1] receive the matched blocks, each with one
 * more holder (the caller, who releases them like its own).
 *
 * kv_prefix_evict: drops up to n_blocks index entries whose block no one
 * but the index holds, least recently matched or published first; their
 * blocks return to the free list.  Returns the number dropped.
 *
 * kv_prefix_size: entries in the index. */
tdl_status kv_prefix_publish(tdl_kv_cache* kv, const uint64_t* keys, const int32_t* blocks,
                             int32_t n);
tdl_status kv_prefix_match(tdl_kv_cache* kv, const uint64_t* keys, int32_t n, int32_t* blocks,
                           int32_t* n_matched);
int32_t kv_prefix_evict(tdl_kv_cache* kv, int32_t n_blocks);
int32_t kv_prefix_size(const tdl_kv_cache* kv);

/* TDL_U8_ASYM / TDL_U4_ASYM only: sets the per-channel (kv head, d)
 * parameters of K and of V from n_tokens float32 rows k, v [n_tokens, Hkv,
 * D] (device): scale = (max - min) / L with L = 255 (u8) or 15 (u4),
 * zero_point = round_half_even(-min / scale), scale 1 for a flat channel
 * ([HET] 2.6; the pages give the formula for 8 bits only, u4 takes the same
 * one with 15 levels).  Later writes use them. */
tdl_status kv_cache_calibrate(tdl_kv_cache* kv, tdl_stream stream, const float* k,
                              const float* v, int64_t n_tokens);

/* Writes K/V rows into the cache: rows cu_rows[i] .. cu_rows[i+1]-1 of k, v
 * ([rows, Hkv, D], src_dtype TDL_F32 or TDL_BF16, device) belong to sequence
 * i and go to positions start_pos[i] + 0, 1, ... through block_tables
 * (device int32 [n_seqs, max_blocks]).  cu_rows, start_pos: device int32.
 * bf16 caches round to nearest even; u8 / u4 caches quantise with
 * clamp(round_half_even(x / scale) + zero_point, 0, L), L = 255 / 15. */
tdl_status kv_cache_write(tdl_kv_cache* kv, tdl_stream stream, int32_t n_seqs,
                          const int32_t* cu_rows, const int32_t* start_pos,
                          const int32_t* block_tables, int32_t max_blocks, int32_t src_dtype,
                          const void* k, const void* v, int32_t n_rows);

/* ------------------------------------------------------------ A8W8 GEMM */

/* int8 x int8 GEMM with a dequantising epilogue ([HET] 4.5, activation
 * quantisation: int8 activations and weights on the int8 matrix units,
 * accumulated in int32, then out = C * a_scale[m] * b_scale[n]).
 * A [M, K] and B [N, K] int8, row-major (B in Linear layout), 16-byte
 * aligned; a_scale [M], b_scale [N] float32; out [M, N] float32; C_accum
 * [M, N] int32 receives the exact sums when not NULL (all device memory).
 * K must be a positive multiple of 16; M or N == 0 is a no-op.  The sums are
 * exact while |C| < 2^31 (K <= 131072 always is).  Enqueued on the stream;
 * no allocation, no synchronisation. */
tdl_status gemm_a8w8(tdl_stream stream, const void* A, const void* B, const float* a_scale,
                     const float* b_scale, int32_t* C_accum, float* out, int32_t M, int32_t N,
                     int32_t K);

/* ---------------------------------------------------- GGUF Q8_0 import */

/* Splits GGUF's interleaved Q8_0 tensor data into the arrays layer_create
 * takes for TDL_Q8_0 weights.  The TFFInfer page loads Qwen3-8B as a Q8_0
 * GGUF file (section 1.1) and stores a quantised row of `cols` values as
 * cols/32 consecutive blocks (section 3.4, block-aware strides).  A block is
 * 34 bytes: the scale as a little-endian IEEE binary16, then the 32 int8
 * codes of columns 32b .. 32b+31 in order.
 * blocks: rows * cols/32 blocks, row-major, 2-byte aligned; codes: int8
 * [rows, cols], 16-byte aligned; scales: fp16 [rows, cols/32], 2-byte
 * aligned (all device memory, caller-owned).  cols must be a positive
 * multiple of 32; rows == 0 is a no-op.  A bit-exact copy; enqueued on the
 * stream, no allocation, no synchronisation. */
tdl_status q80_import_gguf(tdl_stream stream, const void* blocks, int64_t rows, int64_t cols,
                           void* codes, void* scales);

/* --------------------------------------------------------------- errors */

const char* tdl_status_string(tdl_status s);
const char* tdl_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* TDL_H */
