// Launch interface of the gfx950 kernels (internal to libtdl).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace tdl {

// ----------------------------------------------------------------- GEMM
// C = epilogue(A[M,K] * B[N,K]^T), row-major, B either of A's element type or
// Q8_0 (int8 codes [N,K] + fp16 scales [N,K/32]).  The epilogue fixes the
// operand type: fp16 for the first three, bf16 for EPI_RESID_BF16.
enum GemmEpilogue {
  EPI_BIAS_F32 = 0,    // fp16 operands; C f32  = acc + bias[n] (bias may be null)
  EPI_RESID_F32 = 1,   // fp16 operands; C f32  = acc + resid_bf16[m, n]
  EPI_RESID_BF16 = 2,  // bf16 operands; C bf16 = acc + resid_f32[m, n]
  EPI_SILU_GATE = 3    // fp16 operands; C bf16 [M, N/2] = silu(gate) * up,
                       // gate/up in alternating 16-column groups of B
};

// Weight formats of the GEMMs: bf16/fp16 elements; Q8_0 (int8 codes, one
// fp16 scale per 32 along K); per-row int8 (int8 codes, one fp32 scale and
// one zero point per output row: W = (code - zp) * scale).
enum WeightFmt : int { kWDense = 0, kWQ80 = 1, kWIQ8 = 2 };

struct GemmArgs {
  const void* A;
  int lda;
  const void* B;
  int ldb;
  const __half* B_scale;  // Q8_0 only, [N, K/32]
  const float* B_rscale;  // per-row int8 only, [N]
  const float* B_rzp;     // per-row int8 only, [N] (zero points as floats)
  int M, N, K;
  const float* bias;
  const void* resid;
  int ldr;
  void* C;
  int ldc;
  float* ws;         // split-K partial slices [splits][M][N] fp32
  int splits;
  int k_tiles_per_split;
  int b_packed;      // B (bf16/fp16, K % 64 == 0, N % 16 == 0) in the tiled
                     // layout written by pack_weights instead of row-major;
                     // the large-M kernels take such B only in that layout
  // Split tail (large-M kernels, splits == 1): workgroups past full_tiles
  // each take 1/tail_splits of the K range (tail_kps k-tiles) of one of the
  // remaining tiles and write an fp32 partial to tail_ws; a reduction kernel
  // sums them and applies the epilogue.  tail_splits == 0: off.
  int full_tiles;
  int tail_splits;
  int tail_kps;
  float* tail_ws;
  // Decode-sized kernel: the N/16 row groups (pairs of groups with the
  // SiLU-gate epilogue) are dealt out evenly over rng_count row ranges;
  // workgroup b takes range b % rng_count and K split b / rng_count.
  int rng_count;
};

// Picks a tile configuration and split count for (M, N, K) and returns the
// workspace floats it needs (for sizing at create time).  With splits > 1 a
// reduction kernel follows the GEMM.
struct GemmPlan {
  int cfg;          // tile configuration id
  int splits;
  int k_tiles_per_split;
  int grid;
  size_t ws_floats;   // workspace: split-K slices or split-tail partials
  int full_tiles;     // split tail: tiles computed whole (the rest are split)
  int tail_splits;    // 0 = no split tail
  int tail_kps;
  int rng_count;      // decode-sized kernel: row ranges
};
// packed: B in the packed tile layout (Q8_0 codes: pack_codes), which opens
// the direct-load tiles to Q8_0.
GemmPlan gemm_plan(int M, int N, int K, int wf, int epi, bool packed = false);
// Decode-sized M (<= 128, K % 32 == 0): weights streamed straight from HBM
// into MFMA operands, activations shared through LDS (cfg >= 100).
bool skinny_plan(int M, int N, int K, int wf, int epi, GemmPlan* pl);
hipError_t gemm_skinny_launch(const GemmPlan& pl, const GemmArgs& a, int wf, int epi,
                              hipStream_t s);
// reduce = false leaves split-K partials in a.ws for a consumer that sums them
// (only meaningful when plan.splits > 1).
hipError_t gemm_launch(const GemmPlan& plan, GemmArgs a, int wf, int epi, hipStream_t s,
                       bool reduce = true);

// -------------------------------------------------------- element-wise
// y[r] = fp16(x[r] * rsqrt(mean(x[r]^2) + eps) * g), x bf16 or f32.
hipError_t rmsnorm_bf16in(const void* x, const float* g, void* y, int rows, int H, float eps,
                          hipStream_t s);
hipError_t rmsnorm_f32in(const float* x, const float* g, void* y, int rows, int H, float eps,
                         hipStream_t s);
// h = sum of `splits` fp32 partial slices [splits][rows][H] + resid (bf16),
// written to h (fp32), and y = fp16(RMSNorm(h) * g): the split-K reduction of
// the output projection fused with its residual and the second RMSNorm.
hipError_t rmsnorm_splits_resid(const float* ws, int splits, const void* resid, float* h,
                                const float* g, void* y, int rows, int H, float eps, hipStream_t s);

// Per-call sequence description shared by the row-wise and attention
// kernels.  Arrays are device int32.  Three forms: rows_are_seqs (decode:
// row r = sequence r, q_len 1, ctx_len[r]); q_start null (one sequence,
// q_len0 rows from position ctx0); otherwise the general q_start / q_len /
// ctx_len arrays.
struct SeqInfo {
  const int* q_start;
  const int* q_len;
  const int* ctx_len;
  int n_seqs;
  int q_len0;
  int ctx0;
  const int* tables;  // [n_seqs, max_blocks]; null = identity (block = pos/16)
  int max_blocks;
  int rows_are_seqs;  // 1: row r is sequence r with one new token at ctx_len[r]
};

// Cache element formats.  u4 packs two codes per byte, low nibble first:
// byte 4j + b of a K row (one token, D/2 bytes) holds channels 8j + b and
// 8j + 4 + b; byte (c, slot) of a V block-head tile [D/2][16] holds channels
// 2c and 2c + 1 of that token.  Every byte belongs to one token, so writers
// of different tokens never share a byte.
enum KvFmt : int { kKvBf16 = 0, kKvU8 = 1, kKvU4 = 2 };

struct KvPool {
  void* k;          // [blocks][Hkv][16][D] (u4: [blocks][Hkv][16][D/2] bytes)
  void* v;          // [blocks][Hkv][D][16] (u4: [blocks][Hkv][D/2][16] bytes)
  int fmt;          // KvFmt
  const float* k_scale;
  const int* k_zp;
  const float* v_scale;
  const int* v_zp;
  // per-block x per-channel mode (u8 / u4): exponents e of the factor 2^e
  // that block b's KV head g applies to the per-channel scales,
  // exps[(b * Hkv + g) * 2 + 0] for K and + 1 for V; null: per-channel only
  int8_t* exps;
};
constexpr int kMaxBlockExp = 7;  // block factors 2^0 .. 2^7

// fp16 copies of the new tokens' K and V of the first n_seqs prefill
// sequences of a call, in the prefill attention kernel's tile layout
// (written by the RoPE kernel, read by prefill attention).  Per KV head g:
// K rows [rows][D] at k + g * rows * D, element (r, d) at prefill_k_index;
// V blocks of 16 rows at v + g * rows * D, element (r, d) at
// prefill_v_index.  Row r of sequence i's chunk is prefill_stage_base(seq, i)
// + r.  rows % 16 == 0.
constexpr int kStagedSeqs = 64;  // prefill sequences of one call with a staged copy
struct PrefillStage {
  _Float16* k;
  _Float16* v;
  int rows;
  int n_seqs;
};
// Staging rows sized for max_tokens new rows: every sequence starts on a
// 16-row boundary, and the last tile of a sequence may read 64 rows on.
__host__ __device__ constexpr int prefill_stage_rows(int max_tokens) {
  return ((max_tokens + 16 * kStagedSeqs + 64) + 15) & ~15;
}
__device__ __forceinline__ int prefill_stage_base(const SeqInfo& s, int i) {
  return s.q_start ? ((s.q_start[i] + 15 * i + 15) & ~15) : 0;
}
__device__ __forceinline__ int prefill_stage_vperm(int p) {  // an involution
  return (p & 12) == 4 ? p + 4 : (p & 12) == 8 ? p - 4 : p;
}
// K: the 16-byte chunk c of row r sits at chunk c ^ swz(r).  A 128-byte-wide
// read of 16 lanes (one chunk each, rows r..r+15 of one chunk column) then
// touches 16 distinct chunk positions of the 64 four-byte LDS banks: rows of
// 256 bytes (D = 128) take r & 15; rows of 128 bytes (D = 64, two rows per
// bank line) take a swizzle distinct over the 8 rows of each parity.
__device__ __forceinline__ int prefill_k_swz(int r, int D) {
  return D == 128 ? (r & 15) : ((r & 7) ^ ((r >> 3) & 1));
}
__device__ __forceinline__ int prefill_k_index(int r, int d, int D) {
  return r * D + ((((d >> 3) ^ prefill_k_swz(r, D))) << 3) + (d & 7);
}
// V: a block of 16 rows is two halves [2][D][8]; row r of the block goes to
// half vperm(r) >> 3, place vperm(r) & 7 (the keys an MFMA lane group feeds
// for one channel are one 16-byte piece, and a half's channels are
// consecutive pieces).  Index relative to the tile or staging base.
__device__ __forceinline__ int prefill_v_index(int r, int d, int D) {
  const int vp = prefill_stage_vperm(r & 15);
  return (r >> 4) * 16 * D + ((vp >> 3) * D + d) * 8 + (vp & 7);
}

// Per row of qkv (float32 [rows][(Hq+2Hkv)*D]): optional per-head RMSNorm of
// q and k, RoPE of q and k (half-split pairs, cos/sin table [max_pos][D/2]),
// q -> q_out [rows][Hq][D] float32, k and v -> the pool slot of the row's
// position (rounded once, from fp32).  splits > 1: qkv holds that many fp32
// partial slices [splits][rows][(Hq+2Hkv)*D] of the projection, summed here
// in slice order, plus bias (may be null).
// The rows of sequences < stage.n_seqs also write their K and V (the values
// the cache holds, to fp16) into the prefill staging copy.
hipError_t rope_kv_write(const void* qkv, int rows, int Hq, int Hkv, int D, const float2* tab,
                         const float* q_norm, const float* k_norm, float eps, void* q_out,
                         SeqInfo seq, KvPool pool, PrefillStage stage, hipStream_t s, int splits = 1,
                         const float* bias = nullptr, int q_skip = 0);

// Writes caller K/V rows into the pool (kv_cache_write).
hipError_t kv_write_rows(const void* k, const void* v, int src_f32, int rows, int Hkv, int D,
                         SeqInfo seq, KvPool pool, hipStream_t s);
// Per-channel min/max -> scale = (max - min) / levels, zero point
// (kv_cache_calibrate; levels 255 for u8 codes, 15 for u4).
hipError_t kv_calibrate(const float* x, int64_t n_tokens, int channels, int levels, float* scale,
                        int* zp, hipStream_t s);

// cos/sin table of RoPE angles pos * theta^(-2i/D), formed in float64.
hipError_t rope_table_build(float2* tab, int max_pos, int D, double theta, hipStream_t s);

// Weight conversion of n elements from f32 or bf16 to bf16 (dst_f16 = 0) or
// to fp16 (dst_f16 = 1; values beyond +-65504 saturate and are counted in
// *n_saturated, a device int).
hipError_t convert_weights(const void* src, int src_f32, void* dst, int dst_f16, int64_t n,
                           int* n_saturated, hipStream_t s);
// gate/up interleave: dst row (32*(j/16) + j%16) = gate row j, (+16) = up row j.
hipError_t interleave_gate_up(const void* gate, const void* up, int elem_bytes_row, int I,
                              void* dst, hipStream_t s);
hipError_t copy_f32(const float* src, float* dst, int64_t n, hipStream_t s);
// Row-major [N][K] 2-byte weights -> tiles of 16 rows x 32 k (1 KB), tile
// (n/16, k/32) at ((k/32) * N/16 + n/16) * 512 elements (all row groups of a
// 32-k slice side by side), inside a tile [k/8 % 4][n % 16][k % 8]: the
// 16-byte chunk lane l of a 16x16x32 MFMA fragment needs (row l%16, k
// 8*(l/16)..+7) is chunk l of its tile, so a fragment load, from memory or
// from a tile copied to LDS as is, is one contiguous 1 KB access.  Needs
// N % 16 == 0, K % 32 == 0.
// Q8_0 codes [N][K] int8 and scales [N][K/32] fp16 -> dst [N][K] fp16
// (dst_f16 = 1, saturating) or bf16: code * scale rounded to nearest even.
hipError_t expand_q80(const void* codes, const void* scales, int N, int K, void* dst, int dst_f16,
                      hipStream_t s);
// GGUF Q8_0 blocks [n_blocks][34 bytes] (2-byte aligned) -> codes
// [n_blocks * 32] int8 (16-byte aligned) and scales [n_blocks] fp16, a copy.
hipError_t q80_from_gguf(const void* blocks, int64_t n_blocks, void* codes, void* scales, hipStream_t s);
// Per-row int8 codes [N][K], scale [N] and zero point [N] (as floats) ->
// dst [N][K] fp16 (saturating) or bf16: (code - zp) * scale rounded once.
hipError_t expand_iq8(const void* codes, const float* scale, const float* zp, int N, int K, void* dst,
                      int dst_f16, hipStream_t s);
// Epilogues of the int8 x int8 GEMM (v = C a_scale[m] b_scale[n]):
// kA8Out: fp32 out = v (and the int32 sums to C if not null); kA8Bias:
// fp32 out = v + bias[n]; kA8ResidF32: fp32 out = v + bf16 resid[m][n];
// kA8ResidBf16: bf16 out = v + fp32 resid[m][n]; kA8SiluGate: bf16
// out[m][16g + c] = silu(v[m][32g + c]) * v[m][32g + 16 + c] (N % 32 == 0).
enum A8EpiKind : int { kA8Out = 0, kA8Bias = 1, kA8ResidF32 = 2, kA8ResidBf16 = 3, kA8SiluGate = 4 };
struct A8Epi {
  int epi;
  const float* bias;
  const void* resid;
  int ldr;
  void* out;
  int ldo;
};
hipError_t a8w8_gemm_epi(const void* A, const void* B, const float* a_scale, const float* b_scale,
                         int32_t* C, const A8Epi& e, int M, int N, int K, hipStream_t s);
// int8 x int8 GEMM: C = A[M,K] B[N,K]^T in int32 (written if C != null),
// out = C * a_scale[m] * b_scale[n] in fp32.  K % 16 == 0.
hipError_t a8w8_gemm(const void* A, const void* B, const float* a_scale, const float* b_scale,
                     int32_t* C, float* out, int M, int N, int K, hipStream_t s);
// Per-row symmetric int8 quantisation of an fp16 (x_bf16 = 0) or bf16 row
// [rows][K]: s[r] = max|x| / 127 (1 for a zero row), q = rint(x / s)
// clipped to +-127.  K % 16 == 0.
hipError_t quant_rows_i8(const void* x, int x_bf16, int rows, int K, int8_t* q, float* s, hipStream_t st);
// int8 [n] -> float [n]
hipError_t i8_to_f32(const void* src, float* dst, int64_t n, hipStream_t s);
hipError_t pack_weights(const void* src, void* dst, int N, int K, hipStream_t s);
// int8 codes [N][K] -> the stream kernel's packed code layout: 1 KB tiles
// (64-k stage st, 16-row group g) at ((st * N/16) + g) KB, lane l's 16 bytes
// = codes of row 16g + l%16 at k = 64st + 8(l/16) .. +7, then the same at
// k + 32 (the two 32-k steps of the stage).  Needs N % 16 == 0, K % 64 == 0.
hipError_t pack_codes(const void* src, void* dst, int N, int K, hipStream_t s);
// Element offset of (n, k) in that layout.
__host__ __device__ inline size_t packed_offset(int n, int k, int N) {
  return ((size_t)(k >> 5) * (N >> 4) + (n >> 4)) * 512 + (size_t)((((k >> 3) & 3) << 4) + (n & 15)) * 8 +
         (k & 7);
}

// ------------------------------------------------------------- attention
// Flash prefill attention over sequences 0..n_prefill-1 of `seq`: keys
// before each chunk from the pool (bf16, u8 or u4) through the tables, the
// chunk's own keys from `st` (sequences < st.n_seqs) or from the pool.  q
// [rows][Hq][D] f32; o [rows][Hq*D] fp16 (saturating).
// Prefill queries taken straight from the QKV projection (rope_fused): the
// attention kernel adds the bias (if not null), applies the Q-norm (gain not
// null) and RoPE as it loads them.  qkv == null: q holds rotated queries.
struct PrefillQ {
  const float* qkv;  // [rows][ldq] fp32, the q heads first
  int ldq;
  const float* bias;  // [Hq * D] or null
  const float* norm;  // [D] or null
  float eps;
  const float2* rope;  // [max_pos][D/2] (cos, sin)
};
hipError_t attn_prefill(const void* q, const PrefillQ& qsrc, KvPool pool, SeqInfo seq, PrefillStage st,
                        int n_prefill, int max_q_len, int Hq, int Hkv, int D, void* o, hipStream_t s);

// Paged decode attention for decode sequences first_seq .. first_seq+batch-1
// (one query row each).  Each sequence's context is cut into partitions of
// part_blocks blocks; `part` holds the partitions' (O, m, l) and a merge
// kernel combines them.
constexpr int kMaxDecodeSeqs = 2048;        // sequences in one decode launch
constexpr int kMaxDecodePosition = 131072;  // longest context (keys) per sequence
struct DecodePlan {
  int part_blocks;
  int max_parts;
  size_t part_floats;        // partial-result workspace of this launch
  size_t part_floats_bound;  // >= part_floats of any max_ctx_len up to this one
};
DecodePlan decode_plan(int batch, int Hq, int Hkv, int D, int max_ctx_len, int fmt);
hipError_t attn_decode(const DecodePlan& plan, const void* q, KvPool pool, SeqInfo seq,
                       int first_seq, int batch, int Hq, int Hkv, int D, void* o, float* part,
                       hipStream_t s);

}  // namespace tdl
