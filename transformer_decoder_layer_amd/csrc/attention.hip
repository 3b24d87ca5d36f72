// Paged decode attention: grouped-query attention of one new token per
// sequence over the block-paged KV cache (prefill attention is in
// prefill_attention.hip).
//
// KV pool layout (elements): K [block][kv_head][slot 0..15][d] -- one head's
// block is one contiguous tile (the per-block base address of the paged
// kernel on the devpress engine page, section 4.3); V [block][kv_head][d]
// [slot], so that the 16 tokens of a channel are contiguous and feed the
// key-dimension of the P*V matrix product directly.
//
// The kernel computes S^T = K * Q^T on the MFMA units (keys as rows), so
// the softmax of one query row lives in one lane (plus its partner lanes),
// and O^T = V^T * P^T, whose B operand is exactly the register layout the
// first product leaves P in -- P never goes through LDS.  Scores are scaled
// by log2(e)/sqrt(D) so exp2 gives e^(s - m); softmax is the online form
// (running max m, denominator l, rescaled accumulator) of the TFFInfer page,
// section 3.7.2 item 5, with the per-tile update written in full.
//
// A workgroup owns (sequence, KV head, context partition); its four
// waves walk the partition's blocks through the block table, one 16-token
// block per step, with the whole query-head group packed into the 16 columns
// of one MFMA tile.  u8 / u4 caches are dequantised in registers: a code c
// becomes the fp16 value 1024 + c (u8) or 64 + c (u4) exactly (a byte
// permute per two codes, after a nibble mask for u4); the K scale is folded
// into q and the zero point and bias into a per-head constant, the V scale,
// zero point and bias are applied once at the end.
// A second kernel merges the partitions' (m, l, acc) triples of each
// (sequence, KV head) in partition order.

#include "common.h"
#include "kernels.h"

#include <algorithm>
#include <type_traits>

namespace tdl {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 8.f;  // slack of the running maximum (log2 units)

typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

// fp32 -> fp16, saturating at the fp16 range
__device__ __forceinline__ f16 to_f16(float v) { return f32_to_f16_sat(v); }

__device__ __forceinline__ int seq_row(const SeqInfo& s, int sidx) {
  if (s.rows_are_seqs) return sidx;
  return s.q_start ? s.q_start[sidx] : 0;
}
__device__ __forceinline__ int seq_qlen(const SeqInfo& s, int sidx) {
  if (s.rows_are_seqs) return 1;
  return s.q_start ? s.q_len[sidx] : s.q_len0;
}
__device__ __forceinline__ int seq_ctx(const SeqInfo& s, int sidx) {
  if (s.rows_are_seqs || s.q_start) return s.ctx_len[sidx];
  return s.ctx0;
}
__device__ __forceinline__ int seq_block(const SeqInfo& s, int sidx, int lblk) {
  if (!s.tables) return lblk;
  return s.tables[(size_t)sidx * s.max_blocks + lblk];
}

// ================================================================= decode
struct DecArgs {
  const float* q;
  KvPool pool;
  SeqInfo seq;
  int first_seq;
  int Hq, Hkv;
  int part_blocks, max_parts;
  float* part;  // [batch][Hkv][max_parts][16*D + 32]: unnormalised O, then (m, l)
  f16* o;
};

constexpr int kPartStride(int D) { return 16 * D + 32; }

// Blocks of a decode sequence with ctx cached tokens (ctx + 1 keys), cut to
// what the launch was sized for (max_parts partitions of part_blocks) and to
// the block-table width: the device arrays are trusted, and this keeps a
// context above the host's max_ctx_len bound inside the partition workspace,
// the merge kernel's LDS and the table row.
__device__ __forceinline__ int dec_blocks(const DecArgs& a, int ctx) {
  int n = cdiv(max(ctx, 0) + 1, kBlockTokens);
  n = min(n, a.max_parts * a.part_blocks);
  if (a.seq.tables && a.seq.max_blocks > 0) n = min(n, a.seq.max_blocks);
  return n;
}

template <int D, int F>
struct DecFrags {
  // K rows (A operand): key lane%16.  bf16: one 16-byte chunk per product
  // s, channels 32s + 8*(lane/16) .. +7; u8: one chunk per product pair,
  // channels 64h + 16*(lane/16) .. +15, the first 8 for product 2h, the
  // last 8 for 2h + 1; u4: one D/8-byte piece for all products, dword s
  // (8 codes) for product s (dec_kchan)
  using KT = typename std::conditional<
      F == kKvBf16, bf16x8,
      typename std::conditional<F == kKvU8 || D == 128, uint4, uint2>::type>::type;
  KT k[F == kKvBf16 ? D / 32 : F == kKvU8 ? D / 64 : 1];
  // V^T rows (A operand), keys 4*(lane/16) .. +3: bf16 / u8: channel 16t +
  // lane%16 of tile t; u4: one dword per tile pair, the low nibbles for
  // tile 2u, the high ones for 2u + 1 (dec_vchan)
  using VT = typename std::conditional<F == kKvBf16, bf16x4, uint32_t>::type;
  VT v[F == kKvU4 ? D / 32 : D / 16];
};

// First of the 8 channels lane group grp feeds to k-slots 8grp .. 8grp+7
// of the key-query product s (any channel order gives the same dot product,
// as long as K and q use the same one).  u8: a lane takes one 16-byte chunk
// (16 channels) of its key row per pair of products; u4: the lane's D/4
// channels of the row at once, dword s of them (channels 8s .. 8s+7 of the
// piece, by the pool's nibble order) for product s.
template <int D, int F>
__device__ __forceinline__ int dec_kchan(int s, int grp) {
  return F == kKvBf16 ? 32 * s + 8 * grp
       : F == kKvU8   ? 64 * (s >> 1) + 16 * grp + 8 * (s & 1)
                      : (D / 4) * grp + 8 * s;
}
// Channel of row i of output tile t (row i of the V^T operand).  u4: a
// dword of the [channel pair][key] tile gives channel 2c in its low
// nibbles and 2c + 1 in its high ones: tiles 2u and 2u + 1 take the even
// and odd channels of pairs 16u .. 16u + 15.
template <int F>
__device__ __forceinline__ int dec_vchan(int t, int i) {
  return F == kKvU4 ? 2 * (16 * (t >> 1) + i) + (t & 1) : 16 * t + i;
}

// LDS staging of one block-head: K (16 keys x D codes or elements), then
// for u8 / u4 the V^T tile (as many bytes again); bf16 V^T fragments load
// straight into registers (each of their loads already reads whole cache
// lines).  16-byte chunks; K chunk c of key r sits at slot r * CPR + (c ^
// x(r)), so the 8 lanes that read a 128-byte LDS row together (same chunk,
// keys r..r+7) hit 8 different bank quads, while each copy instruction
// still reads 1 KB of whole key rows.  (u4 with D = 64: 32-byte rows, read
// 8 bytes per lane, not swizzled.)
template <int D, int F>
struct DecStage {
  static constexpr int kRow = F == kKvBf16 ? 2 * D : F == kKvU8 ? D : D / 2;  // bytes per key row
  static constexpr int kK = kBlockTokens * kRow;   // K bytes
  static constexpr int kV = F == kKvBf16 ? 0 : kK; // V^T bytes ([D or D/2][16] bytes)
  static constexpr int kBytes = kK + kV;
  static constexpr int kInst = kBytes / 1024;      // copy instructions
  static constexpr int CPR = kRow / 16;            // chunks per key row
  static_assert(CPR >= 2 && kBytes % 1024 == 0, "head dim");
  __device__ static int x(int r) { return CPR >= 8 ? (r & 7) : CPR == 4 ? ((r >> 1) & 3) : 0; }
  __device__ static int k_slot(int r, int c) { return r * CPR + (c ^ x(r)); }
  // source byte offset of the chunk that goes to slot s
  __device__ static int k_src(int s) {
    const int r = s / CPR;
    return r * kRow + 16 * ((s % CPR) ^ x(r));
  }
};
constexpr int kDecStages = 3;  // blocks per wave in rotation (one read, two in flight)
// Each of the three stage arrays holds one stage of every wave; after the
// loop the first two hold the waves' O^T tiles (half the waves each).
template <int D, int F, int NW>
constexpr int dec_stage_array_bytes() {
  constexpr int o = NW / 2 * D * 16 * 4;
  constexpr int st = NW * DecStage<D, F>::kBytes;
  return o > st ? o : st;
}

// bf16 V^T fragments straight from the pool into registers
template <int D, int F>
__device__ __forceinline__ void dec_load_v(DecFrags<D, F>& f, const DecArgs& a, int phys, int g,
                                           int col, int grp) {
  static_assert(F == kKvBf16, "code blocks are staged through LDS whole");
  const size_t hb = ((size_t)phys * a.Hkv + g) * (kBlockTokens * D);
  const bf16* vb = (const bf16*)a.pool.v + hb;
#pragma unroll
  for (int t = 0; t < D / 16; ++t)
    f.v[t] = *(const bf16x4*)(vb + (16 * t + col) * kBlockTokens + 4 * grp);
}

// u8 codes as fp16 operands: the fp16 value with bit pattern 0x6400 | c is
// exactly 1024 + c for a code c in 0..255 (unit spacing in [1024, 2048)), so
// one byte permute turns two codes into two biased fp16 values; the bias
// 1024 goes into the zero points.
constexpr float kU8Bias = 1024.f;
__device__ __forceinline__ uint32_t u8x2_biased(uint32_t w, uint32_t sel) {
  return __builtin_amdgcn_perm(0x64646464u, w, sel);  // selectors 4..7: the 0x64 bytes
}
__device__ __forceinline__ f16x8 u8x8_to_f16_biased(uint32_t w0, uint32_t w1) {
  typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4v;
  const u32x4v r = {u8x2_biased(w0, 0x04010400u), u8x2_biased(w0, 0x04030402u),
                    u8x2_biased(w1, 0x04010400u), u8x2_biased(w1, 0x04030402u)};
  return __builtin_bit_cast(f16x8, r);
}
__device__ __forceinline__ f16x4 u8x4_to_f16_biased(uint32_t w) {
  const u32x2 r = {u8x2_biased(w, 0x04010400u), u8x2_biased(w, 0x04030402u)};
  return __builtin_bit_cast(f16x4, r);
}

// u4 codes as fp16 operands: a code c in the high nibble of a byte under
// the byte 0x54 is the fp16 value 2^6 * (1 + 16c / 1024) = 64 + c exactly
// (unit spacing in [64, 128)); the bias 64 goes into the zero points.  A
// dword of 8 codes holds channels b (low nibble) and 4 + b (high) in byte b.
constexpr float kU4Bias = 64.f;
__device__ __forceinline__ uint32_t u4x2_biased(uint32_t hi_nibbles, uint32_t sel) {
  return __builtin_amdgcn_perm(0x54545454u, hi_nibbles, sel);
}
__device__ __forceinline__ f16x8 u4x8_to_f16_biased(uint32_t w) {
  typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4v;
  const uint32_t lo = (w << 4) & 0xF0F0F0F0u, hi = w & 0xF0F0F0F0u;
  const u32x4v r = {u4x2_biased(lo, 0x04010400u), u4x2_biased(lo, 0x04030402u),
                    u4x2_biased(hi, 0x04010400u), u4x2_biased(hi, 0x04030402u)};
  return __builtin_bit_cast(f16x8, r);
}
// the low (n = 0) or high (n = 1) nibbles of the 4 bytes, in byte order
__device__ __forceinline__ f16x4 u4x4_to_f16_biased(uint32_t w, int n) {
  const uint32_t x = (n ? w : w << 4) & 0xF0F0F0F0u;
  const u32x2 r = {u4x2_biased(x, 0x04010400u), u4x2_biased(x, 0x04030402u)};
  return __builtin_bit_cast(f16x4, r);
}

// Four-wave workgroups (several per CU) are held to at least three waves
// per SIMD: left to itself the compiler gives them up to 220 registers,
// which caps every format at two waves per SIMD however many workgroups
// there are.
template <int D, int F, int NW>
__global__ __launch_bounds__(NW * 64, NW == 4 ? 3 : 2) void attn_decode_kernel(DecArgs a) {
  constexpr bool Q = F != kKvBf16;  // codes with per-channel scale / zero point
  constexpr bool U4 = F == kKvU4;
  constexpr float kBias = U4 ? kU4Bias : kU8Bias;
  constexpr int NT = D / 16;  // 16-channel tiles of the output
  static_assert(NW == 4 || NW == 8, "waves per workgroup");
  __shared__ float sm_m[NW][16], sm_l[NW][16], sm_lv[NW][16];
  // Stage j of every wave's block rotation lives in its own array, so
  // the compiler can tell a wave's reads of one stage from the copies still
  // landing in the others (one array would make every read wait for all
  // copies).  After the loop st0 / st1 hold the waves' accumulators.
  constexpr int SZ = dec_stage_array_bytes<D, F, NW>();
  __shared__ __attribute__((aligned(16))) uint8_t st0[SZ];
  __shared__ __attribute__((aligned(16))) uint8_t st1[SZ];
  __shared__ __attribute__((aligned(16))) uint8_t st2[SZ];
  // wave w's O^T tile [D][16] floats, columns XOR-swizzled by row
  auto o_tile = [&](int w) { return (float*)(w < NW / 2 ? st0 : st1) + (w % (NW / 2)) * D * 16; };
  auto o_idx = [](int d, int hh) { return d * 16 + (hh ^ (d & 15)); };

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // partition index slowest: consecutive workgroups (which the dispatcher
  // deals round-robin to the 8 XCDs) are different (sequence, KV head)
  // pairs, so the first partitions -- the only ones short sequences have --
  // spread over every XCD instead of piling onto those whose index
  // matches a multiple of the partition count
  const int g = blockIdx.x, b = blockIdx.y, p = blockIdx.z;
  const int sidx = a.first_seq + b;
  const int n_rep = a.Hq / a.Hkv;
  const int col = lane & 15, grp = lane >> 4;
  const bool head_ok = col < n_rep;
  const int ctx = seq_ctx(a.seq, sidx);
  const int row = seq_row(a.seq, sidx);

  // query fragments (B operand of S^T = K Q^T): q[head col][channels of
  // dec_kchan], carried as a pair hi + lo so the fp32 query keeps its
  // precision (MFMA time is free here).  bf16 cache: bf16 pairs.  u8 / u4
  // cache: fp16 pairs of q' = q * k_scale * 2^e (the K scale folded in, 2^e
  // puts the head's largest |q'| in [128, 256) and comes back out through
  // the score scale); the codes enter as bias + c, so the zero point and
  // bias enter through corr = sum_d q'[d] * (bias + zp[d]) in fp32.
  using QT = typename std::conditional<Q, f16x8, bf16x8>::type;
  using PT = typename std::conditional<Q, f16x4, bf16x4>::type;
  QT qf[D / 32];
  QT qlo[D / 32];
  float corr = 0.f;
  float sc = kLog2e * rsqrtf((float)D);
  {
    const float* qp = a.q + ((size_t)row * a.Hq + g * n_rep + col) * D;
    float qv[D / 32][8];
    float amax = 0.f;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[s][e] = 0.f;
      if (head_ok) {
        const float* qs = qp + dec_kchan<D, F>(s, grp);
        const float4 x0 = *(const float4*)qs, x1 = *(const float4*)(qs + 4);
        qv[s][0] = x0.x; qv[s][1] = x0.y; qv[s][2] = x0.z; qv[s][3] = x0.w;
        qv[s][4] = x1.x; qv[s][5] = x1.y; qv[s][6] = x1.z; qv[s][7] = x1.w;
      }
      if constexpr (Q) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          qv[s][e] *= a.pool.k_scale[g * D + dec_kchan<D, F>(s, grp) + e];
          amax = fmaxf(amax, fabsf(qv[s][e]));
        }
      }
    }
    float qscale = 1.f;
    if constexpr (Q) {
      amax = max_xor32(max_xor16(amax));
      int ex = 0;
      frexpf(amax, &ex);  // amax = f * 2^ex, f in [0.5, 1); ex = 0 for amax 0
      const int sh = min(100, max(-100, 8 - ex));
      qscale = ldexpf(1.f, sh);
      sc = ldexpf(sc, -sh);
    }
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      QT hi, lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float qs = qv[s][e] * qscale;
        if constexpr (Q) {
          corr += qs * (kBias + (float)a.pool.k_zp[g * D + dec_kchan<D, F>(s, grp) + e]);
          hi[e] = (_Float16)qs;
          lo[e] = (_Float16)(qs - (float)hi[e]);
        } else {
          hi[e] = f32_to_bf16(qs);
          lo[e] = f32_to_bf16(qs - (float)hi[e]);
        }
      }
      qf[s] = hi;
      qlo[s] = lo;
    }
    if constexpr (Q) {
      corr = sum_xor32(sum_xor16(corr));
    }
  }

  // the sequence's context is cut into n_parts partitions of (nearly) equal
  // size, at most part_blocks blocks each (a context beyond the host bound
  // is cut to it: wrong output, but no access outside the workspace or the
  // block table)
  const int n_blk = dec_blocks(a, ctx);
  const int n_keys = min(ctx + 1, n_blk * kBlockTokens);
  const int n_parts = cdiv(n_blk, a.part_blocks);
  if (p >= n_parts) return;
  const int part_size = cdiv(n_blk, n_parts);
  const int blk0 = p * part_size;
  const int blk1 = min(n_blk, blk0 + part_size);

  f32x4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  // per-block x per-channel caches: sum of P 2^eV (the weight of the V zero
  // point, P entering the V product scaled by its block's factor)
  float lv_run = 0.f;

  // this wave's blocks: blk0 + wave + NW i, i < cnt <= 128; the table
  // entries come in two loads (entry i in lane i % 64 of my_phys[i / 64])
  const int cnt = blk1 - blk0 > wave ? cdiv(blk1 - blk0 - wave, NW) : 0;
  int my_phys[2] = {0, 0};
#pragma unroll
  for (int h = 0; h < 2; ++h)
    if (64 * h + lane < cnt) my_phys[h] = seq_block(a.seq, sidx, blk0 + wave + NW * (64 * h + lane));

  // ex: the block's factor exponents (eK in the low byte, eV in the high;
  // 0 without block scales), P <= 2^kLazy times 2^eV <= 2^7 stays in the fp16
  // range
  auto compute = [&](const DecFrags<D, F>& f, int i, int ex) {
    const int blk = blk0 + wave + NW * i;
    const float sck = Q ? ldexpf(sc, (int8_t)(ex & 0xff)) : sc;
    const float fvb = Q ? ldexpf(1.f, (int8_t)(ex >> 8)) : 1.f;
    // S^T[key][head]: A = K rows (key = lane%16), B = Q^T (hi + lo, two
    // independent accumulation chains)
    f32x4 st = f32x4{0.f, 0.f, 0.f, 0.f}, st_lo = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      QT kf;
      if constexpr (U4) {
        kf = u4x8_to_f16_biased(reinterpret_cast<const uint32_t*>(&f.k[0])[s]);
      } else if constexpr (Q) {
        const uint4 w = f.k[s >> 1];
        kf = (s & 1) ? u8x8_to_f16_biased(w.z, w.w) : u8x8_to_f16_biased(w.x, w.y);
      } else {
        kf = f.k[s];
      }
      st = mfma16x16x32(kf, qf[s], st);
      st_lo = mfma16x16x32(kf, qlo[s], st_lo);
    }
    st += st_lo;
    // lane holds S[head col][key 4grp + r]; only the sequence's last block
    // has unwritten slots (wave-uniform test)
    const int key0 = blk * kBlockTokens + 4 * grp;
    const bool partial = (blk + 1) * kBlockTokens > n_keys;
    float sv[4];
    float mb = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sv[r] = (st[r] - corr) * sck;
      mb = fmaxf(mb, sv[r]);
    }
    if (partial) {
      mb = -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (key0 + r >= n_keys) sv[r] = -INFINITY;
        mb = fmaxf(mb, sv[r]);
      }
    }
    mb = max_xor32(max_xor16(mb));
    // the reference point of the exponentials moves (and the accumulators
    // are rescaled) only when a block's maximum exceeds it by more than
    // kLazy: P <= 2^kLazy keeps its hi + lo pair exact enough, softmax
    // does not depend on the reference point
    if (__builtin_amdgcn_ballot_w64(mb > m_run + kLazy) != 0) {
      const float m_new = fmaxf(m_run, mb);
      const float alpha = exp2f(m_run - m_new);  // 0 on the first block
      m_run = m_new;
      l_run *= alpha;
      lv_run *= alpha;
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t] *= alpha;
    }
    // bf16 cache: P as a pair hi + lo of bf16 (the weights keep fp32
    // precision).  Code caches: P rounded once to fp16 (2^-12 relative), and
    // the denominators summed from the same rounded values, so that the
    // bias + zero point taken out at the end cancels what the products put
    // in up to fp32 rounding (one MFMA per tile instead of two: these
    // kernels are bound by the per-block chain, not by bytes)
    PT pf, pl;
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float pv = exp2f(sv[r] - m_run);
      if constexpr (Q) {
        const _Float16 ph = (_Float16)pv;
        pf[r] = (_Float16)((float)ph * fvb);  // exact: a power of two (P <= 2^8, 2^eV <= 2^7)
        psum += (float)ph;
      } else {
        pf[r] = f32_to_bf16(pv);
        pl[r] = f32_to_bf16(pv - (float)pf[r]);
        psum += pv;
      }
    }
    l_run += psum;
    lv_run += psum * fvb;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      PT vf;
      if constexpr (U4) {
        vf = u4x4_to_f16_biased(f.v[t >> 1], t & 1);  // finite, so P = 0 cancels unwritten slots
      } else if constexpr (Q) {
        vf = u8x4_to_f16_biased(f.v[t]);  // finite, so P = 0 cancels unwritten slots
      } else {
        vf = f.v[t];
        if (partial) {  // unwritten slots of the last block may hold any bits: zero V
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (key0 + r >= n_keys) vf[r] = (bf16)0.f;
        }
      }
      acc[t] = mfma16x16x16(vf, pf, acc[t]);
      if constexpr (!Q) acc[t] = mfma16x16x16(vf, pl, acc[t]);
    }
  };

  // Loads past the wave's last block repeat that block (valid addresses)
  // and are never computed.  The explicit waits count this wave's
  // vector-memory operations in program order; the scheduling barriers keep
  // the compiler from moving loads or their uses across them.
  {
    // K (and u8 / u4 V) blocks go to LDS as whole cache lines (16 bytes per lane,
    // 1 KB per instruction; kDecStages blocks per wave in rotation) and the
    // fragments are read back from there.  Read in place as register
    // fragments, K would cost 2-4x the cache-line requests (a fragment load
    // takes 32-64 bytes of each of 16 key rows), and requests, not bytes,
    // bound this kernel.
    using St = DecStage<D, F>;
    constexpr int NB = kDecStages;
    // (u8 / u4: plus one 2-byte load of the block's factor exponents, from a
    // dummy address without block scales, so that every path counts alike)
    constexpr int LOADS = St::kInst + (Q ? 1 : D / 16);
    constexpr int kWaitIn = (NB - 2) * LOADS;  // blocks i+1 .. i+NB-2 may be in flight
    constexpr int kWait = (kWaitIn & 15) | (7 << 4) | (15 << 8) | (((kWaitIn >> 4) & 3) << 14);
    static_assert(NB == 3, "one LDS array per stage");
    auto stage = [&](int j) { return (j == 0 ? st0 : j == 1 ? st1 : st2) + wave * St::kBytes; };
    DecFrags<D, F> fv[Q ? 1 : NB];  // bf16: V^T register sets in rotation
    int exr[NB] = {0, 0, 0};        // u8 / u4: the blocks' exponents in rotation
    const bool has_exp = a.pool.exps != nullptr;
    if (cnt > 0) {
      auto phys_of = [&](int i) {
        i = min(i, cnt - 1);  // wave-uniform
        return __shfl(i < 64 ? my_phys[0] : my_phys[1], i & 63, 64);
      };
      auto issue = [&](int i, int buf) {
        const int phys = phys_of(i);
        const size_t hb = ((size_t)phys * a.Hkv + g) * (kBlockTokens * St::kRow);
        const uint8_t* kb = (const uint8_t*)a.pool.k + hb;
        const uint8_t* vb = (const uint8_t*)a.pool.v + hb;  // V^T tile, same size (codes)
        uint8_t* kd = stage(buf);
        // stage byte o = 1024j + 16 lane comes from K (swizzled) while o <
        // kK, then from V^T in order (u4 with D = 64: both in one copy)
#pragma unroll
        for (int j = 0; j < St::kInst; ++j) {
          const int o = 1024 * j + 16 * lane;
          const bool in_k = St::kK % 1024 == 0 ? 1024 * j < St::kK : o < St::kK;
          const uint8_t* src = in_k ? kb + St::k_src(o / 16) : vb + (o - St::kK);
          __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(kd + 1024 * j), 16, 0, 0);
        }
        if constexpr (!Q) dec_load_v<D, F>(fv[buf], a, phys, g, col, grp);
        if constexpr (Q) {
          const uint16_t* ep = has_exp ? (const uint16_t*)(a.pool.exps + ((size_t)phys * a.Hkv + g) * 2)
                                       : (const uint16_t*)a.pool.k_zp;
          exr[buf] = *ep;
        }
      };
#pragma unroll
      for (int j = 0; j < NB - 1; ++j) issue(j, j);
      for (int i = 0; i < cnt; i += NB) {
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          __builtin_amdgcn_sched_barrier(0);
          __builtin_amdgcn_s_waitcnt(kWait);
          __builtin_amdgcn_sched_barrier(0);
          issue(i + j + NB - 1, (j + NB - 1) % NB);
          __builtin_amdgcn_sched_barrier(0);
          if (j == 0 || i + j < cnt) {
            const uint8_t* kd = stage(j);
            DecFrags<D, F> f;
            using KT = typename DecFrags<D, F>::KT;
            if constexpr (St::CPR == 2) {  // u4, D = 64: 8 bytes of the 32-byte row
              f.k[0] = *(const KT*)(kd + col * St::kRow + 8 * grp);
            } else {
#pragma unroll
              for (int h = 0; h < St::kRow / 64; ++h)
                f.k[h] = *(const KT*)(kd + St::k_slot(col, 4 * h + grp) * 16);
            }
            if constexpr (Q) {
#pragma unroll
              for (int t = 0; t < (U4 ? D / 32 : D / 16); ++t)
                f.v[t] = *(const uint32_t*)(kd + St::kK + (16 * t + col) * 16 + 4 * grp);
            } else {
#pragma unroll
              for (int t = 0; t < D / 16; ++t) f.v[t] = fv[j].v[t];
            }
            compute(f, i + j, Q && has_exp ? exr[j] : 0);
          }
        }
      }
      __builtin_amdgcn_s_waitcnt(0);  // the last (unused) copies land before LDS is reused
    }
    __syncthreads();  // every wave is done with its stages before they take the accumulators
  }

  // ---- merge the waves: acc[t][r] = O^T[dec_vchan(t, 4grp + r)][head col]
  l_run = sum_xor32(sum_xor16(l_run));
  lv_run = sum_xor32(sum_xor16(lv_run));
  if (lane < 16) {
    sm_m[wave][lane] = m_run;
    sm_l[wave][lane] = l_run;
    sm_lv[wave][lane] = lv_run;
  }
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) o_tile(wave)[o_idx(dec_vchan<F>(t, 4 * grp + r), col)] = acc[t][r];
  __syncthreads();

  float* pp = a.part + (((size_t)b * a.Hkv + g) * a.max_parts + p) * kPartStride(D);
  for (int e = tid; e < 16 * D; e += NW * 64) {
    const int hh = e / D, d = e % D;
    if (hh >= n_rep) continue;
    float M = sm_m[0][hh];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, sm_m[w][hh]);
    float O = 0.f, L = 0.f, Lv = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = exp2f(sm_m[w][hh] - M);  // 0 for a wave with no blocks
      O += o_tile(w)[o_idx(d, hh)] * f;
      L += sm_l[w][hh] * f;
      Lv += sm_lv[w][hh] * f;
    }
    if constexpr (Q) {  // O = sum P 2^eV (bias + c): take out sum P 2^eV (bias + zp)
      const int ch = g * D + d;
      O = a.pool.v_scale[ch] * (O - (kBias + (float)a.pool.v_zp[ch]) * Lv);
    }
    if (n_parts == 1) {
      a.o[(size_t)row * a.Hq * D + (size_t)(g * n_rep + hh) * D + d] = to_f16(O / L);
    } else {
      pp[hh * D + d] = O;
      if (d == 0) {
        pp[16 * D + 2 * hh] = M;
        pp[16 * D + 2 * hh + 1] = L;
      }
    }
  }
}

// Merges the context partitions of sequences with more than one: one
// workgroup per (sequence, KV head).  The per-(partition, head) weights
// exp2(m_p - M) / L come first (LDS), then every output element sums its
// partitions with independent loads.
constexpr int kMaxDecodeParts = 256;
constexpr int kMaxPartBlocks = 512;  // two block-table entries per lane and wave

template <int D>
__global__ __launch_bounds__(256) void attn_decode_merge_kernel(DecArgs a) {
  __shared__ float sw[kMaxDecodeParts][16];  // m, then the partition weight
  __shared__ float sl[kMaxDecodeParts][16];
  const int g = blockIdx.x, b = blockIdx.y;
  const int sidx = a.first_seq + b;
  const int n_rep = a.Hq / a.Hkv;
  const int n_blk = dec_blocks(a, seq_ctx(a.seq, sidx));
  const int n_parts = cdiv(n_blk, a.part_blocks);
  if (n_parts <= 1) return;
  const int row = seq_row(a.seq, sidx);
  const float* base = a.part + ((size_t)b * a.Hkv + g) * a.max_parts * kPartStride(D);
  for (int e = threadIdx.x; e < n_parts * 16; e += 256) {
    const int q = e / 16, hh = e % 16;
    if (hh < n_rep) {
      sw[q][hh] = base[q * kPartStride(D) + 16 * D + 2 * hh];
      sl[q][hh] = base[q * kPartStride(D) + 16 * D + 2 * hh + 1];
    }
  }
  __syncthreads();
  if (threadIdx.x < n_rep) {
    const int hh = threadIdx.x;
    float M = -INFINITY;
    for (int q = 0; q < n_parts; ++q) M = fmaxf(M, sw[q][hh]);
    float L = 0.f;
    for (int q = 0; q < n_parts; ++q) L += sl[q][hh] * exp2f(sw[q][hh] - M);
    const float inv = 1.f / L;
    for (int q = 0; q < n_parts; ++q) sw[q][hh] = exp2f(sw[q][hh] - M) * inv;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < n_rep * D; e += 256) {
    const int hh = e / D;
    float O = 0.f;
    int q = 0;
    for (; q + 4 <= n_parts; q += 4) {
      const float o0 = base[(q + 0) * kPartStride(D) + e], o1 = base[(q + 1) * kPartStride(D) + e];
      const float o2 = base[(q + 2) * kPartStride(D) + e], o3 = base[(q + 3) * kPartStride(D) + e];
      O += o0 * sw[q][hh];
      O += o1 * sw[q + 1][hh];
      O += o2 * sw[q + 2][hh];
      O += o3 * sw[q + 3][hh];
    }
    for (; q < n_parts; ++q) O += base[q * kPartStride(D) + e] * sw[q][hh];
    a.o[(size_t)row * a.Hq * D + (size_t)g * n_rep * D + e] = to_f16(O);
  }
}

}  // namespace

DecodePlan decode_plan(int batch, int Hq, int Hkv, int D, int max_ctx_len, int fmt) {
  (void)Hq;
  DecodePlan pl{};
  const int max_blk = cdiv(max_ctx_len, kBlockTokens);
  // Parts per sequence (for the longest one; each sequence is cut into
  // near-equal parts of at most part_blocks blocks).  Measured on ragged
  // batches: enough (sequence, KV head) pairs x parts for one workgroup per
  // CU, and no part above ~2 MB of cache (257 bf16 / 171 u8 or u4 blocks
  // of a 128-wide head; code blocks cost more compute per byte, and u4
  // timings hardly move between 128 and 257); more, shorter parts only add
  // workgroup start-up, partial writes and the merge.
  const int pairs = batch * Hkv;
  const int cap = std::min(kMaxPartBlocks, (fmt == kKvBf16 ? 257 : 171) * 128 / D);
  int parts = std::max(cdiv(256, pairs), cdiv(max_blk, cap));
  parts = std::max(1, std::min(parts, max_blk));
  int pb = cdiv(max_blk, parts);
  while (cdiv(max_blk, pb) > kMaxDecodeParts) ++pb;  // the merge kernel's LDS bound
  pl.part_blocks = pb;
  pl.max_parts = cdiv(max_blk, pb);
  pl.part_floats = pl.max_parts > 1 ? (size_t)batch * Hkv * pl.max_parts * kPartStride(D) : 0;
  // parts never falls as max_ctx_len grows and max_parts <= parts: this
  // bounds part_floats for every shorter context at this batch size
  pl.part_floats_bound = (size_t)batch * Hkv * parts * kPartStride(D);
  return pl;
}

hipError_t attn_decode(const DecodePlan& pl, const void* q, KvPool pool, SeqInfo seq, int first_seq,
                       int batch, int Hq, int Hkv, int D, void* o, float* part, hipStream_t s) {
  if (batch == 0) return hipSuccess;
  if (pl.part_blocks > kMaxPartBlocks) return hipErrorInvalidValue;
  DecArgs a{(const float*)q, pool, seq, first_seq, Hq, Hkv, pl.part_blocks, pl.max_parts, part,
            (f16*)o};
  dim3 grid(Hkv, batch, pl.max_parts);
  // at most one workgroup per CU: eight waves per workgroup (twice the
  // blocks in flight for each (sequence, KV head); the longest sequence sets
  // the time); otherwise four (two workgroups per CU)
  const bool wide = (size_t)Hkv * batch * pl.max_parts <= 256;
#define TDL_DECODE_CASE(DD, FF)                                                   \
  if (D == DD && pool.fmt == FF) {                                                \
    if (wide) attn_decode_kernel<DD, FF, 8><<<grid, 512, 0, s>>>(a);              \
    else attn_decode_kernel<DD, FF, 4><<<grid, 256, 0, s>>>(a);                   \
  }
  TDL_DECODE_CASE(128, kKvBf16) TDL_DECODE_CASE(128, kKvU8) TDL_DECODE_CASE(128, kKvU4)
  TDL_DECODE_CASE(64, kKvBf16) TDL_DECODE_CASE(64, kKvU8) TDL_DECODE_CASE(64, kKvU4)
#undef TDL_DECODE_CASE
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.max_parts == 1) return e;
  dim3 mgrid(Hkv, batch);
  if (D == 128) attn_decode_merge_kernel<128><<<mgrid, 256, 0, s>>>(a);
  else attn_decode_merge_kernel<64><<<mgrid, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace tdl
