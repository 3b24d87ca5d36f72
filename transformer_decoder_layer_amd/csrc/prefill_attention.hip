// Causal grouped-query flash attention for prefill rows (gfx950).
//
// A workgroup owns one KV head g and 32 query positions of one sequence,
// with one wave per query head of the group, or of a part of the group (the
// group of a KV head is split over several workgroups when that is needed to
// fill the chip):
// each 32-key K/V tile sits in LDS once and feeds every head that shares it,
// so no repeat_kv copy is made (the Qwen2.5-7B single-layer page, section 3, expands the 4 KV
// heads to 28; here the expansion is only an index).  Both products run on
// 32x32x16 fp16 MFMAs: S^T = K Q^T (keys as rows, so a query's scores sit in
// one lane pair) and O^T = V^T P^T, whose B operand is exactly the register
// layout the first product leaves P in.  Softmax is the online form of the
// TFFInfer page, section 3.7.2 item 5 (running max, denominator, rescaled
// accumulator), written per tile, with scores scaled by log2(e)/sqrt(D) so
// exp2 gives e^(s - m).
//
// Keys come from two places:
//  * the call's own new tokens ("chunk"), for the first kStagedSeqs prefill
//    sequences: the RoPE kernel stages their K and V once as fp16 in this
//    kernel's tile layout (prefill_stage_* below), so a tile is two
//    contiguous 8 KB pieces that go straight from memory into LDS with
//    global_load_lds (no registers, no conversion); four LDS stages, tiles
//    issued three ahead, and each tile's Q K^T is computed one tile early so
//    its MFMAs overlap the previous tile's softmax in the same wave;
//  * the paged cache (the tokens before the chunk, and the chunk itself for
//    sequences past kStagedSeqs): blocks gathered through the block table
//    into registers, converted to fp16 (bf16 exactly; u8 / u4 codes
//    dequantised as (c - zero_point) * scale, the page's formula in the
//    devpress engine article, section 2.6, times the block's factor 2^e in
//    per-block x per-channel caches) and stored to LDS.
// Either way the LDS tile holds the values the cache holds, rounded once to
// fp16 (exact for bf16 inside the fp16 range).

#include "common.h"
#include "kernels.h"

namespace tdl {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 8.f;  // slack of the running maximum (log2 units)
constexpr int PQ = 32;        // queries per workgroup (one MFMA column block)
constexpr int PK = 32;        // keys per tile (one MFMA row block)
constexpr int NB = PK / 16;   // 16-token blocks per tile

typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// max and sum of a lane's 16 values as trees: the max in three-input steps
// (v_max3, 3 dependent instructions, not 8), the sum in 4 dependent adds
__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }
__device__ __forceinline__ float max16(const float (&v)[16]) {
  float m[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) m[i] = max3f(v[3 * i], v[3 * i + 1], v[3 * i + 2]);
  return fmaxf(max3f(m[0], m[1], m[2]), max3f(m[3], m[4], v[15]));
}
__device__ __forceinline__ float sum16(const float (&v)[16]) {
  float m[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) m[i] = v[2 * i] + v[2 * i + 1];
#pragma unroll
  for (int w = 4; w >= 1; w /= 2)
#pragma unroll
    for (int i = 0; i < w; ++i) m[i] += m[i + w];
  return m[0];
}

// ------------------------------------------------------------ tile layout
// One LDS tile: K [PK keys][D] fp16 at prefill_k_index, then V at kK +
// prefill_v_index: the staging copy's layout, so that a tile is a straight
// copy of PK staged rows.
template <int D>
struct Tile {
  static constexpr int kK = PK * D;  // fp16 elements of K
  static constexpr int kElems = 2 * PK * D;
  static constexpr int kBytes = 2 * kElems;
  static constexpr int kInst = kBytes / 1024;  // 1 KB direct copies per tile
};
template <int D>
__device__ __forceinline__ int k_at(int key, int chunk) {
  return key * D + ((chunk ^ prefill_k_swz(key, D)) << 3);
}
template <int D>
__device__ __forceinline__ int v_at(int key, int d) {
  return Tile<D>::kK + prefill_v_index(key, d, D);
}

// ------------------------------------------------------- sequence lookups
__device__ __forceinline__ int p_row(const SeqInfo& s, int i) { return s.q_start ? s.q_start[i] : 0; }
__device__ __forceinline__ int p_qlen(const SeqInfo& s, int i) { return s.q_start ? s.q_len[i] : s.q_len0; }
__device__ __forceinline__ int p_ctx(const SeqInfo& s, int i) { return s.q_start ? s.ctx_len[i] : s.ctx0; }

struct PrefillArgs {
  const float* q;  // [rows][Hq][D] fp32, after RoPE (unless qs.qkv)
  PrefillQ qs;     // queries from the QKV projection, finished on load
  KvPool pool;
  SeqInfo seq;
  PrefillStage st;
  int Hq, Hkv;
  int n_rep;    // query heads per KV head
  int n_split;  // workgroups per (KV head, query tile): n_rep / NH rounded up
  int n_qtiles;
  int paired;
  f16* o;  // [rows][Hq * D]
};

// ------------------------------------------------------------ the kernel
// One wave per query head: NH heads of one KV head's group per workgroup.
// When the group is split over n_split workgroups, the last one may have
// fewer heads than waves; its spare waves repeat its last head (computed,
// never stored) and still share the copies.
//
// KS = 2 (short prompts, where the grid leaves CUs idle and the longest
// query tile's key loop sets the time): two key groups of NH waves each take
// half of the staged key tiles of the same query tile and heads, in
// lockstep (the workgroup's barriers are shared; the group with fewer tiles
// repeats a copy and skips the products), and group 1's running maximum,
// denominator and accumulators are merged into group 0's through LDS at the
// end.  Keys from the paged cache are converted by all threads and taken by
// group 0 alone.
// (Four waves of one key group: at most 256 registers each, so that two
// workgroups share a CU and each SIMD has two waves to switch between --
// Qwen3-8B's 2048-token chunk 67 -> 63 us, against a few spills; two key
// groups of two heads need more registers than that.)
template <int D, int NH, int F, int KS>
__global__ __launch_bounds__(NH * KS * 64, KS == 1 && NH == 4 ? 2 : 1) void attn_prefill_kernel(PrefillArgs a) {
  using T = Tile<D>;
  static_assert(KS == 1 || KS == 2, "key groups");
  constexpr int NW = NH;  // waves per key group
  constexpr int NT = NH * KS * 64;
  // four stages, each its own array so that the compiler can tell a copy
  // landing in one stage from reads of another (key group k uses elements
  // k * kElems of each)
  __shared__ __attribute__((aligned(16))) f16 s0[KS * T::kElems];
  __shared__ __attribute__((aligned(16))) f16 s1[KS * T::kElems];
  __shared__ __attribute__((aligned(16))) f16 s2[KS * T::kElems];
  __shared__ __attribute__((aligned(16))) f16 s3[KS * T::kElems];
  // u8 / u4 caches: this KV head's per-channel scale and zero point of K and V
  __shared__ float dq[4][D];

  const int tid = threadIdx.x, lane = tid & 63;
  // key group and head wave within it (compile-time 0 and tid / 64 for one
  // key group, so that each stage pointer stays a known array)
  const int kg = KS == 1 ? 0 : (tid >> 6) / NH;
  const int wave = KS == 1 ? tid >> 6 : (tid >> 6) % NH;
  // (query tile slot x, KV head g) from the flat workgroup index.  The
  // dispatcher deals workgroups round-robin to the 8 XCDs (each with its own
  // L2): when the head count divides 8, each XCD takes whole heads, so an
  // L2 holds the K/V of 8 / Hkv heads at most instead of all of them.
  const int sidx = blockIdx.z;
  int g, xslot, head0;
  {
    const int U = a.Hkv * a.n_split;  // (KV head, part of its group) units
    const int L = blockIdx.x, nx = (int)gridDim.x / U;
    int u;
    if (8 % U == 0 && (nx * U) % 8 == 0) {
      const int xcd = L & 7, j = L >> 3;
      u = xcd % U;
      xslot = xcd / U + (8 / U) * j;
    } else {
      u = L / nx;
      xslot = L % nx;
    }
    g = u / a.n_split;
    head0 = (u % a.n_split) * NH;
  }
  const bool own = head0 + wave < a.n_rep;
  const int h = g * a.n_rep + min(head0 + wave, a.n_rep - 1);
  const int ql = lane & 31, G = lane >> 5;
  const int q_len = p_qlen(a.seq, sidx);
  const int ctx = p_ctx(a.seq, sidx);
  const int nq_seq = cdiv(q_len, PQ);
  const bool staged = sidx < a.st.n_seqs;
  // keys read from the paged cache: the context, plus the chunk itself when
  // this sequence has no staged copy
  const int n_pool_keys = staged ? ctx : ctx + q_len;
  const float sc = kLog2e * rsqrtf((float)D);
  const int* tab = a.seq.tables + (size_t)sidx * a.seq.max_blocks;  // never null here
  constexpr int fmt = F;  // the cache's element format
  if (fmt != kKvBf16) {  // read before the first barrier of the item loop
    for (int i = tid; i < D; i += NT) {
      dq[0][i] = a.pool.k_scale[g * D + i];
      dq[1][i] = (float)a.pool.k_zp[g * D + i];
      dq[2][i] = a.pool.v_scale[g * D + i];
      dq[3][i] = (float)a.pool.v_zp[g * D + i];
    }
  }

  const int n_items = a.paired ? 2 : 1;
  for (int item = 0; item < n_items; ++item) {
    int qt;
    if (a.paired) {
      qt = item == 0 ? xslot : a.n_qtiles - 1 - xslot;
      if (item == 1 && qt == xslot) break;  // odd count: the middle tile once
    } else {
      qt = a.n_qtiles - 1 - xslot;  // longest first
    }
    if (qt >= nq_seq) continue;  // uniform over the workgroup
    const int row0 = p_row(a.seq, sidx) + qt * PQ;
    const int q_lo = qt * PQ;                      // chunk-local query index of lane 0
    const int q_hi = min(q_lo + PQ, q_len) - 1;    // last valid chunk-local query
    const int my_q = q_lo + ql;                    // chunk-local query of this lane

    // Q fragments (B operand of S^T = K Q^T): q[my_q][16s + 8G .. +7] * sc
    f16x8 qf[D / 16];
    if (a.qs.qkv) {
      // from the QKV projection: bias, Q-norm over the head (this lane holds
      // half its channels, lane ^ 32 the other half) and RoPE, whose pairs
      // (c, c + D/2) sit in steps s and s + D/32 of the same lane
      const bool valid = my_q < q_len;
      float xv[D / 16][8];
      const float* src = a.qs.qkv + (size_t)(row0 + ql) * a.qs.ldq + (size_t)h * D + 8 * G;
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        if (valid) {
          const float4 x0 = *(const float4*)(src + 16 * s), x1 = *(const float4*)(src + 16 * s + 4);
          xv[s][0] = x0.x; xv[s][1] = x0.y; xv[s][2] = x0.z; xv[s][3] = x0.w;
          xv[s][4] = x1.x; xv[s][5] = x1.y; xv[s][6] = x1.z; xv[s][7] = x1.w;
          if (a.qs.bias) {
#pragma unroll
            for (int e = 0; e < 8; ++e) xv[s][e] += a.qs.bias[h * D + 16 * s + 8 * G + e];
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) xv[s][e] = 0.f;
        }
      }
      if (a.qs.norm) {
        float ss = 0.f;
#pragma unroll
        for (int s = 0; s < D / 16; ++s)
#pragma unroll
          for (int e = 0; e < 8; ++e) ss += xv[s][e] * xv[s][e];
        ss = sum_xor32(ss);
        const float inv = rsqrtf(ss / (float)D + a.qs.eps);
#pragma unroll
        for (int s = 0; s < D / 16; ++s)
#pragma unroll
          for (int e = 0; e < 8; ++e) xv[s][e] = xv[s][e] * inv * a.qs.norm[16 * s + 8 * G + e];
      }
      const float2* cs = a.qs.rope + (size_t)(ctx + min(my_q, q_len - 1)) * (D / 2) + 8 * G;
#pragma unroll
      for (int s = 0; s < D / 32; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float2 c = cs[16 * s + e];
          const float x1 = xv[s][e], x2 = xv[s + D / 32][e];
          xv[s][e] = x1 * c.x - x2 * c.y;
          xv[s + D / 32][e] = x1 * c.y + x2 * c.x;
        }
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        f16x8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = f32_to_f16_sat(xv[s][e] * sc);
        qf[s] = v;
      }
    } else {
      const bool valid = my_q < q_len;
      const float* qp = a.q + ((size_t)(row0 + ql) * a.Hq + h) * D + 8 * G;
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        f16x8 v{};
        if (valid) {
          const float4 x0 = *(const float4*)(qp + 16 * s), x1 = *(const float4*)(qp + 16 * s + 4);
          v[0] = f32_to_f16_sat(x0.x * sc); v[1] = f32_to_f16_sat(x0.y * sc);
          v[2] = f32_to_f16_sat(x0.z * sc); v[3] = f32_to_f16_sat(x0.w * sc);
          v[4] = f32_to_f16_sat(x1.x * sc); v[5] = f32_to_f16_sat(x1.y * sc);
          v[6] = f32_to_f16_sat(x1.z * sc); v[7] = f32_to_f16_sat(x1.w * sc);
        }
        qf[s] = v;
      }
    }

    f32x16 acc[D / 32];
#pragma unroll
    for (int t = 0; t < D / 32; ++t) acc[t] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;

    // S^T of one tile (32 keys x 32 queries), one accumulation chain over
    // the D/16 channel steps
    auto qk = [&](const f16* tile) {
      f32x16 e{};
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        const f16x8 kf = *(const f16x8*)(tile + k_at<D>(ql, 2 * s + G));
        e = mfma32(kf, qf[s], e);
      }
      return e;
    };
    // keys past `lim` (this lane's last visible key, tile-relative; a lane
    // holds keys 8(r/4) + 4G + r%4) get -inf
    auto mask = [&](f32x16& st, int lim) {
      const int l4 = lim - 4 * G;
#pragma unroll
      for (int r = 0; r < 16; ++r) st[r] = 8 * (r >> 2) + (r & 3) > l4 ? -INFINITY : st[r];
    };
    // online-softmax update, without a branch: the reference point m moves
    // only when some row's maximum passes it by more than kLazy (P stays
    // below 2^kLazy), alpha = 2^(m_old - m_new) is 1 unless it moved, and the
    // accumulators take alpha afterwards (rescale).  Returns whether it
    // moved (wave-uniform) and P (fp16) in the B-operand layout of
    // O^T += V^T P^T.
    auto softmax = [&](const f32x16& st, f16x8 (&pb)[2], float& alpha) {
      float sv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) sv[r] = st[r];
      const float mt = max_xor32(max16(sv));
      const bool mv = __builtin_amdgcn_ballot_w64(mt > m_run + kLazy) != 0;
      const float m_new = mv ? fmaxf(m_run, mt) : m_run;
      alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 1 if unmoved, 0 on the first tile
      m_run = m_new;
      float pv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        pv[r] = __builtin_amdgcn_exp2f(sv[r] - m_new);  // 0 where masked
        pb[r >> 3][r & 7] = (f16)pv[r];
      }
      l_run = l_run * alpha + sum16(pv);
      return mv;
    };
    auto rescale = [&](bool moved, float alpha) {
      if (moved) {
#pragma unroll
        for (int t = 0; t < D / 32; ++t) acc[t] *= alpha;
      }
    };
    // O^T += V^T P^T, 16 keys per MFMA
    auto pv = [&](const f16* tile, const f16x8 (&pb)[2]) {
#pragma unroll
      for (int kc = 0; kc < NB; ++kc)
#pragma unroll
        for (int t = 0; t < D / 32; ++t) {
          const f16x8 vf = *(const f16x8*)(tile + T::kK + kc * 16 * D + (G * D + 32 * t + ql) * 8);
          acc[t] = mfma32(vf, pb[kc], acc[t]);
        }
    };
    // one whole tile: scores, mask, softmax, P V (no overlap)
    auto plain_tile = [&](const f16* tile, bool masked, int lim) {
      f32x16 st = qk(tile);
      if (masked) mask(st, lim);
      f16x8 pb[2];
      float alpha;
      const bool mv = softmax(st, pb, alpha);
      rescale(mv, alpha);
      pv(tile, pb);
    };

    // ------------------------------------------------ keys from the cache
    // positions 0 .. n_pool_keys-1, as far as this query tile sees them
    const int last_pos = ctx + q_hi;
    const int n_pool_tiles = cdiv(min(n_pool_keys, last_pos + 1), PK);
    __syncthreads();  // the previous item's last tile may still be read
    if (n_pool_tiles > 0) {
      // 16-byte source chunks of one tile (NB block-heads of K, then of V)
      constexpr int ebits = fmt == kKvBf16 ? 16 : fmt == kKvU8 ? 8 : 4;
      constexpr int cpb = 16 * D * ebits / 8 / 16;  // chunks per block-head (K or V)
      constexpr int nchunks = 2 * NB * cpb;
      constexpr int MAXC = (nchunks + NT - 1) / NT;
      uint4 rc[MAXC];
      int ph0, ph1;  // physical blocks of the tile (selected, never indexed)
      // per-block x per-channel caches: the two blocks' factors 2^e of the
      // K and V scales (1 otherwise)
      float fk0 = 1.f, fk1 = 1.f, fv0 = 1.f, fv1 = 1.f;
      static_assert(NB == 2, "two blocks per tile");
      auto load_table = [&](int t) {
        auto entry = [&](int b) {
          const int lblk = t * NB + b;
          return tab[lblk * kBlockTokens < n_pool_keys ? lblk : 0];
        };
        ph0 = entry(0);
        ph1 = entry(1);
        if constexpr (fmt != kKvBf16) {
          if (a.pool.exps) {
            const int8_t* e0 = a.pool.exps + ((size_t)ph0 * a.Hkv + g) * 2;
            const int8_t* e1 = a.pool.exps + ((size_t)ph1 * a.Hkv + g) * 2;
            fk0 = ldexpf(1.f, e0[0]);
            fv0 = ldexpf(1.f, e0[1]);
            fk1 = ldexpf(1.f, e1[0]);
            fv1 = ldexpf(1.f, e1[1]);
          }
        }
      };
      auto load_regs = [&]() {
#pragma unroll
        for (int i = 0; i < MAXC; ++i) {
          int c = tid + i * NT;
          // opaque to the optimiser: the chunk's coordinates are recomputed
          // here rather than hoisted and kept live through the whole kernel
          asm volatile("" : "+v"(c));
          if (c < nchunks) {
            const bool isk = c < NB * cpb;
            const int cc = isk ? c : c - NB * cpb;
            const int b = cc / cpb, within = cc % cpb;
            const size_t head = ((size_t)(b == 0 ? ph0 : ph1) * a.Hkv + g) * (size_t)(cpb * 16);
            const uint8_t* src = (const uint8_t*)(isk ? a.pool.k : a.pool.v) + head + within * 16;
            rc[i] = *(const uint4*)src;
          }
        }
      };
      // convert and store one tile to LDS; keys at or past n_pool_keys become 0
      auto store = [&](int t, f16* tile) {
        const int key0 = t * PK;
#pragma unroll
        for (int i = 0; i < MAXC; ++i) {
          __builtin_amdgcn_sched_barrier(0);  // one chunk's conversion at a time
          int c = tid + i * NT;
          asm volatile("" : "+v"(c));
          if (c >= nchunks) continue;
          const bool isk = c < NB * cpb;
          const int cc = isk ? c : c - NB * cpb;
          const int b = cc / cpb, within = cc % cpb;
          const uint32_t w[4] = {rc[i].x, rc[i].y, rc[i].z, rc[i].w};
          if constexpr (fmt == kKvBf16) {
            if (isk) {  // 8 channels of one key row
              const int slot = (within * 8) / D, d0 = (within * 8) % D;
              const int key = b * 16 + slot;
              f16x8 v;
#pragma unroll
              for (int e = 0; e < 8; ++e)
                v[e] = f32_to_f16_sat(__uint_as_float(e & 1 ? w[e >> 1] & 0xffff0000u : w[e >> 1] << 16));
              if (key0 + key >= n_pool_keys) v = f16x8{};
              *(f16x8*)(tile + k_at<D>(key, d0 >> 3)) = v;
            } else {  // 8 slots of one channel: V block [d][16]
              const int d = (within * 8) / 16, s0 = (within * 8) % 16;
#pragma unroll
              for (int u = 0; u < 2; ++u) {  // 4 keys per unit
                f16x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  const int k = 4 * u + e;
                  const float f = __uint_as_float(k & 1 ? w[k >> 1] & 0xffff0000u : w[k >> 1] << 16);
                  v[e] = key0 + b * 16 + s0 + k < n_pool_keys ? f32_to_f16_sat(f) : (f16)0.f;
                }
                *(f16x4*)(tile + v_at<D>(b * 16 + s0 + 4 * u, d)) = v;
              }
            }
          } else if constexpr (fmt == kKvU8) {
            if (isk) {  // 16 channels of one key row
              const int slot = (within * 16) / D, d0 = (within * 16) % D;
              const int key = b * 16 + slot;
              const bool ok = key0 + key < n_pool_keys;
              const float fb = b ? fk1 : fk0;
#pragma unroll
              for (int hh = 0; hh < 2; ++hh) {
                f16x8 v;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                  const int d = d0 + 8 * hh + e;
                  const int code = (w[(8 * hh + e) >> 2] >> (8 * (e & 3))) & 255;
                  v[e] = ok ? f32_to_f16_sat(((float)code - dq[1][d]) * dq[0][d] * fb) : (f16)0.f;
                }
                *(f16x8*)(tile + k_at<D>(key, (d0 >> 3) + hh)) = v;
              }
            } else {  // 16 slots of one channel
              const int d = within;
              const float vs = dq[2][d] * (b ? fv1 : fv0), vz = dq[3][d];
#pragma unroll
              for (int u = 0; u < 4; ++u) {
                f16x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  const int code = (w[u] >> (8 * e)) & 255;
                  v[e] = key0 + b * 16 + 4 * u + e < n_pool_keys ? f32_to_f16_sat(((float)code - vz) * vs)
                                                                   : (f16)0.f;
                }
                *(f16x4*)(tile + v_at<D>(b * 16 + 4 * u, d)) = v;
              }
            }
          } else {  // u4
            if (isk) {  // 32 channels of one key row: byte 4j + i holds 8j + i, 8j + 4 + i
              const int slot = (within * 32) / D, c0 = (within * 32) % D;
              const int key = b * 16 + slot;
              const bool ok = key0 + key < n_pool_keys;
              const float fb = b ? fk1 : fk0;
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                f16x8 v;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                  const int d = c0 + 8 * j + e;
                  const int byte = (w[j] >> (8 * (e & 3))) & 255;
                  const int code = e < 4 ? byte & 15 : byte >> 4;
                  v[e] = ok ? f32_to_f16_sat(((float)code - dq[1][d]) * dq[0][d] * fb) : (f16)0.f;
                }
                *(f16x8*)(tile + k_at<D>(key, (c0 >> 3) + j)) = v;
              }
            } else {  // one channel pair (2c, 2c + 1) of 16 slots
              const int c = within;
#pragma unroll
              for (int n = 0; n < 2; ++n) {
                const int d = 2 * c + n;
                const float vs = dq[2][d] * (b ? fv1 : fv0), vz = dq[3][d];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                  f16x4 v;
#pragma unroll
                  for (int e = 0; e < 4; ++e) {
                    const int byte = (w[u] >> (8 * e)) & 255;
                    const int code = n ? byte >> 4 : byte & 15;
                    v[e] = key0 + b * 16 + 4 * u + e < n_pool_keys ? f32_to_f16_sat(((float)code - vz) * vs)
                                                                     : (f16)0.f;
                  }
                  *(f16x4*)(tile + v_at<D>(b * 16 + 4 * u, d)) = v;
                }
              }
            }
          }
        }
      };
      // one pool tile: mask past this lane's query position and past the
      // pool's keys, then the softmax update and P V
      auto pool_tile = [&](int t, const f16* tile) {
        if (kg != 0) return;  // wave-uniform
        const int key_base = t * PK;
        const bool masked = key_base + PK - 1 > ctx + q_lo || key_base + PK > n_pool_keys;
        plain_tile(tile, masked, min(ctx + my_q, n_pool_keys - 1) - key_base);
      };
      // two stages: the next tile's gather and conversion (into the other
      // stage) before this tile's products, so that the registers of the
      // gather are free while the products run
      load_table(0);
      load_regs();
      store(0, s0);
      __syncthreads();
      for (int t = 0; t < n_pool_tiles; t += 2) {
        if (t + 1 < n_pool_tiles) {
          load_table(t + 1);
          load_regs();
          store(t + 1, s1);
        }
        __builtin_amdgcn_sched_barrier(0);
        pool_tile(t, s0);
        __syncthreads();
        if (t + 1 >= n_pool_tiles) break;
        if (t + 2 < n_pool_tiles) {
          load_table(t + 2);
          load_regs();
          store(t + 2, s0);
        }
        __builtin_amdgcn_sched_barrier(0);
        pool_tile(t + 1, s1);
        __syncthreads();
      }
    }

    // ----------------------------------------------- the staged chunk keys
    if (staged) {
      const int n_all = cdiv(q_hi + 1, PK);  // chunk tiles this query tile sees
      // this key group's tiles: tb .. tb + n_st - 1 (every group steps
      // through n_steps tiles; copies past its last tile repeat a valid one)
      const int n_steps = cdiv(n_all, KS);
      const int tb = kg * n_steps;
      const int n_st = min(n_all - tb, n_steps);  // may be 0 for group 1
      const int t_last = max(min(tb + n_st, n_all) - 1, 0);
      const size_t base = (size_t)g * a.st.rows + prefill_stage_base(a.seq, sidx);
      const f16* ksrc = a.st.k + base * D;
      const f16* vsrc = a.st.v + base * D;
      f16* const g0 = s0 + kg * T::kElems;
      f16* const g1 = s1 + kg * T::kElems;
      f16* const g2 = s2 + kg * T::kElems;
      f16* const g3 = s3 + kg * T::kElems;
      constexpr int L = (T::kInst + NW - 1) / NW;  // copies per wave and tile
      // copy i of a tile: K (first half) or V (second half), 1 KB each;
      // waves past the last copy repeat it (the same bytes to the same place)
      // (t: this group's tile index, 0-based)
      auto issue = [&](int t, f16* tile) {
        const int ta = min(tb + t, t_last);
#pragma unroll
        for (int j = 0; j < L; ++j) {
          const int i = min(wave + NW * j, T::kInst - 1);
          const bool isk = i < T::kInst / 2;
          const int off = (isk ? i : i - T::kInst / 2) * 512;  // fp16 elements
          const f16* src = (isk ? ksrc : vsrc) + (size_t)ta * PK * D + off + lane * 8;
          __builtin_amdgcn_global_load_lds((const void*)src,
                                           (lds_void*)(tile + (isk ? 0 : T::kK) + off), 16, 0, 0);
        }
      };
      auto wait_one_tile = [&]() {  // this wave's copies of the newest tile may stay in flight
        constexpr int W = (L & 15) | (7 << 4) | (15 << 8) | (((L >> 4) & 3) << 14);
        __builtin_amdgcn_s_waitcnt(W);
      };
      // __syncthreads() would add a release fence, which waits for every
      // outstanding load (the copies of the tiles ahead included); the waits
      // here already cover this wave's copies of the tile the next step
      // reads, and the LDS reads of this step have been consumed
      auto barrier = [&]() {
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
      };
      auto masked_at = [&](int t) { return (tb + t) * PK + PK - 1 > q_lo || (tb + t) * PK + PK > q_len; };
      auto lim_at = [&](int t) { return min(my_q, q_len - 1) - (tb + t) * PK; };

      // Every step issues the same copies (past the last tile they repeat it,
      // into a stage no step reads again), so every wait counts the same
      // number of copies on every path.
      __builtin_amdgcn_sched_barrier(0);
      issue(0, g0);
      issue(1, g1);
      issue(2, g2);
      __builtin_amdgcn_sched_barrier(0);
      wait_one_tile();
      __builtin_amdgcn_sched_barrier(0);
      barrier();
      __builtin_amdgcn_sched_barrier(0);
      f32x16 sa = qk(g0), sb;
      // step t: tiles t and t+1 are in LDS, S(t) in registers.  Issue tile
      // t+3; read K(t+1)'s fragments; the row maxima of S(t) and the lazy
      // reference update; then S(t+1) = Q K(t+1)^T one MFMA at a time, each
      // followed by its share of P(t) = 2^(S(t) - m) (the VALU and TRANS work
      // runs while the MFMA does; past the last tile the scores of a repeated
      // tile are computed and never used), at a raised wave priority, which
      // lets the SIMD's other wave fill the gaps; read V(t)'s fragments half way;
      // O += P(t) V(t); wait for tile t+2.  Tiles that need a mask take it
      // first.  The fences keep this order: every LDS read is issued well
      // before the MFMA that takes it.
      auto step = [&](int t, f16* cur, f16* nxt, f16* fill, f32x16& scur, f32x16& snxt) {
        issue(t + 3, fill);
        if (t < n_st) {
          constexpr int NS = D / 16;       // MFMAs of Q K^T
          constexpr int EPS = 16 / NS;     // exponentials per MFMA
          f16x8 kf[NS];
#pragma unroll
          for (int s = 0; s < NS; ++s) kf[s] = *(const f16x8*)(nxt + k_at<D>(ql, 2 * s + G));
          __builtin_amdgcn_sched_barrier(0);
          if (masked_at(t)) {  // a branch, not selects on every tile
            mask(scur, lim_at(t));
            __builtin_amdgcn_sched_barrier(0);
          }
          float sv[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) sv[r] = scur[r];
          const float mt = max_xor32(max16(sv));
          const bool mv = __builtin_amdgcn_ballot_w64(mt > m_run + kLazy) != 0;
          const float m_new = mv ? fmaxf(m_run, mt) : m_run;
          const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
          m_run = m_new;
          __builtin_amdgcn_sched_barrier(0);
          f32x16 e{};
          f16x8 vf[NB][D / 32];
          float pv16[16];
          __builtin_amdgcn_s_setprio(1);
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            e = mfma32(kf[s], qf[s], e);
#pragma unroll
            for (int j = 0; j < EPS; ++j) {
              const int r = EPS * s + j;
              pv16[r] = __builtin_amdgcn_exp2f(scur[r] - m_new);  // 0 where masked
              asm volatile("" : "+v"(pv16[r]));  // computed here, beside this MFMA
            }
            if (s == NS / 2 - 1) {
#pragma unroll
              for (int kc = 0; kc < NB; ++kc)
#pragma unroll
                for (int u = 0; u < D / 32; ++u)
                  vf[kc][u] = *(const f16x8*)(cur + T::kK + kc * 16 * D + (G * D + 32 * u + ql) * 8);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
          __builtin_amdgcn_s_setprio(0);
          snxt = e;
          f16x8 pb[2];
#pragma unroll
          for (int r = 0; r < 16; ++r) pb[r >> 3][r & 7] = (f16)pv16[r];
          l_run = l_run * alpha + sum16(pv16);
          rescale(mv, alpha);
#pragma unroll
          for (int kc = 0; kc < NB; ++kc)
#pragma unroll
            for (int u = 0; u < D / 32; ++u) acc[u] = mfma32(vf[kc][u], pb[kc], acc[u]);
        }
        __builtin_amdgcn_sched_barrier(0);
        wait_one_tile();
        __builtin_amdgcn_sched_barrier(0);
        barrier();
        __builtin_amdgcn_sched_barrier(0);
      };
      // whole groups of four steps (steps past the last tile only copy and
      // wait), so that each of the four keeps its own stage arrays
      for (int t = 0; t < n_steps; t += 4) {
        step(t, g0, g1, g3, sa, sb);
        step(t + 1, g1, g2, g0, sb, sa);
        step(t + 2, g2, g3, g1, sa, sb);
        step(t + 3, g3, g0, g2, sb, sa);
      }
      __builtin_amdgcn_s_waitcnt(0);  // the repeated copies past the last tile
    }

    // ---------------------------------------- key group 1 into key group 0
    if constexpr (KS == 2) {
      __syncthreads();  // every wave is done with the stage arrays
      // wave w of group 1 writes its state -- D/2 accumulator floats, m and
      // l per lane -- to record w of the (now free) stage arrays, where wave
      // w of group 0, the same head, reads it
      constexpr int PER = D / 32 * 16 + 2;
      static_assert(NH * PER * 64 * 4 <= 4 * KS * T::kBytes, "merge buffer");
      auto slot = [&](int i) -> float& {  // element i of this lane's record, spread over s0..s3
        const int flat = (wave * PER + i) * 64 + lane;
        constexpr int per_arr = KS * T::kElems / 2;  // floats per stage array
        const int arr = flat / per_arr, off = flat % per_arr;
        float* base = (float*)(arr == 0 ? s0 : arr == 1 ? s1 : arr == 2 ? s2 : s3);
        return base[off];
      };
      if (kg == 1) {
#pragma unroll
        for (int t = 0; t < D / 32; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) slot(16 * t + r) = acc[t][r];
        slot(PER - 2) = m_run;
        slot(PER - 1) = l_run;
      }
      __syncthreads();
      if (kg == 0) {
        const float m1 = slot(PER - 2), l1 = slot(PER - 1);
        const float m = fmaxf(m_run, m1);
        // a group without keys has m = -inf: its weight is 0
        const float f0 = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m);
        const float f1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - m);
#pragma unroll
        for (int t = 0; t < D / 32; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[t][r] = acc[t][r] * f0 + slot(16 * t + r) * f1;
        l_run = l_run * f0 + l1 * f1;
        m_run = m;
      }
    }

    // ------------------------------------------------------------ output
    const float l = sum_xor32(l_run);
    if (own && kg == 0 && my_q < q_len) {
      const float inv = 1.f / l;
      f16* op = a.o + (size_t)(row0 + ql) * a.Hq * D + (size_t)h * D;
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          f16x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = f32_to_f16_sat(acc[t][4 * q4 + e] * inv);
          *(f16x4*)(op + 32 * t + 8 * q4 + 4 * G) = v4;
        }
    }
  }
}

}  // namespace

hipError_t attn_prefill(const void* q, const PrefillQ& qsrc, KvPool pool, SeqInfo seq, PrefillStage st,
                        int n_prefill, int max_q_len, int Hq, int Hkv, int D, void* o, hipStream_t s) {
  if (n_prefill == 0 || max_q_len == 0) return hipSuccess;
  PrefillArgs a{};
  a.q = (const float*)q;
  a.qs = qsrc;
  a.pool = pool;
  a.seq = seq;
  a.st = st;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.n_rep = Hq / Hkv;
  a.n_qtiles = cdiv(max_q_len, PQ);
  a.o = (f16*)o;
  // Heads per workgroup: the whole group while that gives a workgroup per
  // CU, else at most four (a group of seven or eight heads in two
  // workgroups, each reading the same K/V tiles).
  const long whole = (long)a.n_qtiles * Hkv * n_prefill;
  int nh = a.n_rep;
  if (whole < 256 && nh > 4) nh = 4;
  // still fewer workgroups than CUs (short prompts, where the last query
  // tile's key loop sets the time): groups of at most two heads, each with
  // two key groups that take half of the key tiles (four waves of up to 512
  // registers; four heads x two key groups in eight waves would spill)
  const bool ks2 = a.n_qtiles > 1 && whole * cdiv(a.n_rep, nh) < 256;
  if (ks2) nh = nh < 2 ? nh : 2;
  a.n_split = cdiv(a.n_rep, nh);
  // pair query tiles (x, n-1-x) when that still leaves a workgroup per CU
  a.paired = (long)cdiv(a.n_qtiles, 2) * Hkv * a.n_split * n_prefill >= 256 ? 1 : 0;
  const dim3 grid((a.paired ? cdiv(a.n_qtiles, 2) : a.n_qtiles) * Hkv * a.n_split, 1, n_prefill);
#define TDL_PREFILL_FMT(DD, NH, KS)                                                \
  if (pool.fmt == kKvU8)                                                           \
    attn_prefill_kernel<DD, NH, kKvU8, KS><<<grid, NH * KS * 64, 0, s>>>(a);       \
  else if (pool.fmt == kKvU4)                                                      \
    attn_prefill_kernel<DD, NH, kKvU4, KS><<<grid, NH * KS * 64, 0, s>>>(a);       \
  else                                                                             \
    attn_prefill_kernel<DD, NH, kKvBf16, KS><<<grid, NH * KS * 64, 0, s>>>(a);
#define TDL_PREFILL_CASE(DD, NH)                                                   \
  if (D == DD && nh == NH) {                                                       \
    if constexpr (NH <= 2) {                                                       \
      if (ks2) {                                                                   \
        TDL_PREFILL_FMT(DD, NH, 2)                                                 \
        return hipGetLastError();                                                  \
      }                                                                            \
    }                                                                              \
    TDL_PREFILL_FMT(DD, NH, 1)                                                     \
    return hipGetLastError();                                                      \
  }
  TDL_PREFILL_CASE(128, 1) TDL_PREFILL_CASE(128, 2) TDL_PREFILL_CASE(128, 4)
  TDL_PREFILL_CASE(128, 7) TDL_PREFILL_CASE(128, 8)
  TDL_PREFILL_CASE(64, 1) TDL_PREFILL_CASE(64, 2) TDL_PREFILL_CASE(64, 4)
  TDL_PREFILL_CASE(64, 7) TDL_PREFILL_CASE(64, 8)
#undef TDL_PREFILL_CASE
#undef TDL_PREFILL_FMT
  return hipErrorInvalidValue;
}

}  // namespace tdl
