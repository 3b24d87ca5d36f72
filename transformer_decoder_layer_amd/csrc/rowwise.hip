// Row-wise kernels: RMSNorm, Q/K-norm + RoPE + KV-slot write, KV-cache
// writes and per-channel int8 calibration, weight conversion, RoPE table.

#include "common.h"
#include "kernels.h"

namespace tdl {

namespace {

// ------------------------------------------------------------- RMSNorm
// One workgroup per row (the "one block per row" layout of the RMSNorm kernel
// on the Qwen2.5-7B single-layer page, section 2), one thread per CH chunks of
// 8 columns: the row is read once with 16-byte vector loads and kept in
// registers; fp32 sum of squares reduced within each wave by lane shuffles
// and across the waves through LDS; y = x * rsqrt(sum/H + eps) * g.

__device__ __forceinline__ void load8(const bf16* p, float* v) {
  const bf16x8 t = *(const bf16x8*)p;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (float)t[e];
}
__device__ __forceinline__ void load8(const float* p, float* v) {
  const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// Sum over the workgroup (at most 16 waves) of one value per thread.
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float t = 0.f;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) t += red[w];
  return t;
}

// Threads (a multiple of 64, at most 1024) and chunks of 8 per thread for a
// row of H columns (H % 64 == 0); false if H is too long.  Many rows: at
// least two chunks per thread (more loads in flight per resident thread);
// few rows (decode): one, for parallelism.
bool row_shape(int H, int rows, int* threads, int* ch) {
  const int chunks = H / 8;
  for (int c = rows >= 1024 ? 2 : 1; c <= 4; c *= 2) {
    const int t = (cdiv(chunks, c) + 63) / 64 * 64;
    if (t <= 1024) {
      *threads = t;
      *ch = c;
      return true;
    }
  }
  return false;
}

template <typename TIn, int CH>
__global__ __launch_bounds__(1024) void rmsnorm_kernel(const TIn* __restrict__ x,
                                                       const float* __restrict__ g,
                                                       f16* __restrict__ y, int H, float eps) {
  __shared__ float red[16];
  const int row = blockIdx.x, nt = blockDim.x;
  const TIn* xr = x + (size_t)row * H;
  f16* yr = y + (size_t)row * H;
  float v[CH][8], gg[CH][8];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const int c = (threadIdx.x + nt * j) * 8;
    const bool ok = c < H;
    load8(xr + (ok ? c : 0), v[j]);
    load8(g + (ok ? c : 0), gg[j]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[j][e] = ok ? v[j][e] : 0.f;
      ss += v[j][e] * v[j][e];
    }
  }
  const float inv = rsqrtf(block_sum(ss, red) / (float)H + eps);
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const int c = (threadIdx.x + nt * j) * 8;
    if (c >= H) break;
    f16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = f32_to_f16_sat(v[j][e] * inv * gg[j][e]);
    *(f16x8*)(yr + c) = o;
  }
}

// ---------------------------------------------------- sequence lookups
__device__ __forceinline__ int find_seq(const SeqInfo& s, int row) {
  if (s.rows_are_seqs) return row;
  if (!s.q_start) return 0;
  int lo = 0, hi = s.n_seqs - 1;
  while (lo < hi) {  // last sequence whose q_start <= row
    const int mid = (lo + hi + 1) >> 1;
    if (s.q_start[mid] <= row) lo = mid; else hi = mid - 1;
  }
  return lo;
}
__device__ __forceinline__ int row_position(const SeqInfo& s, int seq, int row) {
  if (s.rows_are_seqs) return s.ctx_len[row];
  if (!s.q_start) return s.ctx0 + row;
  return s.ctx_len[seq] + row - s.q_start[seq];
}
// One past the last row of sequence `seq` in this call.  q_start without
// q_len is the cumulative form (kv_cache_write's cu_rows, n_seqs + 1
// entries).
__device__ __forceinline__ int seq_end_row(const SeqInfo& s, int seq, int row) {
  if (s.rows_are_seqs) return row + 1;
  if (!s.q_start) return s.q_len0;
  return s.q_len ? s.q_start[seq] + s.q_len[seq] : s.q_start[seq + 1];
}
// Physical block of token `pos` of sequence `seq` (the page table lookup,
// get_location of the TFFInfer page section 3.6.4).
__device__ __forceinline__ int block_of(const SeqInfo& s, int seq, int pos) {
  if (!s.tables) return pos / kBlockTokens;
  return s.tables[(size_t)seq * s.max_blocks + pos / kBlockTokens];
}

// Quantise one value in a block with factor 2^e: clamp(round_half_even((x /
// scale) * 2^-e) + zp, 0, top), with a correctly rounded fp32 divide and an
// exact power-of-two scaling (top 255 for u8 codes, 15 for u4; e = 0 is the
// per-channel quantiser).
__device__ __forceinline__ int quant_code(float x, float scale, int zp, int top, int e = 0) {
  const float q = __builtin_rintf(ldexpf(__fdiv_rn(x, scale), -e));
  const int c = (int)q + zp;
  return c < 0 ? 0 : (c > top ? top : c);
}
// Smallest e in [0, kMaxBlockExp] for which x quantises without clamping
// (kMaxBlockExp if none does).
__device__ __forceinline__ int exp_needed(float x, float scale, int zp, int top) {
  const float q = __fdiv_rn(x, scale);
  for (int e = 0; e < kMaxBlockExp; ++e) {
    const float c = __builtin_rintf(ldexpf(q, -e)) + (float)zp;
    if (c >= 0.f && c <= (float)top) return e;
  }
  return kMaxBlockExp;
}
// The factor exponent of block blk, KV head g (kv 0: K, 1: V); 0 without
// block scales.
__device__ __forceinline__ int pool_exp(const KvPool& pool, int blk, int g, int Hkv, int kv) {
  return pool.exps ? (int)pool.exps[((size_t)blk * Hkv + g) * 2 + kv] : 0;
}
__device__ __forceinline__ int wave_max_i(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  return v;
}

// bf16 / u8 pools: one element per (slot, d); u8 codes in a block with
// factors 2^ek (K) and 2^ev (V)
template <int F>
__device__ __forceinline__ void store_kv(const KvPool& pool, int blk, int g, int Hkv, int D, int slot,
                                         int d, float kval, float vval, int ek = 0, int ev = 0) {
  const size_t head = ((size_t)blk * Hkv + g) * kBlockTokens * D;
  const size_t kidx = head + (size_t)slot * D + d;   // K: [blk][g][slot][d]
  const size_t vidx = head + (size_t)d * kBlockTokens + slot;  // V: [blk][g][d][slot]
  if constexpr (F == kKvU8) {
    const int ch = g * D + d;
    ((uint8_t*)pool.k)[kidx] = (uint8_t)quant_code(kval, pool.k_scale[ch], pool.k_zp[ch], 255, ek);
    ((uint8_t*)pool.v)[vidx] = (uint8_t)quant_code(vval, pool.v_scale[ch], pool.v_zp[ch], 255, ev);
  } else {
    ((bf16*)pool.k)[kidx] = f32_to_bf16(kval);
    ((bf16*)pool.v)[vidx] = f32_to_bf16(vval);
  }
}

// u4 pools: byte offsets of a block-head tile (8*D bytes for K and for V)
__device__ __forceinline__ size_t u4_head(int blk, int g, int Hkv, int D) {
  return ((size_t)blk * Hkv + g) * kBlockTokens * (D / 2);
}
// K byte of channel d (d & 4 == 0; its partner d + 4 is the high nibble)
__device__ __forceinline__ int u4_kbyte(int slot, int d, int D) {
  return slot * (D / 2) + 4 * (d >> 3) + (d & 3);
}
// V byte of channel d (d even; its partner d + 1 is the high nibble)
__device__ __forceinline__ int u4_vbyte(int slot, int d) { return (d >> 1) * kBlockTokens + slot; }

// ------------------------------------------------ Q/K-norm + RoPE + KV
// One workgroup (4 waves) per row; each wave takes one head at a time: the
// Q heads, then the K heads (RoPE and, for K, the cache write together with
// the matching V head).  Q and K heads share the launch, as the RoPE kernel
// of the Qwen2.5-7B page (section 2) does with its unified head indexing.
// Half-split pairs (i, i + D/2): lane i < D/2 owns pair i.
//
// Per-block x per-channel caches take two launches.  mode 1: the row at
// slot 0 of a block (the call writes the block's first slot) computes the
// rotated K and the V of every row this call writes into that block and
// stores the block's factor exponents (the smallest that leaves no code
// clamped, per KV head, K and V separately); every other row does nothing.
// mode 0: every row quantises with its block's exponents (set by this call's
// mode-1 launch, or by the call that wrote the block's first slot).
// SB: split-K slices read per batch of loads (1, 4 or 8 by the slice count;
// a larger batch costs registers and occupancy); F: the pool's format; RPW:
// rows per workgroup (mode 0 only): each wave issues the loads of all its
// rows' inputs before it rotates and stores any of them, one chain of
// dependent loads for RPW rows instead of one per row.
template <int SB, int F, int RPW>
__global__ __launch_bounds__(256) void rope_kv_kernel(const float* __restrict__ qkv, int rows, int Hq,
                                                      int Hkv, int D, const float2* __restrict__ tab,
                                                      const float* __restrict__ qn,
                                                      const float* __restrict__ kn, float eps,
                                                      float* __restrict__ q_out, SeqInfo seq,
                                                      KvPool pool, PrefillStage stage, int splits,
                                                      const float* __restrict__ bias, int hpw, int mode,
                                                      int q_skip) {
  static_assert(RPW >= 1, "rows per workgroup");
  // Several rows per workgroup (long prompts): consecutive row groups, which
  // write the same V^T lines of their cache blocks (one 2-byte slot per
  // token and channel), go to one XCD, whose L2 then merges those partial
  // line writes; workgroups are dealt to the 8 XCDs round-robin, so XCD x
  // takes the x-th contiguous range of row groups (a bijection on the grid)
  int bid = blockIdx.x;
  if constexpr (RPW > 1) {
    const int G = gridDim.x, per = G / 8, rem = G % 8, x = bid % 8, slot = bid / 8;
    bid = x * per + min(x, rem) + slot;
  }
  const int row0 = bid * RPW;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = D >> 1;
  const int ldq = (Hq + 2 * Hkv) * D;
  const size_t slice = (size_t)rows * ldq;
  // the rows' sequences, positions and cache slots
  int r_sidx[RPW], r_pos[RPW], r_blk[RPW], r_slot[RPW], r_srow[RPW];
  bool r_ok[RPW], r_staged[RPW];
#pragma unroll
  for (int rr = 0; rr < RPW; ++rr) {
    const int row = min(row0 + rr, rows - 1);
    r_ok[rr] = row0 + rr < rows;
    r_sidx[rr] = find_seq(seq, row);
    r_pos[rr] = row_position(seq, r_sidx[rr], row);
    r_blk[rr] = block_of(seq, r_sidx[rr], r_pos[rr]);
    r_slot[rr] = r_pos[rr] % kBlockTokens;
    // the row of the prefill staging copy (sequences < stage.n_seqs)
    r_staged[rr] = mode == 0 && !seq.rows_are_seqs && r_sidx[rr] < stage.n_seqs;
    r_srow[rr] = r_staged[rr] ? prefill_stage_base(seq, r_sidx[rr]) + row -
                                    (seq.q_start ? seq.q_start[r_sidx[rr]] : 0)
                              : 0;
  }
  // mode 1 (RPW = 1): only the rows at slot 0, for the rows of this call in the block
  int n_blk_rows = 1;
  if (mode == 1) {
    if (r_slot[0] != 0) return;
    n_blk_rows = min(kBlockTokens, min(seq_end_row(seq, r_sidx[0], row0), rows) - row0);
  }
  // elements c[0..NC) of row row0+i's projection: the partial slices in
  // order (+ bias), read SB slices at a time with every load of a batch
  // issued before the first add (slice indices past the last repeat it and
  // add nothing)
  auto vals = [&](int i, auto& c, auto& out) {
    constexpr int NC = sizeof(out) / sizeof(float);
    const float* src = qkv + (size_t)min(row0 + i, rows - 1) * ldq;
    if constexpr (SB == 1) {  // one slice (splits == 1): plain loads, nothing waits for them here
#pragma unroll
      for (int k = 0; k < NC; ++k) out[k] = src[c[k]];
    } else
    for (int s0 = 0; s0 < splits; s0 += SB) {
      float t[SB][NC];
#pragma unroll
      for (int u = 0; u < SB; ++u)
#pragma unroll
        for (int k = 0; k < NC; ++k) t[u][k] = src[(size_t)min(s0 + u, splits - 1) * slice + c[k]];
#pragma unroll
      for (int u = 0; u < SB; ++u) {  // a select, not a branch: the loads stay unconditional
        const bool live = s0 + u < splits;
#pragma unroll
        for (int k = 0; k < NC; ++k) out[k] = s0 + u == 0 ? t[u][k] : out[k] + (live ? t[u][k] : 0.f);
      }
    }
    if (bias) {
#pragma unroll
      for (int k = 0; k < NC; ++k) out[k] += bias[c[k]];
    }
  };
  const bool act = lane < half;
  const int ln = act ? lane : 0;  // lanes past D/2 load a valid element and store nothing
  // the (cos, sin) pair of channel pair `lane` at position p
  auto rope_cs = [&](int p) { return act ? tab[(size_t)p * half + lane] : make_float2(1.f, 0.f); };
  // head h normalised (Q/K) and rotated: channels ln, ln + D/2 (x holds
  // their projections)
  auto rotate = [&](int h, float x1, float x2, float2 cs, float& r1, float& r2) {
    const bool is_q = h < Hq;
    if (!act) x1 = x2 = 0.f;
    const float* gn = is_q ? qn : kn;
    if (gn) {  // per-head RMSNorm over D
      const float ss = wave_sum(x1 * x1 + x2 * x2);
      const float inv = rsqrtf(ss / (float)D + eps);
      if (act) {
        x1 = x1 * inv * gn[lane];
        x2 = x2 * inv * gn[lane + half];
      }
    }
    r1 = x1 * cs.x - x2 * cs.y;
    r2 = x1 * cs.y + x2 * cs.x;
  };
  constexpr int top = F == kKvU8 ? 255 : 15;

  // one wave per head: workgroup (rows, y) takes heads hpw*y .. hpw*y + hpw-1
  for (int h = hpw * blockIdx.y + wave; h < min(Hq + Hkv, hpw * ((int)blockIdx.y + 1)); h += 4) {
    const bool is_q = h < Hq;
    if (mode == 1) {  // wave-uniform
      if (is_q) continue;
      const int g = h - Hq;
      const int vc = (Hq + Hkv + g) * D;
      const int c1 = g * D + ln, c2 = c1 + half;
      int ek = 0, ev = 0;
      for (int i = 0; i < n_blk_rows; ++i) {
        const int cols[4] = {h * D + ln, h * D + ln + half, vc + ln, vc + ln + half};
        float x[4];
        vals(i, cols, x);
        float r1, r2;
        rotate(h, x[0], x[1], rope_cs(r_pos[0] + i), r1, r2);
        const float v1 = x[2], v2 = x[3];
        if (act) {
          ek = max(ek, max(exp_needed(r1, pool.k_scale[c1], pool.k_zp[c1], top),
                           exp_needed(r2, pool.k_scale[c2], pool.k_zp[c2], top)));
          ev = max(ev, max(exp_needed(v1, pool.v_scale[c1], pool.v_zp[c1], top),
                           exp_needed(v2, pool.v_scale[c2], pool.v_zp[c2], top)));
        }
      }
      ek = wave_max_i(ek);
      ev = wave_max_i(ev);
      if (lane == 0) {
        pool.exps[((size_t)r_blk[0] * Hkv + g) * 2] = (int8_t)ek;
        pool.exps[((size_t)r_blk[0] * Hkv + g) * 2 + 1] = (int8_t)ev;
      }
      continue;
    }
    // rows whose queries the prefill attention rotates as it loads them
    bool live[RPW], any = false;
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
      live[rr] = r_ok[rr] && !(is_q && r_sidx[rr] < q_skip);
      any = any || live[rr];
    }
    if (!any) continue;  // wave-uniform: e.g. every row's queries rotated by prefill attention
    if (is_q) {  // wave-uniform
      const int cols[2] = {h * D + ln, h * D + ln + half};
      float x[RPW][2];
      float2 cs[RPW];
#pragma unroll
      for (int rr = 0; rr < RPW; ++rr) {
        vals(rr, cols, x[rr]);
        cs[rr] = rope_cs(r_pos[rr]);
      }
#pragma unroll
      for (int rr = 0; rr < RPW; ++rr) {
        if (!live[rr]) continue;  // wave-uniform
        float r1, r2;
        rotate(h, x[rr][0], x[rr][1], cs[rr], r1, r2);
        if (act) {
          float* qo = q_out + ((size_t)(row0 + rr) * Hq + h) * D;
          qo[lane] = r1;
          qo[lane + half] = r2;
        }
      }
      continue;
    }
    const int g = h - Hq;
    const int vc = (Hq + Hkv + g) * D;
    const int cols[4] = {h * D + ln, h * D + ln + half, vc + ln, vc + ln + half};
    float x[RPW][4];
    float2 cs[RPW];
    int ekr[RPW], evr[RPW];
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
      vals(rr, cols, x[rr]);
      cs[rr] = rope_cs(r_pos[rr]);
      ekr[rr] = pool_exp(pool, r_blk[rr], g, Hkv, 0);
      evr[rr] = pool_exp(pool, r_blk[rr], g, Hkv, 1);
    }
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
      if (!live[rr]) continue;  // wave-uniform
      float r1, r2;
      rotate(h, x[rr][0], x[rr][1], cs[rr], r1, r2);
      const float v1 = x[rr][2], v2 = x[rr][3];
      const int ek = ekr[rr], ev = evr[rr];
      const int blk = r_blk[rr], slot = r_slot[rr];
      if (r_staged[rr] && act) {
        // fp16 copy of what the cache holds (bf16-rounded, or the dequantised
        // code) for prefill attention
        const int c1 = g * D + lane, c2 = c1 + half;
        float sk1, sk2, sv1, sv2;
        if constexpr (F == kKvBf16) {
          sk1 = (float)f32_to_bf16(r1); sk2 = (float)f32_to_bf16(r2);
          sv1 = (float)f32_to_bf16(v1); sv2 = (float)f32_to_bf16(v2);
        } else {
          const float fk = ldexpf(1.f, ek), fv = ldexpf(1.f, ev);
          sk1 = (float)(quant_code(r1, pool.k_scale[c1], pool.k_zp[c1], top, ek) - pool.k_zp[c1]) * (pool.k_scale[c1] * fk);
          sk2 = (float)(quant_code(r2, pool.k_scale[c2], pool.k_zp[c2], top, ek) - pool.k_zp[c2]) * (pool.k_scale[c2] * fk);
          sv1 = (float)(quant_code(v1, pool.v_scale[c1], pool.v_zp[c1], top, ev) - pool.v_zp[c1]) * (pool.v_scale[c1] * fv);
          sv2 = (float)(quant_code(v2, pool.v_scale[c2], pool.v_zp[c2], top, ev) - pool.v_zp[c2]) * (pool.v_scale[c2] * fv);
        }
        const int srow = r_srow[rr];
        const size_t hb = (size_t)g * stage.rows * D;
        stage.k[hb + prefill_k_index(srow, lane, D)] = f32_to_f16_sat(sk1);
        stage.k[hb + prefill_k_index(srow, lane + half, D)] = f32_to_f16_sat(sk2);
        stage.v[hb + prefill_v_index(srow, lane, D)] = f32_to_f16_sat(sv1);
        stage.v[hb + prefill_v_index(srow, lane + half, D)] = f32_to_f16_sat(sv2);
      }
      if constexpr (F != kKvU4) {
        if (act) {
          store_kv<F>(pool, blk, g, Hkv, D, slot, lane, r1, v1, ek, ev);
          store_kv<F>(pool, blk, g, Hkv, D, slot, lane + half, r2, v2, ek, ev);
        }
      } else {
        // u4: lane i holds channels i and i + D/2; a byte pairs channels d,
        // d + 4 (K) or d, d + 1 (V), whose codes sit in lanes i ^ 4 / i ^ 1
        // (D/2 is a multiple of 8, so partners of active lanes are active).
        // Every lane takes part in the exchange.
        const int c1 = g * D + ln, c2 = c1 + half;
        const int k1 = quant_code(r1, pool.k_scale[c1], pool.k_zp[c1], 15, ek);
        const int k2 = quant_code(r2, pool.k_scale[c2], pool.k_zp[c2], 15, ek);
        const int w1 = quant_code(v1, pool.v_scale[c1], pool.v_zp[c1], 15, ev);
        const int w2 = quant_code(v2, pool.v_scale[c2], pool.v_zp[c2], 15, ev);
        const int pk1 = __shfl_xor(k1, 4, 64), pk2 = __shfl_xor(k2, 4, 64);
        const int pw1 = __shfl_xor(w1, 1, 64), pw2 = __shfl_xor(w2, 1, 64);
        if (act) {
          const size_t hb = u4_head(blk, g, Hkv, D);
          uint8_t* kp = (uint8_t*)pool.k + hb;
          uint8_t* vp = (uint8_t*)pool.v + hb;
          if (!(lane & 4)) {
            kp[u4_kbyte(slot, lane, D)] = (uint8_t)(k1 | (pk1 << 4));
            kp[u4_kbyte(slot, lane + half, D)] = (uint8_t)(k2 | (pk2 << 4));
          }
          if (!(lane & 1)) {
            vp[u4_vbyte(slot, lane)] = (uint8_t)(w1 | (pw1 << 4));
            vp[u4_vbyte(slot, lane + half)] = (uint8_t)(w2 | (pw2 << 4));
          }
        }
      }
    }
  }
}

// h = sum of the split slices (in order) + residual, one chunk of 8 columns
// per thread (H <= 8192), written once; then y = RMSNorm(h) * g.  The slices
// are read SB at a time, every load of a batch issued before the first add.
constexpr int kSplitNormMaxH = 8192;
template <int SB>
__global__ __launch_bounds__(1024) void rmsnorm_splits_kernel(const float* __restrict__ ws, int splits,
                                                              const bf16* __restrict__ resid,
                                                              float* __restrict__ h,
                                                              const float* __restrict__ g,
                                                              f16* __restrict__ y, int H, float eps) {
  __shared__ float red[16];
  const int row = blockIdx.x;
  const size_t slice = (size_t)gridDim.x * H;
  const int c = threadIdx.x * 8;
  const bool ok = c < H;
  const size_t o = (size_t)row * H + (ok ? c : 0);
  const bf16x8 r = *(const bf16x8*)(resid + o);
  float gg[8];
  load8(g + (ok ? c : 0), gg);
  float p[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < splits; s0 += SB) {
    float4 a[SB], b[SB];
#pragma unroll
    for (int u = 0; u < SB; ++u) {  // slices past the last repeat it and add nothing
      const float* src = ws + (size_t)min(s0 + u, splits - 1) * slice + o;
      a[u] = *(const float4*)src;
      b[u] = *(const float4*)(src + 4);
    }
#pragma unroll
    for (int u = 0; u < SB; ++u) {  // a select, not a branch: the loads stay unconditional
      const bool live = s0 + u < splits;
      p[0] += live ? a[u].x : 0.f; p[1] += live ? a[u].y : 0.f;
      p[2] += live ? a[u].z : 0.f; p[3] += live ? a[u].w : 0.f;
      p[4] += live ? b[u].x : 0.f; p[5] += live ? b[u].y : 0.f;
      p[6] += live ? b[u].z : 0.f; p[7] += live ? b[u].w : 0.f;
    }
  }
  float v[8], ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    v[e] = ok ? p[e] + (float)r[e] : 0.f;
    ss += v[e] * v[e];
  }
  const float inv = rsqrtf(block_sum(ss, red) / (float)H + eps);
  if (!ok) return;
  *(float4*)(h + o) = make_float4(v[0], v[1], v[2], v[3]);
  *(float4*)(h + o + 4) = make_float4(v[4], v[5], v[6], v[7]);
  f16x8 o8;
#pragma unroll
  for (int e = 0; e < 8; ++e) o8[e] = f32_to_f16_sat(v[e] * inv * gg[e]);
  *(f16x8*)(y + o) = o8;
}

// ---------------------------------------------------- cache writes
// One workgroup per row.  Per-block x per-channel caches take two launches,
// as for the RoPE kernel: mode 1, the row at slot 0 of a block sets the
// block's exponents from the rows this call writes into it; mode 0, every
// row quantises with its block's exponents.
__global__ __launch_bounds__(256) void kv_write_kernel(const void* __restrict__ k,
                                                       const void* __restrict__ v, int src_f32,
                                                       int Hkv, int D, SeqInfo seq, KvPool pool, int mode) {
  const int row = blockIdx.x;
  const int sidx = find_seq(seq, row);
  const int pos = row_position(seq, sidx, row);
  const int blk = block_of(seq, sidx, pos);
  const int slot = pos % kBlockTokens;
  auto ld = [&](const void* p, size_t i) {
    return src_f32 ? ((const float*)p)[i] : (float)((const bf16*)p)[i];
  };
  if (mode == 1) {
    if (slot != 0) return;
    const int nr = min(kBlockTokens, min(seq_end_row(seq, sidx, row), (int)gridDim.x) - row);
    const int top = pool.fmt == kKvU8 ? 255 : 15;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int g = wave; g < Hkv; g += blockDim.x / 64) {  // one wave per KV head
      int ek = 0, ev = 0;
      for (int i = 0; i < nr; ++i)
        for (int d = lane; d < D; d += 64) {
          const size_t idx = (size_t)(row + i) * Hkv * D + (size_t)g * D + d;
          const int ch = g * D + d;
          ek = max(ek, exp_needed(ld(k, idx), pool.k_scale[ch], pool.k_zp[ch], top));
          ev = max(ev, exp_needed(ld(v, idx), pool.v_scale[ch], pool.v_zp[ch], top));
        }
      ek = wave_max_i(ek);
      ev = wave_max_i(ev);
      if (lane == 0) {
        pool.exps[((size_t)blk * Hkv + g) * 2] = (int8_t)ek;
        pool.exps[((size_t)blk * Hkv + g) * 2 + 1] = (int8_t)ev;
      }
    }
    return;
  }
  if (pool.fmt != kKvU4) {
    for (int e = threadIdx.x; e < Hkv * D; e += blockDim.x) {
      const size_t idx = (size_t)row * Hkv * D + e;
      const int g = e / D;
      const int ek = pool_exp(pool, blk, g, Hkv, 0), ev = pool_exp(pool, blk, g, Hkv, 1);
      if (pool.fmt == kKvU8)
        store_kv<kKvU8>(pool, blk, g, Hkv, D, slot, e % D, ld(k, idx), ld(v, idx), ek, ev);
      else
        store_kv<kKvBf16>(pool, blk, g, Hkv, D, slot, e % D, ld(k, idx), ld(v, idx), ek, ev);
    }
    return;
  }
  // u4: one thread per K byte and V byte (two channels each)
  const int hd = D / 2;
  for (int e = threadIdx.x; e < Hkv * hd; e += blockDim.x) {
    const int g = e / hd, i = e % hd;
    const int dk = 8 * (i >> 2) + (i & 3), dv = 2 * i;  // low-nibble channels
    const size_t src = (size_t)row * Hkv * D + (size_t)g * D;
    const int ck = g * D + dk, cv = g * D + dv;
    const int ek = pool_exp(pool, blk, g, Hkv, 0), ev = pool_exp(pool, blk, g, Hkv, 1);
    const int klo = quant_code(ld(k, src + dk), pool.k_scale[ck], pool.k_zp[ck], 15, ek);
    const int khi = quant_code(ld(k, src + dk + 4), pool.k_scale[ck + 4], pool.k_zp[ck + 4], 15, ek);
    const int vlo = quant_code(ld(v, src + dv), pool.v_scale[cv], pool.v_zp[cv], 15, ev);
    const int vhi = quant_code(ld(v, src + dv + 1), pool.v_scale[cv + 1], pool.v_zp[cv + 1], 15, ev);
    const size_t hb = u4_head(blk, g, Hkv, D);
    ((uint8_t*)pool.k)[hb + u4_kbyte(slot, dk, D)] = (uint8_t)(klo | (khi << 4));
    ((uint8_t*)pool.v)[hb + u4_vbyte(slot, dv)] = (uint8_t)(vlo | (vhi << 4));
  }
}

// Per-channel min / max over n tokens: one thread per channel walks the
// tokens of its slice; partial results merge with atomics on ordered ints.
__device__ __forceinline__ int f2ord(float f) {
  const int i = __float_as_int(f);
  return i >= 0 ? i : i ^ 0x7fffffff;
}
__device__ __forceinline__ float ord2f(int i) { return __int_as_float(i >= 0 ? i : i ^ 0x7fffffff); }

__global__ void minmax_kernel(const float* __restrict__ x, int64_t n, int C, int rows_per_block,
                              int* __restrict__ mn, int* __restrict__ mx) {
  const int c = blockIdx.y * blockDim.x + threadIdx.x;
  if (c >= C) return;
  const int64_t r0 = (int64_t)blockIdx.x * rows_per_block;
  const int64_t r1 = min(n, r0 + rows_per_block);
  float lo = INFINITY, hi = -INFINITY;
  for (int64_t r = r0; r < r1; ++r) {
    const float v = x[r * C + c];
    lo = fminf(lo, v);
    hi = fmaxf(hi, v);
  }
  if (r0 < r1) {
    atomicMin(&mn[c], f2ord(lo));
    atomicMax(&mx[c], f2ord(hi));
  }
}
__global__ void minmax_init(int* mn, int* mx, int C) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c < C) {
    mn[c] = 0x7fffffff;
    mx[c] = (int)0x80000000;
  }
}
// scale = (max - min) / 255 (1 for a flat channel); zp = rint(-min / scale)
// -- the per-channel formula of the devpress engine page, section 2.6.
__global__ void calib_finish(const int* mn, const int* mx, int C, float levels, float* scale,
                             int* zp) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= C) return;
  const float lo = ord2f(mn[c]), hi = ord2f(mx[c]);
  float s = __fdiv_rn(hi - lo, levels);
  if (s == 0.f) s = 1.0f;
  scale[c] = s;
  zp[c] = (int)__builtin_rintf(__fdiv_rn(-lo, s));
}

// ----------------------------------------------------- weight set-up
__global__ void convert_kernel(const void* __restrict__ src, int src_f32, void* __restrict__ dst,
                               int dst_f16, int64_t n, int* __restrict__ n_sat) {
  int sat = 0;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const float v = src_f32 ? ((const float*)src)[i] : (float)((const bf16*)src)[i];
    if (dst_f16) {
      sat += fabsf(v) > kF16Max;
      ((f16*)dst)[i] = f32_to_f16_sat(v);
    } else {
      ((bf16*)dst)[i] = f32_to_bf16(v);
    }
  }
  if (sat) atomicAdd(n_sat, sat);
}
// Q8_0 -> fp16 or bf16 weights: w[n][k] = code[n][k] * scale[n][k/32], the
// product (exact in fp32) rounded to nearest even, fp16 saturating.  One
// thread per 8 codes.
__global__ void expand_q80_kernel(const int8_t* __restrict__ codes, const __half* __restrict__ scales,
                                  int N, int K, void* __restrict__ dst, int dst_f16) {
  const int64_t n8 = (int64_t)N * (K / 8);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int n = (int)(i / (K / 8)), k = (int)(i % (K / 8)) * 8;
    const float sc = __half2float(scales[(size_t)n * (K / 32) + k / 32]);
    const uint2 c = *(const uint2*)(codes + (size_t)n * K + k);
    const uint32_t w[2] = {c.x, c.y};
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (float)(int8_t)(w[e >> 2] >> (8 * (e & 3))) * sc;
    if (dst_f16) {
      f16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = f32_to_f16_sat(v[e]);
      *(f16x8*)((f16*)dst + (size_t)n * K + k) = o;
    } else {
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = f32_to_bf16(v[e]);
      *(bf16x8*)((bf16*)dst + (size_t)n * K + k) = o;
    }
  }
}
// per-row int8: (code - zp[n]) * scale[n], rounded once to the stored type
__global__ void expand_iq8_kernel(const int8_t* __restrict__ codes, const float* __restrict__ scale,
                                  const float* __restrict__ zp, int N, int K, void* __restrict__ dst,
                                  int dst_f16) {
  const int64_t n8 = (int64_t)N * (K / 8);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int n = (int)(i / (K / 8)), k = (int)(i % (K / 8)) * 8;
    const float sc = scale[n], z = zp[n];
    const uint2 c = *(const uint2*)(codes + (size_t)n * K + k);
    const uint32_t w[2] = {c.x, c.y};
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = ((float)(int8_t)(w[e >> 2] >> (8 * (e & 3))) - z) * sc;
    if (dst_f16) {
      f16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = f32_to_f16_sat(v[e]);
      *(f16x8*)((f16*)dst + (size_t)n * K + k) = o;
    } else {
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = f32_to_bf16(v[e]);
      *(bf16x8*)((bf16*)dst + (size_t)n * K + k) = o;
    }
  }
}
__global__ void i8_to_f32_kernel(const int8_t* __restrict__ src, float* __restrict__ dst, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = (float)src[i];
}
__global__ void copy_f32_kernel(const float* __restrict__ src, float* __restrict__ dst, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}
// dst row 32*(j/16) + j%16 <- gate row j; dst row 32*(j/16) + 16 + j%16 <- up row j
__global__ void interleave_kernel(const uint8_t* __restrict__ gate, const uint8_t* __restrict__ up,
                                  int row_bytes, int I, uint8_t* __restrict__ dst) {
  const int drow = blockIdx.x;  // 0 .. 2I-1
  const int grp = drow / 32, w = drow % 32;
  const int j = grp * 16 + (w % 16);
  const uint8_t* s = (w < 16 ? gate : up) + (size_t)j * row_bytes;
  uint8_t* d = dst + (size_t)drow * row_bytes;
  for (int b = threadIdx.x * 4; b < row_bytes; b += blockDim.x * 4)
    *(uint32_t*)(d + b) = *(const uint32_t*)(s + b);
}

// one thread per 16-byte chunk (8 elements of one row), written to its
// packed position
__global__ void pack_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, int N, int K) {
  const int64_t chunks = (int64_t)N * (K / 8);
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < chunks;
       c += (int64_t)gridDim.x * blockDim.x) {
    const int n = (int)(c / (K / 8)), k = (int)(c % (K / 8)) * 8;
    dst[packed_offset(n, k, N) / 8] = src[c];
  }
}

// one thread per 16-byte destination chunk of the packed code layout
__global__ void pack_codes_kernel(const int8_t* __restrict__ src, uint4* __restrict__ dst, int N, int K) {
  const int64_t chunks = (int64_t)N * (K / 16);
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < chunks;
       c += (int64_t)gridDim.x * blockDim.x) {
    const int l = (int)(c & 63);
    const int64_t tile = c >> 6;
    const int g = (int)(tile % (N / 16)), st = (int)(tile / (N / 16));
    const int n = 16 * g + (l & 15), k = 64 * st + 8 * (l >> 4);
    const uint2 lo = *(const uint2*)(src + (size_t)n * K + k);
    const uint2 hi = *(const uint2*)(src + (size_t)n * K + k + 32);
    dst[c] = make_uint4(lo.x, lo.y, hi.x, hi.y);
  }
}

__global__ void rope_table_kernel(float2* tab, int max_pos, int D, double theta) {
  const int half = D / 2;
  const int64_t n = (int64_t)max_pos * half;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int pos = (int)(idx / half), i = (int)(idx % half);
    const double a = (double)pos * pow(theta, -2.0 * i / D);
    double sn, cn;
    sincos(a, &sn, &cn);
    tab[idx] = make_float2((float)cn, (float)sn);
  }
}

}  // namespace

hipError_t rmsnorm_splits_resid(const float* ws, int splits, const void* resid, float* h,
                                const float* g, void* y, int rows, int H, float eps, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (H % 64 != 0 || H > kSplitNormMaxH || splits < 1) return hipErrorInvalidValue;
  const int nt = (H / 8 + 63) / 64 * 64;
  if (splits <= 4)
    rmsnorm_splits_kernel<4><<<rows, nt, 0, s>>>(ws, splits, (const bf16*)resid, h, g, (f16*)y, H, eps);
  else
    rmsnorm_splits_kernel<8><<<rows, nt, 0, s>>>(ws, splits, (const bf16*)resid, h, g, (f16*)y, H, eps);
  return hipGetLastError();
}

template <typename TIn>
hipError_t rmsnorm_launch(const TIn* x, const float* g, void* y, int rows, int H, float eps,
                          hipStream_t s) {
  if (rows == 0) return hipSuccess;
  int nt, ch;
  if (H % 64 != 0 || !row_shape(H, rows, &nt, &ch)) return hipErrorInvalidValue;
  switch (ch) {
    case 1: rmsnorm_kernel<TIn, 1><<<rows, nt, 0, s>>>(x, g, (f16*)y, H, eps); break;
    case 2: rmsnorm_kernel<TIn, 2><<<rows, nt, 0, s>>>(x, g, (f16*)y, H, eps); break;
    default: rmsnorm_kernel<TIn, 4><<<rows, nt, 0, s>>>(x, g, (f16*)y, H, eps); break;
  }
  return hipGetLastError();
}

hipError_t rmsnorm_bf16in(const void* x, const float* g, void* y, int rows, int H, float eps,
                          hipStream_t s) {
  return rmsnorm_launch((const bf16*)x, g, y, rows, H, eps, s);
}
hipError_t rmsnorm_f32in(const float* x, const float* g, void* y, int rows, int H, float eps,
                         hipStream_t s) {
  return rmsnorm_launch(x, g, y, rows, H, eps, s);
}

hipError_t rope_kv_write(const void* qkv, int rows, int Hq, int Hkv, int D, const float2* tab,
                         const float* q_norm, const float* k_norm, float eps, void* q_out,
                         SeqInfo seq, KvPool pool, PrefillStage stage, hipStream_t s, int splits,
                         const float* bias, int q_skip) {
  if (rows == 0) return hipSuccess;
  // few rows (decode): four heads per workgroup for parallelism; many rows
  // (prefill): all heads of four rows in one workgroup (the exponent pass:
  // one row per workgroup)
  const int hpw = rows >= 1024 ? Hq + Hkv : 4;
  if (splits < 1) return hipErrorInvalidValue;
  auto launch = [&](int mode) {
    const int rpw = rows >= 1024 && mode == 0 ? 4 : 1;
    const dim3 grid(cdiv(rows, rpw), cdiv(Hq + Hkv, hpw));
#define TDL_ROPE_KV(SB, F, R)                                                                            \
  rope_kv_kernel<SB, F, R><<<grid, 256, 0, s>>>((const float*)qkv, rows, Hq, Hkv, D, tab, q_norm, k_norm, \
                                                eps, (float*)q_out, seq, pool, stage, splits, bias, hpw,   \
                                                mode, q_skip)
#define TDL_ROPE_KV_R(SB, F)              \
  if (rpw == 4) TDL_ROPE_KV(SB, F, 4);    \
  else TDL_ROPE_KV(SB, F, 1);
#define TDL_ROPE_KV_SB(F)                   \
  if (splits == 1) { TDL_ROPE_KV_R(1, F) }  \
  else if (splits <= 4) { TDL_ROPE_KV_R(4, F) } \
  else { TDL_ROPE_KV_R(8, F) }
    if (pool.fmt == kKvU8) { TDL_ROPE_KV_SB(kKvU8) }
    else if (pool.fmt == kKvU4) { TDL_ROPE_KV_SB(kKvU4) }
    else { TDL_ROPE_KV_SB(kKvBf16) }
#undef TDL_ROPE_KV_SB
#undef TDL_ROPE_KV_R
#undef TDL_ROPE_KV
    return hipGetLastError();
  };
  if (pool.exps && pool.fmt != kKvBf16) {  // the blocks' exponents first
    const hipError_t e = launch(1);
    if (e != hipSuccess) return e;
  }
  return launch(0);
}

hipError_t kv_write_rows(const void* k, const void* v, int src_f32, int rows, int Hkv, int D,
                         SeqInfo seq, KvPool pool, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (pool.exps && pool.fmt != kKvBf16) {  // the blocks' exponents first
    kv_write_kernel<<<rows, 256, 0, s>>>(k, v, src_f32, Hkv, D, seq, pool, 1);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  kv_write_kernel<<<rows, 256, 0, s>>>(k, v, src_f32, Hkv, D, seq, pool, 0);
  return hipGetLastError();
}

hipError_t kv_calibrate(const float* x, int64_t n, int C, int levels, float* scale, int* zp,
                        hipStream_t s) {
  // min/max scratch lives in the zero-point array (int) and the scale array
  // reinterpreted as int until calib_finish overwrites both.
  int* mn = zp;
  int* mx = (int*)scale;
  minmax_init<<<cdiv(C, 256), 256, 0, s>>>(mn, mx, C);
  const int rows_per_block = 256;
  const int64_t nb = (n + rows_per_block - 1) / rows_per_block;
  if (nb > 0) {
    dim3 grid((unsigned)nb, cdiv(C, 256));
    minmax_kernel<<<grid, 256, 0, s>>>(x, n, C, rows_per_block, mn, mx);
  }
  calib_finish<<<cdiv(C, 256), 256, 0, s>>>(mn, mx, C, (float)levels, scale, zp);
  return hipGetLastError();
}

hipError_t rope_table_build(float2* tab, int max_pos, int D, double theta, hipStream_t s) {
  rope_table_kernel<<<1024, 256, 0, s>>>(tab, max_pos, D, theta);
  return hipGetLastError();
}

hipError_t convert_weights(const void* src, int src_f32, void* dst, int dst_f16, int64_t n,
                           int* n_saturated, hipStream_t s) {
  convert_kernel<<<2048, 256, 0, s>>>(src, src_f32, dst, dst_f16, n, n_saturated);
  return hipGetLastError();
}

hipError_t expand_q80(const void* codes, const void* scales, int N, int K, void* dst, int dst_f16,
                      hipStream_t s) {
  if (K % 32 != 0) return hipErrorInvalidValue;
  expand_q80_kernel<<<2048, 256, 0, s>>>((const int8_t*)codes, (const __half*)scales, N, K, dst, dst_f16);
  return hipGetLastError();
}

// Per-row symmetric int8 quantisation (the A8W8 path's activations): one
// workgroup per row, the row's absolute maximum by a block reduction, then
// codes round-half-even(x / s) with a correctly rounded fp32 divide, eight
// per thread and store.
template <typename T>
__global__ __launch_bounds__(256) void quant_rows_kernel(const T* __restrict__ x, int K, int8_t* __restrict__ q,
                                                         float* __restrict__ s) {
  const int row = blockIdx.x;
  const T* xr = x + (size_t)row * K;
  __shared__ float red[4];
  float m = 0.f;
  for (int k = threadIdx.x * 8; k < K; k += 256 * 8) {
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf((float)xr[k + e]));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float sc = m == 0.f ? 1.f : __fdiv_rn(m, 127.f);
  if (threadIdx.x == 0) s[row] = sc;
  int8_t* qr = q + (size_t)row * K;
  for (int k = threadIdx.x * 8; k < K; k += 256 * 8) {
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float c = __builtin_rintf(__fdiv_rn((float)xr[k + e], sc));
      c = fminf(fmaxf(c, -127.f), 127.f);
      w[e >> 2] |= ((uint32_t)(int)c & 0xffu) << (8 * (e & 3));
    }
    *(uint2*)(qr + k) = make_uint2(w[0], w[1]);
  }
}

hipError_t quant_rows_i8(const void* x, int x_bf16, int rows, int K, int8_t* q, float* s, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  if (K % 16) return hipErrorInvalidValue;
  if (x_bf16)
    quant_rows_kernel<bf16><<<rows, 256, 0, st>>>((const bf16*)x, K, q, s);
  else
    quant_rows_kernel<f16><<<rows, 256, 0, st>>>((const f16*)x, K, q, s);
  return hipGetLastError();
}

// GGUF Q8_0 blocks (34 bytes: binary16 scale, then 32 int8 codes) to split
// codes and scales; one thread per block, blocks in row-major order map to
// codes at 32 i and scales at i.  Reads in 2-byte words (the blocks are only
// 2-byte aligned), writes the codes as two 16-byte stores.
__global__ void q80_gguf_kernel(const uint16_t* __restrict__ blocks, int64_t n, int8_t* __restrict__ codes,
                                uint16_t* __restrict__ scales) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const uint16_t* b = blocks + 17 * i;
    uint32_t w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j] = (uint32_t)b[1 + 2 * j] | ((uint32_t)b[2 + 2 * j] << 16);
    scales[i] = b[0];
    uint4* dst = (uint4*)(codes + 32 * i);
    dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
    dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
  }
}

hipError_t q80_from_gguf(const void* blocks, int64_t n_blocks, void* codes, void* scales, hipStream_t s) {
  if (n_blocks == 0) return hipSuccess;
  const int grid = (int)std::min<int64_t>((n_blocks + 255) / 256, 4096);
  q80_gguf_kernel<<<grid, 256, 0, s>>>((const uint16_t*)blocks, n_blocks, (int8_t*)codes, (uint16_t*)scales);
  return hipGetLastError();
}

hipError_t expand_iq8(const void* codes, const float* scale, const float* zp, int N, int K, void* dst,
                      int dst_f16, hipStream_t s) {
  if (K % 8 != 0) return hipErrorInvalidValue;
  expand_iq8_kernel<<<2048, 256, 0, s>>>((const int8_t*)codes, scale, zp, N, K, dst, dst_f16);
  return hipGetLastError();
}

hipError_t i8_to_f32(const void* src, float* dst, int64_t n, hipStream_t s) {
  i8_to_f32_kernel<<<256, 256, 0, s>>>((const int8_t*)src, dst, n);
  return hipGetLastError();
}

hipError_t interleave_gate_up(const void* gate, const void* up, int row_bytes, int I, void* dst,
                              hipStream_t s) {
  interleave_kernel<<<2 * I, 256, 0, s>>>((const uint8_t*)gate, (const uint8_t*)up, row_bytes, I,
                                          (uint8_t*)dst);
  return hipGetLastError();
}

hipError_t pack_weights(const void* src, void* dst, int N, int K, hipStream_t s) {
  if (N % 16 != 0 || K % 32 != 0) return hipErrorInvalidValue;
  pack_kernel<<<2048, 256, 0, s>>>((const uint4*)src, (uint4*)dst, N, K);
  return hipGetLastError();
}

hipError_t pack_codes(const void* src, void* dst, int N, int K, hipStream_t s) {
  if (N % 16 != 0 || K % 64 != 0) return hipErrorInvalidValue;
  pack_codes_kernel<<<2048, 256, 0, s>>>((const int8_t*)src, (uint4*)dst, N, K);
  return hipGetLastError();
}

hipError_t copy_f32(const float* src, float* dst, int64_t n, hipStream_t s) {
  copy_f32_kernel<<<256, 256, 0, s>>>(src, dst, n);
  return hipGetLastError();
}

}  // namespace tdl
