// GEMM for decode-sized row counts (M <= 128): C = epilogue(A[M,K] B[N,K]^T)
// where the weight matrix B is streamed from HBM exactly once.
//
// With few rows every weight element is used only M times, so the kernel is
// bound by HBM bandwidth; what matters is keeping enough weight bytes in
// flight on every CU and never draining that stream.  Layout of the work:
//
//  * A workgroup owns a range of 16-row groups and a K range.  The N/16
//    groups are dealt out as evenly as possible over the row ranges (so
//    that, with one workgroup per CU, every CU streams the same bytes: the
//    busiest CU sets the time); a range has at most RW groups.  Its waves
//    form KW k-slices of RW row waves; a row wave streams its 16 rows over
//    its slice's part of the K range.  Spare row waves (range shorter than
//    RW) repeat the last live wave's loads -- cache hits -- so that every
//    wave issues the same loads, and store nothing.  (With the SiLU-gate
//    epilogue the gate and up rows of an output column sit in neighbouring
//    row waves, ranges hold whole pairs, and the two meet in LDS at the end.)
//  * Weights go straight from HBM into MFMA operand registers (16 bytes =
//    8 consecutive k of one row per lane), in NS rotating register sets: the
//    loads of stage s + NS - 1 are issued before the MFMAs of stage s, so
//    NS - 1 stages of every wave are always in flight.  In the packed tile
//    layout (pack_weights) a fragment is one contiguous 1 KB read; row-major
//    weights give each load 16 rows x 64 bytes, which HBM serves markedly
//    slower.
//  * The activations of a stage (all M rows x 64 k) are shared by the four
//    row waves of a slice: they go from global memory (L2-resident) into an
//    LDS ring of kStages buffers with direct-to-LDS loads, each of the four
//    waves fetching a quarter.  One wait on the load counter plus one
//    barrier per stage covers both the register and the LDS data (loads
//    complete in issue order).
//  * k-slices meet in LDS at the end; splits of K across workgroups (only
//    where the row count alone cannot fill the GPU) go through the shared
//    split-K reduction kernel.
//
// Q8_0 weights: a lane loads 8 int8 codes of its row per 32-k step plus the
// block's fp16 scale; the codes convert exactly to fp16 and the scale
// multiplies that step's MFMA product in fp32.  Per-row int8 weights (the
// per-channel weight-only GEMV of the devpress heterogeneous-engine page,
// section 4.4): a lane loads 8 codes per step; code - zero point (an
// integer in [-255, 255], exact in fp16 and bf16) is the MFMA operand, and
// the row's fp32 scale multiplies the finished sum once.

#include "common.h"
#include "kernels.h"

#include <algorithm>
#include <type_traits>

namespace tdl {

namespace {

constexpr int kStageK = 64;  // k per stage (two 32-k MFMA steps)
constexpr int kMaxStages = 8;

// Eight int8 codes (two words) as fp16 values c - off, for an integer off
// with |c - off| < 1024: the byte c ^ 0x80 = c + 128 under the exponent byte
// 0x64 is the fp16 number 1024 + c + 128 (one byte permute per two codes),
// and one packed subtract of 1152 + off leaves c - off exactly.
__device__ __forceinline__ f16x8 codes_to_f16(uint2 c, _Float16 off1152) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const uint32_t w[2] = {c.x ^ 0x80808080u, c.y ^ 0x80808080u};
  f16x8 o;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    // bytes (u0, 0x64, u1, 0x64) from (w, 0x64646464)
    const uint32_t bits = __builtin_amdgcn_perm(0x64646464u, w[q >> 1], (q & 1) ? 0x04030402u : 0x04010400u);
    const h2 v = __builtin_bit_cast(h2, bits) - h2{off1152, off1152};
    o[2 * q] = v.x;
    o[2 * q + 1] = v.y;
  }
  return o;
}

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding and leaves the other counters alone.
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | (((n >> 4) & 3) << 14); }

template <int WF, typename T> struct BFrag;
template <typename T> struct BFrag<kWDense, T> { typename Mfma<T>::v8 v; };
template <typename T> struct BFrag<kWQ80, T> { uint2 codes; uint32_t scale; };
template <typename T> struct BFrag<kWIQ8, T> { uint2 codes; };

// (at most 128 registers up to 64 rows of A: four waves per SIMD, i.e. two
// 8-wave workgroups per CU, so that every workgroup of a launch is resident
// at once; 128 rows of A need more and run two waves per SIMD; the 8-stage
// ring of the int8-code variants holds twice the LDS and halves both)
// RW row waves per k-slice (64 * RW / 4 ... 16 * RW weight rows per
// workgroup), NS pipeline stages (= LDS ring buffers = register sets).
template <typename T, int WF, int MT, int KW, int RW, int NS, int EPI, bool PACKED = false>
__global__ __launch_bounds__(64 * RW * KW) __attribute__((amdgpu_waves_per_eu((MT == 8 ? 2 : 4) / (NS > 4 ? 2 : 1))))
void gemm_stream_kernel(GemmArgs p) {
  constexpr bool Q80 = WF == kWQ80, IQ8 = WF == kWIQ8;
  constexpr int kRowWaves = RW, kStages = NS;
  static_assert(NS >= 3 && NS <= kMaxStages && RW % 2 == 0, "stream GEMM shape");
  typedef typename Mfma<T>::v8 T8;
  constexpr int FN = 1;                              // 16-row fragments per wave
  constexpr int AE = MT * 16 * kStageK;              // A elements per slice and stage
  constexpr int A_CHUNKS = 2 * MT;                   // 1 KB direct loads per slice and stage
  constexpr int A_PER_WAVE = (A_CHUNKS + RW - 1) / RW;  // per wave (the last chunk repeats)
  // packed int8 codes: one 16-byte load per stage (both 32-k steps), plus the
  // two block scales for Q8_0
  constexpr bool IQ8P = IQ8 && PACKED, Q80P = Q80 && PACKED;
  constexpr int LOADS = A_PER_WAVE + FN * (IQ8P ? 1 : Q80P ? 3 : 2 * (Q80 ? 2 : 1));  // vector-memory ops per stage
  // stages per barrier: the 1 KB stages of the 8-deep int8-code ring are
  // waited for and synchronised two at a time (the same bytes per barrier as
  // a 2 KB stage), keeping 6 stages in flight
  constexpr int SPB = IQ8 && NS == 8 ? 2 : 1;
  static_assert(NS % SPB == 0 && NS - 2 * SPB >= 1 && SPB <= 2, "stages per barrier");
  // separate arrays (not one indexed array): the compiler can then tell that
  // reading one buffer does not depend on the loads still filling another
  // (arrays past NS are never referenced and take no LDS)
  __shared__ __attribute__((aligned(16))) T ring0[KW * AE];
  __shared__ __attribute__((aligned(16))) T ring1[KW * AE];
  __shared__ __attribute__((aligned(16))) T ring2[KW * AE];
  __shared__ __attribute__((aligned(16))) T ring3[KW * AE];
  __shared__ __attribute__((aligned(16))) T ring4[KW * AE];
  __shared__ __attribute__((aligned(16))) T ring5[KW * AE];
  __shared__ __attribute__((aligned(16))) T ring6[KW * AE];
  __shared__ __attribute__((aligned(16))) T ring7[KW * AE];
  T* const rings[kMaxStages] = {ring0, ring1, ring2, ring3, ring4, ring5, ring6, ring7};

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave % kRowWaves, wk = wave / kRowWaves;
  // this workgroup's row range (ng <= RW groups from row n0) and K split
  constexpr int PG = EPI == EPI_SILU_GATE ? 2 : 1;  // groups per unit dealt out
  const int units = cdiv(p.N, 16) / PG;
  const int rng = blockIdx.x % p.rng_count;
  const int split = blockIdx.x / p.rng_count;
  const int g0 = (int)((long)rng * units / p.rng_count) * PG;
  const int ng = (int)((long)(rng + 1) * units / p.rng_count) * PG - g0;
  const int n0 = g0 * 16;
  const bool live = wr < ng;
  const int KS32 = p.K / 32;
  const int KS = cdiv(KS32, 2);                       // stages over the whole K
  const int ks0 = split * p.k_tiles_per_split;        // this split's stages
  const int ks1 = min(ks0 + p.k_tiles_per_split, KS);
  const int per_slice = cdiv(max(ks1 - ks0, 0), KW);  // stages per slice (all slices alike)
  const int my0 = ks0 + wk * per_slice;               // this slice's stages: [my0, my1)
  const int my1 = min(my0 + per_slice, ks1);
  const int last = max(my1 - 1, 0);                   // loads past the end repeat the last stage
  // the single-stage ring runs whole turns (an exit test per step measured
  // slower for it); the paired ring's last turn stops after the slice's last
  // stage (the same count for every wave of the workgroup), and what it
  // issued past that point is drained after the loop
  const int n_iter = SPB > 1 ? per_slice : cdiv(per_slice, kStages) * kStages;

  const T* __restrict__ A = (const T*)p.A;
  const int r16 = lane & 15, g8 = (lane >> 4) * 8;

  // this wave's direct-load chunks of A: chunk c = tokens 8c .. 8c+7, lane
  // L loads token 8c + L/8 into 16-byte position L%8, holding source chunk
  // (L%8) ^ (token%8); chunks past the stage repeat the last one (the same
  // bytes to the same place)
  const T* a_src[A_PER_WAVE];
  int a_dst[A_PER_WAVE];
#pragma unroll
  for (int q = 0; q < A_PER_WAVE; ++q) {
    const int c = min(wr * A_PER_WAVE + q, A_CHUNKS - 1);
    const int t = 8 * c + (lane >> 3);
    a_src[q] = A + (size_t)min(t, p.M - 1) * p.lda + (((lane & 7) ^ (t & 7)) << 3);
    a_dst[q] = wk * AE + 8 * c * kStageK;
  }
  const int a_c8 = ((lane & 7) ^ ((lane >> 3) & 7)) << 3;  // that chunk's first k

  // weight rows of this lane: spare waves repeat the last live wave's rows;
  // rows past N are clamped (computed, never stored)
  size_t b_row[FN];
#pragma unroll
  for (int f = 0; f < FN; ++f) b_row[f] = (size_t)min(n0 + 16 * (min(wr, ng - 1) * FN + f) + r16, p.N - 1);

  BFrag<WF, T> breg[kStages][FN][2];
  // per-row int8: this lane's row scale and zero point
  float rsc[FN], rzp[FN];
  _Float16 zp1152[FN];  // 1152 + zero point, exact in fp16 (|zp| <= 128)
#pragma unroll
  for (int f = 0; f < FN; ++f) {
    rsc[f] = IQ8 ? p.B_rscale[b_row[f]] : 1.f;
    rzp[f] = IQ8 ? p.B_rzp[b_row[f]] : 0.f;
    zp1152[f] = (_Float16)(1152.f + rzp[f]);
  }
  f32x4 acc[MT][FN];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int f = 0; f < FN; ++f) acc[i][f] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto issue = [&](int it, T* ring, BFrag<WF, T> (&b)[FN][2]) {
    const int st = min(my0 + it, last);
    const int k0 = st * kStageK;
    // A: the whole stage chunk; a k past K (a half stage at the end) reads
    // the row's first chunk instead, multiplied by zeroed weights
    const int a_off = k0 + a_c8 < p.K ? k0 : -a_c8;
#pragma unroll
    for (int q = 0; q < A_PER_WAVE; ++q)
      __builtin_amdgcn_global_load_lds((const void*)(a_src[q] + a_off), (lds_void*)&ring[a_dst[q]], 16, 0,
                                       0);
    if constexpr (IQ8P || Q80P) {
      // tile (stage, row group): one contiguous 1 KB read per wave
#pragma unroll
      for (int f = 0; f < FN; ++f) {
        const uint4 c = *(const uint4*)((const int8_t*)p.B +
                                        ((size_t)st * (p.N >> 4) + (b_row[f] >> 4)) * 1024 + lane * 16);
        b[f][0].codes = make_uint2(c.x, c.y);
        b[f][1].codes = make_uint2(c.z, c.w);
        if constexpr (Q80P) {
#pragma unroll
          for (int u = 0; u < 2; ++u)
            b[f][u].scale = *(const uint16_t*)(p.B_scale + b_row[f] * (p.ldb / 32) + min(2 * st + u, KS32 - 1));
        }
      }
      return;
    }
#pragma unroll
    for (int f = 0; f < FN; ++f)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int ks = min(2 * st + u, KS32 - 1);
        const int k = ks * 32 + g8;
        if constexpr (Q80) {
          b[f][u].codes = *(const uint2*)((const int8_t*)p.B + b_row[f] * p.ldb + k);
          b[f][u].scale = *(const uint16_t*)(p.B_scale + b_row[f] * (p.ldb / 32) + ks);
        } else if constexpr (IQ8) {
          b[f][u].codes = *(const uint2*)((const int8_t*)p.B + b_row[f] * p.ldb + k);
        } else if constexpr (PACKED) {
          // fragment = chunk `lane` of tile (row group, ks): one 1 KB read
          b[f][u].v = *(const T8*)((const T*)p.B + ((size_t)ks * (p.N >> 4) + (b_row[f] >> 4)) * 512 + lane * 8);
        } else {
          b[f][u].v = *(const T8*)((const T*)p.B + b_row[f] * p.ldb + k);
        }
      }
  };

  auto compute = [&](int it, const T* ring, const BFrag<WF, T> (&b)[FN][2]) {
    const int st = my0 + it;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const bool valid = st < my1 && 2 * st + u < KS32;
      T8 bv[FN];
      float sc[FN];
#pragma unroll
      for (int f = 0; f < FN; ++f) {
        if constexpr (Q80 && std::is_same<T, f16>::value) {
          bv[f] = codes_to_f16(b[f][u].codes, (_Float16)1152.f);
          sc[f] = valid ? __half2float(__ushort_as_half((unsigned short)b[f][u].scale)) : 0.f;
        } else if constexpr (Q80) {
          T8 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[e] = (T)(float)(int8_t)(b[f][u].codes.x >> (8 * e));
            v[4 + e] = (T)(float)(int8_t)(b[f][u].codes.y >> (8 * e));
          }
          bv[f] = v;
          sc[f] = valid ? __half2float(__ushort_as_half((unsigned short)b[f][u].scale)) : 0.f;
        } else if constexpr (IQ8 && std::is_same<T, f16>::value) {
          bv[f] = valid ? codes_to_f16(b[f][u].codes, zp1152[f]) : T8{};
        } else if constexpr (IQ8) {
          T8 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[e] = (T)((float)(int8_t)(b[f][u].codes.x >> (8 * e)) - rzp[f]);
            v[4 + e] = (T)((float)(int8_t)(b[f][u].codes.y >> (8 * e)) - rzp[f]);
          }
          bv[f] = valid ? v : T8{};
        } else {
          bv[f] = valid ? b[f][u].v : T8{};
        }
      }
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        // token 16i + r16, chunk 4u + lane/16, swizzled by token % 8 = lane % 8
        const T8 a = *(const T8*)&ring[wk * AE + (16 * i + r16) * kStageK +
                                       (((4 * u + (lane >> 4)) ^ (lane & 7)) << 3)];
#pragma unroll
        for (int f = 0; f < FN; ++f) {
          if constexpr (Q80) {
            const f32x4 t = Mfma<T>::mma(a, bv[f], f32x4{0.f, 0.f, 0.f, 0.f});
            acc[i][f] += t * sc[f];
          } else {
            acc[i][f] = Mfma<T>::mma(a, bv[f], acc[i][f]);
          }
        }
      }
    }
  };

  // one pipeline step: wait for stage it (kStages - 2 later stages may stay
  // in flight), barrier (every wave's share of the A chunk has landed and
  // every wave is done with the buffer refilled next), refill, compute.
  // Scheduling barriers keep the compiler from moving register reads of a
  // stage's loads, or the loads themselves, across these points: the wait
  // counts assume program order.  The paired ring's step does the same for
  // two stages (kStages - 4 later ones in flight), the second refill issued
  // between the two computes (the loads keep their order, so the counts
  // hold; both buffers were freed before the barrier).
  if constexpr (SPB == 1) {
#pragma unroll
    for (int j = 0; j < kStages - 1; ++j) issue(j, rings[j], breg[j]);
    for (int it = 0; it < n_iter; it += kStages) {
#pragma unroll
      for (int j = 0; j < kStages; ++j) {
        const int jn = (j + kStages - 1) % kStages;
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm((kStages - 2) * LOADS));
        asm volatile("s_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        issue(it + j + kStages - 1, rings[jn], breg[jn]);
        __builtin_amdgcn_sched_barrier(0);
        compute(it + j, rings[j], breg[j]);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < kStages - 2; ++j) issue(j, rings[j], breg[j]);
    for (int it = 0; it < n_iter; it += kStages) {
#pragma unroll
      for (int j = 0; j < kStages; j += 2) {
        if (it + j >= per_slice) break;
        const int jn = (j + kStages - 2) % kStages;
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm((kStages - 4) * LOADS));
        asm volatile("s_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        issue(it + j + kStages - 2, rings[jn], breg[jn]);
        __builtin_amdgcn_sched_barrier(0);
        compute(it + j, rings[j], breg[j]);
        __builtin_amdgcn_sched_barrier(0);
        issue(it + j + kStages - 1, rings[jn + 1], breg[jn + 1]);
        __builtin_amdgcn_sched_barrier(0);
        compute(it + j + 1, rings[j + 1], breg[j + 1]);
      }
    }
  }
  // the last refills are still landing in the ring: drain them before the
  // ring is reused or the workgroup exits
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  if constexpr (IQ8) {  // the row scale, once per output (and per partial)
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int f = 0; f < FN; ++f) acc[i][f] *= rsc[f];
  }

  // ---- k-slices meet in LDS, summed in a fixed order
  if constexpr (KW > 1) {
    f32x4* red = (f32x4*)ring0;  // (KW-1) x RW waves x MT x 64 lanes x 16 B <= ring0
    static_assert((KW - 1) * kRowWaves * MT * 64 * 16 <= KW * AE * (int)sizeof(T), "ring0 too small");
    __syncthreads();
    if (wk > 0) {
#pragma unroll
      for (int i = 0; i < MT; ++i) red[(((wk - 1) * kRowWaves + wr) * MT + i) * 64 + lane] = acc[i][0];
    }
    __syncthreads();
    if (wk == 0) {
#pragma unroll
      for (int w = 1; w < KW; ++w)
#pragma unroll
        for (int i = 0; i < MT; ++i) acc[i][0] += red[(((w - 1) * kRowWaves + wr) * MT + i) * 64 + lane];
    }
  }

  // from here on slice 0 holds the sums: acc[i][0][r] =
  // C[16i + 4*(lane/16) + r][n0 + 16*wr + lane%16]
  const int rb = 4 * (lane >> 4);
  const int n = n0 + 16 * wr + r16;
  if (p.splits > 1) {
    if (wk > 0 || !live || n >= p.N) return;
    float* part = p.ws + (size_t)split * p.M * p.N;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 16 * i + rb + r;
        if (m < p.M) part[(size_t)m * p.N + n] = acc[i][0][r];
      }
    return;
  }
  if constexpr (EPI == EPI_SILU_GATE) {
    // row waves 2j hold gate rows n0 + 32j + [0,16), waves 2j+1 the matching
    // up rows: the up waves hand their sums over through LDS (two pairs per
    // ring buffer, from buffer 1 on)
    const int pair = wr >> 1;
    f32x4* xch = (f32x4*)(pair < 2 ? ring1 : pair < 4 ? ring2 : ring3) + (pair % 2) * MT * 64;
    static_assert(2 * MT * 64 * 16 <= KW * AE * (int)sizeof(T) && 1 + (RW / 2 - 1) / 2 < NS && RW <= 12,
                  "exchange space");
    __syncthreads();  // every wave is done reading the ring
    if (wk == 0 && (wr & 1)) {
#pragma unroll
      for (int i = 0; i < MT; ++i) xch[i * 64 + lane] = acc[i][0];
    }
    __syncthreads();
    if (wk > 0 || (wr & 1) || !live || n >= p.N) return;
    const int jcol = (n0 + 16 * wr) / 2 + r16;
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const f32x4 up = xch[i * 64 + lane];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 16 * i + rb + r;
        if (m < p.M) {
          const float g = acc[i][0][r];
          ((bf16*)p.C)[(size_t)m * p.ldc + jcol] = f32_to_bf16(g / (1.0f + __expf(-g)) * up[r]);
        }
      }
    }
  } else {
    if (wk > 0 || !live || n >= p.N) return;
    // the residual is never the output: its loads all issue before the
    // stores, unconditionally from clamped addresses (a guarded load would
    // be a branch that waits for its own result)
    const bf16* __restrict__ Rb = (const bf16*)p.resid;
    const float* __restrict__ Rf = (const float*)p.resid;
    const float bias = (EPI == EPI_BIAS_F32 && p.bias) ? p.bias[n] : 0.f;
    float add[MT][4];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const size_t off = (size_t)min(16 * i + rb + r, p.M - 1) * p.ldr + n;
        if constexpr (EPI == EPI_BIAS_F32) add[i][r] = bias;
        else if constexpr (EPI == EPI_RESID_F32) add[i][r] = bf16_to_f32(Rb[off]);
        else add[i][r] = Rf[off];
      }
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 16 * i + rb + r;
        if (m >= p.M) continue;
        const float v = acc[i][0][r] + add[i][r];
        if constexpr (EPI == EPI_RESID_BF16) ((bf16*)p.C)[(size_t)m * p.ldc + n] = f32_to_bf16(v);
        else ((float*)p.C)[(size_t)m * p.ldc + n] = v;
      }
  }
}

template <int WF, int MT, int KW, int RW, int NS, bool PK>
hipError_t launch_stream2(int grid, int epi, const GemmArgs& a, hipStream_t s) {
  constexpr int threads = 64 * RW * KW;
  switch (epi) {
    case EPI_BIAS_F32:
      gemm_stream_kernel<f16, WF, MT, KW, RW, NS, EPI_BIAS_F32, PK><<<grid, threads, 0, s>>>(a);
      break;
    case EPI_RESID_F32:
      gemm_stream_kernel<f16, WF, MT, KW, RW, NS, EPI_RESID_F32, PK><<<grid, threads, 0, s>>>(a);
      break;
    case EPI_RESID_BF16:
      gemm_stream_kernel<bf16, WF, MT, KW, RW, NS, EPI_RESID_BF16, PK><<<grid, threads, 0, s>>>(a);
      break;
    default:
      gemm_stream_kernel<f16, WF, MT, KW, RW, NS, EPI_SILU_GATE, PK><<<grid, threads, 0, s>>>(a);
      break;
  }
  return hipGetLastError();
}

template <int WF, int MT, int KW, int RW, int NS>
hipError_t launch_stream(int grid, int epi, const GemmArgs& a, hipStream_t s) {
  if constexpr (WF != kWDense) {
    return a.b_packed ? launch_stream2<WF, MT, KW, RW, NS, true>(grid, epi, a, s)
                      : launch_stream2<WF, MT, KW, RW, NS, false>(grid, epi, a, s);
  } else {
    return a.b_packed ? launch_stream2<kWDense, MT, KW, RW, NS, true>(grid, epi, a, s)
                      : launch_stream2<kWDense, MT, KW, RW, NS, false>(grid, epi, a, s);
  }
}

}  // namespace

// Shapes of the stream kernel that are built: (MT, RW, NS, KW).
// cfg = 10000 + 1000 * MT + 100 * RW + 10 * NS + KW.
int stream_cfg(int MT, int RW, int NS, int KW) { return 10000 + 1000 * MT + 100 * RW + 10 * NS + KW; }

// Row waves per workgroup that are built (RW), and the pipeline depth: 4
// stages of 2 KB per wave (bf16/fp16, Q8_0); per-row int8 stages carry 1 KB
// (64 k of 16 rows): an 8-buffer ring, waited for and synchronised two
// stages at a time, keeps 6 of them in flight, twice the stages of bf16's
// 3 and as many bytes, at the same bytes per barrier.
constexpr int kStreamRW[3] = {4, 8, 10};
constexpr int kStreamNS = 4;
constexpr int kStreamNSIQ8 = 8;

// Chooses (RW, row ranges, K splits) by a model of the decode-sized stream,
// fitted to measurements on the Qwen2.5-7B decode shapes: a CU streams its
// weight bytes at ~1.5 us latency with its stages in flight (2 KB each) per
// live row wave, up to ~22 GB/s, and the GPU at ~5.5 TB/s; the busiest CU
// sets the time.  K splits add streams (and fp32 partials that are written
// and read once more).
bool skinny_plan(int M, int N, int K, int wf, int epi, GemmPlan* pl) {
  if (M > 128 || K % 32 != 0) return false;
  constexpr int kCUs = 256;
  const int MT = M <= 32 ? 2 : M <= 64 ? 4 : 8;
  const int PG = epi == EPI_SILU_GATE ? 2 : 1;
  const int units = cdiv(N, 16) / PG;
  if (units < 1) return false;
  const int KS = cdiv(K / 32, 2);
  // weight bytes per element (Q8_0: + fp16 scale per 32)
  const double wb = wf == kWQ80 ? 1.0625 : wf == kWIQ8 ? 1.0 : 2.0;
  const double total = (double)N * K * wb;
  // Spare row waves (a range shorter than RW), which repeat a live wave's
  // loads and MFMAs, slow the live ones: rate x live/RW.  4-wave
  // workgroups (two per CU, each loading its own A chunks) measured slower
  // than 8-wave ones on every decode shape.  128 rows of A (MT 8): each
  // weight byte costs twice the MFMA and LDS work, so a live row wave
  // streams slower (measured on the Qwen3-8B shapes: ~2.7 GB/s against ~4
  // at 64 rows).
  const bool big = MT == 8;
  const double wave_lat = big ? 2.3e-6 : 1.5e-6;
  const int NS = wf == kWIQ8 ? kStreamNSIQ8 : kStreamNS;
  const double stage_bytes = wf == kWIQ8 ? 1024.0 : 2048.0;  // per live row wave
  const int in_flight = wf == kWIQ8 ? NS - 2 : NS - 1;  // stages in flight during a compute
  double best = 1e300;
  for (int RW : kStreamRW) {
    if (RW < 8 && units > 16) continue;  // (tiny N: too few row groups for 8 waves)
    const int per = RW / PG;  // units per range at most
    const int rmin = cdiv(units, per);
    for (int s = 1; s <= 16; ++s) {
      const int kps = cdiv(KS, s), sp = cdiv(KS, kps);
      if (sp != s || (sp > 1 && kps < 2 * (in_flight + 1))) continue;
      const int cands[3] = {rmin, kCUs / sp, 2 * kCUs / sp};
      for (int R : cands) {
        if (R < rmin || R > units || R < 1) continue;
        const int W = R * sp;
        const int wg_per_cu = cdiv(W, kCUs);
        const int groups = cdiv(units, R) * PG;          // live row waves of the largest range
        const double wg_bytes = (double)groups * 16 * kps * 64 * wb;
        double rate = std::min(22e9, wg_per_cu * groups * in_flight * stage_bytes / wave_lat);
        rate *= (double)groups / RW;
        double t = std::max(wg_per_cu * wg_bytes / rate, total / 5.5e12);
        if (sp > 1) t += 2.0 * sp * (double)M * N * 4.0 / 5.0e12;
        t += 1e-9 * RW;  // ties: fewer waves
        if (t < best) {
          best = t;
          *pl = GemmPlan{};
          pl->cfg = stream_cfg(MT, RW, NS, 1);
          pl->rng_count = R;
          pl->splits = sp;
          pl->k_tiles_per_split = kps;
          pl->grid = W;
          pl->ws_floats = sp > 1 ? (size_t)sp * M * N : 0;
        }
      }
    }
  }
  return best < 1e300;
}

hipError_t gemm_skinny_launch(const GemmPlan& pl, const GemmArgs& a, int wf, int epi,
                              hipStream_t s) {
#define TDL_STREAM_CFG(MT, RW, NS, KW)                                                      \
  if (pl.cfg == stream_cfg(MT, RW, NS, KW))                                                 \
    return wf == kWQ80   ? launch_stream<kWQ80, MT, KW, RW, NS>(pl.grid, epi, a, s)         \
           : wf == kWIQ8 ? launch_stream<kWIQ8, MT, KW, RW, NS>(pl.grid, epi, a, s)         \
                         : launch_stream<kWDense, MT, KW, RW, NS>(pl.grid, epi, a, s);
  TDL_STREAM_CFG(2, 4, 4, 1) TDL_STREAM_CFG(2, 8, 4, 1) TDL_STREAM_CFG(2, 10, 4, 1)
  TDL_STREAM_CFG(4, 4, 4, 1) TDL_STREAM_CFG(4, 8, 4, 1) TDL_STREAM_CFG(4, 10, 4, 1)
  TDL_STREAM_CFG(8, 4, 4, 1) TDL_STREAM_CFG(8, 8, 4, 1) TDL_STREAM_CFG(8, 10, 4, 1)
#undef TDL_STREAM_CFG
#define TDL_STREAM_CFG_IQ8(MT, RW, NS, KW)                                                  \
  if (pl.cfg == stream_cfg(MT, RW, NS, KW) && wf == kWIQ8)                                  \
    return launch_stream<kWIQ8, MT, KW, RW, NS>(pl.grid, epi, a, s);
  TDL_STREAM_CFG_IQ8(2, 4, 8, 1) TDL_STREAM_CFG_IQ8(2, 8, 8, 1) TDL_STREAM_CFG_IQ8(2, 10, 8, 1)
  TDL_STREAM_CFG_IQ8(4, 4, 8, 1) TDL_STREAM_CFG_IQ8(4, 8, 8, 1) TDL_STREAM_CFG_IQ8(4, 10, 8, 1)
  TDL_STREAM_CFG_IQ8(8, 4, 8, 1) TDL_STREAM_CFG_IQ8(8, 8, 8, 1) TDL_STREAM_CFG_IQ8(8, 10, 8, 1)
#undef TDL_STREAM_CFG_IQ8
  return hipErrorInvalidValue;
}

}  // namespace tdl
