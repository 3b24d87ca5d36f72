// GEMM for decode-sized row counts (M <= 128): C = epilogue(A[M,K] B[N,K]^T)
// where the weight matrix B is streamed from HBM exactly once.
//
// With few rows every weight element is used only M times, so the kernel is
// bound by HBM bandwidth, not by the matrix cores.  The design therefore
// keeps as many weight bytes in flight as possible and touches no LDS on the
// streaming path: each lane loads its MFMA operand fragments straight from
// global memory (16 bytes = 8 consecutive k of one row), for the weights
// from HBM and for the activations from L2, where the small A matrix stays
// resident.  A workgroup owns 64 weight rows; its four waves take contiguous
// quarters of the workgroup's K range, so each wave streams 64 rows x its
// quarter, with the loads of the next k32-steps in flight while the
// current ones feed the MFMAs.  The four
// partial sums meet in LDS; when the K range is also split across
// workgroups (long K, few rows of N) the slices go to memory and the shared
// split-K reduction kernel finishes them.
//
// Q8_0 weights: lane loads 8 int8 codes (one 32-code block per k32 step
// across the four lane groups), converts them exactly, and the block's fp16
// scale multiplies that MFMA's partial product.

#include "common.h"
#include "kernels.h"

namespace tdl {

namespace {

constexpr int kU = 2;  // k32 steps per load group

template <typename T, bool Q80, int MT, int EPI>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(GemmArgs p) {
  typedef typename Mfma<T>::v8 T8;
  constexpr int FN = 4;  // 64 weight rows per workgroup, 16 per MFMA tile
  __shared__ f32x4 red[3][MT][FN][64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n_tiles = cdiv(p.N, 64);
  const int split = blockIdx.x / n_tiles;
  const int n0 = (blockIdx.x % n_tiles) * 64;
  const int KS = p.K / 32;                          // k32 steps
  const int s0 = split * p.k_tiles_per_split;       // this workgroup's steps
  const int s1 = min(s0 + p.k_tiles_per_split, KS);
  const int per_wave = cdiv(s1 - s0, 4);
  const int w0 = s0 + wave * per_wave;
  const int w1 = min(w0 + per_wave, s1);
  const int r16 = lane & 15, g8 = (lane >> 4) * 8;

  const T* __restrict__ A = (const T*)p.A;
  const T* arow[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) arow[i] = A + (size_t)min(16 * i + r16, p.M - 1) * p.lda + g8;
  size_t brow[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) brow[j] = (size_t)min(n0 + 16 * j + r16, p.N - 1);

  f32x4 acc[MT][FN];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // one k32 step of operands: 4 weight fragments (+ Q8_0 scales), MT
  // activation fragments.  Steps past the wave's range load from a clamped
  // (valid) address and zero their activation fragments, so the loop below
  // needs no branches and the compiler can count outstanding loads exactly.
  struct Step {
    T8 b[FN];
    T8 a[MT];
    float sc[Q80 ? FN : 1];
    bool valid;
  };
  auto load = [&](Step& st, int step) {
    st.valid = step < w1;
    const int k = min(step, KS - 1) * 32;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      if constexpr (Q80) {
        const uint2 c = *(const uint2*)((const int8_t*)p.B + brow[j] * p.ldb + k + g8);
        T8 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = (T)(float)(int8_t)(c.x >> (8 * e));
          v[4 + e] = (T)(float)(int8_t)(c.y >> (8 * e));
        }
        st.b[j] = v;
        st.sc[j] = __half2float(p.B_scale[brow[j] * (p.ldb / 32) + (k >> 5)]);
      } else {
        st.b[j] = *(const T8*)((const T*)p.B + brow[j] * p.ldb + k + g8);
      }
    }
#pragma unroll
    for (int i = 0; i < MT; ++i) st.a[i] = *(const T8*)(arow[i] + k);
  };
  auto mma = [&](const Step& st) {
    T8 a[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) a[i] = st.valid ? st.a[i] : T8{};
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        if constexpr (Q80) {
          const f32x4 t = Mfma<T>::mma(a[i], st.b[j], f32x4{0.f, 0.f, 0.f, 0.f});
          acc[i][j] += t * st.sc[j];
        } else {
          acc[i][j] = Mfma<T>::mma(a[i], st.b[j], acc[i][j]);
        }
      }
  };

  // groups of kU steps: the next group's loads are issued before this
  // group's MFMAs, so a group's worth of weight bytes is always in flight
  // (two register sets used alternately: no copies between iterations,
  // whose reads of freshly loaded registers would force a wait)
  const int n_groups = w1 > w0 ? cdiv(w1 - w0, kU) : 0;
  Step sa[kU], sb[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) load(sa[u], w0 + u);
  for (int gi = 0; gi < n_groups; gi += 2) {
#pragma unroll
    for (int u = 0; u < kU; ++u) load(sb[u], w0 + (gi + 1) * kU + u);
#pragma unroll
    for (int u = 0; u < kU; ++u) mma(sa[u]);
#pragma unroll
    for (int u = 0; u < kU; ++u) load(sa[u], w0 + (gi + 2) * kU + u);
#pragma unroll
    for (int u = 0; u < kU; ++u) mma(sb[u]);
  }

  // ---- the four waves' partial sums meet in LDS (fixed order: 0+1+2+3)
  if (wave > 0) {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) red[wave - 1][i][j][lane] = acc[i][j];
  }
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int w = 0; w < 3; ++w)
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] += red[w][i][j][lane];

  // acc[i][j][r] = C[16i + 4*(lane/16) + r][n0 + 16j + lane%16]
  const int col = lane & 15;
  const int rb = 4 * (lane >> 4);
  if (p.splits > 1) {
    float* part = p.ws + (size_t)split * p.M * p.N;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = n0 + 16 * j + col;
      if (n >= p.N) continue;
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = 16 * i + rb + r;
          if (m < p.M) part[(size_t)m * p.N + n] = acc[i][j][r];
        }
    }
    return;
  }
  if constexpr (EPI == EPI_SILU_GATE) {
#pragma unroll
    for (int jp = 0; jp < FN / 2; ++jp) {
      const int ng = n0 + 32 * jp;
      if (ng + col >= p.N) continue;
      const int jcol = ng / 2 + col;
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = 16 * i + rb + r;
          if (m < p.M) {
            const float g = acc[i][2 * jp][r], u = acc[i][2 * jp + 1][r];
            ((bf16*)p.C)[(size_t)m * p.ldc + jcol] = f32_to_bf16(g / (1.0f + __expf(-g)) * u);
          }
        }
    }
  } else {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = n0 + 16 * j + col;
      if (n >= p.N) continue;
      const float bias = (EPI == EPI_BIAS_F32 && p.bias) ? p.bias[n] : 0.f;
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = 16 * i + rb + r;
          if (m >= p.M) continue;
          const float v = acc[i][j][r];
          if constexpr (EPI == EPI_BIAS_F32) {
            ((float*)p.C)[(size_t)m * p.ldc + n] = v + bias;
          } else if constexpr (EPI == EPI_RESID_F32) {
            ((float*)p.C)[(size_t)m * p.ldc + n] =
                v + bf16_to_f32(((const bf16*)p.resid)[(size_t)m * p.ldr + n]);
          } else {
            ((bf16*)p.C)[(size_t)m * p.ldc + n] =
                f32_to_bf16(v + ((const float*)p.resid)[(size_t)m * p.ldr + n]);
          }
        }
    }
  }
}

template <bool Q80, int MT>
hipError_t launch_mt(int grid, int epi, const GemmArgs& a, hipStream_t s) {
  switch (epi) {
    case EPI_BIAS_F32:
      gemm_skinny_kernel<f16, Q80, MT, EPI_BIAS_F32><<<grid, 256, 0, s>>>(a);
      break;
    case EPI_RESID_F32:
      gemm_skinny_kernel<f16, Q80, MT, EPI_RESID_F32><<<grid, 256, 0, s>>>(a);
      break;
    case EPI_RESID_BF16:
      gemm_skinny_kernel<bf16, Q80, MT, EPI_RESID_BF16><<<grid, 256, 0, s>>>(a);
      break;
    default:
      gemm_skinny_kernel<f16, Q80, MT, EPI_SILU_GATE><<<grid, 256, 0, s>>>(a);
      break;
  }
  return hipGetLastError();
}

}  // namespace

bool skinny_plan(int M, int N, int K, GemmPlan* pl) {
  if (M > 128 || K % 32 != 0) return false;
  const int n_tiles = cdiv(N, 64);
  const int KS = K / 32;
  // split K across workgroups until there are ~2 per CU, keeping >= 16 k32
  // steps (4 per wave) per workgroup
  int splits = 1;
  while (n_tiles * splits < 480 && KS / (splits * 2) >= 16) splits *= 2;
  pl->cfg = M <= 64 ? 10 : 11;
  pl->k_tiles_per_split = cdiv(KS, splits);
  pl->splits = cdiv(KS, pl->k_tiles_per_split);
  pl->grid = n_tiles * pl->splits;
  pl->ws_floats = pl->splits > 1 ? (size_t)pl->splits * M * N : 0;
  return true;
}

hipError_t gemm_skinny_launch(const GemmPlan& pl, const GemmArgs& a, bool q80, int epi,
                              hipStream_t s) {
  if (pl.cfg == 10) return q80 ? launch_mt<true, 4>(pl.grid, epi, a, s) : launch_mt<false, 4>(pl.grid, epi, a, s);
  return q80 ? launch_mt<true, 8>(pl.grid, epi, a, s) : launch_mt<false, 8>(pl.grid, epi, a, s);
}

}  // namespace tdl
