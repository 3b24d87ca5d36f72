// bf16 / Q8_0 GEMM for gfx950: C = epilogue(A[M,K] * B[N,K]^T).
//
// Both operands are K-contiguous (the row-major "out = in @ W^T" form with W
// stored [out, in], as the Qwen2.5-7B single-layer page derives in its
// section 4 "cuBLAS Row-Major 陷阱"), which is the natural operand order of
// the MFMA units: every lane feeds 8 consecutive k values of one row of A
// and one row of B.
//
// Structure: a BM x BN x 64 tile per workgroup, staged through LDS with
// double buffering (global loads of tile k+1 in flight while tile k feeds
// the MFMAs); LDS rows are 128 bytes and the 16-byte chunk index is XOR-ed
// with (row & 7) so the 16 lanes of an MFMA operand read hit distinct banks
// (the swizzle idea of the TFFInfer page, section 3.7.2 item 3, re-derived
// for 64-lane ds_read_b128).  Each wave owns a (BM/WM) x (BN/WN) sub-tile of
// 16x16 MFMA accumulators.
//
// Q8_0 weights (blocks of 32 int8 codes with one fp16 scale along K): the
// codes convert exactly to bf16 when staged to LDS; one 16x16x32 MFMA covers
// exactly one block, and its partial product is scaled by the block's scale
// before accumulation, so the result is the exact W8 x bf16 product up to
// fp32 rounding (no activation quantisation).
//
// Split-K: the K range is cut into `splits` slices; each workgroup writes its
// fp32 partial tile, and the last workgroup to arrive on a tile (an arrival
// counter, reset by that workgroup) sums the partials in slice order --
// deterministic -- and runs the epilogue.
//
// Epilogues: bias (QKV projection), residual add (output and down
// projections) and SiLU-gate (the gate/up projection writes only
// silu(gate) * up; gate and up rows alternate in groups of 16).
//
// Operand type T is bf16 or fp16 (same MFMA rate on gfx950).  The layer uses
// fp16 where the activation is bounded (RMSNorm outputs, attention output)
// for its three extra significant bits, bf16 where it is not (the SwiGLU
// product feeding the down projection).

#include "common.h"
#include "kernels.h"

namespace tdl {

namespace {

constexpr int BK = 64;  // k elements per tile (128 bytes of bf16 per row)

__device__ __forceinline__ int swz(int row, int chunk) {  // offset in bf16 elements
  return row * BK + ((chunk ^ (row & 7)) << 3);
}

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + __expf(-z)); }

template <int BM, int BN, int WM, int WN, bool Q80, int EPI, typename T>
__global__ __launch_bounds__(WM* WN * 64) void gemm_kernel(GemmArgs p) {
  typedef typename Mfma<T>::v8 T8;
  constexpr int NT = WM * WN * 64;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  constexpr int A_CHUNKS = BM * BK / 8;            // 16-byte chunks per A tile
  constexpr int B_CHUNKS = Q80 ? BN * BK / 16 : BN * BK / 8;  // global chunks
  constexpr int A_PER_T = (A_CHUNKS + NT - 1) / NT;
  constexpr int B_PER_T = (B_CHUNKS + NT - 1) / NT;
  static_assert(FM >= 1 && FN >= 1, "wave tile");
  static_assert(EPI != EPI_SILU_GATE || (WTN % 32) == 0, "SiLU-gate needs 32-column wave tiles");

  __shared__ __attribute__((aligned(16))) T As[2][BM * BK];
  __shared__ __attribute__((aligned(16))) T Bs[2][BN * BK];
  __shared__ float Ss[Q80 ? 2 : 1][Q80 ? BN * 2 : 1];
  __shared__ int s_last;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // ---- tile coordinates: grouped ordering (8 M-tiles share B panels)
  const int tiles_m = cdiv(p.M, BM), tiles_n = cdiv(p.N, BN);
  const int split = blockIdx.x % p.splits;
  const int tile = blockIdx.x / p.splits;
  constexpr int GROUP = 8;
  const int group_size = GROUP * tiles_n;
  const int gidx = tile / group_size;
  const int first_m = gidx * GROUP;
  const int gm = min(tiles_m - first_m, GROUP);
  const int tm = first_m + (tile % group_size) % gm;
  const int tn = (tile % group_size) / gm;
  const int m0 = tm * BM, n0 = tn * BN;

  const int KT = cdiv(p.K, BK);
  const int kt0 = split * p.k_tiles_per_split;
  const int kt1 = min(kt0 + p.k_tiles_per_split, KT);

  const T* __restrict__ A = (const T*)p.A;

  uint4 ra[A_PER_T];
  uint4 rb[B_PER_T];
  float rs[Q80 ? 2 : 1];

  auto load_tile = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) {
      const int c = tid + i * NT;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (c < A_CHUNKS) {
        const int r = c / (BK / 8), kc = (c % (BK / 8)) * 8;
        if (m0 + r < p.M && k0 + kc < p.K)
          v = *(const uint4*)(A + (size_t)(m0 + r) * p.lda + k0 + kc);
      }
      ra[i] = v;
    }
    if constexpr (!Q80) {
      const T* __restrict__ B = (const T*)p.B;
#pragma unroll
      for (int i = 0; i < B_PER_T; ++i) {
        const int c = tid + i * NT;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (c < B_CHUNKS) {
          const int r = c / (BK / 8), kc = (c % (BK / 8)) * 8;
          if (n0 + r < p.N && k0 + kc < p.K)
            v = *(const uint4*)(B + (size_t)(n0 + r) * p.ldb + k0 + kc);
        }
        rb[i] = v;
      }
    } else {
      const int8_t* __restrict__ B = (const int8_t*)p.B;
#pragma unroll
      for (int i = 0; i < B_PER_T; ++i) {
        const int c = tid + i * NT;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (c < B_CHUNKS) {
          const int r = c / (BK / 16), kc = (c % (BK / 16)) * 16;
          if (n0 + r < p.N && k0 + kc < p.K)
            v = *(const uint4*)(B + (size_t)(n0 + r) * p.ldb + k0 + kc);
        }
        rb[i] = v;
      }
      // scales: BN rows x 2 blocks
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int c = tid + i * NT;
        float s = 0.f;
        if (c < BN * 2) {
          const int r = c >> 1, kb = c & 1;
          if (n0 + r < p.N && k0 + kb * 32 < p.K)
            s = __half2float(p.B_scale[(size_t)(n0 + r) * (p.ldb / 32) + (k0 / 32) + kb]);
        }
        rs[i] = s;
      }
    }
  };

  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) {
      const int c = tid + i * NT;
      if (c < A_CHUNKS) {
        const int r = c / (BK / 8), ch = c % (BK / 8);
        *(uint4*)(&As[buf][swz(r, ch)]) = ra[i];
      }
    }
    if constexpr (!Q80) {
#pragma unroll
      for (int i = 0; i < B_PER_T; ++i) {
        const int c = tid + i * NT;
        if (c < B_CHUNKS) {
          const int r = c / (BK / 8), ch = c % (BK / 8);
          *(uint4*)(&Bs[buf][swz(r, ch)]) = rb[i];
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < B_PER_T; ++i) {
        const int c = tid + i * NT;
        if (c < B_CHUNKS) {
          const int r = c / (BK / 16), ch = (c % (BK / 16)) * 2;
          const uint32_t w[4] = {rb[i].x, rb[i].y, rb[i].z, rb[i].w};
          T8 lo, hi;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            lo[e] = (T)(float)(int8_t)(w[e >> 2] >> ((e & 3) * 8));
            hi[e] = (T)(float)(int8_t)(w[2 + (e >> 2)] >> ((e & 3) * 8));
          }
          *(T8*)(&Bs[buf][swz(r, ch)]) = lo;
          *(T8*)(&Bs[buf][swz(r, ch + 1)]) = hi;
        }
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int c = tid + i * NT;
        if (c < BN * 2) Ss[buf][c] = rs[i];
      }
    }
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (kt0 < kt1) {
    load_tile(kt0);
    store_tile(0);
  }
  __syncthreads();

  for (int kt = kt0; kt < kt1; ++kt) {
    const int cur = (kt - kt0) & 1;
    const bool more = kt + 1 < kt1;
    if (more) load_tile(kt + 1);
#pragma unroll
    for (int kk = 0; kk < BK / 32; ++kk) {
      T8 af[FM], bfr[FN];
      const int ch = kk * 4 + (lane >> 4);
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = *(const T8*)(&As[cur][swz(wm * WTM + i * 16 + (lane & 15), ch)]);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[j] = *(const T8*)(&Bs[cur][swz(wn * WTN + j * 16 + (lane & 15), ch)]);
      if constexpr (!Q80) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) acc[i][j] = Mfma<T>::mma(af[i], bfr[j], acc[i][j]);
      } else {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const float sc = Ss[cur][(wn * WTN + j * 16 + (lane & 15)) * 2 + kk];
#pragma unroll
          for (int i = 0; i < FM; ++i) {
            const f32x4 t = Mfma<T>::mma(af[i], bfr[j], f32x4{0.f, 0.f, 0.f, 0.f});
            acc[i][j] += t * sc;
          }
        }
      }
    }
    if (more) store_tile(cur ^ 1);
    __syncthreads();
  }

  // ---- split-K: publish the partial tile; the last arrival reduces
  if (p.splits > 1) {
    constexpr int ACC = FM * FN * 4;
    const int tile_id = tm * tiles_n + tn;
    float* base = p.ws + (size_t)tile_id * p.splits * ACC * NT;
    {
      float* mine = base + (size_t)split * ACC * NT;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) mine[((i * FN + j) * 4 + r) * NT + tid] = acc[i][j][r];
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) {
      const int prev = atomicAdd(&p.counters[tile_id], 1);
      s_last = (prev == p.splits - 1);
      if (s_last) p.counters[tile_id] = 0;  // ready for the next call
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < p.splits; ++s) {
      const float* part = base + (size_t)s * ACC * NT;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] += part[((i * FN + j) * 4 + r) * NT + tid];
    }
  }

  // ---- epilogue.  acc[i][j][r] = C[m0 + wm*WTM + i*16 + 4*(lane/16) + r]
  //                                  [n0 + wn*WTN + j*16 + lane%16]
  const int col = lane & 15;
  const int rbase = m0 + wm * WTM + 4 * (lane >> 4);
  if constexpr (EPI == EPI_SILU_GATE) {
    bf16* __restrict__ C = (bf16*)p.C;
#pragma unroll
    for (int jp = 0; jp < FN / 2; ++jp) {
      const int ng = n0 + wn * WTN + jp * 32;  // first gate column of the pair
      const int jcol = ng / 2 + col;           // output column
      if (ng + col >= p.N) continue;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = rbase + i * 16 + r;
          if (m < p.M) {
            const float g = acc[i][2 * jp][r], u = acc[i][2 * jp + 1][r];
            C[(size_t)m * p.ldc + jcol] = f32_to_bf16(silu_f(g) * u);
          }
        }
    }
  } else {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = n0 + wn * WTN + j * 16 + col;
      if (n >= p.N) continue;
      float bias = 0.f;
      if constexpr (EPI == EPI_BIAS_F32)
        if (p.bias) bias = p.bias[n];
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = rbase + i * 16 + r;
          if (m >= p.M) continue;
          const float v = acc[i][j][r];
          if constexpr (EPI == EPI_BIAS_F32) {
            ((float*)p.C)[(size_t)m * p.ldc + n] = v + bias;
          } else if constexpr (EPI == EPI_RESID_F32) {
            const float res = bf16_to_f32(((const bf16*)p.resid)[(size_t)m * p.ldr + n]);
            ((float*)p.C)[(size_t)m * p.ldc + n] = v + res;
          } else {
            const float res = ((const float*)p.resid)[(size_t)m * p.ldr + n];
            ((bf16*)p.C)[(size_t)m * p.ldc + n] = f32_to_bf16(v + res);
          }
        }
    }
  }
}

struct Cfg {
  int BM, BN, NT;
};
// cfg 0: 128x128 (2x2 waves of 64x64) for many rows;
// cfg 1: 64x128 (1x4 waves of 64x32) for decode-sized M;
// cfg 2: 128x128 (1x4 waves of 128x32) for M in (64, 128].
constexpr Cfg kCfgs[3] = {{128, 128, 256}, {64, 128, 256}, {128, 128, 256}};

template <bool Q80, int EPI, typename T>
hipError_t launch_cfg(int cfg, int grid, const GemmArgs& a, hipStream_t s) {
  switch (cfg) {
    case 0:
      gemm_kernel<128, 128, 2, 2, Q80, EPI, T><<<grid, 256, 0, s>>>(a);
      break;
    case 1:
      gemm_kernel<64, 128, 1, 4, Q80, EPI, T><<<grid, 256, 0, s>>>(a);
      break;
    default:
      gemm_kernel<128, 128, 1, 4, Q80, EPI, T><<<grid, 256, 0, s>>>(a);
      break;
  }
  return hipGetLastError();
}

// The operand type follows the epilogue: the down projection (residual into
// a bf16 output) takes bf16 operands, the other three fp16.
template <bool Q80>
hipError_t launch_epi(int cfg, int grid, int epi, const GemmArgs& a, hipStream_t s) {
  switch (epi) {
    case EPI_BIAS_F32: return launch_cfg<Q80, EPI_BIAS_F32, f16>(cfg, grid, a, s);
    case EPI_RESID_F32: return launch_cfg<Q80, EPI_RESID_F32, f16>(cfg, grid, a, s);
    case EPI_RESID_BF16: return launch_cfg<Q80, EPI_RESID_BF16, bf16>(cfg, grid, a, s);
    default: return launch_cfg<Q80, EPI_SILU_GATE, f16>(cfg, grid, a, s);
  }
}

}  // namespace

GemmPlan gemm_plan(int M, int N, int K, bool q80, int epi) {
  (void)q80;
  (void)epi;
  GemmPlan pl{};
  pl.cfg = M <= 64 ? 1 : (M <= 128 ? 2 : 0);
  const Cfg c = kCfgs[pl.cfg];
  const int tiles = cdiv(M, c.BM) * cdiv(N, c.BN);
  const int KT = cdiv(K, BK);
  // enough workgroups to cover the 256 CUs about twice, each slice >= 4 k-tiles
  int splits = 1;
  while (tiles * splits < 512 && KT / (splits * 2) >= 4) splits *= 2;
  pl.k_tiles_per_split = cdiv(KT, splits);
  pl.splits = cdiv(KT, pl.k_tiles_per_split);
  pl.grid = tiles * pl.splits;
  pl.ws_floats = pl.splits > 1 ? (size_t)tiles * pl.splits * c.BM * c.BN : 0;
  pl.n_counters = pl.splits > 1 ? tiles : 0;
  return pl;
}

hipError_t gemm_launch(const GemmPlan& pl, GemmArgs a, bool q80, int epi, hipStream_t s) {
  a.splits = pl.splits;
  a.k_tiles_per_split = pl.k_tiles_per_split;
  if (q80) return launch_epi<true>(pl.cfg, pl.grid, epi, a, s);
  return launch_epi<false>(pl.cfg, pl.grid, epi, a, s);
}

}  // namespace tdl
