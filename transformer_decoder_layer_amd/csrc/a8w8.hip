// int8 x int8 GEMM with a dequantising epilogue (the activation-quantised
// GEMM of the devpress heterogeneous-engine page, section 4.5): C = A B^T
// accumulated in int32 on the int8 MFMA units, then out = C * a_scale[m] *
// b_scale[n] in fp32.  A [M, K] and B [N, K] are int8, row-major (B in
// Linear layout).
//
// A workgroup (4 waves, 2 x 2) owns a 128 x 128 tile of C; each wave a
// 64 x 64 quarter as 4 x 4 MFMA tiles of 16 x 16 (v_mfma_i32_16x16x64_i8:
// one 64-wide k step per instruction).  A and B k-slices of 64 bytes per row
// go global -> registers -> LDS, double-buffered: the next slice's loads are
// issued before the current slice's MFMAs.  In LDS a row is 4 chunks of 16
// bytes; chunk c of row r sits at position c ^ ((r >> 2) & 3), so the 16
// rows one fragment read touches (same chunk) fall on distinct banks.
//
// K % 64 == 0 (every slice whole): 256 x 128 tiles of 8 waves (4 x 2, each
// still 64 x 64), the slices going straight to LDS instead (direct-to-LDS
// copies, 1 KB = 16 rows per instruction, the swizzle applied on the source
// side) into a ring of three stages, one LDS array per stage, so that two
// slices are in flight during each step's MFMAs.

#include "common.h"
#include "kernels.h"

namespace tdl {

namespace {

constexpr int kTile = 128;  // rows of A and of B per workgroup
constexpr int kStep = 64;   // k per step (bytes per row and step)

__device__ __forceinline__ int lds_off(int r, int c) { return r * kStep + 16 * (c ^ ((r >> 2) & 3)); }

// The epilogue of one wave's 64 x 64 quarter at (mw, nw): v = C a_scale[m]
// b_scale[n] in fp32, then by e.epi: fp32 out (and the int32 sums to C);
// + bias[n] (fp32 out); + bf16 residual (fp32 out); + fp32 residual (bf16
// out); or SiLU(gate) * up, the gate and up columns interleaved in groups of
// 16 (columns 32g .. 32g+15 gate, 32g+16 .. +31 up: fragments j and j + 1
// of a lane pair them) into bf16 column 16g + c.
template <typename Acc>
__device__ __forceinline__ void a8w8_store(const Acc& acc, const A8Epi& e, const float* __restrict__ a_scale,
                                           const float* __restrict__ b_scale, int32_t* __restrict__ C, int M,
                                           int N, int mw, int nw, int lane) {
  const int rq = 4 * (lane >> 4), cq = lane & 15;
  if (e.epi == kA8SiluGate) {
#pragma unroll
    for (int j = 0; j < 4; j += 2) {
      const int ng = nw + 16 * j + cq, nu = ng + 16;
      if (nu >= N) continue;
      const float sg = b_scale[ng], su = b_scale[nu];
      const int oc = (nw + 16 * j) / 2 + cq;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = mw + 16 * i + rq + r;
          if (m >= M) continue;
          const float sa = a_scale[m];
          const float g = (float)acc[i][j][r] * sa * sg, u = (float)acc[i][j + 1][r] * sa * su;
          ((bf16*)e.out)[(size_t)m * e.ldo + oc] = f32_to_bf16(g / (1.0f + __expf(-g)) * u);
        }
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = nw + 16 * j + cq;
    if (n >= N) continue;
    const float sb = b_scale[n];
    const float bias = e.epi == kA8Bias && e.bias ? e.bias[n] : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = mw + 16 * i + rq + r;
        if (m >= M) continue;
        const int32_t c = acc[i][j][r];
        const float v = (float)c * a_scale[m] * sb;
        const size_t o = (size_t)m * e.ldo + n;
        switch (e.epi) {
          case kA8ResidF32:
            ((float*)e.out)[o] = v + (float)((const bf16*)e.resid)[(size_t)m * e.ldr + n];
            break;
          case kA8ResidBf16:
            ((bf16*)e.out)[o] = f32_to_bf16(v + ((const float*)e.resid)[(size_t)m * e.ldr + n]);
            break;
          default:  // kA8Out, kA8Bias
            if (C) C[(size_t)m * N + n] = c;
            ((float*)e.out)[o] = v + bias;
        }
      }
  }
}

__global__ __launch_bounds__(256) void a8w8_gemm_kernel(const int8_t* __restrict__ A,
                                                        const int8_t* __restrict__ B,
                                                        const float* __restrict__ a_scale,
                                                        const float* __restrict__ b_scale,
                                                        int32_t* __restrict__ C, A8Epi e,
                                                        int M, int N, int K) {
  __shared__ __attribute__((aligned(16))) int8_t As[2][kTile * kStep];
  __shared__ __attribute__((aligned(16))) int8_t Bs[2][kTile * kStep];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * kTile, n0 = blockIdx.x * kTile;
  const int steps = (K + kStep - 1) / kStep;

  // this thread's two 16-byte chunks of each tile: chunk q = tid + 256 i,
  // row q / 4, chunk q % 4; rows past M / N and k past K read as zero
  struct Regs {
    i32x4 a[2], b[2];
  };
  auto load = [&](int s, Regs& R) {
    i32x4* ra = R.a;
    i32x4* rb = R.b;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = tid + 256 * i, r = q >> 2, k = s * kStep + 16 * (q & 3);
      const bool kin = k < K;
      ra[i] = (m0 + r < M && kin) ? *(const i32x4*)(A + (size_t)(m0 + r) * K + k) : i32x4{0, 0, 0, 0};
      rb[i] = (n0 + r < N && kin) ? *(const i32x4*)(B + (size_t)(n0 + r) * K + k) : i32x4{0, 0, 0, 0};
    }
  };
  auto store = [&](int buf, const Regs& R) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = tid + 256 * i, r = q >> 2, c = q & 3;
      *(i32x4*)&As[buf][lds_off(r, c)] = R.a[i];
      *(i32x4*)&Bs[buf][lds_off(r, c)] = R.b[i];
    }
  };

  i32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = i32x4{0, 0, 0, 0};

  auto mma_step = [&](int buf) {
    // fragments: lane l takes row l % 16 of a 16-row tile, chunk l / 16
    i32x4 af[4], bfr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      af[i] = *(const i32x4*)&As[buf][lds_off(wm * 64 + 16 * i + (lane & 15), lane >> 4)];
      bfr[i] = *(const i32x4*)&Bs[buf][lds_off(wn * 64 + 16 * i + (lane & 15), lane >> 4)];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], bfr[j], acc[i][j], 0, 0, 0);
  };
  Regs R;
  load(0, R);
  store(0, R);
  __syncthreads();
  for (int s = 0; s < steps; ++s) {
    const int buf = s & 1;
    if (s + 1 < steps) load(s + 1, R);  // in flight during this step's MFMAs
    mma_step(buf);
    if (s + 1 < steps) {
      store(buf ^ 1, R);  // the other buffer: last read a step ago, before the barrier below
      __syncthreads();
    }
  }

  // acc[i][j][r] = C[row 16i + 4(lane/16) + r][col 16j + lane%16] of the wave's quarter
  a8w8_store(acc, e, a_scale, b_scale, C, M, N, m0 + wm * 64, n0 + wn * 64, lane);
}

// Direct-to-LDS variant (K % 64 == 0).  Each wave issues 2 copies of A
// (instructions w and w + 8 of the 16 per A tile) and 1 of B (instruction w
// of 8) per stage; rows past M / N are clamped to the last row (computed,
// never stored).  Loads past the last stage repeat it into a buffer that is
// not read again, so every step waits for the same count.
constexpr int kRing = 3;
constexpr int kTileM = 256;
constexpr int vm_wait(int n) { return (n & 15) | (7 << 4) | (15 << 8) | (((n >> 4) & 3) << 14); }

__global__ __launch_bounds__(512) void a8w8_gemm_direct_kernel(const int8_t* __restrict__ A,
                                                               const int8_t* __restrict__ B,
                                                               const float* __restrict__ a_scale,
                                                               const float* __restrict__ b_scale,
                                                               int32_t* __restrict__ C, A8Epi e, int M,
                                                               int N, int K) {
  __shared__ __attribute__((aligned(16))) int8_t A0[kTileM * kStep];
  __shared__ __attribute__((aligned(16))) int8_t A1[kTileM * kStep];
  __shared__ __attribute__((aligned(16))) int8_t A2[kTileM * kStep];
  __shared__ __attribute__((aligned(16))) int8_t B0[kTile * kStep];
  __shared__ __attribute__((aligned(16))) int8_t B1[kTile * kStep];
  __shared__ __attribute__((aligned(16))) int8_t B2[kTile * kStep];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * kTileM, n0 = blockIdx.x * kTile;
  const int steps = K / kStep;

  // this wave's copy instructions: A rows 16j .. 16j+15 for j = wave and
  // wave + 8, B rows 16 wave ..; lane l lands at row 16j + l/4, position
  // l%4, holding source chunk (l%4) ^ ((row >> 2) & 3)
  const int8_t* a_src[2];
  const int8_t* b_src;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int j = wave + 8 * h, r = 16 * j + (lane >> 2);
    a_src[h] = A + (size_t)min(m0 + r, M - 1) * K + 16 * ((lane & 3) ^ ((r >> 2) & 3));
  }
  {
    const int r = 16 * wave + (lane >> 2);
    b_src = B + (size_t)min(n0 + r, N - 1) * K + 16 * ((lane & 3) ^ ((r >> 2) & 3));
  }
  auto issue = [&](int s, int8_t* Ad, int8_t* Bd) {
    const size_t k0 = (size_t)min(s, steps - 1) * kStep;
#pragma unroll
    for (int h = 0; h < 2; ++h)
      __builtin_amdgcn_global_load_lds((const void*)(a_src[h] + k0), (lds_void*)(Ad + 1024 * (wave + 8 * h)), 16,
                                       0, 0);
    __builtin_amdgcn_global_load_lds((const void*)(b_src + k0), (lds_void*)(Bd + 1024 * wave), 16, 0, 0);
  };

  i32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = i32x4{0, 0, 0, 0};
  auto mma = [&](const int8_t* Ab, const int8_t* Bb) {
    i32x4 af[4], bfr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      af[i] = *(const i32x4*)&Ab[lds_off(wm * 64 + 16 * i + (lane & 15), lane >> 4)];
      bfr[i] = *(const i32x4*)&Bb[lds_off(wn * 64 + 16 * i + (lane & 15), lane >> 4)];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], bfr[j], acc[i][j], 0, 0, 0);
  };

  issue(0, A0, B0);
  issue(1, A1, B1);
  for (int s = 0; s < steps; s += kRing) {
#pragma unroll
    for (int j = 0; j < kRing; ++j) {
      // stage s + j landed for every wave (only stage s + j + 1 may be in
      // flight), and every wave is done with the buffer refilled next
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(vm_wait(3));
      asm volatile("s_barrier" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      const int nb = (j + 2) % kRing;
      issue(s + j + 2, nb == 0 ? A0 : nb == 1 ? A1 : A2, nb == 0 ? B0 : nb == 1 ? B1 : B2);
      __builtin_amdgcn_sched_barrier(0);
      if (j == 0 || s + j < steps) mma(j == 0 ? A0 : j == 1 ? A1 : A2, j == 0 ? B0 : j == 1 ? B1 : B2);
    }
  }
  __builtin_amdgcn_s_waitcnt(vm_wait(0));  // the last (unused) copies land before the workgroup ends

  a8w8_store(acc, e, a_scale, b_scale, C, M, N, m0 + wm * 64, n0 + wn * 64, lane);
}

}  // namespace

hipError_t a8w8_gemm_epi(const void* A, const void* B, const float* a_scale, const float* b_scale,
                         int32_t* C, const A8Epi& e, int M, int N, int K, hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  if (M < 0 || N < 0 || K < 16 || K % 16 != 0) return hipErrorInvalidValue;
  if (e.epi == kA8SiluGate && N % 32 != 0) return hipErrorInvalidValue;
  if (K % kStep == 0) {
    dim3 grid((N + kTile - 1) / kTile, (M + kTileM - 1) / kTileM);
    a8w8_gemm_direct_kernel<<<grid, 512, 0, s>>>((const int8_t*)A, (const int8_t*)B, a_scale, b_scale, C, e,
                                                 M, N, K);
    return hipGetLastError();
  }
  dim3 grid((N + kTile - 1) / kTile, (M + kTile - 1) / kTile);
  a8w8_gemm_kernel<<<grid, 256, 0, s>>>((const int8_t*)A, (const int8_t*)B, a_scale, b_scale, C, e, M, N, K);
  return hipGetLastError();
}

hipError_t a8w8_gemm(const void* A, const void* B, const float* a_scale, const float* b_scale,
                     int32_t* C, float* out, int M, int N, int K, hipStream_t s) {
  A8Epi e{};
  e.epi = kA8Out;
  e.out = out;
  e.ldo = N;
  return a8w8_gemm_epi(A, B, a_scale, b_scale, C, e, M, N, K, s);
}

}  // namespace tdl
