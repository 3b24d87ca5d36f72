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
// fp32 partial tile and a reduction kernel sums the slices in order --
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

#include <cmath>

namespace tdl {

namespace {

constexpr int BK = 64;  // k elements per tile (128 bytes of bf16 per row)

__device__ __forceinline__ int swz(int row, int chunk) {  // offset in bf16 elements
  return row * BK + ((chunk ^ (row & 7)) << 3);
}

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + __expf(-z)); }

// Eight int8 codes (little-endian bytes of c) as an exact MFMA operand.
// fp16: code + 128 is a byte u; the half with exponent byte 0x64 and u as its
// low mantissa bits is 1024 + u (one byte permute per two codes), and
// subtracting 1152 leaves the code exactly.  bf16 (7 fraction bits) cannot
// hold 1024 + u: u goes through the byte-to-float conversion instead.
template <typename T> struct Q80Codes;
template <> struct Q80Codes<f16> {
  __device__ static f16x8 cvt(uint2 c) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const uint32_t w[2] = {c.x ^ 0x80808080u, c.y ^ 0x80808080u};
    f16x8 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // bytes (u0, 0x64, u1, 0x64) from (w, 0x64646464)
      const uint32_t bits = __builtin_amdgcn_perm(0x64646464u, w[q >> 1], (q & 1) ? 0x04030402u : 0x04010400u);
      const h2 v = __builtin_bit_cast(h2, bits) - h2{(_Float16)1152.f, (_Float16)1152.f};
      o[2 * q] = v.x;
      o[2 * q + 1] = v.y;
    }
    return o;
  }
};
template <> struct Q80Codes<bf16> {
  __device__ static bf16x8 cvt(uint2 c) {
    const uint32_t w[2] = {c.x ^ 0x80808080u, c.y ^ 0x80808080u};
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (bf16)((float)((w[e >> 2] >> (8 * (e & 3))) & 0xffu) - 128.f);
    return o;
  }
};


// Result of one wave's FM x FN accumulator block whose top-left output
// element is (mw, nw): v[i][j][r] = C[mw + i*16 + 4*(lane/16) + r][nw + j*16 +
// lane%16].  One split: the epilogue; several: the fp32 partial tile goes to
// ws[split][M][N] and a second kernel sums the slices in order and applies
// the epilogue (no cross-workgroup handshake, which would need device-wide
// L2 write-backs on a multi-XCD part).
//
// GUARD = false for a wave block that lies inside the output (the common
// case): no per-element branches.  A guarded store is a branch, and the
// compiler waits (vmcnt(0), which counts earlier stores too) for a loaded
// bias inside every such branch, one memory round trip per element; the
// bias loads are unconditional from clamped addresses for the same reason.
// Residual epilogues normally go through LDS (resid_epilogue).
template <int EPI, int FM, int FN, bool GUARD>
__device__ __forceinline__ void gemm_store_block(const GemmArgs& p, const f32x4 (&v)[FM][FN], int mw,
                                                 int nw, int split, int lane) {
  const int col = lane & 15;
  const int rbase = mw + 4 * (lane >> 4);
  auto in_range = [&](int m, int n) { return !GUARD || (m < p.M && n < p.N); };
  if (p.splits > 1) {
    float* part = p.ws + (size_t)split * p.M * p.N;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = nw + j * 16 + col;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = rbase + i * 16 + r;
          if (in_range(m, n)) part[(size_t)m * p.N + n] = v[i][j][r];
        }
    }
    return;
  }
  if constexpr (EPI == EPI_SILU_GATE) {
    bf16* __restrict__ C = (bf16*)p.C;
#pragma unroll
    for (int jp = 0; jp < FN / 2; ++jp) {
      const int ng = nw + jp * 32;   // first gate column of the pair
      const int jcol = ng / 2 + col;  // output column
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = rbase + i * 16 + r;
          if (in_range(m, ng + col)) {
            const float g = v[i][2 * jp][r], u = v[i][2 * jp + 1][r];
            C[(size_t)m * p.ldc + jcol] = f32_to_bf16(silu_f(g) * u);
          }
        }
    }
  } else if constexpr (EPI == EPI_BIAS_F32) {
    float* __restrict__ Cf = (float*)p.C;
    float bias[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) bias[j] = p.bias ? p.bias[min(nw + j * 16 + col, p.N - 1)] : 0.f;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = nw + j * 16 + col;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = rbase + i * 16 + r;
          if (in_range(m, n)) Cf[(size_t)m * p.ldc + n] = v[i][j][r] + bias[j];
        }
    }
  } else {
    // residual epilogue without LDS: only for residual rows that are not
    // 16-byte aligned (resid_epilogue serves the rest), element by element
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = nw + j * 16 + col;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = rbase + i * 16 + r;
          if (!in_range(m, n)) continue;
          if constexpr (EPI == EPI_RESID_F32)
            ((float*)p.C)[(size_t)m * p.ldc + n] =
                v[i][j][r] + bf16_to_f32(((const bf16*)p.resid)[(size_t)m * p.ldr + n]);
          else
            ((bf16*)p.C)[(size_t)m * p.ldc + n] =
                f32_to_bf16(v[i][j][r] + ((const float*)p.resid)[(size_t)m * p.ldr + n]);
        }
    }
  }
}

template <int EPI, int FM, int FN>
__device__ __forceinline__ void gemm_store(const GemmArgs& p, const f32x4 (&v)[FM][FN], int mw, int nw,
                                           int split, int lane) {
  // wave-uniform: the whole FM*16 x FN*16 block inside the output
  if (mw + FM * 16 <= p.M && nw + FN * 16 <= p.N)
    gemm_store_block<EPI, FM, FN, false>(p, v, mw, nw, split, lane);
  else
    gemm_store_block<EPI, FM, FN, true>(p, v, mw, nw, split, lane);
}

// Residual epilogue through LDS, after the main loop (whose last barrier
// leaves the stage buffers free).  Each wave copies the residual rows of its
// block into its own LDS slice with 16-byte direct-to-LDS loads -- one
// coalesced round trip, no registers held -- then adds them element by
// element from LDS and stores.  FMP 16-row fragments per pass (fp32
// residuals take two passes in the eight-wave tiles).  Rows past M and
// chunks past N are clamped to valid addresses and never stored.
template <int EPI, int FM, int FN, int FMP>
__device__ __forceinline__ void resid_epilogue(const GemmArgs& p, const f32x4 (&v)[FM][FN], int mw,
                                               int nw, int lane, char* slice) {
  typedef typename std::conditional<EPI == EPI_RESID_F32, bf16, float>::type R;
  constexpr int WTN = FN * 16;
  constexpr int EPC = 16 / (int)sizeof(R);  // elements per 16-byte chunk
  constexpr int CPR = WTN / EPC;            // chunks per row
  constexpr int INSTS = FMP * 16 * CPR / 64;
  static_assert(WTN % EPC == 0 && (FMP * 16 * CPR) % 64 == 0 && FM % FMP == 0, "residual slice");
  const R* __restrict__ Rp = (const R*)p.resid;
  const bool full = mw + FM * 16 <= p.M && nw + WTN <= p.N;
  const int col = lane & 15, g4 = 4 * (lane >> 4);
  const R* sl = (const R*)slice;
#pragma unroll
  for (int i0 = 0; i0 < FM; i0 += FMP) {
#pragma unroll
    for (int t = 0; t < INSTS; ++t) {
      const int c = t * 64 + lane;
      const int gm = min(mw + i0 * 16 + c / CPR, p.M - 1);
      const int gn = min(nw + (c % CPR) * EPC, p.N - EPC);
      __builtin_amdgcn_global_load_lds((const void*)(Rp + (size_t)gm * p.ldr + gn),
                                       (lds_void*)(slice + t * 1024), 16, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
    for (int ii = 0; ii < FMP; ++ii)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int n = nw + j * 16 + col;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = mw + (i0 + ii) * 16 + g4 + r;
          float res;
          if constexpr (EPI == EPI_RESID_F32) res = bf16_to_f32(sl[(ii * 16 + g4 + r) * WTN + j * 16 + col]);
          else res = sl[(ii * 16 + g4 + r) * WTN + j * 16 + col];
          if (full || (m < p.M && n < p.N)) {
            const float val = v[i0 + ii][j][r] + res;
            if constexpr (EPI == EPI_RESID_BF16) ((bf16*)p.C)[(size_t)m * p.ldc + n] = f32_to_bf16(val);
            else ((float*)p.C)[(size_t)m * p.ldc + n] = val;
          }
        }
        // one column group's LDS reads at a time (register bound)
        __builtin_amdgcn_sched_barrier(0);
      }
    // the next pass refills the slice: this wave's LDS reads must be done
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Largest divisor of FM whose pass (FMP x 16 rows x BYTES_PER_ROW) fits CAP.
template <int FM, int BYTES_PER_I, int CAP>
constexpr int resid_fmp() {
  for (int f = FM; f >= 1; --f)
    if (FM % f == 0 && f * BYTES_PER_I <= CAP) return f;
  return 0;
}

// Output tile `tile` in the walk order: groups of 8 M-tiles sharing a B
// panel.
template <int BM, int BN>
__device__ __forceinline__ void tile_coords(const GemmArgs& p, int tile, int* m0, int* n0) {
  const int tiles_m = cdiv(p.M, BM), tiles_n = cdiv(p.N, BN);
  constexpr int GROUP = 8;
  const int group_size = GROUP * tiles_n;
  const int gidx = tile / group_size;
  const int first_m = gidx * GROUP;
  const int gm = min(tiles_m - first_m, GROUP);
  *m0 = (first_m + (tile % group_size) % gm) * BM;
  *n0 = ((tile % group_size) / gm) * BN;
}

// Tile of a workgroup.  Workgroups are dispatched round-robin over the 8
// XCDs (each with its own L2); remap so that consecutive logical ids run on
// one XCD.  With a split tail, the workgroups past full_tiles (dispatched
// last) are (tail tile, K slice) pairs: *tail >= 0.
template <int BM, int BN>
__device__ __forceinline__ void tile_of(const GemmArgs& p, int* m0, int* n0, int* split, int* tail) {
  int bid = blockIdx.x;
  int tile;
  *tail = -1;
  if (p.tail_splits > 1 && bid >= p.full_tiles) {
    const int tb = bid - p.full_tiles;
    *tail = tb / p.tail_splits;
    *split = tb % p.tail_splits;
    tile = p.full_tiles + *tail;
  } else {
    const int nwg = p.tail_splits > 1 ? p.full_tiles : (int)gridDim.x;
    const int per = nwg / 8, rem = nwg % 8;
    const int xcd = bid % 8, slot = bid / 8;
    bid = xcd * per + min(xcd, rem) + slot;
    *split = bid % p.splits;
    tile = bid / p.splits;
  }
  tile_coords<BM, BN>(p, tile, m0, n0);
}

// Split-tail partials: [tail tile][split][i][j][thread] of f32x4, i.e. each
// thread's accumulator registers as they are (16-byte coalesced stores).
template <int FM, int FN, int NT>
__device__ __forceinline__ size_t tail_offset(const GemmArgs& p, int tail, int split, int i, int j,
                                              int tid) {
  return ((((size_t)tail * p.tail_splits + split) * FM + i) * FN + j) * NT + tid;
}

// DIRECT: operand tiles go from global memory straight into LDS
// (global_load_lds_dwordx4, no staging registers).  A: each lane fetches the
// 16-byte chunk that belongs at its fixed LDS slot, so the XOR swizzle is
// applied on the source side.  B: weights in the packed tile layout
// (pack_weights); one load instruction copies one 1 KB tile as is, and a
// B fragment is then chunk `lane` of a tile in LDS (linear, conflict-free).
// Q8_0 (Q80 && DIRECT): the codes in the packed code layout (pack_codes),
// one 1 KB tile per 16 rows and 64 k; a lane's 16 bytes hold its fragments
// of both 32-k steps, converted exactly to the operand type after the LDS
// read; each lane loads its columns' two block scales per tile into
// registers, one tile ahead, and every 32-k step's MFMA product is scaled by
// its block's scale in fp32 (the Q8_0 arithmetic, no rounded weight copy).
// Needs K % 64 == 0 and packed weights.
template <int BM, int BN, int WM, int WN, bool Q80, int EPI, typename T, bool DIRECT>
__global__ __launch_bounds__(WM* WN * 64) void gemm_kernel(GemmArgs p) {
  typedef typename Mfma<T>::v8 T8;
  constexpr bool Q80D = Q80 && DIRECT;
  constexpr int NW = WM * WN;
  constexpr int NT = WM * WN * 64;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  constexpr int A_CHUNKS = BM * BK / 8;            // 16-byte chunks per A tile
  constexpr int B_CHUNKS = Q80 ? BN * BK / 16 : BN * BK / 8;  // global chunks
  constexpr int A_PER_T = DIRECT ? 1 : (A_CHUNKS + NT - 1) / NT;
  constexpr int B_PER_T = DIRECT ? 1 : (B_CHUNKS + NT - 1) / NT;
  static_assert(FM >= 1 && FN >= 1, "wave tile");
  static_assert(EPI != EPI_SILU_GATE || (WTN % 32) == 0, "SiLU-gate needs 32-column wave tiles");

  // two LDS stages as separate arrays: the direct path selects them
  // statically, so the compiler can tell an in-flight LDS fill of one stage
  // from reads of the other and does not wait for the fill
  __shared__ __attribute__((aligned(16))) T As0[BM * BK];
  __shared__ __attribute__((aligned(16))) T As1[BM * BK];
  // (Q8_0 direct: BN rows of 64 one-byte codes)
  __shared__ __attribute__((aligned(16))) T Bs0[Q80D ? BN * BK / 2 : BN * BK];
  __shared__ __attribute__((aligned(16))) T Bs1[Q80D ? BN * BK / 2 : BN * BK];
  __shared__ float Ss[Q80 && !DIRECT ? 2 : 1][Q80 && !DIRECT ? BN * 2 : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int col_l = lane & 15;

  int m0, n0, split, tail;
  tile_of<BM, BN>(p, &m0, &n0, &split, &tail);

  const int KT = cdiv(p.K, BK);
  const int kps = tail >= 0 ? p.tail_kps : p.k_tiles_per_split;
  const int kt0 = split * kps;
  const int kt1 = min(kt0 + kps, KT);

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

  // direct path: instruction i of a tile fills LDS rows 8i .. 8i+7 (1 KB);
  // lane L lands at row 8i + L/8, physical chunk L%8 = logical chunk ^ (row&7)
  auto issue_tile = [&](int kt, T* Ad, T* Bd) {
    const int k0 = kt * BK;
    const int r8 = lane >> 3, pc = lane & 7;
#pragma unroll
    for (int i = wave; i < BM / 8; i += NW) {
      const int row = i * 8 + r8;
      const int grow = min(m0 + row, p.M - 1);  // rows past M are computed, never stored
      const T* src = A + (size_t)grow * p.lda + k0 + ((pc ^ (row & 7)) << 3);
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)&Ad[i * 512], 16, 0, 0);
    }
    const int NG = p.N >> 4;
    if constexpr (Q80D) {
      // codes: instruction i copies the tile of row group i (groups past N
      // repeat the last one: computed, never stored)
      const int8_t* __restrict__ Bq = (const int8_t*)p.B;
#pragma unroll
      for (int i = wave; i < BN / 16; i += NW) {
        const int grp = min((n0 >> 4) + i, NG - 1);
        const int8_t* src = Bq + ((size_t)kt * NG + grp) * 1024 + lane * 16;
        __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)&Bd[i * 512], 16, 0, 0);
      }
      return;
    }
    // B: instruction i copies tile (k slice i / (BN/16), row group i % (BN/16));
    // groups past N repeat the last one (computed, never stored)
    const T* __restrict__ B = (const T*)p.B;
#pragma unroll
    for (int i = wave; i < BN / 8; i += NW) {
      const int ks = (k0 >> 5) + i / (BN / 16);
      const int grp = min((n0 >> 4) + i % (BN / 16), NG - 1);
      const T* src = B + ((size_t)ks * NG + grp) * 512 + lane * 8;
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)&Bd[i * 512], 16, 0, 0);
    }
  };

  auto store_tile = [&](int buf) {
    T* Ab = buf ? As1 : As0;
    T* Bb = buf ? Bs1 : Bs0;
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) {
      const int c = tid + i * NT;
      if (c < A_CHUNKS) {
        const int r = c / (BK / 8), ch = c % (BK / 8);
        *(uint4*)(&Ab[swz(r, ch)]) = ra[i];
      }
    }
    if constexpr (!Q80) {
#pragma unroll
      for (int i = 0; i < B_PER_T; ++i) {
        const int c = tid + i * NT;
        if (c < B_CHUNKS) {
          const int r = c / (BK / 8), ch = c % (BK / 8);
          *(uint4*)(&Bb[swz(r, ch)]) = rb[i];
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
          *(T8*)(&Bb[swz(r, ch)]) = lo;
          *(T8*)(&Bb[swz(r, ch + 1)]) = hi;
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

  // Q8_0 direct: this lane's block scales (two fp16 per column, for the two
  // 32-k steps of tile kt), columns past N clamped
  auto load_scales = [&](int kt, uint32_t (&sc)[FN]) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = min(n0 + wn * WTN + j * 16 + col_l, p.N - 1);
      sc[j] = *(const uint32_t*)(p.B_scale + (size_t)n * (p.K / 32) + 2 * kt);
    }
  };
  // one k-tile of MFMAs from a Q8_0 direct stage
  auto compute_q80 = [&](const T* Ab, const T* Bb, const uint32_t (&sc)[FN]) {
    uint2 bq[FN][2];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const uint4 c = *(const uint4*)((const int8_t*)Bb + ((wn * WTN + j * 16) / 16) * 1024 + lane * 16);
      bq[j][0] = make_uint2(c.x, c.y);
      bq[j][1] = make_uint2(c.z, c.w);
    }
#pragma unroll
    for (int kk = 0; kk < BK / 32; ++kk) {
      T8 af[FM];
      const int ch = kk * 4 + (lane >> 4);
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = *(const T8*)(&Ab[swz(wm * WTM + i * 16 + (lane & 15), ch)]);
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const T8 bfr = Q80Codes<T>::cvt(bq[j][kk]);
        const float s = __half2float(__ushort_as_half((unsigned short)(sc[j] >> (16 * kk))));
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const f32x4 t = Mfma<T>::mma(af[i], bfr, f32x4{0.f, 0.f, 0.f, 0.f});
          acc[i][j] += t * s;
        }
      }
    }
  };

  // one k-tile of MFMAs from the given LDS stage
  auto compute = [&](const T* Ab, const T* Bb, int sbuf) {
#pragma unroll
    for (int kk = 0; kk < BK / 32; ++kk) {
      // all A fragments of the wave tile, then one B fragment at a time
      T8 af[FM];
      const int ch = kk * 4 + (lane >> 4);
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = *(const T8*)(&Ab[swz(wm * WTM + i * 16 + (lane & 15), ch)]);
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const T8 bfr = DIRECT ? *(const T8*)(&Bb[(kk * (BN / 16) + (wn * WTN + j * 16) / 16) * 512 + lane * 8])
                              : *(const T8*)(&Bb[swz(wn * WTN + j * 16 + (lane & 15), ch)]);
        if constexpr (!Q80) {
#pragma unroll
          for (int i = 0; i < FM; ++i) acc[i][j] = Mfma<T>::mma(af[i], bfr, acc[i][j]);
        } else {
          const float sc = Ss[sbuf][(wn * WTN + j * 16 + (lane & 15)) * 2 + kk];
#pragma unroll
          for (int i = 0; i < FM; ++i) {
            const f32x4 t = Mfma<T>::mma(af[i], bfr, f32x4{0.f, 0.f, 0.f, 0.f});
            acc[i][j] += t * sc;
          }
        }
      }
    }
  };

  if constexpr (Q80D) {
    // as below, with each stage's block scales in registers beside it
    uint32_t sc0[FN], sc1[FN];
    if (kt0 < kt1) {
      issue_tile(kt0, As0, Bs0);
      load_scales(kt0, sc0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int kt = kt0; kt < kt1; kt += 2) {
      if (kt + 1 < kt1) {
        issue_tile(kt + 1, As1, Bs1);
        load_scales(kt + 1, sc1);
      }
      compute_q80(As0, Bs0, sc0);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (kt + 1 < kt1) {
        if (kt + 2 < kt1) {
          issue_tile(kt + 2, As0, Bs0);
          load_scales(kt + 2, sc0);
        }
        compute_q80(As1, Bs1, sc1);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
      }
    }
  } else if constexpr (DIRECT) {
    // stage 0 holds tile kt, stage 1 tile kt+1; the fill of the next tile
    // runs while this one feeds the MFMAs
    if (kt0 < kt1) issue_tile(kt0, As0, Bs0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int kt = kt0; kt < kt1; kt += 2) {
      if (kt + 1 < kt1) issue_tile(kt + 1, As1, Bs1);
      compute(As0, Bs0, 0);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (kt + 1 < kt1) {
        if (kt + 2 < kt1) issue_tile(kt + 2, As0, Bs0);
        compute(As1, Bs1, 1);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
      }
    }
  } else {
    if (kt0 < kt1) {
      load_tile(kt0);
      store_tile(0);
    }
    __syncthreads();
    for (int kt = kt0; kt < kt1; ++kt) {
      const int cur = (kt - kt0) & 1;
      const bool more = kt + 1 < kt1;
      if (more) load_tile(kt + 1);
      compute(cur ? As1 : As0, cur ? Bs1 : Bs0, cur);
      if (more) store_tile(cur ^ 1);
      __syncthreads();
    }
  }

  if (tail >= 0) {  // a K slice of a tail tile: the partial, as the registers hold it
    f32x4* ws = (f32x4*)p.tail_ws;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) ws[tail_offset<FM, FN, NT>(p, tail, split, i, j, tid)] = acc[i][j];
    return;
  }
  if constexpr (EPI == EPI_RESID_F32 || EPI == EPI_RESID_BF16) {
    // residual through LDS when its rows are 16-byte aligned (the main
    // loop's last barrier has left the stage buffers free)
    constexpr int RB = EPI == EPI_RESID_F32 ? 2 : 4;
    constexpr int SPA = NW / 4;  // wave slices per stage array
    static_assert(NW == 4 || NW == 8, "four stage arrays shared by the waves");
    constexpr int CAP = (int)(sizeof(As0) < sizeof(Bs0) ? sizeof(As0) : sizeof(Bs0)) / SPA;
    constexpr int FMP = resid_fmp<FM, 16 * WTN * RB, CAP>();
    static_assert(FMP >= 1, "residual slice does not fit");
    const int epc = 16 / RB;
    if (p.splits == 1 && ((uintptr_t)p.resid & 15) == 0 && p.ldr % epc == 0 && p.N % epc == 0) {
      const int arr = wave / SPA;
      T* base = arr == 0 ? As0 : arr == 1 ? As1 : arr == 2 ? Bs0 : Bs1;
      char* slice = (char*)base + (wave % SPA) * CAP;
      resid_epilogue<EPI, FM, FN, FMP>(p, acc, m0 + wm * WTM, n0 + wn * WTN, lane, slice);
      return;
    }
  }
  gemm_store<EPI, FM, FN>(p, acc, m0 + wm * WTM, n0 + wn * WTN, split, lane);
}

// Sum of the split-K slices in slice order, then the epilogue; one thread per
// 4 consecutive output columns (per gate/up pair for the SiLU-gate form).
// The slices are read SB at a time, every load of a batch issued before the
// first add (slice indices past the last repeat it and add nothing).
template <int EPI, int SB>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmArgs p) {
  const int Nout = EPI == EPI_SILU_GATE ? p.N / 2 : p.N;
  const int cols4 = Nout / 4;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)p.M * cols4) return;
  const int m = (int)(idx / cols4), c = (int)(idx % cols4) * 4;
  const size_t slice = (size_t)p.M * p.N;
  float out[4];
  if constexpr (EPI == EPI_SILU_GATE) {
    // output column j -> gate column 32*(j/16) + j%16, up column +16
    const int ng = 32 * (c / 16) + (c % 16);
    float g[4] = {0.f, 0.f, 0.f, 0.f}, u[4] = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < p.splits; s0 += SB) {
      float4 a[SB], b[SB];
#pragma unroll
      for (int q = 0; q < SB; ++q) {
        const float* src = p.ws + min(s0 + q, p.splits - 1) * slice + (size_t)m * p.N + ng;
        a[q] = *(const float4*)src;
        b[q] = *(const float4*)(src + 16);
      }
#pragma unroll
      for (int q = 0; q < SB; ++q) {  // a select, not a branch: the loads stay unconditional
        const bool live = s0 + q < p.splits;
        g[0] += live ? a[q].x : 0.f; g[1] += live ? a[q].y : 0.f;
        g[2] += live ? a[q].z : 0.f; g[3] += live ? a[q].w : 0.f;
        u[0] += live ? b[q].x : 0.f; u[1] += live ? b[q].y : 0.f;
        u[2] += live ? b[q].z : 0.f; u[3] += live ? b[q].w : 0.f;
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = silu_f(g[e]) * u[e];
    bf16* C = (bf16*)p.C + (size_t)m * p.ldc + c;
#pragma unroll
    for (int e = 0; e < 4; ++e) C[e] = f32_to_bf16(out[e]);
  } else {
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < p.splits; s0 += SB) {
      float4 a[SB];
#pragma unroll
      for (int q = 0; q < SB; ++q) a[q] = *(const float4*)(p.ws + min(s0 + q, p.splits - 1) * slice + (size_t)m * p.N + c);
#pragma unroll
      for (int q = 0; q < SB; ++q) {  // a select, not a branch: the loads stay unconditional
        const bool live = s0 + q < p.splits;
        v[0] += live ? a[q].x : 0.f; v[1] += live ? a[q].y : 0.f;
        v[2] += live ? a[q].z : 0.f; v[3] += live ? a[q].w : 0.f;
      }
    }
    // the residual is never the output: its loads all issue before the stores
    const bf16* __restrict__ Rb = (const bf16*)p.resid;
    const float* __restrict__ Rf = (const float*)p.resid;
    float add[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int n = c + e;
      if constexpr (EPI == EPI_BIAS_F32) add[e] = p.bias ? p.bias[n] : 0.f;
      else if constexpr (EPI == EPI_RESID_F32) add[e] = bf16_to_f32(Rb[(size_t)m * p.ldr + n]);
      else add[e] = Rf[(size_t)m * p.ldr + n];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int n = c + e;
      if constexpr (EPI == EPI_RESID_BF16) ((bf16*)p.C)[(size_t)m * p.ldc + n] = f32_to_bf16(v[e] + add[e]);
      else ((float*)p.C)[(size_t)m * p.ldc + n] = v[e] + add[e];
    }
  }
}

// Sums the K slices of the split-tail tiles in slice order (deterministic)
// and applies the epilogue: one 64-thread workgroup per (wave block, tail
// tile), grid (NW, tail tiles).  Bias and SiLU-gate epilogues only.
template <int BM, int BN, int WM, int WN, int EPI>
__global__ __launch_bounds__(64) void tail_reduce_kernel(GemmArgs p) {
  constexpr int NT = WM * WN * 64;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  static_assert(EPI == EPI_BIAS_F32 || EPI == EPI_SILU_GATE, "split tail: no residual epilogues");
  const int wave = blockIdx.x, tail = blockIdx.y, lane = threadIdx.x;
  const int tid = wave * 64 + lane;
  const int wm = wave / WN, wn = wave % WN;
  int m0, n0;
  tile_coords<BM, BN>(p, p.full_tiles + tail, &m0, &n0);
  const f32x4* ws = (const f32x4*)p.tail_ws;
  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = ws[tail_offset<FM, FN, NT>(p, tail, 0, i, j, tid)];
  for (int sp = 1; sp < p.tail_splits; ++sp)
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] += ws[tail_offset<FM, FN, NT>(p, tail, sp, i, j, tid)];
  gemm_store<EPI, FM, FN>(p, acc, m0 + wm * WTM, n0 + wn * WTN, 0, lane);
}

struct Cfg {
  int BM, BN;
  float eff;  // relative per-tile efficiency, for the planner
};
// cfg 0: 256x256 (2x4 waves of 128x64);  cfg 1: 256x224 (4x2 waves of
// 64x112: N = 3584 splits into 16 tiles);  cfg 2: 128x128 (2x2 waves of
// 64x64);  cfg 3: 64x128 (1x4 waves of 64x32) and cfg 4: 128x128 (1x4 waves
// of 128x32) for decode-sized M;  cfg 5: 256x288 (4x2 waves of 64x144: N =
// 4608 splits into 16 tiles, so 4096 rows make one tile per CU);  cfg 6:
// 192x256 (2x4 waves of 96x64: 2112 = 11 x 192 rows without a mostly empty
// last row of tiles).  Eight-wave tiles keep two waves per SIMD.
constexpr int kNumCfgs = 7;
constexpr Cfg kCfgs[kNumCfgs] = {{256, 256, 1.0f}, {256, 224, 0.96f}, {128, 128, 0.4f},
                                 {64, 128, 0.35f},  {128, 128, 0.5f},  {256, 288, 0.98f},
                                 {192, 256, 0.78f}};

template <bool Q80, int EPI, typename T, bool DIRECT>
hipError_t launch_cfg2(int cfg, int grid, const GemmArgs& a, hipStream_t s) {
  switch (cfg) {
    case 0:  // the planner gives the eight-wave 256x256 tiles bf16/fp16 weights only
      if constexpr (!Q80) gemm_kernel<256, 256, 2, 4, Q80, EPI, T, DIRECT><<<grid, 512, 0, s>>>(a);
      else return hipErrorInvalidValue;
      break;
    case 1:
      if constexpr (!Q80 && EPI != EPI_SILU_GATE)
        gemm_kernel<256, 224, 4, 2, Q80, EPI, T, DIRECT><<<grid, 512, 0, s>>>(a);
      else return hipErrorInvalidValue;
      break;
    case 2:
      gemm_kernel<128, 128, 2, 2, Q80, EPI, T, DIRECT><<<grid, 256, 0, s>>>(a);
      break;
    case 5:
      if constexpr (!Q80 && EPI != EPI_SILU_GATE)
        gemm_kernel<256, 288, 4, 2, Q80, EPI, T, DIRECT><<<grid, 512, 0, s>>>(a);
      else return hipErrorInvalidValue;
      break;
    case 6:
      if constexpr (!Q80 || DIRECT) gemm_kernel<192, 256, 2, 4, Q80, EPI, T, DIRECT><<<grid, 512, 0, s>>>(a);
      else return hipErrorInvalidValue;
      break;
    case 3:
      gemm_kernel<64, 128, 1, 4, Q80, EPI, T, DIRECT><<<grid, 256, 0, s>>>(a);
      break;
    default:
      gemm_kernel<128, 128, 1, 4, Q80, EPI, T, DIRECT><<<grid, 256, 0, s>>>(a);
      break;
  }
  return hipGetLastError();
}

template <bool Q80, int EPI, typename T>
hipError_t launch_cfg(int cfg, int grid, const GemmArgs& a, hipStream_t s) {
  if (a.b_packed) {
    if (a.K % BK != 0 || a.N % 16 != 0) return hipErrorInvalidValue;
    return launch_cfg2<Q80, EPI, T, true>(cfg, grid, a, s);
  }
  return launch_cfg2<Q80, EPI, T, false>(cfg, grid, a, s);
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

hipError_t tail_reduce(const GemmPlan& pl, const GemmArgs& a, int epi, hipStream_t s) {
  const int tail = (pl.grid - pl.full_tiles) / pl.tail_splits;
#define TDL_TAIL_CASE(CFG, BM, BN, WM, WN)                                                     \
  if (pl.cfg == CFG) {                                                                       \
    const dim3 grid(WM * WN, tail);                                                          \
    if (epi == EPI_SILU_GATE) tail_reduce_kernel<BM, BN, WM, WN, EPI_SILU_GATE><<<grid, 64, 0, s>>>(a); \
    else if (epi == EPI_BIAS_F32) tail_reduce_kernel<BM, BN, WM, WN, EPI_BIAS_F32><<<grid, 64, 0, s>>>(a); \
    else return hipErrorInvalidValue;                                                        \
    return hipGetLastError();                                                                \
  }
  TDL_TAIL_CASE(0, 256, 256, 2, 4)
  TDL_TAIL_CASE(2, 128, 128, 2, 2)
  TDL_TAIL_CASE(6, 192, 256, 2, 4)
#undef TDL_TAIL_CASE
  if (pl.cfg == 1 && epi == EPI_BIAS_F32) {
    tail_reduce_kernel<256, 224, 4, 2, EPI_BIAS_F32><<<dim3(8, tail), 64, 0, s>>>(a);
    return hipGetLastError();
  }
  if (pl.cfg == 5 && epi == EPI_BIAS_F32) {
    tail_reduce_kernel<256, 288, 4, 2, EPI_BIAS_F32><<<dim3(8, tail), 64, 0, s>>>(a);
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

template <int SB>
hipError_t splitk_reduce(const GemmArgs& a, int epi, int blocks, hipStream_t s) {
  switch (epi) {
    case EPI_BIAS_F32: splitk_reduce_kernel<EPI_BIAS_F32, SB><<<blocks, 256, 0, s>>>(a); break;
    case EPI_RESID_F32: splitk_reduce_kernel<EPI_RESID_F32, SB><<<blocks, 256, 0, s>>>(a); break;
    case EPI_RESID_BF16: splitk_reduce_kernel<EPI_RESID_BF16, SB><<<blocks, 256, 0, s>>>(a); break;
    default: splitk_reduce_kernel<EPI_SILU_GATE, SB><<<blocks, 256, 0, s>>>(a); break;
  }
  return hipGetLastError();
}

}  // namespace

// Chooses the tile configuration and split-K factor with the lowest estimated
// time: rounds of workgroups over the 256 CUs times the per-workgroup work,
// divided by the configuration's relative efficiency.
GemmPlan gemm_plan(int M, int N, int K, int wf, int epi, bool packed) {
  const bool q80 = wf == kWQ80;  // per-row int8 has no large-M kernel: callers expand it
  constexpr int kCUs = 256;
  {
    GemmPlan sk{};
    if (skinny_plan(M, N, K, wf, epi, &sk)) return sk;
  }
  const int KT = cdiv(K, BK);
  GemmPlan best{};
  double best_cost = 1e300;
  for (int cfg = 0; cfg < kNumCfgs; ++cfg) {
    const Cfg c = kCfgs[cfg];
    if (cfg == 1 && (epi == EPI_SILU_GATE || N % 224 != 0)) continue;
    if (cfg == 5 && (epi == EPI_SILU_GATE || N % 288 != 0)) continue;
    // Q8_0: row-major codes take the four-wave register path; packed codes
    // also the eight-wave 192x256 tiles (the larger eight-wave tiles would
    // spill with the scales and codes beside the accumulators)
    if (q80 && (cfg <= 1 || cfg == 5 || (!packed && cfg == 6))) continue;
    if ((cfg == 3 || cfg == 4) && M > 128) continue;  // the decode shapes only
    if (cfg == 3 && M > 64) continue;
    const int tiles = cdiv(M, c.BM) * cdiv(N, c.BN);
    for (int splits = 1; splits <= 16; ++splits) {
      if (splits > 1 && KT / splits < 4) break;
      const int kps = cdiv(KT, splits);
      const int sp = cdiv(KT, kps);
      if (sp != splits) continue;  // the same plan as a smaller count
      const int wgs = tiles * sp;
      const double rounds = std::ceil((double)wgs / kCUs);
      double cost = rounds * (double)c.BM * c.BN * kps / c.eff;
      // split-K: the fp32 partial slices make a round trip through memory
      // (about 0.01 cost units per byte: a unit is ~25 ps of a CU, a byte
      // ~0.25 ps of the chip) and the reduction is a second launch
      if (sp > 1) cost += 0.01 * 2.0 * sp * (double)M * N * 4.0 + 2.4e5;
      if (cost < best_cost) {
        best_cost = cost;
        best = GemmPlan{};
        best.cfg = cfg;
        best.splits = sp;
        best.k_tiles_per_split = kps;
        best.grid = wgs;
        best.ws_floats = sp > 1 ? (size_t)sp * M * N : 0;
      }
    }
    // split tail: when the last round of whole tiles would be at most half
    // full, its tiles are cut along K into enough slices to fill the chip;
    // their fp32 partials make a round trip through memory (about 0.01 cost
    // units per byte, plus a second launch)
    const int full = tiles / kCUs * kCUs, tail = tiles - full;
    if (full > 0 && tail > 0 && 2 * tail <= kCUs && (epi == EPI_BIAS_F32 || epi == EPI_SILU_GATE) &&
        cfg != 3 && cfg != 4) {
      const int ts = std::min(kCUs / tail, KT / 8);
      if (ts >= 2) {
        const int tkps = cdiv(KT, ts);
        const int tsp = cdiv(KT, tkps);
        const double bytes = 2.0 * tail * tsp * (double)c.BM * c.BN * 4.0;
        const double cost = (double)(full / kCUs) * c.BM * c.BN * KT / c.eff +
                            (double)c.BM * c.BN * tkps / c.eff + 0.01 * bytes + 2.4e5;
        if (cost < best_cost) {
          best_cost = cost;
          best = GemmPlan{};
          best.cfg = cfg;
          best.splits = 1;
          best.k_tiles_per_split = KT;
          best.full_tiles = full;
          best.tail_splits = tsp;
          best.tail_kps = tkps;
          best.grid = full + tail * tsp;
          best.ws_floats = (size_t)tail * tsp * c.BM * c.BN;
        }
      }
    }
  }
  return best;
}

hipError_t gemm_launch(const GemmPlan& pl, GemmArgs a, int wf, int epi, hipStream_t s, bool reduce) {
  a.splits = pl.splits;
  a.k_tiles_per_split = pl.k_tiles_per_split;
  a.full_tiles = pl.full_tiles;
  a.tail_splits = pl.tail_splits;
  a.tail_kps = pl.tail_kps;
  a.tail_ws = pl.tail_splits > 1 ? a.ws : nullptr;
  a.rng_count = pl.rng_count;
  if (pl.tail_splits > 1 && (!a.ws || pl.splits != 1)) return hipErrorInvalidValue;
  if (pl.cfg < 10 && wf == kWIQ8) return hipErrorInvalidValue;
  const hipError_t e = pl.cfg >= 10     ? gemm_skinny_launch(pl, a, wf, epi, s)
                       : wf == kWQ80 ? launch_epi<true>(pl.cfg, pl.grid, epi, a, s)
                                        : launch_epi<false>(pl.cfg, pl.grid, epi, a, s);
  if (e != hipSuccess) return e;
  if (pl.tail_splits > 1) return tail_reduce(pl, a, epi, s);
  if (pl.splits == 1 || !reduce) return e;
  const int Nout = epi == EPI_SILU_GATE ? a.N / 2 : a.N;
  const int64_t threads = (int64_t)a.M * (Nout / 4);
  const int blocks = (int)((threads + 255) / 256);
  if (a.splits <= 4) return splitk_reduce<4>(a, epi, blocks, s);
  if (a.splits <= 8) return splitk_reduce<8>(a, epi, blocks, s);
  return splitk_reduce<16>(a, epi, blocks, s);
}

}  // namespace tdl
